"""Shared helpers for the GPU parity tests: run the HIP path through the
C-ABI binding and the oracle on the same seeded inputs."""
import concurrent.futures as cf
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import kv_cache_top_srht_amd as pk  # noqa: E402
from kv_cache_top_srht_amd import synth  # noqa: E402

# attention outputs in bf16: |gpu - oracle| <= 2e-2 (the bar the method's
# parity statement sets); fp32 outputs are held to 1e-4.
ATTN_TOL_BF16 = 2e-2
ATTN_TOL_FP32 = 1e-4


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pk.lib()  # fail loudly if the library is missing


def case(msg):
    print("[case] " + msg, flush=True)


def gpu_layer(w, capacity=None, layer=0):
    dev = "cuda"
    lay = synth.make_layer(w, dev, layer=layer, capacity=capacity)
    cfg = pk.config_for(w, capacity=capacity or w.N)
    L = pk.Layer(cfg, lay["signs"], lay["K"], w.N, k=w.k, device=dev)
    return lay, cfg, L


def host_f32(t):
    return t.float().cpu().numpy()


def oracle_encode_heads(orc, w, K_host, signs, heads, n=None, workers=8):
    """Oracle encode of keys [0, n) of each (b, h) in `heads` (list of bh)."""
    n = n or w.N
    Kf = K_host.reshape(-1, K_host.shape[-2], K_host.shape[-1])

    def one(bh):
        return orc.encode_keys(signs, Kf[bh, :n], w.m)

    with cf.ThreadPoolExecutor(workers) as ex:
        return dict(zip(heads, ex.map(one, heads)))


def oracle_retrieve_heads(orc, w, Q_host, enc, signs, heads, workers=8):
    """Oracle retrieval for each (b, h) in `heads` given its encode."""
    G = w.G

    def one(bh):
        b, h = divmod(bh, w.n_kv_heads)
        ids, nib, wq = enc[bh]
        return orc.retrieve_head(signs, Q_host[b, h * G:(h + 1) * G], ids, nib,
                                 wq, m=w.m, rho=w.rho, tiers=w.tiers, S=w.sinks,
                                 k=w.k, num=w.cand_num, den=w.cand_den)

    with cf.ThreadPoolExecutor(workers) as ex:
        return dict(zip(heads, ex.map(one, heads)))


def gpu_intermediates(L, BH):
    return {
        "lut": pk.pariskv_debug_intermediate(L.handle, L.k, L.ws, pk.DEBUG_LUT, BH),
        "yq": pk.pariskv_debug_intermediate(L.handle, L.k, L.ws, pk.DEBUG_YQ, BH),
        "scores": pk.pariskv_debug_intermediate(L.handle, L.k, L.ws,
                                                pk.DEBUG_SCORES, BH),
        "cand": pk.pariskv_debug_intermediate(L.handle, L.k, L.ws, pk.DEBUG_CAND, BH),
        "est": pk.pariskv_debug_intermediate(L.handle, L.k, L.ws, pk.DEBUG_EST, BH),
        "thresh": pk.pariskv_debug_intermediate(L.handle, L.k, L.ws,
                                                pk.DEBUG_THRESH, BH),
    }


def vote_table(lut, m):
    """The oracle's per-subspace vote LUT [B][2^m] as the byte-indexed table
    the scan reads: row s is indexed by byte s of a key's ids, which holds
    one id for m = 8 and the ids of subspaces 2s (low nibble) and 2s + 1
    (high nibble) for m = 4."""
    if m == 8:
        return lut
    v = np.arange(256)
    return (lut[0::2][:, v & 15].astype(np.int32) +
            lut[1::2][:, v >> 4].astype(np.int32)).astype(np.uint8)


def assert_retrieval_equal(w, gi, idx, est_out, ref, bh):
    r = ref
    assert np.array_equal(gi["lut"][bh].reshape(16, 256), vote_table(r["lut"], w.m)), bh
    assert np.array_equal(gi["yq"][bh].view(np.uint32), r["yq"].view(np.uint32)), bh
    assert np.array_equal(gi["scores"][bh].astype(np.int32), r["scores"]), bh
    assert gi["thresh"][bh][3] == r["C"]
    assert np.array_equal(gi["cand"][bh], r["cand"]), bh
    assert np.array_equal(gi["est"][bh].view(np.uint32), r["est"].view(np.uint32)), bh
    assert np.array_equal(idx[bh], r["idx"]), bh
    if est_out is not None:
        # estimates of the selected non-sink keys, aligned with idx[S:]
        pos = np.searchsorted(r["cand"], idx[bh][w.sinks:])
        assert np.array_equal(est_out[bh].view(np.uint32),
                              r["est"][pos].view(np.uint32)), bh
