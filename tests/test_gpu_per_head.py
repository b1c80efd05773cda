"""Unshared (per-query-head) retrieval: each query head retrieves its own
top-k with its own query over its KV head's index, and attends to its own
rows.  Checked against the oracle's single-query retrieval (a group of one
head) and attention per query head."""
import numpy as np
import pytest
import torch

from gpu_helpers import (ATTN_TOL_BF16, assert_retrieval_equal, case,
                         gpu_intermediates, host_f32, need_gpu,
                         oracle_encode_heads, pk, synth)

pytestmark = pytest.mark.gpu

W = synth.Workload

CASES = {
    "gqa": W("per head, GQA 4", 2, 2, 8, 128, 5003, "bf16", k=128, seed=71,
             per_query_head=True),
    "sinks": W("per head, sinks", 1, 3, 6, 128, 7001, "bf16", cand_num=1,
               cand_den=10, k=200, sinks=64, seed=72, per_query_head=True),
    # large enough for chunks of 512 or more keys, where one scan pass serves
    # all G query heads of a KV head: G = 4 with 2048-key chunks, G = 8 and
    # G = 2 (m = 4) with 512-key chunks
    "gqa4_long": W("per head, GQA 4, 140K", 1, 8, 32, 128, 140000, "bf16",
                   k=1024, seed=73, per_query_head=True),
    "gqa8": W("per head, GQA 8", 1, 2, 16, 128, 70000, "bf16", k=512, sinks=16,
              seed=74, per_query_head=True),
    "gqa2_m4": W("per head, GQA 2, m 4", 4, 4, 8, 128, 40000, "bf16", B=32,
                 k=256, seed=75, per_query_head=True),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("name", list(CASES))
def test_per_query_head_retrieval(orc, name):
    w = CASES[name]
    case("%s: batch=%d Hkv=%d Hq=%d N=%d k=%d S=%d" % (
        w.name, w.batch, w.n_kv_heads, w.n_q_heads, w.N, w.k, w.sinks))
    G = w.G
    lay = synth.make_layer(w, "cuda")
    K, V, Q = lay["K"], lay["V"], lay["Q"]
    cfg = pk.config_for(w)
    L = pk.Layer(cfg, lay["signs"], K, w.N - 2, k=w.k)
    for _ in range(2):   # appended keys are encoded once per KV head
        n = L.size
        L.append(K[:, :, n:], 1, rows_per_head=w.N)
    U = w.batch * w.n_q_heads
    idx = torch.empty(U, w.k, dtype=torch.int32, device="cuda")
    est = torch.empty(U, w.kprime, dtype=torch.float32, device="cuda")
    L.retrieve(Q, idx, est)
    out = torch.empty_like(Q)
    L.attend(Q, K, V, idx, out)
    torch.cuda.synchronize()
    Kh, Vh, Qh = host_f32(K), host_f32(V), host_f32(Q)
    BH = w.batch * w.n_kv_heads
    enc = oracle_encode_heads(orc, w, Kh, lay["signs"], list(range(BH)))
    ids, nib, wq = pk.pariskv_debug_export(L.handle, 0, w.N, BH, B=w.B)
    for bh in range(BH):
        assert np.array_equal(ids[bh], enc[bh][0])
        assert np.array_equal(nib[bh], enc[bh][1])
        assert np.array_equal(wq[bh], enc[bh][2])
    gi = gpu_intermediates(L, U)
    ih, eh, oh = idx.cpu().numpy(), est.cpu().numpy(), host_f32(out)
    for u in range(U):
        b, hq = divmod(u, w.n_q_heads)
        kvh = b * w.n_kv_heads + hq // G
        ref = orc.retrieve_head(lay["signs"], Qh[b, hq:hq + 1], *enc[kvh], m=w.m,
                                rho=w.rho, tiers=w.tiers, S=w.sinks, k=w.k,
                                num=w.cand_num, den=w.cand_den)
        assert_retrieval_equal(w, gi, ih, eh, ref, u)
        ref_o = orc.attention(Qh[b, hq:hq + 1], Kh[b, hq // G], Vh[b, hq // G], ih[u],
                              w.d ** -0.5)
        assert np.max(np.abs(oh[b, hq] - ref_o[0])) <= ATTN_TOL_BF16
    # the event-timed entry point runs the same kernels
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    out2 = torch.empty_like(Q)
    pk.pariskv_sparse_attn_per_query_head_profiled(
        Q, K, V, w.N, idx, w.k, w.batch, w.n_q_heads, w.n_kv_heads, w.d,
        pk.PARISKV_DTYPE_BF16, w.d ** -0.5, out2, L.attn_ws, ev)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    assert ev[0].elapsed_time(ev[1]) > 0
    L.close()
