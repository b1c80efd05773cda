"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the Llama-3-8B-shaped 32K layer end to end on every head;
the 8 x 128K batched layer and the 1M-token layer on sampled (batch, KV
head) pairs (the oracle re-encodes the whole sampled head and runs the whole
retrieval for it), plus sampled windows of the index for every head, and
attention of the sampled heads over the GPU-selected rows."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

from gpu_helpers import (ATTN_TOL_BF16, assert_retrieval_equal, case,
                         gpu_intermediates, gpu_layer, host_f32, need_gpu,
                         oracle_retrieve_heads, pk, synth)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def full_case(orc, name, heads, windows):
    w = synth.WORKLOADS[name]
    case("full size %s, sampled heads %s" % (name, heads))
    lay, cfg, L = gpu_layer(w)
    BH = w.batch * w.n_kv_heads
    idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
    est = torch.empty(BH, w.kprime, dtype=torch.float32, device="cuda")
    L.retrieve(lay["Q"], idx, est)
    out = torch.empty_like(lay["Q"])
    L.attend(lay["Q"], lay["K"], lay["V"], idx, out)
    torch.cuda.synchronize()
    Kflat = lay["K"].reshape(BH, -1, w.d)
    # index windows of every head against the oracle's encode of those rows
    for lo, hi in windows:
        ids, nib, wq = pk.pariskv_debug_export(L.handle, lo, hi, BH)
        Kw = Kflat[:, lo:hi].float().cpu().numpy()
        for bh in range(BH):
            o_ids, o_nib, o_w = orc.encode_keys(lay["signs"], Kw[bh], w.m)
            assert np.array_equal(ids[bh], o_ids)
            assert np.array_equal(nib[bh], o_nib)
            assert np.array_equal(wq[bh], o_w)
    # whole retrieval of the sampled heads
    Kh = {bh: Kflat[bh].float().cpu().numpy() for bh in heads}
    Qh = host_f32(lay["Q"])
    with cf.ThreadPoolExecutor(len(heads)) as ex:
        enc = dict(zip(heads, ex.map(
            lambda bh: orc.encode_keys(lay["signs"], Kh[bh], w.m), heads)))
    ref = oracle_retrieve_heads(orc, w, Qh, enc, lay["signs"], heads)
    gi = gpu_intermediates(L, BH)
    ih, eh, oh = idx.cpu().numpy(), est.cpu().numpy(), host_f32(out)
    Vflat = lay["V"].reshape(BH, -1, w.d)
    for bh in heads:
        assert_retrieval_equal(w, gi, ih, eh, ref[bh], bh)
        b, h = divmod(bh, w.n_kv_heads)
        G = w.G
        rows = ih[bh]
        Ksel = Kflat[bh][torch.from_numpy(rows).long().cuda()].float().cpu().numpy()
        Vsel = Vflat[bh][torch.from_numpy(rows).long().cuda()].float().cpu().numpy()
        ref_o = orc.attention(Qh[b, h * G:(h + 1) * G], Ksel, Vsel,
                              np.arange(len(rows), dtype=np.int32), w.d ** -0.5)
        assert np.max(np.abs(oh[b, h * G:(h + 1) * G] - ref_o)) <= ATTN_TOL_BF16
    L.close()
    return w, ih, Kh, Qh


def test_llama8b_32k_all_heads(orc):
    w = synth.WORKLOADS["llama8b_32k"]
    full_case(orc, "llama8b_32k", list(range(8)), [(0, w.N)])


def test_batched_128k_sampled(orc):
    full_case(orc, "batched_128k", [0, 37, 63],
              [(0, 256), (65536, 67584), (129024, 131072)])


def test_million_sampled(orc):
    full_case(orc, "million", [0, 5],
              [(0, 512), (524288, 526336), (1046528, 1048576)])
