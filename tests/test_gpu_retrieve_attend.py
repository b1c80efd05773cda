"""Retrieval and sparse attention in one call (pariskv_retrieve_attend) on
the GPU: the selection equals the oracle's bit for bit (top-k positions and
their estimates, through the one-kernel top-k and the histogram + select
pair), the attention over the selected rows is within the bf16 / fp32 bar of
the oracle's, and every output equals that of the separate
pariskv_retrieve_topk + pariskv_sparse_attn calls bit for bit.  Shapes: the
query-group sizes 1, 2, 4 and 8, sinks, per-query-head retrieval, fp32, ties
filling the top-k, and many top-k slices."""
import numpy as np
import pytest
import torch

from gpu_helpers import (ATTN_TOL_BF16, ATTN_TOL_FP32, case, host_f32, need_gpu,
                         oracle_encode_heads, oracle_retrieve_heads, pk, synth)

pytestmark = pytest.mark.gpu

W = synth.Workload

CASES = {
    # name: (workload, tied copies of a key along the group's mean query)
    "g4_sinks": (W("g4 sinks", 2, 2, 8, 128, 30000, "bf16", k=512, sinks=64, seed=101), 0),
    "g1_fp32": (W("g1 fp32", 1, 3, 3, 128, 9000, "fp32", k=200, sinks=5, seed=102), 0),
    "g2": (W("g2", 1, 4, 8, 128, 20000, "bf16", k=300, seed=103), 0),
    "g8_separate": (W("g8", 1, 2, 16, 128, 20000, "bf16", k=300, seed=104), 0),
    "per_query_head": (W("per query head", 1, 2, 8, 128, 12000, "bf16", k=256, sinks=8,
                         per_query_head=True, seed=105), 0),
    # 60000 candidates: 15 top-k slices
    "many_slices": (W("1 head, 300K keys, 20%", 1, 1, 4, 128, 300000, "bf16", cand_num=1,
                      cand_den=5, k=4096, seed=106), 0),
    # 75000 candidates: 19 top-k slices
    "beyond_one_kernel": (W("1 head, 150K keys, 50%", 1, 1, 4, 128, 150000, "bf16",
                            cand_num=1, cand_den=2, k=2048, seed=107), 0),
    "tied_copies": (W("ties", 1, 1, 4, 128, 40000, "bf16", cand_num=1, cand_den=5, k=1024,
                      seed=108), 5000),
    "tiny_k": (W("k = S + 1", 1, 2, 8, 128, 3000, "bf16", k=17, sinks=16, seed=109), 0),
    # k = 64, two 32-row chunks: a partial buffer of 1056 bytes, not the
    # 256-byte multiple the attention's workspace size is rounded to
    "one_chunk": (W("one chunk", 1, 1, 1, 128, 4096, "fp32", cand_num=1, cand_den=10, k=64,
                    seed=110), 0),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("name", list(CASES))
def test_retrieve_attend(orc, name):
    w, copies = CASES[name]
    case("retrieve+attend %s: batch=%d Hkv=%d Hq=%d N=%d k=%d S=%d %s" % (
        name, w.batch, w.n_kv_heads, w.n_q_heads, w.N, w.k, w.sinks, w.dtype))
    lay = synth.make_layer(w, "cuda")
    K, V, Q = lay["K"], lay["V"], lay["Q"]
    if copies:
        qbar = Q[0, 0:w.G].float().mean(0) * 4
        K[0, 0, 1000:1000 + copies] = qbar.to(K.dtype)
    cfg = pk.config_for(w)
    L = pk.Layer(cfg, lay["signs"], K, w.N, k=w.k)
    U = w.batch * (w.n_q_heads if w.per_query_head else w.n_kv_heads)
    idx = torch.full((U, w.k), -1, dtype=torch.int32, device="cuda")
    est = torch.full((U, w.kprime), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full_like(Q, float("nan"))
    L.retrieve_attend(Q, K, V, idx, out, est)
    idx2 = torch.full_like(idx, -1)
    est2 = torch.full_like(est, float("nan"))
    out2 = torch.full_like(out, float("nan"))
    L.retrieve(Q, idx2, est2)
    L.attend(Q, K, V, idx2, out2)
    torch.cuda.synchronize()
    ih, eh, oh = idx.cpu().numpy(), est.cpu().numpy(), host_f32(out)
    assert np.array_equal(ih, idx2.cpu().numpy())
    assert np.array_equal(eh.view(np.uint32), est2.cpu().numpy().view(np.uint32))
    tol = ATTN_TOL_BF16 if w.dtype == "bf16" else ATTN_TOL_FP32
    assert np.array_equal(out.cpu().view(torch.int16 if w.dtype == "bf16" else torch.int32),
                          out2.cpu().view(torch.int16 if w.dtype == "bf16" else torch.int32))
    Kh, Vh, Qh = host_f32(K), host_f32(V), host_f32(Q)
    G = w.G
    units = range(U) if U <= 8 else (0, U // 2, U - 1)
    if w.per_query_head:
        for u in units:
            b, hq = divmod(u, w.n_q_heads)
            h = hq // G
            ids, nib, wq = orc.encode_keys(lay["signs"], Kh[b, h], w.m)
            ref = orc.retrieve_head(lay["signs"], Qh[b, hq:hq + 1], ids, nib, wq, m=w.m,
                                    rho=w.rho, tiers=w.tiers, S=w.sinks, k=w.k,
                                    num=w.cand_num, den=w.cand_den)
            assert np.array_equal(ih[u], ref["idx"]), u
            ref_o = orc.attention(Qh[b, hq:hq + 1], Kh[b, h], Vh[b, h], ref["idx"],
                                  w.d ** -0.5)
            assert np.max(np.abs(oh[b, hq:hq + 1] - ref_o)) <= tol, u
        L.close()
        return
    enc = oracle_encode_heads(orc, w, Kh, lay["signs"], list(units))
    ref = oracle_retrieve_heads(orc, w, Qh, enc, lay["signs"], list(units))
    for u in units:
        r = ref[u]
        assert np.array_equal(ih[u], r["idx"]), u
        pos = np.searchsorted(r["cand"], ih[u][w.sinks:])
        assert np.array_equal(eh[u].view(np.uint32), r["est"][pos].view(np.uint32)), u
        b, h = divmod(u, w.n_kv_heads)
        ref_o = orc.attention(Qh[b, h * G:(h + 1) * G], Kh[b, h], Vh[b, h], r["idx"],
                              w.d ** -0.5)
        assert np.max(np.abs(oh[b, h * G:(h + 1) * G] - ref_o)) <= tol, u
    if copies:
        assert np.array_equal(ih[0], np.arange(1000, 1000 + w.k))
    L.close()
