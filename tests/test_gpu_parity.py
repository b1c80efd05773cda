"""GPU parity: the HIP path, called through the C-ABI binding, against the
CPU oracle on the same seeded inputs.

Bar: bit-exact bucket ids, RSQ-IP codes, fp16 calibration bits, vote LUT,
rotated query, vote scores, candidate lists, estimates and top-k lists;
attention within 2e-2 absolute (bf16 outputs) / 1e-4 (fp32 outputs).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (ATTN_TOL_BF16, ATTN_TOL_FP32, assert_retrieval_equal,
                         case, gpu_intermediates, gpu_layer, host_f32, need_gpu,
                         oracle_encode_heads, oracle_retrieve_heads, pk, synth)

pytestmark = pytest.mark.gpu

W = synth.Workload


SMALL = {
    "tiny": synth.WORKLOADS["tiny"],
    "gqa_ragged": W("gqa ragged", 2, 2, 8, 128, 5003, "bf16", k=128, seed=11),
    "sinks": W("sinks", 1, 3, 6, 128, 7001, "bf16", cand_num=1, cand_den=10,
               k=200, sinks=64, seed=12),
    "all_selected": W("all selected", 1, 2, 2, 128, 300, "bf16", cand_num=1,
                      cand_den=1, k=300, seed=13),
    "c_equals_kprime": W("C == k'", 1, 1, 4, 128, 2000, "fp32", k=500, seed=14),
    "short": W("N < 256", 2, 1, 8, 128, 100, "bf16", cand_num=1, cand_den=10,
               k=10, seed=15),
    "one_head_many_chunks": W("1 head, 70K keys", 1, 1, 4, 128, 70001, "bf16",
                              k=700, seed=16),
    "batched_kpt2": W("64 heads, 20K keys", 8, 8, 32, 128, 20000, "bf16",
                      k=256, sinks=16, seed=17),
    # other query-side parameters: scores up to 128 and 240 (the compaction's
    # byte-wise compare path needs scores below 128), rho = 1 and 2
    "rho8_tiers8": W("rho 8, tiers 8..1", 1, 2, 8, 128, 30000, "bf16", rho=8,
                     tiers=(8, 7, 6, 5, 4, 3, 2, 1), k=512, seed=18),
    "wide_tiers": W("rho 4, tiers 15/10/5/1", 1, 2, 8, 128, 30000, "bf16",
                    tiers=(15, 10, 5, 1), cand_num=1, cand_den=10, k=512, seed=19),
    # 241 score bins and 313 chunks of 256 keys: the threshold kernel's rows
    # exceed one round of register-held loads (re-read path)
    "wide_tiers_long": W("tiers 15/10/5/1, 80K keys", 1, 1, 4, 128, 80000, "bf16",
                         tiers=(15, 10, 5, 1), k=1024, seed=37),
    "rho2": W("rho 2, tiers 2/1", 2, 2, 8, 128, 20000, "bf16", rho=2, tiers=(2, 1),
              k=300, seed=20),
    "rho1": W("rho 1", 1, 4, 4, 128, 20000, "bf16", rho=1, tiers=(1,),
              cand_num=1, cand_den=10, k=300, seed=21),
    # 32 subspaces of 4 coordinates: scores up to 128 (general compare path),
    # up to 96 (byte-wise path), and rho 8 of 16 centroids
    "m4": W("32 subspaces of 4", 2, 2, 8, 128, 20000, "bf16", B=32, k=256,
            seed=22),
    "m4_sinks_fp32": W("m 4, sinks, fp32", 1, 2, 4, 128, 9001, "fp32", B=32,
                       rho=2, tiers=(3, 1), cand_num=1, cand_den=10, k=200,
                       sinks=32, seed=23),
    "m4_rho8": W("m 4, rho 8", 1, 2, 8, 128, 30000, "bf16", B=32, rho=8,
                 tiers=(7, 6, 5, 4, 3, 2, 1, 1), k=512, seed=24),
    # one head of 100K keys at m = 4: 391 chunks of 256 keys, above the
    # fused-threshold limit, so the separate threshold and the m = 4
    # compaction that reads it
    "m4_many_chunks": W("m 4, 1 head, 100K keys", 1, 1, 4, 128, 100000, "bf16", B=32,
                        k=1024, seed=39),
    # degenerate sizes: one key to select, one eligible key, E a whole number
    # of 256-key chunks (no partial chunk) and one key more (a 1-key chunk)
    # 1600 candidates of 8000 keys: the resident single kernel near its
    # limits (8192 keys, 2048 candidates)
    "cands_1600": W("8000 keys, 20% candidates", 1, 2, 8, 128, 8000, "bf16", cand_num=1,
                    cand_den=5, k=512, seed=38),
    "kprime_one": W("k' = 1", 1, 2, 8, 128, 700, "bf16", k=33, sinks=32, seed=25),
    "e_one": W("E = 1", 1, 1, 4, 128, 17, "bf16", k=17, sinks=16, seed=26),
    "e_chunks_exact": W("E = 16 chunks", 1, 1, 4, 128, 4096, "bf16", k=64, seed=27),
    "e_chunks_plus_one": W("E = 16 chunks + 1", 1, 1, 4, 128, 4097, "bf16", k=64,
                           seed=28),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


PATHS = {"pipeline": pk.PATH_PIPELINE, "single": pk.PATH_SINGLE}


def run_case(orc, w, capacity=None, extra_rows=0, path="pipeline"):
    case("%s: batch=%d Hkv=%d Hq=%d N=%d k=%d S=%d %s, %s path" % (
        w.name, w.batch, w.n_kv_heads, w.n_q_heads, w.N, w.k, w.sinks, w.dtype, path))
    lay, cfg, L = gpu_layer(w, capacity=capacity)
    L.set_path(PATHS[path])
    assert L.path == PATHS[path]
    BH = w.batch * w.n_kv_heads
    idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
    est = torch.empty(BH, w.kprime, dtype=torch.float32, device="cuda")
    L.retrieve(lay["Q"], idx, est)
    torch.cuda.synchronize()
    return lay, cfg, L, idx, est


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name", list(SMALL))
def test_retrieve_parity_small(orc, name, path):
    """Every intermediate and output against the oracle, on the multi-kernel
    pipeline and on the single-kernel path (one block per unit)."""
    w = SMALL[name]
    lay, cfg, L, idx, est = run_case(orc, w, path=path)
    BH = w.batch * w.n_kv_heads
    ids, nib, wq = pk.pariskv_debug_export(L.handle, 0, w.N, BH, B=w.B)
    Kh = host_f32(lay["K"])
    Qh = host_f32(lay["Q"])
    heads = list(range(BH))
    enc = oracle_encode_heads(orc, w, Kh, lay["signs"], heads)
    for bh in heads:
        o_ids, o_nib, o_w = enc[bh]
        assert np.array_equal(ids[bh], o_ids), bh
        assert np.array_equal(nib[bh], o_nib), bh
        assert np.array_equal(wq[bh], o_w), bh
    ref = oracle_retrieve_heads(orc, w, Qh, enc, lay["signs"], heads)
    gi = gpu_intermediates(L, BH)
    ih, eh = idx.cpu().numpy(), est.cpu().numpy()
    for bh in heads:
        assert_retrieval_equal(w, gi, ih, eh, ref[bh], bh)
    # attention over the selected rows
    out = torch.empty_like(lay["Q"])
    L.attend(lay["Q"], lay["K"], lay["V"], idx, out)
    torch.cuda.synchronize()
    Vh = host_f32(lay["V"])
    oh = host_f32(out)
    tol = ATTN_TOL_BF16 if w.dtype == "bf16" else ATTN_TOL_FP32
    for bh in heads:
        b, h = divmod(bh, w.n_kv_heads)
        G = w.G
        ref_o = orc.attention(Qh[b, h * G:(h + 1) * G], Kh[b, h], Vh[b, h],
                              ih[bh], w.d ** -0.5)
        assert np.max(np.abs(oh[b, h * G:(h + 1) * G] - ref_o)) <= tol, bh
    L.close()


@pytest.mark.parametrize("dtype,n0,steps,B", [("bf16", 1000, [1, 7, 100, 1], 16),
                                              ("fp32", 33, [16, 1, 250], 16),
                                              ("bf16", 500, [1, 3, 60], 32)])
def test_append_equals_build(orc, dtype, n0, steps, B):
    """Appending keys in pieces encodes exactly what a one-shot build does,
    and both equal the oracle (decode keys need no re-clustering)."""
    total = n0 + sum(steps)
    w = W("append", 2, 2, 8, 128, total, dtype, B=B, k=64, seed=21)
    case("append %s n0=%d steps=%s B=%d" % (dtype, n0, steps, B))
    lay = synth.make_layer(w, "cuda", capacity=total + 5)
    cfg = pk.config_for(w, capacity=total + 5)
    full = pk.Layer(cfg, lay["signs"], lay["K"], total, k=64)
    inc = pk.Layer(cfg, lay["signs"], lay["K"], n0, k=64)
    pos = n0
    for s in steps:
        inc.append(lay["K"][:, :, pos:], s, rows_per_head=lay["K"].shape[2])
        pos += s
    assert inc.size == total
    torch.cuda.synchronize()
    BH = w.batch * w.n_kv_heads
    a = pk.pariskv_debug_export(full.handle, 0, total, BH, B=B)
    b = pk.pariskv_debug_export(inc.handle, 0, total, BH, B=B)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    enc = oracle_encode_heads(orc, w, host_f32(lay["K"]), lay["signs"],
                              list(range(BH)), n=total)
    for bh in range(BH):
        for x, y in zip(a, enc[bh]):
            assert np.array_equal(x[bh], y)


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("B", [16, 32])
def test_ties_duplicates_and_zero_keys(orc, B, path):
    """Duplicated keys tie on both the vote score and the estimate; all-zero
    keys have w = 0 and estimate 0 (and -0 vs +0 must not matter)."""
    w = W("ties", 1, 2, 4, 128, 3000, "bf16", B=B, cand_num=1, cand_den=5, k=300,
          seed=31)
    case("ties/duplicates/zero keys B=%d, %s path" % (B, path))
    lay = synth.make_layer(w, "cuda")
    K = lay["K"]
    K[:, :, 1000:1600] = K[:, :, 100:700]        # duplicates
    K[:, :, 2000:2100] = 0                        # zero keys
    K[:, :, 2100:2200] = -K[:, :, 2200:2300]      # opposite keys
    cfg = pk.config_for(w)
    L = pk.Layer(cfg, lay["signs"], K, w.N, k=w.k)
    L.set_path(PATHS[path])
    BH = 2
    idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
    est = torch.empty(BH, w.kprime, dtype=torch.float32, device="cuda")
    L.retrieve(lay["Q"], idx, est)
    torch.cuda.synchronize()
    Kh, Qh = host_f32(K), host_f32(lay["Q"])
    enc = oracle_encode_heads(orc, w, Kh, lay["signs"], [0, 1])
    ref = oracle_retrieve_heads(orc, w, Qh, enc, lay["signs"], [0, 1])
    gi = gpu_intermediates(L, BH)
    for bh in range(BH):
        assert_retrieval_equal(w, gi, idx.cpu().numpy(), est.cpu().numpy(),
                               ref[bh], bh)
    L.close()


@pytest.mark.parametrize("N,den,k,copies,path", [
    (100000, 20, 1024, 0, "pipeline"),    # 5000 candidates: 2 top-k slices, one kernel
    (40000, 5, 1024, 5000, "pipeline"),   # 2 slices, threshold bin of 5000 equal keys
    (60000, 5, 2048, 8000, "pipeline"),   # 3 slices, threshold bin of 8000 equal keys
    (80000, 5, 2048, 0, "pipeline"),      # 16000 candidates: 4 slices, the one-kernel limit
    (90000, 5, 2048, 0, "pipeline"),      # 18000 candidates: 5 slices, histogram + select
    (90000, 5, 2048, 8000, "pipeline"),   # 5 slices and the select's radix select of a tied bin
    (327680, 5, 4096, 0, "pipeline"),     # 65536 candidates: 16 slices, every row in registers
    (150000, 2, 4096, 0, "pipeline"),     # 75000 candidates: 19 slices, generic select
    (150000, 2, 4096, 8000, "pipeline"),  # 19 slices and the radix select of a tied bin
    # the single-kernel path: its top-k over 2 and 4 slices, and its radix select
    (100000, 20, 1024, 0, "single"),
    (40000, 5, 1024, 5000, "single"),
    (80000, 5, 2048, 0, "single"),
])
def test_topk_paths(orc, N, den, k, copies, path):
    """The top-k's paths: one kernel up to 4 slices of 4096 candidates, the
    histogram + select pair above that (up to 16 slices the select holds
    every histogram row in registers; above, the generic select), and a
    threshold bin holding more than 4096 members (identical keys tie exactly
    on score and estimate; the lower positions win); the single-kernel
    retrieval's own top-k up to 4 slices."""
    w = W("topk paths", 1, 1, 4, 128, N, "bf16", cand_num=1, cand_den=den, k=k,
          seed=33)
    case("top-k paths N=%d f=1/%d k=%d copies=%d, %s path" % (N, den, k, copies, path))
    lay = synth.make_layer(w, "cuda")
    K = lay["K"]
    if copies:
        # keys along the group's mean query, scaled up: the top centroid in
        # every subspace (maximal vote score) and the largest estimates
        qbar = lay["Q"][0, 0:4].float().mean(0) * 4
        K[0, 0, 1000:1000 + copies] = qbar.to(K.dtype)
    cfg = pk.config_for(w)
    L = pk.Layer(cfg, lay["signs"], K, w.N, k=w.k)
    L.set_path(PATHS[path])
    idx = torch.empty(1, w.k, dtype=torch.int32, device="cuda")
    est = torch.empty(1, w.kprime, dtype=torch.float32, device="cuda")
    L.retrieve(lay["Q"], idx, est)
    torch.cuda.synchronize()
    Kh, Qh = host_f32(K), host_f32(lay["Q"])
    enc = oracle_encode_heads(orc, w, Kh, lay["signs"], [0])
    ref = oracle_retrieve_heads(orc, w, Qh, enc, lay["signs"], [0])
    gi = gpu_intermediates(L, 1)
    assert_retrieval_equal(w, gi, idx.cpu().numpy(), est.cpu().numpy(), ref[0], 0)
    if copies:
        # the tied copies fill the top-k in position order
        assert np.array_equal(idx.cpu().numpy()[0], np.arange(1000, 1000 + w.k))
    L.close()


@pytest.mark.parametrize("dtype,B", [("bf16", 16), ("fp32", 32)])
def test_decode_steps_single_kernel(orc, dtype, B):
    """Decode steps: one key appended per (b, h) and a retrieval each step. The
    single kernel encodes the deferred key itself before scanning; its
    outputs equal the pipeline's at every step and the oracle's at the end."""
    n0, steps = 3000, 6
    total = n0 + steps
    w = W("decode steps", 2, 2, 8, 128, total, dtype, B=B, k=96, sinks=8, seed=35)
    case("decode steps %s B=%d" % (dtype, B))
    lay = synth.make_layer(w, "cuda", capacity=total + 5)
    cfg = pk.config_for(w, capacity=total + 5)
    K, Q = lay["K"], lay["Q"]
    rows = K.shape[2]
    single = pk.Layer(cfg, lay["signs"], K, n0, k=w.k)
    pipe = pk.Layer(cfg, lay["signs"], K, n0, k=w.k)
    single.set_path(pk.PATH_SINGLE)
    pipe.set_path(pk.PATH_PIPELINE)
    BH = w.batch * w.n_kv_heads
    for t in range(steps):
        outs = []
        for L in (single, pipe):
            L.append(K[:, :, n0 + t:], 1, rows_per_head=rows)
            idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
            est = torch.empty(BH, w.kprime, dtype=torch.float32, device="cuda")
            L.retrieve(Q, idx, est)
            torch.cuda.synchronize()
            outs.append((idx.cpu().numpy(), est.cpu().numpy().view(np.uint32)))
        assert np.array_equal(outs[0][0], outs[1][0]), t
        assert np.array_equal(outs[0][1], outs[1][1]), t
    assert single.size == total
    Kh, Qh = host_f32(K), host_f32(Q)
    heads = list(range(BH))
    enc = oracle_encode_heads(orc, w, Kh, lay["signs"], heads, n=total)
    ref = oracle_retrieve_heads(orc, w, Qh, enc, lay["signs"], heads)
    a = pk.pariskv_debug_export(single.handle, 0, total, BH, B=B)
    gi = gpu_intermediates(single, BH)
    for bh in heads:
        for x, y in zip(a, enc[bh]):
            assert np.array_equal(x[bh], y), bh
        assert_retrieval_equal(w, gi, outs[0][0], outs[0][1].view(np.float32), ref[bh], bh)
    single.close()
    pipe.close()


def test_deterministic_repeat():
    w = SMALL["batched_kpt2"]
    case("determinism")
    lay, cfg, L = gpu_layer(w)
    BH = w.batch * w.n_kv_heads
    outs = []
    for _ in range(3):
        idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
        est = torch.empty(BH, w.kprime, dtype=torch.float32, device="cuda")
        L.retrieve(lay["Q"], idx, est)
        outs.append((idx.cpu().numpy(), est.cpu().numpy().view(np.uint32)))
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0])
        assert np.array_equal(o[1], outs[0][1])
    L.close()


@pytest.mark.parametrize("G,dtype,k,N", [(1, "fp32", 77, 500), (2, "bf16", 64, 64),
                                         (4, "bf16", 1000, 3000),
                                         (8, "bf16", 129, 4096),
                                         (4, "bf16", 4096, 4096)])
def test_attention_dense_and_sparse(orc, G, dtype, k, N):
    """Split-K attention vs fp64 softmax attention; k = N is full attention."""
    case("attention G=%d %s k=%d N=%d" % (G, dtype, k, N))
    Hkv, B = 2, 2
    w = W("attn", B, Hkv, Hkv * G, 128, N, dtype, k=k, seed=41)
    lay = synth.make_layer(w, "cuda")
    gen = torch.Generator(device="cpu").manual_seed(5)
    idx = torch.stack([torch.sort(torch.randperm(N, generator=gen)[:k]).values
                       for _ in range(B * Hkv)]).to(torch.int32).cuda()
    ws = torch.empty(pk.pariskv_attn_workspace_bytes(B, Hkv * G, k, 128),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(lay["Q"])
    pk.pariskv_sparse_attn(lay["Q"], lay["K"], lay["V"], N, idx, k, B, Hkv * G,
                           Hkv, 128, pk.PARISKV_DTYPE_BF16 if dtype == "bf16"
                           else pk.PARISKV_DTYPE_FP32, 128 ** -0.5, out, ws)
    torch.cuda.synchronize()
    Qh, Kh, Vh = host_f32(lay["Q"]), host_f32(lay["K"]), host_f32(lay["V"])
    ih, oh = idx.cpu().numpy(), host_f32(out)
    tol = ATTN_TOL_BF16 if dtype == "bf16" else ATTN_TOL_FP32
    for bh in range(B * Hkv):
        b, h = divmod(bh, Hkv)
        ref = orc.attention(Qh[b, h * G:(h + 1) * G], Kh[b, h], Vh[b, h], ih[bh],
                            128 ** -0.5)
        assert np.max(np.abs(oh[b, h * G:(h + 1) * G] - ref)) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_attention_large_grid(orc, dtype):
    """The attention's other launch shapes: 16 x 8 KV heads with k = 512 make
    1024 blocks of 64-row chunks (the split's 4-rows-per-lane form) and 512
    (b, query head) pairs (the one-block merge); sampled heads against fp64
    softmax attention."""
    B, Hkv, G, k, N = 16, 8, 4, 512, 2048
    case("attention large grid %s B=%d Hkv=%d G=%d k=%d N=%d" % (dtype, B, Hkv, G, k, N))
    w = W("attn grid", B, Hkv, Hkv * G, 128, N, dtype, k=k, seed=43)
    lay = synth.make_layer(w, "cuda")
    gen = torch.Generator(device="cpu").manual_seed(7)
    idx = torch.stack([torch.sort(torch.randperm(N, generator=gen)[:k]).values
                       for _ in range(B * Hkv)]).to(torch.int32).cuda()
    ws = torch.empty(pk.pariskv_attn_workspace_bytes(B, Hkv * G, k, 128),
                     dtype=torch.uint8, device="cuda")
    out = torch.full_like(lay["Q"], float("nan"))
    pk.pariskv_sparse_attn(lay["Q"], lay["K"], lay["V"], N, idx, k, B, Hkv * G,
                           Hkv, 128, pk.PARISKV_DTYPE_BF16 if dtype == "bf16"
                           else pk.PARISKV_DTYPE_FP32, 128 ** -0.5, out, ws)
    torch.cuda.synchronize()
    Qh, Kh, Vh = host_f32(lay["Q"]), host_f32(lay["K"]), host_f32(lay["V"])
    ih, oh = idx.cpu().numpy(), host_f32(out)
    assert not np.isnan(oh).any()
    tol = ATTN_TOL_BF16 if dtype == "bf16" else ATTN_TOL_FP32
    for bh in (0, 37, 64, 127):
        b, h = divmod(bh, Hkv)
        ref = orc.attention(Qh[b, h * G:(h + 1) * G], Kh[b, h], Vh[b, h], ih[bh],
                            128 ** -0.5)
        assert np.max(np.abs(oh[b, h * G:(h + 1) * G] - ref)) <= tol


def test_append_to_capacity(orc):
    """Appends fill the index exactly to its capacity (then one more key is
    refused on the host); the full index retrieves as the oracle does."""
    N0, cap = 3000, 3040
    w = W("append to capacity", 1, 2, 8, 128, cap, "bf16", k=100, sinks=4, seed=29)
    case("append to capacity N0=%d cap=%d" % (N0, cap))
    lay = synth.make_layer(w, "cuda")
    cfg = pk.config_for(w, capacity=cap)
    L = pk.Layer(cfg, lay["signs"], lay["K"], N0, k=w.k)
    L.append(lay["K"][:, :, N0:], cap - N0 - 1, rows_per_head=cap)
    L.append(lay["K"][:, :, cap - 1:], 1, rows_per_head=cap)
    assert L.size == cap
    with pytest.raises(pk.PariskvError):
        L.append(lay["K"][:, :, cap - 1:], 1, rows_per_head=cap)
    BH = w.batch * w.n_kv_heads
    idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
    est = torch.empty(BH, w.kprime, dtype=torch.float32, device="cuda")
    L.retrieve(lay["Q"], idx, est)
    torch.cuda.synchronize()
    Kh, Qh = host_f32(lay["K"]), host_f32(lay["Q"])
    enc = oracle_encode_heads(orc, w, Kh, lay["signs"], list(range(BH)))
    ref = oracle_retrieve_heads(orc, w, Qh, enc, lay["signs"], list(range(BH)))
    gi = gpu_intermediates(L, BH)
    for bh in range(BH):
        assert_retrieval_equal(w, gi, idx.cpu().numpy(), est.cpu().numpy(), ref[bh], bh)
    L.close()
