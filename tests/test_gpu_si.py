"""Self-Indexing workload ("Self-Indexing KVCache: Predicting Sparse
Attention from Compressed Keys", Methodology A-C) on the GPU against the
oracle: means, centroids, sign ids and the LUT bit-exact (both sides
accumulate the build in fp64 and round once to fp32; the LUT follows one
stated fp32 order), attention over the selection within the bf16 bar.

Scores: the oracle sums a key's 32 LUT entries in sub-vector order, the
kernel sums them in byte pairs (the order of its byte-indexed table).  Any
fp32 summation of n terms lies within gamma_{n-1} * sum|terms| of the exact
sum (Higham, Accuracy and Stability, 4.2), so the two differ by at most
tol = 2 gamma_31 sum|terms| per key, which the tests assert.  The top-k
then agrees except across the selection boundary: a key the GPU took and
the oracle did not (e) and one the oracle took and the GPU did not (m) are
allowed only when o_m - o_e <= tol_e + tol_m (GPU order puts e first, so
g_e >= g_m), and every such pair is reported."""
import numpy as np
import pytest
import torch

U32 = 2.0 ** -24
GAMMA31 = 31 * U32 / (1 - 31 * U32)

from gpu_helpers import ATTN_TOL_BF16, ATTN_TOL_FP32, case, host_f32, need_gpu, pk, synth

pytestmark = pytest.mark.gpu

W = synth.Workload

CASES = {
    # name: (workload, prefill keys, appended key counts)
    "gqa": (W("si gqa", 2, 2, 8, 128, 5003, "bf16", k=128, seed=81), 4990, [1, 12]),
    "sinks": (W("si sinks", 1, 3, 6, 128, 7001, "bf16", k=200, sinks=64, seed=82), 7001, []),
    "fp32_g1": (W("si fp32", 1, 2, 2, 128, 3001, "fp32", k=100, seed=83), 2900, [101]),
    # 8 heads x 140K keys: 2048-key chunks, candidates over several top-k slices
    "long": (W("si 8 x 140K", 1, 8, 32, 128, 140000, "bf16", k=1024, sinks=16, seed=84),
             139990, [10]),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def run_si(orc, w, n0, appends, K=None):
    N = n0 + sum(appends)
    assert N == w.N
    lay = synth.make_layer(w, "cuda")
    if K is not None:
        lay["K"] = K
    K, V, Q = lay["K"], lay["V"], lay["Q"]
    cfg = pk.si_config_for(w)
    L = pk.SiLayer(cfg, K, n0, k=w.k)
    for s in appends:
        L.append(K[:, :, L.size:], s, rows_per_head=w.N)
    assert L.size == N
    BH = w.batch * w.n_kv_heads
    idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
    sc = torch.empty(BH, w.k - w.sinks, dtype=torch.float32, device="cuda")
    L.retrieve(Q, idx, sc)
    out = torch.empty_like(Q)
    L.attend(Q, K, V, idx, out)
    torch.cuda.synchronize()
    E = N - w.sinks
    g = dict(
        export=pk.pariskv_si_debug_export(L.handle, 0, N, BH),
        lut=pk.pariskv_si_debug_intermediate(L.handle, w.k, L.ws, pk.SI_DEBUG_LUT, BH, E),
        scores=pk.pariskv_si_debug_intermediate(L.handle, w.k, L.ws, pk.SI_DEBUG_SCORES, BH, E),
        meta=pk.pariskv_si_debug_intermediate(L.handle, w.k, L.ws, pk.SI_DEBUG_META, BH, E),
        idx=idx.cpu().numpy(), sc=sc.cpu().numpy(), out=host_f32(out))
    L.close()
    return lay, g


def check_head(orc, w, n0, lay, g, bh, Kh, Qh, Vh):
    ids, mean, cb = g["export"]
    b, h = divmod(bh, w.n_kv_heads)
    G, S = w.G, w.sinks
    m_o, ids_o, cb_o = orc.si_build(Kh[b, h, :n0], S)
    if w.N > n0:
        ids_o = np.concatenate([ids_o, orc.si_ids(Kh[b, h, n0:w.N], m_o)])
    assert np.array_equal(mean[bh].view(np.uint32), m_o.view(np.uint32)), bh
    assert np.array_equal(cb[bh].view(np.uint32), cb_o.view(np.uint32)), bh
    assert np.array_equal(ids[bh], ids_o), bh
    ref = orc.si_retrieve_head(Qh[b, h * G:(h + 1) * G], ids_o, cb_o, S=S, k=w.k)
    assert np.array_equal(g["lut"][bh].view(np.uint32), ref["lut"].view(np.uint32)), bh
    # per-key bound on |kernel score - oracle score| from the LUT terms
    lut64 = ref["lut"].astype(np.float64)
    B = lut64.shape[0]
    terms = np.abs(lut64[np.arange(B)[None], ids_o[S:].astype(np.int64)])
    tol = 2 * GAMMA31 * terms.sum(axis=1)
    o = ref["scores"].astype(np.float64)
    gsc = g["scores"][bh].astype(np.float64)
    assert np.all(np.abs(gsc - o) <= tol), (bh, float(np.max(np.abs(gsc - o) - tol)))
    gi, oi = g["idx"][bh], ref["idx"]
    # the selection is exact for the kernel's own scores: (score desc, position asc)
    own = np.sort(np.lexsort((np.arange(len(gsc)), -g["scores"][bh]))[:w.k - S] + S)
    assert np.array_equal(gi, np.concatenate([np.arange(S), own])), bh
    extra = np.setdiff1d(gi[S:], oi[S:]) - S
    miss = np.setdiff1d(oi[S:], gi[S:]) - S
    assert len(extra) == len(miss), bh
    for e in extra:
        for m in miss:
            assert o[m] - o[e] <= tol[e] + tol[m], (bh, e + S, m + S)
    if len(extra):
        case("head %d: %d boundary swaps within tolerance: %s" % (
            bh, len(extra), ", ".join("%d<->%d (oracle %.9g vs %.9g)" % (
                e + S, m + S, o[e], o[m]) for e, m in zip(extra, miss))))
    # scores reported for the selection, aligned with idx[S:]
    gs = g["sc"][bh].astype(np.float64)
    assert np.all(np.abs(gs - o[gi[S:] - S]) <= tol[gi[S:] - S]), bh
    T, gt, eq, Cn = g["meta"][bh]
    assert gt + eq == Cn and gt < w.k - S <= Cn
    atol = ATTN_TOL_BF16 if w.dtype == "bf16" else ATTN_TOL_FP32
    ref_o = orc.attention(Qh[b, h * G:(h + 1) * G], Kh[b, h], Vh[b, h], g["idx"][bh],
                          w.d ** -0.5)
    assert np.max(np.abs(g["out"][b, h * G:(h + 1) * G] - ref_o)) <= atol, bh


@pytest.mark.parametrize("name", list(CASES))
def test_si_parity(orc, name):
    w, n0, appends = CASES[name]
    case("%s: batch=%d Hkv=%d Hq=%d N=%d (prefill %d) k=%d S=%d %s" % (
        w.name, w.batch, w.n_kv_heads, w.n_q_heads, w.N, n0, w.k, w.sinks, w.dtype))
    lay, g = run_si(orc, w, n0, appends)
    Kh, Qh, Vh = host_f32(lay["K"]), host_f32(lay["Q"]), host_f32(lay["V"])
    BH = w.batch * w.n_kv_heads
    heads = range(BH) if BH <= 8 else (0, BH // 2, BH - 1)
    for bh in heads:
        check_head(orc, w, n0, lay, g, bh, Kh, Qh, Vh)


def test_si_all_scores_tied(orc):
    """Every non-sink key identical: every score ties, the threshold bin holds
    all of them (more than one top-k block ranks pairwise), and the selection
    is the k' lowest positions."""
    w = W("si ties", 1, 2, 4, 128, 20000, "bf16", k=300, sinks=8, seed=85)
    case("all scores tied, N=%d k=%d" % (w.N, w.k))
    lay = synth.make_layer(w, "cuda")
    K = lay["K"]
    K[:, :, w.sinks:] = K[:, :, w.sinks:w.sinks + 1]
    lay2, g = run_si(orc, w, w.N, [], K=K)
    Kh, Qh, Vh = host_f32(K), host_f32(lay2["Q"]), host_f32(lay2["V"])
    for bh in range(2):
        check_head(orc, w, w.N, lay2, g, bh, Kh, Qh, Vh)
        assert np.array_equal(g["idx"][bh], np.arange(w.k))
