"""Decode steps captured into a HIP graph: the benchmark's timed region
replays such a graph (per step: one appended key per (b, h), a retrieval and
the sparse attention). Each replay must give, bit for bit, the outputs of the
same steps launched eagerly on an identical index, also with eager work and
synchronizations between the replays. (The eager path itself is checked
against the oracle by the parity tests.)"""
import numpy as np
import pytest
import torch

from gpu_helpers import case, need_gpu, pk, synth

pytestmark = pytest.mark.gpu

W = synth.Workload

CASES = {
    # more than 256 chunks of 2048 keys per unit: the separate threshold
    # kernel, as on the million-token layer
    "chunks_293": (W("8 heads x 600K", 1, 8, 32, 128, 600000, "bf16", k=1024, seed=41),
                   "pipeline"),
    # few chunks: the threshold found inside the compaction
    "fused_threshold": (W("4 heads x 20K", 2, 2, 8, 128, 20000, "bf16", k=256, sinks=16,
                          seed=42), "pipeline"),
    # the single-kernel retrieval (resident variant for these sizes)
    "single_kernel": (W("2 heads x 6K", 1, 2, 8, 128, 6000, "bf16", k=128, seed=43),
                      "single"),
    # unshared retrieval: one unit per query head, the grouped scan
    "per_query_head": (W("per query head, 2 x 4 heads x 30K", 1, 2, 8, 128, 30000, "bf16",
                         k=256, per_query_head=True, seed=44), "pipeline"),
    # the Self-Indexing index and its retrieval
    "self_indexing": (W("Self-Indexing, 4 heads x 100K", 1, 4, 16, 128, 100000, "bf16",
                        k=512, sinks=16, seed=45), "si"),
}
STEPS = 4
REPLAYS = 3


def run_steps(L, lay, Qs, n0, idx_bufs, out_bufs, scale):
    K, V = lay["K"], lay["V"]
    rows = K.shape[2]
    for t in range(len(Qs)):
        L.append(K[:, :, n0 + t:], 1, rows_per_head=rows)
        L.retrieve(Qs[t], idx_bufs[t])
        L.attend(Qs[t], K, V, idx_bufs[t], out_bufs[t], scale)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_eager(name):
    need_gpu()
    w, path = CASES[name]
    case("graph %s (%s)" % (name, path))
    n0 = w.N - STEPS
    lay = synth.make_layer(w, "cuda", capacity=w.N + 8)
    cfg = pk.config_for(w, capacity=w.N + 8)
    # per-step queries: the layer's query plus a seeded perturbation
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    Q = lay["Q"]
    Qs = [(Q.float() + 0.05 * torch.randn(Q.shape, generator=g, device="cuda")).to(Q.dtype)
          for _ in range(STEPS)]
    U = w.batch * (w.n_q_heads if w.per_query_head else w.n_kv_heads)
    scale = w.d ** -0.5

    def new_layer():
        if path == "si":
            return pk.SiLayer(pk.si_config_for(w, capacity=w.N + 8), lay["K"], n0, k=w.k)
        L = pk.Layer(cfg, lay["signs"], lay["K"], n0, k=w.k)
        L.set_path(pk.PATH_SINGLE if path == "single" else pk.PATH_PIPELINE)
        return L

    # eager reference on one index
    A = new_layer()
    idx_e = [torch.empty(U, w.k, dtype=torch.int32, device="cuda") for _ in range(STEPS)]
    out_e = [torch.empty_like(Q) for _ in range(STEPS)]
    run_steps(A, lay, Qs, n0, idx_e, out_e, scale)
    torch.cuda.synchronize()
    ref_idx = [x.cpu().numpy() for x in idx_e]
    ref_out = [x.view(torch.int16).cpu().numpy() for x in out_e]

    # the same steps captured on an identical index
    B = new_layer()
    idx_g = [torch.empty(U, w.k, dtype=torch.int32, device="cuda") for _ in range(STEPS)]
    out_g = [torch.empty_like(Q) for _ in range(STEPS)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        run_steps(B, lay, Qs, n0, idx_g, out_g, scale)
    torch.cuda.synchronize()
    assert B.size == A.size == w.N

    scratch_idx = torch.empty(U, w.k, dtype=torch.int32, device="cuda")
    scratch_out = torch.empty_like(Q)
    for r in range(REPLAYS):
        for x in idx_g + out_g:
            x.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for t in range(STEPS):
            assert np.array_equal(idx_g[t].cpu().numpy(), ref_idx[t]), (name, r, t)
            assert np.array_equal(out_g[t].view(torch.int16).cpu().numpy(), ref_out[t]), \
                (name, r, t)
        # eager work between replays: the last step's retrieval and attention
        # again on the reference index (it holds the same keys as then),
        # torch kernels, and a synchronization
        A.retrieve(Qs[-1], scratch_idx)
        A.attend(Qs[-1], lay["K"], lay["V"], scratch_idx, scratch_out, scale)
        _ = (torch.randn(1 << 20, device="cuda") * 2.0).sum().item()
        torch.cuda.synchronize()
        assert np.array_equal(scratch_idx.cpu().numpy(), ref_idx[-1]), (name, r)
        assert np.array_equal(scratch_out.view(torch.int16).cpu().numpy(), ref_out[-1]), \
            (name, r)
    del graph
    A.close()
    B.close()
