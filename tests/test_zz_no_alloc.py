"""The retrieval entry point that allocates nothing
(pariskv_retrieve_topk_noalloc, for callers that cannot allocate device
memory) against pariskv_retrieve_topk with a caller workspace: the same
top-k positions and estimates, bit for bit, on two calls in a row, the
second on a smaller index, smaller k and fewer heads (the shared scratch
keeps the first call's contents), on both retrieval paths; and a request
beyond the scratch is refused."""
import numpy as np
import pytest
import torch

from gpu_helpers import case, gpu_layer, need_gpu, pk, synth

pytestmark = pytest.mark.gpu

W = synth.Workload


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def both(w, path):
    lay, cfg, L = gpu_layer(w)
    L.set_path(pk.PATH_SINGLE if path == "single" else pk.PATH_PIPELINE)
    BH = w.batch * w.n_kv_heads
    out = []
    for fn in ("ws", "noalloc"):
        idx = torch.full((BH, w.k), -1, dtype=torch.int32, device="cuda")
        est = torch.full((BH, w.kprime), float("nan"), dtype=torch.float32, device="cuda")
        if fn == "ws":
            L.retrieve(lay["Q"], idx, est)
        else:
            pk.pariskv_retrieve_topk_noalloc(L.handle, lay["Q"], w.k, idx, est)
        torch.cuda.synchronize()
        out.append((idx.cpu().numpy(), est.cpu().numpy().view(np.uint32)))
    L.close()
    return out


@pytest.mark.parametrize("path", ["pipeline", "single"])
def test_noalloc_equals_workspace_entry_point(path):
    big = W("noalloc big", 2, 4, 16, 128, 60000 if path == "pipeline" else 9000, "bf16",
            k=512, sinks=8, seed=91)
    small = W("noalloc small", 1, 2, 4, 128, 3001, "bf16", k=64, seed=92)
    for w in (big, small):
        case("noalloc %s: batch=%d Hkv=%d N=%d k=%d" % (path, w.batch, w.n_kv_heads, w.N, w.k))
        (i0, e0), (i1, e1) = both(w, path)
        assert np.array_equal(i0, i1)
        assert np.array_equal(e0, e1)
        assert (i0 >= 0).all()


def test_noalloc_refuses_beyond_its_scratch():
    # 64 retrieval units (per query head) over 300K-key capacity: the
    # workspace is about 57 MiB, more than the 32 MiB scratch
    w = W("noalloc over", 1, 8, 64, 128, 1000, "bf16", k=512, per_query_head=True, seed=93)
    case("noalloc refusal")
    cfg = pk.config_for(w, capacity=300000)
    assert pk.pariskv_retrieve_workspace_bytes(cfg, w.k) > pk.NOALLOC_SCRATCH_BYTES
    lay = synth.make_layer(w, "cuda")
    L = pk.Layer(cfg, lay["signs"], lay["K"], w.N, k=w.k)
    idx = torch.empty(w.batch * w.n_q_heads, w.k, dtype=torch.int32, device="cuda")
    with pytest.raises(pk.PariskvError) as ei:
        pk.pariskv_retrieve_topk_noalloc(L.handle, lay["Q"], w.k, idx, None)
    assert ei.value.rc == pk.PARISKV_ERR_WORKSPACE
    L.close()
