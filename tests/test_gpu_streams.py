"""A decode key appended on one stream and retrieved on another: the
deferred encode runs in the retrieval's first kernel on the retrieval's
stream, which the caller has ordered after the append's writes (an event
recorded on the append stream and waited for by the retrieval stream), so the
scan sees the new key.  Checked against the oracle on both retrieval paths,
with a long kernel queued on the append stream just before the key's row is
written, so an encode that did not wait for that stream would read a stale
row."""
import numpy as np
import pytest
import torch

from gpu_helpers import (assert_retrieval_equal, case, gpu_intermediates,
                         host_f32, need_gpu, oracle_encode_heads,
                         oracle_retrieve_heads, pk, synth)

pytestmark = pytest.mark.gpu

W = synth.Workload


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("path", ["pipeline", "single"])
def test_append_on_one_stream_retrieve_on_another(orc, path):
    n0, steps = 5000, 3
    total = n0 + steps
    w = W("two streams", 2, 2, 8, 128, total, "bf16", k=128, sinks=4, seed=41)
    case("append on stream A, retrieve on stream B, %s" % path)
    lay = synth.make_layer(w, "cuda", capacity=total)
    K, Q = lay["K"], lay["Q"]
    Kfinal = K.clone()
    K[:, :, n0:] = 0                   # rows written step by step on stream A
    cfg = pk.config_for(w, capacity=total)
    L = pk.Layer(cfg, lay["signs"], K, n0, k=w.k)
    L.set_path(pk.PATH_SINGLE if path == "single" else pk.PATH_PIPELINE)
    torch.cuda.synchronize()
    BH = w.batch * w.n_kv_heads
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
    est = torch.empty(BH, w.kprime, dtype=torch.float32, device="cuda")
    busy = torch.empty(4096, 4096, device="cuda")
    for t in range(steps):
        n = n0 + t + 1
        with torch.cuda.stream(a):
            busy.copy_(torch.randn(4096, 4096, device="cuda") @ busy.new_ones(4096, 4096))
            K[:, :, n - 1:n] = Kfinal[:, :, n - 1:n]
            L.append(K[:, :, n - 1:], 1, rows_per_head=total, stream=a)
            ev = torch.cuda.Event()
            ev.record(a)
        b.wait_event(ev)
        L.retrieve(Q, idx, est, stream=b)
    b.synchronize()
    a.synchronize()
    torch.cuda.synchronize()
    assert L.size == total
    Kh, Qh = host_f32(Kfinal), host_f32(Q)
    heads = list(range(BH))
    enc = oracle_encode_heads(orc, w, Kh, lay["signs"], heads, n=total)
    got = pk.pariskv_debug_export(L.handle, 0, total, BH)
    for bh in heads:
        for x, y in zip(got, enc[bh]):
            assert np.array_equal(x[bh], y), bh
    ref = oracle_retrieve_heads(orc, w, Qh, enc, lay["signs"], heads)
    gi = gpu_intermediates(L, BH)
    ih, eh = idx.cpu().numpy(), est.cpu().numpy()
    for bh in heads:
        assert_retrieval_equal(w, gi, ih, eh, ref[bh], bh)
    L.close()
