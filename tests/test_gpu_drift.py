"""Long-generation drift on the GPU against the oracle ("Technical Summary:
ParisKV", Problem Statement 2 "Decoding Drift" and Core Algorithmic
Innovations 1 "Analytic Centroids"): after a prefill, every decode step
appends one key per (b, h) whose channel mean has moved further along 16
channels, and retrieves with a query from the same moved distribution.  The
centroids are data-independent, so the appended keys are encoded with no
re-clustering; at checkpoints along the drift the index (ids, codes and w of
every key, prefill and appended), the retrieval (vote table, yq, scores,
candidates, estimates, top-k) and the attention over the selection are
compared with the oracle.  The drift workload's recipe at reduced size:
batch 2, 4 KV heads, 4 query heads each, bf16, 8192 prefill keys, T = 64
steps, so step T reaches the full +1.5 sigma shift, k = 256."""
import numpy as np
import pytest
import torch

from gpu_helpers import (ATTN_TOL_BF16, assert_retrieval_equal, case,
                         gpu_intermediates, host_f32, need_gpu,
                         oracle_encode_heads, oracle_retrieve_heads, pk, synth)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("path", ["pipeline", "single"])
def test_drift_steps_match_oracle(orc, path):
    T, n0 = 64, 8192
    w = synth.WORKLOADS["drift"].scaled(batch=2, n_kv_heads=4, n_q_heads=16, N=n0, k=256,
                                        decode_steps=T)
    case("drift %s: batch=%d Hkv=%d Hq=%d prefill=%d steps=%d k=%d" % (
        path, w.batch, w.n_kv_heads, w.n_q_heads, n0, T, w.k))
    cap = n0 + T
    lay = synth.make_layer(w, "cuda", capacity=cap)
    K, V = lay["K"], lay["V"]
    chans = synth.drift_channels(w)
    cfg = pk.config_for(w, capacity=cap)
    L = pk.Layer(cfg, lay["signs"], K, n0, k=w.k)
    L.set_path(pk.PATH_SINGLE if path == "single" else pk.PATH_PIPELINE)
    BH = w.batch * w.n_kv_heads
    idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
    est = torch.empty(BH, w.kprime, dtype=torch.float32, device="cuda")
    heads = list(range(BH))
    checks = 0
    for t in range(1, T + 1):
        knew, Q, vnew = synth.drift_step(w, t, lay["scales"], chans, "cuda")
        n = n0 + t
        K[:, :, n - 1:n] = knew
        V[:, :, n - 1:n] = vnew
        L.append(K[:, :, n - 1:], 1, rows_per_head=cap)
        L.retrieve(Q, idx, est)
        out = torch.empty_like(Q)
        L.attend(Q, K, V, idx, out)
        if t not in (1, 16, 40, T):
            continue
        checks += 1
        torch.cuda.synchronize()
        wn = w.scaled(N=n)
        Kh, Vh, Qh = host_f32(K), host_f32(V), host_f32(Q)
        enc = oracle_encode_heads(orc, wn, Kh, lay["signs"], heads, n=n)
        got = pk.pariskv_debug_export(L.handle, 0, n, BH)
        for bh in heads:
            for x, y in zip(got, enc[bh]):
                assert np.array_equal(x[bh], y), (t, bh)
        ref = oracle_retrieve_heads(orc, wn, Qh, enc, lay["signs"], heads)
        gi = gpu_intermediates(L, BH)
        ih, eh, oh = idx.cpu().numpy(), est.cpu().numpy(), host_f32(out)
        G = w.G
        for bh in heads:
            assert_retrieval_equal(wn, gi, ih, eh, ref[bh], bh)
            b, h = divmod(bh, w.n_kv_heads)
            ref_o = orc.attention(Qh[b, h * G:(h + 1) * G], Kh[b, h], Vh[b, h], ih[bh],
                                  w.d ** -0.5)
            assert np.max(np.abs(oh[b, h * G:(h + 1) * G] - ref_o)) <= ATTN_TOL_BF16, (t, bh)
        # the drifted keys sit on their channels' shifted means: the last
        # key's drift channels average well above zero in units of s
        if t == T:
            s = lay["scales"].numpy()
            for bh in heads:
                b, h = divmod(bh, w.n_kv_heads)
                z = Kh[b, h, n0:n][:, chans[b, h]] / s[h, chans[b, h]]
                assert z[-16:].mean() > 0.75
    assert checks == 4
    L.close()
