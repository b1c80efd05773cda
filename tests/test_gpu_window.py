"""Sliding-window regions ("Technical Summary: ParisKV", System-Level
Innovations 2): sinks, retrieval region (indexed, rows in a far store), local
tokens and an update buffer in a near-store ring; a full buffer moves the
oldest local tokens into the retrieval region.  Checked against the oracle on
the logical key/value sequence: the index holds exactly the encoded keys
[0, S + R), retrieval equals the oracle's over that prefix, and attention
equals the oracle's over the retrieved rows plus every local and buffer
token."""
import numpy as np
import pytest
import torch

from gpu_helpers import (ATTN_TOL_BF16, assert_retrieval_equal, case,
                         gpu_intermediates, host_f32, need_gpu,
                         oracle_encode_heads, oracle_retrieve_heads, pk, synth)

pytestmark = pytest.mark.gpu

W = synth.Workload


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


# (far store, prefill tokens N0).  With N0 = 2000 the retrieval region starts
# at R0 = 1920, a multiple of the ring (96 slots), so every promotion takes
# contiguous slots; with N0 = 2013, R0 = 1933 and the third promotion (step
# 95) takes slots 77..95 and then 0..12 of the ring.
@pytest.mark.parametrize("far,N0", [("device", 2000), ("host", 2000), ("device", 2013)])
def test_window_sequence(orc, far, N0):
    S, L, U = 16, 64, 32
    B, Hkv, G, d = 1, 2, 4, 128
    steps, k = 100, 160
    cap = N0 + steps + 64
    w = W("window", B, Hkv, Hkv * G, d, cap, "bf16", k=k, sinks=S, seed=61)
    case("window S=%d L=%d U=%d N0=%d far store in %s memory" % (S, L, U, N0, far))
    lay = synth.make_layer(w, "cuda")
    K, V, Q = lay["K"], lay["V"], lay["Q"]        # logical rows, position p at row p
    BH = B * Hkv
    ring = L + U
    R0 = N0 - L - S
    cfg = pk.config_for(w, capacity=cap)
    Lx = pk.Layer(cfg, lay["signs"], K, S + R0, k=k)  # index over [0, S + R0)
    Kn = torch.zeros(B, Hkv, S + ring, d, dtype=K.dtype, device="cuda")
    Vn = torch.zeros_like(Kn)
    Kn[:, :, :S] = K[:, :, :S]
    Vn[:, :, :S] = V[:, :, :S]
    for p in range(S + R0, S + R0 + L):
        Kn[:, :, S + (p - S) % ring] = K[:, :, p]
        Vn[:, :, S + (p - S) % ring] = V[:, :, p]
    if far == "host":
        Kf = torch.empty(K.shape, dtype=K.dtype, pin_memory=True)
        Vf = torch.empty(V.shape, dtype=V.dtype, pin_memory=True)
        Kf.zero_()
        Vf.zero_()
    else:
        Kf, Vf = torch.zeros_like(K), torch.zeros_like(V)
    Kf[:, :, S:S + R0] = K[:, :, S:S + R0].to(Kf.device)
    Vf[:, :, S:S + R0] = V[:, :, S:S + R0].to(Vf.device)
    win = pk.pariskv_window_create(Lx.handle, L, U, Kn, Vn, Kf, Vf, cap)
    ws = torch.empty(pk.pariskv_window_attn_workspace_bytes(win, k), dtype=torch.uint8,
                     device="cuda")
    idx = torch.empty(BH, k, dtype=torch.int32, device="cuda")
    est = torch.empty(BH, k - S, dtype=torch.float32, device="cuda")
    out = torch.empty_like(Q)
    Kh, Vh, Qh = host_f32(K), host_f32(V), host_f32(Q)
    checks = 0
    for t in range(steps):
        p = N0 + t
        pk.pariskv_window_append(win, K[:, :, p:], V[:, :, p:], cap)
        n_tok, R, tail = pk.pariskv_window_state(win)
        assert n_tok == p + 1 and tail == n_tok - S - R and L <= tail <= L + U - 1
        assert Lx.size == S + R
        if t not in (0, U - 2, U - 1, U, 2 * U - 1, 3 * U - 1, steps - 1):
            continue
        checks += 1
        Lx.retrieve(Q, idx, est)
        pk.pariskv_window_attn(win, Q, idx, k, d ** -0.5, out, ws)
        torch.cuda.synchronize()
        # index = the oracle's encoding of keys [0, S + R)
        wR = w.scaled(N=S + R)
        enc = oracle_encode_heads(orc, wR, Kh, lay["signs"], list(range(BH)), n=S + R)
        ids, nib, wq = pk.pariskv_debug_export(Lx.handle, 0, S + R, BH)
        for bh in range(BH):
            assert np.array_equal(ids[bh], enc[bh][0])
            assert np.array_equal(nib[bh], enc[bh][1])
            assert np.array_equal(wq[bh], enc[bh][2])
        ref = oracle_retrieve_heads(orc, wR, Qh, enc, lay["signs"], list(range(BH)))
        gi = gpu_intermediates(Lx, BH)
        ih, eh, oh = idx.cpu().numpy(), est.cpu().numpy(), host_f32(out)
        for bh in range(BH):
            assert_retrieval_equal(wR, gi, ih, eh, ref[bh], bh)
            rows = np.concatenate([ih[bh], np.arange(S + R, n_tok)]).astype(np.int32)
            ref_o = orc.attention(Qh[0, bh * G:(bh + 1) * G], Kh[0, bh], Vh[0, bh], rows,
                                  d ** -0.5)
            assert np.max(np.abs(oh[0, bh * G:(bh + 1) * G] - ref_o)) <= ATTN_TOL_BF16
    assert checks == 7
    # the retrieval region's rows reached the far store
    torch.cuda.synchronize()
    _, R, _ = pk.pariskv_window_state(win)
    assert torch.equal(Kf[:, :, S:S + R].cpu(), K[:, :, S:S + R].cpu())
    assert torch.equal(Vf[:, :, S:S + R].cpu(), V[:, :, S:S + R].cpu())
    pk.pariskv_window_destroy(win)
    Lx.close()
