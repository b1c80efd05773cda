"""Keys and values in pinned host memory (mapped into the GPU's address
space): the kernels read them over the host link, as in the offload of
"Technical Summary: ParisKV", System-Level Innovations 1 (full-precision KV
kept in host memory, only the selected rows fetched).  Same kernels as the
device-resident path, so results must be identical bit for bit; attention is
also checked against the oracle."""
import numpy as np
import pytest
import torch

from gpu_helpers import ATTN_TOL_BF16, case, host_f32, need_gpu, pk, synth

pytestmark = pytest.mark.gpu

W = synth.Workload


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def pinned_copy(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def test_attention_host_resident_kv(orc):
    case("attention with K and V in pinned host memory")
    B, Hkv, G, N, k = 1, 8, 4, 20000, 1024
    w = W("host kv", B, Hkv, Hkv * G, 128, N, "bf16", k=k, seed=51)
    lay = synth.make_layer(w, "cuda")
    Kh, Vh = pinned_copy(lay["K"]), pinned_copy(lay["V"])
    gen = torch.Generator(device="cpu").manual_seed(9)
    idx = torch.stack([torch.sort(torch.randperm(N, generator=gen)[:k]).values
                       for _ in range(B * Hkv)]).to(torch.int32).cuda()
    ws = torch.empty(pk.pariskv_attn_workspace_bytes(B, Hkv * G, k, 128),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for K, V in ((lay["K"], lay["V"]), (Kh, Vh), (lay["K"], Vh)):
        out = torch.empty_like(lay["Q"])
        pk.pariskv_sparse_attn(lay["Q"], K, V, N, idx, k, B, Hkv * G, Hkv, 128,
                               pk.PARISKV_DTYPE_BF16, 128 ** -0.5, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0], outs[2])
    Qf, Kf, Vf = host_f32(lay["Q"]), host_f32(Kh), host_f32(Vh)
    oh = outs[1].float().numpy()
    ih = idx.cpu().numpy()
    for bh in (0, 5):
        h = bh
        ref = orc.attention(Qf[0, h * G:(h + 1) * G], Kf[0, h], Vf[0, h], ih[bh],
                            128 ** -0.5)
        assert np.max(np.abs(oh[0, h * G:(h + 1) * G] - ref)) <= ATTN_TOL_BF16


def test_index_from_host_keys():
    case("index build and append from keys in pinned host memory")
    N, extra = 9000, 40
    w = W("host keys", 2, 4, 16, 128, N, "bf16", k=256, sinks=8, seed=52)
    cap = N + extra
    lay = synth.make_layer(w, "cuda", capacity=cap)
    Kh = pinned_copy(lay["K"])
    BH = w.batch * w.n_kv_heads
    res = []
    for K in (lay["K"], Kh):
        cfg = pk.config_for(w, capacity=cap)
        L = pk.Layer(cfg, lay["signs"], K, N, k=w.k, device="cuda")
        for r in range(extra):   # one key per (b, h) per step
            n = L.size
            L.append(K[:, :, n:], 1, rows_per_head=cap)
        idx = torch.empty(BH, w.k, dtype=torch.int32, device="cuda")
        est = torch.empty(BH, w.kprime, dtype=torch.float32, device="cuda")
        L.retrieve(lay["Q"], idx, est)
        torch.cuda.synchronize()
        ids, nib, wq = pk.pariskv_debug_export(L.handle, 0, N + extra, BH)
        res.append((ids, nib, wq, idx.cpu().numpy(),
                    est.cpu().numpy().view(np.uint32)))
        L.close()
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)
