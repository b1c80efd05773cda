"""Seeded synthetic inputs for the retrieval path.

This module draws inputs only; it holds none of the method's arithmetic.  The
pages measure on LLM benchmarks with trained models that are not available
here, so these shapes and distributions stand in for them: LLM-shaped decode
layers (d = 128, grouped-query attention with 4 query heads per KV head) with
keys whose channels have heavy-tailed scales and a few outlier channels.

Recipe (per workload):
  * srht signs: numpy PCG64(srht_seed), d draws of {+1, -1}.
  * channel scales s[h, c] = exp(0.5 g), g ~ N(0, 1), per KV head; 4 distinct
    channels per head get s *= 8 (read as a standard-deviation multiplier).
  * keys   K[b, h, i, :] = s[h] * N(0, I)
  * queries Q[b, h*G + g, :] = s[h] * N(0, I)
  * values V ~ N(0, 1)
  * bf16 workloads round the fp32 draws to bf16 (round-to-nearest-even);
    the tiny workload stays fp32 and plants 8 keys q + 0.1 N(0, I) at
    distinct positions.
  * drift workload: after the prefill, step t of T appends one key per
    (b, h) with mean mu_t = 1.5 s t / T on 16 distinct channels per (b, h);
    the step's query is drawn from the same shifted distribution.
Large tensors are drawn with torch generators on the target device.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_kv_heads: int
    n_q_heads: int
    d: int
    N: int
    dtype: str            # "bf16" or "fp32"
    B: int = 16           # subspaces
    rho: int = 4          # centroids kept per subspace
    tiers: tuple = (4, 3, 2, 1)
    cand_num: int = 1     # candidate fraction = cand_num / cand_den
    cand_den: int = 20
    k: int = 1024
    sinks: int = 0
    planted: int = 0
    seed: int = 1000
    srht_seed: int = 1
    decode_steps: int = 0  # drift workload: keys appended one per step
    drift_channels: int = 16
    drift_sigma: float = 1.5
    per_query_head: bool = False  # unshared retrieval: one per query head

    @property
    def m(self) -> int:
        return self.d // self.B

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def E(self) -> int:
        return self.N - self.sinks

    @property
    def kprime(self) -> int:
        return self.k - self.sinks

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # d=128, N=4096 fp32 keys, one query, B=16 (m=8), rho=4 tiers 4/3/2/1,
    # 10% candidates, k=64, 8 planted keys.
    "tiny": Workload("tiny single head", 1, 1, 1, 128, 4096, "fp32",
                     cand_num=1, cand_den=10, k=64, planted=8, seed=1001),
    # Llama-3-8B-shaped decode layer: 32 q / 8 KV heads, N=32768, 5%, k=1024.
    "llama8b_32k": Workload("Llama-3-8B-shaped decode layer, 32K context",
                            1, 8, 32, 128, 32768, "bf16", k=1024, seed=1002),
    # batched long input: batch 8, N=131072, 5%, k=2048, 64 sinks.
    "batched_128k": Workload("batched long-input decode, 8 x 128K", 8, 8, 32,
                             128, 131072, "bf16", k=2048, sinks=64, seed=1003),
    # long-generation drift: batch 4, prefill 32768 then 32768 decode steps.
    "drift": Workload("long-generation drift, 4 x (32K prefill + 32K decode)",
                      4, 8, 32, 128, 32768, "bf16", k=1024, seed=1004,
                      decode_steps=32768),
    # million-token context: batch 1, N=1048576, 5%, k=4096.
    "million": Workload("million-token context, 1 x 1M", 1, 8, 32, 128,
                        1048576, "bf16", k=4096, seed=1005),
}


def srht_signs(d: int, seed: int = 1) -> np.ndarray:
    """d random signs (+1/-1 as int8) for the rotation's diagonal."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bits = rng.integers(0, 2, size=d)
    return np.where(bits == 1, -1, 1).astype(np.int8)


def channel_scales(n_kv_heads: int, d: int, seed: int,
                   n_outliers: int = 4, outlier: float = 8.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    s = np.exp(0.5 * rng.standard_normal((n_kv_heads, d)))
    for h in range(n_kv_heads):
        ch = rng.choice(d, size=n_outliers, replace=False)
        s[h, ch] *= outlier
    return s.astype(np.float32)


def torch_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_layer(w: Workload, device="cpu", layer: int = 0, capacity=None,
               with_values: bool = True):
    """Draw one layer's K, V (capacity rows per (b, h), first N filled) and Q.

    Returns dict(K, V, Q, scales, signs) with K/V [batch, H_kv, capacity, d]
    and Q [batch, H_q, d] in the workload dtype on `device`.
    """
    cap = int(capacity or w.N)
    dt = torch_dtype(w)
    seed = w.seed * 1000 + layer
    scales = torch.from_numpy(channel_scales(w.n_kv_heads, w.d, seed))
    g = _gen(device, seed + 1)
    sc = scales.to(device)
    K = torch.empty(w.batch, w.n_kv_heads, cap, w.d, dtype=dt, device=device)
    V = torch.empty(w.batch, w.n_kv_heads, cap, w.d, dtype=dt, device=device) \
        if with_values else None
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            x = torch.randn(w.N, w.d, generator=g, device=device)
            K[b, h, :w.N] = (x * sc[h]).to(dt)
            if cap > w.N:
                K[b, h, w.N:] = 0
            if with_values:
                v = torch.randn(w.N, w.d, generator=g, device=device)
                V[b, h, :w.N] = v.to(dt)
                if cap > w.N:
                    V[b, h, w.N:] = 0
    q = torch.randn(w.batch, w.n_q_heads, w.d, generator=g, device=device)
    head_of = torch.arange(w.n_q_heads, device=device) // w.G
    Q = (q * sc[head_of][None]).to(dt)
    if w.planted:
        # planted keys near the (first) query head of each group
        rng = np.random.Generator(np.random.PCG64(seed + 2))
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                pos = rng.choice(np.arange(w.sinks, w.N), size=w.planted,
                                 replace=False)
                qv = Q[b, h * w.G].float()
                for p in pos:
                    eps = torch.randn(w.d, generator=g, device=device)
                    K[b, h, int(p)] = (qv + 0.1 * eps).to(dt)
    return dict(K=K, V=V, Q=Q, scales=scales,
                signs=srht_signs(w.d, w.srht_seed))


def planted_positions(w: Workload, layer: int = 0):
    """The planted positions make_layer used, per (b, h)."""
    seed = w.seed * 1000 + layer
    rng = np.random.Generator(np.random.PCG64(seed + 2))
    out = []
    for b in range(w.batch):
        row = []
        for h in range(w.n_kv_heads):
            row.append(np.sort(rng.choice(np.arange(w.sinks, w.N),
                                          size=w.planted, replace=False)))
        out.append(row)
    return out


def drift_channels(w: Workload, seed_offset: int = 7) -> np.ndarray:
    """[batch, H_kv, drift_channels] distinct channel ids per (b, h)."""
    rng = np.random.Generator(np.random.PCG64(w.seed * 1000 + seed_offset))
    return np.stack([np.stack([rng.choice(w.d, w.drift_channels, replace=False)
                               for _ in range(w.n_kv_heads)])
                     for _ in range(w.batch)])


def drift_step(w: Workload, t: int, scales: torch.Tensor, chans: np.ndarray,
               device="cpu"):
    """Decode step t (1..T) of the drift workload: one new key per (b, h)
    and the step's queries, both with the drifted channel means."""
    T = w.decode_steps
    g = _gen(device, w.seed * 1000003 + t)
    dt = torch_dtype(w)
    sc = scales.to(device)
    mu = torch.zeros(w.batch, w.n_kv_heads, w.d, device=device)
    ch = torch.from_numpy(chans).to(device).long()
    frac = w.drift_sigma * t / T
    mu.scatter_(2, ch, (frac * sc[None].expand(w.batch, -1, -1)).gather(2, ch))
    k = torch.randn(w.batch, w.n_kv_heads, 1, w.d, generator=g, device=device)
    knew = (k * sc[None, :, None] + mu[:, :, None]).to(dt)
    q = torch.randn(w.batch, w.n_q_heads, w.d, generator=g, device=device)
    head_of = torch.arange(w.n_q_heads, device=device) // w.G
    Q = (q * sc[head_of][None] + mu[:, head_of]).to(dt)
    v = torch.randn(w.batch, w.n_kv_heads, 1, w.d, generator=g, device=device)
    return knew, Q, v.to(dt)
