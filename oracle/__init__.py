"""CPU oracle for the ParisKV decode-step retrieval path (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(``kv_cache_top_srht_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, -O2 -ffp-contract=off); this
module only marshals numpy arrays.  Every function cites, in ``oracle.c``, the
passage of "Technical Summary: ParisKV" (or, for the Self-Indexing workload,
of "Self-Indexing KVCache") it follows; the pins that check each
function against closed forms, invariants and brute force are in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (plain gcc, no GPU code)."""
    if force or not os.path.exists(_SO) or \
            os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or \
                os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_SO)
        P = C.c_void_p
        i32, i64, f32, f64 = C.c_int32, C.c_int64, C.c_float, C.c_double
        sig = {
            "orc_f32_to_f16": (C.c_uint16, [f32]),
            "orc_f16_to_f32": (f32, [C.c_uint16]),
            "orc_codebook": (i32, [i32, P, P]),
            "orc_codebook_f32": (i32, [i32, P, P]),
            "orc_rot_scale": (f32, [i32]),
            "orc_srht_signs": (i32, [C.c_uint64, i32, P]),
            "orc_splitmix64": (i32, [C.c_uint64, i32, P]),
            "orc_rotate": (i32, [i32, P, P, P]),
            "orc_encode_keys": (i32, [i32, i32, P, i64, P, P, P, P]),
            "orc_query_prep": (i32, [i32, i32, i32, P, P, i32, P, P, P, P]),
            "orc_vote_scores": (i32, [i32, i32, i64, i64, P, P, P]),
            "orc_cand_count": (i64, [i64, i64, i64, i64]),
            "orc_candidates": (i32, [i64, i64, P, i64, P]),
            "orc_rerank": (i32, [i32, i32, P, P, P, i64, P, P]),
            "orc_topk": (i32, [i64, P, P, i64, i64, P]),
            "orc_attention": (i32, [i32, i32, i64, P, P, P, P, f64, P]),
            "orc_exact_topk": (i32, [i32, i32, P, i64, i64, P, i64, P]),
            "orc_si_build": (i32, [i32, i64, i64, P, P, P, P]),
            "orc_si_ids": (i32, [i32, i64, P, P, P]),
            "orc_si_lut": (i32, [i32, i32, P, P, P]),
            "orc_si_scores": (i32, [i32, i64, i64, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ok(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)


# -- scalar helpers ---------------------------------------------------------

def f32_to_f16(x) -> np.ndarray:
    x = _c(x, np.float32).ravel()
    fn = lib().orc_f32_to_f16
    return np.array([fn(float(v)) for v in x], dtype=np.uint16)


def f16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16).ravel()
    fn = lib().orc_f16_to_f32
    return np.array([fn(int(v)) for v in h], dtype=np.float32)


def codebook(m: int):
    L = np.zeros(8, np.float64)
    t = np.zeros(7, np.float64)
    _ok(lib().orc_codebook(m, _p(L), _p(t)))
    return L, t


def codebook_f32(m: int):
    L = np.zeros(8, np.float32)
    t = np.zeros(7, np.float32)
    _ok(lib().orc_codebook_f32(m, _p(L), _p(t)))
    return L, t


def srht_signs(seed: int, d: int) -> np.ndarray:
    """The rotation's signs D from a seed (SplitMix64 top bits), int8 [d]."""
    D = np.zeros(d, np.int8)
    _ok(lib().orc_srht_signs(int(seed), int(d), _p(D)))
    return D


def splitmix64(seed: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.uint64)
    _ok(lib().orc_splitmix64(int(seed), int(n), _p(out)))
    return out


def rot_scale(d: int) -> np.float32:
    return np.float32(lib().orc_rot_scale(d))


# -- pipeline steps (one (batch, KV head) at a time) -------------------------

def rotate(signs, x) -> np.ndarray:
    signs = _c(signs, np.int8)
    x = _c(x, np.float32)
    d = signs.shape[0]
    flat = x.reshape(-1, d)
    out = np.empty_like(flat)
    for r in range(flat.shape[0]):
        _ok(lib().orc_rotate(d, _p(signs), _p(flat[r]), _p(out[r])))
    return out.reshape(x.shape)


def encode_keys(signs, X, m: int):
    """-> ids uint8 [n, B], nib uint8 [n, d/2], w uint16 (fp16 bits) [n, B]."""
    signs = _c(signs, np.int8)
    X = _c(X, np.float32)
    d = signs.shape[0]
    n = X.shape[0]
    B = d // m
    ids = np.zeros((n, B), np.uint8)
    nib = np.zeros((n, d // 2), np.uint8)
    w = np.zeros((n, B), np.uint16)
    _ok(lib().orc_encode_keys(d, m, _p(signs), n, _p(X), _p(ids), _p(nib),
                              _p(w)))
    return ids, nib, w


def query_prep(signs, Q, m: int, rho: int, tiers):
    """Q: [G, d] fp32 query heads of one KV group.
    -> yq fp32 [d], lut uint8 [B, 2^m], top int32 [B, rho]."""
    signs = _c(signs, np.int8)
    Q = _c(Q, np.float32)
    d = signs.shape[0]
    G = Q.shape[0]
    B = d // m
    tiers = _c(tiers, np.int32)
    yq = np.zeros(d, np.float32)
    lut = np.zeros((B, 1 << m), np.uint8)
    top = np.zeros((B, rho), np.int32)
    _ok(lib().orc_query_prep(d, m, rho, _p(tiers), _p(signs), G, _p(Q),
                             _p(yq), _p(lut), _p(top)))
    return yq, lut, top


def vote_scores(ids, lut, S: int, m: int) -> np.ndarray:
    ids = _c(ids, np.uint8)
    lut = _c(lut, np.uint8)
    N, B = ids.shape
    sc = np.zeros(max(N - S, 0), np.int32)
    _ok(lib().orc_vote_scores(B, m, N, S, _p(ids), _p(lut), _p(sc)))
    return sc


def cand_count(E: int, kprime: int, num: int, den: int) -> int:
    return int(lib().orc_cand_count(E, kprime, num, den))


def candidates(scores, S: int, C: int) -> np.ndarray:
    scores = _c(scores, np.int32)
    E = scores.shape[0]
    out = np.zeros(C, np.int32)
    _ok(lib().orc_candidates(E, S, _p(scores), C, _p(out)))
    return out


def rerank(nib, w, yq, cand, m: int) -> np.ndarray:
    nib = _c(nib, np.uint8)
    w = _c(w, np.uint16)
    yq = _c(yq, np.float32)
    cand = _c(cand, np.int32)
    d = yq.shape[0]
    est = np.zeros(cand.shape[0], np.float32)
    _ok(lib().orc_rerank(d, m, _p(nib), _p(w), _p(yq), cand.shape[0],
                         _p(cand), _p(est)))
    return est


def topk(cand, est, kprime: int, S: int) -> np.ndarray:
    cand = _c(cand, np.int32)
    est = _c(est, np.float32)
    out = np.zeros(S + kprime, np.int32)
    _ok(lib().orc_topk(cand.shape[0], _p(cand), _p(est), kprime, S, _p(out)))
    return out


def attention(Q, K, V, idx, scale: float) -> np.ndarray:
    """Q [G, d]; K, V [rows, d] fp32 values; idx int32 [k] -> fp64 [G, d]."""
    Q = _c(Q, np.float32)
    K = _c(K, np.float32)
    V = _c(V, np.float32)
    idx = _c(idx, np.int32)
    G, d = Q.shape
    out = np.zeros((G, d), np.float64)
    _ok(lib().orc_attention(d, G, idx.shape[0], _p(Q), _p(K), _p(V), _p(idx),
                            float(scale), _p(out)))
    return out


def exact_topk(Q, K, S: int, kprime: int) -> np.ndarray:
    Q = _c(Q, np.float32)
    K = _c(K, np.float32)
    G, d = Q.shape
    out = np.zeros(kprime, np.int64)
    _ok(lib().orc_exact_topk(d, G, _p(Q), K.shape[0], S, _p(K), kprime,
                             _p(out)))
    return out


def retrieve_head(signs, Q, ids, nib, w, *, m, rho, tiers, S, k, num, den):
    """Whole retrieval for one (batch, KV head): every intermediate.

    Q: [G, d] fp32 values of the group's query heads; ids/nib/w: the encoded
    keys [N, ...].  Returns a dict with yq, lut, scores, C, cand, est, idx.
    """
    N = ids.shape[0]
    E = N - S
    kprime = k - S
    if not (0 <= S < k <= N):
        raise ValueError("need 0 <= S < k <= N")
    yq, lut, top = query_prep(signs, Q, m, rho, tiers)
    sc = vote_scores(ids, lut, S, m)
    Cn = cand_count(E, kprime, num, den)
    cand = candidates(sc, S, Cn)
    est = rerank(nib, w, yq, cand, m)
    idx = topk(cand, est, kprime, S)
    return dict(yq=yq, lut=lut, top=top, scores=sc, C=Cn, cand=cand, est=est,
                idx=idx)


# ------------------------------------------------------- Self-Indexing ----

def si_build(X, S: int):
    """Prefill index of one (b, h): X [n, d] fp32 keys, S sinks.
    -> mean fp32 [d], ids uint8 [n, d/4], cb fp32 [d/4, 16, 4]."""
    X = _c(X, np.float32)
    n, d = X.shape
    mean = np.zeros(d, np.float32)
    ids = np.zeros((n, d // 4), np.uint8)
    cb = np.zeros((d // 4, 16, 4), np.float32)
    _ok(lib().orc_si_build(d, n, S, _p(X), _p(mean), _p(ids), _p(cb)))
    return mean, ids, cb


def si_ids(X, mean):
    """Sign ids of appended keys with the prefill means -> uint8 [n, d/4]."""
    X = _c(X, np.float32)
    mean = _c(mean, np.float32)
    n, d = X.shape
    ids = np.zeros((n, d // 4), np.uint8)
    _ok(lib().orc_si_ids(d, n, _p(X), _p(mean), _p(ids)))
    return ids


def si_lut(Q, cb):
    """Q [G, d] fp32 query heads of one KV group -> lut fp32 [d/4, 16]."""
    Q = _c(Q, np.float32)
    cb = _c(cb, np.float32)
    G, d = Q.shape
    lut = np.zeros((d // 4, 16), np.float32)
    _ok(lib().orc_si_lut(d, G, _p(Q), _p(cb), _p(lut)))
    return lut


def si_scores(ids, lut, S: int):
    ids = _c(ids, np.uint8)
    lut = _c(lut, np.float32)
    n, B = ids.shape
    sc = np.zeros(max(n - S, 0), np.float32)
    _ok(lib().orc_si_scores(4 * B, n, S, _p(ids), _p(lut), _p(sc)))
    return sc


def si_retrieve_head(Q, ids, cb, *, S, k):
    """Self-Indexing retrieval for one (batch, KV head): LUT, scores of keys
    [S, N), and the top-k (sinks first, then the k - S best scores by
    (score desc, position asc), ascending) with their scores."""
    N = ids.shape[0]
    if not (0 <= S < k <= N):
        raise ValueError("need 0 <= S < k <= N")
    lut = si_lut(Q, cb)
    sc = si_scores(ids, lut, S)
    cand = np.arange(S, N, dtype=np.int32)
    idx = topk(cand, sc, k - S, S)
    return dict(lut=lut, scores=sc, idx=idx, est=sc[idx[S:] - S])
