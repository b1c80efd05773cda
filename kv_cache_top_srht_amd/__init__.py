"""MI355X (gfx950) ParisKV decode-step retrieval: Python binding.

Thin ctypes layer over ``libpariskv.so`` (C ABI in ``include/pariskv.h``).
Functions carry the C entry points' names and only marshal arguments: torch
tensors provide device memory and streams, every step of the path runs in the
library's HIP kernels.  There is no CPU fallback: if the library is not built,
every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(_PKG, "libpariskv.so")

PARISKV_OK = 0
(PARISKV_ERR_INVALID_ARG, PARISKV_ERR_UNSUPPORTED, PARISKV_ERR_CAPACITY,
 PARISKV_ERR_WORKSPACE, PARISKV_ERR_HIP, PARISKV_ERR_NOMEM) = range(-1, -7, -1)
PARISKV_DTYPE_BF16 = 0
PARISKV_DTYPE_FP32 = 1
PARISKV_RETRIEVE_STAGES = 6

DEBUG_LUT, DEBUG_YQ, DEBUG_SCORES, DEBUG_CAND, DEBUG_EST, DEBUG_THRESH = range(6)
# retrieval paths (pariskv_set_retrieval_path)
PATH_AUTO, PATH_PIPELINE, PATH_SINGLE = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 32 << 20   # PARISKV_NOALLOC_SCRATCH_BYTES


class PariskvError(RuntimeError):
    def __init__(self, rc: int, msg: str):
        super().__init__("pariskv error %d: %s" % (rc, msg))
        self.rc = rc


class pariskv_config(C.Structure):
    _fields_ = [
        ("head_dim", C.c_int32),
        ("n_subspaces", C.c_int32),
        ("rho", C.c_int32),
        ("tier_w", C.c_int32 * 8),
        ("cand_num", C.c_int32),
        ("cand_den", C.c_int32),
        ("n_sink", C.c_int32),
        ("batch", C.c_int32),
        ("n_kv_heads", C.c_int32),
        ("n_q_heads", C.c_int32),
        ("key_dtype", C.c_int32),
        ("capacity", C.c_int64),
        ("per_query_head", C.c_int32),
    ]


class pariskv_si_config(C.Structure):
    _fields_ = [
        ("head_dim", C.c_int32),
        ("n_sink", C.c_int32),
        ("batch", C.c_int32),
        ("n_kv_heads", C.c_int32),
        ("n_q_heads", C.c_int32),
        ("key_dtype", C.c_int32),
        ("capacity", C.c_int64),
    ]


_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise RuntimeError(
                "libpariskv.so is not built (expected at %s); run "
                "`python -c 'import __graft_entry__ as g; g.build()'`" % SO_PATH)
        L = C.CDLL(SO_PATH)
        P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        cfgp = C.POINTER(pariskv_config)
        sig = {
            "pariskv_index_bytes": (i32, [cfgp, C.POINTER(sz)]),
            "pariskv_retrieve_workspace_bytes": (i32, [cfgp, i32, C.POINTER(sz)]),
            "pariskv_attn_workspace_bytes": (i32, [i32, i32, i32, i32, C.POINTER(sz)]),
            "pariskv_build_index": (i32, [cfgp, P, P, sz, P, i64, i64, P, C.POINTER(P)]),
            "pariskv_append_keys": (i32, [P, P, i64, i64, P]),
            "pariskv_index_size": (i64, [P]),
            "pariskv_index_destroy": (None, [P]),
            "pariskv_retrieve_topk": (i32, [P, P, i32, P, P, P, sz, P]),
            "pariskv_retrieve_topk_noalloc": (i32, [P, P, i32, P, P, P]),
            "pariskv_retrieve_attend_workspace_bytes": (i32, [cfgp, i32, C.POINTER(sz)]),
            "pariskv_retrieve_attend": (i32, [P, P, P, P, i64, i32, C.c_float, P, P, P, P, sz,
                                              P]),
            "pariskv_retrieve_attend_profiled": (i32, [P, P, P, P, i64, i32, C.c_float, P, P,
                                                       P, P, sz, P, P]),
            "pariskv_retrieve_topk_profiled": (i32, [P, P, i32, P, P, P, sz, P,
                                                     C.POINTER(P)]),
            "pariskv_stage_name": (C.c_char_p, [i32]),
            "pariskv_sparse_attn": (i32, [P, P, P, i64, P, i32, i32, i32, i32, i32,
                                          i32, C.c_float, P, P, sz, P]),
            "pariskv_sparse_attn_profiled": (i32, [P, P, P, i64, P, i32, i32, i32, i32,
                                                   i32, i32, C.c_float, P, P, sz, P,
                                                   C.POINTER(P)]),
            "pariskv_debug_export": (i32, [P, i64, i64, P, P, P]),
            "pariskv_debug_intermediate": (i32, [P, i32, P, sz, i32, P, sz]),
            "pariskv_retrieve_sizes": (i32, [P, i32, C.POINTER(i64), C.POINTER(i64)]),
            "pariskv_set_retrieval_path": (i32, [P, i32]),
            "pariskv_retrieval_path": (i32, [P, i32]),
            "pariskv_codebook": (i32, [i32, P, P]),
            "pariskv_rot_scale": (C.c_float, [i32]),
            "pariskv_srht_signs_from_seed": (i32, [C.c_uint64, i32, P]),
            "pariskv_status_string": (C.c_char_p, [i32]),
            "pariskv_sparse_attn_per_query_head": (i32, [P, P, P, i64, P, i32, i32, i32,
                                                         i32, i32, i32, C.c_float, P, P,
                                                         sz, P]),
            "pariskv_sparse_attn_per_query_head_profiled": (
                i32, [P, P, P, i64, P, i32, i32, i32, i32, i32, i32, C.c_float, P, P, sz, P,
                      C.POINTER(P)]),
            "pariskv_window_create": (i32, [P, i64, i64, P, P, P, P, i64, C.POINTER(P)]),
            "pariskv_window_append": (i32, [P, P, P, i64, P]),
            "pariskv_window_state": (i32, [P, C.POINTER(i64), C.POINTER(i64),
                                           C.POINTER(i64)]),
            "pariskv_window_attn_workspace_bytes": (i32, [P, i32, C.POINTER(sz)]),
            "pariskv_window_attn": (i32, [P, P, P, i32, C.c_float, P, P, sz, P]),
            "pariskv_window_attn_profiled": (i32, [P, P, P, i32, C.c_float, P, P, sz, P,
                                                   C.POINTER(P)]),
            "pariskv_window_destroy": (None, [P]),
            "pariskv_si_index_bytes": (i32, [P, C.POINTER(sz)]),
            "pariskv_si_build_workspace_bytes": (i32, [P, i64, C.POINTER(sz)]),
            "pariskv_si_retrieve_workspace_bytes": (i32, [P, i32, C.POINTER(sz)]),
            "pariskv_si_build_index": (i32, [P, P, sz, P, i64, i64, P, sz, P,
                                              C.POINTER(P)]),
            "pariskv_si_append_keys": (i32, [P, P, i64, i64, P]),
            "pariskv_si_index_size": (i64, [P]),
            "pariskv_si_index_destroy": (None, [P]),
            "pariskv_si_retrieve_topk": (i32, [P, P, i32, P, P, P, sz, P]),
            "pariskv_si_retrieve_topk_profiled": (i32, [P, P, i32, P, P, P, sz, P,
                                                        C.POINTER(P)]),
            "pariskv_si_debug_export": (i32, [P, i64, i64, P, P, P]),
            "pariskv_si_debug_intermediate": (i32, [P, i32, P, sz, i32, P, sz]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def pariskv_status_string(rc: int) -> str:
    return lib().pariskv_status_string(rc).decode()


def _check(rc: int):
    if rc != PARISKV_OK:
        raise PariskvError(rc, pariskv_status_string(rc))


def _ptr(t):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _events(events):
    arr = (C.c_void_p * len(events))()
    for i, e in enumerate(events):
        arr[i] = e.cuda_event if hasattr(e, "cuda_event") else int(e)
    return arr


# ---------------------------------------------------------------- config ----

def make_config(*, head_dim=128, n_subspaces=16, rho=4, tiers=(4, 3, 2, 1),
                cand_num=1, cand_den=20, n_sink=0, batch=1, n_kv_heads=8,
                n_q_heads=32, key_dtype=PARISKV_DTYPE_BF16, capacity,
                per_query_head=False):
    c = pariskv_config()
    c.head_dim, c.n_subspaces, c.rho = head_dim, n_subspaces, rho
    for i in range(8):
        c.tier_w[i] = int(tiers[i]) if i < len(tiers) else 0
    c.cand_num, c.cand_den, c.n_sink = cand_num, cand_den, n_sink
    c.batch, c.n_kv_heads, c.n_q_heads = batch, n_kv_heads, n_q_heads
    c.key_dtype, c.capacity = key_dtype, int(capacity)
    c.per_query_head = 1 if per_query_head else 0
    return c


def config_for(w, capacity=None):
    """pariskv_config for a synth.Workload."""
    return make_config(head_dim=w.d, n_subspaces=w.B, rho=w.rho, tiers=w.tiers,
                       cand_num=w.cand_num, cand_den=w.cand_den, n_sink=w.sinks,
                       batch=w.batch, n_kv_heads=w.n_kv_heads,
                       n_q_heads=w.n_q_heads,
                       key_dtype=PARISKV_DTYPE_BF16 if w.dtype == "bf16"
                       else PARISKV_DTYPE_FP32,
                       capacity=capacity or w.N,
                       per_query_head=getattr(w, "per_query_head", False))


# ------------------------------------------------------------ C entry points

def pariskv_index_bytes(cfg) -> int:
    n = C.c_size_t()
    _check(lib().pariskv_index_bytes(C.byref(cfg), C.byref(n)))
    return n.value


def pariskv_retrieve_workspace_bytes(cfg, k: int) -> int:
    n = C.c_size_t()
    _check(lib().pariskv_retrieve_workspace_bytes(C.byref(cfg), k, C.byref(n)))
    return n.value


def pariskv_attn_workspace_bytes(batch, n_q_heads, k, head_dim=128) -> int:
    n = C.c_size_t()
    _check(lib().pariskv_attn_workspace_bytes(batch, n_q_heads, k, head_dim,
                                              C.byref(n)))
    return n.value


def pariskv_build_index(cfg, srht_signs, index_buf, K, k_rows_per_head, n_keys,
                        stream=None):
    """Returns the opaque handle (c_void_p)."""
    signs = np.ascontiguousarray(srht_signs, dtype=np.int8)
    h = C.c_void_p()
    _check(lib().pariskv_build_index(
        C.byref(cfg), signs.ctypes.data_as(C.c_void_p), _ptr(index_buf),
        _nbytes(index_buf), _ptr(K), int(k_rows_per_head), int(n_keys),
        _stream(stream), C.byref(h)))
    return h


def pariskv_append_keys(handle, K_new, new_rows_per_head, n_new, stream=None):
    _check(lib().pariskv_append_keys(handle, _ptr(K_new), int(new_rows_per_head),
                                     int(n_new), _stream(stream)))


def pariskv_index_size(handle) -> int:
    return int(lib().pariskv_index_size(handle))


def pariskv_index_destroy(handle):
    lib().pariskv_index_destroy(handle)


def pariskv_retrieve_topk(handle, Q, k, out_idx, out_est, ws, stream=None):
    _check(lib().pariskv_retrieve_topk(handle, _ptr(Q), int(k), _ptr(out_idx),
                                       _ptr(out_est), _ptr(ws), _nbytes(ws),
                                       _stream(stream)))


def pariskv_retrieve_attend_workspace_bytes(cfg, k) -> int:
    n = C.c_size_t(0)
    _check(lib().pariskv_retrieve_attend_workspace_bytes(C.byref(cfg), int(k), C.byref(n)))
    return n.value


def pariskv_retrieve_attend(handle, Q, K, V, kv_rows_per_head, k, scale, out_idx, out_est,
                            out, ws, stream=None):
    _check(lib().pariskv_retrieve_attend(handle, _ptr(Q), _ptr(K), _ptr(V),
                                         int(kv_rows_per_head), int(k), float(scale),
                                         _ptr(out_idx), _ptr(out_est), _ptr(out), _ptr(ws),
                                         _nbytes(ws), _stream(stream)))


def pariskv_retrieve_attend_profiled(handle, Q, K, V, kv_rows_per_head, k, scale, out_idx,
                                     out_est, out, ws, events, stream=None):
    _check(lib().pariskv_retrieve_attend_profiled(
        handle, _ptr(Q), _ptr(K), _ptr(V), int(kv_rows_per_head), int(k), float(scale),
        _ptr(out_idx), _ptr(out_est), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream),
        _events(events)))


def pariskv_retrieve_topk_noalloc(handle, Q, k, out_idx, out_est, stream=None):
    _check(lib().pariskv_retrieve_topk_noalloc(handle, _ptr(Q), int(k), _ptr(out_idx),
                                               _ptr(out_est), _stream(stream)))


def pariskv_retrieve_topk_profiled(handle, Q, k, out_idx, out_est, ws, events,
                                   stream=None):
    _check(lib().pariskv_retrieve_topk_profiled(
        handle, _ptr(Q), int(k), _ptr(out_idx), _ptr(out_est), _ptr(ws),
        _nbytes(ws), _stream(stream), _events(events)))


def pariskv_sparse_attn_per_query_head(Q, K, V, kv_rows_per_head, idx, k, batch,
                                       n_q_heads, n_kv_heads, head_dim, dtype, scale, out,
                                       ws, stream=None):
    _check(lib().pariskv_sparse_attn_per_query_head(
        _ptr(Q), _ptr(K), _ptr(V), int(kv_rows_per_head), _ptr(idx), int(k), int(batch),
        int(n_q_heads), int(n_kv_heads), int(head_dim), int(dtype), C.c_float(scale),
        _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)))


def pariskv_sparse_attn_per_query_head_profiled(Q, K, V, kv_rows_per_head, idx, k,
                                                batch, n_q_heads, n_kv_heads, head_dim,
                                                dtype, scale, out, ws, events, stream=None):
    _check(lib().pariskv_sparse_attn_per_query_head_profiled(
        _ptr(Q), _ptr(K), _ptr(V), int(kv_rows_per_head), _ptr(idx), int(k), int(batch),
        int(n_q_heads), int(n_kv_heads), int(head_dim), int(dtype), C.c_float(scale),
        _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream), _events(events)))


def pariskv_window_create(index_handle, n_local, n_update, K_near, V_near, K_far,
                          V_far, far_rows_per_head):
    h = C.c_void_p()
    _check(lib().pariskv_window_create(index_handle, int(n_local), int(n_update),
                                       _ptr(K_near), _ptr(V_near), _ptr(K_far),
                                       _ptr(V_far), int(far_rows_per_head), C.byref(h)))
    return h


def pariskv_window_append(w, K_new, V_new, new_rows_per_head, stream=None):
    _check(lib().pariskv_window_append(w, _ptr(K_new), _ptr(V_new),
                                       int(new_rows_per_head), _stream(stream)))


def pariskv_window_state(w):
    """(tokens per (b, h), retrieval-region size R, attended tail L + u)."""
    a, b, c = C.c_int64(), C.c_int64(), C.c_int64()
    _check(lib().pariskv_window_state(w, C.byref(a), C.byref(b), C.byref(c)))
    return a.value, b.value, c.value


def pariskv_window_attn_workspace_bytes(w, k) -> int:
    n = C.c_size_t()
    _check(lib().pariskv_window_attn_workspace_bytes(w, int(k), C.byref(n)))
    return n.value


def pariskv_window_attn(w, Q, idx, k, scale, out, ws, stream=None):
    _check(lib().pariskv_window_attn(w, _ptr(Q), _ptr(idx), int(k), C.c_float(scale),
                                     _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)))


def pariskv_window_attn_profiled(w, Q, idx, k, scale, out, ws, events, stream=None):
    _check(lib().pariskv_window_attn_profiled(w, _ptr(Q), _ptr(idx), int(k),
                                              C.c_float(scale), _ptr(out), _ptr(ws),
                                              _nbytes(ws), _stream(stream),
                                              _events(events)))


def pariskv_window_destroy(w):
    lib().pariskv_window_destroy(w)


def pariskv_stage_name(s: int):
    r = lib().pariskv_stage_name(s)
    return r.decode() if r else None


def pariskv_sparse_attn(Q, K, V, kv_rows_per_head, idx, k, batch, n_q_heads,
                        n_kv_heads, head_dim, dtype, scale, out, ws, stream=None):
    _check(lib().pariskv_sparse_attn(
        _ptr(Q), _ptr(K), _ptr(V), int(kv_rows_per_head), _ptr(idx), int(k),
        batch, n_q_heads, n_kv_heads, head_dim, dtype, float(scale), _ptr(out),
        _ptr(ws), _nbytes(ws), _stream(stream)))


def pariskv_sparse_attn_profiled(Q, K, V, kv_rows_per_head, idx, k, batch,
                                 n_q_heads, n_kv_heads, head_dim, dtype, scale,
                                 out, ws, events, stream=None):
    _check(lib().pariskv_sparse_attn_profiled(
        _ptr(Q), _ptr(K), _ptr(V), int(kv_rows_per_head), _ptr(idx), int(k),
        batch, n_q_heads, n_kv_heads, head_dim, dtype, float(scale), _ptr(out),
        _ptr(ws), _nbytes(ws), _stream(stream), _events(events)))


def pariskv_debug_export(handle, lo, hi, BH, B=16, d=128):
    n = hi - lo
    ids = np.zeros((BH, n, B), np.uint8)
    nib = np.zeros((BH, n, d // 2), np.uint8)
    w = np.zeros((BH, n, B), np.uint16)
    _check(lib().pariskv_debug_export(handle, lo, hi, ids.ctypes.data_as(C.c_void_p),
                                      nib.ctypes.data_as(C.c_void_p),
                                      w.ctypes.data_as(C.c_void_p)))
    return ids, nib, w


def pariskv_set_retrieval_path(handle, path):
    _check(lib().pariskv_set_retrieval_path(handle, int(path)))


def pariskv_retrieval_path(handle, k):
    r = lib().pariskv_retrieval_path(handle, int(k))
    if r < 0:
        _check(r)
    return r


def pariskv_retrieve_sizes(handle, k):
    E, Cn = C.c_int64(), C.c_int64()
    _check(lib().pariskv_retrieve_sizes(handle, int(k), C.byref(E), C.byref(Cn)))
    return E.value, Cn.value


def pariskv_debug_intermediate(handle, k, ws, which, BH, d=128):
    E, Cn = pariskv_retrieve_sizes(handle, k)
    shape, dt = {
        DEBUG_LUT: ((BH, 16, 256), np.uint8),   # the scan's byte-indexed table
        DEBUG_YQ: ((BH, d), np.float32),
        DEBUG_SCORES: ((BH, E), np.uint8),
        DEBUG_CAND: ((BH, Cn), np.int32),
        DEBUG_EST: ((BH, Cn), np.float32),
        DEBUG_THRESH: ((BH, 4), np.int32),
    }[which]
    out = np.zeros(shape, dt)
    _check(lib().pariskv_debug_intermediate(handle, int(k), _ptr(ws), _nbytes(ws),
                                            which, out.ctypes.data_as(C.c_void_p),
                                            out.nbytes))
    return out


def pariskv_codebook(m: int):
    L = np.zeros(8, np.float32)
    t = np.zeros(7, np.float32)
    _check(lib().pariskv_codebook(m, L.ctypes.data_as(C.c_void_p),
                                  t.ctypes.data_as(C.c_void_p)))
    return L, t


def pariskv_rot_scale(d: int) -> np.float32:
    return np.float32(lib().pariskv_rot_scale(d))


def pariskv_srht_signs_from_seed(seed: int, d: int) -> np.ndarray:
    """The rotation's signs (int8 +-1, [d]) from a 64-bit seed."""
    out = np.zeros(d, np.int8)
    _check(lib().pariskv_srht_signs_from_seed(int(seed) & (2 ** 64 - 1), int(d),
                                              out.ctypes.data_as(C.c_void_p)))
    return out


# ------------------------------------------------------ convenience holder --

class Layer:
    """One layer's index over caller-owned torch device buffers.

    Allocates the index buffer and the retrieval / attention workspaces as
    torch uint8 tensors on `device` (plumbing only) and keeps the handle.
    """

    def __init__(self, cfg, signs, K, n_keys, *, k, device="cuda", stream=None):
        import torch
        self.cfg = cfg
        self.k = int(k)
        # retrieval units: (b, KV head), or (b, query head) when unshared
        self.BH = cfg.batch * (cfg.n_q_heads if cfg.per_query_head else cfg.n_kv_heads)
        self.index_buf = torch.empty(pariskv_index_bytes(cfg), dtype=torch.uint8,
                                     device=device)
        self.ws = torch.empty(pariskv_retrieve_workspace_bytes(cfg, self.k),
                              dtype=torch.uint8, device=device)
        self.attn_ws = torch.empty(
            pariskv_attn_workspace_bytes(cfg.batch, cfg.n_q_heads, self.k,
                                         cfg.head_dim),
            dtype=torch.uint8, device=device)
        self.handle = pariskv_build_index(cfg, signs, self.index_buf, K,
                                          K.shape[2], n_keys, stream)

    @property
    def size(self) -> int:
        return pariskv_index_size(self.handle)

    def append(self, K_new, n_new, rows_per_head=None, stream=None):
        pariskv_append_keys(self.handle, K_new,
                            rows_per_head if rows_per_head is not None
                            else K_new.shape[2], n_new, stream)

    def set_path(self, path):
        pariskv_set_retrieval_path(self.handle, path)

    @property
    def path(self) -> int:
        return pariskv_retrieval_path(self.handle, self.k)

    def retrieve(self, Q, out_idx, out_est=None, stream=None):
        pariskv_retrieve_topk(self.handle, Q, self.k, out_idx, out_est, self.ws,
                              stream)

    def attend_workspace(self):
        """The workspace of retrieve_attend (allocated on first use)."""
        import torch
        if getattr(self, "ra_ws", None) is None:
            self.ra_ws = torch.empty(pariskv_retrieve_attend_workspace_bytes(self.cfg, self.k),
                                     dtype=torch.uint8, device=self.ws.device)
        return self.ra_ws

    def retrieve_attend(self, Q, K, V, out_idx, out, out_est=None, scale=None, stream=None):
        """Retrieval and the attention over the selected rows in one call."""
        self.attend_workspace()
        c = self.cfg
        pariskv_retrieve_attend(self.handle, Q, K, V, K.shape[2], self.k,
                                scale if scale is not None else c.head_dim ** -0.5,
                                out_idx, out_est, out, self.ra_ws, stream)

    def attend(self, Q, K, V, idx, out, scale=None, stream=None):
        c = self.cfg
        fn = pariskv_sparse_attn_per_query_head if c.per_query_head else pariskv_sparse_attn
        fn(Q, K, V, K.shape[2], idx, self.k, c.batch, c.n_q_heads, c.n_kv_heads,
           c.head_dim, c.key_dtype, scale if scale is not None else c.head_dim ** -0.5,
           out, self.attn_ws, stream)

    def close(self):
        if self.handle:
            pariskv_index_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------- Self-Indexing ----

PARISKV_SI_STAGES = 6
SI_DEBUG_LUT, SI_DEBUG_SCORES, SI_DEBUG_META = 0, 1, 2


def make_si_config(*, head_dim=128, n_sink=0, batch=1, n_kv_heads=1, n_q_heads=1,
                   key_dtype=PARISKV_DTYPE_BF16, capacity=4096):
    c = pariskv_si_config()
    c.head_dim, c.n_sink, c.batch = head_dim, n_sink, batch
    c.n_kv_heads, c.n_q_heads, c.key_dtype, c.capacity = (n_kv_heads, n_q_heads,
                                                          key_dtype, capacity)
    return c


def si_config_for(w, capacity=None):
    """pariskv_si_config for a synth.Workload (its shapes and sinks)."""
    return make_si_config(head_dim=w.d, n_sink=w.sinks, batch=w.batch,
                          n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads,
                          key_dtype=PARISKV_DTYPE_BF16 if w.dtype == "bf16"
                          else PARISKV_DTYPE_FP32, capacity=capacity or w.N)


def _size_call(fn, *args) -> int:
    n = C.c_size_t()
    _check(fn(*args, C.byref(n)))
    return n.value


def pariskv_si_index_bytes(cfg) -> int:
    return _size_call(lib().pariskv_si_index_bytes, C.byref(cfg))


def pariskv_si_build_workspace_bytes(cfg, n_keys) -> int:
    return _size_call(lib().pariskv_si_build_workspace_bytes, C.byref(cfg), int(n_keys))


def pariskv_si_retrieve_workspace_bytes(cfg, k) -> int:
    return _size_call(lib().pariskv_si_retrieve_workspace_bytes, C.byref(cfg), int(k))


def pariskv_si_build_index(cfg, index_buf, K, k_rows_per_head, n_keys, build_ws,
                           stream=None):
    h = C.c_void_p()
    _check(lib().pariskv_si_build_index(C.byref(cfg), _ptr(index_buf), _nbytes(index_buf),
                                        _ptr(K), int(k_rows_per_head), int(n_keys),
                                        _ptr(build_ws), _nbytes(build_ws),
                                        _stream(stream), C.byref(h)))
    return h


def pariskv_si_append_keys(handle, K_new, new_rows_per_head, n_new, stream=None):
    _check(lib().pariskv_si_append_keys(handle, _ptr(K_new), int(new_rows_per_head),
                                        int(n_new), _stream(stream)))


def pariskv_si_index_size(handle) -> int:
    return int(lib().pariskv_si_index_size(handle))


def pariskv_si_index_destroy(handle):
    lib().pariskv_si_index_destroy(handle)


def pariskv_si_retrieve_topk(handle, Q, k, out_idx, out_score, ws, stream=None):
    _check(lib().pariskv_si_retrieve_topk(handle, _ptr(Q), int(k), _ptr(out_idx),
                                          _ptr(out_score), _ptr(ws), _nbytes(ws),
                                          _stream(stream)))


def pariskv_si_retrieve_topk_profiled(handle, Q, k, out_idx, out_score, ws, events,
                                      stream=None):
    _check(lib().pariskv_si_retrieve_topk_profiled(
        handle, _ptr(Q), int(k), _ptr(out_idx), _ptr(out_score), _ptr(ws), _nbytes(ws),
        _stream(stream), _events(events)))


def pariskv_si_debug_export(handle, lo, hi, BH, d=128):
    n = hi - lo
    ids = np.zeros((BH, n, d // 4), np.uint8)
    mean = np.zeros((BH, d), np.float32)
    cb = np.zeros((BH, d // 4, 16, 4), np.float32)
    _check(lib().pariskv_si_debug_export(handle, int(lo), int(hi),
                                         ids.ctypes.data_as(C.c_void_p),
                                         mean.ctypes.data_as(C.c_void_p),
                                         cb.ctypes.data_as(C.c_void_p)))
    return ids, mean, cb


def pariskv_si_debug_intermediate(handle, k, ws, which, BH, E, d=128):
    shape, dt = {
        SI_DEBUG_LUT: ((BH, d // 4, 16), np.float32),
        SI_DEBUG_SCORES: ((BH, E), np.float32),
        SI_DEBUG_META: ((BH, 4), np.int32),
    }[which]
    out = np.zeros(shape, dt)
    _check(lib().pariskv_si_debug_intermediate(handle, int(k), _ptr(ws), _nbytes(ws), which,
                                               out.ctypes.data_as(C.c_void_p),
                                               out.nbytes))
    return out


class SiLayer:
    """One layer's Self-Indexing index over torch device buffers (the index,
    the build scratch, released after the build, and the retrieval and
    attention workspaces)."""

    def __init__(self, cfg, K, n_keys, *, k, device="cuda", stream=None):
        import torch
        self.cfg = cfg
        self.k = int(k)
        self.BH = cfg.batch * cfg.n_kv_heads
        self.index_buf = torch.empty(pariskv_si_index_bytes(cfg), dtype=torch.uint8,
                                     device=device)
        build_ws = torch.empty(pariskv_si_build_workspace_bytes(cfg, n_keys),
                               dtype=torch.uint8, device=device)
        self.ws = torch.empty(pariskv_si_retrieve_workspace_bytes(cfg, self.k),
                              dtype=torch.uint8, device=device)
        self.attn_ws = torch.empty(
            pariskv_attn_workspace_bytes(cfg.batch, cfg.n_q_heads, self.k, cfg.head_dim),
            dtype=torch.uint8, device=device)
        self.handle = pariskv_si_build_index(cfg, self.index_buf, K, K.shape[2], n_keys,
                                             build_ws, stream)
        # the build's kernels must finish before the scratch is released
        (stream or torch.cuda.current_stream()).synchronize()
        del build_ws

    @property
    def size(self) -> int:
        return pariskv_si_index_size(self.handle)

    def append(self, K_new, n_new, rows_per_head=None, stream=None):
        pariskv_si_append_keys(self.handle, K_new,
                               rows_per_head if rows_per_head is not None
                               else K_new.shape[2], n_new, stream)

    def retrieve(self, Q, out_idx, out_score=None, stream=None):
        pariskv_si_retrieve_topk(self.handle, Q, self.k, out_idx, out_score, self.ws, stream)

    def attend(self, Q, K, V, idx, out, scale=None, stream=None):
        c = self.cfg
        pariskv_sparse_attn(Q, K, V, K.shape[2], idx, self.k, c.batch, c.n_q_heads,
                            c.n_kv_heads, c.head_dim, c.key_dtype,
                            scale if scale is not None else c.head_dim ** -0.5, out,
                            self.attn_ws, stream)

    def close(self):
        if self.handle:
            pariskv_si_index_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
