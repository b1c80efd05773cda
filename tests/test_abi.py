"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every symbol include/pariskv.h declares, validates arguments on the host,
sizes buffers, and its constants agree with the oracle's independently
derived ones.  No kernel is launched here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pariskv.h")


@pytest.fixture(scope="module")
def pk():
    import kv_cache_top_srht_amd as pk
    pk.lib()
    return pk


def declared_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"PARISKV_API\s+[\w\s\*]+?\b(pariskv_\w+)\s*\(",
                                 src, re.S)))


def test_exports_every_declared_symbol(pk):
    names = declared_symbols()
    assert len(names) >= 18
    L = C.CDLL(pk.SO_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_no_oracle_in_product():
    """The product package neither imports nor links the oracle."""
    pkg = os.path.join(ROOT, "kv_cache_top_srht_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "liboracle" not in txt and "oracle.c" not in txt, f


def test_codebook_matches_oracle(pk, orc):
    for m in (4, 8):
        L, t = pk.pariskv_codebook(m)
        L2, t2 = orc.codebook_f32(m)
        assert np.array_equal(L.view(np.uint32), L2.view(np.uint32))
        assert np.array_equal(t.view(np.uint32), t2.view(np.uint32))


def test_rot_scale_matches_oracle(pk, orc):
    for d in (2, 8, 64, 128, 256, 1024):
        assert pk.pariskv_rot_scale(d) == orc.rot_scale(d)


def test_seeded_signs_match_oracle(pk, orc):
    """The library's seed -> signs helper and the oracle's own SplitMix64
    give the same rotation diagonal (the generator itself is pinned by its
    known answers in the oracle's tests)."""
    for seed in (0, 1, 2 ** 63 + 12345, 2 ** 64 - 1):
        for d in (1, 64, 128, 1024):
            assert np.array_equal(pk.pariskv_srht_signs_from_seed(seed, d),
                                  orc.srht_signs(seed, d))
    with pytest.raises(Exception):
        pk.pariskv_srht_signs_from_seed(1, 0)


def test_sizes(pk):
    c = pk.make_config(capacity=1 << 20, batch=1, n_kv_heads=8, n_q_heads=32)
    # ids 16 B + a 128-byte record (codes 64 B + w 32 B) per key and head
    assert pk.pariskv_index_bytes(c) == 8 * (1 << 20) * 144
    ws = pk.pariskv_retrieve_workspace_bytes(c, 4096)
    assert 8 * (1 << 20) < ws < 64 * (1 << 20)
    # one 132-float partial per query head and 32-row chunk of the k rows
    assert pk.pariskv_attn_workspace_bytes(1, 32, 4096, 128) == 32 * 128 * 132 * 4


@pytest.mark.parametrize("field,value,rc", [
    ("head_dim", 96, -1), ("head_dim", 64, -2), ("n_subspaces", 32, 0),
    ("n_subspaces", 8, -1),
    ("n_subspaces", 7, -1), ("rho", 0, -1), ("rho", 9, -1),
    ("cand_num", 0, -1), ("cand_den", 0, -1), ("n_q_heads", 30, -1),
    ("key_dtype", 5, -1), ("capacity", 0, -1), ("n_sink", -1, -1),
    ("n_q_heads", 24, -2), ("n_q_heads", 128, -2), ("per_query_head", 2, -1),
])
def test_config_validation(pk, field, value, rc):
    c = pk.make_config(capacity=4096)
    setattr(c, field, value)
    n = C.c_size_t()
    assert pk.lib().pariskv_index_bytes(C.byref(c), C.byref(n)) == rc


def test_tier_overflow_rejected(pk):
    c = pk.make_config(capacity=4096, tiers=(16, 3, 2, 1))
    n = C.c_size_t()
    assert pk.lib().pariskv_index_bytes(C.byref(c), C.byref(n)) == -1
    # 32 subspaces of 4: the largest score is 32 times the top tier
    c = pk.make_config(capacity=4096, tiers=(7, 3, 2, 1))
    c.n_subspaces = 32
    assert pk.lib().pariskv_index_bytes(C.byref(c), C.byref(n)) == 0
    c = pk.make_config(capacity=4096, tiers=(8, 3, 2, 1))
    c.n_subspaces = 32
    assert pk.lib().pariskv_index_bytes(C.byref(c), C.byref(n)) == -1
    # 64 subspaces of 2: a valid configuration this build has no kernels for
    c = pk.make_config(capacity=4096, tiers=(3, 2, 1, 1))
    c.n_subspaces = 64
    assert pk.lib().pariskv_index_bytes(C.byref(c), C.byref(n)) == -2


def test_host_side_argument_errors(pk):
    lib = pk.lib()
    c = pk.make_config(capacity=4096, batch=1, n_kv_heads=1, n_q_heads=4)
    h = C.c_void_p()
    signs = np.ones(128, np.int8)
    sp = signs.ctypes.data_as(C.c_void_p)
    # null index buffer
    assert lib.pariskv_build_index(C.byref(c), sp, None, 0, None, 0, 0, None,
                                   C.byref(h)) == -1
    # buffer too small (fake, never dereferenced: rejected before launch)
    fake = C.c_void_p(0x10000000)
    assert lib.pariskv_build_index(C.byref(c), sp, fake, 10, None, 0, 0, None,
                                   C.byref(h)) == -4
    # capacity
    assert lib.pariskv_build_index(C.byref(c), sp, fake, 1 << 30, fake, 8192,
                                   8192, None, C.byref(h)) == -3
    # signs must be +-1
    bad = np.zeros(128, np.int8)
    assert lib.pariskv_build_index(C.byref(c), bad.ctypes.data_as(C.c_void_p),
                                   fake, 1 << 30, None, 0, 0, None,
                                   C.byref(h)) == -1
    # an empty build creates a handle without launching anything
    assert lib.pariskv_build_index(C.byref(c), sp, fake, 1 << 30, None, 0, 0,
                                   None, C.byref(h)) == 0
    assert lib.pariskv_index_size(h) == 0
    out = C.c_void_p(0x20000000)
    # k > N
    assert lib.pariskv_retrieve_topk(h, fake, 10, out, None, fake, 1 << 30,
                                     None) == -1
    assert lib.pariskv_append_keys(h, fake, 5000, 5000, None) == -3
    assert lib.pariskv_append_keys(h, fake, 10, 20, None) == -1
    assert lib.pariskv_append_keys(h, None, 1, 1, None) == -1
    lib.pariskv_index_destroy(h)
    # attention: unsupported group size / head_dim
    assert lib.pariskv_sparse_attn(fake, fake, fake, 10, fake, 4, 1, 3, 1, 128,
                                   0, C.c_float(0.1), fake, fake, 1 << 20,
                                   None) == -2
    assert lib.pariskv_sparse_attn(fake, fake, fake, 10, fake, 4, 1, 4, 1, 64,
                                   0, C.c_float(0.1), fake, fake, 1 << 20,
                                   None) == -2
    assert lib.pariskv_sparse_attn(fake, fake, fake, 10, fake, 4, 1, 4, 1, 128,
                                   0, C.c_float(0.1), fake, fake, 16,
                                   None) == -4


def test_status_strings(pk):
    for rc in range(0, -7, -1):
        assert pk.pariskv_status_string(rc) != "unknown status"
    assert [pk.pariskv_stage_name(s) for s in range(6)] == [
        "query_prep", "vote_scan", "threshold", "compact_rerank",
        "topk", "topk_second_pass"]
    assert pk.pariskv_stage_name(6) is None
