"""Pins for the oracle's Self-Indexing functions ("Self-Indexing KVCache:
Predicting Sparse Attention from Compressed Keys", Methodology A-C): each
checked against closed forms on designed inputs, invariants the method
implies, and a second route to the same quantity.
"""
import numpy as np

D = 128


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def skewed_keys(n, d, seed):
    r = rng(seed)
    s = np.exp(0.5 * r.standard_normal(d))
    s[r.choice(d, 4, replace=False)] *= 8
    return (r.standard_normal((n, d)) * s).astype(np.float32)


def dyadic(r, shape, lo=1, hi=64):
    """Values k/8 with 1 <= |k| < 64 and random signs: sums of a few hundred
    of them are exact in fp32 and fp64."""
    v = r.integers(lo, hi, shape) / 8.0
    return (v * np.where(r.integers(0, 2, shape) == 1, -1.0, 1.0)).astype(np.float32)


def test_si_mean_is_channel_mean_of_indexed_keys(orc):
    """Keys t + z_i and t - z_i in pairs (dyadic values): the channel mean of
    the indexed keys is exactly t; the sink rows, whatever they hold, do not
    enter it; and the two keys of a pair get complementary sign ids."""
    r = rng(1)
    S, m = 5, 200
    t = (r.integers(-40, 40, D) / 16.0).astype(np.float32)
    z = dyadic(r, (m, D))
    X = np.concatenate([r.standard_normal((S, D)).astype(np.float32) * 100,
                        t + z, t - z]).astype(np.float32)
    mean, ids, cb = orc.si_build(X, S)
    assert np.array_equal(mean, t)
    assert np.array_equal(ids[S:S + m], 15 - ids[S + m:])        # z has no zeros
    # sinks are outside the means and the codebook
    X2 = X.copy()
    X2[:S] = -X2[:S] + 3
    mean2, ids2, cb2 = orc.si_build(X2, S)
    assert np.array_equal(mean2, mean) and np.array_equal(cb2, cb)
    assert np.array_equal(ids2[S:], ids[S:])


def test_si_ids_are_sign_patterns_of_centred_keys(orc):
    X = skewed_keys(500, D, 2)
    mean, ids, cb = orc.si_build(X, 0)
    Y = X.astype(np.float64) - mean.astype(np.float64)
    want = np.zeros((500, D // 4), np.int64)
    for j in range(4):
        want += (Y[:, j::4] < 0).astype(np.int64) << j
    near = np.abs(Y) < 1e-6 * np.abs(X).max()
    ok = ~near.reshape(500, D // 4, 4).any(axis=2)
    assert np.array_equal(ids[ok], want[ok])
    # appended keys are coded with the same means
    assert np.array_equal(orc.si_ids(X[100:300], mean), ids[100:300])


def test_si_translation_invariance(orc):
    """A dyadic shift of every key moves the means by the shift and leaves the
    centred keys, hence ids and centroids, bit for bit unchanged (256
    indexed keys: the means are exact)."""
    r = rng(3)
    X = dyadic(r, (263, D))
    shift = (r.integers(-20, 20, D) / 4.0).astype(np.float32)
    a = orc.si_build(X, 7)
    b = orc.si_build((X + shift).astype(np.float32), 7)
    assert np.array_equal(b[0], a[0] + shift)
    assert np.array_equal(b[1], a[1]) and np.array_equal(b[2], a[2])


def test_si_centroids_are_cluster_means(orc):
    """Each non-empty centroid has its cluster's sign pattern, and the
    count-weighted centroids add up to the sum of the centred keys (about
    zero): a wrong count, a missing centring or a swapped index fails."""
    X = skewed_keys(3000, D, 4)
    S = 40
    mean, ids, cb = orc.si_build(X, S)
    Y = X[S:].astype(np.float64) - mean.astype(np.float64)
    for b in range(D // 4):
        cnt = np.bincount(ids[S:, b], minlength=16)
        for p in range(16):
            if cnt[p] == 0:
                assert not cb[b, p].any()
                continue
            for j in range(4):
                if (p >> j) & 1:
                    assert cb[b, p, j] < 0
                else:
                    assert cb[b, p, j] >= 0
        tot = (cnt[:, None] * cb[b].astype(np.float64)).sum(axis=0)
        ysum = Y[:, 4 * b:4 * b + 4].sum(axis=0)
        scale = np.abs(Y[:, 4 * b:4 * b + 4]).sum(axis=0)
        assert np.all(np.abs(tot - ysum) <= 1e-6 * scale)
        assert np.all(np.abs(ysum) <= 1e-3 * scale)


def test_si_exact_when_clusters_are_pure(orc):
    """Closed form: when every member of a cluster is the same vector (and
    the keys are symmetric, so the means are 0), each centroid is that
    vector and the score is the exact inner product <qbar, k>."""
    r = rng(5)
    base = np.abs(dyadic(r, (D // 4, 16, 4)))
    sgn = np.array([[-1.0 if (p >> j) & 1 else 1.0 for j in range(4)] for p in range(16)])
    V = (base * sgn[None]).astype(np.float32)           # V[b, p] has sign pattern p
    # V[b, 15 - p] = -V[b, p], so a key and its negation use paired clusters
    V[:, 8:] = -V[:, 7::-1]
    n = 300
    P = r.integers(0, 16, (n, D // 4))
    K = V[np.arange(D // 4)[None], P].reshape(n, D)
    X = np.concatenate([K, -K]).astype(np.float32)
    mean, ids, cb = orc.si_build(X, 0)
    assert not mean.any()
    assert np.array_equal(ids[:n], P)
    used = np.zeros((D // 4, 16), bool)
    used[np.arange(D // 4)[None], P] = True
    used[np.arange(D // 4)[None], 15 - P] = True
    assert np.array_equal(cb[used], V[used])
    Q = skewed_keys(4, D, 6)
    lut = orc.si_lut(Q, cb)
    sc = orc.si_scores(ids, lut, 0)
    qbar = Q.astype(np.float64).mean(axis=0)
    truth = X.astype(np.float64) @ qbar
    scale = np.abs(X).astype(np.float64) @ np.abs(qbar)
    assert np.all(np.abs(sc - truth) <= 1e-5 * scale)


def test_si_score_equals_dot_with_reconstruction(orc):
    """Second route: the LUT-GEMV score of a key equals <qbar, k_hat>, k_hat
    the concatenation of its centroids (fp64 matmul), to fp32 rounding."""
    X = skewed_keys(2000, D, 7)
    mean, ids, cb = orc.si_build(X, 16)
    Q = skewed_keys(2, D, 8)
    lut = orc.si_lut(Q, cb)
    sc = orc.si_scores(ids, lut, 16)
    khat = cb[np.arange(D // 4)[None], ids[16:].astype(np.int64)].reshape(-1, D)
    qbar = (Q[0].astype(np.float32) + Q[1]) * np.float32(0.5)
    truth = khat.astype(np.float64) @ qbar.astype(np.float64)
    scale = np.abs(khat).astype(np.float64) @ np.abs(qbar).astype(np.float64)
    assert np.all(np.abs(sc - truth) <= 2e-6 * scale)
    # the lookup table itself: <qbar_b, c_{b,p}>
    ref = np.einsum("bj,bpj->bp", qbar.reshape(D // 4, 4).astype(np.float64),
                    cb.astype(np.float64))
    assert np.all(np.abs(lut - ref) <= 1e-6 * (np.abs(qbar).max() * np.abs(cb).max() * 4))


def test_si_retrieval_prefers_high_inner_products(orc):
    """The selection is the top-k by score (sinks first), and on skewed keys
    the scores track the true inner products (a coarse property: the pages
    give no error bound)."""
    X = skewed_keys(4000, D, 9)
    S, k = 8, 200
    mean, ids, cb = orc.si_build(X, S)
    Q = skewed_keys(4, D, 10)
    out = orc.si_retrieve_head(Q, ids, cb, S=S, k=k)
    assert np.array_equal(out["idx"][:S], np.arange(S))
    sel = out["idx"][S:]
    assert np.all(np.diff(sel) > 0)
    sc = out["scores"]
    order = np.lexsort((np.arange(len(sc)), -sc))[:k - S] + S
    assert np.array_equal(np.sort(order), sel)
    truth = X[S:].astype(np.float64) @ Q.astype(np.float64).mean(axis=0)
    assert np.corrcoef(sc, truth)[0, 1] > 0.7


def test_si_score_is_the_sum_of_its_lut_entries(orc):
    """[SI] Methodology B defines a key's score as the sum of its LUT entries.
    Dyadic entries (small integers times 2^-6) make every fp32 sum exact, so
    the oracle must equal the exact sum; for arbitrary entries it must lie
    within the forward-error bound of a sequential fp32 sum of B terms,
    gamma_{B-1} * sum |entries| (Higham, Accuracy and Stability, 4.2)."""
    r = rng(11)
    B, n = D // 4, 3000
    ids = r.integers(0, 16, (n, B)).astype(np.uint8)
    lut = (r.integers(-512, 513, (B, 16)) * 2.0 ** -6).astype(np.float32)
    terms = lut.astype(np.float64)[np.arange(B)[None], ids.astype(np.int64)]
    sc = orc.si_scores(ids, lut, 5)
    assert np.array_equal(sc.astype(np.float64), terms[5:].sum(axis=1))
    lut = r.standard_normal((B, 16)).astype(np.float32)
    terms = lut.astype(np.float64)[np.arange(B)[None], ids.astype(np.int64)]
    sc = orc.si_scores(ids, lut, 0)
    u = 2.0 ** -24
    gamma = (B - 1) * u / (1 - (B - 1) * u)
    assert np.all(np.abs(sc - terms.sum(axis=1)) <= gamma * np.abs(terms).sum(axis=1))
    # a term left out or taken from the wrong sub-vector breaks the bound
    assert np.any(np.abs(terms[:, 1:].sum(axis=1) - terms.sum(axis=1)) >
                  gamma * np.abs(terms).sum(axis=1))
