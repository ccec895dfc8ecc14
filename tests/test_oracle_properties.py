"""Property tests of the CPU oracle (hypothesis) over random small shapes.

Every property is fixed by the mathematics, not by the oracle itself: exact
integer or dyadic arithmetic (fp32 represents those sums exactly, so any
summation order gives the same bits), the symmetry and pair count of the
Gram matrix, the linearity of sum pooling, and the plain chain rule through
the interaction in exact integer arithmetic.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def bag_cases(draw, max_k=4, max_b=6, max_d=12, max_rows=20, max_len=6):
    """K tables (rows per table 1..max_rows), B bags per table (lengths
    0..max_len: empty bags included), integer table values in [-64, 64]."""
    K = draw(st.integers(1, max_k))
    B = draw(st.integers(1, max_b))
    d = draw(st.integers(1, max_d))
    rows = [draw(st.integers(1, max_rows)) for _ in range(K)]
    seed = draw(st.integers(0, 2**31 - 1))
    g = np.random.default_rng(seed)
    lens = g.integers(0, max_len + 1, size=K * B)
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    idx = np.concatenate([g.integers(0, rows[k], size=off[(k + 1) * B] - off[k * B]) for k in range(K)]
                         + [np.zeros(0, dtype=np.int64)]).astype(np.int64)
    tabs = [g.integers(-64, 65, size=(rows[k], d)).astype(np.float32) for k in range(K)]
    return K, B, d, rows, tabs, idx, off, g


def _brute_pool(tabs, idx, off, B, d):
    """int64 sums over each bag (exact)."""
    K = len(tabs)
    out = np.zeros((B, K * d), dtype=np.int64)
    for k in range(K):
        for b in range(B):
            a, e = off[k * B + b], off[k * B + b + 1]
            for p in range(a, e):
                out[b, k * d:(k + 1) * d] += tabs[k][idx[p]].astype(np.int64)
    return out


@SETTINGS
@given(bag_cases())
def test_prop_embbag_integer_tables_equal_integer_sums(orc, case):
    K, B, d, rows, tabs, idx, off, _ = case
    got = orc.embbag_fwd(tabs, idx, off, B)
    assert np.array_equal(got.astype(np.int64), _brute_pool(tabs, idx, off, B, d))
    # an empty bag is +0.0, never -0.0
    for k in range(K):
        for b in range(B):
            if off[k * B + b] == off[k * B + b + 1]:
                assert not np.signbit(got[b, k * d:(k + 1) * d]).any()


@SETTINGS
@given(bag_cases())
def test_prop_embbag_linear_in_the_tables(orc, case):
    """pool(T1 + T2) = pool(T1) + pool(T2) bit for bit on dyadic tables (every
    partial sum is exact in fp32)."""
    K, B, d, rows, tabs, idx, off, g = case
    t1 = [t / 8.0 for t in tabs]
    t2 = [g.integers(-64, 65, size=t.shape).astype(np.float32) / 16.0 for t in tabs]
    s = [(a + b).astype(np.float32) for a, b in zip(t1, t2)]
    lhs = orc.embbag_fwd(s, idx, off, B)
    rhs = orc.embbag_fwd(t1, idx, off, B) + orc.embbag_fwd(t2, idx, off, B)
    assert np.array_equal(lhs, rhs)


@SETTINGS
@given(bag_cases())
def test_prop_embbag_bag_permutation(orc, case):
    """Reordering the bags of the batch reorders the pooled rows the same way."""
    K, B, d, rows, tabs, idx, off, g = case
    perm = g.permutation(B)
    lens = np.diff(off)
    new_idx, new_lens = [], []
    for k in range(K):
        for b in perm:
            a, e = off[k * B + b], off[k * B + b + 1]
            new_idx.append(idx[a:e])
            new_lens.append(lens[k * B + b])
    new_off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(new_lens, out=new_off[1:])
    new_idx = np.concatenate(new_idx + [np.zeros(0, dtype=np.int64)]).astype(np.int64)
    a = orc.embbag_fwd(tabs, idx, off, B)
    b = orc.embbag_fwd(tabs, new_idx, new_off, B)
    assert np.array_equal(a[perm], b)


@SETTINGS
@given(st.integers(2, 10), st.integers(1, 16), st.integers(1, 4), st.integers(0, 2**31 - 1))
def test_prop_interact_integer_gram(orc, n, d, B, seed):
    """Pairs equal the exact integer dot products, strict lower triangle,
    row-major; the dense part is X[0]; the Gram matrix is symmetric."""
    g = np.random.default_rng(seed)
    X = g.integers(-8, 9, size=(B, n, d)).astype(np.float32)
    out = orc.interact_fwd(X)
    P = n * (n - 1) // 2
    assert out.shape == (B, d + P)
    Xi = X.astype(np.int64)
    for b in range(B):
        assert np.array_equal(out[b, :d], X[b, 0])
        gram = Xi[b] @ Xi[b].T
        assert np.array_equal(gram, gram.T)
        col = d
        for i in range(n):
            for j in range(i):
                assert out[b, col] == gram[i, j]
                col += 1


@SETTINGS
@given(st.integers(2, 9), st.integers(1, 12), st.integers(1, 3), st.integers(0, 2**31 - 1))
def test_prop_interact_bwd_integer_chain_rule(orc, n, d, B, seed):
    """dX_i = [i = 0] g_dense + sum over pairs (i, j) and (j, i) of g_pair X_j,
    computed exactly in int64."""
    g = np.random.default_rng(seed)
    X = g.integers(-6, 7, size=(B, n, d)).astype(np.float32)
    P = n * (n - 1) // 2
    G = g.integers(-6, 7, size=(B, d + P)).astype(np.float32)
    got = orc.interact_bwd(X, G)
    Xi, Gi = X.astype(np.int64), G.astype(np.int64)
    for b in range(B):
        ref = np.zeros((n, d), dtype=np.int64)
        ref[0] += Gi[b, :d]
        col = d
        for i in range(n):
            for j in range(i):
                ref[i] += Gi[b, col] * Xi[b, j]
                ref[j] += Gi[b, col] * Xi[b, i]
                col += 1
        assert np.array_equal(got[b].astype(np.int64), ref)


@SETTINGS
@given(bag_cases(max_len=5), st.integers(1, 5))
def test_prop_sparse_sgd_dyadic_exact(orc, case, lr_log2):
    """With dyadic tables, gradients and lr = 2^-j every sum and product is
    exact: each touched row becomes T - lr * (sum of its occurrences' bag
    gradients), every other row is unchanged."""
    K, B, d, rows, tabs, idx, off, g = case
    lr = 2.0 ** -lr_log2
    T0 = [t / 4.0 for t in tabs]
    G = (g.integers(-32, 33, size=(B, (K + 1) * d)).astype(np.float32) / 8.0).astype(np.float32)
    tabs_dev = [t.copy() for t in T0]
    orc.embbag_bwd_sgd(tabs_dev, idx, off, B, G, d, lr)
    ref = [t.astype(np.float64).copy() for t in T0]
    acc = [np.zeros_like(r) for r in ref]
    touched = [np.zeros(r.shape[0], dtype=bool) for r in ref]
    for k in range(K):
        for b in range(B):
            for p in range(off[k * B + b], off[k * B + b + 1]):
                acc[k][idx[p]] += G[b, d + k * d:d + (k + 1) * d]
                touched[k][idx[p]] = True
    for k in range(K):
        exp = ref[k] - lr * acc[k]
        assert np.array_equal(tabs_dev[k][touched[k]], exp[touched[k]].astype(np.float32))
        assert np.array_equal(tabs_dev[k][~touched[k]], T0[k][~touched[k]])


@SETTINGS
@given(st.lists(st.floats(min_value=-2.0**100, max_value=2.0**100, allow_nan=False, width=32), min_size=1, max_size=64))
def test_prop_bf16_round_nearest_neighbour(orc, xs):
    """bf16 rounding keeps bf16 values, is monotone, and returns the nearer of
    the two bf16 values that bracket its input (the one with an even last
    mantissa bit on a tie)."""
    x = np.array(sorted(xs), dtype=np.float32)
    r = orc.bf16_round(x)
    assert np.array_equal(orc.bf16_round(r), r)
    assert np.all(np.diff(r) >= 0)
    rb = r.view(np.uint32)
    assert np.all((rb & 0xFFFF) == 0)
    lo_bits = x.view(np.uint32) & np.uint32(0xFFFF0000)       # toward zero
    hi_bits = lo_bits + np.uint32(0x10000)                      # away from zero
    lo, hi = lo_bits.view(np.float32), hi_bits.view(np.float32)
    assert np.all((rb == lo_bits) | (rb == hi_bits))
    xd = x.astype(np.float64)
    dlo, dhi = np.abs(xd - lo), np.abs(xd - hi)
    assert np.all(np.where(dlo < dhi, rb == lo_bits, True))
    assert np.all(np.where(dhi < dlo, rb == hi_bits, True))
    tie = dlo == dhi
    assert np.all(np.where(tie, (rb & np.uint32(0x10000)) == 0, True))
