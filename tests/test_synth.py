"""Input generators: counter-based table values, permutation, Zipf, recipes."""
import math

import numpy as np
import pytest

from synth import rng as R
from synth import workloads as W


def test_splitmix64_published_outputs():
    # First four outputs of SplitMix64 seeded with 0 (Steele, Lea & Flood 2014;
    # the widely reproduced reference sequence used to seed xoshiro generators).
    got = [int(x) for x in R.splitmix64_stream(0, 4)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]


def test_fmix_scalar_matches_vector():
    xs = [0, 1, 2**63, 2**64 - 1, 0x123456789ABCDEF]
    assert [R.fmix_int(x) for x in xs] == [int(v) for v in R.fmix(np.array(xs, dtype=np.uint64))]


def test_table_values_range_and_exactness():
    rows, d = 1000, 16
    v = R.table_rows(7, 3, rows, np.arange(rows), d)
    a = float(R.table_scale(rows))
    assert v.dtype == np.float32 and v.shape == (rows, d)
    assert v.min() >= -a and v.max() < a
    # value = a * t with t = k * 2**-24 exactly, |k| <= 2**24: t is recoverable
    t = v.astype(np.float64) / a
    assert abs(t.mean()) < 0.02 and abs(t.var() - 1 / 3) < 0.02  # U(-1,1): mean 0, var 1/3
    # row subsets regenerate the same values
    sub = np.array([999, 0, 500, 500])
    assert np.array_equal(R.table_rows(7, 3, rows, sub, d), v[sub])
    # different tables and seeds differ
    assert not np.array_equal(R.table_rows(7, 4, rows, sub, d), v[sub])
    assert not np.array_equal(R.table_rows(8, 3, rows, sub, d), v[sub])


@pytest.mark.parametrize("m", [1, 2, 3, 17, 1000, 4099])
def test_feistel_is_bijection(m):
    p = R.FeistelPermutation(m, 12345)
    y = p(np.arange(m))
    assert y.min() >= 0 and y.max() < m
    assert np.unique(y).size == m


def test_zipf_matches_pmf():
    m, alpha, n = 50, 1.1, 400_000
    g = R.stream_rng(0, 99)
    r = R.zipf_ranks(g, m, alpha, n)
    pmf = np.arange(1, m + 1, dtype=np.float64) ** -alpha
    pmf /= pmf.sum()
    obs = np.bincount(r, minlength=m)
    chi2 = ((obs - n * pmf) ** 2 / (n * pmf)).sum()
    # 49 degrees of freedom: the 99.9% quantile is about 85
    assert chi2 < 85, chi2


def test_bag_lengths_and_offsets():
    w = W.get("embbag").scaled(B=4096, rows=1000, K=3)
    idx, off = W.indices_offsets(w)
    assert off.shape == (w.K * w.B + 1,) and off[0] == 0 and np.all(np.diff(off) >= 1)
    lens = np.diff(off)
    assert abs(lens.mean() - 20) < 0.5
    assert idx.min() >= 0 and idx.max() < 1000
    # deterministic
    idx2, off2 = W.indices_offsets(w)
    assert np.array_equal(idx, idx2) and np.array_equal(off, off2)


def test_workload_closed_forms():
    # Pairs n(n-1)/2 and top-MLP input widths d + pairs of the workloads.
    ws = W.workloads()
    assert (ws["tiny"].pairs, ws["tiny"].top_in) == (36, 52)
    assert (ws["forward"].pairs, ws["forward"].top_in) == (351, 479)
    assert (ws["interaction"].pairs, ws["interaction"].top_in) == (5050, 5114)
    assert (ws["train"].pairs, ws["train"].top_in) == (36, 164)
    for w in ws.values():
        if w.top:
            assert w.top[0] == w.top_in
        if w.bottom:
            assert w.bottom[-1] == w.d and w.bottom[0] == w.dense_dim


def test_forward_cardinalities():
    rows = W.get("forward").rows
    assert len(rows) == 26
    assert all(100 <= m <= 4e7 for m in rows)
    assert 1.8e8 <= sum(rows) <= 2.2e8


def test_compact_rows_roundtrip():
    w = W.get("tiny")
    idx, off = W.indices_offsets(w)
    tabs, local, row_ids = W.compact_rows(w, idx, off)
    for k in range(w.K):
        a, b = off[k * w.B], off[(k + 1) * w.B]
        assert np.array_equal(row_ids[k][local[a:b]], idx[a:b])
        full = R.table_rows(w.seed, k, w.rows[k], np.arange(w.rows[k]), w.d)
        assert np.array_equal(tabs[k], full[row_ids[k]])


def test_mlp_params_bf16_exact():
    w = W.get("forward")
    for Wf, bits, b in W.mlp_params(w, "bottom"):
        assert bits is not None and bits.dtype == np.uint16
        back = (bits.astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(back, Wf)
        fan_in = Wf.shape[1]
        sd = math.sqrt(2 / (fan_in + Wf.shape[0]))
        assert abs(Wf.std() - sd) < 0.2 * sd
