"""EmbeddingBag forward on the GPU against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from dlrm_cases import DEV, banner, bits, to_dev
from synth import device as SD
from synth import rng as R
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _run(tables_dev, idx, off, B, d, out_ld=None, col0=0, nnz=None):
    """nnz: None passes offsets[K*B] (the bench's call), -1 leaves the work
    split to the bag count alone."""
    import deep_learning_recommendation_amd as D

    K = len(tables_dev)
    out_ld = K * d if out_ld is None else out_ld
    out = torch.full((B, out_ld), float("nan"), dtype=torch.float32, device=DEV)
    ptrs = D.device_pointer_array(tables_dev)
    nnz = int(off[-1]) if nnz is None else nnz
    D.dlrm_embbag_fwd(ptrs, K, d, to_dev(idx), to_dev(off), B, out, out_ld, col0, nnz=nnz)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _rand_case(seed, K, B, d, rows, max_len, empty_frac=0.1):
    g = np.random.default_rng(seed)
    lens = g.integers(1, max_len + 1, size=K * B)
    lens[g.random(K * B) < empty_frac] = 0
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    idx = np.concatenate([g.integers(0, rows[k], size=off[(k + 1) * B] - off[k * B]) for k in range(K)])
    tabs = [g.standard_normal((rows[k], d)).astype(np.float32) for k in range(K)]
    return tabs, idx.astype(np.int64), off


@pytest.mark.parametrize("d", [4, 16, 64, 128, 132, 256, 260, 1024])
@pytest.mark.parametrize("max_len,nnz_known", [(45, True), (45, False), (2, True), (300, True)])
def test_embbag_random_ragged_bitexact(d, max_len, nnz_known):
    """Bag lengths set the bags per lane group (1 .. G - 1) when nnz is given."""
    K, B = 3, 701  # B not a multiple of any chunk size: ragged tail
    banner(f"embbag random d={d} K={K} B={B} max_len={max_len} nnz_known={nnz_known}")
    tabs, idx, off = _rand_case(d + max_len, K, B, d, [50, 333, 7], max_len)
    got = _run([to_dev(t) for t in tabs], idx, off, B, d, nnz=None if nnz_known else -1)
    ref = oracle.embbag_fwd(tabs, idx, off, B)
    assert np.array_equal(bits(got), bits(ref))


def test_embbag_strided_output_and_empty_bags():
    K, B, d = 4, 300, 32
    banner("embbag strided output")
    tabs, idx, off = _rand_case(7, K, B, d, [20, 20, 20, 20], 6, empty_frac=0.4)
    ld, col0 = (K + 3) * d + 8, d + 4
    got = _run([to_dev(t) for t in tabs], idx, off, B, d, out_ld=ld, col0=col0)
    ref = oracle.embbag_fwd(tabs, idx, off, B, out_ld=ld, out_col0=col0)
    sl = slice(col0, col0 + K * d)
    assert np.array_equal(bits(got[:, sl]), bits(ref[:, sl]))
    assert np.isnan(got[:, :col0]).all() and np.isnan(got[:, col0 + K * d:]).all()  # nothing else written
    empty = np.diff(off) == 0
    assert empty.any()


def test_embbag_all_bags_empty_and_single_bag():
    d = 16
    banner("embbag degenerate bags")
    tabs = [np.random.default_rng(0).standard_normal((5, d)).astype(np.float32)]
    off = np.zeros(9, dtype=np.int64)
    got = _run([to_dev(t) for t in tabs], np.zeros(1, np.int64), off, 8, d)
    assert np.all(got == 0) and not np.signbit(got).any()
    idx = np.array([4, 4, 0, 4], dtype=np.int64)
    off = np.array([0, 4], dtype=np.int64)
    got = _run([to_dev(t) for t in tabs], idx, off, 1, d)
    assert np.array_equal(bits(got), bits(oracle.embbag_fwd(tabs, idx, off, 1)))


def test_embbag_tiny_workload_equals_row_lookup():
    w = W.get("tiny")
    banner("embbag tiny workload")
    idx, off = W.indices_offsets(w)
    tabs_dev = SD.make_tables(w)
    got = _run(tabs_dev, idx, off, w.B, w.d).reshape(w.B, w.K, w.d)
    for k in range(w.K):
        host = R.table_rows(w.seed, k, w.rows[k], np.arange(w.rows[k]), w.d)
        assert np.array_equal(tabs_dev[k].cpu().numpy().view(np.uint32), host.view(np.uint32))  # device fill == host hash
        assert np.array_equal(bits(got[:, k]), bits(host[idx[k * w.B:(k + 1) * w.B]]))


def test_embbag_zipf_multihot_scaled():
    w = W.get("embbag").scaled(B=2048, rows=20000, K=5)
    banner("embbag zipf multi-hot scaled")
    idx, off = W.indices_offsets(w)
    tabs_dev = SD.make_tables(w)
    got = _run(tabs_dev, idx, off, w.B, w.d)
    tabs, local, _ = W.compact_rows(w, idx, off)
    ref = oracle.embbag_fwd(tabs, local, off, w.B)
    assert np.array_equal(bits(got), bits(ref))


@pytest.mark.parametrize("name", ["embbag", "interaction"])
def test_embbag_full_size_sampled(name):
    """Full-size workload in the benchmark's launch configuration; sampled bags
    against the oracle on regenerated rows."""
    import deep_learning_recommendation_amd as D

    w = W.get(name)
    banner(f"embbag full size {name}: K={w.K} rows={w.rows[0]} B={w.B}")
    idx, off = W.indices_offsets(w)
    tabs_dev = SD.make_tables(w)
    out = torch.empty((w.B, w.K * w.d), dtype=torch.float32, device=DEV)
    D.dlrm_embbag_fwd(D.device_pointer_array(tabs_dev), w.K, w.d, to_dev(idx), to_dev(off), w.B, out, w.K * w.d, 0,
                      nnz=len(idx))
    torch.cuda.synchronize()
    samples = np.sort(np.random.default_rng(1).choice(w.B, 512, replace=False))
    samples[-1] = w.B - 1  # include the ragged end
    got = out[torch.from_numpy(samples).to(DEV)].cpu().numpy()
    sidx, soff = W.sub_bags(idx, off, w.K, w.B, samples)
    ws = w.scaled(B=len(samples))
    tabs, local, _ = W.compact_rows(ws, sidx, soff)
    ref = oracle.embbag_fwd(tabs, local, soff, len(samples))
    del tabs_dev
    torch.cuda.empty_cache()
    assert np.array_equal(bits(got), bits(ref))


def test_check_indices_counts_bad_entries():
    import deep_learning_recommendation_amd as D

    banner("check_indices")
    K, B = 3, 100
    rows = np.array([10, 20, 30], dtype=np.int64)
    g = np.random.default_rng(3)
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(g.integers(0, 4, K * B), out=off[1:])
    idx = np.concatenate([g.integers(0, rows[k], off[(k + 1) * B] - off[k * B]) for k in range(K)])
    idx[3] = -1
    idx[-1] = 30
    idx[len(idx) // 2] = 10**9
    bad = torch.zeros(1, dtype=torch.int64, device=DEV)
    D.dlrm_check_indices(to_dev(idx), to_dev(off), K, B, to_dev(rows), bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 3


# ----------------------------------------------------------------- low-precision table rows

def _run_lp(tabs_dev, sbs_dev, dtype, idx, off, B, d, nnz=None):
    import deep_learning_recommendation_amd as D

    K = len(tabs_dev)
    out = torch.full((B, K * d), float("nan"), dtype=torch.float32, device=DEV)
    code = D.DLRM_BF16 if dtype == "bf16" else D.DLRM_I8
    sbp = D.device_pointer_array(sbs_dev) if sbs_dev is not None else None
    D.dlrm_embbag_fwd_lp(D.device_pointer_array(tabs_dev), code, sbp, K, d, to_dev(idx), to_dev(off), B, out, K * d, 0,
                         nnz=int(off[-1]) if nnz is None else nnz)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _lp_tables(g, dtype, rows, d):
    """bf16: high halves of random fp32 values (uint16); int8: random bytes
    with per-row scale and bias."""
    if dtype == "bf16":
        tabs = [(g.standard_normal((m, d)).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
                for m in rows]
        return tabs, None
    tabs = [g.integers(-128, 128, size=(m, d)).astype(np.int8) for m in rows]
    sbs = [np.stack([g.uniform(1e-3, 2e-2, m), g.normal(0, 1e-2, m)], axis=1).astype(np.float32) for m in rows]
    return tabs, sbs


def _dev_lp(tabs, sbs):
    td = [to_dev(t.view(np.int16) if t.dtype == np.uint16 else t) for t in tabs]
    return td, (None if sbs is None else [to_dev(s) for s in sbs])


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
@pytest.mark.parametrize("d", [4, 16, 64, 128, 132, 256, 260, 1024])
def test_embbag_lp_random_ragged_bitexact(dtype, d):
    K, B = 3, 701
    banner(f"embbag lp {dtype} d={d} K={K} B={B}")
    g = np.random.default_rng(d + (7 if dtype == "int8" else 0))
    rows = [50, 333, 7]
    tabs, sbs = _lp_tables(g, dtype, rows, d)
    _, idx, off = _rand_case(d + 3, K, B, d, rows, 45)
    td, sd = _dev_lp(tabs, sbs)
    got = _run_lp(td, sd, dtype, idx, off, B, d)
    ref = oracle.embbag_fwd_lp(tabs, dtype, idx, off, B, scale_bias=sbs)
    assert np.array_equal(bits(got), bits(ref))
    got2 = _run_lp(td, sd, dtype, idx, off, B, d, nnz=-1)  # other work split, same bits
    assert np.array_equal(bits(got2), bits(ref))


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
def test_embbag_lp_device_fill_matches_host_generator(dtype):
    w = W.get("tiny")
    banner(f"embbag lp device fill {dtype}")
    tabs_dev, sbs_dev = SD.make_tables_lp(w, dtype)
    torch.cuda.synchronize()
    for k in range(w.K):
        ids = np.arange(w.rows[k])
        if dtype == "bf16":
            host = R.table_rows_bf16(w.seed, k, w.rows[k], ids, w.d)
            assert np.array_equal(tabs_dev[k].cpu().numpy().view(np.uint16), host)
        else:
            q, sb = R.table_rows_i8(w.seed, k, w.rows[k], ids, w.d)
            assert np.array_equal(tabs_dev[k].cpu().numpy(), q)
            assert np.array_equal(sbs_dev[k].cpu().numpy().view(np.uint32), sb.view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
def test_embbag_lp_full_size_sampled(dtype):
    """The gather microbenchmark's full-size workload with bf16 / int8 rows, in
    the benchmark's launch configuration; sampled bags against the oracle on
    regenerated rows."""
    w = W.get("embbag")
    banner(f"embbag lp full size {dtype}: K={w.K} rows={w.rows[0]} B={w.B}")
    idx, off = W.indices_offsets(w)
    tabs_dev, sbs_dev = SD.make_tables_lp(w, dtype)
    out = torch.empty((w.B, w.K * w.d), dtype=torch.float32, device=DEV)
    import deep_learning_recommendation_amd as D

    code = D.DLRM_BF16 if dtype == "bf16" else D.DLRM_I8
    sbp = D.device_pointer_array(sbs_dev) if sbs_dev is not None else None
    D.dlrm_embbag_fwd_lp(D.device_pointer_array(tabs_dev), code, sbp, w.K, w.d, to_dev(idx), to_dev(off), w.B, out,
                         w.K * w.d, 0, nnz=len(idx))
    torch.cuda.synchronize()
    samples = np.sort(np.random.default_rng(2).choice(w.B, 512, replace=False))
    samples[-1] = w.B - 1
    got = out[torch.from_numpy(samples).to(DEV)].cpu().numpy()
    sidx, soff = W.sub_bags(idx, off, w.K, w.B, samples)
    S = len(samples)
    tabs, sbs, local = [], [], np.empty_like(sidx)
    for k in range(w.K):
        a, b = int(soff[k * S]), int(soff[(k + 1) * S])
        u, inv = np.unique(sidx[a:b], return_inverse=True)
        local[a:b] = inv
        if dtype == "bf16":
            tabs.append(R.table_rows_bf16(w.seed, k, w.rows[k], u, w.d))
        else:
            q, sb = R.table_rows_i8(w.seed, k, w.rows[k], u, w.d)
            tabs.append(q)
            sbs.append(sb)
    ref = oracle.embbag_fwd_lp(tabs, dtype, local, soff, S, scale_bias=sbs if dtype == "int8" else None)
    del tabs_dev, sbs_dev
    torch.cuda.empty_cache()
    assert np.array_equal(bits(got), bits(ref))
