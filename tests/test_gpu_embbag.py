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
