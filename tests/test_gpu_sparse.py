"""Sparse backward with row-wise SGD on the GPU against the oracle: every
touched row bit-exact, untouched rows bitwise unchanged."""
import numpy as np
import pytest
import torch

import oracle
from dlrm_cases import DEV, banner, bits, to_dev
from synth import device as SD
from synth import rng as R
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _run_sgd(tabs_dev, rows, idx, off, B, d, G, g_col0, lr):
    import deep_learning_recommendation_amd as D

    K = len(tabs_dev)
    nnz = int(off[-1])
    G_dev = to_dev(G)
    ws = torch.empty((D.dlrm_embbag_bwd_sgd_workspace_size(K, B, nnz, d),), dtype=torch.uint8, device=DEV)
    D.dlrm_embbag_bwd_sgd(D.device_pointer_array(tabs_dev), K, d, rows, to_dev(idx), to_dev(off), B, nnz, G_dev,
                          G.shape[1], g_col0, lr, ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("d,K,hot", [(16, 3, False), (128, 4, True), (64, 2, True), (132, 2, False), (8, 5, True)])
def test_sparse_sgd_random_bitexact(d, K, hot):
    B = 611
    rows = [97, 1000, 5, 400, 33][:K]
    banner(f"sparse sgd random d={d} K={K} hot={hot}")
    g = np.random.default_rng(d * 10 + K)
    lens = g.integers(0, 30, size=K * B)
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    idx = []
    for k in range(K):
        n = off[(k + 1) * B] - off[k * B]
        if hot:  # a few rows with thousands of occurrences (hot-row path)
            r = np.where(g.random(n) < 0.6, g.integers(0, 2, n), g.integers(0, rows[k], n))
        else:
            r = g.integers(0, rows[k], n)
        idx.append(r)
    idx = np.concatenate(idx).astype(np.int64)
    tabs = [g.standard_normal((rows[k], d)).astype(np.float32) for k in range(K)]
    G = (g.standard_normal((B, (K + 1) * d)) * 0.01).astype(np.float32)
    tabs_dev = [to_dev(t) for t in tabs]
    _run_sgd(tabs_dev, rows, idx, off, B, d, G, d, 0.01)
    ref = [t.copy() for t in tabs]
    oracle.embbag_bwd_sgd(ref, idx, off, B, G, d, 0.01)
    for k in range(K):
        assert np.array_equal(bits(tabs_dev[k].cpu().numpy()), bits(ref[k]))
    if hot:
        counts = np.bincount(idx[off[0]:off[B]], minlength=rows[0])
        assert counts.max() >= 128  # the hot path was exercised


def _hot_case(g, B, L, rows, counts):
    """Indices of one table: row i occurs counts[i] times, the remaining
    positions fall uniformly on the other rows; positions are shuffled."""
    n = B * L
    fixed = np.repeat(np.arange(len(counts)), counts)
    rest = g.integers(len(counts), rows, n - len(fixed))
    r = np.concatenate([fixed, rest])
    g.shuffle(r)
    return r


@pytest.mark.parametrize("d", [4, 64, 100, 132, 256, 1024])
def test_sparse_sgd_hot_segment_lengths(d):
    """Segments at and around the hot-path threshold and its 64-occurrence
    blocks (127, 128, 129, 191, 192, 193), one long segment of 20000
    occurrences, and column slices of 64 with a ragged last slice."""
    B, L, K = 4096, 8, 2
    rows = [5000, 3000]
    banner(f"sparse sgd hot segment lengths d={d}")
    g = np.random.default_rng(100 + d)
    counts = [[20000, 127, 128, 129, 191, 192, 193, 64, 65, 1], [1000, 256, 257, 300, 128, 5]]
    idx = np.concatenate([_hot_case(g, B, L, rows[k], counts[k]) for k in range(K)]).astype(np.int64)
    off = np.arange(K * B + 1, dtype=np.int64) * L
    tabs = [g.standard_normal((rows[k], d)).astype(np.float32) for k in range(K)]
    G = (g.standard_normal((B, (K + 1) * d)) * 0.01).astype(np.float32)
    tabs_dev = [to_dev(t) for t in tabs]
    _run_sgd(tabs_dev, rows, idx, off, B, d, G, d, 0.01)
    ref = [t.copy() for t in tabs]
    oracle.embbag_bwd_sgd(ref, idx, off, B, G, d, 0.01)
    for k in range(K):
        assert np.array_equal(bits(tabs_dev[k].cpu().numpy()), bits(ref[k])), k


def test_sparse_sgd_many_hot_segments():
    """About a thousand segments of ~200 occurrences each: far more hot
    items than blocks, so every block runs many items through its ring."""
    B, L, K, d = 2048, 100, 1, 128
    rows = [1000]
    banner("sparse sgd many hot segments")
    g = np.random.default_rng(7)
    idx = g.integers(0, rows[0], B * L).astype(np.int64)
    off = np.arange(K * B + 1, dtype=np.int64) * L
    tabs = [g.standard_normal((rows[0], d)).astype(np.float32)]
    G = (g.standard_normal((B, d)) * 0.01).astype(np.float32)
    tabs_dev = [to_dev(t) for t in tabs]
    _run_sgd(tabs_dev, rows, idx, off, B, d, G, 0, 0.01)
    ref = [t.copy() for t in tabs]
    oracle.embbag_bwd_sgd(ref, idx, off, B, G, 0, 0.01)
    assert np.array_equal(bits(tabs_dev[0].cpu().numpy()), bits(ref[0]))


def test_sparse_sgd_empty_batch_is_noop():
    banner("sparse sgd empty")
    d, K, B = 16, 2, 10
    tabs = [np.random.default_rng(0).standard_normal((10, d)).astype(np.float32) for _ in range(K)]
    tabs_dev = [to_dev(t) for t in tabs]
    off = np.zeros(K * B + 1, dtype=np.int64)
    G = np.ones((B, K * d), np.float32)
    _run_sgd(tabs_dev, [10, 10], np.zeros(1, np.int64), off, B, d, G, 0, 0.01)
    for k in range(K):
        assert np.array_equal(bits(tabs_dev[k].cpu().numpy()), bits(tabs[k]))


def test_sparse_sgd_train_scaled():
    w = W.get("train").scaled(B=1024, rows=200_000)
    banner("sparse sgd train scaled")
    idx, off = W.indices_offsets(w)
    tabs_dev = SD.make_tables(w)
    G = W.upstream_grad(w).reshape(w.B, -1)
    _run_sgd(tabs_dev, w.rows, idx, off, w.B, w.d, G, w.d, w.lr)
    tabs, local, row_ids = W.compact_rows(w, idx, off)
    oracle.embbag_bwd_sgd(tabs, local, off, w.B, G, w.d, w.lr)
    for k in range(w.K):
        got = tabs_dev[k][torch.from_numpy(row_ids[k]).to(DEV)].cpu().numpy()
        assert np.array_equal(bits(got), bits(tabs[k]))


@pytest.mark.parametrize("two_streams", [False, True])
def test_sparse_sgd_train_full_size(two_streams):
    """The training workload at full size (8 x 5e7 x 128 tables, 6.5M
    lookups with Zipf(1.2) hot rows): every touched row bit-exact, 1e5
    random untouched rows unchanged.  two_streams: prepare, then apply with
    the short segments on a second stream."""
    import deep_learning_recommendation_amd as D

    w = W.get("train")
    banner(f"sparse sgd train full size: {w.K} x {w.rows[0]} x {w.d} two_streams={two_streams}")
    idx, off = W.indices_offsets(w)
    tabs_dev = SD.make_tables(w)
    G = W.upstream_grad(w).reshape(w.B, -1)
    if two_streams:
        nnz = int(off[-1])
        ws = torch.empty((D.dlrm_embbag_bwd_sgd_workspace_size(w.K, w.B, nnz, w.d),), dtype=torch.uint8, device=DEV)
        ptrs = D.device_pointer_array(tabs_dev)
        idx_d, off_d, G_d = to_dev(idx), to_dev(off), to_dev(G)
        D.dlrm_embbag_bwd_sgd_prepare(w.K, w.rows, idx_d, off_d, w.B, nnz, ws)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        D.dlrm_embbag_bwd_sgd_apply(ptrs, w.K, w.d, w.rows, w.B, nnz, G_d, G.shape[1], w.d, w.lr, ws, side=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
    else:
        _run_sgd(tabs_dev, w.rows, idx, off, w.B, w.d, G, w.d, w.lr)
    tabs, local, row_ids = W.compact_rows(w, idx, off)
    oracle.embbag_bwd_sgd(tabs, local, off, w.B, G, w.d, w.lr)
    g = np.random.default_rng(5)
    for k in range(w.K):
        got = tabs_dev[k][torch.from_numpy(row_ids[k]).to(DEV)].cpu().numpy()
        assert np.array_equal(bits(got), bits(tabs[k])), k
        probe = np.setdiff1d(g.integers(0, w.rows[k], 100_000 // w.K), row_ids[k])
        now = tabs_dev[k][torch.from_numpy(probe).to(DEV)].cpu().numpy()
        assert np.array_equal(bits(now), bits(R.table_rows(w.seed, k, w.rows[k], probe, w.d)))
    del tabs_dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("two_streams", [False, True])
@pytest.mark.parametrize("d,K", [(128, 4), (64, 2), (132, 3)])
def test_sparse_prepare_apply_two_calls(d, K, two_streams):
    """dlrm_embbag_bwd_sgd_prepare on a second stream (beside unrelated work
    on the first), then dlrm_embbag_bwd_sgd_apply twice from the same
    prepared workspace: two SGD steps, each bit-exact against the oracle.
    two_streams: the apply's short segments run on a second stream of the
    caller (forked from and joined back into the first)."""
    import deep_learning_recommendation_amd as D

    B = 733
    rows = [97, 1000, 5, 400][:K]
    banner(f"sparse sgd prepare/apply d={d} K={K}")
    g = np.random.default_rng(900 + d + K)
    lens = g.integers(0, 40, size=K * B)
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    idx = []
    for k in range(K):
        n = off[(k + 1) * B] - off[k * B]
        idx.append(np.where(g.random(n) < 0.5, g.integers(0, 2, n), g.integers(0, rows[k], n)))
    idx = np.concatenate(idx).astype(np.int64)
    nnz = int(off[-1])
    tabs = [g.standard_normal((rows[k], d)).astype(np.float32) for k in range(K)]
    G = (g.standard_normal((B, (K + 1) * d)) * 0.01).astype(np.float32)
    tabs_dev = [to_dev(t) for t in tabs]
    ptrs = D.device_pointer_array(tabs_dev)
    idx_d, off_d, G_d = to_dev(idx), to_dev(off), to_dev(G)
    ws = torch.empty((D.dlrm_embbag_bwd_sgd_workspace_size(K, B, nnz, d),), dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)  # whatever the workspace held before, prepare defines it
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    busy = torch.empty((1 << 26,), dtype=torch.float32, device=DEV)
    with torch.cuda.stream(side):
        D.dlrm_embbag_bwd_sgd_prepare(K, rows, idx_d, off_d, B, nnz, ws)
    busy.fill_(1.0)  # unrelated work on the first stream meanwhile
    torch.cuda.current_stream().wait_stream(side)
    ref = [t.copy() for t in tabs]
    cur = torch.cuda.current_stream()
    for step in range(2):
        if two_streams:
            side.wait_stream(cur)
            D.dlrm_embbag_bwd_sgd_apply(ptrs, K, d, rows, B, nnz, G_d, G.shape[1], d, 0.01, ws, side=side)
            cur.wait_stream(side)
        else:
            D.dlrm_embbag_bwd_sgd_apply(ptrs, K, d, rows, B, nnz, G_d, G.shape[1], d, 0.01, ws)
        torch.cuda.synchronize()
        oracle.embbag_bwd_sgd(ref, idx, off, B, G, d, 0.01)
        for k in range(K):
            assert np.array_equal(bits(tabs_dev[k].cpu().numpy()), bits(ref[k])), (step, k)
    counts = np.bincount(idx[off[0]:off[B]], minlength=rows[0])
    assert counts.max() >= 128  # the hot-row path was exercised
