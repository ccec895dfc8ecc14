"""Interaction (Gram, strict lower triangle, concat) on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from dlrm_cases import DEV, banner, bf16_row_tolerance, bits, interaction_tolerance, to_dev

pytestmark = pytest.mark.gpu


def _run(X, out_dtype=torch.float32, out_ld=None):
    import deep_learning_recommendation_amd as D

    B, n, d = X.shape
    width = d + n * (n - 1) // 2
    out_ld = ((width + 7) // 8) * 8 if out_ld is None else out_ld
    out = torch.full((B, out_ld), 7.0, dtype=out_dtype, device=DEV)
    D.dlrm_interact_fwd(to_dev(X), B, n, d, n * d, out, out_ld)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), width


# (n, d): MFMA register path for every tile count and chunk width, plus the
# generic path (n*d beyond the register budget)
SHAPES = [(2, 4), (9, 16), (9, 128), (17, 32), (27, 128), (33, 64), (64, 128), (101, 64), (128, 64), (128, 16),
          (27, 256), (33, 256), (101, 128), (5, 12), (27, 100)]


@pytest.mark.parametrize("n,d", SHAPES)
def test_interact_fp32_within_dot_product_bound(n, d):
    B = 37  # not a multiple of the 4 samples per block
    banner(f"interact fp32 n={n} d={d}")
    X = np.random.default_rng(n * 7 + d).standard_normal((B, n, d)).astype(np.float32)
    got, width = _run(X)
    ref = oracle.interact_fwd(X)
    assert np.array_equal(bits(got[:, :d]), bits(ref[:, :d]))  # dense row copied exactly
    tol = interaction_tolerance(X)
    assert np.all(np.abs(got[:, d:width].astype(np.float64) - ref[:, d:]) <= tol)
    pad_end = min(((width + 7) // 8) * 8, got.shape[1])
    assert np.all(got[:, width:pad_end] == 0)


@pytest.mark.parametrize("n,d", [(9, 16), (16, 64), (17, 16), (27, 128), (32, 32), (33, 128), (101, 64), (101, 128),
                                 (128, 64)])
def test_interact_integer_X_bitexact(n, d):
    # small integers: every product and partial sum is exact in fp32, so any
    # accumulation order (MFMA included) gives the oracle's value exactly;
    # this pins the tile and triangle index mapping
    B = 9
    banner(f"interact integer n={n} d={d}")
    X = np.random.default_rng(n + d).integers(-6, 7, size=(B, n, d)).astype(np.float32)
    got, width = _run(X)
    ref = oracle.interact_fwd(X)
    assert np.array_equal(bits(got[:, :width]), bits(ref))
    # bf16 rows: the exact values rounded once to nearest even, at the same
    # packed positions (the bf16 store path of the same kernel)
    got_b, _ = _run(X, torch.bfloat16)
    ref_b = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    assert np.array_equal(bits(got_b[:, :width]), bits(ref_b))
    # the row's padding up to the next multiple of 8 elements is zero
    assert np.all(got[:, width:] == 0) and np.all(got_b[:, width:] == 0)


def test_interact_bf16_output():
    B, n, d = 64, 27, 128
    banner("interact bf16 out")
    X = np.random.default_rng(5).standard_normal((B, n, d)).astype(np.float32)
    got, width = _run(X, torch.bfloat16)
    ref = oracle.interact_fwd(X)
    ref_b = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    # each value is the bf16 rounding of an fp32 result within the fp32 bound
    assert np.all(np.abs(got[:, :width] - ref) <= bf16_row_tolerance(X, ref))
    assert (got[:, :width] == ref_b).mean() > 0.99


def test_interact_workload_shapes_full_batch():
    # the three interaction shapes of the workloads at their full batch
    for (B, n, d) in [(32768, 27, 128), (16384, 101, 64), (8192, 9, 128)]:
        banner(f"interact full batch B={B} n={n} d={d}")
        X = (np.random.default_rng(B).standard_normal((B, n, d)) * 0.1).astype(np.float32)
        got, width = _run(X)
        rows = np.random.default_rng(0).choice(B, 64, replace=False)
        rows[-1] = B - 1
        ref = oracle.interact_fwd(X[rows])
        tol = interaction_tolerance(X[rows])
        assert np.all(np.abs(got[rows, d:width].astype(np.float64) - ref[:, d:]) <= tol)
        assert np.array_equal(bits(got[rows, :d]), bits(ref[:, :d]))


@pytest.mark.parametrize("K,d,out_bf16", [(8, 16, False), (26, 128, True), (26, 128, False), (100, 64, True),
                                          (8, 128, True), (3, 12, False), (31, 64, True)])
def test_fused_gather_interaction(K, d, out_bf16):
    """dlrm_embbag_interact_fwd against dlrm_embbag_fwd + dlrm_interact_fwd on
    the GPU (bit for bit) and against the oracle (pooled rows exact, pairs
    within the dot-product bound), on ragged multi-hot bags with empty ones."""
    import deep_learning_recommendation_amd as D

    B = 203
    n = K + 1
    banner(f"fused gather+interaction K={K} d={d} bf16={out_bf16}")
    g = np.random.default_rng(K * 100 + d)
    rows = [int(x) for x in g.integers(5, 300, size=K)]
    lens = g.integers(0, 6, size=K * B)
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    idx = np.concatenate([g.integers(0, rows[k], off[(k + 1) * B] - off[k * B]) for k in range(K)]).astype(np.int64)
    tabs = [(g.standard_normal((rows[k], d)) * 0.3).astype(np.float32) for k in range(K)]
    x0 = g.standard_normal((B, d)).astype(np.float32)
    tdev = [to_dev(t) for t in tabs]
    ptrs = D.device_pointer_array(tdev)
    width = d + n * (n - 1) // 2
    ld = ((width + 7) // 8) * 8
    dt = torch.bfloat16 if out_bf16 else torch.float32
    # two-call path
    X = torch.zeros((B, n, d), dtype=torch.float32, device=DEV)
    X[:, 0, :] = to_dev(x0)
    D.dlrm_embbag_fwd(ptrs, K, d, to_dev(idx), to_dev(off), B, X, n * d, d, nnz=len(idx))
    two = torch.full((B, ld), 3.0, dtype=dt, device=DEV)
    D.dlrm_interact_fwd(X, B, n, d, n * d, two, ld)
    one = torch.full((B, ld), 5.0, dtype=dt, device=DEV)
    D.dlrm_embbag_interact_fwd(to_dev(x0), d, ptrs, K, d, to_dev(idx), to_dev(off), B, one, ld)
    torch.cuda.synchronize()
    vt = torch.int16 if out_bf16 else torch.int32
    assert torch.equal(one.view(vt), two.view(vt))
    # oracle
    E = oracle.embbag_fwd(tabs, idx, off, B).reshape(B, K, d)
    Xr = np.concatenate([x0[:, None, :], E], axis=1)
    ref = oracle.interact_fwd(Xr)
    got = one.float().cpu().numpy()
    if out_bf16:
        assert np.all(np.abs(got[:, :width] - ref) <= bf16_row_tolerance(Xr, ref))
    else:
        assert np.array_equal(bits(got[:, :d]), bits(ref[:, :d]))
        assert np.all(np.abs(got[:, d:width].astype(np.float64) - ref[:, d:]) <= interaction_tolerance(Xr))
    assert np.all(got[:, width:] == 0)


# ------------------------------------------------------------------ backward

def _run_bwd(X, g):
    import deep_learning_recommendation_amd as D

    B, n, d = X.shape
    dX = torch.full((B, n * d), 7.0, dtype=torch.float32, device=DEV)
    D.dlrm_interact_bwd(to_dev(X), B, n, d, n * d, to_dev(g), g.shape[1], dX, n * d)
    torch.cuda.synchronize()
    return dX.cpu().numpy().reshape(B, n, d)


def _bwd_bound(X, g):
    # fp32 accumulation of n products per output: n u (sum |g_pair X| + |g_dense|)
    n = X.shape[1]
    mag = oracle.interact_bwd(np.abs(X), np.abs(g)).astype(np.float64)
    return (n + 2) * 2.0 ** -24 * mag + 1e-30


BWD_SHAPES = [(2, 4), (9, 16), (9, 128), (17, 32), (27, 128), (33, 64), (101, 64), (128, 64), (5, 12), (27, 100),
              (101, 128), (128, 128), (64, 256)]


@pytest.mark.parametrize("n,d", BWD_SHAPES)
def test_interact_bwd_within_bound(n, d):
    B = 37
    banner(f"interact bwd n={n} d={d}")
    rng = np.random.default_rng(1000 + n * 7 + d)
    X = rng.standard_normal((B, n, d)).astype(np.float32)
    g = rng.standard_normal((B, d + n * (n - 1) // 2)).astype(np.float32)
    got = _run_bwd(X, g)
    ref = oracle.interact_bwd(X, g)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= _bwd_bound(X, g))
    # and the "1e-5 relative" reading against the sum of magnitudes
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 1e-5 * oracle.interact_bwd(np.abs(X), np.abs(g)) + 1e-30)


@pytest.mark.parametrize("n,d", [(9, 16), (27, 128), (101, 64)])
def test_interact_bwd_integer_exact(n, d):
    # small integers: every product and partial sum is exact in fp32, so any
    # accumulation order gives the oracle's value; pins the S and X index maps
    B = 9
    banner(f"interact bwd integer n={n} d={d}")
    rng = np.random.default_rng(n + d)
    X = rng.integers(-4, 5, size=(B, n, d)).astype(np.float32)
    g = rng.integers(-3, 4, size=(B, d + n * (n - 1) // 2)).astype(np.float32)
    assert np.array_equal(bits(_run_bwd(X, g)), bits(oracle.interact_bwd(X, g)))


def test_interact_bwd_workload_shapes_full_batch():
    for (B, n, d) in [(8192, 9, 128), (32768, 27, 128), (16384, 101, 64)]:
        banner(f"interact bwd full batch B={B} n={n} d={d}")
        rng = np.random.default_rng(B + n)
        X = (rng.standard_normal((B, n, d)) * 0.1).astype(np.float32)
        g = (rng.standard_normal((B, d + n * (n - 1) // 2)) * 1e-3).astype(np.float32)
        got = _run_bwd(X, g)
        rows = np.random.default_rng(1).choice(B, 64, replace=False)
        rows[-1] = B - 1
        ref = oracle.interact_bwd(X[rows], g[rows])
        bound = 1e-5 * oracle.interact_bwd(np.abs(X[rows]), np.abs(g[rows])) + 1e-30
        assert np.all(np.abs(got[rows].astype(np.float64) - ref) <= bound)


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
@pytest.mark.parametrize("K,d,bags", [(8, 32, "ragged"), (26, 128, "mostly_one"), (26, 128, "ragged"),
                                      (100, 64, "ragged"), (3, 96, "mostly_one"), (31, 64, "mostly_one"),
                                      (15, 160, "ragged")])
def test_fused_gather_interaction_lp(dtype, K, d, bags):
    """dlrm_embbag_interact_fwd_lp against the oracle (dense part exact, pairs
    within the bf16 row bound), and against dlrm_embbag_fwd_lp +
    dlrm_interact_fwd: dense part bit for bit, pairs within the same bound
    (the fused kernel feeds the MFMAs eight consecutive columns per lane, so
    the pair sums run in another order); d = 160 leaves lane groups past the
    row end in the last 32-column pair."""
    import deep_learning_recommendation_amd as D

    B, n = 203, K + 1
    banner(f"fused gather+interaction lp {dtype} K={K} d={d} bags={bags}")
    g = np.random.default_rng(K * 10 + d + (1 if dtype == "int8" else 0))
    rows = [int(x) for x in g.integers(5, 300, size=K)]
    if bags == "ragged":
        lens = g.integers(0, 6, size=K * B)
    else:
        lens = np.ones(K * B, dtype=np.int64)
        odd = g.random(K * B) < 0.02
        lens[odd] = g.choice([0, 2], size=int(odd.sum()))
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    idx = np.concatenate([g.integers(0, rows[k], off[(k + 1) * B] - off[k * B]) for k in range(K)]).astype(np.int64)
    if dtype == "bf16":
        tabs = [((g.standard_normal((m, d)) * 0.3).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
                for m in rows]
        sbs = None
        tdev = [to_dev(t.view(np.int16)) for t in tabs]
        sdev = None
    else:
        tabs = [g.integers(-128, 128, size=(m, d)).astype(np.int8) for m in rows]
        sbs = [np.stack([g.uniform(1e-3, 5e-3, m), g.normal(0, 1e-2, m)], axis=1).astype(np.float32) for m in rows]
        tdev = [to_dev(t) for t in tabs]
        sdev = [to_dev(sb) for sb in sbs]
    code = D.DLRM_BF16 if dtype == "bf16" else D.DLRM_I8
    ptrs = D.device_pointer_array(tdev)
    sbp = D.device_pointer_array(sdev) if sdev is not None else None
    x0 = g.standard_normal((B, d)).astype(np.float32)
    width = d + n * (n - 1) // 2
    ld = ((width + 7) // 8) * 8
    X = torch.zeros((B, n, d), dtype=torch.float32, device=DEV)
    X[:, 0, :] = to_dev(x0)
    D.dlrm_embbag_fwd_lp(ptrs, code, sbp, K, d, to_dev(idx), to_dev(off), B, X, n * d, d, nnz=len(idx))
    two = torch.full((B, ld), 3.0, dtype=torch.bfloat16, device=DEV)
    D.dlrm_interact_fwd(X, B, n, d, n * d, two, ld)
    one = torch.full((B, ld), 5.0, dtype=torch.bfloat16, device=DEV)
    D.dlrm_embbag_interact_fwd_lp(to_dev(x0), d, ptrs, code, sbp, K, d, to_dev(idx), to_dev(off), B, one, ld)
    torch.cuda.synchronize()
    E = oracle.embbag_fwd_lp(tabs, dtype, idx, off, B, scale_bias=sbs).reshape(B, K, d)
    Xr = np.concatenate([x0[:, None, :], E], axis=1)
    ref = oracle.interact_fwd(Xr)
    tol = bf16_row_tolerance(Xr, ref)
    got = one.float().cpu().numpy()
    got2 = two.float().cpu().numpy()
    assert torch.equal(one[:, :d].view(torch.int16), two[:, :d].view(torch.int16))
    assert np.all(np.abs(got[:, :width] - ref) <= tol)
    assert np.all(np.abs(got2[:, :width] - ref) <= tol)
    assert np.all(got[:, width:] == 0)


def test_fused_lp_needs_32_column_multiple():
    import deep_learning_recommendation_amd as D

    banner("fused lp unsupported width")
    K, d, B = 3, 16, 4
    tdev = [torch.zeros((5, d), dtype=torch.int16, device=DEV) for _ in range(K)]
    off = to_dev(np.arange(K * B + 1, dtype=np.int64))
    idx = to_dev(np.zeros(K * B, dtype=np.int64))
    x0 = torch.zeros((B, d), dtype=torch.float32, device=DEV)
    out = torch.zeros((B, 32), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(D.DLRMError):
        D.dlrm_embbag_interact_fwd_lp(x0, d, D.device_pointer_array(tdev), D.DLRM_BF16, None, K, d, idx, off, B, out, 32)
