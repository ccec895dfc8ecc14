"""Interaction (Gram, strict lower triangle, concat) on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from dlrm_cases import DEV, banner, bits, interaction_tolerance, to_dev

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


@pytest.mark.parametrize("n,d", [(9, 16), (27, 128), (101, 64), (101, 128), (128, 64)])
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


def test_interact_bf16_output():
    B, n, d = 64, 27, 128
    banner("interact bf16 out")
    X = np.random.default_rng(5).standard_normal((B, n, d)).astype(np.float32)
    got, width = _run(X, torch.bfloat16)
    ref = oracle.interact_fwd(X)
    ref_b = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    # each value is the bf16 rounding of an fp32 result within the fp32 bound:
    # at most one bf16 ulp from the oracle's rounding
    ulp = np.abs(ref_b) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(got[:, :width] - ref_b) <= ulp)
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
