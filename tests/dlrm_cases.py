"""Shared helpers for the GPU parity tests: seeded inputs, device state and
the oracle-side references (no GPU result ever feeds the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import device as SD
from synth import rng as R
from synth import workloads as W

DEV = "cuda"


def banner(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def oracle_forward(w, dense, idx, off, bottom, top, samples=None, tables=None):
    """Forward pass of the listed samples with the oracle.

    ``bottom``/``top`` are lists of (W fp32 values, bits, b).  Tables are
    regenerated on the host for the rows the sampled bags touch (or taken
    from ``tables`` when given as full host arrays)."""
    B = w.B
    if samples is None:
        samples = np.arange(B)
    sidx, soff = W.sub_bags(idx, off, w.K, B, samples)
    S = len(samples)
    ws = w.scaled(B=S)
    if tables is None:
        tabs, local, _ = W.compact_rows(ws, sidx, soff)
    else:
        tabs, local = tables, sidx
    quant = w.mlp_dtype == "bf16"
    x0, _, _ = oracle.mlp_fwd(dense[samples], [p[0] for p in bottom], [p[2] for p in bottom], quant, True)
    E = oracle.embbag_fwd(tabs, local, soff, S)
    X = np.concatenate([x0, E], axis=1).reshape(S, w.n, w.d)
    top_in = oracle.interact_fwd(X)
    logit, prob, _ = oracle.mlp_fwd(top_in, [p[0] for p in top], [p[2] for p in top], quant, False)
    return X, top_in, logit[:, 0], prob


def device_model(w, train=False, tables=None, batch=0, fused=True):
    """Pipeline state on the GPU for workload ``w`` (tables filled on device)."""
    from deep_learning_recommendation_amd import pipeline as PL

    if tables is None:
        tables = SD.make_tables(w)
    bf16 = w.mlp_dtype == "bf16"
    bottom = W.mlp_params(w, "bottom")
    top = W.mlp_params(w, "top")
    bp = PL.make_mlp(w.bottom, [p[0] for p in bottom], [p[2] for p in bottom], bf16)
    tp = PL.make_mlp(w.top, [p[0] for p in top], [p[2] for p in top], bf16)
    model = PL.DLRM(w.B, w.K, w.d, w.rows, tables, bp, tp, train=train, fused=fused)
    return model, bottom, top


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def interaction_tolerance(X):
    """1e-5 * sum_c |x_ic x_jc| per packed pair, plus a tiny absolute floor."""
    Xa = np.abs(X.astype(np.float64))
    B, n, d = X.shape
    ii, jj = np.tril_indices(n, -1)
    mag = np.einsum("bic,bjc->bij", Xa, Xa)[:, ii, jj]
    return 1e-5 * mag + 1e-30


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def bf16_row_tolerance(X, ref_row):
    """Bound for a bf16 top-MLP input row against the oracle's fp32 row:
    the device's fp32 value lies within tol = 1e-5 sum|x_i x_j| (pairs) or is
    exact (dense part), then one bf16 rounding adds at most 2**-8 of it."""
    d = X.shape[2]
    tol = np.zeros_like(ref_row, dtype=np.float64)
    tol[:, d:d + interaction_tolerance(X).shape[1]] = interaction_tolerance(X)
    return tol + 2.0 ** -8 * (np.abs(ref_row.astype(np.float64)) + tol) + 1e-30
