"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each pin checks the oracle against something other than itself: a
hand-worked example, closed forms, exact (dyadic) arithmetic, invariants,
brute-force enumeration, or an independent library routine (torch on the
CPU in fp64).
"""
import json
import os

import numpy as np
import pytest
import torch

from synth import rng as R
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U32 = 2.0 ** -24  # unit roundoff of fp32


def _rand_bags(g, K, B, rows, max_len, empty_ok=True):
    lo = 0 if empty_ok else 1
    lens = g.integers(lo, max_len + 1, size=K * B)
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    idx = np.empty(off[-1], dtype=np.int64)
    for k in range(K):
        a, b = off[k * B], off[(k + 1) * B]
        idx[a:b] = g.integers(0, rows[k], size=b - a)
    return idx, off


# --------------------------------------------------------------------------- hand-worked example

def test_hand_example_forward_and_sgd(orc):
    ex = json.load(open(os.path.join(GOLDEN, "dlrm_hand_example.json")))
    d = ex["d"]
    tabs = [np.array(t, dtype=np.float32) for t in ex["tables"]]
    bags = ex["bags"]
    K, B = len(tabs), 1
    off = np.array([0, len(bags[0]), len(bags[0]) + len(bags[1])], dtype=np.int64)
    idx = np.array(bags[0] + bags[1], dtype=np.int64)
    xd, _, _ = orc.mlp_fwd(np.array([ex["dense"]], np.float32), [np.array(w, np.float32) for w in ex["bottom"]["W"]],
                           [np.array(b, np.float32) for b in ex["bottom"]["b"]], False, True)
    assert xd.tolist() == [ex["expect"]["x_dense"]]
    e = orc.embbag_fwd(tabs, idx, off, B)
    assert e.reshape(K, d).tolist() == ex["expect"]["e"]
    X = np.concatenate([xd, e], axis=1).reshape(1, K + 1, d)
    top_in = orc.interact_fwd(X)
    assert top_in[0, d:].tolist() == ex["expect"]["Z"]
    assert top_in[0].tolist() == ex["expect"]["top_in"]
    Ws = [np.array(w, np.float32) for w in ex["top"]["W"]]
    bs = [np.array(b, np.float32) for b in ex["top"]["b"]]
    logit, prob, acts = orc.mlp_fwd(top_in, Ws, bs, False, False, save_acts=True)
    assert acts[1][0].tolist() == ex["expect"]["hidden"]
    assert logit[0, 0] == ex["expect"]["logit"] and prob[0] == ex["expect"]["prob"]
    sg = ex["sgd"]
    G = np.array(sg["G"], dtype=np.float32).reshape(1, -1)
    orc.embbag_bwd_sgd(tabs, idx, off, B, G, d, sg["lr"])
    assert [t.tolist() for t in tabs] == sg["expect_tables"]


# --------------------------------------------------------------------------- embedding bag

def test_embbag_one_index_bag_is_row_lookup(orc):
    w = W.get("tiny")
    idx, off = W.indices_offsets(w)
    tabs = [R.table_rows(w.seed, k, w.rows[k], np.arange(w.rows[k]), w.d) for k in range(w.K)]
    out = orc.embbag_fwd(tabs, idx, off, w.B).reshape(w.B, w.K, w.d)
    for k in range(w.K):
        ref = tabs[k][idx[k * w.B:(k + 1) * w.B]]
        assert np.array_equal(out[:, k, :].view(np.uint32), ref.view(np.uint32))


def test_embbag_dyadic_exact_and_linear(orc):
    # Table values j/16 with |j| <= 64: every partial sum of <= 60 terms is a
    # multiple of 1/16 below 2**20 in magnitude, hence exact in fp32; the
    # pooled value must equal the integer sum / 16 bit for bit.
    g = np.random.default_rng(1)
    K, B, d, rows = 3, 40, 12, [7, 5, 9]
    ints = [g.integers(-64, 65, size=(m, d)) for m in rows]
    tabs = [(t / 16.0).astype(np.float32) for t in ints]
    idx, off = _rand_bags(g, K, B, rows, 60)
    out = orc.embbag_fwd(tabs, idx, off, B).reshape(B, K, d)
    for k in range(K):
        for b in range(B):
            s = ints[k][idx[off[k * B + b]:off[k * B + b + 1]]].sum(axis=0)
            assert np.array_equal(out[b, k], (s / 16.0).astype(np.float32))
    # linearity: pooling the two halves of every bag and adding equals pooling the bag
    lens = np.diff(off)
    cut = off[:-1] + lens // 2
    first = np.concatenate([idx[off[i]:cut[i]] for i in range(K * B)])
    second = np.concatenate([idx[cut[i]:off[i + 1]] for i in range(K * B)])
    off1 = np.concatenate([[0], np.cumsum(lens // 2)])
    off2 = np.concatenate([[0], np.cumsum(lens - lens // 2)])
    p1 = orc.embbag_fwd(tabs, first, off1, B)
    p2 = orc.embbag_fwd(tabs, second, off2, B)
    assert np.array_equal(out.reshape(B, -1), p1 + p2)


def test_embbag_brute_force_tiny(orc):
    # Enumerate every bag and add its rows one at a time in fp32, in bag order.
    g = np.random.default_rng(2)
    K, B, d, rows = 2, 4, 5, [6, 3]
    tabs = [g.standard_normal((m, d)).astype(np.float32) for m in rows]
    idx, off = _rand_bags(g, K, B, rows, 6)
    out = orc.embbag_fwd(tabs, idx, off, B, out_ld=K * d + 3, out_col0=3)
    for k in range(K):
        for b in range(B):
            acc = [np.float32(0.0)] * d
            for p in range(off[k * B + b], off[k * B + b + 1]):
                acc = [np.float32(acc[c] + tabs[k][idx[p], c]) for c in range(d)]
            got = out[b, 3 + k * d: 3 + (k + 1) * d]
            assert np.array_equal(got, np.array(acc, dtype=np.float32))
    assert np.all(out[:, :3] == 0)


def test_embbag_against_torch_fp64(orc):
    # torch.nn.functional.embedding_bag(mode="sum") in fp64; the fp32 oracle
    # must lie within the recursive-summation bound (L-1) u sum|T|.
    g = np.random.default_rng(3)
    K, B, d, rows = 3, 64, 32, [100, 50, 200]
    tabs = [g.standard_normal((m, d)).astype(np.float32) for m in rows]
    idx, off = _rand_bags(g, K, B, rows, 40)
    out = orc.embbag_fwd(tabs, idx, off, B).reshape(B, K, d).astype(np.float64)
    for k in range(K):
        a = off[k * B]
        ti = torch.from_numpy(idx[a:off[(k + 1) * B]])
        to = torch.from_numpy(off[k * B:(k + 1) * B] - a)
        wt = torch.from_numpy(tabs[k].astype(np.float64))
        ref = torch.nn.functional.embedding_bag(ti, wt, to, mode="sum").numpy()
        absw = torch.nn.functional.embedding_bag(ti, wt.abs(), to, mode="sum").numpy()
        L = np.diff(off[k * B:(k + 1) * B + 1])[:, None]
        bound = np.maximum(L - 1, 0) * U32 * absw * 1.0001
        assert np.all(np.abs(out[:, k] - ref) <= bound)


def test_embbag_empty_bag_is_positive_zero(orc):
    tabs = [np.full((4, 8), -3.0, np.float32)]
    off = np.array([0, 0, 2, 2], dtype=np.int64)
    idx = np.array([1, 2], dtype=np.int64)
    out = orc.embbag_fwd(tabs, idx, off, 3)
    assert np.all(out[0] == 0) and not np.any(np.signbit(out[0]))
    assert np.all(out[2] == 0) and not np.any(np.signbit(out[2]))
    assert np.all(out[1] == -6.0)


# --------------------------------------------------------------------------- low-precision table rows

def test_embbag_lp_bf16_is_exact_widening(orc):
    """bf16 rows widen exactly: tables whose fp32 values have zero low halves
    give, stored as their high halves, the fp32 lookup's result bit for bit."""
    g = np.random.default_rng(11)
    K, B, d, rows = 3, 40, 12, [9, 30, 5]
    f32 = [g.standard_normal((m, d)).astype(np.float32) for m in rows]
    f32 = [(t.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32) for t in f32]
    b16 = [(t.view(np.uint32) >> np.uint32(16)).astype(np.uint16) for t in f32]
    idx, off = _rand_bags(g, K, B, rows, 7)
    got = orc.embbag_fwd_lp(b16, "bf16", idx, off, B)
    ref = orc.embbag_fwd(f32, idx, off, B)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_embbag_lp_int8_unit_scale_is_integer_sum(orc):
    """Scale 1 and bias 0: every pooled value is the integer sum of the bag's
    bytes (exact in fp32 at these sizes), by brute force in int64."""
    g = np.random.default_rng(12)
    K, B, d, rows = 2, 33, 8, [17, 6]
    q = [g.integers(-128, 128, size=(m, d)).astype(np.int8) for m in rows]
    sb = [np.tile(np.array([1.0, 0.0], np.float32), (m, 1)) for m in rows]
    idx, off = _rand_bags(g, K, B, rows, 9)
    got = orc.embbag_fwd_lp(q, "int8", idx, off, B, scale_bias=sb)
    for k in range(K):
        for b in range(B):
            a, e = off[k * B + b], off[k * B + b + 1]
            want = q[k][idx[a:e]].astype(np.int64).sum(axis=0) if e > a else np.zeros(d, np.int64)
            assert np.array_equal(got[b, k * d:(k + 1) * d], want.astype(np.float32))


def test_embbag_lp_int8_two_roundings(orc):
    """(s * q) + z is rounded after the product and again after the sum: with
    s = 1 + 2^-23, q = 127, z = -127 the product 127 + 127 * 2^-23 rounds to
    127 + 2^-16 (the fp32 spacing at 127 is 2^-17), so the value is exactly
    2^-16; a fused multiply-add would give 127 * 2^-23.  A bag of the row twice
    pools to 2^-15."""
    s = np.float32(1.0 + 2.0 ** -23)
    q = [np.full((1, 4), 127, np.int8)]
    sb = [np.array([[s, -127.0]], np.float32)]
    off = np.array([0, 1, 3], dtype=np.int64)
    idx = np.array([0, 0, 0], dtype=np.int64)
    got = orc.embbag_fwd_lp(q, "int8", idx, off, 2, scale_bias=sb)
    assert np.all(got[0] == np.float32(2.0 ** -16))
    assert np.all(got[1] == np.float32(2.0 ** -15))
    assert 2.0 ** -16 != 127 * 2.0 ** -23


def test_embbag_lp_int8_affine_dyadic(orc):
    """Dyadic scale and bias: (q / 8) + 1/2 is exact, so the pooled values
    equal the exact rational sums."""
    from fractions import Fraction

    g = np.random.default_rng(13)
    K, B, d, rows = 1, 25, 4, [11]
    q = [g.integers(-128, 128, size=(rows[0], d)).astype(np.int8)]
    sb = [np.tile(np.array([0.125, 0.5], np.float32), (rows[0], 1))]
    idx, off = _rand_bags(g, K, B, rows, 6)
    got = orc.embbag_fwd_lp(q, "int8", idx, off, B, scale_bias=sb)
    for b in range(B):
        for c in range(d):
            want = sum((Fraction(int(q[0][r, c]), 8) + Fraction(1, 2) for r in idx[off[b]:off[b + 1]]), Fraction(0))
            assert Fraction(float(got[b, c])) == want


# --------------------------------------------------------------------------- interaction

@pytest.mark.parametrize("n,d", [(9, 16), (27, 128), (101, 64), (2, 4), (1, 8)])
def test_interact_integer_X_exact_against_integer_gram(orc, n, d):
    # Small-integer X: every dot product is an exact integer; the oracle must
    # reproduce numpy's integer Gram matrix at tril_indices(n, -1) bit for bit.
    g = np.random.default_rng(n * 1000 + d)
    B = 5
    Xi = g.integers(-8, 9, size=(B, n, d))
    out = orc.interact_fwd(Xi.astype(np.float32))
    assert out.shape == (B, d + n * (n - 1) // 2)
    ii, jj = np.tril_indices(n, -1)
    for b in range(B):
        gram = Xi[b] @ Xi[b].T
        assert np.array_equal(out[b, :d], Xi[b, 0].astype(np.float32))
        assert np.array_equal(out[b, d:], gram[ii, jj].astype(np.float32))


def test_interact_against_torch_bmm_fp64(orc):
    g = np.random.default_rng(5)
    B, n, d = 16, 27, 128
    X = g.standard_normal((B, n, d)).astype(np.float32)
    out = orc.interact_fwd(X)
    Xt = torch.from_numpy(X.astype(np.float64))
    gram = torch.bmm(Xt, Xt.transpose(1, 2).contiguous()).numpy()
    mag = torch.bmm(Xt.abs(), Xt.abs().transpose(1, 2).contiguous()).numpy()
    ii, jj = np.tril_indices(n, -1)
    ref, m = gram[:, ii, jj], mag[:, ii, jj]
    # one fp32 rounding of an fp64 sum: |err| <= u |ref| + d * 2**-53 * sum|x_i x_j|
    assert np.all(np.abs(out[:, d:] - ref) <= U32 * np.abs(ref) + 2 * d * 2.0 ** -53 * m)


def test_interact_symmetry_under_row_permutation(orc):
    # X X^T is symmetric: permuting the embedding rows permutes the pairs;
    # Z[pi(i), pi(j)] of the permuted input equals Z[i, j] of the original.
    g = np.random.default_rng(6)
    B, n, d = 4, 9, 16
    X = g.standard_normal((B, n, d)).astype(np.float32)
    perm = np.concatenate([[0], 1 + g.permutation(n - 1)])
    Xp = np.empty_like(X)
    Xp[:, perm] = X
    z = orc.interact_fwd(X)[:, d:]
    zp = orc.interact_fwd(Xp)[:, d:]

    def at(zz, i, j):
        i, j = max(i, j), min(i, j)
        return zz[:, i * (i - 1) // 2 + j]

    for i in range(1, n):
        for j in range(i):
            assert np.array_equal(at(zp, perm[i], perm[j]), at(z, i, j))


def test_interact_orthogonal_and_identical_rows(orc):
    n, d = 9, 16
    X = np.zeros((1, n, d), np.float32)
    for i in range(n):
        X[0, i, i] = i + 1.0  # orthogonal rows
    assert np.all(orc.interact_fwd(X)[0, d:] == 0)
    v = np.random.default_rng(7).standard_normal(d).astype(np.float32)
    Y = np.tile(v, (1, n, 1))
    z = orc.interact_fwd(Y)[0, d:]
    assert np.allclose(z, float((v.astype(np.float64) ** 2).sum()), rtol=1e-6) and np.all(z == z[0])


def test_interact_bwd_against_autograd(orc):
    # the interaction's forward map built from torch ops in fp64, differentiated
    # by autograd: dL/dX for L = sum(g * [X_0, tril(X X^T)])
    rng = np.random.default_rng(11)
    B, n, d = 5, 27, 32
    X = rng.standard_normal((B, n, d)).astype(np.float32)
    g = rng.standard_normal((B, d + n * (n - 1) // 2)).astype(np.float32)
    Xt = torch.from_numpy(X.astype(np.float64)).requires_grad_(True)
    ii, jj = np.tril_indices(n, -1)
    gram = torch.bmm(Xt, Xt.transpose(1, 2))
    y = torch.cat([Xt[:, 0, :], gram[:, ii, jj]], dim=1)
    (y * torch.from_numpy(g.astype(np.float64))).sum().backward()
    ref = Xt.grad.numpy()
    got = orc.interact_bwd(X, g)
    # one fp32 rounding of an fp64 sum
    mag = np.abs(ref) + 1e-30
    assert np.all(np.abs(got - ref) <= 2.0 ** -24 * mag + 1e-12)


def test_interact_bwd_finite_differences(orc):
    # central differences of the oracle's own forward, L(X) = sum(g * y(X)),
    # on small integer-valued inputs where y is exact in fp32
    rng = np.random.default_rng(12)
    B, n, d = 2, 6, 5
    X = rng.integers(-3, 4, size=(B, n, d)).astype(np.float32)
    g = rng.integers(-2, 3, size=(B, d + n * (n - 1) // 2)).astype(np.float32)
    got = orc.interact_bwd(X, g)

    def loss(Xv):
        return float((orc.interact_fwd(Xv).astype(np.float64) * g).sum())

    h = 0.5  # L is quadratic in X: central differences are exact for any h
    for b in range(B):
        for i in range(n):
            for c in range(d):
                Xp, Xm = X.copy(), X.copy()
                Xp[b, i, c] += h
                Xm[b, i, c] -= h
                fd = (loss(Xp) - loss(Xm)) / (2 * h)
                assert fd == got[b, i, c], (b, i, c, fd, got[b, i, c])


def test_interact_bwd_structure(orc):
    rng = np.random.default_rng(13)
    B, n, d = 3, 9, 16
    X = rng.standard_normal((B, n, d)).astype(np.float32)
    P = n * (n - 1) // 2
    # no pair gradient: only the dense row receives the dense part of g
    g = np.zeros((B, d + P), np.float32)
    g[:, :d] = rng.standard_normal((B, d))
    dX = orc.interact_bwd(X, g)
    assert np.array_equal(dX[:, 0], g[:, :d]) and np.all(dX[:, 1:] == 0)
    # a single pair (i, j) = (4, 2) with weight 1: rows 4 and 2 receive X_2 and X_4
    g = np.zeros((B, d + P), np.float32)
    g[:, d + 4 * 3 // 2 + 2] = 1.0
    dX = orc.interact_bwd(X, g)
    assert np.array_equal(dX[:, 4], X[:, 2]) and np.array_equal(dX[:, 2], X[:, 4])
    others = [r for r in range(n) if r not in (2, 4)]
    assert np.all(dX[:, others] == 0)


# --------------------------------------------------------------------------- MLP

def test_bf16_round_against_torch(orc):
    g = np.random.default_rng(8)
    exps = np.arange(-149, 128)
    vals = [np.ldexp(g.random(64) + 0.5, int(e)) for e in exps]  # every binade, incl. subnormal
    x = np.concatenate(vals + [[0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]])
    x = np.concatenate([x, -x]).astype(np.float32)
    # exact ties: low 16 bits = 0x8000 with both parities of bit 16
    ties = (np.array([0x3F808000, 0x3F818000, 0x40008000, 0x00018000], dtype=np.uint32)).view(np.float32)
    x = np.concatenate([x, ties])
    got = orc.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    nan = orc.bf16_round(np.array([np.nan], np.float32))
    assert np.isnan(nan[0])


def _torch_mlp(x, Ws, bs, quant, last_relu):
    h = torch.from_numpy(x.astype(np.float64))
    for l, (w, b) in enumerate(zip(Ws, bs)):
        if quant:
            h = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)
        h = torch.nn.functional.linear(h, torch.from_numpy(w.astype(np.float64)), torch.from_numpy(b.astype(np.float64)))
        if l < len(Ws) - 1 or last_relu:
            h = torch.relu(h)
        h = h.to(torch.float32).to(torch.float64)  # each layer's output is stored in fp32
    return h.numpy()


@pytest.mark.parametrize("name,which", [("tiny", "bottom"), ("tiny", "top"), ("forward", "bottom"), ("forward", "top")])
def test_mlp_against_torch_linear(orc, name, which):
    w = W.get(name)
    params = W.mlp_params(w, which)
    Ws, bs = [p[0] for p in params], [p[2] for p in params]
    g = np.random.default_rng(9)
    x = (g.lognormal(0, 1, size=(64, Ws[0].shape[1])) if which == "bottom" else g.standard_normal((64, Ws[0].shape[1]))).astype(np.float32)
    quant = w.mlp_dtype == "bf16"
    last_relu = which == "bottom"
    out, prob, _ = orc.mlp_fwd(x, Ws, bs, quant, last_relu)
    ref = _torch_mlp(x, Ws, bs, quant, last_relu)
    # Both sides round each layer's exact result once to fp32 (and identically
    # to bf16 at layer inputs), so they may differ only where fp64 rounding
    # of the sum differs: allow a few fp32 ulps.
    assert np.allclose(out, ref, rtol=4 * U32, atol=1e-30)
    if prob is not None:
        assert np.allclose(prob, 1 / (1 + np.exp(-ref[:, 0])), rtol=1e-6)


def test_mlp_identity_weights_give_relu(orc):
    x = np.random.default_rng(10).standard_normal((8, 16)).astype(np.float32)
    I = np.eye(16, dtype=np.float32)
    z = np.zeros(16, np.float32)
    out, _, _ = orc.mlp_fwd(x, [I, I], [z, z], False, True)
    assert np.array_equal(out, np.maximum(x, 0))
    out, _, _ = orc.mlp_fwd(x, [I], [z], False, False)
    assert np.array_equal(out, x)


def test_mlp_bwd_against_autograd(orc):
    g = np.random.default_rng(11)
    dims = [13, 32, 16, 1]
    Ws = [(g.standard_normal((dims[i + 1], dims[i])) * np.sqrt(2 / dims[i])).astype(np.float32) for i in range(3)]
    Ws = [torch.from_numpy(w).to(torch.bfloat16).float().numpy() for w in Ws]
    bs = [g.uniform(-0.2, 0.2, dims[i + 1]).astype(np.float32) for i in range(3)]
    x = g.lognormal(0, 1, size=(48, 13)).astype(np.float32)
    y = (g.random(48) < 0.5).astype(np.float32)
    logit, prob, acts = orc.mlp_fwd(x, Ws, bs, True, False, save_acts=True)
    dY = ((prob - y) / 48).astype(np.float32).reshape(-1, 1)
    dWs, dbs, dX = orc.mlp_bwd(Ws, acts, dY, False, want_dx=True)
    # autograd in fp64 through the same bf16-rounded layer inputs
    tw = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in Ws]
    tb = [torch.tensor(b, dtype=torch.float64, requires_grad=True) for b in bs]
    tx = torch.tensor(acts[0], dtype=torch.float64, requires_grad=True)
    h = tx
    for l in range(3):
        if l > 0:
            h = h + (torch.from_numpy(acts[l].astype(np.float64)) - h).detach()  # same rounded input, identity gradient
        h = torch.nn.functional.linear(h, tw[l], tb[l])
        if l < 2:
            h = torch.relu(h)
    loss = torch.nn.functional.binary_cross_entropy_with_logits(h[:, 0], torch.from_numpy(y.astype(np.float64)))
    loss.backward()
    for l in range(3):
        assert np.allclose(dWs[l], tw[l].grad.numpy(), rtol=1e-5, atol=1e-9)
        assert np.allclose(dbs[l], tb[l].grad.numpy(), rtol=1e-5, atol=1e-9)
    assert np.allclose(dX, tx.grad.numpy(), rtol=1e-5, atol=1e-9)


def test_mlp_bwd_finite_differences(orc):
    # Central differences of the scalar L = sum(out * R) w.r.t. a few weights,
    # fp32 network without bf16 rounding (so the loss is piecewise linear and
    # smooth away from ReLU kinks).
    g = np.random.default_rng(12)
    dims = [5, 7, 3]
    Ws = [g.standard_normal((dims[i + 1], dims[i])).astype(np.float32) for i in range(2)]
    bs = [g.standard_normal(dims[i + 1]).astype(np.float32) for i in range(2)]
    x = g.standard_normal((6, 5)).astype(np.float32)
    Rw = g.standard_normal((6, 3)).astype(np.float32)
    out, _, acts = orc.mlp_fwd(x, Ws, bs, False, False, save_acts=True)
    dWs, dbs, _ = orc.mlp_bwd(Ws, acts, Rw, False)

    def loss(Wl):
        h = x.astype(np.float64)
        for l in range(2):
            h = h @ Wl[l].T.astype(np.float64) + bs[l]
            if l == 0:
                h = np.maximum(h, 0)
        return float((h * Rw).sum())

    eps = 1e-4
    for l in range(2):
        for (o, i) in [(0, 0), (1, 2), (dims[l + 1] - 1, dims[l] - 1)]:
            Wp = [w.astype(np.float64).copy() for w in Ws]
            Wm = [w.astype(np.float64).copy() for w in Ws]
            Wp[l][o, i] += eps
            Wm[l][o, i] -= eps
            fd = (loss(Wp) - loss(Wm)) / (2 * eps)
            assert abs(fd - dWs[l][o, i]) <= 1e-4 * max(1.0, abs(fd))


# --------------------------------------------------------------------------- sparse backward + SGD

def _sort_based_sgd(tabs, idx, off, B, G, g_col0, lr, block=128):
    """Second formulation: stable sort of (table, row) keys, then segmented
    fp32 sums over the sorted occurrences (in blocks of `block` occurrences,
    each summed from +0, the block sums added from +0) and one update per
    unique row."""
    K, d = len(tabs), tabs[0].shape[1]
    out = [t.copy() for t in tabs]
    bag = np.repeat(np.arange(K * B), np.diff(off))
    tbl = bag // B
    key = tbl.astype(np.int64) * (1 << 40) + idx
    order = np.argsort(key, kind="stable")
    sk = key[order]
    heads = np.flatnonzero(np.concatenate([[True], sk[1:] != sk[:-1]]))
    ends = np.concatenate([heads[1:], [len(sk)]])
    for h, e in zip(heads, ends):
        k, r = int(sk[h] >> 40), int(sk[h] & ((1 << 40) - 1))
        gsum = np.zeros(d, np.float32)
        occ = order[h:e]
        for j0 in range(0, len(occ), block):
            part = np.zeros(d, np.float32)
            for q in occ[j0:j0 + block]:
                b = bag[q] % B
                part = (part + G[b, g_col0 + k * d: g_col0 + (k + 1) * d]).astype(np.float32)
            gsum = (gsum + part).astype(np.float32)
        out[k][r] = (out[k][r] - (np.float32(lr) * gsum).astype(np.float32)).astype(np.float32)
    return out


def test_sparse_sgd_matches_sort_based_formulation(orc):
    g = np.random.default_rng(13)
    K, B, d, rows = 3, 50, 16, [20, 7, 33]
    tabs = [g.standard_normal((m, d)).astype(np.float32) for m in rows]
    idx, off = _rand_bags(g, K, B, rows, 12)
    G = (g.standard_normal((B, (K + 1) * d)) * 0.01).astype(np.float32)
    ref = _sort_based_sgd(tabs, idx, off, B, G, d, 0.01)
    got = [t.copy() for t in tabs]
    orc.embbag_bwd_sgd(got, idx, off, B, G, d, 0.01)
    for a, b in zip(got, ref):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_sparse_sgd_long_rows_sum_in_blocks_of_128(orc):
    """Rows with up to several hundred occurrences: the update follows the blocked order
    (blocks of 128 in position order, block sums added in order); up to 129
    occurrences that is the plain left-to-right sum, and on the long rows the
    two orders give different bits (so the order is really pinned)."""
    g = np.random.default_rng(18)
    K, B, d = 2, 600, 8
    rows = [6, 40]
    lens = g.integers(0, 5, size=K * B)
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    idx = np.concatenate([np.minimum(g.zipf(1.3, size=off[(k + 1) * B] - off[k * B]) - 1, rows[k] - 1)
                          for k in range(K)]).astype(np.int64)
    tabs = [g.standard_normal((m, d)).astype(np.float32) for m in rows]
    # gradients of mixed magnitude, so that the summation order shows in the bits
    G = (g.standard_normal((B, K * d)) * np.exp2(g.integers(-12, 12, size=(B, K * d)))).astype(np.float32)
    got = [t.copy() for t in tabs]
    orc.embbag_bwd_sgd(got, idx, off, B, G, 0, 0.01)
    blocked = _sort_based_sgd(tabs, idx, off, B, G, 0, 0.01, block=128)
    plain = _sort_based_sgd(tabs, idx, off, B, G, 0, 0.01, block=1 << 30)
    for k in range(K):
        assert np.array_equal(got[k].view(np.uint32), blocked[k].view(np.uint32))
        cnt = np.bincount(idx[off[k * B]:off[(k + 1) * B]], minlength=rows[k])
        short = cnt <= 129
        assert np.array_equal(blocked[k][short].view(np.uint32), plain[k][short].view(np.uint32))
    assert max(np.bincount(idx[off[k * B]:off[(k + 1) * B]]).max() for k in range(K)) > 400
    assert any(not np.array_equal(blocked[k].view(np.uint32), plain[k].view(np.uint32)) for k in range(K))


def test_sparse_sgd_single_occurrence_and_untouched(orc):
    tabs = [np.random.default_rng(14).standard_normal((10, 8)).astype(np.float32)]
    before = tabs[0].copy()
    idx = np.array([3], dtype=np.int64)
    off = np.array([0, 1], dtype=np.int64)
    G = np.random.default_rng(15).standard_normal((1, 8)).astype(np.float32)
    orc.embbag_bwd_sgd(tabs, idx, off, 1, G, 0, 0.01)
    exp = (before[3] - (np.float32(0.01) * G[0]).astype(np.float32)).astype(np.float32)
    assert np.array_equal(tabs[0][3], exp)
    mask = np.ones(10, bool)
    mask[3] = False
    assert np.array_equal(tabs[0][mask].view(np.uint32), before[mask].view(np.uint32))


def test_sparse_sgd_dyadic_exact(orc):
    # G = j/64 with |j| <= 32 and lr = 2**-7: every sum and the update are
    # exact, so the result equals integer arithmetic whatever the grouping.
    g = np.random.default_rng(16)
    K, B, d, rows = 2, 30, 8, [5, 9]
    tint = [g.integers(-1000, 1001, size=(m, d)) for m in rows]
    tabs = [(t / 2.0 ** 13).astype(np.float32) for t in tint]
    idx, off = _rand_bags(g, K, B, rows, 20)
    Gi = g.integers(-32, 33, size=(B, K * d))
    G = (Gi / 64.0).astype(np.float32)
    orc.embbag_bwd_sgd(tabs, idx, off, B, G, 0, 2.0 ** -7)
    for k in range(K):
        acc = np.zeros((rows[k], d), np.int64)
        for b in range(B):
            for p in range(off[k * B + b], off[k * B + b + 1]):
                acc[idx[p]] += Gi[b, k * d:(k + 1) * d]
        # T - 2**-7 * acc/64 = (T * 2**13 - acc) / 2**13
        exp = ((tint[k] - acc) / 2.0 ** 13).astype(np.float32)
        assert np.array_equal(tabs[k], exp)


def test_sparse_sgd_against_index_add_fp64(orc):
    # Conservation and accuracy against torch index_add_ in fp64.
    g = np.random.default_rng(17)
    K, B, d, rows = 2, 200, 16, [40, 300]
    tabs = [g.standard_normal((m, d)).astype(np.float32) for m in rows]
    idx, off = _rand_bags(g, K, B, rows, 30)
    G = g.standard_normal((B, K * d)).astype(np.float32)
    got = [t.copy() for t in tabs]
    lr = 0.01
    orc.embbag_bwd_sgd(got, idx, off, B, G, 0, lr)
    for k in range(K):
        a, e = off[k * B], off[(k + 1) * B]
        bag = np.repeat(np.arange(B), np.diff(off[k * B:(k + 1) * B + 1]))
        src = torch.from_numpy(G[bag, k * d:(k + 1) * d].astype(np.float64))
        gsum = torch.zeros(rows[k], d, dtype=torch.float64).index_add_(0, torch.from_numpy(idx[a:e]), src).numpy()
        gabs = torch.zeros(rows[k], d, dtype=torch.float64).index_add_(0, torch.from_numpy(idx[a:e]), src.abs()).numpy()
        cnt = np.bincount(idx[a:e], minlength=rows[k])[:, None]
        ref = tabs[k].astype(np.float64) - lr * gsum
        # sum error (S-1) u sum|G|, times lr, plus the two final roundings
        bound = lr * np.maximum(cnt - 1, 0) * U32 * gabs * 1.001 + U32 * (np.abs(ref) + lr * np.abs(gsum)) * 2.001
        assert np.all(np.abs(got[k].astype(np.float64) - ref) <= bound + 1e-30)
        # conservation: total applied update equals lr * sum of all G routed to table k
        applied = (tabs[k].astype(np.float64) - got[k].astype(np.float64)).sum()
        assert abs(applied - lr * src.numpy().sum()) <= 1e-4 * lr * np.abs(src.numpy()).sum()
