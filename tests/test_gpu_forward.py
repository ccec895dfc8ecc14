"""End-to-end forward pass (and training step) on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from dlrm_cases import DEV, banner, bf16_row_tolerance, bits, device_model, oracle_forward, to_dev
from synth import device as SD
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _forward(w, model, batch=0):
    dense = W.dense(w, batch)
    idx, off = W.indices_offsets(w, batch)
    model.forward(to_dev(dense), to_dev(idx), to_dev(off))
    torch.cuda.synchronize()
    return dense, idx, off


def _both(w):
    """Run the two-call path (X materialised) and the fused path on the same
    inputs; the top-MLP input rows must agree bit for bit."""
    model, bottom, top = device_model(w, fused=False)
    dense, idx, off = _forward(w, model)
    fused, _, _ = device_model(w, tables=model.tables, fused=True)
    _forward(w, fused)
    a = model.top_in.view(torch.int16 if model.top_in.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    b = fused.top_in.view(torch.int16 if fused.top_in.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    width = model.top_w
    assert np.array_equal(a[:, :width], b[:, :width])
    assert np.array_equal(model.logit.cpu().numpy(), fused.logit.cpu().numpy())
    return model, fused, bottom, top, dense, idx, off


def test_forward_tiny_fp32():
    w = W.get("tiny")
    banner("forward tiny (fp32 network)")
    model, fused, bottom, top, dense, idx, off = _both(w)
    X, top_in, logit, prob = oracle_forward(w, dense, idx, off, bottom, top)
    gX = model.X.cpu().numpy()
    assert np.array_equal(bits(gX[:, 1:]), bits(X[:, 1:]))  # pooled embeddings bit-exact
    # fp32 network: bottom output and logit within 1e-5 * max(1, |ref|) (each
    # layer is one fp32 multiply-add chain, within gamma_65 ~ 3.9e-6 of
    # sum |w x| + |b|, two layers compounding), the probability within 1e-6
    # (sigma is 1/4-Lipschitz)
    assert np.all(np.abs(gX[:, 0] - X[:, 0]) <= 1e-5 * np.maximum(1, np.abs(X[:, 0])))
    gl = fused.logit.cpu().numpy()[:, 0]
    assert np.all(np.abs(gl - logit) <= 1e-5 * np.maximum(1.0, np.abs(logit)))
    assert np.max(np.abs(fused.prob.cpu().numpy() - prob)) <= 1e-6


@pytest.mark.parametrize("name,B,rows", [("forward", 2000, 10_000), ("interaction", 1000, 10_000),
                                         ("train", 1000, 10_000)])
def test_forward_bf16_scaled(name, B, rows):
    w = W.get(name).scaled(B=B, rows=rows)
    banner(f"forward {name} scaled B={B} rows={rows}")
    model, fused, bottom, top, dense, idx, off = _both(w)
    X, top_in, logit, prob = oracle_forward(w, dense, idx, off, bottom, top)
    gX = model.X.cpu().numpy()
    assert np.array_equal(bits(gX[:, 1:]), bits(X[:, 1:]))
    gl = fused.logit.cpu().numpy()[:, 0]
    assert np.max(np.abs(gl - logit)) <= 2e-2
    assert np.max(np.abs(fused.prob.cpu().numpy() - prob)) <= 2e-2 / 4


def test_forward_full_size_sampled():
    """The full forward workload in the benchmark's launch configuration (26
    tables, about 2e8 rows, batch 32768).  The fused and the two-call paths
    give bit-identical top-MLP inputs and logits for the whole batch; on
    sampled samples the pooled rows are bit-exact against the oracle, the
    dense part of the top-MLP input is the bf16 rounding of the device's own
    bottom-MLP output, the pairs are within the bf16 row bound of the
    oracle's interaction of [device x_dense; oracle pooled rows], and the
    logits are within 2e-2 of the oracle's whole forward pass."""
    w = W.get("forward")
    banner(f"forward full size: rows={sum(w.rows)} B={w.B}")
    model, bottom, top = device_model(w, fused=False)
    dense, idx, off = _forward(w, model)
    fused, _, _ = device_model(w, tables=model.tables, fused=True)
    _forward(w, fused)
    width = model.top_w
    assert torch.equal(model.top_in[:, :width].view(torch.int16), fused.top_in[:, :width].view(torch.int16))
    assert torch.equal(model.logit.view(torch.int32), fused.logit.view(torch.int32))
    samples = np.sort(np.random.default_rng(2).choice(w.B, 256, replace=False))
    samples[-1] = w.B - 1
    sel = torch.from_numpy(samples).to(DEV)
    gl = fused.logit[sel].cpu().numpy()[:, 0]
    gtop = fused.top_in[sel].float().cpu().numpy()
    gX = model.X[sel].cpu().numpy()
    del model, fused
    torch.cuda.empty_cache()
    X, top_in, logit, prob = oracle_forward(w, dense, idx, off, bottom, top, samples=samples)
    d = w.d
    assert np.array_equal(bits(gX[:, 1:]), bits(X[:, 1:]))  # pooled rows bit-exact
    # dense part: the device's x_dense rounded to bf16 (exactly)
    xd = torch.from_numpy(np.ascontiguousarray(gX[:, 0])).to(torch.bfloat16).float().numpy()
    assert np.array_equal(bits(gtop[:, :d]), bits(xd))
    # pairs: the oracle's interaction of the device's own X (its x_dense
    # comes from the bf16 bottom MLP), within the dot-product bound plus
    # one bf16 rounding
    Xd = np.concatenate([gX[:, :1], X[:, 1:]], axis=1)
    ref_row = oracle.interact_fwd(Xd)
    tol = bf16_row_tolerance(Xd, ref_row)
    assert np.all(np.abs(gtop[:, d:w.top_in] - ref_row[:, d:]) <= tol[:, d:])
    # the bottom MLP output against the oracle's (bf16 network, fp32 row)
    assert np.max(np.abs(gX[:, 0] - X[:, 0])) <= 2e-2 * max(1.0, float(np.abs(X[:, 0]).max()))
    assert np.max(np.abs(gl - logit)) <= 2e-2


def test_forward_interaction_full_size_sampled():
    """The interaction-heavy workload at full size (100 tables of 100,000
    rows, batch 16384, bags of 4): pooled rows bit-exact and logits within
    2e-2 on sampled samples (the two-call path, which the pipeline takes for
    bags of four)."""
    w = W.get("interaction")
    banner(f"interaction workload full size: K={w.K} B={w.B}")
    model, bottom, top = device_model(w, fused="auto")
    dense, idx, off = _forward(w, model)
    assert not model.use_fused(int(off[-1]))
    samples = np.sort(np.random.default_rng(4).choice(w.B, 192, replace=False))
    samples[-1] = w.B - 1
    sel = torch.from_numpy(samples).to(DEV)
    gl = model.logit[sel].cpu().numpy()[:, 0]
    gX = model.X[sel].cpu().numpy()
    gtop = model.top_in[sel].float().cpu().numpy()
    del model
    torch.cuda.empty_cache()
    X, top_in, logit, prob = oracle_forward(w, dense, idx, off, bottom, top, samples=samples)
    assert np.array_equal(bits(gX[:, 1:]), bits(X[:, 1:]))
    Xd = np.concatenate([gX[:, :1], X[:, 1:]], axis=1)
    ref_row = oracle.interact_fwd(Xd)
    tol = bf16_row_tolerance(Xd, ref_row)
    assert np.all(np.abs(gtop[:, w.d:w.top_in] - ref_row[:, w.d:]) <= tol[:, w.d:])
    assert np.max(np.abs(gl - logit)) <= 2e-2


@pytest.mark.parametrize("prepared,side", [(False, False), (True, False), (True, True)])
def test_train_step_scaled(prepared, side):
    """prepared: the sparse update's index half runs on a second stream
    beside the forward (sparse_prepare), the update after the backward
    (side: with its short segments on a third stream)."""
    import deep_learning_recommendation_amd as D  # noqa: F401

    w = W.get("train").scaled(B=1024, rows=100_000)
    banner(f"train step scaled prepared={prepared}")
    model, bottom, top = device_model(w, train=True)
    dense, idx, off = W.dense(w), *W.indices_offsets(w)
    G = W.upstream_grad(w)
    y = W.labels(w)
    idx_d, off_d = to_dev(idx), to_dev(off)
    nnz = int(off[-1])
    side = torch.cuda.Stream()
    if prepared:
        model.sparse_workspace(nnz)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            model.sparse_prepare(idx_d, off_d, nnz)
    model.forward(to_dev(dense), idx_d, off_d)
    torch.cuda.current_stream().wait_stream(side)
    model.backward(to_dev(y), to_dev(G), idx_d, off_d, nnz, w.lr, prepared=prepared,
                   side=torch.cuda.Stream() if side else None)
    torch.cuda.synchronize()
    # sparse update: bit-exact on every touched row
    tabs, local, row_ids = W.compact_rows(w, idx, off)
    oracle.embbag_bwd_sgd(tabs, local, off, w.B, G.reshape(w.B, -1), w.d, w.lr)
    for k in range(w.K):
        got = model.tables[k][torch.from_numpy(row_ids[k]).to(DEV)].cpu().numpy()
        assert np.array_equal(bits(got), bits(tabs[k]))
    # dense gradients of the top MLP from the BCE loss
    X, top_in, logit, prob = oracle_forward(w, dense, idx, off, bottom, top)
    _, _, acts = oracle.mlp_fwd(top_in, [p[0] for p in top], [p[2] for p in top], True, False, save_acts=True)
    dY = ((prob - y) / w.B).astype(np.float32).reshape(-1, 1)
    rW, rb, _ = oracle.mlp_bwd([p[0] for p in top], acts, dY, False)
    for l in range(len(rW)):
        g = model.dW_top[l].cpu().numpy()
        assert np.linalg.norm(g - rW[l]) <= 2e-2 * np.linalg.norm(rW[l]), l


def test_train_full_backward_chain_scaled():
    """Loss -> top MLP (input gradient) -> interaction backward -> bottom MLP
    and sparse SGD.  The gradient of X against the oracle's chain within the
    MLP-backward tolerance (the top MLP's bf16 backward dominates); the table
    update from the device's own X gradient bit-exact."""
    w = W.get("train").scaled(B=512, rows=50_000)
    banner("train full backward chain scaled")
    model, bottom, top = device_model(w, train=True, fused=False)
    dense, idx, off = W.dense(w), *W.indices_offsets(w)
    y = W.labels(w)
    idx_d, off_d = to_dev(idx), to_dev(off)
    model.forward(to_dev(dense), idx_d, off_d)
    model.backward_chain(to_dev(y), idx_d, off_d, int(off[-1]), w.lr)
    torch.cuda.synchronize()
    G = model.G.cpu().numpy()
    # oracle chain
    X, top_in, logit, prob = oracle_forward(w, dense, idx, off, bottom, top)
    _, _, acts = oracle.mlp_fwd(top_in, [p[0] for p in top], [p[2] for p in top], True, False, save_acts=True)
    dY = ((prob - y) / w.B).astype(np.float32).reshape(-1, 1)
    _, _, g_top = oracle.mlp_bwd([p[0] for p in top], acts, dY, False, want_dx=True)
    G_ref = oracle.interact_bwd(X, g_top)
    assert np.linalg.norm(G - G_ref) <= 2e-2 * np.linalg.norm(G_ref)
    # the sparse update consumed rows 1..K of the device's G: bit-exact
    tabs, local, row_ids = W.compact_rows(w, idx, off)
    oracle.embbag_bwd_sgd(tabs, local, off, w.B, G.reshape(w.B, -1), w.d, w.lr)
    for k in range(w.K):
        got = model.tables[k][torch.from_numpy(row_ids[k]).to(DEV)].cpu().numpy()
        assert np.array_equal(bits(got), bits(tabs[k])), k
    # bottom MLP weight gradients from row 0 of the device's G
    _, _, acts_b = oracle.mlp_fwd(dense, [p[0] for p in bottom], [p[2] for p in bottom], True, True, save_acts=True)
    rW, _, _ = oracle.mlp_bwd([p[0] for p in bottom], acts_b, G[:, 0, :], True)
    for l in range(len(rW)):
        g = model.dW_bot[l].cpu().numpy()
        assert np.linalg.norm(g - rW[l]) <= 2e-2 * np.linalg.norm(rW[l]), l


@pytest.mark.parametrize("name,expect_fused", [("forward", True), ("interaction", False), ("train", False)])
def test_forward_auto_path(name, expect_fused):
    """fused="auto" takes the fused call for one-index bags and the two calls
    for longer bags; either way the logits equal the explicit path's bits."""
    w = W.get(name).scaled(B=700, rows=8_000)
    banner(f"forward auto path {name}")
    auto, _, _ = device_model(w, fused="auto")
    dense, idx, off = _forward(w, auto)
    assert auto.use_fused(int(off[-1])) == expect_fused
    ref, _, _ = device_model(w, tables=auto.tables, fused=expect_fused)
    _forward(w, ref)
    assert np.array_equal(auto.logit.cpu().numpy().view(np.uint32), ref.logit.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
@pytest.mark.parametrize("fused", [True, False])
def test_forward_lowprec_rows_equal_widened_fp32(dtype, fused):
    """A forward pass from bf16 / int8 table rows against the same model on
    fp32 tables holding the decoded values (bf16 widened; (s * q) + z in two
    fp32 roundings, computed here with separate torch ops): bit for bit on the
    two-call path; on the fused path the dense part bit for bit and the
    logits within 1e-3 (the pair sums run in another column order there)."""
    from deep_learning_recommendation_amd import pipeline as PL

    w = W.get("forward").scaled(B=700, rows=8_000)
    banner(f"forward from {dtype} rows fused={fused}")
    tabs, sbs = SD.make_tables_lp(w, dtype)
    if dtype == "bf16":
        f32 = [(t.to(torch.int32) << 16).view(torch.float32).contiguous() for t in tabs]
    else:
        f32 = [(t.to(torch.float32) * sb[:, 0:1]) + sb[:, 1:2] for t, sb in zip(tabs, sbs)]
    ref, bottom, top = device_model(w, tables=f32, fused=fused)
    dense, idx, off = _forward(w, ref)
    bf16 = w.mlp_dtype == "bf16"
    bp = PL.make_mlp(w.bottom, [p[0] for p in bottom], [p[2] for p in bottom], bf16)
    tp = PL.make_mlp(w.top, [p[0] for p in top], [p[2] for p in top], bf16)
    lp = PL.DLRM(w.B, w.K, w.d, w.rows, tabs, bp, tp, fused=fused, table_dtype=dtype, scale_bias=sbs)
    _forward(w, lp)
    if not fused:
        assert np.array_equal(lp.logit.cpu().numpy().view(np.uint32), ref.logit.cpu().numpy().view(np.uint32))
        assert np.array_equal(lp.top_in.view(torch.int16).cpu().numpy(), ref.top_in.view(torch.int16).cpu().numpy())
    else:
        a = lp.top_in[:, :w.d].view(torch.int16).cpu().numpy()
        b = ref.top_in[:, :w.d].view(torch.int16).cpu().numpy()
        assert np.array_equal(a, b)
        assert np.max(np.abs(lp.logit.cpu().numpy() - ref.logit.cpu().numpy())) <= 1e-3


def test_forward_padded_top_layer_bit_identical():
    """A forward-only model reads the 479-wide interaction rows as K = 512
    (zero weight columns over zero input columns): its logits equal those of
    the unpadded model bit for bit, and the input columns past the
    interaction's written width stay zero after the forward pass."""
    from deep_learning_recommendation_amd import pipeline as PL

    w = W.get("forward").scaled(B=3000, rows=20_000)
    banner("forward padded vs unpadded top layer")
    padded, bottom, top = device_model(w, fused=True)
    assert padded.top.dims[0] == 512 and padded.top_ld == 512
    dense, idx, off = _forward(w, padded)
    bf16 = w.mlp_dtype == "bf16"
    bp = PL.make_mlp(w.bottom, [p[0] for p in bottom], [p[2] for p in bottom], bf16)
    tp = PL.make_mlp(w.top, [p[0] for p in top], [p[2] for p in top], bf16)
    plain = PL.DLRM(w.B, w.K, w.d, w.rows, padded.tables, bp, tp, fused=True, pad_top=False)
    assert plain.top.dims[0] == 479
    _forward(w, plain)
    assert torch.equal(padded.logit.view(torch.int32), plain.logit.view(torch.int32))
    assert torch.count_nonzero(padded.top_in[:, padded.top_written:]).item() == 0
    assert torch.equal(padded.top_in[:, :padded.top_written].view(torch.int16),
                       plain.top_in[:, :plain.top_written].view(torch.int16))
