"""End-to-end forward pass (and training step) on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from dlrm_cases import DEV, banner, bits, device_model, interaction_tolerance, oracle_forward, to_dev
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _forward(w, model, batch=0):
    dense = W.dense(w, batch)
    idx, off = W.indices_offsets(w, batch)
    model.forward(to_dev(dense), to_dev(idx), to_dev(off))
    torch.cuda.synchronize()
    return dense, idx, off


def test_forward_tiny_fp32():
    w = W.get("tiny")
    banner("forward tiny (fp32 network)")
    model, bottom, top = device_model(w)
    dense, idx, off = _forward(w, model)
    X, top_in, logit, prob = oracle_forward(w, dense, idx, off, bottom, top)
    gX = model.X.cpu().numpy()
    assert np.array_equal(bits(gX[:, 1:]), bits(X[:, 1:]))  # pooled embeddings bit-exact
    assert np.all(np.abs(gX[:, 0] - X[:, 0]) <= 1e-4 * np.maximum(1, np.abs(X[:, 0])))
    gl = model.logit.cpu().numpy()[:, 0]
    assert np.all(np.abs(gl - logit) <= 1e-4 * np.maximum(1.0, np.abs(logit)))
    assert np.max(np.abs(model.prob.cpu().numpy() - prob)) <= 1e-5


@pytest.mark.parametrize("name,B,rows", [("forward", 2000, 10_000), ("interaction", 1000, 10_000),
                                         ("train", 1000, 10_000)])
def test_forward_bf16_scaled(name, B, rows):
    w = W.get(name).scaled(B=B, rows=rows)
    banner(f"forward {name} scaled B={B} rows={rows}")
    model, bottom, top = device_model(w)
    dense, idx, off = _forward(w, model)
    X, top_in, logit, prob = oracle_forward(w, dense, idx, off, bottom, top)
    gX = model.X.cpu().numpy()
    assert np.array_equal(bits(gX[:, 1:]), bits(X[:, 1:]))
    gl = model.logit.cpu().numpy()[:, 0]
    assert np.max(np.abs(gl - logit)) <= 2e-2
    assert np.max(np.abs(model.prob.cpu().numpy() - prob)) <= 2e-2 / 4


def test_forward_full_size_sampled():
    """The full forward workload in the benchmark's launch configuration
    (26 tables, about 2e8 rows, batch 32768): sampled samples against the
    oracle."""
    w = W.get("forward")
    banner(f"forward full size: rows={sum(w.rows)} B={w.B}")
    model, bottom, top = device_model(w)
    dense, idx, off = _forward(w, model)
    samples = np.sort(np.random.default_rng(2).choice(w.B, 256, replace=False))
    samples[-1] = w.B - 1
    sel = torch.from_numpy(samples).to(DEV)
    gX = model.X[sel].cpu().numpy()
    gl = model.logit[sel].cpu().numpy()[:, 0]
    gtop = model.top_in[sel].float().cpu().numpy()
    del model
    torch.cuda.empty_cache()
    X, top_in, logit, prob = oracle_forward(w, dense, idx, off, bottom, top, samples=samples)
    assert np.array_equal(bits(gX[:, 1:]), bits(X[:, 1:]))
    # interaction values (bf16 row): within one bf16 ulp of the oracle's
    ref_b = torch.from_numpy(top_in).to(torch.bfloat16).float().numpy()
    assert np.all(np.abs(gtop[:, :w.top_in] - ref_b) <= np.abs(ref_b) * 2.0 ** -7 + 2e-2 * 2.0 ** -7)
    assert np.max(np.abs(gl - logit)) <= 2e-2


def test_train_step_scaled():
    import deep_learning_recommendation_amd as D  # noqa: F401

    w = W.get("train").scaled(B=1024, rows=100_000)
    banner("train step scaled")
    model, bottom, top = device_model(w, train=True)
    dense, idx, off = W.dense(w), *W.indices_offsets(w)
    G = W.upstream_grad(w)
    y = W.labels(w)
    idx_d, off_d = to_dev(idx), to_dev(off)
    model.forward(to_dev(dense), idx_d, off_d)
    model.backward(to_dev(y), to_dev(G), idx_d, off_d, int(off[-1]), w.lr)
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
