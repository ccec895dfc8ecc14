"""MLP forward/backward on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from dlrm_cases import DEV, banner, to_dev
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _mlp_dev(dims, params, bf16):
    from deep_learning_recommendation_amd import pipeline as PL

    return PL.make_mlp(dims, [p[0] for p in params], [p[2] for p in params], bf16)


def _fwd(mp, x, last_relu, save=False, in_bf16=False):
    import deep_learning_recommendation_amd as D

    B = x.shape[0]
    xin = to_dev(x)
    if in_bf16:
        ld = ((x.shape[1] + 7) // 8) * 8
        xb = torch.zeros((B, ld), dtype=torch.bfloat16, device=DEV)
        xb[:, :x.shape[1]] = xin.to(torch.bfloat16)
        xin = xb
    out_w = mp.dims[-1]
    out = torch.empty((B, out_w), dtype=torch.float32, device=DEV)
    prob = torch.empty((B,), dtype=torch.float32, device=DEV) if out_w == 1 else None
    ws = torch.empty((max(256, D.dlrm_mlp_workspace_size(B, mp.dims, mp.w_dtype, save)),), dtype=torch.uint8,
                     device=DEV)
    D.dlrm_mlp_fwd(xin, xin.shape[1], B, mp.dims, mp.Ws, mp.w_ld, mp.biases, mp.w_dtype,
                   D.DLRM_ACT_RELU if last_relu else D.DLRM_ACT_NONE, out, out_w, prob, ws, save)
    torch.cuda.synchronize()
    return out, prob, ws


@pytest.mark.parametrize("name,which", [("forward", "bottom"), ("forward", "top"), ("interaction", "bottom"),
                                        ("interaction", "top"), ("train", "top")])
def test_mlp_bf16_forward(name, which):
    w = W.get(name)
    dims = w.bottom if which == "bottom" else w.top
    B = 1000  # ragged against every tile size
    banner(f"mlp bf16 {name}/{which} dims={dims} B={B}")
    params = W.mlp_params(w, which)
    g = np.random.default_rng(11)
    if which == "bottom":
        x = (g.lognormal(0, 1, (B, dims[0])) if w.dense_dist == "lognormal" else g.standard_normal((B, dims[0])))
    else:
        x = g.standard_normal((B, dims[0])) * 0.5
    x = x.astype(np.float32)
    mp = _mlp_dev(dims, params, True)
    out, prob, _ = _fwd(mp, x, which == "bottom", in_bf16=(which == "top"))
    ref, ref_p, _ = oracle.mlp_fwd(x, [p[0] for p in params], [p[2] for p in params], True, which == "bottom")
    got = out.cpu().numpy()
    if which == "top":
        # logits: 2e-2 absolute (bf16 MLP against the bf16-emulating oracle)
        assert np.max(np.abs(got - ref)) <= 2e-2
        assert np.max(np.abs(prob.cpu().numpy() - ref_p)) <= 2e-2 / 4  # sigma is 1/4-Lipschitz
    else:
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err <= 1e-2, err
        assert np.max(np.abs(got - ref)) <= 2e-2 * max(1.0, np.abs(ref).max())


def test_mlp_f32_tiny_network():
    w = W.get("tiny")
    for which in ("bottom", "top"):
        dims = w.bottom if which == "bottom" else w.top
        banner(f"mlp fp32 tiny/{which}")
        params = W.mlp_params(w, which)
        x = np.random.default_rng(3).standard_normal((w.B, dims[0])).astype(np.float32)
        mp = _mlp_dev(dims, params, False)
        out, prob, _ = _fwd(mp, x, which == "bottom")
        ref, ref_p, _ = oracle.mlp_fwd(x, [p[0] for p in params], [p[2] for p in params], False, which == "bottom")
        # fp32 FMA chains over K <= 64 per layer against fp64 sums: within
        # 1e-5 * max(1, |ref|): each layer is one fp32 multiply-add chain,
        # within gamma_65 ~ 3.9e-6 of sum |w x| + |b|, two layers compounding
        assert np.all(np.abs(out.cpu().numpy() - ref) <= 1e-5 * np.maximum(1.0, np.abs(ref)))
        if prob is not None:
            assert np.max(np.abs(prob.cpu().numpy() - ref_p)) <= 1e-6


def test_mlp_identity_layers_exact():
    # W = I, b = 0 on bf16-representable inputs: every output is exact
    import deep_learning_recommendation_amd as D  # noqa: F401

    banner("mlp identity")
    d = 64
    I = np.eye(d, dtype=np.float32)
    z = np.zeros(d, np.float32)
    params = [(I, None, z), (I, None, z)]
    x = torch.randn(333, d).to(torch.bfloat16).float().numpy()
    mp = _mlp_dev((d, d, d), params, True)
    out, _, _ = _fwd(mp, x, True)
    assert np.array_equal(out.cpu().numpy(), np.maximum(x, 0))


def test_device_bf16_rounding_matches_torch():
    # fp32 input -> bf16 rounding on the device (the layer-0 conversion),
    # then an identity layer (one exact nonzero product per output): the fp32
    # output must be the nearest-even bf16 of the input, bit for bit, for
    # ties of both parities and values across the normal range.  (The bf16
    # MFMA reads subnormal operands as zero, so the identity layer cannot
    # show the rounding of values below 2**-126.)
    import deep_learning_recommendation_amd as D  # noqa: F401

    banner("device bf16 rounding")
    g = np.random.default_rng(4)
    vals = [np.ldexp(g.random(48) + 1.0, int(e)) for e in range(-126, 127, 3)]
    ties = np.array([0x3F808000, 0x3F818000, 0x40008000, 0x00818000, 0x00808000, 0x7F7F7FFF, 0x3F80FFFF],
                    dtype=np.uint32).view(np.float32)
    x = np.concatenate(vals + [ties, [1.0, 3.0e38]]).astype(np.float32)  # no signed zero: -0 + (+0 products) = +0
    x = np.concatenate([x, -x])
    d = 64
    x = np.concatenate([x, np.zeros((-len(x)) % d, np.float32)]).reshape(-1, d)
    I = np.eye(d, dtype=np.float32)
    mp = _mlp_dev((d, d), [(I, None, np.zeros(d, np.float32))], True)
    out, _, _ = _fwd(mp, x, False)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = out.cpu().numpy()
    bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
    detail = [(hex(int(x.view(np.uint32).flat[i])), hex(int(got.view(np.uint32).flat[i])),
               hex(int(ref.view(np.uint32).flat[i]))) for i in bad[:8]]
    assert bad.size == 0, f"{bad.size} mismatches (input, device, reference): {detail}"


@pytest.mark.parametrize("which,B", [("bottom", 520), ("top", 520), ("bottom", 517), ("top", 61),
                                     ("bottom", 8192), ("top", 8192), ("bottom", 8191), ("top", 8191)])
def test_mlp_bf16_backward(which, B):
    """The training workload's bottom and top MLPs, backward, against the
    oracle: dW, db and dX within 2e-2 in norm, and every db element within
    2e-2 of the sum of magnitudes it adds up (sum over b of |delta[b][o]|,
    bounded above by the same backward through |W| from |dY|).  B = 8192 is
    the training workload's own batch; 8191 leaves a ragged batch tile."""
    import deep_learning_recommendation_amd as D

    w = W.get("train")
    dims = w.bottom if which == "bottom" else w.top
    banner(f"mlp backward train/{which} B={B}")
    params = W.mlp_params(w, which)
    g = np.random.default_rng(21)
    x = (g.lognormal(0, 1, (B, dims[0])) if which == "bottom" else g.standard_normal((B, dims[0])) * 0.5)
    x = x.astype(np.float32)
    mp = _mlp_dev(dims, params, True)
    last_relu = which == "bottom"
    out, prob, ws = _fwd(mp, x, last_relu, save=True, in_bf16=(which == "top"))
    if which == "top":
        y = (g.random(B) < 0.5).astype(np.float32)
        dY_dev = torch.empty((B,), dtype=torch.float32, device=DEV)
        D.dlrm_bce_grad(out, 1, to_dev(y), B, dY_dev)
        torch.cuda.synchronize()
        dY = dY_dev.cpu().numpy().reshape(B, 1)
        # BCE seed (sigma(logit) - y) / B against the oracle's own forward
        ref_logit, ref_p, _ = oracle.mlp_fwd(x, [p[0] for p in params], [p[2] for p in params], True, False)
        assert np.max(np.abs(dY[:, 0] - (ref_p - y) / B)) <= 2e-2 / 4 / B + 1e-9
    else:
        dY = (g.standard_normal((B, dims[-1])) * 0.01).astype(np.float32)
        dY_dev = to_dev(dY)
    dWs = [torch.empty((o, i), dtype=torch.float32, device=DEV) for i, o in zip(dims[:-1], dims[1:])]
    dbs = [torch.empty((o,), dtype=torch.float32, device=DEV) for o in dims[1:]]
    dX = torch.empty((B, dims[0]), dtype=torch.float32, device=DEV)
    wsb = torch.empty((D.dlrm_mlp_bwd_workspace_size(B, dims),), dtype=torch.uint8, device=DEV)
    D.dlrm_mlp_bwd(B, dims, mp.Ws, mp.w_ld, D.DLRM_ACT_RELU if last_relu else D.DLRM_ACT_NONE, ws, out, dims[-1],
                   dY_dev, dims[-1], dWs, dbs, dX, dims[0], wsb)
    torch.cuda.synchronize()
    # oracle backward from its own saved activations (same bf16 rounding points)
    _, _, acts = oracle.mlp_fwd(x, [p[0] for p in params], [p[2] for p in params], True, last_relu, save_acts=True)
    rW, rb, rX = oracle.mlp_bwd([p[0] for p in params], acts, dY, last_relu, want_dx=True)

    def rel(a, b):
        return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)

    # sum over b of |delta[b][o]| is at most the bias gradient of the same
    # network run backward through |W| from |dY| (same ReLU masks)
    _, mag, _ = oracle.mlp_bwd([np.abs(p[0]) for p in params], acts, np.abs(dY), last_relu)
    for l in range(len(dims) - 1):
        assert rel(dWs[l].cpu().numpy(), rW[l]) <= 2e-2, (l, rel(dWs[l].cpu().numpy(), rW[l]))
        got_b = dbs[l].cpu().numpy()
        assert rel(got_b, rb[l]) <= 2e-2, (l, rel(got_b, rb[l]))
        err = np.abs(got_b.astype(np.float64) - rb[l])
        bound = 2e-2 * mag[l].astype(np.float64) + 1e-30
        assert np.all(err <= bound), (l, int(np.argmax(err / bound)), float(np.max(err / bound)))
    assert rel(dX.cpu().numpy(), rX) <= 2e-2


def _int_params(dims, seed, density):
    """Weights in {-1, 0, 1} (nonzero with probability `density`) and biases
    in {-2, .., 2}: every value exact in bf16."""
    g = np.random.default_rng(seed)
    out = []
    for fi, fo in zip(dims[:-1], dims[1:]):
        Wf = g.integers(-1, 2, size=(fo, fi)) * (g.random((fo, fi)) < density)
        b = g.integers(-2, 3, size=fo)
        out.append((Wf.astype(np.float32), None, b.astype(np.float32)))
    return out


@pytest.mark.parametrize("dims,B,padded", [((64, 256, 128, 64), 8192, True), ((64, 256, 128, 64), 1000, True),
                                           ((20, 136, 72, 8), 8191, True), ((20, 132, 72, 8), 777, False),
                                           ((24, 136, 64, 1), 8192, True), ((24, 136, 64, 1), 333, True)])
def test_mlp_bf16_backward_integer_exact(dims, B, padded):
    """Integer inputs, weights, biases and upstream gradients, small enough
    that every sum the forward and the backward form is an integer below
    2^23 in magnitude (checked on the oracle's sums of magnitudes): each
    fp32 sum is then exact in any order and each bf16 rounding sees the same
    value on both sides, so dW, db and dX equal the oracle's bit for bit.
    This pins the weight-gradient GEMM that reads delta and the activations
    k-major (transposing LDS reads; ragged batch tails at 1000, 8191 and 777
    rows; outputs of 72 and 8 columns) and the input-gradient GEMM that reads
    W k-major, or, with weight rows of 20 and 132 values (no 16-byte pitch),
    through a transposed copy; a last layer of one output takes the
    single-output kernels."""
    import deep_learning_recommendation_amd as D
    from deep_learning_recommendation_amd import pipeline as PL

    banner(f"mlp backward integer-exact dims={dims} B={B} padded={padded}")
    params = _int_params(dims, 5 + B, 0.25)
    g = np.random.default_rng(B)
    x = g.integers(-1, 2, size=(B, dims[0])).astype(np.float32)
    dY = g.integers(-1, 2, size=(B, dims[-1])).astype(np.float32)
    Ws = [p[0] for p in params]
    bs = [p[2] for p in params]
    # sums of magnitudes: the same network on |x|, |W|, |b| (forward) and on
    # |W|, |dY| (backward) bounds every partial sum
    _, _, acts_abs = oracle.mlp_fwd(np.abs(x), [np.abs(w) for w in Ws], [np.abs(b) for b in bs], False, True,
                                    save_acts=True)
    mW, mb, mX = oracle.mlp_bwd([np.abs(w) for w in Ws], acts_abs, np.abs(dY), True, want_dx=True)
    assert max(float(np.max(a)) for a in acts_abs[1:]) < 2.0 ** 23
    assert max(float(np.max(m)) for m in list(mW) + list(mb) + [mX]) < 2.0 ** 23

    if padded:
        mp = _mlp_dev(dims, params, True)
    else:  # weight rows of exactly fi values
        Wd = [torch.as_tensor(w).to(device=DEV, dtype=torch.bfloat16).contiguous() for w in Ws]
        mp = PL.MLPParams(tuple(dims), Wd, [int(w.shape[1]) for w in Ws],
                          [torch.as_tensor(b).to(DEV).contiguous() for b in bs], D.DLRM_BF16)
    out, _, ws = _fwd(mp, x, True, save=True)
    dY_dev = to_dev(dY)
    dWs = [torch.empty((o, i), dtype=torch.float32, device=DEV) for i, o in zip(dims[:-1], dims[1:])]
    dbs = [torch.empty((o,), dtype=torch.float32, device=DEV) for o in dims[1:]]
    dX = torch.empty((B, dims[0]), dtype=torch.float32, device=DEV)
    wsb = torch.empty((D.dlrm_mlp_bwd_workspace_size(B, dims),), dtype=torch.uint8, device=DEV)
    D.dlrm_mlp_bwd(B, dims, mp.Ws, mp.w_ld, D.DLRM_ACT_RELU, ws, out, dims[-1], dY_dev, dims[-1], dWs, dbs, dX,
                   dims[0], wsb)
    torch.cuda.synchronize()
    ref_out, _, acts = oracle.mlp_fwd(x, Ws, bs, True, True, save_acts=True)
    assert np.array_equal(out.cpu().numpy(), ref_out.astype(np.float32))
    rW, rb, rX = oracle.mlp_bwd(Ws, acts, dY, True, want_dx=True)
    for l in range(len(dims) - 1):
        assert np.array_equal(dWs[l].cpu().numpy(), rW[l].astype(np.float32)), l
        assert np.array_equal(dbs[l].cpu().numpy(), rb[l].astype(np.float32)), l
    assert np.array_equal(dX.cpu().numpy(), rX.astype(np.float32))


def _bf16_params(dims, seed):
    """Glorot-normal weights stored as bf16 (their fp32 values), U(+-1/sqrt(fan_in)) biases."""
    g = np.random.default_rng(seed)
    out = []
    for fi, fo in zip(dims[:-1], dims[1:]):
        Wf = (g.standard_normal((fo, fi)) * np.sqrt(2.0 / (fi + fo))).astype(np.float32)
        Wf = torch.from_numpy(Wf).to(torch.bfloat16).to(torch.float32).numpy()
        b = g.uniform(-1 / np.sqrt(fi), 1 / np.sqrt(fi), fo).astype(np.float32)
        out.append((Wf, None, b))
    return out


@pytest.mark.parametrize("K0,B,last_relu", [(13, 1000, True), (13, 128, False), (5, 257, True), (16, 3, True),
                                            (1, 131, True), (9, 1, False)])
def test_mlp_three_layer_bottom_shape(K0, B, last_relu):
    """Networks K0 -> 512 -> 256 -> 128 (the bottom-MLP shape, which runs as
    one fused kernel): ragged batches, narrow inputs, with and without the
    last ReLU; with saved activations the output is bit-identical and the
    backward from them matches the oracle."""
    import deep_learning_recommendation_amd as D

    dims = (K0, 512, 256, 128)
    banner(f"mlp three-layer bottom shape K0={K0} B={B} relu={last_relu}")
    params = _bf16_params(dims, 100 + K0 + B)
    x = np.random.default_rng(K0 * 7 + B).lognormal(0, 1, (B, K0)).astype(np.float32)
    mp = _mlp_dev(dims, params, True)
    out, _, _ = _fwd(mp, x, last_relu)
    ref, _, acts = oracle.mlp_fwd(x, [p[0] for p in params], [p[2] for p in params], True, last_relu, save_acts=True)
    got = out.cpu().numpy()
    err = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= 1e-2, err
    assert np.max(np.abs(got - ref)) <= 2e-2 * max(1.0, np.abs(ref).max())
    # saved activations: same output bits, and the backward reads them correctly
    out_s, _, ws = _fwd(mp, x, last_relu, save=True)
    assert torch.equal(out_s, out)
    dY = np.random.default_rng(5).standard_normal((B, 128)).astype(np.float32) * 0.1
    dW = [torch.empty((o, i), dtype=torch.float32, device=DEV) for i, o in zip(dims[:-1], dims[1:])]
    db = [torch.empty((o,), dtype=torch.float32, device=DEV) for o in dims[1:]]
    wsb = torch.empty((max(256, D.dlrm_mlp_bwd_workspace_size(B, dims)),), dtype=torch.uint8, device=DEV)
    D.dlrm_mlp_bwd(B, dims, mp.Ws, mp.w_ld, D.DLRM_ACT_RELU if last_relu else D.DLRM_ACT_NONE, ws, out_s, 128,
                   to_dev(dY), 128, dW, db, None, 0, wsb)
    torch.cuda.synchronize()
    rW, rb, _ = oracle.mlp_bwd([p[0] for p in params], acts, dY, last_relu)
    for l in range(3):
        g = dW[l].cpu().numpy()
        assert np.linalg.norm(g - rW[l]) <= 2e-2 * max(np.linalg.norm(rW[l]), 1e-30), l


def test_mlp_three_layer_bottom_shape_strided_output():
    """Output rows with a leading dimension that is not a multiple of 4
    (element stores) inside a wider buffer: the columns around the block
    stay untouched."""
    import deep_learning_recommendation_amd as D

    dims, B, ld = (13, 512, 256, 128), 300, 131
    banner("mlp three-layer bottom shape, strided output")
    params = _bf16_params(dims, 7)
    x = np.random.default_rng(8).lognormal(0, 1, (B, 13)).astype(np.float32)
    mp = _mlp_dev(dims, params, True)
    out = torch.full((B, ld), 7.0, dtype=torch.float32, device=DEV)
    ws = torch.empty((max(256, D.dlrm_mlp_workspace_size(B, dims, mp.w_dtype, False)),), dtype=torch.uint8,
                     device=DEV)
    D.dlrm_mlp_fwd(to_dev(x), 13, B, dims, mp.Ws, mp.w_ld, mp.biases, mp.w_dtype, D.DLRM_ACT_RELU, out, ld, None,
                   ws, False)
    torch.cuda.synchronize()
    ref, _, _ = oracle.mlp_fwd(x, [p[0] for p in params], [p[2] for p in params], True, True)
    got = out.cpu().numpy()
    assert np.all(got[:, 128:] == 7.0)
    assert np.linalg.norm(got[:, :128] - ref) <= 1e-2 * np.linalg.norm(ref)


@pytest.mark.parametrize("M,N,K,out_bf16,relu", [(32768, 1024, 1024, True, True), (32768, 512, 1024, True, True),
                                                 (32768, 256, 512, True, False), (1000, 1024, 479, True, True),
                                                 (257, 96, 40, False, True), (8192, 1024, 164, False, False),
                                                 (300, 1, 256, False, False), (4097, 33, 1000, True, True)])
def test_linear_fwd_against_oracle(M, N, K, out_bf16, relu):
    """One bf16 layer through dlrm_linear_fwd (the kernels every bf16 MLP
    layer runs): each output within the fp32 summation bound
    (K + 2) 2^-24 (sum_k |w x| + |b|) of the oracle's fp64 sum, plus one bf16
    rounding for bf16 outputs.  The top-MLP shapes run at the forward
    workload's batch."""
    import deep_learning_recommendation_amd as D

    banner(f"linear M={M} N={N} K={K} bf16_out={out_bf16} relu={relu}")
    g = np.random.default_rng(M + N + K)
    x = torch.from_numpy(g.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    Wt = torch.from_numpy((g.standard_normal((N, K)) * np.sqrt(2.0 / (K + N))).astype(np.float32)).to(torch.bfloat16)
    b = g.uniform(-1 / np.sqrt(K), 1 / np.sqrt(K), N).astype(np.float32)
    lda = ((K + 7) // 8) * 8
    xa = torch.zeros((M, lda), dtype=torch.bfloat16)
    xa[:, :K] = x
    wa = torch.zeros((N, lda), dtype=torch.bfloat16)
    wa[:, :K] = Wt
    C = torch.empty((M, N), dtype=torch.bfloat16 if out_bf16 else torch.float32, device=DEV)
    D.dlrm_linear_fwd(xa.to(DEV), lda, wa.to(DEV), lda, to_dev(b), C, N, M, N, K,
                      D.DLRM_ACT_RELU if relu else D.DLRM_ACT_NONE)
    torch.cuda.synchronize()
    got = C.float().cpu().numpy()
    # sampled rows for the large shapes (the oracle runs them in seconds)
    rows = np.arange(M) if M <= 4097 else np.sort(g.choice(M, 2048, replace=False))
    xf, wf = x.float().numpy()[rows], Wt.float().numpy()
    ref, _, _ = oracle.mlp_fwd(xf, [wf], [b], True, relu)
    mag, _, _ = oracle.mlp_fwd(np.abs(xf), [np.abs(wf)], [np.abs(b)], True, False)
    tol = (K + 2) * 2.0 ** -24 * mag.astype(np.float64)
    if out_bf16:
        tol = tol + 2.0 ** -8 * (np.abs(ref) + tol)
    err = np.abs(got[rows].astype(np.float64) - ref)
    assert np.all(err <= tol + 1e-30), float(np.max(err / (tol + 1e-30)))


@pytest.mark.parametrize("dims,B,save", [((64, 256, 1), 32768, False), ((40, 200, 1), 32769, True),
                                         ((64, 256, 1), 8192, False), ((64, 256, 1), 1000, True),
                                         ((40, 200, 1), 1000, False), ((40, 200, 1), 129, True),
                                         ((512, 256, 1), 333, False), ((96, 64, 1), 1, False),
                                         ((64, 256, 256, 1), 777, True), ((40, 100, 1), 513, True),
                                         ((136, 37, 1), 300, False)])
def test_mlp_hidden_and_logit_layer_integer_exact(dims, B, save):
    """A hidden layer of at most 256 outputs followed by the single-output
    layer runs as one launch (the logit summed in the GEMM's epilogue).  With
    integer inputs, weights and biases every sum is an exact integer, so the
    logit, the sigmoid input and (when saved) the hidden rows equal the
    oracle's bit for bit: 128-row tiles (batches of 32768 and more) and
    64-row tiles (smaller batches), ragged batches (1, 129, 333, 777, 1000,
    32769), hidden widths of 200, 100 and 64 inside the 256-wide tile (and
    37, whose rows have no 16-byte pitch), and k of 40, 96 and 136 (not a
    multiple of 64) besides 64, 256 and 512."""
    import deep_learning_recommendation_amd as D

    banner(f"mlp hidden+logit integer-exact dims={dims} B={B} save={save}")
    params = _int_params(dims, 31 + B, 0.25)
    g = np.random.default_rng(B + 3)
    x = g.integers(-2, 3, size=(B, dims[0])).astype(np.float32)
    Ws = [p[0] for p in params]
    bs = [p[2] for p in params]
    _, _, acts_abs = oracle.mlp_fwd(np.abs(x), [np.abs(w) for w in Ws], [np.abs(b) for b in bs], False, False,
                                    save_acts=True)
    # every partial sum an integer below 2^23 in magnitude (the same network
    # on |x|, |W|, |b| bounds them): exact in fp32 in any order, so both
    # sides round the same hidden values to bf16 and form the same logit
    assert max(float(np.max(a)) for a in acts_abs[1:]) < 2.0 ** 23
    ref_out, ref_p, acts = oracle.mlp_fwd(x, Ws, bs, True, False, save_acts=True)
    mp = _mlp_dev(dims, params, True)
    out, prob, ws = _fwd(mp, x, False, save=save)
    assert np.array_equal(out.cpu().numpy(), ref_out.astype(np.float32))
    assert np.max(np.abs(prob.cpu().numpy() - ref_p)) <= 1e-6
    if save:
        # the hidden rows the backward pass reads: the last hidden layer's
        # bf16 output in the forward workspace, as the backward locates it
        dWs = [torch.empty((o, i), dtype=torch.float32, device=DEV) for i, o in zip(dims[:-1], dims[1:])]
        dbs = [torch.empty((o,), dtype=torch.float32, device=DEV) for o in dims[1:]]
        ones = torch.ones((B, 1), dtype=torch.float32, device=DEV)
        wsb = torch.empty((D.dlrm_mlp_bwd_workspace_size(B, dims),), dtype=torch.uint8, device=DEV)
        D.dlrm_mlp_bwd(B, dims, mp.Ws, mp.w_ld, D.DLRM_ACT_NONE, ws, out, 1, ones, 1, dWs, dbs, None, 0, wsb)
        torch.cuda.synchronize()
        # dW of the logit layer with dY = 1 is the column sum of its input rows
        ref_dw = acts[-2].astype(np.float64).sum(axis=0)
        assert np.array_equal(dWs[-1].cpu().numpy()[0], ref_dw.astype(np.float32))
