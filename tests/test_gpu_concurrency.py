"""The library keeps no per-call state: calls on two streams at once, with
disjoint outputs and workspaces, give the results each gives alone (pooled
rows and updated table rows bit for bit against the oracle, MLP outputs bit
for bit against the same call made alone)."""
import numpy as np
import pytest
import torch

import oracle
from dlrm_cases import DEV, banner, bits, to_dev

pytestmark = pytest.mark.gpu


def _bags(g, K, B, rows, max_len, hot):
    lens = g.integers(0, max_len + 1, size=K * B)
    off = np.zeros(K * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    idx = []
    for k in range(K):
        n = off[(k + 1) * B] - off[k * B]
        r = np.where(g.random(n) < 0.5, g.integers(0, 2, n), g.integers(0, rows[k], n)) if hot else \
            g.integers(0, rows[k], n)
        idx.append(r)
    return np.concatenate(idx).astype(np.int64), off


def test_embbag_and_sparse_update_on_two_streams():
    """Two independent lookups and two independent sparse updates (separate
    tables, gradients and workspaces), each pair launched alternately on two
    streams with no synchronisation between them."""
    import deep_learning_recommendation_amd as D

    banner("two streams: lookup and sparse update")
    K, B, d = 3, 1500, 64
    rows = [400, 2000, 37]
    cases = []
    for s in range(2):
        g = np.random.default_rng(100 + s)
        idx, off = _bags(g, K, B, rows, 40, hot=(s == 1))
        tabs = [g.standard_normal((rows[k], d)).astype(np.float32) for k in range(K)]
        G = (g.standard_normal((B, K * d)) * 0.01).astype(np.float32)
        cases.append((idx, off, tabs, G))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    dev = []
    for idx, off, tabs, G in cases:
        tdev = [to_dev(t) for t in tabs]
        nnz = int(off[-1])
        dev.append(dict(tabs=tdev, ptrs=D.device_pointer_array(tdev), idx=to_dev(idx), off=to_dev(off), G=to_dev(G),
                        nnz=nnz, out=torch.full((B, K * d), float("nan"), dtype=torch.float32, device=DEV),
                        ws=torch.empty((D.dlrm_embbag_bwd_sgd_workspace_size(K, B, nnz, d),), dtype=torch.uint8,
                                       device=DEV)))
    torch.cuda.synchronize()
    for c, st in zip(dev, streams):
        D.dlrm_embbag_fwd(c["ptrs"], K, d, c["idx"], c["off"], B, c["out"], K * d, 0, stream=st, nnz=c["nnz"])
    for c, st in zip(dev, streams):
        D.dlrm_embbag_bwd_sgd(c["ptrs"], K, d, rows, c["idx"], c["off"], B, c["nnz"], c["G"], K * d, 0, 0.01,
                              c["ws"], stream=st)
    torch.cuda.synchronize()
    for (idx, off, tabs, G), c in zip(cases, dev):
        ref = oracle.embbag_fwd(tabs, idx, off, B)
        assert np.array_equal(bits(c["out"].cpu().numpy()), bits(ref))
        upd = [t.copy() for t in tabs]
        oracle.embbag_bwd_sgd(upd, idx, off, B, G, 0, 0.01)
        for k in range(K):
            assert np.array_equal(bits(c["tabs"][k].cpu().numpy()), bits(upd[k])), k


def test_mlp_forward_on_two_streams_equals_alone():
    """The same bf16 network on two batches at once (separate workspaces and
    outputs), repeated back to back on two streams: every output equals the
    output of the call made alone."""
    import deep_learning_recommendation_amd as D
    from deep_learning_recommendation_amd import pipeline as PL

    banner("two streams: MLP forward")
    dims = (128, 512, 256, 1)
    g = np.random.default_rng(7)
    Ws = [(g.standard_normal((o, i)) * np.sqrt(2.0 / i)).astype(np.float32) for i, o in zip(dims[:-1], dims[1:])]
    bs = [(g.standard_normal(o) * 0.1).astype(np.float32) for o in dims[1:]]
    mp = PL.make_mlp(dims, Ws, bs, True)
    B = 5000
    xs = [torch.as_tensor((g.standard_normal((B, dims[0])) * 0.5).astype(np.float32)).to(torch.bfloat16).to(DEV)
          for _ in range(2)]

    def run(x, stream, ws, out, prob):
        D.dlrm_mlp_fwd(x, dims[0], B, mp.dims, mp.Ws, mp.w_ld, mp.biases, mp.w_dtype, D.DLRM_ACT_NONE, out, 1, prob,
                       ws, False, stream)

    wsz = max(256, D.dlrm_mlp_workspace_size(B, dims, mp.w_dtype, False))
    alone = []
    for x in xs:
        ws = torch.empty((wsz,), dtype=torch.uint8, device=DEV)
        out = torch.empty((B, 1), dtype=torch.float32, device=DEV)
        prob = torch.empty((B,), dtype=torch.float32, device=DEV)
        run(x, torch.cuda.current_stream(), ws, out, prob)
        torch.cuda.synchronize()
        alone.append((out.clone(), prob.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [(torch.empty((wsz,), dtype=torch.uint8, device=DEV), torch.empty((B, 1), dtype=torch.float32, device=DEV),
             torch.empty((B,), dtype=torch.float32, device=DEV)) for _ in range(2)]
    torch.cuda.synchronize()
    for _ in range(4):
        for x, st, (ws, out, prob) in zip(xs, streams, bufs):
            run(x, st, ws, out, prob)
    torch.cuda.synchronize()
    for (a_out, a_prob), (_, out, prob) in zip(alone, bufs):
        assert torch.equal(out.view(torch.int32), a_out.view(torch.int32))
        assert torch.equal(prob.view(torch.int32), a_prob.view(torch.int32))
