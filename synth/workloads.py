"""The five synthetic DLRM workloads and their seeded input recipes.

Shapes follow the model the pages describe (per-feature tables m_k x d, one
shared d, a bottom MLP that outputs d, the n(n-1)/2 pairwise interaction and a
top MLP ending in a sigmoid).  Sizes and distributions are those of the five
benchmark workloads:

* ``tiny``        batch 128, 8 tables 1000 x 16, one uniform index per bag, fp32 MLPs
* ``embbag``      26 tables 1M x 128, batch 65536, bag length 1+Poisson(19),
                  Zipf(1.05) ranks through a seeded permutation
* ``forward``     batch 32768, 26 tables of log-uniform cardinality in [100, 4e7]
                  (about 2e8 rows), one Zipf(1.1) index per bag, bf16 MLPs
* ``interaction`` batch 16384, 100 tables 1e5 x 64, 4 uniform indices per bag
* ``train``       batch 8192, 8 tables 5e7 x 128, 100 Zipf(1.2) indices per bag,
                  upstream gradient N(0, 0.01), SGD lr 0.01

No step of the model is computed here.  Every array is seeded; the GPU path
and the CPU oracle receive identical values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import rng as R

# stream ids (one independent random stream per tensor kind)
S_DENSE, S_LABELS, S_LENGTHS, S_INDICES, S_PERM, S_W, S_B, S_GRAD, S_CARD = range(1, 10)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    K: int
    d: int
    rows: tuple
    bag: str            # "fixed" (every bag has bag_len indices) | "poisson" (1 + Poisson(bag_len - 1))
    bag_len: int
    index_dist: str     # "uniform" | "zipf"
    alpha: float
    dense_dim: int
    dense_dist: str     # "normal" | "lognormal"
    bottom: tuple       # layer widths, input first
    top: tuple          # layer widths, input first
    mlp_dtype: str      # "f32" | "bf16"
    train: bool = False
    lr: float = 0.01
    notes: str = field(default="", compare=False)

    @property
    def n(self) -> int:
        return self.K + 1

    @property
    def pairs(self) -> int:
        return self.n * (self.n - 1) // 2

    @property
    def top_in(self) -> int:
        return self.d + self.pairs

    def scaled(self, B: int | None = None, rows: int | None = None, K: int | None = None) -> "Workload":
        """Same recipe at a smaller batch / table count / cardinality (tests)."""
        import dataclasses
        K2 = self.K if K is None else K
        rows2 = self.rows[:K2] if rows is None else tuple([rows] * K2)
        top = self.top
        if K2 != self.K and top:
            n2 = K2 + 1
            top = (self.d + n2 * (n2 - 1) // 2,) + tuple(top[1:])
        return dataclasses.replace(self, B=self.B if B is None else B, K=K2, rows=rows2, top=top)


def forward_cardinalities(seed: int = 3, lo: float = 100.0, hi: float = 4e7, K: int = 26,
                          total_lo: float = 1.8e8, total_hi: float = 2.2e8) -> tuple:
    """26 log-uniform cardinalities in [lo, hi] whose total is about 2e8 rows.

    Independent log-uniform draws average about 8e7 rows in total, so the
    recipe takes the first sub-seed s = 0, 1, ... whose draws sum into
    [1.8e8, 2.2e8].
    """
    for s in range(100000):
        g = R.stream_rng(seed, S_CARD, s)
        m = np.floor(np.exp(g.uniform(math.log(lo), math.log(hi), size=K))).astype(np.int64)
        if total_lo <= m.sum() <= total_hi:
            return tuple(int(x) for x in m)
    raise RuntimeError("no cardinality seed found")


def _build() -> dict:
    w = {}
    w["tiny"] = Workload("tiny", 1, B=128, K=8, d=16, rows=(1000,) * 8, bag="fixed", bag_len=1,
                         index_dist="uniform", alpha=0.0, dense_dim=13, dense_dist="normal",
                         bottom=(13, 64, 16), top=(52, 64, 1), mlp_dtype="f32")
    w["embbag"] = Workload("embbag", 2, B=65536, K=26, d=128, rows=(1_000_000,) * 26, bag="poisson",
                           bag_len=20, index_dist="zipf", alpha=1.05, dense_dim=0, dense_dist="normal",
                           bottom=(), top=(), mlp_dtype="f32")
    w["forward"] = Workload("forward", 3, B=32768, K=26, d=128, rows=forward_cardinalities(), bag="fixed",
                            bag_len=1, index_dist="zipf", alpha=1.1, dense_dim=13, dense_dist="lognormal",
                            bottom=(13, 512, 256, 128), top=(479, 1024, 1024, 512, 256, 1), mlp_dtype="bf16")
    w["interaction"] = Workload("interaction", 4, B=16384, K=100, d=64, rows=(100_000,) * 100, bag="fixed",
                                bag_len=4, index_dist="uniform", alpha=0.0, dense_dim=32, dense_dist="normal",
                                bottom=(32, 256, 64), top=(5114, 512, 1), mlp_dtype="bf16")
    w["train"] = Workload("train", 5, B=8192, K=8, d=128, rows=(50_000_000,) * 8, bag="fixed", bag_len=100,
                          index_dist="zipf", alpha=1.2, dense_dim=13, dense_dist="lognormal",
                          bottom=(13, 512, 256, 128), top=(164, 1024, 1024, 512, 256, 1), mlp_dtype="bf16",
                          train=True, lr=0.01)
    return w


_WORKLOADS = None


def workloads() -> dict:
    global _WORKLOADS
    if _WORKLOADS is None:
        _WORKLOADS = _build()
    return _WORKLOADS


def get(name: str) -> Workload:
    return workloads()[name]


# ----------------------------------------------------------------------------- inputs

def dense(w: Workload, batch: int = 0) -> np.ndarray:
    g = R.stream_rng(w.seed, S_DENSE, batch)
    if w.dense_dist == "lognormal":
        x = g.lognormal(0.0, 1.0, size=(w.B, w.dense_dim))
    else:
        x = g.standard_normal(size=(w.B, w.dense_dim))
    return x.astype(np.float32)


def labels(w: Workload, batch: int = 0) -> np.ndarray:
    g = R.stream_rng(w.seed, S_LABELS, batch)
    return (g.random(w.B) < 0.5).astype(np.float32)


def bag_lengths(w: Workload, k: int, batch: int = 0) -> np.ndarray:
    if w.bag == "fixed":
        return np.full(w.B, w.bag_len, dtype=np.int64)
    g = R.stream_rng(w.seed, S_LENGTHS, batch, k)
    return 1 + g.poisson(w.bag_len - 1, size=w.B).astype(np.int64)


def permutation(w: Workload, k: int) -> R.FeistelPermutation:
    return R.FeistelPermutation(w.rows[k], R.fmix_int(w.seed * 1000003 + S_PERM * 7919 + k))


def table_indices(w: Workload, k: int, count: int, batch: int = 0) -> np.ndarray:
    g = R.stream_rng(w.seed, S_INDICES, batch, k)
    m = w.rows[k]
    if w.index_dist == "zipf":
        return permutation(w, k)(R.zipf_ranks(g, m, w.alpha, count))
    return g.integers(0, m, size=count, dtype=np.int64)


def indices_offsets(w: Workload, batch: int = 0):
    """int64 indices [nnz] and CSR offsets [K*B + 1], table-major: bag (k, b)
    owns indices[offsets[k*B + b] : offsets[k*B + b + 1]]."""
    lengths = np.concatenate([bag_lengths(w, k, batch) for k in range(w.K)])
    offsets = np.zeros(w.K * w.B + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    idx = np.empty(int(offsets[-1]), dtype=np.int64)
    for k in range(w.K):
        a, b = int(offsets[k * w.B]), int(offsets[(k + 1) * w.B])
        idx[a:b] = table_indices(w, k, b - a, batch)
    return idx, offsets


def mlp_params(w: Workload, which: str):
    """Weights and biases of the bottom ("bottom") or top ("top") MLP.

    W_l ~ N(0, 2/(fan_in + fan_out)) (Glorot normal) as [out][in] row-major;
    b_l ~ U(-1/sqrt(fan_in), +1/sqrt(fan_in)).  Glorot scaling keeps the
    logits of log-normal dense inputs O(1); see the rounding-sensitivity note
    in the design document.
    For bf16 MLPs the weights are drawn in fp32 and stored as bf16 (round to
    nearest even, by torch); ``W`` then holds the fp32 values of those bf16
    numbers and ``W_bits`` their uint16 encodings.
    """
    import torch

    dims = w.bottom if which == "bottom" else w.top
    sid = 0 if which == "bottom" else 1
    out = []
    for l in range(len(dims) - 1):
        fi, fo = dims[l], dims[l + 1]
        g = R.stream_rng(w.seed, S_W, sid, l)
        W = (g.standard_normal(size=(fo, fi)) * math.sqrt(2.0 / (fi + fo))).astype(np.float32)
        gb = R.stream_rng(w.seed, S_B, sid, l)
        b = gb.uniform(-1.0 / math.sqrt(fi), 1.0 / math.sqrt(fi), size=fo).astype(np.float32)
        bits = None
        if w.mlp_dtype == "bf16":
            tb = torch.from_numpy(W).to(torch.bfloat16)
            bits = tb.view(torch.int16).numpy().view(np.uint16).copy()
            W = tb.to(torch.float32).numpy()
        out.append((W, bits, b))
    return out


def upstream_grad(w: Workload, batch: int = 0) -> np.ndarray:
    """Synthetic gradient of the loss w.r.t. X, shape [B][K+1][d], N(0, sigma=0.01)."""
    g = R.stream_rng(w.seed, S_GRAD, batch)
    return (g.standard_normal(size=(w.B, w.n, w.d)) * 0.01).astype(np.float32)


def compact_rows(w: Workload, idx: np.ndarray, offsets: np.ndarray, seed_tables: int | None = None):
    """Rows each table's bags touch, regenerated on the host.

    Returns (tables, local_idx, row_ids): ``tables[k]`` holds the touched rows
    of table k in ascending row order, ``row_ids[k]`` their row numbers, and
    ``local_idx`` is ``idx`` rewritten to positions in ``tables[k]``.
    """
    seed = w.seed if seed_tables is None else seed_tables
    tables, row_ids = [], []
    local = np.empty_like(idx)
    for k in range(w.K):
        a, b = int(offsets[k * w.B]), int(offsets[(k + 1) * w.B])
        u, inv = np.unique(idx[a:b], return_inverse=True)
        local[a:b] = inv
        row_ids.append(u)
        tables.append(R.table_rows(seed, k, w.rows[k], u, w.d))
    return tables, local, row_ids


def sub_bags(idx: np.ndarray, offsets: np.ndarray, K: int, B: int, samples) -> tuple:
    """Indices and offsets of the listed samples' bags only (same order)."""
    samples = np.asarray(samples)
    S = len(samples)
    lens = np.empty(K * S, dtype=np.int64)
    parts = []
    for k in range(K):
        a = offsets[k * B + samples]
        e = offsets[k * B + samples + 1]
        lens[k * S:(k + 1) * S] = e - a
        parts.extend(idx[x:y] for x, y in zip(a, e))
    new_off = np.zeros(K * S + 1, dtype=np.int64)
    np.cumsum(lens, out=new_off[1:])
    new_idx = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    return new_idx, new_off
