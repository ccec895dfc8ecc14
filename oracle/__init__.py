"""CPU oracle for the DLRM hot path -- TEST INFRASTRUCTURE ONLY.

ctypes wrapper around ``dlrm_oracle.c`` (plain C, fp64 except where the
bit-exact contract fixes fp32 bag-order sums).  Only ``tests/``, the smoke
check and the benchmark's CPU-baseline leg may import this package; the GPU
library and its Python binding never do, and share no code with it.

All arrays are numpy, C-contiguous; tables are lists of float32 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "dlrm_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11", "-shared", "-fPIC"]

_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def build(out: str = LIB_PATH, extra: list | None = None) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", *CFLAGS, *(extra or []), SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def lib(path: str | None = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _bind(L):
    L.oracle_num_threads.restype = ctypes.c_int
    L.oracle_set_threads.argtypes = [ctypes.c_int]
    L.oracle_bf16_round.argtypes = [_P, _P, _I64]
    L.oracle_embbag_fwd.argtypes = [_P, _I32, _I32, _P, _P, _I64, _P, _I64, _I64]
    L.oracle_embbag_fwd_lp.argtypes = [_P, _I32, _P, _I32, _I32, _P, _P, _I64, _P, _I64, _I64]
    L.oracle_interact_fwd.argtypes = [_P, _I64, _I32, _I32, _I64, _P, _I64]
    L.oracle_interact_bwd.argtypes = [_P, _I64, _I32, _I32, _I64, _P, _I64, _P, _I64]
    L.oracle_mlp_fwd.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _I32, _I32, _P, _I64, _P, _P]
    L.oracle_mlp_bwd.argtypes = [_I64, _I32, _P, _P, _P, _I32, _P, _P, _P, _P]
    L.oracle_embbag_bwd_sgd.argtypes = [_P, _P, _I32, _I32, _P, _P, _I64, _P, _I64, _I64, ctypes.c_float]
    return L


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _ptr_array(arrs):
    t = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    return t


def _c(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype or not a.flags.c_contiguous:
        a = np.ascontiguousarray(a, dtype=dtype)
    return a


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def bf16_round(x, L=None) -> np.ndarray:
    L = L or lib()
    x = _c(x, np.float32)
    out = np.empty_like(x)
    L.oracle_bf16_round(_ptr(x), _ptr(out), x.size)
    return out


def embbag_fwd(tables, idx, offsets, B: int, out=None, out_ld=None, out_col0: int = 0, L=None) -> np.ndarray:
    """Sum-pooled bags; returns out (default [B][K*d])."""
    L = L or lib()
    tables = [_c(t, np.float32) for t in tables]
    K, d = len(tables), tables[0].shape[1]
    idx, offsets = _c(idx, np.int64), _c(offsets, np.int64)
    assert offsets.shape[0] == K * B + 1
    if out is None:
        out_ld = K * d if out_ld is None else out_ld
        out = np.zeros((B, out_ld), dtype=np.float32)
    out_ld = out.shape[1] if out_ld is None else out_ld
    ptrs = _ptr_array(tables)
    L.oracle_embbag_fwd(ptrs, K, d, _ptr(idx), _ptr(offsets), B, _ptr(out), out_ld, out_col0)
    return out


def embbag_fwd_lp(tables, dtype: str, idx, offsets, B: int, scale_bias=None, out=None, out_ld=None, out_col0: int = 0,
                  L=None) -> np.ndarray:
    """Sum-pooled bags from low-precision rows: dtype "bf16" (tables are
    uint16 arrays of bf16 bit patterns) or "int8" (int8 tables with
    ``scale_bias[k]`` float32 [m_k][2] = per-row scale and bias)."""
    L = L or lib()
    code = {"bf16": 1, "int8": 2}[dtype]
    tables = [_c(t, np.uint16 if code == 1 else np.int8) for t in tables]
    K, d = len(tables), tables[0].shape[1]
    idx, offsets = _c(idx, np.int64), _c(offsets, np.int64)
    assert offsets.shape[0] == K * B + 1
    sbp = None
    if code == 2:
        scale_bias = [_c(a, np.float32) for a in scale_bias]
        assert all(a.shape == (t.shape[0], 2) for a, t in zip(scale_bias, tables))
        sbp = _ptr_array(scale_bias)
    if out is None:
        out_ld = K * d if out_ld is None else out_ld
        out = np.zeros((B, out_ld), dtype=np.float32)
    out_ld = out.shape[1] if out_ld is None else out_ld
    L.oracle_embbag_fwd_lp(_ptr_array(tables), code, sbp, K, d, _ptr(idx), _ptr(offsets), B, _ptr(out), out_ld,
                           out_col0)
    return out


def interact_fwd(X, L=None) -> np.ndarray:
    """X [B][n][d] -> [B][d + n(n-1)/2]."""
    L = L or lib()
    X = _c(X, np.float32)
    B, n, d = X.shape
    out = np.zeros((B, d + n * (n - 1) // 2), dtype=np.float32)
    L.oracle_interact_fwd(_ptr(X), B, n, d, n * d, _ptr(out), out.shape[1])
    return out


def interact_bwd(X, g, L=None) -> np.ndarray:
    """X [B][n][d], g [B][d + n(n-1)/2] (gradient of the top-MLP input row)
    -> dX [B][n][d]."""
    L = L or lib()
    X = _c(X, np.float32)
    B, n, d = X.shape
    g = _c(g, np.float32).reshape(B, -1)
    assert g.shape[1] >= d + n * (n - 1) // 2
    dX = np.zeros((B, n, d), dtype=np.float32)
    L.oracle_interact_bwd(_ptr(X), B, n, d, n * d, _ptr(g), g.shape[1], _ptr(dX), n * d)
    return dX


def mlp_fwd(x, Ws, bs, quant_bf16: bool, last_relu: bool, save_acts: bool = False, L=None):
    """Returns (out [B][dims[L]], prob or None, acts or None)."""
    L = L or lib()
    x = _c(x, np.float32)
    B = x.shape[0]
    Ws = [_c(w, np.float32) for w in Ws]
    bs = [_c(b, np.float32) for b in bs]
    dims = np.array([Ws[0].shape[1]] + [w.shape[0] for w in Ws], dtype=np.int32)
    nl = len(Ws)
    out = np.zeros((B, dims[-1]), dtype=np.float32)
    prob = np.zeros(B, dtype=np.float32) if dims[-1] == 1 else None
    acts = [np.zeros((B, int(dims[l])), dtype=np.float32) for l in range(nl + 1)] if save_acts else None
    L.oracle_mlp_fwd(_ptr(x), x.shape[1], B, nl, _ptr(dims), _ptr_array(Ws), _ptr_array(bs), int(quant_bf16),
                     int(last_relu), _ptr(out), out.shape[1], _ptr(prob) if prob is not None else None,
                     _ptr_array(acts) if acts is not None else None)
    return out, prob, acts


def mlp_bwd(Ws, acts, dY, last_relu: bool, want_dx: bool = False, L=None):
    """Returns (dWs, dbs, dX or None)."""
    L = L or lib()
    Ws = [_c(w, np.float32) for w in Ws]
    acts = [_c(a, np.float32) for a in acts]
    dY = _c(dY, np.float32)
    B = dY.shape[0]
    dims = np.array([Ws[0].shape[1]] + [w.shape[0] for w in Ws], dtype=np.int32)
    dWs = [np.zeros_like(w) for w in Ws]
    dbs = [np.zeros(w.shape[0], dtype=np.float32) for w in Ws]
    dX = np.zeros((B, int(dims[0])), dtype=np.float32) if want_dx else None
    L.oracle_mlp_bwd(B, len(Ws), _ptr(dims), _ptr_array(Ws), _ptr_array(acts), int(last_relu), _ptr(dY),
                     _ptr_array(dWs), _ptr_array(dbs), _ptr(dX) if dX is not None else None)
    return dWs, dbs, dX


def embbag_bwd_sgd(tables, idx, offsets, B: int, G, g_col0: int, lr: float, L=None):
    """Updates ``tables`` (list of float32 arrays) in place; G is [B][g_ld]."""
    L = L or lib()
    for t in tables:
        assert t.dtype == np.float32 and t.flags.c_contiguous
    K, d = len(tables), tables[0].shape[1]
    rows = np.array([t.shape[0] for t in tables], dtype=np.int64)
    idx, offsets = _c(idx, np.int64), _c(offsets, np.int64)
    G = _c(G, np.float32).reshape(B, -1)
    assert 0 <= g_col0 and g_col0 + K * d <= G.shape[1], "G has no room for K blocks of d columns at g_col0"
    L.oracle_embbag_bwd_sgd(_ptr_array(tables), _ptr(rows), K, d, _ptr(idx), _ptr(offsets), B, _ptr(G),
                            G.shape[1], g_col0, ctypes.c_float(lr))
    return tables
