"""Fill device-resident synthetic embedding tables (``libsynth.so``).

The tables of the large workloads (up to 205 GB) never exist on the host: the
GPU generates them in place from the same counter-based formula that
``synth.rng.table_rows`` evaluates on the host for the rows a test touches.
"""
from __future__ import annotations

import ctypes
import os

from . import rng as R

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        _lib = ctypes.CDLL(LIB_PATH)
        _lib.synth_fill_table.restype = ctypes.c_int
        _lib.synth_fill_table.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64,
                                          ctypes.c_float, ctypes.c_void_p]
        _lib.synth_fill_table_bf16.restype = ctypes.c_int
        _lib.synth_fill_table_bf16.argtypes = _lib.synth_fill_table.argtypes
        _lib.synth_fill_table_i8.restype = ctypes.c_int
        _lib.synth_fill_table_i8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p]
    return _lib


def fill_table(t, seed: int, table: int, stream=None) -> None:
    """Fill the contiguous fp32 CUDA tensor ``t`` ([rows][d]) in place."""
    import torch

    assert t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and t.dim() == 2
    rows, d = t.shape
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = lib().synth_fill_table(ctypes.c_void_p(t.data_ptr()), rows, d, R.table_key(seed, table),
                                float(R.table_scale(rows)), ctypes.c_void_p(s))
    if rc != 0:
        raise RuntimeError(f"synth_fill_table failed with code {rc}")


def make_tables(w, device="cuda", seed: int | None = None):
    """Allocate and fill the K tables of workload ``w`` on the device."""
    import torch

    seed = w.seed if seed is None else seed
    out = []
    for k in range(w.K):
        t = torch.empty((w.rows[k], w.d), dtype=torch.float32, device=device)
        fill_table(t, seed, k)
        out.append(t)
    return out


def make_tables_lp(w, dtype: str, device="cuda", seed: int | None = None):
    """Low-precision tables of workload ``w``: ``dtype`` "bf16" gives K
    int16 tensors of bf16 bit patterns (``synth.rng.table_rows_bf16``) and
    ``None``; "int8" gives K int8 tensors and K float32 [m_k][2] (scale,
    bias) tensors (``synth.rng.table_rows_i8``)."""
    import torch

    seed = w.seed if seed is None else seed
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    tabs, sbs = [], []
    for k in range(w.K):
        rows, a = w.rows[k], float(R.table_scale(w.rows[k]))
        if dtype == "bf16":
            t = torch.empty((rows, w.d), dtype=torch.int16, device=device)
            rc = lib().synth_fill_table_bf16(ctypes.c_void_p(t.data_ptr()), rows, w.d, R.table_key(seed, k), a, s)
        else:
            t = torch.empty((rows, w.d), dtype=torch.int8, device=device)
            sb = torch.empty((rows, 2), dtype=torch.float32, device=device)
            rc = lib().synth_fill_table_i8(ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(sb.data_ptr()), rows, w.d,
                                           R.table_key(seed, k), R.scale_bias_key(seed, k), a, s)
            sbs.append(sb)
        if rc != 0:
            raise RuntimeError(f"synth fill ({dtype}) failed with code {rc}")
        tabs.append(t)
    return tabs, (sbs if dtype == "int8" else None)
