"""ctypes binding of libdlrm.so: same entry points, argument marshalling only.

Tensors are torch CUDA tensors (torch supplies device memory and streams);
every computation runs in the library's HIP kernels.  A non-zero status
raises :class:`DLRMError`.  If the library is not built the import of any
entry point raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdlrm.so")

DLRM_OK, DLRM_E_INVALID, DLRM_E_WORKSPACE, DLRM_E_HIP, DLRM_E_UNSUPPORTED = 0, -1, -2, -3, -4
DLRM_F32, DLRM_BF16, DLRM_I8 = 0, 1, 2
DLRM_ACT_NONE, DLRM_ACT_RELU = 0, 1

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "dlrm_abi_version": (ctypes.c_int, []),
    "dlrm_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "dlrm_last_hip_error": (ctypes.c_int, []),
    "dlrm_embbag_fwd": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _I64, _I64, _P, _I64, _I64, _P]),
    "dlrm_embbag_fwd_lp": (ctypes.c_int, [_P, _I32, _P, _I32, _I32, _P, _P, _I64, _I64, _P, _I64, _I64, _P]),
    "dlrm_embbag_interact_fwd_lp": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _I32, _I32, _P, _P, _I64, _P, _I32, _I64,
                                                   _P]),
    "dlrm_interact_fwd": (ctypes.c_int, [_P, _I64, _I32, _I32, _I64, _P, _I32, _I64, _P]),
    "dlrm_embbag_interact_fwd": (ctypes.c_int, [_P, _I64, _P, _I32, _I32, _P, _P, _I64, _P, _I32, _I64, _P]),
    "dlrm_interact_bwd": (ctypes.c_int, [_P, _I64, _I32, _I32, _I64, _P, _I64, _P, _I64, _P]),
    "dlrm_mlp_workspace_size": (_SZ, [_I64, _I32, _P, _I32, _I32]),
    "dlrm_mlp_fwd": (ctypes.c_int, [_P, _I32, _I64, _I64, _I32, _P, _P, _P, _P, _I32, _I32, _P, _I64, _P, _P, _SZ,
                                    _I32, _P]),
    "dlrm_linear_fwd": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _I32, _I64, _I64, _I32, _I32, _I32, _P]),
    "dlrm_mlp_bwd_workspace_size": (_SZ, [_I64, _I32, _P]),
    "dlrm_mlp_bwd": (ctypes.c_int, [_I64, _I32, _P, _P, _P, _I32, _P, _P, _I64, _P, _I64, _P, _P, _P, _I64, _P, _SZ,
                                    _P]),
    "dlrm_bce_grad": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P]),
    "dlrm_embbag_bwd_sgd_workspace_size": (_SZ, [_I32, _I64, _I64, _I32]),
    "dlrm_embbag_bwd_sgd": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _I64, _I64, _P, _I64, _I64, ctypes.c_float,
                                           _P, _SZ, _P]),
    "dlrm_embbag_bwd_sgd_prepare": (ctypes.c_int, [_I32, _P, _P, _P, _I64, _I64, _P, _SZ, _P]),
    "dlrm_embbag_bwd_sgd_apply": (ctypes.c_int, [_P, _I32, _I32, _P, _I64, _I64, _P, _I64, _I64, ctypes.c_float, _P,
                                                 _SZ, _P, _P]),
    "dlrm_embbag_bwd_sgd_noalloc": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _I64, _I64, _P, _I64, _I64,
                                                   ctypes.c_float, _P]),
    "dlrm_check_indices": (ctypes.c_int, [_P, _P, _I32, _I64, _P, _P, _P]),
}

EXPORTS = tuple(_SIGNATURES)

_lib = None


class DLRMError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _load().dlrm_strerror(status).decode()
        if status == DLRM_E_HIP:
            msg += f" (hipError {_load().dlrm_last_hip_error()})"
        super().__init__(f"{fn}: status {status}: {msg}")


def _load(path: str | None = None):
    global _lib
    if _lib is None or path is not None:
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is not built; run __graft_entry__.build() (no CPU fallback exists)")
        lib = ctypes.CDLL(p)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        if path is not None:
            return lib
        _lib = lib
    return _lib


def lib():
    return _load()


def _check(fn: str, status: int) -> None:
    if status != DLRM_OK:
        raise DLRMError(fn, status)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _host_i32(vals):
    return (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])


def _host_ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def device_pointer_array(tensors):
    """Device int64 array of the tensors' device addresses (for `tables`)."""
    import torch

    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=tensors[0].device)


def _dtype_code(t) -> int:
    import torch

    return DLRM_BF16 if t.dtype == torch.bfloat16 else DLRM_F32


def dlrm_abi_version() -> int:
    return int(lib().dlrm_abi_version())


def dlrm_embbag_fwd(table_ptrs, K: int, d: int, indices, offsets, B: int, out, out_ld: int, out_col0: int = 0,
                    stream=None, nnz: int = -1) -> None:
    """nnz: offsets[K*B] when known on the host (sizes the work split), else -1."""
    _check("dlrm_embbag_fwd", lib().dlrm_embbag_fwd(_ptr(table_ptrs), K, d, _ptr(indices), _ptr(offsets), B, nnz,
                                                     _ptr(out), out_ld, out_col0, _stream(stream)))


def dlrm_embbag_fwd_lp(table_ptrs, table_dtype: int, scale_bias_ptrs, K: int, d: int, indices, offsets, B: int, out,
                       out_ld: int, out_col0: int = 0, stream=None, nnz: int = -1) -> None:
    """Low-precision table rows: table_dtype DLRM_BF16, or DLRM_I8 with
    scale_bias_ptrs (K device pointers to fp32 [m_k][2]); None for bf16."""
    sb = _ptr(scale_bias_ptrs) if scale_bias_ptrs is not None else None
    _check("dlrm_embbag_fwd_lp", lib().dlrm_embbag_fwd_lp(_ptr(table_ptrs), table_dtype, sb, K, d, _ptr(indices),
                                                           _ptr(offsets), B, nnz, _ptr(out), out_ld, out_col0,
                                                           _stream(stream)))


def dlrm_interact_fwd(X, B: int, n: int, d: int, x_ld: int, out, out_ld: int, stream=None) -> None:
    _check("dlrm_interact_fwd", lib().dlrm_interact_fwd(_ptr(X), B, n, d, x_ld, _ptr(out), _dtype_code(out), out_ld,
                                                         _stream(stream)))


def dlrm_embbag_interact_fwd(x_dense, xd_ld: int, table_ptrs, K: int, d: int, indices, offsets, B: int, out,
                             out_ld: int, stream=None) -> None:
    _check("dlrm_embbag_interact_fwd", lib().dlrm_embbag_interact_fwd(_ptr(x_dense), xd_ld, _ptr(table_ptrs), K, d,
                                                                       _ptr(indices), _ptr(offsets), B, _ptr(out),
                                                                       _dtype_code(out), out_ld, _stream(stream)))


def dlrm_embbag_interact_fwd_lp(x_dense, xd_ld: int, table_ptrs, table_dtype: int, scale_bias_ptrs, K: int, d: int,
                                indices, offsets, B: int, out, out_ld: int, stream=None) -> None:
    sb = _ptr(scale_bias_ptrs) if scale_bias_ptrs is not None else None
    _check("dlrm_embbag_interact_fwd_lp", lib().dlrm_embbag_interact_fwd_lp(
        _ptr(x_dense), xd_ld, _ptr(table_ptrs), table_dtype, sb, K, d, _ptr(indices), _ptr(offsets), B, _ptr(out),
        _dtype_code(out), out_ld, _stream(stream)))


def dlrm_interact_bwd(X, B: int, n: int, d: int, x_ld: int, g, g_ld: int, dX, dx_ld: int, stream=None) -> None:
    _check("dlrm_interact_bwd", lib().dlrm_interact_bwd(_ptr(X), B, n, d, x_ld, _ptr(g), g_ld, _ptr(dX), dx_ld,
                                                         _stream(stream)))


def dlrm_mlp_workspace_size(B: int, dims, w_dtype: int, save_acts: bool) -> int:
    return int(lib().dlrm_mlp_workspace_size(B, len(dims) - 1, _host_i32(dims), w_dtype, int(save_acts)))


def dlrm_mlp_fwd(inp, in_ld: int, B: int, dims, Ws, w_ld, biases, w_dtype: int, last_act: int, out, out_ld: int,
                 prob, ws, save_acts: bool, stream=None) -> None:
    L = len(dims) - 1
    wld = _host_i32(w_ld) if w_ld is not None else None
    _check("dlrm_mlp_fwd", lib().dlrm_mlp_fwd(_ptr(inp), _dtype_code(inp), in_ld, B, L, _host_i32(dims), _host_ptrs(Ws),
                                               wld, _host_ptrs(biases), w_dtype, last_act, _ptr(out), out_ld,
                                               _ptr(prob), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                               int(save_acts), _stream(stream)))


def dlrm_linear_fwd(A, lda: int, W, ldw: int, bias, C, ldc: int, M: int, N: int, K: int, act: int,
                    stream=None) -> None:
    """One bf16 layer C = act(A W^T + b); C's dtype (fp32 or bf16) selects the output."""
    _check("dlrm_linear_fwd", lib().dlrm_linear_fwd(_ptr(A), lda, _ptr(W), ldw, _ptr(bias), _ptr(C), _dtype_code(C),
                                                     ldc, M, N, K, act, _stream(stream)))


def dlrm_mlp_bwd_workspace_size(B: int, dims) -> int:
    return int(lib().dlrm_mlp_bwd_workspace_size(B, len(dims) - 1, _host_i32(dims)))


def dlrm_mlp_bwd(B: int, dims, Ws, w_ld, last_act: int, fwd_ws, out, out_ld: int, dY, dy_ld: int, dWs, dbs, dX,
                 dx_ld: int, ws, stream=None) -> None:
    L = len(dims) - 1
    wld = _host_i32(w_ld) if w_ld is not None else None
    _check("dlrm_mlp_bwd", lib().dlrm_mlp_bwd(B, L, _host_i32(dims), _host_ptrs(Ws), wld, last_act, _ptr(fwd_ws),
                                               _ptr(out), out_ld, _ptr(dY), dy_ld, _host_ptrs(dWs), _host_ptrs(dbs),
                                               _ptr(dX), dx_ld, _ptr(ws), ws.numel() * ws.element_size(),
                                               _stream(stream)))


def dlrm_bce_grad(logit, logit_ld: int, y, B: int, dY, stream=None) -> None:
    _check("dlrm_bce_grad", lib().dlrm_bce_grad(_ptr(logit), logit_ld, _ptr(y), B, _ptr(dY), _stream(stream)))


def dlrm_embbag_bwd_sgd_workspace_size(K: int, B: int, nnz: int, d: int) -> int:
    return int(lib().dlrm_embbag_bwd_sgd_workspace_size(K, B, nnz, d))


def dlrm_embbag_bwd_sgd(table_ptrs, K: int, d: int, rows, indices, offsets, B: int, nnz: int, G, g_ld: int,
                        g_col0: int, lr: float, ws, stream=None) -> None:
    rows_h = (ctypes.c_int64 * K)(*[int(r) for r in rows])
    _check("dlrm_embbag_bwd_sgd", lib().dlrm_embbag_bwd_sgd(_ptr(table_ptrs), K, d, rows_h, _ptr(indices),
                                                             _ptr(offsets), B, nnz, _ptr(G), g_ld, g_col0,
                                                             ctypes.c_float(lr), _ptr(ws),
                                                             ws.numel() * ws.element_size(), _stream(stream)))


def dlrm_embbag_bwd_sgd_noalloc(table_ptrs, K: int, d: int, rows, indices, offsets, B: int, nnz: int, G, g_ld: int,
                                g_col0: int, lr: float, stream=None) -> None:
    """dlrm_embbag_bwd_sgd on the library's static device scratch (no workspace)."""
    rows_h = (ctypes.c_int64 * K)(*[int(r) for r in rows])
    _check("dlrm_embbag_bwd_sgd_noalloc",
           lib().dlrm_embbag_bwd_sgd_noalloc(_ptr(table_ptrs), K, d, rows_h, _ptr(indices), _ptr(offsets), B, nnz,
                                             _ptr(G), g_ld, g_col0, ctypes.c_float(lr), _stream(stream)))


def dlrm_embbag_bwd_sgd_prepare(K: int, rows, indices, offsets, B: int, nnz: int, ws, stream=None) -> None:
    rows_h = (ctypes.c_int64 * K)(*[int(r) for r in rows])
    _check("dlrm_embbag_bwd_sgd_prepare",
           lib().dlrm_embbag_bwd_sgd_prepare(K, rows_h, _ptr(indices), _ptr(offsets), B, nnz, _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream)))


def dlrm_embbag_bwd_sgd_apply(table_ptrs, K: int, d: int, rows, B: int, nnz: int, G, g_ld: int, g_col0: int,
                              lr: float, ws, stream=None, side=None) -> None:
    """side: an optional second torch stream for the short segments; the
    caller orders it (side.wait_stream(stream) before the call,
    stream.wait_stream(side) after it)."""
    rows_h = (ctypes.c_int64 * K)(*[int(r) for r in rows])
    side_h = ctypes.c_void_p(side.cuda_stream) if side is not None else None
    _check("dlrm_embbag_bwd_sgd_apply",
           lib().dlrm_embbag_bwd_sgd_apply(_ptr(table_ptrs), K, d, rows_h, B, nnz, _ptr(G), g_ld, g_col0,
                                           ctypes.c_float(lr), _ptr(ws), ws.numel() * ws.element_size(),
                                           _stream(stream), side_h))


def dlrm_check_indices(indices, offsets, K: int, B: int, rows_dev, bad_count, stream=None) -> None:
    _check("dlrm_check_indices", lib().dlrm_check_indices(_ptr(indices), _ptr(offsets), K, B, _ptr(rows_dev),
                                                           _ptr(bad_count), _stream(stream)))
