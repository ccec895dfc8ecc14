"""The DLRM forward pass and training step as a sequence of libdlrm calls.

Holds device buffers (torch tensors: memory only) and orders the C-ABI
calls on one stream; it performs no arithmetic itself.

Forward ([SU] "briansu.co DLRM", How it works and Key equations):
  1. dlrm_mlp_fwd(bottom)   dense [B][13] -> x_dense              (fp32)
  2. dlrm_embbag_fwd        bags of K tables -> X[:, 1..K, :]     (fp32)
  3. dlrm_interact_fwd      X -> [x_dense, tril(X X^T)]           (bf16 row)
  4. dlrm_mlp_fwd(top)      -> logit, sigmoid(logit)
With ``fused=True`` steps 2 and 3 are one dlrm_embbag_interact_fwd call and
X never goes to memory; with ``fused=False`` x_dense is row 0 of X and the
two calls run separately.  ``fused="auto"`` (the default) keeps X and picks
per batch: the fused call for short bags, where the lookups are latency-bound
and skipping X's write and re-read pays, the two calls for long bags, where
the standalone lookup keeps more rows in flight (measured crossover below).
Training step (sum-pooled tables, row-wise SGD):
  forward with saved activations, dlrm_bce_grad, dlrm_mlp_bwd(top),
  dlrm_mlp_bwd(bottom) seeded by the X row-0 gradient, and
  dlrm_embbag_bwd_sgd with the X rows 1..K gradient (or its index half,
  dlrm_embbag_bwd_sgd_prepare, on a second stream beside the forward and
  dlrm_embbag_bwd_sgd_apply once the gradient exists).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib as C


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


@dataclass
class MLPParams:
    dims: tuple
    Ws: list        # device tensors [out][w_ld] (bf16 or fp32)
    w_ld: list
    biases: list    # device fp32 [out]
    w_dtype: int


def make_mlp(dims, weights, biases, bf16: bool, device="cuda") -> MLPParams:
    """Device copies of host weights, rows padded to a multiple of 8 elements
    (bf16) so the MFMA GEMM reads every operand with 16-byte loads."""
    Ws, lds, bs = [], [], []
    for W, b in zip(weights, biases):
        out_f, in_f = W.shape
        if bf16:
            ld = _round_up(in_f, 8)
            Wd = torch.zeros((out_f, ld), dtype=torch.bfloat16, device=device)
            Wd[:, :in_f] = torch.as_tensor(W).to(device=device, dtype=torch.bfloat16)
        else:
            ld = in_f
            Wd = torch.as_tensor(W, dtype=torch.float32).to(device).contiguous()
        Ws.append(Wd)
        lds.append(ld)
        bs.append(torch.as_tensor(b, dtype=torch.float32).to(device).contiguous())
    return MLPParams(tuple(int(x) for x in dims), Ws, lds, bs, C.DLRM_BF16 if bf16 else C.DLRM_F32)


def pad_first_layer(mlp: MLPParams, k_pad: int) -> MLPParams:
    """The same MLP with its first layer's input widened to k_pad by zero
    weight columns: the products of the zero columns add exact zeros, so
    the outputs are unchanged, and a k that is a multiple of 64 takes the
    GEMM's 64-wide k-tiles."""
    W0 = mlp.Ws[0]
    out_f = W0.shape[0]
    Wp = torch.zeros((out_f, k_pad), dtype=W0.dtype, device=W0.device)
    Wp[:, :W0.shape[1]] = W0
    return MLPParams((k_pad,) + tuple(mlp.dims[1:]), [Wp] + list(mlp.Ws[1:]), [k_pad] + list(mlp.w_ld[1:]),
                     mlp.biases, mlp.w_dtype)


# Mean bag length up to which "auto" takes the fused lookup + interaction.
AUTO_FUSED_MAX_MEAN_BAG = 2.0


class DLRM:
    """Device state and call sequence for one batch size."""

    def __init__(self, B: int, K: int, d: int, rows, tables, bottom: MLPParams, top: MLPParams, train: bool = False,
                 device="cuda", fused="auto", table_dtype: str = "f32", scale_bias=None, pad_top: bool = True):
        """table_dtype "f32", or "bf16" / "int8" rows (forward only) with, for
        int8, ``scale_bias`` = K fp32 [m_k][2] tensors.  A forward-only model
        widens the top MLP's first layer with zero columns unless ``pad_top``
        is False (see ``pad_first_layer``); ``self.top`` holds the layers the
        calls use."""
        self.B, self.K, self.d, self.n = B, K, d, K + 1
        self.rows = [int(r) for r in rows]
        self.tables = tables
        self.table_ptrs = C.device_pointer_array(tables)
        if table_dtype not in ("f32", "bf16", "int8"):
            raise ValueError("table_dtype must be 'f32', 'bf16' or 'int8'")
        if table_dtype != "f32" and train:
            raise ValueError("the sparse SGD update needs fp32 table rows")
        self.table_dtype = table_dtype
        self.table_code = {"bf16": C.DLRM_BF16, "int8": C.DLRM_I8}.get(table_dtype)
        self.scale_bias = scale_bias
        self.sb_ptrs = C.device_pointer_array(scale_bias) if scale_bias is not None else None
        self.bottom, self.top = bottom, top
        self.train = train
        if fused not in (True, False, "auto"):
            raise ValueError("fused must be True, False or 'auto'")
        self.fused = fused
        n, dev = self.n, device
        self.P = n * (n - 1) // 2
        self.top_w = d + self.P
        if fused is True:
            self.X = None
            self.x0 = torch.empty((B, d), dtype=torch.float32, device=dev)
            self.x0_ld = d
        else:
            self.X = torch.empty((B, n, d), dtype=torch.float32, device=dev)
            self.x0 = self.X
            self.x0_ld = n * d
        top_dtype = torch.bfloat16 if top.w_dtype == C.DLRM_BF16 else torch.float32
        self.top_ld = _round_up(self.top_w, 8) if top_dtype == torch.bfloat16 else _round_up(self.top_w, 4)
        if pad_top and not train and top_dtype == torch.bfloat16 and self.top_w >= 256 and self.top_w % 64 != 0:
            # forward only: the top MLP reads the interaction rows as K =
            # top_w rounded up to 64 (zero columns), e.g. 512 for 479
            # (measured faster)
            self.top_ld = _round_up(self.top_w, 64)
            self.top = top = pad_first_layer(top, self.top_ld)
        # zero-filled once: the interaction calls write columns below
        # round_up(top_w, 8) only (zeros from top_w on), so the columns up to
        # top_ld stay zero and meet zero weight columns
        self.top_written = min(_round_up(self.top_w, 8), self.top_ld)
        self.top_in = torch.zeros((B, self.top_ld), dtype=top_dtype, device=dev)
        self.logit = torch.empty((B, 1), dtype=torch.float32, device=dev)
        self.prob = torch.empty((B,), dtype=torch.float32, device=dev)
        save = bool(train)
        self.ws_bot = self._ws(C.dlrm_mlp_workspace_size(B, bottom.dims, bottom.w_dtype, save))
        self.ws_top = self._ws(C.dlrm_mlp_workspace_size(B, top.dims, top.w_dtype, save))
        if train:
            self.ws_bot_bwd = self._ws(C.dlrm_mlp_bwd_workspace_size(B, bottom.dims))
            self.ws_top_bwd = self._ws(C.dlrm_mlp_bwd_workspace_size(B, top.dims))
            self.dW_bot = [torch.empty((o, i), dtype=torch.float32, device=dev)
                           for i, o in zip(bottom.dims[:-1], bottom.dims[1:])]
            self.db_bot = [torch.empty((o,), dtype=torch.float32, device=dev) for o in bottom.dims[1:]]
            self.dW_top = [torch.empty((o, i), dtype=torch.float32, device=dev)
                           for i, o in zip(top.dims[:-1], top.dims[1:])]
            self.db_top = [torch.empty((o,), dtype=torch.float32, device=dev) for o in top.dims[1:]]
            self.dlogit = torch.empty((B,), dtype=torch.float32, device=dev)
            self.ws_sparse = None
            if fused is not True:  # full backward chain: gradient of the top input row, then of X
                self.g_top = torch.empty((B, self.top_w), dtype=torch.float32, device=dev)
                self.G = torch.empty((B, n, d), dtype=torch.float32, device=dev)

    @staticmethod
    def _ws(nbytes: int):
        return torch.empty((max(nbytes, 256),), dtype=torch.uint8, device="cuda")

    def use_fused(self, nnz: int) -> bool:
        """Whether a batch of nnz lookups takes the fused lookup + interaction
        (from low-precision rows only for d a multiple of 32)."""
        if self.fused == "auto":
            if self.table_dtype != "f32" and self.d % 32 != 0:
                return False
            return nnz <= AUTO_FUSED_MAX_MEAN_BAG * self.K * self.B
        return bool(self.fused)

    def forward(self, dense, indices, offsets, stream=None):
        B, n, d = self.B, self.n, self.d
        save = self.train
        C.dlrm_mlp_fwd(dense, dense.shape[1], B, self.bottom.dims, self.bottom.Ws, self.bottom.w_ld,
                       self.bottom.biases, self.bottom.w_dtype, C.DLRM_ACT_RELU, self.x0, self.x0_ld, None,
                       self.ws_bot, save, stream)
        lp = self.table_dtype != "f32"
        if self.use_fused(indices.numel()):
            if lp:
                C.dlrm_embbag_interact_fwd_lp(self.x0, self.x0_ld, self.table_ptrs, self.table_code, self.sb_ptrs,
                                              self.K, d, indices, offsets, B, self.top_in, self.top_ld, stream)
            else:
                C.dlrm_embbag_interact_fwd(self.x0, self.x0_ld, self.table_ptrs, self.K, d, indices, offsets, B,
                                           self.top_in, self.top_ld, stream)
        else:
            if lp:
                C.dlrm_embbag_fwd_lp(self.table_ptrs, self.table_code, self.sb_ptrs, self.K, d, indices, offsets, B,
                                     self.X, n * d, d, stream, nnz=indices.numel())
            else:
                C.dlrm_embbag_fwd(self.table_ptrs, self.K, d, indices, offsets, B, self.X, n * d, d, stream,
                                  nnz=indices.numel())
            C.dlrm_interact_fwd(self.X, B, n, d, n * d, self.top_in, self.top_ld, stream)
        C.dlrm_mlp_fwd(self.top_in, self.top_ld, B, self.top.dims, self.top.Ws, self.top.w_ld, self.top.biases,
                       self.top.w_dtype, C.DLRM_ACT_NONE, self.logit, 1, self.prob, self.ws_top, save, stream)
        return self.logit, self.prob

    def sparse_workspace(self, nnz: int):
        need = C.dlrm_embbag_bwd_sgd_workspace_size(self.K, self.B, nnz, self.d)
        if self.ws_sparse is None or self.ws_sparse.numel() < need:
            self.ws_sparse = self._ws(need)
        return self.ws_sparse

    def sparse_prepare(self, indices, offsets, nnz: int, stream=None):
        """The index half of the sparse update (keys, sort, segments): it
        needs only this batch's indices, so it can run on a second stream
        beside the forward and the dense backward; ``backward(...,
        prepared=True)`` then applies it (the caller orders the two)."""
        C.dlrm_embbag_bwd_sgd_prepare(self.K, self.rows, indices, offsets, self.B, nnz, self.sparse_workspace(nnz),
                                      stream)

    def _sparse_update(self, G, indices, offsets, nnz, lr, prepared, stream, side=None):
        B, n, d = self.B, self.n, self.d
        if prepared:
            C.dlrm_embbag_bwd_sgd_apply(self.table_ptrs, self.K, d, self.rows, B, nnz, G, n * d, d, lr,
                                        self.sparse_workspace(nnz), stream, side)
        else:
            C.dlrm_embbag_bwd_sgd(self.table_ptrs, self.K, d, self.rows, indices, offsets, B, nnz, G, n * d, d, lr,
                                  self.sparse_workspace(nnz), stream)

    def backward(self, labels, G, indices, offsets, nnz: int, lr: float, stream=None, prepared: bool = False,
                 side=None):
        """Dense gradients (top: from the BCE loss; bottom: from G[:, 0, :]) and
        the sparse SGD update of the tables from G[:, 1..K, :] (from a
        ``sparse_prepare`` of this batch when ``prepared``; then ``side``, a
        second torch stream, may take the update's short segments, forked
        from and joined back into the update's stream here)."""
        B, n, d = self.B, self.n, self.d
        C.dlrm_bce_grad(self.logit, 1, labels, B, self.dlogit, stream)
        C.dlrm_mlp_bwd(B, self.top.dims, self.top.Ws, self.top.w_ld, C.DLRM_ACT_NONE, self.ws_top, self.logit, 1,
                       self.dlogit, 1, self.dW_top, self.db_top, None, 0, self.ws_top_bwd, stream)
        C.dlrm_mlp_bwd(B, self.bottom.dims, self.bottom.Ws, self.bottom.w_ld, C.DLRM_ACT_RELU, self.ws_bot, self.x0,
                       self.x0_ld, G, n * d, self.dW_bot, self.db_bot, None, 0, self.ws_bot_bwd, stream)
        if prepared and side is not None:
            cur = stream if stream is not None else torch.cuda.current_stream()
            side.wait_stream(cur)
            self._sparse_update(G, indices, offsets, nnz, lr, prepared, stream, side)
            cur.wait_stream(side)
        else:
            self._sparse_update(G, indices, offsets, nnz, lr, prepared, stream)

    def backward_chain(self, labels, indices, offsets, nnz: int, lr: float, stream=None, prepared: bool = False):
        """The whole training backward from the loss: BCE seed, top MLP (with
        the gradient of its input row), interaction backward to the gradient
        of X, then the bottom MLP from row 0 and the sparse SGD update from
        rows 1..K.  Needs X (a model built with fused=False or "auto") and
        the two-call forward of this batch."""
        if self.fused is True or not self.train:
            raise ValueError("backward_chain needs a training model built with fused=False or 'auto'")
        if self.use_fused(indices.numel()):
            raise ValueError("backward_chain needs X: this batch's forward took the fused path")
        B, n, d = self.B, self.n, self.d
        C.dlrm_bce_grad(self.logit, 1, labels, B, self.dlogit, stream)
        C.dlrm_mlp_bwd(B, self.top.dims, self.top.Ws, self.top.w_ld, C.DLRM_ACT_NONE, self.ws_top, self.logit, 1,
                       self.dlogit, 1, self.dW_top, self.db_top, self.g_top, self.top_w, self.ws_top_bwd, stream)
        C.dlrm_interact_bwd(self.X, B, n, d, n * d, self.g_top, self.top_w, self.G, n * d, stream)
        C.dlrm_mlp_bwd(B, self.bottom.dims, self.bottom.Ws, self.bottom.w_ld, C.DLRM_ACT_RELU, self.ws_bot, self.x0,
                       self.x0_ld, self.G, n * d, self.dW_bot, self.db_bot, None, 0, self.ws_bot_bwd, stream)
        self._sparse_update(self.G, indices, offsets, nnz, lr, prepared, stream)
