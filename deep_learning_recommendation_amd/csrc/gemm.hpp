// Internal GEMM-family launchers used by the MLP forward and backward.
#pragma once

#include "common.hpp"

namespace dlrm {

// C[M][N] = act(A[M][K] * W[N][K]^T + bias[N]) on bf16 operands with fp32
// accumulation (MFMA).  A, W: bf16 bits; C: fp32 or bf16 (out_bf16).
int gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, const float* bias, void* C,
              int64_t ldc, bool out_bf16, int M, int N, int K, bool relu, hipStream_t s);
// As gemm_bf16 without bias or activation, with operands that may be stored
// k-major: a_kmajor, A is [K][M] (lda its pitch) instead of [M][K];
// w_kmajor, W is [K][N] instead of [N][K].  The k-major forms need 16-byte
// aligned rows with a pitch that is a multiple of 8 and fp32 output
// (DLRM_E_UNSUPPORTED otherwise).
int gemm_bf16_ex(const uint16_t* A, int64_t lda, bool a_kmajor, const uint16_t* W, int64_t ldw, bool w_kmajor,
                 void* C, int64_t ldc, bool out_bf16, int M, int N, int K, hipStream_t s);
// Input gradient of a ReLU layer, fused: g = A W^T (no bias; W k-major,
// i.e. stored [K][N], with w_kmajor), then delta = bf16(g) where y > 0 and
// 0 elsewhere, written row-major to dlt [M][ldd] and, when dout.dT is set,
// transposed to dout.dT [N][ldt], and per block of *tile_rows rows the fp32
// column sums of delta to dout.dbp[(row / *tile_rows)][N].
struct DeltaOut {
  const uint16_t* y = nullptr;  // bf16 [M][ldy], the mask source
  int64_t ldy = 0;
  uint16_t* dT = nullptr;
  int64_t ldt = 0;
  float* dbp = nullptr;
};
int gemm_bf16_delta(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, bool w_kmajor, int M, int N,
                    int K, uint16_t* dlt, int64_t ldd, const DeltaOut& dout, int* tile_rows, hipStream_t s);
// A hidden ReLU layer followed by a single-output layer, in one launch:
// h = bf16(relu(A W^T + bias)) with N <= 256 (one block tile holds a row's
// every column), then out[m] = act(sum_n h[m][n] w[n] + b) in fp32, and
// prob[m] = 1 / (1 + exp(-out[m])) when prob is set.  h is written to H
// [M][ldh] only when H is set (the backward pass reads it).
struct DotOut {
  const uint16_t* w = nullptr;  // bf16 [N], the single-output layer's weight row
  const float* b = nullptr;     // its bias (nullable)
  float* out = nullptr;         // fp32 [M] with pitch ldo
  int64_t ldo = 1;
  float* prob = nullptr;  // nullable
  int relu = 0;           // ReLU on out
};
int gemm_bf16_dot(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, const float* bias, uint16_t* H,
                  int64_t ldh, int M, int N, int K, const DotOut& dot, hipStream_t s);
// Split-K partials with both operands k-major: part[z][M][N] = the sum over
// slice z of k of A[k][m] W[k][n] (A [K][M], W [K][N]), e.g. a weight
// gradient delta^T x straight from the row-major delta and activations.
int gemm_bf16_splitk_kmajor(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, float* part, int M,
                            int N, int K, int splits, hipStream_t s);

// N == 1 layer: out[m] = sum_k A[m][k] w[k] + bias; prob = sigmoid(out).
int gemv_bf16(const uint16_t* A, int64_t lda, const uint16_t* w, const float* bias, float* out, int64_t ldo,
              float* prob, int M, int K, bool relu, hipStream_t s);

// fp32 network: C = act(A W^T + bias), A fp32, W fp32.
int gemm_f32(const float* A, int64_t lda, const float* W, int64_t ldw, const float* bias, float* C, int64_t ldc,
             float* prob, int M, int N, int K, bool relu, hipStream_t s);

// out[c][r] = in[r][c] (bf16 bits).
int transpose_bf16(const uint16_t* in, int64_t ld_in, uint16_t* out, int64_t ld_out, int R, int C, hipStream_t s);

// out[r][c] = bf16(in[r][c]) for c < C, zero for C <= c < ld_pad_to.
int convert_to_bf16(const float* in, int64_t ld_in, uint16_t* out, int64_t ld_out, int R, int C, hipStream_t s);

}  // namespace dlrm
