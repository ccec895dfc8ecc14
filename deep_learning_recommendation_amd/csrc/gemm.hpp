// Internal GEMM-family launchers used by the MLP forward and backward.
#pragma once

#include "common.hpp"

namespace dlrm {

// C[M][N] = act(A[M][K] * W[N][K]^T + bias[N]) on bf16 operands with fp32
// accumulation (MFMA).  A, W: bf16 bits; C: fp32 or bf16 (out_bf16).
// With splits > 1, each of `splits` K-slices writes fp32 partials to
// part[z][M][N] (no bias or activation) and reduce_splits() finishes.
int gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, const float* bias, void* C,
              int64_t ldc, bool out_bf16, int M, int N, int K, bool relu, hipStream_t s);
// Input gradient of a ReLU layer, fused: g = A W^T (no bias), then
// delta = bf16(g) where y > 0 and 0 elsewhere, written row-major to dlt
// [M][ldd] and transposed to dout.dT [N][ldt], and per block of *tile_rows
// rows the fp32 column sums of delta to dout.dbp[(row / *tile_rows)][N].
struct DeltaOut {
  const uint16_t* y = nullptr;  // bf16 [M][ldy], the mask source
  int64_t ldy = 0;
  uint16_t* dT = nullptr;
  int64_t ldt = 0;
  float* dbp = nullptr;
};
int gemm_bf16_delta(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, int M, int N, int K,
                    uint16_t* dlt, int64_t ldd, const DeltaOut& dout, int* tile_rows, hipStream_t s);
int gemm_bf16_splitk(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, float* part, int M, int N,
                     int K, int splits, hipStream_t s);
int reduce_splits(const float* part, int splits, int M, int N, const float* bias, float* C, int64_t ldc,
                  bool relu, hipStream_t s);

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
