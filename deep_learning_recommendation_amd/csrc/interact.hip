// Pairwise dot-product interaction: Z = tril(X X^T) without the diagonal,
// packed row by row after the dense vector.
//
// Model: briansu.co DLRM, Key equations (Interaction: Z = tril(X X^T) with
// X = [x_dense; e_1..e_K]; Output: the top MLP reads [x_dense, vec(Z)]);
// "Deep Learning Recommendation Model (DLRM)" explainer, Key Method Details,
// Interaction layer (only the n(n-1)/2 pairs of distinct vectors).
//
// Kernel design (gfx950): one wave per sample.  The sample's n x d matrix is
// loaded straight into registers as 16-row tiles: lane l holds rows
// T*16 + (l % 16) and, for every 16-wide k chunk, the four consecutive
// columns 4*(l / 16) .. +3.  That is exactly the A operand of
// v_mfma_f32_16x16x4_f32 for the tile's rows and the B operand for X^T, so
// Gram block (I, J) is a chain of 4*ceil(d/16) MFMAs on register data, with
// the k order permuted inside each chunk (fp32 sums in any order meet the
// d*u error bound).  Only blocks with J <= I are computed.  fp32 MFMA runs
// at twice the rate of unpacked fp32 VALU FMAs, so it wins even where
// padding to 16 rows wastes part of a block.  The kernel is bound by HBM
// (reading X, writing the packed rows).
#include "common.hpp"

namespace dlrm {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void put(float* p, float v) { *p = v; }
__device__ __forceinline__ void put(uint16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void put4(float* p, f4 v) { *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ void put4(uint16_t* p, f4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

template <int NT, int DC, typename OutT>
__global__ __launch_bounds__(256) void interact_mfma_kernel(const float* __restrict__ X, int64_t B, int n, int d,
                                                            int64_t x_ld, OutT* __restrict__ out, int64_t out_ld,
                                                            int pad_end) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;  // whole wave
  const float* __restrict__ xb = X + b * x_ld;
  OutT* __restrict__ ob = out + b * out_ld;
  const int r16 = lane & 15, g = lane >> 4;

  f4 x[NT][DC];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int row = t * 16 + r16;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int kk = c * 16 + 4 * g;
      if (row < n && kk < d) {
        const float4 v = *reinterpret_cast<const float4*>(xb + (int64_t)row * d + kk);
        x[t][c] = f4{v.x, v.y, v.z, v.w};
      } else {
        x[t][c] = f4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // dense vector first: row 0 lives in lanes 0, 16, 32, 48 of tile 0
  if (r16 == 0) {
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int kk = c * 16 + 4 * g;
      if (kk < d) put4(ob + kk, x[0][c]);
    }
  }

#pragma unroll
  for (int I = 0; I < NT; ++I) {
    f4 acc[NT];
#pragma unroll
    for (int J = 0; J <= I; ++J) acc[J] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float a = x[I][c][s];
#pragma unroll
        for (int J = 0; J <= I; ++J) acc[J] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, x[J][c][s], acc[J], 0, 0, 0);
      }
    }
    // D[i][j] of block (I, J): lane holds i = 4*(l/16) + r, j = l % 16
#pragma unroll
    for (int J = 0; J <= I; ++J) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = I * 16 + 4 * g + r;
        const int j = J * 16 + r16;
        if (i < n && j < i) put(ob + d + i * (i - 1) / 2 + j, acc[J][r]);
      }
    }
  }

  const int end = d + n * (n - 1) / 2;
  for (int col = end + lane; col < pad_end; col += 64) put(ob + col, 0.f);
}

// Any shape: one thread per (sample, output column).  fp32 FMA chain.
template <typename OutT>
__global__ __launch_bounds__(256) void interact_generic_kernel(const float* __restrict__ X, int64_t B, int n, int d,
                                                               int64_t x_ld, OutT* __restrict__ out, int64_t out_ld,
                                                               int pad_end) {
  const int64_t width = pad_end;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * width) return;
  const int64_t b = t / width;
  const int col = (int)(t - b * width);
  const float* xb = X + b * x_ld;
  float v = 0.f;
  const int P = n * (n - 1) / 2;
  if (col < d) {
    v = xb[col];
  } else if (col < d + P) {
    const int q = col - d;
    int i = 1;
    while ((i + 1) * i / 2 <= q) ++i;
    const int j = q - i * (i - 1) / 2;
    const float* xi = xb + (int64_t)i * d;
    const float* xj = xb + (int64_t)j * d;
    for (int c = 0; c < d; ++c) v = __builtin_fmaf(xi[c], xj[c], v);
  }
  put(out + b * out_ld + col, v);
}

template <int NT, int DC, typename OutT>
void launch_mfma(const float* X, int64_t B, int n, int d, int64_t x_ld, OutT* out, int64_t out_ld, int pad_end,
                 hipStream_t s) {
  hipLaunchKernelGGL((interact_mfma_kernel<NT, DC, OutT>), dim3((unsigned)ceil_div(B, 4)), dim3(256), 0, s, X, B, n,
                     d, x_ld, out, out_ld, pad_end);
}

template <int DC, typename OutT>
bool dispatch_nt(int NT, const float* X, int64_t B, int n, int d, int64_t x_ld, OutT* out, int64_t out_ld,
                 int pad_end, hipStream_t s) {
  // x[NT][DC] must fit in 128 registers per lane: NT * DC <= 32
  constexpr int kMaxNT = (32 / DC) < 8 ? (32 / DC) : 8;
  if (NT > kMaxNT) return false;
  switch (NT) {
    case 1: launch_mfma<1, DC>(X, B, n, d, x_ld, out, out_ld, pad_end, s); return true;
    case 2: launch_mfma<2, DC>(X, B, n, d, x_ld, out, out_ld, pad_end, s); return true;
    case 3: if constexpr (kMaxNT >= 3) { launch_mfma<3, DC>(X, B, n, d, x_ld, out, out_ld, pad_end, s); return true; } break;
    case 4: if constexpr (kMaxNT >= 4) { launch_mfma<4, DC>(X, B, n, d, x_ld, out, out_ld, pad_end, s); return true; } break;
    case 5: if constexpr (kMaxNT >= 5) { launch_mfma<5, DC>(X, B, n, d, x_ld, out, out_ld, pad_end, s); return true; } break;
    case 6: if constexpr (kMaxNT >= 6) { launch_mfma<6, DC>(X, B, n, d, x_ld, out, out_ld, pad_end, s); return true; } break;
    case 7: if constexpr (kMaxNT >= 7) { launch_mfma<7, DC>(X, B, n, d, x_ld, out, out_ld, pad_end, s); return true; } break;
    case 8: if constexpr (kMaxNT >= 8) { launch_mfma<8, DC>(X, B, n, d, x_ld, out, out_ld, pad_end, s); return true; } break;
  }
  return false;
}

template <typename OutT>
void run(const float* X, int64_t B, int n, int d, int64_t x_ld, OutT* out, int64_t out_ld, int pad_end,
         hipStream_t s) {
  const int NT = (n + 15) / 16;
  const int dc = (d + 15) / 16;
  bool done = false;
  if (dc <= 1) done = dispatch_nt<1>(NT, X, B, n, d, x_ld, out, out_ld, pad_end, s);
  else if (dc <= 2) done = dispatch_nt<2>(NT, X, B, n, d, x_ld, out, out_ld, pad_end, s);
  else if (dc <= 4) done = dispatch_nt<4>(NT, X, B, n, d, x_ld, out, out_ld, pad_end, s);
  else if (dc <= 8) done = dispatch_nt<8>(NT, X, B, n, d, x_ld, out, out_ld, pad_end, s);
  else if (dc <= 16) done = dispatch_nt<16>(NT, X, B, n, d, x_ld, out, out_ld, pad_end, s);
  if (!done) {
    const int64_t total = B * (int64_t)pad_end;
    hipLaunchKernelGGL((interact_generic_kernel<OutT>), dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, s, X, B,
                       n, d, x_ld, out, out_ld, pad_end);
  }
}

}  // namespace
}  // namespace dlrm

using namespace dlrm;

extern "C" int dlrm_interact_fwd(const float* X, int64_t B, int32_t n, int32_t d, int64_t x_ld, void* out,
                                 int32_t out_dtype, int64_t out_ld, hipStream_t stream) {
  if (!X || !out || B < 1 || n < 2 || n > 128 || d < 4 || d > 256 || (d % 4) != 0) return DLRM_E_INVALID;
  if (out_dtype != DLRM_F32 && out_dtype != DLRM_BF16) return DLRM_E_INVALID;
  const int64_t width = d + (int64_t)n * (n - 1) / 2;
  if (x_ld < (int64_t)n * d || (x_ld % 4) != 0 || !aligned16(X)) return DLRM_E_INVALID;
  if (out_ld < width || (out_ld % 4) != 0 || !aligned16(out)) return DLRM_E_INVALID;
  if (ceil_div(B, 4) > 0x7fffffffLL || B * out_ld > (int64_t)1 << 40) return DLRM_E_UNSUPPORTED;
  const int pad_end = (int)(round_up(width, 8) < out_ld ? round_up(width, 8) : out_ld);
  if (out_dtype == DLRM_F32)
    run<float>(X, B, n, d, x_ld, static_cast<float*>(out), out_ld, pad_end, stream);
  else
    run<uint16_t>(X, B, n, d, x_ld, static_cast<uint16_t*>(out), out_ld, pad_end, stream);
  return launch_status();
}
