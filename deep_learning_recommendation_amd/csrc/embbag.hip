// Embedding lookup with sum pooling (forward) and index validation.
//
// Model: each categorical feature owns a table of m_k rows of width d and
// looks up rows by id ("Deep Learning Recommendation Model (DLRM)"
// explainer, Key Method Details, Embedding tables; briansu.co DLRM, How it
// works).  A bag of ids is pooled by summation in bag order, fp32, from +0.
//
// Kernel design (gfx950, wave64):
//  * A "group" of G lanes owns one row: G = d/4 rounded up to a power of two
//    (min 2, max 64), each lane loads 16 bytes (float4) per row, so a row of
//    d = 128 is one 512-byte coalesced load by 32 lanes and a wave serves two
//    groups.  Wider rows give each lane V float4 columns.
//  * Each group handles a chunk of CB consecutive bags of one table and
//    streams through their indices as one flat run: U row loads are in
//    flight before the first add, and the next U indices are fetched while
//    those adds run, so one-index bags (the pages' plain lookup) keep as many
//    bytes in flight as long bags do.
//  * CB follows the mean bag length L when the caller passes nnz:
//    CB = round(sqrt(64 / L)), about sqrt(64 L) rows per chunk.  Small
//    chunks balance the groups' work (chunks of ~500 rows left the last
//    groups running alone: 69% of HBM peak on bags of 1 + Poisson(19), 84%
//    at two bags per chunk); one-index bags need several per chunk to fill
//    the U-deep pipeline (best at 8).  Measured optima: L = 1: 8 bags,
//    L = 4: 4, L = 20: 2, L = 100: 1.
//  * Each column's sum is one serial chain in bag order inside one lane,
//    which makes the result bit-identical to a sequential fp32 sum.
#include "common.hpp"

#include <cmath>

namespace dlrm {
namespace {

// Table-row formats.  A lane loads one piece of a row (kVec x 4 consecutive
// columns) and turns it into kVec float4 when it is added:
//   fp32: 16 bytes, 4 columns.
//   bf16: 16 bytes, 8 columns (4 when d is not a multiple of 8), each value
//         widened exactly.
//   int8: 16 bytes, 16 columns (4 when d is not a multiple of 16), each value
//         dequantised with the row's scale s and bias z as (s * q) + z, two
//         fp32 roundings (no fused multiply-add).
// Loads are kept raw until the add so that the rows in flight cost the same
// registers in every format.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float deq(uint32_t u, int sh, float2 sz) {
  return __fadd_rn(__fmul_rn(sz.x, (float)(int8_t)(u >> sh)), sz.y);
}
__device__ __forceinline__ float4 deq4(uint32_t u, float2 sz) {
  return make_float4(deq(u, 0, sz), deq(u, 8, sz), deq(u, 16, sz), deq(u, 24, sz));
}
struct RowF32 {
  typedef float T;
  typedef uint4 Raw;
  static constexpr int kVec = 1;
  static constexpr bool kScaled = false;
  __device__ static Raw load(const T* row, int ch) { return *reinterpret_cast<const uint4*>(row + 4 * ch); }
  __device__ static void decode(Raw r, float2, float4 (&o)[kVec]) {
    o[0] = make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w));
  }
};
struct RowBF16 {
  typedef uint16_t T;
  typedef uint2 Raw;
  static constexpr int kVec = 1;
  static constexpr bool kScaled = false;
  __device__ static Raw load(const T* row, int ch) { return *reinterpret_cast<const uint2*>(row + 4 * ch); }
  __device__ static void decode(Raw r, float2, float4 (&o)[kVec]) {
    o[0] = make_float4(bf_lo(r.x), bf_hi(r.x), bf_lo(r.y), bf_hi(r.y));
  }
};
struct RowBF16x8 {
  typedef uint16_t T;
  typedef uint4 Raw;
  static constexpr int kVec = 2;
  static constexpr bool kScaled = false;
  __device__ static Raw load(const T* row, int ch) { return *reinterpret_cast<const uint4*>(row + 8 * ch); }
  __device__ static void decode(Raw r, float2, float4 (&o)[kVec]) {
    o[0] = make_float4(bf_lo(r.x), bf_hi(r.x), bf_lo(r.y), bf_hi(r.y));
    o[1] = make_float4(bf_lo(r.z), bf_hi(r.z), bf_lo(r.w), bf_hi(r.w));
  }
};
struct RowI8 {
  typedef int8_t T;
  typedef uint32_t Raw;
  static constexpr int kVec = 1;
  static constexpr bool kScaled = true;
  __device__ static Raw load(const T* row, int ch) { return *reinterpret_cast<const uint32_t*>(row + 4 * ch); }
  __device__ static void decode(Raw r, float2 sz, float4 (&o)[kVec]) { o[0] = deq4(r, sz); }
};
struct RowI8x16 {
  typedef int8_t T;
  typedef uint4 Raw;
  static constexpr int kVec = 4;
  static constexpr bool kScaled = true;
  __device__ static Raw load(const T* row, int ch) { return *reinterpret_cast<const uint4*>(row + 16 * ch); }
  __device__ static void decode(Raw r, float2 sz, float4 (&o)[kVec]) {
    o[0] = deq4(r.x, sz);
    o[1] = deq4(r.y, sz);
    o[2] = deq4(r.z, sz);
    o[3] = deq4(r.w, sz);
  }
};

// NC pieces per lane (piece ch = lane-in-group + j * G), U rows in flight.
template <int NC, int U, typename R = RowF32>
__global__ __launch_bounds__(256) void embbag_fwd_kernel(const typename R::T* const* __restrict__ tables,
                                                         const float* const* __restrict__ scale_bias, int32_t d,
                                                         int32_t g_log2, int32_t CB,
                                                         const int64_t* __restrict__ idx,
                                                         const int64_t* __restrict__ off, int64_t B,
                                                         int64_t chunks_per_table, int64_t total_chunks,
                                                         float* __restrict__ out, int64_t out_ld,
                                                         int64_t out_col0) {
  constexpr int KV = R::kVec;
  const int lane = threadIdx.x & 63;
  const int G = 1 << g_log2;
  const int gl = lane & (G - 1);
  const int gbase = lane - gl;
  const int64_t chunk = (int64_t)blockIdx.x * (blockDim.x >> g_log2) + (threadIdx.x >> g_log2);
  if (chunk >= total_chunks) return;  // whole group leaves together

  const int64_t k = chunk / chunks_per_table;
  const int64_t b0 = (chunk - k * chunks_per_table) * CB;
  const int nb = (int)min((int64_t)CB, B - b0);  // 1 <= nb <= CB <= G - 1
  const int64_t bag0 = k * B + b0;
  // lane j of the group holds the start of bag j; lane nb holds the end of the chunk
  const int64_t my_off = off[bag0 + min(gl, nb)];
  const typename R::T* __restrict__ T = tables[k];
  const float2* __restrict__ SB = R::kScaled ? reinterpret_cast<const float2*>(scale_bias[k]) : nullptr;
  const int npc = d / (4 * KV);  // pieces per row

  const int64_t P0 = __shfl(my_off, gbase, 64);
  const int64_t P1 = __shfl(my_off, gbase + nb, 64);
  int cb = 0;
  int64_t cur_end = __shfl(my_off, gbase + 1, 64);
  float* obase = out + out_col0 + k * (int64_t)d;

  float4 acc[NC][KV];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int v = 0; v < KV; ++v) acc[j][v] = make_float4(0.f, 0.f, 0.f, 0.f);

  auto flush = [&]() {
    float* o = obase + (b0 + cb) * out_ld;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int ch = gl + j * G;
#pragma unroll
      for (int v = 0; v < KV; ++v) {
        if (ch < npc) *reinterpret_cast<float4*>(o + 4 * (KV * ch + v)) = acc[j][v];
        acc[j][v] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    ++cb;
    cur_end = __shfl(my_off, gbase + min(cb + 1, nb), 64);
  };

  int64_t ridx[U];
#pragma unroll
  for (int u = 0; u < U; ++u) ridx[u] = (P0 + u < P1) ? idx[P0 + u] : 0;

  for (int64_t p = P0; p < P1; p += U) {
    typename R::Raw raw[U][NC];
    float2 sz[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const typename R::T* row = T + ridx[u] * (int64_t)d;
      sz[u] = (R::kScaled && p + u < P1) ? SB[ridx[u]] : make_float2(0.f, 0.f);
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int ch = gl + j * G;
        raw[u][j] = (p + u < P1 && ch < npc) ? R::load(row, ch) : typename R::Raw{};
      }
    }
    const int64_t pn = p + U;
#pragma unroll
    for (int u = 0; u < U; ++u) ridx[u] = (pn + u < P1) ? idx[pn + u] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (p + u < P1) {
        while (p + u >= cur_end) flush();
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          float4 t[KV];
          R::decode(raw[u][j], sz[u], t);
#pragma unroll
          for (int v = 0; v < KV; ++v) {
            acc[j][v].x = acc[j][v].x + t[v].x;
            acc[j][v].y = acc[j][v].y + t[v].y;
            acc[j][v].z = acc[j][v].z + t[v].z;
            acc[j][v].w = acc[j][v].w + t[v].w;
          }
        }
      }
    }
  }
  while (cb < nb) flush();
}

__global__ __launch_bounds__(256) void check_indices_kernel(const int64_t* __restrict__ idx,
                                                            const int64_t* __restrict__ off, int64_t K,
                                                            int64_t B, const int64_t* __restrict__ rows,
                                                            unsigned long long* bad) {
  __shared__ unsigned long long s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  const int64_t kb = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned long long local = 0;
  if (kb < K * B) {
    const int64_t k = kb / B;
    const int64_t a = off[kb], e = off[kb + 1];
    if (e < a) {
      ++local;
    } else {
      const int64_t m = rows[k];
      for (int64_t p = a; p < e; ++p) {
        const int64_t r = idx[p];
        local += (r < 0 || r >= m) ? 1ull : 0ull;
      }
    }
    if (kb == 0 && a != 0) ++local;
  }
  if (local) atomicAdd(&s_bad, local);
  __syncthreads();
  if (threadIdx.x == 0 && s_bad) atomicAdd(bad, s_bad);
}

}  // namespace
}  // namespace dlrm

using namespace dlrm;

namespace dlrm {
namespace {
template <typename R>
int launch_embbag(const typename R::T* const* tables, const float* const* scale_bias, int32_t K, int32_t d,
                  const int64_t* indices, const int64_t* offsets, int64_t B, int64_t nnz, float* out, int64_t out_ld,
                  int64_t out_col0, hipStream_t stream) {
  const int npc = d / (4 * R::kVec);  // pieces per row, one per lane
  int g_log2 = 1;
  while ((1 << g_log2) < npc && g_log2 < 6) ++g_log2;
  const int G = 1 << g_log2;
  const int Vneed = (npc + G - 1) / G;  // 1..4 pieces per lane
  const int64_t bags = (int64_t)K * B;
  // CB <= G - 1; without nnz, enough chunks to fill the chip several times over
  int64_t cb = bags / 65536;
  if (nnz > 0) cb = (int64_t)(sqrt(64.0 * (double)bags / (double)nnz) + 0.5);
  if (cb < 1) cb = 1;
  if (cb > G - 1) cb = G - 1;
  const int CB = (int)cb;
  const int64_t chunks_per_table = ceil_div(B, CB);
  const int64_t total = (int64_t)K * chunks_per_table;
  const int groups_per_block = 256 / G;
  const int64_t blocks = ceil_div(total, groups_per_block);
  if (blocks > 0x7fffffffLL) return DLRM_E_UNSUPPORTED;
  const dim3 grid((unsigned)blocks), block(256);
  if (Vneed == 1)
    hipLaunchKernelGGL((embbag_fwd_kernel<1, 8, R>), grid, block, 0, stream, tables, scale_bias, d, g_log2, CB,
                       indices, offsets, B, chunks_per_table, total, out, out_ld, out_col0);
  else if (Vneed == 2)
    hipLaunchKernelGGL((embbag_fwd_kernel<2, 4, R>), grid, block, 0, stream, tables, scale_bias, d, g_log2, CB,
                       indices, offsets, B, chunks_per_table, total, out, out_ld, out_col0);
  else
    hipLaunchKernelGGL((embbag_fwd_kernel<4, 2, R>), grid, block, 0, stream, tables, scale_bias, d, g_log2, CB,
                       indices, offsets, B, chunks_per_table, total, out, out_ld, out_col0);
  return launch_status();
}

int check_embbag_args(const void* tables, int32_t K, int32_t d, const int64_t* indices, const int64_t* offsets,
                      int64_t B, float* out, int64_t out_ld, int64_t out_col0) {
  if (!tables || !indices || !offsets || !out) return DLRM_E_INVALID;
  if (K < 1 || B < 1 || d < 4 || d > 1024 || (d % 4) != 0) return DLRM_E_INVALID;
  if (out_col0 < 0 || out_ld < out_col0 + (int64_t)K * d) return DLRM_E_INVALID;
  if (!aligned16(out) || (out_ld % 4) != 0 || (out_col0 % 4) != 0) return DLRM_E_INVALID;
  return DLRM_OK;
}
}  // namespace
}  // namespace dlrm

extern "C" int dlrm_embbag_fwd(const float* const* tables, int32_t K, int32_t d, const int64_t* indices,
                               const int64_t* offsets, int64_t B, int64_t nnz, float* out, int64_t out_ld,
                               int64_t out_col0, hipStream_t stream) {
  const int rc = check_embbag_args(tables, K, d, indices, offsets, B, out, out_ld, out_col0);
  if (rc != DLRM_OK) return rc;
  return launch_embbag<RowF32>(tables, nullptr, K, d, indices, offsets, B, nnz, out, out_ld, out_col0, stream);
}

extern "C" int dlrm_embbag_fwd_lp(const void* const* tables, int32_t table_dtype, const float* const* scale_bias,
                                  int32_t K, int32_t d, const int64_t* indices, const int64_t* offsets, int64_t B,
                                  int64_t nnz, float* out, int64_t out_ld, int64_t out_col0, hipStream_t stream) {
  const int rc = check_embbag_args(tables, K, d, indices, offsets, B, out, out_ld, out_col0);
  if (rc != DLRM_OK) return rc;
  if (table_dtype == DLRM_BF16) {
    const auto* t = reinterpret_cast<const uint16_t* const*>(tables);
    if (d % 8 == 0) return launch_embbag<RowBF16x8>(t, nullptr, K, d, indices, offsets, B, nnz, out, out_ld, out_col0, stream);
    return launch_embbag<RowBF16>(t, nullptr, K, d, indices, offsets, B, nnz, out, out_ld, out_col0, stream);
  }
  if (table_dtype == DLRM_I8) {
    if (!scale_bias) return DLRM_E_INVALID;
    const auto* t = reinterpret_cast<const int8_t* const*>(tables);
    if (d % 16 == 0)
      return launch_embbag<RowI8x16>(t, scale_bias, K, d, indices, offsets, B, nnz, out, out_ld, out_col0, stream);
    return launch_embbag<RowI8>(t, scale_bias, K, d, indices, offsets, B, nnz, out, out_ld, out_col0, stream);
  }
  return DLRM_E_INVALID;
}

extern "C" int dlrm_check_indices(const int64_t* indices, const int64_t* offsets, int32_t K, int64_t B,
                                  const int64_t* rows_dev, int64_t* bad_count, hipStream_t stream) {
  if (!indices || !offsets || !rows_dev || !bad_count || K < 1 || B < 1) return DLRM_E_INVALID;
  const int64_t bags = (int64_t)K * B;
  const int64_t blocks = ceil_div(bags, 256);
  if (blocks > 0x7fffffffLL) return DLRM_E_UNSUPPORTED;
  hipLaunchKernelGGL(check_indices_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, indices, offsets,
                     (int64_t)K, B, rows_dev, reinterpret_cast<unsigned long long*>(bad_count));
  return launch_status();
}
