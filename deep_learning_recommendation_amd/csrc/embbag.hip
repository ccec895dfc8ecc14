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

template <int V, int U>
__global__ __launch_bounds__(256) void embbag_fwd_kernel(const float* const* __restrict__ tables, int32_t d,
                                                         int32_t g_log2, int32_t CB,
                                                         const int64_t* __restrict__ idx,
                                                         const int64_t* __restrict__ off, int64_t B,
                                                         int64_t chunks_per_table, int64_t total_chunks,
                                                         float* __restrict__ out, int64_t out_ld,
                                                         int64_t out_col0) {
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
  const float* __restrict__ T = tables[k];
  const int d4 = d >> 2;

  const int64_t P0 = __shfl(my_off, gbase, 64);
  const int64_t P1 = __shfl(my_off, gbase + nb, 64);
  int cb = 0;
  int64_t cur_end = __shfl(my_off, gbase + 1, 64);
  float* obase = out + out_col0 + k * (int64_t)d;

  float4 acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);

  auto flush = [&]() {
    float* o = obase + (b0 + cb) * out_ld;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int c4 = gl + j * G;
      if (c4 < d4) *reinterpret_cast<float4*>(o + 4 * c4) = acc[j];
      acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    ++cb;
    cur_end = __shfl(my_off, gbase + min(cb + 1, nb), 64);
  };

  int64_t ridx[U];
#pragma unroll
  for (int u = 0; u < U; ++u) ridx[u] = (P0 + u < P1) ? idx[P0 + u] : 0;

  for (int64_t p = P0; p < P1; p += U) {
    float4 v[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* row = T + ridx[u] * (int64_t)d;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int c4 = gl + j * G;
        v[u][j] = (p + u < P1 && c4 < d4) ? *reinterpret_cast<const float4*>(row + 4 * c4)
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
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
        for (int j = 0; j < V; ++j) {
          acc[j].x = acc[j].x + v[u][j].x;
          acc[j].y = acc[j].y + v[u][j].y;
          acc[j].z = acc[j].z + v[u][j].z;
          acc[j].w = acc[j].w + v[u][j].w;
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

extern "C" int dlrm_embbag_fwd(const float* const* tables, int32_t K, int32_t d, const int64_t* indices,
                               const int64_t* offsets, int64_t B, int64_t nnz, float* out, int64_t out_ld,
                               int64_t out_col0, hipStream_t stream) {
  if (!tables || !indices || !offsets || !out) return DLRM_E_INVALID;
  if (K < 1 || B < 1 || d < 4 || d > 1024 || (d % 4) != 0) return DLRM_E_INVALID;
  if (out_col0 < 0 || out_ld < out_col0 + (int64_t)K * d) return DLRM_E_INVALID;
  if (!aligned16(out) || (out_ld % 4) != 0 || (out_col0 % 4) != 0) return DLRM_E_INVALID;

  const int d4 = d / 4;
  int g_log2 = 1;
  while ((1 << g_log2) < d4 && g_log2 < 6) ++g_log2;
  const int G = 1 << g_log2;
  const int Vneed = (d4 + G - 1) / G;  // 1..4
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
    hipLaunchKernelGGL((embbag_fwd_kernel<1, 8>), grid, block, 0, stream, tables, d, g_log2, CB, indices, offsets, B,
                       chunks_per_table, total, out, out_ld, out_col0);
  else if (Vneed == 2)
    hipLaunchKernelGGL((embbag_fwd_kernel<2, 4>), grid, block, 0, stream, tables, d, g_log2, CB, indices, offsets, B,
                       chunks_per_table, total, out, out_ld, out_col0);
  else
    hipLaunchKernelGGL((embbag_fwd_kernel<4, 2>), grid, block, 0, stream, tables, d, g_log2, CB, indices, offsets, B,
                       chunks_per_table, total, out, out_ld, out_col0);
  return launch_status();
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
