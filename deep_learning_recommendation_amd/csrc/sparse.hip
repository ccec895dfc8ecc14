// Sparse embedding backward with row-wise SGD, applied in place.
//
// Sum pooling hands each bag's gradient unchanged to every row the bag
// looked up, once per occurrence (the lookup of "Deep Learning
// Recommendation Model (DLRM)" explainer, Key Method Details, Embedding
// tables; training by binary cross-entropy, Key Method Details, Loss).  The
// per-row gradient must be one serial fp32 sum in position order, so the
// path is:
//   1. keys: one (table, row) key and one bag id per index position
//      (position order = table-major bag order);
//   2. a stable least-significant-digit radix sort on the keys, 8 bits per
//      pass; stability keeps equal keys in position order;
//   3. run-length segmentation (head flags, device-wide exclusive scan);
//   4. one fused kernel: each segment's gradient sum over its occurrences in
//      sorted order (fp32, from +0) and the update T <- T - lr * g.
// Hot rows (Zipf heads with 10^5 occurrences) make step 4's longest serial
// chain the latency floor; segments of at least kHot occurrences are taken
// by dedicated waves that split the row's columns one per lane and are
// dispatched before the rest.
#include "common.hpp"

namespace dlrm {
namespace {

constexpr int RT = 256;                // threads per sort block
constexpr int RITEMS = 16;             // keys per thread per tile
constexpr int RTILE = RT * RITEMS;     // 4096 keys per tile
constexpr int SCAN_ITEMS = 8;
constexpr int SCAN_TILE = 256 * SCAN_ITEMS;
constexpr int kHot = 512;              // occurrences from which a segment is "hot"
constexpr int kHeavyBlocks = 256;      // blocks (4 waves each) reserved for hot segments
constexpr int kLightBlocks = 2048;

// ------------------------------------------------------------------ keys

__global__ __launch_bounds__(256) void build_keys_kernel(const int64_t* __restrict__ idx,
                                                         const int64_t* __restrict__ off, int64_t KB, int64_t B,
                                                         int row_bits, uint32_t* __restrict__ keys,
                                                         int32_t* __restrict__ vals) {
  __shared__ int64_t s_off[257];
  const int64_t kb0 = (int64_t)blockIdx.x * 256;
  const int nb = (int)min((int64_t)256, KB - kb0);
  for (int j = threadIdx.x; j <= nb; j += blockDim.x) s_off[j] = off[kb0 + j];
  __syncthreads();
  const int64_t p0 = s_off[0], p1 = s_off[nb];
  for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    int lo = 0, hi = nb - 1;  // largest j with s_off[j] <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    const int64_t kb = kb0 + lo;
    const int64_t k = kb / B;
    keys[p] = ((uint32_t)k << row_bits) | (uint32_t)idx[p];
    vals[p] = (int32_t)(kb - k * B);
  }
}

// ------------------------------------------------------------------ radix sort

__global__ __launch_bounds__(RT) void radix_hist_kernel(const uint32_t* __restrict__ keys, int n, int shift,
                                                        uint32_t* __restrict__ hist, int nblocks) {
  __shared__ uint32_t cnt[256];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int base = blockIdx.x * RTILE;
#pragma unroll
  for (int i = 0; i < RITEMS; ++i) {
    const int p = base + i * RT + threadIdx.x;
    if (p < n) atomicAdd(&cnt[(keys[p] >> shift) & 255u], 1u);
  }
  __syncthreads();
  hist[(int64_t)threadIdx.x * nblocks + blockIdx.x] = cnt[threadIdx.x];
}

// Stable scatter: the tile is taken in RITEMS rounds of 256 consecutive keys;
// inside a round a key's rank is (keys of its digit in earlier rounds) +
// (in earlier waves of this round) + (in lower lanes of its wave), the last
// term found by matching the 8 digit bits with wave ballots.
__global__ __launch_bounds__(RT) void radix_scatter_kernel(const uint32_t* __restrict__ kin,
                                                           const int32_t* __restrict__ vin,
                                                           uint32_t* __restrict__ kout, int32_t* __restrict__ vout,
                                                           int n, int shift, const uint32_t* __restrict__ offs,
                                                           int nblocks) {
  __shared__ uint32_t run[256];
  __shared__ uint32_t wcnt[4][256];
  __shared__ uint32_t woff[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  run[tid] = offs[(int64_t)tid * nblocks + blockIdx.x];
#pragma unroll
  for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < RITEMS; ++r) {
    const int p = blockIdx.x * RTILE + r * RT + tid;
    const bool valid = p < n;
    const uint32_t key = valid ? kin[p] : 0u;
    const int32_t val = valid ? vin[p] : 0;
    const uint32_t digit = (key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (digit >> b) & 1u;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint32_t rank = (uint32_t)__popcll(peers & lt);
    if (valid && (peers & lt) == 0ull) wcnt[wave][digit] = (uint32_t)__popcll(peers);
    __syncthreads();
    {
      uint32_t acc = run[tid];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        woff[w][tid] = acc;
        acc += wcnt[w][tid];
        wcnt[w][tid] = 0;
      }
      run[tid] = acc;
    }
    __syncthreads();
    if (valid) {
      const uint32_t pos = woff[wave][digit] + rank;
      kout[pos] = key;
      vout[pos] = val;
    }
  }
}

// ------------------------------------------------------------------ scans

// block-wide exclusive scan of one value per thread (256 threads); returns
// the exclusive prefix and writes the block total to *total
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t c = s_wave[w];
    if (w < wave) before += c;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// input views for the generic scan
struct ArrayIn {
  const uint32_t* a;
  __device__ uint32_t operator()(int64_t i) const { return a[i]; }
};
struct HeadIn {  // 1 where a new run of equal keys starts
  const uint32_t* k;
  __device__ uint32_t operator()(int64_t i) const { return (i == 0 || k[i] != k[i - 1]) ? 1u : 0u; }
};

template <class In>
__global__ __launch_bounds__(256) void scan_reduce_kernel(In in, int64_t n, uint32_t* __restrict__ bsum) {
  __shared__ uint32_t s_wave[4];
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i)
    if (base + i < n) s += in(base + i);
  uint32_t total;
  block_exclusive_scan(s, s_wave, &total);
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// single block: exclusive scan of bsum[0..nb) in place, total to *total_out
__global__ __launch_bounds__(256) void scan_top_kernel(uint32_t* __restrict__ bsum, int nb,
                                                       uint32_t* __restrict__ total_out) {
  __shared__ uint32_t s_wave[4];
  __shared__ uint32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nb; base += 256) {
    const int i = base + threadIdx.x;
    const uint32_t v = i < nb ? bsum[i] : 0u;
    uint32_t total;
    const uint32_t ex = block_exclusive_scan(v, s_wave, &total);
    const uint32_t c = carry;
    if (i < nb) bsum[i] = c + ex;
    __syncthreads();
    if (threadIdx.x == 0) carry = c + total;
    __syncthreads();
  }
  if (threadIdx.x == 0 && total_out) *total_out = carry;
}

// out[i] = exclusive prefix (array mode)
__global__ __launch_bounds__(256) void scan_apply_array_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                               const uint32_t* __restrict__ bsum,
                                                               uint32_t* __restrict__ out) {
  __shared__ uint32_t s_wave[4];
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
  uint32_t v[SCAN_ITEMS], s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    v[i] = (base + i < n) ? in[base + i] : 0u;
    s += v[i];
  }
  uint32_t total;
  uint32_t run = bsum[blockIdx.x] + block_exclusive_scan(s, s_wave, &total);
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    if (base + i < n) out[base + i] = run;
    run += v[i];
  }
}

// seg_start[run id] = position of each run head; seg_start[U] = n
__global__ __launch_bounds__(256) void scan_apply_heads_kernel(const uint32_t* __restrict__ keys, int64_t n,
                                                               const uint32_t* __restrict__ bsum,
                                                               int32_t* __restrict__ seg_start,
                                                               const uint32_t* __restrict__ nseg) {
  __shared__ uint32_t s_wave[4];
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
  HeadIn h{keys};
  uint32_t v[SCAN_ITEMS], s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    v[i] = (base + i < n) ? h(base + i) : 0u;
    s += v[i];
  }
  uint32_t total;
  uint32_t run = bsum[blockIdx.x] + block_exclusive_scan(s, s_wave, &total);
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    if (v[i]) seg_start[run] = (int32_t)(base + i);
    run += v[i];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) seg_start[*nseg] = (int32_t)n;
}

__global__ __launch_bounds__(256) void find_hot_kernel(const int32_t* __restrict__ seg_start,
                                                       const uint32_t* __restrict__ nseg, int32_t* __restrict__ hot,
                                                       uint32_t* __restrict__ nhot) {
  const uint32_t U = *nseg;
  for (uint32_t s = blockIdx.x * blockDim.x + threadIdx.x; s < U; s += gridDim.x * blockDim.x) {
    if (seg_start[s + 1] - seg_start[s] >= kHot) hot[atomicAdd(nhot, 1u)] = (int32_t)s;
  }
}

// ------------------------------------------------------------------ reduce + SGD

template <int V>
__global__ __launch_bounds__(256) void segment_sgd_kernel(float* const* __restrict__ tables, int d, int g_log2,
                                                          int row_bits, const uint32_t* __restrict__ keys,
                                                          const int32_t* __restrict__ bags,
                                                          const int32_t* __restrict__ seg_start,
                                                          const uint32_t* __restrict__ nseg,
                                                          const int32_t* __restrict__ hot,
                                                          const uint32_t* __restrict__ nhot,
                                                          const float* __restrict__ G, int64_t g_ld, int64_t g_col0,
                                                          float lr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t row_mask = (row_bits >= 32) ? 0xffffffffu : ((1u << row_bits) - 1u);
  if (blockIdx.x < kHeavyBlocks) {
    // hot segments: one wave per (segment, 64-column slice), one column per lane
    const int slices = (d + 63) / 64;
    const uint32_t items = *nhot * (uint32_t)slices;
    for (uint32_t it = blockIdx.x * 4 + wave; it < items; it += kHeavyBlocks * 4) {
      const int32_t s = hot[it / slices];
      const int col = (int)(it % slices) * 64 + lane;
      const int32_t beg = seg_start[s], end = seg_start[s + 1];
      const uint32_t key = keys[beg];
      const int k = (int)(key >> row_bits);
      const int64_t r = (int64_t)(key & row_mask);
      if (col < d) {
        const float* gcol = G + g_col0 + (int64_t)k * d + col;
        float acc = 0.f;
        int32_t q = beg;
        for (; q + 8 <= end; q += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = gcol[(int64_t)bags[q + u] * g_ld];
#pragma unroll
          for (int u = 0; u < 8; ++u) acc = acc + v[u];
        }
        for (; q < end; ++q) acc = acc + gcol[(int64_t)bags[q] * g_ld];
        float* t = tables[k] + r * d + col;
        *t = __fsub_rn(*t, __fmul_rn(lr, acc));
      }
    }
    return;
  }
  // all other segments: a group of G lanes (float4 each) per segment
  const int GL = 1 << g_log2;  // lanes per group
  const int gl = lane & (GL - 1);
  const int groups_per_block = 256 >> g_log2;
  const int64_t gid = (int64_t)(blockIdx.x - kHeavyBlocks) * groups_per_block + (threadIdx.x >> g_log2);
  const int64_t ngroups = (int64_t)(gridDim.x - kHeavyBlocks) * groups_per_block;
  const int d4 = d >> 2;
  const uint32_t U = *nseg;
  for (int64_t s = gid; s < U; s += ngroups) {
    const int32_t beg = seg_start[s], end = seg_start[s + 1];
    if (end - beg >= kHot) continue;
    const uint32_t key = keys[beg];
    const int k = (int)(key >> row_bits);
    const int64_t r = (int64_t)(key & row_mask);
    float4* trow = reinterpret_cast<float4*>(tables[k] + r * d);
    float4 tv[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int c4 = gl + j * GL;
      tv[j] = c4 < d4 ? trow[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float* gbase = G + g_col0 + (int64_t)k * d;
    float4 acc[V];
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int U = 8 / V;
    for (int32_t q = beg; q < end; q += U) {
      float4 v[U][V];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = q + u < end;
        const int64_t bag = ok ? (int64_t)bags[q + u] : 0;
        const float4* grow = reinterpret_cast<const float4*>(gbase + bag * g_ld);
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const int c4 = gl + j * GL;
          v[u][j] = (ok && c4 < d4) ? grow[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (q + u < end) {
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
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int c4 = gl + j * GL;
      if (c4 < d4) {
        float4 o;
        o.x = __fsub_rn(tv[j].x, __fmul_rn(lr, acc[j].x));
        o.y = __fsub_rn(tv[j].y, __fmul_rn(lr, acc[j].y));
        o.z = __fsub_rn(tv[j].z, __fmul_rn(lr, acc[j].z));
        o.w = __fsub_rn(tv[j].w, __fmul_rn(lr, acc[j].w));
        trow[c4] = o;
      }
    }
  }
}

int bits_for(int64_t x) {  // bits needed to hold 0..x
  int b = 0;
  while (b < 63 && (x >> b) != 0) ++b;
  return b;
}

struct SparseLayout {
  size_t keys[2], vals[2], hist, bsum, seg, counters, hot, bytes;
  int64_t nblocks, hist_n, scan_nb_hist, scan_nb_keys;
};

void sparse_layout(int64_t nnz, SparseLayout* L) {
  Carver cv(nullptr);
  auto take = [&](size_t bytes) {
    cv.used = (size_t)round_up((int64_t)cv.used, 256);
    const size_t at = cv.used;
    cv.used += bytes;
    return at;
  };
  const int64_t n = nnz > 0 ? nnz : 1;
  L->nblocks = ceil_div(n, RTILE);
  L->hist_n = 256 * L->nblocks;
  L->scan_nb_hist = ceil_div(L->hist_n, SCAN_TILE);
  L->scan_nb_keys = ceil_div(n, SCAN_TILE);
  L->keys[0] = take(4 * (size_t)n);
  L->keys[1] = take(4 * (size_t)n);
  L->vals[0] = take(4 * (size_t)n);
  L->vals[1] = take(4 * (size_t)n);
  L->hist = take(4 * (size_t)L->hist_n);
  const int64_t nb = L->scan_nb_hist > L->scan_nb_keys ? L->scan_nb_hist : L->scan_nb_keys;
  L->bsum = take(4 * (size_t)nb);
  L->seg = take(4 * (size_t)(n + 1));
  L->counters = take(4 * 16);
  L->hot = take(4 * (size_t)(n / kHot + 1));
  L->bytes = cv.bytes();
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

}  // namespace
}  // namespace dlrm

using namespace dlrm;

extern "C" size_t dlrm_embbag_bwd_sgd_workspace_size(int32_t K, int64_t B, int64_t nnz, int32_t d) {
  (void)K;
  (void)B;
  (void)d;
  if (nnz < 0) return 0;
  SparseLayout L;
  sparse_layout(nnz, &L);
  return L.bytes;
}

extern "C" int dlrm_embbag_bwd_sgd(float* const* tables, int32_t K, int32_t d, const int64_t* rows,
                                   const int64_t* indices, const int64_t* offsets, int64_t B, int64_t nnz,
                                   const float* G, int64_t g_ld, int64_t g_col0, float lr, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!tables || !rows || !indices || !offsets || !G) return DLRM_E_INVALID;
  if (K < 1 || B < 1 || d < 4 || d > 1024 || (d % 4) != 0) return DLRM_E_INVALID;
  if (nnz < 0 || nnz > 0x7fffffffLL || B > 0x7fffffffLL) return DLRM_E_INVALID;
  if (g_col0 < 0 || g_ld < g_col0 + (int64_t)K * d || (g_ld % 4) != 0 || (g_col0 % 4) != 0 || !aligned16(G))
    return DLRM_E_INVALID;
  int64_t max_rows = 1;
  for (int k = 0; k < K; ++k) {
    if (rows[k] < 1) return DLRM_E_INVALID;
    max_rows = rows[k] > max_rows ? rows[k] : max_rows;
  }
  const int row_bits = bits_for(max_rows - 1) > 0 ? bits_for(max_rows - 1) : 1;
  const int table_bits = bits_for(K - 1);
  if (row_bits + table_bits > 32) return DLRM_E_UNSUPPORTED;
  if (nnz == 0) return DLRM_OK;
  SparseLayout L;
  sparse_layout(nnz, &L);
  if (!ws || ws_bytes < L.bytes) return DLRM_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return DLRM_E_INVALID;
  char* w = static_cast<char*>(ws);
  uint32_t* keys[2] = {reinterpret_cast<uint32_t*>(w + L.keys[0]), reinterpret_cast<uint32_t*>(w + L.keys[1])};
  int32_t* vals[2] = {reinterpret_cast<int32_t*>(w + L.vals[0]), reinterpret_cast<int32_t*>(w + L.vals[1])};
  uint32_t* hist = reinterpret_cast<uint32_t*>(w + L.hist);
  uint32_t* bsum = reinterpret_cast<uint32_t*>(w + L.bsum);
  int32_t* seg = reinterpret_cast<int32_t*>(w + L.seg);
  uint32_t* counters = reinterpret_cast<uint32_t*>(w + L.counters);  // [0] segments, [1] hot segments
  int32_t* hot = reinterpret_cast<int32_t*>(w + L.hot);
  const int n = (int)nnz;
  const int64_t KB = (int64_t)K * B;

  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, counters, 16);
  hipLaunchKernelGGL(build_keys_kernel, dim3((unsigned)ceil_div(KB, 256)), dim3(256), 0, stream, indices, offsets, KB,
                     B, row_bits, keys[0], vals[0]);
  const int key_bits = row_bits + table_bits;
  const int passes = (key_bits + 7) / 8;
  const int nblocks = (int)L.nblocks;
  int cur = 0;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * 8;
    hipLaunchKernelGGL(radix_hist_kernel, dim3(nblocks), dim3(RT), 0, stream, keys[cur], n, shift, hist, nblocks);
    hipLaunchKernelGGL((scan_reduce_kernel<ArrayIn>), dim3((unsigned)L.scan_nb_hist), dim3(256), 0, stream,
                       ArrayIn{hist}, L.hist_n, bsum);
    hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(256), 0, stream, bsum, (int)L.scan_nb_hist, nullptr);
    hipLaunchKernelGGL(scan_apply_array_kernel, dim3((unsigned)L.scan_nb_hist), dim3(256), 0, stream, hist, L.hist_n,
                       bsum, hist);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(nblocks), dim3(RT), 0, stream, keys[cur], vals[cur], keys[cur ^ 1],
                       vals[cur ^ 1], n, shift, hist, nblocks);
    cur ^= 1;
  }
  // run-length segmentation of the sorted keys
  hipLaunchKernelGGL((scan_reduce_kernel<HeadIn>), dim3((unsigned)L.scan_nb_keys), dim3(256), 0, stream,
                     HeadIn{keys[cur]}, (int64_t)n, bsum);
  hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(256), 0, stream, bsum, (int)L.scan_nb_keys, &counters[0]);
  hipLaunchKernelGGL(scan_apply_heads_kernel, dim3((unsigned)L.scan_nb_keys), dim3(256), 0, stream, keys[cur],
                     (int64_t)n, bsum, seg, &counters[0]);
  hipLaunchKernelGGL(find_hot_kernel, dim3(1024), dim3(256), 0, stream, seg, &counters[0], hot, &counters[1]);
  // per-segment sums and the in-place update
  const int d4 = d / 4;
  int g_log2 = 0;
  while ((1 << g_log2) < d4 && g_log2 < 6) ++g_log2;
  const int V = (d4 + (1 << g_log2) - 1) >> g_log2;
  const dim3 grid(kHeavyBlocks + kLightBlocks), block(256);
  if (V == 1)
    hipLaunchKernelGGL((segment_sgd_kernel<1>), grid, block, 0, stream, tables, d, g_log2, row_bits, keys[cur],
                       vals[cur], seg, &counters[0], hot, &counters[1], G, g_ld, g_col0, lr);
  else if (V == 2)
    hipLaunchKernelGGL((segment_sgd_kernel<2>), grid, block, 0, stream, tables, d, g_log2, row_bits, keys[cur],
                       vals[cur], seg, &counters[0], hot, &counters[1], G, g_ld, g_col0, lr);
  else
    hipLaunchKernelGGL((segment_sgd_kernel<4>), grid, block, 0, stream, tables, d, g_log2, row_bits, keys[cur],
                       vals[cur], seg, &counters[0], hot, &counters[1], G, g_ld, g_col0, lr);
  return launch_status();
}
