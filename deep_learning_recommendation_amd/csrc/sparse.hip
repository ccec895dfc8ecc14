// Sparse embedding backward with row-wise SGD, applied in place.
//
// Sum pooling hands each bag's gradient unchanged to every row the bag
// looked up, once per occurrence (the lookup of "Deep Learning
// Recommendation Model (DLRM)" explainer, Key Method Details, Embedding
// tables; training by binary cross-entropy, Key Method Details, Loss).  A
// row's gradient is the fp32 sum of its occurrences' gradients in a fixed
// order: position order, in blocks of kHot = 128 occurrences (each block
// summed from +0, then the block sums in order; up to 129 occurrences that
// is the plain left-to-right sum).  The path:
//   1. keys: one (table, row) key and one bag id per index position
//      (position order = table-major bag order);
//   2. a stable least-significant-digit radix sort over the row bits of the
//      keys (8 or 9 bits per pass); stability keeps equal keys in position
//      order, and since positions are table-major, equal rows of different
//      tables stay in table order, so every (table, row) key forms one run;
//   3. run-length segmentation (head flags, device-wide exclusive scan); runs
//      of at least kHot occurrences ("hot", the Zipf heads with up to 10^5
//      occurrences) are listed apart;
//   4. the sums and the update T <- T - lr * g: short runs one lane group
//      each, in sorted order; hot runs in three steps, their block list
//      (with the index work of steps 1-3), their blocks' sums in parallel
//      (one lane group per block), then per run the block sums in order and
//      the update.  The blocked order keeps a 10^5-occurrence row
//      from being one serial chain of 10^5 dependent adds.
#include "common.hpp"

#include <mutex>

namespace dlrm {
namespace {

constexpr int RT = 256;                // threads per sort block
constexpr int ITEMS = 16;              // keys per thread per tile
constexpr int TILE = RT * ITEMS;       // 4096 positions per tile
constexpr int kMaxDigits = 512;        // buckets of a digit of at most 9 bits
constexpr int kHot = 128;              // occurrences from which a segment is "hot", and its block size
// Persistent blocks of the short-segment kernel and of the hot-run kernels:
// four and two per CU.  In a training step the update runs beside the MLP
// GEMMs, whose workgroups find room only where these leave it; twice as many
// blocks made each update alone under 1% faster but the training step 1-2%
// slower (1.245 -> 1.233 ms with the synthetic gradient, 1.297 -> 1.285 ms
// for the whole chain, 2.72 -> 2.67 ms with uniform indices); fewer (768 /
// 384) slowed the uniform-index update by 15%.
constexpr int kLightBlocks = 1024;
constexpr int kHotBlocks = 512;

// ------------------------------------------------------------------ keys

// One group of G lanes per bag (G about the mean bag length, at most 64):
// the group walks the bag's positions with stride G, so the index reads and
// the key and bag-id writes of a wave are contiguous runs.
__global__ __launch_bounds__(256) void build_keys_kernel(const int64_t* __restrict__ idx,
                                                         const int64_t* __restrict__ off, int64_t KB, int64_t B,
                                                         int g_log2, int row_bits, uint32_t* __restrict__ keys,
                                                         int32_t* __restrict__ vals) {
  const int G = 1 << g_log2;
  const int64_t bag = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> g_log2;
  if (bag >= KB) return;  // whole group
  const int gl = threadIdx.x & (G - 1);
  const int64_t a = off[bag], e = off[bag + 1];
  const int64_t k = bag / B;
  const uint32_t hi = (uint32_t)k << row_bits;
  const int32_t b = (int32_t)(bag - k * B);
#pragma unroll 4
  for (int64_t p = a + gl; p < e; p += G) {
    keys[p] = hi | (uint32_t)idx[p];
    vals[p] = b;
  }
}

// ------------------------------------------------------------------ radix sort
//
// A pass is four kernels without any waiting between blocks: the per-tile
// digit counts (tile_hist_kernel, counts[tile][digit]); their sums over
// chunks of 64 tiles (chunk_sum_kernel); the offsets, each (tile, digit)'s
// first position = the digit's start (the totals of the digits below it) +
// the digit's count in earlier chunks + in earlier tiles of its chunk
// (tile_offset_kernel); and the stable scatter of each tile
// (scatter_kernel), which ranks its keys with wave ballots and writes them
// through LDS in digit order, so each digit's keys of a tile leave as one
// contiguous span.
constexpr int kChunk = 64;  // tiles per chunk of the offset scan

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

// Tile t's keys: wave w holds positions w * 1024 + 64 i + lane of the tile
// (item i), the layout the scatter ranks in.
__device__ __forceinline__ int tile_pos(int wave, int i, int lane) { return wave * (TILE / 4) + 64 * i + lane; }

// counts[tile][digit] of one pass (per-wave LDS counters).
template <int DB>
__global__ __launch_bounds__(RT) void tile_hist_kernel(const uint32_t* __restrict__ keys, int n, int shift,
                                                       uint32_t* __restrict__ counts, int tiles) {
  constexpr int NB = 1 << DB;
  __shared__ uint32_t cnt[4][NB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4 * NB; i += RT) (&cnt[0][0])[i] = 0u;
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * TILE;
  const int cnt_n = (int)(n - t0 < TILE ? n - t0 : TILE);
  uint32_t key[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int q = tile_pos(wave, i, lane);
    key[i] = q < cnt_n ? keys[t0 + q] : 0u;
  }
#pragma unroll
  for (int i = 0; i < ITEMS; ++i)
    if (tile_pos(wave, i, lane) < cnt_n) atomicAdd(&cnt[wave][(key[i] >> shift) & (uint32_t)(NB - 1)], 1u);
  __syncthreads();
  for (int dg = tid; dg < NB; dg += RT)
    counts[(int64_t)blockIdx.x * NB + dg] = cnt[0][dg] + cnt[1][dg] + cnt[2][dg] + cnt[3][dg];
}

// sums[chunk][digit] = the digit's count over the chunk's tiles: block
// (chunk, 64-digit group), lane = digit, wave w takes 16 of the 64 tiles.
template <int DB>
__global__ __launch_bounds__(RT) void chunk_sum_kernel(const uint32_t* __restrict__ counts, int tiles,
                                                       uint32_t* __restrict__ sums) {
  constexpr int NB = 1 << DB;
  __shared__ uint32_t part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int dg = blockIdx.y * 64 + lane;
  const int t0 = blockIdx.x * kChunk + wave * (kChunk / 4);
  uint32_t v[kChunk / 4];
#pragma unroll
  for (int i = 0; i < kChunk / 4; ++i) v[i] = t0 + i < tiles ? counts[(int64_t)(t0 + i) * NB + dg] : 0u;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kChunk / 4; ++i) s += v[i];
  part[wave][lane] = s;
  __syncthreads();
  if (wave == 0) sums[(int64_t)blockIdx.x * NB + dg] = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
}

// sum of col[0], col[stride], ..., col[(rows - 1) stride], eight loads in flight
__device__ __forceinline__ uint32_t column_sum(const uint32_t* __restrict__ col, int64_t stride, int rows) {
  uint32_t t = 0;
  for (int r0 = 0; r0 < rows; r0 += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = r0 + u < rows ? col[(int64_t)(r0 + u) * stride] : 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) t += v[u];
  }
  return t;
}

// offsets[tile][digit] for the tiles of chunk blockIdx.x and the digits of
// group blockIdx.y: the digit totals (all chunk sums: every block redoes
// the sums and their exclusive scan over digits), the digit's count in
// earlier chunks, then in earlier tiles of the chunk (wave w: tiles
// 16 w .. 16 w + 15, after the three waves before it).
template <int DB>
__global__ __launch_bounds__(RT) void tile_offset_kernel(const uint32_t* __restrict__ counts,
                                                         const uint32_t* __restrict__ sums, int tiles,
                                                         uint32_t* __restrict__ offsets) {
  constexpr int NB = 1 << DB, DPT = NB / RT;
  __shared__ uint32_t s_wave[4];
  __shared__ uint32_t dstart[NB];
  __shared__ uint32_t part[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunks = (tiles + kChunk - 1) / kChunk;
  const int chunk = blockIdx.x;
  // digit totals and starts (thread: digits DPT tid .. DPT tid + DPT - 1)
  uint32_t tot[DPT];
  uint32_t tsum = 0;
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    tot[j] = column_sum(sums + tid * DPT + j, NB, chunks);
    tsum += tot[j];
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan(tsum, s_wave, &total);
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    dstart[tid * DPT + j] = run;
    run += tot[j];
  }
  __syncthreads();
  const int dg = blockIdx.y * 64 + lane;
  uint32_t base = dstart[dg] + column_sum(sums + dg, NB, chunk);
  const int t0 = chunk * kChunk + wave * (kChunk / 4);
  uint32_t v[kChunk / 4];
#pragma unroll
  for (int i = 0; i < kChunk / 4; ++i) v[i] = t0 + i < tiles ? counts[(int64_t)(t0 + i) * NB + dg] : 0u;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kChunk / 4; ++i) s += v[i];
  part[wave][lane] = s;
  __syncthreads();
  for (int w = 0; w < wave; ++w) base += part[w][lane];
#pragma unroll
  for (int i = 0; i < kChunk / 4; ++i) {
    if (t0 + i < tiles) offsets[(int64_t)(t0 + i) * NB + dg] = base;
    base += v[i];
  }
}

// One pass: stable scatter of tile blockIdx.x by the digit at `shift`.  The
// rank of a key is (its digit's count in earlier waves) + (in earlier items
// of its wave) + (in lower lanes of its item), the last from DB ballots.
template <int DB>
__global__ __launch_bounds__(RT) void scatter_kernel(const uint32_t* __restrict__ kin, const int32_t* __restrict__ vin,
                                                     uint32_t* __restrict__ kout, int32_t* __restrict__ vout, int n,
                                                     int shift, const uint32_t* __restrict__ offsets, int tiles) {
  constexpr int NB = 1 << DB, DPT = NB / RT;  // digits per thread (contiguous)
  __shared__ uint32_t wcnt[4][NB];           // per-wave counts, then per-wave offsets
  __shared__ uint32_t lstart[NB];            // tile-local start of each digit
  __shared__ uint32_t gbase[NB];             // global position of a digit's span minus its tile-local start
  __shared__ uint32_t lkeys[TILE];
  __shared__ int32_t lvals[TILE];
  __shared__ uint32_t s_wave[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  for (int i = tid; i < 4 * NB; i += RT) (&wcnt[0][0])[i] = 0u;
  __syncthreads();
  const int64_t t0 = (int64_t)tile * TILE;
  const int cnt = (int)(n - t0 < TILE ? n - t0 : TILE);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t key[ITEMS];
  int32_t val[ITEMS];
  uint32_t rank[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int q = tile_pos(wave, i, lane);
    key[i] = q < cnt ? kin[t0 + q] : 0u;
    val[i] = q < cnt ? vin[t0 + q] : 0;
  }
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const bool valid = tile_pos(wave, i, lane) < cnt;
    const uint32_t dg = (key[i] >> shift) & (uint32_t)(NB - 1);
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const bool bit = (dg >> b) & 1u;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    // every lane reads the count before its group's lowest lane adds to it
    const uint32_t before = valid ? wcnt[wave][dg] : 0u;
    rank[i] = before + (uint32_t)__popcll(peers & below);
    if (valid && (peers & below) == 0ull) wcnt[wave][dg] = before + (uint32_t)__popcll(peers);
  }
  __syncthreads();
  uint32_t tc[DPT];
  uint32_t tsum = 0;
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int dg = tid * DPT + j;
    uint32_t run = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t c = wcnt[w][dg];
      wcnt[w][dg] = run;
      run += c;
    }
    tc[j] = run;
    tsum += run;
  }
  uint32_t total;
  uint32_t lrun = block_exclusive_scan(tsum, s_wave, &total);
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int dg = tid * DPT + j;
    lstart[dg] = lrun;
    gbase[dg] = offsets[(int64_t)tile * NB + dg] - lrun;
    lrun += tc[j];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (tile_pos(wave, i, lane) < cnt) {
      const uint32_t dg = (key[i] >> shift) & (uint32_t)(NB - 1);
      const uint32_t lp = lstart[dg] + wcnt[wave][dg] + rank[i];
      lkeys[lp] = key[i];
      lvals[lp] = val[i];
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int j = tid; j < cnt; j += RT) {
    const uint32_t k = lkeys[j];
    const uint32_t pos = gbase[(k >> shift) & (uint32_t)(NB - 1)] + (uint32_t)j;
    kout[pos] = k;
    vout[pos] = lvals[j];
  }
}

// ------------------------------------------------------------------ segments
//
// Run-length segmentation of the sorted keys, the same three steps: run
// heads per tile (heads_count_kernel), their exclusive scan over tiles
// (heads_scan_kernel: the run count to counters[0], seg_start[runs] = n),
// and seg_start[run] / seg_key[run] at every head (heads_write_kernel).  A
// head whose key is still there kHot - 1 positions later starts a hot run;
// its length class floor(log2(length)) follows from probes at 2^j - 1
// positions after the head (the run is contiguous), and the run joins the
// list of its class.  The update takes hot runs class by class, longest
// class first, so the longest serial chains start first.
constexpr int kHotClassMin = 7;   // 2^7 = kHot
constexpr int kHotClassMax = 30;  // runs shorter than 2^31
static_assert((1 << kHotClassMin) == kHot, "hot runs start at class kHotClassMin");
constexpr int kHotCountBase = 16;  // counters[kHotCountBase + class]: hot runs of each class

// first slot of class c's list: the classes below it hold at most
// n >> c' + 1 runs each
__host__ __device__ inline int64_t hot_class_base(int64_t n, int c) {
  int64_t b = 0;
  for (int q = kHotClassMin; q < c; ++q) b += (n >> q) + 1;
  return b;
}

// head ballots of a tile: item i of wave w is position w * 1024 + 64 i + lane;
// the key before a position comes from the lane below (lane 0: from lane 63
// of the item before, or memory for the wave's first position)
__device__ __forceinline__ void tile_heads(const uint32_t* __restrict__ keys, int n, int64_t t0, int cnt,
                                           uint32_t (&key)[ITEMS], uint64_t (&head)[ITEMS]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int q = tile_pos(wave, i, lane);
    key[i] = q < cnt ? keys[t0 + q] : 0u;
  }
  const int64_t p0 = t0 + tile_pos(wave, 0, 0);
  const uint32_t first_prev = (lane == 0 && p0 > 0 && p0 - t0 < cnt) ? keys[p0 - 1] : 0u;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int q = tile_pos(wave, i, lane);
    const uint32_t up = (uint32_t)__shfl_up((int)key[i], 1, 64);
    const uint32_t wrap = i > 0 ? (uint32_t)__shfl((int)key[i > 0 ? i - 1 : 0], 63, 64) : first_prev;
    const uint32_t prev = lane > 0 ? up : wrap;
    const bool h = q < cnt && (t0 + q == 0 || prev != key[i]);
    head[i] = __ballot(h);
  }
}

__global__ __launch_bounds__(RT) void heads_count_kernel(const uint32_t* __restrict__ keys, int n,
                                                         uint32_t* __restrict__ tile_runs) {
  __shared__ uint32_t s_wcnt[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TILE;
  const int cnt = (int)(n - t0 < TILE ? n - t0 : TILE);
  uint32_t key[ITEMS];
  uint64_t head[ITEMS];
  tile_heads(keys, n, t0, cnt, key, head);
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) c += (uint32_t)__popcll(head[i]);
  if (lane == 0) s_wcnt[wave] = c;
  __syncthreads();
  if (threadIdx.x == 0) tile_runs[blockIdx.x] = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
}

// one block: exclusive scan of the tiles' run counts in place
__global__ __launch_bounds__(RT) void heads_scan_kernel(uint32_t* __restrict__ tile_runs, int tiles, int n,
                                                        int32_t* __restrict__ seg_start,
                                                        uint32_t* __restrict__ counters) {
  __shared__ uint32_t s_wave[4];
  uint32_t carry = 0;
  for (int base = 0; base < tiles; base += RT) {
    const int i = base + threadIdx.x;
    const uint32_t v = i < tiles ? tile_runs[i] : 0u;
    uint32_t total;
    const uint32_t ex = block_exclusive_scan(v, s_wave, &total);
    if (i < tiles) tile_runs[i] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) {
    counters[0] = carry;
    seg_start[carry] = n;
  }
}

__global__ __launch_bounds__(RT) void heads_write_kernel(const uint32_t* __restrict__ keys, int n,
                                                         const uint32_t* __restrict__ tile_runs,
                                                         int32_t* __restrict__ seg_start,
                                                         uint32_t* __restrict__ seg_key, int32_t* __restrict__ hot,
                                                         uint32_t* __restrict__ counters) {
  __shared__ uint32_t s_wcnt[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TILE;
  const int cnt = (int)(n - t0 < TILE ? n - t0 : TILE);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t key[ITEMS];
  uint64_t head[ITEMS];
  tile_heads(keys, n, t0, cnt, key, head);
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) c += (uint32_t)__popcll(head[i]);
  if (lane == 0) s_wcnt[wave] = c;
  __syncthreads();
  uint32_t run = tile_runs[blockIdx.x];
  for (int w = 0; w < wave; ++w) run += s_wcnt[w];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int64_t p = t0 + tile_pos(wave, i, lane);
    const bool h = (head[i] >> lane) & 1ull;
    const uint32_t r = run + (uint32_t)__popcll(head[i] & below);
    run += (uint32_t)__popcll(head[i]);
    bool is_hot = false;
    if (h) {
      seg_start[r] = (int32_t)p;
      seg_key[r] = key[i];
      is_hot = p + kHot - 1 < n && keys[p + kHot - 1] == key[i];
    }
    // each hot run's class: len >= 2^j exactly for j <= floor(log2 len), so
    // the class is kHotClassMin plus the number of matching probes 2^j - 1
    // positions on (lane j - kHotClassMin - 1 probes j, all at once)
    uint64_t hm = __ballot(is_hot);
    while (hm) {
      const int src = __ffsll((long long)hm) - 1;
      hm &= hm - 1;
      const int64_t hp = t0 + tile_pos(wave, i, src);
      const uint32_t hk = (uint32_t)__shfl((int)key[i], src, 64);
      const int j = kHotClassMin + 1 + lane;
      const int64_t q = hp + (1ll << (j < 62 ? j : 62)) - 1;
      const bool match = j <= kHotClassMax && q < n && keys[q] == hk;
      const int cls = kHotClassMin + (int)__popcll(__ballot(match));
      if (lane == src) {
        const uint32_t at = atomicAdd(&counters[kHotCountBase + cls], 1u);
        hot[hot_class_base(n, cls) + at] = (int32_t)r;
      }
    }
  }
}

// ------------------------------------------------------------------ reduce + SGD

// Short segments (per wave).  A wave takes 64 consecutive segments at a
// time, its first chunk fixed and the others from a shared counter (waves
// that start early and late share the work as they come), and loads what
// every one of them needs first at once, one segment
// per lane: its start, end and key, then the bag of its first occurrence.
// A group of 2^g_log2 lanes (V float4 of a row each) then takes its share
// of the 64 segments kLightBatch at a time: the table rows and the first
// gradient rows of the batch are in flight together (most short segments
// have one occurrence: that is all they need), then each segment's further
// occurrences follow in order, up to one bag id per lane loaded at once and
// U gradient rows in flight, each bag id broadcast from its lane.  (Batches
// of 2 and 4 segments measured slower on the training workload: the
// registers they hold cut the waves per SIMD from 7 to 3.)
constexpr int kLightBatch = 1;
template <int V, int U>
__device__ __forceinline__ void light_phase(float* const* __restrict__ tables, int d, int g_log2, int row_bits,
                                            const uint32_t* __restrict__ seg_key, const int32_t* __restrict__ bags,
                                            const int32_t* __restrict__ seg_start,
                                            const uint32_t* __restrict__ nseg, const float* __restrict__ G,
                                            int64_t g_ld, int64_t g_col0, float lr, uint32_t* __restrict__ next) {
  const int lane = threadIdx.x & 63;
  const uint32_t row_mask = (row_bits >= 32) ? 0xffffffffu : ((1u << row_bits) - 1u);
  const int GL = 1 << g_log2;  // lanes per group
  const int gl = lane & (GL - 1);
  const int wgroups = 64 >> g_log2;  // groups per wave
  const int grp = lane >> g_log2;
  const int per_group = 64 / wgroups;  // segments of a chunk per group
  const int d4 = d >> 2;
  const uint32_t nsegs = *nseg;
  // a wave's first chunk is fixed (wave w: chunk w), the rest come from the
  // shared counter after all first chunks: same-address atomics queue at
  // the cache, one every few nanoseconds, so one per chunk would have set a
  // floor of its own
  const uint32_t waves = gridDim.x * (blockDim.x >> 6);
  uint32_t c0 = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 64u;
  for (bool first = true;; first = false) {
    if (!first) {
      uint32_t c = 0;
      if (lane == 0) c = atomicAdd(next, 64u);
      c0 = (uint32_t)__shfl((int)c, 0, 64) + waves * 64u;
    }
    if (c0 >= nsegs) break;  // whole wave
    // lane i: segment c0 + i
    const uint32_t ms = c0 + (uint32_t)lane;
    const bool mvalid = ms < nsegs;
    const int32_t mbeg = mvalid ? seg_start[ms] : 0;
    const int32_t mend = mvalid ? seg_start[ms + 1] : 0;
    const uint32_t mkey = mvalid ? seg_key[ms] : 0u;
    const bool mlight = mvalid && mend - mbeg < kHot;
    const int32_t mbag0 = mlight ? bags[mbeg] : 0;
    for (int r0 = 0; r0 < per_group; r0 += kLightBatch) {
      // the batch: segments grp + (r0 + j) * wgroups of the chunk
      int32_t beg[kLightBatch], len[kLightBatch];
      float4* trow[kLightBatch];
      const float* gbase[kLightBatch];
      float4 tv[kLightBatch][V], g0[kLightBatch][V];
#pragma unroll
      for (int j = 0; j < kLightBatch; ++j) {
        const int src = grp + (r0 + j) * wgroups;
        const bool in = r0 + j < per_group;
        const int sl = in ? src : 0;
        beg[j] = __shfl(mbeg, sl, 64);
        const int32_t e = __shfl(mend, sl, 64);
        const uint32_t key = (uint32_t)__shfl((int)mkey, sl, 64);
        const bool light = in && __shfl((int)mlight, sl, 64) != 0;
        const int32_t bag0 = __shfl(mbag0, sl, 64);
        len[j] = light ? e - beg[j] : 0;
        const int k = (int)(key >> row_bits);
        const int64_t r = (int64_t)(key & row_mask);
        trow[j] = reinterpret_cast<float4*>(tables[light ? k : 0] + r * d);
        gbase[j] = G + g_col0 + (int64_t)k * d;
        const float4* grow = reinterpret_cast<const float4*>(gbase[j] + (int64_t)bag0 * g_ld);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int c4 = gl + v * GL;
          const bool ok = light && c4 < d4;
          tv[j][v] = ok ? trow[j][c4] : make_float4(0.f, 0.f, 0.f, 0.f);
          g0[j][v] = ok ? grow[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int j = 0; j < kLightBatch; ++j) {
        if (len[j] == 0) continue;  // whole group
        float4 acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {  // the sum starts from +0
          acc[v].x = 0.f + g0[j][v].x;
          acc[v].y = 0.f + g0[j][v].y;
          acc[v].z = 0.f + g0[j][v].z;
          acc[v].w = 0.f + g0[j][v].w;
        }
        for (int32_t q0 = beg[j] + 1; q0 < beg[j] + len[j]; q0 += GL) {
          const int m = min(GL, beg[j] + len[j] - q0);
          const int32_t my_bag = gl < m ? bags[q0 + gl] : 0;
          for (int u0 = 0; u0 < m; u0 += U) {
            float4 vv[U][V];
#pragma unroll
            for (int u = 0; u < U; ++u) {
              const bool ok = u0 + u < m;
              const int64_t bag = __shfl(my_bag, ok ? u0 + u : 0, GL);
              const float4* grow = reinterpret_cast<const float4*>(gbase[j] + bag * g_ld);
#pragma unroll
              for (int v = 0; v < V; ++v) {
                const int c4 = gl + v * GL;
                vv[u][v] = (ok && c4 < d4) ? grow[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
              }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
              if (u0 + u < m) {
#pragma unroll
                for (int v = 0; v < V; ++v) {
                  acc[v].x = acc[v].x + vv[u][v].x;
                  acc[v].y = acc[v].y + vv[u][v].y;
                  acc[v].z = acc[v].z + vv[u][v].z;
                  acc[v].w = acc[v].w + vv[u][v].w;
                }
              }
            }
          }
        }
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int c4 = gl + v * GL;
          if (c4 < d4) {
            float4 o;
            o.x = __fsub_rn(tv[j][v].x, __fmul_rn(lr, acc[v].x));
            o.y = __fsub_rn(tv[j][v].y, __fmul_rn(lr, acc[v].y));
            o.z = __fsub_rn(tv[j][v].z, __fmul_rn(lr, acc[v].z));
            o.w = __fsub_rn(tv[j][v].w, __fmul_rn(lr, acc[v].w));
            trow[j][c4] = o;
          }
        }
      }
    }
  }
}

// The short segments (many small persistent blocks).
template <int V>
__global__ __launch_bounds__(256) void light_sgd_kernel(float* const* __restrict__ tables, int d, int g_log2,
                                                        int row_bits, const uint32_t* __restrict__ seg_key,
                                                        const int32_t* __restrict__ bags,
                                                        const int32_t* __restrict__ seg_start,
                                                        const uint32_t* __restrict__ nseg,
                                                        const float* __restrict__ G, int64_t g_ld, int64_t g_col0,
                                                        float lr, uint32_t* __restrict__ next) {
  light_phase<V, 8 / V>(tables, d, g_log2, row_bits, seg_key, bags, seg_start, nseg, G, g_ld, g_col0, lr, next);
}

// Hot runs.  Run number u counts the runs class by class, longest class
// first, in list order.  hot_map_kernel gives run u its segment (hseg[u]),
// reserves its ceil(length / kHot) blocks (hoff[u], hcnt[u]: an atomic
// counter hands out the ranges, so where a run's blocks lie varies from
// call to call, but not their order or their sums) and describes every
// block (occurrences [beg, end), key); hot_part_kernel sums each block's
// gradient rows in sorted order from +0 into hpart[block];
// hot_final_kernel adds a run's block sums in order from +0 and updates the
// row.
struct HotBlock {
  int32_t beg, end;
  uint32_t key;
  int32_t pad;
};
constexpr int kHotRunsAt = 4, kHotBlocksAt = 5;  // counters[]: hot runs, hot blocks (cleared by the prepare)

// one wave per run (grid-stride), lanes over its blocks
__global__ __launch_bounds__(256) void hot_map_kernel(const int32_t* __restrict__ seg_start,
                                                      const uint32_t* __restrict__ seg_key,
                                                      const int32_t* __restrict__ hot, int64_t n,
                                                      uint32_t* __restrict__ counters, int32_t* __restrict__ hseg,
                                                      int32_t* __restrict__ hoff, int32_t* __restrict__ hcnt,
                                                      HotBlock* __restrict__ blocks) {
  __shared__ uint32_t cls_first[kHotClassMax + 1], cls_end[kHotClassMax + 1], cls_cnt[kHotClassMax + 1];
  if (threadIdx.x >= kHotClassMin && threadIdx.x <= kHotClassMax)  // the class counts, loaded side by side
    cls_cnt[threadIdx.x] = counters[kHotCountBase + threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t first = 0;
    for (int c = kHotClassMax; c >= kHotClassMin; --c) {
      cls_first[c] = first;
      first += cls_cnt[c];
      cls_end[c] = first;
    }
    if (blockIdx.x == 0) counters[kHotRunsAt] = first;
  }
  __syncthreads();
  const uint32_t total = cls_end[kHotClassMin];
  const int lane = threadIdx.x & 63;
  const uint32_t waves = gridDim.x * (blockDim.x >> 6);
  // a wave takes 64 runs (one per lane) and reserves their blocks with one
  // atomic (one counter shared by every wave: an atomic per run would queue)
  // (runs gi, gi + groups, gi + 2 groups, ...: the classes are longest
  // first, so each wave gets a share of the long runs' blocks to write)
  const uint32_t groups = (total + 63) / 64;
  for (uint32_t gi = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); gi < groups; gi += waves) {
    const uint32_t u = gi + groups * (uint32_t)lane;
    int32_t sg = 0, beg = 0, end = 0, nb = 0;
    uint32_t key = 0;
    if (u < total) {
      int c = kHotClassMax;
      while (c > kHotClassMin && u >= cls_end[c]) --c;
      sg = hot[hot_class_base(n, c) + (u - cls_first[c])];
      beg = seg_start[sg];
      end = seg_start[sg + 1];
      key = seg_key[sg];
      nb = (end - beg + kHot - 1) / kHot;
    }
    int32_t incl = nb;  // inclusive prefix over the wave's lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    int32_t base = 0;
    if (lane == 63) base = (int32_t)atomicAdd(&counters[kHotBlocksAt], (uint32_t)incl);
    base = __shfl(base, 63, 64);
    const int32_t q0 = base + incl - nb;
    if (u < total) {
      hseg[u] = sg;
      hoff[u] = q0;
      hcnt[u] = nb;
    }
    for (int r = 0; r < 64; ++r) {  // every lane writes blocks of run r
      const int32_t nbr = __shfl(nb, r, 64);
      if (nbr == 0) continue;
      const int32_t q0r = __shfl(q0, r, 64), begr = __shfl(beg, r, 64), endr = __shfl(end, r, 64);
      const uint32_t keyr = (uint32_t)__shfl((int)key, r, 64);
      for (int32_t j = lane; j < nbr; j += 64) {
        HotBlock hb;
        hb.beg = begr + j * kHot;
        hb.end = min(endr, hb.beg + kHot);
        hb.key = keyr;
        hb.pad = 0;
        blocks[q0r + j] = hb;
      }
    }
  }
}

// A group of 2^g_log2 lanes per item (V float4 of a row per lane, the
// columns of a slice); the groups of a wave walk the items with the grid's
// stride.
struct Groups {
  int gl, grp, per_wave, GL;
  __device__ Groups(int g_log2) {
    const int lane = threadIdx.x & 63;
    GL = 1 << g_log2;
    gl = lane & (GL - 1);
    grp = lane >> g_log2;
    per_wave = 64 >> g_log2;
  }
  __device__ uint32_t first() const {
    return (uint32_t)((blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * per_wave + grp);
  }
  __device__ uint32_t stride() const { return (uint32_t)(gridDim.x * (blockDim.x >> 6) * per_wave); }
};

template <int V, int U>
__global__ __launch_bounds__(256) void hot_part_kernel(int d, int g_log2, int row_bits,
                                                       const HotBlock* __restrict__ blocks,
                                                       const uint32_t* __restrict__ counters,
                                                       const int32_t* __restrict__ bags, const float* __restrict__ G,
                                                       int64_t g_ld, int64_t g_col0, float* __restrict__ hpart) {
  const Groups gp(g_log2);
  const int d4 = d >> 2, cols4 = gp.GL * V;  // float4 columns per slice
  const int slices = (d4 + cols4 - 1) / cols4;
  const uint32_t items = counters[kHotBlocksAt] * (uint32_t)slices;
  for (uint32_t it = gp.first(); it < items; it += gp.stride()) {
    const uint32_t q = it / (uint32_t)slices;
    const int c40 = (int)(it - q * (uint32_t)slices) * cols4;
    const HotBlock hb = blocks[q];
    const int k = (int)(hb.key >> row_bits);
    const float* gbase = G + g_col0 + (int64_t)k * d;
    float4 acc[V], cur[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      acc[v] = make_float4(0.f, 0.f, 0.f, 0.f);
      cur[v] = acc[v];
    }
    // a long row's occurrences come in runs of one bag (a Zipf head shows
    // up many times in one bag, and those positions are adjacent): a row
    // is loaded only where the bag changes (all of a batch's loads go out
    // first) and added again while it does not
    int32_t last_bag = -1;
    for (int32_t p0 = hb.beg; p0 < hb.end; p0 += gp.GL) {
      const int m = min(gp.GL, hb.end - p0);
      const int32_t my_bag = gp.gl < m ? bags[p0 + gp.gl] : 0;
      for (int u0 = 0; u0 < m; u0 += U) {
        float4 vv[U][V];
        bool fresh[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = u0 + u < m;
          const int32_t bag = __shfl(my_bag, ok ? u0 + u : 0, gp.GL);
          fresh[u] = ok && bag != last_bag;
          if (ok) last_bag = bag;
          if (fresh[u]) {
            const float4* grow = reinterpret_cast<const float4*>(gbase + (int64_t)bag * g_ld);
#pragma unroll
            for (int v = 0; v < V; ++v) {
              const int c4 = c40 + gp.gl + v * gp.GL;
              vv[u][v] = c4 < d4 ? grow[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (u0 + u < m) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
              if (fresh[u]) cur[v] = vv[u][v];
              acc[v].x = acc[v].x + cur[v].x;
              acc[v].y = acc[v].y + cur[v].y;
              acc[v].z = acc[v].z + cur[v].z;
              acc[v].w = acc[v].w + cur[v].w;
            }
          }
        }
      }
    }
    float4* dst = reinterpret_cast<float4*>(hpart + (int64_t)q * d);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c4 = c40 + gp.gl + v * gp.GL;
      if (c4 < d4) dst[c4] = acc[v];
    }
  }
}

template <int V, int U>
__global__ __launch_bounds__(256) void hot_final_kernel(float* const* __restrict__ tables, int d, int g_log2,
                                                        int row_bits, const uint32_t* __restrict__ counters,
                                                        const int32_t* __restrict__ hseg,
                                                        const int32_t* __restrict__ hoff,
                                                        const int32_t* __restrict__ hcnt,
                                                        const uint32_t* __restrict__ seg_key,
                                                        const float* __restrict__ hpart, float lr) {
  const Groups gp(g_log2);
  const uint32_t row_mask = (row_bits >= 32) ? 0xffffffffu : ((1u << row_bits) - 1u);
  const int d4 = d >> 2, cols4 = gp.GL * V;
  const int slices = (d4 + cols4 - 1) / cols4;
  const uint32_t items = counters[kHotRunsAt] * (uint32_t)slices;
  for (uint32_t it = gp.first(); it < items; it += gp.stride()) {
    const uint32_t u = it / (uint32_t)slices;
    const int c40 = (int)(it - u * (uint32_t)slices) * cols4;
    const int32_t q0 = hoff[u], q1 = q0 + hcnt[u];
    const uint32_t key = seg_key[hseg[u]];
    const int k = (int)(key >> row_bits);
    const int64_t r = (int64_t)(key & row_mask);
    float4 acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int32_t q = q0; q < q1; q += U) {
      float4 vv[U][V];
#pragma unroll
      for (int u2 = 0; u2 < U; ++u2) {
        const int32_t qq = q + u2 < q1 ? q + u2 : q1 - 1;
        const float4* src = reinterpret_cast<const float4*>(hpart + (int64_t)qq * d);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int c4 = c40 + gp.gl + v * gp.GL;
          vv[u2][v] = c4 < d4 ? src[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u2 = 0; u2 < U; ++u2) {
        if (q + u2 < q1) {
#pragma unroll
          for (int v = 0; v < V; ++v) {
            acc[v].x = acc[v].x + vv[u2][v].x;
            acc[v].y = acc[v].y + vv[u2][v].y;
            acc[v].z = acc[v].z + vv[u2][v].z;
            acc[v].w = acc[v].w + vv[u2][v].w;
          }
        }
      }
    }
    float4* trow = reinterpret_cast<float4*>(tables[k] + r * d);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c4 = c40 + gp.gl + v * gp.GL;
      if (c4 < d4) {
        const float4 t = trow[c4];
        float4 o;
        o.x = __fsub_rn(t.x, __fmul_rn(lr, acc[v].x));
        o.y = __fsub_rn(t.y, __fmul_rn(lr, acc[v].y));
        o.z = __fsub_rn(t.z, __fmul_rn(lr, acc[v].z));
        o.w = __fsub_rn(t.w, __fmul_rn(lr, acc[v].w));
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
  size_t keys[2], vals[2], counts, sums, offsets, seg, seg_key, counters, hot, hseg, hoff, hcnt, hblocks, hpart, bytes;
  int64_t tiles;
};

// counters: [0] segments, [3] next short-segment chunk, [kHotRunsAt] hot
// runs, [kHotBlocksAt] their blocks, [kHotCountBase + c] hot runs of class
// c (cleared on every prepare)
constexpr int kCounters = 48;
static_assert(kHotCountBase + kHotClassMax < kCounters, "hot class counters");

// Everything up to the hot-run buffers is what the prepare step needs; the
// block sums (n / 64 blocks at most: a run of L >= kHot occurrences has
// ceil(L / kHot) < 2 L / kHot blocks) take d floats each and come last.
void sparse_layout(int64_t nnz, int d, SparseLayout* L) {
  Carver cv(nullptr);
  auto take = [&](size_t bytes) {
    cv.used = (size_t)round_up((int64_t)cv.used, 256);
    const size_t at = cv.used;
    cv.used += bytes;
    return at;
  };
  const int64_t n = nnz > 0 ? nnz : 1;
  L->tiles = ceil_div(n, TILE);
  L->keys[0] = take(4 * (size_t)n);
  L->keys[1] = take(4 * (size_t)n);
  L->vals[0] = take(4 * (size_t)n);
  L->vals[1] = take(4 * (size_t)n);
  L->counts = take(4 * (size_t)kMaxDigits * L->tiles);
  L->sums = take(4 * (size_t)kMaxDigits * ceil_div(L->tiles, kChunk));
  L->offsets = take(4 * (size_t)kMaxDigits * L->tiles);
  L->seg = take(4 * (size_t)(n + 1));
  L->seg_key = take(4 * (size_t)n);
  L->counters = take(4 * (size_t)kCounters);
  L->hot = take(4 * (size_t)hot_class_base(n, kHotClassMax + 1));
  const int64_t max_runs = n / kHot + 1, max_blocks = n / (kHot / 2) + 1;
  L->hseg = take(4 * (size_t)max_runs);
  L->hoff = take(4 * (size_t)max_runs);
  L->hcnt = take(4 * (size_t)max_runs);
  L->hblocks = take(sizeof(HotBlock) * (size_t)max_blocks);
  L->hpart = take(4 * (size_t)max_blocks * (size_t)(d > 0 ? d : 0));
  L->bytes = cv.bytes();
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace
}  // namespace dlrm

namespace dlrm {
namespace {
struct SparseBufs;
int sgd_segments(float* const* tables, int d, int row_bits, int cur, const SparseBufs& b, int64_t n,
                 const float* G, int64_t g_ld, int64_t g_col0, float lr, hipStream_t stream, hipStream_t side);
}  // namespace
}  // namespace dlrm

using namespace dlrm;

extern "C" size_t dlrm_embbag_bwd_sgd_workspace_size(int32_t K, int64_t B, int64_t nnz, int32_t d) {
  (void)K;
  (void)B;
  if (nnz < 0 || d < 0) return 0;
  SparseLayout L;
  sparse_layout(nnz, d, &L);
  return L.bytes;
}

namespace dlrm {
namespace {
// Checks shared by the three entry points; the key widths follow from the
// table count and the largest table.
int check_sparse(int32_t K, const int64_t* rows, int64_t B, int64_t nnz, int* row_bits, int* table_bits) {
  if (!rows || K < 1 || B < 1 || B > 0x7fffffffLL || nnz < 0 || nnz > 0x7fffffffLL) return DLRM_E_INVALID;
  int64_t max_rows = 1;
  for (int k = 0; k < K; ++k) {
    if (rows[k] < 1) return DLRM_E_INVALID;
    max_rows = rows[k] > max_rows ? rows[k] : max_rows;
  }
  *row_bits = bits_for(max_rows - 1) > 0 ? bits_for(max_rows - 1) : 1;
  *table_bits = bits_for(K - 1);
  if (*row_bits + *table_bits > 32) return DLRM_E_UNSUPPORTED;
  return DLRM_OK;
}

struct SparseBufs {
  uint32_t* keys[2];
  int32_t* vals[2];
  uint32_t* counts;
  uint32_t* sums;
  uint32_t* offsets;
  int32_t* seg;
  uint32_t* seg_key;
  uint32_t* counters;
  int32_t* hot;
  int32_t* hseg;
  int32_t* hoff;
  int32_t* hcnt;
  HotBlock* hblocks;
  float* hpart;
};

// d = 0: the prepare step's view (no block sums)
int sparse_bufs(int64_t nnz, int d, void* ws, size_t ws_bytes, SparseLayout* L, SparseBufs* b) {
  sparse_layout(nnz, d, L);
  if (!ws || ws_bytes < L->bytes) return DLRM_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return DLRM_E_INVALID;
  char* w = static_cast<char*>(ws);
  b->keys[0] = reinterpret_cast<uint32_t*>(w + L->keys[0]);
  b->keys[1] = reinterpret_cast<uint32_t*>(w + L->keys[1]);
  b->vals[0] = reinterpret_cast<int32_t*>(w + L->vals[0]);
  b->vals[1] = reinterpret_cast<int32_t*>(w + L->vals[1]);
  b->counts = reinterpret_cast<uint32_t*>(w + L->counts);
  b->sums = reinterpret_cast<uint32_t*>(w + L->sums);
  b->offsets = reinterpret_cast<uint32_t*>(w + L->offsets);
  b->seg = reinterpret_cast<int32_t*>(w + L->seg);
  b->seg_key = reinterpret_cast<uint32_t*>(w + L->seg_key);
  b->counters = reinterpret_cast<uint32_t*>(w + L->counters);
  b->hot = reinterpret_cast<int32_t*>(w + L->hot);
  b->hseg = reinterpret_cast<int32_t*>(w + L->hseg);
  b->hoff = reinterpret_cast<int32_t*>(w + L->hoff);
  b->hcnt = reinterpret_cast<int32_t*>(w + L->hcnt);
  b->hblocks = reinterpret_cast<HotBlock*>(w + L->hblocks);
  b->hpart = reinterpret_cast<float*>(w + L->hpart);
  return DLRM_OK;
}

// The sort runs over the row bits only: positions are table-major (the
// bags of table k come before those of table k + 1), so a stable sort by
// row leaves equal rows in table order and every (table, row) key in one
// run.  Digits of 8 bits, or 9 where that saves a pass (26 row bits: three
// passes of 9 instead of four of 8).  The sorted keys and bag ids end in
// buffer passes % 2.
struct SortPlan {
  int passes, digit_bits;
};
SortPlan sort_plan(int row_bits) {
  const int p8 = (row_bits + 7) / 8, p9 = (row_bits + 8) / 9;
  return p9 < p8 ? SortPlan{p9, 9} : SortPlan{p8, 8};
}
}  // namespace
}  // namespace dlrm

extern "C" int dlrm_embbag_bwd_sgd_prepare(int32_t K, const int64_t* rows, const int64_t* indices,
                                           const int64_t* offsets, int64_t B, int64_t nnz, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  if (!indices || !offsets) return DLRM_E_INVALID;
  int row_bits = 0, table_bits = 0;
  int rc = check_sparse(K, rows, B, nnz, &row_bits, &table_bits);
  if (rc != DLRM_OK) return rc;
  if (nnz == 0) return DLRM_OK;
  SparseLayout L;
  SparseBufs b;
  if ((rc = sparse_bufs(nnz, 0, ws, ws_bytes, &L, &b)) != DLRM_OK) return rc;
  const int n = (int)nnz;
  const int64_t KB = (int64_t)K * B;

  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, b.counters, kCounters);
  {
    int kg = 0;  // lanes per bag: the mean bag length rounded up to a power of two, at most 64
    while ((1LL << kg) * KB < nnz && kg < 6) ++kg;
    const int64_t kblocks = ceil_div(KB << kg, 256);
    if (kblocks > 0x7fffffffLL) return DLRM_E_UNSUPPORTED;
    hipLaunchKernelGGL(build_keys_kernel, dim3((unsigned)kblocks), dim3(256), 0, stream, indices, offsets, KB, B, kg,
                       row_bits, b.keys[0], b.vals[0]);
  }
  const SortPlan plan = sort_plan(row_bits);
  const unsigned tiles = (unsigned)L.tiles;
  const dim3 chunk_grid((unsigned)ceil_div(L.tiles, kChunk), (unsigned)((1 << plan.digit_bits) / 64));
  int cur = 0;
  for (int pass = 0; pass < plan.passes; ++pass) {
    const int shift = pass * plan.digit_bits;
#define DLRM_PASS(DB)                                                                                                hipLaunchKernelGGL(tile_hist_kernel<DB>, dim3(tiles), dim3(RT), 0, stream, b.keys[cur], n, shift, b.counts,                          (int)tiles);                                                                                    hipLaunchKernelGGL(chunk_sum_kernel<DB>, chunk_grid, dim3(RT), 0, stream, b.counts, (int)tiles, b.sums);           hipLaunchKernelGGL(tile_offset_kernel<DB>, chunk_grid, dim3(RT), 0, stream, b.counts, b.sums, (int)tiles,                             b.offsets);                                                                                     hipLaunchKernelGGL(scatter_kernel<DB>, dim3(tiles), dim3(RT), 0, stream, b.keys[cur], b.vals[cur],                                   b.keys[cur ^ 1], b.vals[cur ^ 1], n, shift, b.offsets, (int)tiles)
    if (plan.digit_bits == 9) {
      DLRM_PASS(9);
    } else {
      DLRM_PASS(8);
    }
#undef DLRM_PASS
    cur ^= 1;
  }
  hipLaunchKernelGGL(heads_count_kernel, dim3(tiles), dim3(RT), 0, stream, b.keys[cur], n, b.counts);
  hipLaunchKernelGGL(heads_scan_kernel, dim3(1), dim3(RT), 0, stream, b.counts, (int)tiles, n, b.seg, b.counters);
  hipLaunchKernelGGL(heads_write_kernel, dim3(tiles), dim3(RT), 0, stream, b.keys[cur], n, b.counts, b.seg,
                     b.seg_key, b.hot, b.counters);
  // the hot runs' block list (indices only, so it belongs to this step)
  hipLaunchKernelGGL(hot_map_kernel, dim3(kHotBlocks), dim3(256), 0, stream, b.seg, b.seg_key, b.hot, (int64_t)n,
                     b.counters, b.hseg, b.hoff, b.hcnt, b.hblocks);
  return launch_status() != DLRM_OK ? DLRM_E_HIP : DLRM_OK;
}

extern "C" int dlrm_embbag_bwd_sgd_apply(float* const* tables, int32_t K, int32_t d, const int64_t* rows, int64_t B,
                                         int64_t nnz, const float* G, int64_t g_ld, int64_t g_col0, float lr, void* ws,
                                         size_t ws_bytes, hipStream_t stream, hipStream_t side) {
  if (!tables || !G) return DLRM_E_INVALID;
  if (d < 4 || d > 1024 || (d % 4) != 0) return DLRM_E_INVALID;
  if (g_col0 < 0 || g_ld < g_col0 + (int64_t)K * d || (g_ld % 4) != 0 || (g_col0 % 4) != 0 || !aligned16(G))
    return DLRM_E_INVALID;
  int row_bits = 0, table_bits = 0;
  int rc = check_sparse(K, rows, B, nnz, &row_bits, &table_bits);
  if (rc != DLRM_OK) return rc;
  if (nnz == 0) return DLRM_OK;
  SparseLayout L;
  SparseBufs b;
  if ((rc = sparse_bufs(nnz, d, ws, ws_bytes, &L, &b)) != DLRM_OK) return rc;
  const int cur = sort_plan(row_bits).passes & 1;
  // the short segments' work counter starts from zero on every call, so one
  // prepared workspace can be applied more than once; it is cleared on the
  // stream whose kernel takes work from it
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, side ? side : stream, b.counters + 3, 1);
  if (launch_status() != DLRM_OK) return DLRM_E_HIP;
  return sgd_segments(tables, d, row_bits, cur, b, nnz, G, g_ld, g_col0, lr, stream, side);
}

// ------------------------------------------------------------------ no-allocation form
//
// dlrm_embbag_bwd_sgd_noalloc keeps the workspace of dlrm_embbag_bwd_sgd in
// a file-scope device array instead of a caller buffer.  Every GPU that runs
// the library holds its own copy of the array from the moment the library's
// code object is loaded on it until the process ends.  In host code the
// array's name is only a host-side stand-in: the device address comes from
// hipGetSymbolAddress, resolved once per device with that device current
// (on the entry point's first call there) and kept per device.
constexpr size_t kNoallocScratchBytes = (size_t)DLRM_NOALLOC_SCRATCH_MB << 20;
static __device__ __attribute__((aligned(256))) char scratch[kNoallocScratchBytes];

namespace dlrm {
namespace {
void* noalloc_scratch() {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_hip_error = (int)e;
      return nullptr;
    }
    ptr[dev] = p;
  }
  return ptr[dev];
}
}  // namespace
}  // namespace dlrm

extern "C" int dlrm_embbag_bwd_sgd_noalloc(float* const* tables, int32_t K, int32_t d, const int64_t* rows,
                                           const int64_t* indices, const int64_t* offsets, int64_t B, int64_t nnz,
                                           const float* G, int64_t g_ld, int64_t g_col0, float lr,
                                           hipStream_t stream) {
  if (nnz < 0 || nnz > 0x7fffffffLL) return DLRM_E_INVALID;
  if (d < 0) return DLRM_E_INVALID;
  SparseLayout L;
  sparse_layout(nnz, d, &L);
  if (L.bytes > kNoallocScratchBytes) return DLRM_E_WORKSPACE;
  void* ws = noalloc_scratch();
  if (!ws) return DLRM_E_HIP;
  // the same kernels as dlrm_embbag_bwd_sgd on the static scratch (its
  // counters are cleared by a kernel at the start of each call)
  return dlrm_embbag_bwd_sgd(tables, K, d, rows, indices, offsets, B, nnz, G, g_ld, g_col0, lr, ws,
                             kNoallocScratchBytes, stream);
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
  const int rc = dlrm_embbag_bwd_sgd_prepare(K, rows, indices, offsets, B, nnz, ws, ws_bytes, stream);
  if (rc != DLRM_OK) return rc;
  return dlrm_embbag_bwd_sgd_apply(tables, K, d, rows, B, nnz, G, g_ld, g_col0, lr, ws, ws_bytes, stream, nullptr);
}

namespace dlrm {
namespace {
int sgd_segments(float* const* tables, int d, int row_bits, int cur, const SparseBufs& b, int64_t n,
                 const float* G, int64_t g_ld, int64_t g_col0, float lr, hipStream_t stream, hipStream_t side) {
  // lane groups: short segments with half as many lanes as float4 columns
  // (two float4 per lane), hot blocks and runs with one float4 per lane;
  // groups of at most 64 lanes
  const int d4 = d / 4;
  int l2 = 0;
  while ((1 << l2) < d4) ++l2;
  const int g_log2 = l2 > 0 ? (l2 - 1 < 6 ? l2 - 1 : 6) : 0;
  const int V = (d4 + (1 << g_log2) - 1) >> g_log2;
  const int h_log2 = l2 < 6 ? l2 : 6;
  const dim3 blk(256), hot_grid(kHotBlocks);
  const int32_t* vals = b.vals[cur];
  // hot runs on `stream` (their block list came with the prepare step)
  hipLaunchKernelGGL((hot_part_kernel<1, 16>), hot_grid, blk, 0, stream, d, h_log2, row_bits, b.hblocks, b.counters,
                     vals, G, g_ld, g_col0, b.hpart);
  hipLaunchKernelGGL((hot_final_kernel<1, 32>), hot_grid, blk, 0, stream, tables, d, h_log2, row_bits, b.counters,
                     b.hseg, b.hoff, b.hcnt, b.seg_key, b.hpart, lr);
  if (launch_status() != DLRM_OK) return DLRM_E_HIP;
  // short segments beside them on `side`, or after them
  const dim3 grid(kLightBlocks);
  hipStream_t ls = side ? side : stream;
#define DLRM_LIGHT(VV)                                                                                         \
  hipLaunchKernelGGL((light_sgd_kernel<VV>), grid, blk, 0, ls, tables, d, g_log2, row_bits, b.seg_key, vals, b.seg, \
                     b.counters, G, g_ld, g_col0, lr, b.counters + 3)
  if (V == 1) DLRM_LIGHT(1);
  else if (V == 2) DLRM_LIGHT(2);
  else DLRM_LIGHT(4);
#undef DLRM_LIGHT
  return launch_status();
}
}  // namespace
}  // namespace dlrm
