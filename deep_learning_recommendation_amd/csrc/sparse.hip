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
//   2. a stable least-significant-digit radix sort over the row bits of the
//      keys (8 or 9 bits per pass); stability keeps equal keys in position
//      order, and since positions are table-major, equal rows of different
//      tables stay in table order, so every (table, row) key forms one run;
//   3. run-length segmentation (head flags, device-wide exclusive scan);
//   4. one fused kernel: each segment's gradient sum over its occurrences in
//      sorted order (fp32, from +0) and the update T <- T - lr * g.
// Hot rows (Zipf heads with 10^5 occurrences) make step 4's longest serial
// chain the latency floor.  Step 4 is one persistent launch with one block
// per CU.  Segments of at least kHot occurrences come first, as
// producer/consumer items: per (segment, 64-column slice) one wave adds, one
// column per lane, from an LDS ring that six other waves keep filled, so the
// serial adds never wait on memory.  Hot items are handed out longest first;
// a block that finds none left turns its seven waves to the short segments
// (one lane group each, chunks taken from a second counter), so the CUs that
// the few longest chains leave free take the rest of the work meanwhile.
#include "common.hpp"

#include <mutex>

namespace dlrm {
namespace {

constexpr int RT = 256;                // threads per sort block
constexpr int ITEMS = 16;              // keys per thread per tile
constexpr int TILE = RT * ITEMS;       // 4096 positions per tile
constexpr int kMaxDigits = 512;        // buckets of a digit of at most 9 bits
constexpr int kHot = 128;              // occurrences from which a segment is "hot"
constexpr int kHB = 64;                // occurrences per LDS ring slot
constexpr int kSlots = 8;              // ring slots
constexpr int kRS = kHB + 4;           // floats per column row of a slot (padded: conflict-free 16-byte reads)
constexpr int kLoaders = 6;            // loader waves per hot block (plus one adder)
constexpr int kAdder = 3;              // the adder's wave index: alone on its SIMD when waves go round-robin
constexpr int kApplyThreads = 64 * (kLoaders + 1);
constexpr int kLightBlocks = 2048;     // persistent blocks of the standalone short-segment kernel

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

// Hand-over flags in LDS, read and written as workgroup-scope atomics so
// that every access really goes to LDS and stays in program order.
__device__ __forceinline__ int32_t lds_load(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The adder's loop over the full blocks of an item, scheduled by hand.  Every
// instruction between two dependent adds lengthens the chain (measured on
// gfx950: a dependent fp32 add issues every 4.4 cycles; a 16-byte LDS read
// placed between two adds adds about 15 cycles, four of them back to back
// about 6 cycles each; a satisfied wait about 4), so a block runs as four
// steps of [four 16-byte reads, one wait, sixteen adds], the reads for the
// step after next, the waits counted exactly (one wave's LDS accesses complete
// in order).  Step buffers live in v192..v255 (A, B: steps 0 and 1, reloaded
// from the next block during steps 2 and 3; C, D: steps 2 and 3).  The slot
// is released (consumed = block + 1) right after its last reads are issued:
// they are performed before any later access of this wave, so before the
// loader can see the release.  The next block's flag is read before its first
// reads; if it was not yet up, those reads are dropped and issued again once
// it is.
#define HOT_RD(v0, v3, op, off) "ds_read_b128 v[" #v0 ":" #v3 "], %[" #op "] offset:" #off "\n\t"
#define HOT_RD_A(op) HOT_RD(192, 195, op, 0) HOT_RD(196, 199, op, 16) HOT_RD(200, 203, op, 32) HOT_RD(204, 207, op, 48)
#define HOT_RD_B(op) HOT_RD(208, 211, op, 64) HOT_RD(212, 215, op, 80) HOT_RD(216, 219, op, 96) HOT_RD(220, 223, op, 112)
#define HOT_RD_C(op) HOT_RD(224, 227, op, 128) HOT_RD(228, 231, op, 144) HOT_RD(232, 235, op, 160) HOT_RD(236, 239, op, 176)
#define HOT_RD_D(op) HOT_RD(240, 243, op, 192) HOT_RD(244, 247, op, 208) HOT_RD(248, 251, op, 224) HOT_RD(252, 255, op, 240)
#define HOT_ADD(v) "v_add_f32 %[acc], %[acc], v" #v "\n\t"
#define HOT_ADD4(a, b, c, e) HOT_ADD(a) HOT_ADD(b) HOT_ADD(c) HOT_ADD(e)
#define HOT_ADDS_A HOT_ADD4(192, 193, 194, 195) HOT_ADD4(196, 197, 198, 199) HOT_ADD4(200, 201, 202, 203) HOT_ADD4(204, 205, 206, 207)
#define HOT_ADDS_B HOT_ADD4(208, 209, 210, 211) HOT_ADD4(212, 213, 214, 215) HOT_ADD4(216, 217, 218, 219) HOT_ADD4(220, 221, 222, 223)
#define HOT_ADDS_C HOT_ADD4(224, 225, 226, 227) HOT_ADD4(228, 229, 230, 231) HOT_ADD4(232, 233, 234, 235) HOT_ADD4(236, 237, 238, 239)
#define HOT_ADDS_D HOT_ADD4(240, 241, 242, 243) HOT_ADD4(244, 245, 246, 247) HOT_ADD4(248, 249, 250, 251) HOT_ADD4(252, 253, 254, 255)
static_assert(kHB == 64 && kSlots == 8, "the adder loop takes 64-occurrence blocks in an 8-slot ring");
static_assert(64 * kRS * sizeof(float) == 0x4400, "the adder loop's slot stride");
__device__ __forceinline__ void hot_adder_full_blocks(float& acc, int32_t base, int32_t nfull, const float* lane_col,
                                                      const int32_t* ready, int32_t* consumed) {
  const uint32_t col = (uint32_t)reinterpret_cast<uintptr_t>(lane_col);  // LDS byte addresses
  const uint32_t rdy = (uint32_t)reinterpret_cast<uintptr_t>(ready);
  const uint32_t cons = (uint32_t)reinterpret_cast<uintptr_t>(consumed);
  uint32_t s_t, s_tn, s_exp, s_slot, s_off, s_fa, s_fl, s_c, v_cur, v_nxt, v_fa, v_fl, v_tmp;
  uint64_t s_ex;
  __asm__ volatile(
      // block 0: wait for its flag, then issue steps 0 and 1
      "s_mov_b32 %[t], 0\n\t"
      "s_mov_b32 %[exp], %[base]\n\t"
      "s_and_b32 %[slot], %[exp], 7\n\t"
      "s_lshl_b32 %[fa], %[slot], 2\n\t"
      "s_add_u32 %[fa], %[fa], %[rdy]\n\t"
      "v_mov_b32 %[vfa], %[fa]\n"
      "HOT_W0_%=:\n\t"
      "ds_read_b32 %[vfl], %[vfa]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_readfirstlane_b32 %[fl], %[vfl]\n\t"
      "s_cmp_eq_u32 %[fl], %[exp]\n\t"
      "s_cbranch_scc1 HOT_R0_%=\n\t"
      "s_sleep 1\n\t"
      "s_branch HOT_W0_%=\n"
      "HOT_R0_%=:\n\t"
      "s_mul_i32 %[off], %[slot], 0x4400\n\t"
      "v_add_u32 %[cur], %[off], %[col]\n\t"
      HOT_RD_A(cur) HOT_RD_B(cur)
      "HOT_L_%=:\n\t"
      // the next block (after the last one, this block again: those reads are dropped)
      "s_add_u32 %[tn], %[t], 1\n\t"
      "s_cmp_lt_u32 %[tn], %[nfull]\n\t"
      "s_cselect_b32 %[tn], %[tn], %[t]\n\t"
      "s_add_u32 %[exp], %[base], %[tn]\n\t"
      "s_and_b32 %[slot], %[exp], 7\n\t"
      "s_mul_i32 %[off], %[slot], 0x4400\n\t"
      "v_add_u32 %[nxt], %[off], %[col]\n\t"
      "s_lshl_b32 %[fa], %[slot], 2\n\t"
      "s_add_u32 %[fa], %[fa], %[rdy]\n\t"
      "v_mov_b32 %[vfa], %[fa]\n\t"
      // step 0: A in flight or done, B, C younger
      HOT_RD_C(cur)
      "s_waitcnt lgkmcnt(8)\n\t"
      HOT_ADDS_A
      // step 1: this block's last reads, then its release
      HOT_RD_D(cur)
      "s_add_u32 %[c], %[base], %[t]\n\t"
      "s_add_u32 %[c], %[c], 1\n\t"
      "v_mov_b32 %[tmp], %[c]\n\t"
      "s_mov_b64 %[ex], exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "ds_write_b32 %[cons], %[tmp]\n\t"
      "s_mov_b64 exec, %[ex]\n\t"
      "s_waitcnt lgkmcnt(9)\n\t"
      HOT_ADDS_B
      // step 2: the next block's flag and its step 0
      "ds_read_b32 %[vfl], %[vfa]\n\t"
      HOT_RD_A(nxt)
      "s_waitcnt lgkmcnt(10)\n\t"
      HOT_ADDS_C
      // step 3: the next block's step 1
      HOT_RD_B(nxt)
      "s_waitcnt lgkmcnt(10)\n\t"
      HOT_ADDS_D
      "s_add_u32 %[t], %[t], 1\n\t"
      "s_cmp_ge_u32 %[t], %[nfull]\n\t"
      "s_cbranch_scc1 HOT_D_%=\n\t"
      "s_waitcnt lgkmcnt(8)\n\t"
      "v_readfirstlane_b32 %[fl], %[vfl]\n\t"
      "v_mov_b32 %[cur], %[nxt]\n\t"
      "s_cmp_eq_u32 %[fl], %[exp]\n\t"
      "s_cbranch_scc1 HOT_L_%=\n\t"
      // the flag was not up when read: drop those reads, wait, read again
      "s_waitcnt lgkmcnt(0)\n"
      "HOT_S_%=:\n\t"
      "s_sleep 1\n\t"
      "ds_read_b32 %[vfl], %[vfa]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_readfirstlane_b32 %[fl], %[vfl]\n\t"
      "s_cmp_eq_u32 %[fl], %[exp]\n\t"
      "s_cbranch_scc0 HOT_S_%=\n\t"
      HOT_RD_A(cur) HOT_RD_B(cur)
      "s_branch HOT_L_%=\n"
      "HOT_D_%=:\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [acc] "+v"(acc), [t] "=&s"(s_t), [tn] "=&s"(s_tn), [exp] "=&s"(s_exp), [slot] "=&s"(s_slot),
        [off] "=&s"(s_off), [fa] "=&s"(s_fa), [fl] "=&s"(s_fl), [c] "=&s"(s_c), [ex] "=&s"(s_ex),
        [cur] "=&v"(v_cur), [nxt] "=&v"(v_nxt), [vfa] "=&v"(v_fa), [vfl] "=&v"(v_fl), [tmp] "=&v"(v_tmp)
      : [base] "s"(base), [nfull] "s"(nfull), [rdy] "s"(rdy), [col] "v"(col), [cons] "v"(cons)
      : "memory", "scc",
        "v192", "v193", "v194", "v195", "v196", "v197", "v198", "v199", "v200", "v201", "v202", "v203", "v204",
        "v205", "v206", "v207", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215", "v216", "v217",
        "v218", "v219", "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228", "v229", "v230",
        "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243",
        "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255");
}
#undef HOT_RD
#undef HOT_RD_A
#undef HOT_RD_B
#undef HOT_RD_C
#undef HOT_RD_D
#undef HOT_ADD
#undef HOT_ADD4
#undef HOT_ADDS_A
#undef HOT_ADDS_B
#undef HOT_ADDS_C
#undef HOT_ADDS_D

// Hot segments (first phase of the apply kernel).  A block (7 waves) takes
// (segment, 64-column slice) items from a global counter until none is left.  Wave kAdder is the adder (the only wave on its
// SIMD when the waves are placed round-robin): lane j owns column j of the
// slice and adds the occurrences in sorted order, reading them from LDS.
// The other six waves are loaders: block t of the segment (occurrences
// 64t..64t+63) goes to ring slot (running block number) mod kSlots, loaded
// by loader t mod 6.  A slot is column-major (column c's 64 occurrences are
// contiguous, rows padded to kRS floats), so the adder reads four
// consecutive occurrences of its column with one 16-byte LDS read.  A loader lane loads a 4 x 4 piece
// (4 occurrences x 4 columns) of the block into registers, transposes it
// and writes four 16-byte column pieces.  Hand-over per slot: the loader
// waits until the adder has finished the slot's previous block
// ("consumed"), writes, and publishes the running block number in
// ready[slot].
struct HotLds {
  float ring[kSlots][64 * kRS];
  int32_t ready[kSlots];
  int32_t consumed;
  uint32_t s_item;
  int32_t s_seg;
  uint32_t cls_first[kHotClassMax + 1];  // first hot run number of each class (classes longest first)
  uint32_t cls_end[kHotClassMax + 1];
  uint32_t cls_base[kHotClassMax + 1];   // its list's first slot
  uint32_t s_items;
};

__device__ __forceinline__ void hot_phase(HotLds& sm, float* const* __restrict__ tables, int d, int row_bits,
                                          const uint32_t* __restrict__ seg_key, const int32_t* __restrict__ bags,
                                          const int32_t* __restrict__ seg_start, const int32_t* __restrict__ hot,
                                          const uint32_t* __restrict__ counters, int64_t n,
                                          const float* __restrict__ G,
                                          int64_t g_ld, int64_t g_col0, float lr,
                                          uint32_t* __restrict__ next_item) {
  auto& ring = sm.ring;
  auto& ready = sm.ready;
  auto& consumed = sm.consumed;
  auto& s_item = sm.s_item;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kSlots) ready[tid] = -1;
  if (tid == 0) consumed = 0;
  const uint32_t row_mask = (row_bits >= 32) ? 0xffffffffu : ((1u << row_bits) - 1u);
  const int slices = (d + 63) >> 6;
  // the class table, once per block (the item loop resolves a run number
  // from LDS)
  if (tid == 0) {
    uint32_t first = 0;
    for (int c = kHotClassMax; c >= kHotClassMin; --c) {
      const uint32_t k = counters[kHotCountBase + c];
      sm.cls_first[c] = first;
      sm.cls_end[c] = first + k;
      sm.cls_base[c] = (uint32_t)hot_class_base(n, c);
      first += k;
    }
    sm.s_items = first * (uint32_t)slices;
  }
  int32_t base = 0;  // running block number of this block's first ring use in the current item
  for (;;) {
    __syncthreads();
    if (tid == 0) {
      const uint32_t it = atomicAdd(next_item, 1u);
      s_item = it;
      if (it < sm.s_items) {
        const uint32_t run = it / (uint32_t)slices;
        int c = kHotClassMax;
        while (c > kHotClassMin && run >= sm.cls_end[c]) --c;
        sm.s_seg = hot[sm.cls_base[c] + run - sm.cls_first[c]];
      }
    }
    __syncthreads();
    const uint32_t item = s_item;
    if (item >= sm.s_items) break;
    const int32_t s = sm.s_seg;
    const int col0 = (int)(item % slices) * 64;
    const int cols = min(64, d - col0);
    const int32_t beg = seg_start[s], end = seg_start[s + 1];
    const uint32_t key = seg_key[s];
    const int k = (int)(key >> row_bits);
    const int64_t r = (int64_t)(key & row_mask);
    const int32_t nblk = (end - beg + kHB - 1) / kHB;
    if (wave == kAdder) {
      const int32_t len = end - beg;
      const int32_t nfull = len / kHB;
      float acc = 0.f;
      if (nfull > 0) hot_adder_full_blocks(acc, base, nfull, &ring[0][lane * kRS], ready, &consumed);
      if (nfull * kHB < len) {  // the last, partial block
        const int32_t t = nfull;
        while (lds_load(&ready[(base + t) & (kSlots - 1)]) != base + t) __builtin_amdgcn_s_sleep(1);
        compiler_fence();
        const float* col = &ring[(base + t) & (kSlots - 1)][lane * kRS];
        for (int o = 0; o < len - nfull * kHB; ++o) acc = acc + col[o];
        compiler_fence();
        if (lane == 0) consumed = base + t + 1;
      }
      if (lane < cols) {
        float* t = tables[k] + r * d + col0 + lane;
        *t = __fsub_rn(*t, __fmul_rn(lr, acc));
      }
    } else {
      // Loader: lane (c4, sub) = (lane / 4, lane % 4) brings columns
      // 4 c4 .. 4 c4 + 3 of occurrences 4 (sub + 4 m) + r (m, r = 0..3): 16
      // global loads of 16 bytes, each 4 x 4 piece transposed in registers
      // and written as four 16-byte column pieces.  Three blocks of the
      // wave are in flight: while block t is written to its slot, the rows
      // of its next block (t + kLoaders) are loading and the bag ids of the
      // one after.
      const int c4 = min(lane >> 2, cols / 4 - 1);
      const int sub = lane & 3;
      const float* gsrc = G + g_col0 + (int64_t)k * d + col0 + 4 * c4;
      auto occ = [&](int i) { return 4 * (sub + 4 * (i >> 2)) + (i & 3); };
      auto load_bags = [&](int32_t t, int32_t (&bag)[16]) {
        const int32_t q0 = beg + t * kHB, last = end - 1;
#pragma unroll
        for (int i = 0; i < 16; ++i) bag[i] = bags[min(q0 + occ(i), last)];
      };
      // rows of a partial block past its end re-read its last row (bag ids
      // were clamped); the adder never reads them
      auto load_rows = [&](const int32_t (&bag)[16], float4 (&v)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const float4*>(gsrc + (int64_t)bag[i] * g_ld);
      };
      int32_t t = wave < kAdder ? wave : wave - 1;
      int32_t bag[16];
      float4 v[16];
      if (t < nblk) {
        load_bags(t, bag);
        load_rows(bag, v);
        if (t + kLoaders < nblk) load_bags(t + kLoaders, bag);
      }
      for (; t < nblk; t += kLoaders) {
        const int32_t g = base + t;
        const int slot = g & (kSlots - 1);
        float4 vn[16];
        if (t + kLoaders < nblk) {
          load_rows(bag, vn);
          if (t + 2 * kLoaders < nblk) load_bags(t + 2 * kLoaders, bag);
        }
        while (lds_load(&consumed) < g - kSlots + 1) __builtin_amdgcn_s_sleep(1);
        compiler_fence();
        float* dst = &ring[slot][0];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 a = v[4 * m], b = v[4 * m + 1], c = v[4 * m + 2], e = v[4 * m + 3];
          float* p = dst + (4 * c4) * kRS + 4 * (sub + 4 * m);
          *reinterpret_cast<float4*>(p) = make_float4(a.x, b.x, c.x, e.x);
          *reinterpret_cast<float4*>(p + kRS) = make_float4(a.y, b.y, c.y, e.y);
          *reinterpret_cast<float4*>(p + 2 * kRS) = make_float4(a.z, b.z, c.z, e.z);
          *reinterpret_cast<float4*>(p + 3 * kRS) = make_float4(a.w, b.w, c.w, e.w);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the slot is written before its flag
        compiler_fence();
        if (lane == 0) lds_store(&ready[slot], g);
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = vn[i];
      }
    }
    base += nblk;
  }
}

// Short segments (per wave).  A wave takes 64 consecutive segments from a
// shared counter (waves that start early and late share the work as they
// come) and loads what every one of them needs first at once, one segment
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
  for (;;) {
    uint32_t c0 = 0;
    if (lane == 0) c0 = atomicAdd(next, 64u);
    c0 = (uint32_t)__shfl((int)c0, 0, 64);
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

// The hot segments alone (the two-stream form: the short ones run beside it
// on the caller's second stream).
__global__ __launch_bounds__(kApplyThreads) void hot_sgd_kernel(
    float* const* __restrict__ tables, int d, int row_bits, const uint32_t* __restrict__ seg_key,
    const int32_t* __restrict__ bags, const int32_t* __restrict__ seg_start, const int32_t* __restrict__ hot,
    const uint32_t* __restrict__ counters, int64_t n, const float* __restrict__ G, int64_t g_ld, int64_t g_col0,
    float lr,
    uint32_t* __restrict__ next_item) {
  __shared__ __attribute__((aligned(16))) HotLds sm;
  hot_phase(sm, tables, d, row_bits, seg_key, bags, seg_start, hot, counters, n, G, g_ld, g_col0, lr, next_item);
}

// The short segments alone (many small persistent blocks; the two-stream
// form).
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

// The segment sums and the in-place update: hot items first, then the
// short segments, in one launch (one block per CU).
template <int V>
__global__ __launch_bounds__(kApplyThreads) void sgd_apply_kernel(
    float* const* __restrict__ tables, int d, int g_log2, int row_bits, const uint32_t* __restrict__ seg_key,
    const int32_t* __restrict__ bags, const int32_t* __restrict__ seg_start, const int32_t* __restrict__ hot,
    const uint32_t* __restrict__ counters, int64_t n, const float* __restrict__ G, int64_t g_ld, int64_t g_col0,
    float lr, uint32_t* __restrict__ next) {
  __shared__ __attribute__((aligned(16))) HotLds sm;
  // counters: [0] segments, hot runs per class; next: [0] hot item, [1] short-segment chunk
  hot_phase(sm, tables, d, row_bits, seg_key, bags, seg_start, hot, counters, n, G, g_ld, g_col0, lr, &next[0]);
  light_phase<V, 16 / V>(tables, d, g_log2, row_bits, seg_key, bags, seg_start, &counters[0], G, g_ld, g_col0, lr,
                         &next[1]);
}

int bits_for(int64_t x) {  // bits needed to hold 0..x
  int b = 0;
  while (b < 63 && (x >> b) != 0) ++b;
  return b;
}

struct SparseLayout {
  size_t keys[2], vals[2], counts, sums, offsets, seg, seg_key, counters, hot, bytes;
  int64_t tiles;
};

// counters: [0] segments, [2] next hot item, [3] next short-segment chunk,
// [kHotCountBase + c] hot runs of class c (cleared on every prepare)
constexpr int kCounters = 48;
static_assert(kHotCountBase + kHotClassMax < kCounters, "hot class counters");

void sparse_layout(int64_t nnz, SparseLayout* L) {
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
  L->bytes = cv.bytes();
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace
}  // namespace dlrm

namespace dlrm {
namespace {
int sgd_segments(float* const* tables, int d, int row_bits, const uint32_t* seg_key, const int32_t* vals,
                 const int32_t* seg, const int32_t* hot, uint32_t* counters, int64_t n, const float* G,
                 int64_t g_ld, int64_t g_col0, float lr, hipStream_t stream, hipStream_t side);
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
};

int sparse_bufs(int64_t nnz, void* ws, size_t ws_bytes, SparseLayout* L, SparseBufs* b) {
  sparse_layout(nnz, L);
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
  if ((rc = sparse_bufs(nnz, ws, ws_bytes, &L, &b)) != DLRM_OK) return rc;
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
  if ((rc = sparse_bufs(nnz, ws, ws_bytes, &L, &b)) != DLRM_OK) return rc;
  const int cur = sort_plan(row_bits).passes & 1;
  // the work counters start from zero on every call, so one prepared
  // workspace can be applied more than once; each stream clears the counter
  // its own kernel takes work from
  if (side) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, b.counters + 2, 1);
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, side, b.counters + 3, 1);
  } else {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, b.counters + 2, 2);
  }
  if (launch_status() != DLRM_OK) return DLRM_E_HIP;
  return sgd_segments(tables, d, row_bits, b.seg_key, b.vals[cur], b.seg, b.hot, b.counters, nnz, G, g_ld, g_col0,
                      lr, stream, side);
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
  SparseLayout L;
  sparse_layout(nnz, &L);
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
int sgd_segments(float* const* tables, int d, int row_bits, const uint32_t* seg_key, const int32_t* vals,
                 const int32_t* seg, const int32_t* hot, uint32_t* counters, int64_t n, const float* G,
                 int64_t g_ld, int64_t g_col0, float lr, hipStream_t stream, hipStream_t side) {
  // short segments: half as many lanes as float4 columns (two float4 per
  // lane), at most 64
  const int d4 = d / 4;
  int l2 = 0;
  while ((1 << l2) < d4) ++l2;
  const int g_log2 = l2 > 0 ? (l2 - 1 < 6 ? l2 - 1 : 6) : 0;
  const int V = (d4 + (1 << g_log2) - 1) >> g_log2;
  const dim3 cus((unsigned)device_cu_count()), apply_block(kApplyThreads);
  if (side) {
    // long segments on `stream`, short ones on `side` at the same time
    hipLaunchKernelGGL(hot_sgd_kernel, cus, apply_block, 0, stream, tables, d, row_bits, seg_key, vals, seg,
                       hot, counters, n, G, g_ld, g_col0, lr, counters + 2);
    if (launch_status() != DLRM_OK) return DLRM_E_HIP;
    const dim3 grid(kLightBlocks), block(256);
#define DLRM_LIGHT(VV)                                                                                            \
  hipLaunchKernelGGL((light_sgd_kernel<VV>), grid, block, 0, side, tables, d, g_log2, row_bits, seg_key, vals, seg, \
                     counters, G, g_ld, g_col0, lr, counters + 3)
    if (V == 1) DLRM_LIGHT(1);
    else if (V == 2) DLRM_LIGHT(2);
    else DLRM_LIGHT(4);
#undef DLRM_LIGHT
    return launch_status();
  }
#define DLRM_APPLY(VV)                                                                                          \
  hipLaunchKernelGGL((sgd_apply_kernel<VV>), cus, apply_block, 0, stream, tables, d, g_log2, row_bits, seg_key, \
                     vals, seg, hot, counters, n, G, g_ld, g_col0, lr, counters + 2)
  if (V == 1) DLRM_APPLY(1);
  else if (V == 2) DLRM_APPLY(2);
  else DLRM_APPLY(4);
#undef DLRM_APPLY
  return launch_status();
}
}  // namespace
}  // namespace dlrm
