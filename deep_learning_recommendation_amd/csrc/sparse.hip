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
// chain the latency floor.  Segments of at least kHot occurrences go to a
// producer/consumer kernel: per (segment, 64-column slice) one wave adds, one
// column per lane, from an LDS ring that seven other waves keep filled with
// direct global-to-LDS loads, so the serial adds never wait on memory.  Hot
// items are handed out longest first.  The remaining (short) segments take
// one lane group each.
#include "common.hpp"

#include <mutex>

namespace dlrm {
namespace {

constexpr int RT = 256;                // threads per sort block
constexpr int RITEMS = 16;             // keys per thread per tile
constexpr int RTILE = RT * RITEMS;     // 4096 keys per tile
constexpr int SCAN_ITEMS = 8;
constexpr int SCAN_TILE = 256 * SCAN_ITEMS;
constexpr int kHot = 128;              // occurrences from which a segment is "hot"
constexpr int kHotBlocks = 256;        // persistent blocks of the hot kernel (one per CU)
constexpr int kHB = 64;                // occurrences per LDS ring slot
constexpr int kSlots = 8;              // ring slots
constexpr int kRS = kHB + 4;           // floats per column row of a slot (padded: conflict-free 16-byte reads)
constexpr int kLoaders = 6;            // loader waves per hot block (plus one adder)
constexpr int kAdder = 3;              // the adder's wave index: alone on its SIMD when waves go round-robin
constexpr int kLightBlocks = 2048;

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

__global__ __launch_bounds__(RT) void radix_hist_kernel(const uint32_t* __restrict__ keys, int n, int shift,
                                                        uint32_t* __restrict__ hist, int nblocks) {
  __shared__ uint32_t cnt[256];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int base = blockIdx.x * RTILE;
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // lanes with equal digits found by eight ballots; the lowest of them adds
  // the group's count (Zipf keys share digits, so one atomic per group
  // instead of one per key)
  uint32_t kv[RITEMS];
#pragma unroll
  for (int i = 0; i < RITEMS; ++i) {
    const int p = base + i * RT + threadIdx.x;
    kv[i] = p < n ? keys[p] : 0u;
  }
#pragma unroll
  for (int i = 0; i < RITEMS; ++i) {
    const int p = base + i * RT + threadIdx.x;
    const bool valid = p < n;
    const uint32_t digit = (kv[i] >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (digit >> b) & 1u;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    if (valid && (peers & lt) == 0ull) atomicAdd(&cnt[digit], (uint32_t)__popcll(peers));
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
                                                               uint32_t* __restrict__ seg_key,
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
    if (v[i]) {
      seg_start[run] = (int32_t)(base + i);
      seg_key[run] = keys[base + i];
    }
    run += v[i];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) seg_start[*nseg] = (int32_t)n;
}

__global__ __launch_bounds__(256) void find_hot_kernel(const int32_t* __restrict__ seg_start,
                                                       const uint32_t* __restrict__ nseg, int32_t* __restrict__ hot,
                                                       uint32_t* __restrict__ nhot) {
  const uint32_t U = *nseg;
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint32_t stride = gridDim.x * blockDim.x;
  // every lane of a wave runs the same number of iterations (ballots below)
  for (uint32_t s0 = blockIdx.x * blockDim.x; s0 < U; s0 += stride) {
    const uint32_t s = s0 + threadIdx.x;
    const bool is_hot = s < U && seg_start[s + 1] - seg_start[s] >= kHot;
    const uint64_t m = __ballot(is_hot);
    if (m == 0ull) continue;
    uint32_t at = 0;
    if (lane == __ffsll((long long)m) - 1) at = atomicAdd(nhot, (uint32_t)__popcll(m));
    at = __shfl(at, __ffsll((long long)m) - 1, 64);
    if (is_hot) hot[at + __popcll(m & below)] = (int32_t)s;
  }
}

// One block: hot segments regrouped by floor(log2(length)), longest group
// first, so the longest serial chains start first (order inside a group is
// arbitrary; every segment's result is independent of it).
__global__ __launch_bounds__(256) void order_hot_kernel(const int32_t* __restrict__ seg_start,
                                                        const int32_t* __restrict__ hot,
                                                        const uint32_t* __restrict__ nhot,
                                                        int32_t* __restrict__ ordered) {
  __shared__ uint32_t cnt[32];
  const uint32_t n = *nhot;
  if (threadIdx.x < 32) cnt[threadIdx.x] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int32_t h = hot[i];
    atomicAdd(&cnt[31 - __clz(seg_start[h + 1] - seg_start[h])], 1u);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t c = cnt[b];
      cnt[b] = run;
      run += c;
    }
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int32_t h = hot[i];
    ordered[atomicAdd(&cnt[31 - __clz(seg_start[h + 1] - seg_start[h])], 1u)] = h;
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

// Hot segments.  A block (7 waves) takes (segment, 64-column slice) items
// from a global counter.  Wave kAdder is the adder (the only wave on its
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
__global__ __launch_bounds__(64 * (kLoaders + 1)) void hot_sgd_kernel(float* const* __restrict__ tables, int d, int row_bits,
                                                      const uint32_t* __restrict__ seg_key,
                                                      const int32_t* __restrict__ bags,
                                                      const int32_t* __restrict__ seg_start,
                                                      const int32_t* __restrict__ hot,
                                                      const uint32_t* __restrict__ nhot,
                                                      const float* __restrict__ G, int64_t g_ld, int64_t g_col0,
                                                      float lr, uint32_t* __restrict__ next_item) {
  __shared__ __attribute__((aligned(16))) float ring[kSlots][64 * kRS];
  __shared__ int32_t ready[kSlots];
  __shared__ int32_t consumed;
  __shared__ uint32_t s_item;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kSlots) ready[tid] = -1;
  if (tid == 0) consumed = 0;
  const uint32_t row_mask = (row_bits >= 32) ? 0xffffffffu : ((1u << row_bits) - 1u);
  const int slices = (d + 63) >> 6;
  const uint32_t items = *nhot * (uint32_t)slices;
  int32_t base = 0;  // running block number of this block's first ring use in the current item
  for (;;) {
    __syncthreads();
    if (tid == 0) s_item = atomicAdd(next_item, 1u);
    __syncthreads();
    const uint32_t item = s_item;
    if (item >= items) break;
    const int32_t s = hot[item / slices];
    const int col0 = (int)(item % slices) * 64;
    const int cols = min(64, d - col0);
    const int32_t beg = seg_start[s], end = seg_start[s + 1];
    const uint32_t key = seg_key[s];
    const int k = (int)(key >> row_bits);
    const int64_t r = (int64_t)(key & row_mask);
    const int32_t nblk = (end - beg + kHB - 1) / kHB;
    if (wave == kAdder) {
      // The adds run as one stream over the full blocks, 16 values (four
      // 16-byte LDS reads) per step, with the reads issued three steps
      // ahead: twelve reads in flight (lgkmcnt counts up to 15).  Measured
      // on one wave, wider steps keep the adder closest to its add rate.
      constexpr int kStep = 16, kAhead = 3, kSteps = kHB / kStep, kBufs = 4, kReads = kStep / 4;
      const int32_t len = end - beg;
      const int32_t nfull = len / kHB;
      float acc = 0.f;
      float v[kBufs][kStep];
      // occurrences kStep * st .. + kStep - 1 of this lane's column
      auto step_load = [&](int32_t t, int st, float* dst) {
        const float* p = &ring[(base + t) & (kSlots - 1)][lane * kRS + st * kStep];
#pragma unroll
        for (int q = 0; q < kStep; q += 4) {
          const float4 a = *reinterpret_cast<const float4*>(p + q);
          dst[q] = a.x;
          dst[q + 1] = a.y;
          dst[q + 2] = a.z;
          dst[q + 3] = a.w;
        }
      };
      auto wait_ready = [&](int32_t t) {
        while (lds_load(&ready[(base + t) & (kSlots - 1)]) != base + t) __builtin_amdgcn_s_sleep(1);
        compiler_fence();
      };
      // The next block's flag is read with a plain LDS load just before its
      // first data reads and checked at the end of this block.  One wave's
      // LDS accesses execute in order and a loader writes its flag only
      // after its data writes have completed, so a flag that shows the block
      // proves the data reads after it saw the data; otherwise (rare) those
      // reads are repeated once the flag is up.  Plain accesses keep the
      // compiler's waits exact (an atomic or a loop-carried use would drain
      // every read in flight).
      auto flag = [&](int32_t t) { return ready[(base + t) & (kSlots - 1)]; };
      if (nfull > 0) {
        wait_ready(0);
#pragma unroll
        for (int st = 0; st < kAhead; ++st) step_load(0, st, v[st]);
      }
      for (int32_t t = 0; t < nfull; ++t) {
        const bool more = t + 1 < nfull;
        const int32_t tn = more ? t + 1 : t;
        int32_t fl = base + tn;
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          // reads kAhead steps ahead, then this step's adds; the scheduling
          // barrier keeps the compiler from hoisting every read to the top
          if (st + kAhead == kSteps) {
            compiler_fence();
            fl = flag(tn);
            compiler_fence();
          }
          if (st + kAhead < kSteps)
            step_load(t, st + kAhead, v[(st + kAhead) & (kBufs - 1)]);
          else
            step_load(tn, st + kAhead - kSteps, v[(st + kAhead) & (kBufs - 1)]);
          // this step's values were read kAhead steps ago: the kAhead * kReads
          // younger reads (and at most one flag access) may still be in flight
          __builtin_amdgcn_s_waitcnt(0xc07f & ~0x0f00 | ((kAhead * kReads) << 8));
#pragma unroll
          for (int o = 0; o < kStep; ++o) acc = acc + v[st & (kBufs - 1)][o];
          __asm__ volatile("" : "+v"(acc));  // this step's adds stay in this step
          __builtin_amdgcn_sched_barrier(0);
        }
        compiler_fence();
        if (lane == 0) consumed = base + t + 1;
        if (more && fl != base + t + 1) {  // the next block's first reads came too early
          wait_ready(t + 1);
#pragma unroll
          for (int st = 0; st < kAhead; ++st) step_load(t + 1, st, v[st]);
        }
      }
      if (nfull * kHB < len) {  // the last, partial block
        const int32_t t = nfull;
        wait_ready(t);
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

// Short segments: a group of 2^g_log2 lanes (V float4 each) per segment.
// The group loads up to one bag id per lane at once, then walks the bags in
// order with U gradient rows in flight, broadcasting each bag id from its lane.
// Waves take chunks of kLightChunk segments per group from a shared counter,
// so the blocks that become resident early (beside the hot kernel) and late
// (after its short items end) share the work as they come.
constexpr int kLightChunk = 16;
template <int V>
__global__ __launch_bounds__(256) void light_sgd_kernel(float* const* __restrict__ tables, int d, int g_log2,
                                                        int row_bits, const uint32_t* __restrict__ seg_key,
                                                        const int32_t* __restrict__ bags,
                                                        const int32_t* __restrict__ seg_start,
                                                        const uint32_t* __restrict__ nseg,
                                                        const float* __restrict__ G, int64_t g_ld, int64_t g_col0,
                                                        float lr, uint32_t* __restrict__ next) {
  constexpr int U = 8 / V;
  const int lane = threadIdx.x & 63;
  const uint32_t row_mask = (row_bits >= 32) ? 0xffffffffu : ((1u << row_bits) - 1u);
  const int GL = 1 << g_log2;  // lanes per group
  const int gl = lane & (GL - 1);
  const int wgroups = 64 >> g_log2;  // groups per wave
  const int grp = lane >> g_log2;
  const int d4 = d >> 2;
  const uint32_t nsegs = *nseg;
  const uint32_t per_wave = (uint32_t)(wgroups * kLightChunk);
  for (;;) {
    uint32_t c0 = 0;
    if (lane == 0) c0 = atomicAdd(next, per_wave);
    c0 = (uint32_t)__shfl((int)c0, 0, 64);
    if (c0 >= nsegs) break;  // whole wave
    for (int i = 0; i < kLightChunk; ++i) {
      const uint32_t s = c0 + (uint32_t)(i * wgroups + grp);
      if (s >= nsegs) break;  // whole group (later segments of the chunk are past the end too)
      const int32_t beg = seg_start[s], end = seg_start[s + 1];
      const uint32_t key = seg_key[s];
      if (end - beg >= kHot) continue;
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
      for (int32_t q0 = beg; q0 < end; q0 += GL) {
        const int m = min(GL, end - q0);
        const int32_t my_bag = gl < m ? bags[q0 + gl] : 0;
        for (int u0 = 0; u0 < m; u0 += U) {
          float4 v[U][V];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const bool ok = u0 + u < m;
            const int64_t bag = __shfl(my_bag, ok ? u0 + u : 0, GL);
            const float4* grow = reinterpret_cast<const float4*>(gbase + bag * g_ld);
#pragma unroll
            for (int j = 0; j < V; ++j) {
              const int c4 = gl + j * GL;
              v[u][j] = (ok && c4 < d4) ? grow[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (u0 + u < m) {
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
}

int bits_for(int64_t x) {  // bits needed to hold 0..x
  int b = 0;
  while (b < 63 && (x >> b) != 0) ++b;
  return b;
}

struct SparseLayout {
  size_t keys[2], vals[2], hist, bsum, seg, seg_key, counters, hot, hot_ordered, bytes;
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
  L->seg_key = take(4 * (size_t)n);
  L->counters = take(4 * 16);
  L->hot = take(4 * (size_t)(n / kHot + 1));
  L->hot_ordered = take(4 * (size_t)(n / kHot + 1));
  L->bytes = cv.bytes();
}

// A second stream per device (default priority) for the short segments,
// which run beside the hot-segment kernel: that kernel's critical path is a
// few serial chains on a few CUs while the rest of the chip would idle.
hipStream_t side_stream() {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev]) {
    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    streams[dev] = s;
  }
  return streams[dev];
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

}  // namespace
}  // namespace dlrm

namespace dlrm {
namespace {
int sgd_segments(float* const* tables, int d, int row_bits, const uint32_t* seg_key, const int32_t* vals,
                 const int32_t* seg, const int32_t* hot_ordered, uint32_t* counters, const float* G, int64_t g_ld,
                 int64_t g_col0, float lr, hipStream_t stream, hipStream_t side);
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
  uint32_t* hist;
  uint32_t* bsum;
  int32_t* seg;
  uint32_t* seg_key;
  uint32_t* counters;  // [0] segments, [1] hot segments, [2] next hot item, [3] next short-segment chunk
  int32_t* hot;
  int32_t* hot_ordered;
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
  b->hist = reinterpret_cast<uint32_t*>(w + L->hist);
  b->bsum = reinterpret_cast<uint32_t*>(w + L->bsum);
  b->seg = reinterpret_cast<int32_t*>(w + L->seg);
  b->seg_key = reinterpret_cast<uint32_t*>(w + L->seg_key);
  b->counters = reinterpret_cast<uint32_t*>(w + L->counters);
  b->hot = reinterpret_cast<int32_t*>(w + L->hot);
  b->hot_ordered = reinterpret_cast<int32_t*>(w + L->hot_ordered);
  return DLRM_OK;
}

// Sort passes for the key width: the sorted keys and bag ids end in buffer
// passes % 2.
int sort_passes(int row_bits, int table_bits) { return (row_bits + table_bits + 7) / 8; }
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

  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, b.counters, 16);
  {
    int kg = 0;  // lanes per bag: the mean bag length rounded up to a power of two, at most 64
    while ((1LL << kg) * KB < nnz && kg < 6) ++kg;
    const int64_t kblocks = ceil_div(KB << kg, 256);
    if (kblocks > 0x7fffffffLL) return DLRM_E_UNSUPPORTED;
    hipLaunchKernelGGL(build_keys_kernel, dim3((unsigned)kblocks), dim3(256), 0, stream, indices, offsets, KB, B, kg,
                       row_bits, b.keys[0], b.vals[0]);
  }
  const int passes = sort_passes(row_bits, table_bits);
  const int nblocks = (int)L.nblocks;
  int cur = 0;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * 8;
    hipLaunchKernelGGL(radix_hist_kernel, dim3(nblocks), dim3(RT), 0, stream, b.keys[cur], n, shift, b.hist, nblocks);
    hipLaunchKernelGGL((scan_reduce_kernel<ArrayIn>), dim3((unsigned)L.scan_nb_hist), dim3(256), 0, stream,
                       ArrayIn{b.hist}, L.hist_n, b.bsum);
    hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(256), 0, stream, b.bsum, (int)L.scan_nb_hist, nullptr);
    hipLaunchKernelGGL(scan_apply_array_kernel, dim3((unsigned)L.scan_nb_hist), dim3(256), 0, stream, b.hist,
                       L.hist_n, b.bsum, b.hist);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(nblocks), dim3(RT), 0, stream, b.keys[cur], b.vals[cur],
                       b.keys[cur ^ 1], b.vals[cur ^ 1], n, shift, b.hist, nblocks);
    cur ^= 1;
  }
  // run-length segmentation of the sorted keys
  hipLaunchKernelGGL((scan_reduce_kernel<HeadIn>), dim3((unsigned)L.scan_nb_keys), dim3(256), 0, stream,
                     HeadIn{b.keys[cur]}, (int64_t)n, b.bsum);
  hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(256), 0, stream, b.bsum, (int)L.scan_nb_keys, &b.counters[0]);
  hipLaunchKernelGGL(scan_apply_heads_kernel, dim3((unsigned)L.scan_nb_keys), dim3(256), 0, stream, b.keys[cur],
                     (int64_t)n, b.bsum, b.seg, b.seg_key, &b.counters[0]);
  hipLaunchKernelGGL(find_hot_kernel, dim3(1024), dim3(256), 0, stream, b.seg, &b.counters[0], b.hot, &b.counters[1]);
  hipLaunchKernelGGL(order_hot_kernel, dim3(1), dim3(256), 0, stream, b.seg, b.hot, &b.counters[1], b.hot_ordered);
  return launch_status() != DLRM_OK ? DLRM_E_HIP : DLRM_OK;
}

extern "C" int dlrm_embbag_bwd_sgd_apply(float* const* tables, int32_t K, int32_t d, const int64_t* rows, int64_t B,
                                         int64_t nnz, const float* G, int64_t g_ld, int64_t g_col0, float lr, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
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
  const int cur = sort_passes(row_bits, table_bits) & 1;
  // the work counters start from zero on every call, so one prepared
  // workspace can be applied more than once
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, b.counters + 2, 2);
  if (launch_status() != DLRM_OK) return DLRM_E_HIP;
  // per-segment sums and the in-place update: the long segments on `stream`,
  // the short ones (disjoint rows) on the side stream at the same time, joined
  // back into `stream` before returning
  hipStream_t side = side_stream();
  hipEvent_t fork = nullptr, join = nullptr;
  if (!side || hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess) return DLRM_E_HIP;
  if (hipEventCreateWithFlags(&join, hipEventDisableTiming) != hipSuccess) {
    (void)hipEventDestroy(fork);
    return DLRM_E_HIP;
  }
  if (hipEventRecord(fork, stream) != hipSuccess || hipStreamWaitEvent(side, fork, 0) != hipSuccess) rc = DLRM_E_HIP;
  if (rc == DLRM_OK)
    rc = sgd_segments(tables, d, row_bits, b.seg_key, b.vals[cur], b.seg, b.hot_ordered, b.counters, G, g_ld, g_col0,
                      lr, stream, side);
  // the join is recorded even after a failed launch, so `stream` never
  // waits on an event that was not recorded
  if (hipEventRecord(join, side) != hipSuccess || hipStreamWaitEvent(stream, join, 0) != hipSuccess) rc = DLRM_E_HIP;
  (void)hipEventDestroy(fork);
  (void)hipEventDestroy(join);
  return rc;
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
  return dlrm_embbag_bwd_sgd_apply(tables, K, d, rows, B, nnz, G, g_ld, g_col0, lr, ws, ws_bytes, stream);
}

namespace dlrm {
namespace {
int sgd_segments(float* const* tables, int d, int row_bits, const uint32_t* seg_key, const int32_t* vals,
                 const int32_t* seg, const int32_t* hot_ordered, uint32_t* counters, const float* G, int64_t g_ld,
                 int64_t g_col0, float lr, hipStream_t stream, hipStream_t side) {
  hipLaunchKernelGGL(hot_sgd_kernel, dim3(kHotBlocks), dim3(64 * (kLoaders + 1)), 0, stream, tables, d, row_bits, seg_key,
                     vals, seg, hot_ordered, &counters[1], G, g_ld, g_col0, lr, &counters[2]);
  if (launch_status() != DLRM_OK) return DLRM_E_HIP;
  // short segments: half as many lanes as float4 columns (two float4 per
  // lane), at most 64
  const int d4 = d / 4;
  int l2 = 0;
  while ((1 << l2) < d4) ++l2;
  const int g_log2 = l2 > 0 ? (l2 - 1 < 6 ? l2 - 1 : 6) : 0;
  const int V = (d4 + (1 << g_log2) - 1) >> g_log2;
  const dim3 grid(kLightBlocks), block(256);
  if (V == 1)
    hipLaunchKernelGGL((light_sgd_kernel<1>), grid, block, 0, side, tables, d, g_log2, row_bits, seg_key, vals, seg,
                       &counters[0], G, g_ld, g_col0, lr, &counters[3]);
  else if (V == 2)
    hipLaunchKernelGGL((light_sgd_kernel<2>), grid, block, 0, side, tables, d, g_log2, row_bits, seg_key, vals, seg,
                       &counters[0], G, g_ld, g_col0, lr, &counters[3]);
  else
    hipLaunchKernelGGL((light_sgd_kernel<4>), grid, block, 0, side, tables, d, g_log2, row_bits, seg_key, vals, seg,
                       &counters[0], G, g_ld, g_col0, lr, &counters[3]);
  return launch_status();
}
}  // namespace
}  // namespace dlrm
