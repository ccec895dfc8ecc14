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
// columns 4*(l / 16) .. +3.  Two chunks side by side give each lane eight
// values of one row, the operand shape of v_mfma_f32_16x16x32_bf16 (the k
// order inside the 32 columns is permuted, identically for both operands).
//
// Precision: the inputs are fp32 and the pairs need about fp32 accuracy, but
// bf16 MFMA runs at 16 times the fp32 MFMA rate.  Every value is split
// exactly into three bf16 parts, v = h + m + l (h: the top 8 significant
// bits by truncation, m: the top 8 of the remainder, l: the rest, which has
// at most 8 significant bits), and the Gram block sums the six products
// hh, hm, mh, hl, mm, lh with fp32 accumulation.  Each bf16 product is exact
// in fp32; the dropped terms ml, lm, ll are below 2^-20 |a b|, so with the
// fp32 accumulation error the result stays within a few 1e-6 of
// sum_c |x_ic x_jc|.  Six bf16 products cost 6/16 of one fp32 MFMA pass.
// Only blocks with J <= I are computed.  The packed output row is assembled
// in LDS and written with full 16-byte stores.  The kernel is bound by HBM
// (reading X, writing the packed rows).
#include "common.hpp"

#include <type_traits>

namespace dlrm {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Exact split of eight fp32 values (a then b) into bf16 parts h + m + l.
// Both subtractions are exact (each operand pair shares a binade), and the
// final remainder has at most 8 significant bits, so it is a bf16 value.
struct Parts {
  bf16x8 h, m, l;
};
__device__ __forceinline__ Parts split3(f4 a, f4 b) {
  uint32_t hb[8], mb[8], lb[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float v = k < 4 ? a[k] : b[k - 4];
    const uint32_t u = __float_as_uint(v);
    const float r1 = v - __uint_as_float(u & 0xffff0000u);
    const uint32_t ur = __float_as_uint(r1);
    const float r2 = r1 - __uint_as_float(ur & 0xffff0000u);
    hb[k] = u;
    mb[k] = ur;
    lb[k] = __float_as_uint(r2);
  }
  u32x4 h, m, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = (hb[2 * i] >> 16) | (hb[2 * i + 1] & 0xffff0000u);
    m[i] = (mb[2 * i] >> 16) | (mb[2 * i + 1] & 0xffff0000u);
    l[i] = (lb[2 * i] >> 16) | (lb[2 * i + 1] & 0xffff0000u);
  }
  return Parts{__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, m), __builtin_bit_cast(bf16x8, l)};
}

// acc += the six significant products of the split rows p (tile I) and q (tile J)
__device__ __forceinline__ f4 gram6(const Parts& p, const Parts& q, f4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p.l, q.h, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p.h, q.l, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p.m, q.m, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p.m, q.h, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p.h, q.m, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(p.h, q.h, acc, 0, 0, 0);
}

__device__ __forceinline__ void put(float* p, float v) { *p = v; }
__device__ __forceinline__ void put(uint16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void put4(float* p, f4 v) { *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ void put4(uint16_t* p, f4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// Where the rows of X come from: a materialised X, or (fused path) row 0
// from the bottom MLP output and rows 1..K pooled on the fly from the tables.
struct RowSource {
  const float* X;                 // X (plain) or x_dense rows (fused)
  int64_t x_ld;
  const float* const* tables;     // fused only
  const int64_t* idx;
  const int64_t* off;
  const float* const* scale_bias;  // fused from int8 rows only: per-row (scale, bias)
};

// Formats of the table rows the fused kernel reads: fp32 (four columns per
// 16-byte load); bf16 (widened exactly) and int8 with the row's scale s and
// bias z, value (s * q) + z with two fp32 roundings (no fused multiply-add),
// eight consecutive columns per load.
struct FRowF32 {
  typedef float T;
  static constexpr bool kScaled = false;
};
struct FRowBF16 {
  typedef uint16_t T;
  static constexpr bool kScaled = false;
  // columns col .. col + 7 (16 bytes)
  __device__ static void load8(const T* row, int col, float2, f4& lo, f4& hi) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 u = *(const __attribute__((address_space(1))) u32x4*)(row + col);
    lo = f4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
            __uint_as_float(u[1] & 0xffff0000u)};
    hi = f4{__uint_as_float(u[2] << 16), __uint_as_float(u[2] & 0xffff0000u), __uint_as_float(u[3] << 16),
            __uint_as_float(u[3] & 0xffff0000u)};
  }
};
struct FRowI8 {
  typedef int8_t T;
  static constexpr bool kScaled = true;
  // columns col .. col + 7 (8 bytes)
  __device__ static void load8(const T* row, int col, float2 sz, f4& lo, f4& hi) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 u = *(const __attribute__((address_space(1))) u32x2*)(row + col);
    auto deq = [&](uint32_t w, int sh) { return __fadd_rn(__fmul_rn(sz.x, (float)(int8_t)(w >> sh)), sz.y); };
    lo = f4{deq(u[0], 0), deq(u[0], 8), deq(u[0], 16), deq(u[0], 24)};
    hi = f4{deq(u[1], 0), deq(u[1], 8), deq(u[1], 16), deq(u[1], 24)};
  }
};

// Gram blocks of one sample held in registers (x[t][c]: rows t*16 + lane%16,
// columns col_of(c, lane/16) .. +3) into the sample's packed output row `ob`
// (in LDS): dense vector first, then the strict lower triangle row by row,
// then zeros up to pad_end.  The k loop is outermost so the MFMAs of all
// blocks (J <= I) interleave as independent accumulation chains; a single
// block is split into two partial chains.
// 16-byte load through a global-address-space pointer (a plain pointer that
// came out of memory would otherwise turn into a flat load)
__device__ __forceinline__ f4 ld4(const float* p) { return *(const __attribute__((address_space(1))) f4*)(p); }

// Pointer select with both operands computed up front: keeps the compiler
// from moving the address arithmetic into a branch (a branch before a load
// makes the loads after it wait for every load before it).
__device__ __forceinline__ const float* pick(bool c, const float* a, const float* b) {
  uint64_t ua = reinterpret_cast<uint64_t>(a), ub = reinterpret_cast<uint64_t>(b);
  __asm__ volatile("" : "+v"(ua), "+v"(ub));
  return reinterpret_cast<const float*>(c ? ua : ub);
}

// Column of register chunk c for lane group g: 16-wide chunks, four columns
// each (WIDE = false), or 32-wide chunk pairs, eight consecutive columns each
// (WIDE: one 16-byte load of a low-precision row).  Every row of a sample uses
// the same mapping, so the Gram matrix sees one consistent k order.
template <bool WIDE>
__device__ __forceinline__ int col_of(int c, int g) {
  return WIDE ? 32 * (c >> 1) + 8 * g + 4 * (c & 1) : c * 16 + 4 * g;
}

template <int NT, int DC, typename OutT, bool WIDE = false>
__device__ __forceinline__ void gram_row(f4 (&x)[NT][DC], int n, int d, int pad_end, OutT* ob, int lane) {
  const int r16 = lane & 15, g = lane >> 4;
  if (r16 == 0) {  // row 0 lives in lanes 0, 16, 32, 48 of tile 0
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int kk = col_of<WIDE>(c, g);
      if (kk < d) put4(ob + kk, x[0][c]);
    }
  }
  // D[i][j] of block (I, J): lane holds i = 16 I + a_r (a_r = 4 (l/16) + r)
  // and j = 16 J + l % 16, whose packed position d + i (i - 1) / 2 + j is
  // P_r + I Q_r + (128 I^2 - 8 I + 16 J) with the per-lane P_r = d +
  // a_r (a_r - 1) / 2 + l % 16 and Q_r = 16 a_r, so each store costs one
  // multiply-add; lanes off the strict lower triangle (or past row n) are
  // masked off.
  int P[4], Q[4];
  bool below[4];  // j < i inside a diagonal block
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int a = 4 * g + r;
    P[r] = d + a * (a - 1) / 2 + r16;
    Q[r] = 16 * a;
    below[r] = r16 < a;
  }
  auto store_block = [&](int I, int J, f4 v) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool keep = I * 16 + 4 * g + r < n && (J < I || below[r]);
      if (keep) put(ob + (P[r] + I * Q[r] + (128 * I * I - 8 * I + 16 * J)), v[r]);
    }
  };
  // chunk pairs (2p, 2p + 1); an odd last chunk pairs with zeros
  constexpr int DP = (DC + 1) / 2;
  auto parts = [&](int t, int p) {
    return split3(x[t][2 * p], 2 * p + 1 < DC ? x[t][2 * p + 1] : f4{0.f, 0.f, 0.f, 0.f});
  };
  if constexpr (NT <= 2) {
    // every block live at once, the rows split one chunk pair at a time; a
    // single block runs as two partial chains
    constexpr int NB = NT * (NT + 1) / 2;
    constexpr int NCH = NB == 1 ? 2 : 1;
    f4 acc[NB][NCH];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int h = 0; h < NCH; ++h) acc[q][h] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < DP; ++p) {
      Parts xs[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) xs[t] = parts(t, p);
      int q = 0;
#pragma unroll
      for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = 0; J <= I; ++J, ++q) acc[q][p % NCH] = gram6(xs[I], xs[J], acc[q][p % NCH]);
    }
    int q = 0;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J, ++q) store_block(I, J, NCH == 2 ? acc[q][0] + acc[q][NCH - 1] : acc[q][0]);
  } else {
    // all rows split once, then one block row at a time (bounded
    // accumulator registers)
    Parts xs[NT][DP];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int p = 0; p < DP; ++p) xs[t][p] = parts(t, p);
#pragma unroll
    for (int I = 0; I < NT; ++I) {
      f4 acc[NT];
#pragma unroll
      for (int J = 0; J < NT; ++J) acc[J] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < DP; ++p)
#pragma unroll
        for (int J = 0; J <= I; ++J) acc[J] = gram6(xs[I][p], xs[J][p], acc[J]);
#pragma unroll
      for (int J = 0; J <= I; ++J) store_block(I, J, acc[J]);
    }
  }
  const int end = d + n * (n - 1) / 2;
  for (int col = end + lane; col < pad_end; col += 64) put(ob + col, 0.f);
}

// Copy a wave's finished row from LDS to global memory in 16-byte (or
// 8-byte) chunks.
__device__ __forceinline__ void row_out(const char* rowb, char* dst, int bytes, int wide, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int off = 0;
  if (wide) {
    for (off = lane * 16; off + 16 <= bytes; off += 64 * 16)
      *reinterpret_cast<uint4*>(dst + off) = *reinterpret_cast<const uint4*>(rowb + off);
    off = bytes & ~15;
  }
  for (int o = off + lane * 8; o + 8 <= bytes; o += 64 * 8)
    *reinterpret_cast<uint2*>(dst + o) = *reinterpret_cast<const uint2*>(rowb + o);
  // the row buffer is reused by this wave's next sample
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Materialised X: one wave per sample, at least two waves per SIMD (the
// split rows of the largest shapes would otherwise take the whole register
// file).
template <int NT, int DC, typename OutT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void interact_mfma_kernel(RowSource src, int64_t B, int n, int d,
                                                            OutT* __restrict__ out, int64_t out_ld, int pad_end,
                                                            int row_bytes, int wide) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  if (b >= B) return;  // whole wave
  char* rowb = smem + wave * row_bytes;
  const int r16 = lane & 15, g = lane >> 4;
  const float* __restrict__ xb = src.X + b * src.x_ld;
  // every load is issued (rows past n re-read row 0, columns past d the last
  // four) and masked afterwards, so that the loads go out back to back
  f4 x[NT][DC];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int row = t * 16 + r16;
    const float* rp = xb + (int64_t)(row < n ? row : 0) * d;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int kk = c * 16 + 4 * g;
      x[t][c] = ld4(rp + (kk < d ? kk : d - 4));
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int c = 0; c < DC; ++c)
      if (!(t * 16 + r16 < n && c * 16 + 4 * g < d)) x[t][c] = f4{0.f, 0.f, 0.f, 0.f};
  gram_row<NT, DC, OutT>(x, n, d, pad_end, reinterpret_cast<OutT*>(rowb), lane);
  row_out(rowb, reinterpret_cast<char*>(out + b * out_ld), pad_end * (int)sizeof(OutT), wide, lane);
}

// Fused pooled lookup + interaction: one wave per sample.  Row 0 is the
// dense vector, row 1 + k the pooled bag (k, b), summed in bag order from +0
// exactly as the standalone lookup.  All bag offsets of the sample are read
// first, then all first indices, then all rows, so each dependent step has
// every load of the sample in flight.
// Register budget per lane: the rows (4 per column chunk and tile), bag
// metadata, and for the persistent form the next sample's metadata.  Small
// shapes run persistent (metadata of sample b + stride loaded during sample
// b) at 4 waves per SIMD; larger ones one sample per wave, where the extra
// metadata would cost a wave of occupancy (measured slower).
template <int NT, int DC>
constexpr bool fused_persistent() { return NT <= 2 && NT * DC <= 8; }
template <int NT, int DC>
constexpr int fused_waves() {
  return fused_persistent<NT, DC>() ? 4 : (NT * (4 * DC + 12) < 112 ? 4 : 2);
}

template <int NT, int DC, typename OutT, typename R = FRowF32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(fused_waves<NT, DC>()))) void fused_kernel(
    RowSource src, int64_t B, int n, int d, OutT* __restrict__ out,
                                                    int64_t out_ld, int pad_end, int row_bytes, int wide) {
  constexpr bool kF32 = std::is_same<R, FRowF32>::value;
  typedef typename R::T TT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int64_t stride = (int64_t)gridDim.x * waves;
  int64_t b = (int64_t)blockIdx.x * waves + wave;
  char* rowb = smem + wave * row_bytes;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t* __restrict__ off = src.off;
  const int64_t* __restrict__ idx = src.idx;
  constexpr bool kPersist = fused_persistent<NT, DC>();
  // One sample per wave: the block's bag offsets are loaded together.  For
  // table k the waves' bags start and end at off[k B + s0 .. s0 + waves],
  // neighbours in memory, so the block asks for (n - 1) (waves + 1)
  // consecutive-by-table values instead of every wave asking for its own
  // 2 (n - 1) scattered ones.
  const int per = waves + 1;
  const int64_t* so = reinterpret_cast<const int64_t*>(smem + waves * row_bytes);
  if constexpr (!kPersist) {
    const int64_t s0 = (int64_t)blockIdx.x * waves, last = (int64_t)(n - 1) * B;
    int64_t* sw = reinterpret_cast<int64_t*>(smem + waves * row_bytes);
    for (int t = threadIdx.x; t < (n - 1) * per; t += blockDim.x) {
      const int64_t pos = (int64_t)(t / per) * B + s0 + t % per;
      sw[t] = off[pos < last ? pos : last];
    }
    __syncthreads();
  }
  if (b >= B) return;  // whole wave

  // Every load below is issued unconditionally from a valid address (lanes
  // with nothing to load read the offsets array or the dense row) and masked
  // afterwards: with no branch between them the loads of one level go out
  // back to back instead of one memory latency each.  The wave walks the
  // samples b, b + stride, ...; the bag offsets of the next sample are loaded
  // with this sample's rows and its first indices during this sample's Gram
  // matrix, so only the row loads wait on memory.
  const TT* tb[NT];
  const float2* sbt[NT];
  bool bagrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int row = t * 16 + r16;
    bagrow[t] = row >= 1 && row < n;
    tb[t] = reinterpret_cast<const TT*>(src.tables[bagrow[t] ? row - 1 : 0]);
    sbt[t] = R::kScaled ? reinterpret_cast<const float2*>(src.scale_bias[bagrow[t] ? row - 1 : 0]) : nullptr;
  }
  auto load_offsets = [&](int64_t s, int64_t (&o0)[NT], int64_t (&o1)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (kPersist) {
        const int64_t bag = (bagrow[t] && s < B) ? (int64_t)(t * 16 + r16 - 1) * B + s : 0;
        o0[t] = off[bag];
        o1[t] = off[bag + 1];
      } else {  // this wave's sample, from the block's offsets in LDS
        const int k = bagrow[t] ? t * 16 + r16 - 1 : 0;
        o0[t] = so[k * per + wave];
        o1[t] = so[k * per + wave + 1];
      }
    }
  };
  int64_t pb[NT], r0[NT];
  int len[NT];
  auto take_meta = [&](int64_t s, const int64_t (&o0)[NT], const int64_t (&o1)[NT], int64_t (&p)[NT],
                       int (&l)[NT], int64_t (&r)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      p[t] = o0[t];
      l[t] = (bagrow[t] && s < B) ? (int)(o1[t] - o0[t]) : 0;
      r[t] = *(l[t] > 0 ? idx + p[t] : off);
    }
  };
  {
    int64_t o0[NT], o1[NT];
    load_offsets(b, o0, o1);
    take_meta(b, o0, o1, pb, len, r0);
  }
  for (;;) {
    const float* __restrict__ x0 = src.X + b * src.x_ld;
    // first row of every bag (0 + row, the sum's start) and the dense row
    f4 x[NT][DC];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row = t * 16 + r16;
      if constexpr (kF32) {
        const float* rp = pick(row != 0 && len[t] > 0, tb[t] + r0[t] * (int64_t)d, x0);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const int kk = c * 16 + 4 * g;
          x[t][c] = ld4(rp + (kk < d ? kk : d - 4));
        }
      } else {
        // table rows, eight columns per load (row 0 of the table for lanes
        // with no row: a valid address, masked below), and the dense row for
        // the lanes of row 0
        const int64_t rr = (row != 0 && len[t] > 0) ? r0[t] : 0;
        const TT* rp = tb[t] + rr * (int64_t)d;
        const float2 sz = R::kScaled ? sbt[t][rr] : make_float2(0.f, 0.f);
#pragma unroll
        for (int c = 0; c < DC; c += 2) {
          const int col = col_of<true>(c, g);
          R::load8(rp, col < d ? col : d - 8, sz, x[t][c], x[t][c + 1]);
        }
        if (t == 0) {
#pragma unroll
          for (int c = 0; c < DC; ++c) {
            const int col = col_of<true>(c, g);
            const f4 xd = ld4(x0 + (col < d ? col : d - 4));
            if (row == 0) x[0][c] = xd;
          }
        }
      }
    }
    const int64_t bn = kPersist ? b + stride : B;
    int64_t o0n[NT], o1n[NT];
    if constexpr (kPersist) load_offsets(bn, o0n, o1n);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row = t * 16 + r16;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bool live = col_of<!kF32>(c, g) < d;
        if (row == 0) {
          if (!live) x[t][c] = f4{0.f, 0.f, 0.f, 0.f};
        } else if (len[t] > 0 && live) {
          x[t][c] = f4{0.f + x[t][c][0], 0.f + x[t][c][1], 0.f + x[t][c][2], 0.f + x[t][c][3]};
        } else {
          x[t][c] = f4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    // remaining bag positions, in order; the index of position q+1 is loaded
    // while the rows of position q are in flight
    int maxlen = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) maxlen = len[t] > maxlen ? len[t] : maxlen;
    if (maxlen > 1) {
      int64_t rq[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) rq[t] = *(1 < len[t] ? idx + pb[t] + 1 : off);
      for (int q = 1; q < maxlen; ++q) {
        const float* rp[NT];
        const TT* rq_row[NT];
        float2 sz[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (kF32) {
            rp[t] = pick(q < len[t], tb[t] + rq[t] * (int64_t)d, x0);
          } else {
            const int64_t rr = q < len[t] ? rq[t] : 0;
            rq_row[t] = tb[t] + rr * (int64_t)d;
            sz[t] = R::kScaled ? sbt[t][rr] : make_float2(0.f, 0.f);
          }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) rq[t] = *(q + 1 < len[t] ? idx + pb[t] + q + 1 : off);
        // x is never -0 here (every sum starts from +0), so adding +0 for a
        // finished bag leaves it bit for bit unchanged
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (kF32) {
#pragma unroll
            for (int c = 0; c < DC; ++c) {
              const int kk = c * 16 + 4 * g;
              const f4 v = ld4(rp[t] + (kk < d ? kk : d - 4));
              x[t][c] = x[t][c] + ((q < len[t] && kk < d) ? v : f4{0.f, 0.f, 0.f, 0.f});
            }
          } else {
#pragma unroll
            for (int c = 0; c < DC; c += 2) {
              const int col = col_of<true>(c, g);
              f4 lo, hi;
              R::load8(rq_row[t], col < d ? col : d - 8, sz[t], lo, hi);
              const bool on = q < len[t] && col < d;
              x[t][c] = x[t][c] + (on ? lo : f4{0.f, 0.f, 0.f, 0.f});
              x[t][c + 1] = x[t][c + 1] + (on ? hi : f4{0.f, 0.f, 0.f, 0.f});
            }
          }
        }
      }
    }
    if constexpr (kPersist) take_meta(bn, o0n, o1n, pb, len, r0);  // next sample's first indices, in flight during the Gram matrix
    gram_row<NT, DC, OutT, !kF32>(x, n, d, pad_end, reinterpret_cast<OutT*>(rowb), lane);
    row_out(rowb, reinterpret_cast<char*>(out + b * out_ld), pad_end * (int)sizeof(OutT), wide, lane);
    if (bn >= B) break;
    b = bn;
  }
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

template <int MODE>
struct FRowOf { typedef FRowF32 type; };
template <>
struct FRowOf<2> { typedef FRowBF16 type; };
template <>
struct FRowOf<3> { typedef FRowI8 type; };

// MODE 0: materialised X; 1: fused from fp32 rows; 2: bf16 rows; 3: int8 rows
template <int NT, int DC, typename OutT, int MODE>
void launch_mfma(const RowSource& src, int64_t B, int n, int d, OutT* out, int64_t out_ld, int pad_end,
                 hipStream_t s) {
  // row buffer: pad_end elements
  const int row_bytes = (int)round_up((int64_t)pad_end * (int64_t)sizeof(OutT), 16);
  int spb = 65536 / row_bytes;  // samples (waves) per block within 64 KB of LDS
  spb = spb < 1 ? 1 : (spb > 4 ? 4 : spb);
  const int wide = ((out_ld * (int64_t)sizeof(OutT)) % 16) == 0;
  if constexpr (MODE > 0) {
    // persistent waves: as many blocks as stay resident, each wave walking
    // the samples with the grid's stride
    typedef typename FRowOf<MODE>::type R;
    // rows, then (one sample per wave) the block's bag offsets
    const size_t lds = (size_t)spb * row_bytes +
                       (fused_persistent<NT, DC>() ? 0 : (size_t)(n - 1) * (size_t)(spb + 1) * sizeof(int64_t));
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu,
                                                     reinterpret_cast<const void*>(fused_kernel<NT, DC, OutT, R>),
                                                     64 * spb, lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    int64_t grid = ceil_div(B, spb);
    if (fused_persistent<NT, DC>() && grid > (int64_t)per_cu * device_cu_count()) grid = (int64_t)per_cu * device_cu_count();
    hipLaunchKernelGGL((fused_kernel<NT, DC, OutT, R>), dim3((unsigned)grid), dim3(64 * spb), lds, s, src, B, n, d,
                       out, out_ld, pad_end, row_bytes, wide);
  } else
    hipLaunchKernelGGL((interact_mfma_kernel<NT, DC, OutT>), dim3((unsigned)ceil_div(B, spb)), dim3(64 * spb),
                       (size_t)spb * row_bytes, s, src, B, n, d, out, out_ld, pad_end, row_bytes, wide);
}

template <int DC, typename OutT, int MODE>
bool dispatch_nt(int NT, const RowSource& src, int64_t B, int n, int d, OutT* out, int64_t out_ld, int pad_end,
                 hipStream_t s) {
  // x[NT][DC] must fit in 128 registers per lane: NT * DC <= 32
  constexpr int kMaxNT = (32 / DC) < 8 ? (32 / DC) : 8;
  if (NT > kMaxNT) return false;
  switch (NT) {
    case 1: launch_mfma<1, DC, OutT, MODE>(src, B, n, d, out, out_ld, pad_end, s); return true;
    case 2: launch_mfma<2, DC, OutT, MODE>(src, B, n, d, out, out_ld, pad_end, s); return true;
    case 3: if constexpr (kMaxNT >= 3) { launch_mfma<3, DC, OutT, MODE>(src, B, n, d, out, out_ld, pad_end, s); return true; } break;
    case 4: if constexpr (kMaxNT >= 4) { launch_mfma<4, DC, OutT, MODE>(src, B, n, d, out, out_ld, pad_end, s); return true; } break;
    case 5: if constexpr (kMaxNT >= 5) { launch_mfma<5, DC, OutT, MODE>(src, B, n, d, out, out_ld, pad_end, s); return true; } break;
    case 6: if constexpr (kMaxNT >= 6) { launch_mfma<6, DC, OutT, MODE>(src, B, n, d, out, out_ld, pad_end, s); return true; } break;
    case 7: if constexpr (kMaxNT >= 7) { launch_mfma<7, DC, OutT, MODE>(src, B, n, d, out, out_ld, pad_end, s); return true; } break;
    case 8: if constexpr (kMaxNT >= 8) { launch_mfma<8, DC, OutT, MODE>(src, B, n, d, out, out_ld, pad_end, s); return true; } break;
  }
  return false;
}

// ------------------------------------------------------------------ backward
// One wave per sample.  The sample's X rows and pair gradients are staged in
// LDS (row stride d + 16 floats, so the four 16-lane groups of an MFMA
// operand read hit distinct banks); then dX = S X with S the symmetric
// n x n matrix of pair gradients (zero diagonal) runs on fp32 MFMA 16x16x4:
// A operand S[i][j] (lane: i = 16I + l%16, j = 4ks + l/16), B operand X[j][c]
// (lane: j = 4ks + l/16, c = 16ct + l%16), D rows 16I + 4(l/16) + r.
template <int CT>
__global__ __launch_bounds__(256) void interact_bwd_kernel(const float* __restrict__ X, int64_t B, int n, int d,
                                                           int64_t x_ld, const float* __restrict__ g, int64_t g_ld,
                                                           float* __restrict__ dX, int64_t dx_ld, int xs,
                                                           int wave_floats) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  if (b >= B) return;  // whole wave
  float* xsm = sm + (int64_t)wave * wave_floats;  // [n][xs]
  const int P = n * (n - 1) / 2;
  float* psm = xsm + n * xs;                      // [P]
  const float* __restrict__ xb = X + b * x_ld;
  const float* __restrict__ gb = g + b * g_ld;
  const int d4 = d >> 2;
  for (int e = lane; e < n * d4; e += 64) {
    const int row = e / d4, c4 = e - row * d4;
    *reinterpret_cast<float4*>(xsm + row * xs + 4 * c4) = *reinterpret_cast<const float4*>(xb + row * d + 4 * c4);
  }
  for (int e = lane; e < P; e += 64) psm[e] = gb[d + e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int r16 = lane & 15, q = lane >> 4;
  const int NT = (n + 15) >> 4, KS = (n + 3) >> 2;
  for (int I = 0; I < NT; ++I) {
    const int i = 16 * I + r16;
    f4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f4{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < KS; ++ks) {
      const int j = 4 * ks + q;
      // S[i][j]: zero on the diagonal and outside n (read from a clamped,
      // valid address and masked)
      const int hi = i > j ? i : j, lo = i > j ? j : i;
      const bool live = i < n && j < n && i != j;
      const int pidx = live ? hi * (hi - 1) / 2 + lo : 0;
      const float sv = psm[P > 0 ? pidx : 0];
      const float a = live ? sv : 0.f;
      const int jr = j < n ? j : n - 1;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const float xv = xsm[jr * xs + 16 * ct + r16];
        const float bv = j < n ? xv : 0.f;
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc[ct], 0, 0, 0);
      }
    }
    float* __restrict__ ob = dX + b * dx_ld;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = 16 * ct + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * I + 4 * q + r;
        if (row < n && c < d) ob[row * d + c] = acc[ct][r] + (row == 0 ? gb[c] : 0.f);
      }
    }
  }
}

constexpr int kBwdLdsMax = 160 * 1024;  // LDS of one workgroup on gfx950

inline int bwd_wave_floats(int n, int d) { return (int)round_up((int64_t)n * (d + 16) + (int64_t)n * (n - 1) / 2, 4); }

template <int CT>
int launch_bwd(const float* X, int64_t B, int n, int d, int64_t x_ld, const float* g, int64_t g_ld, float* dX,
               int64_t dx_ld, hipStream_t s) {
  const int xs = d + 16;
  const int wave_floats = bwd_wave_floats(n, d);
  int spb = (int)(65536 / ((int64_t)wave_floats * 4));  // waves per block within 64 KB of LDS
  spb = spb < 1 ? 1 : (spb > 4 ? 4 : spb);
  const size_t lds = (size_t)spb * wave_floats * 4;
  if (lds > 65536) {  // one large sample per block: allow the full LDS once
    static bool raised[kMaxDevices] = {false};
    const int dev = current_device();
    if (!raised[dev]) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(interact_bwd_kernel<CT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kBwdLdsMax) != hipSuccess)
        return DLRM_E_HIP;
      raised[dev] = true;
    }
  }
  hipLaunchKernelGGL((interact_bwd_kernel<CT>), dim3((unsigned)ceil_div(B, spb)), dim3(64 * spb), lds, s, X, B, n,
                     d, x_ld, g, g_ld, dX, dx_ld, xs, wave_floats);
  return DLRM_OK;
}

template <typename OutT, int MODE>
bool dispatch(const RowSource& src, int64_t B, int n, int d, OutT* out, int64_t out_ld, int pad_end, hipStream_t s) {
  const int NT = (n + 15) / 16;
  const int dc = (d + 15) / 16;
  if (dc <= 1) return dispatch_nt<1, OutT, MODE>(NT, src, B, n, d, out, out_ld, pad_end, s);
  if (dc <= 2) return dispatch_nt<2, OutT, MODE>(NT, src, B, n, d, out, out_ld, pad_end, s);
  if (dc <= 4) return dispatch_nt<4, OutT, MODE>(NT, src, B, n, d, out, out_ld, pad_end, s);
  if (dc <= 8) return dispatch_nt<8, OutT, MODE>(NT, src, B, n, d, out, out_ld, pad_end, s);
  if (dc <= 16) return dispatch_nt<16, OutT, MODE>(NT, src, B, n, d, out, out_ld, pad_end, s);
  return false;
}

template <typename OutT>
void run(const float* X, int64_t B, int n, int d, int64_t x_ld, OutT* out, int64_t out_ld, int pad_end,
         hipStream_t s) {
  const RowSource src{X, x_ld, nullptr, nullptr, nullptr, nullptr};
  if (!dispatch<OutT, 0>(src, B, n, d, out, out_ld, pad_end, s)) {
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

namespace dlrm {
namespace {
// Checks shared by the fused entry points; sets *pad_end.
int check_fused(const float* x_dense, int64_t xd_ld, const void* tables, int32_t K, int32_t d, const int64_t* indices,
                const int64_t* offsets, int64_t B, void* out, int32_t out_dtype, int64_t out_ld, int* pad_end) {
  if (!x_dense || !tables || !indices || !offsets || !out || K < 1 || B < 1) return DLRM_E_INVALID;
  const int n = K + 1;
  if (n > 128 || d < 4 || d > 256 || (d % 4) != 0) return DLRM_E_INVALID;
  if (out_dtype != DLRM_F32 && out_dtype != DLRM_BF16) return DLRM_E_INVALID;
  const int64_t width = d + (int64_t)n * (n - 1) / 2;
  if (xd_ld < d || (xd_ld % 4) != 0 || !aligned16(x_dense)) return DLRM_E_INVALID;
  if (out_ld < width || (out_ld % 4) != 0 || !aligned16(out)) return DLRM_E_INVALID;
  if (ceil_div(B, 4) > 0x7fffffffLL || B * out_ld > (int64_t)1 << 40) return DLRM_E_UNSUPPORTED;
  *pad_end = (int)(round_up(width, 8) < out_ld ? round_up(width, 8) : out_ld);
  return DLRM_OK;
}
}  // namespace
}  // namespace dlrm

extern "C" int dlrm_embbag_interact_fwd(const float* x_dense, int64_t xd_ld, const float* const* tables, int32_t K,
                                        int32_t d, const int64_t* indices, const int64_t* offsets, int64_t B,
                                        void* out, int32_t out_dtype, int64_t out_ld, hipStream_t stream) {
  int pad_end = 0;
  const int rc = check_fused(x_dense, xd_ld, tables, K, d, indices, offsets, B, out, out_dtype, out_ld, &pad_end);
  if (rc != DLRM_OK) return rc;
  const int n = K + 1;
  const RowSource src{x_dense, xd_ld, tables, indices, offsets, nullptr};
  bool ok;
  if (out_dtype == DLRM_F32)
    ok = dispatch<float, 1>(src, B, n, d, static_cast<float*>(out), out_ld, pad_end, stream);
  else
    ok = dispatch<uint16_t, 1>(src, B, n, d, static_cast<uint16_t*>(out), out_ld, pad_end, stream);
  if (!ok) return DLRM_E_UNSUPPORTED;  // (K + 1) x d does not fit the register-resident layout
  return launch_status();
}

extern "C" int dlrm_embbag_interact_fwd_lp(const float* x_dense, int64_t xd_ld, const void* const* tables,
                                           int32_t table_dtype, const float* const* scale_bias, int32_t K, int32_t d,
                                           const int64_t* indices, const int64_t* offsets, int64_t B, void* out,
                                           int32_t out_dtype, int64_t out_ld, hipStream_t stream) {
  int pad_end = 0;
  const int rc = check_fused(x_dense, xd_ld, tables, K, d, indices, offsets, B, out, out_dtype, out_ld, &pad_end);
  if (rc != DLRM_OK) return rc;
  if (table_dtype != DLRM_BF16 && table_dtype != DLRM_I8) return DLRM_E_INVALID;
  if (table_dtype == DLRM_I8 && !scale_bias) return DLRM_E_INVALID;
  if (out_dtype != DLRM_BF16) return DLRM_E_UNSUPPORTED;  // low-precision rows feed a bf16 top MLP
  if (d % 32 != 0) return DLRM_E_UNSUPPORTED;             // eight columns per lane load, 32-wide chunk pairs
  const int n = K + 1;
  const RowSource src{x_dense, xd_ld, reinterpret_cast<const float* const*>(tables), indices, offsets,
                      table_dtype == DLRM_I8 ? scale_bias : nullptr};
  uint16_t* o = static_cast<uint16_t*>(out);
  const bool ok = table_dtype == DLRM_BF16 ? dispatch<uint16_t, 2>(src, B, n, d, o, out_ld, pad_end, stream)
                                           : dispatch<uint16_t, 3>(src, B, n, d, o, out_ld, pad_end, stream);
  if (!ok) return DLRM_E_UNSUPPORTED;
  return launch_status();
}

extern "C" int dlrm_interact_bwd(const float* X, int64_t B, int32_t n, int32_t d, int64_t x_ld, const float* g,
                                 int64_t g_ld, float* dX, int64_t dx_ld, hipStream_t stream) {
  if (!X || !g || !dX) return DLRM_E_INVALID;
  if (B < 1 || n < 2 || n > 128 || d < 4 || d > 256 || (d % 4) != 0) return DLRM_E_INVALID;
  if (x_ld < (int64_t)n * d || (x_ld % 4) != 0 || !aligned16(X)) return DLRM_E_INVALID;
  if (g_ld < (int64_t)d + (int64_t)n * (n - 1) / 2 || dx_ld < (int64_t)n * d) return DLRM_E_INVALID;
  if ((int64_t)bwd_wave_floats(n, d) * 4 > kBwdLdsMax) return DLRM_E_UNSUPPORTED;
  const int ct = (d + 15) / 16;
  int rc;
  if (ct <= 1) rc = launch_bwd<1>(X, B, n, d, x_ld, g, g_ld, dX, dx_ld, stream);
  else if (ct <= 2) rc = launch_bwd<2>(X, B, n, d, x_ld, g, g_ld, dX, dx_ld, stream);
  else if (ct <= 4) rc = launch_bwd<4>(X, B, n, d, x_ld, g, g_ld, dX, dx_ld, stream);
  else if (ct <= 8) rc = launch_bwd<8>(X, B, n, d, x_ld, g, g_ld, dX, dx_ld, stream);
  else rc = launch_bwd<16>(X, B, n, d, x_ld, g, g_ld, dX, dx_ld, stream);
  return rc != DLRM_OK ? rc : launch_status();
}
