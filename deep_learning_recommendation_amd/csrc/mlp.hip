// Multilayer perceptrons of the model: the bottom MLP (dense features -> d)
// and the top MLP (interaction row -> logit -> sigmoid), "Deep Learning
// Recommendation Model (DLRM)" explainer, Key Method Details (Bottom MLP, Top
// MLP, Loss); briansu.co DLRM, Key equations (Output).
//
// Forward: one launch per layer.  bf16 networks keep hidden activations as
// bf16 rows padded to a multiple of 8 elements so every MFMA operand load is
// 16 bytes; the first layer of a narrow input (K <= 32, e.g. 13 dense
// features) uses a VALU kernel, N == 1 output layers a GEMV with the sigmoid
// fused, everything else the bf16 MFMA GEMM with bias + ReLU + convert fused
// in its epilogue.
//
// Backward (bf16 networks): per layer, dW = delta^T x as a split-K MFMA GEMM
// over the batch (partials summed in a fixed order) and delta W, whose
// epilogue applies the ReLU mask of the layer below, rounds to bf16 and
// writes that layer's delta in both layouts with its bias-gradient partials
// (a deterministic two-stage column sum); only the last layer's delta, from
// the caller's fp32 dY, takes a separate pass.  Transposed copies make every
// GEMM the K-contiguous form the MFMA kernel reads.
#include "gemm.hpp"

namespace dlrm {
namespace {

struct FwdLayout {
  size_t bytes = 0;
  size_t act_off[65];  // act_off[l]: layer l's input buffer (l = 0 .. L-1); ~0 if none
  int64_t act_ld[65];
  bool act_bf16 = true;
};

// Shared by forward and backward: where layer inputs live in the forward workspace.
bool fwd_layout(int64_t B, int32_t L, const int32_t* dims, int32_t w_dtype, int32_t save_acts, FwdLayout* lay) {
  if (L < 1 || L > 64 || B < 1) return false;
  for (int l = 0; l <= L; ++l)
    if (dims[l] < 1) return false;
  Carver cv(nullptr);
  const bool bf = (w_dtype == DLRM_BF16);
  lay->act_bf16 = bf;
  const size_t esz = bf ? 2 : 4;
  for (int l = 0; l <= L; ++l) {
    lay->act_off[l] = ~(size_t)0;
    lay->act_ld[l] = bf ? round_up(dims[l], 8) : dims[l];
  }
  // layer 0's input: a bf16 copy of the caller's input (always for bf16 nets:
  // fp32 inputs are rounded once here; kept for the backward pass)
  if (bf) {
    cv.take<char>(esz * (size_t)(B * lay->act_ld[0]));
    lay->act_off[0] = 0;
  }
  if (save_acts) {
    for (int l = 1; l < L; ++l) {
      cv.used = (size_t)round_up((int64_t)cv.used, 256);
      lay->act_off[l] = cv.used;
      cv.used += esz * (size_t)(B * lay->act_ld[l]);
    }
  } else {
    int64_t wmax = 0;
    for (int l = 1; l < L; ++l) wmax = lay->act_ld[l] > wmax ? lay->act_ld[l] : wmax;
    size_t ping = 0, pong = 0;
    if (L > 1) {
      cv.used = (size_t)round_up((int64_t)cv.used, 256);
      ping = cv.used;
      cv.used += esz * (size_t)(B * wmax);
      cv.used = (size_t)round_up((int64_t)cv.used, 256);
      pong = cv.used;
      cv.used += esz * (size_t)(B * wmax);
    }
    for (int l = 1; l < L; ++l) lay->act_off[l] = (l & 1) ? ping : pong;
  }
  lay->bytes = cv.bytes();
  return true;
}

__global__ __launch_bounds__(256) void copy_bf16_kernel(const uint16_t* __restrict__ in, int64_t ldi,
                                                        uint16_t* __restrict__ out, int64_t ldo, int R, int C,
                                                        int Cpad) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)R * Cpad) return;
  const int r = (int)(t / Cpad), c = (int)(t - (int64_t)r * Cpad);
  out[(int64_t)r * ldo + c] = c < C ? in[(int64_t)r * ldi + c] : (uint16_t)0;
}

// ------------------------------------------------------------------ fused bottom MLP
//
// A three-layer bf16 network K0 (<= 16) -> 512 -> 256 -> 128 with ReLU after
// the hidden layers (the bottom-MLP shape 13-512-256-128) in one kernel.  A
// workgroup of eight waves (two per SIMD) owns 128 rows: waves w and w + 4
// share rows 32 w .. 32 w + 31 and split the columns of layers 2 and 3 in
// halves, so each SIMD runs two independent MFMA chains.  Every activation
// of a wave's rows stays in registers: with the W fragment as the first
// MFMA operand, a lane holds one row and groups of four consecutive output
// columns, and after bias, ReLU, bf16 rounding and one cross-half lane swap
// (v_permlane32_swap) each lane holds eight consecutive columns -- exactly
// the operand layout of the next layer's MFMA (row l % 32, k = 8 * (l / 32)
// .. +7 of each 16-wide k-step).  The rounding points are those of the
// layer-by-layer path (input, hidden activations in bf16; fp32
// accumulation; fp32 output).
//
// Layer 1 (K0 -> 512, one k-step) is computed by both waves of a pair, two
// output blocks (64 columns) at a time, just before the layer-2 k-steps that
// take them as operands (its weights sit in LDS as MFMA fragments, 16 KB,
// columns at or past K0 zeroed).  The weights of layers 2 and 3 stream through a
// ring of four 32 KB LDS stages, loaded straight from global memory
// (global_load_lds_dwordx4, coalesced rows): ten chunks, eight of W2 (64 k x
// 256 rows) and two of W3 (128 k x 128 rows), three in flight ahead of the
// one being used.  The two halves of layer 2's output meet in the two
// stages layer 2 leaves free (16 KB per 32 rows), so that each wave has all
// 256 k of layer 3.  The output rows are written in fp32; for training the
// bf16 input and hidden activations the backward pass reads are written as
// well.
constexpr int kF3Rows = 128, kF3D1 = 512, kF3D2 = 256, kF3D3 = 128, kF3K0 = 16;
constexpr int kF3Waves = 8;
constexpr int kF3Stage = 32768, kF3Ring = 4 * kF3Stage;
constexpr int kF3W1Lds = kF3Ring + 4096;        // W1 fragments (16 KB) after the bias vectors
constexpr int kF3Lds = kF3W1Lds + kF3D1 * 32;  // the ring, the three bias vectors (2 KB, 1 KB, 512 B), W1
constexpr int kF3Chunks = 10;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// row pieces (16 bytes) of chunk c: W2 rows hold 64 k (8 pieces), W3 rows
// 128 k (16); a row's pieces are XOR-swizzled so that the 16 lanes one LDS
// cycle serves (16 consecutive rows, one logical piece) hit distinct banks
__device__ __forceinline__ int f3_cpr(int c) { return c < 8 ? 8 : 16; }
__device__ __forceinline__ int f3_swz(int row, int cpr) { return cpr == 8 ? ((row >> 1) & 7) : (row & 15); }

// bf16 rounding, optional ReLU and the cross-half swap of one 32 x 32
// accumulator block: lo = columns 8*(l/32) .. +7, hi = columns 16 + 8*(l/32)
// .. +7.  The ReLU acts on the rounded pair (a sign test: negative values
// and -0 become +0), which equals rounding the ReLU output for every
// non-NaN value.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t p) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, p), s16x2{0, 0}));
}
__device__ __forceinline__ void f3_pack(const f32x16_t& a, bool relu, uint4& lo, uint4& hi) {
  uint32_t pk[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t p = pack_bf16x2(a[4 * g + 2 * h], a[4 * g + 2 * h + 1]);
      pk[g][h] = relu ? relu_bf16x2(p) : p;
    }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto s01 = __builtin_amdgcn_permlane32_swap(pk[0][h], pk[1][h], false, false);
    const auto s23 = __builtin_amdgcn_permlane32_swap(pk[2][h], pk[3][h], false, false);
    pk[0][h] = s01[0];
    pk[1][h] = s01[1];
    pk[2][h] = s23[0];
    pk[3][h] = s23[1];
  }
  lo = make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]);
  hi = make_uint4(pk[2][0], pk[2][1], pk[3][0], pk[3][1]);
}

// accumulators of one 32 x 32 block start from the bias (in LDS): register
// v is column col0 + 8*(v/4) + 4*(l/32) + v%4
__device__ __forceinline__ void f3_bias(f32x16_t& acc, const char* b, int col0, int half) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float4 v = *reinterpret_cast<const float4*>(b + (col0 + 8 * g + 4 * half) * 4);
    acc[4 * g] = v.x;
    acc[4 * g + 1] = v.y;
    acc[4 * g + 2] = v.z;
    acc[4 * g + 3] = v.w;
  }
}

__global__ __launch_bounds__(64 * kF3Waves) __attribute__((amdgpu_waves_per_eu(2, 2))) void mlp3_fused_kernel(
    const float* __restrict__ in, int64_t in_ld, int K0, int M, const uint16_t* __restrict__ W1, int64_t w1_ld,
    const float* __restrict__ b1, const uint16_t* __restrict__ W2, int64_t w2_ld, const float* __restrict__ b2,
    const uint16_t* __restrict__ W3, int64_t w3_ld, const float* __restrict__ b3, int relu3, float* __restrict__ out,
    int64_t out_ld, int vec_out, uint16_t* __restrict__ act0, int64_t ld0, uint16_t* __restrict__ act1,
    uint16_t* __restrict__ act2) {
  extern __shared__ __attribute__((aligned(1024))) char f3_smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = wave & 3, ch = wave >> 2;  // row group, column half
  const int r32 = lane & 31, half = lane >> 5;
  const int row = blockIdx.x * kF3Rows + rg * 32 + r32;  // this lane's row (all layers)
  const bool row_ok = row < M;

  // chunk c of the weight ring into stage c % 4: 32 instructions of 1 KB,
  // four per wave; instruction j of wave w fills rows (4w + j) * (64 / cpr) ..
  auto issue = [&](int c) {
    char* st = f3_smem + (c & 3) * kF3Stage;
    const int cpr = f3_cpr(c), rpi = 64 / cpr;
    const uint16_t* base = c < 8 ? W2 : W3;
    const int64_t ld = c < 8 ? w2_ld : w3_ld;
    const int k0 = c < 8 ? c * 64 : (c - 8) * 128;
    const int lrow = lane / cpr, lpc = lane % cpr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = (wave * 4 + j) * rpi + lrow;
      lds_dma16_opaque(base + (int64_t)n * ld + k0 + (lpc ^ f3_swz(n, cpr)) * 8, st + (wave * 4 + j) * 1024);
    }
  };
  // the B fragments of k-step ks of chunk c for output blocks tn0 .. tn0+TN-1
  auto read_b = [&](int c, int ks, bf16x8_t* fb, int tn0, int TN) {
    const char* st = f3_smem + (c & 3) * kF3Stage;
    const int cpr = f3_cpr(c);
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int tn = tn0 + t;
      const int n = tn * 32 + r32;
      fb[t] = *reinterpret_cast<const bf16x8_t*>(st + n * cpr * 16 + (((2 * ks + half) ^ f3_swz(n, cpr)) * 16));
    }
  };
  // wait until at most `younger` chunks issued after the awaited one are
  // still in flight (four instructions per chunk per wave)
  auto wait_younger = [&](int younger) {
    if (younger >= 4) wait_vmcnt<16>();
    else if (younger == 3) wait_vmcnt<12>();
    else if (younger == 2) wait_vmcnt<8>();
    else if (younger == 1) wait_vmcnt<4>();
    else wait_vmcnt<0>();
  };

  // bias vectors into LDS first (one 1 KB instruction for each of waves 0-3;
  // lanes past the end of b3 re-read its start into the padding)
  if (wave < 4) {
    char* ba = f3_smem + kF3Ring;
    const int off = wave * 1024 + lane * 16;
    const float* src = off < 2048 ? b1 + off / 4 : off < 3072 ? b2 + (off - 2048) / 4 : off < 3584 ? b3 + (off - 3072) / 4 : b3;
    lds_dma16_opaque(src, ba + wave * 1024);
  }
  // ---- layer 1's operands: this lane's input row (k = 8*(l/32) .. +7, bf16,
  // in registers) and the W1 fragments of the 16 output blocks in LDS
  // (fragment (b, h, r): row 32 b + r, k = 8 h .. 8 h + 7; columns at or past
  // K0 zeroed).  Branch-free, so that every load is in flight at once:
  // out-of-range positions re-read an in-range one and are masked afterwards.
  float x[8];
  {
    const float* src = in + (int64_t)(row_ok ? row : M - 1) * in_ld;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int k = half * 8 + q;
      x[q] = src[k < K0 ? k : K0 - 1];
    }
  }
  uint4 w1p[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = threadIdx.x + i * 64 * kF3Waves;  // fragment: row p / 2, k-half p % 2
    const int kh = p & 1;
    w1p[i] = *reinterpret_cast<const uint4*>(W1 + (int64_t)(p >> 1) * w1_ld + (kh * 8 < K0 ? kh * 8 : 0));
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any is used
  uint32_t win[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = half * 8 + 2 * q;
    const uint32_t lo = k < K0 ? (uint32_t)f32_to_bf16(x[2 * q]) : 0u;
    const uint32_t hi = k + 1 < K0 ? (uint32_t)f32_to_bf16(x[2 * q + 1]) : 0u;
    win[q] = lo | (hi << 16);
  }
  uint4* w1s = reinterpret_cast<uint4*>(f3_smem + kF3W1Lds);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = threadIdx.x + i * 64 * kF3Waves;
    const int n = p >> 1, kh = p & 1;
    uint32_t v[4] = {w1p[i].x, w1p[i].y, w1p[i].z, w1p[i].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = kh * 8 + 2 * q;
      v[q] = k >= K0 ? 0u : (k + 1 >= K0 ? (v[q] & 0xffffu) : v[q]);
    }
    w1s[((n >> 5) * 2 + kh) * 32 + (n & 31)] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  // the plain loads and the bias vectors have landed before any chunk is
  // issued, so no later wait of the compiler's covers a chunk; the W1
  // fragments are in LDS for every wave after the barrier
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  issue(0);
  issue(1);
  issue(2);
  issue(3);
  const char* bias1 = f3_smem + kF3Ring;
  const char* bias2 = bias1 + 2048;
  const char* bias3 = bias1 + 3072;
  const uint4 ua = make_uint4(win[0], win[1], win[2], win[3]);
  if (ch == 0 && act0 != nullptr && row_ok && half * 8 < ld0)
    *reinterpret_cast<uint4*>(act0 + (int64_t)row * ld0 + half * 8) = ua;
  const bf16x8_t a1 = as_bf16x8(ua);

  // ---- layers 1 and 2: chunk c (k-steps 4c .. 4c+3 of layer 2) takes layer
  // 1's output blocks 2c and 2c+1; this wave's four output blocks of layer 2
  // are 4 ch .. 4 ch + 3
  uint4 h1[4];
  auto layer1 = [&](int c) {
    f32x16_t acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f3_bias(acc[j], bias1, (2 * c + j) * 32, half);
      const uint4 w = w1s[((2 * c + j) * 2 + half) * 32 + r32];
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), a1, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) f3_pack(acc[j], true, h1[2 * j], h1[2 * j + 1]);
    if (ch == 0 && act1 != nullptr && row_ok) {
      uint16_t* g = act1 + (int64_t)row * kF3D1 + 8 * half;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        *reinterpret_cast<uint4*>(g + (2 * c + j) * 32) = h1[2 * j];
        *reinterpret_cast<uint4*>(g + (2 * c + j) * 32 + 16) = h1[2 * j + 1];
      }
    }
  };
  f32x16_t acc2[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) f3_bias(acc2[t], bias2, (4 * ch + t) * 32, half);
  bf16x8_t fb[2][4];
  wait_younger(3);  // chunk 0
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  read_b(0, 0, fb[0], 4 * ch, 4);
  layer1(0);
  int buf = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) {
        read_b(c, ks + 1, fb[buf ^ 1], 4 * ch, 4);
      } else {
        // hand-over to chunk c+1: after the barrier every wave's reads of
        // chunk c are done, so chunk c+4 can load into its stage.  Layer 3
        // starts with both of its chunks resident.
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        wait_younger(c < 7 ? (7 - c < 2 ? 7 - c : 2) : 0);
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (c + 4 < kF3Chunks) issue(c + 4);
        if (c < 7) read_b(c + 1, 0, fb[buf ^ 1], 4 * ch, 4);
        else read_b(8, 0, fb[buf ^ 1], 2 * ch, 2);
      }
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8_t a = as_bf16x8(h1[ks]);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc2[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][t], a, acc2[t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      buf ^= 1;
    }
    if (c < 7) layer1(c + 1);
  }
  // layer 2's activations become layer 3's operands: this wave's k-steps
  // 8 ch .. 8 ch + 7, the partner's through LDS stages 2 and 3 (free: the
  // last hand-over barrier came after every read of chunks 6 and 7)
  uint4 mine[8], other[8];  // k-steps 8 ch .. 8 ch + 7, and the partner's
#pragma unroll
  for (int t = 0; t < 4; ++t) f3_pack(acc2[t], true, mine[2 * t], mine[2 * t + 1]);
  {
    uint4* xch = reinterpret_cast<uint4*>(f3_smem + 2 * kF3Stage) + rg * 16 * 64;
#pragma unroll
    for (int q = 0; q < 8; ++q) xch[(8 * ch + q) * 64 + lane] = mine[q];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    compiler_fence();
#pragma unroll
    for (int q = 0; q < 8; ++q) other[q] = xch[(8 * (1 - ch) + q) * 64 + lane];
  }
  if (act2 != nullptr && row_ok) {
    uint16_t* g = act2 + (int64_t)row * kF3D2 + 8 * half;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      *reinterpret_cast<uint4*>(g + (4 * ch + t) * 32) = mine[2 * t];
      *reinterpret_cast<uint4*>(g + (4 * ch + t) * 32 + 16) = mine[2 * t + 1];
    }
  }

  // ---- layer 3: 256 -> 128, this wave's 64 columns (output blocks 2 ch and
  // 2 ch + 1; chunks 8 and 9 hold k 0-127 and 128-255)
  f32x16_t acc3[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) f3_bias(acc3[j], bias3, (2 * ch + j) * 32, half);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    if (ks < 15) read_b(8 + ((ks + 1) >> 3), (ks + 1) & 7, fb[buf ^ 1], 2 * ch, 2);
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8_t a = as_bf16x8((ks < 8) == (ch == 0) ? mine[ks & 7] : other[ks & 7]);
#pragma unroll
    for (int j = 0; j < 2; ++j) acc3[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], a, acc3[j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    buf ^= 1;
  }
  if (row_ok) {
    float* o = out + (int64_t)row * out_ld + 4 * half;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = acc3[j][4 * g + q];
          if (relu3) v[q] = v[q] > 0.f ? v[q] : 0.f;
        }
        float* d = o + (2 * ch + j) * 32 + 8 * g;
        if (vec_out) {
          *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) d[q] = v[q];
        }
      }
  }
}

template <typename YT>
__device__ __forceinline__ bool positive(const YT* p);
template <>
__device__ __forceinline__ bool positive<float>(const float* p) {
  return *p > 0.f;
}
template <>
__device__ __forceinline__ bool positive<uint16_t>(const uint16_t* p) {
  return bf16_to_f32(*p) > 0.f;
}

// One pass over the upstream gradient of a layer: delta = g * 1[y > 0] (or
// g) rounded to bf16 and stored row-major [B][ldd] (the operand of both the
// input-gradient and the weight-gradient GEMMs), plus fp32 column sums of
// delta per 32-row chunk (for the bias gradient).
// Block: 32 rows x 256 columns; wave w takes rows w, w+4, ..., lane l the
// four consecutive columns 4l .. 4l+3 (16-byte loads of g, 8- or 16-byte
// loads of y, 8-byte stores of delta when `vec`), eight rows' loads in flight
// before the first is used.  The column sums add the rows in the same order
// as a one-row-at-a-time walk.
constexpr int kDRows = 32, kDCols = 256, kDBatch = 8;
template <typename YT>
struct YLoad;
template <>
struct YLoad<float> {
  typedef float4 V;
  __device__ static V load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static bool pos(const V& v, int e) { return (e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w) > 0.f; }
};
template <>
struct YLoad<uint16_t> {
  typedef uint2 V;
  __device__ static V load(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ static bool pos(const V& v, int e) {
    const uint32_t w = (e < 2) ? v.x : v.y;
    return bf16_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu))) > 0.f;
  }
};
template <typename YT>
__global__ __launch_bounds__(256) void delta_db_kernel(const float* __restrict__ g, int64_t ldg,
                                                       const YT* __restrict__ y, int64_t ldy, int relu,
                                                       uint16_t* __restrict__ dlt, int64_t ldd,
                                                       float* __restrict__ part, int B, int N, int vec) {
  __shared__ float red[4][kDCols];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * kDCols, r0 = blockIdx.y * kDRows;
  const int cl = 4 * lane, c = c0 + cl;
  const bool full = vec && c + 4 <= N;  // this lane's four columns by vector accesses
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = wave; i0 < kDRows; i0 += 4 * kDBatch) {
    float4 gv[kDBatch];
    typename YLoad<YT>::V yv[kDBatch];
#pragma unroll
    for (int t = 0; t < kDBatch; ++t) {
      const int r = r0 + i0 + 4 * t;
      if (full && r < B) {
        gv[t] = *reinterpret_cast<const float4*>(g + (int64_t)r * ldg + c);
        if (relu) yv[t] = YLoad<YT>::load(y + (int64_t)r * ldy + c);
      }
    }
#pragma unroll
    for (int t = 0; t < kDBatch; ++t) {
      const int i = i0 + 4 * t, r = r0 + i;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (full) {
          v[e] = (r < B) ? (e == 0 ? gv[t].x : e == 1 ? gv[t].y : e == 2 ? gv[t].z : gv[t].w) : 0.f;
          if (relu && r < B && !YLoad<YT>::pos(yv[t], e)) v[e] = 0.f;
        } else {
          v[e] = 0.f;
          if (r < B && c + e < N) {
            v[e] = g[(int64_t)r * ldg + c + e];
            if (relu && !positive<YT>(y + (int64_t)r * ldy + c + e)) v[e] = 0.f;
          }
        }
      }
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = f32_to_bf16(v[e]);
        sum[e] = sum[e] + v[e];
      }
      if (r < B) {
        uint16_t* o = dlt + (int64_t)r * ldd + c;
        if (full) {
          *reinterpret_cast<uint2*>(o) =
              make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < N) o[e] = h[e];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) red[wave][cl + e] = sum[e];
  __syncthreads();
  {
    const int cc = threadIdx.x, col = c0 + cc;
    if (col < N) part[(int64_t)blockIdx.y * N + col] = ((red[0][cc] + red[1][cc]) + red[2][cc]) + red[3][cc];
  }
}

// The same pass for a layer of one output (the logit layer): a lane per
// row, so the rows' loads go out together; a wave per kDRows-row chunk,
// whose sum is a fixed tree over its lanes.
__global__ __launch_bounds__(256) void delta1_kernel(const float* __restrict__ g, int64_t ldg,
                                                     const float* __restrict__ y, int64_t ldy, int relu,
                                                     uint16_t* __restrict__ dlt, int64_t ldd,
                                                     float* __restrict__ part, int B) {
  static_assert(kDRows <= 64, "a chunk per wave");
  const int lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int r = chunk * kDRows + lane;
  const bool live = lane < kDRows && r < B;
  float v = 0.f;
  if (live) {
    v = g[(int64_t)r * ldg];
    if (relu && !(y[(int64_t)r * ldy] > 0.f)) v = 0.f;
    dlt[(int64_t)r * ldd] = f32_to_bf16(v);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = v + __shfl_xor(v, o);
  if (lane == 0 && chunk * kDRows < B) part[chunk] = v;
}

// One launch finishes the gradients of up to kFinLayers layers, after the
// whole backward pass (each layer keeps its own partials): per layer, blocks
// [0, rblocks) add the split-K partials of dW in split order (eight loads
// in flight); each other block sums the per-chunk partials of 64 entries of
// db, wave w taking chunks w, w + 4, ... in order and the four wave sums
// added in wave order.
constexpr int kFinLayers = 16;
struct FinLayer {
  const float* part;
  float* dW;
  const float* dbp;
  float* db;
  int64_t ldw;
  int splits, M, N, rblocks, chunks, block0;
};
struct FinArgs {
  FinLayer l[kFinLayers];
  int count;
};
__global__ __launch_bounds__(256) void grad_finalize_kernel(FinArgs args) {
  int li = 0;
  while (li + 1 < args.count && (int)blockIdx.x >= args.l[li + 1].block0) ++li;
  const FinLayer& f = args.l[li];
  const int blk = (int)blockIdx.x - f.block0;
  const int M = f.M, N = f.N;
  if (blk < f.rblocks) {
    const int64_t t = (int64_t)blk * blockDim.x + threadIdx.x;
    const int64_t MN = (int64_t)M * N;
    if (t >= MN) return;
    const int i = (int)(t / N), j = (int)(t - (int64_t)i * N);
    float v = 0.f;
    for (int z0 = 0; z0 < f.splits; z0 += 8) {
      float p[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) p[q] = (z0 + q < f.splits) ? f.part[(z0 + q) * MN + t] : 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (z0 + q < f.splits) v = v + p[q];
    }
    f.dW[(int64_t)i * f.ldw + j] = v;
    return;
  }
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int o = (blk - f.rblocks) * 64 + lane;
  float s = 0.f;
  if (o < M)
    for (int c0 = wave; c0 < f.chunks; c0 += 32) {
      float v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = (c0 + 4 * t < f.chunks) ? f.dbp[(int64_t)(c0 + 4 * t) * M + o] : 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (c0 + 4 * t < f.chunks) s = s + v[t];
    }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && o < M) f.db[o] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}


// Layers with a single output (the top MLP's logit layer) as two plain
// kernels instead of degenerate GEMMs.  A block covers kR1Rows rows and 256
// columns: thread t takes eight consecutive columns (16-byte loads; a row
// pitch that is a multiple of 8 keeps the last chunk inside the row) and the
// rows t / 32, t / 32 + 8, ... of the chunk, all its loads in flight at
// once; the eight row groups' sums are then added in group order.
constexpr int kR1Rows = 128, kR1Per = kR1Rows / 8;

__device__ __forceinline__ void unpack8(const uint4 q, float (&f)[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = bf16_to_f32((uint16_t)(w[e >> 1] >> (16 * (e & 1))));
}

// Adds the eight row groups' column sums of this block in group order; the
// threads of group 0 return the totals.
__device__ __forceinline__ void r1_group_sum(float (&acc)[8], float (*red)[256]) {
  const int t = threadIdx.x, rg = t >> 5, cg = t & 31;
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][cg * 8 + e] = acc[e];
  __syncthreads();
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = red[0][cg * 8 + e];
#pragma unroll
      for (int g = 1; g < 8; ++g) v = v + red[g][cg * 8 + e];
      acc[e] = v;
    }
  }
}

// A single-output layer's backward in one pass over its input rows x (the
// saved activations of the ReLU layer below, which are also the mask):
//   weight gradient: part[z][i] = the fp32 sum over the rows of chunk z of
//     delta[b] x[b][i] (each product of two bf16 values is exact), added up
//     across chunks like split-K partials;
//   with do_delta, the delta of the layer below as the GEMM epilogue forms
//     it: bf16(+0 + delta[b] w[i]) where x[b][i] > 0, else +0 (columns past
//     fi written as 0), and per chunk the fp32 column sums of the rounded
//     values.
__global__ __launch_bounds__(256) void rank1_kernel(const uint16_t* __restrict__ dlt, int64_t ldd,
                                                    const uint16_t* __restrict__ x, int64_t ldx, int B, int fi,
                                                    float* __restrict__ part, int do_delta,
                                                    const uint16_t* __restrict__ w, uint16_t* __restrict__ out,
                                                    int64_t ldo, float* __restrict__ dbp) {
  __shared__ float red[8][256];
  const int t = threadIdx.x, rg = t >> 5, z = blockIdx.y;
  const int c = blockIdx.x * 256 + (t & 31) * 8;
  const bool live = c < fi;
  const int cl = live ? c : 0;  // lanes past the row read its first chunk (results dropped)
  uint4 q[kR1Per];
  float dv[kR1Per];
#pragma unroll
  for (int r = 0; r < kR1Per; ++r) {
    const int b = z * kR1Rows + rg + 8 * r, bb = b < B ? b : B - 1;
    q[r] = *reinterpret_cast<const uint4*>(x + (int64_t)bb * ldx + cl);
    dv[r] = bf16_to_f32(dlt[(int64_t)bb * ldd]);
  }
  float wv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) wv[e] = (do_delta && c + e < fi) ? bf16_to_f32(w[c + e]) : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float accd[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < kR1Per; ++r) {
    const int b = z * kR1Rows + rg + 8 * r;
    float f[8];
    unpack8(q[r], f);
    const float d = b < B ? dv[r] : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + d * f[e];
    if (do_delta) {
      uint32_t h[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t v = (c + e < fi && f[e] > 0.f) ? f32_to_bf16(0.f + dv[r] * wv[e]) : (uint16_t)0;
        h[e >> 1] |= (uint32_t)v << (16 * (e & 1));
        if (b < B) accd[e] = accd[e] + bf16_to_f32(v);
      }
      if (b < B && live) *reinterpret_cast<uint4*>(out + (int64_t)b * ldo + c) = make_uint4(h[0], h[1], h[2], h[3]);
    }
  }
  r1_group_sum(acc, red);
  if (rg == 0)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c + e < fi) part[(int64_t)z * fi + c + e] = acc[e];
  if (!do_delta) return;
  __syncthreads();  // group 0 has read red
  r1_group_sum(accd, red);
  if (rg == 0)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c + e < fi) dbp[(int64_t)z * fi + c + e] = accd[e];
}

// Batch slices of a layer's weight-gradient GEMM: about 256 tiles of 128 x
// 128 in all (fewer slices were as fast and write fewer partials; measured
// with slices for 256 tiles 0.290 ms per dense backward, 512 0.297, 1024
// 0.309), each slice at least 128 rows of the batch.  Single-output layers
// take one slice per kR1Rows rows.
constexpr int kMaxSplits = 64;
int wgrad_splits(int64_t B, int fo, int fi) {
  if (fo == 1) return (int)ceil_div(B, kR1Rows);
  const int64_t tiles = ceil_div(fo, 128) * ceil_div(fi, 128);
  int64_t s = ceil_div(256, tiles);
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > ceil_div(B, 128)) s = ceil_div(B, 128);
  return s < 1 ? 1 : (int)s;
}

__global__ __launch_bounds__(256) void bce_grad_kernel(const float* __restrict__ logit, int64_t ld,
                                                       const float* __restrict__ y, int64_t B, float* __restrict__ dY) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const float s = 1.f / (1.f + expf(-logit[b * ld]));
  dY[b] = (s - y[b]) / (float)B;
}

struct BwdLayout {
  size_t dlt[2], wT, part[64], dbp[64], bytes;
  int64_t ld_dlt;
};

bool bwd_layout(int64_t B, int32_t L, const int32_t* dims, BwdLayout* lay) {
  if (L < 1 || L > 64 || B < 1) return false;
  int64_t wmax = 0, wfo = 0;
  for (int l = 0; l <= L; ++l) {
    if (dims[l] < 1) return false;
    wmax = dims[l] > wmax ? dims[l] : wmax;
  }
  for (int l = 0; l < L; ++l) wfo = dims[l + 1] > wfo ? dims[l + 1] : wfo;
  Carver cv(nullptr);
  lay->ld_dlt = round_up(wfo, 8);
  auto take = [&](size_t bytes) {
    cv.used = (size_t)round_up((int64_t)cv.used, 256);
    const size_t at = cv.used;
    cv.used += bytes;
    return at;
  };
  for (int i = 0; i < 2; ++i) lay->dlt[i] = take(2 * (size_t)(B * lay->ld_dlt));
  lay->wT = take(2 * (size_t)(wmax * lay->ld_dlt));
  // every layer keeps its weight-gradient partials and its bias-gradient
  // chunk partials (at most one chunk per kDRows rows) until the one
  // finishing launch at the end
  static_assert(kDRows <= kR1Rows && kDRows <= 128, "chunks of at least kDRows rows");
  for (int l = 0; l < L; ++l) {
    lay->part[l] = take(4 * (size_t)wgrad_splits(B, dims[l + 1], dims[l]) * dims[l] * dims[l + 1]);
    lay->dbp[l] = take(4 * (size_t)(ceil_div(B, kDRows) * dims[l + 1]));
  }
  lay->bytes = cv.bytes();
  return true;
}

}  // namespace
}  // namespace dlrm

using namespace dlrm;

extern "C" size_t dlrm_mlp_workspace_size(int64_t B, int32_t L, const int32_t* dims, int32_t w_dtype,
                                          int32_t save_acts) {
  if (!dims) return 0;
  FwdLayout lay;
  if (!fwd_layout(B, L, dims, w_dtype, save_acts, &lay)) return 0;
  return lay.bytes ? lay.bytes : 256;
}

extern "C" int dlrm_mlp_fwd(const void* in, int32_t in_dtype, int64_t in_ld, int64_t B, int32_t L,
                            const int32_t* dims, const void* const* W, const int32_t* w_ld, const float* const* bias,
                            int32_t w_dtype, int32_t last_act, float* out, int64_t out_ld, float* prob, void* ws,
                            size_t ws_bytes, int32_t save_acts, hipStream_t stream) {
  if (!in || !dims || !W || !bias || !out) return DLRM_E_INVALID;
  if (w_dtype != DLRM_F32 && w_dtype != DLRM_BF16) return DLRM_E_INVALID;
  if (in_dtype != DLRM_F32 && in_dtype != DLRM_BF16) return DLRM_E_INVALID;
  if (w_dtype == DLRM_F32 && in_dtype != DLRM_F32) return DLRM_E_INVALID;
  if (last_act != DLRM_ACT_NONE && last_act != DLRM_ACT_RELU) return DLRM_E_INVALID;
  if (B < 1 || B > 0x7fffffffLL) return DLRM_E_INVALID;
  FwdLayout lay;
  if (!fwd_layout(B, L, dims, w_dtype, save_acts, &lay)) return DLRM_E_INVALID;
  if (in_ld < dims[0] || out_ld < dims[L]) return DLRM_E_INVALID;
  for (int l = 0; l < L; ++l) {
    if (!W[l] || !bias[l]) return DLRM_E_INVALID;
    if (w_ld && w_ld[l] < dims[l]) return DLRM_E_INVALID;
  }
  if (prob && dims[L] != 1) return DLRM_E_INVALID;
  if (lay.bytes > 0 && (!ws || ws_bytes < lay.bytes)) return DLRM_E_WORKSPACE;
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 255u)) return DLRM_E_INVALID;
  char* wsb = static_cast<char*>(ws);
  const int M = (int)B;
  int rc = DLRM_OK;

  if (w_dtype == DLRM_F32) {
    const float* src = static_cast<const float*>(in);
    int64_t ld_src = in_ld;
    for (int l = 0; l < L && rc == DLRM_OK; ++l) {
      const int fi = dims[l], fo = dims[l + 1];
      const bool last = (l == L - 1);
      const bool relu = !last || last_act == DLRM_ACT_RELU;
      float* dst = last ? out : reinterpret_cast<float*>(wsb + lay.act_off[l + 1]);
      const int64_t ld_dst = last ? out_ld : lay.act_ld[l + 1];
      const int64_t wl = w_ld ? w_ld[l] : fi;
      rc = gemm_f32(src, ld_src, static_cast<const float*>(W[l]), wl, bias[l], dst, ld_dst, last ? prob : nullptr, M,
                    fo, fi, relu, stream);
      src = dst;
      ld_src = ld_dst;
    }
    return rc;
  }

  // the bottom-MLP shape K0 (<= 16) -> 512 -> 256 -> 128 with aligned
  // weights runs as one fused kernel
  if (in_dtype == DLRM_F32 && L == 3 && dims[0] <= kF3K0 && dims[1] == kF3D1 && dims[2] == kF3D2 &&
      dims[3] == kF3D3 && w_ld != nullptr) {
    bool ok = true;
    for (int l = 0; l < 3; ++l) ok = ok && aligned16(W[l]) && aligned16(bias[l]) && (w_ld[l] % 8) == 0;
    if (ok) {
      const int dev = current_device();
      static bool raised[kMaxDevices] = {false};
      if (!raised[dev]) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(mlp3_fused_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kF3Lds) != hipSuccess)
          return DLRM_E_HIP;
        raised[dev] = true;
      }
      const int vec_out = (out_ld % 4) == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0;
      uint16_t* a0 = save_acts ? reinterpret_cast<uint16_t*>(wsb + lay.act_off[0]) : nullptr;
      uint16_t* a1 = save_acts ? reinterpret_cast<uint16_t*>(wsb + lay.act_off[1]) : nullptr;
      uint16_t* a2 = save_acts ? reinterpret_cast<uint16_t*>(wsb + lay.act_off[2]) : nullptr;
      hipLaunchKernelGGL(mlp3_fused_kernel, dim3((unsigned)ceil_div(B, kF3Rows)), dim3(64 * kF3Waves), kF3Lds, stream,
                         static_cast<const float*>(in), in_ld, dims[0], M, static_cast<const uint16_t*>(W[0]),
                         (int64_t)w_ld[0], bias[0], static_cast<const uint16_t*>(W[1]), (int64_t)w_ld[1], bias[1],
                         static_cast<const uint16_t*>(W[2]), (int64_t)w_ld[2], bias[2],
                         (int)(last_act == DLRM_ACT_RELU), out, out_ld, vec_out, a0, lay.act_ld[0], a1, a2);
      return launch_status();
    }
  }

  // bf16 network: an fp32 input is rounded once into the workspace; a bf16
  // input is read in place unless it must be kept for the backward pass
  uint16_t* act0 = reinterpret_cast<uint16_t*>(wsb + lay.act_off[0]);
  const uint16_t* in0 = act0;
  int64_t ld0 = lay.act_ld[0];
  if (in_dtype == DLRM_F32) {
    rc = convert_to_bf16(static_cast<const float*>(in), in_ld, act0, lay.act_ld[0], M, dims[0], stream);
  } else if (!save_acts) {
    in0 = static_cast<const uint16_t*>(in);
    ld0 = in_ld;
  } else {
    const int Cpad = (int)lay.act_ld[0];
    const int64_t total = (int64_t)M * Cpad;
    hipLaunchKernelGGL(copy_bf16_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(in), in_ld, act0, lay.act_ld[0], M, dims[0], Cpad);
    rc = launch_status();
  }
  for (int l = 0; l < L && rc == DLRM_OK; ++l) {
    const int fi = dims[l], fo = dims[l + 1];
    const bool last = (l == L - 1);
    const bool relu = !last || last_act == DLRM_ACT_RELU;
    const uint16_t* src = l == 0 ? in0 : reinterpret_cast<const uint16_t*>(wsb + lay.act_off[l]);
    const int64_t ld_src = l == 0 ? ld0 : lay.act_ld[l];
    const uint16_t* w = static_cast<const uint16_t*>(W[l]);
    const int64_t wl = w_ld ? w_ld[l] : fi;
    void* dst = last ? static_cast<void*>(out) : static_cast<void*>(wsb + lay.act_off[l + 1]);
    const int64_t ld_dst = last ? out_ld : lay.act_ld[l + 1];
    if (l == L - 2 && dims[L] == 1) {
      // a hidden layer of at most 256 outputs followed by the single-output
      // layer: one launch computes both (the hidden rows are written only
      // when the backward pass will read them)
      DotOut dot;
      dot.w = static_cast<const uint16_t*>(W[L - 1]);
      dot.b = bias[L - 1];
      dot.out = out;
      dot.ldo = out_ld;
      dot.prob = prob;
      dot.relu = last_act == DLRM_ACT_RELU;
      rc = gemm_bf16_dot(src, ld_src, w, wl, bias[l], save_acts ? static_cast<uint16_t*>(dst) : nullptr, ld_dst, M, fo,
                         fi, dot, stream);
      if (rc == DLRM_OK) break;
      if (rc != DLRM_E_UNSUPPORTED) return rc;
      rc = DLRM_OK;
    }
    if (last && fo == 1)
      rc = gemv_bf16(src, ld_src, w, bias[l], out, out_ld, prob, M, fi, relu, stream);
    else
      rc = gemm_bf16(src, ld_src, w, wl, bias[l], dst, ld_dst, !last, M, fo, fi, relu, stream);
  }
  return rc;
}

extern "C" int dlrm_linear_fwd(const void* A, int64_t lda, const void* W, int64_t ldw, const float* bias, void* C,
                               int32_t out_dtype, int64_t ldc, int64_t M, int32_t N, int32_t K, int32_t act,
                               hipStream_t stream) {
  if (!A || !W || !C) return DLRM_E_INVALID;
  if (out_dtype != DLRM_F32 && out_dtype != DLRM_BF16) return DLRM_E_INVALID;
  if (act != DLRM_ACT_NONE && act != DLRM_ACT_RELU) return DLRM_E_INVALID;
  if (M < 1 || M > 0x7fffffffLL || N < 1 || K < 1 || lda < K || ldw < K || ldc < N) return DLRM_E_INVALID;
  const uint16_t* a = static_cast<const uint16_t*>(A);
  const uint16_t* w = static_cast<const uint16_t*>(W);
  if (N == 1) {
    if (out_dtype != DLRM_F32) return DLRM_E_INVALID;
    return gemv_bf16(a, lda, w, bias, static_cast<float*>(C), ldc, nullptr, (int)M, K, act == DLRM_ACT_RELU, stream);
  }
  return gemm_bf16(a, lda, w, ldw, bias, C, ldc, out_dtype == DLRM_BF16, (int)M, N, K, act == DLRM_ACT_RELU, stream);
}

extern "C" size_t dlrm_mlp_bwd_workspace_size(int64_t B, int32_t L, const int32_t* dims) {
  if (!dims) return 0;
  BwdLayout lay;
  if (!bwd_layout(B, L, dims, &lay)) return 0;
  return lay.bytes;
}

extern "C" int dlrm_mlp_bwd(int64_t B, int32_t L, const int32_t* dims, const void* const* W, const int32_t* w_ld,
                            int32_t last_act, const void* fwd_ws, const float* out, int64_t out_ld, const float* dY,
                            int64_t dy_ld, float* const* dW, float* const* db, float* dX, int64_t dx_ld, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  if (!dims || !W || !fwd_ws || !dY || !dW || !db) return DLRM_E_INVALID;
  if (last_act != DLRM_ACT_NONE && last_act != DLRM_ACT_RELU) return DLRM_E_INVALID;
  if (last_act == DLRM_ACT_RELU && !out) return DLRM_E_INVALID;
  if (B < 1 || B > 0x7fffffffLL) return DLRM_E_INVALID;
  FwdLayout fl;
  BwdLayout bl;
  if (!fwd_layout(B, L, dims, DLRM_BF16, 1, &fl) || !bwd_layout(B, L, dims, &bl)) return DLRM_E_INVALID;
  if (dy_ld < dims[L] || (out && out_ld < dims[L]) || (dX && dx_ld < dims[0])) return DLRM_E_INVALID;
  for (int l = 0; l < L; ++l) {
    if (!W[l] || !dW[l] || !db[l]) return DLRM_E_INVALID;
    if (w_ld && w_ld[l] < dims[l]) return DLRM_E_INVALID;
  }
  if (!ws || ws_bytes < bl.bytes) return DLRM_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) || (reinterpret_cast<uintptr_t>(fwd_ws) & 255u)) return DLRM_E_INVALID;

  const char* fws = static_cast<const char*>(fwd_ws);
  char* w = static_cast<char*>(ws);
  uint16_t* dlt[2] = {reinterpret_cast<uint16_t*>(w + bl.dlt[0]), reinterpret_cast<uint16_t*>(w + bl.dlt[1])};
  uint16_t* wT = reinterpret_cast<uint16_t*>(w + bl.wT);
  auto part_of = [&](int l) { return reinterpret_cast<float*>(w + bl.part[l]); };
  auto dbp_of = [&](int l) { return reinterpret_cast<float*>(w + bl.dbp[l]); };
  const int M = (int)B;
  FinArgs fin;
  fin.count = 0;
  int fin_blocks = 0;
  // the finishing launch for the layers recorded so far
  auto finish = [&]() -> int {
    if (fin.count == 0) return DLRM_OK;
    hipLaunchKernelGGL(grad_finalize_kernel, dim3((unsigned)fin_blocks), dim3(256), 0, stream, fin);
    fin.count = 0;
    fin_blocks = 0;
    return launch_status();
  };
  const dim3 b1(256);
  int rc = DLRM_OK;
  int db_chunks = 0;  // row chunks of the bias-gradient partials in dbp

  // 1. the last layer's delta from dY (fp32) and its bias gradient; every
  //    earlier layer's delta comes out of the input-gradient GEMM of the
  //    layer above it.  The weight-gradient GEMMs read the row-major delta
  //    and activations k-major (transposing reads from LDS), so no
  //    transposed copies are made.
  {
    const int fo = dims[L];
    const bool relu = last_act == DLRM_ACT_RELU;
    const float* y = relu ? out : dY;  // mask source unused when relu == 0
    const int64_t ldy = relu ? out_ld : dy_ld;
    auto al = [](const void* p, int64_t ld, int esz, int bytes) {
      return (reinterpret_cast<uintptr_t>(p) % bytes) == 0 && ((ld * esz) % bytes) == 0;
    };
    const int vec = al(dY, dy_ld, 4, 16) && al(dlt[0], bl.ld_dlt, 2, 8) && al(y, ldy, 4, 16);
    const int chunks = (int)ceil_div(B, kDRows);
    if (fo == 1)
      hipLaunchKernelGGL(delta1_kernel, dim3((unsigned)ceil_div(chunks, 4)), b1, 0, stream, dY, dy_ld, y, ldy, (int)relu,
                         dlt[0], bl.ld_dlt, dbp_of(L - 1), M);
    else
      hipLaunchKernelGGL((delta_db_kernel<float>), dim3((unsigned)ceil_div(fo, kDCols), (unsigned)chunks), b1, 0,
                         stream, dY, dy_ld, y, ldy, (int)relu, dlt[0], bl.ld_dlt, dbp_of(L - 1), M, fo, vec);
    db_chunks = chunks;
    rc = launch_status();
  }
  int cur = 0;
  for (int l = L - 1; l >= 0 && rc == DLRM_OK; --l) {
    const int fi = dims[l], fo = dims[l + 1];
    // 2. dW = delta^T x  (M = fo, N = fi, K = B), split over the batch;
    //    delta [B][fo] and x [B][fi] are both read k-major
    const uint16_t* x = reinterpret_cast<const uint16_t*>(fws + fl.act_off[l]);
    const int splits = wgrad_splits(B, fo, fi);
    const bool rank1_delta = fo == 1 && l > 0;  // a single-output layer above a ReLU layer
    if (fo == 1) {
      // its weight gradient and, above a ReLU layer, the delta below in one pass
      hipLaunchKernelGGL(rank1_kernel, dim3((unsigned)ceil_div(fi, 256), (unsigned)splits), b1, 0, stream, dlt[cur],
                         bl.ld_dlt, x, fl.act_ld[l], M, fi, part_of(l), (int)rank1_delta,
                         static_cast<const uint16_t*>(W[l]), dlt[cur ^ 1], bl.ld_dlt, rank1_delta ? dbp_of(l - 1) : nullptr);
      rc = launch_status();
    } else {
      rc = gemm_bf16_splitk_kmajor(dlt[cur], bl.ld_dlt, x, fl.act_ld[l], part_of(l), fo, fi, M, splits, stream);
    }
    if (rc != DLRM_OK) break;
    // dW from the partials and db from the partials the layer's delta left:
    // recorded here, computed by one launch after the last layer (nothing
    // in the pass reads dW or db)
    {
      if (fin.count == kFinLayers && (rc = finish()) != DLRM_OK) break;
      FinLayer& f = fin.l[fin.count++];
      f.part = part_of(l);
      f.dW = dW[l];
      f.dbp = dbp_of(l);
      f.db = db[l];
      f.ldw = fi;
      f.splits = splits;
      f.M = fo;
      f.N = fi;
      f.rblocks = (int)ceil_div((int64_t)fo * fi, 256);
      f.chunks = db_chunks;
      f.block0 = fin_blocks;
      fin_blocks += f.rblocks + (int)ceil_div(fo, 64);
    }
    if (l == 0 && !dX) break;
    // 3. the input gradient delta W  (M = B, N = fi, K = fo): W [fo][fi] is
    //    read k-major where its rows allow, else through a transposed copy
    const int64_t wl = w_ld ? w_ld[l] : fi;
    const uint16_t* Wl = static_cast<const uint16_t*>(W[l]);
    if (rank1_delta) {  // the delta below came out of the weight-gradient pass
      db_chunks = (int)ceil_div(B, kR1Rows);
      cur ^= 1;
      continue;
    }
    const bool wk = aligned16(Wl) && (wl % 8) == 0;
    if (!wk && (rc = transpose_bf16(Wl, wl, wT, bl.ld_dlt, fo, fi, stream)) != DLRM_OK) break;
    const uint16_t* wop = wk ? Wl : wT;
    const int64_t wop_ld = wk ? wl : bl.ld_dlt;
    if (l == 0) {  // the MLP input's gradient, fp32
      rc = gemm_bf16_ex(dlt[cur], bl.ld_dlt, false, wop, wop_ld, wk, dX, dx_ld, false, M, fi, fo, stream);
      break;
    }
    // layer l-1 is a ReLU layer whose output is layer l's input x: its delta
    // (masked by x > 0, bf16, row-major) and bias-gradient partials come
    // straight out of the GEMM
    DeltaOut dout;
    dout.y = x;
    dout.ldy = fl.act_ld[l];
    dout.dbp = dbp_of(l - 1);
    int tile_rows = 128;
    if ((rc = gemm_bf16_delta(dlt[cur], bl.ld_dlt, wop, wop_ld, wk, M, fi, fo, dlt[cur ^ 1], bl.ld_dlt, dout,
                              &tile_rows, stream)) != DLRM_OK)
      break;
    db_chunks = (int)ceil_div(B, tile_rows);
    cur ^= 1;
  }
  if (rc == DLRM_OK) rc = finish();
  return rc;
}

extern "C" int dlrm_bce_grad(const float* logit, int64_t logit_ld, const float* y, int64_t B, float* dY,
                             hipStream_t stream) {
  if (!logit || !y || !dY || B < 1 || logit_ld < 1) return DLRM_E_INVALID;
  hipLaunchKernelGGL(bce_grad_kernel, dim3((unsigned)ceil_div(B, 256)), dim3(256), 0, stream, logit, logit_ld, y, B,
                     dY);
  return launch_status();
}
