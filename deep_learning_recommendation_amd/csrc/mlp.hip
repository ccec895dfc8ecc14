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
// Backward (bf16 networks): per layer, delta = g * 1[y > 0] (bf16 for the
// MFMA operands), db by a deterministic two-stage column sum, dW = delta^T x
// as a split-K MFMA GEMM over the batch (partials summed in a fixed order),
// and g_prev = delta W.  Transposed copies make every GEMM the K-contiguous
// form the MFMA kernel reads.
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
// workgroup of four waves (one per SIMD) owns 128 rows, each wave 32 of
// them, and every activation of a wave's rows stays in its registers: with
// the W fragment as the first MFMA operand, a lane holds one row and groups
// of four consecutive output columns, and after bias, ReLU, bf16 rounding
// and one cross-half lane swap (v_permlane32_swap) each lane holds eight
// consecutive columns -- exactly the operand layout of the next layer's
// MFMA (row l % 32, k = 8 * (l / 32) .. +7 of each 16-wide k-step).  The
// rounding points are those of the layer-by-layer path (input, hidden
// activations in bf16; fp32 accumulation; fp32 output).
//
// The weights of layers 2 and 3 stream through a ring of four 32 KB LDS
// stages, loaded straight from global memory (global_load_lds_dwordx4,
// coalesced rows): ten chunks, eight of W2 (64 k x 256 rows) and two of W3
// (128 k x 128 rows), three in flight ahead of the one being used.  Layer
// 1's weights (512 x K0) are read as fragments from global memory.  The
// output rows are written in fp32; for training the bf16 input and hidden
// activations the backward pass reads are written as well.
constexpr int kF3Rows = 128, kF3D1 = 512, kF3D2 = 256, kF3D3 = 128, kF3K0 = 16;
constexpr int kF3Stage = 32768, kF3Ring = 4 * kF3Stage;
constexpr int kF3Lds = kF3Ring + 4096;  // the ring, then the three bias vectors (2 KB, 1 KB, 512 B)
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

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void mlp3_fused_kernel(
    const float* __restrict__ in, int64_t in_ld, int K0, int M, const uint16_t* __restrict__ W1, int64_t w1_ld,
    const float* __restrict__ b1, const uint16_t* __restrict__ W2, int64_t w2_ld, const float* __restrict__ b2,
    const uint16_t* __restrict__ W3, int64_t w3_ld, const float* __restrict__ b3, int relu3, float* __restrict__ out,
    int64_t out_ld, int vec_out, uint16_t* __restrict__ act0, int64_t ld0, uint16_t* __restrict__ act1,
    uint16_t* __restrict__ act2) {
  extern __shared__ __attribute__((aligned(1024))) char f3_smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const int row = blockIdx.x * kF3Rows + wave * 32 + r32;  // this lane's row (all layers)
  const bool row_ok = row < M;

  // chunk c of the weight ring into stage c % 4: 32 instructions of 1 KB,
  // eight per wave; instruction j of wave w fills rows (8w + j) * (64 / cpr) ..
  auto issue = [&](int c) {
    char* st = f3_smem + (c & 3) * kF3Stage;
    const int cpr = f3_cpr(c), rpi = 64 / cpr;
    const uint16_t* base = c < 8 ? W2 : W3;
    const int64_t ld = c < 8 ? w2_ld : w3_ld;
    const int k0 = c < 8 ? c * 64 : (c - 8) * 128;
    const int lrow = lane / cpr, lpc = lane % cpr;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = (wave * 8 + j) * rpi + lrow;
      lds_dma16_opaque(base + (int64_t)n * ld + k0 + (lpc ^ f3_swz(n, cpr)) * 8, st + (wave * 8 + j) * 1024);
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
  // wait until at most `younger` chunks issued after the awaited one are still in flight
  auto wait_younger = [&](int younger) {
    if (younger >= 4) wait_vmcnt<32>();
    else if (younger == 3) wait_vmcnt<24>();
    else if (younger == 2) wait_vmcnt<16>();
    else if (younger == 1) wait_vmcnt<8>();
    else wait_vmcnt<0>();
  };

  // bias vectors into LDS first (one 1 KB instruction per wave; lanes past
  // the end of b3 re-read its start into the padding)
  {
    char* ba = f3_smem + kF3Ring;
    const int off = wave * 1024 + lane * 16;
    const float* src = off < 2048 ? b1 + off / 4 : off < 3072 ? b2 + (off - 2048) / 4 : off < 3584 ? b3 + (off - 3072) / 4 : b3;
    lds_dma16_opaque(src, ba + wave * 1024);
  }
  // ---- operands of layer 1 in registers: this lane's input row (k = 8*(l/32)
  // .. +7, bf16) and the W1 fragments of the 16 output blocks (rows 32b + l%32,
  // the same k; columns at or past K0 read as zero).  Branch-free, so that
  // every load is in flight at once: out-of-range positions re-read an
  // in-range one and are masked afterwards.
  float x[8];
  {
    const float* src = in + (int64_t)(row_ok ? row : M - 1) * in_ld;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int k = half * 8 + q;
      x[q] = src[k < K0 ? k : K0 - 1];
    }
  }
  uint4 w1f[kF3D1 / 32];
  const int w1k = half * 8 < K0 ? half * 8 : 0;  // an in-range start for lanes whose k is all masked
#pragma unroll
  for (int b = 0; b < kF3D1 / 32; ++b)
    w1f[b] = *reinterpret_cast<const uint4*>(W1 + (int64_t)(b * 32 + r32) * w1_ld + w1k);
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any is used
  uint32_t win[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = half * 8 + 2 * q;
    const uint32_t lo = k < K0 ? (uint32_t)f32_to_bf16(x[2 * q]) : 0u;
    const uint32_t hi = k + 1 < K0 ? (uint32_t)f32_to_bf16(x[2 * q + 1]) : 0u;
    win[q] = lo | (hi << 16);
  }
#pragma unroll
  for (int b = 0; b < kF3D1 / 32; ++b) {
    uint32_t x[4] = {w1f[b].x, w1f[b].y, w1f[b].z, w1f[b].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = half * 8 + 2 * q;
      x[q] = k >= K0 ? 0u : (k + 1 >= K0 ? (x[q] & 0xffffu) : x[q]);
    }
    w1f[b] = make_uint4(x[0], x[1], x[2], x[3]);
  }
  // the plain loads and the bias vectors have landed before any chunk is
  // issued, so no later wait of the compiler's covers a chunk
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  issue(0);
  issue(1);
  issue(2);
  issue(3);
  const char* bias1 = f3_smem + kF3Ring;
  const char* bias2 = bias1 + 2048;
  const char* bias3 = bias1 + 3072;

  // ---- layer 1: K0 -> 512, 16 output blocks of 32 columns, one k-step
  uint4 h1[32];  // bf16 layer-1 activations in layer-2 operand order (k-step s = h1[s])
  {
    const uint4 ua = make_uint4(win[0], win[1], win[2], win[3]);
    if (act0 != nullptr && row_ok && half * 8 < ld0) *reinterpret_cast<uint4*>(act0 + (int64_t)row * ld0 + half * 8) = ua;
    const bf16x8_t a1 = as_bf16x8(ua);
    // four blocks at a time, so that four independent MFMA and packing
    // chains interleave
#pragma unroll
    for (int b0 = 0; b0 < kF3D1 / 32; b0 += 4) {
      f32x16_t acc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f3_bias(acc[j], bias1, (b0 + j) * 32, half);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w1f[b0 + j]), a1, acc[j], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) f3_pack(acc[j], true, h1[2 * (b0 + j)], h1[2 * (b0 + j) + 1]);
    }
    if (act1 != nullptr && row_ok) {
      uint16_t* g = act1 + (int64_t)row * kF3D1 + 8 * half;
#pragma unroll
      for (int b = 0; b < kF3D1 / 32; ++b) {
        *reinterpret_cast<uint4*>(g + b * 32) = h1[2 * b];
        *reinterpret_cast<uint4*>(g + b * 32 + 16) = h1[2 * b + 1];
      }
    }
  }

  // ---- layer 2: 512 -> 256 (chunks 0 .. 7, four k-steps each, 8 output blocks)
  f32x16_t acc2[8];
#pragma unroll
  for (int tn = 0; tn < 8; ++tn) f3_bias(acc2[tn], bias2, tn * 32, half);
  bf16x8_t fb[2][8];
  wait_younger(3);  // chunk 0
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  read_b(0, 0, fb[0], 0, 8);
  int buf = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) {
        read_b(c, ks + 1, fb[buf ^ 1], 0, 8);
      } else {
        // hand-over to chunk c+1: after the barrier every wave's reads of
        // chunk c are done, so chunk c+4 can load into its stage.  Layer 3
        // starts with both of its chunks resident.
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        wait_younger(c < 7 ? (7 - c < 2 ? 7 - c : 2) : 0);
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (c + 4 < kF3Chunks) issue(c + 4);
        if (c < 7) read_b(c + 1, 0, fb[buf ^ 1], 0, 8);
        else read_b(8, 0, fb[buf ^ 1], 0, 2);
      }
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8_t a = as_bf16x8(h1[c * 4 + ks]);
#pragma unroll
      for (int tn = 0; tn < 8; ++tn) acc2[tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][tn], a, acc2[tn], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      buf ^= 1;
    }
  }
  // layer 2's activations become layer 3's operands
  uint4 h2[16];
#pragma unroll
  for (int tn = 0; tn < 8; ++tn) f3_pack(acc2[tn], true, h2[2 * tn], h2[2 * tn + 1]);
  if (act2 != nullptr && row_ok) {
    uint16_t* g = act2 + (int64_t)row * kF3D2 + 8 * half;
#pragma unroll
    for (int tn = 0; tn < 8; ++tn) {
      *reinterpret_cast<uint4*>(g + tn * 32) = h2[2 * tn];
      *reinterpret_cast<uint4*>(g + tn * 32 + 16) = h2[2 * tn + 1];
    }
  }

  // ---- layer 3: 256 -> 128 in two halves of 64 columns (chunks 8 and 9
  // hold k 0-127 and 128-255); each half's fp32 rows are stored while the
  // next half computes
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f32x16_t acc3[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) f3_bias(acc3[j], bias3, (2 * hf + j) * 32, half);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      if (ks < 15) read_b(8 + ((ks + 1) >> 3), (ks + 1) & 7, fb[buf ^ 1], 2 * hf, 2);
      else if (hf == 0) read_b(8, 0, fb[buf ^ 1], 2, 2);
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8_t a = as_bf16x8(h2[ks]);
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
          float* d = o + (2 * hf + j) * 32 + 8 * g;
          if (vec_out) {
            *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) d[q] = v[q];
          }
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
// g) rounded to bf16 and stored row-major [B][ldd] (for the input gradient)
// and transposed [N][ldt] (for the weight gradient, K = batch contiguous),
// plus fp32 column sums of delta per 64-row chunk (for the bias gradient).
// Block: 64 rows x 256 columns; wave w takes rows w, w+4, ..., lane l the
// four consecutive columns 4l .. 4l+3 (16-byte loads of g, 8- or 16-byte
// loads of y, 8-byte stores of delta when `vec`), eight rows' loads in flight
// before the first is used.  The column sums add the rows in the same order
// as a one-row-at-a-time walk.
constexpr int kDRows = 64, kDCols = 256, kDBatch = 8;
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
                                                       uint16_t* __restrict__ dltT, int64_t ldt,
                                                       float* __restrict__ part, int B, int N, int vec) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kDRows][kDCols + 8];
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
      *reinterpret_cast<uint2*>(&tile[i][cl]) =
          make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
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
    if (col < N) {
      // column cc of the tile is row col of delta^T: 64 rows, 8 per 16-byte store
      uint16_t* dst = dltT + (int64_t)col * ldt + r0;
#pragma unroll
      for (int j = 0; j < kDRows / 8; ++j) {
        if (r0 + 8 * j >= B) break;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (uint32_t)tile[8 * j + 2 * q][cc] | ((uint32_t)tile[8 * j + 2 * q + 1][cc] << 16);
        *reinterpret_cast<uint4*>(dst + 8 * j) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

// db[o] = sum of the per-chunk partials: 64 columns per block, wave w sums
// chunks w, w+4, ... and the four wave sums are added in wave order.
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ part, int chunks, int N,
                                                           float* __restrict__ db) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int o = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (o < N)
    for (int c0 = wave; c0 < chunks; c0 += 32) {  // eight loads in flight, added in chunk order
      float v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = (c0 + 4 * t < chunks) ? part[(int64_t)(c0 + 4 * t) * N + o] : 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (c0 + 4 * t < chunks) s = s + v[t];
    }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && o < N) db[o] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

__global__ __launch_bounds__(256) void bce_grad_kernel(const float* __restrict__ logit, int64_t ld,
                                                       const float* __restrict__ y, int64_t B, float* __restrict__ dY) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const float s = 1.f / (1.f + expf(-logit[b * ld]));
  dY[b] = (s - y[b]) / (float)B;
}

struct BwdLayout {
  size_t g[2], dlt, dltT, xT, wT, part, dbp, bytes;
  int64_t ld_dlt, ld_B, splits_max;
};

constexpr int kMaxSplits = 16;

bool bwd_layout(int64_t B, int32_t L, const int32_t* dims, BwdLayout* lay) {
  if (L < 1 || L > 64 || B < 1) return false;
  int64_t wmax = 0, wfo = 0, prod = 0;
  for (int l = 0; l <= L; ++l) {
    if (dims[l] < 1) return false;
    wmax = dims[l] > wmax ? dims[l] : wmax;
  }
  for (int l = 0; l < L; ++l) {
    wfo = dims[l + 1] > wfo ? dims[l + 1] : wfo;
    const int64_t p = (int64_t)dims[l] * dims[l + 1];
    prod = p > prod ? p : prod;
  }
  Carver cv(nullptr);
  lay->ld_dlt = round_up(wfo, 8);
  lay->ld_B = round_up(B, 8);
  lay->splits_max = kMaxSplits;
  auto take = [&](size_t bytes) {
    cv.used = (size_t)round_up((int64_t)cv.used, 256);
    const size_t at = cv.used;
    cv.used += bytes;
    return at;
  };
  lay->g[0] = take(4 * (size_t)(B * wmax));
  lay->g[1] = take(4 * (size_t)(B * wmax));
  lay->dlt = take(2 * (size_t)(B * lay->ld_dlt));
  lay->dltT = take(2 * (size_t)(wfo * lay->ld_B));
  lay->xT = take(2 * (size_t)(wmax * lay->ld_B));
  lay->wT = take(2 * (size_t)(wmax * lay->ld_dlt));
  lay->part = take(4 * (size_t)(kMaxSplits * prod));
  lay->dbp = take(4 * (size_t)(ceil_div(B, kDRows) * wfo));
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
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
      static bool raised[64] = {false};
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
      hipLaunchKernelGGL(mlp3_fused_kernel, dim3((unsigned)ceil_div(B, kF3Rows)), dim3(256), kF3Lds, stream,
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
    if (last && fo == 1)
      rc = gemv_bf16(src, ld_src, w, bias[l], out, out_ld, prob, M, fi, relu, stream);
    else
      rc = gemm_bf16(src, ld_src, w, wl, bias[l], dst, ld_dst, !last, M, fo, fi, relu, stream);
  }
  return rc;
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
  float* gbuf[2] = {reinterpret_cast<float*>(w + bl.g[0]), reinterpret_cast<float*>(w + bl.g[1])};
  uint16_t* dlt = reinterpret_cast<uint16_t*>(w + bl.dlt);
  uint16_t* dltT = reinterpret_cast<uint16_t*>(w + bl.dltT);
  uint16_t* xT = reinterpret_cast<uint16_t*>(w + bl.xT);
  uint16_t* wT = reinterpret_cast<uint16_t*>(w + bl.wT);
  float* part = reinterpret_cast<float*>(w + bl.part);
  float* dbp = reinterpret_cast<float*>(w + bl.dbp);
  const int M = (int)B;
  const int chunks = (int)ceil_div(B, kDRows);

  const float* g = dY;
  int64_t ldg = dy_ld;
  int rc = DLRM_OK;
  for (int l = L - 1; l >= 0 && rc == DLRM_OK; --l) {
    const int fi = dims[l], fo = dims[l + 1];
    const bool relu = (l < L - 1) || last_act == DLRM_ACT_RELU;
    const dim3 b1(256), gd((unsigned)ceil_div(fo, kDCols), (unsigned)chunks);
    // 1. delta (bf16, both layouts) and the bias-gradient partials
    // vector accesses: g 16-byte, delta 8-byte and y (16-byte fp32 / 8-byte bf16) aligned rows
    auto al = [](const void* p, int64_t ld, int esz, int bytes) {
      return (reinterpret_cast<uintptr_t>(p) % bytes) == 0 && ((ld * esz) % bytes) == 0;
    };
    const bool vg = al(g, ldg, 4, 16) && al(dlt, bl.ld_dlt, 2, 8);
    if (l == L - 1) {
      const float* y = relu ? out : g;  // mask source unused when relu == 0
      const int64_t ldy = relu ? out_ld : ldg;
      const int vec = vg && al(y, ldy, 4, 16);
      hipLaunchKernelGGL((delta_db_kernel<float>), gd, b1, 0, stream, g, ldg, y, ldy, (int)relu, dlt, bl.ld_dlt, dltT,
                         bl.ld_B, dbp, M, fo, vec);
    } else {
      const uint16_t* y = reinterpret_cast<const uint16_t*>(fws + fl.act_off[l + 1]);
      const int vec = vg && al(y, fl.act_ld[l + 1], 2, 8);
      hipLaunchKernelGGL((delta_db_kernel<uint16_t>), gd, b1, 0, stream, g, ldg, y, fl.act_ld[l + 1], (int)relu, dlt,
                         bl.ld_dlt, dltT, bl.ld_B, dbp, M, fo, vec);
    }
    hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)ceil_div(fo, 64)), b1, 0, stream, dbp, chunks, fo, db[l]);
    if ((rc = launch_status()) != DLRM_OK) break;
    // 2. dW = delta^T x  (M = fo, N = fi, K = B), split over the batch
    const uint16_t* x = reinterpret_cast<const uint16_t*>(fws + fl.act_off[l]);
    if ((rc = transpose_bf16(x, fl.act_ld[l], xT, bl.ld_B, M, fi, stream)) != DLRM_OK) break;
    const int64_t tiles = ceil_div(fo, 128) * ceil_div(fi, 128);
    int splits = (int)ceil_div(512, tiles);
    if (splits > kMaxSplits) splits = kMaxSplits;
    if (splits > (int)ceil_div(M, 256)) splits = (int)ceil_div(M, 256);
    if (splits < 1) splits = 1;
    if ((rc = gemm_bf16_splitk(dltT, bl.ld_B, xT, bl.ld_B, part, fo, fi, M, splits, stream)) != DLRM_OK) break;
    if ((rc = reduce_splits(part, splits, fo, fi, nullptr, dW[l], fi, false, stream)) != DLRM_OK) break;
    // 3. g_prev = delta W  (M = B, N = fi, K = fo)
    if (l > 0 || dX) {
      const int64_t wl = w_ld ? w_ld[l] : fi;
      if ((rc = transpose_bf16(static_cast<const uint16_t*>(W[l]), wl, wT, bl.ld_dlt, fo, fi, stream)) != DLRM_OK) break;
      float* gp = (l == 0) ? dX : gbuf[l & 1];
      const int64_t ldp = (l == 0) ? dx_ld : fi;
      rc = gemm_bf16(dlt, bl.ld_dlt, wT, bl.ld_dlt, nullptr, gp, ldp, false, M, fi, fo, false, stream);
      g = gp;
      ldg = ldp;
    }
  }
  return rc;
}

extern "C" int dlrm_bce_grad(const float* logit, int64_t logit_ld, const float* y, int64_t B, float* dY,
                             hipStream_t stream) {
  if (!logit || !y || !dY || B < 1 || logit_ld < 1) return DLRM_E_INVALID;
  hipLaunchKernelGGL(bce_grad_kernel, dim3((unsigned)ceil_div(B, 256)), dim3(256), 0, stream, logit, logit_ld, y, B,
                     dY);
  return launch_status();
}
