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
// workgroup of eight waves owns 128 rows: it rounds its fp32 input rows to
// bf16, keeps the 128 x 512 hidden activations and then the 128 x 256 ones
// in LDS (bf16, the rounding points of the layer-by-layer path), and writes
// only the fp32 output rows (and, for training, the bf16 activations the
// backward pass reads).  Weights are read straight from global memory (L2
// resident) as MFMA fragments, a few k-steps ahead.  As in the GEMM, the W
// fragment is the first MFMA operand, so each lane owns one row and groups of
// four consecutive columns; accumulators start from the bias.
constexpr int kF3Rows = 128, kF3D1 = 512, kF3D2 = 256, kF3D3 = 128, kF3K0 = 16;
constexpr int kF3Lds = kF3Rows * kF3D1 * 2;  // 128 KB: the first hidden layer, later the second

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t gld8(const uint16_t* p) {
  return *(const __attribute__((address_space(1))) bf16x8_t*)(p);
}
// byte offset of 16-byte chunk c of row r in an LDS matrix with `cpr` chunks
// per row; the chunk index is XOR-ed with the row's low four bits so that the
// 16 rows one LDS cycle serves hit distinct banks
__device__ __forceinline__ int f3_off(int r, int c, int cpr) { return (r * cpr + (c ^ (r & 15))) * 16; }

// bias + optional ReLU, bf16 rounding and the cross-half swap of one 32 x 32
// accumulator block: returns the two 16-byte chunks this lane owns, columns
// 8*(l/32) .. +7 and 16 + 8*(l/32) .. +7 of the block
__device__ __forceinline__ void f3_pack(const f32x16_t& a, bool relu, uint4& lo, uint4& hi) {
  uint32_t pk[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float v0 = a[4 * g + 2 * h], v1 = a[4 * g + 2 * h + 1];
      if (relu) {
        v0 = v0 > 0.f ? v0 : 0.f;
        v1 = v1 > 0.f ? v1 : 0.f;
      }
      pk[g][h] = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
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

// acc[tm][tn] += sum over K of W-fragments x LDS A-fragments; W rows
// w_rows[tn] (already offset by this lane's 8 k), A rows in LDS with `cpr`
// chunks per row.  The W fragments of the next P - 1 k-steps and the A
// fragments of the next k-step are in flight during each step's MFMAs (the
// scheduling barriers keep the loads ahead of the MFMAs).
template <int TM, int TN, int KSTEPS, int P>
__device__ __forceinline__ void f3_layer(f32x16_t (&acc)[TM][TN], const uint16_t* const (&w_rows)[TN],
                                         const char* lds, int cpr, int row0, int r32, int half) {
  static_assert(KSTEPS % P == 0, "whole prefetch rounds");
  bf16x8_t wb[P][TN], af[2][TM];
#pragma unroll
  for (int p = 0; p < P - 1; ++p)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) wb[p][tn] = gld8(w_rows[tn] + p * 16);
  auto read_a = [&](int ks, int buf) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int r = row0 + tm * 32 + r32;
      af[buf][tm] = *reinterpret_cast<const bf16x8_t*>(lds + f3_off(r, 2 * ks + half, cpr));
    }
  };
  read_a(0, 0);
  for (int ks0 = 0; ks0 < KSTEPS; ks0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int ks = ks0 + p;
      const int ahead = ks + P - 1 < KSTEPS ? ks + P - 1 : KSTEPS - 1;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) wb[(p + P - 1) % P][tn] = gld8(w_rows[tn] + ahead * 16);
      read_a(ks + 1 < KSTEPS ? ks + 1 : KSTEPS - 1, (p + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb[p][tn], af[p & 1][tm], acc[tm][tn], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

__global__ __launch_bounds__(512) void mlp3_fused_kernel(
    const float* __restrict__ in, int64_t in_ld, int K0, int M, const uint16_t* __restrict__ W1, int64_t w1_ld,
    const float* __restrict__ b1, const uint16_t* __restrict__ W2, int64_t w2_ld, const float* __restrict__ b2,
    const uint16_t* __restrict__ W3, int64_t w3_ld, const float* __restrict__ b3, int relu3, float* __restrict__ out,
    int64_t out_ld, int vec_out, uint16_t* __restrict__ act0, int64_t ld0, uint16_t* __restrict__ act1,
    uint16_t* __restrict__ act2) {
  extern __shared__ __attribute__((aligned(16))) char f3_smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves
  const int m0 = blockIdx.x * kF3Rows;
  const int rowl = wm * 64 + r32;           // local row of block tm = 0

  // ---- layer 1: K0 -> 512.  Wave tile 64 x 128, one k-step of 16.
  {
    bf16x8_t a1[2];
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      const int row = min(m0 + rowl + tm * 32, M - 1);
      const float* src = in + (int64_t)row * in_ld;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = half * 8 + 2 * q;
        const uint16_t lo = k < K0 ? f32_to_bf16(src[k]) : (uint16_t)0;
        const uint16_t hi = k + 1 < K0 ? f32_to_bf16(src[k + 1]) : (uint16_t)0;
        w[q] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
      const uint4 u = make_uint4(w[0], w[1], w[2], w[3]);
      a1[tm] = *reinterpret_cast<const bf16x8_t*>(&u);
      // the rounded input rows are layer 1's saved input (the first 4 waves store them)
      if (act0 != nullptr && wn == 0 && m0 + rowl + tm * 32 < M && half * 8 < ld0)
        *reinterpret_cast<uint4*>(act0 + (int64_t)(m0 + rowl + tm * 32) * ld0 + half * 8) = u;
    }
    f32x16_t acc[2][4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const float* bp = b1 + wn * 128 + tn * 32 + 4 * half;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float b = bp[8 * (v >> 2) + (v & 3)];
        acc[0][tn][v] = b;
        acc[1][tn][v] = b;
      }
    }
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      // W1 row, k = 8*half .. +7; columns at or past K0 read as zero
      const uint16_t* wr = W1 + (int64_t)(wn * 128 + tn * 32 + r32) * w1_ld + half * 8;
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (half * 8 < K0) {
        u = *reinterpret_cast<const uint4*>(wr);
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = half * 8 + 2 * q;
          if (k >= K0) w[q] = 0u;
          else if (k + 1 >= K0) w[q] &= 0xffffu;
        }
        u = make_uint4(w[0], w[1], w[2], w[3]);
      }
      const bf16x8_t wb = *reinterpret_cast<const bf16x8_t*>(&u);
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb, a1[tm], acc[tm][tn], 0, 0, 0);
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        uint4 lo, hi;
        f3_pack(acc[tm][tn], true, lo, hi);
        const int r = rowl + tm * 32, c = (wn * 128 + tn * 32) / 8 + half;  // 16-byte chunk of the row
        *reinterpret_cast<uint4*>(f3_smem + f3_off(r, c, 64)) = lo;
        *reinterpret_cast<uint4*>(f3_smem + f3_off(r, c + 2, 64)) = hi;
        if (act1 != nullptr && m0 + r < M) {
          uint16_t* g = act1 + (int64_t)(m0 + r) * kF3D1 + c * 8;
          *reinterpret_cast<uint4*>(g) = lo;
          *reinterpret_cast<uint4*>(g + 16) = hi;
        }
      }
  }
  __syncthreads();

  // ---- layer 2: 512 -> 256.  Wave tile 64 x 64, 32 k-steps.
  {
    f32x16_t acc[2][2];
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const float* bp = b2 + wn * 64 + tn * 32 + 4 * half;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float b = bp[8 * (v >> 2) + (v & 3)];
        acc[0][tn][v] = b;
        acc[1][tn][v] = b;
      }
    }
    const uint16_t* const wr[2] = {W2 + (int64_t)(wn * 64 + r32) * w2_ld + half * 8,
                                   W2 + (int64_t)(wn * 64 + 32 + r32) * w2_ld + half * 8};
    f3_layer<2, 2, kF3D1 / 16, 8>(acc, wr, f3_smem, 64, wm * 64, r32, half);
    __syncthreads();  // every wave is done reading the first hidden layer
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        uint4 lo, hi;
        f3_pack(acc[tm][tn], true, lo, hi);
        const int r = rowl + tm * 32, c = (wn * 64 + tn * 32) / 8 + half;
        *reinterpret_cast<uint4*>(f3_smem + f3_off(r, c, 32)) = lo;
        *reinterpret_cast<uint4*>(f3_smem + f3_off(r, c + 2, 32)) = hi;
        if (act2 != nullptr && m0 + r < M) {
          uint16_t* g = act2 + (int64_t)(m0 + r) * kF3D2 + c * 8;
          *reinterpret_cast<uint4*>(g) = lo;
          *reinterpret_cast<uint4*>(g + 16) = hi;
        }
      }
  }
  __syncthreads();

  // ---- layer 3: 256 -> 128, fp32 out.  Wave tile 64 x 32, 16 k-steps.
  {
    f32x16_t acc[2][1];
    {
      const float* bp = b3 + wn * 32 + 4 * half;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float b = bp[8 * (v >> 2) + (v & 3)];
        acc[0][0][v] = b;
        acc[1][0][v] = b;
      }
    }
    const uint16_t* const wr[1] = {W3 + (int64_t)(wn * 32 + r32) * w3_ld + half * 8};
    f3_layer<2, 1, kF3D2 / 16, 8>(acc, wr, f3_smem, 32, wm * 64, r32, half);
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      const int row = m0 + rowl + tm * 32;
      if (row >= M) continue;
      float* o = out + (int64_t)row * out_ld + wn * 32 + 4 * half;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = acc[tm][0][4 * g + q];
          if (relu3) v[q] = v[q] > 0.f ? v[q] : 0.f;
        }
        if (vec_out) {
          *reinterpret_cast<float4*>(o + 8 * g) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[8 * g + q] = v[q];
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
// columns l, l+64, l+128, l+192, so every global access is coalesced.
constexpr int kDRows = 64, kDCols = 256;
template <typename YT>
__global__ __launch_bounds__(256) void delta_db_kernel(const float* __restrict__ g, int64_t ldg,
                                                       const YT* __restrict__ y, int64_t ldy, int relu,
                                                       uint16_t* __restrict__ dlt, int64_t ldd,
                                                       uint16_t* __restrict__ dltT, int64_t ldt,
                                                       float* __restrict__ part, int B, int N) {
  __shared__ uint16_t tile[kDRows][kDCols + 2];
  __shared__ float red[4][kDCols];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * kDCols, r0 = blockIdx.y * kDRows;
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = wave; i < kDRows; i += 4) {
    const int r = r0 + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int cl = lane + 64 * e, c = c0 + cl;
      float v = 0.f;
      if (r < B && c < N) {
        v = g[(int64_t)r * ldg + c];
        if (relu && !positive<YT>(y + (int64_t)r * ldy + c)) v = 0.f;
      }
      const uint16_t h = f32_to_bf16(v);
      tile[i][cl] = h;
      sum[e] = sum[e] + v;
      if (r < B && c < N) dlt[(int64_t)r * ldd + c] = h;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) red[wave][lane + 64 * e] = sum[e];
  __syncthreads();
  {
    const int cl = threadIdx.x, c = c0 + cl;
    if (c < N) part[(int64_t)blockIdx.y * N + c] = ((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl];
    if (c < N) {
      // column c of the tile is row c of delta^T: 64 rows, 8 per 16-byte store
      uint16_t* dst = dltT + (int64_t)c * ldt + r0;
#pragma unroll
      for (int j = 0; j < kDRows / 8; ++j) {
        if (r0 + 8 * j >= B) break;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (uint32_t)tile[8 * j + 2 * q][cl] | ((uint32_t)tile[8 * j + 2 * q + 1][cl] << 16);
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
    for (int c = wave; c < chunks; c += 4) s = s + part[(int64_t)c * N + o];
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
    for (int l = 0; l < 3; ++l) ok = ok && aligned16(W[l]) && (w_ld[l] % 8) == 0;
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
      hipLaunchKernelGGL(mlp3_fused_kernel, dim3((unsigned)ceil_div(B, kF3Rows)), dim3(512), kF3Lds, stream,
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
    if (l == L - 1) {
      const float* y = relu ? out : g;  // mask source unused when relu == 0
      const int64_t ldy = relu ? out_ld : ldg;
      hipLaunchKernelGGL((delta_db_kernel<float>), gd, b1, 0, stream, g, ldg, y, ldy, (int)relu, dlt, bl.ld_dlt, dltT,
                         bl.ld_B, dbp, M, fo);
    } else {
      const uint16_t* y = reinterpret_cast<const uint16_t*>(fws + fl.act_off[l + 1]);
      hipLaunchKernelGGL((delta_db_kernel<uint16_t>), gd, b1, 0, stream, g, ldg, y, fl.act_ld[l + 1], (int)relu, dlt,
                         bl.ld_dlt, dltT, bl.ld_B, dbp, M, fo);
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
