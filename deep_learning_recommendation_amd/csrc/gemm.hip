// GEMM family for the bottom and top MLPs ("Deep Learning Recommendation
// Model (DLRM)" explainer, Key Method Details: Bottom MLP, Top MLP;
// briansu.co DLRM, Key equations, Output).
//
// gemm_bf16: C = act(A W^T + b) with A [M][K] and W [N][K] both K-contiguous,
// the natural layout of a fully connected layer y = x W^T.  gfx950 bf16 MFMA
// v_mfma_f32_32x32x16_bf16: each lane feeds 8 consecutive k of one row of A
// (row l % 32, k (l / 32) * 8) and of W, so both operands are read from LDS
// with one 16-byte ds_read per fragment.  The fast kernel (16-byte aligned
// operands) is persistent, loads tiles straight from global memory into LDS,
// keeps its accumulators in registers and writes C from registers; a
// generic kernel covers any other layout.
#include "gemm.hpp"

namespace dlrm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 32;
constexpr int LDS_STRIDE = BK + 8;  // bf16 per LDS row: 80 bytes

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ float relu_f(float v) { return v > 0.f ? v : 0.f; }

// bf16 pair with each half kept where the matching half of y is a positive
// bf16 value and zeroed elsewhere
__device__ __forceinline__ uint32_t mask_pair(uint32_t v, uint32_t y) {
  const bool lo = bf16_to_f32((uint16_t)(y & 0xffffu)) > 0.f, hi = bf16_to_f32((uint16_t)(y >> 16)) > 0.f;
  return (lo ? (v & 0xffffu) : 0u) | (hi ? (v & 0xffff0000u) : 0u);
}

// 8 consecutive bf16 (row, k..k+7); zero outside rows x [0, kend).
template <bool VEC>
__device__ __forceinline__ uint4 load_chunk(const uint16_t* __restrict__ base, int64_t ld, int row, int rows, int k,
                                            int kend) {
  if (row >= rows || k >= kend) return make_uint4(0u, 0u, 0u, 0u);
  const uint16_t* p = base + (int64_t)row * ld + k;
  if (VEC && k + 8 <= kend) return *reinterpret_cast<const uint4*>(p);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (k + 2 * i < kend) ? (uint32_t)p[2 * i] : 0u;
    const uint32_t hi = (k + 2 * i + 1 < kend) ? (uint32_t)p[2 * i + 1] : 0u;
    w[i] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Fast path: 16-byte aligned operands with lda, ldw multiples of 8.
//
// Tiles move from global memory straight into LDS with global_load_lds_dwordx4
// (no register staging): each wave instruction fills one contiguous 1 KB
// block of LDS, i.e. 1 KB / (2 BK) rows of a BK-wide bf16 k-slice.  Inside a
// row the 16-byte chunks are XOR-swizzled with row bits so that the 16 lanes
// that one LDS cycle serves read distinct bank groups.  S LDS stages: the
// loads of k-tiles kt+1 .. kt+S-1 run during the MFMAs of k-tile kt; one
// barrier per k-tile.  Rows past M or N re-read the last row (their results
// are never stored); columns past K in the last k-tile are zeroed in LDS.
//
// Interleaving (ILV): with 1, the last MFMAs of each k-tile issue right
// after the barrier (their operands are already in registers) with the next
// tile's loads and first operand reads slotted between them, so the matrix
// cores do not idle while every wave issues its loads at once; with 2, the
// operand reads of every k-step also alternate with its MFMAs.
//
// The MFMA takes the W fragment as its first operand, so each accumulator
// block holds a 32 x 32 piece of C transposed: lane l owns row l % 32 of C
// and, for every group of four registers, four consecutive columns.  The
// epilogue therefore needs no LDS: bias, ReLU and bf16 rounding run in
// registers, one cross-half lane swap (v_permlane32_swap) gives each lane
// eight consecutive columns, and every store is 16 bytes.
//
// With PERSIST a grid of at most (resident workgroups per CU x CUs) walks
// the tiles, and the first k-tiles of the next tile load into LDS while the
// epilogue of the current tile runs; without it each workgroup takes one
// tile (measured 2-4% faster on the MLP shapes, so that is what the MLPs
// use).  Tiles are walked N-fastest; with a grid and tile count divisible by
// 8, each XCD (workgroup b runs on XCD b % 8) takes one contiguous range of
// tiles, so the tiles that share an A panel share one L2.
// Waves per SIMD the register budget allows: wave tiles of 128 x 128 keep
// 256 accumulators and run one wave per SIMD, smaller ones two.
constexpr int fast_waves_per_eu(int WM, int WN) { return WM * WN > 128 * 64 ? 1 : 2; }

template <int BM, int BN, int WM, int WN, typename OutT, bool PARTIAL, int BK, int S, bool PERSIST, int ILV,
          bool DELTA = false, bool KA = false, bool KW = false, bool DOT = false>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) __attribute__((amdgpu_waves_per_eu(fast_waves_per_eu(WM, WN)))) void gemm_bf16_fast_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ W, int64_t ldw,
    const float* __restrict__ bias, OutT* __restrict__ C, int64_t ldc, int M, int N, int K, int relu, int tiles_n,
    int tiles, int k_per_split, int vec_out, DeltaOut dout, DotOut dot) {
  static_assert(BK == 32 || BK == 64, "k-tile of 32 or 64");
  constexpr int RB = BK * 2;                      // bytes per tile row
  constexpr int CPR = BK / 8;                     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                   // rows per 1 KB load instruction
  constexpr int KS = BK / 16;                     // MFMA k-steps per tile
  constexpr int WAVES_N = BN / WN, NWAVES = (BM / WM) * WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_INS = BM * RB / 1024 / NWAVES, B_INS = BN * RB / 1024 / NWAVES, INS = A_INS + B_INS;
  constexpr int STAGE = (BM + BN) * RB;
  // DOT: the per-wave row sums of the single-output layer meet past the stages
  __shared__ __attribute__((aligned(1024))) char smem[S * STAGE + (DOT ? WAVES_N * BM * 4 : 0)];
  // chunk swizzle: the 16 lanes that one LDS cycle serves read 16 rows of
  // one logical chunk; XOR-ing the chunk with row bits above the rows that
  // share a bank group spreads them over all 64 banks
  auto swz = [](int row) { return CPR == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3); };
  // k-major operands (KA: A stored [K][M]; KW: W stored [K][N]).  A tile is
  // then BK rows of k, each BM (BN) values long, loaded as it lies in memory,
  // and the MFMA fragments (eight consecutive k of one row of C's operand)
  // come out of LDS through transposing reads: ds_read_b64_tr_b16 gives lane
  // j of each 16-lane group element j of the 16-wide segment that the group's
  // lanes address, from the four k-rows they point at (lane s: k-row s / 4,
  // elements 4 (s % 4) .. +3).  The 16-byte chunks of a k-row are
  // XOR-swizzled so that the four k-rows of one read fall on distinct banks.
  constexpr int CPKA = BM / 8, CPKW = BN / 8;       // 16-byte chunks per k-row
  constexpr int RPKA = 64 / CPKA, RPKW = 64 / CPKW;  // k-rows per 1 KB load instruction
  auto swzk = [](int krow, int cpk) { return cpk >= 16 ? 4 * (krow & 3) : (cpk == 8 ? 4 * ((krow >> 1) & 1) : 0); };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave - (wave / WAVES_N) * WAVES_N;
  const int kbeg = (int)blockIdx.z * k_per_split;
  const int kend = min(K, kbeg + k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int kpad = (kend + 7) & ~7;

  // this workgroup's tiles: first, first + stride, ... below end
  const int G = gridDim.x;
  int tile = blockIdx.x, stride = G, end = tiles;
  if ((tiles & 7) == 0 && (G & 7) == 0) {
    const int per = tiles >> 3, x = blockIdx.x & 7;
    tile = x * per + (blockIdx.x >> 3);
    stride = G >> 3;
    end = (x + 1) * per;
  }
  if (tile >= end) return;

  // this lane's DMA rows: instruction j of wave w fills rows (w*INS + j)*RPI + lane/CPR
  // (k-major: instruction j fills k-rows (w*INS + j)*RPK + lane/CPK, and
  // a_c / b_c is the column of the lane's chunk within the tile)
  const int lrow = lane / CPR, lpc = lane % CPR;
  int a_r[A_INS], b_r[B_INS], a_c[A_INS], b_c[B_INS];
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    if constexpr (KA) {
      a_r[j] = (wave * A_INS + j) * RPKA + lane / CPKA;
      a_c[j] = ((lane % CPKA) ^ swzk(a_r[j], CPKA)) * 8;
    } else {
      a_r[j] = (wave * A_INS + j) * RPI + lrow;
      a_c[j] = (lpc ^ swz(a_r[j])) * 8;
    }
  }
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    if constexpr (KW) {
      b_r[j] = (wave * B_INS + j) * RPKW + lane / CPKW;
      b_c[j] = ((lane % CPKW) ^ swzk(b_r[j], CPKW)) * 8;
    } else {
      b_r[j] = (wave * B_INS + j) * RPI + lrow;
      b_c[j] = (lpc ^ swz(b_r[j])) * 8;
    }
  }
  // k-major: columns past M (N) read the last whole chunk of the row (their
  // results are never stored); k-rows past the end re-read the last one and
  // are zeroed in LDS
  const int mlast = ((M + 7) & ~7) - 8, nlast = ((N + 7) & ~7) - 8;
  const uint16_t* a_row[A_INS];
  const uint16_t* b_row[B_INS];
  auto rows_of = [&](int t, const uint16_t** ar, const uint16_t** br) {
    const int tm = t / tiles_n, tn = t - (t / tiles_n) * tiles_n;
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
      if constexpr (KA) ar[j] = A + min(tm * BM + a_c[j], mlast);
      else ar[j] = A + (int64_t)min(tm * BM + a_r[j], M - 1) * lda;
    }
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      if constexpr (KW) br[j] = W + min(tn * BN + b_c[j], nlast);
      else br[j] = W + (int64_t)min(tn * BN + b_r[j], N - 1) * ldw;
    }
  };
  auto a_src = [&](int k0, int j) -> const uint16_t* {
    if constexpr (KA) return a_row[j] + (int64_t)min(k0 + a_r[j], kend - 1) * lda;
    else return a_row[j] + min(k0 + a_c[j], kpad - 8);
  };
  auto b_src = [&](int k0, int j) -> const uint16_t* {
    if constexpr (KW) return b_row[j] + (int64_t)min(k0 + b_r[j], kend - 1) * ldw;
    else return b_row[j] + min(k0 + b_c[j], kpad - 8);
  };
  auto issue = [&](int kt) {
    char* st = smem + (kt % S) * STAGE;
    const int k0 = kbeg + kt * BK;
#pragma unroll
    for (int j = 0; j < A_INS; ++j) lds_dma16_opaque(a_src(k0, j), st + (wave * A_INS + j) * 1024);
#pragma unroll
    for (int j = 0; j < B_INS; ++j) lds_dma16_opaque(b_src(k0, j), st + BM * RB + (wave * B_INS + j) * 1024);
  };

  f32x16 acc[TM][TN];
  const int r32 = lane & 31, half = lane >> 5;
  bf16x8 fa[2][TM], fb[2][TN];
  // zero columns [valid, BK) of every A and W row of a partial last k-tile
  auto zero_tail = [&](int kt) {
    const int valid = kend - (kbeg + kt * BK);
    if (valid >= BK) return;
    char* wst = smem + (kt % S) * STAGE;
    // k-major operand: whole k-rows valid .. BK-1; otherwise columns
    // valid .. BK-1 of every row
    auto zero_rows = [&](char* base, int width) {
      for (int e = valid * width / 8 + tid; e < BK * width / 8; e += NWAVES * 64)
        reinterpret_cast<uint4*>(base)[e] = make_uint4(0u, 0u, 0u, 0u);
    };
    auto zero_cols = [&](char* base, int rows) {
      for (int e = tid; e < rows * CPR; e += NWAVES * 64) {
        const int row = e / CPR, c = e % CPR;
        if (c * 8 + 8 > valid) {
          uint16_t* p = reinterpret_cast<uint16_t*>(base + row * RB + ((c ^ swz(row)) * 16));
#pragma unroll
          for (int x = 0; x < 8; ++x)
            if (c * 8 + x >= valid) p[x] = 0;
        }
      }
    };
    if constexpr (KA) zero_rows(wst, BM);
    else zero_cols(wst, BM);
    if constexpr (KW) zero_rows(wst + BM * RB, BN);
    else zero_cols(wst + BM * RB, BN);
    __syncthreads();
  };
  // MFMA operands of k-step ks of the tile in stage st, double-buffered in
  // registers: the reads of step ks+1 are in flight during the MFMAs of ks
  // fragment of rows mb .. mb+31 of a k-major operand (width values per
  // k-row), k-step ks: two transposing reads of four k-rows each
  auto frag_tr = [&](const char* base, int width, int cpk, int ks, int mb) -> bf16x8 {
    const int grp = lane >> 4, sl = lane & 15;
    const int m = mb + 16 * (grp & 1) + 4 * (sl & 3);
    const int kr = ks * 16 + 8 * (grp >> 1) + (sl >> 2);
    typedef short v4s __attribute__((ext_vector_type(4)));
    v4s v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int krow = kr + 4 * h;
      const int off = krow * width * 2 + (((m >> 3) ^ swzk(krow, cpk)) * 16) + (m & 7) * 2;
      v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)((__attribute__((address_space(3))) char*)base + off));
    }
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s r = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
  };
  auto frag_a = [&](const char* st, int ks, int i) -> bf16x8 {
    if constexpr (KA) {
      return frag_tr(st, BM, CPKA, ks, wm * WM + i * 32);
    } else {
      const int c = 2 * ks + half, row = wm * WM + i * 32 + r32;
      return *reinterpret_cast<const bf16x8*>(st + row * RB + ((c ^ swz(row)) * 16));
    }
  };
  auto frag_w = [&](const char* st, int ks, int j) -> bf16x8 {
    if constexpr (KW) {
      return frag_tr(st + BM * RB, BN, CPKW, ks, wn * WN + j * 32);
    } else {
      const int c = 2 * ks + half, row = wn * WN + j * 32 + r32;
      return *reinterpret_cast<const bf16x8*>(st + BM * RB + row * RB + ((c ^ swz(row)) * 16));
    }
  };
  auto load_frags = [&](const char* st, int ks, int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[buf][i] = frag_a(st, ks, i);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[buf][j] = frag_w(st, ks, j);
  };
  auto issue_one = [&](int kt, int j) {
    char* st = smem + (kt % S) * STAGE;
    const int k0 = kbeg + kt * BK;
    if (j < A_INS)
      lds_dma16_opaque(a_src(k0, j), st + (wave * A_INS + j) * 1024);
    else
      lds_dma16_opaque(b_src(k0, j - A_INS), st + BM * RB + (wave * B_INS + j - A_INS) * 1024);
  };
  auto load_one = [&](const char* st, int ks, int buf, int f) {
    if (f < TM) fa[buf][f] = frag_a(st, ks, f);
    else fb[buf][f - TM] = frag_w(st, ks, f - TM);
  };
  auto mfma_one = [&](int buf, int q) {
    const int i = q / TN, j = q % TN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };
  // Pipeline: tiles kt .. kt+S-1 sit in the S LDS stages (tile t in stage
  // t % S).  At the last k-step of tile kt every wave has read its operands
  // of stage kt % S, so after one barrier (which also sees tile kt+1 landed)
  // the loads of tile kt+S go into that stage and the first operands of tile
  // kt+1 are read before the last MFMAs of tile kt run.  Waits count this
  // wave's vector-memory operations, which complete in issue order; the
  // epilogue stores of the previous tile, issued after this tile's first
  // loads, only make the first waits of a tile wait a little longer.
  auto wait_tiles = [&](int younger) {  // at most `younger` tiles' loads still in flight
    if constexpr (S >= 4) {
      if (younger >= 3) { wait_vmcnt<3 * INS>(); return; }
    }
    if constexpr (S >= 3) {
      if (younger >= 2) { wait_vmcnt<2 * INS>(); return; }
    }
    if (younger >= 1) { wait_vmcnt<INS>(); return; }
    wait_vmcnt<0>();
  };
  // k-steps 0..KS-2 of the tile in stage st: read the next step's operands,
  // then this step's MFMAs (the scheduling barriers keep that order)
  constexpr int NQ = TM * TN, NF = TM + TN;
  auto first_steps = [&](const char* st) {
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      if constexpr (ILV >= 2) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
          for (int f2 = 0; f2 < (NF + NQ - 1) / NQ; ++f2) {
            const int f = q * NF / NQ + f2;
            if (f < (q + 1) * NF / NQ) load_one(st, ks + 1, (ks + 1) & 1, f);
          }
          __builtin_amdgcn_sched_barrier(0);
          mfma_one(ks & 1, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        load_frags(st, ks + 1, (ks + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(ks & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  constexpr int LAST = (KS - 1) & 1;  // register buffer of the last k-step
  // hand-over from tile kt to tile kt+1 (see above), then the last MFMAs of kt
  auto turn = [&](int kt, bool load_next, bool zero_next, int younger, bool ilv) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of stage kt % S are done
    wait_tiles(younger);                  // tile kt+1 has landed (this wave's share)
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (ILV >= 1 && ilv) {
      // the last MFMAs of tile kt go first (their operands are in registers);
      // the next tile's loads and first operand reads slot in between them
      constexpr int NOPS = INS + NF;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        mfma_one(LAST, q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int o2 = 0; o2 < (NOPS + NQ - 1) / NQ; ++o2) {
          const int o = q * NOPS / NQ + o2;
          if (o >= (q + 1) * NOPS / NQ) continue;
          if (o < INS) {
            if (load_next) issue_one(kt + S, o);
          } else {
            load_one(smem + ((kt + 1) % S) * STAGE, 0, (LAST + 1) & 1, o - INS);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    if (load_next) issue(kt + S);
    if (zero_next) zero_tail(kt + 1);
    load_frags(smem + ((kt + 1) % S) * STAGE, 0, (LAST + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(LAST);
    __builtin_amdgcn_sched_barrier(0);
  };
  // the steady state has no branch, so every wait is an exact count; the
  // epilogue's kernel arguments are read here so that no scalar load is
  // pending in the loop (that would turn every LDS wait into lgkmcnt(0))
  __asm__ volatile("" : "+s"(bias), "+s"(C), "+s"(ldc), "+s"(vec_out), "+s"(relu));
  const int pre = nk < S ? nk : S;
  rows_of(tile, a_row, b_row);
#pragma unroll
  for (int t = 0; t < S; ++t)
    if (t < nk) issue(t);

  while (true) {
    const int m0 = (tile / tiles_n) * BM, n0 = (tile - (tile / tiles_n) * tiles_n) * BN;
    // Block (tm, tn) of the accumulators: lane l holds C row
    // m0 + wm*WM + tm*32 + l%32 and, in register v, column
    // n0 + wn*WN + tn*32 + 8*(v/4) + 4*(l/32) + v%4.  The accumulators start
    // from the bias (zero for partial sums), so the MFMAs add the products to it.
    const int rowb = m0 + wm * WM + r32, colb = n0 + wn * WN + 4 * half;
    const bool with_bias = !PARTIAL && bias != nullptr;
    if (with_bias && n0 + (wn + 1) * WN <= N) {  // this wave's columns all exist
      const float* bp = bias + colb;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float b0 = bp[j * 32 + 8 * (v >> 2) + (v & 3)];
#pragma unroll
          for (int i = 0; i < TM; ++i) acc[i][j][v] = b0;
        }
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int col = colb + j * 32 + 8 * (v >> 2) + (v & 3);
          const float b0 = (with_bias && col < N) ? bias[col] : 0.f;
#pragma unroll
          for (int i = 0; i < TM; ++i) acc[i][j][v] = b0;
        }
    }
    if (nk > 0) {
      wait_tiles(pre - 1);
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      if (nk == 1) zero_tail(0);
      load_frags(smem, 0, 0);
    }
    int kt = 0;
    for (; kt + S < nk; ++kt) {
      first_steps(smem + (kt % S) * STAGE);
      turn(kt, true, false, S - 2, true);
    }
#pragma unroll
    for (int r = 0; r < S - 1; ++r) {  // at most S - 1 tiles remain after the steady state
      if (kt + 1 < nk) {
        first_steps(smem + (kt % S) * STAGE);
        const int younger = nk - 2 - kt;
        turn(kt, false, kt + 2 == nk, younger < S - 2 ? younger : S - 2, false);
        ++kt;
      }
    }
    if (kt < nk) {
      first_steps(smem + (kt % S) * STAGE);
      mfmas(LAST);
    }

    const int next = PERSIST ? tile + stride : end;
    if (next < end) {
      // every wave's LDS reads of this tile are done: the next tile's first
      // k-tiles load while this tile's epilogue runs
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      rows_of(next, a_row, b_row);
#pragma unroll
      for (int t = 0; t < S; ++t)
        if (t < nk) issue(t);
    }

    const bool full = m0 + BM <= M && n0 + BN <= N && vec_out;
    if constexpr (DOT) {
      // Single-output layer on this tile's rows (the tile spans every column):
      // each lane sums its columns' bf16 hidden values times w, columns in
      // (tn, register) order; the two lanes of a row add their sums, then the
      // waves that split the columns meet in LDS and are added in wave order.
      static_assert(!PARTIAL && !DELTA && sizeof(OutT) == 2, "DOT: bf16 hidden layer");
      float* red = reinterpret_cast<float*>(smem + S * STAGE);  // [WAVES_N][BM]
      float part[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) part[tm] = 0.f;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col0 = colb + tn * 32 + 8 * g;
          float wv[4];
          if (col0 + 4 <= N) {
            const uint2 w4 = *reinterpret_cast<const uint2*>(dot.w + col0);
            wv[0] = bf16_to_f32((uint16_t)(w4.x & 0xffffu)), wv[1] = bf16_to_f32((uint16_t)(w4.x >> 16));
            wv[2] = bf16_to_f32((uint16_t)(w4.y & 0xffffu)), wv[3] = bf16_to_f32((uint16_t)(w4.y >> 16));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) wv[q] = col0 + q < N ? bf16_to_f32(dot.w[col0 + q]) : 0.f;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
              float h = acc[tm][tn][4 * g + q];
              if (relu) h = relu_f(h);
              part[tm] = __builtin_fmaf(bf16_to_f32(f32_to_bf16(h)), wv[q], part[tm]);
            }
        }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        part[tm] = part[tm] + __shfl_xor(part[tm], 32);
        if (half == 0) red[wn * BM + wm * WM + tm * 32 + r32] = part[tm];
      }
      __syncthreads();
      if (tid < BM && m0 + tid < M) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES_N; ++w) v = v + red[w * BM + tid];
        if (dot.b) v = v + dot.b[0];
        if (dot.relu) v = relu_f(v);
        dot.out[(int64_t)(m0 + tid) * dot.ldo] = v;
        if (dot.prob) dot.prob[m0 + tid] = 1.f / (1.f + expf(-v));
      }
      if (C == nullptr) goto tile_done;
    }
    if constexpr (DELTA) {
      // Input gradient of a ReLU layer: g = this tile, masked by the layer
      // input y > 0, rounded to bf16 and written row-major to C; the tile then
      // goes through LDS column-major (the stages are free: every wave is past
      // its last operand read) and leaves transposed into dT, each thread
      // summing eight rows of one column for the bias-gradient partials.
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      uint16_t* lt = reinterpret_cast<uint16_t*>(smem);  // [BN][BM]
      const bool yvec = (dout.ldy % 8) == 0 && (reinterpret_cast<uintptr_t>(dout.y) & 15u) == 0;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          uint32_t pk[4][2];
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h) pk[g][h] = pack_bf16x2(acc[tm][tn][4 * g + 2 * h], acc[tm][tn][4 * g + 2 * h + 1]);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const auto s01 = __builtin_amdgcn_permlane32_swap(pk[0][h], pk[1][h], false, false);
            const auto s23 = __builtin_amdgcn_permlane32_swap(pk[2][h], pk[3][h], false, false);
            pk[0][h] = s01[0];
            pk[1][h] = s01[1];
            pk[2][h] = s23[0];
            pk[3][h] = s23[1];
          }
          // this lane: tile row rl, columns c0 .. c0+7 (lo) and c0+16 .. c0+23 (hi)
          const int rl = wm * WM + tm * 32 + r32, i = m0 + rl;
          const int c0 = wn * WN + tn * 32 + 8 * half;
          uint32_t v[2][4] = {{pk[0][0], pk[0][1], pk[1][0], pk[1][1]}, {pk[2][0], pk[2][1], pk[3][0], pk[3][1]}};
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int j = n0 + c0 + 16 * p;
            uint32_t y[4] = {0u, 0u, 0u, 0u};  // columns past N or rows past M: masked to zero
            if (i < M) {
              const uint16_t* yr = dout.y + (int64_t)i * dout.ldy + j;
              if (yvec && j + 8 <= N) {
                const uint4 yv = *reinterpret_cast<const uint4*>(yr);
                y[0] = yv.x, y[1] = yv.y, y[2] = yv.z, y[3] = yv.w;
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                  if (j + e < N) y[e >> 1] |= (uint32_t)yr[e] << (16 * (e & 1));
              }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) v[p][q] = mask_pair(v[p][q], y[q]);
            if (i < M) {
              uint16_t* cr = reinterpret_cast<uint16_t*>(C) + (int64_t)i * ldc + j;
              if (vec_out && j + 8 <= N) {
                *reinterpret_cast<uint4*>(cr) = make_uint4(v[p][0], v[p][1], v[p][2], v[p][3]);
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                  if (j + e < N) cr[e] = (uint16_t)(v[p][e >> 1] >> (16 * (e & 1)));
              }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) lt[(c0 + 16 * p + e) * BM + rl] = (uint16_t)(v[p][e >> 1] >> (16 * (e & 1)));
          }
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      // transposed rows: item (column jl, row group q), q fastest, so that
      // BM / 8 consecutive lanes write one column's BM rows contiguously
      constexpr int QG = BM / 8, NT = NWAVES * 64;
      const bool tvec = (dout.ldt % 8) == 0 && (reinterpret_cast<uintptr_t>(dout.dT) & 15u) == 0;
#pragma unroll
      for (int it = 0; it < BN * QG / NT; ++it) {
        const int item = it * NT + tid;
        const int q = item % QG, jl = item / QG;
        const uint4 w4 = *reinterpret_cast<const uint4*>(lt + jl * BM + 8 * q);
        const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum = sum + bf16_to_f32((uint16_t)(w[e >> 1] >> (16 * (e & 1))));
#pragma unroll
        for (int o = 1; o < QG; o <<= 1) sum = sum + __shfl_xor(sum, o, QG);
        const int j = n0 + jl, i0 = m0 + 8 * q;
        if (j < N) {
          if (q == 0) dout.dbp[(int64_t)(m0 / BM) * N + j] = sum;
          uint16_t* tr = dout.dT + (int64_t)j * dout.ldt + i0;
          if (!dout.dT) {
          } else if (tvec && i0 + 8 <= M) {
            *reinterpret_cast<uint4*>(tr) = w4;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (i0 + e < M) tr[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
      goto tile_done;
    }
    if constexpr (sizeof(OutT) == 2 && !PARTIAL) {
      if (full) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int tm = 0; tm < TM; ++tm) {
            uint32_t pk[4][2];
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                float v0 = acc[tm][tn][4 * g + 2 * h];
                float v1 = acc[tm][tn][4 * g + 2 * h + 1];
                if (relu) {
                  v0 = relu_f(v0);
                  v1 = relu_f(v1);
                }
                pk[g][h] = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
              }
            // lanes 0-31 gather columns 0-7 and 16-23 of the block, lanes 32-63 columns 8-15 and 24-31
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const auto s01 = __builtin_amdgcn_permlane32_swap(pk[0][h], pk[1][h], false, false);
              const auto s23 = __builtin_amdgcn_permlane32_swap(pk[2][h], pk[3][h], false, false);
              pk[0][h] = s01[0];
              pk[1][h] = s01[1];
              pk[2][h] = s23[0];
              pk[3][h] = s23[1];
            }
            uint16_t* c = reinterpret_cast<uint16_t*>(C) + (int64_t)(rowb + tm * 32) * ldc + n0 + wn * WN + tn * 32 +
                          8 * half;
            *reinterpret_cast<uint4*>(c) = make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]);
            *reinterpret_cast<uint4*>(c + 16) = make_uint4(pk[2][0], pk[2][1], pk[3][0], pk[3][1]);
          }
        goto tile_done;
      }
    }
    if constexpr (sizeof(OutT) == 4) {
      if (full) {  // four consecutive fp32 columns per register group: 16-byte stores
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int j = colb + tn * 32 + 8 * g;
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
              float o[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                o[q] = acc[tm][tn][4 * g + q];
                if (!PARTIAL && relu) o[q] = relu_f(o[q]);
              }
              const int64_t i = rowb + tm * 32;
              float* dst = reinterpret_cast<float*>(C) + (PARTIAL ? ((int64_t)blockIdx.z * M + i) : i) * ldc + j;
              *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            }
          }
        goto tile_done;
      }
    }
    // edge tiles and unaligned outputs: element stores
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = colb + tn * 32 + 8 * (v >> 2) + (v & 3);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int i = rowb + tm * 32;
          if (i < M && j < N) {
            float val = acc[tm][tn][v];
            if (PARTIAL) {
              C[((int64_t)blockIdx.z * M + i) * ldc + j] = val;
            } else {
              if (relu) val = relu_f(val);
              store_out(&C[(int64_t)i * ldc + j], val);
            }
          }
        }
      }
  tile_done:
    if (next >= end) break;
    tile = next;
  }
}

// Resident workgroups per CU of one fast-kernel instance (queried once per
// device).
template <typename Kern>
int fast_occupancy(Kern kern, int threads) {
  static int cached[kMaxDevices] = {0};
  const int dev = current_device();
  if (cached[dev] == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kern, threads, 0) != hipSuccess || v < 1) v = 1;
    cached[dev] = v;
  }
  return cached[dev];
}

template <int BM, int BN, int WM, int WN, typename OutT, bool PARTIAL, int BK = 64, int S = 2, bool PERSIST = false,
          int ILV = 0, bool DELTA = false, bool KA = false, bool KW = false, bool DOT = false>
void launch_fast(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, const float* bias, OutT* C,
                 int64_t ldc, int M, int N, int K, int relu, int splits, int k_per_split, hipStream_t s,
                 DeltaOut dout = DeltaOut{}, DotOut dot = DotOut{}) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int tiles = tm * tn;
  constexpr int threads = (BM / WM) * (BN / WN) * 64;
  auto kern = gemm_bf16_fast_kernel<BM, BN, WM, WN, OutT, PARTIAL, BK, S, PERSIST, ILV, DELTA, KA, KW, DOT>;
  int grid = tiles;
  if constexpr (PERSIST) {
    const int slots = fast_occupancy(kern, threads) * device_cu_count();
    grid = slots / (splits > 0 ? splits : 1);
    if (grid > 8) grid &= ~7;  // a multiple of 8 keeps the per-XCD tile ranges
    grid = grid < 1 ? 1 : (grid < tiles ? grid : tiles);
  }
  constexpr int VW = 16 / (int)sizeof(OutT);
  const int vec_out = (ldc % VW) == 0 && (reinterpret_cast<uintptr_t>(C) & 15u) == 0;
  hipLaunchKernelGGL(kern, dim3(grid, 1, splits), dim3(threads), 0, s, A, lda, W, ldw, bias, C, ldc, M, N, K, relu,
                     tn, tiles, k_per_split, vec_out, dout, dot);
}

// Tile choice: the largest block tile that still gives every CU a tile
// (256 x 128 only where it gives each CU two, or one with a k loop of at
// least 2048: 5120 -> 512 at batch 16384 84.6 -> 82.1 us; with exactly one
// and a shorter k loop, 128 x 128 measured as fast or faster).  Deep k (a multiple of 64, at least 512) runs
// 64-wide k-tiles in two stages, fewer barriers; shallower or ragged k
// 32-wide k-tiles in four stages.  Every choice interleaves the operand reads with the
// MFMAs (measured 3-10% faster than reads first on every MLP shape).
template <typename OutT, bool PARTIAL>
void pick_fast(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, const float* bias, OutT* C,
               int64_t ldc, int M, int N, int K, int relu, int splits, int k_per_split, hipStream_t s) {
  const int64_t t256x256 = ceil_div(M, 256) * ceil_div(N, 256) * splits;
  const int64_t t256x128 = ceil_div(M, 256) * ceil_div(N, 128) * splits;
  // a partial last k-tile (K not a multiple of 64, e.g. 479) measured faster in 32-wide tiles
  const bool deep = k_per_split >= 512 && (k_per_split % 64) == 0 && (K % 64) == 0;
  if (t256x256 >= 256 && deep)
    launch_fast<256, 256, 128, 64, OutT, PARTIAL, 64, 2, false, 2>(A, lda, W, ldw, bias, C, ldc, M, N, K, relu, splits,
                                                                   k_per_split, s);
  else if (t256x256 >= 256)
    launch_fast<256, 256, 128, 64, OutT, PARTIAL, 32, 4, false, 1>(A, lda, W, ldw, bias, C, ldc, M, N, K, relu, splits,
                                                                   k_per_split, s);
  else if (t256x128 >= 512 || (t256x128 >= 256 && deep && k_per_split >= 2048))
    launch_fast<256, 128, 64, 64, OutT, PARTIAL, 64, 2, false, 2>(A, lda, W, ldw, bias, C, ldc, M, N, K, relu, splits,
                                                                  k_per_split, s);
  else
    launch_fast<128, 128, 64, 64, OutT, PARTIAL, 64, 2, false, 2>(A, lda, W, ldw, bias, C, ldc, M, N, K, relu, splits,
                                                                  k_per_split, s);
}

template <int BM, int BN, bool VEC, typename OutT, bool PARTIAL>
__global__ __launch_bounds__(256) void gemm_bf16_generic_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                        const uint16_t* __restrict__ W, int64_t ldw,
                                                        const float* __restrict__ bias, OutT* __restrict__ C,
                                                        int64_t ldc, int M, int N, int K, int relu, int tiles_n,
                                                        int k_per_split) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int AP = BM / 64, BP = BN / 64;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int bid = blockIdx.x;
  const int total = gridDim.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int tile_m = bid / tiles_n, tile_n = bid - tile_m * tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int kbeg = (int)blockIdx.z * k_per_split;
  const int kend = min(K, kbeg + k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  const int lr = tid >> 2, lc = (tid & 3) * 8;
  uint4 ga[AP], gb[BP];
  auto gload = [&](int kt) {
    const int k = kbeg + kt * BK + lc;
#pragma unroll
    for (int i = 0; i < AP; ++i) ga[i] = load_chunk<VEC>(A, lda, m0 + i * 64 + lr, M, k, kend);
#pragma unroll
    for (int i = 0; i < BP; ++i) gb[i] = load_chunk<VEC>(W, ldw, n0 + i * 64 + lr, N, k, kend);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AP; ++i) *reinterpret_cast<uint4*>(&As[buf][(i * 64 + lr) * LDS_STRIDE + lc]) = ga[i];
#pragma unroll
    for (int i = 0; i < BP; ++i) *reinterpret_cast<uint4*>(&Bs[buf][(i * 64 + lr) * LDS_STRIDE + lc]) = gb[i];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kof = ks * 16 + (lane >> 5) * 8;
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * WM + i * 32 + (lane & 31)) * LDS_STRIDE + kof]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn * WN + j * 32 + (lane & 31)) * LDS_STRIDE + kof]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // D layout of a 32x32 block: lane l holds column l % 32 and rows
  // 8*(v/4) + 4*(l/32) + v%4, v = 0..15.
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int j = n0 + wn * WN + tn * 32 + (lane & 31);
    const float bj = (!PARTIAL && bias != nullptr && j < N) ? bias[j] : 0.f;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = m0 + wm * WM + tm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (i < M && j < N) {
          float val = acc[tm][tn][v];
          if (PARTIAL) {
            C[((int64_t)blockIdx.z * M + i) * ldc + j] = val;
          } else {
            val = val + bj;
            if (relu) val = relu_f(val);
            store_out(&C[(int64_t)i * ldc + j], val);
          }
        }
      }
    }
  }
}


// Any layout (unaligned rows or odd leading dimensions): element-wise loads.
template <typename OutT, bool PARTIAL>
void launch_generic(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, const float* bias, OutT* C,
                    int64_t ldc, int M, int N, int K, int relu, int splits, int k_per_split, hipStream_t s) {
  const int tm = (M + 127) / 128, tn = (N + 127) / 128;
  hipLaunchKernelGGL((gemm_bf16_generic_kernel<128, 128, false, OutT, PARTIAL>), dim3(tm * tn, 1, splits), dim3(256),
                     0, s, A, lda, W, ldw, bias, C, ldc, M, N, K, relu, tn, k_per_split);
}

// ---------------------------------------------------------------- GEMV (N == 1)

__global__ __launch_bounds__(256) void gemv_bf16_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                        const uint16_t* __restrict__ w,
                                                        const float* __restrict__ bias, float* __restrict__ out,
                                                        int64_t ldo, float* __restrict__ prob, int M, int K,
                                                        int relu, int vec) {
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float acc = 0.f;
  if (row < M) {
    const uint16_t* a = A + (int64_t)row * lda;
    for (int k = sub * 8; k < K; k += 128) {
      if (vec && k + 8 <= K) {
        const uint4 av = *reinterpret_cast<const uint4*>(a + k);
        const uint4 wv = *reinterpret_cast<const uint4*>(w + k);
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = __builtin_fmaf(bf16_to_f32((uint16_t)(aw[i] & 0xffffu)), bf16_to_f32((uint16_t)(ww[i] & 0xffffu)), acc);
          acc = __builtin_fmaf(bf16_to_f32((uint16_t)(aw[i] >> 16)), bf16_to_f32((uint16_t)(ww[i] >> 16)), acc);
        }
      } else {
        for (int i = 0; i < 8 && k + i < K; ++i) acc = __builtin_fmaf(bf16_to_f32(a[k + i]), bf16_to_f32(w[k + i]), acc);
      }
    }
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) acc = acc + __shfl_xor(acc, o, 16);
  if (sub == 0 && row < M) {
    float v = acc + (bias ? bias[0] : 0.f);
    if (relu) v = relu_f(v);
    out[(int64_t)row * ldo] = v;
    if (prob) prob[row] = 1.f / (1.f + expf(-v));
  }
}

// ---------------------------------------------------------------- fp32 network

__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ W, int64_t ldw,
                                                       const float* __restrict__ bias, float* __restrict__ C,
                                                       int64_t ldc, float* __restrict__ prob, int M, int N, int K,
                                                       int relu) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)M * N) return;
  const int m = (int)(t / N), n = (int)(t - (int64_t)(t / N) * N);
  const float* a = A + (int64_t)m * lda;
  const float* w = W + (int64_t)n * ldw;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = __builtin_fmaf(a[k], w[k], acc);
  float v = acc + bias[n];
  if (relu) v = relu_f(v);
  C[(int64_t)m * ldc + n] = v;
  if (prob && N == 1) prob[m] = 1.f / (1.f + expf(-v));
}

// ---------------------------------------------------------------- helpers

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in, int64_t ldi,
                                                             uint16_t* __restrict__ out, int64_t ldo, int R,
                                                             int C) {
  __shared__ uint16_t tile[64][66];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? in[(int64_t)r * ldi + c] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < R) out[(int64_t)c * ldo + r] = tile[tx][i];
  }
}

// 64 x 64 tile, 16-byte loads and stores (rows of in and out 16-byte aligned).
__global__ __launch_bounds__(256) void transpose_bf16_v8_kernel(const uint16_t* __restrict__ in, int64_t ldi,
                                                                uint16_t* __restrict__ out, int64_t ldo, int R,
                                                                int C) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int t = threadIdx.x, row = t >> 3, grp = t & 7;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = row + 32 * h, r = r0 + i, c = c0 + 8 * grp;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < R) {
      if (c + 8 <= C) {
        v = *reinterpret_cast<const uint4*>(in + (int64_t)r * ldi + c);
      } else if (c < C) {
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = (c + q < C) ? in[(int64_t)r * ldi + c + q] : (uint16_t)0;
        v = make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16), e[4] | ((uint32_t)e[5] << 16),
                       e[6] | ((uint32_t)e[7] << 16));
      }
    }
    *reinterpret_cast<uint4*>(&tile[i][8 * grp]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = row + 32 * h, c = c0 + i, r = r0 + 8 * grp;  // out row c, elements r .. r+7
    if (c >= C || r >= R) continue;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = (uint32_t)tile[8 * grp + 2 * q][i] | ((uint32_t)tile[8 * grp + 2 * q + 1][i] << 16);
    if (r + 8 <= R) {
      *reinterpret_cast<uint4*>(out + (int64_t)c * ldo + r) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (r + q < R) out[(int64_t)c * ldo + r + q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
    }
  }
}

__global__ __launch_bounds__(256) void convert_bf16_kernel(const float* __restrict__ in, int64_t ldi,
                                                           uint16_t* __restrict__ out, int64_t ldo, int R, int C,
                                                           int Cpad) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)R * Cpad) return;
  const int r = (int)(t / Cpad), c = (int)(t - (int64_t)r * Cpad);
  out[(int64_t)r * ldo + c] = c < C ? f32_to_bf16(in[(int64_t)r * ldi + c]) : (uint16_t)0;
}

}  // namespace

int gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, const float* bias, void* C,
              int64_t ldc, bool out_bf16, int M, int N, int K, bool relu, hipStream_t s) {
  if (M <= 0 || N <= 0) return DLRM_OK;
  const bool fast = aligned16(A) && aligned16(W) && (lda % 8) == 0 && (ldw % 8) == 0 && lda >= K && ldw >= K &&
                    (int64_t)256 * lda < ((int64_t)1 << 31) && (int64_t)256 * ldw < ((int64_t)1 << 31);
  const int kps = (int)round_up(K > 0 ? K : 1, 64);
  if (out_bf16) {
    auto* c = static_cast<uint16_t*>(C);
    if (fast) pick_fast<uint16_t, false>(A, lda, W, ldw, bias, c, ldc, M, N, K, relu, 1, kps, s);
    else launch_generic<uint16_t, false>(A, lda, W, ldw, bias, c, ldc, M, N, K, relu, 1, kps, s);
  } else {
    auto* c = static_cast<float*>(C);
    if (fast) pick_fast<float, false>(A, lda, W, ldw, bias, c, ldc, M, N, K, relu, 1, kps, s);
    else launch_generic<float, false>(A, lda, W, ldw, bias, c, ldc, M, N, K, relu, 1, kps, s);
  }
  return launch_status();
}

namespace {
// The fast kernel's operand conditions: 16-byte aligned rows whose pitch is
// a multiple of 8 values and holds a whole row (K values, or M / N values
// for a k-major operand).
bool fast_operand(const uint16_t* p, int64_t ld, int64_t need) {
  return aligned16(p) && (ld % 8) == 0 && ld >= need && (int64_t)256 * ld < ((int64_t)1 << 31);
}
}  // namespace

int gemm_bf16_ex(const uint16_t* A, int64_t lda, bool a_kmajor, const uint16_t* W, int64_t ldw, bool w_kmajor,
                 void* C, int64_t ldc, bool out_bf16, int M, int N, int K, hipStream_t s) {
  if (!a_kmajor && !w_kmajor) return gemm_bf16(A, lda, W, ldw, nullptr, C, ldc, out_bf16, M, N, K, false, s);
  if (M <= 0 || N <= 0) return DLRM_OK;
  if (a_kmajor || out_bf16 || !fast_operand(A, lda, K) || !fast_operand(W, ldw, N)) return DLRM_E_UNSUPPORTED;
  const int kps = (int)round_up(K > 0 ? K : 1, 64);
  launch_fast<128, 128, 64, 64, float, false, 64, 2, false, 2, false, false, true>(
      A, lda, W, ldw, nullptr, static_cast<float*>(C), ldc, M, N, K, 0, 1, kps, s);
  return launch_status();
}

int gemm_bf16_delta(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, bool w_kmajor, int M, int N,
                    int K, uint16_t* dlt, int64_t ldd, const DeltaOut& dout, int* tile_rows, hipStream_t s) {
  if (M <= 0 || N <= 0) return DLRM_OK;
  if (!fast_operand(A, lda, K) || !fast_operand(W, ldw, w_kmajor ? N : K)) return DLRM_E_UNSUPPORTED;
  const int kps = (int)round_up(K > 0 ? K : 1, 64);
  // the largest block tile that still gives every CU a tile (as pick_fast)
  const bool big = ceil_div(M, 256) * ceil_div(N, 256) >= 256, deep = (K % 64) == 0 && K >= 512;
  *tile_rows = big ? 256 : 128;
  if (w_kmajor) {
    if (big && deep)
      launch_fast<256, 256, 128, 64, uint16_t, false, 64, 2, false, 2, true, false, true>(
          A, lda, W, ldw, nullptr, dlt, ldd, M, N, K, 0, 1, kps, s, dout);
    else if (big)
      launch_fast<256, 256, 128, 64, uint16_t, false, 32, 4, false, 1, true, false, true>(
          A, lda, W, ldw, nullptr, dlt, ldd, M, N, K, 0, 1, kps, s, dout);
    else
      launch_fast<128, 128, 64, 64, uint16_t, false, 64, 2, false, 2, true, false, true>(
          A, lda, W, ldw, nullptr, dlt, ldd, M, N, K, 0, 1, kps, s, dout);
  } else {
    if (big && deep)
      launch_fast<256, 256, 128, 64, uint16_t, false, 64, 2, false, 2, true>(A, lda, W, ldw, nullptr, dlt, ldd, M, N, K,
                                                                            0, 1, kps, s, dout);
    else if (big)
      launch_fast<256, 256, 128, 64, uint16_t, false, 32, 4, false, 1, true>(A, lda, W, ldw, nullptr, dlt, ldd, M, N, K,
                                                                            0, 1, kps, s, dout);
    else
      launch_fast<128, 128, 64, 64, uint16_t, false, 64, 2, false, 2, true>(A, lda, W, ldw, nullptr, dlt, ldd, M, N, K,
                                                                           0, 1, kps, s, dout);
  }
  return launch_status();
}

int gemm_bf16_dot(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, const float* bias, uint16_t* H,
                  int64_t ldh, int M, int N, int K, const DotOut& dot, hipStream_t s) {
  if (M <= 0) return DLRM_OK;
  if (N < 1 || N > 256 || K < 1 || !dot.w || !dot.out || (reinterpret_cast<uintptr_t>(dot.w) & 7u) ||
      !fast_operand(A, lda, K) || !fast_operand(W, ldw, K))
    return DLRM_E_UNSUPPORTED;
  // Block tiles of 256 columns (every column of a row in one workgroup):
  // 128 rows (eight waves of 64 x 64) where that gives every CU a tile, else
  // 64 rows (eight waves of 32 x 64); three LDS stages of 64-wide
  // k-tiles (on 512 -> 256 the loads of a short k loop wait on HBM: at
  // batch 32768 13.5 us with three stages, 14.3 with two; at batch 8192 the
  // 64-row tiles take 8.7 us, the 128-row ones 11.4)
  const int kps = (int)round_up(K, 64);
  const bool big = ceil_div(M, 128) >= device_cu_count();
  if ((K % 64) == 0) {
    if (big)
      launch_fast<128, 256, 64, 64, uint16_t, false, 64, 3, false, 2, false, false, false, true>(
          A, lda, W, ldw, bias, H, ldh, M, N, K, 1, 1, kps, s, DeltaOut{}, dot);
    else
      launch_fast<64, 256, 32, 64, uint16_t, false, 64, 3, false, 2, false, false, false, true>(
          A, lda, W, ldw, bias, H, ldh, M, N, K, 1, 1, kps, s, DeltaOut{}, dot);
  } else {
    if (big)
      launch_fast<128, 256, 64, 64, uint16_t, false, 32, 4, false, 1, false, false, false, true>(
          A, lda, W, ldw, bias, H, ldh, M, N, K, 1, 1, kps, s, DeltaOut{}, dot);
    else  // four waves of 64 x 64 (a 32-wide k-tile of 64 rows is half a load per wave of eight)
      launch_fast<64, 256, 64, 64, uint16_t, false, 32, 4, false, 1, false, false, false, true>(
          A, lda, W, ldw, bias, H, ldh, M, N, K, 1, 1, kps, s, DeltaOut{}, dot);
  }
  return launch_status();
}

int gemm_bf16_splitk_kmajor(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, float* part, int M,
                            int N, int K, int splits, hipStream_t s) {
  if (M <= 0 || N <= 0) return DLRM_OK;
  if (!fast_operand(A, lda, M) || !fast_operand(W, ldw, N)) return DLRM_E_UNSUPPORTED;
  const int kps = (int)round_up(ceil_div(K > 0 ? K : 1, splits), 64);
  launch_fast<128, 128, 64, 64, float, true, 64, 2, false, 2, false, true, true>(A, lda, W, ldw, nullptr, part, N, M,
                                                                                N, K, 0, splits, kps, s);
  return launch_status();
}

int gemv_bf16(const uint16_t* A, int64_t lda, const uint16_t* w, const float* bias, float* out, int64_t ldo,
              float* prob, int M, int K, bool relu, hipStream_t s) {
  if (M <= 0) return DLRM_OK;
  const int vec = aligned16(A) && aligned16(w) && (lda % 8) == 0;
  hipLaunchKernelGGL(gemv_bf16_kernel, dim3((unsigned)ceil_div(M, 16)), dim3(256), 0, s, A, lda, w, bias, out, ldo,
                     prob, M, K, (int)relu, vec);
  return launch_status();
}

int gemm_f32(const float* A, int64_t lda, const float* W, int64_t ldw, const float* bias, float* C, int64_t ldc,
             float* prob, int M, int N, int K, bool relu, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  if (total <= 0) return DLRM_OK;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, s, A, lda, W, ldw, bias, C,
                     ldc, prob, M, N, K, (int)relu);
  return launch_status();
}

int transpose_bf16(const uint16_t* in, int64_t ld_in, uint16_t* out, int64_t ld_out, int R, int C, hipStream_t s) {
  if (R <= 0 || C <= 0) return DLRM_OK;
  const dim3 grid((unsigned)ceil_div(C, 64), (unsigned)ceil_div(R, 64));
  if ((ld_in % 8) == 0 && (ld_out % 8) == 0 && aligned16(in) && aligned16(out))
    hipLaunchKernelGGL(transpose_bf16_v8_kernel, grid, dim3(256), 0, s, in, ld_in, out, ld_out, R, C);
  else
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, in, ld_in, out, ld_out, R, C);
  return launch_status();
}

int convert_to_bf16(const float* in, int64_t ld_in, uint16_t* out, int64_t ld_out, int R, int C, hipStream_t s) {
  const int Cpad = (int)(round_up(C, 8) < ld_out ? round_up(C, 8) : ld_out);
  const int64_t total = (int64_t)R * Cpad;
  if (total <= 0) return DLRM_OK;
  hipLaunchKernelGGL(convert_bf16_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, s, in, ld_in, out, ld_out,
                     R, C, Cpad);
  return launch_status();
}

}  // namespace dlrm
