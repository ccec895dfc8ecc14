// Device-side generator for synthetic embedding tables.
//
// Element (r, c) of table t is a * (2u - 1), u = (h >> 40) * 2^-24, where h
// is output number r*d + c + 1 of a SplitMix64 generator (Steele, Lea &
// Flood, OOPSLA 2014) whose state is the table's key.  2u - 1 is an exact
// fp32 number, so the product with a is the only rounding and the host-side
// generator reproduces every value bit for bit.  This file is input
// generation for tests and benchmarks; it computes no step of the model.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t splitmix_out(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float table_value(uint64_t key, uint64_t e, float a) {
  const uint64_t h = splitmix_out(key + (e + 1ull) * kGamma);
  const int32_t top = (int32_t)(h >> 40);                       // 24 bits
  const float t = (float)(top * 2 - (1 << 24)) * 5.9604644775390625e-08f;  // exact
  return __fmul_rn(a, t);
}

__global__ void __launch_bounds__(256) fill_kernel(float4* __restrict__ out, uint64_t n4, uint64_t key, float a) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const uint64_t e = i * 4ull;
    float4 v;
    v.x = table_value(key, e + 0, a);
    v.y = table_value(key, e + 1, a);
    v.z = table_value(key, e + 2, a);
    v.w = table_value(key, e + 3, a);
    __builtin_nontemporal_store(v.x, &out[i].x);
    __builtin_nontemporal_store(v.y, &out[i].y);
    __builtin_nontemporal_store(v.z, &out[i].z);
    __builtin_nontemporal_store(v.w, &out[i].w);
  }
}

// Low-precision tables.  bf16: the high half of the fp32 value above (its
// truncation to bf16).  int8: q = the top 8 bits of the element's SplitMix64
// output as a signed byte; per row r, scale s = a * ((0.5 + u1) * 2^-7) and
// bias z = a * ((2 u2 - 1) * 2^-3) from outputs 2r + 1 and 2r + 2 of the
// row-parameter state (u1 with 23 random bits, u2 with 24: the factors after
// a are exact, so each of s and z is one rounding).
__global__ void __launch_bounds__(256) fill_bf16_kernel(uint2* __restrict__ out, uint64_t n4, uint64_t key, float a) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const uint64_t e = i * 4ull;
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = __float_as_uint(table_value(key, e + j, a)) >> 16;
    out[i] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }
}

__global__ void __launch_bounds__(256) fill_i8_kernel(uint32_t* __restrict__ out, uint64_t n4, uint64_t key) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const uint64_t e = i * 4ull;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= (uint32_t)(splitmix_out(key + (e + j + 1ull) * kGamma) >> 56) << (8 * j);
    out[i] = w;
  }
}

__global__ void __launch_bounds__(256) fill_scale_bias_kernel(float2* __restrict__ out, uint64_t rows, uint64_t key,
                                                              float a) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t r = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows; r += stride) {
    const uint64_t h1 = splitmix_out(key + (2ull * r + 1ull) * kGamma);
    const uint64_t h2 = splitmix_out(key + (2ull * r + 2ull) * kGamma);
    const float u1 = (float)(uint32_t)(h1 >> 41) * 1.1920928955078125e-07f;  // 2^-23, exact
    const float f1 = (0.5f + u1) * 0.0078125f;                                 // exact
    const int32_t top = (int32_t)(h2 >> 40);
    const float f2 = (float)(top * 2 - (1 << 24)) * 7.450580596923828e-09f;  // (2 u2 - 1) 2^-3, exact
    out[r] = make_float2(__fmul_rn(a, f1), __fmul_rn(a, f2));
  }
}

}  // namespace

extern "C" int synth_fill_table_bf16(uint16_t* out, int64_t rows, int32_t d, uint64_t key, float a, hipStream_t s) {
  if (out == nullptr || rows < 0 || d <= 0 || (d % 4) != 0 || (reinterpret_cast<uintptr_t>(out) & 15u)) return -1;
  const uint64_t n4 = (uint64_t)rows * (uint64_t)d / 4ull;
  if (n4 == 0) return 0;
  uint64_t blocks = (n4 + 255) / 256;
  if (blocks > 65536ull * 4) blocks = 65536ull * 4;
  hipLaunchKernelGGL(fill_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<uint2*>(out), n4, key,
                     a);
  return (int)hipGetLastError();
}

// int8 values with key `key`, per-row (scale, bias) pairs with key `sb_key`.
extern "C" int synth_fill_table_i8(int8_t* out, float* scale_bias, int64_t rows, int32_t d, uint64_t key,
                                   uint64_t sb_key, float a, hipStream_t s) {
  if (out == nullptr || scale_bias == nullptr || rows < 0 || d <= 0 || (d % 4) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 15u) || (reinterpret_cast<uintptr_t>(scale_bias) & 7u))
    return -1;
  const uint64_t n4 = (uint64_t)rows * (uint64_t)d / 4ull;
  if (n4 == 0) return 0;
  uint64_t blocks = (n4 + 255) / 256;
  if (blocks > 65536ull * 4) blocks = 65536ull * 4;
  hipLaunchKernelGGL(fill_i8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<uint32_t*>(out), n4,
                     key);
  uint64_t rb = ((uint64_t)rows + 255) / 256;
  if (rb > 65536ull) rb = 65536ull;
  hipLaunchKernelGGL(fill_scale_bias_kernel, dim3((unsigned)rb), dim3(256), 0, s,
                     reinterpret_cast<float2*>(scale_bias), (uint64_t)rows, sb_key, a);
  return (int)hipGetLastError();
}

// Fill table `out` ([rows][d] fp32, d % 4 == 0, 16-byte aligned) with the
// synthetic values for state `key` and half-width `a`.  Returns 0 or a HIP
// error code.
extern "C" int synth_fill_table(float* out, int64_t rows, int32_t d, uint64_t key, float a, hipStream_t s) {
  if (out == nullptr || rows < 0 || d <= 0 || (d % 4) != 0 || (reinterpret_cast<uintptr_t>(out) & 15u)) return -1;
  const uint64_t n4 = (uint64_t)rows * (uint64_t)d / 4ull;
  if (n4 == 0) return 0;
  uint64_t blocks = (n4 + 255) / 256;
  if (blocks > 65536ull * 4) blocks = 65536ull * 4;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<float4*>(out), n4, key, a);
  return (int)hipGetLastError();
}
