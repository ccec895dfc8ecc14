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

}  // namespace

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
