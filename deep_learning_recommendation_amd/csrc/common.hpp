// Internal helpers shared by the libdlrm kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dlrm.h"

namespace dlrm {

// hipError_t of the last failed launch on this thread.
extern thread_local int g_last_hip_error;

inline int launch_status() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return DLRM_E_HIP;
  }
  return DLRM_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32; NaN
// stays NaN, subnormals are rounded, not flushed).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 -> packed bf16 pair (low half = a), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

// s_waitcnt vmcnt(N), expcnt and lgkmcnt left at their maxima (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane i's bytes land at lds + 16 * i; lds must be
// the same for every lane of the wave.  Completion is tracked by vmcnt.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (void __attribute__((address_space(3)))*)lds, 16, 0, 0);
}

// The same 16-byte direct-to-LDS load, issued through inline assembly so the
// compiler's wait-count model does not see an LDS write: with the builtin it
// turns every later LDS-read wait into lgkmcnt(0), exposing each operand read
// of a GEMM k-step.  The asm has no register outputs; completion is still
// vmcnt, which the caller waits for explicitly (followed by a barrier and a
// compiler fence) before any wave reads the destination.
__device__ __forceinline__ void lds_dma16_opaque(const void* src, const void* lds) {
  const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(a) : "memory");
}

// Keeps the compiler from moving memory accesses across this point.
__device__ __forceinline__ void compiler_fence() { __asm__ volatile("" ::: "memory"); }

// Per-device caches (kernel attributes, occupancy, CU counts) are indexed
// by the current device; devices past kMaxDevices share slot 0.
constexpr int kMaxDevices = 64;
inline int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  return dev;
}

// Compute units of the current device (queried once per device).
inline int device_cu_count() {
  static int cached[kMaxDevices] = {0};
  const int dev = current_device();
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) v = 1;
    cached[dev] = v;
  }
  return cached[dev];
}

// Scratch carving: 256-byte aligned sub-buffers of a caller workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t count) {
    used = (size_t)round_up((int64_t)used, 256);
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += sizeof(T) * count;
    return p;
  }
  size_t bytes() const { return (size_t)round_up((int64_t)used, 256); }
};

}  // namespace dlrm
