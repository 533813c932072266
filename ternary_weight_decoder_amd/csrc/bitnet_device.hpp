// Device-side helpers shared by the gfx950 kernels of the ternary projection
// library.  One code path: gfx950 only, wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kUnit = 128;             // codes per packing unit
constexpr int kUnitBytes = 32;         // bytes per packing unit (2 bits per code)
constexpr uint32_t kFieldMask = 0x03030303u;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define BITNET_GLOBAL __attribute__((address_space(1)))

// Loads and stores through global-address-space pointers.  Pointers that arrive
// in structs are generic to the compiler, which would emit flat accesses; those
// count on both vmcnt and lgkmcnt, so every LDS wait would also drain the memory
// pipeline.  T must be a scalar or a native (ext_vector_type) vector: HIP's
// class-based vector types lose the address space on the way.
template <typename T>
__device__ __forceinline__ T ld_global(const void *p) {
  return *(const BITNET_GLOBAL T *)p;
}
template <typename T>
__device__ __forceinline__ void st_global(void *p, T v) {
  *(BITNET_GLOBAL T *)p = v;
}

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding and leaves the other counters alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_wait(int n) {
  return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}
// The same for the LDS / scalar-memory counter alone (vmcnt left at its
// maximum, 63, which never waits).
constexpr int lgkmcnt_wait(int n) { return 0xf | (0x3 << 14) | (0x7 << 4) | ((n & 0xf) << 8); }

// Raw buffer resource over `bytes` bytes at `base` (stride 0; the 32-bit data
// format that untyped buffer loads need on gfx9-family parts).  A load whose
// offset is at or beyond `bytes` returns zeros and makes no memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The four 2-bit fields of one packed dword, each spread into the bytes of one
// output dword.  For dword d of unit t (bytes 4d..4d+3), output dword g holds in
// byte c the field value u = code + 1 of input k = 128t + 32g + 4d + c.
__device__ __forceinline__ v4i unpack_fields(uint32_t d) {
  v4i b;
  b.x = (int)(d & kFieldMask);
  b.y = (int)((d >> 2) & kFieldMask);
  b.z = (int)((d >> 4) & kFieldMask);
  b.w = (int)((d >> 6) & kFieldMask);
  return b;
}

// Offset of input k inside a row of permuted int8 activations.  Inside each
// 128-input unit, natural k = 128t + 32g + 4d + c is stored at 128t + 16d + 4g + c,
// so the 16 activations that meet packed dword d of a unit are 16 contiguous
// bytes (in the byte order unpack_fields produces).
__device__ __forceinline__ int perm_offset(int k) {
  const int t = k >> 7, r = k & 127;
  const int g = r >> 5, d = (r & 31) >> 2, c = r & 3;
  return (t << 7) + (d << 4) + (g << 2) + c;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Round half to even, then clamp to [-127, 127] (v_rndne_f32 + v_med3).
__device__ __forceinline__ int quant_one(float x, float s) {
  float p = x * s;
  float r = __builtin_rintf(p);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

// Dequantization epilogue, exactly rounded: acc * w_scale is exact in fp64
// (|acc| < 2^21 times a 24-bit significand), the fp64 division is correctly
// rounded, and the result is rounded once more to fp32 -- the same operations
// in the same order as the plain definition, so the value is reproduced bit for
// bit.  Used where outputs are few (decode); the prefill epilogue uses one fp32
// factor per row instead.
__device__ __forceinline__ float dequant_exact(int acc, float w_scale, float x_scale) {
  return (float)((double)acc * (double)w_scale / (double)x_scale);
}

}  // namespace bitnet
