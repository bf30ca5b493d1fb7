// Device-side helpers shared by the libstarkv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

#define SKV_LOG2E 1.4426950408889634f

namespace skv {

// ---- scalar conversions (all round-to-nearest-even) ----
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f32_to_f16(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// ---- wave helpers ----
// Wave index within the workgroup, provably uniform to the compiler: branches on values
// derived from it become scalar branches.  This matters around MFMA instructions, which
// do not honour EXEC: an MFMA left in an exec-masked (linearised) branch still executes.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }
__device__ __forceinline__ float wave_sum_xor(float v, int mask) { return v + __shfl_xor(v, mask, 64); }

// ---- 16-byte loads/stores ----
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Load of read-only data at a wave-uniform address through the scalar data cache (the constant
// address space): layer tables that no kernel writes.  Unlike a vector load it needs no VGPRs
// and returns through the scalar cache.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// ---- buffer loads ----
// A buffer resource covering [base, base + bytes) (gfx9 raw layout: no stride, no swizzle).  A
// load whose byte offset lies at or past `bytes` returns zeros and touches no memory, so a
// kernel can issue its loads unconditionally and point the ones it does not need past the end,
// with no branch around them (a branch around a load makes the compiler wait for every load in
// flight where the paths join).  The base must be wave-uniform; bytes < 2^32.
constexpr uint32_t kOOB = 0xFFFFFFF0u;  // an offset past the end of every buffer resource
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// 12 bytes at a 4-byte aligned offset (zeros past the end, like bld16)
__device__ __forceinline__ u32x3 bld12(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x2 bld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// signed nibble / byte extraction
__device__ __forceinline__ int sbyte(uint32_t w, int i) { return (int)(w << (24 - 8 * i)) >> 24; }
__device__ __forceinline__ int snib(uint32_t w, int i) { return (int)(w << (28 - 4 * i)) >> 28; }

// int4 group of 16 channels (8 bytes, channel 2k in the low nibble of byte k) -> 16 int8 in the
// order [0,2,4,...,14, 1,3,...,15] as offset binary (code + 8); see the key-score bias term.
__device__ __forceinline__ i32x4 unpack_int4_group(u32x2 w) {
  uint32_t a = w[0] ^ 0x88888888u, b = w[1] ^ 0x88888888u;
  i32x4 r;
  r[0] = (int)(a & 0x0F0F0F0Fu);
  r[1] = (int)(b & 0x0F0F0F0Fu);
  r[2] = (int)((a >> 4) & 0x0F0F0F0Fu);
  r[3] = (int)((b >> 4) & 0x0F0F0F0Fu);
  return r;
}

// 16 packed 3-bit fields (offset binary, code + 4) of half h of a 32-channel group given as its
// three bit-plane words: word k, byte j = the field of channel 8 j + k + 4 h (bit b from plane b)
__device__ __forceinline__ i32x4 unpack_int3_group(u32x3 p, bool h) {
  const uint32_t s0 = h ? 4u : 0u;
  i32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t s = s0 + (uint32_t)k;
    r[k] = (int)(((p.x >> s) & 0x01010101u) | (((p.y >> s) & 0x01010101u) << 1) | (((p.z >> s) & 0x01010101u) << 2));
  }
  return r;
}

// position within a 16-slot int4 group of fragment element e (see unpack_int4_group)
__device__ __forceinline__ int int4_perm16(int e) { return e < 8 ? 2 * e : 2 * (e - 8) + 1; }

// ---- MFMA wrappers ----
__device__ __forceinline__ f32x4 mfma16_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i32x4 mfma16_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// Row of a 32x32 MFMA result held in register v of a lane in half q (= lane / 32).
__device__ __forceinline__ int d32_row(int v, int q) { return 8 * (v >> 2) + 4 * q + (v & 3); }

// Largest b in [0, n) with off[b] <= x (off ascending, off[0] == 0, n <= 128), found by the whole
// wave in one round of loads: lane l reads off[l + 1] and off[l + 65], and b counts the segment
// starts off[1 .. n-1] that are <= x.  Call with every lane of the wave active.
__device__ __forceinline__ int find_segment_wave(const int* off, int n, int x) {
  const int lane = threadIdx.x & 63;
  const int v0 = off[min(lane + 1, n)];
  const int v1 = off[min(lane + 65, n)];
  const unsigned long long m0 = __ballot(lane + 1 < n && v0 <= x);
  const unsigned long long m1 = __ballot(lane + 65 < n && v1 <= x);
  return __builtin_amdgcn_readfirstlane(__popcll(m0) + __popcll(m1));
}

// binary search: largest b in [0, n) with off[b] <= x  (off ascending, off[0] == 0)
__device__ __forceinline__ int find_segment(const int* off, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---- asynchronous loads straight into LDS
// Lane l's 16 bytes at src land at LDS byte address lds + 16 l (lds wave-uniform; the builtin
// puts it in M0).  The kernel waits with vm_wait<n>() (n = loads it may leave in flight) and a
// barrier before any wave reads the data.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, 0, 0);
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace skv
