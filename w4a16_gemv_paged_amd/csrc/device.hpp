// Device helpers shared by the HIP kernels of libnq (gfx950, wave64): fp16
// vector types, the in-register INT4 unpack of the packed weight tiles, the
// matrix-core operand types, and s_waitcnt encodings.
#pragma once

#include "common.hpp"

namespace nq {

typedef _Float16 half_t;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

// ORs error bits into the optional device flag.
__device__ __forceinline__ void raise_flag(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
}

// Workgroup barrier that orders LDS accesses only: the fences are limited to
// the local address space, so vector-memory loads stay in flight across it
// (a plain __syncthreads() would wait for every outstanding load).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this lane's LDS accesses against the other lanes of its own wave
// (wave-local sync; never a block barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One 32-bit word of eight offset-binary nibbles -> four pairs of exact fp16
// codes: (q[k], q[k+1]), (q[k+2], q[k+3]), (q[k+4], q[k+5]), (q[k+6], q[k+7]).
// A nibble n in bits 0-3 of a 16-bit half, OR'ed with 0x6400, is the half
// 1024 + n; subtracting 1032 leaves q = n - 8 exactly. A nibble in bits 4-7
// gives 1024 + 16n; (1024 + 16n) / 16 - 72 = n - 8, also exact. ``magic``
// (0x64006400) is passed in a register so that each mask-and-insert is a
// single v_and_or_b32 (gfx9 VOP3 cannot take two literal constants).
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t magic, h2 (&o)[4]) {
  const h2 off_lo = {static_cast<half_t>(-1032.0f), static_cast<half_t>(-1032.0f)};
  const h2 sixteenth = {static_cast<half_t>(0.0625f), static_cast<half_t>(0.0625f)};
  const h2 off_hi = {static_cast<half_t>(-72.0f), static_cast<half_t>(-72.0f)};
  const uint32_t w8 = w >> 8;
  o[0] = as_h2((w & 0x000F000Fu) | magic) + off_lo;
  o[1] = __builtin_elementwise_fma(as_h2((w & 0x00F000F0u) | magic), sixteenth, off_hi);
  o[2] = as_h2((w8 & 0x000F000Fu) | magic) + off_lo;
  o[3] = __builtin_elementwise_fma(as_h2((w8 & 0x00F000F0u) | magic), sixteenth, off_hi);
}

__device__ __forceinline__ void unpack8(uint32_t w, h2 (&o)[4]) { unpack8(w, 0x64006400u, o); }

__device__ __forceinline__ float dot2(h2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(a, as_h2(b), c, false);
}

__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

constexpr int kBufferFlags = 0x00020000;    // gfx9 raw buffer descriptor word 3

// acc[i] += d[i] * scale of row 4*(l/16)+i (fp16 scales of four rows in sc)
__device__ __forceinline__ void scale_acc(f4& acc, const f4& d, const u32x2& sc) {
  const h2 s01 = as_h2(sc.x), s23 = as_h2(sc.y);
  acc[0] = fmaf(d[0], static_cast<float>(s01[0]), acc[0]);
  acc[1] = fmaf(d[1], static_cast<float>(s01[1]), acc[1]);
  acc[2] = fmaf(d[2], static_cast<float>(s23[0]), acc[2]);
  acc[3] = fmaf(d[3], static_cast<float>(s23[1]), acc[3]);
}

// Greedy tie rule: larger value wins, equal values go to the lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// s_waitcnt immediates (gfx9 encoding): wait for LDS/scalar memory only, or
// for LDS/scalar memory and until at most n vector-memory operations are
// outstanding.
constexpr int kWaitLgkm0 = 0xC07F;
constexpr int wait_vm_lgkm0(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

}  // namespace nq
