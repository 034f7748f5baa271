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

// One 32-bit word of eight offset-binary nibbles n = q + 8 -> four pairs of
// fp16 values, with no arithmetic: a nibble in bits 0-3 of a 16-bit half
// OR'ed with 0x6400 is the half 1024 + n = q + 1032, a nibble in bits 4-7
// gives 1024 + 16n = 16 (q + 72). Pairs 0 and 2 hold (q[k], q[k+1]) and
// (q[k+4], q[k+5]) in the first form, pairs 1 and 3 hold (q[k+2], q[k+3]) and
// (q[k+6], q[k+7]) in the second. ``magic`` (0x64006400) is passed in a
// register so that each mask-and-insert is a single v_and_or_b32.
//
// The matrix-core products use these biased codes directly: the activations
// are stored with the halves at K offsets 2, 3, 6, 7 (mod 8) multiplied by
// 1/16 (exact for fp16 above the subnormal range), so that
//   sum_k code_k x'_k = sum_k q_k x_k + sum_k bias_k x'_k,
// bias_k = 1032 at offsets 0, 1, 4, 5 and 16 * 72 = 1152 at 2, 3, 6, 7; the
// second term is removed by products with the constant fragment -bias. This
// takes 5 VALU operations per word instead of 9, at the price of fp32
// cancellation of the bias terms (a few 1e-5 relative on a group's sum).
__device__ __forceinline__ void unpack8_biased(uint32_t w, uint32_t magic, h2 (&o)[4]) {
  const uint32_t w8 = w >> 8;
  o[0] = as_h2((w & 0x000F000Fu) | magic);
  o[1] = as_h2((w & 0x00F000F0u) | magic);
  o[2] = as_h2((w8 & 0x000F000Fu) | magic);
  o[3] = as_h2((w8 & 0x00F000F0u) | magic);
}

// The exact codes from the biased ones: (q + 1032) - 1032 and 16 (q + 72) / 16 - 72.
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t magic, h2 (&o)[4]) {
  const h2 off_lo = {static_cast<half_t>(-1032.0f), static_cast<half_t>(-1032.0f)};
  const h2 sixteenth = {static_cast<half_t>(0.0625f), static_cast<half_t>(0.0625f)};
  const h2 off_hi = {static_cast<half_t>(-72.0f), static_cast<half_t>(-72.0f)};
  unpack8_biased(w, magic, o);
  o[0] = o[0] + off_lo;
  o[1] = __builtin_elementwise_fma(o[1], sixteenth, off_hi);
  o[2] = o[2] + off_lo;
  o[3] = __builtin_elementwise_fma(o[3], sixteenth, off_hi);
}

__device__ __forceinline__ void unpack8(uint32_t w, h2 (&o)[4]) { unpack8(w, 0x64006400u, o); }

// Pre-scaling of 8 consecutive activations (K offsets 0..7 mod 8) for the
// biased codes: halves 2, 3, 6, 7 times 1/16.
__device__ __forceinline__ void scale_high_halves(uint32_t (&v)[4]) {
  const h2 sixteenth = {static_cast<half_t>(0.0625f), static_cast<half_t>(0.0625f)};
  v[1] = __builtin_bit_cast(uint32_t, as_h2(v[1]) * sixteenth);
  v[3] = __builtin_bit_cast(uint32_t, as_h2(v[3]) * sixteenth);
}

// 1/16 for the K offsets (mod 8) that meet a high-nibble code, else 1.
__device__ __forceinline__ float high_scale(int e) { return (e & 2) ? 0.0625f : 1.0f; }

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

// The constant MFMA A fragment -bias (every row alike; lane element i is K
// offset 8*(lane/16) + i of the product, i.e. i mod 8 of the group's K).
__device__ __forceinline__ half8 neg_bias_frag() {
  const half_t a = static_cast<half_t>(-1032.0f), b = static_cast<half_t>(-1152.0f);
  return half8{a, a, b, b, a, a, b, b};
}

constexpr int kBufferFlags = 0x00020000;    // gfx9 raw buffer descriptor word 3

// Cache policy of the decode GEMVs' weight and scale loads: non-temporal (the
// instruction's nt bit). Every packed byte is read once per step, so keeping
// it out of the caches' normal replacement order leaves room for what is
// reused; a streaming probe on MI355X read 1 KiB blocks 8% faster with it.
constexpr int kStreamOnce = 2;

// acc[i] += d[i] * scale of row 4*(l/16)+i (fp16 scales of four rows in sc)
__device__ __forceinline__ void scale_acc(f4& acc, const f4& d, const u32x2& sc) {
  const h2 s01 = as_h2(sc.x), s23 = as_h2(sc.y);
  acc[0] = fmaf(d[0], static_cast<float>(s01[0]), acc[0]);
  acc[1] = fmaf(d[1], static_cast<float>(s01[1]), acc[1]);
  acc[2] = fmaf(d[2], static_cast<float>(s23[0]), acc[2]);
  acc[3] = fmaf(d[3], static_cast<float>(s23[1]), acc[3]);
}

// Lane n of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x150 + N, 0xF, 0xF, false));
}

// The same for both words of a pair; n must be a constant once the caller's
// loop is unrolled (the switch then folds away).
__device__ __forceinline__ u32x2 row_bcast2(const u32x2& v, int n) {
  switch (n & 15) {
#define NQ_BCAST_CASE(N) \
  case N:                \
    return u32x2{row_bcast<N>(v.x), row_bcast<N>(v.y)};
    NQ_BCAST_CASE(0) NQ_BCAST_CASE(1) NQ_BCAST_CASE(2) NQ_BCAST_CASE(3)
    NQ_BCAST_CASE(4) NQ_BCAST_CASE(5) NQ_BCAST_CASE(6) NQ_BCAST_CASE(7)
    NQ_BCAST_CASE(8) NQ_BCAST_CASE(9) NQ_BCAST_CASE(10) NQ_BCAST_CASE(11)
    NQ_BCAST_CASE(12) NQ_BCAST_CASE(13) NQ_BCAST_CASE(14) NQ_BCAST_CASE(15)
#undef NQ_BCAST_CASE
  }
  return v;
}

// Greedy tie rule: larger value wins, equal values go to the lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// s_waitcnt immediates (gfx9 encoding): wait for LDS/scalar memory only, or
// for LDS/scalar memory and until at most n vector-memory operations are
// outstanding.
constexpr int kWaitLgkm0 = 0xC07F;
constexpr int kWaitVm0 = 0x0F70;    // s_waitcnt vmcnt(0) alone
constexpr int wait_vm_lgkm0(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

}  // namespace nq
