// HIP kernels of the INT8-activation (W4A8) projection variant of libnq, for
// CDNA4 (gfx950), wave64.
//
// "How To Build Your Own LLM Runtime From Scratch" (daily.dev), Summary and the
// FAQ question on INT8-activation dp4a against FP16-activation INT4 unpack: the
// activations were quantised to INT8 in an extra kernel before each GEMV and
// multiplied with the INT4 weights in integer arithmetic, and that path lost.
// Here the same idea on the matrix cores, two ways:
// * quantize_a8_kernel + gemv_w4a8_kernel<..., QIN = false>: the extra kernel;
// * gemv_w4a8_kernel<..., QIN = true>: the GEMV quantises the fp16 activations
//   in its own prologue (no extra kernel, no int8 round trip through memory).
// Quantisation: per row and group of 128, s = fp32(max |x|) / 127, q =
// round_half_even(fp32(x) / s) clamped to [-127, 127] (q = 0 when s = 0). The
// INT4 codes are used as their stored offset-binary bytes n = q_w + 8 (mask
// and shift only), the group's integer dot product comes from two
// v_mfma_i32_16x16x64_i8, and the offset is removed exactly with the group's
// code sum: sum_k q_w q_x = sum_k n q_x - 8 sum_k q_x. The fp16 weight scale
// and the fp32 activation scale multiply each group's sum in fp32.
#include <algorithm>

#include "device.hpp"

namespace nq {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Byte order of a group's activation codes in memory and LDS: each 8 inputs
// k0..k0+7 are stored as k0, k0+4, k0+1, k0+5, k0+2, k0+6, k0+3, k0+7, the
// order in which the two dwords (w & 0x0F0F0F0F) and (w >> 4) & 0x0F0F0F0F of
// a packed code word hold their nibbles. A lane's 16 consecutive bytes are
// then one MFMA operand on both sides.
struct A8Meta {
  float s;  // activation scale of the (row, group)
  int sum;  // sum of the group's codes
};

// Bytes of the (scale, sum) array of B rows, padded to whole 16-byte copies.
__host__ __device__ inline int a8_meta_bytes(int B, int G) { return (B * G * 8 + 15) / 16 * 16; }

// The 16 lanes of an aligned team hold the 128 inputs of one group, lane t the
// 8 inputs 8t..8t+7 (lane-team shuffles only). Returns the 8 codes in stored
// byte order and, in every lane, the group's scale and code sum.
__device__ __forceinline__ void quantize_group8(const half_t (&v)[8], uint32_t& lo, uint32_t& hi, float& s,
                                                int& sum) {
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(static_cast<float>(v[e])));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
  s = a / 127.0f;
  int q[8];
  int ls = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float r = s > 0.0f ? static_cast<float>(v[e]) / s : 0.0f;
    q[e] = min(127, max(-127, static_cast<int>(rintf(r))));
    ls += q[e];
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) ls += __shfl_xor(ls, o);
  sum = ls;
  auto b = [](int x) { return static_cast<uint32_t>(x) & 0xFFu; };
  lo = b(q[0]) | (b(q[4]) << 8) | (b(q[1]) << 16) | (b(q[5]) << 24);
  hi = b(q[2]) | (b(q[6]) << 8) | (b(q[3]) << 16) | (b(q[7]) << 24);
}

// grid ceil(B*G*16 / 256), 256 threads: one 16-lane team per (row, group).
// xq: int8 [B][K] in stored byte order, then meta [B][G].
__global__ __launch_bounds__(256) void quantize_a8_kernel(const half_t* x, int B, int K, uint8_t* xq) {
  const int G = K / kGroup;
  const int team = (blockIdx.x * blockDim.x + threadIdx.x) >> 4, t = threadIdx.x & 15;
  const bool ok = team < B * G;  // team-uniform
  const int b = ok ? team / G : 0, g = ok ? team % G : 0;
  half_t v[8];
  *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(b) * K + g * kGroup + 8 * t);
  uint32_t lo, hi;
  float s;
  int sum;
  quantize_group8(v, lo, hi, s, sum);
  if (!ok) return;
  *reinterpret_cast<uint2*>(xq + static_cast<int64_t>(b) * K + g * kGroup + 8 * t) = make_uint2(lo, hi);
  if (t == 0) {
    A8Meta* meta = reinterpret_cast<A8Meta*>(xq + static_cast<int64_t>(B) * K);
    meta[b * G + g] = A8Meta{s, sum};
  }
}

// 1 KiB weight loads in flight per wave: 5 rather than 7, as for the W4A16
// GEMV (fused gate/up at batch 1 13.5-14.1 against 14.7 us, same box).
constexpr int kA8Depth = 5;

struct A8Params {
  const uint8_t* codes;
  const uint8_t* scales;
  int N, K, kind, head_dim, G, T, tpw, ks;
  const half_t* x;    // QIN: fp16 [B][K]
  const uint8_t* xq;  // !QIN: quantised activations + meta (quantize_a8_kernel output)
  const half_t* bias;
  void* y;
};

// Work split as in the W4A16 GEMV: a workgroup holds tpw tiles x ks K-slices,
// one wave each; wave (tl, ksi) walks groups ksi, ksi + ks, ... of its tile
// with a kA8Depth-deep ring of 1 KiB code blocks and one scale window per ring
// pass. The activation codes and (scale, sum) pairs of the whole row sit in
// LDS (all of K: the launcher checks that it fits).
template <int B, int EPI, bool QIN>
__global__ __launch_bounds__(1024) void gemv_w4a8_kernel(A8Params p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = blockDim.x >> 6;
  const int col = lane & 15, kb = lane >> 4;
  const int tl = wave / p.ks, ksi = wave % p.ks;
  const int t = static_cast<int>(blockIdx.x) * p.tpw + tl;
  const bool tile_ok = t < p.T;
  const int K = p.K, G = p.G;
  // LDS: [B][K] codes | [B][G] meta (padded to 16 bytes) | 128-byte zero block
  //      (the operands of the columns past the batch: 32 * (lane / 16) + 16 m
  //      + 16 bytes) | red [nw][B][16] | (QIN) [B][K] fp16
  uint8_t* xs = smem;
  A8Meta* meta = reinterpret_cast<A8Meta*>(smem + B * K);
  uint8_t* zero = smem + B * K + a8_meta_bytes(B, G);
  float* red = reinterpret_cast<float*>(zero + 128);
  half_t* xf = reinterpret_cast<half_t*>(red + nw * B * 16);
  if (tid < 32) reinterpret_cast<uint32_t*>(zero)[tid] = 0u;

  // (1) activations into LDS by DMA, 16 bytes per lane
  {
    const int row_items = QIN ? K / 8 : K / 16;              // 16-byte items per row
    const int meta_items = QIN ? 0 : a8_meta_bytes(B, G) / 16;
    const int items = B * row_items + meta_items;
    for (int i0 = wave * 64; i0 < items; i0 += nw * 64) {
      const int i = i0 + lane;
      if (i < items) {
        const void* src;
        void* dst;
        if (i < B * row_items) {
          const int b = i / row_items, j = i - b * row_items;
          if constexpr (QIN) {
            src = p.x + static_cast<int64_t>(b) * K + 8 * j;
            dst = xf + b * K + 8 * j;
          } else {
            src = p.xq + static_cast<int64_t>(b) * K + 16 * j;
            dst = xs + b * K + 16 * j;
          }
        } else {
          const int j = i - B * row_items;
          src = p.xq + static_cast<int64_t>(B) * K + 16 * j;
          dst = reinterpret_cast<uint8_t*>(meta) + 16 * j;
        }
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // (2) the weight ring and the first scale window (past the tile: zeros)
  const int tq = tile_ok ? t : 0;
  const int wbytes = tile_ok ? G * kBlockBytes : 0, sbytes = tile_ok ? G * 32 : 0;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.codes) + static_cast<size_t>(tq) * G * kBlockBytes, 0, wbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.scales) + static_cast<size_t>(tq) * G * 32, 0, sbytes, kBufferFlags);
  const int n_c = (G - ksi + p.ks - 1) / p.ks;
  auto load_scales = [&](int w0) {
    const int bi = w0 + col;
    const int g = ksi + p.ks * bi;
    return __builtin_amdgcn_raw_buffer_load_b64(srs, (col < kA8Depth && bi < n_c) ? g * 32 + kb * 8 : sbytes, 0, kStreamOnce);
  };
  u32x2 swin = load_scales(0);
  u32x4 wv[kA8Depth];
#pragma unroll
  for (int u = 0; u < kA8Depth; ++u) {
    const int g = ksi + p.ks * u;
    wv[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, lane * 16, u < n_c ? g * kBlockBytes : wbytes, kStreamOnce);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kA8Depth + 1));  // this wave's LDS copies have landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  // (3) quantise in place (QIN): one 16-lane team per (row, group)
  if constexpr (QIN) {
    for (int team = tid >> 4; team < B * G; team += blockDim.x >> 4) {
      const int b = team / G, g = team % G, tt = tid & 15;
      half_t v[8];
      *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(xf + b * K + g * kGroup + 8 * tt);
      uint32_t lo, hi;
      float s;
      int sum;
      quantize_group8(v, lo, hi, s, sum);
      *reinterpret_cast<uint2*>(xs + b * K + g * kGroup + 8 * tt) = make_uint2(lo, hi);
      if (tt == 0) meta[b * G + g] = A8Meta{s, sum};
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }

  // (4) the stream: per block, two integer MFMAs, the offset correction, and
  //     the two scales in fp32
  const uint8_t* xlane = (col < B ? xs + col * K : zero) + 32 * kb;
  const int xstep = col < B ? kGroup : 0;
  const int mcol = col < B ? col : 0;
  f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto block = [&](const int u, const int i) {
    const int g = ksi + p.ks * i;
    const uint8_t* xg = xlane + g * xstep;
    const u32x4 w = wv[u];
    i32x4 d = {0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t w0 = w[2 * m], w1 = w[2 * m + 1];
      const i32x4 a = {static_cast<int>(w0 & 0x0F0F0F0Fu), static_cast<int>((w0 >> 4) & 0x0F0F0F0Fu),
                       static_cast<int>(w1 & 0x0F0F0F0Fu), static_cast<int>((w1 >> 4) & 0x0F0F0F0Fu)};
      const i32x4 bx = *reinterpret_cast<const i32x4*>(xg + 16 * m);
      d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bx, d, 0, 0, 0);
    }
    const A8Meta mt = meta[mcol * G + g];
    const float sx = col < B ? mt.s : 0.0f;
    const int off = 8 * mt.sum;
    const f4 f = {static_cast<float>(d[0] - off) * sx, static_cast<float>(d[1] - off) * sx,
                  static_cast<float>(d[2] - off) * sx, static_cast<float>(d[3] - off) * sx};
    scale_acc(acc, f, row_bcast2(swin, u));
  };
  // Every window but the last refills each slot it consumes, on every path (a
  // block past the wave's last reads past the tile and returns 0): the loads
  // in flight are then the same on every path, and the compiler's wait for a
  // block counts only what is older than it. The last window refills nothing.
  int ib = 0;
  for (; ib + kA8Depth < n_c; ib += kA8Depth) {
    const u32x2 snext = load_scales(ib + kA8Depth);
#pragma unroll
    for (int u = 0; u < kA8Depth; ++u) {
      const int i = ib + u;
      block(u, i);
      const int gn = ksi + p.ks * (i + kA8Depth);
      wv[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, lane * 16, i + kA8Depth < n_c ? gn * kBlockBytes : wbytes,
                                                    kStreamOnce);
    }
    swin = snext;
  }
  if (ib < n_c) {
#pragma unroll
    for (int u = 0; u < kA8Depth; ++u)
      if (ib + u < n_c) block(u, ib + u);
  }

  // (5) K slices summed through LDS, then the epilogue on (tile, batch row, tile row) items
  if (col < B) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * B + col) * 16 + 4 * kb + i] = acc[i];
  }
  __syncthreads();
  const int items = p.tpw * B * 16;
  for (int it = tid; it < items; it += blockDim.x) {
    const int tl2 = it / (B * 16), b = (it / 16) % B, rr = it & 15;
    const int64_t tt = static_cast<int64_t>(blockIdx.x) * p.tpw + tl2;
    if (tt >= p.T) continue;
    float yv = 0.0f, yp = 0.0f;
    for (int k2 = 0; k2 < p.ks; ++k2) {
      yv += red[((tl2 * p.ks + k2) * B + b) * 16 + rr];
      yp += red[((tl2 * p.ks + k2) * B + b) * 16 + (rr ^ 8)];
    }
    const int64_t n = tile_row_logical(p.kind, p.N, p.head_dim, tt, rr);
    const int64_t N = p.N;
    if constexpr (EPI == NQ_EPI_STORE_F16) {
      if (n < N) static_cast<half_t*>(p.y)[b * N + n] = static_cast<half_t>(yv);
    } else if constexpr (EPI == NQ_EPI_BIAS_F16) {
      if (n < N) static_cast<half_t*>(p.y)[b * N + n] = static_cast<half_t>(yv + static_cast<float>(p.bias[n]));
    } else if constexpr (EPI == NQ_EPI_RESIDUAL_F16) {
      if (n < N) {
        half_t* yo = static_cast<half_t*>(p.y) + b * N + n;
        *yo = static_cast<half_t>(static_cast<float>(*yo) + yv);
      }
    } else if constexpr (EPI == NQ_EPI_SWIGLU_F16) {
      if (rr < 8) {
        const float a = yv / (1.0f + expf(-yv)) * yp;
        static_cast<half_t*>(p.y)[b * (N / 2) + 8 * tt + rr] = static_cast<half_t>(a);
      }
    } else if constexpr (EPI == NQ_EPI_STORE_F32) {
      if (n < N) static_cast<float*>(p.y)[b * N + n] = yv;
    }
  }
}

size_t a8_buffer_bytes(int32_t batch, int32_t K) {
  return static_cast<size_t>(batch) * K + a8_meta_bytes(batch, K / kGroup);
}

hipError_t launch_quantize_a8(const void* x, int32_t batch, int32_t K, void* xq, hipStream_t s) {
  const int teams = batch * (K / kGroup);
  quantize_a8_kernel<<<dim3((teams * 16 + 255) / 256), dim3(256), 0, s>>>(static_cast<const half_t*>(x), batch, K,
                                                                          static_cast<uint8_t*>(xq));
  return hipGetLastError();
}

struct A8Shape {
  int tpw, ks;
  size_t lds;
};

// Launch shape as for the W4A16 GEMV: short K-slices for few tiles, two tiles
// by two slices for many.
static A8Shape a8_shape(int T, int G, int K, int B, bool qin) {
  A8Shape s;
  if (T >= 1024) {
    s.ks = B >= 4 ? 1 : 2;
    s.tpw = B >= 4 ? 8 : 2;
  } else {
    s.ks = std::min(8, (G + 6) / 7);
    s.tpw = T >= 256 ? 2 : 1;
  }
  s.ks = std::max(1, std::min(s.ks, G));
  const int nw = s.tpw * s.ks;
  s.lds = static_cast<size_t>(B) * K + a8_meta_bytes(B, G) + 128 +
          static_cast<size_t>(nw) * B * 16 * 4 + (qin ? static_cast<size_t>(B) * K * 2 : 0);
  return s;
}

constexpr size_t kA8MaxLds = 150 * 1024;

bool a8_fused_fits(int32_t N, int32_t K, int32_t batch) {
  return a8_shape(static_cast<int>(tiles_of(N)), K / kGroup, K, batch, true).lds <= kA8MaxLds;
}

template <int B, int EPI, bool QIN>
static hipError_t launch_a8_kernel(dim3 grid, dim3 block, size_t lds, hipStream_t s, const A8Params& p) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_w4a8_kernel<B, EPI, QIN>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  gemv_w4a8_kernel<B, EPI, QIN><<<grid, block, lds, s>>>(p);
  return hipGetLastError();
}

template <int B, bool QIN>
static hipError_t launch_a8_e(int epi, dim3 grid, dim3 block, size_t lds, hipStream_t s, const A8Params& p) {
  switch (epi) {
    case NQ_EPI_STORE_F16: return launch_a8_kernel<B, NQ_EPI_STORE_F16, QIN>(grid, block, lds, s, p);
    case NQ_EPI_BIAS_F16: return launch_a8_kernel<B, NQ_EPI_BIAS_F16, QIN>(grid, block, lds, s, p);
    case NQ_EPI_RESIDUAL_F16: return launch_a8_kernel<B, NQ_EPI_RESIDUAL_F16, QIN>(grid, block, lds, s, p);
    case NQ_EPI_SWIGLU_F16: return launch_a8_kernel<B, NQ_EPI_SWIGLU_F16, QIN>(grid, block, lds, s, p);
    case NQ_EPI_STORE_F32: return launch_a8_kernel<B, NQ_EPI_STORE_F32, QIN>(grid, block, lds, s, p);
    default: return hipErrorInvalidValue;
  }
}

template <bool QIN>
static hipError_t launch_a8_b(int batch, int epi, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                              const A8Params& p) {
  switch (batch) {
    case 1: return launch_a8_e<1, QIN>(epi, grid, block, lds, s, p);
    case 2: return launch_a8_e<2, QIN>(epi, grid, block, lds, s, p);
    case 3: return launch_a8_e<3, QIN>(epi, grid, block, lds, s, p);
    case 4: return launch_a8_e<4, QIN>(epi, grid, block, lds, s, p);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_w4a8(const void* packed, int32_t N, int32_t K, int32_t kind, int32_t head_dim, int32_t batch,
                            const void* x, const void* xq, const void* bias, void* y, int epi, hipStream_t s) {
  A8Params p{};
  p.codes = static_cast<const uint8_t*>(packed);
  p.scales = p.codes + codes_bytes(N, K);
  p.N = N;
  p.K = K;
  p.kind = kind;
  p.head_dim = head_dim;
  p.G = K / kGroup;
  p.T = static_cast<int>(tiles_of(N));
  p.x = static_cast<const half_t*>(x);
  p.xq = static_cast<const uint8_t*>(xq);
  p.bias = static_cast<const half_t*>(bias);
  p.y = y;
  const bool qin = xq == nullptr;
  const A8Shape sh = a8_shape(p.T, p.G, K, batch, qin);
  if (sh.lds > kA8MaxLds) return hipErrorInvalidValue;
  p.tpw = sh.tpw;
  p.ks = sh.ks;
  const dim3 grid((p.T + sh.tpw - 1) / sh.tpw), block(sh.tpw * sh.ks * 64);
  return qin ? launch_a8_b<true>(batch, epi, grid, block, sh.lds, s, p)
             : launch_a8_b<false>(batch, epi, grid, block, sh.lds, s, p);
}

}  // namespace nq
