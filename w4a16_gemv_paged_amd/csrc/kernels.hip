// HIP kernels of libnq for CDNA4 (gfx950), wave64.
//
// * W4A16 GEMV (fused Q/K/V/O and gate/up/down projections and the LM head;
//   "How to build your own LLM runtime from scratch", section "What it actually
//   builds"): packed INT4 tiles streamed with one 1 KiB coalesced load per wave
//   and group, nibbles turned into exact fp16 codes in registers, v_dot2_f32_f16
//   against fp16 activations staged in LDS, fp32 accumulation, the group scale
//   applied to the fp32 partial sum, and fused epilogues (bias + RoPE + KV-page
//   append, residual add, SwiGLU, fp32 logits + argmax partials).
// * Split-K paged decode attention ("What it actually builds": 16-token pages;
//   daily.dev FAQ on the barrier inside a warp-id branch): each wave stages its
//   own K/V pages in its own LDS slice and synchronises only itself; the single
//   block-wide barrier sits in uniform control flow after the page loop, so
//   partial tail pages are masked by position, never by a divergent barrier.
// * Small kernels: embedding gather, KV append, argmax finalize, device unpack.
#include <algorithm>

#include "common.hpp"

namespace nq {

typedef _Float16 half_t;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

// ORs error bits into the optional device flag.
__device__ __forceinline__ void raise_flag(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
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
// gives 1024 + 16n; (1024 + 16n) / 16 - 72 = n - 8, also exact.
__device__ __forceinline__ void unpack8(uint32_t w, h2 (&o)[4]) {
  const uint32_t magic = 0x64006400u;
  const h2 off_lo = {static_cast<half_t>(-1032.0f), static_cast<half_t>(-1032.0f)};
  const h2 sixteenth = {static_cast<half_t>(0.0625f), static_cast<half_t>(0.0625f)};
  const h2 off_hi = {static_cast<half_t>(-72.0f), static_cast<half_t>(-72.0f)};
  const uint32_t w8 = w >> 8;
  o[0] = as_h2((w & 0x000F000Fu) | magic) + off_lo;
  o[1] = __builtin_elementwise_fma(as_h2((w & 0x00F000F0u) | magic), sixteenth, off_hi);
  o[2] = as_h2((w8 & 0x000F000Fu) | magic) + off_lo;
  o[3] = __builtin_elementwise_fma(as_h2((w8 & 0x00F000F0u) | magic), sixteenth, off_hi);
}

__device__ __forceinline__ float dot2(h2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(a, as_h2(b), c, false);
}

// ============================================================== GEMV

struct GemvParams {
  const uint4* codes;
  const half_t* scales;
  int N, K, kind, head_dim, G, T, tpw, ks, ch;
  const half_t* x;
  const half_t* gain;
  float eps;
  const half_t* bias;
  void* y;
  half_t* y2;
  int epi;
  float* amax_val;
  int32_t* amax_idx;
  const int32_t* pos;
  const int32_t* pt;
  int max_pages, num_pages, n_heads, n_kv;
  half_t* kv_k;
  half_t* kv_v;
  const float* rope;
  int max_pos;
  int32_t* err;
};

constexpr int kUnroll = 8;

template <int B>
__device__ __forceinline__ void gemv_group(const uint4& wv, half_t s, const half_t* xs, int xstride,
                                           int gl, int kq, float (&acc)[B]) {
  h2 q[4][4];
  unpack8(wv.x, q[0]);
  unpack8(wv.y, q[1]);
  unpack8(wv.z, q[2]);
  unpack8(wv.w, q[3]);
  const float sf = static_cast<float>(s);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const uint4* xv = reinterpret_cast<const uint4*>(xs + b * xstride + gl * 128 + kq * 32);
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 xx = xv[j];
      p = dot2(q[j][0], xx.x, p);
      p = dot2(q[j][1], xx.y, p);
      p = dot2(q[j][2], xx.z, p);
      p = dot2(q[j][3], xx.w, p);
    }
    acc[b] = fmaf(p, sf, acc[b]);
  }
}

template <int B>
__global__ __launch_bounds__(1024) void gemv_w4a16_kernel(GemvParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const int tl = wave / p.ks, ksi = wave % p.ks;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * p.tpw + tl;
  const bool tile_ok = t < p.T;  // wave-uniform
  const int xstride = p.ch * 128;
  half_t* xs = reinterpret_cast<half_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + static_cast<size_t>(B) * xstride * 2);
  float* rs = red + nw * B * 16;
  float* lg = rs + B;  // [tpw][B][16] logits for the argmax partials

  if (p.gain) {
    float ss[B];
#pragma unroll
    for (int b = 0; b < B; ++b) ss[b] = 0.0f;
    for (int i = tid; i < p.K / 8; i += blockDim.x) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint4 v = *reinterpret_cast<const uint4*>(p.x + static_cast<int64_t>(b) * p.K + i * 8);
        const half_t* hv = reinterpret_cast<const half_t*>(&v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = static_cast<float>(hv[e]);
          ss[b] = fmaf(f, f, ss[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = ss[b];
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0) red[wave * B + b] = v;
    }
    __syncthreads();
    if (tid < B) {
      float v = 0.0f;
      for (int w = 0; w < nw; ++w) v += red[w * B + tid];
      rs[tid] = 1.0f / sqrtf(v / static_cast<float>(p.K) + p.eps);
    }
  }

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;

  for (int c0 = 0; c0 < p.G; c0 += p.ch) {
    const int c1 = min(p.G, c0 + p.ch);
    const int n8 = (c1 - c0) * 16;  // 16-byte items per batch row in this chunk
    __syncthreads();
    for (int i = tid; i < B * n8; i += blockDim.x) {
      const int b = i / n8, j = i - b * n8;
      const int64_t k = static_cast<int64_t>(c0) * 128 + j * 8;
      uint4 v = *reinterpret_cast<const uint4*>(p.x + static_cast<int64_t>(b) * p.K + k);
      if (p.gain) {
        const uint4 gv = *reinterpret_cast<const uint4*>(p.gain + k);
        half_t* hv = reinterpret_cast<half_t*>(&v);
        const half_t* gh = reinterpret_cast<const half_t*>(&gv);
        const float sc = rs[b];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          hv[e] = static_cast<half_t>(static_cast<float>(hv[e]) * sc * static_cast<float>(gh[e]));
      }
      *reinterpret_cast<uint4*>(xs + b * xstride + j * 8) = v;
    }
    __syncthreads();
    if (tile_ok) {
      const uint4* wp = p.codes + static_cast<size_t>(t) * p.G * 64 + lane;
      const half_t* sp = p.scales + static_cast<size_t>(t) * p.G * 16 + r;
      int g = c0 + ksi;
      for (; g + (kUnroll - 1) * p.ks < c1; g += kUnroll * p.ks) {
        uint4 wv[kUnroll];
        half_t sv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          wv[u] = wp[static_cast<size_t>(g + u * p.ks) * 64];
          sv[u] = sp[static_cast<size_t>(g + u * p.ks) * 16];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) gemv_group<B>(wv[u], sv[u], xs, xstride, g + u * p.ks - c0, kq, acc);
      }
      for (; g < c1; g += p.ks) {
        const uint4 wv = wp[static_cast<size_t>(g) * 64];
        const half_t sv = sp[static_cast<size_t>(g) * 16];
        gemv_group<B>(wv, sv, xs, xstride, g - c0, kq, acc);
      }
    }
  }

  // sum the four K quarters of each row, then hand the wave's rows to LDS
#pragma unroll
  for (int b = 0; b < B; ++b) {
    acc[b] += __shfl_xor(acc[b], 16);
    acc[b] += __shfl_xor(acc[b], 32);
  }
  __syncthreads();  // xs and red may be reused below
  if (lane < 16) {
#pragma unroll
    for (int b = 0; b < B; ++b) red[(wave * B + b) * 16 + r] = acc[b];
  }
  __syncthreads();

  const int items = p.tpw * B * 16;
  for (int i = tid; i < items; i += blockDim.x) {
    const int tl2 = i / (B * 16), b = (i / 16) % B, rr = i & 15;
    const int64_t tt = static_cast<int64_t>(blockIdx.x) * p.tpw + tl2;
    if (tt >= p.T) continue;
    float yv = 0.0f, yp = 0.0f;
    for (int k2 = 0; k2 < p.ks; ++k2) {
      yv += red[((tl2 * p.ks + k2) * B + b) * 16 + rr];
      yp += red[((tl2 * p.ks + k2) * B + b) * 16 + (rr ^ 8)];
    }
    const int64_t n = tile_row_logical(p.kind, p.N, p.head_dim, tt, rr);
    const int64_t N = p.N;
    switch (p.epi) {
      case NQ_EPI_STORE_F16:
        if (n < N) static_cast<half_t*>(p.y)[b * N + n] = static_cast<half_t>(yv);
        break;
      case NQ_EPI_BIAS_F16:
        if (n < N) static_cast<half_t*>(p.y)[b * N + n] = static_cast<half_t>(yv + static_cast<float>(p.bias[n]));
        break;
      case NQ_EPI_RESIDUAL_F16:
        if (n < N) {
          half_t* yo = static_cast<half_t*>(p.y) + b * N + n;
          const half_t v = static_cast<half_t>(static_cast<float>(*yo) + yv);
          *yo = v;
          if (p.y2) p.y2[b * N + n] = v;
        }
        break;
      case NQ_EPI_SWIGLU_F16:
        if (rr < 8) {
          const int64_t I = N / 2;
          const float a = yv / (1.0f + expf(-yv)) * yp;
          static_cast<half_t*>(p.y)[b * I + 8 * tt + rr] = static_cast<half_t>(a);
        }
        break;
      case NQ_EPI_STORE_F32:
        if (n < N && p.y) static_cast<float*>(p.y)[b * N + n] = yv;
        lg[(tl2 * B + b) * 16 + rr] = (n < N) ? yv : -INFINITY;
        break;
      case EPI_QKV_ROPE_KV: {
        const int d = p.head_dim, half = d / 2;
        const int hb = static_cast<int>(n / d), i2 = static_cast<int>(n % d);
        const half_t v16 = static_cast<half_t>(yv + static_cast<float>(p.bias[n]));
        const int ps = p.pos[b];
        half_t outv = v16;
        if (hb < p.n_heads + p.n_kv) {
          const int64_t np = tile_row_logical(p.kind, p.N, p.head_dim, tt, rr ^ 8);
          const half_t p16 = static_cast<half_t>(yp + static_cast<float>(p.bias[np]));
          if (ps < 0 || ps >= p.max_pos) {
            raise_flag(p.err, 1);
            break;
          }
          const int j = i2 % half;
          const float c = p.rope[(static_cast<int64_t>(ps) * half + j) * 2];
          const float sn = p.rope[(static_cast<int64_t>(ps) * half + j) * 2 + 1];
          const float xi = static_cast<float>(v16), xp = static_cast<float>(p16);
          outv = static_cast<half_t>(i2 < half ? xi * c - xp * sn : xi * c + xp * sn);
        }
        if (hb < p.n_heads) {
          static_cast<half_t*>(p.y)[(static_cast<int64_t>(b) * p.n_heads + hb) * d + i2] = outv;
        } else {
          const bool is_k = hb < p.n_heads + p.n_kv;
          const int kvh = is_k ? hb - p.n_heads : hb - p.n_heads - p.n_kv;
          const int pg = ps / kPageTokens;
          if (ps < 0 || pg >= p.max_pages) {
            raise_flag(p.err, 1);
            break;
          }
          const int page = p.pt[static_cast<int64_t>(b) * p.max_pages + pg];
          if (page < 0 || page >= p.num_pages) {
            raise_flag(p.err, 1);
            break;
          }
          half_t* base = is_k ? p.kv_k : p.kv_v;
          base[((static_cast<int64_t>(page) * p.n_kv + kvh) * kPageTokens + ps % kPageTokens) * d + i2] = outv;
        }
        break;
      }
      default:
        break;
    }
  }

  if (p.epi == NQ_EPI_STORE_F32 && p.amax_val) {
    __syncthreads();
    if (tid < p.tpw * B) {
      const int tl2 = tid / B, b = tid % B;
      const int64_t tt = static_cast<int64_t>(blockIdx.x) * p.tpw + tl2;
      if (tt < p.T) {
        float best = -INFINITY;
        int bi = 0x7fffffff;
        bool nan = false;
        for (int rr = 0; rr < 16; ++rr) {
          const float v = lg[(tl2 * B + b) * 16 + rr];
          const int n = static_cast<int>(tile_row_logical(p.kind, p.N, p.head_dim, tt, rr));
          if (v != v) { nan = true; continue; }
          if (n < p.N && (v > best || (v == best && n < bi))) { best = v; bi = n; }
        }
        if (nan) raise_flag(p.err, 8);
        p.amax_val[static_cast<int64_t>(b) * p.T + tt] = best;
        p.amax_idx[static_cast<int64_t>(b) * p.T + tt] = bi;
      }
    }
  }
}

struct GemvShape {
  int tpw, ks, ch, threads;
  size_t lds;
};

static GemvShape gemv_shape(int T, int G, int B) {
  GemvShape s;
  s.ks = std::min(16, std::max(1, (G + 6) / 7));
  s.tpw = 1;
  while (s.tpw * 2 * s.ks <= 16 && T / (s.tpw * 2) >= 1024) s.tpw *= 2;
  s.ch = std::min(G, std::max(1, (48 * 1024) / (B * 256)));
  s.threads = s.tpw * s.ks * 64;
  const int nw = s.tpw * s.ks;
  s.lds = static_cast<size_t>(B) * s.ch * 256 + static_cast<size_t>(nw) * B * 16 * 4 + B * 4 +
          static_cast<size_t>(s.tpw) * B * 16 * 4;
  return s;
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  GemvParams p{};
  p.N = a.N;
  p.K = a.K;
  p.kind = a.kind;
  p.head_dim = a.head_dim;
  p.G = a.K / kGroup;
  p.T = static_cast<int>(tiles_of(a.N));
  const GemvShape sh = gemv_shape(p.T, p.G, a.batch);
  p.tpw = sh.tpw;
  p.ks = sh.ks;
  p.ch = sh.ch;
  p.codes = static_cast<const uint4*>(a.packed);
  p.scales = reinterpret_cast<const half_t*>(static_cast<const uint8_t*>(a.packed) + codes_bytes(a.N, a.K));
  p.x = static_cast<const half_t*>(a.x);
  p.gain = static_cast<const half_t*>(a.norm_gain);
  p.eps = a.eps;
  p.bias = static_cast<const half_t*>(a.bias);
  p.y = a.y;
  p.y2 = static_cast<half_t*>(a.y2);
  p.epi = a.epi;
  p.amax_val = a.amax_val;
  p.amax_idx = a.amax_idx;
  p.pos = a.pos;
  p.pt = a.page_table;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.n_heads = a.n_heads;
  p.n_kv = a.n_kv;
  p.kv_k = static_cast<half_t*>(a.kv_k);
  p.kv_v = static_cast<half_t*>(a.kv_v);
  p.rope = a.rope;
  p.max_pos = a.max_pos;
  p.err = a.err;
  const dim3 grid((p.T + p.tpw - 1) / p.tpw), block(sh.threads);
  switch (a.batch) {
#define NQ_CASE(BB) \
  case BB: gemv_w4a16_kernel<BB><<<grid, block, sh.lds, stream>>>(p); break;
    NQ_CASE(1) NQ_CASE(2) NQ_CASE(3) NQ_CASE(4) NQ_CASE(5) NQ_CASE(6) NQ_CASE(7) NQ_CASE(8)
#undef NQ_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ============================================================== attention

constexpr int kMinPagesPerSplit = 2;
constexpr int kMaxSplits = 64;

int attn_splits_for(int32_t max_pages) {
  return std::max(1, std::min(kMaxSplits, (max_pages + kMinPagesPerSplit - 1) / kMinPagesPerSplit));
}

size_t attn_partial_bytes(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t splits) {
  return static_cast<size_t>(batch) * n_heads * splits * (head_dim + 2) * sizeof(float);
}

__device__ __forceinline__ void split_range(int len, int max_pages, int S, int s, int& p0, int& p1) {
  int npages = (len + kPageTokens - 1) / kPageTokens;
  npages = min(npages, max_pages);
  const int per = max(kMinPagesPerSplit, (npages + S - 1) / S);
  p0 = s * per;
  p1 = min(npages, p0 + per);
}

struct AttnParams {
  const half_t* q;
  const half_t* kp;
  const half_t* vp;
  const int32_t* pt;
  int max_pages, num_pages;
  const int32_t* lens;
  int len_add;
  half_t* out;
  float* po;
  float* pml;
  int n_heads, n_kv, S;
  int32_t* err;
};

// grid (S, n_kv, B), 256 threads = 4 waves. Wave w walks pages p0+w, p0+w+4, ...
template <int D, int REP>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnParams a) {
  constexpr int DC = D / 4;       // dims per lane in the score phase
  constexpr int DPL = D / 64;     // dims per lane in the PV phase
  constexpr int PAGE_U4 = 16 * D * 2 / 16;  // uint4 per page
  constexpr int U4_PER_LANE = PAGE_U4 / 64;
  __shared__ __align__(16) half_t lk[4][16 * D];
  __shared__ __align__(16) half_t lv[4][16 * D];
  __shared__ float lp[4][REP][16];
  __shared__ float red_m[4][REP], red_l[4][REP];
  __shared__ float red_o[4][REP][D];

  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = lane >> 2, c = lane & 3;
  const int len = a.lens[b] + a.len_add;
  if (len > a.max_pages * kPageTokens) {
    if (s == 0 && tid == 0) raise_flag(a.err, 2);
  }
  int p0, p1;
  split_range(len, a.max_pages, a.S, s, p0, p1);
  if (len <= 0 || p0 >= p1) return;  // block-uniform

  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  h2 qr[REP][DC / 2];
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    const uint4* src = reinterpret_cast<const uint4*>(
        a.q + (static_cast<int64_t>(b) * a.n_heads + kvh * REP + h) * D + c * DC);
#pragma unroll
    for (int j = 0; j < DC / 8; ++j) {
      const uint4 v = src[j];
      qr[h][4 * j + 0] = as_h2(v.x);
      qr[h][4 * j + 1] = as_h2(v.y);
      qr[h][4 * j + 2] = as_h2(v.z);
      qr[h][4 * j + 3] = as_h2(v.w);
    }
  }
  float m[REP], l[REP], o[REP][DPL];
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.0f;
  }

  for (int pg = p0 + w; pg < p1; pg += 4) {  // wave-uniform trip count, no block barrier inside
    const int page = a.pt[static_cast<int64_t>(b) * a.max_pages + pg];
    const bool page_ok = page >= 0 && page < a.num_pages;
    if (!page_ok) {
      if (lane == 0) raise_flag(a.err, 2);
      continue;
    }
    const int valid = min(kPageTokens, len - pg * kPageTokens);
    const uint4* ksrc = reinterpret_cast<const uint4*>(a.kp + (static_cast<int64_t>(page) * a.n_kv + kvh) * 16 * D);
    const uint4* vsrc = reinterpret_cast<const uint4*>(a.vp + (static_cast<int64_t>(page) * a.n_kv + kvh) * 16 * D);
    uint4 kreg[U4_PER_LANE], vreg[U4_PER_LANE];
#pragma unroll
    for (int i = 0; i < U4_PER_LANE; ++i) {
      kreg[i] = ksrc[i * 64 + lane];
      vreg[i] = vsrc[i * 64 + lane];
    }
    wave_sync();  // every lane is done with the previous page's LDS
#pragma unroll
    for (int i = 0; i < U4_PER_LANE; ++i) {
      reinterpret_cast<uint4*>(lk[w])[i * 64 + lane] = kreg[i];
      reinterpret_cast<uint4*>(lv[w])[i * 64 + lane] = vreg[i];
    }
    wave_sync();

    // scores: lane (t, c) covers token t, dims [c*DC, c*DC + DC)
    float sc[REP];
    const uint4* kr = reinterpret_cast<const uint4*>(lk[w] + t * D + c * DC);
#pragma unroll
    for (int h = 0; h < REP; ++h) sc[h] = 0.0f;
#pragma unroll
    for (int j = 0; j < DC / 8; ++j) {
      const uint4 kk = kr[j];
#pragma unroll
      for (int h = 0; h < REP; ++h) {
        sc[h] = dot2(qr[h][4 * j + 0], kk.x, sc[h]);
        sc[h] = dot2(qr[h][4 * j + 1], kk.y, sc[h]);
        sc[h] = dot2(qr[h][4 * j + 2], kk.z, sc[h]);
        sc[h] = dot2(qr[h][4 * j + 3], kk.w, sc[h]);
      }
    }
    float pr[REP];
#pragma unroll
    for (int h = 0; h < REP; ++h) {
      float v = sc[h];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v = (t < valid) ? v * scale : -INFINITY;
      float mx = v;
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      mx = fmaxf(mx, __shfl_xor(mx, 8));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[h], mx);
      const float alpha = expf(m[h] - mnew);
      pr[h] = expf(v - mnew);
      l[h] = l[h] * alpha + (c == 0 ? pr[h] : 0.0f);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[h][e] *= alpha;
      m[h] = mnew;
    }
    if (c == 0) {
#pragma unroll
      for (int h = 0; h < REP; ++h) lp[w][h][t] = pr[h];
    }
    wave_sync();
    // PV: lane owns dims [lane*DPL, lane*DPL + DPL)
#pragma unroll 4
    for (int t2 = 0; t2 < kPageTokens; ++t2) {
      float vv[DPL];
      if (DPL == 2) {
        const h2 v2 = *reinterpret_cast<const h2*>(lv[w] + t2 * D + lane * 2);
        vv[0] = static_cast<float>(v2[0]);
        vv[DPL - 1] = static_cast<float>(v2[1]);
      } else {
        vv[0] = static_cast<float>(lv[w][t2 * D + lane]);
      }
      const bool ok = t2 < valid;
#pragma unroll
      for (int e = 0; e < DPL; ++e) vv[e] = ok ? vv[e] : 0.0f;
#pragma unroll
      for (int h = 0; h < REP; ++h) {
        const float pv = lp[w][h][t2];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[h][e] = fmaf(pv, vv[e], o[h][e]);
      }
    }
  }

  // combine the four waves (uniform control flow: every wave reaches the barrier)
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    float v = l[h];
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) {
      red_m[w][h] = m[h];
      red_l[w][h] = v;
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) red_o[w][h][lane * DPL + e] = o[h][e];
  }
  __syncthreads();
  for (int i = tid; i < REP * D; i += 256) {
    const int h = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, red_m[ww][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = (red_m[ww][h] == -INFINITY) ? 0.0f : expf(red_m[ww][h] - M);
      L = fmaf(f, red_l[ww][h], L);
      O = fmaf(f, red_o[ww][h][d], O);
    }
    const int64_t row = (static_cast<int64_t>(b) * a.n_heads + kvh * REP + h) * a.S + s;
    a.po[row * D + d] = O;
    if (d == 0) {
      a.pml[row * 2] = M;
      a.pml[row * 2 + 1] = L;
    }
  }
}

// grid (n_heads, B), D threads
template <int D>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnParams a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int len = a.lens[b] + a.len_add;
  half_t* out = a.out + (static_cast<int64_t>(b) * a.n_heads + h) * D;
  if (len <= 0) {
    out[d] = static_cast<half_t>(0.0f);
    return;
  }
  int npages = min((len + kPageTokens - 1) / kPageTokens, a.max_pages);
  const int per = max(kMinPagesPerSplit, (npages + a.S - 1) / a.S);
  const int nact = (npages + per - 1) / per;
  const int64_t row0 = (static_cast<int64_t>(b) * a.n_heads + h) * a.S;
  float M = -INFINITY;
  for (int s = 0; s < nact; ++s) M = fmaxf(M, a.pml[(row0 + s) * 2]);
  float L = 0.0f, O = 0.0f;
  for (int s = 0; s < nact; ++s) {
    const float ms = a.pml[(row0 + s) * 2];
    const float f = (ms == -INFINITY) ? 0.0f : expf(ms - M);
    L = fmaf(f, a.pml[(row0 + s) * 2 + 1], L);
    O = fmaf(f, a.po[(row0 + s) * D + d], O);
  }
  out[d] = static_cast<half_t>(L > 0.0f ? O / L : 0.0f);
}

template <int D, int REP>
static void launch_attn_t(const AttnParams& p, int batch, hipStream_t s) {
  attn_split_kernel<D, REP><<<dim3(p.S, p.n_kv, batch), dim3(256), 0, s>>>(p);
  attn_combine_kernel<D><<<dim3(p.n_heads, batch), dim3(D), 0, s>>>(p);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  AttnParams p{};
  p.q = static_cast<const half_t*>(a.q);
  p.kp = static_cast<const half_t*>(a.k_pool);
  p.vp = static_cast<const half_t*>(a.v_pool);
  p.pt = a.page_table;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.lens = a.lens;
  p.len_add = a.len_add;
  p.out = static_cast<half_t*>(a.out);
  p.po = a.part_o;
  p.pml = a.part_ml;
  p.n_heads = a.n_heads;
  p.n_kv = a.n_kv;
  p.S = a.splits;
  p.err = a.err;
  const int rep = a.n_heads / a.n_kv;
#define NQ_ATT(DD, RR) \
  if (a.head_dim == DD && rep == RR) { launch_attn_t<DD, RR>(p, a.batch, s); return hipGetLastError(); }
  NQ_ATT(128, 7) NQ_ATT(128, 8) NQ_ATT(128, 4) NQ_ATT(128, 2) NQ_ATT(128, 1)
  NQ_ATT(64, 4) NQ_ATT(64, 7) NQ_ATT(64, 8) NQ_ATT(64, 2) NQ_ATT(64, 1)
#undef NQ_ATT
  return hipErrorInvalidValue;
}

// ============================================================== small kernels

// grid (B), 64 * ceil(n_kv * d / 8 / 64) threads: one 16-byte item per thread
__global__ void kv_append_kernel(half_t* kp, half_t* vp, int n_kv, int d, const int32_t* pt,
                                 int max_pages, int num_pages, const int32_t* pos,
                                 const half_t* k, const half_t* v, int32_t* err) {
  const int b = blockIdx.x;
  const int ps = pos[b];
  const int pg = ps / kPageTokens;
  if (ps < 0 || pg >= max_pages) {
    if (threadIdx.x == 0) raise_flag(err, 1);
    return;
  }
  const int page = pt[static_cast<int64_t>(b) * max_pages + pg];
  if (page < 0 || page >= num_pages) {
    if (threadIdx.x == 0) raise_flag(err, 1);
    return;
  }
  const int items = n_kv * d / 8;
  for (int i = threadIdx.x; i < items; i += blockDim.x) {
    const int h = (i * 8) / d, e = (i * 8) % d;
    const int64_t dst = ((static_cast<int64_t>(page) * n_kv + h) * kPageTokens + ps % kPageTokens) * d + e;
    const int64_t src = (static_cast<int64_t>(b) * n_kv + h) * d + e;
    *reinterpret_cast<uint4*>(kp + dst) = *reinterpret_cast<const uint4*>(k + src);
    *reinterpret_cast<uint4*>(vp + dst) = *reinterpret_cast<const uint4*>(v + src);
  }
}

hipError_t launch_kv_append(void* k_pool, void* v_pool, int32_t batch, int32_t n_kv, int32_t head_dim,
                            const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                            const int32_t* pos, const void* k, const void* v, int32_t* err,
                            hipStream_t s) {
  kv_append_kernel<<<dim3(batch), dim3(64), 0, s>>>(
      static_cast<half_t*>(k_pool), static_cast<half_t*>(v_pool), n_kv, head_dim, page_table, max_pages,
      num_pages, pos, static_cast<const half_t*>(k), static_cast<const half_t*>(v), err);
  return hipGetLastError();
}

__global__ void embed_kernel(const half_t* E, int vocab, int H, const int32_t* tokens, half_t* h,
                             int32_t* err) {
  const int b = blockIdx.x;
  int tok = tokens[b];
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0) raise_flag(err, 4);
    tok = 0;
  }
  const uint4* src = reinterpret_cast<const uint4*>(E + static_cast<int64_t>(tok) * H);
  uint4* dst = reinterpret_cast<uint4*>(h + static_cast<int64_t>(b) * H);
  for (int i = threadIdx.x; i < H / 8; i += blockDim.x) dst[i] = src[i];
}

hipError_t launch_embed(const void* embed, int32_t vocab, int32_t hidden, const int32_t* tokens,
                        int32_t batch, void* h, int32_t* err, hipStream_t s) {
  embed_kernel<<<dim3(batch), dim3(256), 0, s>>>(static_cast<const half_t*>(embed), vocab, hidden, tokens,
                                                 static_cast<half_t*>(h), err);
  return hipGetLastError();
}

// grid (B), 256 threads: reduce per-tile (max, lowest index) partials.
__global__ __launch_bounds__(256) void argmax_finalize_kernel(const float* vals, const int32_t* idx,
                                                              int T, int* tokens, int* pos, int* hist,
                                                              int hist_len) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int t = tid; t < T; t += 256) {
    const float v = vals[static_cast<int64_t>(b) * T + t];
    const int i = idx[static_cast<int64_t>(b) * T + t];
    if (v > best || (v == best && i < bi)) { best = v; bi = i; }
  }
  sv[tid] = best;
  si[tid] = bi;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if (tid < off) {
      const float v = sv[tid + off];
      const int i = si[tid + off];
      if (v > sv[tid] || (v == sv[tid] && i < si[tid])) { sv[tid] = v; si[tid] = i; }
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int tok = si[0] == 0x7fffffff ? 0 : si[0];
    const int p = pos[b];
    tokens[b] = tok;
    if (hist && p + 1 >= 0 && p + 1 < hist_len) hist[static_cast<int64_t>(b) * hist_len + p + 1] = tok;
    pos[b] = p + 1;
  }
}

hipError_t launch_argmax_finalize(const float* vals, const int32_t* idx, int32_t tiles, int32_t batch,
                                  int32_t /*vocab*/, int32_t* tokens, int32_t* pos, int32_t* hist,
                                  int32_t hist_len, int32_t* /*err*/, hipStream_t s) {
  argmax_finalize_kernel<<<dim3(batch), dim3(256), 0, s>>>(vals, idx, tiles, tokens, pos, hist, hist_len);
  return hipGetLastError();
}

// grid (T * G), 64 threads: decode block (t, g) with the GEMV's unpack.
__global__ void unpack_dev_kernel(const uint4* codes, const uint16_t* scales, int N, int K, int kind,
                                  int head_dim, int G, int8_t* q_out, uint16_t* s_out) {
  const int64_t blk = blockIdx.x;
  const int64_t t = blk / G;
  const int g = static_cast<int>(blk % G);
  const int lane = threadIdx.x, r = lane & 15, kq = lane >> 4;
  const int64_t n = tile_row_logical(kind, N, head_dim, t, r);
  if (n >= N) return;
  const uint4 wv = codes[blk * 64 + lane];
  const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
  int8_t* dst = q_out + n * static_cast<int64_t>(K) + static_cast<int64_t>(g) * 128 + kq * 32;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h2 q[4];
    unpack8(words[j], q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[8 * j + 2 * i] = static_cast<int8_t>(static_cast<float>(q[i][0]));
      dst[8 * j + 2 * i + 1] = static_cast<int8_t>(static_cast<float>(q[i][1]));
    }
  }
  if (kq == 0) s_out[n * G + g] = scales[blk * 16 + r];
}

hipError_t launch_unpack_dev(const void* packed, int32_t N, int32_t K, int32_t kind, int32_t head_dim,
                             int8_t* q_out, uint16_t* s_out, hipStream_t s) {
  const int G = K / kGroup;
  const int64_t T = tiles_of(N);
  const uint16_t* scales =
      reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) + codes_bytes(N, K));
  unpack_dev_kernel<<<dim3(static_cast<unsigned>(T * G)), dim3(64), 0, s>>>(
      static_cast<const uint4*>(packed), scales, N, K, kind, head_dim, G, q_out, s_out);
  return hipGetLastError();
}

}  // namespace nq
