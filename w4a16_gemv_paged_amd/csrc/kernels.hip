// HIP kernels of libnq for CDNA4 (gfx950), wave64.
//
// * W4A16 GEMV (fused Q/K/V/O and gate/up/down projections and the LM head;
//   "How to build your own LLM runtime from scratch", section "What it actually
//   builds"): packed INT4 tiles streamed with one 1 KiB coalesced buffer load
//   per wave and group, nibbles turned into exact fp16 codes in registers, the
//   multiply-accumulate on the matrix cores (v_mfma_f32_16x16x32_f16, the
//   batch in the MFMA columns) against fp16 activations staged in LDS, the
//   group scale applied to the fp32 partial sums, and fused epilogues (bias +
//   RoPE + KV-page append, residual add, SwiGLU, fp32 logits + argmax partials).
// * Split-K paged decode attention ("What it actually builds": 16-token pages;
//   daily.dev FAQ on the barrier inside a warp-id branch): scores and P.V on
//   the matrix cores with the GQA query heads as the MFMA columns, K and V
//   pages read straight into operand registers, one online softmax per lane;
//   the single block-wide barrier sits in uniform control flow after the page
//   loop, so partial tail pages are masked by position, never by a divergent
//   barrier.
// * Small kernels: embedding gather, KV append, argmax finalize, device unpack.
#include <algorithm>

#include "device.hpp"

namespace nq {

// ============================================================== GEMV
//
// Work split: the T = N/16 row tiles of the packed matrix are cut into
// (tile, K-slice) pieces; a workgroup holds tpw tiles x ks K-slices, one wave
// each. A wave walks the 1 KiB (tile, group) blocks of its slice, groups
// g = slice + ks*i, keeping kDepth buffer loads in flight (a ring refilled as
// each block is consumed). Each block is 16 rows x 128 K: lane l holds row
// l%16 and K range 32*(l/16)..+31, i.e. one 16x16x32 MFMA A-fragment per
// 32-bit word. The activations sit in LDS as the MFMA B operand (column =
// batch row, zero beyond the batch). Per group the four MFMA partial sums of a
// row are scaled by that row's fp16 group scale in fp32. Slices of a tile are
// summed through LDS, then the fused epilogue runs on (tile, batch, row) items.

// 1 KiB weight loads in flight per wave. With the ring kept full (below), 5
// beat the earlier 7 on one box: batch-8 decode step 2.557 against 2.607 ms,
// GEMV sweep aggregate 44.9% against 43.4% of 8 TB/s at batch 1 and 41.6%
// against 39.9% at batch 4; 3, 4 and 6 came within 0.01 ms of 5 at batch 8,
// 9 and 11 were slower (2.648, 2.688 ms).
constexpr int kDepth = 5;
constexpr int kGemvCUs = 256;               // MI355X compute units: one workgroup each in an even spread
constexpr size_t kLdsMax = 160 * 1024;      // LDS of a workgroup on gfx950
constexpr size_t kLdsX = 152 * 1024;        // LDS budget for staged activations and gain
// Staged rows of a batch > 1 are padded by 16 bytes, so that the rows' items at
// the same K start in different LDS banks: the matrix-core reads of the batch
// columns and the RMSNorm pass read one K offset of every row at once.
constexpr int kRowPad = 8;

struct GemvParams {
  const uint8_t* codes;
  const uint8_t* scales;
  int N, K, kind, head_dim, G, T, tpw, ks, ch, xrow;
  int bal;  // tiles spread evenly over the grid (9 or 10 of 2368 over 256 workgroups), else tpw each
  const half_t* x;
  const half_t* gain;
  float eps;
  const half_t* bias;
  void* y;
  half_t* y2;
  // embedding gather folded into the prologue: x row b = embed[tokens[b]], and
  // workgroup 0 also stores it to h_out (the residual stream)
  const half_t* embed;
  const int32_t* tokens_in;
  int vocab;
  half_t* h_out;
  // LM head: per-workgroup greedy (max, index) partials [B][gridDim.x]
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

// The 16x16x32 MFMAs over one (tile, group) block: d[i] = sum over the
// group's 128 K of q[row 4*(l/16)+i][k] * x[col l%16][k] (unscaled), from the
// biased codes: per K step one product with the constant -bias fragment (it
// needs only x, so the first one goes ahead of the weights) and one with the
// codes. The activations are pre-scaled in LDS when PRESCALED (the RMSNorm
// pass does it for free), else here in registers.
template <bool PRESCALED>
__device__ __forceinline__ f4 gemv_block_mfma(const u32x4& w, const half_t* xg, uint32_t magic, const half8& nbias) {
  f4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t xv[4];
    *reinterpret_cast<u32x4*>(xv) = *reinterpret_cast<const u32x4*>(xg + j * 8);
    if constexpr (!PRESCALED) scale_high_halves(xv);
    const half8 xb = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(xv));
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(nbias, xb, d, 0, 0, 0);
    h2 q[4];
    unpack8_biased(w[j], magic, q);
    const u32x4 qa = {__builtin_bit_cast(uint32_t, q[0]), __builtin_bit_cast(uint32_t, q[1]),
                      __builtin_bit_cast(uint32_t, q[2]), __builtin_bit_cast(uint32_t, q[3])};
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, qa), xb, d, 0, 0, 0);
  }
  return d;
}

// The RMSNorm prologue over the staged rows: x * gain in place, pre-scaled for
// the biased codes (fp16 products, as the GEMV forms them), and each wave's
// partial sum of x^2 per batch row (1/rms multiplies the outputs later).
// Thread t takes row t % BP (B rounded up to a power of two; threads of rows
// >= B stay idle) and every (blockDim / BP)-th 16-byte item of it, so a
// wave's partial sums of row b sit in the lanes congruent to b mod BP and
// log2(64 / BP) shuffle steps reduce every row at once. Returns, in lane b <
// B, the wave's sum for row b. h_out (if set) receives the rows as staged.
template <int B>
__device__ __forceinline__ float gain_rows(half_t* xs, int xrow, const half_t* gs, int n8, half_t* h_out,
                                           int64_t K, int64_t k0) {
  constexpr int BP = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8;
  static_assert(B <= 8, "batch rows");
  const int tid = threadIdx.x;
  const int b = tid % BP;
  const h2 sixteenth = {static_cast<half_t>(0.0625f), static_cast<half_t>(0.0625f)};
  float s = 0.0f;
  if (b < B) {
    for (int j = tid / BP; j < n8; j += blockDim.x / BP) {
      uint4 v = *reinterpret_cast<const uint4*>(xs + b * xrow + j * 8);
      const uint4 gv = *reinterpret_cast<const uint4*>(gs + j * 8);
      if (h_out) *reinterpret_cast<uint4*>(h_out + b * K + k0 + j * 8) = v;
      h2* x = reinterpret_cast<h2*>(&v);
      const h2* g = reinterpret_cast<const h2*>(&gv);
#pragma unroll
      for (int q = 0; q < 4; ++q) s = __builtin_amdgcn_fdot2(x[q], x[q], s, false);
      x[0] = x[0] * g[0];
      x[1] = (x[1] * g[1]) * sixteenth;
      x[2] = x[2] * g[2];
      x[3] = (x[3] * g[3]) * sixteenth;
      *reinterpret_cast<uint4*>(xs + b * xrow + j * 8) = v;
    }
  }
  for (int o = 32; o >= BP; o >>= 1) s += __shfl_xor(s, o);
  return s;
}

template <int B, int EPI, bool GAIN>
__global__ __launch_bounds__(1024) void gemv_w4a16_kernel(GemvParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = blockDim.x >> 6;
  const int col = lane & 15, kb = lane >> 4;
  const int tl = wave / p.ks, ksi = wave % p.ks;
  // this workgroup's tiles [t0, t1): tpw each, or an even share of the T tiles
  // (at most tpw) so that no CU gets a second workgroup's worth of work
  const int t0 = p.bal ? static_cast<int>(static_cast<int64_t>(blockIdx.x) * p.T / gridDim.x)
                       : static_cast<int>(blockIdx.x) * p.tpw;
  const int t1 = p.bal ? static_cast<int>((static_cast<int64_t>(blockIdx.x) + 1) * p.T / gridDim.x)
                       : min(p.T, t0 + p.tpw);
  const int t = t0 + tl;
  const bool tile_ok = t < t1;  // wave-uniform
  const int xrow = p.xrow;       // halfs per staged row: a multiple of 512 (1 KiB), padded at batch > 1
  // LDS: [B] activation rows | gain row (GAIN) | zero block | red | ssq | lg
  half_t* xs = reinterpret_cast<half_t*>(smem);
  half_t* gs = xs + B * xrow;
  half_t* zero = gs + (GAIN ? xrow : 0);
  float* red = reinterpret_cast<float*>(zero + 128);  // [nw][B][16]
  float* ssq = red + nw * B * 16;                      // [nw][B]
  float* lg = ssq + nw * B;                            // [tpw][B][16]
  const uint32_t magic = opaque(0x64006400u);
  const half8 nbias = neg_bias_frag();
  const int items = p.tpw * B * 16;

  // Inputs of the fused QKV epilogue (bias, position, RoPE cos/sin, page id)
  // do not depend on the GEMV: fetch them now, their latency hides under the
  // weight stream.
  float e_bias = 0.0f, e_pbias = 0.0f, e_cos = 1.0f, e_sin = 0.0f;
  int e_pos = 0, e_page = -1;
  if constexpr (EPI == EPI_QKV_ROPE_KV) {
    if (tid < items) {
      const int tl2 = tid / (B * 16), b = (tid / 16) % B, rr = tid & 15;
      const int64_t tt = static_cast<int64_t>(t0) + tl2;
      if (tt < t1) {
        const int64_t n = tile_row_logical(p.kind, p.N, p.head_dim, tt, rr);
        const int64_t np = tile_row_logical(p.kind, p.N, p.head_dim, tt, rr ^ 8);
        e_bias = static_cast<float>(p.bias[n]);
        e_pbias = static_cast<float>(p.bias[np]);
        e_pos = p.pos[b];
        const int half = p.head_dim / 2;
        if (e_pos >= 0 && e_pos < p.max_pos) {
          const int j = static_cast<int>(n % p.head_dim) % half;
          const float2 cs = *reinterpret_cast<const float2*>(p.rope + (static_cast<int64_t>(e_pos) * half + j) * 2);
          e_cos = cs.x;
          e_sin = cs.y;
        }
        const int pg = e_pos / kPageTokens;
        if (e_pos >= 0 && pg < p.max_pages) e_page = p.pt[static_cast<int64_t>(b) * p.max_pages + pg];
      }
    }
  }

  // The residual the epilogue adds to does not depend on the GEMV either.
  half_t e_res = static_cast<half_t>(0.0f);  // kept as loaded: converting it here would wait for it
  if constexpr (EPI == NQ_EPI_RESIDUAL_F16) {
    if (tid < items) {
      const int tl2 = tid / (B * 16), b = (tid / 16) % B, rr = tid & 15;
      const int64_t tt = static_cast<int64_t>(t0) + tl2;
      if (tt < t1) {
        const int64_t n = tile_row_logical(p.kind, p.N, p.head_dim, tt, rr);
        if (n < p.N) e_res = static_cast<const half_t*>(p.y)[b * static_cast<int64_t>(p.N) + n];
      }
    }
  }

  // Buffer descriptors over this tile's codes and scales: the per-group offset
  // is a scalar, the per-lane offset a constant; reads past the tile give 0.
  const int tq = tile_ok ? t : 0;
  const int wbytes = tile_ok ? p.G * kBlockBytes : 0, sbytes = tile_ok ? p.G * 32 : 0;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.codes) + static_cast<size_t>(tq) * p.G * kBlockBytes, 0, wbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.scales) + static_cast<size_t>(tq) * p.G * 32, 0, sbytes, kBufferFlags);
  const int wvoff = lane * 16;
  // B fragment of this lane: its batch row, or the zero block for columns >= B
  const half_t* xlane = (col < B ? xs + col * xrow : zero) + kb * 32;
  const int xstep = col < B ? 128 : 0;
  if (tid < 16) reinterpret_cast<uint4*>(zero)[tid] = make_uint4(0u, 0u, 0u, 0u);

  // input token ids (embedding gather in the prologue): lane b holds row b's
  int tok_lane = 0;
  if (p.embed) {
    tok_lane = lane < B ? p.tokens_in[lane] : 0;
    if (lane < B && (tok_lane < 0 || tok_lane >= p.vocab) && blockIdx.x == 0 && wave == 0) raise_flag(p.err, 4);
  }

  u32x4 wv[kDepth];
  f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float ss = 0.0f;  // lane b < B: this wave's sum of x^2 of row b over the chunks so far

  auto chunk = [&](const int c0) {
    const int c1 = min(p.G, c0 + p.ch);
    const int n_c = (c1 - c0 - ksi + p.ks - 1) / p.ks;  // this wave's groups in the chunk (may be <= 0)
    const int n8 = (c1 - c0) * 16;                      // 16-byte items per staged row
    const int rblk = (n8 + 63) / 64;                    // 1 KiB blocks per staged row
    if (c0 > 0) __syncthreads();                        // the previous chunk is consumed
    // (1) Activations (and gain) straight into LDS, one 1 KiB block per wave
    //     instruction, issued before the weights: the memory counter retires
    //     in order, so they can be waited for without waiting for the weights.
    //     Block j of every row goes to wave j mod nw; the row loop keeps the
    //     per-copy address work to increments.
#pragma unroll 1
    for (int r = 0; r < B + (GAIN ? 1 : 0); ++r) {
      const half_t* src;
      half_t* dst;
      if (r < B) {
        const half_t* xr = p.x + static_cast<int64_t>(r) * p.K;
        if (p.embed) {  // activation row r is the embedding row of the input token
          int tok = __builtin_amdgcn_readlane(tok_lane, r);
          if (tok < 0 || tok >= p.vocab) tok = 0;
          xr = p.embed + static_cast<int64_t>(tok) * p.K;
        }
        src = xr + static_cast<int64_t>(c0) * 128;
        dst = xs + r * xrow;
      } else {
        src = p.gain + static_cast<int64_t>(c0) * 128;
        dst = gs;
      }
      for (int j = wave; j < rblk; j += nw) {
        const int item = j * 64 + lane;
        if (item < n8) __builtin_amdgcn_global_load_lds(src + item * 8, dst + j * 512, 16, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // (2) The scale window of the first kDepth blocks and the weight ring:
    //     exactly kDepth + 1 loads per wave (absent groups read past the tile
    //     and return 0), so the wait below is exact. In a scale window, lane
    //     (row kb, column c < kDepth) holds the scales of rows 4kb..4kb+3 for
    //     block w0 + c; block i takes them from lane i % kDepth of its row. One
    //     64-lane load thus serves kDepth blocks instead of one.
    auto load_scales = [&](int w0) {
      const int bi = w0 + col;
      const int g = c0 + ksi + p.ks * bi;
      return __builtin_amdgcn_raw_buffer_load_b64(srs, (col < kDepth && bi < n_c) ? g * 32 + kb * 8 : sbytes, 0, kStreamOnce);
    };
    u32x2 swin = load_scales(0);
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const bool ok = u < n_c;
      const int g = c0 + ksi + p.ks * u;
      wv[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, wvoff, ok ? g * kBlockBytes : wbytes, kStreamOnce);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kDepth + 1));  // this wave's LDS writes have landed
    __builtin_amdgcn_s_barrier();                     // ... and every wave's
    __builtin_amdgcn_sched_barrier(0);
    // (3) x * gain in place, pre-scaled for the biased codes, and sum(x^2)
    //     (1/rms multiplies the outputs later); workgroup 0 also stores the
    //     gathered embedding rows as the residual
    if constexpr (GAIN) {
      ss += gain_rows<B>(xs, xrow, gs, n8, blockIdx.x == 0 ? p.h_out : nullptr, p.K, static_cast<int64_t>(c0) * 128);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // (4) the scale of block i is applied while block i+1 is on the matrix
    //     cores; the next scale window is requested a window ahead
    //     Windows with a later one refill every slot they consume (a block
    //     past the wave's last reads past the tile and returns 0), so every
    //     path has the same loads in flight and the compiler's wait for a
    //     block counts only what is older than it; the last window refills
    //     nothing.
    int ib = 0;
    for (; ib + kDepth < n_c; ib += kDepth) {
      const u32x2 snext = load_scales(ib + kDepth);
      f4 dprev;
      u32x2 sprev;
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int i = ib + u;
        const f4 d = gemv_block_mfma<GAIN>(wv[u], xlane + (ksi + p.ks * i) * xstep, magic, nbias);
        if (u > 0) scale_acc(acc, dprev, sprev);
        dprev = d;
        sprev = row_bcast2(swin, u);
        const int gn = c0 + ksi + p.ks * (i + kDepth);
        wv[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, wvoff, i + kDepth < n_c ? gn * kBlockBytes : wbytes,
                                                      kStreamOnce);
      }
      scale_acc(acc, dprev, sprev);
      swin = snext;
    }
    if (ib < n_c) {
      f4 dprev;
      u32x2 sprev;
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int i = ib + u;
        if (i < n_c) {
          const f4 d = gemv_block_mfma<GAIN>(wv[u], xlane + (ksi + p.ks * i) * xstep, magic, nbias);
          if (u > 0) scale_acc(acc, dprev, sprev);
          dprev = d;
          sprev = row_bcast2(swin, u);
        }
      }
      scale_acc(acc, dprev, sprev);
    }
  };
  if (p.ch >= p.G) {
    chunk(0);  // the whole K in one chunk: straight-line code, no loop-carried waits
  } else {
    for (int c0 = 0; c0 < p.G; c0 += p.ch) chunk(c0);
  }

  // per-wave partial sums of x^2, and the tile rows of this wave
  if constexpr (GAIN) {
    if (lane < B) ssq[wave * B + lane] = ss;
  }
  __syncthreads();  // every wave is done reading xs; red is free
  if (col < B) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * B + col) * 16 + 4 * kb + i] = acc[i];
  }
  __syncthreads();

  for (int i = tid; i < items; i += blockDim.x) {
    const int tl2 = i / (B * 16), b = (i / 16) % B, rr = i & 15;
    const int64_t tt = static_cast<int64_t>(t0) + tl2;
    if (tt >= t1) continue;
    float rsb = 1.0f;
    if constexpr (GAIN) {
      float v = 0.0f;
      for (int w = 0; w < nw; ++w) v += ssq[w * B + b];
      rsb = 1.0f / sqrtf(v / static_cast<float>(p.K) + p.eps);
    }
    float yv = 0.0f, yp = 0.0f;
    for (int k2 = 0; k2 < p.ks; ++k2) {
      yv += red[((tl2 * p.ks + k2) * B + b) * 16 + rr];
      yp += red[((tl2 * p.ks + k2) * B + b) * 16 + (rr ^ 8)];
    }
    yv *= rsb;
    yp *= rsb;
    const int64_t n = tile_row_logical(p.kind, p.N, p.head_dim, tt, rr);
    const int64_t N = p.N;
    if constexpr (EPI == NQ_EPI_STORE_F16) {
      if (n < N) static_cast<half_t*>(p.y)[b * N + n] = static_cast<half_t>(yv);
    } else if constexpr (EPI == NQ_EPI_BIAS_F16) {
      if (n < N) static_cast<half_t*>(p.y)[b * N + n] = static_cast<half_t>(yv + static_cast<float>(p.bias[n]));
    } else if constexpr (EPI == NQ_EPI_RESIDUAL_F16) {
      if (n < N) {
        half_t* yo = static_cast<half_t*>(p.y) + b * N + n;
        const float r = static_cast<float>(i == tid ? e_res : *yo);  // prefetched for item tid
        const half_t v = static_cast<half_t>(r + yv);
        *yo = v;
        if (p.y2) p.y2[b * N + n] = v;
      }
    } else if constexpr (EPI == NQ_EPI_SWIGLU_F16) {
      if (rr < 8) {
        const int64_t I = N / 2;
        const float a = yv / (1.0f + expf(-yv)) * yp;
        static_cast<half_t*>(p.y)[b * I + 8 * tt + rr] = static_cast<half_t>(a);
      }
    } else if constexpr (EPI == NQ_EPI_STORE_F32) {
      if (n < N && p.y) static_cast<float*>(p.y)[b * N + n] = yv;
      lg[(tl2 * B + b) * 16 + rr] = (n < N) ? yv : -INFINITY;
    } else if constexpr (EPI == EPI_QKV_ROPE_KV) {
      // prefetched values belong to item tid; further items (if any) load theirs here
      float bn = e_bias, bp = e_pbias, cs = e_cos, sn = e_sin;
      int ps = e_pos, page = e_page;
      const int d = p.head_dim, half = d / 2;
      const int hb = static_cast<int>(n / d), i2 = static_cast<int>(n % d);
      if (i != tid) {
        const int64_t np = tile_row_logical(p.kind, p.N, p.head_dim, tt, rr ^ 8);
        bn = static_cast<float>(p.bias[n]);
        bp = static_cast<float>(p.bias[np]);
        ps = p.pos[b];
        cs = 1.0f;
        sn = 0.0f;
        if (ps >= 0 && ps < p.max_pos) {
          cs = p.rope[(static_cast<int64_t>(ps) * half + i2 % half) * 2];
          sn = p.rope[(static_cast<int64_t>(ps) * half + i2 % half) * 2 + 1];
        }
        const int pg = ps / kPageTokens;
        page = (ps >= 0 && pg < p.max_pages) ? p.pt[static_cast<int64_t>(b) * p.max_pages + pg] : -1;
      }
      const half_t v16 = static_cast<half_t>(yv + bn);
      half_t outv = v16;
      bool ok = true;
      if (hb < p.n_heads + p.n_kv) {
        const half_t p16 = static_cast<half_t>(yp + bp);
        if (ps < 0 || ps >= p.max_pos) {
          raise_flag(p.err, 1);
          ok = false;
        } else {
          const float xi = static_cast<float>(v16), xp = static_cast<float>(p16);
          outv = static_cast<half_t>(i2 < half ? xi * cs - xp * sn : xi * cs + xp * sn);
        }
      }
      if (ok && hb < p.n_heads) {
        static_cast<half_t*>(p.y)[(static_cast<int64_t>(b) * p.n_heads + hb) * d + i2] = outv;
      } else if (ok) {
        const bool is_k = hb < p.n_heads + p.n_kv;
        const int kvh = is_k ? hb - p.n_heads : hb - p.n_heads - p.n_kv;
        if (page < 0 || page >= p.num_pages) {
          raise_flag(p.err, 1);
        } else {
          const int64_t blk = (static_cast<int64_t>(page) * p.n_kv + kvh) * kPageTokens * d;
          const int slot = ps % kPageTokens;
          if (is_k) {
            p.kv_k[blk + slot * d + i2] = outv;              // token-major
          } else {
            p.kv_v[blk + i2 * kPageTokens + slot] = outv;    // dim-major
          }
        }
      }
    }
  }

  if constexpr (EPI == NQ_EPI_STORE_F32) {
    if (p.amax_val) {
      __syncthreads();
      // this workgroup's best (value, index) per batch row
      if (tid < B) {
        const int b = tid;
        float best = -INFINITY;
        int bi = 0x7fffffff;
        bool nan = false;
        for (int tl2 = 0; tl2 < p.tpw; ++tl2) {
          const int64_t tt = static_cast<int64_t>(t0) + tl2;
          if (tt >= t1) break;
          for (int rr = 0; rr < 16; ++rr) {
            const float v = lg[(tl2 * B + b) * 16 + rr];
            const int n = static_cast<int>(tile_row_logical(p.kind, p.N, p.head_dim, tt, rr));
            if (v != v) {
              nan = true;
              continue;
            }
            if (n < p.N && better(v, n, best, bi)) {
              best = v;
              bi = n;
            }
          }
        }
        if (nan) raise_flag(p.err, 8);
        p.amax_val[static_cast<int64_t>(b) * gridDim.x + blockIdx.x] = best;
        p.amax_idx[static_cast<int64_t>(b) * gridDim.x + blockIdx.x] = bi;
      }
    }
  }
}

// ---------------------------------------------------------------- streaming GEMV
//
// For matrices with very many tiles (at least 16 per workgroup: the LM head)
// a fixed grid of kStreamGroups workgroups of kStreamWaves waves streams the
// whole matrix: workgroup i owns the contiguous tiles
// [T*i/kStreamGroups, T*(i+1)/kStreamGroups) and stages the activations (and
// the gain) in LDS once. Its tiles are cut into chunks of at most
// kStreamChunk consecutive groups; waves take chunks from an LDS counter as
// they finish, so fast and slow waves end together, and each wave keeps two
// chunks in flight (the next one is loaded before the current one is
// computed). A chunk's partial sums go to the chunk's own LDS slot, and the
// epilogue adds a tile's slots in chunk order, so the result does not depend
// on which wave took which chunk.

constexpr int kStreamGroups = 256;
constexpr int kStreamWaves = 16;
constexpr int kStreamChunk = 8;  // groups per chunk (ring slots per chunk buffer)

struct StreamPlan {
  bool ok = false;
  int tiles_per_group = 0, chunks_per_tile = 0;
  size_t lds = 0;
  int xrow = 0;
};

static StreamPlan stream_plan(int T, int G, int B, bool gain) {
  StreamPlan s;
  s.tiles_per_group = (T + kStreamGroups - 1) / kStreamGroups;
  s.chunks_per_tile = (G + kStreamChunk - 1) / kStreamChunk;
  s.xrow = (G * 128 + 511) / 512 * 512 + (B > 1 ? kRowPad : 0);
  const int rows = B + (gain ? 1 : 0);
  const size_t xbytes = static_cast<size_t>(rows) * s.xrow * 2;
  const size_t lg = static_cast<size_t>(s.tiles_per_group) * B * 16 * 4;  // argmax logits, reuse the x rows
  s.lds = std::max(xbytes, lg) + 256 + 16 +
          static_cast<size_t>(s.tiles_per_group) * s.chunks_per_tile * B * 16 * 4 +  // chunk partials
          static_cast<size_t>(kStreamWaves) * B * 4;                                // sum of squares
  // measured: the LM head gains (9504 tiles), gate/up (2368 tiles) is faster
  // with one tile set per workgroup
  s.ok = T >= 16 * kStreamGroups && s.lds <= 150 * 1024;
  return s;
}

template <int B, int EPI, bool GAIN>
__global__ __launch_bounds__(64 * kStreamWaves) void gemv_stream_kernel(GemvParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NW = kStreamWaves;
  constexpr int CH = kStreamChunk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kb = lane >> 4;
  const int G = p.G, xrow = p.xrow, cpt = p.ks;  // ks carries the chunks per tile
  const int t0 = static_cast<int>(static_cast<int64_t>(p.T) * blockIdx.x / gridDim.x);
  const int t1 = static_cast<int>(static_cast<int64_t>(p.T) * (blockIdx.x + 1) / gridDim.x);
  const int ntl = t1 - t0;                  // tiles of this workgroup (<= p.tpw)
  const int nb = ntl * G;                   // their blocks, contiguous in memory
  const int Q = ntl * cpt;                  // chunks
  // LDS: [B] activation rows | gain row | zero block | counter | part | ssq
  half_t* xs = reinterpret_cast<half_t*>(smem);
  half_t* gs = xs + B * xrow;
  const int xbytes = (B + (GAIN ? 1 : 0)) * xrow * 2;
  const int lgbytes = p.tpw * B * 16 * 4;
  half_t* zero = reinterpret_cast<half_t*>(smem + (xbytes > lgbytes ? xbytes : lgbytes));
  int* next_chunk = reinterpret_cast<int*>(zero + 128);
  float* part = reinterpret_cast<float*>(next_chunk + 4);  // [chunk][B][16]
  float* ssq = part + p.tpw * cpt * B * 16;                  // [NW][B]
  float* lg = reinterpret_cast<float*>(smem);                // [tile][B][16], after the stream
  const uint32_t magic = opaque(0x64006400u);
  const half8 nbias = neg_bias_frag();

  // the residual the epilogue adds to: one prefetched item per thread
  half_t e_res = static_cast<half_t>(0.0f);  // kept as loaded: converting it here would wait for it
  if constexpr (EPI == NQ_EPI_RESIDUAL_F16) {
    if (tid < ntl * B * 16) {
      const int j = tid / (B * 16), b = (tid / 16) % B, rr = tid & 15;
      const int64_t n = tile_row_logical(p.kind, p.N, p.head_dim, t0 + j, rr);
      if (n < p.N) e_res = static_cast<const half_t*>(p.y)[b * static_cast<int64_t>(p.N) + n];
    }
  }

  // descriptors over this workgroup's codes and scales (reads past the end give 0)
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.codes) + static_cast<size_t>(t0) * G * kBlockBytes, 0, nb * kBlockBytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.scales) + static_cast<size_t>(t0) * G * 32, 0, nb * 32, kBufferFlags);
  const int wvoff = lane * 16;
  const half_t* xlane = (col < B ? xs + col * xrow : zero) + kb * 32;
  const int xstep = col < B ? 128 : 0;
  if (tid < 16) reinterpret_cast<uint4*>(zero)[tid] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) *next_chunk = 2 * NW;       // chunks w and NW + w start on wave w

  // (1) activations and gain into LDS, issued before the weights
  {
    const int n8 = G * 16;                  // 16-byte items per row
    const int rblk = (n8 + 63) / 64;        // 1 KiB blocks per row
#pragma unroll 1
    for (int r = 0; r < B + (GAIN ? 1 : 0); ++r) {  // block j of every row on wave j mod NW
      const half_t* src = r < B ? p.x + static_cast<int64_t>(r) * p.K : p.gain;
      half_t* dst = r < B ? xs + r * xrow : gs;
      for (int j = wave; j < rblk; j += NW) {
        const int item = j * 64 + lane;
        if (item < n8) __builtin_amdgcn_global_load_lds(src + item * 8, dst + j * 512, 16, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // chunk q = (tile q / cpt, groups [c*G/cpt, (c+1)*G/cpt) with c = q % cpt);
  // slot s of a chunk buffer holds the chunk's group g0 + s, or zeros
  auto chunk_range = [&](int q, int& g0, int& g1, int& j) {
    j = q / cpt;
    const int c = q - j * cpt;
    g0 = c * G / cpt;
    g1 = (c + 1) * G / cpt;
  };
  // The chunk's scales come in one 64-lane load: lane (row kb, column c < CH)
  // holds rows 4kb..4kb+3 of slot c; slot s2 takes them from lane s2 of its row.
  auto load_chunk = [&](int q, u32x4 (&w)[CH], u32x2& sc) {
    int g0, g1, j;
    chunk_range(q, g0, g1, j);
    const bool in = q < Q;
    const int fs = (in && col < CH && g0 + col < g1) ? j * G + g0 + col : nb;
    sc = __builtin_amdgcn_raw_buffer_load_b64(srs, fs * 32 + kb * 8, 0, kStreamOnce);
#pragma unroll
    for (int s2 = 0; s2 < CH; ++s2) {
      const int f = (in && g0 + s2 < g1) ? j * G + g0 + s2 : nb;   // nb: out of range, reads 0
      w[s2] = __builtin_amdgcn_raw_buffer_load_b128(wrs, wvoff, f * kBlockBytes, kStreamOnce);
    }
  };
  auto compute_chunk = [&](int q, const u32x4 (&w)[CH], const u32x2& sc) {
    int g0, g1, j;
    chunk_range(q, g0, g1, j);
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s2 = 0; s2 < CH; ++s2) {
      const int g = min(g0 + s2, g1 - 1);  // a zero slot reads a valid activation group
      const f4 d = gemv_block_mfma<GAIN>(w[s2], xlane + g * xstep, magic, nbias);
      scale_acc(acc, d, row_bcast2(sc, s2));
    }
    if (col < B) {
#pragma unroll
      for (int i = 0; i < 4; ++i) part[(q * B + col) * 16 + 4 * kb + i] = acc[i];
    }
  };
  auto grab = [&]() -> int {
    int q = 0;
    if (lane == 0) q = atomicAdd(next_chunk, 1);
    return __builtin_amdgcn_readfirstlane(q);
  };

  // (2) The activations land before any weight is requested. Every workgroup
  //     reads the same few KiB at the same moment; behind a flood of weight
  //     requests those lines would wait for several microseconds, in front of
  //     it they cost one memory round trip. Then the first two chunks of each
  //     wave are requested.
  __builtin_amdgcn_s_waitcnt(0);     // activation copies and the chunk counter
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  u32x4 wa[CH], wb[CH];
  u32x2 sa, sb;
  int qa = wave;
  int qb = NW + wave;
  load_chunk(qa, wa, sa);
  load_chunk(qb, wb, sb);
  __builtin_amdgcn_sched_barrier(0);
  // (3) x * gain in place, pre-scaled for the biased codes, and each wave's
  //     share of sum(x^2) per batch row
  if constexpr (GAIN) {
    const float sw = gain_rows<B>(xs, xrow, gs, G * 16, nullptr, 0, 0);
    if (lane < B) ssq[wave * B + lane] = sw;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }

  // (4) stream: compute the older chunk while the newer one is in flight, then
  // refill its buffer with a freshly taken chunk. Chunk numbers only grow, so
  // the first one past the end means every later one is too.
  for (;;) {
    if (qa >= Q) break;
    compute_chunk(qa, wa, sa);
    qa = grab();
    load_chunk(qa, wa, sa);
    if (qb >= Q) break;
    compute_chunk(qb, wb, sb);
    qb = grab();
    load_chunk(qb, wb, sb);
  }
  __syncthreads();

  // (5) epilogue over (tile, batch row, tile row) items
  const int items = ntl * B * 16;
  for (int i = tid; i < items; i += blockDim.x) {
    const int j = i / (B * 16), b = (i / 16) % B, rr = i & 15;
    const int64_t tt = t0 + j;
    float yv = 0.0f, yp = 0.0f;
    for (int c = 0; c < cpt; ++c) {
      yv += part[((j * cpt + c) * B + b) * 16 + rr];
      yp += part[((j * cpt + c) * B + b) * 16 + (rr ^ 8)];
    }
    float rs = 1.0f;
    if constexpr (GAIN) {
      float v = 0.0f;
      for (int w = 0; w < NW; ++w) v += ssq[w * B + b];
      rs = 1.0f / sqrtf(v / static_cast<float>(p.K) + p.eps);
    }
    yv *= rs;
    yp *= rs;
    const int64_t n = tile_row_logical(p.kind, p.N, p.head_dim, tt, rr);
    const int64_t N = p.N;
    if constexpr (EPI == NQ_EPI_STORE_F16) {
      if (n < N) static_cast<half_t*>(p.y)[b * N + n] = static_cast<half_t>(yv);
    } else if constexpr (EPI == NQ_EPI_BIAS_F16) {
      if (n < N) static_cast<half_t*>(p.y)[b * N + n] = static_cast<half_t>(yv + static_cast<float>(p.bias[n]));
    } else if constexpr (EPI == NQ_EPI_RESIDUAL_F16) {
      if (n < N) {
        half_t* yo = static_cast<half_t*>(p.y) + b * N + n;
        const float r = static_cast<float>(i == tid ? e_res : *yo);
        const half_t v = static_cast<half_t>(r + yv);
        *yo = v;
        if (p.y2) p.y2[b * N + n] = v;
      }
    } else if constexpr (EPI == NQ_EPI_SWIGLU_F16) {
      if (rr < 8) {
        const int64_t I = N / 2;
        const float a = yv / (1.0f + expf(-yv)) * yp;
        static_cast<half_t*>(p.y)[b * I + 8 * tt + rr] = static_cast<half_t>(a);
      }
    } else if constexpr (EPI == NQ_EPI_STORE_F32) {
      if (n < N && p.y) static_cast<float*>(p.y)[b * N + n] = yv;
      lg[(j * B + b) * 16 + rr] = (n < N) ? yv : -INFINITY;
    }
  }

  if constexpr (EPI == NQ_EPI_STORE_F32) {
    if (p.amax_val) {
      __syncthreads();
      // this workgroup's best (value, index) per batch row: wave b scans its row
      if (wave < B) {
        const int b = wave;
        float best = -INFINITY;
        int bi = 0x7fffffff;
        bool nan = false;
        for (int i = lane; i < ntl * 16; i += 64) {
          const int j = i / 16, rr = i & 15;
          const float v = lg[(j * B + b) * 16 + rr];
          const int n = static_cast<int>(tile_row_logical(p.kind, p.N, p.head_dim, t0 + j, rr));
          if (v != v) {
            nan = true;
          } else if (n < p.N && better(v, n, best, bi)) {
            best = v;
            bi = n;
          }
        }
        for (int o = 32; o >= 1; o >>= 1) {
          const float ov = __shfl_xor(best, o);
          const int oi = __shfl_xor(bi, o);
          if (better(ov, oi, best, bi)) {
            best = ov;
            bi = oi;
          }
        }
        nan = __any(nan);
        if (lane == 0) {
          if (nan) raise_flag(p.err, 8);
          p.amax_val[static_cast<int64_t>(b) * gridDim.x + blockIdx.x] = best;
          p.amax_idx[static_cast<int64_t>(b) * gridDim.x + blockIdx.x] = bi;
        }
      }
    }
  }
}

struct GemvShape {
  int tpw, ks, ch, xrow, threads, grid, bal;
  size_t lds;
};

// Launch shape, from sweeps of (tiles per workgroup, K-slices) on MI355X at
// the decode shapes and batches 1, 4 and 8. Matrices with few tiles
// (T < 1024: the QKV, O and down projections) split K: two tiles per
// workgroup from 256 tiles, each wave owning about 7 groups; one tile per
// workgroup below that, with up to 8 slices of at least 3 groups each.
// Matrices with many tiles (gate/up, LM head) already fill the chip with
// workgroups: two tiles x two K-slices at batch 1-3, then one slice of four
// (batch 4-5) or eight tiles (batch 6-8), where each loaded block feeds more
// matrix-core columns. The workgroup count matters as much: with 264
// workgroups of 9 tiles (8 CUs holding two) gate/up took 28.5 us against 17
// us. From batch 4 the tiles are therefore spread evenly over one workgroup
// per CU (9 or 10 tiles of gate/up each; batch 8 22.6 against 28.3 us with 8
// tiles per workgroup). The staged activations (plus the gain) get at most
// kLdsX bytes; longer K is processed in chunks.
static GemvShape gemv_shape(int T, int G, int B, bool gain) {
  GemvShape s;
  s.bal = 0;
  if (T >= 1024 && B >= 4) {
    s.ks = 1;
    s.tpw = std::min(16, (T + kGemvCUs - 1) / kGemvCUs);  // at most 16 waves per workgroup
    s.grid = std::max(kGemvCUs, (T + s.tpw - 1) / s.tpw);  // every share holds at most tpw tiles
    s.bal = 1;
  } else if (T >= 1024) {
    s.ks = 2;
    s.tpw = 2;
  } else if (T >= 256) {
    s.ks = std::min(8, (G + 6) / 7);
    s.tpw = 2;
  } else {
    s.ks = std::min(8, std::max(1, G / 3));
    s.tpw = 1;
  }
  s.ks = std::max(1, std::min(s.ks, G));
  const int rows = B + (gain ? 1 : 0);
  const int nw = s.tpw * s.ks;
  // zero block, cross-wave partials, sums of squares, argmax logits
  const size_t extras = 256 + static_cast<size_t>(nw) * B * 16 * 4 + static_cast<size_t>(nw) * B * 4 +
                        static_cast<size_t>(s.tpw) * B * 16 * 4;
  const size_t budget = std::min(kLdsX, kLdsMax - extras);
  const int fit = static_cast<int>(budget / (static_cast<size_t>(rows) * 256)) / 4 * 4;  // whole 1 KiB blocks
  // a chunk's groups are dealt out to the K-slices afresh, so it need not be a
  // multiple of them: at batch 8 the down projection's 148 groups take two
  // chunks of 76 and 72 (19.3 us) instead of three of 64, 64 and 20 (20.7 us)
  s.ch = G <= fit ? G : std::max(4, fit);
  s.xrow = (s.ch * 128 + 511) / 512 * 512 + (B > 1 ? kRowPad : 0);
  s.threads = s.tpw * s.ks * 64;
  if (!s.bal) s.grid = (T + s.tpw - 1) / s.tpw;
  s.lds = static_cast<size_t>(rows) * s.xrow * 2 + extras;
  return s;
}

int gemv_grid_size(int32_t N, int32_t K, int32_t batch) {
  const int T = static_cast<int>(tiles_of(N));
  if (stream_plan(T, K / kGroup, batch, true).ok) return kStreamGroups;
  return gemv_shape(T, K / kGroup, batch, true).grid;
}

// Lets a streaming kernel take more than the default 64 KiB of dynamic LDS (once per kernel).
template <int B, int EPI, bool GAIN>
static hipError_t allow_stream_lds() {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_stream_kernel<B, EPI, GAIN>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
  return e;
}

template <int B, bool GAIN>
static hipError_t launch_stream_e(int epi, size_t lds, hipStream_t stream, const GemvParams& p) {
  const dim3 grid(kStreamGroups), block(64 * kStreamWaves);
  hipError_t e = hipSuccess;
  switch (epi) {
    case NQ_EPI_STORE_F16: e = allow_stream_lds<B, NQ_EPI_STORE_F16, GAIN>(); break;
    case NQ_EPI_BIAS_F16: e = allow_stream_lds<B, NQ_EPI_BIAS_F16, GAIN>(); break;
    case NQ_EPI_RESIDUAL_F16: e = allow_stream_lds<B, NQ_EPI_RESIDUAL_F16, GAIN>(); break;
    case NQ_EPI_SWIGLU_F16: e = allow_stream_lds<B, NQ_EPI_SWIGLU_F16, GAIN>(); break;
    case NQ_EPI_STORE_F32: e = allow_stream_lds<B, NQ_EPI_STORE_F32, GAIN>(); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  switch (epi) {
    case NQ_EPI_STORE_F16: gemv_stream_kernel<B, NQ_EPI_STORE_F16, GAIN><<<grid, block, lds, stream>>>(p); break;
    case NQ_EPI_BIAS_F16: gemv_stream_kernel<B, NQ_EPI_BIAS_F16, GAIN><<<grid, block, lds, stream>>>(p); break;
    case NQ_EPI_RESIDUAL_F16: gemv_stream_kernel<B, NQ_EPI_RESIDUAL_F16, GAIN><<<grid, block, lds, stream>>>(p); break;
    case NQ_EPI_SWIGLU_F16: gemv_stream_kernel<B, NQ_EPI_SWIGLU_F16, GAIN><<<grid, block, lds, stream>>>(p); break;
    case NQ_EPI_STORE_F32: gemv_stream_kernel<B, NQ_EPI_STORE_F32, GAIN><<<grid, block, lds, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int B>
static hipError_t launch_stream_g(bool gain, int epi, size_t lds, hipStream_t stream, const GemvParams& p) {
  return gain ? launch_stream_e<B, true>(epi, lds, stream, p) : launch_stream_e<B, false>(epi, lds, stream, p);
}

static hipError_t launch_stream_b(int batch, bool gain, int epi, size_t lds, hipStream_t stream, const GemvParams& p) {
  switch (batch) {
    case 1: return launch_stream_g<1>(gain, epi, lds, stream, p);
    case 2: return launch_stream_g<2>(gain, epi, lds, stream, p);
    case 3: return launch_stream_g<3>(gain, epi, lds, stream, p);
    case 4: return launch_stream_g<4>(gain, epi, lds, stream, p);
    case 5: return launch_stream_g<5>(gain, epi, lds, stream, p);
    case 6: return launch_stream_g<6>(gain, epi, lds, stream, p);
    case 7: return launch_stream_g<7>(gain, epi, lds, stream, p);
    case 8: return launch_stream_g<8>(gain, epi, lds, stream, p);
    default: return hipErrorInvalidValue;
  }
}

// Lets a GEMV instance take more than the default 64 KiB of dynamic LDS (once per instance).
template <int B, int EPI, bool GAIN>
static hipError_t allow_gemv_lds() {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_w4a16_kernel<B, EPI, GAIN>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
  return e;
}

template <int B, bool GAIN>
static hipError_t launch_gemv_e(int epi, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const GemvParams& p) {
  if (lds > 64 * 1024) {
    hipError_t e = hipSuccess;
    switch (epi) {
      case NQ_EPI_STORE_F16: e = allow_gemv_lds<B, NQ_EPI_STORE_F16, GAIN>(); break;
      case NQ_EPI_BIAS_F16: e = allow_gemv_lds<B, NQ_EPI_BIAS_F16, GAIN>(); break;
      case NQ_EPI_RESIDUAL_F16: e = allow_gemv_lds<B, NQ_EPI_RESIDUAL_F16, GAIN>(); break;
      case NQ_EPI_SWIGLU_F16: e = allow_gemv_lds<B, NQ_EPI_SWIGLU_F16, GAIN>(); break;
      case NQ_EPI_STORE_F32: e = allow_gemv_lds<B, NQ_EPI_STORE_F32, GAIN>(); break;
      case EPI_QKV_ROPE_KV: e = allow_gemv_lds<B, EPI_QKV_ROPE_KV, GAIN>(); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  switch (epi) {
    case NQ_EPI_STORE_F16: gemv_w4a16_kernel<B, NQ_EPI_STORE_F16, GAIN><<<grid, block, lds, stream>>>(p); break;
    case NQ_EPI_BIAS_F16: gemv_w4a16_kernel<B, NQ_EPI_BIAS_F16, GAIN><<<grid, block, lds, stream>>>(p); break;
    case NQ_EPI_RESIDUAL_F16: gemv_w4a16_kernel<B, NQ_EPI_RESIDUAL_F16, GAIN><<<grid, block, lds, stream>>>(p); break;
    case NQ_EPI_SWIGLU_F16: gemv_w4a16_kernel<B, NQ_EPI_SWIGLU_F16, GAIN><<<grid, block, lds, stream>>>(p); break;
    case NQ_EPI_STORE_F32: gemv_w4a16_kernel<B, NQ_EPI_STORE_F32, GAIN><<<grid, block, lds, stream>>>(p); break;
    case EPI_QKV_ROPE_KV: gemv_w4a16_kernel<B, EPI_QKV_ROPE_KV, GAIN><<<grid, block, lds, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int B>
static hipError_t launch_gemv_g(bool gain, int epi, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                const GemvParams& p) {
  return gain ? launch_gemv_e<B, true>(epi, grid, block, lds, stream, p)
              : launch_gemv_e<B, false>(epi, grid, block, lds, stream, p);
}

static hipError_t launch_gemv_b(int batch, bool gain, int epi, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                const GemvParams& p) {
  switch (batch) {
    case 1: return launch_gemv_g<1>(gain, epi, grid, block, lds, stream, p);
    case 2: return launch_gemv_g<2>(gain, epi, grid, block, lds, stream, p);
    case 3: return launch_gemv_g<3>(gain, epi, grid, block, lds, stream, p);
    case 4: return launch_gemv_g<4>(gain, epi, grid, block, lds, stream, p);
    case 5: return launch_gemv_g<5>(gain, epi, grid, block, lds, stream, p);
    case 6: return launch_gemv_g<6>(gain, epi, grid, block, lds, stream, p);
    case 7: return launch_gemv_g<7>(gain, epi, grid, block, lds, stream, p);
    case 8: return launch_gemv_g<8>(gain, epi, grid, block, lds, stream, p);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  GemvParams p{};
  p.N = a.N;
  p.K = a.K;
  p.kind = a.kind;
  p.head_dim = a.head_dim;
  p.G = a.K / kGroup;
  p.T = static_cast<int>(tiles_of(a.N));
  const GemvShape sh = gemv_shape(p.T, p.G, a.batch, a.norm_gain != nullptr);
  p.tpw = sh.tpw;
  p.ks = sh.ks;
  p.bal = sh.bal;
  p.ch = sh.ch;
  p.xrow = sh.xrow;
  p.codes = static_cast<const uint8_t*>(a.packed);
  p.scales = static_cast<const uint8_t*>(a.packed) + codes_bytes(a.N, a.K);
  p.x = static_cast<const half_t*>(a.x);
  p.gain = static_cast<const half_t*>(a.norm_gain);
  p.eps = a.eps;
  p.bias = static_cast<const half_t*>(a.bias);
  p.y = a.y;
  p.y2 = static_cast<half_t*>(a.y2);
  p.embed = static_cast<const half_t*>(a.embed);
  p.tokens_in = a.tokens_in;
  p.vocab = a.vocab;
  p.h_out = static_cast<half_t*>(a.h_out);
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
  const StreamPlan sp = stream_plan(p.T, p.G, a.batch, a.norm_gain != nullptr);
  if (sp.ok && a.epi != EPI_QKV_ROPE_KV && !a.embed) {
    p.tpw = sp.tiles_per_group;  // the streaming kernel reads tpw / ks as tiles per group / chunks per tile
    p.ks = sp.chunks_per_tile;
    p.xrow = sp.xrow;
    return launch_stream_b(a.batch, a.norm_gain != nullptr, a.epi, sp.lds, stream, p);
  }
  const dim3 grid(sh.grid), block(sh.threads);
  return launch_gemv_b(a.batch, a.norm_gain != nullptr, a.epi, grid, block, sh.lds, stream, p);
}

// ============================================================== attention
//
// Split-K paged decode attention on the matrix cores. Workgroup (split s, KV
// head, sequence) covers pages [s*per, (s+1)*per) of the sequence; its
// kAttnWaves waves take pages w, w + kAttnWaves, ... and each keeps the next
// page's loads in flight while it computes the current one. The query heads
// of a KV head (GQA) are the 16 columns of the MFMA tiles, so every K/V page
// is loaded once for all of them:
//   scores  S^T[t][h] = sum_d K[t][d] Q[h][d]    v_mfma_f32_16x16x32_f16, A = K page
//                                                (token-major, as stored), B = Q^T
//   output  O^T[d][h] += sum_t V^T[d][t] P^T[t][h]  v_mfma_f32_16x16x16_f16, A = V page
//                                                (dim-major, as stored), B = the
//                                                probabilities the lane just computed
// so both operands come straight from HBM in register order, with no LDS
// round trip. Each lane ends up owning one head (lane % 16) for the online
// softmax, so the running max, sum and the rescale of O stay in the lane.
// Tokens at or beyond the length are masked by position (scores to -inf, V
// to 0), whatever the slot holds. The only block-wide barrier sits in uniform
// control flow after the page loop ("How To Build Your Own LLM Runtime From
// Scratch", FAQ on the barrier inside a warp-id branch). When one workgroup
// covers the whole context it writes the output; otherwise workgroups write
// (max, sum, output) partials and the combine kernel merges them with the
// log-sum-exp rule. A batch of one takes fixed splits of one page per wave.
// Larger batches split by the actual lengths, not the table width: every
// workgroup of a fixed grid of S per KV head reads the lengths, takes per =
// the page count per split that spreads all sequences' pages over the grid,
// and finds its (sequence, split) from the running sum of the sequences'
// split counts ceil(pages_b / per). A ragged batch then gives every workgroup
// about the same number of pages, and the grid (hence a captured graph) does
// not depend on the lengths. Workgroups are 4 waves, so that three of them
// fit on a CU at the kernel's register count: 12 waves per CU where one
// 8-wave workgroup gives 8. A batch of one fills the CUs three times over; a
// larger batch takes one workgroup per CU, whose longer splits stream faster.

constexpr int kAttnWaves = 4;
constexpr int kMaxPagesPerWave = 128;  // a split holds at most kAttnWaves * 128 pages
constexpr int kPidRegs = (kMaxPagesPerWave + 63) / 64;  // page ids held one per lane and register
// waves per SIMD the register budget is sized for (at most 168 registers):
// whole workgroups of kAttnWaves waves on the 4 SIMDs of a CU
constexpr int kAttnWavesPerSimd = kAttnWaves == 4 ? 3 : 2;
static_assert(kAttnMaxSplits % 64 == 0, "combine weight slots");
constexpr int kAttnTargetGroups = 768;  // batch 1: three 4-wave workgroups per CU
// Batches of several sequences: one 4-wave workgroup per CU, each with longer
// splits. The batch-8 step at 1.4k-16k context took 2.635 ms/step with 256
// workgroups, 2.652 with 512 and 2.689 with 768 (same box); 128, 192, 384 and
// 640, which leave CUs idle or unevenly loaded, took 3.10, 2.87, 2.85 and 2.79,
// and 256 workgroups of 8 waves 2.669.
constexpr int kAttnBatchGroups = 256;

// Pages per split for S workgroups per KV head over B sequences holding P
// pages in all: the fewest such that sum_b ceil(pages_b / per) <= S (each ceil
// adds less than one split, hence S - B), and at least the wave count. It is
// not rounded up to a multiple of the wave count: the waves of a split then
// differ by one page, and fewer of them hold the most pages (the batch-8 step
// at 1.4k-16k context took 2.798 against 2.821 ms with the rounding).
__host__ __device__ __forceinline__ int attn_pages_per_split(int P, int S, int B) {
  const int room = S - B > 0 ? S - B : 1;
  const int per = (P + room - 1) / room;
  return per > kAttnWaves ? per : kAttnWaves;
}

AttnPlan attn_plan(int32_t batch, int32_t n_kv, int32_t max_pages) {
  AttnPlan p;
  if (batch < 1 || max_pages < 1) {
    p.S = 0;
    return p;
  }
  const int pages4 = (max_pages + kAttnWaves - 1) / kAttnWaves;
  const int target = std::max(1, (batch == 1 ? kAttnTargetGroups : kAttnBatchGroups) / std::max(1, n_kv));
  if (max_pages <= kAttnWaves || (batch == 1 && pages4 <= target)) {
    // fixed splits of one page per wave (one split when the table is that
    // short): the page ids do not wait for the length, and a batch of one
    // cannot be imbalanced
    p.S = pages4;
    p.per = kAttnWaves;
    return p;
  }
  if (batch > kAttnMaxBatch) {
    p.S = 0;
    return p;
  }
  // splits by length: enough to fill the chip, no more than the table can use
  // (one page per wave), at least one more than the batch, and enough that no
  // wave holds more than kMaxPagesPerWave pages
  const int64_t cap = static_cast<int64_t>(kAttnWaves) * kMaxPagesPerWave;
  const int64_t all = static_cast<int64_t>(batch) * max_pages;
  int64_t S = std::min<int64_t>(target, static_cast<int64_t>(batch) * pages4);
  S = std::max<int64_t>(S, (all + cap - 1) / cap + batch);
  S = std::max<int64_t>(S, batch + 1);
  if (S > kAttnMaxSplits || attn_pages_per_split(static_cast<int>(all), static_cast<int>(S), batch) > cap) {
    p.S = 0;  // beyond what the kernels cover
    return p;
  }
  p.S = static_cast<int32_t>(S);
  p.per = attn_pages_per_split(static_cast<int>(all), p.S, batch);  // the largest any lengths give
  p.dyn = 1;
  return p;
}

size_t attn_partial_bytes(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t splits) {
  return static_cast<size_t>(batch) * n_heads * splits * (head_dim + 2) * sizeof(float);
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
  int n_heads, n_kv, S, per, batch, dyn;
  int32_t* err;
};

// The split of workgroup w (of a.S per KV head) for the current lengths: lane
// j < batch takes sequence j's page count; returns false for a workgroup past
// the last split. Every lane gets the same (b, s, per, np_b).
__device__ __forceinline__ bool attn_split_of(const AttnParams& a, int w, int& b, int& s, int& per, int& npb) {
  const int lane = threadIdx.x & 63;
  int np = 0;
  if (lane < a.batch) {
    const int L = a.lens[lane] + a.len_add;
    np = L > 0 ? min((L + kPageTokens - 1) / kPageTokens, a.max_pages) : 0;
  }
  int P = np;
  for (int o = 32; o >= 1; o >>= 1) P += __shfl_xor(P, o);
  per = attn_pages_per_split(P, a.S, a.batch);
  const int sb = (np + per - 1) / per;
  int start = sb;  // inclusive running sum over lanes, then exclusive
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(start, o);
    if (lane >= o) start += v;
  }
  start -= sb;
  const unsigned long long hit = __ballot(sb > 0 && w >= start && w < start + sb);
  if (!hit) return false;
  b = __builtin_ctzll(hit);
  s = w - __shfl(start, b);
  npb = __shfl(np, b);
  return true;
}

// A K/V page load, with the non-temporal hint when NT: a batch of several
// sequences reads every page of every sequence once per layer, and the hint
// took the batch-8 step at 1.4k-16k context from 2.796 to 2.685 ms; a batch of
// one reads them plainly (with the hint its kernel took 26.3 against 24.9 us at
// 32767 tokens and 11.8 against 11.1 us at 4097).
template <bool NT, typename T>
__device__ __forceinline__ T page_load(const half_t* ptr) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const T*>(ptr));
  else return *reinterpret_cast<const T*>(ptr);
}

template <int D, int REP, bool NT>
__global__ __launch_bounds__(64 * kAttnWaves) __attribute__((amdgpu_waves_per_eu(kAttnWavesPerSimd)))
void attn_decode_kernel(AttnParams a) {
  static_assert((D == 64 || D == 128) && REP >= 1 && REP <= 16, "unsupported head shape");
  constexpr int NW = kAttnWaves;
  constexpr int KJ = D / 32;  // score MFMAs per page
  constexpr int VC = D / 16;  // P.V MFMAs per page
  constexpr int DP = D + 4;   // padded LDS row (bank spread across heads)
  __shared__ float red_m[NW][16], red_l[NW][16];
  __shared__ __align__(16) float red_o[NW][REP][DP];

  const int kvh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  int b = blockIdx.z, s = blockIdx.x, per = a.per, npb = 0;
  if (a.dyn) {  // split by the current lengths (block-uniform)
    if (!attn_split_of(a, blockIdx.x, b, s, per, npb)) return;
    b = __builtin_amdgcn_readfirstlane(b);
    s = __builtin_amdgcn_readfirstlane(s);
    per = __builtin_amdgcn_readfirstlane(per);
  }
  const int p0 = s * per;
  const int pend = min(a.max_pages, p0 + per);
  // Q^T fragments: lane holds head r16, dims 32j + 8*g4 .. +7 (zero for the
  // padding heads r16 >= REP, which load head 0 and discard it)
  half8 qf[KJ];
  {
    const half_t* qh =
        a.q + (static_cast<int64_t>(b) * a.n_heads + kvh * REP + (r16 < REP ? r16 : 0)) * D + 8 * g4;
#pragma unroll
    for (int j = 0; j < KJ; ++j) qf[j] = *reinterpret_cast<const half8*>(qh + 32 * j);
  }
  // this wave's page ids, one per lane; they do not depend on the length, so
  // these loads overlap with the length load
  int pid[kPidRegs];
#pragma unroll
  for (int r = 0; r < kPidRegs; ++r) {
    const int myp = p0 + w + (lane + 64 * r) * NW;
    pid[r] = myp < pend ? a.pt[static_cast<int64_t>(b) * a.max_pages + myp] : -1;
  }
  auto page_id = [&](int k) {  // k is wave-uniform
    int id = __builtin_amdgcn_readlane(pid[0], k & 63);
#pragma unroll
    for (int r = 1; r < kPidRegs; ++r)
      if ((k >> 6) == r) id = __builtin_amdgcn_readlane(pid[r], k & 63);
    return id;
  };
  const int len = __builtin_amdgcn_readfirstlane(a.lens[b] + a.len_add);
  const int npages = min((len + kPageTokens - 1) / kPageTokens, a.max_pages);
  if (s == 0 && tid == 0 && len > a.max_pages * kPageTokens) raise_flag(a.err, 2);  // (a length past the table)
  const int64_t row0 = (static_cast<int64_t>(b) * a.n_heads + kvh * REP) * a.S;
  if (len <= 0 || p0 >= npages) {  // block-uniform
    if (a.S == 1) {                // empty context: zero output
      for (int i = tid; i < REP * D; i += 64 * NW)
        a.out[(static_cast<int64_t>(b) * a.n_heads + kvh * REP + i / D) * D + i % D] = static_cast<half_t>(0.0f);
    } else if (tid < REP) {        // an empty split: weight 0 in the combine
      a.pml[(row0 + static_cast<int64_t>(tid) * a.S + s) * 2] = -INFINITY;
      a.pml[(row0 + static_cast<int64_t>(tid) * a.S + s) * 2 + 1] = 0.0f;
    }
    return;
  }
  const int p1 = min(npages, pend);
  const int nmine = p0 + w < p1 ? (p1 - p0 - w + NW - 1) / NW : 0;  // wave-uniform

  if (r16 >= REP) {
#pragma unroll
    for (int j = 0; j < KJ; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[j][e] = static_cast<half_t>(0.0f);
  }
  const float qscale = 1.4426950408889634f / sqrtf(static_cast<float>(D));  // log2(e) / sqrt(d)

  f4 o[VC];
#pragma unroll
  for (int c = 0; c < VC; ++c) o[c] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, l = 0.0f;

  // page k of this wave: K rows t = r16 (dims 32j + 8*g4 ..), V^T rows d = 16c + r16
  // (tokens 4*g4 .. +3). An id outside the pool reads page 0 and is skipped.
  auto load = [&](int k, half8 (&kf)[KJ], half4 (&vf)[VC]) {
    const int id = page_id(k);
    const int idc = (id >= 0 && id < a.num_pages) ? id : 0;
    const int64_t base = (static_cast<int64_t>(idc) * a.n_kv + kvh) * (kPageTokens * D);
    const half_t* kb = a.kp + base + r16 * D + 8 * g4;
    const half_t* vb = a.vp + base + r16 * kPageTokens + 4 * g4;
#pragma unroll
    for (int j = 0; j < KJ; ++j) kf[j] = page_load<NT, half8>(kb + 32 * j);
#pragma unroll
    for (int c = 0; c < VC; ++c) vf[c] = page_load<NT, half4>(vb + 16 * c * kPageTokens);
  };
  // A page whose id is outside the pool counts as empty (and is reported after
  // the loop), so the loop body stays free of branches around memory ops.
  bool bad = false;
  auto compute = [&](int k, const half8 (&kf)[KJ], half4 (&vf)[VC]) {
    const int id = page_id(k);
    const bool okp = id >= 0 && id < a.num_pages;
    bad |= !okp;
    const int valid = okp ? min(kPageTokens, len - (p0 + w + k * NW) * kPageTokens) : 0;
    f4 sc = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < KJ; ++j) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[j], qf[j], sc, 0, 0, 0);
    // lane holds S^T[t = 4*g4 + i][h = r16]
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (4 * g4 + i < valid) ? sc[i] * qscale : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);  // -inf only while every page so far was empty
    const float alpha = mnew == -INFINITY ? 1.0f : exp2f(m - mnew);
    half4 pf;
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pf[i] = static_cast<half_t>(sv[i] == -INFINITY ? 0.0f : exp2f(sv[i] - mnew));
      ps += static_cast<float>(pf[i]);
    }
    l = l * alpha + ps;
    m = mnew;
    if (valid < kPageTokens) {  // tail page: unused slots may hold anything (NaN poison included)
#pragma unroll
      for (int c = 0; c < VC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * g4 + i >= valid) vf[c][i] = static_cast<half_t>(0.0f);
    }
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      o[c] *= alpha;
      o[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf[c], pf, o[c], 0, 0, 0);
    }
  };

  if (nmine > 0) {
    half8 kA[KJ], kB[KJ];
    half4 vA[VC], vB[VC];
    load(0, kA, vA);
    // the loads of page k+1 are issued before page k is computed; the last
    // page is loaded again in place of a page past the end (uniform wait counts)
    for (int k = 0; k < nmine; k += 2) {
      load(min(k + 1, nmine - 1), kB, vB);
      compute(k, kA, vA);
      if (k + 1 >= nmine) break;
      load(min(k + 2, nmine - 1), kA, vA);
      compute(k + 1, kB, vB);
    }
  }

  if (bad && lane == 0) raise_flag(a.err, 2);

  // combine the waves (uniform control flow: every wave reaches the barrier)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (g4 == 0) {
    red_m[w][r16] = m;
    red_l[w][r16] = l;
  }
  if (r16 < REP) {
#pragma unroll
    for (int c = 0; c < VC; ++c) *reinterpret_cast<f4*>(&red_o[w][r16][16 * c + 4 * g4]) = o[c];
  }
  __syncthreads();
  for (int i = tid; i < REP * D; i += 64 * NW) {
    const int h = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, red_m[ww][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = (red_m[ww][h] == -INFINITY) ? 0.0f : exp2f(red_m[ww][h] - M);
      L = fmaf(f, red_l[ww][h], L);
      O = fmaf(f, red_o[ww][h][d], O);
    }
    if (a.S == 1) {
      a.out[(static_cast<int64_t>(b) * a.n_heads + kvh * REP + h) * D + d] = static_cast<half_t>(L > 0.0f ? O / L : 0.0f);
    } else {
      const int64_t row = row0 + static_cast<int64_t>(h) * a.S + s;
      a.po[row * D + d] = O;
      if (d == 0) {
        a.pml[row * 2] = M;
        a.pml[row * 2 + 1] = L;
      }
    }
  }
}

// grid (n_heads, B), 1024 threads: merge the split partials of one query head
// (maxima in log2 units). Thread group g of 1024 / D takes splits g, g + G,
// ..., so a long split list is read G rows at a time; the group sums are then
// added in group order (the result does not depend on timing). The splits of
// sequence b are the ceil(pages_b / per) ones the attention kernel derived
// from the same lengths; the first loads go out before that count is known.
template <int D>
__global__ __launch_bounds__(1024) void attn_combine_kernel(AttnParams a) {
  constexpr int G = 1024 / D;
  constexpr int kEarly = 8;  // partials per thread loaded before the weights are known
  constexpr int kSlots = kAttnMaxSplits / 64;  // splits per lane in the weight pass
  __shared__ float wgt[kAttnMaxSplits];
  __shared__ float part[G][D];
  __shared__ float inv_l;
  __shared__ int n_live;
  const int h = blockIdx.x, b = blockIdx.y;
  const int d = threadIdx.x % D, g = threadIdx.x / D;
  const int S = a.S;
  const int64_t rb = (static_cast<int64_t>(b) * a.n_heads + h) * S;
  float pv[kEarly];
#pragma unroll
  for (int i = 0; i < kEarly; ++i) {
    const int s = g + G * i;
    pv[i] = s < S ? a.po[(rb + s) * D + d] : 0.0f;
  }
  if (threadIdx.x < 64) {  // one wave: the softmax weights of the splits
    const int lane = threadIdx.x;
    // fixed splits: every one wrote its row (an empty one with max -inf), so
    // nothing waits for the length; splits by length: sequence b has the
    // ceil(pages_b / per) the attention kernel derived from the same lengths
    int sb = S;
    if (a.dyn) {
      int np = 0;
      if (lane < a.batch) {
        const int L = a.lens[lane] + a.len_add;
        np = L > 0 ? min((L + kPageTokens - 1) / kPageTokens, a.max_pages) : 0;
      }
      int P = np;
      for (int o = 32; o >= 1; o >>= 1) P += __shfl_xor(P, o);
      const int per = attn_pages_per_split(P, S, a.batch);
      sb = (__shfl(np, b) + per - 1) / per;
    }
    float m0[kSlots], l0[kSlots];
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const int sj = lane + 64 * j;
      m0[j] = sj < sb ? a.pml[(rb + sj) * 2] : -INFINITY;
      l0[j] = sj < sb ? a.pml[(rb + sj) * 2 + 1] : 0.0f;
      M = fmaxf(M, m0[j]);
    }
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.0f;
    int last = -1;  // the last split with a weight: the ones after it hold nothing
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const float f = (m0[j] == -INFINITY) ? 0.0f : exp2f(m0[j] - M);
      L = fmaf(f, l0[j], L);
      wgt[lane + 64 * j] = f;
      if (f != 0.0f) last = lane + 64 * j;
    }
    for (int o = 32; o >= 1; o >>= 1) {
      L += __shfl_xor(L, o);
      last = max(last, __shfl_xor(last, o));
    }
    if (lane == 0) {
      inv_l = L > 0.0f ? 1.0f / L : 0.0f;
      n_live = last + 1;
    }
  }
  __syncthreads();
  // an empty split's output row was never written: its weight selects 0, not 0 * (stale value)
  const int nl = n_live;
  float O = 0.0f;
#pragma unroll
  for (int i = 0; i < kEarly; ++i) {
    const int s = g + G * i;
    if (s < nl && wgt[s] != 0.0f) O = fmaf(wgt[s], pv[i], O);
  }
  for (int s0 = G * kEarly; s0 < nl; s0 += G * kEarly) {  // later splits kEarly per thread at a time
#pragma unroll
    for (int i = 0; i < kEarly; ++i) {
      const int s = s0 + g + G * i;
      pv[i] = (s < nl && wgt[s] != 0.0f) ? a.po[(rb + s) * D + d] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kEarly; ++i) {
      const int s = s0 + g + G * i;
      if (s < nl && wgt[s] != 0.0f) O = fmaf(wgt[s], pv[i], O);
    }
  }
  part[g][d] = O;
  __syncthreads();
  if (g == 0) {
    float t = 0.0f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) t += part[gg][d];
    a.out[(static_cast<int64_t>(b) * a.n_heads + h) * D + d] = static_cast<half_t>(t * inv_l);
  }
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
  p.per = a.per;
  p.batch = a.batch;
  p.dyn = a.dyn;
  p.err = a.err;
  const int rep = a.n_heads / a.n_kv;
  if (p.S < 1 || p.S > kAttnMaxSplits || (p.dyn && a.batch > kAttnMaxBatch)) return hipErrorInvalidValue;
  // splits by length: S workgroups per KV head, each finds its (sequence,
  // split); fixed splits: S per (KV head, sequence)
  const dim3 grid(p.S, p.n_kv, p.dyn ? 1 : a.batch), block(64 * kAttnWaves);
#define NQ_ATT(DD, RR)                                                                   \
  if (a.head_dim == DD && rep == RR) {                                                   \
    if (a.batch > 1) attn_decode_kernel<DD, RR, true><<<grid, block, 0, s>>>(p);         \
    else attn_decode_kernel<DD, RR, false><<<grid, block, 0, s>>>(p);                    \
    if (p.S > 1) attn_combine_kernel<DD><<<dim3(a.n_heads, a.batch), dim3(1024), 0, s>>>(p); \
    return hipGetLastError();                                                            \
  }
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
  const int slot = ps % kPageTokens;
  for (int i = threadIdx.x; i < items; i += blockDim.x) {
    const int h = (i * 8) / d, e = (i * 8) % d;
    const int64_t blk = (static_cast<int64_t>(page) * n_kv + h) * kPageTokens * d;
    const int64_t src = (static_cast<int64_t>(b) * n_kv + h) * d + e;
    *reinterpret_cast<uint4*>(kp + blk + slot * d + e) = *reinterpret_cast<const uint4*>(k + src);  // token-major
    const uint4 vv = *reinterpret_cast<const uint4*>(v + src);
    const half_t* vh = reinterpret_cast<const half_t*>(&vv);
#pragma unroll
    for (int j = 0; j < 8; ++j) vp[blk + (e + j) * kPageTokens + slot] = vh[j];  // dim-major
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

// grid (B), 1024 threads: reduce the LM head's per-workgroup (max, index)
// partials of one batch row, write the greedy token, its history entry, and
// advance the position (or set it to pos_set >= 0; pos may be null then).
__global__ __launch_bounds__(1024) void argmax_finalize_kernel(const float* vals, const int32_t* idx, int P,
                                                               int32_t* tokens, int32_t* pos, int32_t* hist,
                                                               int hist_len, int pos_set) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = tid; i < P; i += 1024) {
    const float v = vals[static_cast<int64_t>(b) * P + i];
    const int ix = idx[static_cast<int64_t>(b) * P + i];
    if (better(v, ix, best, bi)) {
      best = v;
      bi = ix;
    }
  }
  for (int o = 32; o >= 1; o >>= 1) {
    const float v = __shfl_xor(best, o);
    const int ix = __shfl_xor(bi, o);
    if (better(v, ix, best, bi)) {
      best = v;
      bi = ix;
    }
  }
  if (lane == 0) {
    sv[w] = best;
    si[w] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < static_cast<int>(blockDim.x >> 6); ++k)
      if (better(sv[k], si[k], best, bi)) {
        best = sv[k];
        bi = si[k];
      }
    const int tok = bi == 0x7fffffff ? 0 : bi;
    tokens[b] = tok;
    if (pos_set >= 0) {
      if (pos) pos[b] = pos_set;
    } else {
      const int ps = pos[b];
      if (hist && ps + 1 >= 0 && ps + 1 < hist_len) hist[static_cast<int64_t>(b) * hist_len + ps + 1] = tok;
      pos[b] = ps + 1;
    }
  }
}

hipError_t launch_argmax_finalize(const float* vals, const int32_t* idx, int32_t partials, int32_t batch,
                                  int32_t* tokens, int32_t* pos, int32_t* hist, int32_t hist_len, int32_t pos_set,
                                  hipStream_t s) {
  argmax_finalize_kernel<<<dim3(batch), dim3(1024), 0, s>>>(vals, idx, partials, tokens, pos, hist, hist_len,
                                                            pos_set);
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
