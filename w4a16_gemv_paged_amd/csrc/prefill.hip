// HIP kernels of the chunked prefill of libnq for CDNA4 (gfx950), wave64.
//
// A prompt goes through the model a chunk of M tokens at a time rather than one
// token per decode step, which is what the time to first token of "How To
// Build Your Own LLM Runtime From Scratch" (daily.dev, Summary) depends on:
// * RMSNorm over the M rows of a chunk (with the embedding gather before the
//   first layer), written once as fp16 activations.
// * W4A16 GEMM on the matrix cores: the packed INT4 tiles of the decode GEMV
//   (same layout: a lane's 16-byte load of a (tile, group) block is its four
//   v_mfma_f32_16x16x32_f16 A fragments after the in-register unpack) times
//   the chunk's fp16 rows as the B operand (the chunk's tokens are the MFMA
//   columns), the group scale applied to the fp32 partial sums, and fused
//   epilogues (bias + RoPE + K/V page writes, residual add, SwiGLU).
// * Causal paged attention of the chunk's queries over the pages of their
//   sequence (earlier chunks and this one): scores and P.V on the matrix cores
//   with the chunk's tokens as the MFMA columns, K and V pages read straight
//   into operand registers, masked by position.
#include <algorithm>

#include "device.hpp"

namespace nq {

// ============================================================== RMSNorm rows

// grid (M), 256 threads. One rounding to fp16 at the end; 1/rms in fp32.
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const half_t* h, const half_t* embed,
                                                           const int32_t* tokens, int vocab, half_t* h_out,
                                                           const half_t* gain, float eps, half_t* xn, int H,
                                                           int32_t* err) {
  __shared__ float red[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const half_t* src = h + static_cast<int64_t>(m) * H;
  if (embed) {
    int tok = tokens[m];
    if (tok < 0 || tok >= vocab) {
      if (tid == 0) raise_flag(err, 4);
      tok = 0;
    }
    src = embed + static_cast<int64_t>(tok) * H;
  }
  const int n8 = H / 8;
  float ss = 0.0f;
  for (int i = tid; i < n8; i += 256) {
    const uint4 v = reinterpret_cast<const uint4*>(src)[i];
    const half_t* e = reinterpret_cast<const half_t*>(&v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(static_cast<float>(e[j]), static_cast<float>(e[j]), ss);
    if (embed) reinterpret_cast<uint4*>(h_out + static_cast<int64_t>(m) * H)[i] = v;
  }
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / static_cast<float>(H) + eps);
  for (int i = tid; i < n8; i += 256) {
    uint4 v = reinterpret_cast<const uint4*>(src)[i];
    const uint4 gv = reinterpret_cast<const uint4*>(gain)[i];
    half_t* e = reinterpret_cast<half_t*>(&v);
    const half_t* g = reinterpret_cast<const half_t*>(&gv);
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = static_cast<half_t>(static_cast<float>(e[j]) * r * static_cast<float>(g[j]));
    reinterpret_cast<uint4*>(xn + static_cast<int64_t>(m) * H)[i] = v;
  }
}

hipError_t launch_rmsnorm_rows(const void* h_in, const void* embed, const int32_t* tokens, int32_t vocab,
                               void* h_out, const void* gain, float eps, void* xn, int32_t M, int32_t H,
                               int32_t* err, hipStream_t s) {
  rmsnorm_rows_kernel<<<dim3(M), dim3(256), 0, s>>>(
      static_cast<const half_t*>(h_in), static_cast<const half_t*>(embed), tokens, vocab,
      static_cast<half_t*>(h_out), static_cast<const half_t*>(gain), eps, static_cast<half_t*>(xn), H, err);
  return hipGetLastError();
}

// ============================================================== GEMM
//
// Work split: a workgroup of 4 waves owns 4*WT consecutive row tiles (wave w
// the WT tiles from (4*rb + w)*WT) and 16*TT consecutive rows of the chunk.
// The K loop walks the 128-wide groups. Per group the workgroup's activation
// block (16*TT rows x 128 K) sits in LDS, laid out as 4*TT MFMA B operands of
// 1 KiB (slot (tt, j): lane l holds row 16tt + l%16, K 32*(l/16) + 8j .. +7,
// matching the K order of the packed A fragments), so every B read is one
// conflict-free 16-byte ds_read per lane. Wave w fills slot (tt, j = w) with
// one 16-byte global load per lane, two groups ahead in registers; the LDS
// block is double-buffered with one LDS-only barrier per group. Weights are
// read straight into registers, PD groups ahead. A group's four MFMAs per
// (tile, token tile) accumulate unscaled sums d, then acc += d * scale (fp32),
// so the codes stay exact, as in the decode GEMV.

struct GemmParams {
  const uint8_t* codes;
  const uint8_t* scales;
  int N, K, kind, head_dim, G, T, M;
  int tok_blocks, work;
  const half_t* x;
  const half_t* bias;
  void* y;
  half_t* y2;
  int pos0;
  const int32_t* pt;
  int max_pages, num_pages, n_heads, n_kv;
  half_t* kv_k;
  half_t* kv_v;
  const float* rope;
  int max_pos;
  int32_t* err;
};

constexpr int kGemmWaves = 4;

template <int WT, int TT, int PD, int EPI>
__global__ __launch_bounds__(64 * kGemmWaves) void gemm_w4a16_kernel(GemmParams p) {
  static_assert(PD % 2 == 0, "the weight ring is unrolled in pairs of groups");
  constexpr int NW = kGemmWaves;
  constexpr int XSLOT = 1024;
  constexpr int XSTAGE = TT * 4 * XSLOT;
  __shared__ __align__(16) unsigned char xs[2 * XSTAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kb = lane >> 4;
  // Workgroup i runs on XCD i % 8; each XCD takes a contiguous range of work
  // items (row-block major), so a row block's weights are fetched into one
  // XCD's L2 and reused there by its token blocks.
  const int per = gridDim.x / 8;
  const int work = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (work >= p.work) return;  // whole workgroup
  const int rb = work / p.tok_blocks, mb = work - rb * p.tok_blocks;
  const int t0 = (rb * NW + wave) * WT;
  // this wave's tiles inside the matrix (kept in a scalar register: the buffer
  // descriptors below must be uniform)
  const int nt = __builtin_amdgcn_readfirstlane(max(0, min(WT, p.T - t0)));
  const int m0 = mb * 16 * TT;
  const uint32_t magic = opaque(0x64006400u);

  // Weight and scale reads of tiles past the matrix, and of the padding
  // groups past G, are out of the buffer range and return 0.
  const size_t tb = static_cast<size_t>(nt > 0 ? t0 : 0) * p.G;
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.codes) + tb * kBlockBytes, 0, nt * p.G * kBlockBytes,
                                        kBufferFlags);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.scales) + tb * 32, 0, nt * p.G * 32, kBufferFlags);
  auto load_w = [&](int g, u32x4 (&w)[WT], u32x2 (&s)[WT]) {
    const bool in = g < p.G;
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const int blk = i * p.G + g;
      w[i] = __builtin_amdgcn_raw_buffer_load_b128(wrs, in ? blk * kBlockBytes + lane * 16 : nt * p.G * kBlockBytes, 0, 0);
      s[i] = __builtin_amdgcn_raw_buffer_load_b64(srs, in ? blk * 32 + kb * 8 : nt * p.G * 32, 0, 0);
    }
  };
  // Activation rows past the chunk are clamped to its last row (their output
  // columns are discarded), groups past G to the last group (their weights
  // are zero).
  const half_t* xrow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
    xrow[tt] = p.x + static_cast<int64_t>(min(m0 + 16 * tt + col, p.M - 1)) * p.K + 32 * kb + 8 * wave;
  auto load_x = [&](int g, u32x4 (&xr)[TT]) {
    const int gl = min(g, p.G - 1);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) xr[tt] = *reinterpret_cast<const u32x4*>(xrow[tt] + gl * kGroup);
  };
  auto store_x = [&](int stage, const u32x4 (&xr)[TT]) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      *reinterpret_cast<u32x4*>(xs + stage * XSTAGE + (tt * 4 + wave) * XSLOT + lane * 16) = xr[tt];
  };

  u32x4 xr[2][TT];
  u32x4 wv[PD][WT];
  u32x2 sv[PD][WT];
  load_x(0, xr[0]);
  load_x(1, xr[1]);
#pragma unroll
  for (int u = 0; u < PD; ++u) load_w(u, wv[u], sv[u]);
  store_x(0, xr[0]);
  load_x(2, xr[0]);
  lds_barrier();

  f4 acc[WT][TT];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[i][tt] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // Every wave runs the same number of groups (a multiple of PD); groups past
  // G read zero weights and scales and add nothing.
  const int gpad = (p.G + PD - 1) / PD * PD;
  for (int g0 = 0; g0 < gpad; g0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int g = g0 + u;
      const unsigned char* st = xs + (u & 1) * XSTAGE;  // g0 is even
      f4 d[WT][TT];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8 bx[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) bx[tt] = *reinterpret_cast<const half8*>(st + (tt * 4 + j) * XSLOT + lane * 16);
#pragma unroll
        for (int i = 0; i < WT; ++i) {
          h2 q[4];
          unpack8(wv[u][i][j], magic, q);
          const u32x4 qa = {__builtin_bit_cast(uint32_t, q[0]), __builtin_bit_cast(uint32_t, q[1]),
                            __builtin_bit_cast(uint32_t, q[2]), __builtin_bit_cast(uint32_t, q[3])};
          const half8 a = __builtin_bit_cast(half8, qa);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            d[i][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bx[tt], j == 0 ? f4{0.0f, 0.0f, 0.0f, 0.0f} : d[i][tt],
                                                              0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) scale_acc(acc[i][tt], d[i][tt], sv[u][i]);
      load_w(g + PD, wv[u], sv[u]);
      // activations of group g+1 into the other stage (its readers passed the
      // previous barrier), and group g+3 into the registers just freed
      store_x((u + 1) & 1, xr[(u + 1) & 1]);
      load_x(g + 3, xr[(u + 1) & 1]);
      lds_barrier();
    }
  }

  // ---- epilogue: acc[i][tt][r] is tile t0+i, tile row 4*kb + r, chunk row m0 + 16tt + col
#pragma unroll
  for (int i = 0; i < WT; ++i) {
    const int t = t0 + i;
    if (t >= p.T) continue;  // wave-uniform
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int m = m0 + 16 * tt + col;
      const bool mok = m < p.M;
      const f4 v = acc[i][tt];
      f4 vp = v;  // the same rows of the other half tile (row r ^ 8 lives in lane ^ 32)
      if constexpr (EPI == NQ_EPI_SWIGLU_F16 || EPI == EPI_PREFILL_QKV) {
#pragma unroll
        for (int r = 0; r < 4; ++r) vp[r] = __shfl_xor(v[r], 32);
      }
      if (!mok) continue;
      const int64_t N = p.N;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = 4 * kb + r;
        const int64_t n = tile_row_logical(p.kind, p.N, p.head_dim, t, rr);
        const float yv = v[r], yp = vp[r];
        if constexpr (EPI == NQ_EPI_STORE_F16) {
          if (n < N) static_cast<half_t*>(p.y)[m * N + n] = static_cast<half_t>(yv);
        } else if constexpr (EPI == NQ_EPI_BIAS_F16) {
          if (n < N) static_cast<half_t*>(p.y)[m * N + n] = static_cast<half_t>(yv + static_cast<float>(p.bias[n]));
        } else if constexpr (EPI == NQ_EPI_STORE_F32) {
          if (n < N) static_cast<float*>(p.y)[m * N + n] = yv;
        } else if constexpr (EPI == NQ_EPI_RESIDUAL_F16) {
          if (n < N) {
            half_t* yo = static_cast<half_t*>(p.y) + m * N + n;
            const half_t o = static_cast<half_t>(static_cast<float>(*yo) + yv);
            *yo = o;
            if (p.y2) p.y2[m * N + n] = o;
          }
        } else if constexpr (EPI == NQ_EPI_SWIGLU_F16) {
          if (kb < 2) {  // gate rows; the matching up rows are in lane ^ 32
            const float a = yv / (1.0f + expf(-yv)) * yp;
            static_cast<half_t*>(p.y)[m * (N / 2) + 8 * t + rr] = static_cast<half_t>(a);
          }
        } else if constexpr (EPI == EPI_PREFILL_QKV) {
          const int np = static_cast<int>(tile_row_logical(p.kind, p.N, p.head_dim, t, rr ^ 8));
          const int dd = p.head_dim, half = dd / 2;
          const int hb = static_cast<int>(n / dd), i2 = static_cast<int>(n % dd);
          const int ps = p.pos0 + m;
          const half_t v16 = static_cast<half_t>(yv + static_cast<float>(p.bias[n]));
          half_t outv = v16;
          if (hb < p.n_heads + p.n_kv) {  // q and k: rotate-half RoPE at position ps
            if (ps < 0 || ps >= p.max_pos) {
              raise_flag(p.err, 1);
              continue;
            }
            const float2 cs =
                *reinterpret_cast<const float2*>(p.rope + (static_cast<int64_t>(ps) * half + i2 % half) * 2);
            const float xi = static_cast<float>(v16);
            const float xp = static_cast<float>(static_cast<half_t>(yp + static_cast<float>(p.bias[np])));
            outv = static_cast<half_t>(i2 < half ? xi * cs.x - xp * cs.y : xi * cs.x + xp * cs.y);
          }
          if (hb < p.n_heads) {
            static_cast<half_t*>(p.y)[(static_cast<int64_t>(m) * p.n_heads + hb) * dd + i2] = outv;
          } else {
            const bool is_k = hb < p.n_heads + p.n_kv;
            const int kvh = is_k ? hb - p.n_heads : hb - p.n_heads - p.n_kv;
            const int pg = ps / kPageTokens;
            const int page = (ps >= 0 && pg < p.max_pages) ? p.pt[pg] : -1;
            if (page < 0 || page >= p.num_pages) {
              raise_flag(p.err, 1);
            } else {
              const int64_t blk = (static_cast<int64_t>(page) * p.n_kv + kvh) * kPageTokens * dd;
              const int slot = ps % kPageTokens;
              if (is_k) {
                p.kv_k[blk + slot * dd + i2] = outv;            // token-major
              } else {
                p.kv_v[blk + i2 * kPageTokens + slot] = outv;   // dim-major
              }
            }
          }
        }
      }
    }
  }
}

struct GemmShape {
  int wt, tt;
};

// Tiles per wave and token tiles per workgroup: as many token tiles as the
// chunk fills (the A fragments are reused across them), but enough workgroups
// to cover the 256 CUs.
static GemmShape gemm_shape(int T, int M) {
  const int mt = (M + 15) / 16;
  if (mt <= 1) return {4, 1};
  const int wg2 = (T + 15) / 16 * ((mt + 1) / 2);
  if (wg2 >= 256) return {4, 2};
  return {2, 2};
}

template <int WT, int TT>
static hipError_t launch_gemm_e(int epi, dim3 grid, hipStream_t s, const GemmParams& p) {
  constexpr int PD = 2;
  const dim3 block(64 * kGemmWaves);
  switch (epi) {
    case NQ_EPI_STORE_F16: gemm_w4a16_kernel<WT, TT, PD, NQ_EPI_STORE_F16><<<grid, block, 0, s>>>(p); break;
    case NQ_EPI_BIAS_F16: gemm_w4a16_kernel<WT, TT, PD, NQ_EPI_BIAS_F16><<<grid, block, 0, s>>>(p); break;
    case NQ_EPI_RESIDUAL_F16: gemm_w4a16_kernel<WT, TT, PD, NQ_EPI_RESIDUAL_F16><<<grid, block, 0, s>>>(p); break;
    case NQ_EPI_SWIGLU_F16: gemm_w4a16_kernel<WT, TT, PD, NQ_EPI_SWIGLU_F16><<<grid, block, 0, s>>>(p); break;
    case NQ_EPI_STORE_F32: gemm_w4a16_kernel<WT, TT, PD, NQ_EPI_STORE_F32><<<grid, block, 0, s>>>(p); break;
    case EPI_PREFILL_QKV: gemm_w4a16_kernel<WT, TT, PD, EPI_PREFILL_QKV><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  GemmParams p{};
  p.codes = static_cast<const uint8_t*>(a.packed);
  p.scales = p.codes + codes_bytes(a.N, a.K);
  p.N = a.N;
  p.K = a.K;
  p.kind = a.kind;
  p.head_dim = a.head_dim;
  p.G = a.K / kGroup;
  p.T = static_cast<int>(tiles_of(a.N));
  p.M = a.M;
  p.x = static_cast<const half_t*>(a.x);
  p.bias = static_cast<const half_t*>(a.bias);
  p.y = a.y;
  p.y2 = static_cast<half_t*>(a.y2);
  p.pos0 = a.pos0;
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
  const GemmShape sh = gemm_shape(p.T, a.M);
  const int row_blocks = (p.T + kGemmWaves * sh.wt - 1) / (kGemmWaves * sh.wt);
  p.tok_blocks = (a.M + 16 * sh.tt - 1) / (16 * sh.tt);
  p.work = row_blocks * p.tok_blocks;
  const dim3 grid((p.work + 7) / 8 * 8);
  if (sh.wt == 4 && sh.tt == 1) return launch_gemm_e<4, 1>(a.epi, grid, s, p);
  if (sh.wt == 4 && sh.tt == 2) return launch_gemm_e<4, 2>(a.epi, grid, s, p);
  return launch_gemm_e<2, 2>(a.epi, grid, s, p);
}

// ============================================================== prefill attention
//
// grid (ceil(M/16), n_heads), one wave per workgroup: query head h of the
// chunk rows 16*qb .. +15 (the MFMA columns), positions pos0 + row. The wave
// walks the sequence's pages 0 .. (last position of the block)/16 with one
// online softmax per column; keys after a column's own position are masked,
// and V slots past the block's last position are zeroed (a page's unwritten
// slots may hold anything). The longest blocks are scheduled first.

struct PrefillAttnParams {
  const half_t* q;
  const half_t* kp;
  const half_t* vp;
  const int32_t* pt;
  int max_pages, num_pages;
  int M, pos0, n_heads, n_kv;
  half_t* out;
  int32_t* err;
};

template <int D>
__global__ __launch_bounds__(64) void attn_prefill_kernel(PrefillAttnParams a) {
  constexpr int KJ = D / 32;  // score MFMAs per page
  constexpr int VC = D / 16;  // P.V MFMAs per page
  const int qb = static_cast<int>(gridDim.x) - 1 - static_cast<int>(blockIdx.x);
  const int h = blockIdx.y;
  const int kvh = h / (a.n_heads / a.n_kv);
  const int lane = threadIdx.x, r16 = lane & 15, g4 = lane >> 4;
  const int mq = qb * 16 + r16;
  const int qpos = a.pos0 + min(mq, a.M - 1);              // this column's position
  const int last = a.pos0 + min(qb * 16 + 15, a.M - 1);    // the block's last position
  int npages = last / kPageTokens + 1;
  if (npages > a.max_pages) {
    if (lane == 0) raise_flag(a.err, 2);
    npages = a.max_pages;
  }
  half8 qf[KJ];
  {
    const half_t* qh = a.q + (static_cast<int64_t>(min(mq, a.M - 1)) * a.n_heads + h) * D + 8 * g4;
#pragma unroll
    for (int j = 0; j < KJ; ++j) qf[j] = *reinterpret_cast<const half8*>(qh + 32 * j);
  }
  const float qscale = 1.4426950408889634f / sqrtf(static_cast<float>(D));  // log2(e) / sqrt(d)
  f4 o[VC];
#pragma unroll
  for (int c = 0; c < VC; ++c) o[c] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, l = 0.0f;
  bool bad = false;
  int pid = -1;  // page ids of the current batch of 64 pages, one per lane

  auto load = [&](int k, half8 (&kf)[KJ], half4 (&vf)[VC]) {
    const int id = __builtin_amdgcn_readlane(pid, k);
    const int idc = (id >= 0 && id < a.num_pages) ? id : 0;
    const int64_t base = (static_cast<int64_t>(idc) * a.n_kv + kvh) * (kPageTokens * D);
    const half_t* kb = a.kp + base + r16 * D + 8 * g4;
    const half_t* vb = a.vp + base + r16 * kPageTokens + 4 * g4;
#pragma unroll
    for (int j = 0; j < KJ; ++j) kf[j] = *reinterpret_cast<const half8*>(kb + 32 * j);
#pragma unroll
    for (int c = 0; c < VC; ++c) vf[c] = *reinterpret_cast<const half4*>(vb + 16 * c * kPageTokens);
  };
  auto compute = [&](int k, int page, const half8 (&kf)[KJ], half4 (&vf)[VC]) {
    const int id = __builtin_amdgcn_readlane(pid, k);
    const bool okp = id >= 0 && id < a.num_pages;
    bad |= !okp;
    f4 sc = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < KJ; ++j) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[j], qf[j], sc, 0, 0, 0);
    // lane holds S^T[key 16*page + 4*g4 + i][column r16]
    const int kpos0 = page * kPageTokens + 4 * g4;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (okp && kpos0 + i <= qpos) ? sc[i] * qscale : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
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
    if (!okp || page * kPageTokens + kPageTokens - 1 > last) {  // unwritten slots: zero V
#pragma unroll
      for (int c = 0; c < VC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!okp || kpos0 + i > last) vf[c][i] = static_cast<half_t>(0.0f);
    }
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      o[c] *= alpha;
      o[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf[c], pf, o[c], 0, 0, 0);
    }
  };

  for (int p0 = 0; p0 < npages; p0 += 64) {
    const int nk = min(64, npages - p0);
    pid = lane < nk ? a.pt[p0 + lane] : -1;
    half8 kA[KJ], kB[KJ];
    half4 vA[VC], vB[VC];
    load(0, kA, vA);
    for (int k = 0; k < nk; k += 2) {
      load(min(k + 1, nk - 1), kB, vB);
      compute(k, p0 + k, kA, vA);
      if (k + 1 >= nk) break;
      load(min(k + 2, nk - 1), kA, vA);
      compute(k + 1, p0 + k + 1, kB, vB);
    }
  }
  if (bad && lane == 0) raise_flag(a.err, 2);

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (mq < a.M) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    half_t* orow = a.out + (static_cast<int64_t>(mq) * a.n_heads + h) * D;
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      half4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = static_cast<half_t>(o[c][i] * inv);
      *reinterpret_cast<half4*>(orow + 16 * c + 4 * g4) = ov;
    }
  }
}

hipError_t launch_attn_prefill(const PrefillAttnArgs& a, hipStream_t s) {
  PrefillAttnParams p{};
  p.q = static_cast<const half_t*>(a.q);
  p.kp = static_cast<const half_t*>(a.k_pool);
  p.vp = static_cast<const half_t*>(a.v_pool);
  p.pt = a.page_table;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.M = a.M;
  p.pos0 = a.pos0;
  p.n_heads = a.n_heads;
  p.n_kv = a.n_kv;
  p.out = static_cast<half_t*>(a.out);
  p.err = a.err;
  const dim3 grid((a.M + 15) / 16, a.n_heads);
  if (a.head_dim == 128) {
    attn_prefill_kernel<128><<<grid, dim3(64), 0, s>>>(p);
  } else if (a.head_dim == 64) {
    attn_prefill_kernel<64><<<grid, dim3(64), 0, s>>>(p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nq
