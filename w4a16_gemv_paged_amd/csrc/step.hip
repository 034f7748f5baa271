// The whole batch-1 greedy decode step as one persistent kernel on MI355X.
//
// "How to build your own LLM runtime from scratch", section "The one lesson
// that generalizes": at batch 1 the fixed cost around each kernel, not the
// arithmetic, decides the step time. Here every projection, the attention and
// the LM head run inside one launch of kPsWG co-resident workgroups (one per
// CU), and the weights never stop streaming at a stage boundary: each
// streaming wave keeps a register ring of kPsRing 1 KiB weight blocks in
// flight along its whole sequence of blocks (layer by layer: QKV, O, gate/up,
// down; then the LM head), so while a stage's results are handed over, the
// next stages' weights are already on their way.
//
// Roles inside a workgroup of kPsWaves waves:
//   * streaming waves 0..kPsStream-1: W4A16 GEMV blocks (the INT4 unpack and
//     matrix-core products of the multi-kernel GEMV, on activations staged in
//     LDS with the RMSNorm gain and the 1/16 pre-scale of the biased codes
//     already applied), partial sums per tile into LDS;
//   * the control wave: epilogues (bias, RoPE, KV-page write, residual,
//     SwiGLU, logits and greedy choice), the hand-off of every stage's output
//     to all workgroups, and the staging of the next stage's input in LDS;
//   * attention waves: split-K paged decode attention of one split of the
//     pages of one KV head (GQA heads as the matrix-core columns), the merge
//     of their split's heads and its stores, and a share of the SwiGLU
//     epilogue.
//
// Hand-offs between workgroups: a stage's outputs are written with sc1 stores
// (coherent across the XCDs' L2s), then a hierarchical barrier: each
// workgroup stores its arrival in a flag its XCD's L2 holds, the first
// workgroup of each XCD publishes the XCD's arrival once all of its 32
// workgroups are in, and every workgroup waits for the 8 XCD flags; the inputs
// are then read with sc1 loads. While a KV head's attention splits fit one
// XCD they all run there, and their merge waits for that XCD's workgroups
// only (plain stores and a flag in that XCD's L2). Every wait is bounded: a
// wait that runs out sets error bit 16 and an abort flag, and all later waits
// return at once, so every wave always reaches the end of the kernel.
#include <mutex>

#include "device.hpp"

namespace nq {

namespace {

constexpr int kPsStream = 7;                  // streaming waves
constexpr int kPsCtrl = kPsStream;            // the control wave
constexpr int kPsAttWave0 = kPsStream + 1;    // first attention wave
constexpr int kPsAtt = 4;                     // attention waves
constexpr int kPsWaves = kPsStream + 1 + kPsAtt;
constexpr int kPsSeg = kPsSegGroups;          // blocks (groups) per unit: a tile's summation segment
constexpr int kPsRingUnits = 6;               // units in flight per streaming wave
constexpr int kPsRing = kPsRingUnits * kPsSeg;  // weight blocks in flight per streaming wave
constexpr int kPsPerXcd = kPsWG / kPsXcds;    // workgroups per XCD
constexpr int kAbortBit = 16;

__device__ __forceinline__ const half_t* hc(const uint16_t* x) { return reinterpret_cast<const half_t*>(x); }
__device__ __forceinline__ half_t* hm(uint16_t* x) { return reinterpret_cast<half_t*>(x); }

__device__ __forceinline__ int ld_sc1(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc1(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A plain store (kept in the XCD's L2, which every workgroup of the XCD reads
// through), completed before the asm block ends.
__device__ __forceinline__ void st_xcd(int* p, int v) {
  asm volatile("global_store_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : : "v"(p), "v"(v) : "memory");
}

// Workgroup barrier of this kernel: the wave's LDS accesses are complete, then
// s_barrier. The weight loads in flight are not waited for: the compiler's
// LDS-scoped fences would make it wait for every outstanding load here (and so
// drain the weight ring at every stage boundary). The asm is a compiler
// barrier for memory accesses.
__device__ __forceinline__ void ps_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}
constexpr int kSc1 = 16;  // cache-policy operand of buffer / LDS-DMA ops: sc1

// Values handed between workgroups, one per lane at any address: relaxed
// agent-scope atomics, i.e. global loads and stores with sc1 (a buffer op would
// need the address in scalar registers and loop over the lanes).
__device__ __forceinline__ void st_h_sc1(half_t* p, half_t v) {
  __hip_atomic_store(reinterpret_cast<unsigned short*>(p), __builtin_bit_cast(unsigned short, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_f_sc1(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_f_sc1(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_i_sc1(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// GEMV stage kinds in the step's sequence (per layer QKV, ATT, O, GU, D; then LM)
enum PsKind : int { K_QKV = 0, K_ATT = 1, K_O = 2, K_GU = 3, K_D = 4, K_LM = 5 };

// A tile's K is summed over fixed segments of kPsSeg groups (units), each
// computed whole by one wave and added in segment order, so a row's result
// does not depend on the tile or workgroup it falls in (rows with equal
// weights give bitwise equal outputs). The waves split a workgroup's (tile,
// segment) units evenly; unit u is segment u % nseg of tile u / nseg.
struct Geo {  // one GEMV stage for this workgroup and wave
  int T, G, t0, nt;     // tiles of the matrix, groups per tile, this workgroup's tiles [t0, t0+nt)
  int nseg;             // segments per tile
  int u0, u1;           // this wave's units [u0, u1) of the workgroup's nt * nseg
};

__device__ __forceinline__ Geo ps_geo(const PsParams& p, int kind, int wg, int wave) {
  Geo g{};
  int N = 0, K = 0;
  switch (kind) {
    case K_QKV: N = (p.nh + 2 * p.nkv) * p.hd; K = p.H; break;
    case K_O: N = p.H; K = p.nh * p.hd; break;
    case K_GU: N = 2 * p.I; K = p.H; break;
    case K_D: N = p.H; K = p.I; break;
    case K_LM: N = p.V; K = p.H; break;
    default: return g;
  }
  g.T = (N + 15) / 16;
  g.G = K / kGroup;
  g.t0 = static_cast<int>(static_cast<int64_t>(g.T) * wg / kPsWG);
  g.nt = static_cast<int>(static_cast<int64_t>(g.T) * (wg + 1) / kPsWG) - g.t0;
  g.nseg = (g.G + kPsSeg - 1) / kPsSeg;
  const int nu = g.nt * g.nseg;
  g.u0 = nu * wave / kPsStream;
  g.u1 = nu * (wave + 1) / kPsStream;
  return g;
}

__device__ __forceinline__ const uint8_t* ps_matrix(const PsParams& p, int layer, int kind) {
  switch (kind) {
    case K_QKV: return p.layer[layer].qkv;
    case K_O: return p.layer[layer].o;
    case K_GU: return p.layer[layer].gu;
    case K_D: return p.layer[layer].d;
    default: return p.lm;
  }
}

__device__ __forceinline__ int ps_stage_kind(int st, int L) { return st >= 5 * L ? K_LM : st % 5; }
__device__ __forceinline__ int ps_stage_layer(int st, int L) { return st >= 5 * L ? L - 1 : st / 5; }

// LDS layout (bytes): xs [kmax] fp16 | gs [H] fp16 | part [tiles][16 rows][segments, padded to 4] f32 |
// att_m [kPsAtt][16] | att_l [kPsAtt][16] | att_o [kPsAtt][16][hd + 4] | geo |
// sca [sc_a] | scb [sc_b]
struct PsLds {
  half_t* xs;
  half_t* gs;
  float* part;
  float* att_m;
  float* att_l;
  float* att_o;
  int* geo;        // [kPsStream][6 kinds][4] each streaming wave's stage geometry
  uint8_t* sca;    // the group scales of this workgroup's tiles: QKV, gate/up, LM head stages
  uint8_t* scb;    // O and down stages
  float* rsv;      // the gate/up input's 1/rms, for the waves that share its epilogue
};

__device__ __forceinline__ PsLds ps_lds(unsigned char* smem, const PsParams& p) {
  PsLds s;
  s.xs = reinterpret_cast<half_t*>(smem);
  s.gs = s.xs + p.kmax;
  s.part = reinterpret_cast<float*>(s.gs + p.H);
  s.att_m = s.part + p.maxu * 16;
  s.att_l = s.att_m + kPsAtt * 16;
  s.att_o = s.att_l + kPsAtt * 16;
  s.geo = reinterpret_cast<int*>(s.att_o + kPsAtt * 16 * (p.hd + 4));
  s.sca = reinterpret_cast<uint8_t*>(s.geo + kPsStream * 6 * 4);
  s.scb = s.sca + p.sc_a;
  s.rsv = reinterpret_cast<float*>(s.scb + p.sc_b);
  return s;
}

// ---------------------------------------------------------------- hand-off

// Control wave: this workgroup's stores are complete; arrive with epoch
// ``target`` and wait until every workgroup has arrived (bounded). x is the
// XCD the workgroup runs on, li its slot among that XCD's workgroups.
__device__ void ps_sync(const PsParams& p, int target, int x, int li) {
  const int lane = threadIdx.x & 63;
  __builtin_amdgcn_s_waitcnt(0);
  if (ld_sc1(p.abort) != 0) return;
  if (lane == 0) st_xcd(p.xflag + x * 64 + li, target);
  bool ok = false;
  for (int it = 0; it < p.max_polls; ++it) {
    bool mine = true;
    if (lane < kPsPerXcd) mine = (ld_sc1(p.xflag + x * 64 + lane) - target) >= 0;
    if (__all(mine)) {
      ok = true;
      break;
    }
    if ((it & 31) == 31 && ld_sc1(p.abort) != 0) return;
    __builtin_amdgcn_s_sleep(1);
  }
  if (ok) {
    // the XCD's arrival, one copy (cache line) per reading XCD: an XCD's 32
    // workgroups poll their own row, so no line has more than 32 pollers
    if (li == 0 && lane < kPsXcds) st_sc1(p.xcdflag + (lane * kPsXcds + x) * 16, target);
    ok = false;
    for (int it = 0; it < p.max_polls; ++it) {
      bool mine = true;
      if (lane < kPsXcds) mine = (ld_sc1(p.xcdflag + (x * kPsXcds + lane) * 16) - target) >= 0;
      if (__all(mine)) {
        ok = true;
        break;
      }
      if ((it & 31) == 31 && ld_sc1(p.abort) != 0) return;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  if (!ok && lane == 0) {
    st_sc1(p.abort, 1);
    raise_flag(p.err, kAbortBit);
  }
}

// Control wave: a barrier of the 32 workgroups of XCD x only. Their arrivals
// (epoch ``target``) sit in the second cache line of the XCD's flag row, held
// by the XCD's L2 like the first; bounded like ps_sync.
__device__ void ps_xcd_sync(const PsParams& p, int target, int x, int li) {
  const int lane = threadIdx.x & 63;
  __builtin_amdgcn_s_waitcnt(0);
  if (ld_sc1(p.abort) != 0) return;
  int* row = p.xflag + x * 64 + kPsPerXcd;
  if (lane == 0) st_xcd(row + li, target);
  for (int it = 0; it < p.max_polls; ++it) {
    bool mine = true;
    if (lane < kPsPerXcd) mine = (ld_sc1(row + lane) - target) >= 0;
    if (__all(mine)) return;
    if ((it & 31) == 31 && ld_sc1(p.abort) != 0) return;
    __builtin_amdgcn_s_sleep(1);
  }
  if (lane == 0) {
    st_sc1(p.abort, 1);
    raise_flag(p.err, kAbortBit);
  }
}

// Control wave: stage K fp16 values into LDS (DMA, 1 KiB per instruction);
// sc1 for values written by other workgroups in this launch.
__device__ __forceinline__ void ps_dma(half_t* dst, const half_t* src, int K, bool coherent) {
  const int lane = threadIdx.x & 63;
  const int n8 = K / 8;  // 16-byte items
  for (int j = 0; j * 64 < n8; ++j) {
    const int item = j * 64 + lane;
    if (item < n8) {
      if (coherent)
        __builtin_amdgcn_global_load_lds(src + item * 8, dst + j * 512, 16, 0, kSc1);
      else
        __builtin_amdgcn_global_load_lds(src + item * 8, dst + j * 512, 16, 0, 0);
    }
  }
}

// The GEMV's activations are staged pre-scaled: the biased high-nibble codes
// are 16 times their value, so the activations at K offsets 2, 3, 6, 7 mod 8
// are taken times 1/16 (exact in fp16 but for subnormals). Stages with an
// RMSNorm also take the gain here; the norm's 1/rms is applied to the outputs.
// The O and down stages' inputs are written pre-scaled by their producers.
__device__ __forceinline__ half_t ps_prescale(half_t v, int k) {
  return v * static_cast<half_t>(high_scale(k & 7));
}

// Control wave: the staged row of K activations in xs taken times fp16(gain *
// pre-scale) in place (fp16 products, as the GEMV would form them; the gain is
// staged in gs). Returns this lane's part of the sum of squares of the row
// before the gain (fp32 accumulation of exact fp16 products).
__device__ __forceinline__ float ps_stage_gain(half_t* xs, const half_t* gs, int K) {
  const int lane = threadIdx.x & 63;
  const h2 sixteenth = {static_cast<half_t>(0.0625f), static_cast<half_t>(0.0625f)};
  constexpr int kBatch = 4;  // items read before any is written back: one LDS latency per batch
  float ss = 0.0f;
  for (int i0 = lane; i0 < K / 8; i0 += 64 * kBatch) {
    uint4 v[kBatch], gv[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = i0 + 64 * k;
      if (i < K / 8) {
        v[k] = *reinterpret_cast<const uint4*>(xs + i * 8);
        gv[k] = *reinterpret_cast<const uint4*>(gs + i * 8);
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = i0 + 64 * k;
      if (i < K / 8) {
        h2* x = reinterpret_cast<h2*>(&v[k]);
        const h2* g = reinterpret_cast<const h2*>(&gv[k]);
#pragma unroll
        for (int q = 0; q < 4; ++q) ss = __builtin_amdgcn_fdot2(x[q], x[q], ss, false);
        x[0] = x[0] * g[0];
        x[1] = x[1] * (g[1] * sixteenth);
        x[2] = x[2] * g[2];
        x[3] = x[3] * (g[3] * sixteenth);
        *reinterpret_cast<uint4*>(xs + i * 8) = v[k];
      }
    }
  }
  return ss;
}

// Control wave: 1/rms of a staged row from the lanes' sums of squares.
__device__ __forceinline__ float ps_rms(float ss, int K, float eps) {
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  return 1.0f / sqrtf(ss / static_cast<float>(K) + eps);
}

// ---------------------------------------------------------------- GEMV block

// The unscaled 16-row products of one 1 KiB block with the staged
// (pre-scaled) activations: per K step a product with the constant -bias
// fragment and one with the biased codes (as in the multi-kernel GEMV). All 16
// matrix-core columns carry the same batch row.
__device__ __forceinline__ f4 ps_block(const u32x4& w, const half_t* xg, uint32_t magic, const half8& nbias) {
  f4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half8 xb = *reinterpret_cast<const half8*>(xg + j * 8);
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(nbias, xb, d, 0, 0, 0);
    h2 q[4];
    unpack8_biased(w[j], magic, q);
    const u32x4 qa = {__builtin_bit_cast(uint32_t, q[0]), __builtin_bit_cast(uint32_t, q[1]),
                      __builtin_bit_cast(uint32_t, q[2]), __builtin_bit_cast(uint32_t, q[3])};
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, qa), xb, d, 0, 0, 0);
  }
  return d;
}

// A tile row's sum over its segments (row-major partials, segments padded to 4),
// added in segment order.
__device__ __forceinline__ float ps_tile_sum(const PsLds& s, const Geo& g0, int tl, int rr) {
  const int sp = (g0.nseg + 3) & ~3;
  const float* r = s.part + (tl * 16 + rr) * sp;
  float v = 0.0f;
  for (int q = 0; q < sp; q += 4) {
    const f4 c = *reinterpret_cast<const f4*>(r + q);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (q + e < g0.nseg) v += c[e];
  }
  return v;
}

// The gate/up epilogue's share of wave wi (0 the control wave, 1.. the
// attention waves): a tile's 8 outputs, SwiGLU of its gate and up rows,
// pre-scaled for the down projection.
__device__ __forceinline__ void ps_gu_epilogue(const PsParams& p, const PsLds& s, int wi, float rs) {
  const int lane = threadIdx.x & 63;
  const Geo gg = ps_geo(p, K_GU, blockIdx.x, 0);
  for (int i = wi * 64 + lane; i < gg.nt * 8; i += (1 + kPsAtt) * 64) {
    const int tl = i / 8, rr = i & 7;
    const float gv = ps_tile_sum(s, gg, tl, rr) * rs, uv = ps_tile_sum(s, gg, tl, rr + 8) * rs;
    st_h_sc1(hm(p.act) + 8 * (gg.t0 + tl) + rr, ps_prescale(static_cast<half_t>(gv / (1.0f + expf(-gv)) * uv), rr));
  }
}

// Barriers each role passes at the end of a stage of the given kind (the
// first barrier of a GEMV stage means "partial sums in LDS", the last one
// "the next stage's input is staged"); before the first stage, one.
__device__ __forceinline__ int ps_end_barriers(int kind) { return kind == K_LM ? 1 : (kind == K_ATT || kind == K_GU) ? 3 : 2; }

// ---------------------------------------------------------------- streaming waves

__device__ __forceinline__ void ps_streaming(const PsParams& p, const PsLds& s, int wave_id) {
  // every cursor below is wave-uniform and lives in scalar registers (the
  // weight loads take their descriptors from them)
  const int wave = __builtin_amdgcn_readfirstlane(wave_id);
  const int lane = threadIdx.x & 63;
  const int kb = lane >> 4;
  const int wg = blockIdx.x;
  const int L = p.L;
  const int last = 5 * L;  // the LM stage
  const uint32_t magic = opaque(0x64006400u);
  const half8 nbias = neg_bias_frag();

  // This wave's geometry of each GEMV kind (the same in every layer), once,
  // into its LDS table: units, first unit, groups per tile, segments per tile.
  int* geo = s.geo + wave * 6 * 4;
  if (lane < 6) {
    const Geo g = ps_geo(p, lane, wg, wave);
    const bool gemv = lane != K_ATT;
    geo[lane * 4 + 0] = gemv ? g.u1 - g.u0 : 0;
    geo[lane * 4 + 1] = gemv ? g.u0 : 0;
    geo[lane * 4 + 2] = gemv ? g.G : 1;
    geo[lane * 4 + 3] = gemv ? g.nseg : 1;
  }
  wave_sync();
  auto field = [&](int kind, int f) { return __builtin_amdgcn_readfirstlane(geo[kind * 4 + f]); };
  auto units = [&](int st) { return field(ps_stage_kind(st, L), 0); };
  // units of the whole sequence, processed in passes of kPsRingUnits
  const int per_layer = units(K_QKV) + units(K_O) + units(K_GU) + units(K_D);
  const int total = L * per_layer + units(last);
  const int passes = (total + kPsRingUnits - 1) / kPsRingUnits;

  // Load cursor: stage, units requested, (tile, segment) of the next unit,
  // and the descriptor of this workgroup's tiles of the stage's matrix. Once
  // the sequence is requested the descriptor is zero-length: its loads return
  // 0 and touch no memory, so every slot is refilled the same way. The blocks
  // past a tile's last group (a short last segment) read the next tile's
  // blocks, or zeros past the workgroup's tiles; their products are dropped.
  int lst = 0, lk = 0, lnu = 0, lG = 1, lnseg = 1, ltl = 0, lseg = 0;
  bool lend = false;
  __amdgpu_buffer_rsrc_t lw = rsrc(nullptr, 0);
  auto load_stage = [&](int st) {
    const int kind = ps_stage_kind(st, L);
    lnu = field(kind, 0);
    const int u0 = field(kind, 1);
    lG = field(kind, 2);
    lnseg = field(kind, 3);
    ltl = u0 / lnseg;
    lseg = u0 - ltl * lnseg;
    lk = 0;
    const Geo gk = ps_geo(p, kind, wg, wave);
    lw = rsrc(ps_matrix(p, ps_stage_layer(st, L), kind) + static_cast<size_t>(gk.t0) * lG * kBlockBytes,
              static_cast<uint32_t>(gk.nt) * lG * kBlockBytes);
  };
  auto skip_empty_loads = [&]() {
    while (!lend && lk >= lnu) {
      if (lst >= last) {  // the whole sequence is requested
        lend = true;
        lw = rsrc(nullptr, 0);
        break;
      }
      ++lst;
      if (units(lst) > 0) load_stage(lst);
    }
  };
  // (the unit's offset goes into the per-lane offset, which the descriptor's
  // range check covers)
  auto load_unit = [&](u32x4& w0, u32x4& w1, u32x4& w2, u32x4& w3) {
    const int o = (ltl * lG + lseg * kPsSeg) * kBlockBytes + lane * 16;
    w0 = __builtin_amdgcn_raw_buffer_load_b128(lw, o, 0, kStreamOnce);
    __builtin_amdgcn_sched_barrier(0);
    w1 = __builtin_amdgcn_raw_buffer_load_b128(lw, o + kBlockBytes, 0, kStreamOnce);
    __builtin_amdgcn_sched_barrier(0);
    w2 = __builtin_amdgcn_raw_buffer_load_b128(lw, o + 2 * kBlockBytes, 0, kStreamOnce);
    __builtin_amdgcn_sched_barrier(0);
    w3 = __builtin_amdgcn_raw_buffer_load_b128(lw, o + 3 * kBlockBytes, 0, kStreamOnce);
    __builtin_amdgcn_sched_barrier(0);
    if (!lend) {
      ++lk;
      if (++lseg == lnseg) {
        lseg = 0;
        ++ltl;
      }
    }
    skip_empty_loads();
  };
  if (units(0) > 0) load_stage(0);
  skip_empty_loads();

  // The ring, one unit (kPsSeg blocks) per step. Loads are issued in the
  // order their slots are consumed (the scheduling barriers keep the compiler
  // from reordering them), so the wait before a unit is for its own loads.
  u32x4 wv[kPsRing];
#pragma unroll
  for (int k = 0; k < kPsRingUnits; ++k) load_unit(wv[4 * k], wv[4 * k + 1], wv[4 * k + 2], wv[4 * k + 3]);

  // Compute cursor: stage, units left, (tile, segment) of the next unit, the
  // stage's group scales in LDS (staged by the control wave).
  bool done = false;
  int cst = 0, cleft = 0, cG = 1, cnseg = 1, ctl = 0, cseg = 0, csp = 4;
  const uint8_t* csc = s.sca;
  auto enter_stage = [&](int st) {
    const int kind = ps_stage_kind(st, L);
    cleft = field(kind, 0);
    const int u0 = field(kind, 1);
    cG = field(kind, 2);
    cnseg = field(kind, 3);
    csp = (cnseg + 3) & ~3;
    ctl = u0 / cnseg;
    cseg = u0 - ctl * cnseg;
    csc = (kind == K_O || kind == K_D) ? s.scb : s.sca;
  };
  // the ends of the current stage and of every empty stage after it
  auto end_stages = [&]() {
    for (;;) {
      const int nb = ps_end_barriers(ps_stage_kind(cst, L));
      for (int b = 0; b < nb; ++b) ps_barrier();
      if (cst >= last) {
        done = true;  // what remains of the last pass is padding
        return;
      }
      ++cst;
      if (units(cst) > 0) break;
    }
    enter_stage(cst);
  };
  // one unit: kPsSeg blocks of tile ctl, groups g0 .. g0 + kPsSeg - 1 (those
  // past the tile's last group, if any, dropped); its partial sums into LDS
  auto compute_unit = [&](const u32x4& w0, const u32x4& w1, const u32x4& w2, const u32x4& w3) {
    const int g0 = cseg * kPsSeg;
    const int len = min(kPsSeg, cG - g0);
    const half_t* xg = s.xs + g0 * kGroup + kb * 32;
    const uint8_t* sg = csc + (ctl * cG + g0) * 32 + kb * 8;
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto blk = [&](const u32x4& w, int i) {
      scale_acc(acc, ps_block(w, xg + i * kGroup, magic, nbias), *reinterpret_cast<const u32x2*>(sg + 32 * i));
    };
    if (len == kPsSeg) {
      // block i's scale is applied while block i + 1 is on the matrix cores
      auto sc = [&](int i) { return *reinterpret_cast<const u32x2*>(sg + 32 * i); };
      const f4 d0 = ps_block(w0, xg, magic, nbias);
      const f4 d1 = ps_block(w1, xg + kGroup, magic, nbias);
      scale_acc(acc, d0, sc(0));
      const f4 d2 = ps_block(w2, xg + 2 * kGroup, magic, nbias);
      scale_acc(acc, d1, sc(1));
      const f4 d3 = ps_block(w3, xg + 3 * kGroup, magic, nbias);
      scale_acc(acc, d2, sc(2));
      scale_acc(acc, d3, sc(3));
    } else {  // a tile's short last segment (len >= 1)
      blk(w0, 0);
      if (len > 1) blk(w1, 1);
      if (len > 2) blk(w2, 2);
    }
    if ((lane & 15) == 0) {  // row-major partials: a tile row's segments are contiguous
      float* dst = s.part + (ctl * 16 + 4 * kb) * csp + cseg;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i * csp] = acc[i];
    }
  };
  ps_barrier();  // the first stage's input is staged
  if (units(0) > 0) enter_stage(0);
  else end_stages();

  for (int pass = 0; pass < passes; ++pass) {
#pragma unroll
    for (int k = 0; k < kPsRingUnits; ++k) {
      if (!done) compute_unit(wv[4 * k], wv[4 * k + 1], wv[4 * k + 2], wv[4 * k + 3]);
      load_unit(wv[4 * k], wv[4 * k + 1], wv[4 * k + 2], wv[4 * k + 3]);
      if (!done) {
        if (++cseg == cnseg) {
          cseg = 0;
          ++ctl;
        }
        if (--cleft == 0) end_stages();
      }
    }
  }
  if (!done) end_stages();  // (no unit at all in any stage)
}

// ---------------------------------------------------------------- attention waves

struct AttPlan {
  int len, npages, per, S;  // context length, pages, pages per split, splits per KV head
  bool local;               // every split of a KV head on one XCD (slots 0..S-1 of XCD j * 8 / nkv)
};

// Splits of kPsSplitPages pages (one per attention wave) while there are
// workgroups for them: a split's pages are dealt to the workgroup's attention
// waves in turn, and a wave's pages are a chain of load latencies (two pages
// in flight), while more splits cost only a few loads per lane of the merge.
// Up to 32 splits per KV head sit on one XCD, whose workgroups merge them
// after a barrier of that XCD alone; beyond that the splits spread over all
// workgroups, which all merge after a full hand-off. At most kPsMaxSplits
// splits per KV head and one workgroup per split; longer contexts take more
// pages per split, up to 64 per wave.
constexpr int kPsSplitPages = 4;
__device__ __forceinline__ AttPlan ps_att_plan(int len, int nkv) {
  AttPlan a;
  a.len = len;
  a.npages = len > 0 ? (len + kPageTokens - 1) / kPageTokens : 0;
  const int smax = min(kPsMaxSplits, kPsWG / nkv);
  int S = (a.npages + kPsSplitPages - 1) / kPsSplitPages;
  S = S < 1 ? 1 : (S > smax ? smax : S);
  int per = (a.npages + S - 1) / S;
  per = (per + kPsAtt - 1) / kPsAtt * kPsAtt;
  a.per = per < kPsAtt ? kPsAtt : per;
  a.S = (a.npages + a.per - 1) / a.per;
  a.local = a.S <= kPsPerXcd && kPsXcds % nkv == 0;
  return a;
}

// The (KV head j, split sp) of the workgroup in slot li of XCD x, if it has
// one. With a local plan, KV head j's splits are slots 0..S-1 of XCD
// j * 8 / nkv, so that their merge waits for that XCD alone; otherwise the
// splits are dealt over the slots x * 32 + li in order.
__device__ __forceinline__ bool ps_att_split(const AttPlan& ap, int nkv, int x, int li, int& j, int& sp) {
  if (ap.local) {
    const int step = kPsXcds / nkv;
    if (x % step != 0 || li >= ap.S) return false;
    j = x / step;
    sp = li;
    return true;
  }
  const int v = x * kPsPerXcd + li;
  if (v >= nkv * ap.S) return false;
  j = v / ap.S;
  sp = v % ap.S;
  return true;
}

constexpr int kPsAttRing = 2;  // pages in flight per attention wave

template <int D, int REP>
__device__ __forceinline__ void ps_attention(const PsParams& p, const PsLds& s, int aw_id, int pos_in) {
  const int aw = __builtin_amdgcn_readfirstlane(aw_id), pos = __builtin_amdgcn_readfirstlane(pos_in);
  constexpr int KJ = D / 32, VC = D / 16;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int L = p.L;
  const AttPlan ap = ps_att_plan(pos + 1, p.nkv);
  // the XCD (hardware register XCC_ID) and, once the control wave has its
  // ticket, the slot of this workgroup decide its split
  const int x = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_s_getreg((31 << 11) | 20) & 0xf) & (kPsXcds - 1);
  ps_barrier();  // the first stage's input is staged (and the slot is in LDS)
  const int li = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(s.rsv)[1]);
  int j = 0, sp = 0;
  const bool active = ps_att_split(ap, p.nkv, x, li, j, sp) && pos >= 0 && ap.npages <= p.max_pages;
  if (!active) j = sp = 0;
  const int p0 = sp * ap.per, p1 = min(ap.npages, p0 + ap.per);
  // this wave's pages: p0 + aw + k * kPsAtt for k < nmine (at most 64)
  const int nmine = active && p0 + aw < p1 ? (p1 - p0 - aw + kPsAtt - 1) / kPsAtt : 0;
  // the page holding this step's token is the last page of the context; its
  // K and V rows of this token are written by other workgroups in this launch
  const bool fresh = nmine > 0 && p0 + aw + (nmine - 1) * kPsAtt == ap.npages - 1;
  const float qscale = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  int pid_reg = -1;  // page id of this wave's k-th page held in lane k
  if (lane < nmine) pid_reg = p.pt[p0 + aw + lane * kPsAtt];
  auto page_id = [&](int k) { return __builtin_amdgcn_readlane(pid_reg, k & 63); };

  // Page k of layer l's K and V into registers, with sc1 loads (coherent with
  // the other XCDs' stores of this step's token; the pages are read once per
  // step, so bypassing the XCD's L2 costs nothing). Past the wave's last page
  // the loads take a zero-length descriptor: they return zeros and touch no
  // memory, so every page slot issues the same loads and the waits stay exact.
  auto load_l = [&](int l, int k, half8 (&kf)[KJ], half4 (&vf)[VC]) {
    const half_t* kp = hc(p.kpool) + static_cast<size_t>(l) * 2 * p.layer_pool;
    const half_t* vp = kp + p.layer_pool;
    const int id = page_id(k);
    const bool ok = k < nmine && id >= 0 && id < p.num_pages;
    const int64_t base = (static_cast<int64_t>(ok ? id : 0) * p.nkv + j) * (kPageTokens * D);
    const uint32_t bytes = ok ? kPageTokens * D * 2 : 0;
    const __amdgpu_buffer_rsrc_t kr = rsrc(kp + base, bytes);
    const __amdgpu_buffer_rsrc_t vr = rsrc(vp + base, bytes);
#pragma unroll
    for (int jj = 0; jj < KJ; ++jj)
      kf[jj] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(kr, (r16 * D + 8 * g4 + 32 * jj) * 2, 0, kSc1));
#pragma unroll
    for (int c = 0; c < VC; ++c)
      vf[c] = __builtin_bit_cast(half4, __builtin_amdgcn_raw_buffer_load_b64(vr, ((16 * c + r16) * kPageTokens + 4 * g4) * 2, 0, kSc1));
  };
  // A layer's first pages are requested long before its QKV results exist
  // (layer 0's here, the next layer's once this one's gate/up outputs are
  // stored), unless the wave holds this step's token.
  half8 kA[kPsAttRing][KJ];
  half4 vA[kPsAttRing][VC];
  if (!fresh) {
#pragma unroll
    for (int r = 0; r < kPsAttRing; ++r) load_l(0, r, kA[r], vA[r]);
  }

  for (int l = 0; l < L; ++l) {
    auto load = [&](int k, half8 (&kf)[KJ], half4 (&vf)[VC]) { load_l(l, k, kf, vf); };

    ps_barrier();  // QKV partials
    ps_barrier();  // q and this step's K/V are everywhere

    f4 o[VC];
#pragma unroll
    for (int c = 0; c < VC; ++c) o[c] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, lsum = 0.0f;
    bool bad = false;
    if (nmine > 0) {
      if (fresh) {
#pragma unroll
        for (int r = 0; r < kPsAttRing; ++r) load(r, kA[r], vA[r]);
      }
      half8 qf[KJ];
      {
        const __amdgpu_buffer_rsrc_t qr = rsrc(p.qbuf, static_cast<uint32_t>(p.nh) * D * 2);
        const int qo = ((j * REP + (r16 < REP ? r16 : 0)) * D + 8 * g4) * 2;
#pragma unroll
        for (int jj = 0; jj < KJ; ++jj)
          qf[jj] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(qr, qo + 64 * jj, 0, kSc1));
        // q (and the first pages) complete before the loop, so that the waits
        // inside it are for the page each step consumes only
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (r16 >= REP) {
#pragma unroll
          for (int jj = 0; jj < KJ; ++jj) qf[jj] = half8{};
        }
      }
      auto compute = [&](int k, const half8 (&kf)[KJ], half4 (&vf)[VC]) {  // vf is masked in place
        const int id = page_id(k);
        const bool okp = id >= 0 && id < p.num_pages;
        bad |= !okp;
        const int valid = okp ? min(kPageTokens, ap.len - (p0 + aw + k * kPsAtt) * kPageTokens) : 0;
        f4 sc = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int jj = 0; jj < KJ; ++jj) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[jj], qf[jj], sc, 0, 0, 0);
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = (4 * g4 + i < valid) ? sc[i] * qscale : -INFINITY;
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
        lsum = lsum * alpha + ps;
        m = mnew;
        if (valid < kPageTokens) {
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
      // kPsAttRing pages in flight: page k's slot is refilled with page
      // k + kPsAttRing as soon as page k is consumed
      for (int k0 = 0; k0 < nmine; k0 += kPsAttRing) {
#pragma unroll
        for (int r = 0; r < kPsAttRing; ++r) {
          if (k0 + r < nmine) compute(k0 + r, kA[r], vA[r]);
          load(k0 + r + kPsAttRing, kA[r], vA[r]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else if (!fresh) {
      __builtin_amdgcn_s_waitcnt(0);  // (zero-length loads)
    }
    if (bad && lane == 0) raise_flag(p.err, 2);
    // this wave's (max, sum, output) of each head into LDS for the control wave
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (g4 == 0) {
      s.att_m[aw * 16 + r16] = m;
      s.att_l[aw * 16 + r16] = lsum;
    }
#pragma unroll
    for (int c = 0; c < VC; ++c) *reinterpret_cast<f4*>(&s.att_o[(aw * 16 + r16) * (D + 4) + 16 * c + 4 * g4]) = o[c];
    ps_barrier();  // attention partials in LDS
    if (active) {
      // this split: the four waves' partials merged per head, heads aw, aw + 4,
      // ... on this wave (a lane takes columns lane + 64 c), then stored: the
      // attention output itself with one split, else the split's (output,
      // max, sum) of each head
      constexpr int R = D + 4;      // a head's row of split partials: output, max, sum, pad
      constexpr int NPH = D / 64;   // columns per head per lane
      static_assert(D % 64 == 0, "whole columns per lane");
      for (int h = aw; h < REP; h += kPsAtt) {
        float M = -INFINITY;
#pragma unroll
        for (int a = 0; a < kPsAtt; ++a) M = fmaxf(M, s.att_m[a * 16 + h]);
        float Ls = 0.0f, Oh[NPH];
#pragma unroll
        for (int c = 0; c < NPH; ++c) Oh[c] = 0.0f;
#pragma unroll
        for (int a = 0; a < kPsAtt; ++a) {
          const float ma = s.att_m[a * 16 + h];
          const float f = ma == -INFINITY ? 0.0f : exp2f(ma - M);
          Ls = fmaf(f, s.att_l[a * 16 + h], Ls);
#pragma unroll
          for (int c = 0; c < NPH; ++c) Oh[c] = fmaf(f, s.att_o[(a * 16 + h) * (D + 4) + lane + 64 * c], Oh[c]);
        }
        if (ap.S == 1) {
#pragma unroll
          for (int c = 0; c < NPH; ++c) {
            const int d = lane + 64 * c;
            st_h_sc1(hm(p.ao) + static_cast<int64_t>(j * REP + h) * D + d,
                     ps_prescale(static_cast<half_t>(Ls > 0.0f ? Oh[c] / Ls : 0.0f), d));
          }
        } else {
          float* part = p.apart + static_cast<int64_t>(j * kPsMaxSplits + sp) * REP * R + h * R;
          if (ap.local) {  // read on this XCD only: plain stores, held by its L2
#pragma unroll
            for (int c = 0; c < NPH; ++c) part[lane + 64 * c] = Oh[c];
            if (lane < 2) part[D + lane] = lane == 0 ? M : Ls;
          } else {
#pragma unroll
            for (int c = 0; c < NPH; ++c) st_f_sc1(part + lane + 64 * c, Oh[c]);
            if (lane < 2) st_f_sc1(part + D + lane, lane == 0 ? M : Ls);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the stores are complete before the control wave arrives
    ps_barrier();  // split partials stored
    ps_barrier();  // O input staged
    ps_barrier();  // O partials
    ps_barrier();  // gate/up input staged
    ps_barrier();  // gate/up partials
    ps_gu_epilogue(p, s, 1 + aw, *s.rsv);
    __builtin_amdgcn_s_waitcnt(0);  // the stores are complete before the control wave arrives
    if (l + 1 < L && !fresh) {
#pragma unroll
      for (int r = 0; r < kPsAttRing; ++r) load_l(l + 1, r, kA[r], vA[r]);
    }
    ps_barrier();  // gate/up outputs stored
    ps_barrier();  // down input staged
    ps_barrier();  // down partials
    ps_barrier();  // next stage's input staged
  }
  ps_barrier();  // LM partials
}

// ---------------------------------------------------------------- control wave

// Control wave: the group scales of this workgroup's tiles of one stage (one
// contiguous run of the packed matrix: tile-major, 32 bytes per tile and
// group) into an LDS buffer, by DMA. The streaming waves read them there, so a
// weight block is one load. Complete before the next hand-off's wait.
__device__ __forceinline__ void ps_dma_scales(const PsParams& p, uint8_t* dst, int kind, int layer) {
  const int lane = threadIdx.x & 63;
  const Geo g = ps_geo(p, kind, blockIdx.x, 0);
  const uint8_t* src = ps_matrix(p, layer, kind) + static_cast<size_t>(g.T) * g.G * kBlockBytes +
                       static_cast<size_t>(g.t0) * g.G * 32;
  const int n16 = g.nt * g.G * 2;  // 16-byte items
  for (int c = 0; c * 64 < n16; ++c) {
    const int item = c * 64 + lane;
    if (item < n16) __builtin_amdgcn_global_load_lds(src + item * 16, dst + c * 1024, 16, 0, 0);
  }
}

// Control wave: the attention outputs [o0, o0 + m) (below oend) merged over
// the S splits in memory and stored pre-scaled. Lane i + m g (i < m outputs,
// g < G groups) takes splits g, g + G, ... of output i, four at a time (their
// loads issued together); the G groups are then merged in group order.
template <int D, int REP>
__device__ __forceinline__ void ps_merge_splits(const PsParams& p, int S, int o0, int oend, int m, int G) {
  const int lane = threadIdx.x & 63;
  constexpr int R = D + 4;
  const int i = lane % m, g = lane / m;
  const int o = o0 + i;
  float M = -INFINITY, Ls = 0.0f, O = 0.0f;
  if (g < G && o < oend) {
    const int head = o / D, d = o % D, j = head / REP, h = head % REP;
    const float* pb = p.apart + static_cast<int64_t>(j * kPsMaxSplits) * REP * R + h * R;
    for (int q0 = g; q0 < S; q0 += 4 * G) {
      float mq[4], lq[4], oq[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + G * u;
        mq[u] = -INFINITY;
        lq[u] = oq[u] = 0.0f;
        if (q < S) {
          const float* r = pb + static_cast<int64_t>(q) * REP * R;
          mq[u] = ld_f_sc1(r + D);
          lq[u] = ld_f_sc1(r + D + 1);
          oq[u] = ld_f_sc1(r + d);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (mq[u] != -INFINITY) {
          const float Mn = fmaxf(M, mq[u]);
          const float a = M == -INFINITY ? 0.0f : exp2f(M - Mn), b = exp2f(mq[u] - Mn);
          Ls = Ls * a + lq[u] * b;
          O = O * a + oq[u] * b;
          M = Mn;
        }
      }
    }
  }
  // the G groups of output i, in group order (lanes i, i + m, ...)
  float Mt = __shfl(M, i), Lt = __shfl(Ls, i), Ot = __shfl(O, i);
  for (int gg = 1; gg < G; ++gg) {
    const float mg = __shfl(M, i + gg * m), lg = __shfl(Ls, i + gg * m), og = __shfl(O, i + gg * m);
    if (mg != -INFINITY) {
      const float Mn = fmaxf(Mt, mg);
      const float a = Mt == -INFINITY ? 0.0f : exp2f(Mt - Mn), b = exp2f(mg - Mn);
      Lt = Lt * a + lg * b;
      Ot = Ot * a + og * b;
      Mt = Mn;
    }
  }
  if (g == 0 && o < oend) st_h_sc1(hm(p.ao) + o, ps_prescale(static_cast<half_t>(Lt > 0.0f ? Ot / Lt : 0.0f), o % D));
}

template <int D, int REP>
__device__ __forceinline__ void ps_control(const PsParams& p, const PsLds& s, int pos, int tok, int x,
                                           int slot_ticket) {
  const int lane = threadIdx.x & 63;
  const int wg = blockIdx.x;
  const int L = p.L;
  // this workgroup's slot among the 32 on its XCD (every launch takes exactly
  // 32 tickets per XCD), and its epoch: every slot holds the number of
  // hand-offs every workgroup has passed
  const int li = slot_ticket % kPsPerXcd;
  int epoch = __builtin_amdgcn_readfirstlane(ld_sc1(p.xflag + x * 64 + li));
  int xepoch = __builtin_amdgcn_readfirstlane(ld_sc1(p.xflag + x * 64 + kPsPerXcd + li));  // XCD-local barriers
  const AttPlan ap = ps_att_plan(pos + 1, p.nkv);
  const int qkv_n = (p.nh + 2 * p.nkv) * D;
  // optional stage stamps (realtime counter, 100 MHz): row l of this
  // workgroup holds layer l's 16 events, row L the kernel start, the LM
  // head's partials and the end of this wave's work
  auto stamp = [&](int row, int ev) {
    if (p.stage_trace && lane == 0)
      p.stage_trace[(static_cast<int64_t>(wg) * (L + 1) + row) * 16 + ev] = __builtin_amdgcn_s_memrealtime();
  };
  stamp(L, 0);

  // the residual rows of this workgroup's O / down tile (the same tiles: both
  // have N = H) stay in this wave's lanes 0..15 from layer to layer
  const Geo go = ps_geo(p, K_O, wg, 0);
  const Geo gd = ps_geo(p, K_D, wg, 0);  // the same tiles as go; its K, hence its wave split, differs
  half_t hres = static_cast<half_t>(0.0f);

  // the first stages' scales; stage 0 input: the embedding row of the input
  // token, and the first gain
  ps_dma_scales(p, s.sca, K_QKV, 0);
  ps_dma_scales(p, s.scb, K_O, 0);
  ps_dma(s.xs, hc(p.embed) + static_cast<int64_t>(tok) * p.H, p.H, false);
  ps_dma(s.gs, hc(p.layer[0].g1), p.H, false);
  __builtin_amdgcn_s_waitcnt(0);
  if (go.nt > 0 && lane < 16) hres = s.xs[go.t0 * 16 + lane];
  float ss = ps_stage_gain(s.xs, s.gs, p.H);
  if (lane == 0) reinterpret_cast<int*>(s.rsv)[1] = li;  // for the attention waves
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  ps_barrier();  // stage 0 input staged
  float rs = ps_rms(ss, p.H, p.eps);

  auto tile_sum = [&](const Geo& g0, int tl, int rr) { return ps_tile_sum(s, g0, tl, rr); };

  for (int l = 0; l < L; ++l) {
    const PsLayer& Ly = p.layer[l];
    // ---- QKV: prefetch the epilogue's inputs while the streaming waves work
    const Geo gq = ps_geo(p, K_QKV, wg, 0);
    const int items = gq.nt * 16;
    float e_bias[2] = {0.0f, 0.0f}, e_pbias[2] = {0.0f, 0.0f}, e_cos[2] = {1.0f, 1.0f}, e_sin[2] = {0.0f, 0.0f};
    int e_page = -1;
    const bool pos_ok = pos >= 0 && pos < p.max_pos && pos / kPageTokens < p.max_pages;
    if (pos_ok) e_page = p.pt[pos / kPageTokens];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      if (i < items) {
        const int tl = i / 16, rr = i & 15;
        const int64_t n = tile_row_logical(NQ_MAT_QKV, qkv_n, D, gq.t0 + tl, rr);
        const int64_t np = tile_row_logical(NQ_MAT_QKV, qkv_n, D, gq.t0 + tl, rr ^ 8);
        e_bias[r] = static_cast<float>(hc(Ly.bias)[n]);
        e_pbias[r] = static_cast<float>(hc(Ly.bias)[np]);
        if (pos_ok) {
          const int jj = static_cast<int>(n % D) % (D / 2);
          const float2 cs = *reinterpret_cast<const float2*>(p.rope + (static_cast<int64_t>(pos) * (D / 2) + jj) * 2);
          e_cos[r] = cs.x;
          e_sin[r] = cs.y;
        }
      }
    }
    ps_barrier();  // QKV partials
    stamp(l, 0);
    ps_dma_scales(p, s.sca, K_GU, l);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      if (i < items) {
        const int tl = i / 16, rr = i & 15;
        const float yv = tile_sum(gq, tl, rr) * rs, yp = tile_sum(gq, tl, rr ^ 8) * rs;
        const int64_t n = tile_row_logical(NQ_MAT_QKV, qkv_n, D, gq.t0 + tl, rr);
        const int hb = static_cast<int>(n / D), i2 = static_cast<int>(n % D);
        const half_t v16 = static_cast<half_t>(yv + e_bias[r]);
        half_t outv = v16;
        if (hb < p.nh + p.nkv) {
          const float xi = static_cast<float>(v16), xp = static_cast<float>(static_cast<half_t>(yp + e_pbias[r]));
          outv = static_cast<half_t>(i2 < D / 2 ? xi * e_cos[r] - xp * e_sin[r] : xi * e_cos[r] + xp * e_sin[r]);
        }
        if (hb < p.nh) {
          st_h_sc1(hm(p.qbuf) + n, outv);
        } else if (!pos_ok) {
          raise_flag(p.err, 1);
        } else if (e_page < 0 || e_page >= p.num_pages) {
          raise_flag(p.err, 1);
        } else {
          const bool is_k = hb < p.nh + p.nkv;
          const int kvh = is_k ? hb - p.nh : hb - p.nh - p.nkv;
          const int64_t blk = (static_cast<int64_t>(e_page) * p.nkv + kvh) * kPageTokens * D;
          const int slot = pos % kPageTokens;
          half_t* kp = hm(p.kpool) + static_cast<size_t>(l) * 2 * p.layer_pool;
          if (is_k)
            st_h_sc1(kp + blk + slot * D + i2, outv);                          // token-major
          else
            st_h_sc1(kp + p.layer_pool + blk + i2 * kPageTokens + slot, outv);  // dim-major
        }
      }
    }
    stamp(l, 1);
    ps_sync(p, ++epoch, x, li);
    stamp(l, 2);
    ps_barrier();  // q and this step's K/V are everywhere

    // ---- attention: merge the attention waves' partials, then the splits
    ps_barrier();  // attention partials in LDS
    stamp(l, 3);
    ps_barrier();  // split partials stored (by the attention waves)
    if (ap.S > 1) {
      // Every split is in memory. With a local plan, the 32 workgroups of each
      // KV head's XCD merge that head's outputs (the others go on to the
      // hand-off); otherwise every workgroup merges its share of all outputs.
      if (!ap.local) {
        ps_sync(p, ++epoch, x, li);
        const int m = (p.nh * D + kPsWG - 1) / kPsWG;  // 4 m <= 64: nh * D <= 4096
        ps_merge_splits<D, REP>(p, ap.S, wg * m, p.nh * D, m, 4);
      } else if (x % (kPsXcds / p.nkv) == 0) {
        ps_xcd_sync(p, ++xepoch, x, li);
        constexpr int m = (REP * D + kPsPerXcd - 1) / kPsPerXcd;
        static_assert(m <= 64, "a lane per output");
        const int o0 = x / (kPsXcds / p.nkv) * REP * D;
        ps_merge_splits<D, REP>(p, ap.S, o0 + li * m, o0 + REP * D, m, 64 / m < 4 ? 64 / m : 4);
      }
    }
    stamp(l, 4);
    ps_sync(p, ++epoch, x, li);
    stamp(l, 5);
    ps_dma(s.xs, hc(p.ao), p.nh * D, true);
    __builtin_amdgcn_s_waitcnt(0);
    ps_barrier();  // O input staged

    // ---- O + residual
    ps_barrier();  // O partials
    stamp(l, 6);
    ps_dma_scales(p, s.scb, K_D, l);
    if (go.nt > 0 && lane < 16) {
      const float y = tile_sum(go, 0, lane);
      hres = static_cast<half_t>(static_cast<float>(hres) + y);
      st_h_sc1(hm(p.hbuf) + go.t0 * 16 + lane, hres);
    }
    stamp(l, 7);
    ps_sync(p, ++epoch, x, li);
    stamp(l, 8);
    ps_dma(s.xs, hc(p.hbuf), p.H, true);
    ps_dma(s.gs, hc(Ly.g2), p.H, false);
    __builtin_amdgcn_s_waitcnt(0);
    ss = ps_stage_gain(s.xs, s.gs, p.H);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    ps_barrier();  // gate/up input staged
    rs = ps_rms(ss, p.H, p.eps);
    if (lane == 0) *s.rsv = rs;  // for the attention waves' share of the epilogue (read after the next barrier)

    // ---- gate/up + SwiGLU
    ps_barrier();  // gate/up partials
    stamp(l, 9);
    if (l + 1 < L) ps_dma_scales(p, s.sca, K_QKV, l + 1);
    else ps_dma_scales(p, s.sca, K_LM, l);
    ps_gu_epilogue(p, s, 0, rs);
    ps_barrier();  // gate/up outputs stored (the attention waves' share too)
    stamp(l, 10);
    ps_sync(p, ++epoch, x, li);
    stamp(l, 11);
    ps_dma(s.xs, hc(p.act), p.I, true);
    __builtin_amdgcn_s_waitcnt(0);
    ps_barrier();  // down input staged

    // ---- down + residual
    ps_barrier();  // down partials
    stamp(l, 12);
    if (l + 1 < L) ps_dma_scales(p, s.scb, K_O, l + 1);
    if (gd.nt > 0 && lane < 16) {
      const float y = tile_sum(gd, 0, lane);
      hres = static_cast<half_t>(static_cast<float>(hres) + y);
      st_h_sc1(hm(p.hbuf) + go.t0 * 16 + lane, hres);
      if (p.layer_out) hm(p.layer_out)[static_cast<int64_t>(l) * p.H + go.t0 * 16 + lane] = hres;
    }
    stamp(l, 13);
    ps_sync(p, ++epoch, x, li);
    stamp(l, 14);
    ps_dma(s.xs, hc(p.hbuf), p.H, true);
    ps_dma(s.gs, hc(l + 1 < L ? p.layer[l + 1].g1 : p.gfinal), p.H, false);
    __builtin_amdgcn_s_waitcnt(0);
    ss = ps_stage_gain(s.xs, s.gs, p.H);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    ps_barrier();  // next layer's QKV (or the LM head's) input staged
    stamp(l, 15);
    rs = ps_rms(ss, p.H, p.eps);
  }

  // ---- LM head: fp32 logits, this workgroup's greedy (max, index), and the
  // last workgroup to finish merges all of them
  ps_barrier();  // LM partials
  stamp(L, 1);
  const Geo gl = ps_geo(p, K_LM, wg, 0);
  float best = -INFINITY;
  int bi = 0x7fffffff;
  bool nan = false;
  for (int i = lane; i < gl.nt * 16; i += 64) {
    const int tl = i / 16, rr = i & 15;
    const int n = (gl.t0 + tl) * 16 + rr;
    if (n >= p.V) continue;
    const float y = tile_sum(gl, tl, rr) * rs;
    if (p.logits) p.logits[n] = y;
    if (y != y) {
      nan = true;
    } else if (better(y, n, best, bi)) {
      best = y;
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
  if (__any(nan) && lane == 0) raise_flag(p.err, 8);
  if (lane == 0) {
    st_f_sc1(p.lmval + wg, best);
    __hip_atomic_store(p.lmidx + wg, bi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(p.cnt + 15 * 16, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old == kPsWG - 1) {
    if (lane == 0) st_sc1(p.cnt + 15 * 16, 0);
    best = -INFINITY;
    bi = 0x7fffffff;
    for (int w = lane; w < kPsWG; w += 64) {
      const float v = ld_f_sc1(p.lmval + w);
      const int ix = ld_i_sc1(p.lmidx + w);
      if (better(v, ix, best, bi)) {
        best = v;
        bi = ix;
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
    if (lane == 0) {
      const int t = bi == 0x7fffffff ? 0 : bi;
      p.tokens[0] = t;
      if (p.hist && pos + 1 >= 0 && pos + 1 < p.hist_len) p.hist[pos + 1] = t;
      p.pos[0] = pos + 1;
    }
  }
  stamp(L, 2);
}

template <int D, int REP>
__global__ __launch_bounds__(64 * kPsWaves) __attribute__((amdgpu_waves_per_eu(3)))
void decode_step_kernel(PsParams /* read in place below */) {
  extern __shared__ __align__(16) unsigned char smem[];
  // The parameters are read where the launch put them (the kernel-argument
  // segment), not copied into private memory: they are 2 KiB and indexed by
  // layer at run time.
  const PsParams& p = *(const PsParams*)(__builtin_amdgcn_kernarg_segment_ptr());
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const PsLds s = ps_lds(smem, p);
  // the step's input token and position, read once by every wave
  const int pos = __builtin_amdgcn_readfirstlane(p.pos[0]);
  int tok = __builtin_amdgcn_readfirstlane(p.tokens[0]);
  // The control and attention waves carry the chain between the stages; at a
  // higher issue priority they go ahead of the streaming waves that share
  // their SIMDs (1.3134 against 1.3153 ms/token; the control wave alone, no
  // change).
  if (wave >= kPsCtrl) __builtin_amdgcn_s_setprio(3);
  if (wave == kPsCtrl) {
    const int lane = threadIdx.x & 63;
    // The XCD this workgroup runs on (hardware register XCC_ID): workgroups are
    // dealt to the XCDs in turn, but the turn does not restart at XCD 0 with
    // every launch. One workgroup per CU makes it exactly 32 per XCD; a ticket
    // from the XCD's counter gives each its slot. The ticket's latency hides
    // under the first stage.
    int x = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_s_getreg((31 << 11) | 20) & 0xf);
    int ticket = 0;
    if (lane == 0) ticket = __hip_atomic_fetch_add(p.cnt + 14 * 16 + (x & 7), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    if (lane == 0) {
      if (x >= kPsXcds) {
        st_sc1(p.abort, 1);
        raise_flag(p.err, kAbortBit);
      }
      if (blockIdx.x == 0) {
        if (tok < 0 || tok >= p.V) raise_flag(p.err, 4);
        if (pos < 0 || (pos + kPageTokens) / kPageTokens > p.max_pages) raise_flag(p.err, 2);  // context past the table
        if (ld_sc1(p.abort) != 0) raise_flag(p.err, kAbortBit);  // an earlier step gave up waiting
      }
    }
    if (tok < 0 || tok >= p.V) tok = 0;
    ps_control<D, REP>(p, s, pos, tok, x & 7, ticket);
  } else if (wave < kPsStream) {
    ps_streaming(p, s, wave);
  } else {
    ps_attention<D, REP>(p, s, wave - kPsAttWave0, pos);
  }
}

}  // namespace

size_t ps_lds_bytes(const PsParams& p) {
  const size_t xs = static_cast<size_t>(p.kmax + p.H) * 2;
  const size_t part = static_cast<size_t>(p.maxu) * 16 * 4;
  const size_t att = static_cast<size_t>(kPsAtt) * 16 * 4 * 2 + static_cast<size_t>(kPsAtt) * 16 * (p.hd + 4) * 4;
  const size_t need = xs + part + att + kPsStream * 6 * 4 * 4 + static_cast<size_t>(p.sc_a) + p.sc_b + 16;
  // at least 81 KiB: one workgroup per CU, whatever the registers allow
  return need < 96 * 1024 ? 96 * 1024 : need;
}

template <int D, int REP>
static hipError_t launch_ps(const PsParams& p, size_t lds, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_step_kernel<D, REP>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 152 * 1024);
  if (attr != hipSuccess) return attr;
  decode_step_kernel<D, REP><<<dim3(kPsWG), dim3(64 * kPsWaves), lds, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_decode_step_persistent(const PsParams& p, hipStream_t s) {
  const size_t lds = ps_lds_bytes(p);
  if (lds > 152 * 1024) return hipErrorInvalidValue;
  const int rep = p.nh / p.nkv;
  if (p.hd == 128 && rep == 7) return launch_ps<128, 7>(p, lds, s);
  if (p.hd == 64 && rep == 4) return launch_ps<64, 4>(p, lds, s);
  return hipErrorInvalidValue;
}

bool ps_device_ok() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static signed char ok[kMaxDevices] = {};  // 0 unknown, 1 yes, -1 no
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(mu);
  if (ok[dev] == 0) {
    int cus = 0, per_cu = 0;
    bool good = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus == kPsWG;
    // one workgroup of each instance resident per CU at the largest LDS size it is launched with
    for (const void* k : {reinterpret_cast<const void*>(decode_step_kernel<128, 7>),
                          reinterpret_cast<const void*>(decode_step_kernel<64, 4>)}) {
      good = good && hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, 152 * 1024) == hipSuccess &&
             hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64 * kPsWaves, 152 * 1024) == hipSuccess &&
             per_cu >= 1;
    }
    ok[dev] = good ? 1 : -1;
  }
  return ok[dev] == 1;
}

bool ps_supported(int head_dim, int n_heads, int n_kv) {
  const int rep = n_kv > 0 ? n_heads / n_kv : 0;
  return (head_dim == 128 && rep == 7) || (head_dim == 64 && rep == 4);
}

}  // namespace nq
