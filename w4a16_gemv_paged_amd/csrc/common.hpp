// Internal declarations shared by the host code and the kernel launchers of libnq.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "nq.h"

namespace nq {

constexpr int kTileRows = 16;      // rows per packed tile
constexpr int kGroup = 128;        // quantisation group along K
constexpr int kBlockBytes = 1024;  // packed codes of one (tile, group)
constexpr int kPageTokens = 16;    // KV tokens per page
constexpr int kMaxBatch = 8;

// Record a message for nq_last_error() and return s.
nq_status fail(nq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
nq_status hip_fail(hipError_t e, const char* what);
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Logical row held by tile row r of tile t (see nq_mat_kind).
__host__ __device__ inline int64_t tile_row_logical(int kind, int64_t N, int head_dim, int64_t t,
                                                    int r) {
  if (kind == NQ_MAT_QKV) {
    const int64_t tiles_per_head = head_dim / 16;
    const int64_t hb = t / tiles_per_head, u = t % tiles_per_head;
    return hb * head_dim + (r < 8 ? 8 * u + r : head_dim / 2 + 8 * u + (r - 8));
  }
  if (kind == NQ_MAT_GATE_UP) {
    const int64_t half = N / 2;
    return r < 8 ? 8 * t + r : half + 8 * t + (r - 8);
  }
  return 16 * t + r;
}

// Validates (N, K, group, kind, head_dim) for packing; sets the error message.
nq_status check_pack_args(int32_t N, int32_t K, int32_t group, nq_mat_kind kind, int32_t head_dim);

inline int64_t padded_rows(int32_t N) { return (static_cast<int64_t>(N) + 15) / 16 * 16; }
inline int64_t tiles_of(int32_t N) { return padded_rows(N) / 16; }
inline size_t codes_bytes(int32_t N, int32_t K) {
  return static_cast<size_t>(tiles_of(N)) * (K / kGroup) * kBlockBytes;
}

// ------------------------------------------------------------------ kernels

// Internal epilogues beyond the public nq_epilogue values.
enum InternalEpi : int {
  EPI_QKV_ROPE_KV = 16,  // bias, RoPE on q/k, q -> qbuf, k/v -> KV pool (decode step)
  EPI_PREFILL_QKV = 17,  // the same for the rows of a prefill chunk, positions pos0 + row, one sequence
};

struct GemvArgs {
  const void* packed = nullptr;
  int32_t N = 0, K = 0, kind = 0, head_dim = 0, batch = 1;
  const void* x = nullptr;          // fp16 [B][K]
  const void* norm_gain = nullptr;  // fp16 [K] or null
  float eps = 1e-6f;
  const void* bias = nullptr;       // fp16 [N]
  void* y = nullptr;                // output
  void* y2 = nullptr;               // optional copy of the residual output (layer_out)
  int epi = 0;
  // embedding gather folded into the prologue (layer 0 of the step)
  const void* embed = nullptr;
  const int32_t* tokens_in = nullptr;
  int32_t vocab = 0;
  void* h_out = nullptr;
  // LM head: per-workgroup greedy (max, index) partials [B][grid]
  float* amax_val = nullptr;
  int32_t* amax_idx = nullptr;
  // QKV epilogue
  const int32_t* pos = nullptr;
  const int32_t* page_table = nullptr;
  int32_t max_pages = 0, num_pages = 0, n_heads = 0, n_kv = 0;
  void* kv_k = nullptr;             // layer's K pool base
  void* kv_v = nullptr;             // layer's V pool base
  const float* rope = nullptr;      // [max_pos][d/2][2]
  int32_t max_pos = 0;
  int32_t* err = nullptr;
};
hipError_t launch_gemv(const GemvArgs& a, hipStream_t s);
int gemv_grid_size(int32_t N, int32_t K, int32_t batch);

struct AttnArgs {
  const void* q = nullptr;          // fp16 [B][nh][d]
  const void* k_pool = nullptr;     // layer K base: [page][nkv][16 tokens][d]
  const void* v_pool = nullptr;     // layer V base: [page][nkv][d][16 tokens]
  const int32_t* page_table = nullptr;
  int32_t max_pages = 0, num_pages = 0;
  const int32_t* lens = nullptr;    // [B]
  int32_t len_add = 0;              // 1 when lens points at positions (decode step)
  void* out = nullptr;              // fp16 [B][nh][d]
  float* part_o = nullptr;          // [B][nh][S][d]
  float* part_ml = nullptr;         // [B][nh][S][2]
  int32_t batch = 1, n_heads = 0, n_kv = 0, head_dim = 0;
  int32_t splits = 1, per = 8;      // from attn_plan(batch, n_kv, max_pages)
  int32_t dyn = 0;                  // the same plan's split mode
  int32_t* err = nullptr;
};
// Split of the pages over workgroups. Fixed (dyn 0): S splits of ``per`` pages
// of every sequence. By length (dyn 1): S workgroups per KV head share all
// sequences' pages, ``per`` the most pages one split can get. S = 0: the batch
// and table width are beyond what the kernels cover.
struct AttnPlan {
  int32_t S = 1, per = 8, dyn = 0;
};
constexpr int32_t kAttnMaxSplits = 1024;  // workgroups per KV head
constexpr int32_t kAttnMaxBatch = 64;     // sequences of a split-by-length launch
AttnPlan attn_plan(int32_t batch, int32_t n_kv, int32_t max_pages);
// Largest page-table width the attention kernels cover (32768 pages, 524288
// tokens); the batch times the width is bounded further by attn_plan (S = 0).
constexpr int32_t kAttnMaxPages = 32768;
size_t attn_partial_bytes(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t splits);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// Library-owned device scratch (scratch.hip) of the entry points that allocate
// nothing: kAttnScratchBytes per GPU; static_scratch gives the current device's
// address (looked up once per device).
constexpr size_t kAttnScratchBytes = NQ_ATTN_SCRATCH_BYTES;
hipError_t static_scratch(void** out);

hipError_t launch_kv_append(void* k_pool, void* v_pool, int32_t batch, int32_t n_kv,
                            int32_t head_dim, const int32_t* page_table, int32_t max_pages,
                            int32_t num_pages, const int32_t* pos, const void* k, const void* v,
                            int32_t* err, hipStream_t s);

// tokens[b] = greedy token; then pos[b] += 1 (and hist[b][pos+1] = token), or
// pos[b] = pos_set when pos_set >= 0 (pos may be null then).
hipError_t launch_argmax_finalize(const float* vals, const int32_t* idx, int32_t partials, int32_t batch,
                                  int32_t* tokens, int32_t* pos, int32_t* hist, int32_t hist_len, int32_t pos_set,
                                  hipStream_t s);

// ------------------------------------------------------------ persistent batch-1 step

// The whole batch-1 decode step as one launch of kPsWG co-resident
// workgroups (step.hip): one per CU of an MI355X, kPsXcds XCDs of 32 CUs.
constexpr int kPsWG = 256;
constexpr int kPsXcds = 8;
constexpr int kPsMaxSplits = 64;    // attention splits per KV head (at most 14 KV heads)
constexpr int kPsMaxLayers = 32;    // per-layer pointers travel in the kernel arguments
constexpr int kPsMaxPages = 16384;  // page-table width (64 splits of 4 waves x 64 pages)
constexpr int kPsSegGroups = 4;     // groups per fixed summation segment of a tile

struct PsLayer {
  const uint8_t* qkv;
  const uint16_t* bias;   // fp16
  const uint8_t* o;
  const uint8_t* gu;
  const uint8_t* d;
  const uint16_t* g1;     // fp16 gains
  const uint16_t* g2;
};

struct PsParams {
  PsLayer layer[kPsMaxLayers];
  int L, H, I, nh, nkv, hd, V;
  int kmax, maxu;                   // longest staged row; most (tile, segment) slots per workgroup, segments padded to 4
  int sc_a, sc_b;                   // LDS bytes of the scale buffers (QKV / gate-up / LM; O / down)
  const uint16_t* embed;
  const uint16_t* gfinal;
  const uint8_t* lm;
  const float* rope;
  int max_pos;
  uint16_t* kpool;                  // K pool of layer 0; V of layer l at + (2l + 1) * layer_pool
  size_t layer_pool;                // fp16 elements of one layer's K (or V) pages
  int num_pages;
  const int32_t* pt;                // the sequence's page-table row
  int max_pages;
  int32_t* tokens;
  int32_t* pos;
  int32_t* hist;
  int hist_len;
  float* logits;                    // optional [V]
  uint16_t* layer_out;              // optional [L][H]
  int32_t* err;
  float eps;
  // workspace: hand-off flags, counters and buffers
  int* xflag;                       // [8][64] per-workgroup epochs, one row per XCD: 0-31 hand-offs, 32-63 XCD-only barriers
  int* xcdflag;                     // [8 reading XCDs][8 XCDs][16] per-XCD epochs, a line each
  int* cnt;                         // [16][16] row 14: per-XCD slot tickets; row 15: LM head
  int* abort;
  uint16_t* hbuf;                   // [H] residual stream
  uint16_t* qbuf;                   // [nh * hd] q after RoPE
  uint16_t* ao;                     // [nh * hd] attention output
  uint16_t* act;                    // [I] SwiGLU output
  float* apart;                     // [nkv][kPsMaxSplits][nh / nkv][hd + 4] split partials: output, max, sum, pad
  float* lmval;                     // [kPsWG] greedy partials
  int32_t* lmidx;
  int max_polls;                    // bound of every wait
  unsigned long long* stage_trace;  // optional [kPsWG][L + 1][16] realtime stamps (see nq_model_set_step_trace)
};
size_t ps_lds_bytes(const PsParams& p);
bool ps_supported(int head_dim, int n_heads, int n_kv);
hipError_t launch_decode_step_persistent(const PsParams& p, hipStream_t s);
// The current device can hold the persistent step: kPsWG CUs, one workgroup
// of the kernel resident on each (checked once per device).
bool ps_device_ok();

// ------------------------------------------------------------ chunked prefill

constexpr int32_t kPrefillMaxChunk = 4096;  // rows of one prefill GEMM / attention call

struct GemmArgs {
  const void* packed = nullptr;
  int32_t N = 0, K = 0, kind = 0, head_dim = 0, M = 0;
  const void* x = nullptr;          // fp16 [M][K]
  const void* bias = nullptr;       // fp16 [N]
  void* y = nullptr;
  void* y2 = nullptr;               // RESIDUAL: optional copy of the result [M][N]
  int epi = 0;
  int32_t pos0 = 0;                 // EPI_PREFILL_QKV
  const int32_t* page_table = nullptr;
  int32_t max_pages = 0, num_pages = 0, n_heads = 0, n_kv = 0;
  void* kv_k = nullptr;
  void* kv_v = nullptr;
  const float* rope = nullptr;
  int32_t max_pos = 0;
  int32_t* err = nullptr;
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

// xn[m] = fp16(x / sqrt(mean(x^2) + eps) * gain) for m < M, with x = h[m], or
// x = embed[tokens[m]] when embed is given (then h[m] = x is stored too).
hipError_t launch_rmsnorm_rows(const void* h_in, const void* embed, const int32_t* tokens, int32_t vocab,
                               void* h_out, const void* gain, float eps, void* xn, int32_t M, int32_t H,
                               int32_t* err, hipStream_t s);

struct PrefillAttnArgs {
  const void* q = nullptr;          // fp16 [M][nh][d]
  const void* k_pool = nullptr;
  const void* v_pool = nullptr;
  const int32_t* page_table = nullptr;  // one sequence: [max_pages]
  int32_t max_pages = 0, num_pages = 0;
  int32_t M = 0, pos0 = 0, n_heads = 0, n_kv = 0, head_dim = 0;
  void* out = nullptr;              // fp16 [M][nh][d]
  int32_t* err = nullptr;
};
hipError_t launch_attn_prefill(const PrefillAttnArgs& a, hipStream_t s);

// ------------------------------------------------------------ W4A8 variant

// Bytes of the INT8 activations of `batch` rows of K inputs: the codes, then
// the (float scale, int32 code sum) pairs of every (row, group), padded to 16.
size_t a8_buffer_bytes(int32_t batch, int32_t K);
hipError_t launch_quantize_a8(const void* x, int32_t batch, int32_t K, void* xq, hipStream_t s);
// Whether the GEMV can quantise its own activations (all of K in LDS).
bool a8_fused_fits(int32_t N, int32_t K, int32_t batch);
// xq == nullptr: quantise x in the prologue; else read the quantised xq.
hipError_t launch_gemv_w4a8(const void* packed, int32_t N, int32_t K, int32_t kind, int32_t head_dim, int32_t batch,
                            const void* x, const void* xq, const void* bias, void* y, int epi, hipStream_t s);

hipError_t launch_unpack_dev(const void* packed, int32_t N, int32_t K, int32_t kind,
                             int32_t head_dim, int8_t* q_out, uint16_t* s_out, hipStream_t s);

}  // namespace nq
