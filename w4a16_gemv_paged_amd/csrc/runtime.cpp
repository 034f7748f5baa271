// Host runtime of libnq: model and KV-cache handles, the decode-step driver,
// HIP-graph capture of the step, and the kernel-level entry points.
//
// The step enqueues, per layer, the fused projections of "How to build your own
// LLM runtime from scratch" ("What it actually builds") and the paged decode
// attention, then the LM head and the greedy argmax; capturing that sequence in
// one graph turns a token into one launch ("The one lesson that generalizes").
#include <algorithm>
#include <cstring>
#include <vector>

#include "common.hpp"

using namespace nq;

struct nq_model {
  nq_config cfg{};
  std::vector<nq_layer_ptrs> layers;
  std::vector<char> bound;
  const void* embed = nullptr;
  const void* final_norm = nullptr;
  const void* lm = nullptr;
  const float* rope = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  int32_t step_mode = NQ_STEP_AUTO;
  uint64_t* step_trace = nullptr;   // stage stamps of the persistent step (measurement), or null
};

struct nq_kv {
  nq_config cfg{};
  void* pool = nullptr;
  size_t bytes = 0;
  int32_t num_pages = 0;
};

struct nq_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int32_t kernels = 0;
};

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Workspace {
  // the persistent step's hand-off state and buffers: first, at offsets that
  // do not depend on the batch or table width, so that the epoch flags a
  // workgroup left at the end of one step are where the next step looks
  int* xflag;
  int* xcdflag;
  int* cnt;
  int* abort;
  void* ps_h;
  void* ps_q;
  void* ps_ao;
  void* ps_act;
  float* apart;
  float* lmval;
  int32_t* lmidx;
  int32_t* err;
  void* h;
  void* qbuf;
  void* attn_o;
  void* act;
  float* part_o;
  float* part_ml;
  float* amax_val;
  int32_t* amax_idx;
  AttnPlan attn;
  size_t total;
};

Workspace carve(const nq_config& c, int32_t batch, int32_t max_pages, uint8_t* base) {
  Workspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  const int32_t qd = c.n_heads * c.head_dim;
  w.xflag = reinterpret_cast<int*>(take(static_cast<size_t>(kPsXcds) * 64 * 4));
  w.xcdflag = reinterpret_cast<int*>(take(static_cast<size_t>(kPsXcds) * kPsXcds * 16 * 4));
  w.cnt = reinterpret_cast<int*>(take(16 * 16 * 4));
  w.abort = reinterpret_cast<int*>(take(256));
  w.ps_h = take(static_cast<size_t>(c.hidden) * 2);
  w.ps_q = take(static_cast<size_t>(qd) * 2);
  w.ps_ao = take(static_cast<size_t>(qd) * 2);
  w.ps_act = take(static_cast<size_t>(c.intermediate) * 2);
  w.apart = reinterpret_cast<float*>(take(static_cast<size_t>(c.n_kv_heads) * kPsMaxSplits *
                                          (c.n_heads / c.n_kv_heads) * (c.head_dim + 4) * 4));
  w.lmval = reinterpret_cast<float*>(take(kPsWG * 4));
  w.lmidx = reinterpret_cast<int32_t*>(take(kPsWG * 4));
  w.attn = attn_plan(batch, c.n_kv_heads, max_pages);
  w.err = reinterpret_cast<int32_t*>(take(256));
  w.h = take(static_cast<size_t>(batch) * c.hidden * 2);
  w.qbuf = take(static_cast<size_t>(batch) * qd * 2);
  w.attn_o = take(static_cast<size_t>(batch) * qd * 2);
  w.act = take(static_cast<size_t>(batch) * c.intermediate * 2);
  w.part_o = reinterpret_cast<float*>(take(static_cast<size_t>(batch) * c.n_heads * w.attn.S * c.head_dim * 4));
  w.part_ml = reinterpret_cast<float*>(take(static_cast<size_t>(batch) * c.n_heads * w.attn.S * 2 * 4));
  const int64_t P = gemv_grid_size(c.vocab, c.hidden, batch);
  w.amax_val = reinterpret_cast<float*>(take(static_cast<size_t>(batch) * P * 4));
  w.amax_idx = reinterpret_cast<int32_t*>(take(static_cast<size_t>(batch) * P * 4));
  w.total = off;
  return w;
}

size_t layer_pool_elems(const nq_config& c, int32_t num_pages) {
  return static_cast<size_t>(num_pages) * c.n_kv_heads * kPageTokens * c.head_dim;
}

nq_status check_io(const nq_model* m, const nq_step_io* io) {
  if (!io) return fail(NQ_ERR_INVALID_ARG, "null step io");
  if (io->batch < 1 || io->batch > m->cfg.max_batch)
    return fail(NQ_ERR_INVALID_ARG, "batch %d outside 1..%d", io->batch, m->cfg.max_batch);
  if (io->max_pages < 1) return fail(NQ_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (io->max_pages > kAttnMaxPages) return fail(NQ_ERR_OUT_OF_RANGE, "max_pages %d > %d", io->max_pages, kAttnMaxPages);
  if (!io->page_table || !io->tokens || !io->pos)
    return fail(NQ_ERR_INVALID_ARG, "page_table, tokens and pos are required");
  if (io->token_hist && io->hist_len < 1) return fail(NQ_ERR_INVALID_ARG, "hist_len must be >= 1");
  return NQ_OK;
}

nq_status check_model_ready(const nq_model* m, const nq_kv* kv, const nq_step_io* io) {
  if (!m || !kv) return fail(NQ_ERR_INVALID_ARG, "null model or kv");
  for (int i = 0; i < m->cfg.layers; ++i)
    if (!m->bound[i]) return fail(NQ_ERR_STATE, "layer %d not bound", i);
  if (!m->embed || !m->final_norm || !m->lm) return fail(NQ_ERR_STATE, "head not bound");
  if (!m->rope) return fail(NQ_ERR_STATE, "RoPE table not bound");
  if (!m->ws) return fail(NQ_ERR_STATE, "workspace not bound");
  nq_status st = check_io(m, io);
  if (st != NQ_OK) return st;
  const Workspace w = carve(m->cfg, io->batch, io->max_pages, nullptr);
  if (w.total > m->ws_bytes)
    return fail(NQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes", m->ws_bytes, w.total);
  const nq_config& a = m->cfg;
  const nq_config& b = kv->cfg;
  if (a.layers != b.layers || a.n_kv_heads != b.n_kv_heads || a.head_dim != b.head_dim)
    return fail(NQ_ERR_INVALID_ARG, "KV cache config does not match the model");
  return NQ_OK;
}

// Whether a step of this model and io runs as the persistent batch-1 kernel.
bool use_persistent(const nq_model* m, const nq_step_io* io) {
  const nq_config& c = m->cfg;
  if (m->step_mode != NQ_STEP_AUTO || io->batch != 1) return false;
  if (c.layers > kPsMaxLayers || io->max_pages > kPsMaxPages) return false;
  // a split holds at most 64 pages per attention wave, and every split its workgroup
  if (c.n_kv_heads < 1 || io->max_pages > 256 * std::min(kPsMaxSplits, kPsWG / c.n_kv_heads)) return false;
  if (!ps_supported(c.head_dim, c.n_heads, c.n_kv_heads) || c.n_kv_heads > 14) return false;
  // at most 8 QKV tiles and one O / down tile per workgroup (the control
  // wave's epilogue lanes)
  const int64_t t_qkv = tiles_of((c.n_heads + 2 * c.n_kv_heads) * c.head_dim), t_h = tiles_of(c.hidden);
  if (t_qkv > 8 * kPsWG || t_h > kPsWG || c.n_heads * c.head_dim != c.hidden) return false;
  return ps_device_ok();
}

int enqueue_step_persistent(nq_model* m, nq_kv* kv, const nq_step_io* io, hipStream_t s) {
  const nq_config& c = m->cfg;
  Workspace w = carve(c, 1, io->max_pages, static_cast<uint8_t*>(m->ws));
  PsParams p{};
  for (int l = 0; l < c.layers; ++l) {
    const nq_layer_ptrs& L = m->layers[l];
    p.layer[l] = PsLayer{static_cast<const uint8_t*>(L.qkv_packed), static_cast<const uint16_t*>(L.qkv_bias),
                         static_cast<const uint8_t*>(L.o_packed), static_cast<const uint8_t*>(L.gate_up_packed),
                         static_cast<const uint8_t*>(L.down_packed), static_cast<const uint16_t*>(L.attn_norm),
                         static_cast<const uint16_t*>(L.mlp_norm)};
  }
  p.L = c.layers;
  p.H = c.hidden;
  p.I = c.intermediate;
  p.nh = c.n_heads;
  p.nkv = c.n_kv_heads;
  p.hd = c.head_dim;
  p.V = c.vocab;
  p.kmax = std::max(c.hidden, c.intermediate);
  // most (tile, segment) units of one matrix per workgroup
  const int64_t qkv_rows = static_cast<int64_t>(c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int64_t shapes[5][2] = {{qkv_rows, c.hidden}, {c.hidden, c.hidden}, {2LL * c.intermediate, c.hidden},
                                {c.hidden, c.intermediate}, {c.vocab, c.hidden}};
  int64_t maxu = 1, sc[5] = {};
  for (int k = 0; k < 5; ++k) {
    const int64_t tiles = (tiles_of(static_cast<int32_t>(shapes[k][0])) + kPsWG - 1) / kPsWG;
    const int64_t segs = (shapes[k][1] / kGroup + kPsSegGroups - 1) / kPsSegGroups;
    maxu = std::max(maxu, tiles * ((segs + 3) / 4 * 4));  // segments of a tile row padded to 4
    sc[k] = tiles * (shapes[k][1] / kGroup) * 32;  // a workgroup's group scales
  }
  p.maxu = static_cast<int>(maxu);
  p.sc_a = static_cast<int>(std::max({sc[0], sc[2], sc[4]}));
  p.sc_b = static_cast<int>(std::max(sc[1], sc[3]));
  p.embed = static_cast<const uint16_t*>(m->embed);
  p.gfinal = static_cast<const uint16_t*>(m->final_norm);
  p.lm = static_cast<const uint8_t*>(m->lm);
  p.rope = m->rope;
  p.max_pos = c.max_pos;
  p.kpool = static_cast<uint16_t*>(kv->pool);
  p.layer_pool = layer_pool_elems(c, kv->num_pages);
  p.num_pages = kv->num_pages;
  p.pt = io->page_table;
  p.max_pages = io->max_pages;
  p.tokens = io->tokens;
  p.pos = io->pos;
  p.hist = io->token_hist;
  p.hist_len = io->hist_len;
  p.logits = io->logits;
  p.layer_out = static_cast<uint16_t*>(io->layer_out);
  p.err = io->err_flag ? io->err_flag : w.err;
  p.eps = c.rms_eps;
  p.xflag = w.xflag;
  p.xcdflag = w.xcdflag;
  p.cnt = w.cnt;
  p.abort = w.abort;
  p.hbuf = static_cast<uint16_t*>(w.ps_h);
  p.qbuf = static_cast<uint16_t*>(w.ps_q);
  p.ao = static_cast<uint16_t*>(w.ps_ao);
  p.act = static_cast<uint16_t*>(w.ps_act);
  p.stage_trace = reinterpret_cast<unsigned long long*>(m->step_trace);
  p.apart = w.apart;
  p.lmval = w.lmval;
  p.lmidx = w.lmidx;
  p.max_polls = 1 << 20;
  const hipError_t e = launch_decode_step_persistent(p, s);
  if (e != hipSuccess) return hip_fail(e, "persistent step launch"), -1;
  return 1;
}

// Enqueue one decode step. Returns the number of kernels launched (>= 0) or -1.
int enqueue_step(nq_model* m, nq_kv* kv, const nq_step_io* io, hipStream_t s) {
  if (use_persistent(m, io)) return enqueue_step_persistent(m, kv, io, s);
  const nq_config& c = m->cfg;
  const int B = io->batch;
  Workspace w = carve(c, B, io->max_pages, static_cast<uint8_t*>(m->ws));
  int32_t* err = io->err_flag ? io->err_flag : w.err;
  const int qkv_n = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const size_t lp = layer_pool_elems(c, kv->num_pages);
  uint16_t* pool = static_cast<uint16_t*>(kv->pool);
  int launches = 0;
  hipError_t e = hipSuccess;
  for (int l = 0; l < c.layers; ++l) {
    const nq_layer_ptrs& L = m->layers[l];
    uint16_t* kbase = pool + static_cast<size_t>(l) * 2 * lp;
    uint16_t* vbase = kbase + lp;

    GemvArgs q{};
    q.packed = L.qkv_packed;
    q.N = qkv_n;
    q.K = c.hidden;
    q.kind = NQ_MAT_QKV;
    q.head_dim = c.head_dim;
    q.batch = B;
    q.x = w.h;
    if (l == 0) {  // the embedding gather happens in this kernel's prologue
      q.x = nullptr;
      q.embed = m->embed;
      q.tokens_in = io->tokens;
      q.vocab = c.vocab;
      q.h_out = w.h;
    }
    q.norm_gain = L.attn_norm;
    q.eps = c.rms_eps;
    q.bias = L.qkv_bias;
    q.y = w.qbuf;
    q.epi = EPI_QKV_ROPE_KV;
    q.pos = io->pos;
    q.page_table = io->page_table;
    q.max_pages = io->max_pages;
    q.num_pages = kv->num_pages;
    q.n_heads = c.n_heads;
    q.n_kv = c.n_kv_heads;
    q.kv_k = kbase;
    q.kv_v = vbase;
    q.rope = m->rope;
    q.max_pos = c.max_pos;
    q.err = err;
    if ((e = launch_gemv(q, s)) != hipSuccess) return hip_fail(e, "qkv gemv launch"), -1;

    AttnArgs at{};
    at.q = w.qbuf;
    at.k_pool = kbase;
    at.v_pool = vbase;
    at.page_table = io->page_table;
    at.max_pages = io->max_pages;
    at.num_pages = kv->num_pages;
    at.lens = io->pos;
    at.len_add = 1;
    at.out = w.attn_o;
    at.part_o = w.part_o;
    at.part_ml = w.part_ml;
    at.batch = B;
    at.n_heads = c.n_heads;
    at.n_kv = c.n_kv_heads;
    at.head_dim = c.head_dim;
    at.splits = w.attn.S;
    at.per = w.attn.per;
    at.dyn = w.attn.dyn;
    at.err = err;
    if ((e = launch_attention(at, s)) != hipSuccess) return hip_fail(e, "attention launch"), -1;

    GemvArgs o{};
    o.packed = L.o_packed;
    o.N = c.hidden;
    o.K = c.n_heads * c.head_dim;
    o.kind = NQ_MAT_PLAIN;
    o.batch = B;
    o.x = w.attn_o;
    o.y = w.h;
    o.epi = NQ_EPI_RESIDUAL_F16;
    o.err = err;
    if ((e = launch_gemv(o, s)) != hipSuccess) return hip_fail(e, "o gemv launch"), -1;

    GemvArgs gu{};
    gu.packed = L.gate_up_packed;
    gu.N = 2 * c.intermediate;
    gu.K = c.hidden;
    gu.kind = NQ_MAT_GATE_UP;
    gu.batch = B;
    gu.x = w.h;
    gu.norm_gain = L.mlp_norm;
    gu.eps = c.rms_eps;
    gu.y = w.act;
    gu.epi = NQ_EPI_SWIGLU_F16;
    gu.err = err;
    if ((e = launch_gemv(gu, s)) != hipSuccess) return hip_fail(e, "gate/up gemv launch"), -1;

    GemvArgs dn{};
    dn.packed = L.down_packed;
    dn.N = c.hidden;
    dn.K = c.intermediate;
    dn.kind = NQ_MAT_PLAIN;
    dn.batch = B;
    dn.x = w.act;
    dn.y = w.h;
    dn.y2 = io->layer_out ? static_cast<uint16_t*>(io->layer_out) + static_cast<size_t>(l) * B * c.hidden : nullptr;
    dn.epi = NQ_EPI_RESIDUAL_F16;
    dn.err = err;
    if ((e = launch_gemv(dn, s)) != hipSuccess) return hip_fail(e, "down gemv launch"), -1;
    launches += w.attn.S > 1 ? 6 : 5;  // the combine kernel runs only when pages are split
  }
  GemvArgs lm{};
  lm.packed = m->lm;
  lm.N = c.vocab;
  lm.K = c.hidden;
  lm.kind = NQ_MAT_LM_HEAD;
  lm.batch = B;
  lm.x = w.h;
  lm.norm_gain = m->final_norm;
  lm.eps = c.rms_eps;
  lm.y = io->logits;
  lm.epi = NQ_EPI_STORE_F32;
  lm.amax_val = w.amax_val;
  lm.amax_idx = w.amax_idx;
  lm.err = err;
  if ((e = launch_gemv(lm, s)) != hipSuccess) return hip_fail(e, "lm head launch"), -1;
  e = launch_argmax_finalize(w.amax_val, w.amax_idx, gemv_grid_size(c.vocab, c.hidden, B), B, io->tokens, io->pos,
                             io->token_hist, io->hist_len, -1, s);
  if (e != hipSuccess) return hip_fail(e, "argmax launch"), -1;
  return launches + 2;
}

struct PrefillWs {
  int32_t* err;
  int32_t* tok;  // next token when the caller passes none
  void* h;
  void* xn;
  void* qbuf;
  void* attn_o;
  void* act;
  float* amax_val;
  int32_t* amax_idx;
  size_t total;
};

PrefillWs carve_prefill(const nq_config& c, int32_t chunk, uint8_t* base) {
  PrefillWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  const size_t qd = static_cast<size_t>(c.n_heads) * c.head_dim;
  uint8_t* flags = take(256);
  w.err = reinterpret_cast<int32_t*>(flags);
  w.tok = reinterpret_cast<int32_t*>(flags ? flags + 64 : nullptr);
  w.h = take(static_cast<size_t>(chunk) * c.hidden * 2);
  w.xn = take(static_cast<size_t>(chunk) * c.hidden * 2);
  w.qbuf = take(static_cast<size_t>(chunk) * qd * 2);
  w.attn_o = take(static_cast<size_t>(chunk) * qd * 2);
  w.act = take(static_cast<size_t>(chunk) * c.intermediate * 2);
  const int64_t P = gemv_grid_size(c.vocab, c.hidden, 1);
  w.amax_val = reinterpret_cast<float*>(take(static_cast<size_t>(P) * 4));
  w.amax_idx = reinterpret_cast<int32_t*>(take(static_cast<size_t>(P) * 4));
  w.total = off;
  return w;
}

// Enqueue a chunked prefill. Returns the number of kernels launched or -1.
int enqueue_prefill(nq_model* m, nq_kv* kv, const nq_prefill_io* io, hipStream_t s) {
  const nq_config& c = m->cfg;
  PrefillWs w = carve_prefill(c, io->chunk, static_cast<uint8_t*>(io->workspace));
  int32_t* err = io->err_flag ? io->err_flag : w.err;
  const int qkv_n = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const size_t lp = layer_pool_elems(c, kv->num_pages);
  uint16_t* pool = static_cast<uint16_t*>(kv->pool);
  const int n = io->n_tokens;
  int launches = 0, mc = 0;
  hipError_t e = hipSuccess;
  for (int c0 = 0; c0 < n; c0 += io->chunk) {
    mc = std::min(io->chunk, n - c0);
    const int pos0 = io->start_pos + c0;
    for (int l = 0; l < c.layers; ++l) {
      const nq_layer_ptrs& L = m->layers[l];
      uint16_t* kbase = pool + static_cast<size_t>(l) * 2 * lp;
      uint16_t* vbase = kbase + lp;
      // layer 0 gathers the chunk's embedding rows into the residual stream
      if ((e = launch_rmsnorm_rows(w.h, l == 0 ? m->embed : nullptr, io->tokens + c0, c.vocab, w.h, L.attn_norm,
                                   c.rms_eps, w.xn, mc, c.hidden, err, s)) != hipSuccess)
        return hip_fail(e, "prefill norm launch"), -1;

      GemmArgs q{};
      q.packed = L.qkv_packed;
      q.N = qkv_n;
      q.K = c.hidden;
      q.kind = NQ_MAT_QKV;
      q.head_dim = c.head_dim;
      q.M = mc;
      q.x = w.xn;
      q.bias = L.qkv_bias;
      q.y = w.qbuf;
      q.epi = EPI_PREFILL_QKV;
      q.pos0 = pos0;
      q.page_table = io->page_table;
      q.max_pages = io->max_pages;
      q.num_pages = kv->num_pages;
      q.n_heads = c.n_heads;
      q.n_kv = c.n_kv_heads;
      q.kv_k = kbase;
      q.kv_v = vbase;
      q.rope = m->rope;
      q.max_pos = c.max_pos;
      q.err = err;
      if ((e = launch_gemm(q, s)) != hipSuccess) return hip_fail(e, "prefill qkv launch"), -1;

      PrefillAttnArgs at{};
      at.q = w.qbuf;
      at.k_pool = kbase;
      at.v_pool = vbase;
      at.page_table = io->page_table;
      at.max_pages = io->max_pages;
      at.num_pages = kv->num_pages;
      at.M = mc;
      at.pos0 = pos0;
      at.n_heads = c.n_heads;
      at.n_kv = c.n_kv_heads;
      at.head_dim = c.head_dim;
      at.out = w.attn_o;
      at.err = err;
      if ((e = launch_attn_prefill(at, s)) != hipSuccess) return hip_fail(e, "prefill attention launch"), -1;

      GemmArgs o{};
      o.packed = L.o_packed;
      o.N = c.hidden;
      o.K = c.n_heads * c.head_dim;
      o.kind = NQ_MAT_PLAIN;
      o.M = mc;
      o.x = w.attn_o;
      o.y = w.h;
      o.epi = NQ_EPI_RESIDUAL_F16;
      o.err = err;
      if ((e = launch_gemm(o, s)) != hipSuccess) return hip_fail(e, "prefill o launch"), -1;

      if ((e = launch_rmsnorm_rows(w.h, nullptr, nullptr, c.vocab, nullptr, L.mlp_norm, c.rms_eps, w.xn, mc,
                                   c.hidden, err, s)) != hipSuccess)
        return hip_fail(e, "prefill norm launch"), -1;

      GemmArgs gu{};
      gu.packed = L.gate_up_packed;
      gu.N = 2 * c.intermediate;
      gu.K = c.hidden;
      gu.kind = NQ_MAT_GATE_UP;
      gu.M = mc;
      gu.x = w.xn;
      gu.y = w.act;
      gu.epi = NQ_EPI_SWIGLU_F16;
      gu.err = err;
      if ((e = launch_gemm(gu, s)) != hipSuccess) return hip_fail(e, "prefill gate/up launch"), -1;

      GemmArgs dn{};
      dn.packed = L.down_packed;
      dn.N = c.hidden;
      dn.K = c.intermediate;
      dn.kind = NQ_MAT_PLAIN;
      dn.M = mc;
      dn.x = w.act;
      dn.y = w.h;
      dn.y2 = io->layer_out
                  ? static_cast<uint16_t*>(io->layer_out) + (static_cast<size_t>(l) * n + c0) * c.hidden
                  : nullptr;
      dn.epi = NQ_EPI_RESIDUAL_F16;
      dn.err = err;
      if ((e = launch_gemm(dn, s)) != hipSuccess) return hip_fail(e, "prefill down launch"), -1;
      launches += 7;
    }
  }
  // the first generated token: LM head of the prompt's last row
  GemvArgs lm{};
  lm.packed = m->lm;
  lm.N = c.vocab;
  lm.K = c.hidden;
  lm.kind = NQ_MAT_LM_HEAD;
  lm.batch = 1;
  lm.x = static_cast<const uint16_t*>(w.h) + static_cast<size_t>(mc - 1) * c.hidden;
  lm.norm_gain = m->final_norm;
  lm.eps = c.rms_eps;
  lm.y = io->logits;
  lm.epi = NQ_EPI_STORE_F32;
  lm.amax_val = w.amax_val;
  lm.amax_idx = w.amax_idx;
  lm.err = err;
  if ((e = launch_gemv(lm, s)) != hipSuccess) return hip_fail(e, "prefill lm head launch"), -1;
  e = launch_argmax_finalize(w.amax_val, w.amax_idx, gemv_grid_size(c.vocab, c.hidden, 1), 1,
                             io->next_token ? io->next_token : w.tok, io->pos_out, nullptr, 0,
                             io->start_pos + n, s);
  if (e != hipSuccess) return hip_fail(e, "prefill argmax launch"), -1;
  return launches + 2;
}

}  // namespace

extern "C" {

nq_status nq_gemv_w4a16(const void* packed, int32_t N, int32_t K, nq_mat_kind kind, int32_t head_dim,
                        int32_t batch, const void* x, const void* norm_gain, float eps, const void* bias,
                        void* y, nq_epilogue epi, void* stream) {
  nq_status st = check_pack_args(N, K, kGroup, kind, head_dim);
  if (st != NQ_OK) return st;
  if (!packed || !x || !y) return fail(NQ_ERR_INVALID_ARG, "nq_gemv_w4a16: null packed, x or y");
  if (!aligned16(packed) || !aligned16(x) || (norm_gain && !aligned16(norm_gain)))
    return fail(NQ_ERR_INVALID_ARG, "nq_gemv_w4a16: packed, x and norm_gain must be 16-byte aligned");
  if (batch < 1 || batch > kMaxBatch) return fail(NQ_ERR_INVALID_ARG, "batch %d outside 1..8", batch);
  if (epi < NQ_EPI_STORE_F16 || epi > NQ_EPI_STORE_F32)
    return fail(NQ_ERR_INVALID_ARG, "unknown epilogue %d", static_cast<int>(epi));
  if (epi == NQ_EPI_SWIGLU_F16 && kind != NQ_MAT_GATE_UP)
    return fail(NQ_ERR_INVALID_ARG, "SwiGLU epilogue needs a GATE_UP matrix");
  if (epi != NQ_EPI_SWIGLU_F16 && kind == NQ_MAT_GATE_UP)
    return fail(NQ_ERR_INVALID_ARG, "a GATE_UP matrix needs the SwiGLU epilogue");
  if (epi == NQ_EPI_BIAS_F16 && !bias) return fail(NQ_ERR_INVALID_ARG, "bias epilogue needs bias");
  if (!(eps > 0.0f) && norm_gain) return fail(NQ_ERR_INVALID_ARG, "eps must be > 0");
  GemvArgs a{};
  a.packed = packed;
  a.N = N;
  a.K = K;
  a.kind = kind;
  a.head_dim = head_dim;
  a.batch = batch;
  a.x = x;
  a.norm_gain = norm_gain;
  a.eps = eps;
  a.bias = bias;
  a.y = y;
  a.epi = epi;
  hipError_t e = launch_gemv(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "nq_gemv_w4a16 launch");
  return NQ_OK;
}

nq_status nq_gemm_w4a16(const void* packed, int32_t N, int32_t K, nq_mat_kind kind, int32_t head_dim, int32_t M,
                        const void* x, const void* bias, void* y, nq_epilogue epi, void* stream) {
  nq_status st = check_pack_args(N, K, kGroup, kind, head_dim);
  if (st != NQ_OK) return st;
  if (!packed || !x || !y) return fail(NQ_ERR_INVALID_ARG, "nq_gemm_w4a16: null packed, x or y");
  if (!aligned16(packed) || !aligned16(x))
    return fail(NQ_ERR_INVALID_ARG, "nq_gemm_w4a16: packed and x must be 16-byte aligned");
  if (M < 1 || M > kPrefillMaxChunk) return fail(NQ_ERR_INVALID_ARG, "M %d outside 1..%d", M, kPrefillMaxChunk);
  if (epi < NQ_EPI_STORE_F16 || epi > NQ_EPI_STORE_F32)
    return fail(NQ_ERR_INVALID_ARG, "unknown epilogue %d", static_cast<int>(epi));
  if (epi == NQ_EPI_SWIGLU_F16 && kind != NQ_MAT_GATE_UP)
    return fail(NQ_ERR_INVALID_ARG, "SwiGLU epilogue needs a GATE_UP matrix");
  if (epi != NQ_EPI_SWIGLU_F16 && kind == NQ_MAT_GATE_UP)
    return fail(NQ_ERR_INVALID_ARG, "a GATE_UP matrix needs the SwiGLU epilogue");
  if (epi == NQ_EPI_BIAS_F16 && !bias) return fail(NQ_ERR_INVALID_ARG, "bias epilogue needs bias");
  GemmArgs a{};
  a.packed = packed;
  a.N = N;
  a.K = K;
  a.kind = kind;
  a.head_dim = head_dim;
  a.M = M;
  a.x = x;
  a.bias = bias;
  a.y = y;
  a.epi = epi;
  hipError_t e = launch_gemm(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "nq_gemm_w4a16 launch");
  return NQ_OK;
}

size_t nq_a8_bytes(int32_t batch, int32_t K) {
  if (batch < 1 || batch > 4 || K <= 0 || K % kGroup != 0) return 0;
  return a8_buffer_bytes(batch, K);
}

nq_status nq_quantize_a8(const void* x, int32_t batch, int32_t K, void* xq, void* stream) {
  if (!x || !xq) return fail(NQ_ERR_INVALID_ARG, "nq_quantize_a8: null x or xq");
  if (!aligned16(x) || !aligned16(xq)) return fail(NQ_ERR_INVALID_ARG, "x and xq must be 16-byte aligned");
  if (batch < 1 || batch > 4) return fail(NQ_ERR_INVALID_ARG, "batch %d outside 1..4", batch);
  if (K <= 0 || K % kGroup != 0) return fail(NQ_ERR_INVALID_ARG, "K must be a positive multiple of 128");
  hipError_t e = launch_quantize_a8(x, batch, K, xq, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "nq_quantize_a8 launch");
  return NQ_OK;
}

nq_status nq_gemv_w4a8(const void* packed, int32_t N, int32_t K, nq_mat_kind kind, int32_t head_dim, int32_t batch,
                       const void* x, const void* xq, const void* bias, void* y, nq_epilogue epi, void* stream) {
  nq_status st = check_pack_args(N, K, kGroup, kind, head_dim);
  if (st != NQ_OK) return st;
  if (!packed || !y || (!x && !xq)) return fail(NQ_ERR_INVALID_ARG, "nq_gemv_w4a8: null packed, y, or both x and xq");
  if (!aligned16(packed) || (x && !aligned16(x)) || (xq && !aligned16(xq)))
    return fail(NQ_ERR_INVALID_ARG, "nq_gemv_w4a8: packed, x and xq must be 16-byte aligned");
  if (batch < 1 || batch > 4) return fail(NQ_ERR_INVALID_ARG, "batch %d outside 1..4", batch);
  if (epi < NQ_EPI_STORE_F16 || epi > NQ_EPI_STORE_F32)
    return fail(NQ_ERR_INVALID_ARG, "unknown epilogue %d", static_cast<int>(epi));
  if (epi == NQ_EPI_SWIGLU_F16 && kind != NQ_MAT_GATE_UP)
    return fail(NQ_ERR_INVALID_ARG, "SwiGLU epilogue needs a GATE_UP matrix");
  if (epi != NQ_EPI_SWIGLU_F16 && kind == NQ_MAT_GATE_UP)
    return fail(NQ_ERR_INVALID_ARG, "a GATE_UP matrix needs the SwiGLU epilogue");
  if (epi == NQ_EPI_BIAS_F16 && !bias) return fail(NQ_ERR_INVALID_ARG, "bias epilogue needs bias");
  if (!xq && !a8_fused_fits(N, K, batch))
    return fail(NQ_ERR_UNSUPPORTED, "K=%d at batch %d does not fit LDS for in-kernel quantisation; "
                                     "quantise with nq_quantize_a8 first", K, batch);
  hipError_t e = launch_gemv_w4a8(packed, N, K, kind, head_dim, batch, x, xq, bias, y, epi,
                                  static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return fail(NQ_ERR_UNSUPPORTED, "nq_gemv_w4a8: shape does not fit LDS");
  if (e != hipSuccess) return hip_fail(e, "nq_gemv_w4a8 launch");
  return NQ_OK;
}

nq_status nq_unpack_weights_dev(const void* packed_dev, int32_t N, int32_t K, int32_t group,
                                nq_mat_kind kind, int32_t head_dim, int8_t* q_out_dev, uint16_t* s_out_dev,
                                void* stream) {
  nq_status st = check_pack_args(N, K, group, kind, head_dim);
  if (st != NQ_OK) return st;
  if (!packed_dev || !q_out_dev || !s_out_dev) return fail(NQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(packed_dev)) return fail(NQ_ERR_INVALID_ARG, "packed must be 16-byte aligned");
  hipError_t e = launch_unpack_dev(packed_dev, N, K, kind, head_dim, q_out_dev, s_out_dev,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "unpack launch");
  return NQ_OK;
}

size_t nq_kv_pool_bytes(const nq_config* cfg, int32_t num_pages) {
  if (nq_config_check(cfg) != NQ_OK || num_pages <= 0) return 0;
  return static_cast<size_t>(cfg->layers) * 2 * layer_pool_elems(*cfg, num_pages) * 2;
}

nq_status nq_kv_alloc(const nq_config* cfg, void* pool_dev, size_t bytes, int32_t num_pages, nq_kv** out) {
  nq_status st = nq_config_check(cfg);
  if (st != NQ_OK) return st;
  if (!pool_dev || !out) return fail(NQ_ERR_INVALID_ARG, "nq_kv_alloc: null pool or out");
  if (num_pages <= 0) return fail(NQ_ERR_INVALID_ARG, "num_pages must be positive");
  if (!aligned16(pool_dev)) return fail(NQ_ERR_INVALID_ARG, "pool must be 16-byte aligned");
  if (bytes < nq_kv_pool_bytes(cfg, num_pages))
    return fail(NQ_ERR_INVALID_ARG, "pool too small: %zu < %zu", bytes, nq_kv_pool_bytes(cfg, num_pages));
  nq_kv* kv = new nq_kv;
  kv->cfg = *cfg;
  kv->pool = pool_dev;
  kv->bytes = bytes;
  kv->num_pages = num_pages;
  *out = kv;
  return NQ_OK;
}

void nq_kv_free(nq_kv* kv) { delete kv; }

nq_status nq_kv_append(nq_kv* kv, int32_t layer, int32_t batch, const int32_t* page_table, int32_t max_pages,
                       const int32_t* pos, const void* k, const void* v, int32_t* err_flag, void* stream) {
  if (!kv) return fail(NQ_ERR_INVALID_ARG, "null kv");
  if (layer < 0 || layer >= kv->cfg.layers) return fail(NQ_ERR_OUT_OF_RANGE, "layer %d out of range", layer);
  if (batch < 1) return fail(NQ_ERR_INVALID_ARG, "batch must be >= 1");
  if (max_pages < 1) return fail(NQ_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (!page_table || !pos || !k || !v) return fail(NQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(k) || !aligned16(v)) return fail(NQ_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  const size_t lp = layer_pool_elems(kv->cfg, kv->num_pages);
  uint16_t* kb = static_cast<uint16_t*>(kv->pool) + static_cast<size_t>(layer) * 2 * lp;
  hipError_t e = launch_kv_append(kb, kb + lp, batch, kv->cfg.n_kv_heads, kv->cfg.head_dim, page_table, max_pages,
                                  kv->num_pages, pos, k, v, err_flag, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv append launch");
  return NQ_OK;
}

size_t nq_attn_workspace_bytes(const nq_config* cfg, int32_t batch, int32_t max_pages) {
  if (nq_config_check(cfg) != NQ_OK || batch < 1 || max_pages < 1 || max_pages > kAttnMaxPages) return 0;
  const int S = attn_plan(batch, cfg->n_kv_heads, max_pages).S;
  if (S < 1) return 0;
  return align256(static_cast<size_t>(batch) * cfg->n_heads * S * cfg->head_dim * 4) +
         align256(static_cast<size_t>(batch) * cfg->n_heads * S * 2 * 4);
}

}  // extern "C"

namespace {

// Argument checks shared by nq_attn_decode and nq_attn_decode_static (the
// workspace is checked by each caller).
nq_status check_attn_args(const nq_kv* kv, int32_t layer, int32_t batch, const void* q, const int32_t* page_table,
                          int32_t max_pages, const int32_t* lens, const void* out) {
  if (!kv) return fail(NQ_ERR_INVALID_ARG, "null kv");
  if (layer < 0 || layer >= kv->cfg.layers) return fail(NQ_ERR_OUT_OF_RANGE, "layer %d out of range", layer);
  if (batch < 1) return fail(NQ_ERR_INVALID_ARG, "batch must be >= 1");
  if (max_pages < 1) return fail(NQ_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (max_pages > kAttnMaxPages) return fail(NQ_ERR_OUT_OF_RANGE, "max_pages %d > %d", max_pages, kAttnMaxPages);
  if (!q || !page_table || !lens || !out) return fail(NQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(q)) return fail(NQ_ERR_INVALID_ARG, "q must be 16-byte aligned");
  return NQ_OK;
}

// Enqueues the attention of a checked call with its partials in ``workspace``.
nq_status enqueue_attn(const nq_kv* kv, int32_t layer, int32_t batch, const void* q, const int32_t* page_table,
                       int32_t max_pages, const int32_t* lens, void* out, void* workspace, int32_t* err_flag,
                       void* stream) {
  const size_t lp = layer_pool_elems(kv->cfg, kv->num_pages);
  const uint16_t* kb = static_cast<const uint16_t*>(kv->pool) + static_cast<size_t>(layer) * 2 * lp;
  AttnArgs a{};
  a.q = q;
  a.k_pool = kb;
  a.v_pool = kb + lp;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.num_pages = kv->num_pages;
  a.lens = lens;
  a.len_add = 0;
  a.out = out;
  a.batch = batch;
  a.n_heads = kv->cfg.n_heads;
  a.n_kv = kv->cfg.n_kv_heads;
  a.head_dim = kv->cfg.head_dim;
  const AttnPlan plan = attn_plan(batch, kv->cfg.n_kv_heads, max_pages);
  if (plan.S < 1)
    return fail(NQ_ERR_OUT_OF_RANGE, "batch %d x max_pages %d is beyond the attention kernels", batch, max_pages);
  a.splits = plan.S;
  a.per = plan.per;
  a.dyn = plan.dyn;
  a.part_o = static_cast<float*>(workspace);
  const size_t o_bytes = align256(static_cast<size_t>(batch) * a.n_heads * a.splits * a.head_dim * 4);
  a.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + o_bytes);
  a.err = err_flag;
  hipError_t e = launch_attention(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return NQ_OK;
}

}  // namespace

extern "C" {

nq_status nq_attn_decode(const nq_kv* kv, int32_t layer, int32_t batch, const void* q, const int32_t* page_table,
                         int32_t max_pages, const int32_t* lens, void* out, void* workspace, size_t ws_bytes,
                         int32_t* err_flag, void* stream) {
  nq_status st = check_attn_args(kv, layer, batch, q, page_table, max_pages, lens, out);
  if (st != NQ_OK) return st;
  if (!workspace) return fail(NQ_ERR_INVALID_ARG, "null workspace");
  if (!aligned16(workspace)) return fail(NQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (ws_bytes < nq_attn_workspace_bytes(&kv->cfg, batch, max_pages))
    return fail(NQ_ERR_INVALID_ARG, "attention workspace too small");
  return enqueue_attn(kv, layer, batch, q, page_table, max_pages, lens, out, workspace, err_flag, stream);
}

nq_status nq_attn_decode_static(const nq_kv* kv, int32_t layer, int32_t batch, const void* q,
                                const int32_t* page_table, int32_t max_pages, const int32_t* lens, void* out,
                                int32_t* err_flag, void* stream) {
  nq_status st = check_attn_args(kv, layer, batch, q, page_table, max_pages, lens, out);
  if (st != NQ_OK) return st;
  const size_t need = nq_attn_workspace_bytes(&kv->cfg, batch, max_pages);
  if (need == 0)
    return fail(NQ_ERR_OUT_OF_RANGE, "batch %d x max_pages %d is beyond the attention kernels", batch, max_pages);
  if (need > kAttnScratchBytes)
    return fail(NQ_ERR_OUT_OF_RANGE, "batch %d x max_pages %d needs %zu bytes of split partials, more than the "
                "%zu-byte library scratch", batch, max_pages, need, kAttnScratchBytes);
  void* ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "attention scratch lookup");
  return enqueue_attn(kv, layer, batch, q, page_table, max_pages, lens, out, ws, err_flag, stream);
}

nq_status nq_attn_prefill(const nq_kv* kv, int32_t layer, int32_t n_q, int32_t start_pos, const void* q,
                          const int32_t* page_table, int32_t max_pages, void* out, int32_t* err_flag,
                          void* stream) {
  if (!kv) return fail(NQ_ERR_INVALID_ARG, "null kv");
  if (layer < 0 || layer >= kv->cfg.layers) return fail(NQ_ERR_OUT_OF_RANGE, "layer %d out of range", layer);
  if (n_q < 1 || n_q > kPrefillMaxChunk) return fail(NQ_ERR_INVALID_ARG, "n_q %d outside 1..%d", n_q, kPrefillMaxChunk);
  if (start_pos < 0) return fail(NQ_ERR_INVALID_ARG, "start_pos must be >= 0");
  if (max_pages < 1) return fail(NQ_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (!q || !page_table || !out) return fail(NQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(q) || !aligned16(out)) return fail(NQ_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (static_cast<int64_t>(start_pos) + n_q > static_cast<int64_t>(max_pages) * kPageTokens)
    return fail(NQ_ERR_OUT_OF_RANGE, "positions up to %lld exceed max_pages * 16",
                static_cast<long long>(start_pos) + n_q - 1);
  const size_t lp = layer_pool_elems(kv->cfg, kv->num_pages);
  const uint16_t* kb = static_cast<const uint16_t*>(kv->pool) + static_cast<size_t>(layer) * 2 * lp;
  PrefillAttnArgs a{};
  a.q = q;
  a.k_pool = kb;
  a.v_pool = kb + lp;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.num_pages = kv->num_pages;
  a.M = n_q;
  a.pos0 = start_pos;
  a.n_heads = kv->cfg.n_heads;
  a.n_kv = kv->cfg.n_kv_heads;
  a.head_dim = kv->cfg.head_dim;
  a.out = out;
  a.err = err_flag;
  hipError_t e = launch_attn_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  return NQ_OK;
}

nq_status nq_model_create(const nq_config* cfg, nq_model** out) {
  nq_status st = nq_config_check(cfg);
  if (st != NQ_OK) return st;
  if (!out) return fail(NQ_ERR_INVALID_ARG, "null out");
  nq_model* m = new nq_model;
  m->cfg = *cfg;
  m->layers.assign(cfg->layers, nq_layer_ptrs{});
  m->bound.assign(cfg->layers, 0);
  *out = m;
  return NQ_OK;
}

nq_status nq_model_bind_layer(nq_model* m, int32_t layer, const nq_layer_ptrs* p) {
  if (!m || !p) return fail(NQ_ERR_INVALID_ARG, "null model or pointers");
  if (layer < 0 || layer >= m->cfg.layers) return fail(NQ_ERR_OUT_OF_RANGE, "layer %d out of range", layer);
  const void* req[] = {p->qkv_packed, p->qkv_bias, p->o_packed, p->gate_up_packed, p->down_packed,
                       p->attn_norm, p->mlp_norm};
  for (const void* q : req) {
    if (!q) return fail(NQ_ERR_INVALID_ARG, "layer %d: null pointer", layer);
    if (!aligned16(q)) return fail(NQ_ERR_INVALID_ARG, "layer %d: pointer not 16-byte aligned", layer);
  }
  m->layers[layer] = *p;
  m->bound[layer] = 1;
  return NQ_OK;
}

nq_status nq_model_bind_head(nq_model* m, const void* embed, const void* final_norm, const void* lm_packed) {
  if (!m || !embed || !final_norm || !lm_packed) return fail(NQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(embed) || !aligned16(final_norm) || !aligned16(lm_packed))
    return fail(NQ_ERR_INVALID_ARG, "head pointers must be 16-byte aligned");
  m->embed = embed;
  m->final_norm = final_norm;
  m->lm = lm_packed;
  return NQ_OK;
}

nq_status nq_model_bind_rope(nq_model* m, const void* rope) {
  if (!m || !rope) return fail(NQ_ERR_INVALID_ARG, "null pointer");
  m->rope = static_cast<const float*>(rope);
  return NQ_OK;
}

size_t nq_workspace_bytes(const nq_config* cfg, int32_t batch, int32_t max_pages) {
  if (nq_config_check(cfg) != NQ_OK || batch < 1 || batch > cfg->max_batch || max_pages < 1 ||
      max_pages > kAttnMaxPages)
    return 0;
  return carve(*cfg, batch, max_pages, nullptr).total;
}

nq_status nq_model_bind_workspace(nq_model* m, void* ws, size_t bytes) {
  if (!m || !ws) return fail(NQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(ws)) return fail(NQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  m->ws = ws;
  m->ws_bytes = bytes;
  return NQ_OK;
}

nq_status nq_model_set_step_trace(nq_model* m, uint64_t* device_buf, int64_t bytes) {
  if (!m) return fail(NQ_ERR_INVALID_ARG, "null model");
  if (!device_buf) {
    m->step_trace = nullptr;
    return NQ_OK;
  }
  const int64_t need = static_cast<int64_t>(kPsWG) * (m->cfg.layers + 1) * 16 * 8;
  if (bytes < need) return fail(NQ_ERR_INVALID_ARG, "step trace buffer of %lld bytes, need %lld", static_cast<long long>(bytes),
                                static_cast<long long>(need));
  if (reinterpret_cast<uintptr_t>(device_buf) % 8 != 0) return fail(NQ_ERR_INVALID_ARG, "step trace buffer not 8-byte aligned");
  m->step_trace = device_buf;
  return NQ_OK;
}

nq_status nq_model_set_step_mode(nq_model* m, int32_t mode) {
  if (!m) return fail(NQ_ERR_INVALID_ARG, "null model");
  if (mode != NQ_STEP_AUTO && mode != NQ_STEP_KERNELS) return fail(NQ_ERR_INVALID_ARG, "unknown step mode %d", mode);
  m->step_mode = mode;
  return NQ_OK;
}

int32_t nq_step_kernels(const nq_model* m, int32_t batch, int32_t max_pages) {
  if (!m || batch < 1) return -1;
  nq_step_io io{};
  io.batch = batch;
  io.max_pages = max_pages;
  if (use_persistent(m, &io)) return 1;
  const AttnPlan a = attn_plan(batch, m->cfg.n_kv_heads, max_pages);
  return m->cfg.layers * (a.S > 1 ? 6 : 5) + 2;
}

void nq_model_destroy(nq_model* m) { delete m; }

nq_status nq_decode_step(nq_model* m, nq_kv* kv, const nq_step_io* io, void* stream) {
  nq_status st = check_model_ready(m, kv, io);
  if (st != NQ_OK) return st;
  if (enqueue_step(m, kv, io, static_cast<hipStream_t>(stream)) < 0) return NQ_ERR_HIP;
  return NQ_OK;
}

size_t nq_prefill_workspace_bytes(const nq_config* cfg, int32_t chunk) {
  if (nq_config_check(cfg) != NQ_OK || chunk < 1 || chunk > kPrefillMaxChunk) return 0;
  return carve_prefill(*cfg, chunk, nullptr).total;
}

nq_status nq_prefill(nq_model* m, nq_kv* kv, const nq_prefill_io* io, void* stream) {
  if (!m || !kv || !io) return fail(NQ_ERR_INVALID_ARG, "null model, kv or io");
  for (int i = 0; i < m->cfg.layers; ++i)
    if (!m->bound[i]) return fail(NQ_ERR_STATE, "layer %d not bound", i);
  if (!m->embed || !m->final_norm || !m->lm) return fail(NQ_ERR_STATE, "head not bound");
  if (!m->rope) return fail(NQ_ERR_STATE, "RoPE table not bound");
  const nq_config& c = m->cfg;
  if (c.layers != kv->cfg.layers || c.n_kv_heads != kv->cfg.n_kv_heads || c.head_dim != kv->cfg.head_dim)
    return fail(NQ_ERR_INVALID_ARG, "KV cache config does not match the model");
  if (io->n_tokens < 1) return fail(NQ_ERR_INVALID_ARG, "n_tokens must be >= 1");
  if (io->start_pos < 0) return fail(NQ_ERR_INVALID_ARG, "start_pos must be >= 0");
  if (io->chunk < 1 || io->chunk > kPrefillMaxChunk)
    return fail(NQ_ERR_INVALID_ARG, "chunk %d outside 1..%d", io->chunk, kPrefillMaxChunk);
  if (io->max_pages < 1) return fail(NQ_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (!io->tokens || !io->page_table || !io->workspace)
    return fail(NQ_ERR_INVALID_ARG, "tokens, page_table and workspace are required");
  if (!aligned16(io->workspace)) return fail(NQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (io->ws_bytes < carve_prefill(c, io->chunk, nullptr).total)
    return fail(NQ_ERR_INVALID_ARG, "prefill workspace too small: %zu < %zu bytes", io->ws_bytes,
                carve_prefill(c, io->chunk, nullptr).total);
  const int64_t end = static_cast<int64_t>(io->start_pos) + io->n_tokens;
  if (end > static_cast<int64_t>(io->max_pages) * kPageTokens)
    return fail(NQ_ERR_OUT_OF_RANGE, "positions up to %lld exceed max_pages * 16", static_cast<long long>(end - 1));
  if (end > c.max_pos)
    return fail(NQ_ERR_OUT_OF_RANGE, "positions up to %lld exceed max_pos %d", static_cast<long long>(end - 1),
                c.max_pos);
  if (enqueue_prefill(m, kv, io, static_cast<hipStream_t>(stream)) < 0) return NQ_ERR_HIP;
  return NQ_OK;
}

nq_status nq_graph_capture(nq_model* m, nq_kv* kv, const nq_step_io* io, void* stream, nq_graph** out) {
  nq_status st = check_model_ready(m, kv, io);
  if (st != NQ_OK) return st;
  if (!out) return fail(NQ_ERR_INVALID_ARG, "null out");
  if (!stream) return fail(NQ_ERR_STATE, "cannot capture the null stream");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone) return fail(NQ_ERR_STATE, "stream is already capturing");
  if ((e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal)) != hipSuccess)
    return hip_fail(e, "hipStreamBeginCapture");
  const int n = enqueue_step(m, kv, io, s);
  hipGraph_t g = nullptr;
  hipError_t e2 = hipStreamEndCapture(s, &g);
  if (n < 0) {
    if (g) (void)hipGraphDestroy(g);
    return NQ_ERR_HIP;
  }
  if (e2 != hipSuccess) return hip_fail(e2, "hipStreamEndCapture");
  hipGraphExec_t ex = nullptr;
  if ((e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0)) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(e, "hipGraphInstantiate");
  }
  nq_graph* gr = new nq_graph;
  gr->graph = g;
  gr->exec = ex;
  gr->kernels = n;
  *out = gr;
  return NQ_OK;
}

nq_status nq_graph_launch(nq_graph* g, void* stream) {
  if (!g) return fail(NQ_ERR_INVALID_ARG, "null graph");
  hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  return NQ_OK;
}

int32_t nq_graph_kernel_count(const nq_graph* g) { return g ? g->kernels : -1; }

void nq_graph_destroy(nq_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}

nq_status nq_check_device_error(int32_t* err_flag_dev, void* stream) {
  if (!err_flag_dev) return fail(NQ_ERR_INVALID_ARG, "null err flag");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int32_t v = 0;
  if ((e = hipMemcpy(&v, err_flag_dev, sizeof v, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "reading err flag");
  if (v != 0) {
    const int32_t zero = 0;
    if ((e = hipMemcpy(err_flag_dev, &zero, sizeof zero, hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "resetting err flag");
    return fail(NQ_ERR_DEVICE_FAULT, "device error flag 0x%x (1 KV write, 2 attention read, 4 token id, 8 NaN logits)", v);
  }
  return NQ_OK;
}

}  // extern "C"
