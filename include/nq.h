/*
 * nq.h — C ABI of the MI355X (gfx950) W4A16 paged greedy-decode library (libnq.so).
 *
 * What the library computes is the single-token greedy decode step of a
 * Qwen2-style decoder whose projection weights are symmetric group-wise INT4
 * (group 128, fp16 scales) and whose activations are fp16, with decode
 * attention over a paged KV cache of 16 tokens per page, and the capture of
 * that whole step into one HIP graph. Sources:
 *   - "How to build your own LLM runtime from scratch" (spokes-wiki), section
 *     "What it actually builds": INT4 group-128 symmetric weights, paged KV
 *     cache of 16 tokens per 4 KiB page, fused GEMVs for Q/K/V/O and
 *     gate/up/down, graph capture of the token loop; greedy sampling only
 *     (intro paragraph); launch overhead as the dominant cost ("The one lesson
 *     that generalizes").
 *   - "How To Build Your Own LLM Runtime From Scratch" (daily.dev), Summary and
 *     FAQ: fp16 activations with INT4 weights, 28 layers, the block barrier
 *     that corrupted softmax at partial tail pages.
 *
 * Conventions (all entry points):
 *   - Every call returns nq_status; NQ_OK is 0. nq_last_error() gives a
 *     thread-local message for the last failing call on this thread.
 *   - Arguments are validated before anything is enqueued, so a call that
 *     fails validation has no side effects. No C++ exception crosses the ABI.
 *   - Device memory is owned by the caller (the library never allocates device
 *     memory; the one device buffer it owns is the fixed scratch array of
 *     nq_attn_decode_static, part of the loaded code object); handles store raw
 *     device pointers, which must stay valid while the handle (and any graph
 *     captured from it) is in use.
 *   - "stream" is a hipStream_t passed as void*. Nothing in the decode step
 *     synchronises; results are ready when the stream is.
 *   - Device pointers that the kernels read with 128-bit loads (packed weights,
 *     activations, the KV pool, the workspace) must be 16-byte aligned.
 *   - fp16 means IEEE binary16, passed as raw bits (uint16_t / void*).
 */
#ifndef NQ_H
#define NQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */

typedef enum nq_status {
  NQ_OK = 0,
  NQ_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment, bad enum */
  NQ_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement     */
  NQ_ERR_OUT_OF_RANGE = 3,  /* value outside representable / configured range  */
  NQ_ERR_HIP = 4,           /* a HIP runtime call failed (message has details) */
  NQ_ERR_STATE = 5,         /* call not allowed in the current state           */
  NQ_ERR_DEVICE_FAULT = 6,  /* a kernel flagged a range error (err_flag != 0)  */
  NQ_ERR_IO = 7             /* a file could not be read, written or mapped, or
                               is not a valid packed-weight container          */
} nq_status;

/* Name of a status code ("NQ_OK", ...). Never NULL. */
const char* nq_status_str(nq_status s);

/* Message of the last failing call on the calling thread ("" if none). */
const char* nq_last_error(void);

/* Version of the packed-weight tile layout described at nq_pack_weights. */
int32_t nq_layout_version(void);

/* ---------------------------------------------------------- packed weights */

/* Which rows a 16-row tile co-locates, so that a fused epilogue finds the rows
 * it combines in the same tile. */
typedef enum nq_mat_kind {
  NQ_MAT_PLAIN = 0,    /* tile t holds logical rows 16t .. 16t+15                    */
  NQ_MAT_QKV = 1,      /* fused [Wq; Wk; Wv] (row = head-major, dim-minor). Tile t of
                          head block hb = t / (d/16), u = t % (d/16): rows r < 8 are
                          hb*d + 8u + r, rows r >= 8 are hb*d + d/2 + 8u + (r-8), i.e.
                          the rotate-half RoPE pairs (i, i + d/2) of one head.        */
  NQ_MAT_GATE_UP = 2,  /* fused [Wg; Wu] with N = 2*I: tile t rows r < 8 are gate rows
                          8t + r, rows r >= 8 are up rows I + 8t + (r-8).             */
  NQ_MAT_LM_HEAD = 3   /* same row order as PLAIN                                   */
} nq_mat_kind;

/* Bytes of the packed form of an N x K matrix: ceil(N/16)*16 * K/2 (codes) +
 * ceil(N/16)*16 * K/group * 2 (fp16 scales). Returns 0 if the arguments are
 * invalid (K % group != 0, group != 128, N <= 0). */
size_t nq_packed_size(int32_t N, int32_t K, int32_t group);

/*
 * Quantise and repack a float32 weight matrix (host only; no GPU needed).
 *
 * Quantisation (symmetric, group-wise along K, group = 128; the pages give the
 * group size and the symmetric format, section "What it actually builds"):
 *   a   = max |w[n, 128g .. 128g+127]|                       (float32)
 *   s16 = fp16_round_half_even(float32(a / 7.0f))
 *   q   = clamp(round_half_even(double(w) / double(s16)), -8, 7), 0 if s16 == 0
 * so |w - q*s16| <= s16/2 and the codes used lie in [-7, 7].
 *
 * Packed layout, version 1 ("t16g128"): with Np = ceil(N/16)*16, T = Np/16
 * tiles and G = K/128 groups,
 *   codes  : T*G blocks of 1024 bytes, block (t, g) at byte (t*G + g)*1024.
 *            The 16-byte chunk c (0..63) of a block, at byte 16c, holds tile
 *            row r = c % 16 and K range k0 = 128g + 32*(c/16) .. k0+31, as four
 *            little-endian 32-bit words; word j holds k0+8j .. k0+8j+7 with
 *            nibble slot m (bits 4m..4m+3) holding k0 + 8j + (m < 4 ? 2m : 2(m-4)+1),
 *            stored offset-binary as q + 8.
 *   scales : at byte T*G*1024: fp16 s16 of (tile t, group g, tile row r) at
 *            element (t*G + g)*16 + r.
 *   Tile row r of tile t is the logical row given by nq_mat_kind. Rows beyond
 *   N (PLAIN / LM_HEAD only) are zero codes (q = 0) with scale 0.
 *
 * w         : host float32 [N][K], row-major (torch Linear [out, in] layout).
 * kind      : row co-location (see nq_mat_kind). QKV needs head_dim % 16 == 0
 *             and N % head_dim == 0; GATE_UP needs N % 16 == 0.
 * head_dim  : used by NQ_MAT_QKV only (else ignored).
 * packed_out: host buffer of nq_packed_size(N, K, group) bytes.
 * q_out     : optional host int8 [N][K], codes in LOGICAL row order.
 * s_out     : optional host uint16 [N][K/group], fp16 scale bits, logical order.
 * Errors: NQ_ERR_INVALID_ARG (null w / packed_out, K % 128, group != 128, bad
 * kind or shape for kind); NQ_ERR_OUT_OF_RANGE (non-finite weight, or a scale
 * that overflows fp16). Runs on several host threads.
 */
nq_status nq_pack_weights(const float* w, int32_t N, int32_t K, int32_t group,
                          nq_mat_kind kind, int32_t head_dim, void* packed_out,
                          int8_t* q_out, uint16_t* s_out);

/* Inverse of the repacking (host): codes and scale bits in logical row order.
 * Same argument rules as nq_pack_weights; q_out [N][K], s_out [N][K/group]. */
nq_status nq_unpack_weights(const void* packed, int32_t N, int32_t K, int32_t group,
                            nq_mat_kind kind, int32_t head_dim, int8_t* q_out,
                            uint16_t* s_out);

/* Device twin of nq_unpack_weights: decodes every nibble with the same
 * in-register unpack the GEMV kernels use (fp16 exponent-bias trick) and writes
 * int8 codes [N][K] and fp16 scale bits [N][K/group] (device pointers) in
 * logical row order. For bit-exactness tests. */
nq_status nq_unpack_weights_dev(const void* packed_dev, int32_t N, int32_t K,
                                int32_t group, nq_mat_kind kind, int32_t head_dim,
                                int8_t* q_out_dev, uint16_t* s_out_dev, void* stream);

/* ----------------------------------------------------------------- GEMV */

typedef enum nq_epilogue {
  NQ_EPI_STORE_F16 = 0,    /* y[b][n] = fp16(W x_b)                                   */
  NQ_EPI_BIAS_F16 = 1,     /* y[b][n] = fp16(W x_b + bias[n])                          */
  NQ_EPI_RESIDUAL_F16 = 2, /* y[b][n] = fp16(y[b][n] + W x_b)   (y read, then written) */
  NQ_EPI_SWIGLU_F16 = 3,   /* kind GATE_UP, I = N/2: y[b][j] = fp16(silu(g_j) * u_j),
                              g_j = (W x_b)[j], u_j = (W x_b)[I + j]; y is [B][I]     */
  NQ_EPI_STORE_F32 = 4     /* y[b][n] = float32(W x_b)                                 */
} nq_epilogue;

/*
 * Batched W4A16 GEMV: y_b = W x_b for b < batch (the fused Q/K/V/O and
 * gate/up/down projections of "What it actually builds"), fp32 accumulation.
 *
 * packed   : device, output of nq_pack_weights for (N, K, kind, head_dim).
 * batch    : 1 .. 8.
 * x        : device fp16 [batch][K].
 * norm_gain: optional device fp16 [K]. If non-NULL the input is first
 *            RMS-normalised: x_b <- fp16(x_b / sqrt(mean(x_b^2) + eps) * gain).
 * bias     : device fp16 [N] (logical order), NQ_EPI_BIAS_F16 only.
 * y        : device output, fp16 or fp32 per the epilogue, [batch][N] (or [batch][N/2]
 *            for SwiGLU). Must not overlap x (except RESIDUAL, which reads y).
 * Errors: NQ_ERR_INVALID_ARG for null/misaligned pointers, K % 128, batch out
 * of 1..8, or an epilogue that does not fit the kind. NQ_ERR_HIP on launch.
 */
nq_status nq_gemv_w4a16(const void* packed, int32_t N, int32_t K, nq_mat_kind kind,
                        int32_t head_dim, int32_t batch, const void* x,
                        const void* norm_gain, float eps, const void* bias, void* y,
                        nq_epilogue epi, void* stream);

/*
 * W4A16 GEMM for a chunk of M activation rows: y_m = W x_m for m < M, the same
 * packed weights, arithmetic and epilogues as nq_gemv_w4a16 (fp32
 * accumulation of exact INT4 codes times fp16 activations, the fp16 group
 * scale applied to each group's fp32 partial sum) on the matrix cores with
 * the rows as the MFMA columns. It is the projection step of the chunked
 * prefill (nq_prefill): the prompt's tokens go through the fused Q/K/V/O and
 * gate/up/down projections of "What it actually builds" a chunk at a time.
 *
 * M        : 1 .. 4096 rows.
 * x        : device fp16 [M][K] (no RMSNorm prologue: normalise beforehand).
 * bias, y, epi: as nq_gemv_w4a16 with batch = M.
 * Errors: NQ_ERR_INVALID_ARG for null/misaligned pointers, K % 128, M out of
 * 1..4096, or an epilogue that does not fit the kind; NQ_ERR_HIP on launch.
 */
nq_status nq_gemm_w4a16(const void* packed, int32_t N, int32_t K, nq_mat_kind kind,
                        int32_t head_dim, int32_t M, const void* x, const void* bias,
                        void* y, nq_epilogue epi, void* stream);

/* ------------------------------------------------------------- W4A8 variant */

/*
 * INT8-activation variant of the projections ("How To Build Your Own LLM
 * Runtime From Scratch" (daily.dev), Summary and the FAQ question on
 * INT8-activation dp4a against FP16-activation INT4 unpack: the activations
 * are quantised to INT8 before the GEMV and multiplied with the INT4 weights in
 * integer arithmetic). The pages give no quantisation rule; this library uses
 * one scale per row and group of 128 inputs:
 *   s = fp32(max |x| over the group) / 127,
 *   q = clamp(round_half_even(fp32(x) / s), -127, 127)   (q = 0 when s = 0),
 * the group's integer sum of q_w * q multiplied by the fp16 weight scale and s
 * in fp32. Batch 1..4.
 *
 * Quantised activations of `batch` rows of K inputs take nq_a8_bytes(batch, K)
 * device bytes: batch*K int8 codes (each 8 inputs k0..k0+7 stored in the order
 * k0, k0+4, k0+1, k0+5, k0+2, k0+6, k0+3, k0+7), then per (row, group) a float
 * scale and the int32 sum of the group's codes, padded to 16 bytes.
 */
size_t nq_a8_bytes(int32_t batch, int32_t K);

/* Quantise fp16 x [batch][K] (device) into xq (device, nq_a8_bytes bytes,
 * 16-byte aligned). Errors: NQ_ERR_INVALID_ARG (null/misaligned pointers,
 * K % 128, batch outside 1..4). */
nq_status nq_quantize_a8(const void* x, int32_t batch, int32_t K, void* xq, void* stream);

/* y = W x with INT8 activations. xq non-NULL: the activations quantised by
 * nq_quantize_a8 (x is ignored); xq NULL: the kernel quantises fp16 x itself
 * in its prologue, which needs all of K of the batch in LDS
 * (NQ_ERR_UNSUPPORTED otherwise; quantise first then). The same arithmetic
 * either way, bit for bit. packed, kind, head_dim, bias, y and epi as
 * nq_gemv_w4a16 (no RMSNorm prologue; epilogues STORE_F16, BIAS_F16,
 * RESIDUAL_F16, SWIGLU_F16, STORE_F32). */
nq_status nq_gemv_w4a8(const void* packed, int32_t N, int32_t K, nq_mat_kind kind,
                       int32_t head_dim, int32_t batch, const void* x, const void* xq,
                       const void* bias, void* y, nq_epilogue epi, void* stream);

/* ------------------------------------------------------------ model config */

typedef struct nq_config {
  int32_t layers;        /* decoder layers (28 for the 7B shape)                        */
  int32_t hidden;        /* H, multiple of 128                                          */
  int32_t intermediate;  /* I, multiple of 128                                          */
  int32_t n_heads;       /* query heads                                                 */
  int32_t n_kv_heads;    /* KV heads; n_heads % n_kv_heads == 0, ratio <= 8             */
  int32_t head_dim;      /* d: 64 or 128                                                */
  int32_t vocab;         /* V                                                           */
  float rms_eps;         /* RMSNorm epsilon (1e-6)                                      */
  float rope_theta;      /* RoPE base (1e6)                                             */
  int32_t group;         /* quantisation group, must be 128                             */
  int32_t page_tokens;   /* tokens per KV page, must be 16                              */
  int32_t max_batch;     /* largest batch a step will be called with (1 .. 8)           */
  int32_t max_pos;       /* positions covered by the RoPE table (max context length)    */
} nq_config;

/* Checks a configuration; NQ_OK or NQ_ERR_INVALID_ARG / NQ_ERR_UNSUPPORTED. */
nq_status nq_config_check(const nq_config* cfg);

/* -------------------------------------------------- packed-weight container */

/*
 * One file holding a model's configuration and its tensors, with the
 * projections already in the packed tile layout, written once offline and
 * memory-mapped at load so that loading does no repacking ("How to build your
 * own LLM runtime from scratch", "What it actually builds": the INT4 weights
 * live in a memory-mapped binary file with a magic-byte header).
 *
 * Format version 1 (little-endian): a 4096-byte header (magic "NQPACKW4",
 * format version, the packed tile layout version of nq_layout_version, the
 * model configuration without max_batch / max_pos, the tensor count and the
 * position of the tensor table, an FNV-1a 64 checksum of the header); the
 * tensors, each at a 4096-byte aligned offset; the tensor table (per tensor:
 * a NUL-terminated name of at most 47 bytes, role, matrix kind, shape, offset,
 * size and the FNV-1a 64 checksum of its bytes). Opening checks the magic,
 * versions, header checksum and that every record is consistent and inside the
 * file; nq_container_verify also checks the tensor checksums.
 */
typedef enum nq_tensor_role {
  NQ_TENSOR_PACKED = 1,  /* nq_pack_weights output of an N x K matrix of kind mat_kind */
  NQ_TENSOR_F16 = 2      /* fp16 [N][K] (a vector has K = 1)                          */
} nq_tensor_role;

typedef struct nq_tensor_desc {
  char name[48];
  int32_t role;       /* nq_tensor_role                                */
  int32_t mat_kind;   /* NQ_TENSOR_PACKED: nq_mat_kind                 */
  int32_t N, K;
  int32_t head_dim;   /* NQ_TENSOR_PACKED of kind QKV                  */
  uint64_t bytes;     /* nq_packed_size(N, K, 128) or N * K * 2        */
} nq_tensor_desc;

typedef struct nq_container_writer nq_container_writer;
typedef struct nq_container nq_container;

/* Streaming writer: create, add exactly n_tensors tensors (host memory), finish.
 * Errors: NQ_ERR_INVALID_ARG (bad config, name, duplicate, size that does not
 * match role and shape), NQ_ERR_IO (file errors), NQ_ERR_STATE (count).
 * nq_container_finish frees the writer whatever it returns. */
nq_status nq_container_create(const char* path, const nq_config* cfg, int32_t n_tensors,
                              nq_container_writer** out);
nq_status nq_container_add(nq_container_writer* w, const nq_tensor_desc* desc, const void* data);
nq_status nq_container_finish(nq_container_writer* w);

/* Maps a container read-only. Errors: NQ_ERR_IO (missing, truncated or invalid
 * file, other layout version). */
nq_status nq_container_open(const char* path, nq_container** out);
/* The stored configuration (max_batch and max_pos set to 1: runtime choices). */
nq_status nq_container_config(const nq_container* c, nq_config* out);
int32_t nq_container_count(const nq_container* c);
/* Description and host pointer (into the mapping, valid until close) of a
 * tensor by name or by index. NQ_ERR_OUT_OF_RANGE if there is none. */
nq_status nq_container_tensor(const nq_container* c, const char* name, nq_tensor_desc* desc,
                              const void** data);
nq_status nq_container_tensor_at(const nq_container* c, int32_t index, nq_tensor_desc* desc,
                                 const void** data);
/* Recomputes every tensor checksum (reads the whole file). NQ_ERR_IO on a mismatch. */
nq_status nq_container_verify(const nq_container* c);
void nq_container_close(nq_container* c);

/* ---------------------------------------------------------------- KV cache */

/*
 * Paged KV cache ("What it actually builds": 16 tokens per 4 KiB page, pages
 * reached through a page table). The pool is caller-owned device memory:
 *   pool[layer][0 = K][page][kv_head][slot 0..15][head_dim]  fp16 (token-major)
 *   pool[layer][1 = V][page][kv_head][head_dim][slot 0..15]  fp16 (dim-major)
 * so one (layer, K or V, page, kv_head) block is 16 * head_dim fp16 (4096 bytes
 * at head_dim 128). Token p of sequence b is in page page_table[b][p / 16],
 * slot p % 16. Page ids are chosen by the caller (any permutation of the pool;
 * -1 marks an unused table entry). K is stored after RoPE. V is dim-major so
 * that the attention's P.V product reads it in matrix-core operand order.
 */
typedef struct nq_kv nq_kv;

size_t nq_kv_pool_bytes(const nq_config* cfg, int32_t num_pages);

/* Builds a descriptor over a caller-owned pool of num_pages pages (bytes must be
 * at least nq_kv_pool_bytes). No device work. */
nq_status nq_kv_alloc(const nq_config* cfg, void* pool_dev, size_t bytes,
                      int32_t num_pages, nq_kv** out);

/*
 * Writes one token's K and V per sequence into the pool:
 *   pool[layer][0][pt[b][pos[b]/16]][h][pos[b]%16][:] = k[b][h][:]
 *   pool[layer][1][pt[b][pos[b]/16]][h][:][pos[b]%16] = v[b][h][:]
 * page_table: device int32 [batch][max_pages]; pos: device int32 [batch];
 * k, v: device fp16 [batch][n_kv_heads][head_dim].
 * err_flag: optional device int32; a position beyond max_pages*16, or a page id
 * outside [0, num_pages), skips that write and ORs 1 into *err_flag
 * (see nq_check_device_error).
 */
nq_status nq_kv_append(nq_kv* kv, int32_t layer, int32_t batch, const int32_t* page_table,
                       int32_t max_pages, const int32_t* pos, const void* k, const void* v,
                       int32_t* err_flag, void* stream);

void nq_kv_free(nq_kv* kv);

/* ----------------------------------------------------- decode attention */

/* Scratch bytes nq_attn_decode needs for its split-K partials; 0 for an invalid
 * configuration or a batch and table width beyond the kernels (see below). */
size_t nq_attn_workspace_bytes(const nq_config* cfg, int32_t batch, int32_t max_pages);

/*
 * Split-K paged decode attention for one layer (GQA): for query head h of
 * sequence b, with kv = h / (n_heads / n_kv_heads),
 *   o[b][h] = sum_t softmax_t(q[b][h] . k_t / sqrt(d)) v_t   over t < lens[b]
 * (scaled dot-product attention with a stable softmax; "Build Crude
 * Implementations for Learning", "nanoGPT level", and the "Inference Zero To
 * Hero" preface). Partial tail pages are handled: slots at or beyond lens[b]
 * are never used, whatever they hold.
 * q: device fp16 [batch][n_heads][head_dim]; out: device fp16, same shape.
 * lens: device int32 [batch] (0 gives a zero output row).
 * max_pages: page_table row stride, 1..32768 (NQ_ERR_OUT_OF_RANGE beyond).
 * batch: 1..64 when the pages are split by length (batch > 1 and max_pages > 4);
 * with batch * max_pages beyond what 1024 workgroups per KV head of at most 512
 * pages cover, the call fails with NQ_ERR_OUT_OF_RANGE (and the workspace
 * size is 0). The pages of a sequence are spread over the splits by the
 * current lengths, so results agree with a batch-1 call within rounding, not
 * bitwise.
 * workspace: device, nq_attn_workspace_bytes(cfg, batch, max_pages) bytes for
 * the split partials; calls that share a workspace must not overlap.
 * err_flag: optional device int32 (bad page id or length -> ORs 2, output 0).
 */
nq_status nq_attn_decode(const nq_kv* kv, int32_t layer, int32_t batch, const void* q,
                         const int32_t* page_table, int32_t max_pages, const int32_t* lens,
                         void* out, void* workspace, size_t ws_bytes, int32_t* err_flag,
                         void* stream);

/*
 * The same split-K paged decode attention with no workspace argument and no
 * allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors are those of nq_attn_decode. The split
 * partials live in a library-owned device array of NQ_ATTN_SCRATCH_BYTES
 * (24 MiB) on each GPU, held until the process ends; its address is looked up
 * on the first call on a device. A call whose nq_attn_workspace_bytes(cfg,
 * batch, max_pages) exceeds NQ_ATTN_SCRATCH_BYTES fails with
 * NQ_ERR_OUT_OF_RANGE before anything is enqueued (batch 1 covers any table
 * width; at the 7B shape, 28 heads of 128, batch 8 covers up to 192 splits).
 * Every call on one GPU shares that array and leaves its partials there: calls
 * that may overlap on one GPU (other streams, other threads) race, and the
 * caller must order them. Nothing in the array needs to start at zero (every
 * split writes its partial row before the merge reads it).
 */
#define NQ_ATTN_SCRATCH_BYTES (24u << 20)
nq_status nq_attn_decode_static(const nq_kv* kv, int32_t layer, int32_t batch, const void* q,
                                const int32_t* page_table, int32_t max_pages, const int32_t* lens,
                                void* out, int32_t* err_flag, void* stream);

/*
 * Causal paged attention of n_q consecutive queries of one sequence (the
 * attention step of the chunked prefill): query row i sits at position
 * start_pos + i and, for query head h with kv = h / (n_heads / n_kv_heads),
 *   out[i][h] = sum_{t <= start_pos + i} softmax_t(q[i][h] . k_t / sqrt(d)) v_t
 * (scaled dot-product attention with the causal mask, "Build Crude
 * Implementations for Learning", section "nanoGPT level"). K and V of every
 * position up to start_pos + n_q - 1 must already be in the pool; slots after
 * that in the last page are never used, whatever they hold.
 * q, out: device fp16 [n_q][n_heads][head_dim]; page_table: device int32
 * [max_pages], this sequence's row. n_q: 1 .. 4096; start_pos >= 0 and
 * start_pos + n_q <= max_pages * 16 (else NQ_ERR_OUT_OF_RANGE).
 * err_flag: optional device int32 (a page id outside the pool ORs 2).
 */
nq_status nq_attn_prefill(const nq_kv* kv, int32_t layer, int32_t n_q, int32_t start_pos,
                          const void* q, const int32_t* page_table, int32_t max_pages,
                          void* out, int32_t* err_flag, void* stream);

/* -------------------------------------------------------------- the model */

typedef struct nq_model nq_model;

/* Per-layer device pointers (all caller-owned). */
typedef struct nq_layer_ptrs {
  const void* qkv_packed;      /* nq_pack_weights(kind QKV) of [Wq; Wk; Wv], N = (nh+2nkv)d, K = H */
  const void* qkv_bias;        /* fp16 [(nh + 2 nkv) d], logical order                             */
  const void* o_packed;        /* PLAIN, N = H, K = nh d                                           */
  const void* gate_up_packed;  /* GATE_UP of [Wg; Wu], N = 2I, K = H                               */
  const void* down_packed;     /* PLAIN, N = H, K = I                                              */
  const void* attn_norm;       /* fp16 [H] RMSNorm gain before attention                           */
  const void* mlp_norm;        /* fp16 [H] RMSNorm gain before the MLP                             */
} nq_layer_ptrs;

nq_status nq_model_create(const nq_config* cfg, nq_model** out);
nq_status nq_model_bind_layer(nq_model* m, int32_t layer, const nq_layer_ptrs* p);
/* embed: fp16 [V][H]; final_norm: fp16 [H]; lm_packed: kind LM_HEAD, N = V, K = H. */
nq_status nq_model_bind_head(nq_model* m, const void* embed, const void* final_norm,
                             const void* lm_packed);

/* RoPE table: float32 [max_pos][head_dim/2][2] = (cos, sin) of
 * pos * theta^(-2i/d), computed on the host in double precision. */
size_t nq_rope_table_bytes(const nq_config* cfg);
nq_status nq_rope_table_fill(const nq_config* cfg, float* host_out);
nq_status nq_model_bind_rope(nq_model* m, const void* rope_table_dev);

/* Scratch the decode step needs at a given batch and page-table width. The
 * workspace must be zero-filled by the caller once, before its first use; the
 * library leaves its counters at zero between steps. */
size_t nq_workspace_bytes(const nq_config* cfg, int32_t batch, int32_t max_pages);
nq_status nq_model_bind_workspace(nq_model* m, void* ws_dev, size_t bytes);

void nq_model_destroy(nq_model* m);

/* ------------------------------------------------------------ decode step */

typedef struct nq_step_io {
  int32_t batch;            /* 1 .. cfg.max_batch                                          */
  int32_t max_pages;        /* page_table row stride (pages per sequence), 1..32768        */
  const int32_t* page_table;/* device int32 [batch][max_pages]                             */
  int32_t* tokens;          /* device int32 [batch]: in = token at pos, out = greedy next  */
  int32_t* pos;             /* device int32 [batch]: in = position of the input token;
                               the step appends K/V there and adds 1                       */
  float* logits;            /* optional device float32 [batch][vocab]                      */
  void* layer_out;          /* optional device fp16 [layers][batch][H]: hidden state after
                               each layer (debug; may be captured)                         */
  int32_t* token_hist;      /* optional device int32 [batch][hist_len]: the step writes
                               token_hist[b][pos+1] = next token (if pos+1 < hist_len)     */
  int32_t hist_len;
  int32_t* err_flag;        /* optional device int32: device-side range errors OR bits in
                               (1 = KV write, 2 = attention read, 4 = token id, 8 = NaN
                               logits, 16 = the persistent step's workgroups could not
                               all run at once); NULL uses a flag inside the workspace     */
} nq_step_io;

/*
 * One greedy decode step for a batch (everything on the device, enqueued on
 * stream): embedding gather; per layer RMSNorm -> fused QKV GEMV + bias ->
 * RoPE -> K/V page append at pos -> split-K paged attention over [0, pos] ->
 * O GEMV + residual -> RMSNorm -> gate/up GEMV + SwiGLU -> down GEMV +
 * residual; final RMSNorm -> LM-head GEMV -> argmax (lowest index on ties)
 * -> tokens, pos += 1. That is 6 kernels per layer (attention is a split
 * kernel and a combine kernel; 5 when max_pages is small enough that one
 * workgroup covers a sequence's pages) plus 2 (LM head, argmax); the gather
 * runs in layer 0's QKV kernel.
 * Errors: NQ_ERR_STATE if the model is not fully bound; NQ_ERR_INVALID_ARG for
 * bad io; NQ_ERR_HIP on launch failure.
 */
nq_status nq_decode_step(nq_model* m, nq_kv* kv, const nq_step_io* io, void* stream);

/*
 * How a step is launched. NQ_STEP_AUTO (the default): at batch 1 the whole
 * step is one persistent kernel when the device and model allow it (an
 * MI355X's 256 CUs, head_dim 128 with 7 query heads per KV head or head_dim
 * 64 with 4, at most 32 layers, at most 14 KV heads, max_pages <= 256 *
 * min(64, 256 / n_kv_heads) (16384 for 4 KV heads), n_heads * head_dim ==
 * hidden); other batches, and batch 1 otherwise, take the kernels listed
 * above. NQ_STEP_KERNELS: always those kernels. Both compute the same
 * operation (the persistent kernel splits the reductions differently, so the
 * two agree within rounding, not bitwise).
 *
 * The persistent kernel runs 256 co-resident workgroups, one per CU, that
 * hand each stage's output to the next through flags in the workspace; the
 * workspace must be zeroed before its first step (a fresh hipMemset is
 * enough) and must not be shared by steps that may run at the same time.
 * Every wait inside it is bounded: if the workgroups cannot all be resident
 * (another kernel occupying CUs), the step ends with err_flag bit 16 and
 * garbage results, and the workspace must be zeroed again before the next
 * step.
 */
enum { NQ_STEP_AUTO = 0, NQ_STEP_KERNELS = 1 };
nq_status nq_model_set_step_mode(nq_model* m, int32_t mode);

/* Kernels one step of this model launches at this batch and table width (1
 * for the persistent kernel), or -1 for invalid arguments. Host only. */
int32_t nq_step_kernels(const nq_model* m, int32_t batch, int32_t max_pages);

/*
 * Measurement hook of the persistent step: when device_buf is set, every
 * persistent step enqueued (or captured) afterwards writes, per workgroup w of
 * 256 and row r of layers + 1, 16 uint64 stamps of the GPU's constant 100 MHz
 * realtime counter at buf[(w * (layers + 1) + r) * 16 + e]. Row l < layers,
 * events 0-15: the QKV partials are in, before and after the QKV hand-off, the
 * attention partials are in, before and after the attention hand-off, the O
 * partials are in, before and after the O hand-off, the gate/up partials, before
 * and after its hand-off, the down partials, before and after its hand-off, the
 * next stage's input staged. Row layers, events 0-2: the workgroup's start, the
 * LM head's partials are in, its last work done. Other entries are not
 * written. bytes must be at least 256 * (layers + 1) * 16 * 8, device_buf 8-byte
 * aligned device memory the caller owns; NULL turns the stamps off (the
 * default). Steps of one kernel per stage write nothing. The stamps change
 * no result.
 */
nq_status nq_model_set_step_trace(nq_model* m, uint64_t* device_buf, int64_t bytes);

/* ---------------------------------------------------------- chunked prefill */

/*
 * Chunked prefill of one sequence's prompt (everything on the device): the
 * tokens go through the model a chunk at a time instead of one decode step
 * per token, which is what the time to first token depends on ("How To Build
 * Your Own LLM Runtime From Scratch" (daily.dev), Summary; the runtime the
 * pages describe is decode-only and its prefill is not described). For each
 * chunk of up to `chunk` tokens, per layer: RMSNorm of the chunk's rows ->
 * fused QKV GEMM + bias -> RoPE -> K/V page writes at their positions ->
 * causal paged attention over positions [0, own position] -> O GEMM +
 * residual -> RMSNorm -> gate/up GEMM + SwiGLU -> down GEMM + residual
 * (7 kernels per layer). After the last chunk: final RMSNorm -> LM head of the
 * last token -> greedy argmax (lowest index on ties), 2 kernels. The result
 * equals feeding the tokens one by one through nq_decode_step up to rounding
 * order, and the KV pages it writes are what decode steps then read.
 */
typedef struct nq_prefill_io {
  int32_t n_tokens;          /* prompt tokens of this call, >= 1                                */
  int32_t start_pos;         /* position of the first of them (K/V of earlier positions must
                                already be in the pool), >= 0                                  */
  const int32_t* tokens;     /* device int32 [n_tokens]                                        */
  const int32_t* page_table; /* device int32 [max_pages]: this sequence's row                  */
  int32_t max_pages;         /* start_pos + n_tokens <= max_pages * 16                         */
  int32_t chunk;             /* tokens per chunk, 1 .. 4096                                    */
  int32_t* next_token;       /* optional device int32: greedy token after the last prompt token */
  int32_t* pos_out;          /* optional device int32: set to start_pos + n_tokens (the position
                                of next_token in a following decode step)                     */
  float* logits;             /* optional device float32 [vocab] at the last prompt token       */
  void* layer_out;           /* optional device fp16 [layers][n_tokens][H]: hidden state after
                                each layer (debug)                                             */
  int32_t* err_flag;         /* optional device int32 (bits as nq_step_io); NULL uses a flag in
                                the workspace                                                   */
  void* workspace;           /* device, nq_prefill_workspace_bytes(cfg, chunk) bytes            */
  size_t ws_bytes;
} nq_prefill_io;

/* Scratch bytes nq_prefill needs at a chunk size (0 for invalid arguments). */
size_t nq_prefill_workspace_bytes(const nq_config* cfg, int32_t chunk);

/* Errors: NQ_ERR_STATE if the model is not fully bound (its decode workspace
 * is not needed); NQ_ERR_INVALID_ARG / NQ_ERR_OUT_OF_RANGE for bad io
 * (positions past max_pages * 16 or cfg.max_pos); NQ_ERR_HIP on launch. */
nq_status nq_prefill(nq_model* m, nq_kv* kv, const nq_prefill_io* io, void* stream);

/* ---------------------------------------------------------- graph capture */

/*
 * Captures one decode step (the same kernels as nq_decode_step) into a HIP
 * graph, so that a token costs one launch ("What it actually builds": graph
 * capture of the token-generation loop; "The one lesson that generalizes").
 * Every per-step value lives in device memory (tokens, pos, page table), so
 * replays chain with no host updates. batch and max_pages are fixed per graph.
 * Errors: NQ_ERR_STATE for the null stream or a stream already capturing.
 */
typedef struct nq_graph nq_graph;

nq_status nq_graph_capture(nq_model* m, nq_kv* kv, const nq_step_io* io, void* stream,
                           nq_graph** out);
nq_status nq_graph_launch(nq_graph* g, void* stream);
/* Number of kernel nodes in the captured step. */
int32_t nq_graph_kernel_count(const nq_graph* g);
void nq_graph_destroy(nq_graph* g);

/* ---------------------------------------------------------------- errors */

/* Synchronises stream, reads *err_flag_dev, and returns NQ_ERR_DEVICE_FAULT (with
 * the flag bits in the message) if it is non-zero; the flag is then reset to 0. */
nq_status nq_check_device_error(int32_t* err_flag_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NQ_H */
