// Host-side part of libnq: status strings, error text, the offline INT4
// quantiser + tile repacker and its inverse, and the RoPE table.
//
// The quantiser follows the group-wise symmetric INT4 format named in
// "How to build your own LLM runtime from scratch", section "What it actually
// builds" (group size 128): per (row, 128-wide K group) an fp16 scale
// s = fp16(max|w| / 7) and codes q = round_half_even(w / s) in [-7, 7].
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "common.hpp"

namespace nq {

static thread_local std::string g_last_error;

nq_status fail(nq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

nq_status hip_fail(hipError_t e, const char* what) {
  return fail(NQ_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

void clear_error() { g_last_error.clear(); }

// IEEE binary32 -> binary16, round to nearest, ties to even.
static uint16_t f32_to_f16_bits(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return static_cast<uint16_t>(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
  if (ax >= 0x477ff000u) return static_cast<uint16_t>(sign | 0x7c00u);  // >= 65520 rounds to inf
  if (ax < 0x38800000u) {
    // below the smallest normal half (2^-14): result is m * 2^-24, m = rne(|f| * 2^24)
    float a;
    std::memcpy(&a, &ax, 4);
    const float m = std::nearbyint(a * 16777216.0f);  // exact scaling; default mode is RNE
    return static_cast<uint16_t>(sign | static_cast<uint32_t>(m));
  }
  // normal: rebias the exponent (127 -> 15) and round 23 -> 10 mantissa bits
  const uint32_t r = ax - (112u << 23) + 0x0fffu + ((ax >> 13) & 1u);
  return static_cast<uint16_t>(sign | (r >> 13));
}

static float f16_bits_to_f32(uint16_t h) {
  const uint32_t sign = static_cast<uint32_t>(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  float v;
  if (e == 0) {
    v = std::ldexp(static_cast<float>(m), -24);
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = std::ldexp(static_cast<float>(m | 0x400u), static_cast<int>(e) - 25);
  }
  uint32_t b;
  std::memcpy(&b, &v, 4);
  b |= sign;
  std::memcpy(&v, &b, 4);
  return v;
}

nq_status check_pack_args(int32_t N, int32_t K, int32_t group, nq_mat_kind kind, int32_t head_dim) {
  if (group != kGroup) return fail(NQ_ERR_INVALID_ARG, "group must be 128 (got %d)", group);
  if (N <= 0 || K <= 0) return fail(NQ_ERR_INVALID_ARG, "N and K must be positive (N=%d K=%d)", N, K);
  if (K % kGroup != 0) return fail(NQ_ERR_INVALID_ARG, "K=%d is not a multiple of 128", K);
  switch (kind) {
    case NQ_MAT_PLAIN:
    case NQ_MAT_LM_HEAD:
      break;
    case NQ_MAT_QKV:
      if (head_dim <= 0 || head_dim % 16 != 0 || N % head_dim != 0)
        return fail(NQ_ERR_INVALID_ARG, "QKV needs head_dim %% 16 == 0 and N %% head_dim == 0 (N=%d d=%d)",
                    N, head_dim);
      break;
    case NQ_MAT_GATE_UP:
      if (N % 16 != 0) return fail(NQ_ERR_INVALID_ARG, "GATE_UP needs N %% 16 == 0 (N=%d)", N);
      break;
    default:
      return fail(NQ_ERR_INVALID_ARG, "unknown matrix kind %d", static_cast<int>(kind));
  }
  return NQ_OK;
}

// Nibble slot m of word j of a 32-k chunk holds k offset 8j + kslot(m).
static inline int kslot(int m) { return m < 4 ? 2 * m : 2 * (m - 4) + 1; }

template <class F>
static void parallel_for(int64_t n, F&& fn) {
  unsigned hw = std::thread::hardware_concurrency();
  int64_t nt = std::max<int64_t>(1, std::min<int64_t>({static_cast<int64_t>(hw ? hw : 1), 32, n}));
  if (nt == 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> th;
  const int64_t per = (n + nt - 1) / nt;
  for (int64_t i = 0; i < nt; ++i) {
    const int64_t a = i * per, b = std::min(n, a + per);
    if (a >= b) break;
    th.emplace_back([&fn, a, b] { fn(a, b); });
  }
  for (auto& t : th) t.join();
}

}  // namespace nq

using namespace nq;

extern "C" {

const char* nq_status_str(nq_status s) {
  switch (s) {
    case NQ_OK: return "NQ_OK";
    case NQ_ERR_INVALID_ARG: return "NQ_ERR_INVALID_ARG";
    case NQ_ERR_UNSUPPORTED: return "NQ_ERR_UNSUPPORTED";
    case NQ_ERR_OUT_OF_RANGE: return "NQ_ERR_OUT_OF_RANGE";
    case NQ_ERR_HIP: return "NQ_ERR_HIP";
    case NQ_ERR_STATE: return "NQ_ERR_STATE";
    case NQ_ERR_DEVICE_FAULT: return "NQ_ERR_DEVICE_FAULT";
    case NQ_ERR_IO: return "NQ_ERR_IO";
  }
  return "NQ_ERR_UNKNOWN";
}

const char* nq_last_error(void) { return g_last_error.c_str(); }

int32_t nq_layout_version(void) { return 1; }

size_t nq_packed_size(int32_t N, int32_t K, int32_t group) {
  if (group != kGroup || N <= 0 || K <= 0 || K % kGroup != 0) return 0;
  const size_t rows = static_cast<size_t>(padded_rows(N));
  return rows * (K / 2) + rows * (K / kGroup) * 2;
}

nq_status nq_pack_weights(const float* w, int32_t N, int32_t K, int32_t group, nq_mat_kind kind,
                          int32_t head_dim, void* packed_out, int8_t* q_out, uint16_t* s_out) {
  if (!w || !packed_out) return fail(NQ_ERR_INVALID_ARG, "nq_pack_weights: null w or packed_out");
  nq_status st = check_pack_args(N, K, group, kind, head_dim);
  if (st != NQ_OK) return st;
  const int64_t T = tiles_of(N), G = K / kGroup;
  uint8_t* codes = static_cast<uint8_t*>(packed_out);
  uint16_t* scales = reinterpret_cast<uint16_t*>(codes + codes_bytes(N, K));
  std::atomic<int> bad{0};  // 1 = non-finite weight, 2 = scale overflow

  parallel_for(T, [&](int64_t t0, int64_t t1) {
    uint8_t qrow[kGroup];
    for (int64_t t = t0; t < t1; ++t) {
      for (int r = 0; r < kTileRows; ++r) {
        const int64_t n = tile_row_logical(kind, N, head_dim, t, r);
        for (int64_t g = 0; g < G; ++g) {
          uint16_t sbits = 0;
          if (n < N) {
            const float* src = w + n * static_cast<int64_t>(K) + g * kGroup;
            float a = 0.0f;
            bool finite = true;
            for (int i = 0; i < kGroup; ++i) {
              finite = finite && std::isfinite(src[i]);
              a = std::max(a, std::fabs(src[i]));
            }
            if (!finite) { bad.store(1); continue; }
            sbits = f32_to_f16_bits(a / 7.0f);
            if ((sbits & 0x7fffu) >= 0x7c00u) { bad.store(2); continue; }
            const double sd = static_cast<double>(f16_bits_to_f32(sbits));
            for (int i = 0; i < kGroup; ++i) {
              int q = 0;
              if (sd != 0.0) {
                double v = std::nearbyint(static_cast<double>(src[i]) / sd);
                q = static_cast<int>(std::min(7.0, std::max(-8.0, v)));
              }
              qrow[i] = static_cast<uint8_t>(q);
              if (q_out) q_out[n * static_cast<int64_t>(K) + g * kGroup + i] = static_cast<int8_t>(q);
            }
            if (s_out) s_out[n * G + g] = sbits;
          } else {
            std::memset(qrow, 0, sizeof qrow);
          }
          scales[(t * G + g) * kTileRows + r] = sbits;
          // chunk c = 16*kq + r of block (t, g)
          uint8_t* blk = codes + (t * G + g) * kBlockBytes;
          for (int kq = 0; kq < 4; ++kq) {
            uint32_t* chunk = reinterpret_cast<uint32_t*>(blk + 16 * (16 * kq + r));
            for (int j = 0; j < 4; ++j) {
              uint32_t word = 0;
              for (int m = 0; m < 8; ++m) {
                const int k = 32 * kq + 8 * j + kslot(m);
                const uint32_t nib = (static_cast<uint32_t>(static_cast<int8_t>(qrow[k]) + 8)) & 0xfu;
                word |= nib << (4 * m);
              }
              chunk[j] = word;  // little-endian host
            }
          }
        }
      }
    }
  });
  if (bad.load() == 1) return fail(NQ_ERR_OUT_OF_RANGE, "nq_pack_weights: non-finite weight");
  if (bad.load() == 2) return fail(NQ_ERR_OUT_OF_RANGE, "nq_pack_weights: group scale overflows fp16");
  return NQ_OK;
}

nq_status nq_unpack_weights(const void* packed, int32_t N, int32_t K, int32_t group,
                            nq_mat_kind kind, int32_t head_dim, int8_t* q_out, uint16_t* s_out) {
  if (!packed || !q_out || !s_out) return fail(NQ_ERR_INVALID_ARG, "nq_unpack_weights: null pointer");
  nq_status st = check_pack_args(N, K, group, kind, head_dim);
  if (st != NQ_OK) return st;
  const int64_t T = tiles_of(N), G = K / kGroup;
  const uint8_t* codes = static_cast<const uint8_t*>(packed);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(codes + codes_bytes(N, K));
  parallel_for(T, [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; ++t)
      for (int r = 0; r < kTileRows; ++r) {
        const int64_t n = tile_row_logical(kind, N, head_dim, t, r);
        if (n >= N) continue;
        for (int64_t g = 0; g < G; ++g) {
          s_out[n * G + g] = scales[(t * G + g) * kTileRows + r];
          const uint8_t* blk = codes + (t * G + g) * kBlockBytes;
          for (int kq = 0; kq < 4; ++kq) {
            const uint32_t* chunk = reinterpret_cast<const uint32_t*>(blk + 16 * (16 * kq + r));
            for (int j = 0; j < 4; ++j)
              for (int m = 0; m < 8; ++m) {
                const int k = 32 * kq + 8 * j + kslot(m);
                const int nib = static_cast<int>((chunk[j] >> (4 * m)) & 0xfu);
                q_out[n * static_cast<int64_t>(K) + g * kGroup + k] = static_cast<int8_t>(nib - 8);
              }
          }
        }
      }
  });
  return NQ_OK;
}

nq_status nq_config_check(const nq_config* c) {
  if (!c) return fail(NQ_ERR_INVALID_ARG, "null config");
  if (c->layers <= 0 || c->hidden <= 0 || c->intermediate <= 0 || c->n_heads <= 0 ||
      c->n_kv_heads <= 0 || c->vocab <= 0 || c->max_batch <= 0 || c->max_pos <= 0)
    return fail(NQ_ERR_INVALID_ARG, "config: sizes must be positive");
  if (c->group != kGroup) return fail(NQ_ERR_INVALID_ARG, "config: group must be 128");
  if (c->page_tokens != kPageTokens) return fail(NQ_ERR_INVALID_ARG, "config: page_tokens must be 16");
  if (c->hidden % kGroup || c->intermediate % kGroup)
    return fail(NQ_ERR_INVALID_ARG, "config: hidden and intermediate must be multiples of 128");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(NQ_ERR_UNSUPPORTED, "config: head_dim must be 64 or 128 (got %d)", c->head_dim);
  if (c->n_heads % c->n_kv_heads) return fail(NQ_ERR_INVALID_ARG, "config: n_heads %% n_kv_heads != 0");
  if (c->n_heads / c->n_kv_heads > 8)
    return fail(NQ_ERR_UNSUPPORTED, "config: more than 8 query heads per KV head");
  if ((static_cast<int64_t>(c->n_heads) * c->head_dim) % kGroup)
    return fail(NQ_ERR_INVALID_ARG, "config: n_heads*head_dim must be a multiple of 128");
  if (c->max_batch > kMaxBatch) return fail(NQ_ERR_UNSUPPORTED, "config: max_batch > 8");
  if (!(c->rms_eps > 0.0f) || !(c->rope_theta > 1.0f))
    return fail(NQ_ERR_INVALID_ARG, "config: rms_eps must be > 0 and rope_theta > 1");
  return NQ_OK;
}

size_t nq_rope_table_bytes(const nq_config* c) {
  if (nq_config_check(c) != NQ_OK) return 0;
  return static_cast<size_t>(c->max_pos) * (c->head_dim / 2) * 2 * sizeof(float);
}

// cos/sin of pos * theta^(-2i/d), evaluated in double precision, stored float32.
nq_status nq_rope_table_fill(const nq_config* c, float* out) {
  nq_status st = nq_config_check(c);
  if (st != NQ_OK) return st;
  if (!out) return fail(NQ_ERR_INVALID_ARG, "nq_rope_table_fill: null output");
  const int half = c->head_dim / 2;
  std::vector<double> inv(half);
  for (int i = 0; i < half; ++i)
    inv[i] = std::pow(static_cast<double>(c->rope_theta), -2.0 * i / c->head_dim);
  parallel_for(c->max_pos, [&](int64_t p0, int64_t p1) {
    for (int64_t p = p0; p < p1; ++p)
      for (int i = 0; i < half; ++i) {
        const double a = static_cast<double>(p) * inv[i];
        out[(p * half + i) * 2 + 0] = static_cast<float>(std::cos(a));
        out[(p * half + i) * 2 + 1] = static_cast<float>(std::sin(a));
      }
  });
  return NQ_OK;
}

}  // extern "C"
