// Packed-weight container of libnq: one file holding a model's configuration
// and its tensors in the packed tile layout, written once offline and
// memory-mapped at load, so that loading does no repacking ("How to build your
// own LLM runtime from scratch", "What it actually builds": the INT4 weights
// live in a memory-mapped binary file with a magic-byte header).
//
// File layout (little-endian), format version 1:
//   [0, 4096)   header: magic "NQPACKW4", format version, packed-tile layout
//               version, model configuration, tensor count, table offset and
//               size, header checksum
//   data        each tensor at a 4096-byte aligned offset
//   table       one 96-byte record per tensor (name, role, matrix kind,
//               shape, offset, size, FNV-1a 64 checksum of the bytes)
// The table is written last, so a writer streams tensors without holding them.
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstring>
#include <string>
#include <vector>

#include "common.hpp"

using namespace nq;

namespace {

constexpr char kMagic[8] = {'N', 'Q', 'P', 'A', 'C', 'K', 'W', '4'};
constexpr uint32_t kFormatVersion = 1;
constexpr uint64_t kAlign = 4096;
constexpr uint64_t kHeaderBytes = 4096;

// Serialised model configuration (the runtime-only fields max_batch and max_pos
// are not part of a model file).
struct FileConfig {
  int32_t layers, hidden, intermediate, n_heads, n_kv_heads, head_dim, vocab;
  float rms_eps, rope_theta;
  int32_t group, page_tokens;
};

struct FileHeader {
  char magic[8];
  uint32_t format_version;
  uint32_t layout_version;
  FileConfig cfg;
  uint32_t n_tensors;
  uint32_t reserved;
  uint64_t table_offset;
  uint64_t table_bytes;
  uint64_t header_checksum;  // FNV-1a 64 of the bytes before this field
};

struct FileRecord {
  char name[48];
  int32_t role, mat_kind, N, K, head_dim, reserved;
  uint64_t offset, bytes, checksum;
};
static_assert(sizeof(FileRecord) == 96, "record size is part of the format");

uint64_t fnv1a(const void* p, size_t n, uint64_t h = 0xcbf29ce484222325ull) {
  const unsigned char* b = static_cast<const unsigned char*>(p);
  for (size_t i = 0; i < n; ++i) {
    h ^= b[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Bytes a tensor of this description must have; 0 if the description is invalid.
uint64_t expected_bytes(const nq_tensor_desc& d) {
  if (d.N <= 0 || d.K <= 0) return 0;
  if (d.role == NQ_TENSOR_PACKED) {
    if (check_pack_args(d.N, d.K, kGroup, static_cast<nq_mat_kind>(d.mat_kind), d.head_dim) != NQ_OK) return 0;
    return nq_packed_size(d.N, d.K, kGroup);
  }
  if (d.role == NQ_TENSOR_F16) return static_cast<uint64_t>(d.N) * d.K * 2;
  return 0;
}

bool name_ok(const char* name) {
  const size_t n = strnlen(name, sizeof(FileRecord::name));
  return n > 0 && n < sizeof(FileRecord::name);
}

}  // namespace

struct nq_container_writer {
  int fd = -1;
  std::string path;
  FileHeader hdr{};
  uint64_t pos = kHeaderBytes;
  std::vector<FileRecord> recs;
  int32_t expected = 0;
  bool failed = false;
};

struct nq_container {
  void* map = nullptr;
  size_t size = 0;
  FileHeader hdr{};
  std::vector<FileRecord> recs;
};

extern "C" {

nq_status nq_container_create(const char* path, const nq_config* cfg, int32_t n_tensors, nq_container_writer** out) {
  if (!path || !cfg || !out) return fail(NQ_ERR_INVALID_ARG, "nq_container_create: null argument");
  if (n_tensors < 1) return fail(NQ_ERR_INVALID_ARG, "n_tensors must be >= 1");
  nq_status st = nq_config_check(cfg);
  if (st != NQ_OK) return st;
  const int fd = ::open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
  if (fd < 0) return fail(NQ_ERR_IO, "cannot create %s", path);
  nq_container_writer* w = new nq_container_writer;
  w->fd = fd;
  w->path = path;
  memcpy(w->hdr.magic, kMagic, sizeof kMagic);
  w->hdr.format_version = kFormatVersion;
  w->hdr.layout_version = static_cast<uint32_t>(nq_layout_version());
  w->hdr.cfg = FileConfig{cfg->layers, cfg->hidden, cfg->intermediate, cfg->n_heads, cfg->n_kv_heads, cfg->head_dim,
                          cfg->vocab, cfg->rms_eps, cfg->rope_theta, cfg->group, cfg->page_tokens};
  w->expected = n_tensors;
  *out = w;
  return NQ_OK;
}

static bool write_all(int fd, const void* p, size_t n, uint64_t off) {
  const char* b = static_cast<const char*>(p);
  while (n > 0) {
    const ssize_t k = ::pwrite(fd, b, n, static_cast<off_t>(off));
    if (k <= 0) return false;
    b += k;
    n -= static_cast<size_t>(k);
    off += static_cast<uint64_t>(k);
  }
  return true;
}

nq_status nq_container_add(nq_container_writer* w, const nq_tensor_desc* desc, const void* data) {
  if (!w || !desc || !data) return fail(NQ_ERR_INVALID_ARG, "nq_container_add: null argument");
  if (w->failed) return fail(NQ_ERR_STATE, "writer failed earlier");
  if (static_cast<int32_t>(w->recs.size()) >= w->expected)
    return fail(NQ_ERR_STATE, "more tensors than announced (%d)", w->expected);
  if (!name_ok(desc->name)) return fail(NQ_ERR_INVALID_ARG, "tensor name empty or longer than 47 bytes");
  for (const FileRecord& r : w->recs)
    if (strncmp(r.name, desc->name, sizeof r.name) == 0) return fail(NQ_ERR_INVALID_ARG, "duplicate tensor %s", desc->name);
  const uint64_t bytes = expected_bytes(*desc);
  if (bytes == 0 || bytes != desc->bytes)
    return fail(NQ_ERR_INVALID_ARG, "tensor %s: %llu bytes do not match its role and shape", desc->name,
                static_cast<unsigned long long>(desc->bytes));
  FileRecord r{};
  memcpy(r.name, desc->name, strnlen(desc->name, sizeof r.name));
  r.role = desc->role;
  r.mat_kind = desc->mat_kind;
  r.N = desc->N;
  r.K = desc->K;
  r.head_dim = desc->head_dim;
  r.offset = w->pos;
  r.bytes = bytes;
  r.checksum = fnv1a(data, bytes);
  if (!write_all(w->fd, data, bytes, r.offset)) {
    w->failed = true;
    return fail(NQ_ERR_IO, "write to %s failed", w->path.c_str());
  }
  w->pos = align_up(r.offset + bytes);
  w->recs.push_back(r);
  return NQ_OK;
}

nq_status nq_container_finish(nq_container_writer* w) {
  if (!w) return fail(NQ_ERR_INVALID_ARG, "null writer");
  nq_status st = NQ_OK;
  if (w->failed) {
    st = fail(NQ_ERR_STATE, "writer failed earlier");
  } else if (static_cast<int32_t>(w->recs.size()) != w->expected) {
    st = fail(NQ_ERR_STATE, "%zu tensors written, %d announced", w->recs.size(), w->expected);
  } else {
    w->hdr.n_tensors = static_cast<uint32_t>(w->recs.size());
    w->hdr.table_offset = w->pos;
    w->hdr.table_bytes = w->recs.size() * sizeof(FileRecord);
    w->hdr.header_checksum = fnv1a(&w->hdr, offsetof(FileHeader, header_checksum));
    std::vector<char> page(kHeaderBytes, 0);
    memcpy(page.data(), &w->hdr, sizeof w->hdr);
    if (!write_all(w->fd, w->recs.data(), w->hdr.table_bytes, w->hdr.table_offset) ||
        !write_all(w->fd, page.data(), page.size(), 0) || ::fsync(w->fd) != 0)
      st = fail(NQ_ERR_IO, "write to %s failed", w->path.c_str());
  }
  ::close(w->fd);
  delete w;
  return st;
}

nq_status nq_container_open(const char* path, nq_container** out) {
  if (!path || !out) return fail(NQ_ERR_INVALID_ARG, "nq_container_open: null argument");
  const int fd = ::open(path, O_RDONLY);
  if (fd < 0) return fail(NQ_ERR_IO, "cannot open %s", path);
  struct stat sb {};
  if (::fstat(fd, &sb) != 0 || sb.st_size < static_cast<off_t>(kHeaderBytes)) {
    ::close(fd);
    return fail(NQ_ERR_IO, "%s: not a packed-weight container (too short)", path);
  }
  const size_t size = static_cast<size_t>(sb.st_size);
  void* map = ::mmap(nullptr, size, PROT_READ, MAP_PRIVATE, fd, 0);
  ::close(fd);
  if (map == MAP_FAILED) return fail(NQ_ERR_IO, "cannot map %s", path);
  auto bad = [&](const char* why) {
    ::munmap(map, size);
    return fail(NQ_ERR_IO, "%s: %s", path, why);
  };
  FileHeader h{};
  memcpy(&h, map, sizeof h);
  if (memcmp(h.magic, kMagic, sizeof kMagic) != 0) return bad("bad magic (not a packed-weight container)");
  if (h.header_checksum != fnv1a(&h, offsetof(FileHeader, header_checksum))) return bad("header checksum mismatch");
  if (h.format_version != kFormatVersion) return bad("unsupported format version");
  if (h.layout_version != static_cast<uint32_t>(nq_layout_version())) return bad("packed tile layout version differs");
  if (h.n_tensors == 0 || h.table_bytes != static_cast<uint64_t>(h.n_tensors) * sizeof(FileRecord) ||
      h.table_offset < kHeaderBytes || h.table_offset > size || h.table_bytes > size - h.table_offset)
    return bad("tensor table outside the file");
  nq_container* c = new nq_container;
  c->map = map;
  c->size = size;
  c->hdr = h;
  c->recs.resize(h.n_tensors);
  memcpy(c->recs.data(), static_cast<const char*>(map) + h.table_offset, h.table_bytes);
  for (uint32_t i = 0; i < h.n_tensors; ++i) {
    const FileRecord& r = c->recs[i];
    nq_tensor_desc d{};
    memcpy(d.name, r.name, sizeof r.name);
    d.role = r.role;
    d.mat_kind = r.mat_kind;
    d.N = r.N;
    d.K = r.K;
    d.head_dim = r.head_dim;
    d.bytes = r.bytes;
    const bool ok = name_ok(r.name) && expected_bytes(d) == r.bytes && r.offset % kAlign == 0 &&
                    r.offset >= kHeaderBytes && r.offset <= size && r.bytes <= size - r.offset;
    bool dup = false;
    for (uint32_t j = 0; j < i; ++j) dup |= strncmp(c->recs[j].name, r.name, sizeof r.name) == 0;
    if (!ok || dup) {
      delete c;
      return bad("invalid tensor record");
    }
  }
  *out = c;
  return NQ_OK;
}

nq_status nq_container_config(const nq_container* c, nq_config* out) {
  if (!c || !out) return fail(NQ_ERR_INVALID_ARG, "null argument");
  const FileConfig& f = c->hdr.cfg;
  nq_config cfg{};
  cfg.layers = f.layers;
  cfg.hidden = f.hidden;
  cfg.intermediate = f.intermediate;
  cfg.n_heads = f.n_heads;
  cfg.n_kv_heads = f.n_kv_heads;
  cfg.head_dim = f.head_dim;
  cfg.vocab = f.vocab;
  cfg.rms_eps = f.rms_eps;
  cfg.rope_theta = f.rope_theta;
  cfg.group = f.group;
  cfg.page_tokens = f.page_tokens;
  cfg.max_batch = 1;
  cfg.max_pos = 1;
  *out = cfg;
  return NQ_OK;
}

int32_t nq_container_count(const nq_container* c) { return c ? static_cast<int32_t>(c->recs.size()) : -1; }

static nq_status describe(const nq_container* c, const FileRecord& r, nq_tensor_desc* desc, const void** data) {
  if (desc) {
    *desc = nq_tensor_desc{};
    memcpy(desc->name, r.name, sizeof r.name);
    desc->role = r.role;
    desc->mat_kind = r.mat_kind;
    desc->N = r.N;
    desc->K = r.K;
    desc->head_dim = r.head_dim;
    desc->bytes = r.bytes;
  }
  if (data) *data = static_cast<const char*>(c->map) + r.offset;
  return NQ_OK;
}

nq_status nq_container_tensor_at(const nq_container* c, int32_t index, nq_tensor_desc* desc, const void** data) {
  if (!c) return fail(NQ_ERR_INVALID_ARG, "null container");
  if (index < 0 || index >= static_cast<int32_t>(c->recs.size()))
    return fail(NQ_ERR_OUT_OF_RANGE, "tensor index %d out of range", index);
  return describe(c, c->recs[index], desc, data);
}

nq_status nq_container_tensor(const nq_container* c, const char* name, nq_tensor_desc* desc, const void** data) {
  if (!c || !name) return fail(NQ_ERR_INVALID_ARG, "null argument");
  for (const FileRecord& r : c->recs)
    if (strncmp(r.name, name, sizeof r.name) == 0) return describe(c, r, desc, data);
  return fail(NQ_ERR_OUT_OF_RANGE, "no tensor named %s", name);
}

nq_status nq_container_verify(const nq_container* c) {
  if (!c) return fail(NQ_ERR_INVALID_ARG, "null container");
  for (const FileRecord& r : c->recs)
    if (fnv1a(static_cast<const char*>(c->map) + r.offset, r.bytes) != r.checksum)
      return fail(NQ_ERR_IO, "tensor %.48s: checksum mismatch", r.name);
  return NQ_OK;
}

void nq_container_close(nq_container* c) {
  if (!c) return;
  if (c->map) ::munmap(c->map, c->size);
  delete c;
}

}  // extern "C"
