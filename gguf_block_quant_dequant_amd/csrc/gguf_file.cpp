// GGUF file reader (C ABI and layout in include/gguf_file.h): maps the file
// read-only and walks it with a bounds-checked cursor. The file is untrusted:
// no read goes past the mapping, every count and size is checked for overflow
// and against the bytes left, and anything that breaks the layout is reported
// as GGUF_QK_ERR_FORMAT.
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/gguf_file.h"
#include "../../include/gguf_qk.h"

static_assert(__BYTE_ORDER__ == __ORDER_LITTLE_ENDIAN__,
              "the reader copies little-endian file fields directly");

struct gguf_file {
  const uint8_t* map = nullptr;
  uint64_t size = 0;
  int32_t version = 0;
  uint64_t alignment = 32;
  uint64_t data_offset = 0;
  struct Kv {
    std::string key;
    int32_t type = -1;
    int32_t elem_type = -1;
    int64_t count = 1;
    uint64_t data = 0;     // offset of the value payload in the file
    uint64_t nbytes = 0;
    std::vector<uint64_t> str_offsets;   // string arrays: offset of each element's length field
  };
  struct Tensor {
    std::string name;
    int32_t type = -1;
    int32_t n_dims = 0;
    int64_t dims[4] = {1, 1, 1, 1};
    uint64_t offset = 0;   // absolute
    int64_t nbytes = -1;
  };
  std::vector<Kv> kvs;
  std::vector<Tensor> tensors;
};

namespace {

constexpr int kMaxArrayDepth = 4;

struct Cursor {
  const uint8_t* base;
  uint64_t size;
  uint64_t pos;   // invariant: pos <= size

  uint64_t left() const { return size - pos; }
  bool take(uint64_t n, uint64_t* at) {
    if (n > left()) return false;
    *at = pos;
    pos += n;
    return true;
  }
  bool u32(uint32_t* v) {
    uint64_t at;
    if (!take(4, &at)) return false;
    std::memcpy(v, base + at, 4);
    return true;
  }
  bool u64(uint64_t* v) {
    uint64_t at;
    if (!take(8, &at)) return false;
    std::memcpy(v, base + at, 8);
    return true;
  }
  // A string: u64 byte count, then the bytes. Returns the offset of the bytes.
  bool str(uint64_t* at, uint64_t* len) { return u64(len) && take(*len, at); }
};

int64_t scalar_width(uint32_t t) {
  switch (t) {
    case GGUF_VALUE_U8: case GGUF_VALUE_I8: case GGUF_VALUE_BOOL: return 1;
    case GGUF_VALUE_U16: case GGUF_VALUE_I16: return 2;
    case GGUF_VALUE_U32: case GGUF_VALUE_I32: case GGUF_VALUE_F32: return 4;
    case GGUF_VALUE_U64: case GGUF_VALUE_I64: case GGUF_VALUE_F64: return 8;
    default: return -1;
  }
}

// Reads the payload of an array whose element type and count were just read.
// `offsets` (top-level string arrays only) receives each element's offset.
bool read_array_payload(Cursor& c, uint32_t et, uint64_t n, int depth,
                        std::vector<uint64_t>* offsets) {
  const int64_t w = scalar_width(et);
  if (w > 0) {
    if (n > c.left() / (uint64_t)w) return false;
    uint64_t at;
    return c.take(n * (uint64_t)w, &at);
  }
  if (et == GGUF_VALUE_STRING) {
    if (n > c.left() / 8) return false;   // every element needs at least its length field
    if (offsets) offsets->reserve(n);
    for (uint64_t i = 0; i < n; ++i) {
      if (offsets) offsets->push_back(c.pos);
      uint64_t at, len;
      if (!c.str(&at, &len)) return false;
    }
    return true;
  }
  if (et == GGUF_VALUE_ARRAY) {
    if (depth >= kMaxArrayDepth) return false;
    if (n > c.left() / 12) return false;  // element type + count per element
    for (uint64_t i = 0; i < n; ++i) {
      uint32_t et2;
      uint64_t n2;
      if (!c.u32(&et2) || !c.u64(&n2)) return false;
      if (!read_array_payload(c, et2, n2, depth + 1, nullptr)) return false;
    }
    return true;
  }
  return false;
}

bool read_kv(Cursor& c, gguf_file::Kv& kv) {
  uint64_t at, len;
  if (!c.str(&at, &len)) return false;
  kv.key.assign(reinterpret_cast<const char*>(c.base + at), len);
  uint32_t t;
  if (!c.u32(&t)) return false;
  kv.type = (int32_t)t;
  const int64_t w = scalar_width(t);
  if (w > 0) {
    kv.nbytes = (uint64_t)w;
    return c.take(kv.nbytes, &kv.data);
  }
  if (t == GGUF_VALUE_STRING) {
    if (!c.str(&kv.data, &len)) return false;
    kv.nbytes = len;
    return true;
  }
  if (t == GGUF_VALUE_ARRAY) {
    uint32_t et;
    uint64_t n;
    if (!c.u32(&et) || !c.u64(&n)) return false;
    if (n > (uint64_t)INT64_MAX) return false;
    kv.elem_type = (int32_t)et;
    kv.count = (int64_t)n;
    kv.data = c.pos;
    if (!read_array_payload(c, et, n, 1, et == GGUF_VALUE_STRING ? &kv.str_offsets : nullptr))
      return false;
    kv.nbytes = c.pos - kv.data;
    return true;
  }
  return false;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

int parse(gguf_file* f) {
  Cursor c{f->map, f->size, 0};
  uint64_t at;
  if (!c.take(4, &at) || std::memcmp(f->map, "GGUF", 4) != 0) return GGUF_QK_ERR_FORMAT;
  uint32_t version;
  uint64_t n_tensors, n_kv;
  if (!c.u32(&version) || !c.u64(&n_tensors) || !c.u64(&n_kv)) return GGUF_QK_ERR_FORMAT;
  if (version != 2 && version != 3) return GGUF_QK_ERR_FORMAT;
  f->version = (int32_t)version;
  // each entry takes at least 12 bytes (key length + type), each record 28
  if (n_kv > c.left() / 12 || n_tensors > c.left() / 28) return GGUF_QK_ERR_FORMAT;
  f->kvs.resize(n_kv);
  for (auto& kv : f->kvs)
    if (!read_kv(c, kv)) return GGUF_QK_ERR_FORMAT;
  for (const auto& kv : f->kvs) {
    if (kv.key != "general.alignment") continue;
    uint32_t a;
    if (kv.type != GGUF_VALUE_U32) return GGUF_QK_ERR_FORMAT;
    std::memcpy(&a, f->map + kv.data, 4);
    if (a == 0 || (a & (a - 1)) != 0) return GGUF_QK_ERR_FORMAT;
    f->alignment = a;
    break;
  }
  f->tensors.resize(n_tensors);
  std::vector<uint64_t> rel(n_tensors);
  for (uint64_t i = 0; i < n_tensors; ++i) {
    auto& t = f->tensors[i];
    uint64_t len;
    if (!c.str(&at, &len)) return GGUF_QK_ERR_FORMAT;
    t.name.assign(reinterpret_cast<const char*>(f->map + at), len);
    uint32_t nd;
    if (!c.u32(&nd) || nd < 1 || nd > 4) return GGUF_QK_ERR_FORMAT;
    t.n_dims = (int32_t)nd;
    for (uint32_t d = 0; d < nd; ++d) {
      uint64_t v;
      if (!c.u64(&v) || v > (uint64_t)INT64_MAX) return GGUF_QK_ERR_FORMAT;
      t.dims[d] = (int64_t)v;
    }
    uint32_t type;
    if (!c.u32(&type) || !c.u64(&rel[i])) return GGUF_QK_ERR_FORMAT;
    t.type = (int32_t)type;
  }
  // the data blob starts at the next multiple of the alignment
  const uint64_t pad = (f->alignment - c.pos % f->alignment) % f->alignment;
  if (pad > c.left() && n_tensors > 0) return GGUF_QK_ERR_FORMAT;
  f->data_offset = c.pos + pad;
  for (uint64_t i = 0; i < n_tensors; ++i) {
    auto& t = f->tensors[i];
    if (rel[i] % f->alignment != 0) return GGUF_QK_ERR_FORMAT;
    if (rel[i] > f->size - f->data_offset) return GGUF_QK_ERR_FORMAT;
    t.offset = f->data_offset + rel[i];
    const int64_t nb = gguf_tensor_nbytes(t.type, t.n_dims, t.dims);
    if (nb == GGUF_QK_ERR_SHAPE) return GGUF_QK_ERR_FORMAT;
    t.nbytes = nb >= 0 ? nb : -1;
    if (nb >= 0 && (uint64_t)nb > f->size - t.offset) return GGUF_QK_ERR_FORMAT;
  }
  return GGUF_QK_OK;
}

}  // namespace

extern "C" {

int64_t gguf_tensor_nbytes(int32_t type, int32_t n_dims, const int64_t* dims) {
  if (!dims || n_dims < 1 || n_dims > 4) return GGUF_QK_ERR_SHAPE;
  int64_t block_bytes, block_weights;
  switch (type) {
    case GGUF_TENSOR_F32: block_bytes = 4; block_weights = 1; break;
    case GGUF_TENSOR_F16: case GGUF_TENSOR_BF16: block_bytes = 2; block_weights = 1; break;
    case GGUF_TENSOR_Q4_0: block_bytes = 18; block_weights = 32; break;
    case GGUF_TENSOR_Q8_0: block_bytes = 34; block_weights = 32; break;
    case GGUF_TENSOR_Q4_K: block_bytes = 144; block_weights = 256; break;
    case GGUF_TENSOR_Q6_K: block_bytes = 210; block_weights = 256; break;
    default: return GGUF_QK_ERR_FORMAT;
  }
  for (int d = 0; d < n_dims; ++d)
    if (dims[d] < 0) return GGUF_QK_ERR_SHAPE;
  if (dims[0] % block_weights) return GGUF_QK_ERR_SHAPE;
  int64_t rows = 1;
  for (int d = 1; d < n_dims; ++d)
    if (!mul_ok(rows, dims[d], &rows)) return GGUF_QK_ERR_SHAPE;
  int64_t row_bytes, total;
  if (!mul_ok(dims[0] / block_weights, block_bytes, &row_bytes)) return GGUF_QK_ERR_SHAPE;
  if (!mul_ok(row_bytes, rows, &total)) return GGUF_QK_ERR_SHAPE;
  return total;
}

int gguf_file_open(const char* path, gguf_file** out) {
  if (!path || !out) return GGUF_QK_ERR_NULL;
  *out = nullptr;
  const int fd = ::open(path, O_RDONLY | O_CLOEXEC);
  if (fd < 0) return GGUF_QK_ERR_IO;
  struct stat st;
  if (::fstat(fd, &st) != 0 || !S_ISREG(st.st_mode)) {
    ::close(fd);
    return GGUF_QK_ERR_IO;
  }
  if (st.st_size < 24) {   // shorter than the header
    ::close(fd);
    return GGUF_QK_ERR_FORMAT;
  }
  void* m = ::mmap(nullptr, (size_t)st.st_size, PROT_READ, MAP_PRIVATE, fd, 0);
  ::close(fd);
  if (m == MAP_FAILED) return GGUF_QK_ERR_IO;
  gguf_file* f = new (std::nothrow) gguf_file;
  if (!f) {
    ::munmap(m, (size_t)st.st_size);
    return GGUF_QK_ERR_IO;
  }
  f->map = static_cast<const uint8_t*>(m);
  f->size = (uint64_t)st.st_size;
  int status;
  try {
    status = parse(f);
  } catch (...) {   // allocation failure on a hostile count
    status = GGUF_QK_ERR_FORMAT;
  }
  if (status != GGUF_QK_OK) {
    gguf_file_close(f);
    return status;
  }
  *out = f;
  return GGUF_QK_OK;
}

void gguf_file_close(gguf_file* f) {
  if (!f) return;
  if (f->map) ::munmap(const_cast<uint8_t*>(f->map), (size_t)f->size);
  delete f;
}

int32_t gguf_file_version(const gguf_file* f) { return f ? f->version : GGUF_QK_ERR_NULL; }
int64_t gguf_file_tensor_count(const gguf_file* f) {
  return f ? (int64_t)f->tensors.size() : GGUF_QK_ERR_NULL;
}
int64_t gguf_file_kv_count(const gguf_file* f) { return f ? (int64_t)f->kvs.size() : GGUF_QK_ERR_NULL; }
int64_t gguf_file_alignment(const gguf_file* f) { return f ? (int64_t)f->alignment : GGUF_QK_ERR_NULL; }
int64_t gguf_file_data_offset(const gguf_file* f) {
  return f ? (int64_t)f->data_offset : GGUF_QK_ERR_NULL;
}
int64_t gguf_file_size(const gguf_file* f) { return f ? (int64_t)f->size : GGUF_QK_ERR_NULL; }

int gguf_file_tensor(const gguf_file* f, int64_t i, gguf_tensor_info* out) {
  if (!f || !out) return GGUF_QK_ERR_NULL;
  if (i < 0 || (uint64_t)i >= f->tensors.size()) return GGUF_QK_ERR_NOT_FOUND;
  const auto& t = f->tensors[i];
  out->name = t.name.c_str();
  out->type = t.type;
  out->n_dims = t.n_dims;
  for (int d = 0; d < 4; ++d) out->dims[d] = t.dims[d];
  out->offset = (int64_t)t.offset;
  out->nbytes = t.nbytes;
  out->data = f->map + t.offset;
  return GGUF_QK_OK;
}

int gguf_file_kv(const gguf_file* f, int64_t i, gguf_kv_info* out) {
  if (!f || !out) return GGUF_QK_ERR_NULL;
  if (i < 0 || (uint64_t)i >= f->kvs.size()) return GGUF_QK_ERR_NOT_FOUND;
  const auto& kv = f->kvs[i];
  out->key = kv.key.c_str();
  out->type = kv.type;
  out->elem_type = kv.elem_type;
  out->count = kv.count;
  out->data = f->map + kv.data;
  out->nbytes = (int64_t)kv.nbytes;
  return GGUF_QK_OK;
}

int64_t gguf_file_find_tensor(const gguf_file* f, const char* name) {
  if (!f || !name) return GGUF_QK_ERR_NULL;
  for (size_t i = 0; i < f->tensors.size(); ++i)
    if (f->tensors[i].name == name) return (int64_t)i;
  return GGUF_QK_ERR_NOT_FOUND;
}

int64_t gguf_file_find_kv(const gguf_file* f, const char* key) {
  if (!f || !key) return GGUF_QK_ERR_NULL;
  for (size_t i = 0; i < f->kvs.size(); ++i)
    if (f->kvs[i].key == key) return (int64_t)i;
  return GGUF_QK_ERR_NOT_FOUND;
}

int gguf_file_kv_array_string(const gguf_file* f, int64_t i, int64_t j, const char** str,
                              int64_t* len) {
  if (!f || !str || !len) return GGUF_QK_ERR_NULL;
  if (i < 0 || (uint64_t)i >= f->kvs.size()) return GGUF_QK_ERR_NOT_FOUND;
  const auto& kv = f->kvs[i];
  if (kv.type != GGUF_VALUE_ARRAY || kv.elem_type != GGUF_VALUE_STRING) return GGUF_QK_ERR_FORMAT;
  if (j < 0 || (uint64_t)j >= kv.str_offsets.size()) return GGUF_QK_ERR_NOT_FOUND;
  uint64_t n;
  std::memcpy(&n, f->map + kv.str_offsets[j], 8);   // checked while parsing
  *str = reinterpret_cast<const char*>(f->map + kv.str_offsets[j] + 8);
  *len = (int64_t)n;
  return GGUF_QK_OK;
}

int gguf_file_upload_tensor(const gguf_file* f, int64_t i, void* dst, hipStream_t stream) {
  if (!f || !dst) return GGUF_QK_ERR_NULL;
  if (i < 0 || (uint64_t)i >= f->tensors.size()) return GGUF_QK_ERR_NOT_FOUND;
  if ((reinterpret_cast<uintptr_t>(dst) & 15u) != 0) return GGUF_QK_ERR_ALIGN;
  const auto& t = f->tensors[i];
  if (t.nbytes < 0) return GGUF_QK_ERR_FORMAT;
  if (t.nbytes == 0) return GGUF_QK_OK;
  // the source is the file mapping: wait for the copy on the stream, so that
  // the file may be closed (and unmapped) as soon as this returns
  if (hipMemcpyAsync(dst, f->map + t.offset, (size_t)t.nbytes, hipMemcpyHostToDevice, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return GGUF_QK_ERR_LAUNCH;
  }
  return GGUF_QK_OK;
}

}  // extern "C"
