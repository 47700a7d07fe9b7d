/*
 * gguf_file.h -- GGUF file reader of libgguf_qk.so (C ABI): maps a GGUF file,
 * walks its header, metadata and tensor records, and hands out the raw block
 * bytes of each tensor (as a host pointer into the mapping, or copied to
 * device memory) for the multiply entry points of gguf_qk.h.
 *
 * File layout read here ("GGUF Inferencer in R", section 2.1, byte blueprint;
 * "GGUF: The File Format Powering Local LLM Inference", "What is stored inside
 * a GGUF file" and its worked byte count). Every number is little-endian:
 *   header   "GGUF" magic, u32 version, u64 tensor count, u64 metadata count
 *   metadata per entry: key (string), u32 value type, value
 *   tensors  per record: name (string), u32 number of dimensions, u64 size of
 *            each dimension (fastest first: dims[0] is the row length),
 *            u32 tensor type, u64 offset of the data from the start of the
 *            data blob
 *   padding  zero bytes up to the next multiple of the alignment (32)
 *   data     the tensors' bytes
 * A string is a u64 byte count followed by that many UTF-8 bytes (the width
 * the worked byte count fixes: a 20-character key costs 8 + 20 bytes). An
 * array value is a u32 element type, a u64 element count and the elements.
 *
 * Readings where the pages are silent (GGUF's own conventions, recorded as
 * format facts): value type ids 0 u8, 1 i8, 2 u16, 3 i16, 4 u32, 5 i32,
 * 6 f32, 7 bool (one byte), 8 string, 9 array, 10 u64, 11 i64, 12 f64 (the
 * pages name 4, 8 and 9); tensor type ids 0 F32, 1 F16, 2 Q4_0, 8 Q8_0,
 * 12 Q4_K, 14 Q6_K, 30 BF16 (the pages name F32 = 0 and Q8_0 = 8); a
 * "general.alignment" u32 entry, when present, replaces the alignment of 32.
 * Versions 2 and 3 share this layout and are accepted.
 *
 * The file is untrusted input: every read is bounds-checked, every size and
 * count is checked for overflow and against the file size, and a file that
 * breaks the layout is rejected with GGUF_QK_ERR_FORMAT (never read past the
 * mapping). Tensor data ranges are checked against the file size for every
 * tensor whose type has a known block size.
 *
 * Ownership: gguf_file_open returns a handle that owns the mapping and every
 * string and pointer handed out for it; they stay valid until
 * gguf_file_close. A handle may be read from several threads at once.
 */
#ifndef GGUF_FILE_H
#define GGUF_FILE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes of this header (the others are in gguf_qk.h). */
#define GGUF_QK_ERR_FORMAT (-8)      /* the bytes do not follow the GGUF layout */
#define GGUF_QK_ERR_IO (-9)          /* the file cannot be opened or mapped */
#define GGUF_QK_ERR_NOT_FOUND (-10)  /* no tensor or key of that name / index out of range */

/* Tensor type ids (see the readings above). */
#define GGUF_TENSOR_F32 0
#define GGUF_TENSOR_F16 1
#define GGUF_TENSOR_Q4_0 2
#define GGUF_TENSOR_Q8_0 8
#define GGUF_TENSOR_Q4_K 12
#define GGUF_TENSOR_Q6_K 14
#define GGUF_TENSOR_BF16 30

/* Metadata value type ids. */
#define GGUF_VALUE_U8 0
#define GGUF_VALUE_I8 1
#define GGUF_VALUE_U16 2
#define GGUF_VALUE_I16 3
#define GGUF_VALUE_U32 4
#define GGUF_VALUE_I32 5
#define GGUF_VALUE_F32 6
#define GGUF_VALUE_BOOL 7
#define GGUF_VALUE_STRING 8
#define GGUF_VALUE_ARRAY 9
#define GGUF_VALUE_U64 10
#define GGUF_VALUE_I64 11
#define GGUF_VALUE_F64 12

typedef struct gguf_file gguf_file;   /* opaque handle */

typedef struct gguf_tensor_info {
  const char* name;     /* NUL-terminated, owned by the handle */
  int32_t type;         /* tensor type id */
  int32_t n_dims;       /* 1..4 */
  int64_t dims[4];      /* fastest first; unused entries are 1 */
  int64_t offset;       /* absolute byte offset of the data in the file */
  int64_t nbytes;       /* data bytes, or -1 for a type whose block size is not known */
  const void* data;     /* host pointer to the data inside the mapping */
} gguf_tensor_info;

typedef struct gguf_kv_info {
  const char* key;      /* NUL-terminated, owned by the handle */
  int32_t type;         /* value type id */
  int32_t elem_type;    /* element type of an array, else -1 */
  int64_t count;        /* elements of an array, else 1 */
  const void* data;     /* scalar: its bytes; string: its characters (not NUL-terminated);
                           array: the first element */
  int64_t nbytes;       /* bytes at data: scalar width, string length, or the array payload */
} gguf_kv_info;

/* Bytes of a tensor of `type` with `dims` (fastest first): rows x row bytes,
 * where the row is dims[0] weights and rows is the product of the others.
 * F32 4, F16/BF16 2 bytes per weight; Q8_0 34 and Q4_0 18 bytes per 32
 * weights; Q4_K 144 and Q6_K 210 bytes per 256 weights ("GGUF: The File
 * Format...", bytes per block in the bits-per-weight listing). Returns
 * GGUF_QK_ERR_SHAPE for a row length the type's blocks do not divide, a
 * dimension < 0, or overflow; GGUF_QK_ERR_FORMAT for an unknown type. */
int64_t gguf_tensor_nbytes(int32_t type, int32_t n_dims, const int64_t* dims);

/* Maps and parses `path`. On success *out is a new handle (GGUF_QK_OK). */
int gguf_file_open(const char* path, gguf_file** out);

/* Unmaps and frees; NULL is ignored. */
void gguf_file_close(gguf_file* f);

int32_t gguf_file_version(const gguf_file* f);
int64_t gguf_file_tensor_count(const gguf_file* f);
int64_t gguf_file_kv_count(const gguf_file* f);
int64_t gguf_file_alignment(const gguf_file* f);
/* Absolute file offset of the data blob (after the padding). */
int64_t gguf_file_data_offset(const gguf_file* f);
int64_t gguf_file_size(const gguf_file* f);

/* Record i (0-based, in file order). */
int gguf_file_tensor(const gguf_file* f, int64_t i, gguf_tensor_info* out);
int gguf_file_kv(const gguf_file* f, int64_t i, gguf_kv_info* out);

/* Index of the tensor / key with that exact name, or GGUF_QK_ERR_NOT_FOUND. */
int64_t gguf_file_find_tensor(const gguf_file* f, const char* name);
int64_t gguf_file_find_kv(const gguf_file* f, const char* key);

/* Element j of string-array entry i: pointer to its characters and length. */
int gguf_file_kv_array_string(const gguf_file* f, int64_t i, int64_t j, const char** str,
                              int64_t* len);

/* Copies tensor i's bytes to device memory `dst` (at least nbytes, 16-byte
 * aligned) on `stream` and returns once the copy has completed: the call
 * synchronizes `stream` (work queued on it before the call finishes too), so
 * the mapping it reads from may be closed as soon as the call returns. Fails
 * with GGUF_QK_ERR_FORMAT for a tensor of unknown size, GGUF_QK_ERR_LAUNCH if
 * the copy or the synchronization fails. */
int gguf_file_upload_tensor(const gguf_file* f, int64_t i, void* dst, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GGUF_FILE_H */
