/*
 * gguf_qk.h -- C ABI of libgguf_qk.so: dequantization of GGUF block-quantized
 * weight matrices (Q8_0, Q4_K) and the fused dequantize-and-multiply against
 * activations on an AMD Instinct MI355X (gfx950).
 *
 * Formats (bytes exactly as a GGUF file stores them, never repacked):
 *
 *  Q8_0  34-byte blocks of 32 consecutive weights of one row: a little-endian
 *        fp16 multiplier d, then 32 int8 values q; w = q * d.
 *        ("GGUF Inferencer in R", section 2.1, byte blueprint of a Q8_0 tensor;
 *        "GGUF: The File Format Powering Local LLM Inference", "How a Q8_0
 *        block is stored".)
 *
 *  Q4_K  144-byte super-blocks of 256 weights of one row, 8 sub-blocks of 32,
 *        each sub-block with a 6-bit scale and a 6-bit min
 *        ("GGUF: The File Format...", k-quant paragraph and bits-per-weight
 *        table). Field placement (GGUF's on-disk layout; not printed on those
 *        pages): bytes 0-1 fp16 d, 2-3 fp16 dmin, 4-15 twelve bytes S holding
 *        the 8 scales sc[j] and 8 mins m[j] (j<4: sc=S[j]&63, m=S[j+4]&63;
 *        j>=4: sc=(S[j+4]&15)|((S[j-4]>>6)<<4), m=(S[j+4]>>4)|((S[j]>>6)<<4)),
 *        16-143 quants: byte 32g+l holds weight 64g+l in its low nibble and
 *        weight 64g+32+l in its high nibble. w = d*sc[j]*q - dmin*m[j].
 *
 * Matrix layout: W is rows x cols (cols = K fastest), stored as `rows` runs of
 * gguf_row_bytes(type, cols) bytes with no padding between rows ("GGUF
 * Inferencer in R", section 2.1: Q8_0 x cols/32 chunks per row, rows back to
 * back). The matvec computes y[r] = sum_k w[r,k] x[k] (culpeo.ws blog, the
 * naive-implementation post, matvec(w:[r,c], x:[c]) -> [r]).
 *
 * Conventions for every entry point below:
 *  - All pointers are DEVICE pointers into memory the caller owns and
 *    allocated (the output memory is always provided by the caller, as in the
 *    culpeo.ws naive-implementation post). The library keeps no pointer after
 *    returning.
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *    without synchronizing. Device-side faults surface at the caller's next
 *    synchronization, as for any HIP operation.
 *  - Arguments are validated before any HIP call; a failed call enqueues
 *    nothing and returns a negative status. rows == 0 (or n_tokens == 0)
 *    returns GGUF_QK_OK without launching anything.
 *  - Outputs are fully overwritten (never accumulated into).
 *  - W needs 16-byte alignment; x, y, X, Y need 16-byte alignment.
 *  - Scratch: kernels that split K over blocks or count row groups (the
 *    prefill and small-batch multiplies, the fused gate/up and norm
 *    epilogues, the fallback GEMV kernels) keep partial sums and counters in
 *    a scratch slot inside the library: a static device array of
 *    GGUF_QK_STREAM_SLOTS slots per device, nothing allocated at call time.
 *    The first such call on a stream takes a free slot for that stream and
 *    the stream keeps it until gguf_qk_stream_release; later calls on the
 *    stream reuse it. Calls on one stream run in stream order and calls on
 *    different streams use different slots, so calls on any streams may
 *    overlap in time. A call that needs a slot when every slot of the device
 *    is held by other streams returns GGUF_QK_ERR_LIMIT and enqueues
 *    nothing. The per-thread default stream (hipStreamPerThread) is one
 *    stream per calling thread. A HIP graph captured from a stream keeps
 *    that stream's slot in its kernels: do not replay it while other work
 *    that uses the same slot may run.
 */
#ifndef GGUF_QK_H
#define GGUF_QK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GGUF_QK_ABI_VERSION 2

/* Scratch slots per device (streams that may hold scratch at one time). */
#define GGUF_QK_STREAM_SLOTS 8

/* Status codes. */
#define GGUF_QK_OK 0
#define GGUF_QK_ERR_NULL (-1)     /* a required pointer is NULL */
#define GGUF_QK_ERR_SHAPE (-2)    /* rows/n_tokens < 0, cols <= 0, cols not a multiple of
                                     32 (Q8_0) or 256 (Q4_K), or a byte size overflows */
#define GGUF_QK_ERR_ALIGN (-3)    /* a pointer is not 16-byte aligned */
#define GGUF_QK_ERR_ALIAS (-4)    /* an output range overlaps an input range */
#define GGUF_QK_ERR_DEVICE (-5)   /* no HIP device, or the current device is not gfx950 */
#define GGUF_QK_ERR_LAUNCH (-6)   /* the kernel launch failed */
#define GGUF_QK_ERR_LIMIT (-7)    /* request exceeds a documented library limit */

/* Tensor type ids as a GGUF tensor-info record stores them: 8 = Q8_0 ("GGUF
 * Inferencer in R", section 2.1, example tensor entry); 12 = Q4_K (GGUF's id,
 * not printed on those pages). */
#define GGUF_QK_TYPE_Q8_0 8
#define GGUF_QK_TYPE_Q4_K 12
/* GGUF's ids of two more block types ("GGUF: The File Format...", their block
 * sizes: Q4_0 18 bytes per 32 weights, Q6_K 210 per 256). */
#define GGUF_QK_TYPE_Q4_0 2
#define GGUF_QK_TYPE_Q6_K 14

/* ABI version of the loaded library (GGUF_QK_ABI_VERSION it was built with). */
int gguf_qk_abi_version(void);

/* Static text for a status code; never NULL. */
const char* gguf_qk_strerror(int status);

/* Bytes of one row of `cols` weights of `type`, or a negative status
 * (GGUF_QK_ERR_SHAPE for an unknown type or a cols the type cannot hold). */
int64_t gguf_row_bytes(int type, int64_t cols);

/* --- standalone dequantization ------------------------------------------ */

/* out[r*cols + k] = w[r,k] as fp32 (row-major [rows x cols]). The value is
 * bit-exact: Q8_0's q*d is exact in fp32; Q4_K's d*sc*q and dmin*m are exact
 * and their difference is rounded once to nearest-even. */
int dequant_q8_0(const void* W, float* out, int64_t rows, int64_t cols, hipStream_t stream);
int dequant_q4_k(const void* W, float* out, int64_t rows, int64_t cols, hipStream_t stream);

/* out = bf16 bit patterns of the fp32 dequant above, rounded to nearest-even
 * (the tile type of the prefill path). */
int dequant_q4_k_bf16(const void* W, uint16_t* out, int64_t rows, int64_t cols,
                      hipStream_t stream);

/* --- decode: fused dequant x vector (batch 1) ----------------------------- */

/* y[r] = sum_k w[r,k] * x[k]; x fp32 [cols], y fp32 [rows]. fp32 arithmetic,
 * any summation order; deterministic (two calls give identical bits).
 * Q8_0 needs cols % 32 == 0, Q4_K cols % 256 == 0. */
int gguf_qmatvec_q8_0(const void* W, const float* x, float* y, int64_t rows, int64_t cols,
                      hipStream_t stream);
int gguf_qmatvec_q4_k(const void* W, const float* x, float* y, int64_t rows, int64_t cols,
                      hipStream_t stream);

/* --- the other block types of GGUF files: Q4_0 and Q6_K ------------------- */

/* Q4_0 ("GGUF: The File Format...", "How a Q8_0 block is stored": the same
 * recipe with 4-bit integers; 18-byte blocks of 32 weights). Field placement
 * (GGUF's layout, not on the pages): fp16 d in bytes 0-1, then 16 bytes; byte
 * j holds the code of weight j in its low nibble and of weight j + 16 in its
 * high nibble; w = (code - 8) * d. cols % 32 == 0.
 *
 * Q6_K (210-byte super-blocks of 256 weights, same listing). Field placement
 * (GGUF's layout): bytes 0-127 ql (low 4 bits of the 6-bit codes), 128-191 qh
 * (high 2 bits), 192-207 sixteen int8 scales of 16 weights each, 208-209 fp16
 * d. Weight 128 n + 32 k + l (n = 0..1, k = 0..3, l = 0..31) has low bits
 * ql[64 n + l + 32 (k & 1)] >> (k >= 2 ? 4 : 0) & 15 and high bits
 * qh[32 n + l] >> 2 k & 3; w = d * scale[i / 16] * (code - 32).
 * cols % 256 == 0.
 *
 * Dequant: fp32 [rows x cols], bit-exact (both products are exact in fp32).
 * GEMV: y = W x in fp32 as gguf_qmatvec_q8_0 (any summation order,
 * deterministic). In gguf_qmatvec_batch these two types run one launch per
 * GEMV (a Q4_K_M file keeps some tensors in Q6_K); gguf_qmatvec_batch_ep has
 * no epilogue for them. */
int dequant_q4_0(const void* W, float* out, int64_t rows, int64_t cols, hipStream_t stream);
int dequant_q6_k(const void* W, float* out, int64_t rows, int64_t cols, hipStream_t stream);
int gguf_qmatvec_q4_0(const void* W, const float* x, float* y, int64_t rows, int64_t cols,
                      hipStream_t stream);
int gguf_qmatvec_q6_k(const void* W, const float* x, float* y, int64_t rows, int64_t cols,
                      hipStream_t stream);

/* --- decode step: an ordered list of GEMVs -------------------------------- */

/* One GEMV of a list: y[r] = sum_k w[r,k] x[k] as above. */
typedef struct gguf_qk_gemv {
  const void* W;   /* device, rows x gguf_row_bytes(type, cols) bytes */
  const float* x;  /* device, cols floats */
  float* y;        /* device, rows floats (written) */
  int64_t rows;
  int64_t cols;
  int32_t type;    /* GGUF_QK_TYPE_Q8_0 or GGUF_QK_TYPE_Q4_K */
  int32_t stage;   /* adjacent entries with equal stage form one step */
  int32_t reserved[2];
} gguf_qk_gemv;

/* Runs the GEMVs of `list` (a HOST array of n entries, read during the call)
 * as a sequence of steps on `stream`: adjacent entries with the same `stage`
 * form one step and may run concurrently (in one launch when they share a
 * format), so within a step no y may overlap another entry's y, x or W
 * (GGUF_QK_ERR_ALIAS). Each step starts after the previous step has finished,
 * exactly as if every step were issued separately on the stream, so an entry
 * may read as x what an earlier step wrote as y. This is the decode step of a
 * transformer layer: q/k/v read the same normalised input, so do gate/up
 * ("GGUF Inferencer in R", section 5.2: Q, K and V come from the same normed
 * input; G and U likewise). Every entry is validated before anything is
 * enqueued. */
int gguf_qmatvec_batch(const gguf_qk_gemv* list, int32_t n, hipStream_t stream);

/* --- decode step with the neighbouring steps fused ------------------------ */

/* What the GEMV of a list entry does with its outputs besides storing y: the
 * steps either side of the decode GEMVs ("GGUF Inferencer in R", section 5.2:
 * RMSN(v) = norm * v / sqrt(mean(v^2) + epsilon) before q/k/v and before
 * gate/up; Activation = SiLU(G) * U with SiLU(x) = x / (1 + exp(-x)); the
 * residual adds after the output and down projections), folded into the
 * GEMV that produces or consumes the vector so that they cost no launch.
 * A NULL pointer (or pair 0) switches a part off. */
typedef struct gguf_qk_gemv_ep {
  /* Input RMSN: y is scaled by 1 / sqrt(sum(scale_ss[0..scale_n)) / cols + eps).
   * With x = v * norm (elementwise) and scale_ss the partial sums of v^2,
   * y = W RMSN(v): RMSN's scalar factor moves past the product. */
  const float* scale_ss;
  int64_t scale_n;
  float eps;
  /* 0: none. 1: this entry is the gate of a pair whose up is the next entry;
   * 2: the up of the previous entry. The pair (same stage, type and rows) writes
   * act = SiLU(y_gate) * y_up (rows floats, the same pointer in both). */
  int32_t pair;
  /* y = residual + ... (rows floats; may be y itself, not a partial overlap). */
  const float* residual;
  /* Output half of the next RMSN: norm_out = y * norm_w (rows floats) and,
   * where ss_out is given, ss_out[j] = sum of y^2 over rows 64 j .. 64 j + 63
   * (ceil(rows / 64) floats), the scale_ss of the GEMVs that read norm_out.
   * norm_w and norm_out together or neither; ss_out only with them. */
  const float* norm_w;
  float* norm_out;
  float* ss_out;
  float* act;
  /* Input RMSN from the vector itself, in place of scale_ss: v (cols floats,
   * 16-byte aligned), with x = v * norm; the GEMV forms sum(v^2) in a fixed
   * order and scales y by 1 / sqrt(sum(v^2) / cols + eps). The producer of v
   * then needs no ss_out, and no row-group completion between its blocks.
   * NULL: off. At most one of scale_ss and scale_v. */
  const float* scale_v;
} gguf_qk_gemv_ep;

/* gguf_qmatvec_batch with an epilogue per entry (ep: n entries, or NULL for
 * none). Entries with epilogues must be Q4_K, or Q8_0 with cols % 256 == 0
 * (GGUF_QK_ERR_SHAPE otherwise).
 * Epilogue arrays need 4-byte alignment; their outputs may not overlap any
 * input or output of the step. The fp32 sums of the scale and of ss_out run
 * in fixed orders: results are deterministic. */
int gguf_qmatvec_batch_ep(const gguf_qk_gemv* list, const gguf_qk_gemv_ep* ep, int32_t n,
                          hipStream_t stream);

/* The same steps standalone, on vectors of n fp32 (16-byte aligned):
 *   gguf_rmsnorm_prep_f32: vw = v * norm_w and ss[j] = sum of v^2 over
 *     elements 64 j .. 64 j + 63 (the input half of a fused RMSN, for a
 *     vector no GEMV epilogue produced, such as the first layer's input);
 *   gguf_rmsnorm_f32: out = RMSN(v) (one block; for the unfused path);
 *   gguf_swiglu_f32: out = SiLU(g) * u;  gguf_add_f32: out = a + b
 *     (out may be one of the inputs exactly). */
int gguf_rmsnorm_prep_f32(const float* v, const float* norm_w, float* vw, float* ss, int64_t n,
                          hipStream_t stream);
int gguf_rmsnorm_f32(const float* v, const float* norm_w, float eps, float* out, int64_t n,
                     hipStream_t stream);
int gguf_swiglu_f32(const float* g, const float* u, float* out, int64_t n, hipStream_t stream);
int gguf_add_f32(const float* a, const float* b, float* out, int64_t n, hipStream_t stream);

/* --- prefill: fused dequant x matrix (small batch, MFMA) ------------------ */

/* Y[n, r] = sum_k X[n, k] * w[r, k] for n < n_tokens. X bf16 row-major
 * [n_tokens x cols], Y bf16 row-major [n_tokens x rows]. The prefill is the
 * decode math with the whole prompt as one matrix ("GGUF Inferencer in R",
 * section 1 and section 4). Weights are dequantized to bf16 (nearest-even)
 * tiles, multiplied on the matrix cores with fp32 accumulation, and Y is
 * rounded to nearest-even bf16. */
int gguf_qmatmul_q4_k(const void* W, const uint16_t* X, uint16_t* Y, int64_t n_tokens,
                      int64_t rows, int64_t cols, hipStream_t stream);

/* The same for n (1 .. 4) Q4_K matrices W[0..n-1] of rows[m] rows and the same
 * cols that multiply one X (the query, key and value projections, or gate
 * and up, read the same normalized input: "GGUF Inferencer in R", section 4,
 * and the culpeo.ws naive-implementation post, the layer loop), in one
 * launch: Y[m] bf16 [n_tokens x rows[m]]. Arrays W, Y and rows are host
 * arrays of n entries; the matrices and outputs are device buffers with the
 * single-matrix rules (alignment, no output overlapping any input or another
 * output). Every matrix is validated before anything is launched; an error
 * launches nothing. rows[m] = 0 skips matrix m (with n > 1 its W[m] and
 * Y[m] are not looked at and may be null). Results equal the
 * single-matrix call's within the bf16 bar (the K split, which sets the
 * fp32 summation order, is chosen for the whole group). */
int gguf_qmatmul_q4_k_multi(const void* const* W, uint16_t* const* Y, const int64_t* rows, int32_t n,
                            const uint16_t* X, int64_t n_tokens, int64_t cols, hipStream_t stream);

/* --- small batch: fused dequant x a few fp32 vectors (MFMA) --------------- */

/* Y[n, r] = sum_k X[n, k] * w[r, k] for n < n_tokens: the fp32 matvec above
 * applied to each token row of X at once (culpeo.ws naive-implementation
 * post, the matvec op; "GGUF Inferencer in R", section 1: several tokens make
 * the activation a matrix). X fp32 row-major [n_tokens x cols], Y fp32
 * row-major [n_tokens x rows]. Same accuracy bar as the matvec (fp32
 * accumulation): the integer quants enter the matrix cores exactly, each x
 * as a pair of bf16 whose sum is x within 2^-16 |x|, and every block scale is
 * applied in fp32. Deterministic. Built for a few tokens (1 to 64; blocks of
 * 32 tokens x 128 rows, weights re-read per 32 tokens); cols must be a
 * multiple of 256 for both formats (GGUF_QK_ERR_SHAPE otherwise). */
int gguf_qmatmul_f32_q8_0(const void* W, const float* X, float* Y, int64_t n_tokens,
                          int64_t rows, int64_t cols, hipStream_t stream);
int gguf_qmatmul_f32_q4_k(const void* W, const float* X, float* Y, int64_t n_tokens,
                          int64_t rows, int64_t cols, hipStream_t stream);

/* The same for n (1 .. 4) matrices of one type that multiply one X (as for
 * the prefill above: q, k, v, or gate and up, read the same input), in one
 * launch: Y[m] fp32 [n_tokens x rows[m]]. W, Y and rows are host arrays of
 * n entries, with the single-matrix rules per matrix and no output
 * overlapping another; all are validated before anything is launched.
 * rows[m] = 0 skips matrix m (with n > 1 its W[m] and Y[m] may be null).
 * Results are within the same bar as the single-matrix call (the K split is
 * chosen for the whole group). */
int gguf_qmatmul_f32_q8_0_multi(const void* const* W, float* const* Y, const int64_t* rows, int32_t n,
                                const float* X, int64_t n_tokens, int64_t cols, hipStream_t stream);
int gguf_qmatmul_f32_q4_k_multi(const void* const* W, float* const* Y, const int64_t* rows, int32_t n,
                                const float* X, int64_t n_tokens, int64_t cols, hipStream_t stream);

/* --- measurement ---------------------------------------------------------- */

/* Kernel family of the calling thread's most recent GEMV launch through this
 * library (gguf_qmatvec_*, gguf_qmatvec_batch*), for tests and diagnostics:
 * which launch form a call actually took (0 before any). Host state only. */
#define GGUF_QK_LAUNCH_NONE 0
#define GGUF_QK_LAUNCH_LK_SINGLE 1   /* lanes along K, one GEMV, descriptor as scalar arguments */
#define GGUF_QK_LAUNCH_LK_TWO 2      /* lanes along K, two GEMVs of one x, scalar arguments */
#define GGUF_QK_LAUNCH_LK_THREE 3    /* lanes along K, three GEMVs of one x, packed scalar arguments */
#define GGUF_QK_LAUNCH_LK_GROUP 4    /* lanes along K, up to four GEMVs from a descriptor array */
#define GGUF_QK_LAUNCH_LK_LONG 5     /* lanes along K, rows of more than 16 super-blocks */
#define GGUF_QK_LAUNCH_LKS 6         /* K split over the waves of a block (odd and long rows) */
#define GGUF_QK_LAUNCH_SPLIT_K 7     /* split-K block or lane-per-row kernels (scratch) */
#define GGUF_QK_LAUNCH_OTHER 8       /* Q4_0 / Q6_K lane-quad kernel */
#define GGUF_QK_LAUNCH_ROWWISE 9     /* Q8_0 rows that are not whole 256-weight chunks */
int gguf_qk_last_launch(void);

/* Releases the scratch slot held by `stream` on the current device (for
 * hipStreamPerThread: the calling thread's), so that another stream can take
 * it. The caller guarantees that no work of this library enqueued on the
 * stream is still pending (synchronize the stream first). Releasing a stream
 * that holds no slot does nothing. Returns GGUF_QK_OK, or GGUF_QK_ERR_DEVICE. */
int gguf_qk_stream_release(hipStream_t stream);

/* Streaming-read probe: reads `bytes` (a multiple of 16) from device buffer
 * `buf` once with 16-byte vector loads spread over every compute unit, and
 * writes nothing unless the XOR of all words equals 0x9E3779B9, in which case
 * it stores that word to *sink. Timing it gives the device's achievable read
 * bandwidth, the practical ceiling for the weight stream. */
int gguf_qk_probe_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);

/* Latency probe: one wave of 64 lanes; lane l starts at entry l of `next` (n
 * uint32 entries, n a power of two, 64 <= n <= 2^31, device memory) and follows
 * i = next[i] & (n - 1) `steps` times, every load waiting for the one before.
 * Writes out[0] = the elapsed ticks of the device's constant 100 MHz clock
 * between the first load and the completion of the last, out[1] = lane 0's
 * last index (out: 2 uint64 in device memory, 16-byte aligned). Entries past
 * n are masked into range, so any buffer contents are safe. With `next` a
 * single cycle spread over a buffer larger than a cache level, out[0] * 10 ns /
 * steps is that level's (or HBM's) latency for a dependent load. */
int gguf_qk_probe_latency(const uint32_t* next, int64_t n, int64_t steps, uint64_t* out, hipStream_t stream);

/* Stage timelines of the decode GEMV kernels (measurement; the instrumented
 * build libgguf_qk_timeline.so only, compiled with GQK_TIMELINE: in the
 * default library both calls return GGUF_QK_ERR_LIMIT and do nothing).
 * gguf_qk_timeline_setup(mult) clears the record buffer and arms the kernels
 * (mult odd; 0 disarms): from then on every wave of a lanes-along-K launch
 * writes a 32-byte record {six uint32 time stamps of the 100 MHz device
 * clock: entry, loads issued, activations staged, first row step stored, last
 * row step computed, end; HW_ID; XCD id} at [slot][wave index in the grid] of
 * a [4096][2048] array, slot = (key * mult mod 2^64) >> 52 with key the
 * launch's first weight pointer (waves past 2048 are not recorded; the
 * caller picks mult so that the launches it traces take distinct slots).
 * gguf_qk_timeline_fetch copies that whole array (bytes must be
 * 4096 * 2048 * 32) to host memory, synchronously. The instrumented build
 * allocates its record buffer (256 MiB) on the first setup call. */
int gguf_qk_timeline_setup(uint64_t mult);
int gguf_qk_timeline_fetch(void* host_out, int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* GGUF_QK_H */
