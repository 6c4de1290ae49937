/*
 * qgemv.h -- dense-and-sparse quantized matrix-vector product for MI355X (gfx950).
 *
 *   y[b][i] = sum_j dequant(W_dense)[i][j] * x[b][j]  +  sum_{p in row i} values[p] * x[b][col_idx[p]]
 *
 * The operation is the dense-and-sparse decomposition W = W_dense + W_sparse of
 * the page "SqueezeLLM (Dense-and-Sparse Quantization)", section
 * "2. Dense-and-Sparse decomposition", applied to an activation vector.  The
 * dense part holds 3- or 4-bit codes; they decode either through an FP16
 * (scale, zero) pair per group of 16 weights along K (page "SpQR
 * (Sparse-Quantized Representation)", section "Quantification d'un modèle":
 * wbits 3, groupsize 16) or through a per-output-row FP16 lookup table of
 * 2^bits entries (SqueezeLLM page, section "Non-uniform quantization via
 * Lloyd-Max optimisé").  The sparse part holds FP16 outliers in CSR form
 * (SpQR page, section "Le format de stockage sparse": values FP16, col_idx,
 * row_ptr).  A third dense decode, QGEMV_FMT_BPDQ, follows the page "BPDQ:
 * Bit-Plane Decomposition Quantization on a Variable Grid for Large Language
 * Models", section "1. Formulation de la Grille Variable": the code's bit
 * planes select per-group FP16 coefficients, d = C0 + sum_t C_t * B_t.
 *
 * A fourth, QGEMV_FMT_HPTQ, follows the page on GPTQ as Babai's algorithm,
 * section "3. Applications Pratiques et Algorithmes" (HPTQ): every weight,
 * outliers included, is an integer on one unclipped grid with an FP16 step
 * per row and group of 128, and the integers are stored as a canonical
 * prefix (Huffman) code; there is no sparse part.
 *
 * Flow: qgemv_packed_size + qgemv_repack (host, offline) turn the canonical
 * arrays below into one self-describing blob laid out for the gfx950 kernels;
 * the caller copies the blob to device memory it owns; qgemv_create binds a
 * plan to it; qgemv_run enqueues the product on a HIP stream.
 *
 * Every entry point returns an int status: QGEMV_OK (0) or a negative
 * qgemv_status.  No entry point aborts, throws or prints.  All entry points
 * are thread-safe; runs of one plan on different streams with distinct y
 * buffers may overlap, except uniform-code runs at batch 8/16, which share
 * the plan's workspace (qgemv_run) or the device's scratch
 * (qgemv_run_noalloc) and must not overlap in time.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QGEMV_OK = 0,
  QGEMV_ERR_INVALID_ARG = -1,   /* null pointer, bad alignment, inconsistent sizes      */
  QGEMV_ERR_MALFORMED_CSR = -2, /* row_ptr not monotone / not ending at nnz, col out of
                                   range or not strictly ascending within a row          */
  QGEMV_ERR_UNSUPPORTED = -3,   /* bits, format, group size, K or batch outside the
                                   supported set (see qgemv_weights and qgemv_run)      */
  QGEMV_ERR_HIP = -4,           /* a HIP runtime call failed; qgemv_last_hip_error()
                                   returns its hipError_t value                          */
  QGEMV_ERR_SIZE = -5,          /* destination / blob buffer too small, or the blob
                                   header does not match the descriptor                  */
  QGEMV_ERR_SCRATCH = -6        /* qgemv_run_noalloc: the shape needs more workspace
                                   than the library's static scratch holds               */
} qgemv_status;

typedef enum {
  QGEMV_FMT_UNIFORM = 0, /* d = scale[i][g] * (q - zero[i][g]),  g = j / group_size */
  QGEMV_FMT_LUT = 1,     /* d = lut[i][q]                                            */
  QGEMV_FMT_BPDQ = 2,    /* d = coefs[i][g][0] + sum_{t=1..bits} coefs[i][g][t] *
                            ((q >> (t-1)) & 1),  g = j / group_size                  */
  QGEMV_FMT_HPTQ = 3     /* d = scale[i][g] * q, q the integer of weight (i, j)'s
                            prefix codeword in the stream,  g = j / 128             */
} qgemv_format;

/*
 * Canonical ("the pages'") weight format.  All arrays are host memory,
 * little-endian, row-major, borrowed for the duration of the call only.
 *
 *   M, K        W is M x K (out x in).  K % 32 == 0, 32 <= K <= 16384, M >= 1.
 *   bits        3 or 4 (BPDQ: 3).
 *   format      qgemv_format.
 *   group_size  groups run along K.  16 for QGEMV_FMT_UNIFORM; 32, 64 or 128
 *               for QGEMV_FMT_BPDQ, with K % group_size == 0; ignored for LUT.
 *   nnz         number of CSR entries, >= 0.
 *   codes       uint8 [M][K*bits/8]: row i is one contiguous bitstream starting
 *               at byte i*K*bits/8; code j occupies bits [j*bits, j*bits+bits),
 *               least significant bit first.
 *   scales      FP16 bits [M][K/group_size] (UNIFORM), else NULL.  Finite.
 *   zeros       FP16 bits [M][K/group_size] (UNIFORM), else NULL.  Integer
 *               valued in [0, 2^bits - 1].
 *   lut         FP16 bits [M][2^bits] (LUT), else NULL.  Finite.
 *   coefs       FP16 bits [M][K/group_size][bits+1] (BPDQ), else NULL: the
 *               group's C0, then C1 .. C_bits (plane t = bit t-1 of the code).
 *               Finite.
 *
 * QGEMV_FMT_HPTQ uses these instead of the fixed-width fields:
 *   bits        ignored; group_size 128; K % 128 == 0; nnz 0 (no CSR).
 *   codes       the stream: one sequence of codewords, row 0 first, each
 *               written most significant bit first, packed into bytes most
 *               significant bit first; row i starts at bit row_bits[i].
 *   scales      FP16 bits [M][K/128], finite: the steps.
 *   huff_nsym   number of codewords, 1 .. 4096.
 *   huff_len    uint8 [huff_nsym]: codeword lengths 1 .. 16, non-decreasing,
 *               with sum 2^-len <= 1.
 *   huff_sym    int16 [huff_nsym]: the integer of each codeword, |q| <= 2048,
 *               strictly ascending among codewords of equal length.  The
 *               codewords are canonical: in this order, each is the previous
 *               one plus 1, shifted left by the growth in length (the first
 *               is all zeros).
 *   row_bits    int64 [M+1]: row_bits[0] = 0, row i holds exactly K codewords
 *               in bits [row_bits[i], row_bits[i+1]).
 * An HPTQ plan runs at every batch (1, 8, 16); the decode is the same.
 *   row_ptr     int32 [M+1]: row_ptr[0] = 0, non-decreasing, row_ptr[M] = nnz.
 *   col_idx     int32 [nnz]: 0 <= c < K, strictly ascending inside a row.
 *   values      FP16 bits [nnz], finite.  col_idx/values may be NULL iff nnz == 0.
 */
typedef struct {
  int32_t M, K;
  int32_t bits;
  int32_t format;
  int32_t group_size;
  int64_t nnz;
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* zeros;
  const uint16_t* lut;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const uint16_t* values;
  const uint16_t* coefs;
  int32_t huff_nsym;
  const uint8_t* huff_len;
  const int16_t* huff_sym;
  const int64_t* row_bits;
} qgemv_weights;

typedef struct qgemv_plan* qgemv_handle;

/*
 * Validate w (every array, see qgemv_weights) and report the size in bytes of
 * the repacked blob.  Host only; touches no GPU.
 * Errors: INVALID_ARG (null w/bytes, null array, negative nnz), UNSUPPORTED,
 * MALFORMED_CSR.
 */
int qgemv_packed_size(const qgemv_weights* w, size_t* bytes);

/*
 * Validate w and write the gfx950 blob into dst_host (host memory of at least
 * qgemv_packed_size bytes).  Host only.  The blob is a pure function of w.
 * Errors: as qgemv_packed_size, plus SIZE when bytes is too small.
 */
int qgemv_repack(const qgemv_weights* w, void* dst_host, size_t bytes);

/*
 * Host-side inverse of the code repacking: read a blob in host memory and
 * write the canonical codes, one uint8 per weight, to codes_out [M][K] (host,
 * codes_bytes long; M and K are the blob header's).  For tests of the
 * repacker without a GPU.  HPTQ blobs: UNSUPPORTED (their integers do not fit
 * one byte).
 * Errors: INVALID_ARG (null pointer), SIZE (blob shorter than its header says,
 * header not recognised, any header field different from what the repacker
 * writes for the header's own M, K, bits, format, group and nnz, or
 * codes_bytes < M*K), UNSUPPORTED (an HPTQ blob).
 */
int qgemv_unpack_host(const void* blob_host, size_t bytes, uint8_t* codes_out, size_t codes_bytes);

/*
 * Bind a plan to a blob already copied to device memory (packed_dev, bytes,
 * 256-byte aligned).  shape supplies M, K, bits, format, group_size and nnz;
 * its array pointers are ignored.  The blob's header is read back once
 * (synchronous device-to-host copy) and must match shape.  The caller keeps
 * the blob alive and unmodified until qgemv_destroy.  qgemv_create
 * allocates no device memory (see qgemv_run for the batch-8/16 workspace).
 * The plan belongs to the device current at this call.
 * Errors: INVALID_ARG, UNSUPPORTED, SIZE (bytes too small or header mismatch),
 * HIP.
 */
int qgemv_create(qgemv_handle* out, const qgemv_weights* shape, const void* packed_dev, size_t bytes);

/*
 * Enqueue y = dequant(W_dense) x + W_sparse x on `stream` (a hipStream_t; NULL
 * = the default stream).  x_dev: FP16 [batch][K] device memory, 16-byte
 * aligned, contiguous.  y_dev: fp32 [batch][M] device memory, 16-byte
 * aligned; every element is overwritten.  batch must be 1, 8 or 16.
 * Asynchronous: errors of the running kernel surface at the caller's next
 * synchronisation.
 * Workspace: with uniform codes at batch 8 or 16 the K dimension is split
 * across workgroups whose partial sums meet in a device workspace of the
 * plan (S * ceil(M/16) * 16 * 16 * 4 bytes of partials, S <= 8, plus 1 KiB
 * of counters).  The first such run of a plan allocates it (hipMalloc on the
 * plan's device, counters cleared in stream order) and must not be captured
 * into a graph; later runs, captured or not, reuse it.  Runs of one plan at
 * batch 8/16 that overlap in time (other streams) share it and race.
 * Errors: INVALID_ARG (null handle/pointer, misalignment, workspace first
 * needed under stream capture), UNSUPPORTED (batch), HIP (launch or
 * allocation failure).
 */
int qgemv_run(qgemv_handle h, const void* x_dev, float* y_dev, int32_t batch, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * product as qgemv_run, with the same arguments and result, that allocates
 * nothing.  Where qgemv_run would use the plan's workspace (uniform codes at
 * batch 8/16), this call uses instead a static device array of 16 MiB that
 * the library holds on each device it runs on until the process ends; its
 * address is looked up once per device.  Shapes needing more (1 KiB +
 * S * ceil(M/16) * 16 * batch * 4 bytes, S <= 8) are refused with
 * QGEMV_ERR_SCRATCH.  Every such call on one device shares that array: calls
 * that overlap in time (other streams, other threads, other plans) race.  The
 * array's counters are zero at load and every completed call leaves them as
 * it found them (a multiple of 8), so nothing needs clearing between calls.
 * Errors: as qgemv_run (no allocation failure), plus SCRATCH.
 */
int qgemv_run_noalloc(qgemv_handle h, const void* x_dev, float* y_dev, int32_t batch, void* stream);

/*
 * Enqueue a kernel that decodes the blob's codes back to canonical order, one
 * uint8 per weight, into codes_dev [M][K] (device memory).  Uses the same
 * unpacking as the product kernels; for bit-exact checks of the codes.
 * Errors: INVALID_ARG, HIP, UNSUPPORTED (HPTQ plans).
 */
int qgemv_debug_unpack(qgemv_handle h, uint8_t* codes_dev, void* stream);

/*
 * Measurement utility, not an operation of the method: enqueue one read of
 * src_dev[0 .. bytes) (device memory, 16-byte aligned; bytes a multiple of 16,
 * 1 .. 2^30) with 16-byte non-temporal loads, and write one uint32 per thread
 * to sink_dev (device memory, 4-byte aligned, sink_words >= 256 words; the
 * grid has min(1024, sink_words / 256) workgroups of 256 threads, T threads
 * in all).  sink_dev[t] is the XOR of the dwords of the 16-byte pieces t,
 * t + T, t + 2T, ... of src_dev, so the read can be checked.  Timing it gives
 * the streaming-read rate of the GPU, the ceiling the GEMV is compared with.
 * Errors: INVALID_ARG (null or misaligned pointer, bytes or sink_words out of
 * range), HIP (launch failure).
 */
int qgemv_read_probe(const void* src_dev, uint64_t bytes, uint32_t* sink_dev, int32_t sink_words, void* stream);

/* Release the plan and its workspace, if any (the plan's enqueued work must
 * have completed).  NULL is accepted. */
int qgemv_destroy(qgemv_handle h);

/* Static description of a status code; never NULL. */
const char* qgemv_error_string(int status);

/* hipError_t of the most recent QGEMV_ERR_HIP on the calling thread (0 if none). */
int qgemv_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
