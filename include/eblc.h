/*
 * eblc.h -- C ABI of libeblc.so, an error-bounded lossy compressor for float32 fields on
 * AMD Instinct MI355X (gfx950).
 *
 * The interface is shaped like the provider ABI described on the "DevitoComp provider
 * interface" page (devitocodes.com, DevitoPRO extension docs): a plan is created once with
 * the tensor's dims/strides and an options string carrying the error tolerance; the plan
 * reports limits (maximum compressed size, payload alignment, sidecar size); compress and
 * decompress run on a caller-supplied stream.  The names are this library's own.
 *
 * Method (one fixed chain; "Pipeline Specialization Internals", FZGPUModules site):
 *   linear quantization with step 2*eb (inv2eb = 1/(2*eb)) checked against the exact
 *   reconstruction -> 1-D Lorenzo deltas reset at every block -> zigzag -> one bit width per
 *   32-value segment and fixed-length bit packing -> outliers (values that cannot be coded)
 *   escape to a side list of (u32 index, f32 bits) ordered by index -> an exclusive scan of
 *   the variable segment sizes and compaction into one self-describing stream.  Decompress is
 *   the exact inverse.
 *
 * A second coder, selected per plan (coder=chunk), follows the page's chunk-cooperative chain
 * Quant -> Diff -> Bitshuffle -> RZE over chunks of 4, 8 or 16 KiB: the same quantizer and
 * escapes, the first difference inside each chunk, zigzag, the chunk's 32 bit planes (word
 * b*G+g holds bit b of the 32 codes of group g, G = V/32), and zero-word elimination (a bitmap
 * of the V plane words, then the nonzero ones).
 *
 * Stream (little-endian, every section 16-byte aligned, pad bytes zero):
 *   [0,128)            header (magic "EBLC", version 2, mode, rank, dims, n, eb, step,
 *                      outlier count, section offsets, total length)
 *   [128, ...)         bitpack coder (mode 0): one width byte per 32-value segment
 *                      (nseg = ceil(n/32)); chunk coder (mode 2): one u32 word count per chunk
 *   offset table       one u32 per group of 8192 values after the first: the payload words
 *                      before that group (ceil(n/8192) - 1 entries), so that a decoder finds
 *                      any group's payload without a scan of the sizes
 *   block means        centered streams only (center=1): one i32 per block
 *   payload            bitpack: sum(widths) u32 words; chunk: each chunk's bitmap and nonzero
 *                      plane words, chunk after chunk (the last chunk padded with zero codes)
 *   outlier indices    m x u32, strictly ascending
 *   outlier values     m x u32 (raw float32 bits)
 * A RAW stream (bound unusable or 0, more outliers than side_max, or a coded stream that
 * would be larger than the input) holds the header followed by the input bytes.
 *
 * Threading: a plan is used by one host thread at a time; distinct plans may run
 * concurrently on distinct streams.  All device pointers must come from hipMalloc (or
 * torch) on the plan's device and be 16-byte aligned, except the field pointer of a padded
 * plan (`in` of compress, `out` of decompress), which needs 4-byte alignment only.  The field
 * pointer addresses the plan's layout (contiguous, or padded through its strides).
 */
#ifndef EBLC_H
#define EBLC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ABI version; a header and a library of different versions must not be mixed ("Provider
 * layout": a private header implements the same ABI version as the public one). */
#define EBLC_ABI_VERSION 1

typedef struct eblc_plan eblc_plan_t; /* opaque; owned by the library */

/* Status codes.  UNSUPPORTED is the provider interface's answer for an execution kind or a
 * tensor layout the provider does not handle ("Provider layout": providers may support any
 * subset of the execution kinds). */
typedef enum {
    EBLC_OK = 0,
    EBLC_UNSUPPORTED = 1,      /* execution kind, dtype, rank or strides not handled */
    EBLC_INVALID_ARGUMENT = 2, /* NULL/misaligned pointer, bad option, n out of range */
    EBLC_CAPACITY = 3,         /* out_capacity smaller than the stream; required size returned */
    EBLC_CORRUPT_STREAM = 4,   /* stream header or sections inconsistent with the plan */
    EBLC_DEVICE_ERROR = 5,     /* a HIP runtime call failed */
    EBLC_OUT_OF_MEMORY = 6,    /* workspace allocation failed at plan creation */
    EBLC_TOO_LARGE = 7         /* eblc_compress_noalloc: field larger than its static scratch */
} eblc_status;

/* Where the pointers live ("Provider layout": HOST uses host pointers and a thread count and
 * no stream; CUDA/HIP use device-accessible pointers and an optional native stream).  This
 * provider implements HIP only; HOST and CUDA return EBLC_UNSUPPORTED. */
typedef enum {
    EBLC_EXECUTION_HOST = 0,
    EBLC_EXECUTION_CUDA = 1,
    EBLC_EXECUTION_HIP = 2
} eblc_execution_kind;

typedef struct {
    eblc_execution_kind kind;
    int device;  /* HIP device ordinal the plan's workspace lives on */
    int threads; /* ignored for HIP */
} eblc_execution_t;

/* Limits ("Provider layout": the provider reports its payload alignment, a nonzero power of
 * two; "Dummy provider": the maximum compressed size is reported by the provider). */
typedef struct {
    size_t max_compressed_bytes; /* 128 + align16(4 n): a RAW stream, the largest possible */
    size_t payload_alignment;    /* 16 */
    size_t sidecar_bytes;        /* 0: the stream is self-describing */
    size_t sidecar_alignment;    /* 1 */
} eblc_limits_t;

typedef enum { EBLC_FLOAT32 = 0 } eblc_dtype;

/* Result record of an asynchronous compress, written by the device when the call's work
 * completes on its stream. */
typedef struct {
    uint64_t compressed_bytes; /* stream length; with status CAPACITY, the required capacity */
    uint32_t status;           /* EBLC_OK or EBLC_CAPACITY */
    uint32_t reserved;
} eblc_result_t;

/* Returns EBLC_ABI_VERSION of the library. */
int eblc_abi_version(void);

/* Create a plan.
 *   exec     execution descriptor; kind must be EBLC_EXECUTION_HIP (else UNSUPPORTED).
 *   dtype    EBLC_FLOAT32 (else UNSUPPORTED).
 *   rank     1..4; dims[rank] > 0, slowest to fastest ("Provider layout": dimensions and
 *            strides in slowest-to-fastest order, strides in elements).  n = prod(dims)
 *            must be below 2^32 (outlier indices are u32).
 *   strides  NULL (contiguous), or row-major strides in elements with padding allowed: the
 *            fastest stride is 1 and each outer stride is at least the extent times the stride
 *            of the dimension below it (a solver's halo-padded array).  compress reads, and
 *            decompress writes, the dims' values through these strides and touches no padding
 *            element; 128-bit access is kept when the fastest extent and every outer stride are
 *            multiples of 4.  Other layouts (transposed, overlapping, zero or negative strides)
 *            are UNSUPPORTED.
 *   options  NULL or "" -> relative error 1e-4 (the default bound named in "Priming");
 *            a bare decimal -> relative error (what DevitoPRO passes, "Provider layout");
 *            else ';'-separated key=value pairs:
 *              rel=<eps> | abs=<eb>   exactly one; finite, >= 0; 0 means lossless (RAW)
 *              block=<B>              Lorenzo reset period: a multiple of 32 from 32 to 1024, or
 *                                     2048 ("Pipeline Specialization Internals", Forward
 *                                     declaration: the block size is a multiple of 32); a
 *                                     block that is not a power of two may start anywhere on a
 *                                     32-value boundary; default 256
 *              outlier_log2=<T>       codes with |q| >= 2^T escape; 1..30; default 30
 *              side_max=<m>           largest outlier list; 0..n; default min(n, 2^23)
 *              coder=bitpack|chunk    bitpack (default) or the chunk coder
 *              chunk_bytes=<b>        chunk coder only: 4096, 8192 (default) or 16384 input
 *                                     bytes per chunk; the chunk is also the reset period of
 *                                     the difference, so block= is refused with coder=chunk
 *              center=0|1             bitpack coder only: predict each block's first code by
 *                                     the block's mean code (kept in a means section) instead
 *                                     of 0; default 0
 *              lanes=<k>              1..8, default 1: fields a batch call codes per kernel
 *                                     launch, each in a workspace of its own (the workspace
 *                                     grows k-fold); the streams are identical for every k
 *            Unknown keys, repeated keys, NaN or negative values -> INVALID_ARGUMENT.
 *   plan_out receives the plan.  The plan allocates its whole workspace here and nothing
 *            per call: about 4.4 n bytes per lane (the encoder's payload slots 4 n, its
 *            escape staging n/4, escape masks n/8 and size staging n/32), plus 4 n / B for
 *            the block means and small arrays.
 * INVALID_ARGUMENT also when the field's largest payload would reach 2^32 words (the scans
 * count in 32 bits): 32 words per 32-value segment for the bitpack coder, so n <= 2^32 - 32;
 * for the chunk coder ceil(n / V) (V + V / 32) < 2^32.  DEVICE_ERROR when no HIP device can be
 * queried.
 * The relative error is eps * (max - min) over the finite input values, resolved on the
 * device at every compress call ("Priming": the quantizer's value-range scan). */
eblc_status eblc_plan_create(const eblc_execution_t *exec, eblc_dtype dtype, int rank,
                             const int64_t *dims, const int64_t *strides, const char *options,
                             eblc_plan_t **plan_out);

/* Fill *out with the plan's limits ("DevitoComp provider interface", Provider layout: the
 * provider reports its limits, among them the payload alignment, in a limits record; Dummy
 * provider: a maximum compressed size, there the raw size).  INVALID_ARGUMENT on NULL. */
eblc_status eblc_plan_limits(const eblc_plan_t *plan, eblc_limits_t *out);

/* The largest stream a compress of this plan writes: 128 + align16(4 n), a RAW stream ("DevitoComp
 * provider interface", Dummy provider: the provider reports a maximum compressed size, the raw
 * size for a copy).  0 for a NULL plan. */
size_t eblc_max_compressed_bytes(const eblc_plan_t *plan);

/* The alignment the stream's start needs: 16 ("DevitoComp provider interface", Provider layout:
 * the required compressed-payload alignment, a nonzero power of two).  0 for a NULL plan. */
size_t eblc_payload_alignment(const eblc_plan_t *plan);

/* Compress n floats at device pointer `in` into device buffer `out` of out_capacity bytes,
 * enqueued on `stream` (a hipStream_t; NULL = default stream).  The call waits for its own
 * work once, to return *compressed_bytes (like the fused chunk encoder that syncs before
 * returning the archive length, "nvrtc_chunk_fusion.h File Reference",
 * launchGenericChunkFusion).  Returns OK with *compressed_bytes set, or CAPACITY with
 * *compressed_bytes = the required size (then `out` holds no valid stream; nothing is
 * written at or past out_capacity).  `in` and `out` must not overlap.  sidecar must be NULL.
 * Output is deterministic: the same input and plan give the same bytes. */
eblc_status eblc_compress(eblc_plan_t *plan, const float *in, void *out, size_t out_capacity,
                          size_t *compressed_bytes, void *sidecar, void *stream);

/* Asynchronous compress: enqueues the same work as eblc_compress on `stream` and returns at
 * once, without waiting ("Provider layout": device work may remain queued on the supplied
 * stream).  When the work completes, the device writes the call's eblc_result_t at `result`,
 * which must be 8-byte aligned device memory or pinned host memory (hipHostMalloc) that
 * stays valid until then.  The plan's workspace is shared by its calls, so calls on one plan
 * must be ordered on one stream.  Errors detectable on the host are returned at once
 * (INVALID_ARGUMENT, DEVICE_ERROR); capacity is reported in the record. */
eblc_status eblc_compress_async(eblc_plan_t *plan, const float *in, void *out, size_t out_capacity,
                                eblc_result_t *result, void *stream);

/* Compress without allocating anything, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The same
 * work as eblc_compress_async on a plan created with exec, rank, dims, strides and options, with
 * the same arguments, checks, stream and result record, but no plan: the call's workspace is a
 * static device array of 24 MiB that the library holds on every device it runs this call on
 * until the process ends, and the option string is parsed without heap allocation.  Fields of
 * up to 2^22 values (every coder and option) fit it; a larger one returns EBLC_TOO_LARGE before
 * anything is enqueued.  The option lanes is refused (INVALID_ARGUMENT).  The device's address
 * of the array is looked up at the first call on that device.  All calls on one device share the
 * array: calls that overlap on one device (on different streams, or from different host threads
 * without ordering) race and may corrupt each other's streams; calls ordered on one stream are
 * safe.  Nothing in the array needs clearing between calls: every value a call reads there is
 * written earlier in the same call (the previous call's payload size only picks a store
 * policy).  Decompress the stream with any plan of the same shape and coder. */
eblc_status eblc_compress_noalloc(const eblc_execution_t *exec, int rank, const int64_t *dims,
                                  const int64_t *strides, const char *options, const float *in, void *out,
                                  size_t out_capacity, eblc_result_t *result, void *stream);

/* Batched asynchronous compress: count fields of the plan's shape, in[k] -> out[k] with
 * capacity out_capacity[k], result record k at results + k, enqueued on `stream` with no host
 * wait (the snapshot-batch case of a solver saving many time steps).  The fields are coded in
 * groups of up to `lanes` (a plan option), one kernel launch per stage for each group, each
 * field of a group in a workspace of its own, so the short single-workgroup stages of a group's
 * fields run side by side and the launches are `lanes` times fewer.  The three pointer arrays
 * are host arrays of device pointers; `results` as for eblc_compress_async.  All arguments are
 * checked before anything is enqueued. */
eblc_status eblc_compress_batch(eblc_plan_t *plan, int count, const float *const *in, void *const *out,
                                const size_t *out_capacity, eblc_result_t *results, void *stream);

/* Decompress a stream of compressed_bytes at device pointer `in` into n floats at `out`,
 * enqueued on `stream`; returns without waiting ("Provider layout": device work may remain
 * queued on the supplied stream).  compressed_bytes may be the stream's length or any larger
 * count of readable bytes up to max_compressed_bytes: the stream's own length is read from its
 * header on the device and must not exceed it, so a stream from eblc_compress_async can be
 * decompressed without the host ever reading its length.  The host checks 128 + (size of the
 * width or word-count section) + (size of the offset table) <= compressed_bytes <=
 * max_compressed_bytes (else CORRUPT_STREAM at once).  A plan decodes RAW streams and coded
 * streams of its own coder (and, for the chunk coder, of its own chunk size); any other stream
 * is CORRUPT_STREAM.  Header or section problems found on the device (wrong magic/version/
 * dims/n/offsets, widths above 32, chunk word counts outside [V/32, V + V/32] or unequal to the
 * bitmap's count, an offset-table entry that does not index the payload the sizes describe,
 * outlier indices not strictly ascending below n) set a sticky CORRUPT_STREAM that
 * eblc_plan_status returns; the contents of `out` are then unspecified.  sidecar must be
 * NULL. */
eblc_status eblc_decompress(eblc_plan_t *plan, const void *in, size_t compressed_bytes,
                            const void *sidecar, float *out, void *stream);

/* Batched decompress: count streams of the plan's shape, in[k] (compressed_bytes[k] readable
 * bytes, as for eblc_decompress) -> out[k], enqueued on `stream` without waiting, in groups of
 * `lanes` streams per launch as eblc_compress_batch does.  The three arrays are host arrays.
 * All arguments are checked before anything is enqueued; device-side problems set the plan's
 * sticky CORRUPT_STREAM. */
eblc_status eblc_decompress_batch(eblc_plan_t *plan, int count, const void *const *in,
                                  const size_t *compressed_bytes, float *const *out, void *stream);

/* Wait for `stream`, then return and clear the plan's sticky device error (OK if none).  Device
 * work may stay queued when a call returns ("DevitoComp provider interface", Provider layout), so
 * problems only the device finds (a corrupt stream) are reported by this later call.
 * INVALID_ARGUMENT on NULL; DEVICE_ERROR when the wait or the read of the record fails. */
eblc_status eblc_plan_status(eblc_plan_t *plan, void *stream);

/* Wait for the device, then free the plan and its workspace.  Like the pool buffers of the
 * "Architecture" page (FZGPUModules site, buffer ownership: valid until the pipeline is
 * destroyed), the workspace lives until this call; streams already written stay the caller's.
 * NULL is a no-op. */
void eblc_plan_destroy(eblc_plan_t *plan);

/* Static string naming a status: the eblc_status codes above, UNSUPPORTED among them for the
 * execution kinds and layouts this provider does not take ("DevitoComp provider interface",
 * Provider layout); "unknown status" for any other value. */
const char *eblc_status_string(eblc_status s);

/* ---- measurement hooks (not part of the provider shape) --------------------------------
 * eblc_plan_set_profiling(plan, k, kernels, every) with 0 < k <= 8192 and every >= 1 waits for
 * the device, then binds a HIP event pair to each of the plan's next k timed kernel launches
 * (the kernel dispatch itself records them, on the stream the launch runs on); k = 0 turns
 * recording off.  kernels is NULL or "" (every kernel), or a comma-separated list of the names
 * to time (range, encode, scan, compact, decode, patch); only the
 * every-th, 2·every-th, ... compress and decompress launch sequences (counted apart; a batch
 * call makes one per group of fields) are timed.  A timed dispatch still costs the stream a few
 * microseconds, so naming few kernels and sampling keep the rest of the work undisturbed.
 * eblc_plan_kernel_times waits for the recorded events and writes, for each kernel name in
 * order of its first launch (at most max_kernels of them), the static name, the mean duration
 * in milliseconds and the number of launches recorded; then it clears the records (recording
 * goes on while k launches have not been recorded in all).  It returns how many kernel names
 * were recorded, or -1 when recording is off or on error. */
eblc_status eblc_plan_set_profiling(eblc_plan_t *plan, int max_launches, const char *kernels, int every);
int eblc_plan_kernel_times(eblc_plan_t *plan, const char **names, float *ms, int *launches,
                           int max_kernels);

#ifdef __cplusplus
}
#endif
#endif /* EBLC_H */
