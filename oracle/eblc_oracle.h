/*
 * eblc_oracle.h -- plain single-threaded CPU oracle of the error-bounded float32 codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls this
 * code.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may use it.
 * It shares no source with the GPU library: every constant, header offset and formula
 * below is written out again here, on purpose, from the stream definition.
 *
 * What it computes (sources: "Pipeline Specialization Internals" on the FZGPUModules
 * site, sections "Roles and strategies", "Forward declaration / Conventions",
 * "Inverse declaration", "Priming" and "The device policy contract"; the
 * "nvrtc_chunk_fusion.h File Reference" entries for launchNvrtcChunkFusedEncode and
 * launchGenericChunkFusion; the "DevitoComp provider interface" page):
 *
 *   1. bound resolution (absolute, or relative to the finite value range),
 *   2. linear quantization with step 2*eb (inv2eb = 1/(2*eb)), verified against the
 *      decoder's exact reconstruction, with escape of unrepresentable values,
 *   3. 1-D Lorenzo deltas that reset at every block start,
 *   4. zigzag,
 *   5. one bit width per 32-value segment,
 *   6. fixed-length bit packing of each segment,
 *   7. an outlier side list ordered by index,
 *   8. stream assembly (128-byte header + widths + payload + outlier indices + values),
 *   9. the exact inverse;
 * and the second, chunk-cooperative coder of the same page ("Chunk-cooperative path (brief)"):
 * the same quantizer, a first difference reset at every chunk, a bit-plane shuffle and zero-
 * word elimination (RZE) per chunk.
 *
 * Floating point: fp32, IEEE round-to-nearest-even, no FMA contraction (built with
 * -ffp-contract=off), denormals preserved.  The bound is resolved in fp64.
 *
 * Parity status: every function here is pinned by tests/test_oracle_*.py (closed forms,
 * brute force on tiny inputs, round-trip invariants and two hand-derived streams in
 * tests/golden/).
 */
#ifndef EBLC_ORACLE_H
#define EBLC_ORACLE_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Result codes of oracle_decompress (mirrors the library's meaning, values chosen here). */
#define ORACLE_OK 0
#define ORACLE_CORRUPT 4
#define ORACLE_CAPACITY 3

/* Step 1: resolve the bound.  rel != 0: eb = eps * (max - min) over finite x; else eb = eps.
 * Writes eb_f (fp32, rounded toward zero from the fp64 value), s = 2*eb_f, r = f32(1/s).
 * Returns 1 when the bound is usable (eb_f positive normal, s and r finite), else 0. */
int oracle_resolve_bound(const float *x, uint64_t n, int rel, double eps,
                         float *eb_f, float *s, float *r);

/* Step 2 for one value.  Returns 1 if the value escapes, else 0 with *q set. */
int oracle_quantize_one(float x, float eb_f, float s, float r, int T, int32_t *q);

/* Steps 2-5 over a whole array, exposing every intermediate for tests.
 * q[n], esc[n] (0/1), d[n], z[n]; widths[ceil(n/32)].  Escaped values have q = 0. */
void oracle_codes(const float *x, uint64_t n, float eb_f, float s, float r, int T, uint32_t B,
                  int32_t *q, uint8_t *esc, int32_t *d, uint32_t *z, uint8_t *widths);

/* Step 6: pack z (n values, padded with zeros to whole segments) at the given widths into
 * words[].  Returns the number of 32-bit words written (sum of widths). */
uint64_t oracle_pack(const uint32_t *z, uint64_t n, const uint8_t *widths, uint32_t *words);

/* Inverse of step 6 for one segment: value j of a segment of width w stored at words. */
uint32_t oracle_unpack_one(const uint32_t *words, uint32_t w, uint32_t j);

/* Size of the stream the oracle would write for these parameters, given sum of widths
 * and outlier count (closed form of the layout, the offset table included: one u32 for each
 * group of 8192 values after the first, padded to 16 bytes). */
uint64_t oracle_stream_bytes(uint64_t n, uint64_t sum_widths, uint64_t m);
uint64_t oracle_raw_bytes(uint64_t n);

/* Whole compressor.  dims[rank] slowest to fastest, n = product.  Writes the stream into out
 * (capacity cap) and returns its byte length; if cap is too small nothing is written and the
 * required length is returned in *required with return value 0. */
uint64_t oracle_compress(const float *x, int rank, const uint64_t *dims, int rel, double eps,
                         uint32_t B, int T, uint64_t side_max,
                         uint8_t *out, uint64_t cap, uint64_t *required);

/* Lorenzo centering: means[b] = floor((2 S + c) / (2 c)) for the c codes of block b summing to
 * S (the block's mean code rounded half up; escaped values count as 0). */
void oracle_block_means(const int32_t *q, uint64_t n, uint32_t B, int32_t *means);
uint64_t oracle_stream_bytes_centered(uint64_t n, uint32_t B, uint64_t sum_widths, uint64_t m);

/* oracle_compress with optional Lorenzo centering (center = 1): each block's first difference
 * is taken against the block's mean code, and the means follow the widths as one i32 per block
 * (header flags word = 1). */
uint64_t oracle_compress_ex(const float *x, int rank, const uint64_t *dims, int rel, double eps,
                            uint32_t B, int T, uint64_t side_max, int center,
                            uint8_t *out, uint64_t cap, uint64_t *required);

/* Chunk-cooperative coder steps (V codes per chunk, V a multiple of 32).  Bitshuffle: word
 * b * (V/32) + g of `words` holds bit b of codes 32g .. 32g+31 (code j at bit j).  RZE: out =
 * bitmap of the nonzero words (W/32 words), then those words in order; returns its length.
 * oracle_unrze returns 0, or -1 for an inconsistent input. */
void oracle_bitshuffle(const uint32_t *z, uint32_t V, uint32_t *words);
void oracle_unbitshuffle(const uint32_t *words, uint32_t V, uint32_t *z);
uint32_t oracle_rze(const uint32_t *words, uint32_t W, uint32_t *out);
int oracle_unrze(const uint32_t *in, uint32_t len, uint32_t W, uint32_t *words);
/* Size of a chunk-coder stream of n values in chunks of V (offset table included). */
uint64_t oracle_chunk_stream_bytes(uint64_t n, uint32_t V, uint64_t sum_words, uint64_t m);

/* Whole compressor with the chunk-cooperative coder: Quant -> Diff (first difference reset at
 * every chunk, zigzag-folded) -> Bitshuffle -> RZE over chunks of V = 1024, 2048 or 4096
 * values (4, 8 or 16 KiB of input).  Same bound, outlier and RAW rules as oracle_compress;
 * stream mode 2.  Same return convention as oracle_compress. */
uint64_t oracle_compress_chunked(const float *x, int rank, const uint64_t *dims, int rel, double eps,
                                 uint32_t V, int T, uint64_t side_max,
                                 uint8_t *out, uint64_t cap, uint64_t *required);

/* Whole decompressor (either coder).  Reads len bytes; writes n_out floats.  Returns ORACLE_OK,
 * ORACLE_CORRUPT (header or sections inconsistent) or ORACLE_CAPACITY (n_out too small). */
int oracle_decompress(const uint8_t *in, uint64_t len, float *out, uint64_t n_out);

/* Number of elements a stream decodes to (0 if the header is not a valid one). */
uint64_t oracle_stream_elements(const uint8_t *in, uint64_t len);

#ifdef __cplusplus
}
#endif
#endif
