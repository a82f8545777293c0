/*
 * eblc_oracle.cpp -- plain single-threaded CPU oracle of the error-bounded float32 codec.
 *
 * TEST INFRASTRUCTURE ONLY (see eblc_oracle.h).  Slow on purpose: every step is its own
 * loop over the whole array, in the order the method is described, with no blocking,
 * fusion or reordering.  Built with g++ -O2 -ffp-contract=off -fno-fast-math.
 */
#include "eblc_oracle.h"

#include <cmath>
#include <cstring>
#include <vector>

namespace {

/* ---- stream layout constants, written out independently of the GPU library ---------- */
const uint32_t kMagic = 0x434C4245u; /* "EBLC" little-endian */
const uint16_t kVersion = 2;
const uint16_t kHeaderBytes = 128;
const uint8_t kModeLossy = 0;
const uint8_t kModeRaw = 1;
const uint8_t kModeChunk = 2; /* the chunk-cooperative coder: Quant -> Diff -> Bitshuffle -> RZE */
const uint32_t kSeg = 32; /* values per bitpack segment */

uint64_t align16(uint64_t v) { return (v + 15u) / 16u * 16u; }

/* The offset table, an index of this codec's own container (the pages' concatenated output
 * records each buffer's size ahead of its data, "Architecture", Execution Flow, Compression,
 * so that a file describes itself): the payload words that precede each group of
 * kGroupValues values, one u32 per group after the first, in a section of its own right after
 * the size section (widths or chunk word counts), padded to 16 bytes.  A decoder takes any
 * group's payload offset from it. */
const uint64_t kGroupValues = 8192;

uint64_t table_bytes(uint64_t n) {
    uint64_t groups = (n + kGroupValues - 1) / kGroupValues;
    return groups > 1 ? align16(4 * (groups - 1)) : 0;
}

/* The table's entries from the payload words of each coded unit (a segment of the bitpack
 * coder, a chunk of the chunk coder), units_per_group units to a group: entry g - 1 is the
 * sum over the units before group g. */
std::vector<uint32_t> table_entries(const std::vector<uint64_t> &unit_words, uint64_t units_per_group) {
    std::vector<uint32_t> t;
    uint64_t acc = 0;
    for (uint64_t u = 0; u < unit_words.size(); ++u) {
        if (u > 0 && u % units_per_group == 0) t.push_back((uint32_t)acc);
        acc += unit_words[u];
    }
    return t;
}

void put_u8(uint8_t *p, uint64_t off, uint8_t v) { p[off] = v; }
void put_u16(uint8_t *p, uint64_t off, uint16_t v) { std::memcpy(p + off, &v, 2); }
void put_u32(uint8_t *p, uint64_t off, uint32_t v) { std::memcpy(p + off, &v, 4); }
void put_u64(uint8_t *p, uint64_t off, uint64_t v) { std::memcpy(p + off, &v, 8); }
void put_f32(uint8_t *p, uint64_t off, float v) { std::memcpy(p + off, &v, 4); }
uint8_t get_u8(const uint8_t *p, uint64_t off) { return p[off]; }
uint16_t get_u16(const uint8_t *p, uint64_t off) { uint16_t v; std::memcpy(&v, p + off, 2); return v; }
uint32_t get_u32(const uint8_t *p, uint64_t off) { uint32_t v; std::memcpy(&v, p + off, 4); return v; }
uint64_t get_u64(const uint8_t *p, uint64_t off) { uint64_t v; std::memcpy(&v, p + off, 8); return v; }
float get_f32(const uint8_t *p, uint64_t off) { float v; std::memcpy(&v, p + off, 4); return v; }
uint32_t f32_bits(float v) { uint32_t b; std::memcpy(&b, &v, 4); return b; }
float bits_f32(uint32_t b) { float v; std::memcpy(&v, &b, 4); return v; }

/* The decoder's reconstruction of a code: convert the int32 code to fp32 (round to nearest
 * even), then multiply by the step s = 2*eb in fp32.  "Inverse declaration" on the
 * Pipeline Specialization Internals page: the dequant step is 2*abs_eb and the harness
 * multiplies the code by it. */
float dequant(int32_t q, float s) {
    float qf = (float)q;
    float y = qf * s;
    return y;
}

/* Acceptance test for a candidate code: the fp32 difference must be within eb, and the
 * guard |x| >= |y|/2 keeps that fp32 difference exact (Sterbenz), so the test is exact. */
bool accept(float x, float y, float eb_f) {
    float diff = x - y;
    bool within = std::fabs(diff) <= eb_f;
    float half_y = 0.5f * std::fabs(y);
    bool guard = std::fabs(x) >= half_y;
    return within && guard;
}

} // namespace

extern "C" {

/* Step 1: bound resolution.  "Priming" on the Pipeline Specialization Internals page: the
 * quantizer runs a value-range scan to resolve its bound before the fused kernel runs.
 * The DevitoComp provider interface page ("Configuring the error tolerance") makes the
 * user's error a non-negative relative tolerance; the relative bound is eps times the
 * range of the finite values.  The fp64 bound is rounded toward zero to fp32 so that the
 * fp32 bound never exceeds the requested one. */
int oracle_resolve_bound(const float *x, uint64_t n, int rel, double eps,
                         float *eb_f_out, float *s_out, float *r_out) {
    double eb_d;
    if (rel) {
        bool any = false;
        float mn = 0.0f, mx = 0.0f;
        for (uint64_t i = 0; i < n; ++i) {
            float v = x[i];
            if (!std::isfinite(v)) continue;
            if (!any) { mn = v; mx = v; any = true; continue; }
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
        if (!any) {
            *eb_f_out = 0.0f; *s_out = 0.0f; *r_out = 0.0f;
            return 0;
        }
        double range = (double)mx - (double)mn;
        eb_d = eps * range;
    } else {
        eb_d = eps;
    }
    float eb_f = (float)eb_d;
    if (std::isfinite(eb_f) && (double)eb_f > eb_d) {
        eb_f = std::nextafter(eb_f, 0.0f);
    }
    float s = 2.0f * eb_f;
    double inv = 1.0 / (double)s;
    float r = (float)inv;
    int valid = std::isnormal(eb_f) && eb_f > 0.0f && std::isfinite(s) && std::isfinite(r);
    if (!valid) {
        *eb_f_out = 0.0f; *s_out = 0.0f; *r_out = 0.0f;
        return 0;
    }
    *eb_f_out = eb_f; *s_out = s; *r_out = r;
    return 1;
}

/* Step 2: linear quantization of one value ("Roles and strategies": the linear quantizer is
 * Elementwise; "Conventions": it multiplies by inv2eb = 1/(2 eb) inside the predictor).
 * The code is round-to-nearest-even of x*inv2eb, then checked against the decoder's exact
 * reconstruction; if that misses the bound, the one neighbouring code toward x is tried; if
 * both miss, or the value is not finite, or the code needs 2^T or more in magnitude, the
 * value escapes to the outlier list. */
int oracle_quantize_one(float x, float eb_f, float s, float r, int T, int32_t *q_out) {
    float p = x * r;
    float q0f = std::nearbyint(p);
    /* non-finite x or product, or a code of 2^30 or more in magnitude */
    if (!(std::fabs(q0f) < 1073741824.0f)) return 1;
    int32_t q = (int32_t)q0f;
    float y = dequant(q, s);
    if (!accept(x, y, eb_f)) {
        int32_t qn = (x > y) ? q + 1 : q - 1;
        float yn = dequant(qn, s);
        if (!accept(x, yn, eb_f)) return 1;
        q = qn;
    }
    int64_t mag = q < 0 ? -(int64_t)q : (int64_t)q;
    if (mag >= ((int64_t)1 << T)) return 1;
    *q_out = q;
    return 0;
}

/* Steps 2-5 over the array.  Lorenzo ("Roles and strategies": 1-D Lorenzo is RegionLocal
 * with a region reset; "Inverse declaration": its undelta is a plain first difference
 * inverse): d_i = q_i - q_{i-1}, except at a block start (i mod B == 0) where the
 * prediction is 0 and d_i = q_i.  Zigzag (named as the interior transform in "The device
 * policy contract"): z = (d << 1) ^ (d >> 31).  Width (AdaptiveBitpack is the SegmentCodec
 * with one metadata byte per segment): the bit length of the OR of the segment's 32 z
 * values, the tail past n counting as zeros. */
void oracle_codes(const float *x, uint64_t n, float eb_f, float s, float r, int T, uint32_t B,
                  int32_t *q, uint8_t *esc, int32_t *d, uint32_t *z, uint8_t *widths) {
    /* quantize every value; an escaped value is coded as 0 */
    for (uint64_t i = 0; i < n; ++i) {
        int32_t qi = 0;
        int e = oracle_quantize_one(x[i], eb_f, s, r, T, &qi);
        esc[i] = (uint8_t)e;
        q[i] = e ? 0 : qi;
    }
    /* Lorenzo deltas with a reset at every block start */
    for (uint64_t i = 0; i < n; ++i) {
        if (i % B == 0) d[i] = q[i];
        else d[i] = q[i] - q[i - 1];
    }
    /* zigzag */
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t du = (uint32_t)d[i];
        uint32_t sign = (uint32_t)(d[i] >> 31);
        z[i] = (du << 1) ^ sign;
    }
    /* one width per 32-value segment */
    uint64_t nseg = (n + kSeg - 1) / kSeg;
    for (uint64_t k = 0; k < nseg; ++k) {
        uint32_t acc = 0;
        for (uint64_t j = 0; j < kSeg; ++j) {
            uint64_t i = k * kSeg + j;
            if (i < n) acc |= z[i];
        }
        uint32_t w = 0;
        while (w < 32 && (acc >> w) != 0) ++w;
        widths[k] = (uint8_t)w;
    }
}

/* Step 6: fixed-length packing.  Segment k holds w_k little-endian 32-bit words; value j of
 * the segment occupies bits [j*w, j*w + w) of the segment's bit string, bit t living in
 * word t/32 at position t%32.  Segments follow each other with no gap. */
uint64_t oracle_pack(const uint32_t *z, uint64_t n, const uint8_t *widths, uint32_t *words) {
    uint64_t nseg = (n + kSeg - 1) / kSeg;
    uint64_t base = 0;
    for (uint64_t k = 0; k < nseg; ++k) {
        uint32_t w = widths[k];
        for (uint32_t t = 0; t < w; ++t) words[base + t] = 0;
        for (uint32_t j = 0; j < kSeg; ++j) {
            uint64_t i = k * kSeg + j;
            uint32_t v = (i < n) ? z[i] : 0u;
            for (uint32_t b = 0; b < w; ++b) {
                uint32_t bit = (v >> b) & 1u;
                uint64_t t = (uint64_t)j * w + b;
                words[base + t / 32] |= bit << (t % 32);
            }
        }
        base += w;
    }
    return base;
}

uint32_t oracle_unpack_one(const uint32_t *words, uint32_t w, uint32_t j) {
    uint32_t v = 0;
    for (uint32_t b = 0; b < w; ++b) {
        uint64_t t = (uint64_t)j * w + b;
        uint32_t bit = (words[t / 32] >> (t % 32)) & 1u;
        v |= bit << b;
    }
    return v;
}

uint64_t oracle_stream_bytes(uint64_t n, uint64_t sum_widths, uint64_t m) {
    uint64_t nseg = (n + kSeg - 1) / kSeg;
    uint64_t payload_off = kHeaderBytes + align16(nseg) + table_bytes(n);
    uint64_t oidx_off = payload_off + align16(4 * sum_widths);
    uint64_t oval_off = oidx_off + align16(4 * m);
    return oval_off + align16(4 * m);
}

uint64_t oracle_raw_bytes(uint64_t n) { return kHeaderBytes + align16(4 * n); }

/* floor(a / b) for b > 0 (C++ division truncates toward zero). */
static int64_t floor_div(int64_t a, int64_t b) {
    int64_t qd = a / b;
    if ((a % b) != 0 && a < 0) qd -= 1;
    return qd;
}

/* Lorenzo centering ("Pipeline Specialization Internals", Inverse declaration, where the
 * fused inverse excludes centeringActive(): a centered predictor's inverse is not the plain
 * first-difference one).  Reading: the mean code of each block -- the exact mean of the
 * block's codes (escaped values count as code 0) rounded half up, mu = floor((2 S + c) /
 * (2 c)) for c codes summing to S -- is subtracted before the first difference, so the block's
 * first code is predicted by mu instead of 0 and the other differences are unchanged.  The
 * means are kept in a means stream (one i32 per block) and added back after the prefix sum. */
void oracle_block_means(const int32_t *q, uint64_t n, uint32_t B, int32_t *means) {
    uint64_t nblocks = (n + B - 1) / B;
    for (uint64_t b = 0; b < nblocks; ++b) {
        int64_t S = 0;
        int64_t c = 0;
        for (uint64_t i = b * B; i < n && i < (b + 1) * B; ++i) {
            S += q[i];
            c += 1;
        }
        means[b] = (int32_t)floor_div(2 * S + c, 2 * c);
    }
}

/* Stream size of the bitpack coder with the optional means section (4 bytes per block). */
uint64_t oracle_stream_bytes_centered(uint64_t n, uint32_t B, uint64_t sum_widths, uint64_t m) {
    uint64_t nblocks = (n + B - 1) / B;
    return oracle_stream_bytes(n, sum_widths, m) + align16(4 * nblocks);
}

/* Chunk coder, "Bitshuffle" ("Pipeline Specialization Internals", Chunk-cooperative path: a
 * Transform between Diff and the coder).  The chunk's V codes (V a multiple of 32) form
 * G = V / 32 groups of 32; word b * G + g of the output holds bit b of every code of group g,
 * code j of the group at bit j.  So the output is the chunk's bit planes, plane 0 first, and
 * planes above the widest code are zero words. */
void oracle_bitshuffle(const uint32_t *z, uint32_t V, uint32_t *words) {
    uint32_t G = V / 32;
    for (uint32_t k = 0; k < V; ++k) words[k] = 0;
    for (uint32_t g = 0; g < G; ++g) {
        for (uint32_t j = 0; j < 32; ++j) {
            uint32_t v = z[32 * g + j];
            for (uint32_t b = 0; b < 32; ++b) {
                uint32_t bit = (v >> b) & 1u;
                words[b * G + g] |= bit << j;
            }
        }
    }
}

void oracle_unbitshuffle(const uint32_t *words, uint32_t V, uint32_t *z) {
    uint32_t G = V / 32;
    for (uint32_t g = 0; g < G; ++g) {
        for (uint32_t j = 0; j < 32; ++j) {
            uint32_t v = 0;
            for (uint32_t b = 0; b < 32; ++b) {
                uint32_t bit = (words[b * G + g] >> j) & 1u;
                v |= bit << b;
            }
            z[32 * g + j] = v;
        }
    }
}

/* Chunk coder, "RZE" (the SegmentCodec of the chunk chain): zero words are dropped.  Output:
 * a bitmap of W / 32 words (bit k, in word k / 32 at position k % 32, is set when word k is
 * nonzero), then the nonzero words in order.  Returns the output length in words. */
uint32_t oracle_rze(const uint32_t *words, uint32_t W, uint32_t *out) {
    uint32_t nbm = W / 32;
    for (uint32_t i = 0; i < nbm; ++i) out[i] = 0;
    uint32_t k = nbm;
    for (uint32_t i = 0; i < W; ++i) {
        if (words[i] != 0) {
            out[i / 32] |= 1u << (i % 32);
            out[k] = words[i];
            ++k;
        }
    }
    return k;
}

/* Inverse of RZE for one chunk of W words from len input words.  Returns 0, or -1 when the
 * input is inconsistent (length not bitmap + popcount, or a zero word under a set bit). */
int oracle_unrze(const uint32_t *in, uint32_t len, uint32_t W, uint32_t *words) {
    uint32_t nbm = W / 32;
    if (len < nbm) return -1;
    uint32_t k = nbm;
    for (uint32_t i = 0; i < W; ++i) {
        uint32_t bit = (in[i / 32] >> (i % 32)) & 1u;
        if (bit) {
            if (k >= len) return -1;
            words[i] = in[k];
            if (words[i] == 0) return -1;
            ++k;
        } else {
            words[i] = 0;
        }
    }
    if (k != len) return -1;
    return 0;
}

/* Size of a chunk-coder stream of n values in chunks of V from its total chunk words and
 * outlier count. */
uint64_t oracle_chunk_stream_bytes(uint64_t n, uint32_t V, uint64_t sum_words, uint64_t m) {
    uint64_t nchunks = (n + V - 1) / V;
    uint64_t payload_off = kHeaderBytes + align16(4 * nchunks) + table_bytes(n);
    uint64_t oidx_off = payload_off + align16(4 * sum_words);
    uint64_t oval_off = oidx_off + align16(4 * m);
    return oval_off + align16(4 * m);
}

/* The 128-byte header: magic, version, layout of the sections (all offsets from the start). */
static void write_header(uint8_t *out, uint8_t mode, int rank, const uint64_t *dims, uint64_t n,
                         uint8_t log2_seg, int T, uint32_t B, float eb_f, float s, float r,
                         uint64_t m, uint64_t payload_bytes, uint64_t payload_off, uint64_t oidx_off,
                         uint64_t oval_off, uint64_t total) {
    put_u32(out, 0, kMagic);
    put_u16(out, 4, kVersion);
    put_u16(out, 6, kHeaderBytes);
    put_u8(out, 8, mode);
    put_u8(out, 9, (uint8_t)rank);
    put_u8(out, 10, log2_seg);
    put_u8(out, 11, (uint8_t)T);
    put_u32(out, 12, B);
    for (int a = 0; a < 4; ++a) put_u64(out, 16 + 8 * a, a < rank ? dims[a] : 0);
    put_u64(out, 48, n);
    put_f32(out, 56, eb_f);
    put_f32(out, 60, s);
    put_f32(out, 64, r);
    put_u32(out, 68, 0);
    put_u64(out, 72, m);
    put_u64(out, 80, payload_bytes);
    put_u64(out, 88, kHeaderBytes);
    put_u64(out, 96, payload_off);
    put_u64(out, 104, oidx_off);
    put_u64(out, 112, oval_off);
    put_u64(out, 120, total);
}

/* Steps 1-8: the whole compressor, in order.  The outlier list holds (u32 index, raw fp32
 * bits) pairs in ascending index order (the "nvrtc_chunk_fusion.h File Reference" names the
 * side list as u32 indices plus float values; the order is fixed here by index).  The stream
 * falls back to a raw copy when the bound is unusable, when more values escape than the
 * side list may hold, or when the coded stream would be larger than the raw one (the
 * DevitoComp dummy provider reports the raw size as the maximum compressed size).  With
 * `center`, the block means are taken from the codes (oracle_block_means), every block's first
 * difference is taken against its mean, the widths follow from those codes, and the means
 * stream sits between the widths and the payload; header word 68 (flags) is 1. */
uint64_t oracle_compress_ex(const float *x, int rank, const uint64_t *dims, int rel, double eps,
                            uint32_t B, int T, uint64_t side_max, int center,
                            uint8_t *out, uint64_t cap, uint64_t *required) {
    uint64_t n = 1;
    for (int a = 0; a < rank; ++a) n *= dims[a];
    uint64_t nseg = (n + kSeg - 1) / kSeg;
    uint64_t nblocks = (n + B - 1) / B;

    float eb_f = 0.0f, s = 0.0f, r = 0.0f;
    int valid = oracle_resolve_bound(x, n, rel, eps, &eb_f, &s, &r);

    std::vector<int32_t> q, d, means;
    std::vector<uint8_t> esc, widths;
    std::vector<uint32_t> z, words;
    std::vector<uint32_t> oidx, oval;
    uint64_t sum_w = 0;
    bool raw = !valid;
    if (!raw) {
        q.resize(n); d.resize(n); esc.resize(n); z.resize(n); widths.resize(nseg);
        oracle_codes(x, n, eb_f, s, r, T, B, q.data(), esc.data(), d.data(), z.data(), widths.data());
        if (center) {
            /* centering: the first difference of each block against the block's mean code */
            means.resize(nblocks);
            oracle_block_means(q.data(), n, B, means.data());
            for (uint64_t b = 0; b < nblocks; ++b) {
                uint64_t i = b * B;
                d[i] = (int32_t)((uint32_t)q[i] - (uint32_t)means[b]);
                z[i] = ((uint32_t)d[i] << 1) ^ (uint32_t)(d[i] >> 31);
            }
            for (uint64_t k = 0; k < nseg; ++k) {
                uint32_t acc = 0;
                for (uint64_t j = 0; j < kSeg; ++j) {
                    uint64_t i = k * kSeg + j;
                    if (i < n) acc |= z[i];
                }
                uint32_t w = 0;
                while (w < 32 && (acc >> w) != 0) ++w;
                widths[k] = (uint8_t)w;
            }
        }
        for (uint64_t k = 0; k < nseg; ++k) sum_w += widths[k];
        words.assign(sum_w, 0u);
        oracle_pack(z.data(), n, widths.data(), words.data());
        for (uint64_t i = 0; i < n; ++i) {
            if (esc[i]) { oidx.push_back((uint32_t)i); oval.push_back(f32_bits(x[i])); }
        }
        uint64_t coded = center ? oracle_stream_bytes_centered(n, B, sum_w, oidx.size())
                                : oracle_stream_bytes(n, sum_w, oidx.size());
        if (oidx.size() > side_max) raw = true;
        else if (coded > oracle_raw_bytes(n)) raw = true;
    }

    uint64_t m = raw ? 0 : oidx.size();
    uint64_t msec = (!raw && center) ? align16(4 * nblocks) : 0;
    uint64_t total = raw ? oracle_raw_bytes(n) : oracle_stream_bytes(n, sum_w, m) + msec;
    if (required) *required = total;
    if (total > cap) return 0;

    std::memset(out, 0, total);
    if (raw) {
        uint64_t end = oracle_raw_bytes(n);
        write_header(out, kModeRaw, rank, dims, n, 5, T, B, eb_f, s, r, 0, 4 * n, kHeaderBytes, end, end, end);
        std::memcpy(out + kHeaderBytes, x, 4 * n);
        return total;
    }
    uint64_t table_off = kHeaderBytes + align16(nseg);
    uint64_t means_off = table_off + table_bytes(n);
    uint64_t payload_off = means_off + msec;
    uint64_t oidx_off = payload_off + align16(4 * sum_w);
    uint64_t oval_off = oidx_off + align16(4 * m);
    write_header(out, kModeLossy, rank, dims, n, 5, T, B, eb_f, s, r, m, 4 * sum_w, payload_off,
                 oidx_off, oval_off, total);
    if (center) put_u32(out, 68, 1u);
    for (uint64_t k = 0; k < nseg; ++k) out[kHeaderBytes + k] = widths[k];
    if (center)
        for (uint64_t b = 0; b < nblocks; ++b) put_u32(out, means_off + 4 * b, (uint32_t)means[b]);
    for (uint64_t t = 0; t < sum_w; ++t) put_u32(out, payload_off + 4 * t, words[t]);
    for (uint64_t k = 0; k < m; ++k) {
        put_u32(out, oidx_off + 4 * k, oidx[k]);
        put_u32(out, oval_off + 4 * k, oval[k]);
    }
    /* the offset table: segments of 32 values, kGroupValues / 32 to a group */
    std::vector<uint64_t> seg_words(widths.begin(), widths.end());
    std::vector<uint32_t> table = table_entries(seg_words, kGroupValues / kSeg);
    for (uint64_t g = 0; g < table.size(); ++g) put_u32(out, table_off + 4 * g, table[g]);
    return total;
}

uint64_t oracle_compress(const float *x, int rank, const uint64_t *dims, int rel, double eps,
                         uint32_t B, int T, uint64_t side_max,
                         uint8_t *out, uint64_t cap, uint64_t *required) {
    return oracle_compress_ex(x, rank, dims, rel, eps, B, T, side_max, 0, out, cap, required);
}

/* The chunk-cooperative coder, whole compressor ("Pipeline Specialization Internals",
 * Chunk-cooperative path: Quant -> Diff -> Bitshuffle -> RZE over chunks of 4096, 8192 or
 * 16384 input bytes, i.e. V = 1024, 2048 or 4096 float32 values).  Quant is the same verified
 * linear quantizer with the same outlier escape; Diff is the first difference inside the chunk
 * (0 predicts the chunk's first code), folded by the zigzag map so small magnitudes have empty
 * high bits; Bitshuffle and RZE as above.  The last chunk is padded with zero codes to V.
 * Stream: header (mode 2, log2_seg = log2 V, B = V), one u32 word count per chunk where the
 * widths of the bitpack coder go, the chunks' RZE outputs back to back, then the outliers.
 * RAW fallbacks as for the bitpack coder. */
uint64_t oracle_compress_chunked(const float *x, int rank, const uint64_t *dims, int rel, double eps,
                                 uint32_t V, int T, uint64_t side_max,
                                 uint8_t *out, uint64_t cap, uint64_t *required) {
    uint64_t n = 1;
    for (int a = 0; a < rank; ++a) n *= dims[a];
    uint64_t nchunks = (n + V - 1) / V;
    uint8_t log2v = 0;
    while ((1u << log2v) < V) ++log2v;

    float eb_f = 0.0f, s = 0.0f, r = 0.0f;
    int valid = oracle_resolve_bound(x, n, rel, eps, &eb_f, &s, &r);

    std::vector<int32_t> q, d;
    std::vector<uint8_t> esc, widths;
    std::vector<uint32_t> z, payload, sizes;
    std::vector<uint32_t> oidx, oval;
    bool raw = !valid;
    if (!raw) {
        q.resize(n); d.resize(n); esc.resize(n); z.resize(n); widths.resize((n + 31) / 32);
        /* Quant and Diff: the Lorenzo deltas with a reset every V values, zigzag-folded */
        oracle_codes(x, n, eb_f, s, r, T, V, q.data(), esc.data(), d.data(), z.data(), widths.data());
        std::vector<uint32_t> zc(V), words(V), cout(V + V / 32);
        for (uint64_t c = 0; c < nchunks; ++c) {
            for (uint32_t i = 0; i < V; ++i) {
                uint64_t gi = c * V + i;
                zc[i] = gi < n ? z[gi] : 0u;
            }
            oracle_bitshuffle(zc.data(), V, words.data());
            uint32_t len = oracle_rze(words.data(), V, cout.data());
            sizes.push_back(len);
            for (uint32_t i = 0; i < len; ++i) payload.push_back(cout[i]);
        }
        for (uint64_t i = 0; i < n; ++i) {
            if (esc[i]) { oidx.push_back((uint32_t)i); oval.push_back(f32_bits(x[i])); }
        }
        if (oidx.size() > side_max) raw = true;
        else if (oracle_chunk_stream_bytes(n, V, payload.size(), oidx.size()) > oracle_raw_bytes(n)) raw = true;
    }

    uint64_t total = raw ? oracle_raw_bytes(n) : oracle_chunk_stream_bytes(n, V, payload.size(), oidx.size());
    if (required) *required = total;
    if (total > cap) return 0;
    std::memset(out, 0, total);
    if (raw) {
        uint64_t end = oracle_raw_bytes(n);
        write_header(out, kModeRaw, rank, dims, n, log2v, T, V, eb_f, s, r, 0, 4 * n, kHeaderBytes, end, end, end);
        std::memcpy(out + kHeaderBytes, x, 4 * n);
        return total;
    }
    uint64_t m = oidx.size();
    uint64_t table_off = kHeaderBytes + align16(4 * nchunks);
    uint64_t payload_off = table_off + table_bytes(n);
    uint64_t oidx_off = payload_off + align16(4 * payload.size());
    uint64_t oval_off = oidx_off + align16(4 * m);
    write_header(out, kModeChunk, rank, dims, n, log2v, T, V, eb_f, s, r, m, 4 * payload.size(),
                 payload_off, oidx_off, oval_off, total);
    for (uint64_t c = 0; c < nchunks; ++c) put_u32(out, kHeaderBytes + 4 * c, sizes[c]);
    for (uint64_t t = 0; t < payload.size(); ++t) put_u32(out, payload_off + 4 * t, payload[t]);
    for (uint64_t k = 0; k < m; ++k) {
        put_u32(out, oidx_off + 4 * k, oidx[k]);
        put_u32(out, oval_off + 4 * k, oval[k]);
    }
    /* the offset table: chunks of V values, kGroupValues / V to a group */
    std::vector<uint64_t> chunk_words(sizes.begin(), sizes.end());
    std::vector<uint32_t> table = table_entries(chunk_words, kGroupValues / V);
    for (uint64_t g = 0; g < table.size(); ++g) put_u32(out, table_off + 4 * g, table[g]);
    return total;
}

/* Header checks shared by oracle_decompress and oracle_stream_elements.  Returns n, or 0
 * when the header is not one this codec writes. */
static uint64_t check_header(const uint8_t *in, uint64_t len) {
    if (len < kHeaderBytes) return 0;
    if (get_u32(in, 0) != kMagic) return 0;
    if (get_u16(in, 4) != kVersion || get_u16(in, 6) != kHeaderBytes) return 0;
    uint8_t mode = get_u8(in, 8), rank = get_u8(in, 9), log2_seg = get_u8(in, 10), T = get_u8(in, 11);
    uint32_t B = get_u32(in, 12);
    if (mode != kModeLossy && mode != kModeRaw && mode != kModeChunk) return 0;
    if (rank < 1 || rank > 4 || T < 1 || T > 30) return 0;
    bool chunk_params = log2_seg >= 10 && log2_seg <= 12 && B == (1u << log2_seg);
    if (mode == kModeChunk && !chunk_params) return 0;
    if (mode == kModeLossy && log2_seg != 5) return 0;
    if (mode == kModeRaw && log2_seg != 5 && !chunk_params) return 0;
    if (B < 32 || B % 32 != 0 || B > (1u << 20)) return 0;
    uint64_t n = 1;
    for (int a = 0; a < 4; ++a) {
        uint64_t da = get_u64(in, 16 + 8 * a);
        if (a < rank) {
            if (da == 0 || da >= (1ull << 32)) return 0;
            n *= da;
            if (n >= (1ull << 32)) return 0;
        } else if (da != 0) {
            return 0;
        }
    }
    if (get_u64(in, 48) != n) return 0;
    uint32_t flags = get_u32(in, 68);
    if (flags > 1 || (flags == 1 && mode != kModeLossy) || get_u64(in, 88) != kHeaderBytes) return 0;
    uint64_t m = get_u64(in, 72), pb = get_u64(in, 80);
    uint64_t po = get_u64(in, 96), oi = get_u64(in, 104), ov = get_u64(in, 112), tot = get_u64(in, 120);
    if (mode == kModeRaw) {
        uint64_t end = kHeaderBytes + align16(4 * n);
        if (m != 0 || pb != 4 * n || po != kHeaderBytes || oi != end || ov != end || tot != end) return 0;
    } else {
        float eb_f = get_f32(in, 56), s = get_f32(in, 60);
        if (!(std::isnormal(eb_f) && eb_f > 0.0f && std::isfinite(s) && s == 2.0f * eb_f)) return 0;
        if (m > n || pb % 4 != 0) return 0;
        if (mode == kModeLossy) {
            uint64_t nseg = (n + kSeg - 1) / kSeg;
            uint64_t msec = flags ? align16(4 * ((n + B - 1) / B)) : 0;
            if (pb > 4ull * 32 * nseg || po != kHeaderBytes + align16(nseg) + table_bytes(n) + msec) return 0;
        } else {
            uint64_t nchunks = (n + B - 1) / B;
            if (pb > 4ull * nchunks * (B + B / 32) || po != kHeaderBytes + align16(4 * nchunks) + table_bytes(n))
                return 0;
        }
        if (oi != po + align16(pb) || ov != oi + align16(4 * m) || tot != ov + align16(4 * m)) return 0;
    }
    if (tot > len) return 0;
    return n;
}

uint64_t oracle_stream_elements(const uint8_t *in, uint64_t len) { return check_header(in, len); }

/* The bitpack coder's inverse of steps 4-6: per segment read its width, unpack its 32 values
 * and undo the zigzag into d.  Returns false when the widths are inconsistent. */
static bool widths_to_deltas(const uint8_t *in, uint64_t n, uint64_t pb, uint64_t po, int32_t *d) {
    uint64_t nseg = (n + kSeg - 1) / kSeg;

    /* widths, and the payload size they imply */
    std::vector<uint8_t> widths(nseg);
    uint64_t sum_w = 0;
    for (uint64_t k = 0; k < nseg; ++k) {
        widths[k] = in[kHeaderBytes + k];
        if (widths[k] > 32) return false;
        sum_w += widths[k];
    }
    if (4 * sum_w != pb) return false;

    /* unpack + unzigzag */
    std::vector<uint32_t> words(sum_w);
    for (uint64_t t = 0; t < sum_w; ++t) words[t] = get_u32(in, po + 4 * t);
    uint64_t base = 0;
    for (uint64_t k = 0; k < nseg; ++k) {
        for (uint32_t j = 0; j < kSeg; ++j) {
            uint64_t i = k * kSeg + j;
            if (i >= n) break;
            uint32_t zv = oracle_unpack_one(words.data() + base, widths[k], j);
            d[i] = (int32_t)((zv >> 1) ^ (0u - (zv & 1u)));
        }
        base += widths[k];
    }
    return true;
}

/* Step 9: the inverse.  Per segment: read its width, unpack its 32 values, undo the zigzag
 * d = (z >> 1) ^ -(z & 1), then the code is the running sum of d from the block start
 * (undelta of the first-difference predictor), and the value is f32(f32(q) * s)
 * ("Inverse declaration": dequant step 2*eb).  Finally every outlier is written back with
 * its exact bits. */
int oracle_decompress(const uint8_t *in, uint64_t len, float *out, uint64_t n_out) {
    uint64_t n = check_header(in, len);
    if (n == 0) return ORACLE_CORRUPT;
    if (n_out < n) return ORACLE_CAPACITY;
    uint8_t mode = get_u8(in, 8);
    if (mode == kModeRaw) {
        std::memcpy(out, in + kHeaderBytes, 4 * n);
        return ORACLE_OK;
    }
    uint32_t B = get_u32(in, 12);
    float s = get_f32(in, 60);
    uint64_t m = get_u64(in, 72), pb = get_u64(in, 80);
    uint64_t po = get_u64(in, 96), oi = get_u64(in, 104), ov = get_u64(in, 112);
    std::vector<int32_t> d(n);
    if (mode == kModeChunk) {
        /* chunk coder: per chunk, undo RZE and Bitshuffle, then the zigzag */
        uint32_t V = B;
        uint64_t nchunks = (n + V - 1) / V;
        uint64_t sum = 0;
        for (uint64_t c = 0; c < nchunks; ++c) sum += get_u32(in, kHeaderBytes + 4 * c);
        if (4 * sum != pb) return ORACLE_CORRUPT;
        std::vector<uint32_t> cin(V + V / 32), words(V), zc(V);
        uint64_t base = 0;
        for (uint64_t c = 0; c < nchunks; ++c) {
            uint32_t len = get_u32(in, kHeaderBytes + 4 * c);
            if (len < V / 32 || len > V + V / 32) return ORACLE_CORRUPT;
            for (uint32_t t = 0; t < len; ++t) cin[t] = get_u32(in, po + 4 * (base + t));
            if (oracle_unrze(cin.data(), len, V, words.data()) != 0) return ORACLE_CORRUPT;
            oracle_unbitshuffle(words.data(), V, zc.data());
            for (uint32_t i = 0; i < V; ++i) {
                uint64_t gi = c * V + i;
                if (gi >= n) break;
                uint32_t zv = zc[i];
                d[gi] = (int32_t)((zv >> 1) ^ (0u - (zv & 1u)));
            }
            base += len;
        }
    } else {
        if (!widths_to_deltas(in, n, pb, po, d.data())) return ORACLE_CORRUPT;
    }
    /* the offset table must index the payload the sizes section describes */
    {
        std::vector<uint64_t> unit_words;
        uint64_t units_per_group;
        if (mode == kModeChunk) {
            for (uint64_t c = 0; c < (n + B - 1) / B; ++c) unit_words.push_back(get_u32(in, kHeaderBytes + 4 * c));
            units_per_group = kGroupValues / B;
        } else {
            for (uint64_t k = 0; k < (n + kSeg - 1) / kSeg; ++k) unit_words.push_back(in[kHeaderBytes + k]);
            units_per_group = kGroupValues / kSeg;
        }
        std::vector<uint32_t> table = table_entries(unit_words, units_per_group);
        uint64_t table_off = kHeaderBytes + (mode == kModeChunk ? align16(4 * ((n + B - 1) / B))
                                                                : align16((n + kSeg - 1) / kSeg));
        for (uint64_t g = 0; g < table.size(); ++g)
            if (get_u32(in, table_off + 4 * g) != table[g]) return ORACLE_CORRUPT;
    }
    /* undelta: running sum from each block start (from the block's mean when the stream is
     * centered, else from 0), then dequantize */
    uint32_t flags = get_u32(in, 68);
    uint64_t means_off = kHeaderBytes + align16((n + kSeg - 1) / kSeg) + table_bytes(n);
    int32_t qprev = 0;
    for (uint64_t i = 0; i < n; ++i) {
        int32_t qi;
        if (i % B == 0) {
            int32_t mu = flags ? (int32_t)get_u32(in, means_off + 4 * (i / B)) : 0;
            qi = (int32_t)((uint32_t)mu + (uint32_t)d[i]);
        } else {
            qi = (int32_t)((uint32_t)qprev + (uint32_t)d[i]);
        }
        out[i] = dequant(qi, s);
        qprev = qi;
    }
    /* outliers: strictly ascending indices below n */
    for (uint64_t k = 0; k < m; ++k) {
        uint32_t idx = get_u32(in, oi + 4 * k);
        if (idx >= n) return ORACLE_CORRUPT;
        if (k > 0 && idx <= get_u32(in, oi + 4 * (k - 1))) return ORACLE_CORRUPT;
        out[idx] = bits_f32(get_u32(in, ov + 4 * k));
    }
    return ORACLE_OK;
}

} /* extern "C" */
