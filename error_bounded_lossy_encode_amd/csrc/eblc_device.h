/*
 * eblc_device.h -- device primitives shared by the gfx950 kernels of libeblc.so: wave-level
 * DPP scans and moves, non-temporal global access, the caller's memory layout, and the
 * quantizer ("Pipeline Specialization Internals", FZGPUModules site: linear quantization with
 * step 2*eb, inv2eb = 1/(2*eb), the zigzag Transform).  Every function is inline and has
 * internal linkage in each kernel source that includes it.
 */
#ifndef EBLC_DEVICE_H
#define EBLC_DEVICE_H

#include "eblc_internal.h"

#include <float.h>

namespace eblc {
namespace {

/* ---- wave-level primitives ---------------------------------------------------------------- */

constexpr int kDppQuadXor1 = 0xB1;     /* quad_perm [1,0,3,2] */
constexpr int kDppQuadXor2 = 0x4E;     /* quad_perm [2,3,0,1] */
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf, bool BOUND_CTRL = false>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, BOUND_CTRL);
}

/* Inclusive prefix sum over the 64 lanes (row-local Hillis-Steele, then row broadcasts). */
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += dpp<kDppRowShr1, 0xf, true>(0, v);
    v += dpp<kDppRowShr2, 0xf, true>(0, v);
    v += dpp<kDppRowShr4, 0xf, true>(0, v);
    v += dpp<kDppRowShr8, 0xf, true>(0, v);
    v += dpp<kDppRowBcast15, 0xa>(0, v);
    v += dpp<kDppRowBcast31, 0xc>(0, v);
    return v;
}

/* Inclusive prefix sum restricted to aligned segments of seglen lanes (8, 16, 32 or 64);
 * dist = lane index within its segment. */
__device__ __forceinline__ uint32_t wave_seg_scan(uint32_t v, uint32_t dist, uint32_t seglen) {
    uint32_t t;
    t = dpp<kDppRowShr1, 0xf, true>(0, v);
    v += (dist >= 1) ? t : 0u;
    t = dpp<kDppRowShr2, 0xf, true>(0, v);
    v += (dist >= 2) ? t : 0u;
    t = dpp<kDppRowShr4, 0xf, true>(0, v);
    v += (dist >= 4) ? t : 0u;
    t = dpp<kDppRowShr8, 0xf, true>(0, v);
    v += (dist >= 8) ? t : 0u;
    if (seglen >= 32) v += dpp<kDppRowBcast15, 0xa>(0, v);
    if (seglen >= 64) v += dpp<kDppRowBcast31, 0xc>(0, v);
    return v;
}

__device__ __forceinline__ uint32_t readlane(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

/* Orders this wave's LDS traffic across lanes (compiler and hardware). */
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void lds_or(uint32_t *p, uint32_t v) {
    __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

__device__ __forceinline__ uint64_t align16(uint64_t v) { return (v + 15u) & ~(uint64_t)15u; }

/* Non-temporal 128-bit global access, for data streamed exactly once (the field on compress,
 * the reconstruction on decompress): the lines bypass cache allocation. */
typedef float v4f32 __attribute__((ext_vector_type(4)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld_nt(const float4 *p) {
    const v4f32 t = __builtin_nontemporal_load(reinterpret_cast<const v4f32 *>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
    const v4u32 t = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void st_nt(float4 *p, const float4 &v) {
    const v4f32 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<v4f32 *>(p));
}

__device__ __forceinline__ void st_nt(uint4 *p, const uint4 &v) {
    const v4u32 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<v4u32 *>(p));
}

/* ---- the caller's memory layout ------------------------------------------------------------ */

__device__ __forceinline__ uint32_t div_m(uint32_t v, uint64_t m) {
    return m == 0 ? v : (uint32_t)__umul64hi((uint64_t)v, m);
}

/* Element offset of flattened value i (i < 2^32) in the caller's array; *col receives i's
 * position in its row. */
template <bool STRIDED>
__device__ __forceinline__ uint64_t elem_off(const Layout &lo, uint64_t i, uint32_t *col_out = nullptr) {
    if (!STRIDED) return i;
    const uint32_t ii = (uint32_t)i;
    const uint32_t row = div_m(ii, lo.mL);
    const uint32_t col = ii - row * lo.L;
    if (col_out != nullptr) *col_out = col;
    if (lo.rank == 2) return col + (uint64_t)row * lo.s1;
    const uint32_t r1 = div_m(row, lo.m1);
    const uint32_t c1 = row - r1 * lo.o1;
    if (lo.rank == 3) return col + (uint64_t)c1 * lo.s1 + (uint64_t)r1 * lo.s2;
    const uint32_t r2 = div_m(r1, lo.m2);
    const uint32_t c2 = r1 - r2 * lo.o2;
    return col + (uint64_t)c1 * lo.s1 + (uint64_t)c2 * lo.s2 + (uint64_t)r2 * lo.s3;
}

/* 128-bit non-temporal access at a 4-byte aligned address (gfx950 executes dword-aligned
 * multi-dword global accesses). */
typedef float v4f32u __attribute__((ext_vector_type(4), aligned(4)));

__device__ __forceinline__ float4 ld_nt_u(const float *p) {
    const v4f32u t = __builtin_nontemporal_load(reinterpret_cast<const v4f32u *>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void st_nt_u(float *p, const float4 &v) {
    const v4f32u t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<v4f32u *>(p));
}

/* Values i .. i+3 (i a multiple of 4, all below n), streamed once: one 128-bit access when they
 * are contiguous in memory (16-byte aligned with a vectorisable layout, else whenever they sit
 * in one row), one access per value when a row boundary splits them. */
template <bool STRIDED>
__device__ __forceinline__ float4 load4(const float *x, const Layout &lo, uint64_t i) {
    if (!STRIDED) return ld_nt(reinterpret_cast<const float4 *>(x + i));
    uint32_t col;
    const uint64_t off = elem_off<true>(lo, i, &col);
    if (lo.vec) return ld_nt(reinterpret_cast<const float4 *>(x + off));
    if (col + 3 < lo.L) return ld_nt_u(x + off);
    return make_float4(x[off], x[elem_off<true>(lo, i + 1)], x[elem_off<true>(lo, i + 2)],
                       x[elem_off<true>(lo, i + 3)]);
}

template <bool STRIDED>
__device__ __forceinline__ void store4(float *y, const Layout &lo, uint64_t i, const float4 &v) {
    if (!STRIDED) {
        st_nt(reinterpret_cast<float4 *>(y + i), v);
        return;
    }
    uint32_t col;
    const uint64_t off = elem_off<true>(lo, i, &col);
    if (lo.vec) {
        st_nt(reinterpret_cast<float4 *>(y + off), v);
    } else if (col + 3 < lo.L) {
        st_nt_u(y + off, v);
    } else {
        y[off] = v.x;
        y[elem_off<true>(lo, i + 1)] = v.y;
        y[elem_off<true>(lo, i + 2)] = v.z;
        y[elem_off<true>(lo, i + 3)] = v.w;
    }
}

/* ---- quantizer ------------------------------------------------------------------------------ */

struct QParams {
    float eb, s, r, tlim; /* tlim = 2^T */
    uint32_t T;
};

/* A code is accepted when its fp32 reconstruction is within eb of x; the second clause
 * (|x| >= |y|/2) makes the fp32 difference exact, so the test is exact. */
__device__ __forceinline__ bool accept(float x, float y, float eb) {
    const float diff = x - y;
    const float half_y = 0.5f * fabsf(y);
    return (fabsf(diff) <= eb) && (fabsf(x) >= half_y);
}

/* Full rule for a value that missed the fast test: escape if not finite or the rounded code is
 * 2^30 or more in magnitude; else keep the rounded code if accepted, else its neighbour toward
 * x if accepted, else escape; finally escape codes of 2^T or more in magnitude. */
__device__ __forceinline__ int32_t quantize_slow(float x, float q0f, QParams qp, uint32_t *esc) {
    if (!(fabsf(q0f) < 1073741824.0f)) {
        *esc = 1;
        return 0;
    }
    int32_t q = (int32_t)q0f;
    const float y = q0f * qp.s;
    if (!accept(x, y, qp.eb)) {
        const int32_t qn = (x > y) ? q + 1 : q - 1;
        const float yn = (float)qn * qp.s;
        if (!accept(x, yn, qp.eb)) {
            *esc = 1;
            return 0;
        }
        q = qn;
    }
    const uint32_t mag = q < 0 ? (uint32_t)(-q) : (uint32_t)q;
    if (mag >= (1u << qp.T)) {
        *esc = 1;
        return 0;
    }
    *esc = 0;
    return q;
}

__device__ __forceinline__ uint32_t zigzag(int32_t d) {
    return ((uint32_t)d << 1) ^ (uint32_t)(d >> 31);
}

__device__ __forceinline__ int32_t unzigzag(uint32_t z) {
    return (int32_t)((z >> 1) ^ (0u - (z & 1u)));
}

/* Sum over the wave of v (every lane gets it). */
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return readlane(wave_incl_scan(v), 63); }

/* Exclusive prefix of group g from the scanned prefixes of the super-groups of kSuperGroups
 * groups (spre) and the sums of the groups before g in its super-group (gsum), by one wave: lane
 * l loads the sum of group (g rounded down to a super-group) + l when that group comes before g,
 * and the wave adds them.  The loads do not depend on each other, so they go out with the
 * caller's.  (Scalar loads of the same 64 sums were slower.) */
__device__ __forceinline__ uint32_t group_prefix(const uint32_t *spre, const uint32_t *gsum, uint32_t g) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t g0 = g & ~(uint32_t)(kSuperGroups - 1);
    const uint32_t v = g0 + lane < g ? gsum[g0 + lane] : 0u;
    return spre[g / kSuperGroups] + wave_sum(v);
}

/* ---- the stream header, read by each decoding workgroup ---------------------------------------- */

__device__ __forceinline__ uint64_t ld64(const uint32_t *h, int i) {
    return (uint64_t)h[i] | ((uint64_t)h[i + 1] << 32);
}

/* One load for the wave: lane l < 32 takes header word l, and lanes 32 and 33 take the
 * offset-table entries a decoding workgroup of table group g needs (entries g - 1 and g, clamped
 * into the table; a field of one group has no table and they load nothing).  The host refuses a
 * stream shorter than its header, size section and offset table, so every word lies inside the
 * caller's bytes before anything is checked. */
__device__ __forceinline__ uint32_t load_header_lanes(const uint8_t *in, const PlanArgs &pa, uint32_t g) {
    const uint32_t lane = threadIdx.x & 63;
    uint64_t idx = lane;
    if (lane >= 32) {
        const uint32_t e = lane == 32 ? (g > 0 ? g - 1 : 0u) : (g + 1 < pa.ngroups ? g : pa.ngroups - 2);
        idx = (kHeaderBytes + pa.wsec) / 4 + e;
    }
    const bool on = lane < 32 || (lane < 34 && pa.ngroups > 1);
    return on ? reinterpret_cast<const uint32_t *>(in)[idx] : 0u;
}

__device__ __forceinline__ uint64_t readlane64(uint32_t v, int lane) {
    return (uint64_t)readlane(v, lane) | ((uint64_t)readlane(v, lane + 1) << 32);
}

/* The plan's header template for lane l < 32 (DevInfo::hdr_want / hdr_mask), loaded with the
 * header. */
__device__ __forceinline__ uint2 load_header_template(const DevInfo *info) {
    const uint32_t l = threadIdx.x & 31;
    return make_uint2(info->hdr_want[l], info->hdr_mask[l]);
}

/* The 128-byte header (lanes 0-31 of hv, from load_header_lanes) checked against the plan:
 * magic, format version, coder and its parameters (a plan decodes coded streams of its own coder
 * and chunk size, and every RAW stream), rank, dims, n, the bound, and a layout of sections --
 * sizes, offset table, block means, payload, outlier indices and values -- that ends inside the
 * in_bytes the caller passed.  The words the plan fixes are compared lane by lane with the
 * plan's template (tmpl, from load_header_template), the offsets with the layout the other
 * fields give, in one ballot.  One wave per call makes this check, in the outlier-patch kernel,
 * and reports a failure (the decoders, which would carry its registers into their tile loops,
 * only bound their reads); it takes the plan's fields it needs as values (n, the coder's V, the
 * size section's bytes, the table groups and the largest payload). */
__device__ __forceinline__ bool header_ok(uint32_t hv, uint2 tmpl, uint64_t in_bytes, uint64_t n, uint32_t V,
                                          uint64_t wsec, uint32_t ngroups, uint64_t max_pw) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t w2 = readlane(hv, 2), B = readlane(hv, 3), flags = readlane(hv, 17);
    const float eb_f = __uint_as_float(readlane(hv, 14)), s = __uint_as_float(readlane(hv, 15));
    const uint64_t m = readlane64(hv, 18), pb = readlane64(hv, 20), total = readlane64(hv, 30);
    const uint32_t mode = w2 & 0xff, log2seg = (w2 >> 16) & 0xff, T = w2 >> 24;
    bool ok = T >= 1 && T <= 30 && flags <= 1 && (flags == 0 || mode == 0);
    const bool bitpack_params = log2seg == 5 && ((B >= 32 && B <= 1024 && B % 32 == 0) || B == 2048);
    const bool chunk_params = log2seg >= 10 && log2seg <= 12 && B == (1u << (log2seg & 31));
    const bool raw = mode == 1;
    uint64_t po, oi, ov, end;
    if (raw) {
        /* the header, then the input bytes */
        ok = ok && (bitpack_params || chunk_params) && m == 0 && pb == 4 * n;
        po = kHeaderBytes;
        oi = ov = end = kHeaderBytes + align16(4 * n);
    } else {
        /* sizes, offset table, block means (centered), payload, outlier indices and values; the
         * payload holds at most every word the coder may write */
        ok = ok && (V == 0 ? mode == 0 && bitpack_params : mode == 2 && chunk_params && B == V);
        ok = ok && eb_f >= FLT_MIN && eb_f <= FLT_MAX && fabsf(s) <= FLT_MAX && s == 2.0f * eb_f;
        ok = ok && m <= n && (pb & 3) == 0 && pb / 4 <= max_pw;
        /* a centered stream's means: one per block of its B (n < 2^32: a 32-bit division) */
        uint64_t msec = 0;
        if (flags != 0 && B != 0) {
            const uint32_t n32 = (uint32_t)n;
            msec = align16(4ull * (n32 / B + (n32 % B != 0 ? 1u : 0u)));
        }
        po = kHeaderBytes + wsec + table_bytes(ngroups) + msec;
        oi = po + align16(pb);
        ov = oi + align16(4 * m);
        end = ov + align16(4 * m);
    }
    ok = ok && total == end && total <= in_bytes;
    /* lanes 24-29: the offsets of the payload, outlier indices and values */
    const uint64_t off = lane < 26 ? po : lane < 28 ? oi : ov;
    const uint32_t off32 = (lane & 1) ? (uint32_t)(off >> 32) : (uint32_t)off;
    const bool bad = lane < 32 && ((hv & tmpl.y) != tmpl.x || (lane >= 24 && lane < 30 && hv != off32));
    return ok && __ballot(bad) == 0;
}

/* The header fields a decoding wave works from, read from hv without the full check: each
 * wave bounds every read it bases on them by the caller's bytes, and rejects (without a report)
 * a mode, block or flags word no stream holds, so a stream whose header fails the full check --
 * made once per call, by one wave of the outlier patch (header_ok) -- can only leave `out`
 * unspecified. */
struct StreamView {
    bool sane;          /* mode 0-2, flags 0-1, B a multiple of 32 from 32 to 4096 */
    uint32_t mode, flags, B;
    float s;
    uint64_t pw, po;
};

__device__ __forceinline__ StreamView view_header(uint32_t hv) {
    StreamView V;
    V.mode = readlane(hv, 2) & 0xff;
    V.B = readlane(hv, 3);
    V.flags = readlane(hv, 17);
    V.s = __uint_as_float(readlane(hv, 15));
    V.pw = readlane64(hv, 20) / 4;
    V.po = readlane64(hv, 24);
    V.sane = V.mode <= 2 && V.flags <= 1 && V.B >= 32 && V.B <= 4096 && V.B % 32 == 0;
    return V;
}

/* Payload offset (in words) of table group g and of the group after it, from the entries
 * load_header_lanes placed in lanes 32 and 33 of hv: group 0 starts at 0, and the group after
 * the last ends at the payload's end, pw. */
__device__ __forceinline__ void table_range(uint32_t hv, uint32_t g, uint32_t ngroups, uint64_t pw,
                                            uint64_t &t0, uint64_t &t1) {
    t0 = g > 0 ? readlane(hv, 32) : 0u;
    t1 = g + 1 < ngroups ? (uint64_t)readlane(hv, 33) : pw;
}

/* ---- the fields of a launch ------------------------------------------------------------------ */

/* Entry f of a kernel-argument array, by selects on the wave-uniform f: indexing the array
 * directly with a value known only at run time would copy the argument to scratch memory. */
template <typename T>
__device__ __forceinline__ T pick(const T (&a)[kMaxFields], uint32_t f) {
    T v = a[0];
#pragma unroll
    for (int k = 1; k < kMaxFields; ++k) v = f == (uint32_t)k ? a[k] : v;
    return v;
}

/* p moved on by d bytes, by pointer arithmetic (an integer round trip would hide from the
 * compiler that the result still points into global memory). */
template <typename T>
__device__ __forceinline__ T *shift(T *p, uint64_t d) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(p) + d);
}

/* The workspace of lane f: every array of lane 0's, d = f * stride bytes further on. */
__device__ __forceinline__ Workspace lane_ws(const Workspace &w, uint32_t f, uint64_t stride) {
    const uint64_t d = (uint64_t)f * stride;
    Workspace r;
    r.info = shift(w.info, d);
    r.scratch = shift(w.scratch, d);
    r.chunk_words = shift(w.chunk_words, d);
    r.chunk_esc = shift(w.chunk_esc, d);
    r.chunk_tmask = shift(w.chunk_tmask, d);
    r.group_words = shift(w.group_words, d);
    r.group_esc = shift(w.group_esc, d);
    r.gpre_words = shift(w.gpre_words, d);
    r.gpre_esc = shift(w.gpre_esc, d);
    r.emask = shift(w.emask, d);
    r.stage_idx = shift(w.stage_idx, d);
    r.stage_val = shift(w.stage_val, d);
    r.widths = shift(w.widths, d);
    r.range_part = shift(w.range_part, d);
    r.means = shift(w.means, d);
    return r;
}

}  // namespace
}  // namespace eblc

#endif
