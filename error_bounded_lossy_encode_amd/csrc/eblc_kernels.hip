/*
 * eblc_kernels.hip -- gfx950 kernels of the error-bounded float32 codec.
 *
 * Method ("Pipeline Specialization Internals", FZGPUModules site): a linear quantizer with
 * step 2*eb absorbed into a 1-D Lorenzo predictor that resets at every block ("Roles and
 * strategies", "Forward declaration / Conventions"), zigzag, and an adaptive fixed-length
 * bitpack coder with one width byte per segment ("The device policy contract"); the inverse
 * unpacks, undoes the zigzag, prefix-sums inside each block and multiplies by 2*eb
 * ("Inverse declaration").  Like the chunk encoder of "nvrtc_chunk_fusion.h File
 * Reference" (launchNvrtcChunkFusedEncode), the encode kernel fills a fixed-size scratch slot
 * and a size per chunk, and a separate scan and pack tail compacts the slots; unlike it, the
 * outlier list is written in index order by its own kernel, so the stream is deterministic.
 *
 * gfx950 mapping: one wave64 owns a 2048-value chunk; a tile of 256 values is one 128-bit
 * load per lane (4 consecutive values); all intermediates stay in VGPRs; cross-lane work uses
 * DPP (wave_shr, quad_perm, row_half_mirror, row_shr, row_bcast); the packed payload of a
 * chunk is assembled in LDS with ds_or and leaves in 128-bit stores.  No MFMA: nothing here
 * is a contraction.  Built with -ffp-contract=off and IEEE denormals so the fp32 arithmetic is
 * the plain IEEE sequence written below.
 */
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
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf, bool BOUND_CTRL = false>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, BOUND_CTRL);
}

/* OR over the 8 lanes of an aligned 8-lane group (one 32-value segment). */
__device__ __forceinline__ uint32_t or8(uint32_t v) {
    v |= dpp<kDppQuadXor1>(0, v);
    v |= dpp<kDppQuadXor2>(0, v);
    v |= dpp<kDppRowHalfMirror>(0, v);
    return v;
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

/* ---- bound resolution -------------------------------------------------------------------- */

/* eb = eps * (max - min) in fp64, rounded toward zero to fp32; s = 2 eb; r = f32(1 / s).  An
 * unusable bound (no finite value, zero, subnormal, overflow) marks the plan's call RAW. */
__device__ void resolve_bound(float mn, float mx, double eps, DevInfo *info) {
    float eb_f = 0.0f, s = 0.0f, r = 0.0f;
    uint32_t valid = 0;
    if (mn <= mx) {
        const double range = (double)mx - (double)mn;
        const double eb_d = eps * range;
        float e = (float)eb_d;
        if (fabsf(e) <= FLT_MAX && (double)e > eb_d) {
            uint32_t b = __float_as_uint(e);
            if ((b & 0x7fffffffu) != 0) b -= 1;
            e = __uint_as_float(b);
        }
        const float s2 = 2.0f * e;
        const double inv = 1.0 / (double)s2;
        const float rr = (float)inv;
        if (e >= FLT_MIN && e <= FLT_MAX && fabsf(s2) <= FLT_MAX && fabsf(rr) <= FLT_MAX) {
            eb_f = e;
            s = s2;
            r = rr;
            valid = 1;
        }
    }
    info->eb_f = eb_f;
    info->s = s;
    info->r = r;
    info->valid = valid;
}

/* Finite-only running min / max.  Non-finite values are replaced by the neutral element. */
__device__ __forceinline__ void minmax_finite(float v, float &mn, float &mx) {
    const bool fin = fabsf(v) <= FLT_MAX;
    mn = fminf(mn, fin ? v : INFINITY);
    mx = fmaxf(mx, fin ? v : -INFINITY);
}

__device__ __forceinline__ void minmax4(const float4 &a, float &mn, float &mx) {
    minmax_finite(a.x, mn, mx);
    minmax_finite(a.y, mn, mx);
    minmax_finite(a.z, mn, mx);
    minmax_finite(a.w, mn, mx);
}

constexpr int kRangeUnroll = 8;

/* K1a: per-block min / max over the finite values.  The sweep runs from the end of the array
 * to its start (iteration k of every thread reads the k-th stride from the end), so the front
 * of the field is the most recently read when the encode kernel starts on it. */
__global__ __launch_bounds__(256) void range_partial_kernel(const float *__restrict__ x, uint64_t n,
                                                            float *__restrict__ part) {
    __shared__ float s_mn[4], s_mx[4];
    float mn[4] = {INFINITY, INFINITY, INFINITY, INFINITY};
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    const uint64_t n4 = n / 4;
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    const uint64_t tid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    uint64_t k = tid;
    for (; k + (kRangeUnroll - 1) * stride < n4; k += kRangeUnroll * stride) {
        float4 v[kRangeUnroll];
#pragma unroll
        for (int u = 0; u < kRangeUnroll; ++u) v[u] = x4[n4 - 1 - (k + u * stride)];
#pragma unroll
        for (int u = 0; u < kRangeUnroll; ++u) minmax4(v[u], mn[u & 3], mx[u & 3]);
    }
    for (; k < n4; k += stride) minmax4(x4[n4 - 1 - k], mn[0], mx[0]);
    if (tid < n - 4 * n4) minmax_finite(x[4 * n4 + tid], mn[1], mx[1]);
    float a = fminf(fminf(mn[0], mn[1]), fminf(mn[2], mn[3]));
    float b = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
    for (int o = 32; o >= 1; o >>= 1) {
        a = fminf(a, __shfl_xor(a, o));
        b = fmaxf(b, __shfl_xor(b, o));
    }
    const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) { s_mn[wave] = a; s_mx[wave] = b; }
    __syncthreads();
    if (threadIdx.x == 0) {
        part[2 * blockIdx.x] = fminf(fminf(s_mn[0], s_mn[1]), fminf(s_mn[2], s_mn[3]));
        part[2 * blockIdx.x + 1] = fmaxf(fmaxf(s_mx[0], s_mx[1]), fmaxf(s_mx[2], s_mx[3]));
    }
}

/* K1b: one workgroup folds the per-block partials and resolves the bound. */
__global__ __launch_bounds__(256) void range_resolve_kernel(const float *__restrict__ part, uint32_t nparts,
                                                            DevInfo *info, double eps) {
    __shared__ float s_mn[4], s_mx[4];
    float a = INFINITY, b = -INFINITY;
    for (uint32_t i = threadIdx.x; i < nparts; i += 256) {
        a = fminf(a, part[2 * i]);
        b = fmaxf(b, part[2 * i + 1]);
    }
    for (int o = 32; o >= 1; o >>= 1) {
        a = fminf(a, __shfl_xor(a, o));
        b = fmaxf(b, __shfl_xor(b, o));
    }
    const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) { s_mn[wave] = a; s_mx[wave] = b; }
    __syncthreads();
    if (threadIdx.x == 0) {
        a = fminf(fminf(s_mn[0], s_mn[1]), fminf(s_mn[2], s_mn[3]));
        b = fmaxf(fmaxf(s_mx[0], s_mx[1]), fmaxf(s_mx[2], s_mx[3]));
        resolve_bound(a, b, eps, info);
    }
}

/* ---- K2: fused encode ------------------------------------------------------------------------ */

/* Per-wave state of the chunk being encoded. */
struct EncState {
    int32_t carry;    /* code of the value before the tile (Lorenzo predecessor of lane 0) */
    uint32_t words;   /* payload words of the chunk so far */
    uint32_t escs;    /* escapes in the chunk so far */
    uint32_t tmask;   /* tiles with at least one escape */
};

/* One tile of 256 values: 4 consecutive values per lane.  FULL = every value of the tile is
 * below n (no tail masking). */
template <bool FULL>
__device__ __forceinline__ void encode_tile(const float4 v, uint64_t e0, uint64_t n, const QParams &qp,
                                            uint32_t bmask, int t, uint32_t *pay, uint8_t *wid,
                                            uint32_t *emask_tile, EncState &st) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t j = lane & 7;
    const float xs[4] = {v.x, v.y, v.z, v.w};
    float q0f[4];
    int32_t q[4];
    bool fast[4];
    /* quantize: rint(x * inv2eb); the fast test (code below 2^T and accepted) is branch free */
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float p = xs[k] * qp.r;
        q0f[k] = rintf(p);
        const float y = q0f[k] * qp.s;
        const float diff = xs[k] - y;
        const float half_y = 0.5f * fabsf(y);
        fast[k] = ((uint32_t)(fabsf(q0f[k]) < qp.tlim) & (uint32_t)(fabsf(diff) <= qp.eb) &
                   (uint32_t)(fabsf(xs[k]) >= half_y)) != 0;
        q[k] = (int32_t)q0f[k];
    }
    uint32_t esc = 0;
    const bool all_fast = ((uint32_t)fast[0] & (uint32_t)fast[1] & (uint32_t)fast[2] & (uint32_t)fast[3]) != 0;
    if (__ballot(!all_fast)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (!fast[k]) {
                uint32_t e;
                q[k] = quantize_slow(xs[k], q0f[k], qp, &e);
                esc |= e << k;
            }
        }
    }
    /* Lorenzo: previous value's code (previous lane, or the carry for lane 0), 0 at a block start */
    const int32_t prev = (int32_t)dpp<kDppWaveShr1>((uint32_t)st.carry, (uint32_t)q[3]);
    const bool reset = ((uint32_t)e0 & bmask) == 0;
    uint32_t z[4];
    z[0] = zigzag(reset ? q[0] : q[0] - prev);
    z[1] = zigzag(q[1] - q[0]);
    z[2] = zigzag(q[2] - q[1]);
    z[3] = zigzag(q[3] - q[2]);
    st.carry = (int32_t)readlane((uint32_t)q[3], 63);
    if (!FULL) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (e0 + k >= n) z[k] = 0;
    }
    /* segment width: bit length of the OR of its 32 codes */
    const uint32_t orv = or8(z[0] | z[1] | z[2] | z[3]);
    const uint32_t w = orv ? 32u - (uint32_t)__builtin_clz(orv) : 0u;
    /* word offset of the segment in the chunk: scan of widths over the tile's 8 segments */
    const uint32_t incl = wave_incl_scan(j == 0 ? w : 0u);
    const uint32_t seg_words = st.words + incl - w;
    wid[t * 8 + (lane >> 3)] = (uint8_t)w;
    /* pack: value k of lane j sits at bit (4j + k) w of its segment.  The lane's 4w bits are
     * emitted low word first; only words holding bits are OR-ed into LDS (at most 5, and only
     * the first and last can be shared with a neighbouring lane). */
    const uint32_t bitpos = 32u * seg_words + 4u * w * j;
    uint32_t wi = bitpos >> 5;
    uint32_t nb = bitpos & 31u;
    uint64_t acc = (uint64_t)z[0] << nb;
    nb += w;
#pragma unroll
    for (int k = 1; k <= 4; ++k) {
        if (nb >= 32) {
            lds_or(pay + wi, (uint32_t)acc);
            ++wi;
            acc >>= 32;
            nb -= 32;
        }
        if (k < 4) {
            acc |= (uint64_t)z[k] << nb;
            nb += w;
        }
    }
    if (nb > 0) lds_or(pay + wi, (uint32_t)acc);
    st.words += readlane(incl, 63);
    /* escapes: per-segment bitmask (element 4j + k of the segment) and counts */
    if (__ballot(esc != 0)) {
        const uint32_t segm = or8(esc << (4 * j));
        if (j == 0) emask_tile[lane >> 3] = segm;
        st.escs += (uint32_t)(__popcll(__ballot(esc & 1u)) + __popcll(__ballot(esc & 2u)) +
                              __popcll(__ballot(esc & 4u)) + __popcll(__ballot(esc & 8u)));
        st.tmask |= 1u << t;
    }
}

template <bool FULL>
__device__ __forceinline__ void encode_chunk(const float *__restrict__ x, uint64_t cbase, uint64_t n,
                                             const QParams &qp, uint32_t bmask, uint32_t *pay,
                                             uint8_t *wid, uint32_t *emask_chunk, EncState &st) {
    const uint32_t lane = threadIdx.x & 63;
    float4 v[kTilesPerChunk];
    if (FULL) {
        const float4 *src = reinterpret_cast<const float4 *>(x + cbase) + lane;
#pragma unroll
        for (int t = 0; t < kTilesPerChunk; ++t) v[t] = src[t * (kTile / 4)];
    } else {
#pragma unroll
        for (int t = 0; t < kTilesPerChunk; ++t) {
            const uint64_t e = cbase + (uint64_t)t * kTile + 4 * lane;
            v[t].x = e + 0 < n ? x[e + 0] : 0.0f;
            v[t].y = e + 1 < n ? x[e + 1] : 0.0f;
            v[t].z = e + 2 < n ? x[e + 2] : 0.0f;
            v[t].w = e + 3 < n ? x[e + 3] : 0.0f;
        }
    }
    wave_lds_sync();
    const uint32_t ntiles = FULL ? kTilesPerChunk : (uint32_t)((n - cbase + kTile - 1) / kTile);
#pragma unroll
    for (int t = 0; t < kTilesPerChunk; ++t) {
        if (FULL || (uint32_t)t < ntiles)
            encode_tile<FULL>(v[t], cbase + (uint64_t)t * kTile + 4 * lane, n, qp, bmask, t, pay, wid,
                              emask_chunk + t * 8, st);
    }
}

/* One wave per chunk.  Per tile: quantize 4 values per lane, Lorenzo delta against the previous
 * value (previous lane by wave_shr, previous tile by a carried code, 0 at a block start),
 * zigzag, the segment width from an 8-lane OR, the segment's word offset from a wave scan, and
 * the packed bits OR-ed into the chunk's LDS buffer.  Outputs: the chunk's words in its scratch
 * slot, its 64 width bytes, its word and escape counts, the escape bitmask of every tile that
 * has an escape, and per-workgroup sums for the scan. */
__global__ __launch_bounds__(kBlockThreads) void encode_kernel(
    const float *__restrict__ x, PlanArgs pa, Workspace ws, uint8_t *__restrict__ widths_dst,
    uint64_t widths_bytes) {
    __shared__ uint4 s_pay4[kWavesPerBlock][kChunk / 4 + 1];
    __shared__ uint4 s_wid4[kWavesPerBlock][kSegsPerChunk / 16];
    __shared__ uint32_t s_grp[2][kWavesPerBlock];

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t c = blockIdx.x * kWavesPerBlock + wave;
    const DevInfo *info = ws.info;
    EncState st = {0, 0, 0, 0};

    if (c < pa.nchunks && info->valid) {
        QParams qp;
        qp.eb = info->eb_f;
        qp.s = info->s;
        qp.r = info->r;
        qp.T = pa.T;
        qp.tlim = (float)(1u << pa.T);
        uint32_t *pay = reinterpret_cast<uint32_t *>(s_pay4[wave]);
        uint8_t *wid = reinterpret_cast<uint8_t *>(s_wid4[wave]);
        const uint4 zero4 = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < kChunk / 4 / kWave; ++i) s_pay4[wave][lane + kWave * i] = zero4;
        if (lane < kSegsPerChunk / 16) s_wid4[wave][lane] = zero4;
        const uint64_t cbase = (uint64_t)c * kChunk;
        uint32_t *emask_chunk = ws.emask + (uint64_t)c * kSegsPerChunk;
        if (cbase + kChunk <= pa.n)
            encode_chunk<true>(x, cbase, pa.n, qp, pa.B - 1, pay, wid, emask_chunk, st);
        else
            encode_chunk<false>(x, cbase, pa.n, qp, pa.B - 1, pay, wid, emask_chunk, st);
        wave_lds_sync();
        /* chunk payload -> scratch slot, widths -> stream (or staging) */
        uint4 *dst = reinterpret_cast<uint4 *>(ws.scratch + cbase);
        const uint32_t nvec = (st.words + 3) >> 2;
        for (uint32_t i = lane; i < nvec; i += kWave) dst[i] = s_pay4[wave][i];
        if (lane < kSegsPerChunk / 16) {
            const uint64_t off = (uint64_t)c * kSegsPerChunk + 16u * lane;
            if (off < widths_bytes) *reinterpret_cast<uint4 *>(widths_dst + off) = s_wid4[wave][lane];
        }
        if (lane == 0) {
            ws.chunk_words[c] = st.words;
            ws.chunk_esc[c] = st.escs;
            ws.chunk_tmask[c] = st.tmask;
        }
    }
    if (lane == 0) {
        s_grp[0][wave] = st.words;
        s_grp[1][wave] = st.escs;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        ws.group_words[blockIdx.x] = s_grp[0][0] + s_grp[0][1] + s_grp[0][2] + s_grp[0][3];
        ws.group_esc[blockIdx.x] = s_grp[1][0] + s_grp[1][1] + s_grp[1][2] + s_grp[1][3];
    }
}

/* ---- K3 / K6b: single-workgroup exclusive scan over groups -------------------------------- */

/* Exclusive prefix of a[0..ng) and b[0..ng) into pa_out / pb_out; returns the totals in
 * tot[0], tot[1] (visible to every thread after the call).  1024 threads, 4 items each per
 * round. */
__device__ void block_scan2(const uint32_t *__restrict__ a, const uint32_t *__restrict__ b,
                            uint32_t *__restrict__ pa_out, uint32_t *__restrict__ pb_out,
                            uint32_t ng, uint32_t *tot) {
    __shared__ uint32_t s_wa[kScanThreads / kWave], s_wb[kScanThreads / kWave];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t carry_a = 0, carry_b = 0;
    for (uint32_t base = 0; base < ng; base += 4 * kScanThreads) {
        const uint32_t i0 = base + 4 * tid;
        uint32_t va[4], vb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            va[k] = (i0 + k < ng) ? a[i0 + k] : 0u;
            vb[k] = (b != nullptr && i0 + k < ng) ? b[i0 + k] : 0u;
        }
        const uint32_t ta = va[0] + va[1] + va[2] + va[3];
        const uint32_t tb = vb[0] + vb[1] + vb[2] + vb[3];
        const uint32_t ia = wave_incl_scan(ta);
        const uint32_t ib = wave_incl_scan(tb);
        if (lane == 63) { s_wa[wave] = ia; s_wb[wave] = ib; }
        __syncthreads();
        uint32_t oa = 0, ob = 0, sa = 0, sb = 0;
        for (uint32_t w = 0; w < kScanThreads / kWave; ++w) {
            const uint32_t xa = s_wa[w], xb = s_wb[w];
            if (w < wave) { oa += xa; ob += xb; }
            sa += xa;
            sb += xb;
        }
        uint32_t ea = carry_a + oa + ia - ta;
        uint32_t eb = carry_b + ob + ib - tb;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (i0 + k < ng) {
                pa_out[i0 + k] = ea;
                if (pb_out != nullptr) pb_out[i0 + k] = eb;
            }
            ea += va[k];
            eb += vb[k];
        }
        carry_a += sa;
        carry_b += sb;
        __syncthreads();
    }
    tot[0] = carry_a;
    tot[1] = carry_b;
}

/* Compress finalize: totals -> stream layout, RAW decision, header. */
__global__ __launch_bounds__(kScanThreads) void scan_compress_kernel(PlanArgs pa, Workspace ws,
                                                                     uint8_t *out, uint64_t cap) {
    __shared__ uint32_t s_hdr[32];
    __shared__ uint32_t s_fits;
    uint32_t tot[2];
    block_scan2(ws.group_words, ws.group_esc, ws.gpre_words, ws.gpre_esc, pa.ngroups, tot);
    DevInfo *info = ws.info;
    if (threadIdx.x == 0) {
        const uint64_t n = pa.n;
        const uint64_t S = tot[0], m = tot[1];
        const uint64_t raw_total = kHeaderBytes + align16(4 * n);
        const uint64_t payload_off = kHeaderBytes + align16(pa.nseg);
        const uint64_t lossy_total = payload_off + align16(4 * S) + 2 * align16(4 * m);
        const bool valid = info->valid != 0;
        const bool raw = !valid || m > pa.side_max || lossy_total > raw_total;
        uint64_t f_m, f_pb, f_po, f_oi, f_ov, f_tot;
        if (raw) {
            f_m = 0; f_pb = 4 * n; f_po = kHeaderBytes;
            f_oi = raw_total; f_ov = raw_total; f_tot = raw_total;
        } else {
            f_m = m; f_pb = 4 * S; f_po = payload_off;
            f_oi = payload_off + align16(4 * S);
            f_ov = f_oi + align16(4 * m);
            f_tot = f_ov + align16(4 * m);
        }
        const uint32_t fits = f_tot <= cap ? 1u : 0u;
        info->mode = raw ? 1u : 0u;
        info->m = f_m;
        info->payload_words = f_pb / 4;
        info->payload_off = f_po;
        info->oidx_off = f_oi;
        info->oval_off = f_ov;
        info->total = f_tot;
        info->fits = fits;
        s_fits = fits;
        uint32_t *h = s_hdr;
        h[0] = kMagic;
        h[1] = kVersion | (kHeaderBytes << 16);
        h[2] = (raw ? 1u : 0u) | (pa.rank << 8) | (5u << 16) | (pa.T << 24);
        h[3] = pa.B;
        for (int a = 0; a < 4; ++a) {
            h[4 + 2 * a] = (uint32_t)pa.dims[a];
            h[5 + 2 * a] = (uint32_t)(pa.dims[a] >> 32);
        }
        const uint64_t u64s[8] = {n, 0, f_m, f_pb, kHeaderBytes, f_po, f_oi, f_ov};
        h[12] = (uint32_t)u64s[0];
        h[13] = (uint32_t)(u64s[0] >> 32);
        h[14] = __float_as_uint(info->eb_f);
        h[15] = __float_as_uint(info->s);
        h[16] = __float_as_uint(info->r);
        h[17] = 0;
        for (int a = 2; a < 8; ++a) {
            h[18 + 2 * (a - 2)] = (uint32_t)u64s[a];
            h[19 + 2 * (a - 2)] = (uint32_t)(u64s[a] >> 32);
        }
        h[30] = (uint32_t)f_tot;
        h[31] = (uint32_t)(f_tot >> 32);
    }
    __syncthreads();
    if (s_fits && threadIdx.x < 32) reinterpret_cast<uint32_t *>(out)[threadIdx.x] = s_hdr[threadIdx.x];
}

/* Word offset of chunk c in the packed payload (or outlier rank), from the group prefix plus
 * the chunks before c in its group. */
__device__ __forceinline__ uint32_t chunk_offset(const uint32_t *gpre, const uint32_t *per_chunk,
                                                 uint32_t c) {
    const uint32_t g = c / kChunksPerGroup;
    uint32_t o = gpre[g];
    for (uint32_t k = g * kChunksPerGroup; k < c; ++k) o += per_chunk[k];
    return o;
}

/* ---- K4: compaction of the scratch slots (or the RAW copy) -------------------------------- */

__global__ __launch_bounds__(kBlockThreads) void compact_kernel(const float *__restrict__ x,
                                                                PlanArgs pa, Workspace ws,
                                                                uint8_t *__restrict__ out,
                                                                const uint8_t *__restrict__ widths_src) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t c = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (c >= pa.nchunks) return;
    const DevInfo *info = ws.info;
    if (!info->fits) return;
    const uint64_t n = pa.n;
    const uint64_t cbase = (uint64_t)c * kChunk;
    const bool last = c == pa.nchunks - 1;
    if (info->mode == 1) {
        const uint64_t cnt = (n - cbase < (uint64_t)kChunk) ? n - cbase : (uint64_t)kChunk;
        uint32_t *dstw = reinterpret_cast<uint32_t *>(out + kHeaderBytes) + cbase;
        const uint32_t *srcw = reinterpret_cast<const uint32_t *>(x) + cbase;
        if (cnt == (uint64_t)kChunk) {
            const uint4 *s4 = reinterpret_cast<const uint4 *>(srcw);
            uint4 *d4 = reinterpret_cast<uint4 *>(dstw);
#pragma unroll
            for (int i = 0; i < kChunk / 4 / kWave; ++i) d4[lane + kWave * i] = s4[lane + kWave * i];
        } else {
            for (uint32_t i = lane; i < cnt; i += kWave) dstw[i] = srcw[i];
        }
        if (last) {
            const uint64_t end = kHeaderBytes + 4 * n;
            const uint64_t pad = align16(4 * n) - 4 * n;
            if (lane < pad / 4) reinterpret_cast<uint32_t *>(out + end)[lane] = 0u;
        }
        return;
    }
    const uint32_t W = chunk_offset(ws.gpre_words, ws.chunk_words, c);
    const uint32_t P = ws.chunk_words[c];
    uint32_t *dst = reinterpret_cast<uint32_t *>(out + info->payload_off) + W;
    const uint32_t *src = ws.scratch + cbase;
    for (uint32_t i = lane; i < P; i += kWave) dst[i] = src[i];
    if (widths_src != nullptr && lane < kSegsPerChunk / 16) {
        const uint64_t off = (uint64_t)c * kSegsPerChunk + 16u * lane;
        if (off < align16(pa.nseg))
            *reinterpret_cast<uint4 *>(out + kHeaderBytes + off) =
                *reinterpret_cast<const uint4 *>(widths_src + off);
    }
    if (last) {
        const uint64_t pend = info->payload_off + 4 * info->payload_words;
        const uint64_t pad = info->oidx_off - pend;
        if (lane < pad / 4) reinterpret_cast<uint32_t *>(out + pend)[lane] = 0u;
    }
}

/* ---- K5: outliers in index order ------------------------------------------------------------ */

__global__ __launch_bounds__(kBlockThreads) void outlier_kernel(const float *__restrict__ x,
                                                                PlanArgs pa, Workspace ws,
                                                                uint8_t *__restrict__ out) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t c = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (c >= pa.nchunks) return;
    const DevInfo *info = ws.info;
    if (!info->fits || info->mode == 1) return;
    const uint64_t m = info->m;
    uint32_t *oidx = reinterpret_cast<uint32_t *>(out + info->oidx_off);
    uint32_t *oval = reinterpret_cast<uint32_t *>(out + info->oval_off);
    if (c == pa.nchunks - 1) {
        const uint64_t pad = (align16(4 * m) - 4 * m) / 4;
        if (lane < pad) {
            oidx[m + lane] = 0u;
            oval[m + lane] = 0u;
        }
    }
    if (ws.chunk_esc[c] == 0) return;
    const uint32_t O = chunk_offset(ws.gpre_esc, ws.chunk_esc, c);
    const uint32_t tm = ws.chunk_tmask[c];
    uint32_t mask = ((tm >> (lane >> 3)) & 1u) ? ws.emask[(uint64_t)c * kSegsPerChunk + lane] : 0u;
    const uint32_t cnt = (uint32_t)__popc(mask);
    uint32_t rank = O + wave_incl_scan(cnt) - cnt;
    const uint64_t segbase = (uint64_t)c * kChunk + 32u * lane;
    const uint32_t *xb = reinterpret_cast<const uint32_t *>(x);
    while (mask) {
        const uint32_t bit = (uint32_t)__builtin_ctz(mask);
        const uint64_t idx = segbase + bit;
        oidx[rank] = (uint32_t)idx;
        oval[rank] = xb[idx];
        ++rank;
        mask &= mask - 1;
    }
}

/* ---- K6a: decode sizes ---------------------------------------------------------------------- */

/* One thread per chunk: payload words of the chunk = sum of its width bytes; a width above 32
 * flags the stream.  Quads of threads form the groups the scan runs over. */
__global__ __launch_bounds__(256) void decode_sizes_kernel(const uint8_t *__restrict__ in,
                                                           PlanArgs pa, Workspace ws) {
    const uint32_t c = blockIdx.x * 256 + threadIdx.x;
    uint32_t sum = 0, bad = 0;
    if (c < pa.nchunks) {
        const uint64_t s0 = (uint64_t)c * kSegsPerChunk;
        const uint64_t segs = (pa.nseg - s0 < (uint64_t)kSegsPerChunk) ? pa.nseg - s0 : (uint64_t)kSegsPerChunk;
        const uint8_t *wp = in + kHeaderBytes + s0;
        if (segs == (uint64_t)kSegsPerChunk) {
            const uint4 *w4 = reinterpret_cast<const uint4 *>(wp);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 v = w4[i];
                const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    sum = __builtin_amdgcn_sad_u8(vv[k], 0u, sum);
                    bad |= (((vv[k] & 0x7F7F7F7Fu) + 0x5F5F5F5Fu) | vv[k]) & 0x80808080u;
                }
            }
        } else {
            for (uint64_t k = 0; k < segs; ++k) {
                const uint32_t w = wp[k];
                sum += w;
                bad |= w > 32 ? 1u : 0u;
            }
        }
        ws.chunk_words[c] = sum;
    }
    uint32_t g = sum;
    g += dpp<kDppQuadXor1>(0, g);
    g += dpp<kDppQuadXor2>(0, g);
    if ((threadIdx.x & 3) == 0 && c / kChunksPerGroup < pa.ngroups) ws.group_words[c / kChunksPerGroup] = g;
    if (bad) atomicOr(&ws.info->width_bad, 1u);
}

/* ---- K6b: decode scan + header validation ------------------------------------------------- */

__device__ __forceinline__ uint64_t ld64(const uint32_t *h, int i) {
    return (uint64_t)h[i] | ((uint64_t)h[i + 1] << 32);
}

__global__ __launch_bounds__(kScanThreads) void scan_decompress_kernel(const uint8_t *__restrict__ in,
                                                                       uint64_t in_bytes, PlanArgs pa,
                                                                       Workspace ws) {
    uint32_t tot[2];
    block_scan2(ws.group_words, nullptr, ws.gpre_words, nullptr, pa.ngroups, tot);
    if (threadIdx.x != 0) return;
    DevInfo *info = ws.info;
    const uint32_t *h = reinterpret_cast<const uint32_t *>(in);
    uint32_t hw[32];
    for (int i = 0; i < 32; ++i) hw[i] = h[i];
    const uint64_t n = pa.n;
    const uint32_t mode = hw[2] & 0xff, rank = (hw[2] >> 8) & 0xff, log2seg = (hw[2] >> 16) & 0xff;
    const uint32_t T = hw[2] >> 24, B = hw[3];
    bool ok = hw[0] == kMagic && (hw[1] & 0xffff) == kVersion && (hw[1] >> 16) == kHeaderBytes;
    ok = ok && (mode == 0 || mode == 1) && rank == pa.rank && log2seg == 5 && T >= 1 && T <= 30;
    ok = ok && B >= 32 && B <= 2048 && (B & (B - 1)) == 0;
    for (int a = 0; a < 4; ++a) ok = ok && ld64(hw, 4 + 2 * a) == pa.dims[a];
    ok = ok && ld64(hw, 12) == n && hw[17] == 0 && ld64(hw, 22) == kHeaderBytes;
    const uint64_t m = ld64(hw, 18), pb = ld64(hw, 20), po = ld64(hw, 24), oi = ld64(hw, 26);
    const uint64_t ov = ld64(hw, 28), total = ld64(hw, 30);
    const float eb_f = __uint_as_float(hw[14]), s = __uint_as_float(hw[15]);
    if (mode == 1) {
        const uint64_t end = kHeaderBytes + align16(4 * n);
        ok = ok && m == 0 && pb == 4 * n && po == kHeaderBytes && oi == end && ov == end && total == end;
    } else {
        ok = ok && eb_f >= FLT_MIN && eb_f <= FLT_MAX && fabsf(s) <= FLT_MAX && s == 2.0f * eb_f;
        ok = ok && m <= n && (pb & 3) == 0 && pb == 4 * (uint64_t)tot[0] && info->width_bad == 0;
        ok = ok && po == kHeaderBytes + align16(pa.nseg) && oi == po + align16(pb);
        ok = ok && ov == oi + align16(4 * m) && total == ov + align16(4 * m);
    }
    ok = ok && total <= in_bytes;
    const uint32_t err = ok ? 0u : 1u;
    info->err = err;
    info->sticky |= err;
    info->width_bad = 0;
    info->mode = mode;
    info->m = ok ? m : 0;
    info->payload_off = po;
    info->oidx_off = oi;
    info->oval_off = ov;
    info->dec_s = s;
}

/* ---- K7: fused decode ------------------------------------------------------------------------ */

/* One wave per chunk: stage the chunk's packed words in LDS (128-bit loads), then per tile
 * unpack each lane's 4 values, undo the zigzag, prefix-sum inside each block (in-lane, then a
 * segmented DPP scan across lanes, plus the carry from the previous tile when a block spans
 * tiles), dequantize with f32(f32(q) * s) and store 4 values with one 128-bit store. */
__global__ __launch_bounds__(kBlockThreads) void decode_kernel(const uint8_t *__restrict__ in,
                                                               PlanArgs pa, Workspace ws,
                                                               float *__restrict__ out) {
    __shared__ uint4 s_pay4[kWavesPerBlock][kChunk / 4 + 2];
    __shared__ uint32_t s_w[kWavesPerBlock][kSegsPerChunk];
    __shared__ uint32_t s_so[kWavesPerBlock][kSegsPerChunk];

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t c = blockIdx.x * kWavesPerBlock + wave;
    if (c >= pa.nchunks) return;
    const DevInfo *info = ws.info;
    if (info->err) return;
    const uint64_t n = pa.n;
    const uint64_t cbase = (uint64_t)c * kChunk;
    const bool full = cbase + kChunk <= n;
    if (info->mode == 1) {
        const uint64_t cnt = full ? (uint64_t)kChunk : n - cbase;
        const uint32_t *srcw = reinterpret_cast<const uint32_t *>(in + kHeaderBytes) + cbase;
        uint32_t *dstw = reinterpret_cast<uint32_t *>(out) + cbase;
        if (full) {
            const uint4 *s4 = reinterpret_cast<const uint4 *>(srcw);
            uint4 *d4 = reinterpret_cast<uint4 *>(dstw);
#pragma unroll
            for (int i = 0; i < kChunk / 4 / kWave; ++i) d4[lane + kWave * i] = s4[lane + kWave * i];
        } else {
            for (uint32_t i = lane; i < cnt; i += kWave) dstw[i] = srcw[i];
        }
        return;
    }
    const uint32_t W = chunk_offset(ws.gpre_words, ws.chunk_words, c);
    const uint32_t P = ws.chunk_words[c];
    const uint64_t sw = info->payload_off / 4 + W; /* stream word index of the chunk's first word */
    const uint64_t a0 = sw & ~(uint64_t)3;
    const uint32_t lb = (uint32_t)(sw - a0);
    const uint32_t units = (lb + P + 3) >> 2;
    const uint4 *src = reinterpret_cast<const uint4 *>(in) + a0 / 4;
    for (uint32_t u = lane; u < units; u += kWave) s_pay4[wave][u] = src[u];
    const uint64_t seg = (uint64_t)c * kSegsPerChunk + lane;
    const uint32_t wl = seg < pa.nseg ? (uint32_t)in[kHeaderBytes + seg] : 0u;
    const uint32_t so = wave_incl_scan(wl) - wl;
    s_w[wave][lane] = wl;
    s_so[wave][lane] = so;
    wave_lds_sync();

    const uint32_t *pay = reinterpret_cast<const uint32_t *>(s_pay4[wave]);
    const float s = info->dec_s;
    const uint32_t B = pa.B;
    const uint32_t seglen = (B / 4 < 64u) ? B / 4 : 64u;
    const uint32_t dist = lane & (seglen - 1);
    const uint32_t ntiles = full ? kTilesPerChunk : (uint32_t)((n - cbase + kTile - 1) / kTile);
    const uint32_t j = lane & 7;
    int32_t carry = 0;
#pragma unroll
    for (int t = 0; t < kTilesPerChunk; ++t) {
        if ((uint32_t)t < ntiles) {
            const uint32_t g = (uint32_t)t * 8 + (lane >> 3);
            const uint32_t w = s_w[wave][g];
            const uint32_t bp = 32u * (lb + s_so[wave][g]) + 4u * w * j;
            const uint32_t mask = w >= 32 ? 0xffffffffu : ((1u << w) - 1u);
            int32_t cs[4];
            int32_t run = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t pos = bp + (uint32_t)k * w;
                const uint32_t wi = pos >> 5;
                const uint64_t pair = (uint64_t)pay[wi] | ((uint64_t)pay[wi + 1] << 32);
                const uint32_t z = (uint32_t)(pair >> (pos & 31u)) & mask;
                run += unzigzag(z);
                cs[k] = run;
            }
            const uint32_t incl = wave_seg_scan((uint32_t)cs[3], dist, seglen);
            const bool open = (((uint32_t)t * kTile) & (B - 1)) != 0;
            const int32_t base = (int32_t)(incl - (uint32_t)cs[3]) + (open ? carry : 0);
            int32_t q[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = base + cs[k];
            carry = (int32_t)readlane((uint32_t)q[3], 63);
            float4 o;
            o.x = (float)q[0] * s;
            o.y = (float)q[1] * s;
            o.z = (float)q[2] * s;
            o.w = (float)q[3] * s;
            const uint64_t e0 = cbase + (uint64_t)t * kTile + 4 * lane;
            if (full) {
                *reinterpret_cast<float4 *>(out + e0) = o;
            } else {
                if (e0 + 0 < n) out[e0 + 0] = o.x;
                if (e0 + 1 < n) out[e0 + 1] = o.y;
                if (e0 + 2 < n) out[e0 + 2] = o.z;
                if (e0 + 3 < n) out[e0 + 3] = o.w;
            }
        }
    }
}

/* ---- K8: outlier patch ------------------------------------------------------------------------ */

__global__ __launch_bounds__(256) void patch_kernel(const uint8_t *__restrict__ in, PlanArgs pa,
                                                    Workspace ws, float *__restrict__ out) {
    DevInfo *info = ws.info;
    if (info->err || info->mode == 1) return;
    const uint64_t m = info->m;
    const uint32_t *oidx = reinterpret_cast<const uint32_t *>(in + info->oidx_off);
    const uint32_t *oval = reinterpret_cast<const uint32_t *>(in + info->oval_off);
    uint32_t *ob = reinterpret_cast<uint32_t *>(out);
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    for (uint64_t k = (uint64_t)blockIdx.x * 256 + threadIdx.x; k < m; k += stride) {
        const uint32_t idx = oidx[k];
        const bool ok = idx < pa.n && (k == 0 || oidx[k - 1] < idx);
        if (ok) ob[idx] = oval[k];
        else atomicOr(&info->sticky, 1u);
    }
}

}  // namespace

/* ---- launchers ------------------------------------------------------------------------------- */

hipError_t launch_range(const float *x, const PlanArgs &pa, const Workspace &ws, double eps,
                        hipStream_t stream) {
    const uint64_t want = (pa.n / 4 + 256 * 16 - 1) / (256 * 16);
    const uint32_t grid = (uint32_t)(want < 1 ? 1 : (want > (uint64_t)kRangeBlocksMax ? kRangeBlocksMax : want));
    hipLaunchKernelGGL(range_partial_kernel, dim3(grid), dim3(256), 0, stream, x, pa.n, ws.range_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(range_resolve_kernel, dim3(1), dim3(256), 0, stream, ws.range_part, grid, ws.info,
                       eps);
    return hipGetLastError();
}

hipError_t launch_encode(const float *x, const PlanArgs &pa, const Workspace &ws,
                         uint8_t *widths_dst, uint64_t widths_bytes, hipStream_t stream) {
    hipLaunchKernelGGL(encode_kernel, dim3(pa.ngroups), dim3(kBlockThreads), 0, stream, x, pa, ws,
                       widths_dst, widths_bytes);
    return hipGetLastError();
}

hipError_t launch_scan_compress(const PlanArgs &pa, const Workspace &ws, uint8_t *out,
                                uint64_t out_capacity, hipStream_t stream) {
    hipLaunchKernelGGL(scan_compress_kernel, dim3(1), dim3(kScanThreads), 0, stream, pa, ws, out,
                       out_capacity);
    return hipGetLastError();
}

hipError_t launch_compact(const float *x, const PlanArgs &pa, const Workspace &ws, uint8_t *out,
                          const uint8_t *widths_src, hipStream_t stream) {
    hipLaunchKernelGGL(compact_kernel, dim3(pa.ngroups), dim3(kBlockThreads), 0, stream, x, pa, ws,
                       out, widths_src);
    return hipGetLastError();
}

hipError_t launch_outliers(const float *x, const PlanArgs &pa, const Workspace &ws, uint8_t *out,
                           hipStream_t stream) {
    hipLaunchKernelGGL(outlier_kernel, dim3(pa.ngroups), dim3(kBlockThreads), 0, stream, x, pa, ws,
                       out);
    return hipGetLastError();
}

hipError_t launch_decode_sizes(const uint8_t *in, const PlanArgs &pa, const Workspace &ws,
                               hipStream_t stream) {
    const uint32_t grid = (pa.nchunks + 255) / 256;
    hipLaunchKernelGGL(decode_sizes_kernel, dim3(grid), dim3(256), 0, stream, in, pa, ws);
    return hipGetLastError();
}

hipError_t launch_scan_decompress(const uint8_t *in, uint64_t in_bytes, const PlanArgs &pa,
                                  const Workspace &ws, hipStream_t stream) {
    hipLaunchKernelGGL(scan_decompress_kernel, dim3(1), dim3(kScanThreads), 0, stream, in, in_bytes,
                       pa, ws);
    return hipGetLastError();
}

hipError_t launch_decode(const uint8_t *in, const PlanArgs &pa, const Workspace &ws, float *out,
                         hipStream_t stream) {
    hipLaunchKernelGGL(decode_kernel, dim3(pa.ngroups), dim3(kBlockThreads), 0, stream, in, pa, ws,
                       out);
    return hipGetLastError();
}

hipError_t launch_patch(const uint8_t *in, const PlanArgs &pa, const Workspace &ws, float *out,
                        hipStream_t stream) {
    uint64_t want = (pa.side_max + 255) / 256;
    uint32_t grid = (uint32_t)(want < 1 ? 1 : (want > (uint64_t)kPatchBlocksMax ? kPatchBlocksMax : want));
    hipLaunchKernelGGL(patch_kernel, dim3(grid), dim3(256), 0, stream, in, pa, ws, out);
    return hipGetLastError();
}

}  // namespace eblc
