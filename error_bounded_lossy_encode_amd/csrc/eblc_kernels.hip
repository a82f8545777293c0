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
 * compaction writes the outlier list in index order, so the stream is deterministic.  The
 * stream also carries an offset table (the payload words before each group of 8192 values),
 * so the decoder needs no scan: it decodes, then a small kernel patches the outliers.
 *
 * gfx950 mapping: one wave64 owns a 2048-value chunk; a tile of 256 values is one 128-bit
 * load per lane (4 consecutive values); all intermediates stay in VGPRs; cross-lane work uses
 * DPP (wave_shr, quad_perm, row_half_mirror, row_shr, row_bcast); the packed payload of a
 * chunk is assembled in LDS with ds_or and leaves in 128-bit stores.  No MFMA: nothing here
 * is a contraction.  Built with -ffp-contract=off and IEEE denormals so the fp32 arithmetic is
 * the plain IEEE sequence written below.
 */
#include "eblc_device.h"

namespace eblc {
namespace {

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

/* K1a: per-workgroup min / max over the finite values.  Workgroup b reads float4 elements
 * [b kRangeSpan, (b + 1) kRangeSpan), 16 per thread, all issued before any is used, with
 * non-temporal loads: the field is streamed once and must not evict what the caches hold (on
 * gfx950 a plain load of a line also forces out dirty lines left by earlier writes, which
 * halves the read rate).  The last workgroup also takes the n mod 4 trailing values. */
template <bool STRIDED>
__device__ __forceinline__ void range_partial_body(const float *__restrict__ x,
                                                   uint64_t n, Layout lo,
                                                   float *__restrict__ part) {
    __shared__ float s_mn[kRangeThreads / kWave], s_mx[kRangeThreads / kWave];
    float mn[4] = {INFINITY, INFINITY, INFINITY, INFINITY};
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    const uint64_t n4 = n / 4;
    const uint64_t base = (uint64_t)blockIdx.x * kRangeSpan + threadIdx.x;
    if (base + (uint64_t)(kRangeVec - 1) * kRangeThreads < n4) {
        float4 v[kRangeVec];
#pragma unroll
        for (int u = 0; u < kRangeVec; ++u) v[u] = load4<STRIDED>(x, lo, 4 * (base + (uint64_t)u * kRangeThreads));
#pragma unroll
        for (int u = 0; u < kRangeVec; ++u) minmax4(v[u], mn[u & 3], mx[u & 3]);
    } else {
        for (int u = 0; u < kRangeVec; ++u) {
            const uint64_t i = base + (uint64_t)u * kRangeThreads;
            if (i < n4) minmax4(load4<STRIDED>(x, lo, 4 * i), mn[u & 3], mx[u & 3]);
        }
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x < (n & 3u))
        minmax_finite(x[elem_off<STRIDED>(lo, 4 * n4 + threadIdx.x)], mn[1], mx[1]);
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
        for (int w = 1; w < kRangeThreads / kWave; ++w) {
            a = fminf(a, s_mn[w]);
            b = fmaxf(b, s_mx[w]);
        }
        part[2 * blockIdx.x] = a;
        part[2 * blockIdx.x + 1] = b;
    }
}

template <bool STRIDED>
__global__ __launch_bounds__(kRangeThreads) void range_partial_kernel(Fields fs, uint64_t n, Layout lo,
                                                                      Workspace ws) {
    const uint32_t f = blockIdx.y;
    range_partial_body<STRIDED>(reinterpret_cast<const float *>(pick(fs.src, f)), n, lo,
                                lane_ws(ws, f, fs.ws_stride).range_part);
}

/* K1b: one workgroup folds the per-workgroup partials and resolves the bound. */
__device__ __forceinline__ void range_resolve_body(const float *__restrict__ part,
                                                   uint32_t nparts, DevInfo *info,
                                                   double eps) {
    if (nparts == 0) {
        /* an absolute bound: the same rule with a range of exactly 1 (eps * 1.0 = eps) */
        if (threadIdx.x == 0) resolve_bound(0.0f, 1.0f, eps, info);
        return;
    }
    __shared__ float s_mn[kScanThreads / kWave], s_mx[kScanThreads / kWave];
    float a = INFINITY, b = -INFINITY;
    /* kResolveBatch partials per thread in flight before any is folded (min and max do not
     * depend on the order) */
    const float2 *p2 = reinterpret_cast<const float2 *>(part);
    for (uint32_t i0 = threadIdx.x; i0 < nparts; i0 += kResolveBatch * kScanThreads) {
        float2 v[kResolveBatch];
#pragma unroll
        for (int u = 0; u < kResolveBatch; ++u) {
            const uint32_t i = i0 + (uint32_t)u * kScanThreads;
            v[u] = i < nparts ? p2[i] : make_float2(INFINITY, -INFINITY);
        }
#pragma unroll
        for (int u = 0; u < kResolveBatch; ++u) {
            a = fminf(a, v[u].x);
            b = fmaxf(b, v[u].y);
        }
    }
    for (int o = 32; o >= 1; o >>= 1) {
        a = fminf(a, __shfl_xor(a, o));
        b = fmaxf(b, __shfl_xor(b, o));
    }
    const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) { s_mn[wave] = a; s_mx[wave] = b; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kScanThreads / kWave; ++w) {
            a = fminf(a, s_mn[w]);
            b = fmaxf(b, s_mx[w]);
        }
        resolve_bound(a, b, eps, info);
    }
}

__global__ __launch_bounds__(kScanThreads) void range_resolve_kernel(Fields fs, Workspace ws, uint32_t nparts,
                                                                     double eps) {
    const Workspace w = lane_ws(ws, blockIdx.y, fs.ws_stride);
    range_resolve_body(w.range_part, nparts, w.info, eps);
}

/* ---- K2: fused encode ------------------------------------------------------------------------ */

/* Per-wave totals of the chunk being encoded. */
struct EncState {
    uint32_t words;   /* payload words of the chunk */
    uint32_t escs;    /* escapes in the chunk */
    uint32_t tmask;   /* tiles with at least one escape */
};

/* OR over the kSegLanes lanes (4 or 8, aligned) holding one 32-value segment on compress. */
__device__ __forceinline__ uint32_t seg_or(uint32_t v) {
    v |= dpp<kDppQuadXor1>(0, v);
    v |= dpp<kDppQuadXor2>(0, v);
    if (kSegLanes == 8) v |= dpp<kDppRowHalfMirror>(0, v);
    return v;
}

/* Number of significant bits of v (0 for 0): v_ffbh_u32 gives the leading-zero count, or
 * 0xffffffff for 0, and 32 minus it with unsigned saturation is the bit length. */
__device__ __forceinline__ uint32_t bit_length(uint32_t v) {
    uint32_t lz, w;
    asm("v_ffbh_u32 %0, %1" : "=v"(lz) : "v"(v));
    asm("v_sub_u32_e64 %0, 32, %1 clamp" : "=v"(w) : "v"(lz));
    return w;
}

/* The full quantization rule for the values of one encode tile that missed the fast test (bit k
 * of `slow`: value k of the lane), and the tile's escapes: per-segment bitmask (value V j + k of
 * the segment), the chunk's first kEscStage escapes staged as (index, bits) in index order, and
 * the count.  e0 is the lane's first value index. */
__device__ __forceinline__ void slow_tile(const float xs[kEncLaneVals], uint32_t slow, uint64_t e0,
                                          const QParams &qp, int t, uint32_t *emask_tile,
                                          uint32_t *stage_idx, uint32_t *stage_val,
                                          int32_t q[kEncLaneVals], EncState &st) {
    constexpr int V = kEncLaneVals;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t j = lane & (kSegLanes - 1);
    /* A rounded code above 2^T in magnitude (or NaN) escapes whatever the bound test and its
     * neighbour give: the neighbour is at least 2^T too.  Such values skip the full rule; the
     * rest of the missed values (near a cell boundary, or exactly 2^T) run it. */
    uint32_t esc = 0, full = 0;
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const bool sure = !(fabsf(rintf(xs[k] * qp.r)) <= qp.tlim);
        esc |= (((slow >> k) & 1u) && sure ? 1u : 0u) << k;
        full |= (((slow >> k) & 1u) && !sure ? 1u : 0u) << k;
    }
#pragma unroll
    for (int k = 0; k < V; ++k)
        if ((esc >> k) & 1u) q[k] = 0;
    if (__ballot(full != 0)) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            if ((full >> k) & 1u) {
                uint32_t e;
                q[k] = quantize_slow(xs[k], rintf(xs[k] * qp.r), qp, &e);
                esc |= e << k;
            }
        }
    }
    if (__ballot(esc != 0)) {
        const uint32_t segm = seg_or(esc << (V * j));
        if (j == 0) emask_tile[lane / kSegLanes] = segm;
        const uint32_t ecnt = (uint32_t)__popc(esc);
        const uint32_t eincl = wave_incl_scan(ecnt);
        uint32_t r = st.escs + eincl - ecnt;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            if ((esc >> k) & 1u) {
                if (r < (uint32_t)kEscStage) {
                    stage_idx[r] = (uint32_t)(e0 + k);
                    stage_val[r] = __float_as_uint(xs[k]);
                }
                ++r;
            }
        }
        st.escs += readlane(eincl, 63);
        st.tmask |= 1u << t;
    }
}

/* Lorenzo delta of one tile's codes against the previous value (the previous lane's last value
 * by wave_shr, the previous tile's through `carry`, 0 when `reset`), zigzag; codes past n are 0.
 * Writes the zigzag codes to z and returns the bit width of the lane's 32-value segment, or 0
 * without WIDTH (centering changes a block's first code first). */
template <bool FULL, bool WIDTH>
__device__ __forceinline__ uint32_t finish_tile(const int32_t q[kEncLaneVals], uint64_t e0, uint64_t n, bool reset,
                                                int32_t &carry, uint32_t z[kEncLaneVals]) {
    constexpr int V = kEncLaneVals;
    const int32_t prev = (int32_t)dpp<kDppWaveShr1>((uint32_t)carry, (uint32_t)q[V - 1]);
    z[0] = zigzag(reset ? q[0] : q[0] - prev);
#pragma unroll
    for (int k = 1; k < V; ++k) z[k] = zigzag(q[k] - q[k - 1]);
    carry = (int32_t)readlane((uint32_t)q[V - 1], 63);
    if (!FULL) {
#pragma unroll
        for (int k = 0; k < V; ++k)
            if (e0 + k >= n) z[k] = 0;
    }
    if (!WIDTH) return 0;
    /* segment width: bit length of the OR of its 32 codes */
    uint32_t orv = z[0];
#pragma unroll
    for (int k = 1; k < V; ++k) orv |= z[k];
    return bit_length(seg_or(orv));
}

/* A lane's code sum in two exact halves (the low 16 bits of each code, and the rest), for
 * centering sums that may pass 32 bits. */
__device__ __forceinline__ void split_sum(const int32_t q[kEncLaneVals], uint32_t &slo, int32_t &shi) {
    slo = 0;
    shi = 0;
#pragma unroll
    for (int k = 0; k < kEncLaneVals; ++k) {
        slo += (uint32_t)q[k] & 0xFFFFu;
        shi += q[k] >> 16;
    }
}

/* OR n consecutive codes of width w, already joined into `bits` (code k at bit k w), into the
 * LDS payload at bit position pos: the bits land in at most two words. */
__device__ __forceinline__ void or_bits(uint32_t *pay, uint32_t pos, uint32_t bits) {
    const uint64_t sh = (uint64_t)bits << (pos & 31u);
    uint32_t *p = pay + (pos >> 5);
    lds_or(p, (uint32_t)sh);
    lds_or(p + 1, (uint32_t)(sh >> 32));
}

/* OR one lane's kEncLaneVals codes of width w into the chunk's LDS payload; code k of the lane
 * sits at bit bit0 + k w (little-endian words, low bits first).  Codes are first joined into
 * registers of at most 32 bits -- four at a time up to width 8, two up to width 16, else one --
 * and each register lands in at most two words.  Only a lane's first and last word can be
 * shared with its neighbours, hence the OR. */
__device__ __forceinline__ void pack_lane(const uint32_t z[kEncLaneVals], uint32_t w, uint32_t bit0,
                                          uint32_t *pay) {
    if (w > 16) {
#pragma unroll
        for (int k = 0; k < kEncLaneVals; ++k) or_bits(pay, bit0 + (uint32_t)k * w, z[k]);
    } else if (w > 8) {
#pragma unroll
        for (int k = 0; k < kEncLaneVals; k += 2) or_bits(pay, bit0 + (uint32_t)k * w, z[k] | (z[k + 1] << w));
    } else if (w != 0) {
#pragma unroll
        for (int k = 0; k < kEncLaneVals; k += 4) {
            const uint32_t joined = z[k] | (z[k + 1] << w) | (z[k + 2] << (2 * w)) | (z[k + 3] << (3 * w));
            or_bits(pay, bit0 + (uint32_t)k * w, joined);
        }
    }
}

/* Bit width of the segment (kSegLanes lanes) holding a lane's codes. */
__device__ __forceinline__ uint32_t seg_width(const uint32_t z[kEncLaneVals]) {
    uint32_t orv = z[0];
#pragma unroll
    for (int k = 1; k < kEncLaneVals; ++k) orv |= z[k];
    return bit_length(seg_or(orv));
}

/* Sum over aligned groups of seglen lanes (8, 16, 32 or 64), returned in every lane of the
 * group: DPP butterflies inside rows, ds_swizzle across the two rows of a half, readlane across
 * the halves. */
__device__ __forceinline__ uint32_t seg_allsum(uint32_t v, uint32_t seglen) {
    v += dpp<kDppQuadXor1>(0, v);
    v += dpp<kDppQuadXor2>(0, v);
    v += dpp<kDppRowHalfMirror>(0, v);
    if (seglen >= 16) v += dpp<kDppRowMirror>(0, v);
    if (seglen >= 32) v += (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
    if (seglen >= 64) v = readlane(v, 0) + readlane(v, 32);
    return v;
}

/* Lorenzo centering: the mean of a block's c codes rounded half up, floor((2 S + c) / (2 c)),
 * from S = hi * 2^16 + lo; an arithmetic shift when c is a power of two (a whole block of a
 * power-of-two B).  block_mean32 is the same for |S| < 2^29 (codes below 2^T with
 * T + log2 B <= 29), in 32-bit arithmetic. */
__device__ __forceinline__ int32_t block_mean32(int32_t S, uint32_t c) {
    const int32_t num = 2 * S + (int32_t)c;
    if ((c & (c - 1u)) == 0) return num >> (__builtin_ctz(c) + 1);
    const int32_t den = 2 * (int32_t)c;
    int32_t qd = num / den;
    if ((num % den) != 0 && num < 0) qd -= 1;
    return qd;
}

__device__ __forceinline__ int32_t block_mean(uint32_t lo, int32_t hi, uint64_t c) {
    const int64_t num = 2 * ((int64_t)hi * 65536 + (int64_t)lo) + (int64_t)c;
    if ((c & (c - 1u)) == 0) return (int32_t)(num >> (__builtin_ctzll(c) + 1));
    const int64_t den = 2 * (int64_t)c;
    int64_t qd = num / den;
    if ((num % den) != 0 && num < 0) qd -= 1;
    return (int32_t)qd;
}

/* Centering modes of the encoder: none; blocks shorter than a tile whose code sums fit 32 bits
 * (B < 256 and T + log2 B <= 29); any power-of-two block; any block that is not a power of two;
 * blocks of exactly one tile whose sums fit 32 bits (B = 256, the default, and T <= 21), whose
 * sum and mean are wave-uniform.  The tile modes keep neither the per-tile totals nor the
 * 64-bit mean of the others, and so fewer registers. */
constexpr int kCenterOff = 0, kCenterTile = 1, kCenterAny = 2, kCenterGen = 3, kCenterWhole = 4;

/* Where the Lorenzo blocks lie relative to an encode chunk (wave-uniform).  For a block B that
 * is not a power of two, r0 is the chunk start's offset in its block, bk0 the block holding the
 * chunk's first value, and mB = floor(2^32 / B) + 1, so that a / B is the high word of a mB for
 * the small a (below 2^13) the chunk's offsets take. */
struct BlockPos {
    uint32_t B, log2B, r0, bk0, mB;
};

/* The code a value gets from the encoder: the fast test, else the full rule; 0 if it escapes. */
__device__ __forceinline__ int32_t code_of(float xv, const QParams &qp) {
    const float q0f = rintf(xv * qp.r);
    if ((fabsf(xv - q0f * qp.s) <= qp.eb) && (fabsf(q0f) < qp.tlim)) return (int32_t)q0f;
    uint32_t e;
    const int32_t q = quantize_slow(xv, q0f, qp, &e);
    return e ? 0 : q;
}

/* One encode chunk of kEncTiles tiles.  Pass 1 codes every tile and records the segment widths
 * in LDS (the codes stay in VGPRs); one wave scan of the widths gives every segment's word
 * offset in the chunk; pass 2 packs each tile at those offsets.  `carry` is the code of the
 * value before the chunk when the chunk does not start a Lorenzo block.  GB: the block is not a
 * power of two, so a lane starts a block when (r0 + 256 t + 4 lane) mod B is 0. */
template <bool FULL, bool STRIDED, int CM, bool GB>
__device__ __forceinline__ void encode_chunk(const float *__restrict__ x, const Layout &lo, uint64_t cbase, uint64_t n,
                                             const QParams &qp, const BlockPos &bp, int32_t carry,
                                             uint32_t *pay, uint8_t *wid, uint32_t *emask_chunk,
                                             uint32_t *stage_idx, uint32_t *stage_val, EncState &st,
                                             int32_t *__restrict__ means, bool narrow,
                                             uint32_t *__restrict__ slot, bool slot_nt) {
    const uint32_t bmask = bp.B - 1, log2B = bp.log2B;
    constexpr int V = kEncLaneVals;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t j = lane & (kSegLanes - 1), g = lane / kSegLanes;
    float xs[kEncTiles][V];
    if (FULL) {
#pragma unroll
        for (int t = 0; t < kEncTiles; ++t) {
#pragma unroll
            for (int h = 0; h < V / 4; ++h) {
                const float4 a = load4<STRIDED>(x, lo, cbase + (uint64_t)t * kEncTile + V * lane + 4 * h);
                xs[t][4 * h] = a.x; xs[t][4 * h + 1] = a.y; xs[t][4 * h + 2] = a.z; xs[t][4 * h + 3] = a.w;
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < kEncTiles; ++t) {
            const uint64_t e = cbase + (uint64_t)t * kEncTile + V * lane;
#pragma unroll
            for (int k = 0; k < V; ++k) xs[t][k] = e + k < n ? x[elem_off<STRIDED>(lo, e + k)] : 0.0f;
        }
    }
    const uint32_t ntiles = FULL ? kEncTiles : (uint32_t)((n - cbase + kEncTile - 1) / kEncTile);
    /* a lane's first value starts a block when its offset in the tile does and the tile does
     * (a power-of-two block) */
    const bool lane_at_block = ((V * lane) & bmask) == 0;
    uint32_t z[kEncTiles][V];
    uint32_t w[kEncTiles];
    /* Quantize: rint(x inv2eb) is kept when its reconstruction is within eb and the code is below
     * 2^T.  This is the full rule's first acceptance exactly: its extra clause |x| >= |y|/2
     * cannot fail here.  For q0 = 0 it is trivial; for |q0| >= 2, |y| >= 4 eb and a rounded
     * |x - y| <= eb forces |x - y| <= 2 eb; for |q0| = 1, rint gives 1 only when f32(x r) > 1/2,
     * which with r within 2^-24 of 1/(2 eb) puts x above the largest float below eb.  NaN fails
     * the eb test, infinities the 2^T test.  Every tile is tested first, without branches; the
     * full rule runs only in a wave where some value missed the test. */
    int32_t q[kEncTiles][V];
    /* tested in groups of kTestGroup tiles: a lane passes when all its values are within eb
     * and its largest |code| is below 2^T; a wave with a failing lane re-tests value by value
     * and runs the full rule where needed */
    constexpr int kTestGroup = 2;
#pragma unroll
    for (int t0 = 0; t0 < kEncTiles; t0 += kTestGroup) {
        bool lane_fast = true;
#pragma unroll
        for (int t = t0; t < t0 + kTestGroup; ++t) {
            float qabs = 0.0f;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float q0f = rintf(xs[t][k] * qp.r);
                lane_fast = lane_fast && (fabsf(xs[t][k] - q0f * qp.s) <= qp.eb);
                qabs = fmaxf(qabs, fabsf(q0f));
                q[t][k] = (int32_t)q0f;
            }
            lane_fast = lane_fast && (qabs < qp.tlim);
        }
        if (__ballot(!lane_fast)) {
#pragma unroll
            for (int t = t0; t < t0 + kTestGroup; ++t) {
                uint32_t ts = 0; /* bit k: value k missed the test */
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float q0f = rintf(xs[t][k] * qp.r);
                    const bool ok = (fabsf(xs[t][k] - q0f * qp.s) <= qp.eb) && (fabsf(q0f) < qp.tlim);
                    ts |= (ok ? 0u : 1u) << k;
                }
                if ((FULL || (uint32_t)t < ntiles) && __ballot(ts != 0))
                    slow_tile(xs[t], ts, cbase + (uint64_t)t * kEncTile + V * lane, qp, t,
                              emask_chunk + t * kSegsPerEncTile, stage_idx, stage_val, q[t], st);
            }
        }
    }
    /* Lorenzo centering: a block's first code was coded against 0 (z = zigzag(q)); it is
     * recoded against the block's mean code, which goes to the means staging, and the segment
     * widths follow.  A power-of-two block lies inside the chunk (B <= 2048): one of at most one
     * tile is finished with its tile; a longer one keeps its tiles' wave-uniform code sums until
     * the tile loop ends.  Any other block (kCenterGen) may cross the chunk's ends: the tile loop
     * keeps a chunk-wide prefix of the lanes' code sums in the pack buffer (unused until pass 2),
     * and the blocks are finished after it. */
    const uint32_t B = bp.B;
    const bool in_tile = B <= (uint32_t)kEncTile;
    uint32_t tlo[kEncTiles];
    int32_t thi[kEncTiles];
    uint32_t run_lo = 0, run_hi = 0;
    uint32_t *pre_lo = pay, *pre_hi = pay + kEncTiles * kWave;
#pragma unroll
    for (int t = 0; t < kEncTiles; ++t) {
        tlo[t] = 0;
        thi[t] = 0;
        if (FULL || (uint32_t)t < ntiles) {
            bool reset;
            if (GB) {
                const uint32_t a = bp.r0 + (uint32_t)t * kEncTile + V * lane;
                reset = a == __umulhi(a, bp.mB) * B;
            } else {
                reset = lane_at_block && (((uint32_t)cbase + (uint32_t)t * kEncTile) & bmask) == 0;
            }
            /* a block inside the tile changes its first code before the segment width is taken */
            constexpr bool kTileBlocks = CM == kCenterTile || CM == kCenterWhole;
            constexpr bool kWholeTile = CM == kCenterWhole;
            w[t] = finish_tile<FULL, !kTileBlocks>(q[t], cbase + (uint64_t)t * kEncTile + V * lane, n, reset, carry,
                                                   z[t]);
            uint32_t slo = 0;
            int32_t shi = 0;
            if (CM == kCenterAny || CM == kCenterGen) split_sum(q[t], slo, shi);
            if (kTileBlocks || (CM == kCenterAny && in_tile)) {
                const uint32_t seglen = B / V; /* lanes per block */
                /* narrow codes: one exact 32-bit sum (the codes' sum wraps exactly); else the two
                 * halves */
                const bool narrow_sums = kTileBlocks || narrow;
                uint32_t lo_s, hi_s = 0;
                if (kTileBlocks) {
                    uint32_t s32 = 0;
#pragma unroll
                    for (int k = 0; k < V; ++k) s32 += (uint32_t)q[t][k];
                    if (kWholeTile) {
                        /* the tile is the block: its sum, mean and recoded first code are
                         * wave-uniform, and only lane 0's first code changes.  Segment 0's OR
                         * leaves that code out and takes the recoded one. */
                        const uint32_t S = wave_sum(s32);
                        const uint64_t b0 = cbase + (uint64_t)t * kEncTile;
                        uint32_t orv = z[t][1] | z[t][2] | z[t][3] | (lane == 0 ? 0u : z[t][0]);
                        orv = seg_or(orv);
                        if (FULL || b0 < n) {
                            const uint32_t c = (FULL || n - b0 >= (uint64_t)B) ? B : (uint32_t)(n - b0);
                            const int32_t mu = block_mean32((int32_t)S, c);
                            const uint32_t z0 = zigzag((int32_t)(readlane((uint32_t)q[t][0], 0) - (uint32_t)mu));
                            if (lane == 0) {
                                z[t][0] = z0;
                                means[b0 >> log2B] = mu;
                            }
                            if (lane < (uint32_t)kSegLanes) orv |= z0;
                        }
                        w[t] = bit_length(orv);
                        if (j == 0) wid[t * kSegsPerEncTile + g] = (uint8_t)w[t];
                        continue;
                    }
                    lo_s = seg_allsum(s32, seglen);
                } else if (narrow_sums) {
                    lo_s = seg_allsum(slo + ((uint32_t)shi << 16), seglen);
                } else {
                    lo_s = seg_allsum(slo, seglen);
                    hi_s = seg_allsum((uint32_t)shi, seglen);
                }
                const uint64_t e0 = cbase + (uint64_t)t * kEncTile + V * lane;
                if (lane_at_block && e0 < n) {
                    /* a whole block (every block of a full chunk) has c = B, a power of two */
                    const uint64_t c = (FULL || n - e0 >= (uint64_t)B) ? (uint64_t)B : n - e0;
                    const int32_t mu = narrow_sums ? block_mean32((int32_t)lo_s, (uint32_t)c)
                                                   : block_mean(lo_s, (int32_t)hi_s, c);
                    /* the block's first code, coded against its mean instead of 0 */
                    z[t][0] = zigzag((int32_t)((uint32_t)q[t][0] - (uint32_t)mu));
                    means[e0 >> log2B] = mu;
                }
                w[t] = seg_width(z[t]);
            } else if (CM == kCenterAny) {
                tlo[t] = seg_allsum(slo, 64);
                thi[t] = (int32_t)seg_allsum((uint32_t)shi, 64);
            } else if (CM == kCenterGen) {
                /* inclusive prefix over the chunk's lanes (wrapping u32 sums: every block's
                 * difference of two prefixes is far inside the 32-bit range) */
                const uint32_t il = wave_incl_scan(slo) + run_lo;
                const uint32_t ih = wave_incl_scan((uint32_t)shi) + run_hi;
                pre_lo[t * kWave + lane] = il;
                pre_hi[t * kWave + lane] = ih;
                run_lo = readlane(il, 63);
                run_hi = readlane(ih, 63);
            }
            if (j == 0) wid[t * kSegsPerEncTile + g] = (uint8_t)w[t];
        }
    }
    if (CM == kCenterAny && !in_tile) {
        /* blocks of B / 256 tiles: each block's sum from its tiles' totals, at its first tile */
        const uint32_t tpb = B / kEncTile;
#pragma unroll
        for (int t = 0; t < kEncTiles; ++t) {
            const uint64_t bstart = cbase + (uint64_t)t * kEncTile;
            if (((uint32_t)(t * kEncTile) & bmask) == 0 && bstart < n) {
                uint32_t lo_s = 0;
                int32_t hi_s = 0;
#pragma unroll
                for (int t2 = t; t2 < kEncTiles; ++t2) {
                    if ((uint32_t)t2 < (uint32_t)t + tpb) {
                        lo_s += tlo[t2];
                        hi_s += thi[t2];
                    }
                }
                const uint64_t c = (n - bstart < (uint64_t)B) ? n - bstart : (uint64_t)B;
                const int32_t mu = block_mean(lo_s, hi_s, c);
                if (lane == 0) {
                    z[t][0] = zigzag((int32_t)((uint32_t)unzigzag(z[t][0]) - (uint32_t)mu));
                    means[bstart >> log2B] = mu;
                }
                w[t] = seg_width(z[t]);
                if (j == 0) wid[t * kSegsPerEncTile + g] = (uint8_t)w[t];
            }
        }
    }
    if (CM == kCenterGen) {
        wave_lds_sync();
        /* The last block starting in the chunk may run on past it: its codes there are coded
         * again here, by the same rule (an escape counts 0), to complete its sum.  Block starts
         * lie on 32-value boundaries, so a lane's four values are all inside the block or all
         * outside it; only n can cut them. */
        uint32_t look_lo = 0, look_hi = 0;
        const uint32_t f0 = bp.r0 == 0 ? 0u : B - bp.r0; /* first block start in the chunk */
        if (f0 < (uint32_t)kEncChunk) {
            const uint32_t last = f0 + B * __umulhi((uint32_t)kEncChunk - 1u - f0, bp.mB);
            const uint64_t bend = cbase + last + B;
            const uint64_t end = bend < n ? bend : n;
            if (end > cbase + kEncChunk) {
                for (uint64_t i = cbase + kEncChunk + V * lane; i < end; i += kEncTile) {
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        if (i + k < end) {
                            const int32_t qv = code_of(x[elem_off<STRIDED>(lo, i + k)], qp);
                            look_lo += (uint32_t)qv & 0xFFFFu;
                            look_hi += (uint32_t)(qv >> 16);
                        }
                    }
                }
                look_lo = readlane(wave_incl_scan(look_lo), 63);
                look_hi = readlane(wave_incl_scan(look_hi), 63);
            }
        }
        const uint32_t last_slot = ntiles * kWave - 1u;
#pragma unroll
        for (int t = 0; t < kEncTiles; ++t) {
            if (FULL || (uint32_t)t < ntiles) {
                const uint32_t a = bp.r0 + (uint32_t)t * kEncTile + V * lane;
                const uint32_t qd = __umulhi(a, bp.mB);
                const uint64_t e0 = cbase + (uint64_t)t * kEncTile + V * lane;
                if (a == qd * B && e0 < n) {
                    const uint32_t u0 = (uint32_t)t * kWave + lane;
                    const uint32_t ue = u0 + B / V - 1u;
                    const uint32_t uc = ue < last_slot ? ue : last_slot;
                    uint32_t lo_s = pre_lo[uc] - (u0 ? pre_lo[u0 - 1] : 0u);
                    uint32_t hi_s = pre_hi[uc] - (u0 ? pre_hi[u0 - 1] : 0u);
                    if (ue > last_slot) {
                        lo_s += look_lo;
                        hi_s += look_hi;
                    }
                    const uint64_t c = (n - e0 < (uint64_t)B) ? n - e0 : (uint64_t)B;
                    const int32_t mu = block_mean(lo_s, (int32_t)hi_s, c);
                    z[t][0] = zigzag((int32_t)((uint32_t)unzigzag(z[t][0]) - (uint32_t)mu));
                    means[bp.bk0 + qd] = mu;
                }
                w[t] = seg_width(z[t]);
                if (j == 0) wid[t * kSegsPerEncTile + g] = (uint8_t)w[t];
            }
        }
    }
    wave_lds_sync();
    const uint32_t wl = lane < (uint32_t)kEncSegs ? (uint32_t)wid[lane] : 0u;
    const uint32_t incl = wave_incl_scan(wl);
    const uint32_t excl = incl - wl;
    st.words = readlane(incl, kEncSegs - 1);
    /* Pass 2: pack into the LDS buffer (kEncPayWords words), then 128-bit stores to the slot.
     * A chunk whose words do not fit is packed in two halves (tiles 0-3, then 4-7): segments
     * hold whole words, so the halves share none.  Only the words used are cleared. */
    const uint32_t total = st.words;
    const uint32_t half = readlane(incl, kEncSegs / 2 - 1);
    const bool one_pass = total + 1 <= (uint32_t)kEncPayWords;
    uint32_t offs[kEncTiles];
#pragma unroll
    for (int t = 0; t < kEncTiles; ++t)
        offs[t] = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((t * kSegsPerEncTile + g) * 4), (int)excl);
    uint4 *pay4 = reinterpret_cast<uint4 *>(pay);
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h == 1 && one_pass) break;
        const uint32_t w0 = (one_pass || h == 0) ? 0u : half;                 /* first word of the pass */
        const uint32_t nw = one_pass ? total : (h == 0 ? half : total - half); /* words of the pass */
        for (uint32_t i = lane; i < (nw + 4) / 4; i += kWave) pay4[i] = zero4;
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < kEncTiles; ++t) {
            const bool mine = one_pass || (h == 0 ? t < kEncTiles / 2 : t >= kEncTiles / 2);
            if ((FULL || (uint32_t)t < ntiles) && mine)
                pack_lane(z[t], w[t], 32u * (offs[t] - w0) + (uint32_t)V * w[t] * j, pay);
        }
        wave_lds_sync();
        if (w0 == 0) {
            uint4 *dst = reinterpret_cast<uint4 *>(slot);
            if (slot_nt) {
                for (uint32_t i = lane; i < (nw + 3) / 4; i += kWave) st_nt(dst + i, pay4[i]);
            } else {
                for (uint32_t i = lane; i < (nw + 3) / 4; i += kWave) dst[i] = pay4[i];
            }
        } else {
            for (uint32_t i = lane; i < nw; i += kWave) slot[w0 + i] = pay[i];
        }
        wave_lds_sync();
    }
}

constexpr uint64_t kSlotCacheBytes = 128ull << 20;

/* One wave per encode chunk, kEncWaves chunks per workgroup.  Outputs per chunk: its packed
 * words in its scratch slot, its width bytes (into the stream, or into staging when the output
 * buffer cannot hold them), its word and escape counts and, for a chunk with more escapes than
 * the staging holds, the escape bitmask of every tile with an escape; per workgroup, the sums
 * the device-wide scan runs over. */
template <bool STRIDED, int CM, bool GB>
__device__ __forceinline__ void encode_body(
    const float *__restrict__ x, PlanArgs pa, Workspace ws, uint8_t *__restrict__ widths_dst,
    uint64_t widths_bytes, uint32_t grp) {
    __shared__ uint4 s_pay4[kEncWaves][kEncPayWords / 4];
    __shared__ uint4 s_wid4[kEncWaves][kEncSegs / 16];
    __shared__ uint32_t s_stage[kEncWaves][2][kEscStage];
    __shared__ uint32_t s_emask[kEncWaves][kEncSegs];
    __shared__ uint32_t s_grp[2][kEncWaves];

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t c = grp * kEncWaves + wave;
    const DevInfo *info = ws.info;
    EncState st = {0, 0, 0};

    if (c < pa.nchunks && info->valid) {
        /* The scratch slots take plain stores, so the compaction finds them in the 256 MB
         * last-level cache, unless the fields of this launch wrote more than kSlotCacheBytes of
         * payload on their lanes' previous calls: payloads that large do not stay there, and
         * non-temporal stores then write them faster (the stream does not depend on this). */
        const bool slot_nt = (uint64_t)gridDim.y * info->payload_words * 4u > kSlotCacheBytes;
        QParams qp;
        qp.eb = info->eb_f;
        qp.s = info->s;
        qp.r = info->r;
        qp.T = pa.T;
        qp.tlim = (float)(1u << pa.T);
        uint32_t *pay = reinterpret_cast<uint32_t *>(s_pay4[wave]);
        uint8_t *wid = reinterpret_cast<uint8_t *>(s_wid4[wave]);
        if (lane < kEncSegs / 16) s_wid4[wave][lane] = make_uint4(0, 0, 0, 0);
        wave_lds_sync();
        const uint64_t cbase = (uint64_t)c * kEncChunk;
        BlockPos bp;
        bp.B = pa.B;
        bp.log2B = pa.log2B;
        bp.r0 = 0;
        bp.bk0 = 0;
        bp.mB = 0;
        if (GB) {
            bp.bk0 = (uint32_t)cbase / pa.B;
            bp.r0 = (uint32_t)cbase - bp.bk0 * pa.B;
            bp.mB = 0xFFFFFFFFu / pa.B + 1u;
        }
        const bool at_block = GB ? bp.r0 == 0 : ((uint32_t)cbase & (pa.B - 1)) == 0;
        /* centering: a block's code sum fits 32 bits (|S| < 2^29) when codes stay below 2^T */
        const bool narrow = pa.T + pa.log2B <= 29;
        /* Lorenzo predecessor of the chunk's first value: 0 at a block start, else the code of
         * the value before the chunk (0 if that value escapes) */
        int32_t carry = 0;
        if (!at_block) carry = code_of(x[elem_off<STRIDED>(pa.lay, cbase - 1)], qp);
        uint32_t *emask_chunk = s_emask[wave];
        uint32_t *stage_idx = s_stage[wave][0];
        uint32_t *stage_val = s_stage[wave][1];
        if (cbase + kEncChunk <= pa.n)
            encode_chunk<true, STRIDED, CM, GB>(x, pa.lay, cbase, pa.n, qp, bp, carry, pay, wid, emask_chunk,
                                                stage_idx, stage_val, st, ws.means, narrow, ws.scratch + cbase,
                                                slot_nt);
        else
            encode_chunk<false, STRIDED, CM, GB>(x, pa.lay, cbase, pa.n, qp, bp, carry, pay, wid, emask_chunk,
                                                 stage_idx, stage_val, st, ws.means, narrow, ws.scratch + cbase,
                                                 slot_nt);
        /* widths -> stream (or staging) */
        if (lane < kEncSegs / 16) {
            const uint64_t off = (uint64_t)c * kEncSegs + 16u * lane;
            if (off < widths_bytes) *reinterpret_cast<uint4 *>(widths_dst + off) = s_wid4[wave][lane];
        }
        if (lane < st.escs && lane < (uint32_t)kEscStage) {
            ws.stage_idx[(uint64_t)c * kEscStage + lane] = stage_idx[lane];
            ws.stage_val[(uint64_t)c * kEscStage + lane] = stage_val[lane];
        }
        /* the escape bitmasks of the tiles with escapes, gathered in LDS: the compaction reads
         * them only for a chunk with more escapes than the staging holds */
        if (st.escs > (uint32_t)kEscStage && ((st.tmask >> (lane / kSegsPerEncTile)) & 1u))
            ws.emask[(uint64_t)c * kEncSegs + lane] = emask_chunk[lane];
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
        uint32_t sw = 0, se = 0;
#pragma unroll
        for (int k = 0; k < kEncWaves; ++k) {
            sw += s_grp[0][k];
            se += s_grp[1][k];
        }
        ws.group_words[grp] = sw;
        ws.group_esc[grp] = se;
    }
}

/* The encoder walks a field's groups from the last to the first: the range pass has just read
 * them first to last, so the workgroups dispatched first find the tail of the input in the
 * last-level cache. */
template <bool STRIDED, int CM, bool GB>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    const uint32_t f = blockIdx.y;
    const Workspace w = lane_ws(ws, f, fs.ws_stride);
    uint8_t *wd = (fs.wdirect >> f) & 1u ? pick(fs.dst, f) + kHeaderBytes : w.widths;
    encode_body<STRIDED, CM, GB>(reinterpret_cast<const float *>(pick(fs.src, f)), pa, w, wd, pa.wsec,
                             pa.ngroups - 1 - blockIdx.x);
}

/* ---- K3: single-workgroup exclusive scan over groups ---------------------------------------- */

/* Exclusive prefix of a[0..ng) and b[0..ng) at every kSuperGroups-th item, into pa_out /
 * pb_out at index item / kSuperGroups; returns the totals in tot[0], tot[1] (valid in every
 * thread).  Each round covers kScanThreads * kScanItems items: a thread loads 16 consecutive
 * items with 128-bit loads (the arrays are 256-byte aligned), sums them, the sums are scanned
 * across the wave with DPP and across the 16 waves through LDS, and the thread holding a
 * super-group's first item writes its prefix. */
__device__ void block_scan2(const uint32_t *__restrict__ a, const uint32_t *__restrict__ b,
                            uint32_t *__restrict__ pa_out, uint32_t *__restrict__ pb_out,
                            uint32_t ng, uint32_t *tot) {
    static_assert(kSuperGroups % kScanItems == 0, "a thread's items lie in one super-group");
    constexpr int kWaves = kScanThreads / kWave;
    constexpr int kV = kScanItems / 4;
    __shared__ uint32_t s_wa[kWaves], s_wb[kWaves];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t carry_a = 0, carry_b = 0;
    for (uint32_t base = 0; base < ng; base += kScanThreads * kScanItems) {
        const uint32_t i0 = base + kScanItems * tid;
        uint32_t va[kScanItems], vb[kScanItems];
        if (i0 + kScanItems <= ng) {
#pragma unroll
            for (int k = 0; k < kV; ++k) {
                const uint4 t = reinterpret_cast<const uint4 *>(a + i0)[k];
                va[4 * k] = t.x; va[4 * k + 1] = t.y; va[4 * k + 2] = t.z; va[4 * k + 3] = t.w;
                const uint4 u = b != nullptr ? reinterpret_cast<const uint4 *>(b + i0)[k] : make_uint4(0, 0, 0, 0);
                vb[4 * k] = u.x; vb[4 * k + 1] = u.y; vb[4 * k + 2] = u.z; vb[4 * k + 3] = u.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < kScanItems; ++k) {
                va[k] = (i0 + k < ng) ? a[i0 + k] : 0u;
                vb[k] = (b != nullptr && i0 + k < ng) ? b[i0 + k] : 0u;
            }
        }
        uint32_t ta = 0, tb = 0;
#pragma unroll
        for (int k = 0; k < kScanItems; ++k) {
            ta += va[k];
            tb += vb[k];
        }
        const uint32_t ia = wave_incl_scan(ta);
        const uint32_t ib = wave_incl_scan(tb);
        if (lane == 63) { s_wa[wave] = ia; s_wb[wave] = ib; }
        __syncthreads();
        uint32_t oa = 0, ob = 0, sa = 0, sb = 0;
#pragma unroll
        for (uint32_t w = 0; w < (uint32_t)kWaves; ++w) {
            const uint32_t xa = s_wa[w], xb = s_wb[w];
            oa += (w < wave) ? xa : 0u;
            ob += (w < wave) ? xb : 0u;
            sa += xa;
            sb += xb;
        }
        if (i0 < ng && (i0 % kSuperGroups) == 0) {
            pa_out[i0 / kSuperGroups] = carry_a + oa + ia - ta;
            if (pb_out != nullptr) pb_out[i0 / kSuperGroups] = carry_b + ob + ib - tb;
        }
        carry_a += sa;
        carry_b += sb;
        __syncthreads();
    }
    tot[0] = carry_a;
    tot[1] = carry_b;
}

/* Where a compressed stream's sections go, from its payload words S and escapes m: RAW when
 * the bound is unusable, when more values escape than the side list holds or when the coded
 * stream would be larger than the raw one; fits when the whole stream fits the caller's cap. */
struct StreamPlace {
    bool raw;
    uint32_t fits;
    uint64_t m, pb, po, oi, ov, tot;
};

__device__ __forceinline__ StreamPlace place_stream(const PlanArgs &pa, uint64_t S, uint64_t m, bool valid,
                                                    uint64_t cap) {
    const uint64_t n = pa.n;
    const uint64_t raw_total = kHeaderBytes + align16(4 * n);
    const uint64_t payload_off = kHeaderBytes + pa.wsec + table_bytes(pa.ngroups) + pa.msec;
    const uint64_t lossy_total = payload_off + align16(4 * S) + 2 * align16(4 * m);
    StreamPlace P;
    P.raw = !valid || m > pa.side_max || lossy_total > raw_total;
    if (P.raw) {
        P.m = 0; P.pb = 4 * n; P.po = kHeaderBytes;
        P.oi = raw_total; P.ov = raw_total; P.tot = raw_total;
    } else {
        P.m = m; P.pb = 4 * S; P.po = payload_off;
        P.oi = payload_off + align16(4 * S);
        P.ov = P.oi + align16(4 * m);
        P.tot = P.ov + align16(4 * m);
    }
    P.fits = P.tot <= cap ? 1u : 0u;
    return P;
}

/* The placement as the compaction reads it back from the workspace. */
__device__ __forceinline__ StreamPlace place_from_info(const DevInfo *info) {
    StreamPlace P;
    P.raw = info->mode == 1;
    P.fits = info->fits;
    P.m = info->m;
    P.pb = 4 * info->payload_words;
    P.po = info->payload_off;
    P.oi = info->oidx_off;
    P.ov = info->oval_off;
    P.tot = info->total;
    return P;
}

/* One thread: the placement into the workspace and the caller's result record (length, or
 * the required capacity, then the status), and the 128-byte header into h. */
__device__ __forceinline__ void publish_stream(const PlanArgs &pa, const StreamPlace &P, DevInfo *info,
                                               uint64_t *result, uint32_t h[32]) {
    info->mode = P.raw ? 1u : (pa.V ? 2u : 0u);
    info->m = P.m;
    info->payload_words = P.pb / 4;
    info->payload_off = P.po;
    info->oidx_off = P.oi;
    info->oval_off = P.ov;
    info->total = P.tot;
    info->fits = P.fits;
    if (result != nullptr) {
        result[0] = P.tot;
        result[1] = P.fits ? 0u : 3u;
    }
    h[0] = kMagic;
    h[1] = kVersion | (kHeaderBytes << 16);
    h[2] = (P.raw ? 1u : (pa.V ? 2u : 0u)) | (pa.rank << 8) | (pa.log2seg << 16) | (pa.T << 24);
    h[3] = pa.B;
    for (int a = 0; a < 4; ++a) {
        h[4 + 2 * a] = (uint32_t)pa.dims[a];
        h[5 + 2 * a] = (uint32_t)(pa.dims[a] >> 32);
    }
    const uint64_t u64s[8] = {pa.n, 0, P.m, P.pb, kHeaderBytes, P.po, P.oi, P.ov};
    h[12] = (uint32_t)u64s[0];
    h[13] = (uint32_t)(u64s[0] >> 32);
    h[14] = __float_as_uint(info->eb_f);
    h[15] = __float_as_uint(info->s);
    h[16] = __float_as_uint(info->r);
    h[17] = (!P.raw && pa.center) ? 1u : 0u; /* flags: bit 0 = centered */
    for (int a = 2; a < 8; ++a) {
        h[18 + 2 * (a - 2)] = (uint32_t)u64s[a];
        h[19 + 2 * (a - 2)] = (uint32_t)(u64s[a] >> 32);
    }
    h[30] = (uint32_t)P.tot;
    h[31] = (uint32_t)(P.tot >> 32);
}

/* Compress finalize: totals -> stream layout, RAW decision, header. */
__device__ __forceinline__ void scan_compress_body(PlanArgs pa, Workspace ws,
                                                   uint8_t *out, uint64_t cap,
                                                   uint64_t *result) {
    __shared__ uint32_t s_hdr[32];
    __shared__ uint32_t s_fits;
    DevInfo *info = ws.info;
    /* the bound's validity, read before the scan so that its load overlaps it */
    const uint32_t valid0 = info->valid;
    uint32_t tot[2];
    block_scan2(ws.group_words, ws.group_esc, ws.gpre_words, ws.gpre_esc, pa.ngroups, tot);
    if (threadIdx.x == 0) {
        const StreamPlace P = place_stream(pa, tot[0], tot[1], valid0 != 0, cap);
        publish_stream(pa, P, info, result, s_hdr);
        s_fits = P.fits;
    }
    __syncthreads();
    if (s_fits && threadIdx.x < 32) reinterpret_cast<uint32_t *>(out)[threadIdx.x] = s_hdr[threadIdx.x];
}

__global__ __launch_bounds__(kScanThreads) void scan_compress_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    const uint32_t f = blockIdx.y;
    scan_compress_body(pa, lane_ws(ws, f, fs.ws_stride), pick(fs.dst, f), pick(fs.bytes, f), pick(fs.result, f));
}


/* ---- K4: compaction of the scratch slots and the ordered outliers (or the RAW copy) ------- */

/* Outliers of encode chunk c (cnt of them, from outlier rank O on), written by one wave: copied
 * from the encoder's staging when they all fit there; otherwise lane l < kEncSegs owns segment
 * l, takes its escape bitmask, ranks its escapes after O and the lanes before it, and writes
 * (index, raw bits) in ascending index order, re-reading the values from the input. */
template <bool STRIDED>
__device__ __forceinline__ void write_chunk_outliers(const float *__restrict__ x, const Layout &lo, const Workspace &ws,
                                                     uint32_t c, uint32_t cnt, uint32_t O,
                                                     uint32_t *oidx, uint32_t *oval) {
    const uint32_t lane = threadIdx.x & 63;
    if (cnt == 0) return;
    if (cnt <= (uint32_t)kEscStage) {
        /* all of the chunk's escapes were staged by the encoder, in index order */
        const uint32_t *si = ws.stage_idx + (uint64_t)c * kEscStage;
        const uint32_t *sv = ws.stage_val + (uint64_t)c * kEscStage;
        if (lane < cnt) {
            oidx[O + lane] = si[lane];
            oval[O + lane] = sv[lane];
        }
        return;
    }
    const uint32_t tm = ws.chunk_tmask[c];
    uint32_t mask = (lane < (uint32_t)kEncSegs && ((tm >> (lane / kSegsPerEncTile)) & 1u))
                        ? ws.emask[(uint64_t)c * kEncSegs + lane] : 0u;
    const uint32_t lcnt = (uint32_t)__popc(mask);
    uint32_t rank = O + wave_incl_scan(lcnt) - lcnt;
    const uint64_t segbase = (uint64_t)c * kEncChunk + 32u * lane;
    const uint32_t *xb = reinterpret_cast<const uint32_t *>(x);
    while (mask) {
        const uint32_t bit = (uint32_t)__builtin_ctz(mask);
        const uint64_t idx = segbase + bit;
        oidx[rank] = (uint32_t)idx;
        oval[rank] = xb[elem_off<STRIDED>(lo, idx)];
        ++rank;
        mask &= mask - 1;
    }
}

/* A chunk's payload of P words goes from its 16-byte aligned scratch slot to stream word Dw of
 * the (16-byte aligned) payload section.  Destination words fall into a head [Dw, bs), whole
 * 128-bit units [bs, be) and a tail [be, Dw + P), bs and be being Dw and Dw + P rounded up and
 * down to 4 words.  Head and tail words can share a 16-byte unit with the neighbouring chunks, so
 * they are stored one by one; each whole unit is assembled from two aligned source units shifted
 * by the wave-uniform word offset (bs - Dw) mod 4. */

/* Words r..r+3 of the eight words A, B (r in 0..3), by selects on the bits of r.  The empty asm
 * keeps both units whole in registers first: without it the compiler narrows the loads to the
 * words each value of r uses and moves them into per-r branches, and one such build loaded the
 * wrong word for r = 3. */
__device__ __forceinline__ uint4 shift_units(uint4 A, uint4 B, uint32_t r) {
    asm("" : "+v"(A.x), "+v"(A.y), "+v"(A.z), "+v"(A.w), "+v"(B.x), "+v"(B.y), "+v"(B.z));
    const bool odd = (r & 1u) != 0;
    const uint32_t w0 = odd ? A.y : A.x, w1 = odd ? A.z : A.y, w2 = odd ? A.w : A.z;
    const uint32_t w3 = odd ? B.x : A.w, w4 = odd ? B.y : B.x, w5 = odd ? B.z : B.y;
    return (r & 2u) != 0 ? make_uint4(w2, w3, w4, w5) : make_uint4(w0, w1, w2, w3);
}


/* The payloads of a group whose chunks are all small (at most 64 destination units each), copied
 * by one wave (chunk k from its slot src + k slot words to stream word dw[k]): the loads of every
 * chunk (both source units of each destination unit, the head and tail words) are issued before
 * the first store, so the group waits for one memory latency. */
template <int CPG>
__device__ __forceinline__ void copy_group_payload(const uint32_t *__restrict__ src, uint32_t slot,
                                                   const uint32_t words[CPG], const uint64_t dw[CPG],
                                                   uint32_t *__restrict__ pay) {
    const uint32_t lane = threadIdx.x & 63;
    uint4 A[CPG], B[CPG];
    uint32_t hv[CPG], tv[CPG];
#pragma unroll
    for (int k = 0; k < CPG; ++k) {
        const uint32_t *sk = src + (uint64_t)k * slot;
        const uint64_t De = dw[k] + words[k];
        const uint64_t bs = (dw[k] + 3) & ~(uint64_t)3, be = De & ~(uint64_t)3;
        const uint64_t head_end = bs < De ? bs : De;
        const uint64_t tail_start = be > bs ? be : bs;
        const uint32_t units = be > bs ? (uint32_t)((be - bs) >> 2) : 0u;
        const uint32_t rn = bs != dw[k] ? 1u : 0u;
        hv[k] = lane < head_end - dw[k] ? sk[lane] : 0u;
        tv[k] = tail_start < De && lane < De - tail_start ? sk[tail_start - dw[k] + lane] : 0u;
        A[k] = B[k] = make_uint4(0, 0, 0, 0);
        if (units != 0) {
            /* clamped indices: the last source unit holding a needed word is units - 1 + rn */
            const uint4 *s4 = reinterpret_cast<const uint4 *>(sk);
            A[k] = s4[min(lane, units - 1)];
            B[k] = s4[min(lane + rn, units - 1 + rn)];
        }
    }
#pragma unroll
    for (int k = 0; k < CPG; ++k) {
        const uint64_t De = dw[k] + words[k];
        const uint64_t bs = (dw[k] + 3) & ~(uint64_t)3, be = De & ~(uint64_t)3;
        const uint64_t head_end = bs < De ? bs : De;
        const uint64_t tail_start = be > bs ? be : bs;
        const uint32_t units = be > bs ? (uint32_t)((be - bs) >> 2) : 0u;
        if (lane < units) reinterpret_cast<uint4 *>(pay + bs)[lane] = shift_units(A[k], B[k], (uint32_t)(bs - dw[k]));
        if (lane < head_end - dw[k]) pay[dw[k] + lane] = hv[k];
        if (tail_start < De && lane < De - tail_start) pay[tail_start + lane] = tv[k];
    }
}

/* One round of a chunk's copy: destination units [t0, t0 + 256) of the chunk's whole units, four
 * per lane, with the source words they need; the first round also carries the head and tail
 * words.  Unit t takes source words r .. r+3 of source units t and t+1: unit t+1 comes from the
 * next lane (DPP wave_shl1), or for the last lane from the next batch's first unit, or from one
 * more unit loaded for the round. */
constexpr int kCopyBatch = 2; /* units per lane per round of a larger chunk's copy */

struct CopyRound {
    uint4 A[kCopyBatch];
    uint4 E;
    uint32_t hv, tv;
};

struct ChunkGeom {
    const uint32_t *src;
    uint64_t dw, bs, tail_start, de;
    uint32_t units, r, rn;
};

__device__ __forceinline__ ChunkGeom chunk_geom(const uint32_t *src, uint32_t P, uint64_t dw) {
    ChunkGeom g;
    g.src = src;
    g.dw = dw;
    g.de = dw + P;
    g.bs = (dw + 3) & ~(uint64_t)3;
    const uint64_t be = g.de & ~(uint64_t)3;
    g.tail_start = be > g.bs ? be : g.bs;
    g.units = be > g.bs ? (uint32_t)((be - g.bs) >> 2) : 0u;
    g.r = (uint32_t)(g.bs - dw);
    g.rn = g.r != 0 ? 1u : 0u;
    return g;
}

__device__ __forceinline__ void load_round(const ChunkGeom &g, uint32_t t0, CopyRound &R) {
    const uint32_t lane = threadIdx.x & 63;
    const uint4 *s4 = reinterpret_cast<const uint4 *>(g.src);
    /* the last source unit holding a needed word is units - 1 + rn; indices clamp to it */
    const uint32_t lastu = g.units - 1 + g.rn;
#pragma unroll
    for (int i = 0; i < kCopyBatch; ++i) R.A[i] = s4[min(t0 + lane + (uint32_t)(kWave * i), lastu)];
    R.E = s4[min(t0 + (uint32_t)(kWave * kCopyBatch), lastu)];
    R.hv = R.tv = 0;
    if (t0 == 0) {
        const uint64_t head_end = g.bs < g.de ? g.bs : g.de;
        if (lane < head_end - g.dw) R.hv = g.src[lane];
        if (g.tail_start < g.de && lane < g.de - g.tail_start) R.tv = g.src[g.tail_start - g.dw + lane];
    }
}

__device__ __forceinline__ uint32_t shl1(uint32_t v, uint32_t last_lane_value) {
    return dpp<0x130>(last_lane_value, v); /* wave_shl1: lane l takes lane l + 1's value */
}

__device__ __forceinline__ void store_round(const ChunkGeom &g, uint32_t t0, const CopyRound &R,
                                            uint32_t *__restrict__ pay) {
    const uint32_t lane = threadIdx.x & 63;
    uint4 *d4 = reinterpret_cast<uint4 *>(pay + g.bs);
#pragma unroll
    for (int i = 0; i < kCopyBatch; ++i) {
        const uint4 nx = i + 1 < kCopyBatch ? R.A[i + 1 < kCopyBatch ? i + 1 : i] : R.E;
        uint4 B;
        B.x = shl1(R.A[i].x, readlane(nx.x, 0));
        B.y = shl1(R.A[i].y, readlane(nx.y, 0));
        B.z = shl1(R.A[i].z, readlane(nx.z, 0));
        B.w = shl1(R.A[i].w, readlane(nx.w, 0));
        const uint32_t t = t0 + lane + (uint32_t)(kWave * i);
        if (t < g.units) d4[t] = shift_units(R.A[i], B, g.r);
    }
    if (t0 == 0) {
        const uint64_t head_end = g.bs < g.de ? g.bs : g.de;
        if (lane < head_end - g.dw) pay[g.dw + lane] = R.hv;
        if (g.tail_start < g.de && lane < g.de - g.tail_start) pay[g.tail_start + lane] = R.tv;
    }
}

/* The payloads of the chunks of a group in `mask` (bit k: chunk k, from src + k slot words to
 * stream word dw[k]), one round after another, each round's loads issued before the previous
 * round's stores. */
template <int CPG>
__device__ __forceinline__ void copy_chunks_pipelined(const uint32_t *__restrict__ src, uint32_t slot,
                                                      const uint32_t words[CPG], const uint64_t dw[CPG],
                                                      uint32_t mask, uint32_t *__restrict__ pay) {
    constexpr uint32_t kRound = kCopyBatch * kWave;
    /* the words and destination of chunk k, by selects on the wave-uniform k (an indexed read
     * of the arrays would place them in memory) */
#define EBLC_CHUNK_GEOM(K, OUT)                                       \
    do {                                                              \
        uint32_t P_ = words[0];                                       \
        uint64_t d_ = dw[0];                                          \
        _Pragma("unroll") for (int j_ = 1; j_ < CPG; ++j_) {          \
            P_ = (K) == j_ ? words[j_] : P_;                          \
            d_ = (K) == j_ ? dw[j_] : d_;                             \
        }                                                             \
        OUT = chunk_geom(src + (uint64_t)(K) * slot, P_, d_);         \
    } while (0)
    if (mask == 0) return;
    int k = __builtin_ctz(mask);
    mask &= mask - 1;
    ChunkGeom g;
    EBLC_CHUNK_GEOM(k, g);
    uint32_t t0 = 0;
    CopyRound cur;
    load_round(g, 0, cur);
#pragma unroll 1
    for (;;) {
        /* the next round: of this chunk, or the first of the next chunk */
        ChunkGeom gn = g;
        uint32_t tn = t0 + kRound;
        bool more = tn < g.units;
        if (!more && mask != 0) {
            k = __builtin_ctz(mask);
            mask &= mask - 1;
            EBLC_CHUNK_GEOM(k, gn);
            tn = 0;
            more = true;
        }
        CopyRound nxt;
        if (more) load_round(gn, tn, nxt);
        store_round(g, t0, cur, pay);
        if (!more) break;
        g = gn;
        t0 = tn;
        cur = nxt;
    }
#undef EBLC_CHUNK_GEOM
}

/* Chunks of at most this many payload words and kEscStage escapes are small. */
constexpr uint32_t kSmallChunkWords = 4 * kWave;

/* One wave per group of kEncChunksPerGroup encode chunks, kWavesPerBlock groups per workgroup.  A
 * group of small chunks -- most groups of a well-compressed field -- issues the loads of all four
 * chunks together (copy_group_payload), so it waits for one memory latency; a group with a larger
 * chunk copies its chunks in rounds, each round's loads issued before the previous round's
 * stores (copy_chunks_pipelined).  (A wave per chunk left every wave waiting on its own chain of
 * loads, twice the chains in all on the 512^3 field.)  Then the group's outliers, its
 * offset-table entry, its share of the size section when it was staged and its block means.  In
 * RAW mode the wave copies the group's input values instead.  The last group also zeroes the
 * pads after the payload, the outlier sections and the offset table. */
template <bool STRIDED>
__device__ __forceinline__ void compact_body(const float *__restrict__ x,
                                             PlanArgs pa, Workspace ws,
                                             uint8_t *__restrict__ out,
                                             const uint8_t *__restrict__ widths_src,
                                             const StreamPlace &P, uint32_t grp, uint32_t gw, uint32_t ge) {
    constexpr int CPG = kEncChunksPerGroup;
    const uint32_t lane = threadIdx.x & 63;
    /* every small input of the group up front, in one round of loads */
    uint32_t words[CPG], escs[CPG];
#pragma unroll
    for (int k = 0; k < CPG; ++k) {
        const uint32_t ck = grp * CPG + k;
        words[k] = ck < pa.nchunks ? ws.chunk_words[ck] : 0u;
        escs[k] = ck < pa.nchunks ? ws.chunk_esc[ck] : 0u;
    }
    const uint32_t fits = P.fits, mode = P.raw ? 1u : 0u;
    const uint64_t payload_off = P.po, oidx_off = P.oi, oval_off = P.ov;
    const uint64_t m = P.m, payload_words = P.pb / 4;
    if (!fits) return;
    const uint64_t n = pa.n;
    const uint64_t gbase = (uint64_t)grp * CPG * kEncChunk;
    const bool last = grp == pa.ngroups - 1;
    if (mode == 1) {
        constexpr uint32_t kGroupVals = CPG * kEncChunk;
        const uint64_t cnt = (n - gbase < (uint64_t)kGroupVals) ? n - gbase : (uint64_t)kGroupVals;
        uint32_t *dstw = reinterpret_cast<uint32_t *>(out + kHeaderBytes) + gbase;
        const uint32_t *srcw = reinterpret_cast<const uint32_t *>(x) + gbase;
        if (STRIDED) {
            const uint32_t *xb = reinterpret_cast<const uint32_t *>(x);
            for (uint32_t i = lane; i < cnt; i += kWave) dstw[i] = xb[elem_off<true>(pa.lay, gbase + i)];
        } else if (cnt == (uint64_t)kGroupVals) {
            constexpr int kPer = 4; /* 128-bit units per lane per round */
            const uint4 *s4 = reinterpret_cast<const uint4 *>(srcw);
            uint4 *d4 = reinterpret_cast<uint4 *>(dstw);
            for (uint32_t b = 0; b < kGroupVals / 4; b += kPer * kWave) {
                uint4 t[kPer];
#pragma unroll
                for (int i = 0; i < kPer; ++i) t[i] = ld_nt(s4 + b + lane + kWave * i);
#pragma unroll
                for (int i = 0; i < kPer; ++i) st_nt(d4 + b + lane + kWave * i, t[i]);
            }
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
    uint64_t dw[CPG];
    uint32_t O[CPG];
    bool small = true;
    {
        uint32_t W = gw, E = ge;
#pragma unroll
        for (int k = 0; k < CPG; ++k) {
            dw[k] = W;
            O[k] = E;
            W += words[k];
            E += escs[k];
            small = small && words[k] <= kSmallChunkWords && escs[k] <= (uint32_t)kEscStage;
        }
    }
    uint32_t *pay = reinterpret_cast<uint32_t *>(out + payload_off);
    uint32_t *oidx = reinterpret_cast<uint32_t *>(out + oidx_off);
    uint32_t *oval = reinterpret_cast<uint32_t *>(out + oval_off);
    /* the offset table's entry for the group: the payload words before it */
    uint32_t *table = reinterpret_cast<uint32_t *>(out + kHeaderBytes + pa.wsec);
    if (lane == 0 && grp != 0) table[grp - 1] = gw;
    if (small) {
        copy_group_payload<CPG>(ws.scratch + (uint64_t)grp * CPG * pa.slot, pa.slot, words, dw, pay);
    } else {
        uint32_t mask = 0;
#pragma unroll
        for (int k = 0; k < CPG; ++k)
            if (grp * CPG + (uint32_t)k < pa.nchunks && words[k] != 0) mask |= 1u << k;
        copy_chunks_pipelined<CPG>(ws.scratch + (uint64_t)grp * CPG * pa.slot, pa.slot, words, dw, mask, pay);
    }
    /* the outliers, after the payload (few groups have any): the chunks' staged escapes, loaded
     * together, or for a chunk with more, its escapes ranked from its segments' bitmasks */
    uint32_t any_esc = 0;
#pragma unroll
    for (int k = 0; k < CPG; ++k) any_esc |= escs[k];
    if (any_esc != 0) {
        uint32_t si[CPG], sv[CPG];
#pragma unroll
        for (int k = 0; k < CPG; ++k) {
            const uint64_t ck = (uint64_t)grp * CPG + k;
            si[k] = sv[k] = 0;
            if (escs[k] <= (uint32_t)kEscStage && lane < escs[k]) {
                si[k] = ws.stage_idx[ck * kEscStage + lane];
                sv[k] = ws.stage_val[ck * kEscStage + lane];
            }
        }
#pragma unroll
        for (int k = 0; k < CPG; ++k) {
            const uint32_t ck = grp * CPG + k;
            if (escs[k] <= (uint32_t)kEscStage) {
                if (lane < escs[k]) {
                    oidx[O[k] + lane] = si[k];
                    oval[O[k] + lane] = sv[k];
                }
            } else if (ck < pa.nchunks) {
                write_chunk_outliers<STRIDED>(x, pa.lay, ws, ck, escs[k], O[k], oidx, oval);
            }
        }
    }
    if (widths_src != nullptr) {
        /* the group's share of the size section, staged by the encoder */
        for (uint32_t i = lane; i < pa.wpg / 4; i += kWave) {
            const uint64_t off = (uint64_t)grp * pa.wpg + 4u * i;
            if (off < pa.wsec)
                *reinterpret_cast<uint32_t *>(out + kHeaderBytes + off) = *reinterpret_cast<const uint32_t *>(widths_src + off);
        }
    }
    if (pa.center) {
        /* the means of the blocks that start in the group, staged by the encoder, into the
         * means section */
        const uint64_t gend = gbase + (uint64_t)CPG * kEncChunk;
        const uint64_t b0 = (gbase + pa.B - 1) / pa.B;
        const uint64_t b1e = (gend + pa.B - 1) / pa.B;
        const uint64_t b1 = b1e < pa.nblocks ? b1e : pa.nblocks;
        int32_t *mdst = reinterpret_cast<int32_t *>(out + kHeaderBytes + pa.wsec + table_bytes(pa.ngroups));
        for (uint64_t b = b0 + lane; b < b1; b += kWave) mdst[b] = ws.means[b];
        if (last && lane < (pa.msec - 4 * pa.nblocks) / 4) mdst[pa.nblocks + lane] = 0;
    }
    if (last) {
        const uint64_t pend = payload_off + 4 * payload_words;
        const uint64_t pad = oidx_off - pend;
        if (lane < pad / 4) reinterpret_cast<uint32_t *>(out + pend)[lane] = 0u;
        const uint64_t opad = (align16(4 * m) - 4 * m) / 4;
        if (lane < opad) {
            oidx[m + lane] = 0u;
            oval[m + lane] = 0u;
        }
        const uint32_t entries = pa.ngroups - 1;
        if (lane < table_bytes(pa.ngroups) / 4 - entries) table[entries + lane] = 0u;
    }
}

template <bool STRIDED>
__global__ __launch_bounds__(kBlockThreads) void compact_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    const uint32_t f = blockIdx.y;
    const Workspace w = lane_ws(ws, f, fs.ws_stride);
    const uint32_t grp = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (grp >= pa.ngroups) return;
    const uint32_t gw = group_prefix(w.gpre_words, w.group_words, grp);
    const uint32_t ge = group_prefix(w.gpre_esc, w.group_esc, grp);
    compact_body<STRIDED>(reinterpret_cast<const float *>(pick(fs.src, f)), pa, w, pick(fs.dst, f),
                          (fs.wdirect >> f) & 1u ? nullptr : w.widths, place_from_info(w.info), grp, gw, ge);
}

/* Exclusive prefixes of a[0..ng) and b[0..ng), ng <= kFoldGroups, into LDS (s_a, s_b), and their
 * totals (every thread): thread t sums items 8t .. 8t+7 (two 128-bit loads of each array, which
 * are 256-byte aligned), a wave scan and the four waves' totals through LDS give its start. */
constexpr uint32_t kFoldGroups = kBlockThreads * 8;
__device__ __forceinline__ void fold_scan(const uint32_t *__restrict__ a, const uint32_t *__restrict__ b,
                                          uint32_t ng, uint32_t *s_a, uint32_t *s_b, uint32_t &ta, uint32_t &tb) {
    __shared__ uint32_t s_t[kWavesPerBlock][2];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t i0 = 8 * tid;
    uint32_t va[8], vb[8];
    if (i0 + 8 <= ng) {
        const uint4 a0 = reinterpret_cast<const uint4 *>(a + i0)[0], a1 = reinterpret_cast<const uint4 *>(a + i0)[1];
        const uint4 b0 = reinterpret_cast<const uint4 *>(b + i0)[0], b1 = reinterpret_cast<const uint4 *>(b + i0)[1];
        va[0] = a0.x; va[1] = a0.y; va[2] = a0.z; va[3] = a0.w; va[4] = a1.x; va[5] = a1.y; va[6] = a1.z; va[7] = a1.w;
        vb[0] = b0.x; vb[1] = b0.y; vb[2] = b0.z; vb[3] = b0.w; vb[4] = b1.x; vb[5] = b1.y; vb[6] = b1.z; vb[7] = b1.w;
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            va[k] = i0 + k < ng ? a[i0 + k] : 0u;
            vb[k] = i0 + k < ng ? b[i0 + k] : 0u;
        }
    }
    uint32_t sa = 0, sb = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        sa += va[k];
        sb += vb[k];
    }
    const uint32_t ia = wave_incl_scan(sa), ib = wave_incl_scan(sb);
    if (lane == 63) {
        s_t[wave][0] = ia;
        s_t[wave][1] = ib;
    }
    __syncthreads();
    uint32_t ea = ia - sa, eb = ib - sb;
    ta = tb = 0;
#pragma unroll
    for (uint32_t w = 0; w < (uint32_t)kWavesPerBlock; ++w) {
        const uint32_t xa = s_t[w][0], xb = s_t[w][1];
        ea += w < wave ? xa : 0u;
        eb += w < wave ? xb : 0u;
        ta += xa;
        tb += xb;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (i0 + k < ng) {
            s_a[i0 + k] = ea;
            s_b[i0 + k] = eb;
        }
        ea += va[k];
        eb += vb[k];
    }
    __syncthreads();
}

/* K3 + K4 for fields of at most kFoldGroups groups (2^24 values): every compaction workgroup
 * scans the group sums itself (fold_scan) and places the stream (place_stream), the same in
 * each, and workgroup 0 writes the placement, the result record and the header, so the
 * single-workgroup scan launch is not needed. */
template <bool STRIDED>
__global__ __launch_bounds__(kBlockThreads) void compact_scan_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    __shared__ uint32_t s_pw[kFoldGroups], s_pe[kFoldGroups];
    __shared__ uint32_t s_hdr[32];
    const uint32_t f = blockIdx.y;
    const Workspace w = lane_ws(ws, f, fs.ws_stride);
    uint8_t *out = pick(fs.dst, f);
    const uint32_t valid = w.info->valid;
    uint32_t S, M;
    fold_scan(w.group_words, w.group_esc, pa.ngroups, s_pw, s_pe, S, M);
    const StreamPlace P = place_stream(pa, S, M, valid != 0, pick(fs.bytes, f));
    if (blockIdx.x == 0) {
        if (threadIdx.x == 0) publish_stream(pa, P, w.info, pick(fs.result, f), s_hdr);
        __syncthreads();
        if (P.fits && threadIdx.x < 32) reinterpret_cast<uint32_t *>(out)[threadIdx.x] = s_hdr[threadIdx.x];
    }
    const uint32_t grp = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (grp >= pa.ngroups) return;
    compact_body<STRIDED>(reinterpret_cast<const float *>(pick(fs.src, f)), pa, w, out,
                          (fs.wdirect >> f) & 1u ? nullptr : w.widths, P, grp, s_pw[grp], s_pe[grp]);
}

/* ---- K7: fused decode ------------------------------------------------------------------------ */

/* The tile loop of one decode chunk whose packed words and segment widths are staged in LDS:
 * per tile unpack each lane's 4 values, undo the zigzag, prefix-sum inside each block (in-lane,
 * then across lanes, plus the carry from the previous tile when a block spans tiles; CENTERED:
 * plus the block's mean code mu[t] at its start), dequantize with f32(f32(q) * s) and store 4
 * values with one 128-bit store.
 *   A power-of-two block (GB = false) starts a decode chunk, and its blocks are aligned groups
 * of lanes: a segmented DPP scan.  Any other block (a multiple of 32, GB = true) may start at
 * any 8-lane boundary: a lane's offset in its block is (r0 + 256 t + 4 lane) mod B, with r0 the
 * chunk start's offset in its block; the lane's prefix is the plain wave scan minus the scan at
 * its block's first lane (ds_bpermute), or plus the carry when its block began before the tile;
 * carry starts at carry0, the code before the chunk when the chunk starts inside a block. */
template <bool STRIDED, bool CENTERED, bool GB>
__device__ __forceinline__ void decode_tiles(const PlanArgs &pa, float s, uint32_t B, const int32_t mu[kDecTiles],
                                             const uint32_t *pay, const uint32_t *s_w, const uint32_t *s_so,
                                             uint32_t lb, uint64_t cbase, bool full, float *__restrict__ out,
                                             int32_t carry0, uint32_t r0, uint32_t mB) {
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t n = pa.n;
    /* s and B are the stream's, validated by the header check */
    const uint32_t seglen = (B / 4 < 64u) ? B / 4 : 64u;
    const uint32_t dist = lane & (seglen - 1);
    const uint32_t ntiles = full ? kDecTiles : (uint32_t)((n - cbase + kTile - 1) / kTile);
    const uint32_t j = lane & 7;
    int32_t carry = GB ? carry0 : 0;
#pragma unroll
    for (int t = 0; t < kDecTiles; ++t) {
        if ((uint32_t)t < ntiles) {
            const uint32_t g = (uint32_t)t * 8 + (lane >> 3);
            const uint32_t w = s_w[g];
            const uint32_t bp = 32u * (lb + s_so[g]) + 4u * w * j;
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
            int32_t base;
            if (GB) {
                const uint32_t a = r0 + (uint32_t)t * kTile + 4u * lane;
                const uint32_t rem = a - __umulhi(a, mB) * B; /* offset of the lane's first value in its block */
                const uint32_t incl = wave_incl_scan((uint32_t)cs[3]);
                const uint32_t excl = incl - (uint32_t)cs[3];
                const bool opened = rem / 4u > lane;       /* the block began before this tile */
                const uint32_t bsl = opened ? 0u : lane - rem / 4u;
                const uint32_t e_bs = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(4u * bsl), (int)excl);
                base = opened ? (int32_t)(excl + (uint32_t)carry) : (int32_t)(excl - e_bs);
                if (CENTERED && !opened) base += mu[t];
            } else {
                const uint32_t incl = wave_seg_scan((uint32_t)cs[3], dist, seglen);
                const bool open = (((uint32_t)t * kTile) & (B - 1)) != 0;
                base = (int32_t)(incl - (uint32_t)cs[3]) + (open ? carry : 0);
                if (CENTERED) base += mu[t];
            }
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
                store4<STRIDED>(out, pa.lay, e0, o);
            } else {
                if (e0 + 0 < n) out[elem_off<STRIDED>(pa.lay, e0 + 0)] = o.x;
                if (e0 + 1 < n) out[elem_off<STRIDED>(pa.lay, e0 + 1)] = o.y;
                if (e0 + 2 < n) out[elem_off<STRIDED>(pa.lay, e0 + 2)] = o.z;
                if (e0 + 3 < n) out[elem_off<STRIDED>(pa.lay, e0 + 3)] = o.w;
            }
        }
    }
}

/* The code before a decode chunk that starts inside a block of a non-power-of-two B: the sum of
 * the deltas of the block's r0 / 32 segments before the chunk (at most 31, the last segments of
 * the previous chunk; r0 < B <= 1024), read from the stream just before the chunk's words.  Eight
 * lanes take a segment, four values each, eight segments per round; a value's two words are
 * read only when its bits span them, so no read leaves those segments' words. */
__device__ __forceinline__ int32_t open_block_sum(const uint8_t *__restrict__ in, uint64_t seg_end, uint32_t nseg,
                                                  const uint32_t *__restrict__ words_end, uint64_t limit, bool &ok) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wpre = lane < nseg ? (uint32_t)in[kHeaderBytes + seg_end - nseg + lane] : 0u;
    const uint32_t incl = wave_incl_scan(wpre);
    const uint32_t total = readlane(incl, 63);
    const uint32_t so = incl - wpre;
    /* those segments' words lie inside the payload (limit words precede the chunk's) and their
     * widths are at most 32, or the stream is corrupt */
    ok = __ballot(wpre > 32u) == 0 && total <= limit;
    if (!ok) return 0;
    const uint32_t *pw = words_end - total;
    const uint32_t j = lane & 7;
    int32_t sum = 0;
    for (uint32_t g0 = 0; g0 < nseg; g0 += 8) {
        const uint32_t g = g0 + (lane >> 3);
        const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(4u * (g & 63u)), (int)wpre);
        const uint32_t o = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(4u * (g & 63u)), (int)so);
        if (g < nseg && w != 0) {
            const uint32_t mask = w >= 32 ? 0xffffffffu : ((1u << w) - 1u);
            const uint32_t bp = 32u * o + 4u * w * j;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t pos = bp + (uint32_t)k * w;
                const uint32_t wi = pos >> 5, sh = pos & 31u;
                const uint32_t lo = pw[wi];
                const uint32_t hi = sh + w > 32u ? pw[wi + 1] : 0u;
                const uint64_t pair = (uint64_t)lo | ((uint64_t)hi << 32);
                sum += unzigzag((uint32_t)(pair >> sh) & mask);
            }
        }
    }
    return (int32_t)readlane(wave_incl_scan((uint32_t)sum), 63);
}

/* One workgroup per table group, one wave per chunk: the workgroup stages the group's packed
 * words in LDS (128-bit loads), each wave its chunk's segment widths and word offsets, then
 * each wave runs decode_tiles on its chunk (the centered copy for a centered stream, the
 * general-block copy for a block that is not a power of two). */
template <bool STRIDED>
__device__ __forceinline__ void decode_body(const uint8_t *__restrict__ in, uint64_t in_bytes,
                                            PlanArgs pa, Workspace ws,
                                            float *__restrict__ out) {
    constexpr uint32_t kGroupUnits = kDecChunksPerGroup * kDecChunk / 4 + 2;
    __shared__ uint4 s_pay4[kGroupUnits];
    __shared__ uint32_t s_w[kWavesPerBlock][kDecSegs];
    __shared__ uint32_t s_so[kWavesPerBlock][kDecSegs];

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t grp = blockIdx.x;
    const uint32_t c = grp * kWavesPerBlock + wave; /* may be past the last chunk in the last group */
    /* The group's payload is the range the offset table gives it, so the workgroup's staging
     * loads go out as soon as the header and the table entries are in (one round of loads: all
     * lie inside the bytes the host lets through), while the widths are still on their way; a
     * staging load that would leave the caller's bytes is not issued (no valid stream asks for
     * one).  Lane l of every wave sums the width bytes of the group's segments 4l .. 4l+3 (chunk
     * l / 16; bytes past the last segment count 0), which places each chunk in the group and
     * checks the group: no width above 32 and exactly the words the table gives it.  The whole
     * header is checked (and a bad one reported) by the outlier patch. */
    const uint32_t hv = load_header_lanes(in, pa, grp);
    const uint64_t gseg = (uint64_t)grp * (kDecChunksPerGroup * kDecSegs) + 4u * lane;
    uint32_t wq = gseg < pa.nseg ? *reinterpret_cast<const uint32_t *>(in + kHeaderBytes + gseg) : 0u;
    const uint64_t seg = (uint64_t)c * kDecSegs + lane;
    const uint32_t wl = seg < pa.nseg ? (uint32_t)in[kHeaderBytes + seg] : 0u;
    const StreamView H = view_header(hv);
    const uint64_t n = pa.n;
    if (!H.sane) return; /* the same in every wave of the workgroup, as every test before the barrier */
    const uint64_t cbase = (uint64_t)c * kDecChunk;
    const bool full = cbase + kDecChunk <= n;
    if (H.mode == 1) {
        if (c >= pa.dchunks || kHeaderBytes + 4 * n > in_bytes) return;
        const uint64_t cnt = full ? (uint64_t)kDecChunk : n - cbase;
        const uint32_t *srcw = reinterpret_cast<const uint32_t *>(in + kHeaderBytes) + cbase;
        uint32_t *dstw = reinterpret_cast<uint32_t *>(out) + cbase;
        if (STRIDED) {
            uint32_t *ob = reinterpret_cast<uint32_t *>(out);
            for (uint32_t i = lane; i < cnt; i += kWave) ob[elem_off<true>(pa.lay, cbase + i)] = srcw[i];
        } else if (full) {
            const uint4 *s4 = reinterpret_cast<const uint4 *>(srcw);
            uint4 *d4 = reinterpret_cast<uint4 *>(dstw);
            uint4 t[kDecChunk / 4 / kWave];
#pragma unroll
            for (int i = 0; i < kDecChunk / 4 / kWave; ++i) t[i] = ld_nt(s4 + lane + kWave * i);
#pragma unroll
            for (int i = 0; i < kDecChunk / 4 / kWave; ++i) st_nt(d4 + lane + kWave * i, t[i]);
        } else {
            for (uint32_t i = lane; i < cnt; i += kWave) dstw[i] = srcw[i];
        }
        return;
    }
    uint64_t t0, t1;
    table_range(hv, grp, pa.ngroups, H.pw, t0, t1);
    const uint64_t gw0 = H.po / 4 + t0;  /* stream word index of the group's first word */
    const uint64_t a0 = gw0 & ~(uint64_t)3;
    const uint32_t lb = (uint32_t)(gw0 - a0);
    const uint64_t lim = in_bytes / 16;
    const bool range_ok = t0 <= t1 && t1 <= H.pw && t1 - t0 <= (uint64_t)(kDecChunksPerGroup * kDecChunk);
    const uint32_t units = range_ok ? (uint32_t)((lb + (t1 - t0) + 3) >> 2) : 0u;
    if (!range_ok || a0 / 4 > lim || units > lim - a0 / 4) {
        if (wave == 0 && lane == 0 && !range_ok) atomicOr(&ws.info->sticky, 1u);
        return;
    }
    /* every staging load of the group is issued before the first LDS store */
    constexpr int kRounds = (kGroupUnits + kBlockThreads - 1) / kBlockThreads;
    const uint4 *src = reinterpret_cast<const uint4 *>(in) + a0 / 4;
    uint4 v[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        const uint32_t u = threadIdx.x + (uint32_t)r * kBlockThreads;
        v[r] = make_uint4(0, 0, 0, 0);
        if (u < units) v[r] = src[u];
    }
    if (gseg < pa.nseg && pa.nseg - gseg < 4) wq &= (1u << (8u * (uint32_t)(pa.nseg - gseg))) - 1u;
    const uint32_t gincl = wave_incl_scan(__builtin_amdgcn_sad_u8(wq, 0u, 0u));
    const uint32_t before = wave > 0 ? readlane(gincl, 16 * (int)wave - 1) : 0u;
    const uint32_t gtot = readlane(gincl, 63);
    const uint32_t wbad = (((wq & 0x7F7F7F7Fu) + 0x5F5F5F5Fu) | wq) & 0x80808080u;
    if (__ballot(wbad != 0) != 0 || t1 - t0 != gtot) {
        if (wave == 0 && lane == 0) atomicOr(&ws.info->sticky, 1u);
        return;
    }
    const uint64_t W = t0 + before;       /* payload words before the chunk */
    const uint64_t sw = H.po / 4 + W;     /* stream word index of the chunk's first word */
    /* the stream's block; for one that is not a power of two, the chunk start's offset in its
     * block (r0), the block holding the chunk's first value (bk0) and the reciprocal of B for
     * the small divisions of decode_tiles */
    const uint32_t B = H.B;
    const bool gb = (B & (B - 1)) != 0;
    uint32_t r0 = 0, bk0 = 0, mB = 0;
    if (gb) {
        mB = 0xFFFFFFFFu / B + 1u;
        bk0 = (uint32_t)cbase / B;
        r0 = (uint32_t)cbase - bk0 * B;
    }
    /* a centered stream's blocks start from their mean code: in each tile, every lane whose block
     * starts in the tile takes its block's mean, loaded once the header is checked, while the
     * staging loads are still in flight (lanes past n read nothing: their blocks' means may lie
     * past the stream's end) */
    const bool centered = (H.flags & 1u) != 0;
    const uint64_t mbase = kHeaderBytes + pa.wsec + table_bytes(pa.ngroups);
    const int32_t *means = reinterpret_cast<const int32_t *>(in + mbase);
    const uint64_t mlim = in_bytes > mbase ? (in_bytes - mbase) / 4 : 0; /* means inside the caller's bytes */
    int32_t mu[kDecTiles];
#pragma unroll
    for (int t = 0; t < kDecTiles; ++t) {
        const uint64_t ev = cbase + (uint64_t)t * kTile + 4 * lane;
        mu[t] = 0;
        if (centered && ev < n) {
            if (gb) {
                const uint32_t a = r0 + (uint32_t)t * kTile + 4u * lane;
                const uint32_t q = __umulhi(a, mB);
                if ((a - q * B) / 4u <= lane && bk0 + q < mlim) mu[t] = means[bk0 + q];
            } else if ((((uint32_t)t * kTile) & (B - 1)) == 0) {
                const uint64_t b = ev >> (uint32_t)__builtin_ctz(B);
                if (b < mlim) mu[t] = means[b];
            }
        }
    }
    const uint32_t so = wave_incl_scan(wl) - wl;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        const uint32_t u = threadIdx.x + (uint32_t)r * kBlockThreads;
        if (u < units) s_pay4[u] = v[r];
    }
    s_w[wave][lane] = wl;
    s_so[wave][lane] = so;
    __syncthreads();
    if (c >= pa.dchunks) return;
    /* the chunk's words sit at word lb + before of the group's staging */
    const uint32_t *pay = reinterpret_cast<const uint32_t *>(s_pay4);
    const uint32_t lbc = lb + before;
    if (gb) {
        int32_t carry0 = 0;
        if (r0 != 0) {
            bool ok;
            carry0 = open_block_sum(in, (uint64_t)c * kDecSegs, r0 / 32u,
                                    reinterpret_cast<const uint32_t *>(in) + sw, W, ok);
            if (!ok) {
                if (lane == 0) atomicOr(&ws.info->sticky, 1u);
                return;
            }
            if (centered && bk0 < mlim) carry0 += means[bk0];
        }
        if (centered)
            decode_tiles<STRIDED, true, true>(pa, H.s, B, mu, pay, s_w[wave], s_so[wave], lbc, cbase, full, out, carry0,
                                              r0, mB);
        else
            decode_tiles<STRIDED, false, true>(pa, H.s, B, mu, pay, s_w[wave], s_so[wave], lbc, cbase, full, out, carry0,
                                               r0, mB);
    } else if (centered) {
        /* a centered stream takes its own copy of the tile loop, so the plain one stays as it is */
        decode_tiles<STRIDED, true, false>(pa, H.s, B, mu, pay, s_w[wave], s_so[wave], lbc, cbase, full, out, 0, 0, 0);
    } else {
        decode_tiles<STRIDED, false, false>(pa, H.s, B, mu, pay, s_w[wave], s_so[wave], lbc, cbase, full, out, 0, 0, 0);
    }
}

template <bool STRIDED>
__global__ __launch_bounds__(kBlockThreads) void decode_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    const uint32_t f = blockIdx.y;
    decode_body<STRIDED>(pick(fs.src, f), pick(fs.bytes, f), pa, lane_ws(ws, f, fs.ws_stride),
                         reinterpret_cast<float *>(pick(fs.dst, f)));
}

/* ---- K8: outlier patch ------------------------------------------------------------------------ */

template <bool STRIDED>
__device__ __forceinline__ void patch_body(const uint8_t *__restrict__ in, uint64_t in_bytes, PlanArgs pa,
                                           Workspace ws, float *__restrict__ out) {
    DevInfo *info = ws.info;
    const uint32_t hv = load_header_lanes(in, pa, 0);
    /* the first wave checks the whole header and reports a bad one (the decoders only bound
     * their reads); the others need only the outlier sections inside the caller's bytes */
    if (blockIdx.x == 0 && threadIdx.x < kWave &&
        !header_ok(hv, load_header_template(info), in_bytes, pa.n, pa.V, pa.wsec, pa.ngroups, pa.max_pw)) {
        if (threadIdx.x == 0) atomicOr(&info->sticky, 1u);
        return;
    }
    const StreamView V = view_header(hv);
    const uint64_t m = readlane64(hv, 18), oi = readlane64(hv, 26), ov = readlane64(hv, 28);
    const uint64_t q = in_bytes / 4;
    if (!V.sane || V.mode == 1 || m > q || (oi | ov) % 4 != 0 || oi / 4 > q - m || ov / 4 > q - m) return;
    const uint32_t *oidx = reinterpret_cast<const uint32_t *>(in + oi);
    const uint32_t *oval = reinterpret_cast<const uint32_t *>(in + ov);
    uint32_t *ob = reinterpret_cast<uint32_t *>(out);
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    for (uint64_t k = (uint64_t)blockIdx.x * 256 + threadIdx.x; k < m; k += stride) {
        const uint32_t idx = oidx[k];
        const bool ok = idx < pa.n && (k == 0 || oidx[k - 1] < idx);
        if (ok) ob[elem_off<STRIDED>(pa.lay, idx)] = oval[k];
        else atomicOr(&info->sticky, 1u);
    }
}

template <bool STRIDED>
__global__ __launch_bounds__(256) void patch_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    const uint32_t f = blockIdx.y;
    patch_body<STRIDED>(pick(fs.src, f), pick(fs.bytes, f), pa, lane_ws(ws, f, fs.ws_stride),
                        reinterpret_cast<float *>(pick(fs.dst, f)));
}

}  // namespace

/* ---- launchers ------------------------------------------------------------------------------- */

hipError_t launch_range(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws, double eps,
                        hipStream_t stream) {
    const uint32_t grid = range_blocks(pa.n);
    if (pa.lay.strided)
        eblc_launch<false>(range_partial_kernel<true>, dim3(grid, nf), dim3(kRangeThreads), 0, stream, fs, pa.n,
                           pa.lay, ws);
    else
        eblc_launch<false>(range_partial_kernel<false>, dim3(grid, nf), dim3(kRangeThreads), 0, stream, fs, pa.n,
                           pa.lay, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    eblc_launch(range_resolve_kernel, dim3(1, nf), dim3(kScanThreads), 0, stream, fs, ws, grid, eps);
    return hipGetLastError();
}

hipError_t launch_resolve_abs(const Workspace &ws, double eps, hipStream_t stream) {
    Fields fs{};
    eblc_launch(range_resolve_kernel, dim3(1, 1), dim3(kScanThreads), 0, stream, fs, ws, 0u, eps);
    return hipGetLastError();
}

hipError_t launch_encode(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                         hipStream_t stream) {
    const bool gb = (pa.B & (pa.B - 1)) != 0;
    const bool narrow = pa.T + pa.log2B <= 29;
    const int cm = !pa.center ? kCenterOff
                   : gb ? kCenterGen
                   : (pa.B == (uint32_t)kEncTile && narrow) ? kCenterWhole
                   : (pa.B < (uint32_t)kEncTile && narrow) ? kCenterTile : kCenterAny;
    const dim3 grid(pa.ngroups, nf), block(kEncThreads);
#define EBLC_ENCODE(S, C, G) eblc_launch((encode_kernel<S, C, G>), grid, block, 0, stream, fs, pa, ws)
    if (pa.lay.strided) {
        if (cm == kCenterWhole) EBLC_ENCODE(true, kCenterWhole, false);
        else if (cm == kCenterTile) EBLC_ENCODE(true, kCenterTile, false);
        else if (cm == kCenterAny) EBLC_ENCODE(true, kCenterAny, false);
        else if (cm == kCenterGen) EBLC_ENCODE(true, kCenterGen, true);
        else if (gb) EBLC_ENCODE(true, kCenterOff, true);
        else EBLC_ENCODE(true, kCenterOff, false);
    } else {
        if (cm == kCenterWhole) EBLC_ENCODE(false, kCenterWhole, false);
        else if (cm == kCenterTile) EBLC_ENCODE(false, kCenterTile, false);
        else if (cm == kCenterAny) EBLC_ENCODE(false, kCenterAny, false);
        else if (cm == kCenterGen) EBLC_ENCODE(false, kCenterGen, true);
        else if (gb) EBLC_ENCODE(false, kCenterOff, true);
        else EBLC_ENCODE(false, kCenterOff, false);
    }
#undef EBLC_ENCODE
    return hipGetLastError();
}

hipError_t launch_scan_compress(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                                hipStream_t stream) {
    eblc_launch(scan_compress_kernel, dim3(1, nf), dim3(kScanThreads), 0, stream, fs, pa, ws);
    return hipGetLastError();
}

hipError_t launch_compact(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                          hipStream_t stream) {
    const dim3 grid((pa.ngroups + kWavesPerBlock - 1) / kWavesPerBlock, nf), block(kBlockThreads);
    if (pa.lay.strided)
        eblc_launch(compact_kernel<true>, grid, block, 0, stream, fs, pa, ws);
    else
        eblc_launch(compact_kernel<false>, grid, block, 0, stream, fs, pa, ws);
    return hipGetLastError();
}

bool compact_folds_scan(const PlanArgs &pa) { return pa.ngroups <= kFoldGroups; }

hipError_t launch_compact_scan(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                               hipStream_t stream) {
    const dim3 grid((pa.ngroups + kWavesPerBlock - 1) / kWavesPerBlock, nf), block(kBlockThreads);
    if (pa.lay.strided)
        eblc_launch(compact_scan_kernel<true>, grid, block, 0, stream, fs, pa, ws);
    else
        eblc_launch(compact_scan_kernel<false>, grid, block, 0, stream, fs, pa, ws);
    return hipGetLastError();
}

hipError_t launch_decode(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                         hipStream_t stream) {
    const dim3 grid(pa.dgroups, nf), block(kBlockThreads);
    if (pa.lay.strided)
        eblc_launch(decode_kernel<true>, grid, block, 0, stream, fs, pa, ws);
    else
        eblc_launch(decode_kernel<false>, grid, block, 0, stream, fs, pa, ws);
    return hipGetLastError();
}

hipError_t launch_patch(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                        hipStream_t stream) {
    uint64_t want = (pa.side_max + 255) / 256;
    uint32_t grid = (uint32_t)(want < 1 ? 1 : (want > (uint64_t)kPatchBlocksMax ? kPatchBlocksMax : want));
    if (pa.lay.strided)
        eblc_launch(patch_kernel<true>, dim3(grid, nf), dim3(256), 0, stream, fs, pa, ws);
    else
        eblc_launch(patch_kernel<false>, dim3(grid, nf), dim3(256), 0, stream, fs, pa, ws);
    return hipGetLastError();
}

}  // namespace eblc
