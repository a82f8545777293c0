/*
 * eblc_chunk.hip -- gfx950 kernels of the chunk-cooperative coder: Quant -> Diff ->
 * Bitshuffle -> RZE over chunks of 4096, 8192 or 16384 input bytes ("Pipeline Specialization
 * Internals", FZGPUModules site, Chunk-cooperative path).  A chunk of V float32 values is coded
 * on its own: the verified linear quantizer (same rule and escapes as the bitpack coder), the
 * first difference inside the chunk (0 predicts its first code) folded by zigzag, the chunk's
 * 32 bit planes (plane-major: word b * G + g holds bit b of the 32 codes of group g, G = V /
 * 32, code j of a group at bit j), and zero-word elimination (a bitmap of the V words, then the
 * nonzero words in order).  The scan, compaction and outlier kernels of the bitpack coder
 * serve this coder unchanged; only the scratch slot stride and the size section differ.
 *
 * gfx950 mapping.  A tile is 64 consecutive values, one per lane.  Bitshuffle is a 32 x 32 bit
 * transpose inside each half-wave (five butterfly stages: ds_swizzle or DPP for the partner
 * lane, v_alignbit for the rotate, v_bfi for the merge), after which lane 32 h + b holds the
 * plane-b word of the tile's group h: one LDS store per lane per tile puts it at its plane-major
 * place.  LDS planes are padded by two words so those stores and the plane reads of RZE are
 * free of bank conflicts.  RZE walks only the planes below the chunk's highest code bit: a
 * ballot per 64 words gives two bitmap words, and mbcnt the compacted position.  Decoding runs
 * the same steps backwards; the transpose is its own inverse.
 */
#include "eblc_device.h"

namespace eblc {
namespace {

constexpr int kCTile = 64;                     /* values per tile: one per lane */
constexpr int kCTilesPerWave = kEncChunk / kCTile;

template <int V>
struct ChunkGeom {
    static constexpr int G = V / 32;            /* groups of 32 codes = words per bit plane */
    static constexpr int PS = G + 2;            /* LDS words per plane (2 words of padding) */
    static constexpr int LDSW = 32 * PS;        /* LDS words of one chunk's planes */
    static constexpr int BM = V / 32;           /* bitmap words of RZE */
    static constexpr int BATCHES = (G + 63) / 64; /* 64-word batches per plane */
    static constexpr int WAVES = V > kEncChunk ? V / kEncChunk : 1;      /* encode waves per chunk */
    static constexpr int PER_WAVE = V < kEncChunk ? kEncChunk / V : 1;   /* chunks per encode wave */
    static constexpr int TILES = V / kCTile;
    /* The decoder's LDS: 1024-value chunks are decoded from their words as staged (RAW: up to
     * BM + V words from a 16-byte unit boundary, 3 words before and 3 after, then the bitmap's
     * popcount prefix); 2048-value chunks from their rebuilt planes; 4096-value chunks from
     * the rebuilt planes of half a chunk at a time (HALVES). */
    static constexpr bool RAW = V == 1024;
    static constexpr bool HALVES = V == 4096;
    static constexpr int PSH = 64 + 2;          /* LDS words per plane of a half */
    static constexpr int RAWW = 4 * ((3 + BM + V + 3) / 4);
    static constexpr int DEC_LDSW = RAW ? RAWW + BM : HALVES ? 32 * PSH : LDSW; /* per wave */
    static_assert(DEC_LDSW % 4 == 0, "whole 16-byte units");
    static_assert(V == 1024 || V == 2048 || V == 4096, "chunk of 4, 8 or 16 KiB");
    static_assert(PER_WAVE * (BM + V) <= WAVES * (kEncChunk + kEncChunk / 32), "scratch slots of 2112 words");
};

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

/* old with lane `at` (wave-uniform) replaced by the wave-uniform value v. */
__device__ __forceinline__ uint32_t writelane(uint32_t old, uint32_t v, uint32_t at) {
    return (threadIdx.x & 63u) == at ? v : old;
}

/* OR over all 64 lanes (DPP inside rows, then the four rows' lanes 0, 16, 32 and 48). */
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
    v |= dpp<kDppQuadXor1>(0, v);
    v |= dpp<kDppQuadXor2>(0, v);
    v |= dpp<kDppRowHalfMirror>(0, v);
    v |= dpp<kDppRowMirror>(0, v);
    return readlane(v, 0) | readlane(v, 16) | readlane(v, 32) | readlane(v, 48);
}

/* 32 x 32 bit transpose inside each half-wave: on exit bit j of lane 32 h + b is bit b of lane
 * 32 h + j's word on entry.  Five butterfly stages s = 16, 8, 4, 2, 1 pair lane l with l ^ s;
 * the lower lane of a pair keeps its bits whose index has bit s clear and takes its partner's
 * such bits shifted up by s, the upper lane keeps the others and takes its partner's shifted
 * down.  For s = 16 and 8 both are byte moves, one v_perm_b32 each (selector bytes 0-3 pick
 * the partner's bytes, 4-7 the lane's own); for s = 4, 2, 1 the partner's word is rotated by
 * s (v_alignbit) and merged under the stage mask (v_bfi). */
struct Transpose {
    uint32_t sel16, sel8, keep[3], rot[3];
    __device__ __forceinline__ explicit Transpose(uint32_t lane) {
        sel16 = (lane & 16u) ? 0x07060302u : 0x01000504u;
        sel8 = (lane & 8u) ? 0x07030501u : 0x02060004u;
        const uint32_t m[3] = {0x0F0F0F0Fu, 0x33333333u, 0x55555555u};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const uint32_t sh = 4u >> k;
            const bool lower = (lane & sh) == 0;
            keep[k] = lower ? m[k] : ~m[k];
            rot[k] = lower ? 32u - sh : sh;
        }
    }
    /* bits of a under m, of b elsewhere (one v_bfi_b32) */
    static __device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
        return b ^ ((a ^ b) & m);
    }
    __device__ __forceinline__ uint32_t operator()(uint32_t v) const {
        uint32_t p;
        p = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F); /* lane ^ 16 */
        v = __builtin_amdgcn_perm(v, p, sel16);
        p = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x201F); /* lane ^ 8 */
        v = __builtin_amdgcn_perm(v, p, sel8);
        p = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F); /* lane ^ 4 */
        v = bfi(keep[0], v, __builtin_amdgcn_alignbit(p, p, rot[0]));
        p = dpp<kDppQuadXor2>(0, v);                                /* lane ^ 2 */
        v = bfi(keep[1], v, __builtin_amdgcn_alignbit(p, p, rot[1]));
        p = dpp<kDppQuadXor1>(0, v);                                /* lane ^ 1 */
        v = bfi(keep[2], v, __builtin_amdgcn_alignbit(p, p, rot[2]));
        return v;
    }
};

/* q minus the code of the lane to the left (lane 0: carry).  The subtraction must stay apart
 * from the DPP move: where carry is known to be 0 the compiler folds the pair into one
 * v_subrev_u32_dpp (wave_shr, bound_ctrl), and on gfx950 that returned the negated difference.
 * The empty asm hides the moved value from that fold and emits nothing. */
__device__ __forceinline__ int32_t diff_left(int32_t q, int32_t carry) {
    uint32_t prev = dpp<kDppWaveShr1>((uint32_t)carry, (uint32_t)q);
    asm("" : "+v"(prev));
    return q - (int32_t)prev;
}

__device__ __forceinline__ float ld_nt_f(const float *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt_f(float *p, float v) { __builtin_nontemporal_store(v, p); }

/* ---- K2c: chunk encode ------------------------------------------------------------------------ */

/* Escape bookkeeping of one encode chunk, kept as in the bitpack encoder: the count, a bit per
 * 256-value tile with an escape, and (lane l) the escape bitmask of 32-value segment l. */
struct ChunkEsc {
    uint32_t escs = 0, tmask = 0, emask = 0;
};

/* Phase 1 of the chunk encoder for one wave's 2048 values: per 64-value tile quantize, take
 * the first difference (the carry supplies lane 0's predecessor: the previous tile's last code,
 * 0 at a chunk's first value), zigzag, OR into the chunk's code OR, transpose, and store the
 * 64 plane words at their plane-major LDS places.  FULL: all 2048 values lie below n. */
template <int V, bool FULL, bool STRIDED>
__device__ __forceinline__ void encode_tiles(const float *__restrict__ x, const Layout &lo, uint64_t cbase,
                                             uint64_t n, const QParams &qp, int32_t carry, uint32_t wave,
                                             uint32_t (*s_words)[ChunkGeom<V>::LDSW], uint32_t *stage_idx,
                                             uint32_t *stage_val, uint32_t orz[ChunkGeom<V>::PER_WAVE],
                                             ChunkEsc &es) {
    using Gm = ChunkGeom<V>;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t h = lane >> 5, b = lane & 31;
    const Transpose tr(lane);
    float xs[kCTilesPerWave];
#pragma unroll
    for (int t = 0; t < kCTilesPerWave; ++t) {
        const uint64_t i = cbase + (uint64_t)t * kCTile + lane;
        if (FULL) xs[t] = ld_nt_f(x + elem_off<STRIDED>(lo, i));
        else xs[t] = i < n ? x[elem_off<STRIDED>(lo, i)] : 0.0f;
    }
#pragma unroll
    for (int t = 0; t < kCTilesPerWave; ++t) {
        const float xv = xs[t];
        /* Quant: the bitpack encoder's fast test (exactly the full rule's acceptance), the full
         * rule in a wave where some lane misses it */
        const float q0f = rintf(xv * qp.r);
        const bool fast = (fabsf(xv - q0f * qp.s) <= qp.eb) && (fabsf(q0f) < qp.tlim);
        int32_t q = (int32_t)q0f;
        if (__ballot(!fast)) {
            uint32_t e = 0;
            if (!fast) q = quantize_slow(xv, q0f, qp, &e);
            const uint64_t M = __ballot(e != 0);
            if (M) {
                es.emask = writelane(es.emask, (uint32_t)M, 2u * t);
                es.emask = writelane(es.emask, (uint32_t)(M >> 32), 2u * t + 1u);
                es.tmask |= 1u << (t / 4);
                const uint32_t r = es.escs + mbcnt64(M);
                if (e && r < (uint32_t)kEscStage) {
                    stage_idx[r] = (uint32_t)(cbase + (uint64_t)t * kCTile + lane);
                    stage_val[r] = __float_as_uint(xv);
                }
                es.escs += (uint32_t)__popcll(M);
            }
        }
        /* Diff: lane 0 takes the carry (0 at a chunk start), the others their left neighbour */
        if (t > 0 && (t * kCTile) % V == 0) carry = 0;
        uint32_t z = zigzag(diff_left(q, carry));
        carry = (int32_t)readlane((uint32_t)q, 63);
        if (!FULL && cbase + (uint64_t)t * kCTile + lane >= n) z = 0; /* padding codes */
        orz[(t * kCTile) / V] |= z;
        /* Bitshuffle: lane 32 h + b -> plane b of group (off mod V) / 32 + h */
        const uint32_t wd = tr(z);
        const uint32_t off = wave * kEncChunk + (uint32_t)t * kCTile; /* value offset in the group */
        s_words[off / V][b * Gm::PS + (off & (uint32_t)(V - 1)) / 32u + h] = wd;
    }
}

/* RZE of one chunk from its LDS planes into dst: the bitmap (V / 32 words; bit k of word k / 32
 * set when plane word k is nonzero), then the nonzero words in order.  Planes at and above wmax
 * are zero and skipped.  Returns the chunk's word count. */
template <int V>
__device__ __forceinline__ uint32_t rze_chunk(const uint32_t *pl, uint32_t wmax, uint32_t *dst) {
    using Gm = ChunkGeom<V>;
    const uint32_t lane = threadIdx.x & 63;
    uint32_t bm0 = 0, bm1 = 0; /* lane l: bitmap word l (and 64 + l) */
    uint32_t run = 0;
    for (uint32_t pb = 0; pb < wmax; ++pb) {
#pragma unroll
        for (int kk = 0; kk < Gm::BATCHES; ++kk) {
            const uint32_t gi = 64u * kk + lane;
            const uint32_t word = (Gm::G >= 64 || gi < (uint32_t)Gm::G) ? pl[pb * Gm::PS + gi] : 0u;
            const uint64_t M = __ballot(word != 0);
            if (word) dst[Gm::BM + run + mbcnt64(M)] = word;
            run += (uint32_t)__popcll(M);
            const uint32_t wi = (pb * Gm::G + 64u * kk) / 32u;
            if (wi < 64) bm0 = writelane(bm0, (uint32_t)M, wi);
            else bm1 = writelane(bm1, (uint32_t)M, wi - 64);
            if (Gm::G >= 64) {
                if (wi + 1 < 64) bm0 = writelane(bm0, (uint32_t)(M >> 32), wi + 1);
                else bm1 = writelane(bm1, (uint32_t)(M >> 32), wi + 1 - 64);
            }
        }
    }
    if (lane < (uint32_t)(Gm::BM < 64 ? Gm::BM : 64)) dst[lane] = bm0;
    if (Gm::BM > 64) dst[64 + lane] = bm1;
    return Gm::BM + run;
}

/* Workgroup of 4 waves over 8192 values; wave w owns the 2048 values of encode chunk c (the
 * unit of the escape bookkeeping and of the scratch slots the compaction copies), which hold
 * 2048 / V coder chunks, or half of one when V = 4096.  Phase 1 (every wave): encode_tiles.
 * Phase 2 (after a barrier; the wave owning a chunk's first values): RZE of the chunk into the
 * scratch slot and its word count into the size section (stream or staging).  A wave's chunks
 * lie back to back in its slot, and a 4096-value chunk fills the slots of both its waves (the
 * second reports 0 words), so the compaction's copy of each slot in order yields the chunks in
 * order. */
template <int V, bool STRIDED>
__device__ __forceinline__ void chunk_encode_body(const float *__restrict__ x, PlanArgs pa,
                                                  Workspace ws, uint8_t *__restrict__ sizes_dst,
                                                  uint64_t sizes_bytes) {
    using Gm = ChunkGeom<V>;
    constexpr int kBufs = kEncWaves * kEncChunk / V;
    __shared__ uint32_t s_words[kBufs][Gm::LDSW];
    __shared__ uint32_t s_stage[kEncWaves][2][kEscStage];
    __shared__ uint32_t s_or[kEncWaves][Gm::PER_WAVE];
    __shared__ uint32_t s_grp[2][kEncWaves];

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t c = blockIdx.x * kEncWaves + wave;
    const DevInfo *info = ws.info;
    const uint64_t n = pa.n;
    const uint64_t cbase = (uint64_t)c * kEncChunk;
    ChunkEsc es;
    uint32_t wsum = 0;

    if (info->valid) {  /* the same for every workgroup: the barrier below is uniform */
        QParams qp;
        qp.eb = info->eb_f;
        qp.s = info->s;
        qp.r = info->r;
        qp.T = pa.T;
        qp.tlim = (float)(1u << pa.T);
        /* the predecessor of the wave's first value when it does not start a chunk (second half
         * of a 4096-value chunk): the code of the value before it, 0 if that value escapes */
        int32_t carry = 0;
        if ((cbase & (uint64_t)(V - 1)) != 0 && cbase < n) {
            const float xp = x[elem_off<STRIDED>(pa.lay, cbase - 1)];
            uint32_t e;
            const int32_t qprev = quantize_slow(xp, rintf(xp * qp.r), qp, &e);
            carry = e ? 0 : qprev;
        }
        uint32_t orz[Gm::PER_WAVE];
#pragma unroll
        for (int k = 0; k < Gm::PER_WAVE; ++k) orz[k] = 0;
        if (cbase + kEncChunk <= n)
            encode_tiles<V, true, STRIDED>(x, pa.lay, cbase, n, qp, carry, wave, s_words, s_stage[wave][0],
                                           s_stage[wave][1], orz, es);
        else
            encode_tiles<V, false, STRIDED>(x, pa.lay, cbase, n, qp, carry, wave, s_words, s_stage[wave][0],
                                            s_stage[wave][1], orz, es);
#pragma unroll
        for (int k = 0; k < Gm::PER_WAVE; ++k) {
            const uint32_t o = wave_or(orz[k]);
            if (lane == 0) s_or[wave][k] = o;
        }
        __syncthreads();

        const uint64_t ncv = (n + V - 1) / V;
        if (Gm::WAVES == 1 || (wave & 1u) == 0) {
            uint32_t *slot = ws.scratch + (uint64_t)c * pa.slot;
            uint32_t *sz = reinterpret_cast<uint32_t *>(sizes_dst);
#pragma unroll
            for (int k = 0; k < Gm::PER_WAVE; ++k) {
                const uint64_t cv = (cbase + (uint64_t)k * V) / V;
                if (cv < ncv) {
                    uint32_t orc = s_or[wave][k];
                    if (Gm::WAVES == 2) orc |= s_or[wave + 1][0];
                    const uint32_t wmax = orc ? 32u - (uint32_t)__builtin_clz(orc) : 0u;
                    const uint32_t size = rze_chunk<V>(s_words[(wave * kEncChunk + (uint32_t)k * V) / V], wmax,
                                                       slot + wsum);
                    wsum += size;
                    if (lane == 0 && 4 * cv < sizes_bytes) sz[cv] = size;
                    if (cv == ncv - 1) {
                        /* zero the size section's pad up to its 16-byte end */
                        const uint64_t pz = cv + 1 + lane;
                        if (pz < align16(4 * ncv) / 4 && 4 * pz < sizes_bytes) sz[pz] = 0u;
                    }
                }
            }
        }
        if (c < pa.nchunks) {
            if (lane < es.escs && lane < (uint32_t)kEscStage) {
                ws.stage_idx[(uint64_t)c * kEscStage + lane] = s_stage[wave][0][lane];
                ws.stage_val[(uint64_t)c * kEscStage + lane] = s_stage[wave][1][lane];
            }
            /* the escape bitmasks are read by the compaction only for a chunk with more escapes
             * than the staging holds */
            if (es.tmask && es.escs > (uint32_t)kEscStage) ws.emask[(uint64_t)c * kEncSegs + lane] = es.emask;
            if (lane == 0) {
                ws.chunk_words[c] = wsum;
                ws.chunk_esc[c] = es.escs;
                ws.chunk_tmask[c] = es.tmask;
            }
        }
    }
    if (c >= pa.nchunks) {
        wsum = 0;
        es.escs = 0;
    }
    if (lane == 0) {
        s_grp[0][wave] = wsum;
        s_grp[1][wave] = es.escs;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t sw = 0, se = 0;
#pragma unroll
        for (int k = 0; k < kEncWaves; ++k) {
            sw += s_grp[0][k];
            se += s_grp[1][k];
        }
        ws.group_words[blockIdx.x] = sw;
        ws.group_esc[blockIdx.x] = se;
    }
}

template <int V, bool STRIDED>
__global__ __launch_bounds__(kEncThreads) void chunk_encode_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    const uint32_t f = blockIdx.y;
    const Workspace w = lane_ws(ws, f, fs.ws_stride);
    uint8_t *sd = (fs.wdirect >> f) & 1u ? pick(fs.dst, f) + kHeaderBytes : w.widths;
    chunk_encode_body<V, STRIDED>(reinterpret_cast<const float *>(pick(fs.src, f)), pa, w, sd, pa.wsec);
}

/* ---- K7c: chunk decode ------------------------------------------------------------------------ */

/* Decode tiles [t0, t0 + NT) of a chunk: lane 32 h + b reads plane b of group 2 t + h (planes
 * at and above wmax are zero), the transpose turns that into one code per lane, then the zigzag
 * inverse and a wave prefix sum plus the carry (the previous tile's last code) undo the first
 * difference, and f32(f32(q) * s) is stored.  The NT tiles' transposes and scans are
 * independent; only the carry chains them. */
/* Word g of bit plane b of a chunk (the word of the plane for group g), for the tile loops. */
/* From planes rebuilt in LDS, PS words per plane, holding groups g0 onwards. */
struct PlaneFetch {
    const uint32_t *pl;
    uint32_t ps, g0;
    __device__ __forceinline__ uint32_t operator()(uint32_t b, uint32_t g) const { return pl[b * ps + g - g0]; }
};

/* From the chunk's RZE words staged as they lie in the stream (raw[0] = the first bitmap word)
 * and the exclusive popcount prefix of the bitmap words: a word whose bitmap bit is clear is 0,
 * else it is nonzero word number (prefix + the set bits below it in its bitmap word). */
template <int V>
struct RawFetch {
    const uint32_t *raw;
    const uint32_t *pre;
    __device__ __forceinline__ uint32_t operator()(uint32_t b, uint32_t g) const {
        const uint32_t wi = b * (uint32_t)ChunkGeom<V>::G + g, k = wi >> 5, j = wi & 31u;
        const uint32_t bmw = raw[k];
        const uint32_t below = (uint32_t)__popc(bmw & ((1u << j) - 1u));
        return ((bmw >> j) & 1u) ? raw[ChunkGeom<V>::BM + pre[k] + below] : 0u;
    }
};

template <int V, int NT, bool FULL, bool STRIDED, typename F>
__device__ __forceinline__ void decode_tiles(const F &fetch, uint32_t t0, uint32_t wmax, const Transpose &tr,
                                             float s, uint32_t &carry, float *__restrict__ out, const Layout &lo,
                                             uint32_t cbase, uint32_t n) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t h = lane >> 5, b = lane & 31;
    uint32_t incl[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const uint32_t word = b < wmax ? fetch(b, 2u * (t0 + k) + h) : 0u;
        incl[k] = wave_incl_scan((uint32_t)unzigzag(tr(word)));
    }
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const uint32_t q = incl[k] + carry;
        carry = readlane(q, 63);
        const float y = (float)(int32_t)q * s;
        const uint32_t i = cbase + (t0 + k) * kCTile + lane;
        if (FULL || i < n) st_nt_f(out + elem_off<STRIDED>(lo, i), y);
    }
}

/* Decode 4 NQ full tiles from tile t0 on, four at a time: each tile's transpose gives one code
 * per lane (value 64 t + lane), the four tiles' codes go through a 1 KB LDS scratch so that lane
 * l holds values 4 l .. 4 l + 3 of the 256, and then one in-lane running sum, one wave scan of
 * the lane totals and the carry undo the first difference for all four tiles, and one 128-bit
 * store writes the lane's four values.  The scratch belongs to the wave: a wave-level release /
 * acquire after the stores and again after the read orders every lane's accesses, so the next
 * group's stores cannot pass this group's read (by the compiler or by the LDS). */
template <int V, int NQ, bool STRIDED, typename F>
__device__ __forceinline__ void decode_quads(const F &fetch, uint32_t t0, uint32_t wmax, const Transpose &tr,
                                             float s, uint32_t &carry, float *__restrict__ out, const Layout &lo,
                                             uint32_t cbase, uint32_t *sx) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t h = lane >> 5, b = lane & 31;
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
        const uint32_t t = t0 + 4u * g;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t word = b < wmax ? fetch(b, 2u * (t + k) + h) : 0u;
            sx[64 * k + lane] = (uint32_t)unzigzag(tr(word));
        }
        wave_lds_sync();
        const uint4 v = reinterpret_cast<const uint4 *>(sx)[lane];
        wave_lds_sync();
        const uint32_t r1 = v.x + v.y, r2 = r1 + v.z, r3 = r2 + v.w;
        const uint32_t incl = wave_incl_scan(r3);
        const uint32_t base = carry + incl - r3;
        carry += readlane(incl, 63);
        float4 o;
        o.x = (float)(int32_t)(base + v.x) * s;
        o.y = (float)(int32_t)(base + r1) * s;
        o.z = (float)(int32_t)(base + r2) * s;
        o.w = (float)(int32_t)(base + r3) * s;
        store4<STRIDED>(out, lo, (uint64_t)cbase + (uint64_t)t * kCTile + 4u * lane, o);
    }
}

/* One wave per chunk.  The chunk's bitmap sits in two VGPRs (lane l: bitmap words l and
 * 64 + l); its popcount must equal the chunk's word count minus the bitmap, else the stream is
 * flagged.  A 1024-value chunk is staged in LDS as its words lie in the stream, loaded
 * together with the bitmap, and each tile reads a plane word from it by its rank among the
 * nonzero words (RawFetch).  Larger chunks rebuild their planes below the highest nonzero one
 * in LDS (a 4096-value chunk half a chunk at a time): per 64-word batch the batch's bitmap bits
 * and mbcnt give each present word's position (PlaneFetch); all of a rebuild's loads are issued
 * before its LDS stores.  Then the tile loops, eight tiles at a time for a full chunk.  (A
 * 2048-value chunk read in place was slower: 134 -> 149 us on the 512^3 field.) */
template <int V, bool STRIDED>
__device__ __forceinline__ void chunk_decode_body(const uint8_t *__restrict__ in, PlanArgs pa,
                                                  Workspace ws, float *__restrict__ out) {
    using Gm = ChunkGeom<V>;
    __shared__ uint4 s_lds4[kWavesPerBlock][Gm::DEC_LDSW / 4];
    __shared__ uint4 s_x4[kWavesPerBlock][4 * kCTile / 4];
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t c = blockIdx.x * kWavesPerBlock + wave;
    if (c >= pa.dchunks) return;
    DevInfo *info = ws.info;
    if (info->err) return;
    const uint32_t n = (uint32_t)pa.n;
    const uint32_t cbase = c * (uint32_t)V;
    const uint32_t cnt = (n - cbase < (uint32_t)V) ? n - cbase : (uint32_t)V;
    if (info->mode == 1) {
        const uint32_t *srcw = reinterpret_cast<const uint32_t *>(in + kHeaderBytes) + cbase;
        uint32_t *ob = reinterpret_cast<uint32_t *>(out);
        if (!STRIDED && cnt == (uint32_t)V) {
            const uint4 *s4 = reinterpret_cast<const uint4 *>(srcw);
            uint4 *d4 = reinterpret_cast<uint4 *>(ob + cbase);
            uint4 t[V / 4 / kWave];
#pragma unroll
            for (int i = 0; i < V / 4 / kWave; ++i) t[i] = ld_nt(s4 + lane + kWave * i);
#pragma unroll
            for (int i = 0; i < V / 4 / kWave; ++i) st_nt(d4 + lane + kWave * i, t[i]);
        } else {
            for (uint32_t i = lane; i < cnt; i += kWave) ob[elem_off<STRIDED>(pa.lay, cbase + i)] = srcw[i];
        }
        return;
    }
    const uint32_t W = chunk_offset<kDecChunksPerGroup>(ws.gpre_words, ws.chunk_words, c);
    const uint32_t P = ws.chunk_words[c];
    const uint32_t *blob = reinterpret_cast<const uint32_t *>(in + info->payload_off) + W;
    const uint32_t bm0 = lane < (uint32_t)(Gm::BM < 64 ? Gm::BM : 64) ? blob[lane] : 0u;
    const uint32_t bm1 = Gm::BM > 64 ? blob[64 + lane] : 0u;
    /* RAW: all of the chunk's words, as they lie in the stream, are loaded with its bitmap
     * (16-byte units from the unit holding its first word) */
    constexpr int kRounds = Gm::RAW ? (Gm::RAWW / 4 + kWave - 1) / kWave : 1;
    uint4 v[kRounds];
    uint32_t lb = 0, units = 0;
    if constexpr (Gm::RAW) {
        const uint64_t sw = info->payload_off / 4 + W;
        const uint64_t a0 = sw & ~(uint64_t)3;
        lb = (uint32_t)(sw - a0);
        units = (lb + P + 3) >> 2;
        if (units > (uint32_t)(Gm::RAWW / 4)) units = Gm::RAWW / 4;
        const uint4 *src = reinterpret_cast<const uint4 *>(in) + a0 / 4;
        const uint32_t rounds = (units + kWave - 1) / kWave;
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const uint32_t u = lane + (uint32_t)r * kWave;
            v[r] = make_uint4(0, 0, 0, 0);
            if ((uint32_t)r < rounds && u < units) v[r] = src[u];
        }
    }
    const uint32_t pc = wave_incl_scan((uint32_t)__popc(bm0) + (uint32_t)__popc(bm1));
    if (readlane(pc, 63) + Gm::BM != P) {
        if (lane == 0) atomicOr(&info->sticky, 1u);
        return;
    }
    const uint64_t nz0 = __ballot(bm0 != 0), nz1 = __ballot(bm1 != 0);
    int top = -1;
    if (nz1) top = 64 + 63 - __clzll((long long)nz1);
    else if (nz0) top = 63 - __clzll((long long)nz0);
    const uint32_t wmax = top < 0 ? 0u : (uint32_t)top * 32u / Gm::G + 1u;
    uint32_t *pl = reinterpret_cast<uint32_t *>(s_lds4[wave]);
    const Transpose tr(lane);
    const float s = info->dec_s;
    uint32_t carry = 0;
    uint32_t *sx = reinterpret_cast<uint32_t *>(s_x4[wave]);
    if constexpr (Gm::HALVES) {
        /* A 4096-value chunk goes through a half-size buffer: the planes' words of groups 0-63
         * (tiles 0-31), then those of groups 64-127 (tiles 32-63), each half's loads issued
         * before its LDS stores.  The running word count covers both halves' bitmap bits, and
         * the running sum carries from the first half into the second. */
        constexpr int PSH = Gm::PSH;
        const uint32_t ntiles = (cnt + kCTile - 1) / kCTile;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint32_t t0 = 32u * hh;
            if (t0 >= ntiles) break;
            uint32_t wv[32];
            uint32_t run = 0;
#pragma unroll
            for (int pb = 0; pb < 32; ++pb) {
                wv[pb] = 0;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if ((uint32_t)pb < wmax) {
                        const uint32_t wi = (pb * Gm::G + 64 * kk) / 32;
                        const uint32_t lo = wi < 64 ? readlane(bm0, (int)wi) : readlane(bm1, (int)(wi - 64));
                        const uint32_t hi = wi + 1 < 64 ? readlane(bm0, (int)(wi + 1)) : readlane(bm1, (int)(wi + 1 - 64));
                        const uint64_t M = (uint64_t)lo | ((uint64_t)hi << 32);
                        if (kk == hh && ((M >> lane) & 1u)) wv[pb] = blob[Gm::BM + run + mbcnt64(M)];
                        run += (uint32_t)__popcll(M);
                    }
                }
            }
            wave_lds_sync(); /* the first half's reads are done before the second half's stores */
#pragma unroll
            for (int pb = 0; pb < 32; ++pb)
                if ((uint32_t)pb < wmax) pl[pb * PSH + lane] = wv[pb];
            wave_lds_sync();
            const PlaneFetch fetch{pl, (uint32_t)PSH, 2u * t0};
            if (cnt == (uint32_t)V) {
                for (uint32_t t = t0; t < t0 + 32u; t += 8)
                    decode_quads<V, 2, STRIDED>(fetch, t, wmax, tr, s, carry, out, pa.lay, cbase, sx);
            } else {
                const uint32_t te = ntiles < t0 + 32u ? ntiles : t0 + 32u;
                for (uint32_t t = t0; t < te; ++t)
                    decode_tiles<V, 1, false, STRIDED>(fetch, t, wmax, tr, s, carry, out, pa.lay, cbase, n);
            }
        }
    } else if constexpr (Gm::RAW) {
        /* the staged words into LDS, the bitmap's exclusive popcount prefix after them; the
         * tile loops then read each plane word in place */
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const uint32_t u = lane + (uint32_t)r * kWave;
            if (u < units) s_lds4[wave][u] = v[r];
        }
        if (lane < (uint32_t)Gm::BM) pl[Gm::RAWW + lane] = pc - (uint32_t)__popc(bm0);
        wave_lds_sync();
        const RawFetch<V> fetch{pl + lb, pl + Gm::RAWW};
        if (cnt == (uint32_t)V) {
            for (uint32_t t = 0; t < (uint32_t)Gm::TILES; t += 8)
                decode_quads<V, 2, STRIDED>(fetch, t, wmax, tr, s, carry, out, pa.lay, cbase, sx);
        } else {
            const uint32_t ntiles = (cnt + kCTile - 1) / kCTile;
            for (uint32_t t = 0; t < ntiles; ++t)
                decode_tiles<V, 1, false, STRIDED>(fetch, t, wmax, tr, s, carry, out, pa.lay, cbase, n);
        }
    } else {
        /* un-RZE: every plane's loads first (into registers), then the LDS stores */
        uint32_t wv[32 * Gm::BATCHES];
        uint32_t run = 0;
#pragma unroll
        for (int pb = 0; pb < 32; ++pb) {
#pragma unroll
            for (int kk = 0; kk < Gm::BATCHES; ++kk) {
                uint32_t word = 0;
                if ((uint32_t)pb < wmax) {
                    const uint32_t wi = (pb * Gm::G + 64 * kk) / 32;
                    const uint32_t lo = wi < 64 ? readlane(bm0, (int)wi) : readlane(bm1, (int)(wi - 64));
                    uint32_t hi = 0;
                    if (Gm::G >= 64) hi = wi + 1 < 64 ? readlane(bm0, (int)(wi + 1)) : readlane(bm1, (int)(wi + 1 - 64));
                    const uint64_t M = (uint64_t)lo | ((uint64_t)hi << 32);
                    if ((M >> lane) & 1u) word = blob[Gm::BM + run + mbcnt64(M)];
                    run += (uint32_t)__popcll(M);
                }
                wv[pb * Gm::BATCHES + kk] = word;
            }
        }
#pragma unroll
        for (int pb = 0; pb < 32; ++pb) {
            if ((uint32_t)pb < wmax) {
#pragma unroll
                for (int kk = 0; kk < Gm::BATCHES; ++kk) {
                    const uint32_t gi = 64u * kk + lane;
                    if (Gm::G >= 64 || gi < (uint32_t)Gm::G) pl[pb * Gm::PS + gi] = wv[pb * Gm::BATCHES + kk];
                }
            }
        }
        wave_lds_sync();
        const PlaneFetch fetch{pl, (uint32_t)Gm::PS, 0u};
        if (cnt == (uint32_t)V) {
            for (uint32_t t = 0; t < (uint32_t)Gm::TILES; t += 8)
                decode_quads<V, 2, STRIDED>(fetch, t, wmax, tr, s, carry, out, pa.lay, cbase, sx);
        } else {
            const uint32_t ntiles = (cnt + kCTile - 1) / kCTile;
            for (uint32_t t = 0; t < ntiles; ++t)
                decode_tiles<V, 1, false, STRIDED>(fetch, t, wmax, tr, s, carry, out, pa.lay, cbase, n);
        }
    }
}

template <int V, bool STRIDED>
__global__ __launch_bounds__(kBlockThreads) void chunk_decode_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    const uint32_t f = blockIdx.y;
    chunk_decode_body<V, STRIDED>(pick(fs.src, f), pa, lane_ws(ws, f, fs.ws_stride),
                                  reinterpret_cast<float *>(pick(fs.dst, f)));
}

template <int V>
hipError_t chunk_encode_v(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                          hipStream_t stream) {
    const dim3 grid(pa.ngroups, nf), block(kEncThreads);
    if (pa.lay.strided)
        eblc_launch((chunk_encode_kernel<V, true>), grid, block, 0, stream, fs, pa, ws);
    else
        eblc_launch((chunk_encode_kernel<V, false>), grid, block, 0, stream, fs, pa, ws);
    return hipGetLastError();
}

template <int V>
hipError_t chunk_decode_v(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                          hipStream_t stream) {
    const dim3 grid(pa.dgroups, nf), block(kBlockThreads);
    if (pa.lay.strided)
        eblc_launch((chunk_decode_kernel<V, true>), grid, block, 0, stream, fs, pa, ws);
    else
        eblc_launch((chunk_decode_kernel<V, false>), grid, block, 0, stream, fs, pa, ws);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_encode(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                               hipStream_t stream) {
    switch (pa.V) {
        case 1024: return chunk_encode_v<1024>(fs, nf, pa, ws, stream);
        case 2048: return chunk_encode_v<2048>(fs, nf, pa, ws, stream);
        case 4096: return chunk_encode_v<4096>(fs, nf, pa, ws, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_decode(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                               hipStream_t stream) {
    switch (pa.V) {
        case 1024: return chunk_decode_v<1024>(fs, nf, pa, ws, stream);
        case 2048: return chunk_decode_v<2048>(fs, nf, pa, ws, stream);
        case 4096: return chunk_decode_v<4096>(fs, nf, pa, ws, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace eblc
