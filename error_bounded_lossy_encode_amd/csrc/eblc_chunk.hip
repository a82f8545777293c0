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
 * gfx950 mapping.  Lane L of a wave owns group L of the wave's 2048 values (values 32 L .. 32 L
 * + 31), so every step but RZE runs inside the lane, on its registers:
 *  - the field arrives by coalesced 128-bit loads and passes through LDS, where group L's eight
 *    16-byte quads sit in slots 8 L .. 8 L + 7 with the quad index XORed by (L ^ L / 8) mod 8:
 *    the coalesced writes and each lane's reads of its own quads then hit distinct banks;
 *  - Quant and Diff run over the lane's 32 values; the first value's predecessor is the last
 *    code of the lane to the left (one DPP move);
 *  - Bitshuffle is the transpose of the lane's 32 x 32 bit matrix: five stages of block swaps
 *    between register pairs (v_perm_b32 for the 16- and 8-bit blocks, a shift and v_bfi_b32
 *    for the 4-, 2- and 1-bit ones), after which register b holds the group's plane-b word;
 *  - the zigzag fold is applied to planes: plane 0 of the folded codes is the sign plane of the
 *    differences and plane b >= 1 is their plane b - 1 XOR the sign plane, one XOR per plane
 *    instead of three operations per code;
 *  - RZE walks the planes: a ballot of the wave's nonzero words gives the plane's bitmap bits,
 *    and mbcnt the place of each nonzero word.
 * A 1024-value chunk is half a wave; a 4096-value chunk spans two waves of a workgroup, which
 * trade their per-plane word counts through LDS.  Decoding runs the steps backwards (the
 * transpose is its own inverse): one vector load brings the chunk's bitmap words (lane k, word
 * k), readlane hands each plane's bitmap to the whole wave, each lane loads its group's nonzero
 * words under it, unfolds the zigzag on planes, transposes, and sums its
 * differences after a wave scan of the lane totals; the values go back through LDS in the same
 * swizzled order for coalesced stores.
 */
#include "eblc_device.h"

#include <utility>

namespace eblc {
namespace {

constexpr int kWaveQuads = kEncChunk / 4;      /* 16-byte quads of a wave's 2048 values */
constexpr int kLaneQuads = kWaveQuads / kWave;  /* quads per lane in a coalesced pass */

template <int V>
struct ChunkGeom {
    static constexpr int G = V / 32;            /* groups of 32 codes = words per bit plane */
    static constexpr int BM = V / 32;           /* bitmap words of RZE */
    static constexpr int WAVES = V > kEncChunk ? V / kEncChunk : 1;      /* waves per chunk */
    static constexpr int PER_WAVE = V < kEncChunk ? kEncChunk / V : 1;   /* chunks per wave */
    static_assert(V == 1024 || V == 2048 || V == 4096, "chunk of 4, 8 or 16 KiB");
    static_assert(PER_WAVE * (BM + V) <= WAVES * (kEncChunk + kEncChunk / 32), "scratch slots of 2112 words");
};

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

/* old with lane AT replaced by the wave-uniform value v (one v_writelane_b32; its lane select is
 * an immediate, as a second scalar operand would break the one-scalar-read limit).  v goes
 * through readfirstlane, which is free for a value in an SGPR and otherwise makes sure the asm
 * gets one: the compiler may keep a copy of a uniform value in a VGPR. */
template <int AT>
__device__ __forceinline__ uint32_t writelane(uint32_t old, uint32_t v) {
    asm("v_writelane_b32 %0, %1, %2" : "+v"(old) : "s"(__builtin_amdgcn_readfirstlane(v)), "n"(AT));
    return old;
}

using Planes = std::make_integer_sequence<int, 32>;

/* LDS slot (16 bytes) of quad g of a wave's 2048 values: group L = g / 8 keeps slots 8 L ..
 * 8 L + 7 with the quad's index in its group XORed by (L ^ L / 8) mod 8.  Eight lanes reading
 * quad j of their eight groups, and sixteen lanes writing 16 consecutive quads, then touch 128
 * (256) distinct bytes modulo the bank width.  For g = 64 k + l (k < 8) the slot is 64 k +
 * (quad_slot(l) ^ k), and for g = 8 L + j it is quad_slot(8 L) ^ j. */
__device__ __forceinline__ uint32_t quad_slot(uint32_t g) {
    const uint32_t L = g >> 3;
    return (g & ~7u) | ((g ^ L ^ (L >> 3)) & 7u);
}

__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

/* One stage of the transpose: for every register pair (k, k + J) below N, k without bit J, the
 * bits of k whose index has bit J set trade places with the bits of k + J whose index has it
 * clear. */
template <int J, int N>
__device__ __forceinline__ void swap_stage(uint32_t w[32], uint32_t m) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
        if (k & J) continue;
        const uint32_t a = w[k], b = w[k + J];
        w[k] = bfi(m, a, b << J);
        w[k + J] = bfi(m, a >> J, b);
    }
}

/* The 8-, 4-, 2- and 1-bit stages on w[0..N). */
template <int N>
__device__ __forceinline__ void low_stages(uint32_t w[32]) {
#pragma unroll
    for (int k = 0; k < N; ++k) { /* bytes: (a0, b0, a2, b2) and (a1, b1, a3, b3) */
        if (k & 8) continue;
        const uint32_t a = w[k], b = w[k + 8];
        w[k] = __builtin_amdgcn_perm(b, a, 0x06020400u);
        w[k + 8] = __builtin_amdgcn_perm(b, a, 0x07030501u);
    }
    swap_stage<4, N>(w, 0x0F0F0F0Fu);
    swap_stage<2, N>(w, 0x33333333u);
    swap_stage<1, N>(w, 0x55555555u);
}

/* 32 x 32 bit transpose in place: on exit bit i of w[b] is bit b of w[i] on entry.  (The stages
 * act on different bits of the row and column indexes, so they commute.) */
__device__ __forceinline__ void transpose32(uint32_t w[32]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) { /* 16-bit blocks: (a.lo, b.lo) and (a.hi, b.hi) */
        const uint32_t a = w[k], b = w[k + 16];
        w[k] = __builtin_amdgcn_perm(b, a, 0x05040100u);
        w[k + 16] = __builtin_amdgcn_perm(b, a, 0x07060302u);
    }
    low_stages<32>(w);
}

/* The transpose of 32 codes that are sign extensions of their low 16 bits, into planes 0-15
 * (planes 16-31 would all equal plane 15): the 16-bit stage only gathers the low halves, and the
 * other stages run on half the registers. */
__device__ __forceinline__ void transpose_low16(uint32_t w[32]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k] = __builtin_amdgcn_perm(w[k + 16], w[k], 0x05040100u);
    low_stages<16>(w);
}

/* The lane's group leaves LDS as 32 values in order; sx is the wave's 2048-value staging. */
__device__ __forceinline__ void read_group(const uint4 *sx, uint32_t v[32]) {
    const uint32_t s0 = quad_slot(8u * (threadIdx.x & 63));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint4 u = sx[s0 ^ (uint32_t)j];
        v[4 * j] = u.x;
        v[4 * j + 1] = u.y;
        v[4 * j + 2] = u.z;
        v[4 * j + 3] = u.w;
    }
}

/* Word i of p, i < 2^30: the byte offset is formed in 32 bits, so the load takes the pointer in
 * SGPRs and one VGPR offset. */
__device__ __forceinline__ uint32_t word_at(const uint32_t *p, uint32_t i) {
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(p) + 4u * i);
}

__device__ __forceinline__ uint32_t lds_value(const uint4 *sx, uint32_t v) {
    return reinterpret_cast<const uint32_t *>(sx)[4u * quad_slot(v >> 2) + (v & 3u)];
}

/* ---- K2c: chunk encode ------------------------------------------------------------------------ */

/* The wave's 2048 values from value cbase on (0 from n on) into LDS.  FULL: all below n. */
template <bool FULL, bool STRIDED>
__device__ __forceinline__ void stage_values(const float *__restrict__ x, const Layout &lo, uint64_t cbase,
                                             uint64_t n, uint4 *sx) {
    const uint32_t lane = threadIdx.x & 63;
    if (FULL) {
        float4 v[kLaneQuads];
#pragma unroll
        for (int k = 0; k < kLaneQuads; ++k) v[k] = load4<STRIDED>(x, lo, cbase + 4u * (kWave * k + lane));
        const uint32_t s0 = quad_slot(lane);
#pragma unroll
        for (int k = 0; k < kLaneQuads; ++k)
            sx[kWave * k + (s0 ^ (uint32_t)k)] = make_uint4(__float_as_uint(v[k].x), __float_as_uint(v[k].y),
                                                            __float_as_uint(v[k].z), __float_as_uint(v[k].w));
    } else {
        uint32_t *sw = reinterpret_cast<uint32_t *>(sx);
#pragma unroll 4
        for (int k = 0; k < kEncChunk / kWave; ++k) {
            const uint32_t v = kWave * k + lane;
            const uint64_t i = cbase + v;
            const float xv = i < n ? x[elem_off<STRIDED>(lo, i)] : 0.0f;
            sw[4u * quad_slot(v >> 2) + (v & 3u)] = __float_as_uint(xv);
        }
    }
    wave_lds_sync();
}

/* Quant of the lane's group: q[i] is value i's code (0 if it escapes); returns the escape
 * bitmask (bit i: value i).  The fast test is the full rule's first acceptance exactly (the
 * bitpack encoder states why); the full rule runs only in a wave where a lane misses it, on
 * values read again from LDS so that the first pass keeps no copy of them. */
__device__ __forceinline__ uint32_t quantize_group(const uint4 *sx, const QParams &qp, int32_t q[32], float &qmax) {
    uint32_t xv[32];
    read_group(sx, xv);
    bool fast = true;
    float qabs = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const float x = __uint_as_float(xv[i]);
        const float q0f = rintf(x * qp.r);
        fast = fast && (fabsf(x - q0f * qp.s) <= qp.eb);
        qabs = fmaxf(qabs, fabsf(q0f));
        q[i] = (int32_t)q0f;
    }
    fast = fast && (qabs < qp.tlim);
    qmax = qabs;
    uint32_t emask = 0;
    if (__ballot(!fast)) {
        /* the full rule, a quad at a time from LDS (the scheduling barriers keep each quad's read
         * next to its use, so that the pass does not hold all 32 values next to the codes) */
        wave_lds_sync();
        const uint32_t s0 = quad_slot(8u * (threadIdx.x & 63));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            const uint4 u = sx[s0 ^ (uint32_t)j];
            const float xf[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                                 __uint_as_float(u.w)};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = 4 * j + k;
                const float q0f = rintf(xf[k] * qp.r);
                if (!((fabsf(xf[k] - q0f * qp.s) <= qp.eb) && (fabsf(q0f) < qp.tlim))) {
                    uint32_t e;
                    q[i] = quantize_slow(xf[k], q0f, qp, &e);
                    emask |= e << i;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return emask;
}

/* The chunk's first kEscStage escapes, in index order, into the staging of encode chunk c, and
 * the escape count and tile mask (bit t: some value of 256-value tile t escapes). */
__device__ __forceinline__ void stage_escapes(const uint4 *sx, uint32_t emask, uint64_t cbase, uint32_t c,
                                              const Workspace &ws, uint32_t &escs, uint32_t &tmask) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t cnt = (uint32_t)__popc(emask);
    const uint32_t incl = wave_incl_scan(cnt);
    escs = readlane(incl, 63);
    uint32_t r = incl - cnt;
    uint32_t m = emask;
    while (m && r < (uint32_t)kEscStage) {
        const uint32_t i = (uint32_t)__builtin_ctz(m);
        const uint32_t v = 32u * lane + i;
        ws.stage_idx[(uint64_t)c * kEscStage + r] = (uint32_t)(cbase + v);
        ws.stage_val[(uint64_t)c * kEscStage + r] = lds_value(sx, v);
        ++r;
        m &= m - 1;
    }
    const uint64_t E = __ballot(emask != 0);
    tmask = 0;
#pragma unroll
    for (int t = 0; t < kEncChunk / kEncTile; ++t)
        if ((E >> (kSegsPerEncTile * t)) & ((1u << kSegsPerEncTile) - 1u)) tmask |= 1u << t;
}

/* Diff of the lane's codes into w: the first value's predecessor is the last code of the lane to
 * the left, `carry` for lane 0 (and 0 for lane 32 when it starts a 1024-value chunk).  Values at
 * and after n (FULL: none) get difference 0, the padding codes.  The subtraction of the moved
 * code stays apart from the DPP move: where carry is known to be 0 the compiler folds the pair
 * into one v_subrev_u32_dpp (wave_shr, bound_ctrl), and on gfx950 that returned the negated
 * difference.  The empty asm hides the moved value from that fold and emits nothing. */
template <int V, bool FULL>
__device__ __forceinline__ void diff_group(const int32_t q[32], uint32_t carry, uint64_t gbase, uint64_t n,
                                           uint32_t w[32]) {
    uint32_t prev = dpp<kDppWaveShr1>(carry, (uint32_t)q[31]);
    asm("" : "+v"(prev));
    if (V < kEncChunk && (threadIdx.x & 63) == 32) prev = 0;
#pragma unroll
    for (int i = 31; i > 0; --i) w[i] = (uint32_t)q[i] - (uint32_t)q[i - 1];
    w[0] = (uint32_t)q[0] - prev;
    if (!FULL) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (gbase + (uint64_t)i >= n) w[i] = 0;
    }
}

/* Zigzag fold of the codes whose planes w[0..NPL) hold, applied to the planes: NPL = 32, or 16
 * for codes that are sign extensions of their low 16 bits (their folded planes 16-31 are 0). */
template <int NPL>
__device__ __forceinline__ void zigzag_planes(uint32_t w[32]) {
    const uint32_t sgn = w[NPL - 1];
#pragma unroll
    for (int b = NPL - 1; b > 0; --b) w[b] = w[b - 1] ^ sgn;
    w[0] = sgn;
}

/* The inverse of the full fold. */
__device__ __forceinline__ void unzigzag_planes(uint32_t w[32]) {
    const uint32_t sgn = w[0];
#pragma unroll
    for (int b = 0; b < 31; ++b) w[b] = w[b + 1] ^ sgn;
    w[31] = sgn;
}

/* RZE, plane by plane.  Plane B's words are the wave's w[B]; M = ballot(w[B] != 0).  A plane
 * with no nonzero word only has its (zero) bitmap bits. */

/* A 2048-value chunk (the wave's 64 groups): bitmap words 2 B, 2 B + 1 are M's halves. */
template <int B>
__device__ __forceinline__ void rze_wave_plane(const uint32_t w[32], uint32_t *__restrict__ dst, uint32_t &bm,
                                               uint32_t &run) {
    constexpr uint32_t BM = ChunkGeom<2048>::BM;
    const uint64_t M = __ballot(w[B] != 0);
    if (M) {
        if (w[B] != 0) dst[BM + run + mbcnt64(M)] = w[B];
        run += (uint32_t)__popcll(M);
        bm = writelane<2 * B>(bm, (uint32_t)M);
        bm = writelane<2 * B + 1>(bm, (uint32_t)(M >> 32));
    }
}

/* Returns the chunk's word count. */
template <int... B>
__device__ __forceinline__ uint32_t rze_wave(std::integer_sequence<int, B...>, const uint32_t w[32],
                                             uint32_t *__restrict__ dst) {
    uint32_t bm = 0, run = 0;
    (rze_wave_plane<B>(w, dst, bm, run), ...);
    dst[threadIdx.x & 63] = bm;
    return ChunkGeom<2048>::BM + run;
}

/* Two 1024-value chunks, A in lanes 0-31 and B in lanes 32-63, back to back (B from word sizeA
 * on): bitmap word B of each is its half of M. */
template <int B>
__device__ __forceinline__ void rze_halves_plane(const uint32_t w[32], uint32_t sizeA, uint32_t *__restrict__ dst,
                                                 uint32_t &bm, uint32_t &rA, uint32_t &rB) {
    constexpr uint32_t BM = ChunkGeom<1024>::BM;
    const uint64_t M = __ballot(w[B] != 0);
    if (M) {
        const uint32_t lo = (uint32_t)M, hi = (uint32_t)(M >> 32);
        if (w[B] != 0) {
            const uint32_t pos = (threadIdx.x & 32) ? sizeA + BM + rB + __builtin_amdgcn_mbcnt_hi(hi, 0u)
                                                    : BM + rA + __builtin_amdgcn_mbcnt_lo(lo, 0u);
            dst[pos] = w[B];
        }
        rA += (uint32_t)__popc(lo);
        rB += (uint32_t)__popc(hi);
        bm = writelane<B>(bm, lo);
        bm = writelane<32 + B>(bm, hi);
    }
}

/* Chunk B is present when hasB; the word counts go to sizes[0..1]. */
template <int... B>
__device__ __forceinline__ void rze_halves(std::integer_sequence<int, B...>, const uint32_t w[32], bool hasB,
                                           uint32_t *__restrict__ dst, uint32_t sizes[2]) {
    constexpr uint32_t BM = ChunkGeom<1024>::BM;
    const uint32_t lane = threadIdx.x & 63;
    uint32_t ra = 0;
#pragma unroll
    for (int b = 0; b < (int)sizeof...(B); ++b) ra += (uint32_t)__popc((uint32_t)__ballot(w[b] != 0));
    const uint32_t sizeA = BM + ra;
    uint32_t rA = 0, rB = 0, bm = 0;
    (rze_halves_plane<B>(w, sizeA, dst, bm, rA, rB), ...);
    if (lane < 32 || hasB) dst[lane < 32 ? lane : sizeA + lane - 32u] = bm;
    sizes[0] = sizeA;
    sizes[1] = hasB ? BM + rB : 0u;
}

/* A 4096-value chunk whose groups 64 p .. 64 p + 63 this wave holds: bitmap words 4 B + 2 p,
 * 4 B + 2 p + 1 are M's halves, and the wave's words of plane B follow the partner's when p = 1.
 * base (lane B) is the number of the chunk's words before them. */
template <int B>
__device__ __forceinline__ void rze_pair_plane(const uint32_t w[32], uint32_t base, uint32_t *__restrict__ dst,
                                               uint32_t &bm) {
    constexpr uint32_t BM = ChunkGeom<4096>::BM;
    const uint64_t M = __ballot(w[B] != 0);
    if (M) {
        const uint32_t pb = readlane(base, B);
        if (w[B] != 0) dst[BM + pb + mbcnt64(M)] = w[B];
        bm = writelane<2 * B>(bm, (uint32_t)M);
        bm = writelane<2 * B + 1>(bm, (uint32_t)(M >> 32));
    }
}

template <int B>
__device__ __forceinline__ void plane_count(const uint32_t w[32], uint32_t &cnt) {
    cnt = writelane<B>(cnt, (uint32_t)__popcll(__ballot(w[B] != 0)));
}

/* p: the wave's parity; the partner (wave ^ 1 of the workgroup) holds the chunk's other half.
 * The waves trade per-plane word counts through their LDS stagings (xs: this wave's, xp: the
 * partner's), so both must make the call.  Writes when `live`; returns the chunk's word count
 * for p = 0, else 0. */
template <int... B>
__device__ __forceinline__ uint32_t rze_pair(std::integer_sequence<int, B...>, const uint32_t w[32], uint32_t p,
                                             bool live, uint32_t *xs, const uint32_t *xp,
                                             uint32_t *__restrict__ dst) {
    constexpr uint32_t BM = ChunkGeom<4096>::BM;
    const uint32_t lane = threadIdx.x & 63;
    uint32_t cnt = 0; /* lane b: this wave's nonzero words of plane b */
    (plane_count<B>(w, cnt), ...);
    wave_lds_sync();
    if (lane < 32) xs[lane] = cnt;
    __syncthreads();
    const uint32_t other = lane < 32 ? xp[lane] : 0u;
    const uint32_t c0 = p ? other : cnt;
    const uint32_t tot = cnt + other;
    const uint32_t incl = wave_incl_scan(tot);
    const uint32_t base = incl - tot + (p ? c0 : 0u);
    const uint32_t total = BM + readlane(incl, 63);
    if (!live) return 0;
    uint32_t bm = 0;
    (rze_pair_plane<B>(w, base, dst, bm), ...);
    dst[4u * (lane >> 1) + 2u * p + (lane & 1u)] = bm;
    return p ? 0u : total;
}

/* RZE of the wave's planes w[B...] into the scratch slot(s) of its coder chunk(s), and their
 * word counts into the size section sz (of sizes_bytes bytes).  Returns the words the wave's
 * slot takes; last_cv is the last coder chunk it sized (unchanged if none).  For V = 4096 both
 * waves of the pair must call (they trade counts through LDS: xs is this wave's staging, xp the
 * partner's). */
template <int V, int... B>
__device__ __forceinline__ uint32_t rze_chunks(std::integer_sequence<int, B...> planes, const uint32_t w[32],
                                               uint32_t c, uint32_t wave, const PlanArgs &pa, const Workspace &ws,
                                               uint4 *xs, const uint32_t *xp, uint32_t *sz, uint64_t sizes_bytes,
                                               uint32_t &last_cv) {
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t ncv = (pa.n + V - 1) / V;
    uint32_t wsum = 0;
    if constexpr (V == 2048) {
        if (c < pa.nchunks) {
            wsum = rze_wave(planes, w, ws.scratch + (uint64_t)c * pa.slot);
            if (lane == 0 && 4ull * c < sizes_bytes) sz[c] = wsum;
            last_cv = c;
        }
    } else if constexpr (V == 1024) {
        if (c < pa.nchunks) {
            const bool hasB = 2ull * c + 1 < ncv;
            uint32_t sizes[2];
            rze_halves(planes, w, hasB, ws.scratch + (uint64_t)c * pa.slot, sizes);
            wsum = sizes[0] + sizes[1];
            if (lane == 0 && 8ull * c < sizes_bytes) sz[2 * c] = sizes[0];
            if (lane == 0 && hasB && 8ull * c + 4 < sizes_bytes) sz[2 * c + 1] = sizes[1];
            last_cv = hasB ? 2 * c + 1 : 2 * c;
        }
    } else {
        const uint32_t p = wave & 1u;
        const uint32_t ce = c - p;
        const bool live = ce < pa.nchunks;
        wsum = rze_pair(planes, w, p, live, reinterpret_cast<uint32_t *>(xs), xp, ws.scratch + (uint64_t)ce * pa.slot);
        if (live && p == 0) {
            if (lane == 0 && 2ull * ce < sizes_bytes) sz[ce / 2] = wsum;
            last_cv = ce / 2;
        }
    }
    return wsum;
}

/* Workgroup of 4 waves over 8192 values; wave w owns the 2048 values of encode chunk c (the unit
 * of the escape bookkeeping and of the scratch slots the compaction copies), which hold 2048 / V
 * coder chunks, or half of one when V = 4096.  A wave's chunks lie back to back in its slot, and
 * a 4096-value chunk fills the slots of both its waves from the first one's (the second reports 0
 * words), so the compaction's copy of each slot in order yields the chunks in order.  The LDS is
 * the four waves' 8 KiB stagings and nothing else (32 KiB, five workgroups per CU); the group's
 * word and escape sums reuse it at the end. */
template <int V, bool STRIDED>
__device__ __forceinline__ void chunk_encode_body(const float *__restrict__ x, PlanArgs pa,
                                                  Workspace ws, uint8_t *__restrict__ sizes_dst,
                                                  uint64_t sizes_bytes) {
    __shared__ uint4 s_x[kEncWaves][kWaveQuads];

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t c = blockIdx.x * kEncWaves + wave;
    const DevInfo *info = ws.info;
    const uint64_t n = pa.n;
    const uint64_t cbase = (uint64_t)c * kEncChunk;
    uint4 *sx = s_x[wave];
    uint32_t wsum = 0, escs = 0;

    if (info->valid) {  /* the same for every workgroup: the barriers below are uniform */
        QParams qp;
        qp.eb = info->eb_f;
        qp.s = info->s;
        qp.r = info->r;
        qp.T = pa.T;
        qp.tlim = (float)(1u << pa.T);
        /* the predecessor of the wave's first value when it does not start a chunk (second half
         * of a 4096-value chunk): the code of the value before it, 0 if that value escapes */
        uint32_t carry = 0;
        if (V > kEncChunk && (cbase & (uint64_t)(V - 1)) != 0 && cbase < n) {
            const float xp = x[elem_off<STRIDED>(pa.lay, cbase - 1)];
            uint32_t e;
            const int32_t qprev = quantize_slow(xp, rintf(xp * qp.r), qp, &e);
            carry = e ? 0u : (uint32_t)qprev;
        }
        const bool full = cbase + kEncChunk <= n;
        if (full) stage_values<true, STRIDED>(x, pa.lay, cbase, n, sx);
        else stage_values<false, STRIDED>(x, pa.lay, cbase, n, sx);
        int32_t q[32];
        float qmax;
        const uint32_t emask = quantize_group(sx, qp, q, qmax);
        uint32_t tmask = 0;
        if (c < pa.nchunks && __ballot(emask != 0)) stage_escapes(sx, emask, cbase, c, ws, escs, tmask);
        uint32_t w[32];
        const uint64_t gbase = cbase + 32u * lane;
        if (full) diff_group<V, true>(q, carry, gbase, n, w);
        else diff_group<V, false>(q, carry, gbase, n, w);
        /* Bitshuffle: codes within 16 bits (every |q| below 2^14, so every difference below
         * 2^15) take the half transpose, and RZE skips their zero planes 16-31 */
        const bool low16 = !__ballot(!(qmax < 16383.0f)) && carry + 16383u <= 32766u;
        uint32_t *sz = reinterpret_cast<uint32_t *>(sizes_dst);
        const uint64_t ncv = (n + V - 1) / V;
        uint32_t last_cv = 0xFFFFFFFFu; /* the coder chunk this wave sized last */
        if (low16) {
            transpose_low16(w);
            zigzag_planes<16>(w);
            wsum = rze_chunks<V>(std::make_integer_sequence<int, 16>{}, w, c, wave, pa, ws, sx,
                                 reinterpret_cast<const uint32_t *>(s_x[wave ^ 1u]), sz, sizes_bytes, last_cv);
        } else {
            transpose32(w);
#pragma unroll
            for (int b = 0; b < 32; ++b) asm volatile("" : "+v"(w[b]));
            zigzag_planes<32>(w);
            wsum = rze_chunks<V>(Planes{}, w, c, wave, pa, ws, sx, reinterpret_cast<const uint32_t *>(s_x[wave ^ 1u]),
                                 sz, sizes_bytes, last_cv);
        }
        if ((uint64_t)last_cv == ncv - 1) {
            /* zero the size section's pad up to its 16-byte end */
            const uint64_t pz = ncv + lane;
            if (pz < align16(4 * ncv) / 4 && 4 * pz < sizes_bytes) sz[pz] = 0u;
        }
        if (c < pa.nchunks) {
            /* the escape bitmasks are read by the compaction only for a chunk with more escapes
             * than the staging holds */
            if (tmask && escs > (uint32_t)kEscStage) ws.emask[(uint64_t)c * kEncSegs + lane] = emask;
            if (lane == 0) {
                ws.chunk_words[c] = wsum;
                ws.chunk_esc[c] = escs;
                ws.chunk_tmask[c] = tmask;
            }
        }
    }
    if (c >= pa.nchunks) {
        wsum = 0;
        escs = 0;
    }
    __syncthreads(); /* every wave is done with its staging; the group sums reuse wave 0's */
    uint32_t *s_grp = reinterpret_cast<uint32_t *>(s_x[0]);
    if (lane == 0) {
        s_grp[wave] = wsum;
        s_grp[kEncWaves + wave] = escs;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t sw = 0, se = 0;
#pragma unroll
        for (int k = 0; k < kEncWaves; ++k) {
            sw += s_grp[k];
            se += s_grp[kEncWaves + k];
        }
        ws.group_words[blockIdx.x] = sw;
        ws.group_esc[blockIdx.x] = se;
    }
}

template <int V, bool STRIDED>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(5))) void chunk_encode_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    const uint32_t f = blockIdx.y;
    const Workspace w = lane_ws(ws, f, fs.ws_stride);
    uint8_t *sd = (fs.wdirect >> f) & 1u ? pick(fs.dst, f) + kHeaderBytes : w.widths;
    chunk_encode_body<V, STRIDED>(reinterpret_cast<const float *>(pick(fs.src, f)), pa, w, sd, pa.wsec);
}

/* ---- K7c: chunk decode ------------------------------------------------------------------------ */

/* Un-RZE: group `lane`'s plane words, w[b] = plane b's word (0 where its bitmap bit is clear).
 * The bitmap comes by one vector load the caller issues (lane l: bitmap word l), its bit count
 * is checked against the chunk's word count before any word is loaded under it (so a corrupt
 * stream reads nothing outside its chunk), and each plane below the highest one with a nonzero
 * word takes its bitmap bits and its running word count by readlane.  Returns false for a count
 * mismatch.  The plane loop is unrolled: plane B's bitmap bits and count sit at compile-time
 * lanes. */

/* A 2048-value chunk: plane B's bits are bitmap words 2 B and 2 B + 1. */
template <int B>
__device__ __forceinline__ void unrze_wave_plane(const uint32_t *blob, uint32_t bm, uint32_t pre, uint32_t wmax,
                                                 uint32_t w[32]) {
    constexpr uint32_t BM = ChunkGeom<2048>::BM;
    w[B] = 0;
    if ((uint32_t)B < wmax) {
        const uint64_t M = (uint64_t)readlane(bm, 2 * B) | ((uint64_t)readlane(bm, 2 * B + 1) << 32);
        if (__builtin_amdgcn_inverse_ballot_w64(M)) w[B] = word_at(blob, BM + readlane(pre, 2 * B) + mbcnt64(M));
    }
}

template <int... B>
__device__ __forceinline__ bool unrze_wave(std::integer_sequence<int, B...>, const uint32_t *blob, uint32_t P,
                                           uint32_t bm, uint32_t w[32]) {
    constexpr uint32_t BM = ChunkGeom<2048>::BM;
    const uint32_t pc = (uint32_t)__popc(bm);
    const uint32_t incl = wave_incl_scan(pc);
    if (readlane(incl, 63) + BM != P) return false;
    const uint64_t nz = __ballot(bm != 0);
    const uint32_t wmax = nz ? (uint32_t)(63 - __clzll((long long)nz)) / 2u + 1u : 0u;
    (unrze_wave_plane<B>(blob, bm, incl - pc, wmax, w), ...);
    return true;
}

/* Two 1024-value chunks: A (P words from blob) in lanes 0-31, B (P2 words from blob + P, absent
 * when P2 = 0) in lanes 32-63; plane B's bits are word B of each bitmap.  bm: lane l < 32 holds
 * word l of A's bitmap, lane 32 + l word l of B's (0 without B). */
template <int B>
__device__ __forceinline__ void unrze_halves_plane(const uint32_t *blob, uint32_t P, uint32_t bm, uint32_t pre,
                                                   uint32_t wmax, uint32_t w[32]) {
    constexpr uint32_t BM = ChunkGeom<1024>::BM;
    w[B] = 0;
    if ((uint32_t)B < wmax) {
        const uint32_t lo = readlane(bm, B), hi = readlane(bm, 32 + B);
        const uint64_t M = (uint64_t)lo | ((uint64_t)hi << 32);
        if (__builtin_amdgcn_inverse_ballot_w64(M)) {
            const uint32_t off = (threadIdx.x & 32) ? P + BM + readlane(pre, 32 + B) + __builtin_amdgcn_mbcnt_hi(hi, 0u)
                                                    : BM + readlane(pre, B) + __builtin_amdgcn_mbcnt_lo(lo, 0u);
            w[B] = word_at(blob, off);
        }
    }
}

template <int... B>
__device__ __forceinline__ bool unrze_halves(std::integer_sequence<int, B...>, const uint32_t *blob, uint32_t P,
                                             uint32_t P2, uint32_t bm, uint32_t w[32]) {
    constexpr uint32_t BM = ChunkGeom<1024>::BM;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t pc = (uint32_t)__popc(bm);
    const uint32_t incl = wave_seg_scan(pc, lane & 31, 32);
    if (readlane(incl, 31) + BM != P || (P2 && readlane(incl, 63) + BM != P2)) return false;
    const uint64_t nz = __ballot(bm != 0);
    const uint32_t nlo = (uint32_t)nz, nhi = (uint32_t)(nz >> 32);
    const uint32_t wmax = (nlo | nhi) ? 31u - (uint32_t)__builtin_clz(nlo | nhi) + 1u : 0u;
    (unrze_halves_plane<B>(blob, P, bm, incl - pc, wmax, w), ...);
    return true;
}

/* A 4096-value chunk, half H (groups 64 H .. 64 H + 63): plane B's bits are bitmap words 4 B + 2 H
 * and 4 B + 2 H + 1, which sit in bm0 (words 0-63) or bm1 (words 64-127) with their exclusive
 * bit-count prefixes pre0, pre1. */
template <int H, int B>
__device__ __forceinline__ void unrze_quarter_plane(const uint32_t *blob, uint32_t bm0, uint32_t bm1, uint32_t pre0,
                                                    uint32_t pre1, uint32_t wmax, uint32_t w[32]) {
    constexpr uint32_t BM = ChunkGeom<4096>::BM;
    constexpr int K = 4 * B + 2 * H;
    w[B] = 0;
    if ((uint32_t)B < wmax) {
        const uint32_t bm = K < 64 ? bm0 : bm1, pre = K < 64 ? pre0 : pre1;
        const uint64_t M = (uint64_t)readlane(bm, K & 63) | ((uint64_t)readlane(bm, (K & 63) + 1) << 32);
        if (__builtin_amdgcn_inverse_ballot_w64(M)) w[B] = word_at(blob, BM + readlane(pre, K & 63) + mbcnt64(M));
    }
}

template <int... B>
__device__ __forceinline__ bool unrze_pair(std::integer_sequence<int, B...>, const uint32_t *blob, uint32_t P,
                                           uint32_t bm0, uint32_t bm1, uint32_t w0[32], uint32_t w1[32]) {
    constexpr uint32_t BM = ChunkGeom<4096>::BM;
    const uint32_t c0 = (uint32_t)__popc(bm0), c1 = (uint32_t)__popc(bm1);
    const uint32_t i0 = wave_incl_scan(c0), i1 = wave_incl_scan(c1);
    const uint32_t t0 = readlane(i0, 63);
    if (t0 + readlane(i1, 63) + BM != P) return false;
    const uint64_t nz0 = __ballot(bm0 != 0), nz1 = __ballot(bm1 != 0);
    const uint32_t top = nz1 ? 64u + (uint32_t)(63 - __clzll((long long)nz1)) : nz0 ? (uint32_t)(63 - __clzll((long long)nz0)) : 0u;
    const uint32_t wmax = (nz0 | nz1) ? top / 4u + 1u : 0u;
    (unrze_quarter_plane<0, B>(blob, bm0, bm1, i0 - c0, t0 + i1 - c1, wmax, w0), ...);
    (unrze_quarter_plane<1, B>(blob, bm0, bm1, i0 - c0, t0 + i1 - c1, wmax, w1), ...);
    return true;
}

/* Values of the lane's group from its plane words, in place: unfold, transpose, and sum the
 * differences from the group's start, which the wave scan of the lane totals (segments of SEG
 * lanes, one per chunk) and the carry give; w[i] becomes the bits of f32(f32(q_i) * s).  Returns
 * the carry for what follows the wave's last group. */
template <int SEG>
__device__ __forceinline__ uint32_t decode_group(uint32_t w[32], uint32_t carry, float s) {
    unzigzag_planes(w);
    transpose32(w);
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) tot += w[i];
    const uint32_t incl = SEG == 64 ? wave_incl_scan(tot) : wave_seg_scan(tot, threadIdx.x & 31, 32);
    uint32_t run = carry + incl - tot;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        run += w[i];
        w[i] = __float_as_uint((float)(int32_t)run * s);
    }
    return carry + readlane(incl, 63);
}

/* The wave's 2048 decoded values (lane: its group's 32, as bits) to out from value base on, cnt
 * of them, through the LDS staging sy. */
template <bool STRIDED>
__device__ __forceinline__ void store_values(const uint32_t y[32], uint4 *sy, float *__restrict__ out,
                                             const Layout &lo, uint32_t base, uint32_t cnt) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t s0 = quad_slot(8u * lane);
    wave_lds_sync(); /* earlier reads of the staging are done */
#pragma unroll
    for (int j = 0; j < 8; ++j) sy[s0 ^ (uint32_t)j] = make_uint4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
    wave_lds_sync();
    if (cnt == (uint32_t)kEncChunk) {
        const uint32_t s1 = quad_slot(lane);
#pragma unroll
        for (int k = 0; k < kLaneQuads; ++k) {
            const uint4 v = sy[kWave * k + (s1 ^ (uint32_t)k)];
            store4<STRIDED>(out, lo, (uint64_t)base + 4u * (kWave * k + lane),
                            make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                        __uint_as_float(v.w)));
        }
    } else {
#pragma unroll 4
        for (int k = 0; k < kEncChunk / kWave; ++k) {
            const uint32_t v = kWave * k + lane;
            if (v < cnt) out[elem_off<STRIDED>(lo, (uint64_t)base + v)] = __uint_as_float(lds_value(sy, v));
        }
    }
}

/* One wave per 2048 values (two 1024-value chunks, or one 2048-value chunk), or per 4096-value
 * chunk taken as two halves with the running sum carried from the first into the second. */
template <int V, bool STRIDED>
__device__ __forceinline__ void chunk_decode_body(const uint8_t *__restrict__ in, uint64_t in_bytes, PlanArgs pa,
                                                  Workspace ws, float *__restrict__ out) {
    constexpr uint32_t U = V > kEncChunk ? V : kEncChunk; /* values per wave */
    constexpr uint32_t CPT = kEncChunksPerGroup * kEncChunk / V; /* chunks per offset-table group */
    __shared__ uint4 s_y[kWavesPerBlock][kWaveQuads];
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t u = blockIdx.x * kWavesPerBlock + wave;
    const uint32_t n = (uint32_t)pa.n;
    if ((uint64_t)u * U >= n) return;
    const uint32_t ubase = u * U;
    DevInfo *info = ws.info;
    /* The chunk's place in the payload: its group's offset from the offset table plus the word
     * counts of the group's chunks before it.  Lane l < CPT loads the count of the group's chunk
     * l, so every wave of the group sees the same counts.  The header, the table entries and the
     * counts come in one round of loads (all lie inside the bytes the host lets through) and the
     * chunk's bitmap loads go out next; a bitmap load that would leave the caller's bytes is not
     * issued (no valid stream asks for one).  Every wave checks its group's counts against the
     * table; the whole header is checked (and a bad one reported) by the outlier patch. */
    const uint32_t c = V < kEncChunk ? 2 * u : u;
    const uint32_t g = c / CPT, k = c % CPT;
    const uint32_t cl = g * CPT + lane;
    const uint32_t hv = load_header_lanes(in, pa, g);
    const uint32_t cw = lane < CPT && cl < pa.dchunks ? reinterpret_cast<const uint32_t *>(in + kHeaderBytes)[cl] : 0u;
    const uint32_t gincl = wave_incl_scan(cw);
    const uint32_t gtot = readlane(gincl, 63);
    const StreamView H = view_header(hv);
    const uint64_t W = (uint64_t)(g > 0 ? readlane(hv, 32) : 0u) + (k > 0 ? readlane(gincl, (int)k - 1) : 0u);
    const uint32_t P = readlane(cw, (int)k);
    const uint32_t P2 = V == 1024 ? readlane(cw, (int)k + 1) : 0u; /* 0 past the last chunk */
    const bool cbad = lane < CPT && cl < pa.dchunks && (cw < V / 32 || cw > V + V / 32);
    const bool any_bad = __ballot(cbad) != 0;
    const uint64_t ws0 = H.po / 4 + W; /* stream word index of the chunk's first word */
    const bool inb = !any_bad && ws0 <= in_bytes / 4 && (uint64_t)P + P2 <= in_bytes / 4 - ws0;
    const uint32_t *blob = reinterpret_cast<const uint32_t *>(in) + ws0;
    uint32_t bm0 = 0, bm1 = 0;
    if (inb) {
        if constexpr (V == 1024) {
            if (lane < 32) bm0 = blob[lane];
            else if (P2) bm0 = blob[P + lane - 32];
        } else if constexpr (V == 2048) {
            bm0 = blob[lane];
        } else {
            bm0 = blob[lane];
            bm1 = blob[64 + lane];
        }
    }
    if (!H.sane) return;
    if (H.mode == 1) {
        if (kHeaderBytes + 4ull * n > in_bytes) return;
        const uint32_t cnt = n - ubase < U ? n - ubase : U;
        const uint32_t *srcw = reinterpret_cast<const uint32_t *>(in + kHeaderBytes) + ubase;
        uint32_t *ob = reinterpret_cast<uint32_t *>(out);
        if (!STRIDED && cnt == U) {
            const uint4 *s4 = reinterpret_cast<const uint4 *>(srcw);
            uint4 *d4 = reinterpret_cast<uint4 *>(ob + ubase);
            uint4 t[U / 4 / kWave];
#pragma unroll
            for (int i = 0; i < (int)(U / 4 / kWave); ++i) t[i] = ld_nt(s4 + lane + kWave * i);
#pragma unroll
            for (int i = 0; i < (int)(U / 4 / kWave); ++i) st_nt(d4 + lane + kWave * i, t[i]);
        } else {
            for (uint32_t i = lane; i < cnt; i += kWave) ob[elem_off<STRIDED>(pa.lay, ubase + i)] = srcw[i];
        }
        return;
    }
    /* the group: each count in [V/32, V + V/32], and the table's range for it holds exactly its
     * words and ends inside the payload (over every group, these accept exactly the tables that
     * index the payload the counts describe) */
    uint64_t t0, t1;
    table_range(hv, g, pa.ngroups, H.pw, t0, t1);
    if (any_bad || t0 > t1 || t1 > H.pw || t1 - t0 != gtot) {
        if (k == 0 && lane == 0) atomicOr(&info->sticky, 1u);
        return;
    }
    /* (a stream whose group passes reads nothing past the caller's bytes, unless its header is
     * bad, which the outlier patch reports) */
    if (!inb) return;
    const float s = H.s;
    uint4 *sy = s_y[wave];
    const uint32_t cnt = n - ubase < (uint32_t)kEncChunk ? n - ubase : (uint32_t)kEncChunk;
    uint32_t w[32];
    if constexpr (V == 1024) {
        if (!unrze_halves(Planes{}, blob, P, P2, bm0, w)) {
            if (lane == 0) atomicOr(&info->sticky, 1u);
            return;
        }
        decode_group<32>(w, 0, s);
        store_values<STRIDED>(w, sy, out, pa.lay, ubase, cnt);
    } else if constexpr (V == 2048) {
        if (!unrze_wave(Planes{}, blob, P, bm0, w)) {
            if (lane == 0) atomicOr(&info->sticky, 1u);
            return;
        }
        decode_group<64>(w, 0, s);
        store_values<STRIDED>(w, sy, out, pa.lay, ubase, cnt);
    } else {
        /* both halves' words are loaded before either is decoded */
        uint32_t w1[32];
        if (!unrze_pair(Planes{}, blob, P, bm0, bm1, w, w1)) {
            if (lane == 0) atomicOr(&info->sticky, 1u);
            return;
        }
        const uint32_t carry = decode_group<64>(w, 0, s);
        store_values<STRIDED>(w, sy, out, pa.lay, ubase, cnt);
        const uint32_t hbase = ubase + kEncChunk;
        if (hbase < n) {
            decode_group<64>(w1, carry, s);
            store_values<STRIDED>(w1, sy, out, pa.lay, hbase,
                                  n - hbase < (uint32_t)kEncChunk ? n - hbase : (uint32_t)kEncChunk);
        }
    }
}

template <int V, bool STRIDED>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(5))) void chunk_decode_kernel(Fields fs, PlanArgs pa, Workspace ws) {
    const uint32_t f = blockIdx.y;
    chunk_decode_body<V, STRIDED>(pick(fs.src, f), pick(fs.bytes, f), pa, lane_ws(ws, f, fs.ws_stride),
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
    /* waves: one per 2048 values (two 1024-value chunks), or one per chunk */
    const uint32_t waves = V < kEncChunk ? (pa.dchunks + 1) / 2 : pa.dchunks;
    const dim3 grid((waves + kWavesPerBlock - 1) / kWavesPerBlock, nf), block(kBlockThreads);
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
