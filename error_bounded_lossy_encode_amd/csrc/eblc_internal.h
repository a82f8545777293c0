/*
 * eblc_internal.h -- shared between the host plan code and the gfx950 kernels of libeblc.so.
 *
 * Work decomposition (all sizes in 32-bit values):
 *   compress:   tile  = one wave64 step, kEncLaneVals consecutive values per lane (128-bit
 *                       loads), so a 32-value bitpack segment is kSegLanes lanes
 *               chunk = kEncTiles tiles; one wave owns one chunk
 *               group = kEncWaves chunks = one encode workgroup
 *   decompress: tile  = 256 values, 4 consecutive values per lane, a segment is 8 lanes
 *               chunk = 8 tiles = 2048 values = 64 segments; one wave owns one chunk
 *               group = 4 chunks = one 256-thread workgroup
 * Both groups hold 8192 values; the device-wide scans run over groups (compress: it writes one
 * prefix per super-group of 64 groups, and a group adds the sums of the groups before it in its
 * super-group).  The chunk coder keeps
 * the encode chunks and groups (its coder chunks of V values fill whole encode chunks, or two)
 * and decodes one coder chunk per wave, four per group.  The Lorenzo block B is a multiple
 * of 32 up to 1024, or 2048.  A power of two starts every chunk; any other block may start
 * inside a chunk at a 32-value boundary and cross chunk ends.  An encode chunk that does not
 * start a block takes its first prediction from the code of the value before it; a decode chunk
 * that does not sums the deltas of the block's segments before it.  The only other cross-wave
 * dependency is the exclusive scan of payload sizes and outlier counts on compress; decompress
 * has none, since the stream's offset table gives each group's payload start.
 */
#ifndef EBLC_INTERNAL_H
#define EBLC_INTERNAL_H

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eblc {

constexpr int kWave = 64;
constexpr int kTile = 256;
constexpr int kEncLaneVals = 4;                  /* consecutive values per lane on compress */
constexpr int kEncTile = kWave * kEncLaneVals;
constexpr int kSegLanes = 32 / kEncLaneVals;     /* lanes per segment on compress */
constexpr int kSegsPerEncTile = kEncTile / 32;
constexpr int kEncChunk = 2048;                  /* values per encode chunk */
constexpr int kEncTiles = kEncChunk / kEncTile;
constexpr int kEncSegs = kEncChunk / 32;
constexpr int kEncWaves = 8192 / kEncChunk;       /* waves (chunks) per encode workgroup */
constexpr int kEncThreads = kWave * kEncWaves;
constexpr int kEncChunksPerGroup = kEncWaves;
constexpr int kEncPayWords = kEncChunk / 2 + 4;  /* LDS pack buffer per wave: half a chunk's worst case */
constexpr int kDecTiles = 8;
constexpr int kDecChunk = kTile * kDecTiles;     /* 2048 values */
constexpr int kDecSegs = kDecChunk / 32;         /* 64 segments */
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWave * kWavesPerBlock;
constexpr int kDecChunksPerGroup = kWavesPerBlock;
constexpr int kEscStage = 64;                    /* escapes staged per encode chunk */
constexpr int kSuperGroups = 64;                /* groups per super-group of the device-wide scans */
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 16;                   /* items per scan thread per round */
constexpr int kRangeThreads = 256;
constexpr int kRangeVec = 16;                    /* float4 loads per range thread */
constexpr uint64_t kRangeSpan = (uint64_t)kRangeThreads * kRangeVec; /* float4 per range block */
constexpr int kPatchBlocksMax = 1024;
constexpr uint32_t kHeaderBytes = 128;
constexpr uint32_t kMagic = 0x434C4245u;          /* "EBLC" */
constexpr uint32_t kVersion = 2;               /* format 2: with the offset table */
constexpr int kMaxKernelsPerCall = 8;
constexpr int kResolveBatch = 8;                /* range partials in flight per thread of the resolve */

/* Device-resident state of a plan (one per plan, in its workspace). */
struct DevInfo {
    /* resolved bound: abs mode writes it once at plan creation, rel mode at every compress */
    float eb_f, s, r;
    uint32_t valid;
    /* outcome of the last compress */
    uint32_t mode;          /* 0 bitpack coder, 1 raw, 2 chunk coder */
    uint32_t sticky;        /* decompress: set by a corrupt stream, until eblc_plan_status reads it */
    uint32_t fits;          /* compress: total <= out_capacity */
    uint32_t pad;
    uint64_t m;
    uint64_t payload_words;
    uint64_t payload_off;
    uint64_t oidx_off;
    uint64_t oval_off;
    uint64_t total;
    /* decompress: the header words a stream of the plan must hold, word i under mask i (magic,
     * version and header size, rank, dims, n, the size section's offset; mask 0 elsewhere),
     * written at plan creation so that each decoding wave compares them lane by lane */
    uint32_t hdr_want[32];
    uint32_t hdr_mask[32];
};

/* Where the caller's values live.  The codec works on the row-major flattened index i over the
 * dims; the array may be padded (each outer stride at least the extent below it, fastest stride
 * 1), so value i sits at element offset(i) of the caller's pointer.  Divisions use exact
 * reciprocals: for v < 2^32 and d >= 2, v / d = floor(v * (floor(2^64 / d) + 1) / 2^64). */
struct Layout {
    uint32_t strided;       /* 0: offset(i) = i */
    uint32_t vec;           /* each 4-aligned group of 4 values is contiguous and 16-byte aligned */
    uint32_t rank;
    uint32_t L;             /* fastest extent */
    uint32_t o1, o2;        /* extents of the next two dims, fast to slow (rank 4 uses both) */
    uint64_t mL, m1, m2;    /* reciprocals of L, o1, o2 (0 when the divisor is 1) */
    uint64_t s1, s2, s3;    /* strides of the outer dims, fast to slow */
};

/* Plan constants passed by value to the kernels. */
struct PlanArgs {
    uint64_t n;
    uint64_t nseg;
    uint64_t dims[4];
    uint32_t rank;
    uint32_t B;             /* Lorenzo block: a multiple of 32 up to 1024, or 2048 (the chunk, for the
                               chunk coder) */
    uint32_t T;             /* outlier log2 */
    uint32_t V;             /* chunk coder: values per chunk (1024, 2048, 4096); 0: bitpack coder */
    uint32_t log2seg;       /* header field: 5 (32-value segments), or log2 V */
    uint32_t slot;          /* scratch words per encode chunk: 2048, or 2112 for the chunk coder */
    uint32_t wpg;           /* bytes of the size section per encode group */
    uint64_t wsec;          /* bytes of the size section: align16(nseg), or align16(4 chunks) */
    uint32_t center;        /* Lorenzo centering: each block's first code predicted by its mean */
    uint32_t log2B;         /* ceil(log2 B) */
    uint64_t nblocks;       /* ceil(n / B) */
    uint64_t msec;          /* bytes of the means section on compress: align16(4 nblocks), or 0 */
    uint32_t nchunks;       /* encode chunks */
    uint32_t ngroups;       /* encode groups */
    uint32_t dchunks;       /* decode chunks (the coder's chunks for the chunk coder) */
    uint32_t dgroups;       /* decode groups */
    uint64_t side_max;
    uint64_t max_pw;        /* max_payload_words(n, V): the largest payload a stream can hold */
    Layout lay;             /* memory layout of the compress input and decompress output */
};

/* Workspace pointers (all device memory owned by the plan). */
struct Workspace {
    DevInfo *info;
    uint32_t *scratch;       /* (nchunks + 1) * slot words: per-chunk payload slots */
    uint32_t *chunk_words;   /* [nchunks] payload words per encode chunk */
    uint32_t *chunk_esc;     /* [nchunks] escapes per encode chunk */
    uint32_t *chunk_tmask;   /* [nchunks] bit t set if tile t of the encode chunk has an escape */
    uint32_t *group_words;   /* [ngroups] */
    uint32_t *group_esc;     /* [ngroups] */
    uint32_t *gpre_words;    /* [nsuper] exclusive prefix of the words of each super-group of kSuperGroups
                                groups (a group adds the sums of its super-group's groups before it) */
    uint32_t *gpre_esc;      /* [nsuper] the same for the escapes */
    uint32_t *emask;         /* [nchunks * kEncSegs] escape bitmask per segment (chunks with more
                                than kEscStage escapes, tiles with escapes) */
    uint32_t *stage_idx;     /* [nchunks * kEscStage] first escapes of each chunk: index ... */
    uint32_t *stage_val;     /* [nchunks * kEscStage] ... and raw value bits, in index order */
    uint8_t *widths;         /* [nchunks * kEncSegs] size section staging when the output is too small */
    float *range_part;       /* [2 * range_blocks(n)] per-block min / max */
    int32_t *means;          /* [nblocks] block means of a centered compress */
};

/* The offset table right after the size section: one u32 per group of 8192 values (an encode
 * and a decode group) after the first, the payload words before that group, padded to 16
 * bytes.  The block means (centered streams) and the payload follow it. */
__host__ __device__ inline uint64_t table_bytes(uint32_t ngroups) {
    return ngroups > 1 ? (4ull * (ngroups - 1) + 15) & ~15ull : 0;
}

/* The most payload words a field of n values can take: 32 per segment (bitpack), or every plane
 * word and bitmap word of every chunk (chunk coder with chunks of V values). */
__host__ __device__ inline uint64_t max_payload_words(uint64_t n, uint32_t V) {
    if (V == 0) return 32 * ((n + 31) / 32);
    return ((n + V - 1) / V) * (uint64_t)(V + V / 32);
}

/* Workgroups of the range pass: one per kRangeSpan float4 (16384 values), at least one. */
inline uint32_t range_blocks(uint64_t n) {
    const uint64_t b = (n / 4 + kRangeSpan - 1) / kRangeSpan;
    return (uint32_t)(b < 1 ? 1 : b);
}

/* The caller's buffers of the fields one launch codes: field f = blockIdx.y, f < gridDim.y <=
 * kMaxFields, runs in the workspace of lane f, which lies f * ws_stride bytes after lane 0's.
 * One call codes one field; a batch call codes up to kMaxFields fields per launch. */
constexpr int kMaxFields = 8;
struct Fields {
    const uint8_t *src[kMaxFields];  /* compress: the field; decompress: the stream */
    uint8_t *dst[kMaxFields];        /* compress: the stream; decompress: the field */
    uint64_t bytes[kMaxFields];      /* compress: capacity of dst; decompress: readable bytes of src */
    uint64_t *result[kMaxFields];    /* compress: the result record (length, status) */
    uint64_t ws_stride;              /* bytes between the workspaces of consecutive lanes */
    uint32_t wdirect;                /* compress: bit f set when field f's size section goes straight
                                        into its stream (else into its workspace's staging) */
    uint32_t pad;
};

/* Events the next launcher's kernels record into, set by the host's measurement hook around
 * one launcher call (both null otherwise).  The launcher's first kernel records its start in
 * `start` and its last kernel its end in `stop`, through the kernel dispatch's own timestamps
 * (hipExtLaunchKernel), so timing adds no marker packets to the stream. */
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
extern thread_local LaunchEvents g_launch_events;

/* Launch one kernel; kLast = false for a launcher's kernels before its last one. */
template <bool kLast = true, typename F, typename... Args>
inline void eblc_launch(F kernel, const dim3 &grid, const dim3 &block, uint32_t shmem, hipStream_t stream,
                        Args... args) {
    const hipEvent_t start = g_launch_events.start;
    g_launch_events.start = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, start, kLast ? g_launch_events.stop : nullptr, 0u,
                          args...);
}

/* Kernel launchers (eblc_kernels.hip).  Each codes the first nf (1..kMaxFields) fields of fs,
 * enqueued on `stream`, and returns the launch error. */
hipError_t launch_range(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws, double eps,
                        hipStream_t stream);
/* The bound of an absolute eps, resolved on the device into the workspace's DevInfo (one field,
 * lane 0) by the rule the host applies at plan creation. */
hipError_t launch_resolve_abs(const Workspace &ws, double eps, hipStream_t stream);
hipError_t launch_encode(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                         hipStream_t stream);
hipError_t launch_scan_compress(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                                hipStream_t stream);
hipError_t launch_compact(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                          hipStream_t stream);
/* Scan and compaction in one launch, for fields of at most 2048 groups (2^24 values): each
 * compaction workgroup scans the group sums itself; launch_compact_scan replaces
 * launch_scan_compress + launch_compact when compact_folds_scan(pa). */
bool compact_folds_scan(const PlanArgs &pa);
hipError_t launch_compact_scan(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                               hipStream_t stream);
hipError_t launch_decode(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                         hipStream_t stream);
hipError_t launch_patch(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                        hipStream_t stream);

/* The chunk coder (eblc_chunk.hip): encode in place of launch_encode, decode in place of
 * launch_decode; the other stages are shared. */
hipError_t launch_chunk_encode(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                               hipStream_t stream);
hipError_t launch_chunk_decode(const Fields &fs, uint32_t nf, const PlanArgs &pa, const Workspace &ws,
                               hipStream_t stream);

}  // namespace eblc

#endif
