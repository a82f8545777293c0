/*
 * eblc_api.hip -- host side of libeblc.so: the C ABI declared in include/eblc.h.
 *
 * The plan mirrors the provider plan of the "DevitoComp provider interface" page: created once
 * per tensor shape and tolerance ("Configuring the error tolerance": the error is fixed at plan
 * creation), it owns a workspace allocated up front (the PREALLOCATE policy of the FZGPUModules
 * "Architecture" page, MemoryPool section), so compress and decompress allocate nothing.
 * Compress enqueues range (relative mode) -> encode -> scan -> compaction with outliers on the
 * caller's stream and waits once to return the stream length; decompress enqueues decode
 * (which takes each group's payload offset from the stream's offset table) -> outlier patch and
 * returns at once.
 */
#include "eblc.h"
#include "eblc_internal.h"

#include <cerrno>
#include <cfloat>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <string_view>
#include <vector>

using namespace eblc;

namespace eblc {
thread_local LaunchEvents g_launch_events;
}  // namespace eblc

namespace {
constexpr int kMaxLanes = kMaxFields;      /* fields (each with its workspace) of one launch */
constexpr size_t kMaxTimedLaunches = 8192; /* event pairs the measurement hook may hold */
}  // namespace

struct eblc_plan {
    int device = 0;
    int rank = 0;
    int64_t dims[4] = {0, 0, 0, 0};
    uint64_t n = 0;
    bool rel = true;
    double eps = 1e-4;
    PlanArgs pa{};
    /* lane 0's workspace; lane k's lies k * ws_stride bytes further on.  A launch codes up to
     * `lanes` fields, field k in lane k's workspace; single calls use lane 0 */
    int lanes = 1;
    Workspace ws{};
    uint64_t ws_stride = 0;
    void *ws_base = nullptr;
    eblc_result_t *host_result = nullptr; /* pinned host slot the synchronous compress reads */
    /* measurement hook: an event pair per launch, up to the pool's size, since enabling */
    std::vector<hipEvent_t> ev_pool;
    std::vector<const char *> ev_names;
    size_t ev_used = 0;
    std::string ev_filter;      /* ",name,name," of the kernels to time; empty: every kernel */
    uint32_t ev_every = 1;      /* time every ev_every-th compress and decompress call */
    uint64_t ev_calls[2] = {0, 0};
    bool ev_sampled = true;     /* the current call is timed */
};

namespace {

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

/* Device guard: switch to the plan's device for the call, restore the caller's afterwards. */
struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) return;
        ok = prev == dev || hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

/* The option parser works on views of the caller's string and copies a value into a stack
 * buffer only to convert it, so parsing allocates nothing. */
constexpr size_t kMaxValueChars = 63;

bool parse_double(std::string_view s, double *out) {
    if (s.empty() || s.size() > kMaxValueChars) return false;
    char buf[kMaxValueChars + 1];
    std::memcpy(buf, s.data(), s.size());
    buf[s.size()] = '\0';
    char *e = nullptr;
    errno = 0;
    const double v = std::strtod(buf, &e);
    if (e == buf || *e != '\0' || errno == ERANGE) return false;
    *out = v;
    return true;
}

bool parse_u64(std::string_view s, uint64_t *out) {
    if (s.empty() || s.size() > 20) return false;
    uint64_t v = 0;
    for (char ch : s) {
        if (ch < '0' || ch > '9') return false;
        const uint64_t d = (uint64_t)(ch - '0');
        if (v > (UINT64_MAX - d) / 10) return false;
        v = v * 10 + d;
    }
    *out = v;
    return true;
}

std::string_view trim(std::string_view s) {
    size_t a = 0, b = s.size();
    while (a < b && (s[a] == ' ' || s[a] == '\t')) ++a;
    while (b > a && (s[b - 1] == ' ' || s[b - 1] == '\t')) --b;
    return s.substr(a, b - a);
}

struct Options {
    bool rel = true;
    double eps = 1e-4;
    uint32_t B = 256;
    uint32_t T = 30;
    bool side_set = false;
    uint64_t side_max = 0;
    bool chunk_coder = false;   /* coder=chunk: Quant -> Diff -> Bitshuffle -> RZE */
    bool center = false;        /* center=1: Lorenzo centering (bitpack coder) */
    uint32_t V = 0;             /* chunk coder: values per chunk */
    uint32_t lanes = 1;         /* fields of a batch call in flight at once */
};

/* Options string ("Provider layout": a provider-defined string; DevitoPRO passes the relative
 * error as a decimal, or NULL for the provider default). */
eblc_status parse_options(const char *opts, Options *o) {
    if (opts == nullptr) return EBLC_OK;
    const std::string_view all = trim(std::string_view(opts));
    if (all.empty()) return EBLC_OK;
    double v;
    if (parse_double(all, &v)) {
        if (!std::isfinite(v) || v < 0) return EBLC_INVALID_ARGUMENT;
        o->rel = true;
        o->eps = v;
        return EBLC_OK;
    }
    bool seen_eb = false, seen_block = false, seen_t = false, seen_coder = false, seen_chunk = false;
    bool seen_center = false, seen_lanes = false;
    uint64_t chunk_bytes = 8192;
    size_t pos = 0;
    for (;;) {
        size_t end = all.find(';', pos);
        const bool final_item = end == std::string_view::npos;
        if (final_item) end = all.size();
        const std::string_view item = trim(all.substr(pos, end - pos));
        pos = end + 1;
        if (!item.empty()) {
            const size_t eq = item.find('=');
            if (eq == std::string_view::npos) return EBLC_INVALID_ARGUMENT;
            const std::string_view key = trim(item.substr(0, eq)), val = trim(item.substr(eq + 1));
            if (key == "rel" || key == "abs") {
                if (seen_eb || !parse_double(val, &v) || !std::isfinite(v) || v < 0) return EBLC_INVALID_ARGUMENT;
                seen_eb = true;
                o->rel = key == "rel";
                o->eps = v;
            } else if (key == "block") {
                /* a multiple of 32 ("Pipeline Specialization Internals", Forward declaration: the
                 * block size must be a multiple of 32) up to 1024, or 2048 */
                uint64_t b;
                if (seen_block || !parse_u64(val, &b) || !((b >= 32 && b <= 1024 && b % 32 == 0) || b == 2048))
                    return EBLC_INVALID_ARGUMENT;
                seen_block = true;
                o->B = (uint32_t)b;
            } else if (key == "outlier_log2") {
                uint64_t t;
                if (seen_t || !parse_u64(val, &t) || t < 1 || t > 30) return EBLC_INVALID_ARGUMENT;
                seen_t = true;
                o->T = (uint32_t)t;
            } else if (key == "coder") {
                if (seen_coder || (val != "bitpack" && val != "chunk")) return EBLC_INVALID_ARGUMENT;
                seen_coder = true;
                o->chunk_coder = val == "chunk";
            } else if (key == "center") {
                if (seen_center || (val != "0" && val != "1")) return EBLC_INVALID_ARGUMENT;
                seen_center = true;
                o->center = val == "1";
            } else if (key == "chunk_bytes") {
                if (seen_chunk || !parse_u64(val, &chunk_bytes) ||
                    (chunk_bytes != 4096 && chunk_bytes != 8192 && chunk_bytes != 16384))
                    return EBLC_INVALID_ARGUMENT;
                seen_chunk = true;
            } else if (key == "lanes") {
                uint64_t k;
                if (seen_lanes || !parse_u64(val, &k) || k < 1 || k > (uint64_t)kMaxLanes)
                    return EBLC_INVALID_ARGUMENT;
                seen_lanes = true;
                o->lanes = (uint32_t)k;
            } else if (key == "side_max") {
                uint64_t m;
                if (o->side_set || !parse_u64(val, &m)) return EBLC_INVALID_ARGUMENT;
                o->side_set = true;
                o->side_max = m;
            } else {
                return EBLC_INVALID_ARGUMENT;
            }
        }
        if (final_item) break;
    }
    /* the chunk is the chunk coder's reset period: no block with it, no chunk without it */
    if (o->chunk_coder) {
        if (seen_block || o->center) return EBLC_INVALID_ARGUMENT;
        o->V = (uint32_t)(chunk_bytes / 4);
        o->B = o->V;
    } else if (seen_chunk) {
        return EBLC_INVALID_ARGUMENT;
    }
    return EBLC_OK;
}


/* The header words every stream this plan decodes holds, and their masks (DevInfo). */
void header_template(const PlanArgs &pa, DevInfo *info) {
    auto put = [&](int i, uint32_t want, uint32_t mask) {
        info->hdr_want[i] = want;
        info->hdr_mask[i] = mask;
    };
    put(0, kMagic, ~0u);
    put(1, kVersion | (kHeaderBytes << 16), ~0u);
    put(2, pa.rank << 8, 0xff00u); /* the rank byte; mode, segment and T are checked apart */
    for (int a = 0; a < 4; ++a) {
        put(4 + 2 * a, (uint32_t)pa.dims[a], ~0u);
        put(5 + 2 * a, (uint32_t)(pa.dims[a] >> 32), ~0u);
    }
    put(12, (uint32_t)pa.n, ~0u);
    put(13, (uint32_t)(pa.n >> 32), ~0u);
    put(22, kHeaderBytes, ~0u);
    put(23, 0u, ~0u);
}

/* Absolute bound resolved on the host with the same fp64 -> fp32 round-toward-zero rule the
 * device uses for the relative bound. */
void resolve_abs(double eps, DevInfo *info) {
    const double eb_d = eps;
    float e = (float)eb_d;
    if (std::fabs(e) <= FLT_MAX && (double)e > eb_d) e = std::nextafter(e, 0.0f);
    const float s = 2.0f * e;
    const double inv = 1.0 / (double)s;
    const float r = (float)inv;
    const bool valid = e >= FLT_MIN && e <= FLT_MAX && std::fabs(s) <= FLT_MAX && std::fabs(r) <= FLT_MAX;
    info->eb_f = valid ? e : 0.0f;
    info->s = valid ? s : 0.0f;
    info->r = valid ? r : 0.0f;
    info->valid = valid ? 1u : 0u;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

/* The field pointer of a call: 16-byte aligned for a contiguous plan; for a padded plan any
 * 4-byte aligned pointer (a halo's first interior element often is not 16-byte aligned). */
bool field_ptr_ok(const eblc_plan *plan, const void *p) {
    return plan->pa.lay.strided ? aligned4(p) : aligned16(p);
}

/* Device address of lane k's DevInfo. */
DevInfo *lane_info(const eblc_plan *plan, int k) {
    return reinterpret_cast<DevInfo *>(reinterpret_cast<uint8_t *>(plan->ws.info) + (uint64_t)k * plan->ws_stride);
}

eblc_status hip_status(hipError_t e) { return e == hipSuccess ? EBLC_OK : EBLC_DEVICE_ERROR; }

/* Whether the measurement hook's name filter (",name,name,"; empty: every kernel) names `name`. */
bool timed_kernel(const eblc_plan *p, const char *name) {
    if (p->ev_filter.empty()) return true;
    const size_t len = std::strlen(name);
    for (size_t at = p->ev_filter.find(name); at != std::string::npos; at = p->ev_filter.find(name, at + 1))
        if (p->ev_filter[at - 1] == ',' && p->ev_filter[at + len] == ',') return true;
    return false;
}

/* Measurement hook: the launcher's kernels record the next event pair of the plan's pool while
 * it has room (see LaunchEvents). */
template <typename F>
hipError_t timed(eblc_plan *p, const char *name, F &&launch) {
    if (2 * p->ev_used + 2 > p->ev_pool.size() || !p->ev_sampled || !timed_kernel(p, name)) return launch();
    const size_t k = p->ev_used++;
    p->ev_names[k] = name;
    g_launch_events.start = p->ev_pool[2 * k];
    g_launch_events.stop = p->ev_pool[2 * k + 1];
    const hipError_t e = launch();
    g_launch_events = LaunchEvents{};
    return e;
}

eblc_status check_compress_args(const eblc_plan *plan, const float *in, const void *out) {
    if (in == nullptr || out == nullptr) return EBLC_INVALID_ARGUMENT;
    if (!field_ptr_ok(plan, in) || !aligned16(out)) return EBLC_INVALID_ARGUMENT;
    return EBLC_OK;
}

eblc_status check_decompress_args(const eblc_plan *plan, const void *in, size_t compressed_bytes, const float *out) {
    if (in == nullptr || out == nullptr) return EBLC_INVALID_ARGUMENT;
    if (!aligned16(in) || !field_ptr_ok(plan, out)) return EBLC_INVALID_ARGUMENT;
    /* every stream (RAW ones too) reaches past its header, size section and offset table */
    if (compressed_bytes < kHeaderBytes + plan->pa.wsec + table_bytes(plan->pa.ngroups) ||
        compressed_bytes > kHeaderBytes + align_up(4 * plan->pa.n, 16))
        return EBLC_CORRUPT_STREAM;
    return EBLC_OK;
}

/* The plan's kernel arguments for a launch coding `fields`: 128-bit access to a padded field
 * only when every field pointer of the launch is 16-byte aligned too. */
PlanArgs launch_args(const eblc_plan *plan, const void *const *fields, int nf) {
    PlanArgs pa = plan->pa;
    for (int k = 0; k < nf; ++k)
        if (pa.lay.strided && !aligned16(fields[k])) pa.lay.vec = 0;
    return pa;
}

/* Enqueue the compress of nf <= lanes fields on `st`, field k in lane k's workspace, one
 * launch per stage: range (relative mode) -> encode -> scan (which writes result record k at
 * results + k) -> compaction with outliers. */
hipError_t enqueue_compress(eblc_plan *plan, int nf, const float *const *in, void *const *out,
                            const size_t *out_capacity, eblc_result_t *results, hipStream_t st) {
    const PlanArgs pa = launch_args(plan, reinterpret_cast<const void *const *>(in), nf);
    const Workspace &ws = plan->ws;
    plan->ev_sampled = plan->ev_calls[0]++ % plan->ev_every == plan->ev_every - 1;
    Fields fs{};
    fs.ws_stride = plan->ws_stride;
    for (int k = 0; k < nf; ++k) {
        fs.src[k] = reinterpret_cast<const uint8_t *>(in[k]);
        fs.dst[k] = static_cast<uint8_t *>(out[k]);
        fs.bytes[k] = out_capacity[k];
        fs.result[k] = reinterpret_cast<uint64_t *>(results + k);
        /* the size section goes straight into the stream when the buffer holds it */
        if (out_capacity[k] >= kHeaderBytes + pa.wsec) fs.wdirect |= 1u << k;
    }
    const uint32_t n = (uint32_t)nf;
    hipError_t e = hipSuccess;
    if (plan->rel) e = timed(plan, "range", [&] { return launch_range(fs, n, pa, ws, plan->eps, st); });
    if (e == hipSuccess)
        e = timed(plan, "encode", [&] {
            return pa.V ? launch_chunk_encode(fs, n, pa, ws, st) : launch_encode(fs, n, pa, ws, st);
        });
    if (compact_folds_scan(pa)) {
        if (e == hipSuccess) e = timed(plan, "compact", [&] { return launch_compact_scan(fs, n, pa, ws, st); });
    } else {
        if (e == hipSuccess) e = timed(plan, "scan", [&] { return launch_scan_compress(fs, n, pa, ws, st); });
        if (e == hipSuccess) e = timed(plan, "compact", [&] { return launch_compact(fs, n, pa, ws, st); });
    }
    return e;
}

/* Enqueue the decompress of nf <= lanes streams on `st`, stream k in lane k's workspace:
 * decode (every workgroup checks the header and its group's entry of the offset table) ->
 * outlier patch. */
hipError_t enqueue_decompress(eblc_plan *plan, int nf, const void *const *in, const size_t *compressed_bytes,
                              float *const *out, hipStream_t st) {
    const PlanArgs pa = launch_args(plan, reinterpret_cast<const void *const *>(out), nf);
    const Workspace &ws = plan->ws;
    plan->ev_sampled = plan->ev_calls[1]++ % plan->ev_every == plan->ev_every - 1;
    Fields fs{};
    fs.ws_stride = plan->ws_stride;
    for (int k = 0; k < nf; ++k) {
        fs.src[k] = static_cast<const uint8_t *>(in[k]);
        fs.dst[k] = reinterpret_cast<uint8_t *>(out[k]);
        fs.bytes[k] = compressed_bytes[k];
    }
    const uint32_t n = (uint32_t)nf;
    hipError_t e = timed(plan, "decode", [&] {
        return pa.V ? launch_chunk_decode(fs, n, pa, ws, st) : launch_decode(fs, n, pa, ws, st);
    });
    if (e == hipSuccess) e = timed(plan, "patch", [&] { return launch_patch(fs, n, pa, ws, st); });
    return e;
}

/* Run the `count` calls of a batch in groups of up to `lanes`, one group after another on
 * `st`: call(first, nf) enqueues calls first .. first + nf - 1 as one launch per stage. */
template <typename F>
hipError_t run_batch(eblc_plan *plan, int count, F &&call) {
    for (int k0 = 0; k0 < count; k0 += plan->lanes) {
        const int nf = count - k0 < plan->lanes ? count - k0 : plan->lanes;
        hipError_t e = call(k0, nf);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

/* floor(2^64 / d) + 1, the exact reciprocal for dividing 32-bit values by d >= 2; 0 for d = 1. */
uint64_t reciprocal(uint64_t d) {
    if (d <= 1) return 0;
    return (uint64_t)(((unsigned __int128)1 << 64) / d) + 1;
}

/* Layout of the caller's array from dims and strides (slowest to fastest, strides in elements,
 * "Provider layout").  Accepted: NULL or row-major strides with padding -- fastest stride 1 and
 * each outer stride at least the extent times the stride of the dimension below it.  Anything
 * else (transposed, overlapping, zero or negative strides) is UNSUPPORTED. */
eblc_status make_layout(int rank, const int64_t *dims, const int64_t *strides, Layout *lay) {
    *lay = Layout{};
    lay->rank = (uint32_t)rank;
    lay->L = (uint32_t)dims[rank - 1];
    lay->vec = 1;
    if (strides == nullptr) return EBLC_OK;
    bool contiguous = true;
    int64_t expect = 1;
    for (int a = rank - 1; a >= 0; --a) {
        if (strides[a] != expect) contiguous = false;
        expect *= dims[a];
    }
    if (contiguous) return EBLC_OK;
    if (strides[rank - 1] != 1) return EBLC_UNSUPPORTED;
    unsigned __int128 span = 1;  /* elements a padded array of these strides covers */
    for (int a = rank - 2; a >= 0; --a) {
        if (strides[a] <= 0 || (unsigned __int128)strides[a] < (unsigned __int128)strides[a + 1] * (uint64_t)dims[a + 1])
            return EBLC_UNSUPPORTED;
    }
    for (int a = 0; a < rank; ++a) span += (unsigned __int128)(dims[a] - 1) * (uint64_t)strides[a];
    if (span >= ((unsigned __int128)1 << 62)) return EBLC_UNSUPPORTED;
    lay->strided = 1;
    bool vec = lay->L % 4 == 0;
    for (int a = 0; a < rank - 1; ++a) vec = vec && strides[a] % 4 == 0;
    lay->vec = vec ? 1u : 0u;
    lay->mL = reciprocal(lay->L);
    if (rank >= 2) lay->s1 = (uint64_t)strides[rank - 2];
    if (rank >= 3) {
        lay->o1 = (uint32_t)dims[rank - 2];
        lay->m1 = reciprocal(lay->o1);
        lay->s2 = (uint64_t)strides[rank - 3];
    }
    if (rank >= 4) {
        lay->o2 = (uint32_t)dims[rank - 3];
        lay->m2 = reciprocal(lay->o2);
        lay->s3 = (uint64_t)strides[rank - 4];
    }
    return EBLC_OK;
}

/* Plan constants from the shape, strides and options, with every check that needs no device:
 * rank 1..4, dims > 0 with n < 2^32, the layout, the options, side_max <= n and the 32-bit limit
 * on payload words. */
eblc_status setup_args(int rank, const int64_t *dims, const int64_t *strides, const char *options, Options *o,
                       PlanArgs *out) {
    if (rank < 1 || rank > 4) return EBLC_UNSUPPORTED;
    uint64_t n = 1;
    for (int a = 0; a < rank; ++a) {
        if (dims[a] <= 0) return EBLC_INVALID_ARGUMENT;
        if ((uint64_t)dims[a] >= (1ull << 32)) return EBLC_INVALID_ARGUMENT;
        n *= (uint64_t)dims[a];
        if (n >= (1ull << 32)) return EBLC_INVALID_ARGUMENT;
    }
    Layout lay{};
    eblc_status ls = make_layout(rank, dims, strides, &lay);
    if (ls != EBLC_OK) return ls;
    eblc_status st = parse_options(options, o);
    if (st != EBLC_OK) return st;
    if (!o->side_set) o->side_max = n < (1ull << 23) ? n : (1ull << 23);
    if (o->side_max > n) return EBLC_INVALID_ARGUMENT;
    /* the scans add payload words in 32-bit arithmetic: the largest payload a field can take
     * must stay below 2^32 words */
    if (max_payload_words(n, o->chunk_coder ? o->V : 0) >= (1ull << 32)) return EBLC_INVALID_ARGUMENT;
    PlanArgs &pa = *out;
    pa = PlanArgs{};
    pa.n = n;
    pa.nseg = (n + 31) / 32;
    for (int a = 0; a < 4; ++a) pa.dims[a] = a < rank ? (uint64_t)dims[a] : 0;
    pa.rank = (uint32_t)rank;
    pa.B = o->B;
    pa.T = o->T;
    pa.nchunks = (uint32_t)((n + kEncChunk - 1) / kEncChunk);
    pa.ngroups = (pa.nchunks + kEncChunksPerGroup - 1) / kEncChunksPerGroup;
    if (o->chunk_coder) {
        pa.V = o->V;
        pa.log2seg = (uint32_t)__builtin_ctz(o->V);
        pa.slot = kEncChunk + kEncChunk / 32;
        pa.wpg = 4u * (kEncChunksPerGroup * kEncChunk / o->V);
        pa.dchunks = (uint32_t)((n + o->V - 1) / o->V);
        pa.wsec = align_up(4ull * pa.dchunks, 16);
    } else {
        pa.V = 0;
        pa.log2seg = 5;
        pa.slot = kEncChunk;
        pa.wpg = kEncChunksPerGroup * kEncSegs;
        pa.dchunks = (uint32_t)((n + kDecChunk - 1) / kDecChunk);
        pa.wsec = align_up(pa.nseg, 16);
    }
    pa.dgroups = (pa.dchunks + kDecChunksPerGroup - 1) / kDecChunksPerGroup;
    pa.center = o->center ? 1u : 0u;
    pa.log2B = 0; /* ceil(log2 B) */
    while ((1u << pa.log2B) < pa.B) ++pa.log2B;
    pa.nblocks = (n + pa.B - 1) / pa.B;
    pa.msec = o->center ? align_up(4 * pa.nblocks, 16) : 0;
    pa.side_max = o->side_max;
    pa.max_pw = max_payload_words(n, pa.V);
    pa.lay = lay;
    return EBLC_OK;
}

/* Bytes of one lane's workspace, its arrays 256-byte aligned; with base non-null also the
 * arrays' addresses from base on. */
uint64_t carve_workspace(const PlanArgs &pa, uint8_t *base, Workspace *ws) {
    const uint64_t nc = pa.nchunks, ng = pa.ngroups;
    uint64_t off = 0;
    auto carve = [&](uint64_t bytes) {
        const uint64_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const uint64_t o_info = carve(sizeof(DevInfo));
    /* one spare slot: a 4096-value chunk of the chunk coder spills into its second wave's slot */
    const uint64_t o_scratch = carve(((uint64_t)pa.nchunks + 1) * pa.slot * 4);
    const uint64_t o_cw = carve(nc * 4), o_ce = carve(nc * 4), o_ct = carve(nc * 4);
    const uint64_t o_gw = carve(ng * 4), o_ge = carve(ng * 4);
    const uint64_t o_pw = carve(ng * 4), o_pe = carve(ng * 4);
    const uint64_t o_em = carve(nc * kEncSegs * 4);
    const uint64_t o_wd = carve(nc * kEncSegs);
    const uint64_t o_si = carve(nc * kEscStage * 4), o_sv = carve(nc * kEscStage * 4);
    const uint64_t o_rp = carve(2 * (uint64_t)range_blocks(pa.n) * 4);
    const uint64_t o_mu = carve(pa.nblocks * 4);
    if (base != nullptr && ws != nullptr) {
        uint8_t *b = base;
        ws->info = reinterpret_cast<DevInfo *>(b + o_info);
        ws->scratch = reinterpret_cast<uint32_t *>(b + o_scratch);
        ws->chunk_words = reinterpret_cast<uint32_t *>(b + o_cw);
        ws->chunk_esc = reinterpret_cast<uint32_t *>(b + o_ce);
        ws->chunk_tmask = reinterpret_cast<uint32_t *>(b + o_ct);
        ws->group_words = reinterpret_cast<uint32_t *>(b + o_gw);
        ws->group_esc = reinterpret_cast<uint32_t *>(b + o_ge);
        ws->gpre_words = reinterpret_cast<uint32_t *>(b + o_pw);
        ws->gpre_esc = reinterpret_cast<uint32_t *>(b + o_pe);
        ws->emask = reinterpret_cast<uint32_t *>(b + o_em);
        ws->widths = b + o_wd;
        ws->stage_idx = reinterpret_cast<uint32_t *>(b + o_si);
        ws->stage_val = reinterpret_cast<uint32_t *>(b + o_sv);
        ws->range_part = reinterpret_cast<float *>(b + o_rp);
        ws->means = reinterpret_cast<int32_t *>(b + o_mu);
    }
    return off;
}

/* ---- the compress entry point that allocates nothing -------------------------------------- */

constexpr uint64_t kScratchBytes = 24ull << 20;    /* the static scratch: one workspace */
constexpr uint64_t kScratchMaxValues = 1ull << 22; /* largest field it takes */
constexpr int kMaxDevices = 64;

}  // namespace

/* The workspace of eblc_compress_noalloc: every device the library runs that call on holds one
 * copy until the process ends.  Host code never hands this name to a kernel -- on the host it
 * is only a stand-in for the symbol; a device's copy is addressed through the pointer that
 * hipGetSymbolAddress returns on that device. */
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void *g_scratch_dev[kMaxDevices] = {};

/* Device address of `scratch` on device dev, which must be current: looked up once per device,
 * at the first call there. */
eblc_status scratch_address(int dev, void **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_dev[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return EBLC_DEVICE_ERROR;
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return EBLC_OK;
}

}  // namespace

extern "C" {

int eblc_abi_version(void) { return EBLC_ABI_VERSION; }

const char *eblc_status_string(eblc_status s) {
    switch (s) {
        case EBLC_OK: return "ok";
        case EBLC_UNSUPPORTED: return "unsupported";
        case EBLC_INVALID_ARGUMENT: return "invalid argument";
        case EBLC_CAPACITY: return "output capacity too small";
        case EBLC_CORRUPT_STREAM: return "corrupt stream";
        case EBLC_DEVICE_ERROR: return "device error";
        case EBLC_OUT_OF_MEMORY: return "out of memory";
        case EBLC_TOO_LARGE: return "field too large for the static scratch";
    }
    return "unknown status";
}

eblc_status eblc_plan_create(const eblc_execution_t *exec, eblc_dtype dtype, int rank,
                             const int64_t *dims, const int64_t *strides, const char *options,
                             eblc_plan_t **plan_out) {
    if (plan_out == nullptr || exec == nullptr || dims == nullptr) return EBLC_INVALID_ARGUMENT;
    *plan_out = nullptr;
    if (exec->kind != EBLC_EXECUTION_HIP) return EBLC_UNSUPPORTED;
    if (dtype != EBLC_FLOAT32) return EBLC_UNSUPPORTED;
    Options o;
    PlanArgs pa{};
    eblc_status st = setup_args(rank, dims, strides, options, &o, &pa);
    if (st != EBLC_OK) return st;

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) return EBLC_DEVICE_ERROR;
    if (exec->device < 0 || exec->device >= ndev) return EBLC_INVALID_ARGUMENT;
    DeviceGuard guard(exec->device);
    if (!guard.ok) return EBLC_DEVICE_ERROR;

    eblc_plan *p = new (std::nothrow) eblc_plan();
    if (p == nullptr) return EBLC_OUT_OF_MEMORY;
    p->device = exec->device;
    p->rank = rank;
    for (int a = 0; a < rank; ++a) p->dims[a] = dims[a];
    p->n = pa.n;
    p->rel = o.rel;
    p->eps = o.eps;
    p->pa = pa;
    /* workspace: one allocation, carved into 256-byte aligned arrays, `lanes` times over */
    const uint64_t bytes = carve_workspace(pa, nullptr, nullptr);
    p->lanes = (int)o.lanes;
    if (hipMalloc(&p->ws_base, bytes * o.lanes) != hipSuccess) {
        delete p;
        return EBLC_OUT_OF_MEMORY;
    }
    p->ws_stride = bytes;
    carve_workspace(pa, static_cast<uint8_t *>(p->ws_base), &p->ws);

    if (hipHostMalloc(reinterpret_cast<void **>(&p->host_result), sizeof(eblc_result_t), hipHostMallocDefault) != hipSuccess) {
        eblc_plan_destroy(p);
        return EBLC_OUT_OF_MEMORY;
    }
    DevInfo init;
    std::memset(&init, 0, sizeof(init));
    if (!o.rel) resolve_abs(o.eps, &init);
    header_template(pa, &init);
    for (int lane = 0; lane < p->lanes; ++lane) {
        if (hipMemcpy(lane_info(p, lane), &init, sizeof(init), hipMemcpyHostToDevice) != hipSuccess) {
            eblc_plan_destroy(p);
            return EBLC_DEVICE_ERROR;
        }
    }
    *plan_out = p;
    return EBLC_OK;
}

eblc_status eblc_plan_limits(const eblc_plan_t *plan, eblc_limits_t *out) {
    if (plan == nullptr || out == nullptr) return EBLC_INVALID_ARGUMENT;
    out->max_compressed_bytes = kHeaderBytes + align_up(4 * plan->n, 16);
    out->payload_alignment = 16;
    out->sidecar_bytes = 0;
    out->sidecar_alignment = 1;
    return EBLC_OK;
}

size_t eblc_max_compressed_bytes(const eblc_plan_t *plan) {
    return plan == nullptr ? 0 : (size_t)(kHeaderBytes + align_up(4 * plan->n, 16));
}

size_t eblc_payload_alignment(const eblc_plan_t *plan) { return plan == nullptr ? 0 : 16; }

eblc_status eblc_compress(eblc_plan_t *plan, const float *in, void *out, size_t out_capacity,
                          size_t *compressed_bytes, void *sidecar, void *stream) {
    if (plan == nullptr || compressed_bytes == nullptr) return EBLC_INVALID_ARGUMENT;
    if (sidecar != nullptr) return EBLC_INVALID_ARGUMENT;
    eblc_status s0 = check_compress_args(plan, in, out);
    if (s0 != EBLC_OK) return s0;
    DeviceGuard guard(plan->device);
    if (!guard.ok) return EBLC_DEVICE_ERROR;
    hipStream_t st = static_cast<hipStream_t>(stream);
    /* the compress tail (scan, or the compaction that scans for itself) writes the result record
     * straight into the plan's pinned host slot */
    plan->host_result->compressed_bytes = 0;
    plan->host_result->status = EBLC_DEVICE_ERROR;
    void *outs[1] = {out};
    const size_t caps[1] = {out_capacity};
    hipError_t e = enqueue_compress(plan, 1, &in, outs, caps, plan->host_result, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return EBLC_DEVICE_ERROR;
    *compressed_bytes = (size_t)plan->host_result->compressed_bytes;
    return static_cast<eblc_status>(plan->host_result->status);
}

eblc_status eblc_compress_async(eblc_plan_t *plan, const float *in, void *out, size_t out_capacity,
                                eblc_result_t *result, void *stream) {
    if (plan == nullptr || result == nullptr || (reinterpret_cast<uintptr_t>(result) & 7u) != 0)
        return EBLC_INVALID_ARGUMENT;
    eblc_status s0 = check_compress_args(plan, in, out);
    if (s0 != EBLC_OK) return s0;
    DeviceGuard guard(plan->device);
    if (!guard.ok) return EBLC_DEVICE_ERROR;
    void *outs[1] = {out};
    const size_t caps[1] = {out_capacity};
    return hip_status(enqueue_compress(plan, 1, &in, outs, caps, result, static_cast<hipStream_t>(stream)));
}

eblc_status eblc_compress_noalloc(const eblc_execution_t *exec, int rank, const int64_t *dims,
                                  const int64_t *strides, const char *options, const float *in, void *out,
                                  size_t out_capacity, eblc_result_t *result, void *stream) {
    if (exec == nullptr || dims == nullptr || result == nullptr || (reinterpret_cast<uintptr_t>(result) & 7u) != 0)
        return EBLC_INVALID_ARGUMENT;
    if (exec->kind != EBLC_EXECUTION_HIP) return EBLC_UNSUPPORTED;
    Options o;
    PlanArgs pa{};
    eblc_status st = setup_args(rank, dims, strides, options, &o, &pa);
    if (st != EBLC_OK) return st;
    if (o.lanes != 1) return EBLC_INVALID_ARGUMENT; /* a batch option */
    const uint64_t bytes = carve_workspace(pa, nullptr, nullptr);
    if (pa.n > kScratchMaxValues || bytes > kScratchBytes) return EBLC_TOO_LARGE;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) return EBLC_DEVICE_ERROR;
    if (exec->device < 0 || exec->device >= ndev || exec->device >= kMaxDevices) return EBLC_INVALID_ARGUMENT;
    DeviceGuard guard(exec->device);
    if (!guard.ok) return EBLC_DEVICE_ERROR;
    void *base = nullptr;
    st = scratch_address(exec->device, &base);
    if (st != EBLC_OK) return st;
    /* a plan on the stack over the static scratch: no workspace or events of its own */
    eblc_plan job;
    job.device = exec->device;
    job.rank = rank;
    for (int a = 0; a < rank; ++a) job.dims[a] = dims[a];
    job.n = pa.n;
    job.rel = o.rel;
    job.eps = o.eps;
    job.pa = pa;
    job.lanes = 1;
    job.ws_stride = bytes;
    carve_workspace(pa, static_cast<uint8_t *>(base), &job.ws);
    st = check_compress_args(&job, in, out);
    if (st != EBLC_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    /* a relative bound is resolved by the range pass; an absolute one by one small kernel, since
     * the scratch holds the previous call's bound */
    if (!o.rel) {
        const hipError_t e = launch_resolve_abs(job.ws, o.eps, hs);
        if (e != hipSuccess) return EBLC_DEVICE_ERROR;
    }
    void *outs[1] = {out};
    const size_t caps[1] = {out_capacity};
    return hip_status(enqueue_compress(&job, 1, &in, outs, caps, result, hs));
}

eblc_status eblc_compress_batch(eblc_plan_t *plan, int count, const float *const *in, void *const *out,
                                const size_t *out_capacity, eblc_result_t *results, void *stream) {
    if (plan == nullptr || count < 0 || (count > 0 && (in == nullptr || out == nullptr ||
                                                       out_capacity == nullptr || results == nullptr)))
        return EBLC_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(results) & 7u) != 0) return EBLC_INVALID_ARGUMENT;
    for (int k = 0; k < count; ++k) {
        eblc_status s0 = check_compress_args(plan, in[k], out[k]);
        if (s0 != EBLC_OK) return s0;
    }
    DeviceGuard guard(plan->device);
    if (!guard.ok) return EBLC_DEVICE_ERROR;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(run_batch(plan, count, [&](int k, int nf) {
        return enqueue_compress(plan, nf, in + k, out + k, out_capacity + k, results + k, st);
    }));
}

eblc_status eblc_decompress(eblc_plan_t *plan, const void *in, size_t compressed_bytes,
                            const void *sidecar, float *out, void *stream) {
    if (plan == nullptr || sidecar != nullptr) return EBLC_INVALID_ARGUMENT;
    eblc_status s0 = check_decompress_args(plan, in, compressed_bytes, out);
    if (s0 != EBLC_OK) return s0;
    DeviceGuard guard(plan->device);
    if (!guard.ok) return EBLC_DEVICE_ERROR;
    return hip_status(enqueue_decompress(plan, 1, &in, &compressed_bytes, &out, static_cast<hipStream_t>(stream)));
}

eblc_status eblc_decompress_batch(eblc_plan_t *plan, int count, const void *const *in,
                                  const size_t *compressed_bytes, float *const *out, void *stream) {
    if (plan == nullptr || count < 0 || (count > 0 && (in == nullptr || compressed_bytes == nullptr || out == nullptr)))
        return EBLC_INVALID_ARGUMENT;
    for (int k = 0; k < count; ++k) {
        eblc_status s0 = check_decompress_args(plan, in[k], compressed_bytes[k], out[k]);
        if (s0 != EBLC_OK) return s0;
    }
    DeviceGuard guard(plan->device);
    if (!guard.ok) return EBLC_DEVICE_ERROR;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(run_batch(plan, count, [&](int k, int nf) {
        return enqueue_decompress(plan, nf, in + k, compressed_bytes + k, out + k, st);
    }));
}

eblc_status eblc_plan_status(eblc_plan_t *plan, void *stream) {
    if (plan == nullptr) return EBLC_INVALID_ARGUMENT;
    DeviceGuard guard(plan->device);
    if (!guard.ok) return EBLC_DEVICE_ERROR;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(st) != hipSuccess) return EBLC_DEVICE_ERROR;
    bool corrupt = false;
    for (int lane = 0; lane < plan->lanes; ++lane) {
        uint32_t sticky = 0;
        uint32_t *at = &lane_info(plan, lane)->sticky;
        if (hipMemcpy(&sticky, at, 4, hipMemcpyDeviceToHost) != hipSuccess) return EBLC_DEVICE_ERROR;
        if (sticky) {
            const uint32_t zero = 0;
            if (hipMemcpy(at, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return EBLC_DEVICE_ERROR;
            corrupt = true;
        }
    }
    return corrupt ? EBLC_CORRUPT_STREAM : EBLC_OK;
}

namespace {
void free_events(eblc_plan *plan) {
    for (hipEvent_t ev : plan->ev_pool)
        if (ev) (void)hipEventDestroy(ev);
    plan->ev_pool.clear();
    plan->ev_names.clear();
    plan->ev_used = 0;
}
}  // namespace

void eblc_plan_destroy(eblc_plan_t *plan) {
    if (plan == nullptr) return;
    {
        DeviceGuard guard(plan->device);
        (void)hipDeviceSynchronize();
        free_events(plan);
        if (plan->host_result) (void)hipHostFree(plan->host_result);
        if (plan->ws_base) (void)hipFree(plan->ws_base);
    }
    delete plan;
}

eblc_status eblc_plan_set_profiling(eblc_plan_t *plan, int max_launches, const char *kernels, int every) {
    if (plan == nullptr || max_launches < 0 || (size_t)max_launches > kMaxTimedLaunches || every < 1)
        return EBLC_INVALID_ARGUMENT;
    DeviceGuard guard(plan->device);
    if (!guard.ok) return EBLC_DEVICE_ERROR;
    if (hipDeviceSynchronize() != hipSuccess) return EBLC_DEVICE_ERROR;
    free_events(plan);
    plan->ev_filter.clear();
    if (kernels != nullptr && kernels[0] != '\0') plan->ev_filter = "," + std::string(kernels) + ",";
    plan->ev_every = (uint32_t)every;
    plan->ev_calls[0] = plan->ev_calls[1] = 0;
    if (max_launches == 0) return EBLC_OK;
    plan->ev_pool.assign(2 * (size_t)max_launches, nullptr);
    plan->ev_names.assign((size_t)max_launches, nullptr);
    for (auto &ev : plan->ev_pool) {
        if (hipEventCreate(&ev) != hipSuccess) {
            free_events(plan);
            return EBLC_DEVICE_ERROR;
        }
    }
    return EBLC_OK;
}

int eblc_plan_kernel_times(eblc_plan_t *plan, const char **names, float *ms, int *launches, int max_kernels) {
    if (plan == nullptr || plan->ev_pool.empty() || max_kernels < 0) return -1;
    DeviceGuard guard(plan->device);
    if (!guard.ok) return -1;
    /* fold the recorded launches by kernel name, in order of first launch */
    const char *kname[kMaxKernelsPerCall * 2] = {};
    double total[kMaxKernelsPerCall * 2] = {};
    int cnt[kMaxKernelsPerCall * 2] = {};
    int nk = 0;
    for (size_t k = 0; k < plan->ev_used; ++k) {
        if (hipEventSynchronize(plan->ev_pool[2 * k + 1]) != hipSuccess) return -1;
        float t = 0.0f;
        if (hipEventElapsedTime(&t, plan->ev_pool[2 * k], plan->ev_pool[2 * k + 1]) != hipSuccess) return -1;
        int j = 0;
        while (j < nk && std::strcmp(kname[j], plan->ev_names[k]) != 0) ++j;
        if (j == nk) {
            if (nk == kMaxKernelsPerCall * 2) return -1;
            kname[nk++] = plan->ev_names[k];
        }
        total[j] += t;
        cnt[j] += 1;
    }
    for (int j = 0; j < nk && j < max_kernels; ++j) {
        if (names) names[j] = kname[j];
        if (ms) ms[j] = (float)(total[j] / cnt[j]);
        if (launches) launches[j] = cnt[j];
    }
    plan->ev_used = 0;
    return nk;
}

}  // extern "C"
