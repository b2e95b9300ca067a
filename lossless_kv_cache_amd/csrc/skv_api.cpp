// skv_api.cpp -- the C ABI declared in include/skv.h.
//
// Host side of the coding path: argument and shape checks, the registry of
// library-owned table blobs and their per-device expanded copies, container
// header validation, and the launches on the caller's stream.  The encoder
// is deterministic, as a compressor feeding exact reconstruction must be
// (VeriCache page, section "Compressor interface").
#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <thread>
#include <unordered_map>
#include <utility>
#include <vector>

#include "skv_internal.h"

namespace {

struct Blob {
    uint8_t* bytes = nullptr;
    size_t size = 0;
    uint64_t hash = 0;
    skv_shape shape{};                       // tokens = 0
    std::mutex dev_mu;
    std::map<int, skv::DevTables> dev;       // device ordinal -> expanded tables
    std::mutex part_mu;
    std::map<std::pair<uint32_t, uint32_t>, void*> parts;   // (first layer, layers) -> registered sub-blob
};

std::atomic<bool> g_timing_on{false};

std::mutex g_mu;
std::unordered_map<const void*, Blob*> g_blobs;

Blob* find_blob(const void* p) {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_blobs.find(p);
    return it == g_blobs.end() ? nullptr : it->second;
}

int register_blob(uint8_t* bytes, size_t size, void** out) {
    Blob* b = new (std::nothrow) Blob;
    if (!b) {
        std::free(bytes);
        return SKV_ERR_NOMEM;
    }
    b->bytes = bytes;
    b->size = size;
    b->hash = skv::fnv1a64(bytes, size);
    b->shape = skv_shape{SKV_ABI_VERSION, bytes[6], bytes[7], skv::rd32(bytes + 12), skv::rd32(bytes + 16), 0,
                         skv::rd32(bytes + 20)};
    {
        std::lock_guard<std::mutex> lk(g_mu);
        g_blobs[bytes] = b;
    }
    *out = bytes;
    return SKV_OK;
}

// Expanded tables of blob b on the current device (built on first use).
int device_tables(Blob* b, hipStream_t st, const skv::DevTables** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SKV_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(b->dev_mu);
    auto it = b->dev.find(dev);
    if (it == b->dev.end()) {
        skv::DevTables t;
        if (skv::build_dev_tables(b->bytes, &t, st) != hipSuccess) return SKV_ERR_DEVICE;
        it = b->dev.emplace(dev, t).first;
    }
    *out = &it->second;
    return SKV_OK;
}

bool same_geometry(const skv_shape& blob, const skv_shape& s) {
    return blob.dtype == s.dtype && blob.mode == s.mode && blob.layers == s.layers && blob.kv == s.kv &&
           blob.channels == s.channels;
}

uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// Encoder workspace of a shape: the kernels' scratch, plus the mapped side
// input of the odd tokens in the decoded-neighbour-map mode.
uint64_t encode_need(const skv_shape& s) {
    const uint64_t need = skv::encode_work_bytes(skv::stream_count(s), skv::kSyms * skv::elem_bytes(s.dtype));
    return s.mode == SKV_CHECKERBOARD_MAP ? need + align256(uint64_t(s.tokens) * s.channels * 2) : need;
}

// Small device-to-host reads on the caller's stream (the container size, a
// header, the integrity word).  They go through a pinned staging buffer and
// an event that the calling thread polls, so the host sees the value as soon
// as the copy lands: a blocking stream synchronization wakes the thread
// noticeably later, and the decoder's header read and integrity check sit
// between kernels.  Each thread keeps one staging buffer and event per
// device for its lifetime.
constexpr size_t kStagingBytes = 256;
struct Staging {
    void* host = nullptr;
    hipEvent_t ev = nullptr;
};

// Worker threads that the library starts and joins itself release their
// staging buffers when they end; a caller's thread keeps its own until the
// process exits.
thread_local bool t_release_staging = false;
struct StagingSet {
    std::map<int, Staging> per_dev;
    ~StagingSet() {
        if (!t_release_staging) return;
        for (auto& kv : per_dev) {
            if (kv.second.ev) (void)hipEventDestroy(kv.second.ev);
            if (kv.second.host) (void)hipHostFree(kv.second.host);
        }
    }
};

int read_back(void* dst, const void* src, size_t n, hipStream_t st) {
    thread_local StagingSet staging;
    if (n > kStagingBytes) return SKV_ERR_ARG;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SKV_ERR_DEVICE;
    Staging& sg = staging.per_dev[dev];
    if (!sg.host) {
        if (hipHostMalloc(&sg.host, kStagingBytes, hipHostMallocDefault) != hipSuccess) {
            sg.host = nullptr;
            return SKV_ERR_NOMEM;
        }
        if (hipEventCreateWithFlags(&sg.ev, hipEventDisableTiming) != hipSuccess) {
            (void)hipHostFree(sg.host);
            sg.host = nullptr;
            sg.ev = nullptr;
            return SKV_ERR_DEVICE;
        }
    }
    if (hipMemcpyAsync(sg.host, src, n, hipMemcpyDeviceToHost, st) != hipSuccess) return SKV_ERR_DEVICE;
    if (hipEventRecord(sg.ev, st) != hipSuccess) return SKV_ERR_DEVICE;
    hipError_t e;
    while ((e = hipEventQuery(sg.ev)) == hipErrorNotReady) std::this_thread::yield();
    if (e != hipSuccess) return SKV_ERR_DEVICE;
    std::memcpy(dst, sg.host, n);
    return SKV_OK;
}

}  // namespace

extern "C" {

uint32_t skv_version(void) { return SKV_ABI_VERSION; }

const char* skv_strerror(int status) {
    switch (status) {
        case SKV_OK: return "ok";
        case SKV_ERR_ARG: return "invalid argument";
        case SKV_ERR_SHAPE: return "unsupported shape";
        case SKV_ERR_CAPACITY: return "buffer too small";
        case SKV_ERR_CORRUPT: return "corrupt container";
        case SKV_ERR_TABLES: return "table blob invalid or mismatched";
        case SKV_ERR_DEVICE: return "HIP runtime error";
        case SKV_ERR_NOMEM: return "out of memory";
        case SKV_ERR_BUSY: return "store entry in use";
        default: return "unknown status";
    }
}

int skv_fit_tables(const skv_shape* s, const void* calib_target, const void* calib_aux, uint32_t calib_tokens,
                   void** tables_blob, size_t* blob_bytes) {
    if (!s || !calib_target || !calib_aux || !tables_blob || !blob_bytes) return SKV_ERR_ARG;
    if (!skv::shape_supported(*s, false) || calib_tokens == 0) return SKV_ERR_SHAPE;
    if (s->mode == SKV_CHECKERBOARD_MAP) return SKV_ERR_SHAPE;       // its tables need the map: skv_fit_tables_map
    if (s->mode == SKV_CHECKERBOARD && calib_tokens % 2 != 0) return SKV_ERR_SHAPE;
    const size_t size = skv::blob_size(*s);
    uint8_t* bytes = static_cast<uint8_t*>(std::malloc(size));
    if (!bytes) return SKV_ERR_NOMEM;
    const int rc = skv::fit_tables_host(*s, calib_target, calib_aux, calib_tokens, bytes, size);
    if (rc != SKV_OK) {
        std::free(bytes);
        return rc;
    }
    *blob_bytes = size;
    return register_blob(bytes, size, tables_blob);
}

int skv_fit_tables_map(const skv_shape* s, const void* calib_coef, const void* calib_G, uint32_t calib_tokens,
                       const skv_nbr_map* map, void** tables_blob, size_t* blob_bytes) {
    if (!s || !calib_coef || !calib_G || !map || !map->V || !map->U || !tables_blob || !blob_bytes)
        return SKV_ERR_ARG;
    if (s->mode != SKV_CHECKERBOARD_MAP || !skv::shape_supported(*s, false) || calib_tokens == 0 ||
        calib_tokens % 2 != 0)
        return SKV_ERR_SHAPE;
    if (!skv::map_params_ok(map->rank, map->shift_h, map->shift_m)) return SKV_ERR_ARG;
    const size_t size = skv::blob_size(*s) + skv::map_section_bytes(map->rank, s->channels);
    uint8_t* bytes = static_cast<uint8_t*>(std::malloc(size));
    if (!bytes) return SKV_ERR_NOMEM;
    const int rc = skv::fit_tables_map_host(*s, static_cast<const int16_t*>(calib_coef),
                                            static_cast<const int16_t*>(calib_G), calib_tokens, *map, bytes, size);
    if (rc != SKV_OK) {
        std::free(bytes);
        return rc;
    }
    *blob_bytes = size;
    return register_blob(bytes, size, tables_blob);
}

int skv_load_tables(const void* blob, size_t blob_bytes, void** tables_blob) {
    if (!blob || !tables_blob) return SKV_ERR_ARG;
    const int rc = skv::validate_blob(static_cast<const uint8_t*>(blob), blob_bytes);
    if (rc != SKV_OK) return rc;
    uint8_t* bytes = static_cast<uint8_t*>(std::malloc(blob_bytes));
    if (!bytes) return SKV_ERR_NOMEM;
    std::memcpy(bytes, blob, blob_bytes);
    return register_blob(bytes, blob_bytes, tables_blob);
}

void skv_free(void* tables_blob) {
    if (!tables_blob) return;
    Blob* b = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_blobs.find(tables_blob);
        if (it == g_blobs.end()) return;
        b = it->second;
        g_blobs.erase(it);
    }
    for (auto& kv : b->parts) skv_free(kv.second);
    int cur = 0;
    const bool have = hipGetDevice(&cur) == hipSuccess;
    for (auto& kv : b->dev) {
        if (hipSetDevice(kv.first) == hipSuccess) skv::free_dev_tables(&kv.second);
    }
    if (have) (void)hipSetDevice(cur);
    std::free(b->bytes);
    delete b;
}

// The encoder's launch arguments for the streams of shape s, its workspace
// carved from w for `carve` streams (encode_need-sized for all of them,
// 256-byte aligned).  Set up as a single pass over the whole container.
static skv::EncodeLaunch encode_launch(const Blob* b, const skv_shape& s, const void* d_target, const void* d_aux,
                                       void* d_out, size_t out_capacity, uint8_t* w, uint64_t carve = 0) {
    const uint64_t n = skv::stream_count(s);
    const uint64_t m = carve ? carve : n;
    const uint32_t raw = skv::kSyms * skv::elem_bytes(s.dtype);
    skv::EncodeLaunch a{};
    a.target = d_target;
    a.aux = d_aux;
    a.aux_odd = d_aux;
    a.scratch = w;
    w += align256(2 * m * raw);
    a.meta = reinterpret_cast<uint32_t*>(w);
    w += align256(4 * m);
    const uint64_t nb = (m + 1023) / 1024;
    a.block_sum = reinterpret_cast<uint32_t*>(w);
    w += align256(4 * nb);
    a.block_off = reinterpret_cast<uint64_t*>(w);
    w += align256(8 * nb);
    a.total = reinterpret_cast<uint64_t*>(w);
    w += 256;
    if (s.mode == SKV_CHECKERBOARD_MAP) {
        a.map_side = reinterpret_cast<int16_t*>(w);                    // odd rows written by the map
        a.aux_odd = a.map_side;
    }
    a.out = static_cast<uint8_t*>(d_out);
    a.out_capacity = out_capacity;
    a.blob_hash = b->hash;
    a.shape = s;
    a.n_streams = n;
    a.sid_base = 0;
    a.n_total = n;
    a.pay_base = nullptr;
    a.last = 1;
    a.container = s;
    return a;
}

// A pass of the encoder: whole slabs [slab0, slab0 + nslab) (slab = layer x
// K|V), or token blocks [tb0, tb0 + ntb) of slab slab0.  Either way a
// contiguous run of the container's streams.
struct Pass {
    uint32_t slab0, nslab, tb0, ntb;
};

// How a cache is cut into passes: one pass; `step` whole slabs per pass; or
// `step` token blocks of one slab per pass.  per_pass: the streams a pass's
// workspace is carved for.
struct Plan {
    enum { kOne, kSlabs, kBlocks } kind;
    uint32_t step, passes;
    uint64_t per_pass;
};

static uint32_t token_blocks(const skv_shape& s) {
    return skv::is_checkerboard(s.mode) ? s.tokens / (2 * skv::kSteps) : s.tokens / skv::kSteps;
}

static Pass pass_at(const Plan& pl, const skv_shape& s, uint32_t c) {
    const uint32_t slabs = s.layers * s.kv, ntb = token_blocks(s);
    if (pl.kind == Plan::kOne) return Pass{0, slabs, 0, ntb};
    if (pl.kind == Plan::kSlabs) return Pass{c * pl.step, std::min(pl.step, slabs - c * pl.step), 0, ntb};
    const uint32_t per_slab = (ntb + pl.step - 1) / pl.step;
    const uint32_t t0 = (c % per_slab) * pl.step;
    return Pass{c / per_slab, 1, t0, std::min(pl.step, ntb - t0)};
}

// The fewest passes whose workspace fits in `budget` bytes (0: no limit):
// one pass when the whole cache fits, else as many whole slabs per pass as
// fit, else as many token blocks of a slab.  Checkerboard shapes take one
// pass (the odd tokens are coded against the even ones).  Returns false, with
// *min_bytes the smallest workspace that works, when nothing fits.
static bool plan_passes(const skv_shape& s, uint64_t budget, Plan* pl, uint64_t* min_bytes) {
    const uint64_t n = skv::stream_count(s);
    const uint32_t raw = skv::kSyms * skv::elem_bytes(s.dtype);
    const uint32_t slabs = s.layers * s.kv, ncg = s.channels / skv::kLanes, ntb = token_blocks(s);
    if (budget == 0 || budget >= encode_need(s)) {
        *pl = Plan{Plan::kOne, 0, 1, n};
        return true;
    }
    *min_bytes = skv::is_checkerboard(s.mode) ? encode_need(s) : skv::encode_work_bytes(ncg, raw);
    if (skv::is_checkerboard(s.mode)) return false;
    // the largest stream count whose workspace fits (the size grows with the count)
    uint64_t lo = 0, hi = n;
    while (lo < hi) {
        const uint64_t mid = (lo + hi + 1) / 2;
        if (skv::encode_work_bytes(mid, raw) <= budget) lo = mid;
        else hi = mid - 1;
    }
    const uint64_t per_slab = uint64_t(ntb) * ncg;
    if (lo >= per_slab) {
        const uint32_t k = uint32_t(std::min<uint64_t>(lo / per_slab, slabs));
        *pl = Plan{Plan::kSlabs, k, (slabs + k - 1) / k, uint64_t(k) * per_slab};
        return true;
    }
    const uint32_t j = uint32_t(lo / ncg);
    if (j == 0) return false;
    *pl = Plan{Plan::kBlocks, j, slabs * ((ntb + j - 1) / j), uint64_t(j) * ncg};
    return true;
}

// The device tables seen from slab slab0 on (a pass's slab 0).
static skv::DevTables tables_from_slab(const skv::DevTables& t, const skv_shape& s, uint32_t slab0) {
    skv::DevTables u = t;
    if (slab0 == 0) return u;
    const uint64_t off = uint64_t(slab0) * (s.mode == SKV_RESIDUAL_EXP ? skv::kExpClasses : s.channels);
    u.n_tables -= uint32_t(off);
    if (u.n) u.n += off;
    if (u.enc) u.enc += off * 256;
    if (u.fc) u.fc += off * 256;
    if (u.slot) u.slot += off * skv::kM;
    if (u.base) u.base += slab0;
    return u;
}

// Code the cache in the planned passes, each into the same workspace, and
// pack every pass's streams into d_out; *payload receives the payload size.
// A pass's payload offset carries over on the device (two running totals,
// alternating), so the host waits once, at the end: through the pinned
// staging buffer, or (plain) a plain copy and a stream synchronization, which
// allocate nothing.
static int encode_passes(const Blob* b, const skv_shape& s, const skv::DevTables& t, const Plan& plan,
                         const void* d_target, const void* d_aux, void* d_out, size_t out_capacity, uint8_t* w,
                         hipStream_t stream, uint64_t* payload, bool plain = false) {
    const uint32_t eb = skv::elem_bytes(s.dtype);
    const uint32_t ncg = s.channels / skv::kLanes, ntb = token_blocks(s);
    const uint64_t n = skv::stream_count(s);
    const uint64_t* slots = nullptr;
    for (uint32_t c = 0; c < plan.passes; ++c) {
        const Pass p = pass_at(plan, s, c);
        skv_shape ps = s;
        if (plan.kind != Plan::kOne) {
            ps.layers = p.nslab;
            ps.kv = 1;
            ps.tokens = p.ntb * skv::kSteps;
        }
        const size_t off = (size_t(p.slab0) * s.tokens + size_t(p.tb0) * skv::kSteps) * s.channels * eb;
        skv::EncodeLaunch a = encode_launch(b, ps, static_cast<const uint8_t*>(d_target) + off,
                                            static_cast<const uint8_t*>(d_aux) + off, d_out, out_capacity, w,
                                            plan.per_pass);
        uint64_t* tot = a.total;
        slots = tot;
        a.total = tot + ((c + 1) & 1);
        a.pay_base = c ? tot + (c & 1) : nullptr;
        a.sid_base = (uint64_t(p.slab0) * ntb + p.tb0) * ncg;
        a.n_total = n;
        a.last = c + 1 == plan.passes;
        a.container = s;
        const skv::DevTables u = tables_from_slab(t, s, p.slab0);
        if (skv::launch_encode(a, u, stream) != hipSuccess) return SKV_ERR_DEVICE;
    }
    const uint64_t* fin = slots + (plan.passes & 1);
    if (!plain) return read_back(payload, fin, 8, stream);
    if (hipMemcpyAsync(payload, fin, 8, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return SKV_ERR_DEVICE;
    return SKV_OK;
}

static int encode_impl(const void* tables_blob, const skv_shape* s, const void* d_target, const void* d_aux,
                       void* d_out, size_t out_capacity, size_t* out_bytes, void* d_work, size_t* work_bytes,
                       hipStream_t stream, bool timing) {
    if (!tables_blob || !s || !out_bytes || !work_bytes) return SKV_ERR_ARG;
    if (!skv::shape_supported(*s, true)) return SKV_ERR_SHAPE;
    Blob* b = find_blob(tables_blob);
    if (!b) return SKV_ERR_ARG;
    if (!same_geometry(b->shape, *s)) return SKV_ERR_TABLES;
    const uint64_t n = skv::stream_count(*s);
    const uint32_t raw = skv::kSyms * skv::elem_bytes(s->dtype);
    const uint64_t bound = skv::kHeaderBytes + 8 * (n + 1) + n * raw;
    const uint64_t need = encode_need(*s);
    if (!d_out || !d_work) {
        if (!d_out) *out_bytes = bound;
        if (!d_work) *work_bytes = need;
        return SKV_OK;
    }
    Plan plan{};
    uint64_t min_bytes = 0;
    if (!plan_passes(*s, *work_bytes, &plan, &min_bytes)) {
        *work_bytes = min_bytes;
        return SKV_ERR_CAPACITY;
    }
    if (!d_target || !d_aux) return SKV_ERR_ARG;
    const skv::DevTables* t = nullptr;
    int rc = device_tables(b, stream, &t);
    if (rc != SKV_OK) return rc;

    if (timing) skv::timing_reset();
    uint64_t payload = 0;
    rc = encode_passes(b, *s, *t, plan, d_target, d_aux, d_out, out_capacity, static_cast<uint8_t*>(d_work), stream,
                       &payload);
    if (rc != SKV_OK) return rc;
    if (timing) skv::timing_collect();
    const uint64_t total = skv::kHeaderBytes + 8 * (n + 1) + payload;
    *out_bytes = total;
    return total > out_capacity ? SKV_ERR_CAPACITY : SKV_OK;
}

int skv_encode(const void* tables_blob, const skv_shape* s, const void* d_target, const void* d_aux, void* d_out,
               size_t out_capacity, size_t* out_bytes, void* d_work, size_t* work_bytes, hipStream_t stream) {
    return encode_impl(tables_blob, s, d_target, d_aux, d_out, out_capacity, out_bytes, d_work, work_bytes, stream,
                       true);
}

int skv_encode_workspace(const skv_shape* s, uint64_t max_bytes, size_t* work_bytes, uint32_t* passes) {
    if (!s || !work_bytes || !passes) return SKV_ERR_ARG;
    if (!skv::shape_supported(*s, true)) return SKV_ERR_SHAPE;
    Plan plan{};
    uint64_t min_bytes = 0;
    if (!plan_passes(*s, max_bytes, &plan, &min_bytes)) {
        *work_bytes = min_bytes;
        return SKV_ERR_CAPACITY;
    }
    *work_bytes = plan.kind == Plan::kOne ? encode_need(*s)
                                          : skv::encode_work_bytes(plan.per_pass, skv::kSyms * skv::elem_bytes(s->dtype));
    *passes = plan.passes;
    return SKV_OK;
}

int skv_encode_noalloc(const void* tables_blob, const skv_shape* s, const void* d_target, const void* d_aux,
                       void* d_out, size_t out_capacity, size_t* out_bytes, hipStream_t stream) {
    if (!tables_blob || !s || !out_bytes) return SKV_ERR_ARG;
    if (!skv::shape_supported(*s, true)) return SKV_ERR_SHAPE;
    Blob* b = find_blob(tables_blob);
    if (!b) return SKV_ERR_ARG;
    if (!same_geometry(b->shape, *s)) return SKV_ERR_TABLES;
    const uint64_t n = skv::stream_count(*s);
    const uint32_t raw = skv::kSyms * skv::elem_bytes(s->dtype);
    const uint64_t bound = skv::kHeaderBytes + 8 * (n + 1) + n * raw;
    Plan plan{};
    uint64_t min_bytes = 0;
    if (!plan_passes(*s, skv::kNoAllocWorkBytes, &plan, &min_bytes)) return SKV_ERR_SHAPE;
    if (!d_out) {
        *out_bytes = bound;
        return SKV_OK;
    }
    if (!d_target || !d_aux) return SKV_ERR_ARG;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SKV_ERR_DEVICE;
    const skv::DevTables* t = nullptr;
    {
        // resident tables only: building them would allocate
        std::lock_guard<std::mutex> lk(b->dev_mu);
        auto it = b->dev.find(dev);
        if (it == b->dev.end()) return SKV_ERR_ARG;
        t = &it->second;
    }
    if (dev < 0 || dev >= 64) return SKV_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(skv::noalloc_lock(dev));
    uint8_t* w = nullptr;
    if (skv::noalloc_workspace(dev, &w) != hipSuccess) return SKV_ERR_DEVICE;
    skv::timing_reset();
    uint64_t payload = 0;
    const int rc = encode_passes(b, *s, *t, plan, d_target, d_aux, d_out, out_capacity, w, stream, &payload, true);
    if (rc != SKV_OK) return rc;
    skv::timing_collect();
    const uint64_t total = skv::kHeaderBytes + 8 * (n + 1) + payload;
    *out_bytes = total;
    return total > out_capacity ? SKV_ERR_CAPACITY : SKV_OK;
}

// Decode of token blocks [tb0, tb1) of every slab of a container (all of them
// for skv_decode).  tb1 = 0 stands for the container's last token block + 1.
static int decode_blocks(const void* tables_blob, const void* d_in, size_t in_bytes, bool range, uint32_t token_begin,
                         uint32_t token_end, const void* d_aux, void* d_out, size_t out_capacity, void* d_work,
                         size_t* work_bytes, hipStream_t stream, bool timing = true) {
    if (!tables_blob || !work_bytes) return SKV_ERR_ARG;
    Blob* b = find_blob(tables_blob);
    if (!b) return SKV_ERR_ARG;
    // the status word; a checkerboard range also decodes the even tokens of
    // the block after it (256 rows) into the workspace
    const bool cb = skv::is_checkerboard(b->shape.mode);
    const uint64_t need = 256 + (cb && range ? align256(2ull * skv::kSteps * b->shape.channels * 2) : 0);
    if (!d_work) {
        *work_bytes = need;
        return SKV_OK;
    }
    if (*work_bytes < need) {
        *work_bytes = need;
        return SKV_ERR_CAPACITY;
    }
    if (!d_in || !d_aux || !d_out) return SKV_ERR_ARG;
    if (in_bytes < skv::kHeaderBytes) return SKV_ERR_CORRUPT;
    uint8_t h[skv::kHeaderBytes];
    int rc = read_back(h, d_in, sizeof h, stream);
    if (rc != SKV_OK) return rc;
    if (std::memcmp(h, "SKV1", 4) != 0 || skv::rd16(h + 4) != 1) return SKV_ERR_CORRUPT;
    if (h[8] != skv::kProbBits || h[9] != skv::kLanes || skv::rd16(h + 10) != skv::kSteps) return SKV_ERR_CORRUPT;
    skv_shape s{SKV_ABI_VERSION, h[6], h[7], skv::rd32(h + 12), skv::rd32(h + 16), skv::rd32(h + 20),
                skv::rd32(h + 24)};
    if (!skv::shape_supported(s, true)) return SKV_ERR_CORRUPT;
    const uint64_t n = skv::stream_count(s);
    if (skv::rd64(h + 32) != n) return SKV_ERR_CORRUPT;
    if (skv::rd64(h + 40) != b->hash || !same_geometry(b->shape, s)) return SKV_ERR_TABLES;
    const uint64_t payload = skv::rd64(h + 48);
    const uint64_t head = skv::kHeaderBytes + 8 * (n + 1);
    if (in_bytes < head || in_bytes - head < payload) return SKV_ERR_CORRUPT;
    // the decoded part: whole token blocks (128 tokens; checkerboard: 128 even and 128 odd)
    skv_shape part = s;
    uint32_t tb_base = 0;
    const uint32_t blk = cb ? 2 * skv::kSteps : skv::kSteps;
    if (range) {
        if (token_begin >= token_end || token_end > s.tokens || token_begin % blk != 0 || token_end % blk != 0)
            return SKV_ERR_SHAPE;
        // checkerboard ranges take the per-stream decoder, which keeps a range under 2 GiB
        if (cb && uint64_t(token_end - token_begin) * s.channels * 2 >= (1ull << 31)) return SKV_ERR_SHAPE;
        part.tokens = token_end - token_begin;
        tb_base = token_begin / blk;
    }
    if (out_capacity < skv::element_count(part) * skv::elem_bytes(part.dtype)) return SKV_ERR_CAPACITY;
    const skv::DevTables* t = nullptr;
    rc = device_tables(b, stream, &t);
    if (rc != SKV_OK) return rc;
    skv::DecodeLaunch a{};
    a.index = reinterpret_cast<const uint64_t*>(static_cast<const uint8_t*>(d_in) + skv::kHeaderBytes);
    a.pay = static_cast<const uint8_t*>(d_in) + head;
    a.payload_bytes = payload;
    a.aux = d_aux;
    // decoded-neighbour map: the odd pass reads its side input from the output's odd rows,
    // where the map of the decoded even rows is written between the passes
    a.aux_odd = s.mode == SKV_CHECKERBOARD_MAP ? d_out : d_aux;
    a.out = d_out;
    a.status = static_cast<uint32_t*>(d_work);
    a.shape = part;
    a.n_streams = skv::stream_count(part);
    a.tb_base = tb_base;
    a.ntb_index = s.tokens / blk;
    // a checkerboard range before the container's end: the next block's even rows after the status word
    a.next_rows = cb && range && token_end < s.tokens
                      ? reinterpret_cast<int16_t*>(static_cast<uint8_t*>(d_work) + 256)
                      : nullptr;
    if (skv::launch_clear_u32(a.status, 1, stream) != hipSuccess) return SKV_ERR_DEVICE;
    if (timing) skv::timing_reset();
    if (skv::launch_decode(a, *t, stream) != hipSuccess) return SKV_ERR_DEVICE;
    uint32_t status = 0;
    rc = read_back(&status, a.status, 4, stream);
    if (rc != SKV_OK) return rc;
    if (timing) skv::timing_collect();
    return status ? SKV_ERR_CORRUPT : SKV_OK;
}

int skv_decode(const void* tables_blob, const void* d_in, size_t in_bytes, const void* d_aux, void* d_out,
               size_t out_capacity, void* d_work, size_t* work_bytes, hipStream_t stream) {
    return decode_blocks(tables_blob, d_in, in_bytes, false, 0, 0, d_aux, d_out, out_capacity, d_work, work_bytes,
                         stream);
}

int skv_decode_range(const void* tables_blob, const void* d_in, size_t in_bytes, uint32_t token_begin,
                     uint32_t token_end, const void* d_aux, void* d_out, size_t out_capacity, void* d_work,
                     size_t* work_bytes, hipStream_t stream) {
    return decode_blocks(tables_blob, d_in, in_bytes, true, token_begin, token_end, d_aux, d_out, out_capacity, d_work,
                         work_bytes, stream);
}

// The tables of layers [l0, l0 + nl) of a residual-mode blob as a blob of
// their own (header with the part's layer and table counts, the part's
// records, and in exponent mode its slabs' base bytes), registered once and
// kept with the parent until skv_free releases both.
static int layer_part(Blob* b, uint32_t l0, uint32_t nl, Blob** out) {
    std::lock_guard<std::mutex> lk(b->part_mu);
    auto key = std::make_pair(l0, nl);
    auto it = b->parts.find(key);
    if (it == b->parts.end()) {
        skv_shape one = b->shape, part = b->shape;
        one.layers = 1;
        part.layers = nl;
        const uint64_t per_layer = skv::table_count(one);
        const size_t size = skv::blob_size(part);
        uint8_t* bytes = static_cast<uint8_t*>(std::malloc(size));
        if (!bytes) return SKV_ERR_NOMEM;
        std::memcpy(bytes, b->bytes, skv::kHeaderBytes);
        skv::wr32(bytes + 8, uint32_t(per_layer * nl));
        skv::wr32(bytes + 12, nl);
        skv::wr64(bytes + 32, size);
        std::memcpy(bytes + skv::kHeaderBytes, b->bytes + skv::kHeaderBytes + l0 * per_layer * skv::kTableRecord,
                    nl * per_layer * skv::kTableRecord);
        if (b->shape.mode == SKV_RESIDUAL_EXP) {
            const size_t bases = skv::kHeaderBytes + skv::table_count(b->shape) * skv::kTableRecord;
            std::memcpy(bytes + skv::kHeaderBytes + nl * per_layer * skv::kTableRecord,
                        b->bytes + bases + size_t(l0) * b->shape.kv, size_t(nl) * b->shape.kv);
        }
        int rc = skv::validate_blob(bytes, size);
        void* handle = nullptr;
        if (rc == SKV_OK) {
            rc = register_blob(bytes, size, &handle);
        } else {
            std::free(bytes);
        }
        if (rc != SKV_OK) return rc;
        it = b->parts.emplace(key, handle).first;
    }
    *out = find_blob(it->second);
    return *out ? SKV_OK : SKV_ERR_TABLES;
}

int skv_transfer(const void* tables_blob, const skv_shape* s, uint32_t layers_per_chunk, const void* d_target,
                 const void* d_aux_send, void* h_wire, size_t wire_capacity, size_t* wire_bytes,
                 uint64_t* chunk_offsets, const void* d_aux_recv, void* d_out, size_t out_capacity, void* d_work,
                 size_t* work_bytes, hipStream_t stream) {
    if (!tables_blob || !s || !wire_bytes || !work_bytes) return SKV_ERR_ARG;
    if (!skv::shape_supported(*s, true) || skv::is_checkerboard(s->mode)) return SKV_ERR_SHAPE;
    Blob* b = find_blob(tables_blob);
    if (!b) return SKV_ERR_ARG;
    if (!same_geometry(b->shape, *s)) return SKV_ERR_TABLES;
    if (layers_per_chunk == 0 || layers_per_chunk > s->layers) return SKV_ERR_ARG;

    const uint32_t nc = (s->layers + layers_per_chunk - 1) / layers_per_chunk;
    skv_shape cs = *s;
    cs.layers = layers_per_chunk;
    const uint32_t raw = skv::kSyms * skv::elem_bytes(s->dtype);
    const uint64_t n_chunk = skv::stream_count(cs);
    const uint64_t bound_chunk = skv::kHeaderBytes + 8 * (n_chunk + 1) + n_chunk * raw;
    const uint64_t n_all = skv::stream_count(*s);
    const uint64_t wire_bound = uint64_t(nc) * (skv::kHeaderBytes + 8) + 8 * n_all + n_all * raw;
    const uint64_t enc_need = skv::encode_work_bytes(n_chunk, raw);
    const uint64_t dec_need = 256;
    const uint64_t slot = align256(bound_chunk);
    const uint64_t need = 4 * slot + align256(enc_need) + dec_need;
    if (!h_wire || !d_work) {
        if (!h_wire) *wire_bytes = wire_bound;
        if (!d_work) *work_bytes = need;
        return SKV_OK;
    }
    if (*work_bytes < need) {
        *work_bytes = need;
        return SKV_ERR_CAPACITY;
    }
    if (!d_target || !d_aux_send || !d_aux_recv || !d_out || !chunk_offsets) return SKV_ERR_ARG;
    if (g_timing_on) return SKV_ERR_ARG;
    const uint64_t layer_bytes = uint64_t(s->kv) * s->tokens * s->channels * skv::elem_bytes(s->dtype);
    if (out_capacity < layer_bytes * s->layers) return SKV_ERR_CAPACITY;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SKV_ERR_DEVICE;
    std::vector<Blob*> part(nc);
    std::vector<skv_shape> shp(nc);
    for (uint32_t c = 0; c < nc; ++c) {
        const uint32_t l0 = c * layers_per_chunk;
        shp[c] = *s;
        shp[c].layers = std::min(layers_per_chunk, s->layers - l0);
        const int rc = layer_part(b, l0, shp[c].layers, &part[c]);
        if (rc != SKV_OK) return rc;
    }

    // streams (default priority) and per-chunk events
    hipStream_t s_enc = nullptr, s_d2h = nullptr, s_h2d = nullptr, s_dec = nullptr;
    hipEvent_t ev_start = nullptr;
    std::vector<hipEvent_t> ev_enc(nc, nullptr), ev_d2h(nc, nullptr), ev_h2d(nc, nullptr);
    bool ok = hipStreamCreateWithFlags(&s_enc, hipStreamNonBlocking) == hipSuccess &&
              hipStreamCreateWithFlags(&s_d2h, hipStreamNonBlocking) == hipSuccess &&
              hipStreamCreateWithFlags(&s_h2d, hipStreamNonBlocking) == hipSuccess &&
              hipStreamCreateWithFlags(&s_dec, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&ev_start, hipEventDisableTiming) == hipSuccess;
    for (uint32_t c = 0; ok && c < nc; ++c)
        ok = hipEventCreateWithFlags(&ev_enc[c], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&ev_d2h[c], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&ev_h2d[c], hipEventDisableTiming) == hipSuccess;
    // the caller's earlier work on its stream (inputs, outputs) comes first
    ok = ok && hipEventRecord(ev_start, stream) == hipSuccess &&
         hipStreamWaitEvent(s_enc, ev_start, 0) == hipSuccess &&
         hipStreamWaitEvent(s_dec, ev_start, 0) == hipSuccess;
    // device tables of every part before either side starts
    const skv::DevTables* dt = nullptr;
    for (uint32_t c = 0; ok && c < nc; ++c) ok = device_tables(part[c], s_enc, &dt) == SKV_OK;

    uint8_t* w = static_cast<uint8_t*>(d_work);
    uint8_t* cont[2] = {w, w + slot};
    uint8_t* recv[2] = {w + 2 * slot, w + 3 * slot};
    uint8_t* enc_work = w + 4 * slot;
    uint8_t* dec_work = enc_work + align256(enc_need);
    uint8_t* wire = static_cast<uint8_t*>(h_wire);
    const uint8_t* tgt = static_cast<const uint8_t*>(d_target);
    const uint8_t* aux_s = static_cast<const uint8_t*>(d_aux_send);
    const uint8_t* aux_r = static_cast<const uint8_t*>(d_aux_recv);
    uint8_t* out = static_cast<uint8_t*>(d_out);

    std::mutex mu;
    std::condition_variable cv;
    uint32_t produced = 0;                    // chunks whose device-to-host copy is queued
    bool stop = false;
    int send_rc = ok ? SKV_OK : SKV_ERR_DEVICE, recv_rc = SKV_OK;
    std::vector<uint64_t> size(nc, 0);

    // Receiver: host-to-device copy of each chunk as it arrives (the next
    // chunk's copy queued before the current chunk's decode), then decode.
    auto receiver = [&] {
        t_release_staging = true;
        if (hipSetDevice(dev) != hipSuccess) {
            std::lock_guard<std::mutex> lk(mu);
            recv_rc = SKV_ERR_DEVICE;
            stop = true;
            cv.notify_all();
            return;
        }
        uint32_t next = 0;
        for (uint32_t c = 0; c < nc; ++c) {
            uint32_t avail;
            {
                std::unique_lock<std::mutex> lk(mu);
                cv.wait(lk, [&] { return produced > c || stop; });
                if (produced <= c) return;
                avail = produced;
            }
            int rc = SKV_OK;
            for (; rc == SKV_OK && next < avail && next <= c + 1; ++next) {
                // recv[next & 1] last held chunk next - 2, decoded before this point
                if (hipStreamWaitEvent(s_h2d, ev_d2h[next], 0) != hipSuccess ||
                    hipMemcpyAsync(recv[next & 1], wire + chunk_offsets[next], size[next], hipMemcpyHostToDevice,
                                   s_h2d) != hipSuccess ||
                    hipEventRecord(ev_h2d[next], s_h2d) != hipSuccess)
                    rc = SKV_ERR_DEVICE;
            }
            if (rc == SKV_OK && hipStreamWaitEvent(s_dec, ev_h2d[c], 0) != hipSuccess) rc = SKV_ERR_DEVICE;
            const uint64_t off = uint64_t(c) * layers_per_chunk * layer_bytes;
            size_t wb = dec_need;
            if (rc == SKV_OK)
                rc = decode_blocks(part[c]->bytes, recv[c & 1], size[c], false, 0, 0, aux_r + off, out + off,
                                   shp[c].layers * layer_bytes, dec_work, &wb, s_dec, false);
            if (rc != SKV_OK) {
                std::lock_guard<std::mutex> lk(mu);
                recv_rc = rc;
                stop = true;
                cv.notify_all();
                return;
            }
        }
    };
    std::thread rx;
    if (send_rc == SKV_OK) rx = std::thread(receiver);

    // Sender (this thread): encode chunk c into cont[c & 1] while the copies
    // and the decode of earlier chunks proceed on their own streams.
    uint64_t wire_off = 0;
    for (uint32_t c = 0; send_rc == SKV_OK && c < nc; ++c) {
        {
            std::lock_guard<std::mutex> lk(mu);
            if (stop) break;
        }
        int rc = SKV_OK;
        if (c >= 2 && hipStreamWaitEvent(s_enc, ev_d2h[c - 2], 0) != hipSuccess) rc = SKV_ERR_DEVICE;
        const uint64_t off = uint64_t(c) * layers_per_chunk * layer_bytes;
        size_t bytes = 0, wb = enc_need;
        if (rc == SKV_OK)
            rc = encode_impl(part[c]->bytes, &shp[c], tgt + off, aux_s + off, cont[c & 1], bound_chunk, &bytes, enc_work,
                             &wb, s_enc, false);
        if (rc == SKV_OK && bytes > wire_capacity - wire_off) rc = SKV_ERR_CAPACITY;
        if (rc == SKV_OK &&
            (hipEventRecord(ev_enc[c], s_enc) != hipSuccess || hipStreamWaitEvent(s_d2h, ev_enc[c], 0) != hipSuccess ||
             hipMemcpyAsync(wire + wire_off, cont[c & 1], bytes, hipMemcpyDeviceToHost, s_d2h) != hipSuccess ||
             hipEventRecord(ev_d2h[c], s_d2h) != hipSuccess))
            rc = SKV_ERR_DEVICE;
        std::lock_guard<std::mutex> lk(mu);
        if (rc != SKV_OK) {
            send_rc = rc;
            stop = true;
        } else {
            chunk_offsets[c] = wire_off;
            size[c] = bytes;
            wire_off += bytes;
            produced = c + 1;
        }
        cv.notify_all();
    }
    if (rx.joinable()) rx.join();
    // nothing queued by this call may still run once it returns
    for (hipStream_t st : {s_enc, s_d2h, s_h2d, s_dec})
        if (st && hipStreamSynchronize(st) != hipSuccess && send_rc == SKV_OK) send_rc = SKV_ERR_DEVICE;
    for (uint32_t c = 0; c < nc; ++c)
        for (hipEvent_t e : {ev_enc[c], ev_d2h[c], ev_h2d[c]})
            if (e) (void)hipEventDestroy(e);
    if (ev_start) (void)hipEventDestroy(ev_start);
    for (hipStream_t st : {s_enc, s_d2h, s_h2d, s_dec})
        if (st) (void)hipStreamDestroy(st);
    if (send_rc == SKV_ERR_CAPACITY) {
        *wire_bytes = wire_bound;
        return send_rc;
    }
    if (send_rc != SKV_OK) return send_rc;
    if (recv_rc != SKV_OK) return recv_rc;
    chunk_offsets[nc] = wire_off;
    *wire_bytes = wire_off;
    return SKV_OK;
}

int skv_kernel_timing(int enable) {
    const int rc = skv::timing_enable(enable != 0);
    if (rc == SKV_OK) g_timing_on = enable != 0;
    return rc;
}

int skv_kernel_times(const char** names, float* ms, int capacity) {
    if (capacity < 0) return SKV_ERR_ARG;
    return skv::timing_read(names, ms, capacity);
}

}  // extern "C"

namespace skv {

int encode_begin(const void* tables_blob, const skv_shape* s, const void* d_target, const void* d_aux, void* d_work,
                 size_t work_bytes, hipStream_t stream, PendingEncode* pe) {
    if (!tables_blob || !s || !pe || !d_target || !d_aux || !d_work) return SKV_ERR_ARG;
    if (!shape_supported(*s, true)) return SKV_ERR_SHAPE;
    Blob* b = find_blob(tables_blob);
    if (!b) return SKV_ERR_ARG;
    if (!same_geometry(b->shape, *s)) return SKV_ERR_TABLES;
    if (work_bytes < encode_need(*s)) return SKV_ERR_CAPACITY;
    const DevTables* t = nullptr;
    int rc = device_tables(b, stream, &t);
    if (rc != SKV_OK) return rc;
    pe->a = encode_launch(b, *s, d_target, d_aux, nullptr, 0, static_cast<uint8_t*>(d_work));
    pe->t = t;
    if (launch_encode(pe->a, *t, stream, kEncodeCode) != hipSuccess) return SKV_ERR_DEVICE;
    uint64_t payload = 0;
    rc = read_back(&payload, pe->a.total, 8, stream);
    if (rc != SKV_OK) return rc;
    pe->container_bytes = kHeaderBytes + 8 * (pe->a.n_streams + 1) + payload;
    return SKV_OK;
}

int encode_finish(PendingEncode* pe, void* d_out, size_t out_capacity, hipStream_t stream) {
    if (!pe || !d_out) return SKV_ERR_ARG;
    if (out_capacity < pe->container_bytes) return SKV_ERR_CAPACITY;
    pe->a.out = static_cast<uint8_t*>(d_out);
    pe->a.out_capacity = out_capacity;
    if (launch_encode(pe->a, *pe->t, stream, kEncodePack) != hipSuccess) return SKV_ERR_DEVICE;
    // the read of the magic waits for the pack kernels
    uint8_t magic[4];
    const int rc = read_back(magic, d_out, sizeof magic, stream);
    if (rc != SKV_OK) return rc;
    return std::memcmp(magic, "SKV1", 4) == 0 ? SKV_OK : SKV_ERR_DEVICE;
}

}  // namespace skv
