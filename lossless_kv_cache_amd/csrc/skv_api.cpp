// skv_api.cpp -- the C ABI declared in include/skv.h.
//
// Host side of the coding path: argument and shape checks, the registry of
// library-owned table blobs and their per-device expanded copies, container
// header validation, and the launches on the caller's stream.  The encoder
// is deterministic, as a compressor feeding exact reconstruction must be
// (VeriCache page, section "Compressor interface").
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <thread>
#include <unordered_map>

#include "skv_internal.h"

namespace {

struct Blob {
    uint8_t* bytes = nullptr;
    size_t size = 0;
    uint64_t hash = 0;
    skv_shape shape{};                       // tokens = 0
    std::mutex dev_mu;
    std::map<int, skv::DevTables> dev;       // device ordinal -> expanded tables
};

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

int read_back(void* dst, const void* src, size_t n, hipStream_t st) {
    thread_local std::map<int, Staging> staging;
    if (n > kStagingBytes) return SKV_ERR_ARG;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SKV_ERR_DEVICE;
    Staging& sg = staging[dev];
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
        default: return "unknown status";
    }
}

int skv_fit_tables(const skv_shape* s, const void* calib_target, const void* calib_aux, uint32_t calib_tokens,
                   void** tables_blob, size_t* blob_bytes) {
    if (!s || !calib_target || !calib_aux || !tables_blob || !blob_bytes) return SKV_ERR_ARG;
    if (!skv::shape_supported(*s, false) || calib_tokens == 0) return SKV_ERR_SHAPE;
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
    int cur = 0;
    const bool have = hipGetDevice(&cur) == hipSuccess;
    for (auto& kv : b->dev) {
        if (hipSetDevice(kv.first) == hipSuccess) skv::free_dev_tables(&kv.second);
    }
    if (have) (void)hipSetDevice(cur);
    std::free(b->bytes);
    delete b;
}

int skv_encode(const void* tables_blob, const skv_shape* s, const void* d_target, const void* d_aux, void* d_out,
               size_t out_capacity, size_t* out_bytes, void* d_work, size_t* work_bytes, hipStream_t stream) {
    if (!tables_blob || !s || !out_bytes || !work_bytes) return SKV_ERR_ARG;
    if (!skv::shape_supported(*s, true)) return SKV_ERR_SHAPE;
    Blob* b = find_blob(tables_blob);
    if (!b) return SKV_ERR_ARG;
    if (!same_geometry(b->shape, *s)) return SKV_ERR_TABLES;
    const uint64_t n = skv::stream_count(*s);
    const uint32_t raw = skv::kSyms * skv::elem_bytes(s->dtype);
    const uint64_t bound = skv::kHeaderBytes + 8 * (n + 1) + n * raw;
    const uint64_t need = skv::encode_work_bytes(n, raw);
    if (!d_out || !d_work) {
        if (!d_out) *out_bytes = bound;
        if (!d_work) *work_bytes = need;
        return SKV_OK;
    }
    if (*work_bytes < need) {
        *work_bytes = need;
        return SKV_ERR_CAPACITY;
    }
    if (!d_target || !d_aux) return SKV_ERR_ARG;
    const skv::DevTables* t = nullptr;
    int rc = device_tables(b, stream, &t);
    if (rc != SKV_OK) return rc;

    uint8_t* w = static_cast<uint8_t*>(d_work);
    skv::EncodeLaunch a{};
    a.target = d_target;
    a.aux = d_aux;
    a.scratch = w;
    w += align256(2 * n * raw);
    a.meta = reinterpret_cast<uint32_t*>(w);
    w += align256(4 * n);
    const uint64_t nb = (n + 1023) / 1024;
    a.block_sum = reinterpret_cast<uint32_t*>(w);
    w += align256(4 * nb);
    a.block_off = reinterpret_cast<uint64_t*>(w);
    w += align256(8 * nb);
    a.total = reinterpret_cast<uint64_t*>(w);
    a.out = static_cast<uint8_t*>(d_out);
    a.out_capacity = out_capacity;
    a.blob_hash = b->hash;
    a.shape = *s;
    a.n_streams = n;
    skv::timing_reset();
    if (skv::launch_encode(a, *t, stream) != hipSuccess) return SKV_ERR_DEVICE;
    uint64_t payload = 0;
    rc = read_back(&payload, a.total, 8, stream);
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
                         size_t* work_bytes, hipStream_t stream) {
    if (!tables_blob || !work_bytes) return SKV_ERR_ARG;
    Blob* b = find_blob(tables_blob);
    if (!b) return SKV_ERR_ARG;
    const uint64_t need = 256;
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
    // the decoded part: whole token blocks of a residual container
    skv_shape part = s;
    uint32_t tb_base = 0;
    if (range) {
        if (s.mode == SKV_CHECKERBOARD || token_begin >= token_end || token_end > s.tokens ||
            token_begin % skv::kSteps != 0 || token_end % skv::kSteps != 0)
            return SKV_ERR_SHAPE;
        part.tokens = token_end - token_begin;
        tb_base = token_begin / skv::kSteps;
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
    a.out = d_out;
    a.status = static_cast<uint32_t*>(d_work);
    a.shape = part;
    a.n_streams = skv::stream_count(part);
    a.tb_base = tb_base;
    a.ntb_index = s.tokens / skv::kSteps;
    if (skv::launch_clear_u32(a.status, 1, stream) != hipSuccess) return SKV_ERR_DEVICE;
    skv::timing_reset();
    if (skv::launch_decode(a, *t, stream) != hipSuccess) return SKV_ERR_DEVICE;
    uint32_t status = 0;
    rc = read_back(&status, a.status, 4, stream);
    if (rc != SKV_OK) return rc;
    skv::timing_collect();
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

int skv_kernel_timing(int enable) { return skv::timing_enable(enable != 0); }

int skv_kernel_times(const char** names, float* ms, int capacity) {
    if (capacity < 0) return SKV_ERR_ARG;
    return skv::timing_read(names, ms, capacity);
}

}  // extern "C"
