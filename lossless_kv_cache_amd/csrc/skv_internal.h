// skv_internal.h -- private declarations shared by the libskv sources.
//
// Format constants: rANS with 12-bit probabilities (M = 4096), 32-bit state
// normalized to [2^16, 2^32), 16-bit words; a stream is 32 interleaved lanes
// x 128 steps; direct alphabets hold at most 255 symbols plus an escape.
#pragma once

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <hip/hip_runtime.h>

#include "../../include/skv.h"

namespace skv {

constexpr uint32_t kProbBits = 12;
constexpr uint32_t kM = 1u << kProbBits;
constexpr uint32_t kStateLow = 1u << 16;
constexpr int kLanes = 32;
constexpr int kSteps = 128;
constexpr int kSyms = kLanes * kSteps;
constexpr int kMaxDirect = 255;
constexpr size_t kHeaderBytes = 64;
constexpr size_t kTableRecord = 514;  // u16 n + u16 freq[256]
constexpr uint32_t kCbHead = 32;       // checkerboard decoder: symbols per table whose starts it keeps in LDS
constexpr size_t kStateBytes = 4 * kLanes;
constexpr uint32_t kStreamHead = 4 * kLanes + 4;   // final states + word count
constexpr uint64_t kRawBit = 1ull << 63;
constexpr int kMaxTimedKernels = 16;

inline uint32_t elem_bytes(uint32_t dtype) { return dtype == SKV_E4M3 ? 1u : 2u; }
// Modes that code [tokens][channels] coefficients in two passes (even, odd tokens).
__host__ __device__ inline bool is_checkerboard(uint32_t mode) {
    return mode == SKV_CHECKERBOARD || mode == SKV_CHECKERBOARD_MAP;
}
// Map section of an SKV_CHECKERBOARD_MAP blob, after the records:
// u32 rank | u32 shift_h | u32 shift_m | u32 0 | int8 V[rank][2C] | int8 U[C][rank].
constexpr size_t kMapHeader = 16;
inline uint64_t map_section_bytes(uint32_t rank, uint32_t channels) {
    return kMapHeader + 3ull * rank * channels;
}
inline bool map_params_ok(uint32_t rank, uint32_t sh_h, uint32_t sh_m) {
    return rank >= 16 && rank <= 256 && (rank & (rank - 1)) == 0 && sh_h <= 40 && sh_m <= 30;
}

// Exponent-conditioned mode: a value's table is chosen by its predictor's
// exponent field (bf16 bits 14..7, e4m3 bits 6..3) as the class E - base,
// clamped to [0, 15], with one base per (layer, K|V) slab.
constexpr uint32_t kExpClasses = 16;
__host__ __device__ inline uint32_t exp_field(uint32_t p, uint32_t dtype) {
    return dtype == SKV_E4M3 ? (p >> 3) & 0xFu : (p >> 7) & 0xFFu;
}
__host__ __device__ inline uint32_t exp_class(uint32_t p, uint32_t dtype, uint32_t base) {
    const uint32_t e = exp_field(p, dtype);
    const uint32_t c = e < base ? 0u : e - base;
    return c < kExpClasses - 1 ? c : kExpClasses - 1;
}

// Shape checks shared by fit / encode / decode.
bool shape_supported(const skv_shape& s, bool need_tokens);
uint64_t table_count(const skv_shape& s);
uint64_t blob_size(const skv_shape& s);      // header + records (+ class bases)
uint64_t stream_count(const skv_shape& s);
uint64_t element_count(const skv_shape& s);

// Host table fit (fp64).  Writes a complete blob (header + records).
int fit_tables_host(const skv_shape& s, const void* calib_t, const void* calib_a, uint32_t calib_tokens,
                    uint8_t* blob, size_t blob_bytes);
// SKV_CHECKERBOARD_MAP: the fit with the map applied to the calibration rows,
// then the map section (blob_bytes = blob_size(s) + map_section_bytes).
int fit_tables_map_host(const skv_shape& s, const int16_t* calib_coef, const int16_t* calib_G,
                        uint32_t calib_tokens, const skv_nbr_map& map, uint8_t* blob, size_t blob_bytes);
// Side input with the map applied, on the host: Gout = G on even tokens, G' on odd ones.
void nbr_map_host(const int16_t* coef, const int16_t* G, uint32_t T, uint32_t C, const skv_nbr_map& map,
                  int16_t* Gout);
int validate_blob(const uint8_t* blob, size_t bytes);
uint64_t fnv1a64(const uint8_t* p, size_t n);

inline void wr16(uint8_t* p, uint32_t v) { p[0] = uint8_t(v); p[1] = uint8_t(v >> 8); }
inline void wr32(uint8_t* p, uint32_t v) { for (int i = 0; i < 4; ++i) p[i] = uint8_t(v >> (8 * i)); }
inline void wr64(uint8_t* p, uint64_t v) { for (int i = 0; i < 8; ++i) p[i] = uint8_t(v >> (8 * i)); }
inline uint32_t rd16(const uint8_t* p) { return uint32_t(p[0]) | (uint32_t(p[1]) << 8); }
inline uint32_t rd32(const uint8_t* p) { return rd16(p) | (rd16(p + 2) << 16); }
inline uint64_t rd64(const uint8_t* p) { return uint64_t(rd32(p)) | (uint64_t(rd32(p + 4)) << 32); }

// ------------------------------------------------------------------ device
// Expanded tables resident in HBM (built once per blob and device).
struct DevTables {
    uint32_t n_tables = 0;
    uint32_t max_n = 0;            // largest direct-symbol count over all tables
    uint32_t* n = nullptr;         // [n_tables] direct-symbol count (ESC index)
    uint4* enc = nullptr;          // [n_tables][256] {freq<<20, divisor magic, 4096-freq, cum<<16 | shift}
    uint32_t* fc = nullptr;        // [n_tables][256] freq | cum<<16
    uint8_t* slot = nullptr;       // [n_tables][4096] slot -> symbol
    // checkerboard blobs: the slots of each table past its first kCbHead symbols (the decoder keeps the
    // starts of those in LDS), one entry per slot: symbol (255 for the escape symbol) | freq << 8 |
    // cum << 20; table j's run starts at tail_base[j]
    uint32_t* tail = nullptr;
    uint32_t* tail_base = nullptr;
    uint2* enc8 = nullptr;         // checkerboard blobs: [n_tables][256] encode entries packed in 8 bytes:
                                   // {magic, f | start << 12 | shift << 24 | inc << 29 | escape << 30}
    uint8_t* base = nullptr;       // exponent-mode blobs: [slabs] class base
    // decoded-neighbour-map blobs: the map (rank 0 otherwise)
    uint32_t map_rank = 0, map_sh_h = 0, map_sh_m = 0;
    int8_t* map_v = nullptr;       // [rank][2C]
    int8_t* map_u = nullptr;       // [C][rank]
};

struct EncodeLaunch {
    const void* target;
    const void* aux;
    const void* aux_odd;    // side input of the odd pass (checkerboard modes): aux, or the mapped side input
    int16_t* map_side;      // decoded-neighbour map: [tokens][channels] workspace for the mapped side input
    uint8_t* scratch;       // [n_streams][2 * raw_bytes]: states, escapes (back of 1st half), words (back of 2nd)
    uint32_t* meta;         // [n_streams] bytes | raw<<31
    uint32_t* block_sum;    // [n_blocks]
    uint64_t* block_off;    // [n_blocks]
    uint64_t* total;        // payload bytes
    uint8_t* out;           // container
    uint64_t out_capacity;
    uint64_t blob_hash;
    skv_shape shape;         // of the streams coded by this launch (a chunk of the container's)
    uint64_t n_streams;
    // A cache coded a chunk at a time (a contiguous run of its streams per launch):
    // the chunk's first stream in the container, the container's stream count and
    // shape, the payload offset of the chunk's first stream (device; null = 0; the
    // chunk's running total lands in *total), and whether the chunk is the last
    // (which writes the header and the final index entry).
    uint64_t sid_base;
    uint64_t n_total;
    const uint64_t* pay_base;
    uint32_t last;
    skv_shape container;
};

struct DecodeLaunch {
    const uint64_t* index;   // the container's stream offsets (n_streams + 1 of its own)
    const uint8_t* pay;      // the container's payload
    uint64_t payload_bytes;
    const void* aux;
    const void* aux_odd;     // side input of the odd pass (checkerboard modes): aux, or out (mapped in place)
    void* out;
    uint32_t* status;
    skv_shape shape;         // of the decoded range (aux and out layout)
    uint64_t n_streams;      // streams decoded
    uint32_t tb_base;        // first token block of the range in the container
    uint32_t ntb_index;      // token blocks per slab in the container
    // checkerboard range that stops before the container's end: 256 rows for
    // the token block after the range, whose even tokens are decoded first
    // (its first row is the right neighbour of the range's last odd token);
    // aux then continues with that block's side input.  Null otherwise.
    int16_t* next_rows;
};

hipError_t build_dev_tables(const uint8_t* blob, DevTables* t, hipStream_t stream);
void free_dev_tables(DevTables* t);
// Encoder phases: kEncodeCode codes the streams into the workspace and sums
// their sizes (the payload size lands in *a.total); kEncodePack writes the
// header, index and streams into a.out.  Between the two, a.out and
// a.out_capacity may change.
constexpr uint32_t kEncodeCode = 1, kEncodePack = 2, kEncodeAll = 3;
hipError_t launch_encode(const EncodeLaunch& a, const DevTables& t, hipStream_t stream, uint32_t phases = kEncodeAll);
hipError_t launch_decode(const DecodeLaunch& a, const DevTables& t, hipStream_t stream);

// The encoder in two calls, for callers that place the container once its
// size is known (the prefix-cache store).  encode_begin validates as
// skv_encode does, codes the streams into d_work (encode workspace size) and
// blocks until pe->container_bytes is known; encode_finish writes the
// container to d_out and returns once it is there.  The blob and d_work must
// stay alive between the two calls, on the same stream.
struct PendingEncode {
    EncodeLaunch a;
    const DevTables* t;
    uint64_t container_bytes;
};
int encode_begin(const void* tables_blob, const skv_shape* s, const void* d_target, const void* d_aux, void* d_work,
                 size_t work_bytes, hipStream_t stream, PendingEncode* pe);
int encode_finish(PendingEncode* pe, void* d_out, size_t out_capacity, hipStream_t stream);
hipError_t launch_clear_u32(uint32_t* p, uint32_t n, hipStream_t stream);
// Decoded-neighbour map on the device: out[t] = G'[t] for every odd token t,
// from the even rows of coef (out may be coef itself: only odd rows are written).
// right: the row after coef's last (a range's next even token, 16-byte
// aligned like the others), or null at the end of the cache.
hipError_t launch_nbr_map(const int16_t* coef, const int16_t* G, int16_t* out, uint32_t tokens, uint32_t channels,
                          const DevTables& t, hipStream_t stream, const int16_t* right = nullptr);
uint64_t encode_work_bytes(uint64_t n_streams, uint32_t raw_bytes);

// Fixed device workspace of skv_encode_noalloc (SKV_NOALLOC_WORK_BYTES).
// noalloc_workspace: the current device's address of it (dev = the current
// device, 0 <= dev < 64), looked up once per device; call it holding
// noalloc_lock(dev), which also serializes the calls that use it.
constexpr size_t kNoAllocWorkBytes = size_t(SKV_NOALLOC_WORK_BYTES);
hipError_t noalloc_workspace(int dev, uint8_t** ptr);
std::mutex& noalloc_lock(int dev);

// per-kernel timing diagnostics (process-wide, not for concurrent callers)
int timing_enable(bool on);
void timing_reset();
void timing_collect();
int timing_read(const char** names, float* ms, int cap);

}  // namespace skv
