// skv_kernels.hip -- gfx950 kernels of the coding path.
//
//   expand_tables   blob records -> per-table encode entries (frequency,
//                   start, divisor magic), decode slot->symbol maps and
//                   (frequency, start) words, resident in HBM
//   encode_streams  symbolize + 32-lane interleaved rANS encode, one
//                   stream per half wavefront; words placed by ballot
//   stream_block_sums / stream_block_scan / place_streams / copy_streams
//                   stream sizes -> exclusive scan -> u64 index, header, and
//                   the compacted container
//   decode_streams  rANS decode + reconstruction, one stream per half
//                   wavefront; checkerboard mode runs it twice
//
// The residual of the target against the predictor is what is coded
// ("Speculative KV coding ..." page, section "Core idea"); the coder is rANS
// against per-channel Laplace tables (DCKV page, section "How it differs"),
// and checkerboard mode shifts the table by a mean from the side input and,
// on odd tokens, from the two decoded even neighbours (same section).
// Everything on the device is integer arithmetic.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include <hip/hip_ext.h>

#include "skv_internal.h"

// Workspace of skv_encode_noalloc, for callers that cannot allocate device
// memory: one fixed array, of which the runtime holds a copy on every GPU
// the library runs on until the process ends.  Host code never uses this
// name as an address (on the host it stands for the symbol, not for device
// memory): it asks the runtime for the current device's address of it once
// per device (noalloc_workspace below) and passes that address to kernels.
static __device__ __align__(256) uint8_t scratch[skv::kNoAllocWorkBytes];

namespace skv {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu[kMaxDevices];     // one call at a time per device
uint8_t* g_noalloc_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_workspace(int dev, uint8_t** ptr) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!g_noalloc_ptr[dev]) {
        // the caller holds g_noalloc_mu[dev] and has made `dev` current
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_noalloc_ptr[dev] = static_cast<uint8_t*>(p);
    }
    *ptr = g_noalloc_ptr[dev];
    return hipSuccess;
}

std::mutex& noalloc_lock(int dev) { return g_noalloc_mu[dev]; }

namespace {

constexpr uint32_t kStreamsPerBlock = 8;    // 256 threads = 4 wavefronts x 2 streams
constexpr uint32_t kScanBlock = 1024;

struct Geo {
    uint32_t C, T, ncg, ntb;
};

__device__ __forceinline__ Geo geometry(const skv_shape& s) {
    Geo g;
    g.C = s.channels;
    g.T = s.tokens;
    g.ncg = s.channels / kLanes;
    g.ntb = (!is_checkerboard(s.mode) ? s.tokens : s.tokens / 2) / kSteps;
    return g;
}

// --------------------------------------------------------------- symbol maps
// Order-preserving integer of a 16-bit / 8-bit sign-magnitude pattern.
__device__ __forceinline__ uint32_t ord16(uint32_t u) {
    const uint32_t neg = 0u - (u >> 15);                 // all ones when the sign is set
    return (u ^ (0x8000u | (neg & 0x7FFFu))) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t unord16(uint32_t o) {
    const uint32_t pos = 0u - (o >> 15);                 // all ones when o came from a non-negative value
    return (o ^ (0xFFFFu ^ (pos & 0x7FFFu))) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t ord8(uint32_t u) {
    const uint32_t neg = 0u - (u >> 7);
    return (u ^ (0x80u | (neg & 0x7Fu))) & 0xFFu;
}
__device__ __forceinline__ uint32_t unord8(uint32_t o) {
    const uint32_t pos = 0u - (o >> 7);
    return (o ^ (0xFFu ^ (pos & 0x7Fu))) & 0xFFu;
}
// zigzag of an N-bit two's-complement value held in the low N bits
__device__ __forceinline__ uint32_t zig16(uint32_t r) { return ((r << 1) ^ (0u - ((r >> 15) & 1u))) & 0xFFFFu; }
__device__ __forceinline__ uint32_t zig8(uint32_t r) { return ((r << 1) ^ (0u - ((r >> 7) & 1u))) & 0xFFu; }
__device__ __forceinline__ uint32_t unzig(uint32_t z) { return (z >> 1) ^ (0u - (z & 1u)); }   // mod 2^32

// --------------------------------------------------------------- tables
__global__ __launch_bounds__(256) void expand_tables(const uint8_t* rec, uint32_t* tn, uint4* enc, uint32_t* fc,
                                                     uint8_t* slot, uint32_t* tail, const uint32_t* tail_base,
                                                     uint2* enc8) {
    __shared__ uint32_t cum[257];
    const uint32_t j = blockIdx.x, tid = threadIdx.x;
    const uint8_t* r = rec + size_t(j) * kTableRecord;
    const uint32_t n = uint32_t(r[0]) | (uint32_t(r[1]) << 8);
    const uint32_t f = tid <= n ? (uint32_t(r[2 + 2 * tid]) | (uint32_t(r[3 + 2 * tid]) << 8)) : 0u;
    cum[tid + 1] = f;
    if (tid == 0) cum[0] = 0;
    __syncthreads();
    for (uint32_t d = 1; d < 256; d <<= 1) {
        const uint32_t v = (tid + 1 >= d) ? cum[tid + 1 - d] : 0u;
        __syncthreads();
        cum[tid + 1] += v;
        __syncthreads();
    }
    const uint32_t c = cum[tid];
    if (tid == 0) tn[j] = n;
    // encode entry: renormalization bound f * 2^20, divisor magic m,
    // (4096 - f) | inc << 24 and l | start << 16, where
    // floor(x / f) = mulhi(x + inc, m) >> l for every x < 2^32 - 1.  With
    // 2^l < f < 2^(l+1), m rounds 2^(32+l) / f up when that error is at most
    // 2^l and down otherwise (then inc = 1); one of the two always holds
    // (Robison, "N-bit unsigned division via N-bit multiply-add").  Powers of
    // two shift, and f = 1 uses m = 2^32 - 1 with inc = 1.
    // entries past n repeat the escape symbol's entry; escape entries carry bit 8 of w
    // (a kernel may then look a symbol up by min(z, 255) without reading n)
    const uint32_t se = min(tid, n);
    const uint32_t fe = uint32_t(r[2 + 2 * se]) | (uint32_t(r[3 + 2 * se]) << 8);
    const uint32_t ce = cum[se];
    uint4 e = make_uint4(0u, 0u, 0u, 0u);
    if (fe > 0) {
        const uint32_t f = fe, c = ce;
        uint32_t m, inc = 0, l = 0;
        if ((f & (f - 1)) == 0) {
            while ((1u << (l + 1)) <= f) ++l;                   // f = 2^l
            if (l == 0) {
                m = 0xFFFFFFFFu;
                inc = 1;
            } else {
                m = 0x80000000u;
                l -= 1;
            }
        } else {
            while ((2u << l) <= f) ++l;
            const uint64_t P = 1ull << (32 + l);
            const uint64_t mu = (P + f - 1) / f;
            if (mu * f - P <= (1ull << l)) {
                m = uint32_t(mu);
            } else {
                m = uint32_t(mu - 1);
                inc = 1;
            }
        }
        e.x = f << 20;
        e.y = m;
        e.z = (kM - f) | (inc << 24);
        e.w = l | (c << 16) | (tid >= n ? 0x100u : 0u);
    }
    enc[size_t(j) * 256 + tid] = e;
    // the same entry in 8 bytes (checkerboard tables: f < 4096, start < 4096, shift < 12)
    if (enc8)
        enc8[size_t(j) * 256 + tid] = make_uint2(e.y, (e.x >> 20) | ((e.w >> 16) << 12) | ((e.w & 31u) << 24) |
                                                          ((e.z >> 24) << 29) | (((e.w >> 8) & 1u) << 30));
    fc[size_t(j) * 256 + tid] = f | (c << 16);
    uint8_t* st = slot + size_t(j) * kM;
    for (uint32_t q = c; q < c + f; ++q) st[q] = uint8_t(tid);
    if (tail) {
        // checkerboard tables: the slots from the start of symbol min(kCbHead, n) on (f < 4096)
        const uint32_t ts = cum[min(kCbHead, n)];
        uint32_t* tt = tail + tail_base[j] - ts;
        const uint32_t ent = (tid == n ? 255u : tid) | (f << 8) | (c << 20);
        for (uint32_t q = max(c, ts); q < c + f; ++q) tt[q] = ent;
    }
}

// --------------------------------------------------------------- encode
// One rANS put shared by every lane of a wavefront.  Lanes whose state is too
// large for their symbol first emit their low 16 bits; inside a stream the
// words are ranked from lane 31 down to lane 0 (reverse of the decoder's
// refill order) and written backwards from the end of the stream's scratch.
__device__ __forceinline__ void emit_words(uint32_t& x, uint32_t& cnt, bool emit, uint32_t lane, uint32_t half,
                                           uint16_t* words, uint32_t maxw) {
    const uint64_t b = __ballot(emit);
    const uint32_t mine = uint32_t(b >> half);
    if (emit) {
        const uint32_t above = __popc(uint32_t((uint64_t)mine >> (lane + 1)));
        const uint32_t pos = cnt + above;
        if (pos < maxw) words[pos] = uint16_t(x & 0xFFFFu);
        x >>= 16;
    }
    cnt += __popc(mine);
}

template <uint32_t DT, uint32_t MODE>
__global__ __launch_bounds__(256) void encode_streams(EncodeLaunch a, DevTables t) {
    const uint32_t tid = threadIdx.x;
    const uint64_t sid = uint64_t(blockIdx.x) * kStreamsPerBlock + (tid >> 5);
    if (sid >= a.n_streams) return;
    const uint32_t lane = tid & 31u, half = tid & 32u;
    const Geo g = geometry(a.shape);
    const uint32_t cg = uint32_t(sid % g.ncg);
    const uint32_t tb = uint32_t((sid / g.ncg) % g.ntb);
    const uint32_t slab = uint32_t(sid / (uint64_t(g.ncg) * g.ntb));
    const uint32_t ch = cg * kLanes + lane;
    constexpr uint32_t EB = DT == SKV_E4M3 ? 1u : 2u;
    constexpr uint32_t RAW = kSyms * EB;
    constexpr uint32_t MAXW = (RAW - kStreamHead) / 2;     // more words or escapes mean a raw stream
    constexpr uint32_t MAXE = (RAW - kStreamHead) / EB;
    uint8_t* area = a.scratch + sid * (2 * RAW);
    uint16_t* wfwd = reinterpret_cast<uint16_t*>(area + RAW);           // words, emission order
    uint8_t* efwd = area + kStreamHead;                                  // escaped values, emission order
    const uint32_t res_table = slab * g.C + ch;

    uint32_t x = kStateLow, cnt = 0, ecnt = 0;
    for (int k = kSteps - 1; k >= 0; --k) {
        uint32_t z, table;
        if (MODE != SKV_CHECKERBOARD) {
            const size_t idx = (size_t(slab) * g.T + size_t(tb) * kSteps + k) * g.C + ch;
            uint32_t pv;
            if (DT == SKV_E4M3) {
                const uint32_t tv = static_cast<const uint8_t*>(a.target)[idx];
                pv = static_cast<const uint8_t*>(a.aux)[idx];
                z = zig8((ord8(tv) - ord8(pv)) & 0xFFu);
            } else {
                const uint32_t tv = static_cast<const uint16_t*>(a.target)[idx];
                pv = static_cast<const uint16_t*>(a.aux)[idx];
                z = zig16((ord16(tv) - ord16(pv)) & 0xFFFFu);
            }
            table = MODE == SKV_RESIDUAL ? res_table : slab * kExpClasses + exp_class(pv, DT, t.base[slab]);
        } else {
            const uint32_t tok = 2u * (tb * kSteps + uint32_t(k)) + slab;
            const int16_t* coef = static_cast<const int16_t*>(a.target);
            const int16_t* G = static_cast<const int16_t*>(slab ? a.aux_odd : a.aux);
            int32_t mu = G[size_t(tok) * g.C + ch];
            if (slab == 1) {
                const int32_t l = coef[size_t(tok - 1) * g.C + ch];
                const int32_t r = (tok + 1 < g.T) ? int32_t(coef[size_t(tok + 1) * g.C + ch]) : l;
                mu += 8 * (l + r);
            }
            const int32_t kk = mu >> 4;
            table = ch * 16u + uint32_t(mu & 15);
            z = zig16(uint32_t(int32_t(coef[size_t(tok) * g.C + ch]) - kk) & 0xFFFFu);
        }
        const uint32_t n = t.n[table];
        const bool esc = z >= n;
        const uint32_t s = esc ? n : z;
        {
            // escaped values keep decode order: ranked like the words, written backwards
            const uint64_t b = __ballot(esc);
            const uint32_t mine = uint32_t(b >> half);
            if (esc) {
                const uint32_t pos = ecnt + __popc(uint32_t((uint64_t)mine >> (lane + 1)));
                if (pos < MAXE) {
                    if (EB == 1) efwd[pos] = uint8_t(z);
                    else reinterpret_cast<uint16_t*>(efwd)[pos] = uint16_t(z);
                }
            }
            ecnt += __popc(mine);
        }
        const uint4 e = t.enc[size_t(table) * 256 + s];
        emit_words(x, cnt, x >= e.x, lane, half, wfwd, MAXW);
        const uint32_t qt = __umulhi(x + (e.z >> 24), e.y) >> (e.w & 31u);    // floor(x / f)
        x = x + (e.w >> 16) + __umul24(qt, e.z);
    }
    reinterpret_cast<uint32_t*>(area)[lane] = x;
    if (lane == 0) {
        const uint32_t bytes = (kStreamHead + 2 * cnt + EB * ecnt + 3) & ~3u;
        a.meta[sid] = bytes >= RAW ? 0x80000000u : (cnt | (ecnt << 14));
    }
}

// Stream of this half-wave in the checkerboard kernels: a block codes HW
// token blocks of one channel group (64 bytes of each int16 row), and the
// blocks dispatched to one XCD (round-robin over the 8 XCDs) sweep one pair of
// channel groups after another, the two groups of a pair taking the same
// token blocks side by side: the two halves of a 128-byte row line are read
// (and written) by blocks that run together on one XCD, and the tables the
// XCD reads at a time (16 per component, two groups) stay in its L2.  Returns
// the block's index in group-major order (channel group, then token blocks).
// HW: half-waves (streams) per block.
template <uint32_t HW = 8>
__device__ __forceinline__ uint32_t cb_block(const Geo& g) {
    const uint32_t bpc = (g.ntb + HW - 1) / HW;            // blocks per channel group
    const uint32_t total = g.ncg * bpc;
    const uint32_t b = blockIdx.x;
    if (total % 8 != 0) return b;
    const uint32_t q = (b % 8) * (total / 8) + b / 8;      // position in the XCD's sweep
    if (g.ncg % 2 != 0) return q;
    const uint32_t pair = q / (2 * bpc), r = q % (2 * bpc);
    return (2 * pair + (r & 1u)) * bpc + r / 2;
}
// The channel group of this block (the same for all its half-waves; ncg or
// more for a block past the last one).
template <uint32_t HW = 8>
__device__ __forceinline__ uint32_t cb_group(const Geo& g) { return cb_block<HW>(g) / ((g.ntb + HW - 1) / HW); }
template <uint32_t HW = 8>
__device__ __forceinline__ bool cb_stream(const Geo& g, uint64_t first, uint64_t& sid) {
    const uint32_t bpc = (g.ntb + HW - 1) / HW;
    const uint32_t w = cb_block<HW>(g);
    const uint32_t cg = w / bpc, tb = (w % bpc) * HW + (threadIdx.x >> 5);
    if (cg >= g.ncg || tb >= g.ntb) return false;
    const uint64_t pass = first / (uint64_t(g.ncg) * g.ntb);
    sid = (pass * g.ntb + tb) * g.ncg + cg;
    return true;
}

// Checkerboard encoder.  The 32,768 tables (16 shifted tables per
// component) stay in device memory; a block's 16 streams share one channel
// group, and the packed entries of symbols 0..11 of its 32 x 16 tables sit in
// LDS, so only larger symbols read their entry from device memory.  None of a
// step's reads depends on the rANS state, so they are all issued ahead of the
// state chain, in batches of 8 steps (steps run from 127 down to 0):
//   * the coefficients, side inputs and neighbours of batch j + 1 are loaded
//     while batch j is coded;
//   * the table entries of batch j are requested before batch j + 1's loads,
//     so waiting for them never waits for those;
//   * words and escaped values go to per-stream LDS rings and out to the
//     workspace once per batch, so no store is pending while the batch waits
//     on its loads (loads and stores share one counter and complete out of
//     order with respect to each other, so a pending store turns every wait
//     into a wait for everything).
// Every load is issued unconditionally (a lane without a device-memory entry
// reads the first entry), so the number of loads in flight is the same on
// every path and each wait names exactly the loads it needs.  Output order
// and format are those of encode_streams.
constexpr uint32_t kCbEncHead = 12;                      // symbols per table whose entries stay in LDS
constexpr uint32_t kCbEncStreams = 16;                   // streams (half-waves) per block
constexpr uint32_t kCbEncLane = 16 * kCbEncHead + 1;     // entries per lane: an odd count spreads the lanes'
                                                         // 8-byte reads over the bank pairs
constexpr uint32_t kCbEncBatch = 8;                      // steps per batch
constexpr uint32_t kCbEncRing = kCbEncBatch * kLanes;    // words a stream can emit in one batch
constexpr uint32_t kCbEncEsc = 64;                       // escaped values per batch kept in LDS (more go out at once)

template <bool PASS>
__device__ __forceinline__ void encode_cb_stream(const EncodeLaunch& a, const DevTables& t, const Geo& g,
                                                 uint64_t sid, const uint2* ehead, uint16_t* wring,
                                                 uint16_t* ering) {
    constexpr uint32_t RAW = 2 * kSyms;
    constexpr uint32_t MAXW = (RAW - kStreamHead) / 2;     // more words or escapes mean a raw stream
    constexpr uint32_t MAXE = (RAW - kStreamHead) / 2;
    constexpr uint32_t B = kCbEncBatch, NB = kSteps / kCbEncBatch;
    const uint32_t lane = threadIdx.x & 31u, half = threadIdx.x & 32u;
    const uint32_t cg = uint32_t(sid % g.ncg);
    const uint32_t tb = uint32_t((sid / g.ncg) % g.ntb);
    const uint32_t ch = cg * kLanes + lane;
    uint8_t* area = a.scratch + sid * (2 * RAW);
    uint16_t* wfwd = reinterpret_cast<uint16_t*>(area + RAW);           // words, emission order
    uint16_t* efwd = reinterpret_cast<uint16_t*>(area + kStreamHead);   // escaped values, emission order
    const uint32_t C = g.C;
    const uint2* lhead = ehead + lane * kCbEncLane;
    // rows are addressed from the block's first row (uniform) with 32-bit byte offsets: a block's 16
    // token blocks span 4096 rows
    const uint32_t tb0 = __builtin_amdgcn_readfirstlane(tb & ~(kCbEncStreams - 1u));
    const size_t row0 = size_t(2u * tb0 * kSteps) * C;
    const char* cbase = reinterpret_cast<const char*>(static_cast<const int16_t*>(a.target) + row0);
    const char* gbase = reinterpret_cast<const char*>(static_cast<const int16_t*>(PASS ? a.aux_odd : a.aux) + row0);
    const char* tbase = reinterpret_cast<const char*>(t.enc8);
    const uint32_t tok0 = 2u * ((tb - tb0) * kSteps) + (PASS ? 1u : 0u);      // row of step 0, from row0
    const bool last_blk = 2u * (tb * kSteps + kSteps - 1u) + 2u >= g.T;       // step 127's right row is past the end
    auto at = [](const char* base, uint32_t off) { return int32_t(*reinterpret_cast<const int16_t*>(base + off)); };

    // inputs of batch j: step 127 - B j - i in slot i (j = NB loads step 0 again, unused)
    int32_t ic[B], ig[B], il[B], ir[B];
    auto load_batch = [&](uint32_t j) {
#pragma unroll
        for (uint32_t i = 0; i < B; ++i) {
            const uint32_t k = j < NB ? kSteps - 1 - B * j - i : 0u;
            const uint32_t o = 2u * ((tok0 + 2u * k) * C + ch);               // byte offset of the step's element
            ic[i] = at(cbase, o);
            ig[i] = at(gbase, o);
            if constexpr (PASS) {
                il[i] = at(cbase, o - 2u * C);
                ir[i] = at(cbase, last_blk && k == kSteps - 1 ? o - 2u * C : o + 2u * C);
            }
        }
    };
    uint32_t x = kStateLow, cnt = 0, ecnt = 0, wdone = 0, edone = 0;
    load_batch(0);
    for (uint32_t j = 0; j < NB; ++j) {
        // symbols and table entries of batch j
        uint32_t zs[B];                                    // symbol | shift << 16
        uint2 ge[B];                                       // device-memory entry (symbols past the LDS head)
#pragma unroll
        for (uint32_t i = 0; i < B; ++i) {
            int32_t mu = ig[i];
            if constexpr (PASS) mu += 8 * (il[i] + ir[i]);
            const int32_t kk = mu >> 4;
            const uint32_t sh = uint32_t(mu & 15);
            const uint32_t z = zig16(uint32_t(ic[i] - kk) & 0xFFFFu);
            zs[i] = z | (sh << 16);
            // entries past the table's n repeat its escape entry, flagged in bit 30
            const uint32_t eo = z < kCbEncHead ? 0u : 8u * ((ch * 16u + sh) * 256u + min(z, 255u));
            ge[i] = *reinterpret_cast<const uint2*>(tbase + eo);
        }
        load_batch(j + 1);
#pragma unroll
        for (uint32_t i = 0; i < B; ++i) {
            const uint32_t z = zs[i] & 0xFFFFu, sh = zs[i] >> 16;
            const uint2 le = lhead[sh * kCbEncHead + min(z, kCbEncHead - 1)];
            const uint2 e = z < kCbEncHead ? le : ge[i];
            // escaped values keep decode order: ranked like the words, written backwards
            const bool esc = (e.y & 0x40000000u) != 0;
            const uint32_t me = uint32_t(__ballot(esc) >> half);
            if (esc) {
                const uint32_t pos = ecnt + __popc(uint32_t(uint64_t(me) >> (lane + 1)));
                if (pos - edone < kCbEncEsc) ering[pos % kCbEncEsc] = uint16_t(z);
                else if (pos < MAXE) efwd[pos] = uint16_t(z);
            }
            ecnt += __popc(me);
            // the state update
            const uint32_t m = e.x, w = e.y;
            const uint32_t f = w & 0xFFFu;
            const bool emit = x >= (f << 20);
            const uint32_t mw = uint32_t(__ballot(emit) >> half);
            if (emit) {
                const uint32_t pos = cnt + __popc(uint32_t(uint64_t(mw) >> (lane + 1)));
                wring[pos % kCbEncRing] = uint16_t(x & 0xFFFFu);
                x >>= 16;
            }
            cnt += __popc(mw);
            const uint32_t qt = __umulhi(x + __builtin_amdgcn_ubfe(w, 29, 1), m) >>
                                __builtin_amdgcn_ubfe(w, 24, 5);                    // floor(x / f)
            x = x + __builtin_amdgcn_ubfe(w, 12, 12) + qt * (kM - f);
        }
        // the batch's words and escaped values out to the workspace (the lanes of this stream wrote
        // them; LDS operations of one wavefront complete in order)
        for (uint32_t i = wdone + lane; i < min(cnt, MAXW); i += kLanes) wfwd[i] = wring[i % kCbEncRing];
        wdone = cnt;
        const uint32_t eend = min(min(ecnt, edone + kCbEncEsc), MAXE);
        for (uint32_t i = edone + lane; i < eend; i += kLanes) efwd[i] = ering[i % kCbEncEsc];
        edone = ecnt;
    }
    reinterpret_cast<uint32_t*>(area)[lane] = x;
    if (lane == 0) {
        const uint32_t bytes = (kStreamHead + 2 * cnt + 2 * ecnt + 3) & ~3u;
        a.meta[sid] = bytes >= RAW ? 0x80000000u : (cnt | (ecnt << 14));
    }
}

__global__ __launch_bounds__(kCbEncStreams * 32) void encode_cb(EncodeLaunch a, DevTables t) {
    __shared__ uint2 ehead[kLanes * kCbEncLane];            // [lane][shift][symbol 0..11]
    __shared__ uint16_t wring[kCbEncStreams * kCbEncRing];  // [stream][word position mod kCbEncRing]
    __shared__ uint16_t ering[kCbEncStreams * kCbEncEsc];   // [stream][escape position mod kCbEncEsc]
    const uint32_t tid = threadIdx.x;
    const Geo g = geometry(a.shape);
    const uint64_t per = uint64_t(g.ncg) * g.ntb;            // streams per pass
    {
        const uint32_t bcg = cb_group<kCbEncStreams>(g);
        if (bcg >= g.ncg) return;                              // the whole block
        for (uint32_t i = tid; i < kLanes * 16 * kCbEncHead; i += blockDim.x) {
            const uint32_t j = i / kCbEncHead, z = i % kCbEncHead;     // j = lane * 16 + shift
            ehead[(j / 16) * kCbEncLane + (j % 16) * kCbEncHead + z] =
                t.enc8[(size_t(bcg) * (kLanes * 16) + j) * 256 + z];
        }
        __syncthreads();
    }
    uint64_t sid;
    if (!cb_stream<kCbEncStreams>(g, uint64_t(blockIdx.y) * per, sid)) return;
    // blockIdx.y is the pass: every stream of the block is of that pass
    uint16_t* wr = wring + (tid >> 5) * kCbEncRing;
    uint16_t* er = ering + (tid >> 5) * kCbEncEsc;
    if (blockIdx.y) encode_cb_stream<true>(a, t, g, sid, ehead, wr, er);
    else encode_cb_stream<false>(a, t, g, sid, ehead, wr, er);
}

// --------------------------------------------------------------- index + compaction
// meta word of a stream: bit 31 = stored raw; else rANS word count in bits
// 0..13 and escaped-value count in bits 14..27.
__device__ __forceinline__ uint32_t meta_bytes(uint32_t m, uint32_t raw) {
    const uint32_t eb = raw / kSyms;
    return (m >> 31) ? raw : (kStreamHead + 2 * (m & 0x3FFFu) + eb * ((m >> 14) & 0x3FFFu) + 3) & ~3u;
}

__global__ __launch_bounds__(kScanBlock) void stream_block_sums(const uint32_t* meta, uint64_t n, uint32_t raw,
                                                               uint32_t* bsum) {
    __shared__ uint32_t part[kScanBlock / 64];
    const uint64_t i = uint64_t(blockIdx.x) * kScanBlock + threadIdx.x;
    uint32_t v = i < n ? meta_bytes(meta[i], raw) : 0u;
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (uint32_t w = 0; w < kScanBlock / 64; ++w) s += part[w];
        bsum[blockIdx.x] = s;
    }
}

// Exclusive scan of the block sums by one workgroup, a kScanBlock run at a
// time, starting from *base (the payload before this chunk of streams; null: 0).
__global__ __launch_bounds__(kScanBlock) void stream_block_scan(const uint32_t* bsum, uint32_t nb, uint64_t* boff,
                                                               uint64_t* total, const uint64_t* base0) {
    __shared__ uint64_t wsum[kScanBlock / 64];
    __shared__ uint64_t carry;
    if (threadIdx.x == 0) carry = base0 ? *base0 : 0ull;
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    for (uint32_t base = 0; base < nb; base += kScanBlock) {
        const uint32_t i = base + threadIdx.x;
        const uint64_t v = i < nb ? uint64_t(bsum[i]) : 0ull;
        uint64_t incl = v;
        for (uint32_t d = 1; d < 64; d <<= 1) {
            const uint64_t o = __shfl_up(incl, d, 64);
            if (lane >= d) incl += o;
        }
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        uint64_t before = carry;
        for (uint32_t q = 0; q < w; ++q) before += wsum[q];
        if (i < nb) boff[i] = before + incl - v;
        __syncthreads();
        if (threadIdx.x == kScanBlock - 1) carry = before + incl;
        __syncthreads();
    }
    if (threadIdx.x == 0) *total = carry;
}

template <uint32_t DT, uint32_t MODE>
__global__ __launch_bounds__(kScanBlock) void place_streams(EncodeLaunch a, const uint64_t* boff) {
    __shared__ uint32_t wsum[kScanBlock / 64];
    constexpr uint32_t EB = DT == SKV_E4M3 ? 1u : 2u;
    constexpr uint32_t RAW = kSyms * EB;
    const uint64_t n = a.n_streams, N = a.n_total;
    const uint64_t head = kHeaderBytes + 8 * (N + 1);
    const uint64_t total = *a.total;
    if (head + total > a.out_capacity) return;        // caller reports SKV_ERR_CAPACITY
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint64_t first = uint64_t(blockIdx.x) * kScanBlock;
    const uint64_t i = first + threadIdx.x;
    const uint32_t m = i < n ? a.meta[i] : 0u;
    const uint32_t v = i < n ? meta_bytes(m, RAW) : 0u;
    uint32_t incl = v;
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    uint64_t off = boff[blockIdx.x];
    for (uint32_t q = 0; q < w; ++q) off += wsum[q];
    off += incl - v;
    uint64_t* index = reinterpret_cast<uint64_t*>(a.out + kHeaderBytes) + a.sid_base;
    if (i < n) index[i] = off | (uint64_t(m >> 31) << 63);
    if (a.last && i == n - 1) index[n] = total;
    if (a.last && i == 0) {
        uint8_t* h = a.out;
        const skv_shape& cs = a.container;
        const uint32_t words[16] = {
            0x31564B53u,                                                    // "SKV1"
            1u | (cs.dtype << 16) | (cs.mode << 24),
            kProbBits | (uint32_t(kLanes) << 8) | (uint32_t(kSteps) << 16),
            cs.layers, cs.kv, cs.tokens, cs.channels, 0u,
            uint32_t(N), uint32_t(N >> 32),
            uint32_t(a.blob_hash), uint32_t(a.blob_hash >> 32),
            uint32_t(total), uint32_t(total >> 32), 0u, 0u};
        for (int q = 0; q < 16; ++q) reinterpret_cast<uint32_t*>(h)[q] = words[q];
    }
}

// One wavefront per stream: copy its bytes from the scratch area to its place
// in the container (states, word count, words and escaped values reversed from
// emission into decode order, zero pad; raw streams gather the target tile).
// Words move a dword at a time: with an even word count, container dword j is
// scratch dword cnt/2 - 1 - j with its halves swapped; with an odd count it
// takes the low half of one scratch dword and the high half of the one below.
template <uint32_t DT, uint32_t MODE>
__global__ __launch_bounds__(256) void copy_streams(EncodeLaunch a) {
    constexpr uint32_t EB = DT == SKV_E4M3 ? 1u : 2u;
    constexpr uint32_t RAW = kSyms * EB;
    const uint64_t n = a.n_streams;
    const uint64_t sid = uint64_t(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (sid >= n) return;
    const uint64_t head = kHeaderBytes + 8 * (a.n_total + 1);
    if (head + *a.total > a.out_capacity) return;        // caller reports SKV_ERR_CAPACITY
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t* index = reinterpret_cast<const uint64_t*>(a.out + kHeaderBytes) + a.sid_base;
    uint8_t* dst = a.out + head + (index[sid] & ~kRawBit);
    const uint32_t ms = a.meta[sid];
    const uint8_t* src = a.scratch + sid * (2 * RAW);
    if (ms >> 31) {
        // raw stream: 128 rows of 32 channels from the target, 16 bytes per lane per pass
        const Geo g = geometry(a.shape);
        const uint32_t cg = uint32_t(sid % g.ncg);
        const uint32_t tb = uint32_t((sid / g.ncg) % g.ntb);
        const uint32_t slab = uint32_t(sid / (uint64_t(g.ncg) * g.ntb));
        constexpr uint32_t PER_ROW = kLanes * EB / 16;          // 16-byte pieces per row segment
        for (uint32_t e = lane; e < kSteps * PER_ROW; e += 64) {
            const uint32_t k = e / PER_ROW, piece = e % PER_ROW;
            const uint32_t tok = MODE != SKV_CHECKERBOARD ? tb * kSteps + k : 2u * (tb * kSteps + k) + slab;
            const size_t idx = MODE != SKV_CHECKERBOARD ? (size_t(slab) * g.T + tok) * g.C + cg * kLanes
                                                    : size_t(tok) * g.C + cg * kLanes;
            const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.target) + idx * EB + piece * 16);
            *reinterpret_cast<uint4*>(dst + e * 16) = v;
        }
        return;
    }
    const uint32_t cnt = ms & 0x3FFFu, ecnt = (ms >> 14) & 0x3FFFu;
    const uint32_t used = kStreamHead + 2 * cnt + EB * ecnt;
    const uint32_t total = (used + 3) & ~3u;
    // range-checked views of the stream's scratch and its container bytes: an access at
    // kOut is dropped (loads return 0), so no load or store below needs a branch
    constexpr uint32_t kOut = 0x80000000u;
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), (short)0, int(2 * RAW), 0x00020000);
    const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, int(total), 0x00020000);
    const uint32_t nd = cnt / 2;                              // container dwords holding two words
    const bool odd = (cnt & 1u) != 0;
    // one batch of container word dwords [j0, j0 + 256): even count, scratch dword nd - 1 - j
    // with its halves swapped; odd count, the low half of scratch dword (cnt - 1) / 2 - j and
    // the high half of the one below.  All loads are issued before the stores.
    constexpr uint32_t B = 4;
    auto words = [&](uint32_t j0, uint32_t (&wa)[B], uint32_t (&wb)[B]) {
#pragma unroll
        for (uint32_t k = 0; k < B; ++k) {
            const uint32_t j = j0 + lane + 64 * k;
            const uint32_t e = odd ? (cnt - 1) / 2 - j : nd - 1 - j;
            wa[k] = __builtin_amdgcn_raw_buffer_load_b32(srs, j < nd ? RAW + 4 * e : kOut, 0, 0);
            wb[k] = __builtin_amdgcn_raw_buffer_load_b32(srs, j < nd && odd ? RAW + 4 * e - 4 : kOut, 0, 0);
        }
    };
    auto put_words = [&](uint32_t j0, const uint32_t (&wa)[B], const uint32_t (&wb)[B]) {
#pragma unroll
        for (uint32_t k = 0; k < B; ++k) {
            const uint32_t j = j0 + lane + 64 * k;
            const uint32_t v = odd ? (wa[k] & 0xFFFFu) | (wb[k] & 0xFFFF0000u) : __builtin_amdgcn_alignbit(wa[k], wa[k], 16);
            __builtin_amdgcn_raw_buffer_store_b32(v, drs, j < nd ? kStreamHead + 4 * j : kOut, 0, 0);
        }
    };
    // escaped values [q0, q0 + 64), reversed
    auto esc_at = [&](uint32_t q0) {
        const uint32_t q = q0 + lane;
        const uint32_t o = q < ecnt ? kStreamHead + EB * (ecnt - 1 - q) : kOut;
        return EB == 1 ? uint32_t(__builtin_amdgcn_raw_buffer_load_b8(srs, o, 0, 0))
                       : uint32_t(__builtin_amdgcn_raw_buffer_load_b16(srs, o, 0, 0));
    };
    auto put_esc = [&](uint32_t q0, uint32_t v) {
        const uint32_t q = q0 + lane;
        const uint32_t o = q < ecnt ? kStreamHead + 2 * cnt + EB * q : kOut;
        if (EB == 1) __builtin_amdgcn_raw_buffer_store_b8(uint8_t(v), drs, o, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b16(uint16_t(v), drs, o, 0, 0);
    };
    const uint32_t hv = __builtin_amdgcn_raw_buffer_load_b32(srs, lane < 32 ? 4 * lane : kOut, 0, 0);
    const uint32_t w0 = __builtin_amdgcn_raw_buffer_load_b32(srs, RAW, 0, 0);     // scratch word 0 (low half)
    uint32_t wa[B], wb[B];
    words(0, wa, wb);
    const uint32_t ev = esc_at(0);
    // states and count, words, the lone last word of an odd count, escaped values, zero pad
    __builtin_amdgcn_raw_buffer_store_b32(lane == 32 ? cnt : hv, drs, lane <= 32 ? 4 * lane : kOut, 0, 0);
    put_words(0, wa, wb);
    __builtin_amdgcn_raw_buffer_store_b16(uint16_t(w0), drs, odd && lane == 0 ? kStreamHead + 2 * (cnt - 1) : kOut, 0, 0);
    put_esc(0, ev);
    __builtin_amdgcn_raw_buffer_store_b8(uint8_t(0), drs, used + lane < total ? used + lane : kOut, 0, 0);
    // long streams: further batches
    for (uint32_t j0 = 64 * B; j0 < nd; j0 += 64 * B) {
        words(j0, wa, wb);
        put_words(j0, wa, wb);
    }
    for (uint32_t q0 = 64; q0 < ecnt; q0 += 64) put_esc(q0, esc_at(q0));
}

// --------------------------------------------------------------- decode
__device__ __forceinline__ void refill(uint32_t& x, uint32_t& p, bool need, uint32_t lane, uint32_t half,
                                       const uint16_t* W, uint32_t navail, bool& bad) {
    const uint64_t b = __ballot(need);
    const uint32_t mine = uint32_t(b >> half);
    if (need) {
        const uint32_t pos = p + __popc(mine & ((1u << lane) - 1u));
        uint32_t w = 0;
        if (pos < navail) w = W[pos];
        else bad = true;
        x = (x << 16) | w;
    }
    p += __popc(mine);
}

// Index position of stream (slab, tb, cg) of a decode.  The container numbers
// its streams over its own token blocks (ntb_index per slab); a range decode
// covers token blocks tb_base onwards of every slab, numbered from 0 here.
__device__ __forceinline__ uint64_t index_pos(const DecodeLaunch& a, uint32_t slab, uint32_t tb, uint32_t cg,
                                              uint32_t ncg) {
    return (uint64_t(slab) * a.ntb_index + a.tb_base + tb) * ncg + cg;
}

template <uint32_t DT, uint32_t MODE>
__global__ __launch_bounds__(256) void decode_streams(DecodeLaunch a, DevTables t, uint64_t first, uint64_t count) {
    const uint32_t tid = threadIdx.x;
    const uint64_t local = uint64_t(blockIdx.x) * kStreamsPerBlock + (tid >> 5);
    if (local >= count) return;
    const uint64_t sid = first + local;
    const uint32_t lane = tid & 31u, half = tid & 32u;
    const Geo g = geometry(a.shape);
    const uint32_t cg = uint32_t(sid % g.ncg);
    const uint32_t tb = uint32_t((sid / g.ncg) % g.ntb);
    const uint32_t slab = uint32_t(sid / (uint64_t(g.ncg) * g.ntb));
    const uint32_t ch = cg * kLanes + lane;
    constexpr uint32_t EB = DT == SKV_E4M3 ? 1u : 2u;
    constexpr uint32_t RAW = kSyms * EB;
    const uint64_t* index = a.index;
    const uint8_t* pay = a.pay;
    const uint64_t ip = MODE != SKV_CHECKERBOARD ? index_pos(a, slab, tb, cg, g.ncg) : sid;
    const uint64_t e0 = index[ip], e1 = index[ip + 1];
    const uint64_t off = e0 & ~kRawBit, end = e1 & ~kRawBit;
    bool bad = false;
    if (end < off || end > a.payload_bytes) {
        if (lane == 0) atomicOr(a.status, 1u);
        return;
    }
    const uint64_t size = end - off;
    auto out_index = [&](uint32_t k) -> size_t {
        if (MODE != SKV_CHECKERBOARD) return (size_t(slab) * g.T + size_t(tb) * kSteps + k) * g.C + ch;
        return size_t(2u * (tb * kSteps + k) + slab) * g.C + ch;
    };
    if (e0 & kRawBit) {
        if (size != RAW) {
            if (lane == 0) atomicOr(a.status, 1u);
            return;
        }
        for (uint32_t k = 0; k < uint32_t(kSteps); ++k) {
            if (EB == 1) static_cast<uint8_t*>(a.out)[out_index(k)] = pay[off + k * kLanes + lane];
            else static_cast<uint16_t*>(a.out)[out_index(k)] =
                reinterpret_cast<const uint16_t*>(pay + off)[k * kLanes + lane];
        }
        return;
    }
    const uint8_t* sp = pay + off;
    if (size < kStreamHead || size % 4 != 0) {
        if (lane == 0) atomicOr(a.status, 1u);
        return;
    }
    const uint32_t nw = reinterpret_cast<const uint32_t*>(sp)[32];
    if (nw > (size - kStreamHead) / 2) {
        if (lane == 0) atomicOr(a.status, 1u);
        return;
    }
    uint32_t x = reinterpret_cast<const uint32_t*>(sp)[lane];
    if (x < kStateLow) bad = true;
    const uint16_t* W = reinterpret_cast<const uint16_t*>(sp + kStreamHead);
    const uint8_t* E = sp + kStreamHead + 2 * nw;
    const uint32_t ecap = uint32_t((size - kStreamHead - 2 * nw) / EB);
    uint32_t p = 0, ep = 0;
    const uint32_t res_table = slab * g.C + ch;
    for (uint32_t k = 0; k < uint32_t(kSteps); ++k) {
        const size_t oi = out_index(k);
        uint32_t table;
        int32_t kk = 0;
        if (MODE == SKV_RESIDUAL) {
            table = res_table;
        } else if (MODE == SKV_RESIDUAL_EXP) {
            const uint32_t pv = DT == SKV_E4M3 ? uint32_t(static_cast<const uint8_t*>(a.aux)[oi])
                                               : uint32_t(static_cast<const uint16_t*>(a.aux)[oi]);
            table = slab * kExpClasses + exp_class(pv, DT, t.base[slab]);
        } else {
            const uint32_t tok = 2u * (tb * kSteps + k) + slab;
            const int16_t* dec = static_cast<const int16_t*>(a.out);
            // the odd pass's side input may be the output's odd rows (mapped in place): read before the store
            int32_t mu = static_cast<const int16_t*>(slab ? a.aux_odd : a.aux)[oi];
            if (slab == 1) {
                const int32_t l = dec[size_t(tok - 1) * g.C + ch];
                const int32_t r = (tok + 1 < g.T) ? int32_t(dec[size_t(tok + 1) * g.C + ch]) : l;
                mu += 8 * (l + r);
            }
            kk = mu >> 4;
            table = ch * 16u + uint32_t(mu & 15);
        }
        const uint32_t n = t.n[table];
        const uint32_t slot = x & (kM - 1u);
        const uint32_t s = t.slot[size_t(table) * kM + slot];
        const uint32_t fcv = t.fc[size_t(table) * 256 + s];
        x = (fcv & 0x0FFFu) * (x >> kProbBits) + slot - (fcv >> 16);
        refill(x, p, x < kStateLow, lane, half, W, nw, bad);
        const bool esc = s == n;
        uint32_t z = s;
        {
            const uint64_t b = __ballot(esc);
            const uint32_t mine = uint32_t(b >> half);
            if (esc) {
                const uint32_t pos = ep + __popc(mine & ((1u << lane) - 1u));
                uint32_t v = 0;
                if (pos < ecap) v = EB == 1 ? uint32_t(E[pos]) : uint32_t(reinterpret_cast<const uint16_t*>(E)[pos]);
                else bad = true;
                if (v < n) bad = true;
                z = v;
            }
            ep += __popc(mine);
        }
        if (MODE != SKV_CHECKERBOARD) {
            if (DT == SKV_E4M3) {
                const uint32_t pv = static_cast<const uint8_t*>(a.aux)[oi];
                static_cast<uint8_t*>(a.out)[oi] = uint8_t(unord8((ord8(pv) + unzig(z)) & 0xFFu));
            } else {
                const uint32_t pv = static_cast<const uint16_t*>(a.aux)[oi];
                static_cast<uint16_t*>(a.out)[oi] = uint16_t(unord16((ord16(pv) + unzig(z)) & 0xFFFFu));
            }
        } else {
            static_cast<int16_t*>(a.out)[oi] = int16_t(uint16_t(uint32_t(kk) + unzig(z)));
        }
    }
    if (x != kStateLow || p != nw) bad = true;
    const uint32_t used = kStreamHead + 2 * nw + EB * ep;
    if (((used + 3) & ~3u) != size) bad = true;
    else if (lane < size - used && sp[used + lane] != 0) bad = true;   // zero pad
    if (bad) atomicOr(a.status, 1u);
}

// Checkerboard decoder.  A step's side input and decoded neighbours (and from
// them its table and mean) do not depend on the rANS state; its table lookup
// does.  The block's streams share one channel group, whose 32 x 16 tables
// the block reads throughout: the starts of each table's first 32 symbols
// (and of the 33rd) sit in LDS, so a slot below the 33rd start finds its
// symbol by binary search there (start and frequency from neighbouring
// starts); the other slots read one entry (symbol, frequency, start) of the
// table's tail map in device memory, requested before the search so that the
// two overlap.  Loads and stores share one counter, and a wait for a load is
// also a wait for every load issued before it (and for every store), so a
// lookup in device memory waits for whatever else is in flight.  The steps
// therefore run in batches of 8 with nothing else in flight inside a batch:
//   * the side inputs and neighbours of batch j + 1 are loaded, and batch j's
//     outputs stored, between the two batches;
//   * words come from a 384-word ring of the stream in LDS, escaped values
//     from a 128-value ring; both are refilled between batches (128-word
//     chunks, one or two, and 64 values at a time) so that a batch never runs
//     out of words and rarely of escaped values (past the ring, a value is
//     read from device memory);
//   * each table's direct-symbol count, for the escape check, sits in LDS.
// The block's LDS (53 KB) and registers (at most 80) leave room for three
// blocks per CU.  Output and checks are those of decode_streams.
// RANGE: token blocks tb_base onwards of the container (the shape is the
// range's, rows are numbered from its start), and the range's last odd token
// takes its right neighbour from next_rows when the range stops early.
constexpr uint32_t kCbDecStreams = 16;                   // streams (half-waves) per block
constexpr uint32_t kCbHeadRow = kCbHead + 1;
// a lane's 16 rows take an odd number of dwords, so lanes start on different banks
constexpr uint32_t kCbHeadLane = 16 * kCbHeadRow + 2;
constexpr uint32_t kCbDecBatch = 8;                      // steps per batch
constexpr uint32_t kCbWordRing = 384, kCbWordChunk = 128;   // words per stream ring / per refill
constexpr uint32_t kCbEscRing = 128, kCbEscChunk = 64;      // escaped values per stream ring / per refill

template <bool PASS, bool RANGE>
__device__ __forceinline__ void decode_cb_stream(const DecodeLaunch& a, const DevTables& t, const Geo& g,
                                                 uint64_t sid, const uint16_t* head, const uint16_t* nlds,
                                                 const uint32_t* tbase, uint32_t* wring, uint32_t* ering) {
    constexpr uint32_t RAW = 2 * kSyms;
    constexpr uint32_t B = kCbDecBatch, NB = kSteps / kCbDecBatch;
    const uint32_t lane = threadIdx.x & 31u, half = threadIdx.x & 32u;
    const uint32_t cg = uint32_t(sid % g.ncg);
    const uint32_t tb = uint32_t((sid / g.ncg) % g.ntb);
    const uint32_t ch = cg * kLanes + lane;
    const uint32_t C = g.C;
    const uint64_t xid = RANGE ? index_pos(a, PASS ? 1u : 0u, tb, cg, g.ncg) : sid;
    const uint64_t e0 = a.index[xid], e1 = a.index[xid + 1];
    const uint64_t off = e0 & ~kRawBit, end = e1 & ~kRawBit;
    int16_t* out = static_cast<int16_t*>(a.out);
    // rows are addressed from the block's first row (uniform) with 32-bit element offsets: a block's
    // 16 token blocks span 4096 rows (plus the row after them)
    const uint32_t tb0 = __builtin_amdgcn_readfirstlane(tb & ~(kCbDecStreams - 1u));
    const size_t row0 = size_t(2u * tb0 * kSteps) * C;
    int16_t* obase = out + row0;
    // the odd pass's side input may be the output's odd rows (mapped in place): a lane loads each
    // element's side input in the batch before the one that stores the element
    const int16_t* gbase = static_cast<const int16_t*>(PASS ? a.aux_odd : a.aux) + row0;
    const uint32_t tok0 = 2u * (tb - tb0) * kSteps;          // the stream's first even row, from row0
    auto row_off = [&](uint32_t k) { return (tok0 + 2u * k + (PASS ? 1u : 0u)) * C + ch; };
    if (end < off || end > a.payload_bytes) {
        if (lane == 0) atomicOr(a.status, 1u);
        return;
    }
    const uint64_t size = end - off;
    if (e0 & kRawBit) {
        if (size != RAW) {
            if (lane == 0) atomicOr(a.status, 1u);
            return;
        }
        // a raw stream: its 4096 values in (step, lane) order, 16 steps loaded before any is stored
        const int16_t* rv = reinterpret_cast<const int16_t*>(a.pay + off);
        for (uint32_t k0 = 0; k0 < uint32_t(kSteps); k0 += 16) {
            int16_t v[16];
#pragma unroll
            for (uint32_t i = 0; i < 16; ++i) v[i] = rv[(k0 + i) * kLanes + lane];
#pragma unroll
            for (uint32_t i = 0; i < 16; ++i) obase[row_off(k0 + i)] = v[i];
        }
        return;
    }
    const uint8_t* sp = a.pay + off;
    if (size < kStreamHead || size % 4 != 0) {
        if (lane == 0) atomicOr(a.status, 1u);
        return;
    }
    const uint32_t nw = reinterpret_cast<const uint32_t*>(sp)[32];
    if (nw > (size - kStreamHead) / 2) {
        if (lane == 0) atomicOr(a.status, 1u);
        return;
    }
    bool bad = false;
    uint32_t x = reinterpret_cast<const uint32_t*>(sp)[lane];
    if (x < kStateLow) bad = true;
    const uint32_t body = uint32_t(size) - kStreamHead;       // bytes of words, escaped values and pad
    const uint32_t ebase = kStreamHead + 2 * nw;              // byte offset of the escaped values
    const uint32_t ecap = (body - 2 * nw) / 2;
    const uint32_t below = (1u << lane) - 1u;
    const uint16_t* wr16 = reinterpret_cast<const uint16_t*>(wring);
    const uint16_t* er16 = reinterpret_cast<const uint16_t*>(ering);

    // ring refills: every load is in bounds of the stream (a lane past it reads the stream's first
    // dword and keeps 0); words past the count are never used by a valid stream
    // a batch consumes at most 256 words; between batches one or two 128-word chunks come in
    uint32_t wc[4], ec;
    auto load_words = [&](uint32_t c, uint32_t r) {         // words 128 c .. 128 c + 127: dword q * 32 + lane in wc[2 r + q]
#pragma unroll
        for (uint32_t q = 0; q < 2; ++q) {
            const uint32_t bo = 4u * (kCbWordChunk / 2 * c + q * kLanes + lane);
            const bool in = bo + 4 <= body;
            const uint32_t v = *reinterpret_cast<const uint32_t*>(sp + (in ? kStreamHead + bo : 0u));
            wc[2 * r + q] = in ? v : 0u;
        }
    };
    auto write_words = [&](uint32_t c, uint32_t r) {
#pragma unroll
        for (uint32_t q = 0; q < 2; ++q)
            wring[(kCbWordChunk / 2 * c + q * kLanes + lane) % (kCbWordRing / 2)] = wc[2 * r + q];
    };
    auto load_esc = [&](uint32_t c) {                       // escaped values 64 c + 2 lane, + 1 in ec
        const uint32_t i0 = kCbEscChunk * c + 2 * lane;
        const bool in0 = i0 < ecap, in1 = i0 + 1 < ecap;
        const uint32_t v0 = *reinterpret_cast<const uint16_t*>(sp + (in0 ? ebase + 2 * i0 : 0u));
        const uint32_t v1 = *reinterpret_cast<const uint16_t*>(sp + (in1 ? ebase + 2 * i0 + 2 : 0u));
        ec = (in0 ? v0 : 0u) | ((in1 ? v1 : 0u) << 16);
    };
    auto write_esc = [&](uint32_t c) { ering[(kCbEscChunk / 2 * c + lane) % (kCbEscRing / 2)] = ec; };
    // side inputs (and the even neighbours) of batch j; j = NB reloads batch 0 (unused)
    int32_t gin[B], ev[B + 1];
    auto load_inputs = [&](uint32_t j) {
        const uint32_t k0 = j < NB ? B * j : 0u;
#pragma unroll
        for (uint32_t i = 0; i < B; ++i) gin[i] = gbase[row_off(k0 + i)];
        if constexpr (PASS) {
#pragma unroll
            for (uint32_t i = 0; i <= B; ++i) {
                // even row left of odd step k0 + i; the last one is the right neighbour of step k0 + 7
                const uint32_t eo = (tok0 + 2u * (k0 + i)) * C + ch;
                if (i < B) {
                    ev[i] = obase[eo];
                } else {
                    const bool past = 2u * (tb * kSteps + k0 + i) >= g.T;   // the row after the cache
                    const int16_t* src = obase + (past ? eo - 2u * C : eo);
                    if constexpr (RANGE)
                        if (past && a.next_rows) src = a.next_rows + ch;
                    ev[i] = *src;
                }
            }
        }
    };

    uint32_t p = 0, ep = 0;                                  // words and escaped values consumed
    uint32_t wl = 2 * kCbWordChunk, el = 2 * kCbEscChunk;    // loaded (next chunk to load at wl, el)
    uint32_t elw = el;                                       // escaped values in the ring
    load_words(0, 0);
    load_words(1, 1);
    write_words(0, 0);
    write_words(1, 1);
    load_esc(0);
    write_esc(0);
    load_esc(1);
    write_esc(1);
    load_inputs(0);
    uint32_t wpend = 0;                                      // chunks loaded after the last batch (0..2)
    bool epend = false;
    for (uint32_t j = 0; j < NB; ++j) {
        if (wpend == 2) {
            write_words(wl / kCbWordChunk - 2, 0);
            write_words(wl / kCbWordChunk - 1, 1);
        } else if (wpend == 1) {
            write_words(wl / kCbWordChunk - 1, 0);
        }
        if (epend) write_esc(el / kCbEscChunk - 1);
        elw = el;
        uint32_t o[B / 2];                                   // outputs, two per register
#pragma unroll
        for (uint32_t i = 0; i < B; ++i) {
            int32_t mu = gin[i];
            if constexpr (PASS) mu += 8 * (ev[i] + ev[i + 1]);
            const int32_t kk = mu >> 4;
            const uint32_t table = ch * 16u + uint32_t(mu & 15);
            const uint32_t slot = x & (kM - 1u);
            const uint32_t sh = table & 15u;
            const uint32_t hb = lane * kCbHeadLane + sh * kCbHeadRow;
            const uint32_t ts = head[hb + kCbHead];
            const bool hit = slot < ts;
            // slots past the LDS head: one read of the table's tail map, issued before the binary
            // search so that the two overlap
            uint32_t te = 0;
            if (!hit) te = t.tail[tbase[lane * 16u + sh] + (slot - ts)];
            // symbols 0..31: binary search of the starts in LDS
            uint32_t zc = 0;
#pragma unroll
            for (uint32_t step = kCbHead / 2; step; step >>= 1) zc += head[hb + zc + step] <= slot ? step : 0u;
            const uint32_t c0 = head[hb + zc], c1 = head[hb + zc + 1];
            const uint32_t fq = hit ? c1 - c0 : (te >> 8) & 0x0FFFu;
            const uint32_t cs = hit ? c0 : te >> 20;
            const uint32_t s = hit ? zc : te & 255u;
            x = fq * (x >> kProbBits) + slot - cs;
            // refill in lane order from the word ring
            const bool need = x < kStateLow;
            const uint32_t mine = uint32_t(__ballot(need) >> half);
            if (need) {
                const uint32_t wi = p + __popc(mine & below);
                if (wi >= nw) bad = true;
                x = (x << 16) | uint32_t(wr16[wi % kCbWordRing]);
            }
            p += __popc(mine);
            // escaped values, in lane order, from the escape ring (past it, from device memory)
            const bool esc = !hit && (te & 255u) == 255u;
            const uint32_t me = uint32_t(__ballot(esc) >> half);
            uint32_t z = s;
            if (esc) {
                const uint32_t pos = ep + __popc(me & below);
                uint32_t v = 0;
                if (pos >= ecap) bad = true;
                else if (pos < elw) v = er16[pos % kCbEscRing];
                else v = *reinterpret_cast<const uint16_t*>(sp + ebase + 2 * pos);
                if (v < nlds[lane * 16u + sh]) bad = true;   // a canonical encoder codes such a value directly
                z = v;
            }
            ep += __popc(me);
            const uint32_t ov = (uint32_t(kk) + unzig(z)) & 0xFFFFu;
            o[i / 2] = i % 2 ? o[i / 2] | (ov << 16) : ov;
        }
        // between batches: this batch's outputs, the next batch's inputs, the rings' next chunks
#pragma unroll
        for (uint32_t i = 0; i < B; ++i) obase[row_off(B * j + i)] = int16_t(uint16_t(o[i / 2] >> (16 * (i % 2))));
        load_inputs(j + 1);
        // words [p, p + 256) must be in the ring at the next batch's start; a chunk overwrites the
        // words 384 before it, which are consumed once wl < p + 256
        wpend = 0;
        if (wl < p + 2 * kCbWordChunk) {
            load_words(wl / kCbWordChunk, 0);
            wl += kCbWordChunk;
            wpend = 1;
            if (wl < p + 2 * kCbWordChunk) {
                load_words(wl / kCbWordChunk, 1);
                wl += kCbWordChunk;
                wpend = 2;
            }
        }
        epend = el <= ep + kCbEscChunk;
        if (epend) {
            load_esc(el / kCbEscChunk);
            el += kCbEscChunk;
        }
    }
    if (x != kStateLow || p != nw) bad = true;
    const uint32_t used = kStreamHead + 2 * nw + 2 * ep;
    if (((used + 3) & ~3u) != size) bad = true;
    else if (lane < size - used && sp[used + lane] != 0) bad = true;   // zero pad
    if (bad) atomicOr(a.status, 1u);
}

template <bool RANGE = false>
__global__ __launch_bounds__(kCbDecStreams * 32) __attribute__((amdgpu_waves_per_eu(6))) void decode_cb(DecodeLaunch a, DevTables t, uint64_t first,
                                                               uint64_t count) {
    __shared__ uint16_t head[kLanes * kCbHeadLane];                     // [lane][shift][symbol 0..32] starts
    __shared__ uint16_t nlds[kLanes * 16];                              // [lane][shift] direct symbols
    __shared__ uint32_t tbase[kLanes * 16];                             // [lane][shift] first tail-map entry
    __shared__ uint32_t wring[kCbDecStreams * kCbWordRing / 2];         // [stream][word pair mod 256]
    __shared__ uint32_t ering[kCbDecStreams * kCbEscRing / 2];          // [stream][escape pair mod 64]
    const uint32_t tid = threadIdx.x;
    const Geo g = geometry(a.shape);
    {
        const uint32_t bcg = cb_group<kCbDecStreams>(g);
        if (bcg >= g.ncg) return;                              // the whole block
        // starts of symbols 0..32 of each table, those past a table's escape symbol repeating its start
        for (uint32_t i = tid; i < kLanes * 16 * kCbHeadRow; i += blockDim.x) {
            const uint32_t j = i / kCbHeadRow, z = i % kCbHeadRow;     // j = lane * 16 + shift
            const uint32_t table = bcg * (kLanes * 16) + j;
            const uint32_t rt = min(kCbHead, t.n[table]);
            head[(j / 16) * kCbHeadLane + (j % 16) * kCbHeadRow + z] =
                uint16_t(t.fc[size_t(table) * 256 + min(z, rt)] >> 16);
        }
        for (uint32_t i = tid; i < kLanes * 16; i += blockDim.x) {
            nlds[i] = uint16_t(t.n[bcg * (kLanes * 16) + i]);
            tbase[i] = t.tail_base[bcg * (kLanes * 16) + i];
        }
        __syncthreads();
    }
    uint64_t sid;
    if (!cb_stream<kCbDecStreams>(g, first, sid)) return;
    uint32_t* wr = wring + (tid >> 5) * (kCbWordRing / 2);
    uint32_t* er = ering + (tid >> 5) * (kCbEscRing / 2);
    // every stream of the launch is of one pass
    if (first >= uint64_t(g.ncg) * g.ntb) decode_cb_stream<true, RANGE>(a, t, g, sid, head, nlds, tbase, wr, er);
    else decode_cb_stream<false, RANGE>(a, t, g, sid, head, nlds, tbase, wr, er);
}

// =============================================================== LDS kernels
// Residual mode.  A workgroup owns one channel group (32 channels = one stream
// width) of one slab over a range of token blocks, so the 32 lane tables sit
// in LDS for the workgroup's lifetime.  Each thread runs lane `lane` of S
// streams at once (independent rANS chains interleaved for latency hiding).
// Blocks are numbered so that the channel groups sharing 128-byte rows of the
// cache land on the same XCD back to back (dispatch is round-robin over the
// 8 XCDs), which lets that XCD's L2 serve the other quarters or halves of each
// line.
struct LdsGeo {
    uint32_t groups;   // line groups = slabs x token-block chunks x (channel groups / (G cgw))
    uint32_t G;        // workgroups per line group
    uint32_t ntbc;     // token-block chunks per slab
    uint32_t tbc;      // token blocks per chunk
    uint32_t cgw;      // channel groups per workgroup
};

struct LdsPos {
    uint32_t slab, cg, tb_begin, tb_end;
    bool valid;
};

__device__ __forceinline__ LdsPos lds_position(const Geo& geo, const LdsGeo& lg) {
    const uint32_t b = blockIdx.x;
    const uint32_t g = (b / (8u * lg.G)) * 8u + (b % 8u);
    LdsPos r;
    r.valid = g < lg.groups;
    const uint32_t c = (b / 8u) % lg.G;
    const uint32_t ncgg = geo.ncg / (lg.G * lg.cgw);
    r.cg = ((g % ncgg) * lg.G + c) * lg.cgw;
    const uint32_t rest = g / ncgg;
    const uint32_t tbc = rest % lg.ntbc;
    r.slab = rest / lg.ntbc;
    r.tb_begin = tbc * lg.tbc;
    r.tb_end = min(r.tb_begin + lg.tbc, geo.ntb);
    return r;
}

// Streams of one round: the token blocks tb0, tb0+1, ... of this half-wave.
// FULL rounds have all S streams present, so the loop body needs no
// activity predicates; partial rounds (short token ranges) use ACT = true.

// Decoder LDS layout: static LUTs (e4m3 only) and, dynamically, (freq, start)
// words [fs + 1][32] then slot->symbol maps [32][4096 >> HALF].  With HALF, a map entry covers a
// pair of slots and holds the symbol of the even one; the odd slot belongs to
// the next symbol exactly when that symbol starts there.
template <uint32_t DT, int S, int D, bool ACT, bool HALF>
__device__ __forceinline__ void decode_round(const DecodeLaunch& a, const LdsPos& ps, const Geo& geo, uint32_t tb0,
                                             const uint8_t* lut, const uint32_t* lfc, const uint8_t* lslot,
                                             uint32_t n, bool& bad) {
    constexpr uint32_t EB = DT == SKV_E4M3 ? 1u : 2u;
    constexpr uint32_t RAW = kSyms * EB;
    const uint32_t lane = threadIdx.x & 31u, half = threadIdx.x & 32u;
    const uint32_t ltmask = (1u << lane) - 1u;
    const uint64_t* index = a.index;
    const uint8_t* pay = a.pay;
    const uint32_t rowb = geo.C * EB;                      // bytes per cache row
    // slab bases are uniform over the workgroup; lanes add 32-bit offsets
    const size_t slab_b = size_t(ps.slab) * geo.T * rowb + size_t(ps.cg) * kLanes * EB;
    const uint8_t* aux = static_cast<const uint8_t*>(a.aux) + slab_b;
    uint8_t* out = static_cast<uint8_t*>(a.out) + slab_b;
    const uint8_t* my_slot = lslot + lane * (kM >> (HALF ? 1 : 0));

    // Per stream: state, word / escape cursors and bounds.  A stream that is
    // absent, raw or malformed runs as an idle chain: its escape symbol can never
    // match (256), its cursors never trip the checks and its reads stay inside the
    // payload.  Only partial rounds need to mask stores.
    uint32_t x[S], p[S], ep[S], nwc[S], nwl[S], ecc[S], ecl[S], ns[S], off[S], sz[S];
    const uint16_t* W[S];
    const uint8_t* E[S];
    bool act[S], rawc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint32_t tb = tb0 + s;
        const bool present = !ACT || tb < ps.tb_end;
        off[s] = (present ? tb : tb0) * kSteps * rowb + lane * EB;
        x[s] = kStateLow;
        p[s] = ep[s] = 0;
        nwc[s] = ecc[s] = 0xFFFFFFFFu;       // check bounds (idle: never reached)
        nwl[s] = ecl[s] = 0;                 // clamp bounds for reads
        ns[s] = 256;
        sz[s] = 0;
        W[s] = reinterpret_cast<const uint16_t*>(pay);
        E[s] = pay;
        act[s] = rawc[s] = false;
        if (!present) continue;
        const uint64_t sid = index_pos(a, ps.slab, tb, ps.cg, geo.ncg);
        const uint64_t e0 = index[sid], e1 = index[sid + 1];
        const uint64_t o = e0 & ~kRawBit, end = e1 & ~kRawBit;
        const uint64_t size = end - o;
        const uint8_t* sp = pay + o;
        if (end < o || end > a.payload_bytes) {
            bad = true;
            continue;
        }
        if (e0 & kRawBit) {
            if (size != RAW) bad = true;
            else rawc[s] = true;             // copied after the coded streams of the round
            E[s] = sp;
            continue;
        }
        uint32_t nw = 0;
        bool ok = size >= kStreamHead && size % 4 == 0;
        if (ok) {
            nw = reinterpret_cast<const uint32_t*>(sp)[32];
            ok = nw <= (size - kStreamHead) / 2;
        }
        if (!ok) {
            bad = true;
            continue;
        }
        act[s] = true;
        x[s] = reinterpret_cast<const uint32_t*>(sp)[lane];
        if (x[s] < kStateLow) bad = true;
        sz[s] = uint32_t(size);
        const uint32_t ecap = uint32_t((size - kStreamHead - 2 * nw) / EB);
        nwc[s] = nw;
        ecc[s] = ecap;
        nwl[s] = nw ? nw - 1 : 0;
        ecl[s] = ecap ? ecap - 1 : 0;
        ns[s] = n;
        W[s] = nw ? reinterpret_cast<const uint16_t*>(sp + kStreamHead) : reinterpret_cast<const uint16_t*>(sp);
        E[s] = ecap ? sp + kStreamHead + 2 * nw : sp;
    }

    uint32_t pbuf[S][D];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int d = 0; d < D; ++d)
            pbuf[s][d] = EB == 1 ? uint32_t(aux[off[s] + d * rowb])
                                 : uint32_t(*reinterpret_cast<const uint16_t*>(aux + off[s] + d * rowb));
    for (uint32_t kk = 0; kk < uint32_t(kSteps); kk += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const uint32_t k = kk + d;
            const uint32_t kn = min(k + uint32_t(D), uint32_t(kSteps) - 1u);
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const uint32_t pv = pbuf[s][d];
                const uint32_t slot = x[s] & (kM - 1u);
                uint32_t sym, fcv;
                if (HALF) {
                    const uint32_t s0 = my_slot[slot >> 1];
                    const uint32_t f0 = lfc[s0 * kLanes + lane];
                    const uint32_t f1 = lfc[(s0 + 1) * kLanes + lane];
                    const bool adv = slot >= (f1 >> 16);   // start past the last symbol is a sentinel
                    sym = adv ? s0 + 1 : s0;
                    fcv = adv ? f1 : f0;
                } else {
                    sym = my_slot[slot];
                    fcv = lfc[sym * kLanes + lane];
                }
                uint32_t xs = (fcv & 0xFFFFu) * (x[s] >> kProbBits) + slot - (fcv >> 16);
                // Refill in lane order from the stream's words.  Reads are clamped
                // into the stream; running past its words shows in the final count.
                const uint32_t mw = uint32_t(__ballot(xs < kStateLow) >> half);
                const bool need = (mw >> lane) & 1u;
                const uint32_t w = W[s][min(p[s] + __popc(mw & ltmask), nwl[s])];
                p[s] += __popc(mw);
                // escaped values, in lane order, from the escape region
                const uint32_t me = uint32_t(__ballot(sym == ns[s]) >> half);
                const bool esc = (me >> lane) & 1u;
                const uint32_t ei = min(ep[s] + __popc(me & ltmask), ecl[s]);
                const uint32_t v = EB == 1 ? uint32_t(E[s][ei]) : uint32_t(reinterpret_cast<const uint16_t*>(E[s])[ei]);
                ep[s] += __popc(me);
                // the next predictor row is requested after this step's payload reads:
                // waits for those reads then leave it in flight
                pbuf[s][d] = EB == 1 ? uint32_t(aux[off[s] + kn * rowb])
                                     : uint32_t(*reinterpret_cast<const uint16_t*>(aux + off[s] + kn * rowb));
                x[s] = need ? ((xs << 16) | w) : xs;
                if (esc && v < n) bad = true;      // a canonical encoder codes such a value directly
                const uint32_t z = esc ? v : sym;
                uint32_t t;
                if (DT == SKV_E4M3) t = lut[512 + uint32_t(lut[pv]) + uint32_t(lut[256 + z])];
                else t = unord16((ord16(pv) + unzig(z)) & 0xFFFFu);
                if (!ACT || act[s] || rawc[s]) {
                    if (EB == 1) out[off[s] + k * rowb] = uint8_t(t);
                    else *reinterpret_cast<uint16_t*>(out + off[s] + k * rowb) = uint16_t(t);
                }
            }
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        if (rawc[s]) {
            // raw stream: its elements in (step, lane) order replace what the idle chain wrote
            const uint8_t* sp = E[s];
            for (uint32_t k = 0; k < uint32_t(kSteps); ++k) {
                if (EB == 1) out[off[s] + k * rowb] = sp[k * kLanes + lane];
                else *reinterpret_cast<uint16_t*>(out + off[s] + k * rowb) =
                    reinterpret_cast<const uint16_t*>(sp)[k * kLanes + lane];
            }
        }
        if (!act[s]) continue;
        if (x[s] != kStateLow || p[s] != nwc[s] || ep[s] > ecc[s]) bad = true;
        const uint8_t* sp = pay + (index[index_pos(a, ps.slab, tb0 + s, ps.cg, geo.ncg)] & ~kRawBit);
        const uint32_t used = kStreamHead + 2 * nwc[s] + EB * ep[s];
        if (((used + 3) & ~3u) != sz[s]) bad = true;
        else if (lane < sz[s] - used && sp[used + lane] != 0) bad = true;   // zero pad
    }
}

template <uint32_t DT, int S, int D, bool HALF>
__global__ __launch_bounds__(1024, HALF ? 8 : 4) void decode_lds(DecodeLaunch a, DevTables t, uint32_t fs, LdsGeo lg) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ uint8_t lut[DT == SKV_E4M3 ? 1024 : 4];                    // e4m3: ord | unzig | unord x2
    const Geo geo = geometry(a.shape);
    const LdsPos ps = lds_position(geo, lg);
    if (!ps.valid) return;
    const uint32_t tab0 = ps.slab * geo.C + ps.cg * kLanes;
    constexpr uint32_t MAPN = kM >> (HALF ? 1 : 0);                         // map entries per table
    uint32_t* lfc = reinterpret_cast<uint32_t*>(lds);                      // [fs + 1 symbols][32 lanes]
    uint8_t* lslot = lds + kLanes * (fs + 1) * 4;                          // [32 lanes][MAPN]
    for (uint32_t i = threadIdx.x; i < kLanes * (fs + 1); i += blockDim.x) {
        const uint32_t sym = i / kLanes, j = i % kLanes;
        lfc[i] = sym < fs ? t.fc[size_t(tab0 + j) * 256 + sym] : 0xFFFF0000u;   // sentinel start past 4095
    }
    if (DT == SKV_E4M3)
        for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) {
            lut[i] = uint8_t(ord8(i));
            lut[256 + i] = uint8_t(unzig(i));
            lut[512 + i] = uint8_t(unord8(i));
            lut[768 + i] = uint8_t(unord8(i));
        }
    __syncthreads();
    // slot -> symbol maps: each thread fills one dword (4 entries) of every map,
    // finding the first symbol by binary search over the symbol starts
    constexpr uint32_t STRIDE = HALF ? 2u : 1u;
    for (uint32_t d = threadIdx.x; d < kLanes * (MAPN / 4); d += blockDim.x) {
        const uint32_t j = d / (MAPN / 4), slot0 = (d % (MAPN / 4)) * 4 * STRIDE;
        const uint32_t nn = t.n[tab0 + j];
        uint32_t lo = 0, hi = nn;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            if ((lfc[mid * kLanes + j] >> 16) <= slot0) lo = mid;
            else hi = mid - 1;
        }
        uint32_t word = 0, sym = lo;
        for (uint32_t q = 0; q < 4; ++q) {
            while (sym < nn && (lfc[(sym + 1) * kLanes + j] >> 16) <= slot0 + q * STRIDE) ++sym;
            word |= sym << (8 * q);
        }
        reinterpret_cast<uint32_t*>(lslot)[d] = word;
    }
    __syncthreads();

    const uint32_t lane = threadIdx.x & 31u;
    const uint32_t hw = threadIdx.x >> 5, nhw = blockDim.x >> 5;
    const uint32_t n = t.n[tab0 + lane];
    bool bad = false;
    for (uint32_t tb0 = ps.tb_begin + hw * S; tb0 < ps.tb_end; tb0 += nhw * S) {
        if (tb0 + S <= ps.tb_end) decode_round<DT, S, D, false, HALF>(a, ps, geo, tb0, lut, lfc, lslot, n, bad);
        else decode_round<DT, S, D, true, HALF>(a, ps, geo, tb0, lut, lfc, lslot, n, bad);
    }
    if (bad) atomicOr(a.status, 1u);
}

// Encoder scratch per stream (2 x raw bytes): final states [0, 128), escaped
// values from 132 and words from `raw`, both in emission order (the compaction
// reverses them into decode order).  Inside a half-wave, hardware lane L runs
// format lane 31 - L, so "emitted earlier in this step" means "lower hardware
// lane".  The two half-waves of a wavefront run two streams in lockstep; their
// word and escape counts are wave-uniform scalars and a lane finds its slot
// with mbcnt over the whole 64-lane ballot.  Counts stop advancing the write
// position once a stream is certain to be stored raw, so a stream never writes
// outside its own scratch area (any slot at or past the limit implies raw).
template <uint32_t DT, int S, int D, bool ACT>
__device__ __forceinline__ void encode_round(const EncodeLaunch& a, const LdsPos& ps, const Geo& geo, uint32_t tb0,
                                             const uint4* lenc, const uint8_t* zlut, uint32_t n) {
    static_assert(D >= 2, "the one-step lookahead reads the next ring slot");
    constexpr uint32_t EB = DT == SKV_E4M3 ? 1u : 2u;
    constexpr uint32_t RAW = kSyms * EB;
    constexpr uint32_t MAXW = (RAW - kStreamHead) / 2;
    constexpr uint32_t MAXE = (RAW - kStreamHead) / EB;
    constexpr uint32_t kDrop = 0x80000000u;                // buffer offset past the range: the store is dropped
    static_assert(kStreamHead + EB * (MAXE + 32) <= 2 * RAW && RAW + 2 * (MAXW + 32) <= 2 * RAW,
                  "clamped slots stay inside the stream's scratch area");
    const uint32_t hl = threadIdx.x & 31u;
    const bool upper = (threadIdx.x & 32u) != 0;
    const uint32_t fsh = upper ? 16u : 0u;                 // which 16-bit field of a packed pair is this half's
    const uint32_t lane = 31u - hl;                        // format lane
    const uint32_t rowb = geo.C * EB;
    const size_t slab_b = size_t(ps.slab) * geo.T * rowb + size_t(ps.cg) * kLanes * EB;
    const uint8_t* tgt = static_cast<const uint8_t*>(a.target) + slab_b;
    const uint8_t* aux = static_cast<const uint8_t*>(a.aux) + slab_b;
    // the workgroup's streams are ncg apart in stream order: 32-bit offsets from a common base,
    // stores go through a buffer resource spanning the workgroup's scratch (span < 2^31, host-checked)
    const uint64_t sid0 = (uint64_t(ps.slab) * geo.ntb + ps.tb_begin) * geo.ncg + ps.cg;
    uint8_t* wgs = a.scratch + sid0 * (2 * RAW);
    const uint32_t sstride = geo.ncg * (2 * RAW);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        wgs, (short)0, int((ps.tb_end - ps.tb_begin - 1) * sstride + 2 * RAW), 0x00020000);

    // upper-half slots carry a bias of 32 (mbcnt_lo counts the whole lower half for them)
    const uint32_t bias_b = upper ? 32u : 0u;
    uint32_t x[S], off[S], ao[S], wbase[S], ebase[S];
    uint32_t wlo[S], whi[S], elo[S], ehi[S];               // wave-uniform counts per half
    bool act[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint32_t tb = tb0 + s;
        act[s] = !ACT || tb < ps.tb_end;
        const uint32_t tbs = act[s] ? tb : tb0;
        off[s] = tbs * kSteps * rowb + lane * EB;
        ao[s] = (tbs - ps.tb_begin) * sstride;
        wbase[s] = ao[s] + RAW - 2 * bias_b;
        ebase[s] = ao[s] + kStreamHead - EB * bias_b;
        x[s] = kStateLow;
        wlo[s] = whi[s] = elo[s] = ehi[s] = 0;
    }
    // target / predictor values D steps ahead (steps run backwards)
    using V = std::conditional_t<EB == 1, uint8_t, uint16_t>;
    V tbuf[S][D], pbuf[S][D];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const uint32_t o = off[s] + (kSteps - 1 - d) * rowb;
            tbuf[s][d] = *reinterpret_cast<const V*>(tgt + o);
            pbuf[s][d] = *reinterpret_cast<const V*>(aux + o);
        }
    // e4m3: zlut[0, 256) is the order-preserving map of a byte, zlut[256, 768)
    // the zigzag of (a - b) mod 256 at index 512 + a - b
    auto symbol_of = [&](uint32_t tv, uint32_t pv) -> uint32_t {
        return DT == SKV_E4M3 ? uint32_t(zlut[512u + uint32_t(zlut[tv]) - uint32_t(zlut[pv])])
                              : zig16((ord16(tv) - ord16(pv)) & 0xFFFFu);
    };
    // symbol value and table entry run one step ahead of the state chain
    uint32_t zc[S];
    uint4 ec[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        zc[s] = symbol_of(tbuf[s][0], pbuf[s][0]);
        ec[s] = lenc[min(zc[s], n) * kLanes + lane];
    }
    for (int kk = kSteps - 1; kk >= 0; kk -= D) {
        uint32_t zs[S][D];                                 // this iteration's symbols, for the escape pass
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int k = kk - d;
            const uint32_t kn = uint32_t(max(k - D, 0));
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const uint32_t z = zc[s];
                const uint4 e = ec[s];
                zs[s][d] = z;
                // next step's symbol and entry (step k - 1, held in ring slot d + 1)
                const uint32_t zn = symbol_of(tbuf[s][(d + 1) % D], pbuf[s][(d + 1) % D]);
                const uint4 en = lenc[min(zn, n) * kLanes + lane];
                const uint32_t o = off[s] + kn * rowb;
                tbuf[s][d] = *reinterpret_cast<const V*>(tgt + o);
                pbuf[s][d] = *reinterpret_cast<const V*>(aux + o);
                // words leave before the state absorbs the symbol
                uint32_t xs = x[s];
                const bool emit = (!ACT || act[s]) && xs >= e.x;
                const uint64_t mw = __ballot(emit);
                const uint32_t mlo = uint32_t(mw), mhi = uint32_t(mw >> 32), plo = __popc(mlo);
                const uint32_t pk = min(wlo[s], MAXW) | ((min(whi[s], MAXW) + 32u - plo) << 16);
                const uint32_t slot =
                    __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, __builtin_amdgcn_ubfe(pk, fsh, 16)));
                __builtin_amdgcn_raw_buffer_store_b16(uint16_t(xs & 0xFFFFu), wrs,
                                                      emit ? wbase[s] + 2 * slot : kDrop, 0, 0);
                wlo[s] += plo;
                whi[s] += __popc(mhi);
                xs = emit ? xs >> 16 : xs;
                const uint32_t qt = __umulhi(xs + (e.z >> 24), e.y) >> (e.w & 31u);   // floor(xs / f)
                x[s] = (xs + (e.w >> 16)) + __umul24(qt, e.z);    // quotient < 2^20, low 24 bits: 4096 - f
                zc[s] = zn;
                ec[s] = en;
            }
        }
        // escaped values of this iteration, in emission order (rare: skipped by the whole wavefront)
#pragma unroll
        for (int s = 0; s < S; ++s) {
            uint32_t zm = zs[s][0];
#pragma unroll
            for (int d = 1; d < D; ++d) zm = max(zm, zs[s][d]);
            if (__ballot((!ACT || act[s]) && zm >= n) == 0) continue;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const uint32_t z = zs[s][d];
                const bool esc = (!ACT || act[s]) && z >= n;
                const uint64_t me = __ballot(esc);
                const uint32_t mlo = uint32_t(me), mhi = uint32_t(me >> 32), plo = __popc(mlo);
                const uint32_t pk = min(elo[s], MAXE) | ((min(ehi[s], MAXE) + 32u - plo) << 16);
                const uint32_t slot =
                    __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, __builtin_amdgcn_ubfe(pk, fsh, 16)));
                const uint32_t eo = esc ? ebase[s] + EB * slot : kDrop;
                if (EB == 1) __builtin_amdgcn_raw_buffer_store_b8(uint8_t(z), wrs, eo, 0, 0);
                else __builtin_amdgcn_raw_buffer_store_b16(uint16_t(z), wrs, eo, 0, 0);
                elo[s] += plo;
                ehi[s] += __popc(mhi);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        if (!act[s]) continue;
        reinterpret_cast<uint32_t*>(wgs + ao[s])[lane] = x[s];
        if (hl == 0) {
            const uint32_t cnt = upper ? whi[s] : wlo[s], ecnt = upper ? ehi[s] : elo[s];
            const uint64_t sid = sid0 + uint64_t(tb0 + s - ps.tb_begin) * geo.ncg;
            const uint32_t bytes = (kStreamHead + 2 * cnt + EB * ecnt + 3) & ~3u;
            a.meta[sid] = bytes >= RAW ? 0x80000000u : (cnt | (ecnt << 14));
        }
    }
}

template <uint32_t DT, int S, int D>
__global__ __launch_bounds__(1024) void encode_lds(EncodeLaunch a, DevTables t, uint32_t fs, LdsGeo lg) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ uint8_t zlut[DT == SKV_E4M3 ? 768 : 4];                   // e4m3: ord | zigzag of a difference
    const Geo geo = geometry(a.shape);
    const LdsPos ps = lds_position(geo, lg);
    if (!ps.valid) return;
    const uint32_t tab0 = ps.slab * geo.C + ps.cg * kLanes;
    uint4* lenc = reinterpret_cast<uint4*>(lds);                            // [fs symbols][32 lanes]
    for (uint32_t i = threadIdx.x; i < kLanes * fs; i += blockDim.x) {
        const uint32_t sym = i / kLanes, j = i % kLanes;
        lenc[i] = t.enc[size_t(tab0 + j) * 256 + sym];
    }
    if (DT == SKV_E4M3)
        for (uint32_t i = threadIdx.x; i < 512; i += blockDim.x) {
            if (i < 256) zlut[i] = uint8_t(ord8(i));
            zlut[256 + i] = uint8_t(zig8((i - 256u) & 0xFFu));
        }
    __syncthreads();
    const uint32_t lane = 31u - (threadIdx.x & 31u);      // format lane (reversed within the half-wave)
    const uint32_t hw = threadIdx.x >> 5, nhw = blockDim.x >> 5;
    const uint32_t n = t.n[tab0 + lane];
    for (uint32_t tb0 = ps.tb_begin + hw * S; tb0 < ps.tb_end; tb0 += nhw * S) {
        if (tb0 + S <= ps.tb_end) encode_round<DT, S, D, false>(a, ps, geo, tb0, lenc, zlut, n);
        else encode_round<DT, S, D, true>(a, ps, geo, tb0, lenc, zlut, n);
    }
}

// --------------------------------------------------------------- tiled e4m3 encode
// The e4m3 encoder moves data in wide pieces and gathers bytes from LDS.  Each
// wavefront runs two streams (one per half) in 8-step tiles: a lane loads 8
// bytes of target and of predictor (8 channels of one token), maps both to
// the order-preserving code and subtracts them bytewise in registers, and
// stores the 8 difference bytes in the wavefront's LDS tile; after that every
// lane reads its own channel for the tile's 8 steps and zigzags it through a
// 256-byte table.  Emitted words go to a 128-word LDS ring per stream and
// leave in 128-byte chunks as soon as a chunk is full.  The scratch layout is
// the one the compaction reads: states [0, 128), escaped values from 132 and
// words from `raw`, both in emission order.
constexpr uint32_t kTileSteps = 8;
constexpr uint32_t kRingWords = 512;                      // eight 64-word chunks per stream
constexpr uint32_t kTileLds = 2 * kTileSteps * kLanes;    // difference bytes of both halves
constexpr uint32_t kRingLds = 2 * kRingWords * 2;
constexpr uint32_t kTileWaveLds = kTileLds + kRingLds;

// Bytewise sign flip of 4 packed e4m3 codes: v ^ 0x7F in the bytes whose sign
// bit is set.  The order-preserving code of a byte is flip(u) ^ 0x80, so the
// difference of two order codes mod 256 is the difference of their flips.
// v_perm_b32 spreads a sign into a whole byte only from bytes 1 and 3 of each
// source dword; with v << 8 as the second dword, the signs of v's bytes 0, 1,
// 2, 3 sit at permute bytes 5, 1, 7, 3 (selectors 10, 8, 11, 9).
__device__ __forceinline__ uint32_t sflip8x4(uint32_t v) {
    return v ^ (__builtin_amdgcn_perm(v << 8, v, 0x090B080Au) & 0x7F7F7F7Fu);
}
// bytewise (a - b) mod 256
__device__ __forceinline__ uint32_t sub8x4(uint32_t a, uint32_t b) {
    return ((a | 0x80808080u) - (b & 0x7F7F7F7Fu)) ^ (~(a ^ b) & 0x80808080u);
}

template <uint32_t DT>
__global__ __launch_bounds__(1024) void encode_tiles(EncodeLaunch a, DevTables t, uint32_t fs, LdsGeo lg) {
    static_assert(DT == SKV_E4M3, "byte elements");
    constexpr uint32_t RAW = kSyms;
    constexpr uint32_t MAXE = RAW - kStreamHead;
    constexpr uint32_t kDrop = 0x80000000u;               // buffer offset past the range: the access is dropped
    constexpr uint32_t kChunks = RAW / 128;                // 64-word chunks that fit the words region
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ uint8_t zig[256];
    const Geo geo = geometry(a.shape);
    const LdsPos ps = lds_position(geo, lg);
    if (!ps.valid) return;
    const uint32_t tab0 = ps.slab * geo.C + ps.cg * kLanes;
    uint4* lenc = reinterpret_cast<uint4*>(lds);                            // [fs symbols][32 lanes]
    for (uint32_t i = threadIdx.x; i < kLanes * fs; i += blockDim.x) {
        const uint32_t sym = i / kLanes, j = i % kLanes;
        lenc[i] = t.enc[size_t(tab0 + j) * 256 + sym];
    }
    for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) zig[i] = uint8_t(zig8(i));
    __syncthreads();

    const uint32_t wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
    const uint32_t hl = threadIdx.x & 31u;
    const bool upper = (threadIdx.x & 32u) != 0;
    const uint32_t fsh = upper ? 16u : 0u;
    const uint32_t lane = 31u - hl;                        // format lane (reversed within the half)
    const uint32_t n = t.n[tab0 + lane];
    uint8_t* tile = lds + size_t(kLanes) * fs * 16 + wave * kTileWaveLds;
    uint8_t* ring = tile + kTileLds;
    // tile: [half][step][32 channels]; this lane loads 8 channels of one step and reads its channel back
    const uint32_t ld_row = hl >> 2, ld_q = hl & 3u;
    uint2* tile_st = reinterpret_cast<uint2*>(tile + (upper ? kTileSteps * kLanes : 0u) + ld_row * kLanes + ld_q * 8);
    const uint8_t* tile_rd = tile + (upper ? kTileSteps * kLanes : 0u) + lane;
    uint16_t* ring_h = reinterpret_cast<uint16_t*>(ring + (upper ? kRingWords * 2 : 0u));

    const uint32_t rowb = geo.C;
    const size_t slab_b = size_t(ps.slab) * geo.T * rowb + size_t(ps.cg) * kLanes;
    const uint8_t* tgt = static_cast<const uint8_t*>(a.target) + slab_b + ld_q * 8;
    const uint8_t* aux = static_cast<const uint8_t*>(a.aux) + slab_b + ld_q * 8;
    const uint64_t sid0 = (uint64_t(ps.slab) * geo.ntb + ps.tb_begin) * geo.ncg + ps.cg;
    uint8_t* wgs = a.scratch + sid0 * (2 * RAW);
    const uint32_t sstride = geo.ncg * (2 * RAW);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        wgs, (short)0, int((ps.tb_end - ps.tb_begin - 1) * sstride + 2 * RAW), 0x00020000);

    // z of one tile: difference bytes into LDS, then each lane's channel through the zigzag table
    auto stage = [&](uint2 tv, uint2 pv, uint32_t* z) {
        *tile_st = make_uint2(sub8x4(sflip8x4(tv.x), sflip8x4(pv.x)), sub8x4(sflip8x4(tv.y), sflip8x4(pv.y)));
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (uint32_t r = 0; r < kTileSteps; ++r) z[r] = zig[tile_rd[r * kLanes]];
        __builtin_amdgcn_wave_barrier();
    };
    const uint32_t* ring32 = reinterpret_cast<const uint32_t*>(ring_h);

    for (uint32_t r0 = ps.tb_begin + 2 * wave; r0 < ps.tb_end; r0 += 2 * nwave) {
        const uint32_t tb = r0 + (upper ? 1u : 0u);
        const bool act = tb < ps.tb_end;
        const uint32_t tbs = act ? tb : r0;
        const uint32_t ao = (tbs - ps.tb_begin) * sstride;
        const uint32_t ebase = ao + kStreamHead - (upper ? 32u : 0u);   // upper-half slots carry a bias of 32
        const uint32_t wreg = ao + RAW;
        const uint8_t* tsrc = tgt + size_t(tbs * kSteps + ld_row) * rowb;
        const uint8_t* psrc = aux + size_t(tbs * kSteps + ld_row) * rowb;
        const size_t tstride = size_t(kTileSteps) * rowb;
        constexpr int kTiles = kSteps / kTileSteps;

        uint32_t zc[kTileSteps], zn[kTileSteps];
        uint2 tv = *reinterpret_cast<const uint2*>(tsrc + (kTiles - 1) * tstride);
        uint2 pv = *reinterpret_cast<const uint2*>(psrc + (kTiles - 1) * tstride);
        stage(tv, pv, zc);
        tv = *reinterpret_cast<const uint2*>(tsrc + (kTiles - 2) * tstride);
        pv = *reinterpret_cast<const uint2*>(psrc + (kTiles - 2) * tstride);

        uint32_t x = kStateLow;
        uint32_t wp = 0;                                   // word counts: lower half | upper half << 16
        uint32_t fl = 0;                                   // chunks stored: lower half | upper half << 16
        uint32_t elo = 0, ehi = 0;                         // escape counts per half
        uint4 ec = lenc[min(zc[kTileSteps - 1], n) * kLanes + lane];
        for (int j = kTiles - 1; j >= 0; --j) {
            if (j > 0) {
                stage(tv, pv, zn);
                if (j > 1) {
                    tv = *reinterpret_cast<const uint2*>(tsrc + size_t(j - 2) * tstride);
                    pv = *reinterpret_cast<const uint2*>(psrc + size_t(j - 2) * tstride);
                }
            }
#pragma unroll
            for (int r = kTileSteps - 1; r >= 0; --r) {
                const uint4 e = ec;
                const uint32_t znext = r > 0 ? zc[r - 1] : zn[kTileSteps - 1];
                ec = lenc[min(znext, n) * kLanes + lane];
                // words leave before the state absorbs the symbol (an idle half runs a copy of its
                // partner's stream into its own ring and stores nothing)
                uint32_t xs = x;
                const bool emit = xs >= e.x;
                const uint64_t mw = __ballot(emit);
                const uint32_t mlo = uint32_t(mw), mhi = uint32_t(mw >> 32);
                const uint32_t pp = __popc(mlo) | (__popc(mhi) << 16);
                // ring slot: this half's count mod 512 plus the emitting lanes below (mbcnt_lo counts the
                // entire lower half for an upper lane, which the packed base subtracts again)
                const uint32_t pk = (wp - (pp << 16)) & 0x01FF01FFu;
                const uint32_t slot =
                    __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, __builtin_amdgcn_ubfe(pk, fsh, 16)));
                if (emit) ring_h[slot & (kRingWords - 1)] = uint16_t(xs & 0xFFFFu);
                xs = emit ? xs >> 16 : xs;
                const uint32_t qt = __umulhi(xs + (e.z >> 24), e.y) >> (e.w & 31u);   // floor(xs / f)
                // x = xs + qt (4096 - f) + start, the start taken from the high half of e.w
                const uint32_t xq = __umul24(qt, e.z) + xs;
                asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
                    : "=v"(x) : "v"(xq), "v"(e.w));
                wp += pp;
            }
            // completed 64-word chunks leave the ring (a tile adds at most 256 words per stream, so
            // the 512-word ring never overruns the chunks still waiting)
            const uint32_t done = (wp >> 6) & 0x03FF03FFu;
            while (fl != done) {
                __builtin_amdgcn_wave_barrier();
                const uint32_t ck = __builtin_amdgcn_ubfe(fl, fsh, 16);
                const bool mine = act && ck < __builtin_amdgcn_ubfe(done, fsh, 16);
                const uint32_t w = ring32[(ck & (kRingWords / 64 - 1)) * 32 + hl];
                __builtin_amdgcn_raw_buffer_store_b32(w, wrs, mine && ck < kChunks ? wreg + ck * 128 + 4 * hl : kDrop,
                                                      0, 0);
                fl += ((fl & 0xFFFFu) != (done & 0xFFFFu) ? 1u : 0u) + ((fl >> 16) != (done >> 16) ? 0x10000u : 0u);
                __builtin_amdgcn_wave_barrier();
            }
            // escaped values of this tile, in emission order (rare: skipped by the whole wavefront)
            uint32_t zm = zc[0];
#pragma unroll
            for (uint32_t r = 1; r < kTileSteps; ++r) zm = max(zm, zc[r]);
            if (__ballot(zm >= n) != 0) {
#pragma unroll
                for (int r = kTileSteps - 1; r >= 0; --r) {
                    const bool esc = zc[r] >= n;
                    const uint64_t me = __ballot(esc);
                    if (me == 0) continue;
                    const uint32_t mlo = uint32_t(me), mhi = uint32_t(me >> 32), plo = __popc(mlo);
                    const uint32_t pk = min(elo, MAXE) | ((min(ehi, MAXE) + 32u - plo) << 16);
                    const uint32_t slot = __builtin_amdgcn_mbcnt_hi(
                        mhi, __builtin_amdgcn_mbcnt_lo(mlo, __builtin_amdgcn_ubfe(pk, fsh, 16)));
                    __builtin_amdgcn_raw_buffer_store_b8(uint8_t(zc[r]), wrs, act && esc ? ebase + slot : kDrop, 0,
                                                         0);
                    elo += plo;
                    ehi += __popc(mhi);
                }
            }
#pragma unroll
            for (uint32_t r = 0; r < kTileSteps; ++r) zc[r] = zn[r];
        }
        // the partial last chunk, the final states and the stream's counts
        __builtin_amdgcn_wave_barrier();
        const uint32_t cnt = __builtin_amdgcn_ubfe(wp, fsh, 16), ecnt = upper ? ehi : elo;
        const uint32_t ck = cnt >> 6;
        const uint32_t w = ring32[(ck & (kRingWords / 64 - 1)) * 32 + hl];
        __builtin_amdgcn_raw_buffer_store_b32(
            w, wrs, act && ck < kChunks && 2 * hl < (cnt & 63u) ? wreg + ck * 128 + 4 * hl : kDrop, 0, 0);
        __builtin_amdgcn_wave_barrier();
        if (act) {
            reinterpret_cast<uint32_t*>(wgs + ao)[lane] = x;
            if (hl == 0) {
                const uint64_t sid = sid0 + uint64_t(tb - ps.tb_begin) * geo.ncg;
                const uint32_t bytes = (kStreamHead + 2 * cnt + ecnt + 3) & ~3u;
                a.meta[sid] = bytes >= RAW ? 0x80000000u : (cnt | (ecnt << 14));
            }
        }
    }
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

// The same coder with a workgroup on 2 NC adjacent channel groups: chain c
// of a lane codes channel group 2c + (upper half), so a wavefront codes the
// 2 NC streams of one token block and every row load covers 64 NC contiguous
// bytes of target and predictor.  With NC = 2 a load instruction reads whole
// 128-byte lines, each line once; with NC = 1 the two workgroups sharing a
// line run on one XCD and reach it through its L2.  The tables of the groups
// sit in LDS ([symbols][64 NC columns]); a stream's words go through a
// 128-word ring that stores each completed 64-word chunk at once.
constexpr uint32_t kPairRing = 128;
__host__ __device__ constexpr uint32_t encode_groups_lds(uint32_t nc, uint32_t fs) {
    return 2 * nc * kLanes * fs * 16 + 16 * (kTileSteps * 2 * nc * kLanes + 2 * nc * kPairRing * 2);
}
// Exponent-class tables ([16 classes][fs] entries and the classes' n) with 16-bit tile entries
__host__ __device__ constexpr uint32_t encode_exp_lds(uint32_t fs) {
    return kExpClasses * (fs + 1) * 16 + kExpClasses + 8 * (kTileSteps * 2 * kLanes * 2 + 2 * kPairRing * 2) + 16;
}

// Z8(d): zigzag symbols of 4 signed residual bytes, (d << 1) per byte with the
// byte's sign spread over it (v_perm selectors 8..11 give a byte's sign)
__device__ __forceinline__ uint32_t zig8x4(uint32_t d) {
    return ((d << 1) & 0xFEFEFEFEu) ^ __builtin_amdgcn_perm(d << 8, d, 0x090B080Au);
}

// EXP: exponent-class tables (one table per slab and predictor exponent class);
// a tile entry is 16 bits, the symbol and the class of one position.
template <uint32_t NC, bool EXP = false>
__device__ __forceinline__ void encode_groups_body(const EncodeLaunch& a, const DevTables& t, uint32_t fs,
                                                   const LdsGeo& lg) {
    static_assert(!EXP || NC == 1, "exponent classes: two channel groups");
    constexpr uint32_t RAW = kSyms;
    constexpr uint32_t MAXE = RAW - kStreamHead;
    constexpr uint32_t kDrop = 0x80000000u;               // buffer offset past the range: the access is dropped
    constexpr uint32_t kChunks = RAW / 128;                // 64-word chunks that fit the words region
    constexpr uint32_t NG = 2 * NC;                        // channel groups of the workgroup
    constexpr uint32_t RL = NG * kLanes;                   // bytes of a tile row = table columns
    constexpr uint32_t LW = RL / 8;                        // bytes a lane loads per row (8 lanes a row)
    constexpr uint32_t TE = EXP ? 2 : 1;                   // bytes of a tile entry
    constexpr uint32_t WLDS = kTileSteps * RL * TE + NG * kPairRing * 2;
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ uint8_t zig[256];
    const Geo geo = geometry(a.shape);
    const LdsPos ps = lds_position(geo, lg);
    if (!ps.valid) return;
    // first table of the groups (EXP: of the slab's classes)
    const uint32_t tab0 = EXP ? ps.slab * kExpClasses : ps.slab * geo.C + ps.cg * kLanes;
    constexpr uint32_t NT = EXP ? kExpClasses : RL;        // tables held
    // EXP: a class takes fs + 1 entries (an odd number of 16-byte entries), so that the same symbol of
    // different classes falls in different LDS banks
    const uint32_t cstride = EXP ? fs + 1 : fs;
    uint4* lenc = reinterpret_cast<uint4*>(lds);           // [fs symbols][RL columns] or [16 classes][fs + 1]
    for (uint32_t i = threadIdx.x; i < NT * fs; i += blockDim.x) {
        if constexpr (EXP) {
            const uint32_t q = i / fs, sym = i % fs;       // entries past n repeat the escape entry, flagged
            lenc[q * cstride + sym] = t.enc[size_t(tab0 + q) * 256 + sym];
        } else {
            const uint32_t sym = i / RL, j = i % RL;
            lenc[i] = t.enc[size_t(tab0 + j) * 256 + sym];
        }
    }
    uint8_t* nq = lds + size_t(NT) * cstride * 16;         // EXP: n of each class
    if (EXP && threadIdx.x < kExpClasses) nq[threadIdx.x] = uint8_t(t.n[tab0 + threadIdx.x]);
    for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) zig[i] = uint8_t(zig8(i));
    __syncthreads();

    const uint32_t wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
    const uint32_t hl = threadIdx.x & 31u;
    const bool upper = (threadIdx.x & 32u) != 0;
    const uint32_t fsh = upper ? 16u : 0u;
    const uint32_t lane = 31u - hl;                        // format lane (reversed within the half)
    uint8_t* tile = lds + ((size_t(NT) * cstride * 16 + (EXP ? 16 : 0)) + wave * WLDS);
    uint8_t* ring = tile + kTileSteps * RL * TE;
    // tile: [step][RL channels]; a lane loads LW channels of one step and reads its chains' channels back
    const uint32_t ld_row = (threadIdx.x & 63u) >> 3, ld_q = (threadIdx.x & 7u) * LW;
    uint8_t* tile_st = tile + (ld_row * RL + ld_q) * TE;
    uint32_t tl[NC], n[NC], ring_b[NC];
    const uint8_t* tile_rd[NC];
    const uint32_t* ring32[NC];
#pragma unroll
    for (uint32_t c = 0; c < NC; ++c) {
        const uint32_t grp = 2 * c + (upper ? 1u : 0u);
        tl[c] = grp * kLanes + lane;                       // table column of the chain's channel
        n[c] = EXP ? 0u : t.n[tab0 + tl[c]];
        tile_rd[c] = tile + (grp * kLanes + lane) * TE;
        ring_b[c] = uint32_t(uintptr_t(ring)) + grp * kPairRing * 2;   // LDS byte offsets
        ring32[c] = reinterpret_cast<const uint32_t*>(ring + grp * kPairRing * 2);
    }

    const uint32_t rowb = geo.C;
    // target and predictor rows of the slab's channel groups through one buffer resource each:
    // the lane's row and byte offsets in a register, the tile's row offset in a scalar
    const size_t slab_b = size_t(ps.slab) * geo.T * rowb + size_t(ps.cg) * kLanes;
    const int slab_n = int(uint32_t(geo.T - 1) * rowb + RL);
    const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(a.target) + slab_b), (short)0, slab_n, 0x00020000);
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(a.aux) + slab_b), (short)0, slab_n, 0x00020000);
    const uint64_t sid0 = (uint64_t(ps.slab) * geo.ntb + ps.tb_begin) * geo.ncg + ps.cg;
    uint8_t* wgs = a.scratch + sid0 * (2 * RAW);
    const uint32_t sstride = geo.ncg * (2 * RAW);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        wgs, (short)0, int((ps.tb_end - ps.tb_begin - 1) * sstride + NG * 2 * RAW), 0x00020000);

    typedef uint32_t Row[LW / 4];
    // z of one tile: difference bytes into LDS, then each chain's channel through the zigzag table
    // (EXP: symbol | class << 8 per position, formed in registers)
    auto stage = [&](const Row& tv, const Row& pv, uint32_t (&z)[NC][kTileSteps]) {
        uint32_t d[LW / 4];
#pragma unroll
        for (uint32_t k = 0; k < LW / 4; ++k) d[k] = sub8x4(sflip8x4(tv[k]), sflip8x4(pv[k]));
        if constexpr (EXP) {
            uint32_t w[LW / 2];
#pragma unroll
            for (uint32_t k = 0; k < LW / 4; ++k) {
                const uint32_t zz = zig8x4(d[k]), cc = (pv[k] >> 3) & 0x0F0F0F0Fu;
                w[2 * k] = __builtin_amdgcn_perm(cc, zz, 0x05010400u);
                w[2 * k + 1] = __builtin_amdgcn_perm(cc, zz, 0x07030602u);
            }
            *reinterpret_cast<uint4*>(tile_st) = make_uint4(w[0], w[1], w[2], w[3]);
        } else if constexpr (LW == 8) {
            *reinterpret_cast<uint2*>(tile_st) = make_uint2(d[0], d[1]);
        } else {
            *reinterpret_cast<uint4*>(tile_st) = make_uint4(d[0], d[1], d[2], d[3]);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (uint32_t c = 0; c < NC; ++c)
#pragma unroll
            for (uint32_t r = 0; r < kTileSteps; ++r) {
                if constexpr (EXP) z[c][r] = *reinterpret_cast<const uint16_t*>(tile_rd[c] + r * RL * 2);
                else z[c][r] = zig[tile_rd[c][r * RL]];
            }
        __builtin_amdgcn_wave_barrier();
    };
    // table entry of a position (EXP: class table, symbols past the table's n read its escape entry)
    auto entry = [&](uint32_t c, uint32_t zv) -> uint4 {
        if constexpr (EXP) return lenc[(zv >> 8) * cstride + min(zv & 0xFFu, fs - 1)];
        else return lenc[min(zv, n[c]) * RL + tl[c]];
    };

    for (uint32_t tb = ps.tb_begin + wave; tb < ps.tb_end; tb += nwave) {
        uint32_t ao[NC];
#pragma unroll
        for (uint32_t c = 0; c < NC; ++c) ao[c] = (tb - ps.tb_begin) * sstride + (2 * c + (upper ? 1u : 0u)) * (2 * RAW);
        const uint32_t lo = (tb * kSteps + ld_row) * rowb + ld_q;
        const uint32_t trow = kTileSteps * rowb;
        auto load = [&](uint32_t j, Row& tv, Row& pv) {
            if constexpr (LW == 8) {
                const auto t2 = __builtin_amdgcn_raw_buffer_load_b64(trs, lo, j * trow, 0);
                const auto p2 = __builtin_amdgcn_raw_buffer_load_b64(prs, lo, j * trow, 0);
                tv[0] = t2[0], tv[1] = t2[1], pv[0] = p2[0], pv[1] = p2[1];
            } else {
                const auto t4 = __builtin_amdgcn_raw_buffer_load_b128(trs, lo, j * trow, 0);
                const auto p4 = __builtin_amdgcn_raw_buffer_load_b128(prs, lo, j * trow, 0);
#pragma unroll
                for (uint32_t k = 0; k < 4; ++k) tv[k] = t4[k], pv[k] = p4[k];
            }
        };
        constexpr int kTiles = kSteps / kTileSteps;
        static_assert(kTiles % 2 == 0, "tiles are taken in pairs");

        uint32_t za[NC][kTileSteps], zb[NC][kTileSteps];
        Row tv, pv;
        load(kTiles - 1, tv, pv);
        stage(tv, pv, za);
        load(kTiles - 2, tv, pv);

        uint32_t x[NC], wp[NC], elo[NC], ehi[NC];         // wp: word counts, lower half | upper half << 16
        uint32_t escf[NC];                                 // EXP: entries' flags of the tile (bit 8: escape)
        uint4 ec[NC];
#pragma unroll
        for (uint32_t c = 0; c < NC; ++c) {
            x[c] = kStateLow;
            wp[c] = elo[c] = ehi[c] = 0;
            ec[c] = entry(c, za[c][kTileSteps - 1]);
        }
        // one tile: zc holds its symbols, zn receives the next tile's (two arrays that trade roles, so
        // no copy between tiles)
        auto tile_pass = [&](int j, uint32_t (&zc)[NC][kTileSteps], uint32_t (&zn)[NC][kTileSteps]) {
            if (j > 0) {
                stage(tv, pv, zn);
                if (j > 1) load(uint32_t(j - 2), tv, pv);
            }
#pragma unroll
            for (int r = kTileSteps - 1; r >= 0; --r) {
                uint32_t wn[NC], cross[NC];
#pragma unroll
                for (uint32_t c = 0; c < NC; ++c) {
                    const uint4 e = ec[c];
                    const uint32_t znext = r > 0 ? zc[c][r - 1] : zn[c][kTileSteps - 1];
                    ec[c] = entry(c, znext);
                    if constexpr (EXP) escf[c] = (r == kTileSteps - 1 ? 0u : escf[c]) | e.w;
                    // words leave before the state absorbs the symbol
                    // emit = x >= threshold, as a lane mask in vcc and a copy in mw; xs = x, or x >> 16
                    // where a word leaves (one select reading the high half of x).  A VALU read of an SGPR
                    // that a VALU wrote needs two wait states in between: the copy and one nop
                    uint32_t xs;
                    uint64_t mw;
                    asm("v_cmp_ge_u32_e32 vcc, %2, %3\n\t"
                        "s_mov_b64 %1, vcc\n\t"
                        "s_nop 0\n\t"
                        "v_cndmask_b32_sdwa %0, %2, %2, vcc dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
                        "src1_sel:WORD_1"
                        : "=v"(xs), "=s"(mw)
                        : "v"(x[c]), "v"(e.x)
                        : "vcc");
                    const uint32_t mlo = uint32_t(mw), mhi = uint32_t(mw >> 32);
                    const uint32_t plo = __popc(mlo);
                    const uint32_t pp = plo | (__popc(mhi) << 16);
                    // ring slot: this half's count plus the emitting lanes below it in the half, mod 128;
                    // an upper lane's mbcnt_lo counts every emitting lane of the lower half, which its
                    // base (the upper count less that number, formed on the scalar unit) takes back out
                    const uint32_t slot = __builtin_amdgcn_mbcnt_hi(
                        mhi, __builtin_amdgcn_mbcnt_lo(mlo, __builtin_amdgcn_ubfe(wp[c] - (plo << 16), fsh, 7)));
                    uint32_t ra;
                    asm("v_lshl_add_u32 %0, %1, 1, %2" : "=v"(ra) : "v"(slot & (kPairRing - 1)), "v"(ring_b[c]));
                    // the word is stored by the emitting lanes only (exec narrowed to mw and restored)
                    uint64_t keep;
                    asm volatile("s_and_saveexec_b64 %0, %1\n\t"
                                 "ds_write_b16 %2, %3\n\t"
                                 "s_or_b64 exec, exec, %0"
                                 : "=&s"(keep)
                                 : "s"(mw), "v"(ra), "v"(x[c])
                                 : "memory");
                    const uint32_t qt = __umulhi(xs + (e.z >> 24), e.y) >> (e.w & 31u);   // floor(xs / f)
                    // x = xs + qt (4096 - f) + start, the start taken from the high half of e.w
                    const uint32_t xq = __umul24(qt, e.z) + xs;
                    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
                        "src1_sel:WORD_1"
                        : "=v"(x[c]) : "v"(xq), "v"(e.w));
                    // a completed 64-word chunk leaves the ring (at most one per step and stream: bit 6
                    // of the half's count changes)
                    wn[c] = wp[c] + pp;
                    cross[c] = (wn[c] ^ wp[c]) & 0x00400040u;
                }
#pragma unroll
                for (uint32_t c = 0; c < NC; ++c) {
                    if (cross[c]) {
                        __builtin_amdgcn_wave_barrier();
                        const uint32_t ck = __builtin_amdgcn_ubfe(wp[c] >> 6, fsh, 10);
                        const uint32_t w = ring32[c][(ck & 1u) * 32 + hl];
                        const bool mine = __builtin_amdgcn_ubfe(cross[c], fsh + 6, 1) != 0;
                        __builtin_amdgcn_raw_buffer_store_b32(
                            w, wrs, mine && ck < kChunks ? ao[c] + RAW + ck * 128 + 4 * hl : kDrop, 0, 0);
                        __builtin_amdgcn_wave_barrier();
                    }
                    wp[c] = wn[c];
                }
            }
            // escaped values of this tile, in emission order (rare: skipped by the whole wavefront)
#pragma unroll
            for (uint32_t c = 0; c < NC; ++c) {
                if constexpr (EXP) {
                    if (__ballot((escf[c] & 0x100u) != 0) == 0) continue;
                } else {
                    uint32_t zm = zc[c][0];
#pragma unroll
                    for (uint32_t r = 1; r < kTileSteps; ++r) zm = max(zm, zc[c][r]);
                    if (__ballot(zm >= n[c]) == 0) continue;
                }
                // upper-half slots carry a bias of 32 (mbcnt_lo counts the whole lower half for them)
                const uint32_t ebase = ao[c] + kStreamHead - (upper ? 32u : 0u);
#pragma unroll
                for (int r = kTileSteps - 1; r >= 0; --r) {
                    const bool esc = EXP ? (zc[c][r] & 0xFFu) >= nq[zc[c][r] >> 8] : zc[c][r] >= n[c];
                    const uint64_t me = __ballot(esc);
                    if (me == 0) continue;
                    const uint32_t mlo = uint32_t(me), mhi = uint32_t(me >> 32), plo = __popc(mlo);
                    const uint32_t pk = min(elo[c], MAXE) | ((min(ehi[c], MAXE) + 32u - plo) << 16);
                    const uint32_t slot = __builtin_amdgcn_mbcnt_hi(
                        mhi, __builtin_amdgcn_mbcnt_lo(mlo, __builtin_amdgcn_ubfe(pk, fsh, 16)));
                    __builtin_amdgcn_raw_buffer_store_b8(uint8_t(zc[c][r]), wrs, esc ? ebase + slot : kDrop, 0, 0);
                    elo[c] += plo;
                    ehi[c] += __popc(mhi);
                }
            }
        };
        for (int j = kTiles - 1; j > 0; j -= 2) {
            tile_pass(j, za, zb);
            tile_pass(j - 1, zb, za);
        }
        // the partial last chunk, the final states and the streams' counts
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (uint32_t c = 0; c < NC; ++c) {
            const uint32_t cnt = __builtin_amdgcn_ubfe(wp[c], fsh, 16), ecnt = upper ? ehi[c] : elo[c];
            const uint32_t ck = cnt >> 6;
            const uint32_t w = ring32[c][(ck & 1u) * 32 + hl];
            __builtin_amdgcn_raw_buffer_store_b32(
                w, wrs, ck < kChunks && 2 * hl < (cnt & 63u) ? ao[c] + RAW + ck * 128 + 4 * hl : kDrop, 0, 0);
            reinterpret_cast<uint32_t*>(wgs + ao[c])[lane] = x[c];
            if (hl == 0) {
                const uint64_t sid = sid0 + uint64_t(tb - ps.tb_begin) * geo.ncg + 2 * c + (upper ? 1u : 0u);
                const uint32_t bytes = (kStreamHead + 2 * cnt + ecnt + 3) & ~3u;
                a.meta[sid] = bytes >= RAW ? 0x80000000u : (cnt | (ecnt << 14));
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// two channel groups with the slab's exponent-class tables; 512-thread workgroups, three per CU
// (the class bookkeeping needs more than the 64 registers of eight waves per SIMD)
constexpr uint32_t kExpEncThreads = 512;
__global__ __launch_bounds__(kExpEncThreads) __attribute__((amdgpu_waves_per_eu(6))) void encode_pairs_exp(
    EncodeLaunch a, DevTables t, uint32_t fs, LdsGeo lg) {
    encode_groups_body<1, true>(a, t, fs, lg);
}
// two channel groups, two workgroups per CU.  (Four groups, whole 128-byte lines read once by one
// wavefront, fit one workgroup per CU and measured slower: 1.94 ms against 1.75 ms on a
// 36 x 2 x 32768 x 1024 cache, the lost occupancy costing more than the line re-reads.)
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8))) void encode_pairs(EncodeLaunch a, DevTables t,
                                                                                          uint32_t fs, LdsGeo lg) {
    encode_groups_body<1>(a, t, fs, lg);
}

// --------------------------------------------------------------- tiled bf16 encode
// The tiled encoder for 16-bit elements: one channel group per workgroup, the
// two half-waves of a wavefront on two token blocks, 8-step tiles.  A lane
// loads 16 bytes of target and of predictor (8 channels of one token), forms
// the 8 zigzag symbols with 16-bit packed arithmetic (order-preserving flips,
// difference mod 2^16, zigzag) and stores them in the wavefront's LDS tile;
// each lane then reads its own channel's symbols for the tile's 8 steps.
// Emitted words go to a 128-word LDS ring per stream that stores each
// completed 64-word chunk at once; escaped values (16 bits) are stored per
// tile.  The tables of 256 symbols take 128 KB, so one workgroup runs per CU.
// EXP (exponent-class tables): the slab's 16 class tables in LDS, [class]
// [fs + 1] entries (an odd count, so the same symbol of different classes
// falls in different banks; entries past a table's n repeat its flagged
// escape entry), and 32-bit tile entries z | class << 16, the class formed
// from the predictor with packed 16-bit arithmetic.
constexpr uint32_t kBfTileLds = 2 * kTileSteps * kLanes * 2;            // symbols of both halves
constexpr uint32_t kBfEncWaveLds = kBfTileLds + 2 * kPairRing * 2;
__host__ __device__ constexpr uint32_t encode_bf16_lds(uint32_t fs) { return kLanes * fs * 16 + 16 * kBfEncWaveLds; }
constexpr uint32_t kBfTileLdsExp = 2 * kTileSteps * kLanes * 4;         // 32-bit entries of both halves
constexpr uint32_t kBfEncWaveLdsExp = kBfTileLdsExp + 2 * kPairRing * 2;
__host__ __device__ constexpr uint32_t encode_bf16_exp_lds(uint32_t fs) {
    return kExpClasses * (fs + 1) * 16 + 16 + 16 * kBfEncWaveLdsExp;
}

// v ^ 0x7FFF in each 16-bit half whose sign bit is set (the order-preserving
// code of a bf16 pattern is this flip ^ 0x8000); v_perm selectors 8 and 9
// spread the signs of bytes 1 and 3 over their halves
__device__ __forceinline__ uint32_t sflip16x2(uint32_t v) {
    return v ^ (__builtin_amdgcn_perm(v, v, 0x09090808u) & 0x7FFF7FFFu);
}
// zigzag symbols of two 16-bit residuals r (two's complement halves): 2r, or -2r - 1 when negative
__device__ __forceinline__ uint32_t zig16x2(uint32_t r) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    const us2 d = __builtin_bit_cast(us2, r) << us2{1, 1};
    return __builtin_bit_cast(uint32_t, d) ^ __builtin_amdgcn_perm(r, r, 0x09090808u);
}
// zigzag symbols of target - predictor for two bf16 patterns each
__device__ __forceinline__ uint32_t sym16x2(uint32_t t, uint32_t p) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    const us2 d = __builtin_bit_cast(us2, sflip16x2(t)) - __builtin_bit_cast(us2, sflip16x2(p));
    return zig16x2(__builtin_bit_cast(uint32_t, d));
}
// exponent classes of two bf16 predictors: min(max(E - base, 0), 15) per 16-bit half, E the
// exponent field (bits 14..7); base2 = base in both halves
__device__ __forceinline__ uint32_t cls16x2(uint32_t p, uint32_t base2) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    const us2 e = __builtin_bit_cast(us2, (p >> 7) & 0x00FF00FFu);
    const us2 c = __builtin_elementwise_sub_sat(e, __builtin_bit_cast(us2, base2));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(c, us2{15, 15}));
}

template <bool EXP>
__global__ __launch_bounds__(1024) void encode_bf16(EncodeLaunch a, DevTables t, uint32_t fs, LdsGeo lg) {
    constexpr uint32_t RAW = 2 * kSyms;
    constexpr uint32_t MAXE = (RAW - kStreamHead) / 2;
    constexpr uint32_t kDrop = 0x80000000u;               // buffer offset past the range: the access is dropped
    constexpr uint32_t kChunks = RAW / 128;                // 64-word chunks that fit the words region
    extern __shared__ __align__(16) uint8_t lds[];
    const Geo geo = geometry(a.shape);
    const LdsPos ps = lds_position(geo, lg);
    if (!ps.valid) return;
    const uint32_t tab0 = EXP ? ps.slab * kExpClasses : ps.slab * geo.C + ps.cg * kLanes;
    // tables: [fs symbols][32 lanes], or (EXP) [16 classes][fs + 1] then n of each class
    const uint32_t cstride = fs + 1;
    uint4* lenc = reinterpret_cast<uint4*>(lds);
    uint8_t* nq = lds + size_t(kExpClasses) * cstride * 16;
    if constexpr (EXP) {
        for (uint32_t i = threadIdx.x; i < kExpClasses * cstride; i += blockDim.x) {
            const uint32_t q = i / cstride, sym = i % cstride;
            lenc[i] = t.enc[size_t(tab0 + q) * 256 + min(sym, 255u)];
        }
        if (threadIdx.x < kExpClasses) nq[threadIdx.x] = uint8_t(t.n[tab0 + threadIdx.x]);
    } else {
        for (uint32_t i = threadIdx.x; i < kLanes * fs; i += blockDim.x) {
            const uint32_t sym = i / kLanes, j = i % kLanes;
            lenc[i] = t.enc[size_t(tab0 + j) * 256 + sym];
        }
    }
    __syncthreads();

    const uint32_t wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
    const uint32_t hl = threadIdx.x & 31u;
    const bool upper = (threadIdx.x & 32u) != 0;
    const uint32_t fsh = upper ? 16u : 0u;
    const uint32_t lane = 31u - hl;                        // format lane (reversed within the half)
    const uint32_t n = EXP ? 0u : t.n[tab0 + lane];
    constexpr uint32_t TE = EXP ? 4 : 2;                   // bytes of a tile entry
    constexpr uint32_t WLDS = EXP ? kBfEncWaveLdsExp : kBfEncWaveLds;
    uint8_t* tile = lds + (EXP ? size_t(kExpClasses) * cstride * 16 + 16 : size_t(kLanes) * fs * 16) + wave * WLDS;
    uint8_t* ring = tile + 2 * kTileSteps * kLanes * TE;
    // tile: [half][step][32 channels] entries; this lane loads 8 channels of one step and reads its channel back
    const uint32_t ld_row = hl >> 2, ld_q = hl & 3u;
    constexpr uint32_t kHalfTile = kTileSteps * kLanes * TE;
    uint4* tile_st = reinterpret_cast<uint4*>(tile + (upper ? kHalfTile : 0u) + ld_row * kLanes * TE + ld_q * 8 * TE);
    const uint8_t* tile_rd = tile + (upper ? kHalfTile : 0u) + lane * TE;
    const uint32_t base2 = EXP ? uint32_t(t.base[ps.slab]) * 0x00010001u : 0u;
    uint16_t* ring_h = reinterpret_cast<uint16_t*>(ring + (upper ? kPairRing * 2 : 0u));
    const uint32_t* ring32 = reinterpret_cast<const uint32_t*>(ring_h);

    const uint32_t rowb = geo.C * 2;
    const size_t slab_b = size_t(ps.slab) * geo.T * rowb + size_t(ps.cg) * kLanes * 2;
    const uint8_t* tgt = static_cast<const uint8_t*>(a.target) + slab_b + ld_q * 16;
    const uint8_t* aux = static_cast<const uint8_t*>(a.aux) + slab_b + ld_q * 16;
    const uint64_t sid0 = (uint64_t(ps.slab) * geo.ntb + ps.tb_begin) * geo.ncg + ps.cg;
    uint8_t* wgs = a.scratch + sid0 * (2 * RAW);
    const uint32_t sstride = geo.ncg * (2 * RAW);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        wgs, (short)0, int((ps.tb_end - ps.tb_begin - 1) * sstride + 2 * RAW), 0x00020000);

    // symbols of one tile: 8 per lane into LDS, then each lane's channel for the tile's 8 steps
    // (EXP: entries z | class << 16)
    auto stage = [&](uint4 tv, uint4 pv, uint32_t* z) {
        const uint4 zz = make_uint4(sym16x2(tv.x, pv.x), sym16x2(tv.y, pv.y), sym16x2(tv.z, pv.z), sym16x2(tv.w, pv.w));
        if constexpr (EXP) {
            const uint4 cc = make_uint4(cls16x2(pv.x, base2), cls16x2(pv.y, base2), cls16x2(pv.z, base2),
                                        cls16x2(pv.w, base2));
            tile_st[0] = make_uint4(__builtin_amdgcn_perm(cc.x, zz.x, 0x05040100u),
                                    __builtin_amdgcn_perm(cc.x, zz.x, 0x07060302u),
                                    __builtin_amdgcn_perm(cc.y, zz.y, 0x05040100u),
                                    __builtin_amdgcn_perm(cc.y, zz.y, 0x07060302u));
            tile_st[1] = make_uint4(__builtin_amdgcn_perm(cc.z, zz.z, 0x05040100u),
                                    __builtin_amdgcn_perm(cc.z, zz.z, 0x07060302u),
                                    __builtin_amdgcn_perm(cc.w, zz.w, 0x05040100u),
                                    __builtin_amdgcn_perm(cc.w, zz.w, 0x07060302u));
        } else {
            *tile_st = zz;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (uint32_t r = 0; r < kTileSteps; ++r)
            z[r] = EXP ? *reinterpret_cast<const uint32_t*>(tile_rd + r * kLanes * TE)
                       : *reinterpret_cast<const uint16_t*>(tile_rd + r * kLanes * TE);
        __builtin_amdgcn_wave_barrier();
    };
    // table entry of a position (EXP: the class table's, symbols past its n reading its escape entry)
    auto entry = [&](uint32_t zv) -> uint4 {
        if constexpr (EXP) return lenc[(zv >> 16) * cstride + min(zv & 0xFFFFu, fs - 1)];
        return lenc[min(zv, n) * kLanes + lane];
    };

    for (uint32_t r0 = ps.tb_begin + 2 * wave; r0 < ps.tb_end; r0 += 2 * nwave) {
        const uint32_t tb = r0 + (upper ? 1u : 0u);
        const bool act = tb < ps.tb_end;
        const uint32_t tbs = act ? tb : r0;
        const uint32_t ao = (tbs - ps.tb_begin) * sstride;
        const uint32_t ebase = ao + kStreamHead - (upper ? 64u : 0u);   // upper-half slots carry a bias of 32 values
        const uint32_t wreg = ao + RAW;
        const uint8_t* tsrc = tgt + size_t(tbs * kSteps + ld_row) * rowb;
        const uint8_t* psrc = aux + size_t(tbs * kSteps + ld_row) * rowb;
        const size_t tstride = size_t(kTileSteps) * rowb;
        constexpr int kTiles = kSteps / kTileSteps;

        uint32_t zc[kTileSteps], zn[kTileSteps];
        uint4 tv = *reinterpret_cast<const uint4*>(tsrc + (kTiles - 1) * tstride);
        uint4 pv = *reinterpret_cast<const uint4*>(psrc + (kTiles - 1) * tstride);
        stage(tv, pv, zc);
        tv = *reinterpret_cast<const uint4*>(tsrc + (kTiles - 2) * tstride);
        pv = *reinterpret_cast<const uint4*>(psrc + (kTiles - 2) * tstride);

        uint32_t x = kStateLow;
        uint32_t wp = 0;                                   // word counts: lower half | upper half << 16
        uint32_t elo = 0, ehi = 0;                         // escape counts per half
        uint4 ec = entry(zc[kTileSteps - 1]);
        for (int j = kTiles - 1; j >= 0; --j) {
            uint32_t escf = 0;                             // EXP: the tile's entry flags (bit 8: escape)
            if (j > 0) {
                stage(tv, pv, zn);
                if (j > 1) {
                    tv = *reinterpret_cast<const uint4*>(tsrc + size_t(j - 2) * tstride);
                    pv = *reinterpret_cast<const uint4*>(psrc + size_t(j - 2) * tstride);
                }
            }
#pragma unroll
            for (int r = kTileSteps - 1; r >= 0; --r) {
                const uint4 e = ec;
                const uint32_t znext = r > 0 ? zc[r - 1] : zn[kTileSteps - 1];
                ec = entry(znext);
                if constexpr (EXP) escf |= e.w;
                // words leave before the state absorbs the symbol (an idle half runs a copy of its
                // partner's stream into its own ring and stores nothing)
                uint32_t xs = x;
                const bool emit = xs >= e.x;
                const uint64_t mw = __ballot(emit);
                const uint32_t mlo = uint32_t(mw), mhi = uint32_t(mw >> 32);
                const uint32_t pp = __popc(mlo) | (__popc(mhi) << 16);
                // ring slot: this half's count mod 128 plus the emitting lanes below (mbcnt_lo counts the
                // entire lower half for an upper lane, which the packed base subtracts again)
                const uint32_t pk = (wp - (pp << 16)) & 0x007F007Fu;
                const uint32_t slot =
                    __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, __builtin_amdgcn_ubfe(pk, fsh, 16)));
                if (emit) ring_h[slot & (kPairRing - 1)] = uint16_t(xs & 0xFFFFu);
                xs = emit ? xs >> 16 : xs;
                const uint32_t qt = __umulhi(xs + (e.z >> 24), e.y) >> (e.w & 31u);   // floor(xs / f)
                // x = xs + qt (4096 - f) + start, the start taken from the high half of e.w
                const uint32_t xq = __umul24(qt, e.z) + xs;
                asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
                    : "=v"(x) : "v"(xq), "v"(e.w));
                // a completed 64-word chunk leaves the ring (at most one per step and stream)
                const uint32_t cross = ((wp & 0x003F003Fu) + pp) & 0x00400040u;
                if (cross) {
                    __builtin_amdgcn_wave_barrier();
                    const uint32_t ck = __builtin_amdgcn_ubfe(wp >> 6, fsh, 10);
                    const uint32_t w = ring32[(ck & 1u) * 32 + hl];
                    const bool mine = act && __builtin_amdgcn_ubfe(cross, fsh + 6, 1) != 0;
                    __builtin_amdgcn_raw_buffer_store_b32(
                        w, wrs, mine && ck < kChunks ? wreg + ck * 128 + 4 * hl : kDrop, 0, 0);
                    __builtin_amdgcn_wave_barrier();
                }
                wp += pp;
            }
            // escaped values of this tile, in emission order (rare: skipped by the whole wavefront)
            bool any;
            if constexpr (EXP) {
                any = (escf & 0x100u) != 0;
            } else {
                uint32_t zm = zc[0];
#pragma unroll
                for (uint32_t r = 1; r < kTileSteps; ++r) zm = max(zm, zc[r]);
                any = zm >= n;
            }
            if (__ballot(any) != 0) {
#pragma unroll
                for (int r = kTileSteps - 1; r >= 0; --r) {
                    const bool esc = EXP ? (zc[r] & 0xFFFFu) >= nq[zc[r] >> 16] : zc[r] >= n;
                    const uint64_t me = __ballot(esc);
                    if (me == 0) continue;
                    const uint32_t mlo = uint32_t(me), mhi = uint32_t(me >> 32), plo = __popc(mlo);
                    const uint32_t pk = min(elo, MAXE) | ((min(ehi, MAXE) + 32u - plo) << 16);
                    const uint32_t slot = __builtin_amdgcn_mbcnt_hi(
                        mhi, __builtin_amdgcn_mbcnt_lo(mlo, __builtin_amdgcn_ubfe(pk, fsh, 16)));
                    __builtin_amdgcn_raw_buffer_store_b16(uint16_t(zc[r] & 0xFFFFu), wrs,
                                                          act && esc ? ebase + 2 * slot : kDrop, 0, 0);
                    elo += plo;
                    ehi += __popc(mhi);
                }
            }
#pragma unroll
            for (uint32_t r = 0; r < kTileSteps; ++r) zc[r] = zn[r];
        }
        // the partial last chunk, the final states and the stream's counts
        __builtin_amdgcn_wave_barrier();
        const uint32_t cnt = __builtin_amdgcn_ubfe(wp, fsh, 16), ecnt = upper ? ehi : elo;
        const uint32_t ck = cnt >> 6;
        const uint32_t w = ring32[(ck & 1u) * 32 + hl];
        __builtin_amdgcn_raw_buffer_store_b32(
            w, wrs, act && ck < kChunks && 2 * hl < (cnt & 63u) ? wreg + ck * 128 + 4 * hl : kDrop, 0, 0);
        __builtin_amdgcn_wave_barrier();
        if (act) {
            reinterpret_cast<uint32_t*>(wgs + ao)[lane] = x;
            if (hl == 0) {
                const uint64_t sid = sid0 + uint64_t(tb - ps.tb_begin) * geo.ncg;
                const uint32_t bytes = (kStreamHead + 2 * cnt + 2 * ecnt + 3) & ~3u;
                a.meta[sid] = bytes >= RAW ? 0x80000000u : (cnt | (ecnt << 14));
            }
        }
    }
}

// --------------------------------------------------------------- tiled e4m3 decode
// One workgroup owns the 32 tables of a channel group: the complete
// slot -> symbol maps (4096 bytes per table) and per symbol the 16-bit
// values 4096 - frequency and start, so a pop is one map byte, two 16-bit
// reads and x' = x - (x >> 12) * (4096 - f) - start.  A map byte is the
// symbol's signed residual plus 128 (the escape symbol gets the byte its
// zigzag value would have), and the (4096 - f, start) rows are indexed by
// that byte, so the reconstruction needs no zigzag decode.  Each half wavefront runs
// one stream (kDecChains streams per half wavefront are supported; two chains
// hide more LDS latency but measured slower, the kernel being bound by its
// predictor and output traffic rather than by the chain).  Words come from a
// 128-word ring per stream in LDS, refilled with one 32-word chunk per 4-step
// tile; a chunk is requested one tile before it is written and predictor rows
// two tiles before they are used, so global loads are rarely waited for.  A
// tile whose steps needed a word the ring did not hold yet is decoded again
// from its saved state with words read from global memory.  A step only
// flags escapes; a tile with any escaped symbol ranks and reads them at its
// end.  Symbols of 4 steps then go through a 4 x 32 byte tile in LDS so that
// every lane reconstructs 4 channels of one token with bytewise arithmetic on
// 4-byte predictor loads and stores.
constexpr uint32_t kDecChains = 1;                           // streams per half wavefront
constexpr uint32_t kDecTile = 4;                             // steps per tile
constexpr uint32_t kDecRing = 128;                           // words per stream ring
constexpr uint32_t kDecChunk = 32;                           // words per ring chunk
constexpr uint32_t kDecSlots = kDecRing / kDecChunk;         // chunks a ring holds
constexpr uint32_t kDecSlotBits = 2;
constexpr uint32_t kDecFirst = 2;                            // chunk requested at the start of a stream
static_assert(kDecSlots == 4, "the ring upkeep assumes 4 chunks");
constexpr uint32_t kDecStreams = (1024 / 32) * kDecChains;   // streams in flight per workgroup
constexpr uint32_t kDecEscWin = 128;                         // bytes of escape region per stream held in a register

// LDS: maps [32][4096] | 4096 - f [fs][32] u16 | start [fs][32] u16 | rings [streams][RING words] | tiles [streams][4][32]
__host__ __device__ constexpr uint32_t dec_e4m3_rings(uint32_t fs) {
    return (kLanes * kM + 2 * fs * kLanes * 2 + 255) & ~255u;
}
__host__ __device__ constexpr uint32_t dec_e4m3_lds(uint32_t fs) {
    return dec_e4m3_rings(fs) + kDecStreams * (2 * kDecRing + kDecTile * kLanes);
}
// Exponent-class tables: maps [16 classes][4096] | 4096 - f [16][128] u16 | start [16][128] u16 | rings |
// tiles | class tiles [streams][32 lanes][4 steps] | n [16].  Rows cover residual bytes 64..191: byte 64
// (residual -64, zigzag 127) holds the escape symbol, which with at most 126 direct symbols is never a
// direct one, so escaped positions read 0x40 in every class.
constexpr uint32_t kExpRows = 128;
// a class's rows take 260 bytes, so that the same residual byte of different classes falls in
// different LDS banks
constexpr uint32_t kExpRowStride = kExpRows * 2 + 4;
constexpr uint32_t kExpRowBytes = kExpClasses * kExpRowStride;
constexpr uint32_t kExpEscByte = 128u - kExpRows / 2;
__host__ __device__ constexpr uint32_t dec_exp_rings() { return (kExpClasses * kM + 2 * kExpRowBytes + 255) & ~255u; }
__host__ __device__ constexpr uint32_t dec_exp_lds() {
    return dec_exp_rings() + kDecStreams * (2 * kDecRing + 2 * kDecTile * kLanes) + kExpClasses;
}

// bytewise helpers on 4 packed e4m3 codes / symbols
__device__ __forceinline__ uint32_t add8x4(uint32_t a, uint32_t b) {
    return ((a & 0x7F7F7F7Fu) + (b & 0x7F7F7F7Fu)) ^ ((a ^ b) & 0x80808080u);
}
// target codes from predictor codes and residual bytes b = r + 128: the
// order-preserving code of a byte is flip(u) ^ 0x80, so ord(t) = ord(p) + r
// mod 256 becomes flip(t) = flip(p) + (b ^ 0x80) mod 256 (flip is its own
// inverse), and a bytewise sum with b ^ 0x80 is the sum with b, ^ 0x80
__device__ __forceinline__ uint32_t recon8x4(uint32_t p, uint32_t b) {
    return sflip8x4(add8x4(sflip8x4(p), b) ^ 0x80808080u);
}
// residual byte r + 128 of a zigzag symbol value z < 256
__device__ __forceinline__ uint32_t rbyte(uint32_t z) { return (unzig(z) + 128u) & 0xFFu; }

// Rank of each flagged lane among the flagged lanes of its half plus the
// half's running count (lower half in bits 0..15 of C, upper half in bits
// 16..31); advances C.  `lowm` is all ones in the lower half and zero in the
// upper half, so an upper lane's mbcnt_lo sees none of the lower half's
// flags and no scalar work sits between the ballot and the rank.
__device__ __forceinline__ uint32_t half_rank(uint64_t m, uint32_t& C, uint32_t fsh, uint32_t lowm) {
    const uint32_t lo = uint32_t(m), hi = uint32_t(m >> 32);
    const uint32_t base = __builtin_amdgcn_ubfe(C, fsh, 16);
    C += uint32_t(__popc(lo)) | (uint32_t(__popc(hi)) << 16);
    return __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo & lowm, base));
}

// 0x80 in every byte of v that is zero, 0 elsewhere (exact per byte: no carry
// crosses a byte boundary)
__device__ __forceinline__ uint32_t zero_bytes(uint32_t v) {
    return ~(((v & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | v) & 0x80808080u;
}

// Decoder state of one chain: the lane's rANS state and the packed counts
// of words and escaped values consumed by the two streams of the chain.
struct DecState {
    uint32_t x, P, E;
};

struct DecLane {
    uint32_t mapb, gb, fsh, lowm;
    __amdgpu_buffer_rsrc_t rs;
};

struct DecChain {
    uint32_t ringb, tileb, woff;
};

// The steps of one tile for both chains.  GLOBAL = false takes words from the
// rings, GLOBAL = true from the streams in memory (a tile decoded again).  A
// step is written stage by stage over the two chains (map bytes, then table
// rows, then ring words) so that their LDS reads are in flight together, and
// it is branch-free: the refill select is a v_cndmask on the ballot mask,
// which keeps the ring read unconditional.  `pre` runs before the first
// step's map reads and `post` right after them, so work on the previous tile
// fills the wait for those reads.
//
// EXP (exponent-class tables): the maps and rows belong to the step's class,
// taken from cw (the lane's class byte of every step, class << 4): the map
// of class q sits at q * 4096 from mapb and its rows at q * kExpRowStride from gb.
template <bool GLOBAL, uint32_t FS, bool EXP = false, class Pre, class Post>
__device__ __forceinline__ void dec_tile_steps(DecState (&st)[kDecChains], const DecLane& L,
                                               const DecChain (&ch)[kDecChains], uint32_t (&sy)[kDecChains][kDecTile],
                                               Pre&& pre, Post&& post, const uint32_t (&cw)[kDecChains] = {}) {
#pragma unroll
    for (uint32_t r = 0; r < kDecTile; ++r) {
        uint32_t sym[kDecChains], g[kDecChains], cu[kDecChains], xn[kDecChains], idx[kDecChains], w[kDecChains];
        uint32_t mb[kDecChains], rb[kDecChains];
        uint64_t mw[kDecChains];
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            if constexpr (EXP) {
                const uint32_t q = __builtin_amdgcn_ubfe(cw[c], 8 * r + 4, 4);
                mb[c] = (q << 12) + L.mapb;
                rb[c] = q * kExpRowStride + L.gb;
            } else {
                mb[c] = L.mapb;
                rb[c] = L.gb;
            }
        }
        if (r == 0) pre();
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c)
            sym[c] = *reinterpret_cast<const lds_u8*>((st[c].x & (kM - 1u)) | mb[c]);
        if (r == 0) post();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            // the byte load already zero-extends; an empty asm hides the extension from the compiler
            asm("" : "+v"(sym[c]));
            // rows: [residual byte][32 lanes] per lane, or [class][128 residual bytes] shared
            const uint32_t ga = EXP ? (sym[c] << 1) + rb[c] : (sym[c] << 6) + rb[c];
            g[c] = *reinterpret_cast<const lds_u16*>(ga);                                       // 4096 - f
            cu[c] = *reinterpret_cast<const lds_u16*>(ga + (EXP ? kExpRowBytes : FS * kLanes * 2));  // start
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            xn[c] = st[c].x - (__umul24(st[c].x >> kProbBits, g[c]) + cu[c]);
            // refill in lane order
            mw[c] = __ballot(xn[c] < kStateLow);
            idx[c] = half_rank(mw[c], st[c].P, L.fsh, L.lowm);
            if (GLOBAL) w[c] = __builtin_amdgcn_raw_buffer_load_b16(L.rs, ch[c].woff + 2 * idx[c], 0, 0);
            else w[c] = *reinterpret_cast<const lds_u16*>(((idx[c] << 1) & (2 * kDecRing - 2)) | ch[c].ringb);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            uint32_t x;
            asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(x) : "v"(xn[c]), "v"((xn[c] << 16) | w[c]), "s"(mw[c]));
            st[c].x = x;
            sy[c][r] = sym[c];
        }
    }
}

template <uint32_t FS, bool EXP = false>
__global__ __launch_bounds__(1024, 1) void decode_e4m3(DecodeLaunch a, DevTables t, LdsGeo lg) {
    static_assert(!EXP || FS == kExpRows, "exponent-class rows cover 128 residual bytes");
    constexpr uint32_t OFF_G = EXP ? kExpClasses * kM : kLanes * kM;
    constexpr uint32_t OFF_C = EXP ? OFF_G + kExpRowBytes : OFF_G + FS * kLanes * 2;
    constexpr uint32_t OFF_R = EXP ? dec_exp_rings() : dec_e4m3_rings(FS);
    constexpr uint32_t OFF_T = OFF_R + kDecStreams * 2 * kDecRing;
    constexpr uint32_t OFF_K = OFF_T + kDecStreams * kDecTile * kLanes;     // class tiles (EXP)
    constexpr uint32_t OFF_N = OFF_K + kDecStreams * kDecTile * kLanes;     // n of each class (EXP)
    constexpr uint32_t kTiles = kSteps / kDecTile;
    extern __shared__ __align__(16) uint8_t lds[];
    const uint32_t lb = uint32_t(uintptr_t(lds));                  // LDS offset of the dynamic block
    const Geo geo = geometry(a.shape);
    const LdsPos ps = lds_position(geo, lg);
    if (!ps.valid) return;
    const uint32_t tid = threadIdx.x;
    const uint32_t tab0 = EXP ? ps.slab * kExpClasses : ps.slab * geo.C + ps.cg * kLanes;
    // rows by residual byte: row = r + FS/2 for the symbol of residual r (|r| < FS/2 when n < FS)
    constexpr uint32_t RB = 128u - FS / 2;                        // residual byte of row 0
    uint16_t* lg16 = reinterpret_cast<uint16_t*>(lds + OFF_G);    // [FS rows][32 lanes] or [16 classes][64 rows]
    uint16_t* lc16 = reinterpret_cast<uint16_t*>(lds + OFF_C);
    if constexpr (EXP) {
        for (uint32_t i = tid; i < kExpClasses * kExpRows; i += blockDim.x) {
            const uint32_t q = i / kExpRows, row = i % kExpRows;
            const uint32_t n = t.n[tab0 + q];
            // row 0 (residual byte 64) is the class's escape symbol
            const uint32_t z = row == 0 ? n : zig8((row + RB - 128u) & 0xFFu);
            const uint32_t fc = t.fc[size_t(tab0 + q) * 256 + z];
            lg16[q * (kExpRowStride / 2) + row] = uint16_t(kM - (fc & 0xFFFFu));
            lc16[q * (kExpRowStride / 2) + row] = uint16_t(fc >> 16);
        }
        if (tid < kExpClasses) lds[OFF_N + tid] = uint8_t(t.n[tab0 + tid]);
    } else {
        for (uint32_t i = tid; i < FS * kLanes; i += blockDim.x) {
            const uint32_t row = i / kLanes;
            const uint32_t z = zig8((row + RB - 128u) & 0xFFu);     // symbol of the row's residual
            const uint32_t fc = t.fc[size_t(tab0 + i % kLanes) * 256 + z];
            lg16[i] = uint16_t(kM - (fc & 0xFFFFu));
            lc16[i] = uint16_t(fc >> 16);                         // symbols past n: start 4096
        }
    }
    __syncthreads();
    if constexpr (EXP) {
        // the 16 class maps of the slab, contiguous in memory; a byte becomes the residual byte of its
        // symbol, the escape symbol's becomes 0x40
        const uint4* src = reinterpret_cast<const uint4*>(t.slot + size_t(tab0) * kM);
        uint4* dst = reinterpret_cast<uint4*>(lds);
        auto rb4 = [](uint32_t z) {
            const uint32_t l = z & 0x01010101u;
            return ((z >> 1) & 0x7F7F7F7Fu) ^ ((l << 8) - l) ^ 0x80808080u;
        };
#pragma unroll
        for (uint32_t k = 0; k < kExpClasses * kM / 16 / 1024; ++k) {
            const uint32_t e = k * 1024 + tid;
            const uint32_t n4 = (t.n[tab0 + e / (kM / 16)] & 0xFFu) * 0x01010101u;
            const uint4 v = src[e];
            auto cv = [&](uint32_t z) {
                const uint32_t m = (zero_bytes(z ^ n4) >> 7) * 0xFFu;   // bytes holding the escape symbol
                return (rb4(z) & ~m) | (kExpEscByte * 0x01010101u & m);
            };
            dst[e] = make_uint4(cv(v.x), cv(v.y), cv(v.z), cv(v.w));
        }
    } else {
        // maps: the 32 slot -> symbol tables of the group are contiguous in memory; each byte
        // becomes the residual byte of its symbol, unzig(z) + 128 = unzig(z) ^ 0x80, 4 at a time
        const uint4* src = reinterpret_cast<const uint4*>(t.slot + size_t(tab0) * kM);
        uint4* dst = reinterpret_cast<uint4*>(lds);
        auto rb4 = [](uint32_t z) {
            const uint32_t l = z & 0x01010101u;
            return ((z >> 1) & 0x7F7F7F7Fu) ^ ((l << 8) - l) ^ 0x80808080u;
        };
#pragma unroll
        for (uint32_t k = 0; k < kLanes * kM / 16 / 1024; ++k) {
            const uint4 v = src[k * 1024 + tid];
            dst[k * 1024 + tid] = make_uint4(rb4(v.x), rb4(v.y), rb4(v.z), rb4(v.w));
        }
    }
    __syncthreads();

    const uint32_t wave = tid >> 6, nwave = blockDim.x >> 6;
    const uint32_t hl = tid & 31u;
    const bool upper = (tid & 32u) != 0;
    const uint32_t r4 = hl >> 3, q4 = (hl & 7u) * 4;               // tile-domain row and byte column

    const uint32_t rowb = geo.C;
    const uint64_t* index = a.index;
    const uint8_t* pay = a.pay;
    const uint64_t sfirst = index_pos(a, ps.slab, ps.tb_begin, ps.cg, geo.ncg);
    const uint64_t slast = index_pos(a, ps.slab, ps.tb_end - 1, ps.cg, geo.ncg);
    const uint64_t wlo = index[sfirst] & ~kRawBit, whi = index[slast + 1] & ~kRawBit;
    if (whi < wlo || whi > a.payload_bytes || whi - wlo >= (1ull << 31)) {
        if (tid == 0) atomicOr(a.status, 1u);
        return;
    }
    DecLane L;
    if constexpr (EXP) {
        L.mapb = lb;                                               // class q's map at q * 4096
        L.gb = lb + OFF_G - RB * 2;                                // class q, residual byte b at q * 260 + b * 2 + gb
    } else {
        L.mapb = lb + hl * kM;
        L.gb = lb + OFF_G + hl * 2 - RB * kLanes * 2;              // row of residual byte b at b * 64 + gb
    }
    L.fsh = upper ? 16u : 0u;
    L.lowm = upper ? 0u : 0xFFFFFFFFu;
    // every payload read of the workgroup goes through one range-checked resource
    L.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pay + wlo), (short)0, int(whi - wlo), 0x00020000);
    // tile-domain bytes: the escape symbol's map byte and n of the lane's 4 channels (exponent
    // classes: 0x40 in every class; n by the position's class)
    uint32_t escp = 0, np = 0;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        const uint32_t nk = EXP ? 0u : t.n[tab0 + q4 + k];
        escp |= (EXP ? kExpEscByte : rbyte(nk)) << (8 * k);
        np |= min(nk, 255u) << (8 * k);
    }
    // predictor and output rows of the slab's channel group, 32-bit offsets from one base each
    const size_t slab_b = size_t(ps.slab) * geo.T * rowb + size_t(ps.cg) * kLanes;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const uint8_t*>(a.aux) + slab_b)), (short)0,
        int(uint32_t(geo.T - 1) * rowb + kLanes), 0x00020000);
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<void*>(static_cast<uint8_t*>(a.out) + slab_b), (short)0, int(uint32_t(geo.T - 1) * rowb + kLanes),
        0x00020000);
    bool bad = false;

    // index entries of a round's streams, requested one round ahead (an absent stream reads the
    // entries of the workgroup's last stream)
    constexpr uint32_t kRound = 2 * kDecChains;
    uint64_t ix0[kDecChains], ix1[kDecChains];
    auto fetch_index = [&](uint32_t tb0) {
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            const uint32_t tbc = min(tb0 + 2 * c + (upper ? 1u : 0u), ps.tb_end - 1);
            const uint64_t sid = index_pos(a, ps.slab, tbc, ps.cg, geo.ncg);
            ix0[c] = index[sid];
            ix1[c] = index[sid + 1];
        }
    };
    fetch_index(ps.tb_begin + kRound * wave);
    uint32_t padv = 0;                              // pad bytes of the previous round, checked late

    for (uint32_t tb0 = ps.tb_begin + kRound * wave; tb0 < ps.tb_end; tb0 += kRound * nwave) {
        DecChain ch[kDecChains];
        DecState st[kDecChains];
        uint32_t tb[kDecChains], nw[kDecChains], size[kDecChains], rel[kDecChains];
        uint32_t cw[kDecChains], pva[kDecChains], pvb[kDecChains], rowo[kDecChains];
        uint32_t ew[kDecChains], ea[kDecChains], ewr[kDecChains];
        // ring upkeep, both halves packed (lower in bits 0..15): ldk = chunk held in cw,
        // wrk = last chunk written to the ring, live = 0x8000 in the field of a half with
        // a coded stream
        uint32_t ldk[kDecChains], wrk[kDecChains], live[kDecChains];
        uint32_t ktb[kDecChains], cls[kDecChains];                 // class tile base, class word (EXP)
        bool coded[kDecChains], raw[kDecChains];
        uint64_t e0[kDecChains], e1[kDecChains];
        uint32_t x0[kDecChains], c0[kDecChains], c1[kDecChains];
        // every header and ring load of the round is issued before any of them is checked
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            e0[c] = ix0[c];
            e1[c] = ix1[c];
            const uint64_t o = e0[c] & ~kRawBit;
            rel[c] = o >= wlo && o - wlo < (1ull << 31) ? uint32_t(o - wlo) : 0u;
            nw[c] = __builtin_amdgcn_raw_buffer_load_b32(L.rs, rel[c] + 128, 0, 0);
            x0[c] = __builtin_amdgcn_raw_buffer_load_b32(L.rs, rel[c] + 4 * hl, 0, 0);
            const uint32_t woff = rel[c] + kStreamHead;
            c0[c] = __builtin_amdgcn_raw_buffer_load_b16(L.rs, woff + 2 * hl, 0, 0);
            c1[c] = __builtin_amdgcn_raw_buffer_load_b16(L.rs, woff + 2 * kDecChunk + 2 * hl, 0, 0);
            cw[c] = __builtin_amdgcn_raw_buffer_load_b16(L.rs, woff + 2 * kDecChunk * kDecFirst + 2 * hl, 0, 0);
        }
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            tb[c] = tb0 + 2 * c + (upper ? 1u : 0u);
            // byte offset of this lane's first tile-domain row; an absent stream reads rows of tb0
            rowo[c] = ((tb[c] < ps.tb_end ? tb[c] : tb0) * kSteps + r4) * rowb + q4;
            pva[c] = __builtin_amdgcn_raw_buffer_load_b32(prs, rowo[c], 0, 0);
            pvb[c] = __builtin_amdgcn_raw_buffer_load_b32(prs, rowo[c] + kDecTile * rowb, 0, 0);
        }
        if (tb0 + kRound * nwave < ps.tb_end) fetch_index(tb0 + kRound * nwave);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            const uint32_t hs = (tid >> 5) * kDecChains + c;          // stream slot in the workgroup
            ch[c].ringb = lb + OFF_R + hs * 2 * kDecRing;             // 256-byte aligned
            ch[c].tileb = lb + OFF_T + hs * kDecTile * kLanes + hl;
            ktb[c] = lb + OFF_K + hs * kDecTile * kLanes;
            // ---- stream header checks (every lane of the half holds the same entries)
            uint32_t x = kStateLow;
            size[c] = 0;
            coded[c] = raw[c] = false;
            if (tb[c] < ps.tb_end) {
                const uint64_t o = e0[c] & ~kRawBit, end = e1[c] & ~kRawBit;
                if (end < o || o < wlo || end > whi) {
                    bad = true;
                } else if (e0[c] & kRawBit) {
                    if (end - o != kSyms) bad = true;
                    else raw[c] = true;
                } else {
                    size[c] = uint32_t(end - o);
                    if (size[c] < kStreamHead || size[c] % 4 != 0 || nw[c] > (size[c] - kStreamHead) / 2) {
                        bad = true;
                    } else {
                        coded[c] = true;
                        x = x0[c];
                        if (x < kStateLow) bad = true;
                    }
                }
            }
            if (!coded[c]) nw[c] = 0;
            const uint64_t cm = __ballot(coded[c]);
            live[c] = (uint32_t(cm) ? 0x8000u : 0u) | ((cm >> 32) ? 0x80000000u : 0u);
            // word offset in the window (a stream that is not coded reads from the window start)
            const uint32_t woff = coded[c] ? rel[c] + kStreamHead : 0u;
            ch[c].woff = woff;
            // escape window: the 4-byte aligned dwords from the start of the escape region (which
            // sits 0 or 2 bytes past a dword boundary); a stream's dwords never cross its padded end
            ea[c] = (woff + 2 * nw[c]) & 3u;
            ew[c] = __builtin_amdgcn_raw_buffer_load_b32(L.rs, ((woff + 2 * nw[c]) & ~3u) + 4 * hl, 0, 0);
            // ring: chunk k (words [32k, 32k + 32)) sits in slot k % slots; chunks 0 and 1 now,
            // the next one (chunk 1 again for a 2-chunk ring) requested for the first tile end
            lds_u16* ring16 = reinterpret_cast<lds_u16*>(ch[c].ringb);
            ring16[hl] = c0[c];
            ring16[kDecChunk + hl] = c1[c];
            ldk[c] = kDecFirst * 0x00010001u;
            wrk[c] = 0x00010001u;
            st[c] = DecState{x, 0u, 0u};
            ewr[c] = 0;
        }
        if (padv != 0) bad = true;
        __builtin_amdgcn_wave_barrier();

        // A tile's symbols go to the tile buffer at the end of its steps; the next tile's first
        // step reads them back transposed (lane hl: step r4, lanes q4..q4+3 of its half, so the
        // lanes of a half and the bytes of a lane run in decode order), resolves escaped values,
        // reconstructs and stores the rows and reloads pv with the row two tiles ahead.
        // EXP: the classes of a tile go through the class tile (the lane's predictor row r4, bytes q4..q4+3
        // in, the lane's own channel's 4 steps out); a class byte holds class << 4
        auto put_classes = [&](const uint32_t (&pv)[kDecChains]) {
            if constexpr (EXP) {
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c) {
                    const uint32_t v = (pv[c] << 1) & 0xF0F0F0F0u;
#pragma unroll
                    for (uint32_t j = 0; j < 4; ++j)
                        *reinterpret_cast<lds_u8*>(ktb[c] + (q4 + j) * kDecTile + r4) = uint8_t(v >> (8 * j));
                }
            }
        };
        auto get_classes = [&]() {
            if constexpr (EXP) {
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c)
                    cls[c] = *reinterpret_cast<const lds_u32*>(ktb[c] + hl * kDecTile);
            }
        };
        uint32_t zt[kDecChains];
        auto fetch_tile = [&]() {
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c)
                zt[c] = *reinterpret_cast<const lds_u32*>(ch[c].tileb - hl + r4 * kLanes + q4);
        };
        auto finish = [&](uint32_t T, uint32_t (&pv)[kDecChains]) {
            uint32_t ef[kDecChains];
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) ef[c] = zero_bytes(zt[c] ^ escp);
            uint32_t efa = 0;
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) efa |= ef[c];
            if (__builtin_expect(__ballot(efa != 0) != 0, 0)) {
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c) {
                    const uint64_t m1 = __ballot(ef[c] != 0);
                    if (m1 == 0) continue;
                    // index of the lane's first escaped value in the stream's escape region: the
                    // half's count so far plus the values of lower lanes (usually one per lane)
                    uint32_t E1 = 0;
                    uint32_t eidx = __builtin_amdgcn_ubfe(st[c].E, L.fsh, 16) + half_rank(m1, E1, L.fsh, L.lowm);
                    st[c].E += E1;
                    uint32_t f = ef[c], v = zt[c];
                    if (__ballot((f & (f - 1u)) != 0) != 0) {
                        const uint32_t cnt = __popc(f);
                        for (uint32_t j = 1; j < 4; ++j) {
                            const uint64_t m = __ballot(cnt > j);
                            if (m == 0) break;
                            uint32_t E = 0;
                            eidx += half_rank(m, E, L.fsh, L.lowm);
                            st[c].E += E;
                        }
                    }
                    // the lane's escaped bytes in order; the first 128 bytes of a stream's escape
                    // region come from the window register, later ones from memory
                    do {
                        const uint32_t sh = (__builtin_ctz(f | 0x80000000u) >> 3) * 8;   // byte of the value
                        const uint32_t pos = eidx + ea[c];
                        const uint32_t wv = __builtin_amdgcn_ds_bpermute(
                            int(((pos >> 2) + (upper ? 32u : 0u)) << 2), int(ewr[c]));
                        uint32_t e = (wv >> ((pos & 3u) * 8)) & 0xFFu;
                        if (__ballot(f != 0 && pos >= kDecEscWin) != 0) {
                            const uint32_t g = __builtin_amdgcn_raw_buffer_load_b8(
                                L.rs, ch[c].woff + 2 * nw[c] + eidx, 0, 0);
                            e = pos >= kDecEscWin ? g : e;
                        }
                        if (f != 0) {
                            // a canonical encoder codes a value below n directly
                            const uint32_t nv = EXP ? uint32_t(*reinterpret_cast<const lds_u8*>(
                                                          lb + OFF_N + ((pv[c] >> (sh + 3)) & 0xFu)))
                                                    : (np >> sh) & 0xFFu;
                            if (coded[c] && e < nv) bad = true;
                            v = (v & ~(0xFFu << sh)) | (rbyte(e) << sh);
                            f &= f - 1u;
                            ++eidx;
                        }
                    } while (__ballot(f != 0) != 0);
                    zt[c] = v;
                }
            }
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) {
                if (coded[c])
                    __builtin_amdgcn_raw_buffer_store_b32(recon8x4(pv[c], zt[c]), ors, rowo[c], T * kDecTile * rowb, 0);
                if (T + 2 < kTiles)
                    pv[c] = __builtin_amdgcn_raw_buffer_load_b32(prs, rowo[c], (T + 2) * kDecTile * rowb, 0);
            }
        };
        // one tile: its steps (with the previous tile's finish inside the first one), its symbols
        // to the tile buffer, ring upkeep; pvp holds the previous tile's predictor row
        auto tile_at = [&](uint32_t T, uint32_t (&pvp)[kDecChains]) {
            if (T == 1) {
                // the window dword again, written by a VALU move: its load is waited for once, here,
                // and not in the escape path, where the wait would also cover every later load (the
                // predictor rows requested two tiles ahead)
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c) asm volatile("v_mov_b32 %0, %1" : "=v"(ewr[c]) : "v"(ew[c]));
            }
            uint32_t sy[kDecChains][kDecTile];
            DecState s0[kDecChains];
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) s0[c] = st[c];
            get_classes();
            __builtin_amdgcn_wave_barrier();
            dec_tile_steps<false, FS, EXP>(
                st, L, ch, sy, [&] { if (T > 0) fetch_tile(); }, [&] { if (T > 0) finish(T - 1, pvp); }, cls);
            // a half of a coded stream that read past the last chunk written (word count above
            // 32 (wrk + 1) in its field) decodes the tile again from memory
            uint32_t over = 0;
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c)
                over |= ~((wrk[c] << 5) + 0x80208020u - st[c].P) & live[c];
            if (__builtin_expect(over != 0, 0)) {
                // the escape count keeps what the previous tile's finish added meanwhile
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c) {
                    st[c].x = s0[c].x;
                    st[c].P = s0[c].P;
                }
                dec_tile_steps<true, FS, EXP>(st, L, ch, sy, [] {}, [] {}, cls);
            }
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c)
#pragma unroll
                for (uint32_t r = 0; r < kDecTile; ++r)
                    *reinterpret_cast<lds_u8*>(ch[c].tileb + r * kLanes) = uint8_t(sy[c][r]);
            // the next tile's classes: its predictor row is in pvp (the initial load after tile 0, the
            // reload of the finish above after later tiles)
            if (T + 1 < kTiles) put_classes(pvp);
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) {
                // the chunk in cw goes into its slot; the next one is requested while the ring
                // has a free slot (chunk ldk + 1 fits when ldk <= words consumed / 32 + slots - 2)
                reinterpret_cast<lds_u16*>(ch[c].ringb)[__builtin_amdgcn_ubfe(ldk[c], L.fsh, kDecSlotBits) * kDecChunk + hl] =
                    cw[c];
                wrk[c] = ldk[c];
                const uint32_t room = ((st[c].P >> 5) & 0x07FF07FFu) + (0x8000u + kDecSlots - 2) * 0x00010001u - ldk[c];
                ldk[c] += (room >> 15) & 0x00010001u;
                cw[c] = __builtin_amdgcn_raw_buffer_load_b16(
                    L.rs, ch[c].woff + 2 * kDecChunk * __builtin_amdgcn_ubfe(ldk[c], L.fsh, 16) + 2 * hl, 0, 0);
            }
            __builtin_amdgcn_wave_barrier();
        };
        put_classes(pva);
        __builtin_amdgcn_wave_barrier();
        for (uint32_t T = 0; T < kTiles; T += 2) {
            tile_at(T, pvb);
            tile_at(T + 1, pva);
        }
        fetch_tile();
        finish(kTiles - 1, pvb);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            // ---- stream checks: states back at L, every word and escape consumed, zero pad
            if (coded[c]) {
                const uint32_t pc = __builtin_amdgcn_ubfe(st[c].P, L.fsh, 16);
                const uint32_t ec = __builtin_amdgcn_ubfe(st[c].E, L.fsh, 16);
                const uint32_t used = kStreamHead + 2 * nw[c] + ec;
                if (st[c].x != kStateLow || pc != nw[c] || used > size[c]) bad = true;
                else if (((used + 3) & ~3u) != size[c]) bad = true;
                // the pad bytes are read now and checked at the next round's start
                padv |= __builtin_amdgcn_raw_buffer_load_b8(L.rs, hl < size[c] - used ? rel[c] + used + hl : 0x80000000u,
                                                            0, 0);
            }
            if (raw[c]) {
                // raw stream: its 4096 codes in (step, lane) order, copied row by row
                for (uint32_t T = 0; T < kTiles; ++T) {
                    const uint32_t k = T * kDecTile + r4;
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __builtin_amdgcn_raw_buffer_load_b32(L.rs, rel[c] + k * kLanes + q4, 0, 0), ors,
                        rowo[c] + T * kDecTile * rowb, 0, 0);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (bad || padv != 0) atomicOr(a.status, 1u);
}

// --------------------------------------------------------------- tiled bf16 decode
// The e4m3 decoder's structure (word rings, tile transposition, escapes
// resolved once per tile) for 16-bit elements, whose tables use up to 255
// direct symbols.  The 32 slot -> symbol maps would not fit next to 257-row
// tables, so each map keeps the symbol of every even slot (2048 bytes per
// table); the odd slot belongs to that symbol or to the next one, which then
// starts there, so a step reads the rows of both and keeps the second when the
// slot is at or past its start.  Rows are indexed by symbol (the escape
// symbol is n), the 4 symbols of a tile row go through 16-bit arithmetic
// (zigzag decode, order-preserving map, residual add mod 2^16) two per dword,
// and predictor and output rows move 8 bytes per lane.
constexpr uint32_t kBf16Rows = 257;                          // 256 symbols and a sentinel
// a bf16 stream uses about 40 words per tile, so its ring takes 64-word chunks (two words per lane)
constexpr uint32_t kBfChunk = 64;                            // words per ring chunk
constexpr uint32_t kBfRing = 256;                            // words per stream ring (4 chunks)
constexpr uint32_t kBfSlots = kBfRing / kBfChunk;
constexpr uint32_t kBfFirst = 2;                             // chunk requested at the start of a stream
__host__ __device__ constexpr uint32_t dec_bf16_rings() { return (kLanes * (kM / 2) + kBf16Rows * kLanes * 4 + 511) & ~511u; }
__host__ __device__ constexpr uint32_t dec_bf16_lds() {
    return dec_bf16_rings() + kDecStreams * (2 * kBfRing + kDecTile * kLanes);
}
// Exponent-class tables: half maps [16 classes][2048] | rows [16 classes][257] u32 | rings | tiles |
// class tiles [streams][32 channels][4 steps] | n [16]
constexpr uint32_t kBfExpRowStride = kBf16Rows * 4;     // 1028 bytes: a class's rows start one bank further
__host__ __device__ constexpr uint32_t dec_bf16_exp_rings() {
    return (kExpClasses * (kM / 2) + kExpClasses * kBfExpRowStride + 511) & ~511u;
}
__host__ __device__ constexpr uint32_t dec_bf16_exp_lds() {
    return dec_bf16_exp_rings() + kDecStreams * (2 * kBfRing + 2 * kDecTile * kLanes) + kExpClasses;
}

__device__ __forceinline__ uint2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ void st8(uint2 v, __amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    const v2u w = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, soff, 0);
}
// targets of two predictor values and two zigzag symbols: ord(t) = ord(p) + r
// mod 2^16 is flip(t) = flip(p) + r mod 2^16
__device__ __forceinline__ uint32_t recon16x2(uint32_t p, uint32_t z) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    const uint32_t r = ((z >> 1) & 0x7FFF7FFFu) ^ __umul24(z & 0x00010001u, 0xFFFFu);
    const us2 s = __builtin_bit_cast(us2, sflip16x2(p)) + __builtin_bit_cast(us2, r);
    return sflip16x2(__builtin_bit_cast(uint32_t, s));
}

// The steps of one tile (see dec_tile_steps); the map lookup reads the rows of
// the even slot's symbol and of the next symbol.  EXP: a step's class (from
// the class word, class << 4 per step byte) picks the half map and the rows.
template <bool GLOBAL, bool EXP = false, class Pre, class Post>
__device__ __forceinline__ void dec_tile_steps_bf16(DecState (&st)[kDecChains], const DecLane& L,
                                                    const DecChain (&ch)[kDecChains],
                                                    uint32_t (&sy)[kDecChains][kDecTile], Pre&& pre, Post&& post,
                                                    const uint32_t (&cw)[kDecChains] = {}) {
#pragma unroll
    for (uint32_t r = 0; r < kDecTile; ++r) {
        uint32_t s0[kDecChains], e0[kDecChains], e1[kDecChains], xn[kDecChains], idx[kDecChains], w[kDecChains];
        uint32_t mb[kDecChains], rb[kDecChains];
        uint64_t mw[kDecChains];
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            if constexpr (EXP) {
                const uint32_t q = __builtin_amdgcn_ubfe(cw[c], 8 * r + 4, 4);
                mb[c] = (q << 11) + L.mapb;
                rb[c] = q * kBfExpRowStride + L.gb;
            } else {
                mb[c] = L.mapb;
                rb[c] = L.gb;
            }
        }
        if (r == 0) pre();
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c)
            s0[c] = *reinterpret_cast<const lds_u8*>(__builtin_amdgcn_ubfe(st[c].x, 1, 11) | mb[c]);
        if (r == 0) post();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            asm("" : "+v"(s0[c]));
            // rows: [symbol][32 lanes] per lane, or [class][257 symbols] shared
            const uint32_t ra = EXP ? (s0[c] << 2) + rb[c] : (s0[c] << 7) + rb[c];
            e0[c] = *reinterpret_cast<const lds_u32*>(ra);
            e1[c] = *reinterpret_cast<const lds_u32*>(ra + (EXP ? 4u : kLanes * 4));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            const bool adv = (st[c].x & (kM - 1u)) >= (e1[c] >> 16);
            const uint32_t e = adv ? e1[c] : e0[c];
            sy[c][r] = s0[c] + (adv ? 1u : 0u);
            // x - (x >> 12) (4096 - f) - start, both from the row word
            uint32_t m, y;
            asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
                : "=v"(m) : "v"(st[c].x >> kProbBits), "v"(e));
            asm("v_sub_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
                : "=v"(y) : "v"(st[c].x - m), "v"(e));
            xn[c] = y;
            mw[c] = __ballot(xn[c] < kStateLow);
            idx[c] = half_rank(mw[c], st[c].P, L.fsh, L.lowm);
            if (GLOBAL) w[c] = __builtin_amdgcn_raw_buffer_load_b16(L.rs, ch[c].woff + 2 * idx[c], 0, 0);
            else w[c] = *reinterpret_cast<const lds_u16*>(((idx[c] << 1) & (2 * kBfRing - 2)) | ch[c].ringb);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            uint32_t x;
            asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(x) : "v"(xn[c]), "v"((xn[c] << 16) | w[c]), "s"(mw[c]));
            st[c].x = x;
        }
    }
}

template <bool EXP>
__global__ __launch_bounds__(1024, 1) void decode_bf16(DecodeLaunch a, DevTables t, LdsGeo lg) {
    constexpr uint32_t NT = EXP ? kExpClasses : kLanes;           // tables held
    constexpr uint32_t OFF_G = NT * (kM / 2);
    constexpr uint32_t OFF_R = EXP ? dec_bf16_exp_rings() : dec_bf16_rings();
    constexpr uint32_t OFF_T = OFF_R + kDecStreams * 2 * kBfRing;
    constexpr uint32_t OFF_K = OFF_T + kDecStreams * kDecTile * kLanes;     // class tiles (EXP)
    constexpr uint32_t OFF_N = OFF_K + kDecStreams * kDecTile * kLanes;     // n of each class (EXP)
    constexpr uint32_t kTiles = kSteps / kDecTile;
    extern __shared__ __align__(16) uint8_t lds[];
    const uint32_t lb = uint32_t(uintptr_t(lds));                  // LDS offset of the dynamic block
    const Geo geo = geometry(a.shape);
    const LdsPos ps = lds_position(geo, lg);
    if (!ps.valid) return;
    const uint32_t tid = threadIdx.x;
    const uint32_t tab0 = EXP ? ps.slab * kExpClasses : ps.slab * geo.C + ps.cg * kLanes;
    // rows by symbol: (4096 - f) | start << 16; symbols past n and the sentinel row 256 start at 4096
    uint32_t* lrow = reinterpret_cast<uint32_t*>(lds + OFF_G);           // [257 rows][32 lanes] or [16][257]
    for (uint32_t i = tid; i < kBf16Rows * NT; i += blockDim.x) {
        const uint32_t row = EXP ? i % kBf16Rows : i / kLanes, tq = EXP ? i / kBf16Rows : i % kLanes;
        const uint32_t fc = row < 256 ? t.fc[size_t(tab0 + tq) * 256 + row] : (kM << 16);
        lrow[i] = (kM - (fc & 0xFFFFu)) | (fc & 0xFFFF0000u);
    }
    if (EXP && tid < kExpClasses) lds[OFF_N + tid] = uint8_t(min(t.n[tab0 + tid], 255u));
    {
        // half maps: the symbol of every even slot (the odd slot belongs to the same symbol or
        // to the next one, which then starts there), from the group's (or the slab's class
        // tables') contiguous slot maps
        const uint4* src = reinterpret_cast<const uint4*>(t.slot + size_t(tab0) * kM);
        uint2* dst = reinterpret_cast<uint2*>(lds);
#pragma unroll
        for (uint32_t q = 0; q < NT * kM / 16 / 1024; ++q) {
            const uint4 v = src[q * 1024 + tid];
            dst[q * 1024 + tid] = make_uint2(__builtin_amdgcn_perm(v.y, v.x, 0x06040200u),
                                             __builtin_amdgcn_perm(v.w, v.z, 0x06040200u));
        }
    }
    __syncthreads();

    const uint32_t wave = tid >> 6, nwave = blockDim.x >> 6;
    const uint32_t hl = tid & 31u;
    const bool upper = (tid & 32u) != 0;
    const uint32_t r4 = hl >> 3, q4 = (hl & 7u) * 4;               // tile-domain row and byte column

    const uint32_t rowb = geo.C * 2;
    const uint64_t* index = a.index;
    const uint8_t* pay = a.pay;
    const uint64_t sfirst = index_pos(a, ps.slab, ps.tb_begin, ps.cg, geo.ncg);
    const uint64_t slast = index_pos(a, ps.slab, ps.tb_end - 1, ps.cg, geo.ncg);
    const uint64_t wlo = index[sfirst] & ~kRawBit, whi = index[slast + 1] & ~kRawBit;
    if (whi < wlo || whi > a.payload_bytes || whi - wlo >= (1ull << 31)) {
        if (tid == 0) atomicOr(a.status, 1u);
        return;
    }
    DecLane L;
    L.mapb = EXP ? lb : lb + hl * (kM / 2);                        // EXP: class q's half map at q * 2048
    L.gb = EXP ? lb + OFF_G : lb + OFF_G + hl * 4;                  // row z at z * 128 + gb (EXP: q * 1028 + z * 4)
    L.fsh = upper ? 16u : 0u;
    L.lowm = upper ? 0u : 0xFFFFFFFFu;
    // every payload read of the workgroup goes through one range-checked resource
    L.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pay + wlo), (short)0, int(whi - wlo), 0x00020000);
    // tile-domain bytes: n (the escape symbol) of the lane's 4 channels (EXP: by each position's
    // class, formed per tile from its predictors)
    uint32_t np = 0;
    if constexpr (!EXP) {
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) np |= min(t.n[tab0 + q4 + k], 255u) << (8 * k);
    }
    const uint32_t base2 = EXP ? uint32_t(t.base[ps.slab]) * 0x00010001u : 0u;
    // predictor and output rows of the slab's channel group, 32-bit offsets from one base each
    const size_t slab_b = size_t(ps.slab) * geo.T * rowb + size_t(ps.cg) * kLanes * 2;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const uint8_t*>(a.aux) + slab_b)), (short)0,
        int(uint32_t(geo.T - 1) * rowb + 2 * kLanes), 0x00020000);
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<void*>(static_cast<uint8_t*>(a.out) + slab_b), (short)0,
        int(uint32_t(geo.T - 1) * rowb + 2 * kLanes), 0x00020000);
    bool bad = false;

    // index entries of a round's streams, requested one round ahead (an absent stream reads the
    // entries of the workgroup's last stream)
    constexpr uint32_t kRound = 2 * kDecChains;
    uint64_t ix0[kDecChains], ix1[kDecChains];
    auto fetch_index = [&](uint32_t tb0) {
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            const uint32_t tbc = min(tb0 + 2 * c + (upper ? 1u : 0u), ps.tb_end - 1);
            const uint64_t sid = index_pos(a, ps.slab, tbc, ps.cg, geo.ncg);
            ix0[c] = index[sid];
            ix1[c] = index[sid + 1];
        }
    };
    fetch_index(ps.tb_begin + kRound * wave);
    uint32_t padv = 0;                              // pad bytes of the previous round, checked late

    for (uint32_t tb0 = ps.tb_begin + kRound * wave; tb0 < ps.tb_end; tb0 += kRound * nwave) {
        DecChain ch[kDecChains];
        DecState st[kDecChains];
        uint32_t tb[kDecChains], nw[kDecChains], size[kDecChains], rel[kDecChains];
        uint32_t cw[kDecChains], rowo[kDecChains];
        uint2 pva[kDecChains], pvb[kDecChains];
        uint32_t ew[kDecChains], ea[kDecChains], ewr[kDecChains];
        // ring upkeep, both halves packed (lower in bits 0..15): ldk = chunk held in cw,
        // wrk = last chunk written to the ring, live = 0x8000 in the field of a half with
        // a coded stream
        uint32_t ldk[kDecChains], wrk[kDecChains], live[kDecChains];
        uint32_t ktb[kDecChains], cls[kDecChains];                 // class tile base, class word (EXP)
        bool coded[kDecChains], raw[kDecChains];
        uint64_t e0[kDecChains], e1[kDecChains];
        uint32_t x0[kDecChains], c0[kDecChains], c1[kDecChains];
        // every header and ring load of the round is issued before any of them is checked
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            e0[c] = ix0[c];
            e1[c] = ix1[c];
            const uint64_t o = e0[c] & ~kRawBit;
            rel[c] = o >= wlo && o - wlo < (1ull << 31) ? uint32_t(o - wlo) : 0u;
            nw[c] = __builtin_amdgcn_raw_buffer_load_b32(L.rs, rel[c] + 128, 0, 0);
            x0[c] = __builtin_amdgcn_raw_buffer_load_b32(L.rs, rel[c] + 4 * hl, 0, 0);
            const uint32_t woff = rel[c] + kStreamHead;
            c0[c] = __builtin_amdgcn_raw_buffer_load_b32(L.rs, woff + 4 * hl, 0, 0);
            c1[c] = __builtin_amdgcn_raw_buffer_load_b32(L.rs, woff + 2 * kBfChunk + 4 * hl, 0, 0);
            cw[c] = __builtin_amdgcn_raw_buffer_load_b32(L.rs, woff + 2 * kBfChunk * kBfFirst + 4 * hl, 0, 0);
        }
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            tb[c] = tb0 + 2 * c + (upper ? 1u : 0u);
            // byte offset of this lane's first tile-domain row; an absent stream reads rows of tb0
            rowo[c] = ((tb[c] < ps.tb_end ? tb[c] : tb0) * kSteps + r4) * rowb + 2 * q4;
            pva[c] = ld8(prs, rowo[c], 0);
            pvb[c] = ld8(prs, rowo[c], kDecTile * rowb);
        }
        if (tb0 + kRound * nwave < ps.tb_end) fetch_index(tb0 + kRound * nwave);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            const uint32_t hs = (tid >> 5) * kDecChains + c;          // stream slot in the workgroup
            ch[c].ringb = lb + OFF_R + hs * 2 * kBfRing;              // 512-byte aligned
            ch[c].tileb = lb + OFF_T + hs * kDecTile * kLanes + hl;
            ktb[c] = lb + OFF_K + hs * kDecTile * kLanes;
            // ---- stream header checks (every lane of the half holds the same entries)
            uint32_t x = kStateLow;
            size[c] = 0;
            coded[c] = raw[c] = false;
            if (tb[c] < ps.tb_end) {
                const uint64_t o = e0[c] & ~kRawBit, end = e1[c] & ~kRawBit;
                if (end < o || o < wlo || end > whi) {
                    bad = true;
                } else if (e0[c] & kRawBit) {
                    if (end - o != 2 * kSyms) bad = true;
                    else raw[c] = true;
                } else {
                    size[c] = uint32_t(end - o);
                    if (size[c] < kStreamHead || size[c] % 4 != 0 || nw[c] > (size[c] - kStreamHead) / 2) {
                        bad = true;
                    } else {
                        coded[c] = true;
                        x = x0[c];
                        if (x < kStateLow) bad = true;
                    }
                }
            }
            if (!coded[c]) nw[c] = 0;
            const uint64_t cm = __ballot(coded[c]);
            live[c] = (uint32_t(cm) ? 0x8000u : 0u) | ((cm >> 32) ? 0x80000000u : 0u);
            // word offset in the window (a stream that is not coded reads from the window start)
            const uint32_t woff = coded[c] ? rel[c] + kStreamHead : 0u;
            ch[c].woff = woff;
            // escape window: the 4-byte aligned dwords from the start of the escape region (which
            // sits 0 or 2 bytes past a dword boundary), 64 values; a stream's dwords never cross its
            // padded end
            ea[c] = (woff + 2 * nw[c]) & 3u;
            ew[c] = __builtin_amdgcn_raw_buffer_load_b32(L.rs, ((woff + 2 * nw[c]) & ~3u) + 4 * hl, 0, 0);
            // ring: chunk k (words [64k, 64k + 64), two per lane) sits in slot k % 4; chunks 0
            // and 1 now, chunk 2 requested for the first tile end
            lds_u32* ring32 = reinterpret_cast<lds_u32*>(ch[c].ringb);
            ring32[hl] = c0[c];
            ring32[kBfChunk / 2 + hl] = c1[c];
            ldk[c] = kBfFirst * 0x00010001u;
            wrk[c] = 0x00010001u;
            st[c] = DecState{x, 0u, 0u};
            ewr[c] = 0;
        }
        if (padv != 0) bad = true;
        __builtin_amdgcn_wave_barrier();

        // A tile's symbols go to the tile buffer at the end of its steps; the next tile's first
        // step reads them back transposed (lane hl: step r4, lanes q4..q4+3 of its half, so the
        // lanes of a half and the bytes of a lane run in decode order), resolves escaped values,
        // reconstructs and stores the rows and reloads pv with the row two tiles ahead.
        // EXP: the classes of a tile go through the class tile (the lane's predictor row r4, channels
        // q4..q4+3 in, the lane's own channel's 4 steps out); a class byte holds class << 4
        auto put_classes = [&](const uint2 (&pv)[kDecChains]) {
            if constexpr (EXP) {
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c) {
                    const uint32_t ca = cls16x2(pv[c].x, base2) << 4, cb = cls16x2(pv[c].y, base2) << 4;
                    const uint32_t v = __builtin_amdgcn_perm(cb, ca, 0x06040200u);   // 4 class bytes, channel order
#pragma unroll
                    for (uint32_t j = 0; j < 4; ++j)
                        *reinterpret_cast<lds_u8*>(ktb[c] + (q4 + j) * kDecTile + r4) = uint8_t(v >> (8 * j));
                }
            }
        };
        auto get_classes = [&]() {
            if constexpr (EXP) {
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c)
                    cls[c] = *reinterpret_cast<const lds_u32*>(ktb[c] + hl * kDecTile);
            }
        };
        uint32_t zt[kDecChains];
        auto fetch_tile = [&]() {
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c)
                zt[c] = *reinterpret_cast<const lds_u32*>(ch[c].tileb - hl + r4 * kLanes + q4);
        };
        auto finish = [&](uint32_t T, uint2 (&pv)[kDecChains]) {
            uint32_t ef[kDecChains], npc[kDecChains];
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) {
                if constexpr (EXP) {
                    // n of each position's class
                    const uint32_t ca = cls16x2(pv[c].x, base2), cb = cls16x2(pv[c].y, base2);
                    const uint32_t nl = lb + OFF_N;
                    npc[c] = uint32_t(*reinterpret_cast<const lds_u8*>(nl + (ca & 0xFu))) |
                             (uint32_t(*reinterpret_cast<const lds_u8*>(nl + (ca >> 16))) << 8) |
                             (uint32_t(*reinterpret_cast<const lds_u8*>(nl + (cb & 0xFu))) << 16) |
                             (uint32_t(*reinterpret_cast<const lds_u8*>(nl + (cb >> 16))) << 24);
                } else {
                    npc[c] = np;
                }
                ef[c] = zero_bytes(zt[c] ^ npc[c]);
            }
            // the lane's 4 symbols as 16-bit values, two per dword
            uint32_t zz[kDecChains][2];
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) {
                zz[c][0] = __builtin_amdgcn_perm(0u, zt[c], 0x0c010c00u);
                zz[c][1] = __builtin_amdgcn_perm(0u, zt[c], 0x0c030c02u);
            }
            uint32_t efa = 0;
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) efa |= ef[c];
            if (__builtin_expect(__ballot(efa != 0) != 0, 0)) {
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c) {
                    const uint64_t m1 = __ballot(ef[c] != 0);
                    if (m1 == 0) continue;
                    // index of the lane's first escaped value in the stream's escape region: the
                    // half's count so far plus the values of lower lanes (usually one per lane)
                    uint32_t E1 = 0;
                    uint32_t eidx = __builtin_amdgcn_ubfe(st[c].E, L.fsh, 16) + half_rank(m1, E1, L.fsh, L.lowm);
                    st[c].E += E1;
                    uint32_t f = ef[c];
                    if (__ballot((f & (f - 1u)) != 0) != 0) {
                        const uint32_t cnt = __popc(f);
                        for (uint32_t j = 1; j < 4; ++j) {
                            const uint64_t m = __ballot(cnt > j);
                            if (m == 0) break;
                            uint32_t E = 0;
                            eidx += half_rank(m, E, L.fsh, L.lowm);
                            st[c].E += E;
                        }
                    }
                    // the lane's escaped values in order (16 bits each); the first 128 bytes of a
                    // stream's escape region come from the window register, later ones from memory
                    do {
                        const uint32_t kv = __builtin_ctz(f | 0x80000000u) >> 3;         // value 0..3
                        const uint32_t pos = 2 * eidx + ea[c];
                        const uint32_t wv = __builtin_amdgcn_ds_bpermute(
                            int(((pos >> 2) + (upper ? 32u : 0u)) << 2), int(ewr[c]));
                        uint32_t e = (wv >> ((pos & 3u) * 8)) & 0xFFFFu;
                        if (__ballot(f != 0 && pos >= kDecEscWin) != 0) {
                            const uint32_t g = __builtin_amdgcn_raw_buffer_load_b16(
                                L.rs, ch[c].woff + 2 * nw[c] + 2 * eidx, 0, 0);
                            e = pos >= kDecEscWin ? g : e;
                        }
                        if (f != 0) {
                            // a canonical encoder codes a value below n directly
                            if (coded[c] && e < ((npc[c] >> (8 * kv)) & 0xFFu)) bad = true;
                            const uint32_t sh = (kv & 1u) * 16;
                            if (kv < 2) zz[c][0] = (zz[c][0] & ~(0xFFFFu << sh)) | (e << sh);
                            else zz[c][1] = (zz[c][1] & ~(0xFFFFu << sh)) | (e << sh);
                            f &= f - 1u;
                            ++eidx;
                        }
                    } while (__ballot(f != 0) != 0);
                }
            }
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) {
                if (coded[c])
                    st8(make_uint2(recon16x2(pv[c].x, zz[c][0]), recon16x2(pv[c].y, zz[c][1])), ors, rowo[c],
                        T * kDecTile * rowb);
                if (T + 2 < kTiles) pv[c] = ld8(prs, rowo[c], (T + 2) * kDecTile * rowb);
            }
        };
        // one tile: its steps (with the previous tile's finish inside the first one), its symbols
        // to the tile buffer, ring upkeep; pvp holds the previous tile's predictor row
        auto tile_at = [&](uint32_t T, uint2 (&pvp)[kDecChains]) {
            if (T == 1) {
                // the window dword again, written by a VALU move: its load is waited for once, here,
                // and not in the escape path, where the wait would also cover every later load (the
                // predictor rows requested two tiles ahead)
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c) asm volatile("v_mov_b32 %0, %1" : "=v"(ewr[c]) : "v"(ew[c]));
            }
            uint32_t sy[kDecChains][kDecTile];
            DecState s0[kDecChains];
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) s0[c] = st[c];
            get_classes();
            __builtin_amdgcn_wave_barrier();
            dec_tile_steps_bf16<false, EXP>(
                st, L, ch, sy, [&] { if (T > 0) fetch_tile(); }, [&] { if (T > 0) finish(T - 1, pvp); }, cls);
            // a half of a coded stream that read past the last chunk written (word count above
            // 64 (wrk + 1) in its field) decodes the tile again from memory
            uint32_t over = 0;
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c)
                over |= ~((wrk[c] << 6) + 0x80408040u - st[c].P) & live[c];
            if (__builtin_expect(over != 0, 0)) {
                // the escape count keeps what the previous tile's finish added meanwhile
#pragma unroll
                for (uint32_t c = 0; c < kDecChains; ++c) {
                    st[c].x = s0[c].x;
                    st[c].P = s0[c].P;
                }
                dec_tile_steps_bf16<true, EXP>(st, L, ch, sy, [] {}, [] {}, cls);
            }
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c)
#pragma unroll
                for (uint32_t r = 0; r < kDecTile; ++r)
                    *reinterpret_cast<lds_u8*>(ch[c].tileb + r * kLanes) = uint8_t(sy[c][r]);
            // the next tile's classes: its predictor row is in pvp (the initial load after tile 0, the
            // reload of the finish above after later tiles)
            if (T + 1 < kTiles) put_classes(pvp);
#pragma unroll
            for (uint32_t c = 0; c < kDecChains; ++c) {
                // the chunk in cw goes into its slot; the next one is requested while the ring
                // has a free slot (chunk ldk + 1 fits when ldk <= words consumed / 64 + slots - 2)
                reinterpret_cast<lds_u32*>(ch[c].ringb)[__builtin_amdgcn_ubfe(ldk[c], L.fsh, 2) * (kBfChunk / 2) + hl] =
                    cw[c];
                wrk[c] = ldk[c];
                const uint32_t room = ((st[c].P >> 6) & 0x03FF03FFu) + (0x8000u + kBfSlots - 2) * 0x00010001u - ldk[c];
                ldk[c] += (room >> 15) & 0x00010001u;
                cw[c] = __builtin_amdgcn_raw_buffer_load_b32(
                    L.rs, ch[c].woff + 2 * kBfChunk * __builtin_amdgcn_ubfe(ldk[c], L.fsh, 16) + 4 * hl, 0, 0);
            }
            __builtin_amdgcn_wave_barrier();
        };
        put_classes(pva);
        __builtin_amdgcn_wave_barrier();
        for (uint32_t T = 0; T < kTiles; T += 2) {
            tile_at(T, pvb);
            tile_at(T + 1, pva);
        }
        fetch_tile();
        finish(kTiles - 1, pvb);
#pragma unroll
        for (uint32_t c = 0; c < kDecChains; ++c) {
            // ---- stream checks: states back at L, every word and escape consumed, zero pad
            if (coded[c]) {
                const uint32_t pc = __builtin_amdgcn_ubfe(st[c].P, L.fsh, 16);
                const uint32_t ec = __builtin_amdgcn_ubfe(st[c].E, L.fsh, 16);
                const uint32_t used = kStreamHead + 2 * nw[c] + 2 * ec;
                if (st[c].x != kStateLow || pc != nw[c] || used > size[c]) bad = true;
                else if (((used + 3) & ~3u) != size[c]) bad = true;
                // the pad bytes are read now and checked at the next round's start
                padv |= __builtin_amdgcn_raw_buffer_load_b8(L.rs, hl < size[c] - used ? rel[c] + used + hl : 0x80000000u,
                                                            0, 0);
            }
            if (raw[c]) {
                // raw stream: its 4096 values in (step, lane) order, copied row by row (the payload
                // is only 4-byte aligned)
                for (uint32_t T = 0; T < kTiles; ++T) {
                    const uint32_t o = rel[c] + (T * kDecTile + r4) * 2 * kLanes + 2 * q4;
                    st8(make_uint2(__builtin_amdgcn_raw_buffer_load_b32(L.rs, o, 0, 0),
                                   __builtin_amdgcn_raw_buffer_load_b32(L.rs, o + 4, 0, 0)),
                        ors, rowo[c], T * kDecTile * rowb);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (bad || padv != 0) atomicOr(a.status, 1u);
}

// --------------------------------------------------------------- decoded-neighbour map
// Side input of the odd tokens with the neighbour map applied (checkerboard
// mode with a decoded-neighbour map; DCKV page, "How it differs": an odd
// position is predicted from both decoded neighbours through a low-rank
// linear map).  For each odd token t, with n its left row then its right row
// (the last odd token repeats its left row), each value saturated to at most
// 32639:  q = clamp(round(V n / 2^sh_h), -128, 127),
//         out[t] = clamp16(G[t] + round(U q / 2^sh_m)),
// rounding half up.  Both products run on the int8 matrix units
// (v_mfma_i32_16x16x64_i8), whose 32-bit sums are exact here:
//   1. H = N V^T for a block of 16 tokens per wavefront.  An int16 input
//      splits into int8 halves, n = 256 hi + lo with lo in [-128, 127] and
//      hi in [-128, 127] (this is why inputs saturate at 32639), so H =
//      256 (N_hi V^T) + N_lo V^T, each sum at most 4096 * 2^14 < 2^31, put
//      together in 64 bits.
//   2. q, rounded and clamped, goes to LDS (the wavefront's 16 rows, rank
//      padded with zeros to a multiple of 64), and Q U^T runs over 16-channel
//      tiles, added to G and stored.
// A lane's operand bytes are 16 consecutive k of its row (A) or column (B);
// the product pairs the same byte positions of A and B, so any order the
// hardware gives k within a 64-wide step sums the same terms.  Output tile:
// lane l, element r holds row 4 (l / 16) + r, column l % 16.
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr uint32_t kMapTok = 64;                 // odd tokens per workgroup, 16 per wavefront

__device__ __forceinline__ int64_t round_half_up(int64_t v, uint32_t s) {
    return s ? (v + (int64_t(1) << (s - 1))) >> s : v;
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// int8 halves of four int16 inputs (two dwords of two values, the first in
// the low half), each saturated to at most 32639: lo is x mod 256 as a signed
// byte, and hi = (x - lo) / 256 is byte 1 of the 16-bit x + 128 (no carry out
// after the saturation).  Packed 16-bit min and add, then byte permutes.
__device__ __forceinline__ void split4(uint32_t d0, uint32_t d1, uint32_t& lo, uint32_t& hi) {
    const s16x2 cap = {32639, 32639}, half = {128, 128};
    const s16x2 a = __builtin_elementwise_min(__builtin_bit_cast(s16x2, d0), cap);
    const s16x2 b = __builtin_elementwise_min(__builtin_bit_cast(s16x2, d1), cap);
    lo = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a), 0x06040200u);
    hi = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b + half), __builtin_bit_cast(uint32_t, a + half),
                               0x07050301u);
}

// 16 consecutive int16 of a row as 8 dwords: two 16-byte loads when VEC (the
// arrays are 16-byte aligned), else element loads
template <bool VEC>
__device__ __forceinline__ void load16(const int16_t* p, uint32_t (&d)[8]) {
    if (VEC) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
        d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = uint32_t(uint16_t(p[2 * i])) | (uint32_t(uint16_t(p[2 * i + 1])) << 16);
    }
}

// KT: rank / 16; VEC: coef, G and out 16-byte aligned.  right: the row after
// the last one (the last odd token's right neighbour), or null for the end of
// the cache (the last odd token repeats its left row).
template <uint32_t KT, bool VEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KT <= 4 ? 4 : 1))) void nbr_map(const int16_t* coef, const int16_t* __restrict__ G, int16_t* out,
                                               uint32_t T, uint32_t C, const int8_t* __restrict__ V,
                                               const int8_t* __restrict__ U, uint32_t sh_h, uint32_t sh_m,
                                               const int16_t* right) {
    constexpr uint32_t K = 16 * KT;
    constexpr uint32_t KP = (K + 63) / 64 * 64;             // rank padded to whole 64-wide steps
    constexpr uint32_t KB = KP / 64;
    __shared__ __align__(16) int8_t qs[kMapTok * KP];
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint32_t g4 = lane >> 4, r16 = lane & 15u;
    const uint32_t u0 = blockIdx.x * kMapTok + w * 16;      // first odd index of this wavefront
    const uint32_t nodd = T / 2;
    const uint32_t W2 = 2 * C;

    // 1. H = N V^T over the 2C inputs of odd token u: [its left row | its right
    //    row], i.e. even rows 2u and 2u + 2.  The workgroup's 64 odd tokens
    //    share 65 even rows, so the sum runs by column block: for columns
    //    [x, x + 64) the workgroup loads the 65 rows' columns and both matching
    //    V slices (V[:, x..] for left rows, V[:, C + x..] for right rows) into
    //    LDS once, and each wavefront takes the left and the right product of
    //    its 16 tokens from there (a lane's A row: slot 16 w + r16 on the left,
    //    the next slot on the right).  The next block's tiles are loaded into
    //    registers while the current one multiplies.  A 32-wide last block
    //    (C an odd multiple of 32) is one product: k-quarters 0-1 from the left
    //    row, 2-3 from the right one.
    constexpr uint32_t kSlots = kMapTok + 1;                // even rows of the workgroup
    constexpr uint32_t kAVec = (kSlots * 8 + 255) / 256;    // 16-byte pieces of the row tile per thread
    constexpr uint32_t kVVec = (2 * K * 4 + 255) / 256;     // of the V tiles
    __shared__ __align__(16) int16_t atile[2][kSlots * 64]; // two buffers: [slot][64 columns]
    __shared__ __align__(16) int8_t vtile[2][2 * K * 64];   // two buffers: [side][rank][64 columns]
    __shared__ v4i sink[64];                                // stores of pieces past the tiles (any content)
    v4i hi[KT], lo[KT];
#pragma unroll
    for (uint32_t j = 0; j < KT; ++j) hi[j] = lo[j] = v4i{0, 0, 0, 0};
    {
        const uint32_t ub = blockIdx.x * kMapTok;              // first odd index of the workgroup
        // even row of slot e: row 2 (ub + e); the slot past the cache's end (the last odd token's
        // right neighbour) is `right`, or the last odd token's left row again
        auto slot_row = [&](uint32_t e) __attribute__((always_inline)) -> const int16_t* {
            const uint32_t r = 2 * (ub + e);
            return r < T ? coef + size_t(r) * C : (right ? right : coef + size_t(r - 2) * C);
        };
        v4i ar[kAVec], vr[kVVec];                          // (native vectors: kept in registers)
        // a block is 64 or 32 columns wide: 8 or 4 sixteen-byte pieces per row slot, 4 or 2 per V row
        // and side (shifts: 3 or 2, 2 or 1)
        auto load_block = [&](uint32_t x) __attribute__((always_inline)) {
            const uint32_t ws = C - x >= 64 ? 3u : 2u;
#pragma unroll
            for (uint32_t i = 0; i < kAVec; ++i) {
                const uint32_t idx0 = threadIdx.x + 256 * i;
                const uint32_t idx = idx0 < (kSlots << ws) ? idx0 : 0u;     // (past the tile: piece 0 again, unused)
                const int16_t* src = slot_row(idx >> ws) + x + 8 * (idx & ((1u << ws) - 1u));
                if (VEC) {
                    ar[i] = *reinterpret_cast<const v4i*>(src);
                } else {
                    uint32_t d[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        d[q] = uint32_t(uint16_t(src[2 * q])) | (uint32_t(uint16_t(src[2 * q + 1])) << 16);
                    ar[i] = v4i{int(d[0]), int(d[1]), int(d[2]), int(d[3])};
                }
            }
            const uint32_t vs = ws - 1u;
#pragma unroll
            for (uint32_t i = 0; i < kVVec; ++i) {
                const uint32_t idx0 = threadIdx.x + 256 * i;
                const uint32_t idx = idx0 < (2 * K << vs) ? idx0 : 0u;
                const uint32_t r = idx >> vs;                  // side * K + rank
                const uint32_t sd = r / K, rk = r % K;
                vr[i] = *reinterpret_cast<const v4i*>(V + size_t(rk) * W2 + sd * C + x +
                                                        16 * (idx & ((1u << vs) - 1u)));
            }
        };
        // pieces past the tiles go to a sink, so that every thread stores every piece
        auto store_block = [&](uint32_t x, uint32_t bf) __attribute__((always_inline)) {
            const uint32_t ws = C - x >= 64 ? 3u : 2u, vs = ws - 1u;
#pragma unroll
            for (uint32_t i = 0; i < kAVec; ++i) {
                const uint32_t idx = threadIdx.x + 256 * i;
                v4i* dst = idx < (kSlots << ws)
                               ? reinterpret_cast<v4i*>(atile[bf] + (idx >> ws) * 64 + 8 * (idx & ((1u << ws) - 1u)))
                               : sink + (threadIdx.x & 63u);
                *dst = ar[i];
            }
#pragma unroll
            for (uint32_t i = 0; i < kVVec; ++i) {
                const uint32_t idx = threadIdx.x + 256 * i;
                v4i* dst = idx < (2 * K << vs)
                               ? reinterpret_cast<v4i*>(vtile[bf] + (idx >> vs) * 64 + 16 * (idx & ((1u << vs) - 1u)))
                               : sink + (threadIdx.x & 63u);
                *dst = vr[i];
            }
        };
        // one product: A = 16 int16 inputs of the lane (split into int8 halves), B = V rows
        auto product = [&](const int16_t* arow, const int8_t* vside) __attribute__((always_inline)) {
            uint32_t cur[8];
            const uint4 c0 = reinterpret_cast<const uint4*>(arow)[0], c1 = reinterpret_cast<const uint4*>(arow)[1];
            cur[0] = c0.x; cur[1] = c0.y; cur[2] = c0.z; cur[3] = c0.w;
            cur[4] = c1.x; cur[5] = c1.y; cur[6] = c1.z; cur[7] = c1.w;
            uint32_t pl[4], ph[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) split4(cur[2 * d], cur[2 * d + 1], pl[d], ph[d]);
            const v4i ah = {int(ph[0]), int(ph[1]), int(ph[2]), int(ph[3])};
            const v4i al = {int(pl[0]), int(pl[1]), int(pl[2]), int(pl[3])};
#pragma unroll
            for (uint32_t j = 0; j < KT; ++j) {
                const v4i bv = *reinterpret_cast<const v4i*>(vside + (j * 16 + r16) * 64);
                hi[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah, bv, hi[j], 0, 0, 0);
                lo[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, bv, lo[j], 0, 0, 0);
            }
        };
        // two tile buffers: block b in buffer b & 1; block b + 1 goes into the other buffer while block b
        // multiplies (that buffer's last reader, block b - 1, ended at the barrier before), so one
        // barrier per block
        const uint32_t e = w * 16 + r16;                     // the lane's left slot
        load_block(0);
        store_block(0, 0);
        if (64 < C) load_block(64);
        __syncthreads();
        for (uint32_t x = 0, bf = 0; x < C; x += 64, bf ^= 1u) {
            const int16_t* at = atile[bf];
            const int8_t* vt = vtile[bf];
            if (x + 64 <= C) {
                product(at + e * 64 + 16 * g4, vt + 16 * g4);                         // left rows
                product(at + (e + 1) * 64 + 16 * g4, vt + K * 64 + 16 * g4);          // right rows
            } else {
                const uint32_t q = g4 & 1u, sd = g4 >> 1;     // 32-wide block
                product(at + (e + sd) * 64 + 16 * q, vt + sd * K * 64 + 16 * q);
            }
            if (x + 64 < C) store_block(x + 64, bf ^ 1u);
            if (x + 128 < C) load_block(x + 128);
            __syncthreads();
        }
    }
    // 2. q to LDS: element r of tile j is token 4 g4 + r of the wavefront, rank column 16 j + r16
    int8_t* qw = qs + size_t(w) * 16 * KP;
#pragma unroll
    for (uint32_t j = 0; j < KT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t h = int64_t(hi[j][r]) * 256 + int64_t(lo[j][r]);
            const int64_t q0 = round_half_up(h, sh_h);
            const int64_t q = q0 < -128 ? -128 : (q0 > 127 ? 127 : q0);
            qw[(4 * g4 + r) * KP + j * 16 + r16] = int8_t(q);
        }
    if constexpr (KP > K)
        for (uint32_t i = lane; i < 16 * (KP - K); i += 64) qw[(i / (KP - K)) * KP + K + i % (KP - K)] = 0;
    __syncthreads();

    // 3. out = G + round(U Q^T), transposed so that a lane holds 4 consecutive
    //    channels of one token: A = U rows (channels), B = the wavefront's q
    //    rows (tokens); element r of a tile is channel 4 g4 + r of token r16.
    //    Rounds of 64 channels (up to four 16-channel tiles; channels are a
    //    multiple of 32, not always of 64): the round's U rows go into LDS once
    //    for the workgroup (the V tile's space), and the next round's U rows and
    //    side inputs are loaded while the current round multiplies.
    v4i bq[KB];
#pragma unroll
    for (uint32_t kb = 0; kb < KB; ++kb)
        bq[kb] = *reinterpret_cast<const v4i*>(qw + r16 * KP + kb * 64 + 16 * g4);
    const uint32_t u = u0 + r16;
    const size_t row = size_t(2 * min(u, nodd - 1) + 1) * C;
    constexpr uint32_t kUPieces = K / 16;                   // 16-byte pieces of a U row
    constexpr uint32_t kUVec = (64 * kUPieces + 255) / 256;
    int8_t* const ubuf = vtile[0];                           // two buffers of [64 channels][K]
    v4i ur[kUVec];
    uint2 gv[4], gn[4];
    auto load_round = [&](uint32_t c0) __attribute__((always_inline)) {
        const uint32_t pieces = min(64u, C - c0) * kUPieces;
#pragma unroll
        for (uint32_t i = 0; i < kUVec; ++i) {
            const uint32_t idx0 = threadIdx.x + 256 * i;
            const uint32_t idx = idx0 < pieces ? idx0 : 0u;
            ur[i] = *reinterpret_cast<const v4i*>(U + size_t(c0 + idx / kUPieces) * K + 16 * (idx % kUPieces));
        }
        const uint32_t ntile = min(4u, (C - c0) / 16);       // 2 or 4
#pragma unroll
        for (uint32_t tt = 0; tt < 4; ++tt) {
            const int16_t* gp = G + row + c0 + 16 * (tt < ntile ? tt : 0u) + 4 * g4;
            if (VEC) {
                gn[tt] = *reinterpret_cast<const uint2*>(gp);
            } else {
                gn[tt].x = uint32_t(uint16_t(gp[0])) | (uint32_t(uint16_t(gp[1])) << 16);
                gn[tt].y = uint32_t(uint16_t(gp[2])) | (uint32_t(uint16_t(gp[3])) << 16);
            }
        }
    };
    auto store_round = [&](uint32_t c0, uint32_t bf) __attribute__((always_inline)) {
        const uint32_t pieces = min(64u, C - c0) * kUPieces;
#pragma unroll
        for (uint32_t i = 0; i < kUVec; ++i) {
            const uint32_t idx = threadIdx.x + 256 * i;
            v4i* dst = idx < pieces ? reinterpret_cast<v4i*>(ubuf + bf * 64 * K + 16 * idx) : sink + (threadIdx.x & 63u);
            *dst = ur[i];
        }
    };
    // as in the first product: round r's U rows in buffer r & 1, one barrier per round (phase 1's
    // last barrier and phase 2's leave the V tiles free)
    load_round(0);
    store_round(0, 0);
#pragma unroll
    for (uint32_t tt = 0; tt < 4; ++tt) gv[tt] = gn[tt];
    if (64 < C) load_round(64);
    __syncthreads();
    for (uint32_t c0 = 0, bf = 0; c0 < C; c0 += 64, bf ^= 1u) {
        const int8_t* utile = ubuf + bf * 64 * K;
        const uint32_t ntile = min(4u, (C - c0) / 16);       // 2 or 4
#pragma unroll
        for (uint32_t tt = 0; tt < 4; ++tt) {
            if (tt >= ntile) break;
            v4i acc = {0, 0, 0, 0};
#pragma unroll
            for (uint32_t kb = 0; kb < KB; ++kb) {
                const uint32_t kk = kb * 64 + 16 * g4;
                const v4i au = kk < K ? *reinterpret_cast<const v4i*>(utile + (16 * tt + r16) * K + kk)
                                      : v4i{0, 0, 0, 0};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(au, bq[kb], acc, 0, 0, 0);
            }
            const int32_t gq[4] = {int32_t(int16_t(gv[tt].x & 0xFFFFu)), int32_t(gv[tt].x) >> 16,
                                   int32_t(int16_t(gv[tt].y & 0xFFFFu)), int32_t(gv[tt].y) >> 16};
            uint32_t o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int32_t v = gq[r] + int32_t(round_half_up(acc[r], sh_m));
                o[r] = uint32_t(uint16_t(int16_t(v < -32768 ? -32768 : (v > 32767 ? 32767 : v))));
            }
            if (u < nodd) {
                int16_t* op = out + row + c0 + 16 * tt + 4 * g4;
                if (VEC) {
                    *reinterpret_cast<uint2*>(op) = uint2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) op[r] = int16_t(uint16_t(o[r]));
                }
            }
        }
        if (c0 + 64 < C) {
            store_round(c0 + 64, bf ^ 1u);
#pragma unroll
            for (uint32_t tt = 0; tt < 4; ++tt) gv[tt] = gn[tt];
        }
        if (c0 + 128 < C) load_round(c0 + 128);
        __syncthreads();
    }
}

__global__ void clear_u32(uint32_t* p, uint32_t n) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Optional per-kernel timing: a HIP event pair on each launch on the caller's
// stream, read back after the call's final synchronization.
struct KernelTiming {
    bool on = false;
    int count = 0;
    hipEvent_t ev[2 * kMaxTimedKernels] = {};
    const char* name[kMaxTimedKernels] = {};
    float ms[kMaxTimedKernels] = {};
    int done = 0;
};
KernelTiming g_timing;

// `launch` dispatches one kernel with hipExtLaunchKernelGGL and the event pair it
// is given (null when timing is off): the events take the kernel's own start
// and end times, with no marker packets between the launches.
template <class F>
void timed(const char* name, hipStream_t st, F&& launch) {
    KernelTiming& T = g_timing;
    if (T.on && T.count < kMaxTimedKernels) {
        launch(T.ev[2 * T.count], T.ev[2 * T.count + 1]);
        T.name[T.count++] = name;
    } else {
        launch(nullptr, nullptr);
    }
}

constexpr uint32_t kLdsThreads = 1024;

constexpr size_t kLdsLimit = 160 * 1024;

// Work decomposition of the LDS kernels for a residual-mode shape.
// max_tbc: token blocks per workgroup at most (a whole slab's 256 for the tiled kernels but the e4m3
// pair encoders, whose workgroups take 128: measured faster than 256, 64 or 32 on the Qwen3-8B-shaped cache)
constexpr uint32_t kPairChunk = 128;
LdsGeo lds_geometry(const skv_shape& s, uint32_t cgw = 1, uint32_t max_tbc = 256) {
    const uint32_t ncg = s.channels / kLanes, ntb = s.tokens / kSteps;
    const uint32_t line = s.dtype == SKV_E4M3 ? 4u : 2u;    // channel groups per 128-byte row segment
    LdsGeo g;
    g.cgw = cgw;
    g.G = (ncg % line == 0) ? line : (ncg % 2 == 0 ? 2u : 1u);
    g.G = std::max(1u, g.G / cgw);
    g.tbc = std::min<uint32_t>(ntb, max_tbc);
    // a workgroup's encoder scratch (tbc streams, ncg apart) is addressed with offsets below 2^31
    const uint64_t sstride = uint64_t(ncg) * 2 * kSyms * (s.dtype == SKV_E4M3 ? 1u : 2u);
    while (g.tbc > 1 && uint64_t(g.tbc) * sstride >= (1ull << 31)) g.tbc /= 2;
    g.ntbc = (ntb + g.tbc - 1) / g.tbc;
    g.groups = s.layers * s.kv * g.ntbc * (ncg / (g.G * cgw));
    return g;
}

inline uint32_t lds_grid(const LdsGeo& g) { return ((g.groups + 7) / 8) * 8 * g.G; }
// The tiled kernels address a slab's rows (a whole matrix in checkerboard mode)
// with 32-bit byte offsets; larger slabs take the per-step kernels.
inline bool slab_fits(const skv_shape& s) {
    const uint64_t eb = s.dtype == SKV_E4M3 ? 1u : 2u;
    return uint64_t(s.tokens) * s.channels * eb < (1ull << 31);
}
inline uint32_t fc_stride(const DevTables& t) { return (t.max_n + 1 + 3) & ~3u; }

size_t decode_lds_bytes(const DevTables& t, uint32_t dtype, bool half) {
    return size_t(kLanes) * (kM >> (half ? 1 : 0)) + size_t(kLanes) * (fc_stride(t) + 1) * 4;
}
size_t encode_lds_bytes(const DevTables& t, uint32_t dtype) { return size_t(kLanes) * fc_stride(t) * 16; }

template <class K>
hipError_t allow_lds(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               int(bytes));
}

template <uint32_t KT>
hipError_t nbr_map_kt(const int16_t* coef, const int16_t* G, int16_t* out, uint32_t T, uint32_t C,
                      const DevTables& t, hipStream_t st, const int16_t* right) {
    const bool vec = (reinterpret_cast<uintptr_t>(coef) | reinterpret_cast<uintptr_t>(G) |
                      reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(right)) % 16 == 0;
    timed("nbr_map", st, [&](hipEvent_t e0, hipEvent_t e1) {
        const dim3 grid(T / 2 / kMapTok), block(256);
        if (vec)
            hipExtLaunchKernelGGL((nbr_map<KT, true>), grid, block, 0, st, e0, e1, 0, coef, G, out, T, C, t.map_v,
                                  t.map_u, t.map_sh_h, t.map_sh_m, right);
        else
            hipExtLaunchKernelGGL((nbr_map<KT, false>), grid, block, 0, st, e0, e1, 0, coef, G, out, T, C, t.map_v,
                                  t.map_u, t.map_sh_h, t.map_sh_m, right);
    });
    return hipGetLastError();
}

// Encoder phase 1: the streams into the workspace, their sizes summed.
template <uint32_t DT, uint32_t MODE>
hipError_t encode_code(const EncodeLaunch& a, const DevTables& t, hipStream_t st) {
    const uint64_t n = a.n_streams;
    const uint32_t nb = uint32_t((n + kScanBlock - 1) / kScanBlock);
    if (MODE == SKV_CHECKERBOARD && a.shape.mode == SKV_CHECKERBOARD_MAP) {
        // the odd pass codes against the side input mapped from the true (= decoded) even rows
        const hipError_t e = launch_nbr_map(static_cast<const int16_t*>(a.target), static_cast<const int16_t*>(a.aux),
                                            a.map_side, a.shape.tokens, a.shape.channels, t, st, nullptr);
        if (e != hipSuccess) return e;
    }
    const uint32_t eg = uint32_t((n + kStreamsPerBlock - 1) / kStreamsPerBlock);
    const size_t lb = encode_lds_bytes(t, DT);
    const size_t lt = size_t(kLanes) * fc_stride(t) * 16 + (kLdsThreads / 64) * kTileWaveLds;
    const bool aligned = (reinterpret_cast<uintptr_t>(a.target) | reinterpret_cast<uintptr_t>(a.aux)) % 8 == 0;
    const uint32_t ncg = a.shape.channels / kLanes;
    const bool aligned16 = (reinterpret_cast<uintptr_t>(a.target) | reinterpret_cast<uintptr_t>(a.aux)) % 16 == 0;
    const bool fits = slab_fits(a.shape);
    if (DT == SKV_BF16 && MODE == SKV_RESIDUAL && fits && aligned16 && encode_bf16_lds(fc_stride(t)) <= kLdsLimit) {
        const LdsGeo lg = lds_geometry(a.shape);
        const size_t lp = encode_bf16_lds(fc_stride(t));
        hipError_t e = allow_lds(encode_bf16<false>, lp);
        if (e != hipSuccess) return e;
        timed("encode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(encode_bf16<false>, dim3(lds_grid(lg)), dim3(kLdsThreads), lp, st, e0, e1, 0, a, t,
                                  fc_stride(t), lg);
        });
    } else if (DT == SKV_BF16 && MODE == SKV_RESIDUAL_EXP && fits && aligned16 &&
               encode_bf16_exp_lds(fc_stride(t)) <= kLdsLimit) {
        const LdsGeo lg = lds_geometry(a.shape);
        const size_t lp = encode_bf16_exp_lds(fc_stride(t));
        hipError_t e = allow_lds(encode_bf16<true>, lp);
        if (e != hipSuccess) return e;
        timed("encode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(encode_bf16<true>, dim3(lds_grid(lg)), dim3(kLdsThreads), lp, st, e0, e1, 0, a, t,
                                  fc_stride(t), lg);
        });
    } else if (DT == SKV_E4M3 && MODE == SKV_RESIDUAL_EXP && fits && ncg % 4 == 0 && aligned &&
               3 * (encode_exp_lds(fc_stride(t)) + 256) <= kLdsLimit) {
        const LdsGeo lg = lds_geometry(a.shape, 2, kPairChunk);
        const size_t lp = encode_exp_lds(fc_stride(t));
        hipError_t e = allow_lds(encode_pairs_exp, lp);
        if (e != hipSuccess) return e;
        timed("encode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(encode_pairs_exp, dim3(lds_grid(lg)), dim3(kExpEncThreads), lp, st, e0, e1, 0, a, t,
                                  fc_stride(t), lg);
        });
    } else if (DT == SKV_E4M3 && MODE == SKV_RESIDUAL && fits && ncg % 4 == 0 &&
               2 * encode_groups_lds(1, fc_stride(t)) + 512 <= kLdsLimit && aligned) {
        const LdsGeo lg = lds_geometry(a.shape, 2, kPairChunk);
        const size_t lp = encode_groups_lds(1, fc_stride(t));
        hipError_t e = allow_lds(encode_pairs, lp);
        if (e != hipSuccess) return e;
        timed("encode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(encode_pairs, dim3(lds_grid(lg)), dim3(kLdsThreads), lp, st, e0, e1, 0, a, t, fc_stride(t), lg);
        });
    } else if (DT == SKV_E4M3 && MODE == SKV_RESIDUAL && fits && lt <= kLdsLimit && aligned) {
        const LdsGeo lg = lds_geometry(a.shape);
        auto k = encode_tiles<SKV_E4M3>;
        hipError_t e = allow_lds(k, lt);
        if (e != hipSuccess) return e;
        timed("encode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(k, dim3(lds_grid(lg)), dim3(kLdsThreads), lt, st, e0, e1, 0, a, t, fc_stride(t), lg);
        });
    } else if (MODE == SKV_RESIDUAL && fits && lb <= kLdsLimit) {
        const LdsGeo lg = lds_geometry(a.shape);
        auto k = encode_lds<DT, 1, 4>;
        hipError_t e = allow_lds(k, lb);
        if (e != hipSuccess) return e;
        timed("encode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(k, dim3(lds_grid(lg)), dim3(kLdsThreads), lb, st, e0, e1, 0, a, t, fc_stride(t), lg);
        });
    } else if (MODE == SKV_CHECKERBOARD && fits) {
        // two steps between stages: longer lags measured no faster (more registers, fewer waves)
        const Geo g{a.shape.channels, a.shape.tokens, a.shape.channels / kLanes, a.shape.tokens / 2 / kSteps};
        const dim3 grid(g.ncg * ((g.ntb + kCbEncStreams - 1) / kCbEncStreams), 2);       // y: pass
        timed("encode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(encode_cb, grid, dim3(kCbEncStreams * 32), 0, st, e0, e1, 0, a, t);
        });
    } else {
        timed("encode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL((encode_streams<DT, MODE>), dim3(eg), dim3(256), 0, st, e0, e1, 0, a, t);
        });
    }
    timed("stream_block_sums", st, [&](hipEvent_t e0, hipEvent_t e1) {
        hipExtLaunchKernelGGL(stream_block_sums, dim3(nb), dim3(kScanBlock), 0, st, e0, e1, 0, a.meta, n,
                           kSyms * (DT == SKV_E4M3 ? 1u : 2u), a.block_sum);
    });
    timed("stream_block_scan", st, [&](hipEvent_t e0, hipEvent_t e1) {
        hipExtLaunchKernelGGL(stream_block_scan, dim3(1), dim3(kScanBlock), 0, st, e0, e1, 0, a.block_sum, nb, a.block_off,
                              a.total, a.pay_base);
    });
    return hipGetLastError();
}

// Encoder phase 2: header, index and streams into a.out.
template <uint32_t DT, uint32_t MODE>
hipError_t encode_pack(const EncodeLaunch& a, hipStream_t st) {
    const uint64_t n = a.n_streams;
    const uint32_t nb = uint32_t((n + kScanBlock - 1) / kScanBlock);
    timed("place_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
        hipExtLaunchKernelGGL((place_streams<DT, MODE>), dim3(nb), dim3(kScanBlock), 0, st, e0, e1, 0, a, a.block_off);
    });
    timed("copy_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
        hipExtLaunchKernelGGL((copy_streams<DT, MODE>), dim3(uint32_t((n + 3) / 4)), dim3(256), 0, st, e0, e1, 0, a);
    });
    return hipGetLastError();
}

template <uint32_t DT, uint32_t MODE>
hipError_t encode_all(const EncodeLaunch& a, const DevTables& t, hipStream_t st, uint32_t phases) {
    if (phases & kEncodeCode) {
        const hipError_t e = encode_code<DT, MODE>(a, t, st);
        if (e != hipSuccess) return e;
    }
    return phases & kEncodePack ? encode_pack<DT, MODE>(a, st) : hipSuccess;
}

template <uint32_t DT, uint32_t MODE>
hipError_t decode_all(const DecodeLaunch& a, const DevTables& t, hipStream_t st) {
    const bool fits = slab_fits(a.shape);
    // rows by residual byte: FS rows hold every symbol of tables with fewer than FS direct symbols
    // (FS = 128: 156 KB of LDS); wider tables take the per-table LDS decoder
    static_assert(dec_e4m3_lds(128) <= kLdsLimit, "128-row tables fit in LDS");
    if (DT == SKV_E4M3 && MODE == SKV_RESIDUAL && fits && t.max_n + 1 <= 128) {
        const LdsGeo lg = lds_geometry(a.shape);
        const uint32_t fs = t.max_n + 1 <= 32 ? 32u : (t.max_n + 1 <= 64 ? 64u : 128u);
        auto k = fs == 32 ? decode_e4m3<32> : (fs == 64 ? decode_e4m3<64> : decode_e4m3<128>);
        const size_t lb = dec_e4m3_lds(fs);
        hipError_t e = allow_lds(k, lb);
        if (e != hipSuccess) return e;
        timed("decode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(k, dim3(lds_grid(lg)), dim3(kLdsThreads), lb, st, e0, e1, 0, a, t, lg);
        });
        return hipGetLastError();
    }
    if (DT == SKV_E4M3 && MODE == SKV_RESIDUAL_EXP && fits &&
        t.max_n + 2 <= kExpRows && dec_exp_lds() <= kLdsLimit) {
        const LdsGeo lg = lds_geometry(a.shape);
        auto k = decode_e4m3<kExpRows, true>;
        hipError_t e = allow_lds(k, dec_exp_lds());
        if (e != hipSuccess) return e;
        timed("decode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(k, dim3(lds_grid(lg)), dim3(kLdsThreads), dec_exp_lds(), st, e0, e1, 0, a, t, lg);
        });
        return hipGetLastError();
    }
    // the bf16 decoder moves predictor and output rows 8 bytes per lane
    const bool aligned8 = (reinterpret_cast<uintptr_t>(a.aux) | reinterpret_cast<uintptr_t>(a.out)) % 8 == 0;
    if (DT == SKV_BF16 && MODE == SKV_RESIDUAL && fits && aligned8 && dec_bf16_lds() <= kLdsLimit) {
        const LdsGeo lg = lds_geometry(a.shape);
        hipError_t e = allow_lds(decode_bf16<false>, dec_bf16_lds());
        if (e != hipSuccess) return e;
        timed("decode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(decode_bf16<false>, dim3(lds_grid(lg)), dim3(kLdsThreads), dec_bf16_lds(), st, e0, e1,
                                  0, a, t, lg);
        });
        return hipGetLastError();
    }
    if (DT == SKV_BF16 && MODE == SKV_RESIDUAL_EXP && fits && aligned8 && dec_bf16_exp_lds() <= kLdsLimit) {
        const LdsGeo lg = lds_geometry(a.shape);
        hipError_t e = allow_lds(decode_bf16<true>, dec_bf16_exp_lds());
        if (e != hipSuccess) return e;
        timed("decode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(decode_bf16<true>, dim3(lds_grid(lg)), dim3(kLdsThreads), dec_bf16_exp_lds(), st, e0,
                                  e1, 0, a, t, lg);
        });
        return hipGetLastError();
    }
    const size_t lb = decode_lds_bytes(t, DT, true);
    if (MODE == SKV_RESIDUAL && fits && lb <= kLdsLimit) {
        const LdsGeo lg = lds_geometry(a.shape);
        auto k = decode_lds<DT, 1, 4, true>;
        hipError_t e = allow_lds(k, lb);
        if (e != hipSuccess) return e;
        timed("decode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL(k, dim3(lds_grid(lg)), dim3(kLdsThreads), lb, st, e0, e1, 0, a, t, fc_stride(t), lg);
        });
        return hipGetLastError();
    }
    const uint64_t passes = MODE == SKV_CHECKERBOARD ? 2 : 1;
    const uint64_t per = a.n_streams / passes;
    const uint32_t grid = uint32_t((per + kStreamsPerBlock - 1) / kStreamsPerBlock);
    const uint32_t ncg = a.shape.channels / kLanes;
    auto cb_grid = [&](uint64_t streams) {
        return dim3(uint32_t(ncg * ((streams / ncg + kCbDecStreams - 1) / kCbDecStreams)));
    };
    // a checkerboard range (token blocks from tb_base, or fewer than the container's)
    const bool range = MODE == SKV_CHECKERBOARD && (a.tb_base != 0 || a.ntb_index != a.shape.tokens / 2 / kSteps);
    if (range && !fits) return hipErrorInvalidValue;
    if (range && a.next_rows) {
        // the even tokens of the block after the range, into next_rows; the block's side input
        // follows the range's in aux
        DecodeLaunch x = a;
        x.shape.tokens = 2 * kSteps;
        x.n_streams = 2 * uint64_t(ncg);
        x.tb_base = a.tb_base + a.shape.tokens / (2 * kSteps);
        x.aux = static_cast<const int16_t*>(a.aux) + size_t(a.shape.tokens) * a.shape.channels;
        x.aux_odd = x.aux;
        x.out = a.next_rows;
        x.next_rows = nullptr;
        timed("decode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            hipExtLaunchKernelGGL((decode_cb<true>), cb_grid(ncg), dim3(kCbDecStreams * 32), 0, st, e0, e1, 0, x,
                                  t, 0, ncg);
        });
    }
    for (uint64_t ps = 0; ps < passes; ++ps) {
        if (ps == 1 && a.shape.mode == SKV_CHECKERBOARD_MAP) {
            // the map of the decoded even rows, written into the output's odd rows (the odd pass's side input)
            int16_t* o = static_cast<int16_t*>(a.out);
            const hipError_t e = launch_nbr_map(o, static_cast<const int16_t*>(a.aux), o, a.shape.tokens,
                                                a.shape.channels, t, st, a.next_rows);
            if (e != hipSuccess) return e;
        }
        timed("decode_streams", st, [&](hipEvent_t e0, hipEvent_t e1) {
            if (MODE == SKV_CHECKERBOARD && range)
                hipExtLaunchKernelGGL((decode_cb<true>), cb_grid(per), dim3(kCbDecStreams * 32), 0, st, e0, e1, 0, a, t,
                                      ps * per, per);
            else if (MODE == SKV_CHECKERBOARD && fits)
                hipExtLaunchKernelGGL((decode_cb<false>), cb_grid(per), dim3(kCbDecStreams * 32), 0, st, e0, e1, 0, a, t,
                                      ps * per, per);
            else
                hipExtLaunchKernelGGL((decode_streams<DT, MODE>), dim3(grid), dim3(256), 0, st, e0, e1, 0, a, t, ps * per, per);
        });
    }
    return hipGetLastError();
}

}  // namespace

uint64_t encode_work_bytes(uint64_t n_streams, uint32_t raw_bytes) {
    auto al = [](uint64_t v) { return (v + 255) & ~uint64_t(255); };
    const uint64_t nb = (n_streams + kScanBlock - 1) / kScanBlock;
    return al(2 * n_streams * raw_bytes) + al(4 * n_streams) + al(4 * nb) + al(8 * nb) + 256;
}

hipError_t build_dev_tables(const uint8_t* blob, DevTables* t, hipStream_t st) {
    const uint32_t nt = rd32(blob + 8);
    uint8_t* rec = nullptr;
    hipError_t e = hipMalloc(&rec, size_t(nt) * kTableRecord);
    if (e == hipSuccess) e = hipMalloc(&t->n, size_t(nt) * 4);
    if (e == hipSuccess) e = hipMalloc(&t->enc, size_t(nt) * 256 * sizeof(uint4));
    if (e == hipSuccess) e = hipMalloc(&t->fc, size_t(nt) * 256 * 4 + 16);   // + one entry read past the last row
    if (e == hipSuccess) e = hipMalloc(&t->slot, size_t(nt) * kM);
    std::vector<uint32_t> tail_base;
    if (e == hipSuccess && is_checkerboard(blob[7])) {
        // each table's tail: the slots from the start of symbol min(kCbHead, n) to the end
        tail_base.resize(nt);
        uint64_t total = 0;
        for (uint32_t j = 0; j < nt; ++j) {
            const uint8_t* r = blob + kHeaderBytes + size_t(j) * kTableRecord;
            const uint32_t n = std::min(kCbHead, rd16(r));
            uint32_t ts = 0;
            for (uint32_t z = 0; z < n; ++z) ts += rd16(r + 2 + 2 * z);
            tail_base[j] = uint32_t(total);
            total += kM - std::min<uint32_t>(ts, kM);
        }
        if (total >> 32) e = hipErrorInvalidValue;
        if (e == hipSuccess) e = hipMalloc(&t->tail, std::max<uint64_t>(total, 1) * 4);
        if (e == hipSuccess) e = hipMalloc(&t->tail_base, size_t(nt) * 4);
        if (e == hipSuccess)
            e = hipMemcpyAsync(t->tail_base, tail_base.data(), size_t(nt) * 4, hipMemcpyHostToDevice, st);
    }
    if (e == hipSuccess && is_checkerboard(blob[7])) e = hipMalloc(&t->enc8, size_t(nt) * 256 * sizeof(uint2));
    if (e == hipSuccess && blob[7] == SKV_CHECKERBOARD_MAP) {
        // the map section follows the records (validated with the blob)
        const uint8_t* m = blob + kHeaderBytes + size_t(nt) * kTableRecord;
        const uint32_t C = rd32(blob + 20);
        t->map_rank = rd32(m);
        t->map_sh_h = rd32(m + 4);
        t->map_sh_m = rd32(m + 8);
        const size_t nv = size_t(t->map_rank) * 2 * C, nu = size_t(t->map_rank) * C;
        e = hipMalloc(&t->map_v, nv);
        if (e == hipSuccess) e = hipMalloc(&t->map_u, nu);
        if (e == hipSuccess) e = hipMemcpyAsync(t->map_v, m + kMapHeader, nv, hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipMemcpyAsync(t->map_u, m + kMapHeader + nv, nu, hipMemcpyHostToDevice, st);
    }
    const size_t nbase = blob[7] == SKV_RESIDUAL_EXP ? size_t(rd32(blob + 12)) * rd32(blob + 16) : 0;
    if (e == hipSuccess && nbase) e = hipMalloc(&t->base, nbase);
    if (e == hipSuccess && nbase)
        e = hipMemcpyAsync(t->base, blob + kHeaderBytes + size_t(nt) * kTableRecord, nbase, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(rec, blob + kHeaderBytes, size_t(nt) * kTableRecord, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(expand_tables, dim3(nt), dim3(256), 0, st, rec, t->n, t->enc, t->fc, t->slot, t->tail,
                           t->tail_base, t->enc8);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (rec) (void)hipFree(rec);
    t->n_tables = nt;
    t->max_n = 0;
    for (uint32_t j = 0; j < nt; ++j) t->max_n = std::max(t->max_n, rd16(blob + kHeaderBytes + size_t(j) * kTableRecord));
    if (e != hipSuccess) free_dev_tables(t);
    return e;
}

void free_dev_tables(DevTables* t) {
    if (t->n) (void)hipFree(t->n);
    if (t->enc) (void)hipFree(t->enc);
    if (t->fc) (void)hipFree(t->fc);
    if (t->slot) (void)hipFree(t->slot);
    if (t->tail) (void)hipFree(t->tail);
    if (t->tail_base) (void)hipFree(t->tail_base);
    if (t->enc8) (void)hipFree(t->enc8);
    if (t->base) (void)hipFree(t->base);
    if (t->map_v) (void)hipFree(t->map_v);
    if (t->map_u) (void)hipFree(t->map_u);
    *t = DevTables{};
}

hipError_t launch_nbr_map(const int16_t* coef, const int16_t* G, int16_t* out, uint32_t T, uint32_t C,
                          const DevTables& t, hipStream_t st, const int16_t* right) {
    switch (t.map_rank) {
        case 16: return nbr_map_kt<1>(coef, G, out, T, C, t, st, right);
        case 32: return nbr_map_kt<2>(coef, G, out, T, C, t, st, right);
        case 64: return nbr_map_kt<4>(coef, G, out, T, C, t, st, right);
        case 128: return nbr_map_kt<8>(coef, G, out, T, C, t, st, right);
        case 256: return nbr_map_kt<16>(coef, G, out, T, C, t, st, right);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_encode(const EncodeLaunch& a, const DevTables& t, hipStream_t st, uint32_t phases) {
    if (is_checkerboard(a.shape.mode)) return encode_all<SKV_INT16, SKV_CHECKERBOARD>(a, t, st, phases);
    if (a.shape.mode == SKV_RESIDUAL_EXP)
        return a.shape.dtype == SKV_E4M3 ? encode_all<SKV_E4M3, SKV_RESIDUAL_EXP>(a, t, st, phases)
                                         : encode_all<SKV_BF16, SKV_RESIDUAL_EXP>(a, t, st, phases);
    if (a.shape.dtype == SKV_E4M3) return encode_all<SKV_E4M3, SKV_RESIDUAL>(a, t, st, phases);
    return encode_all<SKV_BF16, SKV_RESIDUAL>(a, t, st, phases);
}

hipError_t launch_decode(const DecodeLaunch& a, const DevTables& t, hipStream_t st) {
    if (is_checkerboard(a.shape.mode)) return decode_all<SKV_INT16, SKV_CHECKERBOARD>(a, t, st);
    if (a.shape.mode == SKV_RESIDUAL_EXP)
        return a.shape.dtype == SKV_E4M3 ? decode_all<SKV_E4M3, SKV_RESIDUAL_EXP>(a, t, st)
                                         : decode_all<SKV_BF16, SKV_RESIDUAL_EXP>(a, t, st);
    if (a.shape.dtype == SKV_E4M3) return decode_all<SKV_E4M3, SKV_RESIDUAL>(a, t, st);
    return decode_all<SKV_BF16, SKV_RESIDUAL>(a, t, st);
}

int timing_enable(bool on) {
    KernelTiming& T = g_timing;
    if (on == T.on) return SKV_OK;
    for (int i = 0; i < 2 * kMaxTimedKernels; ++i) {
        if (on) {
            if (hipEventCreate(&T.ev[i]) != hipSuccess) return SKV_ERR_DEVICE;
        } else if (T.ev[i]) {
            (void)hipEventDestroy(T.ev[i]);
            T.ev[i] = nullptr;
        }
    }
    T.on = on;
    T.count = T.done = 0;
    return SKV_OK;
}

void timing_reset() { g_timing.count = 0; }

void timing_collect() {
    KernelTiming& T = g_timing;
    if (!T.on) return;
    for (int i = 0; i < T.count; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, T.ev[2 * i], T.ev[2 * i + 1]) != hipSuccess) ms = -1.f;
        T.ms[i] = ms;
    }
    T.done = T.count;
}

int timing_read(const char** names, float* ms, int cap) {
    const KernelTiming& T = g_timing;
    int n = 0;
    for (; n < T.done && n < cap; ++n) {
        if (names) names[n] = T.name[n];
        if (ms) ms[n] = T.ms[n];
    }
    return n;
}

hipError_t launch_clear_u32(uint32_t* p, uint32_t n, hipStream_t st) {
    hipLaunchKernelGGL(clear_u32, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace skv
