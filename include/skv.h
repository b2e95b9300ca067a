/*
 * skv.h -- C ABI of libskv: lossless KV-cache coding on MI355X (gfx950).
 *
 * The library codes a target KV cache against a predictor cache that the
 * decoder can reproduce on its own, so only the residual is stored, and the
 * decoder returns the original bytes exactly ("Speculative KV coding:
 * losslessly compressing KV cache by up to ~4x", section "Core idea").
 * The residual is entropy-coded with rANS against static per-channel
 * discretized-Laplace tables fitted once on calibration data (same page,
 * "What to use as the predictor"; "DCKV compresses the prompt KV cache of
 * hybrid language models with learned transform coding", section "How it
 * differs": GPU rANS, Laplace integrated over quantization cells).  The
 * checkerboard mode codes DCKV-style transform coefficients whose Laplace is
 * shifted by a token-conditioned mean, even tokens first and odd tokens
 * from their decoded neighbours (DCKV page, "How it differs").
 *
 * Conventions for every call:
 *   - returns SKV_OK (0) or a negative skv_status; nothing is thrown;
 *   - "host" pointers are CPU memory, "device" pointers are HIP device
 *     memory of the current device; the caller owns every buffer it passes;
 *   - device work runs on the caller's hipStream_t (0 = legacy default);
 *   - on error, output buffers hold unspecified bytes, but nothing outside
 *     the given buffers is written.
 * Byte layouts of the table blob and of the container are fixed,
 * little-endian, and described next to the calls that produce them.
 */
#ifndef SKV_H
#define SKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKV_ABI_VERSION 1u

typedef enum {
    SKV_OK = 0,
    SKV_ERR_ARG = -1,      /* null / invalid argument, unknown blob pointer       */
    SKV_ERR_SHAPE = -2,    /* tokens or channels not multiples of the tile sizes,
                              dtype/mode combination not supported, ABI mismatch  */
    SKV_ERR_CAPACITY = -3, /* an output or work buffer is too small               */
    SKV_ERR_CORRUPT = -4,  /* container malformed or a stream fails its checks   */
    SKV_ERR_TABLES = -5,   /* table blob malformed, or not the one a container
                              was coded with (hash mismatch), or shape mismatch  */
    SKV_ERR_DEVICE = -6,   /* a HIP runtime call failed                           */
    SKV_ERR_NOMEM = -7,    /* host or device allocation failed                   */
    SKV_ERR_BUSY = -8      /* a store entry is pinned (in use)                   */
} skv_status;

typedef enum { SKV_BF16 = 1, SKV_E4M3 = 2, SKV_INT16 = 3 } skv_dtype;
typedef enum { SKV_RESIDUAL = 0, SKV_CHECKERBOARD = 1, SKV_RESIDUAL_EXP = 2, SKV_CHECKERBOARD_MAP = 3 } skv_mode;

/* Cache shape.  Residual mode: arrays are [layers][kv][tokens][channels]
 * of bf16 bit patterns (2 B) or e4m3 codes (1 B), channel fastest; tokens a
 * multiple of 128, channels a multiple of 32.  Checkerboard modes
 * (SKV_CHECKERBOARD, SKV_CHECKERBOARD_MAP): dtype SKV_INT16, layers = kv = 1,
 * arrays are [tokens][channels] int16 with tokens a multiple of 256.  SKV_RESIDUAL_EXP codes the same arrays as
 * SKV_RESIDUAL with tables conditioned on the predictor instead of the
 * channel (see skv_fit_tables).  abi_version must be SKV_ABI_VERSION. */
typedef struct {
    uint32_t abi_version;
    uint32_t dtype;      /* skv_dtype */
    uint32_t mode;       /* skv_mode  */
    uint32_t layers, kv, tokens, channels;
} skv_shape;

/* Fit the frequency tables once from calibration data (host only, fp64).
 *   calib_target, calib_aux (host):
 *     residual mode: target / predictor elements, [layers][kv][calib_tokens][channels];
 *     checkerboard:  int16 coefficients / int16 side input G (each token's
 *                    mean in 1/16 cells), [calib_tokens][channels], calib_tokens even.
 *   s->tokens is ignored.
 * Each table is a Laplace integrated over unit cells (location 0, or f/16
 * for shifted table f in checkerboard mode; scale = mean |residual| over
 * calibration values with |residual| <= 127, floored at 0.05), with a direct
 * range of n symbols z = 0..n-1 and an escape symbol (index n) whose
 * probability is the smoothed calibration escape rate (#z >= n + 1) / (N + 2),
 * quantized to 12-bit frequencies >= 1 summing to 4096 (largest remainder,
 * ties to the smaller index).  n is 1 + the largest z <= 254 whose cell mass
 * is at least 2^-12, raised in residual modes to the slab's calibration tail
 * floor -- the smallest z in [1, 255] such that at most floor(N / 1024) of the
 * N calibration symbols of the table's (layer, K|V) slab are z or larger --
 * and at most 255.
 * SKV_RESIDUAL_EXP (a finer residual model, "Speculative KV coding" page,
 * "Early results"; conditional models, DCKV page, "How it differs"): one
 * table per (layer, K|V) slab and predictor exponent class -- the class of a
 * value is its predictor's exponent field (bf16 bits 14..7, e4m3 bits 6..3)
 * minus the slab's base, clamped to [0, 15]; the base starts the window of
 * 16 exponents that holds the most calibration predictors (the lowest such
 * window); each table is the Laplace above fitted to the slab's calibration
 * values of its class (the slab's pooled scale when fewer than 64 of them
 * have |residual| <= 127), with the slab's tail floor and the class's escape
 * rate.  Its blob has layers * kv * 16 records followed by one base byte per
 * slab.
 * On success *tables_blob points to a library-owned, immutable blob of
 * *blob_bytes bytes (layout: 64 B header "SKVT" | u16 version | u8 dtype |
 * u8 mode | u32 n_tables | u32 layers | u32 kv | u32 channels | u32
 * calib_tokens | u32 0 | u64 total bytes | 24 B zero; then n_tables records
 * of u16 n, u16 freq[256]).  Release it with skv_free. */
int skv_fit_tables(const skv_shape* s, const void* calib_target, const void* calib_aux,
                   uint32_t calib_tokens, void** tables_blob, size_t* blob_bytes);

/* Tables of SKV_CHECKERBOARD_MAP, the checkerboard mode with a map over the
 * decoded neighbours (DCKV page, "How it differs": an odd position is
 * predicted from both decoded neighbours and its own token embedding through
 * a low-rank linear map).  The embedding part is the side input G, as in
 * SKV_CHECKERBOARD; the neighbour part is a rank-k map in exact integer
 * arithmetic whose output, in 1/16 cells, is added to an odd token's side
 * input before its mean is formed:
 *   n      = the token's left row then its right row (2 * channels values;
 *            the last odd token repeats its left row), each saturated to
 *            at most 32639
 *   q_j    = sum_i V[j][i] n_i / 2^shift_h rounded half up, clamped to
 *            [-128, 127]                                       (j < rank)
 *   m_c    = sum_j U[c][j] q_j / 2^shift_m rounded half up
 *   G'[t][c] = G[t][c] + m_c clamped to [-32768, 32767]
 * and the odd token's mean (1/16 cells) is G' + 8 * (left + right), as in
 * SKV_CHECKERBOARD, which this mode equals when U is zero.  The tables are
 * those of skv_fit_tables fitted with G' in place of G on the odd
 * calibration tokens (the map applied to the calibration's own even rows).
 *   calib_coef, calib_G (host): [calib_tokens][channels] int16, calib_tokens even.
 *   map (host): rank a power of two from 16 to 256, shift_h <= 40,
 *     shift_m <= 30 (else SKV_ERR_ARG); V int8 [rank][2 * channels] and U
 *     int8 [channels][rank], row-major, copied into the blob.
 * The blob is that of skv_fit_tables (mode byte 3) followed by the map:
 * u32 rank | u32 shift_h | u32 shift_m | u32 0 | V | U.  The codec computes
 * the map between its two passes on the GPU's int8 matrix units (exact:
 * 32-bit sums); encoding needs tokens * channels * 2 more workspace bytes,
 * decoding writes G' into the output's odd rows before decoding them. */
typedef struct {
    uint32_t rank;
    uint32_t shift_h;
    uint32_t shift_m;
    const int8_t* V;
    const int8_t* U;
} skv_nbr_map;
int skv_fit_tables_map(const skv_shape* s, const void* calib_coef, const void* calib_G, uint32_t calib_tokens,
                       const skv_nbr_map* map, void** tables_blob, size_t* blob_bytes);

/* Copy a blob produced elsewhere (same layout as above) into a library-owned
 * blob after validating it: every table has 1 <= n <= 255, freq[0..n] >= 1
 * summing to 4096 and zeros beyond (and, for SKV_CHECKERBOARD_MAP, a valid
 * map section).  Release with skv_free. */
int skv_load_tables(const void* blob, size_t blob_bytes, void** tables_blob);

/* Encode (device).  The sender codes the residual of the target cache
 * against the predictor's cache with an entropy coder ("Speculative KV
 * coding" page, section "Core idea", flow steps 1-2: the sender has the
 * target and predictor caches and entropy-codes their difference); the coder is rANS
 * against the fitted tables (DCKV page, "How it differs").  d_target and
 * d_aux (predictor, or G in checkerboard mode) are device arrays of the
 * shape's layout; neither is written.  Residual of a value: r = (ord t - ord
 * p) mod 2^N read as signed (N = 16 for bf16, 8 for e4m3; ord maps a sign-
 * magnitude pattern to an order-preserving integer), symbol z = zigzag(r).
 * Stream s = (slab * token blocks + token block) * channel groups + channel
 * group; lane i codes channel 32 * group + i, step k token 128 * block + k
 * (checkerboard: the slab is the pass, token 2 * (128 * block + k) + pass).
 * The container written to d_out:
 *   64 B header: "SKV1" | u16 1 | u8 dtype | u8 mode | u8 12 | u8 32 | u16 128 |
 *                u32 layers | u32 kv | u32 tokens | u32 channels | u32 0 |
 *                u64 n_streams | u64 FNV-1a-64 of the blob | u64 payload bytes | u64 0
 *   index: (n_streams+1) u64 payload offsets, bit 63 = stream stored raw,
 *          last entry = payload bytes
 *   payload: streams (32 lanes x 128 steps) in id order.  A coded stream is
 *          32 u32 final rANS states (lane order) | u32 word count W | W u16
 *          words in decode order (by step, then lane) | the escaped values
 *          (z >= the lane's direct count: u16 for 16-bit elements, u8 for
 *          e4m3) in decode order | zero bytes up to a multiple of 4.  A stream
 *          whose coded size would reach its raw size is stored raw: its 4096
 *          target elements in (step, lane) order.
 * Two-phase sizing: with d_out == NULL, *out_bytes receives the bound (every
 * stream raw); with d_work == NULL, *work_bytes receives the workspace need
 * of a single pass over the cache.  Otherwise out_capacity must hold the
 * container (else SKV_ERR_CAPACITY and *out_bytes = the size needed).  A
 * workspace smaller than the single-pass need codes the cache in passes of
 * whole (layer, K|V) slabs, or of whole token blocks of one slab, that fit
 * in it, one after another into the same workspace; the container is the
 * same.  Below one token block's need (and, for checkerboard shapes, below
 * the single-pass need) the call returns SKV_ERR_CAPACITY with *work_bytes
 * = the smallest workable size (see skv_encode_workspace).  Blocks the host
 * until the container size is known (one stream synchronization). */
int skv_encode(const void* tables_blob, const skv_shape* s, const void* d_target, const void* d_aux,
               void* d_out, size_t out_capacity, size_t* out_bytes,
               void* d_work, size_t* work_bytes, hipStream_t stream);

/* Encoder workspace for a memory budget (host only; no device call): with
 * max_bytes == 0 or at least the single-pass need, *work_bytes = that need
 * and *passes = 1; below it, the workspace skv_encode uses when given
 * max_bytes and the number of passes it then makes; below the smallest
 * workable size, SKV_ERR_CAPACITY with *work_bytes = that size. */
int skv_encode_workspace(const skv_shape* s, uint64_t max_bytes, size_t* work_bytes, uint32_t* passes);

/* Encode without allocating (device), for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same container as skv_encode for the
 * same inputs and blob; the workspace is a fixed array of
 * SKV_NOALLOC_WORK_BYTES that the library keeps on every device it runs on
 * until the process ends, so no workspace argument is taken and nothing is
 * allocated or freed by the call.
 *   - The cache is coded in as many passes as the array needs (as
 *     skv_encode does with a workspace of SKV_NOALLOC_WORK_BYTES: 64 MiB
 *     holds about 8,000 e4m3 or 4,000 bf16 streams of 4096 values per
 *     pass); a checkerboard shape, which takes one pass, whose workspace
 *     exceeds the array returns SKV_ERR_SHAPE.
 *   - The blob's device tables must already be on the current device (any
 *     earlier skv_encode, skv_decode, skv_decode_range or skv_transfer with
 *     this blob on this device puts them there; building them allocates),
 *     else SKV_ERR_ARG.
 *   - d_out == NULL sets *out_bytes to the bound; else out_capacity must
 *     hold the container (SKV_ERR_CAPACITY, *out_bytes = the size needed).
 *   - Calls on one device share its array.  The library runs them one at a
 *     time (each returns only after its kernels have finished with the
 *     array), so calls from several threads do not race; the array keeps the
 *     last call's contents, none of which a call reads before writing it.
 * Blocks the host until the container size is known. */
#define SKV_NOALLOC_WORK_BYTES (64u << 20)
int skv_encode_noalloc(const void* tables_blob, const skv_shape* s, const void* d_target, const void* d_aux,
                       void* d_out, size_t out_capacity, size_t* out_bytes, hipStream_t stream);

/* Decode (device).  The receiver replays the predictor, decodes the
 * residual and adds it back, which returns the original bytes exactly
 * ("Speculative KV coding" page, section "Core idea", flow steps 3-4; the stored
 * cache is restored in full before use, DCKV page, "How it works").  d_in holds in_bytes of container;
 * d_aux is the predictor (or G) in the shape's layout, with at least
 * out_capacity bytes readable; d_out receives the reconstruction
 * (out_capacity bytes available).  The shape comes from the header, which is
 * validated against the blob (hash, dtype, mode, layers, kv, channels).
 * With d_work == NULL, *work_bytes receives the workspace need.  Every
 * stream checks that its rANS states end at 2^16 and that it consumed its
 * words exactly; any failure returns SKV_ERR_CORRUPT.  Checkerboard
 * containers decode in two launches on the same stream: even tokens, then
 * odd tokens.  Blocks the host to read the header and the integrity word. */
int skv_decode(const void* tables_blob, const void* d_in, size_t in_bytes, const void* d_aux,
               void* d_out, size_t out_capacity, void* d_work, size_t* work_bytes, hipStream_t stream);

/* Decode a token range (device).  A stored shared prefix, such as a system
 * prompt, is reused by restoring the part of its cache that a request needs
 * ("Speculative KV coding" page, section "Where it can be used": prefix
 * caching; VeriCache page, "Application to remote prefix caching"); the
 * container's offset index locates the streams of the range, so nothing
 * outside it is read or decoded.
 *   token_begin, token_end: the tokens [token_begin, token_end), with
 *     token_begin < token_end <= the container's tokens (else SKV_ERR_SHAPE).
 *   Residual modes (either table kind): both multiples of 128, the range of
 *     every (layer, K|V) slab; d_aux and d_out are device arrays
 *     [layers][kv][token_end - token_begin][channels] -- the predictor of the
 *     range and its reconstruction (out_capacity bytes available).
 *   Checkerboard modes: both multiples of 256 (a block of 128 even and 128
 *     odd tokens), the range under 2 GiB; d_out is [token_end - token_begin]
 *     [channels].  The last odd token of the range needs the even token
 *     token_end, whose stream is decoded whole, so unless token_end is the
 *     container's last token d_aux holds the side input G of tokens
 *     [token_begin, token_end + 256) -- the range then the next block --
 *     else of [token_begin, token_end).  The workspace need is 256 +
 *     512 * channels bytes (the next block's even rows).
 * Header and blob rules as for skv_decode.  Every stream decoded is checked
 * as in skv_decode (SKV_ERR_CORRUPT); streams outside the range are not
 * read, so damage there goes unnoticed.  Blocks the host to read the header
 * and the integrity word. */
int skv_decode_range(const void* tables_blob, const void* d_in, size_t in_bytes, uint32_t token_begin,
                     uint32_t token_end, const void* d_aux, void* d_out, size_t out_capacity, void* d_work,
                     size_t* work_bytes, hipStream_t stream);

/* Transfer pipeline (device -> host -> device).  Moving a prefilled cache
 * to the server that decodes ("Speculative KV coding" page, section "Where
 * it can be used": disaggregated prefill over a slow link) with its copies
 * and the GPU work on separate streams so that they overlap (VeriCache page,
 * "Hardware basis of the parallel execution").  The cache is cut into chunks
 * of layers_per_chunk whole layers (the last chunk may be shorter); chunk c
 * is encoded into a container of its own (the tables of its layers, as a
 * blob of those layers that skv_free releases with tables_blob), copied to
 * the host buffer h_wire, copied back to the device and decoded into d_out,
 * while chunk c + 1 is being encoded.  The sender encodes on the calling
 * thread; a receiver thread started and joined by this call copies back and
 * decodes.  Residual-mode shapes (either table kind) only, else
 * SKV_ERR_SHAPE.
 *   d_target, d_aux_send: the sender's cache and predictor, device arrays of
 *     shape s.
 *   h_wire: host memory of wire_capacity bytes (page-locked, e.g. from
 *     hipHostMalloc, for the copies to overlap; pageable memory works but
 *     serializes them).  Receives the chunk containers back to back;
 *     chunk_offsets (host, ceil(layers / layers_per_chunk) + 1 entries)
 *     receives each one's byte offset and, last, the total, also stored in
 *     *wire_bytes.  Each chunk container decodes on its own with
 *     skv_decode and the tables of its layers.
 *   d_aux_recv, d_out: the receiver's predictor (shape s) and the
 *     reconstruction (out_capacity bytes available).
 *   d_work: device workspace of *work_bytes bytes: two container buffers on
 *     each side plus the encoder's and decoder's workspaces.
 * Two-phase sizing as in skv_encode: h_wire == NULL sets *wire_bytes to the
 * bound (every stream raw), d_work == NULL sets *work_bytes to the need.
 * layers_per_chunk must be 1..layers (SKV_ERR_ARG).  Per-kernel timing must
 * be off (SKV_ERR_ARG), since its state is process-wide.  A chunk that does
 * not fit in the rest of h_wire stops the pipeline with SKV_ERR_CAPACITY and
 * *wire_bytes = the bound; any encode or decode error stops it with that
 * status; either way d_out is then unspecified.  The caller's stream is
 * ordered before the pipeline's streams; the call returns once every copy
 * and kernel it queued has finished. */
int skv_transfer(const void* tables_blob, const skv_shape* s, uint32_t layers_per_chunk, const void* d_target,
                 const void* d_aux_send, void* h_wire, size_t wire_capacity, size_t* wire_bytes,
                 uint64_t* chunk_offsets, const void* d_aux_recv, void* d_out, size_t out_capacity, void* d_work,
                 size_t* work_bytes, hipStream_t stream);

/* Prefix-cache store.  Keeping the caches of shared prefixes (system
 * prompts, retrieved documents) compressed lets the same memory hold more of
 * them, which raises the hit rate ("Speculative KV coding" page, section
 * "Where it can be used": prefix caching; VeriCache page, "Application to
 * remote prefix caching"); a request restores only the prefix it shares
 * through skv_decode_range.  A store keeps containers in an arena the caller
 * owns and allocates no device memory itself (the arena outlives the store;
 * the store never reads or writes arena bytes except through skv_store_put
 * and skv_store_decode).
 *
 * Entries are keyed by block hashes: hashes[b] identifies tokens
 * [128 b, 128 b + 128) together with everything before them (a chained hash
 * of the token ids, for instance), so two caches share their first m blocks
 * exactly when their first m hashes are equal.  A lookup returns the entry
 * holding the longest leading run of the query's hashes (ties: the most
 * recently used), checking all of that run's hashes, not only the last.
 *
 * Space: the arena is cut into 256-byte granules; an entry takes its
 * container rounded up, at the lowest free offset where it fits.  When no
 * free run is long enough, entries are evicted least recently used first
 * (use = commit or lookup hit) until one is; pinned entries and open
 * reservations are never evicted, and if evicting every other entry still
 * would not make room, nothing is evicted and the call returns
 * SKV_ERR_CAPACITY.  Entry ids start at 1 and are never reused.  Calls on
 * one store may come from several threads (a mutex serializes the
 * bookkeeping; skv_store_put and skv_store_decode run their GPU work
 * outside it).
 *
 *   skv_store_create: arena (256-byte aligned, else SKV_ERR_ARG) of
 *     arena_bytes (a multiple of 256, at least 256).  *store receives the
 *     handle; release it with skv_store_destroy (entries are dropped, the
 *     arena is not touched).
 *   skv_store_reserve: room for a container of `bytes` that the caller
 *     writes itself (for instance one received from another server); *entry
 *     and *addr receive the id and the arena address.  The entry stays out
 *     of lookups and eviction until skv_store_commit (the caller has
 *     finished writing) or skv_store_abort.  nblocks 1..2^20 hashes are
 *     copied (SKV_ERR_ARG otherwise).
 *   skv_store_commit: the reservation holds `bytes` (at most the reserved
 *     size) of container; the unused granules return to the free space and
 *     the entry becomes visible and most recently used.
 *   skv_store_abort: drop a reservation.
 *   skv_store_put (device): encode a cache into the store -- skv_encode's
 *     arguments, the container placed once its size is known (the streams
 *     are coded into d_work, the space reserved, then the container written
 *     there) -- and commit it with nblocks = tokens / 128 hashes (else
 *     SKV_ERR_ARG).  d_work == NULL sets *work_bytes to the need
 *     (skv_encode's).  Blocks until the entry is committed; *entry and
 *     *container_bytes receive its id and size.
 *   skv_store_lookup: *hit receives the best entry for the query (entry 0
 *     and matched_blocks 0 on a miss).  A hit pins the entry (it cannot be
 *     evicted or erased) until skv_store_release.
 *   skv_store_decode (device): decode tokens [token_begin, token_end) of an
 *     entry through skv_decode_range (token_end == 0: the whole container
 *     through skv_decode), with that call's arguments and rules (workspace
 *     sizing included); the entry is pinned during the call.
 *   skv_store_erase: remove an entry now (SKV_ERR_BUSY while pinned).
 *   Unknown or already removed ids return SKV_ERR_ARG. */
typedef struct skv_store skv_store;
typedef struct {
    uint64_t entry;            /* 0 on a miss                               */
    uint32_t matched_blocks;   /* leading query blocks the entry holds      */
    uint32_t entry_blocks;     /* blocks the entry holds                    */
    const void* container;     /* its container in the arena                */
    uint64_t container_bytes;
} skv_store_hit;
typedef struct {
    uint64_t arena_bytes;
    uint64_t used_bytes;       /* granules held by entries and reservations */
    uint64_t largest_free;     /* longest free run                          */
    uint64_t container_bytes;  /* committed entries' container bytes        */
    uint64_t entries;          /* committed entries                         */
    uint64_t pinned;           /* committed entries pinned by lookups       */
    uint64_t inserts, evictions, hits, misses, hit_blocks;
} skv_store_info;
int skv_store_create(void* arena, uint64_t arena_bytes, skv_store** store);
void skv_store_destroy(skv_store* store);
int skv_store_reserve(skv_store* store, const uint64_t* hashes, uint32_t nblocks, uint64_t bytes, uint64_t* entry,
                      void** addr);
int skv_store_commit(skv_store* store, uint64_t entry, uint64_t bytes);
int skv_store_abort(skv_store* store, uint64_t entry);
int skv_store_put(skv_store* store, const uint64_t* hashes, uint32_t nblocks, const void* tables_blob,
                  const skv_shape* s, const void* d_target, const void* d_aux, void* d_work, size_t* work_bytes,
                  hipStream_t stream, uint64_t* entry, uint64_t* container_bytes);
int skv_store_lookup(skv_store* store, const uint64_t* hashes, uint32_t nblocks, skv_store_hit* hit);
int skv_store_release(skv_store* store, uint64_t entry);
int skv_store_decode(skv_store* store, const void* tables_blob, uint64_t entry, uint32_t token_begin,
                     uint32_t token_end, const void* d_aux, void* d_out, size_t out_capacity, void* d_work,
                     size_t* work_bytes, hipStream_t stream);
int skv_store_erase(skv_store* store, uint64_t entry);
int skv_store_stats(skv_store* store, skv_store_info* stats);

/* Release a library-owned blob and its device copies.  NULL is a no-op. */
void skv_free(void* tables_blob);

/* Diagnostics.  skv_kernel_timing(1) creates HIP events on the current
 * device; from then on every skv_encode / skv_decode records an event pair
 * around each kernel it launches on the caller's stream.
 * skv_kernel_times fills names[i] (static strings) and ms[i] (elapsed
 * milliseconds) for the kernels of the last call, in launch order, and
 * returns their count (at most `capacity`; either array may be NULL).
 * skv_kernel_timing(0) releases the events.  Process-wide state: callers
 * encoding concurrently should not enable it. */
int skv_kernel_timing(int enable);
int skv_kernel_times(const char** names, float* ms, int capacity);

/* Library ABI version (SKV_ABI_VERSION) and a static message per status. */
uint32_t skv_version(void);
const char* skv_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* SKV_H */
