/*
 * skv_oracle.c -- plain, slow, scalar CPU oracle for lossless KV-cache coding.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table
 * or constant generator with the GPU path: both are written independently
 * from the same format description.
 *
 * Sources (web pages; cited by title and section):
 *   [SKC]  "Speculative KV coding: losslessly compressing KV cache by up to
 *          ~4x" (Korean summary, aisparkup.com/posts/13411).  Sections used:
 *          "Core idea of Speculative KV Coding" (cache is a deterministic
 *          function of prompt and weights; code the residual between the
 *          target cache and a predictor's cache with an arithmetic coder; the
 *          decoder replays the predictor and adds the residual back),
 *          "What to use as the predictor" (residual statistics are measured
 *          once on a little calibration data and then frozen).
 *   [DCKV] "DCKV compresses the prompt KV cache of hybrid language models
 *          with learned transform coding" (onedev.kr/papers/1428).  Section
 *          "How it differs": entropy coding is GPU rANS; the static model is
 *          a per-component Laplace integrated over the quantization cells;
 *          a token-conditioned model shifts each coefficient's Laplace by a
 *          predicted mean; a checkerboard context model codes even positions
 *          from the token condition alone and odd positions from their two
 *          already decoded neighbours plus their own token embedding, so
 *          decoding takes two token-parallel passes.
 *   [VeriCache] "VeriCache" (llm-wiki.hwlabs.dev, ai-frontier 91), section
 *          "Compressor interface": a compressor must be deterministic.
 *
 * The pages fix none of the bit-level details; every such choice below is a
 * reading of the pages (rANS with 12-bit probabilities, 32 interleaved
 * lanes x 128 steps per stream, ordered-integer residual with zigzag, escape
 * symbol whose raw value is stored in the stream's escape region, raw
 * fallback, container and table-blob layout).  The rANS steps follow the published definition of range
 * asymmetric numeral systems (J. Duda, "Asymmetric numeral systems",
 * arXiv:1311.2540) with word-wise renormalization and lane interleaving as
 * in F. Giesen, "Interleaved entropy coders" (arXiv:1402.3392).
 *
 * Everything here is integer except the table fit, which is fp64 and fixes
 * its order of operations so that an independent implementation following
 * the same description reaches the same integer frequencies.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SKVO_M 4096u          /* 2^12: total of every frequency table        */
#define SKVO_L 65536u         /* lower end of the normalized state interval */
#define SKVO_LANES 32
#define SKVO_STEPS 128
#define SKVO_SYMS (SKVO_LANES * SKVO_STEPS)
#define SKVO_MAX_DIRECT 255
#define SKVO_HDR 64
#define SKVO_TAB_BYTES 514    /* u16 n + u16 freq[256] */

enum { DT_BF16 = 1, DT_E4M3 = 2, DT_INT16 = 3 };
enum { MODE_RESIDUAL = 0, MODE_CHECKERBOARD = 1, MODE_RESIDUAL_EXP = 2, MODE_CHECKERBOARD_MAP = 3 };
enum { E_OK = 0, E_ARG = -1, E_SHAPE = -2, E_CAPACITY = -3, E_CORRUPT = -4, E_TABLES = -5 };

/* ------------------------------------------------------------------ */
/* Little-endian byte helpers                                          */
/* ------------------------------------------------------------------ */
static void put16(uint8_t* p, uint32_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put32(uint8_t* p, uint32_t v) { for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static void put64(uint8_t* p, uint64_t v) { for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static uint32_t get16(const uint8_t* p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }
static uint32_t get32(const uint8_t* p) {
    uint32_t v = 0;
    for (int i = 3; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}
static uint64_t get64(const uint8_t* p) {
    uint64_t v = 0;
    for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}

/* FNV-1a, 64-bit: identifies the table blob inside a container. */
uint64_t skvo_fnv1a64(const uint8_t* p, size_t n) {
    uint64_t h = 0xcbf29ce484222325ull;
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 0x100000001b3ull;
    }
    return h;
}

/* ------------------------------------------------------------------ */
/* Symbolizer.  [SKC] "Core idea": code the difference between the true  */
/* cache and the predictor's cache.  Reading: the difference is taken on  */
/* order-preserving integers of the element bit patterns, modulo 2^N.    */
/* ------------------------------------------------------------------ */

/* Order-preserving map of an N-bit sign-magnitude float pattern to an
 * unsigned integer: non-negative patterns move above all negative ones,
 * negative patterns are mirrored so that larger magnitude means smaller. */
uint32_t skvo_ord(uint32_t u, int nbits) {
    uint32_t top = 1u << (nbits - 1);
    uint32_t all = (nbits == 32) ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
    if (u & top) return u ^ all;   /* negative: flip every bit */
    return u ^ top;                /* non-negative: set the top bit */
}

uint32_t skvo_inv_ord(uint32_t o, int nbits) {
    uint32_t top = 1u << (nbits - 1);
    uint32_t all = (1u << nbits) - 1u;
    if (o & top) return o ^ top;
    return o ^ all;
}

/* Signed residual r in [-2^(N-1), 2^(N-1)) with ord(t) = ord(p) + r mod 2^N. */
int32_t skvo_residual(uint32_t t, uint32_t p, int nbits) {
    int64_t span = (int64_t)1 << nbits;
    int64_t d = ((int64_t)skvo_ord(t, nbits) - (int64_t)skvo_ord(p, nbits)) % span;
    if (d < 0) d += span;
    if (d >= span / 2) d -= span;
    return (int32_t)d;
}

/* Zigzag: 0,-1,1,-2,2,... -> 0,1,2,3,4,... */
uint32_t skvo_zigzag(int32_t r) {
    if (r >= 0) return 2u * (uint32_t)r;
    return 2u * (uint32_t)(-(int64_t)r) - 1u;
}

int32_t skvo_unzigzag(uint32_t z) {
    if ((z & 1u) == 0) return (int32_t)(z / 2u);
    return -(int32_t)((z + 1u) / 2u);
}

/* Inverse of the residual: element pattern t from predictor p and r. */
uint32_t skvo_reconstruct(uint32_t p, int32_t r, int nbits) {
    int64_t span = (int64_t)1 << nbits;
    int64_t o = ((int64_t)skvo_ord(p, nbits) + r) % span;
    if (o < 0) o += span;
    return skvo_inv_ord((uint32_t)o, nbits);
}

/* Exponent class of a predictor element (exponent-conditioned residual
 * tables).  [DCKV] "How it differs": the static per-component model gives way
 * to models conditioned on what the decoder already knows; [SKC] "Early
 * results" leaves a finer residual model open.  Reading: the residual of a
 * value is modelled by a table chosen by its predictor's exponent field
 * (bf16: bits 14..7, e4m3: bits 6..3), as the class E - base clamped to
 * [0, 15], with base fixed per (layer, K|V) slab at fit time. */
uint32_t skvo_exp_class(uint32_t p, int dtype, uint32_t base) {
    uint32_t e = (dtype == DT_E4M3) ? ((p >> 3) & 0xFu) : ((p >> 7) & 0xFFu);
    uint32_t c = e < base ? 0u : e - base;
    return c > 15u ? 15u : c;
}

/* [DCKV] "How it differs": a predicted mean shifts the Laplace.  Reading:
 * the mean is held in 1/16-cell units mu_q; its integer part k (floor) shifts
 * the coefficient, its sixteenths f choose one of 16 shifted tables. */
void skvo_dckv_split(int32_t mu_q, int32_t* k, int32_t* f) {
    int32_t kk;
    if (mu_q >= 0) kk = mu_q / 16;
    else kk = -((-mu_q + 15) / 16);   /* floor for negative values */
    *k = kk;
    *f = mu_q - 16 * kk;
}

/* Map a signed value to int16 by wrapping modulo 2^16. */
static int32_t wrap16(int64_t v) {
    int64_t w = v % 65536;
    if (w < 0) w += 65536;
    if (w >= 32768) w -= 65536;
    return (int32_t)w;
}

/* Coefficient c (int16) with mean mu_q -> (symbol value z, table index f). */
uint32_t skvo_dckv_symbol(int32_t c, int32_t mu_q, int32_t* f_out) {
    int32_t k, f;
    skvo_dckv_split(mu_q, &k, &f);
    *f_out = f;
    return skvo_zigzag(wrap16((int64_t)c - k));
}

int32_t skvo_dckv_reconstruct(uint32_t z, int32_t mu_q) {
    int32_t k, f;
    skvo_dckv_split(mu_q, &k, &f);
    return wrap16((int64_t)k + skvo_unzigzag(z));
}

/* Mean (1/16 cells) of coefficient (t, comp): even tokens take the side
 * input G; odd tokens add the mean of their two even neighbours, given in
 * sixteenths as 8 * (left + right).  The last odd token has no right
 * neighbour and repeats its left one. */
int32_t skvo_dckv_mean(const int16_t* coef, const int16_t* G, uint32_t T, uint32_t C,
                       uint32_t t, uint32_t comp) {
    int32_t mu = G[(size_t)t * C + comp];
    if (t & 1u) {
        int32_t left = coef[(size_t)(t - 1) * C + comp];
        int32_t right = (t + 1 < T) ? coef[(size_t)(t + 1) * C + comp] : left;
        mu += 8 * (left + right);
    }
    return mu;
}

/* Decoded-neighbour map.  [DCKV] "How it differs": an odd position is
 * predicted from both of its already decoded neighbours and its own token
 * embedding through a low-rank linear map.  Reading: the embedding part is
 * the side input G (as above); the neighbour part is a rank-k map applied to
 * the two decoded neighbour rows in exact integer arithmetic, whose output,
 * in 1/16 cells, is added to the odd token's side input:
 *   n        the left row then the right row of the odd token (2C values;
 *            the last odd token repeats its left row), each value saturated
 *            to at most 32639
 *   h_j      = sum over i < 2C of V[j][i] * n_i               (exact)
 *   q_j      = h_j / 2^sh1 rounded half up, clamped to [-128, 127]
 *   m_c      = (sum over j < k of U[c][j] * q_j) / 2^sh2 rounded half up
 *   G'[t][c] = G[t][c] + m_c clamped to [-32768, 32767]
 * V is int8 [k][2C] and U int8 [C][k], both row-major.  Even tokens keep
 * G.  The mean of an odd coefficient is then G' + 8 * (left + right), as in
 * the checkerboard mode, which the map reduces to when U is zero. */
typedef struct {
    uint32_t k, sh1, sh2;
    const int8_t* V;
    const int8_t* U;
} skvo_map;

/* v / 2^s rounded half up: floor((v + 2^(s-1)) / 2^s). */
static int64_t round_shift(int64_t v, uint32_t s) {
    if (s == 0) return v;
    int64_t d = (int64_t)1 << s;
    int64_t a = v + d / 2;
    int64_t q = a / d;
    if (a % d != 0 && a < 0) q -= 1;   /* C division truncates toward zero */
    return q;
}

static int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* Side input with the map applied: Gout[t] = G[t] on even tokens, G'[t] on
 * odd ones, computed from the even rows of `coef`. */
static void dckv_map_side(const int16_t* coef, const int16_t* G, uint32_t T, uint32_t C, const skvo_map* m,
                          int16_t* Gout, int nthreads) {
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 8) num_threads(nthreads)
    for (int64_t tt = 0; tt < (int64_t)T; ++tt) {
        uint32_t t = (uint32_t)tt;
        const int16_t* g = G + (size_t)t * C;
        int16_t* o = Gout + (size_t)t * C;
        if (!(t & 1u)) {
            memcpy(o, g, (size_t)C * sizeof(int16_t));
            continue;
        }
        uint32_t left = t - 1, right = (t + 1 < T) ? t + 1 : t - 1;
        int64_t* n = (int64_t*)malloc(2 * (size_t)C * sizeof(int64_t));
        int64_t* q = (int64_t*)malloc((size_t)m->k * sizeof(int64_t));
        for (uint32_t i = 0; i < C; ++i) {
            int64_t a = coef[(size_t)left * C + i], b = coef[(size_t)right * C + i];
            n[i] = a > 32639 ? 32639 : a;
            n[C + i] = b > 32639 ? 32639 : b;
        }
        for (uint32_t j = 0; j < m->k; ++j) {
            int64_t h = 0;
            for (uint32_t i = 0; i < 2 * C; ++i) h += (int64_t)m->V[(size_t)j * 2 * C + i] * n[i];
            q[j] = clamp64(round_shift(h, m->sh1), -128, 127);
        }
        for (uint32_t c = 0; c < C; ++c) {
            int64_t acc = 0;
            for (uint32_t j = 0; j < m->k; ++j) acc += (int64_t)m->U[(size_t)c * m->k + j] * q[j];
            o[c] = (int16_t)clamp64((int64_t)g[c] + round_shift(acc, m->sh2), -32768, 32767);
        }
        free(n);
        free(q);
    }
}

/* The map on caller-supplied arrays (tests): coef, G and Gout are [T][C]. */
int skvo_dckv_map(const int16_t* coef, const int16_t* G, uint32_t T, uint32_t C, uint32_t k, uint32_t sh1,
                  uint32_t sh2, const int8_t* V, const int8_t* U, int16_t* Gout, int nthreads) {
    if (!coef || !G || !V || !U || !Gout || k == 0 || sh1 > 40 || sh2 > 30) return E_ARG;
    skvo_map m = {k, sh1, sh2, V, U};
    dckv_map_side(coef, G, T, C, &m, Gout, nthreads);
    return E_OK;
}

/* ------------------------------------------------------------------ */
/* Frequency tables                                                    */
/* ------------------------------------------------------------------ */
typedef struct {
    uint32_t n;              /* direct symbols 0..n-1; symbol n is ESC */
    uint32_t freq[257];
    uint32_t cum[258];
} skvo_table;

static void table_cum(skvo_table* t) {
    t->cum[0] = 0;
    for (uint32_t s = 0; s <= t->n; ++s) t->cum[s + 1] = t->cum[s] + t->freq[s];
}

/* ------------------------------------------------------------------ */
/* rANS primitive (single lane).  Duda's range variant with 12-bit      */
/* probabilities, 32-bit state kept in [2^16, 2^32) and 16-bit words.   */
/* ------------------------------------------------------------------ */

/* Push one symbol (frequency f, cumulative start c) into state *x.  When the
 * state is too large to absorb the symbol, its low 16 bits leave first;
 * returns 1 and stores them in *w in that case. */
int skvo_rans_put(uint32_t* x, uint32_t f, uint32_t c, uint16_t* w) {
    int out = 0;
    if ((uint64_t)*x >= ((uint64_t)f << 20)) {
        *w = (uint16_t)(*x & 0xFFFFu);
        *x >>= 16;
        out = 1;
    }
    *x = (*x / f) * SKVO_M + (*x % f) + c;
    return out;
}

/* Pop: the symbol whose slot range holds x mod 2^12, given the table's
 * frequency and cumulative arrays; x is updated, no renormalization. */
uint32_t skvo_rans_pop(uint32_t* x, const uint32_t* freq, const uint32_t* cum, uint32_t nsym) {
    uint32_t slot = *x & (SKVO_M - 1u);
    uint32_t s = 0;
    while (s + 1 < nsym && cum[s + 1] <= slot) ++s;
    *x = freq[s] * (*x >> 12) + slot - cum[s];
    return s;
}

/* ------------------------------------------------------------------ */
/* One stream: 32 interleaved lanes x `steps` steps.                   */
/*   z[k*32 + i]   symbol value of lane i at step k                     */
/*   tab[k*32 + i] table used by lane i at step k                       */
/*   ebytes        bytes of an escaped value (2 for 16-bit elements,    */
/*                 1 for 8-bit ones)                                    */
/* A value z < n is coded directly as symbol z; a larger one codes the  */
/* ESC symbol (index n) and its raw value goes to the stream's escape   */
/* region.  Decode order per step: every lane pops its symbol, then the */
/* lanes whose state fell below 2^16 take the next word, in lane order. */
/* The encoder pushes the symbols in exactly the reverse order and      */
/* finally reverses its word list.                                      */
/* Layout: 32 final states (u32, lane order) | u32 word count | words   */
/* (u16) | escaped values (u8 or u16) in decode order, i.e. by step,    */
/* then lane | zero bytes up to a multiple of 4.  Returns the size.     */
/* ------------------------------------------------------------------ */
static size_t pad4(size_t n) { return (n + 3) & ~(size_t)3; }

size_t skvo_stream_encode(int steps, int ebytes, const uint32_t* z, const skvo_table* const* tab,
                          uint8_t* out, size_t cap) {
    uint32_t x[SKVO_LANES];
    size_t nsym = (size_t)steps * SKVO_LANES;
    uint16_t* w = (uint16_t*)malloc(nsym * sizeof(uint16_t) + 2);
    uint32_t* esc = (uint32_t*)malloc(nsym * sizeof(uint32_t) + 4);
    size_t nw = 0, ne = 0;
    /* escaped values, in decode order */
    for (size_t j = 0; j < nsym; ++j)
        if (z[j] >= tab[j]->n) esc[ne++] = z[j];
    for (int i = 0; i < SKVO_LANES; ++i) x[i] = SKVO_L;
    for (int k = steps - 1; k >= 0; --k) {
        for (int i = SKVO_LANES - 1; i >= 0; --i) {
            const skvo_table* t = tab[k * SKVO_LANES + i];
            uint32_t zz = z[k * SKVO_LANES + i];
            uint32_t s = zz < t->n ? zz : t->n;
            if (skvo_rans_put(&x[i], t->freq[s], t->cum[s], &w[nw])) ++nw;
        }
    }
    size_t head = 4 * SKVO_LANES + 4;
    size_t bytes = pad4(head + 2 * nw + (size_t)ebytes * ne);
    if (bytes <= cap) {
        memset(out, 0, bytes);
        for (int i = 0; i < SKVO_LANES; ++i) put32(out + 4 * i, x[i]);
        put32(out + 4 * SKVO_LANES, (uint32_t)nw);
        uint8_t* o = out + head;
        for (size_t j = 0; j < nw; ++j) put16(o + 2 * j, w[nw - 1 - j]);
        o += 2 * nw;
        for (size_t j = 0; j < ne; ++j) {
            if (ebytes == 1) o[j] = (uint8_t)esc[j];
            else put16(o + 2 * j, esc[j]);
        }
    }
    free(w);
    free(esc);
    return bytes;
}

/* Returns E_OK and fills z[k*32+i], or E_CORRUPT when the stream does not
 * decode to a canonical encoding that uses exactly its words and escapes. */
int skvo_stream_decode(int steps, int ebytes, const uint8_t* in, size_t nbytes,
                       const skvo_table* const* tab, uint32_t* z) {
    size_t head = 4 * SKVO_LANES + 4;
    if (nbytes < head || (nbytes % 4) != 0) return E_CORRUPT;
    uint32_t x[SKVO_LANES];
    for (int i = 0; i < SKVO_LANES; ++i) {
        x[i] = get32(in + 4 * i);
        if (x[i] < SKVO_L) return E_CORRUPT;
    }
    size_t nw = get32(in + 4 * SKVO_LANES);
    if (nw > (nbytes - head) / 2) return E_CORRUPT;
    const uint8_t* W = in + head;
    const uint8_t* E = W + 2 * nw;
    size_t ecap = (nbytes - head - 2 * nw) / (size_t)ebytes;
    size_t p = 0, e = 0;
    for (int k = 0; k < steps; ++k) {
        uint32_t sym[SKVO_LANES];
        for (int i = 0; i < SKVO_LANES; ++i) {
            const skvo_table* t = tab[k * SKVO_LANES + i];
            sym[i] = skvo_rans_pop(&x[i], t->freq, t->cum, t->n + 1);
        }
        for (int i = 0; i < SKVO_LANES; ++i)
            if (x[i] < SKVO_L) {
                if (p >= nw) return E_CORRUPT;
                x[i] = (x[i] << 16) | get16(W + 2 * p++);
            }
        for (int i = 0; i < SKVO_LANES; ++i) {
            uint32_t n = tab[k * SKVO_LANES + i]->n;
            if (sym[i] == n) {
                if (e >= ecap) return E_CORRUPT;
                uint32_t v = (ebytes == 1) ? E[e] : get16(E + 2 * e);
                ++e;
                if (v < n) return E_CORRUPT;   /* a canonical encoder codes it directly */
                z[k * SKVO_LANES + i] = v;
            } else {
                z[k * SKVO_LANES + i] = sym[i];
            }
        }
    }
    for (int i = 0; i < SKVO_LANES; ++i)
        if (x[i] != SKVO_L) return E_CORRUPT;
    if (p != nw) return E_CORRUPT;
    size_t used = head + 2 * nw + (size_t)ebytes * e;
    if (pad4(used) != nbytes) return E_CORRUPT;
    for (size_t j = used; j < nbytes; ++j)
        if (in[j] != 0) return E_CORRUPT;
    return E_OK;
}

/* ------------------------------------------------------------------ */
/* Shapes, table blob, container                                       */
/* ------------------------------------------------------------------ */
typedef struct {
    uint32_t dtype, mode, layers, kv, tokens, channels;
} skvo_shape;

static int elem_bytes(uint32_t dtype) { return dtype == DT_E4M3 ? 1 : 2; }
/* Modes that code [layers][kv][tokens][channels] residuals against a predictor. */
static int residual_like(uint32_t mode) { return mode == MODE_RESIDUAL || mode == MODE_RESIDUAL_EXP; }
/* Modes that code [tokens][channels] coefficients in two checkerboard passes. */
static int checkerboard_like(uint32_t mode) { return mode == MODE_CHECKERBOARD || mode == MODE_CHECKERBOARD_MAP; }
static int elem_bits(uint32_t dtype) { return dtype == DT_E4M3 ? 8 : 16; }

static int shape_ok(const skvo_shape* s) {
    if (s->dtype < DT_BF16 || s->dtype > DT_INT16) return 0;
    if (s->channels == 0 || s->channels % SKVO_LANES) return 0;
    if (residual_like(s->mode)) {
        if (s->dtype == DT_INT16) return 0;
        if (s->layers == 0 || s->kv == 0 || s->tokens == 0) return 0;
        return s->tokens % SKVO_STEPS == 0;
    }
    if (checkerboard_like(s->mode)) {
        if (s->dtype != DT_INT16 || s->layers != 1 || s->kv != 1) return 0;
        return s->tokens > 0 && s->tokens % (2 * SKVO_STEPS) == 0;
    }
    return 0;
}

static uint64_t n_tables_of(const skvo_shape* s) {
    if (s->mode == MODE_RESIDUAL) return (uint64_t)s->layers * s->kv * s->channels;
    if (s->mode == MODE_RESIDUAL_EXP) return (uint64_t)s->layers * s->kv * 16;
    return (uint64_t)s->channels * 16;
}

/* Bytes after the table records: one class base per slab (exponent mode). */
static uint64_t n_bases_of(const skvo_shape* s) {
    return s->mode == MODE_RESIDUAL_EXP ? (uint64_t)s->layers * s->kv : 0;
}

static uint64_t n_streams_of(const skvo_shape* s) {
    uint64_t cg = s->channels / SKVO_LANES;
    if (residual_like(s->mode))
        return (uint64_t)s->layers * s->kv * (s->tokens / SKVO_STEPS) * cg;
    return 2ull * (s->tokens / 2 / SKVO_STEPS) * cg;
}

uint64_t skvo_blob_bytes(const skvo_shape* s) { return SKVO_HDR + n_tables_of(s) * SKVO_TAB_BYTES + n_bases_of(s); }

/* Map section after the records of a decoded-neighbour-map blob:
 * u32 k | u32 sh1 | u32 sh2 | u32 0 | int8 V[k][2C] | int8 U[C][k]. */
#define SKVO_MAP_HDR 16
static uint64_t map_bytes(uint32_t k, uint32_t C) { return SKVO_MAP_HDR + 3ull * k * C; }
uint64_t skvo_blob_bytes_map(const skvo_shape* s, uint32_t k) { return skvo_blob_bytes(s) + map_bytes(k, s->channels); }

/* Map parameters accepted in a blob: rank a power of two from 16 to 256. */
static int map_params_ok(uint32_t k, uint32_t sh1, uint32_t sh2) {
    return k >= 16 && k <= 256 && (k & (k - 1)) == 0 && sh1 <= 40 && sh2 <= 30;
}

/* Parse a table blob: header fields must match the shape, every table must
 * hold 1..255 direct symbols plus ESC, positive frequencies summing to 2^12
 * and zeros beyond ESC. */
static int parse_blob_map(const uint8_t* blob, size_t nbytes, const skvo_shape* s, skvo_table** out,
                          const uint8_t** bases, skvo_map* map) {
    if (nbytes < SKVO_HDR || memcmp(blob, "SKVT", 4) != 0 || get16(blob + 4) != 1) return E_TABLES;
    if (blob[6] != s->dtype || blob[7] != s->mode) return E_TABLES;
    uint64_t nt = n_tables_of(s);
    if (get32(blob + 8) != nt || get32(blob + 12) != s->layers || get32(blob + 16) != s->kv ||
        get32(blob + 20) != s->channels)
        return E_TABLES;
    if (s->mode == MODE_CHECKERBOARD_MAP) {
        uint64_t at = skvo_blob_bytes(s);
        if (nbytes < at + SKVO_MAP_HDR) return E_TABLES;
        const uint8_t* mh = blob + at;
        uint32_t k = get32(mh), sh1 = get32(mh + 4), sh2 = get32(mh + 8);
        if (!map_params_ok(k, sh1, sh2) || get32(mh + 12) != 0) return E_TABLES;
        if (get64(blob + 32) != nbytes || nbytes != at + map_bytes(k, s->channels)) return E_TABLES;
        if (map) {
            map->k = k;
            map->sh1 = sh1;
            map->sh2 = sh2;
            map->V = (const int8_t*)(mh + SKVO_MAP_HDR);
            map->U = map->V + 2ull * k * s->channels;
        }
    } else if (get64(blob + 32) != nbytes || nbytes != skvo_blob_bytes(s)) {
        return E_TABLES;
    }
    skvo_table* t = (skvo_table*)malloc(nt * sizeof(skvo_table));
    for (uint64_t j = 0; j < nt; ++j) {
        const uint8_t* p = blob + SKVO_HDR + j * SKVO_TAB_BYTES;
        uint32_t n = get16(p), sum = 0;
        if (n < 1 || n > SKVO_MAX_DIRECT) { free(t); return E_TABLES; }
        t[j].n = n;
        for (uint32_t q = 0; q < 256; ++q) {
            uint32_t f = get16(p + 2 + 2 * q);
            if (q <= n && f == 0) { free(t); return E_TABLES; }
            if (q > n && f != 0) { free(t); return E_TABLES; }
            if (q <= n) { t[j].freq[q] = f; sum += f; }
        }
        if (sum != SKVO_M) { free(t); return E_TABLES; }
        table_cum(&t[j]);
    }
    *out = t;
    *bases = blob + SKVO_HDR + nt * SKVO_TAB_BYTES;   /* n_bases_of(s) bytes */
    return E_OK;
}

static int parse_blob(const uint8_t* blob, size_t nbytes, const skvo_shape* s, skvo_table** out,
                      const uint8_t** bases) {
    return parse_blob_map(blob, nbytes, s, out, bases, NULL);
}

/* Stream id -> (slab, token block, channel group); see the container layout:
 * channel groups vary fastest, then token blocks, then slabs.  A slab is one
 * (layer, K|V) plane in residual mode and one checkerboard pass otherwise. */
typedef struct { uint64_t slab, tb, cg; } stream_pos;

static stream_pos stream_at(const skvo_shape* s, uint64_t id) {
    uint64_t ncg = s->channels / SKVO_LANES;
    uint64_t ntb = (residual_like(s->mode) ? s->tokens : s->tokens / 2) / SKVO_STEPS;
    stream_pos sp;
    sp.cg = id % ncg;
    sp.tb = (id / ncg) % ntb;
    sp.slab = id / (ncg * ntb);
    return sp;
}

/* Token (row) coded at step k of a stream. */
static uint64_t token_of(const skvo_shape* s, stream_pos sp, int k) {
    uint64_t j = sp.tb * SKVO_STEPS + (uint64_t)k;
    if (residual_like(s->mode)) return j;
    return 2 * j + sp.slab;   /* pass 0: even tokens, pass 1: odd tokens */
}

static uint32_t load_elem(const void* a, int dtype, size_t idx) {
    if (dtype == DT_E4M3) return ((const uint8_t*)a)[idx];
    return ((const uint16_t*)a)[idx];
}

static void store_elem(void* a, int dtype, size_t idx, uint32_t v) {
    if (dtype == DT_E4M3) ((uint8_t*)a)[idx] = (uint8_t)v;
    else ((uint16_t*)a)[idx] = (uint16_t)v;
}

/* Symbols and tables of one stream, gathered from the full arrays.
 * residual: aux = predictor cache; checkerboard: aux = side input G and the
 * neighbours come from `tgt` (the true coefficients on the encode side, the
 * already decoded even tokens on the decode side). */
static void gather_stream(const skvo_shape* s, const skvo_table* tabs, const uint8_t* bases, const void* tgt,
                          const void* aux, uint64_t id, uint32_t* z, const skvo_table** tp, int with_z) {
    stream_pos sp = stream_at(s, id);
    size_t C = s->channels;
    for (int k = 0; k < SKVO_STEPS; ++k) {
        uint64_t tok = token_of(s, sp, k);
        for (int i = 0; i < SKVO_LANES; ++i) {
            size_t ch = sp.cg * SKVO_LANES + (size_t)i;
            if (residual_like(s->mode)) {
                size_t idx = ((size_t)sp.slab * s->tokens + tok) * C + ch;
                if (s->mode == MODE_RESIDUAL)
                    tp[k * SKVO_LANES + i] = &tabs[sp.slab * C + ch];
                else
                    tp[k * SKVO_LANES + i] =
                        &tabs[sp.slab * 16 + skvo_exp_class(load_elem(aux, s->dtype, idx), (int)s->dtype, bases[sp.slab])];
                if (with_z)
                    z[k * SKVO_LANES + i] = skvo_zigzag(skvo_residual(load_elem(tgt, s->dtype, idx),
                                                                      load_elem(aux, s->dtype, idx),
                                                                      elem_bits(s->dtype)));
            } else {
                int32_t mu = skvo_dckv_mean((const int16_t*)tgt, (const int16_t*)aux, s->tokens, C,
                                            (uint32_t)tok, (uint32_t)ch);
                int32_t kk, f;
                skvo_dckv_split(mu, &kk, &f);
                tp[k * SKVO_LANES + i] = &tabs[ch * 16 + (size_t)f];
                if (with_z) {
                    int32_t c = ((const int16_t*)tgt)[tok * C + ch];
                    z[k * SKVO_LANES + i] = skvo_dckv_symbol(c, mu, &f);
                }
            }
        }
    }
}

static void write_header(uint8_t* h, const skvo_shape* s, uint64_t nstreams, uint64_t hash, uint64_t payload) {
    memset(h, 0, SKVO_HDR);
    memcpy(h, "SKV1", 4);
    put16(h + 4, 1);
    h[6] = (uint8_t)s->dtype;
    h[7] = (uint8_t)s->mode;
    h[8] = 12;
    h[9] = SKVO_LANES;
    put16(h + 10, SKVO_STEPS);
    put32(h + 12, s->layers);
    put32(h + 16, s->kv);
    put32(h + 20, s->tokens);
    put32(h + 24, s->channels);
    put64(h + 32, nstreams);
    put64(h + 40, hash);
    put64(h + 48, payload);
}

/* Upper bound of a container for this shape (every stream raw). */
uint64_t skvo_bound(const skvo_shape* s) {
    uint64_t n = n_streams_of(s);
    return SKVO_HDR + 8 * (n + 1) + n * (uint64_t)SKVO_SYMS * elem_bytes(s->dtype);
}

/* Encode one stream of the arrays into `out` (capacity raw size).  Returns
 * the stream's byte count; *raw is set when the stream is stored raw. */
static size_t encode_one(const skvo_shape* s, const skvo_table* tabs, const uint8_t* bases, const void* tgt,
                         const void* aux, uint64_t id, uint8_t* out, int* raw) {
    uint32_t z[SKVO_SYMS];
    const skvo_table* tp[SKVO_SYMS];
    int eb = elem_bytes(s->dtype);
    size_t rawb = (size_t)SKVO_SYMS * eb;
    gather_stream(s, tabs, bases, tgt, aux, id, z, tp, 1);
    const size_t tcap = 4 * SKVO_LANES + 4 + 4 * (size_t)SKVO_SYMS + 4;
    uint8_t* tmp = (uint8_t*)malloc(tcap);
    size_t nb = skvo_stream_encode(SKVO_STEPS, eb, z, tp, tmp, tcap);
    if (nb >= rawb) {
        /* Raw fallback: the stream's target elements in (step, lane) order. */
        stream_pos sp = stream_at(s, id);
        for (int k = 0; k < SKVO_STEPS; ++k) {
            uint64_t tok = token_of(s, sp, k);
            for (int i = 0; i < SKVO_LANES; ++i) {
                size_t ch = sp.cg * SKVO_LANES + (size_t)i;
                size_t idx = residual_like(s->mode) ? ((size_t)sp.slab * s->tokens + tok) * s->channels + ch
                                                    : tok * s->channels + ch;
                uint32_t v = load_elem(tgt, s->dtype, idx);
                if (eb == 1) out[k * SKVO_LANES + i] = (uint8_t)v;
                else put16(out + 2 * (k * SKVO_LANES + i), v);
            }
        }
        *raw = 1;
        free(tmp);
        return rawb;
    }
    memcpy(out, tmp, nb);
    *raw = 0;
    free(tmp);
    return nb;
}

/* Whole-container encode.  Returns the container size (>0) or an error.
 * When `cap` is too small nothing is written and E_CAPACITY is returned with
 * *need set to the size. */
int64_t skvo_encode(const uint8_t* blob, size_t blob_bytes, const skvo_shape* s, const void* tgt,
                    const void* aux, uint8_t* out, uint64_t cap, uint64_t* need, int nthreads) {
    if (!blob || !s || !tgt || !aux) return E_ARG;
    if (!shape_ok(s)) return E_SHAPE;
    skvo_table* tabs = NULL;
    const uint8_t* bases = NULL;
    skvo_map map;
    int rc = parse_blob_map(blob, blob_bytes, s, &tabs, &bases, &map);
    if (rc) return rc;
    int16_t* gmap = NULL;
    if (s->mode == MODE_CHECKERBOARD_MAP) {
        /* odd tokens take the side input with the map of their true (= decoded) even neighbours */
        gmap = (int16_t*)malloc((size_t)s->tokens * s->channels * sizeof(int16_t));
        dckv_map_side((const int16_t*)tgt, (const int16_t*)aux, s->tokens, s->channels, &map, gmap, nthreads);
        aux = gmap;
    }
    uint64_t n = n_streams_of(s);
    size_t rawb = (size_t)SKVO_SYMS * elem_bytes(s->dtype);
    uint8_t* tmp = (uint8_t*)malloc(n * rawb);
    uint64_t* size = (uint64_t*)malloc(n * sizeof(uint64_t));
    int* raw = (int*)malloc(n * sizeof(int));
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
    for (int64_t id = 0; id < (int64_t)n; ++id)
        size[id] = encode_one(s, tabs, bases, tgt, aux, (uint64_t)id, tmp + (size_t)id * rawb, &raw[id]);
    uint64_t payload = 0;
    for (uint64_t id = 0; id < n; ++id) payload += size[id];
    uint64_t total = SKVO_HDR + 8 * (n + 1) + payload;
    if (need) *need = total;
    free(gmap);
    if (!out || cap < total) {
        free(tmp); free(size); free(raw); free(tabs);
        return out ? E_CAPACITY : (int64_t)total;
    }
    write_header(out, s, n, skvo_fnv1a64(blob, blob_bytes), payload);
    uint8_t* idx = out + SKVO_HDR;
    uint8_t* pay = idx + 8 * (n + 1);
    uint64_t off = 0;
    for (uint64_t id = 0; id < n; ++id) {
        put64(idx + 8 * id, off | ((uint64_t)raw[id] << 63));
        memcpy(pay + off, tmp + (size_t)id * rawb, size[id]);
        off += size[id];
    }
    put64(idx + 8 * n, off);
    free(tmp); free(size); free(raw); free(tabs);
    return (int64_t)total;
}

/* Read the shape stored in a container header (no validation of tables). */
int skvo_container_shape(const uint8_t* in, uint64_t in_bytes, skvo_shape* s) {
    if (!in || in_bytes < SKVO_HDR || memcmp(in, "SKV1", 4) != 0 || get16(in + 4) != 1) return E_CORRUPT;
    s->dtype = in[6];
    s->mode = in[7];
    s->layers = get32(in + 12);
    s->kv = get32(in + 16);
    s->tokens = get32(in + 20);
    s->channels = get32(in + 24);
    return E_OK;
}

static int decode_one(const skvo_shape* s, const skvo_table* tabs, const uint8_t* bases, const uint8_t* src,
                      uint64_t nb, int raw, const void* aux, void* out, uint64_t id) {
    uint32_t z[SKVO_SYMS];
    const skvo_table* tp[SKVO_SYMS];
    int eb = elem_bytes(s->dtype), nbits = elem_bits(s->dtype);
    stream_pos sp = stream_at(s, id);
    size_t C = s->channels;
    if (raw) {
        if (nb != (uint64_t)SKVO_SYMS * eb) return E_CORRUPT;
    } else {
        /* tables first: in checkerboard mode they depend on the decoded even tokens */
        gather_stream(s, tabs, bases, out, aux, id, NULL, tp, 0);
        int rc = skvo_stream_decode(SKVO_STEPS, eb, src, nb, tp, z);
        if (rc) return rc;
    }
    for (int k = 0; k < SKVO_STEPS; ++k) {
        uint64_t tok = token_of(s, sp, k);
        for (int i = 0; i < SKVO_LANES; ++i) {
            size_t ch = sp.cg * SKVO_LANES + (size_t)i;
            size_t idx = residual_like(s->mode) ? ((size_t)sp.slab * s->tokens + tok) * C + ch : tok * C + ch;
            uint32_t v;
            if (raw) {
                v = (eb == 1) ? src[k * SKVO_LANES + i] : get16(src + 2 * (k * SKVO_LANES + i));
            } else if (residual_like(s->mode)) {
                v = skvo_reconstruct(load_elem(aux, s->dtype, idx), skvo_unzigzag(z[k * SKVO_LANES + i]), nbits);
            } else {
                int32_t mu = skvo_dckv_mean((const int16_t*)out, (const int16_t*)aux, s->tokens, (uint32_t)C,
                                            (uint32_t)tok, (uint32_t)ch);
                v = (uint16_t)skvo_dckv_reconstruct(z[k * SKVO_LANES + i], mu);
            }
            store_elem(out, s->dtype, idx, v);
        }
    }
    return E_OK;
}

/* Whole-container decode into `out` (same layout and size as the target).
 * `blob` must be the table blob whose hash the container carries. */
int skvo_decode(const uint8_t* blob, size_t blob_bytes, const uint8_t* in, uint64_t in_bytes, const void* aux,
                void* out, uint64_t out_bytes, int nthreads) {
    skvo_shape s;
    if (!blob || !in || !aux || !out) return E_ARG;
    int rc = skvo_container_shape(in, in_bytes, &s);
    if (rc) return rc;
    if (in[8] != 12 || in[9] != SKVO_LANES || get16(in + 10) != SKVO_STEPS) return E_CORRUPT;
    if (!shape_ok(&s)) return E_CORRUPT;
    uint64_t n = n_streams_of(&s);
    if (get64(in + 32) != n) return E_CORRUPT;
    uint64_t elems = (uint64_t)s.tokens * s.channels * (residual_like(s.mode) ? (uint64_t)s.layers * s.kv : 1);
    if (out_bytes < elems * elem_bytes(s.dtype)) return E_CAPACITY;
    if (get64(in + 40) != skvo_fnv1a64(blob, blob_bytes)) return E_TABLES;
    skvo_table* tabs = NULL;
    const uint8_t* bases = NULL;
    skvo_map map;
    rc = parse_blob_map(blob, blob_bytes, &s, &tabs, &bases, &map);
    if (rc) return rc;
    uint64_t payload = get64(in + 48);
    uint64_t head = SKVO_HDR + 8 * (n + 1);
    if (in_bytes < head || in_bytes - head < payload) { free(tabs); return E_CORRUPT; }
    const uint8_t* idx = in + SKVO_HDR;
    const uint8_t* pay = in + head;
    const uint64_t mask = ~(1ull << 63);
    if (get64(idx + 8 * n) != payload) { free(tabs); return E_CORRUPT; }
    for (uint64_t id = 0; id < n; ++id) {
        uint64_t a = get64(idx + 8 * id) & mask, b = get64(idx + 8 * (id + 1)) & mask;
        if (b < a || b > payload) { free(tabs); return E_CORRUPT; }
    }
    if (nthreads < 1) nthreads = 1;
    int passes = residual_like(s.mode) ? 1 : 2;
    uint64_t per = n / passes;
    int bad = 0;
    int16_t* gmap = NULL;
    const void* pass_aux = aux;
    for (int ps = 0; ps < passes; ++ps) {
        if (ps == 1 && s.mode == MODE_CHECKERBOARD_MAP) {
            /* the map reads the decoded even tokens */
            gmap = (int16_t*)malloc((size_t)s.tokens * s.channels * sizeof(int16_t));
            dckv_map_side((const int16_t*)out, (const int16_t*)aux, s.tokens, s.channels, &map, gmap, nthreads);
            pass_aux = gmap;
        }
        /* checkerboard: the odd pass starts only once every even token is decoded */
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads) reduction(| : bad)
        for (int64_t j = 0; j < (int64_t)per; ++j) {
            uint64_t id = (uint64_t)ps * per + (uint64_t)j;
            uint64_t e = get64(idx + 8 * id);
            uint64_t a = e & mask, b = get64(idx + 8 * (id + 1)) & mask;
            int r = decode_one(&s, tabs, bases, pay + a, b - a, (int)(e >> 63), pass_aux, out, id);
            if (r) bad = 1;
        }
        if (bad) break;
    }
    free(gmap);
    free(tabs);
    return bad ? E_CORRUPT : E_OK;
}

/* ------------------------------------------------------------------ */
/* Table fit (host, fp64).  [SKC] "What to use as the predictor": the    */
/* residual statistics are measured once on calibration data and fixed.  */
/* [DCKV] "How it differs": per-component Laplace integrated over the    */
/* quantization cells; the token-conditioned mean shifts it.            */
/* ------------------------------------------------------------------ */

/* Mass of the unit cell [v - 1/2, v + 1/2] under Laplace(location m, scale b). */
double skvo_cell_mass(double v, double m, double b) {
    double lo = v - 0.5 - m, hi = v + 0.5 - m;
    if (lo >= 0.0) return 0.5 * (exp(-lo / b) - exp(-hi / b));
    if (hi <= 0.0) return 0.5 * (exp(hi / b) - exp(lo / b));
    return 1.0 - 0.5 * exp(-hi / b) - 0.5 * exp(lo / b);
}

/* Largest-remainder quantization of q[0..m-1] (sum 4096) to integer
 * frequencies >= 1 summing to exactly 4096. */
void skvo_quantize(const double* q, int m, uint32_t* f) {
    int64_t sum = 0;
    double rem[257];
    for (int i = 0; i < m; ++i) {
        double fl = floor(q[i]);
        f[i] = fl < 1.0 ? 1u : (uint32_t)fl;
        rem[i] = q[i] - (double)f[i];
        sum += f[i];
    }
    int64_t R = (int64_t)SKVO_M - sum;
    if (R > 0) {
        int used[257] = {0};
        for (int64_t r = 0; r < R; ++r) {
            int best = -1;
            for (int i = 0; i < m; ++i)
                if (!used[i] && (best < 0 || rem[i] > rem[best])) best = i;
            used[best] = 1;
            f[best] += 1;
        }
    }
    while (R < 0) {
        int best = -1;
        for (int i = 0; i < m; ++i)
            if (f[i] > 1 && (best < 0 || f[i] > f[best])) best = i;
        f[best] -= 1;
        ++R;
    }
}

/* Direct range: z = 0 always; then every z <= 254 up to the last one whose
 * cell mass reaches 2^-12 (one slot of the 12-bit table). */
static uint32_t direct_count(const double* p) {
    uint32_t n = 1;
    for (uint32_t z = 0; z < 255; ++z)
        if (p[z] >= 1.0 / 4096.0) n = z + 1;
    return n;
}

/* Calibration tail of one (layer, K|V) slab: the smallest z in [1, 255] such
 * that at most floor(count / 1024) of the slab's calibration symbols are z or
 * larger.  Every table of the slab codes at least the symbols below it
 * directly, so that escapes stay near 1/1024 of the symbols even where the
 * Laplace tail is lighter than the data's. */
static uint32_t tail_count(const uint32_t* z, uint64_t count) {
    uint64_t hist[256] = {0};
    for (uint64_t i = 0; i < count; ++i) hist[z[i] > 255 ? 255 : z[i]] += 1;
    uint64_t allow = count / 1024, above = 0;
    uint32_t q = 255;
    /* walk down from 255: q stays the smallest z whose tail count is within the allowance */
    for (uint32_t v = 255; v >= 1; --v) {
        above += hist[v];
        if (above > allow) break;
        q = v;
    }
    return q;
}

/* Build one table from cell masses p[0..254], direct count n and escape
 * probability pe: direct masses are rescaled to 1 - pe, ESC gets pe. */
static void build_table(const double* p, uint32_t n, double pe, uint8_t* dst) {
    double S = 0.0, q[256];
    uint32_t f[256];
    for (uint32_t z = 0; z < n; ++z) S += p[z];
    double w = (1.0 - pe) / S;
    for (uint32_t z = 0; z < n; ++z) q[z] = 4096.0 * (p[z] * w);
    q[n] = 4096.0 * pe;
    skvo_quantize(q, (int)n + 1, f);
    memset(dst, 0, SKVO_TAB_BYTES);
    put16(dst, n);
    for (uint32_t z = 0; z <= n; ++z) put16(dst + 2 + 2 * z, f[z]);
}

static void blob_header(uint8_t* h, const skvo_shape* s, uint32_t calib_tokens, uint64_t total) {
    memset(h, 0, SKVO_HDR);
    memcpy(h, "SKVT", 4);
    put16(h + 4, 1);
    h[6] = (uint8_t)s->dtype;
    h[7] = (uint8_t)s->mode;
    put32(h + 8, (uint32_t)n_tables_of(s));
    put32(h + 12, s->layers);
    put32(h + 16, s->kv);
    put32(h + 20, s->channels);
    put32(h + 24, calib_tokens);
    put64(h + 32, total);
}

/* Fit every table from calibration arrays.
 *   residual mode:     calib_t, calib_a = target / predictor elements,
 *                      [layers][kv][calib_tokens][channels]
 *   checkerboard mode: calib_t = int16 coefficients, calib_a = int16 G,
 *                      [calib_tokens][channels], calib_tokens even
 * Writes skvo_blob_bytes(s) bytes to blob (when cap allows). */
static void fit_checkerboard(const int16_t* coef, const int16_t* G, uint32_t calib_tokens, size_t C, uint8_t* rec);

int skvo_fit_tables(const skvo_shape* s, const void* calib_t, const void* calib_a, uint32_t calib_tokens,
                    uint8_t* blob, uint64_t cap, uint64_t* blob_bytes) {
    if (!s || !calib_t || !calib_a || !blob_bytes) return E_ARG;
    if (s->mode == MODE_CHECKERBOARD_MAP) return E_SHAPE;   /* takes skvo_fit_tables_map */
    skvo_shape cs = *s;
    cs.tokens = residual_like(s->mode) ? SKVO_STEPS : 2 * SKVO_STEPS;   /* tokens do not matter here */
    if (!shape_ok(&cs) || calib_tokens == 0) return E_SHAPE;
    if (s->mode == MODE_CHECKERBOARD && (calib_tokens % 2)) return E_SHAPE;
    uint64_t total = skvo_blob_bytes(s);
    *blob_bytes = total;
    if (!blob || cap < total) return E_CAPACITY;
    blob_header(blob, s, calib_tokens, total);
    size_t C = s->channels;
    double p[255];
    if (s->mode == MODE_RESIDUAL_EXP) {
        /* Exponent-conditioned tables: per slab, the class base is the first of
         * the 16 consecutive exponents that hold the most calibration
         * predictors (the smallest such base on ties); the table of class q
         * is a Laplace fitted to the slab's calibration values of class q
         * (the slab's pooled scale when fewer than 64 of them are within
         * |r| <= 127), with the slab's tail floor and the class's own escape
         * rate.  Sums run over the slab's values in element order. */
        int nbits = elem_bits(s->dtype);
        uint32_t emax = s->dtype == DT_E4M3 ? 15u : 255u;
        uint64_t slabs = (uint64_t)s->layers * s->kv;
        uint64_t per_slab = (uint64_t)calib_tokens * C;
        uint32_t* zs = (uint32_t*)malloc(per_slab * sizeof(uint32_t));
        int32_t* rs = (int32_t*)malloc(per_slab * sizeof(int32_t));
        uint8_t* cls = (uint8_t*)malloc(per_slab);
        if (!zs || !rs || !cls) { free(zs); free(rs); free(cls); return E_ARG; }
        uint8_t* bases = blob + SKVO_HDR + n_tables_of(s) * SKVO_TAB_BYTES;
        for (uint64_t sl = 0; sl < slabs; ++sl) {
            uint64_t hist[256] = {0};
            for (uint64_t i = 0; i < per_slab; ++i) {
                size_t idx = (size_t)sl * per_slab + i;
                uint32_t pv = load_elem(calib_a, s->dtype, idx);
                rs[i] = skvo_residual(load_elem(calib_t, s->dtype, idx), pv, nbits);
                zs[i] = skvo_zigzag(rs[i]);
                hist[(s->dtype == DT_E4M3) ? ((pv >> 3) & 0xFu) : ((pv >> 7) & 0xFFu)] += 1;
            }
            uint32_t zq = tail_count(zs, per_slab);
            uint32_t base = 0;
            uint64_t best = 0;
            for (uint32_t b0 = 0; b0 + 15 <= emax; ++b0) {
                uint64_t cnt = 0;
                for (uint32_t e = b0; e <= b0 + 15; ++e) cnt += hist[e];
                if (b0 == 0 || cnt > best) { best = cnt; base = b0; }
            }
            bases[sl] = (uint8_t)base;
            double sum_all = 0.0;
            uint64_t cnt_all = 0;
            for (uint64_t i = 0; i < per_slab; ++i) {
                cls[i] = (uint8_t)skvo_exp_class(load_elem(calib_a, s->dtype, (size_t)sl * per_slab + i), (int)s->dtype, base);
                if (rs[i] <= 127 && rs[i] >= -127) { sum_all += (double)(rs[i] < 0 ? -rs[i] : rs[i]); ++cnt_all; }
            }
            double b_all = cnt_all ? sum_all / (double)cnt_all : 0.0;
            if (b_all < 0.05) b_all = 0.05;
            for (uint32_t q = 0; q < 16; ++q) {
                double sum = 0.0;
                uint64_t cnt = 0, members = 0;
                for (uint64_t i = 0; i < per_slab; ++i) {
                    if (cls[i] != q) continue;
                    ++members;
                    if (rs[i] <= 127 && rs[i] >= -127) { sum += (double)(rs[i] < 0 ? -rs[i] : rs[i]); ++cnt; }
                }
                double b = cnt >= 64 ? sum / (double)cnt : b_all;
                if (b < 0.05) b = 0.05;
                for (uint32_t z = 0; z < 255; ++z) p[z] = skvo_cell_mass((double)skvo_unzigzag(z), 0.0, b);
                uint32_t n = direct_count(p);
                if (n < zq) n = zq;
                uint64_t esc = 0;
                for (uint64_t i = 0; i < per_slab; ++i)
                    if (cls[i] == q && zs[i] >= n) ++esc;
                double pe = ((double)esc + 1.0) / ((double)members + 2.0);
                build_table(p, n, pe, blob + SKVO_HDR + (sl * 16 + q) * SKVO_TAB_BYTES);
            }
        }
        free(zs);
        free(rs);
        free(cls);
        return E_OK;
    }
    if (s->mode == MODE_RESIDUAL) {
        int nbits = elem_bits(s->dtype);
        uint64_t slabs = (uint64_t)s->layers * s->kv;
        uint64_t per_slab = (uint64_t)calib_tokens * C;
        uint32_t* zs = (uint32_t*)malloc(per_slab * sizeof(uint32_t));
        if (!zs) return E_ARG;
        for (uint64_t sl = 0; sl < slabs; ++sl) {
            for (uint64_t i = 0; i < per_slab; ++i) {
                size_t idx = (size_t)sl * per_slab + i;
                zs[i] = skvo_zigzag(skvo_residual(load_elem(calib_t, s->dtype, idx), load_elem(calib_a, s->dtype, idx), nbits));
            }
            uint32_t zq = tail_count(zs, per_slab);
            for (size_t ch = 0; ch < C; ++ch) {
                double sum = 0.0;
                uint64_t cnt = 0;
                for (uint32_t t = 0; t < calib_tokens; ++t) {
                    size_t idx = ((size_t)sl * calib_tokens + t) * C + ch;
                    int32_t r = skvo_residual(load_elem(calib_t, s->dtype, idx), load_elem(calib_a, s->dtype, idx), nbits);
                    if (r <= 127 && r >= -127) { sum += (double)(r < 0 ? -r : r); ++cnt; }
                }
                double b = cnt ? sum / (double)cnt : 0.0;
                if (b < 0.05) b = 0.05;
                for (uint32_t z = 0; z < 255; ++z) p[z] = skvo_cell_mass((double)skvo_unzigzag(z), 0.0, b);
                uint32_t n = direct_count(p);
                if (n < zq) n = zq;   /* zq <= 255 */
                uint64_t esc = 0;
                for (uint32_t t = 0; t < calib_tokens; ++t) {
                    size_t idx = ((size_t)sl * calib_tokens + t) * C + ch;
                    uint32_t z = skvo_zigzag(skvo_residual(load_elem(calib_t, s->dtype, idx), load_elem(calib_a, s->dtype, idx), nbits));
                    if (z >= n) ++esc;
                }
                double pe = ((double)esc + 1.0) / ((double)calib_tokens + 2.0);
                build_table(p, n, pe, blob + SKVO_HDR + (sl * C + ch) * SKVO_TAB_BYTES);
            }
        }
        free(zs);
        return E_OK;
    }
    if (s->mode != MODE_CHECKERBOARD) return E_SHAPE;   /* the map mode takes skvo_fit_tables_map */
    fit_checkerboard((const int16_t*)calib_t, (const int16_t*)calib_a, calib_tokens, C, blob + SKVO_HDR);
    return E_OK;
}

/* Checkerboard tables (16 shifted tables per component) from calibration
 * coefficients and their side input G, [N][C], N even. */
static void fit_checkerboard(const int16_t* coef, const int16_t* G, uint32_t calib_tokens, size_t C, uint8_t* rec) {
    for (size_t ch = 0; ch < C; ++ch) {
        double sum = 0.0;
        uint64_t cnt = 0;
        for (uint32_t t = 0; t < calib_tokens; ++t) {
            int32_t mu = skvo_dckv_mean(coef, G, calib_tokens, (uint32_t)C, t, (uint32_t)ch);
            double e = (double)coef[(size_t)t * C + ch] - (double)mu / 16.0;
            double a = e < 0 ? -e : e;
            if (a <= 127.0) { sum += a; ++cnt; }
        }
        double b = cnt ? sum / (double)cnt : 0.0;
        if (b < 0.05) b = 0.05;
        double pf[16][255];
        uint32_t nf[16];
        for (int f = 0; f < 16; ++f) {
            for (uint32_t z = 0; z < 255; ++z) pf[f][z] = skvo_cell_mass((double)skvo_unzigzag(z), (double)f / 16.0, b);
            nf[f] = direct_count(pf[f]);
        }
        uint64_t esc = 0;
        for (uint32_t t = 0; t < calib_tokens; ++t) {
            int32_t mu = skvo_dckv_mean(coef, G, calib_tokens, (uint32_t)C, t, (uint32_t)ch), f;
            uint32_t z = skvo_dckv_symbol(coef[(size_t)t * C + ch], mu, &f);
            if (z >= nf[f]) ++esc;
        }
        double pe = ((double)esc + 1.0) / ((double)calib_tokens + 2.0);
        for (int f = 0; f < 16; ++f)
            build_table(pf[f], nf[f], pe, rec + (ch * 16 + (size_t)f) * SKVO_TAB_BYTES);
    }
}

/* Tables of the decoded-neighbour-map mode: the checkerboard fit on the
 * calibration rows with their side input G' (the map applied to the
 * calibration's own even rows), then the map itself after the records. */
int skvo_fit_tables_map(const skvo_shape* s, const int16_t* calib_coef, const int16_t* calib_G,
                        uint32_t calib_tokens, uint32_t k, uint32_t sh1, uint32_t sh2, const int8_t* V,
                        const int8_t* U, uint8_t* blob, uint64_t cap, uint64_t* blob_bytes) {
    if (!s || !calib_coef || !calib_G || !V || !U || !blob_bytes) return E_ARG;
    if (s->mode != MODE_CHECKERBOARD_MAP) return E_SHAPE;
    skvo_shape cs = *s;
    cs.tokens = 2 * SKVO_STEPS;
    if (!shape_ok(&cs) || calib_tokens == 0 || (calib_tokens % 2)) return E_SHAPE;
    if (!map_params_ok(k, sh1, sh2)) return E_ARG;
    uint64_t total = skvo_blob_bytes_map(s, k);
    *blob_bytes = total;
    if (!blob || cap < total) return E_CAPACITY;
    size_t C = s->channels;
    blob_header(blob, s, calib_tokens, total);
    skvo_map m = {k, sh1, sh2, V, U};
    int16_t* gmap = (int16_t*)malloc((size_t)calib_tokens * C * sizeof(int16_t));
    dckv_map_side(calib_coef, calib_G, calib_tokens, (uint32_t)C, &m, gmap, 1);
    fit_checkerboard(calib_coef, gmap, calib_tokens, C, blob + SKVO_HDR);
    free(gmap);
    uint8_t* mh = blob + skvo_blob_bytes(s);
    memset(mh, 0, SKVO_MAP_HDR);
    put32(mh, k);
    put32(mh + 4, sh1);
    put32(mh + 8, sh2);
    memcpy(mh + SKVO_MAP_HDR, V, 2ull * k * C);
    memcpy(mh + SKVO_MAP_HDR + 2ull * k * C, U, (size_t)k * C);
    return E_OK;
}

/* ------------------------------------------------------------------ */
/* Single-stream entry points for sampled checks on large inputs.       */
/* The caller passes the stream's 4096 inputs already gathered in        */
/* (step, lane) order, and for the checkerboard odd pass the left/right  */
/* neighbour coefficients of each position.                              */
/* ------------------------------------------------------------------ */

/* Tile encode.  residual: tile_t/tile_a = target/predictor elements and
 * `tables` = the 32 lane tables' blob indices; checkerboard: tile_t =
 * coefficients, tile_a = G, nb_l/nb_r = neighbours (odd pass) or NULL,
 * tables = the 32 component indices.  Writes <= raw size bytes. */
int64_t skvo_encode_tile(const uint8_t* blob, size_t blob_bytes, const skvo_shape* s, const void* tile_t,
                         const void* tile_a, const int16_t* nb_l, const int16_t* nb_r, const uint32_t* lane_ids,
                         uint8_t* out, int* raw) {
    skvo_table* tabs = NULL;
    const uint8_t* bases = NULL;
    int rc = parse_blob(blob, blob_bytes, s, &tabs, &bases);
    if (rc) return rc;
    uint32_t z[SKVO_SYMS];
    const skvo_table* tp[SKVO_SYMS];
    int eb = elem_bytes(s->dtype), nbits = elem_bits(s->dtype);
    for (int j = 0; j < SKVO_SYMS; ++j) {
        uint32_t lane = lane_ids[j % SKVO_LANES];
        if (residual_like(s->mode)) {
            /* exponent mode: every lane id is the stream's slab */
            tp[j] = s->mode == MODE_RESIDUAL
                        ? &tabs[lane]
                        : &tabs[(size_t)lane * 16 + skvo_exp_class(load_elem(tile_a, s->dtype, j), (int)s->dtype, bases[lane])];
            z[j] = skvo_zigzag(skvo_residual(load_elem(tile_t, s->dtype, j), load_elem(tile_a, s->dtype, j), nbits));
        } else {
            int32_t mu = ((const int16_t*)tile_a)[j], f;
            if (nb_l) mu += 8 * ((int32_t)nb_l[j] + (int32_t)nb_r[j]);
            z[j] = skvo_dckv_symbol(((const int16_t*)tile_t)[j], mu, &f);
            tp[j] = &tabs[(size_t)lane * 16 + (size_t)f];
        }
    }
    size_t rawb = (size_t)SKVO_SYMS * eb;
    const size_t tcap = 4 * SKVO_LANES + 4 + 4 * (size_t)SKVO_SYMS + 4;
    uint8_t* tmp = (uint8_t*)malloc(tcap);
    size_t nb = skvo_stream_encode(SKVO_STEPS, eb, z, tp, tmp, tcap);
    if (nb >= rawb) {
        memcpy(out, tile_t, rawb);   /* (step, lane) order = tile order */
        *raw = 1;
        nb = rawb;
    } else {
        memcpy(out, tmp, nb);
        *raw = 0;
    }
    free(tmp);
    free(tabs);
    return (int64_t)nb;
}

/* Table of a blob as (n, freq[0..n]); for tests. */
int skvo_blob_table(const uint8_t* blob, size_t blob_bytes, uint64_t j, uint32_t* n, uint32_t* freq) {
    if (blob_bytes < SKVO_HDR) return E_TABLES;
    uint64_t nt = get32(blob + 8);
    if (j >= nt || SKVO_HDR + (j + 1) * SKVO_TAB_BYTES > blob_bytes) return E_ARG;
    const uint8_t* p = blob + SKVO_HDR + j * SKVO_TAB_BYTES;
    *n = get16(p);
    for (int q = 0; q < 256; ++q) freq[q] = get16(p + 2 + 2 * q);
    return E_OK;
}

/* Generic stream codec over caller-supplied tables, for pins on tiny
 * inputs: tabs_n[j], tabs_freq[j*257 ...] describe table j; tab_of[k*32+i]
 * selects the table of each position. */
static skvo_table* make_tables(int ntab, const uint32_t* tabs_n, const uint32_t* tabs_freq) {
    skvo_table* t = (skvo_table*)calloc((size_t)ntab, sizeof(skvo_table));
    for (int j = 0; j < ntab; ++j) {
        t[j].n = tabs_n[j];
        for (uint32_t q = 0; q <= tabs_n[j]; ++q) t[j].freq[q] = tabs_freq[j * 257 + q];
        table_cum(&t[j]);
    }
    return t;
}

int64_t skvo_stream_encode_ext(int steps, int ebytes, int ntab, const uint32_t* tabs_n, const uint32_t* tabs_freq,
                               const uint32_t* tab_of, const uint32_t* z, uint8_t* out, uint64_t cap) {
    skvo_table* t = make_tables(ntab, tabs_n, tabs_freq);
    const skvo_table** tp = (const skvo_table**)malloc((size_t)steps * SKVO_LANES * sizeof(*tp));
    for (int j = 0; j < steps * SKVO_LANES; ++j) tp[j] = &t[tab_of[j]];
    size_t nb = skvo_stream_encode(steps, ebytes, z, tp, out, cap);
    free(tp);
    free(t);
    return (int64_t)nb;
}

int skvo_stream_decode_ext(int steps, int ebytes, int ntab, const uint32_t* tabs_n, const uint32_t* tabs_freq,
                           const uint32_t* tab_of, const uint8_t* in, uint64_t nbytes, uint32_t* z) {
    skvo_table* t = make_tables(ntab, tabs_n, tabs_freq);
    const skvo_table** tp = (const skvo_table**)malloc((size_t)steps * SKVO_LANES * sizeof(*tp));
    for (int j = 0; j < steps * SKVO_LANES; ++j) tp[j] = &t[tab_of[j]];
    int rc = skvo_stream_decode(steps, ebytes, in, nbytes, tp, z);
    free(tp);
    free(t);
    return rc;
}

uint64_t skvo_n_streams(const skvo_shape* s) { return shape_ok(s) ? n_streams_of(s) : 0; }
