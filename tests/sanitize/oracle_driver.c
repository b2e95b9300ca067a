/* Drives the oracle (built together with this file under AddressSanitizer
 * and UndefinedBehaviorSanitizer) through fits, encodes and decodes of small
 * synthetic caches in every mode, then through damaged inputs: every byte of
 * a container's head and many payload bytes flipped, truncations, and
 * damaged table blobs.  Test infrastructure: the sanitizers report any
 * out-of-bounds access, use after free, leak or undefined operation, and
 * the exit status says whether every round trip was exact. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct { uint32_t dtype, mode, layers, kv, tokens, channels; } skvo_shape;
uint64_t skvo_blob_bytes(const skvo_shape* s);
uint64_t skvo_blob_bytes_map(const skvo_shape* s, uint32_t k);
uint64_t skvo_bound(const skvo_shape* s);
int skvo_fit_tables(const skvo_shape* s, const void* ct, const void* ca, uint32_t calib_tokens, uint8_t* blob,
                    uint64_t cap, uint64_t* bytes);
int skvo_fit_tables_map(const skvo_shape* s, const int16_t* cc, const int16_t* cg, uint32_t calib_tokens, uint32_t k,
                        uint32_t sh1, uint32_t sh2, const int8_t* V, const int8_t* U, uint8_t* blob, uint64_t cap,
                        uint64_t* bytes);
int64_t skvo_encode(const uint8_t* blob, size_t blob_bytes, const skvo_shape* s, const void* tgt, const void* aux,
                    uint8_t* out, uint64_t cap, uint64_t* need, int nthreads);
int skvo_decode(const uint8_t* blob, size_t blob_bytes, const uint8_t* in, uint64_t in_bytes, const void* aux,
                void* out, uint64_t out_bytes, int nthreads);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {           /* xorshift64* */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (uint32_t)((rng * 0x2545F4914F6CDD1Dull) >> 32);
}
/* a value near the predictor: small residuals mostly, a few far ones */
static uint32_t near(uint32_t p, uint32_t mask) {
    uint32_t r = next32();
    int32_t d = (r & 0xFF) < 4 ? (int32_t)(next32() & mask) : (int32_t)(r % 9) - 4;
    return (p + (uint32_t)d) & mask;
}

static int run(uint32_t dtype, uint32_t mode, uint32_t layers, uint32_t kv, uint32_t tokens, uint32_t channels) {
    skvo_shape s = {dtype, mode, layers, kv, tokens, channels};
    int eb = dtype == 2 ? 1 : 2;
    uint32_t mask = eb == 1 ? 0xFFu : 0xFFFFu;
    size_t n = (size_t)layers * kv * tokens * channels, nc = (size_t)layers * kv * 256 * channels;
    uint8_t *t = malloc(n * eb), *p = malloc(n * eb), *ct = malloc(nc * eb), *cp = malloc(nc * eb);
    for (size_t i = 0; i < n; ++i) {
        uint32_t pv = next32() & mask, tv = near(pv, mask);
        if (mode == 1 || mode == 3) pv = (uint32_t)((int32_t)(next32() % 4001) - 2000) & mask;  /* G, 1/16 cells */
        if (eb == 1) { p[i] = (uint8_t)pv; t[i] = (uint8_t)tv; }
        else { ((uint16_t*)p)[i] = (uint16_t)pv; ((uint16_t*)t)[i] = (uint16_t)tv; }
    }
    for (size_t i = 0; i < nc * eb; ++i) { cp[i] = p[i % (n * eb)]; ct[i] = t[i % (n * eb)]; }
    int8_t* V = NULL;
    int8_t* U = NULL;
    uint64_t bb = 0;
    uint8_t* blob;
    if (mode == 3) {
        V = malloc(16 * 2 * channels);
        U = malloc(16 * channels);
        for (uint32_t i = 0; i < 32 * channels; ++i) V[i] = (int8_t)(next32() % 21) - 10;
        for (uint32_t i = 0; i < 16 * channels; ++i) U[i] = (int8_t)(next32() % 9) - 4;
        bb = skvo_blob_bytes_map(&s, 16);
        blob = malloc(bb);
        if (skvo_fit_tables_map(&s, (int16_t*)ct, (int16_t*)cp, 256, 16, 6, 2, V, U, blob, bb, &bb)) return 1;
    } else {
        bb = skvo_blob_bytes(&s);
        blob = malloc(bb);
        if (skvo_fit_tables(&s, ct, cp, 256, blob, bb, &bb)) return 1;
    }
    uint64_t cap = skvo_bound(&s), need = 0;
    uint8_t* c = malloc(cap);
    int64_t cb = skvo_encode(blob, bb, &s, t, p, c, cap, &need, 2);
    if (cb <= 0) return 2;
    uint8_t* back = malloc(n * eb);
    if (skvo_decode(blob, bb, c, (uint64_t)cb, p, back, n * eb, 2) || memcmp(back, t, n * eb)) return 3;
    /* damaged containers: the decoder must return (any status) without a memory error */
    uint8_t* bad = malloc((size_t)cb);
    uint64_t nstream = 0;
    memcpy(&nstream, c + 32, 8);
    uint64_t head = 64 + 8 * (nstream + 1);
    for (uint64_t i = 0; i < (uint64_t)cb; i += (i < head ? 1 + head / 64 : 1 + (uint64_t)cb / 300)) {
        memcpy(bad, c, (size_t)cb);
        bad[i] ^= (uint8_t)(1u << (next32() & 7));
        (void)skvo_decode(blob, bb, bad, (uint64_t)cb, p, back, n * eb, 1);
    }
    for (uint64_t cut = 0; cut < (uint64_t)cb; cut += 1 + (uint64_t)cb / 32)
        (void)skvo_decode(blob, bb, c, cut, p, back, n * eb, 1);
    /* index entries pointing anywhere */
    for (int k = 0; k < 32; ++k) {
        memcpy(bad, c, (size_t)cb);
        uint64_t v = ((uint64_t)next32() << 32) | next32(), at = 64 + 8 * (next32() % (nstream + 1));
        memcpy(bad + at, &v, 8);
        (void)skvo_decode(blob, bb, bad, (uint64_t)cb, p, back, n * eb, 1);
    }
    /* damaged blobs */
    uint8_t* b2 = malloc(bb);
    for (uint64_t i = 0; i < bb; i += 1 + bb / 96) {
        memcpy(b2, blob, bb);
        b2[i] ^= 0x5A;
        (void)skvo_decode(b2, bb, c, (uint64_t)cb, p, back, n * eb, 1);
        (void)skvo_encode(b2, bb, &s, t, p, bad, (uint64_t)cb, &need, 1);
    }
    (void)skvo_decode(blob, bb / 2, c, (uint64_t)cb, p, back, n * eb, 1);
    free(b2); free(bad); free(back); free(c); free(blob); free(V); free(U);
    free(t); free(p); free(ct); free(cp);
    return 0;
}

int main(void) {
    int rc = 0;
    rc |= run(1, 0, 2, 2, 256, 64);        /* bf16, per-channel tables */
    rc |= run(2, 0, 1, 2, 384, 96) << 4;   /* e4m3 */
    rc |= run(1, 2, 1, 2, 256, 64) << 8;   /* bf16, exponent-class tables */
    rc |= run(2, 2, 2, 1, 256, 32) << 12;  /* e4m3, exponent-class tables */
    rc |= run(3, 1, 1, 1, 512, 64) << 16;  /* checkerboard */
    rc |= run(3, 3, 1, 1, 512, 64) << 20;  /* checkerboard with the neighbour map */
    printf("oracle driver: %s (%x)\n", rc ? "FAILED" : "ok", rc);
    return rc != 0;
}
