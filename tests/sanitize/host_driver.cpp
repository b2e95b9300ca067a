// Drives the library's host code (the fp64 table fit in every mode, the
// neighbour-map fit and blob validation), built under AddressSanitizer and
// UndefinedBehaviorSanitizer, through fits of small synthetic calibration
// arrays and through validation of damaged, truncated and random blobs.
// Test infrastructure: the sanitizers report any invalid access or
// undefined operation; the exit status says whether every fitted blob
// validated and every damaged one was handled.
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../lossless_kv_cache_amd/csrc/skv_internal.h"

static uint64_t rng = 0x2545F4914F6CDD1Dull;
static uint32_t next32() {
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return uint32_t((rng * 0x9E3779B97F4A7C15ull) >> 32);
}

static int fit_and_damage(uint32_t dtype, uint32_t mode, uint32_t layers, uint32_t kv, uint32_t channels) {
    skv_shape s{SKV_ABI_VERSION, dtype, mode, layers, kv, 0, channels};
    if (!skv::shape_supported(s, false)) return 1;
    const uint32_t N = 256;
    const size_t n = size_t(layers) * kv * N * channels;
    const uint32_t eb = skv::elem_bytes(dtype), mask = eb == 1 ? 0xFFu : 0xFFFFu;
    std::vector<uint8_t> t(n * eb), a(n * eb);
    for (size_t i = 0; i < n; ++i) {
        uint32_t pv = next32() & mask, d = (next32() & 0xFF) < 3 ? next32() : next32() % 7 - 3;
        if (skv::is_checkerboard(mode)) pv = uint32_t(int32_t(next32() % 4001) - 2000) & mask;
        const uint32_t tv = (pv + d) & mask;
        if (eb == 1) {
            a[i] = uint8_t(pv);
            t[i] = uint8_t(tv);
        } else {
            reinterpret_cast<uint16_t*>(a.data())[i] = uint16_t(pv);
            reinterpret_cast<uint16_t*>(t.data())[i] = uint16_t(tv);
        }
    }
    std::vector<uint8_t> blob;
    std::vector<int8_t> V, U;
    if (mode == SKV_CHECKERBOARD_MAP) {
        const uint32_t k = 32;
        V.resize(size_t(k) * 2 * channels);
        U.resize(size_t(channels) * k);
        for (auto& v : V) v = int8_t(int(next32() % 255) - 127);
        for (auto& u : U) u = int8_t(int(next32() % 255) - 127);
        const skv_nbr_map m{k, 12, 3, V.data(), U.data()};
        blob.resize(skv::blob_size(s) + skv::map_section_bytes(k, channels));
        if (skv::fit_tables_map_host(s, reinterpret_cast<const int16_t*>(t.data()),
                                     reinterpret_cast<const int16_t*>(a.data()), N, m, blob.data(), blob.size()))
            return 2;
    } else {
        blob.resize(skv::blob_size(s));
        if (skv::fit_tables_host(s, t.data(), a.data(), N, blob.data(), blob.size())) return 2;
    }
    if (skv::validate_blob(blob.data(), blob.size()) != SKV_OK) return 3;
    std::vector<uint8_t> bad;
    for (size_t i = 0; i < blob.size(); i += 1 + blob.size() / 2000) {
        bad = blob;
        bad[i] ^= uint8_t(1u << (next32() & 7));
        (void)skv::validate_blob(bad.data(), bad.size());
    }
    for (size_t cut = 0; cut < blob.size(); cut += 1 + blob.size() / 97) (void)skv::validate_blob(blob.data(), cut);
    // random bytes after a plausible header
    for (int r = 0; r < 50; ++r) {
        bad = blob;
        for (size_t i = 8; i < std::min<size_t>(bad.size(), 80); ++i) bad[i] = uint8_t(next32());
        (void)skv::validate_blob(bad.data(), bad.size());
    }
    return 0;
}

int main() {
    int rc = 0;
    rc |= fit_and_damage(SKV_BF16, SKV_RESIDUAL, 2, 2, 64);
    rc |= fit_and_damage(SKV_E4M3, SKV_RESIDUAL, 1, 2, 96) << 4;
    rc |= fit_and_damage(SKV_BF16, SKV_RESIDUAL_EXP, 1, 2, 64) << 8;
    rc |= fit_and_damage(SKV_E4M3, SKV_RESIDUAL_EXP, 2, 1, 32) << 12;
    rc |= fit_and_damage(SKV_INT16, SKV_CHECKERBOARD, 1, 1, 64) << 16;
    rc |= fit_and_damage(SKV_INT16, SKV_CHECKERBOARD_MAP, 1, 1, 64) << 20;
    std::printf("host driver: %s (%x)\n", rc ? "FAILED" : "ok", rc);
    return rc != 0;
}
