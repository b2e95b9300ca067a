// skv_fit.cpp -- host-side table fit, blob validation and hashing.
//
// Statistics are measured once on calibration data and then frozen
// ("Speculative KV coding ..." page, section "What to use as the
// predictor").  The model is a Laplace per channel (or per component and
// shift) integrated over unit quantization cells (DCKV page, "How it
// differs").  Everything here is fp64 and runs once; the coding kernels
// only ever see the resulting integer frequencies.
//
// The order of floating-point operations is part of the format: the scale
// is an exact sum divided once, the cell mass uses one of three closed forms
// chosen by the cell's position, the direct masses are summed in symbol order
// and rescaled as 4096 * (P * ((1 - p_esc) / sum)).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <vector>

#include "skv_internal.h"

namespace skv {

bool shape_supported(const skv_shape& s, bool need_tokens) {
    if (s.abi_version != SKV_ABI_VERSION) return false;
    if (s.channels == 0 || s.channels % kLanes != 0) return false;
    if (s.mode == SKV_RESIDUAL || s.mode == SKV_RESIDUAL_EXP) {
        if (s.dtype != SKV_BF16 && s.dtype != SKV_E4M3) return false;
        if (s.layers == 0 || s.kv == 0) return false;
        return !need_tokens || (s.tokens > 0 && s.tokens % kSteps == 0);
    }
    if (is_checkerboard(s.mode)) {
        if (s.dtype != SKV_INT16 || s.layers != 1 || s.kv != 1) return false;
        return !need_tokens || (s.tokens > 0 && s.tokens % (2 * kSteps) == 0);
    }
    return false;
}

uint64_t table_count(const skv_shape& s) {
    if (s.mode == SKV_RESIDUAL) return uint64_t(s.layers) * s.kv * s.channels;
    if (s.mode == SKV_RESIDUAL_EXP) return uint64_t(s.layers) * s.kv * kExpClasses;
    return uint64_t(s.channels) * 16;
}

uint64_t blob_size(const skv_shape& s) {
    const uint64_t bases = s.mode == SKV_RESIDUAL_EXP ? uint64_t(s.layers) * s.kv : 0;
    return kHeaderBytes + table_count(s) * kTableRecord + bases;
}

uint64_t stream_count(const skv_shape& s) {
    uint64_t groups = s.channels / kLanes;
    if (!is_checkerboard(s.mode)) return uint64_t(s.layers) * s.kv * (s.tokens / kSteps) * groups;
    return 2 * uint64_t(s.tokens / (2 * kSteps)) * groups;
}

uint64_t element_count(const skv_shape& s) {
    return uint64_t(s.layers) * s.kv * s.tokens * s.channels;
}

uint64_t fnv1a64(const uint8_t* p, size_t n) {
    uint64_t h = 0xcbf29ce484222325ull;   // FNV-1a 64-bit offset basis
    const uint64_t prime = 0x100000001b3ull;
    for (size_t i = 0; i < n; ++i) h = (h ^ p[i]) * prime;
    return h;
}

namespace {

// Mass of [v - 1/2, v + 1/2] under a Laplace of location m and scale b.
double laplace_cell(double v, double m, double b) {
    const double lo = v - 0.5 - m;
    const double hi = v + 0.5 - m;
    if (lo >= 0.0) return 0.5 * (std::exp(-lo / b) - std::exp(-hi / b));
    if (hi <= 0.0) return 0.5 * (std::exp(hi / b) - std::exp(lo / b));
    return 1.0 - 0.5 * std::exp(-hi / b) - 0.5 * std::exp(lo / b);
}

// Signed value of zigzag code z (0, -1, 1, -2, ...).
inline int32_t unzig(uint32_t z) { return (z & 1u) ? -int32_t((z + 1) >> 1) : int32_t(z >> 1); }

// ordered-integer residual of two N-bit float patterns, as signed N-bit.
inline int32_t ordered_residual(uint32_t t, uint32_t p, int nbits) {
    const uint32_t span = 1u << nbits, half = span >> 1, mask = span - 1;
    auto ordv = [&](uint32_t u) { return (u & half) ? (~u & mask) : (u | half); };
    uint32_t d = (ordv(t) - ordv(p)) & mask;
    return d >= half ? int32_t(d) - int32_t(span) : int32_t(d);
}

inline uint32_t zig_of(int32_t r, int nbits) {
    const uint32_t mask = (1u << nbits) - 1u;
    return (uint32_t(r) << 1 ^ uint32_t(r >> 31)) & mask;
}

// checkerboard mean in sixteenths (int32): G, plus 8 x (left + right) on odd rows
inline int32_t cb_mean(const int16_t* coef, const int16_t* G, uint32_t T, uint32_t C, uint32_t t, uint32_t c) {
    int32_t m = G[size_t(t) * C + c];
    if (t % 2 == 1) {
        const int32_t l = coef[size_t(t - 1) * C + c];
        const int32_t r = (t + 1 < T) ? coef[size_t(t + 1) * C + c] : l;
        m += 8 * (l + r);
    }
    return m;
}

struct Record {
    uint32_t n;
    uint32_t f[256];
};

// Largest-remainder rounding of q (sums to 4096) to frequencies >= 1.
void round_freqs(const std::vector<double>& q, uint32_t* f) {
    const size_t m = q.size();
    std::vector<double> rem(m);
    int64_t total = 0;
    for (size_t i = 0; i < m; ++i) {
        const double fl = std::floor(q[i]);
        f[i] = fl < 1.0 ? 1u : uint32_t(fl);
        rem[i] = q[i] - double(f[i]);
        total += f[i];
    }
    int64_t left = int64_t(kM) - total;
    if (left > 0) {
        std::vector<uint32_t> order(m);
        std::iota(order.begin(), order.end(), 0u);
        std::stable_sort(order.begin(), order.end(), [&](uint32_t a, uint32_t b) { return rem[a] > rem[b]; });
        for (int64_t i = 0; i < left; ++i) f[order[size_t(i)]] += 1;
    }
    for (; left < 0; ++left) {
        size_t best = m;
        for (size_t i = 0; i < m; ++i)
            if (f[i] > 1 && (best == m || f[i] > f[best])) best = i;
        f[best] -= 1;
    }
}

// Table from cell masses over z = 0..254, escape probability pe; the direct
// range covers every cell of mass >= 2^-12 and at least the first nmin symbols.
Record make_record(const double* mass, double pe, uint32_t nmin = 1) {
    Record r{};
    uint32_t n = 1;
    for (uint32_t z = 0; z < 255; ++z)
        if (mass[z] >= 1.0 / double(kM)) n = z + 1;
    n = std::max(n, std::min(nmin, 255u));
    double sum = 0.0;
    for (uint32_t z = 0; z < n; ++z) sum += mass[z];
    const double scale = (1.0 - pe) / sum;
    std::vector<double> q(n + 1);
    for (uint32_t z = 0; z < n; ++z) q[z] = double(kM) * (mass[z] * scale);
    q[n] = double(kM) * pe;
    r.n = n;
    round_freqs(q, r.f);
    return r;
}

void put_record(uint8_t* dst, const Record& r) {
    std::memset(dst, 0, kTableRecord);
    wr16(dst, r.n);
    for (uint32_t s = 0; s <= r.n; ++s) wr16(dst + 2 + 2 * s, r.f[s]);
}

void masses_for(double m, double b, double* out) {
    for (uint32_t z = 0; z < 255; ++z) out[z] = laplace_cell(double(unzig(z)), m, b);
}

// Smallest direct range (z in [1, 255]) that leaves at most total / 1024 of a
// slab's calibration symbols to escape.  The Laplace fit sets the direct range
// of each table from its masses; where the data's tail is heavier than the
// Laplace's, this floor keeps escapes near 1/1024 of the symbols.
uint32_t slab_tail_floor(const std::vector<uint64_t>& above_count_by_z, uint64_t total) {
    // above_count_by_z[z] = number of calibration symbols >= z (z = 0..255)
    const uint64_t budget = total / 1024;
    uint32_t z = 1;
    while (z < 255 && above_count_by_z[z] > budget) ++z;
    return z;
}

void fit_checkerboard(const int16_t* coef, const int16_t* G, uint32_t N, uint32_t C, uint8_t* rec);

}  // namespace

int fit_tables_host(const skv_shape& s, const void* calib_t, const void* calib_a, uint32_t calib_tokens,
                    uint8_t* blob, size_t blob_bytes) {
    const uint64_t nt = table_count(s);
    if (blob_bytes != blob_size(s)) return SKV_ERR_ARG;
    std::memset(blob, 0, kHeaderBytes);
    std::memcpy(blob, "SKVT", 4);
    wr16(blob + 4, 1);
    blob[6] = uint8_t(s.dtype);
    blob[7] = uint8_t(s.mode);
    wr32(blob + 8, uint32_t(nt));
    wr32(blob + 12, s.layers);
    wr32(blob + 16, s.kv);
    wr32(blob + 20, s.channels);
    wr32(blob + 24, calib_tokens);
    wr64(blob + 32, blob_bytes);
    uint8_t* rec = blob + kHeaderBytes;
    const uint32_t C = s.channels, N = calib_tokens;
    double mass[255];

    if (s.mode == SKV_RESIDUAL_EXP) {
        // One table per (slab, predictor exponent class).  The class base of a
        // slab starts the window of 16 exponents that holds the most
        // calibration predictors (the lowest such window); the table of a
        // class is the Laplace of the class's calibration residuals (the
        // slab's pooled scale below 64 in-range values), with the slab's
        // tail floor and the class's escape rate.  Sums run in element order.
        const int nbits = s.dtype == SKV_E4M3 ? 8 : 16;
        const uint32_t emax = s.dtype == SKV_E4M3 ? 15u : 255u;
        const uint64_t slabs = uint64_t(s.layers) * s.kv;
        const size_t per = size_t(N) * C;
        auto elem = [&](const void* a, size_t i) -> uint32_t {
            return nbits == 8 ? static_cast<const uint8_t*>(a)[i] : static_cast<const uint16_t*>(a)[i];
        };
        std::vector<int32_t> r(per);
        std::vector<uint8_t> cls(per);
        std::vector<uint64_t> above(257);
        uint8_t* bases = blob + kHeaderBytes + nt * kTableRecord;
        for (uint64_t sl = 0; sl < slabs; ++sl) {
            std::fill(above.begin(), above.end(), 0ull);
            uint64_t hist[256] = {};
            for (size_t i = 0; i < per; ++i) {
                const uint32_t pv = elem(calib_a, sl * per + i);
                r[i] = ordered_residual(elem(calib_t, sl * per + i), pv, nbits);
                above[std::min<uint32_t>(zig_of(r[i], nbits), 255u)] += 1;
                hist[exp_field(pv, s.dtype)] += 1;
            }
            for (int z = 254; z >= 0; --z) above[size_t(z)] += above[size_t(z) + 1];
            const uint32_t floor_n = slab_tail_floor(above, per);
            uint32_t base = 0;
            uint64_t best = 0, win = 0;
            for (uint32_t e = 0; e < 16; ++e) win += hist[e];
            best = win;
            for (uint32_t b0 = 1; b0 + 15 <= emax; ++b0) {
                win += hist[b0 + 15] - hist[b0 - 1];
                if (win > best) {
                    best = win;
                    base = b0;
                }
            }
            bases[sl] = uint8_t(base);
            double acc_all = 0.0;
            uint64_t used_all = 0;
            for (size_t i = 0; i < per; ++i) {
                cls[i] = uint8_t(exp_class(elem(calib_a, sl * per + i), s.dtype, base));
                if (std::abs(r[i]) <= 127) {
                    acc_all += double(std::abs(r[i]));
                    ++used_all;
                }
            }
            const double b_all = std::max(used_all ? acc_all / double(used_all) : 0.0, 0.05);
            for (uint32_t q = 0; q < kExpClasses; ++q) {
                double acc = 0.0;
                uint64_t used = 0, members = 0;
                for (size_t i = 0; i < per; ++i) {
                    if (cls[i] != q) continue;
                    ++members;
                    if (std::abs(r[i]) <= 127) {
                        acc += double(std::abs(r[i]));
                        ++used;
                    }
                }
                const double b = std::max(used >= 64 ? acc / double(used) : b_all, 0.05);
                masses_for(0.0, b, mass);
                const Record R = make_record(mass, 0.0, floor_n);
                uint64_t esc = 0;
                for (size_t i = 0; i < per; ++i) esc += cls[i] == q && zig_of(r[i], nbits) >= R.n;
                const double pe = (double(esc) + 1.0) / (double(members) + 2.0);
                put_record(rec + (sl * kExpClasses + q) * kTableRecord, make_record(mass, pe, floor_n));
            }
        }
        return SKV_OK;
    }

    if (s.mode == SKV_RESIDUAL) {
        const int nbits = s.dtype == SKV_E4M3 ? 8 : 16;
        const uint64_t slabs = uint64_t(s.layers) * s.kv;
        auto elem = [&](const void* a, size_t i) -> uint32_t {
            return nbits == 8 ? static_cast<const uint8_t*>(a)[i] : static_cast<const uint16_t*>(a)[i];
        };
        std::vector<int32_t> r(N);
        std::vector<uint64_t> above(257);
        for (uint64_t sl = 0; sl < slabs; ++sl) {
            // the slab's pooled symbol counts, turned into counts of symbols >= z
            std::fill(above.begin(), above.end(), 0ull);
            for (size_t i = size_t(sl) * N * C, e = i + size_t(N) * C; i < e; ++i)
                above[std::min<uint32_t>(zig_of(ordered_residual(elem(calib_t, i), elem(calib_a, i), nbits), nbits), 255u)] += 1;
            for (int z = 254; z >= 0; --z) above[size_t(z)] += above[size_t(z) + 1];
            const uint32_t floor_n = slab_tail_floor(above, uint64_t(N) * C);
            for (uint32_t c = 0; c < C; ++c) {
                double acc = 0.0;
                uint64_t used = 0;
                for (uint32_t t = 0; t < N; ++t) {
                    const size_t i = (size_t(sl) * N + t) * C + c;
                    r[t] = ordered_residual(elem(calib_t, i), elem(calib_a, i), nbits);
                    const int32_t a = std::abs(r[t]);
                    if (a <= 127) {
                        acc += double(a);
                        ++used;
                    }
                }
                double b = used ? acc / double(used) : 0.0;
                b = std::max(b, 0.05);
                masses_for(0.0, b, mass);
                Record R = make_record(mass, 0.0, floor_n);   // direct range does not depend on pe
                uint64_t esc = 0;
                for (uint32_t t = 0; t < N; ++t) esc += zig_of(r[t], nbits) >= R.n;
                const double pe = (double(esc) + 1.0) / (double(N) + 2.0);
                put_record(rec + (sl * C + c) * kTableRecord, make_record(mass, pe, floor_n));
            }
        }
        return SKV_OK;
    }

    if (s.mode != SKV_CHECKERBOARD) return SKV_ERR_SHAPE;     // the map mode fits through fit_tables_map_host
    fit_checkerboard(static_cast<const int16_t*>(calib_t), static_cast<const int16_t*>(calib_a), N, C, rec);
    return SKV_OK;
}

namespace {

// Checkerboard records (16 shifted tables per component) from calibration
// coefficients and their side input, [N][C].
void fit_checkerboard(const int16_t* coef, const int16_t* G, uint32_t N, uint32_t C, uint8_t* rec) {
    std::vector<int32_t> mu(N);
    for (uint32_t c = 0; c < C; ++c) {
        double acc = 0.0;
        uint64_t used = 0;
        for (uint32_t t = 0; t < N; ++t) {
            mu[t] = cb_mean(coef, G, N, C, t, c);
            const double e = std::fabs(double(coef[size_t(t) * C + c]) - double(mu[t]) / 16.0);
            if (e <= 127.0) {
                acc += e;
                ++used;
            }
        }
        double b = used ? acc / double(used) : 0.0;
        b = std::max(b, 0.05);
        double shifted[16][255];
        uint32_t ndir[16];
        for (int f = 0; f < 16; ++f) {
            masses_for(double(f) / 16.0, b, shifted[f]);
            ndir[f] = make_record(shifted[f], 0.0).n;
        }
        uint64_t esc = 0;
        for (uint32_t t = 0; t < N; ++t) {
            const int32_t k = mu[t] >> 4;   // arithmetic shift: floor
            const int32_t f = mu[t] & 15;
            const int32_t d = int32_t(int16_t(uint16_t(uint32_t(coef[size_t(t) * C + c] - k))));
            esc += zig_of(d, 16) >= ndir[f];
        }
        const double pe = (double(esc) + 1.0) / (double(N) + 2.0);
        for (int f = 0; f < 16; ++f) put_record(rec + (size_t(c) * 16 + f) * kTableRecord, make_record(shifted[f], pe));
    }
}

// floor((v + 2^(s-1)) / 2^s): v / 2^s rounded half up (arithmetic shift).
inline int64_t round_half_up(int64_t v, uint32_t s) { return s ? (v + (int64_t(1) << (s - 1))) >> s : v; }

}  // namespace

void nbr_map_host(const int16_t* coef, const int16_t* G, uint32_t T, uint32_t C, const skv_nbr_map& map,
                  int16_t* Gout) {
    const uint32_t K = map.rank, W = 2 * C;
    std::vector<int64_t> in(W), q(K);
    for (uint32_t t = 0; t < T; ++t) {
        std::memcpy(Gout + size_t(t) * C, G + size_t(t) * C, size_t(C) * 2);
        if (t % 2 == 0) continue;
        const int16_t* l = coef + size_t(t - 1) * C;
        const int16_t* r = t + 1 < T ? coef + size_t(t + 1) * C : l;
        for (uint32_t i = 0; i < C; ++i) {
            in[i] = std::min<int64_t>(l[i], 32639);
            in[C + i] = std::min<int64_t>(r[i], 32639);
        }
        for (uint32_t j = 0; j < K; ++j) {
            const int8_t* v = map.V + size_t(j) * W;
            int64_t h = 0;
            for (uint32_t i = 0; i < W; ++i) h += int64_t(v[i]) * in[i];
            q[j] = std::clamp<int64_t>(round_half_up(h, map.shift_h), -128, 127);
        }
        for (uint32_t c = 0; c < C; ++c) {
            const int8_t* u = map.U + size_t(c) * K;
            int64_t m = 0;
            for (uint32_t j = 0; j < K; ++j) m += int64_t(u[j]) * q[j];
            const int64_t g = int64_t(G[size_t(t) * C + c]) + round_half_up(m, map.shift_m);
            Gout[size_t(t) * C + c] = int16_t(std::clamp<int64_t>(g, -32768, 32767));
        }
    }
}

int fit_tables_map_host(const skv_shape& s, const int16_t* calib_coef, const int16_t* calib_G,
                        uint32_t calib_tokens, const skv_nbr_map& map, uint8_t* blob, size_t blob_bytes) {
    const uint32_t C = s.channels;
    if (blob_bytes != blob_size(s) + map_section_bytes(map.rank, C)) return SKV_ERR_ARG;
    std::memset(blob, 0, kHeaderBytes);
    std::memcpy(blob, "SKVT", 4);
    wr16(blob + 4, 1);
    blob[6] = uint8_t(s.dtype);
    blob[7] = uint8_t(s.mode);
    wr32(blob + 8, uint32_t(table_count(s)));
    wr32(blob + 12, s.layers);
    wr32(blob + 16, s.kv);
    wr32(blob + 20, C);
    wr32(blob + 24, calib_tokens);
    wr64(blob + 32, blob_bytes);
    std::vector<int16_t> g2(size_t(calib_tokens) * C);
    nbr_map_host(calib_coef, calib_G, calib_tokens, C, map, g2.data());
    fit_checkerboard(calib_coef, g2.data(), calib_tokens, C, blob + kHeaderBytes);
    uint8_t* m = blob + blob_size(s);
    std::memset(m, 0, kMapHeader);
    wr32(m, map.rank);
    wr32(m + 4, map.shift_h);
    wr32(m + 8, map.shift_m);
    std::memcpy(m + kMapHeader, map.V, size_t(map.rank) * 2 * C);
    std::memcpy(m + kMapHeader + size_t(map.rank) * 2 * C, map.U, size_t(map.rank) * C);
    return SKV_OK;
}

int validate_blob(const uint8_t* b, size_t bytes) {
    if (bytes < kHeaderBytes || std::memcmp(b, "SKVT", 4) != 0 || rd16(b + 4) != 1) return SKV_ERR_TABLES;
    skv_shape s{SKV_ABI_VERSION, b[6], b[7], rd32(b + 12), rd32(b + 16), 0, rd32(b + 20)};
    if (!shape_supported(s, false)) return SKV_ERR_TABLES;
    const uint64_t nt = table_count(s);
    uint64_t want = blob_size(s);
    if (s.mode == SKV_CHECKERBOARD_MAP) {
        if (bytes < want + kMapHeader) return SKV_ERR_TABLES;
        const uint8_t* m = b + want;
        if (!map_params_ok(rd32(m), rd32(m + 4), rd32(m + 8)) || rd32(m + 12) != 0) return SKV_ERR_TABLES;
        want += map_section_bytes(rd32(m), s.channels);
    }
    if (rd32(b + 8) != nt || rd64(b + 32) != bytes || bytes != want) return SKV_ERR_TABLES;
    for (uint64_t j = 0; j < nt; ++j) {
        const uint8_t* r = b + kHeaderBytes + j * kTableRecord;
        const uint32_t n = rd16(r);
        if (n < 1 || n > uint32_t(kMaxDirect)) return SKV_ERR_TABLES;
        uint32_t sum = 0;
        for (uint32_t q = 0; q < 256; ++q) {
            const uint32_t f = rd16(r + 2 + 2 * q);
            if (q <= n ? f == 0 : f != 0) return SKV_ERR_TABLES;
            sum += f;
        }
        if (sum != kM) return SKV_ERR_TABLES;
    }
    return SKV_OK;
}

}  // namespace skv
