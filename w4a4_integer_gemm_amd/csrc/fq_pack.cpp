// Host-side weight packer: fold the smoothing vector and the block Hadamard
// rotation into each weight row, then round it per row to symmetric INT8/INT4
// codes with one float32 scale (vla.cpp FoldQuant page: INT8 or INT4 codes
// with per-row scales in a block-Hadamard, SmoothQuant-folded frame; the
// bring-up exporter does "rotation and per-row RTN").
//
// Fold algebra (dequant-mode commit of that page): the activation frame is
// R(x/a) or R(x)/a, so for the product to stay x . w_n the stored row is
// u_n = R(a . w_n) (fold before) or a . R(w_n) (fold after).  The fold runs in
// float64; the butterfly runs its stages with span 1, 2, ..., b/2 and then
// scales by 1/sqrt(b).  Codes round half-to-even against the stored float32
// scale s_n = (float)(max|u_n| / qmax) and clamp to +-qmax.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/fq.h"
#include "fq_internal.h"

namespace {

void rotate_row(double* u, int32_t K, int32_t b) {
    if (b > 1) {
        for (int32_t base = 0; base < K; base += b) {
            double* blk = u + base;
            for (int32_t span = 1; span < b; span *= 2)
                for (int32_t i0 = 0; i0 < b; i0 += 2 * span)
                    for (int32_t i = i0; i < i0 + span; ++i) {
                        const double lo = blk[i], hi = blk[i + span];
                        blk[i] = lo + hi;
                        blk[i + span] = lo - hi;
                    }
        }
    }
    const double norm = 1.0 / std::sqrt(static_cast<double>(b));
    for (int32_t k = 0; k < K; ++k) u[k] *= norm;
}

size_t code_row_bytes(int32_t K, int32_t bits) {
    return bits == 8 ? size_t(K) : bits == FQ_CODES_E2M3 ? size_t(3 * (K / 4)) : size_t(K / 2);
}

// FP6 E2M3 pattern of an integer code |q| <= 7: the exponent is the position of
// the leading one plus the bias 1, the three mantissa bits the ones below it
// (q = 2^(e-1) (1 + m/8)); 0 is the zero pattern.
uint32_t e2m3_pattern(int32_t q) {
    if (q == 0) return 0;
    const uint32_t sign = q < 0 ? 32u : 0u;
    const int32_t mag = q < 0 ? -q : q;
    const int32_t e = mag >= 4 ? 3 : mag >= 2 ? 2 : 1;
    const int32_t m = ((mag * 8) >> (e - 1)) - 8;
    return sign | uint32_t(e << 3) | uint32_t(m);
}

// Value of an E2M3 pattern (exponent 0 is subnormal: m/8).
double e2m3_number(uint32_t f) {
    const int32_t e = (f >> 3) & 3, m = f & 7;
    const double mag = e == 0 ? m / 8.0 : std::ldexp(1.0 + m / 8.0, e - 1);
    return (f & 32) ? -mag : mag;
}

void pack_rows(const float* W, int32_t n0, int32_t n1, int32_t K, const float* a, int32_t fold_after, int32_t b,
               int32_t bits, uint8_t* codes, float* wscale) {
    const int32_t qmax = bits == 8 ? 127 : 7;
    const size_t row_bytes = code_row_bytes(K, bits);
    std::vector<double> u(K);
    std::vector<int32_t> q(K);
    for (int32_t n = n0; n < n1; ++n) {
        const float* w = W + int64_t(n) * K;
        for (int32_t k = 0; k < K; ++k) u[k] = static_cast<double>(w[k]);
        if (a && !fold_after)
            for (int32_t k = 0; k < K; ++k) u[k] *= static_cast<double>(a[k]);
        rotate_row(u.data(), K, b);
        if (a && fold_after)
            for (int32_t k = 0; k < K; ++k) u[k] *= static_cast<double>(a[k]);
        double amax = 0.0;
        for (int32_t k = 0; k < K; ++k) amax = std::max(amax, std::fabs(u[k]));
        const float s = static_cast<float>(amax / qmax);
        const double sd = static_cast<double>(s);
        for (int32_t k = 0; k < K; ++k) {
            double r = s > 0.0f ? std::nearbyint(u[k] / sd) : 0.0;
            r = std::min<double>(std::max<double>(r, -qmax), qmax);
            q[k] = static_cast<int32_t>(r);
        }
        uint8_t* row = codes + size_t(n) * row_bytes;
        if (bits == 8) {
            for (int32_t k = 0; k < K; ++k) row[k] = static_cast<uint8_t>(static_cast<int8_t>(q[k]));
        } else if (bits == FQ_CODES_E2M3) {
            // four 6-bit fields -> three bytes, value k at bits 6k .. 6k+5
            for (int32_t j = 0; j < K / 4; ++j) {
                uint32_t w = 0;
                for (int32_t i = 0; i < 4; ++i) w |= e2m3_pattern(q[4 * j + i]) << (6 * i);
                row[3 * j + 0] = uint8_t(w);
                row[3 * j + 1] = uint8_t(w >> 8);
                row[3 * j + 2] = uint8_t(w >> 16);
            }
        } else {
            for (int32_t j = 0; j < K / 2; ++j)
                row[j] = static_cast<uint8_t>((q[2 * j] & 0xF) | ((q[2 * j + 1] & 0xF) << 4));
        }
        wscale[n] = s;
    }
}

// Dequantised row in the original frame: v = s q, then R(v)/a (fold before) or
// R(v/a) (fold after); R is its own inverse, so this undoes the packer's fold.
void dequant_rows(const uint8_t* codes, const float* wscale, int32_t n0, int32_t n1, int32_t K, const float* a,
                  int32_t fold_after, int32_t b, int32_t bits, float* W) {
    const size_t row_bytes = code_row_bytes(K, bits);
    std::vector<double> v(K);
    for (int32_t n = n0; n < n1; ++n) {
        const uint8_t* row = codes + size_t(n) * row_bytes;
        const double s = static_cast<double>(wscale[n]);
        for (int32_t k = 0; k < K; ++k) {
            double q;
            if (bits == 8) {
                q = static_cast<int8_t>(row[k]);
            } else if (bits == FQ_CODES_E2M3) {
                const uint8_t* t = row + 3 * (k / 4);
                const uint32_t w = uint32_t(t[0]) | (uint32_t(t[1]) << 8) | (uint32_t(t[2]) << 16);
                q = e2m3_number((w >> (6 * (k % 4))) & 63u);
            } else {
                const int32_t nib = (row[k / 2] >> (4 * (k & 1))) & 0xF;
                q = nib >= 8 ? nib - 16 : nib;
            }
            v[k] = s * q;
        }
        if (a && fold_after)
            for (int32_t k = 0; k < K; ++k) v[k] /= static_cast<double>(a[k]);
        rotate_row(v.data(), K, b);
        if (a && !fold_after)
            for (int32_t k = 0; k < K; ++k) v[k] /= static_cast<double>(a[k]);
        float* w = W + int64_t(n) * K;
        for (int32_t k = 0; k < K; ++k) w[k] = static_cast<float>(v[k]);
    }
}

// Shared argument checks of the two host row transforms; returns FQ_OK or sets the message.
fq_status check_rows(const char* fn, int32_t N, int32_t K, const float* ascale, int32_t fold_after, int32_t hblock,
                     int32_t wbits) {
    char buf[256];
    auto fail = [&](fq_status s) {
        fq::set_error(buf);
        return s;
    };
    if (wbits != 8 && wbits != 4 && wbits != FQ_CODES_E2M3) {
        snprintf(buf, sizeof buf, "%s: wbits=%d is not a supported code width (4, 8, or 6 for E2M3)", fn, wbits);
        return fail(FQ_ERR_UNSUPPORTED);
    }
    if (N < 1) {
        snprintf(buf, sizeof buf, "%s: N=%d must be >= 1", fn, N);
        return fail(FQ_ERR_SHAPE);
    }
    if (K < 128 || K > 65536 || K % 128) {
        snprintf(buf, sizeof buf, "%s: K=%d must be a multiple of 128 in [128, 65536] (%d/128 = %.2f)", fn, K, K,
                 K / 128.0);
        return fail(FQ_ERR_SHAPE);
    }
    if (hblock < 1 || hblock > 256 || (hblock & (hblock - 1))) {
        snprintf(buf, sizeof buf, "%s: hblock=%d must be a power of two in [1, 256]", fn, hblock);
        return fail(FQ_ERR_SHAPE);
    }
    if (K % hblock) {
        snprintf(buf, sizeof buf, "%s: K=%d not divisible by hblock=%d (%d/%d = %.2f)", fn, K, hblock, K, hblock,
                 double(K) / hblock);
        return fail(FQ_ERR_SHAPE);
    }
    if (fold_after != 0 && fold_after != 1) {
        snprintf(buf, sizeof buf, "%s: fold_after=%d must be 0 or 1", fn, fold_after);
        return fail(FQ_ERR_ARG);
    }
    if (ascale)
        for (int32_t k = 0; k < K; ++k)
            if (!(ascale[k] > 0.0f) || !std::isfinite(ascale[k])) {
                snprintf(buf, sizeof buf, "%s: ascale[%d]=%g must be finite and > 0", fn, k, double(ascale[k]));
                return fail(FQ_ERR_ARG);
            }
    return FQ_OK;
}

// Runs rows [0, N) of `fn(n0, n1)` on up to 16 host threads.  No exception
// leaves it: a range whose thread cannot be started runs on the calling
// thread, and a range that throws (an allocation failure) is reported by the
// false return.
template <class F>
bool parallel_rows(int32_t N, F fn) {
    std::atomic<bool> ok{true};
    auto run = [&](int32_t n0, int32_t n1) {
        try {
            fn(n0, n1);
        } catch (...) {
            ok.store(false);
        }
    };
    unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    nt = std::min<unsigned>(nt, unsigned(N));
    std::vector<std::thread> pool;
    try {
        pool.reserve(nt);
    } catch (...) {
        nt = 1;
    }
    const int32_t per = (N + int32_t(nt) - 1) / int32_t(nt);
    // range t = rows [t per, (t + 1) per); the calling thread takes range 0
    for (unsigned t = 1; t < nt; ++t) {
        const int32_t n0 = int32_t(t) * per, n1 = std::min(N, n0 + per);
        if (n0 >= n1) break;
        try {
            pool.emplace_back(run, n0, n1);
        } catch (...) {
            run(n0, n1);
        }
    }
    run(0, std::min(N, per));
    for (auto& th : pool) th.join();
    return ok.load();
}

}  // namespace

extern "C" fq_status fq_pack_weights(const float* W, int32_t N, int32_t K, const float* ascale, int32_t fold_after,
                                     int32_t hblock, int32_t wbits, void* codes_out, float* wscale_out) {
    fq::clear_error();
    auto fail = [](fq_status s, const std::string& m) {
        fq::set_error(m);
        return s;
    };
    if (!W || !codes_out || !wscale_out) return fail(FQ_ERR_ARG, "fq_pack_weights: W, codes_out or wscale_out is NULL");
    const fq_status st = check_rows("fq_pack_weights", N, K, ascale, fold_after, hblock, wbits);
    if (st != FQ_OK) return st;
    if (!parallel_rows(N, [&](int32_t n0, int32_t n1) {
            pack_rows(W, n0, n1, K, ascale, fold_after, hblock, wbits, static_cast<uint8_t*>(codes_out), wscale_out);
        }))
        return fail(FQ_ERR_ARG, "fq_pack_weights: host memory for the row buffers could not be allocated");
    return FQ_OK;
}

extern "C" fq_status fq_dequant_rows(const void* codes, const float* wscale, int32_t N, int32_t K,
                                     const float* ascale, int32_t fold_after, int32_t hblock, int32_t wbits,
                                     float* W_out) {
    fq::clear_error();
    if (!codes || !wscale || !W_out) {
        fq::set_error("fq_dequant_rows: codes, wscale or W_out is NULL");
        return FQ_ERR_ARG;
    }
    const fq_status st = check_rows("fq_dequant_rows", N, K, ascale, fold_after, hblock, wbits);
    if (st != FQ_OK) return st;
    for (int32_t n = 0; n < N; ++n)
        if (!(wscale[n] >= 0.0f) || !std::isfinite(wscale[n])) {
            char buf[128];
            snprintf(buf, sizeof buf, "fq_dequant_rows: wscale[%d]=%g must be finite and >= 0", n, double(wscale[n]));
            fq::set_error(buf);
            return FQ_ERR_ARG;
        }
    if (!parallel_rows(N, [&](int32_t n0, int32_t n1) {
            dequant_rows(static_cast<const uint8_t*>(codes), wscale, n0, n1, K, ascale, fold_after, hblock, wbits,
                         W_out);
        })) {
        fq::set_error("fq_dequant_rows: host memory for the row buffers could not be allocated");
        return FQ_ERR_ARG;
    }
    return FQ_OK;
}
