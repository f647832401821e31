// api.cpp -- host side of the C ABI declared in include/fftconv.h:
// argument validation, status codes and per-thread error text, the per-device
// twiddle-table cache, K_f layout, and dispatch to the fused (N <= 16384) or
// multi-pass (larger N) kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/fftconv.h"
#include "fftconv_internal.hpp"

using namespace fftconv;

namespace {

thread_local std::string g_last_error;

fftconv_status_t fail(fftconv_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

fftconv_status_t ok() { return FFTCONV_OK; }

int log2_exact(int64_t n) {
    if (n <= 0 || (n & (n - 1)) != 0) return -1;
    int l = 0;
    while ((int64_t(1) << l) < n) ++l;
    return l;
}

bool dtype_ok(int dt) { return dt == FFTCONV_F32 || dt == FFTCONV_F16 || dt == FFTCONV_BF16; }
size_t elem_bytes(int dt) { return dt == FFTCONV_F32 ? 4 : 2; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

std::mutex g_tables_mu;
std::map<std::pair<int, int>, Tables> g_tables;

hipError_t build_tables(int logn, Tables *out) {
    const int64_t n = int64_t(1) << logn;
    std::vector<float2> tw(n), tw2(n);
    const double pi = 3.14159265358979323846264338327950288;
    for (int64_t j = 0; j < n; ++j) {
        const double a = -2.0 * pi * (double)j / (double)n;
        tw[j] = make_float2((float)std::cos(a), (float)std::sin(a));
        const double b = -pi * (double)j / (double)n;
        tw2[j] = make_float2((float)std::cos(b), (float)std::sin(b));
    }
    float2 *d = nullptr;
    hipError_t e = hipMalloc(&d, sizeof(float2) * 2 * n);
    if (e != hipSuccess) return e;
    e = hipMemcpy(d, tw.data(), sizeof(float2) * n, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(d + n, tw2.data(), sizeof(float2) * n, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return e;
    }
    out->tw = d;
    out->tw2 = d + n;
    return hipSuccess;
}

std::mutex g_mp_mu;
std::map<std::pair<int, int>, MpTables> g_mp_tables;

hipError_t upload(const std::vector<float2> &v, const float2 **out) {
    float2 *d = nullptr;
    hipError_t e = hipMalloc(&d, sizeof(float2) * v.size());
    if (e != hipSuccess) return e;
    e = hipMemcpy(d, v.data(), sizeof(float2) * v.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return e;
    }
    *out = d;
    return hipSuccess;
}

}  // namespace

namespace fftconv {

namespace {
std::mutex g_pair_mu;
std::map<int, PairTables> g_pair_tables;

// K slot 8g + j of a chained operand <-> row index within a 32-row span
int rho(int k) {
    const int g = k / 8, j = k % 8;
    return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

hipError_t upload_h(const std::vector<_Float16> &v, const void **out) {
    void *d = nullptr;
    hipError_t e = hipMalloc(&d, sizeof(_Float16) * v.size());
    if (e != hipSuccess) return e;
    e = hipMemcpy(d, v.data(), sizeof(_Float16) * v.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return e;
    }
    *out = d;
    return hipSuccess;
}
}  // namespace

hipError_t get_pair_tables(PairTables *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_pair_mu);
    auto it = g_pair_tables.find(dev);
    if (it != g_pair_tables.end()) {
        *out = it->second;
        return hipSuccess;
    }
    const double pi = 3.14159265358979323846264338327950288;
    auto ang = [&](double num, double den) { return 2.0 * pi * num / den; };
    std::vector<_Float16> f1r(4 * 64 * 8), f1i(4 * 64 * 8), f2r(2 * 64 * 8), f2i(2 * 64 * 8),
        f3r(4 * 64 * 8), f3i(4 * 64 * 8);
    std::vector<_Float16> tw1(512 * 8), tw3(512 * 8);
    for (int l = 0; l < 64; ++l) {
        const int g = l / 16, c = l % 16;
        for (int j = 0; j < 8; ++j) {
            const int r = rho(8 * g + j);
            for (int nt = 0; nt < 4; ++nt) {   // S1: F64[n_s = r][f_s = 16 nt + c] 2^-kPairS1Log2
                const double a = -ang((double)r * (16 * nt + c), 64);
                f1r[(nt * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::cos(a), -kPairS1Log2);
                f1i[(nt * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::sin(a), -kPairS1Log2);
            }
            for (int mt = 0; mt < 2; ++mt) {   // S2: F32[f_f = 16 mt + c][n_f = r] 2^-kPairS2Log2
                const double a = -ang((double)(16 * mt + c) * r, 32);
                f2r[(mt * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::cos(a), -kPairS2Log2);
                f2i[(mt * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::sin(a), -kPairS2Log2);
            }
            for (int ks = 0; ks < 2; ++ks)     // S1': conj F64[f_s = 32 ks + r][n_s = 16 nt + c] 2^-kPairS1Log2
                for (int nt = 0; nt < 2; ++nt) {
                    const double a = ang((double)(32 * ks + r) * (16 * nt + c), 64);
                    f3r[((ks * 2 + nt) * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::cos(a), -kPairS1Log2);
                    f3i[((ks * 2 + nt) * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::sin(a), -kPairS1Log2);
                }
        }
        for (int i = 0; i < 4; ++i) {
            for (int mt = 0; mt < 2; ++mt)     // rows n_f = 16 mt + 4g + i, cols f_s = 16 nt + c
                for (int nt = 0; nt < 4; ++nt) {
                    const double a = -ang((double)(16 * mt + 4 * g + i) * (16 * nt + c), 2048);
                    tw1[((mt * 4 + nt) * 64 + l) * 8 + i] = (_Float16)std::cos(a);
                    tw1[((mt * 4 + nt) * 64 + l) * 8 + 4 + i] = (_Float16)std::sin(a);
                }
            for (int nt = 0; nt < 4; ++nt)     // rows f_s = 16 nt + 4g + i, cols n_f = 16 nt2 + c
                for (int nt2 = 0; nt2 < 2; ++nt2) {
                    const double a = ang((double)(16 * nt2 + c) * (16 * nt + 4 * g + i), 2048);
                    tw3[((nt * 2 + nt2) * 64 + l) * 8 + i] = (_Float16)std::cos(a);
                    tw3[((nt * 2 + nt2) * 64 + l) * 8 + 4 + i] = (_Float16)std::sin(a);
                }
        }
    }
    PairTables t{};
    e = upload_h(f1r, &t.f1r);
    if (e == hipSuccess) e = upload_h(f1i, &t.f1i);
    if (e == hipSuccess) e = upload_h(f2r, &t.f2r);
    if (e == hipSuccess) e = upload_h(f2i, &t.f2i);
    if (e == hipSuccess) e = upload_h(f3r, &t.f3r);
    if (e == hipSuccess) e = upload_h(f3i, &t.f3i);
    if (e == hipSuccess) e = upload_h(tw1, &t.tw1);
    if (e == hipSuccess) e = upload_h(tw3, &t.tw3);
    if (e != hipSuccess) return e;
    g_pair_tables[dev] = t;
    *out = t;
    return hipSuccess;
}

namespace {
std::mutex g_pair3_mu;
std::map<int, Pair3Tables> g_pair3_tables;
}  // namespace

hipError_t get_pair3_tables(Pair3Tables *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_pair3_mu);
    auto it = g_pair3_tables.find(dev);
    if (it != g_pair3_tables.end()) {
        *out = it->second;
        return hipSuccess;
    }
    const double pi = 3.14159265358979323846264338327950288;
    const double M2 = 32768.0;
    std::vector<_Float16> fr(2 * 64 * 8), fi(2 * 64 * 8), tw1(4 * 64 * 8), tw3(4 * 64 * 8),
        two1((size_t)64 * 2 * 64 * 8), two2((size_t)32 * 4 * 64 * 8), far_(2 * 64 * 8), fai_(2 * 64 * 8),
        fbr_(2 * 64 * 8), fbi_(2 * 64 * 8), rtw((size_t)8 * 8 * 32 * 8);
    auto put8 = [](std::vector<_Float16> &v, size_t chunk, int i, double ang) {
        v[chunk * 8 + i] = (_Float16)std::cos(ang);
        v[chunk * 8 + 4 + i] = (_Float16)std::sin(ang);
    };
    for (int l = 0; l < 64; ++l) {
        const int g = l / 16, c = l % 16;
        for (int t = 0; t < 2; ++t)
            for (int j = 0; j < 8; ++j) {   // DFT-32 tile t: w32^{rho(8g+j) (16 t + c)} 2^-kDft32Log2
                const double a = -2.0 * pi * (double)rho(8 * g + j) * (16 * t + c) / 32.0;
                fr[(t * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::cos(a), -kDft32Log2);
                fi[(t * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::sin(a), -kDft32Log2);
                // row-pass tiles with f_a in the order row_fa (A: rows; B: K slots)
                const double aa = -2.0 * pi * (double)rho(8 * g + j) * row_fa(t, c) / 32.0;
                far_[(t * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::cos(aa), -kDft32Log2);
                fai_[(t * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::sin(aa), -kDft32Log2);
                const double ab = -2.0 * pi * (double)row_fa(j / 4, 4 * g + j % 4) * (16 * t + c) / 32.0;
                fbr_[(t * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::cos(ab), -kDft32Log2);
                fbi_[(t * 64 + l) * 8 + j] = (_Float16)std::ldexp(std::sin(ab), -kDft32Log2);
            }
        for (int i = 0; i < 4; ++i) {
            for (int mt = 0; mt < 2; ++mt)      // rows n_a = 16mt + 4g + i, cols f_b = 16nt + c
                for (int nt = 0; nt < 2; ++nt)
                    put8(tw1, (mt * 2 + nt) * 64 + l, i, -2.0 * pi * (double)(16 * mt + 4 * g + i) * (16 * nt + c) / 1024.0);
            for (int nt = 0; nt < 2; ++nt)      // rows f_b = 16nt + 4g + i, cols n_a = 16nt2 + c (conj)
                for (int nt2 = 0; nt2 < 2; ++nt2)
                    put8(tw3, (nt * 2 + nt2) * 64 + l, i, 2.0 * pi * (double)(16 * nt2 + c) * (16 * nt + 4 * g + i) / 1024.0);
            for (int T = 0; T < 64; ++T)        // rows f_c = 16nt + 4g + i, cols n_ab = 16(T & ~1) + 2c + (T & 1)
                for (int nt = 0; nt < 2; ++nt) {
                    const int64_t nab = 16 * (T & ~1) + 2 * c + (T & 1);
                    const double a = (double)((int64_t)(16 * nt + 4 * g + i) * nab % 32768);
                    put8(two1, ((size_t)T * 2 + nt) * 64 + l, i, -2.0 * pi * a / M2);
                }
            for (int fc = 0; fc < 32; ++fc)     // rows n_b = 16nt3 + 4g + i, cols n_a = 16nt2 + c (conj)
                for (int nt3 = 0; nt3 < 2; ++nt3)
                    for (int nt2 = 0; nt2 < 2; ++nt2) {
                        const int64_t nab = (16 * nt2 + c) + 32 * (16 * nt3 + 4 * g + i);
                        const double a = (double)((int64_t)fc * nab % 32768);
                        put8(two2, (((size_t)fc * 2 + nt3) * 2 + nt2) * 64 + l, i, 2.0 * pi * a / M2);
                    }
        }
    }
    for (int fc = 0; fc < 8; ++fc)   // row pass outer twiddle omega_8192^{f_c (n_a + 32 (4 q + k))}
        for (int q = 0; q < 8; ++q)
            for (int na = 0; na < 32; ++na)
                for (int k = 0; k < 4; ++k)
                    put8(rtw, ((size_t)fc * 8 + q) * 32 + na, k,
                         -2.0 * pi * (double)((fc * (na + 32 * (4 * q + k))) % 8192) / 8192.0);
    Pair3Tables t{};
    e = upload_h(fr, &t.fr);
    if (e == hipSuccess) e = upload_h(fi, &t.fi);
    if (e == hipSuccess) e = upload_h(tw1, &t.tw1);
    if (e == hipSuccess) e = upload_h(tw3, &t.tw3);
    if (e == hipSuccess) e = upload_h(two1, &t.two1);
    if (e == hipSuccess) e = upload_h(two2, &t.two2);
    if (e == hipSuccess) e = upload_h(far_, &t.far_);
    if (e == hipSuccess) e = upload_h(fai_, &t.fai_);
    if (e == hipSuccess) e = upload_h(fbr_, &t.fbr_);
    if (e == hipSuccess) e = upload_h(fbi_, &t.fbi_);
    if (e == hipSuccess) e = upload_h(rtw, &t.rtw);
    // outer stages for R = 4, 8, 16 (M = 1024 R): 32 / R sub-pairs share one workgroup
    for (int i = 0; i < 3 && e == hipSuccess; ++i) {
        const int logr = 2 + i, R = 1 << logr, nch = R / 2;
        const double M = 1024.0 * R, sc = std::ldexp(1.0, -p16_outer_log2(logr));
        std::vector<_Float16> o1r(2 * 64 * 8, (_Float16)0.f), o1i(2 * 64 * 8, (_Float16)0.f),
            o3r(64 * 8, (_Float16)0.f), o3i(64 * 8, (_Float16)0.f), ot1((size_t)64 * 2 * 64 * 8),
            ot2((size_t)32 * 4 * 64 * 8);
        for (int l = 0; l < 64; ++l) {
            const int g = l / 16, c = l % 16;
            for (int j = 0; j < 8; ++j) {
                // phase 1: rows rho = 16 nt + c, K slots 4 g + j (j < 4)
                for (int nt = 0; nt < 2; ++nt) {
                    const int rw = 16 * nt + c, k = 4 * g + j;
                    if (j < 4 && rw / R == k / nch) {
                        const double a = -2.0 * pi * (double)((rw % R) * (k % nch) % R) / R;
                        o1r[(nt * 64 + l) * 8 + j] = (_Float16)(sc * std::cos(a));
                        o1i[(nt * 64 + l) * 8 + j] = (_Float16)(sc * std::sin(a));
                    }
                }
                // phase 3: column c = (sub-pair c / nch, n_c = c mod nch), K slot row rho(8 g + j)
                const int rw = rho(8 * g + j);
                if (rw / R == c / nch) {
                    const double a = -2.0 * pi * (double)((rw % R) * (c % nch) % R) / R;
                    o3r[l * 8 + j] = (_Float16)(sc * std::cos(a));
                    o3i[l * 8 + j] = (_Float16)(sc * std::sin(a));
                }
            }
            for (int ii = 0; ii < 4; ++ii) {
                for (int T = 0; T < 64; ++T)        // rows rho = 16 nt + 4 g + i (f_c = rho mod R), cols n_ab
                    for (int nt = 0; nt < 2; ++nt) {
                        const int64_t nab = 16 * (T & ~1) + 2 * c + (T & 1);
                        const int64_t fcv = (16 * nt + 4 * g + ii) % R;
                        put8(ot1, ((size_t)T * 2 + nt) * 64 + l, ii, -2.0 * pi * (double)(fcv * nab % (int64_t)M) / M);
                    }
                for (int rw2 = 0; rw2 < 32; ++rw2)  // row rho (f_c = rho mod R); rows n_b = 16nt3 + 4g + i, cols n_a
                    for (int nt3 = 0; nt3 < 2; ++nt3)
                        for (int nt2 = 0; nt2 < 2; ++nt2) {
                            const int64_t nab = (16 * nt2 + c) + 32 * (16 * nt3 + 4 * g + ii);
                            const int64_t fcv = rw2 % R;
                            put8(ot2, (((size_t)rw2 * 2 + nt3) * 2 + nt2) * 64 + l, ii,
                                 2.0 * pi * (double)(fcv * nab % (int64_t)M) / M);
                        }
            }
        }
        e = upload_h(o1r, &t.o1r[i]);
        if (e == hipSuccess) e = upload_h(o1i, &t.o1i[i]);
        if (e == hipSuccess) e = upload_h(o3r, &t.o3r[i]);
        if (e == hipSuccess) e = upload_h(o3i, &t.o3i[i]);
        if (e == hipSuccess) e = upload_h(ot1, &t.ot1[i]);
        if (e == hipSuccess) e = upload_h(ot2, &t.ot2[i]);
    }
    if (e != hipSuccess) return e;
    g_pair3_tables[dev] = t;
    *out = t;
    return hipSuccess;
}

hipError_t get_mp_tables(int logn, MpTables *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_mp_mu);
    auto key = std::make_pair(dev, logn);
    auto it = g_mp_tables.find(key);
    if (it != g_mp_tables.end()) {
        *out = it->second;
        return hipSuccess;
    }
    const MpSplit sp = mp_split(logn);
    const int64_t n = int64_t(1) << logn, n1 = int64_t(1) << sp.log1;
    const double pi = 3.14159265358979323846264338327950288;
    std::vector<float2> w2row(n1), lo(2048), hi(n / 2048);
    for (int64_t j = 0; j < n1; ++j) {
        const double a = -pi * (double)j / (double)n;
        w2row[j] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
    for (int64_t j = 0; j < 2048; ++j) {
        const double a = -2.0 * pi * (double)j / (double)n;
        lo[j] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
    for (int64_t j = 0; j < n / 2048; ++j) {
        const double a = -2.0 * pi * (double)(2048 * j) / (double)n;
        hi[j] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
    MpTables t{};
    e = upload(w2row, &t.w2row);
    if (e == hipSuccess) e = upload(lo, &t.big_lo);
    if (e == hipSuccess) e = upload(hi, &t.big_hi);
    if (e == hipSuccess && sp.log1 >= kMpColMinLog1) {
        // Operand tiles of the matrix-core column passes (A operands of the complex
        // 16x16x32 products: lane l holds row l % 16, K slots 8 (l / 16) .. + 7), each tile
        // three planes (re, im, -im) of 64 lanes x 8 fp16.  Entries outside a tile's
        // rows or K range are zero.  Order: pass-1 stage 1 (RB / 16 tiles of the RB-point
        // DFT over n_b < RB/2, rows f_b), pass-1 stage 2 (one tile per f_b: the RA-point
        // DFT over n_a times omega_N1^{n_a f_b}, rows f_a), pass-3 stage 1 (the RA-point
        // DFT over f_a, rows n_a, times 2^-mp_c3_log2), pass-3 stage 2 (one tile per n_a:
        // the RB-point DFT over f_b times omega_N1^{n_a f_b}, rows n_b < RB/2).
        const int rb = 1 << mp_col_rb_log2(sp.log1), ra = (int)n1 / rb, t1 = rb / 16;
        const int ntiles = t1 + rb + 1 + ra;
        std::vector<_Float16> col((size_t)ntiles * 3 * 64 * 8, (_Float16)0.f);
        auto put = [&](int tile, int l, int j, int64_t num, int64_t den, double scale) {
            const double a = -2.0 * pi * (double)(num % den) / (double)den;
            const size_t o = ((size_t)tile * 3 * 64 + l) * 8 + j;
            col[o] = (_Float16)(scale * std::cos(a));
            col[o + 64 * 8] = (_Float16)(scale * std::sin(a));
            col[o + 2 * 64 * 8] = (_Float16)(-scale * std::sin(a));
        };
        const double s3 = std::ldexp(1.0, -mp_c3_log2(sp.log1));
        for (int l = 0; l < 64; ++l) {
            const int r = l % 16;
            for (int j = 0; j < 8; ++j) {
                const int k = 8 * (l / 16) + j;
                for (int m = 0; m < t1; ++m)        // rows f_b = 16 m + r, K = n_b
                    if (k < rb / 2) put(m, l, j, (int64_t)k * (16 * m + r), rb, 1.0);
                for (int fb = 0; fb < rb; ++fb)      // rows f_a = r, K = n_a
                    if (k < ra && r < ra) put(t1 + fb, l, j, (int64_t)k * (r * rb + fb), n1, 1.0);
                if (k < ra && r < ra) put(t1 + rb, l, j, (int64_t)k * r, ra, s3);   // rows n_a, K = f_a
                for (int na = 0; na < ra; ++na)      // rows n_b = r, K = f_b
                    if (k < rb && r < rb / 2) put(t1 + rb + 1 + na, l, j, (int64_t)k * (r * ra + na), n1, 1.0);
            }
        }
        e = upload_h(col, &t.col);
    }
    if (e != hipSuccess) return e;
    g_mp_tables[key] = t;
    *out = t;
    return hipSuccess;
}

hipError_t get_tables(int logn, Tables *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_tables_mu);
    auto key = std::make_pair(dev, logn);
    auto it = g_tables.find(key);
    if (it != g_tables.end()) {
        *out = it->second;
        return hipSuccess;
    }
    Tables t{};
    e = build_tables(logn, &t);
    if (e != hipSuccess) return e;
    g_tables[key] = t;
    *out = t;
    return hipSuccess;
}

namespace {
std::mutex g_ready_mu;
std::map<int, bool> g_ready;   // devices whose every table is built
}  // namespace

// Scratch of fftconv_fwd_noalloc (the three-pass intermediate of a chunk of
// sequences): a file-scope device array, one copy per device, held until the
// process ends.  On the host its name is only a stand-in: the device address
// is looked up per device by scratch_address() and only that address is ever
// handed to kernels.
constexpr size_t kScratchBytes = size_t(72) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::map<int, void *> g_scratch;   // device -> address of its copy of `scratch`
}  // namespace

// Looks the current device's address of `scratch` up (first call per device)
// or returns the one found before.
static hipError_t scratch_address(bool lookup, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch.find(dev);
    if (it != g_scratch.end()) {
        *out = it->second;
        return hipSuccess;
    }
    *out = nullptr;
    if (!lookup) return hipSuccess;
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
    *out = ptr;
    return hipSuccess;
}

hipError_t init_device_tables() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_ready_mu);
    if (g_ready.count(dev)) return hipSuccess;
    Tables t{};
    // twiddles of every on-chip size (2^10 .. 2^14), of every multi-pass outer
    // size (2^2 .. 2^9) and of the multi-pass row (2^13)
    for (int l = 2; l <= kFusedMaxLog && e == hipSuccess; ++l) e = get_tables(l, &t);
    MpTables m{};
    for (int l = kFusedMaxLog + 1; l <= kMaxLog && e == hipSuccess; ++l) e = get_mp_tables(l, &m);
    PairTables p{};
    if (e == hipSuccess) e = get_pair_tables(&p);
    Pair3Tables p3{};
    if (e == hipSuccess) e = get_pair3_tables(&p3);
    if (e == hipSuccess) g_ready[dev] = true;
    return e;
}

bool device_tables_ready() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lk(g_ready_mu);
    return g_ready.count(dev) != 0;
}

MpSplit mp_split(int logn) {
    // inner (on-chip) transform of 2^log2 points, outer of 2^log1 points
    MpSplit s;
    s.log2 = 13;            // on-chip rows of 8192 points (two rows of fp32 fill 128 KiB of LDS)
    s.log1 = logn - s.log2;
    return s;
}

int64_t mp_ws_bytes(int st) {
    // one complex value per point in the storage type
    return st == ST_F32 ? 8 : 4;
}

int64_t mp_chunk(int logn, int st) {
    // keep one chunk's complex intermediate near 128 MiB; from N = 2^22 on near 1 GiB (at
    // 16 MiB per sequence a 128 MiB chunk is 8 sequences, and the passes' launches then
    // lose 3-4 % of a call to their tails; at N = 2^20 the chunk size made no difference)
    const int64_t per_seq = mp_ws_bytes(st) << logn;
    const int64_t target = logn >= 22 ? int64_t(1) << 30 : int64_t(128) << 20;
    int64_t c = target / per_seq;
    return c < 1 ? 1 : c;
}

}  // namespace fftconv

// ----------------------------------------------------------------- C ABI
extern "C" {

const char *fftconv_status_string(fftconv_status_t s) {
    switch (s) {
    case FFTCONV_OK: return "ok";
    case FFTCONV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FFTCONV_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case FFTCONV_ERR_WORKSPACE: return "workspace too small";
    case FFTCONV_ERR_FILTER_MISMATCH: return "prepared filter does not match the call";
    case FFTCONV_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *fftconv_last_error(void) { return g_last_error.c_str(); }

fftconv_status_t fftconv_init(void) {
    g_last_error.clear();
    hipError_t e = init_device_tables();
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "building the constant tables: %s", hipGetErrorString(e));
    void *sp = nullptr;
    e = scratch_address(true, &sp);
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
    return ok();
}

int64_t fftconv_mask_blocks(int64_t N) {
    const int l = log2_exact(N);
    return (l >= kMinLog && l <= kMaxLog) ? kMaskBlocks : 0;
}

size_t fftconv_filter_bytes(int64_t H, int64_t N, fftconv_dtype_t dtype) {
    const int l = log2_exact(N);
    if (l < kMinLog || l > kMaxLog || H < 1 || !dtype_ok(dtype)) return 0;
    return kf_bins_off(H) + (size_t)H * (size_t)kf_slots(l, dtype) * bin_bytes(dtype);
}

size_t fftconv_workspace_bytes(int64_t B, int64_t H, int64_t N, fftconv_dtype_t dtype) {
    const int l = log2_exact(N);
    if (l < kMinLog || l > kMaxLog || B < 0 || H < 0 || !dtype_ok(dtype)) return 0;
    if (l <= kFusedMaxLog) return 0;
    int64_t S = B * H;
    const int64_t c = mp_chunk(l, dtype);
    if (S > c) S = c;
    // per sequence: the intermediate, then the fp32 rows 0 and N1/2
    return (size_t)S * ((size_t)N * (size_t)mp_ws_bytes(dtype) + kMpSelfBytes);
}

// The prepare steps; conj = true stores the conjugated spectrum (backward pass).
static fftconv_status_t prepare_impl(const void *k, int64_t H, int64_t L, int64_t N, fftconv_dtype_t dtype,
                                     void *K_f, size_t K_f_bytes, void *workspace, size_t workspace_bytes,
                                     bool conj, hipStream_t stream);

fftconv_status_t fftconv_prepare_filter(const void *k, int64_t H, int64_t L, int64_t N,
                                        fftconv_dtype_t dtype, void *K_f, size_t K_f_bytes,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    return prepare_impl(k, H, L, N, dtype, K_f, K_f_bytes, workspace, workspace_bytes, false, stream);
}

static fftconv_status_t prepare_impl(const void *k, int64_t H, int64_t L, int64_t N, fftconv_dtype_t dtype,
                                     void *K_f, size_t K_f_bytes, void *workspace, size_t workspace_bytes,
                                     bool conj, hipStream_t stream) {
    g_last_error.clear();
    const float ysgn = conj ? -1.0f : 1.0f;
    if (!dtype_ok(dtype)) return fail(FFTCONV_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    const int l = log2_exact(N);
    if (l < kMinLog || l > kMaxLog)
        return fail(FFTCONV_ERR_UNSUPPORTED, "N=%lld must be a power of two in [2^%d, 2^%d]",
                    (long long)N, kMinLog, kMaxLog);
    if (H < 1) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "H=%lld must be >= 1", (long long)H);
    if (L < 1 || L > N)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "L_filter=%lld must be in [1, N=%lld]",
                    (long long)L, (long long)N);
    if (!k || !K_f) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "k and K_f must be non-null");
    if (!aligned16(k) || !aligned16(K_f))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "k and K_f must be 16-byte aligned");
    const size_t need = fftconv_filter_bytes(H, N, dtype);
    if (K_f_bytes < need)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "K_f has %zu bytes, needs %zu", K_f_bytes, need);
    if (overlap(k, (size_t)H * (size_t)L * elem_bytes(dtype), K_f, need))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "k overlaps K_f");
    const size_t wneed = fftconv_workspace_bytes(1, H, N, dtype);
    if (wneed > 0 && (workspace == nullptr || workspace_bytes < wneed))
        return fail(FFTCONV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, wneed);
    if (wneed > 0 && !aligned16(workspace))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

    // the first prepare on a device builds every constant table of the library
    // (synchronous), so that the forward calls that follow neither allocate nor block
    hipError_t e = init_device_tables();
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "building the constant tables: %s", hipGetErrorString(e));

    char *base = static_cast<char *>(K_f);
    float *kscale = reinterpret_cast<float *>(base + kf_scale_off());
    void *kbins = base + kf_bins_off(H);
    const bool fused = l <= kFusedMaxLog;
    const MpSplit sp = mp_split(l);
    KfHeader hdr{};
    hdr.magic = kKfMagic;
    hdr.version = kKfVersion;
    hdr.N = N;
    hdr.H = H;
    hdr.L = L;
    hdr.dtype = (int32_t)dtype;
    hdr.layout = !fused ? KF_ROWS
                        : (use_pair_kernel(l, dtype) ? KF_PAIR : (use_pair3_kernel(l, dtype) ? KF_PAIR3 : KF_NATURAL));
    hdr.scale_off = (int64_t)kf_scale_off();
    hdr.bins_off = (int64_t)kf_bins_off(H);
    hdr.n1 = fused ? 0 : (int64_t(1) << sp.log1);
    hdr.n2 = fused ? N : (int64_t(1) << sp.log2);

    e = launch_write_header(hdr, K_f, stream);
    if (e == hipSuccess)
        e = launch_filter_scale(dtype, k, H, L, kf_norm_log2(l, dtype), kf_target_log2(l, dtype), kscale,
                                stream);
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "filter setup launch: %s", hipGetErrorString(e));
    if (fused && use_pair3_kernel(l, dtype) && !conj) {
        // N = 2048 .. 16384, half precision: the transform of the N = 16384 kernels
        e = launch_pair16k_prepare(l, dtype, k, L, kbins, kscale, H, stream);
    } else if (fused) {
        Tables tb{};
        e = get_tables(l, &tb);
        if (e == hipSuccess) e = launch_fused_prepare(l, dtype, k, L, kbins, kscale, tb, H, ysgn, stream);
    } else {
        const int64_t c = mp_chunk(l, dtype);
        for (int64_t h0 = 0; h0 < H && e == hipSuccess; h0 += c) {
            const int64_t n = H - h0 < c ? H - h0 : c;
            e = launch_multipass_prepare(l, dtype, k, L, kbins, kscale, workspace, H, h0, n, ysgn, stream);
        }
    }
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "prepare launch: %s", hipGetErrorString(e));
    return ok();
}

// The forward call's argument checks; FFTCONV_OK with an empty g_last_error when the call
// has work to enqueue, FFTCONV_OK with `*empty` set when B * H = 0.
static fftconv_status_t fwd_args(const void *u, const void *K_f, const void *w, const void *v, void *out,
                                 int64_t B, int64_t H, int64_t N, int64_t L, const uint8_t *mask,
                                 fftconv_dtype_t dtype, void *workspace, size_t workspace_bytes, bool *empty,
                                 bool check_workspace = true) {
    *empty = false;
    if (!dtype_ok(dtype)) return fail(FFTCONV_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    const int l = log2_exact(N);
    if (l < kMinLog || l > kMaxLog)
        return fail(FFTCONV_ERR_UNSUPPORTED, "N=%lld must be a power of two in [2^%d, 2^%d]",
                    (long long)N, kMinLog, kMaxLog);
    if (B < 0 || H < 0)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "B=%lld and H=%lld must be >= 0", (long long)B,
                    (long long)H);
    if (L < 1 || L > N)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "L_filter=%lld must be in [1, N=%lld]",
                    (long long)L, (long long)N);
    if (B * H == 0) {
        *empty = true;
        return ok();
    }
    if (!u || !K_f || !out) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "u, K_f and out must be non-null");
    if (!aligned16(u) || !aligned16(K_f) || !aligned16(out) || (w && !aligned16(w)) ||
        (v && !aligned16(v)) || (mask && !aligned16(mask)))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
    const size_t nbytes = (size_t)B * (size_t)H * (size_t)N * elem_bytes(dtype);
    const size_t kfb = fftconv_filter_bytes(H, N, dtype);
    if (overlap(out, nbytes, u, nbytes) || overlap(out, nbytes, w, nbytes) ||
        overlap(out, nbytes, v, nbytes) || overlap(out, nbytes, K_f, kfb) ||
        overlap(out, nbytes, mask, (size_t)H * kMaskBlocks))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "out overlaps an input");
    if (!check_workspace) return FFTCONV_OK;
    const size_t wneed = fftconv_workspace_bytes(B, H, N, dtype);
    if (wneed > 0 && (workspace == nullptr || workspace_bytes < wneed))
        return fail(FFTCONV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, wneed);
    if (wneed > 0 && !aligned16(workspace))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (wneed > 0 && (overlap(workspace, wneed, out, nbytes) || overlap(workspace, wneed, u, nbytes)))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "workspace overlaps a tensor");
    return FFTCONV_OK;
}

// The forward call's launches, after fwd_args accepted the arguments.  The
// three-pass path runs `chunk` sequences at a time through the workspace,
// which holds chunk * (N complex values + the two self-paired rows).
static fftconv_status_t fwd_enqueue(const void *u, const void *K_f, const void *w, const void *v, void *out,
                                    int64_t B, int64_t H, int64_t N, int64_t L, const uint8_t *mask,
                                    fftconv_dtype_t dtype, void *workspace, int64_t chunk, hipStream_t stream) {
    const int l = log2_exact(N);
    const char *chk = std::getenv("FFTCONV_CHECK");
    if (chk && chk[0] == '1') {
        KfHeader hdr{};
        hipError_t e = hipMemcpyAsync(&hdr, K_f, sizeof hdr, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "reading the K_f header: %s", hipGetErrorString(e));
        if (hdr.magic != kKfMagic || hdr.version != kKfVersion || hdr.N != N || hdr.H != H ||
            hdr.L != L || hdr.dtype != (int32_t)dtype)
            return fail(FFTCONV_ERR_FILTER_MISMATCH,
                        "K_f header (N=%lld H=%lld L=%lld dtype=%d) does not match the call "
                        "(N=%lld H=%lld L=%lld dtype=%d)",
                        (long long)hdr.N, (long long)hdr.H, (long long)hdr.L, hdr.dtype,
                        (long long)N, (long long)H, (long long)L, (int)dtype);
    }

    const char *base = static_cast<const char *>(K_f);
    const float *kscale = reinterpret_cast<const float *>(base + kf_scale_off());
    const void *kbins = base + kf_bins_off(H);
    hipError_t e = hipSuccess;
    if (use_pair_kernel(l, dtype)) {
        e = launch_pair_conv(l, dtype, u, w, v, out, kbins, kscale, mask, B, H, stream);
    } else if (use_pair3_kernel(l, dtype)) {
        e = launch_pair16k_conv(l, dtype, u, w, v, out, kbins, kscale, mask, B, H, stream);
    } else if (l <= kFusedMaxLog) {
        Tables tb{};
        e = get_tables(l, &tb);
        if (e == hipSuccess)
            e = launch_fused_conv(l, dtype, u, w, v, out, kbins, kscale, mask, tb, B, H, stream);
    } else {
        const int64_t S = B * H;
        for (int64_t s0 = 0; s0 < S && e == hipSuccess; s0 += chunk) {
            const int64_t n = S - s0 < chunk ? S - s0 : chunk;
            e = launch_multipass_conv(l, dtype, u, w, v, out, kbins, kscale, mask, workspace, H,
                                      s0, n, stream);
        }
    }
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "fwd launch: %s", hipGetErrorString(e));
    return ok();
}

fftconv_status_t fftconv_fwd(const void *u, const void *K_f, const void *w, const void *v,
                             void *out, int64_t B, int64_t H, int64_t N, int64_t L,
                             const uint8_t *mask, fftconv_dtype_t dtype, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    bool empty = false;
    const fftconv_status_t chk_st =
        fwd_args(u, K_f, w, v, out, B, H, N, L, mask, dtype, workspace, workspace_bytes, &empty);
    if (chk_st != FFTCONV_OK || empty) return chk_st;
    const int l = log2_exact(N);
    return fwd_enqueue(u, K_f, w, v, out, B, H, N, L, mask, dtype, workspace,
                       l > kFusedMaxLog ? mp_chunk(l, dtype) : 0, stream);
}

size_t fftconv_fwd_noalloc_scratch_bytes(void) { return kScratchBytes; }

fftconv_status_t fftconv_fwd_noalloc(const void *u, const void *K_f, const void *w, const void *v, void *out,
                                     int64_t B, int64_t H, int64_t N, int64_t L, const uint8_t *mask,
                                     fftconv_dtype_t dtype, hipStream_t stream) {
    g_last_error.clear();
    bool empty = false;
    const fftconv_status_t chk_st =
        fwd_args(u, K_f, w, v, out, B, H, N, L, mask, dtype, nullptr, 0, &empty, false);
    if (chk_st != FFTCONV_OK || empty) return chk_st;
    void *sp = nullptr;
    hipError_t e = scratch_address(false, &sp);
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
    if (sp == nullptr || !device_tables_ready())
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "fftconv_init() has not run on this device");
    const int l = log2_exact(N);
    int64_t chunk = 0;
    if (l > kFusedMaxLog) {
        // as many sequences per chunk as the scratch holds (at most the usual chunk)
        const size_t per_seq = ((size_t)N * (size_t)mp_ws_bytes(dtype) + kMpSelfBytes);
        if (per_seq > kScratchBytes)
            return fail(FFTCONV_ERR_UNSUPPORTED, "one sequence of N=%lld needs %zu scratch bytes, the maximum is %zu",
                        (long long)N, per_seq, kScratchBytes);
        chunk = (int64_t)(kScratchBytes / per_seq);
        const int64_t usual = mp_chunk(l, dtype);
        if (chunk > usual) chunk = usual;
        if (overlap(sp, kScratchBytes, out, (size_t)B * H * N * elem_bytes(dtype)))
            return fail(FFTCONV_ERR_INVALID_ARGUMENT, "out overlaps the library's scratch");
    }
    return fwd_enqueue(u, K_f, w, v, out, B, H, N, L, mask, dtype, sp, chunk, stream);
}

// ---- backward pass ---------------------------------------------------------
// Workspace regions, each 256-byte aligned: the conjugated spectrum of K_f;
// x = u w; the spectra of the sequences x as filters of their own channel;
// the per-sequence correlations; the repeated mask rows; the forward
// workspace (the same size serves the B*H-channel prepare and forward).
// N = 2048 .. 16384 (fp16 / bf16) instead: the batch-row pairs' spectra of u w
// and their scales (per group of channels sharing a workgroup), and the per-pair
// correlations.
struct BwdLayout {
    size_t kc, x, kx, part, mrep, fws, spec, pscale, total;
};

static BwdLayout bwd_layout(int64_t B, int64_t H, int64_t N, fftconv_dtype_t dtype) {
    BwdLayout o{};
    const int64_t S = B * H;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    o.kc = take(fftconv_filter_bytes(H, N, dtype));
    // (kc: the conjugated spectrum, used when only one of du, dw is asked for or outside the
    // matrix-core sizes; the two-output call conjugates the bins as it reads them)
    // N = 1024 (fp16 / bf16): du, dw and dk come from kernels that need no other scratch
    // (the dk chain's areas below are then empty)
    // N = 2048 .. 16384 (fp16 / bf16): per-group spectra of the batch-row pairs of u*w
    // (a group is the 2^(14 - log2 N) channels of one workgroup) and one partial row per pair
    const int l = log2_exact(N);
    const bool p16 = use_pair3_kernel(l, dtype);
    const bool chain = !use_pair_kernel(l, dtype) && !p16;
    const int64_t PB = (B + 1) / 2, Pch = p16 ? (int64_t)1 << (14 - l) : 1;
    const int64_t groups = (H + Pch - 1) / Pch * PB;
    o.spec = take(p16 ? (size_t)groups * kP16SpecBytes : 0);
    o.pscale = take(p16 ? (size_t)(groups * Pch) * sizeof(float) : 0);   // one per pair of rows
    o.part = take(p16 ? (size_t)(PB * H) * (size_t)N * elem_bytes(dtype) : 0);
    o.x = take(chain ? (size_t)S * (size_t)N * elem_bytes(dtype) : 0);
    o.kx = take(chain && S > 0 ? fftconv_filter_bytes(S, N, dtype) : 0);
    if (chain) o.part = take((size_t)S * (size_t)N * elem_bytes(dtype));
    o.mrep = take(chain ? (size_t)S * kMaskBlocks : 0);
    o.fws = take(chain ? fftconv_workspace_bytes(1, S, N, dtype) : fftconv_workspace_bytes(B, H, N, dtype));
    o.total = off;
    return o;
}

size_t fftconv_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, fftconv_dtype_t dtype) {
    const int l = log2_exact(N);
    if (l < kMinLog || l > kMaxLog || B < 0 || H < 1 || !dtype_ok(dtype)) return 0;
    return bwd_layout(B, H, N, dtype).total;
}

// Conjugate every stored bin of a prepared spectrum of H channels (src may be dst).
static hipError_t conj_spectrum(const void *src, void *dst, int64_t H, int64_t N, fftconv_dtype_t dtype,
                                hipStream_t stream) {
    const int l = log2_exact(N);
    const size_t boff = kf_bins_off(H);
    hipError_t e = hipSuccess;
    if (src != dst) e = hipMemcpyAsync(dst, src, boff, hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return e;
    const bool pair = l <= kFusedMaxLog && (use_pair_kernel(l, dtype) || use_pair3_kernel(l, dtype));
    const int kind = pair ? 0 : (dtype == FFTCONV_F32 ? 2 : 1);
    const int64_t per_channel = kf_slots(l, dtype) * (int64_t)bin_bytes(dtype);
    return launch_conj_bins(static_cast<const char *>(src) + boff, static_cast<char *>(dst) + boff, H,
                            per_channel, kind, stream);
}

fftconv_status_t fftconv_bwd(const void *dy, const void *u, const void *K_f, const void *w, const void *v,
                             void *du, void *dk, void *dw, void *dv, int64_t B, int64_t H, int64_t N,
                             int64_t L, const uint8_t *mask, fftconv_dtype_t dtype, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    if (!dtype_ok(dtype)) return fail(FFTCONV_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    const int l = log2_exact(N);
    if (l < kMinLog || l > kMaxLog)
        return fail(FFTCONV_ERR_UNSUPPORTED, "N=%lld must be a power of two in [2^%d, 2^%d]",
                    (long long)N, kMinLog, kMaxLog);
    if (B < 0 || H < 0)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "B=%lld and H=%lld must be >= 0", (long long)B,
                    (long long)H);
    if (L < 1 || L > N)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "L_filter=%lld must be in [1, N=%lld]",
                    (long long)L, (long long)N);
    if (H == 0) return ok();
    if (dw && !w) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "dw needs the input gate w");
    if (dv && !v) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "dv needs the output gate v");
    if (!K_f || (B > 0 && (!dy || !u)))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "dy, u and K_f must be non-null");
    const void *ptrs[] = {dy, u, K_f, w, v, du, dk, dw, dv, mask};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    const size_t nbytes = (size_t)B * (size_t)H * (size_t)N * elem_bytes(dtype);
    const size_t kbytes = (size_t)H * (size_t)L * elem_bytes(dtype);
    const void *ins[] = {dy, u, w, v};
    for (const void *o : {(const void *)du, (const void *)dw, (const void *)dv})
        for (const void *i : ins)
            if (o && i && overlap(o, nbytes, i, nbytes))
                return fail(FFTCONV_ERR_INVALID_ARGUMENT, "a gradient overlaps an input");
    if (dk)
        for (const void *i : ins)
            if (i && overlap(dk, kbytes, i, nbytes))
                return fail(FFTCONV_ERR_INVALID_ARGUMENT, "dk overlaps an input");
    const BwdLayout lay = bwd_layout(B, H, N, dtype);
    if (!workspace || workspace_bytes < lay.total)
        return fail(FFTCONV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, lay.total);
    if (!aligned16(workspace)) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

    char *ws = static_cast<char *>(workspace);
    void *fws = ws + lay.fws;
    const size_t fws_bytes = lay.total - lay.fws;
    fftconv_status_t st = FFTCONV_OK;
    // N = 2048 .. 16384 (fp16 / bf16) with dk: the dk chain below; at N = 16384 its first
    // pass also forms dv from the same transforms of u w
    const bool p16dk = dk && B > 0 && use_pair3_kernel(l, dtype);
    const bool dv_in_dk = p16dk && dv && l == 14;
    // dv = dy * conv(u w, k): the forward pass with dy as the output gate
    if (dv && B > 0 && !dv_in_dk) {
        st = fftconv_fwd(u, K_f, w, dy, dv, B, H, N, L, mask, dtype, fws, fws_bytes, stream);
        if (st != FFTCONV_OK) return st;
    }
    // du = w * corr(v dy, k), dw = u * corr(v dy, k): the product with conj K
    if ((du || dw) && B > 0) {
        hipError_t e = hipSuccess;
        if (du && dw && (use_pair_kernel(l, dtype) || use_pair3_kernel(l, dtype))) {
            // N = 1024 .. 16384 (fp16 / bf16): one call forms both from the same transforms,
            // conjugating the stored spectrum as it reads it
            const char *kb = static_cast<const char *>(K_f);
            const float *ksc = reinterpret_cast<const float *>(kb + kf_scale_off());
            e = use_pair_kernel(l, dtype)
                    ? launch_pair_conv(l, dtype, dy, v, w, du, kb + kf_bins_off(H), ksc, mask, B, H, stream, u, dw)
                    : launch_pair16k_conv(l, dtype, dy, v, w, du, kb + kf_bins_off(H), ksc, mask, B, H, stream, u, dw);
            if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "du, dw: %s", hipGetErrorString(e));
        } else {
            // otherwise the forward call on a conjugated copy of the spectrum
            e = conj_spectrum(K_f, ws + lay.kc, H, N, dtype, stream);
            if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "conjugating K_f: %s", hipGetErrorString(e));
            if (du) {
                st = fftconv_fwd(dy, ws + lay.kc, v, w, du, B, H, N, L, mask, dtype, fws, fws_bytes, stream);
                if (st != FFTCONV_OK) return st;
            }
            if (dw) {
                st = fftconv_fwd(dy, ws + lay.kc, v, u, dw, B, H, N, L, mask, dtype, fws, fws_bytes, stream);
                if (st != FFTCONV_OK) return st;
            }
        }
    }
    // dk[h, s] = sum_b corr(v dy, u w)[b, h, s].  N = 1024 (fp16 / bf16): one kernel
    // accumulates the pairs' spectrum products per channel on chip.
    if (dk && B > 0 && use_pair_kernel(l, dtype)) {
        hipError_t e = launch_pair_dk(dtype, dy, u, w, v, dk, mask, B, H, L, stream);
        if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "dk: %s", hipGetErrorString(e));
    } else if (p16dk) {
        // N = 2048 .. 16384 (fp16 / bf16): the pairs' spectra of u w (at N = 16384 with dv
        // from the same transforms), then one correlation per pair
        const char *kb = static_cast<const char *>(K_f);
        hipError_t e = launch_pair16k_dk(l, dtype, dy, u, w, v, ws + lay.part, ws + lay.spec,
                                         reinterpret_cast<float *>(ws + lay.pscale), mask, B, H, stream,
                                         dv_in_dk ? dv : nullptr,
                                         kb + kf_bins_off(H), reinterpret_cast<const float *>(kb + kf_scale_off()));
        if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "dk pairs: %s", hipGetErrorString(e));
        e = launch_dk_reduce(dtype, ws + lay.part, dk, (B + 1) / 2, H, N, L, stream);
        if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "dk reduction: %s", hipGetErrorString(e));
    } else if (dk) {
        // otherwise each x = u w is the filter of its own channel b H + h; the mask rows
        // repeat per batch row
        const int64_t S = B * H;
        hipError_t e = hipSuccess;
        if (S > 0) {
            const void *x = u;
            if (w) {
                e = launch_gate_product(dtype, u, w, ws + lay.x, S * N, stream);
                if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "gate product: %s", hipGetErrorString(e));
                x = ws + lay.x;
            }
            // the sequences' spectra, stored conjugated
            st = prepare_impl(x, S, N, N, dtype, ws + lay.kx, fftconv_filter_bytes(S, N, dtype), fws, fws_bytes,
                              true, stream);
            if (st != FFTCONV_OK) return st;
            const uint8_t *mrep = nullptr;
            if (mask) {
                e = launch_mask_repeat(mask, reinterpret_cast<uint8_t *>(ws + lay.mrep), H, S, stream);
                if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "mask rows: %s", hipGetErrorString(e));
                mrep = reinterpret_cast<const uint8_t *>(ws + lay.mrep);
            }
            st = fftconv_fwd(dy, ws + lay.kx, v, nullptr, ws + lay.part, 1, S, N, N, mrep, dtype, fws, fws_bytes,
                             stream);
            if (st != FFTCONV_OK) return st;
        }
        e = launch_dk_reduce(dtype, ws + lay.part, dk, B, H, N, L, stream);
        if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "dk reduction: %s", hipGetErrorString(e));
    }
    g_last_error.clear();
    return ok();
}

// ---- forward from time-domain taps ------------------------------------------
// The spectrum is prepared into the head of the workspace on the call's stream, then
// the forward call reads it; the remaining workspace serves both as scratch (they run
// one after the other on the stream).
static size_t round_up256(size_t n) { return (n + 255) & ~size_t(255); }

size_t fftconv_fwd_taps_workspace_bytes(int64_t B, int64_t H, int64_t N, fftconv_dtype_t dtype) {
    const size_t kf = fftconv_filter_bytes(H, N, dtype);
    if (kf == 0 || B < 0) return 0;
    const size_t a = fftconv_workspace_bytes(1, H, N, dtype), b = fftconv_workspace_bytes(B, H, N, dtype);
    return round_up256(kf) + (a > b ? a : b);
}

fftconv_status_t fftconv_fwd_taps(const void *u, const void *k, const void *w, const void *v, void *out,
                                  int64_t B, int64_t H, int64_t N, int64_t L, const uint8_t *mask,
                                  fftconv_dtype_t dtype, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    g_last_error.clear();
    if (!dtype_ok(dtype)) return fail(FFTCONV_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    const int l = log2_exact(N);
    if (l < kMinLog || l > kMaxLog)
        return fail(FFTCONV_ERR_UNSUPPORTED, "N=%lld must be a power of two in [2^%d, 2^%d]",
                    (long long)N, kMinLog, kMaxLog);
    if (B < 0 || H < 0)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "B=%lld and H=%lld must be >= 0", (long long)B,
                    (long long)H);
    if (L < 1 || L > N)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "L_filter=%lld must be in [1, N=%lld]",
                    (long long)L, (long long)N);
    if (B * H == 0) return ok();
    if (!k) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "k must be non-null");
    const size_t need = fftconv_fwd_taps_workspace_bytes(B, H, N, dtype);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(FFTCONV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (!aligned16(workspace) || !aligned16(k))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "k and workspace must be 16-byte aligned");
    const size_t nbytes = (size_t)B * (size_t)H * (size_t)N * elem_bytes(dtype);
    const size_t kbytes = (size_t)H * (size_t)L * elem_bytes(dtype);
    if (overlap(workspace, need, k, kbytes) || overlap(workspace, need, u, nbytes) ||
        overlap(workspace, need, w, nbytes) || overlap(workspace, need, v, nbytes) ||
        overlap(workspace, need, out, nbytes) || overlap(workspace, need, mask, (size_t)H * kMaskBlocks))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "workspace overlaps an argument");
    if (overlap(out, nbytes, k, kbytes)) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "out overlaps k");
    char *ws = static_cast<char *>(workspace);
    const size_t kf = round_up256(fftconv_filter_bytes(H, N, dtype));
    bool empty = false;
    fftconv_status_t chk_st =
        fwd_args(u, ws, w, v, out, B, H, N, L, mask, dtype, ws + kf, workspace_bytes - kf, &empty);
    if (chk_st != FFTCONV_OK) return chk_st;
    const fftconv_status_t st =
        prepare_impl(k, H, L, N, dtype, ws, kf, ws + kf, workspace_bytes - kf, false, stream);
    if (st != FFTCONV_OK) return st;
    return fftconv_fwd(u, ws, w, v, out, B, H, N, L, mask, dtype, ws + kf, workspace_bytes - kf, stream);
}

// ---- chunked short-filter path ---------------------------------------------
// The short path covers a sequence with windows of 2 kShortBlock samples at a hop of
// kShortBlock (the transform of the N = kShortBlock kernels, 2048 points); a filter of at
// most kShortBlock taps leaves the window's second half free of wrap-around.
constexpr int64_t kShortBlock = 1024;

size_t fftconv_short_filter_bytes(int64_t H, fftconv_dtype_t dtype) {
    if (dtype != FFTCONV_F16 && dtype != FFTCONV_BF16) return 0;
    return fftconv_filter_bytes(H, kShortBlock, dtype);
}

fftconv_status_t fftconv_prepare_short_filter(const void *k, int64_t H, int64_t L, fftconv_dtype_t dtype,
                                              void *K_s, size_t K_s_bytes, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != FFTCONV_F16 && dtype != FFTCONV_BF16)
        return fail(FFTCONV_ERR_UNSUPPORTED, "the short-filter path needs fp16 or bf16 storage");
    if (L < 1 || L > kShortBlock)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "L_filter=%lld must be in [1, %lld]", (long long)L,
                    (long long)(kShortBlock));
    // the spectrum of the filter zero-padded to the window (2048 points)
    return prepare_impl(k, H, L, kShortBlock, dtype, K_s, K_s_bytes, nullptr, 0, false, stream);
}

fftconv_status_t fftconv_fwd_short(const void *u, const void *K_s, const void *w, const void *v, void *out,
                                   int64_t B, int64_t H, int64_t N, int64_t L, fftconv_dtype_t dtype,
                                   hipStream_t stream) {
    g_last_error.clear();
    if (dtype != FFTCONV_F16 && dtype != FFTCONV_BF16)
        return fail(FFTCONV_ERR_UNSUPPORTED, "the short-filter path needs fp16 or bf16 storage");
    if (N < kShortBlock || N % kShortBlock != 0)
        return fail(FFTCONV_ERR_UNSUPPORTED, "N=%lld must be a positive multiple of %lld", (long long)N,
                    (long long)kShortBlock);
    if (B < 0 || H < 0) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "B and H must be >= 0");
    if (L < 1 || L > kShortBlock)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "L_filter=%lld must be in [1, %lld]", (long long)L,
                    (long long)(kShortBlock));
    if (B * H == 0) return ok();
    if (!u || !K_s || !out) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "u, K_s and out must be non-null");
    if (!aligned16(u) || !aligned16(K_s) || !aligned16(out) || (w && !aligned16(w)) || (v && !aligned16(v)))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
    const size_t nbytes = (size_t)B * (size_t)H * (size_t)N * elem_bytes(dtype);
    if (overlap(out, nbytes, u, nbytes) || overlap(out, nbytes, w, nbytes) || overlap(out, nbytes, v, nbytes) ||
        overlap(out, nbytes, K_s, fftconv_short_filter_bytes(H, dtype)))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "out overlaps an input");
    const char *base = static_cast<const char *>(K_s);
    const float *kscale = reinterpret_cast<const float *>(base + kf_scale_off());
    const void *kbins = base + kf_bins_off(H);
    const hipError_t e = launch_pair_conv_win(dtype, u, w, v, out, kbins, kscale, B, H, N, stream);
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "fwd_short launch: %s", hipGetErrorString(e));
    return ok();
}

fftconv_status_t fftconv_bwd_short(const void *dy, const void *u, const void *K_s, const void *w, const void *v,
                                   void *du, void *dk, void *dw, void *dv, int64_t B, int64_t H, int64_t N,
                                   int64_t L, fftconv_dtype_t dtype, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != FFTCONV_F16 && dtype != FFTCONV_BF16)
        return fail(FFTCONV_ERR_UNSUPPORTED, "the short-filter path needs fp16 or bf16 storage");
    if (N < kShortBlock || N % kShortBlock != 0)
        return fail(FFTCONV_ERR_UNSUPPORTED, "N=%lld must be a positive multiple of %lld", (long long)N,
                    (long long)kShortBlock);
    if (B < 0 || H < 0) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "B and H must be >= 0");
    if (L < 1 || L > kShortBlock)
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "L_filter=%lld must be in [1, %lld]", (long long)L,
                    (long long)(kShortBlock));
    if (H == 0) return ok();
    if (dw && !w) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "dw needs the input gate w");
    if (dv && !v) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "dv needs the output gate v");
    if (!K_s || (B > 0 && (!dy || !u)))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "dy, u and K_s must be non-null");
    const void *ptrs[] = {dy, u, K_s, w, v, du, dk, dw, dv};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    const size_t nbytes = (size_t)B * (size_t)H * (size_t)N * elem_bytes(dtype);
    const size_t kbytes = (size_t)H * (size_t)L * elem_bytes(dtype);
    const size_t ksb = fftconv_short_filter_bytes(H, dtype);
    const void *ins[] = {dy, u, w, v};
    for (const void *o : {(const void *)du, (const void *)dw, (const void *)dv}) {
        if (!o) continue;
        for (const void *i : ins)
            if (i && overlap(o, nbytes, i, nbytes))
                return fail(FFTCONV_ERR_INVALID_ARGUMENT, "a gradient overlaps an input");
        if (overlap(o, nbytes, K_s, ksb)) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "a gradient overlaps K_s");
    }
    if (dk) {
        for (const void *i : ins)
            if (i && overlap(dk, kbytes, i, nbytes))
                return fail(FFTCONV_ERR_INVALID_ARGUMENT, "dk overlaps an input");
        if (overlap(dk, kbytes, K_s, ksb)) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "dk overlaps K_s");
    }
    const char *base = static_cast<const char *>(K_s);
    const float *kscale = reinterpret_cast<const float *>(base + kf_scale_off());
    const void *kbins = base + kf_bins_off(H);
    hipError_t e = hipSuccess;
    if (B > 0) {
        // dv = dy * conv(u w, k): the windowed forward kernel with dy as the output gate
        if (dv) {
            e = launch_pair_conv_win(dtype, u, w, dy, dv, kbins, kscale, B, H, N, stream);
            if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "dv: %s", hipGetErrorString(e));
        }
        // du = w * corr(v dy, k), dw = u * corr(v dy, k): the correlation kernel, both from
        // one call when both are asked for
        if (du && dw) {
            e = launch_pair_conv_win(dtype, dy, v, w, du, kbins, kscale, B, H, N, stream, true, u, dw);
        } else if (du) {
            e = launch_pair_conv_win(dtype, dy, v, w, du, kbins, kscale, B, H, N, stream, true);
        } else if (dw) {
            e = launch_pair_conv_win(dtype, dy, v, u, dw, kbins, kscale, B, H, N, stream, true);
        }
        if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "du, dw: %s", hipGetErrorString(e));
    }
    if (dk) {
        e = B > 0 ? launch_pair_dk(dtype, dy, u, w, v, dk, nullptr, B, H, L, stream, N)
                  : launch_dk_reduce(dtype, nullptr, dk, 0, H, N, L, stream);   // (no rows: zeros)
        if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "dk: %s", hipGetErrorString(e));
    }
    return ok();
}

// ---- group-axis circular convolution ----------------------------------------
static bool eq_group_ok(int64_t T) { return T == 4 || T == 8 || T == 16; }

size_t fftconv_eqlinear_weight_bytes(int64_t T, int64_t C_out, int64_t C_in, fftconv_dtype_t dtype) {
    if (!eq_group_ok(T) || C_out < 1 || C_in < 1 || !dtype_ok(dtype)) return 0;
    // (T/2 + 1) complex matrices: fp32 for fp32 storage, fp16 otherwise
    return (size_t)(T / 2 + 1) * 2 * (size_t)C_out * (size_t)C_in * (dtype == FFTCONV_F32 ? 4 : 2);
}

fftconv_status_t fftconv_eqlinear_prepare(const void *W, int64_t T, int64_t C_out, int64_t C_in,
                                          fftconv_dtype_t dtype, void *W_f, size_t W_f_bytes,
                                          hipStream_t stream) {
    g_last_error.clear();
    if (!dtype_ok(dtype)) return fail(FFTCONV_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    if (!eq_group_ok(T)) return fail(FFTCONV_ERR_UNSUPPORTED, "group order T=%lld must be 4, 8 or 16", (long long)T);
    if (C_in < 32 || C_in % 32 != 0 || C_out < 32 || C_out % 32 != 0)
        return fail(FFTCONV_ERR_UNSUPPORTED, "C_in=%lld and C_out=%lld must be positive multiples of 32",
                    (long long)C_in, (long long)C_out);
    if (!W || !W_f) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "W and W_f must be non-null");
    if (!aligned16(W) || !aligned16(W_f))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "W and W_f must be 16-byte aligned");
    const size_t need = fftconv_eqlinear_weight_bytes(T, C_out, C_in, dtype);
    if (W_f_bytes < need) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "W_f has %zu bytes, needs %zu", W_f_bytes, need);
    if (overlap(W, (size_t)T * C_out * C_in * elem_bytes(dtype), W_f, need))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "W overlaps W_f");
    const hipError_t e = launch_eqlinear_prepare(dtype, (int)T, W, W_f, C_out, C_in, stream);
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "eqlinear prepare launch: %s", hipGetErrorString(e));
    return ok();
}

fftconv_status_t fftconv_eqlinear_fwd(const void *x, const void *W_f, void *y, int64_t N, int64_t T,
                                      int64_t C_in, int64_t C_out, fftconv_dtype_t dtype, hipStream_t stream) {
    g_last_error.clear();
    if (!dtype_ok(dtype)) return fail(FFTCONV_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    if (!eq_group_ok(T)) return fail(FFTCONV_ERR_UNSUPPORTED, "group order T=%lld must be 4, 8 or 16", (long long)T);
    if (C_in < 32 || C_in % 32 != 0 || C_out < 32 || C_out % 32 != 0)
        return fail(FFTCONV_ERR_UNSUPPORTED, "C_in=%lld and C_out=%lld must be positive multiples of 32",
                    (long long)C_in, (long long)C_out);
    if (N < 0) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "N must be >= 0");
    if (N == 0) return ok();
    if (!x || !W_f || !y) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "x, W_f and y must be non-null");
    if (!aligned16(x) || !aligned16(W_f) || !aligned16(y))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
    const size_t ybytes = (size_t)N * T * C_out * elem_bytes(dtype);
    if (overlap(y, ybytes, x, (size_t)N * T * C_in * elem_bytes(dtype)) ||
        overlap(y, ybytes, W_f, fftconv_eqlinear_weight_bytes(T, C_out, C_in, dtype)))
        return fail(FFTCONV_ERR_INVALID_ARGUMENT, "y overlaps an input");
    const hipError_t e = launch_eqlinear(dtype, (int)T, x, W_f, y, N, C_in, C_out, stream);
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "eqlinear launch: %s", hipGetErrorString(e));
    return ok();
}

fftconv_status_t fftconv_export_filter_rfft(const void *K_f, int64_t H, int64_t N,
                                            fftconv_dtype_t dtype, double *host_out,
                                            hipStream_t stream) {
    g_last_error.clear();
    if (!dtype_ok(dtype)) return fail(FFTCONV_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    const int l = log2_exact(N);
    if (l < kMinLog || l > kMaxLog) return fail(FFTCONV_ERR_UNSUPPORTED, "unsupported N=%lld", (long long)N);
    if (H < 1 || !K_f || !host_out) return fail(FFTCONV_ERR_INVALID_ARGUMENT, "bad arguments");
    const size_t bytes = fftconv_filter_bytes(H, N, dtype);
    std::vector<unsigned char> hbuf(bytes);
    hipError_t e = hipMemcpyAsync(hbuf.data(), K_f, bytes, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(FFTCONV_ERR_HIP, "copy: %s", hipGetErrorString(e));
    KfHeader hdr;
    std::memcpy(&hdr, hbuf.data(), sizeof hdr);
    if (hdr.magic != kKfMagic || hdr.N != N || hdr.H != H || hdr.dtype != (int32_t)dtype)
        return fail(FFTCONV_ERR_FILTER_MISMATCH, "K_f header does not match");
    const float *kscale = reinterpret_cast<const float *>(hbuf.data() + hdr.scale_off);
    const unsigned char *bins = hbuf.data() + hdr.bins_off;
    const int64_t n1 = hdr.n1, n2 = hdr.n2;
    for (int64_t h = 0; h < H; ++h) {
        // stored = K * s_h with s_h = 1 / (scale * norm)
        const int64_t slots = kf_slots(l, dtype);
        const double inv_sh = (double)kscale[h] * std::ldexp(1.0, kf_norm_log2(l, dtype));
        auto get = [&](int64_t slot, double *re, double *im) {
            if (dtype == FFTCONV_F32) {
                const float *p = reinterpret_cast<const float *>(bins) + 2 * (h * slots + slot);
                *re = p[0];
                *im = p[1];
            } else {
                const _Float16 *p = reinterpret_cast<const _Float16 *>(bins) + 2 * (h * slots + slot);
                *re = (double)p[0];
                *im = (double)p[1];
            }
            *re *= inv_sh;
            *im *= inv_sh;
        };
        double *o = host_out + h * (N + 1) * 2;
        if (hdr.layout == KF_PAIR || hdr.layout == KF_PAIR3) {
            const _Float16 *p = reinterpret_cast<const _Float16 *>(bins) + h * slots * 2;
            for (int64_t f = 0; f <= N; ++f) {
                const int logr = log2_exact(N) - 9;
                int64_t a = hdr.layout == KF_PAIR ? pair_kf_index(f) : pair3_kf_index(f, logr);
                double sign = 1.0;
                if (a < 0) {   // row not stored: conjugate of the mirror bin 2N - f
                    a = pair3_kf_index(2 * N - f, logr);
                    sign = -1.0;
                }
                o[2 * f] = (double)p[a] * inv_sh;
                o[2 * f + 1] = sign * (double)p[a + 4] * inv_sh;
            }
            continue;
        }
        double r0, i0;
        get(0, &r0, &i0);
        o[0] = r0; o[1] = 0.0;
        o[2 * N] = i0; o[2 * N + 1] = 0.0;
        for (int64_t f = 1; f < N; ++f) {
            int64_t slot = f;
            if (hdr.layout == KF_ROWS) {
                // bin f = f1 + n1 f2 lives in row f1 at column f2 (fp32) or at the
                // matrix-core position of f2 (half precision)
                const int64_t f1 = f % n1, f2 = f / n1;
                slot = f1 * n2 + (dtype == FFTCONV_F32 ? f2 : (int64_t)mp_chain_pos((uint32_t)f2));
            }
            get(slot, &o[2 * f], &o[2 * f + 1]);
        }
    }
    return ok();
}

}  // extern "C"
