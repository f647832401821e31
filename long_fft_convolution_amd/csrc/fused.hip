// fused.hip -- single-kernel gated causal FFT convolution for N <= 16384.
//
// One workgroup owns SPW whole sequences (FlashFFTConv summary page,
// "Approach": the whole convolution is fused on chip up to long sequence
// lengths; "Measured effects" row on fusing gating: the gates are applied in
// the same kernel).  Per sequence of N real samples:
//
//   1. x = u * w, packed as z[m] = x[2m] + i x[2m+1] (m < N/2; z is zero for
//      m >= N/2 because of the zero padding to 2N): the 2N-point real FFT
//      becomes an N-point complex FFT.
//   2. Z = FFT_N(z) by Stockham radix stages: the first reads HBM directly,
//      the others exchange through LDS, the last keeps its outputs in
//      registers.  Each lane owns the butterflies j and P - j (P = N / R) of
//      the last radix-R stage, so bins f and N - f meet in one lane.
//   3. In registers, per bin pair (f, N - f): unpack the real spectrum
//      X[f], X[N-f] from Z, multiply by the filter spectrum, and repack the
//      product for the inverse half-length transform.
//   4. Inverse FFT (computed as conj(FFT(conj(.)))) with the stage order
//      reversed; the last stage writes only the needed outputs t < N, times
//      the output gate v, straight to HBM.
//
// All arithmetic is fp32; storage is fp32, fp16 or bf16.
#include "fft_device.hpp"
#include "fft_stages.hpp"
#include "fftconv_internal.hpp"

#include <type_traits>

namespace fftconv {

template <int LOGN> struct FusedPlan {
    static constexpr int NC = 1 << LOGN;           // complex points = N
    static constexpr int R = 16;                   // radix of the main stages
    static constexpr int P = NC / R;               // butterflies per radix-R stage
    static constexpr int TS = P / 2;               // lanes per sequence
    static constexpr int MR = (LOGN - 1) / 4;      // number of radix-R stages
    static constexpr int R1 = NC >> (4 * MR);      // first (forward) / last (inverse) radix
    static constexpr int NB1 = (NC / R1) / TS;     // radix-R1 butterflies per lane
    static constexpr int SPW = TS >= 256 ? 1 : 256 / TS;  // sequences per workgroup
    static constexpr int THREADS = TS * SPW;
    static_assert(R1 >= 2 && R1 <= 16, "radix plan");
};

// Forward middle stages: stage index I (0-based among the radix-R stages),
// NS = R1 * R^I, for I < MR - 1 (the last radix-R stage is done separately).
template <int LOGN, int I>
__device__ __forceinline__ void fwd_middle(float2 *buf, int ts, const float2 *__restrict__ tw) {
    using Pl = FusedPlan<LOGN>;
    if constexpr (I < Pl::MR - 1) {
        constexpr int NS = Pl::R1 << (4 * I);
        stage_lds<Pl::NC, Pl::R, Pl::TS, NS>(buf, ts, tw);
        fwd_middle<LOGN, I + 1>(buf, ts, tw);
    }
}
// Inverse middle stages: NS = R^I for I in [1, MR).
template <int LOGN, int I>
__device__ __forceinline__ void inv_middle(float2 *buf, int ts, const float2 *__restrict__ tw) {
    using Pl = FusedPlan<LOGN>;
    if constexpr (I < Pl::MR) {
        constexpr int NS = 1 << (4 * I);
        stage_lds<Pl::NC, Pl::R, Pl::TS, NS>(buf, ts, tw);
        inv_middle<LOGN, I + 1>(buf, ts, tw);
    }
}

template <typename TK>
__device__ __forceinline__ float2 kbin(const TK *__restrict__ krow, const uint8_t *__restrict__ mrow,
                                       float ks, int f, int NC) {
    float2 k = cscale(kio<TK>::load(krow + f), ks);
    if (mrow != nullptr) {
        int blk = f / (NC / kMaskBlocks);
        if (!mrow[blk]) k = make_float2(0.f, 0.f);
    }
    return k;
}

template <int LOGN, typename T, typename TK>
__global__ void __launch_bounds__(FusedPlan<LOGN>::THREADS)
fused_conv_kernel(const T *__restrict__ u, const T *__restrict__ w, const T *__restrict__ v,
                  T *__restrict__ out, const TK *__restrict__ kbins,
                  const float *__restrict__ kscale, const uint8_t *__restrict__ mask,
                  const float2 *__restrict__ tw, const float2 *__restrict__ tw2, int64_t B,
                  int64_t H) {
    using Pl = FusedPlan<LOGN>;
    constexpr int NC = Pl::NC, R = Pl::R, P = Pl::P, TS = Pl::TS, R1 = Pl::R1;
    extern __shared__ float2 lds[];
    const int tid = threadIdx.x;
    const int sw = tid / TS, ts = tid % TS;
    float2 *buf = lds + sw * NC;

    const int64_t S = B * H;
    const int64_t lb = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t sl = lb * Pl::SPW + sw;        // logical sequence: channel-major, batch fastest
    const bool valid = sl < S;
    const int64_t h = valid ? sl / B : 0;
    const int64_t b = valid ? sl % B : 0;
    const int64_t base = (b * H + h) * (int64_t)NC;

    // ---- forward stage 0 (radix R1, NS = 1) straight from HBM; inputs m >= N/2 are zero
#pragma unroll
    for (int i = 0; i < Pl::NB1; ++i) {
        const int j = ts + i * TS;
        float2 a[R1];
#pragma unroll
        for (int r = 0; r < R1; ++r) {
            a[r] = make_float2(0.f, 0.f);
            if (r < R1 / 2 && valid) {
                const int m = j + r * (NC / R1);
                float2 x = io<T>::load2(u + base + 2 * m);
                if (w != nullptr) {
                    const float2 g = io<T>::load2(w + base + 2 * m);
                    x = make_float2(x.x * g.x, x.y * g.y);
                }
                a[r] = x;
            }
        }
        dft_inplace<R1>(a);
#pragma unroll
        for (int q = 0; q < R1; ++q) buf[j * R1 + q] = a[q];
    }
    __syncthreads();

    fwd_middle<LOGN, 0>(buf, ts, tw);

    // ---- last forward stage (radix R, NS = P): butterflies jA, jB kept in registers
    const int jA = ts;
    const int jB = ts == 0 ? P / 2 : P - ts;
    float2 A[R], Bv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        A[r] = buf[jA + r * P];
        Bv[r] = buf[jB + r * P];
    }
    __syncthreads();
#pragma unroll
    for (int r = 1; r < R; ++r) {
        A[r] = cmul(A[r], tw[r * jA]);
        Bv[r] = cmul(Bv[r], tw[r * jB]);
    }
    dft_inplace<R>(A);
    dft_inplace<R>(Bv);
    // A[q] = Z[jA + q P], Bv[q] = Z[jB + q P]

    // ---- pointwise product with the filter spectrum, bin pairs (f, N - f)
    const float ks = valid ? kscale[h] : 0.f;
    const TK *krow = kbins + h * (int64_t)NC;
    const uint8_t *mrow = mask != nullptr ? mask + h * kMaskBlocks : nullptr;
    if (ts != 0) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int f = jA + q * P;
            const int g = NC - f;                  // = jB + (R - 1 - q) P
            middle_pair(A[q], Bv[R - 1 - q], kbin<TK>(krow, mrow, ks, f, NC),
                        kbin<TK>(krow, mrow, ks, g, NC), tw2[f]);
        }
    } else {
        {   // f = 0 (and N): slot 0 holds (K[0], K[N])
            float2 k0 = cscale(kio<TK>::load(krow), ks);
            float kf0 = k0.x, kgN = k0.y;
            if (mrow != nullptr) {
                if (!mrow[0]) kf0 = 0.f;
                if (!mrow[kMaskBlocks - 1]) kgN = 0.f;
            }
            float2 z = A[0], z2 = A[0];
            middle_pair(z, z2, make_float2(kf0, 0.f), make_float2(kgN, 0.f), make_float2(1.f, 0.f));
            A[0] = z;
        }
        {   // f = N/2, paired with itself
            float2 z = A[R / 2], z2 = A[R / 2];
            const float2 kh = kbin<TK>(krow, mrow, ks, NC / 2, NC);
            middle_pair(z, z2, kh, kh, tw2[NC / 2]);
            A[R / 2] = z;
        }
#pragma unroll
        for (int q = 1; q < R / 2; ++q) {
            const int f = q * P;
            middle_pair(A[q], A[R - q], kbin<TK>(krow, mrow, ks, f, NC),
                        kbin<TK>(krow, mrow, ks, NC - f, NC), tw2[f]);
        }
#pragma unroll
        for (int q = 0; q < R / 2; ++q) {
            const int f = P / 2 + q * P;
            middle_pair(Bv[q], Bv[R - 1 - q], kbin<TK>(krow, mrow, ks, f, NC),
                        kbin<TK>(krow, mrow, ks, NC - f, NC), tw2[f]);
        }
    }

    // ---- inverse stage 0 (radix R, NS = 1) from registers
    dft_inplace<R>(A);
    dft_inplace<R>(Bv);
#pragma unroll
    for (int q = 0; q < R; ++q) {
        buf[jA * R + q] = A[q];
        buf[jB * R + q] = Bv[q];
    }
    __syncthreads();

    inv_middle<LOGN, 1>(buf, ts, tw);

    // ---- last inverse stage (radix R1, NS = N / R1) straight to HBM, outputs t < N only
#pragma unroll
    for (int i = 0; i < Pl::NB1; ++i) {
        const int j = ts + i * TS;
        float2 a[R1];
#pragma unroll
        for (int r = 0; r < R1; ++r) a[r] = buf[j + r * (NC / R1)];
#pragma unroll
        for (int r = 1; r < R1; ++r) a[r] = cmul(a[r], tw[r * j]);
        dft_inplace<R1>(a);
#pragma unroll
        for (int q = 0; q < R1 / 2; ++q) {
            const int m = j + q * (NC / R1);
            float2 y = make_float2(a[q].x, -a[q].y);   // conj back: z'[m] = y[2m] + i y[2m+1]
            if (valid) {
                if (v != nullptr) {
                    const float2 g = io<T>::load2(v + base + 2 * m);
                    y = make_float2(y.x * g.x, y.y * g.y);
                }
                io<T>::store2(out + base + 2 * m, y);
            }
        }
    }
}

// Filter preparation for the fused layout: per channel, the forward
// transform of z[m] = k[2m] + i k[2m+1] (taps beyond L are zero: for a
// partial filter only the loads holding taps are issued), then the real
// spectrum X[f], f in [0, N], scaled by s_h, stored in natural order with
// slot 0 = (X[0], X[N]).
template <int LOGN, typename T, typename TK, int LAYOUT>
__global__ void __launch_bounds__(FusedPlan<LOGN>::THREADS)
fused_prepare_kernel(const T *__restrict__ k, int64_t L, TK *__restrict__ kbins,
                     const float *__restrict__ kscale, const float2 *__restrict__ tw,
                     const float2 *__restrict__ tw2, int64_t H, float ysgn) {
    using Pl = FusedPlan<LOGN>;
    constexpr int NC = Pl::NC, R = Pl::R, P = Pl::P, TS = Pl::TS, R1 = Pl::R1;
    extern __shared__ float2 lds[];
    const int tid = threadIdx.x;
    const int sw = tid / TS, ts = tid % TS;
    float2 *buf = lds + sw * NC;
    const int64_t h = (int64_t)blockIdx.x * Pl::SPW + sw;
    const bool valid = h < H;
    const T *krow_in = k + (valid ? h : 0) * L;

#pragma unroll
    for (int i = 0; i < Pl::NB1; ++i) {
        const int j = ts + i * TS;
        float2 a[R1];
#pragma unroll
        for (int r = 0; r < R1; ++r) {
            a[r] = make_float2(0.f, 0.f);
            const int m = j + r * (NC / R1);
            if (r < R1 / 2 && valid && 2 * m < L) {
                a[r].x = io<T>::load1(krow_in + 2 * m);
                if (2 * m + 1 < L) a[r].y = io<T>::load1(krow_in + 2 * m + 1);
            }
        }
        dft_inplace<R1>(a);
#pragma unroll
        for (int q = 0; q < R1; ++q) buf[j * R1 + q] = a[q];
    }
    __syncthreads();
    fwd_middle<LOGN, 0>(buf, ts, tw);

    const int jA = ts;
    const int jB = ts == 0 ? P / 2 : P - ts;
    float2 A[R], Bv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        A[r] = buf[jA + r * P];
        Bv[r] = buf[jB + r * P];
    }
#pragma unroll
    for (int r = 1; r < R; ++r) {
        A[r] = cmul(A[r], tw[r * jA]);
        Bv[r] = cmul(Bv[r], tw[r * jB]);
    }
    dft_inplace<R>(A);
    dft_inplace<R>(Bv);
    if (!valid) return;

    // N = 16384: the fp16 row (every slot of it is written below) is assembled in the
    // LDS buffer, which is free once every lane holds its A, Bv, and stored as 16-byte
    // words; stored directly, each bin would take four scattered 2-byte stores
    constexpr bool STAGE = LAYOUT == KF_PAIR3 && LOGN == 14;
    static_assert(!STAGE || (Pl::SPW == 1 && 17 * 1024 * 4 <= Pl::NC * (int)sizeof(float2)),
                  "one sequence per workgroup, its row fits the LDS buffer");
    if (STAGE) __syncthreads();
    constexpr bool PAIR = LAYOUT != KF_NATURAL;
    // s_h = 1 / (scale[h] * norm), exact (both powers of two)
    const float sh = 1.0f / (kscale[h] * (float)(PAIR ? 2 * NC : 4 * NC));
    constexpr int64_t kRowSlots = LAYOUT == KF_PAIR3 ? ((1 << (LOGN - 10)) + 1) * 1024 : (PAIR ? 2 * NC : NC);
    TK *krow = kbins + h * kRowSlots;
    _Float16 *const row16 = STAGE ? reinterpret_cast<_Float16 *>(lds) : reinterpret_cast<_Float16 *>(krow);
    // one real-spectrum bin: natural order, or a matrix-core kernel's lane
    // order (the Hermitian mirror 2N - f is stored as well where its row is)
    auto index_of = [](int64_t f) -> int64_t {
        return LAYOUT == KF_PAIR3 ? pair3_kf_index(f, LOGN - 9) : pair_kf_index(f);
    };
    // ysgn = -1 stores the conjugated spectrum (the correlation of the backward pass)
    auto put = [&](int f, float2 x) {
        x.y *= ysgn;
        if (!PAIR) {
            kio<TK>::store(krow + f, x);
        } else {
            _Float16 *kh = row16;
            const int64_t a = index_of(f);
            if (a >= 0) {
                kh[a] = (_Float16)x.x;
                kh[a + 4] = (_Float16)x.y;
            }
            if (f != 0 && f != NC) {
                const int64_t b = index_of(2 * NC - f);
                if (b >= 0) {
                    kh[b] = (_Float16)x.x;
                    kh[b + 4] = (_Float16)(-x.y);
                }
            }
        }
    };
    // X[f] = (Xe + Wf Xo)/2, X[g] = conj(Xe - Wf Xo)/2 (Xe, Xo as in middle_pair)
    auto emit = [&](float2 zf, float2 zg, int f, bool both) {
        const float2 bc = cconj(zg);
        const float2 xe = cadd(zf, bc);
        const float2 xo = cmul_negi(csub(zf, bc));
        const float2 wxo = cmul(tw2[f], xo);
        put(f, cscale(cadd(xe, wxo), 0.5f * sh));
        if (both) put(NC - f, cscale(cconj(csub(xe, wxo)), 0.5f * sh));
    };
    if (ts != 0) {
#pragma unroll
        for (int q = 0; q < R; ++q) emit(A[q], Bv[R - 1 - q], jA + q * P, true);
    } else {
        // X[0] = Re Z0 + Im Z0, X[N] = Re Z0 - Im Z0 (both real)
        const float x0 = (A[0].x + A[0].y) * sh, xn = (A[0].x - A[0].y) * sh;
        if (!PAIR) {
            kio<TK>::store(krow, make_float2(x0, xn));   // natural layout: slot 0 = (X[0], X[N])
        } else {
            put(0, make_float2(x0, 0.f));
            put(NC, make_float2(xn, 0.f));
        }
        emit(A[R / 2], A[R / 2], NC / 2, false);
#pragma unroll
        for (int q = 1; q < R / 2; ++q) emit(A[q], A[R - q], q * P, true);
#pragma unroll
        for (int q = 0; q < R / 2; ++q) emit(Bv[q], Bv[R - 1 - q], P / 2 + q * P, true);
    }
    if (STAGE) {
        __syncthreads();
        const uint4 *src = reinterpret_cast<const uint4 *>(lds);
        uint4 *dst = reinterpret_cast<uint4 *>(krow);
        for (int i = tid; i < (int)(kRowSlots * sizeof(TK) / 16); i += Pl::THREADS) dst[i] = src[i];
    }
}

// ------------------------------------------------------------------ launchers
template <int LOGN, typename T, typename TK>
static hipError_t launch_conv_t(const void *u, const void *w,
                                const void *v, void *out, const void *kbins, const float *kscale,
                                const uint8_t *mask, const Tables &tb, int64_t B, int64_t H,
                                hipStream_t stream) {
    using Pl = FusedPlan<LOGN>;
    const int64_t S = B * H;
    const int64_t blocks = (S + Pl::SPW - 1) / Pl::SPW;
    const size_t lds = (size_t)Pl::SPW * Pl::NC * sizeof(float2);
    auto kern = fused_conv_kernel<LOGN, T, TK>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(Pl::THREADS), lds, stream,
                       (const T *)u, (const T *)w, (const T *)v, (T *)out, (const TK *)kbins,
                       kscale, mask, tb.tw, tb.tw2, B, H);
    return hipGetLastError();
}

template <int LOGN, typename T, typename TK>
static hipError_t launch_prep_t(const void *k, int64_t L, void *kbins, const float *kscale,
                                const Tables &tb, int64_t H, float ysgn, hipStream_t stream) {
    using Pl = FusedPlan<LOGN>;
    const int64_t blocks = (H + Pl::SPW - 1) / Pl::SPW;
    const size_t lds = (size_t)Pl::SPW * Pl::NC * sizeof(float2);
    constexpr bool kHalf = !std::is_same<T, float>::value;
    constexpr int kLayout =
        (LOGN == 10 && kHalf) ? KF_PAIR : ((LOGN >= 11 && LOGN <= 14 && kHalf) ? KF_PAIR3 : KF_NATURAL);
    static_assert(kLayout == KF_NATURAL || std::is_same<TK, __half2>::value, "pair layouts store fp16 bins");
    auto kern = fused_prepare_kernel<LOGN, T, TK, kLayout>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(Pl::THREADS), lds, stream,
                       (const T *)k, L, (TK *)kbins, kscale, tb.tw, tb.tw2, H, ysgn);
    return hipGetLastError();
}

template <int LOGN>
static hipError_t conv_by_type(int st, const void *u, const void *w,
                               const void *v, void *out, const void *kbins, const float *kscale,
                               const uint8_t *mask, const Tables &tb, int64_t B, int64_t H,
                               hipStream_t stream) {
    switch (st) {
    case ST_F32:
        return launch_conv_t<LOGN, float, float2>(u, w, v, out, kbins, kscale,
                                                  mask, tb, B, H, stream);
    case ST_F16:
        return launch_conv_t<LOGN, __half, __half2>(u, w, v, out, kbins, kscale,
                                                    mask, tb, B, H, stream);
    default:
        return launch_conv_t<LOGN, __hip_bfloat16, __half2>(u, w, v, out, kbins,
                                                            kscale, mask, tb, B, H, stream);
    }
}

template <int LOGN>
static hipError_t prep_by_type(int st, const void *k, int64_t L, void *kbins, const float *kscale,
                               const Tables &tb, int64_t H, float ysgn, hipStream_t stream) {
    switch (st) {
    case ST_F32: return launch_prep_t<LOGN, float, float2>(k, L, kbins, kscale, tb, H, ysgn, stream);
    case ST_F16: return launch_prep_t<LOGN, __half, __half2>(k, L, kbins, kscale, tb, H, ysgn, stream);
    default:
        return launch_prep_t<LOGN, __hip_bfloat16, __half2>(k, L, kbins, kscale, tb, H, ysgn, stream);
    }
}

hipError_t launch_fused_conv(int logn, int st, const void *u,
                             const void *w, const void *v, void *out, const void *kbins,
                             const float *kscale, const uint8_t *mask, const Tables &tb,
                             int64_t B, int64_t H, hipStream_t stream) {
    switch (logn) {
    case 10: return conv_by_type<10>(st, u, w, v, out, kbins, kscale, mask, tb, B, H, stream);
    case 11: return conv_by_type<11>(st, u, w, v, out, kbins, kscale, mask, tb, B, H, stream);
    case 12: return conv_by_type<12>(st, u, w, v, out, kbins, kscale, mask, tb, B, H, stream);
    case 13: return conv_by_type<13>(st, u, w, v, out, kbins, kscale, mask, tb, B, H, stream);
    case 14: return conv_by_type<14>(st, u, w, v, out, kbins, kscale, mask, tb, B, H, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fused_prepare(int logn, int st, const void *k, int64_t L, void *kbins,
                                const float *kscale, const Tables &tb, int64_t H,
                                float ysgn, hipStream_t stream) {
    switch (logn) {
    case 10: return prep_by_type<10>(st, k, L, kbins, kscale, tb, H, ysgn, stream);
    case 11: return prep_by_type<11>(st, k, L, kbins, kscale, tb, H, ysgn, stream);
    case 12: return prep_by_type<12>(st, k, L, kbins, kscale, tb, H, ysgn, stream);
    case 13: return prep_by_type<13>(st, k, L, kbins, kscale, tb, H, ysgn, stream);
    case 14: return prep_by_type<14>(st, k, L, kbins, kscale, tb, H, ysgn, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fftconv
