// multipass.hip -- gated causal FFT convolution for N > 16384 in three passes
// through HBM (FlashFFTConv summary page, "Problem" and "Limitations": at long
// lengths the I/O between memory levels dominates; "Approach": the transform
// is an order-p decomposition into small dense transforms).
//
// The half-length real transform of the fused kernel is kept: per sequence
// z[m] = x[2m] + i x[2m+1], m < N (z = 0 for m >= N/2), an N-point complex
// FFT.  N = N1 * N2 with N2 = 8192 on chip; m = n2 + N2 n1 and
// f = f1 + N1 f2 (four-step factorisation):
//
//   Z[f1 + N1 f2] = sum_n2 w_N2^{n2 f2} w_N^{n2 f1} sum_n1 w_N1^{n1 f1} z[n2 + N2 n1]
//
//   pass 1  per column n2: DFT over n1 (rows n1 >= N1/2 are zero and never
//           read), twiddle w_N^{n2 f1}, store row-major a[f1][n2] (workspace);
//   pass 2  per row pair (f1, N1 - f1): the two row FFTs over n2 put bins f
//           and N - f in one workgroup (f = f1 + N1 f2 pairs with
//           N - f = (N1 - f1) + N1 (N2 - 1 - f2)); the filter product and the
//           repacking of the bin-pair step; inverse row FFTs; store back;
//   pass 3  per column n2: conjugate twiddle, inverse DFT over f1 keeping only
//           n1 < N1/2 (outputs t < N), output gate, store.
//
// Workspace: one fp32 complex value per point and sequence of the chunk.
#include "fft_device.hpp"
#include "fft_stages.hpp"
#include "fftconv_internal.hpp"

namespace fftconv {

constexpr int kMpLog2 = 13;                // on-chip row length N2 = 8192
constexpr int kMpThreads = 256;

// omega_N^a for a in [0, N): two-level table lookup (a = hi * 2048 + lo)
__device__ __forceinline__ float2 tw_big(const float2 *__restrict__ lo, const float2 *__restrict__ hi,
                                         uint32_t a) {
    return cmul(hi[a >> 11], lo[a & 2047u]);
}

struct MpArgs {
    const float2 *tw1;      // exp(-2 pi i j / N1), j < N1
    const float2 *tw2;      // exp(-2 pi i j / N2), j < N2
    const float2 *w2n2;     // exp(-pi i j / N2),   j < N2   (omega_{2 N2}^j)
    const float2 *w2row;    // exp(-pi i j / N),    j < N1   (omega_{2N}^{f1})
    const float2 *big_lo;   // exp(-2 pi i j / N),  j < 2048
    const float2 *big_hi;   // exp(-2 pi i 2048 j / N), j < N / 2048
};

// ---------------------------------------------------------------- pass 1
// grid (N2 / NCOL, nseq); block 256.  SRC_FILTER: input is the filter row
// k[h, :L] (prepare); else u * w of sequence seq0 + blockIdx.y.
template <int LOG1, typename T, bool SRC_FILTER>
__global__ void __launch_bounds__(kMpThreads)
mp_pass1_kernel(const T *__restrict__ src, const T *__restrict__ gate, int64_t L, int64_t seq0,
                float2 *__restrict__ ws, MpArgs ta) {
    using Pl = LdsFftPlan<LOG1>;
    constexpr int N1 = 1 << LOG1, N2 = 1 << kMpLog2;
    constexpr int64_t NC = (int64_t)N1 * N2;
    constexpr int TS = Pl::TS, NCOL = kMpThreads / TS, STRIDE = N1 + 1;
    extern __shared__ float2 lds[];
    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * NCOL;
    const int64_t s = seq0 + blockIdx.y;
    const T *row = src + s * (SRC_FILTER ? L : NC);
    const T *grow = (!SRC_FILTER && gate != nullptr) ? gate + s * NC : nullptr;

    // load rows n1 < N1/2 (coalesced along n2), zero the rest
    for (int idx = tid; idx < N1 * NCOL; idx += kMpThreads) {
        const int n1 = idx / NCOL, col = idx % NCOL;
        float2 z = make_float2(0.f, 0.f);
        if (n1 < N1 / 2) {
            const int64_t m = (int64_t)(c0 + col) + (int64_t)N2 * n1;
            if (SRC_FILTER) {
                if (2 * m < L) z.x = io<T>::load1(row + 2 * m);
                if (2 * m + 1 < L) z.y = io<T>::load1(row + 2 * m + 1);
            } else {
                z = io<T>::load2(row + 2 * m);
                if (grow != nullptr) {
                    const float2 g = io<T>::load2(grow + 2 * m);
                    z = make_float2(z.x * g.x, z.y * g.y);
                }
            }
        }
        lds[col * STRIDE + n1] = z;
    }
    __syncthreads();
    fft_lds<LOG1>(lds + (tid / TS) * STRIDE, tid % TS, ta.tw1);
    float2 *out = ws + blockIdx.y * NC;
    for (int idx = tid; idx < N1 * NCOL; idx += kMpThreads) {
        const int f1 = idx / NCOL, col = idx % NCOL;
        const uint32_t n2 = (uint32_t)(c0 + col);
        const uint32_t a = (uint32_t)(((uint64_t)n2 * (uint64_t)f1) & (uint64_t)(NC - 1));
        out[(int64_t)f1 * N2 + n2] = cmul(lds[col * STRIDE + f1], tw_big(ta.big_lo, ta.big_hi, a));
    }
}

// ---------------------------------------------------------------- pass 2
// One work item of the bin-pair step in a row-pair workgroup.  Rows A, B in
// LDS (natural order after the row FFTs).  Workgroup 0 holds rows 0 and N1/2
// (each paired with itself); the others rows f1 and N1 - f1.
struct PairItem {
    int ia, ib;       // LDS indices of the two bins (ib == ia: single)
    int64_t f, g;     // bins (g = N - f; f == 0 uses K[N] as partner)
};

template <int N1, int N2>
__device__ __forceinline__ bool pair_item(int w, int f1, PairItem &it) {
    constexpr int64_t NC = (int64_t)N1 * N2;
    if (f1 != 0) {
        if (w >= N2) return false;
        it.ia = w;
        it.ib = N2 + (N2 - 1 - w);
        it.f = f1 + (int64_t)N1 * w;
        it.g = NC - it.f;
        return true;
    }
    if (w < N2 / 2) {                      // row N1/2 (LDS row B): f2 <-> N2 - 1 - f2
        it.ia = N2 + w;
        it.ib = N2 + (N2 - 1 - w);
        it.f = N1 / 2 + (int64_t)N1 * w;
        it.g = NC - it.f;
        return true;
    }
    if (w < N2) {                          // row 0 (LDS row A): f2 <-> N2 - f2
        const int f2 = w - N2 / 2;
        it.ia = f2;
        it.ib = f2 == 0 ? 0 : N2 - f2;
        it.f = (int64_t)N1 * f2;
        it.g = f2 == 0 ? 0 : NC - it.f;
        return true;
    }
    if (w == N2) {                         // f = N/2, paired with itself
        it.ia = it.ib = N2 / 2;
        it.f = it.g = NC / 2;
        return true;
    }
    return false;
}

template <int N1, int N2>
__device__ __forceinline__ int64_t kslot(int64_t f) {
    return (f % N1) * N2 + f / N1;       // row-major (f1, f2); f = 0 -> slot 0
}

template <int N1, int N2>
__device__ __forceinline__ float2 omega2n(int64_t f, const MpArgs &ta) {
    return cmul(ta.w2row[f % N1], ta.w2n2[f / N1]);
}

// grid (N1 / 2, nseq); block 512 (256 lanes per row).  PREPARE: forward only,
// writes the filter spectrum; else the full filter product and inverse rows.
template <int LOG1, typename TK, bool PREPARE>
__global__ void __launch_bounds__(2 * kMpThreads)
mp_pass2_kernel(float2 *__restrict__ ws, const TK *__restrict__ kbins_in, TK *__restrict__ kbins_out,
                const float *__restrict__ kscale, const uint8_t *__restrict__ mask, int64_t H,
                int64_t seq0, MpArgs ta) {
    constexpr int N1 = 1 << LOG1, N2 = 1 << kMpLog2;
    constexpr int64_t NC = (int64_t)N1 * N2;
    constexpr int TS = LdsFftPlan<kMpLog2>::TS;   // 256
    extern __shared__ float2 lds[];
    const int tid = threadIdx.x;
    const int f1 = blockIdx.x;
    const int rowA = f1, rowB = f1 == 0 ? N1 / 2 : N1 - f1;
    const int64_t s = seq0 + blockIdx.y;
    const int64_t h = s % H;
    float2 *wsq = ws + blockIdx.y * NC;

    for (int i = tid; i < N2; i += 2 * kMpThreads) {
        lds[i] = wsq[(int64_t)rowA * N2 + i];
        lds[N2 + i] = wsq[(int64_t)rowB * N2 + i];
    }
    __syncthreads();
    fft_lds<kMpLog2>(lds + (tid / TS) * N2, tid % TS, ta.tw2);

    const float ks = kscale[h];
    if (PREPARE) {
        const float sh = 1.0f / (ks * 4.0f * (float)NC);
        TK *krow = kbins_out + h * NC;
        for (int w = tid; w <= N2; w += 2 * kMpThreads) {
            PairItem it;
            if (!pair_item<N1, N2>(w, f1, it)) continue;
            const float2 zf = lds[it.ia], zg = lds[it.ib];
            const float2 bc = cconj(zg);
            const float2 xe = cadd(zf, bc);
            const float2 xo = cmul_negi(csub(zf, bc));
            const float2 wxo = cmul(it.f == 0 ? make_float2(1.f, 0.f) : omega2n<N1, N2>(it.f, ta), xo);
            const float2 xf = cscale(cadd(xe, wxo), 0.5f * sh);
            const float2 xg = cscale(cconj(csub(xe, wxo)), 0.5f * sh);
            if (it.f == 0) {
                kio<TK>::store(krow, make_float2(xf.x, xg.x));   // (X[0], X[N])
            } else {
                kio<TK>::store(krow + kslot<N1, N2>(it.f), xf);
                if (it.ib != it.ia) kio<TK>::store(krow + kslot<N1, N2>(it.g), xg);
            }
        }
        return;
    }

    const TK *krow = kbins_in + h * NC;
    const uint8_t *mrow = mask != nullptr ? mask + h * kMaskBlocks : nullptr;
    constexpr int64_t G = NC / kMaskBlocks;
    auto kval = [&](int64_t f) -> float2 {
        float2 k = cscale(kio<TK>::load(krow + kslot<N1, N2>(f)), ks);
        if (mrow != nullptr && !mrow[f / G]) k = make_float2(0.f, 0.f);
        return k;
    };
    for (int w = tid; w <= N2; w += 2 * kMpThreads) {
        PairItem it;
        if (!pair_item<N1, N2>(w, f1, it)) continue;
        float2 zf = lds[it.ia], zg = lds[it.ib];
        float2 Kf, Kg, Wf;
        if (it.f == 0) {
            float2 k0 = cscale(kio<TK>::load(krow), ks);
            float a = k0.x, b = k0.y;
            if (mrow != nullptr) {
                if (!mrow[0]) a = 0.f;
                if (!mrow[kMaskBlocks - 1]) b = 0.f;
            }
            Kf = make_float2(a, 0.f);
            Kg = make_float2(b, 0.f);
            Wf = make_float2(1.f, 0.f);
        } else {
            Kf = kval(it.f);
            Kg = it.ib == it.ia ? Kf : kval(it.g);
            Wf = omega2n<N1, N2>(it.f, ta);
        }
        middle_pair(zf, zg, Kf, Kg, Wf);
        lds[it.ia] = zf;
        if (it.ib != it.ia) lds[it.ib] = zg;
    }
    __syncthreads();
    fft_lds<kMpLog2>(lds + (tid / TS) * N2, tid % TS, ta.tw2);
    // rows now hold conj of the inverse row transform; pass 3 undoes the conj
    for (int i = tid; i < N2; i += 2 * kMpThreads) {
        wsq[(int64_t)rowA * N2 + i] = lds[i];
        wsq[(int64_t)rowB * N2 + i] = lds[N2 + i];
    }
}

// ---------------------------------------------------------------- pass 3
template <int LOG1, typename T>
__global__ void __launch_bounds__(kMpThreads)
mp_pass3_kernel(const float2 *__restrict__ ws, const T *__restrict__ v, T *__restrict__ out,
                int64_t seq0, MpArgs ta) {
    using Pl = LdsFftPlan<LOG1>;
    constexpr int N1 = 1 << LOG1, N2 = 1 << kMpLog2;
    constexpr int64_t NC = (int64_t)N1 * N2;
    constexpr int TS = Pl::TS, NCOL = kMpThreads / TS, STRIDE = N1 + 1;
    extern __shared__ float2 lds[];
    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * NCOL;
    const int64_t s = seq0 + blockIdx.y;
    const float2 *wsq = ws + blockIdx.y * NC;
    for (int idx = tid; idx < N1 * NCOL; idx += kMpThreads) {
        const int f1 = idx / NCOL, col = idx % NCOL;
        const uint32_t n2 = (uint32_t)(c0 + col);
        const uint32_t a = (uint32_t)(((uint64_t)n2 * (uint64_t)f1) & (uint64_t)(NC - 1));
        // stored value is conj(b); conj(b * w^-a) = conj(b) * w^a
        lds[col * STRIDE + f1] = cmul(wsq[(int64_t)f1 * N2 + n2], tw_big(ta.big_lo, ta.big_hi, a));
    }
    __syncthreads();
    fft_lds<LOG1>(lds + (tid / TS) * STRIDE, tid % TS, ta.tw1);
    const T *vrow = v != nullptr ? v + s * NC : nullptr;
    T *orow = out + s * NC;
    for (int idx = tid; idx < (N1 / 2) * NCOL; idx += kMpThreads) {
        const int n1 = idx / NCOL, col = idx % NCOL;
        const int64_t m = (int64_t)(c0 + col) + (int64_t)N2 * n1;
        const float2 r = lds[col * STRIDE + n1];
        float2 y = make_float2(r.x, -r.y);
        if (vrow != nullptr) {
            const float2 g = io<T>::load2(vrow + 2 * m);
            y = make_float2(y.x * g.x, y.y * g.y);
        }
        io<T>::store2(orow + 2 * m, y);
    }
}

// ---------------------------------------------------------------- tables
static hipError_t mp_args(int logn, MpArgs *a) {
    Tables t1{}, t2{};
    const int log1 = logn - kMpLog2;
    hipError_t e = get_tables(log1, &t1);       // tw: omega_N1
    if (e == hipSuccess) e = get_tables(kMpLog2, &t2);   // tw: omega_N2, tw2: omega_2N2
    if (e != hipSuccess) return e;
    MpTables mt{};
    e = get_mp_tables(logn, &mt);
    if (e != hipSuccess) return e;
    a->tw1 = t1.tw;
    a->tw2 = t2.tw;
    a->w2n2 = t2.tw2;
    a->w2row = mt.w2row;
    a->big_lo = mt.big_lo;
    a->big_hi = mt.big_hi;
    return hipSuccess;
}

template <int LOG1>
static size_t lds_cols() {
    using Pl = LdsFftPlan<LOG1>;
    return (size_t)(kMpThreads / Pl::TS) * ((1 << LOG1) + 1) * sizeof(float2);
}

template <typename K>
static hipError_t allow_lds(K kern, size_t bytes) {
    return hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <int LOG1, typename T, typename TK>
static hipError_t conv_t(const void *u, const void *w, const void *v, void *out, const void *kbins,
                         const float *kscale, const uint8_t *mask, void *work, int64_t H,
                         int64_t seq0, int64_t nseq, hipStream_t stream) {
    constexpr int N2 = 1 << kMpLog2, NCOL = kMpThreads / LdsFftPlan<LOG1>::TS;
    MpArgs ta{};
    hipError_t e = mp_args(LOG1 + kMpLog2, &ta);
    if (e != hipSuccess) return e;
    float2 *ws = (float2 *)work;
    const size_t l1 = lds_cols<LOG1>(), l2 = 2 * (size_t)N2 * sizeof(float2);
    auto k1 = mp_pass1_kernel<LOG1, T, false>;
    auto k2 = mp_pass2_kernel<LOG1, TK, false>;
    auto k3 = mp_pass3_kernel<LOG1, T>;
    if ((e = allow_lds(k1, l1)) != hipSuccess) return e;
    if ((e = allow_lds(k2, l2)) != hipSuccess) return e;
    if ((e = allow_lds(k3, l1)) != hipSuccess) return e;
    hipLaunchKernelGGL(k1, dim3(N2 / NCOL, (unsigned)nseq), dim3(kMpThreads), l1, stream,
                       (const T *)u, (const T *)w, (int64_t)0, seq0, ws, ta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k2, dim3((1 << LOG1) / 2, (unsigned)nseq), dim3(2 * kMpThreads), l2, stream,
                       ws, (const TK *)kbins, (TK *)nullptr, kscale, mask, H, seq0, ta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k3, dim3(N2 / NCOL, (unsigned)nseq), dim3(kMpThreads), l1, stream,
                       (const float2 *)ws, (const T *)v, (T *)out, seq0, ta);
    return hipGetLastError();
}

template <int LOG1, typename T, typename TK>
static hipError_t prep_t(const void *k, int64_t L, void *kbins, const float *kscale, void *work,
                         int64_t H, int64_t h0, int64_t nseq, hipStream_t stream) {
    constexpr int N2 = 1 << kMpLog2, NCOL = kMpThreads / LdsFftPlan<LOG1>::TS;
    MpArgs ta{};
    hipError_t e = mp_args(LOG1 + kMpLog2, &ta);
    if (e != hipSuccess) return e;
    float2 *ws = (float2 *)work;
    const size_t l1 = lds_cols<LOG1>(), l2 = 2 * (size_t)N2 * sizeof(float2);
    auto k1 = mp_pass1_kernel<LOG1, T, true>;
    auto k2 = mp_pass2_kernel<LOG1, TK, true>;
    if ((e = allow_lds(k1, l1)) != hipSuccess) return e;
    if ((e = allow_lds(k2, l2)) != hipSuccess) return e;
    hipLaunchKernelGGL(k1, dim3(N2 / NCOL, (unsigned)nseq), dim3(kMpThreads), l1, stream,
                       (const T *)k, (const T *)nullptr, L, h0, ws, ta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k2, dim3((1 << LOG1) / 2, (unsigned)nseq), dim3(2 * kMpThreads), l2, stream,
                       ws, (const TK *)nullptr, (TK *)kbins, kscale, (const uint8_t *)nullptr, H,
                       h0, ta);
    return hipGetLastError();
}

template <int LOG1>
static hipError_t conv_st(int st, const void *u, const void *w, const void *v, void *out,
                          const void *kbins, const float *kscale, const uint8_t *mask, void *work,
                          int64_t H, int64_t seq0, int64_t nseq, hipStream_t stream) {
    switch (st) {
    case ST_F32:
        return conv_t<LOG1, float, float2>(u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    case ST_F16:
        return conv_t<LOG1, __half, __half2>(u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    default:
        return conv_t<LOG1, __hip_bfloat16, __half2>(u, w, v, out, kbins, kscale, mask, work, H, seq0,
                                                     nseq, stream);
    }
}

template <int LOG1>
static hipError_t prep_st(int st, const void *k, int64_t L, void *kbins, const float *kscale,
                          void *work, int64_t H, int64_t h0, int64_t nseq, hipStream_t stream) {
    switch (st) {
    case ST_F32: return prep_t<LOG1, float, float2>(k, L, kbins, kscale, work, H, h0, nseq, stream);
    case ST_F16: return prep_t<LOG1, __half, __half2>(k, L, kbins, kscale, work, H, h0, nseq, stream);
    default:
        return prep_t<LOG1, __hip_bfloat16, __half2>(k, L, kbins, kscale, work, H, h0, nseq, stream);
    }
}

hipError_t launch_multipass_conv(int logn, int st, const void *u, const void *w, const void *v,
                                 void *out, const void *kbins, const float *kscale,
                                 const uint8_t *mask, void *work, int64_t H, int64_t seq0,
                                 int64_t nseq, hipStream_t stream) {
    switch (logn - kMpLog2) {
    case 2: return conv_st<2>(st, u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    case 3: return conv_st<3>(st, u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    case 4: return conv_st<4>(st, u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    case 5: return conv_st<5>(st, u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    case 6: return conv_st<6>(st, u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    case 7: return conv_st<7>(st, u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    case 8: return conv_st<8>(st, u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    case 9: return conv_st<9>(st, u, w, v, out, kbins, kscale, mask, work, H, seq0, nseq, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_multipass_prepare(int logn, int st, const void *k, int64_t L, void *kbins,
                                    const float *kscale, void *work, int64_t H, int64_t h0,
                                    int64_t nseq, hipStream_t stream) {
    switch (logn - kMpLog2) {
    case 2: return prep_st<2>(st, k, L, kbins, kscale, work, H, h0, nseq, stream);
    case 3: return prep_st<3>(st, k, L, kbins, kscale, work, H, h0, nseq, stream);
    case 4: return prep_st<4>(st, k, L, kbins, kscale, work, H, h0, nseq, stream);
    case 5: return prep_st<5>(st, k, L, kbins, kscale, work, H, h0, nseq, stream);
    case 6: return prep_st<6>(st, k, L, kbins, kscale, work, H, h0, nseq, stream);
    case 7: return prep_st<7>(st, k, L, kbins, kscale, work, H, h0, nseq, stream);
    case 8: return prep_st<8>(st, k, L, kbins, kscale, work, H, h0, nseq, stream);
    case 9: return prep_st<9>(st, k, L, kbins, kscale, work, H, h0, nseq, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fftconv
