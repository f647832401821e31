// fft_stages.hpp -- LDS Stockham stages and the half-length real-transform
// bin-pair step, shared by the fused and the multi-pass kernels.
#pragma once

#include "fft_device.hpp"

namespace fftconv {

// Generic Stockham stage through LDS: radix R, NS = product of the previous
// radices.  Butterfly j reads src[j + r P], multiplies by the twiddle
// omega_{NS R}^{r k} (k = j mod NS), takes the radix-R DFT and writes
// dst[(j - k) R + k + q NS].  In place: all lanes read, barrier, all write.
template <int NC, int R, int TS, int NS>
__device__ __forceinline__ void stage_lds(float2 *buf, int ts, const float2 *__restrict__ tw) {
    constexpr int P = NC / R;
    constexpr int NB = P / TS;
    float2 a[NB][R];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int j = ts + i * TS;
#pragma unroll
        for (int r = 0; r < R; ++r) a[i][r] = buf[j + r * P];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int j = ts + i * TS;
        const int k = j & (NS - 1);
        if (NS > 1) {
#pragma unroll
            for (int r = 1; r < R; ++r) a[i][r] = cmul(a[i][r], tw[(r * k) * (NC / (NS * R))]);
        }
        dft_inplace<R>(a[i]);
        const int base = (j - k) * R + k;
#pragma unroll
        for (int q = 0; q < R; ++q) buf[base + q * NS] = a[i][q];
    }
    __syncthreads();
}

// Forward FFT of NPTS points held in LDS (natural order in and out) by TS
// lanes: one radix-R1 stage then radix-16 stages, NPTS = R1 * 16^m.
template <int LOGP> struct LdsFftPlan {
    static constexpr int NPTS = 1 << LOGP;
    static constexpr int M16 = LOGP <= 4 ? 0 : (LOGP - 1) / 4;
    static constexpr int R1 = NPTS >> (4 * M16);
    static constexpr int TS = NPTS >= 64 ? NPTS / 32 : 1;   // lanes per transform
    static_assert(R1 >= 2 && R1 <= 16, "radix plan");
};

template <int NPTS, int TS, int I, int M16, int NS>
__device__ __forceinline__ void fft_lds_r16(float2 *buf, int ts, const float2 *__restrict__ tw) {
    if constexpr (I < M16) {
        stage_lds<NPTS, 16, TS, NS>(buf, ts, tw);
        fft_lds_r16<NPTS, TS, I + 1, M16, NS * 16>(buf, ts, tw);
    }
}

// tw: exp(-2 pi i j / NPTS), j < NPTS.  Ends with a barrier.
template <int LOGP>
__device__ __forceinline__ void fft_lds(float2 *buf, int ts, const float2 *__restrict__ tw) {
    using Pl = LdsFftPlan<LOGP>;
    stage_lds<Pl::NPTS, Pl::R1, Pl::TS, 1>(buf, ts, tw);
    fft_lds_r16<Pl::NPTS, Pl::TS, 0, Pl::M16, Pl::R1>(buf, ts, tw);
}

// One bin pair (f, g = N - f) of the half-length real transform.  In: the
// complex spectrum values Z[f], Z[g]; the filter bins Kf = K[f]/(4N),
// Kg = K[g]/(4N); Wf = omega_{2N}^f.  Out (in place): conj(Z'[f]),
// conj(Z'[g]) where Z' is the half-length spectrum of the product's inverse.
//   X[f] = Xe + Wf Xo, X[g] = conj(Xe - Wf Xo) with Xe = Z[f] + conj(Z[g]),
//   Xo = -i (Z[f] - conj(Z[g]))  (both twice their textbook values);
//   Y = X K;  Ye = Y[f] + conj(Y[g]),  Yo = (Y[f] - conj(Y[g])) conj(Wf);
//   Z'[f] = Ye + i Yo,  Z'[g] = conj(Ye) + i conj(Yo).
// f = 0 fits the same formula with Z[g] = Z[0] and Kg = K[N]; the self-paired
// f = N/2 with Z[g] = Z[f], Kg = Kf.
__device__ __forceinline__ void middle_pair(float2 &zf, float2 &zg, float2 Kf, float2 Kg,
                                            float2 Wf) {
    const float2 bc = cconj(zg);
    const float2 xe = cadd(zf, bc);
    const float2 xo = cmul_negi(csub(zf, bc));
    const float2 wxo = cmul(Wf, xo);
    const float2 xf = cadd(xe, wxo);
    const float2 xg = cconj(csub(xe, wxo));
    const float2 yf = cmul(xf, Kf);
    const float2 ygc = cconj(cmul(xg, Kg));
    const float2 ye = cadd(yf, ygc);
    const float2 yo = cmul(csub(yf, ygc), cconj(Wf));
    // conj(Z'[f]) = conj(ye) - i conj(yo);  conj(Z'[g]) = ye - i yo
    zf = make_float2(ye.x - yo.y, -ye.y - yo.x);
    zg = make_float2(ye.x + yo.y, ye.y - yo.x);
}

}  // namespace fftconv
