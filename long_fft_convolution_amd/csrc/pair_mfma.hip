// pair_mfma.hip -- gated causal FFT convolution for N = 1024 on the MFMA
// matrix cores (fp16 operands, fp32 accumulation).
//
// FlashFFTConv summary page, "Approach": the FFT convolution is rewritten as
// an order-p Monarch decomposition into matrix-matrix products, with the
// permutations done as on-chip transposes.  Here, on gfx950:
//
//  * Two real sequences of the same channel are packed as one complex
//    sequence z = x_a + i x_b (x = u * w), zero-padded to M = 2N = 2048.  With
//    a real filter, irfft-by-parts is unnecessary: IFFT(FFT(z) K) = y_a + i y_b.
//  * M = 64 * 32, m = n_f + 32 n_s, f = f_s + 64 f_f (four-step):
//        Z[f_s + 64 f_f] = sum_nf w32^{nf ff} w2048^{nf fs} sum_ns w64^{ns fs} z[nf + 32 ns]
//    Stage S1 contracts n_s (only n_s < 32 is non-zero: half the work), S2
//    contracts n_f; the inverse S2' contracts f_f and S1' contracts f_s and
//    produces only n_s < 32 (outputs t < N).
//  * Every stage is a complex-as-real product on v_mfma_f32_16x16x32_f16
//    (4 real MFMAs per complex 16x16x32 tile).  The accumulator layout of one
//    stage (lane l holds rows 4(l/16)+i of column l%16) is reused as the next
//    stage's operand layout by permuting the contraction index:
//    K slot 8g + j <-> row 4g + j (j < 4) of tile 0, row 4g + j - 4 of tile 1.
//    So the stages chain in registers; only the input goes through LDS.
//  * Twiddles and the filter product are fp32 on the VALU between stages.
//
// One wave owns one sequence pair at a time and loops over pairs
// (persistent); the DFT blocks stay in registers across pairs.
#include "fft_device.hpp"
#include "fftconv_internal.hpp"

namespace fftconv {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 consecutive storage elements -> fp32
template <typename T> struct io8;
template <> struct io8<__half> {
    static __device__ __forceinline__ void load(const __half *p, float *o) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(p);
        const _Float16 *hv = reinterpret_cast<const _Float16 *>(&raw);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (float)hv[i];
    }
    static __device__ __forceinline__ void load4(const __half *p, float *o) {
        const uint2 raw = *reinterpret_cast<const uint2 *>(p);
        const _Float16 *hv = reinterpret_cast<const _Float16 *>(&raw);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (float)hv[i];
    }
    static __device__ __forceinline__ void store4(__half *p, const float *v) {
        _Float16 hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = (_Float16)v[i];
        *reinterpret_cast<uint2 *>(p) = *reinterpret_cast<const uint2 *>(hv);
    }
};
template <> struct io8<__hip_bfloat16> {
    static __device__ __forceinline__ void load(const __hip_bfloat16 *p, float *o) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void load4(const __hip_bfloat16 *p, float *o) {
        const uint2 raw = *reinterpret_cast<const uint2 *>(p);
        o[0] = __uint_as_float(raw.x << 16);
        o[1] = __uint_as_float(raw.x & 0xffff0000u);
        o[2] = __uint_as_float(raw.y << 16);
        o[3] = __uint_as_float(raw.y & 0xffff0000u);
    }
    static __device__ __forceinline__ void store4(__hip_bfloat16 *p, const float *v) {
        uint32_t w[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            __hip_bfloat16 a = __float2bfloat16(v[2 * i]), b = __float2bfloat16(v[2 * i + 1]);
            w[i] = (uint32_t)(*reinterpret_cast<uint16_t *>(&a)) |
                   ((uint32_t)(*reinterpret_cast<uint16_t *>(&b)) << 16);
        }
        *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    }
};

// (re, im) fp32 accumulators of two row tiles -> fp16 operand planes
__device__ __forceinline__ h8 pack8(const f4 &t0, const f4 &t1) {
    h8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = (_Float16)t0[i];
        r[4 + i] = (_Float16)t1[i];
    }
    return r;
}

// ρ^{-1}: input row n_s < 32 -> K slot within the S1 operand
__device__ __forceinline__ int kslot_of(int ns) {
    const int t = ns >> 4, r = ns & 15;
    return 8 * (r >> 2) + 4 * t + (r & 3);
}

constexpr int kPairWaves = 4;
constexpr int kPlane = 32 * 32;     // fp16 elements per LDS plane (rows n_f, K slots)

template <typename T>
__global__ void __launch_bounds__(64 * kPairWaves)
pair1k_kernel(const T *__restrict__ u, const T *__restrict__ w, const T *__restrict__ v,
              T *__restrict__ out, const uint4 *__restrict__ kbins, const float *__restrict__ kscale,
              const uint8_t *__restrict__ mask, PairTables tb, int64_t B, int64_t H) {
    constexpr int N = 1024;
    __shared__ float2 s_tw1[2 * 4 * 64 * 4];
    __shared__ float2 s_tw3[4 * 2 * 64 * 4];
    __shared__ _Float16 s_z[kPairWaves][2][kPlane];

    const int tid = threadIdx.x;
    for (int i = tid; i < 2048; i += 64 * kPairWaves) {
        s_tw1[i] = tb.tw1[i];
        s_tw3[i] = tb.tw3[i];
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
    const h8 *F1r = reinterpret_cast<const h8 *>(tb.f1r), *F1i = reinterpret_cast<const h8 *>(tb.f1i);
    const h8 *F2r = reinterpret_cast<const h8 *>(tb.f2r), *F2i = reinterpret_cast<const h8 *>(tb.f2i);
    const h8 *F3r = reinterpret_cast<const h8 *>(tb.f3r), *F3i = reinterpret_cast<const h8 *>(tb.f3i);
    h8 c1r[4], c1i[4], c2r[2], c2i[2], c3r[4], c3i[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        c1r[t] = F1r[t * 64 + lane];
        c1i[t] = F1i[t * 64 + lane];
        c3r[t] = F3r[t * 64 + lane];
        c3i[t] = F3i[t * 64 + lane];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        c2r[t] = F2r[t * 64 + lane];
        c2i[t] = F2i[t * 64 + lane];
    }

    // pair p = h * PB + bp (batch fastest); each XCD walks one contiguous range
    const int64_t PB = (B + 1) / 2;
    const int64_t P = H * PB;
    const uint32_t nwg = gridDim.x, xcd = blockIdx.x % 8, wg_local = blockIdx.x / 8;
    const uint32_t wg_on_xcd = nwg / 8 + (xcd < nwg % 8 ? 1u : 0u);
    const int64_t p_begin = P * xcd / 8, p_end = P * (xcd + 1) / 8;
    const int64_t stride = (int64_t)wg_on_xcd * kPairWaves;
    _Float16 *zr = s_z[wave][0], *zi = s_z[wave][1];
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};

    for (int64_t p = p_begin + (int64_t)wg_local * kPairWaves + wave; p < p_end; p += stride) {
        const int64_t h = p / PB, bp = p % PB;
        const int64_t ba = 2 * bp, bb = 2 * bp + 1;
        const bool has_b = bb < B;
        const int64_t oa = (ba * H + h) * N, ob = (has_b ? bb * H + h : 0) * N;

        // ---- load x = u * w of both sequences, scatter into the transposed LDS planes
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int m0 = 8 * lane + 512 * r;
            float xa[8], xb[8], g8[8];
            io8<T>::load(u + oa + m0, xa);
            if (w != nullptr) {
                io8<T>::load(w + oa + m0, g8);
#pragma unroll
                for (int e = 0; e < 8; ++e) xa[e] *= g8[e];
            }
            if (has_b) {
                io8<T>::load(u + ob + m0, xb);
                if (w != nullptr) {
                    io8<T>::load(w + ob + m0, g8);
#pragma unroll
                    for (int e = 0; e < 8; ++e) xb[e] *= g8[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) xb[e] = 0.f;
            }
            const int ns = m0 >> 5, nf0 = m0 & 31, ks = kslot_of(ns);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                zr[(nf0 + e) * 32 + ks] = (_Float16)xa[e];
                zi[(nf0 + e) * 32 + ks] = (_Float16)xb[e];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        h8 dr[2], di[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            dr[mt] = *reinterpret_cast<const h8 *>(zr + (16 * mt + c) * 32 + 8 * g);
            di[mt] = *reinterpret_cast<const h8 *>(zi + (16 * mt + c) * 32 + 8 * g);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const h8 ndi0 = -di[0], ndi1 = -di[1];

        const float ks = kscale[h];
        const uint4 *krow = kbins + h * 512;
        const uint8_t *mrow = mask != nullptr ? mask + h * kMaskBlocks : nullptr;

        // T3 operand planes for S1' : [ks][nt2] (rows f_s of tiles nt = 2ks, 2ks+1)
        f4 t3r[4][2], t3i[4][2];

#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            // ---- S1: rows n_f (tiles mt), column tile nt of f_s; then twiddle w2048^{nf fs}
            f4 t1r[2], t1i[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                f4 ar = mfma(dr[mt], c1r[nt], zero4);
                ar = mfma(mt == 0 ? ndi0 : ndi1, c1i[nt], ar);
                f4 ai = mfma(dr[mt], c1i[nt], zero4);
                ai = mfma(di[mt], c1r[nt], ai);
                const float4 *tw = reinterpret_cast<const float4 *>(s_tw1 + ((mt * 4 + nt) * 64 + lane) * 4);
                const float4 w01 = tw[0], w23 = tw[1];
                const float wr[4] = {w01.x, w01.z, w23.x, w23.z}, wi[4] = {w01.y, w01.w, w23.y, w23.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float re = ar[i], im = ai[i];
                    t1r[mt][i] = fmaf(re, wr[i], -im * wi[i]);
                    t1i[mt][i] = fmaf(re, wi[i], im * wr[i]);
                }
            }
            const h8 br = pack8(t1r[0], t1r[1]), bi = pack8(t1i[0], t1i[1]);
            const h8 nbi = -bi;
            // ---- S2: rows f_f (tiles mt2), column tile nt; then the filter product
            f4 yr[2], yi[2];
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2) {
                f4 ar = mfma(c2r[mt2], br, zero4);
                ar = mfma(c2i[mt2], nbi, ar);
                f4 ai = mfma(c2r[mt2], bi, zero4);
                ai = mfma(c2i[mt2], br, ai);
                const uint4 kraw = krow[(mt2 * 4 + nt) * 64 + lane];
                const _Float16 *kh = reinterpret_cast<const _Float16 *>(&kraw);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float kr = (float)kh[i] * ks, ki = (float)kh[4 + i] * ks;
                    if (mrow != nullptr) {
                        const int f = 16 * nt + c + 64 * (16 * mt2 + 4 * g + i);
                        const int fr = f <= N ? f : 2 * N - f;
                        int blk = fr / (N / kMaskBlocks);
                        blk = blk > kMaskBlocks - 1 ? kMaskBlocks - 1 : blk;
                        if (!mrow[blk]) kr = ki = 0.f;
                    }
                    const float re = ar[i], im = ai[i];
                    yr[mt2][i] = fmaf(re, kr, -im * ki);
                    yi[mt2][i] = fmaf(re, ki, im * kr);
                }
            }
            const h8 a2r = pack8(yr[0], yr[1]), a2i = pack8(yi[0], yi[1]);
            const h8 na2r = -a2r;
            // ---- S2': rows f_s (this tile nt), column tiles nt2 of n_f; then conj twiddle
#pragma unroll
            for (int nt2 = 0; nt2 < 2; ++nt2) {
                f4 ar = mfma(a2r, c2r[nt2], zero4);
                ar = mfma(a2i, c2i[nt2], ar);
                f4 ai = mfma(na2r, c2i[nt2], zero4);
                ai = mfma(a2i, c2r[nt2], ai);
                const float4 *tw = reinterpret_cast<const float4 *>(s_tw3 + ((nt * 2 + nt2) * 64 + lane) * 4);
                const float4 w01 = tw[0], w23 = tw[1];
                const float wr[4] = {w01.x, w01.z, w23.x, w23.z}, wi[4] = {w01.y, w01.w, w23.y, w23.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float re = ar[i], im = ai[i];
                    t3r[nt][nt2][i] = fmaf(re, wr[i], -im * wi[i]);
                    t3i[nt][nt2][i] = fmaf(re, wi[i], im * wr[i]);
                }
            }
        }

        // ---- S1': rows n_f (tiles nt2), columns n_s (tiles nt3, n_s < 32 only), K = f_s
#pragma unroll
        for (int nt2 = 0; nt2 < 2; ++nt2) {
            const h8 a0r = pack8(t3r[0][nt2], t3r[1][nt2]), a0i = pack8(t3i[0][nt2], t3i[1][nt2]);
            const h8 a1r = pack8(t3r[2][nt2], t3r[3][nt2]), a1i = pack8(t3i[2][nt2], t3i[3][nt2]);
            const h8 na0i = -a0i, na1i = -a1i;
#pragma unroll
            for (int nt3 = 0; nt3 < 2; ++nt3) {
                f4 ar = mfma(a0r, c3r[nt3], zero4);
                ar = mfma(na0i, c3i[nt3], ar);
                ar = mfma(a1r, c3r[2 + nt3], ar);
                ar = mfma(na1i, c3i[2 + nt3], ar);
                f4 ai = mfma(a0r, c3i[nt3], zero4);
                ai = mfma(a0i, c3r[nt3], ai);
                ai = mfma(a1r, c3i[2 + nt3], ai);
                ai = mfma(a1i, c3r[2 + nt3], ai);
                // rows n_f = 16 nt2 + 4g + i, column n_s = 16 nt3 + c: m = n_f + 32 n_s
                const int m = 16 * nt2 + 4 * g + 32 * (16 * nt3 + c);
                float ya[4] = {ar[0], ar[1], ar[2], ar[3]}, yb[4] = {ai[0], ai[1], ai[2], ai[3]};
                if (v != nullptr) {
                    float g4[4];
                    io8<T>::load4(v + oa + m, g4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) ya[i] *= g4[i];
                    if (has_b) {
                        io8<T>::load4(v + ob + m, g4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) yb[i] *= g4[i];
                    }
                }
                io8<T>::store4(out + oa + m, ya);
                if (has_b) io8<T>::store4(out + ob + m, yb);
            }
        }
    }
}

hipError_t launch_pair_conv(int logn, int st, const void *u, const void *w, const void *v,
                            void *out, const void *kbins, const float *kscale, const uint8_t *mask,
                            int64_t B, int64_t H, hipStream_t stream) {
    if (logn != 10 || st == ST_F32) return hipErrorInvalidValue;
    PairTables tb{};
    hipError_t e = get_pair_tables(&tb);
    if (e != hipSuccess) return e;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v_ = 0;
        if (hipDeviceGetAttribute(&v_, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v_ > 0)
            cus = v_;
    }
    const int64_t pairs = H * ((B + 1) / 2);
    int64_t blocks = (int64_t)cus;                           // one resident 4-wave workgroup per CU
    const int64_t need = (pairs + kPairWaves - 1) / kPairWaves;
    if (blocks > need) blocks = need < 8 ? 8 : (need + 7) / 8 * 8;
    if (st == ST_F16) {
        hipLaunchKernelGGL(pair1k_kernel<__half>, dim3((unsigned)blocks), dim3(64 * kPairWaves), 0,
                           stream, (const __half *)u, (const __half *)w, (const __half *)v,
                           (__half *)out, (const uint4 *)kbins, kscale, mask, tb, B, H);
    } else {
        hipLaunchKernelGGL(pair1k_kernel<__hip_bfloat16>, dim3((unsigned)blocks),
                           dim3(64 * kPairWaves), 0, stream, (const __hip_bfloat16 *)u,
                           (const __hip_bfloat16 *)w, (const __hip_bfloat16 *)v,
                           (__hip_bfloat16 *)out, (const uint4 *)kbins, kscale, mask, tb, B, H);
    }
    return hipGetLastError();
}

}  // namespace fftconv
