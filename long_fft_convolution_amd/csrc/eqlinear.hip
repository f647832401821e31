// eqlinear.hip -- circular convolution along a group axis composed with a
// channel linear map (the Flash EQ-Linear abstract page: the equivariant
// linear layer is exactly this, and the Fourier convolution theorem along the
// group dimension with the real DFT's conjugate symmetry makes it cheaper):
//
//   y[n, t, d] = sum_{s < T} sum_{c} W[s, d, c] x[n, (t - s) mod T, c]
//
// With X_f = sum_t x[t] w_T^{tf} and W_f = sum_s W[s] w_T^{sf}, Y_f = W_f X_f for
// f = 0 .. T/2 (the other half is conjugate), and y is the inverse real DFT.
// Per frequency the channel map is a dense complex product, done on the MFMA
// matrix cores (v_mfma_f32_16x16x32_f16, fp16 operands, fp32 accumulation);
// the small DFTs along the group axis run on the VALU and never leave the chip.
//
// Workgroup: 16 tokens x DSPAN = 64 output channels, 4 waves; wave w owns the
// column tile [16 w, 16 w + 16) of the span.  One tile per wave keeps the
// accumulators of all T/2 + 1 frequencies small enough for four waves per
// SIMD, which measured 20 % faster than two tiles per wave at two waves per
// SIMD (and than 64-token workgroups that read each weight fragment once per
// 64 tokens: the weight reads from L2 are not the limit).
//   A  per chunk of 32 input channels: the real DFT of the 16 tokens' group
//      rows (one channel pair per lane), written to LDS as the fp16 operand
//      rows of every frequency (double-buffered, one barrier per chunk);
//   B  per frequency: real (f = 0, T/2) or complex (4 products) 16x16x32 tiles
//      against the transformed weights read from global memory (L2-resident);
//   C  the inverse real DFT of each accumulator element, staged in LDS and
//      stored as rows of DSPAN contiguous channels.
#include "fft_device.hpp"
#include "fftconv_internal.hpp"
#include "cmfma.hpp"

#include <type_traits>

namespace fftconv {
namespace eq {
using namespace cmfma;

template <typename S> struct st;
template <> struct st<__half> {
    static __device__ __forceinline__ float2 ld2(const __half *p) {
        return __half22float2(*reinterpret_cast<const __half2 *>(p));
    }
    static __device__ __forceinline__ uint16_t bits(float v) {
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    }
};
template <> struct st<__hip_bfloat16> {
    static __device__ __forceinline__ float2 ld2(const __hip_bfloat16 *p) {
        const uint32_t b = *reinterpret_cast<const uint32_t *>(p);
        return make_float2(__uint_as_float(b << 16), __uint_as_float(b & 0xffff0000u));
    }
    static __device__ __forceinline__ uint16_t bits(float v) {
        const __hip_bfloat16 h = __float2bfloat16(v);
        return __builtin_bit_cast(uint16_t, h);
    }
};

template <int T> struct Plan {
    static constexpr int NF = T / 2 + 1;             // frequencies 0 .. T/2
    static constexpr int NT = 1;                     // one column tile of 16 per wave (occupancy)
    static constexpr int DSPAN = 4 * 16 * NT;        // output channels per workgroup
    static constexpr size_t kXBytes = (size_t)2 * NF * 2 * 16 * 32 * 2;    // [buf][f][plane][token][32] fp16
    static constexpr size_t kYBytes = (size_t)16 * T * DSPAN * 2;         // [token][t][DSPAN] storage
    static constexpr size_t kLds = kXBytes > kYBytes ? kXBytes : kYBytes;
};

// a * w_T^q for a compile-time q
template <int T>
__device__ __forceinline__ float2 rot(float2 a, int q) {
    return twiddle_const<T>(a, q % T);
}
}  // namespace eq

// Weights W (T, C_out, C_in) -> W_f planes [f][re, im][C_out][C_in] fp16, f <= T/2,
// scaled by 1/T (the inverse DFT's factor).  One thread per (d, c).
template <int T, typename S>
__global__ void __launch_bounds__(256)
eqlinear_prepare_kernel(const S *__restrict__ W, _Float16 *__restrict__ Wf, int64_t Cout, int64_t Cin) {
    using P = eq::Plan<T>;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t DC = Cout * Cin;
    if (i >= DC) return;
    float ws[T];
#pragma unroll
    for (int s = 0; s < T; ++s) {
        const S v = W[s * DC + i];
        ws[s] = std::is_same<S, __half>::value ? __half2float(*reinterpret_cast<const __half *>(&v))
                                               : __bfloat162float(*reinterpret_cast<const __hip_bfloat16 *>(&v));
    }
#pragma unroll
    for (int f = 0; f < P::NF; ++f) {
        float2 acc = make_float2(0.f, 0.f);
#pragma unroll
        for (int s = 0; s < T; ++s) acc = cadd(acc, eq::rot<T>(make_float2(ws[s], 0.f), s * f));
        Wf[(2 * f + 0) * DC + i] = (_Float16)(acc.x * (1.0f / T));
        Wf[(2 * f + 1) * DC + i] = (_Float16)(acc.y * (1.0f / T));
    }
}

// grid: 8 D ceil(N / 128) workgroups (D = ceil(C_out / DSPAN)); block 256; dynamic LDS Plan<T>::kLds
template <int T, typename S>
__global__ void __launch_bounds__(256)
eqlinear_kernel(const S *__restrict__ x, const _Float16 *__restrict__ Wf, S *__restrict__ y, int64_t Ntok,
                int64_t Cin, int64_t Cout) {
    using namespace eq;
    using P = Plan<T>;
    constexpr int NF = P::NF, NT = P::NT, DSPAN = P::DSPAN;
    extern __shared__ __align__(16) _Float16 smem[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, c = lane & 15;
    // 1-D grid: workgroup L runs on XCD L % 8; the D output-channel spans of one
    // token tile are L, L + 8, ..., so they share an XCD and its L2 and x is
    // read from HBM once per tile
    const uint32_t L = blockIdx.x, q = L / 8, D = (uint32_t)((Cout + DSPAN - 1) / DSPAN);
    const int64_t tt = (int64_t)(q / D) * 8 + (L % 8);
    if (tt * 16 >= Ntok) return;   // (whole workgroup: before any barrier)
    const int64_t n0 = tt * 16;
    const int64_t d0 = (int64_t)(q % D) * DSPAN;
    const int64_t dw = d0 + 16 * NT * wave;              // this wave's first output channel
    const bool active = dw < Cout;                       // (C_out is a multiple of 16 NT)
    const int64_t DC = Cout * Cin;
    const int nchunk = (int)(Cin / 32);

    // ---- A: the real DFT along the group axis of one chunk, into LDS buffer b
    const int tok = tid >> 4, cp = tid & 15;
    const int64_t n = n0 + tok;
    const int64_t nsafe = n < Ntok ? n : Ntok - 1;
    // raw input of one chunk (two channels per lane, T group elements), loaded a
    // chunk ahead so that the loads overlap the previous chunk's products
    typedef uint32_t Raw[T];
    auto load_a = [&](int kc, Raw &raw) {
#pragma unroll
        for (int t = 0; t < T; ++t)
            raw[t] = *reinterpret_cast<const uint32_t *>(x + (nsafe * T + t) * Cin + 32 * kc + 2 * cp);
    };
    auto stage_a = [&](const Raw &raw, int b) {
        float2 xv[T];
#pragma unroll
        for (int t = 0; t < T; ++t) xv[t] = st<S>::ld2(reinterpret_cast<const S *>(&raw[t]));
        if (n >= Ntok) {
#pragma unroll
            for (int t = 0; t < T; ++t) xv[t] = make_float2(0.f, 0.f);
        }
        // the two channels as one complex sequence z = x0 + i x1: one T-point DFT,
        // then X0[f] = (Z[f] + conj Z[T-f]) / 2, X1[f] = (Z[f] - conj Z[T-f]) / 2i
        float2 zf[T];
        Dft<T>::run(xv, zf);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const float2 za = zf[f], zb = cconj(zf[(T - f) % T]);
            const float2 a0 = cscale(cadd(za, zb), 0.5f);
            const float2 dd = csub(za, zb);
            const float2 a1 = make_float2(0.5f * dd.y, -0.5f * dd.x);
            _Float16 *pr = smem + (((b * NF + f) * 2 + 0) * 16 + tok) * 32 + 2 * cp;
            _Float16 *pi = smem + (((b * NF + f) * 2 + 1) * 16 + tok) * 32 + 2 * cp;
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<h2 *>(pr) = h2{(_Float16)a0.x, (_Float16)a1.x};
            *reinterpret_cast<h2 *>(pi) = h2{(_Float16)a0.y, (_Float16)a1.y};
        }
    };

    f4 accr[NF][NT], acci[NF][NT];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            accr[f][j] = f4{0.f, 0.f, 0.f, 0.f};
            acci[f][j] = f4{0.f, 0.f, 0.f, 0.f};
        }

    Raw raw;
    load_a(0, raw);
    stage_a(raw, 0);
    __syncthreads();
    for (int kc = 0; kc < nchunk; ++kc) {
        const int b = kc & 1;
        if (kc + 1 < nchunk) load_a(kc + 1, raw);
        if (active) {
            // ---- B: per frequency, rows = tokens (A from LDS), columns = output channels
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const bool cplx = f != 0 && 2 * f != T;
                const h8 ar = *reinterpret_cast<const h8 *>(smem + (((b * NF + f) * 2 + 0) * 16 + c) * 32 + 8 * g);
                h8 ai{};
                if (cplx) ai = *reinterpret_cast<const h8 *>(smem + (((b * NF + f) * 2 + 1) * 16 + c) * 32 + 8 * g);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int64_t d = dw + 16 * j + c;
                    const uint32_t eo = (uint32_t)(2 * (d * Cin + 32 * kc + 8 * g));
                    const h8 wr = ldu<h8>(Wf + (2 * f) * DC, eo);
                    accr[f][j] = mfma(ar, wr, accr[f][j]);
                    if (cplx) {
                        const h8 wi = ldu<h8>(Wf + (2 * f + 1) * DC, eo);
                        accr[f][j] = mfma(neg8(ai), wi, accr[f][j]);
                        acci[f][j] = mfma(ar, wi, acci[f][j]);
                        acci[f][j] = mfma(ai, wr, acci[f][j]);
                    }
                }
            }
        }
        // the next chunk's transform goes to the other buffer, which every wave
        // finished reading before the previous barrier
        if (kc + 1 < nchunk) stage_a(raw, b ^ 1);
        __syncthreads();
    }

    // ---- C: inverse real DFT per element (W_f carries the 1/T), staged as rows
    uint16_t *sy = reinterpret_cast<uint16_t *>(smem);   // [token][t][DSPAN]
    if (active) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int dl = 16 * NT * wave + 16 * j + c;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tk = 4 * g + i;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    float v = accr[0][j][i] + ((t & 1) ? -accr[NF - 1][j][i] : accr[NF - 1][j][i]);
#pragma unroll
                    for (int f = 1; f < NF - 1; ++f) {
                        // Re(Y_f exp(+2 pi i t f / T)) = Re(Y_f conj(w_T^{tf}))
                        const float2 e = rot<T>(make_float2(1.f, 0.f), t * f);   // cos - i sin
                        v += 2.f * (accr[f][j][i] * e.x + acci[f][j][i] * e.y);
                    }
                    sy[(tk * T + t) * DSPAN + dl] = st<S>::bits(v);
                }
            }
        }
    }
    __syncthreads();
    // rows of DSPAN channels: 16 tokens x T rows; each lane stores 8 channels (16 bytes)
    constexpr int kRowLanes = DSPAN / 8;
    const int64_t dvalid = Cout - d0 < DSPAN ? Cout - d0 : DSPAN;
    for (int r = tid / kRowLanes; r < 16 * T; r += 256 / kRowLanes) {
        const int tk = r / T, t = r - tk * T;
        const int dl = 8 * (tid % kRowLanes);
        const int64_t nn = n0 + tk;
        if (nn < Ntok && dl < dvalid) {
            const uint4 q = *reinterpret_cast<const uint4 *>(sy + r * DSPAN + dl);
            stnt<uint4>(y + (nn * T + t) * Cout + d0 + dl, q);   // (written once: streaming)
        }
    }
}

// ---- fp32 storage: the same operator with fp32 arithmetic throughout ----------
// (the Flash EQ-Linear abstract page: the layer is provided in both FP32 and FP16
// precision).  The per-frequency channel products run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: A lane l holds row l % 16 at K slot l / 16, B column
// l % 16 at K slot l / 16).  Per chunk of 32 input channels the K index is
// permuted: MFMA step k of lane group g contracts channel 8 g + k, so each lane
// reads its eight channels of a token (A, from LDS) and of an output channel (B,
// the weights, L2-resident) as two 16-byte words.  Workgroup: 16 tokens x 64
// output channels, four waves of one 16-channel column tile.
namespace eq {
template <int T> struct Plan32 {
    static constexpr int NF = T / 2 + 1;
    static constexpr int DSPAN = 64;
    static constexpr size_t kXBytes = (size_t)2 * NF * 2 * 16 * 32 * 4;   // [buf][f][plane][token][32] fp32
    static constexpr size_t kYBytes = (size_t)16 * T * DSPAN * 4;        // [token][t][DSPAN] fp32
    static constexpr size_t kLds = kXBytes > kYBytes ? kXBytes : kYBytes;
};
__device__ __forceinline__ f4 mfma32(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
}  // namespace eq

// W (T, C_out, C_in) fp32 -> W_f planes [f][re, im][C_out][C_in] fp32, f <= T/2, scaled by 1/T
template <int T>
__global__ void __launch_bounds__(256)
eqlinear_prepare32_kernel(const float *__restrict__ W, float *__restrict__ Wf, int64_t Cout, int64_t Cin) {
    using P = eq::Plan32<T>;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t DC = Cout * Cin;
    if (i >= DC) return;
    float ws[T];
#pragma unroll
    for (int s = 0; s < T; ++s) ws[s] = W[s * DC + i];
#pragma unroll
    for (int f = 0; f < P::NF; ++f) {
        float2 acc = make_float2(0.f, 0.f);
#pragma unroll
        for (int s = 0; s < T; ++s) acc = cadd(acc, eq::rot<T>(make_float2(ws[s], 0.f), s * f));
        Wf[(2 * f + 0) * DC + i] = acc.x * (1.0f / T);
        Wf[(2 * f + 1) * DC + i] = acc.y * (1.0f / T);
    }
}

// grid and workgroup order as eqlinear_kernel; dynamic LDS Plan32<T>::kLds
template <int T>
__global__ void __launch_bounds__(256)
eqlinear32_kernel(const float *__restrict__ x, const float *__restrict__ Wf, float *__restrict__ y, int64_t Ntok,
                  int64_t Cin, int64_t Cout) {
    using namespace eq;
    using P = Plan32<T>;
    constexpr int NF = P::NF, DSPAN = P::DSPAN;
    extern __shared__ __align__(16) float smem32[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, c = lane & 15;
    const uint32_t L = blockIdx.x, q = L / 8, D = (uint32_t)((Cout + DSPAN - 1) / DSPAN);
    const int64_t tt = (int64_t)(q / D) * 8 + (L % 8);
    if (tt * 16 >= Ntok) return;   // (whole workgroup: before any barrier)
    const int64_t n0 = tt * 16;
    const int64_t d0 = (int64_t)(q % D) * DSPAN;
    const int64_t dw = d0 + 16 * wave;
    const bool active = dw < Cout;
    const int64_t DC = Cout * Cin;
    const int nchunk = (int)(Cin / 32);

    // ---- A: two channels per lane (token tok, channels 2 cp, 2 cp + 1), one complex
    // T-point DFT, split by conjugate symmetry; LDS [buf][f][plane][token][32]
    const int tok = tid >> 4, cp = tid & 15;
    const int64_t n = n0 + tok;
    const int64_t nsafe = n < Ntok ? n : Ntok - 1;
    typedef float2 Raw[T];
    auto load_a = [&](int kc, Raw &raw) {
#pragma unroll
        for (int t = 0; t < T; ++t)
            raw[t] = *reinterpret_cast<const float2 *>(x + (nsafe * T + t) * Cin + 32 * kc + 2 * cp);
    };
    auto stage_a = [&](const Raw &raw, int b) {
        float2 xv[T];
#pragma unroll
        for (int t = 0; t < T; ++t) xv[t] = n < Ntok ? raw[t] : make_float2(0.f, 0.f);
        float2 zf[T];
        Dft<T>::run(xv, zf);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const float2 za = zf[f], zb = cconj(zf[(T - f) % T]);
            const float2 a0 = cscale(cadd(za, zb), 0.5f);
            const float2 dd = csub(za, zb);
            const float2 a1 = make_float2(0.5f * dd.y, -0.5f * dd.x);
            float *pr = smem32 + (((b * NF + f) * 2 + 0) * 16 + tok) * 32 + 2 * cp;
            float *pi = smem32 + (((b * NF + f) * 2 + 1) * 16 + tok) * 32 + 2 * cp;
            *reinterpret_cast<float2 *>(pr) = make_float2(a0.x, a1.x);
            *reinterpret_cast<float2 *>(pi) = make_float2(a0.y, a1.y);
        }
    };

    f4 accr[NF], acci[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        accr[f] = f4{0.f, 0.f, 0.f, 0.f};
        acci[f] = f4{0.f, 0.f, 0.f, 0.f};
    }
    Raw raw;
    load_a(0, raw);
    stage_a(raw, 0);
    __syncthreads();
    for (int kc = 0; kc < nchunk; ++kc) {
        const int b = kc & 1;
        if (kc + 1 < nchunk) load_a(kc + 1, raw);
        if (active) {
            // ---- B: per frequency, rows = tokens (A, LDS), columns = output channels (B, weights)
            const int64_t d = dw + c;
            const float *wrow = Wf + d * Cin + 32 * kc + 8 * g;
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const bool cplx = f != 0 && 2 * f != T;
                const float *ap = smem32 + (((b * NF + f) * 2 + 0) * 16 + c) * 32 + 8 * g;
                const float4 ar0 = *reinterpret_cast<const float4 *>(ap), ar1 = *reinterpret_cast<const float4 *>(ap + 4);
                const float4 wr0 = ldu<float4>(wrow + (2 * f) * DC, 0u), wr1 = ldu<float4>(wrow + (2 * f) * DC, 16u);
                const float ar[8] = {ar0.x, ar0.y, ar0.z, ar0.w, ar1.x, ar1.y, ar1.z, ar1.w};
                const float wr[8] = {wr0.x, wr0.y, wr0.z, wr0.w, wr1.x, wr1.y, wr1.z, wr1.w};
                if (!cplx) {
#pragma unroll
                    for (int k = 0; k < 8; ++k) accr[f] = mfma32(ar[k], wr[k], accr[f]);
                } else {
                    const float *aq = ap + 16 * 32;   // imaginary plane
                    const float4 ai0 = *reinterpret_cast<const float4 *>(aq), ai1 = *reinterpret_cast<const float4 *>(aq + 4);
                    const float4 wi0 = ldu<float4>(wrow + (2 * f + 1) * DC, 0u), wi1 = ldu<float4>(wrow + (2 * f + 1) * DC, 16u);
                    const float ai[8] = {ai0.x, ai0.y, ai0.z, ai0.w, ai1.x, ai1.y, ai1.z, ai1.w};
                    const float wi[8] = {wi0.x, wi0.y, wi0.z, wi0.w, wi1.x, wi1.y, wi1.z, wi1.w};
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        accr[f] = mfma32(ar[k], wr[k], accr[f]);
                        accr[f] = mfma32(-ai[k], wi[k], accr[f]);
                        acci[f] = mfma32(ar[k], wi[k], acci[f]);
                        acci[f] = mfma32(ai[k], wr[k], acci[f]);
                    }
                }
            }
        }
        if (kc + 1 < nchunk) stage_a(raw, b ^ 1);
        __syncthreads();
    }

    // ---- C: inverse real DFT per element (W_f carries the 1/T), staged as fp32 rows
    float *sy = smem32;   // [token][t][DSPAN]
    if (active) {
        const int dl = 16 * wave + c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tk = 4 * g + i;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                float v = accr[0][i] + ((t & 1) ? -accr[NF - 1][i] : accr[NF - 1][i]);
#pragma unroll
                for (int f = 1; f < NF - 1; ++f) {
                    const float2 e = rot<T>(make_float2(1.f, 0.f), t * f);   // cos - i sin
                    v += 2.f * (accr[f][i] * e.x + acci[f][i] * e.y);
                }
                sy[(tk * T + t) * DSPAN + dl] = v;
            }
        }
    }
    __syncthreads();
    // rows of DSPAN channels: 16 tokens x T rows; each lane stores 4 channels (16 bytes)
    constexpr int kRowLanes = DSPAN / 4;
    const int64_t dvalid = Cout - d0 < DSPAN ? Cout - d0 : DSPAN;
    for (int r = tid / kRowLanes; r < 16 * T; r += 256 / kRowLanes) {
        const int tk = r / T, t = r - tk * T;
        const int dl = 4 * (tid % kRowLanes);
        const int64_t nn = n0 + tk;
        if (nn < Ntok && dl < dvalid) {
            const float4 qv = *reinterpret_cast<const float4 *>(sy + r * DSPAN + dl);
            stnt<float4>(y + (nn * T + t) * Cout + d0 + dl, qv);   // (written once: streaming)
        }
    }
}

template <int T>
static hipError_t eq_launch32(const void *x, const void *Wf, void *y, int64_t Ntok, int64_t Cin, int64_t Cout,
                              hipStream_t stream) {
    using P = eq::Plan32<T>;
    auto k = eqlinear32_kernel<T>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)P::kLds);
    if (e != hipSuccess) return e;
    const int64_t D = (Cout + P::DSPAN - 1) / P::DSPAN, tiles = (Ntok + 15) / 16;
    const dim3 grid((unsigned)(((tiles + 7) / 8) * 8 * D));
    hipLaunchKernelGGL(k, grid, dim3(256), P::kLds, stream, (const float *)x, (const float *)Wf, (float *)y, Ntok,
                       Cin, Cout);
    return hipGetLastError();
}

template <int T>
static hipError_t eq_prepare32(const void *W, void *Wf, int64_t Cout, int64_t Cin, hipStream_t stream) {
    const int64_t n = Cout * Cin;
    hipLaunchKernelGGL((eqlinear_prepare32_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (const float *)W, (float *)Wf, Cout, Cin);
    return hipGetLastError();
}

template <int T, typename S>
static hipError_t eq_launch(const void *x, const void *Wf, void *y, int64_t Ntok, int64_t Cin, int64_t Cout,
                            hipStream_t stream) {
    using P = eq::Plan<T>;
    auto k = eqlinear_kernel<T, S>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)P::kLds);
    if (e != hipSuccess) return e;
    const int64_t D = (Cout + P::DSPAN - 1) / P::DSPAN, tiles = (Ntok + 15) / 16;
    const dim3 grid((unsigned)(((tiles + 7) / 8) * 8 * D));
    hipLaunchKernelGGL(k, grid, dim3(256), P::kLds, stream, (const S *)x, (const _Float16 *)Wf, (S *)y, Ntok,
                       Cin, Cout);
    return hipGetLastError();
}

template <int T, typename S>
static hipError_t eq_prepare(const void *W, void *Wf, int64_t Cout, int64_t Cin, hipStream_t stream) {
    const int64_t n = Cout * Cin;
    hipLaunchKernelGGL((eqlinear_prepare_kernel<T, S>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (const S *)W, (_Float16 *)Wf, Cout, Cin);
    return hipGetLastError();
}

int eqlinear_span(int T) {
    switch (T) {
    case 4: return eq::Plan<4>::DSPAN;
    case 8: return eq::Plan<8>::DSPAN;
    case 16: return eq::Plan<16>::DSPAN;
    default: return 0;
    }
}

hipError_t launch_eqlinear_prepare(int st, int T, const void *W, void *Wf, int64_t Cout, int64_t Cin,
                                   hipStream_t stream) {
    if (st == ST_F32) {
        switch (T) {
        case 4: return eq_prepare32<4>(W, Wf, Cout, Cin, stream);
        case 8: return eq_prepare32<8>(W, Wf, Cout, Cin, stream);
        case 16: return eq_prepare32<16>(W, Wf, Cout, Cin, stream);
        default: return hipErrorInvalidValue;
        }
    }
    const bool h = st == ST_F16;
    switch (T) {
    case 4: return h ? eq_prepare<4, __half>(W, Wf, Cout, Cin, stream)
                     : eq_prepare<4, __hip_bfloat16>(W, Wf, Cout, Cin, stream);
    case 8: return h ? eq_prepare<8, __half>(W, Wf, Cout, Cin, stream)
                     : eq_prepare<8, __hip_bfloat16>(W, Wf, Cout, Cin, stream);
    case 16: return h ? eq_prepare<16, __half>(W, Wf, Cout, Cin, stream)
                      : eq_prepare<16, __hip_bfloat16>(W, Wf, Cout, Cin, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_eqlinear(int st, int T, const void *x, const void *Wf, void *y, int64_t Ntok, int64_t Cin,
                           int64_t Cout, hipStream_t stream) {
    if (st == ST_F32) {
        switch (T) {
        case 4: return eq_launch32<4>(x, Wf, y, Ntok, Cin, Cout, stream);
        case 8: return eq_launch32<8>(x, Wf, y, Ntok, Cin, Cout, stream);
        case 16: return eq_launch32<16>(x, Wf, y, Ntok, Cin, Cout, stream);
        default: return hipErrorInvalidValue;
        }
    }
    const bool h = st == ST_F16;
    switch (T) {
    case 4: return h ? eq_launch<4, __half>(x, Wf, y, Ntok, Cin, Cout, stream)
                     : eq_launch<4, __hip_bfloat16>(x, Wf, y, Ntok, Cin, Cout, stream);
    case 8: return h ? eq_launch<8, __half>(x, Wf, y, Ntok, Cin, Cout, stream)
                     : eq_launch<8, __hip_bfloat16>(x, Wf, y, Ntok, Cin, Cout, stream);
    case 16: return h ? eq_launch<16, __half>(x, Wf, y, Ntok, Cin, Cout, stream)
                      : eq_launch<16, __hip_bfloat16>(x, Wf, y, Ntok, Cin, Cout, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fftconv
