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
//  * Twiddles and the filter product are packed fp16 on the VALU between
//    stages (the stored spectrum is scaled so |K| <= 1; the per-channel fp32
//    scale is applied to the fp32 result of the last stage).
//
// One wave owns one sequence pair at a time and loops over pairs
// (persistent), prefetching the next pair's inputs, filter and gate chunks;
// twiddles and two of the three DFT block sets live in LDS so that two
// workgroups of four waves fit per CU.
#include "cmfma.hpp"
#include "fft_device.hpp"
#include "fftconv_internal.hpp"

#include <type_traits>

namespace fftconv {

using cmfma::f4;
using cmfma::h4;
using cmfma::h8;
using cmfma::cat8;
using cmfma::cmul4;
using cmfma::hi4;
using cmfma::lo4;
using cmfma::mfma;
using cmfma::neg8;
using cmfma::to_h4;

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
    static __device__ __forceinline__ void unpack4(const uint2 &raw, float *o) {
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
    static __device__ __forceinline__ uint4 pack8(const float *v) {
        _Float16 hv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = (_Float16)v[i];
        return *reinterpret_cast<const uint4 *>(hv);
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
    static __device__ __forceinline__ void unpack4(const uint2 &raw, float *o) {
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
    static __device__ __forceinline__ uint4 pack8(const float *v) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __hip_bfloat16 a = __float2bfloat16(v[2 * i]), b = __float2bfloat16(v[2 * i + 1]);
            w[i] = (uint32_t)(*reinterpret_cast<uint16_t *>(&a)) |
                   ((uint32_t)(*reinterpret_cast<uint16_t *>(&b)) << 16);
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
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

// raw 16-byte input chunks of one pair: [u_a, w_a, u_b, w_b] x [r = 0, 1]
struct PairRaw {
    uint4 q[2][4];
};
// windowed pair: [block A, B, C] x [r = 0, 1] x [u, w]
struct WinRaw {
    uint4 q[3][2][2];
};

// (without a second row ob == oa: the loads re-read the first row and the caller zeroes
// the result, so that no load sits under a branch)
template <typename T, bool HAS_W>
__device__ __forceinline__ void load_pair_raw(PairRaw &raw, const T *__restrict__ u,
                                              const T *__restrict__ w, int64_t oa, int64_t ob, int lane) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int m0 = 8 * lane + 512 * r;
        raw.q[r][0] = ldnt<uint4>(u + oa + m0);
        raw.q[r][2] = ldnt<uint4>(u + ob + m0);
        if (HAS_W) {
            raw.q[r][1] = ldnt<uint4>(w + oa + m0);
            raw.q[r][3] = ldnt<uint4>(w + ob + m0);
        }
    }
}

template <typename T>
__device__ __forceinline__ void unpack8(const uint4 &q, float *o);
template <>
__device__ __forceinline__ void unpack8<__half>(const uint4 &q, float *o) {
    const _Float16 *hv = reinterpret_cast<const _Float16 *>(&q);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (float)hv[i];
}
template <>
__device__ __forceinline__ void unpack8<__hip_bfloat16>(const uint4 &q, float *o) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// xor of each 32-bit word of eight fp16 values with m (a sign pattern)
__device__ __forceinline__ h8 xor8(const h8 &a, uint32_t m) {
    uint4 q = *reinterpret_cast<const uint4 *>(&a);
    q.x ^= m;
    q.y ^= m;
    q.z ^= m;
    q.w ^= m;
    return *reinterpret_cast<const h8 *>(&q);
}

// x = u * w as eight fp16 values (w absent: x = u).  fp16 storage: one packed
// product (the fp16 product of two fp16 values, correctly rounded, equals the
// fp32 product rounded to fp16); bf16 storage: fp32 product rounded to fp16.
template <typename T>
__device__ __forceinline__ void gate_product(const uint4 &uq, const uint4 &wq, bool gated, h8 &x);
template <>
__device__ __forceinline__ void gate_product<__half>(const uint4 &uq, const uint4 &wq, bool gated, h8 &x) {
    const h8 uu = *reinterpret_cast<const h8 *>(&uq);
    x = gated ? uu * *reinterpret_cast<const h8 *>(&wq) : uu;
}
template <>
__device__ __forceinline__ void gate_product<__hip_bfloat16>(const uint4 &uq, const uint4 &wq, bool gated,
                                                             h8 &x) {
    float a[8], b[8];
    unpack8<__hip_bfloat16>(uq, a);
    if (gated) {
        unpack8<__hip_bfloat16>(wq, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] *= b[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (_Float16)a[e];
}

// The two rows of a pair share one complex transform, and every stage rounds to fp16 at
// the magnitude of the larger row.  zero_rows: a row that is all zero gets the output scale
// 0 (its result is exactly 0, not the rounding of its partner's), from one ballot.
// equalize_pair (channel pairs, where magnitudes differ more): also brings a much smaller
// row near the other: over the wave (one pair per wave) the maxima of |x_a| and |x_b| are
// compared, the smaller row is multiplied by 2^d (d one less than their exponent gap, at
// most 14: exact in fp16) and its output scale by 2^-d.
__device__ __forceinline__ void zero_rows(const h8 (&xa)[2], const h8 (&xb)[2], float &ksa, float &ksb) {
    uint32_t oa = 0, ob = 0;   // (sign bits cleared: a row of -0 is zero too)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const uint4 qa = *reinterpret_cast<const uint4 *>(&xa[r]), qb = *reinterpret_cast<const uint4 *>(&xb[r]);
        oa |= (qa.x | qa.y | qa.z | qa.w) & 0x7fff7fffu;
        ob |= (qb.x | qb.y | qb.z | qb.w) & 0x7fff7fffu;
    }
    if (__builtin_amdgcn_ballot_w64(oa != 0) == 0) ksa = 0.f;
    if (__builtin_amdgcn_ballot_w64(ob != 0) == 0) ksb = 0.f;
}
typedef unsigned short us2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ us2_t absmax2(const h8 &x, us2_t m) {
    // fp16 magnitudes compare as unsigned integers once the sign bit is cleared
    const uint4 q = *reinterpret_cast<const uint4 *>(&x);
    const us2_t a = __builtin_bit_cast(us2_t, q.x & 0x7fff7fffu), b = __builtin_bit_cast(us2_t, q.y & 0x7fff7fffu);
    const us2_t c = __builtin_bit_cast(us2_t, q.z & 0x7fff7fffu), d = __builtin_bit_cast(us2_t, q.w & 0x7fff7fffu);
    return __builtin_elementwise_max(__builtin_elementwise_max(m, __builtin_elementwise_max(a, b)),
                                     __builtin_elementwise_max(c, d));
}
__device__ __forceinline__ void equalize_pair(h8 (&xa)[2], h8 (&xb)[2], float &ksa, float &ksb) {
    us2_t pa = {0, 0}, pb = {0, 0};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        pa = absmax2(xa[r], pa);
        pb = absmax2(xb[r], pb);
    }
    uint32_t ma = pa[0] > pa[1] ? pa[0] : pa[1], mb = pb[0] > pb[1] ? pb[0] : pb[1];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t ta = (uint32_t)__shfl_xor((int)ma, o), tb = (uint32_t)__shfl_xor((int)mb, o);
        ma = ma > ta ? ma : ta;
        mb = mb > tb ? mb : tb;
    }
    if (ma == 0) ksa = 0.f;
    if (mb == 0) ksb = 0.f;
    if (ma != 0 && mb != 0) {
        int d = (int)(ma >> 10) - (int)(mb >> 10);   // exponent gap (fp16 biased exponents)
        const bool up_b = d > 0;
        d = (up_b ? d : -d) - 1;   // (the scaled maximum stays below the other one)
        d = d > 14 ? 14 : d;
        if (d > 0) {
            const _Float16 f = (_Float16)__builtin_ldexpf(1.f, d);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                if (up_b) xb[r] *= f;
                else xa[r] *= f;
            }
            if (up_b) ksb = __builtin_ldexpf(ksb, -d);
            else ksa = __builtin_ldexpf(ksa, -d);
        }
    }
}

// WIN: the chunked short-filter path (overlap-save with the transform's own
// length as the window).  The (B, H, NS) sequences, NS a multiple of 1024, are
// covered by windows of 2048 samples that overlap by half: window j holds the
// samples (j - 1) 1024 .. (j + 1) 1024 - 1 (zeros before the sequence start).
// Its 2048-point circular convolution with a filter of at most 1024 taps equals
// the linear one at the window's outputs 1024 .. 2047 (no tap reaches around
// the window), which are the outputs j 1024 .. j 1024 + 1023 of the sequence.
// The filter spectrum is the same 2048-point one as for N = 1024.  A pair is
// windows (2 jp, 2 jp + 1) of one sequence: three 1024-sample blocks A, B, C
// feed it (window a = A B, window b = B C; an odd last window has no b).
//   Relative to the N = 1024 path, S1 contracts all 64 values of n_s (the
// input fills the window: two K blocks, the second with DFT entries
// w64^{(n_s + 32) f_s} = (-1)^{f_s} w64^{n_s f_s}) and S1' produces n_s = 32 .. 63
// (entries conj w64^{f_s (n_s + 32)} = (-1)^{f_s} conj w64^{f_s n_s}).
// DUAL: the adjoint with two outputs, out = v corr(u w, k) and out2 = v2 corr(u w, k)
// from the same transforms: the product takes conj K, the stored spectrum conjugated
// as it is read (the backward pass forms du = w corr(v dy, k) and dw = u corr(v dy, k)
// in one call).
// CORR (windows only): the adjoint of the windowed convolution, out[t] = sum_s k[s] x[t + s]
// (the backward pass's corr(v dy, k) for the short filter).  Output block j needs the
// input blocks j and j + 1: window j holds the samples j 1024 .. (j + 2) 1024 - 1 (zeros
// past the sequence end), its 2048-point circular correlation with the filter,
// IDFT(DFT(window) conj K), has no wrap-around at the outputs 0 .. 1023, so S1' takes the
// unflipped entries of the N = 1024 path and the filter product the conjugated spectrum.
// A pair is windows (2 jp, 2 jp + 1) fed by the blocks A = 2 jp, B = 2 jp + 1, C = 2 jp + 2.
// LONE (not windows): the last batch row b = B - 1 of an odd B, whose rows would otherwise
// each pair with zeros.  A pair is two channels h = 2q, h' = 2q + 1 of that row (h' = h
// without a partner: H odd): z = x_h + i x_h'.  With the real filters' stored spectra K, K'
// and Z the transform of z, X_h = (Z(f) + conj Z(-f)) / 2 and i X_h' = (Z(f) - conj Z(-f)) / 2,
// so the product that yields y_h + i y_h' is
//   Y(f) = Z(f) (K + K') / 2 + conj Z(-f) (K - K') / 2.
// The bins of Z pass through the wave's LDS to bring Z(-f) to the lane holding Z(f); the
// real part of the result takes h's scale, the imaginary part h''s.
template <typename T, bool MASKED, bool HAS_W, bool HAS_V, bool WIN = false, bool DUAL = false,
          bool CORR = false, bool LONE = false>
__global__ void __launch_bounds__(64 * kPairWaves, MASKED ? 1 : 2)
pair1k_kernel(const T *__restrict__ u, const T *__restrict__ w, const T *__restrict__ v,
              T *__restrict__ out, const uint4 *__restrict__ kbins, const float *__restrict__ kscale,
              const uint8_t *__restrict__ mask, PairTables tb, int64_t B, int64_t H, int64_t NS,
              const T *__restrict__ v2, T *__restrict__ out2) {
    static_assert(!(WIN && MASKED), "the windowed path has no frequency mask");
    static_assert(!DUAL || (HAS_V && (!WIN || CORR)), "a second output has an output gate of its own");
    static_assert(!CORR || WIN, "the correlation mode is a windowed one");
    static_assert(!(LONE && WIN), "channel pairs are for the batch-row path");
    constexpr int N = 1024;
    __shared__ h8 s_tw1[2 * 4 * 64];     // per (mt, nt, lane): cos[4], sin[4]
    __shared__ h8 s_tw3[4 * 2 * 64];     // per (nt, nt2, lane)
    // per wave: the transposed input planes (2 x kPlane fp16), later the fp32 output rows
    // of both sequences (2 x 1024 floats)
    __shared__ __align__(16) float s_z[kPairWaves][2 * 1024];
    // input planes: rows n_f, K slots (two blocks of 32 in a window)
    constexpr int kRow = WIN ? 64 : 32, kPl = 32 * kRow;
    __shared__ h8 s_f1[2][4][64];     // S1 DFT blocks (re, im) per column tile nt
    __shared__ h8 s_f3[2][4][64];     // S1' DFT blocks (re, im) per (ks, nt3)

    const int tid = threadIdx.x;
    for (int i = tid; i < 512; i += 64 * kPairWaves) {
        s_tw1[i] = reinterpret_cast<const h8 *>(tb.tw1)[i];
        s_tw3[i] = reinterpret_cast<const h8 *>(tb.tw3)[i];
    }
    for (int i = tid; i < 256; i += 64 * kPairWaves) {
        s_f1[0][i / 64][i % 64] = reinterpret_cast<const h8 *>(tb.f1r)[i];
        s_f1[1][i / 64][i % 64] = reinterpret_cast<const h8 *>(tb.f1i)[i];
        // windows: S1' produces n_s + 32, i.e. the entries of the odd K slots (odd f_s:
        // element j odd, the upper half of each 32-bit word) change sign
        uint4 a = reinterpret_cast<const uint4 *>(tb.f3r)[i], b = reinterpret_cast<const uint4 *>(tb.f3i)[i];
        if (WIN && !CORR) {
            a = make_uint4(a.x ^ 0x80000000u, a.y ^ 0x80000000u, a.z ^ 0x80000000u, a.w ^ 0x80000000u);
            b = make_uint4(b.x ^ 0x80000000u, b.y ^ 0x80000000u, b.z ^ 0x80000000u, b.w ^ 0x80000000u);
        }
        s_f3[0][i / 64][i % 64] = *reinterpret_cast<const h8 *>(&a);
        s_f3[1][i / 64][i % 64] = *reinterpret_cast<const h8 *>(&b);
    }
    __syncthreads();

    // the wave index is uniform: keep pair bookkeeping and addresses scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, c = lane & 15;
    const h8 *F2r = reinterpret_cast<const h8 *>(tb.f2r), *F2i = reinterpret_cast<const h8 *>(tb.f2i);
    h8 c2r[2], c2i[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        c2r[t] = F2r[t * 64 + lane];
        c2i[t] = F2i[t * 64 + lane];
    }

    // Pair index spaces.  Windows: p = h PB + bp (window pairs of one sequence fastest:
    // neighbouring waves read neighbouring memory); each XCD walks one contiguous range.
    // Batch-row pairs: with H >= 8 each XCD owns the channels [h0, h0 + Hx) and walks
    // p = bp Hx + (h - h0), the channel fastest, so that the waves in flight read the
    // contiguous rows of neighbouring channels while the XCD's filter spectra stay in its
    // L2 (with the batch fastest, neighbouring waves read rows 2 H N elements apart and
    // the HBM pages are poorly used); with H < 8 the XCDs split p = bp H + h.
    const int64_t NW = NS / 1024, JP = (NW + 1) / 2;            // windows, window pairs per sequence
    const int64_t PB = WIN ? B * JP : (B + 1) / 2;               // pairs per channel
    const int64_t P = LONE ? (H + 1) / 2 : H * PB;
    const uint32_t nwg = gridDim.x, xcd = blockIdx.x % 8, wg_local = blockIdx.x / 8;
    const uint32_t wg_on_xcd = nwg / 8 + (xcd < nwg % 8 ? 1u : 0u);
    int64_t p_begin, p_end, h0 = 0, Hx = H;
    if (!WIN && !LONE && H >= 8) {
        h0 = H * xcd / 8;
        Hx = H * (xcd + 1) / 8 - h0;
        p_begin = 0;
        p_end = Hx * PB;
    } else {
        p_begin = P * xcd / 8;
        p_end = P * (xcd + 1) / 8;
    }
    const int64_t stride = (int64_t)wg_on_xcd * kPairWaves;
    _Float16 *zr = reinterpret_cast<_Float16 *>(s_z[wave]), *zi = zr + kPl;
    char *const so = reinterpret_cast<char *>(s_z[wave]);
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // (the host keeps the pair count below 2^31: 32-bit divisions).  oa, ob: where the
    // outputs (and output gates) of sequence / window a and b start; without b, ob == oa.
    // edge: a window pair at the sequence start (its block A lies before it), with CORR one
    // at the sequence end (its block C lies past it)
    auto offsets = [&](int64_t p, int64_t &h, int64_t &oa, int64_t &ob, bool &has_b, bool &edge) {
        int64_t bp;
        if (LONE) {   // channels 2 p, 2 p + 1 of the last batch row
            h = 2 * p;
            has_b = 2 * p + 1 < H;
            edge = false;
            oa = ((B - 1) * H + h) * N;
            ob = has_b ? oa + N : oa;
            return;
        }
        if (WIN) {
            const uint32_t h32 = (uint32_t)p / (uint32_t)PB;
            h = h32;
            bp = (uint32_t)p - h32 * (uint32_t)PB;
        } else {
            const uint32_t b32 = (uint32_t)p / (uint32_t)Hx;
            bp = b32;
            h = h0 + ((uint32_t)p - b32 * (uint32_t)Hx);
        }
        if (WIN) {
            // window pair jp of batch row b: windows 2 jp and 2 jp + 1, outputs at 2 jp 1024
            // and (2 jp + 1) 1024
            const uint32_t b32 = (uint32_t)bp / (uint32_t)JP;
            const int64_t b = b32, jp = (uint32_t)bp - b32 * (uint32_t)JP;
            has_b = 2 * jp + 1 < NW;
            edge = CORR ? 2 * jp + 2 >= NW : jp == 0;
            oa = (b * H + h) * NS + 2 * jp * 1024;
            ob = has_b ? oa + 1024 : oa;
        } else {
            has_b = 2 * bp + 1 < B;
            edge = false;
            oa = (2 * bp * H + h) * N;
            ob = has_b ? oa + H * N : oa;
        }
    };

    // per-pair side data: the filter chunks with the channel scale, and the output-gate rows
    // (contiguous 16-byte chunks in the order the output is stored)
    struct Filt {
        uint4 k[2][4];
        float ks;
        float ks2;   // LONE: the second channel's scale (its chunks are read where used)
    };
    auto load_filt = [&](int64_t pp, Filt &fk) {
        int64_t h, oa, ob;
        bool hb, fst;
        offsets(pp, h, oa, ob, hb, fst);
        const uint4 *krow = kbins + h * 512;
        if (!LONE) {
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) fk.k[mt2][nt] = krow[(mt2 * 4 + nt) * 64 + lane];
        }
        // (the four stages' table factors are undone with the channel scale)
        fk.ks = __builtin_ldexpf(kscale[h], 2 * (kPairS1Log2 + kPairS2Log2));
        if (LONE) fk.ks2 = __builtin_ldexpf(kscale[hb ? h + 1 : h], 2 * (kPairS1Log2 + kPairS2Log2));
        if (CORR || DUAL) {   // conj K: the sign of the imaginary half (elements 4..7) of every chunk
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    fk.k[mt2][nt].z ^= 0x80008000u;
                    fk.k[mt2][nt].w ^= 0x80008000u;
                }
        }
    };
    auto load_gate = [&](const T *gp, int64_t oa, int64_t ob, uint4 (&vg)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            vg[q] = ldnt<uint4>(gp + (q < 2 ? oa : ob) + 512 * (q & 1) + 8 * lane);   // (read once: streaming)
    };
    using Raw = std::conditional_t<WIN, WinRaw, PairRaw>;
    auto load_in = [&](int64_t pp, Raw &raw) {
        int64_t h, oa, ob;
        bool hb, fst;
        offsets(pp, h, oa, ob, hb, fst);
        if constexpr (WIN) {
            // blocks A = [oa - 1024, oa) (before the sequence start for the first pair: the
            // load re-reads B and its product is zeroed), B = [oa, oa + 1024), C = [oa + 1024, oa + 2048):
            // without window b, C re-reads B (its results are not stored).  CORR: A = [oa, ..),
            // B = [oa + 1024, ..), C = [oa + 2048, ..); a block past the sequence end re-reads A
            // and its product is zeroed
            const int64_t oA = CORR ? oa : (fst ? oa : oa - 1024);
            const int64_t oB = CORR ? (hb ? oa + 1024 : oa) : oa;
            const int64_t oC = CORR ? (fst ? oa : oa + 2048) : (hb ? oa + 1024 : oa);
            const int m = 8 * lane;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                raw.q[0][r][0] = *reinterpret_cast<const uint4 *>(u + oA + 512 * r + m);
                raw.q[1][r][0] = *reinterpret_cast<const uint4 *>(u + oB + 512 * r + m);
                raw.q[2][r][0] = *reinterpret_cast<const uint4 *>(u + oC + 512 * r + m);
                if (HAS_W) {
                    raw.q[0][r][1] = *reinterpret_cast<const uint4 *>(w + oA + 512 * r + m);
                    raw.q[1][r][1] = *reinterpret_cast<const uint4 *>(w + oB + 512 * r + m);
                    raw.q[2][r][1] = *reinterpret_cast<const uint4 *>(w + oC + 512 * r + m);
                }
            }
        } else {
            load_pair_raw<T, HAS_W>(raw, u, w, oa, ob, lane);
        }
    };

    // software pipeline: the next pair's inputs are loaded into the registers of this pair's
    // inputs once these are scattered to LDS, its filter chunks into this pair's once S2 has
    // used them (no register copies: a copy of a prefetched set would make the compiler wait
    // for its loads in the middle of the current pair); the gate rows are loaded at the top
    // of their own pair and used at its end
    //   The prefetch loads are issued on every path (the last one re-reads the current pair,
    // a wave with no pair reads its first pair): with a branch around them the compiler has to
    // assume that they may be absent, and each later wait for an older load then waits for
    // the prefetch as well.
    int64_t p = p_begin + (int64_t)wg_local * kPairWaves + wave;
    Raw cur;
    Filt fc;
    // (the same load order as in the loop, so that the waits at the loop head hold for both
    // ways into it)
    load_in(p < p_end ? p : 0, cur);
    __builtin_amdgcn_sched_barrier(0);
    load_filt(p < p_end ? p : 0, fc);
    __builtin_amdgcn_sched_barrier(0);
    for (; p < p_end; p += stride) {
        int64_t h, oa, ob;
        bool has_b;
        bool edge;
        offsets(p, h, oa, ob, has_b, edge);
        const int64_t pn = p + stride < p_end ? p + stride : p;
        uint4 vg[4], vg2[4];
        if (HAS_V) load_gate(v, oa, ob, vg);
        if (DUAL) load_gate(v2, oa, ob, vg2);
        // output scales of the real and the imaginary part (LONE: two channels)
        float ksa = fc.ks, ksb = LONE ? fc.ks2 : fc.ks;

        // ---- x = u * w of both sequences (windows), scattered into the transposed LDS
        // planes: element m = n_f + 32 n_s at row n_f, K block n_s / 32, slot kslot(n_s % 32)
        if constexpr (WIN) {
            h8 xb3[3][2];   // blocks A, B, C
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int r = 0; r < 2; ++r) gate_product<T>(cur.q[k][r][0], cur.q[k][r][1], HAS_W, xb3[k][r]);
            if (CORR) {   // zeros past the sequence end
                if (!has_b) xb3[1][0] = xb3[1][1] = h8{};
                if (edge) xb3[2][0] = xb3[2][1] = h8{};
            } else if (edge) {
                xb3[0][0] = xb3[0][1] = h8{};   // zeros before the sequence start
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {   // window a = (A, B), window b = (B, C)
                const int m0 = 8 * lane + 512 * r;
                const h8 xa = xb3[r >> 1][r & 1], xb = xb3[1 + (r >> 1)][r & 1];
                const int ns = m0 >> 5, nf0 = m0 & 31, kss = 32 * (ns >> 5) + kslot_of(ns & 31);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    zr[(nf0 + e) * kRow + kss] = xa[e];
                    zi[(nf0 + e) * kRow + kss] = xb[e];
                }
            }
        } else if constexpr (LONE) {
            h8 xa[2], xb[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                gate_product<T>(cur.q[r][0], cur.q[r][1], HAS_W, xa[r]);
                gate_product<T>(cur.q[r][2], cur.q[r][3], HAS_W, xb[r]);
                if (!has_b) xb[r] = h8{};
            }
            // (the smaller channel is recovered as a difference (Z(f) - conj Z(-f)) / 2:
            // without the equalisation it is rounded at the larger one's magnitude)
            equalize_pair(xa, xb, ksa, ksb);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int m0 = 8 * lane + 512 * r;
                const int ns = m0 >> 5, nf0 = m0 & 31, kss = kslot_of(ns);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    zr[(nf0 + e) * kRow + kss] = xa[r][e];
                    zi[(nf0 + e) * kRow + kss] = xb[r][e];
                }
            }
        } else {
            h8 xa[2], xb[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                gate_product<T>(cur.q[r][0], cur.q[r][1], HAS_W, xa[r]);
                gate_product<T>(cur.q[r][2], cur.q[r][3], HAS_W, xb[r]);
                if (!has_b) xb[r] = h8{};
            }
            zero_rows(xa, xb, ksa, ksb);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int m0 = 8 * lane + 512 * r;
                const int ns = m0 >> 5, nf0 = m0 & 31, kss = kslot_of(ns);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    zr[(nf0 + e) * kRow + kss] = xa[r][e];
                    zi[(nf0 + e) * kRow + kss] = xb[r][e];
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int KB = WIN ? 2 : 1;   // K blocks of S1
        h8 dr[KB][2], di[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                dr[kb][mt] = *reinterpret_cast<const h8 *>(zr + (16 * mt + c) * kRow + 32 * kb + 8 * g);
                di[kb][mt] = *reinterpret_cast<const h8 *>(zi + (16 * mt + c) * kRow + 32 * kb + 8 * g);
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        __builtin_amdgcn_sched_barrier(0);   // (keep the prefetch loads where they are)
        load_in(pn, cur);
        __builtin_amdgcn_sched_barrier(0);
        h8 ndi[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) ndi[kb][mt] = neg8(di[kb][mt]);
        // second K block (windows): column f_s = 16 nt + c of the DFT changes sign for odd c
        const uint32_t sgn1 = (c & 1) ? 0x80008000u : 0u;
        const uint8_t *mrow = MASKED ? mask + h * kMaskBlocks : nullptr;

        // S1' operands, fp16: a[ks][nt2] (re, im); rows f_s of tiles nt = 2ks (j < 4), 2ks+1 (j >= 4)
        h8 a3r[2][2], a3i[2][2];

        if constexpr (!LONE) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            // ---- S1: rows n_f (tiles mt), column tile nt of f_s; twiddle w2048^{nf fs} (fp16)
            h4 t1r[2], t1i[2];
            h8 f1r[KB], f1i[KB];
            f1r[0] = s_f1[0][nt][lane];
            f1i[0] = s_f1[1][nt][lane];
            if constexpr (WIN) {
                f1r[1] = xor8(f1r[0], sgn1);
                f1i[1] = xor8(f1i[0], sgn1);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                f4 ar = zero4, ai = zero4;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    ar = mfma(dr[kb][mt], f1r[kb], ar);
                    ar = mfma(ndi[kb][mt], f1i[kb], ar);
                    ai = mfma(dr[kb][mt], f1i[kb], ai);
                    ai = mfma(di[kb][mt], f1r[kb], ai);
                }
                t1r[mt] = to_h4(ar);
                t1i[mt] = to_h4(ai);
                cmul4(t1r[mt], t1i[mt], s_tw1[(mt * 4 + nt) * 64 + lane]);
            }
            const h8 br = cat8(t1r[0], t1r[1]), bi = cat8(t1i[0], t1i[1]);
            const h8 nbi = neg8(bi);
            // ---- S2: rows f_f (tiles mt2), column tile nt; filter product (fp16, |K| <= 1)
            h4 yr[2], yi[2];
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2) {
                f4 ar = mfma(c2r[mt2], br, zero4);
                ar = mfma(c2i[mt2], nbi, ar);
                f4 ai = mfma(c2r[mt2], bi, zero4);
                ai = mfma(c2i[mt2], br, ai);
                yr[mt2] = to_h4(ar);
                yi[mt2] = to_h4(ai);
                h8 kk = *reinterpret_cast<const h8 *>(&fc.k[mt2][nt]);
                if (MASKED) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int f = 16 * nt + c + 64 * (16 * mt2 + 4 * g + i);
                        const int fr = f <= N ? f : 2 * N - f;
                        int blk = fr / (N / kMaskBlocks);
                        blk = blk > kMaskBlocks - 1 ? kMaskBlocks - 1 : blk;
                        if (!mrow[blk]) kk[i] = kk[4 + i] = (_Float16)0.f;
                    }
                }
                cmul4(yr[mt2], yi[mt2], kk);
            }
            const h8 a2r = cat8(yr[0], yr[1]), a2i = cat8(yi[0], yi[1]);
            const h8 na2r = neg8(a2r);
            // ---- S2': rows f_s (tile nt), column tiles nt2 of n_f; conj twiddle (fp16)
#pragma unroll
            for (int nt2 = 0; nt2 < 2; ++nt2) {
                f4 ar = mfma(a2r, c2r[nt2], zero4);
                ar = mfma(a2i, c2i[nt2], ar);
                f4 ai = mfma(na2r, c2i[nt2], zero4);
                ai = mfma(a2i, c2r[nt2], ai);
                h4 t3r = to_h4(ar), t3i = to_h4(ai);
                cmul4(t3r, t3i, s_tw3[(nt * 2 + nt2) * 64 + lane]);
                const int ksi = nt >> 1, half = (nt & 1) * 4;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a3r[ksi][nt2][half + i] = t3r[i];
                    a3i[ksi][nt2][half + i] = t3i[i];
                }
            }
        }

        } else {
            // LONE: S1 and S2 of every column tile, the bins of Z into the wave's LDS (word
            // f ^ 16 ((f >> 8) & 3) for bin f, against bank conflicts), then per tile the
            // product with the partner bin Z(-f) and S2'
            uint32_t *const zw = reinterpret_cast<uint32_t *>(s_z[wave]);
            const uint8_t *mrow2 = MASKED ? mask + (has_b ? h + 1 : h) * kMaskBlocks : nullptr;
            // both channels' filter chunks, read here (not prefetched: this launch is one row)
            const uint4 *krow1 = kbins + h * 512, *krow2 = kbins + (has_b ? h + 1 : h) * 512;
            typedef _Float16 h2t __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                h4 t1r[2], t1i[2];
                const h8 f1r = s_f1[0][nt][lane], f1i = s_f1[1][nt][lane];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    f4 ar = mfma(dr[0][mt], f1r, zero4);
                    ar = mfma(ndi[0][mt], f1i, ar);
                    f4 ai = mfma(dr[0][mt], f1i, zero4);
                    ai = mfma(di[0][mt], f1r, ai);
                    t1r[mt] = to_h4(ar);
                    t1i[mt] = to_h4(ai);
                    cmul4(t1r[mt], t1i[mt], s_tw1[(mt * 4 + nt) * 64 + lane]);
                }
                const h8 br = cat8(t1r[0], t1r[1]), bi = cat8(t1i[0], t1i[1]);
                const h8 nbi = neg8(bi);
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2) {
                    f4 ar = mfma(c2r[mt2], br, zero4);
                    ar = mfma(c2i[mt2], nbi, ar);
                    f4 ai = mfma(c2r[mt2], bi, zero4);
                    ai = mfma(c2i[mt2], br, ai);
                    const h4 zr = to_h4(ar), zi = to_h4(ai);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int f = 16 * nt + c + 64 * (16 * mt2 + 4 * g + i);
                        zw[f ^ (g << 4)] = __builtin_bit_cast(uint32_t, h2t{zr[i], zi[i]});
                    }
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const h4 half4 = {(_Float16)0.5f, (_Float16)0.5f, (_Float16)0.5f, (_Float16)0.5f};
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                h4 yr[2], yi[2];
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2) {
                    uint4 q1 = krow1[(mt2 * 4 + nt) * 64 + lane], q2 = krow2[(mt2 * 4 + nt) * 64 + lane];
                    if (DUAL) {   // conj K, conj K'
                        q1.z ^= 0x80008000u;
                        q1.w ^= 0x80008000u;
                        q2.z ^= 0x80008000u;
                        q2.w ^= 0x80008000u;
                    }
                    h8 k1 = *reinterpret_cast<const h8 *>(&q1);
                    h8 k2 = *reinterpret_cast<const h8 *>(&q2);
                    h4 zr, zi, mr, mi;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int f = 16 * nt + c + 64 * (16 * mt2 + 4 * g + i);
                        if (MASKED) {
                            const int fr = f <= N ? f : 2 * N - f;
                            int blk = fr / (N / kMaskBlocks);
                            blk = blk > kMaskBlocks - 1 ? kMaskBlocks - 1 : blk;
                            if (!mrow[blk]) k1[i] = k1[4 + i] = (_Float16)0.f;
                            if (!mrow2[blk]) k2[i] = k2[4 + i] = (_Float16)0.f;
                        }
                        const int fm = (2 * N - f) & (2 * N - 1);   // the partner bin -f
                        const h2t zv = __builtin_bit_cast(h2t, zw[f ^ (g << 4)]);
                        const h2t mv = __builtin_bit_cast(h2t, zw[fm ^ (((fm >> 8) & 3) << 4)]);
                        zr[i] = zv[0];
                        zi[i] = zv[1];
                        mr[i] = mv[0];
                        mi[i] = mv[1];
                    }
                    // A = (K + K') / 2, D = (K - K') / 2; Y = Z A + conj(Z(-f)) D
                    const h4 ar = (lo4(k1) + lo4(k2)) * half4, ai = (hi4(k1) + hi4(k2)) * half4;
                    const h4 er = (lo4(k1) - lo4(k2)) * half4, ei = (hi4(k1) - hi4(k2)) * half4;
                    yr[mt2] = zr * ar - zi * ai + mr * er + mi * ei;
                    yi[mt2] = zr * ai + zi * ar + mr * ei - mi * er;
                }
                const h8 a2r = cat8(yr[0], yr[1]), a2i = cat8(yi[0], yi[1]);
                const h8 na2r = neg8(a2r);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2) {
                    f4 ar = mfma(a2r, c2r[nt2], zero4);
                    ar = mfma(a2i, c2i[nt2], ar);
                    f4 ai = mfma(na2r, c2i[nt2], zero4);
                    ai = mfma(a2i, c2r[nt2], ai);
                    h4 t3r = to_h4(ar), t3i = to_h4(ai);
                    cmul4(t3r, t3i, s_tw3[(nt * 2 + nt2) * 64 + lane]);
                    const int ksi = nt >> 1, half = (nt & 1) * 4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        a3r[ksi][nt2][half + i] = t3r[i];
                        a3i[ksi][nt2][half + i] = t3i[i];
                    }
                }
            }
            // (the reads above before the output rows are staged in the same bytes)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        __builtin_amdgcn_sched_barrier(0);
        load_filt(pn, fc);
        __builtin_amdgcn_sched_barrier(0);

        // ---- S1': rows n_f (tiles nt2), columns n_s (tiles nt3; n_s < 32 only, or n_s - 32 for
        // windows: the outputs m - 1024), K = f_s
#pragma unroll
        for (int nt2 = 0; nt2 < 2; ++nt2) {
            const h8 na0i = neg8(a3i[0][nt2]), na1i = neg8(a3i[1][nt2]);
#pragma unroll
            for (int nt3 = 0; nt3 < 2; ++nt3) {
                const h8 f30r = s_f3[0][nt3][lane], f30i = s_f3[1][nt3][lane];
                const h8 f31r = s_f3[0][2 + nt3][lane], f31i = s_f3[1][2 + nt3][lane];
                f4 ar = mfma(a3r[0][nt2], f30r, zero4);
                ar = mfma(na0i, f30i, ar);
                ar = mfma(a3r[1][nt2], f31r, ar);
                ar = mfma(na1i, f31i, ar);
                f4 ai = mfma(a3r[0][nt2], f30i, zero4);
                ai = mfma(a3i[0][nt2], f30r, ai);
                ai = mfma(a3r[1][nt2], f31i, ai);
                ai = mfma(a3i[1][nt2], f31r, ai);
                // rows n_f = 16 nt2 + 4g + i, column n_s = 16 nt3 + c: m = n_f + 32 n_s, four
                // consecutive m per lane; staged as fp32 rows of both sequences in this wave's
                // LDS (16-byte unit u = m / 4, bit 2 flipped by bit 4 against bank conflicts)
                const int un = 8 * (16 * nt3 + c) + 4 * nt2 + g;
                const int us = un ^ (((un >> 4) & 1) << 2);
                f4 ya = ar * ksa, yb = ai * ksb;
                *reinterpret_cast<f4 *>(so + 16 * us) = ya;
                *reinterpret_cast<f4 *>(so + 4096 + 16 * us) = yb;
            }
        }
        // ---- output gate and store: rows of 8 contiguous elements per lane, 16-byte accesses;
        // without a second row (window) its stores repeat the first one's values
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int qq = (q >= 2 && !has_b) ? q - 2 : q;
            const int u0 = 128 * (qq & 1) + 2 * lane;
            const int s0 = u0 ^ (((u0 >> 4) & 1) << 2), s1 = (u0 + 1) ^ ((((u0 + 1) >> 4) & 1) << 2);
            const f4 y0 = *reinterpret_cast<const f4 *>(so + 4096 * (qq >> 1) + 16 * s0);
            const f4 y1 = *reinterpret_cast<const f4 *>(so + 4096 * (qq >> 1) + 16 * s1);
            float y[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
            const int64_t oq = (q < 2 ? oa : ob) + 512 * (q & 1) + 8 * lane;
            if (DUAL) {
                float g8[8], y2[8];
                unpack8<T>(vg2[q], g8);
#pragma unroll
                for (int e = 0; e < 8; ++e) y2[e] = y[e] * g8[e];
                stnt<uint4>(out2 + oq, io8<T>::pack8(y2));
            }
            if (HAS_V) {
                float g8[8];
                unpack8<T>(vg[q], g8);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] *= g8[e];
            }
            stnt<uint4>(out + oq, io8<T>::pack8(y));   // (written once: streaming)
        }
        // the next pair's input scatter reuses this wave's LDS: order after the reads above
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// ---- dk of the backward pass at N = 1024 -------------------------------------
// dk[h, s] = sum_b corr(g, x)[b, h, s], s < L, with g = v dy and x = u w (the gradient
// of sum(dy out) with respect to the filter).  With the rows of a batch pair packed as
// z_g = g_a + i g_b and z_x = x_a + i x_b (the forward kernel's packing), the spectra
// of the single rows follow from Z(f) and conj Z(M - f), and
//   G_a conj X_a + G_b conj X_b = (P(f) + conj P(M - f)) / 2,  P = Z_g conj Z_x,
// so with S = sum over the channel's pairs of P, DK = (S(f) + conj S(M - f)) / 2 and
// dk = IFFT(DK) = Re IFFT(S) (1/M included).  Per channel: the two forward chains
// (S1, twiddle, S2) of every pair on the matrix cores, P accumulated in fp32 registers,
// a sum over the waves in LDS, and one inverse chain (S2', twiddle, S1', real part).
// An odd last row pairs with zeros, which adds G_a conj X_a exactly (a real row's
// spectrum is Hermitian).  One 8-wave workgroup per CU walks channels
// h = blockIdx.x + k gridDim.x; within a channel wave w takes pairs w, w + 8, ...
constexpr int kDkWaves = 8;

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ __half from_f32<__half>(float x) { return __float2half_rn(x); }
template <> __device__ __forceinline__ __hip_bfloat16 from_f32<__hip_bfloat16>(float x) {
    return __float2bfloat16(x);
}

// With a frequency mask the dropped bins of S are zeroed before the inverse (the mask
// multiplies the spectrum product as it multiplies K in the forward pass, and it is
// symmetric in f, so it commutes with taking the Hermitian part).
// WIN: dk of the chunked short-filter path on (B, H, NS) sequences, NS a multiple of 1024.
// Block j of x contributes sum_t g[t + s] x[t] over its 1024 samples t, which involves g
// at the blocks j and j + 1 only (s < 1024): with x_j zero-padded to 2048 points and the
// window G_j = (g_j, g_{j+1}) (zeros past the sequence end), that is the circular
// correlation IDFT(DFT(G_j) conj DFT(x_j)) at s < 1024, without wrap-around.  A pair packs
// the blocks 2 jp and 2 jp + 1 of one sequence (z_x = x_{2jp} + i x_{2jp+1}, z_g = G_{2jp}
// + i G_{2jp+1}, read from the g blocks A, B, C = 2 jp .. 2 jp + 2); the g chain's S1
// contracts both K blocks as in the windowed forward kernel, the rest is unchanged.
template <typename T, bool HAS_W, bool HAS_V, bool MASKED, bool WIN = false>
__global__ void __launch_bounds__(64 * kDkWaves, 1)
pair1k_dk_kernel(const T *__restrict__ dy, const T *__restrict__ u, const T *__restrict__ w,
                 const T *__restrict__ v, T *__restrict__ dk, const uint8_t *__restrict__ mask,
                 PairTables tb, int64_t B, int64_t H, int64_t L, int64_t NS) {
    static_assert(!(WIN && MASKED), "the windowed path has no frequency mask");
    constexpr int N = 1024, M = 2048, W = kDkWaves;
    constexpr int KG = WIN ? 2 : 1, KR = 32 * KG;   // K blocks of the g chain's S1, g plane row
    // With a gate (more prefetched input registers) the S1 operands are re-read from the
    // planes for every column tile rather than held across the tiles: that removes the
    // register spills of those variants and was faster (N = 1024 backward 304 -> 294 us,
    // gated windows 1.92 -> 1.69 ms); without a gate holding them was faster.
    constexpr bool kTileOps = HAS_W || HAS_V;
    __shared__ h8 s_tw1[2 * 4 * 64];
    __shared__ h8 s_tw3[4 * 2 * 64];
    __shared__ h8 s_f1[3][4][64];   // re, im, -im: S1 takes no negated data operand
    __shared__ h8 s_f3[2][4][64];
    // per wave: the input planes of g and x (2 KG + 2 planes of kPlane fp16), later wave 0's
    // output row; at a channel's end the first 64 KB hold four 16 KB slots of the sum over
    // the waves
    __shared__ __align__(16) _Float16 s_z[W][(2 * KG + 2) * kPlane];

    const int tid = threadIdx.x;
    for (int i = tid; i < 512; i += 64 * W) {
        s_tw1[i] = reinterpret_cast<const h8 *>(tb.tw1)[i];
        s_tw3[i] = reinterpret_cast<const h8 *>(tb.tw3)[i];
    }
    for (int i = tid; i < 256; i += 64 * W) {
        s_f1[0][i / 64][i % 64] = reinterpret_cast<const h8 *>(tb.f1r)[i];
        s_f1[1][i / 64][i % 64] = reinterpret_cast<const h8 *>(tb.f1i)[i];
        s_f1[2][i / 64][i % 64] = neg8(reinterpret_cast<const h8 *>(tb.f1i)[i]);
        s_f3[0][i / 64][i % 64] = reinterpret_cast<const h8 *>(tb.f3r)[i];
        s_f3[1][i / 64][i % 64] = reinterpret_cast<const h8 *>(tb.f3i)[i];
    }
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, c = lane & 15;
    const h8 *F2r = reinterpret_cast<const h8 *>(tb.f2r), *F2i = reinterpret_cast<const h8 *>(tb.f2i);
    h8 c2r[2], c2i[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        c2r[t] = F2r[t * 64 + lane];
        c2i[t] = F2i[t * 64 + lane];
    }
    _Float16 *const zgr = s_z[wave], *const zgi = zgr + KG * kPlane, *const zxr = zgi + KG * kPlane,
                   *const zxi = zxr + kPlane;
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // work items of this wave: channel slot ci, pair slot j -> h = blockIdx.x + ci gridDim.x,
    // bp = wave + W j; slots past the channel's pairs (bp >= PB) add nothing.  Windows: bp =
    // b JP + jp (block pairs of one sequence fastest)
    const int64_t NW = NS / 1024, JP = (NW + 1) / 2;
    const int64_t PB = WIN ? B * JP : (B + 1) / 2, PPW = (PB + W - 1) / W;
    const int64_t NCH = ((int64_t)H - blockIdx.x + gridDim.x - 1) / gridDim.x;   // channels of this workgroup
    const int64_t NI = NCH * PPW;
    // raw 16-byte chunks of one pair: [r][dy_a, v_a, dy_b, v_b, u_a, w_a, u_b, w_b] (rows a
    // and b, or the blocks A and B of a window pair), qc[r][dy, v] of block C (windows)
    struct Raw {
        uint4 q[2][8];
        uint4 qc[2][2];
    };
    // oa, ob (oc): where rows a and b (blocks A, B, C) start; a missing row or block re-reads
    // row a (block A) and its product is zeroed
    auto locate = [&](int64_t i, int64_t &h, int64_t &bp, int64_t &oa, int64_t &ob, int64_t &oc, bool &has_b,
                      bool &has_c, bool &real) {
        const int64_t ci = i / PPW, j = i - ci * PPW;
        h = blockIdx.x + ci * (int64_t)gridDim.x;
        bp = wave + W * j;
        real = bp < PB;
        const int64_t bq = real ? bp : PB - 1;   // (a slot without a pair reads the last pair)
        if (WIN) {   // (the host keeps B JP below 2^31: 32-bit division)
            const uint32_t b32 = (uint32_t)bq / (uint32_t)JP;
            const int64_t b = b32, jp = (uint32_t)bq - b32 * (uint32_t)JP;
            has_b = 2 * jp + 1 < NW;
            has_c = 2 * jp + 2 < NW;
            oa = (b * H + h) * NS + 2 * jp * 1024;
            ob = has_b ? oa + 1024 : oa;
            oc = has_c ? oa + 2048 : oa;
        } else {
            has_b = 2 * bq + 1 < B;
            has_c = false;
            oa = (2 * bq * H + h) * N;
            ob = has_b ? oa + H * N : oa;
            oc = oa;
        }
    };
    auto load_raw = [&](int64_t i, Raw &raw) {
        int64_t h, bp, oa, ob, oc;
        bool hb, hc, real;
        locate(i < NI ? i : NI - 1, h, bp, oa, ob, oc, hb, hc, real);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int m0 = 8 * lane + 512 * r;
            raw.q[r][0] = ldnt<uint4>(dy + oa + m0);
            raw.q[r][2] = ldnt<uint4>(dy + ob + m0);
            raw.q[r][4] = ldnt<uint4>(u + oa + m0);
            raw.q[r][6] = ldnt<uint4>(u + ob + m0);
            if (WIN) raw.qc[r][0] = ldnt<uint4>(dy + oc + m0);
            if (HAS_V) {
                raw.q[r][1] = ldnt<uint4>(v + oa + m0);
                raw.q[r][3] = ldnt<uint4>(v + ob + m0);
                if (WIN) raw.qc[r][1] = ldnt<uint4>(v + oc + m0);
            }
            if (HAS_W) {
                raw.q[r][5] = ldnt<uint4>(w + oa + m0);
                raw.q[r][7] = ldnt<uint4>(w + ob + m0);
            }
        }
    };
    auto wave_sync = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    Raw cur;
    load_raw(0, cur);   // (pinned before the loop in the loop's order, as in the forward kernel)
    __builtin_amdgcn_sched_barrier(0);
    int64_t i = 0;
    for (int64_t ci = 0; ci < NCH; ++ci) {
      f4 Sr[4][2], Si[4][2];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int mt2 = 0; mt2 < 2; ++mt2) Sr[nt][mt2] = Si[nt][mt2] = zero4;
      int64_t h = 0;
      for (int64_t j = 0; j < PPW; ++j, ++i) {
        int64_t bp, oa, ob, oc;
        bool has_b, has_c, real;
        locate(i, h, bp, oa, ob, oc, has_b, has_c, real);
        if (real && WIN) {
            // ---- windows: x blocks A, B zero-padded (32-slot rows); g windows (A, B) and
            // (B, C) over both K blocks (64-slot rows)
            h8 gblk[3][2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                gate_product<T>(cur.q[r][0], cur.q[r][1], HAS_V, gblk[0][r]);
                gate_product<T>(cur.q[r][2], cur.q[r][3], HAS_V, gblk[1][r]);
                gate_product<T>(cur.qc[r][0], cur.qc[r][1], HAS_V, gblk[2][r]);
                if (!has_b) gblk[1][r] = h8{};
                if (!has_c) gblk[2][r] = h8{};
                const int m0 = 8 * lane + 512 * r;
                h8 xa, xb;
                gate_product<T>(cur.q[r][4], cur.q[r][5], HAS_W, xa);
                gate_product<T>(cur.q[r][6], cur.q[r][7], HAS_W, xb);
                if (!has_b) xb = h8{};
                const int ns = m0 >> 5, nf0 = m0 & 31, kss = kslot_of(ns);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    zxr[(nf0 + e) * 32 + kss] = xa[e];
                    zxi[(nf0 + e) * 32 + kss] = xb[e];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m0 = 8 * lane + 512 * r;
                const h8 ga = gblk[r >> 1][r & 1], gb = gblk[1 + (r >> 1)][r & 1];
                const int ns = m0 >> 5, nf0 = m0 & 31, kss = 32 * (ns >> 5) + kslot_of(ns & 31);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    zgr[(nf0 + e) * KR + kss] = ga[e];
                    zgi[(nf0 + e) * KR + kss] = gb[e];
                }
            }
        } else if (real) {
            // ---- g = v dy and x = u w of both rows, scattered into the transposed planes
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int m0 = 8 * lane + 512 * r;
                h8 ga, gb, xa, xb;
                gate_product<T>(cur.q[r][0], cur.q[r][1], HAS_V, ga);
                gate_product<T>(cur.q[r][2], cur.q[r][3], HAS_V, gb);
                gate_product<T>(cur.q[r][4], cur.q[r][5], HAS_W, xa);
                gate_product<T>(cur.q[r][6], cur.q[r][7], HAS_W, xb);
                if (!has_b) {
                    gb = h8{};
                    xb = h8{};
                }
                const int ns = m0 >> 5, nf0 = m0 & 31, kss = kslot_of(ns);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    zgr[(nf0 + e) * 32 + kss] = ga[e];
                    zgi[(nf0 + e) * 32 + kss] = gb[e];
                    zxr[(nf0 + e) * 32 + kss] = xa[e];
                    zxi[(nf0 + e) * 32 + kss] = xb[e];
                }
            }
        }
        wave_sync();
        // S1 operands from the planes (kTileOps: re-read for every column tile)
        h8 dgr[KG][2], dgi[KG][2], dxr[2], dxi[2];
        auto read_ops = [&]() {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int o = (16 * mt + c) * 32 + 8 * g;
#pragma unroll
                for (int kb = 0; kb < KG; ++kb) {
                    dgr[kb][mt] = *reinterpret_cast<const h8 *>(zgr + (16 * mt + c) * KR + 32 * kb + 8 * g);
                    dgi[kb][mt] = *reinterpret_cast<const h8 *>(zgi + (16 * mt + c) * KR + 32 * kb + 8 * g);
                }
                dxr[mt] = *reinterpret_cast<const h8 *>(zxr + o);
                dxi[mt] = *reinterpret_cast<const h8 *>(zxi + o);
            }
        };
        if (!kTileOps) read_ops();
        wave_sync();
        __builtin_amdgcn_sched_barrier(0);
        load_raw(i + 1, cur);   // the next item (clamped: issued on every path)
        __builtin_amdgcn_sched_barrier(0);
        if (real) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                __builtin_amdgcn_sched_barrier(0);   // (one column tile at a time: bounds the live operands)
                if (kTileOps) read_ops();
                const h8 f1r = s_f1[0][nt][lane], f1i = s_f1[1][nt][lane], nf1i = s_f1[2][nt][lane];
                // (windows) the second K block's entries: column f_s = 16 nt + c changes sign
                // for odd c
                const uint32_t sgn1 = (c & 1) ? 0x80008000u : 0u;
                f4 zr_[2][2], zi_[2][2];   // [g / x][mt2]: the S2 accumulators of both chains
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    // S1 with twiddle w2048^{nf fs}, then S2 (as in the forward kernel)
                    h4 t1r[2], t1i[2];
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const h8 dr = q ? dxr[mt] : dgr[0][mt], di = q ? dxi[mt] : dgi[0][mt];
                        f4 ar = mfma(dr, f1r, zero4);
                        ar = mfma(di, nf1i, ar);
                        f4 ai = mfma(dr, f1i, zero4);
                        ai = mfma(di, f1r, ai);
                        if (WIN && q == 0) {
                            const h8 dr1 = dgr[KG - 1][mt], di1 = dgi[KG - 1][mt];
                            ar = mfma(dr1, xor8(f1r, sgn1), ar);
                            ar = mfma(di1, xor8(nf1i, sgn1), ar);
                            ai = mfma(dr1, xor8(f1i, sgn1), ai);
                            ai = mfma(di1, xor8(f1r, sgn1), ai);
                        }
                        t1r[mt] = to_h4(ar);
                        t1i[mt] = to_h4(ai);
                        cmul4(t1r[mt], t1i[mt], s_tw1[(mt * 4 + nt) * 64 + lane]);
                    }
                    const h8 br = cat8(t1r[0], t1r[1]), bi = cat8(t1i[0], t1i[1]);
                    const h8 nbi = neg8(bi);
#pragma unroll
                    for (int mt2 = 0; mt2 < 2; ++mt2) {
                        f4 ar = mfma(c2r[mt2], br, zero4);
                        ar = mfma(c2i[mt2], nbi, ar);
                        f4 ai = mfma(c2r[mt2], bi, zero4);
                        ai = mfma(c2i[mt2], br, ai);
                        zr_[q][mt2] = ar;
                        zi_[q][mt2] = ai;
                    }
                }
                // S += Z_g conj(Z_x)
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2) {
                    Sr[nt][mt2] += zr_[0][mt2] * zr_[1][mt2] + zi_[0][mt2] * zi_[1][mt2];
                    Si[nt][mt2] += zi_[0][mt2] * zr_[1][mt2] - zr_[0][mt2] * zi_[1][mt2];
                }
            }
        }
        if (kTileOps) wave_sync();   // (the operand reads above before the next item's scatter)
      }

        // ---- end of the channel: pairwise sum over the waves (8 -> 4 -> 2 -> 1) through
        // 16 KB slots of the planes region ([nt][mt2][re / im][lane] f4), then the inverse
        // by wave 0 on the sum in its registers
        f4 *const slot = reinterpret_cast<f4 *>(&s_z[0][0]);
        auto put = [&](int k) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2) {
                    slot[k * 1024 + ((nt * 2 + mt2) * 2 + 0) * 64 + lane] = Sr[nt][mt2];
                    slot[k * 1024 + ((nt * 2 + mt2) * 2 + 1) * 64 + lane] = Si[nt][mt2];
                }
        };
        auto add = [&](int k) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2) {
                    Sr[nt][mt2] += slot[k * 1024 + ((nt * 2 + mt2) * 2 + 0) * 64 + lane];
                    Si[nt][mt2] += slot[k * 1024 + ((nt * 2 + mt2) * 2 + 1) * 64 + lane];
                }
        };
        __syncthreads();   // every wave is past its last pair: the planes are free
        if (wave >= 4) put(wave - 4);
        __syncthreads();
        if (wave < 4) add(wave);
        __syncthreads();
        if (wave == 2 || wave == 3) put(wave - 2);
        __syncthreads();
        if (wave < 2) add(wave);
        __syncthreads();
        if (wave == 1) put(0);
        __syncthreads();
        if (wave == 0) add(0);
        __syncthreads();   // (the next pairs' scatters reuse the planes)
        if (wave != 0) continue;
        f4 Tr[4][2], Ti[4][2];
        float mx = 0.f;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2) {
                Tr[nt][mt2] = Sr[nt][mt2];
                Ti[nt][mt2] = Si[nt][mt2];
                if (MASKED) {
                    // (the lane index is laundered so that these channel-invariant indices are
                    // recomputed here, not held in registers across the pair loop)
                    int lc = c, lg = g;
                    asm volatile("" : "+v"(lc), "+v"(lg));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {   // bin f = f_s + 64 f_f of this element
                        const int f = 16 * nt + lc + 64 * (16 * mt2 + 4 * lg + e);
                        const int fr = f <= N ? f : M - f;
                        int blk = fr / (N / kMaskBlocks);
                        blk = blk > kMaskBlocks - 1 ? kMaskBlocks - 1 : blk;
                        if (!mask[h * kMaskBlocks + blk]) Tr[nt][mt2][e] = Ti[nt][mt2][e] = 0.f;
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(Tr[nt][mt2][e]), fabsf(Ti[nt][mt2][e])));
            }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        // scale 2^-e with max |S| 2^-e <= 1: the fp16 operands of the inverse chain
        const int ex = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) : 0;
        // (back also undoes the table factors of the two forward chains and the inverse one)
        const float sc = __builtin_ldexpf(1.f, -ex),
                    back = __builtin_ldexpf(1.f, ex + 3 * (kPairS1Log2 + kPairS2Log2)) / (float)M;
        // S2': rows f_s (tile nt), column tiles nt2 of n_f; conj twiddle (as in the forward kernel)
        h8 a3r[2][2], a3i[2][2];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const h8 a2r = cat8(to_h4(Tr[nt][0] * sc), to_h4(Tr[nt][1] * sc));
            const h8 a2i = cat8(to_h4(Ti[nt][0] * sc), to_h4(Ti[nt][1] * sc));
            const h8 na2r = neg8(a2r);
#pragma unroll
            for (int nt2 = 0; nt2 < 2; ++nt2) {
                f4 ar = mfma(a2r, c2r[nt2], zero4);
                ar = mfma(a2i, c2i[nt2], ar);
                f4 ai = mfma(na2r, c2i[nt2], zero4);
                ai = mfma(a2i, c2r[nt2], ai);
                h4 t3r = to_h4(ar), t3i = to_h4(ai);
                cmul4(t3r, t3i, s_tw3[(nt * 2 + nt2) * 64 + lane]);
                const int ksi = nt >> 1, half = (nt & 1) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a3r[ksi][nt2][half + e] = t3r[e];
                    a3i[ksi][nt2][half + e] = t3i[e];
                }
            }
        }
        // S1': the real part only (rows n_f, columns n_s < 32), staged as one fp32 row of
        // 1024 outputs in wave 0's planes (16-byte unit m / 4, bit 2 flipped by bit 4)
        char *const so = reinterpret_cast<char *>(s_z[0]);
#pragma unroll
        for (int nt2 = 0; nt2 < 2; ++nt2) {
            const h8 na0i = neg8(a3i[0][nt2]), na1i = neg8(a3i[1][nt2]);
#pragma unroll
            for (int nt3 = 0; nt3 < 2; ++nt3) {
                const h8 f30r = s_f3[0][nt3][lane], f30i = s_f3[1][nt3][lane];
                const h8 f31r = s_f3[0][2 + nt3][lane], f31i = s_f3[1][2 + nt3][lane];
                f4 ar = mfma(a3r[0][nt2], f30r, zero4);
                ar = mfma(na0i, f30i, ar);
                ar = mfma(a3r[1][nt2], f31r, ar);
                ar = mfma(na1i, f31i, ar);
                const int un = 8 * (16 * nt3 + c) + 4 * nt2 + g;
                const int us = un ^ (((un >> 4) & 1) << 2);
                *reinterpret_cast<f4 *>(so + 16 * us) = ar * back;
            }
        }
        wave_sync();
        const float *sf = reinterpret_cast<const float *>(so);
        T *drow = dk + h * L;
#pragma unroll
        for (int k = 0; k < N / 64; ++k) {
            const int s = lane + 64 * k;
            const int un = s >> 2, us = un ^ (((un >> 4) & 1) << 2);
            if (s < L) drow[s] = from_f32<T>(sf[4 * us + (s & 3)]);
        }
        wave_sync();   // (the next pair's scatter reuses these planes)
    }
}

hipError_t launch_pair_conv(int logn, int st, const void *u, const void *w, const void *v,
                            void *out, const void *kbins, const float *kscale, const uint8_t *mask,
                            int64_t B, int64_t H, hipStream_t stream, const void *v2, void *out2) {
    if (logn != 10 || st == ST_F32) return hipErrorInvalidValue;
    if (out2 != nullptr && (v == nullptr || v2 == nullptr)) return hipErrorInvalidValue;
    PairTables tb{};
    hipError_t e = get_pair_tables(&tb);
    if (e != hipSuccess) return e;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v_ = 0;
        if (hipDeviceGetAttribute(&v_, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v_ > 0)
            cus = v_;
    }
    if (H * ((B + 1) / 2) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    // An odd B: the rows 0 .. B - 2 as batch-row pairs, the last row as channel pairs (LONE)
    const int64_t Bp = B & ~int64_t(1);
    auto launch = [&](bool lone) {
        const int64_t pairs = lone ? (H + 1) / 2 : H * (Bp / 2);
        if (pairs == 0) return;
        // two resident 4-wave workgroups per CU (one for the masked variant)
        int64_t blocks = (int64_t)cus * (mask ? 1 : 2);
        const int64_t need = (pairs + kPairWaves - 1) / kPairWaves;
        if (blocks > need) blocks = need < 8 ? 8 : (need + 7) / 8 * 8;
        auto go = [&](auto kern, auto *tp) {
            using TT = std::remove_pointer_t<decltype(tp)>;
            hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kPairWaves), 0, stream,
                               (const TT *)u, (const TT *)w, (const TT *)v, (TT *)out,
                               (const uint4 *)kbins, kscale, mask, tb, lone ? B : Bp, H, (int64_t)1024,
                               (const TT *)v2, (TT *)out2);
        };
        // one instantiation per (storage type, mask, gates, row kind): no gate test sits in
        // the pair loop
        auto pick = [&](auto *tp, auto lone_c) {
            using TT = std::remove_pointer_t<decltype(tp)>;
            constexpr bool LN = decltype(lone_c)::value;
            if (out2 != nullptr) {   // two outputs: both output gates present
                switch ((mask ? 2 : 0) | (w ? 1 : 0)) {
                case 0: go(pair1k_kernel<TT, false, false, true, false, true, false, LN>, tp); break;
                case 1: go(pair1k_kernel<TT, false, true, true, false, true, false, LN>, tp); break;
                case 2: go(pair1k_kernel<TT, true, false, true, false, true, false, LN>, tp); break;
                default: go(pair1k_kernel<TT, true, true, true, false, true, false, LN>, tp); break;
                }
                return;
            }
            const int sel = (mask ? 4 : 0) | (w ? 2 : 0) | (v ? 1 : 0);
            switch (sel) {
            case 0: go(pair1k_kernel<TT, false, false, false, false, false, false, LN>, tp); break;
            case 1: go(pair1k_kernel<TT, false, false, true, false, false, false, LN>, tp); break;
            case 2: go(pair1k_kernel<TT, false, true, false, false, false, false, LN>, tp); break;
            case 3: go(pair1k_kernel<TT, false, true, true, false, false, false, LN>, tp); break;
            case 4: go(pair1k_kernel<TT, true, false, false, false, false, false, LN>, tp); break;
            case 5: go(pair1k_kernel<TT, true, false, true, false, false, false, LN>, tp); break;
            case 6: go(pair1k_kernel<TT, true, true, false, false, false, false, LN>, tp); break;
            default: go(pair1k_kernel<TT, true, true, true, false, false, false, LN>, tp); break;
            }
        };
        if (lone) {
            if (st == ST_F16) pick((__half *)nullptr, std::true_type{});
            else pick((__hip_bfloat16 *)nullptr, std::true_type{});
        } else {
            if (st == ST_F16) pick((__half *)nullptr, std::false_type{});
            else pick((__hip_bfloat16 *)nullptr, std::false_type{});
        }
    };
    launch(false);
    if (B & 1) launch(true);
    return hipGetLastError();
}

hipError_t launch_pair_conv_win(int st, const void *u, const void *w, const void *v, void *out,
                                const void *kbins, const float *kscale, int64_t B, int64_t H, int64_t NS,
                                hipStream_t stream, bool corr, const void *v2, void *out2) {
    if (st == ST_F32 || NS < 1024 || NS % 1024 != 0) return hipErrorInvalidValue;
    if (out2 != nullptr && (!corr || v == nullptr || v2 == nullptr)) return hipErrorInvalidValue;
    PairTables tb{};
    hipError_t e = get_pair_tables(&tb);
    if (e != hipSuccess) return e;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v_ = 0;
        if (hipDeviceGetAttribute(&v_, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v_ > 0)
            cus = v_;
    }
    const int64_t pairs = H * B * ((NS / 1024 + 1) / 2);
    if (pairs >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (pairs == 0) return hipSuccess;
    int64_t blocks = (int64_t)cus * 2;
    const int64_t need = (pairs + kPairWaves - 1) / kPairWaves;
    if (blocks > need) blocks = need < 8 ? 8 : (need + 7) / 8 * 8;
    auto go = [&](auto kern, auto *tp) {
        using TT = std::remove_pointer_t<decltype(tp)>;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kPairWaves), 0, stream,
                           (const TT *)u, (const TT *)w, (const TT *)v, (TT *)out,
                           (const uint4 *)kbins, kscale, (const uint8_t *)nullptr, tb, B, H, NS,
                           (const TT *)v2, (TT *)out2);
    };
    auto pick = [&](auto *tp) {
        using TT = std::remove_pointer_t<decltype(tp)>;
        const int sel = (w ? 2 : 0) | (v ? 1 : 0);
        if (corr && out2 != nullptr) {   // two outputs: both output gates present
            if (w) go(pair1k_kernel<TT, false, true, true, true, true, true>, tp);
            else go(pair1k_kernel<TT, false, false, true, true, true, true>, tp);
            return;
        }
        if (corr) {
            switch (sel) {
            case 0: go(pair1k_kernel<TT, false, false, false, true, false, true>, tp); break;
            case 1: go(pair1k_kernel<TT, false, false, true, true, false, true>, tp); break;
            case 2: go(pair1k_kernel<TT, false, true, false, true, false, true>, tp); break;
            default: go(pair1k_kernel<TT, false, true, true, true, false, true>, tp); break;
            }
            return;
        }
        switch (sel) {
        case 0: go(pair1k_kernel<TT, false, false, false, true>, tp); break;
        case 1: go(pair1k_kernel<TT, false, false, true, true>, tp); break;
        case 2: go(pair1k_kernel<TT, false, true, false, true>, tp); break;
        default: go(pair1k_kernel<TT, false, true, true, true>, tp); break;
        }
    };
    if (st == ST_F16) pick((__half *)nullptr);
    else pick((__hip_bfloat16 *)nullptr);
    return hipGetLastError();
}


// NS > 0: the windowed dk of the short-filter path on (B, H, NS) sequences (no mask)
hipError_t launch_pair_dk(int st, const void *dy, const void *u, const void *w, const void *v, void *dk,
                          const uint8_t *mask, int64_t B, int64_t H, int64_t L, hipStream_t stream,
                          int64_t NS) {
    if (st == ST_F32) return hipErrorInvalidValue;
    if (NS != 0 && (NS < 1024 || NS % 1024 != 0 || mask != nullptr)) return hipErrorInvalidValue;
    if (NS != 0 && B * ((NS / 1024 + 1) / 2) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (B <= 0 || H <= 0) return hipSuccess;
    PairTables tb{};
    hipError_t e = get_pair_tables(&tb);
    if (e != hipSuccess) return e;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v_ = 0;
        if (hipDeviceGetAttribute(&v_, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v_ > 0)
            cus = v_;
    }
    const int64_t blocks = H < cus ? H : cus;   // one 8-wave workgroup per CU, channels strided
    auto go = [&](auto kern, auto *tp) {
        using TT = std::remove_pointer_t<decltype(tp)>;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kDkWaves), 0, stream, (const TT *)dy,
                           (const TT *)u, (const TT *)w, (const TT *)v, (TT *)dk, mask, tb, B, H, L, NS);
    };
    auto pick = [&](auto *tp) {
        using TT = std::remove_pointer_t<decltype(tp)>;
        const int sel = (mask ? 4 : 0) | (w ? 2 : 0) | (v ? 1 : 0);
        if (NS != 0) {
            switch (sel) {
            case 0: go(pair1k_dk_kernel<TT, false, false, false, true>, tp); break;
            case 1: go(pair1k_dk_kernel<TT, false, true, false, true>, tp); break;
            case 2: go(pair1k_dk_kernel<TT, true, false, false, true>, tp); break;
            default: go(pair1k_dk_kernel<TT, true, true, false, true>, tp); break;
            }
            return;
        }
        switch (sel) {
        case 0: go(pair1k_dk_kernel<TT, false, false, false>, tp); break;
        case 1: go(pair1k_dk_kernel<TT, false, true, false>, tp); break;
        case 2: go(pair1k_dk_kernel<TT, true, false, false>, tp); break;
        case 3: go(pair1k_dk_kernel<TT, true, true, false>, tp); break;
        case 4: go(pair1k_dk_kernel<TT, false, false, true>, tp); break;
        case 5: go(pair1k_dk_kernel<TT, false, true, true>, tp); break;
        case 6: go(pair1k_dk_kernel<TT, true, false, true>, tp); break;
        default: go(pair1k_dk_kernel<TT, true, true, true>, tp); break;
        }
    };
    if (st == ST_F16) pick((__half *)nullptr);
    else pick((__hip_bfloat16 *)nullptr);
    return hipGetLastError();
}

}  // namespace fftconv
