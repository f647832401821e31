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
// Every DFT is split once more into radix stages held in the registers of one
// lane, with padded (bank-conflict-free) LDS transposes between stages.  All
// arithmetic is fp32.  Workspace: one complex value per point and sequence
// of the chunk, held in the storage type (fp32, fp16 or bf16 pairs), so the
// two passes through it cost as many bytes per point as the input does;
// after it, 2 * 8192 fp32 complex values per sequence for the two rows that
// pair with themselves.
#include "fft_device.hpp"
#include "fft_stages.hpp"
#include "fftconv_internal.hpp"
#include "cmfma.hpp"

#include <type_traits>

namespace fftconv {

constexpr int kMpLog2 = 13;                // on-chip row length N2 = 8192
constexpr int kMpThreads = 512;

// omega_N^a for a in [0, N): two-level table lookup (a = hi * 2048 + lo)
__device__ __forceinline__ float2 tw_big(const float2 *__restrict__ lo, const float2 *__restrict__ hi,
                                         uint32_t a) {
    return cmul(ldu<float2>(hi, 8u * (a >> 11)), ldu<float2>(lo, 8u * (a & 2047u)));
}

struct MpArgs {
    const float2 *tw1;      // exp(-2 pi i j / N1), j < N1
    const float2 *tw2;      // exp(-2 pi i j / N2), j < N2
    const float2 *w2n2;     // exp(-pi i j / N2),   j < N2   (omega_{2 N2}^j)
    const float2 *w2row;    // exp(-pi i j / N),    j < N1   (omega_{2N}^{f1})
    const float2 *big_lo;   // exp(-2 pi i j / N),  j < 2048
    const float2 *big_hi;   // exp(-2 pi i 2048 j / N), j < N / 2048
    const uint4 *col;       // matrix-core column-pass operand tiles (or null)
};

// ------------------------------------------------------------ small helpers
// a[j] *= w^j for j < R (R a power of two, at most 32).  w8 must hold w^8
// (read from a table) when R > 8, so every factor is a product at most four
// deep and stays within a few ulp of the exact root of unity.
template <int R>
__device__ __forceinline__ void apply_pow(float2 *a, float2 w, float2 w8) {
    constexpr int R1 = R < 8 ? R : 8;
    float2 p[R1];
    p[0] = make_float2(1.f, 0.f);
    if constexpr (R1 > 1) p[1] = w;
    if constexpr (R1 > 2) p[2] = cmul(w, w);
    if constexpr (R1 > 3) p[3] = cmul(p[2], w);
    if constexpr (R1 > 4) {
        p[4] = cmul(p[2], p[2]);
        p[5] = cmul(p[4], w);
        p[6] = cmul(p[4], p[2]);
        p[7] = cmul(p[4], p[3]);
    }
#pragma unroll
    for (int i = 1; i < R1; ++i) a[i] = cmul(a[i], p[i]);
    if constexpr (R > 8) {
        const float2 w16 = cmul(w8, w8);
#pragma unroll
        for (int m = 1; m < R / 8; ++m) {
            const float2 q = m == 1 ? w8 : (m == 2 ? w16 : cmul(w16, w8));
#pragma unroll
            for (int i = 0; i < 8; ++i) a[8 * m + i] = cmul(a[8 * m + i], i == 0 ? q : cmul(q, p[i]));
        }
    }
}

// out[q] = sum_{j < R/2} in[j] omega_R^{jq}, q < R: an R-point DFT whose upper
// half of inputs is zero.  Even outputs are the R/2-point DFT of in, odd ones
// that of in[j] omega_R^j.
template <int R>
__device__ __forceinline__ void dft_halfzero(const float2 *in, float2 *out) {
    float2 e[R / 2], o[R / 2], E[R / 2], O[R / 2];
#pragma unroll
    for (int j = 0; j < R / 2; ++j) {
        e[j] = in[j];
        o[j] = twiddle_const<R>(in[j], j);
    }
    Dft<R / 2>::run(e, E);
    Dft<R / 2>::run(o, O);
#pragma unroll
    for (int p = 0; p < R / 2; ++p) {
        out[2 * p] = E[p];
        out[2 * p + 1] = O[p];
    }
}

// out[q] = sum_{j < R} in[j] omega_R^{jq} for q < R/2 only (decimation in time).
template <int R>
__device__ __forceinline__ void dft_halfout(const float2 *in, float2 *out) {
    float2 e[R / 2], o[R / 2], E[R / 2], O[R / 2];
#pragma unroll
    for (int j = 0; j < R / 2; ++j) {
        e[j] = in[2 * j];
        o[j] = in[2 * j + 1];
    }
    Dft<R / 2>::run(e, E);
    Dft<R / 2>::run(o, O);
#pragma unroll
    for (int q = 0; q < R / 2; ++q) out[q] = cadd(E[q], twiddle_const<R>(O[q], q));
}

// ------------------------------------------------------------ column plan
// The N1-point column DFT of passes 1 and 3 is split as N1 = RB * RA with
// n1 = n_a + RA n_b, f1 = f_b + RB f_a.  A workgroup of 512 lanes owns C
// adjacent columns; lane (col, j) = (tid % C, tid / C), j < RA.  The RB * RA
// intermediate values per column pass through LDS in NG groups of RA values
// of f_b, so a workgroup holds at most 64 KiB of LDS and two fit on a CU.
template <int LOG1> struct ColPlan {
    static constexpr int N1 = 1 << LOG1;
    static constexpr int RB = 1 << mp_col_rb_log2(LOG1);
    static constexpr int RA = N1 / RB;
    static constexpr int C = kMpThreads / RA;
    static constexpr int NG = RB / RA;
    static constexpr size_t kLds = (size_t)RA * RA * C * sizeof(float2);
    static_assert(RA >= 2 && RB <= 32 && (NG == 1 || NG == 2), "column plan");
};

// a[fa] *= omega_N^{n2 (fb + RB fa)} for fa < RA
template <int RA, int RB>
__device__ __forceinline__ void column_twiddle(float2 *a, uint32_t n2, uint32_t fb, uint32_t nmask,
                                               const MpArgs &ta) {
    const float2 base = tw_big(ta.big_lo, ta.big_hi, (n2 * fb) & nmask);
    const float2 step = tw_big(ta.big_lo, ta.big_hi, (n2 * (uint32_t)RB) & nmask);
    const float2 step8 = tw_big(ta.big_lo, ta.big_hi, (n2 * (uint32_t)(8 * RB)) & nmask);
#pragma unroll
    for (int i = 0; i < RA; ++i) a[i] = cmul(a[i], base);
    apply_pow<RA>(a, step, step8);
}

// ---------------------------------------------------------------- pass 1
// grid (N2 / C, nseq); block 512.  SRC_FILTER: input is the filter row
// k[h, :L] (prepare); else u * w of sequence seq0 + blockIdx.y.
template <int LOG1, typename T, bool SRC_FILTER>
__global__ void __launch_bounds__(kMpThreads, 4)
mp_pass1_kernel(const T *__restrict__ src, const T *__restrict__ gate, int64_t L, int64_t seq0,
                T *__restrict__ ws, MpArgs ta) {
    using P = ColPlan<LOG1>;
    constexpr int N1 = P::N1, RA = P::RA, RB = P::RB, C = P::C, N2 = 1 << kMpLog2;
    constexpr int64_t NC = (int64_t)N1 * N2;
    extern __shared__ float2 lds[];
    const int tid = threadIdx.x;
    const int col = tid % C, j = tid / C;
    const int c0 = blockIdx.x * C;
    const uint32_t n2 = (uint32_t)(c0 + col);
    const int64_t s = seq0 + blockIdx.y;
    const T *row = src + s * (SRC_FILTER ? L : NC);
    const T *grow = (!SRC_FILTER && gate != nullptr) ? gate + s * NC : nullptr;
    // the half-precision convolution path stores the column transform scaled by
    // 2^-p1 (about 1/sqrt of the N1/2 summed terms), undone by pass 3
    constexpr bool kHalfConv = !SRC_FILTER && sizeof(T) == 2;
    const float p1 = kHalfConv ? __builtin_ldexpf(1.f, -mp_p1_log2(LOG1)) : 1.f;

    // stage 1: lane (col, n_a = j), RB-point DFT over n_b (upper half zero).
    // Element m = n2 + N2 (j + RA n_b): uniform part c0 + N2 RA n_b, lane part
    // col + N2 j.
    const uint32_t lo = (uint32_t)(col + N2 * j);
    float2 y[RB];
    {
        float2 z[RB / 2];
#pragma unroll
        for (int nb = 0; nb < RB / 2; ++nb) {
            const int64_t mu = (int64_t)c0 + (int64_t)N2 * RA * nb;
            float2 t = make_float2(0.f, 0.f);
            if (SRC_FILTER) {
                const int64_t m = mu + lo;
                if (2 * m < L) t.x = io<T>::load1(row + 2 * m);
                if (2 * m + 1 < L) t.y = io<T>::load1(row + 2 * m + 1);
            } else {
                t = io<T>::load2(row + 2 * mu, lo);
                if (grow != nullptr) {
                    const float2 g = io<T>::load2(grow + 2 * mu, lo);
                    t = make_float2(t.x * g.x, t.y * g.y);
                }
                if (kHalfConv) t = make_float2(t.x * p1, t.y * p1);
            }
            z[nb] = t;
        }
        dft_halfzero<RB>(z, y);
    }
    apply_pow<RB>(y, ldu<float2>(ta.tw1, 8u * j), ldu<float2>(ta.tw1, 8u * ((8 * j) & (N1 - 1))));

    T *out = ws + 2 * (int64_t)blockIdx.y * NC;
#pragma unroll
    for (int g = 0; g < P::NG; ++g) {
#pragma unroll
        for (int i = 0; i < RA; ++i) lds[(i * RA + j) * C + col] = y[g * RA + i];
        __syncthreads();
        // stage 2: lane (col, f_b = g RA + j), RA-point DFT over n_a
        float2 a[RA];
#pragma unroll
        for (int i = 0; i < RA; ++i) a[i] = lds[(j * RA + i) * C + col];
        dft_inplace<RA>(a);
        const uint32_t fb = (uint32_t)(g * RA + j);
        column_twiddle<RA, RB>(a, n2, fb, (uint32_t)(NC - 1), ta);
        // row fb + RB f_a: uniform part (g RA + RB f_a) N2 + c0, lane part j N2 + col
        const uint32_t so = (uint32_t)(launder(j) * N2 + launder(col));
#pragma unroll
        for (int fa = 0; fa < RA; ++fa) io<T>::store2(out + 2 * ((int64_t)(g * RA + RB * fa) * N2 + c0), so, a[fa]);
        if (g + 1 < P::NG) __syncthreads();
    }
}

// ---------------------------------------------------------------- pass 3
// SCALED (half-precision storage): the outputs are multiplied by the part of the
// channel scale the row pass left out and the inverse of the column-pass and
// table factors: kscale[h] 2^(kRowKLog2 + 4 kDft32Log2 + p1).
template <int LOG1, typename T, bool SCALED>
__global__ void __launch_bounds__(kMpThreads, 4)
mp_pass3_kernel(const T *__restrict__ ws, const T *__restrict__ v, T *__restrict__ out,
                int64_t seq0, MpArgs ta, const float *__restrict__ kscale, int64_t H) {
    using P = ColPlan<LOG1>;
    constexpr int N1 = P::N1, RA = P::RA, RB = P::RB, C = P::C, N2 = 1 << kMpLog2;
    constexpr int64_t NC = (int64_t)N1 * N2;
    extern __shared__ float2 lds[];
    const int tid = threadIdx.x;
    const int col = tid % C, j = tid / C;
    const int c0 = blockIdx.x * C;
    const uint32_t n2 = (uint32_t)(c0 + col);
    const int64_t s = seq0 + blockIdx.y;
    const T *wsq = ws + 2 * (int64_t)blockIdx.y * NC;
    const uint32_t lo = (uint32_t)(col + N2 * j);

    // stage 2 needs, per lane, the RB-point DFT over f_b at outputs n_b < RB/2.
    // With NG = 2 it is split by decimation in frequency: the two halves of
    // f_b arrive one after the other and are folded at once into
    //   e[f] = x[f] + x[f + RA]          -> outputs n_b = 2m
    //   d[f] = (x[f] - x[f + RA]) w_RB^f -> outputs n_b = 2m + 1
    // so at most RB values (not RB plus the transform's temporaries) are live.
    float2 e[RA], d[RA];
#pragma unroll
    for (int g = 0; g < P::NG; ++g) {
        // stage 1: lane (col, f_b = g RA + j), RA-point DFT over f_a.  The
        // stored rows are conj(b); conj(b omega^-a) = conj(b) omega^a.
        const uint32_t fb = (uint32_t)(g * RA + j);
        float2 a[RA];
#pragma unroll
        for (int fa = 0; fa < RA; ++fa) a[fa] = io<T>::load2(wsq + 2 * ((int64_t)(g * RA + RB * fa) * N2 + c0), lo);
        column_twiddle<RA, RB>(a, n2, fb, (uint32_t)(NC - 1), ta);
        dft_inplace<RA>(a);
        apply_pow<RA>(a, ldu<float2>(ta.tw1, 8u * fb), ldu<float2>(ta.tw1, 8u * ((8 * fb) & (N1 - 1))));
        if (g > 0) __syncthreads();
#pragma unroll
        for (int i = 0; i < RA; ++i) lds[(j * RA + i) * C + col] = a[i];
        __syncthreads();
        if (g == 0) {
#pragma unroll
            for (int i = 0; i < RA; ++i) e[i] = lds[(i * RA + j) * C + col];
        } else {
#pragma unroll
            for (int i = 0; i < RA; ++i) {
                const float2 t = lds[(i * RA + j) * C + col];
                d[i] = twiddle_const<RB>(csub(e[i], t), i);
                e[i] = cadd(e[i], t);
            }
        }
    }
    float2 r[RB / 2];
    if constexpr (P::NG == 2) {
        float2 re[RA / 2], ro[RA / 2];
        dft_halfout<RA>(e, re);
        dft_halfout<RA>(d, ro);
#pragma unroll
        for (int m = 0; m < RA / 2; ++m) {
            r[2 * m] = re[m];
            r[2 * m + 1] = ro[m];
        }
    } else {
        dft_halfout<RB>(e, r);
    }
    if (SCALED) {
        const float comp = __builtin_ldexpf(kscale[s % H], kRowKLog2 + 4 * kDft32Log2 + mp_p1_log2(LOG1));
#pragma unroll
        for (int nb = 0; nb < RB / 2; ++nb) r[nb] = make_float2(r[nb].x * comp, r[nb].y * comp);
    }
    T *orow = out + s * NC;
    const uint32_t lo2 = (uint32_t)(launder(col) + N2 * launder(j));
    // one branch around the whole store loop (not one per store), so that the
    // final butterflies are not sunk into it with their inputs held live
    if (v != nullptr) {
        const T *vrow = v + s * NC;
#pragma unroll
        for (int nb = 0; nb < RB / 2; ++nb) {
            const int64_t mu = (int64_t)c0 + (int64_t)N2 * RA * nb;
            const float2 g = io<T>::load2(vrow + 2 * mu, lo2);
            io<T>::store2(orow + 2 * mu, lo2, make_float2(r[nb].x * g.x, -r[nb].y * g.y));
        }
    } else {
#pragma unroll
        for (int nb = 0; nb < RB / 2; ++nb) {
            const int64_t mu = (int64_t)c0 + (int64_t)N2 * RA * nb;
            io<T>::store2(orow + 2 * mu, lo2, make_float2(r[nb].x, -r[nb].y));
        }
    }
}

// ------------------------------------------- matrix-core column passes (half storage)
// For fp16 / bf16 storage with N1 = RA RB >= 2^kMpColMinLog1 both column passes run
// as two complex-as-real v_mfma_f32_16x16x32_f16 stages (cmfma.hpp) instead of the
// fp32 register DFTs above; same index splits (n1 = n_a + RA n_b, f1 = f_b + RB f_a),
// same results up to fp16 rounding of the stage operands.  A workgroup owns 32
// columns n2 = c0 .. c0 + 31 as two column tiles ct of the products (column 2c + ct
// at lane column c = l % 16, so a lane stores two adjacent columns at once).  The
// stage operands pass through LDS as fp16 planes [ct][re / im][c][row][slot], the
// slot (the contraction index) contiguous: a lane's eight K slots are one 16-byte
// read; lanes whose K slots lie past the transform read a 16-byte zero word.  The
// twiddle between the two stages is folded into the second stage's operand tile
// (one tile per digit), so only the four-step twiddle omega_N^{n2 f1} stays on the
// VALU (fp32, from the two-level table).
namespace colmm {
using cmfma::h8;
using cmfma::f4;
using cmfma::cm_constA;
}  // namespace colmm
using namespace colmm;

template <int LOG1> struct ColMm {
    using P = ColPlan<LOG1>;
    static constexpr int RA = P::RA, RB = P::RB, N1 = P::N1;
    static constexpr int T1 = RB / 16;                  // pass-1 stage-1 tiles (rows f_b)
    static_assert(RB >= 16 && RB <= 32 && RA >= 8 && RA <= 16, "matrix-core column split");
    // per-c strides (bytes) of the LDS planes, 16 bytes of padding against bank conflicts
    static constexpr int C11 = RA * (RB / 2) * 2 + 16;   // pass 1 stage 1: rows n_a, slots n_b
    static constexpr int C12 = RB * RA * 2 + 16;         // pass 1 stage 2: rows f_b, slots n_a
    static constexpr int C31 = RB * RA * 2 + 16;         // pass 3 stage 1: rows f_b, slots f_a
    static constexpr int C32 = RA * RB * 2 + 16;         // pass 3 stage 2: rows n_a, slots f_b
    static constexpr int kRegion = 64 * C12;             // the largest of the four
    static_assert(C11 <= C12 && C31 == C12 && C32 == C12, "LDS regions");
    static constexpr int kZero = kRegion;                // 16 zero bytes
    static constexpr size_t kLds = (size_t)kRegion + 16;
    static constexpr int kTile = 3 * 64;                 // uint4 per operand tile (re, im, -im)
    static constexpr int kC1S1 = 0, kC1S2 = T1 * kTile, kC3S1 = (T1 + RB) * kTile,
                         kC3S2 = (T1 + RB + 1) * kTile;
};

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return __builtin_bit_cast(uint32_t, h2v{(_Float16)a, (_Float16)b});
}
template <typename T> __device__ __forceinline__ float2 t2f(uint32_t w);
template <> __device__ __forceinline__ float2 t2f<__half>(uint32_t w) {
    const h2v h = __builtin_bit_cast(h2v, w);
    return make_float2((float)h[0], (float)h[1]);
}
template <> __device__ __forceinline__ float2 t2f<__hip_bfloat16>(uint32_t w) {
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
template <typename T> __device__ __forceinline__ uint32_t f2t(float2 v);
template <> __device__ __forceinline__ uint32_t f2t<__half>(float2 v) { return pack_h2(v.x, v.y); }
template <> __device__ __forceinline__ uint32_t f2t<__hip_bfloat16>(float2 v) { return io<__hip_bfloat16>::pack(v); }

// one operand tile (three planes) of the table
__device__ __forceinline__ void col_tile(const uint4 *tabs, int base, int lane, h8 &fr, h8 &fi, h8 &nfi) {
    fr = ldu<h8>(tabs + base, 16u * lane);
    fi = ldu<h8>(tabs + base + 64, 16u * lane);
    nfi = ldu<h8>(tabs + base + 128, 16u * lane);
}
// the B operand (re, im planes) at byte offset off of plane 0 (plane 1 is 16 c-strides on),
// or zeros
__device__ __forceinline__ void col_operand(const char *lds, int off, int cstride, bool in, int zero, h8 &br,
                                            h8 &bi) {
    br = *reinterpret_cast<const h8 *>(lds + (in ? off : zero));
    bi = *reinterpret_cast<const h8 *>(lds + (in ? off + 16 * cstride : zero));
}

// pass 1 on the matrix cores: grid (N2 / 32, nseq); block 512.  Input u * w of sequence
// seq0 + blockIdx.y, scaled by 2^-p1 as in mp_pass1_kernel; output the twiddled column
// transform in rows f1 of the workspace.
template <int LOG1, typename T>
__global__ void __launch_bounds__(kMpThreads, 4)
mp_pass1c_kernel(const T *__restrict__ src, const T *__restrict__ gate, int64_t seq0, T *__restrict__ ws,
                 MpArgs ta) {
    using M = ColMm<LOG1>;
    constexpr int RA = M::RA, RB = M::RB, N1 = M::N1, N2 = 1 << kMpLog2;
    constexpr int64_t NC = (int64_t)N1 * N2;
    constexpr uint32_t NM = (uint32_t)(NC - 1);
    extern __shared__ float2 lds[];
    char *const L = reinterpret_cast<char *>(lds);
    const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c0 = blockIdx.x * 32;
    const int64_t s = seq0 + blockIdx.y;
    const T *row = src + s * NC;
    const T *grow = gate != nullptr ? gate + s * NC : nullptr;
    const float p1 = __builtin_ldexpf(1.f, -mp_p1_log2(LOG1));
    const uint4 *tabs = ta.col;
    if (tid == 0) *reinterpret_cast<uint4 *>(L + M::kZero) = make_uint4(0u, 0u, 0u, 0u);

    // ---- inputs z[n1][c0 .. c0 + 31], n1 < N1/2, in row pairs (n_a + 2k RA, n_a + (2k+1) RA):
    // both rows' values of column 2cp + ct form one 32-bit word at slots n_b = 2k, 2k + 1.
    // Every load is issued before the first is used.
    constexpr int R1 = N1 / 128;
    {
        const int cp = tid & 15;
        uint2 qa[R1], qb[R1], ga[R1], gb[R1];
#pragma unroll
        for (int r = 0; r < R1; ++r) {
            const int rp = (tid >> 4) + 32 * r;
            const uint32_t ea = 4u * (uint32_t)((rp % RA + 2 * RA * (rp / RA)) * N2 + c0 + 2 * cp);   // bytes
            qa[r] = ldu<uint2>(row, ea);
            qb[r] = ldu<uint2>(row, ea + 4u * (uint32_t)(RA * N2));
        }
        if (grow != nullptr) {
#pragma unroll
            for (int r = 0; r < R1; ++r) {
                const int rp = (tid >> 4) + 32 * r;
                const uint32_t ea = 4u * (uint32_t)((rp % RA + 2 * RA * (rp / RA)) * N2 + c0 + 2 * cp);
                ga[r] = ldu<uint2>(grow, ea);
                gb[r] = ldu<uint2>(grow, ea + 4u * (uint32_t)(RA * N2));
            }
        }
#pragma unroll
        for (int r = 0; r < R1; ++r) {
            const int rp = (tid >> 4) + 32 * r;
            const int na = rp % RA, k = rp / RA;
            float2 va[2] = {t2f<T>(qa[r].x), t2f<T>(qa[r].y)}, vb[2] = {t2f<T>(qb[r].x), t2f<T>(qb[r].y)};
            if (grow != nullptr) {
                const float2 wa[2] = {t2f<T>(ga[r].x), t2f<T>(ga[r].y)}, wb[2] = {t2f<T>(gb[r].x), t2f<T>(gb[r].y)};
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    va[ct] = make_float2(va[ct].x * wa[ct].x, va[ct].y * wa[ct].y);
                    vb[ct] = make_float2(vb[ct].x * wb[ct].x, vb[ct].y * wb[ct].y);
                }
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int o = (ct * 32 + cp) * M::C11 + (na * (RB / 2) + 2 * k) * 2;
                *reinterpret_cast<uint32_t *>(L + o) = pack_h2(va[ct].x * p1, vb[ct].x * p1);
                *reinterpret_cast<uint32_t *>(L + o + 16 * M::C11) = pack_h2(va[ct].y * p1, vb[ct].y * p1);
            }
        }
    }
    h8 Fr[M::T1], Fi[M::T1], nFi[M::T1];
#pragma unroll
    for (int m = 0; m < M::T1; ++m) col_tile(tabs, M::kC1S1 + m * M::kTile, lane, Fr[m], Fi[m], nFi[m]);
    __syncthreads();

    // ---- stage 1: per (n_a, ct) the RB-point DFT over n_b < RB/2, rows f_b = 16 m + 4 g + i.
    // A wave takes n_a pairs (2p, 2p + 1) so that both values of a slot pair are its own;
    // the results are held until every wave has read its operands (the next planes
    // overwrite these).
    constexpr int NPU = RA / 8;   // (n_a pair, ct) units per wave
    uint32_t hold[NPU][M::T1][2][4];
    {
        const bool in = g < RB / 16;
#pragma unroll
        for (int t = 0; t < NPU; ++t) {
            const int u = wave * NPU + t, p = u >> 1, ct = u & 1;
            f4 cr[2][M::T1], ci[2][M::T1];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                h8 br, bi;
                col_operand(L, (ct * 32 + c) * M::C11 + ((2 * p + h) * (RB / 2) + 8 * g) * 2, M::C11, in,
                            M::kZero, br, bi);
#pragma unroll
                for (int m = 0; m < M::T1; ++m) cm_constA(Fr[m], Fi[m], nFi[m], br, bi, cr[h][m], ci[h][m]);
            }
#pragma unroll
            for (int m = 0; m < M::T1; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    hold[t][m][0][i] = pack_h2(cr[0][m][i], cr[1][m][i]);
                    hold[t][m][1][i] = pack_h2(ci[0][m][i], ci[1][m][i]);
                }
        }
    }
    // stage-2 operand tile of the first unit and the four-step twiddle factors, fetched
    // across the barriers: for column n2 (ct) and rows f1 = f_b + RB (4 g + i) with
    // f_b = wave + 8 t, omega_N^{n2 f1} = P (S8)^t (SR)^i
    h8 Ar, Ai, nAi;
    col_tile(tabs, M::kC1S2 + wave * M::kTile, lane, Ar, Ai, nAi);
    float2 P[2], S8[2], SR[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const uint32_t n2 = (uint32_t)(c0 + 2 * c + ct);
        P[ct] = tw_big(ta.big_lo, ta.big_hi, (n2 * (uint32_t)(wave + 4 * g * RB)) & NM);
        S8[ct] = tw_big(ta.big_lo, ta.big_hi, (n2 * 8u) & NM);
        SR[ct] = tw_big(ta.big_lo, ta.big_hi, (n2 * (uint32_t)RB) & NM);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NPU; ++t) {
        const int u = wave * NPU + t, p = u >> 1, ct = u & 1;
#pragma unroll
        for (int m = 0; m < M::T1; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = (ct * 32 + c) * M::C12 + ((16 * m + 4 * g + i) * RA + 2 * p) * 2;
                *reinterpret_cast<uint32_t *>(L + o) = hold[t][m][0][i];
                *reinterpret_cast<uint32_t *>(L + o + 16 * M::C12) = hold[t][m][1][i];
            }
    }
    __syncthreads();

    // ---- stage 2: per f_b the RA-point DFT over n_a with omega_N1^{n_a f_b} (its table
    // tile), rows f_a = 4 g + i < RA; the four-step twiddle; store rows f1 = f_b + RB f_a
    T *out = ws + 2 * (int64_t)blockIdx.y * NC;
    const bool in = g < RA / 8;
    float2 SR2[2], SR3[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        SR2[ct] = cmul(SR[ct], SR[ct]);
        SR3[ct] = cmul(SR2[ct], SR[ct]);
    }
#pragma unroll
    for (int t = 0; t < RB / 8; ++t) {
        const int fb = wave + 8 * t;
        f4 cr[2], ci[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            h8 br, bi;
            col_operand(L, (ct * 32 + c) * M::C12 + (fb * RA + 8 * g) * 2, M::C12, in, M::kZero, br, bi);
            cm_constA(Ar, Ai, nAi, br, bi, cr[ct], ci[ct]);
        }
        if (t + 1 < RB / 8) col_tile(tabs, M::kC1S2 + (fb + 8) * M::kTile, lane, Ar, Ai, nAi);
        if (4 * g < RA) {
            const uint32_t n2 = (uint32_t)(c0 + 2 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t f1 = (uint32_t)(fb + RB * (4 * g + i));
                float2 y[2];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const float2 tw = i == 0 ? P[ct] : cmul(P[ct], i == 1 ? SR[ct] : (i == 2 ? SR2[ct] : SR3[ct]));
                    y[ct] = cmul(make_float2(cr[ct][i], ci[ct][i]), tw);
                }
                stu(out, 4u * (f1 * (uint32_t)N2 + n2), make_uint2(f2t<T>(y[0]), f2t<T>(y[1])));
            }
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) P[ct] = cmul(P[ct], S8[ct]);
    }
}

// pass 3 on the matrix cores: grid (N2 / 32, nseq); block 512.  The same outputs as
// mp_pass3_kernel<LOG1, T, true> (conjugate, channel and table scales, output gate).
template <int LOG1, typename T>
__global__ void __launch_bounds__(kMpThreads, 4)
mp_pass3c_kernel(const T *__restrict__ ws, const T *__restrict__ v, T *__restrict__ out, int64_t seq0,
                 MpArgs ta, const float *__restrict__ kscale, int64_t H) {
    using M = ColMm<LOG1>;
    constexpr int RA = M::RA, RB = M::RB, N1 = M::N1, N2 = 1 << kMpLog2;
    constexpr int64_t NC = (int64_t)N1 * N2;
    constexpr uint32_t NM = (uint32_t)(NC - 1);
    extern __shared__ float2 lds[];
    char *const L = reinterpret_cast<char *>(lds);
    const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c0 = blockIdx.x * 32;
    const int64_t s = seq0 + blockIdx.y;
    const T *wsq = ws + 2 * (int64_t)blockIdx.y * NC;
    const uint4 *tabs = ta.col;
    if (tid == 0) *reinterpret_cast<uint4 *>(L + M::kZero) = make_uint4(0u, 0u, 0u, 0u);

    // ---- inputs y[f1][c0 .. c0 + 31], all rows, in pairs (f_b + 2k RB, f_b + (2k+1) RB) ->
    // slots f_a = 2k, 2k + 1, times omega_N^{n2 f1} (the stored rows are conj(b), and
    // conj(b omega^-a) = conj(b) omega^a).  Round r reads rows f1 = f0 + 64 r and
    // f0 + 64 r + RB, so the twiddles follow from three table values per column.
    constexpr int R3 = N1 / 64;
    {
        const int cp = tid & 15;
        const uint32_t n2 = (uint32_t)(c0 + 2 * cp);
        const int fb = (tid >> 4) % RB, k0 = (tid >> 4) / RB;
        const uint32_t f0 = (uint32_t)(fb + 2 * RB * k0);
        uint2 qa[R3], qb[R3];
#pragma unroll
        for (int r = 0; r < R3; ++r) {
            qa[r] = ldu<uint2>(wsq, 4u * ((f0 + 64u * r) * (uint32_t)N2 + n2));
            qb[r] = ldu<uint2>(wsq, 4u * ((f0 + 64u * r + RB) * (uint32_t)N2 + n2));
        }
        float2 cur[2], S64[2], SR[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const uint32_t n = n2 + (uint32_t)ct;
            cur[ct] = tw_big(ta.big_lo, ta.big_hi, (n * f0) & NM);
            S64[ct] = tw_big(ta.big_lo, ta.big_hi, (n * 64u) & NM);
            SR[ct] = tw_big(ta.big_lo, ta.big_hi, (n * (uint32_t)RB) & NM);
        }
#pragma unroll
        for (int r = 0; r < R3; ++r) {
            const int k = k0 + r * (32 / RB);
            const float2 qa2[2] = {t2f<T>(qa[r].x), t2f<T>(qa[r].y)}, qb2[2] = {t2f<T>(qb[r].x), t2f<T>(qb[r].y)};
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const float2 va = cmul(qa2[ct], cur[ct]), vb = cmul(qb2[ct], cmul(cur[ct], SR[ct]));
                const int o = (ct * 32 + cp) * M::C31 + (fb * RA + 2 * k) * 2;
                *reinterpret_cast<uint32_t *>(L + o) = pack_h2(va.x, vb.x);
                *reinterpret_cast<uint32_t *>(L + o + 16 * M::C31) = pack_h2(va.y, vb.y);
                cur[ct] = cmul(cur[ct], S64[ct]);
            }
        }
    }
    h8 Fr, Fi, nFi;
    col_tile(tabs, M::kC3S1, lane, Fr, Fi, nFi);
    __syncthreads();

    // ---- stage 1: per (f_b, ct) the RA-point DFT over f_a, rows n_a = 4 g + i < RA; a
    // wave takes f_b pairs (2p, 2p + 1); results held until every wave has read its operands
    constexpr int NPU = RB / 8;
    uint32_t hold[NPU][2][4];
    {
        const bool in = g < RA / 8;
#pragma unroll
        for (int t = 0; t < NPU; ++t) {
            const int u = wave * NPU + t, p = u >> 1, ct = u & 1;
            f4 cr[2], ci[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                h8 br, bi;
                col_operand(L, (ct * 32 + c) * M::C31 + ((2 * p + h) * RA + 8 * g) * 2, M::C31, in, M::kZero,
                            br, bi);
                cm_constA(Fr, Fi, nFi, br, bi, cr[h], ci[h]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hold[t][0][i] = pack_h2(cr[0][i], cr[1][i]);
                hold[t][1][i] = pack_h2(ci[0][i], ci[1][i]);
            }
        }
    }
    // the first stage-2 tile and output gate, fetched across the barriers
    h8 Ar, Ai, nAi;
    col_tile(tabs, M::kC3S2 + wave * M::kTile, lane, Ar, Ai, nAi);
    T *orow = out + s * NC;
    const T *vrow = v != nullptr ? v + s * NC : nullptr;
    auto out_off = [&](int na, int i) {
        return 4u * ((uint32_t)(na + RA * (4 * g + i)) * (uint32_t)N2 + (uint32_t)(c0 + 2 * c));
    };
    uint2 gq[4];
    if (vrow != nullptr && 4 * g < RB / 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) gq[i] = ldu<uint2>(vrow, out_off(wave, i));
    }
    __syncthreads();
    if (4 * g < RA) {
#pragma unroll
        for (int t = 0; t < NPU; ++t) {
            const int u = wave * NPU + t, p = u >> 1, ct = u & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = (ct * 32 + c) * M::C32 + ((4 * g + i) * RB + 2 * p) * 2;
                *reinterpret_cast<uint32_t *>(L + o) = hold[t][0][i];
                *reinterpret_cast<uint32_t *>(L + o + 16 * M::C32) = hold[t][1][i];
            }
        }
    }
    __syncthreads();

    // ---- stage 2: per n_a the RB-point DFT over f_b with omega_N1^{n_a f_b} (its table
    // tile), rows n_b = 4 g + i < RB/2: outputs n1 = n_a + RA n_b (t < N); conjugate,
    // scale, gate, store
    const float comp = __builtin_ldexpf(kscale[s % H], kRowKLog2 + 4 * kDft32Log2 + mp_p1_log2(LOG1) +
                                                           mp_c3_log2(LOG1));
    const bool in = g < RB / 8;
#pragma unroll
    for (int t = 0; t < RA / 8; ++t) {
        const int na = wave + 8 * t;
        f4 cr[2], ci[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            h8 br, bi;
            col_operand(L, (ct * 32 + c) * M::C32 + (na * RB + 8 * g) * 2, M::C32, in, M::kZero, br, bi);
            cm_constA(Ar, Ai, nAi, br, bi, cr[ct], ci[ct]);
        }
        uint2 gn[4];
        if (t + 1 < RA / 8) {
            col_tile(tabs, M::kC3S2 + (na + 8) * M::kTile, lane, Ar, Ai, nAi);
            if (vrow != nullptr && 4 * g < RB / 2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) gn[i] = ldu<uint2>(vrow, out_off(na + 8, i));
            }
        }
        if (4 * g < RB / 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float2 y0 = make_float2(cr[0][i] * comp, -ci[0][i] * comp);
                float2 y1 = make_float2(cr[1][i] * comp, -ci[1][i] * comp);
                if (vrow != nullptr) {
                    const float2 g0 = t2f<T>(gq[i].x), g1 = t2f<T>(gq[i].y);
                    y0 = make_float2(y0.x * g0.x, y0.y * g0.y);
                    y1 = make_float2(y1.x * g1.x, y1.y * g1.y);
                }
                stu(orow, out_off(na, i), make_uint2(f2t<T>(y0), f2t<T>(y1)));
            }
        }
        if (t + 1 < RA / 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) gq[i] = gn[i];
        }
    }
}

// ---------------------------------------------------------------- pass 2
// One row of N2 = 8192 points: n2 = n_a + 256 n_b, n_a = n_c + 16 n_d and
// k = k_b + 32 k_d + 512 k_c (k = f2, the in-row bin):
//   A  per n_a:        32-point DFT over n_b, twiddle omega_8192^{n_a k_b}
//   B  per (n_c, k_b): 16-point DFT over n_d, twiddle omega_256^{n_c k_d}
//   C  per (k_b, k_d): 16-point DFT over n_c
// The inverse runs the same stages in reverse order on conjugated data.
//
// Lanes: stage A (row ra = tid >> 8, n_a = tid & 255); stage B
// (k_b0 = tid & 31, n_c = tid >> 5) holding row A at k_b0 and row B at
// k_b0 ^ 16; stage C (k_b = tid & 31, k_d = tid >> 5) holding row A at
// (k_b, k_d) and row B at (31 - k_b, 15 - k_d), so that every bin pair of the
// bin-pair step sits in one lane.
//
// Two rows do not fit in the LDS share of a workgroup (two workgroups per
// CU), so each transpose runs in two rounds that move half of the data:
//   T1 round h: k_b in [16h, 16h + 16) of both rows,
//               slot (r, k_b & 15, n_a) -> (16 r + (k_b & 15)) * 257 + n_a
//   T2 round h: k_d in [8h, 8h + 8) of both rows,
//               slot (r, k_b, k_d, n_c) -> (32 r + k_b) * 129 + 16 r + 16 (k_d & 7) + n_c
// In every round each lane writes 16 values and reads 16, and the odd
// strides keep the 32 lanes of each half-wave on distinct LDS banks.
constexpr int kT1Row = 257;
constexpr int kT2Row = 129;
constexpr int kP2LdsFloat2 = 64 * kT2Row + 16 + 128;
constexpr size_t kP2Lds = (size_t)kP2LdsFloat2 * sizeof(float2);

// The 128 mask blocks of a channel as two 64-bit words (bit b: block kept).
struct BlockMask {
    uint64_t lo, hi;
    __device__ __forceinline__ bool keep(int b) const { return ((b < 64 ? lo >> b : hi >> (b - 64)) & 1) != 0; }
    // keep bits of blocks 4 j .. 4 j + 3 (bit i of the result: block 4 j + i), j < 32
    __device__ __forceinline__ uint32_t nibble(int j) const {
        return (uint32_t)((j < 16 ? lo >> (4 * j) : hi >> (4 * j - 64)) & 15u);
    }
};
static_assert(kP2LdsFloat2 >= 32 * kT1Row && kP2LdsFloat2 >= 8192, "pass-2 LDS");

// Position of in-row bin f2 in a stored filter row: natural order for fp32
// spectra, the matrix-core order (mp_chain_pos) for half-precision ones.
template <typename TK> __device__ __forceinline__ uint32_t kpos(uint32_t f2);
template <> __device__ __forceinline__ uint32_t kpos<float2>(uint32_t f2) { return f2; }
template <> __device__ __forceinline__ uint32_t kpos<__half2>(uint32_t f2) { return mp_chain_pos(f2); }

// Bin pairs of the workgroup that holds rows 0 and N1/2: each row pairs with
// itself (row 0: f2 <-> N2 - f2; row N1/2: f2 <-> N2 - 1 - f2).  Both rows
// sit in natural order in an fp32 area of the workspace (row 0, then row
// N1/2); lanes take the 8193 pairs in turn.
template <int N1, int N2, typename TK, bool PREPARE, bool MASKED>
__device__ __forceinline__ void self_pairs(float2 *area, const TK *__restrict__ krow,
                                           TK *__restrict__ kout, BlockMask bm, float ks,
                                           const MpArgs &ta, int tid, float ysgn) {
    constexpr int64_t NC = (int64_t)N1 * N2;
    const float sh = 1.0f / (ks * 4.0f * (float)NC);
    for (int it = tid; it <= N2; it += kMpThreads) {
        const bool half_row = it > N2 / 2;             // items 0..N2/2: row 0; the rest: row N1/2
        const int w = half_row ? it - (N2 / 2 + 1) : it;
        const int rbase = half_row ? N1 / 2 : 0;
        float2 *row = area + (half_row ? N2 : 0);
        const int ia = w;
        const int ib = half_row ? N2 - 1 - w : (w == 0 ? 0 : N2 - w);
        const int64_t rb = (int64_t)rbase * N2;
        const uint32_t pa = kpos<TK>((uint32_t)ia), pb = kpos<TK>((uint32_t)ib);
        float2 zf = row[ia], zg = row[ib];
        const bool dc = !half_row && w == 0;   // f = 0: (K[0], K[N]) share slot 0
        const float2 wrow = half_row ? ta.w2row[N1 / 2] : make_float2(1.f, 0.f);
        const float2 Wf = dc ? make_float2(1.f, 0.f) : cmul(wrow, ta.w2n2[w]);
        if (PREPARE) {
            const float2 bc = cconj(zg);
            const float2 xe = cadd(zf, bc);
            const float2 xo = cmul_negi(csub(zf, bc));
            const float2 wxo = cmul(Wf, xo);
            float2 xf = cscale(cadd(xe, wxo), 0.5f * sh);
            float2 xg = cscale(cconj(csub(xe, wxo)), 0.5f * sh);
            xf.y *= ysgn;
            xg.y *= ysgn;
            if (dc) {
                kio<TK>::store(kout, make_float2(xf.x, xg.x));
            } else {
                kio<TK>::store(kout + rb, pa, xf);
                if (ib != ia) kio<TK>::store(kout + rb, pb, xg);
            }
            continue;
        }
        float2 Kf, Kg;
        if (dc) {
            const float2 k0 = cscale(kio<TK>::load(krow), ks);
            Kf = make_float2(MASKED && !bm.keep(0) ? 0.f : k0.x, 0.f);
            Kg = make_float2(MASKED && !bm.keep(kMaskBlocks - 1) ? 0.f : k0.y, 0.f);
        } else {
            Kf = (MASKED && !bm.keep(ia >> 6)) ? make_float2(0.f, 0.f) : cscale(kio<TK>::load(krow + rb, pa), ks);
            Kg = (MASKED && !bm.keep(ib >> 6)) ? make_float2(0.f, 0.f) : cscale(kio<TK>::load(krow + rb, pb), ks);
        }
        middle_pair(zf, zg, Kf, Kg, Wf);
        row[ia] = zf;
        if (ib != ia) row[ib] = zg;
    }
}

// grid (N1 / 2, nseq); block 512.  PREPARE: forward only, writes the filter
// spectrum; else the full filter product and inverse rows.
template <int LOG1, typename T, typename TK, bool PREPARE, bool MASKED>
__global__ void __launch_bounds__(kMpThreads, 4)
mp_pass2_kernel(T *__restrict__ ws, float2 *__restrict__ self_area, const TK *__restrict__ kbins_in,
                TK *__restrict__ kbins_out, const float *__restrict__ kscale,
                const uint8_t *__restrict__ mask, int64_t H, int64_t seq0, MpArgs ta, float ysgn) {
    constexpr int N1 = 1 << LOG1, N2 = 1 << kMpLog2;
    constexpr int64_t NC = (int64_t)N1 * N2;
    extern __shared__ float2 lds[];
    const int tid = threadIdx.x;
    const int f1 = blockIdx.x;
    const int rowA = f1, rowB = f1 == 0 ? N1 / 2 : N1 - f1;
    const int64_t s = seq0 + blockIdx.y;
    const int64_t h = s % H;
    T *wsq = ws + 2 * (int64_t)blockIdx.y * NC;
    const float2 *tw = ta.tw2;
    BlockMask bm{~0ull, ~0ull};
    if (MASKED) {
        const uint8_t *mrow = mask + h * kMaskBlocks;
        bm.lo = __builtin_amdgcn_ballot_w64(mrow[tid & 63] != 0);
        bm.hi = __builtin_amdgcn_ballot_w64(mrow[64 + (tid & 63)] != 0);
    }

    // ---- stage A: lane (row ra, n_a)
    const int ra = __builtin_amdgcn_readfirstlane(tid >> 8), na = tid & 255;
    T *rowp = wsq + 2 * (int64_t)(ra ? rowB : rowA) * N2;
    float2 a[32];
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) a[nb] = io<T>::load2(rowp + 512 * nb, (uint32_t)na);
    dft_pq<8, 4>(a);
    apply_pow<32>(a, ldu<float2>(tw, 8u * na), ldu<float2>(tw, 64u * na));

    // ---- T1, stage B.  p[q] receives, in round q, the row whose k_b lies in
    // half q: row (q ^ hb0) at k_b = 16 q + kl0.
    const int kb0 = tid & 31, ncB = tid >> 5, kl0 = kb0 & 15, hb0 = kb0 >> 4;
    float2 p[2][16];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int kl = 0; kl < 16; ++kl) lds[(16 * ra + kl) * kT1Row + na] = a[16 * q + kl];
        __syncthreads();
        const int r = q ^ hb0;
#pragma unroll
        for (int nd = 0; nd < 16; ++nd) p[q][nd] = lds[(16 * r + kl0) * kT1Row + ncB + 16 * nd];
        __syncthreads();
    }
    {
        const float2 w = ldu<float2>(tw, 256u * ncB), w8 = ldu<float2>(tw, 2048u * ncB);
        dft_pq<4, 4>(p[0]);
        dft_pq<4, 4>(p[1]);
        apply_pow<16>(p[0], w, w8);
        apply_pow<16>(p[1], w, w8);
    }

    // ---- T2, stage C.  The lanes of waves 0-3 (hiw = 0) have k_d < 8: they
    // take row A in round 0 and row B in round 1; waves 4-7 the other way.
    // c[q] is the row received in round q: row A when hiw == q, else row B.
    const int kbC = tid & 31, kdC = tid >> 5, hiw = tid >> 8;
    const int t2p0 = (32 * hb0 + kl0) * kT2Row + 16 * hb0 + ncB;
    const int t2p1 = (32 * (1 - hb0) + 16 + kl0) * kT2Row + 16 * (1 - hb0) + ncB;
    const int t2a = kbC * kT2Row + 16 * (kdC & 7);
    const int t2b = (63 - kbC) * kT2Row + 16 + 16 * ((15 - kdC) & 7);
    float2 c[2][16];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            lds[t2p0 + 16 * i] = p[0][8 * q + i];
            lds[t2p1 + 16 * i] = p[1][8 * q + i];
        }
        __syncthreads();
        const int src = hiw == q ? t2a : t2b;
#pragma unroll
        for (int n = 0; n < 16; ++n) c[q][n] = lds[src + n];
        __syncthreads();
    }
    dft_pq<4, 4>(c[0]);
    dft_pq<4, 4>(c[1]);
    // Row A holds bins kq + 512 kc at (kbC, kdC), row B bins
    // (31 - kbC) + 32 (15 - kdC) + 512 kc = 8191 - (kq + 512 (15 - kc)).
    // So c[0][j] and c[1][15 - j] are always the two bins of one pair:
    //   hiw = 0: (A at k, B at 8191 - k),  k = kq + 512 j
    //   hiw = 1: (B at 8191 - k, A at k),  k = kq + 512 (15 - j)
    // The bin-pair step is symmetric in its two bins (with omega_2N^{N - f} =
    // -conj(omega_2N^f)), so every lane runs the same code on (c[0][j],
    // c[1][15 - j]) with its filter addresses and twiddle chosen per wave.

    // ---- bin-pair step.  The workgroup of rows 0 and N1/2 (f1 = 0), whose
    // rows pair with themselves, first saves its spectra to this sequence's
    // fp32 area (row 0, then row N1/2, natural order), runs the in-lane step
    // like every other workgroup (its results are discarded: rowB = N1/2
    // keeps every access in range), then pairs the bins in the area and
    // reloads.  Keeping the common step outside any branch keeps its register
    // allocation free of the rare path.
    const float ks = kscale[h];
    const int kq = kbC + 32 * kdC;
    float2 *area = self_area + (int64_t)blockIdx.y * 2 * N2;
    const int qa = kq, qb = N2 + (31 - kbC) + 32 * (15 - kdC);   // area offsets of rows A, B
    if (f1 == 0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float2 *dst = area + (hiw == q ? qa : qb);
#pragma unroll
            for (int kc = 0; kc < 16; ++kc) dst[512 * kc] = c[q][kc];
        }
    }
    {
        const float2 wb = cmul(ta.w2row[f1], ldu<float2>(ta.w2n2, 8u * kq));   // omega_2N^{f1 + N1 kq}
        // twiddle of the first bin of pair j is w1 omega_32^j
        const float2 w1 = hiw ? twiddle_const<32>(cconj(wb), 1) : wb;
        // in-row bin of the first element: o1 + 512 j; of the second: o2 + 512 (15 - j)
        const uint32_t o1 = hiw ? 511 - kq : kq, o2 = hiw ? kq : 511 - kq;
        if (PREPARE) {
            if (f1 != 0) {
                const float sh = 1.0f / (ks * 4.0f * (float)NC);
                TK *k1 = kbins_out + h * NC + (int64_t)(hiw ? rowB : rowA) * N2;
                TK *k2 = kbins_out + h * NC + (int64_t)(hiw ? rowA : rowB) * N2;
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const float2 zf = c[0][jj], zg = c[1][15 - jj];
                    const float2 Wf = twiddle_const<32>(w1, jj);
                    const float2 bc = cconj(zg);
                    const float2 xe = cadd(zf, bc);
                    const float2 xo = cmul_negi(csub(zf, bc));
                    const float2 wxo = cmul(Wf, xo);
                    float2 x1 = cscale(cadd(xe, wxo), 0.5f * sh), x2 = cscale(cconj(csub(xe, wxo)), 0.5f * sh);
                    x1.y *= ysgn;   // ysgn = -1: conjugated spectrum
                    x2.y *= ysgn;
                    kio<TK>::store(k1, kpos<TK>(512u * jj + o1), x1);
                    kio<TK>::store(k2, kpos<TK>(512u * (15 - jj) + o2), x2);
                }
                return;
            }
        } else {
            const int hw = __builtin_amdgcn_readfirstlane(hiw);
            const TK *k1 = kbins_in + h * NC + (int64_t)(hw ? rowB : rowA) * N2;
            const TK *k2 = kbins_in + h * NC + (int64_t)(hw ? rowA : rowB) * N2;
            // the mask block of in-row bin b is b >> 6; o1 >> 6 and o2 >> 6 are
            // uniform over the wave (kq >> 6 is the wave's index modulo 4).
            // Masked filter bins are read through buffer views of the two rows:
            // a dropped block takes an offset past the view and reads zero
            // without a branch and without its HBM traffic.
            const int b1 = __builtin_amdgcn_readfirstlane((int)(o1 >> 6));
            const int b2 = __builtin_amdgcn_readfirstlane((int)(o2 >> 6));
            const __amdgpu_buffer_rsrc_t r1 = buffer_view(k1, N2 * (uint32_t)sizeof(TK));
            const __amdgpu_buffer_rsrc_t r2 = buffer_view(k2, N2 * (uint32_t)sizeof(TK));
            // two batches of KB = 8 bin pairs; the scheduling barriers keep the
            // second batch of filter loads from being hoisted over the first
            constexpr int KB = 8;
#pragma unroll
            for (int bt = 0; bt < 16 / KB; ++bt) {
                float2 K1[KB], K2[KB];
#pragma unroll
                for (int i = 0; i < KB; ++i) {
                    const int jj = KB * bt + i;
                    if (MASKED) {
                        const uint32_t e1 = (uint32_t)sizeof(TK) * kpos<TK>(512u * jj + o1);
                        const uint32_t e2 = (uint32_t)sizeof(TK) * kpos<TK>(512u * (15 - jj) + o2);
                        K1[i] = kio<TK>::load(r1, bm.keep(b1 + 8 * jj) ? e1 : kBufferSkip);
                        K2[i] = kio<TK>::load(r2, bm.keep(b2 + 8 * (15 - jj)) ? e2 : kBufferSkip);
                    } else {
                        K1[i] = kio<TK>::load(k1, kpos<TK>(512u * jj + o1));
                        K2[i] = kio<TK>::load(k2, kpos<TK>(512u * (15 - jj) + o2));
                    }
                }
#pragma unroll
                for (int i = 0; i < KB; ++i) {
                    const int jj = KB * bt + i;
                    float2 z1 = c[0][jj], z2 = c[1][15 - jj];
                    middle_pair(z1, z2, cscale(K1[i], ks), cscale(K2[i], ks), twiddle_const<32>(w1, jj));
                    c[0][jj] = z1;
                    c[1][15 - jj] = z2;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (f1 == 0) {
        // The barriers (workgroup scope) order the area's global writes and
        // reads across the workgroup's waves, which share one CU's L1.  A
        // device-scope fence here would write back the whole L2.
        const TK *krow = PREPARE ? nullptr : kbins_in + h * NC;
        TK *kout = PREPARE ? kbins_out + h * NC : nullptr;
        __syncthreads();
        self_pairs<N1, N2, TK, PREPARE, MASKED>(area, krow, kout, bm, ks, ta, tid, ysgn);
        if (PREPARE) return;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const float2 *src = area + (hiw == q ? qa : qb);
#pragma unroll
            for (int kc = 0; kc < 16; ++kc) c[q][kc] = src[512 * kc];
        }
    }
    // c now holds conj(Z') in the same layout; the forward transform of
    // conjugated data is the conjugated inverse transform.  Lane indices are
    // recomputed from a laundered thread id so that no address is held live
    // across the bin-pair step.
    __builtin_amdgcn_sched_barrier(0);
    {
    const int tid2 = launder(tid);
    const int kbC = tid2 & 31, kdC = tid2 >> 5, kb0 = tid2 & 31, ncB = tid2 >> 5, kl0 = kb0 & 15,
              hb0 = kb0 >> 4, na = tid2 & 255, hiw = tid2 >> 8;
    const int t2p0 = (32 * hb0 + kl0) * kT2Row + 16 * hb0 + ncB;
    const int t2p1 = (32 * (1 - hb0) + 16 + kl0) * kT2Row + 16 * (1 - hb0) + ncB;
    const int t2a = kbC * kT2Row + 16 * (kdC & 7);
    const int t2b = (63 - kbC) * kT2Row + 16 + 16 * ((15 - kdC) & 7);

    // ---- stage C' (over k_c -> n_c), twiddle omega_256^{n_c k_d}; c[q] is
    // row A (k_d = kdC) when hiw == q, else row B (k_d = 15 - kdC)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        dft_pq<4, 4>(c[q]);
        const int kd = hiw == q ? kdC : 15 - kdC;
        apply_pow<16>(c[q], ldu<float2>(tw, 256u * kd), ldu<float2>(tw, 2048u * kd));
    }

    // ---- T2' (T2 backwards), stage B' (over k_d -> n_d), twiddle
    // omega_8192^{(n_c + 16 n_d) k_b}; p[q] is at k_b = 16 q + kl0
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int dst = hiw == q ? t2a : t2b;
#pragma unroll
        for (int n = 0; n < 16; ++n) lds[dst + n] = c[q][n];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[0][8 * q + i] = lds[t2p0 + 16 * i];
            p[1][8 * q + i] = lds[t2p1 + 16 * i];
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int kb = 16 * q + kl0;
        dft_pq<4, 4>(p[q]);
        const float2 base = ldu<float2>(tw, 8u * (ncB * kb));
#pragma unroll
        for (int i = 0; i < 16; ++i) p[q][i] = cmul(p[q][i], base);
        apply_pow<16>(p[q], ldu<float2>(tw, 128u * kb), ldu<float2>(tw, 1024u * kb));
    }

    // ---- T1' (T1 backwards), stage A' (over k_b -> n_b), store
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = q ^ hb0;
#pragma unroll
        for (int nd = 0; nd < 16; ++nd) lds[(16 * r + kl0) * kT1Row + ncB + 16 * nd] = p[q][nd];
        __syncthreads();
#pragma unroll
        for (int kl = 0; kl < 16; ++kl) a[16 * q + kl] = lds[(16 * ra + kl) * kT1Row + na];
        __syncthreads();
    }
    dft_pq<8, 4>(a);
    // rows now hold conj of the inverse row transform; pass 3 undoes the conj
    const uint32_t so = (uint32_t)launder(tid & 255);
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) io<T>::store2(rowp + 512 * nb, so, a[nb]);
    }
}

// ---------------------------------------------------------------- pass 2 on the matrix cores
// Half-precision storage runs the row pass on the MFMA matrix cores (fp16
// operands, fp32 accumulation; FlashFFTConv summary page, "Approach": the DFT
// as an order-p chain of matrix products).  A row of 8192 points is split as
// n = n_ab + 1024 n_c, n_ab = n_a + 32 n_b, and bin f2 = f_c + 8 f_b + 256 f_a:
//
//   X[f2] = sum_{n_a} w32^{n_a f_a} w1024^{n_a f_b} sum_{n_b} w32^{n_b f_b}
//             [ w8192^{n_ab f_c} sum_{n_c} w8^{n_c f_c} x[n] ]
//
//   phase 1 (VALU)  per column n_ab: the 8-point DFT over n_c and the twiddle,
//                   into LDS as the fp16 operand rows of the chains (row, f_c);
//   phase 2 (MFMA)  per chain: S1 contracts n_b, twiddle, S2 contracts n_a;
//                   the bin-pair step (filter product and repacking); then the
//                   same stages in the forward direction on conj(Z'), which
//                   gives conj of the inverse transform (S2'' contracts f_a,
//                   twiddle, S1'' contracts f_b, outer twiddle), into LDS;
//   phase 3 (VALU)  per column: the 8-point DFT over f_c, store.
//
// Wave w owns the chains (A, f_c = w) and (B, f_c = 7 - w).  Bin f2 of row A
// pairs with bin 8191 - f2 of row B, which is bin (7 - f_c, 31 - f_b, 31 - f_a)
// of chain (B, 7 - w): tile (1 - mt2, 1 - nt), lane 63 - l, element 3 - i, so
// one lane permutation (ds_bpermute) brings every pair into one lane.  The
// filter rows are stored in the same order (mp_chain_pos): each lane reads the
// four bins of a tile as one 16-byte word.
namespace mm {
using namespace cmfma;
constexpr int kR2Stride = 34;                          // complex values per (chain, n_a) row of R2
constexpr size_t kR1Bytes = (size_t)2 * 16 * 1024 * 2;  // two fp16 planes of 16 chains x 1024
constexpr size_t kR2Bytes = (size_t)16 * 32 * kR2Stride * 4;
constexpr size_t kLds = kR1Bytes > kR2Bytes ? kR1Bytes : kR2Bytes;

__device__ __forceinline__ uint32_t bperm(uint32_t addr, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute((int)addr, (int)v);
}
__device__ __forceinline__ float2 h2f(uint32_t d) {
    const __half2 v = *reinterpret_cast<const __half2 *>(&d);
    return __half22float2(v);
}
__device__ __forceinline__ uint32_t f2h(float2 v) {
    const __half2 h = __floats2half2_rn(v.x, v.y);
    return *reinterpret_cast<const uint32_t *>(&h);
}
// exp(-2 pi i e / 64), e < 4, and exp(-2 pi i / 128)
__device__ __forceinline__ float2 w64(int e) {
    switch (e) {
    case 0: return make_float2(1.0f, 0.0f);
    case 1: return make_float2(9.951847267e-01f, -9.801714033e-02f);
    case 2: return make_float2(9.807852804e-01f, -1.950903220e-01f);
    default: return make_float2(9.569403357e-01f, -2.902846773e-01f);
    }
}
constexpr float kW128c = 9.987954562e-01f, kW128s = -4.906767433e-02f;

// 8-point DFT of complex values held as (re, im) fp16 pairs, out[q] = sum_r in[r] w8^{rq},
// in packed fp16 arithmetic (fp16 storage: the values are fp16 before and after, and a
// DFT-8 grows no partial sum beyond its largest output); radix 2 in time, as Dft<8>.
__device__ __forceinline__ h2v h_negi(h2v a) { return h2v{a[1], -a[0]}; }   // -i a
__device__ __forceinline__ void dft4h(h2v a0, h2v a1, h2v a2, h2v a3, h2v *o) {
    const h2v s0 = a0 + a2, d0 = a0 - a2, s1 = a1 + a3, d1 = h_negi(a1 - a3);
    o[0] = s0 + s1;
    o[2] = s0 - s1;
    o[1] = d0 + d1;
    o[3] = d0 - d1;
}
__device__ __forceinline__ void dft8h(h2v *a) {
    h2v E[4], O[4];
    dft4h(a[0], a[2], a[4], a[6], E);
    dft4h(a[1], a[3], a[5], a[7], O);
    const _Float16 c = (_Float16)7.071067812e-01f;
    // w8^q O[q]: q = 1: ((x + y) c, (y - x) c); q = 2: -i O; q = 3: ((y - x) c, -(x + y) c)
    const h2v t1 = h2v{O[1][0] + O[1][1], O[1][1] - O[1][0]} * c;
    const h2v t2 = h_negi(O[2]);
    const h2v t3 = h2v{O[3][1] - O[3][0], -(O[3][0] + O[3][1])} * c;
    a[0] = E[0] + O[0];
    a[4] = E[0] - O[0];
    a[1] = E[1] + t1;
    a[5] = E[1] - t1;
    a[2] = E[2] + t2;
    a[6] = E[2] - t2;
    a[3] = E[3] + t3;
    a[7] = E[3] - t3;
}
}  // namespace mm

struct MmTables {
    const void *fr, *fi;   // DFT-32 operand tiles [2][64 lanes] x 8 fp16
    const void *tw1;       // w1024^{n_a f_b} in the S1 output layout [mt][nt][lane]: cos[4], sin[4]
    const void *tw3;       // conj of w1024^{n_a f_b} in the S2'' output layout [nt][nt2][lane]
    // S2 (A operand, rows f_a in the tile order row_fa) and S2'' (B operand, K slots
    // f_a in that order): DFT-32 tiles [2][64 lanes] x 8 fp16 (re, im)
    const void *far_, *fai_, *fbr_, *fbi_;
    const void *rtw;       // outer twiddle omega_8192^{f_c n_ab}: [f_c][q][n_a] x (cos[4], sin[4])
};

// grid (N1 / 2, nseq); block 512; dynamic LDS mm::kLds.
template <int LOG1, typename T, bool MASKED>
__global__ void __launch_bounds__(kMpThreads, 4)
mp_pass2m_kernel(T *__restrict__ ws, float2 *__restrict__ self_area, const __half2 *__restrict__ kbins,
                 const float *__restrict__ kscale, const uint8_t *__restrict__ mask, int64_t H, int64_t seq0,
                 MpArgs ta, MmTables mt) {
    using namespace mm;
    constexpr int N1 = 1 << LOG1, N2 = 1 << kMpLog2;
    constexpr int64_t NC = (int64_t)N1 * N2;
    extern __shared__ __align__(16) _Float16 smem[];
    _Float16 *const P0 = smem;                   // R1 plane re: [chain 16][chunk 4][n_a 32][8]
    _Float16 *const P1 = smem + 16 * 1024;       // R1 plane im
    char *const R2 = reinterpret_cast<char *>(smem);   // [chain 16][n_a 32][kR2Stride] half2
    const int tid = threadIdx.x;
    // Workgroup order: the nseq workgroups of the self-paired rows (f1 = 0), which
    // take about three times as long, come first and spread over the XCDs; then
    // f1 = 1 .. N1/2 - 1 of every sequence.
    const uint32_t wg = blockIdx.x + gridDim.x * blockIdx.y, nseq = gridDim.y;
    int f1;
    uint32_t sq;
    if (wg < nseq) {
        f1 = 0;
        sq = wg;
    } else {
        const uint32_t j = wg - nseq;
        f1 = 1 + (int)(j % (uint32_t)(N1 / 2 - 1));
        sq = j / (uint32_t)(N1 / 2 - 1);
    }
    f1 = __builtin_amdgcn_readfirstlane(f1);
    sq = __builtin_amdgcn_readfirstlane(sq);
    const int rowA = f1, rowB = f1 == 0 ? N1 / 2 : N1 - f1;
    const int64_t s = seq0 + sq;
    const int64_t h = s % H;
    T *const wsq = ws + 2 * (int64_t)sq * NC;
    BlockMask bm{~0ull, ~0ull};
    if (MASKED) {
        const uint8_t *mrow = mask + h * kMaskBlocks;
        bm.lo = __builtin_amdgcn_ballot_w64(mrow[tid & 63] != 0);
        bm.hi = __builtin_amdgcn_ballot_w64(mrow[64 + (tid & 63)] != 0);
    }

    // ---- phase 1: lane (row r, quad q, n_a) holds columns n_ab = n_a + 32 (4 q + k), k < 4
    {
        const int r = __builtin_amdgcn_readfirstlane(tid >> 8), q = (tid >> 5) & 7, na = tid & 31;
        const T *rowp = wsq + 2 * (int64_t)(r ? rowB : rowA) * N2;
        const uint32_t lo = (uint32_t)(na + 128 * q);
        // n_b = 4q + k sits in K slot kslot(n_b): chunk q & 3, slot 4 (q >> 2) + k.  The
        // twiddle omega_8192^{n_ab f_c} of the four columns is one fp16 table word
        // (the same table as the inverse chain's outer twiddle), applied to the fp16 planes.
        const uint32_t o = (uint32_t)((q & 3) * 256 + na * 8 + 4 * (q >> 2));
        auto put = [&](int fc, h4 re, h4 im) {
            const uint32_t oc = (uint32_t)((r * 8 + fc) * 1024) + o;
            if (fc > 0) cmul4(re, im, ldu<h8>(mt.rtw, 16u * (uint32_t)((fc * 8 + q) * 32 + na)));
            *reinterpret_cast<h4 *>(P0 + oc) = re;
            *reinterpret_cast<h4 *>(P1 + oc) = im;
        };
        if constexpr (std::is_same<T, __half>::value) {   // the DFT-8 in packed fp16
            h2v y[4][8];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int nc = 0; nc < 8; ++nc)
                    y[k][nc] = __builtin_bit_cast(h2v, ldu<uint32_t>(rowp + 2 * (32 * k + 1024 * nc), 4u * lo));
#pragma unroll
            for (int k = 0; k < 4; ++k) dft8h(y[k]);
#pragma unroll
            for (int fc = 0; fc < 8; ++fc)
                put(fc, h4{y[0][fc][0], y[1][fc][0], y[2][fc][0], y[3][fc][0]},
                    h4{y[0][fc][1], y[1][fc][1], y[2][fc][1], y[3][fc][1]});
        } else {
            float2 y[4][8];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int nc = 0; nc < 8; ++nc) y[k][nc] = io<T>::load2(rowp + 2 * (32 * k + 1024 * nc), lo);
#pragma unroll
            for (int k = 0; k < 4; ++k) dft_inplace<8>(y[k]);
#pragma unroll
            for (int fc = 0; fc < 8; ++fc)
                put(fc, h4{(_Float16)y[0][fc].x, (_Float16)y[1][fc].x, (_Float16)y[2][fc].x, (_Float16)y[3][fc].x},
                    h4{(_Float16)y[0][fc].y, (_Float16)y[1][fc].y, (_Float16)y[2][fc].y, (_Float16)y[3][fc].y});
        }
    }
    __syncthreads();

    // ---- phase 2
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, c = lane & 15;
    const int fcA = wave, fcB = 7 - wave;
    const uint32_t ul = (uint32_t)lane;
    h8 ar[2][2], ai[2][2];   // [chain A / B][mt]: rows n_a = 16 mt + c, K slots 8g..8g+7
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
        const int ch = qc ? 8 + fcB : fcA;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int o = ch * 1024 + g * 256 + (16 * m + c) * 8;
            ar[qc][m] = *reinterpret_cast<const h8 *>(P0 + o);
            ai[qc][m] = *reinterpret_cast<const h8 *>(P1 + o);
        }
    }
    // every wave has its operands; R1 becomes R2 below
    __syncthreads();

    // the DFT-32 operand tiles are read (from the L1 cache) where each stage uses them,
    // so that none is held across the bin-pair step; the negated imaginary plane is
    // formed where it is used
    auto ftile = [&](const void *tab, int t) { return ldu<h8>(tab, 16u * (t * 64 + ul)); };

    // S1 (data A: rows n_a, K = n_b; const B: F, N = f_b) and the twiddle w1024^{n_a f_b}
    h4 t1r[2][2][2], t1i[2][2][2];   // [chain][mt][nt]
    h8 Fr[2], Fi[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        Fr[t] = ftile(mt.fr, t);
        Fi[t] = ftile(mt.fi, t);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const h8 tw = ldu<h8>(mt.tw1, 16u * ((m * 2 + n) * 64 + ul));
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                f4 cr, ci;
                cm_dataA(ar[qc][m], ai[qc][m], Fr[n], Fi[n], neg8(Fi[n]), cr, ci);
                t1r[qc][m][n] = to_h4(cr);
                t1i[qc][m][n] = to_h4(ci);
                cmul4(t1r[qc][m][n], t1i[qc][m][n], tw);
            }
        }

    // S2 (const A: F rows f_a; data B: T1, K = n_a) tile pair by tile pair, the
    // bin-pair step on (A tile (m2, n), mirrored B tile (1 - m2, 1 - n)).  The
    // stored bins (|K s_h| <= 2^14) enter the product times 2^-kRowKLog2; pass 3
    // applies the channel scale.
    const float ks = __builtin_ldexpf(1.f, -kRowKLog2);
    const __half2 *kA = kbins + h * NC + (int64_t)rowA * N2 + fcA * 1024;
    const __half2 *kB = kbins + h * NC + (int64_t)rowB * N2 + fcB * 1024;
    const uint32_t maddr = 4u * (63u - ul);
    // keep bits of this lane's 16 bins of row A (bit 4 (2 m2 + n) + e) and of their
    // row-B partners (bit 16 + the same); the block of A's bin is
    // 4 f_a + 2 n + (c >> 3) with f_a = row_fa(m2, 4 g + e), its partner's 127 minus that
    uint32_t kbits = 0xffffffffu;
    // skip[m2]: no bin of tile m2 (row A) nor of its partners (row B) is kept by the
    // mask, in any lane: the pair's products are zero, so the tile's S2 products,
    // filter loads and bin-pair step are skipped (the same for every wave: a bin's
    // block does not depend on f_c)
    bool skip[2] = {false, false};
    if (MASKED) {
        kbits = 0;
        // the blocks 4 f_a + 2 n + (c >> 3) of A's bins are bits 2 n + (c >> 3) of mask
        // nibble f_a; their partners 127 minus that are bits 3 - 2 n - (c >> 3) of nibble 31 - f_a
        const uint32_t cb = (uint32_t)(c >> 3);
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int fa = row_fa(m2, 4 * g + e);
                const uint32_t na_ = bm.nibble(fa) >> cb, nb_ = bm.nibble(31 - fa) << cb;
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int bit = 4 * (2 * m2 + n) + e;
                    kbits |= ((na_ >> (2 * n)) & 1u) << bit;
                    kbits |= ((nb_ >> (3 - 2 * n)) & 1u) << (16 + bit);
                }
            }
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
            skip[m2] = __builtin_amdgcn_ballot_w64((((kbits >> (8 * m2)) | (kbits >> (16 + 8 * m2))) & 0xffu) != 0) == 0;
    }
    // twiddle of A's bin f2 = f_c + 8 (16 n + c) + 256 f_a, f_a = row_fa(m2, 4 g + e):
    // omega_2N^{rowA + N1 f2} = w2row[rowA] omega_{2 N2}^{f2}; row_fa adds 16 to 4 g + e
    // in tile 0 for g >= 2 (omega_{2 N2}^{4096} = -i) and 8 in tile 1 (omega_{2 N2}^{2048})
    const float2 wbase = cmul(ta.w2row[rowA], ldu<float2>(ta.w2n2, 8u * (uint32_t)(fcA + 8 * c + 1024 * g)));
    float2 *const area = self_area + (int64_t)sq * 2 * N2;
    // conj(Z') of the wave's two chains as fp16 tiles in LDS (the R2 region, free
    // until the barrier below): [wave][chain][m2][n][lane] x (re h4, im h4)
    char *const Yw = reinterpret_cast<char *>(smem) + wave * 8192;
    auto yput = [&](int qc, int m2, int n, uint32_t ln, const h4 &re, const h4 &im) {
        stu(Yw, 16u * (((qc * 2 + m2) * 2 + n) * 64 + ln), cat8(re, im));
    };
    if (f1 == 0) {
        // rows 0 and N1/2 pair with themselves: their spectra go to the area in
        // natural order (the products are formed once more below)
#pragma unroll
        for (int qc = 0; qc < 2; ++qc)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const h8 br = cat8(t1r[qc][0][n], t1r[qc][1][n]), bi = cat8(t1i[qc][0][n], t1i[qc][1][n]);
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    f4 zr, zi;
                    const h8 far_ = ftile(mt.far_, m2), fai_ = ftile(mt.fai_, m2);
                    cm_constA(far_, fai_, neg8(fai_), br, bi, zr, zi);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = (qc ? fcB : fcA) + 8 * (16 * n + c) + 256 * row_fa(m2, 4 * g + e);
                        area[qc * N2 + f] = make_float2(zr[e], zi[e]);
                    }
                }
            }
        // The barriers (workgroup scope) order the area's global writes and reads
        // across the waves, which share one CU's L1.
        __syncthreads();
        self_pairs<N1, N2, __half2, false, MASKED>(area, kbins + h * NC, nullptr, bm, ks, ta, tid, 1.0f);
        __syncthreads();
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                f4 ra, ia, rb, ib;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int fA = fcA + 8 * (16 * n + c) + 256 * row_fa(m2, 4 * g + e);
                    const int fB = fcB + 8 * (16 * n + c) + 256 * row_fa(m2, 4 * g + e);
                    const float2 va = area[fA], vb = area[N2 + fB];
                    ra[e] = va.x;
                    ia[e] = va.y;
                    rb[e] = vb.x;
                    ib[e] = vb.y;
                }
                yput(0, m2, n, ul, to_h4(ra), to_h4(ia));
                yput(1, m2, n, ul, to_h4(rb), to_h4(ib));
            }
    } else {
        // (n outer: the S1 results of A's column tile n and B's 1 - n die after two tile pairs)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                // (a scheduling fence per tile pair keeps the next pair's products and
                // loads from being hoisted here, which would exceed the register budget)
                __builtin_amdgcn_sched_barrier(0);
                // A's tile (m2, n) pairs with B's tile (m2, 1 - n): f_a -> 31 - f_a stays in
                // its tile (row_fa), f_b -> 31 - f_b flips the column tile
                const int mb = m2, nb = 1 - n;
                if (MASKED && skip[m2]) {
                    // every product of this tile pair is zero: its S2 products, filter loads
                    // and bin-pair step are skipped (frequency-sparse filter)
                    const h4 z4 = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
                    yput(0, m2, n, ul, z4, z4);
                    yput(1, mb, nb, ul, z4, z4);
                    continue;
                }
                const h8 far_ = ftile(mt.far_, m2), fai_ = ftile(mt.fai_, m2);
                // filter bins: A's tile (m2, n) and B's tile (mb, nb) read from lane 63 - l
                uint4 qa, qb;
                const uint32_t ea = 16u * ((m2 * 2 + n) * 64 + ul), eb = 16u * ((mb * 2 + nb) * 64 + (63u - ul));
                const int kb0 = 4 * (2 * m2 + n);
                if (MASKED) {
                    const bool anyA = ((kbits >> kb0) & 15u) != 0, anyB = ((kbits >> (16 + kb0)) & 15u) != 0;
                    qa = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       buffer_view(kA, 4096u), anyA ? ea : kBufferSkip, 0, 0));
                    qb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       buffer_view(kB, 4096u), anyB ? eb : kBufferSkip, 0, 0));
                } else {
                    qa = ldu<uint4>(kA, ea);
                    qb = ldu<uint4>(kB, eb);
                }
                f4 zr, zi, mr, mi;
                {
                    const h8 br = cat8(t1r[0][0][n], t1r[0][1][n]), bi = cat8(t1i[0][0][n], t1i[0][1][n]);
                    cm_constA(far_, fai_, neg8(fai_), br, bi, zr, zi);
                }
                {
                    f4 pr, pi;
                    const h8 br = cat8(t1r[1][0][nb], t1r[1][1][nb]), bi = cat8(t1i[1][0][nb], t1i[1][1][nb]);
                    cm_constA(far_, fai_, neg8(fai_), br, bi, pr, pi);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        mr[e] = __uint_as_float(bperm(maddr, __float_as_uint(pr[3 - e])));
                        mi[e] = __uint_as_float(bperm(maddr, __float_as_uint(pi[3 - e])));
                    }
                }
                uint32_t ka[4] = {qa.x, qa.y, qa.z, qa.w}, kb[4] = {qb.w, qb.z, qb.y, qb.x};
                if (MASKED) {
                    // a dropped bin reads as zero (the whole word: both halves of the value)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ka[e] &= 0u - ((kbits >> (kb0 + e)) & 1u);
                        kb[e] &= 0u - ((kbits >> (16 + kb0 + e)) & 1u);
                    }
                }
                const float2 wm = m2 ? cmul(wbase, make_float2(7.071067812e-01f, -7.071067812e-01f))
                                     : (g >= 2 ? cmul_negi(wbase) : wbase);
                const float2 wt = cmul(wm, make_float2(n ? kW128c : 1.f, n ? kW128s : 0.f));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float2 Ka = cscale(h2f(ka[e]), ks), Kb = cscale(h2f(kb[e]), ks);
                    float2 zf = make_float2(zr[e], zi[e]), zg = make_float2(mr[e], mi[e]);
                    middle_pair(zf, zg, Ka, Kb, cmul(wt, w64(e)));
                    zr[e] = zf.x;
                    zi[e] = zf.y;
                    mr[e] = zg.x;
                    mi[e] = zg.y;
                }
                yput(0, m2, n, ul, to_h4(zr), to_h4(zi));
                // B's values go to lane 63 - l of its own layout, elements reversed
                const h4 qr = to_h4(mr), qi = to_h4(mi);
                yput(1, mb, nb, 63u - ul, h4{qr[3], qr[2], qr[1], qr[0]}, h4{qi[3], qi[2], qi[1], qi[0]});
            }
    }
    // forward-direction stages on conj(Z'): S2'' (data A: rows f_b, K = f_a;
    // const B: F, N = n_a), twiddle w1024^{n_a f_b}; S1'' (const A: F rows n_b;
    // data B: K = f_b), outer twiddle w8192^{n_ab f_c}; into R2 as half2
    h4 t3r[2][2][2], t3i[2][2][2];   // [chain][n (f_b tile)][n2 (n_a tile)]
#pragma unroll
    for (int qc = 0; qc < 2; ++qc)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const h8 y0 = ldu<h8>(Yw, 16u * (((qc * 2 + 0) * 2 + n) * 64 + ul));
            const h8 y1 = ldu<h8>(Yw, 16u * (((qc * 2 + 1) * 2 + n) * 64 + ul));
            const h8 dr = cat8(lo4(y0), lo4(y1)), di = cat8(hi4(y0), hi4(y1));
#pragma unroll
            for (int n2 = 0; n2 < 2; ++n2) {
                f4 cr, ci;
                // K slots 8g + j: f_a = row_fa(j / 4, 4g + j % 4), the order of the Y tiles
                const h8 fbr = ftile(mt.fbr_, n2), fbi = ftile(mt.fbi_, n2);
                cm_dataA(dr, di, fbr, fbi, neg8(fbi), cr, ci);
                t3r[qc][n][n2] = to_h4(cr);
                t3i[qc][n][n2] = to_h4(ci);
                h8 tw = ldu<h8>(mt.tw3, 16u * ((n * 2 + n2) * 64 + ul));
                tw = cat8(lo4(tw), -hi4(tw));   // the table holds the conjugate
                cmul4(t3r[qc][n][n2], t3i[qc][n][n2], tw);
            }
        }
    // every wave has read its tiles: the region becomes R2
    __syncthreads();
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
        const int fc = qc ? fcB : fcA;
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
            const h8 br = cat8(t3r[qc][0][n2], t3r[qc][1][n2]), bi = cat8(t3i[qc][0][n2], t3i[qc][1][n2]);
#pragma unroll
            for (int n3 = 0; n3 < 2; ++n3) {
                f4 cr, ci;
                const h8 fr3 = ftile(mt.fr, n3), fi3 = ftile(mt.fi, n3);
                cm_constA(fr3, fi3, neg8(fi3), br, bi, cr, ci);   // rows n_b = 16 n3 + 4g + e, col n_a
                // outer twiddle omega_8192^{f_c n_ab} of (n_a = 16 n2 + c, n_b = 4 (4 n3 + g) + e):
                // the table word (f_c, q = 4 n3 + g, n_a), applied to the fp16 planes
                h4 tr = to_h4(cr), ti = to_h4(ci);
                cmul4(tr, ti, ldu<h8>(mt.rtw, 16u * (uint32_t)((fc * 8 + 4 * n3 + g) * 32 + 16 * n2 + c)));
                uint32_t d[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) d[e] = __builtin_bit_cast(uint32_t, h2v{tr[e], ti[e]});
                // R2[chain][n_a][n_b]: n_b = 16 n3 + 4 g + e are consecutive
                const uint32_t o = (uint32_t)((((qc * 8 + fc) * 32 + 16 * n2 + c) * kR2Stride + 16 * n3 + 4 * g) * 4);
                stu(R2, o, make_uint2(d[0], d[1]));
                stu(R2, o + 8u, make_uint2(d[2], d[3]));
            }
        }
    }
    __syncthreads();

    // ---- phase 3: lane (row r, quad q, n_a): the 8-point DFT over f_c of columns
    // n_ab = n_a + 32 (4 q + k), outputs n_c; store
    {
        const int tid2 = launder(tid);
        const int r = __builtin_amdgcn_readfirstlane(tid2 >> 8), q = (tid2 >> 5) & 7, na = tid2 & 31;
        T *rowp = wsq + 2 * (int64_t)(r ? rowB : rowA) * N2;
        const uint32_t lo = (uint32_t)(na + 128 * q);
        if constexpr (std::is_same<T, __half>::value) {   // the DFT-8 in packed fp16
            h2v y[4][8];
#pragma unroll
            for (int fc = 0; fc < 8; ++fc) {
                const uint32_t o = (uint32_t)((((r * 8 + fc) * 32 + na) * kR2Stride + 4 * q) * 4);
                const uint2 a = ldu<uint2>(R2, o), b = ldu<uint2>(R2, o + 8u);
                y[0][fc] = __builtin_bit_cast(h2v, a.x);
                y[1][fc] = __builtin_bit_cast(h2v, a.y);
                y[2][fc] = __builtin_bit_cast(h2v, b.x);
                y[3][fc] = __builtin_bit_cast(h2v, b.y);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                dft8h(y[k]);
#pragma unroll
                for (int nc = 0; nc < 8; ++nc)
                    stu(rowp + 2 * (32 * k + 1024 * nc), 4u * lo, __builtin_bit_cast(uint32_t, y[k][nc]));
            }
        } else {
            float2 y[4][8];
#pragma unroll
            for (int fc = 0; fc < 8; ++fc) {
                const uint32_t o = (uint32_t)((((r * 8 + fc) * 32 + na) * kR2Stride + 4 * q) * 4);
                const uint2 a = ldu<uint2>(R2, o), b = ldu<uint2>(R2, o + 8u);
                y[0][fc] = h2f(a.x);
                y[1][fc] = h2f(a.y);
                y[2][fc] = h2f(b.x);
                y[3][fc] = h2f(b.y);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                dft_inplace<8>(y[k]);
#pragma unroll
                for (int nc = 0; nc < 8; ++nc) io<T>::store2(rowp + 2 * (32 * k + 1024 * nc), lo, y[k][nc]);
            }
        }
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
    a->col = static_cast<const uint4 *>(mt.col);
    return hipSuccess;
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
    using P = ColPlan<LOG1>;
    constexpr int N2 = 1 << kMpLog2;
    MpArgs ta{};
    hipError_t e = mp_args(LOG1 + kMpLog2, &ta);
    if (e != hipSuccess) return e;
    T *ws = (T *)work;
    float2 *self_area = (float2 *)((char *)work + (size_t)nseq * ((size_t)1 << (LOG1 + kMpLog2)) * 2 * sizeof(T));
    constexpr bool kHalf = std::is_same<TK, __half2>::value;
    // half-precision storage and N1 >= 2^kMpColMinLog1: column passes on the matrix cores
    constexpr bool kColMm = kHalf && LOG1 >= kMpColMinLog1;
    if constexpr (kColMm) {
        if (ta.col == nullptr) return hipErrorNotInitialized;
        auto k1 = mp_pass1c_kernel<LOG1, T>;
        if ((e = allow_lds(k1, ColMm<LOG1>::kLds)) != hipSuccess) return e;
        hipLaunchKernelGGL(k1, dim3(N2 / 32, (unsigned)nseq), dim3(kMpThreads), ColMm<LOG1>::kLds, stream,
                           (const T *)u, (const T *)w, seq0, ws, ta);
    } else {
        auto k1 = mp_pass1_kernel<LOG1, T, false>;
        if ((e = allow_lds(k1, P::kLds)) != hipSuccess) return e;
        hipLaunchKernelGGL(k1, dim3(N2 / P::C, (unsigned)nseq), dim3(kMpThreads), P::kLds, stream,
                           (const T *)u, (const T *)w, (int64_t)0, seq0, ws, ta);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 g2((1 << LOG1) / 2, (unsigned)nseq);
    if constexpr (std::is_same<TK, __half2>::value) {
        // half-precision storage: the row pass on the matrix cores
        Pair3Tables p3{};
        if ((e = get_pair3_tables(&p3)) != hipSuccess) return e;
        const MmTables mt{p3.fr, p3.fi, p3.tw1, p3.tw3, p3.far_, p3.fai_, p3.fbr_, p3.fbi_, p3.rtw};
        auto k2 = mask != nullptr ? mp_pass2m_kernel<LOG1, T, true> : mp_pass2m_kernel<LOG1, T, false>;
        if ((e = allow_lds(k2, mm::kLds)) != hipSuccess) return e;
        hipLaunchKernelGGL(k2, g2, dim3(kMpThreads), mm::kLds, stream, ws, self_area, (const __half2 *)kbins,
                           kscale, mask, H, seq0, ta, mt);
    } else {
        auto k2 = mask != nullptr ? mp_pass2_kernel<LOG1, T, TK, false, true>
                                  : mp_pass2_kernel<LOG1, T, TK, false, false>;
        if ((e = allow_lds(k2, kP2Lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(k2, g2, dim3(kMpThreads), kP2Lds, stream, ws, self_area, (const TK *)kbins,
                           (TK *)nullptr, kscale, mask, H, seq0, ta, 1.0f);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if constexpr (kColMm) {
        auto k3 = mp_pass3c_kernel<LOG1, T>;
        if ((e = allow_lds(k3, ColMm<LOG1>::kLds)) != hipSuccess) return e;
        hipLaunchKernelGGL(k3, dim3(N2 / 32, (unsigned)nseq), dim3(kMpThreads), ColMm<LOG1>::kLds, stream,
                           (const T *)ws, (const T *)v, (T *)out, seq0, ta, kscale, H);
    } else {
        auto k3 = mp_pass3_kernel<LOG1, T, kHalf>;
        if ((e = allow_lds(k3, P::kLds)) != hipSuccess) return e;
        hipLaunchKernelGGL(k3, dim3(N2 / P::C, (unsigned)nseq), dim3(kMpThreads), P::kLds, stream,
                           (const T *)ws, (const T *)v, (T *)out, seq0, ta, kscale, H);
    }
    return hipGetLastError();
}

template <int LOG1, typename T, typename TK>
static hipError_t prep_t(const void *k, int64_t L, void *kbins, const float *kscale, void *work,
                         int64_t H, int64_t h0, int64_t nseq, float ysgn, hipStream_t stream) {
    using P = ColPlan<LOG1>;
    constexpr int N2 = 1 << kMpLog2;
    MpArgs ta{};
    hipError_t e = mp_args(LOG1 + kMpLog2, &ta);
    if (e != hipSuccess) return e;
    T *ws = (T *)work;
    float2 *self_area = (float2 *)((char *)work + (size_t)nseq * ((size_t)1 << (LOG1 + kMpLog2)) * 2 * sizeof(T));
    auto k1 = mp_pass1_kernel<LOG1, T, true>;
    auto k2 = mp_pass2_kernel<LOG1, T, TK, true, false>;
    if ((e = allow_lds(k1, P::kLds)) != hipSuccess) return e;
    if ((e = allow_lds(k2, kP2Lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(k1, dim3(N2 / P::C, (unsigned)nseq), dim3(kMpThreads), P::kLds, stream,
                       (const T *)k, (const T *)nullptr, L, h0, ws, ta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k2, dim3((1 << LOG1) / 2, (unsigned)nseq), dim3(kMpThreads), kP2Lds, stream,
                       ws, self_area, (const TK *)nullptr, (TK *)kbins, kscale, (const uint8_t *)nullptr,
                       H, h0, ta, ysgn);
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
                          void *work, int64_t H, int64_t h0, int64_t nseq, float ysgn, hipStream_t stream) {
    switch (st) {
    case ST_F32: return prep_t<LOG1, float, float2>(k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    case ST_F16: return prep_t<LOG1, __half, __half2>(k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    default:
        return prep_t<LOG1, __hip_bfloat16, __half2>(k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
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
                                    int64_t nseq, float ysgn, hipStream_t stream) {
    switch (logn - kMpLog2) {
    case 2: return prep_st<2>(st, k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    case 3: return prep_st<3>(st, k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    case 4: return prep_st<4>(st, k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    case 5: return prep_st<5>(st, k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    case 6: return prep_st<6>(st, k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    case 7: return prep_st<7>(st, k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    case 8: return prep_st<8>(st, k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    case 9: return prep_st<9>(st, k, L, kbins, kscale, work, H, h0, nseq, ysgn, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fftconv
