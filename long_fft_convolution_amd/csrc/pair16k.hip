// pair16k.hip -- gated causal FFT convolution for N = 16384 on the MFMA
// matrix cores (fp16 operands, fp32 accumulation), one sequence pair per
// workgroup with the whole 32768-point transform on chip.
//
// FlashFFTConv summary page, "Approach": order-p Monarch decomposition of the
// FFT into matrix-matrix products, permutations as on-chip transposes, the
// whole convolution fused.  Here the order is 3:
//
//   two same-channel sequences form z = x_a + i x_b (x = u * w), zero-padded
//   to M = 32768 = 32 * 32 * 32,  m = n_a + 32 n_b + 1024 n_c,
//   f = f_c + 32 f_b + 1024 f_a:
//
//   Z[f] = sum_{n_a} w32^{n_a f_a} w1024^{n_a f_b} sum_{n_b} w32^{n_b f_b}
//            [ wM^{(n_a + 32 n_b) f_c} sum_{n_c} w32^{n_c f_c} z[m] ]
//
//  phase 1  outer DFT-32 over n_c (only n_c < 16 is non-zero) for all
//           n_ab = n_a + 32 n_b, twiddle wM^{n_ab f_c}, into LDS rows f_c;
//  phase 2  per row f_c (each wave owns rows wave + 8 r): the 1024-point
//           two-stage chain of the N = 1024 kernel (contract n_b, twiddle,
//           contract n_a), the filter product, the inverse chain, the
//           conjugate outer twiddle, into LDS laid out by n_ab;
//  phase 3  outer inverse DFT-32 over f_c producing only n_c < 16 (outputs
//           t < N), output scale and gate, store.
//
// All six stages are complex-as-real v_mfma_f32_16x16x32_f16 products with
// one shared set of DFT-32 operand tiles (conjugated for the inverse).  The
// filter spectrum is stored for rows f_c = 0..16 only; a row f_c > 16 reads
// the Hermitian mirror row 32 - f_c (lane 63 - l, tiles flipped, elements
// reversed, conjugated).
#include "fft_device.hpp"
#include "fftconv_internal.hpp"
#include "cmfma.hpp"

#include <type_traits>

namespace fftconv {

namespace p16 {

using namespace cmfma;

// LDS layouts (fp16 element offsets within one plane)
constexpr int kR1Row = 1032;                 // 1024 + 8: rows f_c padded against bank conflicts
constexpr int kR1Plane = 32 * kR1Row;        // [f_c][chunk 4][rot(n_a) 32][8]
constexpr int kR2Plane = 32768;              // [chunk 4][n_ab 1024][8]
// R1 stores n_a at rot(n_a) = (n_a >> 1) | ((n_a & 1) << 4), so that the phase-1 writes of
// the 16 lanes holding n_a = 2c + parity fall on 16 distinct bank groups
__device__ __forceinline__ int r1(int fc, int ks, int na) {
    return fc * kR1Row + (ks >> 3) * 256 + ((na >> 1) | ((na & 1) << 4)) * 8 + (ks & 7);
}
__device__ __forceinline__ int r2(int ks, int nab) { return (ks >> 3) * 8192 + nab * 8 + (ks & 7); }

template <typename T> struct st;
template <> struct st<__half> {
    static __device__ __forceinline__ float cvt_half(uint32_t d, int hi) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(hi ? d >> 16 : d));
    }
    static __device__ __forceinline__ float ld(const __half *p) { return (float)*reinterpret_cast<const _Float16 *>(p); }
    static __device__ __forceinline__ void unpack4(const uint2 &raw, float *o) {
        const _Float16 *hv = reinterpret_cast<const _Float16 *>(&raw);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (float)hv[i];
    }
    static __device__ __forceinline__ uint2 pack4(const float *v) {
        _Float16 hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = (_Float16)v[i];
        return *reinterpret_cast<const uint2 *>(hv);
    }
};
template <> struct st<__hip_bfloat16> {
    static __device__ __forceinline__ float cvt_half(uint32_t d, int hi) {
        return __uint_as_float(hi ? d & 0xffff0000u : d << 16);
    }
    static __device__ __forceinline__ float ld(const __hip_bfloat16 *p) {
        return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t *>(p)) << 16);
    }
    static __device__ __forceinline__ void unpack4(const uint2 &raw, float *o) {
        o[0] = __uint_as_float(raw.x << 16);
        o[1] = __uint_as_float(raw.x & 0xffff0000u);
        o[2] = __uint_as_float(raw.y << 16);
        o[3] = __uint_as_float(raw.y & 0xffff0000u);
    }
    static __device__ __forceinline__ uint2 pack4(const float *v) {
        uint32_t w[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            __hip_bfloat16 a = __float2bfloat16(v[2 * i]), b = __float2bfloat16(v[2 * i + 1]);
            w[i] = (uint32_t)(*reinterpret_cast<uint16_t *>(&a)) |
                   ((uint32_t)(*reinterpret_cast<uint16_t *>(&b)) << 16);
        }
        return make_uint2(w[0], w[1]);
    }
};

constexpr int kWaves = 8;
constexpr int kTilesPerWave = 64 / kWaves;   // 16-column tiles of n_ab in phases 1 and 3
constexpr int kRowsPerWave = 32 / kWaves;    // rows f_c in phase 2
static_assert(kWaves == 8, "the LDS address split below assumes 8 waves");

// filter chunk of row fc for (mt2, nt): rows f_c <= 16 as stored, the others from
// the mirror row 32 - f_c (lane 63 - l, tiles flipped, elements reversed, conjugated)
__device__ __forceinline__ uint4 k_load(const uint4 *kch, int fc, int mt2, int nt, uint32_t lane) {
    const bool mir = fc > 16;
    const uint32_t row = mir ? 32 - fc : fc, a = mir ? 1 - mt2 : mt2, b = mir ? 1 - nt : nt;
    return ldu<uint4>(kch + ((row * 2 + a) * 2 + b) * 64, 16u * (mir ? 63 - lane : lane));
}
__device__ __forceinline__ h8 k_fix(const uint4 &q, bool mir) {
    if (!mir) return *reinterpret_cast<const h8 *>(&q);
    // (e0..e3 | e4..e7) -> (e3, e2, e1, e0 | -e7, -e6, -e5, -e4)
    uint4 t;
    t.x = __builtin_amdgcn_alignbit(q.y, q.y, 16);
    t.y = __builtin_amdgcn_alignbit(q.x, q.x, 16);
    t.z = __builtin_amdgcn_alignbit(q.w, q.w, 16) ^ 0x80008000u;
    t.w = __builtin_amdgcn_alignbit(q.z, q.z, 16) ^ 0x80008000u;
    return *reinterpret_cast<const h8 *>(&t);
}

}  // namespace p16

using namespace p16;

// grid: persistent, one workgroup (kWaves waves) per CU; each workgroup walks an
// XCD-local range of pairs p = h * ceil(B/2) + bp.  An odd B pairs its last row
// with zeros: the second row's loads then re-read the first row (always in
// bounds) and are discarded, so no load sits under a branch.
// DUAL: a second output out2 = v2 * conv(u w, k) from the same transforms (the backward
// pass forms du and dw in one call); the second gate's rows are loaded once the staged
// outputs have freed their registers.
template <typename T, bool MASKED, bool HAS_W, bool HAS_V, bool DUAL = false>
__global__ void __launch_bounds__(64 * kWaves, 1)
pair16k_kernel(const T *__restrict__ u, const T *__restrict__ w, const T *__restrict__ v,
               T *__restrict__ out, const uint4 *__restrict__ kbins, const float *__restrict__ kscale,
               const uint8_t *__restrict__ mask, Pair3Tables tb, int64_t B, int64_t H,
               const T *__restrict__ v2, T *__restrict__ out2) {
    static_assert(!DUAL || HAS_V, "a second output has an output gate of its own");
    constexpr int N = 16384;
    constexpr int M2 = 2 * N;
    extern __shared__ __align__(16) _Float16 smem[];
    _Float16 *P0 = smem;                    // plane 0 (re) of R1 / R2
    _Float16 *P1 = smem + kR1Plane;         // plane 1 (im)
    h8 *s_tw1 = reinterpret_cast<h8 *>(smem + 2 * kR1Plane);   // [mt][nt][lane]
    h8 *s_tw3 = s_tw1 + 4 * 64;                                 // [nt][nt2][lane]
    uint8_t *s_mask = reinterpret_cast<uint8_t *>(s_tw3 + 4 * 64);   // mask row of the pair's channel

    const int tid = threadIdx.x;
    for (int i = tid; i < 256; i += 64 * kWaves) {
        s_tw1[i] = reinterpret_cast<const h8 *>(tb.tw1)[i];
        s_tw3[i] = reinterpret_cast<const h8 *>(tb.tw3)[i];
    }
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, c = lane & 15;
    h8 Fr[2], Fi[2], nFi[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        Fr[t] = reinterpret_cast<const h8 *>(tb.fr)[t * 64 + lane];
        Fi[t] = reinterpret_cast<const h8 *>(tb.fi)[t * 64 + lane];
        nFi[t] = neg8(Fi[t]);
    }
    // outer twiddles of this wave's tiles [tq][nt][lane] and rows [r][nt3][nt2][lane]
    const h8 *twO1 = reinterpret_cast<const h8 *>(tb.two1) + wave * (kTilesPerWave * 2 * 64);
    const h8 *twO2 = reinterpret_cast<const h8 *>(tb.two2) + wave * (4 * 64);
    // Every LDS access below is a per-lane base plus a compile-time offset: r1() / r2()
    // split into lane, wave and constant parts (phase 1 writes, 2a reads, 2b writes, 3 reads).
    const int b1w = 4 * g * kR1Row + 8 * c + 256 * (wave & 3) + 4 * (wave >> 2);
    const int b2r = kR1Row * wave + 256 * g + 8 * (c >> 1) + 128 * (c & 1);
    const int b2w = 8192 * (wave >> 2) + (wave & 3) + 8 * c + 1024 * g;
    const int b3r = 1024 * wave + 8192 * g + 8 * c;
    // Phase-3 staging: fp32 rows rho = 16 seq + n_c of this wave's 128 n_ab, held in this
    // wave's own R2 bytes (plane rho >> 4, chunk (rho >> 2) & 3, n_ab 128 wave .. + 127:
    // 2 KB = four rows per piece); 16-byte units XOR-swizzled by 4 (n_c & 3).
    const uint32_t st_w = 2 * (8192 * (c >> 2) + 1024 * wave) + 512 * (c & 3) + 16 * g;   // + 64 (tt ^ (c & 3))
    const uint32_t st_r = 2 * 1024 * wave + 512 * (lane >> 4);
    const uint32_t st_r0 = st_r + 16 * ((2 * (lane & 15)) ^ (4 * (lane >> 4)));
    const uint32_t st_r1 = st_r + 16 * ((2 * (lane & 15) + 1) ^ (4 * (lane >> 4)));
    _Float16 *const w1r = P0 + b1w, *const w1i = P1 + b1w;
    const _Float16 *const r2r = P0 + b2r, *const r2i = P1 + b2r;
    _Float16 *const w2r = P0 + b2w, *const w2i = P1 + b2w;
    const _Float16 *const r3r = P0 + b3r, *const r3i = P1 + b3r;
    __syncthreads();

    const int64_t PB = (B + 1) / 2, P = H * PB;
    const uint32_t nwg = gridDim.x, xcd = blockIdx.x % 8, wg_local = blockIdx.x / 8;
    const uint32_t wg_on_xcd = nwg / 8 + (xcd < nwg % 8 ? 1u : 0u);
    const int64_t p_begin = P * xcd / 8, p_end = P * (xcd + 1) / 8;

    // per-lane element offset of phase 1 (n_ab = 128 wave + 2c, n_c = 4 g) and phase 3
    const uint32_t m1 = 16 * kTilesPerWave * wave + 2 * c + 4096 * g;
    // phase 3 stores rows of 128 contiguous n_ab: lane l covers n_c = 4k' + (l >> 4),
    // n_ab = 128 wave + 8 (l & 15) + 0..7
    const uint32_t m4 = 16 * kTilesPerWave * wave + 8 * (lane & 15) + 1024 * (lane >> 4);

    // The pair loop is software-pipelined: the first phase-1 batch of the next pair and
    // the output gate of this pair are loaded during the last row of phase 2, the second
    // batch while the first is transformed.  Raw 16-bit values are held until used.
    // Phase 1 reads one dword (two adjacent n_ab) per lane and element: lane (g, c) holds
    // n_ab = 128 wave + 32 q + 2c + par, n_c = 4g + j, for q = 0..3 (two per batch); the
    // 16-column tiles are (q, par), outer twiddle tables indexed by T = 8 wave + 2q + par.
    struct Batch {   // [q in batch][j] raw storage bits of two adjacent n_ab
        uint32_t xa[2][4], xb[2][4], ga[2][4], gb[2][4];
    };
    const uint32_t ul = lane;
    auto pair_base = [&](int64_t pp, int64_t &oa_, int64_t &ob_, bool &hb_) {
        // pairs < 2^31; the quotient is made wave-uniform so that all pair addresses are scalar
        const int64_t hh = __builtin_amdgcn_readfirstlane((uint32_t)pp / (uint32_t)PB), bpp = pp - hh * PB;
        hb_ = 2 * bpp + 1 < B;
        oa_ = (2 * bpp * H + hh) * N;
        ob_ = hb_ ? oa_ + H * N : oa_;
    };
    auto load_batch = [&](int64_t oa_, int64_t ob_, int half, Batch &x) {
        const uint32_t *pua = reinterpret_cast<const uint32_t *>(u + oa_);
        const uint32_t *pub = reinterpret_cast<const uint32_t *>(u + ob_);
        const uint32_t *pwa = reinterpret_cast<const uint32_t *>(w + oa_);
        const uint32_t *pwb = reinterpret_cast<const uint32_t *>(w + ob_);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = (32 * (2 * half + qq) + 1024 * j) / 2;   // in dwords
                x.xa[qq][j] = ldu<uint32_t>(pua + m, 2 * m1);
                x.xb[qq][j] = ldu<uint32_t>(pub + m, 2 * m1);
                if (HAS_W) {
                    x.ga[qq][j] = ldu<uint32_t>(pwa + m, 2 * m1);
                    x.gb[qq][j] = ldu<uint32_t>(pwb + m, 2 * m1);
                }
            }
    };
    auto load_tw = [&](int half, h8 (&tw)[2][2][2]) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int par = 0; par < 2; ++par)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    tw[qq][par][nt] = ldu<h8>(twO1 + ((2 * (2 * half + qq) + par) * 2 + nt) * 64, 16u * ul);
    };
    // phase 1 for one batch: outer DFT over n_c, outer twiddle, into R1; the two q of the
    // batch sit in adjacent K slots, so each (par, nt, i) is one 32-bit write per plane
    auto phase1_batch = [&](const Batch &x, const h8 (&tw)[2][2][2], int half, bool hb_) {
        h4 yr[2][2][2], yi[2][2][2];   // [qq][par][nt]
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int par = 0; par < 2; ++par) {
                h8 br, bi;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float xa = st<T>::cvt_half(x.xa[qq][j], par), xb = st<T>::cvt_half(x.xb[qq][j], par);
                    if (HAS_W) {
                        xa *= st<T>::cvt_half(x.ga[qq][j], par);
                        xb *= st<T>::cvt_half(x.gb[qq][j], par);
                    }
                    br[j] = (_Float16)xa;
                    bi[j] = hb_ ? (_Float16)xb : (_Float16)0.f;
                    br[4 + j] = (_Float16)0.f;
                    bi[4 + j] = (_Float16)0.f;
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f4 ar, ai;
                    cm_constA(Fr[nt], Fi[nt], nFi[nt], br, bi, ar, ai);   // rows f_c = 16nt + 4g + i, cols n_ab
                    yr[qq][par][nt] = to_h4(ar);
                    yi[qq][par][nt] = to_h4(ai);
                    cmul4(yr[qq][par][nt], yi[qq][par][nt], tw[qq][par][nt]);
                }
            }
#pragma unroll
        for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {   // r1(16 nt + 4 g + i, kslot(4 wave + q), 2c + par)
                    const int o = (16 * nt + i) * kR1Row + 128 * par + 2 * half;
                    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                    *reinterpret_cast<h2 *>(w1r + o) = h2{yr[0][par][nt][i], yr[1][par][nt][i]};
                    *reinterpret_cast<h2 *>(w1i + o) = h2{yi[0][par][nt][i], yi[1][par][nt][i]};
                }
    };

    int64_t p = p_begin + wg_local;
    if (p >= p_end) return;
    int64_t oa, ob;
    bool has_b;
    pair_base(p, oa, ob, has_b);
    Batch x0, x1;
    load_batch(oa, ob, 0, x0);
    load_batch(oa, ob, 1, x1);

    for (; p < p_end; p += wg_on_xcd) {
        const int64_t h = __builtin_amdgcn_readfirstlane((uint32_t)p / (uint32_t)PB);
        const float ks = kscale[h];
        int64_t p_nx = p + wg_on_xcd, oa_nx, ob_nx;
        bool hb_nx;
        pair_base(p_nx < p_end ? p_nx : p, oa_nx, ob_nx, hb_nx);

        // the mask row is read in phase 2 only, after the barrier that ends phase 1
        if (MASKED && tid < kMaskBlocks / 4)
            reinterpret_cast<uint32_t *>(s_mask)[tid] = reinterpret_cast<const uint32_t *>(mask + h * kMaskBlocks)[tid];

        // ---- phase 1: outer DFT over n_c for this wave's tiles T of n_ab, two batches
        // (loads are issued in the order they are consumed: vmcnt waits are in order)
        {
            h8 tw0[2][2][2], tw1[2][2][2];
            load_tw(0, tw0);
            load_tw(1, tw1);
            phase1_batch(x0, tw0, 0, has_b);
            phase1_batch(x1, tw1, 1, has_b);
        }
        __syncthreads();

        // ---- phase 2a: this wave's rows f_c = wave + kWaves r into registers (S1 operands);
        // R2 below reuses the same LDS
        h8 ar_[kRowsPerWave][2], ai_[kRowsPerWave][2];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {   // r1(wave + 8 r, 8 g, 16 mt + c)
                const int o = kWaves * kR1Row * r + 64 * mt;
                ar_[r][mt] = *reinterpret_cast<const h8 *>(r2r + o);
                ai_[r][mt] = *reinterpret_cast<const h8 *>(r2i + o);
            }
        }
        const uint4 *kch = kbins + h * (int64_t)(17 * 256);
        uint4 kq[2][2];
#pragma unroll
        for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) kq[mt2][nt] = k_load(kch, wave, mt2, nt, ul);
        __syncthreads();

        // ---- phase 2b: the 1024-point chain per row, filter product, inverse chain;
        // the next row's filter chunks are fetched while this row computes
        uint4 vq[8];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
            const int fc = wave + kWaves * r;
            // the lane offset is re-derived per row so that table byte offsets stay 32-bit
            // values of this block (a hoisted 64-bit address costs two registers per load)
            uint32_t lx = ul;
            asm volatile("" : "+v"(lx));
            h8 kk[2][2];
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) kk[mt2][nt] = k_fix(kq[mt2][nt], fc > 16);
            if (r + 1 < kRowsPerWave) {
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) kq[mt2][nt] = k_load(kch, fc + kWaves, mt2, nt, lx);
            }
            h8 two[2][2];
#pragma unroll
            for (int nt3 = 0; nt3 < 2; ++nt3)
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2)
                    two[nt3][nt2] = ldu<h8>(twO2 + ((kWaves * r * 2 + nt3) * 2 + nt2) * 64, 16u * lx);
            if (r == kRowsPerWave - 1) {   // output gate of this pair, first batch of the next
                if (HAS_V) {
#pragma unroll
                    for (int tt = 0; tt < kTilesPerWave; ++tt) {
                        vq[tt] = ldu_nt<uint4>(v + (tt < 4 ? oa : ob) + 4096 * (tt & 3), 2 * m4);
                    }
                }
                // pinned order: the gate is consumed first, and vmcnt waits are in order
                __builtin_amdgcn_sched_barrier(0);
                load_batch(oa_nx, ob_nx, 0, x0);
                __builtin_amdgcn_sched_barrier(0);
            }
            // S1: data A (M = n_a tiles mt, K = n_b), const B F[nt] (N = f_b); twiddle w1024^{n_a f_b}
            h4 t1r[2][2], t1i[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f4 cr, ci;
                    cm_dataA(ar_[r][mt], ai_[r][mt], Fr[nt], Fi[nt], nFi[nt], cr, ci);
                    t1r[mt][nt] = to_h4(cr);
                    t1i[mt][nt] = to_h4(ci);
                    cmul4(t1r[mt][nt], t1i[mt][nt], s_tw1[(mt * 2 + nt) * 64 + lane]);
                }
            }
            // S2: const A F[mt2] (M = f_a, K = n_a), data B = T1 (K = n_a, N = f_b); filter product
            h4 yr[2][2], yi[2][2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const h8 br = cat8(t1r[0][nt], t1r[1][nt]), bi = cat8(t1i[0][nt], t1i[1][nt]);
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2) {
                    f4 cr, ci;
                    cm_constA(Fr[mt2], Fi[mt2], nFi[mt2], br, bi, cr, ci);   // rows f_a, cols f_b
                    yr[mt2][nt] = to_h4(cr);
                    yi[mt2][nt] = to_h4(ci);
                    h8 kf = kk[mt2][nt];
                    if (MASKED) {
                        // block of bin f (or of its mirror 2N - f); the lane index is laundered
                        // so that these pair-invariant indices are recomputed, not held
                        int lc = c, lg = g;
                        asm volatile("" : "+v"(lc), "+v"(lg));
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int f = fc + 32 * (16 * nt + lc) + 1024 * (16 * mt2 + 4 * lg + i);
                            const int fr_ = f <= N ? f : M2 - f;
                            int blk = fr_ / (N / kMaskBlocks);
                            blk = blk > kMaskBlocks - 1 ? kMaskBlocks - 1 : blk;
                            if (!s_mask[blk]) kf[i] = kf[4 + i] = (_Float16)0.f;
                        }
                    }
                    cmul4(yr[mt2][nt], yi[mt2][nt], kf);
                }
            }
            // S2': data A = T2^T (M = f_b tiles nt, K = f_a), const B conj F[nt2] (N = n_a); conj twiddle
            h4 t3r[2][2], t3i[2][2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const h8 dr = cat8(yr[0][nt], yr[1][nt]), di = cat8(yi[0][nt], yi[1][nt]);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2) {
                    f4 cr, ci;
                    cm_dataA_conj(dr, di, Fr[nt2], Fi[nt2], nFi[nt2], cr, ci);   // rows f_b, cols n_a
                    t3r[nt][nt2] = to_h4(cr);
                    t3i[nt][nt2] = to_h4(ci);
                    cmul4(t3r[nt][nt2], t3i[nt][nt2], s_tw3[(nt * 2 + nt2) * 64 + lane]);
                }
            }
            // S1': const A conj F[nt3] (M = n_b, K = f_b), data B = T3 (K = f_b, N = n_a);
            // conj outer twiddle; into R2 at [kslot(f_c)][n_ab]
#pragma unroll
            for (int nt2 = 0; nt2 < 2; ++nt2) {
                const h8 br = cat8(t3r[0][nt2], t3r[1][nt2]), bi = cat8(t3i[0][nt2], t3i[1][nt2]);
#pragma unroll
                for (int nt3 = 0; nt3 < 2; ++nt3) {
                    f4 cr, ci;
                    cm_constA_conj(Fr[nt3], Fi[nt3], nFi[nt3], br, bi, cr, ci);   // rows n_b, cols n_a
                    h4 qr = to_h4(cr), qi = to_h4(ci);
                    cmul4(qr, qi, two[nt3][nt2]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {   // r2(kslot(f_c), 16 nt2 + c + 32 (16 nt3 + 4 g + i))
                        const int o = 16384 * (r & 1) + 4 * (r >> 1) + 128 * nt2 + 4096 * nt3 + 256 * i;
                        w2r[o] = qr[i];
                        w2i[o] = qi[i];
                    }
                }
            }
        }
        __syncthreads();

        // ---- phase 3: outer inverse over f_c (outputs n_c < 16 only) and output scale for all
        // of this wave's tiles, staged as fp32 in its own R2 bytes once every tile is read,
        // then gated and stored as contiguous 16-byte rows
        f4 ya[kTilesPerWave], yb[kTilesPerWave];
#pragma unroll
        for (int tt = 0; tt < kTilesPerWave; ++tt) {
            // r2(8 g, 16 T + c)
            const h8 dr = *reinterpret_cast<const h8 *>(r3r + 128 * tt);
            const h8 di = *reinterpret_cast<const h8 *>(r3i + 128 * tt);
            cm_dataA_conj(dr, di, Fr[0], Fi[0], nFi[0], ya[tt], yb[tt]);   // rows n_ab = 16T + 4g + i, col n_c = c
            ya[tt] *= ks;
            yb[tt] *= ks;
            __builtin_amdgcn_sched_barrier(0);   // (bounds the live R2 operands)
        }
        {
            char *const s8 = reinterpret_cast<char *>(smem);
            // (re-derived here so that the eight swizzled addresses are not held across pairs)
            uint32_t stw = st_w, cq = 64 * (c & 3);
            asm volatile("" : "+v"(stw), "+v"(cq));
#pragma unroll
            for (int tt = 0; tt < kTilesPerWave; ++tt) {
                const uint32_t o = stw + ((64 * tt) ^ cq);
                stu(s8, o, ya[tt]);                                     // row n_c = c of sequence a
                stu(s8 + 2 * kR1Plane, o, yb[tt]);                      // plane 1: sequence b
            }
            uint4 vq2[8];
            if (DUAL) {   // (issued before the next input batch: vmcnt waits are in order)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    vq2[k] = ldu_nt<uint4>(v2 + (k < 4 ? oa : ob) + 4096 * (k & 3), 2 * m4);
            }
            __builtin_amdgcn_sched_barrier(0);
            // the second input batch of the next pair is fetched while the outputs are stored
            load_batch(oa_nx, ob_nx, 1, x1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                // without a second row (ob == oa) its stores repeat the first row's values
                const int kk = (k >= 4 && !has_b) ? k - 4 : k;
                const char *src = s8 + 2 * ((kk >> 2) * kR1Plane + (kk & 3) * 8192);
                const f4 y0 = ldu<f4>(src, st_r0), y1 = ldu<f4>(src, st_r1);
                float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
                if (DUAL) {
                    float ga[4], gb[4], y2[8];
                    st<T>::unpack4(make_uint2(vq2[k].x, vq2[k].y), ga);
                    st<T>::unpack4(make_uint2(vq2[k].z, vq2[k].w), gb);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        y2[i] = yv[i] * ga[i];
                        y2[4 + i] = yv[4 + i] * gb[i];
                    }
                    const uint2 lo2 = st<T>::pack4(y2), hi2 = st<T>::pack4(y2 + 4);
                    stu_nt(out2 + (k < 4 ? oa : ob) + 4096 * (k & 3), 2 * m4, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
                }
                if (HAS_V) {
                    float ga[4], gb[4];
                    st<T>::unpack4(make_uint2(vq[k].x, vq[k].y), ga);
                    st<T>::unpack4(make_uint2(vq[k].z, vq[k].w), gb);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        yv[i] *= ga[i];
                        yv[4 + i] *= gb[i];
                    }
                }
                const uint2 lo = st<T>::pack4(yv), hi = st<T>::pack4(yv + 4);
                stu_nt(out + (k < 4 ? oa : ob) + 4096 * (k & 3), 2 * m4, make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
        __syncthreads();
        oa = oa_nx;
        ob = ob_nx;
        has_b = hb_nx;
    }
}

hipError_t launch_pair16k_conv(int st_, const void *u, const void *w, const void *v, void *out,
                               const void *kbins, const float *kscale, const uint8_t *mask,
                               int64_t B, int64_t H, hipStream_t stream, const void *v2, void *out2) {
    if (out2 != nullptr && (v == nullptr || v2 == nullptr)) return hipErrorInvalidValue;
    Pair3Tables tb{};
    hipError_t e = get_pair3_tables(&tb);
    if (e != hipSuccess) return e;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
    }
    const int64_t pairs = H * ((B + 1) / 2);
    if (pairs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;   // pair indices are 32-bit
    int64_t blocks = cus;
    if (blocks > pairs) blocks = pairs < 8 ? 8 : pairs;
    const size_t lds = (size_t)2 * kR1Plane * sizeof(_Float16) + 2 * 256 * 16 + kMaskBlocks;
    auto go = [&](auto kern, auto *tp) -> hipError_t {
        using TT = std::remove_pointer_t<decltype(tp)>;
        hipError_t err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kWaves), lds, stream, (const TT *)u,
                           (const TT *)w, (const TT *)v, (TT *)out, (const uint4 *)kbins, kscale, mask, tb,
                           B, H, (const TT *)v2, (TT *)out2);
        return hipGetLastError();
    };
    // one instantiation per (storage type, mask, gates) so that no gate test sits in the loops
    auto pick = [&](auto *tp) -> hipError_t {
        using TT = std::remove_pointer_t<decltype(tp)>;
        if (out2 != nullptr) {   // two outputs: both output gates present
            switch ((mask ? 2 : 0) | (w ? 1 : 0)) {
            case 0: return go(pair16k_kernel<TT, false, false, true, true>, tp);
            case 1: return go(pair16k_kernel<TT, false, true, true, true>, tp);
            case 2: return go(pair16k_kernel<TT, true, false, true, true>, tp);
            default: return go(pair16k_kernel<TT, true, true, true, true>, tp);
            }
        }
        const int sel = (mask ? 4 : 0) | (w ? 2 : 0) | (v ? 1 : 0);
        switch (sel) {
        case 0: return go(pair16k_kernel<TT, false, false, false>, tp);
        case 1: return go(pair16k_kernel<TT, false, false, true>, tp);
        case 2: return go(pair16k_kernel<TT, false, true, false>, tp);
        case 3: return go(pair16k_kernel<TT, false, true, true>, tp);
        case 4: return go(pair16k_kernel<TT, true, false, false>, tp);
        case 5: return go(pair16k_kernel<TT, true, false, true>, tp);
        case 6: return go(pair16k_kernel<TT, true, true, false>, tp);
        default: return go(pair16k_kernel<TT, true, true, true>, tp);
        }
    };
    if (st_ == ST_F16) return pick((__half *)nullptr);
    return pick((__hip_bfloat16 *)nullptr);
}

}  // namespace fftconv
