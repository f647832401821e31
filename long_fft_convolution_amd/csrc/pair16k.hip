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

// Kernel modes.  kConv: the convolution.  kSpec: the forward transform of the pair only;
// the spectrum is stored conjugated and scaled, as a complex "filter" of all 32 rows f_c,
// in the order in which the product step reads it.  kCorr: the convolution with such a
// per-pair spectrum in place of K_f, keeping only the real part of the result (the
// backward pass's filter gradient: with z_x = x_a + i x_b and z_g = g_a + i g_b,
// Re IDFT(conj(Z_x) Z_g) = corr(g_a, x_a) + corr(g_b, x_b)).  kPrep: the filter prepare,
// the forward transform of each channel's zero-padded taps k (one sequence per sub-pair,
// no second row) stored as the prepared spectrum K s_h of that channel (rows f_c <= R/2
// of the KF_PAIR3 layout), with s_h = 2^e from the channel scale already written.
// kConvSpec: the convolution of kConv that also stores the pair's spectrum as kSpec does
// (the backward pass takes dv and the spectra of u w from one pass over u, w).
constexpr int kConv = 0, kSpec = 1, kCorr = 2, kPrep = 3, kConvSpec = 4;
// kPrep: the taps enter the transform scaled by s_h 2^kPrepInLog2, so that sum |k s_h| <= 1
// becomes sum |x| <= 2^14: every stage result stays below 2^14 (a DFT output is at most the
// sum of its inputs' magnitudes, and the table factors only shrink it) while the taps of a
// long filter stay in fp16's normal range (about 2^14 / L each)
constexpr int kPrepInLog2 = 14;
constexpr int kSpecRows = 32 * 2 * 2 * 64;   // uint4 per pair spectrum (all rows f_c)

// filter chunk of row fc (of R = 2^LOGR) for (mt2, nt): rows f_c <= R/2 as stored, the
// others from the mirror row R - f_c (lane 63 - l, tiles flipped, elements reversed,
// conjugated); FULL: a per-pair spectrum with every row stored
template <bool FULL = false, int LOGR = 5>
__device__ __forceinline__ uint4 k_load(const uint4 *kch, int fc, int mt2, int nt, uint32_t lane) {
    if constexpr (FULL) return ldu<uint4>(kch + ((fc * 2 + mt2) * 2 + nt) * 64, 16u * lane);
    constexpr int R = 1 << LOGR;
    const bool mir = fc > R / 2;
    const uint32_t row = mir ? R - fc : fc, a = mir ? 1 - mt2 : mt2, b = mir ? 1 - nt : nt;
    return ldu<uint4>(kch + ((row * 2 + a) * 2 + b) * 64, 16u * (mir ? 63 - lane : lane));
}
// (CONJ: the conjugate of that chunk, for the adjoint)
template <bool CONJ = false>
__device__ __forceinline__ h8 k_fix(const uint4 &q, bool mir) {
    constexpr uint32_t sm = CONJ ? 0x80008000u : 0u, sn = CONJ ? 0u : 0x80008000u;
    uint4 t;
    if (!mir) {
        t = q;
        t.z ^= sm;
        t.w ^= sm;
        return *reinterpret_cast<const h8 *>(&t);
    }
    // (e0..e3 | e4..e7) -> (e3, e2, e1, e0 | -e7, -e6, -e5, -e4)
    t.x = __builtin_amdgcn_alignbit(q.y, q.y, 16);
    t.y = __builtin_amdgcn_alignbit(q.x, q.x, 16);
    t.z = __builtin_amdgcn_alignbit(q.w, q.w, 16) ^ sn;
    t.w = __builtin_amdgcn_alignbit(q.z, q.z, 16) ^ sn;
    return *reinterpret_cast<const h8 *>(&t);
}

}  // namespace p16

using namespace p16;

// grid: persistent, one workgroup (kWaves waves) per CU; each workgroup walks an
// XCD-local range of pairs p = h * ceil(B/2) + bp.  An odd B pairs its last row
// with zeros: the second row's loads then re-read the first row (always in
// bounds) and are discarded, so no load sits under a branch.
// DUAL: the adjoint with two outputs, out = v corr(u w, k) and out2 = v2 corr(u w, k),
// from the same transforms: the product takes conj K, the stored bins conjugated as they
// are read (the backward pass forms du and dw in one call); the second gate's rows are
// loaded once the staged outputs have freed their registers.
// MODE (kConv, kSpec, kCorr, kPrep) above.  kSpec writes spec_out[p] (all 32 rows of the
// workgroup) for group p and scale_out[p P + sp] for its sub-pair sp; kCorr reads them
// through kbins and kscale and writes the rows bp H + h (h: the group's channels) of out.
// kPrep (B = 1): u is the taps k[H][Lk], kscale the channel scales, and spec_out the bins
// of the prepared filter (channel h at h (R/2 + 1) 256 uint4).
// LOGR < 5 (N = 512 R = 2048, 4096, 8192): the 2N-point transform is R = 2^LOGR outer
// rows of 1024; P = 32 / R pairs of P consecutive channels (the same batch rows) share a
// workgroup's 32 rows (sub-pair p = row / R, f_c = row mod R), so phase 2 is unchanged.
// The P channels' rows are adjacent in memory (channel h + p at p N), so every input and
// output offset of the N = 16384 layout (1024 * slot + column) addresses sub-pair p's
// values; past the last channel the loads re-read sub-pair 0 and the stores are skipped.
template <typename T, bool MASKED, bool HAS_W, bool HAS_V, bool DUAL = false, int MODE = kConv, int LOGR = 5>
__global__ void __launch_bounds__(64 * kWaves, 1)
pair16k_kernel(const T *__restrict__ u, const T *__restrict__ w, const T *__restrict__ v,
               T *__restrict__ out, const uint4 *__restrict__ kbins, const float *__restrict__ kscale,
               const uint8_t *__restrict__ mask, Pair3Tables tb, int64_t B, int64_t H,
               const T *__restrict__ v2, T *__restrict__ out2, uint4 *__restrict__ spec_out,
               float *__restrict__ scale_out, P16Outer ot, int64_t Lk) {
    static_assert(!DUAL || HAS_V, "a second output has an output gate of its own");
    static_assert(MODE == kConv || MODE == kConvSpec || (!DUAL && !HAS_V),
                  "the spectrum and correlation modes have no output gate");
    static_assert(MODE != kConvSpec || !DUAL, "one output with the spectrum");
    static_assert(MODE != kSpec || !MASKED, "the spectrum mode stores every bin");
    static_assert(MODE != kPrep || (!MASKED && !HAS_W), "the prepare mode transforms the taps alone");
    static_assert(LOGR >= 2 && LOGR <= 5, "R = 4 .. 32");
    constexpr bool SPEC = MODE == kSpec, CORR = MODE == kCorr, PREP = MODE == kPrep;
    constexpr bool CONV = MODE == kConv || MODE == kConvSpec, FWD = SPEC || PREP;   // FWD: forward transform only
    constexpr bool SPST = SPEC || MODE == kConvSpec;   // stores the pair's spectrum
    constexpr int R = 1 << LOGR, P = 32 / R, NCH = R / 2;   // outer rows, sub-pairs, non-zero n_c
    constexpr int N = 512 * R;
    constexpr int M2 = 2 * N;
    constexpr int kKRows = (R / 2 + 1) * 256;                  // uint4 per channel of K_f
    extern __shared__ __align__(16) _Float16 smem[];
    _Float16 *P0 = smem;                    // plane 0 (re) of R1 / R2
    _Float16 *P1 = smem + kR1Plane;         // plane 1 (im)
    h8 *s_tw1 = reinterpret_cast<h8 *>(smem + 2 * kR1Plane);   // [mt][nt][lane]
    h8 *s_tw3 = s_tw1 + 4 * 64;                                 // [nt][nt2][lane]
    uint8_t *s_mask = reinterpret_cast<uint8_t *>(s_tw3 + 4 * 64);   // mask rows of the P channels
    // R < 32: the outer DFT tiles, [phase-1 re t0, t1, im t0, t1, phase-3 re, im][lane]
    h8 *s_out = reinterpret_cast<h8 *>(s_mask + 8 * kMaskBlocks);
    // kSpec / kCorr: per wave and slot n_c of phase 1, the sum of |input| [wave][32]
    float *const s_part = reinterpret_cast<float *>(s_out + 6 * 64);
    // kConv: bit 8 row + sp set when a wave saw a non-zero input of that row (a, b) of
    // sub-pair sp, ORed over the waves
    uint32_t *const s_zf = reinterpret_cast<uint32_t *>(s_part + kWaves * 32);

    const int tid = threadIdx.x;
    if (tid == 0) *s_zf = 0u;
    for (int i = tid; i < 256; i += 64 * kWaves) {
        s_tw1[i] = reinterpret_cast<const h8 *>(tb.tw1)[i];
        s_tw3[i] = reinterpret_cast<const h8 *>(tb.tw3)[i];
    }
    if constexpr (R < 32) {
        // phase 1 contracts only the slots n_c < R/2 of each sub-pair, half of the tile's K
        // slots (8 g + j, j < 4), so its data operand carries both planes in one h8,
        // (x_a j = 0..3 | x_b j = 0..3), and one product per plane does:
        // Re = [Re O | -Im O] . x, Im = [Im O | Re O] . x  (O: the block-diagonal DFT-R tile)
        if (tid < 128) {
            const h8 o_r = reinterpret_cast<const h8 *>(ot.o1r)[tid], o_i = reinterpret_cast<const h8 *>(ot.o1i)[tid];
            s_out[tid] = cat8(lo4(o_r), lo4(neg8(o_i)));
            s_out[128 + tid] = cat8(lo4(o_i), lo4(o_r));
        } else if (tid < 192) {
            s_out[256 + tid - 128] = reinterpret_cast<const h8 *>(ot.o3r)[tid - 128];
            s_out[320 + tid - 128] = reinterpret_cast<const h8 *>(ot.o3i)[tid - 128];
        }
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
    const h8 *twO1 = reinterpret_cast<const h8 *>(ot.two1) + wave * (kTilesPerWave * 2 * 64);
    const h8 *twO2 = reinterpret_cast<const h8 *>(ot.two2) + wave * (4 * 64);
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

    // groups q = hg PB + bp: channels hg P .. hg P + P - 1, batch rows 2 bp, 2 bp + 1
    const int64_t PB = (B + 1) / 2, HG = (H + P - 1) / P, NQ = HG * PB;
    const uint32_t nwg = gridDim.x, xcd = blockIdx.x % 8, wg_local = blockIdx.x / 8;
    const uint32_t wg_on_xcd = nwg / 8 + (xcd < nwg % 8 ? 1u : 0u);
    const int64_t p_begin = NQ * xcd / 8, p_end = NQ * (xcd + 1) / 8;

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
        // groups < 2^31; the quotient is made wave-uniform so that all pair addresses are scalar
        const int64_t hh = __builtin_amdgcn_readfirstlane((uint32_t)pp / (uint32_t)PB), bpp = pp - hh * PB;
        hb_ = 2 * bpp + 1 < B;
        oa_ = (2 * bpp * H + hh * P) * N;
        ob_ = hb_ ? oa_ + H * N : oa_;
    };
    // channels of group pp (P, or fewer in the last channel group)
    auto group_nv = [&](int64_t pp) -> int {
        if constexpr (P == 1) return 1;
        const int64_t hh = __builtin_amdgcn_readfirstlane((uint32_t)pp / (uint32_t)PB);
        const int64_t r = H - hh * P;
        return (int)(r < P ? r : P);
    };
    // kSpec / kCorr: sum of |x| over the pair's transformed values (this lane's share, per
    // slot n_c = 4 g + j)
    float l1j[4] = {0.f, 0.f, 0.f, 0.f};
    // kConv: the fp16 bits of this lane's inputs ORed (the sign bits are cleared when they
    // are tested), per row and (R = 4, where the two slot halves j < 2, j >= 2 belong to two
    // sub-pairs) slot half
    uint32_t nz[2][2] = {{0u, 0u}, {0u, 0u}};
    // kPrep: the input factor s_h 2^kPrepInLog2 of the channel of slot 4 g + j
    float pin[4] = {0.f, 0.f, 0.f, 0.f};
    auto load_batch = [&](int64_t oa_, int64_t ob_, int half, Batch &x, int nv_) {
        if constexpr (PREP) {
            // slot 4 g + j: sub-pair sp (channel ch0 + sp), n_c; element n_ab + 1024 n_c of
            // the taps row, zero at n >= Lk and past the group's channels
            const int64_t ch0 = oa_ >> (9 + LOGR);   // (B = 1: oa_ = first channel * N)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sp = P > 1 ? (4 * g + j) / NCH : 0, nc = P > 1 ? (4 * g + j) % NCH : 4 * g + j;
                const bool okc = sp < nv_;
                const uint16_t *row = reinterpret_cast<const uint16_t *>(u + (ch0 + (okc ? sp : 0)) * Lk);
#pragma unroll
                for (int qq = 0; qq < 2; ++qq) {
                    const int64_t n = 16 * kTilesPerWave * wave + 32 * (2 * half + qq) + 2 * c + 1024 * nc;
                    const uint32_t lo = okc && n < Lk ? (uint32_t)row[n] : 0u;
                    const uint32_t hi = okc && n + 1 < Lk ? (uint32_t)row[n + 1] : 0u;
                    x.xa[qq][j] = lo | (hi << 16);
                    x.xb[qq][j] = 0u;
                }
            }
            return;
        }
        const uint32_t *pua = reinterpret_cast<const uint32_t *>(u + oa_);
        const uint32_t *pub = reinterpret_cast<const uint32_t *>(u + ob_);
        const uint32_t *pwa = reinterpret_cast<const uint32_t *>(w + oa_);
        const uint32_t *pwb = reinterpret_cast<const uint32_t *>(w + ob_);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // element m1 + 1024 j is slot 4 g + j of sub-pair (4 g + j) / NCH (channel offset
            // included); past the group's channels, sub-pair 0.  P > 1 takes the j term into
            // the lane offset, so that the correction applies to the whole offset.
            uint32_t lo = 2 * m1;
            int mj = 1024 * j;
            if constexpr (P > 1) {
                const int sp = (4 * g + j) / NCH;
                lo = 2u * (uint32_t)(m1 + 1024 * j - (sp >= nv_ ? sp * N : 0));
                mj = 0;
            }
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int m = (32 * (2 * half + qq) + mj) / 2;   // in dwords
                x.xa[qq][j] = ldu<uint32_t>(pua + m, lo);
                x.xb[qq][j] = ldu<uint32_t>(pub + m, lo);
                if (HAS_W) {
                    x.ga[qq][j] = ldu<uint32_t>(pwa + m, lo);
                    x.gb[qq][j] = ldu<uint32_t>(pwb + m, lo);
                }
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
                    if (PREP) xa *= pin[j];
                    br[j] = (_Float16)xa;
                    bi[j] = hb_ ? (_Float16)xb : (_Float16)0.f;
                    br[4 + j] = (_Float16)0.f;
                    bi[4 + j] = (_Float16)0.f;
                    if (SPST || CORR) l1j[j] += fabsf((float)br[j]) + fabsf((float)bi[j]);
                }
                if (CONV) {
                    const uint4 qa = *reinterpret_cast<const uint4 *>(&br), qb = *reinterpret_cast<const uint4 *>(&bi);
                    if constexpr (NCH >= 4) {
                        nz[0][0] |= qa.x | qa.y;
                        nz[1][0] |= qb.x | qb.y;
                    } else {
                        nz[0][0] |= qa.x;
                        nz[0][1] |= qa.y;
                        nz[1][0] |= qb.x;
                        nz[1][1] |= qb.y;
                    }
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f4 ar, ai;
                    if constexpr (R == 32) {
                        cm_constA(Fr[nt], Fi[nt], nFi[nt], br, bi, ar, ai);   // rows f_c = 16nt + 4g + i, cols n_ab
                    } else {   // block-diagonal DFT-R tile (rows: sub-pair, f_c), read at use
                        const h8 bx = cat8(lo4(br), lo4(bi));
                        const f4 z = {0.f, 0.f, 0.f, 0.f};
                        ar = mfma(s_out[nt * 64 + lane], bx, z);
                        ai = mfma(s_out[128 + nt * 64 + lane], bx, z);
                    }
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
    int nv = group_nv(p);
    Batch x0, x1;
    load_batch(oa, ob, 0, x0, nv);
    load_batch(oa, ob, 1, x1, nv);
    // channel of sub-pair sp of the current group (past the last channel: the group's first)
    auto chan = [&](int64_t hg, int sp) -> int64_t { return hg * P + (sp < nv ? sp : 0); };
    // P > 1: element offset correction of an access of sub-pair sp (sub-pair 0 past the last
    // channel); rows gamma = (sp, n_c) of the outputs are 1024 gamma apart
    auto past = [&](int gamma) -> bool { return P > 1 && (gamma / NCH) >= nv; };
    // 16 output-gate values of rows gamma = 4 kq + (lane >> 4) of the row at element row_:
    // P > 1 moves the row term into the lane offset, corrected past the last channel
    auto gate_ld = [&](const T *gp, int64_t row_, int kq) -> uint4 {
        if constexpr (P == 1) return ldu_nt<uint4>(gp + row_ + 4096 * kq, 2 * m4);
        const int gm = 4 * kq + (lane >> 4);
        return ldu_nt<uint4>(gp + row_, 2u * (uint32_t)(4096 * kq + m4 - (past(gm) ? (gm / NCH) * N : 0)));
    };

    for (; p < p_end; p += wg_on_xcd) {
        const int64_t h = __builtin_amdgcn_readfirstlane((uint32_t)p / (uint32_t)PB);   // channel group
        // (the six stages' table factors are undone with the channel scale; kCorr: the pair's)
        const float ks = CONV ? __builtin_ldexpf(kscale[h], 6 * kDft32Log2) : 1.f;
        if constexpr (PREP) {   // s_h = 1 / (kscale 2N), times 2^kPrepInLog2
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sp = P > 1 ? (4 * g + j) / NCH : 0;
                pin[j] = __builtin_ldexpf(1.f / kscale[h * P + (sp < nv ? sp : 0)], kPrepInLog2 - (10 + LOGR));
            }
        }
        const int64_t oo = CORR ? ((p - h * PB) * H + h * P) * N : 0;   // kCorr output row
        int64_t p_nx = p + wg_on_xcd, oa_nx, ob_nx;
        bool hb_nx;
        pair_base(p_nx < p_end ? p_nx : p, oa_nx, ob_nx, hb_nx);
        const int nv_nx = group_nv(p_nx < p_end ? p_nx : p);

        // the mask rows are read in phase 2 only, after the barrier that ends phase 1
        if (MASKED && tid < P * kMaskBlocks / 4) {
            const int64_t mc = P == 1 ? h : chan(h, tid / (kMaskBlocks / 4));
            reinterpret_cast<uint32_t *>(s_mask)[tid] =
                reinterpret_cast<const uint32_t *>(mask + mc * kMaskBlocks)[tid % (kMaskBlocks / 4)];
        }

        // ---- phase 1: outer DFT over n_c for this wave's tiles T of n_ab, two batches
        // (loads are issued in the order they are consumed: vmcnt waits are in order)
        {
            h8 tw0[2][2][2], tw1[2][2][2];
            load_tw(0, tw0);
            load_tw(1, tw1);
            phase1_batch(x0, tw0, 0, has_b);
            phase1_batch(x1, tw1, 1, has_b);
        }
        if (SPST || CORR) {   // per slot: the sum over the 16 lanes of one g, then per wave
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int o = 8; o > 0; o >>= 1) l1j[j] += __shfl_xor(l1j[j], o);
            }
            if (c == 0) *reinterpret_cast<f4 *>(s_part + 32 * wave + 4 * g) = f4{l1j[0], l1j[1], l1j[2], l1j[3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) l1j[j] = 0.f;
        }
        if (CONV) {   // this wave's non-zero rows of sub-pairs, ORed into s_zf
            uint32_t seen = 0u;   // (wave-uniform: built from the ballots)
#pragma unroll
            for (int row = 0; row < 2; ++row)
#pragma unroll
                for (int jh = 0; jh < (NCH >= 4 ? 1 : 2); ++jh) {
                    // (sign bits cleared once here: a product 0 * (-w) is -0)
                    const unsigned long long m = __builtin_amdgcn_ballot_w64((nz[row][jh] & 0x7fff7fffu) != 0u);
                    nz[row][jh] = 0u;
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {   // lanes 16 gg .. 16 gg + 15: slots 4 gg + j
                        const int sp = (4 * gg + 2 * jh) / NCH;
                        if ((m >> (16 * gg)) & 0xffffull) seen |= 1u << (8 * row + sp);
                    }
                }
            if (lane == 0 && seen != 0u) atomicOr(s_zf, seen);
        }
        __syncthreads();
        // kConv: a row of a sub-pair whose inputs are all zero has the result 0, not the
        // rounding of its partner row's values: zrow bit 8 row + sp marks it
        uint32_t zrow = 0u;
        if (CONV) {
            constexpr uint32_t kRows = ((1u << P) - 1u) * 0x101u;
            zrow = __builtin_amdgcn_readfirstlane(~*s_zf & kRows);
        }
        // kSpec / kCorr: |Z[f]| <= sum |z| bounds every bin of a sub-pair's transform, so a
        // spectrum taken after the three forward stages (table factors 2^-kF) and scaled by
        // the power of two 2^e <= 2^(kF + kSpecLog2) / sum |z| stays within |.| <= 2^kSpecLog2
        // (kSpec: the stored spectrum of x; kCorr: the spectrum of g before the product, so
        // that neither is far below fp16's normal range).  Each sub-pair (P > 1: its slots
        // n_c in [sp NCH, sp NCH + NCH)) has its own scale.  kSpec stores the filter scale of
        // that spectrum, 1 / (2^(e - kF) 2N), per sub-pair; kCorr undoes its 2^e in the output
        constexpr int kF = R == 32 ? 3 * kDft32Log2 : 2 * kDft32Log2 + p16_outer_log2(LOGR);
        constexpr int kSpecLog2 = 6;
        // lane l < 16 sums slot l over the waves, then over its sub-pair's NCH slots; every
        // lane then holds the exponent of the sub-pair of slot l (16 slots: n_c < NCH for
        // each of the P sub-pairs)
        int e_l = 0;
        if (SPST || CORR) {
            float t = 0.f;
            if (lane < 16) {
#pragma unroll
                for (int w8 = 0; w8 < kWaves; ++w8) t += s_part[32 * w8 + lane];
            }
#pragma unroll
            for (int o = 1; o < NCH; o <<= 1) t += __shfl_xor(t, o);
            if (t > 0.f && isfinite(t)) {
                e_l = (int)floorf(log2f(__builtin_ldexpf(1.f, kF + kSpecLog2) / t));
                e_l = e_l < -60 ? -60 : (e_l > 60 ? 60 : e_l);
            }
        }
        auto sp_exp = [&](int sp) -> int {
            if constexpr (R == 32) return __builtin_amdgcn_readfirstlane(e_l);
            return __shfl(e_l, sp * NCH);
        };
        float sc[kRowsPerWave];   // per phase-2 row rho = wave + 8 r: its sub-pair's 2^e
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) sc[r] = 1.f;
        if (SPST || CORR) {
#pragma unroll
            for (int r = 0; r < kRowsPerWave; ++r)
                sc[r] = __builtin_ldexpf(1.f, sp_exp(R == 32 ? 0 : (wave + kWaves * r) >> LOGR));
        }
        if (SPST) {
            const int e_mine = sp_exp(lane < P ? lane : 0);   // (all lanes: a shuffle)
            if (tid < P) scale_out[p * P + tid] = __builtin_ldexpf(1.f, kF - e_mine - (10 + LOGR));
        }

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
        // filter rows: row rho = wave + 8 r is f_c = rho mod R of sub-pair rho / R
        // (kCorr: the group's own spectrum, every row rho stored)
        auto kchan = [&](int rho) -> const uint4 * {
            if constexpr (CORR) return kbins + p * (int64_t)kSpecRows;
            if constexpr (R == 32) return kbins + h * (int64_t)kKRows;
            return kbins + chan(h, rho >> LOGR) * (int64_t)kKRows;
        };
        // f_c of row rho (rho < 32)
        auto rowfc = [&](int rho) -> int { return R == 32 ? rho : (rho & (R - 1)); };
        // the filter row read for row rho (kCorr: rho itself)
        auto krow = [&](int rho) -> int { return CORR ? rho : rowfc(rho); };
        uint4 kq[2][2];
        if (!FWD) {
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    kq[mt2][nt] = k_load<CORR, LOGR>(kchan(wave), krow(wave), mt2, nt, ul);
        }
        __syncthreads();
        if (tid == 0) *s_zf = 0u;   // (every thread has read it; the next pair ORs into it)

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
            h8 kk[2][2], two[2][2];
            if (!FWD) {
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) kk[mt2][nt] = k_fix<DUAL>(kq[mt2][nt], !CORR && rowfc(fc) > R / 2);
                if (r + 1 < kRowsPerWave) {
#pragma unroll
                    for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
                            kq[mt2][nt] = k_load<CORR, LOGR>(kchan(fc + kWaves), krow(fc + kWaves), mt2, nt, lx);
                }
#pragma unroll
                for (int nt3 = 0; nt3 < 2; ++nt3)
#pragma unroll
                    for (int nt2 = 0; nt2 < 2; ++nt2)
                        two[nt3][nt2] = ldu<h8>(twO2 + ((kWaves * r * 2 + nt3) * 2 + nt2) * 64, 16u * lx);
            }
            if (r == kRowsPerWave - 1) {   // output gate of this pair, first batch of the next
                if (HAS_V) {
#pragma unroll
                    for (int tt = 0; tt < kTilesPerWave; ++tt) {
                        vq[tt] = gate_ld(v, tt < 4 ? oa : ob, tt & 3);
                    }
                }
                // pinned order: the gate is consumed first, and vmcnt waits are in order
                __builtin_amdgcn_sched_barrier(0);
                load_batch(oa_nx, ob_nx, 0, x0, nv_nx);
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
                    if (PREP) {   // K s_h: rows f_c <= R/2 of the channel's KF_PAIR3 bins
                        constexpr int kFwd = R == 32 ? 3 * kDft32Log2 : 2 * kDft32Log2 + p16_outer_log2(LOGR);
                        constexpr float kOut = kFwd >= kPrepInLog2 ? (float)(1u << (kFwd - kPrepInLog2))
                                                                   : 1.f / (float)(1u << (kPrepInLog2 - kFwd));
                        const int spr = fc >> LOGR;
                        if (rowfc(fc) <= R / 2 && spr < nv) {
                            const h8 q = cat8(to_h4(cr * kOut), to_h4(ci * kOut));
                            stu(spec_out + chan(h, spr) * (int64_t)kKRows + ((rowfc(fc) * 2 + mt2) * 2 + nt) * 64,
                                16u * lx, q);
                        }
                        continue;
                    }
                    if (SPST) {   // conj(Z) 2^e in the order the product step reads it
                        const h8 q = cat8(to_h4(cr * sc[r]), to_h4(ci * -sc[r]));
                        stu(spec_out + p * (int64_t)kSpecRows + ((fc * 2 + mt2) * 2 + nt) * 64, 16u * lx, q);
                        if (SPEC) continue;
                    }
                    if (CORR) {   // the spectrum of g scaled by its sub-pair's 2^e
                        cr *= sc[r];
                        ci *= sc[r];
                    }
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
                            const int f = rowfc(fc) + R * (16 * nt + lc) + 32 * R * (16 * mt2 + 4 * lg + i);
                            const int fr_ = f <= N ? f : M2 - f;
                            int blk = fr_ / (N / kMaskBlocks);
                            blk = blk > kMaskBlocks - 1 ? kMaskBlocks - 1 : blk;
                            if (R < 32) blk += (fc >> LOGR) * kMaskBlocks;
                            if (!s_mask[blk]) kf[i] = kf[4 + i] = (_Float16)0.f;
                        }
                    }
                    cmul4(yr[mt2][nt], yi[mt2][nt], kf);
                }
            }
            if (FWD) continue;
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
        if (FWD) {   // no inverse: the next pair's second input batch, then the next pair
            load_batch(oa_nx, ob_nx, 1, x1, nv_nx);
            __syncthreads();
            oa = oa_nx;
            ob = ob_nx;
            has_b = hb_nx;
            nv = nv_nx;
            continue;
        }
        __syncthreads();

        // ---- phase 3: outer inverse over f_c (outputs n_c < 16 only) and output scale for all
        // of this wave's tiles, staged as fp32 in its own R2 bytes once every tile is read,
        // then gated and stored as contiguous 16-byte rows
        f4 ya[kTilesPerWave], yb[kTilesPerWave];
        // R < 32: the block-diagonal inverse DFT-R tile, and column c = (sub-pair, n_c)
        // takes its channel's scale
        float ksl = ks;
        constexpr int kBack = R == 32 ? 6 * kDft32Log2 : 4 * kDft32Log2 + 2 * p16_outer_log2(LOGR);
        if constexpr (CORR) {   // column c: sub-pair c / NCH, its stored scale and its 2^-e
            const int spc = R == 32 ? 0 : c / NCH;
            ksl = __builtin_ldexpf(kscale[p * P + spc], kBack - sp_exp(spc));
        } else if constexpr (R < 32) {
            ksl = __builtin_ldexpf(kscale[chan(h, c / NCH)], kBack);
        }
        // (an all-zero row of column c's sub-pair: the output scale 0)
        const int spz = R == 32 ? 0 : c / NCH;
        const float ksla = (zrow >> spz) & 1u ? 0.f : ksl, kslb = (zrow >> (8 + spz)) & 1u ? 0.f : ksl;
#pragma unroll
        for (int tt = 0; tt < kTilesPerWave; ++tt) {
            // r2(8 g, 16 T + c)
            const h8 dr = *reinterpret_cast<const h8 *>(r3r + 128 * tt);
            const h8 di = *reinterpret_cast<const h8 *>(r3i + 128 * tt);
            if constexpr (R == 32) {
                cm_dataA_conj(dr, di, Fr[0], Fi[0], nFi[0], ya[tt], yb[tt]);   // rows n_ab = 16T + 4g + i, col n_c = c
            } else {   // the block-diagonal inverse DFT-R tile, read at use
                const h8 f3r = s_out[256 + lane], f3i = s_out[320 + lane];
                cm_dataA_conj(dr, di, f3r, f3i, neg8(f3i), ya[tt], yb[tt]);
            }
            ya[tt] *= ksla;
            yb[tt] *= kslb;
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
                if (!CORR) stu(s8 + 2 * kR1Plane, o, yb[tt]);           // plane 1: sequence b (kCorr: the
                                                                        // real part only, yb is dropped)
            }
            uint4 vq2[8];
            if (DUAL) {   // (issued before the next input batch: vmcnt waits are in order)
#pragma unroll
                for (int k = 0; k < 8; ++k) vq2[k] = gate_ld(v2, k < 4 ? oa : ob, k & 3);
            }
            __builtin_amdgcn_sched_barrier(0);
            // the second input batch of the next pair is fetched while the outputs are stored
            load_batch(oa_nx, ob_nx, 1, x1, nv_nx);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (CORR && k >= 4) break;   // the real part only
                // rows of sub-pairs past the group's last channel are not stored
                const bool skip = past(4 * (k & 3) + (lane >> 4));
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
                    if (!skip)
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
                if (!skip)
                    stu_nt(out + (CORR ? oo : (k < 4 ? oa : ob)) + 4096 * (k & 3), 2 * m4,
                           make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
        __syncthreads();
        oa = oa_nx;
        ob = ob_nx;
        has_b = hb_nx;
        nv = nv_nx;
    }
}

// persistent grid: one workgroup per CU, at most one per group of pairs (and at least 8, one
// per XCD); a group is 32 / R pairs of consecutive channels
static hipError_t p16_grid(int64_t B, int64_t H, int64_t *blocks, int logr = 5) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
    }
    const int64_t P = 32 >> logr;
    const int64_t pairs = (H + P - 1) / P * ((B + 1) / 2);
    if (pairs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;   // pair indices are 32-bit
    *blocks = cus;
    if (*blocks > pairs) *blocks = pairs < 8 ? 8 : pairs;
    return hipSuccess;
}

// LDS: the two planes, the inner twiddle tables, the mask rows of up to 8 channels, the
// outer DFT tiles of R < 32 (six planes of 64 lanes x 16 bytes), the per-wave input sums of
// the spectrum and correlation modes, the non-zero lane masks of the rows
static constexpr size_t kP16Lds =
    (size_t)2 * kR1Plane * sizeof(_Float16) + 2 * 256 * 16 + 8 * kMaskBlocks + 6 * 64 * 16 + 8 * 32 * 4 + 4 * 8;
static_assert(kP16Lds <= 160 * 1024, "LDS of one workgroup");

static P16Outer p16_outer(const Pair3Tables &tb, int logr) {
    if (logr == 5) return P16Outer{tb.fr, tb.fi, tb.fr, tb.fi, tb.two1, tb.two2};
    const int i = logr - 2;
    return P16Outer{tb.o1r[i], tb.o1i[i], tb.o3r[i], tb.o3i[i], tb.ot1[i], tb.ot2[i]};
}

template <int LOGR>
static hipError_t pair16k_conv_r(int st_, const void *u, const void *w, const void *v, void *out,
                                 const void *kbins, const float *kscale, const uint8_t *mask, int64_t B,
                                 int64_t H, hipStream_t stream, const void *v2, void *out2) {
    Pair3Tables tb{};
    hipError_t e = get_pair3_tables(&tb);
    if (e != hipSuccess) return e;
    int64_t blocks = 0;
    if ((e = p16_grid(B, H, &blocks, LOGR)) != hipSuccess) return e;
    const P16Outer ot = p16_outer(tb, LOGR);
    const size_t lds = kP16Lds;
    auto go = [&](auto kern, auto *tp) -> hipError_t {
        using TT = std::remove_pointer_t<decltype(tp)>;
        hipError_t err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kWaves), lds, stream, (const TT *)u,
                           (const TT *)w, (const TT *)v, (TT *)out, (const uint4 *)kbins, kscale, mask, tb,
                           B, H, (const TT *)v2, (TT *)out2, (uint4 *)nullptr, (float *)nullptr, ot, (int64_t)0);
        return hipGetLastError();
    };
    // one instantiation per (storage type, mask, gates) so that no gate test sits in the loops
    auto pick = [&](auto *tp) -> hipError_t {
        using TT = std::remove_pointer_t<decltype(tp)>;
        if (out2 != nullptr) {   // two outputs: both output gates present
            switch ((mask ? 2 : 0) | (w ? 1 : 0)) {
            case 0: return go(pair16k_kernel<TT, false, false, true, true, kConv, LOGR>, tp);
            case 1: return go(pair16k_kernel<TT, false, true, true, true, kConv, LOGR>, tp);
            case 2: return go(pair16k_kernel<TT, true, false, true, true, kConv, LOGR>, tp);
            default: return go(pair16k_kernel<TT, true, true, true, true, kConv, LOGR>, tp);
            }
        }
        const int sel = (mask ? 4 : 0) | (w ? 2 : 0) | (v ? 1 : 0);
        switch (sel) {
        case 0: return go(pair16k_kernel<TT, false, false, false, false, kConv, LOGR>, tp);
        case 1: return go(pair16k_kernel<TT, false, false, true, false, kConv, LOGR>, tp);
        case 2: return go(pair16k_kernel<TT, false, true, false, false, kConv, LOGR>, tp);
        case 3: return go(pair16k_kernel<TT, false, true, true, false, kConv, LOGR>, tp);
        case 4: return go(pair16k_kernel<TT, true, false, false, false, kConv, LOGR>, tp);
        case 5: return go(pair16k_kernel<TT, true, false, true, false, kConv, LOGR>, tp);
        case 6: return go(pair16k_kernel<TT, true, true, false, false, kConv, LOGR>, tp);
        default: return go(pair16k_kernel<TT, true, true, true, false, kConv, LOGR>, tp);
        }
    };
    if (st_ == ST_F16) return pick((__half *)nullptr);
    return pick((__hip_bfloat16 *)nullptr);
}

hipError_t launch_pair16k_conv(int logn, int st_, const void *u, const void *w, const void *v, void *out,
                               const void *kbins, const float *kscale, const uint8_t *mask,
                               int64_t B, int64_t H, hipStream_t stream, const void *v2, void *out2) {
    if (out2 != nullptr && (v == nullptr || v2 == nullptr)) return hipErrorInvalidValue;
    switch (logn) {
    case 11: return pair16k_conv_r<2>(st_, u, w, v, out, kbins, kscale, mask, B, H, stream, v2, out2);
    case 12: return pair16k_conv_r<3>(st_, u, w, v, out, kbins, kscale, mask, B, H, stream, v2, out2);
    case 13: return pair16k_conv_r<4>(st_, u, w, v, out, kbins, kscale, mask, B, H, stream, v2, out2);
    case 14: return pair16k_conv_r<5>(st_, u, w, v, out, kbins, kscale, mask, B, H, stream, v2, out2);
    default: return hipErrorInvalidValue;
    }
}

// Filter gradient partials at N = 16384: for every pair p = h ceil(B/2) + bp of batch rows
// (2 bp, 2 bp + 1) of channel h, part[bp H + h] = corr(dy v, u w) summed over the two rows.
// With dv (N = 16384 only): the first pass also forms dv = dy * conv(u w, k) from the filter
// bins kbins, kscale (mode kConvSpec, masked like the forward call).
// spec (ceil(B/2) H * 128 KiB) and pscale (ceil(B/2) H floats) hold the pairs' conjugated
// spectra of u w between the two launches.
template <int LOGR>
static hipError_t pair16k_dk_r(int st_, const void *dy, const void *u, const void *w, const void *v, void *part,
                               void *spec, float *pscale, const uint8_t *mask, int64_t B, int64_t H,
                               hipStream_t stream, void *dv, const void *kbins, const float *kscale) {
    Pair3Tables tb{};
    hipError_t e = get_pair3_tables(&tb);
    if (e != hipSuccess) return e;
    int64_t blocks = 0;
    if ((e = p16_grid(B, H, &blocks, LOGR)) != hipSuccess) return e;
    const P16Outer ot = p16_outer(tb, LOGR);
    auto go = [&](auto kern, auto *tp, const void *in, const void *gate, void *o, const void *kb,
                  const float *ksc, const uint8_t *m) -> hipError_t {
        using TT = std::remove_pointer_t<decltype(tp)>;
        hipError_t err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)kP16Lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kWaves), kP16Lds, stream, (const TT *)in,
                           (const TT *)gate, (const TT *)nullptr, (TT *)o, (const uint4 *)kb, ksc, m, tb, B, H,
                           (const TT *)nullptr, (TT *)nullptr, (uint4 *)spec, pscale, ot, (int64_t)0);
        return hipGetLastError();
    };
    // the first pass with dv: kConvSpec, dv = dy * conv(u w, k) with dy as the output gate
    auto go_cs = [&](auto kern, auto *tp) -> hipError_t {
        using TT = std::remove_pointer_t<decltype(tp)>;
        hipError_t err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)kP16Lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kWaves), kP16Lds, stream, (const TT *)u,
                           (const TT *)w, (const TT *)dy, (TT *)dv, (const uint4 *)kbins, kscale, mask, tb, B, H,
                           (const TT *)nullptr, (TT *)nullptr, (uint4 *)spec, pscale, ot, (int64_t)0);
        return hipGetLastError();
    };
    auto pick = [&](auto *tp) -> hipError_t {
        using TT = std::remove_pointer_t<decltype(tp)>;
        hipError_t err = hipSuccess;
        if (dv != nullptr) {
            // (N = 16384 only: at R < 32 the combined variants spill 14 to 32 registers)
            if constexpr (LOGR == 5) {
                switch ((mask ? 2 : 0) | (w ? 1 : 0)) {
                case 0: err = go_cs(pair16k_kernel<TT, false, false, true, false, kConvSpec, LOGR>, tp); break;
                case 1: err = go_cs(pair16k_kernel<TT, false, true, true, false, kConvSpec, LOGR>, tp); break;
                case 2: err = go_cs(pair16k_kernel<TT, true, false, true, false, kConvSpec, LOGR>, tp); break;
                default: err = go_cs(pair16k_kernel<TT, true, true, true, false, kConvSpec, LOGR>, tp); break;
                }
            } else {
                return hipErrorInvalidValue;
            }
        } else {
            err = w ? go(pair16k_kernel<TT, false, true, false, false, kSpec, LOGR>, tp, u, w, nullptr, nullptr,
                         nullptr, nullptr)
                    : go(pair16k_kernel<TT, false, false, false, false, kSpec, LOGR>, tp, u, nullptr, nullptr,
                         nullptr, nullptr, nullptr);
        }
        if (err != hipSuccess) return err;
        switch ((mask ? 2 : 0) | (v ? 1 : 0)) {
        case 0:
            return go(pair16k_kernel<TT, false, false, false, false, kCorr, LOGR>, tp, dy, nullptr, part, spec,
                      pscale, mask);
        case 1:
            return go(pair16k_kernel<TT, false, true, false, false, kCorr, LOGR>, tp, dy, v, part, spec, pscale,
                      mask);
        case 2:
            return go(pair16k_kernel<TT, true, false, false, false, kCorr, LOGR>, tp, dy, nullptr, part, spec,
                      pscale, mask);
        default:
            return go(pair16k_kernel<TT, true, true, false, false, kCorr, LOGR>, tp, dy, v, part, spec, pscale,
                      mask);
        }
    };
    if (st_ == ST_F16) return pick((__half *)nullptr);
    return pick((__hip_bfloat16 *)nullptr);
}

hipError_t launch_pair16k_dk(int logn, int st_, const void *dy, const void *u, const void *w, const void *v,
                             void *part, void *spec, float *pscale, const uint8_t *mask, int64_t B,
                             int64_t H, hipStream_t stream, void *dv, const void *kbins, const float *kscale) {
    if (st_ == ST_F32 || (dv != nullptr && (kbins == nullptr || kscale == nullptr))) return hipErrorInvalidValue;
    switch (logn) {
    case 11: return pair16k_dk_r<2>(st_, dy, u, w, v, part, spec, pscale, mask, B, H, stream, dv, kbins, kscale);
    case 12: return pair16k_dk_r<3>(st_, dy, u, w, v, part, spec, pscale, mask, B, H, stream, dv, kbins, kscale);
    case 13: return pair16k_dk_r<4>(st_, dy, u, w, v, part, spec, pscale, mask, B, H, stream, dv, kbins, kscale);
    case 14: return pair16k_dk_r<5>(st_, dy, u, w, v, part, spec, pscale, mask, B, H, stream, dv, kbins, kscale);
    default: return hipErrorInvalidValue;
    }
}

// Filter prepare on the matrix cores (KF_PAIR3 bins of H channels from taps k[H][L]); the
// channel scales kscale[h] are read, not written (the scale kernel runs first).
template <int LOGR>
static hipError_t pair16k_prep_r(int st_, const void *k, int64_t L, void *kbins, const float *kscale, int64_t H,
                                 hipStream_t stream) {
    Pair3Tables tb{};
    hipError_t e = get_pair3_tables(&tb);
    if (e != hipSuccess) return e;
    int64_t blocks = 0;
    if ((e = p16_grid(1, H, &blocks, LOGR)) != hipSuccess) return e;
    const P16Outer ot = p16_outer(tb, LOGR);
    auto go = [&](auto kern, auto *tp) -> hipError_t {
        using TT = std::remove_pointer_t<decltype(tp)>;
        hipError_t err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)kP16Lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kWaves), kP16Lds, stream, (const TT *)k,
                           (const TT *)nullptr, (const TT *)nullptr, (TT *)nullptr, (const uint4 *)nullptr, kscale,
                           (const uint8_t *)nullptr, tb, (int64_t)1, H, (const TT *)nullptr, (TT *)nullptr,
                           (uint4 *)kbins, (float *)nullptr, ot, L);
        return hipGetLastError();
    };
    if (st_ == ST_F16) return go(pair16k_kernel<__half, false, false, false, false, kPrep, LOGR>, (__half *)nullptr);
    return go(pair16k_kernel<__hip_bfloat16, false, false, false, false, kPrep, LOGR>, (__hip_bfloat16 *)nullptr);
}

hipError_t launch_pair16k_prepare(int logn, int st_, const void *k, int64_t L, void *kbins, const float *kscale,
                                  int64_t H, hipStream_t stream) {
    if (st_ == ST_F32 || L < 1 || L > (int64_t(1) << logn)) return hipErrorInvalidValue;
    switch (logn) {
    case 11: return pair16k_prep_r<2>(st_, k, L, kbins, kscale, H, stream);
    case 12: return pair16k_prep_r<3>(st_, k, L, kbins, kscale, H, stream);
    case 13: return pair16k_prep_r<4>(st_, k, L, kbins, kscale, H, stream);
    case 14: return pair16k_prep_r<5>(st_, k, L, kbins, kscale, H, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fftconv
