// fftconv_internal.hpp -- declarations shared by the HIP kernel sources and
// the host-side C ABI (api.cpp).  Not installed; the public interface is
// include/fftconv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fftconv {

// Largest sequence length evaluated by the single fused kernel (the whole
// N-point complex transform of one sequence lives in LDS).
constexpr int kFusedMaxLog = 14;
constexpr int kMinLog = 10;
constexpr int kMaxLog = 22;
constexpr int kMaskBlocks = 128;

enum StorageType : int { ST_F32 = 0, ST_F16 = 1, ST_BF16 = 2 };
enum KfLayout : int { KF_NATURAL = 0, KF_ROWS = 1, KF_PAIR = 2, KF_PAIR3 = 3 };

// Prepared-filter buffer: header at offset 0, per-channel fp32 scales at
// scale_off, bins at bins_off.  Bin element: float2 (fp32 storage) or
// __half2 (fp16 / bf16 storage).  Channel h's bins start at
// bins_off + h * N * sizeof(bin).  Bin slot 0 holds (K[0], K[N]) (both real
// for a real filter); slot f in [1, N) holds K[f] in natural order
// (KF_NATURAL) or in the multi-pass row order (KF_ROWS).  The stored bins are
// K * s_h with s_h a power of two; scale[h] = 1 / (s_h * 4 N) folds the
// normalisation of the half-length real transform pair.
struct KfHeader {
    uint32_t magic;
    uint32_t version;
    int64_t N;
    int64_t H;
    int64_t L;
    int32_t dtype;
    int32_t layout;
    int64_t scale_off;
    int64_t bins_off;
    int64_t n1;   // multi-pass outer size (0 for the fused layout)
    int64_t n2;   // multi-pass inner size
};
constexpr uint32_t kKfMagic = 0x4b544646u;  // "FFTK"
constexpr uint32_t kKfVersion = 4;
constexpr size_t kKfHeaderBytes = 256;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The matrix-core pair kernel handles N = 1024 in fp16/bf16 storage.  Its
// filter layout holds the full 2N-bin spectrum in the order its lanes read
// it: 16-byte chunk q = (mt2 * 4 + nt) * 64 + lane, lane = 16 g + c, holds
// re[0..3] then im[0..3] (fp16) of bins f = 16 nt + c + 64 (16 mt2 + 4 g + i).
inline bool use_pair_kernel(int logn, int st) { return logn == 10 && st != ST_F32; }
// The three-stage matrix-core kernel handles N = 2048 .. 16384 in fp16/bf16
// storage: the 2N-point transform is M = 1024 R points with R = 2N / 1024 =
// 2^logr (logr = logn - 9 = 2 .. 5) outer rows of 1024.  Its filter layout
// (KF_PAIR3) stores the rows f_c = f mod R in [0, R/2] of the 2N-bin spectrum;
// chunk ((f_c * 2 + mt2) * 2 + nt) * 64 + lane holds re[0..3], im[0..3] of bins
// f = f_c + R (16 nt + c) + 32 R (16 mt2 + 4 g + i).
inline bool use_pair3_kernel(int logn, int st) { return logn >= 11 && logn <= 14 && st != ST_F32; }
inline int64_t kf_slots(int logn, int st) {
    if (use_pair_kernel(logn, st)) return int64_t(2) << logn;
    if (use_pair3_kernel(logn, st)) return ((int64_t(1) << (logn - 10)) + 1) * 1024;
    return int64_t(1) << logn;
}
// log2 of the normalisation folded into scale[h]: 4N for the half-length
// real transform (fused, multi-pass), 2N for the pair kernels.
inline int kf_norm_log2(int logn, int st) {
    return (use_pair_kernel(logn, st) || use_pair3_kernel(logn, st)) ? logn + 1 : logn + 2;
}
// Bound on the stored bins |K| * s_h: 2^14 for the layouts the VALU kernels
// rescale in fp32, 1 for the pair layouts whose product is taken in fp16.
inline int kf_target_log2(int logn, int st) {
    return (use_pair_kernel(logn, st) || use_pair3_kernel(logn, st)) ? 0 : 14;
}
// fp16 element offset of the real part of bin f in the KF_PAIR3 layout with
// R = 2^logr outer rows, or -1 when the bin's row is not stored (f mod R > R/2:
// read the mirror 2N - f).
__host__ __device__ inline int64_t pair3_kf_index(int64_t f, int logr = 5) {
    const int64_t R = int64_t(1) << logr;
    const int64_t fc = f & (R - 1), fb = (f >> logr) & 31, fa = f >> (logr + 5);
    if (fc > R / 2) return -1;
    const int64_t mt2 = fa >> 4, g = (fa & 15) >> 2, i = fa & 3, nt = fb >> 4, c = fb & 15;
    return ((((fc * 2 + mt2) * 2 + nt) * 64 + g * 16 + c) * 8) + i;
}
// fp16 element offset of the real part of bin f in the pair layout (imag at +4)
__host__ __device__ inline int64_t pair_kf_index(int64_t f) {
    const int64_t fs = f % 64, ff = f / 64;
    const int64_t mt2 = ff / 16, g = (ff % 16) / 4, i = ff % 4, nt = fs / 16, c = fs % 16;
    return (((mt2 * 4 + nt) * 64 + g * 16 + c) * 8) + i;
}
// Power-of-two factors 2^-k folded into the fp16 DFT operand tables of the
// matrix-core kernels.  With them each fp16 stage result stays within a small
// factor of its input's magnitude (unnormalised stages would grow the
// zero-frequency bin of a sequence with mean m to N * m, past the fp16 range
// for m above a few units); every kernel multiplies its fp32 output scale by
// 2^k for each stage it ran.
constexpr int kPairS1Log2 = 3;   // DFT-64 blocks (S1, S1') of the N = 1024 kernel
constexpr int kPairS2Log2 = 2;   // DFT-32 blocks (S2, S2') of the N = 1024 kernel
constexpr int kDft32Log2 = 2;    // DFT-32 tiles of the N = 16384 kernel and of the multi-pass row pass
// The multi-pass row pass multiplies stored filter bins (|K s_h| <= 2^14 for
// that layout) by 2^-kRowKLog2 in its product, so |product| <= |spectrum|; the
// rest of the channel scale is applied by the last pass in fp32.
constexpr int kRowKLog2 = 14;
// Column-pass factor of the half-precision three-pass path: 2^-p1 with
// p1 = floor((log2 N1 - 1) / 2) + 1 (about 1/sqrt of the N1/2 summed terms)
inline __host__ __device__ constexpr int mp_p1_log2(int log1) { return (log1 - 1) / 2 + 1; }
inline size_t bin_bytes(int st) { return st == ST_F32 ? 8 : 4; }
inline size_t kf_scale_off() { return kKfHeaderBytes; }
inline size_t kf_bins_off(int64_t H) { return kKfHeaderBytes + align_up((size_t)H * 4, 256); }

// Multi-pass split N = n1 * n2 (n2 on chip).
struct MpSplit {
    int log1, log2;
};
MpSplit mp_split(int logn);
// Bytes per workspace point (one complex value in the storage type) and
// sequences processed per multi-pass chunk (bounds the workspace).
int64_t mp_ws_bytes(int st);
// fp32 area per sequence for the two self-paired rows of the row pass
constexpr size_t kMpSelfBytes = 2 * 8192 * 8;
int64_t mp_chunk(int logn, int st);
// The row pass of the half-precision multi-pass path computes the last forward
// stage (over n_a, producing the most significant digit f_a of the in-row bin)
// as two 16-row matrix tiles; tile m2, row r (r < 16) holds
//   f_a = row_fa(m2, r):  m2 = 0: 0..7 and 24..31,   m2 = 1: 8..23,
// so that the middle frequencies of a row (which a low-pass frequency mask
// drops for both bins of every bin pair) fill one whole tile.  The partner of
// f_a, 31 - f_a, is row 15 - r of the same tile.
__host__ __device__ inline int row_fa(int m2, int r) { return m2 ? 8 + r : (r < 8 ? r : 16 + r); }
__host__ __device__ inline int row_tile_of(int fa) { return (fa >= 8 && fa < 24) ? 1 : 0; }
__host__ __device__ inline int row_r_of(int fa) { return fa < 8 ? fa : (fa < 24 ? fa - 8 : fa - 16); }
// Position of in-row bin f2 (row length 8192) in a multi-pass spectrum stored
// in half precision.  Such spectra are kept in the order the matrix-core row
// pass produces them: f2 = f_c + 8 f_b + 256 f_a with f_b = 16 nt + c and
// f_a = row_fa(mt2, 4 g + i) sits at f_c * 1024 + (2 mt2 + nt) * 256 +
// (16 g + c) * 4 + i, so that lane 16 g + c of the wave that owns chain f_c
// reads the four bins i of tile (mt2, nt) as one 16-byte word.  Bin 0 stays at
// position 0.  fp32 spectra keep the natural order.
__host__ __device__ inline uint32_t mp_chain_pos(uint32_t f2) {
    const uint32_t fc = f2 & 7u, fb = (f2 >> 3) & 31u, fa = f2 >> 8;
    const uint32_t mt2 = (uint32_t)row_tile_of((int)fa), r = (uint32_t)row_r_of((int)fa);
    return fc * 1024u + (mt2 * 2u + (fb >> 4)) * 256u + (16u * (r >> 2) + (fb & 15u)) * 4u + (r & 3u);
}

// Per-device, per-size tables (allocated once, read only afterwards).
struct Tables {
    const float2 *tw;    // exp(-2 pi i j / N), j < N
    const float2 *tw2;   // exp(-pi i j / N),   j < N   (= omega_{2N}^j)
};
hipError_t get_tables(int logn, Tables *out);

// Multi-pass extras for N = 2^logn: omega_{2N}^j (j < N1), and the two
// factors of the two-level lookup omega_N^a = hi[a >> 11] * lo[a & 2047].
struct MpTables {
    const float2 *w2row;   // exp(-pi i j / N),          j < N1
    const float2 *big_lo;  // exp(-2 pi i j / N),        j < 2048
    const float2 *big_hi;  // exp(-2 pi i 2048 j / N),   j < N / 2048
    const void *col;       // matrix-core column-pass operand tiles (N1 >= 2^kMpColMinLog1), else null
};
// The column transforms of the three-pass path split N1 = 2^log1 = RA * RB with
// RB = 2^mp_col_rb_log2(log1) (the first stage of the forward column DFT, over the
// coarse input digit) and RA = N1 / RB.
inline __host__ __device__ constexpr int mp_col_rb_log2(int log1) { return (log1 + 1) / 2; }
// Half-precision storage with N1 >= 2^kMpColMinLog1 runs both column passes on the
// matrix cores; the first stage of the inverse column pass (RA points) has its
// table scaled by 2^-mp_c3_log2 (undone with the output scale).
constexpr int kMpColMinLog1 = 8;
inline __host__ __device__ constexpr int mp_c3_log2(int log1) {
    return (log1 - mp_col_rb_log2(log1) + 1) / 2;
}
hipError_t get_mp_tables(int logn, MpTables *out);
// Builds every table of the current device once (hipMalloc and synchronous
// copies); later calls return at once.  device_tables_ready: already built.
hipError_t init_device_tables();
bool device_tables_ready();

// ---- launchers (return the launch status) --------------------------------
hipError_t launch_fused_conv(int logn, int st, const void *u,
                             const void *w, const void *v, void *out, const void *kbins,
                             const float *kscale, const uint8_t *mask, const Tables &tb,
                             int64_t B, int64_t H, hipStream_t stream);
// ysgn = -1 stores the conjugated spectrum (used by the backward pass)
hipError_t launch_fused_prepare(int logn, int st, const void *k, int64_t L, void *kbins,
                                const float *kscale, const Tables &tb, int64_t H,
                                float ysgn, hipStream_t stream);
// backward-pass helpers (bwd.hip); kind: 0 PAIR chunks, 1 fp16 slots, 2 fp32 slots
hipError_t launch_conj_bins(const void *src, void *dst, int64_t H, int64_t bytes_per_channel, int kind,
                            hipStream_t stream);
hipError_t launch_gate_product(int st, const void *u, const void *w, void *x, int64_t n, hipStream_t stream);
hipError_t launch_mask_repeat(const uint8_t *mask, uint8_t *dst, int64_t H, int64_t C, hipStream_t stream);
hipError_t launch_dk_reduce(int st, const void *part, void *dk, int64_t B, int64_t H, int64_t N, int64_t L,
                            hipStream_t stream);
hipError_t launch_filter_scale(int st, const void *k, int64_t H, int64_t L, int norm_log2,
                               int target_log2, float *kscale, hipStream_t stream);

// Lane-order constant tables of the pair kernel (see pair_mfma.hip).
struct PairTables {
    const void *f1r, *f1i;   // S1 DFT-64 blocks, [4][64 lanes][8] fp16
    const void *f2r, *f2i;   // S2 DFT-32 blocks, [2][64][8] fp16
    const void *f3r, *f3i;   // S1' conj DFT-64 blocks, [2 ks * 2 nt][64][8] fp16
    const void *tw1;         // forward twiddles, [2 mt][4 nt][64 lanes]: cos[4], sin[4] fp16
    const void *tw3;         // inverse twiddles, [4 nt][2 nt2][64]: cos[4], sin[4] fp16
};
hipError_t get_pair_tables(PairTables *out);

// Lane-order constant tables of the three-stage kernel (see pair16k.hip).
struct Pair3Tables {
    const void *fr, *fi;     // DFT-32 operand tiles, [2][64 lanes][8] fp16
    const void *tw1;         // inner twiddles w1024^{n_a f_b}, [mt][nt][lane]: cos[4], sin[4]
    const void *tw3;         // inner conj twiddles, [nt][nt2][lane]
    const void *two1;        // outer twiddles wM^{f_c n_ab}, [64 T][2 nt][lane], n_ab = 16(T & ~1) + 2c + (T & 1)
    const void *two2;        // outer conj twiddles, [32 f_c][2 nt3][2 nt2][lane]
    // the multi-pass row pass's last forward stage and first inverse stage, with
    // f_a in the tile order row_fa: A operand [m2][64 lanes][8] (row f_a = row_fa(m2, c),
    // K slot 8g + j <-> n_a = rho(8g + j)) and B operand [n2][64][8] (column
    // n_a = 16 n2 + c, K slot 8g + j <-> f_a = row_fa(j / 4, 4g + j % 4))
    const void *far_, *fai_, *fbr_, *fbi_;
    // the row pass's outer twiddle omega_8192^{f_c n_ab}, n_ab = n_a + 32 (4 q + k):
    // [f_c 8][q 8][n_a 32] x (cos[k], sin[k]) fp16, k < 4
    const void *rtw;
    // outer stages of the three-stage kernel for R = 2^(2 + i) < 32 (i < 3), see
    // P16Outer; for R = 32 the DFT-32 tiles fr, fi and two1, two2 above serve
    const void *o1r[3], *o1i[3], *o3r[3], *o3i[3], *ot1[3], *ot2[3];
};
// Outer-stage tables of the three-stage kernel for one R: the phase-1 DFT (A
// operand, two row tiles: row rho = 16 nt + c is (sub-pair rho / R, f_c = rho mod R),
// K slot 8 g + j (j < 4) is (sub-pair k / (R/2), n_c = k mod (R/2)) with k = 4 g + j;
// zero across sub-pairs), the phase-3 inverse DFT (B operand, one tile: column
// c = (sub-pair, n_c), K slot 8 g + j = row rho(8 g + j)), and the outer twiddles
// omega_M^{f_c n_ab} in the layouts of two1, two2 (row rho standing for f_c = rho mod R).
struct P16Outer {
    const void *o1r, *o1i, *o3r, *o3i, *two1, *two2;
};
// power-of-two factor 2^-p16_outer_log2(logr) folded into each outer-stage table
inline __host__ __device__ constexpr int p16_outer_log2(int logr) { return logr >= 4 ? 2 : 1; }
hipError_t get_pair3_tables(Pair3Tables *out);
// with out2: the adjoint with two outputs, out = v * corr(u w, k) and out2 = v2 * corr(u w, k)
// from the same transforms (v and v2 non-null; kbins is the spectrum of k, conjugated as read)
hipError_t launch_pair16k_conv(int logn, int st, const void *u, const void *w, const void *v, void *out,
                               const void *kbins, const float *kscale, const uint8_t *mask,
                               int64_t B, int64_t H, hipStream_t stream, const void *v2 = nullptr,
                               void *out2 = nullptr);
// the backward pass's filter-gradient partials at N = 2^logn = 2048 .. 16384 (two launches of
// the same kernel): part (ceil(B/2) H, N) rows bp H + h; spec holds kP16SpecBytes per
// workgroup group (ceil(H / P) ceil(B/2) groups, P = 2^(14 - logn) channels) and pscale
// P floats per group (one per pair of batch rows and channel)
constexpr size_t kP16SpecBytes = (size_t)32 * 2 * 2 * 64 * 16;
// With dv (N = 16384 only; kbins, kscale: the prepared filter's bins and scales): the first
// launch also forms dv = dy * conv(u w, k), masked like the forward call, from the same
// transforms.
hipError_t launch_pair16k_dk(int logn, int st, const void *dy, const void *u, const void *w, const void *v,
                             void *part, void *spec, float *pscale, const uint8_t *mask, int64_t B,
                             int64_t H, hipStream_t stream, void *dv = nullptr, const void *kbins = nullptr,
                             const float *kscale = nullptr);
// The filter prepare of the N = 2048 .. 16384 half-precision layout (KF_PAIR3) on the
// matrix cores: the bins of H channels from taps k[H][L], with kscale[h] already written
// by the scale kernel (read here).
hipError_t launch_pair16k_prepare(int logn, int st, const void *k, int64_t L, void *kbins, const float *kscale,
                                  int64_t H, hipStream_t stream);
// with out2: the adjoint with two outputs, out = v * corr(u w, k) and out2 = v2 * corr(u w, k)
// from the same transforms (v and v2 non-null; kbins is the spectrum of k, conjugated as read)
hipError_t launch_pair_conv(int logn, int st, const void *u, const void *w, const void *v,
                            void *out, const void *kbins, const float *kscale, const uint8_t *mask,
                            int64_t B, int64_t H, hipStream_t stream, const void *v2 = nullptr,
                            void *out2 = nullptr);
// dk of the backward pass at N = 1024 (fp16 / bf16): dk (H, L) <- sum over b of
// corr(v dy, u w), the spectrum product masked like K when mask is given (w, v, mask
// may be null).  NS > 0: the same over (B, H, NS) sequences of the short-filter path
// (L <= 1024, NS a multiple of 1024, no mask).
hipError_t launch_pair_dk(int st, const void *dy, const void *u, const void *w, const void *v, void *dk,
                          const uint8_t *mask, int64_t B, int64_t H, int64_t L, hipStream_t stream,
                          int64_t NS = 0);
// Chunked short-filter path: (B, H, NS) sequences, NS a multiple of 1024, as
// half-overlapping windows of 2048 samples, each a 2048-point circular convolution on
// the N = 1024 matrix-core kernel (filters of at most 1024 taps).  corr: the adjoint,
// out = v * corr(u w, k) with corr(x, k)[t] = sum_s k[s] x[t + s], and with out2 != null
// a second output out2 = v2 * corr(u w, k) (v and v2 then both non-null).
hipError_t launch_pair_conv_win(int st, const void *u, const void *w, const void *v, void *out,
                                const void *kbins, const float *kscale, int64_t B, int64_t H, int64_t NS,
                                hipStream_t stream, bool corr = false, const void *v2 = nullptr,
                                void *out2 = nullptr);
// Group-axis circular convolution composed with a channel map (eqlinear.hip).
int eqlinear_span(int T);   // output channels per workgroup (C_out must be a multiple of span / 4)
hipError_t launch_eqlinear_prepare(int st, int T, const void *W, void *Wf, int64_t Cout, int64_t Cin,
                                   hipStream_t stream);
hipError_t launch_eqlinear(int st, int T, const void *x, const void *Wf, void *y, int64_t Ntok, int64_t Cin,
                           int64_t Cout, hipStream_t stream);
hipError_t launch_write_header(const KfHeader &hdr, void *K_f, hipStream_t stream);

hipError_t launch_multipass_conv(int logn, int st, const void *u, const void *w, const void *v,
                                 void *out, const void *kbins, const float *kscale,
                                 const uint8_t *mask, void *work, int64_t H, int64_t seq0,
                                 int64_t nseq, hipStream_t stream);
hipError_t launch_multipass_prepare(int logn, int st, const void *k, int64_t L, void *kbins,
                                    const float *kscale, void *work, int64_t H, int64_t h0,
                                    int64_t nseq, float ysgn, hipStream_t stream);

}  // namespace fftconv
