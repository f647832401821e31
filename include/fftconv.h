/*
 * fftconv.h -- C ABI of the MI355X (gfx950) exact long causal FFT convolution.
 *
 * The operation (FlashFFTConv summary page, "Summary": a fused kernel that
 * computes *exact* FFT convolutions for long sequences, with partial and
 * frequency-sparse variants; "Problem": filters as long as the sequence;
 * "Measured effects", row on fusing gating into the convolution: the gated
 * form) is, for every batch row b and channel h,
 *
 *     out[b,h,t] = v[b,h,t] * sum_{s=0}^{min(t, L-1)} k[h,s] * u[b,h,t-s] * w[b,h,t-s]
 *                = v * irfft( rfft(pad(u*w, 2N)) * rfft(pad(k, 2N)) )[:N]      (t < N)
 *
 * computed through the convolution theorem with an FFT of size 2N.  With a
 * frequency mask ("Approach": sparsity realised by skipping blocks of the
 * matmuls; "Key results": 79 % of frequency-domain filter entries zeroed) the
 * filter spectrum's bins in zeroed blocks are treated as zero:
 *
 *     out = v * irfft( rfft(pad(u*w, 2N)) * (mask o rfft(pad(k, 2N))) )[:N]
 *
 * Mask blocks: the N+1 rfft bins f in [0, N] form 128 blocks of N/128 bins
 * (block = min(f / (N/128), 127), so the Nyquist bin N joins block 127); the
 * Hermitian mirror 2N-f of each bin follows it.
 *
 * Conventions for every function below:
 *  - Tensors are DEVICE pointers owned by the caller, dense and row-major:
 *      u, w, v, out : (B, H, N)  storage dtype
 *      k            : (H, L)     storage dtype
 *      mask         : (H, fftconv_mask_blocks(N)) uint8, 1 = keep, 0 = zero
 *    Every tensor pointer must be 16-byte aligned.  `out` must not overlap
 *    any input.
 *  - K_f (the prepared filter) is a caller-allocated device buffer of
 *    fftconv_filter_bytes() bytes.  Its contents are library-defined and
 *    opaque: a header (magic, version, N, H, L, dtype), one fp32 scale per
 *    channel, then the filter spectrum in the order the forward kernels read
 *    it (fp32 bins for FFTCONV_F32, scaled fp16 bins for FFTCONV_F16 and
 *    FFTCONV_BF16).  It depends on N and dtype, not on B.
 *  - Workspace: sequences longer than the largest on-chip size stream through
 *    HBM in several passes and need fftconv_workspace_bytes() bytes of device
 *    scratch, owned by the caller; 0 bytes (and a NULL pointer) suffice
 *    otherwise.
 *  - Supported sizes: N a power of two in [1024, 4194304]; 1 <= L <= N;
 *    B, H >= 0 (B*H == 0 enqueues nothing and returns FFTCONV_OK).
 *  - Every call is asynchronous on `stream` (a HIP stream, NULL = the default
 *    stream) unless stated otherwise, and returns a status; arguments are
 *    validated before anything is enqueued, so on any error status nothing
 *    was launched.  fftconv_last_error() gives the detail of the calling
 *    thread's last non-OK status.  Calls on different streams may run
 *    concurrently; the library's only shared state is a per-device cache of
 *    constant tables (twiddles, DFT operand tiles) guarded by a mutex.
 *  - Range (fp16 and bf16 storage).  Every size runs on the matrix-core
 *    kernels (N = 1024; N = 2048 .. 16384; the row pass of N > 16384, and its
 *    column passes for N >= 2^21), which round every transform stage to fp16
 *    (fp32 accumulation); power-of-two factors folded into their DFT tables
 *    keep the stage results within a small factor of the input (about
 *    rms(u*w) for a zero-mean input).  Overflow needs |u*w| near the fp16
 *    maximum 65504 (bf16 magnitudes beyond it are not representable on these
 *    paths), or a mean m of u*w whose zero-frequency bin passes it: 32 m at
 *    N = 1024, 64 m to 256 m at N = 2048 .. 16384, at most 4096 m for
 *    N > 16384 (|m| < 15 is safe at every N).  Nothing is clamped: an
 *    overflow gives inf / NaN.  fp32 storage has fp32 range.
 *  - The constant tables of a device are built once, by fftconv_init() or by
 *    the first fftconv_prepare_filter / fftconv_prepare_short_filter on that
 *    device: that one call allocates device memory and copies synchronously.
 *    After it, no call of this library allocates device memory or waits for
 *    the GPU (apart from the functions marked SYNCHRONOUS), so the forward
 *    and backward calls may be captured into a HIP graph.  A forward or
 *    backward call on a device where neither ran builds the tables itself,
 *    allocating and blocking like fftconv_init.
 */
#ifndef FFTCONV_H
#define FFTCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same opaque type as HIP's hipStream_t. */
typedef struct ihipStream_t *hipStream_t;

typedef enum {
    FFTCONV_F32 = 0,  /* fp32 storage, fp32 arithmetic                          */
    FFTCONV_F16 = 1,  /* fp16 storage, fp32 accumulation                        */
    FFTCONV_BF16 = 2  /* bf16 storage, fp32 accumulation                        */
} fftconv_dtype_t;

typedef enum {
    FFTCONV_OK = 0,
    FFTCONV_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, overlap  */
    FFTCONV_ERR_UNSUPPORTED = 2,      /* N not a supported power of two, bad dtype   */
    FFTCONV_ERR_WORKSPACE = 3,        /* workspace smaller than required             */
    FFTCONV_ERR_FILTER_MISMATCH = 4,  /* K_f prepared for another N, H, L or dtype   */
    FFTCONV_ERR_HIP = 5               /* a HIP runtime call or kernel launch failed  */
} fftconv_status_t;

/* Bytes of the prepared-filter buffer K_f for H channels at sequence length N.
 * Returns 0 for unsupported N, dtype or H < 1. */
size_t fftconv_filter_bytes(int64_t H, int64_t N, fftconv_dtype_t dtype);

/* Bytes of device scratch fftconv_fwd needs for B*H sequences of length N
 * (fftconv_prepare_filter needs the value for B = 1).  0 when the whole
 * sequence fits on chip.  Returns 0 for unsupported arguments. */
size_t fftconv_workspace_bytes(int64_t B, int64_t H, int64_t N, fftconv_dtype_t dtype);

/* Number of frequency blocks per channel the mask addresses (128 for every
 * supported N; 0 for unsupported N). */
int64_t fftconv_mask_blocks(int64_t N);

/* Transform the time-domain filter k (H, L_filter) into K_f for sequences of
 * length N: K_f holds rfft(pad(k, 2N)) ("Approach": the filter spectrum the
 * convolution multiplies by; partial convolution = L_filter < N, where only
 * the L_filter taps are read and the padding is implicit).  fp16 / bf16 at
 * N = 2048 .. 16384 transform on the matrix cores with fp16 stages (about
 * 1e-3 relative error of the stored spectrum, like the forward call's own
 * stages); other sizes and fp32 in fp32.  Needs workspace of
 * fftconv_workspace_bytes(1, H, N, dtype) bytes for N beyond the on-chip
 * size.  K_f_bytes must be >= fftconv_filter_bytes(H, N, dtype). */
fftconv_status_t fftconv_prepare_filter(const void *k, int64_t H, int64_t L_filter, int64_t N,
                                        fftconv_dtype_t dtype, void *K_f, size_t K_f_bytes,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* Gated causal FFT convolution (formula in the file header).
 *   u        input (B, H, N), required
 *   K_f      filter prepared by fftconv_prepare_filter for the same H, L_filter,
 *            N and dtype (checked against its header only when the
 *            environment variable FFTCONV_CHECK=1 is set, since that check
 *            synchronises)
 *   w, v     input and output gates (B, H, N); NULL = no gate
 *   out      output (B, H, N)
 *   sparsity_mask  (H, fftconv_mask_blocks(N)) uint8 device array, or NULL
 *            for a dense filter spectrum
 *   workspace / workspace_bytes  device scratch, see fftconv_workspace_bytes */
fftconv_status_t fftconv_fwd(const void *u, const void *K_f, const void *w, const void *v,
                             void *out, int64_t B, int64_t H, int64_t N, int64_t L_filter,
                             const uint8_t *sparsity_mask, fftconv_dtype_t dtype,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): fftconv_fwd
 * with the same arguments except the workspace, which comes from a static
 * device array of the library (fftconv_fwd_noalloc_scratch_bytes() bytes,
 * one copy per device, held until the process ends).  fftconv_init() must
 * have run on the calling thread's current device (else
 * FFTCONV_ERR_INVALID_ARGUMENT); the call then allocates nothing.  Sequences
 * longer than the on-chip size run through the scratch in chunks of as many
 * sequences as it holds (every supported N fits one sequence); the results are
 * those of fftconv_fwd bit for bit.  Every call on one device shares that
 * device's scratch, which keeps the last call's contents (nothing in it needs
 * to start at zero): calls that may overlap in time on one device (other
 * streams, other threads) race and must be serialised by the caller. */
fftconv_status_t fftconv_fwd_noalloc(const void *u, const void *K_f, const void *w, const void *v,
                                     void *out, int64_t B, int64_t H, int64_t N, int64_t L_filter,
                                     const uint8_t *sparsity_mask, fftconv_dtype_t dtype, hipStream_t stream);

/* Bytes of the static scratch of fftconv_fwd_noalloc (72 MiB). */
size_t fftconv_fwd_noalloc_scratch_bytes(void);

/* Device scratch bytes fftconv_fwd_taps needs: the prepared spectrum of the
 * H filters (fftconv_filter_bytes, rounded up to 256 bytes) followed by the
 * larger of the prepare's and the forward call's scratch.  0 for unsupported
 * N or dtype, H < 1 or B < 0. */
size_t fftconv_fwd_taps_workspace_bytes(int64_t B, int64_t H, int64_t N, fftconv_dtype_t dtype);

/* Forward call from the time-domain filter ("Approach", FlashFFTConv summary
 * page: a partial convolution's filter has fewer taps than the sequence, and
 * only the blocks that hold taps are transformed).  Equivalent to
 * fftconv_prepare_filter(k -> a spectrum in the workspace) followed by
 * fftconv_fwd on it, both enqueued on `stream` by this one call, so the
 * caller keeps no prepared filter; the results equal that pair of calls bit
 * for bit.
 *   k         (H, L_filter) device array of taps, same dtype as u, read only
 *   u, w, v, out, sparsity_mask  as in fftconv_fwd; w, v may be NULL
 *   workspace device scratch of fftconv_fwd_taps_workspace_bytes bytes,
 *             16-byte aligned, overlapping no argument; it holds the spectrum
 *             until the forward kernels have read it, so it must not be reused
 *             by another stream before this call's work completes
 * Errors as fftconv_prepare_filter and fftconv_fwd, plus
 * FFTCONV_ERR_WORKSPACE for a short workspace.  B = 0 or H = 0: nothing is
 * enqueued. */
fftconv_status_t fftconv_fwd_taps(const void *u, const void *k, const void *w, const void *v,
                                  void *out, int64_t B, int64_t H, int64_t N, int64_t L_filter,
                                  const uint8_t *sparsity_mask, fftconv_dtype_t dtype,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Device scratch bytes fftconv_bwd needs for this shape (0 for unsupported
 * N or dtype).  It holds room for a conjugated spectrum, u*w, the spectra of the
 * B*H sequences u*w, their correlations with v*dy, and the forward
 * workspace; at N = 1024 with fp16 or bf16 storage only the conjugated
 * spectrum (dk is accumulated on chip there); at N = 2048 .. 16384 with fp16
 * or bf16 storage the conjugated spectrum, the spectra of the batch-row pairs
 * of u*w with their scales, and one correlation row per pair and channel. */
size_t fftconv_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, fftconv_dtype_t dtype);

/* Backward pass of fftconv_fwd: the gradients of sum(dy * out) (the
 * convolutions are trained, FlashFFTConv summary page, "Key results"), with
 * x = u*w and g = v*dy:
 *   dv = dy * conv(x, k)                       (needs v; NULL = skip)
 *   du = w * corr(g, k),  dw = u * corr(g, k)  (dw needs w; NULL = skip)
 *   dk[h, s] = sum_b sum_t g[b,h,t] x[b,h,t-s], s < L_filter  (NULL = skip)
 * where corr(g, k)[t] = sum_s k[s] g[t+s] is the adjoint of the causal
 * convolution: the forward kernels run on the conjugated spectrum of K_f
 * (at N = 1024 .. 16384 in fp16 / bf16 with both du and dw asked for, one
 * kernel forms both and conjugates the bins as it reads K_f; otherwise a
 * conjugated copy is made in the workspace).  At N = 16384 in fp16 / bf16
 * with dv and dk asked for, dv comes from the same pass over u, w as the
 * spectra dk needs.  With a sparsity mask the gradients are those of the
 * masked forward pass.
 *   dy, u, w, v  (B, H, N) device arrays as in fftconv_fwd (w, v may be NULL)
 *   K_f          the spectrum fftconv_fwd used (same H, L_filter, N, dtype)
 *   du, dw, dv   (B, H, N) outputs; dk (H, L_filter) output, all in dtype
 *   workspace    at least fftconv_bwd_workspace_bytes(B, H, N, dtype) bytes
 * Asynchronous on stream; outputs must not overlap inputs. */
fftconv_status_t fftconv_bwd(const void *dy, const void *u, const void *K_f, const void *w, const void *v,
                             void *du, void *dk, void *dw, void *dv, int64_t B, int64_t H, int64_t N,
                             int64_t L_filter, const uint8_t *sparsity_mask, fftconv_dtype_t dtype,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Chunked short-filter path (overlap-save) --------------------------
 * For a filter of at most 1024 taps (the FlashFFTConv summary page, table of
 * measured effects: filters shortened to 2K keep model quality) the
 * convolution needs no transform of the whole sequence.  The sequence is
 * covered by windows of 2048 samples overlapping by half (zeros before the
 * sequence start); each window's 2048-point circular convolution with the
 * filter runs on the matrix cores and keeps the second half of its outputs,
 * which no filter tap wraps around to.  The result is the same causal
 * convolution as fftconv_fwd with this filter.  fp16 and bf16 storage only;
 * no frequency mask (the spectrum is the 2048-point one of the filter).  Its
 * backward pass is fftconv_bwd_short. */

/* Bytes of a short-filter spectrum for H channels (0 for fp32 or H < 1). */
size_t fftconv_short_filter_bytes(int64_t H, fftconv_dtype_t dtype);

/* k (H, L_filter) device array, 1 <= L_filter <= 1024, fp16 or bf16 ->
 * K_s, K_s_bytes >= fftconv_short_filter_bytes(H, dtype).  Asynchronous. */
fftconv_status_t fftconv_prepare_short_filter(const void *k, int64_t H, int64_t L_filter,
                                              fftconv_dtype_t dtype, void *K_s, size_t K_s_bytes,
                                              hipStream_t stream);

/* out = v * causal_conv(u * w, k) with the prepared short filter K_s.
 *   u, w, v, out  (B, H, N) device arrays, N a positive multiple of 1024
 *                 (not necessarily a power of two); w, v may be NULL
 *   L_filter      the filter length K_s was prepared with (<= 1024)
 * Asynchronous on stream; no workspace; out must not overlap the inputs. */
fftconv_status_t fftconv_fwd_short(const void *u, const void *K_s, const void *w, const void *v,
                                   void *out, int64_t B, int64_t H, int64_t N, int64_t L_filter,
                                   fftconv_dtype_t dtype, hipStream_t stream);

/* Backward pass of fftconv_fwd_short (the convolutions are trained,
 * FlashFFTConv summary page, "Key results"): the gradients of sum(dy * out)
 * with x = u*w and g = v*dy,
 *   dv = dy * conv(x, k)                       (needs v; NULL = skip)
 *   du = w * corr(g, k),  dw = u * corr(g, k)  (dw needs w; NULL = skip)
 *   dk[h, s] = sum_b sum_t g[b,h,t+s] x[b,h,t], s < L_filter  (NULL = skip)
 * with corr(g, k)[t] = sum_s k[s] g[t+s] (zero past the sequence end), the
 * same quantities as fftconv_bwd.  dv runs the windowed forward kernel with
 * dy as the output gate; corr takes, for the outputs of block j, the window
 * of blocks j and j+1 and its 2048-point circular correlation with the
 * filter (the conjugated spectrum, first half of the outputs: no
 * wrap-around); dk accumulates, per channel on chip, the spectrum products
 * of those windows of g with the zero-padded blocks of x.
 *   dy, u, w, v   (B, H, N) device arrays, N a positive multiple of 1024;
 *                 w, v may be NULL (absent gates, as in the forward call)
 *   K_s           the short-filter spectrum of the forward call
 *   du, dw, dv    (B, H, N) outputs, dk (H, L_filter) output, all in dtype;
 *                 each may be NULL; none may overlap an input
 * No workspace.  B = 0: dk is set to zero, nothing else is written.
 * Asynchronous on stream. */
fftconv_status_t fftconv_bwd_short(const void *dy, const void *u, const void *K_s, const void *w,
                                   const void *v, void *du, void *dk, void *dw, void *dv, int64_t B,
                                   int64_t H, int64_t N, int64_t L_filter, fftconv_dtype_t dtype,
                                   hipStream_t stream);

/* ---- Group-axis circular convolution (Flash EQ-Linear) ------------------
 * The Flash EQ-Linear abstract page: an equivariant linear layer is a
 * circular convolution along the group dimension composed with a linear map
 * along the channels, computed through the Fourier convolution theorem along
 * the group axis with the real DFT's conjugate symmetry, in FP32 and in FP16
 * precision.  Here, for a cyclic group of order T:
 *   y[n, t, d] = sum_{s < T} sum_{c < C_in} W[s, d, c] x[n, (t - s) mod T, c]
 * x (N, T, C_in), W (T, C_out, C_in), y (N, T, C_out), contiguous, fp32, fp16
 * or bf16 storage; T in {4, 8, 16}; C_in and C_out positive multiples of 32.
 * The per-frequency channel products run on the matrix cores: fp32 operands
 * for fp32 storage, fp16 operands for fp16 and bf16 storage, fp32
 * accumulation throughout. */

/* Bytes of the transformed weights (T/2 + 1 complex matrices, fp32 for fp32
 * storage and fp16 otherwise); 0 when unsupported. */
size_t fftconv_eqlinear_weight_bytes(int64_t T, int64_t C_out, int64_t C_in, fftconv_dtype_t dtype);

/* W (T, C_out, C_in) device array -> W_f (W_f_bytes >= fftconv_eqlinear_weight_bytes).
 * Asynchronous on stream. */
fftconv_status_t fftconv_eqlinear_prepare(const void *W, int64_t T, int64_t C_out, int64_t C_in,
                                          fftconv_dtype_t dtype, void *W_f, size_t W_f_bytes,
                                          hipStream_t stream);

/* y = the group convolution of x with the prepared weights W_f (prepared for the
 * same dtype).  Asynchronous on stream; y must not overlap x or W_f. */
fftconv_status_t fftconv_eqlinear_fwd(const void *x, const void *W_f, void *y, int64_t N, int64_t T,
                                      int64_t C_in, int64_t C_out, fftconv_dtype_t dtype, hipStream_t stream);

/* Static text for a status code. */
const char *fftconv_status_string(fftconv_status_t status);

/* Detail of the calling thread's last non-OK status ("" if none). */
const char *fftconv_last_error(void);

/* Test helper, SYNCHRONOUS: decode K_f into natural-order rfft bins
 * K[h, f] = rfft(pad(k[h], 2N))[f], f in [0, N], as float64 (re, im) pairs in
 * host memory host_out[(H, N+1, 2)]. */
fftconv_status_t fftconv_export_filter_rfft(const void *K_f, int64_t H, int64_t N,
                                            fftconv_dtype_t dtype, double *host_out,
                                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FFTCONV_H */
