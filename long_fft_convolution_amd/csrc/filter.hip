// filter.hip -- small kernels around the prepared filter K_f: the per-channel
// power-of-two scale of the stored spectrum and the header.
//
// fp16 bins hold K * s_h.  Every bin satisfies |K[f]| <= sum_t |k[t]| (triangle
// inequality on the DFT sum), so s_h = 2^floor(log2(2^T / sum|k|)) keeps every
// stored bin below 2^T, inside fp16's range, while the largest bins keep
// fp16's full 11-bit significand (T = 14 where the kernel rescales in fp32
// before the product, T = 0 where the product itself is taken in fp16).  fp32 bins use s_h = 1.  The stored scale is
// scale[h] = 1 / (s_h * norm), which also folds the normalisation of the
// transform pair (norm = 4N for the half-length real transform, 2N for the
// two-sequence complex packing of the matrix-core kernel), so the forward
// kernels multiply once.
#include "fft_device.hpp"
#include "fftconv_internal.hpp"

namespace fftconv {

// sum of |x| over the 16 / sizeof(T) values of one 16-byte word
template <typename T> __device__ __forceinline__ float sum_abs16(const uint4 &q) {
    const T *e = reinterpret_cast<const T *>(&q);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < (int)(16 / sizeof(T)); ++j) s += fabsf(io<T>::load1(e + j));
    return s;
}

constexpr int kScaleThreads = 1024;

// One workgroup per channel.  The row is read as 16-byte words from its first 16-byte
// boundary (rows of odd length start unaligned), four words in flight per thread; the
// few values before that boundary and after the last whole word are read one by one.
// The summation order is fixed, so the scale does not vary from call to call.
template <typename T>
__global__ void __launch_bounds__(kScaleThreads)
filter_scale_kernel(const T *__restrict__ k, int64_t L, int norm_log2, int target_log2, bool unit,
                    float *__restrict__ kscale) {
    __shared__ float part[kScaleThreads / 64];
    const int64_t h = blockIdx.x;
    const int tid = threadIdx.x;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    if (!unit) {
        constexpr int E = 16 / sizeof(T);
        const T *row = k + h * L;
        // rows start at multiples of sizeof(T): the head holds fewer than E values
        int64_t head = (int64_t)(((16u - (uint32_t)(reinterpret_cast<uintptr_t>(row) & 15u)) & 15u) / sizeof(T));
        if (head > L) head = L;
        const int64_t nv = (L - head) / E;
        const uint4 *vec = reinterpret_cast<const uint4 *>(row + head);
        int64_t i = tid;
        for (; i + 3 * kScaleThreads < nv; i += 4 * kScaleThreads) {
            const uint4 q0 = vec[i], q1 = vec[i + kScaleThreads], q2 = vec[i + 2 * kScaleThreads],
                        q3 = vec[i + 3 * kScaleThreads];
            s0 += sum_abs16<T>(q0);
            s1 += sum_abs16<T>(q1);
            s2 += sum_abs16<T>(q2);
            s3 += sum_abs16<T>(q3);
        }
        for (; i < nv; i += kScaleThreads) s0 += sum_abs16<T>(vec[i]);
        if (tid < head) s1 += fabsf(io<T>::load1(row + tid));
        const int64_t t1 = head + nv * E + tid;   // the tail: fewer than E values
        if (t1 < L) s2 += fabsf(io<T>::load1(row + t1));
    }
    float s = (s0 + s1) + (s2 + s3);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if ((tid & 63) == 0) part[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) {
        float tot = 0.f;
        for (int j = 0; j < kScaleThreads / 64; ++j) tot += part[j];
        int e = 0;
        if (!unit && tot > 0.f && isfinite(tot)) {
            e = (int)floorf(log2f(ldexpf(1.0f, target_log2) / tot));
            e = e < -60 ? -60 : (e > 60 ? 60 : e);
        }
        // scale[h] = 1 / (s_h * 2^norm_log2) with s_h = 2^e: a power of two, exact in fp32
        kscale[h] = ldexpf(1.0f, -e - norm_log2);
    }
}

__global__ void write_header_kernel(KfHeader hdr, KfHeader *dst) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *dst = hdr;
}

hipError_t launch_filter_scale(int st, const void *k, int64_t H, int64_t L, int norm_log2,
                               int target_log2, float *kscale, hipStream_t stream) {
    const bool unit = st == ST_F32;
    switch (st) {
    case ST_F32:
        hipLaunchKernelGGL(filter_scale_kernel<float>, dim3((unsigned)H), dim3(kScaleThreads), 0, stream,
                           (const float *)k, L, norm_log2, target_log2, unit, kscale);
        break;
    case ST_F16:
        hipLaunchKernelGGL(filter_scale_kernel<__half>, dim3((unsigned)H), dim3(kScaleThreads), 0, stream,
                           (const __half *)k, L, norm_log2, target_log2, unit, kscale);
        break;
    default:
        hipLaunchKernelGGL(filter_scale_kernel<__hip_bfloat16>, dim3((unsigned)H), dim3(kScaleThreads), 0,
                           stream, (const __hip_bfloat16 *)k, L, norm_log2, target_log2, unit, kscale);
    }
    return hipGetLastError();
}

hipError_t launch_write_header(const KfHeader &hdr, void *K_f, hipStream_t stream) {
    hipLaunchKernelGGL(write_header_kernel, dim3(1), dim3(64), 0, stream, hdr, (KfHeader *)K_f);
    return hipGetLastError();
}

}  // namespace fftconv
