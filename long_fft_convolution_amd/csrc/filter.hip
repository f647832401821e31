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

template <typename T>
__global__ void __launch_bounds__(256)
filter_scale_kernel(const T *__restrict__ k, int64_t L, int norm_log2, int target_log2, bool unit,
                    float *__restrict__ kscale) {
    __shared__ float part[256];
    const int64_t h = blockIdx.x;
    float s = 0.f;
    if (!unit) {
        const T *row = k + h * L;
        for (int64_t t = threadIdx.x; t < L; t += 256) s += fabsf(io<T>::load1(row + t));
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        int e = 0;
        const float tot = part[0];
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
        hipLaunchKernelGGL(filter_scale_kernel<float>, dim3((unsigned)H), dim3(256), 0, stream,
                           (const float *)k, L, norm_log2, target_log2, unit, kscale);
        break;
    case ST_F16:
        hipLaunchKernelGGL(filter_scale_kernel<__half>, dim3((unsigned)H), dim3(256), 0, stream,
                           (const __half *)k, L, norm_log2, target_log2, unit, kscale);
        break;
    default:
        hipLaunchKernelGGL(filter_scale_kernel<__hip_bfloat16>, dim3((unsigned)H), dim3(256), 0,
                           stream, (const __hip_bfloat16 *)k, L, norm_log2, target_log2, unit, kscale);
    }
    return hipGetLastError();
}

hipError_t launch_write_header(const KfHeader &hdr, void *K_f, hipStream_t stream) {
    hipLaunchKernelGGL(write_header_kernel, dim3(1), dim3(64), 0, stream, hdr, (KfHeader *)K_f);
    return hipGetLastError();
}

}  // namespace fftconv
