// bwd.hip -- small kernels of the backward pass.  The transforms themselves
// run on the forward kernels (the host side in api.cpp wires them):
//
//   dv = dy * conv(u w, k)            forward call with dy as the output gate
//   du = w * corr(v dy, k)            forward call on the conjugated spectrum
//   dw = u * corr(v dy, k)            (correlation = product with conj K)
//   dk[h, s] = sum_b corr(v dy, u w)[b, h, s],  s < L
//
// For dk every sequence x = u w is prepared as a filter of its own channel
// (b, h), its spectrum conjugated, and the forward kernels correlate v dy with
// it; a reduction over b follows.  With a frequency mask, the mask multiplies
// the conjugated spectra as it multiplies K in the forward pass, which is the
// adjoint because the mask is real.
#include "fft_device.hpp"
#include "fftconv_internal.hpp"

#include <type_traits>

namespace fftconv {

// Conjugate the stored bins of a prepared spectrum (dst may equal src).  A
// channel's bins are viewed as 16-byte units (q4_per_channel of them).
//   PAIR layouts: each unit is a chunk re[4], im[4] (fp16): words z, w hold
//     the imaginary parts.
//   NATURAL / ROWS: slot 0 holds (K[0], K[N]), both real, and stays; every
//     other slot is one complex bin whose imaginary part is its upper half
//     (fp16 pair: the high 16 bits of a word; fp32 pair: the odd words).
// grid (units / 256, channel stride); lanes index units of one channel.
__global__ void __launch_bounds__(256)
conj_bins_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t H, uint32_t q4_per_channel,
                 int kind) {
    const uint32_t q = blockIdx.x * 256u + threadIdx.x;
    if (q >= q4_per_channel) return;
    uint4 m;
    if (kind == 0) {
        m = make_uint4(0u, 0u, 0x80008000u, 0x80008000u);
    } else if (kind == 1) {
        m = make_uint4(q == 0 ? 0u : 0x80000000u, 0x80000000u, 0x80000000u, 0x80000000u);
    } else {
        m = make_uint4(0u, q == 0 ? 0u : 0x80000000u, 0u, 0x80000000u);
    }
    for (int64_t c = blockIdx.y; c < H; c += gridDim.y) {
        const int64_t i = c * q4_per_channel + q;
        const uint4 x = src[i];
        dst[i] = make_uint4(x.x ^ m.x, x.y ^ m.y, x.z ^ m.z, x.w ^ m.w);
    }
}

// x = u * w elementwise (the product formed in fp32, rounded once to T).
template <typename T>
__global__ void __launch_bounds__(256)
gate_product_kernel(const T *__restrict__ u, const T *__restrict__ w, T *__restrict__ x, int64_t npairs) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < npairs; i += (int64_t)gridDim.x * 256) {
        const float2 a = io<T>::load2(u + 2 * i), b = io<T>::load2(w + 2 * i);
        io<T>::store2(x + 2 * i, make_float2(a.x * b.x, a.y * b.y));
    }
}

// mask rows of the per-sequence channels: dst[c] = mask[c mod H]
__global__ void __launch_bounds__(128)
mask_repeat_kernel(const uint8_t *__restrict__ mask, uint8_t *__restrict__ dst, int64_t H) {
    const int64_t c = blockIdx.x;
    dst[c * kMaskBlocks + threadIdx.x] = mask[(c % H) * kMaskBlocks + threadIdx.x];
}

// dk[h, s] = sum_b part[b H + h, s] for s < L (fp32 sum, rounded once to T).  Grid
// (ceil(L / 2048), channels): a thread sums 8 consecutive s of one channel, one 16-byte
// load per partial row (two for fp32; rows are N-element aligned and s0 + 8 <= N).
template <typename T> __device__ __forceinline__ void load8f(const T *p, float *o);
template <> __device__ __forceinline__ void load8f<float>(const float *p, float *o) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    o[0] = a.x, o[1] = a.y, o[2] = a.z, o[3] = a.w, o[4] = b.x, o[5] = b.y, o[6] = b.z, o[7] = b.w;
}
template <> __device__ __forceinline__ void load8f<__half>(const __half *p, float *o) {
    const uint4 q = *reinterpret_cast<const uint4 *>(p);
    const __half *hv = reinterpret_cast<const __half *>(&q);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = __half2float(hv[i]);
}
template <> __device__ __forceinline__ void load8f<__hip_bfloat16>(const __hip_bfloat16 *p, float *o) {
    const uint4 q = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

template <typename T>
__global__ void __launch_bounds__(256)
dk_reduce_kernel(const T *__restrict__ part, T *__restrict__ dk, int64_t B, int64_t H, int64_t N,
                 int64_t L) {
    const int64_t s0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (s0 >= L) return;
    const int n = L - s0 < 8 ? (int)(L - s0) : 8;
    for (int64_t h = blockIdx.y; h < H; h += gridDim.y) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int64_t b = 0; b < B; ++b) {
            float x[8];
            load8f<T>(part + (b * H + h) * N + s0, x);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += x[i];
        }
        T *o = dk + h * L + s0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i >= n) break;
            if constexpr (std::is_same<T, float>::value) {
                o[i] = acc[i];
            } else if constexpr (std::is_same<T, __half>::value) {
                o[i] = __float2half_rn(acc[i]);
            } else {
                o[i] = __float2bfloat16(acc[i]);
            }
        }
    }
}

static unsigned grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    return (unsigned)(g > 65536 ? 65536 : (g < 1 ? 1 : g));
}

hipError_t launch_conj_bins(const void *src, void *dst, int64_t H, int64_t bytes_per_channel, int kind,
                            hipStream_t stream) {
    const uint32_t q4 = (uint32_t)(bytes_per_channel / 16);
    const dim3 grid((q4 + 255) / 256, (unsigned)(H < 4096 ? H : 4096));
    hipLaunchKernelGGL(conj_bins_kernel, grid, dim3(256), 0, stream, (const uint4 *)src, (uint4 *)dst, H, q4,
                       kind);
    return hipGetLastError();
}

hipError_t launch_gate_product(int st, const void *u, const void *w, void *x, int64_t n, hipStream_t stream) {
    const int64_t npairs = n / 2;
    switch (st) {
    case ST_F32:
        hipLaunchKernelGGL(gate_product_kernel<float>, dim3(grid_for(npairs)), dim3(256), 0, stream,
                           (const float *)u, (const float *)w, (float *)x, npairs);
        break;
    case ST_F16:
        hipLaunchKernelGGL(gate_product_kernel<__half>, dim3(grid_for(npairs)), dim3(256), 0, stream,
                           (const __half *)u, (const __half *)w, (__half *)x, npairs);
        break;
    default:
        hipLaunchKernelGGL(gate_product_kernel<__hip_bfloat16>, dim3(grid_for(npairs)), dim3(256), 0, stream,
                           (const __hip_bfloat16 *)u, (const __hip_bfloat16 *)w, (__hip_bfloat16 *)x, npairs);
    }
    return hipGetLastError();
}

hipError_t launch_mask_repeat(const uint8_t *mask, uint8_t *dst, int64_t H, int64_t C, hipStream_t stream) {
    hipLaunchKernelGGL(mask_repeat_kernel, dim3((unsigned)C), dim3(kMaskBlocks), 0, stream, mask, dst, H);
    return hipGetLastError();
}

hipError_t launch_dk_reduce(int st, const void *part, void *dk, int64_t B, int64_t H, int64_t N, int64_t L,
                            hipStream_t stream) {
    if (H < 1 || L < 1) return hipSuccess;
    const dim3 grid((unsigned)((L + 2047) / 2048), (unsigned)(H < 65535 ? H : 65535));
    switch (st) {
    case ST_F32:
        hipLaunchKernelGGL(dk_reduce_kernel<float>, grid, dim3(256), 0, stream, (const float *)part,
                           (float *)dk, B, H, N, L);
        break;
    case ST_F16:
        hipLaunchKernelGGL(dk_reduce_kernel<__half>, grid, dim3(256), 0, stream, (const __half *)part,
                           (__half *)dk, B, H, N, L);
        break;
    default:
        hipLaunchKernelGGL(dk_reduce_kernel<__hip_bfloat16>, grid, dim3(256), 0, stream,
                           (const __hip_bfloat16 *)part, (__hip_bfloat16 *)dk, B, H, N, L);
    }
    return hipGetLastError();
}

}  // namespace fftconv
