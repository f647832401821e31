// fft_device.hpp -- device building blocks for the gfx950 FFT convolution:
// complex arithmetic in fp32, storage-type conversion, in-register radix-R
// DFTs and the twiddle lookups shared by the fused and multi-pass kernels.
//
// The convolution is evaluated with the convolution theorem (FlashFFTConv
// summary page, "Summary": exact FFT convolution).  Each DFT is split into
// radix stages ("Approach": an order-p decomposition of the FFT into small
// dense transforms with permutations done on chip).  Here each small transform
// is a radix-R DFT held in registers of one lane, and the permutations between
// stages go through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace fftconv {

// --------------------------------------------------------------- complex fp32
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
// multiply by -i
__device__ __forceinline__ float2 cmul_negi(float2 a) { return make_float2(a.y, -a.x); }
// multiply by +i
__device__ __forceinline__ float2 cmul_posi(float2 a) { return make_float2(-a.y, a.x); }
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }

// ------------------------------------------------------- storage conversions
// load2/store2 take an optional element offset e (a lane value): the access
// is then formed as uniform pointer + 32-bit byte offset.
template <typename T> struct io;
template <> struct io<float> {
    static __device__ __forceinline__ float2 load2(const float *p, uint32_t e = 0) {
        return *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(p) + 8u * e);
    }
    static __device__ __forceinline__ void store2(float *p, float2 v) { *reinterpret_cast<float2 *>(p) = v; }
    static __device__ __forceinline__ void store2(float *p, uint32_t e, float2 v) {
        *reinterpret_cast<float2 *>(reinterpret_cast<char *>(p) + 8u * e) = v;
    }
    static __device__ __forceinline__ float load1(const float *p) { return *p; }
};
template <> struct io<__half> {
    static __device__ __forceinline__ float2 load2(const __half *p, uint32_t e = 0) {
        __half2 h = *reinterpret_cast<const __half2 *>(reinterpret_cast<const char *>(p) + 4u * e);
        return __half22float2(h);
    }
    static __device__ __forceinline__ void store2(__half *p, float2 v) {
        *reinterpret_cast<__half2 *>(p) = __floats2half2_rn(v.x, v.y);
    }
    static __device__ __forceinline__ void store2(__half *p, uint32_t e, float2 v) {
        *reinterpret_cast<__half2 *>(reinterpret_cast<char *>(p) + 4u * e) = __floats2half2_rn(v.x, v.y);
    }
    static __device__ __forceinline__ float load1(const __half *p) { return __half2float(*p); }
};
template <> struct io<__hip_bfloat16> {
    static __device__ __forceinline__ float2 load2(const __hip_bfloat16 *p, uint32_t e = 0) {
        uint32_t bits = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(p) + 4u * e);
        return make_float2(__uint_as_float(bits << 16), __uint_as_float(bits & 0xffff0000u));
    }
    static __device__ __forceinline__ uint32_t pack(float2 v) {
        __hip_bfloat16 a = __float2bfloat16(v.x), b = __float2bfloat16(v.y);
        return (uint32_t)(*reinterpret_cast<uint16_t *>(&a)) |
               ((uint32_t)(*reinterpret_cast<uint16_t *>(&b)) << 16);
    }
    static __device__ __forceinline__ void store2(__hip_bfloat16 *p, float2 v) {
        *reinterpret_cast<uint32_t *>(p) = pack(v);
    }
    static __device__ __forceinline__ void store2(__hip_bfloat16 *p, uint32_t e, float2 v) {
        *reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(p) + 4u * e) = pack(v);
    }
    static __device__ __forceinline__ float load1(const __hip_bfloat16 *p) { return __bfloat162float(*p); }
};

// A raw buffer view of `bytes` bytes at p (wave-uniform).  A buffer load
// whose offset lies past the end returns zero without touching memory (the
// buffer unit's range check), so an offset of kBufferSkip reads a zero at no
// HBM cost and without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kBufferSkip = 0x80000000u;

// Filter-spectrum bins: fp32 complex or fp16 complex (same element-offset forms).
template <typename TK> struct kio;
template <> struct kio<float2> {
    static __device__ __forceinline__ float2 load(const float2 *p, uint32_t e = 0) {
        return *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(p) + 8u * e);
    }
    // bin at byte offset off of a buffer view (zero past its end)
    static __device__ __forceinline__ float2 load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        return make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
    }
    static __device__ __forceinline__ void store(float2 *p, float2 v) { *p = v; }
    static __device__ __forceinline__ void store(float2 *p, uint32_t e, float2 v) {
        *reinterpret_cast<float2 *>(reinterpret_cast<char *>(p) + 8u * e) = v;
    }
};
template <> struct kio<__half2> {
    static __device__ __forceinline__ float2 load(const __half2 *p, uint32_t e = 0) {
        return __half22float2(*reinterpret_cast<const __half2 *>(reinterpret_cast<const char *>(p) + 4u * e));
    }
    static __device__ __forceinline__ float2 load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        return __half22float2(*reinterpret_cast<const __half2 *>(&v));
    }
    static __device__ __forceinline__ void store(__half2 *p, float2 v) { *p = __floats2half2_rn(v.x, v.y); }
    static __device__ __forceinline__ void store(__half2 *p, uint32_t e, float2 v) {
        *reinterpret_cast<__half2 *>(reinterpret_cast<char *>(p) + 4u * e) = __floats2half2_rn(v.x, v.y);
    }
};

// ------------------------------------------------ radix-R DFT in registers
// exp(-2 pi i q / 32) for q in [0, 16), from the double-precision values.
__device__ __forceinline__ float2 w32(int q) {
    switch (q) {
    case 0: return make_float2(1.0f, 0.0f);
    case 1: return make_float2(9.807852804e-01f, -1.950903220e-01f);
    case 2: return make_float2(9.238795325e-01f, -3.826834324e-01f);
    case 3: return make_float2(8.314696123e-01f, -5.555702330e-01f);
    case 4: return make_float2(7.071067812e-01f, -7.071067812e-01f);
    case 5: return make_float2(5.555702330e-01f, -8.314696123e-01f);
    case 6: return make_float2(3.826834324e-01f, -9.238795325e-01f);
    case 7: return make_float2(1.950903220e-01f, -9.807852804e-01f);
    case 8: return make_float2(0.0f, -1.0f);
    case 9: return make_float2(-1.950903220e-01f, -9.807852804e-01f);
    case 10: return make_float2(-3.826834324e-01f, -9.238795325e-01f);
    case 11: return make_float2(-5.555702330e-01f, -8.314696123e-01f);
    case 12: return make_float2(-7.071067812e-01f, -7.071067812e-01f);
    case 13: return make_float2(-8.314696123e-01f, -5.555702330e-01f);
    case 14: return make_float2(-9.238795325e-01f, -3.826834324e-01f);
    default: return make_float2(-9.807852804e-01f, -1.950903220e-01f);
    }
}

// Multiply by exp(-2 pi i q / R), 0 <= q < R (R <= 32), with the trivial
// angles done exactly; q >= R/2 uses exp(-2 pi i q / R) = -exp(-2 pi i (q - R/2) / R).
template <int R>
__device__ __forceinline__ float2 twiddle_const(float2 a, int q) {
    if (2 * q >= R) {
        a = make_float2(-a.x, -a.y);
        q -= R / 2;
    }
    if (q == 0) return a;
    if (4 * q == R) return cmul_negi(a);
    if (8 * q == R) {
        const float c = 7.071067812e-01f;
        return make_float2((a.x + a.y) * c, (a.y - a.x) * c);
    }
    if (8 * q == 3 * R) {
        const float c = 7.071067812e-01f;
        return make_float2((a.y - a.x) * c, -(a.x + a.y) * c);
    }
    return cmul(a, w32(q * (32 / R)));
}

// out[q] = sum_r in[r] exp(-2 pi i r q / R), radix-2 decimation in time,
// fully unrolled; in and out may not alias.
template <int R> struct Dft {
    static __device__ __forceinline__ void run(const float2 *in, float2 *out) {
        float2 e[R / 2], o[R / 2], E[R / 2], O[R / 2];
#pragma unroll
        for (int i = 0; i < R / 2; ++i) { e[i] = in[2 * i]; o[i] = in[2 * i + 1]; }
        Dft<R / 2>::run(e, E);
        Dft<R / 2>::run(o, O);
#pragma unroll
        for (int q = 0; q < R / 2; ++q) {
            float2 t = twiddle_const<R>(O[q], q);
            out[q] = cadd(E[q], t);
            out[q + R / 2] = csub(E[q], t);
        }
    }
};
template <> struct Dft<1> {
    static __device__ __forceinline__ void run(const float2 *in, float2 *out) { out[0] = in[0]; }
};
template <> struct Dft<2> {
    static __device__ __forceinline__ void run(const float2 *in, float2 *out) {
        out[0] = cadd(in[0], in[1]);
        out[1] = csub(in[0], in[1]);
    }
};
template <> struct Dft<4> {
    static __device__ __forceinline__ void run(const float2 *in, float2 *out) {
        float2 s0 = cadd(in[0], in[2]), d0 = csub(in[0], in[2]);
        float2 s1 = cadd(in[1], in[3]), d1 = cmul_negi(csub(in[1], in[3]));
        out[0] = cadd(s0, s1);
        out[2] = csub(s0, s1);
        out[1] = cadd(d0, d1);
        out[3] = csub(d0, d1);
    }
};

// In-place DFT of N = P * Q points in two register stages: n = p + P m,
// k = q + Q s.  Step 1, for each p, a Q-point DFT over m, written back in
// place and multiplied by omega_N^{pq}; step 2, for each q, a P-point DFT
// over p.  The result is relabelled into natural order at compile time.
// The scheduling barriers keep step 2's transforms from being interleaved,
// which bounds the registers live at once.
template <int P, int Q>
__device__ __forceinline__ void dft_pq(float2 *a) {
    constexpr int N = P * Q;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float2 t[Q], o[Q];
#pragma unroll
        for (int m = 0; m < Q; ++m) t[m] = a[p + P * m];
        Dft<Q>::run(t, o);
#pragma unroll
        for (int q = 0; q < Q; ++q) a[p + P * q] = twiddle_const<N>(o[q], p * q);
    }
    float2 out[N];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        float2 t[P], o[P];
#pragma unroll
        for (int p = 0; p < P; ++p) t[p] = a[p + P * q];
        Dft<P>::run(t, o);
#pragma unroll
        for (int s = 0; s < P; ++s) out[q + Q * s] = o[s];
    }
#pragma unroll
    for (int k = 0; k < N; ++k) a[k] = out[k];
}

// In-place radix-R DFT of a register array.
template <int R>
__device__ __forceinline__ void dft_inplace(float2 *a) {
    float2 t[R];
#pragma unroll
    for (int i = 0; i < R; ++i) t[i] = a[i];
    Dft<R>::run(t, a);
}

// ------------------------------------------------------ uniform addressing
// Global addresses as a wave-uniform base plus an unsigned 32-bit byte
// offset, which maps onto the scalar-base addressing form of global loads and
// stores (no per-lane 64-bit pointers to keep live).
template <typename V, typename P>
__device__ __forceinline__ V ldu(const P *base, uint32_t byte_off) {
    return *reinterpret_cast<const V *>(reinterpret_cast<const char *>(base) + byte_off);
}
template <typename V, typename P>
__device__ __forceinline__ void stu(P *base, uint32_t byte_off, const V &x) {
    *reinterpret_cast<V *>(reinterpret_cast<char *>(base) + byte_off) = x;
}
// Streaming (non-temporal) forms for data that is read or written once: they do not
// keep the stream in L2 ahead of data that is reused (filter spectra, tables).
template <typename V>
__device__ __forceinline__ V ldnt(const void *p) {
    static_assert(sizeof(V) % 4 == 0 && sizeof(V) <= 16, "32-bit words");
    if constexpr (sizeof(V) == 4) {
        return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const unsigned int *>(p)));
    } else {
        typedef unsigned int w_t __attribute__((ext_vector_type(sizeof(V) / 4)));
        return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const w_t *>(p)));
    }
}
template <typename V>
__device__ __forceinline__ void stnt(void *p, const V &x) {
    static_assert(sizeof(V) % 4 == 0 && sizeof(V) <= 16, "32-bit words");
    if constexpr (sizeof(V) == 4) {
        __builtin_nontemporal_store(__builtin_bit_cast(unsigned int, x), reinterpret_cast<unsigned int *>(p));
    } else {
        typedef unsigned int w_t __attribute__((ext_vector_type(sizeof(V) / 4)));
        __builtin_nontemporal_store(__builtin_bit_cast(w_t, x), reinterpret_cast<w_t *>(p));
    }
}
template <typename V, typename P>
__device__ __forceinline__ V ldu_nt(const P *base, uint32_t byte_off) {
    return ldnt<V>(reinterpret_cast<const char *>(base) + byte_off);
}
template <typename V, typename P>
__device__ __forceinline__ void stu_nt(P *base, uint32_t byte_off, const V &x) {
    stnt<V>(reinterpret_cast<char *>(base) + byte_off, x);
}
// Hide a lane value from loop-invariant code motion so that addresses built
// from it are recomputed where they are used instead of being held live.
__device__ __forceinline__ int launder(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// ------------------------------------------------------------ XCD mapping
// Workgroups are dispatched round-robin over the 8 XCDs of the MI355X
// (workgroup i runs on XCD i % 8).  This maps the hardware block id to a
// logical block id so that each XCD works on one contiguous range of logical
// blocks (a bijection on [0, nblocks)).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblocks) {
    const uint32_t xcds = 8;
    uint32_t x = bid % xcds, local = bid / xcds;
    uint32_t q = nblocks / xcds, r = nblocks % xcds;
    return x * q + (x < r ? x : r) + local;
}

}  // namespace fftconv
