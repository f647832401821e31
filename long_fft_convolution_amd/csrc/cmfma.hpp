// cmfma.hpp -- complex 16x16 tile products on the MFMA matrix cores
// (v_mfma_f32_16x16x32_f16: fp16 operands, fp32 accumulation), shared by the
// matrix-core kernels.  A complex tile is a pair of planes (re, im); with the
// operand layouts of the instruction (A: lane l holds row l % 16, K slots
// 8 (l / 16) .. + 7; B: column l % 16, the same K slots; D: lane l holds rows
// 4 (l / 16) + i of column l % 16), one complex 16x16x32 product is four real
// products.  The accumulator layout of one stage is the operand layout of the
// next once the contraction index is permuted: K slot 8g + j <-> row 4g + j
// (j < 4) of tile 0, row 4g + j - 4 of tile 1 (kslot below).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace fftconv {
namespace cmfma {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ h8 neg8(const h8 &a) {
    uint4 q = *reinterpret_cast<const uint4 *>(&a);
    q.x ^= 0x80008000u;
    q.y ^= 0x80008000u;
    q.z ^= 0x80008000u;
    q.w ^= 0x80008000u;
    return *reinterpret_cast<const h8 *>(&q);
}
__device__ __forceinline__ h4 to_h4(const f4 &a) {
    h4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (_Float16)a[i];
    return r;
}
__device__ __forceinline__ h8 cat8(const h4 &lo, const h4 &hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ h4 lo4(const h8 &a) { return __builtin_shufflevector(a, a, 0, 1, 2, 3); }
__device__ __forceinline__ h4 hi4(const h8 &a) { return __builtin_shufflevector(a, a, 4, 5, 6, 7); }
// (re, im) <- (re, im) * (c + i s); t = {c[0..3], s[0..3]}
__device__ __forceinline__ void cmul4(h4 &re, h4 &im, const h8 &t) {
    const h4 c = lo4(t), s = hi4(t);
    const h4 r = re * c - im * s;
    im = re * s + im * c;
    re = r;
}
// complex 16x16x32 tile products, (re, im) planes; "data A": C = D F, "const A": C = F D.
// The constant's imaginary plane is also held negated (nfi = -Im F), so that no data plane
// is ever negated.
__device__ __forceinline__ void cm_dataA(const h8 &dr, const h8 &di, const h8 &fr, const h8 &fi,
                                         const h8 &nfi, f4 &cr, f4 &ci) {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    cr = mfma(di, nfi, mfma(dr, fr, z));
    ci = mfma(di, fr, mfma(dr, fi, z));
}
__device__ __forceinline__ void cm_constA(const h8 &fr, const h8 &fi, const h8 &nfi, const h8 &dr,
                                          const h8 &di, f4 &cr, f4 &ci) {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    cr = mfma(nfi, di, mfma(fr, dr, z));
    ci = mfma(fi, dr, mfma(fr, di, z));
}
// the same with conj(F)
__device__ __forceinline__ void cm_dataA_conj(const h8 &dr, const h8 &di, const h8 &fr, const h8 &fi,
                                              const h8 &nfi, f4 &cr, f4 &ci) {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    cr = mfma(di, fi, mfma(dr, fr, z));
    ci = mfma(dr, nfi, mfma(di, fr, z));
}
__device__ __forceinline__ void cm_constA_conj(const h8 &fr, const h8 &fi, const h8 &nfi, const h8 &dr,
                                               const h8 &di, f4 &cr, f4 &ci) {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    cr = mfma(fi, di, mfma(fr, dr, z));
    ci = mfma(nfi, dr, mfma(fr, di, z));
}

// K slot (0..31) of row r (0..31) in a chained operand: rows 4g + j of tile 0
// -> slot 8g + j, rows 16 + 4g + j -> slot 8g + 4 + j
__device__ __forceinline__ int kslot(int r) {
    return 8 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3);
}

}  // namespace cmfma
}  // namespace fftconv
