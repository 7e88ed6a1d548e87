// kamera_common.h — device and host helpers shared by the Kamera HIP sources
// (relocation/patch kernels and patch formation).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Division by a runtime constant with a multiply-high (Granlund & Montgomery,
// "Division by invariant integers using multiplication", 1994): for
// 0 <= x < 2^31, x / d = (mulhi(x, mul) + x) >> shr.
struct FastDiv {
    uint32_t d, mul, shr;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    uint64_t mul = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)mul, l};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv& f) {
    return (__umulhi(x, f.mul) + x) >> f.shr;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4 ld_stream(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld_cached(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// A workgroup-uniform read of an input the kernels never write, through the
// constant address space: it becomes a scalar load, which is counted apart
// from the vector loads and so never holds up a wait on them.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* ptr) {
    return *(const __attribute__((address_space(4))) T*)ptr;
}
// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left at their maxima: gfx9 encoding).
// Placed where no vector load can be in flight, it costs nothing and tells the
// compiler's wait tracking so, which otherwise assumes loads of a sibling
// code path may still be pending and makes later loads wait on them.
__device__ __forceinline__ void vm_settled() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ void st_stream(uint16_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// cos/sin of phi = delta * theta_j.  phi reaches ~1e7 rad for the largest
// shifts, where an fp32 product is useless, so phi and its reduction
// r = phi - k*pi/2 (|r| <= pi/4, Cody-Waite with a two-term pi/2) are fp64.
// sin r and cos r then come from their Taylor series in fp32; truncated after
// r^11 and r^12 they are off by < 1e-11 on |r| <= pi/4, so the fp32 rounding
// (a few 1e-8) dominates and the table is far finer than the bf16 spacing of
// the results.  The quadrant k mod 4 picks signs and swaps.
__device__ __forceinline__ float2 rope_cos_sin(double log2_base, int rope_dim, int j, int64_t delta) {
    // theta_j = base^(-2j/R) = 2^(log2(base) * (-2j/R)), fp64 (relative error
    // ~1e-15: ~1e-8 rad on the largest phases).  Pure arithmetic on values
    // every lane already holds, so it overlaps the loads in flight (a table
    // read here would be a vector load issued after the rows, and waiting for
    // it would wait for the rows too).
    const double theta = exp2(log2_base * (-2.0 * (double)j / (double)rope_dim));
    const double kHalfPiHi = 1.5707963267948966;       // fp64(pi/2)
    const double kHalfPiLo = 6.123233995736766e-17;    // pi/2 - kHalfPiHi
    const double kTwoOverPi = 0.6366197723675814;
    const double phi = (double)delta * theta;
    const double k = rint(phi * kTwoOverPi);
    double r = fma(-k, kHalfPiHi, phi);
    r = fma(-k, kHalfPiLo, r);
    const float x = (float)r;
    const float x2 = x * x;
    // sin x = x (1 - x^2/3! + x^4/5! - x^6/7! + x^8/9! - x^10/11!)
    float sp = -2.5052108385441720e-08f;
    sp = fmaf(sp, x2, 2.7557319223985893e-06f);
    sp = fmaf(sp, x2, -1.9841269841269841e-04f);
    sp = fmaf(sp, x2, 8.3333333333333332e-03f);
    sp = fmaf(sp, x2, -1.6666666666666666e-01f);
    const float sn = fmaf(sp * x2, x, x);
    // cos x = 1 - x^2/2! + x^4/4! - x^6/6! + x^8/8! - x^10/10! + x^12/12!
    float cp = 2.0876756987868099e-09f;
    cp = fmaf(cp, x2, -2.7557319223985888e-07f);
    cp = fmaf(cp, x2, 2.4801587301587302e-05f);
    cp = fmaf(cp, x2, -1.3888888888888889e-03f);
    cp = fmaf(cp, x2, 4.1666666666666664e-02f);
    cp = fmaf(cp, x2, -0.5f);
    const float cn = fmaf(cp, x2, 1.0f);
    const int q = (int)((long long)k & 3);
    float c, s;
    switch (q) {
        case 0: c = cn; s = sn; break;
        case 1: c = -sn; s = cn; break;
        case 2: c = -cn; s = -sn; break;
        default: c = sn; s = -cn; break;
    }
    return make_float2(c, s);
}

// Launch with the arguments converted to the kernel's own parameter types:
// a missing, extra or mistyped argument fails to compile instead of handing
// the kernel shifted bytes.
template <typename... P, typename Tuple, size_t... I>
hipError_t launch_tuple(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, Tuple& args,
                        std::index_sequence<I...>) {
    void* ptrs[] = {(void*)&std::get<I>(args)...};
    return hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, stream);
}

template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, const A&... a) {
    static_assert(sizeof...(P) == sizeof...(A), "argument count does not match the kernel");
    std::tuple<std::decay_t<P>...> args(a...);
    return launch_tuple(kernel, grid, block, stream, args, std::index_sequence_for<P...>{});
}

inline bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;
};

inline bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Elements -> byte span of a strided [outer][...][rows][F] region.
inline Span span_of(const void* base, int64_t elems) {
    uintptr_t lo = (uintptr_t)base;
    return Span{lo, lo + (uintptr_t)elems * 2u};
}

}  // namespace
