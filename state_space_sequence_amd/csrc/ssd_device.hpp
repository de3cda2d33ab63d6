// ssd_device.hpp -- device-side building blocks shared by the libssd kernels
// (gfx950 / CDNA4, wave64).
//
// MFMA fragment convention used everywhere in this library.  A "K-step" of a
// 16x16 output tile contracts KS values of k.  For both operands, lane l of
// the wave holds VEC consecutive k values of one row (A) or one column (B):
//
//      row/col = l % 16,     k = k0 + VEC * (l / 16) + j,   j = 0 .. VEC-1
//
//   bf16: VEC = 8, KS = 32, one v_mfma_f32_16x16x32_bf16 per K-step.
//   fp32: VEC = 4, KS = 16, four v_mfma_f32_16x16x4_f32; instruction j takes
//         element j of every lane, so lane group q supplies k = 4q + j.  The
//         contraction covers all 16 k exactly once, and A and B agree on which
//         k each (lane, element) slot carries, which is all a sum over k needs.
//
// The 16x16 fp32 result tile D is spread as: lane l holds
//      D[4 * (l / 16) + i][l % 16],   i = 0 .. 3        (f32x4 element i).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- conversions

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// fptrunc float -> bf16 rounds to nearest even.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// ----------------------------------------------------------------- MFMA traits

template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int VEC = 8;
    static constexpr int KS = 32;
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int VEC = 4;
    static constexpr int KS = 16;
    typedef f32x4 frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
};

// Load VEC consecutive elements (one 16-byte vector) as a fragment.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_frag(const T *p) {
    return *reinterpret_cast<const typename Mma<T>::frag *>(p);
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag zero_frag() {
    typename Mma<T>::frag f;
#pragma unroll
    for (int j = 0; j < Mma<T>::VEC; ++j) f[j] = from_f32<T>(0.f);
    return f;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ----------------------------------------------------------------- wave scan

// Inclusive prefix sum of `v` over the 64 lanes of the wave.
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        float o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

__device__ __forceinline__ double wave_inclusive_scan_f64(double v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        double o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

__device__ __forceinline__ float fast_exp(float v) { return __expf(v); }

// SiLU, v / (1 + e^-v), from the hardware exp and reciprocal (for large
// negative v, e^-v overflows to infinity and the result is 0, the limit).
// The layer's activation after the conv, its gate in the norm, and the
// output gate of the scan and decode calls.
__device__ __forceinline__ float silu_f32(float v) {
    return v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
}

// softplus(v) = log(1 + e^v) in fp32, as max(v, 0) + log1p(t) with
// t = e^-|v| in (0, 1].  log1p(t) is evaluated from the hardware log as
// log(u) * t / (u - 1), u = 1 + t (t itself when u rounds to 1): the
// rounding error of u cancels in the ratio (Goldberg, "What every computer
// scientist should know about floating-point arithmetic", 1991, the log1p
// example), leaving a few ulps.  About ten instructions, against several
// tens for the general log1pf.
__device__ __forceinline__ float softplus_f32(float v) {
    const float t = __expf(-fabsf(v));
    const float u = 1.f + t;
    const float l = u == 1.f ? t : __logf(u) * (t * __builtin_amdgcn_rcpf(u - 1.f));
    return fmaxf(v, 0.f) + l;
}

// The layer's time-step preprocessing (the `_ex` entry points): bias, then
// softplus, then the clamp to [lo, hi].
__device__ __forceinline__ float dt_process(float v, float bias, bool softplus, float lo,
                                            float hi) {
    v += bias;
    if (softplus) v = softplus_f32(v);
    return fminf(fmaxf(v, lo), hi);
}

// a - b for two prefix sums held as (hi, lo) float pairs.  When a and b are
// close, hi_a - hi_b is exact (Sterbenz), so the result keeps the accuracy
// of the small difference instead of the ulp of the large prefixes.
__device__ __forceinline__ float prefix_diff(float a_hi, float a_lo, float b_hi, float b_lo) {
    return (a_hi - b_hi) + (a_lo - b_lo);
}

}  // namespace ssd
