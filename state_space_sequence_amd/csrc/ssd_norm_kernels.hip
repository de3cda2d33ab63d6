// ssd_norm_kernels.hip -- the gated RMS normalisation that follows the scan
// in the Mamba-2 layer.
//
// fla `layers/mamba2.py`: the layer builds `RMSNormGated(intermediate_size,
// eps=norm_eps, norm_before_gate=False)` and applies it as `norm(y, gate)`
// to the scan output y [b, L, H*P] and the gate z (the in-projection's gate
// channels).  With the gate applied before the normalisation, per row:
//
//     g   = y * silu(z)                      (silu(v) = v / (1 + e^-v))
//     out = g / sqrt(mean(g^2) + eps) * w    (mean over the row's dim values)
//
// and with it after (norm_before_gate): out = y / sqrt(mean(y^2) + eps) * w *
// silu(z).  Without a gate it is the plain RMS normalisation.
//
// One wave per row: lane l holds the 16-byte vectors l, l + 64, ... of the
// row (8 values each) in registers, the sum of squares is reduced across the
// wave, and the row is scaled and stored.  It reads y and z and writes out
// once, so it is bound by HBM bandwidth; the output stores carry the
// non-temporal hint.
#include "ssd_device.hpp"
#include "ssd_kernels.hpp"

namespace ssd {

namespace {

__device__ __forceinline__ void nload8(const bf16 *p, float (&v)[8]) {
    const bf16x8 q = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)q[j];
}
__device__ __forceinline__ void nload8(const float *p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = a[j];
        v[4 + j] = b[j];
    }
}
__device__ __forceinline__ void nstore8(bf16 *p, const float (&v)[8]) {
    bf16x8 q;
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = (bf16)v[j];
    __builtin_nontemporal_store(q, reinterpret_cast<bf16x8 *>(p));
}
__device__ __forceinline__ void nstore8(float *p, const float (&v)[8]) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4 *>(p + 4));
}
__device__ __forceinline__ float nsilu(float v) {
    return v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
}

}  // namespace

// grid (ceil(rows / 4)), 256 threads (4 rows per workgroup); NV 16-byte
// vectors per lane cover up to 512 NV values of a row; dim % 8 == 0.
// gate: 0 none, 1 gate before the normalisation, 2 after it.
template <typename T, int NV>
__global__ void __launch_bounds__(256)
k_gated_rmsnorm(const T *__restrict__ y, const T *__restrict__ z, const float *__restrict__ w,
                T *__restrict__ out, int rows, int dim, float eps, int gate) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    const size_t base = (size_t)row * dim;
    float g[NV][8];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = 8 * (lane + 64 * i);
        if (c < dim) {
            nload8(y + base + c, g[i]);
            if (gate == 1) {
                float zv[8];
                nload8(z + base + c, zv);
#pragma unroll
                for (int j = 0; j < 8; ++j) g[i][j] *= nsilu(zv[j]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) ss += g[i][j] * g[i][j];
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    const float rstd = __builtin_amdgcn_rsqf(ss / (float)dim + eps);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = 8 * (lane + 64 * i);
        if (c < dim) {
            float wv[8], o[8];
            nload8(w + c, wv);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = g[i][j] * rstd * wv[j];
            if (gate == 2) {
                float zv[8];
                nload8(z + base + c, zv);
#pragma unroll
                for (int j = 0; j < 8; ++j) o[j] *= nsilu(zv[j]);
            }
            nstore8(out + base + c, o);
        }
    }
}

template <typename T>
hipError_t launch_gated_rmsnorm(const NormArgs &a, hipStream_t stream) {
    const dim3 grid((a.rows + 3) / 4);
    const int nv = (a.dim / 8 + 63) / 64;  // 16-byte vectors per lane
#define SSD_NORM_CASE(NN)                                                                     \
    if (nv <= NN) {                                                                           \
        hipLaunchKernelGGL((k_gated_rmsnorm<T, NN>), grid, dim3(256), 0, stream,             \
                           (const T *)a.y, (const T *)a.z, a.w, (T *)a.out, a.rows, a.dim, a.eps, \
                           a.gate);                                                           \
        return hipGetLastError();                                                             \
    }
    SSD_NORM_CASE(2)
    SSD_NORM_CASE(4)
    SSD_NORM_CASE(8)
    SSD_NORM_CASE(16)
#undef SSD_NORM_CASE
    return hipErrorInvalidValue;
}

template hipError_t launch_gated_rmsnorm<float>(const NormArgs &, hipStream_t);
template hipError_t launch_gated_rmsnorm<bf16>(const NormArgs &, hipStream_t);

}  // namespace ssd
