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
// One workgroup per row, of as many whole waves as the row's 8-value vectors
// (16 bytes in bf16) need at one vector per thread (rows of up to 256 vectors) or two: thread i
// holds vectors i and i + nt of the row (8 values each) in registers, the sum
// of squares is reduced within each wave and then across the waves through
// LDS, and the row is scaled and stored.  (At 5120 values, 320 threads with
// two vectors each run 3% faster than 256 threads with three, half of them
// clamped, by A/B.)  The loads of y and z are unconditional (from a
// clamped vector where a thread has none), so a thread's loads all issue
// before it waits.  It reads y and z and writes out once, so it is bound by
// HBM bandwidth; the output stores carry the non-temporal hint.
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
__device__ __forceinline__ float nsilu(float v) { return silu_f32(v); }

}  // namespace

// grid (rows), nt threads (a multiple of 64, at most 512) with NV 8-value
// vectors per thread covering the row: 8 NV nt >= dim; dim % 8 == 0.  GATE: 0
// none, 1 gate before the normalisation, 2 after it.
template <typename T, int NV, int GATE>
__global__ void __launch_bounds__(512)
k_gated_rmsnorm(const T *__restrict__ y, const T *__restrict__ z, const float *__restrict__ w,
                T *__restrict__ out, int dim, float eps) {
    __shared__ float s_part[8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nt = blockDim.x;
    const size_t base = (size_t)blockIdx.x * dim;
    float g[NV][8], zv[GATE ? NV : 1][8];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = min(8 * (tid + nt * i), dim - 8);
        nload8(y + base + c, g[i]);
        if (GATE) nload8(z + base + c, zv[GATE ? i : 0]);
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const bool valid = 8 * (tid + nt * i) < dim;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (GATE == 1) g[i][j] *= nsilu(zv[GATE ? i : 0][j]);
            if (!valid) g[i][j] = 0.f;
            ss += g[i][j] * g[i][j];
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if (lane == 0) s_part[wave] = ss;
    __syncthreads();
    ss = s_part[0];
    for (int k = 1; k < (nt >> 6); ++k) ss += s_part[k];
    const float rstd = __builtin_amdgcn_rsqf(ss / (float)dim + eps);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = 8 * (tid + nt * i);
        if (c < dim) {
            float wv[8], o[8];
            nload8(w + c, wv);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                o[j] = g[i][j] * rstd * wv[j];
                if (GATE == 2) o[j] *= nsilu(zv[GATE ? i : 0][j]);
            }
            nstore8(out + base + c, o);
        }
    }
}

template <typename T>
hipError_t launch_gated_rmsnorm(const NormArgs &a, hipStream_t stream) {
    // 8-value vectors of a row, per thread (1 up to 256 of them, else 2), and
    // the threads: whole waves, at most 512 (dim <= kMaxNormDim = 8192)
    const int vecs = a.dim / 8, nv = vecs <= 256 ? 1 : 2;
    const int nt = ((vecs + nv - 1) / nv + 63) / 64 * 64;
    if (nt > 512) return hipErrorInvalidValue;
#define SSD_NORM_CASE(NN, GG)                                                               \
    if (nv == NN && a.gate == GG) {                                                         \
        hipLaunchKernelGGL((k_gated_rmsnorm<T, NN, GG>), dim3(a.rows), dim3(nt), 0, stream, \
                           (const T *)a.y, (const T *)a.z, a.w, (T *)a.out, a.dim, a.eps); \
        return hipGetLastError();                                                           \
    }
#define SSD_NORM_GATES(NN) SSD_NORM_CASE(NN, 0) SSD_NORM_CASE(NN, 1) SSD_NORM_CASE(NN, 2)
    SSD_NORM_GATES(1)
    SSD_NORM_GATES(2)
#undef SSD_NORM_GATES
#undef SSD_NORM_CASE
    return hipErrorInvalidValue;
}

template hipError_t launch_gated_rmsnorm<float>(const NormArgs &, hipStream_t);
template hipError_t launch_gated_rmsnorm<bf16>(const NormArgs &, hipStream_t);

}  // namespace ssd
