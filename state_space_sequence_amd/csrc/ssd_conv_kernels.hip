// ssd_conv_kernels.hip -- the causal depthwise convolution that precedes the
// scan in the Mamba-2 layer, and its single-token update.
//
// fla `layers/mamba2.py`, `Mamba2.torch_forward` (and the transformers-style
// layer of the fla model page): the concatenated x | B | C channels go
// through `nn.Conv1d(conv_dim, conv_dim, kernel_size=W, groups=conv_dim,
// padding=W-1)`, truncated to the first seqlen outputs, then the activation
// (SiLU).  Per channel c, with x_t = 0 for t < 0:
//
//     out_t[c] = act(bias[c] + sum_{k<W} w[c][k] x_{t-W+1+k}[c])
//
// The cache of the decode path holds the last W inputs of every channel,
// [batch, conv_dim, W] (zero-padded on the left when the prefix is shorter);
// one decode step rolls it left by one, appends the new input and applies
// the same dot product (`update_conv_state` + the single-token branch).
//
// Both kernels stream their inputs once and are bound by HBM bandwidth.
// Forward: a thread owns 8 consecutive channels (one 16-byte bf16 vector) of
// one batch over a run of 64 tokens, keeps the last W inputs in registers and
// issues the loads of 8 tokens before using them; consecutive lanes take
// consecutive channel groups, so a wave reads 1 KB of each token row.
// Update: a thread owns one channel; its W-element cache row is contiguous.
// The forward's outputs are written once and carry the non-temporal hint
// (measured: 5% shorter on the 2.7B layer's channels; the same hint on the
// loads costs a third more time on a cache-resident 130M-size input).
#include "ssd_device.hpp"
#include "ssd_kernels.hpp"

namespace ssd {

namespace {

constexpr int kConvVec = 8;     // channels per thread (forward)
constexpr int kConvRun = 64;    // tokens per thread (forward)
constexpr int kConvBatch = 8;   // tokens whose loads are in flight together

// 8 consecutive channels of one token as fp32
__device__ __forceinline__ void load8(const bf16 *p, float (&v)[8]) {
    const bf16x8 q = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)q[j];
}
__device__ __forceinline__ void load8(const float *p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = a[j];
        v[4 + j] = b[j];
    }
}
__device__ __forceinline__ void store8(bf16 *p, const float (&v)[8]) {
    bf16x8 q;
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = (bf16)v[j];
    __builtin_nontemporal_store(q, reinterpret_cast<bf16x8 *>(p));
}
__device__ __forceinline__ void store8(float *p, const float (&v)[8]) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4 *>(p + 4));
}

// SiLU v sigmoid(v) = v / (1 + e^-v) (the layer's activation)
__device__ __forceinline__ float silu(float v) { return silu_f32(v); }

}  // namespace

// grid (ceil(D / 8 / nt), ceil(L / 64), batch), nt <= 256 threads; D % 8 == 0.
template <typename T, int W>
__global__ void __launch_bounds__(256)
k_conv1d_fwd(const T *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
             T *__restrict__ out, T *__restrict__ state_out, int L, int D, int act_silu) {
    const int c0 = (blockIdx.x * blockDim.x + threadIdx.x) * kConvVec;
    if (c0 >= D) return;
    const int t0 = blockIdx.y * kConvRun, b = blockIdx.z;
    float wk[W][kConvVec], bj[kConvVec];
#pragma unroll
    for (int j = 0; j < kConvVec; ++j) {
        bj[j] = bias ? bias[c0 + j] : 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k][j] = w[(size_t)(c0 + j) * W + k];
    }
    const T *xb = x + (size_t)b * L * D + c0;
    T *ob = out + (size_t)b * L * D + c0;
    // h[k] = x_{t-W+1+k} for the current token t (h[W-1] is the newest)
    float h[W][kConvVec];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int t = t0 - (W - 1) + k;
        if (t >= 0) {
            load8(xb + (size_t)t * D, h[k + 1]);
        } else {
#pragma unroll
            for (int j = 0; j < kConvVec; ++j) h[k + 1][j] = 0.f;
        }
    }
    const int t1 = min(t0 + kConvRun, L);
    for (int t = t0; t < t1; t += kConvBatch) {
        // (loads from a clamped token, so that all of them issue before any
        // use; the stores are predicated)
        float xv[kConvBatch][kConvVec];
#pragma unroll
        for (int u = 0; u < kConvBatch; ++u) load8(xb + (size_t)min(t + u, L - 1) * D, xv[u]);
#pragma unroll
        for (int u = 0; u < kConvBatch; ++u) {
            if (t + u < t1) {
#pragma unroll
                for (int k = 0; k < W - 1; ++k)
#pragma unroll
                    for (int j = 0; j < kConvVec; ++j) h[k][j] = h[k + 1][j];
#pragma unroll
                for (int j = 0; j < kConvVec; ++j) h[W - 1][j] = xv[u][j];
                float o[kConvVec];
#pragma unroll
                for (int j = 0; j < kConvVec; ++j) {
                    float a = bj[j];
#pragma unroll
                    for (int k = 0; k < W; ++k) a += wk[k][j] * h[k][j];
                    o[j] = act_silu ? silu(a) : a;
                }
                store8(ob + (size_t)(t + u) * D, o);
            }
        }
    }
    // the cache after the sequence, [b][D][W]: x_{L-W} .. x_{L-1} (zeros
    // before the start), from the run that holds the last token
    if (state_out && t1 == L && t0 < L) {
        T *sp = state_out + ((size_t)b * D + c0) * W;
#pragma unroll
        for (int j = 0; j < kConvVec; ++j)
#pragma unroll
            for (int k = 0; k < W; ++k) sp[j * W + k] = from_f32<T>(h[k][j]);
    }
}

// grid (ceil(D / 256), batch), 256 threads: one channel per thread.
template <typename T, int W>
__global__ void __launch_bounds__(256)
k_conv1d_update(T *__restrict__ state, const T *__restrict__ x, const float *__restrict__ w,
                const float *__restrict__ bias, T *__restrict__ out, int D, int act_silu) {
    const int c = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
    if (c >= D) return;
    T *sp = state + ((size_t)b * D + c) * W;
    float v[W];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) v[k] = to_f32(sp[k + 1]);
    v[W - 1] = to_f32(x[(size_t)b * D + c]);
    float a = bias ? bias[c] : 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k) a += w[(size_t)c * W + k] * v[k];
#pragma unroll
    for (int k = 0; k < W; ++k) sp[k] = from_f32<T>(v[k]);
    out[(size_t)b * D + c] = from_f32<T>(act_silu ? silu(a) : a);
}

template <typename T>
hipError_t launch_conv1d_fwd(const ConvArgs &a, hipStream_t stream) {
    // the fewest workgroups of at most 256 threads over a row's 8-channel
    // groups, sized alike (in multiples of 32): 5376 channels take three of
    // 224 threads rather than three of 256 with 96 idle (2% shorter, A/B)
    const int nvec = a.D / kConvVec, nblk = (nvec + 255) / 256;
    const int nthr = ((nvec + nblk - 1) / nblk + 31) / 32 * 32;
    const dim3 grid((nvec + nthr - 1) / nthr, (a.L + kConvRun - 1) / kConvRun, a.batch);
#define SSD_CONV_CASE(WW)                                                                    \
    case WW:                                                                                 \
        hipLaunchKernelGGL((k_conv1d_fwd<T, WW>), grid, dim3(nthr), 0, stream,              \
                           (const T *)a.x, a.w, a.bias, (T *)a.out, (T *)a.state, a.L, a.D, \
                           a.silu);                                                          \
        break;
    switch (a.W) {
        SSD_CONV_CASE(2)
        SSD_CONV_CASE(3)
        SSD_CONV_CASE(4)
        default: return hipErrorInvalidValue;
    }
#undef SSD_CONV_CASE
    return hipGetLastError();
}

template <typename T>
hipError_t launch_conv1d_update(const ConvArgs &a, hipStream_t stream) {
    const dim3 grid((a.D + 255) / 256, a.batch);
#define SSD_CONV_CASE(WW)                                                                    \
    case WW:                                                                                 \
        hipLaunchKernelGGL((k_conv1d_update<T, WW>), grid, dim3(256), 0, stream, (T *)a.state, \
                           (const T *)a.x, a.w, a.bias, (T *)a.out, a.D, a.silu);           \
        break;
    switch (a.W) {
        SSD_CONV_CASE(2)
        SSD_CONV_CASE(3)
        SSD_CONV_CASE(4)
        default: return hipErrorInvalidValue;
    }
#undef SSD_CONV_CASE
    return hipGetLastError();
}

template hipError_t launch_conv1d_fwd<float>(const ConvArgs &, hipStream_t);
template hipError_t launch_conv1d_fwd<bf16>(const ConvArgs &, hipStream_t);
template hipError_t launch_conv1d_update<float>(const ConvArgs &, hipStream_t);
template hipError_t launch_conv1d_update<bf16>(const ConvArgs &, hipStream_t);

}  // namespace ssd
