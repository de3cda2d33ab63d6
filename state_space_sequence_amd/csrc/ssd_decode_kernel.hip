// ssd_decode_kernel.hip -- single-token SSM state update, in place.
//
// One token of the recurrence (fla `layers/mamba2.py`, decode branch of
// `Mamba2.torch_forward`): decay the cached state by exp(dt*A), add
// dt * x (outer) B, then read y = state . C + D x from the UPDATED state.
//
// The step moves 2 * P * N * 4 bytes of fp32 state per (batch, head) and does
// ~5 flops per state element, so it is bound by HBM bandwidth.  A block owns
// one (batch, head); each row p of the state is read and written as float4
// vectors by a group of R lanes (R = the power of two >= N/4, at least 4),
// so a wave streams 64 / R whole rows per access with fully coalesced
// 16-byte lanes.
// The row's dot product with C is reduced with xor shuffles inside the group.
// The state is touched once per step, so its loads and stores carry the
// non-temporal hint (measured: 10% shorter on the 256-batch, 80-head step).
// Optionally D is per (head, headdim column) and the output is gated,
// y = (state . C + D x) silu(z) (the `D` and `z` arguments of the layer's
// `selective_state_update` call; the lrnnx scan's final output step).
#include "ssd_device.hpp"
#include "ssd_kernels.hpp"

namespace ssd {

// Each thread first issues the loads of U rows (U = 8 passes of the
// workgroup over the rows), then updates and stores them, so that every lane
// keeps U 16-byte state loads in flight instead of one.
template <typename T, int R>
__global__ void __launch_bounds__(256)
k_state_update(float *__restrict__ state, const T *__restrict__ x, const float *__restrict__ dt,
               const float *__restrict__ A, const T *__restrict__ Bm, const T *__restrict__ Cm,
               const float *__restrict__ D, T *__restrict__ y, int H, int G, int P, int N,
               const DtProc dtp, const T *__restrict__ z, int D_hdim) {
    constexpr int RP = 256 / R;  // rows per pass of the workgroup
    constexpr int U = 8;         // passes whose loads are in flight together
    const int h = blockIdx.x, b = blockIdx.y, g = h / (H / G);
    const int tid = threadIdx.x;
    const int lr = tid & (R - 1);
    const int n0 = lr * 4;
    const bool nact = n0 < N;
    float dth = dt[(size_t)b * H + h];
    if (dtp.on) dth = dt_process(dth, dtp.bias ? dtp.bias[h] : 0.f, dtp.softplus, dtp.lo, dtp.hi);
    const float alpha = fast_exp(dth * A[h]);
    const float Dh = D ? D[h] : 0.f;
    float Bv[4] = {0.f, 0.f, 0.f, 0.f}, Cv[4] = {0.f, 0.f, 0.f, 0.f};
    if (nact) {
        const T *bp = Bm + ((size_t)b * G + g) * N + n0;
        const T *cp = Cm + ((size_t)b * G + g) * N + n0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Bv[j] = to_f32(bp[j]);
            Cv[j] = to_f32(cp[j]);
        }
    }
    const size_t base = (size_t)(b * H + h) * P;
    for (int p0 = tid / R; p0 < P; p0 += U * RP) {
        f32x4 sv[U];
        float xv[U];
        // (unconditional loads, from a clamped row and column where the lane
        // has none, so that the compiler issues them all before any wait;
        // the stores below are predicated)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = min(p0 + u * RP, P - 1);
            xv[u] = to_f32(x[base + p]);
            sv[u] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(state + (base + p) * N + min(n0, N - 4)));
        }
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * RP;
            const float uu = dth * xv[u];
            f32x4 s4 = sv[u];
#pragma unroll
            for (int j = 0; j < 4; ++j) s4[j] = alpha * s4[j] + uu * Bv[j];
            if (p < P && nact)
                __builtin_nontemporal_store(s4, reinterpret_cast<f32x4 *>(state + (base + p) * N + n0));
            part[u] = nact ? s4[0] * Cv[0] + s4[1] * Cv[1] + s4[2] * Cv[2] + s4[3] * Cv[3] : 0.f;
        }
#pragma unroll
        for (int off = R / 2; off > 0; off >>= 1)
#pragma unroll
            for (int u = 0; u < U; ++u) part[u] += __shfl_xor(part[u], off, kWave);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * RP;
            if (lr == 0 && p < P) {
                const float dp = D_hdim && D ? D[(size_t)h * P + p] : Dh;
                float o = part[u] + dp * xv[u];
                if (z) o *= silu_f32(to_f32(z[base + p]));
                y[base + p] = from_f32<T>(o);
            }
        }
    }
}

template <typename T>
hipError_t launch_state_update(const DecodeArgs &a, hipStream_t stream) {
    // lanes per state row: the power of two >= N / 4 (N is a multiple of 16
    // and at most kMaxDstate, so R is 4 .. 64)
    int R = 4;
    while (R * 4 < a.N) R <<= 1;
    const dim3 grid(a.H, a.batch), block(256);
#define SSD_DECODE_CASE(RR)                                                                    \
    case RR:                                                                                   \
        hipLaunchKernelGGL((k_state_update<T, RR>), grid, block, 0, stream, a.state,          \
                           (const T *)a.x, a.dt, a.A, (const T *)a.B, (const T *)a.C, a.D,    \
                           (T *)a.y, a.H, a.G, a.P, a.N, a.dtp, (const T *)a.z,               \
                           a.D_hdim ? 1 : 0);                                                  \
        break;
    switch (R) {
        SSD_DECODE_CASE(4)
        SSD_DECODE_CASE(8)
        SSD_DECODE_CASE(16)
        SSD_DECODE_CASE(32)
        SSD_DECODE_CASE(64)
        default: return hipErrorInvalidValue;
    }
#undef SSD_DECODE_CASE
    return hipGetLastError();
}

template hipError_t launch_state_update<float>(const DecodeArgs &, hipStream_t);
template hipError_t launch_state_update<bf16>(const DecodeArgs &, hipStream_t);

}  // namespace ssd
