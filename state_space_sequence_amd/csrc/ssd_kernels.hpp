// ssd_kernels.hpp -- internal interface between the C ABI (ssd_api.hip) and
// the kernel files.  Not installed; the public ABI is include/ssd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ssd {

constexpr int kMaxHeaddim = 128;
constexpr int kMaxDstate = 256;
constexpr int kK3TilesPerWave = 8;
constexpr int kK4Prefetch = 4;

// Problem and workspace pointers of one chunked forward call.
struct SplitArgs {
    const void *x;
    const float *dt;
    const float *A;
    const void *B;
    const void *C;
    const float *D;      // may be null
    const float *init;   // may be null
    void *y;
    float *final_state;  // may be null
    int batch, L, H, G, P, N, Q, nchunks;
    // workspace regions
    float *acum_hi;  // [b][H][nc][Q]  fp32 part of the fp64 chunk prefix sums
    float *acum_lo;  // [b][H][nc][Q]  remainder: prefix = hi + lo
    float *dtT;      // [b][H][nc][Q]
    float *cb;    // [b][nc][G][Q][Q]
    float *S;     // [b][nc][H][P][N]
};

// Kernels of one forward call, in launch order.
constexpr int kForwardKernels = 5;
extern const char *const kForwardKernelNames[kForwardKernels];

// Enqueue the forward.  When `events` is non-null, events[i] is recorded on
// `stream` right before kernel i and events[kForwardKernels] after the last.
template <typename T>
hipError_t launch_split_forward(const SplitArgs &a, hipStream_t stream,
                                hipEvent_t *events = nullptr);

struct DecodeArgs {
    float *state;
    const void *x;
    const float *dt;
    const float *A;
    const void *B;
    const void *C;
    const float *D;  // may be null
    void *y;
    int batch, H, G, P, N;
};

template <typename T>
hipError_t launch_state_update(const DecodeArgs &a, hipStream_t stream);

}  // namespace ssd
