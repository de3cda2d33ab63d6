// ssd_backward.hpp -- internal interface of the gradient pass of the chunked
// forward (ssd_chunk_scan_bwd): its arguments and workspace, and the launch
// functions it shares with the split forward.  Not installed; the public ABI
// is include/ssd.h.
#pragma once

#include "ssd_kernels.hpp"

namespace ssd {

// One gradient call.  `f` holds the forward's inputs, shapes and the
// workspace regions of the split forward (prefix sums, C B^T, chunk states),
// which the pass recomputes (f.final_state is not needed: null).
struct BackwardArgs {
    ForwardArgs f;
    const void *dy;        // [b][L][H][P] io type
    const float *dfinal;   // [b][H][P][N], or null (0)
    void *dx;              // [b][L][H][P] io type
    float *ddt;            // [b][L][H]
    float *dA;             // [H]
    void *dB, *dC;         // [b][L][G][N] io type
    float *dD;             // [H], or null
    float *dinit;          // [b][H][P][N], or null
    // workspace
    float *adj;     // [b][nc][H][P][N]: G_c, then the gradient with respect
                    // to the state at the end of chunk c
    double *qpart;  // [b][nc][H][nsl]: partial sums of <that gradient, h_in[c]>
    float *roff;    // [b][H][nc][Q]: <dy_t, e^(acum_t) h_in C_t> per head
    float *dint;    // [b][H][nc][Q]: x_t . (e^(acum_end - acum_t) Lam B_t)
    float *dd;      // [b][H][nc][Q]: x_t . u_t (the direct part of ddt)
    void *wsm;      // [b][nc][G][Q][Q] io type: the group's summed score tiles Ws
    float *wpart;   // [nhg][b][nc][G][Q][Q]: per head group partial Ws (nhg > 1)
    double *rowp;   // [b][H][nc][nrb][Q]: strict row sums of W per (row block's) tile
    double *colp;   // [b][H][nc][nrb][Q]: strict column sums of W per (column block's) tile
    float *dDpart;  // [b][nc][H][nrb]: partial sums of dy . x
    double *dApart; // [b][nc][H]: partial sums of dt * dLoss/d(dt A)
    float *partB, *partC; // [nhg][b][L][G][N]: per head group dB / dC (nhg > 1)
    // with f.side: recorded on the call's stream once the recomputed states
    // are queued (the side stream's dC waits for it)
    hipEvent_t ev_states = nullptr;
};

// Slices of a state (4 elements per thread, 256 threads) in the reverse
// state pass.
inline int bwd_state_slices(int P, int N) { return (P * N + 1023) / 1024; }
// Row blocks of a chunk in the gradient kernels (64 rows, or the chunk).
inline int bwd_row_blocks(int Q) { return Q > 64 ? Q / 64 : 1; }

// Heads per workgroup of the dB and dC kernels, which sum over a group's
// heads: enough head groups for about 2048 workgroups (then each group's
// fp32 partial sum is added up by a separate pass).
inline int bwd_heads_per_group(int batch, int nc, int nrb, int G, int hpg) {
    const long wg = (long)batch * nc * nrb * G;
    long ng = (2048 + wg - 1) / wg;
    if (ng > hpg) ng = hpg;
    if (ng < 1) ng = 1;
    return (int)((hpg + ng - 1) / ng);
}
// Heads per workgroup of the summed-score kernel: enough head groups for
// about 2048 workgroups (each group's fp32 partial tiles are added up by a
// separate pass).
inline int bwd_wsum_heads(int ntile, int nc, int G, int batch, int hpg) {
    const long wg = (long)ntile * nc * G * batch;
    long ng = (2048 + wg - 1) / wg;
    if (ng > hpg) ng = hpg;
    if (ng < 1) ng = 1;
    return (int)((hpg + ng - 1) / ng);
}
inline int bwd_head_groups(int batch, int nc, int nrb, int G, int hpg) {
    const int hpw = bwd_heads_per_group(batch, nc, nrb, G, hpg);
    return (hpg + hpw - 1) / hpw;
}

constexpr int kBackwardKernels = 9;
extern const char *const kBackwardKernelNames[kBackwardKernels];

// The first four kernels of the split forward (k1 .. k4; `cb_done`, if not
// null, recorded on `stream` once k1 and k2 are queued), and k3 in its
// gradient form (G_c = sum_s dy_s exp(acum_s) C_s^T into `out`).
template <typename T>
hipError_t launch_split_states(const ForwardArgs &a, hipStream_t stream, hipEvent_t cb_done = nullptr);
template <typename T>
hipError_t launch_adj_chunk_states(const ForwardArgs &a, const void *dy, float *out,
                                   hipStream_t stream);

// The whole gradient pass.  When `events` is non-null, events[i] is recorded
// right before kernel i and events[kBackwardKernels] after the last.
template <typename T>
hipError_t launch_backward(const BackwardArgs &a, hipStream_t stream,
                           hipEvent_t *events = nullptr);

}  // namespace ssd
