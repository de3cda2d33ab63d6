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

// Time-step preprocessing of the `_ex` entry points: when `on`, the kernels
// use min(max(f(dt + bias_h), lo), hi) with f = softplus if `softplus`,
// else the identity (bias may be null: 0).  Tokens past seqlen keep dt = 0.
struct DtProc {
    bool on = false;
    const float *bias = nullptr;
    bool softplus = false;
    float lo = 0.f, hi = 0.f;
};

// Problem and workspace pointers of one chunked forward call.
struct ForwardArgs {
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
    DtProc dtp;      // dt preprocessing (off: dt is used as given)
    const int *seq_idx = nullptr;  // packed sequences [b][L], or null
    const void *z = nullptr;       // output gate [b][L][H][P] (x's type), or null
    bool D_hdim = false;           // D is [H][P] (else [H])
    // workspace regions shared by both forward paths
    float *acum_hi;  // [b][H][nc][Q]  fp32 part of the fp64 chunk prefix sums
    float *acum_lo;  // [b][H][nc][Q]  remainder: prefix = hi + lo
    float *dtT;      // [b][H][nc][Q]  dt per chunk, 0 past seqlen
    void *cb;        // split path: C B^T per chunk and group, fp32 [b][nc][G][Q][Q]
    float *S;        // split path: chunk states [b][nc][H][P][N]
    int *segst;      // split path, packed sequences: last start per token [b][nc][Q]
    // fused path, segmented sequence (nseg > 1): the states segments
    // 0 .. nseg - 2 leave [nseg - 1][b][H][P][N] (segment 0's from the
    // initial state, the others' from zero) and their log decays
    // [nseg - 1][b][H]
    int nseg = 1;
    float *seg_buf = nullptr;
    float *seg_logdec = nullptr;
    // an auxiliary stream and two events on which the segmented forward
    // overlaps its first phase (null: the phases run on the caller's stream)
    hipStream_t side = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
                     // (acum_hi / acum_lo / dtT unused there)
};

// Fused path: the decay record of one (batch, head, 32-token block), as the
// fused kernel keeps it in LDS, floats: [0, 32) the x' weights
// exp(lambda_e - lambda_s) dt_s / sigma_out, [32, 64) the output factors
// exp(lambda_l - lambda_e) sigma_out (0 when the block is not factored),
// [64, 96) lambda_l - lambda_e, [96, 128) dt_l, then delta = exp(lambda_e),
// the factored flag (1 or 0), lambda_e, sigma_in, sigma_out and the restart
// flag (sigma the scale of the state, h = sigma h~), 2 floats of padding,
// then [136, 168) the start of each token's packed sequence within the block
// (-1: none).  In a block that takes the exact path, [32, 64) holds the
// state-in factor exp(lambda_l) instead (0 past a sequence start).  672
// bytes, a multiple of 16.
constexpr int kVecRec = 168;

// Forward paths.  The split path runs the five kernels of the chunked
// algorithm one after the other with the caller's chunk length and accepts
// every supported shape; the fused path (bf16, dstate 128, headdim a
// multiple of 32) runs one pass over the sequence per (batch, head, headdim
// block) in 32-token blocks with the state in registers.
enum class Path { Split, Fused };

constexpr int kSplitKernels = 5;
constexpr int kFusedKernels = 1;
constexpr int kMaxForwardKernels = 5;
extern const char *const kSplitKernelNames[kSplitKernels];
extern const char *const kFusedKernelNames[kFusedKernels];

// Enqueue a forward.  When `events` is non-null, events[i] is recorded on
// `stream` right before kernel i and events[nkernels] after the last.
template <typename T>
hipError_t launch_split_forward(const ForwardArgs &a, hipStream_t stream,
                                hipEvent_t *events = nullptr);
template <typename T>
hipError_t launch_fused_forward(const ForwardArgs &a, hipStream_t stream,
                                hipEvent_t *events = nullptr);
template <typename T> bool fused_supported(int P, int N, int Q);
// The number of 32-token blocks of the fused path for L tokens.
int fused_nblk(int L);
// log2 of the blocks per rebasing window of the fused loader's resources,
// and whether a row of `row_bytes` (the widest stream) leaves a window of
// at least 8 blocks.
int fused_window_shift(const ForwardArgs &a);
// Sequence segments of the fused forward for a shape (1: one pass), the
// kernels it launches, and their names when segmented.
int fused_segments(int batch, int L, int H, int G, int P);
// The segments of a segmented forward, as a kernel argument: segment 0 has
// `first` blocks, every later one `len` (the last the rest); a launch runs
// segments base .. base + gridDim.z - 1 of nseg.
struct SegPlan {
    int first, len, base, nseg;
};
int fused_kernel_count(int nseg);
extern const char *const kFusedSegKernelNames[2];
bool fused_row_fits(size_t row_bytes);

// k1 of the split path.
void launch_dA_cumsum(const float *dt, const DtProc &dtp, const float *A, float *acum_hi,
                      float *acum_lo, float *dtT, int batch, int L, int H, int nc, int Q,
                      hipStream_t stream, const int *seq_idx = nullptr, int *segst = nullptr);

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
    DtProc dtp;      // dt preprocessing (off: dt is used as given)
    const void *z = nullptr;  // output gate [b][H][P] (x's type), or null
    bool D_hdim = false;      // D is [H][P] (else [H])
};

template <typename T>
hipError_t launch_state_update(const DecodeArgs &a, hipStream_t stream);

// The causal depthwise convolution before the scan (ssd_conv_kernels.hip):
// x, out [batch][L][D] (forward) or [batch][D] (update); w [D][W] and bias
// [D] fp32; state the cache [batch][D][W] (forward: written when non-null;
// update: in and out).
struct ConvArgs {
    const void *x;
    const float *w;
    const float *bias;  // may be null
    void *out;
    void *state;        // forward: may be null
    int batch, L, D, W, silu;
};

template <typename T>
hipError_t launch_conv1d_fwd(const ConvArgs &a, hipStream_t stream);
template <typename T>
hipError_t launch_conv1d_update(const ConvArgs &a, hipStream_t stream);

// The gated RMS normalisation after the scan (ssd_norm_kernels.hip): y, z,
// out [rows][dim]; w [dim] fp32; gate 0 none, 1 before the normalisation
// (the layer's), 2 after it.
struct NormArgs {
    const void *y;
    const void *z;  // may be null when gate == 0
    const float *w;
    void *out;
    int rows, dim, gate;
    float eps;
};
constexpr int kMaxNormDim = 8192;

template <typename T>
hipError_t launch_gated_rmsnorm(const NormArgs &a, hipStream_t stream);

// The opt-in non-finite check (ssd_check_kernels.hip): clear the device's
// flag word, scan a buffer of `nelems` fp32 (elem_bytes 4) or bf16 (2)
// values OR-ing `bit` into the flag when one is a NaN or an infinity, and
// read the flag back (synchronises `stream`).
constexpr unsigned kNonfiniteInput = 1u, kNonfiniteOutput = 2u;
// Fills `bytes` of device memory with quiet-NaN words (the workspace
// poison of the SSD_POISON_WORKSPACE debug mode).
hipError_t launch_poison(void *p, size_t bytes, hipStream_t stream);
hipError_t launch_nonfinite_reset(hipStream_t stream);
hipError_t launch_nonfinite_scan(const void *p, size_t nelems, int elem_bytes, unsigned bit,
                                 hipStream_t stream);
hipError_t read_nonfinite(unsigned *out, hipStream_t stream);

}  // namespace ssd
