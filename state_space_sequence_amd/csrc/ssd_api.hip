// ssd_api.hip -- the extern "C" entry points declared in include/ssd.h:
// argument validation, forward-path choice, workspace layout and kernel
// dispatch.  Validation is plain host code that runs before anything is
// enqueued.
#include "ssd.h"

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "ssd_device.hpp"
#include "ssd_kernels.hpp"
#include "ssd_backward.hpp"

// Scratch of the no-allocation forward (ssd_chunk_scan_fwd_noalloc): every
// GPU that the library runs on holds one copy of this array until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: the device address of the current GPU's copy comes from
// hipGetSymbolAddress (scratch_address below) and only that address is
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

// The device address of `scratch` on the device that runs `stream` (the
// current device for the null stream), looked up once per device with that
// device current and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(hipStream_t stream, void **out) {
    int cur = 0, dev = 0;
    hipError_t err = hipGetDevice(&cur);
    if (err != hipSuccess) return err;
    dev = cur;
    if (stream && (err = hipStreamGetDevice(stream, &dev)) != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (err = hipSetDevice(dev)) != hipSuccess) return err;
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (err == hipSuccess) err = back;
        }
        if (err != hipSuccess) return err;
        if (!p || (uintptr_t)p % kAlign != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// The auxiliary stream and fork/join events on which a segmented fused
// forward overlaps its first phase and the gradient pass two of its kernels
// (a third event marks the recomputed states): one set per device, created
// with that device current at the first call that uses it and kept until
// the process ends (default priority; non-blocking with respect to the null
// stream).
// The mutex is held across each call's fork ... join sequence, so that
// concurrent calls never re-record an event between another call's record
// and its wait.
struct Side {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr, mid = nullptr;
};
std::mutex g_side_mu;
Side g_side[kMaxDevices];

hipError_t side_for(hipStream_t stream, Side *out) {
    int cur = 0, dev = 0;
    hipError_t err = hipGetDevice(&cur);
    if (err != hipSuccess) return err;
    dev = cur;
    if (stream && (err = hipStreamGetDevice(stream, &dev)) != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    Side &sd = g_side[dev];
    if (!sd.stream) {
        if (dev != cur && (err = hipSetDevice(dev)) != hipSuccess) return err;
        Side n;
        err = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking);
        if (err == hipSuccess) err = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
        if (err == hipSuccess) err = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
        if (err == hipSuccess) err = hipEventCreateWithFlags(&n.mid, hipEventDisableTiming);
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (err == hipSuccess) err = back;
        }
        if (err != hipSuccess) return err;
        sd = n;
    }
    *out = sd;
    return hipSuccess;
}

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool is_pow2_chunk(int q) {
    return q == 16 || q == 32 || q == 64 || q == 128 || q == 256;
}

// Checks shared by the workspace query and the forward call.
ssd_status check_forward_shape(int batch, int seqlen, int nheads, int headdim,
                               int dstate, int ngroups, int chunk_len,
                               ssd_dtype io_dtype) {
    if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 ||
        ngroups <= 0 || chunk_len <= 0)
        return SSD_ERR_INVALID_ARGUMENT;
    if (nheads % ngroups != 0) return SSD_ERR_INVALID_ARGUMENT;
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
    if (!is_pow2_chunk(chunk_len)) return SSD_ERR_UNSUPPORTED;
    if (headdim % 16 != 0 || headdim > ssd::kMaxHeaddim) return SSD_ERR_UNSUPPORTED;
    if (dstate % 16 != 0 || dstate > ssd::kMaxDstate) return SSD_ERR_UNSUPPORTED;
    // Every element index must fit the 32-bit block/grid arithmetic used for
    // per-(b,h) bases and the 64-bit offsets used for whole tensors.
    const double elems = (double)batch * seqlen * nheads * headdim;
    const double states = (double)batch * ((seqlen + chunk_len - 1) / chunk_len + 1) *
                          nheads * headdim * dstate;
    if (elems > 9.0e15 || states > 9.0e15 || (double)batch * nheads > 2.0e9)
        return SSD_ERR_UNSUPPORTED;
    // Launch grids put the batch, and (chunks x groups) / (heads x tile
    // groups), on the y and z grid dimensions, which are limited to 65535.
    const long nc = (seqlen + chunk_len - 1) / chunk_len;
    if (batch > 65535 || nc * ngroups > 65535 || (long)nheads * 4 > 65535)
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// The time-step preprocessing options of the `_ex` entry points (NULL: off).
ssd_status check_dt_proc(const ssd_dt_proc *p, ssd::DtProc *out) {
    *out = ssd::DtProc();
    if (!p) return SSD_OK;
    // (a NaN bound fails every comparison below)
    if (!(p->dt_min >= 0.f) || !(p->dt_max >= p->dt_min)) return SSD_ERR_INVALID_ARGUMENT;
    if (p->dt_bias && !aligned(p->dt_bias, 4)) return SSD_ERR_INVALID_ARGUMENT;
    out->on = true;
    out->bias = p->dt_bias;
    out->softplus = p->dt_softplus != 0;
    out->lo = p->dt_min;
    out->hi = p->dt_max;
    return SSD_OK;
}

// Forward path for a shape: the fused kernel where it applies, the split
// kernels otherwise.  SSD_FORWARD_PATH=split|fused overrides the choice (a
// diagnostic switch for comparing the two); forcing "fused" on a shape it
// does not cover is reported as unsupported.
ssd_status choose_path(int /*seqlen*/, int nheads, int ngroups, int headdim, int dstate,
                       int chunk_len, ssd_dtype io, ssd::Path *out) {
    // the fused kernel addresses a batch row with 32-bit offsets from
    // resources rebased every window of blocks: any length fits as long as a
    // window holds a few blocks of the widest stream
    size_t row = (size_t)nheads * headdim > (size_t)ngroups * dstate
                     ? (size_t)nheads * headdim
                     : (size_t)ngroups * dstate;
    row *= 2;
    if ((size_t)nheads * 4 > row) row = (size_t)nheads * 4;
    const bool fits = ssd::fused_row_fits(row);
    const bool fused_ok = fits && (io == SSD_BF16
                              ? ssd::fused_supported<ssd::bf16>(headdim, dstate, chunk_len)
                              : ssd::fused_supported<float>(headdim, dstate, chunk_len));
    const char *env = getenv("SSD_FORWARD_PATH");
    if (env && strcmp(env, "split") == 0) {
        *out = ssd::Path::Split;
    } else if (env && strcmp(env, "fused") == 0) {
        if (!fused_ok) return SSD_ERR_UNSUPPORTED;
        *out = ssd::Path::Fused;
    } else {
        *out = fused_ok ? ssd::Path::Fused : ssd::Path::Split;
    }
    return SSD_OK;
}

// The opt-in non-finite check: SSD_CHECK_FINITE set to anything but "" or
// "0".  Read on every call, like SSD_FORWARD_PATH.
bool poison_requested() {
    const char *e = getenv("SSD_POISON_WORKSPACE");
    return e && e[0] && strcmp(e, "0") != 0;
}

bool finite_check_requested() {
    const char *e = getenv("SSD_CHECK_FINITE");
    return e && e[0] && strcmp(e, "0") != 0;
}

// One call's non-finite check: created once the arguments are validated
// (a rejected call launches nothing), it clears the device flag, scans the
// buffers it is shown, and turns the flag into the call's status.  Off, it
// does nothing.
class FiniteCheck {
  public:
    explicit FiniteCheck(hipStream_t s) : s_(s), on_(finite_check_requested()) {
        if (on_) err_ = ssd::launch_nonfinite_reset(s_);
    }
    void input(const void *p, size_t n, int es) { scan(p, n, es, ssd::kNonfiniteInput); }
    void output(const void *p, size_t n, int es) { scan(p, n, es, ssd::kNonfiniteOutput); }
    // `st`, the status of the call's own launches, unless a check launch
    // failed or a value was not finite (reads the flag back: synchronises)
    ssd_status finish(ssd_status st) {
        if (!on_ || st != SSD_OK) return st;
        if (err_ != hipSuccess) return SSD_ERR_HIP;
        unsigned flag = 0;
        if (ssd::read_nonfinite(&flag, s_) != hipSuccess) return SSD_ERR_HIP;
        return flag ? SSD_ERR_NONFINITE : SSD_OK;
    }

  private:
    void scan(const void *p, size_t n, int es, unsigned bit) {
        if (on_ && err_ == hipSuccess) err_ = ssd::launch_nonfinite_scan(p, n, es, bit, s_);
    }
    hipStream_t s_;
    bool on_;
    hipError_t err_ = hipSuccess;
};

struct Layout {
    size_t acum_hi, acum_lo, dtT, cb, S, segst, total;
    int nseg = 1;            // fused path: sequence segments
    size_t seg_buf = 0, seg_logdec = 0;
};

Layout forward_layout(int batch, int seqlen, int nheads, int headdim, int dstate,
                      int ngroups, int chunk_len, ssd_dtype io, ssd::Path path) {
    const size_t b = batch, H = nheads, P = headdim, N = dstate, G = ngroups;
    (void)io;
    Layout l;
    if (path == ssd::Path::Split) {
        const size_t Q = chunk_len;
        const size_t nc = ((size_t)seqlen + Q - 1) / Q;
        const size_t vec = round_up(b * H * nc * Q * sizeof(float));
        l.acum_hi = 0;
        l.acum_lo = l.acum_hi + vec;
        l.dtT = l.acum_lo + vec;
        l.cb = l.dtT + vec;
        l.S = l.cb + round_up(b * nc * G * Q * Q * sizeof(float));
        // (the packed-sequence starts: always reserved, so the size does
        // not depend on whether a call passes seq_idx)
        l.segst = l.S + round_up(b * nc * H * P * N * sizeof(float));
        l.total = l.segst + round_up(b * nc * Q * sizeof(int));
    } else {
        // the fused kernel keeps every intermediate on chip; a segmented
        // sequence needs the states segments 0 .. nseg - 2 leave and their
        // log decays
        l.acum_hi = l.acum_lo = l.dtT = l.cb = l.S = l.segst = 0;
        l.nseg = ssd::fused_segments(batch, seqlen, nheads, ngroups, headdim);
        const size_t ns = (size_t)(l.nseg - 1);
        l.seg_buf = 0;
        l.seg_logdec = round_up(ns * b * H * P * N * sizeof(float));
        l.total = l.nseg > 1 ? l.seg_logdec + round_up(ns * b * H * sizeof(float)) : 0;
    }
    return l;
}

ssd_status forward_impl(const void *x, const float *dt, const float *A, const void *B,
                        const void *C, const float *D, const float *initial_state,
                        int chunk_len, int ngroups, int batch, int seqlen, int nheads,
                        int headdim, int dstate, ssd_dtype io_dtype, void *y,
                        float *final_state, void *workspace, size_t workspace_bytes,
                        hipStream_t stream, hipEvent_t *events, int *nkernels,
                        const char **names, const ssd_dt_proc *dt_proc,
                        const int *seq_idx = nullptr, bool noalloc = false,
                        const ssd_gate *gate = nullptr) {
    ssd_status st = check_forward_shape(batch, seqlen, nheads, headdim, dstate, ngroups,
                                        chunk_len, io_dtype);
    if (st != SSD_OK) return st;
    ssd::DtProc dtp;
    if ((st = check_dt_proc(dt_proc, &dtp)) != SSD_OK) return st;
    if (!x || !dt || !A || !B || !C || !y) return SSD_ERR_INVALID_ARGUMENT;
    // 16-byte vector accesses on x, B, C, y and the states.
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(dt, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
        (initial_state && !aligned(initial_state, 16)) ||
        (final_state && !aligned(final_state, 16)))
        return SSD_ERR_INVALID_ARGUMENT;
    const void *z = gate ? gate->z : nullptr;
    const bool D_hdim = gate && gate->D_per_channel && D;
    if (z && !aligned(z, 16)) return SSD_ERR_INVALID_ARGUMENT;
    ssd::Path path;
    if ((st = choose_path(seqlen, nheads, ngroups, headdim, dstate, chunk_len, io_dtype, &path)) != SSD_OK) return st;
    if (seq_idx && !aligned(seq_idx, 4)) return SSD_ERR_INVALID_ARGUMENT;
    const Layout lay = forward_layout(batch, seqlen, nheads, headdim, dstate, ngroups,
                                      chunk_len, io_dtype, path);
    if (noalloc) {
        // the library's scratch array stands in for the workspace
        if (lay.total > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
        workspace = nullptr;
        workspace_bytes = 0;
        if (lay.total > 0) {
            if (scratch_address(stream, &workspace) != hipSuccess) return SSD_ERR_HIP;
            workspace_bytes = SSD_NOALLOC_SCRATCH_BYTES;
        }
    } else if (lay.total > 0 &&
               (!workspace || workspace_bytes < lay.total || !aligned(workspace, kAlign))) {
        return SSD_ERR_WORKSPACE;
    }

    ssd::ForwardArgs a;
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.init = initial_state;
    a.y = y;
    a.final_state = final_state;
    a.batch = batch;
    a.L = seqlen;
    a.H = nheads;
    a.G = ngroups;
    a.P = headdim;
    a.N = dstate;
    a.Q = chunk_len;
    a.nchunks = (seqlen + chunk_len - 1) / chunk_len;
    a.dtp = dtp;
    a.seq_idx = seq_idx;
    a.z = z;
    a.D_hdim = D_hdim;
    char *ws = static_cast<char *>(workspace);
    const bool split = path == ssd::Path::Split;
    a.acum_hi = split ? reinterpret_cast<float *>(ws + lay.acum_hi) : nullptr;
    a.acum_lo = split ? reinterpret_cast<float *>(ws + lay.acum_lo) : nullptr;
    a.dtT = split ? reinterpret_cast<float *>(ws + lay.dtT) : nullptr;
    a.cb = split ? ws + lay.cb : nullptr;
    a.S = split ? reinterpret_cast<float *>(ws + lay.S) : nullptr;
    a.segst = split ? reinterpret_cast<int *>(ws + lay.segst) : nullptr;
    a.nseg = split ? 1 : lay.nseg;
    a.seg_buf = a.nseg > 1 ? reinterpret_cast<float *>(ws + lay.seg_buf) : nullptr;
    a.seg_logdec = a.nseg > 1 ? reinterpret_cast<float *>(ws + lay.seg_logdec) : nullptr;

    const int nk = path == ssd::Path::Split ? ssd::kSplitKernels : ssd::fused_kernel_count(a.nseg);
    const char *const *kn = path == ssd::Path::Split ? ssd::kSplitKernelNames
                            : a.nseg > 1             ? ssd::kFusedSegKernelNames
                                                     : ssd::kFusedKernelNames;
    if (nkernels) *nkernels = nk;
    if (names)
        for (int i = 0; i < nk; ++i) names[i] = kn[i];

    const int es = io_dtype == SSD_BF16 ? 2 : 4;
    const size_t nx = (size_t)batch * seqlen * nheads * headdim;
    const size_t nbc = (size_t)batch * seqlen * ngroups * dstate;
    const size_t nst = (size_t)batch * nheads * headdim * dstate;
    FiniteCheck fc(stream);
    fc.input(x, nx, es);
    fc.input(dt, (size_t)batch * seqlen * nheads, 4);
    fc.input(A, nheads, 4);
    fc.input(B, nbc, es);
    fc.input(C, nbc, es);
    fc.input(D, D ? (D_hdim ? (size_t)nheads * headdim : (size_t)nheads) : 0, 4);
    fc.input(initial_state, initial_state ? nst : 0, 4);
    fc.input(dtp.bias, dtp.bias ? nheads : 0, 4);
    fc.input(z, z ? nx : 0, es);

    hipError_t err;
    // Debug mode (SSD_POISON_WORKSPACE set to anything but "" or "0"): the
    // workspace the call uses is filled with NaN first, so an intermediate
    // read before any kernel of the call wrote it shows in the outputs.
    if (lay.total > 0 && poison_requested()) {
        if (ssd::launch_poison(workspace, lay.total, stream) != hipSuccess) return SSD_ERR_HIP;
    }
    if (path == ssd::Path::Split) {
        err = io_dtype == SSD_BF16 ? ssd::launch_split_forward<ssd::bf16>(a, stream, events)
                                   : ssd::launch_split_forward<float>(a, stream, events);
    } else if (a.nseg > 2 && !noalloc) {
        // (the no-allocation entry point creates no stream: its phases run
        // one after the other)
        std::lock_guard<std::mutex> lock(g_side_mu);
        Side sd;
        if (side_for(stream, &sd) != hipSuccess) return SSD_ERR_HIP;
        a.side = sd.stream;
        a.ev_fork = sd.fork;
        a.ev_join = sd.join;
        err = io_dtype == SSD_BF16 ? ssd::launch_fused_forward<ssd::bf16>(a, stream, events)
                                   : ssd::launch_fused_forward<float>(a, stream, events);
    } else {
        err = io_dtype == SSD_BF16 ? ssd::launch_fused_forward<ssd::bf16>(a, stream, events)
                                   : ssd::launch_fused_forward<float>(a, stream, events);
    }
    if (err != hipSuccess) return SSD_ERR_HIP;
    if (events) {
        // unused trailing events are recorded too, so every handle is valid
        for (int i = nk + 1; i <= ssd::kMaxForwardKernels; ++i)
            if (hipEventRecord(events[i], stream) != hipSuccess) return SSD_ERR_HIP;
    }
    fc.output(y, nx, es);
    fc.output(final_state, final_state ? nst : 0, 4);
    return fc.finish(SSD_OK);
}

// ---------------------------------------------------------------- gradients

struct BwdLayout {
    Layout f;   // the split forward's regions, recomputed
    size_t adj, qpart, roff, dint, dd, wsm, wpart, rowp, colp, dDpart, dApart, partB, partC,
        total;
};

BwdLayout backward_layout(int batch, int seqlen, int nheads, int headdim, int dstate,
                          int ngroups, int chunk_len, ssd_dtype io) {
    BwdLayout l;
    l.f = forward_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len, io,
                         ssd::Path::Split);
    const size_t b = batch, H = nheads, P = headdim, N = dstate, Q = chunk_len;
    const size_t nc = ((size_t)seqlen + Q - 1) / Q;
    const size_t nsl = ssd::bwd_state_slices(headdim, dstate);
    const size_t nrb = ssd::bwd_row_blocks(chunk_len);
    const size_t tok = round_up(b * H * nc * Q * sizeof(float));
    size_t off = l.f.total;
    l.adj = off;
    off += round_up(b * nc * H * P * N * sizeof(float));
    l.qpart = off;
    off += round_up(b * nc * H * nsl * sizeof(double));
    l.roff = off;
    off += tok;
    l.dint = off;
    off += tok;
    l.dd = off;
    off += tok;
    l.wsm = off;
    off += round_up(b * nc * ngroups * Q * Q * (io == SSD_BF16 ? 2 : 4));
    {
        const int nt = (int)(nrb * (nrb + 1) / 2), hpg = nheads / ngroups;
        const int hpw = ssd::bwd_wsum_heads(nt, (int)nc, ngroups, batch, hpg);
        const size_t ng = (size_t)((hpg + hpw - 1) / hpw);
        l.wpart = off;
        off += ng > 1 ? round_up(ng * b * nc * ngroups * Q * Q * sizeof(float)) : 0;
    }
    l.rowp = off;
    off += round_up(b * H * nc * nrb * Q * sizeof(double));
    l.colp = off;
    off += round_up(b * H * nc * nrb * Q * sizeof(double));
    l.dDpart = off;
    off += round_up(b * nc * H * nrb * sizeof(float));
    l.dApart = off;
    off += round_up(b * nc * H * sizeof(double));
    // per head group partial dB and dC, when the groups' heads are split
    const int nhg = ssd::bwd_head_groups(batch, (int)nc, (int)nrb, ngroups, nheads / ngroups);
    const size_t part = nhg > 1 ? round_up((size_t)nhg * b * seqlen * ngroups * N * sizeof(float)) : 0;
    l.partB = off;
    off += part;
    l.partC = off;
    off += part;
    l.total = off;
    return l;
}

ssd_status backward_impl(const void *x, const float *dt, const float *A, const void *B,
                         const void *C, const float *D, const float *initial_state,
                         const void *dy, const float *dfinal, int chunk_len, int ngroups,
                         int batch, int seqlen, int nheads, int headdim, int dstate,
                         ssd_dtype io_dtype, void *dx, float *ddt, float *dA, void *dB,
                         void *dC, float *dD, float *dinit, void *workspace,
                         size_t workspace_bytes, hipStream_t stream, hipEvent_t *events,
                         int *nkernels, const char **names) {
    ssd_status st = check_forward_shape(batch, seqlen, nheads, headdim, dstate, ngroups,
                                        chunk_len, io_dtype);
    if (st != SSD_OK) return st;
    if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC)
        return SSD_ERR_INVALID_ARGUMENT;
    // (the gradient kernels put chunks x row blocks on the y grid dimension)
    if ((long)((seqlen + chunk_len - 1) / chunk_len) * ssd::bwd_row_blocks(chunk_len) > 65535)
        return SSD_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(dy, 16) ||
        !aligned(dx, 16) || !aligned(dB, 16) || !aligned(dC, 16) || !aligned(dt, 4) ||
        !aligned(A, 4) || !aligned(ddt, 4) || !aligned(dA, 4) || (D && !aligned(D, 4)) ||
        (dD && !aligned(dD, 4)) || (initial_state && !aligned(initial_state, 16)) ||
        (dfinal && !aligned(dfinal, 16)) || (dinit && !aligned(dinit, 16)))
        return SSD_ERR_INVALID_ARGUMENT;
    const BwdLayout lay = backward_layout(batch, seqlen, nheads, headdim, dstate, ngroups,
                                          chunk_len, io_dtype);
    if (!workspace || workspace_bytes < lay.total || !aligned(workspace, kAlign))
        return SSD_ERR_WORKSPACE;

    char *ws = static_cast<char *>(workspace);
    ssd::BackwardArgs a;
    ssd::ForwardArgs &f = a.f;
    f.x = x;
    f.dt = dt;
    f.A = A;
    f.B = B;
    f.C = C;
    f.D = D;
    f.init = initial_state;
    f.y = nullptr;
    f.batch = batch;
    f.L = seqlen;
    f.H = nheads;
    f.G = ngroups;
    f.P = headdim;
    f.N = dstate;
    f.Q = chunk_len;
    f.nchunks = (seqlen + chunk_len - 1) / chunk_len;
    f.acum_hi = reinterpret_cast<float *>(ws + lay.f.acum_hi);
    f.acum_lo = reinterpret_cast<float *>(ws + lay.f.acum_lo);
    f.dtT = reinterpret_cast<float *>(ws + lay.f.dtT);
    f.cb = ws + lay.f.cb;
    f.S = reinterpret_cast<float *>(ws + lay.f.S);
    f.segst = nullptr;
    f.final_state = nullptr;
    a.dy = dy;
    a.dfinal = dfinal;
    a.dx = dx;
    a.ddt = ddt;
    a.dA = dA;
    a.dB = dB;
    a.dC = dC;
    a.dD = dD;
    a.dinit = dinit;
    a.adj = reinterpret_cast<float *>(ws + lay.adj);
    a.qpart = reinterpret_cast<double *>(ws + lay.qpart);
    a.roff = reinterpret_cast<float *>(ws + lay.roff);
    a.dint = reinterpret_cast<float *>(ws + lay.dint);
    a.dd = reinterpret_cast<float *>(ws + lay.dd);
    a.wsm = ws + lay.wsm;
    a.wpart = reinterpret_cast<float *>(ws + lay.wpart);
    a.rowp = reinterpret_cast<double *>(ws + lay.rowp);
    a.colp = reinterpret_cast<double *>(ws + lay.colp);
    a.partB = reinterpret_cast<float *>(ws + lay.partB);
    a.partC = reinterpret_cast<float *>(ws + lay.partC);
    a.dDpart = reinterpret_cast<float *>(ws + lay.dDpart);
    a.dApart = reinterpret_cast<double *>(ws + lay.dApart);

    if (nkernels) *nkernels = ssd::kBackwardKernels;
    if (names)
        for (int i = 0; i < ssd::kBackwardKernels; ++i) names[i] = ssd::kBackwardKernelNames[i];

    const int es = io_dtype == SSD_BF16 ? 2 : 4;
    const size_t nx = (size_t)batch * seqlen * nheads * headdim;
    const size_t nbc = (size_t)batch * seqlen * ngroups * dstate;
    const size_t nst = (size_t)batch * nheads * headdim * dstate;
    const size_t ntok = (size_t)batch * seqlen * nheads;
    FiniteCheck fc(stream);
    fc.input(x, nx, es);
    fc.input(dt, ntok, 4);
    fc.input(A, nheads, 4);
    fc.input(B, nbc, es);
    fc.input(C, nbc, es);
    fc.input(D, D ? (size_t)nheads : 0, 4);
    fc.input(initial_state, initial_state ? nst : 0, 4);
    fc.input(dy, nx, es);
    fc.input(dfinal, dfinal ? nst : 0, 4);
    if (poison_requested()) {
        if (ssd::launch_poison(workspace, lay.total, stream) != hipSuccess) return SSD_ERR_HIP;
    }
    hipError_t err;
    if (!events) {
        // the score tiles and dC run on the device's side stream beside the
        // recompute, the adjoint products, the reverse state pass and dx
        // (the timed entry point keeps every kernel on `stream`, in order)
        std::lock_guard<std::mutex> lock(g_side_mu);
        Side sd;
        if (side_for(stream, &sd) != hipSuccess) return SSD_ERR_HIP;
        a.f.side = sd.stream;
        a.f.ev_fork = sd.fork;
        a.f.ev_join = sd.join;
        a.ev_states = sd.mid;
        err = io_dtype == SSD_BF16 ? ssd::launch_backward<ssd::bf16>(a, stream, nullptr)
                                   : ssd::launch_backward<float>(a, stream, nullptr);
    } else {
        err = io_dtype == SSD_BF16 ? ssd::launch_backward<ssd::bf16>(a, stream, events)
                                   : ssd::launch_backward<float>(a, stream, events);
    }
    if (err != hipSuccess) return SSD_ERR_HIP;
    fc.output(dx, nx, es);
    fc.output(ddt, ntok, 4);
    fc.output(dA, nheads, 4);
    fc.output(dB, nbc, es);
    fc.output(dC, nbc, es);
    fc.output(dD, dD ? (size_t)nheads : 0, 4);
    fc.output(dinit, dinit ? nst : 0, 4);
    return fc.finish(SSD_OK);
}

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char *ssd_status_string(ssd_status status) {
    switch (status) {
    case SSD_OK: return "success";
    case SSD_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported shape";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP kernel launch failed";
    case SSD_ERR_NONFINITE: return "non-finite value (NaN or infinity) in an input or output";
    }
    return "unknown status";
}

ssd_status ssd_chunk_scan_fwd_workspace_size(int batch, int seqlen, int nheads,
                                             int headdim, int dstate, int ngroups,
                                             int chunk_len, ssd_dtype io_dtype,
                                             size_t *bytes) {
    if (!bytes) return SSD_ERR_INVALID_ARGUMENT;
    ssd_status st = check_forward_shape(batch, seqlen, nheads, headdim, dstate, ngroups,
                                        chunk_len, io_dtype);
    if (st != SSD_OK) return st;
    ssd::Path path;
    if ((st = choose_path(seqlen, nheads, ngroups, headdim, dstate, chunk_len, io_dtype, &path)) != SSD_OK) return st;
    *bytes = forward_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len,
                            io_dtype, path)
                 .total;
    return SSD_OK;
}

ssd_status ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A,
                              const void *B, const void *C, const float *D,
                              const float *initial_state, int chunk_len, int ngroups,
                              int batch, int seqlen, int nheads, int headdim,
                              int dstate, ssd_dtype io_dtype, void *y,
                              float *final_state, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    return forward_impl(x, dt, A, B, C, D, initial_state, chunk_len, ngroups, batch,
                        seqlen, nheads, headdim, dstate, io_dtype, y, final_state,
                        workspace, workspace_bytes, stream, nullptr, nullptr, nullptr,
                        nullptr);
}

ssd_status ssd_chunk_scan_fwd_ex(const void *x, const float *dt, const float *A,
                                 const void *B, const void *C, const float *D,
                                 const float *initial_state, int chunk_len, int ngroups,
                                 int batch, int seqlen, int nheads, int headdim,
                                 int dstate, ssd_dtype io_dtype, void *y,
                                 float *final_state, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream,
                                 const ssd_dt_proc *dt_proc) {
    return forward_impl(x, dt, A, B, C, D, initial_state, chunk_len, ngroups, batch,
                        seqlen, nheads, headdim, dstate, io_dtype, y, final_state,
                        workspace, workspace_bytes, stream, nullptr, nullptr, nullptr,
                        dt_proc);
}

ssd_status ssd_chunk_scan_fwd_varlen(const void *x, const float *dt, const float *A,
                                     const void *B, const void *C, const float *D,
                                     const float *initial_state, int chunk_len, int ngroups,
                                     int batch, int seqlen, int nheads, int headdim,
                                     int dstate, ssd_dtype io_dtype, void *y,
                                     float *final_state, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream,
                                     const int *seq_idx, const ssd_dt_proc *dt_proc) {
    if (!seq_idx) return SSD_ERR_INVALID_ARGUMENT;
    return forward_impl(x, dt, A, B, C, D, initial_state, chunk_len, ngroups, batch,
                        seqlen, nheads, headdim, dstate, io_dtype, y, final_state,
                        workspace, workspace_bytes, stream, nullptr, nullptr, nullptr,
                        dt_proc, seq_idx);
}

ssd_status ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      const float *initial_state, int chunk_len, int ngroups,
                                      int batch, int seqlen, int nheads, int headdim,
                                      int dstate, ssd_dtype io_dtype, void *y,
                                      float *final_state, hipStream_t stream) {
    return forward_impl(x, dt, A, B, C, D, initial_state, chunk_len, ngroups, batch, seqlen,
                        nheads, headdim, dstate, io_dtype, y, final_state, nullptr, 0, stream,
                        nullptr, nullptr, nullptr, nullptr, nullptr, true);
}

ssd_status ssd_chunk_scan_fwd_full(const void *x, const float *dt, const float *A,
                                   const void *B, const void *C, const float *D,
                                   const float *initial_state, int chunk_len, int ngroups,
                                   int batch, int seqlen, int nheads, int headdim, int dstate,
                                   ssd_dtype io_dtype, void *y, float *final_state,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream,
                                   const int *seq_idx, const ssd_dt_proc *dt_proc,
                                   const ssd_gate *gate) {
    return forward_impl(x, dt, A, B, C, D, initial_state, chunk_len, ngroups, batch, seqlen,
                        nheads, headdim, dstate, io_dtype, y, final_state, workspace,
                        workspace_bytes, stream, nullptr, nullptr, nullptr, dt_proc, seq_idx,
                        false, gate);
}

int ssd_chunk_scan_fwd_max_kernels(void) { return ssd::kMaxForwardKernels; }

ssd_status ssd_chunk_scan_fwd_timed(const void *x, const float *dt, const float *A,
                                    const void *B, const void *C, const float *D,
                                    const float *initial_state, int chunk_len,
                                    int ngroups, int batch, int seqlen, int nheads,
                                    int headdim, int dstate, ssd_dtype io_dtype, void *y,
                                    float *final_state, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t *events, int nevents, int *nkernels,
                                    const char **kernel_names) {
    if (!events || nevents < ssd::kMaxForwardKernels + 1) return SSD_ERR_INVALID_ARGUMENT;
    for (int i = 0; i <= ssd::kMaxForwardKernels; ++i)
        if (!events[i]) return SSD_ERR_INVALID_ARGUMENT;
    return forward_impl(x, dt, A, B, C, D, initial_state, chunk_len, ngroups, batch,
                        seqlen, nheads, headdim, dstate, io_dtype, y, final_state,
                        workspace, workspace_bytes, stream, events, nkernels, kernel_names,
                        nullptr);
}

ssd_status ssd_state_update_full(float *state, const void *x, const float *dt,
                                 const float *A, const void *B, const void *C, const float *D,
                                 int ngroups, int batch, int nheads, int headdim, int dstate,
                                 ssd_dtype io_dtype, void *y, hipStream_t stream,
                                 const ssd_dt_proc *dt_proc, const ssd_gate *gate) {
    if (batch <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
        return SSD_ERR_INVALID_ARGUMENT;
    if (nheads % ngroups != 0) return SSD_ERR_INVALID_ARGUMENT;
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
    if (!state || !x || !dt || !A || !B || !C || !y) return SSD_ERR_INVALID_ARGUMENT;
    if (headdim % 16 != 0 || headdim > ssd::kMaxHeaddim) return SSD_ERR_UNSUPPORTED;
    if (dstate % 16 != 0 || dstate > ssd::kMaxDstate) return SSD_ERR_UNSUPPORTED;
    if (batch > 65535 || (double)batch * nheads > 2.0e9) return SSD_ERR_UNSUPPORTED;
    const size_t es = io_dtype == SSD_BF16 ? 2 : 4;
    if (!aligned(state, 16) || !aligned(x, es) || !aligned(B, es) || !aligned(C, es) ||
        !aligned(y, es) || !aligned(dt, 4) || !aligned(A, 4) || (D && !aligned(D, 4)))
        return SSD_ERR_INVALID_ARGUMENT;
    ssd::DtProc dtp;
    const ssd_status st = check_dt_proc(dt_proc, &dtp);
    if (st != SSD_OK) return st;
    const void *z = gate ? gate->z : nullptr;
    const bool D_hdim = gate && gate->D_per_channel && D;
    if (z && !aligned(z, es)) return SSD_ERR_INVALID_ARGUMENT;
    ssd::DecodeArgs a;
    a.state = state;
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.y = y;
    a.batch = batch;
    a.H = nheads;
    a.G = ngroups;
    a.P = headdim;
    a.N = dstate;
    a.dtp = dtp;
    a.z = z;
    a.D_hdim = D_hdim;
    const size_t nst = (size_t)batch * nheads * headdim * dstate;
    const size_t nxh = (size_t)batch * nheads * headdim;
    const size_t nbc = (size_t)batch * ngroups * dstate;
    FiniteCheck fc(stream);
    fc.input(state, nst, 4);
    fc.input(x, nxh, (int)es);
    fc.input(dt, (size_t)batch * nheads, 4);
    fc.input(A, nheads, 4);
    fc.input(B, nbc, (int)es);
    fc.input(C, nbc, (int)es);
    fc.input(D, D ? (D_hdim ? (size_t)nheads * headdim : (size_t)nheads) : 0, 4);
    fc.input(dtp.bias, dtp.bias ? nheads : 0, 4);
    fc.input(z, z ? nxh : 0, (int)es);
    hipError_t err = io_dtype == SSD_BF16 ? ssd::launch_state_update<ssd::bf16>(a, stream)
                                          : ssd::launch_state_update<float>(a, stream);
    if (err != hipSuccess) return SSD_ERR_HIP;
    fc.output(y, nxh, (int)es);
    fc.output(state, nst, 4);
    return fc.finish(SSD_OK);
}

ssd_status ssd_state_update_ex(float *state, const void *x, const float *dt, const float *A,
                               const void *B, const void *C, const float *D, int ngroups,
                               int batch, int nheads, int headdim, int dstate,
                               ssd_dtype io_dtype, void *y, hipStream_t stream,
                               const ssd_dt_proc *dt_proc) {
    return ssd_state_update_full(state, x, dt, A, B, C, D, ngroups, batch, nheads, headdim,
                                 dstate, io_dtype, y, stream, dt_proc, nullptr);
}

ssd_status ssd_state_update(float *state, const void *x, const float *dt, const float *A,
                            const void *B, const void *C, const float *D, int ngroups,
                            int batch, int nheads, int headdim, int dstate,
                            ssd_dtype io_dtype, void *y, hipStream_t stream) {
    return ssd_state_update_full(state, x, dt, A, B, C, D, ngroups, batch, nheads, headdim,
                                 dstate, io_dtype, y, stream, nullptr, nullptr);
}

namespace {

ssd_status check_conv(const void *x, const float *weight, const float *bias, int batch,
                      int seqlen, int dim, int width, int activation, ssd_dtype io_dtype,
                      const void *out) {
    if (batch <= 0 || seqlen <= 0 || dim <= 0 || width <= 0) return SSD_ERR_INVALID_ARGUMENT;
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
    if (activation != SSD_ACT_NONE && activation != SSD_ACT_SILU) return SSD_ERR_INVALID_ARGUMENT;
    if (!x || !weight || !out) return SSD_ERR_INVALID_ARGUMENT;
    if (width < 2 || width > 4 || dim % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (batch > 65535 || (seqlen + 63) / 64 > 65535 || (double)batch * seqlen * dim > 9.0e15)
        return SSD_ERR_UNSUPPORTED;
    if (!aligned(weight, 4) || (bias && !aligned(bias, 4))) return SSD_ERR_INVALID_ARGUMENT;
    return SSD_OK;
}

}  // namespace

ssd_status ssd_causal_conv1d_fwd(const void *x, const float *weight, const float *bias,
                                 int batch, int seqlen, int dim, int width, int activation,
                                 ssd_dtype io_dtype, void *out, void *conv_state,
                                 hipStream_t stream) {
    ssd_status st = check_conv(x, weight, bias, batch, seqlen, dim, width, activation, io_dtype,
                               out);
    if (st != SSD_OK) return st;
    const size_t es = io_dtype == SSD_BF16 ? 2 : 4;
    // 16-byte vectors of 8 channels (bf16) or two of 4 (fp32)
    if (!aligned(x, 16) || !aligned(out, 16) || (conv_state && !aligned(conv_state, es)))
        return SSD_ERR_INVALID_ARGUMENT;
    ssd::ConvArgs a{x, weight, bias, out, conv_state, batch, seqlen, dim, width,
                    activation == SSD_ACT_SILU ? 1 : 0};
    const size_t n = (size_t)batch * seqlen * dim;
    FiniteCheck fc(stream);
    fc.input(x, n, (int)es);
    fc.input(weight, (size_t)dim * width, 4);
    fc.input(bias, bias ? dim : 0, 4);
    const hipError_t err = io_dtype == SSD_BF16 ? ssd::launch_conv1d_fwd<ssd::bf16>(a, stream)
                                                : ssd::launch_conv1d_fwd<float>(a, stream);
    if (err != hipSuccess) return SSD_ERR_HIP;
    fc.output(out, n, (int)es);
    fc.output(conv_state, conv_state ? (size_t)batch * dim * width : 0, (int)es);
    return fc.finish(SSD_OK);
}

ssd_status ssd_causal_conv1d_update(void *conv_state, const void *x, const float *weight,
                                    const float *bias, int batch, int dim, int width,
                                    int activation, ssd_dtype io_dtype, void *out,
                                    hipStream_t stream) {
    ssd_status st = check_conv(x, weight, bias, batch, 1, dim, width, activation, io_dtype, out);
    if (st != SSD_OK) return st;
    if (!conv_state) return SSD_ERR_INVALID_ARGUMENT;
    const size_t es = io_dtype == SSD_BF16 ? 2 : 4;
    if (!aligned(x, es) || !aligned(out, es) || !aligned(conv_state, es))
        return SSD_ERR_INVALID_ARGUMENT;
    ssd::ConvArgs a{x, weight, bias, out, conv_state, batch, 1, dim, width,
                    activation == SSD_ACT_SILU ? 1 : 0};
    const size_t ncache = (size_t)batch * dim * width;
    FiniteCheck fc(stream);
    fc.input(conv_state, ncache, (int)es);
    fc.input(x, (size_t)batch * dim, (int)es);
    fc.input(weight, (size_t)dim * width, 4);
    fc.input(bias, bias ? dim : 0, 4);
    const hipError_t err = io_dtype == SSD_BF16 ? ssd::launch_conv1d_update<ssd::bf16>(a, stream)
                                                : ssd::launch_conv1d_update<float>(a, stream);
    if (err != hipSuccess) return SSD_ERR_HIP;
    fc.output(out, (size_t)batch * dim, (int)es);
    fc.output(conv_state, ncache, (int)es);
    return fc.finish(SSD_OK);
}

ssd_status ssd_gated_rmsnorm_fwd(const void *y, const void *z, const float *weight, int rows,
                                 int dim, float eps, int norm_before_gate, ssd_dtype io_dtype,
                                 void *out, hipStream_t stream) {
    if (rows <= 0 || dim <= 0 || !(eps >= 0.f) || eps > 3.0e38f) return SSD_ERR_INVALID_ARGUMENT;
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
    if (!y || !weight || !out) return SSD_ERR_INVALID_ARGUMENT;
    if (dim % 8 != 0 || dim > ssd::kMaxNormDim) return SSD_ERR_UNSUPPORTED;
    if ((double)rows * dim > 9.0e15) return SSD_ERR_UNSUPPORTED;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(weight, 16) || (z && !aligned(z, 16)))
        return SSD_ERR_INVALID_ARGUMENT;
    ssd::NormArgs a;
    a.y = y;
    a.z = z;
    a.w = weight;
    a.out = out;
    a.rows = rows;
    a.dim = dim;
    a.gate = z ? (norm_before_gate ? 2 : 1) : 0;
    a.eps = eps;
    const int es = io_dtype == SSD_BF16 ? 2 : 4;
    const size_t n = (size_t)rows * dim;
    FiniteCheck fc(stream);
    fc.input(y, n, es);
    fc.input(z, z ? n : 0, es);
    fc.input(weight, dim, 4);
    const hipError_t err = io_dtype == SSD_BF16 ? ssd::launch_gated_rmsnorm<ssd::bf16>(a, stream)
                                                : ssd::launch_gated_rmsnorm<float>(a, stream);
    if (err != hipSuccess) return SSD_ERR_HIP;
    fc.output(out, n, es);
    return fc.finish(SSD_OK);
}

ssd_status ssd_chunk_scan_bwd_workspace_size(int batch, int seqlen, int nheads, int headdim,
                                             int dstate, int ngroups, int chunk_len,
                                             ssd_dtype io_dtype, size_t *bytes) {
    if (!bytes) return SSD_ERR_INVALID_ARGUMENT;
    const ssd_status st = check_forward_shape(batch, seqlen, nheads, headdim, dstate, ngroups,
                                              chunk_len, io_dtype);
    if (st != SSD_OK) return st;
    *bytes = backward_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len,
                             io_dtype)
                 .total;
    return SSD_OK;
}

ssd_status ssd_chunk_scan_bwd(const void *x, const float *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *initial_state,
                              const void *dy, const float *dfinal_state, int chunk_len,
                              int ngroups, int batch, int seqlen, int nheads, int headdim,
                              int dstate, ssd_dtype io_dtype, void *dx, float *ddt, float *dA,
                              void *dB, void *dC, float *dD, float *dinitial_state,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return backward_impl(x, dt, A, B, C, D, initial_state, dy, dfinal_state, chunk_len, ngroups,
                         batch, seqlen, nheads, headdim, dstate, io_dtype, dx, ddt, dA, dB, dC,
                         dD, dinitial_state, workspace, workspace_bytes, stream, nullptr,
                         nullptr, nullptr);
}

int ssd_chunk_scan_bwd_max_kernels(void) { return ssd::kBackwardKernels; }

ssd_status ssd_chunk_scan_bwd_timed(const void *x, const float *dt, const float *A,
                                    const void *B, const void *C, const float *D,
                                    const float *initial_state, const void *dy,
                                    const float *dfinal_state, int chunk_len, int ngroups,
                                    int batch, int seqlen, int nheads, int headdim, int dstate,
                                    ssd_dtype io_dtype, void *dx, float *ddt, float *dA,
                                    void *dB, void *dC, float *dD, float *dinitial_state,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream, hipEvent_t *events, int nevents,
                                    int *nkernels, const char **kernel_names) {
    if (!events || nevents < ssd::kBackwardKernels + 1) return SSD_ERR_INVALID_ARGUMENT;
    for (int i = 0; i <= ssd::kBackwardKernels; ++i)
        if (!events[i]) return SSD_ERR_INVALID_ARGUMENT;
    return backward_impl(x, dt, A, B, C, D, initial_state, dy, dfinal_state, chunk_len, ngroups,
                         batch, seqlen, nheads, headdim, dstate, io_dtype, dx, ddt, dA, dB, dC,
                         dD, dinitial_state, workspace, workspace_bytes, stream, events,
                         nkernels, kernel_names);
}

}  // extern "C"
