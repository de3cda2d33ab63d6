// ssd_check_kernels.hip -- the opt-in check for non-finite values (NaN or
// infinity) in the inputs and outputs of a call, the counterpart of the
// guards burn-mamba `mamba2/ssd/serial.rs` runs on every intermediate of
// `ssd_serial` (its `san` calls) and of the rustdoc's `Mamba2SsdInput::sanity`.
//
// A value is non-finite when its exponent bits are all ones: bits 30..23 of
// an fp32 word, bits 14..7 of a bf16 half-word.  A 32-bit word holding two
// bf16 values therefore carries the high one's exponent where an fp32 value
// keeps it, and the low one's in bits 14..7.
//
// The result is one word per device (a module global): bit 0 set when an
// input held a non-finite value, bit 1 when an output did.  The host clears
// it with a one-thread kernel (no memset node, so the sequence stays legal
// inside stream capture up to the read-back), scans every buffer, and reads
// it back after the call's kernels.
#include "ssd_device.hpp"
#include "ssd_kernels.hpp"

namespace ssd {

__device__ unsigned int g_nonfinite;

__global__ void k_nonfinite_reset() {
    if (blockIdx.x == 0 && threadIdx.x == 0) g_nonfinite = 0u;
}

__device__ __forceinline__ bool word_nonfinite(unsigned w, bool pairs) {
    const bool hi = (w & 0x7F800000u) == 0x7F800000u;
    const bool lo = (w & 0x00007F80u) == 0x00007F80u;
    return hi || (pairs && lo);
}

// Scans `nwords` aligned 32-bit words (fp32 values, or bf16 pairs when
// `pairs`), and the bf16 half-words `head` and `tail` (null when absent:
// a 2-byte aligned start, an odd remainder).  Grid-stride; one atomic OR per
// thread that saw a non-finite value.
__global__ void __launch_bounds__(256)
k_nonfinite_scan(const unsigned *__restrict__ p, size_t nwords, const unsigned short *head,
                 const unsigned short *tail, int pairs, unsigned bit) {
    bool bad = false;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride)
        bad |= word_nonfinite(p[i], pairs != 0);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (head) bad |= (*head & 0x7F80u) == 0x7F80u;
        if (tail) bad |= (*tail & 0x7F80u) == 0x7F80u;
    }
    if (bad) atomicOr(&g_nonfinite, bit);
}

hipError_t launch_nonfinite_reset(hipStream_t stream) {
    hipLaunchKernelGGL(k_nonfinite_reset, dim3(1), dim3(64), 0, stream);
    return hipGetLastError();
}

hipError_t launch_nonfinite_scan(const void *p, size_t nelems, int elem_bytes, unsigned bit,
                                 hipStream_t stream) {
    if (!p || nelems == 0) return hipSuccess;
    const bool pairs = elem_bytes == 2;
    const unsigned short *h = static_cast<const unsigned short *>(p);
    const unsigned short *head = nullptr, *tail = nullptr;
    if (pairs && (reinterpret_cast<uintptr_t>(p) & 3) != 0) {
        // bf16 data on a 2-byte boundary: the first value on its own
        head = h;
        ++h;
        --nelems;
    }
    const size_t nwords = pairs ? nelems / 2 : nelems;
    if (pairs && (nelems & 1)) tail = h + (nelems - 1);
    size_t blocks = (nwords + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(k_nonfinite_scan, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const unsigned *>(h), nwords, head, tail, pairs ? 1 : 0,
                       bit);
    return hipGetLastError();
}

// The workspace poison of the debug mode: every 32-bit word of the
// workspace becomes a quiet NaN (0x7FC00000) before a forward, so a kernel
// that reads an element no earlier kernel of the call wrote passes the NaN
// on to the outputs.  A plain fill kernel (no memset node).
__global__ void __launch_bounds__(256) k_poison(unsigned *__restrict__ p, size_t nwords) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride)
        p[i] = 0x7FC00000u;
}

hipError_t launch_poison(void *p, size_t bytes, hipStream_t stream) {
    const size_t nwords = bytes / 4;
    if (!p || nwords == 0) return hipSuccess;
    size_t blocks = (nwords + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_poison, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<unsigned *>(p), nwords);
    return hipGetLastError();
}

hipError_t read_nonfinite(unsigned *out, hipStream_t stream) {
    hipError_t err = hipMemcpyFromSymbolAsync(out, HIP_SYMBOL(g_nonfinite), sizeof(unsigned), 0,
                                              hipMemcpyDeviceToHost, stream);
    if (err != hipSuccess) return err;
    return hipStreamSynchronize(stream);
}

}  // namespace ssd
