// Drives libssd's host side (argument validation, path choice, workspace
// layout) under AddressSanitizer and UndefinedBehaviorSanitizer (built by
// tests/test_sanitizers.py with the sanitizers on the host pass only).  Test
// infrastructure only.  Every call here must return before anything reaches
// a GPU: workspace queries over many shapes, and calls that validation
// rejects (NULL, misaligned or inconsistent arguments, unsupported shapes,
// a missing workspace).  Prints "ok" and exits 0 on success.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "ssd.h"

static int bad = 0;

static void expect(ssd_status got, ssd_status want, const char *what) {
    if (got != want) {
        std::fprintf(stderr, "%s: status %d, expected %d\n", what, (int)got, (int)want);
        bad = 1;
    }
}

int main() {
    // never dereferenced: validation fails before any device access
    void *const P16 = reinterpret_cast<void *>(uintptr_t(0x10000));
    void *const P2 = reinterpret_cast<void *>(uintptr_t(0x10002));
    float *const F16 = static_cast<float *>(P16);
    size_t n = 0;
    // workspace queries, both paths, segmented and not, every chunk length
    // (chunks x groups beyond 65535 exceed the split path's launch grid)
    for (int q : {16, 32, 64, 128, 256})
        for (int io : {0, 1})
            for (int L : {1, 31, 32, 33, 1000, 16380, 262144}) {
                ssd_status st = ssd_chunk_scan_fwd_workspace_size(2, L, 64, 64, 128, 8, q,
                                                                  (ssd_dtype)io, &n);
                const long grid = (long)((L + q - 1) / q) * 8;
                expect(st, grid > 65535 ? SSD_ERR_UNSUPPORTED : SSD_OK, "workspace query");
            }
    expect(ssd_chunk_scan_fwd_workspace_size(4, 8192, 80, 64, 128, 1, 256, SSD_BF16, &n), SSD_OK,
           "2.7B");
    expect(ssd_chunk_scan_fwd_workspace_size(1, 100, 4, 64, 128, 1, 48, SSD_F32, &n),
           SSD_ERR_UNSUPPORTED, "chunk 48");
    expect(ssd_chunk_scan_fwd_workspace_size(1, 100, 4, 24, 128, 1, 64, SSD_F32, &n),
           SSD_ERR_UNSUPPORTED, "headdim 24");
    expect(ssd_chunk_scan_fwd_workspace_size(1, 100, 6, 64, 128, 4, 64, SSD_F32, &n),
           SSD_ERR_INVALID_ARGUMENT, "heads not a multiple of groups");
    expect(ssd_chunk_scan_fwd_workspace_size(0, 100, 4, 64, 128, 1, 64, SSD_F32, &n),
           SSD_ERR_INVALID_ARGUMENT, "batch 0");
    for (int io : {7, -1, 2, 0x7FFFFFFF})
        expect(ssd_chunk_scan_fwd_workspace_size(1, 100, 4, 64, 128, 1, 64, (ssd_dtype)io, &n),
               SSD_ERR_INVALID_ARGUMENT, "dtype");
    // forward calls that validation rejects
    expect(ssd_chunk_scan_fwd(nullptr, F16, F16, P16, P16, nullptr, nullptr, 64, 1, 1, 100, 4, 64,
                              128, SSD_F32, P16, nullptr, P16, 1 << 20, nullptr),
           SSD_ERR_INVALID_ARGUMENT, "x NULL");
    expect(ssd_chunk_scan_fwd(P2, F16, F16, P16, P16, nullptr, nullptr, 64, 1, 1, 100, 4, 64, 128,
                              SSD_F32, P16, nullptr, P16, 1 << 20, nullptr),
           SSD_ERR_INVALID_ARGUMENT, "x misaligned");
    expect(ssd_chunk_scan_fwd(P16, F16, F16, P16, P16, nullptr, nullptr, 64, 1, 1, 100, 4, 64, 128,
                              SSD_F32, P16, nullptr, nullptr, 0, nullptr),
           SSD_ERR_WORKSPACE, "no workspace");
    expect(ssd_chunk_scan_fwd(P16, F16, F16, P16, P16, nullptr, nullptr, 64, 1, 1, 100, 4, 64, 128,
                              SSD_F32, P16, nullptr, P16, 16, nullptr),
           SSD_ERR_WORKSPACE, "workspace too small");
    expect(ssd_chunk_scan_fwd_varlen(P16, F16, F16, P16, P16, nullptr, nullptr, 64, 1, 1, 100, 4,
                                     64, 128, SSD_BF16, P16, nullptr, nullptr, 0, nullptr,
                                     nullptr, nullptr),
           SSD_ERR_INVALID_ARGUMENT, "varlen without seq_idx");
    ssd_dt_proc bad_dtp = {nullptr, 1, 1.0f, 0.5f};
    expect(ssd_chunk_scan_fwd_ex(P16, F16, F16, P16, P16, nullptr, nullptr, 64, 1, 1, 100, 4, 64,
                                 128, SSD_BF16, P16, nullptr, nullptr, 0, nullptr, &bad_dtp),
           SSD_ERR_INVALID_ARGUMENT, "dt_max below dt_min");
    ssd_gate gate = {P2, 0};
    expect(ssd_chunk_scan_fwd_full(P16, F16, F16, P16, P16, nullptr, nullptr, 64, 1, 1, 100, 4,
                                   64, 128, SSD_BF16, P16, nullptr, nullptr, 0, nullptr, nullptr,
                                   nullptr, &gate),
           SSD_ERR_INVALID_ARGUMENT, "z misaligned");
    expect(ssd_chunk_scan_fwd_noalloc(P16, F16, F16, P16, P16, nullptr, nullptr, 256, 1, 1, 8192,
                                      80, 64, 128, SSD_F32, P16, nullptr, nullptr),
           SSD_ERR_WORKSPACE, "noalloc beyond the scratch");
    // decode, convolution and normalisation validation
    expect(ssd_state_update(nullptr, P16, F16, F16, P16, P16, nullptr, 1, 2, 4, 64, 128, SSD_BF16,
                            P16, nullptr),
           SSD_ERR_INVALID_ARGUMENT, "state NULL");
    expect(ssd_state_update(F16, P16, F16, F16, P16, P16, nullptr, 3, 2, 4, 64, 128, SSD_BF16,
                            P16, nullptr),
           SSD_ERR_INVALID_ARGUMENT, "decode groups");
    expect(ssd_causal_conv1d_fwd(P16, F16, nullptr, 1, 100, 64, 5, SSD_ACT_SILU, SSD_BF16, P16,
                                 nullptr, nullptr),
           SSD_ERR_UNSUPPORTED, "conv width 5");
    expect(ssd_causal_conv1d_update(nullptr, P16, F16, nullptr, 1, 64, 4, SSD_ACT_NONE, SSD_BF16,
                                    P16, nullptr),
           SSD_ERR_INVALID_ARGUMENT, "conv state NULL");
    expect(ssd_gated_rmsnorm_fwd(P16, P16, F16, 0, 64, 1e-5f, 1, SSD_BF16, P16, nullptr),
           SSD_ERR_INVALID_ARGUMENT, "norm rows 0");
    for (int code = 0; code <= 6; ++code)
        if (!ssd_status_string((ssd_status)code)) bad = 1;
    if (ssd_abi_version() != SSD_ABI_VERSION) bad = 1;
    if (!bad) std::printf("ok\n");
    return bad;
}
