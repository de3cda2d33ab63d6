// ssd_fused_kernels.hip -- the chunked SSD forward as one pass over the
// sequence per (batch, head, headdim-block), with the fp32 state held in
// registers the whole way (bf16 inputs; fp32 inputs use the split kernels).
//
// The sequence is processed in 32-token blocks.  For block k starting at
// token b0, with lambda_s = sum_{j=b0..s} dt_j A (the within-block prefix of
// the decay exponent), e = b0 + 31 and h_k the state entering the block:
//
//   y_l     = exp(lambda_l) C_l h_k^T                        state-to-output
//           + sum_{b0<=s<=l} (C_l . B_s) exp(lambda_l - lambda_s) dt_s x_s
//           + D x_l                                          intra-block + skip
//   h_{k+1} = exp(lambda_e) h_k + sum_s exp(lambda_e - lambda_s) dt_s x_s^T B_s
//
// which is the chunked algorithm of the burn-mamba `Mamba2SsdInput` rustdoc
// (`ssd_minimal`: Step 1 intra-chunk output (L o C B^T) X, Step 2 chunk state
// (Eq. 20), Step 3 state passing (Eq. 22), Step 4 state-to-output (Eq. 23))
// and of the five kernels of burn-mamba `mamba2/ssd/serial.rs`, evaluated
// with 32-token blocks: inside a chunk of any length the off-diagonal blocks
// of L o C B^T are low rank (rank dstate), and contracting them through the
// running state is that same factorisation applied within the chunk.  The
// result equals the chunked result for every chunk length up to rounding;
// the work per token does not depend on the chunk length.
//
// Scaled state.  The registers hold h~ with h = sigma h~ for a scalar sigma
// that the kernel tracks, so the per-block decay exp(lambda_e) multiplies
// sigma instead of the 128 x 16 state tile of every wave:
//   x'_s  = exp(lambda_e - lambda_s) dt_s x_s / sigma_{k+1}     (staged, bf16)
//   y_l   = exp(lambda_l - lambda_e) sigma_{k+1} (C_l h~^T + [C B^T]_l x') + D x_l
//   h~   += B^T x'
// with sigma_{k+1} = sigma_k exp(lambda_e).  When sigma_{k+1} would fall
// below exp(-40) the state is rescaled once (h~ *= sigma_k, sigma_k = 1), so
// 1/sigma stays below exp(40) and nothing approaches the fp32 range.
//
// The diagonal block uses the factored weights exp(lambda_l - lambda_e) and
// exp(lambda_e - lambda_s) only when the block's total decay is at most
// exp(-40) away from 1; otherwise both could leave the fp32 range, and the
// block is evaluated with the exact per-element weights
// exp(lambda_l - lambda_s) dt_s (s > l exactly 0, the upper-triangle
// protection of the Kernel 5 page) on raw x, with D on the diagonal, and the
// state decays explicitly (h~ <- sigma_k exp(lambda_e) h~ + B^T x', sigma = 1).
//
// Workgroup = NW waves; wave w owns headdim tile w (16 columns) of the
// block of PB = 16 NW columns.  Per 32-token block:
//   stage (next block, double-buffered LDS): C and B rows straight from
//          global memory into LDS (global_load_lds) in a swizzled layout,
//          x raw and scaled through registers, the causal diagonal block of
//          C B^T (precomputed, in fragment order); decay vectors two
//          blocks ahead;
//   output y^T = h~ C^T + x'^T [C B^T]^T for the wave's 16 headdim columns
//          and both 16-token tiles, with h~ taken straight from the state
//          registers as the MFMA A operand; each lane ends with 4
//          consecutive headdim values of one token (one 8-byte store);
//   state  h~ += B^T x'.
//
// Register state layout: st[m][e] = h~[n][p] for p = 16 wave + (lane % 16)
// and n = 32 (m >> 1) + 8 (lane / 16) + 4 (m & 1) + e, so st[2ks], st[2ks+1]
// are the 8 consecutive n = 32 ks + 8 q .. +7 that the bf16 MFMA fragment of
// K-step ks holds in lane group q.
//
// Operands that the MFMA needs transposed (B^T, x'^T) are read from
// row-major LDS with ds_read_b64_tr_b16: within each 16-lane group, lane 4a+c
// receives element c of the 8-byte reads of lanes a, a+4, a+8, a+12, so
// pointing lane a + 4 e at row kbase + e and 4 consecutive columns of a
// row-major [k][n] tile hands those 4 columns to lanes 4a .. 4a+3.
//
// C / B rows (256 bytes) sit in LDS without padding; 16-byte chunk c of row t
// is stored in slot c ^ swz(t), swz(t) = (t&1) | (t&2)<<1 | (t>>1)&2.  The
// fragment reads of C (16 rows, one chunk) then hit 8 distinct 16-byte bank
// groups per 8 lanes, and the transposed reads of B at most two lanes per
// bank.
#include "ssd_device.hpp"
#include "ssd_kernels.hpp"

namespace ssd {

constexpr int kBlk = 32;                  // tokens per block
constexpr float kSafeDecay = 40.f;        // max -lambda_e for the factored diagonal
constexpr float kRescale = 4.24835426e-18f;  // exp(-40): smallest sigma kept unrescaled
// s_waitcnt immediate for "vmcnt(0)" alone on gfx9-family targets:
// vmcnt = 0, expcnt = 7 and lgkmcnt = 15 (both at their no-wait maximum).
constexpr int kWaitVmcnt0 = 0x0F70;
// ... and for "vmcnt(n)" alone (n < 64; bits 5:4 of n go to bits 15:14)
constexpr int wait_vmcnt_imm(int n) { return kWaitVmcnt0 | (n & 15) | ((n >> 4) << 14); }
// ... and for "lgkmcnt(0)" alone: vmcnt = 63 (bits 3:0 and 15:14), expcnt = 7.
constexpr int kWaitLgkmcnt0 = 0xC07F;
// word 3 of a raw buffer resource on gfx9-family targets (32-bit data format)
constexpr int kBufferWord3 = 0x00020000;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ bf16x4 lds_tr(const unsigned char *base, int byte_off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)((lds_u8 *)(base) + byte_off));
}
__device__ __forceinline__ bf16x8 lds_b128(const unsigned char *base, int byte_off) {
    return *reinterpret_cast<const bf16x8 *>(base + byte_off);
}
__device__ __forceinline__ bf16x8 join(bf16x4 lo, bf16x4 hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ void dma16(const void *gsrc, unsigned char *lds_wave_base) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)gsrc,
                                     (__attribute__((address_space(3))) void *)(lds_wave_base),
                                     16, 0, 0);
}
__device__ __forceinline__ float uniform(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ unsigned pack2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, bf16x2{(bf16)a, (bf16)b});
}
// 16-byte chunk swizzle of a C / B row in LDS (depends on row & 7 only)
__device__ __forceinline__ int cb_swz(int row) {
    return (row & 1) | ((row & 2) << 1) | ((row >> 1) & 2);
}

template <int PB>
struct Fused {
    static constexpr int NW = PB / 16;                 // waves
    static constexpr int NT = 64 * NW;                 // threads
    static constexpr int N = 128;                      // dstate
    static constexpr int ROWB = 2 * N;                 // bytes per C / B row
    static constexpr int MAT = kBlk * ROWB;            // 8 KB per matrix
    static constexpr int NDMA = MAT / 1024;            // wave-wide 16-byte DMAs per matrix
    static constexpr int DPW = NDMA / NW;              // of which per wave
    static constexpr int XC = PB / 8;                  // 16-byte chunks per x row
    static constexpr int XRB = 2 * PB;                 // raw x row bytes (swizzled chunks)
    // one stage (three in flight), filled by DMA: C rows, B rows, C B^T
    // fragments and raw x of block j, and the raw decay vectors (lam_hi,
    // lam_lo, dt: 384 bytes of a 1 KB wave-wide DMA) of block j + 2
    static constexpr int CS = 0;
    static constexpr int BS = MAT;
    static constexpr int CBF = 2 * MAT;                // 2 x 1 KB of C B^T fragments
    static constexpr int XR = CBF + 2048;
    static constexpr int RV = XR + kBlk * XRB;
    static constexpr int STG = RV + 1024;
    // derived per-block vectors (floats), three blocks in flight
    enum { LHI = 0, LLO = 32, DT = 64, CF = 96, RP = 128, EX = 160, DELTA = 192, FLAG = 193,
           VFLOATS = 196 };
    static constexpr int LDS = 3 * STG + 3 * VFLOATS * 4;
    // DMAs every wave issues at the start of every block, all with every lane
    // active: C / B, one C B^T, one x, one decay-vector DMA.  (The block's two
    // y stores follow its end-of-block wait.)
    static constexpr int VM_LOADS = 2 * DPW + 1 + 1 + 1;
    static_assert(NDMA % NW == 0, "DMAs split evenly over the waves");
    static_assert(XC * kBlk == NT, "one x chunk per thread: one x DMA per wave");
    static_assert(STG % 16 == 0, "alignment");
    static_assert(2 * LDS <= 160 * 1024, "two workgroups per compute unit");
    static_assert(VM_LOADS < 64, "vmcnt immediate");
};

// Chunk swizzle of the raw x rows (16-byte chunks, XOR on the chunk index):
// the transposed reads (4 rows x 32 bytes per 16 lanes) land in 4 distinct
// 32-byte bank windows, and the 8-byte reads of the skip term (16 rows, one
// column) at most two lanes per bank.
template <int PB>
__device__ __forceinline__ int x_swz(int row) {
    return PB == 64 ? 2 * (row & 3) + ((row >> 2) & 1) : 2 * ((row >> 1) & 1) + ((row >> 2) & 1);
}

// Workgroup barrier for LDS only: this wave's LDS reads and writes complete
// (lgkmcnt(0)), then s_barrier; the asm "memory" clobber keeps the compiler
// from moving memory accesses across it.  __syncthreads() (or an LDS-scope
// fence) would also make the wave wait for every outstanding global load,
// store and LDS DMA (vmcnt(0)) at each barrier, the prefetches included;
// the LDS writes of global_load_lds are covered by explicit vmcnt waits.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
    asm volatile("s_barrier" ::: "memory");
}

// Scale bookkeeping of one block (identical in every wave).
struct Book {
    float sig_in;   // sigma entering the block
    float sig;      // sigma after the block
    float delta;    // exp(lambda_e)
    bool fac;       // factored diagonal
    bool rescale;   // h~ *= sig_in before the block (factored blocks only)
};

template <int PB>
__global__ void __launch_bounds__(4 * PB)
k_fused_ssd(const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
            const bf16 *__restrict__ cbf, const float *__restrict__ lam_hi,
            const float *__restrict__ lam_lo, const float *__restrict__ dtb,
            const float *__restrict__ D, const float *init, float *final_state,
            bf16 *__restrict__ y, int L, int H, int G, int P, int nblk) {
    typedef Fused<PB> S;
    constexpr int NW = S::NW, N = S::N;
    // Every LDS region that a DMA fills is its own object: the compiler can
    // then see that a DMA in flight never aliases the reads of another
    // region, and does not wait for it before those reads.
    __shared__ __align__(16) unsigned char stg0[S::STG];
    __shared__ __align__(16) unsigned char stg1[S::STG];
    __shared__ __align__(16) unsigned char stg2[S::STG];
    __shared__ __align__(16) float svec[3 * S::VFLOATS];

    const int npb = P / PB;
    const int pb = blockIdx.x % npb, h = blockIdx.x / npb, b = blockIdx.y;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int p0 = pb * PB, pt = wave;
    const size_t bh = (size_t)b * H + h;
    const float Dh = D ? D[h] : 0.f;
    const int GN = G * N, HP = H * P;

    // ---- per-lane LDS byte offsets
    // C fragment of token row 16 lt + r, chunk 4 ks + q:
    //   CS + c_rd[ks & 1] + 128 (ks >> 1) + 4096 lt
    int c_rd[2];
    {
        const int sw = cb_swz(r), s2 = (sw >> 2) & 1, s01 = sw & 3;
#pragma unroll
        for (int par = 0; par < 2; ++par)
            c_rd[par] = r * S::ROWB + 16 * (q ^ s01) + 64 * (par ^ s2);
    }
    // B^T, tile m, token half s: BS + b_tr[s][(m >> 1) & 1] + 128 (m >> 2) + 8 (m & 1)
    int b_tr[2][2];
    {
        const int a = r & 3, e = r >> 2, w0 = e & 1, w2 = (e >> 1) & 1;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                b_tr[s][mb] = (8 * q + e + 4 * s) * S::ROWB + 64 * (mb ^ w2) +
                              16 * (a ^ (w0 | (s << 1)));
    }
    const int cbf_rd = lane * 16;
    // raw x: chunk c of row t sits at XR + xr_off(t, c)
    auto xr_off = [](int t, int c) { return t * S::XRB + 16 * (c ^ x_swz<PB>(t)); };
    // x^T fragment (tokens 8q .. 8q+7, column r of the wave's tile): transposed
    // reads at XR + xr_tr[0] (tokens 8q .. 8q+3) and XR + xr_tr[1] (8q+4 ..)
    int xr_tr[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        xr_tr[s] = xr_off(8 * q + (r >> 2) + 4 * s, 2 * pt + ((r & 3) >> 1)) + 8 * (r & 1);
    // raw x of the skip term: token 16 lt + r, columns 16 pt + 4 q .. +3
    //   XR + xr_skip + 16 XRB lt
    const int xr_skip = xr_off(r, 2 * pt + (q >> 1)) + 8 * (q & 1);
    // x DMA of this wave: LDS bytes 1024 wave + 16 lane of XR, i.e. row
    // xd_row, slot xd_slot, holding global chunk xd_slot ^ x_swz(xd_row)
    const int xd_row = (64 * wave + lane) / S::XC;
    const int xd_chunk = ((64 * wave + lane) % S::XC) ^ x_swz<PB>(xd_row);
    const int xd_off = xd_row * HP + 8 * xd_chunk;  // elements from the block's first row
    // C / B DMA i of this wave covers LDS bytes 1024 (wave + NW i) + 16 lane:
    // row dma_row + 4 NW i, slot lane & 15, holding global chunk dma_chunk
    const int dma_row = 4 * wave + (lane >> 4);
    const int dma_chunk = (lane & 15) ^ cb_swz(dma_row);
    const int dma_off = dma_row * GN * 2 + 16 * dma_chunk;  // bytes
    // decay-vector DMA, 16 bytes per lane: lanes 0-23 copy lam_hi, lam_lo, dt
    // of the block, lanes 24-63 repeat lanes 0-15 (bytes 384-1023 of the
    // region are never read)
    const int vd_arr = (lane < 24 ? lane : (lane & 15)) >> 3, vd_elt = 4 * (lane & 7);
    const size_t vstride = (size_t)(lam_lo - lam_hi);

    // ---- register-resident scaled state
    f32x4 st[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        st[m] = zero4();
        if (init) {
            const float4 v = *reinterpret_cast<const float4 *>(
                init + (bh * P + p0 + 16 * pt + r) * N + 32 * (m >> 1) + 8 * q + 4 * (m & 1));
            st[m] = f32x4{v.x, v.y, v.z, v.w};
        }
    }

    auto stage = [&](int i) -> unsigned char * { return i == 0 ? stg0 : (i == 1 ? stg1 : stg2); };
    auto V = [&](int kb) -> float * { return svec + (kb % 3) * S::VFLOATS; };
    // C, B rows, the C B^T fragments and raw x of block kb into stage `buf`:
    // DPW DMAs per matrix, one C B^T DMA (waves 2w' and 2w'+1 both copy half
    // w' of the 2 KB when NW = 4), one x DMA.  Rows past the end of the
    // sequence repeat its last row.
    auto dma_block = [&](int kb, unsigned char *buf) {
        const int t0 = kb * kBlk;
        const unsigned char *crow =
            reinterpret_cast<const unsigned char *>(Cm + ((size_t)b * L + t0) * GN + (size_t)g * N);
        const unsigned char *brow =
            reinterpret_cast<const unsigned char *>(Bm + ((size_t)b * L + t0) * GN + (size_t)g * N);
        const bf16 *xrow = x + ((size_t)b * L + t0) * HP + (size_t)h * P + p0;
        const int half = NW == 4 ? wave >> 1 : wave;
        const bf16 *cbsrc =
            cbf + (((size_t)b * nblk + kb) * G + g) * (kBlk * kBlk) + 8 * (64 * half + lane);
        // last row of the block inside the sequence (31 except in a partial
        // last block).  One straight-line path: the compiler counts these
        // DMAs exactly only when no branch splits them.
        const int lim = min(L - 1 - t0, kBlk - 1);
#pragma unroll
        for (int i = 0; i < S::DPW; ++i) {
            const int off = min(dma_row + 4 * NW * i, lim) * GN * 2 + 16 * dma_chunk;
            dma16(crow + off, buf + S::CS + 1024 * (wave + NW * i));
            dma16(brow + off, buf + S::BS + 1024 * (wave + NW * i));
        }
        dma16(cbsrc, buf + S::CBF + 1024 * half);
        dma16(xrow + min(xd_row, lim) * HP + 8 * xd_chunk, buf + S::XR + 1024 * wave);
    };
    // raw decay vectors of block kb (lam_hi, lam_lo, dt) into `dst`
    // (the three arrays are equal-size consecutive regions: lam_lo = lam_hi +
    // vstride, dtb = lam_lo + vstride, which the launcher checks)
    auto vec_dma = [&](int kb, unsigned char *buf) {
        dma16(lam_hi + vd_arr * vstride + (bh * nblk + kb) * kBlk + vd_elt, buf + S::RV);
    };
    // derived per-token vectors of block kb (lanes 0-31: token lane; eh, el =
    // the block's last prefix)
    auto vec_derive = [&](int kb, float lh, float ll, float dv, float eh, float el) {
        if (lane < kBlk) {
            float *v = V(kb);
            const bool fac = -(eh + el) <= kSafeDecay;
            v[S::LHI + lane] = lh;
            v[S::LLO + lane] = ll;
            v[S::DT + lane] = dv;
            v[S::CF + lane] = fast_exp(prefix_diff(eh, el, lh, ll)) * dv;
            v[S::RP + lane] = fac ? fast_exp(prefix_diff(lh, ll, eh, el)) : 0.f;
            v[S::EX + lane] = fast_exp(lh + ll);
            if (lane == kBlk - 1) {
                v[S::DELTA] = fast_exp(eh + el);
                v[S::FLAG] = fac ? 1.f : 0.f;
            }
        }
    };
    // ... from the raw vectors in a stage
    auto vec_store = [&](int kb, const unsigned char *buf) {
        const float *raw = reinterpret_cast<const float *>(buf + S::RV);
        const int t = lane & (kBlk - 1);
        vec_derive(kb, raw[t], raw[kBlk + t], raw[2 * kBlk + t], raw[kBlk - 1], raw[2 * kBlk - 1]);
    };
    auto book = [&](int kb, float sig_in) -> Book {
        const float *v = V(kb);
        Book bk;
        bk.sig_in = sig_in;
        bk.delta = uniform(v[S::DELTA]);
        bk.fac = uniform(v[S::FLAG]) != 0.f;
        bk.rescale = false;
        if (bk.fac) {
            bk.sig = sig_in * bk.delta;
            if (bk.sig < kRescale) {
                bk.rescale = true;
                bk.sig = bk.delta;
            }
        } else {
            bk.sig = 1.f;
        }
        return bk;
    };
    // y through a buffer resource over this batch's rows: the stores of
    // tokens past the end fall outside it and are dropped by the hardware
    const __amdgpu_buffer_rsrc_t y_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        y + (size_t)b * L * HP, 0, L * HP * 2, kBufferWord3);
    const int y_boff = (r * HP + h * P + p0 + 16 * pt + 4 * q) * 2;
    auto y_store = [&](int kb, const f32x4 (&acc)[2]) {
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) {
            const u32x2 v = {pack2(acc[lt][0], acc[lt][1]), pack2(acc[lt][2], acc[lt][3])};
            __builtin_amdgcn_raw_buffer_store_b64(
                v, y_rsrc, y_boff + (kb * kBlk + 16 * lt) * HP * 2, 0, 0);
        }
    };

    // ---- prologue.  Every global read in the loop is a DMA into LDS issued
    // two blocks ahead of its use (three stages): C / B rows, C B^T and raw x
    // of block j, and the raw decay vectors of block j + 2, which wave
    // (j + 2) % NW turns into the derived vectors at the start of block j.
    // Past the last block the DMAs repeat it, so every block issues the same
    // global memory instructions.
    Book bk;
    {
        const int last = nblk - 1;
        dma_block(0, stg0);
        vec_dma(min(2, last), stg0);
        dma_block(min(1, last), stg1);
        vec_dma(min(3, last), stg1);
        if (wave < 2 && wave <= last) {
            // the derived vectors of blocks 0 and 1 straight from global memory
            const size_t o = (bh * nblk + wave) * kBlk;
            const int t = lane & (kBlk - 1);
            vec_derive(wave, lam_hi[o + t], lam_lo[o + t], dtb[o + t], lam_hi[o + kBlk - 1],
                       lam_lo[o + kBlk - 1]);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        lds_barrier();
        bk = book(0, 1.f);
    }
    float sig_out = 1.f;

    // block kb, si = kb % 3 (a literal in each unrolled copy)
    auto block = [&](int kb, const int si) {
        unsigned char *cur = stage(si);
        const int last = nblk - 1;
        const float *v = V(kb);
        // ---- global memory issue: the same instructions in every block, in
        // this order (the wait at the end of the block counts them)
        dma_block(min(kb + 2, last), stage((si + 2) % 3));
        vec_dma(min(kb + 4, last), stage((si + 2) % 3));
        __builtin_amdgcn_sched_barrier(0);

        // ---- every LDS operand of the block requested up front, so the
        // reads overlap each other and the MFMAs instead of one round trip
        // per step
        bf16x8 cfr[4][2];  // C fragments of y^T = h~ C^T
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int lt = 0; lt < 2; ++lt)
                cfr[ks][lt] = lds_b128(cur, S::CS + c_rd[ks & 1] + 128 * (ks >> 1) + 4096 * lt);
        // x^T fragment of the block: raw x, tokens 8q .. 8q+7 of column r
        bf16x8 xs = join(lds_tr(cur, S::XR + xr_tr[0]), lds_tr(cur, S::XR + xr_tr[1]));
        const f32x4 cf0 = *reinterpret_cast<const f32x4 *>(v + S::CF + 8 * q);
        const f32x4 cf1 = *reinterpret_cast<const f32x4 *>(v + S::CF + 8 * q + 4);
        bf16x8 cbv[2];  // causal diagonal block of C B^T
        float rpv[2];   // exp(lambda_l - lambda_e) of token 16 lt + r
        bf16x4 xr[2];   // raw x of the skip term
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) {
            cbv[lt] = lds_b128(cur, S::CBF + 1024 * lt + cbf_rd);
            rpv[lt] = v[S::RP + 16 * lt + r];
            xr[lt] = *reinterpret_cast<const bf16x4 *>(cur + S::XR + xr_skip + 16 * S::XRB * lt);
        }
        bf16x8 bt[8];   // B^T fragments of the state update
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int o = 128 * (m >> 2) + 8 * (m & 1);
            bt[m] = join(lds_tr(cur, S::BS + b_tr[0][(m >> 1) & 1] + o),
                         lds_tr(cur, S::BS + b_tr[1][(m >> 1) & 1] + o));
        }

        if (bk.rescale) {
#pragma unroll
            for (int m = 0; m < 8; ++m) st[m] *= bk.sig_in;
        }

        // -------- y^T = h~ C^T for both 16-token tiles
        f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 hb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hb[e] = (bf16)st[2 * ks][e];
                hb[4 + e] = (bf16)st[2 * ks + 1][e];
            }
#pragma unroll
            for (int lt = 0; lt < 2; ++lt) acc[lt] = Mma<bf16>::mma(hb, cfr[ks][lt], acc[lt]);
        }
        if (bk.fac) {
            // x' = exp(lambda_e - lambda_s) dt_s x_s / sigma
            const float inv = __builtin_amdgcn_rcpf(bk.sig);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xs[j] = (bf16)((float)xs[j] * (cf0[j] * inv));
                xs[4 + j] = (bf16)((float)xs[4 + j] * (cf1[j] * inv));
            }
#pragma unroll
            for (int lt = 0; lt < 2; ++lt) {
                acc[lt] = Mma<bf16>::mma(xs, cbv[lt], acc[lt]);
                const float f = rpv[lt] * bk.sig;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[lt][e] = acc[lt][e] * f + Dh * (float)xr[lt][e];
            }
        } else {
            // exact weights exp(lambda_l - lambda_s) dt_s on raw x, D on the diagonal
#pragma unroll
            for (int lt = 0; lt < 2; ++lt) {
                const int row = 16 * lt + r;
                acc[lt] *= v[S::EX + row] * bk.sig_in;
                const float lh = v[S::LHI + row], ll = v[S::LLO + row];
                bf16x8 wgt;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = 8 * q + j;
                    const float w = (float)cbv[lt][j] *
                                    fast_exp(fminf(prefix_diff(lh, ll, v[S::LHI + s], v[S::LLO + s]), 0.f)) *
                                    v[S::DT + s] + (s == row ? Dh : 0.f);
                    wgt[j] = (bf16)(s <= row ? w : 0.f);
                }
                acc[lt] = Mma<bf16>::mma(xs, wgt, acc[lt]);
            }
            // the state update takes x' = exp(lambda_e - lambda_s) dt_s x_s
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xs[j] = (bf16)((float)xs[j] * cf0[j]);
                xs[4 + j] = (bf16)((float)xs[4 + j] * cf1[j]);
            }
        }

        // -------- state: h~ += B^T x'  (exact blocks: h~ <- sig_in delta h~ + B^T x')
        if (!bk.fac) {
            const float sd = bk.sig_in * bk.delta;
#pragma unroll
            for (int m = 0; m < 8; ++m) st[m] *= sd;
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) st[m] = Mma<bf16>::mma(bt[m], xs, st[m]);
        sig_out = bk.sig;
        __builtin_amdgcn_sched_barrier(0);

        // -------- while the MFMAs run: the derived decay vectors of block
        // kb + 2 (one wave; visible after this block's barrier) and the
        // bookkeeping of block kb + 1
        if (kb + 2 < nblk && wave == (kb + 2) % NW) vec_store(kb + 2, cur);
        Book bk1 = bk;
        if (kb + 1 < nblk) bk1 = book(kb + 1, bk.sig);

        // -------- the DMAs of the previous block have landed once at most
        // this block's VM_LOADS DMAs are in flight (loads complete in issue
        // order; a pending store only lengthens the wait); then this block's
        // y stores
        __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(S::VM_LOADS));
        __builtin_amdgcn_sched_barrier(0);
        y_store(kb, acc);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        bk = bk1;
    };

    for (int kb = 0; kb < nblk; kb += 3) {
        block(kb, 0);
        if (kb + 1 < nblk) {
            block(kb + 1, 1);
            if (kb + 2 < nblk) block(kb + 2, 2);
        }
    }
    // no DMA may land in LDS after the workgroup ends
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    if (final_state) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const f32x4 hv = st[m] * sig_out;
            *reinterpret_cast<float4 *>(final_state + (bh * P + p0 + 16 * pt + r) * N +
                                        32 * (m >> 1) + 8 * q + 4 * (m & 1)) =
                make_float4(hv[0], hv[1], hv[2], hv[3]);
        }
    }
}

// Diagonal 32x32 block of C B^T for every 32-token block and group, bf16,
// stored in the MFMA fragment order the fused kernel reads: for row tile
// lt and lane (r, q), the 8 values C B^T[16 lt + r][8 q .. 8 q + 7] are the
// 16 bytes at ((lt * 64) + q * 16 + r) * 16.  Entries with column > row
// (the whole tile at rows 0-15, columns 16-31 included) are zero, so the
// block is already causally masked.
// grid (nblk * G, b), 256 threads; wave w < 3 computes tile (0,0), (1,0) or
// (1,1) and scatters it, wave 3 writes the zero tile.
__global__ void __launch_bounds__(256)
k2b_block_cb(const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm, bf16 *__restrict__ cbf,
             int L, int G, int nblk) {
    constexpr int N = 128;
    const int kb = blockIdx.x / G, g = blockIdx.x % G, b = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;
    const int t0 = kb * kBlk;
    bf16 *out = cbf + (((size_t)b * nblk + kb) * G + g) * (kBlk * kBlk);
    // (row tile, column tile) of this wave; wave 3 owns the zero tile (0, 1)
    const int lt = (wave == 0 || wave == 3) ? 0 : 1;
    const int ct = (wave == 2 || wave == 3) ? 1 : 0;
    f32x4 acc = zero4();
    if (wave < 3) {
        const int tl = t0 + 16 * lt + r, ts = t0 + 16 * ct + r;
#pragma unroll
        for (int kk = 0; kk < N; kk += 32) {
            const bf16x8 a = tl < L ? load_frag(Cm + (((size_t)b * L + tl) * G + g) * N + kk + 8 * q)
                                    : zero_frag<bf16>();
            const bf16x8 bb = ts < L ? load_frag(Bm + (((size_t)b * L + ts) * G + g) * N + kk + 8 * q)
                                     : zero_frag<bf16>();
            acc = Mma<bf16>::mma(a, bb, acc);
        }
    }
    // D layout: lane (r, q) holds rows 16 lt + 4 q + e, column 16 ct + r;
    // entries above the diagonal (s > l) are written as exact zeros
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rr = 4 * q + e, s = 16 * ct + r;
        out[(lt * 64 + (s >> 3) * 16 + rr) * 8 + (s & 7)] =
            s <= 16 * lt + rr ? (bf16)acc[e] : (bf16)0.f;
    }
}

// --------------------------------------------------------------------- launch

const char *const kFusedKernelNames[kFusedKernels] = {"k1_dA_cumsum", "k2b_block_cb",
                                                      "k_fused_ssd"};

template <typename T>
bool fused_supported(int P, int N, int Q) {
    (void)Q;
    return sizeof(T) == 2 && N == 128 && P % 32 == 0;
}
template bool fused_supported<float>(int, int, int);
template bool fused_supported<bf16>(int, int, int);

int fused_nblk(int L) { return (L + kBlk - 1) / kBlk; }

template <int PB>
static hipError_t launch_fused_main(const ForwardArgs &a, hipStream_t stream) {
    typedef Fused<PB> S;
    const int nblk = fused_nblk(a.L);
    // the kernel reaches acum_lo and dtT at fixed strides from acum_hi
    if (a.acum_lo - a.acum_hi != a.dtT - a.acum_lo || a.acum_lo <= a.acum_hi)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_fused_ssd<PB>), dim3(a.H * (a.P / PB), a.batch), dim3(S::NT), 0,
                       stream, (const bf16 *)a.x, (const bf16 *)a.B, (const bf16 *)a.C,
                       (const bf16 *)a.cb, a.acum_hi, a.acum_lo, a.dtT, a.D, a.init,
                       a.final_state, (bf16 *)a.y, a.L, a.H, a.G, a.P, nblk);
    return hipSuccess;
}

// Headdim block per workgroup: 64 columns (4 waves) when that still gives at
// least one workgroup per compute unit, else 32 (2 waves) for more of them.
static int pick_pb(const ForwardArgs &a) {
    const long wg64 = (a.P % 64 == 0) ? (long)a.batch * a.H * (a.P / 64) : 0;
    return wg64 >= 256 ? 64 : 32;
}

template <typename T>
hipError_t launch_fused_forward(const ForwardArgs &a, hipStream_t stream, hipEvent_t *events) {
    if (sizeof(T) != 2) return hipErrorInvalidValue;  // bf16 only (fused_supported)
    int ev = 0;
    auto mark = [&]() -> hipError_t {
        return events ? hipEventRecord(events[ev++], stream) : hipSuccess;
    };
    const int nblk = fused_nblk(a.L);
    hipError_t err;
    if ((err = mark()) != hipSuccess) return err;
    launch_dA_cumsum(a.dt, a.A, a.acum_hi, a.acum_lo, a.dtT, a.batch, a.L, a.H, nblk, kBlk,
                     stream);
    if ((err = mark()) != hipSuccess) return err;
    hipLaunchKernelGGL(k2b_block_cb, dim3(nblk * a.G, a.batch), dim3(256), 0, stream,
                       (const bf16 *)a.B, (const bf16 *)a.C, (bf16 *)a.cb, a.L, a.G, nblk);
    if ((err = mark()) != hipSuccess) return err;
    err = pick_pb(a) == 64 ? launch_fused_main<64>(a, stream) : launch_fused_main<32>(a, stream);
    if (err != hipSuccess) return err;
    if ((err = mark()) != hipSuccess) return err;
    return hipGetLastError();
}

template hipError_t launch_fused_forward<float>(const ForwardArgs &, hipStream_t, hipEvent_t *);
template hipError_t launch_fused_forward<bf16>(const ForwardArgs &, hipStream_t, hipEvent_t *);

}  // namespace ssd
