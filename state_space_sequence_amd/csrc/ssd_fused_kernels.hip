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
// sigma instead of the 128 x 32 state tile of every wave:
//   x'_s  = exp(lambda_e - lambda_s) dt_s x_s / sigma_{k+1}     (bf16)
//   y_l   = exp(lambda_l - lambda_e) sigma_{k+1} (C_l h~^T + [C B^T]_l x') + D x_l
//   h~   += B^T x'
// with sigma_{k+1} = sigma_k exp(lambda_e).  When sigma_{k+1} would fall
// below exp(-60) the scale restarts in that block (h~ *= sigma_k, sigma_k =
// 1, so sigma_{k+1} = exp(lambda_e) >= exp(-60) in a factored block): 1/sigma
// stays below exp(60) and every intermediate far inside the fp32 range.
//
// The diagonal block uses the factored weights exp(lambda_l - lambda_e) (up
// to exp(60)) and exp(lambda_e - lambda_s) (down to exp(-60), so x' keeps
// bf16's relative precision as long as |x_s| dt_s exceeds about 1e-12) only
// when the block's total decay is at most exp(-60).  Beyond that the block is
// evaluated with the exact per-element weights exp(lambda_l - lambda_s) dt_s
// (s > l exactly 0, the upper-triangle protection of the Kernel 5 page) on
// raw x, with D on the diagonal, and the state decays explicitly
// (h~ <- sigma_k exp(lambda_e) h~ + B^T x', sigma = 1).  The per-token
// factors come precomputed per block (k_prep, from fp64 prefixes).
//
// Workgroup = NW = PB / 32 waves; wave w owns headdim columns 32 w .. 32 w +
// 31 of the workgroup's PB columns and computes with
// v_mfma_f32_32x32x16_bf16.  Per 32-token block:
//   stage  three LDS stages filled by buffer-resource DMA two blocks ahead:
//          C and B rows (swizzled), the causal diagonal block of C B^T
//          (precomputed, in fragment order), raw x (swizzled) and the
//          block's decay record;
//   output y^T = h~ C^T + x'^T [C B^T]^T for the wave's 32 columns and the
//          block's 32 tokens, with h~ taken straight from the state
//          registers as the MFMA A operand; each lane ends with 4 runs of 4
//          consecutive headdim values of one token (four 8-byte stores);
//   state  h~ += B^T x'.
//
// Operands that the MFMA needs transposed (B^T, x'^T) are read from
// row-major LDS with ds_read_b64_tr_b16: within each 16-lane group, lane 4a+c
// receives element c of the 8-byte reads of lanes a, a+4, a+8, a+12, so
// pointing lane a + 4 e at row kbase + e and 4 consecutive columns of a
// row-major [k][n] tile hands those 4 columns to lanes 4a .. 4a+3.
#include <stdlib.h>
#include <string.h>

#include "ssd_device.hpp"
#include "ssd_kernels.hpp"

namespace ssd {

constexpr int kBlk = 32;                  // tokens per block
constexpr float kSafeDecay = 60.f;        // max -lambda_e for the factored diagonal
constexpr float kRescale = 8.75651076e-27f;  // exp(-60): smallest sigma kept unrescaled
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
// 16-byte chunk swizzle of the C / B rows and of the raw x rows in LDS (XOR
// on the chunk index; depends on row & 7 only).  It is a bijection on
// row & 7, so the fragment reads of 8 consecutive rows (one chunk each) hit 8
// distinct bank groups, and its bits 1-2 are row & 3, so the transposed reads
// (4 consecutive rows x one aligned 32-byte window each) land in 4 distinct
// 32-byte bank windows.
__device__ __forceinline__ int row_swz(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }
// raw x rows of 64 bytes (4 chunks): the same two properties
__device__ __forceinline__ int row_swz4(int row) { return 2 * ((row >> 1) & 1) + ((row >> 2) & 1); }

// Workgroup layout.  A workgroup covers PB consecutive columns of one
// batch's flattened (head, headdim) columns h P + p (x and y rows are
// contiguous over them): NW = PB / 32 waves of 32 columns each.  With
// PB > P the workgroup spans NH = PB / P heads of one B/C group, which then
// share the staged C and B rows.
template <int PB>
struct Fused {
    static constexpr int NW = PB / 32;                 // compute waves: 32 headdim columns each
    // One more wave (the producer) issues every global memory operation of
    // the workgroup: the DMAs of the stages and the y stores, which the
    // compute waves hand over through LDS.  The compute waves never wait on
    // the vector memory pipeline.
    static constexpr int NT = 64 * (NW + 1);           // threads
    static constexpr int N = 128;                      // dstate
    static constexpr int ROWB = 2 * N;                 // bytes per C / B row
    static constexpr int MAT = kBlk * ROWB;            // 8 KB per matrix
    static constexpr int XC = PB / 8;                  // 16-byte chunks per x row
    static constexpr int XRB = 2 * PB;                 // raw x row bytes
    static constexpr int NRS = PB == 128 ? 2 : 1;      // decay-record slots (heads)
    // one stage: C rows, B rows (column-blocked, blk_off), raw x
    // (column-blocked) and the decay records (kVecRec floats in 1 KB slots)
    // of one block, filled by DMA; the causal diagonal block of C B^T in the
    // MFMA B-fragment order, formed by the producer from the stage's C and B
    // rows; then the block's y for the producer: 32 rows of XRB bytes,
    // 16-byte chunk c of row t in slot c ^ ys_swz(t)
    static constexpr int CS = 0;
    static constexpr int BS = MAT;
    static constexpr int CBF = 2 * MAT;                // 2 x 1 KB of C B^T fragments
    static constexpr int XR = CBF + 2048;
    static constexpr int VR = XR + kBlk * XRB;
    static constexpr int YS = VR + 1024 * NRS;
    static constexpr int STG = YS + kBlk * XRB;
    // floats of the decay record
    enum { CF = 0, RP = 32, LR = 64, DT = 96, DELTA = 128, FLAG = 129, LE = 130 };
    // four stages: the DMAs of a block go out three blocks ahead of its
    // use, and a block's stage is complete one block early: the producer
    // forms its C B^T block and the compute waves read its opening operands
    // during the block before it
    static constexpr int NST = 4;
    // K-step rows m of the C fragments among the opening operands (within
    // the 256 registers per lane that two waves on a SIMD leave each)
    static constexpr int ECF = PB == 128 ? 1 : 2;
    static constexpr int LDS = NST * STG;
    static_assert(PB == 32 || PB == 64 || PB == 128, "one, two or four waves");
    static_assert(STG % 16 == 0, "alignment");
    // (one workgroup per compute unit, which the column choice arranges)
    static_assert(LDS <= 160 * 1024, "LDS per compute unit");
    // the producer's DMAs of a block (C and B, x, records) and y stores.  At
    // the end of block kb it waits for the DMAs of block kb + 2; younger
    // than those are the y stores issued right after them and the DMAs and
    // y stores of block kb + 3
    static constexpr int P_LOADS = 2 * (MAT / 1024) + kBlk * XRB / 1024 + NRS;
    static constexpr int P_STORES = kBlk * XRB / 1024;
    static constexpr int P_WAIT = P_STORES + (NST - 3) * (P_LOADS + P_STORES);
    static_assert(P_WAIT < 64, "vmcnt immediate");
};

template <int PB>
__device__ __forceinline__ int x_swz(int row) { return PB >= 64 ? row_swz(row) : row_swz4(row); }

// Column-blocked LDS layout of the staged C, B and x tiles (32 rows): the
// 16-byte chunk c of row t sits at byte blk_off(t, c), so each block of four
// chunks (32 bf16 columns) is a 2 KB region of 32 rows x 64 bytes, and the
// chunks of a row are rotated by an XOR with (t / 4) % 4.  Over the 64-bank
// LDS (256 bytes per cycle) the fragment reads (16 consecutive rows, one
// chunk each) then hit 16 distinct 16-byte bank groups, the transposed reads
// (4 consecutive rows from a multiple of 4, the same 2 or 4 chunks each) hit
// distinct ones too, and moving to another column block or 16 rows further
// is a constant offset (2048 and 1024 bytes).
__device__ __forceinline__ int blk_off(int t, int c) {
    return 2048 * (c >> 2) + 64 * t + 16 * ((c & 3) ^ ((t >> 2) & 3));
}
// Staging slot of chunk c of y row t (XC chunks per row, rows contiguous):
// c ^ ys_swz(t) spreads 16 consecutive rows over distinct bank groups.
template <int XC>
__device__ __forceinline__ int ys_swz(int t) { return (t / (16 / XC)) & (XC - 1); }

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
// The barrier at the end of a block: every LDS read of the block has been
// consumed by then (the compiler's waits precede each use), so no LDS wait
// is needed before it; an lgkmcnt(0) here would also wait for this block's
// DMAs into LDS still in flight (they count on that counter as well).
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Scale bookkeeping of one block (identical in every wave of a head).
struct Book {
    float sig_in;   // sigma entering the block
    float sig;      // sigma after the block
    float delta;    // exp(lambda_e)
    bool fac;       // factored diagonal
    bool rescale;   // restart the scale: h~ *= sig_in, sigma_in = 1 (factored blocks only)
};

// Bookkeeping of a block from its decay record's delta and factored flag
// (the same in every lane) and the sigma entering it.
__device__ __forceinline__ Book book_of(float dl, float fc, float sig_in) {
    Book bk;
    bk.sig_in = sig_in;
    bk.delta = uniform(dl);
    bk.fac = uniform(fc) != 0.f;
    const float p = sig_in * bk.delta;
    bk.rescale = bk.fac && p < kRescale;
    bk.sig = bk.fac ? (bk.rescale ? bk.delta : p) : 1.f;
    return bk;
}
__device__ __forceinline__ Book book_of(const float *rec, float sig_in) {
    return book_of(rec[kVecRec - 4], rec[kVecRec - 3], sig_in);
}

// MFMA operands of v_mfma_f32_32x32x16_bf16: lane l holds row (A) / column
// (B) l % 32 and k = 8 (l / 32) + j, j = 0..7; result register v of lane l
// is D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Column of MFMA row / column q (0..31) within a wave's 32 headdim columns.
// Output row q = 8 i + 4 hi + c of y^T lands in result register 4 i + c of
// the lanes with l / 32 = hi; with this order those registers hold, in
// order, 16 columns that form two runs of 8: 8 hi + (0..7) and
// 16 + 8 hi + (0..7).  A lane then stores 16 contiguous bytes per run, and
// one store instruction covers 32 contiguous bytes of each token.
__device__ __forceinline__ int col_of(int q) {
    return 8 * ((q >> 2) & 1) + 4 * ((q >> 3) & 1) + 16 * (q >> 4) + (q & 3);
}

// Per wave: flattened columns c0 + 32 wave + (0..31) of head hw, headdim
// columns pw + (0..31).  With lane l, r = l % 32, hi = l / 32, and
// pr = pw + col_of(r):
//   state     st[m][v] = h~[n][pr],  i = v / 4, c = v % 4,
//             n = 32 m + 16 (i / 2) + 8 hi + 4 (i % 2) + c
//             so st[m][8u .. 8u+7] are n = 32 m + 16 u + 8 hi + 0..7, the A
//             fragment of K-step (m, u) of y^T = h~ C^T;
//   output    acc[v] = y[token r][pw + col_of(8 i + 4 hi + c)]: acc[0..7]
//             are columns pw + 8 hi + (0..7), acc[8..15] are columns
//             pw + 16 + 8 hi + (0..7);
//   x'        xs[kk] = x'[token 16 kk + 8 hi + j][pr] (the A fragment of
//             the diagonal block and the B fragment of the state update,
//             K-step kk).
template <int PB>
__global__ void __launch_bounds__(Fused<PB>::NT)
k_fused_ssd(const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
            const float *__restrict__ vrec,
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
    __shared__ __align__(16) unsigned char stg3[S::NST > 3 ? S::STG : 16];

    const int HP = H * P, GN = G * N;
    const int c0 = blockIdx.x * PB, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = (c0 / P) / (H / G);          // the workgroup's B / C group

    auto stage = [&](int i) -> unsigned char * {
        return i == 0 ? stg0 : (i == 1 ? stg1 : (i == 2 ? stg2 : stg3));
    };

    if (wave == NW) {
        // ---- the producer wave: every DMA of the stages and every y store.
        // Buffer resources over the workgroup's slices of C, B, x, the C B^T
        // blocks, the decay records and y, built once; a block adds its byte
        // offset to fixed per-lane offsets.  Rows past the end of the
        // sequence (the ragged tail, and the prefetches past the last block)
        // fall outside a resource's range: the hardware reads them as zeros
        // and drops such stores.
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Cm + (size_t)b * L * GN + (size_t)g * N), 0, (L * GN - g * N) * 2, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Bm + (size_t)b * L * GN + (size_t)g * N), 0, (L * GN - g * N) * 2, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(x + (size_t)b * L * HP + c0), 0, (L * HP - c0) * 2, kBufferWord3);
        // the records of the workgroup's heads (consecutive (batch, head) rows)
        const int h0 = c0 / P;
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vrec + ((size_t)b * H + h0) * nblk * kVecRec), 0, S::NRS * nblk * kVecRec * 4,
            kBufferWord3);
        const __amdgpu_buffer_rsrc_t y_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            y + (size_t)b * L * HP, 0, L * HP * 2, kBufferWord3);
        const unsigned cb_step = kBlk * GN * 2, x_step = kBlk * HP * 2;
        const unsigned v_step = kVecRec * 4;
        typedef __attribute__((address_space(3))) void lds_void;
        // (the block's byte offset goes in the scalar offset, so a DMA
        // costs no vector instruction)
        auto bdma = [](__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff, unsigned char *dst) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, voff, soff, 0, 0);
        };
        // Per-lane offsets.  DMA i fills the 1 KB at 1024 i of a
        // column-blocked tile: column block i / 2, rows 16 (i % 2) + lane / 4,
        // slot lane % 4 (so chunk 4 (i / 2) + ((lane % 4) ^ ((t / 4) % 4)) of
        // row t).  Store i takes y row (64 i + lane) / XC, chunk
        // (64 i + lane) % XC.
        constexpr int NCB = S::MAT / 1024, NXD = kBlk * S::XRB / 1024;
        unsigned pcb[NCB], px[NXD];
#pragma unroll
        for (int i = 0; i < NCB; ++i) {
            const int t = 16 * (i & 1) + (lane >> 2);
            pcb[i] = t * GN * 2 + 16 * (4 * (i >> 1) + ((lane & 3) ^ ((t >> 2) & 3)));
        }
#pragma unroll
        for (int i = 0; i < NXD; ++i) {
            const int t = 16 * (i & 1) + (lane >> 2);
            px[i] = t * HP * 2 + 16 * (4 * (i >> 1) + ((lane & 3) ^ ((t >> 2) & 3)));
        }
        auto pdma = [&](int kb, unsigned char *buf) {
            const unsigned cbo = kb * cb_step, xo = kb * x_step, vo = kb * v_step;
#pragma unroll
            for (int i = 0; i < NCB; ++i) {
                bdma(rc, pcb[i], cbo, buf + S::CS + 1024 * i);
                bdma(rb, pcb[i], cbo, buf + S::BS + 1024 * i);
            }
#pragma unroll
            for (int i = 0; i < NXD; ++i) bdma(rx, px[i], xo, buf + S::XR + 1024 * i);
#pragma unroll
            for (int q = 0; q < S::NRS; ++q)
                bdma(rv, 16 * lane + q * nblk * v_step, vo, buf + S::VR + 1024 * q);
        };
        // The causal diagonal block of C B^T of the block staged in `buf`,
        // from its C and B rows: E = B C^T on MFMA (A: B row s = lane % 32,
        // B: C row l = lane % 32, K-step ks over dstate 16 ks .. 16 ks + 15),
        // so lane (r, hi) ends with E[s][r] = C_r . B_s for s = 8 i + 4 hi + c;
        // entries with s > r are exact zeros.  Written in the fragment order
        // of the diagonal product: K-step kk, lane L hold the 8 values
        // C B^T[L % 32][16 kk + 8 (L / 32) .. +7] as the 16 bytes at
        // CBF + (64 kk + L) * 16.
        const int pr_ = lane & 31, phi = lane >> 5;
        int pc_rd[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) pc_rd[u] = blk_off(pr_, 2 * u + phi);
        auto pcbt = [&](unsigned char *buf) {
            f32x16 e;
#pragma unroll
            for (int v = 0; v < 16; ++v) e[v] = 0.f;
            bf16x8 fb[8], fc[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                fb[ks] = lds_b128(buf, S::BS + pc_rd[ks & 1] + 2048 * (ks >> 1));
                fc[ks] = lds_b128(buf, S::CS + pc_rd[ks & 1] + 2048 * (ks >> 1));
            }
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) e = mma32(fb[ks], fc[ks], e);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s0 = 8 * i + 4 * phi;
                bf16x4 v4;
#pragma unroll
                for (int c = 0; c < 4; ++c) v4[c] = s0 + c <= pr_ ? (bf16)e[4 * i + c] : (bf16)0.f;
                const int kk = s0 >> 4, hs = (s0 >> 3) & 1;
                *reinterpret_cast<bf16x4 *>(buf + S::CBF + ((64 * kk + pr_ + 32 * hs) * 8 + (s0 & 7)) * 2) = v4;
            }
        };
        // per-lane y offsets and LDS staging slots of the stores
        unsigned py[S::P_STORES];
        int pys[S::P_STORES];
#pragma unroll
        for (int i = 0; i < S::P_STORES; ++i) {
            const int pos = 64 * i + lane, t = pos / S::XC, c = pos % S::XC;
            py[i] = (t * HP + c0 + 8 * c) * 2;
            pys[i] = S::YS + t * S::XRB + 16 * (c ^ ys_swz<S::XC>(t));
        }
        auto pstore = [&](int kb, const unsigned char *buf) {
            const unsigned yo = kb * kBlk * HP * 2;
#pragma unroll
            for (int i = 0; i < S::P_STORES; ++i) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(buf + pys[i]);
                __builtin_amdgcn_raw_buffer_store_b128(v, y_rsrc, py[i], yo, 0);
            }
        };
#pragma unroll
        for (int i = 0; i < S::NST - 1; ++i) pdma(i, stage(i));
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        pcbt(stage(0));
        lds_barrier();
        // block kb: refill the stage block kb - 1 used, store its y, form
        // the C B^T block of block kb + 1, then wait for the DMAs of block
        // kb + 2 before the end-of-block barrier
        auto pblock = [&](int kb, const int si) {
            pdma(kb + S::NST - 1, stage((si + S::NST - 1) % S::NST));
            if (kb > 0) pstore(kb - 1, stage((si + S::NST - 1) % S::NST));
            pcbt(stage((si + 1) % S::NST));
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(S::P_WAIT));
            lds_barrier();
        };
        for (int kb = 0; kb < nblk; kb += S::NST) {
            pblock(kb, 0);
            if (kb + 1 < nblk) {
                pblock(kb + 1, 1);
                if (kb + 2 < nblk) {
                    pblock(kb + 2, 2);
                    if constexpr (S::NST > 3) {
                        if (kb + 3 < nblk) pblock(kb + 3, 3);
                    }
                }
            }
        }
        pstore(nblk - 1, stage((nblk - 1) % S::NST));
        // no DMA may land in LDS after the workgroup ends
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        return;
    }

    const int r = lane & 31, hi = lane >> 5;
    const int cw = c0 + 32 * wave;             // this wave's first flattened column
    const int hw = cw / P, pw = cw - hw * P;   // its head and headdim column
    const int slot = (cw - c0) / (PB > P ? P : PB);  // its decay-record slot
    const size_t bh = (size_t)b * H + hw;
    const float Dh = D ? D[hw] : 0.f;

    // ---- per-lane LDS byte offsets (lane = 16 grp + a + 4 e for the
    // transposed reads, which act within each 16-lane group)
    const int a4 = lane & 3, e4 = (lane >> 2) & 3, g1 = (lane >> 4) & 1;
    // C fragment of K-step (m, u): token r, chunk 4 m + 2 u + hi:
    //   CS + c_rd[u] + 2048 m
    int c_rd[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) c_rd[u] = blk_off(r, 2 * u + hi);
    // B^T, state tile m, K-step kk, token half s: token 16 kk + 8 hi + 4 s + e4,
    // n-quad 8 m + 4 g1 + 2 (a4 & 1) + (a4 >> 1):
    //   BS + b_tr[s] + 2048 m + 1024 kk
    int b_tr[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        b_tr[s] = blk_off(8 * hi + 4 * s + e4, 2 * g1 + (a4 & 1)) + 8 * (a4 >> 1);
    // x^T fragment of K-step kk, token half s: token 16 kk + 8 hi + 4 s + e4,
    // for lanes 16 g1 + 4 a4 + (0..3) (MFMA columns q = 16 g1 + 4 a4 + c)
    // the wave's columns 16 g1 + 8 (a4 & 1) + 4 (a4 >> 1) + (0..3) =
    // col_of(q):  XR + xs_tr[s] + 1024 kk
    int xs_tr[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        xs_tr[s] = blk_off(8 * hi + 4 * s + e4, 4 * wave + 2 * g1 + (a4 & 1)) + 8 * (a4 >> 1);
    // raw x of the skip term: token r, the wave's columns 8 hi + (0..7) and
    // 16 + 8 hi + (0..7)
    int xr_skip[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) xr_skip[i] = blk_off(r, 4 * wave + 2 * i + hi);
    const int pr = pw + col_of(r);
    const int cbf_rd = lane * 16;
    const int rec_off = S::VR + 1024 * slot;

    // ---- register-resident scaled state
    f32x16 st[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int v = 0; v < 16; ++v) st[m][v] = 0.f;
        if (init) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 32 * m + 16 * (i >> 1) + 8 * hi + 4 * (i & 1);
                const float4 q4 = *reinterpret_cast<const float4 *>(init + (bh * P + pr) * N + n);
                st[m][4 * i] = q4.x;
                st[m][4 * i + 1] = q4.y;
                st[m][4 * i + 2] = q4.z;
                st[m][4 * i + 3] = q4.w;
            }
        }
    }

    // staging slots of this lane's two 16-byte runs of y (row r, chunks
    // 4 wave + 2 i + hi of the workgroup's row)
    int ys_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        ys_off[i] = S::YS + r * S::XRB + 16 * ((4 * wave + 2 * i + hi) ^ ys_swz<S::XC>(r));
    auto y_stage = [&](unsigned char *cur, const f32x16 &acc) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4 v = {pack2(acc[8 * i], acc[8 * i + 1]), pack2(acc[8 * i + 2], acc[8 * i + 3]),
                             pack2(acc[8 * i + 4], acc[8 * i + 5]), pack2(acc[8 * i + 6], acc[8 * i + 7])};
            *reinterpret_cast<u32x4 *>(cur + ys_off[i]) = v;
        }
    };

    // ---- prologue: the producer's DMAs of the first blocks have landed
    lds_barrier();
    float sig_out = 1.f;  // sigma after the previous block

    // The operands that open a block (read from its stage during the block
    // before): the decay-record fields of the bookkeeping, cf and
    // exp(lambda_r - lambda_e), raw x^T and the C fragments of the first
    // 2 ECF K-steps.
    constexpr int ECF = S::ECF;
    struct Early {
        f32x4 cfv[4];        // cf of tokens 16 kk + 8 hi + 0..7
        bf16x8 xs[2];        // raw x^T, K-steps 0 and 1
        bf16x8 cfr[ECF][2];  // C fragments of y^T = h~ C^T, K-steps (m, u), m < ECF
        float rpv;           // exp(lambda_r - lambda_e)
        float dl, fc;        // the record's delta and factored flag (uniform)
    };
    // The rest of a block's operands, read from its stage during the block.
    struct Ops {
        bf16x8 cfr[4 - ECF][2];  // C fragments, K-steps (m, u), m >= ECF
        bf16x8 cbv[2];     // causal diagonal block of C B^T, K-steps 0 and 1
        bf16x8 bt[4][2];   // B^T fragments of the state update, tile m, K-step kk
        bf16x8 xr[2];      // raw x of the skip term (read for the epilogue)
    };
    auto load_early = [&](const unsigned char *buf, Early &e) {
        const float *v = reinterpret_cast<const float *>(buf + rec_off);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int w4 = 0; w4 < 2; ++w4)
                e.cfv[2 * kk + w4] =
                    *reinterpret_cast<const f32x4 *>(v + S::CF + 16 * kk + 8 * hi + 4 * w4);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            e.xs[kk] = join(lds_tr(buf, S::XR + xs_tr[0] + 1024 * kk),
                            lds_tr(buf, S::XR + xs_tr[1] + 1024 * kk));
#pragma unroll
        for (int m = 0; m < ECF; ++m)
#pragma unroll
            for (int u = 0; u < 2; ++u) e.cfr[m][u] = lds_b128(buf, S::CS + c_rd[u] + 2048 * m);
        e.rpv = v[S::RP + r];
        e.dl = v[S::DELTA];
        e.fc = v[S::FLAG];
    };
    auto load_late = [&](const unsigned char *cur, Ops &o) {
#pragma unroll
        for (int m = ECF; m < 4; ++m)
#pragma unroll
            for (int u = 0; u < 2; ++u) o.cfr[m - ECF][u] = lds_b128(cur, S::CS + c_rd[u] + 2048 * m);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) o.cbv[kk] = lds_b128(cur, S::CBF + 1024 * kk + cbf_rd);
    };
    // B^T fragment q = 2 m + kk of the state update (read during y^T = h~ C^T)
    auto load_bt = [&](const unsigned char *cur, Ops &o, int q) {
        const int m = q >> 1, kk = q & 1;
        const int off = 2048 * m + 1024 * kk;
        o.bt[m][kk] = join(lds_tr(cur, S::BS + b_tr[0] + off), lds_tr(cur, S::BS + b_tr[1] + off));
    };

    // block kb from stage si = kb % NST (a literal in each unrolled copy);
    // e holds its opening operands, nx receives those of block kb + 1
    auto block = [&](int kb, const int si, Early &e, Early &nx) {
        unsigned char *cur = stage(si);
        const float *v = reinterpret_cast<const float *>(cur + rec_off);
        // The block is written as a sequence of chunks fenced by scheduling
        // barriers: each chunk starts one MFMA and then issues vector work
        // that does not depend on it (the next state conversion and x'
        // during y^T = h~ C^T; the epilogue and the reads of the next
        // block's opening operands during the state update), so ALU and LDS
        // issue overlap the matrix pipeline.  A rescaled or exact block edits
        // the operands of the common path in place between the two phases.
        Ops o;
        load_late(cur, o);
        const Book bk = book_of(e.dl, e.fc, sig_out);
        const float xscale = bk.fac ? __builtin_amdgcn_rcpf(bk.sig) : 1.f;
        auto hb_of = [&](int q) {  // bf16 A fragment of K-step q = 2 m + u
            bf16x8 hb;
#pragma unroll
            for (int j = 0; j < 8; ++j) hb[j] = (bf16)st[q >> 1][8 * (q & 1) + j];
            return hb;
        };
        // x' / sigma (the state update operand; also the diagonal operand
        // in a factored block), two values per chunk
        bf16x8 xp[2];
        auto xp_part = [&](int q) {
#pragma unroll
            for (int ee = 0; ee < 2; ++ee) {
                const int kk = q >> 2, j = 2 * (q & 3) + ee;
                xp[kk][j] = (bf16)((float)e.xs[kk][j] * (e.cfv[2 * kk + (j >> 2)][j & 3] * xscale));
            }
        };
        f32x16 acc;
#pragma unroll
        for (int v16 = 0; v16 < 16; ++v16) acc[v16] = 0.f;
        bf16x8 hb = hb_of(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            acc = mma32(hb, (q >> 1) < ECF ? e.cfr[(q >> 1) % ECF][q & 1]
                                           : o.cfr[((q >> 1) - ECF) & 3][q & 1], acc);
            __builtin_amdgcn_sched_barrier(0);
            if (q < 7) hb = hb_of(q + 1);
            xp_part(q);
            load_bt(cur, o, q);
            __builtin_amdgcn_sched_barrier(0);
        }
        // (the empty asm consumes x' here, so no pass sinks its arithmetic
        // out of the chunks above)
        asm volatile("" : "+v"(xp[0]), "+v"(xp[1]));
        float f = e.rpv * bk.sig, dco = Dh;
        if (bk.rescale) {
            // restart of the scale (sigma would fall below exp(-60)): the
            // state and its output so far move to sigma_in = 1
            __builtin_amdgcn_sched_barrier(0);
            acc *= bk.sig_in;
#pragma unroll
            for (int m = 0; m < 4; ++m) st[m] *= bk.sig_in;
        }
        if (!bk.fac) {
            // (a side effect keeps the compiler from evaluating this rare
            // branch unconditionally with selects)
            __builtin_amdgcn_sched_barrier(0);
            // exact block: weights exp(lambda_l - lambda_s) dt_s on raw x with
            // D on the diagonal; h~ <- sigma_in delta h~ + B^T x', sigma = 1.
            // exp(lambda_r) sigma_in (<= 1: the exponent is formed before exp)
            acc *= fast_exp(v[S::LR + r] + v[S::LE]) * bk.sig_in;
            const float lr = v[S::LR + r];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 wgt;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = 16 * kk + 8 * hi + j;
                    const float w = (float)o.cbv[kk][j] * fast_exp(fminf(lr - v[S::LR + s], 0.f)) *
                                        v[S::DT + s] + (s == r ? Dh : 0.f);
                    wgt[j] = (bf16)(s <= r ? w : 0.f);
                }
                acc = mma32(e.xs[kk], wgt, acc);
                // the common diagonal product below then adds zeros
                o.cbv[kk] = zero_frag<bf16>();
            }
            f = 1.f;
            dco = 0.f;
            const float sd = bk.sig_in * bk.delta;
#pragma unroll
            for (int m = 0; m < 4; ++m) st[m] *= sd;
        }
        __builtin_amdgcn_sched_barrier(0);
        // (raw x of the skip term, read here for the epilogue)
#pragma unroll
        for (int i = 0; i < 2; ++i) o.xr[i] = lds_b128(cur, S::XR + xr_skip[i]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) acc = mma32(xp[kk], o.cbv[kk], acc);
        __builtin_amdgcn_sched_barrier(0);
        // state update h~ += B^T x' (K-step 0 of every tile, then K-step 1),
        // with the reads of the next block's opening operands and the
        // epilogue (from the third chunk on, once the diagonal product has
        // landed)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int kk = q >> 2, m = q & 3;
            st[m] = mma32(o.bt[m][kk], xp[kk], st[m]);
            __builtin_amdgcn_sched_barrier(0);
            if (q == 0) load_early(stage((si + 1) % S::NST), nx);
            if (q >= 2) {
                // acc[vv] for the vv with vv * 6 / 16 == q - 2 (the
                // empty asm keeps them in this chunk)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv)
                    if (vv * 6 / 16 == q - 2)
                        acc[vv] = acc[vv] * f + dco * (float)o.xr[vv >> 3][vv & 7];
                asm volatile("" : "+v"(acc));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("" : "+v"(acc));
        sig_out = bk.sig;
        __builtin_amdgcn_sched_barrier(0);
        // y of the block to the producer through this stage's staging rows;
        // the barrier then also publishes it
        y_stage(cur, acc);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
    };

    // unrolled by the stage count, so that every stage address is a literal
    // (and the two sets of opening operands alternate)
    Early ea, eb;
    load_early(stage(0), ea);
    for (int kb = 0; kb < nblk; kb += S::NST) {
        block(kb, 0, ea, eb);
        if (kb + 1 < nblk) {
            block(kb + 1, 1, eb, ea);
            if (kb + 2 < nblk) {
                block(kb + 2, 2, ea, eb);
                if constexpr (S::NST > 3) {
                    if (kb + 3 < nblk) block(kb + 3, 3, eb, ea);
                }
            }
        }
    }

    if (final_state) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 32 * m + 16 * (i >> 1) + 8 * hi + 4 * (i & 1);
                *reinterpret_cast<float4 *>(final_state + (bh * P + pr) * N + n) =
                    make_float4(st[m][4 * i] * sig_out, st[m][4 * i + 1] * sig_out,
                                st[m][4 * i + 2] * sig_out, st[m][4 * i + 3] * sig_out);
            }
    }
}

// ------------------------------------------------------------------------
// The same pass with 16 headdim columns per wave on v_mfma_f32_16x16x32_bf16
// (operands: lane l holds row (A) / column (B) l % 16 and k = 8 (l / 16) + j,
// j = 0..7; result register v of lane l is D[4 (l / 16) + v][l % 16]).  A
// workgroup of NW = PB / 16 waves covers PB columns of one head, so twice as
// many waves share the work of a head: with two of them on a SIMD, one
// wave's vector ALU work issues while the other waits, which a single wave
// per SIMD cannot do.
//
// Per wave: headdim columns pw + (0..15), pw = p0 + 16 wave.  With lane l,
// r = l % 16, g = l / 16:
//   state     st[mt][v] = h~[n][pw + r], n = 32 (mt / 2) + 8 g + 4 (mt % 2) + v
//             (the state update's row order), so st[2 kk] and st[2 kk + 1]
//             together hold n = 32 kk + 8 g + (0..7): the A fragment of
//             K-step kk of y^T = h~ C^T;
//   output    acc[tt][v] = y[token 16 tt + r][pw + 4 g + v];
//   x'        xs = x'[token 8 g + j][pw + r] (the A fragment of the diagonal
//             block and the B fragment of the state update).
template <int PB>
struct Fused16 {
    static constexpr int NW = PB / 16;                 // waves: 16 headdim columns each
    static constexpr int NT = 64 * NW;
    static constexpr int N = 128;
    static constexpr int ROWB = 2 * N;
    static constexpr int MAT = kBlk * ROWB;
    static constexpr int CBD = MAT / 1024 / NW;        // DMAs per matrix and wave
    static constexpr int XC = PB / 8;                  // 16-byte chunks per x row
    static constexpr int XRB = 2 * PB;
    static constexpr int XD = kBlk * XRB / 1024 / NW;  // x DMAs per wave (one)
    static constexpr int MISC = (3 + NW - 1) / NW;     // C B^T halves and the record
    static constexpr int CS = 0;
    static constexpr int BS = MAT;
    static constexpr int CBF = 2 * MAT;
    static constexpr int XR = CBF + 2048;
    static constexpr int VR = XR + kBlk * XRB;
    static constexpr int STG = VR + 1024;
    enum { CF = 0, RP = 32, LR = 64, DT = 96, DELTA = 128, FLAG = 129, LE = 130 };
    static constexpr int LDS = 3 * STG;
    static constexpr int VM_LOADS = 2 * CBD + XD + MISC;
    static constexpr int Y_STORES = 2;
    static_assert(PB == 32 || PB == 64, "two or four waves");
    static_assert(XD == 1, "x DMAs");
    static_assert(2 * LDS <= 160 * 1024, "two workgroups per compute unit");
    static_assert(VM_LOADS + Y_STORES < 64, "vmcnt immediate");
};

__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int PB>
__global__ void __launch_bounds__(64 * (PB / 16))
k_fused16_ssd(const bf16 *__restrict__ x, const bf16 *__restrict__ Bm,
              const bf16 *__restrict__ Cm, const bf16 *__restrict__ cbf,
              const float *__restrict__ vrec, const float *__restrict__ D, const float *init,
              float *final_state, bf16 *__restrict__ y, int L, int H, int G, int P, int nblk) {
    typedef Fused16<PB> S;
    constexpr int NW = S::NW, N = S::N;
    __shared__ __align__(16) unsigned char stg0[S::STG];
    __shared__ __align__(16) unsigned char stg1[S::STG];
    __shared__ __align__(16) unsigned char stg2[S::STG];

    const int HP = H * P, GN = G * N;
    const int npb = P / PB;
    const int pb = blockIdx.x % npb, h = blockIdx.x / npb, b = blockIdx.y;
    const int g_grp = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int p0 = pb * PB, pw = p0 + 16 * wave;
    const size_t bh = (size_t)b * H + h;
    const float Dh = D ? D[h] : 0.f;

    // ---- per-lane LDS byte offsets (transposed reads: within each 16-lane
    // group, lane 4 a + c receives element c of the 8-byte reads of lanes a,
    // a + 4, a + 8, a + 12; here a = lane & 3, e = (lane >> 2) & 3 is the
    // reading lane's k offset)
    const int a4 = lane & 3, e4 = (lane >> 2) & 3;
    // C fragment (tt, kk): token 16 tt + r, chunk 4 kk + g:
    //   CS + c_rd[kk & 1] + 4096 tt + 128 (kk >> 1)
    int c_rd[2];
    {
        const int sw = row_swz(r);
#pragma unroll
        for (int k1 = 0; k1 < 2; ++k1) c_rd[k1] = r * S::ROWB + 16 * ((4 * k1 + g) ^ sw);
    }
    // B^T fragment of state tile mt (rows n = 32 (mt / 2) + 8 a + 4 (mt % 2)
    // + c for the lanes 4 a + c), read half hh: token 8 g + 4 hh + e4:
    //   BS + b_tr[hh][(mt >> 1) & 1] + 128 (mt >> 2) + 8 (mt & 1)
    int b_tr[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int q1 = 0; q1 < 2; ++q1) {
            const int t = 8 * g + 4 * hh + e4;
            b_tr[hh][q1] = t * S::ROWB + 16 * ((4 * q1 + a4) ^ row_swz(t));
        }
    auto xr_off = [](int t, int c) { return t * S::XRB + 16 * (c ^ x_swz<PB>(t)); };
    // x^T fragment, read half hh: token 8 g + 4 hh + e4, columns
    // 16 wave + 4 a4 .. +3:  XR + xs_tr[hh]
    int xs_tr[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
        xs_tr[hh] = xr_off(8 * g + 4 * hh + e4, 2 * wave + (a4 >> 1)) + 8 * (a4 & 1);
    // raw x of the skip term: token 16 tt + r, columns 16 wave + 4 g .. +3
    int xr_skip[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) xr_skip[tt] = xr_off(16 * tt + r, 2 * wave + (g >> 1)) + 8 * (g & 1);
    const int cbf_rd = lane * 16;

    // ---- register-resident scaled state
    f32x4 st[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (init) {
            const int n = 32 * (mt >> 1) + 8 * g + 4 * (mt & 1);
            const float4 q4 = *reinterpret_cast<const float4 *>(init + (bh * P + pw + r) * N + n);
            st[mt] = f32x4{q4.x, q4.y, q4.z, q4.w};
        }
    }

    auto stage = [&](int i) -> unsigned char * { return i == 0 ? stg0 : (i == 1 ? stg1 : stg2); };
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(Cm + (size_t)b * L * GN + (size_t)g_grp * N), 0, (L * GN - g_grp * N) * 2,
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(Bm + (size_t)b * L * GN + (size_t)g_grp * N), 0, (L * GN - g_grp * N) * 2,
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + (size_t)b * L * HP + (size_t)h * P + p0), 0, (L * HP - h * P - p0) * 2,
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t rcb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(cbf + ((size_t)b * nblk * G + g_grp) * (kBlk * kBlk)), 0,
        (nblk * G - g_grp) * (kBlk * kBlk * 2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(vrec + bh * nblk * kVecRec), 0, nblk * kVecRec * 4, kBufferWord3);
    const unsigned cb_step = kBlk * GN * 2, x_step = kBlk * HP * 2;
    const unsigned cbf_step = G * kBlk * kBlk * 2, v_step = kVecRec * 4;
    unsigned dma_cb[S::CBD], dma_x;
#pragma unroll
    for (int i = 0; i < S::CBD; ++i) {
        const int row = 4 * (wave + NW * i) + (lane >> 4);
        dma_cb[i] = row * GN * 2 + 16 * ((lane & 15) ^ row_swz(row));
    }
    {
        const int pos = 64 * wave + lane, row = pos / S::XC;
        dma_x = row * HP * 2 + 16 * ((pos % S::XC) ^ x_swz<PB>(row));
    }
    typedef __attribute__((address_space(3))) void lds_void;
    auto bdma = [](__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned char *dst) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, voff, 0, 0, 0);
    };
    // DMA j (0 <= j < VM_LOADS) of block kb into stage `buf`: C and B rows
    // (alternating), raw x, then this wave's share of the C B^T halves and
    // the record (past the last piece: the record again)
    auto dma_piece = [&](int kb, unsigned char *buf, int j) {
        if (j < 2 * S::CBD) {
            const int i = j >> 1;
            const unsigned o = dma_cb[i] + kb * cb_step;
            if (j & 1)
                bdma(rb, o, buf + S::BS + 1024 * (wave + NW * i));
            else
                bdma(rc, o, buf + S::CS + 1024 * (wave + NW * i));
        } else if (j < 2 * S::CBD + S::XD) {
            bdma(rx, dma_x + kb * x_step, buf + S::XR + 1024 * wave);
        } else {
            int pc = wave + NW * (j - 2 * S::CBD - S::XD);
            if (pc > 2) pc = 2;
            const bool half = pc < 2;
            bdma(half ? rcb : rv,
                 half ? 16 * (64 * pc + lane) + kb * cbf_step : 16 * lane + kb * v_step,
                 buf + (half ? S::CBF + 1024 * pc : S::VR));
        }
    };
    auto dma_block = [&](int kb, unsigned char *buf) {
#pragma unroll
        for (int j = 0; j < S::VM_LOADS; ++j) dma_piece(kb, buf, j);
    };
    const __amdgpu_buffer_rsrc_t y_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        y + (size_t)b * L * HP, 0, L * HP * 2, kBufferWord3);
    const int y_boff = (r * HP + h * P + pw + 4 * g) * 2;
    auto y_store = [&](int kb, const f32x4 (&acc)[2]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const u32x2 v = {pack2(acc[tt][0], acc[tt][1]), pack2(acc[tt][2], acc[tt][3])};
            __builtin_amdgcn_raw_buffer_store_b64(v, y_rsrc,
                                                  y_boff + (kb * kBlk + 16 * tt) * HP * 2, 0, 0);
        }
    };

    dma_block(0, stg0);
    dma_block(1, stg1);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    lds_barrier();
    float sig_out = 1.f;

    struct Ops {
        bf16x8 cfr[2][4];  // C fragments (tt, kk)
        bf16x8 xs;         // raw x^T
        f32x4 cfv[2];      // cf of tokens 8 g + 0..7
        bf16x8 cbv[2];     // causal diagonal block of C B^T, t-tiles 0 and 1
        bf16x8 bt[8];      // B^T fragments of the state tiles
    };
    auto load_ops = [&](const unsigned char *cur, Ops &o) {
        const float *v = reinterpret_cast<const float *>(cur + S::VR);
#pragma unroll
        for (int w4 = 0; w4 < 2; ++w4)
            o.cfv[w4] = *reinterpret_cast<const f32x4 *>(v + S::CF + 8 * g + 4 * w4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                o.cfr[tt][kk] = lds_b128(cur, S::CS + c_rd[kk & 1] + 4096 * tt + 128 * (kk >> 1));
        o.xs = join(lds_tr(cur, S::XR + xs_tr[0]), lds_tr(cur, S::XR + xs_tr[1]));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) o.cbv[tt] = lds_b128(cur, S::CBF + 1024 * tt + cbf_rd);
    };
    auto load_bt = [&](const unsigned char *cur, Ops &o, int mt) {
        const int off = 128 * (mt >> 2) + 8 * (mt & 1);
        o.bt[mt] = join(lds_tr(cur, S::BS + b_tr[0][(mt >> 1) & 1] + off),
                        lds_tr(cur, S::BS + b_tr[1][(mt >> 1) & 1] + off));
    };

    auto block = [&](int kb, const int si) {
        unsigned char *cur = stage(si);
        const float *v = reinterpret_cast<const float *>(cur + S::VR);
        const Book bk = book_of(v, sig_out);
        Ops o;
        load_ops(cur, o);
        float rpv[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) rpv[tt] = v[S::RP + 16 * tt + r];
        bf16x4 xr[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
            xr[tt] = *reinterpret_cast<const bf16x4 *>(cur + S::XR + xr_skip[tt]);
        const float xscale = bk.fac ? __builtin_amdgcn_rcpf(bk.sig) : 1.f;
        auto hb_of = [&](int kk) {
            bf16x8 hb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hb[j] = (bf16)st[2 * kk][j];
                hb[4 + j] = (bf16)st[2 * kk + 1][j];
            }
            return hb;
        };
        bf16x8 xp;
        f32x4 acc[2];
        acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[1] = acc[0];
        bf16x8 hb = hb_of(0);
        __builtin_amdgcn_sched_barrier(0);
        // y^T = h~ C^T: eight MFMAs (K-step kk, t-tile tt), each followed by
        // the next state conversion, one x' value and a B^T fragment
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int kk = q >> 1, tt = q & 1;
            acc[tt] = mma16(hb, o.cfr[tt][kk], acc[tt]);
            __builtin_amdgcn_sched_barrier(0);
            if (tt == 1 && kk < 3) hb = hb_of(kk + 1);
            if (q & 1) {
                // x' values q - 1 and q (tokens 8 g + q - 1, 8 g + q)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int j = q - 1 + e;
                    xp[j] = (bf16)((float)o.xs[j] * (o.cfv[j >> 2][j & 3] * xscale));
                }
            }
            load_bt(cur, o, q);
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("" : "+v"(xp));
        float f[2] = {rpv[0] * bk.sig, rpv[1] * bk.sig};
        float dco = Dh;
        if (bk.rescale) {
            __builtin_amdgcn_sched_barrier(0);
            acc[0] *= bk.sig_in;
            acc[1] *= bk.sig_in;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) st[mt] *= bk.sig_in;
        }
        if (!bk.fac) {
            __builtin_amdgcn_sched_barrier(0);
            // exact block (see the wave-of-32 kernel): per-element weights
            // exp(lambda_t - lambda_s) dt_s on raw x, D on the diagonal
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int t = 16 * tt + r;
                const float lr = v[S::LR + t];
                acc[tt] *= fast_exp(lr + v[S::LE]) * bk.sig_in;
                bf16x8 wgt;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = 8 * g + j;
                    const float w = (float)o.cbv[tt][j] * fast_exp(fminf(lr - v[S::LR + s], 0.f)) *
                                        v[S::DT + s] + (s == t ? Dh : 0.f);
                    wgt[j] = (bf16)(s <= t ? w : 0.f);
                }
                acc[tt] = mma16(o.xs, wgt, acc[tt]);
                o.cbv[tt] = zero_frag<bf16>();
            }
            f[0] = f[1] = 1.f;
            dco = 0.f;
            const float sd = bk.sig_in * bk.delta;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) st[mt] *= sd;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) acc[tt] = mma16(xp, o.cbv[tt], acc[tt]);
        __builtin_amdgcn_sched_barrier(0);
        // state update h~ += B^T x' (eight tiles), with the epilogue and the
        // DMAs of block kb + 2 issued between the MFMAs
        {
            unsigned char *nbuf = stage((si + 2) % 3);
            int j = 0;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                st[mt] = mma16(o.bt[mt], xp, st[mt]);
                __builtin_amdgcn_sched_barrier(0);
                const int jn = (S::VM_LOADS * (mt + 1)) / 8;
                for (; j < jn; ++j) dma_piece(kb + 2, nbuf, j);
                if (mt >= 2 && mt < 6) {
                    // output values 2 (mt - 2), 2 (mt - 2) + 1 of both t-tiles
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int vv = 2 * (mt - 2) + e, tt = vv >> 2, c = vv & 3;
                        acc[tt][c] = acc[tt][c] * f[tt] + dco * (float)xr[tt][c];
                    }
                    asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
        sig_out = bk.sig;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(S::VM_LOADS + S::Y_STORES));
        __builtin_amdgcn_sched_barrier(0);
        y_store(kb, acc);
        __builtin_amdgcn_sched_barrier(0);
        block_barrier();
    };

    for (int kb = 0; kb < nblk; kb += 3) {
        block(kb, 0);
        if (kb + 1 < nblk) {
            block(kb + 1, 1);
            if (kb + 2 < nblk) block(kb + 2, 2);
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    if (final_state) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const int n = 32 * (mt >> 1) + 8 * g + 4 * (mt & 1);
            *reinterpret_cast<float4 *>(final_state + (bh * P + pw + r) * N + n) =
                make_float4(st[mt][0] * sig_out, st[mt][1] * sig_out, st[mt][2] * sig_out,
                            st[mt][3] * sig_out);
        }
    }
}

// Inclusive prefix sum of an fp64 value over each 32-lane half of the wave,
// without LDS round trips: DPP shifts by 1, 2, 4 and 8 within each 16-lane
// row (lanes shifted in from outside the row read 0), then lanes 16..31
// (48..63) add the row total of lane 15 (47), read with v_readlane.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROW_MASK, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROW_MASK, 0xF, true);
    return __builtin_bit_cast(double, (unsigned long long)(unsigned)lo |
                                          ((unsigned long long)(unsigned)hi << 32));
}
__device__ __forceinline__ double lane_f64(double v, int src) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const unsigned lo = __builtin_amdgcn_readlane((unsigned)u, src);
    const unsigned hi = __builtin_amdgcn_readlane((unsigned)(u >> 32), src);
    return __builtin_bit_cast(double, (unsigned long long)lo | ((unsigned long long)hi << 32));
}
__device__ __forceinline__ double scan32_f64(double v, int lane) {
    v += dpp_f64<0x111, 0xF>(v);  // row_shr:1
    v += dpp_f64<0x112, 0xF>(v);  // row_shr:2
    v += dpp_f64<0x114, 0xF>(v);  // row_shr:4
    v += dpp_f64<0x118, 0xF>(v);  // row_shr:8
    const double r0 = lane_f64(v, 15), r2 = lane_f64(v, 47);
    return v + ((lane & 16) ? (lane >= 32 ? r2 : r0) : 0.0);
}
// the value of lane 31 in lanes 0..31 and of lane 63 in lanes 32..63
__device__ __forceinline__ double last_of_half(double v, int lane) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const unsigned lo = (unsigned)u, hi = (unsigned)(u >> 32);
    const unsigned lo0 = __builtin_amdgcn_readlane(lo, 31), hi0 = __builtin_amdgcn_readlane(hi, 31);
    const unsigned lo1 = __builtin_amdgcn_readlane(lo, 63), hi1 = __builtin_amdgcn_readlane(hi, 63);
    const bool up = lane >= 32;
    return __builtin_bit_cast(double, (unsigned long long)(up ? lo1 : lo0) |
                                          ((unsigned long long)(up ? hi1 : hi0) << 32));
}

// Per-block preparation of the fused pass, in one launch.  grid (n_rec +
// n_cb, batch), 256 threads.
//
// Workgroups [0, n_rec): the decay records (one per batch, head and 32-token
// block; layout at kVecRec) of kPrepBlocks consecutive blocks of 8 heads.
// All their dt values are staged through LDS first (32-byte runs over
// heads), then each half-wave takes one head and block at a time: the fp64
// prefix sum of dt A over the block's 32 tokens (dt A is exact in fp64), so
// lambda_l - lambda_s is the difference of two fp64 prefixes rounded once.
//
// Workgroups [n_rec, n_rec + n_cb) (launched for the 16-column kernel; the
// 32-column kernel forms these blocks itself from its staged C and B rows):
// the causal diagonal 32x32 block of C B^T for four (block, group) pairs,
// one per wave, bf16, in the MFMA B-fragment order the fused kernel reads.  W16 = 0 (waves of 32 columns,
// v_mfma_f32_32x32x16_bf16): K-step kk, lane L hold the 8 values
// C B^T[L % 32][16 kk + 8 (L / 32) .. +7] as the 16 bytes at (64 kk + L) * 16.
// W16 = 1 (waves of 16 columns, v_mfma_f32_16x16x32_bf16): token tile tt,
// lane L hold C B^T[16 tt + L % 16][8 (L / 16) .. +7] at (64 tt + L) * 16.
// A wave computes E = B C^T with v_mfma_f32_32x32x16_bf16 (all its row loads
// issued first; rows past the sequence end read as zeros through the buffer
// resource's range): lane (l = L % 32, hi) ends with E[s][l] = C_l . B_s for
// s = 8 i + 4 hi + c, four runs of 4 consecutive s.
constexpr int kPrepBlocks = 8;
template <int W16>
__global__ void __launch_bounds__(256)
k_prep(const float *__restrict__ dt, const float *__restrict__ A, float *__restrict__ vrec,
       const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm, bf16 *__restrict__ cbf, int L,
       int H, int G, int nblk, int n_rec) {
    const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    if ((int)blockIdx.x < n_rec) {
        __shared__ float s_dt[kPrepBlocks][kBlk][9];
        const int nbg = (nblk + kPrepBlocks - 1) / kPrepBlocks;
        const int kb0 = (blockIdx.x % nbg) * kPrepBlocks, h0 = (blockIdx.x / nbg) * 8;
        const int hh = tid >> 5, tt = tid & 31, h = h0 + hh;
        float af = A[h < H ? h : H - 1];
        {
            // (loads through a buffer resource over this batch's dt: tokens
            // past the end read as zeros, and all loads issue before any
            // wait; heads past H feed only half-waves that return below)
            const __amdgpu_buffer_rsrc_t rdt = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(dt + (size_t)b * L * H), 0, (unsigned)((size_t)L * H * 4), kBufferWord3);
            const int lt = tid >> 3, lh = tid & 7;
            float v[kPrepBlocks];
#pragma unroll
            for (int i = 0; i < kPrepBlocks; ++i)
                v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    rdt, (unsigned)(((kb0 + i) * kBlk + lt) * H + h0 + lh) * 4, 0, 0));
#pragma unroll
            for (int i = 0; i < kPrepBlocks; ++i) s_dt[i][lt][lh] = v[i];
            // (A is read here, with the dt loads in flight, not after the
            // barrier)
            asm volatile("" : "+v"(af));
        }
        const double a = (double)af;
        __syncthreads();
        if (h >= H) return;  // whole half-waves, after the only barrier
        float *const rec0 = vrec + (((size_t)b * H + h) * nblk + kb0) * kVecRec;
#pragma unroll
        for (int i = 0; i < kPrepBlocks; ++i) {
            if (kb0 + i >= nblk) break;
            const float d = s_dt[i][tt][hh];
            const double lam = scan32_f64((double)d * a, lane);
            const double lam_e = last_of_half(lam, lane);
            const float le = (float)lam_e;
            const bool fac = -le <= kSafeDecay;
            float *const rec = rec0 + i * kVecRec;
            rec[tt] = fast_exp((float)(lam_e - lam)) * d;
            rec[kBlk + tt] = fac ? fast_exp((float)(lam - lam_e)) : 0.f;
            // the per-element exponents and steps are read by exact blocks only
            if (!fac) {
                rec[2 * kBlk + tt] = (float)(lam - lam_e);
                rec[3 * kBlk + tt] = d;
            }
            if (tt == kBlk - 1)
                *reinterpret_cast<float4 *>(rec + 4 * kBlk) =
                    make_float4(fast_exp(le), fac ? 1.f : 0.f, le, 0.f);
        }
        return;
    }
    constexpr int N = 128;
    // (the wave index read as uniform, so that the buffer resources below
    // stay in scalar registers)
    const int pair = (blockIdx.x - n_rec) * 4 + __builtin_amdgcn_readfirstlane(tid >> 6);
    if (pair >= nblk * G) return;
    const int kb = pair / G, g = pair % G;
    const int r = lane & 31, hi = lane >> 5;
    const size_t base = ((size_t)b * L * G + g) * N;
    const unsigned range = (unsigned)(((size_t)L * G * N - (size_t)g * N) * 2);
    const __amdgpu_buffer_rsrc_t rbr = __builtin_amdgcn_make_buffer_rsrc((void *)(Bm + base), 0, range, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rcr = __builtin_amdgcn_make_buffer_rsrc((void *)(Cm + base), 0, range, kBufferWord3);
    const unsigned roff = (unsigned)((kb * kBlk + r) * G * N + 8 * hi) * 2;
    u32x4 bs[N / 16], cl[N / 16];
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) {
        bs[ks] = __builtin_amdgcn_raw_buffer_load_b128(rbr, roff + 32 * ks, 0, 0);  // A: row s = r
        cl[ks] = __builtin_amdgcn_raw_buffer_load_b128(rcr, roff + 32 * ks, 0, 0);  // B: column l = r
    }
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks)
        acc = mma32(__builtin_bit_cast(bf16x8, bs[ks]), __builtin_bit_cast(bf16x8, cl[ks]), acc);
    bf16 *out = cbf + (((size_t)b * nblk + kb) * G + g) * (kBlk * kBlk);
    // lane (l = r, hi): E[s][l] for s = 8 i + 4 hi + c
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s0 = 8 * i + 4 * hi;
        bf16x4 v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = s0 + c <= r ? (bf16)acc[4 * i + c] : (bf16)0.f;
        size_t dst;
        if (W16) {
            // t-tile r / 16, lane (r % 16) + 16 (s0 / 8), values s0 % 8 .. +3
            dst = (64 * (r >> 4) + (r & 15) + 16 * (s0 >> 3)) * 8 + (s0 & 7);
        } else {
            const int kk = s0 >> 4, hs = (s0 >> 3) & 1;
            dst = (64 * kk + r + 32 * hs) * 8 + (s0 & 7);
        }
        *reinterpret_cast<bf16x4 *>(out + dst) = v4;
    }
}

// --------------------------------------------------------------------- launch

const char *const kFusedKernelNames[kFusedKernels] = {"k_prep", "k_fused_ssd"};

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
    hipLaunchKernelGGL((k_fused_ssd<PB>), dim3(a.H * a.P / PB, a.batch), dim3(S::NT), 0, stream,
                       (const bf16 *)a.x, (const bf16 *)a.B, (const bf16 *)a.C, a.vrec, a.D,
                       a.init, a.final_state, (bf16 *)a.y, a.L, a.H, a.G, a.P, nblk);
    return hipSuccess;
}

template <int PB>
static hipError_t launch_fused16_main(const ForwardArgs &a, hipStream_t stream) {
    typedef Fused16<PB> S;
    const int nblk = fused_nblk(a.L);
    hipLaunchKernelGGL((k_fused16_ssd<PB>), dim3(a.H * (a.P / PB), a.batch), dim3(S::NT), 0,
                       stream, (const bf16 *)a.x, (const bf16 *)a.B, (const bf16 *)a.C,
                       (const bf16 *)a.cb, a.vrec, a.D, a.init, a.final_state, (bf16 *)a.y,
                       a.L, a.H, a.G, a.P, nblk);
    return hipSuccess;
}

// Waves of 32 columns unless SSD_FUSED_WAVE=16 asks for waves of 16 (a
// diagnostic switch for comparing the two layouts).
static bool use_wave16(const ForwardArgs &a) {
    (void)a;
    const char *env = getenv("SSD_FUSED_WAVE");
    return env && strcmp(env, "16") == 0;
}

// Columns per workgroup.  One workgroup per compute unit is the target
// (two 32-column workgroups on one compute unit slow each other down more
// than one 64-column workgroup's two waves do): 128 columns (four waves over
// two heads of one B/C group, which share the staged C and B rows) once
// 64-column workgroups would outnumber the 256 compute units; 64 (two
// waves) once 32-column ones would; else 32 (one wave).
static int pick_pb(const ForwardArgs &a) {
    const long cols = (long)a.batch * a.H * a.P;
    if (a.P == 64 && a.H % 2 == 0 && (a.H / a.G) % 2 == 0 && cols / 64 > 256) return 128;
    if (a.P % 64 == 0 && cols / 32 > 256) return 64;
    return 32;
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
    const bool w16 = use_wave16(a);
    const int n_rec = (nblk + kPrepBlocks - 1) / kPrepBlocks * ((a.H + 7) / 8);
    // (the 32-column kernel forms its C B^T blocks itself)
    const int n_cb = w16 ? (nblk * a.G + 3) / 4 : 0;
    if (w16)
        hipLaunchKernelGGL(k_prep<1>, dim3(n_rec + n_cb, a.batch), dim3(256), 0, stream, a.dt, a.A,
                           a.vrec, (const bf16 *)a.B, (const bf16 *)a.C, (bf16 *)a.cb, a.L, a.H,
                           a.G, nblk, n_rec);
    else
        hipLaunchKernelGGL(k_prep<0>, dim3(n_rec + n_cb, a.batch), dim3(256), 0, stream, a.dt, a.A,
                           a.vrec, (const bf16 *)a.B, (const bf16 *)a.C, (bf16 *)a.cb, a.L, a.H,
                           a.G, nblk, n_rec);
    if ((err = mark()) != hipSuccess) return err;
    if (w16) {
        err = a.P % 64 == 0 ? launch_fused16_main<64>(a, stream) : launch_fused16_main<32>(a, stream);
    } else {
        switch (pick_pb(a)) {
            case 128: err = launch_fused_main<128>(a, stream); break;
            case 64: err = launch_fused_main<64>(a, stream); break;
            default: err = launch_fused_main<32>(a, stream); break;
        }
    }
    if (err != hipSuccess) return err;
    if ((err = mark()) != hipSuccess) return err;
    return hipGetLastError();
}

template hipError_t launch_fused_forward<float>(const ForwardArgs &, hipStream_t, hipEvent_t *);
template hipError_t launch_fused_forward<bf16>(const ForwardArgs &, hipStream_t, hipEvent_t *);

}  // namespace ssd
