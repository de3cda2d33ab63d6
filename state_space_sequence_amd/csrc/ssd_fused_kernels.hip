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
// factors come in each block's decay record (fp32 prefixes), formed by a
// helper wave two blocks ahead.
//
// Workgroup (the Fused struct below): PB / 32 compute waves, wave w owning
// headdim columns 32 w .. 32 w + 31 of the workgroup's PB columns and
// computing with v_mfma_f32_32x32x16_bf16, plus helper waves: a loader that
// issues every DMA into LDS and every y store, and a former that forms the
// decay records and the causal C B^T blocks.  Four LDS stages rotate; per
// 32-token block a compute wave computes
//   output y^T = h~ C^T + x'^T [C B^T]^T for its 32 columns and the block's
//          32 tokens, with h~ taken straight from the state registers as the
//          MFMA A operand, and hands y to the loader through LDS;
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
// cache-policy operand of the buffer intrinsics: bit 1 is the non-temporal
// hint (nt) on this target
constexpr int kNonTemporal = 2;
// word 3 of a raw buffer resource on gfx9-family targets (32-bit data format)
constexpr int kBufferWord3 = 0x00020000;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
__device__ __forceinline__ float uniform(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ unsigned pack2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, bf16x2{(bf16)a, (bf16)b});
}
// Inclusive prefix sum over each 32-lane half of the wave, without LDS
// round trips: DPP shifts by 1, 2, 4 and 8 within each 16-lane row (lanes
// shifted in from outside the row read 0), then lanes 16..31 (48..63) add
// the row total of lane 15 (47), read with v_readlane.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_f32(float v, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}
// A compile-time flag passed to generic lambdas.
template <bool V> struct BoolTag { static constexpr bool value = V; };

// Inclusive running maximum over each half-wave of values >= 0 (the DPP
// shifts bring in 0 past the row start, the identity for such values).
__device__ __forceinline__ float scanmax32(float v, int lane) {
    v = fmaxf(v, dpp_f32<0x111>(v));  // row_shr:1
    v = fmaxf(v, dpp_f32<0x112>(v));  // row_shr:2
    v = fmaxf(v, dpp_f32<0x114>(v));  // row_shr:4
    v = fmaxf(v, dpp_f32<0x118>(v));  // row_shr:8
    const float r0 = lane_f32(v, 15), r2 = lane_f32(v, 47);
    return (lane & 16) ? fmaxf(v, lane >= 32 ? r2 : r0) : v;
}
__device__ __forceinline__ float scan32(float v, int lane) {
    v += dpp_f32<0x111>(v);  // row_shr:1
    v += dpp_f32<0x112>(v);  // row_shr:2
    v += dpp_f32<0x114>(v);  // row_shr:4
    v += dpp_f32<0x118>(v);  // row_shr:8
    const float r0 = lane_f32(v, 15), r2 = lane_f32(v, 47);
    return v + ((lane & 16) ? (lane >= 32 ? r2 : r0) : 0.f);
}
// the value of lane 31 in lanes 0..31 and of lane 63 in lanes 32..63
__device__ __forceinline__ float last_of_half(float v, int lane) {
    const float a = lane_f32(v, 31), c = lane_f32(v, 63);
    return lane >= 32 ? c : a;
}

// Workgroup layout.  A workgroup covers PB consecutive columns of one
// batch's flattened (head, headdim) columns h P + p (x and y rows are
// contiguous over them): NW = PB / 32 waves of 32 columns each.  With
// PB > P the workgroup spans NH = PB / P heads of one B/C group, which then
// share the staged C and B rows.
template <int PB, bool SO = false>
struct Fused {
    static constexpr int NW = PB / 32;                 // compute waves: 32 headdim columns each
    // Helper waves.  The loader (wave NW) issues every global memory
    // operation of the workgroup: the DMAs of the stages and the y stores,
    // which the compute waves hand over through LDS; the compute waves never
    // wait on the vector memory pipeline.  The former forms each block's
    // decay records and C B^T block in LDS.  Waves go to the four SIMDs in
    // turn (wave w to SIMD w % 4), and a helper slows the compute wave whose
    // SIMD it shares by about its own issue time.  With four compute waves
    // the former's two jobs are split over waves NW + 2 (C B^T blocks, on
    // SIMD 2) and NW + 3 (records, on SIMD 3), and wave NW + 1 only takes
    // the barriers, so that no SIMD carries two helpers (the loader shares
    // SIMD 0) and the records wave has time to spare (the time-step
    // preprocessing of the raw dt runs there).  With fewer compute waves
    // every helper has a SIMD of its own.  The state-only pass (SO) forms
    // no C B^T blocks: one former wave (records only) and the loader.
    static constexpr int NHELP = (NW == 4 && !SO) ? 4 : 2;
    static constexpr bool SPLIT_FORMER = NHELP == 4;
    static constexpr int NT = 64 * (NW + NHELP);       // threads
    static constexpr int N = 128;                      // dstate
    static constexpr int ROWB = 2 * N;                 // bytes per C / B row
    static constexpr int MAT = kBlk * ROWB;            // 8 KB per matrix
    static constexpr int XC = PB / 8;                  // 16-byte chunks per x row
    static constexpr int XRB = 2 * PB;                 // raw x row bytes
    static constexpr int NRS = PB == 128 ? 2 : 1;      // decay-record slots (heads)
    // one stage: C rows, B rows (column-blocked, blk_off) and raw x
    // (column-blocked) of one block, filled by DMA, and its dt (token t of
    // head slot q at DTR + 4 (32 q + t)), filled by the DMAs of the block
    // before; the causal diagonal block of C B^T in the
    // MFMA B-fragment order and the decay records (kVecRec floats in 1 KB
    // slots), formed by the former from the stage's C and B rows and dt;
    // then the block's y for the loader: 32 rows of XRB bytes, 16-byte
    // chunk c of row t in slot c ^ ys_swz(t)
    // (the state-only pass has no C rows, C B^T block or y staging, so its
    // stages are 18.5 KB and two of its workgroups fit on a compute unit)
    static constexpr int CS = 0;
    static constexpr int BS = SO ? 0 : MAT;
    static constexpr int CBF = BS + MAT;               // 2 x 1 KB of C B^T fragments
    static constexpr int XR = CBF + (SO ? 0 : 2048);
    static constexpr int VR = XR + kBlk * XRB;
    static constexpr int YS = VR + 1024 * NRS;
    static constexpr int DTR = YS + (SO ? 0 : kBlk * XRB);
    static constexpr int SEQ = DTR + 256;              // seq_idx of the block (varlen), 2 x 32
    static constexpr int STG = SEQ + 256;
    // floats of the decay record
    enum { W = 0, F = 32, LR = 64, DT = 96, DELTA = 128, FLAG = 129, LE = 130, SIGIN = 131,
           SIGOUT = 132, RESC = 133, SEG = 136 };
    // four stages: the DMAs of a block go out three blocks ahead of its
    // use; the former forms a block's decay records two blocks ahead and
    // its C B^T block one block ahead, and the compute waves read its
    // opening operands during the block before it
    static constexpr int NST = 4;
    // K-step rows m of the C fragments among the opening operands (within
    // the 256 registers per lane that two waves on a SIMD leave each)
    static constexpr int ECF = PB == 128 ? 1 : 2;
    static constexpr int LDS = NST * STG;
    static_assert(PB == 32 || PB == 64 || PB == 128, "one, two or four waves");
    static_assert(STG % 16 == 0, "alignment");
    // (one workgroup per compute unit, which the column choice arranges)
    static_assert(LDS <= 160 * 1024, "LDS per compute unit");
    // The loader's vector-memory operations per block: DMAs (C and B, x,
    // and the next block's dt; one more, seq_idx, with packed sequences),
    // y stores, and with the output gate the DMAs of the block's z into its
    // y staging slots.  In block kb it issues the DMAs of block kb + 3, the
    // y stores of block kb - 1, then the z DMAs of block kb + 3, and at its
    // end waits until the DMAs of block kb + 2 have landed (everything older
    // has landed too, the z of block kb + 1 among them).  Younger than the
    // DMAs of block kb + 2 are the stores and z DMAs issued after them in
    // block kb - 1 and all of block kb's operations.  Block 0 stores no y,
    // so in block 1 the count is P_STORES smaller.
    static constexpr int P_LOADS = 2 * (MAT / 1024) + kBlk * XRB / 1024 + 1;
    static constexpr int P_STORES = kBlk * XRB / 1024;
    static_assert(NST == 4, "the wait counts assume four stages");
    static constexpr int wait_count(bool gate, bool varlen, bool block1) {
        return 2 * P_STORES + (gate ? 2 * P_STORES : 0) + P_LOADS + (varlen ? 1 : 0) -
               (block1 ? P_STORES : 0);
    }
    static_assert(wait_count(true, true, false) < 64, "vmcnt immediate");
    // The state-only pass (kEpiState) loads no C rows and stores no y: at
    // the end of block kb everything it issued in block kb is younger than
    // the DMAs of block kb + 2.
    static constexpr int P_LOADS_SO = MAT / 1024 + kBlk * XRB / 1024 + 1;
    static constexpr int wait_count_so(bool varlen) { return P_LOADS_SO + (varlen ? 1 : 0); }
};

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

// A buffer resource over one stream of a batch row (x, y, z, C, B, dt,
// seq_idx), rebased every 2^shift blocks: buffer offsets are 32 bits, and a
// long sequence at a wide row has more than 2^31 bytes.  The resource covers
// the bytes from the start of block k's window to the end of the stream
// (clamped to 2^32 - 1), so rows past the end still read as zeros and their
// stores are dropped; at(k) rebuilds it only when k enters another window
// (a compare and a branch otherwise) and gives block k's offset in it.
struct WinRsrc {
    const char *row0;
    size_t total;
    unsigned blk_bytes;
    int shift, w;
    __amdgpu_buffer_rsrc_t r;
    __device__ void init(const void *p, size_t total_bytes, unsigned blk, int sh) {
        row0 = static_cast<const char *>(p);
        total = total_bytes;
        blk_bytes = blk;
        shift = sh;
        w = -1;
    }
    __device__ __forceinline__ const __amdgpu_buffer_rsrc_t &at(int k, unsigned &soff) {
        const int kw = k >> shift;
        if (kw != w) {
            w = kw;
            const size_t base = ((size_t)kw << shift) * blk_bytes;
            const size_t rem = total > base ? total - base : 0;
            r = __builtin_amdgcn_make_buffer_rsrc((void *)(row0 + base), 0,
                                                  (unsigned)(rem < 0xFFFFFFFFull ? rem : 0xFFFFFFFFull),
                                                  kBufferWord3);
        }
        soff = (unsigned)(k - (kw << shift)) * blk_bytes;
        return r;
    }
};

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
// Output variants (EPI): bit 0, D per (head, headdim column) instead of per
// head; bit 1, the output gate y * silu(z).  EPI = 0 is the plain forward.
// Bit 2 (kEpiState) is the state-only pass of a segmented forward: no C, no
// C B^T, no y; each workgroup writes the state its segment leaves (from the
// initial state in segment 0, from zero in the others) and, per head, the
// segment's total log decay.
constexpr int kEpiDhp = 1, kEpiGate = 2, kEpiState = 4;

template <int PB, int EPI>
__global__ void __launch_bounds__((Fused<PB, (EPI & 4) != 0>::NT))
k_fused_ssd(const bf16 *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
            const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
            const float *__restrict__ D, const float *init_arg, float *final_arg,
            bf16 *__restrict__ y, int L, int H, int G, int P, int nblk, const DtProc dtp,
            const int *__restrict__ seq_idx, const bf16 *__restrict__ z, int win_shift,
            const SegPlan plan, const float *seg_in, float *seg_out, float *seg_logdec) {
    constexpr bool SO = (EPI & kEpiState) != 0;
    typedef Fused<PB, SO> S;
    constexpr int NW = S::NW, N = S::N;
    constexpr bool DHP = (EPI & kEpiDhp) != 0, GATE = (EPI & kEpiGate) != 0;
    // Every LDS region that a DMA fills is its own object: the compiler can
    // then see that a DMA in flight never aliases the reads of another
    // region, and does not wait for it before those reads.
    __shared__ __align__(16) unsigned char stg0[S::STG];
    __shared__ __align__(16) unsigned char stg1[S::STG];
    __shared__ __align__(16) unsigned char stg2[S::STG];
    __shared__ __align__(16) unsigned char stg3[S::NST > 3 ? S::STG : 16];
    // D of the workgroup's columns when it is per (head, headdim column)
    __shared__ __align__(16) float dsh[DHP ? PB : 4];

    const int HP = H * P, GN = G * N;
    // Workgroups are dealt to the 8 XCDs in turn (workgroup i to XCD i % 8),
    // each XCD with its own L2.  With a multiple of 8 workgroups, XCD x gets
    // the consecutive range x * n / 8 .. of (segment, batch, column block)
    // triples, so the workgroups that share a batch's (or group's) C, B and
    // dt rows share few L2s and fetch those rows a few times instead of once
    // per XCD.  (The plain order, which spreads a batch over all eight L2s,
    // made the 8-group layer 28% slower; on the 2.7B layer it was 0.8%
    // faster but fetched 168 MB more per launch, 1.27x the algorithmic
    // bytes, so it is not used.)
    // The sequence may be cut into segments (SegPlan); this launch runs
    // segments plan.base .. plan.base + gridDim.z - 1 (the segment index
    // varies slowest, so a segment's workgroups sit together on the XCDs as
    // a batch's do).
    int c0, b, seg;
    {
        const int nc = H * P / PB, nb = gridDim.y, n = nc * nb * gridDim.z;
        const int i = (blockIdx.z * nb + blockIdx.y) * nc + blockIdx.x;
        const int v = (n % 8 == 0) ? (i % 8) * (n / 8) + i / 8 : i;
        c0 = (v % nc) * PB;
        b = (v / nc) % nb;
        seg = plan.base + v / nc / nb;
    }
    // the workgroup's blocks kb0 .. kb0 + nloc - 1 (the host makes every
    // segment non-empty)
    const int kb0 = seg == 0 ? 0 : plan.first + (seg - 1) * plan.len;
    const int nloc = (seg == 0 ? plan.first : min(nblk, kb0 + plan.len)) - kb0;
    // The state entering the segment: the initial state in segment 0; zero
    // in the state-only pass; in the main pass, chained from the states of
    // the earlier segments (below).  The state leaving it: the final state
    // after the last segment; segment 0's into seg_out[0] when there are
    // more; every segment's own into seg_out[seg] (state-only pass).
    const size_t bHPN = (size_t)gridDim.y * H * P * N;
    const float *init = seg == 0 ? init_arg : (SO ? nullptr : seg_in);
    float *final_state = SO ? seg_out + (size_t)seg * bHPN
                            : (seg == plan.nseg - 1 ? final_arg : (seg == 0 ? seg_out : nullptr));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = (c0 / P) / (H / G);          // the workgroup's B / C group

    auto stage = [&](int i) -> unsigned char * {
        return i == 0 ? stg0 : (i == 1 ? stg1 : (i == 2 ? stg2 : stg3));
    };

    if (wave >= NW) {
        // ---- the loader (wave NW): every DMA of the stages and every y
        // store; the former (wave NW + 1): the records and C B^T blocks.
        // Buffer resources over the workgroup's slices of C, B, x, dt, y and
        // z (WinRsrc: rebased every 2^win_shift blocks, once per window in
        // practice); a block adds its byte offset to fixed per-lane offsets.
        // Rows past the end of the sequence (the ragged tail, and the
        // prefetches past the last block) fall outside a resource's range:
        // the hardware reads them as zeros and drops such stores.  The DMAs
        // of a block, its dt and its y stores are issued at different times,
        // so each has its own resource.
        const size_t Lz = (size_t)L;
        WinRsrc wc, wb, wx, wdt, wy, wz, wseq;
        wc.init(Cm + (size_t)b * Lz * GN + (size_t)g * N, (Lz * GN - g * N) * 2, kBlk * GN * 2,
                win_shift);
        wb.init(Bm + (size_t)b * Lz * GN + (size_t)g * N, (Lz * GN - g * N) * 2, kBlk * GN * 2,
                win_shift);
        wx.init(x + (size_t)b * Lz * HP + c0, (Lz * HP - c0) * 2, kBlk * HP * 2, win_shift);
        // dt of this batch; lane l of the dt DMA reads token l % 32 of head
        // h0 + l / 32 (heads past the workgroup's are read and not used)
        const int h0 = c0 / P;
        wdt.init(dt + (size_t)b * Lz * H, Lz * H * 4, kBlk * H * 4, win_shift);
        wy.init(y + (size_t)b * Lz * HP, Lz * HP * 2, kBlk * HP * 2, win_shift);
        // the gate z, like y (read once: non-temporal)
        wz.init(GATE ? z + (size_t)b * Lz * HP : nullptr, GATE ? Lz * HP * 2 : 0, kBlk * HP * 2,
                win_shift);
        typedef __attribute__((address_space(3))) void lds_void;
        // (the block's byte offset goes in the scalar offset, so a DMA
        // costs no vector instruction).  y is written once and never read
        // back, so its stores carry the non-temporal hint (kNonTemporal);
        // measured, that shortens the 2.7B-shape layer by about 5%.  x is
        // read once too, but its loads carry the hint only with grouped B
        // and C (G > 1), where it keeps the caches for the B and C rows that
        // the workgroups of a group share (10% shorter on the 8-group
        // layer); with one group it costs 3-8%.  C and B rows stay ordinary.
        const bool x_nt = G > 1;
        auto bdma = [](__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff, unsigned char *dst) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, voff, soff, 0, 0);
        };
        auto bdma_nt = [](__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff, unsigned char *dst) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, voff, soff, 0, kNonTemporal);
        };
        const unsigned pdt = ((lane & 31) * H + h0 + (lane >> 5)) * 4;
        // packed sequences: seq_idx of this batch, token lane % 32 into both
        // halves of the stage's SEQ region
        const bool varlen = seq_idx != nullptr;
        wseq.init(varlen ? seq_idx + (size_t)b * Lz : nullptr, varlen ? Lz * 4 : 0, kBlk * 4,
                  win_shift);
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
        // dt of block kb into `buf` (the stage of block kb)
        auto pdt_dma = [&](int kb, unsigned char *buf) {
            unsigned so;
            const __amdgpu_buffer_rsrc_t &rdt = wdt.at(kb, so);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rdt, (lds_void *)(buf + S::DTR), 4, pdt, so,
                                                     0, 0);
            if (varlen) {
                const __amdgpu_buffer_rsrc_t &rseq = wseq.at(kb, so);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rseq, (lds_void *)(buf + S::SEQ), 4,
                                                         (lane & 31) * 4, so, 0, 0);
            }
        };
        // the DMAs of block kb into `buf`, and the dt of block kb + 1 into
        // `nbuf` (the stage of block kb + 1)
        auto pdma = [&](int kb, unsigned char *buf, unsigned char *nbuf) {
            unsigned cbo = 0, bo, xo;
            if constexpr (!SO) wc.at(kb, cbo);
            const __amdgpu_buffer_rsrc_t &rb = wb.at(kb, bo);
            const __amdgpu_buffer_rsrc_t &rx = wx.at(kb, xo);
#pragma unroll
            for (int i = 0; i < NCB; ++i) {
                if constexpr (!SO) bdma(wc.r, pcb[i], cbo, buf + S::CS + 1024 * i);
                bdma(rb, pcb[i], bo, buf + S::BS + 1024 * i);
            }
            if (x_nt) {
#pragma unroll
                for (int i = 0; i < NXD; ++i) bdma_nt(rx, px[i], xo, buf + S::XR + 1024 * i);
            } else {
#pragma unroll
                for (int i = 0; i < NXD; ++i) bdma(rx, px[i], xo, buf + S::XR + 1024 * i);
            }
            pdt_dma(kb + 1, nbuf);
        };
        // The decay record of head slot q = lane / 32 of block kblk, staged
        // in `buf`, from its dt (run through the time-step preprocessing when
        // that is on, tokens past seqlen kept at 0), blocks taken in order:
        // lambda_t = sum_{j <= t}
        // dt_j A (fp32, the block's 32 tokens), lambda_e = lambda_31, delta =
        // exp(lambda_e), factored = (-lambda_e <= 60).  The scale sigma of the
        // head's state (h = sigma h~) is tracked here: sigma_out = sigma_in
        // delta, restarted to delta when that would fall below exp(-60)
        // (RESC), and 1 after an exact block.  Per token
        //   W = exp(lambda_e - lambda_t) dt_t / sigma_out   (x' = W x; 1 for
        //       sigma_out in an exact block),
        //   F = exp(lambda_t - lambda_e) sigma_out          (0 in an exact block),
        //   LR = lambda_t - lambda_e, DT = dt_t,
        // then DELTA, FLAG, LE = lambda_e, SIGIN, SIGOUT, RESC.
        // lambda_e - lambda_t carries an absolute error of a few units of
        // |lambda_e| 2^-24 (below 1e-4 while the block is factored), the
        // relative error it puts on the exp factors.
        const int ph = (h0 + (lane >> 5)) < H ? h0 + (lane >> 5) : H - 1;
        const float pa = A[ph];
        const float pbias = dtp.on && dtp.bias ? dtp.bias[ph] : 0.f;
        float psig = 1.f;  // sigma of this lane's head after the last record formed
        // Packed sequences: token t (> 0, < seqlen) whose seq_idx differs from
        // token t - 1's starts a new sequence, and the state entering it is 0.
        // pseq is the seq_idx of the last token of the previous block.
        bool pfirst = kb0 == 0;
        int pseq = !pfirst && varlen ? seq_idx[(size_t)b * L + (size_t)kb0 * kBlk - 1] : 0;
        // (state-only pass) the segment's total log decay of this lane's
        // head, and whether a sequence starts in it (then its decay is 0)
        float ltot = 0.f;
        bool cut = false;
        // VL: the packed-sequence variant (a compile-time tag, so that the
        // plain one is the code without any of it)
        auto prec_v = [&](unsigned char *buf, int kblk, auto vl_tag) {
            constexpr bool VL = decltype(vl_tag)::value;
            const int t = lane & 31, q = lane >> 5;
            const int tok = kBlk * kblk + t;
            float d = *reinterpret_cast<const float *>(buf + S::DTR + 4 * lane);
            if (dtp.on) d = tok < L ? dt_process(d, pbias, dtp.softplus, dtp.lo, dtp.hi) : 0.f;
            // s0 = the last sequence start at or before t in this block (-1:
            // none), s0e the last one in the block
            float s0 = -1.f, s0e = -1.f;
            if constexpr (VL) {
                const int sq = *reinterpret_cast<const int *>(buf + S::SEQ + 4 * lane);
                const int up = __builtin_amdgcn_update_dpp(0, sq, 0x138, 0xF, 0xF, false);  // wave_shr:1
                const int prev = t == 0 ? (pfirst ? sq : pseq) : up;
                const bool start = tok < L && sq != prev;
                s0 = scanmax32(start ? (float)(t + 1) : 0.f, lane) - 1.f;
                s0e = last_of_half(s0, lane);
                pseq = __builtin_amdgcn_readlane(sq, kBlk - 1);
                pfirst = false;
            }
            const float lam = scan32(d * pa, lane);
            const float le = last_of_half(lam, lane);
            if constexpr (SO) {
                // (records are also formed for up to two blocks past the
                // segment; they are not its own)
                if (kblk < kb0 + nloc) {
                    ltot += le;
                    cut = cut || s0e >= 0.f;
                }
            }
            // a block with a sequence start takes the exact path: the state
            // entering it does not reach past the start (delta = 0), the
            // state-in factor applies before it only, and the state leaving
            // it collects the last sequence only
            const bool fac = (!VL || s0e < 0.f) && -le <= kSafeDecay;
            const float delta = (!VL || s0e < 0.f) ? fast_exp(le) : 0.f;
            const float sig_in = psig, p = sig_in * delta;
            const bool resc = fac && p < kRescale;
            const float sig_out = fac ? (resc ? delta : p) : 1.f;
            const float xsc = fac ? __builtin_amdgcn_rcpf(sig_out) : 1.f;
            psig = sig_out;
            if (q < S::NRS) {
                float *rec = reinterpret_cast<float *>(buf + S::VR + 1024 * q);
                if constexpr (VL) {
                    rec[S::W + t] = (float)t >= s0e ? fast_exp(le - lam) * d * xsc : 0.f;
                    // (exact blocks: the state-in factor exp(lambda_t), before
                    // the block's first sequence start)
                    rec[S::F + t] = fast_exp(fac ? lam - le : lam) *
                                    (fac ? sig_out : (s0 < 0.f ? 1.f : 0.f));
                    rec[S::SEG + t] = s0;
                } else {
                    rec[S::W + t] = fast_exp(le - lam) * d * xsc;
                    rec[S::F + t] = fac ? fast_exp(lam - le) * sig_out : 0.f;
                }
                rec[S::LR + t] = lam - le;
                rec[S::DT + t] = d;
                if (t == kBlk - 1) {
                    *reinterpret_cast<f32x4 *>(rec + S::DELTA) = f32x4{delta, fac ? 1.f : 0.f, le, sig_in};
                    *reinterpret_cast<f32x2 *>(rec + S::SIGOUT) = f32x2{sig_out, resc ? 1.f : 0.f};
                }
            }
        };
        auto prec = [&](unsigned char *buf, int kblk) {
            if (varlen)
                prec_v(buf, kblk, BoolTag<true>{});
            else
                prec_v(buf, kblk, BoolTag<false>{});
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
            unsigned yo;
            const __amdgpu_buffer_rsrc_t &y_rsrc = wy.at(kb, yo);
#pragma unroll
            for (int i = 0; i < S::P_STORES; ++i) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(buf + pys[i]);
                __builtin_amdgcn_raw_buffer_store_b128(v, y_rsrc, py[i], yo, kNonTemporal);
            }
        };
        // The gate's DMAs: z of block kb into the y staging rows of its stage,
        // each 16-byte chunk in the slot that its y chunk will take (DMA i,
        // lane l fills slot 64 i + l: row t = slot / XC and slot column
        // slot % XC, which holds chunk (slot % XC) ^ ys_swz(t)).  Issued after
        // the y stores that read those rows for block kb - 4.
        unsigned pz[GATE ? S::P_STORES : 1];
        if constexpr (GATE) {
#pragma unroll
            for (int i = 0; i < S::P_STORES; ++i) {
                const int pos = 64 * i + lane, t = pos / S::XC;
                const int c = (pos % S::XC) ^ ys_swz<S::XC>(t);
                pz[i] = (t * HP + c0 + 8 * c) * 2;
            }
        }
        auto zdma = [&](int kb, unsigned char *buf) {
            if constexpr (GATE) {
                unsigned zo;
                const __amdgpu_buffer_rsrc_t &rz = wz.at(kb, zo);
#pragma unroll
                for (int i = 0; i < S::P_STORES; ++i) bdma_nt(rz, pz[i], zo, buf + S::YS + 1024 * i);
            }
        };
        // Every wave takes the same barriers: two in the prologue (the DMAs
        // of blocks 0..2 landed; then the C B^T block of block 0 and the
        // records of blocks 0 and 1 formed), then one at the end of every
        // block.
        if (wave == NW) {
            pdt_dma(kb0, stage(0));
#pragma unroll
            for (int i = 0; i < S::NST - 1; ++i) pdma(kb0 + i, stage(i), stage(i + 1));
#pragma unroll
            for (int i = 0; i < S::NST - 1; ++i) zdma(kb0 + i, stage(i));
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            lds_barrier();
            lds_barrier();
            // block kb: refill the stage block kb - 1 used (and the dt slot of
            // block kb + 4 in this block's stage: its records were formed two
            // blocks ago), store block kb - 1's y, then wait for the DMAs of
            // block kb + 2 and the end-of-block barrier
            auto pblock = [&](int j, const int si) {
                const int kb = kb0 + j;
                pdma(kb + S::NST - 1, stage((si + S::NST - 1) % S::NST), stage(si));
                if constexpr (!SO) {
                    if (j > 0) pstore(kb - 1, stage((si + S::NST - 1) % S::NST));
                }
                // The z DMAs refill the staging rows that the y stores above
                // read.  Each store waits for its LDS read, so DMAs issued after
                // the stores cannot land first; nothing may be scheduled across
                // this point (a DMA past the end returns zeros at once, and an
                // early one would zero the y not yet read).
                if constexpr (GATE) __builtin_amdgcn_sched_barrier(0);
                zdma(kb + S::NST - 1, stage((si + S::NST - 1) % S::NST));
                if constexpr (SO) {
                    if (varlen)
                        __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(S::wait_count_so(true)));
                    else
                        __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(S::wait_count_so(false)));
                } else if (j == 1) {
                    if (varlen)
                        __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(S::wait_count(GATE, true, true)));
                    else
                        __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(S::wait_count(GATE, false, true)));
                } else {
                    if (varlen)
                        __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(S::wait_count(GATE, true, false)));
                    else
                        __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(S::wait_count(GATE, false, false)));
                }
                lds_barrier();
            };
            for (int j = 0; j < nloc; j += S::NST) {
                pblock(j, 0);
                if (j + 1 < nloc) {
                    pblock(j + 1, 1);
                    if (j + 2 < nloc) {
                        pblock(j + 2, 2);
                        if (j + 3 < nloc) pblock(j + 3, 3);
                    }
                }
            }
            if constexpr (!SO) pstore(kb0 + nloc - 1, stage((nloc - 1) % S::NST));
            // no DMA may land in LDS after the workgroup ends
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        } else {
            // the former's jobs: C B^T blocks (do_cbt) and records (do_rec)
            const bool do_cbt = !SO && (!S::SPLIT_FORMER || wave == NW + 2);
            const bool do_rec = !S::SPLIT_FORMER || wave == NW + 3;
            lds_barrier();
            if (do_cbt) pcbt(stage(0));
            if (do_rec) {
                prec(stage(0), kb0);
                prec(stage(1), kb0 + 1);
            }
            lds_barrier();
            // block kb: the C B^T block of block kb + 1 and the records of
            // block kb + 2 (whose data landed before the last barrier: the
            // dt of block kb + 2 comes with the DMAs of block kb + 1), then
            // the end-of-block barrier (unrolled by the stage count, so that
            // every stage address is a literal)
            auto fblock = [&](const int si, int kb) {
                if (do_cbt) pcbt(stage((si + 1) % S::NST));
                if (do_rec) prec(stage((si + 2) % S::NST), kb + 2);
                lds_barrier();
            };
            for (int j = 0; j < nloc; j += S::NST) {
                fblock(0, kb0 + j);
                if (j + 1 < nloc) {
                    fblock(1, kb0 + j + 1);
                    if (j + 2 < nloc) {
                        fblock(2, kb0 + j + 2);
                        if (j + 3 < nloc) fblock(3, kb0 + j + 3);
                    }
                }
            }
            if constexpr (SO) {
                // the segment's log decay per head (-inf: a sequence starts
                // in it); workgroups sharing a head write the same value
                const int q = lane >> 5;
                if (do_rec && (lane & 31) == 0 && q < S::NRS && h0 + q < H)
                    seg_logdec[((size_t)seg * gridDim.y + b) * H + h0 + q] =
                        cut ? -__builtin_inff() : ltot;
            }
        }
        return;
    }

    const int r = lane & 31, hi = lane >> 5;
    const int cw = c0 + 32 * wave;             // this wave's first flattened column
    const int hw = cw / P, pw = cw - hw * P;   // its head and headdim column
    const int slot = (cw - c0) / (PB > P ? P : PB);  // its decay-record slot
    const size_t bh = (size_t)b * H + hw;
    const float Dh = !DHP && D ? D[hw] : 0.f;
    if constexpr (DHP) {
        // (published to the other waves by the prologue barriers)
        if (lane < 32) dsh[32 * wave + lane] = D[cw + lane];
    }

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
    if (!SO && seg > 1) {
        // Segment s of the main pass: seg_in[0] is the state leaving segment
        // 0 (its main pass wrote it) and seg_in[k], k >= 1, the state
        // segment k leaves from zero (the state-only pass); with
        // d_k = exp(logdec_k) the state entering k + 1 is
        // d_k (state entering k) + seg_in[k] (the inter-chunk recurrence of
        // the rustdoc's Step 3, over segments), chained here up to s.
        for (int k = 1; k < seg; ++k) {
            const float d = __expf(seg_logdec[((size_t)k * gridDim.y + b) * H + hw]);
            const float *src = seg_in + (size_t)k * bHPN + (bh * P + pr) * N;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = 32 * m + 16 * (i >> 1) + 8 * hi + 4 * (i & 1);
                    const float4 q4 = *reinterpret_cast<const float4 *>(src + n);
                    st[m][4 * i] = d * st[m][4 * i] + q4.x;
                    st[m][4 * i + 1] = d * st[m][4 * i + 1] + q4.y;
                    st[m][4 * i + 2] = d * st[m][4 * i + 2] + q4.z;
                    st[m][4 * i + 3] = d * st[m][4 * i + 3] + q4.w;
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

    // ---- prologue: the first blocks' data, then their records and C B^T
    // blocks
    lds_barrier();
    lds_barrier();

    // The operands that open a block (read from its stage during the block
    // before): the decay-record fields of the bookkeeping, cf and
    // exp(lambda_r - lambda_e), raw x^T and the C fragments of the first
    // 2 ECF K-steps.
    constexpr int ECF = S::ECF;
    struct Early {
        f32x4 cfv[4];        // W (x' weights) of tokens 16 kk + 8 hi + 0..7
        bf16x8 xs[2];        // raw x^T, K-steps 0 and 1
        bf16x8 cfr[ECF][2];  // C fragments of y^T = h~ C^T, K-steps (m, u), m < ECF
        float rpv;           // F of token r (the output factor)
        float fc, rs;        // the record's factored and restart flags (uniform)
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
                    *reinterpret_cast<const f32x4 *>(v + S::W + 16 * kk + 8 * hi + 4 * w4);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            e.xs[kk] = join(lds_tr(buf, S::XR + xs_tr[0] + 1024 * kk),
                            lds_tr(buf, S::XR + xs_tr[1] + 1024 * kk));
        if constexpr (!SO) {
#pragma unroll
            for (int m = 0; m < ECF; ++m)
#pragma unroll
                for (int u = 0; u < 2; ++u) e.cfr[m][u] = lds_b128(buf, S::CS + c_rd[u] + 2048 * m);
        }
        e.rpv = v[S::F + r];
        e.fc = v[S::FLAG];
        e.rs = v[S::RESC];
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
        if constexpr (SO) {
            // the state update only: x' and B^T, the scale restart or the
            // exact block's explicit decay, h~ += B^T x'
            Ops o;
            const bool fac = uniform(e.fc) != 0.f, rescale = uniform(e.rs) != 0.f;
            bf16x8 xp[2];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
#pragma unroll
                for (int ee = 0; ee < 2; ++ee) {
                    const int kk = q >> 2, j = 2 * (q & 3) + ee;
                    xp[kk][j] = (bf16)((float)e.xs[kk][j] * e.cfv[2 * kk + (j >> 2)][j & 3]);
                }
                const int m = q >> 1, kk = q & 1;
                o.bt[m][kk] = join(lds_tr(cur, S::BS + b_tr[0] + 2048 * m + 1024 * kk),
                                   lds_tr(cur, S::BS + b_tr[1] + 2048 * m + 1024 * kk));
            }
            if (rescale || !fac) {
                const float sig_in = uniform(v[S::SIGIN]);
                const float sd = fac ? sig_in : sig_in * uniform(v[S::DELTA]);
#pragma unroll
                for (int m = 0; m < 4; ++m) st[m] *= sd;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int kk = q >> 2, m = q & 3;
                st[m] = mma32(o.bt[m][kk], xp[kk], st[m]);
                if (q == 0) load_early(stage((si + 1) % S::NST), nx);
            }
            (void)kb;
            lds_barrier();
            return;
        }
        // The block is written as a sequence of chunks fenced by scheduling
        // barriers: each chunk starts one MFMA and then issues vector work
        // that does not depend on it (the next state conversion and x'
        // during y^T = h~ C^T; the epilogue and the reads of the next
        // block's opening operands during the state update), so ALU and LDS
        // issue overlap the matrix pipeline.  A rescaled or exact block edits
        // the operands of the common path in place between the two phases.
        Ops o;
        load_late(cur, o);
        const bool fac = uniform(e.fc) != 0.f, rescale = uniform(e.rs) != 0.f;
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
                xp[kk][j] = (bf16)((float)e.xs[kk][j] * e.cfv[2 * kk + (j >> 2)][j & 3]);
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
        float f = e.rpv, dco = Dh;
        if (rescale) {
            // restart of the scale (sigma would fall below exp(-60)): the
            // state and its output so far move to sigma_in = 1
            __builtin_amdgcn_sched_barrier(0);
            const float sig_in = uniform(v[S::SIGIN]);
            acc *= sig_in;
#pragma unroll
            for (int m = 0; m < 4; ++m) st[m] *= sig_in;
        }
        if (!fac) {
            // (a side effect keeps the compiler from evaluating this rare
            // branch unconditionally with selects)
            __builtin_amdgcn_sched_barrier(0);
            // exact block: weights exp(lambda_l - lambda_s) dt_s on raw x with
            // D on the diagonal, within token r's sequence (s >= its start);
            // h~ <- sigma_in delta h~ + B^T x', sigma = 1.  The state-in
            // factor exp(lambda_r) sigma_in (<= 1: the exponent is formed
            // before exp); with packed sequences the record holds exp(lambda_r),
            // 0 past a sequence start.
            const float sig_in = uniform(v[S::SIGIN]);
            acc *= (seq_idx ? e.rpv : fast_exp(v[S::LR + r] + v[S::LE])) * sig_in;
            const float lr = v[S::LR + r];
            // s = 16 kk + 8 hi + j is kept when seg_r <= s <= r: compared as
            // 16 kk + j against per-lane bounds (immediates in the compares)
            const int rlo = (seq_idx ? (int)v[S::SEG + r] : -1) - 8 * hi, rhi = r - 8 * hi;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 wgt;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = 16 * kk + 8 * hi + j, sj = 16 * kk + j;
                    const float w = (float)o.cbv[kk][j] * fast_exp(fminf(lr - v[S::LR + s], 0.f)) *
                                        v[S::DT + s] + (!DHP && sj == rhi ? Dh : 0.f);
                    wgt[j] = (bf16)(sj <= rhi && sj >= rlo ? w : 0.f);
                }
                acc = mma32(e.xs[kk], wgt, acc);
                // the common diagonal product below then adds zeros
                o.cbv[kk] = zero_frag<bf16>();
            }
            f = 1.f;
            dco = 0.f;  // (per-head D went onto the diagonal; per-channel D stays)
            const float sd = sig_in * uniform(v[S::DELTA]);
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
        f32x4 dcol[DHP ? 4 : 1];
        if constexpr (DHP) {
            // D of this lane's columns 8 hi + (0..7) and 16 + 8 hi + (0..7)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dcol[i] = *reinterpret_cast<const f32x4 *>(dsh + 32 * wave + 16 * (i >> 1) +
                                                           8 * hi + 4 * (i & 1));
        }
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
                    if (vv * 6 / 16 == q - 2) {
                        const float dv = DHP ? dcol[vv >> 2][vv & 3] : dco;
                        acc[vv] = acc[vv] * f + dv * (float)o.xr[vv >> 3][vv & 7];
                    }
                asm volatile("" : "+v"(acc));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("" : "+v"(acc));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (GATE) {
            // the gate: this lane's z chunks sit in the staging slots its y
            // chunks will take (DMA'd by the loader three blocks ahead)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bf16x8 zv = lds_b128(cur, ys_off[i]);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[8 * i + j] *= silu_f32((float)zv[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // y of the block to the loader through this stage's staging rows;
        // the barrier then also publishes it
        y_stage(cur, acc);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
    };

    // unrolled by the stage count, so that every stage address is a literal
    // (and the two sets of opening operands alternate)
    Early ea, eb;
    load_early(stage(0), ea);
    for (int j = 0; j < nloc; j += S::NST) {
        block(kb0 + j, 0, ea, eb);
        if (j + 1 < nloc) {
            block(kb0 + j + 1, 1, eb, ea);
            if (j + 2 < nloc) {
                block(kb0 + j + 2, 2, ea, eb);
                if constexpr (S::NST > 3) {
                    if (j + 3 < nloc) block(kb0 + j + 3, 3, eb, ea);
                }
            }
        }
    }

    if (final_state) {
        // h = sigma h~ with the last block's sigma (its record is still staged)
        const float sig_out =
            uniform(reinterpret_cast<const float *>(stage((nloc - 1) % S::NST) + rec_off)[S::SIGOUT]);
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

// --------------------------------------------------------------------- launch

const char *const kFusedKernelNames[kFusedKernels] = {"k_fused_ssd"};

template <typename T>
bool fused_supported(int P, int N, int Q) {
    (void)Q;
    return sizeof(T) == 2 && N == 128 && P % 32 == 0;
}
template bool fused_supported<float>(int, int, int);
template bool fused_supported<bf16>(int, int, int);

int fused_nblk(int L) { return (L + kBlk - 1) / kBlk; }

// The loader's buffer resources are rebased every 2^shift blocks: the
// largest window whose offsets (block offset + a block's rows) stay under
// 2^31 bytes on the widest stream.  SSD_FUSED_WINDOW_SHIFT forces a smaller
// window (a diagnostic: the tests cross many window boundaries with it).
static int window_shift_for(size_t row_bytes) {
    int s = 0;
    while (s < 24 && (((size_t)1 << (s + 1)) + 1) * kBlk * row_bytes < ((size_t)1 << 31)) ++s;
    return s;
}
int fused_window_shift(const ForwardArgs &a) {
    size_t row = (size_t)a.H * a.P * 2;
    row = row > (size_t)a.G * a.N * 2 ? row : (size_t)a.G * a.N * 2;
    row = row > (size_t)a.H * 4 ? row : (size_t)a.H * 4;
    int s = window_shift_for(row);
    if (const char *e = getenv("SSD_FUSED_WINDOW_SHIFT")) {
        const int f = atoi(e);
        if (f >= 2 && f < s) s = f;
    }
    return s;
}
bool fused_row_fits(size_t row_bytes) { return window_shift_for(row_bytes) >= 3; }

// The segments of a forward of nblk blocks cut into nseg: segment 0 has
// `first` blocks and runs while the state-only pass covers segments 1 ..
// nseg - 2, every later segment `len` blocks.  The two kernels of the
// first phase share the chip and slow each other; measured on the 8-group
// layer, segment 0 as long as the others balances the phases best (0.215 ms
// against 0.2165 at 80% and 0.226 at 150%).  SSD_FUSED_SEG0_PCT sets the
// percentage (a diagnostic).
static SegPlan seg_plan(int nblk, int nseg) {
    SegPlan p;
    p.nseg = nseg;
    p.base = 0;
    if (nseg <= 1) {
        p.first = nblk;
        p.len = nblk;
        return p;
    }
    int pct = 100;
    if (const char *e = getenv("SSD_FUSED_SEG0_PCT")) {
        const int v = atoi(e);
        if (v >= 10 && v <= 200) pct = v;
    }
    // len ~ nblk / (nseg - 1 + pct / 100), first = what is left
    p.len = (int)(((long)nblk * 100 + (long)(nseg - 1) * 100 + pct - 1) / ((long)(nseg - 1) * 100 + pct));
    if (p.len < 1) p.len = 1;
    p.first = nblk - (nseg - 1) * p.len;
    while (p.first < 1 && p.len > 1) {
        --p.len;
        p.first = nblk - (nseg - 1) * p.len;
    }
    return p;
}

template <int PB, int EPI>
static void launch_fused_epi(const ForwardArgs &a, hipStream_t stream, SegPlan plan, int nz) {
    constexpr bool SO = (EPI & kEpiState) != 0;
    typedef Fused<PB, SO> S;
    hipLaunchKernelGGL((k_fused_ssd<PB, EPI>), dim3(a.H * a.P / PB, a.batch, nz), dim3(S::NT), 0,
                       stream, (const bf16 *)a.x, a.dt, a.A, (const bf16 *)a.B, (const bf16 *)a.C,
                       a.D, a.init, a.final_state, (bf16 *)a.y, a.L, a.H, a.G, a.P,
                       fused_nblk(a.L), a.dtp, a.seq_idx, (const bf16 *)a.z, fused_window_shift(a),
                       plan, a.seg_buf, a.seg_buf, a.seg_logdec);
}

template <int PB>
static void launch_main_epi(const ForwardArgs &a, hipStream_t stream, SegPlan plan, int nz) {
    const int epi = (a.D_hdim && a.D ? kEpiDhp : 0) | (a.z ? kEpiGate : 0);
    switch (epi) {
        case kEpiDhp: launch_fused_epi<PB, kEpiDhp>(a, stream, plan, nz); break;
        case kEpiGate: launch_fused_epi<PB, kEpiGate>(a, stream, plan, nz); break;
        case kEpiDhp | kEpiGate: launch_fused_epi<PB, kEpiDhp | kEpiGate>(a, stream, plan, nz); break;
        default: launch_fused_epi<PB, 0>(a, stream, plan, nz); break;
    }
}

// One pass, or with segments two phases:
//   1. the main pass over segment 0 (on `stream`; it leaves its state in
//      seg_buf[0]) and, at the same time on the auxiliary stream a.side,
//      the state-only pass over segments 1 .. nseg - 2 (forked from and
//      joined back to `stream` with two events; without a.side the two
//      run one after the other on `stream`);
//   2. the main pass over segments 1 .. nseg - 1.
template <int PB>
static hipError_t launch_fused_main(const ForwardArgs &a, hipStream_t stream, hipEvent_t *events) {
    const int nblk = fused_nblk(a.L);
    SegPlan plan = seg_plan(nblk, PB == 128 ? a.nseg : 1);
    if (plan.nseg <= 1) {
        launch_main_epi<PB>(a, stream, plan, 1);
        return hipSuccess;
    }
    hipError_t err;
    const bool fork = a.side != nullptr && plan.nseg > 2;
    hipStream_t so_stream = fork ? a.side : stream;
    if (fork) {
        if ((err = hipEventRecord(a.ev_fork, stream)) != hipSuccess) return err;
        if ((err = hipStreamWaitEvent(a.side, a.ev_fork, 0)) != hipSuccess) return err;
    }
    SegPlan so = plan;
    so.base = 1;
    if constexpr (PB == 128) {
        if (plan.nseg > 2) launch_fused_epi<PB, kEpiState>(a, so_stream, so, plan.nseg - 2);
    }
    launch_main_epi<PB>(a, stream, plan, 1);
    if (fork) {
        if ((err = hipEventRecord(a.ev_join, a.side)) != hipSuccess) return err;
        if ((err = hipStreamWaitEvent(stream, a.ev_join, 0)) != hipSuccess) return err;
    }
    if (events && (err = hipEventRecord(events[1], stream)) != hipSuccess) return err;
    SegPlan rest = plan;
    rest.base = 1;
    launch_main_epi<PB>(a, stream, rest, plan.nseg - 1);
    return hipSuccess;
}

// Columns per workgroup.  One workgroup per compute unit is the target
// (two 32-column workgroups on one compute unit slow each other down more
// than one 64-column workgroup's two waves do): 128 columns (four waves over
// two heads of one B/C group, which share the staged C and B rows) once
// 64-column workgroups would outnumber the 256 compute units; 64 (two
// waves) once 32-column ones would; else 32 (one wave).
static int pick_pb(const ForwardArgs &a) {
    const long cols = (long)a.batch * a.H * a.P;
    if (a.nseg > 1) return 128;
    if (a.P == 64 && a.H % 2 == 0 && (a.H / a.G) % 2 == 0 && cols / 64 > 256) return 128;
    if (a.P % 64 == 0 && cols / 32 > 256) return 64;
    return 32;
}

// Sequence segments of the fused forward.  A layer with few 128-column
// groups (batch x heads x headdim / 128 below 128) leaves most compute units
// idle when every workgroup walks the whole sequence, each issue-bound on
// one pass.  The sequence is then cut into nseg segments, with
// (nseg - 1) x groups <= 256 and at least 64 blocks per later segment: while
// the main pass runs segment 0, a state-only pass forms the state segments
// 1 .. nseg - 2 leave from zero; then the main pass runs the other
// segments, each from its entering state, which it chains from those states
// as it starts.  Needs the 128-column layout (headdim 64, even heads per
// group).  SSD_FUSED_SEGMENTS=n forces n segments where the layout allows
// (a diagnostic for comparing the two).
int fused_segments(int batch, int L, int H, int G, int P) {
    if (!(P == 64 && H % 2 == 0 && (H / G) % 2 == 0)) return 1;
    const int nblk = fused_nblk(L);
    const long chains = (long)batch * H * P / 128;
    int n = 1;
    if (chains < 128) {
        n = 1 + (int)(256 / chains);
        if (n > 9) n = 9;
        while (n > 1 && nblk / n < 64) --n;
        if (n == 2) n = 1;     // (no segment would overlap the first)
    }
    if (const char *e = getenv("SSD_FUSED_SEGMENTS")) {
        int f = atoi(e);
        if (f >= 1) {
            if (f > 64) f = 64;
            while (f > 1 && nblk / f < 4) --f;
            n = f;
        }
    }
    if (n > nblk) n = nblk;
    return n;
}
int fused_kernel_count(int nseg) { return nseg > 1 ? 2 : 1; }
// (the first phase's two kernels run on two streams and are timed together)
const char *const kFusedSegKernelNames[2] = {"k_fused_ssd_state+seg0", "k_fused_ssd"};

// The fused forward: one launch, or two with segments.
template <typename T>
hipError_t launch_fused_forward(const ForwardArgs &a, hipStream_t stream, hipEvent_t *events) {
    if (sizeof(T) != 2) return hipErrorInvalidValue;  // bf16 only (fused_supported)
    hipError_t err;
    if (events && (err = hipEventRecord(events[0], stream)) != hipSuccess) return err;
    switch (pick_pb(a)) {
        case 128: err = launch_fused_main<128>(a, stream, events); break;
        case 64: err = launch_fused_main<64>(a, stream, events); break;
        default: err = launch_fused_main<32>(a, stream, events); break;
    }
    if (err != hipSuccess) return err;
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (events &&
        (err = hipEventRecord(events[fused_kernel_count(a.nseg)], stream)) != hipSuccess)
        return err;
    return hipSuccess;
}

template hipError_t launch_fused_forward<float>(const ForwardArgs &, hipStream_t, hipEvent_t *);
template hipError_t launch_fused_forward<bf16>(const ForwardArgs &, hipStream_t, hipEvent_t *);

}  // namespace ssd
