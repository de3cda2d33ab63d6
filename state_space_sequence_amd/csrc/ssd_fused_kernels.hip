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
// Workgroup = NW waves, wave w owns headdim tile w (16 columns) of the block
// of PB = 16 NW columns.  Per 32-token block:
//   stage (next block, double-buffered LDS): C and B rows straight from
//          global memory into LDS (global_load_lds), x raw and decay-scaled
//          (x'_s = exp(lambda_e - lambda_s) dt_s x_s) through registers, the
//          diagonal block of C B^T (precomputed, in fragment order);
//          per-token decay vectors two blocks ahead;
//   output 2 row tiles x the wave's headdim tile: C h^T with h^T taken
//          straight from the state registers as the MFMA B operand, then the
//          diagonal block, then D x;
//   state  h <- exp(lambda_e) h + B^T x'.
// Operands that the MFMA needs transposed (B^T, x^T) are read from row-major
// LDS with ds_read_b64_tr_b16: within each 16-lane group, lane 4a+c receives
// element c of the 8-byte reads of lanes a, a+4, a+8, a+12, so pointing lane
// j at row kbase + j/4, columns 4 (j%4) .. +3 of a row-major [k][n] tile
// hands lane n the column n for k = kbase .. kbase+3.
//
// The diagonal block normally runs as
//   exp(lambda_l - lambda_e) * (exp(lambda_e) C h^T + mask(C B^T) x'),
// so its mask is a select on C B^T.  When the block's total decay exceeds
// exp(-40) that form could overflow, and the block is evaluated with the
// exact per-element weights exp(lambda_l - lambda_s) dt_s (s > l exactly 0,
// the upper-triangle protection of the Kernel 5 page) on raw x, with D on
// the diagonal.
#include "ssd_device.hpp"
#include "ssd_kernels.hpp"

namespace ssd {

constexpr int kBlk = 32;            // tokens per block
constexpr float kSafeDecay = 40.f;  // max -lambda_e for the factored diagonal
// s_waitcnt immediate for "vmcnt(0)" alone on gfx9-family targets:
// vmcnt = 0, expcnt = 7 and lgkmcnt = 15 (both at their no-wait maximum).
constexpr int kWaitVmcnt0 = 0x0F70;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ bf16x4 lds_tr(const unsigned char *base, int byte_off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)((lds_u8 *)(base) + byte_off));
}
__device__ __forceinline__ bf16x4 lds_b64(const unsigned char *base, int byte_off) {
    return *reinterpret_cast<const bf16x4 *>(base + byte_off);
}
__device__ __forceinline__ bf16x8 join(bf16x4 lo, bf16x4 hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ void dma16(const void *gsrc, unsigned char *lds_wave_base) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)gsrc,
                                     (__attribute__((address_space(3))) void *)(lds_wave_base),
                                     16, 0, 0);
}

template <int PB>
struct Fused {
    static constexpr int NW = PB / 16;                 // waves
    static constexpr int NT = 64 * NW;                 // threads
    static constexpr int N = 128;                      // dstate
    static constexpr int RC = N / 8 + 1;               // chunks per C/B row (+1 pad)
    static constexpr int RB = RC * 16;                 // bytes per C/B row in LDS
    static constexpr int CB_CHUNKS = kBlk * RC;        // 544
    static constexpr int CB_DMA = (CB_CHUNKS + 63) / 64;   // wave DMAs per C (or B)
    static constexpr int DPW = (CB_DMA + NW - 1) / NW; // of which per wave
    static constexpr int XC = PB / 8;                  // chunks per x row
    static constexpr int XPC = XC + 2;                 // LDS pitch (chunks)
    static constexpr int XB = XPC * 16;                // bytes per x row in LDS
    // one staging buffer
    static constexpr int CS = 0;
    static constexpr int BS = CS + CB_DMA * 1024;
    static constexpr int XR = BS + CB_DMA * 1024;
    static constexpr int XS = XR + kBlk * XB;
    static constexpr int CBF = XS + kBlk * XB;         // 2 x 1 KB of C B^T fragments
    static constexpr int BUF = CBF + 2048;
    // per-block vectors (floats), three of them in flight
    enum { LHI = 0, LLO = 32, DT = 64, CF = 96, RP = 128, EX = 160, DELTA = 192, FLAG = 193,
           VFLOATS = 196 };
    static constexpr int LDS = 2 * BUF + 3 * VFLOATS * 4;
    static_assert(BUF % 16 == 0, "alignment");
    static_assert(LDS <= 65536, "static LDS");
    static_assert(XC * kBlk == NT, "one x chunk per thread");
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
    // Two staging buffers and the vectors as separate LDS objects: the
    // compiler can then see that the DMA filling one buffer never aliases the
    // reads of the other, and does not wait for the DMA before those reads.
    __shared__ __align__(16) unsigned char sbuf0[S::BUF];
    __shared__ __align__(16) unsigned char sbuf1[S::BUF];
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
    const size_t GN = (size_t)G * N, HP = (size_t)H * P;

    // ---- per-lane LDS byte offsets (relative to a staging buffer)
    const int c_rd = (r * S::RC + (q >> 1)) * 16 + (q & 1) * 8;          // C rows, lt 0
    const int b_tr = ((8 * q + (r >> 2)) * S::RC + ((r & 3) >> 1)) * 16 + (r & 1) * 8;
    const int xs_tr = ((8 * q + (r >> 2)) * S::XPC + 2 * pt + ((r & 3) >> 1)) * 16 + (r & 1) * 8;
    const int xr_skip = ((4 * q + (r >> 2)) * S::XPC + 2 * pt + ((r & 3) >> 1)) * 16 + (r & 1) * 8;
    const int cbf_rd = lane * 16;
    // diagonal-block masks: fragment element j of lane (r, q) is column 8q+j
    u32x4 mask[2];
#pragma unroll
    for (int lt = 0; lt < 2; ++lt)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int row = 16 * lt + r, s0 = 8 * q + 2 * d;
            mask[lt][d] = (s0 <= row ? 0x0000FFFFu : 0u) | (s0 + 1 <= row ? 0xFFFF0000u : 0u);
        }
    // x staging: one 16-byte chunk per thread
    const int xs_row = tid / S::XC, xs_chunk = tid % S::XC;
    const int x_st = (xs_row * S::XPC + xs_chunk) * 16;
    // C / B DMA: wave w issues DMAs w, w + NW, ... of the CB_DMA per matrix
    int dma_row[S::DPW], dma_chunk[S::DPW];
#pragma unroll
    for (int i = 0; i < S::DPW; ++i) {
        const int pos = 64 * (wave + NW * i) + lane;
        dma_row[i] = pos / S::RC;
        const int slot = pos % S::RC;
        dma_chunk[i] = slot < N / 8 ? slot : 0;  // pad slot: any valid chunk of the row
    }

    // ---- register-resident state: st[n] = S^T[16 n + 4 q + e][p0 + 16 pt + r]
    f32x4 st[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        st[n] = zero4();
        if (init) {
            const float4 v = *reinterpret_cast<const float4 *>(
                init + (bh * P + p0 + 16 * pt + r) * N + 16 * n + 4 * q);
            st[n] = f32x4{v.x, v.y, v.z, v.w};
        }
    }

    auto V = [&](int kb) -> float * { return svec + (kb % 3) * S::VFLOATS; };
    auto vec_load = [&](int kb, float &lh, float &ll, float &dv) {
        const size_t o = (bh * nblk + kb) * kBlk + lane;
        lh = lam_hi[o];
        ll = lam_lo[o];
        dv = dtb[o];
    };
    auto vec_store = [&](int kb, float lh, float ll, float dv) {
        float *v = V(kb);
        const float eh = __shfl(lh, kBlk - 1, kWave), el = __shfl(ll, kBlk - 1, kWave);
        const float neg_e = -(eh + el);
        v[S::LHI + lane] = lh;
        v[S::LLO + lane] = ll;
        v[S::DT + lane] = dv;
        v[S::CF + lane] = fast_exp(prefix_diff(eh, el, lh, ll)) * dv;
        v[S::RP + lane] = neg_e <= kSafeDecay ? fast_exp(prefix_diff(lh, ll, eh, el)) : 0.f;
        v[S::EX + lane] = fast_exp(lh + ll);
        if (lane == kBlk - 1) {
            v[S::DELTA] = fast_exp(eh + el);
            v[S::FLAG] = neg_e <= kSafeDecay ? 1.f : 0.f;
        }
    };
    // C, B rows and the C B^T fragments of block kb into the buffer at `buf`
    auto dma_block = [&](int kb, unsigned char *buf) {
        const int t0 = kb * kBlk;
        const int lim = L - 1 - t0;
        const bf16 *crow0 = Cm + ((size_t)b * L + t0) * GN + (size_t)g * N;
        const bf16 *brow0 = Bm + ((size_t)b * L + t0) * GN + (size_t)g * N;
#pragma unroll
        for (int i = 0; i < S::DPW; ++i) {
            const int d = wave + NW * i;
            if (d < S::CB_DMA && 64 * d + lane < S::CB_CHUNKS) {
                const size_t off = (size_t)min(dma_row[i], lim) * GN + 8 * dma_chunk[i];
                dma16(crow0 + off, buf + S::CS + 1024 * d);
                dma16(brow0 + off, buf + S::BS + 1024 * d);
            }
        }
        if (wave < 2)
            dma16(cbf + (((size_t)b * nblk + kb) * G + g) * (kBlk * kBlk) + 8 * (64 * wave + lane),
                  buf + S::CBF + 1024 * wave);
    };
    auto x_load = [&](int kb) -> bf16x8 {
        const int t = min(kb * kBlk + xs_row, L - 1);
        return load_frag(x + ((size_t)b * L + t) * HP + h * P + p0 + 8 * xs_chunk);
    };
    auto x_store = [&](int kb, unsigned char *buf, bf16x8 xv) {
        const float cf = V(kb)[S::CF + xs_row];
        bf16x8 xsv;
#pragma unroll
        for (int j = 0; j < 8; ++j) xsv[j] = (bf16)((float)xv[j] * cf);
        *reinterpret_cast<bf16x8 *>(buf + S::XR + x_st) = xv;
        *reinterpret_cast<bf16x8 *>(buf + S::XS + x_st) = xsv;
    };

    // ---- prologue
    {
        float lh, ll, dv;
        if (wave == 0 && lane < kBlk) {
            vec_load(0, lh, ll, dv);
            vec_store(0, lh, ll, dv);
        }
        if (wave == (1 % NW) && lane < kBlk && nblk > 1) {
            vec_load(1, lh, ll, dv);
            vec_store(1, lh, ll, dv);
        }
        dma_block(0, sbuf0);
        const bf16x8 xv = x_load(0);
        __syncthreads();
        x_store(0, sbuf0, xv);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    }

    auto block = [&](int kb, unsigned char *cur, unsigned char *nxt) {
        const bool more1 = kb + 1 < nblk, more2 = kb + 2 < nblk;
        const bool vec_wave = more2 && wave == (kb + 2) % NW && lane < kBlk;
        bf16x8 xv_next = zero_frag<bf16>();
        float nlh = 0.f, nll = 0.f, ndv = 0.f;
        if (more1) {
            dma_block(kb + 1, nxt);
            xv_next = x_load(kb + 1);
        }
        if (vec_wave) vec_load(kb + 2, nlh, nll, ndv);

        const float *v = V(kb);
        const bool factored = v[S::FLAG] != 0.f;
        const float delta = v[S::DELTA];

        // -------- outputs: C h^T for both 16-row tiles
        f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 hb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hb[e] = (bf16)st[2 * ks][e];
                hb[4 + e] = (bf16)st[2 * ks + 1][e];
            }
            const bf16x8 a0 = join(lds_b64(cur, S::CS + c_rd + 64 * ks),
                                   lds_b64(cur, S::CS + c_rd + 64 * ks + 32));
            const bf16x8 a1 = join(lds_b64(cur, S::CS + c_rd + 16 * S::RB + 64 * ks),
                                   lds_b64(cur, S::CS + c_rd + 16 * S::RB + 64 * ks + 32));
            acc0 = Mma<bf16>::mma(a0, hb, acc0);
            acc1 = Mma<bf16>::mma(a1, hb, acc1);
        }
        const bf16x8 xs = join(lds_tr(cur, S::XS + xs_tr), lds_tr(cur, S::XS + xs_tr + 4 * S::XB));
        if (factored) {
            acc0 *= delta;
            acc1 *= delta;
            bf16x8 m0 = *reinterpret_cast<const bf16x8 *>(cur + S::CBF + cbf_rd);
            bf16x8 m1 = *reinterpret_cast<const bf16x8 *>(cur + S::CBF + 1024 + cbf_rd);
            m0 = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, m0) & mask[0]);
            m1 = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, m1) & mask[1]);
            acc0 = Mma<bf16>::mma(m0, xs, acc0);
            acc1 = Mma<bf16>::mma(m1, xs, acc1);
            const f32x4 rp0 = *reinterpret_cast<const f32x4 *>(v + S::RP + 4 * q);
            const f32x4 rp1 = *reinterpret_cast<const f32x4 *>(v + S::RP + 16 + 4 * q);
            const bf16x4 x0 = lds_tr(cur, S::XR + xr_skip);
            const bf16x4 x1 = lds_tr(cur, S::XR + xr_skip + 16 * S::XB);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc0[e] = acc0[e] * rp0[e] + Dh * (float)x0[e];
                acc1[e] = acc1[e] * rp1[e] + Dh * (float)x1[e];
            }
        } else {
            const f32x4 ex0 = *reinterpret_cast<const f32x4 *>(v + S::EX + 4 * q);
            const f32x4 ex1 = *reinterpret_cast<const f32x4 *>(v + S::EX + 16 + 4 * q);
            acc0 *= ex0;
            acc1 *= ex1;
            const bf16x8 xb =
                join(lds_tr(cur, S::XR + xs_tr), lds_tr(cur, S::XR + xs_tr + 4 * S::XB));
#pragma unroll
            for (int lt = 0; lt < 2; ++lt) {
                const int row = 16 * lt + r;
                const bf16x8 cbv =
                    *reinterpret_cast<const bf16x8 *>(cur + S::CBF + 1024 * lt + cbf_rd);
                const float lh = v[S::LHI + row], ll = v[S::LLO + row];
                bf16x8 m;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = 8 * q + j;
                    float w = 0.f;
                    if (s <= row) {
                        w = (float)cbv[j] *
                            fast_exp(prefix_diff(lh, ll, v[S::LHI + s], v[S::LLO + s])) *
                            v[S::DT + s];
                        if (s == row) w += Dh;
                    }
                    m[j] = (bf16)w;
                }
                if (lt == 0)
                    acc0 = Mma<bf16>::mma(m, xb, acc0);
                else
                    acc1 = Mma<bf16>::mma(m, xb, acc1);
            }
        }
        {
            const int t0 = kb * kBlk;
            bf16 *yb = y + ((size_t)b * L + t0) * HP + h * P + p0 + 16 * pt + r;
            if (t0 + kBlk <= L) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    yb[(size_t)(4 * q + e) * HP] = (bf16)acc0[e];
                    yb[(size_t)(16 + 4 * q + e) * HP] = (bf16)acc1[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (t0 + 4 * q + e < L) yb[(size_t)(4 * q + e) * HP] = (bf16)acc0[e];
                    if (t0 + 16 + 4 * q + e < L) yb[(size_t)(16 + 4 * q + e) * HP] = (bf16)acc1[e];
                }
            }
        }

        // -------- state: h <- exp(lambda_e) h + B^T x'
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const bf16x8 a = join(lds_tr(cur, S::BS + b_tr + 32 * n),
                                  lds_tr(cur, S::BS + b_tr + 4 * S::RB + 32 * n));
            st[n] = Mma<bf16>::mma(a, xs, st[n] * delta);
        }

        // -------- stage the next block, vectors two ahead
        if (more1) x_store(kb + 1, nxt, xv_next);
        if (vec_wave) vec_store(kb + 2, nlh, nll, ndv);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    };

    for (int kb = 0; kb < nblk; kb += 2) {
        block(kb, sbuf0, sbuf1);
        if (kb + 1 < nblk) block(kb + 1, sbuf1, sbuf0);
    }

    if (final_state) {
#pragma unroll
        for (int n = 0; n < 8; ++n)
            *reinterpret_cast<float4 *>(final_state + (bh * P + p0 + 16 * pt + r) * N + 16 * n +
                                        4 * q) = make_float4(st[n][0], st[n][1], st[n][2], st[n][3]);
    }
}

// Diagonal 32x32 block of C B^T for every 32-token block and group, bf16,
// stored in the MFMA A-fragment order the fused kernel reads: for row tile
// lt and lane (r, q), the 8 values C B^T[16 lt + r][8 q .. 8 q + 7] are the
// 16 bytes at ((lt * 64) + q * 16 + r) * 16.  The tile above the diagonal
// (rows 0-15, columns 16-31) is written as zeros.
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
    // D layout: lane (r, q) holds rows 16 lt + 4 q + e, column 16 ct + r
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rr = 4 * q + e, s = 16 * ct + r;
        out[(lt * 64 + (s >> 3) * 16 + rr) * 8 + (s & 7)] = (bf16)acc[e];
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
