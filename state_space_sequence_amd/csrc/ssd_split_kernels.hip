// ssd_split_kernels.hip -- the chunked SSD forward as five kernels, one per
// step of the chunked algorithm (burn-mamba `mamba2/ssd/serial.rs`, kernels
// 1-5; burn-mamba `Mamba2SsdInput` rustdoc, `ssd_minimal` Steps 1-4):
//
//   k1_dA_cumsum      per-chunk inclusive prefix sum of dt*A  (`k1_ssd_chunk_cumsum`)
//   k2_chunk_cb       C B^T per chunk and group, causal blocks (`k2_ssd_bmm`)
//   k3_chunk_state    zero-initial state of every chunk, Eq. 20 (`k3_ssd_chunk_state`)
//   k4_state_passing  inter-chunk recurrence, Eq. 22            (`k4_ssd_state_passing`)
//   k5_chunk_scan     y = state-to-output (Eq. 23) + masked intra-chunk
//                     product + D skip                           (`k5_ssd_chunk_scan`)
//
// These kernels accept every supported shape.  Layouts of the workspace
// intermediates (all fp32):
//   acum [b][H][nc][Q]   prefix sums of dt*A inside each chunk (0 past
//                        seqlen), as a two-float pair: the fp64 prefix rounded
//                        to fp32 (hi) and the rounding remainder (lo)
//   dtT  [b][H][nc][Q]   dt re-laid out per chunk (0 past seqlen), after the
//                        time-step preprocessing when it is on; every later
//                        kernel reads dt from here
//   cb   [b][nc][G][Q][Q] C B^T of the chunk (only s-tiles <= l-tile written)
//   S    [b][nc][H][P][N] chunk states, overwritten by k4 with the state
//                         entering each chunk
//   segst [b][nc][Q] int32 packed sequences only: for each token, its
//                         position in the chunk of the last sequence start at
//                         or before it in that chunk (-1: none)
//
// Packed sequences (seq_idx, as the fla layer's `mamba_chunk_scan_combined`
// takes it): token t > 0 whose label differs from token t - 1's starts a new
// sequence, and the state entering it is zero.  In the chunked form a start
// at position st of a chunk cuts every decay path that crosses it: the
// intra-chunk weights keep sources s >= segst[l] only, the entering state
// reaches only the rows before the chunk's first start, the chunk's own state
// collects only its last sequence (s >= segst[Q - 1]), and a chunk with a
// start passes nothing of the state entering it on (decay 0 in k4).
#include "ssd_device.hpp"
#include "ssd_kernels.hpp"

namespace ssd {

// --------------------------------------------------------------------- k1
// grid (nc, ceil(H/16), b), 256 threads.  A block stages dt for 16 heads of
// one chunk through LDS (coalesced over heads), then every wave scans 4 heads:
// each lane sums up to 4 consecutive tokens, the wave scans the lane totals.
//
// The prefix is accumulated in fp64 (dt*A is exact in fp64) and stored as
// hi = fp32(prefix), lo = fp32(prefix - hi).  Consumers need differences
// acum_l - acum_s of two prefixes that can be large (hundreds) while their
// difference is small; in plain fp32 that subtraction loses |acum| * 2^-24
// absolutely, which is the instability the stable segment sum of the fla
// layer (`segment_sum`) avoids.  (hi_l - hi_s) + (lo_l - lo_s) is accurate to
// a few ulps of the difference itself.
//
// With packed sequences the blocks of the first head group also write the
// chunk's segst row: the start flags, then an inclusive max-scan of their
// positions over the chunk (Q <= 256 tokens, one per thread).
__global__ void __launch_bounds__(256)
k1_dA_cumsum(const float *__restrict__ dt, const DtProc dtp, const float *__restrict__ A,
             float *__restrict__ acum_hi, float *__restrict__ acum_lo,
             float *__restrict__ dtT, int L, int H, int nc, int Q,
             const int *__restrict__ seq_idx, int *__restrict__ segst) {
    __shared__ float s_dt[16][257];
    const int c = blockIdx.x, h0 = blockIdx.y * 16, b = blockIdx.z;
    const int tid = threadIdx.x;
    if (seq_idx && blockIdx.y == 0) {
        __shared__ int s_st[256];
        const int t = c * Q + tid;
        const bool start = tid < Q && t > 0 && t < L &&
                           seq_idx[(size_t)b * L + t] != seq_idx[(size_t)b * L + t - 1];
        s_st[tid] = start ? tid : -1;
        __syncthreads();
        for (int d = 1; d < Q; d <<= 1) {
            const int o = tid >= d ? s_st[tid - d] : -1;
            __syncthreads();
            s_st[tid] = max(s_st[tid], o);
            __syncthreads();
        }
        if (tid < Q) segst[((size_t)b * nc + c) * Q + tid] = s_st[tid];
    }
    const int j = tid & 15;
    for (int r = tid >> 4; r < Q; r += 16) {
        const int h = h0 + j, t = c * Q + r;
        float v = 0.f;
        if (h < H && t < L) {
            v = dt[((size_t)b * L + t) * H + h];
            if (dtp.on) v = dt_process(v, dtp.bias ? dtp.bias[h] : 0.f, dtp.softplus, dtp.lo, dtp.hi);
        }
        s_dt[j][r] = v;
    }
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63;
    const int E = Q > 64 ? Q / 64 : 1;
    for (int jj = 0; jj < 4; ++jj) {
        const int hl = wave * 4 + jj, h = h0 + hl;
        if (h >= H) break;
        const double Ah = (double)A[h];
        double a[4];
        float d[4];
        double run = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = 0.0;
            d[e] = 0.f;
            const int idx = lane * E + e;
            if (e < E && idx < Q) {
                d[e] = s_dt[hl][idx];
                run += (double)d[e] * Ah;
                a[e] = run;
            }
        }
        const double incl = wave_inclusive_scan_f64(run, lane);
        double excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 0.0;
        const size_t base = ((size_t)(b * H + h) * nc + c) * Q;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = lane * E + e;
            if (e < E && idx < Q) {
                const double v = excl + a[e];
                const float hi = (float)v;
                acum_hi[base + idx] = hi;
                acum_lo[base + idx] = (float)(v - (double)hi);
                dtT[base + idx] = d[e];
            }
        }
    }
}

// --------------------------------------------------------------------- k2
// grid (npairs, nc*G, b), 256 threads.  Block `pair` covers an (l-block of 64,
// s-block of 64) pair with s-block <= l-block; wave w takes the 16 rows
// l0 = 64*lb + 16*w against four 16-column s-tiles.  Operands are read
// straight from global memory: rows of C and B are contiguous in n, which is
// the MFMA k dimension here.
template <typename T>
__global__ void __launch_bounds__(256)
k2_chunk_cb(const T *__restrict__ Bm, const T *__restrict__ Cm,
            float *__restrict__ cb, int L, int G, int N, int nc, int Q) {
    constexpr int VEC = Mma<T>::VEC, KS = Mma<T>::KS;
    int pair = blockIdx.x, lb = 0;
    while ((lb + 1) * (lb + 2) / 2 <= pair) ++lb;
    const int sb = pair - lb * (lb + 1) / 2;
    const int c = blockIdx.y / G, g = blockIdx.y % G, b = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int l0 = lb * 64 + wave * 16;
    if (l0 >= Q) return;
    const int tl = c * Q + l0 + r;
    const T *crow = Cm + (((size_t)b * L + tl) * G + g) * N;
    int s0[4];
    bool act[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        s0[st] = sb * 64 + st * 16;
        act[st] = s0[st] < Q && s0[st] <= l0 + 15;
    }
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    for (int k0 = 0; k0 < N; k0 += KS) {
        const int k = k0 + VEC * q;
        const bool kin = k < N;
        typename Mma<T>::frag a = (tl < L && kin) ? load_frag(crow + k) : zero_frag<T>();
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (!act[st]) continue;
            const int ts = c * Q + s0[st] + r;
            typename Mma<T>::frag bb =
                (ts < L && kin) ? load_frag(Bm + (((size_t)b * L + ts) * G + g) * N + k)
                                : zero_frag<T>();
            acc[st] = Mma<T>::mma(a, bb, acc[st]);
        }
    }
    const size_t base = ((size_t)(b * nc + c) * G + g) * Q;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        if (!act[st]) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            cb[(base + l0 + 4 * q + i) * Q + s0[st] + r] = acc[st][i];
    }
}

// --------------------------------------------------------------------- k3
// grid (nc, H * ntile_groups, b), 256 threads, dynamic LDS.
// S[p][n] = sum_s x[s][p] * w_s * B[s][n],  w_s = exp(acum_end - acum_s) dt_s.
// The contraction runs over tokens s, which is the slow index of both x and
// B in memory, so 32-token slabs of both are staged transposed in LDS
// (XT[p][s], BT[n][s]) with w_s folded into x on the way in; fragments are
// then 16-byte LDS reads.  Each wave owns up to kK3TilesPerWave 16x16 tiles.
template <typename T>
__global__ void __launch_bounds__(256)
k3_chunk_state(const T *__restrict__ x, const T *__restrict__ Bm,
               const float *__restrict__ acum_hi, const float *__restrict__ acum_lo,
               const float *__restrict__ dtT, float *__restrict__ S, int L, int H,
               int G, int P, int N, int nc, int Q, const int *__restrict__ segst) {
    constexpr int VEC = Mma<T>::VEC, KS = Mma<T>::KS;
    constexpr int KB = 32;
    // fp32: rows of 32 floats, two to a 64-float line, 4-float chunks XOR-swizzled per row; the staging stores
    // (4 consecutive tokens of 16 rows 4 apart per instruction) and the 16-byte fragment reads (16 consecutive
    // rows) then fall on distinct banks at headdim 64 (2-way at dstate 128).  bf16: padded rows.
    constexpr bool SW = sizeof(T) == 4;
    constexpr int PITCH = SW ? KB : KB + 16 / (int)sizeof(T);
    constexpr int TPW = kK3TilesPerWave;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T *XT = reinterpret_cast<T *>(smem_raw);
    T *BT = XT + (size_t)P * PITCH;
    auto at = [](int row, int s) -> int {
        if constexpr (SW) {
            const int g = ((row >> 1) + (row >> 5)) & 15;
            return (row >> 1) * 64 + 4 * ((((row & 1) * 8 + (s >> 2)) ^ g) & 15) + (s & 3);
        } else {
            return row * PITCH + s;
        }
    };

    const int c = blockIdx.x, h = blockIdx.y % H, tg = blockIdx.y / H, b = blockIdx.z;
    const int g = h / (H / G);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;
    const int ntn = N / 16, ntiles = (P / 16) * ntn;
    const float *ah = acum_hi + ((size_t)(b * H + h) * nc + c) * Q;
    const float *al = acum_lo + ((size_t)(b * H + h) * nc + c) * Q;
    const float *dc = dtT + ((size_t)(b * H + h) * nc + c) * Q;
    const float end_hi = ah[Q - 1], end_lo = al[Q - 1];
    // packed sequences: only the chunk's last sequence reaches its end state
    const int s_first = segst ? segst[((size_t)b * nc + c) * Q + Q - 1] : -1;

    f32x4 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = zero4();

    for (int s0 = 0; s0 < Q; s0 += KB) {
        __syncthreads();
        const int pv = P / VEC;
        for (int v = tid; v < KB * pv; v += 256) {
            const int sl = v / pv, p0 = (v % pv) * VEC;
            const int s = s0 + sl, t = c * Q + s;
            const bool in = s < Q && t < L && s >= s_first;
            float w = 0.f;
            typename Mma<T>::frag f = zero_frag<T>();
            if (in) {
                w = fast_exp(prefix_diff(end_hi, end_lo, ah[s], al[s])) * dc[s];
                f = load_frag(x + (((size_t)b * L + t) * H + h) * P + p0);
            }
#pragma unroll
            for (int jj = 0; jj < VEC; ++jj)
                XT[at(p0 + jj, sl)] = from_f32<T>(to_f32(f[jj]) * w);
        }
        const int nv = N / VEC;
        for (int v = tid; v < KB * nv; v += 256) {
            const int sl = v / nv, n0 = (v % nv) * VEC;
            const int s = s0 + sl, t = c * Q + s;
            typename Mma<T>::frag f = zero_frag<T>();
            if (s < Q && t < L) f = load_frag(Bm + (((size_t)b * L + t) * G + g) * N + n0);
#pragma unroll
            for (int jj = 0; jj < VEC; ++jj) BT[at(n0 + jj, sl)] = f[jj];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KB; kk += KS) {
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int t = tg * 4 * TPW + wave + 4 * i;
                if (t >= ntiles) continue;
                const int pt = t / ntn, nt = t % ntn;
                typename Mma<T>::frag a = load_frag(XT + at(pt * 16 + r, kk + VEC * q));
                typename Mma<T>::frag bb = load_frag(BT + at(nt * 16 + r, kk + VEC * q));
                acc[i] = Mma<T>::mma(a, bb, acc[i]);
            }
        }
    }
    float *Sc = S + ((size_t)(b * nc + c) * H + h) * P * N;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = tg * 4 * TPW + wave + 4 * i;
        if (t >= ntiles) continue;
        const int pt = t / ntn, nt = t % ntn;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Sc[(size_t)(pt * 16 + 4 * q + e) * N + nt * 16 + r] = acc[i][e];
    }
}

// --------------------------------------------------------------------- k4
// grid (ceil(P*N/1024), H, b), 256 threads, 4 consecutive state elements per
// thread.  Serial over chunks; S[c] is replaced by the state entering chunk c
// and the state after the last chunk is the final state.  Chunk states are
// read kK4Prefetch chunks ahead so several loads are in flight per thread.
__global__ void __launch_bounds__(256)
k4_state_passing(float *__restrict__ S, const float *__restrict__ acum_hi,
                 const float *init, float *final_state, int H, int PN, int nc,
                 int Q, const int *__restrict__ segst) {
    const int h = blockIdx.y, b = blockIdx.z;
    const int e0 = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e0 >= PN) return;
    const size_t soff = (size_t)(b * H + h) * PN + e0;
    float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init) run = *reinterpret_cast<const float4 *>(init + soff);
    const float *ac = acum_hi + (size_t)(b * H + h) * nc * Q;
    constexpr int PF = kK4Prefetch;
    for (int c0 = 0; c0 < nc; c0 += PF) {
        float4 sv[PF];
        float dec[PF];
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int c = c0 + k;
            if (c < nc) {
                sv[k] = *reinterpret_cast<const float4 *>(S + ((size_t)(b * nc + c) * H + h) * PN + e0);
                // (a chunk with a sequence start passes nothing on)
                dec[k] = segst && segst[((size_t)b * nc + c) * Q + Q - 1] >= 0
                             ? 0.f
                             : fast_exp(ac[(size_t)c * Q + Q - 1]);
            }
        }
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int c = c0 + k;
            if (c < nc) {
                *reinterpret_cast<float4 *>(S + ((size_t)(b * nc + c) * H + h) * PN + e0) = run;
                run.x = dec[k] * run.x + sv[k].x;
                run.y = dec[k] * run.y + sv[k].y;
                run.z = dec[k] * run.z + sv[k].z;
                run.w = dec[k] * run.w + sv[k].w;
            }
        }
    }
    if (final_state) *reinterpret_cast<float4 *>(final_state + soff) = run;
}

// --------------------------------------------------------------------- k5
// grid (nc * nlb, H, b), 256 threads, dynamic LDS; nlb = ceil(Q/64).
// Block (c, lb) produces rows l in [64 lb, 64 lb + 64) of chunk c; wave w
// owns the 16 rows l0 = 64 lb + 16 w and every 16-column p-tile.
//   acc  = C[l] . h_in^T                 (state-to-output, Eq. 23)
//   acc *= exp(acum_l)                   (0 past a sequence start in the chunk)
//   acc += sum_{s<=l} M[l][s] x[s],  M[l][s] = CB[l,s] exp(acum_l - acum_s) dt_s
//                                        (Step 1; s >= segst[l] with packed sequences)
//   y    = acc + D x[l]               (D per head, or per head and column)
//   y   *= silu(z[l])                 (when gated)
// For each 64-token s-block at or before the l-block the workgroup stages x^T
// of the s-block and builds the 64 x 64 tile of M in LDS, in the MFMA operand
// type: each thread forms 16 entries from coalesced reads of the C B^T rows
// and the staged prefix sums and dt, so the product loop is LDS reads and
// MFMAs only.  The mask is a select, so entries above the diagonal are
// exactly 0 (the upper-triangle protection of the Kernel 5 page: no exponent
// of s > l reaches the tile).
template <typename T>
__global__ void __launch_bounds__(256)
k5_chunk_scan(const T *__restrict__ x, const T *__restrict__ Cm,
              const float *__restrict__ cb, const float *__restrict__ S,
              const float *__restrict__ acum_hi, const float *__restrict__ acum_lo,
              const float *__restrict__ dtT, const float *__restrict__ D,
              T *__restrict__ y, int L, int H, int G, int P, int N, int nc, int Q,
              const T *__restrict__ z, int D_hdim, const int *__restrict__ segst) {
    constexpr int VEC = Mma<T>::VEC, KS = Mma<T>::KS;
    constexpr int SB = 64;
    constexpr int PITCH = SB + 16 / (int)sizeof(T);          // rows of the M tile (and of bf16 x^T)
    // fp32 x^T: rows of 64 floats with their 4-float chunks XOR-swizzled by (row + row / 16) mod 16, so the
    // staging stores (4 consecutive tokens of 16 rows 4 apart) and the 16-byte fragment reads (16 consecutive
    // rows) fall on distinct banks at headdim 64; bf16 x^T: padded rows
    constexpr bool SW = sizeof(T) == 4;
    constexpr int XPITCH = SW ? SB : PITCH;
    constexpr int MAXPT = kMaxHeaddim / 16;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T *XT = reinterpret_cast<T *>(smem_raw);                 // [P][XPITCH]: x^T of the s-block
    T *MT = XT + (size_t)P * XPITCH;                          // [64][PITCH]: M of (l-block, s-block)
    auto at = [](int row, int s) -> int {
        if constexpr (SW)
            return row * SB + 4 * (((s >> 2) ^ (row + (row >> 4))) & 15) + (s & 3);
        else
            return row * PITCH + s;
    };
    float *s_hi = reinterpret_cast<float *>(MT + SB * PITCH);  // the s-block's prefix sums, dt
    float *s_lo = s_hi + SB;
    float *s_dt = s_lo + SB;
    float *r_hi = s_dt + SB;                                  // the l-block's prefix sums
    float *r_lo = r_hi + SB;
    int *r_st = reinterpret_cast<int *>(r_lo + SB);           // and sequence starts

    const int nlb = (Q + 63) / 64;
    const int c = blockIdx.x / nlb, lb = blockIdx.x % nlb;
    const int h = blockIdx.y, b = blockIdx.z, g = h / (H / G);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;
    const int l0 = lb * 64 + wave * 16;
    const bool active = l0 < Q;
    const int npt = P / 16;
    const float *ah = acum_hi + ((size_t)(b * H + h) * nc + c) * Q;
    const float *al = acum_lo + ((size_t)(b * H + h) * nc + c) * Q;
    const float *dc = dtT + ((size_t)(b * H + h) * nc + c) * Q;
    const int *sg = segst ? segst + ((size_t)b * nc + c) * Q : nullptr;

    if (tid < SB) {
        const int l = lb * SB + tid;
        r_hi[tid] = l < Q ? ah[l] : 0.f;
        r_lo[tid] = l < Q ? al[l] : 0.f;
        r_st[tid] = sg && l < Q ? sg[l] : -1;
    }
    __syncthreads();

    f32x4 acc[MAXPT];
#pragma unroll
    for (int i = 0; i < MAXPT; ++i) acc[i] = zero4();

    if (active) {
        const float *hin = S + ((size_t)(b * nc + c) * H + h) * P * N;
        const int t = c * Q + l0 + r;
        const T *crow = Cm + (((size_t)b * L + t) * G + g) * N;
        for (int k0 = 0; k0 < N; k0 += KS) {
            const int k = k0 + VEC * q;
            const bool kin = k < N;
            typename Mma<T>::frag a = (t < L && kin) ? load_frag(crow + k) : zero_frag<T>();
#pragma unroll
            for (int pt = 0; pt < MAXPT; ++pt) {
                if (pt >= npt) continue;
                typename Mma<T>::frag bb = zero_frag<T>();
                if (kin) {
                    const float *hp = hin + (size_t)(pt * 16 + r) * N + k;
#pragma unroll
                    for (int jj = 0; jj < VEC; ++jj) bb[jj] = from_f32<T>(hp[jj]);
                }
                acc[pt] = Mma<T>::mma(a, bb, acc[pt]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int li = wave * 16 + 4 * q + i;
            const float e = r_st[li] < 0 ? fast_exp(r_hi[li]) : 0.f;
#pragma unroll
            for (int pt = 0; pt < MAXPT; ++pt) acc[pt][i] *= e;
        }
    }

    const size_t cbase = ((size_t)(b * nc + c) * G + g) * Q;
    const int pv = P / VEC;
    for (int sb = 0; sb <= lb; ++sb) {
        __syncthreads();
        for (int v = tid; v < SB * pv; v += 256) {
            const int sl = v / pv, p0 = (v % pv) * VEC;
            const int s = sb * SB + sl, t = c * Q + s;
            typename Mma<T>::frag f = zero_frag<T>();
            if (s < Q && t < L) f = load_frag(x + (((size_t)b * L + t) * H + h) * P + p0);
#pragma unroll
            for (int jj = 0; jj < VEC; ++jj) XT[at(p0 + jj, sl)] = f[jj];
        }
        if (tid < SB) {
            const int s = sb * SB + tid;
            s_hi[tid] = s < Q ? ah[s] : 0.f;
            s_lo[tid] = s < Q ? al[s] : 0.f;
            s_dt[tid] = s < Q ? dc[s] : 0.f;
        }
        __syncthreads();
        // the tile of M: thread tid forms column j = tid % 64 of rows
        // tid / 64 + 4 k, k = 0..15 (each row read as 64 consecutive floats)
        {
            const int j = tid & (SB - 1), s = sb * SB + j;
            const float shi = s_hi[j], slo = s_lo[j], sdt = s_dt[j];
#pragma unroll 4
            for (int i = tid >> 6; i < SB; i += 4) {
                const int l = lb * SB + i;
                float v = 0.f;
                if (l < Q && s <= l && s >= r_st[i])
                    v = cb[(cbase + l) * Q + s] *
                        fast_exp(prefix_diff(r_hi[i], r_lo[i], shi, slo)) * sdt;
                MT[i * PITCH + j] = from_f32<T>(v);
            }
        }
        __syncthreads();
        if (!active) continue;
        // the diagonal tile stops at the wave's last row (M is 0 beyond it)
        const int kend = sb < lb ? SB : min(SB, (wave * 16 + 16 + KS - 1) / KS * KS);
        for (int kk = 0; kk < kend; kk += KS) {
            const typename Mma<T>::frag m = load_frag(MT + (wave * 16 + r) * PITCH + kk + VEC * q);
#pragma unroll
            for (int pt = 0; pt < MAXPT; ++pt) {
                if (pt >= npt) continue;
                typename Mma<T>::frag bb = load_frag(XT + at(pt * 16 + r, kk + VEC * q));
                acc[pt] = Mma<T>::mma(m, bb, acc[pt]);
            }
        }
    }

    if (!active) return;
    const float Dh = D ? D[h] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int l = l0 + 4 * q + i, t = c * Q + l;
        if (l >= Q || t >= L) continue;
        const size_t ro = (((size_t)b * L + t) * H + h) * P;
#pragma unroll
        for (int pt = 0; pt < MAXPT; ++pt) {
            if (pt >= npt) continue;
            const int p = pt * 16 + r;
            const float xv = to_f32(XT[at(p, l - lb * SB)]);
            const float dp = D_hdim && D ? D[(size_t)h * P + p] : Dh;
            float o = acc[pt][i] + dp * xv;
            if (z) o *= silu_f32(to_f32(z[ro + p]));
            y[ro + p] = from_f32<T>(o);
        }
    }
}

// --------------------------------------------------------------------- launch

const char *const kSplitKernelNames[kSplitKernels] = {
    "k1_dA_cumsum", "k2_chunk_cb", "k3_chunk_state", "k4_state_passing", "k5_chunk_scan"};

void launch_dA_cumsum(const float *dt, const DtProc &dtp, const float *A, float *acum_hi,
                      float *acum_lo, float *dtT, int batch, int L, int H, int nc, int Q,
                      hipStream_t stream, const int *seq_idx, int *segst) {
    hipLaunchKernelGGL(k1_dA_cumsum, dim3(nc, (H + 15) / 16, batch), dim3(256), 0, stream, dt,
                       dtp, A, acum_hi, acum_lo, dtT, L, H, nc, Q, seq_idx, segst);
}

template <typename T>
hipError_t launch_split_forward(const ForwardArgs &a, hipStream_t stream, hipEvent_t *events) {
    const int nc = a.nchunks, Q = a.Q;
    int ev = 0;
    auto mark = [&]() -> hipError_t {
        return events ? hipEventRecord(events[ev++], stream) : hipSuccess;
    };
    hipError_t err;
    if ((err = mark()) != hipSuccess) return err;
    const int *segst = a.seq_idx ? a.segst : nullptr;
    launch_dA_cumsum(a.dt, a.dtp, a.A, a.acum_hi, a.acum_lo, a.dtT, a.batch, a.L, a.H, nc, Q,
                     stream, a.seq_idx, a.segst);
    if ((err = mark()) != hipSuccess) return err;
    const int nlb = (Q + 63) / 64;
    hipLaunchKernelGGL(k2_chunk_cb<T>, dim3(nlb * (nlb + 1) / 2, nc * a.G, a.batch),
                       dim3(256), 0, stream, (const T *)a.B, (const T *)a.C, (float *)a.cb, a.L,
                       a.G, a.N, nc, Q);
    if ((err = mark()) != hipSuccess) return err;
    const int ntiles = (a.P / 16) * (a.N / 16);
    const int ntg = (ntiles + 4 * kK3TilesPerWave - 1) / (4 * kK3TilesPerWave);
    const size_t k3_lds = (size_t)(a.P + a.N) * (32 + 16 / sizeof(T)) * sizeof(T);
    hipLaunchKernelGGL(k3_chunk_state<T>, dim3(nc, a.H * ntg, a.batch), dim3(256), k3_lds,
                       stream, (const T *)a.x, (const T *)a.B, a.acum_hi, a.acum_lo, a.dtT,
                       a.S, a.L, a.H, a.G, a.P, a.N, nc, Q, segst);
    if ((err = mark()) != hipSuccess) return err;
    const int PN = a.P * a.N;
    hipLaunchKernelGGL(k4_state_passing, dim3((PN + 1023) / 1024, a.H, a.batch), dim3(256),
                       0, stream, a.S, a.acum_hi, a.init, a.final_state, a.H, PN, nc, Q, segst);
    if ((err = mark()) != hipSuccess) return err;
    const size_t k5_lds = (size_t)(a.P + 64) * (64 + 16 / sizeof(T)) * sizeof(T) + 6 * 64 * 4;
    hipLaunchKernelGGL(k5_chunk_scan<T>, dim3(nc * nlb, a.H, a.batch), dim3(256), k5_lds,
                       stream, (const T *)a.x, (const T *)a.C, (const float *)a.cb, a.S, a.acum_hi,
                       a.acum_lo, a.dtT, a.D, (T *)a.y, a.L, a.H, a.G, a.P, a.N, nc, Q,
                       (const T *)a.z, a.D_hdim ? 1 : 0, segst);
    if ((err = mark()) != hipSuccess) return err;
    return hipGetLastError();
}

template hipError_t launch_split_forward<float>(const ForwardArgs &, hipStream_t, hipEvent_t *);
template hipError_t launch_split_forward<bf16>(const ForwardArgs &, hipStream_t, hipEvent_t *);

}  // namespace ssd
