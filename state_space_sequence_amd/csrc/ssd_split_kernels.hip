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
#include "ssd_backward.hpp"

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
    // this thread's tokens r0 + 16 k (Q <= 256: at most 16), all loads
    // issued before the first is used
    const int j = tid & 15, r0 = tid >> 4, h = h0 + j;
    float dv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int r = r0 + 16 * k, t = c * Q + r;
        dv[k] = r < Q && h < H && t < L ? dt[((size_t)b * L + t) * H + h] : 0.f;
    }
    const float bias = dtp.on && dtp.bias && h < H ? dtp.bias[h] : 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int r = r0 + 16 * k, t = c * Q + r;
        if (r < Q)
            s_dt[j][r] = dtp.on && h < H && t < L ? dt_process(dv[k], bias, dtp.softplus, dtp.lo, dtp.hi)
                                                  : dv[k];
    }
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63;
    const int E = Q > 64 ? Q / 64 : 1;
    for (int jj = 0; jj < 4; ++jj) {
        const int hl = wave * 4 + jj, hh = h0 + hl;
        if (hh >= H) break;
        const double Ah = (double)A[hh];
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
        const size_t base = ((size_t)(b * H + hh) * nc + c) * Q;
        if (E == 4) {
            // (Q = 256: the lane's 4 tokens as one 16-byte store per array)
            f32x4 vh, vl, vd;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double v = excl + a[e];
                vh[e] = (float)v;
                vl[e] = (float)(v - (double)vh[e]);
                vd[e] = d[e];
            }
            *reinterpret_cast<f32x4 *>(acum_hi + base + 4 * lane) = vh;
            *reinterpret_cast<f32x4 *>(acum_lo + base + 4 * lane) = vl;
            *reinterpret_cast<f32x4 *>(dtT + base + 4 * lane) = vd;
            continue;
        }
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
// the MFMA k dimension here; a K step's loads are issued a step ahead.
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
    // the next K step's operands are loaded while this one's MFMAs run
    typedef typename Mma<T>::frag frag;
    auto load = [&](int k0, frag &a, frag (&bb)[4]) {
        const int k = k0 + VEC * q;
        const bool kin = k < N;
        a = (tl < L && kin) ? load_frag(crow + k) : zero_frag<T>();
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int ts = c * Q + s0[st] + r;
            bb[st] = (act[st] && ts < L && kin) ? load_frag(Bm + (((size_t)b * L + ts) * G + g) * N + k)
                                                : zero_frag<T>();
        }
    };
    frag a, bb[4];
    load(0, a, bb);
    for (int k0 = 0; k0 < N; k0 += KS) {
        const bool more = k0 + KS < N;
        frag an, bn[4];
        if (more) load(k0 + KS, an, bn);
#pragma unroll
        for (int st = 0; st < 4; ++st)
            if (act[st]) acc[st] = Mma<T>::mma(a, bb[st], acc[st]);
        if (more) {
            a = an;
#pragma unroll
            for (int st = 0; st < 4; ++st) bb[st] = bn[st];
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
// ADJ: the same product for the gradient pass, G[p][n] = sum_s dy[s][p] *
// exp(acum_s) * C[s][n] (x -> dy, B -> C, w_s = exp(acum_s)), the part of
// the gradient with respect to the state entering the chunk that the
// chunk's own outputs contribute.
template <typename T, bool ADJ = false>
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
            const bool in = s < Q && t < L && (ADJ || s >= s_first);
            float w = 0.f;
            typename Mma<T>::frag f = zero_frag<T>();
            if (in) {
                w = ADJ ? fast_exp(ah[s]) : fast_exp(prefix_diff(end_hi, end_lo, ah[s], al[s])) * dc[s];
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
// word 3 of a raw buffer resource on gfx9-family targets (32-bit data format)
constexpr int kRawBufferWord3 = 0x00020000;

// LDS of k5, shared by the kernel and its launch, for headdims padded to 64
// or 128 (the padded columns feed only accumulators that are never stored).
// fp32: the source block's x as token rows of a pitch = 16 (mod 64) floats,
// so a fragment read (4 consecutive tokens x 16 consecutive columns) falls
// on 64 distinct banks and staging is a plain 16-byte copy; bf16: x^T, rows
// of 64 + 8.  Then the tile of M (64 rows), two K-slabs of the entering
// state, and float vectors: the chunk's prefix sums, decays and starts by
// row (4 x 256) and the source block's prefix sums, dt and decays (4 x 64).
struct K5Lds {
    static constexpr int kSB = 64;   // the largest row / source block
    static __host__ __device__ constexpr int ppad(int P) { return P <= 64 ? 64 : 128; }
    static __host__ __device__ constexpr int xpitch(int PP, int sz) {
        return sz == 4 ? PP + (80 - PP % 64) % 64 : kSB + 16 / sz;
    }
    static __host__ __device__ constexpr int mpitch(int sz) { return kSB + 16 / sz; }
    static __host__ __device__ constexpr int hpitch(int sz) { return (sz == 4 ? 16 : 32) + 16 / sz; }
    static __host__ __device__ constexpr size_t x_elems(int PP, int sz) {
        return (size_t)(sz == 4 ? kSB : PP) * xpitch(PP, sz);
    }
    static __host__ __device__ constexpr size_t h_elems(int PP, int sz) {
        return (size_t)2 * PP * hpitch(sz);
    }
    static size_t bytes(int P, int sz) {
        const int PP = ppad(P);
        return (x_elems(PP, sz) + (size_t)kSB * mpitch(sz) + h_elems(PP, sz)) * sz +
               (4 * 256 + 4 * kSB) * 4;
    }
};

// acc[i][k] += a[i] b[k] over the fragments' K; the MFMAs run in an order in
// which consecutive ones write different accumulators
template <typename T, int NA, int NB>
__device__ __forceinline__ void mma_grid(const typename Mma<T>::frag (&a)[NA],
                                         const typename Mma<T>::frag (&b)[NB],
                                         f32x4 (&acc)[NA][NB]) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int k = 0; k < NB; ++k)
                    acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][j], b[k][j], acc[i][k], 0, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int k = 0; k < NB; ++k) acc[i][k] = Mma<T>::mma(a[i], b[k], acc[i][k]);
    }
}

// grid (nc * NRB / NOWN, H, b), 256 threads (4 waves), dynamic LDS
// K5Lds::bytes.  Chunk c of head h has NRB row blocks of SB = min(Q, 64)
// rows; workgroup `half` of the chunk owns NOWN of them: {half} alone, or
// {half, NRB - 1 - half} (one long and one short row block, so that the two
// workgroups of a chunk have equal numbers of tiles).  Wave w computes the
// 16-row tile w of each owned row block; NPT 16-column tiles span the
// (padded) headdim.
//   acc  = C[l] . h_in^T                 (state-to-output, Eq. 23)
//   acc *= exp(acum_l)                   (0 past a sequence start in the chunk)
//   acc += sum_{s<=l} M[l][s] x[s],  M[l][s] = CB[l,s] exp(acum_l - acum_s) dt_s
//                                        (Step 1; s >= segst[l] with packed sequences)
//   y    = acc + D x[l]               (D per head, or per head and column)
//   y   *= silu(z[l])                 (when gated)
// The state entering the chunk passes through LDS once, in K-slabs, and x
// once per SB-token source block.  For each (row block, source block) pair at
// or below the diagonal the workgroup builds the tile of M in LDS, in the
// MFMA operand type, each thread forming up to 16 entries of one column from
// coalesced reads of C B^T rows.  On the diagonal tile every entry takes its
// own exponential of a prefix-sum difference, and the mask is a select, so
// entries above the diagonal are exactly 0 (the upper-triangle protection of
// the Kernel 5 page: no exponent of s > l reaches the tile).  Below it the
// decay factors through the block's last source s0: exp(acum_l - acum_s) =
// exp(acum_l - acum_s0) exp(acum_s0 - acum_s), both exponents <= 0 (A <= 0),
// one exponential per row and per source instead of one per entry.  Loads
// run one step ahead of the MFMAs: the next state slab during a slab's
// products, the next tile's C B^T entries (and the next block's x) during a
// tile's.  A row block's outputs are finished right after its diagonal tile,
// while that block's x is staged.
// (three workgroups of 64-column tiles fit a compute unit's LDS; the register
// cap that lets them all run costs a couple of spilled registers)
template <typename T, int NPT, int NRB, int NOWN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NPT == 4 ? 3 : 1)))
k5_chunk_scan(const T *__restrict__ x, const T *__restrict__ Cm,
              const float *__restrict__ cb, const float *__restrict__ S,
              const float *__restrict__ acum_hi, const float *__restrict__ acum_lo,
              const float *__restrict__ dtT, const float *__restrict__ D,
              T *__restrict__ y, int L, int H, int G, int P, int N, int nc, int Q,
              const T *__restrict__ z, int D_hdim, const int *__restrict__ segst) {
    typedef typename Mma<T>::frag frag;
    constexpr int VEC = Mma<T>::VEC, KS = Mma<T>::KS;
    constexpr int SZ = (int)sizeof(T);
    constexpr int SBX = K5Lds::kSB;
    constexpr bool F32 = SZ == 4;
    constexpr int PP = 16 * NPT;                              // the padded headdim
    constexpr int XP = K5Lds::xpitch(PP, SZ);
    constexpr int PITCH = K5Lds::mpitch(SZ);
    constexpr int HPITCH = K5Lds::hpitch(SZ);
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T *XS = reinterpret_cast<T *>(smem_raw);                 // x of the source block (see K5Lds)
    T *MT = XS + K5Lds::x_elems(PP, SZ);                     // [SBX][PITCH]: M of (row block, source block)
    T *HS = MT + (size_t)SBX * PITCH;                         // [2][PP][HPITCH]: K-slabs of the entering state
    float *r_hi = reinterpret_cast<float *>(HS + K5Lds::h_elems(PP, SZ));  // by row of the chunk:
    float *r_lo = r_hi + 256;                                 //   prefix sums (hi + lo),
    float *r_u = r_lo + 256;                                  //   exp(acum_l - acum_s0),
    int *r_st = reinterpret_cast<int *>(r_u + 256);           //   sequence starts
    float *s_hi = reinterpret_cast<float *>(r_st + 256);      // by source of the block: prefix sums,
    float *s_lo = s_hi + SBX;
    float *s_dt = s_lo + SBX;                                 //   dt,
    float *s_v = s_dt + SBX;                                  //   exp(acum_s0 - acum_s) dt_s
    // position of tile column s in an M row: fp32 fragments take the K index
    // s = kk + q + 4 j (lane group q, MFMA j of four), stored at kk + 4 q + j
    // so that a lane's four A values are one 16-byte read; bf16 keeps order
    auto mcol = [](int s) -> int {
        if constexpr (F32)
            return (s & ~15) | ((s & 3) << 2) | ((s >> 2) & 3);
        else
            return s;
    };
    // x of source token s (in the block), column p
    auto xat = [](int s, int p) -> int {
        if constexpr (F32)
            return s * XP + p;
        else
            return p * PITCH + s;
    };

    constexpr int NSPLIT = NRB / NOWN;                        // workgroups per chunk
    const int c = blockIdx.x / NSPLIT, half = blockIdx.x % NSPLIT;
    const int h = blockIdx.y, b = blockIdx.z, g = h / (H / G);
    // (the wave index as a wave-uniform value: row tests become scalar)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    // the owned row blocks, in increasing order
    auto own = [&](int j) -> int { return j == 0 ? half : NRB - 1 - half; };
    const int own_last = own(NOWN - 1);
    const int r = lane & 15, q = lane >> 4;
    const int SB = NRB > 1 || Q >= SBX ? SBX : Q;   // Q / NRB
    const int SBK = SB < KS ? KS : SB;        // columns of a tile the product reads (zeros past SB)
    const bool active = wave * 16 < SB;       // this wave owns tile `wave` of every row block
    const float *ah = acum_hi + ((size_t)(b * H + h) * nc + c) * Q;
    const float *al = acum_lo + ((size_t)(b * H + h) * nc + c) * Q;
    const float *dc = dtT + ((size_t)(b * H + h) * nc + c) * Q;
    const int *sg = segst ? segst + ((size_t)b * nc + c) * Q : nullptr;

    for (int l = tid; l < Q; l += 256) {
        r_hi[l] = ah[l];
        r_lo[l] = al[l];
        r_st[l] = sg ? sg[l] : -1;
    }

    f32x4 acc[NOWN][NPT];
#pragma unroll
    for (int j = 0; j < NOWN; ++j)
#pragma unroll
        for (int i = 0; i < NPT; ++i) acc[j][i] = zero4();

    // ---- state to output: C of every row of the wave, times the state
    // entering the chunk, staged a K-slab (KS dstate columns) at a time into
    // two alternating LDS buffers; the next slab's state and C fragments are
    // loaded while this slab's MFMAs run
    const float *hin = S + ((size_t)(b * nc + c) * H + h) * P * N;
    const T *crow = Cm + (((size_t)b * L + (size_t)c * Q) * G + g) * N;
    constexpr int KQ = KS / VEC;                   // fragments per slab row
    constexpr int HF = (PP * KQ + 255) / 256;      // slab fragments per thread
    const int hv = P * KQ;                         // fragments of a slab (rows past P stay unset)
    frag hf[HF], cf[NOWN], cn[NOWN];
    auto load_slab = [&](int k0) {
#pragma unroll
        for (int u = 0; u < HF; ++u) {
            const int v = tid + 256 * u;
            if (v >= hv) continue;
            const int p = v / KQ, kq = (v % KQ) * VEC;
#pragma unroll
            for (int jj = 0; jj < VEC; ++jj)
                hf[u][jj] = k0 + kq + jj < N ? from_f32<T>(hin[(size_t)p * N + k0 + kq + jj]) : from_f32<T>(0.f);
        }
#pragma unroll
        for (int j = 0; j < NOWN; ++j) {
            cn[j] = zero_frag<T>();
            const int l = own(j) * SB + wave * 16 + r;
            const int k = k0 + VEC * q;
            if (active && (size_t)c * Q + l < (size_t)L && k < N)
                cn[j] = load_frag(crow + (size_t)l * G * N + k);
        }
    };
    load_slab(0);
    for (int k0 = 0, buf = 0; k0 < N; k0 += KS, buf ^= 1) {
        T *hs = HS + (size_t)buf * PP * HPITCH;
#pragma unroll
        for (int u = 0; u < HF; ++u) {
            const int v = tid + 256 * u;
            if (v < hv) *reinterpret_cast<frag *>(hs + (v / KQ) * HPITCH + (v % KQ) * VEC) = hf[u];
        }
#pragma unroll
        for (int j = 0; j < NOWN; ++j) cf[j] = cn[j];
        __syncthreads();
        if (k0 + KS < N) load_slab(k0 + KS);
        if (active) {
            frag bb[NPT];
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) bb[pt] = load_frag(hs + (pt * 16 + r) * HPITCH + VEC * q);
            mma_grid<T>(cf, bb, acc);
        }
    }
    if (active) {
#pragma unroll
        for (int j = 0; j < NOWN; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int l = own(j) * SB + wave * 16 + 4 * q + i;
                const float e = r_st[l] < 0 ? fast_exp(r_hi[l]) : 0.f;
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) acc[j][pt][i] *= e;
            }
        }
    }

    // ---- the intra-chunk product over the pairs (row block lb, source block
    // sb): for sb = 0, 1, ..., the owned lb >= sb in increasing order, so
    // that the diagonal pair (lb = sb) opens its source block.  Per pair: the
    // MFMAs of this pair's tile, meanwhile the loads of the next pair's C B^T
    // entries (and, when the next pair starts a source block, its x); then,
    // after a barrier, the next tile of M built from those registers.
    const size_t cbase = ((size_t)(b * nc + c) * G + g) * Q;
    const int pv = P / VEC;
    const float Dh = D ? D[h] : 0.f;
    const int jc = tid & (SBX - 1);          // the tile column this thread builds
    constexpr int XF = (SBX * PP / VEC + 255) / 256;
    frag xr[XF];                             // x of a source block, in flight
    float cbr[SBX / 4];                      // C B^T entries of the next tile, in flight
    auto load_x = [&](int sb) {
#pragma unroll
        for (int u = 0; u < XF; ++u) {
            const int v = tid + 256 * u;
            xr[u] = zero_frag<T>();
            if (v >= SBK * pv) continue;
            const int sl = v / pv, p0 = (v % pv) * VEC, t = c * Q + sb * SB + sl;
            if (sl < SB && t < L) xr[u] = load_frag(x + (((size_t)b * L + t) * H + h) * P + p0);
        }
    };
    // stage block sb: its x, the prefix sums, dt and decays of its sources,
    // and the decays of the later rows to its last source s0
    auto stage = [&](int sb) {
#pragma unroll
        for (int u = 0; u < XF; ++u) {
            const int v = tid + 256 * u;
            if (v >= SBK * pv) continue;
            const int sl = v / pv, p0 = (v % pv) * VEC;
            if constexpr (F32) {
                *reinterpret_cast<frag *>(XS + xat(sl, p0)) = xr[u];
            } else {
#pragma unroll
                for (int jj = 0; jj < VEC; ++jj) XS[xat(sl, p0 + jj)] = xr[u][jj];
            }
        }
        const int s0 = sb * SB + SB - 1;
        if (tid < SB) {
            const int s = sb * SB + tid;
            const float hi = r_hi[s], lo = r_lo[s], d = dc[s];
            s_hi[tid] = hi;
            s_lo[tid] = lo;
            s_dt[tid] = d;
            s_v[tid] = fast_exp(prefix_diff(r_hi[s0], r_lo[s0], hi, lo)) * d;
        }
        for (int l = s0 + 1 + tid; l < Q; l += 256)
            r_u[l] = fast_exp(prefix_diff(r_hi[l], r_lo[l], r_hi[s0], r_lo[s0]));
    };
    // the entries of tile (lb, sb) in this thread's column: rows tid / 64 + 4 k
    // (buffer loads: one address per thread, the row step in the scalar offset)
    const __amdgpu_buffer_rsrc_t rcb =
        __builtin_amdgcn_make_buffer_rsrc((void *)(cb + cbase * Q), 0, (unsigned)Q * Q * 4, kRawBufferWord3);
    auto load_cb = [&](int lb, int sb) {
        const int voff = ((lb * SB + wave) * Q + sb * SB + jc) * 4;
#pragma unroll
        for (int k = 0; k < SBX / 4; ++k) {
            const int i = wave + 4 * k;
            cbr[k] = 0.f;
            if (i < SB && jc < SB)
                cbr[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rcb, voff, 16 * k * Q, 0));
        }
    };
    // the tile of M from cbr.  On the diagonal each entry takes its own
    // exponential and the causal mask; below it, the factored decays
    auto build = [&](int lb, int sb) {
        if (jc >= SBK) return;
        T *mc = MT + mcol(jc);
        const int s = sb * SB + jc;
        if (lb > sb) {
            const float sv = s_v[jc];
#pragma unroll
            for (int k = 0; k < SBX / 4; ++k) {
                const int i = wave + 4 * k, l = lb * SB + i;
                if (i >= SB) continue;
                const float v = jc < SB && s >= r_st[l] ? cbr[k] * r_u[l] * sv : 0.f;
                mc[i * PITCH] = from_f32<T>(v);
            }
        } else {
            const float shi = s_hi[jc], slo = s_lo[jc], sdt = s_dt[jc];
#pragma unroll
            for (int k = 0; k < SBX / 4; ++k) {
                const int i = wave + 4 * k, l = lb * SB + i;
                if (i >= SB) continue;
                float v = 0.f;
                if (jc < SB && s <= l && s >= r_st[l])
                    v = cbr[k] * fast_exp(prefix_diff(r_hi[l], r_lo[l], shi, slo)) * sdt;
                mc[i * PITCH] = from_f32<T>(v);
            }
        }
    };
    // row block sb is complete (its last source block is its diagonal, whose
    // x is staged): the skip term, the gate, y
    auto finish = [&](const f32x4(&ac)[NPT], int sb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int l = sb * SB + wave * 16 + 4 * q + i, t = c * Q + l;
            if (t >= L) continue;
            const size_t ro = (((size_t)b * L + t) * H + h) * P;
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
                const int p = pt * 16 + r;
                if (p >= P) continue;
                const float xv = to_f32(XS[xat(l - sb * SB, p)]);
                const float dp = D_hdim && D ? D[(size_t)h * P + p] : Dh;
                float o = ac[pt][i] + dp * xv;
                if (z) o *= silu_f32(to_f32(z[ro + p]));
                y[ro + p] = from_f32<T>(o);
            }
        }
    };

    // the pair after (sb, j), if any
    auto next_pair = [&](int sb, int j, int &nsb, int &nj) -> bool {
        nsb = sb;
        nj = j + 1;
        for (;;) {
            if (nj >= NOWN) {
                ++nsb;
                nj = 0;
            }
            if (nsb > own_last) return false;
            if (own(nj) >= nsb) return true;
            ++nj;
        }
    };

    load_x(0);
    load_cb(own(0), 0);
    stage(0);
    __syncthreads();
    build(own(0), 0);
    __syncthreads();
    f32x4 tmp[1][NPT];
    int sb = 0, j = 0;
#pragma nounroll
    for (;;) {
        const int lb = own(j);
        int nsb, nj;
        const bool more = next_pair(sb, j, nsb, nj), next_block = more && nsb != sb;
        if (more) {
            load_cb(own(nj), nsb);
            if (next_block) load_x(nsb);
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) tmp[0][pt] = zero4();
        if (active) {
            // this wave's rows of the tile times x; the diagonal tile stops
            // at the wave's last row (M is 0 beyond it)
            const int kend = sb < lb ? SB : min(SB, (wave * 16 + 16 + KS - 1) / KS * KS);
#pragma unroll
            for (int kk = 0; kk < SBX; kk += KS) {
                if (kk >= kend) break;
                const frag m[1] = {load_frag(MT + (wave * 16 + r) * PITCH + kk + VEC * q)};
                frag bb[NPT];
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) {
                    if constexpr (F32) {
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) bb[pt][jj] = XS[xat(kk + q + 4 * jj, pt * 16 + r)];
                    } else {
                        bb[pt] = load_frag(XS + xat(kk + VEC * q, pt * 16 + r));
                    }
                }
                mma_grid<T>(m, bb, tmp);
            }
        }
        // (one copy of the product above; the sum goes to the row block's
        // accumulators through constant indexes, which keeps them in registers)
        auto add = [&](f32x4(&ac)[NPT]) {
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) ac[pt] += tmp[0][pt];
        };
        if (!more) {
            // the last pair is the diagonal of the last owned row block
            add(acc[NOWN - 1]);
            if (active) finish(acc[NOWN - 1], sb);
            break;
        }
        __syncthreads();   // (the tile of M, and x when replaced, no longer read)
        if (next_block) {
            // a diagonal pair is followed by a pair of its own source block
            // (its row block's rows are finished below, from the staged x)
            // unless it is the last pair, so the pair just done is below
            // the diagonal
            stage(nsb);
            __syncthreads();
        }
        build(own(nj), nsb);
        if (j == 0) add(acc[0]); else add(acc[NOWN - 1]);
        if (lb == sb && active) finish(j == 0 ? acc[0] : acc[NOWN - 1], sb);
        __syncthreads();   // (the next tile of M is built)
        sb = nsb;
        j = nj;
    }
}

// --------------------------------------------------------------------- k3, fp32
// fp32 k3: grid (nc, H * npg * nng, b), 256 threads, dynamic LDS
// K3F32Lds::bytes.  Workgroup (pg, ng) computes the 64 x 128 block
// S[64 pg .., 128 ng ..] of the chunk state (headdim and dstate padded to
// those multiples; padded rows and columns feed only tiles never stored);
// waves form a 2 x 2 grid of 32 x 64 sub-blocks, 2 x 4 tiles of 16 x 16 each.
// The per-token weight w_s (0 before the chunk's last sequence start and
// past the end) is computed once per token; a chunk shorter than a slab
// (16 tokens) leaves the rest of the slab zero.  32-token slabs of x and B go
// to LDS untransposed, w folded into x, as rows of a pitch = 16 (mod 64)
// floats: the fragments take K index s = kk + q + 4 j (lane group q, MFMA j
// of four), so a lane's operands are single floats of 4 consecutive rows x
// 16 consecutive columns, 64 distinct banks.  The next slab is loaded into
// registers while this slab's MFMAs run.
struct K3F32Lds {
    static constexpr int kKB = 32;   // tokens per slab
    static __host__ __device__ constexpr int pitch(int cols) { return cols + (80 - cols % 64) % 64; }
    static size_t bytes() { return ((size_t)kKB * pitch(64) + (size_t)kKB * pitch(128) + 256) * 4; }
};

// (ADJ: the gradient pass's product, as for the bf16 kernel above.)
template <bool ADJ = false>
__global__ void __launch_bounds__(256)
k3_chunk_state_f32(const float *__restrict__ x, const float *__restrict__ Bm,
                   const float *__restrict__ acum_hi, const float *__restrict__ acum_lo,
                   const float *__restrict__ dtT, float *__restrict__ S, int L, int H,
                   int G, int P, int N, int nc, int Q, const int *__restrict__ segst) {
    constexpr int KB = K3F32Lds::kKB;
    constexpr int XP = K3F32Lds::pitch(64), BP = K3F32Lds::pitch(128);
    extern __shared__ __align__(16) unsigned char smem_raw[];
    float *XS = reinterpret_cast<float *>(smem_raw);   // [KB][XP]: w_s x[s][64 pg + p]
    float *BS = XS + KB * XP;                           // [KB][BP]: B[s][128 ng + n]
    float *s_w = BS + KB * BP;                          // [256]: w_s (0 past the chunk)

    const int npg = (P + 63) / 64, nng = (N + 127) / 128;
    const int c = blockIdx.x, b = blockIdx.z;
    const int h = blockIdx.y / (npg * nng), pg = blockIdx.y / nng % npg, ng = blockIdx.y % nng;
    const int g = h / (H / G);
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;
    const int wp = (wave >> 1) * 32, wn = (wave & 1) * 64;   // this wave's sub-block
    const float *ah = acum_hi + ((size_t)(b * H + h) * nc + c) * Q;
    const float *al = acum_lo + ((size_t)(b * H + h) * nc + c) * Q;
    const float *dc = dtT + ((size_t)(b * H + h) * nc + c) * Q;
    {
        const float end_hi = ah[Q - 1], end_lo = al[Q - 1];
        // packed sequences: only the chunk's last sequence reaches its end state
        const int s_first = segst ? segst[((size_t)b * nc + c) * Q + Q - 1] : -1;
        for (int s = tid; s < 256; s += 256) {
            const bool in = s < Q && c * Q + s < L && (ADJ || s >= s_first);
            s_w[s] = !in ? 0.f
                   : ADJ ? fast_exp(ah[s])
                         : fast_exp(prefix_diff(end_hi, end_lo, ah[s], al[s])) * dc[s];
        }
    }

    // slab loads: x rows of 64 columns (16 float4 per token), B rows of 128
    // (32 float4 per token); 2 + 4 per thread
    constexpr int XV = KB * 16 / 256, BV = KB * 32 / 256;
    f32x4 xr[XV], br[BV];
    const int p_lo = 64 * pg, n_lo = 128 * ng;
    auto load = [&](int s0) {
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int v = tid + 256 * u, sl = v >> 4, p = p_lo + 4 * (v & 15), t = c * Q + s0 + sl;
            xr[u] = zero4();
            if (s0 + sl < Q && t < L && p < P) xr[u] = *reinterpret_cast<const f32x4 *>(x + (((size_t)b * L + t) * H + h) * P + p);
        }
#pragma unroll
        for (int u = 0; u < BV; ++u) {
            const int v = tid + 256 * u, sl = v >> 5, n = n_lo + 4 * (v & 31), t = c * Q + s0 + sl;
            br[u] = zero4();
            if (s0 + sl < Q && t < L && n < N) br[u] = *reinterpret_cast<const f32x4 *>(Bm + (((size_t)b * L + t) * G + g) * N + n);
        }
    };

    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] = zero4();

    load(0);
    for (int s0 = 0; s0 < Q; s0 += KB) {
        __syncthreads();   // (the previous slab is no longer read; s_w visible)
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int v = tid + 256 * u, sl = v >> 4;
            const float w = s_w[s0 + sl];
            *reinterpret_cast<f32x4 *>(XS + sl * XP + 4 * (v & 15)) = xr[u] * w;
        }
#pragma unroll
        for (int u = 0; u < BV; ++u) {
            const int v = tid + 256 * u;
            *reinterpret_cast<f32x4 *>(BS + (v >> 5) * BP + 4 * (v & 31)) = br[u];
        }
        __syncthreads();
        if (s0 + KB < Q) load(s0 + KB);
#pragma unroll
        for (int kk = 0; kk < KB; kk += 16) {
            f32x4 a[2], bb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = kk + q + 4 * j;
#pragma unroll
                for (int i = 0; i < 2; ++i) a[i][j] = XS[row * XP + wp + 16 * i + r];
#pragma unroll
                for (int k = 0; k < 4; ++k) bb[k][j] = BS[row * BP + wn + 16 * k + r];
            }
            mma_grid<float>(a, bb, acc);
        }
    }
    float *Sc = S + ((size_t)(b * nc + c) * H + h) * P * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int n = n_lo + wn + 16 * k + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int p = p_lo + wp + 16 * i + 4 * q + e;
                if (p < P && n < N) Sc[(size_t)p * N + n] = acc[i][k][e];
            }
        }
}

// --------------------------------------------------------------------- k3, bf16
// The bf16 chunk state, built as the fp32 one (K3F32Lds): a workgroup
// computes a 64 x 128 block of the state, its waves 2 x 2 sub-blocks of 2 x 4
// tiles; the per-token weight once per token; 32-token slabs of (weighted)
// x and of B staged untransposed in LDS, rows padded by 8 elements; the next
// slab loaded into registers while this slab's MFMAs run.  The MFMA takes K
// (tokens) 8 to a lane, so the fragments come from the transposing LDS read
// (ds_read_b64_tr_b16): within each 16-lane group lane a + 4 e reads 4
// columns 4a .. 4a + 3 of token row kbase + e, and lane 4 a + c receives
// column 4 a + c of the four rows; two reads (rows kbase .. kbase + 7) make a
// fragment.  With the padding, the 16 rows one read touches spread over the
// banks (at most two lanes per bank).
struct K3Bf16Lds {
    static constexpr int kKB = 32;
    static constexpr int kXP = 64 + 8, kBP = 128 + 8;   // row pitches (elements)
    static size_t bytes() { return ((size_t)kKB * (kXP + kBP)) * 2 + 256 * 4; }
};

typedef __bf16 k3_bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) k3_bf16x4 k3_lds_bf16x4;
typedef __attribute__((address_space(3))) unsigned char k3_lds_u8;

__device__ __forceinline__ bf16x8 k3_tr_frag(const bf16 *base, int off0, int off1) {
    const k3_bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (k3_lds_bf16x4 *)((k3_lds_u8 *)base + off0));
    const k3_bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (k3_lds_bf16x4 *)((k3_lds_u8 *)base + off1));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <bool ADJ = false>
__global__ void __launch_bounds__(256)
k3_chunk_state_bf16(const bf16 *__restrict__ x, const bf16 *__restrict__ Bm,
                    const float *__restrict__ acum_hi, const float *__restrict__ acum_lo,
                    const float *__restrict__ dtT, float *__restrict__ S, int L, int H,
                    int G, int P, int N, int nc, int Q, const int *__restrict__ segst) {
    constexpr int KB = K3Bf16Lds::kKB, XP = K3Bf16Lds::kXP, BP = K3Bf16Lds::kBP;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    bf16 *XS = reinterpret_cast<bf16 *>(smem_raw);     // [KB][XP]: w_s x[s][64 pg + p]
    bf16 *BS = XS + KB * XP;                            // [KB][BP]: B[s][128 ng + n]
    float *s_w = reinterpret_cast<float *>(BS + KB * BP);   // [256]

    const int npg = (P + 63) / 64, nng = (N + 127) / 128;
    const int c = blockIdx.x, b = blockIdx.z;
    const int h = blockIdx.y / (npg * nng), pg = blockIdx.y / nng % npg, ng = blockIdx.y % nng;
    const int g = h / (H / G);
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;
    const int wp = (wave >> 1) * 32, wn = (wave & 1) * 64;
    const float *ah = acum_hi + ((size_t)(b * H + h) * nc + c) * Q;
    const float *al = acum_lo + ((size_t)(b * H + h) * nc + c) * Q;
    const float *dc = dtT + ((size_t)(b * H + h) * nc + c) * Q;
    {
        const float end_hi = ah[Q - 1], end_lo = al[Q - 1];
        const int s_first = segst ? segst[((size_t)b * nc + c) * Q + Q - 1] : -1;
        const int s = tid;
        const bool in = s < Q && c * Q + s < L && (ADJ || s >= s_first);
        s_w[s] = !in ? 0.f
               : ADJ ? fast_exp(ah[s])
                     : fast_exp(prefix_diff(end_hi, end_lo, ah[s], al[s])) * dc[s];
    }
    // slab loads, 8 bf16 per piece: x rows of 64 (8 pieces per token), B rows
    // of 128 (16 per token); 1 + 2 per thread
    constexpr int XV = KB * 8 / 256, BV = KB * 16 / 256;
    bf16x8 xr[XV], br[BV];
    const int p_lo = 64 * pg, n_lo = 128 * ng;
    auto load = [&](int s0) {
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int v = tid + 256 * u, sl = v >> 3, p = p_lo + 8 * (v & 7), t = c * Q + s0 + sl;
            xr[u] = zero_frag<bf16>();
            if (s0 + sl < Q && t < L && p < P) xr[u] = load_frag(x + (((size_t)b * L + t) * H + h) * P + p);
        }
#pragma unroll
        for (int u = 0; u < BV; ++u) {
            const int v = tid + 256 * u, sl = v >> 4, n = n_lo + 8 * (v & 15), t = c * Q + s0 + sl;
            br[u] = zero_frag<bf16>();
            if (s0 + sl < Q && t < L && n < N) br[u] = load_frag(Bm + (((size_t)b * L + t) * G + g) * N + n);
        }
    };
    // this lane's read addresses (bytes) within a slab: rows e = r / 4 (+ 4),
    // columns 4 (r % 4) of each 16-column tile, K rows 8 q ..
    const int er = r >> 2, ca = 4 * (r & 3);
    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] = zero4();

    load(0);
    for (int s0 = 0; s0 < Q; s0 += KB) {
        __syncthreads();   // (the previous slab is no longer read; s_w visible)
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int v = tid + 256 * u, sl = v >> 3;
            const float w = s_w[(s0 + sl) & 255];
            bf16x8 f;
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] = (bf16)((float)xr[u][j] * w);
            *reinterpret_cast<bf16x8 *>(XS + sl * XP + 8 * (v & 7)) = f;
        }
#pragma unroll
        for (int u = 0; u < BV; ++u) {
            const int v = tid + 256 * u;
            *reinterpret_cast<bf16x8 *>(BS + (v >> 4) * BP + 8 * (v & 15)) = br[u];
        }
        __syncthreads();
        if (s0 + KB < Q) load(s0 + KB);
        bf16x8 a[2], bb[4];
        const int k0 = 8 * q + er;   // this lane's first K row (token) in the slab
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int col = wp + 16 * i + ca;
            a[i] = k3_tr_frag(XS, (k0 * XP + col) * 2, ((k0 + 4) * XP + col) * 2);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int col = wn + 16 * k + ca;
            bb[k] = k3_tr_frag(BS, (k0 * BP + col) * 2, ((k0 + 4) * BP + col) * 2);
        }
        mma_grid<bf16>(a, bb, acc);
    }
    float *Sc = S + ((size_t)(b * nc + c) * H + h) * P * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int n = n_lo + wn + 16 * k + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int p = p_lo + wp + 16 * i + 4 * q + e;
                if (p < P && n < N) Sc[(size_t)p * N + n] = acc[i][k][e];
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

// k3 (ADJ: its gradient-pass form) on operands xx, bb into out.
template <typename T, bool ADJ>
void launch_k3(const ForwardArgs &a, const void *xx, const void *bb, float *out,
               const int *segst, hipStream_t stream) {
    const int nc = a.nchunks, Q = a.Q;
    if constexpr (sizeof(T) == 4) {
        const int nblk = ((a.P + 63) / 64) * ((a.N + 127) / 128);
        hipLaunchKernelGGL(k3_chunk_state_f32<ADJ>, dim3(nc, a.H * nblk, a.batch), dim3(256),
                           K3F32Lds::bytes(), stream, (const float *)xx, (const float *)bb,
                           a.acum_hi, a.acum_lo, a.dtT, out, a.L, a.H, a.G, a.P, a.N, nc, Q, segst);
    } else {
        const int nblk = ((a.P + 63) / 64) * ((a.N + 127) / 128);
        hipLaunchKernelGGL(k3_chunk_state_bf16<ADJ>, dim3(nc, a.H * nblk, a.batch), dim3(256),
                           K3Bf16Lds::bytes(), stream, (const bf16 *)xx, (const bf16 *)bb,
                           a.acum_hi, a.acum_lo, a.dtT, out, a.L, a.H, a.G, a.P, a.N, nc, Q, segst);
    }
}

// The first four kernels of the forward alone (prefix sums, C B^T, chunk
// states, state passing; a.final_state receives the final state): what the
// gradient pass recomputes.
template <typename T>
hipError_t launch_split_states(const ForwardArgs &a, hipStream_t stream, hipEvent_t cb_done) {
    const int nc = a.nchunks, Q = a.Q;
    launch_dA_cumsum(a.dt, a.dtp, a.A, a.acum_hi, a.acum_lo, a.dtT, a.batch, a.L, a.H, nc, Q,
                     stream);
    const int nlb = (Q + 63) / 64;
    hipLaunchKernelGGL(k2_chunk_cb<T>, dim3(nlb * (nlb + 1) / 2, nc * a.G, a.batch),
                       dim3(256), 0, stream, (const T *)a.B, (const T *)a.C, (float *)a.cb, a.L,
                       a.G, a.N, nc, Q);
    if (cb_done) {
        const hipError_t err = hipEventRecord(cb_done, stream);
        if (err != hipSuccess) return err;
    }
    launch_k3<T, false>(a, a.x, a.B, a.S, nullptr, stream);
    const int PN = a.P * a.N;
    hipLaunchKernelGGL(k4_state_passing, dim3((PN + 1023) / 1024, a.H, a.batch), dim3(256),
                       0, stream, a.S, a.acum_hi, a.init, a.final_state, a.H, PN, nc, Q, nullptr);
    return hipGetLastError();
}

// The gradient pass's chunk products G_c = sum_s dy_s exp(acum_s) C_s^T.
template <typename T>
hipError_t launch_adj_chunk_states(const ForwardArgs &a, const void *dy, float *out,
                                   hipStream_t stream) {
    launch_k3<T, true>(a, dy, a.C, out, nullptr, stream);
    return hipGetLastError();
}

template hipError_t launch_split_states<float>(const ForwardArgs &, hipStream_t, hipEvent_t);
template hipError_t launch_split_states<bf16>(const ForwardArgs &, hipStream_t, hipEvent_t);
template hipError_t launch_adj_chunk_states<float>(const ForwardArgs &, const void *, float *, hipStream_t);
template hipError_t launch_adj_chunk_states<bf16>(const ForwardArgs &, const void *, float *, hipStream_t);

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
    launch_k3<T, false>(a, a.x, a.B, a.S, segst, stream);
    if ((err = mark()) != hipSuccess) return err;
    const int PN = a.P * a.N;
    hipLaunchKernelGGL(k4_state_passing, dim3((PN + 1023) / 1024, a.H, a.batch), dim3(256),
                       0, stream, a.S, a.acum_hi, a.init, a.final_state, a.H, PN, nc, Q, segst);
    if ((err = mark()) != hipSuccess) return err;
    const size_t k5_lds = K5Lds::bytes(a.P, (int)sizeof(T));
    // (the accumulators are sized by the padded headdim and the row blocks of a chunk)
    static_assert(kMaxHeaddim == 128, "k5 pads the headdim to 64 or 128");
    const bool p64 = a.P <= 64;
    const int nrb = Q >= 256 ? 4 : Q >= 128 ? 2 : 1;
    // (a chunk of 4 row blocks takes two workgroups of two blocks each, 2 row blocks two of one)
    auto k5 = nrb == 4 ? (p64 ? k5_chunk_scan<T, 4, 4, 2> : k5_chunk_scan<T, 8, 4, 2>)
            : nrb == 2 ? (p64 ? k5_chunk_scan<T, 4, 2, 1> : k5_chunk_scan<T, 8, 2, 1>)
                       : (p64 ? k5_chunk_scan<T, 4, 1, 1> : k5_chunk_scan<T, 8, 1, 1>);
    const int nsplit = nrb == 1 ? 1 : 2;
    hipLaunchKernelGGL(k5, dim3(nc * nsplit, a.H, a.batch), dim3(256), k5_lds,
                       stream, (const T *)a.x, (const T *)a.C, (const float *)a.cb, a.S, a.acum_hi,
                       a.acum_lo, a.dtT, a.D, (T *)a.y, a.L, a.H, a.G, a.P, a.N, nc, Q,
                       (const T *)a.z, a.D_hdim ? 1 : 0, segst);
    if ((err = mark()) != hipSuccess) return err;
    return hipGetLastError();
}

template hipError_t launch_split_forward<float>(const ForwardArgs &, hipStream_t, hipEvent_t *);
template hipError_t launch_split_forward<bf16>(const ForwardArgs &, hipStream_t, hipEvent_t *);

}  // namespace ssd
