// ssd_backward_kernels.hip -- the gradient pass of the chunked SSD forward
// (ssd_chunk_scan_bwd): the gradients of (y, final_state) with respect to x,
// dt, A, B, C, D and the initial state, recomputing the forward's
// intermediates instead of storing them (the recompute-backward path of the
// burn-mamba rustdoc, `ssd_serial_recalculated`; the pages give only its
// existence, the steps below are the derivative of the four steps of
// `ssd_minimal`, Eqs. 20-23).
//
// Notation, per batch b, head h (group g), chunk c of Q tokens; acum_t the
// chunk's inclusive prefix sum of dt A; h_in[c] the state entering chunk c
// (h_in[nc] the final state); Lam[c] = dLoss/dh_in[c + 1], the gradient with
// respect to the state at the end of chunk c.
//
//   Lam[nc-1] = dfinal;  Lam[c-1] = exp(acum_end[c]) Lam[c] + G_c,
//     G_c = sum_{s in c} exp(acum_s) dy_s (outer) C_s,  dinit = Lam[-1]
//   u_t   = sum_{s >= t} exp(acum_s - acum_t) (C_s . B_t) dy_s
//           + exp(acum_end - acum_t) Lam[c] B_t                          [P]
//   dx_t  = D dy_t + dt_t u_t
//   dB_t  = sum_h dt_t [ sum_{s >= t} exp(acum_s - acum_t) (x_t . dy_s) C_s
//           + exp(acum_end - acum_t) x_t Lam[c] ]                        [N]
//   dC_t  = sum_h [ sum_{s <= t} exp(acum_t - acum_s) dt_s (dy_t . x_s) B_s
//           + exp(acum_t) dy_t h_in[c] ]                                 [N]
//   dLoss/d(dt_t A) = g_t
//     = sum_{s >= t} roff_s + e^(acum_end) <Lam[c], h_in[c]>
//       + sum_{s >= t} sum_{s' < t} W[s][s'] + sum_{s' < t} dt_s' dint_s',
//     roff_s = <dy_s, e^(acum_s) h_in[c] C_s>  (the state part of <dy, y - D x>)
//     dint_s = x_s . (e^(acum_end - acum_s) Lam[c] B_s)  (the state part of x . u)
//     W[s][s'] = e^(acum_s - acum_s') dt_s' (dy_s . x_s') (C_s . B_s'), s' <= s
//   ddt_t = x_t . u_t + A g_t,  dA = sum_t dt_t g_t,  dD = sum_t dy_t . x_t
// g_t is <grad h_t, e^(dt_t A) h_{t-1}> of the serial loop (the fp64
// oracle's backward), regrouped by the chunked factors of Eqs. 20-23.  The
// plainer form, a reverse prefix sum over the chunk of <dy_k, y_k - D x_k> -
// dt_k x_k . u_k, subtracts terms that mostly cancel (the W block below the
// diagonal from both t onwards appears in both); the rectangle sum of W
// (rows >= t, columns < t) keeps only what remains, so g_t and dA keep the
// accuracy of their terms.
#include "ssd_device.hpp"
#include "ssd_backward.hpp"

namespace ssd {

namespace {

// Sum over the 64 lanes of the wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// Four values per lane summed over the 16 lanes of each 16-lane group (the
// lanes r of one MFMA output row group): lane r receives the total of value
// r >> 2.  A butterfly that halves the values each lane holds at its first
// two steps (5 exchanges instead of 16).
template <typename F>
__device__ __forceinline__ F row16_sum4(const F (&v)[4], int r) {
    const bool b3 = r & 8, b2 = r & 4;
    const F k0 = (b3 ? v[2] : v[0]) + __shfl_xor(b3 ? v[0] : v[2], 8, kWave);
    const F k1 = (b3 ? v[3] : v[1]) + __shfl_xor(b3 ? v[1] : v[3], 8, kWave);
    F t = (b2 ? k1 : k0) + __shfl_xor(b2 ? k0 : k1, 4, kWave);
    t += __shfl_xor(t, 2, kWave);
    t += __shfl_xor(t, 1, kWave);
    return t;
}

}  // namespace

// ------------------------------------------------------------ reverse state pass
// grid (nsl, H, b), 256 threads, 4 consecutive state elements per thread.
// Serial over chunks from the last: adj[c] holds G_c on entry and Lam[c] on
// exit; qpart gets each slice's share of <Lam[c], h_in[c]> (fp64).
__global__ void __launch_bounds__(256)
kb_state_passing(float *__restrict__ adj, const float *__restrict__ S,
                 const float *__restrict__ acum_hi,
                 const float *__restrict__ dfinal, float *__restrict__ dinit,
                 double *__restrict__ qpart, int H, int PN, int nc, int Q, int nsl) {
    __shared__ double red[4];
    const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int e0 = (blockIdx.x * 256 + tid) * 4;
    const bool in = e0 < PN;   // (PN is a multiple of 4: all four or none)
    const size_t soff = (size_t)(b * H + h) * PN + e0;
    f32x4 lam = zero4();
    if (in && dfinal) lam = *reinterpret_cast<const f32x4 *>(dfinal + soff);
    const float *ac = acum_hi + (size_t)(b * H + h) * nc * Q;
    for (int c = nc - 1; c >= 0; --c) {
        const size_t off = ((size_t)(b * nc + c) * H + h) * PN + e0;
        double part = 0.0;
        f32x4 G = zero4();
        if (in) {
            G = *reinterpret_cast<const f32x4 *>(adj + off);
            const f32x4 hn = *reinterpret_cast<const f32x4 *>(S + off);
            part = (double)lam[0] * hn[0] + (double)lam[1] * hn[1] + (double)lam[2] * hn[2] +
                   (double)lam[3] * hn[3];
            *reinterpret_cast<f32x4 *>(adj + off) = lam;
        }
        part = wave_sum_f64(part);
        if ((tid & 63) == 0) red[tid >> 6] = part;
        __syncthreads();
        if (tid == 0)
            qpart[((size_t)(b * nc + c) * H + h) * nsl + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
        __syncthreads();
        const float dec = fast_exp(ac[(size_t)c * Q + Q - 1]);
        lam = dec * lam + G;
    }
    if (in && dinit) *reinterpret_cast<f32x4 *>(dinit + soff) = lam;
}

// ------------------------------------------------------------ summed score tiles
// The dB and dC products share one matrix per (batch, chunk, group):
//   Ws[l][s] = sum_h e^(acum_l - acum_s) dt_s (dy_l . x_s)     (s <= l)
// dC_l gets sum_s Ws[l][s] B_s and dB_s gets sum_l Ws[l][s] C_l, so the
// products with B and C run once per group instead of once per head.  The
// dt A gradient needs, per head, the rectangle sums of W = Ws's head term
// times (C_l . B_s); they are the prefix over k < t of (column sum -
// row sum) of W's strict lower triangle (the entries with s < t, less
// those with l < t), so this kernel also writes each head's strict row sums
// (per tile) and column sums (per tile): the fp32 entries summed
// four at a time in fp32, then in fp64 (the prefix subtracts sums much
// larger than the result).
//
// Two launches: DIAG, grid (nrb, nc * G * nhg, b), the diagonal tiles; and
// grid (nrb (nrb - 1) / 2, nc * G * nhg, b), the tiles below them, where
// every entry is strict and the decay factors through the last row of the
// column block (one exponential per row and per column, not per entry).
// 256 threads, dynamic LDS 2 x 64 rows of x (pitch P + 16 / sizeof(T)), and
// 4 KB of column sums.
// Workgroup (lb, sb) (sb <= lb) owns the 64 x 64 tile of rows l in block lb,
// columns s in block sb; wave w its rows 16 w ..; it loops over hpw of the
// group's heads (head group k of nhg) with the tile's sum in registers and
// writes it as Ws in the operand type, or, with several head groups, as an
// fp32 partial sum that a separate pass adds up.
template <typename T, bool DIAG>
__global__ void __launch_bounds__(256)
kb_wsum(const T *__restrict__ x, const T *__restrict__ dy, const float *__restrict__ cb,
        const float *__restrict__ acum_hi, const float *__restrict__ acum_lo,
        const float *__restrict__ dtT, T *__restrict__ ws, float *__restrict__ wpart,
        double *__restrict__ rowp, double *__restrict__ colp, int L, int H, int G, int P,
        int nc, int Q, int hpw) {
    typedef typename Mma<T>::frag frag;
    constexpr int VEC = Mma<T>::VEC, KS = Mma<T>::KS;
    // Workgroups are dealt to the 8 XCDs in turn: when gridDim.y is a
    // multiple of 8 the tiles of one y (which read the same rows of x and
    // dy) are placed 8 apart, so that they share an L2.
    int pair = blockIdx.x, yy = blockIdx.y;
    if ((gridDim.y & 7) == 0) {
        const int id = blockIdx.x + gridDim.x * blockIdx.y, k = id >> 3;
        pair = k % gridDim.x;
        yy = (k / gridDim.x) * 8 + (id & 7);
    }
    int lb = pair, sb = pair;
    if constexpr (!DIAG) {
        lb = 1;
        while ((lb + 1) * lb / 2 <= pair) ++lb;
        sb = pair - lb * (lb - 1) / 2;
    }
    const int hpg = H / G, nhg = (hpg + hpw - 1) / hpw;
    const int hgi = yy % nhg, cg = yy / nhg;
    const int c = cg / G, g = cg % G, b = blockIdx.z;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;
    const int nrb = Q > 64 ? Q / 64 : 1;
    const int SB = Q < 64 ? Q : 64;
    const bool active = wave * 16 < SB;
    const size_t cbase = ((size_t)(b * nc + c) * G + g) * Q;
    // this lane's entries: rows l = lb SB + 16 w + 4 q + i, columns s = sb SB + 16 st + r
    int lrow[4], scol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lrow[i] = lb * SB + wave * 16 + 4 * q + i;
#pragma unroll
    for (int st = 0; st < 4; ++st) scol[st] = sb * SB + st * 16 + r;
    // C . B of the entries (the forward's lower triangle), 0 where unused
    float cbv[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = active && (!DIAG || (st * 16 + r < SB && scol[st] <= lrow[i]));
            cbv[st][i] = ok ? cb[(cbase + lrow[i]) * Q + scol[st]] : 0.f;
        }
    // x rows of block sb, one head at a time, shared by the four waves in
    // LDS (two buffers, rows of pitch XP: conflict-free 16-byte reads along
    // them); the next head's are loaded into registers while one is used
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T *xs = reinterpret_cast<T *>(smem_raw);
    const int XP = P + (sizeof(T) == 4 ? 4 : 8), xchunks = P / VEC, xtotal = SB * xchunks;
    // vector v of the block is row v / xchunks, chunk v % xchunks; the
    // quotient from a float product, exact here (v < 2^11, xchunks <= 32:
    // (v + 1/2) / xchunks is at least 1 / 64 from an integer)
    const float xrcp = 1.f / (float)xchunks;
    auto xrow = [&](int v) -> int { return (int)(((float)v + 0.5f) * xrcp); };
    auto xlds = [&](int v) -> int {
        const int row = xrow(v);
        return row * XP + (v - row * xchunks) * VEC;
    };
    // vectors per thread held across a head (the rest are loaded in place):
    // fp32 a headdim of 64; bf16 half of it, which keeps the kernel within
    // 128 VGPRs (four waves per SIMD, against three with the whole head)
    constexpr int XPF = sizeof(T) == 4 ? 4 : 1;
    frag xpre[XPF];
    // (addresses: a base per block and head, plus a 32-bit offset per lane)
    const int HP = H * P;
    const T *xblk = x + ((size_t)b * L + (size_t)c * Q + sb * SB) * HP + (size_t)g * hpg * P;
    auto xsrc = [&](int hh, int v) -> frag {
        const int row = xrow(v), k = (v - row * xchunks) * VEC;
        return c * Q + sb * SB + row < L ? load_frag(xblk + (size_t)hh * P + (row * HP + k)) : zero_frag<T>();
    };
    const int tr = c * Q + lb * SB + wave * 16 + r;   // this lane's dy row
    const T *dyrow = dy + ((size_t)b * L + c * Q + lb * SB + wave * 16) * HP + (size_t)g * hpg * P + r * HP;
    auto prefetch = [&](int hh) {
#pragma unroll
        for (int u = 0; u < XPF; ++u)
            if (tid + 256 * u < xtotal) xpre[u] = xsrc(hh, tid + 256 * u);
    };
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    const int h0 = hgi * hpw, h1 = min(hpg, h0 + hpw);
    // the four waves' column sums of a head, added up after the next barrier
    // (two buffers by head)
    __shared__ double csum[2][4][64];
    auto put_cols = [&](int hh) {
        if (tid < SB) {
            const double *cw = &csum[(hh - h0) & 1][0][tid];
            colp[(((size_t)(b * H + g * hpg + hh) * nc + c) * nrb + lb) * Q + sb * SB + tid] =
                ((cw[0] + cw[64]) + cw[128]) + cw[192];
        }
    };
    // The per-token vectors the tile needs, in LDS, one head at a time (two
    // buffers), loaded a head ahead, one array per wave: DIAG the block's
    // prefix sums (hi, lo) and dt (waves 0-2); below the diagonal the prefix
    // sums of row block lb (waves 0, 1) and of column block sb (waves 2, 3),
    // and the column block's dt (wave 0 again)
    constexpr int NA = DIAG ? 3 : 5;
    __shared__ float tokv[2][NA][64];
    const float *const tsrc = (wave & 1) ? acum_lo : DIAG && wave == 2 ? dtT : acum_hi;
    const int tblk = (DIAG || wave < 2 ? lb : sb) * SB;
    float tpre = 0.f, tpre2 = 0.f;
    auto tok_load = [&](int hh) {
        const size_t o = ((size_t)(b * H + g * hpg + hh) * nc + c) * Q + lane;
        if (!DIAG || wave < 3) tpre = lane < SB ? tsrc[o + tblk] : 0.f;
        if (!DIAG && wave == 0) tpre2 = lane < SB ? dtT[o + sb * SB] : 0.f;
    };
    if (h0 < h1) {
        prefetch(h0);
        tok_load(h0);
    }
    for (int hh = h0; hh < h1; ++hh) {
        const int h = g * hpg + hh;
        // (the buffer was last read two heads ago, before the previous barrier)
        T *xb = xs + (size_t)((hh - h0) & 1) * 64 * XP;
        const float *tk = &tokv[(hh - h0) & 1][0][0];
        if (!DIAG || wave < 3) tokv[(hh - h0) & 1][wave][lane] = tpre;
        if (!DIAG && wave == 0) tokv[(hh - h0) & 1][NA - 1][lane] = tpre2;
#pragma unroll
        for (int u = 0; u < XPF; ++u) {
            const int v = tid + 256 * u;
            if (v < xtotal) *reinterpret_cast<frag *>(xb + xlds(v)) = xpre[u];
        }
        for (int v = tid + 256 * XPF; v < xtotal; v += 256)
            *reinterpret_cast<frag *>(xb + xlds(v)) = xsrc(hh, v);
        __syncthreads();
        if (hh + 1 < h1) {
            prefetch(hh + 1);
            tok_load(hh + 1);
        }
        // strict row and column sums of W, four products at a time in fp32
        float rs[4] = {0.f, 0.f, 0.f, 0.f}, cs[4] = {0.f, 0.f, 0.f, 0.f};
        if (active) {
            // scores dy_l . x_s over the headdim
            f32x4 z[4] = {zero4(), zero4(), zero4(), zero4()};
            const T *arow = dyrow + (size_t)hh * P;
            for (int k0 = 0; k0 < P; k0 += KS) {
                const int k = k0 + VEC * q;
                const frag za = tr < L && k < P ? load_frag(arow + k) : zero_frag<T>();
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const frag zb = st * 16 + r < SB && k < P ? load_frag(xb + (st * 16 + r) * XP + k)
                                                              : zero_frag<T>();
                    z[st] = Mma<T>::mma(za, zb, z[st]);
                }
            }
            float lhi[4], llo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lhi[i] = tk[wave * 16 + 4 * q + i];
                llo[i] = tk[64 + wave * 16 + 4 * q + i];
            }
            if constexpr (!DIAG) {
                // below the diagonal (blocks of 64, all within the chunk)
                // every entry is strict (s < l) and the decay factors
                // through te, the last row of block sb: e^(acum_l - acum_s)
                // = e^(acum_l - acum_te) e^(acum_te - acum_s), both at most 1
                const float thi = tk[128 + SB - 1], tlo = tk[192 + SB - 1];
                float rf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) rf[i] = fast_exp(prefix_diff(lhi[i], llo[i], thi, tlo));
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const float shi = tk[128 + st * 16 + r], slo = tk[192 + st * 16 + r];
                    const float cf = fast_exp(prefix_diff(thi, tlo, shi, slo)) * tk[256 + st * 16 + r];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v = z[st][i] * rf[i] * cf;
                        acc[st][i] += v;
                        const float w = v * cbv[st][i];
                        rs[i] += w;
                        cs[st] += w;
                    }
                }
            } else {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const bool cin = st * 16 + r < SB;
                    const float shi = tk[st * 16 + r], slo = tk[64 + st * 16 + r];
                    const float sdt = tk[128 + st * 16 + r];   // (0 past SB)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // (exponent clamped at 0: the entries above the
                        // diagonal are selected away)
                        const float e = fast_exp(fminf(prefix_diff(lhi[i], llo[i], shi, slo), 0.f));
                        const float v = cin && scol[st] <= lrow[i] ? z[st][i] * e * sdt : 0.f;
                        acc[st][i] += v;
                        const float w = scol[st] < lrow[i] ? v * cbv[st][i] : 0.f;   // strict
                        rs[i] += w;
                        cs[st] += w;
                    }
                }
            }
        }
        // strict row sums (complete over the tile's columns) and the wave's
        // column sums over its 16 rows, in fp64 from here on (row
        // 4 q + (r >> 2)'s sum in lanes 4 (r >> 2) .. + 3).
        {
            const double rd[4] = {rs[0], rs[1], rs[2], rs[3]};
            const double v = row16_sum4(rd, r);
            const int row = wave * 16 + 4 * q + (r >> 2);
            if (active && (r & 3) == 0 && row < SB)
                rowp[(((size_t)(b * H + h) * nc + c) * nrb + sb) * Q + lb * SB + row] = v;
        }
        // columns: the same over the four row groups (lanes 16 apart) leaves
        // column tile q's sum in row group q; the waves' sums meet in LDS
        {
            const bool b5 = q & 2, b4 = q & 1;
            double k0 = b5 ? cs[2] : cs[0], k1 = b5 ? cs[3] : cs[1];
            k0 += __shfl_xor((double)(b5 ? cs[0] : cs[2]), 32, kWave);
            k1 += __shfl_xor((double)(b5 ? cs[1] : cs[3]), 32, kWave);
            double v = b4 ? k1 : k0;
            v += __shfl_xor(b4 ? k0 : k1, 16, kWave);
            csum[(hh - h0) & 1][wave][q * 16 + r] = v;
        }
        // (the previous head's, visible since this head's barrier)
        if (hh > h0) put_cols(hh - 1);
    }
    if (h0 < h1) {
        __syncthreads();
        put_cols(h1 - 1);
    }
    if (active) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (st * 16 + r < SB && lrow[i] - lb * SB < SB) {
                    const size_t o = (cbase + lrow[i]) * Q + scol[st];
                    if (wpart)
                        wpart[(size_t)hgi * gridDim.z * nc * G * Q * Q + o] = acc[st][i];
                    else
                        ws[o] = from_f32<T>(acc[st][i]);
                }
    }
}

// ------------------------------------------------------------ intra-chunk gradients
// The gradient products with the state and within the chunk.  dx has its
// own kernel (kb_dx); dB and dC share one (kb_mix, MODE):
//   kDb: rows t of group g, columns n: dB_t, summed over the group's heads
//   kDc: rows t of group g, columns n: dC_t, summed over the group's heads
// Each is   out_t = sum_heads rowscale_t stscale_t U_t St  +  sum_s Wt[t][s] V_s:
//            U (K)        St [K x W]        Wt[t][s]                 V
//   kDb:   x_t (P)      Lam              Ws[s][t], s >= t           C_s
//   kDc:   dy_t (P)     h_in             Ws[t][s], s <= t           B_s
// with stscale e^(acum_end - acum_t) (kDb) or e^(acum_t) (kDc), rowscale
// dt_t for kDb, and Ws from kb_wsum.  kDc also writes <dy_t, its state
// part> per head.
//
// grid (nc * nrb, G * nhg, b), 256 threads (4 waves), dynamic LDS
// KbLds::bytes.  Workgroup (c, lb) owns the SB = min(Q, 64) rows of row
// block lb; wave w the 16 rows 16 w .. 16 w + 15; NW 16-column tiles span
// the output width N (padded; padded columns are never stored).  A group's
// heads are split over nhg workgroups for the state products (fp32 partial
// sums, added up afterwards); the first of them also takes the intra-chunk
// product.  Workgroups are dealt to the 8 XCDs in turn; the row blocks of a
// chunk, which read the same states, are placed 8 apart so that they share
// an L2 (when nc is a multiple of 8).
//
// LDS operands keep the layout they arrive in (rows of tokens, of the state
// or of the score tile) and are read across rows where the MFMA wants
// columns: bf16 with the transposing LDS read, fp32 as four scalars with
// the K index kk + q + 4 j, from rows whose pitch puts the 64 lanes in 64
// banks.
enum { kDx = 0, kDb = 1, kDc = 2 };

struct KbLds {
    static constexpr int kSB = 64;
    // V by token: [kSB][vpitch] (fp32: = 16 mod 64 floats; bf16: 8 elements of padding)
    static __host__ __device__ constexpr int vpitch(int WP, int sz) {
        return sz == 4 ? WP + (80 - WP % 64) % 64 : WP + 8;
    }
    static __host__ __device__ constexpr size_t v_elems(int WP, int sz) {
        return (size_t)kSB * vpitch(WP, sz);
    }
    // + the score tile: [kSB][mpitch] (fp32: kDc's rows, read along them,
    // = 4 mod 64 floats; kDb's and kb_dx's, read across them, = 16 mod 64;
    // bf16: 8 elements of padding)
    static __host__ __device__ constexpr int mpitch(int sz, int mode) {
        return sz == 4 ? (mode == kDc ? kSB + 4 : kSB + 16) : kSB + 8;
    }
    static __host__ __device__ constexpr size_t m_elems(int sz) {
        return (size_t)kSB * (sz == 4 ? kSB + 16 : kSB + 8);
    }
    // + a slab of the state: kb_dx [WP][ks + 16 / sz] (Lam's rows cut to
    // the K-slab's columns), kDb / kDc [srows][WP + 16 / sz] (srows of the
    // state's rows, one MFMA K step, at most 8192 values)
    static __host__ __device__ constexpr int ks(int sz) { return sz == 4 ? 16 : 32; }
    static __host__ __device__ constexpr int srows(int WP, int sz) {
        return (sz == 4 ? 16 : 32) < 8192 / WP ? (sz == 4 ? 16 : 32) : 8192 / WP;
    }
    static __host__ __device__ constexpr int spitch(int WP, int sz, int mode) {
        return mode == kDx ? ks(sz) + 16 / sz : WP + 16 / sz;
    }
    static __host__ __device__ constexpr size_t s_elems(int WP, int sz) {
        return (size_t)WP * spitch(WP, sz, kDx) > (size_t)srows(WP, sz) * spitch(WP, sz, kDb)
                   ? (size_t)WP * spitch(WP, sz, kDx)
                   : (size_t)srows(WP, sz) * spitch(WP, sz, kDb);
    }
    // + prefix sums and dt by token and a reduction slot per wave (fp32)
    // (kDb / kDc reuse the space for their fp32 output rows, [kSB][WP + 4])
    static size_t bytes(int WP, int sz) {
        const size_t n = (v_elems(WP, sz) + m_elems(sz) + s_elems(WP, sz)) * sz + 3 * 256 * 4 + 64;
        const size_t o = (size_t)kSB * (WP + 4) * 4;
        return n > o ? n : o;
    }
    // kb_dx: its state slabs are done before the first V block is staged,
    // so they share V's space; + (bf16) the row block's x, then dx, by
    // token, shaped as V
    static size_t dx_bytes(int WP, int sz) {
        const size_t vs = v_elems(WP, sz) > s_elems(WP, sz) ? v_elems(WP, sz) : s_elems(WP, sz);
        return (vs + m_elems(sz) + (sz == 4 ? 0 : v_elems(WP, sz))) * sz + 3 * 256 * 4 + 64;
    }
};

typedef __bf16 kb_bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) kb_bf16x4 kb_lds_bf16x4;
typedef __attribute__((address_space(3))) unsigned char kb_lds_u8;

// The bf16 MFMA operand of K rows k0 .. k0 + 7 and 16 columns c0 .. of a
// row-major LDS tile, read across its rows: lane r + 16 q passes row
// k0 + (r >> 2) (row k0 + 4 + (r >> 2) for the second read) and columns
// c0 + 4 (r & 3) .. + 3, and receives column c0 + r of the four rows each
// read covers.  Called with row = k0 + (r >> 2), col = c0 + 4 (r & 3).
__device__ __forceinline__ bf16x8 kb_tr_frag(const bf16 *tile, int pitch, int row, int col) {
    const kb_bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (kb_lds_bf16x4 *)((kb_lds_u8 *)tile + (row * pitch + col) * 2));
    const kb_bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (kb_lds_bf16x4 *)((kb_lds_u8 *)tile + ((row + 4) * pitch + col) * 2));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Four fp32 values to LDS in the operand type (one 16- or 8-byte store).
template <typename T>
__device__ __forceinline__ void kb_store4(T *dst, f32x4 f) {
    if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<f32x4 *>(dst) = f;
    } else {
        *reinterpret_cast<kb_bf16x4 *>(dst) =
            kb_bf16x4{(bf16)f[0], (bf16)f[1], (bf16)f[2], (bf16)f[3]};
    }
}

// The MFMA operand of a row-major LDS tile read across its rows: K rows
// kk .. (fp32: kk + q + 4 j; bf16: kk + 8 q ..) and columns c0 + r.
template <typename T, int PITCH>
__device__ __forceinline__ typename Mma<T>::frag kb_across(const T *tile, int kk, int c0, int r,
                                                           int q) {
    if constexpr (sizeof(T) == 4) {
        typename Mma<T>::frag v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = tile[(kk + q + 4 * j) * PITCH + c0 + r];
        return v;
    } else {
        return kb_tr_frag(reinterpret_cast<const bf16 *>(tile), PITCH, kk + 8 * q + (r >> 2),
                          c0 + 4 * (r & 3));
    }
}

// ------------------------------------------------------------ dx
// u_t for the SB rows of row block lb of chunk c, head h, and from it dx_t,
// x_t . u_t, the state part x_t . (e^(acum_end - acum_t) Lam B_t) and the
// partial sum of dy . x.  With te the row block's last row, every decay
// that the rows take from beyond te factors through it (A <= 0: each
// factor is at most 1):
//   u_t = f_t [ B_t (e^(acum_end - acum_te) Lam)^T
//               + sum_{s beyond the block} (C_s . B_t) e^(acum_s - acum_te) dy_s ]
//         + sum_{s in the block, s >= t} (C_s . B_t) e^(acum_s - acum_t) dy_s,
//   f_t = e^(acum_te - acum_t),
// so only the diagonal block takes an exponential per entry.
//
// grid (H, nc * nrb, b) (heads fastest: the workgroups running together
// share a chunk's C B^T in L2, and with H a multiple of 8 a head's row
// blocks share an XCD), 256 threads, dynamic LDS KbLds::dx_bytes(16 NW).  Wave
// w owns rows 16 w ..; NW 16-column tiles span P.  The source blocks run
// from the chunk's last down to the diagonal one, which leaves dy of the
// row block itself staged for the epilogue.  The weighted C B^T block is
// staged by source rows s (as it is stored) and read across them.
template <typename T, int NW>
__global__ void __launch_bounds__(256)
kb_dx(const T *__restrict__ x, const T *__restrict__ Bm, const T *__restrict__ dy,
      const float *__restrict__ cb, const float *__restrict__ adj,
      const float *__restrict__ acum_hi, const float *__restrict__ acum_lo,
      const float *__restrict__ dtT, const float *__restrict__ D, T *__restrict__ out,
      float *__restrict__ dint, float *__restrict__ dd, float *__restrict__ dDpart, int L,
      int H, int G, int P, int N, int nc, int Q) {
    typedef typename Mma<T>::frag frag;
    constexpr int VEC = Mma<T>::VEC, KS = Mma<T>::KS;
    constexpr int SZ = (int)sizeof(T);
    constexpr int SBX = KbLds::kSB;
    constexpr int WP = 16 * NW;
    constexpr int VP = KbLds::vpitch(WP, SZ);
    constexpr int PITCH = KbLds::mpitch(SZ, kDx);
    constexpr int SP = KbLds::spitch(WP, SZ, kDx);
    static_assert(KS == KbLds::ks(SZ), "state slab width");
    extern __shared__ __align__(16) unsigned char smem_raw[];
    constexpr size_t VSE = KbLds::v_elems(WP, SZ) > KbLds::s_elems(WP, SZ) ? KbLds::v_elems(WP, SZ)
                                                                           : KbLds::s_elems(WP, SZ);
    T *VS = reinterpret_cast<T *>(smem_raw);            // [SBX][VP]: dy of the source block
    T *SS = VS;                                          // [WP][SP]: a K-slab of Lam's rows (before VS is used)
    T *MT = VS + VSE;                                    // [SBX][PITCH]: weighted C B^T, rows s
    float *r_hi = reinterpret_cast<float *>(MT + KbLds::m_elems(SZ));
    float *r_lo = r_hi + 256;
    float *r_dt = r_lo + 256;
    float *red = r_dt + 256;                             // [16]
    T *XS = reinterpret_cast<T *>(red + 16);             // (bf16) [SBX][VP]: x, then dx, of the row block
    // bf16: x and dx pass through LDS as rows (16-byte accesses); fp32 (whose
    // LDS would then halve the workgroups per CU) keeps x at the lane's
    // output positions in registers and stores dx from them
    constexpr bool XST = SZ != 4;

    const int nrb = Q > SBX ? Q / SBX : 1;
    const int h = blockIdx.x, c = blockIdx.y / nrb, lb = blockIdx.y % nrb, b = blockIdx.z;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;
    const int SB = Q < SBX ? Q : SBX;
    const int SBK = SB < KS ? KS : SB;       // rows the MFMAs read (zeros past SB)
    const bool active = wave * 16 < SB;
    const int g = h / (H / G);
    const int te = lb * SB + SB - 1;         // the row block's last row in the chunk
    const size_t vbase = ((size_t)(b * H + h) * nc + c) * Q;   // prefix sums, dt
    const size_t cbase = ((size_t)(b * nc + c) * G + g) * Q;

    for (int l = tid; l < Q; l += 256) {
        r_hi[l] = acum_hi[vbase + l];
        r_lo[l] = acum_lo[vbase + l];
        r_dt[l] = dtT[vbase + l];
    }
    // x rows of the row block (zero past L or P); per thread NV vectors
    constexpr int wv = WP / VEC, NV = SBX * wv / 256;
    const T *xrow = x + ((size_t)b * L * H + h) * P;
    float xv[XST ? 1 : 4][XST ? 1 : NW];
    if constexpr (XST) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = tid + 256 * u, sl = v / wv, w0 = (v % wv) * VEC, t = c * Q + lb * SB + sl;
            *reinterpret_cast<frag *>(XS + sl * VP + w0) =
                sl < SB && t < L && w0 < P ? load_frag(xrow + (size_t)t * H * P + w0) : zero_frag<T>();
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int l = lb * SB + wave * 16 + 4 * q + i, t = c * Q + l;
            const bool tin = active && t < L && l < Q;
#pragma unroll
            for (int wt = 0; wt < NW; ++wt) {
                const int p = wt * 16 + r;
                xv[i][wt] = tin && p < P ? to_f32(xrow[(size_t)t * H * P + p]) : 0.f;
            }
        }
    }
    // a row-major bf16 tile's values at this lane's output positions (rows
    // 4 q + i of the wave's 16, column 16 wt + r): one transposing read
    auto tr4 = [&](const T *tile, int wt, float (&o)[4]) {
        const kb_bf16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((kb_lds_bf16x4 *)(
            (kb_lds_u8 *)tile + ((wave * 16 + 4 * q + (r >> 2)) * VP + wt * 16 + 4 * (r & 3)) * 2));
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (float)t[i];
    };
    // x at those positions
    auto xat4 = [&](int wt, float (&o)[4]) {
        if constexpr (XST) {
            tr4(XS, wt, o);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = xv[i][wt];
        }
    };
    __syncthreads();
    const float e_te = fast_exp(prefix_diff(r_hi[Q - 1], r_lo[Q - 1], r_hi[te], r_lo[te]));
    float rowf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int l = min(lb * SB + wave * 16 + 4 * q + i, te);
        rowf[i] = fast_exp(prefix_diff(r_hi[te], r_lo[te], r_hi[l], r_lo[l]));
    }

    // ---- the state product B_t (e^(acum_end - acum_te) Lam)^T; Lam passes
    // through LDS in K-slabs of its rows' columns (SS[p][k])
    f32x4 acc[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) acc[i] = zero4();
    const float *st = adj + ((size_t)(b * nc + c) * H + h) * P * N;
    const int tr = c * Q + lb * SB + wave * 16 + r;   // this lane's B row
    const T *urow = Bm + (((size_t)b * L + tr) * G + g) * N;
    constexpr int kq = KS / 4, NSL = WP * kq / 256;   // float4 per thread and slab
    for (int k0 = 0; k0 < N; k0 += KS) {
        const int k = k0 + VEC * q;
        // (the slab's loads are issued before the barrier that frees the previous one)
        f32x4 pre[NSL];
#pragma unroll
        for (int u = 0; u < NSL; ++u) {
            const int v = tid + 256 * u, w = v / kq, kr = (v % kq) * 4;
            pre[u] = w < P && k0 + kr < N ? *reinterpret_cast<const f32x4 *>(st + (size_t)w * N + k0 + kr)
                                          : zero4();
        }
        const frag ua = active && tr < L && k < N ? load_frag(urow + k) : zero_frag<T>();
        __syncthreads();   // (the previous slab is no longer read)
#pragma unroll
        for (int u = 0; u < NSL; ++u) {
            const int v = tid + 256 * u, w = v / kq, kr = (v % kq) * 4;
            kb_store4(SS + w * SP + kr, e_te * pre[u]);
        }
        __syncthreads();
        if (!active) continue;
#pragma unroll
        for (int wt = 0; wt < NW; ++wt)
            acc[wt] = Mma<T>::mma(ua, load_frag(SS + (wt * 16 + r) * SP + VEC * q), acc[wt]);
    }
    if (active) {
        // the state part of x . u, per row (row 4 q + i's in lanes 4 i ..)
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int wt = 0; wt < NW; ++wt) {
            float xs[4];
            xat4(wt, xs);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] += xs[i] * acc[wt][i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= rowf[i];
        const float sv = row16_sum4(v, r);
        const int l = lb * SB + wave * 16 + 4 * q + (r >> 2), t = c * Q + l;
        if ((r & 3) == 0 && l < Q) dint[vbase + l] = t < L ? sv : 0.f;
    }

    // ---- the intra-chunk product, from the chunk's last source block down
    // to the diagonal one
    const T *vsrc = dy + ((size_t)b * L * H + h) * P;
    // per thread and block: NV operand vectors of dy, NC float4 of C B^T
    // (rows and columns up to kSB; those past SBK are zeros never read)
    constexpr int NC = SBX * (SBX / 4) / 256;
    for (int sb = nrb - 1; sb >= lb; --sb) {
        // the block's loads, issued before the barrier that frees the previous block
        frag vpre[NV];
        f32x4 cpre[NC];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = tid + 256 * u, sl = v / wv, w0 = (v % wv) * VEC, ts = c * Q + sb * SB + sl;
            vpre[u] = sl < SB && ts < L && w0 < P ? load_frag(vsrc + (size_t)ts * H * P + w0) : zero_frag<T>();
        }
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int v = tid + 256 * u, sl = v / (SBX / 4), tl = (v % (SBX / 4)) * 4;
            cpre[u] = sl < SB && tl < SB
                          ? *reinterpret_cast<const f32x4 *>(cb + (cbase + sb * SB + sl) * Q + lb * SB + tl)
                          : zero4();
        }
        __syncthreads();   // (the previous block's operands are no longer read)
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = tid + 256 * u, sl = v / wv, w0 = (v % wv) * VEC;
            *reinterpret_cast<frag *>(VS + sl * VP + w0) = vpre[u];
        }
        // MT[s][t] = (C_s . B_t) e^(acum_s - acum_te) beyond the block,
        // (C_s . B_t) e^(acum_s - acum_t) for s >= t in it (the upper
        // triangle, which the forward leaves unwritten, is selected away)
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int v = tid + 256 * u, sl = v / (SBX / 4), tl = (v % (SBX / 4)) * 4;
            f32x4 f = zero4();
            if (sl < SB && tl < SB) {
                const int ls = sb * SB + sl, lt0 = lb * SB + tl;
                const f32x4 cv = cpre[u];
                const float shi = r_hi[ls], slo = r_lo[ls];
                if (sb > lb) {
                    f = cv * fast_exp(prefix_diff(shi, slo, r_hi[te], r_lo[te]));
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int lt = lt0 + j;
                        const float e = fast_exp(fminf(prefix_diff(shi, slo, r_hi[lt], r_lo[lt]), 0.f));
                        f[j] = ls >= lt ? cv[j] * e : 0.f;
                    }
                }
            }
            kb_store4(MT + sl * PITCH + tl, f);
        }
        __syncthreads();
        if (!active) continue;
        if (sb == lb) {
#pragma unroll
            for (int wt = 0; wt < NW; ++wt)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[wt][i] *= rowf[i];
        }
        for (int kk = 0; kk < SBK; kk += KS) {
            const frag mf = kb_across<T, PITCH>(MT, kk, wave * 16, r, q);
#pragma unroll
            for (int wt = 0; wt < NW; ++wt)
                acc[wt] = Mma<T>::mma(mf, kb_across<T, VP>(VS, kk, wt * 16, r, q), acc[wt]);
        }
    }

    // ---- the epilogue: dx, x . u, dD (dy from the staged diagonal block).
    // bf16: each wave puts its rows' dx over their x in XS (only it reads
    // those rows), and the workgroup then stores XS by rows.
    if (active) {
        const float Dh = D ? D[h] : 0.f;
        float dsum = 0.f, ds[4] = {0.f, 0.f, 0.f, 0.f}, dtl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dtl[i] = r_dt[lb * SB + wave * 16 + 4 * q + i];
#pragma unroll
        for (int wt = 0; wt < NW; ++wt) {
            // dy and x at this lane's positions (bf16: read before any of
            // them is overwritten by dx; each lane writes only its own)
            float gv[4], xs[4];
            if constexpr (XST) {
                tr4(VS, wt, gv);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) gv[i] = to_f32(VS[(wave * 16 + 4 * q + i) * VP + wt * 16 + r]);
            }
            xat4(wt, xs);
            const int p = wt * 16 + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = wave * 16 + 4 * q + i, l = lb * SB + sl;
                const float u = acc[wt][i];
                ds[i] += xs[i] * u;
                dsum += gv[i] * xs[i];
                if constexpr (XST) {
                    XS[sl * VP + p] = from_f32<T>(Dh * gv[i] + dtl[i] * u);
                } else {
                    const int t = c * Q + l;
                    if (t < L && l < Q && p < P)
                        out[((size_t)b * L * H + h) * P + (size_t)t * H * P + p] = from_f32<T>(Dh * gv[i] + dtl[i] * u);
                }
            }
        }
        {
            const float sd = row16_sum4(ds, r);
            const int l = lb * SB + wave * 16 + 4 * q + (r >> 2), t = c * Q + l;
            if ((r & 3) == 0 && l < Q) dd[vbase + l] = t < L ? sd : 0.f;
        }
        dsum = wave_sum(dsum);
        if (lane == 0) red[wave] = dsum;
    }
    __syncthreads();
    if constexpr (XST) {
        T *orow = out + ((size_t)b * L * H + h) * P;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = tid + 256 * u, sl = v / wv, w0 = (v % wv) * VEC, t = c * Q + lb * SB + sl;
            if (sl < SB && t < L && w0 < P)
                *reinterpret_cast<frag *>(orow + (size_t)t * H * P + w0) =
                    *reinterpret_cast<const frag *>(XS + sl * VP + w0);
        }
    }
    if (tid == 0) {
        float sdd = 0.f;
        for (int w = 0; w < 4; ++w)
            if (w * 16 < SB) sdd += red[w];
        dDpart[((size_t)(b * nc + c) * H + h) * nrb + lb] = sdd;
    }
}

// ------------------------------------------------------------ dB and dC
template <typename T, int MODE, int NW>
__global__ void __launch_bounds__(256)
kb_mix(const T *__restrict__ x, const T *__restrict__ Bm, const T *__restrict__ Cm,
       const T *__restrict__ dy, const T *__restrict__ wsm, const float *__restrict__ S,
       const float *__restrict__ adj, const float *__restrict__ acum_hi,
       const float *__restrict__ acum_lo, const float *__restrict__ dtT, T *__restrict__ out,
       float *__restrict__ roff, float *__restrict__ part, int L, int H, int G, int P, int N,
       int nc, int Q, int hpw) {
    static_assert(MODE == kDb || MODE == kDc, "dB or dC");
    typedef typename Mma<T>::frag frag;
    constexpr int VEC = Mma<T>::VEC, KS = Mma<T>::KS;
    constexpr int SZ = (int)sizeof(T);
    constexpr bool F32 = SZ == 4;
    constexpr int SBX = KbLds::kSB;
    constexpr int WP = 16 * NW;
    constexpr int VP = KbLds::vpitch(WP, SZ);
    constexpr int PITCH = KbLds::mpitch(SZ, MODE);
    constexpr int SP = KbLds::spitch(WP, SZ, MODE);
    static_assert(KbLds::srows(WP, SZ) % KS == 0, "state slab height");
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T *VS = reinterpret_cast<T *>(smem_raw);                 // [SBX][VP]: V of the source block
    T *MT = VS + KbLds::v_elems(WP, SZ);                      // [SBX][PITCH]: the score tile
    T *SS = MT + KbLds::m_elems(SZ);                          // [SR][SP]: a slab of the state

    const int nrb = Q > SBX ? Q / SBX : 1;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;
    // x = (chunk, row block), y = (group, head group)
    int c, lb;
    {
        const int xi = blockIdx.x;
        if ((nc & 7) == 0) {
            const int m = xi >> 3;
            lb = m % nrb;
            c = (m / nrb) * 8 + (xi & 7);
        } else {
            c = xi / nrb;
            lb = xi % nrb;
        }
    }
    const int b = blockIdx.z;
    const int SB = Q < SBX ? Q : SBX;
    const int SBK = SB < KS ? KS : SB;       // tile columns the MFMAs read (zeros past SB)
    const bool active = wave * 16 < SB;
    const int hpg = H / G;
    // y = g * nhg + k takes heads k hpw .. of group g
    const int nhg = gridDim.y / G, hgi = blockIdx.y % nhg, g = blockIdx.y / nhg;
    const int h_first = g * hpg + hgi * hpw;
    const int h_count = min(hpw, hpg - hgi * hpw);
    const int t0 = c * Q + lb * SB;          // the row block's first token
    const size_t cbase = ((size_t)(b * nc + c) * G + g) * Q;

    f32x4 tot[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) tot[i] = zero4();
    // kDc: the row block's C rows, the same for every head of the group, in
    // VS while the heads run (the intra-chunk product reuses VS afterwards)
    if constexpr (MODE == kDc) {
        constexpr int wvc = WP / VEC;
        for (int v = tid; v < SBX * wvc; v += 256) {
            const int sl = v / wvc, w0 = (v % wvc) * VEC, t = t0 + sl;
            *reinterpret_cast<frag *>(VS + sl * VP + w0) =
                sl < SB && t < L && w0 < N ? load_frag(Cm + (((size_t)b * L + t) * G + g) * N + w0) : zero_frag<T>();
        }
    }

    // ---- the state products U_t St, scaled per row, head by head.  The
    // state passes through LDS in slabs of SR of its rows (SS[k][n]); a
    // slab's loads are issued before the barrier that waits for the
    // previous one to be used.
    constexpr int SR = KbLds::srows(WP, SZ);
    constexpr int NPRE = SR * WP / 1024;   // float4 per thread and slab
    constexpr int wq = WP / 4;
    const int nks = (P + SR - 1) / SR;     // slabs per head
    f32x4 pre[NPRE];
    auto load_slab = [&](int hh, int k0) {
        const float *st = (MODE == kDc ? S : adj) + ((size_t)(b * nc + c) * H + h_first + hh) * P * N;
#pragma unroll
        for (int u = 0; u < NPRE; ++u) {
            const int v = tid + 256 * u, kr = v / wq, w0 = (v % wq) * 4;
            pre[u] = w0 < N && k0 + kr < P ? *reinterpret_cast<const f32x4 *>(st + (size_t)(k0 + kr) * N + w0)
                                           : zero4();
        }
    };
    for (int hh = 0; hh < h_count; ++hh) {
        const int h = h_first + hh;
        const size_t vbase = ((size_t)(b * H + h) * nc + c) * Q;   // prefix sums, dt
        // this lane's rows' prefix sums and dt
        float rh[4], rl[4], rdt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int l = min(lb * SB + wave * 16 + 4 * q + i, Q - 1);
            rh[i] = acum_hi[vbase + l];
            rl[i] = acum_lo[vbase + l];
            rdt[i] = MODE == kDb ? dtT[vbase + l] : 0.f;
        }
        const float end_hi = acum_hi[vbase + Q - 1], end_lo = acum_lo[vbase + Q - 1];
        f32x4 acc[NW];
#pragma unroll
        for (int i = 0; i < NW; ++i) acc[i] = zero4();
        const int tr = t0 + wave * 16 + r;   // this lane's U row
        const T *urow = (MODE == kDb ? x : dy) + (((size_t)b * L + tr) * H + h) * P;
        for (int ks = 0; ks < nks; ++ks) {
            const int k0 = ks * SR;
            frag ua[SR / KS];
#pragma unroll
            for (int j = 0; j < SR / KS; ++j) {
                const int k = k0 + j * KS + VEC * q;
                ua[j] = active && tr < L && k < P ? load_frag(urow + k) : zero_frag<T>();
            }
            load_slab(hh, k0);
            __syncthreads();   // (the previous slab is no longer read)
#pragma unroll
            for (int u = 0; u < NPRE; ++u) {
                const int v = tid + 256 * u, kr = v / wq, w0 = (v % wq) * 4;
                kb_store4(SS + kr * SP + w0, pre[u]);
            }
            __syncthreads();
            if (active) {
#pragma unroll
                for (int j = 0; j < SR / KS; ++j)
#pragma unroll
                    for (int wt = 0; wt < NW; ++wt) {
                        frag sb;
                        if constexpr (F32) {
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj)
                                sb[jj] = SS[(j * KS + VEC * q + jj) * SP + wt * 16 + r];
                        } else {
                            sb = kb_across<T, SP>(SS, j * KS, wt * 16, r, q);
                        }
                        acc[wt] = Mma<T>::mma(ua[j], sb, acc[wt]);
                        // (one K step's operands at a time in registers)
                        if (wt == NW - 1) __builtin_amdgcn_sched_barrier(0);
                    }
            }
        }
        if (active) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = MODE == kDc ? fast_exp(rh[i])
                                            : fast_exp(prefix_diff(end_hi, end_lo, rh[i], rl[i]));
#pragma unroll
                for (int wt = 0; wt < NW; ++wt) acc[wt][i] *= e;
            }
            if constexpr (MODE == kDc) {
                // the state part of <dy, y - D x>, per row (row 4 q + i's
                // in lanes 4 i ..)
                float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int wt = 0; wt < NW; ++wt) {
                    // C at this lane's accumulator positions (rows 4 q + i,
                    // column 16 wt + r): bf16 one transposing read
                    float cv[4];
                    if constexpr (F32) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) cv[i] = to_f32(VS[(wave * 16 + 4 * q + i) * VP + wt * 16 + r]);
                    } else {
                        const kb_bf16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((kb_lds_bf16x4 *)(
                            (kb_lds_u8 *)VS + ((wave * 16 + 4 * q + (r >> 2)) * VP + wt * 16 + 4 * (r & 3)) * 2));
#pragma unroll
                        for (int i = 0; i < 4; ++i) cv[i] = (float)t[i];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] += cv[i] * acc[wt][i];
                }
                const float sv = row16_sum4(v, r);
                const int l = lb * SB + wave * 16 + 4 * q + (r >> 2), t = c * Q + l;
                if ((r & 3) == 0 && l < Q) roff[vbase + l] = t < L ? sv : 0.f;
            }
            // the head's state product into the group's sum (dB: times dt_t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sc = MODE == kDb ? rdt[i] : 1.f;
#pragma unroll
                for (int wt = 0; wt < NW; ++wt) tot[wt][i] += sc * acc[wt][i];
            }
        }
    }

    // ---- the intra-chunk product with the group's summed score tiles (by
    // the first head group only): dC rows lb x Ws[lb][sb] B[sb], sb <= lb;
    // dB rows lb x Ws[sb][lb]^T C[sb], sb >= lb
    if (hgi == 0) {
        const int sb_lo = MODE == kDc ? 0 : lb, sb_hi = MODE == kDc ? lb : nrb - 1;
        const T *vsrc = (MODE == kDb ? Cm : Bm) + ((size_t)b * L * G + g) * N;
        // per thread and block: NV operand vectors of V, NM of the tile (rows
        // and columns up to kSB; those past SBK are zeros never read)
        constexpr int wv = WP / VEC, mv = SBX / VEC, NV = SBX * wv / 256, NM = SBX * mv / 256;
        for (int sb = sb_lo; sb <= sb_hi; ++sb) {
            // the block's loads, issued before the barrier that frees the
            // previous block: V's rows, and the tile as stored (its upper
            // triangle on the diagonal is zero): kDc rows t of this block and
            // columns s of block sb, kDb rows s of block sb and columns t
            const int r0 = MODE == kDc ? lb * SB : sb * SB, c0 = MODE == kDc ? sb * SB : lb * SB;
            frag vpre[NV], mpre[NM];
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                const int v = tid + 256 * u, sl = v / wv, w0 = (v % wv) * VEC, ts = c * Q + sb * SB + sl;
                vpre[u] = sl < SB && ts < L && w0 < N ? load_frag(vsrc + (size_t)ts * G * N + w0)
                                                      : zero_frag<T>();
            }
#pragma unroll
            for (int u = 0; u < NM; ++u) {
                const int v = tid + 256 * u, i = v / mv, j = (v % mv) * VEC;
                mpre[u] = i < SB && j < SB ? load_frag(wsm + (cbase + r0 + i) * Q + c0 + j) : zero_frag<T>();
            }
            __syncthreads();   // (the previous block's V and tile are no longer read)
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                const int v = tid + 256 * u, sl = v / wv, w0 = (v % wv) * VEC;
                *reinterpret_cast<frag *>(VS + sl * VP + w0) = vpre[u];
            }
#pragma unroll
            for (int u = 0; u < NM; ++u) {
                const int v = tid + 256 * u, i = v / mv, j = (v % mv) * VEC;
                *reinterpret_cast<frag *>(MT + i * PITCH + j) = mpre[u];
            }
            __syncthreads();
            if (!active) continue;
            for (int kk = 0; kk < SBK; kk += KS) {
                // A: rows t (this wave's 16), K = s
                frag mf;
                if constexpr (MODE == kDc) {
                    if constexpr (F32) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) mf[j] = MT[(wave * 16 + r) * PITCH + kk + q + 4 * j];
                    } else {
                        mf = load_frag(MT + (wave * 16 + r) * PITCH + kk + 8 * q);
                    }
                } else {
                    mf = kb_across<T, PITCH>(MT, kk, wave * 16, r, q);
                }
#pragma unroll
                for (int wt = 0; wt < NW; ++wt)
                    tot[wt] = Mma<T>::mma(mf, kb_across<T, VP>(VS, kk, wt * 16, r, q), tot[wt]);
            }
        }
    }
    // ---- dB / dC rows of the row block, through LDS (fp32 rows of pitch
    // WP + 4, over the operand buffers) and stored as rows of 4-vectors;
    // several head groups write an fp32 partial sum each, added up afterwards
    constexpr int OP = WP + 4;
    float *OS = reinterpret_cast<float *>(smem_raw);
    __syncthreads();   // (the operand buffers are no longer read)
    if (active) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int wt = 0; wt < NW; ++wt) OS[(wave * 16 + 4 * q + i) * OP + wt * 16 + r] = tot[wt][i];
    }
    __syncthreads();
    constexpr int oq = WP / 4;
    for (int v = tid; v < SB * oq; v += 256) {
        const int row = v / oq, n0 = (v % oq) * 4, t = t0 + row;
        if (t >= L || n0 >= N) continue;
        const f32x4 f = *reinterpret_cast<const f32x4 *>(OS + row * OP + n0);
        const size_t o = (((size_t)b * L + t) * G + g) * N + n0;
        if (part) {
            *reinterpret_cast<f32x4 *>(part + (size_t)hgi * gridDim.z * L * G * N + o) = f;
        } else if constexpr (F32) {
            *reinterpret_cast<f32x4 *>(out + o) = f;
        } else {
            *reinterpret_cast<kb_bf16x4 *>(out + o) = kb_bf16x4{(bf16)f[0], (bf16)f[1], (bf16)f[2], (bf16)f[3]};
        }
    }
}

// ------------------------------------------------------------ head-group sums
// out[e] = the sum over k < nhg of part[k n + e], in that order.
template <typename T>
__global__ void __launch_bounds__(256)
kb_sum_heads(const float *__restrict__ part, T *__restrict__ out, size_t n, int nhg) {
    const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= n) return;   // (n is a multiple of 16)
    f32x4 acc = *reinterpret_cast<const f32x4 *>(part + e);
    for (int k = 1; k < nhg; ++k) acc += *reinterpret_cast<const f32x4 *>(part + (size_t)k * n + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[e + j] = from_f32<T>(acc[j]);
}

// ------------------------------------------------------------ ddt and dA
// Inclusive prefix sum over the workgroup's 256 threads (fp64); `tot` is a
// 4-slot LDS scratch, free again when the call returns.
__device__ __forceinline__ double block_scan_f64(double v, double *tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double inc = wave_inclusive_scan_f64(v, lane);
    if (lane == 63) tot[wave] = inc;
    __syncthreads();
    for (int w = 0; w < wave; ++w) inc += tot[w];
    __syncthreads();
    return inc;
}

// grid (nc, H, b), 256 threads, token t = tid of the chunk: g_t (the
// gradient with respect to dt_t A) from its four parts, ddt_t, and the
// chunk's share of dA, in fp64.  The rectangle sum is the exclusive prefix
// of (strict column sum - strict row sum) of W, each gathered from the
// per-tile partial sums of kb_wsum.
__global__ void __launch_bounds__(256)
kb_ddt(const float *__restrict__ roff, const float *__restrict__ dint,
       const float *__restrict__ dd, const double *__restrict__ rowp,
       const double *__restrict__ colp, const float *__restrict__ dtT,
       const float *__restrict__ acum_hi, const double *__restrict__ qpart,
       const float *__restrict__ A, float *__restrict__ ddt, double *__restrict__ dApart,
       int L, int H, int nc, int Q, int nsl, int nrb) {
    __shared__ double s_tot[4];
    __shared__ double s_red[4];
    __shared__ double s_suf[256];
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t vbase = ((size_t)(b * H + h) * nc + c) * Q;
    const size_t tbase = ((size_t)(b * H + h) * nc + c) * nrb;   // per-tile partials
    const int SB = Q < 64 ? Q : 64;
    const bool in = tid < Q;
    double qc = 0.0;
    for (int i = 0; i < nsl; ++i) qc += qpart[((size_t)(b * nc + c) * H + h) * nsl + i];
    qc *= (double)fast_exp(acum_hi[vbase + Q - 1]);
    const float dtl = in ? dtT[vbase + tid] : 0.f;
    // sum_{s >= t} roff_s: a prefix sum over the reversed order
    const double ro = in ? (double)roff[vbase + (Q - 1 - tid)] : 0.0;
    const double suf_rev = block_scan_f64(ro, s_tot);   // at thread j: sum over s >= Q-1-j
    if (in) s_suf[Q - 1 - tid] = suf_rev;
    // sum_{s' < t} dt_s' dint_s'
    const double di = in ? (double)dtl * dint[vbase + tid] : 0.0;
    const double pre = block_scan_f64(di, s_tot) - di;
    // the rectangle sum
    double cr = 0.0;
    if (in) {
        const int kb = tid / SB;
        for (int lb = kb; lb < nrb; ++lb)
            cr += colp[(tbase + lb) * Q + tid];
        for (int sb = 0; sb <= kb; ++sb) cr -= rowp[(tbase + sb) * Q + tid];
    }
    const double rect = block_scan_f64(cr, s_tot) - cr;
    __syncthreads();
    double gt = 0.0, contrib = 0.0;
    if (in) {
        gt = s_suf[tid] + qc + rect + pre;
        const int t = c * Q + tid;
        if (t < L) ddt[((size_t)b * L + t) * H + h] = (float)((double)dd[vbase + tid] + (double)A[h] * gt);
        contrib = (double)dtl * gt;
    }
    contrib = wave_sum_f64(contrib);
    if (lane == 0) s_red[wave] = contrib;
    __syncthreads();
    if (tid == 0) dApart[(size_t)(b * nc + c) * H + h] = s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

// ------------------------------------------------------------ dA and dD
// grid (H), 256 threads: head h's partial sums, each thread a fixed strided
// share, then a fixed-order tree (deterministic).
__global__ void __launch_bounds__(256)
kb_reduce(const double *__restrict__ dApart, const float *__restrict__ dDpart, float *__restrict__ dA,
          float *__restrict__ dD, int batch, int H, int nc, int nrb) {
    __shared__ double s_a[4], s_d[4];
    const int h = blockIdx.x, tid = threadIdx.x;
    double sa = 0.0, sd = 0.0;
    for (int bc = tid; bc < batch * nc; bc += 256) {
        sa += dApart[(size_t)bc * H + h];
        for (int k = 0; k < nrb; ++k) sd += dDpart[((size_t)bc * H + h) * nrb + k];
    }
    sa = wave_sum_f64(sa);
    sd = wave_sum_f64(sd);
    if ((tid & 63) == 0) {
        s_a[tid >> 6] = sa;
        s_d[tid >> 6] = sd;
    }
    __syncthreads();
    if (tid == 0) {
        dA[h] = (float)(s_a[0] + s_a[1] + s_a[2] + s_a[3]);
        if (dD) dD[h] = (float)(s_d[0] + s_d[1] + s_d[2] + s_d[3]);
    }
}

// ------------------------------------------------------------ launch

const char *const kBackwardKernelNames[kBackwardKernels] = {
    "k1..k4 (recompute)", "kb_adj_chunk_state", "kb_state_passing", "kb_dx", "kb_wsum",
    "kb_dB", "kb_dC", "kb_ddt", "kb_reduce"};

template <typename T, int NW>
static void launch_dx(const BackwardArgs &a, hipStream_t stream) {
    const ForwardArgs &f = a.f;
    const int nrb = bwd_row_blocks(f.Q);
    hipLaunchKernelGGL((kb_dx<T, NW>), dim3(f.H, f.nchunks * nrb, f.batch), dim3(256),
                       KbLds::dx_bytes(16 * NW, (int)sizeof(T)), stream, (const T *)f.x,
                       (const T *)f.B, (const T *)a.dy, (const float *)f.cb, (const float *)a.adj,
                       (const float *)f.acum_hi, (const float *)f.acum_lo, (const float *)f.dtT,
                       f.D, (T *)a.dx, a.dint, a.dd, a.dDpart, f.L, f.H, f.G, f.P, f.N,
                       f.nchunks, f.Q);
}

template <typename T, int MODE, int NW>
static void launch_mix(const BackwardArgs &a, void *out, float *part, hipStream_t stream) {
    const ForwardArgs &f = a.f;
    const int nrb = bwd_row_blocks(f.Q);
    const int hpg = f.H / f.G;
    const int hpw = bwd_heads_per_group(f.batch, f.nchunks, nrb, f.G, hpg);
    const int ny = f.G * ((hpg + hpw - 1) / hpw);
    hipLaunchKernelGGL((kb_mix<T, MODE, NW>), dim3(f.nchunks * nrb, ny, f.batch), dim3(256),
                       KbLds::bytes(16 * NW, (int)sizeof(T)), stream, (const T *)f.x,
                       (const T *)f.B, (const T *)f.C, (const T *)a.dy, (const T *)a.wsm,
                       (const float *)f.S, (const float *)a.adj, (const float *)f.acum_hi,
                       (const float *)f.acum_lo, (const float *)f.dtT, (T *)out, a.roff,
                       ny > f.G ? part : nullptr, f.L, f.H, f.G, f.P, f.N, f.nchunks, f.Q, hpw);
    if (ny > f.G) {
        const size_t n = (size_t)f.batch * f.L * f.G * f.N;
        hipLaunchKernelGGL(kb_sum_heads<T>, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0,
                           stream, (const float *)part, (T *)out, n, ny / f.G);
    }
}

template <typename T>
hipError_t launch_backward(const BackwardArgs &a, hipStream_t stream, hipEvent_t *events) {
    const ForwardArgs &f = a.f;
    int ev = 0;
    auto mark = [&]() -> hipError_t {
        return events ? hipEventRecord(events[ev++], stream) : hipSuccess;
    };
    // Without per-kernel events and with a side stream, the score tiles
    // (which need only the recompute's prefix sums and C B^T) and then dC
    // (which needs them and the recomputed states) run on the side stream,
    // beside the recompute's chunk states and their pass, the adjoint
    // products, the reverse state pass and dx; dB waits for both streams.
    const bool fork = !events && f.side != nullptr && a.ev_states != nullptr;
    auto launch_dc = [&](hipStream_t s) {
        if (f.N <= 128)
            launch_mix<T, kDc, 8>(a, a.dC, a.partC, s);
        else
            launch_mix<T, kDc, 16>(a, a.dC, a.partC, s);
    };
    auto launch_wsum = [&](hipStream_t s) {
        const int nrb = bwd_row_blocks(f.Q);
        const int ntile = nrb * (nrb + 1) / 2, hpg = f.H / f.G;
        const int hpw = bwd_wsum_heads(ntile, f.nchunks, f.G, f.batch, hpg);
        const int nhg = (hpg + hpw - 1) / hpw;
        const size_t lds = 2 * 64 * (size_t)(f.P + (sizeof(T) == 4 ? 4 : 8)) * sizeof(T);
        hipLaunchKernelGGL((kb_wsum<T, true>), dim3(nrb, f.nchunks * f.G * nhg, f.batch),
                           dim3(256), lds, s, (const T *)f.x, (const T *)a.dy,
                           (const float *)f.cb, (const float *)f.acum_hi, (const float *)f.acum_lo,
                           (const float *)f.dtT, (T *)a.wsm, nhg > 1 ? a.wpart : nullptr, a.rowp,
                           a.colp, f.L, f.H, f.G, f.P, f.nchunks, f.Q, hpw);
        if (nrb > 1)
            hipLaunchKernelGGL((kb_wsum<T, false>), dim3(ntile - nrb, f.nchunks * f.G * nhg, f.batch),
                               dim3(256), lds, s, (const T *)f.x, (const T *)a.dy,
                               (const float *)f.cb, (const float *)f.acum_hi,
                               (const float *)f.acum_lo, (const float *)f.dtT, (T *)a.wsm,
                               nhg > 1 ? a.wpart : nullptr, a.rowp, a.colp, f.L, f.H, f.G, f.P,
                               f.nchunks, f.Q, hpw);
        if (nhg > 1) {
            // (entries of a chunk's Q x Q block above its diagonal blocks stay
            // unwritten and are never read)
            const size_t n = (size_t)f.batch * f.nchunks * f.G * f.Q * f.Q;
            hipLaunchKernelGGL(kb_sum_heads<T>, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0,
                               s, (const float *)a.wpart, (T *)a.wsm, n, nhg);
        }
    };
    hipError_t err;
    if ((err = mark()) != hipSuccess) return err;
    // (the fork is recorded once the prefix sums and C B^T are queued, so the
    // score tiles also overlap the recompute's chunk states and their pass)
    if ((err = launch_split_states<T>(f, stream, fork ? f.ev_fork : nullptr)) != hipSuccess)
        return err;
    if (fork) {
        if ((err = hipEventRecord(a.ev_states, stream)) != hipSuccess) return err;
        if ((err = hipStreamWaitEvent(f.side, f.ev_fork, 0)) != hipSuccess) return err;
        launch_wsum(f.side);
        if ((err = hipStreamWaitEvent(f.side, a.ev_states, 0)) != hipSuccess) return err;
        launch_dc(f.side);
        if ((err = hipEventRecord(f.ev_join, f.side)) != hipSuccess) return err;
    }
    if ((err = mark()) != hipSuccess) return err;
    if ((err = launch_adj_chunk_states<T>(f, a.dy, a.adj, stream)) != hipSuccess) return err;
    if ((err = mark()) != hipSuccess) return err;
    const int PN = f.P * f.N, nsl = bwd_state_slices(f.P, f.N);
    hipLaunchKernelGGL(kb_state_passing, dim3(nsl, f.H, f.batch), dim3(256), 0, stream, a.adj,
                       (const float *)f.S, (const float *)f.acum_hi,
                       a.dfinal, a.dinit, a.qpart, f.H, PN, f.nchunks, f.Q, nsl);
    if ((err = mark()) != hipSuccess) return err;
    if (f.P <= 64)
        launch_dx<T, 4>(a, stream);
    else
        launch_dx<T, 8>(a, stream);
    if ((err = mark()) != hipSuccess) return err;
    if (fork) {
        if ((err = hipStreamWaitEvent(stream, f.ev_join, 0)) != hipSuccess) return err;
    } else {
        launch_wsum(stream);
    }
    if ((err = mark()) != hipSuccess) return err;
    if (f.N <= 128)
        launch_mix<T, kDb, 8>(a, a.dB, a.partB, stream);
    else
        launch_mix<T, kDb, 16>(a, a.dB, a.partB, stream);
    if ((err = mark()) != hipSuccess) return err;
    if (!fork) launch_dc(stream);
    if ((err = mark()) != hipSuccess) return err;
    hipLaunchKernelGGL(kb_ddt, dim3(f.nchunks, f.H, f.batch), dim3(256), 0, stream,
                       (const float *)a.roff, (const float *)a.dint, (const float *)a.dd,
                       (const double *)a.rowp, (const double *)a.colp, (const float *)f.dtT,
                       (const float *)f.acum_hi, (const double *)a.qpart, f.A, a.ddt, a.dApart,
                       f.L, f.H, f.nchunks, f.Q, nsl, bwd_row_blocks(f.Q));
    if ((err = mark()) != hipSuccess) return err;
    hipLaunchKernelGGL(kb_reduce, dim3(f.H), dim3(256), 0, stream,
                       (const double *)a.dApart, (const float *)a.dDpart, a.dA, a.dD, f.batch, f.H,
                       f.nchunks, bwd_row_blocks(f.Q));
    if ((err = mark()) != hipSuccess) return err;
    return hipGetLastError();
}

template hipError_t launch_backward<float>(const BackwardArgs &, hipStream_t, hipEvent_t *);
template hipError_t launch_backward<bf16>(const BackwardArgs &, hipStream_t, hipEvent_t *);

}  // namespace ssd
