// falcon_window.hip -- the window rules (Falcon-3 / Falcon-3A, W >= 2) at
// bf16 in a collapsed chunk form ("Fast Weight Attention for Continual
// Learning", authors' abstract: the sliding-window mini-batch update has a
// chunk-parallel form with positive-decay renormalization).
//
// Per tile of C = 32 steps s (tile-local), the window of step s holds the W
// pairs p = s .. s + W - 1 of the tile's E = C + W - 1 distinct pairs
// (x_p, y_p) = (k_{t0 - W + 1 - lag + p}, v_{t0 - W + 1 + p}); the virtual
// row r = s W + w (slot w) learns pair p(r) = s + W - 1 - w.  With g_s the
// tile-local cumulative log decay, D(s, s') = exp(g_s - g_s'), b_s the
// window step eta_s / (sum_{p in win(s)} ||x_p||^2 + eps) and the pair Gram
// G = X X^T, the residuals R of the CW virtual rows solve
//     (I + A) R = G_v Y - diag(gamma_v) G_v Z,   Z = X S0^T,
//     A[r][r'] = [s' < s] D(s, s') b_s' G[p(r)][p(r')],
// (G_v: the CW x E row gather of the pairs; the inner-product rule writes
// R = G_v Y instead).  Every later use of R goes through the pairs:
//     state    S_C = gamma_last S0 + delta^T X,   delta = H^T R,
//              H[r][p] = [p(r) = p] exp(g_last - g_s(r)) b_s(r);
//     outputs  O = diag(gamma) Q S0^T + P R,
//              P[t][r'] = [s' <= t] D(t, s') b_s' (q_t . x_p(r')).
// With M' = (I + A)^-1 G_v and M = (I + A)^-1 diag(gamma_v) G_v (CW x E) the
// state-independent parts collapse to E x E and C x E matrices,
//     N' = H^T M',  N = H^T M,  L' = P M',  L = P M,
//     delta = N' Y - N Z,   O = diag(gamma) Q S0^T + L' Y - L Z,
// which the intra-chunk kernel forms (bf16 MFMA blocked forward
// substitution, diagonal-block inverses from fp32 MFMA products) and stores
// per tile.  The state pass then walks C steps per tile with dense products
// only: X S0^T, [N' | -N] [Y; Z], the state update X^T delta and the
// outputs; no triangular solve is left on its sequential path.  The
// inner-product rule needs no system: delta_p = c_p y_p with
// c_p = sum_{s: p in win(s)} h_s, and L'[t][p] = (q_t . x_p) c'(t, p) with
// c'(t, p) = sum_{s' <= t, p in win(s')} D(t, s') b_s'.
//
// Every decay factor is exp(later - earlier) <= 1 of a log sum that
// restarts at each tile: nothing divides by a cumulative product.
#include "falcon_device.h"
#include "falcon_internal.h"
#include "falcon_records.h"
#include "falcon_rows.h"

namespace falcon {

namespace {

constexpr int kC = kWinC;        // steps per tile
constexpr int kEP = 48;          // pair slots: C + W - 1 <= 39 pairs, three 16-blocks
constexpr int kNPB = kEP / 16;   // pair blocks
constexpr int kNTB = kC / 16;    // step blocks
constexpr float kLog2e = 1.4426950408889634f;

// Record of one (batch*head, tile), bf16 MFMA fragments (64 lanes x 4 values,
// lane (lr, grp) holding M[lr][4 grp + r] of an A fragment, M[4 grp + r][lr]
// of a B fragment):
//   delta family: A fragments of [N' | -N] (pair block pb, K block kb < 6),
//                 B fragments of [L'^T; -L^T] (K block kb < 6, step block tb);
//   inner-product family: B fragments of L'^T (kb < 3);
// then floats: gamma_t = exp(g_t) (32), gamma_last at [32] and, for the
// inner-product family, c_p at [64 + p] (48).
template <bool DELTA>
struct WinRec {
    static constexpr int NFA = DELTA ? kNPB * 2 * kNPB : 0;
    static constexpr int NKB = DELTA ? 2 * kNPB : kNPB;
    static constexpr int NFB = kNTB * NKB;
    static constexpr size_t kA = 0;
    static constexpr size_t kB = (size_t)NFA * 512;
    static constexpr size_t kF = kB + (size_t)NFB * 512;
    static constexpr int NF = 128;
    static constexpr size_t kBytes = (kF + NF * 4 + 255) / 256 * 256;
    static __host__ __device__ constexpr int fa(int pb, int kb) { return pb * 2 * kNPB + kb; }
    static __host__ __device__ constexpr int fb(int tb, int kb) { return tb * NKB + kb; }
};

// Bytes of the records of BH sequences of nt tiles (256-byte multiples).
__host__ __device__ constexpr size_t window_records_bytes(int BH, int nt, bool delta) {
    return (size_t)BH * nt * (delta ? WinRec<true>::kBytes : WinRec<false>::kBytes);
}

// Step and pair of virtual row r (row r = s W + w learns pair s + W - 1 - w).
template <int W>
__host__ __device__ constexpr int row_step(int r) { return r / W; }
template <int W>
__host__ __device__ constexpr int row_pair(int r) { return r / W + W - 1 - (r - (r / W) * W); }

// Strictly lower blocks of A: index of block (rb, cb), cb < rb.
__host__ __device__ constexpr int lblk(int rb, int cb) { return rb * (rb - 1) / 2 + cb; }

// Steps spanned by row block rb and the most over all blocks: the diagonal
// block N of A is nilpotent of that order (each factor lowers the step).
template <int W>
constexpr int max_block_steps() {
    int m = 0;
    for (int rb = 0; rb < kC * W / 16; ++rb) {
        const int n = row_step<W>(16 * rb + 15) - row_step<W>(16 * rb) + 1;
        m = n > m ? n : m;
    }
    return m;
}
// Factors (I + (-N)^(2^j)), j < J, of (I + N)^-1 for N^(2^J) = 0.
template <int W>
constexpr int inv_factors() {
    int j = 0;
    while ((1 << j) < max_block_steps<W>()) ++j;
    return j < 1 ? 1 : j;
}

// ---------------------------------------------------------------------------
// Intra-chunk kernel: persistent, 256 threads, one (batch*head, tile) job at a
// time.
// ---------------------------------------------------------------------------
template <int D, int W, bool DELTA>
struct WinPrepSmem {
    static constexpr int LDX = D + 8;
    static constexpr int CW = kC * W, RB = CW / 16;
    static constexpr int NA = DELTA ? RB * (RB - 1) / 2 : 1;
    uint16_t X[kEP][LDX];                  // pair keys x_p (rows >= E zero)
    uint16_t Q[kC][LDX];                   // queries
    float al[kC], et[kC];                  // gates (padding steps: 1, 0)
    float nrm[kEP];                        // ||x_p||^2
    float g2[kC];                          // log2(e) * g_s
    float bs[kC];                          // window step b_s
    float hs[kC];                          // exp(g_last - g_s) b_s
    float gam[kC];                         // exp(g_s)
    float cf[DELTA ? CW : 1];              // exp2(gref(block of row j) - g2_s(j)) b_s(j)
    float gref[DELTA ? RB : 1];            // g2 at the step of a row block's last row
    float e2[DELTA ? 1 : kC * W];          // exp2(g2_t - g2_{t-d}) b_{t-d}, d < W
    float cpp[DELTA ? 1 : kEP];            // c'(p, p), p < C
    s16x4 Af[NA][64];                      // -A, strictly lower blocks
    s16x4 Tdf[DELTA ? RB : 1][64];         // (I + A_bb)^-1
    s16x4 Pf[kNTB][DELTA ? RB : 1][64];    // P blocks
};

template <int D, int W, bool DELTA>
__global__ __launch_bounds__(256, W <= 6 ? 2 : 1) void win_prep_kernel(ChunkArgs a, void* ws, int ntiles,
                                                       int njobs) {
    using E = EBf16;
    using T = uint16_t;
    using Frag = s16x4;
    using R = WinRec<DELTA>;
    using Smem = WinPrepSmem<D, W, DELTA>;
    constexpr int CPR = D / 8, CW = Smem::CW, RB = Smem::RB;
    constexpr int NP = kC + W - 1;  // pairs of a tile
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    const float eps = a.eps;
    if (a.toff) njobs = a.H * a.toff[a.BH / a.H];  // packed: the tiles that exist

    // The next job's keys, queries and gates are loaded into registers while
    // the current job computes, so their latency is hidden; a job's staging
    // then only moves them into LDS.
    constexpr int NXL = (kEP * CPR + 255) / 256, NQL = (kC * CPR + 255) / 256;
    u32x4 px[NXL], pq[NQL];
    float gal = 1.f, get = 0.f;
    auto valid = [&](int j) __attribute__((always_inline)) {
        const Job jb = job_of(a, j, ntiles);
        return jb.tile < tiles_of(jb.sr.T, kC);  // (uniform over the workgroup)
    };
    auto load_job = [&](int j) __attribute__((always_inline)) {
        const Job jb = job_of(a, j, ntiles);
        const int bh = jb.bh, T_ = jb.sr.T, t0 = jb.tile * kC;
        const T* kg = static_cast<const T*>(a.k) + jb.sr.row0 * D;
        const T* qg = static_cast<const T*>(a.q) + jb.sr.row0 * D;
        const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int c = tid + 256 * it;
            const int p = c / CPR, col = (c % CPR) * 8;
            const int tau = t0 - (W - 1) - a.lag + p;  // key of pair p
            const T* src = nullptr;
            if (c < kEP * CPR && p < NP && tau < T_) {
                if (tau >= 0) src = kg + (size_t)tau * D + col;
                else if (kp) src = kp + (size_t)(W + tau) * D + col;
            }
            px[it] = src ? *reinterpret_cast<const u32x4*>(src) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < NQL; ++it) {
            const int c = tid + 256 * it;
            const int t = c / CPR, col = (c % CPR) * 8;
            pq[it] = (c < kC * CPR && t0 + t < T_)
                         ? *reinterpret_cast<const u32x4*>(qg + (size_t)(t0 + t) * D + col)
                         : u32x4{0u, 0u, 0u, 0u};
        }
        gal = 1.f;
        get = 0.f;
        if (tid < kC && t0 + tid < T_) {
            gal = a.alpha[jb.sr.row0 + t0 + tid];
            get = a.eta[jb.sr.row0 + t0 + tid];
        }
    };
    int job = blockIdx.x;
    while (job < njobs && !valid(job)) job += gridDim.x;
    if (job < njobs) load_job(job);
    while (job < njobs) {
        const Job jb = job_of(a, job, ntiles);
        const int bh = jb.bh, tile = jb.tile;
        char* rec = static_cast<char*>(ws) + ((size_t)bh * ntiles + tile) * R::kBytes;

        // ---- stage pair keys, queries and gates ----
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int c = tid + 256 * it;
            if (c < kEP * CPR) *reinterpret_cast<u32x4*>(&sm.X[c / CPR][(c % CPR) * 8]) = px[it];
        }
#pragma unroll
        for (int it = 0; it < NQL; ++it) {
            const int c = tid + 256 * it;
            if (c < kC * CPR) *reinterpret_cast<u32x4*>(&sm.Q[c / CPR][(c % CPR) * 8]) = pq[it];
        }
        if (tid < kC) {
            sm.al[tid] = gal;
            sm.et[tid] = get;
        }
        int nxt = job + gridDim.x;
        while (nxt < njobs && !valid(nxt)) nxt += gridDim.x;
        lds_barrier();
        if (nxt < njobs) load_job(nxt);

        // ---- pair norms: 4 threads per pair ----
        {
            const int p = tid >> 2, part = tid & 3;
            float n2 = 0.f;
            if (p < kEP) {
#pragma unroll
                for (int c = 0; c < D / 4; c += 8) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.X[p][part * (D / 4) + c]);
                    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float x = E::to_f(e[u]);
                        n2 += x * x;
                    }
                }
            }
            n2 = group_sum_dpp<4>(n2);
            if (p < kEP && part == 0) sm.nrm[p] = n2;
        }
        lds_barrier();

        // ---- log-decay scan, window steps, per-step factors (wave 0) ----
        if (wave == 0) {
            const int s = lane;
            const float lg = wave_scan_dpp(s < kC ? __logf(sm.al[s]) : 0.f);
            const float glast = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lg), kC - 1));
            if (s < kC) {
                float tot = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) tot += sm.nrm[s + w];  // the pairs of step s
                const float den = tot + eps;
                const float b = den > 0.f ? sm.et[s] / den : 0.f;
                sm.g2[s] = lg * kLog2e;
                sm.bs[s] = b;
                sm.hs[s] = __expf(glast - lg) * b;
                sm.gam[s] = __expf(lg);
            }
        }
        lds_barrier();

        // ---- decay factors of the blocks; the Gram blocks on MFMA ----
        if constexpr (DELTA) {
            // column factors split at the last row of the column's block:
            // exp(g_ref - g_s(j)) <= 1, the row's factor exp(g_s(i) - g_ref) <= 1
            for (int j = tid; j < CW; j += 256) {
                const int s = row_step<W>(j), sref = row_step<W>(16 * (j / 16) + 15);
                sm.cf[j] = exp2f(sm.g2[sref] - sm.g2[s]) * sm.bs[s];
                if ((j & 15) == 15) sm.gref[j >> 4] = sm.g2[s];
            }
        } else {
            for (int i = tid; i < kC * W; i += 256) {
                const int t = i / W, d = i - t * W;
                sm.e2[i] = (t - d >= 0) ? exp2f(sm.g2[t] - sm.g2[t - d]) * sm.bs[t - d] : 0.f;
            }
        }
        // Gram block of two groups of 16 rows, rows as eight contiguous
        // contraction elements per lane: with lane l of each operand pointing
        // at its row's first element (plus 8 grp), lane (lr, grp) ends with
        // rowA(4 grp + r) . rowB(lr).  Rows are gathered by the addresses.
        auto gram = [&](const T* ar, const T* br) __attribute__((always_inline)) {
            f32x4 acc = zero4();
#pragma unroll
            for (int m = 0; m < D / 32; ++m)
                acc = E::mma32r(E::load8(ar + 32 * m), E::load8(br + 32 * m), acc);
            return acc;
        };
        lds_barrier();

        if constexpr (DELTA) {
            // ---- -A (strictly lower blocks), the diagonal inverses and P,
            // round-robin over the waves ----
            constexpr int NL = RB * (RB - 1) / 2;
            constexpr int NJ = NL + RB + kNTB * RB;
            auto run_job = [&](const int q) __attribute__((always_inline)) {
                if (q < NL) {
                    int rb = 1;
                    while (lblk(rb + 1, 0) <= q) ++rb;
                    const int cb = q - lblk(rb, 0);
                    const int i = 16 * rb + lr, si = row_step<W>(i);
                    // x_p(j) . x_p(i), j = 16 cb + 4 grp + r, on the matrix cores
                    const f32x4 gv = gram(&sm.X[row_pair<W>(16 * cb + lr)][8 * grp],
                                          &sm.X[row_pair<W>(i)][8 * grp]);
                    const float rf = exp2f(sm.g2[si] - sm.gref[cb]);
                    // factors loaded for every lane, then selected: a load
                    // under a lane condition would become a branch
                    const f32x4 cfv = *reinterpret_cast<const f32x4*>(&sm.cf[16 * cb + 4 * grp]);
                    f32x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * cb + 4 * grp + r;
                        const float e = -(rf * cfv[r] * gv[r]);
                        v[r] = (row_step<W>(j) < si) ? e : 0.f;
                    }
                    sm.Af[q][lane] = E::pack(v);
                } else if (q < NL + RB) {
                    // (I + N)^-1, N the diagonal block (nilpotent: every nonzero
                    // entry lowers the step), as the product of the factors
                    // I + (-N)^(2^j) in fp32 MFMA.  Fragments: a(X) holds
                    // X[lr][4 grp + r], b(X) holds X[4 grp + r][lr]; a product's
                    // accumulator is b(XY), and a(X) = b(X^T).  The chain builds
                    // c(F_{J-1}^T .. F_0^T) = c(Td^T) = a(Td).
                    const int rb = q - NL;
                    // the block's Gram x_p(16 rb + 4 grp + r) . x_p(16 rb + lr),
                    // symmetric, so it serves both fragment layouts of N
                    const T* xr = &sm.X[row_pair<W>(16 * rb + lr)][8 * grp];
                    const f32x4 gv = gram(xr, xr);
                    auto nfac = [&](int i, int j) __attribute__((always_inline)) {
                        const int si = row_step<W>(i), sj = row_step<W>(j);
                        // evaluated for every lane and selected (no branch);
                        // the discarded values may be large but are never used
                        const float e = exp2f(sm.g2[si] - sm.g2[sj]) * sm.bs[sj];
                        return sj < si ? e : 0.f;
                    };
                    f32x4 aN, bN, aI;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        aN[r] = nfac(16 * rb + lr, 16 * rb + 4 * grp + r) * gv[r];
                        bN[r] = nfac(16 * rb + 4 * grp + r, 16 * rb + lr) * gv[r];
                        aI[r] = (lr == 4 * grp + r) ? 1.f : 0.f;
                    }
                    f32x4 Y = aI - aN;  // b(F_0^T) = a(I - N)
                    f32x4 aP = aN, bP = bN;
                    constexpr int J = inv_factors<W>();
#pragma unroll
                    for (int j = 1; j < J; ++j) {
                        const f32x4 bP2 = EFp32::mma16(aP, bP, zero4());  // b(P^2)
                        if (j + 1 < J) aP = EFp32::mma16(bP, aP, zero4());  // a(P^2) = c(P^T P^T)
                        bP = bP2;
                        Y = EFp32::mma16(aI + bP, Y, zero4());  // F_j^T Y, a(F_j^T) = b(F_j)
                    }
                    sm.Tdf[rb][lane] = E::pack(Y);
                } else {
                    const int qq = q - NL - RB;
                    const int tb = qq / RB, rb = qq - tb * RB;
                    const int t = 16 * tb + lr;
                    // fully causal block: every row's step <= every t of the block
                    const bool full = row_step<W>(16 * rb + 15) <= 16 * tb;
                    const float rf = full ? exp2f(sm.g2[t] - sm.gref[rb]) : 0.f;
                    // x_p(j) . q_t, j = 16 rb + 4 grp + r
                    const f32x4 gv = gram(&sm.X[row_pair<W>(16 * rb + lr)][8 * grp], &sm.Q[t][8 * grp]);
                    f32x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * rb + 4 * grp + r, sj = row_step<W>(j);
                        const float qk = gv[r];
                        if (full) {
                            v[r] = rf * sm.cf[j] * qk;
                        } else {
                            const float e = exp2f(sm.g2[t] - sm.g2[sj]) * sm.bs[sj] * qk;
                            v[r] = sj <= t ? e : 0.f;
                        }
                    }
                    sm.Pf[tb][rb][lane] = E::pack(v);
                }
            };
            if constexpr (NJ <= 64) {
                // each wave's jobs q = wave + 4 i unrolled with constant q (the
                // tests on q fold away), so one job's loads and products
                // overlap the previous job's factor arithmetic
                with_const4(wave, [&](auto wc) __attribute__((always_inline)) {
                    constexpr int WV = decltype(wc)::value;
                    static_for<(NJ - WV + 3) / 4>([&](auto ic) __attribute__((always_inline)) {
                        run_job(WV + 4 * decltype(ic)::value);
                    });
                });
            } else {
                for (int q = wave; q < NJ; q += 4) run_job(q);
            }
            lds_barrier();

            // ---- blocked forward substitution (waves 0-2, pair block q each):
            // M'_rb = Td_rb (G_v,rb - sum_{c<rb} A_rb,c M'_c) and the same for M
            // with the gamma-scaled right-hand side; as each block of rows is
            // done it enters N^T = M^T H and L^T = M^T P^T ----
            if (wave < kNPB) {
                const int q = wave;
                Frag Mp[RB], Mg[RB];
                f32x4 nP[kNPB], nG[kNPB], lP[kNTB], lG[kNTB];
#pragma unroll
                for (int i = 0; i < kNPB; ++i) nP[i] = nG[i] = zero4();
#pragma unroll
                for (int i = 0; i < kNTB; ++i) lP[i] = lG[i] = zero4();
                static_for<RB>([&](auto rbc) __attribute__((always_inline)) {
                    constexpr int rb = decltype(rbc)::value;
                    f32x4 acc1, acc2;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * rb + 4 * grp + r;
                        const float one = (row_pair<W>(i) == 16 * q + lr) ? 1.f : 0.f;
                        acc1[r] = one;
                        acc2[r] = one * sm.gam[row_step<W>(i)];
                    }
                    // two blocks c, c + 1 per product
                    static_for<(rb + 1) / 2>([&](auto cc) __attribute__((always_inline)) {
                        constexpr int c = 2 * decltype(cc)::value;
                        const Frag af = sm.Af[lblk(rb, c)][lane];
                        if constexpr (c + 1 < rb) {
                            const Frag af1 = sm.Af[lblk(rb, c + 1)][lane];
                            acc1 = E::mma32(af, af1, Mp[c], Mp[c + 1], acc1);
                            acc2 = E::mma32(af, af1, Mg[c], Mg[c + 1], acc2);
                        } else {
                            acc1 = E::mma16(af, Mp[c], acc1);
                            acc2 = E::mma16(af, Mg[c], acc2);
                        }
                    });
                    const Frag td = sm.Tdf[rb][lane];
                    Mp[rb] = E::pack(E::mma16(td, E::pack(acc1), zero4()));
                    Mg[rb] = E::pack(E::mma16(td, E::pack(acc2), zero4()));
                    // N and L from row blocks rb - 1 and rb together (RB = 2 W is
                    // even); a block whose rows miss pair block pb contributes
                    // zeros of h, one whose steps all follow step block tb zeros of P
                    if constexpr (rb % 2 == 1) {
                        constexpr int r0 = rb - 1;
                        constexpr int plo = row_step<W>(16 * r0), phi_ = row_step<W>(16 * rb + 15) + W - 1;
                        // h of the two blocks' rows, read for every lane and
                        // selected per pair block below
                        f32x4 hs0, hs1;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            hs0[r] = sm.hs[row_step<W>(16 * r0 + 4 * grp + r)];
                            hs1[r] = sm.hs[row_step<W>(16 * rb + 4 * grp + r)];
                        }
                        static_for<kNPB>([&](auto pbc) __attribute__((always_inline)) {
                            constexpr int pb = decltype(pbc)::value;
                            if constexpr (16 * pb <= phi_ && 16 * pb + 15 >= plo) {
                                f32x4 h0, h1;
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int j0 = 16 * r0 + 4 * grp + r, j1 = j0 + 16;
                                    h0[r] = (row_pair<W>(j0) == 16 * pb + lr) ? hs0[r] : 0.f;
                                    h1[r] = (row_pair<W>(j1) == 16 * pb + lr) ? hs1[r] : 0.f;
                                }
                                const Frag hb0 = E::pack(h0), hb1 = E::pack(h1);
                                nP[pb] = E::mma32(Mp[r0], Mp[rb], hb0, hb1, nP[pb]);
                                nG[pb] = E::mma32(Mg[r0], Mg[rb], hb0, hb1, nG[pb]);
                            }
                        });
                        static_for<kNTB>([&](auto tbc) __attribute__((always_inline)) {
                            constexpr int tb = decltype(tbc)::value;
                            if constexpr (row_step<W>(16 * r0) <= 16 * tb + 15) {
                                const Frag pf0 = sm.Pf[tb][r0][lane], pf1 = sm.Pf[tb][rb][lane];
                                lP[tb] = E::mma32(Mp[r0], Mp[rb], pf0, pf1, lP[tb]);
                                lG[tb] = E::mma32(Mg[r0], Mg[rb], pf0, pf1, lG[tb]);
                            }
                        });
                    }
                });
                // the accumulator of N^T block (q, pb) is the A fragment of N
                // block (pb, q); that of L^T block (q, tb) the B fragment of L^T
                // block (q, tb)
                Frag* fa = reinterpret_cast<Frag*>(rec + R::kA);
                Frag* fb = reinterpret_cast<Frag*>(rec + R::kB);
#pragma unroll
                for (int pb = 0; pb < kNPB; ++pb) {
                    fa[R::fa(pb, q) * 64 + lane] = E::pack(nP[pb]);
                    fa[R::fa(pb, kNPB + q) * 64 + lane] = E::pack(-nG[pb]);
                }
#pragma unroll
                for (int tb = 0; tb < kNTB; ++tb) {
                    fb[R::fb(tb, q) * 64 + lane] = E::pack(lP[tb]);
                    fb[R::fb(tb, kNPB + q) * 64 + lane] = E::pack(-lG[tb]);
                }
            } else {
                float* fl = reinterpret_cast<float*>(rec + R::kF);
                if (lane < kC) fl[lane] = sm.gam[lane];
                if (lane == 0) fl[kC] = sm.gam[kC - 1];
            }
        } else {
            // ---- inner-product family: c'(p, p) and c_p, then L'^T ----
            if (tid < kEP) {
                const int p = tid;
                float cq = 0.f, c = 0.f;
                if (p < kC) {
#pragma unroll
                    for (int d = 0; d < W; ++d)
                        if (d <= p) cq += sm.e2[p * W + d];
                }
#pragma unroll
                for (int d = 0; d < W; ++d) {
                    const int s = p - d;  // steps whose window holds pair p
                    if (p < NP && s >= 0 && s < kC) c += sm.hs[s];
                }
                sm.cpp[p] = cq;
                float* fl = reinterpret_cast<float*>(rec + R::kF);
                fl[64 + p] = c;
                if (p < kC) fl[p] = sm.gam[p];
                if (p == 0) fl[kC] = sm.gam[kC - 1];
            }
            lds_barrier();
            Frag* fb = reinterpret_cast<Frag*>(rec + R::kB);
            for (int q = wave; q < kNTB * kNPB; q += 4) {
                const int tb = q / kNPB, kb = q - tb * kNPB;
                const int t = 16 * tb + lr;
                // q_t . x_p, p = 16 kb + 4 grp + r, on the matrix cores
                const f32x4 qk = gram(&sm.X[16 * kb + lr][8 * grp], &sm.Q[t][8 * grp]);
                // both cases evaluated for every lane and selected (a load or
                // transcendental under a lane condition would become a branch)
                float e2v[W];
#pragma unroll
                for (int d = 0; d < W; ++d) e2v[d] = sm.e2[t * W + d];
                const float g2t = sm.g2[t];
                f32x4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = 16 * kb + 4 * grp + r;
                    const float near = exp2f(g2t - sm.g2[min(p, kC - 1)]) * sm.cpp[p];
                    // steps s' in [p - W + 1, t]: d = t - s'
                    float far = 0.f;
#pragma unroll
                    for (int d = 0; d < W; ++d) far += (t - d >= p - W + 1 && t - d >= 0) ? e2v[d] : 0.f;
                    v[r] = qk[r] * (p <= t ? near : far);
                }
                fb[R::fb(tb, kb) * 64 + lane] = E::pack(v);
            }
        }
        lds_barrier();  // the next job's staging overwrites the tiles
        job = nxt;
    }
}

// ---------------------------------------------------------------------------
// Segmented state pass of the inner-product rule.  Its state increments do
// not depend on the state, so after a run of tiles that starts from a state S
// the state is (the product of the run's gamma_last) S plus the state the
// same run reaches from zero.  The state pass therefore cuts each chain of
// ntl tiles into kSegs segments of seg_len(ntl) tiles (a multiple of
// kSegTiles) and runs them all at once; segment s starts from the state after
// s seg_len tiles, which win_seg_kernel forms beforehand: the tiles before
// the last segment in groups of kSegTiles, each group's state from zero
// (part; group 0 from S0) and the product of its gamma_last (gprod),
// combined group by group when a segment starts.  That kernel also keeps a
// copy of S0 for the first segment, so the state pass never reads the
// caller's S0, which S_final may alias.  Calls whose longest chain has fewer
// than kSegMinTiles tiles keep one segment.
// ---------------------------------------------------------------------------
constexpr int kSegTiles = 32;
constexpr int kSegMinTiles = 64;
constexpr int kSegs = 4;
__host__ __device__ constexpr int seg_len(int ntl) {
    return ((ntl + kSegs - 1) / kSegs + kSegTiles - 1) / kSegTiles * kSegTiles;
}
// tiles whose group states a chain of ntl tiles needs: those before its last segment
__host__ __device__ constexpr int seg_prefix(int ntl) {
    return (kSegs - 1) * seg_len(ntl) < ntl ? (kSegs - 1) * seg_len(ntl) : ntl;
}
__host__ __device__ constexpr int seg_groups(int ntiles) {
    return (seg_prefix(ntiles) + kSegTiles - 1) / kSegTiles;
}
// Float offset of the copy of S0 in the segment buffer: after the group
// states and the gates' products (padded to 256 bytes).
__host__ __device__ constexpr size_t seg_s0_offset(int BH, int gmax, int D) {
    return (size_t)BH * gmax * D * D + ((size_t)BH * gmax + 63) / 64 * 64;
}

// One workgroup of D / 16 waves per (group g, batch*head): wave w carries
// value columns 16 w .. 16 w + 15 of the group's state from zero, with the
// state pass's per-tile update S^T = gamma_last S^T + X^T delta,
// delta_p = c_p y_p; every key tile is loaded once for all columns.  Keys and
// values are staged through registers one tile ahead (tile 0 reads the halo
// rows, as the state pass does).
// part: [BH][gmax][D][D] fp32 (S layout, [v][k]), then gprod [BH][gmax],
// then the copy of S0 [BH][D][D] (group 0's workgroups write it).
template <int D>
__global__ __launch_bounds__(4 * D) void win_seg_kernel(ChunkArgs a, const void* ws, int ntiles, int gmax,
                                                        float* part) {
    using E = EBf16;
    using T = uint16_t;
    using Frag = s16x4;
    using R = WinRec<false>;
    constexpr int KB = D / 16, CPR = D / 8, NT = 4 * D;
    constexpr int NXC = kEP * CPR;  // 16-byte pieces of a key (and of a value) tile
    constexpr int NXL = (NXC + NT - 1) / NT;
    __shared__ alignas(16) uint16_t X[kEP * D];  // pair keys, swizzled rows as in the state pass
    __shared__ alignas(16) uint16_t V[kEP * D];  // pair values
    __shared__ alignas(16) float cf[kEP + 16];   // c_p, then gamma_last at [kEP]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, lr = lane & 15;
    const int g = blockIdx.x / a.BH, bh = blockIdx.x - g * a.BH;
    const int W = a.W, NP = kC + W - 1;
    const SeqRows sr = seq_rows(a, bh);
    const int T_ = sr.T, ntl = tiles_of(T_, kC), Lt = seg_prefix(ntl);
    const int j0 = g * kSegTiles, j1 = min(j0 + kSegTiles, Lt);
    const float* s0 = a.S0 ? a.S0 + (size_t)bh * D * D : nullptr;
    if (g == 0 && s0) {
        // the first segment's copy of S0
        float* c = part + seg_s0_offset(a.BH, gmax, D) + (size_t)bh * D * D;
        for (int i = tid; i < D * D / 4; i += NT)
            reinterpret_cast<f32x4*>(c)[i] = reinterpret_cast<const f32x4*>(s0)[i];
    }
    if (j0 >= j1) return;  // a group the state pass does not read
    const T* kg = static_cast<const T*>(a.k) + sr.row0 * D;
    const T* vg = static_cast<const T*>(a.v) + sr.row0 * D;
    const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
    const T* vp = a.v_prev ? static_cast<const T*>(a.v_prev) + (size_t)bh * (W - 1) * D : nullptr;
    const float* recf = reinterpret_cast<const float*>(static_cast<const char*>(ws) +
                                                       (size_t)bh * ntiles * R::kBytes + R::kF);
    constexpr size_t RF = R::kBytes / 4;  // record stride in floats

    u32x4 px[NXL], pv[NXL];
    float pc = 0.f;
    auto load = [&](int j) __attribute__((always_inline)) {
        const int t0 = j * kC;
        const u32x4 zz = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NXL; ++i) {
            const int c = tid + NT * i;
            const int p = c / CPR, col = (c % CPR) * 8;
            const int tau = t0 - (W - 1) - a.lag + p;  // key of pair p
            const T* src = nullptr;
            if (c < NXC && p < NP && tau < T_) {
                if (tau >= 0) src = kg + (size_t)tau * D + col;
                else if (kp) src = kp + (size_t)(W + tau) * D + col;
            }
            px[i] = src ? *reinterpret_cast<const u32x4*>(src) : zz;
        }
#pragma unroll
        for (int i = 0; i < NXL; ++i) {
            const int c = tid + NT * i;
            const int p = c / CPR, col = (c % CPR) * 8;
            const int tv = t0 - (W - 1) + p;  // value of pair p
            const T* src = nullptr;
            if (c < NXC && p < NP && tv < T_) {
                if (tv >= 0) src = vg + (size_t)tv * D + col;
                else if (vp) src = vp + (size_t)(W - 1 + tv) * D + col;
            }
            pv[i] = src ? *reinterpret_cast<const u32x4*>(src) : zz;
        }
        // c_p of the tile's pair slots and its gamma_last
        if (tid <= kEP) pc = recf[(size_t)j * RF + (tid < kEP ? 64 + tid : kC)];
    };
    auto colfrag = [&](int row0, int col0) __attribute__((always_inline)) {
        return E::load_tr(X + swz_off<D>(row0 + 4 * grp + (lr >> 2), col0 + 4 * (lr & 3)));
    };

    // Sacc[kb][r] = S[v][k], v = 16 wave + lr, k = 16 kb + 4 grp + r; group 0
    // starts from S0, the others from zero
    f32x4 Sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
        Sacc[kb] = (g == 0 && s0) ? *reinterpret_cast<const f32x4*>(s0 + (size_t)(16 * wave + lr) * D +
                                                                     16 * kb + 4 * grp)
                                  : zero4();
    float gp = 1.f;
    const Frag z = {0, 0, 0, 0};
    load(j0);
    for (int j = j0; j < j1; ++j) {
#pragma unroll
        for (int i = 0; i < NXL; ++i) {
            const int c = tid + NT * i;
            if (c < NXC) {
                *reinterpret_cast<u32x4*>(&X[swz_off<D>(c / CPR, (c % CPR) * 8)]) = px[i];
                *reinterpret_cast<u32x4*>(&V[c * 8]) = pv[i];
            }
        }
        if (tid <= kEP) cf[tid] = pc;
        lds_barrier();
        if (j + 1 < j1) load(j + 1);
        // delta of the wave's 16 columns: B fragments over the pair blocks
        Frag Db[kNPB];
#pragma unroll
        for (int pb = 0; pb < kNPB; ++pb) {
            const Frag vf = E::load_tr(V + (16 * pb + 4 * grp + (lr >> 2)) * D + 16 * wave + 4 * (lr & 3));
            const f32x4 c4 = *reinterpret_cast<const f32x4*>(&cf[16 * pb + 4 * grp]);
            f32x4 d;
#pragma unroll
            for (int r = 0; r < 4; ++r) d[r] = c4[r] * E::to_f((T)vf[r]);
            Db[pb] = E::pack(d);
        }
        const float glast = cf[kEP];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x4 acc = Sacc[kb] * glast;
            acc = E::mma32(colfrag(0, 16 * kb), colfrag(16, 16 * kb), Db[0], Db[1], acc);
            acc = E::mma32(colfrag(32, 16 * kb), z, Db[2], z, acc);
            Sacc[kb] = acc;
        }
        gp *= glast;
        lds_barrier();  // the next tile's staging overwrites the tiles
    }
    float* pg = part + ((size_t)bh * gmax + g) * D * D + (size_t)(16 * wave + lr) * D + 4 * grp;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) *reinterpret_cast<f32x4*>(pg + 16 * kb) = Sacc[kb];
    if (tid == 0) part[(size_t)a.BH * gmax * D * D + (size_t)bh * gmax + g] = gp;
}

// ---------------------------------------------------------------------------
// State pass: one workgroup per (segment, batch*head, SW-wide value slice),
// walking its tiles in order.  Chain wave c (c < SW / 16) carries 16 columns
// of the slice's state as MFMA accumulators of S^T and forms the products the
// next state needs (X S0^T, delta, the update); output wave c forms those
// columns' outputs of the tile from the state at the tile's start, which its
// chain wave hands over through LDS; the NF fill waves share the fill of
// every tile and issue its loads NF tiles ahead.  One LDS-only barrier per
// tile.  The delta rule runs one segment of 16-column slices; the
// inner-product rule with long chains kSegs segments of 64-column slices.
//
// Key and query tiles hold rows of D elements with no padding, chunks
// swizzled per row (swz_off).
// ---------------------------------------------------------------------------
template <int D, bool DELTA, int SW>
struct WinPassSmem {
    using R = WinRec<DELTA>;
    uint16_t X[2][kEP * D];    // pair keys (swizzled rows)
    uint16_t Q[2][kC * D];     // queries (swizzled rows)
    uint16_t V[2][kEP * SW];   // pair values of the slice's SW columns
    alignas(16) char rec[2][R::kBytes];
    s16x4 SB[2][SW / 16][D / 16][64];  // the state at a tile's start, B fragments of S^T, per chain wave
};

constexpr int kPassFill = 4;  // fill waves = tiles in flight

// SW value columns per workgroup (16 or 32): SW / 16 chain waves and as
// many output waves, each owning 16 columns, then the fill waves.  Wider
// slices share each key and query tile among more columns, so a compute unit
// moves fewer bytes per unit of work.
template <int D, bool DELTA, int SW>
__global__ __launch_bounds__(64 * (2 * (SW / 16) + kPassFill)) void win_pass_kernel(
    ChunkArgs a, const void* ws, int ntiles, int nseg, int gmax, const float* part) {
    using E = EBf16;
    using T = uint16_t;
    using Frag = s16x4;
    using R = WinRec<DELTA>;
    using Smem = WinPassSmem<D, DELTA, SW>;
    constexpr int KB = D / 16, NVS = D / SW, CPR = D / 8, NF = kPassFill, NCW = SW / 16;
    constexpr int RCH = (int)(R::kBytes / 16);  // 16-byte pieces of a record
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    // the segment (inner-product rule: nseg = 2 splits each chain in two)
    const int per = (int)gridDim.x / nseg;
    const int seg = (int)blockIdx.x / per;
    // slices of one sequence on one XCD (workgroup i runs on XCD i mod 8)
    const int blk = (int)blockIdx.x - seg * per, xcd = blk & 7, jj = blk >> 3;
    const int rr = (jj / NVS) * 8 + xcd, vs = jj % NVS;
    if (rr >= a.BH) return;
    const int bh = pass_bh(a, rr);
    const int v0 = vs * SW;
    // a chain or output wave's 16 columns start at vc
    const int cw = NCW == 1 ? 0 : (wave < NCW ? wave : wave - NCW);
    const int vc = v0 + 16 * cw;
    const int W = a.W;
    const int NP = kC + W - 1;
    const SeqRows sr = seq_rows(a, bh);
    const int T_ = sr.T;
    const int ntl = tiles_of(T_, kC);
    // this workgroup's tiles [tb0, tb1); the one that ends the chain writes
    // S_final (the delta rule always runs one segment)
    const bool first = DELTA || seg == 0;
    const int L = (!DELTA && nseg > 1) ? seg_len(ntl) : ntl;
    const int tb0 = first ? 0 : min(seg * L, ntl), tb1 = min(first ? L : seg * L + L, ntl);
    if (!first && tb0 >= tb1) return;  // an empty segment after the chain's end
    const bool ends = tb1 >= ntl;
    const T* qg = static_cast<const T*>(a.q) + sr.row0 * D;
    const T* kg = static_cast<const T*>(a.k) + sr.row0 * D;
    const T* vg = static_cast<const T*>(a.v) + sr.row0 * D + v0;
    const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
    const T* vp = (a.v_prev && W > 1)
                      ? static_cast<const T*>(a.v_prev) + (size_t)bh * (W - 1) * D + v0
                      : nullptr;
    const char* recg = static_cast<const char*>(ws) + (size_t)bh * ntiles * R::kBytes;

    // row fragment (8 bytes) of a swizzled tile: row r, columns c .. c + 3
    auto rowld = [&](const T* m, int r, int c) __attribute__((always_inline)) {
        return E::load(m + swz_off<D>(r, c));
    };
    // column fragment of a swizzled tile: lane (lr, grp) gets
    // M[row0 + 4 grp + r][col0 + lr], r = 0..3
    auto colfrag = [&](const T* m, int row0, int col0) __attribute__((always_inline)) {
        return E::load_tr(m + swz_off<D>(row0 + 4 * grp + (lr >> 2), col0 + 4 * (lr & 3)));
    };
    // the pair values: b(Y block kb) = a(Y^T block kb), rows of 16 elements
    auto vfrag = [&](const T* vb, int kb) __attribute__((always_inline)) {
        return E::load_tr(vb + (16 * kb + 4 * grp + (lr >> 2)) * SW + 16 * cw + 4 * (lr & 3));
    };

    if (wave < NCW) {
        // ---- the state chain ----
        // Sacc[kb][r] = S[v][k], v = vc + lr, k = 16 kb + 4 grp + r
        f32x4 Sacc[KB];
        Frag SB[KB];
        // the state at the tile start: S0, or with segments (whose
        // workgroups must not read S0, which S_final may alias) the copy of
        // S0 for the first segment and, for a later one, the state after
        // group 0 (from S0) carried through the groups before the segment in
        // order, S = gprod_g S + part_g
        const float* s0 = a.S0 ? a.S0 + (size_t)bh * D * D : nullptr;
        if (!DELTA && nseg > 1 && s0)
            s0 = part + seg_s0_offset(a.BH, gmax, D) + (size_t)bh * D * D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            Sacc[kb] = s0 ? *reinterpret_cast<const f32x4*>(s0 + (size_t)(vc + lr) * D + 16 * kb + 4 * grp)
                          : zero4();
        if constexpr (!DELTA) {
            if (seg > 0) {
                const int G = tb0 / kSegTiles;
                const float* pp = part + (size_t)bh * gmax * D * D + (size_t)(vc + lr) * D + 4 * grp;
                const float* gpr = part + (size_t)a.BH * gmax * D * D + (size_t)bh * gmax;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) Sacc[kb] = *reinterpret_cast<const f32x4*>(pp + 16 * kb);
                for (int gg = 1; gg < G; ++gg) {
                    const float f = gpr[gg];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        Sacc[kb] = Sacc[kb] * f + *reinterpret_cast<const f32x4*>(pp + (size_t)gg * D * D + 16 * kb);
                }
            }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            SB[kb] = E::pack(Sacc[kb]);
            sm.SB[0][cw][kb][lane] = SB[kb];
        }
        lds_barrier();
        for (int it = tb0; it < tb1; ++it) {
            const int b = (it - tb0) & 1;
            const T* Xb = sm.X[b];
            const char* rec = sm.rec[b];
            const Frag* FA = reinterpret_cast<const Frag*>(rec + R::kA);
            const float* FL = reinterpret_cast<const float*>(rec + R::kF);
            Frag Vf[kNPB], Db[kNPB];
#pragma unroll
            for (int kb = 0; kb < kNPB; ++kb) Vf[kb] = vfrag(sm.V[b], kb);
            if constexpr (DELTA) {
                // Z = X S0^T (pairs x the slice's columns)
                f32x4 Z[kNPB];
#pragma unroll
                for (int pb = 0; pb < kNPB; ++pb) Z[pb] = zero4();
#pragma unroll
                for (int m = 0; m < D / 32; ++m) {
#pragma unroll
                    for (int pb = 0; pb < kNPB; ++pb)
                        Z[pb] = E::mma32(rowld(Xb, 16 * pb + lr, 32 * m + 4 * grp),
                                         rowld(Xb, 16 * pb + lr, 32 * m + 16 + 4 * grp), SB[2 * m],
                                         SB[2 * m + 1], Z[pb]);
                }
                Frag Zb[kNPB];
#pragma unroll
                for (int pb = 0; pb < kNPB; ++pb) Zb[pb] = E::pack(Z[pb]);
                // delta = [N' | -N] [Y; Z]
#pragma unroll
                for (int pb = 0; pb < kNPB; ++pb) {
                    f32x4 acc = E::mma32(FA[R::fa(pb, 0) * 64 + lane], FA[R::fa(pb, 1) * 64 + lane],
                                         Vf[0], Vf[1], zero4());
                    acc = E::mma32(FA[R::fa(pb, 2) * 64 + lane], FA[R::fa(pb, 3) * 64 + lane], Vf[2],
                                   Zb[0], acc);
                    acc = E::mma32(FA[R::fa(pb, 4) * 64 + lane], FA[R::fa(pb, 5) * 64 + lane], Zb[1],
                                   Zb[2], acc);
                    Db[pb] = E::pack(acc);
                }
            } else {
                // delta_p = c_p y_p
#pragma unroll
                for (int pb = 0; pb < kNPB; ++pb) {
                    const f32x4 c4 = *reinterpret_cast<const f32x4*>(FL + 64 + 16 * pb + 4 * grp);
                    f32x4 d;
#pragma unroll
                    for (int r = 0; r < 4; ++r) d[r] = c4[r] * E::to_f((T)Vf[pb][r]);
                    Db[pb] = E::pack(d);
                }
            }
            // S^T = gamma_last S0^T + X^T delta, handed to the output wave
            const float glast = FL[kC];
            const Frag z = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x4 acc = Sacc[kb] * glast;
                acc = E::mma32(colfrag(Xb, 0, 16 * kb), colfrag(Xb, 16, 16 * kb), Db[0], Db[1], acc);
                acc = E::mma32(colfrag(Xb, 32, 16 * kb), z, Db[2], z, acc);
                Sacc[kb] = acc;
                SB[kb] = E::pack(acc);
                sm.SB[b ^ 1][cw][kb][lane] = SB[kb];
            }
            lds_barrier();
        }
        if (a.S_final && ends) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                *reinterpret_cast<f32x4*>(a.S_final + ((size_t)bh * D + vc + lr) * D + 16 * kb +
                                          4 * grp) = Sacc[kb];
        }
    } else if (wave < 2 * NCW) {
        // ---- the outputs: O^T = (S0 Q^T) diag(gamma) + Y^T L'^T - Z^T L^T;
        // lane ends with O[t = 16 tb + lr][v = vc + 4 grp + r] ----
        T* og = a.o ? static_cast<T*>(a.o) + sr.row0 * D + vc : nullptr;
        lds_barrier();
        for (int it = tb0; it < tb1; ++it) {
            const int b = (it - tb0) & 1, t0 = it * kC;
            const T* Xb = sm.X[b];
            const T* Qb = sm.Q[b];
            const char* rec = sm.rec[b];
            const Frag* FB = reinterpret_cast<const Frag*>(rec + R::kB);
            const float* FL = reinterpret_cast<const float*>(rec + R::kF);
            Frag SB[KB], Vf[kNPB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) SB[kb] = sm.SB[b][cw][kb][lane];
#pragma unroll
            for (int kb = 0; kb < kNPB; ++kb) Vf[kb] = vfrag(sm.V[b], kb);
            Frag Zb[kNPB];
            if constexpr (DELTA) {
                f32x4 Z[kNPB];
#pragma unroll
                for (int pb = 0; pb < kNPB; ++pb) Z[pb] = zero4();
#pragma unroll
                for (int m = 0; m < D / 32; ++m) {
#pragma unroll
                    for (int pb = 0; pb < kNPB; ++pb)
                        Z[pb] = E::mma32(rowld(Xb, 16 * pb + lr, 32 * m + 4 * grp),
                                         rowld(Xb, 16 * pb + lr, 32 * m + 16 + 4 * grp), SB[2 * m],
                                         SB[2 * m + 1], Z[pb]);
                }
#pragma unroll
                for (int pb = 0; pb < kNPB; ++pb) Zb[pb] = E::pack(Z[pb]);
            }
            const Frag z = {0, 0, 0, 0};
#pragma unroll
            for (int tb = 0; tb < kNTB; ++tb) {
                f32x4 acc = zero4();
#pragma unroll
                for (int m = 0; m < D / 32; ++m)
                    acc = E::mma32(SB[2 * m], SB[2 * m + 1], rowld(Qb, 16 * tb + lr, 32 * m + 4 * grp),
                                   rowld(Qb, 16 * tb + lr, 32 * m + 16 + 4 * grp), acc);
                acc = acc * FL[16 * tb + lr];
                if constexpr (DELTA) {
                    acc = E::mma32(Vf[0], Vf[1], FB[R::fb(tb, 0) * 64 + lane],
                                   FB[R::fb(tb, 1) * 64 + lane], acc);
                    acc = E::mma32(Vf[2], Zb[0], FB[R::fb(tb, 2) * 64 + lane],
                                   FB[R::fb(tb, 3) * 64 + lane], acc);
                    acc = E::mma32(Zb[1], Zb[2], FB[R::fb(tb, 4) * 64 + lane],
                                   FB[R::fb(tb, 5) * 64 + lane], acc);
                } else {
                    acc = E::mma32(Vf[0], Vf[1], FB[R::fb(tb, 0) * 64 + lane],
                                   FB[R::fb(tb, 1) * 64 + lane], acc);
                    acc = E::mma32(Vf[2], z, FB[R::fb(tb, 2) * 64 + lane], z, acc);
                }
                const int t = 16 * tb + lr;
                if (og && t0 + t < T_)
                    *reinterpret_cast<Frag*>(og + (size_t)(t0 + t) * D + 4 * grp) = E::pack(acc);
            }
            lds_barrier();
        }
    } else {
        // ---- fill waves: every tile is split over the NF waves (lane l of
        // wave f takes the 16-byte pieces (64 f + l) + 256 i); each lane keeps
        // the pieces of the next NF tiles in registers, slot = tile mod NF ----
        const int fl = 64 * (wave - 2 * NCW) + lane;
        constexpr int VPR = SW / 8;  // 16-byte pieces of a pair value row
        constexpr int NXC = kEP * CPR, NQC = kC * CPR, NVC = kEP * VPR;
        constexpr int NXL = (NXC + 255) / 256, NQL = (NQC + 255) / 256, NVL = (NVC + 255) / 256,
                      NRL = (RCH + 255) / 256;
        u32x4 px[NF][NXL], pq[NF][NQL], pv[NF][NVL], pr[NF][NRL];
        const rsrc_t kr = make_rsrc(kg, (int64_t)T_ * D * 2);
        const rsrc_t qr = make_rsrc(qg, (int64_t)T_ * D * 2);
        const rsrc_t vr = make_rsrc(vg, (int64_t)T_ * D * 2 - (int64_t)v0 * 2);
        const rsrc_t rr_ = make_rsrc(recg, (int64_t)ntiles * R::kBytes);
        // tile 0 may reach into the halo rows before the sequence
        auto issue0 = [&](auto& x, auto& q, auto& v, auto& r) __attribute__((always_inline)) {
            const u32x4 zz = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < NXL; ++i) {
                const int c = fl + 256 * i;
                const int p = c / CPR, col = (c % CPR) * 8;
                const int tau = p - (W - 1) - a.lag;  // key of pair p
                const T* src = nullptr;
                if (c < NXC && p < NP && tau < T_) {
                    if (tau >= 0) src = kg + (size_t)tau * D + col;
                    else if (kp) src = kp + (size_t)(W + tau) * D + col;
                }
                x[i] = src ? *reinterpret_cast<const u32x4*>(src) : zz;
            }
#pragma unroll
            for (int i = 0; i < NVL; ++i) {
                const int c = fl + 256 * i;
                const int p = c / VPR, col = (c % VPR) * 8;
                const int tv = p - (W - 1);  // value of pair p
                const T* src = nullptr;
                if (c < NVC && p < NP && tv < T_) {
                    if (tv >= 0) src = vg + (size_t)tv * D + col;
                    else if (vp) src = vp + (size_t)(W - 1 + tv) * D + col;
                }
                v[i] = src ? *reinterpret_cast<const u32x4*>(src) : zz;
            }
#pragma unroll
            for (int i = 0; i < NQL; ++i) {
                const int c = fl + 256 * i;
                q[i] = buf_load16(qr, c < NQC ? (uint32_t)(c * 16) : kOob);
            }
#pragma unroll
            for (int i = 0; i < NRL; ++i) {
                const int c = fl + 256 * i;
                r[i] = buf_load16(rr_, c < RCH ? (uint32_t)(c * 16) : kOob);
            }
        };
        // tiles >= 1 read rows of the sequence only (tile * C - (W - 1) - lag
        // >= 0 for W <= 8); rows at or past the end read as zeros
        auto issue = [&](int tile, auto& x, auto& q, auto& v, auto& r) __attribute__((always_inline)) {
            const int t0 = tile * kC;
#pragma unroll
            for (int i = 0; i < NXL; ++i) {
                const int c = fl + 256 * i;
                const int p = c / CPR, col = (c % CPR) * 8;
                const int tau = t0 - (W - 1) - a.lag + p;
                x[i] = buf_load16(kr, (c < NXC && p < NP) ? (uint32_t)((tau * D + col) * 2) : kOob);
            }
#pragma unroll
            for (int i = 0; i < NVL; ++i) {
                const int c = fl + 256 * i;
                const int p = c / VPR, col = (c % VPR) * 8;
                const int tv = t0 - (W - 1) + p;
                v[i] = buf_load16(vr, (c < NVC && p < NP && tv < T_) ? (uint32_t)((tv * D + col) * 2)
                                                                    : kOob);
            }
#pragma unroll
            for (int i = 0; i < NQL; ++i) {
                const int c = fl + 256 * i;
                q[i] = buf_load16(qr, c < NQC ? (uint32_t)((t0 * D + c * 8) * 2) : kOob);
            }
#pragma unroll
            for (int i = 0; i < NRL; ++i) {
                const int c = fl + 256 * i;
                r[i] = buf_load16(rr_, c < RCH ? (uint32_t)(tile * R::kBytes + c * 16) : kOob);
            }
        };
        auto store = [&](int rel, const auto& x, const auto& q, const auto& v, const auto& r)
            __attribute__((always_inline)) {
            const int b = rel & 1;
#pragma unroll
            for (int i = 0; i < NXL; ++i) {
                const int c = fl + 256 * i;
                if (c < NXC)
                    *reinterpret_cast<u32x4*>(&sm.X[b][swz_off<D>(c / CPR, (c % CPR) * 8)]) = x[i];
            }
#pragma unroll
            for (int i = 0; i < NVL; ++i) {
                const int c = fl + 256 * i;
                if (c < NVC) *reinterpret_cast<u32x4*>(&sm.V[b][c * 8]) = v[i];
            }
#pragma unroll
            for (int i = 0; i < NQL; ++i) {
                const int c = fl + 256 * i;
                if (c < NQC)
                    *reinterpret_cast<u32x4*>(&sm.Q[b][swz_off<D>(c / CPR, (c % CPR) * 8)]) = q[i];
            }
#pragma unroll
            for (int i = 0; i < NRL; ++i) {
                const int c = fl + 256 * i;
                if (c < RCH) reinterpret_cast<u32x4*>(sm.rec[b])[c] = r[i];
            }
        };
        // The segment's tiles by index i relative to tb0 (n of them): tiles
        // 0 .. NF - 1 in flight; tile 0 is published before the first barrier
        // and tile NF takes its slot.  At step i tile i + 1 moves from slot
        // (i + 1) mod NF into LDS and tile i + 1 + NF is issued into the slot.
        // The barriers order LDS only, so the loads stay in flight across
        // them.  Only the chain's first tile (tb0 = 0) reaches the halo.
        const int n = tb1 - tb0;
        if (n > 0) {
            if (tb0 == 0) issue0(px[0], pq[0], pv[0], pr[0]);
            else issue(tb0, px[0], pq[0], pv[0], pr[0]);
        }
        static_for<NF - 1>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value + 1;
            if (j < n) issue(tb0 + j, px[j], pq[j], pv[j], pr[j]);
        });
        if (n > 0) {
            store(0, px[0], pq[0], pv[0], pr[0]);
            if (NF < n) issue(tb0 + NF, px[0], pq[0], pv[0], pr[0]);
        }
        lds_barrier();
        for (int base = 0; base < n; base += NF) {
            static_for<NF>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value, slot = (j + 1) % NF;
                const int i = base + j;
                if (i < n) {
                    const int ni = i + 1;
                    if (ni < n) {
                        store(ni, px[slot], pq[slot], pv[slot], pr[slot]);
                        if (ni + NF < n) issue(tb0 + ni + NF, px[slot], pq[slot], pv[slot], pr[slot]);
                    }
                    lds_barrier();
                }
            });
        }
    }
}

template <int D, int W, bool DELTA>
hipError_t launch_prep(const ChunkArgs& b, void* ws, int ntiles, hipStream_t stream) {
    using Smem = WinPrepSmem<D, W, DELTA>;
    constexpr int per_cu_lds = (int)(163840 / sizeof(Smem));
    int per_cu = per_cu_lds < 1 ? 1 : (per_cu_lds > 4 ? 4 : per_cu_lds);
    // a persistent grid must be resident at once: no more workgroups per CU
    // than the kernel's registers allow (the larger windows fit one)
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, win_prep_kernel<D, W, DELTA>, 256, 0) == hipSuccess &&
        occ >= 1 && occ < per_cu)
        per_cu = occ;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    const int njobs = b.BH * ntiles;
    const int grid = njobs < cus * per_cu ? njobs : cus * per_cu;
    hipLaunchKernelGGL((win_prep_kernel<D, W, DELTA>), dim3(grid), dim3(256), 0, stream, b, ws,
                       ntiles, njobs);
    return hipGetLastError();
}

template <int D, bool DELTA>
hipError_t launch_prep_w(const ChunkArgs& b, void* ws, int ntiles, hipStream_t stream) {
    switch (b.W) {
        case 2: return launch_prep<D, 2, DELTA>(b, ws, ntiles, stream);
        case 3: return launch_prep<D, 3, DELTA>(b, ws, ntiles, stream);
        case 4: return launch_prep<D, 4, DELTA>(b, ws, ntiles, stream);
        case 5: return launch_prep<D, 5, DELTA>(b, ws, ntiles, stream);
        case 6: return launch_prep<D, 6, DELTA>(b, ws, ntiles, stream);
        case 7: return launch_prep<D, 7, DELTA>(b, ws, ntiles, stream);
        case 8: return launch_prep<D, 8, DELTA>(b, ws, ntiles, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D, bool DELTA>
hipError_t launch_d(const ChunkArgs& a, void* ws, hipStream_t stream) {
    const int ntiles = tiles_of(a.T, kC);
    ChunkArgs b = a;
    b.order = nullptr;
    b.toff = nullptr;
    b.jobs = nullptr;
    hipError_t e = launch_packed_schedule(a, kC, ntiles, b, stream);
    if (e != hipSuccess) return e;
    if (ntiles > 0) {
        e = launch_prep_w<D, DELTA>(b, ws, ntiles, stream);
        if (e != hipSuccess) return e;
    }
    // inner-product rule, long chains: the group states before the last segment
    const int nseg = (!DELTA && ntiles >= kSegMinTiles) ? kSegs : 1;
    const int gmax = nseg > 1 ? seg_groups(ntiles) : 0;
    float* part = nullptr;
    if (nseg > 1) {
        part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        window_records_bytes(b.BH, ntiles, DELTA));
        hipLaunchKernelGGL((win_seg_kernel<D>), dim3(gmax * b.BH), dim3(4 * D), 0, stream, b,
                           (const void*)ws, ntiles, gmax, part);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int bh8 = (b.BH + 7) / 8 * 8;
    if (nseg > 1) {
        // kSegs segments of 64-column slices: as many workgroups as 16-column
        // slices of one segment would be
        if constexpr (!DELTA)
            hipLaunchKernelGGL((win_pass_kernel<D, DELTA, 64>), dim3(nseg * bh8 * (D / 64)),
                               dim3(64 * (2 * 4 + kPassFill)), 0, stream, b, (const void*)ws, ntiles, nseg,
                               gmax, (const float*)part);
    } else {
        hipLaunchKernelGGL((win_pass_kernel<D, DELTA, 16>), dim3(bh8 * (D / 16)),
                           dim3(64 * (2 + kPassFill)), 0, stream, b, (const void*)ws, ntiles, 1, 0,
                           (const float*)nullptr);
    }
    return hipGetLastError();
}

}  // namespace

size_t window_workspace_bytes(int BH, int T, bool delta, int D) {
    const int nt = tiles_of(T, kC);
    size_t bytes = window_records_bytes(BH, nt, delta);
    // the segmented pass's group states [BH][gmax][D][D] fp32, the products
    // of their gates [BH][gmax] fp32 and the copy of S0 [BH][D][D] fp32
    if (!delta && nt >= kSegMinTiles) {
        bytes += (seg_s0_offset(BH, seg_groups(nt), D) + (size_t)BH * D * D) * 4;
    }
    return bytes;
}

hipError_t launch_window(const ChunkArgs& a, int D, bool delta, void* ws, hipStream_t stream) {
    if (a.W < 2 || a.W > 8) return hipErrorInvalidValue;
    if (D == 64) return delta ? launch_d<64, true>(a, ws, stream) : launch_d<64, false>(a, ws, stream);
    if (D == 128) return delta ? launch_d<128, true>(a, ws, stream) : launch_d<128, false>(a, ws, stream);
    return hipErrorInvalidValue;
}

}  // namespace falcon
