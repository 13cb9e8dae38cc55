// falcon_fused.hip -- the inner-product rules (Falcon-1A, and Falcon-2A with
// its per-column write vectors) at bf16 with 64-step tiles, intra-chunk work
// and state pass in one kernel: keys and queries come from HBM once, and no
// per-tile record or write vector makes a round trip through it.
//
// Method ("Fast Weight Attention for Continual Learning", authors' abstract;
// decay-then-write order and the normalized step from the KLA abstract on the
// same listing): per (batch, head) the state S (d_v x d_k) is decayed by
// alpha_t, receives the write y_t u_t^T with x_t = k_{t-lag} and
// u_t = eta_t x_t / (||x_t||^2 + eps) (Falcon-2A: u_tj = eta_t x_tj /
// (|x_tj| ||x_t||_1 + eps), the per-column normalization read as a diagonal
// normalizer), and is read after the write,
// o_t = S_t q_t.  Per 64-step tile, with S0 the state at the tile start, g the
// tile-local cumulative log decay and D(t, s) = exp(g_t - g_s):
//   P[t][j] = [j <= t] D(t, j) (q_t . u_j),
//   O = diag(exp g) Q S0^T + P Y,
//   S = exp(g_last) S0 + Y^T diag(exp(g_last - g)) U.
//
// One workgroup of 12 waves per (batch*head, 64-wide value slice) walks the
// tiles in order; at iteration it
//   waves 0-3  (chain)  tile it, 16 value columns each, the state held as
//                       MFMA accumulators of S^T: the outputs of the wave's
//                       columns for all 64 steps (Q S0^T from the state at
//                       the tile start, plus P Y) and the update's right-hand
//                       side | barrier 1 | the state update;
//   waves 4-7  (intra-chunk, rows of block c of tile it+1) the norms from
//                       the diagonal Gram block, the decay scan, the row
//                       scales and decay factors | barrier 1;
//   waves 8-11 (P, block row w of tile it+1) direct-to-LDS fills (keys,
//                       queries and gates of tile it+2, targets of tile it+1),
//                       the raw products q_t . x_j of the block row | barrier
//                       1 | their causal decay factors from the row scales
//                       of barrier 1, written as B fragments, then the wait
//                       for the fills;
//   barrier 2.
// The chain needs nothing produced within its own iteration, so one
// iteration's intra-chunk work overlaps the state chain of the one before.
// Keys and queries of a tile are used in three iterations (in flight, the
// intra-chunk work, the chain), so they have three LDS buffers; targets,
// gates and the intra-chunk results two.  The per-column rule keeps the keys
// one stage longer (four; fills three tiles ahead): in the half-iteration
// after barrier 1, where the scalar rule's intra-chunk waves are idle, they
// turn tile it+2's keys into x / (|x| ||x||_1 + eps) in place (tiles 0 and 1
// at the prologue's fill, in registers), so the P waves and the chain read
// write vectors, and eta_t becomes the row scale.  Every decay factor is
// exp(later - earlier) <= 1 of a log sum that restarts at each tile.  LDS
// tiles are unpadded with swizzled chunks (swz_off), filled by lanes whose
// source offsets apply the swizzle.
#include <stddef.h>

#include "falcon_device.h"
#include "falcon_internal.h"
#include "falcon_records.h"
#include "falcon_rows.h"

namespace falcon {

namespace {

constexpr int kF = 64;    // steps per tile
constexpr int kFB = 4;    // 16-row blocks per tile
constexpr float kL2e = 1.4426950408889634f;

// per-row factors of a tile
enum : int { kGam = 0, kHrow = 1, kG2 = 2, kRs = 3, kCf = 4, kNFac = 5 };

template <int D, bool COL>
struct FusedSmem {
    // key stages: the per-column rule fills keys one tile further ahead, so
    // that a tile's keys become its write vectors before the P waves read them
    static constexpr int kXS = COL ? 4 : 3;
    uint16_t X[kXS][kF * D];           // keys x_i = k_{t0+i-lag}; per-column rule: x_i / (|x_i| ||x_i||_1 + eps)
    uint16_t Q[3][kF * D];             // queries
    uint16_t Y[2][kF * 64];            // targets, this slice's 64 value columns
    s16x4 Pf[2][kFB][kFB][64];         // P blocks (tb, cb <= tb), B fragments of P^T
    float fac[2][kNFac][kF];           // exp g, exp(g_last - g) r, log2(e) g, r, cf
    float gref[2][kFB];                // log2(e) g at the last row of each block
    float gates[2][2][kF];             // alpha, eta as loaded
    float nrm[kFB][16];                // ||x_i||^2 of each intra-chunk wave's rows
    float pl[kFB][kF];                 // each intra-chunk wave's log-decay scan
    float pe[kFB][kF];                 // and the gates eta, steps past the end 0
};

template <int D, bool COL>
__global__ __launch_bounds__(768) void fused_kernel(ChunkArgs a) {
    using E = EBf16;
    using T = uint16_t;
    using Frag = s16x4;
    using Smem = FusedSmem<D, COL>;
    constexpr int XS = Smem::kXS;       // key stages
    constexpr int XD = XS - 1;          // tiles ahead the key fills run
    constexpr int NB = kFB, KB = D / 16, CPR = D / 8, NVS = D / 64;
    // direct-to-LDS fills: 1 KB per instruction, RPI rows of a D-wide tile
    constexpr int RPI = 1024 / (2 * D), NIX = kF / RPI, MIX = NIX / 4, MIY = 2;
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    const int role = wave >> 2;  // 0 chain, 1 intra-chunk columns, 2 P rows and fills
    const int cw = wave & 3;
    // slices of one sequence on one XCD (workgroup i runs on XCD i mod 8)
    const int blk = blockIdx.x, xcd = blk & 7, jj = blk >> 3;
    const int rr = (jj / NVS) * 8 + xcd, vs = jj % NVS;
    if (rr >= a.BH) return;
    const int bh = pass_bh(a, rr);
    const int v0 = vs * 64;
    const SeqRows sr = seq_rows(a, bh);
    const int T_ = sr.T;
    const int ntl = tiles_of(T_, kF);
    const int lag = a.lag;
    const float eps = a.eps;
    const T* qg = static_cast<const T*>(a.q) + sr.row0 * D;
    const T* kg = static_cast<const T*>(a.k) + sr.row0 * D;
    const T* vg = static_cast<const T*>(a.v) + sr.row0 * D + v0;
    const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * D : nullptr;
    const float* alg = a.alpha + sr.row0;
    const float* etg = a.eta + sr.row0;
    T* og = a.o ? static_cast<T*>(a.o) + sr.row0 * D + v0 : nullptr;

    // 4 (8) consecutive elements of row r from column c of a D-wide tile
    auto xrow = [&](const T* m, int r, int c) __attribute__((always_inline)) {
        return E::load(m + swz_off<D>(r, c));
    };
    auto xrow8 = [&](const T* m, int r, int c) __attribute__((always_inline)) {
        return E::load8(m + swz_off<D>(r, c));
    };
    // column fragments: lane (lr, grp) gets M[row0 + 4 grp + r][col0 + lr]
    auto xcol = [&](const T* m, int row0, int col0) __attribute__((always_inline)) {
        return E::load_tr(m + swz_off<D>(row0 + 4 * grp + (lr >> 2), col0 + 4 * (lr & 3)));
    };
    auto ycol = [&](const T* m, int row0, int col0) __attribute__((always_inline)) {
        return E::load_tr(m + swz_off<64>(row0 + 4 * grp + (lr >> 2), col0 + 4 * (lr & 3)));
    };

    // ---- prologue fills (P waves, through registers, halo included): keys,
    // queries and gates of tiles 0 and 1, targets of tile 0 ----
    if (role == 2) {
        const int ft = tid - 512;
        constexpr int NXP = (2 * kF * CPR) / 256, NQP = NXP, NYP = (kF * 8) / 256;
        u32x4 px[NXP], pq[NQP], py[NYP];
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int it = 0; it < NXP; ++it) {
            const int c = ft + 256 * it;
            const int i = c / CPR, col = (c % CPR) * 8;  // i: row of tiles 0-1
            const int tau = i - lag;
            const T* src = nullptr;
            if (i < kF * (ntl < 2 ? ntl : 2) && tau < T_) {
                if (tau >= 0) src = kg + (size_t)tau * D + col;
                else if (kp) src = kp + col;
            }
            px[it] = src ? *reinterpret_cast<const u32x4*>(src) : z;
        }
        if constexpr (COL) {
            // per-column rule: the write vectors without their step size,
            // u_i / eta_i = x_i / (|x_i| ||x_i||_1 + eps); the CPR lanes of a
            // row are consecutive and aligned, so the norm is a group sum
#pragma unroll
            for (int it = 0; it < NXP; ++it) {
                const uint16_t* h = reinterpret_cast<const uint16_t*>(&px[it]);
                float s1 = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) s1 += fabsf(bf2f(h[e]));
                s1 = group_sum_dpp<CPR>(s1);
                px[it] = col_write8(px[it], s1, 1.f, eps);
            }
        }
#pragma unroll
        for (int it = 0; it < NQP; ++it) {
            const int c = ft + 256 * it;
            const int i = c / CPR, col = (c % CPR) * 8;
            pq[it] = (i < kF * (ntl < 2 ? ntl : 2) && i < T_)
                         ? *reinterpret_cast<const u32x4*>(qg + (size_t)i * D + col)
                         : z;
        }
#pragma unroll
        for (int it = 0; it < NYP; ++it) {
            const int c = ft + 256 * it;
            const int i = c / 8, col = (c % 8) * 8;
            py[it] = (i < T_) ? *reinterpret_cast<const u32x4*>(vg + (size_t)i * D + col) : z;
        }
        const int gi = ft & 63, gt = (ft >> 6) & 1, gk = ft >> 7;  // step, tile, alpha / eta
        const int gs = gt * kF + gi;
        const float gv = gs < T_ ? (gk ? etg[gs] : alg[gs]) : 0.f;
#pragma unroll
        for (int it = 0; it < NXP; ++it) {
            const int c = ft + 256 * it;
            const int i = c / CPR, col = (c % CPR) * 8;
            *reinterpret_cast<u32x4*>(&sm.X[i / kF][swz_off<D>(i % kF, col)]) = px[it];
        }
#pragma unroll
        for (int it = 0; it < NQP; ++it) {
            const int c = ft + 256 * it;
            const int i = c / CPR, col = (c % CPR) * 8;
            *reinterpret_cast<u32x4*>(&sm.Q[i / kF][swz_off<D>(i % kF, col)]) = pq[it];
        }
#pragma unroll
        for (int it = 0; it < NYP; ++it) {
            const int c = ft + 256 * it;
            *reinterpret_cast<u32x4*>(&sm.Y[0][swz_off<64>(c / 8, (c % 8) * 8)]) = py[it];
        }
        sm.gates[gt][gk][gi] = gv;
    }

    // ---- intra-chunk work of tile tt (waves 4-7; wave c takes the rows of
    // block c): norms, decay scan, row scales and decay factors ----
    const int c = cw;
    auto prep1 = [&](int tt) __attribute__((always_inline)) {
        const int t0 = tt * kF, pb = tt & 1;
        const T* xt = sm.X[tt % XS];
        // diagonal Gram block: dg[r] = x_{16c+4grp+r} . x_{16c+lr} (the
        // scalar rule's norms; the per-column rule's keys are already its
        // write vectors)
        f32x4 dg = zero4();
        if constexpr (!COL) {
            s16x8 xc[D / 32];
#pragma unroll
            for (int m = 0; m < D / 32; ++m) xc[m] = xrow8(xt, 16 * c + lr, 32 * m + 8 * grp);
#pragma unroll
            for (int m = 0; m < D / 32; ++m) dg = E::mma32r(xc[m], xc[m], dg);
        }
        const bool valid = t0 + lane < T_;
        const float al = valid ? sm.gates[pb][0][lane] : 1.f;  // steps past the end: identity
        const float et = valid ? sm.gates[pb][1][lane] : 0.f;
        const float lg = wave_scan_dpp(__logf(al));
        const float glast = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lg), kF - 1));
        // the per-step values every lane looks up, through the wave's own LDS rows
        sm.pl[c][lane] = lg;
        sm.pe[c][lane] = et;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (lr == 4 * grp + r) sm.nrm[c][lr] = dg[r];
        __builtin_amdgcn_wave_barrier();
        // row 16 c + lr of this lane, and this block's columns j = 16 c + 4 grp + r
        const float lgr = sm.pl[c][16 * c + lr], etr = sm.pe[c][16 * c + lr];
        const float n2r = sm.nrm[c][lr];
        const float gref = sm.pl[c][16 * c + 15] * kL2e;
        const float denr = n2r + eps;
        // row scale of the write vector: eta / (||x||^2 + eps), or eta for the
        // per-column rule (eta 0 past the end)
        const float rsc = COL ? etr : (denr > 0.f ? etr / denr : 0.f);
        const float g2r = lgr * kL2e;
        if (lane < 16) {
            sm.fac[pb][kGam][16 * c + lr] = __expf(lgr);
            sm.fac[pb][kHrow][16 * c + lr] = __expf(glast - lgr) * rsc;
            sm.fac[pb][kG2][16 * c + lr] = g2r;
            sm.fac[pb][kRs][16 * c + lr] = rsc;
            sm.fac[pb][kCf][16 * c + lr] = exp2f(gref - g2r) * rsc;
        }
        if (lane == 0) sm.gref[pb][c] = gref;
    };
    // per-column rule: the keys of tile tt become x_i / (|x_i| ||x_i||_1 +
    // eps) in place; wave c takes rows 16 c .. 16 c + 15, four lanes a row
    auto to_write = [&](int tt) __attribute__((always_inline)) {
        T* xt = sm.X[tt % XS];
        constexpr int NCH = D / 32;  // 8-column chunks per lane
        const int row = 16 * c + (lane >> 2), q4 = lane & 3;
        u32x4 v[NCH];
        float s1 = 0.f;
#pragma unroll
        for (int m = 0; m < NCH; ++m) {
            v[m] = *reinterpret_cast<const u32x4*>(xt + swz_off<D>(row, 8 * (q4 * NCH + m)));
            const uint16_t* h = reinterpret_cast<const uint16_t*>(&v[m]);
#pragma unroll
            for (int e = 0; e < 8; ++e) s1 += fabsf(bf2f(h[e]));
        }
        s1 = group_sum_dpp<4>(s1);
#pragma unroll
        for (int m = 0; m < NCH; ++m)
            *reinterpret_cast<u32x4*>(xt + swz_off<D>(row, 8 * (q4 * NCH + m))) =
                col_write8(v[m], s1, 1.f, eps);
    };

    // ---- direct-to-LDS fills of the main loop (P waves).  Lane l of fill
    // instruction i of a D-wide tile writes row RPI i + l / CPR, stored chunk
    // l % CPR, which holds the row's chunk (l % CPR) ^ swz_row(row); the
    // 64-wide target tile likewise with 8 rows per instruction ----
    uint32_t dxo[MIX], dyo[MIY];
#pragma unroll
    for (int m = 0; m < MIX; ++m) {
        const int i = cw + 4 * m;
        const int row = RPI * i + lane / CPR, jp = lane % CPR;
        dxo[m] = (uint32_t)((row * D + 8 * (jp ^ swz_row<D>(row))) * 2);
    }
#pragma unroll
    for (int m = 0; m < MIY; ++m) {
        const int i = cw + 4 * m;
        const int row = 8 * i + lane / 8, jp = lane % 8;
        dyo[m] = (uint32_t)((row * D + 8 * (jp ^ swz_row<64>(row))) * 2);
    }
    const uint32_t sm_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) Smem*)&sm;
    // keys of tile tt (t0 >= 2 * 64: no halo) into X[tt % XS]; queries and
    // gates into Q[tt % 3], gates[tt & 1]; rows past the sequence read as zeros
    auto dma_x = [&](int tt) __attribute__((always_inline)) {
        const int t0 = tt * kF;
        const u32x4 rx = make_desc(kg + (size_t)(t0 - lag) * D, (int64_t)(T_ - t0 + lag) * D * 2);
        const uint32_t xb = sm_lds + (uint32_t)(offsetof(Smem, X) + sizeof(sm.X[0]) * (tt % XS));
#pragma unroll
        for (int m = 0; m < MIX; ++m) buf_load16_lds(rx, xb + 1024 * (cw + 4 * m), dxo[m]);
    };
    auto dma_qg = [&](int tt) __attribute__((always_inline)) {
        const int t0 = tt * kF;
        const u32x4 rq = make_desc(qg + (size_t)t0 * D, (int64_t)(T_ - t0) * D * 2);
        const uint32_t qb = sm_lds + (uint32_t)(offsetof(Smem, Q) + sizeof(sm.Q[0]) * (tt % 3));
#pragma unroll
        for (int m = 0; m < MIX; ++m) buf_load16_lds(rq, qb + 1024 * (cw + 4 * m), dxo[m]);
        if (cw < 2) {
            const u32x4 rg = make_desc((cw ? etg : alg) + t0, (int64_t)(T_ - t0) * 4);
            const uint32_t gb = sm_lds + (uint32_t)(offsetof(Smem, gates) + sizeof(sm.gates[0]) * (tt & 1) +
                                                    sizeof(sm.gates[0][0]) * cw);
            buf_load4_lds(rg, gb, (uint32_t)lane * 4);
        }
    };
    // targets of tile tt into Y[tt & 1]
    auto dma_y = [&](int tt) __attribute__((always_inline)) {
        const int t0 = tt * kF;
        const u32x4 ry = make_desc(vg + (size_t)t0 * D, (int64_t)(T_ - t0) * D * 2 - (int64_t)v0 * 2);
        const uint32_t yb = sm_lds + (uint32_t)(offsetof(Smem, Y) + sizeof(sm.Y[0]) * (tt & 1));
#pragma unroll
        for (int m = 0; m < MIY; ++m) buf_load16_lds(ry, yb + 1024 * (cw + 4 * m), dyo[m]);
    };

    // ---- P block row w of tile tt (waves 8-11): the raw products before
    // barrier 1, the decay factors after; lane holds P[t = 16 w + lr][16 cb +
    // 4 grp + r], the B fragment of block (cb, w) of P^T ----
    const int w = cw;
    auto prow1 = [&](int tt, f32x4 (&acc)[NB]) __attribute__((always_inline)) {
        const T* Xb = sm.X[tt % XS];
        const T* Qb = sm.Q[tt % 3];
        s16x8 qq[D / 32];
#pragma unroll
        for (int m = 0; m < D / 32; ++m) qq[m] = xrow8(Qb, 16 * w + lr, 32 * m + 8 * grp);
        with_const4(w, [&](auto wc) __attribute__((always_inline)) {
            constexpr int W = decltype(wc)::value;
            // the blocks cb <= W interleaved, m outer, so that consecutive
            // products accumulate into different blocks
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) acc[cb] = zero4();
#pragma unroll
            for (int m = 0; m < D / 32; ++m)
                static_for<W + 1>([&](auto cbc) __attribute__((always_inline)) {
                    constexpr int cb = decltype(cbc)::value;
                    acc[cb] = E::mma32r(xrow8(Xb, 16 * cb + lr, 32 * m + 8 * grp), qq[m], acc[cb]);
                });
        });
    };
    auto prow2 = [&](int tt, const f32x4 (&acc)[NB]) __attribute__((always_inline)) {
        const int pb = tt & 1;
        const float* g2 = sm.fac[pb][kG2];
        const float* rs = sm.fac[pb][kRs];
        const float* cf = sm.fac[pb][kCf];
        const int t = 16 * w + lr;
        const float g2t = g2[t];
        with_const4(w, [&](auto wc) __attribute__((always_inline)) {
            constexpr int W = decltype(wc)::value;
            static_for<W + 1>([&](auto cbc) __attribute__((always_inline)) {
                constexpr int cb = decltype(cbc)::value;
                const int j0 = 16 * cb + 4 * grp;
                f32x4 v;
                if constexpr (cb < W) {
                    const float rf = exp2f(g2t - sm.gref[pb][cb]);
                    const f32x4 cfv = *reinterpret_cast<const f32x4*>(cf + j0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = rf * cfv[r] * acc[cb][r];
                } else {
                    const f32x4 gj = *reinterpret_cast<const f32x4*>(g2 + j0);
                    const f32x4 rj = *reinterpret_cast<const f32x4*>(rs + j0);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = (j0 + r <= t) ? exp2f(g2t - gj[r]) * rj[r] * acc[cb][r] : 0.f;
                }
                sm.Pf[pb][w][cb][lane] = E::pack(v);
            });
        });
    };

    // the outputs of the wave's 16 columns, O^T = (S0 Q^T) diag(gamma)
    // + Delta^T P^T; lane ends with O[t = 16 tb + lr][v = v0 + 16 cw + 4 grp + r].
    // The four row blocks accumulate side by side (consecutive products go to
    // different blocks) and are stored at the end, rows past the sequence
    // masked by an out-of-range offset rather than a branch.
    auto outputs = [&](int it, const Frag (&SB)[KB], const Frag (&DB)[NB])
        __attribute__((always_inline)) {
        const int b2 = it & 1, t0 = it * kF;
        const T* Qb = sm.Q[it % 3];
        const float* gam = sm.fac[b2][kGam];
        const Frag zf = {0, 0, 0, 0};
        f32x4 acc[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) acc[tb] = zero4();
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
#pragma unroll
            for (int tb = 0; tb < NB; ++tb)
                acc[tb] = E::mma32(SB[2 * m], SB[2 * m + 1], xrow(Qb, 16 * tb + lr, 32 * m + 4 * grp),
                                   xrow(Qb, 16 * tb + lr, 32 * m + 16 + 4 * grp), acc[tb]);
        }
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) acc[tb] = acc[tb] * gam[16 * tb + lr];
        // the causal blocks cb <= tb, two per product
        static_for<NB>([&](auto tbc) __attribute__((always_inline)) {
            constexpr int tb = decltype(tbc)::value;
            const Frag p0 = sm.Pf[b2][tb][0][lane];
            const Frag p1 = tb >= 1 ? sm.Pf[b2][tb][1][lane] : zf;
            acc[tb] = E::mma32(DB[0], DB[1], p0, p1, acc[tb]);
            if constexpr (tb >= 2) {
                const Frag p2 = sm.Pf[b2][tb][2][lane];
                const Frag p3 = tb >= 3 ? sm.Pf[b2][tb][3][lane] : zf;
                acc[tb] = E::mma32(DB[2], DB[3], p2, p3, acc[tb]);
            }
        });
        if (og) {
            const int nrow = T_ - t0;
            const rsrc_t ro = make_rsrc(og + (size_t)t0 * D, (int64_t)nrow * D * 2);
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                const int t = 16 * tb + lr;
                buf_store8(ro, t < nrow ? (uint32_t)((t * D + 16 * cw + 4 * grp) * 2) : kOob, E::pack(acc[tb]));
            }
        }
    };

    // ---- chain wave: tile it; the state slice Sacc[kb][r] = S[v][k],
    // v = v0 + 16 cw + lr, k = 16 kb + 4 grp + r, as accumulators of S^T ----
    // part 1: the outputs and the update's right-hand side HB
    auto chain1 = [&](int it, const f32x4 (&Sacc)[KB], Frag (&HB)[NB])
        __attribute__((always_inline)) {
        const int b2 = it & 1;
        const T* Yb = sm.Y[b2];
        const float* hrow = sm.fac[b2][kHrow];
        Frag SB[KB], DB[NB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) SB[kb] = E::pack(Sacc[kb]);
        // Delta = Y: the targets themselves; and the update's right-hand
        // side diag(hrow) Delta
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            const Frag yf = ycol(Yb, 16 * rb, 16 * cw);
            const f32x4 hv = *reinterpret_cast<const f32x4*>(hrow + 16 * rb + 4 * grp);
            f32x4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = hv[r] * E::to_f((T)yf[r]);
            DB[rb] = yf;
            HB[rb] = E::pack(h);
        }
        outputs(it, SB, DB);
    };
    // part 2: S^T = exp(g_last) S0^T + X^T diag(hrow) Delta
    auto chain2 = [&](int it, f32x4 (&Sacc)[KB], const Frag (&HB)[NB])
        __attribute__((always_inline)) {
        const T* Xb = sm.X[it % XS];
        const float glq = sm.fac[it & 1][kGam][kF - 1];
        // the key column fragments: the first half of the state's blocks
        // requested before the first product, the rest while they run
        constexpr int KH = KB / 2;
        Frag xc[KB][NB];
        auto ldc = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < NB; ++q) xc[kb][q] = xcol(Xb, 16 * q, 16 * kb);
        };
#pragma unroll
        for (int kb = 0; kb < KH; ++kb) ldc(kb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            if (kb + KH < KB) ldc(kb + KH);
            f32x4 acc = Sacc[kb] * glq;
#pragma unroll
            for (int m = 0; m < NB / 2; ++m)
                acc = E::mma32(xc[kb][2 * m], xc[kb][2 * m + 1], HB[2 * m], HB[2 * m + 1], acc);
            Sacc[kb] = acc;
        }
    };
    // ---- the roles' loops: the prologue (fills | tile 0's intra-chunk part
    // 1 and raw P | part 2 and P's factors), then two barriers per tile ----
    if (role == 0) {
        const int vcol = v0 + 16 * cw + lr;
        f32x4 Sacc[KB];
        Frag HB[NB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            Sacc[kb] = a.S0 ? *reinterpret_cast<const f32x4*>(a.S0 + ((size_t)bh * D + vcol) * D +
                                                              16 * kb + 4 * grp)
                            : zero4();
        wait_vm_all();  // the state's loads: no wait inside the loop is owed to them
        __syncthreads();
        __syncthreads();
        __syncthreads();
        for (int it = 0; it < ntl; ++it) {
            chain1(it, Sacc, HB);
            lds_barrier();
            chain2(it, Sacc, HB);
            lds_barrier();
        }
        if (a.S_final) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                *reinterpret_cast<f32x4*>(a.S_final + ((size_t)bh * D + vcol) * D + 16 * kb + 4 * grp) =
                    Sacc[kb];
        }
    } else if (role == 1) {
        __syncthreads();
        if (ntl > 0) prep1(0);
        __syncthreads();
        __syncthreads();
        for (int it = 0; it < ntl; ++it) {
            if (it + 1 < ntl) prep1(it + 1);
            lds_barrier();
            // the per-column rule: tile it+2's keys (filled during iteration
            // it-1, tiles 0-1 converted at the prologue's fill) become write
            // vectors before iteration it+1's P waves read them
            if (COL && it + 2 < ntl) to_write(it + 2);
            lds_barrier();
        }
    } else {
        f32x4 pacc[NB];
        __syncthreads();
        if (ntl > 0) prow1(0, pacc);
        __syncthreads();
        if (ntl > 0) prow2(0, pacc);
        if (COL && ntl > 2) {
            // the per-column rule's third key tile, converted during iteration 0
            dma_x(2);
            wait_vm_all();
        }
        __syncthreads();
        for (int it = 0; it < ntl; ++it) {
            if (it + XD < ntl) dma_x(it + XD);
            if (it + 2 < ntl) dma_qg(it + 2);
            if (it + 1 < ntl) {
                dma_y(it + 1);
                prow1(it + 1, pacc);
            }
            lds_barrier();
            if (it + 1 < ntl) prow2(it + 1, pacc);
            wait_vm_all();
            lds_barrier();
        }
    }
}

}  // namespace

bool fused_supported(const ChunkArgs& a, int dt, int D, int chunk, bool delta) {
    // the inner-product family only: fused, the delta family's intra-chunk
    // solve and its state chain contended for LDS bandwidth and ran slower
    // than the split kernels
    return !delta && dt == 1 && (D == 64 || D == 128) && chunk == 64 && !a.phi && !a.ck_s &&
           (a.norm == kNormScalar || a.norm == kNormColumn || (a.norm == kNormWindow && a.W == 1));
}

hipError_t launch_fused(const ChunkArgs& a, int D, bool delta, hipStream_t stream) {
    const int ntiles = tiles_of(a.T, kF);
    ChunkArgs b = a;
    b.order = nullptr;
    b.toff = nullptr;
    b.jobs = nullptr;
    // packed calls: the sequences longest first
    hipError_t e = launch_packed_schedule(a, kF, ntiles, b, stream);
    if (e != hipSuccess) return e;
    const int nvs = D / 64;
    const int bh8 = (b.BH + 7) / 8 * 8;
    if (delta) return hipErrorInvalidValue;
    const bool col = a.norm == kNormColumn;
    if (D == 128) {
        if (col) hipLaunchKernelGGL((fused_kernel<128, true>), dim3(bh8 * nvs), dim3(768), 0, stream, b);
        else hipLaunchKernelGGL((fused_kernel<128, false>), dim3(bh8 * nvs), dim3(768), 0, stream, b);
    } else {
        if (col) hipLaunchKernelGGL((fused_kernel<64, true>), dim3(bh8 * nvs), dim3(768), 0, stream, b);
        else hipLaunchKernelGGL((fused_kernel<64, false>), dim3(bh8 * nvs), dim3(768), 0, stream, b);
    }
    return hipGetLastError();
}

}  // namespace falcon
