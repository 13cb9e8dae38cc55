// falcon_bwd.hip -- backward pass of the chunk-parallel form on gfx950.
//
// Method ("Fast Weight Attention for Continual Learning", authors' abstract:
// the rules have a chunk-parallel form; this file differentiates it).  Per
// tile of CV rows, with S0 the state at the tile start, g the tile-local
// cumulative log decay, omega_j = r_j x_j the write vectors, the forward is
//   (I + A) Delta = Y - diag(exp g) X S0^T        (A family: Delta = Y)
//   O     = diag(exp g) Q S0^T + P Delta
//   S_end = exp(g_L) S0 + Delta^T diag(exp(g_L - g)) Omega
// with A[i][j] = [j < i] exp(g_i - g_j) x_i.omega_j and
// P[t][j] = [j <= t] exp(g_t - g_j) q_t.omega_j.  Given dO and dS_end:
//   dDelta = P^T dO + diag(hrow) X dS_end^T            hrow_j = exp(g_L-g_j) r_j
//   dR     = (I + A)^-T dDelta                         (A family: dR = dDelta)
//   dS0    = exp(g_L) dS_end + dO^T diag(exp g) Q - dR^T diag(exp g) X
// (the last term only for the delta family), which is a reverse scan over
// the tiles (kernel 1 below), and then, per tile and independently (kernel 2),
//   DP[t][j] = [j <= t] exp(g_t - g_j) dO_t.Delta_j
//   DA[i][j] = -[j < i] exp(g_i - g_j) dR_i.Delta_j
//   dQ     = diag(exp g) dO S0 + DP Omega
//   dX     = -diag(exp g) dR S0 + DA Omega
//   dOmega = DP^T Q + DA^T X + diag(exp(g_L - g)) Delta dS_end
//   dY     = dR
// then the write scale (r = eta / (||x||^2 + eps): dx += r dOmega -
// 2 (r / n) (x.dOmega) x, deta = x.dOmega / n) and the decays: every factor
// exp(later - earlier) moves with g, so dg_s collects x_i.dX_i - omega_i.dOmega_i
// of its rows, q_s.dQ_s, and at the tile's last step exp(g_L) <dS_end, S0> +
// sum_j omega_j.dOmega3_j (dOmega3 the S_end term); dlog(alpha_s) is the sum of
// dg over the tile's steps from s on.
//
// The state at each tile start and Delta come from the forward state pass
// (bf16 checkpoints: the forward itself forms Delta from a bf16 right-hand
// side, so a wider copy would carry no more information), the A / P blocks and diagonal inverses from its
// intra-chunk records: kernel 1 reads them transposed out of LDS
// (ds_read_b64_tr_b16 on the record's fragment order).
#include "falcon_device.h"
#include "falcon_internal.h"
#include "falcon_records.h"

namespace falcon {

namespace {

typedef uint16_t bf;

__device__ __forceinline__ u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }

// Rows of sequence bh in the [rows, d] planes: [row0, row0 + T).  Batched
// calls: row0 = bh * T.  Packed calls: the bounds come from cu, clamped to the
// plane and to the longest sequence allowed (as the forward clamps them), so
// offsets outside the contract cannot move any access out of the buffers.
struct BSeq {
    size_t row0;
    int T;
};
__device__ __forceinline__ BSeq bwd_seq(const BwdArgs& a, int bh) {
    if (!a.cu) return {(size_t)bh * a.T, a.T};
    const int n = bh / a.H, h = bh - n * a.H;
    const int s0 = min(max(a.cu[n], 0), a.Ttot);
    const int s1 = min(min(max(a.cu[n + 1], s0), a.Ttot), s0 + a.T);
    return {(size_t)h * a.Ttot + s0, s1 - s0};
}

// The per-column rule's write vector (col_write) for four bf16 entries whose
// rows may differ (l1 and eta given per entry).
__device__ __forceinline__ s16x4 col_write4(s16x4 x, f32x4 l1, f32x4 eta, float eps) {
    f32x4 u;
#pragma unroll
    for (int r = 0; r < 4; ++r) u[r] = col_write(bf2f((bf)x[r]), l1[r], eta[r], eps);
    return EBf16::pack(u);
}


// Key row of virtual row i of the tile starting at t0 (window 1): k_{t0+i-lag},
// the halo before the sequence, zero outside.
__device__ __forceinline__ u32x4 key_piece(const bf* kg, const bf* kp, int W, int T, int tau,
                                           int col, int D) {
    if (tau >= 0 && tau < T) return *reinterpret_cast<const u32x4*>(kg + (size_t)tau * D + col);
    if (tau < 0 && kp && tau >= -W) return *reinterpret_cast<const u32x4*>(kp + (size_t)(W + tau) * D + col);
    return zero_u4();
}

}  // namespace

// ---------------------------------------------------------------------------
// Kernel 1: reverse scan over the tiles of one (batch*head, 64-wide value
// slice), its 8 waves in two roles.
//
//   waves 0-3 (chain)  tile it: the state gradient slice lives in registers
//                      as accumulators of dS^T (wave cw owns value columns
//                      v0 + 16 cw .. + 15; lane (lr, grp), block kb holds
//                      dS[v = v0 + 16 cw + lr][k = 16 kb + 4 grp + r]), the
//                      operand layout of X dS^T as it stands.  Checkpoint of
//                      dS (the gradient at the tile end, stored straight
//                      from the registers), dDelta, the transposed blocked
//                      substitution, dR to LDS, dS at the tile start.  No
//                      loads: a wave that issues loads waits for its own
//                      stores too (one counter), so the chain issues none.
//   waves 4-7 (fill)   the row stores of dv for tile it+1 from the chain's
//                      LDS dR, and the LDS copies of tile it-1 (keys,
//                      queries, dO slice, record) filled directly from
//                      memory (through registers for the first tiles, whose
//                      keys reach into the halo).
// Two LDS buffers by tile parity; one barrier per tile.
// ---------------------------------------------------------------------------
template <int D, int CV, bool DELTA>
struct BScanSmem {
    using R = Rec<EBf16, CV, DELTA>;
    static constexpr int LDX = D + 8, LDY = 64 + 8;
    bf X[2][CV][LDX];
    bf Q[2][CV][LDX];
    bf dO[2][CV][LDY];
    bf dR[2][CV][LDY];
    alignas(16) char rec[2][R::kBytes];
    uint32_t pf[4][64];  // landing area of the fill waves' L2 warm-up loads (never read)
};

template <int D, int CV, bool DELTA, bool WIN, bool COL>
__global__ __launch_bounds__(512) void bwd_scan_kernel(BwdArgs a) {
    using E = EBf16;
    using Frag = s16x4;
    using R = Rec<E, CV, DELTA>;
    using Smem = BScanSmem<D, CV, DELTA>;
    constexpr int NB = CV / 16, KB = D / 16, CPR = D / 8, NVS = D / 64;
    constexpr int LDX = Smem::LDX, LDY = Smem::LDY;
    constexpr int NXL = (CV * CPR + 255) / 256;
    constexpr int NYL = (CV * 8 + 255) / 256;
    constexpr int RPC = (int)(R::kBytes / 16);
    constexpr int NRL = (RPC + 255) / 256;
    static_assert(NB % 2 == 0, "pairs of 16-row blocks");
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    const bool chain = wave < 4;
    const int cw = wave & 3;
    const int ftid = tid & 255;  // index within the fill role
    // slices of one sequence on one XCD (consecutive workgroups go round the 8)
    const int blk = blockIdx.x, xcd = blk & 7, jj = blk >> 3;
    const int bh = (jj / NVS) * 8 + xcd, vs = jj % NVS;
    if (bh >= a.BH) return;
    const int v0 = vs * 64;
    // a tile holds Ct steps of Wv virtual rows (step s, window slot w) each
    const int W = a.W, Wv = WIN ? W : 1, Ct = CV / Wv, NVR = Ct * Wv, NBQ = (Ct + 15) / 16;
    const BSeq sq = bwd_seq(a, bh);
    const int T_ = sq.T, ntiles = a.ntiles, ntl = tiles_of(T_, Ct), lag = a.lag;
    // with a feature map, q and k are the mapped copies, at the sequence's own
    // rows of the workspace (bh * T)
    const size_t kq0 = a.phi ? (size_t)bh * a.T : sq.row0;
    const bf* kg = static_cast<const bf*>(a.k) + kq0 * D;
    const bf* qg = static_cast<const bf*>(a.q) + kq0 * D;
    const bf* dog = static_cast<const bf*>(a.d_o) + sq.row0 * D + v0;
    const bf* kp = a.k_prev ? static_cast<const bf*>(a.k_prev) + (size_t)bh * W * D : nullptr;
    const char* recg = static_cast<const char*>(a.rec) + (size_t)bh * ntiles * R::kBytes;
    bf* dvg = static_cast<bf*>(a.dv) + sq.row0 * D + v0;
    const int vcol = v0 + 16 * cw + lr;

    // ---- fill: one tile through registers ----
    u32x4 px[NXL], pq[NXL], py[NYL], pr[NRL];
    auto load = [&](int tile) __attribute__((always_inline)) {
        const int t0 = tile * Ct;
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int c = ftid + 256 * it, i = c / CPR, col = (c % CPR) * 8;
            const bool ok = c < CV * CPR;
            // key of virtual row i = (step s, slot w): k_{t0 + s - w - lag}
            const int sx = WIN ? i / Wv : i, wx = WIN ? i - sx * Wv : 0;
            px[it] = (ok && i < NVR) ? key_piece(kg, kp, W, T_, t0 + sx - wx - lag, col, D) : zero_u4();
            pq[it] = (ok && i < Ct && t0 + i < T_)
                         ? *reinterpret_cast<const u32x4*>(qg + (size_t)(t0 + i) * D + col)
                         : zero_u4();
        }
#pragma unroll
        for (int it = 0; it < NYL; ++it) {
            const int c = ftid + 256 * it, i = c / 8, col = (c % 8) * 8;
            py[it] = (c < CV * 8 && i < Ct && t0 + i < T_)
                         ? *reinterpret_cast<const u32x4*>(dog + (size_t)(t0 + i) * D + col)
                         : zero_u4();
        }
        const char* rg = recg + (size_t)tile * R::kBytes;
#pragma unroll
        for (int it = 0; it < NRL; ++it) {
            const int c = ftid + 256 * it;
            pr[it] = c < RPC ? *reinterpret_cast<const u32x4*>(rg + 16 * (size_t)c) : zero_u4();
        }
    };
    auto store = [&](int b) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int c = ftid + 256 * it, i = c / CPR, col = (c % CPR) * 8;
            if (c < CV * CPR) {
                *reinterpret_cast<u32x4*>(&sm.X[b][i][col]) = px[it];
                *reinterpret_cast<u32x4*>(&sm.Q[b][i][col]) = pq[it];
            }
        }
#pragma unroll
        for (int it = 0; it < NYL; ++it) {
            const int c = ftid + 256 * it, i = c / 8, col = (c % 8) * 8;
            if (c < CV * 8) *reinterpret_cast<u32x4*>(&sm.dO[b][i][col]) = py[it];
        }
#pragma unroll
        for (int it = 0; it < NRL; ++it) {
            const int c = ftid + 256 * it;
            if (c < RPC) *reinterpret_cast<u32x4*>(sm.rec[b] + 16 * c) = pr[it];
        }
    };
    // dR of `tile`: the rows of dv (a window of one), or the per-virtual-row
    // gradients a gather sums into dv (windows above one)
    auto store_dv = [&](int tile) __attribute__((always_inline)) {
        const int t0 = tile * Ct, b = tile & 1;
#pragma unroll
        for (int q = 0; q < NYL; ++q) {
            const int c = ftid + 256 * q, i = c / 8, col = (c % 8) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.dR[b][i][col]);
            if constexpr (WIN) {
                if (c < CV * 8)
                    *reinterpret_cast<u32x4*>(static_cast<bf*>(a.ck_r) +
                                              (((size_t)bh * ntiles + tile) * CV + i) * D + v0 + col) = v;
            } else {
                if (c < CV * 8 && t0 + i < T_) *reinterpret_cast<u32x4*>(dvg + (size_t)(t0 + i) * D + col) = v;
            }
        }
    };

    // column fragment of a row-major LDS tile: lane (lr, grp) gets
    // M[row0 + 4 grp + r][col0 + lr]
    auto colfrag = [&](const bf* m, int ld, int row0, int col0) __attribute__((always_inline)) {
        return E::load_tr(m + (size_t)(row0 + 4 * grp + (lr >> 2)) * ld + col0 + 4 * (lr & 3));
    };

    if (!chain) {
        // fill: tile ntl-1 before the loop, then per iteration it: dv of tile
        // it+1 out of LDS and tile it-1 into LDS.  Tiles whose keys lie in
        // the sequence go straight to LDS (buffer_load ... lds, a 16-byte
        // slot per lane, the slots' source offsets fixed relative to the
        // tile, padding and rows past the end reading as zero), waited for
        // before the barrier; the first tiles, whose keys reach into the halo,
        // go through registers.
        constexpr int SPX = LDX / 8, SPY = LDY / 8;
        constexpr int NSX = CV * SPX, NSY = CV * SPY;
        constexpr int NIX = (NSX + 63) / 64, NIY = (NSY + 63) / 64, NIR = (RPC + 63) / 64;
        constexpr int MIX = (NIX + 3) / 4, MIY = (NIY + 3) / 4, MIR = (NIR + 3) / 4;
        const int ow = wave & 3;
        uint32_t dx[MIX], dq[MIX], dy[MIY], dr[MIR];
#pragma unroll
        for (int m = 0; m < MIX; ++m) {
            const int k = 64 * (ow + 4 * m) + lane;
            const int row = k / SPX, wi = k - row * SPX;
            const int s = WIN ? row / Wv : row, w = WIN ? row - s * Wv : 0;
            const bool in = k < NSX && wi < D / 8;
            dx[m] = (in && row < NVR) ? (uint32_t)(((s - w - lag + W) * D + wi * 8) * 2) : kOob;
            dq[m] = (in && row < Ct) ? (uint32_t)((row * D + wi * 8) * 2) : kOob;
        }
#pragma unroll
        for (int m = 0; m < MIY; ++m) {
            const int k = 64 * (ow + 4 * m) + lane;
            const int row = k / SPY, wi = k - row * SPY;
            dy[m] = (k < NSY && wi < 8 && row < Ct) ? (uint32_t)((row * D + wi * 8) * 2) : kOob;
        }
#pragma unroll
        for (int m = 0; m < MIR; ++m) {
            const int k = 64 * (ow + 4 * m) + lane;
            dr[m] = k < RPC ? (uint32_t)(k * 16) : kOob;
        }
        const uint32_t sm_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) Smem*)&sm;
        auto dma = [&](int tile) __attribute__((always_inline)) {
            const int t0 = tile * Ct, b = tile & 1;
            const u32x4 rx = make_desc(kg + (size_t)(t0 - W) * D, (int64_t)(T_ - t0 + W) * D * 2);
            const u32x4 rq = make_desc(qg + (size_t)t0 * D, (int64_t)(T_ - t0) * D * 2);
            const u32x4 ro = make_desc(dog + (size_t)t0 * D, (int64_t)(T_ - t0) * D * 2);
            const u32x4 rr = make_desc(recg + (size_t)tile * R::kBytes, (int64_t)R::kBytes);
            const uint32_t xb = sm_lds + (uint32_t)(offsetof(Smem, X) + sizeof(sm.X[0]) * b);
            const uint32_t qb = sm_lds + (uint32_t)(offsetof(Smem, Q) + sizeof(sm.Q[0]) * b);
            const uint32_t ob = sm_lds + (uint32_t)(offsetof(Smem, dO) + sizeof(sm.dO[0]) * b);
            const uint32_t rb = sm_lds + (uint32_t)(offsetof(Smem, rec) + sizeof(sm.rec[0]) * b);
#pragma unroll
            for (int m = 0; m < MIX; ++m) {
                const int i = ow + 4 * m;
                if (i < NIX && 64 * i + lane < NSX) {
                    buf_load16_lds(rx, xb + 1024 * i, dx[m]);
                    buf_load16_lds(rq, qb + 1024 * i, dq[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < MIY; ++m) {
                const int i = ow + 4 * m;
                if (i < NIY && 64 * i + lane < NSY) buf_load16_lds(ro, ob + 1024 * i, dy[m]);
            }
#pragma unroll
            for (int m = 0; m < MIR; ++m) {
                const int i = ow + 4 * m;
                if (i < NIR && 64 * i + lane < RPC) buf_load16_lds(rr, rb + 1024 * i, dr[m]);
            }
        };
        auto fill = [&](int tile) __attribute__((always_inline)) {
            if (tile * Ct >= W) {
                dma(tile);
            } else {
                load(tile);
                store(tile & 1);
            }
        };
        // L2 warm-up of the tile after next (tile - 1, going down): two 4-byte
        // LDS-DMA loads per lane, one lane per 128-byte line of its keys,
        // queries, dO slice and record, landing in a scratch area nothing
        // reads.  They are the wave's two most recent loads every iteration
        // (offsets past the data read nothing), so the wait before the
        // barrier (vmcnt(2)) covers the fills and lets these run on.
        const uint32_t pfl = sm_lds + (uint32_t)(offsetof(Smem, pf) + 256 * ow);
        auto warm = [&](int tile) __attribute__((always_inline)) {
            const int t0 = tile * Ct;
            const bool ok = tile >= 0 && t0 >= W;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // 0-2: keys, 3-4: queries, 5: dO slice, 6-7: record (wave-uniform)
                const int inst = 2 * __builtin_amdgcn_readfirstlane(ow) + j;
                u32x4 d;
                uint32_t off = kOob;
                if (inst <= 2) {
                    d = make_desc(kg + (size_t)(ok ? t0 - W : 0) * D, ok ? (int64_t)(T_ - t0 + W) * D * 2 : 0);
                    const uint32_t o = (uint32_t)(inst * 64 + lane) * 128;
                    if (ok && o < (uint32_t)((Ct + W) * D * 2)) off = o;
                } else if (inst <= 4) {
                    d = make_desc(qg + (size_t)(ok ? t0 : 0) * D, ok ? (int64_t)(T_ - t0) * D * 2 : 0);
                    const uint32_t o = (uint32_t)((inst - 3) * 64 + lane) * 128;
                    if (ok && o < (uint32_t)(Ct * D * 2)) off = o;
                } else if (inst == 5) {
                    d = make_desc(dog + (size_t)(ok ? t0 : 0) * D, ok ? (int64_t)(T_ - t0) * D * 2 : 0);
                    if (ok && lane < Ct) off = (uint32_t)lane * D * 2;
                } else {
                    d = make_desc(recg + (size_t)(ok ? tile : 0) * R::kBytes, ok ? (int64_t)R::kBytes : 0);
                    const uint32_t o = (uint32_t)((inst - 6) * 64 + lane) * 128;
                    if (ok && o < (uint32_t)R::kBytes) off = o;
                }
                buf_load4_lds(d, pfl, off);
            }
        };
        if (ntl > 0) fill(ntl - 1);
        wait_vm_all();
        lds_barrier();
        for (int it = ntl - 1; it >= 0; --it) {
            if (it + 1 < ntl) store_dv(it + 1);
            if (it >= 1) fill(it - 1);
            warm(it - 2);
            wait_vm_2();
            lds_barrier();
        }
        wait_vm_all();
        if (ntl > 0) store_dv(0);
        return;
    }

    f32x4 dS[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
        dS[kb] = a.dS_final ? *reinterpret_cast<const f32x4*>(a.dS_final + ((size_t)bh * D + vcol) * D +
                                                              16 * kb + 4 * grp)
                            : zero4();
    // the state gradient's initial loads are complete before the loop, so no
    // wait inside it is owed to a load issued out here
    wait_vm_all();
    lds_barrier();
    // transposed record block (element offset `off`): lane (lr, grp) gets
    // M[4 grp + r][lr] of a block stored with M[lr][4 grp + r] at lane (lr, grp)
    for (int it = ntl - 1; it >= 0; --it) {
        const int b = it & 1;
        const char* recb = sm.rec[b];
        auto rec_tr = [&](size_t off) __attribute__((always_inline)) {
            const bf* blkp = reinterpret_cast<const bf*>(recb) + off;
            return E::load_tr(blkp + (size_t)((lr & 3) * 16 + 4 * grp + (lr >> 2)) * 4);
        };
        const bf* Xb = &sm.X[b][0][0];
        const bf* Qb = &sm.Q[b][0][0];
        const bf* dOb = &sm.dO[b][0][0];
        const float* gam = reinterpret_cast<const float*>(recb + R::kScalBytes);
        const float* hrow = gam + CV;
        const float* gq = gam + 2 * CV;
        // the per-column rule writes along u, not x: the A operand of
        // U dS^T is formed from the key rows on the way
        float l1r[NB], etr[NB];
        if constexpr (COL) {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                l1r[rb] = gam[3 * CV + 16 * rb + lr];
                etr[rb] = gam[4 * CV + 16 * rb + lr];
            }
        }

        Frag dSB[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) dSB[kb] = E::pack(dS[kb]);
        {
            // 16-column blocks ([kb][v][16]): one store writes 512 contiguous bytes
            bf* cs = static_cast<bf*>(a.ck_ds) + ((size_t)bh * ntiles + it) * D * D + (size_t)vcol * 16 + 4 * grp;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) *reinterpret_cast<Frag*>(cs + (size_t)kb * D * 16) = dSB[kb];
        }

        // dDelta = diag(hrow) X dS^T + P^T dO   (rows j, columns v)
        f32x4 dd[NB];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) dd[rb] = zero4();
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                const bf* xr = Xb + (size_t)(16 * rb + lr) * LDX + 32 * m + 4 * grp;
                Frag x0 = E::load(xr), x1 = E::load(xr + 16);
                if constexpr (COL) {
                    const f32x4 l = {l1r[rb], l1r[rb], l1r[rb], l1r[rb]};
                    const f32x4 e = {etr[rb], etr[rb], etr[rb], etr[rb]};
                    x0 = col_write4(x0, l, e, a.eps);
                    x1 = col_write4(x1, l, e, a.eps);
                }
                dd[rb] = E::mma32(x0, x1, dSB[2 * m], dSB[2 * m + 1], dd[rb]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            const f32x4 h = *reinterpret_cast<const f32x4*>(hrow + 16 * rb + 4 * grp);
#pragma unroll
            for (int r = 0; r < 4; ++r) dd[rb][r] *= h[r];
        }
        Frag dOc[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) dOc[tb] = colfrag(dOb, LDY, 16 * tb, 16 * cw);
        static_for<NB>([&](auto rbc) __attribute__((always_inline)) {
            constexpr int rb = decltype(rbc)::value;
            static_for<NB>([&](auto tbc) __attribute__((always_inline)) {
                constexpr int tb = decltype(tbc)::value;
                if constexpr (WIN) {
                    // the blocks the record holds: query block tb < NBQ that
                    // reaches back to a row of block rb
                    if (tb < NBQ && (16 * rb) / Wv <= 16 * tb + 15)
                        dd[rb] = E::mma16n(rec_tr(R::kP + (size_t)R::pblk(tb, rb, true) * 256), dOc[tb], dd[rb]);
                } else if constexpr (tb >= rb) {
                    dd[rb] = E::mma16n(rec_tr(R::kP + (size_t)R::pblk(tb, rb, false) * 256), dOc[tb], dd[rb]);
                }
            });
        });

        // dR = (I + A)^-T dDelta, by blocks from the last:
        // dR_b = Td_b^T (dDelta_b + sum_{c>b} (-A)_cb^T dR_c)
        f32x4 dr[NB];
        Frag drb[NB];
        if constexpr (DELTA) {
            static_for<NB>([&](auto qc) __attribute__((always_inline)) {
                constexpr int rb = NB - 1 - decltype(qc)::value;
                f32x4 acc = dd[rb];
                static_for<NB>([&](auto cbc) __attribute__((always_inline)) {
                    constexpr int cb = decltype(cbc)::value;
                    if constexpr (cb > rb)
                        acc = E::mma16n(rec_tr(R::kA + (size_t)R::ablk(cb, rb) * 256), drb[cb], acc);
                });
                dr[rb] = E::mma16n(rec_tr(R::kD + (size_t)rb * 256), E::pack(acc), zero4());
                drb[rb] = E::pack(dr[rb]);
            });
        } else {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) dr[rb] = dd[rb];
        }
        // dv rows leave through LDS (the fill waves store them)
#pragma unroll
        for (int rb = 0; rb < NB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.dR[b][16 * rb + 4 * grp + r][16 * cw + lr] = f2bf(dr[rb][r]);

        // dS at the tile start: exp(g_L) dS + (Q^T diag(gq) dO - X^T diag(gam) dR)^T
        const float gl = gq[Ct - 1];
        Frag bq[NB], bx[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const f32x4 g = *reinterpret_cast<const f32x4*>(gq + 16 * tb + 4 * grp);
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = bf2f((bf)dOc[tb][r]) * g[r];
            bq[tb] = E::pack(v);
        }
        if constexpr (DELTA) {
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) {
                const f32x4 g = *reinterpret_cast<const f32x4*>(gam + 16 * jb + 4 * grp);
                f32x4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = -g[r] * dr[jb][r];
                bx[jb] = E::pack(v);
            }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x4 acc = dS[kb] * gl;
#pragma unroll
            for (int m = 0; m < NB / 2; ++m)
                acc = E::mma32(colfrag(Qb, LDX, 32 * m, 16 * kb), colfrag(Qb, LDX, 32 * m + 16, 16 * kb),
                               bq[2 * m], bq[2 * m + 1], acc);
            // the residuals' S0 term (delta family only: the inner-product
            // family writes its targets, which do not depend on S0)
            if constexpr (DELTA) {
#pragma unroll
                for (int m = 0; m < NB / 2; ++m)
                    acc = E::mma32(colfrag(Xb, LDX, 32 * m, 16 * kb), colfrag(Xb, LDX, 32 * m + 16, 16 * kb),
                                   bx[2 * m], bx[2 * m + 1], acc);
            }
            dS[kb] = acc;
        }
        lds_barrier();
    }
    if (a.dS0) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            *reinterpret_cast<f32x4*>(a.dS0 + ((size_t)bh * D + vcol) * D + 16 * kb + 4 * grp) = dS[kb];
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: one workgroup of 4 waves per (batch*head, tile), two workgroups
// per compute unit (LDS under 80 KB), so that one workgroup's loads overlap
// the other's arithmetic.  The value dimension is contracted in quarters of
// 32 (state, state gradient, Delta, dR and dO of one quarter in LDS at a
// time); the masked, decayed DP and DA then take the staging room for the
// second products.  The gradients leave from the accumulators: the row dot
// products that the write-scale, decay and feature-map derivatives need are
// reduced across the waves through a small LDS table, and each lane stores
// four adjacent entries of a row.
// ---------------------------------------------------------------------------
template <int D, int CV>
struct BGradSmem {
    static constexpr int LDX = D + 8, LDQ = 32 + 8, LDC = CV + 8;
    bf X[CV][LDX];   // keys of the virtual rows
    bf Q[CV][LDX];   // queries of the steps
    struct Quarter {
        bf S0q[32][LDX];  // state at the tile start, 32 value rows ([v][k])
        bf dSq[32][LDX];  // state gradient at the tile end
        bf Dq[32][LDC];   // Delta ([v][i])
        bf dRq[CV][LDQ];  // dR rows ([i][v of the quarter])
        bf dOq[CV][LDQ];  // dO rows ([t][v of the quarter])
    };
    struct Mats {
        bf DP[CV][LDC];   // DP^T [j][t]
        bf DA[CV][LDC];   // DA^T [j][i]
        bf DPr[CV][LDC];  // r_j DP^T
        bf DAr[CV][LDC];  // r_j DA^T
    };
    struct Rows {
        bf K[CV][LDX];    // key gradients (or per-row key gradients), staged for row stores
        bf Qg[CV][LDX];   // query gradients
    };
    union {
        Quarter q;
        Mats m;
        Rows g;
    } u;
    float part[4][4][CV];  // per-wave partial row sums
    // per step s (tile-local): gates, log2(e) * g, the normalizer's
    // denominator and step size, decay gradient, chain-rule factor
    float al[CV], et[CV];
    alignas(16) float gs[CV];
    float den[CV], bst[CV], dg[CV], cn[CV];
    // per virtual row i: its step, log2(e) * g of the step, write scale, ||x||^2,
    // and the row sums x.dX, x.dOmega (q.dQ per step)
    int st[CV];
    alignas(16) float gv[CV];
    alignas(16) float rr[CV];
    float nrm[CV], sX[CV], sO[CV], sQ[CV];
    alignas(16) float l1[CV];  // ||x_i||_1 (per-column rule)
    float sC[CV];              // per-column rule: sum_k dOmega_k x_k |x_k| / den_k^2
    float rowk[2][CV], rowq[2][CV];  // feature map: 1/||raw||, phi . g
    float red[4][2];
};

template <int D, int CV, bool DELTA, bool WIN, bool COL>
__global__ __launch_bounds__(256, 2) void bwd_grad_kernel(BwdArgs a) {
    using E = EBf16;
    using Frag = s16x4;
    using Smem = BGradSmem<D, CV>;
    constexpr int NB = CV / 16, KB = D / 16, CPR = D / 8, NQ = D / 32;
    constexpr int KPW = KB / 4;    // 16-row blocks of k per wave
    constexpr int LDX = Smem::LDX, LDC = Smem::LDC;
    constexpr float kLog2e = 1.4426950408889634f;
    static_assert(NB == 4 && KB % 4 == 0, "one 64-row tile, d a multiple of 64");
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    const int ntiles = a.ntiles;
    const int bh = blockIdx.x / ntiles, tile = blockIdx.x - bh * ntiles;
    // a tile holds Ct steps of Wv virtual rows (step s, window slot w) each
    const int W = a.W, Wv = WIN ? W : 1, Ct = CV / Wv, NVR = Ct * Wv, NBQ = (Ct + 15) / 16;
    if (bh >= a.BH) return;
    const BSeq sq = bwd_seq(a, bh);
    const int T_ = sq.T, lag = a.lag;
    const size_t row0 = sq.row0;
    const int t0 = tile * Ct;
    if (t0 >= T_) return;
    const size_t tix = (size_t)bh * ntiles + tile;

    // ---- keys, queries, gates ----
    {
        const size_t kq0 = a.phi ? (size_t)bh * a.T : row0;  // mapped copies: own rows
        const bf* kg = static_cast<const bf*>(a.k) + kq0 * D;
        const bf* qg = static_cast<const bf*>(a.q) + kq0 * D;
        const bf* kp = a.k_prev ? static_cast<const bf*>(a.k_prev) + (size_t)bh * W * D : nullptr;
        constexpr int NXP = CV * CPR / 256;
        u32x4 px[NXP], pq[NXP];
#pragma unroll
        for (int it = 0; it < NXP; ++it) {
            const int c = tid + 256 * it, i = c / CPR, col = (c % CPR) * 8;
            const int sx = WIN ? i / Wv : i, wx = WIN ? i - sx * Wv : 0;
            px[it] = i < NVR ? key_piece(kg, kp, W, T_, t0 + sx - wx - lag, col, D) : zero_u4();
            pq[it] = (i < Ct && t0 + i < T_) ? *reinterpret_cast<const u32x4*>(qg + (size_t)(t0 + i) * D + col)
                                             : zero_u4();
        }
        if (tid < CV) {
            const bool in = tid < Ct && t0 + tid < T_;
            sm.al[tid] = in ? a.alpha[row0 + t0 + tid] : 1.f;
            sm.et[tid] = in ? a.eta[row0 + t0 + tid] : 0.f;
        }
#pragma unroll
        for (int it = 0; it < NXP; ++it) {
            const int c = tid + 256 * it, i = c / CPR, col = (c % CPR) * 8;
            *reinterpret_cast<u32x4*>(&sm.X[i][col]) = px[it];
            *reinterpret_cast<u32x4*>(&sm.Q[i][col]) = pq[it];
        }
    }
    lds_barrier();
    {
        // norms (4 lanes per row)
        const int row = tid >> 2, part = tid & 3;
        constexpr int EP = D / 4;
        float n2 = 0.f, n1 = 0.f;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
            const float x = bf2f(sm.X[row][part * EP + e]);
            n2 += x * x;
            n1 += fabsf(x);
        }
        n2 = group_sum_dpp<4>(n2);
        n1 = group_sum_dpp<4>(n1);
        if (part == 0) {
            sm.nrm[row] = n2;
            sm.l1[row] = n1;
        }
    }
    lds_barrier();
    if (tid < CV) {
        // per step: the normalizer over the step's rows and the step size
        const int s = tid;
        float n2 = 0.f;
        if (s < Ct)
            for (int w = 0; w < Wv; ++w) n2 += sm.nrm[s * Wv + w];
        const float dn = n2 + a.eps;
        sm.den[s] = dn;
        sm.bst[s] = (s < Ct && dn > 0.f) ? sm.et[s] / dn : 0.f;
    }
    if (wave == 0) {
        // the log-decay scan over the steps (steps past the tile: alpha = 1)
        const float lg = wave_scan_dpp(__logf(sm.al[lane]));
        sm.gs[lane] = lg * kLog2e;
    }
    lds_barrier();
    if (tid < CV) {
        const int i = tid;
        const int si = i < NVR ? i / Wv : (1 << 20);  // padding rows: after every step
        sm.st[i] = si;
        sm.gv[i] = sm.gs[i < NVR ? si : Ct - 1];
        // the per-column rule has no row scale: its write vectors are formed
        // entry by entry (col_write4) where the products need them
        sm.rr[i] = i < NVR ? (COL ? 1.f : sm.bst[si]) : 0.f;
    }

    auto colfrag = [&](const bf* m, int ld, int row0, int col0) __attribute__((always_inline)) {
        return E::load_tr(m + (size_t)(row0 + 4 * grp + (lr >> 2)) * ld + col0 + 4 * (lr & 3));
    };

    // wave w: k blocks KPW w .. KPW w + KPW - 1 of the three gradient tiles
    // (all four column blocks), and row block w of DP^T and DA^T
    const int jbw = wave;
    f32x4 aQ[KPW][NB], aX[KPW][NB], aW[KPW][NB], aP[NB], aA[NB];
#pragma unroll
    for (int kk = 0; kk < KPW; ++kk)
#pragma unroll
        for (int c = 0; c < NB; ++c) aQ[kk][c] = aX[kk][c] = aW[kk][c] = zero4();
#pragma unroll
    for (int c = 0; c < NB; ++c) aP[c] = aA[c] = zero4();
    float sdot = 0.f;  // <dS_end, S0>, this lane's share

    const bf* cks = static_cast<const bf*>(a.ck_s) + tix * D * D;
    const bf* ckds = static_cast<const bf*>(a.ck_ds) + tix * D * D;
    const bf* ckd = static_cast<const bf*>(a.ck_d) + tix * D * CV;
    // dR rows: dv itself for a window of one, else the per-virtual-row copy
    const bf* dRg = WIN ? static_cast<const bf*>(a.ck_r) + tix * CV * D
                        : static_cast<const bf*>(a.dv) + (row0 + t0) * D;
    const bf* dog = static_cast<const bf*>(a.d_o) + (row0 + t0) * D;
    constexpr int NSP = 32 * CPR / 256, NDP = 32 * (CV / 8) / 256, NRP = CV * 4 / 256;
    // not unrolled: an unrolled loop would hoist every quarter's loads to the
    // top (the barriers order LDS only) and run out of registers
    // Quarter qv's pieces are loaded while quarter qv-1 is computed: the
    // registers that carried quarter qv-1 into LDS take quarter qv's loads
    // right after.
    u32x4 pS[NSP], pG[NSP], pD[NDP], pR[NRP], pO[NRP];
    auto load_q = [&](int qv) __attribute__((always_inline)) {
        // the checkpoints are stored in 16-column blocks ([block][v][16]): piece c
        // is half c % 2 of row c / 2 % 32 of the quarter in block c / 64, and
        // consecutive pieces are consecutive 16 bytes
#pragma unroll
        for (int it = 0; it < NSP; ++it) {
            const int c = tid + 256 * it, kb = c >> 6, v = (c >> 1) & 31, h8 = (c & 1) * 8;
            const size_t off = ((size_t)kb * D + 32 * qv + v) * 16 + h8;
            pS[it] = *reinterpret_cast<const u32x4*>(cks + off);
            pG[it] = *reinterpret_cast<const u32x4*>(ckds + off);
        }
#pragma unroll
        for (int it = 0; it < NDP; ++it) {
            const int c = tid + 256 * it, cb = c >> 6, v = (c >> 1) & 31, h8 = (c & 1) * 8;
            pD[it] = *reinterpret_cast<const u32x4*>(ckd + ((size_t)cb * D + 32 * qv + v) * 16 + h8);
        }
#pragma unroll
        for (int it = 0; it < NRP; ++it) {
            const int c = tid + 256 * it, i = c / 4, col = (c % 4) * 8;
            const bool rin = WIN || t0 + i < T_;
            const bool oin = i < Ct && t0 + i < T_;
            pR[it] = rin ? *reinterpret_cast<const u32x4*>(dRg + (size_t)i * D + 32 * qv + col) : zero_u4();
            pO[it] = oin ? *reinterpret_cast<const u32x4*>(dog + (size_t)i * D + 32 * qv + col) : zero_u4();
        }
    };
    load_q(0);
#pragma unroll 1
    for (int qv = 0; qv < NQ; ++qv) {
        lds_barrier();  // the previous quarter's operands are consumed
#pragma unroll
        for (int it = 0; it < NSP; ++it) {
            const int c = tid + 256 * it, v = (c >> 1) & 31, col = (c >> 6) * 16 + (c & 1) * 8;
            *reinterpret_cast<u32x4*>(&sm.u.q.S0q[v][col]) = pS[it];
            *reinterpret_cast<u32x4*>(&sm.u.q.dSq[v][col]) = pG[it];
            const bf* se = reinterpret_cast<const bf*>(&pS[it]);
            const bf* ge = reinterpret_cast<const bf*>(&pG[it]);
#pragma unroll
            for (int e = 0; e < 8; ++e) sdot += bf2f(se[e]) * bf2f(ge[e]);
        }
#pragma unroll
        for (int it = 0; it < NDP; ++it) {
            const int c = tid + 256 * it, v = (c >> 1) & 31, col = (c >> 6) * 16 + (c & 1) * 8;
            *reinterpret_cast<u32x4*>(&sm.u.q.Dq[v][col]) = pD[it];
        }
#pragma unroll
        for (int it = 0; it < NRP; ++it) {
            const int c = tid + 256 * it, i = c / 4, col = (c % 4) * 8;
            *reinterpret_cast<u32x4*>(&sm.u.q.dRq[i][col]) = pR[it];
            *reinterpret_cast<u32x4*>(&sm.u.q.dOq[i][col]) = pO[it];
        }
        if (qv + 1 < NQ) load_q(qv + 1);
        lds_barrier();
        const bf* Dq = &sm.u.q.Dq[0][0];
        // the wave's block jbw is a compile-time constant of each copy, so
        // the causal tests leave no branches between the products
        with_const4(jbw, [&](auto jc) __attribute__((always_inline)) {
            constexpr int JB = decltype(jc)::value;
            const Frag dj0 = colfrag(Dq, LDC, 0, 16 * JB), dj1 = colfrag(Dq, LDC, 16, 16 * JB);
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                // DP^T block (jbw, tb): query block tb reaching back to a row of block jbw
                if (tb < NBQ && (16 * JB) / Wv <= 16 * tb + 15) {
                    const bf* orow = &sm.u.q.dOq[16 * tb + lr][4 * grp];
                    aP[tb] = E::mma32(dj0, dj1, E::load(orow), E::load(orow + 16), aP[tb]);
                }
                // DA^T block (jbw, tb): only rows of later steps, so tb >= jbw
                if (DELTA && tb >= JB) {
                    const bf* rrow = &sm.u.q.dRq[16 * tb + lr][4 * grp];
                    aA[tb] = E::mma32(dj0, dj1, E::load(rrow), E::load(rrow + 16), aA[tb]);
                }
            }
        });
#pragma unroll
        for (int kk = 0; kk < KPW; ++kk) {
            const int kb = KPW * wave + kk;
            const Frag s0 = colfrag(&sm.u.q.S0q[0][0], LDX, 0, 16 * kb);
            const Frag s1 = colfrag(&sm.u.q.S0q[0][0], LDX, 16, 16 * kb);
            const Frag g0 = colfrag(&sm.u.q.dSq[0][0], LDX, 0, 16 * kb);
            const Frag g1 = colfrag(&sm.u.q.dSq[0][0], LDX, 16, 16 * kb);
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if (cb < NBQ) {
                    const bf* orow = &sm.u.q.dOq[16 * cb + lr][4 * grp];
                    aQ[kk][cb] = E::mma32(s0, s1, E::load(orow), E::load(orow + 16), aQ[kk][cb]);
                }
                if constexpr (DELTA) {
                    const bf* rrow = &sm.u.q.dRq[16 * cb + lr][4 * grp];
                    aX[kk][cb] = E::mma32(s0, s1, E::load(rrow), E::load(rrow + 16), aX[kk][cb]);
                }
                aW[kk][cb] = E::mma32(g0, g1, colfrag(Dq, LDC, 0, 16 * cb), colfrag(Dq, LDC, 16, 16 * cb),
                                      aW[kk][cb]);
            }
        }
    }

    // ---- decays; sum_j omega_j . dOmega3_j; DP and DA to LDS ----
    const float gL = sm.gs[Ct - 1];
    float s3 = 0.f;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        const int col = 16 * cb + lr;
        const float eq = exp2f(sm.gs[col]);   // query column (step) col
        const float gc = sm.gv[col];           // virtual row col
        const float ex = exp2f(gc), ew = exp2f(gL - gc), rc = sm.rr[col];
#pragma unroll
        for (int kk = 0; kk < KPW; ++kk) {
            const int kb = KPW * wave + kk;
            aQ[kk][cb] = aQ[kk][cb] * eq;
            aX[kk][cb] = aX[kk][cb] * (-ex);
            aW[kk][cb] = aW[kk][cb] * ew;
            Frag xk = E::load(&sm.X[col][16 * kb + 4 * grp]);
            if constexpr (COL) {
                const float l = sm.l1[col], e = sm.et[col];
                xk = col_write4(xk, f32x4{l, l, l, l}, f32x4{e, e, e, e}, a.eps);
            }
            float p = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) p += bf2f((bf)xk[r]) * aW[kk][cb][r];
            s3 += rc * p;
        }
    }
    s3 = group_sum<64>(s3);
    sdot = group_sum<64>(sdot);
    if (lane == 0) {
        sm.red[wave][0] = s3;
        sm.red[wave][1] = sdot;
    }
    lds_barrier();  // the staging room is free for DP and DA
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
        const int t = 16 * tb + lr;  // query step t (DP) or virtual row t (DA)
        const float gt = sm.gs[t], gi = sm.gv[t];
        const int si = sm.st[t];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * jbw + 4 * grp + r;
            const float gj = sm.gv[j], rj = sm.rr[j];
            const int sj = sm.st[j];
            // evaluated for every lane and selected (no branch around exp2)
            const float ep = aP[tb][r] * exp2f(gt - gj);
            const float vp = (sj <= t && t < Ct) ? ep : 0.f;
            float va = 0.f;
            if constexpr (DELTA) {
                const float ea = -aA[tb][r] * exp2f(gi - gj);
                va = sj < si ? ea : 0.f;
            }
            sm.u.m.DP[j][t] = f2bf(vp);
            sm.u.m.DPr[j][t] = f2bf(vp * rj);
            sm.u.m.DA[j][t] = f2bf(va);
            sm.u.m.DAr[j][t] = f2bf(va * rj);
        }
    }
    lds_barrier();

    // ---- second products ----
    {
        const bf* Xs = &sm.X[0][0];
        const bf* Qs = &sm.Q[0][0];
        const bf* DP = &sm.u.m.DP[0][0];
        const bf* DA = &sm.u.m.DA[0][0];
        const bf* DPr = &sm.u.m.DPr[0][0];
        const bf* DAr = &sm.u.m.DAr[0][0];
#pragma unroll
        for (int kk = 0; kk < KPW; ++kk) {
            const int kb = KPW * wave + kk;
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) {
                const Frag xj = colfrag(Xs, LDX, 16 * jb, 16 * kb);
                const Frag qj = colfrag(Qs, LDX, 16 * jb, 16 * kb);
                // the write vectors omega_j: r_j x_j (the r_j sit in DPr, DAr), or
                // the per-column rule's u_j, entries of rows 16 jb + 4 grp + r
                Frag wj = xj;
                if constexpr (COL) {
                    const int j0 = 16 * jb + 4 * grp;
                    wj = col_write4(xj, *reinterpret_cast<const f32x4*>(&sm.l1[j0]),
                                    *reinterpret_cast<const f32x4*>(&sm.et[j0]), a.eps);
                }
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) {
                    // dQ^T (query block cb): rows of steps up to the block's last
                    if (cb < NBQ && (16 * jb) / Wv <= 16 * cb + 15)
                        aQ[kk][cb] = E::mma16n(wj, colfrag(DPr, LDC, 16 * jb, 16 * cb), aQ[kk][cb]);
                    if (DELTA && jb <= cb)
                        aX[kk][cb] = E::mma16n(wj, colfrag(DAr, LDC, 16 * jb, 16 * cb), aX[kk][cb]);
                    // dOmega^T (row block cb): queries of the steps from the block's first
                    if (jb < NBQ && (16 * cb) / Wv <= 16 * jb + 15)
                        aW[kk][cb] = E::mma16n(qj, E::load(DP + (size_t)(16 * cb + lr) * LDC + 16 * jb + 4 * grp),
                                              aW[kk][cb]);
                    if (DELTA && jb >= cb)
                        aW[kk][cb] = E::mma16n(xj, E::load(DA + (size_t)(16 * cb + lr) * LDC + 16 * jb + 4 * grp),
                                              aW[kk][cb]);
                }
            }
        }
    }

    // ---- row sums across the waves: x_i.dX_i, x_i.dOmega_i, q_t.dQ_t ----
    // lane (lr, grp) holds, for column block cb, row 16 cb + lr and entries
    // k = 16 kb + 4 grp + r of each of its k blocks
    auto row_sum = [&](float v) __attribute__((always_inline)) {
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        return v;
    };
    // (per-column rule: x.dOmega is replaced by sum_k dOmega_k x_k / den_k,
    // and sum_k dOmega_k x_k |x_k| / den_k^2 joins, den_k = |x_k| l1 + eps)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        const int row = 16 * cb + lr;
        const float l1r = COL ? sm.l1[row] : 0.f;
        float pX = 0.f, pO = 0.f, pQ = 0.f, pC = 0.f;
#pragma unroll
        for (int kk = 0; kk < KPW; ++kk) {
            const int kb = KPW * wave + kk;
            const Frag xk = E::load(&sm.X[row][16 * kb + 4 * grp]);
            const Frag qk = E::load(&sm.Q[row][16 * kb + 4 * grp]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = bf2f((bf)xk[r]);
                pX += x * aX[kk][cb][r];
                pQ += bf2f((bf)qk[r]) * aQ[kk][cb][r];
                if constexpr (COL) {
                    const float den = fabsf(x) * l1r + a.eps;
                    const float id = den > 0.f ? 1.f / den : 0.f;
                    pO += aW[kk][cb][r] * x * id;
                    pC += aW[kk][cb][r] * x * fabsf(x) * id * id;
                } else {
                    pO += x * aW[kk][cb][r];
                }
            }
        }
        pX = row_sum(pX);
        pO = row_sum(pO);
        pQ = row_sum(pQ);
        if constexpr (COL) pC = row_sum(pC);
        if (grp == 0) {
            sm.part[wave][0][row] = pX;
            sm.part[wave][1][row] = pO;
            sm.part[wave][2][row] = pQ;
            if constexpr (COL) sm.part[wave][3][row] = pC;  // slot 3: free until the L2 map
        }
    }
    lds_barrier();
    if (tid < CV) {
        float x = 0.f, o = 0.f, q = 0.f, c = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            x += sm.part[w][0][tid];
            o += sm.part[w][1][tid];
            q += sm.part[w][2][tid];
            if constexpr (COL) c += sm.part[w][3][tid];
        }
        sm.sX[tid] = x;
        sm.sO[tid] = o;
        sm.sQ[tid] = q;
        if constexpr (COL) sm.sC[tid] = c;
    }
    lds_barrier();
    if (tid < CV) {
        // per step s: x.dOmega of its rows gives deta and the normalizer's
        // chain-rule factor; the decay gradient collects x.dX - omega.dOmega of
        // its rows and q.dQ
        const int s = tid;
        if constexpr (COL) {
            // u = eta x / den entrywise: deta = sum dOmega x / den,
            // omega . dOmega = eta deta; cn carries eta sum dOmega x |x| / den^2
            const float e = sm.et[s], de = sm.sO[s];
            sm.dg[s] = s < Ct ? sm.sX[s] - e * de + sm.sQ[s] : 0.f;
            sm.cn[s] = s < Ct ? e * sm.sC[s] : 0.f;
            if (s < Ct && t0 + s < T_) a.deta[row0 + t0 + s] = de;
        } else {
            float so = 0.f, sg = 0.f;
            if (s < Ct) {
                for (int w = 0; w < Wv; ++w) {
                    const int i = s * Wv + w;
                    so += sm.sO[i];
                    sg += sm.sX[i] - sm.rr[i] * sm.sO[i];
                }
                sg += sm.sQ[s];
            }
            const float dn = sm.den[s];
            sm.cn[s] = (s < Ct && dn > 0.f) ? 2.f * sm.bst[s] * so / dn : 0.f;
            sm.dg[s] = sg;
            if (s < Ct && t0 + s < T_) a.deta[row0 + t0 + s] = dn > 0.f ? so / dn : 0.f;
        }
    }
    lds_barrier();

    // ---- key and query gradients: dx = dX + r dOmega - cn x, dq = dQ ----
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        const int row = 16 * cb + lr;
        const int si = sm.st[row];
        const float r = sm.rr[row], c = si < Ct ? sm.cn[si] : 0.f;
        const float l1r = COL ? sm.l1[row] : 0.f, er = COL ? sm.et[row] : 0.f;
#pragma unroll
        for (int kk = 0; kk < KPW; ++kk) {
            const int kb = KPW * wave + kk;
            const Frag xk = E::load(&sm.X[row][16 * kb + 4 * grp]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = bf2f((bf)xk[e]);
                if constexpr (COL) {
                    // du_k/dx_k (l1 held) = eta eps / den^2; through l1: -sign(x) eta sum(...)
                    const float den = fabsf(x) * l1r + a.eps;
                    const float id = den > 0.f ? 1.f / den : 0.f;
                    const float sg = x > 0.f ? 1.f : (x < 0.f ? -1.f : 0.f);
                    aX[kk][cb][e] = aX[kk][cb][e] + aW[kk][cb][e] * er * a.eps * id * id - c * sg;
                } else {
                    aX[kk][cb][e] = aX[kk][cb][e] + r * aW[kk][cb][e] - c * x;
                }
            }
        }
    }
    // rows: key row tau = t - lag (a window of one: its only use is as x of
    // step t; a padded step t >= T computes dx = 0, the gradient of the key no
    // step reads), query row t
    auto key_ok = [&](int row) __attribute__((always_inline)) {
        const int t = t0 + row, tau = t - lag;
        return !WIN && (t < T_ + lag) && tau < T_ && (tau >= 0 || (a.dk_prev && a.kp_raw));
    };
    auto key_raw = [&](int row) __attribute__((always_inline)) {
        const int tau = t0 + row - lag;
        return tau >= 0 ? static_cast<const bf*>(a.k_raw) + (row0 + tau) * D
                        : static_cast<const bf*>(a.kp_raw) + ((size_t)bh * W + W + tau) * D;
    };
    auto raw4 = [&](const bf* raw, int kb, float (&kr)[4]) __attribute__((always_inline)) {
        const Frag f = *reinterpret_cast<const Frag*>(raw + 16 * kb + 4 * grp);
#pragma unroll
        for (int e = 0; e < 4; ++e) kr[e] = bf2f((bf)f[e]);
    };
    if (a.phi == 1) {
        // L2 map: g_raw = (g - phi (phi . g)) / ||raw||, phi = raw / ||raw||
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
            const int row = 16 * cb + lr;
            const bool kok = key_ok(row), qok = row < Ct && t0 + row < T_;
            float nk = 0.f, pk = 0.f, nq = 0.f, pq = 0.f;
#pragma unroll
            for (int kk = 0; kk < KPW; ++kk) {
                const int kb = KPW * wave + kk;
                float kr[4];
                if (kok) {
                    raw4(key_raw(row), kb, kr);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        nk += kr[e] * kr[e];
                        pk += kr[e] * aX[kk][cb][e];
                    }
                }
                if (qok) {
                    raw4(static_cast<const bf*>(a.q_raw) + (row0 + t0 + row) * D, kb, kr);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        nq += kr[e] * kr[e];
                        pq += kr[e] * aQ[kk][cb][e];
                    }
                }
            }
            nk = row_sum(nk);
            pk = row_sum(pk);
            nq = row_sum(nq);
            pq = row_sum(pq);
            if (grp == 0) {
                sm.part[wave][0][row] = nk;
                sm.part[wave][1][row] = pk;
                sm.part[wave][2][row] = nq;
                sm.part[wave][3][row] = pq;
            }
        }
        lds_barrier();
        if (tid < CV) {
            float nk = 0.f, pk = 0.f, nq = 0.f, pq = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                nk += sm.part[w][0][tid];
                pk += sm.part[w][1][tid];
                nq += sm.part[w][2][tid];
                pq += sm.part[w][3][tid];
            }
            const float ik = nk > 0.f ? rsqrtf(nk) : 0.f, iq = nq > 0.f ? rsqrtf(nq) : 0.f;
            sm.rowk[0][tid] = ik;
            sm.rowk[1][tid] = pk * ik;  // phi . g
            sm.rowq[0][tid] = iq;
            sm.rowq[1][tid] = pq * iq;
        }
        lds_barrier();
    }
    auto phi_back = [&](float (&g)[4], const float (&kr)[4], float inv, float pd) __attribute__((always_inline)) {
        if (a.phi == 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) g[e] = (g[e] - kr[e] * inv * pd) * inv;
        } else if (a.phi == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sg = 1.f / (1.f + __expf(-kr[e]));
                g[e] = g[e] * sg * (1.f + kr[e] * (1.f - sg));
            }
        }
    };
    auto pack4 = [&](const float (&g)[4]) __attribute__((always_inline)) {
        Frag f;
        f.x = (short)f2bf(g[0]);
        f.y = (short)f2bf(g[1]);
        f.z = (short)f2bf(g[2]);
        f.w = (short)f2bf(g[3]);
        return f;
    };
    // the gradient rows go to LDS (the staging room is free since the second
    // products), then leave as 16-byte row stores
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        const int row = 16 * cb + lr, t = t0 + row;
        if (WIN || key_ok(row)) {
            // the key gradient of the row; with a window before the feature map
            // (the gather sums a key's window rows and applies the map)
            const bf* raw = WIN ? nullptr : key_raw(row);
#pragma unroll
            for (int kk = 0; kk < KPW; ++kk) {
                const int kb = KPW * wave + kk;
                float g[4] = {aX[kk][cb][0], aX[kk][cb][1], aX[kk][cb][2], aX[kk][cb][3]};
                if (!WIN && a.phi) {
                    float kr[4];
                    raw4(raw, kb, kr);
                    phi_back(g, kr, a.phi == 1 ? sm.rowk[0][row] : 0.f, a.phi == 1 ? sm.rowk[1][row] : 0.f);
                }
                *reinterpret_cast<Frag*>(&sm.u.g.K[row][16 * kb + 4 * grp]) = pack4(g);
            }
        }
        if (row < Ct && t < T_) {
            const bf* raw = static_cast<const bf*>(a.q_raw) + (row0 + t) * D;
#pragma unroll
            for (int kk = 0; kk < KPW; ++kk) {
                const int kb = KPW * wave + kk;
                float g[4] = {aQ[kk][cb][0], aQ[kk][cb][1], aQ[kk][cb][2], aQ[kk][cb][3]};
                if (a.phi) {
                    float kr[4];
                    raw4(raw, kb, kr);
                    phi_back(g, kr, a.phi == 1 ? sm.rowq[0][row] : 0.f, a.phi == 1 ? sm.rowq[1][row] : 0.f);
                }
                *reinterpret_cast<Frag*>(&sm.u.g.Qg[row][16 * kb + 4 * grp]) = pack4(g);
            }
        }
    }
    lds_barrier();
    for (int c = tid; c < CV * CPR; c += 256) {
        const int row = c / CPR, col = (c % CPR) * 8, t = t0 + row, tau = t - lag;
        if constexpr (WIN) {
            *reinterpret_cast<u32x4*>(static_cast<bf*>(a.ck_x) + (tix * CV + row) * D + col) =
                *reinterpret_cast<const u32x4*>(&sm.u.g.K[row][col]);
        } else if (key_ok(row)) {
            bf* dst = tau >= 0 ? static_cast<bf*>(a.dk) + (row0 + tau) * D
                               : static_cast<bf*>(a.dk_prev) + ((size_t)bh * W + W + tau) * D;
            *reinterpret_cast<u32x4*>(dst + col) = *reinterpret_cast<const u32x4*>(&sm.u.g.K[row][col]);
        }
        if (row < Ct && t < T_)
            *reinterpret_cast<u32x4*>(static_cast<bf*>(a.dq) + (row0 + t) * D + col) =
                *reinterpret_cast<const u32x4*>(&sm.u.g.Qg[row][col]);
    }
    if constexpr (!WIN) {
        // keys no row of any tile reaches: k_{T-1} (prefix alignment, T a
        // multiple of the tile) and the halo rows same-step pairs never read
        if (t0 + CV == T_ && lag == 1) {
            for (int c = tid; c < CPR; c += 256)
                *reinterpret_cast<u32x4*>(static_cast<bf*>(a.dk) + (row0 + T_ - 1) * D + 8 * c) = zero_u4();
        }
        if (tile == 0 && a.dk_prev) {
            for (int c = tid; c < W * CPR; c += 256) {
                const int row = c / CPR;
                if (lag == 0 || !a.kp_raw || row < W - 1)
                    *reinterpret_cast<u32x4*>(static_cast<bf*>(a.dk_prev) + ((size_t)bh * W + row) * D +
                                              8 * (c % CPR)) = zero_u4();
            }
        }
    }

    // ---- decay gradients: dlog alpha_s = sum over the tile's steps s' >= s of dg ----
    if (wave == 0) {
        float g = lane < Ct ? sm.dg[lane] : 0.f;
        if (lane == Ct - 1) {
            float s3t = 0.f, sdt = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                s3t += sm.red[w][0];
                sdt += sm.red[w][1];
            }
            g += exp2f(gL) * sdt + s3t;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_down(g, off, 64);
            if (lane + off < 64) g += y;
        }
        if (lane < Ct && t0 + lane < T_) a.dalpha[row0 + t0 + lane] = g / sm.al[lane];
    }
}

// ---------------------------------------------------------------------------
// Kernel 3 (windows above one): the gather.  Key tau serves the W rows
// (step tau + lag + w, slot w) and value tau the rows (step tau + w, slot w),
// w = 0..W-1, which can sit in two tiles: the per-virtual-row gradients are
// summed here in fp32, the key sums go through the feature map's derivative,
// and every key and value row (the halo rows included) is written once.
// CPR lanes per row, 8 entries each.
// ---------------------------------------------------------------------------
template <int D, int CV>
__global__ __launch_bounds__(256) void bwd_gather_kernel(BwdArgs a) {
    constexpr int CPR = D / 8, RPB = 256 / CPR;
    const int W = a.W, Ct = CV / W, lag = a.lag, ntiles = a.ntiles;
    const int tid = threadIdx.x, part = tid % CPR;
    const int nrows = a.T + W;  // rows tau = -W .. T-1 of the longest sequence allowed
    const int rid = blockIdx.x * RPB + tid / CPR;
    const int bh = rid / nrows, tau = rid - bh * nrows - W;
    if (bh >= a.BH) return;  // whole row groups: uniform within a DPP group
    const BSeq sq = bwd_seq(a, bh);
    const int T_ = sq.T;
    const size_t row0 = sq.row0;
    if (tau >= T_) return;
    const int col = part * 8;
    auto vrow = [&](int s, int w) {
        return (((size_t)bh * ntiles + s / Ct) * CV + (s % Ct) * W + w) * D + col;
    };
    auto add8 = [&](float (&g)[8], const bf* p) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        const bf* e = reinterpret_cast<const bf*>(&v);
#pragma unroll
        for (int u = 0; u < 8; ++u) g[u] += bf2f(e[u]);
    };
    auto put8 = [&](bf* dst, const float (&g)[8]) {
        u32x4 o;
        bf* e = reinterpret_cast<bf*>(&o);
#pragma unroll
        for (int u = 0; u < 8; ++u) e[u] = f2bf(g[u]);
        *reinterpret_cast<u32x4*>(dst + col) = o;
    };
    // keys: dk_tau = phi'(raw)^T sum_w dx(step tau + lag + w, slot w)
    {
        float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < W; ++w) {
            const int s = tau + lag + w;
            if (s >= 0 && s < T_) add8(g, static_cast<const bf*>(a.ck_x) + vrow(s, w));
        }
        const bf* raw = tau >= 0 ? static_cast<const bf*>(a.k_raw) + (row0 + tau) * D
                                 : (a.kp_raw ? static_cast<const bf*>(a.kp_raw) + ((size_t)bh * W + W + tau) * D
                                             : nullptr);
        if (a.phi && raw) {
            float kr[8];
            const u32x4 v = *reinterpret_cast<const u32x4*>(raw + col);
            const bf* e = reinterpret_cast<const bf*>(&v);
#pragma unroll
            for (int u = 0; u < 8; ++u) kr[u] = bf2f(e[u]);
            if (a.phi == 1) {
                float n2 = 0.f, pk = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    n2 += kr[u] * kr[u];
                    pk += kr[u] * g[u];
                }
                if constexpr (CPR <= 16) {
                    n2 = group_sum_dpp<CPR>(n2);
                    pk = group_sum_dpp<CPR>(pk);
                } else {
                    n2 = group_sum<CPR>(n2);
                    pk = group_sum<CPR>(pk);
                }
                const float inv = n2 > 0.f ? rsqrtf(n2) : 0.f, pd = pk * inv;
#pragma unroll
                for (int u = 0; u < 8; ++u) g[u] = (g[u] - kr[u] * inv * pd) * inv;
            } else {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float sg = 1.f / (1.f + __expf(-kr[u]));
                    g[u] = g[u] * sg * (1.f + kr[u] * (1.f - sg));
                }
            }
        }
        if (!raw) {
#pragma unroll
            for (int u = 0; u < 8; ++u) g[u] = 0.f;  // no halo given: a constant zero key
        }
        if (tau >= 0) put8(static_cast<bf*>(a.dk) + (row0 + tau) * D, g);
        else if (a.dk_prev) put8(static_cast<bf*>(a.dk_prev) + ((size_t)bh * W + W + tau) * D, g);
    }
    // values: dv_tau = sum_w dR(step tau + w, slot w), tau >= -(W - 1)
    if (tau >= -(W - 1)) {
        float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < W; ++w) {
            const int s = tau + w;
            if (s >= 0 && s < T_) add8(g, static_cast<const bf*>(a.ck_r) + vrow(s, w));
        }
        if (tau >= 0) put8(static_cast<bf*>(a.dv) + (row0 + tau) * D, g);
        else if (a.dv_prev) put8(static_cast<bf*>(a.dv_prev) + ((size_t)bh * (W - 1) + W - 1 + tau) * D, g);
    }
}

__global__ void bwd_zero_kernel(bf* p, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool chunk_bwd_supported(int dt, int D, int chunk, int norm, int window) {
    return dt == 1 && (D == 64 || D == 128) && chunk == 64 &&
           (norm == kNormScalar || norm == kNormColumn || (norm == kNormWindow && window >= 1 && window <= 8));
}

template <int D, bool DELTA, bool WIN, bool COL>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
    constexpr int CV = 64;
    const int nvs = D / 64;
    const int bh8 = (a.BH + 7) / 8 * 8;
    hipError_t e;
    if (!WIN && a.cu && a.dk_prev && a.T > 0) {
        // packed: a sequence without steps has no tile whose workgroup would
        // write its halo gradient, so the halo rows start at zero
        const size_t n = (size_t)a.BH * a.W * D;
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           static_cast<bf*>(a.dk_prev), n);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_scan_kernel<D, CV, DELTA, WIN, COL>), dim3(bh8 * nvs), dim3(512), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.T > 0) {
        hipLaunchKernelGGL((bwd_grad_kernel<D, CV, DELTA, WIN, COL>), dim3(a.BH * a.ntiles), dim3(256), 0,
                           stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if constexpr (WIN) {
        // every key and value row, the halo rows included (also for T = 0)
        constexpr int RPB = 256 / (D / 8);
        const long long rows = (long long)a.BH * (a.T + a.W);
        hipLaunchKernelGGL((bwd_gather_kernel<D, CV>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                           stream, a);
        e = hipGetLastError();
    } else if (a.T == 0 && a.dk_prev) {
        const size_t n = (size_t)a.BH * a.W * D;
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           static_cast<bf*>(a.dk_prev), n);
        e = hipGetLastError();
    }
    return e;
}

template <int D>
static hipError_t launch_bwd_dd(const BwdArgs& a, bool delta, bool win, bool col, hipStream_t stream) {
    if (win)
        return delta ? launch_bwd_d<D, true, true, false>(a, stream) : launch_bwd_d<D, false, true, false>(a, stream);
    if (col)
        return delta ? launch_bwd_d<D, true, false, true>(a, stream) : launch_bwd_d<D, false, false, true>(a, stream);
    return delta ? launch_bwd_d<D, true, false, false>(a, stream) : launch_bwd_d<D, false, false, false>(a, stream);
}

hipError_t launch_chunk_bwd(const BwdArgs& a, int D, int chunk, bool delta, hipStream_t stream) {
    if (chunk != 64) return hipErrorInvalidValue;
    const bool win = a.W > 1, col = a.norm == kNormColumn;
    if (D == 64) return launch_bwd_dd<64>(a, delta, win, col, stream);
    if (D == 128) return launch_bwd_dd<128>(a, delta, win, col, stream);
    return hipErrorInvalidValue;
}

}  // namespace falcon
