// falcon_chunk.hip -- chunk-parallel forward pass of the Falcon recurrence
// on gfx950: an intra-chunk kernel (parallel over all tiles) and a
// state-passing kernel (sequential over the tiles of a sequence).
//
// Method ("Fast Weight Attention for Continual Learning", authors' abstract;
// step size and decay-then-delta order from the KLA abstract on the same
// listing): per (batch, head) the state S (d_v x d_k) is decayed by alpha_t,
// corrected towards the prefix-aligned example (x_t, y_t) = (k_{t-1}, v_t)
// with a normalized step, and read after the write, o_t = S_t q_t.  The
// abstract states that a chunk-parallel form exists with positive-decay
// renormalization; this file computes that form.
//
// Chunk algebra (per tile of CV "virtual rows"; a row is one (step s, window
// slot w) example with key x_i, target y_i and write vector omega_i = rs_i
// x_i, or u_i for the per-column rule; S0 is the state at the tile start,
// g_s the tile-local cumulative log decay, D(t,s) = exp(g_t - g_s)):
//   A[i,j] = [s(j) < s(i)] D(s(i),s(j)) (x_i . omega_j),   T = (I + A)^-1
//   P[t,j] = [s(j) <= t]   D(t,s(j))    (q_t . omega_j)
//   residuals   Delta = T (Y - diag(exp g_s(i)) X S0^T)
//               (inner-product family: Delta = Y, no system)
//   outputs     O = diag(exp g_t) Q S0^T + P Delta
//   next state  S = exp(g_last) S0 + sum_j D(last,s(j)) Delta_j omega_j^T
// Every decay factor is exp(later - earlier) <= 1 of a log sum that restarts
// at each tile, so nothing divides by a cumulative product and no tile can
// under- or overflow, whatever T is (the renormalization reading).
//
// Kernel 1, chunk_prep (one workgroup per (batch*head, tile), all tiles at
// once): stages the tile's keys and queries in LDS, scans the log decays,
// forms the Gram blocks on MFMA, masks and decays them, inverts I + A in fp32
// (16x16 diagonal blocks by forward substitution, then the off-diagonal
// blocks level by level) and writes T, P and per-row factors to a workspace
// record, already in the register order of the MFMA operand fragments that
// kernel 2 feeds them into.
//
// Kernel 2, chunk_scan (one workgroup of 4 waves per (batch*head, 64-wide
// slice of d_v), walking the tiles in order): the state slice lives in
// registers as MFMA accumulators of S^T (wave w owns 16 value columns), so it
// is the B operand of X S0^T and Q S0^T as it stands and is updated in place.
// Per tile the only sequential work is four small GEMM stages (X S0^T and
// Q S0^T, T R, P Delta, Omega^T Delta); the next tile's inputs are requested
// before the current tile's arithmetic starts.  Slices of one sequence are
// mapped to one XCD so the second slice's key and query reads hit its L2.
#include "falcon_device.h"
#include "falcon_internal.h"

namespace falcon {

// ---------------------------------------------------------------------------
// workspace record of one (batch*head, tile)
// ---------------------------------------------------------------------------
template <class E, int CV, bool DELTA>
struct Rec {
    static constexpr int NB = CV / 16;
    static constexpr int NBT = DELTA ? NB * (NB + 1) / 2 : 0;  // lower blocks of T
    static constexpr int NBP = NB * NB;                        // blocks of P
    static constexpr size_t kT = 0;                            // element offsets
    static constexpr size_t kP = (size_t)NBT * 256;
    static constexpr size_t kScalBytes = (size_t)(NBT + NBP) * 256 * E::kBytes;
    static constexpr int NSC = 5;  // gam, hrow, gq, l1, erow (CV floats each)
    static constexpr size_t kBytes = (kScalBytes + NSC * CV * 4 + 255) / 256 * 256;
    static __host__ __device__ constexpr int tblk(int b, int c) { return b * (b + 1) / 2 + c; }
};

static inline int tiles_of(int T, int Ct) { return (T + Ct - 1) / Ct; }

// ---------------------------------------------------------------------------
// shared helpers
// ---------------------------------------------------------------------------
struct TileGeom {
    int Wv, Ct, NVR, NBQ;
    __device__ TileGeom(const ChunkArgs& a, int CV) {
        Wv = (a.norm == kNormWindow) ? a.W : 1;
        Ct = CV / Wv;
        NVR = Ct * Wv;
        NBQ = (Ct + 15) / 16;
    }
};

// ---------------------------------------------------------------------------
// Kernel 1: intra-chunk preparation
// ---------------------------------------------------------------------------
template <class E, int D, int CV, bool COL>
struct PrepSmem {
    using T = typename E::T;
    static constexpr int PADE = 16 / E::kBytes;
    static constexpr int LDX = D + PADE;
    T X[CV][LDX];                       // keys x_i (virtual rows)
    union {
        T Q[CV][LDX];                   // queries, until P is formed
        float Tf[CV][CV + 1];           // then T = (I + A)^-1 in fp32
    } u;
    T Om[COL ? CV : 1][LDX];            // per-column write vectors
    float Af[CV][CV + 1];               // masked A in fp32
    float tmp[4][16][17];               // per-wave block-product scratch
    float nrm[CV], l1[CV], eta[CV], alpha[CV];
    float g[CV], rs[CV];
    int step[CV];
};

template <class E, int D, int CV, bool DELTA, bool COL>
__global__ __launch_bounds__(256) void chunk_prep_kernel(ChunkArgs a, void* ws, int ntiles) {
    using T = typename E::T;
    using R = Rec<E, CV, DELTA>;
    constexpr int NB = CV / 16;
    constexpr int EPC = 16 / E::kBytes;
    constexpr int CPR = D / EPC;
    constexpr int NXL = (CV * CPR + 255) / 256;
    constexpr int NJA = DELTA ? NB * (NB + 1) / 2 : 0;
    constexpr int NJ = NJA + NB * NB;
    __shared__ PrepSmem<E, D, CV, COL> sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    const int bh = blockIdx.x / ntiles;
    const int tile = blockIdx.x - bh * ntiles;
    const TileGeom G(a, CV);
    const int Wv = G.Wv, Ct = G.Ct, NVR = G.NVR, NBQ = G.NBQ, W = a.W;
    const int T_ = a.T;
    const int t0 = tile * Ct;
    const float eps = a.eps;
    const T* qg = static_cast<const T*>(a.q) + (size_t)bh * T_ * D;
    const T* kg = static_cast<const T*>(a.k) + (size_t)bh * T_ * D;
    const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
    char* rec = static_cast<char*>(ws) + ((size_t)bh * ntiles + tile) * R::kBytes;
    T* recT = reinterpret_cast<T*>(rec);
    float* recS = reinterpret_cast<float*>(rec + R::kScalBytes);

    // ---- stage keys (virtual rows) and queries ----
    const uint4 z16 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int it = 0; it < NXL; ++it) {
        const int c = tid + 256 * it;
        if (c >= CV * CPR) continue;
        const int i = c / CPR, col = (c % CPR) * EPC;
        const int s = i / Wv, w = i - s * Wv;
        const int t = t0 + s, tau = t - w - 1;  // x_i = k_{t-w-1}
        uint4 xv = z16, qv = z16;
        if (i < NVR && t < T_) {
            if (tau >= 0) xv = *reinterpret_cast<const uint4*>(kg + (size_t)tau * D + col);
            else if (kp) xv = *reinterpret_cast<const uint4*>(kp + (size_t)(W + tau) * D + col);
        }
        if (i < Ct && t0 + i < T_)
            qv = *reinterpret_cast<const uint4*>(qg + (size_t)(t0 + i) * D + col);
        *reinterpret_cast<uint4*>(&sm.X[i][col]) = xv;
        *reinterpret_cast<uint4*>(&sm.u.Q[i][col]) = qv;
    }
    if (tid < CV) {
        const int t = t0 + tid;
        const bool ok = tid < Ct && t < T_;
        sm.alpha[tid] = ok ? a.alpha[(size_t)bh * T_ + t] : 1.f;  // padding steps: identity
        sm.eta[tid] = ok ? a.eta[(size_t)bh * T_ + t] : 0.f;
    }
    __syncthreads();

    // ---- norms (4 threads per row) ----
    {
        const int i = tid >> 2, part = tid & 3;
        float n2 = 0.f, n1 = 0.f;
        if (i < CV) {
#pragma unroll 8
            for (int c = part * (D / 4); c < (part + 1) * (D / 4); ++c) {
                const float x = E::to_f(sm.X[i][c]);
                n2 += x * x;
                n1 += fabsf(x);
            }
        }
        n2 = group_sum<4>(n2);
        n1 = group_sum<4>(n1);
        if (i < CV && part == 0) {
            sm.nrm[i] = n2;
            sm.l1[i] = n1;
        }
    }
    __syncthreads();

    // ---- log-decay scan and row factors (wave 0) ----
    if (wave == 0) {
        const int j = lane;
        float lg = (j < Ct) ? logf(sm.alpha[j]) : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(lg, off, 64);
            if (j >= off) lg += y;
        }
        const float glast = __shfl(lg, Ct - 1, 64);
        float bwin = 0.f;  // window normalizer b_s (lane s)
        if (a.norm == kNormWindow && j < Ct) {
            float tot = 0.f;
            for (int w = 0; w < Wv; ++w) tot += sm.nrm[j * Wv + w];
            const float den = tot + eps;
            bwin = den > 0.f ? sm.eta[j] / den : 0.f;
        }
        const int sj = min(j / Wv, Ct - 1);
        const float gsj = __shfl(lg, sj, 64);
        const float bsj = __shfl(bwin, sj, 64);
        if (j < CV) {
            float r = 0.f;
            if (j < NVR) {
                if (a.norm == kNormScalar) {
                    const float den = sm.nrm[j] + eps;
                    r = den > 0.f ? sm.eta[sj] / den : 0.f;
                } else if (a.norm == kNormColumn) {
                    r = 1.f;
                } else {
                    r = bsj;
                }
            }
            sm.g[j] = lg;
            sm.rs[j] = r;
            sm.step[j] = sj;
            recS[0 * CV + j] = __expf(gsj);               // gam
            recS[1 * CV + j] = __expf(glast - gsj) * r;   // hrow
            recS[2 * CV + j] = __expf(lg);                // gq
            recS[3 * CV + j] = sm.l1[j];                  // l1
            recS[4 * CV + j] = (j < NVR) ? sm.eta[sj] : 0.f;  // erow
        }
    }
    if constexpr (COL) {
        // u_j = eta x_j / (|x_j| ||x||_1 + eps)
        for (int c = tid; c < CV * D; c += 256) {
            const int i = c / D, col = c % D;
            const int s = min(i / Wv, Ct - 1);
            const float x = E::to_f(sm.X[i][col]);
            const float den = fabsf(x) * sm.l1[i] + eps;
            sm.Om[i][col] = E::from_f((i < NVR && den > 0.f) ? sm.eta[s] * x / den : 0.f);
        }
    }
    __syncthreads();

    // ---- Gram blocks, masked and decayed: A -> LDS (fp32), P -> record ----
    for (int q = wave; q < NJ; q += 4) {
        const bool isA = q < NJA;
        int bi, bj;
        if (isA) {
            bi = 0;
            while ((bi + 1) * (bi + 2) / 2 <= q) ++bi;
            bj = q - bi * (bi + 1) / 2;
        } else {
            bi = (q - NJA) / NB;
            bj = (q - NJA) % NB;
        }
        const bool live = isA || (bi < NBQ && (16 * bj) / Wv <= 16 * bi + 15);
        const T* omb = COL ? &sm.Om[0][0] : &sm.X[0][0];
        f32x4 acc = zero4();
        if (isA) {
            // A block (bi, bj): rows x_i (A operand), columns omega_j (B operand)
            const T* ar = &sm.X[16 * bi + lr][0];
            const T* br = omb + (size_t)(16 * bj + lr) * PrepSmem<E, D, CV, COL>::LDX;
#pragma unroll
            for (int m = 0; m < D / 32; ++m)
                acc = E::mma32(E::load(ar + 32 * m + 4 * grp), E::load(ar + 32 * m + 16 + 4 * grp),
                               E::load(br + 32 * m + 4 * grp), E::load(br + 32 * m + 16 + 4 * grp),
                               acc);
            const int j = 16 * bj + lr;
            const int sj = sm.step[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * bi + 4 * grp + r;
                const int si = sm.step[i];
                sm.Af[i][j] = (sj < si) ? __expf(sm.g[si] - sm.g[sj]) * acc[r] * sm.rs[j] : 0.f;
            }
        } else {
            // P^T block: rows omega_j (A operand), columns q_t (B operand), so the
            // accumulator is P in the A-fragment order kernel 2 reads
            T* dst = recT + R::kP + (size_t)(bi * NB + bj) * 256 + lane * 4;
            if (!live) {
                *reinterpret_cast<typename E::Frag*>(dst) = E::pack(zero4());
                continue;
            }
            const T* ar = omb + (size_t)(16 * bj + lr) * PrepSmem<E, D, CV, COL>::LDX;
            const T* br = &sm.u.Q[16 * bi + lr][0];
#pragma unroll
            for (int m = 0; m < D / 32; ++m)
                acc = E::mma32(E::load(ar + 32 * m + 4 * grp), E::load(ar + 32 * m + 16 + 4 * grp),
                               E::load(br + 32 * m + 4 * grp), E::load(br + 32 * m + 16 + 4 * grp),
                               acc);
            const int t = 16 * bi + lr;
            f32x4 pv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * bj + 4 * grp + r;
                const int sj = sm.step[j];
                pv[r] = (sj <= t && t < Ct) ? __expf(sm.g[t] - sm.g[sj]) * acc[r] * sm.rs[j] : 0.f;
            }
            *reinterpret_cast<typename E::Frag*>(dst) = E::pack(pv);
        }
    }
    if constexpr (!DELTA) return;
    __syncthreads();

    // ---- T = (I + A)^-1: diagonal blocks by forward substitution ----
    if (wave < NB && lane < 16) {
        const int b = wave, c = lane;
        float tcol[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) acc -= sm.Af[16 * b + i][16 * b + j] * tcol[j];
            tcol[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.u.Tf[16 * b + i][16 * b + c] = tcol[i];
    }
    __syncthreads();
    // off-diagonal blocks, level L = b - c: T_bc = -T_bb sum_{k=c}^{b-1} A_bk T_kc
    for (int L = 1; L < NB; ++L) {
        const int b = L + wave, c = wave;  // wave w takes block (L + w, w)
        const bool act = b < NB;
        const int i = lane >> 2, j0 = (lane & 3) * 4;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        if (act) {
            for (int k = c; k < b; ++k)
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    const float av = sm.Af[16 * b + i][16 * k + kk];
#pragma unroll
                    for (int e = 0; e < 4; ++e) s4[e] += av * sm.u.Tf[16 * k + kk][16 * c + j0 + e];
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.tmp[wave][i][j0 + e] = s4[e];
        }
        __syncthreads();
        if (act) {
            float t4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const float tv = sm.u.Tf[16 * b + i][16 * b + kk];
#pragma unroll
                for (int e = 0; e < 4; ++e) t4[e] -= tv * sm.tmp[wave][kk][j0 + e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.u.Tf[16 * b + i][16 * c + j0 + e] = t4[e];
        }
        __syncthreads();
    }
    // ---- T blocks to the record in A-fragment order ----
    for (int q = wave; q < R::NBT; q += 4) {
        int b = 0;
        while ((b + 1) * (b + 2) / 2 <= q) ++b;
        const int c = q - b * (b + 1) / 2;
        f32x4 tv;
#pragma unroll
        for (int r = 0; r < 4; ++r) tv[r] = sm.u.Tf[16 * b + lr][16 * c + 4 * grp + r];
        *reinterpret_cast<typename E::Frag*>(recT + R::kT + (size_t)q * 256 + lane * 4) =
            E::pack(tv);
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: state pass
// ---------------------------------------------------------------------------
template <class E, int D, int CV, bool DELTA, bool COL>
struct ScanSmem {
    using T = typename E::T;
    using R = Rec<E, CV, DELTA>;
    static constexpr int PADE = 16 / E::kBytes;
    static constexpr int LDX = D + PADE;
    T X[CV][LDX];               // keys x_i (virtual rows)
    T Q[CV][LDX];               // queries q_t
    T Om[COL ? CV : 1][LDX];    // per-column write vectors u_i
    T Y[CV][64 + PADE];         // targets y_i, this workgroup's 64 value columns
    alignas(16) char rec[R::kBytes];  // this tile's record (T, P, row factors)
};

template <class E, int D, int CV, bool DELTA, bool COL>
__global__ __launch_bounds__(256) void chunk_scan_kernel(ChunkArgs a, const void* ws,
                                                         int ntiles) {
    using T = typename E::T;
    using Frag = typename E::Frag;
    using R = Rec<E, CV, DELTA>;
    using Smem = ScanSmem<E, D, CV, DELTA, COL>;
    constexpr int NB = CV / 16;
    constexpr int KB = D / 16;
    constexpr int EPC = 16 / E::kBytes;
    constexpr int CPR = D / EPC;
    constexpr int NXL = (CV * CPR + 255) / 256;
    constexpr int YCPR = 64 / EPC;
    constexpr int NYL = (CV * YCPR + 255) / 256;
    constexpr int RCH = (int)(R::kBytes / 16);           // 16-byte chunks of a record
    constexpr int NRL = (RCH + 255) / 256;
    constexpr int NVS = D / 64;
    constexpr int LDX = Smem::LDX;
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    // XCD-aware mapping: workgroup i runs on XCD i % 8; keep the slices of a
    // sequence on one XCD.
    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int jj = blk >> 3;
    const int bh = (jj / NVS) * 8 + xcd;
    const int vs = jj % NVS;
    if (bh >= a.BH) return;
    const int v0 = vs * 64;

    const TileGeom G(a, CV);
    const int Wv = G.Wv, Ct = G.Ct, NVR = G.NVR, NBQ = G.NBQ, W = a.W;
    const int T_ = a.T;
    const float eps = a.eps;
    const T* qg = static_cast<const T*>(a.q) + (size_t)bh * T_ * D;
    const T* kg = static_cast<const T*>(a.k) + (size_t)bh * T_ * D;
    const T* vg = static_cast<const T*>(a.v) + (size_t)bh * T_ * D;
    const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
    const T* vp = (a.v_prev && W > 1) ? static_cast<const T*>(a.v_prev) + (size_t)bh * (W - 1) * D
                                      : nullptr;
    const char* recg = static_cast<const char*>(ws) + (size_t)bh * ntiles * R::kBytes;
    T* og = static_cast<T*>(a.o) + (size_t)bh * T_ * D;

    // State slice as accumulators of S^T: Sacc[kb][r] = S[v][k],
    // v = v0 + 16*wave + lr, k = 16*kb + 4*grp + r.
    const int vcol = v0 + 16 * wave + lr;
    f32x4 Sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
        Sacc[kb] = a.S0 ? *reinterpret_cast<const f32x4*>(a.S0 + ((size_t)bh * D + vcol) * D +
                                                          16 * kb + 4 * grp)
                        : zero4();

    // per-thread load geometry (fixed across tiles)
    uint4 px[NXL], pq[NXL], py[NYL], pr[NRL];
    float pl1[COL ? NXL : 1], per[COL ? NXL : 1];

    auto load_tile = [&](int tile) __attribute__((always_inline)) {
        const int t0 = tile * Ct;
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int c = tid + 256 * it;
            const int i = c / CPR, col = (c % CPR) * EPC;
            const int s = i / Wv, w = i - s * Wv;
            const int t = t0 + s, tau = t - w - 1;
            px[it] = make_uint4(0, 0, 0, 0);
            pq[it] = make_uint4(0, 0, 0, 0);
            if (c < CV * CPR) {
                if (i < NVR && t < T_) {
                    if (tau >= 0) px[it] = *reinterpret_cast<const uint4*>(kg + (size_t)tau * D + col);
                    else if (kp)
                        px[it] = *reinterpret_cast<const uint4*>(kp + (size_t)(W + tau) * D + col);
                }
                if (i < Ct && t0 + i < T_)
                    pq[it] = *reinterpret_cast<const uint4*>(qg + (size_t)(t0 + i) * D + col);
                if constexpr (COL) {
                    const float* sc = reinterpret_cast<const float*>(
                        recg + (size_t)tile * R::kBytes + R::kScalBytes);
                    pl1[it] = sc[3 * CV + i];
                    per[it] = sc[4 * CV + i];
                }
            }
        }
#pragma unroll
        for (int it = 0; it < NYL; ++it) {
            const int c = tid + 256 * it;
            const int i = c / YCPR, col = (c % YCPR) * EPC;
            const int s = i / Wv, w = i - s * Wv;
            const int t = t0 + s, tv = t - w;  // y_i = v_{t-w}
            py[it] = make_uint4(0, 0, 0, 0);
            if (c < CV * YCPR && i < NVR && t < T_) {
                if (tv >= 0) py[it] = *reinterpret_cast<const uint4*>(vg + (size_t)tv * D + v0 + col);
                else if (vp)
                    py[it] = *reinterpret_cast<const uint4*>(vp + (size_t)(W - 1 + tv) * D + v0 + col);
            }
        }
        const uint4* rg = reinterpret_cast<const uint4*>(recg + (size_t)tile * R::kBytes);
#pragma unroll
        for (int it = 0; it < NRL; ++it) {
            const int c = tid + 256 * it;
            pr[it] = (c < RCH) ? rg[c] : make_uint4(0, 0, 0, 0);
        }
    };

    auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int c = tid + 256 * it;
            if (c >= CV * CPR) continue;  // (no break: the loop must unroll fully)
            const int i = c / CPR, col = (c % CPR) * EPC;
            *reinterpret_cast<uint4*>(&sm.X[i][col]) = px[it];
            *reinterpret_cast<uint4*>(&sm.Q[i][col]) = pq[it];
            if constexpr (COL) {
                const T* e = reinterpret_cast<const T*>(&px[it]);
                T out[EPC];
#pragma unroll
                for (int u = 0; u < EPC; ++u) {
                    const float x = E::to_f(e[u]);
                    const float den = fabsf(x) * pl1[it] + eps;
                    out[u] = E::from_f(den > 0.f ? per[it] * x / den : 0.f);
                }
                *reinterpret_cast<uint4*>(&sm.Om[i][col]) = *reinterpret_cast<const uint4*>(out);
            }
        }
#pragma unroll
        for (int it = 0; it < NYL; ++it) {
            const int c = tid + 256 * it;
            if (c < CV * YCPR) *reinterpret_cast<uint4*>(&sm.Y[c / YCPR][(c % YCPR) * EPC]) = py[it];
        }
#pragma unroll
        for (int it = 0; it < NRL; ++it) {
            const int c = tid + 256 * it;
            if (c < RCH) reinterpret_cast<uint4*>(sm.rec)[c] = pr[it];
        }
    };

    const int ntl = ntiles;
    if (ntl > 0) load_tile(0);
    for (int tile = 0; tile < ntl; ++tile) {
        const int t0 = tile * Ct;
        store_tile();
        __syncthreads();
        if (tile + 1 < ntl) load_tile(tile + 1);  // in flight during this tile's arithmetic

        const T* recT = reinterpret_cast<const T*>(sm.rec);
        const float* gam = reinterpret_cast<const float*>(sm.rec + R::kScalBytes);
        const float* hrow = gam + CV;
        const float* gq = gam + 2 * CV;

        Frag SB[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) SB[kb] = E::pack(Sacc[kb]);

        // Z = X S0^T (virtual rows) and Zq = Q S0^T
        f32x4 Dl[NB];
        Frag DB[NB];
        if (DELTA) {
            f32x4 Rr[NB];
            Frag RB[NB];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                f32x4 acc = zero4();
                const T* ar = &sm.X[16 * rb + lr][0];
#pragma unroll
                for (int m = 0; m < D / 32; ++m)
                    acc = E::mma32(E::load(ar + 32 * m + 4 * grp), E::load(ar + 32 * m + 16 + 4 * grp),
                                   SB[2 * m], SB[2 * m + 1], acc);
                const f32x4 gm = *reinterpret_cast<const f32x4*>(gam + 16 * rb + 4 * grp);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Rr[rb][r] = E::to_f(sm.Y[16 * rb + 4 * grp + r][16 * wave + lr]) - gm[r] * acc[r];
                RB[rb] = E::pack(Rr[rb]);
            }
            // Delta = T R (T lower triangular in 16-blocks)
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                f32x4 acc = zero4();
#pragma unroll
                for (int cb = 0; cb <= rb; ++cb)
                    acc = E::mma16(E::load(recT + R::kT + (size_t)R::tblk(rb, cb) * 256 + lane * 4),
                                   RB[cb], acc);
                Dl[rb] = acc;
                DB[rb] = E::pack(acc);
            }
        } else {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Dl[rb][r] = E::to_f(sm.Y[16 * rb + 4 * grp + r][16 * wave + lr]);
                DB[rb] = E::pack(Dl[rb]);
            }
        }

        // outputs O = diag(gq) Q S0^T + P Delta
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            if (tb >= NBQ) continue;
            f32x4 acc = zero4();
            const T* ar = &sm.Q[16 * tb + lr][0];
#pragma unroll
            for (int m = 0; m < D / 32; ++m)
                acc = E::mma32(E::load(ar + 32 * m + 4 * grp), E::load(ar + 32 * m + 16 + 4 * grp),
                               SB[2 * m], SB[2 * m + 1], acc);
            const f32x4 gqv = *reinterpret_cast<const f32x4*>(gq + 16 * tb + 4 * grp);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= gqv[r];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if ((16 * cb) / Wv > 16 * tb + 15) continue;
                acc = E::mma16(E::load(recT + R::kP + (size_t)(tb * NB + cb) * 256 + lane * 4),
                               DB[cb], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tb + 4 * grp + r;
                if (t < Ct && t0 + t < T_) og[(size_t)(t0 + t) * D + vcol] = E::from_f(acc[r]);
            }
        }

        // state update S^T = exp(g_last) S0^T + Omega^T diag(hrow) Delta; the A
        // operand Omega^T is read column-wise from the row-major tile
        Frag HB[NB];
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
            const f32x4 hv = *reinterpret_cast<const f32x4*>(hrow + 16 * cb + 4 * grp);
            f32x4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = hv[r] * Dl[cb][r];
            HB[cb] = E::pack(h);
        }
        const float glq = gq[Ct - 1];
        const T* om;
        if constexpr (COL) om = &sm.Om[0][0];
        else om = &sm.X[0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x4 acc = Sacc[kb] * glq;
            const T* col = om + 16 * kb + lr;
            if constexpr (NB == 1) {
                acc = E::mma16(E::gather4(col + (4 * grp) * LDX, LDX), HB[0], acc);
            } else {
#pragma unroll
                for (int m = 0; m < NB / 2; ++m)
                    acc = E::mma32(E::gather4(col + (32 * m + 4 * grp) * LDX, LDX),
                                   E::gather4(col + (32 * m + 16 + 4 * grp) * LDX, LDX), HB[2 * m],
                                   HB[2 * m + 1], acc);
            }
            Sacc[kb] = acc;
        }
        __syncthreads();  // LDS is restaged by the next tile
    }

    if (a.S_final) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            *reinterpret_cast<f32x4*>(a.S_final + ((size_t)bh * D + vcol) * D + 16 * kb + 4 * grp) =
                Sacc[kb];
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <class E, int D, int CV, bool DELTA, bool COL>
static hipError_t launch_one(const ChunkArgs& a, void* ws, hipStream_t stream) {
    const int Wv = (a.norm == kNormWindow) ? a.W : 1;
    const int ntiles = tiles_of(a.T, CV / Wv);
    if (ntiles > 0) {
        hipLaunchKernelGGL((chunk_prep_kernel<E, D, CV, DELTA, COL>), dim3(a.BH * ntiles),
                           dim3(256), 0, stream, a, ws, ntiles);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nvs = D / 64;
    const int bh8 = (a.BH + 7) / 8 * 8;
    hipLaunchKernelGGL((chunk_scan_kernel<E, D, CV, DELTA, COL>), dim3(bh8 * nvs), dim3(256), 0,
                       stream, a, (const void*)ws, ntiles);
    return hipGetLastError();
}

template <class E, int D, bool DELTA, bool COL>
static hipError_t launch_cv(const ChunkArgs& a, int chunk, void* ws, hipStream_t stream) {
    switch (chunk) {
        case 16: return launch_one<E, D, 16, DELTA, COL>(a, ws, stream);
        case 32: return launch_one<E, D, 32, DELTA, COL>(a, ws, stream);
        case 64:
            if constexpr (D == 64 || E::kBytes == 2)
                return launch_one<E, D, 64, DELTA, COL>(a, ws, stream);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <class E, bool DELTA, bool COL>
static hipError_t launch_d(const ChunkArgs& a, int D, int chunk, void* ws, hipStream_t stream) {
    if (D == 64) return launch_cv<E, 64, DELTA, COL>(a, chunk, ws, stream);
    if (D == 128) return launch_cv<E, 128, DELTA, COL>(a, chunk, ws, stream);
    return hipErrorInvalidValue;
}

template <class E>
static hipError_t launch_e(const ChunkArgs& a, int D, int chunk, bool delta, void* ws,
                           hipStream_t stream) {
    const bool col = a.norm == kNormColumn;
    if (delta)
        return col ? launch_d<E, true, true>(a, D, chunk, ws, stream)
                   : launch_d<E, true, false>(a, D, chunk, ws, stream);
    return col ? launch_d<E, false, true>(a, D, chunk, ws, stream)
               : launch_d<E, false, false>(a, D, chunk, ws, stream);
}

bool chunk_supported(int dt, int D, int chunk) {
    if (D != 64 && D != 128) return false;
    if (chunk != 16 && chunk != 32 && chunk != 64) return false;
    if (chunk == 64 && dt == 0 && D == 128) return false;  // fp32 tiles of 64 x 128 exceed LDS
    return true;
}

template <class E, int CV, bool DELTA>
static size_t rec_bytes() {
    return Rec<E, CV, DELTA>::kBytes;
}

size_t chunk_workspace_bytes(int BH, int T, int dt, int chunk, int window, int norm, bool delta) {
    const int Wv = (norm == kNormWindow) ? window : 1;
    const int ntiles = tiles_of(T, chunk / Wv);
    size_t rb = 0;
    if (dt == 1) {
        if (chunk == 16) rb = delta ? rec_bytes<EBf16, 16, true>() : rec_bytes<EBf16, 16, false>();
        if (chunk == 32) rb = delta ? rec_bytes<EBf16, 32, true>() : rec_bytes<EBf16, 32, false>();
        if (chunk == 64) rb = delta ? rec_bytes<EBf16, 64, true>() : rec_bytes<EBf16, 64, false>();
    } else {
        if (chunk == 16) rb = delta ? rec_bytes<EFp32, 16, true>() : rec_bytes<EFp32, 16, false>();
        if (chunk == 32) rb = delta ? rec_bytes<EFp32, 32, true>() : rec_bytes<EFp32, 32, false>();
        if (chunk == 64) rb = delta ? rec_bytes<EFp32, 64, true>() : rec_bytes<EFp32, 64, false>();
    }
    return (size_t)BH * ntiles * rb;
}

hipError_t launch_chunk(const ChunkArgs& a, int dt, int D, int chunk, bool delta, void* ws,
                        hipStream_t stream) {
    if (dt == 1) return launch_e<EBf16>(a, D, chunk, delta, ws, stream);
    return launch_e<EFp32>(a, D, chunk, delta, ws, stream);
}

}  // namespace falcon
