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
//   A[i,j] = [s(j) < s(i)] D(s(i),s(j)) (x_i . omega_j)
//   P[t,j] = [s(j) <= t]   D(t,s(j))    (q_t . omega_j)
//   residuals   (I + A) Delta = Y - diag(exp g_s(i)) X S0^T
//               (inner-product family: Delta = Y, no system)
//   outputs     O = diag(exp g_t) Q S0^T + P Delta
//   next state  S = exp(g_last) S0 + sum_j D(last,s(j)) Delta_j omega_j^T
// Every decay factor is exp(later - earlier) <= 1 of a log sum that restarts
// at each tile, so nothing divides by a cumulative product and no tile can
// under- or overflow, whatever T is (the renormalization reading).
//
// Kernel 1, chunk_prep (one workgroup per (batch*head, tile), all tiles at
// once): stages the tile's keys and queries in LDS, scans the log decays,
// forms the Gram blocks on MFMA with the operands ordered so that each
// accumulator already is the operand fragment kernel 2 needs, masks and
// decays them, inverts the 16 x 16 diagonal blocks of I + A in fp32, and
// writes -A (strictly lower blocks), the diagonal inverses, P and per-row
// factors to a workspace record.
//
// Kernel 2, chunk_scan (one workgroup of 4 waves per (batch*head, 64-wide
// slice of d_v), walking the tiles in order): the state slice lives in
// registers as MFMA accumulators of S^T (wave w owns 16 value columns), so it
// is the B operand of X S0^T and Q S0^T as it stands and is updated in place.
// Per tile: X S0^T, the residuals, a blocked forward substitution
// Delta_b = Td_b (R_b - sum_{c<b} A_bc Delta_c), P Delta, the state update.
// Addresses of the loads are fixed per thread and computed once; loads are
// unconditional (clamped address, zero select), the next tile's loads are in
// flight during the current tile's arithmetic, and outputs leave through LDS
// as 16-byte stores.  Slices of one sequence are mapped to one XCD so the
// second slice's key and query reads hit that XCD's L2.
#include "falcon_device.h"
#include "falcon_internal.h"
#include "falcon_records.h"
#include "falcon_rows.h"

namespace falcon {


constexpr int kCuLds = 4096;  // offsets the schedule kernel copies to LDS

// Packed calls, before the kernels: in one workgroup,
//  * order[i]: sequence indices by tile count, longest first (a counting sort
//    in LDS bins; the order within a bin is immaterial, since no sequence's
//    result depends on when it runs), for the state pass;
//  * toff[n]: exclusive prefix sums of the tile counts in sequence order
//    (toff[N] = all tiles), so the intra-chunk kernel schedules only the
//    tiles that exist.
__global__ __launch_bounds__(1024) void packed_schedule_kernel(ChunkArgs a, int Ct, int nbins,
                                                               int* order, int* toff, int* jobs) {
    // LDS: nbins bins, one partial sum per thread, the total, then (up to
    // kCuLds entries) a copy of the offsets
    extern __shared__ int bins[];
    int* part = bins + nbins;
    int* cul = part + blockDim.x + 1;
    const int N = a.BH / a.H, tid = threadIdx.x, nt = blockDim.x;
    const bool in_lds = N + 1 <= kCuLds;
    for (int b = tid; b < nbins; b += nt) bins[b] = 0;
    if (in_lds)
        for (int i = tid; i <= N; i += nt) cul[i] = a.cu[i];
    __syncthreads();
    // sequence n's rows in head 0's plane (its start is the same in every plane)
    auto seq_rows = [&](const ChunkArgs&, int bh) {
        const int n = bh / a.H;
        return in_lds ? rows_of(a, 0, cul[n], cul[n + 1]) : rows_of(a, 0, a.cu[n], a.cu[n + 1]);
    };
    for (int n = tid; n < N; n += nt)
        atomicAdd(&bins[min(tiles_of(seq_rows(a, n * a.H).T, Ct), nbins - 1)], 1);
    // prefix sums of tile counts: thread t owns sequences [t*per, (t+1)*per)
    const int per = (N + nt - 1) / nt;
    const int n0 = min(tid * per, N), n1 = min(n0 + per, N);
    int sum = 0;
    for (int n = n0; n < n1; ++n) sum += tiles_of(seq_rows(a, n * a.H).T, Ct);
    part[tid] = sum;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int b = nbins - 1; b >= 0; --b) {
            const int c = bins[b];
            bins[b] = acc;
            acc += c;
        }
        acc = 0;
        const int nparts = per > 0 ? (N + per - 1) / per : 0;  // threads that own sequences
        for (int t = 0; t < nparts; ++t) {
            const int c = part[t];
            part[t] = acc;
            acc += c;
        }
        part[nt] = acc;  // all tiles
        toff[N] = acc;
    }
    __syncthreads();
    for (int n = tid; n < N; n += nt)
        order[atomicAdd(&bins[min(tiles_of(seq_rows(a, n * a.H).T, Ct), nbins - 1)], 1)] = n;
    // the job table, j = h * G + g: (row, tile, sequence start, length); head
    // 0's row0 is the sequence's start in every plane
    const int Gall = part[nt];
    auto put = [&](int n, const SeqRows& sr, int g0, int h, int tile) {
        int* e = jobs + 4 * ((size_t)h * Gall + g0 + tile);
        e[0] = n * a.H + h;
        e[1] = tile;
        e[2] = (int)sr.row0;
        e[3] = sr.T;
    };
    int acc = part[tid];
    for (int n = n0; n < n1; ++n) {
        toff[n] = acc;
        const SeqRows sr = seq_rows(a, n * a.H);
        const int ntl = tiles_of(sr.T, Ct);
        if (N >= nt)  // enough sequences: each thread fills its own
            for (int h = 0; h < a.H; ++h)
                for (int tile = 0; tile < ntl; ++tile) put(n, sr, acc, h, tile);
        acc += ntl;
    }
    if (N < nt) {  // few sequences: all threads fill each one
        int g0 = 0;
        for (int n = 0; n < N; ++n) {
            const SeqRows sr = seq_rows(a, n * a.H);
            const int ntl = tiles_of(sr.T, Ct);
            for (int e = tid; e < a.H * ntl; e += nt) put(n, sr, g0, e / ntl, e - (e / ntl) * ntl);
            g0 += ntl;
        }
    }
}

__device__ __forceinline__ u32x4 sel16(bool ok, u32x4 v) {
    return ok ? v : u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Kernel 1: intra-chunk preparation
// ---------------------------------------------------------------------------
template <class E, int D, int CV, bool COL>
struct PrepSmem {
    using T = typename E::T;
    static constexpr int PADE = 16 / E::kBytes;
    static constexpr int LDX = D + PADE;
    T X[CV][LDX];                       // keys x_i (virtual rows)
    T Q[CV][LDX];                       // queries q_t
    T Om[COL ? CV : 1][LDX];            // per-column write vectors
    float Adg[CV / 16][16][17];         // fp32 diagonal blocks of A, then their inverses
    float nrm[CV], l1[CV], eta[CV], alpha[CV];
    float g[CV], rs[CV];
    int step[CV];
};

template <class E, int D, int CV, bool DELTA, bool COL, bool WIN>
__global__ __launch_bounds__(256) void chunk_prep_kernel(ChunkArgs a, void* ws, int ntiles) {
    using T = typename E::T;
    using Frag = typename E::Frag;
    using R = Rec<E, CV, DELTA>;
    using Smem = PrepSmem<E, D, CV, COL>;
    constexpr int NB = CV / 16;
    constexpr int EPC = 16 / E::kBytes;
    constexpr int CPR = D / EPC;
    constexpr int NXL = (CV * CPR + 255) / 256;
    constexpr int LDX = Smem::LDX;
    constexpr int NJA = DELTA ? NB * (NB + 1) / 2 : 0;  // A blocks incl. diagonal
    constexpr int NJ = NJA + NB * NB;
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    const int bh = blockIdx.x / ntiles;
    const int tile = blockIdx.x - bh * ntiles;
    const int W = a.W;
    const int Wv = WIN ? W : 1;
    const int Ct = CV / Wv, NVR = Ct * Wv, NBQ = (Ct + 15) / 16;
    const SeqRows sr = seq_rows(a, bh);
    const int T_ = sr.T;
    if (tile >= tiles_of(T_, Ct)) return;  // a shorter packed sequence: never read
    const int t0 = tile * Ct;
    const float eps = a.eps;
    const T* qg = static_cast<const T*>(a.q) + sr.row0 * D;
    const T* kg = static_cast<const T*>(a.k) + sr.row0 * D;
    const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
    char* rec = static_cast<char*>(ws) + ((size_t)bh * ntiles + tile) * R::kBytes;
    T* recT = reinterpret_cast<T*>(rec);
    float* recS = reinterpret_cast<float*>(rec + R::kScalBytes);

    // ---- stage keys (virtual rows) and queries, with the feature map; with a
    // map, also write the mapped keys, halo keys and queries for the state pass
    T* kq = a.phi ? static_cast<T*>(a.kphi) + mapped_row0(a, bh) * D : nullptr;
    T* qq = a.phi ? static_cast<T*>(a.qphi) + mapped_row0(a, bh) * D : nullptr;
    T* kpq = (a.phi && a.kpphi) ? static_cast<T*>(a.kpphi) + (size_t)bh * W * D : nullptr;
#pragma unroll
    for (int it = 0; it < NXL; ++it) {
        const int c = tid + 256 * it;
        const bool in = c < CV * CPR;
        const int i = (in ? c : 0) / CPR, col = ((in ? c : 0) % CPR) * EPC;
        const int s = WIN ? i / Wv : i, w = WIN ? i - s * Wv : 0;
        const int t = t0 + s, tau = t - w - a.lag;  // x_i = k_{t-w-lag}
        const bool okx = in && i < NVR && t < T_ && (tau >= 0 || kp != nullptr);
        const T* px = tau >= 0 ? kg + (size_t)tau * D + col
                               : (kp ? kp + (size_t)(W + tau) * D + col : kg + col);
        const bool okq = in && i < Ct && t0 + i < T_;
        const T* pq = okq ? qg + (size_t)(t0 + i) * D + col : qg + col;
        u32x4 xv = sel16(okx, *reinterpret_cast<const u32x4*>(okx ? px : kg + col));
        u32x4 qv = sel16(okq, *reinterpret_cast<const u32x4*>(pq));
        xv = phi_piece<E, CPR>(a.phi, xv);  // every lane: the row norm is a group sum
        qv = phi_piece<E, CPR>(a.phi, qv);
        if (in) {
            *reinterpret_cast<u32x4*>(&sm.X[i][col]) = xv;
            *reinterpret_cast<u32x4*>(&sm.Q[i][col]) = qv;
        }
        if (a.phi) {
            if (okx && tau >= 0) *reinterpret_cast<u32x4*>(kq + (size_t)tau * D + col) = xv;
            else if (okx && kpq) *reinterpret_cast<u32x4*>(kpq + (size_t)(W + tau) * D + col) = xv;
            if (okq) *reinterpret_cast<u32x4*>(qq + (size_t)(t0 + i) * D + col) = qv;
        }
    }
    if (tid < CV) {
        const int t = t0 + tid;
        const bool ok = tid < Ct && t < T_;
        sm.alpha[tid] = ok ? a.alpha[sr.row0 + t] : 1.f;  // padding steps: identity
        sm.eta[tid] = ok ? a.eta[sr.row0 + t] : 0.f;
    }
    __syncthreads();

    // ---- norms: 4 threads per row, 16-byte LDS reads ----
    {
        const int i = tid >> 2, part = tid & 3;
        float n2 = 0.f, n1 = 0.f;
        if (i < CV) {
#pragma unroll
            for (int c = 0; c < D / 4; c += EPC) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.X[i][part * (D / 4) + c]);
                const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
                for (int u = 0; u < EPC; ++u) {
                    const float x = E::to_f(e[u]);
                    n2 += x * x;
                    n1 += fabsf(x);
                }
            }
        }
        n2 = group_sum_dpp<4>(n2);
        n1 = group_sum_dpp<4>(n1);
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
        if (WIN && j < Ct) {
            float tot = 0.f;
            for (int w = 0; w < Wv; ++w) tot += sm.nrm[j * Wv + w];
            const float den = tot + eps;
            bwin = den > 0.f ? sm.eta[j] / den : 0.f;
        }
        const int sj = WIN ? min(j / Wv, Ct - 1) : min(j, Ct - 1);
        const float gsj = __shfl(lg, sj, 64);
        const float bsj = __shfl(bwin, sj, 64);
        if (j < CV) {
            float r = 0.f;
            if (j < NVR) {
                if (WIN) {
                    r = bsj;
                } else if (COL) {
                    r = 1.f;
                } else {
                    const float den = sm.nrm[j] + eps;
                    r = den > 0.f ? sm.eta[sj] / den : 0.f;
                }
            }
            sm.g[j] = lg;
            sm.rs[j] = r;
            sm.step[j] = sj;
            recS[0 * CV + j] = __expf(gsj);                   // gam
            recS[1 * CV + j] = __expf(glast - gsj) * r;       // hrow
            recS[2 * CV + j] = __expf(lg);                    // gq
            recS[3 * CV + j] = sm.l1[j];                      // l1
            recS[4 * CV + j] = (j < NVR) ? sm.eta[sj] : 0.f;  // erow
        }
    }
    if constexpr (COL) {
        // u_j = eta x_j / (|x_j| ||x||_1 + eps)
        for (int c = tid; c < CV * CPR; c += 256) {
            const int i = c / CPR, col = (c % CPR) * EPC;
            const int s = WIN ? min(i / Wv, Ct - 1) : min(i, Ct - 1);
            const float et = sm.eta[s], l1 = sm.l1[i];
            const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.X[i][col]);
            const T* e = reinterpret_cast<const T*>(&v);
            u32x4 outv;
            T* out = reinterpret_cast<T*>(&outv);
#pragma unroll
            for (int u = 0; u < EPC; ++u) {
                const float x = E::to_f(e[u]);
                const float den = fabsf(x) * l1 + eps;
                out[u] = E::from_f((i < NVR && den > 0.f) ? et * x / den : 0.f);
            }
            *reinterpret_cast<u32x4*>(&sm.Om[i][col]) = outv;
        }
    }
    __syncthreads();

    // ---- Gram blocks.  Operands are swapped (rows of the second factor as
    // the MFMA A operand) so the accumulator holds the block transposed,
    // i.e. lane (lr, grp) holds M[16b + lr][16c + 4 grp + r]: exactly the A
    // fragment kernel 2 loads. ----
    const T* omb;
    if constexpr (COL) omb = &sm.Om[0][0];
    else omb = &sm.X[0][0];
    for (int q = wave; q < NJ; q += 4) {
        const bool isA = q < NJA;
        int b, c;
        if (isA) {
            b = 0;
            while ((b + 1) * (b + 2) / 2 <= q) ++b;
            c = q - b * (b + 1) / 2;
        } else {
            b = (q - NJA) / NB;
            c = (q - NJA) % NB;
        }
        if (!isA && !(b < NBQ && (16 * c) / Wv <= 16 * b + 15)) continue;  // never read
        const T* ar = omb + (size_t)(16 * c + lr) * LDX;                       // omega_j rows
        const T* br = isA ? &sm.X[16 * b + lr][0] : &sm.Q[16 * b + lr][0];   // x_i / q_t rows
        f32x4 acc = zero4();
#pragma unroll
        for (int m = 0; m < D / 32; ++m)
            acc = E::mma32(E::load(ar + 32 * m + 4 * grp), E::load(ar + 32 * m + 16 + 4 * grp),
                           E::load(br + 32 * m + 4 * grp), E::load(br + 32 * m + 16 + 4 * grp), acc);
        const int i = 16 * b + lr;  // row of A (x_i) or of P (t)
        f32x4 val;
        if (isA) {
            const int si = sm.step[i];
            const float gi = sm.g[si];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * c + 4 * grp + r;
                const int sj = sm.step[j];
                val[r] = (sj < si) ? __expf(gi - sm.g[sj]) * acc[r] * sm.rs[j] : 0.f;
            }
            if (b == c) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.Adg[b][lr][4 * grp + r] = val[r];
            } else {
                *reinterpret_cast<Frag*>(recT + R::kA + (size_t)R::ablk(b, c) * 256 + lane * 4) =
                    E::pack(-val);
            }
        } else {
            const float gi = sm.g[i];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * c + 4 * grp + r;
                const int sj = sm.step[j];
                val[r] = (sj <= i && i < Ct) ? __expf(gi - sm.g[sj]) * acc[r] * sm.rs[j] : 0.f;
            }
            *reinterpret_cast<Frag*>(recT + R::kP + (size_t)R::pblk(b, c, WIN) * 256 + lane * 4) =
                E::pack(val);
        }
    }
    if constexpr (DELTA) {
        __syncthreads();
        // ---- (I + A_bb)^-1 by forward substitution, one column per lane ----
        if (wave < NB && lane < 16) {
            const int b = wave, c = lane;
            float tcol[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) acc -= sm.Adg[b][i][j] * tcol[j];
                tcol[i] = acc;
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.Adg[b][i][c] = tcol[i];
        }
        __syncthreads();
        if (wave < NB) {
            f32x4 tv;
#pragma unroll
            for (int r = 0; r < 4; ++r) tv[r] = sm.Adg[wave][lr][4 * grp + r];
            *reinterpret_cast<Frag*>(recT + R::kD + (size_t)wave * 256 + lane * 4) = E::pack(tv);
        }
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
    // targets y_i of this workgroup's 64 value columns; each wave reads the 16
    // columns it owns, then writes its outputs over them (staged there on
    // their way to HBM), so at fp32, d = 128, chunk 64 the tiles fit LDS
    T Y[CV][64 + PADE];
    alignas(16) char rec[R::kBytes];  // this tile's record
};

template <class E, int D, int CV, bool DELTA, bool COL, bool WIN>
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
    constexpr int RCH = (int)(R::kBytes / 16);  // 16-byte chunks of a record
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
    const int r = (jj / NVS) * 8 + xcd;
    const int vs = jj % NVS;
    if (r >= a.BH) return;
    const int bh = pass_bh(a, r);
    const int v0 = vs * 64;

    const int W = a.W;
    const int Wv = WIN ? W : 1;
    const int Ct = CV / Wv, NVR = Ct * Wv, NBQ = (Ct + 15) / 16;
    const SeqRows sr = seq_rows(a, bh);
    const int T_ = sr.T;
    const float eps = a.eps;
    // with a feature map, q and k are the mapped copies (their own rows)
    const size_t kq0 = a.phi ? mapped_row0(a, bh) : sr.row0;
    const T* qg = static_cast<const T*>(a.q) + kq0 * D;
    const T* kg = static_cast<const T*>(a.k) + kq0 * D;
    const T* vg = static_cast<const T*>(a.v) + sr.row0 * D + v0;
    const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
    const T* vp = (a.v_prev && W > 1)
                      ? static_cast<const T*>(a.v_prev) + (size_t)bh * (W - 1) * D + v0
                      : nullptr;
    const char* recg = static_cast<const char*>(ws) + (size_t)bh * ntiles * R::kBytes;
    T* og = static_cast<T*>(a.o) + sr.row0 * D + v0;

    // State slice as accumulators of S^T: Sacc[kb][r] = S[v][k],
    // v = v0 + 16*wave + lr, k = 16*kb + 4*grp + r.
    const int vcol = v0 + 16 * wave + lr;
    f32x4 Sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
        Sacc[kb] = a.S0 ? *reinterpret_cast<const f32x4*>(a.S0 + ((size_t)bh * D + vcol) * D +
                                                          16 * kb + 4 * grp)
                        : zero4();

    // ---- per-thread load geometry, fixed across tiles ----
    int xi[NXL], xcol[NXL], xoff[NXL], xs[NXL];
    int yi[NYL], ycol[NYL], yoff[NYL], ys[NYL];
#pragma unroll
    for (int it = 0; it < NXL; ++it) {
        const int c = min(tid + 256 * it, CV * CPR - 1);
        xi[it] = c / CPR;
        xcol[it] = (c % CPR) * EPC;
        const int s = WIN ? xi[it] / Wv : xi[it];
        xs[it] = (tid + 256 * it < CV * CPR && xi[it] < NVR) ? s : (1 << 28);  // never valid
        xoff[it] = s - (WIN ? xi[it] - s * Wv : 0) - a.lag;  // key index - t0
    }
#pragma unroll
    for (int it = 0; it < NYL; ++it) {
        const int c = min(tid + 256 * it, CV * YCPR - 1);
        yi[it] = c / YCPR;
        ycol[it] = (c % YCPR) * EPC;
        const int s = WIN ? yi[it] / Wv : yi[it];
        ys[it] = (tid + 256 * it < CV * YCPR && yi[it] < NVR) ? s : (1 << 28);
        yoff[it] = s - (WIN ? yi[it] - s * Wv : 0);  // value index - t0
    }

    u32x4 px[NXL], pq[NXL], py[NYL], pr[NRL];
    float pl1[COL ? NXL : 1], per[COL ? NXL : 1];

    auto load_tile = [&](int tile) __attribute__((always_inline)) {
        const int t0 = tile * Ct;
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int tau = t0 + xoff[it];
            const bool ok = t0 + xs[it] < T_ && (tau >= 0 || kp != nullptr);
            const T* p = tau >= 0 ? kg + (size_t)tau * D : (kp ? kp + (size_t)(W + tau) * D : kg);
            px[it] = sel16(ok, *reinterpret_cast<const u32x4*>((ok ? p : kg) + xcol[it]));
            const int tq = t0 + xi[it];
            const bool okq = xi[it] < Ct && tq < T_ && tid + 256 * it < CV * CPR;
            pq[it] = sel16(okq, *reinterpret_cast<const u32x4*>((okq ? qg + (size_t)tq * D : qg) +
                                                                xcol[it]));
            if constexpr (COL) {
                const float* sc = reinterpret_cast<const float*>(
                    recg + (size_t)tile * R::kBytes + R::kScalBytes);
                pl1[it] = sc[3 * CV + xi[it]];
                per[it] = sc[4 * CV + xi[it]];
            }
        }
#pragma unroll
        for (int it = 0; it < NYL; ++it) {
            const int tv = t0 + yoff[it];
            const bool ok = t0 + ys[it] < T_ && (tv >= 0 || vp != nullptr);
            const T* p = tv >= 0 ? vg + (size_t)tv * D : (vp ? vp + (size_t)(W - 1 + tv) * D : vg);
            py[it] = sel16(ok, *reinterpret_cast<const u32x4*>((ok ? p : vg) + ycol[it]));
        }
        const u32x4* rg = reinterpret_cast<const u32x4*>(recg + (size_t)tile * R::kBytes);
        static_for<NRL>([&](auto itc) __attribute__((always_inline)) {
            constexpr int it = decltype(itc)::value;
            pr[it] = rg[min(tid + 256 * it, RCH - 1)];
        });
    };

    auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            if (tid + 256 * it < CV * CPR) {
                *reinterpret_cast<u32x4*>(&sm.X[xi[it]][xcol[it]]) = px[it];
                *reinterpret_cast<u32x4*>(&sm.Q[xi[it]][xcol[it]]) = pq[it];
                if constexpr (COL) {
                    const T* e = reinterpret_cast<const T*>(&px[it]);
                    u32x4 outv;
                    T* out = reinterpret_cast<T*>(&outv);
#pragma unroll
                    for (int u = 0; u < EPC; ++u) {
                        const float x = E::to_f(e[u]);
                        const float den = fabsf(x) * pl1[it] + eps;
                        out[u] = E::from_f(den > 0.f ? per[it] * x / den : 0.f);
                    }
                    *reinterpret_cast<u32x4*>(&sm.Om[xi[it]][xcol[it]]) = outv;
                }
            }
        }
#pragma unroll
        for (int it = 0; it < NYL; ++it)
            if (tid + 256 * it < CV * YCPR)
                *reinterpret_cast<u32x4*>(&sm.Y[yi[it]][ycol[it]]) = py[it];
        static_for<NRL>([&](auto itc) __attribute__((always_inline)) {
            constexpr int it = decltype(itc)::value;
            if (tid + 256 * it < RCH) reinterpret_cast<u32x4*>(sm.rec)[tid + 256 * it] = pr[it];
        });
    };

    const int ntl = tiles_of(T_, Ct);  // this sequence's tiles (ntiles: the record stride)
    if (ntl > 0) load_tile(0);
    for (int tile = 0; tile < ntl; ++tile) {
        const int t0 = tile * Ct;
        store_tile();
        __syncthreads();
        // next tile's loads, in flight during this tile's arithmetic (the last
        // tile reloads itself: harmless, and keeps the prefetch unconditional)
        load_tile(min(tile + 1, ntl - 1));

        const T* recT = reinterpret_cast<const T*>(sm.rec);
        const float* gam = reinterpret_cast<const float*>(sm.rec + R::kScalBytes);
        const float* hrow = gam + CV;
        const float* gq = gam + 2 * CV;

        // column fragment of a row-major LDS tile: lane (lr, grp) gets
        // M[row0 + 4 grp + r][col0 + lr], r = 0..3
        auto colfrag = [&](const T* m, int ld, int row0, int col0) __attribute__((always_inline)) {
            if constexpr (E::kBytes == 2)
                return E::load_tr(m + (size_t)(row0 + 4 * grp + (lr >> 2)) * ld + col0 + 4 * (lr & 3));
            else
                return E::gather4(m + (size_t)(row0 + 4 * grp) * ld + col0 + lr, ld);
        };
        constexpr int LDY = 64 + Smem::PADE;

        Frag SB[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) SB[kb] = E::pack(Sacc[kb]);

        // Z = X S0^T and Zq = Q S0^T: 2 NB independent accumulation chains
        f32x4 Z[NB], Zq[NB];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            Z[rb] = zero4();
            Zq[rb] = zero4();
        }
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
            Frag xf0[NB], xf1[NB], qf0[NB], qf1[NB];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                const T* xr = &sm.X[16 * rb + lr][32 * m + 4 * grp];
                const T* qr = &sm.Q[16 * rb + lr][32 * m + 4 * grp];
                if (DELTA) {
                    xf0[rb] = E::load(xr);
                    xf1[rb] = E::load(xr + 16);
                }
                qf0[rb] = E::load(qr);
                qf1[rb] = E::load(qr + 16);
            }
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                if (DELTA) Z[rb] = E::mma32(xf0[rb], xf1[rb], SB[2 * m], SB[2 * m + 1], Z[rb]);
                if (rb < NBQ) Zq[rb] = E::mma32(qf0[rb], qf1[rb], SB[2 * m], SB[2 * m + 1], Zq[rb]);
            }
        }

        f32x4 Dl[NB];
        Frag DB[NB];
        if constexpr (DELTA) {
            // residuals R = Y - diag(gam) X S0^T
            f32x4 Rr[NB];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                const Frag yf = colfrag(&sm.Y[0][0], LDY, 16 * rb, 16 * wave);
                const f32x4 gm = *reinterpret_cast<const f32x4*>(gam + 16 * rb + 4 * grp);
#pragma unroll
                for (int r = 0; r < 4; ++r) Rr[rb][r] = E::to_f((T)yf[r]) - gm[r] * Z[rb][r];
            }
            // blocked forward substitution: Delta_b = Td_b (R_b - sum_{c<b} A_bc Delta_c)
            Frag Af[Rec<E, CV, DELTA>::NBA > 0 ? Rec<E, CV, DELTA>::NBA : 1], Tf[NB];
#pragma unroll
            for (int q = 0; q < R::NBA; ++q) Af[q] = E::load(recT + R::kA + (size_t)q * 256 + lane * 4);
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) Tf[rb] = E::load(recT + R::kD + (size_t)rb * 256 + lane * 4);
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                f32x4 acc = Rr[rb];
#pragma unroll
                for (int cb = 0; cb < rb; ++cb) acc = E::mma16(Af[R::ablk(rb, cb)], DB[cb], acc);
                Dl[rb] = E::mma16(Tf[rb], E::pack(acc), zero4());
                DB[rb] = E::pack(Dl[rb]);
            }
        } else {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                const Frag yf = colfrag(&sm.Y[0][0], LDY, 16 * rb, 16 * wave);
#pragma unroll
                for (int r = 0; r < 4; ++r) Dl[rb][r] = E::to_f((T)yf[r]);
                DB[rb] = E::pack(Dl[rb]);
            }
        }

        // outputs O = diag(gq) Q S0^T + P Delta, staged in LDS
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            if (tb >= NBQ) continue;
            f32x4 acc = Zq[tb];
            const f32x4 gqv = *reinterpret_cast<const f32x4*>(gq + 16 * tb + 4 * grp);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= gqv[r];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if (WIN && (16 * cb) / Wv > 16 * tb + 15) continue;
                if (!WIN && cb > tb) continue;
                acc = E::mma16(E::load(recT + R::kP + (size_t)R::pblk(tb, cb, WIN) * 256 + lane * 4),
                               DB[cb], acc);
            }
            // the wave's own target columns, already read (program order)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.Y[16 * tb + 4 * grp + r][16 * wave + lr] = E::from_f(acc[r]);
        }

        // state update S^T = exp(g_last) S0^T + Omega^T diag(hrow) Delta; the A
        // operand Omega^T comes from the row-major tile by column fragments
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
            if constexpr (NB == 1) {
                acc = E::mma16(colfrag(om, LDX, 0, 16 * kb), HB[0], acc);
            } else {
#pragma unroll
                for (int m = 0; m < NB / 2; ++m)
                    acc = E::mma32(colfrag(om, LDX, 32 * m, 16 * kb),
                                   colfrag(om, LDX, 32 * m + 16, 16 * kb), HB[2 * m], HB[2 * m + 1],
                                   acc);
            }
            Sacc[kb] = acc;
        }
        __syncthreads();
        // outputs of this tile to HBM, 16 bytes per lane
#pragma unroll
        for (int it = 0; it < NYL; ++it) {
            const int c = tid + 256 * it;
            const int t = c / YCPR, col = (c % YCPR) * EPC;
            if (c < CV * YCPR && t < Ct && t0 + t < T_)
                *reinterpret_cast<u32x4*>(og + (size_t)(t0 + t) * D + col) =
                    *reinterpret_cast<const u32x4*>(&sm.Y[t][col]);
        }
        __syncthreads();  // the next tile's targets overwrite the staged outputs
    }

    if (a.S_final) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            *reinterpret_cast<f32x4*>(a.S_final + ((size_t)bh * D + vcol) * D + 16 * kb + 4 * grp) =
                Sacc[kb];
    }
}

// ---------------------------------------------------------------------------
// Kernel 2, bf16 form: the state pass, one workgroup per (batch*head, 64-wide
// value slice), its waves in three roles.
//
//   waves 0-3  (chain)  tile `it`: S0 -> bf16 copy in LDS, Z = X S0^T,
//                       residuals, forward substitution -> Delta (bf16 copy
//                       in LDS), state update.  No global memory traffic.
//   waves 4-7  (output) tile `it - 1`: O^T = diag(gq) (S0 Q^T) + Delta^T P^T
//                       from the two LDS copies; at 64-row tiles each wave
//                       takes 16 rows for all 64 value columns and stores
//                       them as whole rows (transposed through its own,
//                       already read, query rows), otherwise each takes 16
//                       value columns and stores from the accumulators.
//   waves 8-11 (fill)   the fills of tile it+1's keys, targets and chain
//                       record and tile it's queries and output record,
//                       direct to LDS.  A wave that issues a tile's worth of
//                       fills stalls on a full memory queue for thousands of
//                       cycles; here no computing wave does.
// For the per-column rule the fill waves also bring in the write vectors u
// that the intra-chunk kernel stored (into the query buffer), and the output
// waves take the queries as register fragments loaded one tile ahead.
// One barrier per tile, fencing LDS only.  Loads use buffer descriptors:
// out-of-range rows read as zero in hardware, and a lane's offsets stay
// fixed from tile to tile.
// ---------------------------------------------------------------------------
template <int D, int CV, bool DELTA, bool COL, bool WIN>
struct PassSmem {
    using R = Rec<EBf16, CV, DELTA>;
    static constexpr int LDX = D + 8;
    static constexpr int LDY = 64 + 8;
    static constexpr int KB = D / 16, NB = CV / 16;
    static constexpr int RECF = (R::NBA + R::NBD) * 512;   // -A and Td fragments (bytes)
    static constexpr int RECB = RECF + R::NSC * CV * 4;     // then the row factors
    static constexpr int PGB = R::npblk(WIN) * 512 + CV * 4;  // P fragments, then gq
    uint16_t X[2][CV][LDX];     // keys x_i
    uint16_t Y[2][CV][LDY];     // targets y_i of this slice's 64 value columns
    uint16_t QU[2][CV][LDX];    // queries q_t; write vectors u_i for the per-column rule
    // bf16 state at the tile start and bf16 Delta, fragment order per chain
    // wave, fragments 2j and 2j + 1 of a lane side by side (one 16-byte read)
    s16x4 SB[2][4][KB / 2][64][2];
    s16x4 DB[2][4][(NB + 1) / 2][64][2];
    alignas(16) char rec[2][RECB];
    alignas(16) char pg[2][PGB];  // the output half's record pieces, staged one tile later
    uint32_t pf[WIN && !COL ? 4 : 1][64];  // landing area of the fill waves' L2 warm-up loads (never read)
};

template <int D, int CV, bool DELTA, bool COL, bool WIN>
__global__ __launch_bounds__(768) void chunk_pass_kernel(ChunkArgs a, const void* ws,
                                                                     int ntiles) {
    using E = EBf16;
    using T = uint16_t;
    using Frag = s16x4;
    using R = Rec<E, CV, DELTA>;
    using Smem = PassSmem<D, CV, DELTA, COL, WIN>;
    constexpr int NB = CV / 16, KB = D / 16, CPR = D / 8, NVS = D / 64;
    constexpr int LDX = Smem::LDX, LDY = Smem::LDY;
    constexpr int NXL = (CV * CPR + 255) / 256;  // 16-byte pieces of a key tile per stager
    constexpr int NYL = (CV * 8 + 255) / 256;    // of a target tile
    constexpr int RCH = Smem::RECB / 16, RFC = Smem::RECF / 16;
    constexpr int NRL = (RCH + 255) / 256;
    constexpr int PCH = Smem::PGB / 16, PFC = R::npblk(WIN) * 32;
    constexpr bool QG = COL;  // queries as register fragments from global memory
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    const bool chain = wave < 4;
    const bool filler = wave >= 8;
    const int cw = wave & 3;  // value-column block (16 columns) of this wave
    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int jj = blk >> 3;
    const int r = (jj / NVS) * 8 + xcd;
    const int vs = jj % NVS;
    if (r >= a.BH) return;
    const int bh = pass_bh(a, r);
    const int v0 = vs * 64;

    const int W = a.W;
    const int Wv = WIN ? W : 1;
    const int Ct = CV / Wv, NVR = Ct * Wv, NBQ = (Ct + 15) / 16;
    const SeqRows sr = seq_rows(a, bh);
    const int T_ = sr.T;
    const float eps = a.eps;
    // with a feature map, q and k are the mapped copies (their own rows)
    const size_t kq0 = a.phi ? mapped_row0(a, bh) : sr.row0;
    const T* qg = static_cast<const T*>(a.q) + kq0 * D;
    const T* kg = static_cast<const T*>(a.k) + kq0 * D;
    const T* vg = static_cast<const T*>(a.v) + sr.row0 * D + v0;
    const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
    const T* vp = (a.v_prev && W > 1)
                      ? static_cast<const T*>(a.v_prev) + (size_t)bh * (W - 1) * D + v0
                      : nullptr;
    const char* recg = static_cast<const char*>(ws) + (size_t)bh * ntiles * R::kBytes;
    T* og = static_cast<T*>(a.o) + sr.row0 * D + v0;
    const int ntl = tiles_of(T_, Ct);  // this sequence's tiles (ntiles: the record stride)

    // ---- chain: state slice as accumulators of S^T (wave cw owns 16 value
    // columns): Sacc[kb][r] = S[v][k], v = v0 + 16 cw + lr, k = 16 kb + 4 grp + r
    const int vcol = v0 + 16 * cw + lr;
    f32x4 Sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
        Sacc[kb] = (chain && a.S0) ? *reinterpret_cast<const f32x4*>(
                                         a.S0 + ((size_t)bh * D + vcol) * D + 16 * kb + 4 * grp)
                                   : zero4();

    // ---- output: staging geometry, fixed across tiles ----
    const int otid = tid & 255;  // index within the output or fill role
    // Each 16-byte piece a stager moves: its row relative to the tile start
    // (key x_i = k_{t0 + s - w - lag}, target y_i = v_{t0 + s - w}), its byte
    // column, and whether it exists.  Loads choose addresses, never data:
    // rows outside the sequence read as zero (descriptor bounds), halo rows
    // come from a second load that is merged when the piece is stored.
    int xrel[NXL], yrel[NYL];
    uint32_t xcb[NXL], ycb[NYL];
    bool xok[NXL], yok[NYL];
#pragma unroll
    for (int it = 0; it < NXL; ++it) {
        const int c = otid + 256 * it;
        const int i = c / CPR, col = (c % CPR) * 8;
        const int s = WIN ? i / Wv : i, w = WIN ? i - s * Wv : 0;
        xok[it] = c < CV * CPR && i < NVR;
        xrel[it] = s - w - a.lag;
        xcb[it] = (uint32_t)col * 2;
    }
#pragma unroll
    for (int it = 0; it < NYL; ++it) {
        const int c = otid + 256 * it;
        const int i = c / 8, col = (c % 8) * 8;
        const int s = WIN ? i / Wv : i, w = WIN ? i - s * Wv : 0;
        yok[it] = c < CV * 8 && i < NVR;
        yrel[it] = s - w;
        ycb[it] = (uint32_t)col * 2;
    }

    u32x4 px[NXL], py[NYL], pr[NRL];
    u32x4 pxh[NXL], pyh[NYL];  // halo rows of the first tiles
    // QG: the queries of one 16-row block (rows 16 (cw % NB) ..) as B fragments,
    // pQa for the tile being output and pQb for the next one
    Frag pQa[QG ? KB : 1], pQb[QG ? KB : 1];

    // keys, targets and the record of `tile` into registers
    auto load_xyr = [&](int tile) __attribute__((always_inline)) {
        const int t0 = tile * Ct;
        const int bx = max(t0 - W, 0), by = max(t0 - W + 1, 0);
        const rsrc_t rx = make_rsrc(kg + (size_t)bx * D, (int64_t)(T_ - bx) * D * 2);
        const rsrc_t ry = make_rsrc(vg + (size_t)by * D, (int64_t)(T_ - by) * D * 2);
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int tau = t0 + xrel[it];
            px[it] = buf_load16(rx, (xok[it] && tau >= 0) ? (uint32_t)((tau - bx) * D * 2) + xcb[it] : kOob);
        }
#pragma unroll
        for (int it = 0; it < NYL; ++it) {
            const int tv = t0 + yrel[it];
            py[it] = buf_load16(ry, (yok[it] && tv >= 0) ? (uint32_t)((tv - by) * D * 2) + ycb[it] : kOob);
        }
        if (t0 < W) {
            // rows before the sequence: the halo, or zero without one
            const rsrc_t hx = make_rsrc(kp ? kp : kg, kp ? (int64_t)W * D * 2 : 0);
#pragma unroll
            for (int it = 0; it < NXL; ++it) {
                const int tau = t0 + xrel[it];
                pxh[it] = buf_load16(hx, (xok[it] && tau < 0) ? (uint32_t)((W + tau) * D * 2) + xcb[it] : kOob);
            }
            const rsrc_t hy = make_rsrc(vp ? vp : vg, vp ? (int64_t)(W - 1) * D * 2 : 0);
#pragma unroll
            for (int it = 0; it < NYL; ++it) {
                const int tv = t0 + yrel[it];
                pyh[it] = buf_load16(hy, (yok[it] && tv < 0) ? (uint32_t)((W - 1 + tv) * D * 2) + ycb[it] : kOob);
            }
        }
        const char* rt = recg + (size_t)tile * R::kBytes;
#pragma unroll
        for (int it = 0; it < NRL; ++it) {
            const int rc = min(otid + 256 * it, RCH - 1);
            pr[it] = *reinterpret_cast<const u32x4*>(
                rt + (rc < RFC ? (size_t)rc * 16 : R::kScalBytes + (size_t)(rc - RFC) * 16));
        }
    };
    // queries of `tile` (per-column rule) as register fragments of the
    // wave's own row block into pQb
    auto load_q = [&](int tile) __attribute__((always_inline)) {
        if constexpr (QG) {
            const int t0 = tile * Ct;
            const rsrc_t rq = make_rsrc(qg + (size_t)t0 * D, (int64_t)(T_ - t0) * D * 2);
            const int t = 16 * (cw % NB) + lr;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                pQb[kb] = buf_load8(rq, t < Ct ? (uint32_t)((t * D + 16 * kb + 4 * grp) * 2) : kOob);
        }
    };
    auto store_xyr = [&](int tile) __attribute__((always_inline)) {
        const int b = tile & 1;
        if (tile * Ct < W) {
#pragma unroll
            for (int it = 0; it < NXL; ++it) px[it] |= pxh[it];
#pragma unroll
            for (int it = 0; it < NYL; ++it) py[it] |= pyh[it];
        }
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int c = otid + 256 * it;
            if (c < CV * CPR) {
                const int i = c / CPR, col = (c % CPR) * 8;
                *reinterpret_cast<u32x4*>(&sm.X[b][i][col]) = px[it];
            }
        }
#pragma unroll
        for (int it = 0; it < NYL; ++it) {
            const int c = otid + 256 * it;
            if (c < CV * 8) *reinterpret_cast<u32x4*>(&sm.Y[b][c / 8][(c % 8) * 8]) = py[it];
        }
#pragma unroll
        for (int it = 0; it < NRL; ++it) {
            const int rc = otid + 256 * it;
            if (rc < RCH) reinterpret_cast<u32x4*>(sm.rec[b])[rc] = pr[it];
        }
    };

    // column fragment of a row-major LDS tile: lane (lr, grp) gets
    // M[row0 + 4 grp + r][col0 + lr], r = 0..3
    auto colfrag = [&](const T* m, int ld, int row0, int col0) __attribute__((always_inline)) {
        return E::load_tr(m + (size_t)(row0 + 4 * grp + (lr >> 2)) * ld + col0 + 4 * (lr & 3));
    };

    // the state and Delta fragments in LDS: one, or a pair read at once
    auto sbf = [&](int b, int c, int kb) __attribute__((always_inline)) { return sm.SB[b][c][kb >> 1][lane][kb & 1]; };
    auto dbf = [&](int b, int c, int cb) __attribute__((always_inline)) { return sm.DB[b][c][cb >> 1][lane][cb & 1]; };
    auto pair_lo = [](s16x8 v) __attribute__((always_inline)) { return Frag{v[0], v[1], v[2], v[3]}; };
    auto pair_hi = [](s16x8 v) __attribute__((always_inline)) { return Frag{v[4], v[5], v[6], v[7]}; };
    auto sbp = [&](int b, int c, int m) __attribute__((always_inline)) {
        return *reinterpret_cast<const s16x8*>(&sm.SB[b][c][m][lane][0]);
    };
    auto dbp = [&](int b, int c, int j) __attribute__((always_inline)) {
        return *reinterpret_cast<const s16x8*>(&sm.DB[b][c][j][lane][0]);
    };

    // ---- chain: one tile ----
    auto chain_tile = [&](int it) __attribute__((always_inline)) {
        const int b = it & 1;
        const T* Xb = &sm.X[b][0][0];
        const T* Yb = &sm.Y[b][0][0];
        const T* recT = reinterpret_cast<const T*>(sm.rec[b]);
        const float* gam = reinterpret_cast<const float*>(sm.rec[b] + Smem::RECF);
        const float* hrow = gam + CV;
        const float* gq = gam + 2 * CV;

        // Reads that do not depend on the state go out first, so their latency
        // overlaps the state's packing and X S0^T: at 64-row tiles of the
        // scalar rule every key fragment of X S0^T, the targets and the
        // system's blocks are all requested before the first product (a
        // scheduling fence keeps the compiler from interleaving them with
        // the products, which would expose one LDS round trip per product).
        constexpr bool XPRE = DELTA && !COL && !WIN && NB == 4;
        Frag yf[NB], Af[R::NBA > 0 ? R::NBA : 1], Tf[NB];
        Frag xq[XPRE ? D / 32 : 1][NB][2];
        f32x4 gm[NB], hv[NB];
        if constexpr (XPRE) {
#pragma unroll
            for (int m = 0; m < D / 32; ++m)
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    const T* xr = Xb + (16 * rb + lr) * LDX + 32 * m + 4 * grp;
                    xq[m][rb][0] = E::load(xr);
                    xq[m][rb][1] = E::load(xr + 16);
                }
        }
        auto load_gates = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                hv[rb] = *reinterpret_cast<const f32x4*>(hrow + 16 * rb + 4 * grp);
                if constexpr (DELTA) gm[rb] = *reinterpret_cast<const f32x4*>(gam + 16 * rb + 4 * grp);
            }
        };
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) yf[rb] = colfrag(Yb, LDY, 16 * rb, 16 * cw);
        if constexpr (!XPRE) load_gates();
        // the system's blocks too, unless registers are short (per-column rule)
        auto load_sys = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) Tf[rb] = E::load(recT + R::kD + (size_t)rb * 256 + lane * 4);
#pragma unroll
            for (int q = 0; q < R::NBA; ++q) Af[q] = E::load(recT + R::kA + (size_t)q * 256 + lane * 4);
        };
        if constexpr (DELTA && !COL) load_sys();
        if constexpr (XPRE) __builtin_amdgcn_sched_barrier(0);
        const float glq = gq[Ct - 1];

        Frag SB[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) SB[kb] = E::pack(Sacc[kb]);
#pragma unroll
        for (int m = 0; m < KB / 2; ++m)
            *reinterpret_cast<s16x8*>(&sm.SB[b][cw][m][lane][0]) =
                s16x8{SB[2 * m][0], SB[2 * m][1], SB[2 * m][2], SB[2 * m][3],
                      SB[2 * m + 1][0], SB[2 * m + 1][1], SB[2 * m + 1][2], SB[2 * m + 1][3]};

        f32x4 Dl[NB];
        Frag DB[NB];
        if constexpr (DELTA) {
            // Z = X S0^T
            f32x4 Z[NB];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) Z[rb] = zero4();
#pragma unroll
            for (int m = 0; m < D / 32; ++m) {
                Frag xf0[NB], xf1[NB];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    if constexpr (XPRE) {
                        xf0[rb] = xq[m][rb][0];
                        xf1[rb] = xq[m][rb][1];
                    } else {
                        const T* xr = Xb + (16 * rb + lr) * LDX + 32 * m + 4 * grp;
                        xf0[rb] = E::load(xr);
                        xf1[rb] = E::load(xr + 16);
                    }
                }
#pragma unroll
                for (int rb = 0; rb < NB; ++rb)
                    Z[rb] = E::mma32(xf0[rb], xf1[rb], SB[2 * m], SB[2 * m + 1], Z[rb]);
            }
            if constexpr (XPRE) load_gates();
            // residuals R = Y - diag(gam) Z, then the blocked forward substitution
            // Delta_b = Td_b (R_b - sum_{c<b} A_bc Delta_c)
            if constexpr (COL) load_sys();
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                f32x4 acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = E::to_f((T)yf[rb][r]) - gm[rb][r] * Z[rb][r];
#pragma unroll
                for (int cb = 0; cb < rb; ++cb) acc = E::mma16(Af[R::ablk(rb, cb)], DB[cb], acc);
                Dl[rb] = E::mma16(Tf[rb], E::pack(acc), zero4());
                DB[rb] = E::pack(Dl[rb]);
            }
        } else {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Dl[rb][r] = E::to_f((T)yf[rb][r]);
                DB[rb] = yf[rb];
            }
        }
#pragma unroll
        for (int j = 0; j < NB / 2; ++j)
            *reinterpret_cast<s16x8*>(&sm.DB[b][cw][j][lane][0]) =
                s16x8{DB[2 * j][0], DB[2 * j][1], DB[2 * j][2], DB[2 * j][3],
                      DB[2 * j + 1][0], DB[2 * j + 1][1], DB[2 * j + 1][2], DB[2 * j + 1][3]};
        if constexpr (NB % 2 == 1) sm.DB[b][cw][NB / 2][lane][0] = DB[NB - 1];

        // S^T = exp(g_last) S0^T + Omega^T diag(hrow) Delta
        Frag HB[NB];
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
            f32x4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = hv[cb][r] * Dl[cb][r];
            HB[cb] = E::pack(h);
        }
        const T* om = COL ? &sm.QU[b][0][0] : Xb;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x4 acc = Sacc[kb] * glq;
            if constexpr (NB == 1) {
                acc = E::mma16(colfrag(om, LDX, 0, 16 * kb), HB[0], acc);
            } else {
#pragma unroll
                for (int m = 0; m < NB / 2; ++m)
                    acc = E::mma32(colfrag(om, LDX, 32 * m, 16 * kb),
                                   colfrag(om, LDX, 32 * m + 16, 16 * kb), HB[2 * m], HB[2 * m + 1],
                                   acc);
            }
            Sacc[kb] = acc;
        }
    };

    // ---- output: one tile, O^T = diag(gq) S0 Q^T + Delta^T P^T ----
    Frag opk[NB];  // outputs of one tile, packed, until they are stored
    auto store_o = [&](int p) __attribute__((always_inline)) {
        const int t0 = p * Ct;
        static_for<NB>([&](auto tbc) __attribute__((always_inline)) {
            constexpr int tb = decltype(tbc)::value;
            // lane holds O[t = 16 tb + lr][v = 16 cw + 4 grp + r]
            const int t = 16 * tb + lr;
            if (tb < NBQ && t < Ct && t0 + t < T_ && a.o)
                *reinterpret_cast<Frag*>(og + (size_t)(t0 + t) * D + 16 * cw + 4 * grp) = opk[tb];
        });
    };
    auto output_tile = [&](int p) __attribute__((always_inline)) {
        const int pb = p & 1;
        const T* Pf = reinterpret_cast<const T*>(sm.pg[pb]);
        const float* gqt = reinterpret_cast<const float*>(sm.pg[pb] + R::npblk(WIN) * 512);
        Frag sb[KB], db[NB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sb[kb] = sbf(pb, cw, kb);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) db[cb] = dbf(pb, cw, cb);
        if (a.ck_s) {
            // checkpoints for the backward pass, in 16-column blocks ([block][v][16]):
            // lane holds S[v][16 kb + 4 grp + r] and Delta[16 cb + 4 grp + r][v] of
            // value row v = vcol, so each store instruction writes 512
            // contiguous bytes
            const size_t tb = (size_t)bh * ntiles + p;
            T* cs = static_cast<T*>(a.ck_s) + tb * D * D + (size_t)vcol * 16 + 4 * grp;
            T* cd = static_cast<T*>(a.ck_d) + tb * D * CV + (size_t)vcol * 16 + 4 * grp;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) *reinterpret_cast<Frag*>(cs + (size_t)kb * D * 16) = sb[kb];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) *reinterpret_cast<Frag*>(cd + (size_t)cb * D * 16) = db[cb];
        }
        if (!a.o) return;  // checkpoint-only run (the backward pass's recompute)
        if constexpr (QG) {
            // Per-column rule: the queries come from global memory, so each
            // wave takes one 16-row block tb (reading the queries once per
            // workgroup) and forms its outputs for the value blocks
            // c2 = cw / NB + k (4 / NB), from every chain wave's state and
            // Delta fragments in LDS; stored at once.
            const int tb = cw % NB;
            const int t = 16 * tb + lr, t0 = p * Ct;
            const float gs = gqt[t];
            const bool st = t < Ct && t0 + t < T_ && a.o;
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int c2 = cw / NB + k * (4 / NB);
                f32x4 acc = zero4();
#pragma unroll
                for (int m = 0; m < D / 32; ++m)
                {
                    const s16x8 sp = sbp(pb, c2, m);
                    acc = E::mma32(pair_lo(sp), pair_hi(sp), pQa[2 * m], pQa[2 * m + 1], acc);
                }
                acc = acc * gs;
#pragma unroll
                for (int cb = 0; cb < NB; ++cb)
                    if (cb <= tb)
                        acc = E::mma16(dbf(pb, c2, cb),
                                       E::load(Pf + (size_t)R::pblk(tb, cb, false) * 256 + lane * 4),
                                       acc);
                if (st)
                    *reinterpret_cast<Frag*>(og + (size_t)(t0 + t) * D + 16 * c2 + 4 * grp) =
                        E::pack(acc);
            }
            return;
        }
        static_for<NB>([&](auto tbc) __attribute__((always_inline)) {
            constexpr int tb = decltype(tbc)::value;
            if (tb < NBQ) {
                f32x4 acc = zero4();
#pragma unroll
                for (int m = 0; m < D / 32; ++m) {
                    const T* qr = &sm.QU[pb][16 * tb + lr][32 * m + 4 * grp];
                    acc = E::mma32(sb[2 * m], sb[2 * m + 1], E::load(qr), E::load(qr + 16), acc);
                }
                acc = acc * gqt[16 * tb + lr];
                static_for<NB>([&](auto cbc) __attribute__((always_inline)) {
                    constexpr int cb = decltype(cbc)::value;
                    if (WIN || cb <= tb) {
                        if (!WIN || (tb < 2 && (16 * cb) / Wv <= 16 * tb + 15))
                            acc = E::mma16(db[cb],
                                           E::load(Pf + (size_t)R::pblk(tb, cb, WIN) * 256 + lane * 4),
                                           acc);
                    }
                });
                opk[tb] = E::pack(acc);
            }
        });
    };

    // ---- output, row-block form (scalar and inner-product rules at 64-row
    // tiles, windows of one): wave cw forms the outputs of query rows
    // 16 cw .. 16 cw + 15 for all 64 value columns, from every recurrence
    // wave's state and Delta fragments.  Its own query rows of the LDS
    // buffer are then free (no other wave reads them, and the next fill of
    // that buffer comes after the barrier), so the wave transposes its
    // outputs through them and stores o as 16-byte row pieces: each store
    // instruction writes 8 whole rows of its 64 value columns (128 bytes)
    // instead of 32 bytes of 16 rows.
    constexpr bool ROWS = !COL && !WIN && NB == 4;
    auto output_rows = [&](int p) __attribute__((always_inline)) {
        const int pb = p & 1, t0 = p * Ct, tb = cw;
        const T* Pf = reinterpret_cast<const T*>(sm.pg[pb]);
        const float* gqt = reinterpret_cast<const float*>(sm.pg[pb] + R::npblk(WIN) * 512);
        if (a.ck_s) {
            // checkpoints, as in output_tile (this wave's own value columns)
            const size_t tt = (size_t)bh * ntiles + p;
            T* cs = static_cast<T*>(a.ck_s) + tt * D * D + (size_t)vcol * 16 + 4 * grp;
            T* cd = static_cast<T*>(a.ck_d) + tt * D * CV + (size_t)vcol * 16 + 4 * grp;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                *reinterpret_cast<Frag*>(cs + (size_t)kb * D * 16) = sbf(pb, cw, kb);
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
                *reinterpret_cast<Frag*>(cd + (size_t)cb * D * 16) = dbf(pb, cw, cb);
        }
        if (!a.o) return;  // checkpoint-only run (the backward pass's recompute)
        // the row block is a compile-time constant of each copy, so the causal
        // block tests below leave no branches between the products, and the
        // four value blocks' products accumulate side by side
        with_const4(tb, [&](auto tbc) __attribute__((always_inline)) {
            constexpr int TB = decltype(tbc)::value;
            T* qrow = &sm.QU[pb][16 * TB][0];
            const Frag zf = {0, 0, 0, 0};
            Frag qf[KB], pf[NB];
#pragma unroll
            for (int m = 0; m < D / 32; ++m) {
                qf[2 * m] = E::load(qrow + lr * LDX + 32 * m + 4 * grp);
                qf[2 * m + 1] = E::load(qrow + lr * LDX + 32 * m + 16 + 4 * grp);
            }
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
                pf[cb] = cb <= TB ? E::load(Pf + (size_t)R::pblk(TB, cb, false) * 256 + lane * 4) : zf;
            const float gs = gqt[16 * TB + lr];
            f32x4 acc[4];
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2) acc[c2] = zero4();
#pragma unroll
            for (int m = 0; m < D / 32; ++m)
#pragma unroll
                for (int c2 = 0; c2 < 4; ++c2)
                {
                    const s16x8 sp = sbp(pb, c2, m);
                    acc[c2] = E::mma32(pair_lo(sp), pair_hi(sp), qf[2 * m], qf[2 * m + 1], acc[c2]);
                }
            // Delta^T P^T over the causal blocks cb <= TB, two per product
            Frag of[4];
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2) {
                acc[c2] = acc[c2] * gs;
                if constexpr (TB >= 1) {
                    const s16x8 dp = dbp(pb, c2, 0);
                    acc[c2] = E::mma32(pair_lo(dp), pair_hi(dp), pf[0], pf[1], acc[c2]);
                } else {
                    acc[c2] = E::mma32(dbf(pb, c2, 0), zf, pf[0], zf, acc[c2]);
                }
                if constexpr (TB >= 3) {
                    const s16x8 dp = dbp(pb, c2, 1);
                    acc[c2] = E::mma32(pair_lo(dp), pair_hi(dp), pf[2], pf[3], acc[c2]);
                } else if constexpr (TB == 2) {
                    acc[c2] = E::mma32(dbf(pb, c2, 2), zf, pf[2], zf, acc[c2]);
                }
                of[c2] = E::pack(acc[c2]);  // O[t = 16 TB + lr][v = 16 c2 + 4 grp + r]
            }
            // transpose through the wave's own query rows (read above, in order)
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2)
                *reinterpret_cast<Frag*>(qrow + lr * LDX + 16 * c2 + 4 * grp) = of[c2];
            const int rr = lane >> 3, pc = lane & 7;  // row (and row + 8), 16-byte piece
            const u32x4 o0 = *reinterpret_cast<const u32x4*>(qrow + rr * LDX + 8 * pc);
            const u32x4 o1 = *reinterpret_cast<const u32x4*>(qrow + (rr + 8) * LDX + 8 * pc);
            // rows past the tile or the sequence: an out-of-range offset, no branch
            const int nrow = min(Ct, T_ - t0), t = 16 * TB + rr;
            const rsrc_t ro = make_rsrc(og + (size_t)t0 * D, (int64_t)nrow * D * 2);
            buf_store16(ro, t < nrow ? (uint32_t)((t * D + 8 * pc) * 2) : kOob, o0);
            buf_store16(ro, t + 8 < nrow ? (uint32_t)(((t + 8) * D + 8 * pc) * 2) : kOob, o1);
        });
    };

    // ---- direct-to-LDS staging (all rules but the per-column one, whose
    // write vectors are derived while staging): every 16-byte slot of an LDS
    // tile is one lane of one buffer_load ... lds, issued by the output waves
    // right after a barrier and waited for before the next one.  A slot's
    // source is fixed relative to its tile, so the offsets are computed once;
    // padding and missing rows read as zero.
    constexpr int SPX = LDX / 8, SPY = LDY / 8;      // slots per key / target row
    constexpr int NSX = CV * SPX, NSY = CV * SPY;    // slots per tile
    constexpr int NIX = (NSX + 63) / 64, NIY = (NSY + 63) / 64;
    constexpr int NIR = (RCH + 63) / 64, NIP = (PCH + 63) / 64;
    constexpr int MIX = (NIX + 3) / 4, MIY = (NIY + 3) / 4, MIR = (NIR + 3) / 4, MIP = (NIP + 3) / 4;
    uint32_t dx[MIX], dq[MIX], dy[MIY], dr[MIR], dp[MIP];
    const int ow = cw;  // index of this wave within its role
    {
#pragma unroll
        for (int m = 0; m < MIX; ++m) {
            const int k = 64 * (ow + 4 * m) + lane;
            const int row = k / SPX, wi = k - row * SPX;
            const int s = WIN ? row / Wv : row, w = WIN ? row - s * Wv : 0;
            const bool in = k < NSX && wi < D / 8;
            dx[m] = (in && row < NVR) ? (uint32_t)(((s - w - a.lag + W) * D + wi * 8) * 2) : kOob;
            dq[m] = (in && row < Ct) ? (uint32_t)((row * D + wi * 8) * 2) : kOob;
        }
#pragma unroll
        for (int m = 0; m < MIY; ++m) {
            const int k = 64 * (ow + 4 * m) + lane;
            const int row = k / SPY, wi = k - row * SPY;
            const int s = WIN ? row / Wv : row, w = WIN ? row - s * Wv : 0;
            dy[m] = (k < NSY && wi < 8 && row < NVR) ? (uint32_t)(((s - w + W - 1) * D + wi * 8) * 2)
                                                      : kOob;
        }
#pragma unroll
        for (int m = 0; m < MIR; ++m) {
            const int k = 64 * (ow + 4 * m) + lane;
            dr[m] = k < RCH ? (uint32_t)(k < RFC ? k * 16 : R::kScalBytes + (k - RFC) * 16) : kOob;
        }
#pragma unroll
        for (int m = 0; m < MIP; ++m) {
            const int k = 64 * (ow + 4 * m) + lane;
            dp[m] = k < PCH ? (uint32_t)(k < PFC ? R::kP * 2 + k * 16 : R::kScalBytes + 2 * CV * 4 + (k - PFC) * 16)
                            : kOob;
        }
    }
    // Fills of one tile, each spread over the four fill waves: keys, targets
    // and the chain's record pieces of a tile with t0 >= W go to buffer
    // tile & 1, as do its queries and the output waves' record pieces.
    // LDS byte addresses of the filled buffers (the workgroup's one LDS
    // object starts at sm_lds)
    const uint32_t sm_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) Smem*)&sm;
    auto lds_of = [&](size_t field, size_t bytes_per_buffer, int b) __attribute__((always_inline)) {
        return sm_lds + (uint32_t)(field + bytes_per_buffer * b);
    };
    // per-column rule: the tile's write vectors (rows as the query slots'
    // rows, from the intra-chunk kernel's copy) into the query/u buffer
    auto dma_u = [&](int tile) __attribute__((always_inline)) {
        if constexpr (COL) {
            const u32x4 ru = make_desc(static_cast<const T*>(a.uws) + ((size_t)bh * ntiles + tile) * CV * D,
                                       (int64_t)CV * D * 2);
            const uint32_t ub = lds_of(offsetof(Smem, QU), sizeof(sm.QU[0]), tile & 1);
#pragma unroll
            for (int m = 0; m < MIX; ++m) {
                const int i = ow + 4 * m;
                if (i < NIX && 64 * i + lane < NSX) buf_load16_lds(ru, ub + 1024 * i, dq[m]);
            }
        }
    };
    auto dma_xr = [&](int tile) __attribute__((always_inline)) {
        const int t0 = tile * Ct, b = tile & 1;
        const u32x4 rx = make_desc(kg + (size_t)(t0 - W) * D, (int64_t)(T_ - t0 + W) * D * 2);
        const u32x4 rr = make_desc(recg + (size_t)tile * R::kBytes, R::kBytes);
        const uint32_t xb = lds_of(offsetof(Smem, X), sizeof(sm.X[0]), b);
        const uint32_t rb = lds_of(offsetof(Smem, rec), sizeof(sm.rec[0]), b);
#pragma unroll
        for (int m = 0; m < MIX; ++m) {
            const int i = ow + 4 * m;
            if (i < NIX && 64 * i + lane < NSX) buf_load16_lds(rx, xb + 1024 * i, dx[m]);
        }
        dma_u(tile);
#pragma unroll
        for (int m = 0; m < MIR; ++m) {
            const int i = ow + 4 * m;
            if (i < NIR && 64 * i + lane < RCH) buf_load16_lds(rr, rb + 1024 * i, dr[m]);
        }
    };
    auto dma_y = [&](int tile) __attribute__((always_inline)) {
        const int t0 = tile * Ct, b = tile & 1;
        const u32x4 ry = make_desc(vg + (size_t)(t0 - W + 1) * D, (int64_t)(T_ - t0 + W - 1) * D * 2);
        const uint32_t yb = lds_of(offsetof(Smem, Y), sizeof(sm.Y[0]), b);
#pragma unroll
        for (int m = 0; m < MIY; ++m) {
            const int i = ow + 4 * m;
            if (i < NIY && 64 * i + lane < NSY) buf_load16_lds(ry, yb + 1024 * i, dy[m]);
        }
    };
    auto dma_qp = [&](int tile) __attribute__((always_inline)) {
        const int t0 = tile * Ct, b = tile & 1;
        const u32x4 rq = make_desc(qg + (size_t)t0 * D, (int64_t)(T_ - t0) * D * 2);
        const u32x4 rr = make_desc(recg + (size_t)tile * R::kBytes, R::kBytes);
        const uint32_t qb = lds_of(offsetof(Smem, QU), sizeof(sm.QU[0]), b);
        const uint32_t pb = lds_of(offsetof(Smem, pg), sizeof(sm.pg[0]), b);
        if constexpr (!COL) {  // the per-column rule's queries are register fragments
#pragma unroll
            for (int m = 0; m < MIX; ++m) {
                const int i = ow + 4 * m;
                if (i < NIX && 64 * i + lane < NSX) buf_load16_lds(rq, qb + 1024 * i, dq[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < MIP; ++m) {
            const int i = ow + 4 * m;
            if (i < NIP && 64 * i + lane < PCH) buf_load16_lds(rr, pb + 1024 * i, dp[m]);
        }
    };

    // ---- pipeline: the chain works on tile it while the output half
    // finishes tile it-1 ----
    {
        // Iteration it.  Output half: store the outputs of tile it-2, start
        // the fills of tile it+1's keys and chain record, compute tile it-1.
        // Chain half: start the fills of tile it+1's targets and tile it's
        // queries and output record, then compute tile it.  Both halves wait
        // for their fills before the barrier, so the fills' latency overlaps
        // the arithmetic.  Tiles that still reach back before the sequence (t0 < W)
        // are staged by the output half through registers, halo included.
        // Each role runs its own loop with the same number of barriers, so
        // the compiler's wait bookkeeping for one role's memory operations
        // never reaches another role's code.  Iteration it: the chain works on
        // tile it, the output waves store tile it-2 and compute tile it-1, the
        // fill waves bring in tile it+1's keys, targets and chain record and
        // tile it's queries and output record.  Every buffer a fill writes
        // was last read in the previous iteration.  Tiles that still reach
        // back before the sequence (t0 < W) are staged by the output waves
        // through registers, halo included.
        const bool out = !chain && !filler;
        if (out && ntl > 0) {
            load_xyr(0);
            store_xyr(0);
            // per-column rule: tile 0's write vectors, and the first queries
            dma_u(0);
            load_q(0);
        }
        // the state's initial loads (chain) are complete before the loops, so
        // no wait inside them is owed to a load issued out here
        if (!filler) wait_vm_all();
        lds_barrier();
        if (chain) {
            for (int it = 0; it <= ntl; ++it) {
                if (it < ntl) chain_tile(it);
                lds_barrier();
            }
        } else if (filler) {
            // direct-to-LDS fills, issued after the barrier and waited for
            // before the next one.  The chain and output waves keep LDS busy,
            // and these fills cost no LDS instruction of their own.  (The
            // inner-product rules once staged through registers one iteration
            // ahead instead: Falcon-3A at window 4 ran 35% slower that way.)
            // L2 warm-up (windows above one): after its fills, each fill wave
            // issues two 4-byte loads per lane, one lane per 128-byte line,
            // over tile it+2's keys, targets and record and tile it+1's
            // queries, landing in a scratch area of LDS that nothing reads.
            // They are the two most recent loads of the wave, so the wait
            // before the barrier (vmcnt(2)) covers the fills and lets them run
            // on into the next iteration; the next iteration's fills then find
            // their lines in L2.  Every iteration issues exactly two (offsets
            // past the data read nothing), and all are drained before the wave
            // ends.  Falcon-3A at window 4 runs 17% faster with them; at
            // 64-step tiles the gain is within run-to-run noise.
            const uint32_t pfl = lds_of(offsetof(Smem, pf), 256, WIN ? ow : 0);
            auto warm = [&](int it) __attribute__((always_inline)) {
                const int tx = it + 2, tq = it + 1;
                const int t0x = tx * Ct, t0q = tq * Ct;
                const bool okx = tx < ntl && t0x >= W, okq = tq < ntl;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // 0-2: keys, 3-4: queries, 5: targets, 6-7: record (wave-uniform)
                    const int inst = 2 * __builtin_amdgcn_readfirstlane(ow) + j;
                    u32x4 d;
                    uint32_t off = kOob;
                    if (inst <= 2) {
                        d = make_desc(kg + (size_t)(okx ? t0x - W : 0) * D, okx ? (int64_t)(T_ - t0x + W) * D * 2 : 0);
                        const uint32_t o = (uint32_t)(inst * 64 + lane) * 128;
                        if (okx && o < (uint32_t)((Ct + W) * D * 2)) off = o;
                    } else if (inst <= 4) {
                        d = make_desc(qg + (size_t)(okq ? t0q : 0) * D, okq ? (int64_t)(T_ - t0q) * D * 2 : 0);
                        const uint32_t o = (uint32_t)((inst - 3) * 64 + lane) * 128;
                        if (okq && o < (uint32_t)(Ct * D * 2)) off = o;
                    } else if (inst == 5) {
                        d = make_desc(vg + (size_t)(okx ? t0x - W + 1 : 0) * D, okx ? (int64_t)(T_ - t0x + W - 1) * D * 2 : 0);
                        if (okx && lane < Ct + W - 1) off = (uint32_t)lane * D * 2;
                    } else {
                        d = make_desc(recg + (size_t)(okx ? tx : 0) * R::kBytes, okx ? (int64_t)R::kBytes : 0);
                        const uint32_t o = (uint32_t)((inst - 6) * 64 + lane) * 128;
                        if (okx && o < (uint32_t)R::kBytes) off = o;
                    }
                    buf_load4_lds(d, pfl, off);
                }
            };
            for (int it = 0; it <= ntl; ++it) {
                if (it + 1 < ntl && (it + 1) * Ct >= W) {
                    dma_xr(it + 1);
                    dma_y(it + 1);
                }
                if (it < ntl) dma_qp(it);
                if constexpr (WIN) {
                    warm(it);
                    wait_vm_2();
                } else {
                    wait_vm_all();
                }
                lds_barrier();
            }
            wait_vm_all();
        } else {
            for (int it = 0; it <= ntl; ++it) {
                if (!ROWS && it >= 2) store_o(it - 2);
                // (without a window W = 1, so only tile 0, in the prologue)
                if (WIN && it + 1 < ntl && (it + 1) * Ct < W) {
                    load_xyr(it + 1);
                    store_xyr(it + 1);
                }
                if (it >= 1) {
                    if constexpr (ROWS)
                        output_rows(it - 1);
                    else
                        output_tile(it - 1);
                }
                if constexpr (QG) {
                    // the queries of tile it+1 load during iteration it
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) pQa[kb] = pQb[kb];
                    if (it + 1 < ntl) load_q(it + 1);
                }
                lds_barrier();
            }
            if (!ROWS && ntl >= 1) store_o(ntl - 1);
        }
    }

    if (chain && a.S_final) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            *reinterpret_cast<f32x4*>(a.S_final + ((size_t)bh * D + vcol) * D + 16 * kb + 4 * grp) =
                Sacc[kb];
    }
}

// ---------------------------------------------------------------------------
// Kernel 1, bf16 form: persistent intra-chunk preparation.  Each workgroup
// walks tiles (batch*head, tile) with a stride of the grid, holding the next
// tile's keys, queries and gates in registers while it works on the current
// one, so the loads of one tile overlap the arithmetic of the previous.
// Per tile: norms, the log-decay scan, the Gram blocks (A: x_i . omega_j,
// P: q_t . omega_j; without a window each wave owns one row block of each and
// reads each column block's operand once for both, with a window the blocks
// go round-robin over the waves), masks and decays from per-row and
// per-column factors, then the 16 x 16 diagonal inverses.
// Blocks of P that the state pass never reads are not written.
// ---------------------------------------------------------------------------
template <int D, int CV, bool COL>
struct Prep2Smem {
    static constexpr int LDX = D + 8;
    uint16_t X[CV][LDX];           // keys x_i (virtual rows)
    uint16_t Q[CV][LDX];           // queries q_t
    uint16_t Om[COL ? CV : 1][LDX];  // per-column write vectors u_i
    alignas(16) float Adg[CV / 16][16][20];  // diagonal blocks of A (fp32), then their inverses
    float al[CV], et[CV];          // gates of the tile's steps (padding: 1, 0)
    alignas(16) float cf[CV];      // column factor exp(g_ref(c) - g_j) r_j, c = block of j
    float gref[CV / 16];           // log2(e) * g at the last row of each block
    float nrm[CV], l1[CV];         // ||x_i||^2, ||x_i||_1
    alignas(16) float gv[CV];      // log2(e) * g of the step of virtual row i
    alignas(16) float gs[CV];      // log2(e) * g_t per step t
    alignas(16) float rs[CV];      // row scale r_i of the write vector
    alignas(16) int step[CV];      // step of virtual row i
};

// Occupancy: three workgroups per compute unit for the A family; two for the
// delta family, whose Gram rows, inverse and prefetch registers would spill
// at three.
template <bool DELTA>
constexpr int kPrepPerCu = DELTA ? 2 : 3;

template <int D, int CV, bool DELTA, bool COL, bool WIN>
__global__ __launch_bounds__(256, kPrepPerCu<DELTA>) void chunk_prep2_kernel(ChunkArgs a, void* ws, int ntiles,
                                                             int njobs) {
    using E = EBf16;
    using T = uint16_t;
    using Frag = s16x4;
    using R = Rec<E, CV, DELTA>;
    using Smem = Prep2Smem<D, CV, COL>;
    constexpr int NB = CV / 16, CPR = D / 8;
    constexpr int NXL = (CV * CPR + 255) / 256;
    constexpr int LDX = Smem::LDX;
    constexpr int NJA = DELTA ? NB * (NB + 1) / 2 : 0;  // A blocks on and below the diagonal
    constexpr int NJP = WIN ? NB * NB : NB * (NB + 1) / 2;
    constexpr float kLog2e = 1.4426950408889634f;
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4,
              lr = lane & 15;
    const int W = a.W;
    const int Wv = WIN ? W : 1;
    const int Ct = CV / Wv, NVR = Ct * Wv, NBQ = (Ct + 15) / 16;
    const float eps = a.eps;

    // staging geometry, fixed across tiles: each 16-byte piece's key row
    // relative to the tile start (x_i = k_{t0 + s - w - lag}), byte column and
    // existence.  Loads choose addresses, never data, so no load is waited
    // for before the next tile is staged: rows outside the sequence read as
    // zero (descriptor bounds) and halo rows come from a second load.
    int xrel[NXL];
    uint32_t xcb[NXL], qvo[NXL];
    bool xok[NXL];
#pragma unroll
    for (int it = 0; it < NXL; ++it) {
        const int c = tid + 256 * it;
        const int i = c / CPR, col = (c % CPR) * 8;
        const int s = WIN ? i / Wv : i, w = WIN ? i - s * Wv : 0;
        xok[it] = c < CV * CPR && i < NVR;
        xrel[it] = s - w - a.lag;
        xcb[it] = (uint32_t)col * 2;
        qvo[it] = (c < CV * CPR && i < Ct) ? (uint32_t)((i * D + col) * 2) : kOob;
    }
    u32x4 px[NXL], pxh[NXL], pq[NXL];
    float pal = 1.f, pet = 0.f;

    auto load = [&](const Job& jb) __attribute__((always_inline)) {
        const int bh = jb.bh, tile = jb.tile;
        const int t0 = tile * Ct;
        const SeqRows sr = jb.sr;
        const int T_ = sr.T;
        const T* kg = static_cast<const T*>(a.k) + sr.row0 * D;
        const T* qg = static_cast<const T*>(a.q) + sr.row0 * D;
        const int bx = max(t0 - W, 0);
        const rsrc_t rx = make_rsrc(kg + (size_t)bx * D, (int64_t)(T_ - bx) * D * 2);
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int tau = t0 + xrel[it];
            px[it] = buf_load16(rx, (xok[it] && tau >= 0) ? (uint32_t)((tau - bx) * D * 2) + xcb[it] : kOob);
        }
        if (t0 < W) {
            const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
            const rsrc_t hx = make_rsrc(kp ? kp : kg, kp ? (int64_t)W * D * 2 : 0);
#pragma unroll
            for (int it = 0; it < NXL; ++it) {
                const int tau = t0 + xrel[it];
                pxh[it] = buf_load16(hx, (xok[it] && tau < 0) ? (uint32_t)((W + tau) * D * 2) + xcb[it] : kOob);
            }
        }
        const rsrc_t rq = make_rsrc(qg + (size_t)t0 * D, (int64_t)(T_ - t0) * D * 2);
#pragma unroll
        for (int it = 0; it < NXL; ++it) pq[it] = buf_load16(rq, qvo[it]);
        if (tid < CV) {
            // an index inside the gates whatever the tile, selected when staged
            const size_t g = (t0 + tid < T_) ? sr.row0 + t0 + tid : 0;
            pal = a.alpha[g];
            pet = a.eta[g];
        }
    };

    // Packed calls read each job's entry from the table one job ahead, with a
    // vector load (counted by vmcnt, so no LDS wait ever waits for it; a scalar
    // load would share lgkmcnt with LDS and stall the next LDS read).
    if (a.toff) njobs = a.H * a.toff[a.BH / a.H];  // packed: the tiles that exist
    const rsrc_t rjobs = make_rsrc(a.jobs, a.jobs ? (int64_t)njobs * 16 : 0);
    auto fetch = [&](int j) __attribute__((always_inline)) {
        return buf_load16(rjobs, (a.jobs && j < njobs) ? (uint32_t)j * 16u : kOob);
    };
    auto decode = [&](int j, u32x4 e) __attribute__((always_inline)) {
        if (!a.jobs) return job_of(a, j, ntiles);
        const int bh = (int)__builtin_amdgcn_readfirstlane(e[0]);
        const int h = bh - (bh / a.H) * a.H;
        return Job{bh, (int)__builtin_amdgcn_readfirstlane(e[1]),
                   {(size_t)h * a.Ttot + (int)__builtin_amdgcn_readfirstlane(e[2]),
                    (int)__builtin_amdgcn_readfirstlane(e[3])}};
    };
    int job = blockIdx.x;
    const u32x4 zero16 = {0u, 0u, 0u, 0u};
    u32x4 e_nxt = a.jobs ? fetch(job + gridDim.x) : zero16;
    Job jcur = decode(job, a.jobs ? fetch(job) : zero16);
    if (job < njobs) load(jcur);
    for (; job < njobs; job += gridDim.x) {
        const Job jb = jcur;
        const int bh = jb.bh, tile = jb.tile;
        const int T_ = jb.sr.T;  // tiles beyond it are identity padding, never read
        char* rec = static_cast<char*>(ws) + ((size_t)bh * ntiles + tile) * R::kBytes;
        T* recT = reinterpret_cast<T*>(rec);
        float* recS = reinterpret_cast<float*>(rec + R::kScalBytes);

        // ---- stage the prefetched tile, then prefetch the next ----
        if (tile * Ct < W) {
#pragma unroll
            for (int it = 0; it < NXL; ++it) px[it] |= pxh[it];
        }
        if (a.phi) {
            // the feature map, and the mapped keys, halo keys and queries for
            // the state pass (a key appearing in several virtual rows is
            // written with the same value by each)
            const int t0 = tile * Ct;
            T* kq = static_cast<T*>(a.kphi) + mapped_row0(a, bh) * D;
            T* qq = static_cast<T*>(a.qphi) + mapped_row0(a, bh) * D;
            T* kpq = a.kpphi ? static_cast<T*>(a.kpphi) + (size_t)bh * W * D : nullptr;
#pragma unroll
            for (int it = 0; it < NXL; ++it) {
                px[it] = phi_piece<E, CPR>(a.phi, px[it]);
                pq[it] = phi_piece<E, CPR>(a.phi, pq[it]);
                const int c = tid + 256 * it;
                const int i = c / CPR, col = (c % CPR) * 8;
                const int tau = t0 + xrel[it];
                if (xok[it] && tau >= 0 && tau < T_)
                    *reinterpret_cast<u32x4*>(kq + (size_t)tau * D + col) = px[it];
                else if (xok[it] && tau < 0 && kpq)
                    *reinterpret_cast<u32x4*>(kpq + (size_t)(W + tau) * D + col) = px[it];
                if (qvo[it] != kOob && t0 + i < T_)
                    *reinterpret_cast<u32x4*>(qq + (size_t)(t0 + i) * D + col) = pq[it];
            }
        }
#pragma unroll
        for (int it = 0; it < NXL; ++it) {
            const int c = tid + 256 * it;
            if (c < CV * CPR) {
                *reinterpret_cast<u32x4*>(&sm.X[c / CPR][(c % CPR) * 8]) = px[it];
                *reinterpret_cast<u32x4*>(&sm.Q[c / CPR][(c % CPR) * 8]) = pq[it];
            }
        }
        if (tid < CV) {
            const bool ok = tid < Ct && tile * Ct + tid < T_;  // padding steps: identity
            sm.al[tid] = ok ? pal : 1.f;
            sm.et[tid] = ok ? pet : 0.f;
        }
        lds_barrier();
        if (job + (int)gridDim.x < njobs) {
            jcur = decode(job + gridDim.x, e_nxt);
            load(jcur);
        }
        if (a.jobs) e_nxt = fetch(job + 2 * gridDim.x);
        // a packed sequence shorter than the longest leaves tiles that the
        // state pass never reads: stage them (the prefetch chain) and move on
        if (tile >= tiles_of(T_, Ct)) continue;

        // ---- norms: 4 threads per row ----
        {
            const int i = tid >> 2, part = tid & 3;
            float n2 = 0.f, n1 = 0.f;
            if (i < CV) {
#pragma unroll
                for (int c = 0; c < D / 4; c += 8) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.X[i][part * (D / 4) + c]);
                    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float x = E::to_f(e[u]);
                        n2 += x * x;
                        n1 += fabsf(x);
                    }
                }
            }
            n2 = group_sum_dpp<4>(n2);
            n1 = group_sum_dpp<4>(n1);
            if (i < CV && part == 0) {
                sm.nrm[i] = n2;
                sm.l1[i] = n1;
            }
        }
        lds_barrier();

        // ---- log-decay scan and row factors (wave 0) ----
        if (wave == 0) {
            const int j = lane;
            const float lg = wave_scan_dpp((j < Ct) ? __logf(sm.al[j]) : 0.f);
            const float glast =
                __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lg), Ct - 1));
            float bwin = 0.f;  // window normalizer of step j
            if (WIN && j < Ct) {
                float tot = 0.f;
                for (int w = 0; w < Wv; ++w) tot += sm.nrm[j * Wv + w];
                const float den = tot + eps;
                bwin = den > 0.f ? sm.et[j] / den : 0.f;
            }
            const int sj = WIN ? min(j / Wv, Ct - 1) : min(j, Ct - 1);
            // without a window a row is its own step (sj = j on the rows kept)
            const float gsj = WIN ? __shfl(lg, sj, 64) : lg;
            const float bsj = WIN ? __shfl(bwin, sj, 64) : 0.f;
            const float esj = WIN ? __shfl(sm.et[j < CV ? j : 0], sj, 64) : sm.et[j < CV ? j : 0];
            if (j < CV) {
                float r = 0.f;
                if (j < NVR) {
                    if (WIN) {
                        r = bsj;
                    } else if (COL) {
                        r = 1.f;
                    } else {
                        const float den = sm.nrm[j] + eps;
                        r = den > 0.f ? esj / den : 0.f;
                    }
                }
                sm.gv[j] = gsj * kLog2e;
                sm.gs[j] = lg * kLog2e;
                sm.rs[j] = r;
                if constexpr (!WIN) {
                    // decays off the diagonal split at the block's last row: both
                    // factors are exp(later - earlier) <= 1
                    const float gref = __shfl(gsj, (j & ~15) + 15, 64);
                    sm.cf[j] = __expf(gref - gsj) * r;
                    if ((j & 15) == 15) sm.gref[j >> 4] = gref * kLog2e;
                }
                sm.step[j] = (j < NVR) ? sj : (1 << 20);  // padding rows: after every step
                recS[0 * CV + j] = __expf(gsj);                  // gam
                recS[1 * CV + j] = __expf(glast - gsj) * r;      // hrow
                recS[2 * CV + j] = __expf(lg);                   // gq
                recS[3 * CV + j] = sm.l1[j];                     // l1
                recS[4 * CV + j] = (j < NVR) ? esj : 0.f;        // erow
            }
        }
        if constexpr (COL) {
            // u_j = eta x_j / (|x_j| ||x||_1 + eps)
            for (int c = tid; c < CV * CPR; c += 256) {
                const int i = c / CPR, col = (c % CPR) * 8;
                const int s = WIN ? min(i / Wv, Ct - 1) : min(i, Ct - 1);
                const float et = (i < NVR) ? sm.et[s] : 0.f, l1 = sm.l1[i];
                const u32x4 outv = col_write8(*reinterpret_cast<const u32x4*>(&sm.X[i][col]), l1, et, eps);
                *reinterpret_cast<u32x4*>(&sm.Om[i][col]) = outv;
                // and for the state pass (rows past the sequence hold zeros)
                *reinterpret_cast<u32x4*>(static_cast<T*>(a.uws) +
                                          (((size_t)bh * ntiles + tile) * CV + i) * D + col) = outv;
            }
        }
        lds_barrier();

        // ---- Gram blocks.  Operands are swapped (rows of omega as the A
        // operand) so lane (lr, grp) holds M[16 b + lr][16 c + 4 grp + r]: the
        // fragment order the state pass reads.
        const T* omb = COL ? &sm.Om[0][0] : &sm.X[0][0];
        if constexpr (!WIN) {
            // Wave w owns A row block w and P row block NB-1-w (the A family:
            // P row block w): its key and query rows are loaded once, and each
            // column block's omega rows serve both products as two independent
            // accumulation chains.
            constexpr int KM = D / 32;
            // the wave's row blocks are compile-time constants of each copy, so
            // the causal tests on the column block leave no branches
            with_const4(wave, [&](auto wc) __attribute__((always_inline)) {
            constexpr int WV = decltype(wc)::value;
            constexpr int bA = WV, bP = DELTA ? NB - 1 - WV : WV;
            if constexpr (WV < NB) {
                s16x8 xa[KM], qp[KM];
#pragma unroll
                for (int m = 0; m < KM; ++m) {
                    if constexpr (DELTA) xa[m] = E::load8(&sm.X[16 * bA + lr][32 * m + 8 * grp]);
                    qp[m] = E::load8(&sm.Q[16 * bP + lr][32 * m + 8 * grp]);
                }
                const int iA = 16 * bA + lr, iP = 16 * bP + lr;
                const float giA = sm.gv[iA], giP = sm.gs[iP];
                static_for<NB>([&](auto cc) __attribute__((always_inline)) {
                    constexpr int c = decltype(cc)::value;
                    constexpr bool doA = DELTA && c <= bA, doP = c <= bP;
                    if constexpr (doA || doP) {
                        const T* ar = omb + (size_t)(16 * c + lr) * LDX + 8 * grp;
                        f32x4 accA = zero4(), accP = zero4();
#pragma unroll
                        for (int m = 0; m < KM; ++m) {
                            const s16x8 om = E::load8(ar + 32 * m);
                            if constexpr (doA) accA = E::mma32r(om, xa[m], accA);
                            if constexpr (doP) accP = E::mma32r(om, qp[m], accP);
                        }
                        const int j0 = 16 * c + 4 * grp;
                        if constexpr (doA) {
                            f32x4 val;
                            if constexpr (c < bA) {
                                // fully unmasked: row factor times column factor
                                const f32x4 cfj = *reinterpret_cast<const f32x4*>(&sm.cf[j0]);
                                const float rf = exp2f(giA - sm.gref[c]);
#pragma unroll
                                for (int r = 0; r < 4; ++r) val[r] = accA[r] * rf * cfj[r];
                                *reinterpret_cast<Frag*>(recT + R::kA + (size_t)R::ablk(bA, c) * 256 +
                                                         lane * 4) = E::pack(-val);
                            } else {
                                const f32x4 gj = *reinterpret_cast<const f32x4*>(&sm.gv[j0]);
                                const f32x4 rj = *reinterpret_cast<const f32x4*>(&sm.rs[j0]);
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int j = j0 + r;
                                    // every lane evaluates, the mask selects (no branch)
                                    const float e = exp2f(giA - gj[r]) * accA[r] * rj[r];
                                    val[r] = (j < iA) ? e : 0.f;
                                    sm.Adg[bA][lr][4 * grp + r] = val[r];
                                }
                            }
                        }
                        if constexpr (doP) {
                            f32x4 val;
                            if constexpr (c < bP) {
                                const f32x4 cfj = *reinterpret_cast<const f32x4*>(&sm.cf[j0]);
                                const float rf = exp2f(giP - sm.gref[c]);
#pragma unroll
                                for (int r = 0; r < 4; ++r) val[r] = accP[r] * rf * cfj[r];
                            } else {
                                const f32x4 gj = *reinterpret_cast<const f32x4*>(&sm.gv[j0]);
                                const f32x4 rj = *reinterpret_cast<const f32x4*>(&sm.rs[j0]);
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int j = j0 + r;
                                    const float e = exp2f(giP - gj[r]) * accP[r] * rj[r];
                                    val[r] = (j <= iP && iP < Ct) ? e : 0.f;
                                }
                            }
                            *reinterpret_cast<Frag*>(recT + R::kP + (size_t)R::pblk(bP, c, WIN) * 256 +
                                                     lane * 4) = E::pack(val);
                        }
                    }
                });
            }
            });
        } else {
            // window: round-robin over the waves
            for (int q = wave; q < NJA + NJP; q += 4) {
                const bool isA = q < NJA;
                int b, c;
                if (isA || !WIN) {
                    const int qq = isA ? q : q - NJA;
                    b = 0;
                    while ((b + 1) * (b + 2) / 2 <= qq) ++b;
                    c = qq - b * (b + 1) / 2;
                } else {
                    b = (q - NJA) / NB;
                    c = (q - NJA) - b * NB;
                    if (!(b < NBQ && (16 * c) / Wv <= 16 * b + 15)) continue;  // never read
                }
                const T* ar = omb + (size_t)(16 * c + lr) * LDX + 8 * grp;
                const T* br = (isA ? &sm.X[16 * b + lr][0] : &sm.Q[16 * b + lr][0]) + 8 * grp;
                f32x4 acc = zero4();
    #pragma unroll
                for (int m = 0; m < D / 32; ++m) acc = E::mma32r(E::load8(ar + 32 * m), E::load8(br + 32 * m), acc);
                const int j0 = 16 * c + 4 * grp;
                const int i = 16 * b + lr;
                f32x4 val;
                if (!WIN && c < b) {
                    // fully unmasked block: row factor times column factor
                    const f32x4 cfj = *reinterpret_cast<const f32x4*>(&sm.cf[j0]);
                    const float rf = exp2f((isA ? sm.gv[i] : sm.gs[i]) - sm.gref[c]);
    #pragma unroll
                    for (int r = 0; r < 4; ++r) val[r] = acc[r] * rf * cfj[r];
                    if (isA)
                        *reinterpret_cast<Frag*>(recT + R::kA + (size_t)R::ablk(b, c) * 256 + lane * 4) =
                            E::pack(-val);
                    else
                        *reinterpret_cast<Frag*>(recT + R::kP + (size_t)R::pblk(b, c, WIN) * 256 + lane * 4) =
                            E::pack(val);
                    continue;
                }
                const f32x4 gj = *reinterpret_cast<const f32x4*>(&sm.gv[j0]);
                const f32x4 rj = *reinterpret_cast<const f32x4*>(&sm.rs[j0]);
                const int4 sj = *reinterpret_cast<const int4*>(&sm.step[j0]);
                if (isA) {
                    const int si = sm.step[i];
                    const float gi = sm.gv[i];
                    val[0] = (sj.x < si) ? exp2f(gi - gj[0]) * acc[0] * rj[0] : 0.f;
                    val[1] = (sj.y < si) ? exp2f(gi - gj[1]) * acc[1] * rj[1] : 0.f;
                    val[2] = (sj.z < si) ? exp2f(gi - gj[2]) * acc[2] * rj[2] : 0.f;
                    val[3] = (sj.w < si) ? exp2f(gi - gj[3]) * acc[3] * rj[3] : 0.f;
                    if (b == c) {
    #pragma unroll
                        for (int r = 0; r < 4; ++r) sm.Adg[b][lr][4 * grp + r] = val[r];
                    } else {
                        *reinterpret_cast<Frag*>(recT + R::kA + (size_t)R::ablk(b, c) * 256 + lane * 4) =
                            E::pack(-val);
                    }
                } else {
                    const bool tv = i < Ct;
                    const float gi = sm.gs[i];
                    val[0] = (tv && sj.x <= i) ? exp2f(gi - gj[0]) * acc[0] * rj[0] : 0.f;
                    val[1] = (tv && sj.y <= i) ? exp2f(gi - gj[1]) * acc[1] * rj[1] : 0.f;
                    val[2] = (tv && sj.z <= i) ? exp2f(gi - gj[2]) * acc[2] * rj[2] : 0.f;
                    val[3] = (tv && sj.w <= i) ? exp2f(gi - gj[3]) * acc[3] * rj[3] : 0.f;
                    *reinterpret_cast<Frag*>(recT + R::kP + (size_t)R::pblk(b, c, WIN) * 256 + lane * 4) =
                        E::pack(val);
                }
            }
        }
        if constexpr (DELTA) {
            lds_barrier();
            // ---- (I + A_bb)^-1 by forward substitution, t_i = delta_ic -
            // sum_{j<i} A_ij t_j for each column c.  Lane 4c + p works on column c
            // and the terms 4p <= j < 4p + 4 of every row's sum; the four partial
            // sums of a row meet in one DPP reduction within the lane quad.  The
            // masked block holds zeros on and above its diagonal, so every lane
            // runs the same unmasked loop.  Wave b owns block b from here on, so
            // no further barrier ----
            if (wave < NB) {
                const int bb = wave;
                const int c = lane >> 2, p = lane & 3;
                float tp[4] = {0.f, 0.f, 0.f, 0.f};  // tp[u] = t_{4p+u} of column c
                // rows four at a time, the next four read while these are used
                f32x4 cur[4], nxt[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) cur[r] = *reinterpret_cast<const f32x4*>(&sm.Adg[bb][r][4 * p]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (q < 3) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            nxt[r] = *reinterpret_cast<const f32x4*>(&sm.Adg[bb][4 * q + 4 + r][4 * p]);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 4 * q + r;
                        float s = 0.f;
                        if (i > 0) {
                            const f32x4 a = cur[r];
                            s = (a[0] * tp[0] + a[1] * tp[1]) + (a[2] * tp[2] + a[3] * tp[3]);
                            s = group_sum_dpp<4>(s);
                        }
                        const float ti = ((i == c) ? 1.f : 0.f) - s;
                        if (p == q) tp[r] = ti;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) cur[r] = nxt[r];
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int u = 0; u < 4; ++u) sm.Adg[bb][4 * p + u][c] = tp[u];
                __builtin_amdgcn_wave_barrier();
                f32x4 tv;
#pragma unroll
                for (int r = 0; r < 4; ++r) tv[r] = sm.Adg[bb][lr][4 * grp + r];
                *reinterpret_cast<Frag*>(recT + R::kD + (size_t)bb * 256 + lane * 4) = E::pack(tv);
            }
        } else {
            // the next tile's staging overwrites the keys and queries the Gram
            // blocks above read
            lds_barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
hipError_t launch_packed_schedule(const ChunkArgs& a, int Ct, int ntiles, ChunkArgs& b,
                                  hipStream_t stream) {
    const int nbins = ntiles + 1;
    if (!(a.cu && a.order_ws && ntiles > 0 && nbins <= 8192)) return hipSuccess;
    // schedule layout: order [N], toff [N+1], then (256-byte aligned) the job
    // table, 4 ints for each of at most BH * ntiles jobs
    const int N = a.BH / a.H;
    int* jobs = a.order_ws + ((2 * (size_t)N + 1 + 63) / 64) * 64;
    const int cul = N + 1 <= kCuLds ? N + 1 : 0;
    hipLaunchKernelGGL(packed_schedule_kernel, dim3(1), dim3(1024), (nbins + 1025 + cul) * sizeof(int),
                       stream, a, Ct, nbins, a.order_ws, a.order_ws + N, jobs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    b.order = a.order_ws;
    b.toff = a.order_ws + N;
    b.jobs = jobs;
    return hipSuccess;
}

template <class E, int D, int CV, bool DELTA, bool COL, bool WIN>
static hipError_t launch_one(const ChunkArgs& a, void* ws, hipStream_t stream) {
    const int Wv = WIN ? a.W : 1;
    const int ntiles = tiles_of(a.T, CV / Wv);
    ChunkArgs b = a;
    b.order = nullptr;
    b.toff = nullptr;
    b.jobs = nullptr;
    // the per-column rule's write vectors follow the records
    if constexpr (E::kBytes == 2 && COL)
        b.uws = static_cast<char*>(ws) + (size_t)a.BH * ntiles * Rec<E, CV, DELTA>::kBytes;
    {
        hipError_t e = launch_packed_schedule(a, CV / Wv, ntiles, b, stream);
        if (e != hipSuccess) return e;
    }
    if (ntiles > 0) {
        if constexpr (E::kBytes == 2) {
            // persistent grid: as many workgroups as fit on the device at once
            // (LDS allows floor(160 KiB / footprint) per compute unit, at most
            // the kernel's occupancy target)
            constexpr int per_cu_lds = (int)(163840 / sizeof(Prep2Smem<D, CV, COL>));
            constexpr int per_cu = per_cu_lds < 1 ? 1
                                                  : (per_cu_lds > kPrepPerCu<DELTA> ? kPrepPerCu<DELTA> : per_cu_lds);
            int dev = 0, cus = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                cus < 1)
                cus = 256;
            const int njobs = a.BH * ntiles;
            const int grid = njobs < cus * per_cu ? njobs : cus * per_cu;
            hipLaunchKernelGGL((chunk_prep2_kernel<D, CV, DELTA, COL, WIN>), dim3(grid), dim3(256),
                               0, stream, b, ws, ntiles, njobs);
        } else {
            hipLaunchKernelGGL((chunk_prep_kernel<E, D, CV, DELTA, COL, WIN>), dim3(a.BH * ntiles),
                               dim3(256), 0, stream, b, ws, ntiles);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.phi) {
        // the state pass reads the mapped keys, halo keys and queries
        b.k = a.kphi;
        b.q = a.qphi;
        b.k_prev = a.k_prev ? a.kpphi : nullptr;
    }
    const int nvs = D / 64;
    const int bh8 = (b.BH + 7) / 8 * 8;
    if constexpr (E::kBytes == 2)
        hipLaunchKernelGGL((chunk_pass_kernel<D, CV, DELTA, COL, WIN>), dim3(bh8 * nvs), dim3(768),
                           0, stream, b, (const void*)ws, ntiles);
    else
        hipLaunchKernelGGL((chunk_scan_kernel<E, D, CV, DELTA, COL, WIN>), dim3(bh8 * nvs),
                           dim3(256), 0, stream, b, (const void*)ws, ntiles);
    return hipGetLastError();
}

template <class E, int D, bool DELTA, bool COL, bool WIN>
static hipError_t launch_cv(const ChunkArgs& a, int chunk, void* ws, hipStream_t stream) {
    switch (chunk) {
        case 16: return launch_one<E, D, 16, DELTA, COL, WIN>(a, ws, stream);
        case 32: return launch_one<E, D, 32, DELTA, COL, WIN>(a, ws, stream);
        case 64: return launch_one<E, D, 64, DELTA, COL, WIN>(a, ws, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class E, bool DELTA, bool COL, bool WIN>
static hipError_t launch_d(const ChunkArgs& a, int D, int chunk, void* ws, hipStream_t stream) {
    if (D == 64) return launch_cv<E, 64, DELTA, COL, WIN>(a, chunk, ws, stream);
    if (D == 128) return launch_cv<E, 128, DELTA, COL, WIN>(a, chunk, ws, stream);
    return hipErrorInvalidValue;
}

template <class E>
static hipError_t launch_e(const ChunkArgs& a, int D, int chunk, bool delta, void* ws,
                           hipStream_t stream) {
    switch (a.norm) {
        case kNormScalar:
            return delta ? launch_d<E, true, false, false>(a, D, chunk, ws, stream)
                         : launch_d<E, false, false, false>(a, D, chunk, ws, stream);
        case kNormColumn:
            return delta ? launch_d<E, true, true, false>(a, D, chunk, ws, stream)
                         : launch_d<E, false, true, false>(a, D, chunk, ws, stream);
        case kNormWindow:
            // a window of one example is the scalar rule
            if (a.W == 1)
                return delta ? launch_d<E, true, false, false>(a, D, chunk, ws, stream)
                             : launch_d<E, false, false, false>(a, D, chunk, ws, stream);
            return delta ? launch_d<E, true, false, true>(a, D, chunk, ws, stream)
                         : launch_d<E, false, false, true>(a, D, chunk, ws, stream);
        default: return hipErrorInvalidValue;
    }
}

bool chunk_supported(int dt, int D, int chunk) {
    if (D != 64 && D != 128) return false;
    if (chunk != 16 && chunk != 32 && chunk != 64) return false;
    return true;
}

template <class E, int CV, bool DELTA>
static size_t rec_bytes() {
    return Rec<E, CV, DELTA>::kBytes;
}

size_t chunk_workspace_bytes(int BH, int T, int dt, int chunk, int window, int norm, bool delta,
                             int D) {
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
    // bf16 per-column rule: the write vectors, chunk x D bf16 per tile
    if (dt == 1 && norm == kNormColumn) rb += (size_t)chunk * D * 2;
    const size_t bytes = (size_t)BH * ntiles * rb;
    // bf16 windows: room for the records of either form (the collapsed one
    // runs the forward, the virtual-row one the backward's checkpoint runs)
    if (dt == 1 && norm == kNormWindow && window >= 2) {
        const size_t wb = window_workspace_bytes(BH, T, delta, D);
        return wb > bytes ? wb : bytes;
    }
    return bytes;
}

bool forward_kernel_differs(const ChunkArgs& a, int dt, int D, int chunk, bool delta) {
    ChunkArgs f = a;
    f.ck_s = f.ck_d = nullptr;
    return (dt == 1 && a.norm == kNormWindow && a.W >= 2 && !a.phi) ||
           fused_supported(f, dt, D, chunk, delta);
}

hipError_t launch_chunk(const ChunkArgs& a, int dt, int D, int chunk, bool delta, void* ws,
                        hipStream_t stream) {
    // the window rules at bf16 run the collapsed form (tiles of kWinC steps);
    // the backward pass's checkpoint runs and the feature maps keep the
    // virtual-row kernels
    if (dt == 1 && a.norm == kNormWindow && a.W >= 2 && !a.ck_s && !a.phi)
        return launch_window(a, D, delta, ws, stream);
    if (fused_supported(a, dt, D, chunk, delta)) return launch_fused(a, D, delta, stream);
    if (dt == 1) return launch_e<EBf16>(a, D, chunk, delta, ws, stream);
    return launch_e<EFp32>(a, D, chunk, delta, ws, stream);
}

}  // namespace falcon
