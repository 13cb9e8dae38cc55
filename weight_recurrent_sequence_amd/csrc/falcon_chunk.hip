// falcon_chunk.hip -- chunk-parallel forward pass of the Falcon recurrence,
// one fused kernel for gfx950.
//
// Method ("Fast Weight Attention for Continual Learning", authors' abstract;
// step size and decay-then-delta order from the KLA abstract on the same
// listing): per (batch, head) the state S (d_v x d_k) is decayed by alpha_t,
// corrected towards the prefix-aligned example (x_t, y_t) = (k_{t-1}, v_t)
// with a normalized step, and read after the write, o_t = S_t q_t.  The
// abstract states that a chunk-parallel form exists with positive-decay
// renormalization; this file computes that form.
//
// Chunk algebra (per tile of CV "virtual rows"; a row is one (step s,
// window slot w) example with key x_i, target y_i, write vector omega_i =
// rs_i * x_i, or u_i for the per-column rule; S0 is the state at the tile
// start, g_s the tile-local cumulative log decay, D(t,s) = exp(g_t - g_s)):
//   residuals   (I + A) Delta = Y - diag(exp g_s(i)) X S0^T,
//               A[i,j] = [s(j) < s(i)] D(s(i),s(j)) (x_i . omega_j)
//               (inner-product family: Delta = Y, no system)
//   outputs     O = diag(exp g_t) Q S0^T + P Delta,
//               P[t,j] = [s(j) <= t] D(t,s(j)) (q_t . omega_j)
//   next state  S = exp(g_last) S0 + sum_j D(last,s(j)) Delta_j omega_j^T
// Every decay factor is exp(later - earlier) <= 1 of a log sum that restarts
// at each tile, so nothing divides by a cumulative product and no tile can
// under- or overflow, whatever T is (the renormalization reading).
//
// Work decomposition (MI355X): one workgroup of 4 waves per (batch*head,
// 64-wide slice of d_v), walking the tiles of its sequence in order.  The
// state slice lives in registers as MFMA accumulators of S^T (wave w owns 16
// value columns), so it is used directly as the B operand of X S0^T and
// Q S0^T and updated in place; HBM sees each input once and the state once.
// Per tile: (L) stage keys, queries, values and gates in LDS; (N) norms,
// log-decay scan, write vectors; (G) Gram blocks X Omega^T and Q Omega^T on
// MFMA, masked and decayed; (I) fp32 inverses of the 16x16 diagonal blocks of
// I + A; (C) the sequential part: residuals, block forward substitution,
// outputs, state update.  Slices of one sequence are mapped to one XCD so
// the second slice's key/query reads hit that XCD's L2.
#include "falcon_device.h"
#include "falcon_internal.h"

namespace falcon {

template <class E, int D, int CV>
struct ChunkSmem {
    using T = typename E::T;
    static constexpr int PADE = 16 / E::kBytes;  // one 16-byte pad per row
    static constexpr int NB = CV / 16;
    T X[CV][D + PADE];      // keys x_i (virtual rows)
    T Q[CV][D + PADE];      // queries q_t
    T Om[CV][D + PADE];     // write vectors u_i (per-column rule only)
    T OmT[D][CV + PADE];    // write directions, transposed: x_i or u_i per column
    T Y[CV][64 + PADE];     // targets y_i, this workgroup's 64 value columns
    T An[CV][CV + PADE];    // -A (strictly lower in steps)
    T P[CV][CV + PADE];     // P (lower in steps, diagonal included)
    T Td[NB][16][16 + PADE];   // (I + A_bb)^-1 of the diagonal blocks
    float Adg[NB][16][17];  // fp32 diagonal blocks of A
    float alpha[CV], eta[CV], nrm[CV], l1[CV];
    float g[CV];            // tile-local cumulative log decay per step
    float gq[CV];           // exp(g_t) per step
    float gam[CV];          // exp(g_s(i)) per virtual row
    float hrow[CV];         // exp(g_last - g_s(i)) * rs_i per virtual row
    float rs[CV];           // row scale of the write vector (eta/(|x|^2+eps), b_s or 1)
    int step[CV];           // s(i), clamped to the tile
};

template <class E, int D, int CV>
constexpr size_t chunk_smem_bytes() {
    return sizeof(ChunkSmem<E, D, CV>);
}

template <class E, int D, int CV, bool DELTA>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(ChunkArgs a) {
    using T = typename E::T;
    using Frag = typename E::Frag;
    constexpr int NB = CV / 16;     // 16-row blocks per tile
    constexpr int KB = D / 16;      // 16-blocks of d_k
    constexpr int EPC = 16 / E::kBytes;  // elements per 16-byte chunk
    constexpr int NVS = D / 64;     // value slices per (batch, head)
    __shared__ ChunkSmem<E, D, CV> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int grp = lane >> 4;
    const int lr = lane & 15;

    // XCD-aware mapping: workgroup i runs on XCD i % 8; keep the slices of a
    // sequence on one XCD.
    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int jj = blk >> 3;
    const int bh = (jj / NVS) * 8 + xcd;
    const int vs = jj % NVS;
    if (bh >= a.BH) return;
    const int v0 = vs * 64;

    const int T_ = a.T;
    const int W = a.W;
    const int Wv = (a.norm == kNormWindow) ? W : 1;
    const int Ct = CV / Wv;          // time steps per tile
    const int NVR = Ct * Wv;         // used virtual rows
    const float eps = a.eps;
    const bool colnorm = (a.norm == kNormColumn);

    const T* qg = static_cast<const T*>(a.q) + (size_t)bh * T_ * D;
    const T* kg = static_cast<const T*>(a.k) + (size_t)bh * T_ * D;
    const T* vg = static_cast<const T*>(a.v) + (size_t)bh * T_ * D;
    const T* kp = a.k_prev ? static_cast<const T*>(a.k_prev) + (size_t)bh * W * D : nullptr;
    const T* vp = (a.v_prev && W > 1) ? static_cast<const T*>(a.v_prev) + (size_t)bh * (W - 1) * D
                                      : nullptr;
    const float* alg = a.alpha + (size_t)bh * T_;
    const float* etg = a.eta + (size_t)bh * T_;
    T* og = static_cast<T*>(a.o) + (size_t)bh * T_ * D;

    // State slice as accumulators of S^T: Sacc[kb][r] = S[v][k],
    // v = v0 + 16*wave + lr, k = 16*kb + 4*grp + r.
    const int vcol = v0 + 16 * wave + lr;
    f32x4 Sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        if (a.S0) {
            Sacc[kb] = *reinterpret_cast<const f32x4*>(a.S0 + ((size_t)bh * D + vcol) * D +
                                                       16 * kb + 4 * grp);
        } else {
            Sacc[kb] = zero4();
        }
    }

    const uint4 z16 = make_uint4(0, 0, 0, 0);

    for (int t0 = 0; t0 < T_; t0 += Ct) {
        // ---------------- (L) stage the tile in LDS ----------------
        for (int c = tid; c < CV * (D / EPC); c += 256) {
            const int i = c / (D / EPC);
            const int col = (c % (D / EPC)) * EPC;
            const int s = i / Wv, w = i - (i / Wv) * Wv;
            const int t = t0 + s;
            const int tau = t - w - 1;  // key index of x_i = k_{t-w-1}
            uint4 val = z16;
            if (i < NVR && t < T_) {
                if (tau >= 0) {
                    val = *reinterpret_cast<const uint4*>(kg + (size_t)tau * D + col);
                } else if (kp) {
                    val = *reinterpret_cast<const uint4*>(kp + (size_t)(W + tau) * D + col);
                }
            }
            *reinterpret_cast<uint4*>(&sm.X[i][col]) = val;
            if (!colnorm) {
                const T* e = reinterpret_cast<const T*>(&val);
#pragma unroll
                for (int u = 0; u < EPC; ++u) sm.OmT[col + u][i] = e[u];
            }
        }
        for (int c = tid; c < CV * (D / EPC); c += 256) {
            const int s = c / (D / EPC);
            const int col = (c % (D / EPC)) * EPC;
            uint4 val = z16;
            if (s < Ct && t0 + s < T_)
                val = *reinterpret_cast<const uint4*>(qg + (size_t)(t0 + s) * D + col);
            *reinterpret_cast<uint4*>(&sm.Q[s][col]) = val;
        }
        for (int c = tid; c < CV * (64 / EPC); c += 256) {
            const int i = c / (64 / EPC);
            const int col = (c % (64 / EPC)) * EPC;
            const int s = i / Wv, w = i - (i / Wv) * Wv;
            const int t = t0 + s;
            const int tv = t - w;  // value index of y_i = v_{t-w}
            uint4 val = z16;
            if (i < NVR && t < T_) {
                if (tv >= 0) {
                    val = *reinterpret_cast<const uint4*>(vg + (size_t)tv * D + v0 + col);
                } else if (vp) {
                    val = *reinterpret_cast<const uint4*>(vp + (size_t)(W - 1 + tv) * D + v0 + col);
                }
            }
            *reinterpret_cast<uint4*>(&sm.Y[i][col]) = val;
        }
        if (tid < CV) {
            const int t = t0 + tid;
            const bool ok = (tid < Ct) && (t < T_);
            sm.alpha[tid] = ok ? alg[t] : 1.0f;   // padding steps are identity steps
            sm.eta[tid] = ok ? etg[t] : 0.0f;
        }
        __syncthreads();

        // ---------------- (N) norms, decay scan, write vectors ----------------
        {
            const int i = tid >> 2, part = tid & 3;
            float n2 = 0.f, n1 = 0.f;
            if (i < CV) {
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
        if (wave == 0) {
            const int j = lane;
            float lg = (j < Ct && j < CV) ? logf(sm.alpha[j]) : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(lg, off, 64);
                if (j >= off) lg += y;
            }
            const float glast = __shfl(lg, Ct - 1, 64);
            // window normalizer b_s (lane s)
            float bwin = 0.f;
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
                sm.g[j] = lg;
                sm.gq[j] = __expf(lg);
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
                sm.rs[j] = r;
                sm.step[j] = sj;
                sm.gam[j] = __expf(gsj);
                sm.hrow[j] = __expf(glast - gsj) * r;
            }
        }
        if (colnorm) {
            // u_j = eta x_j / (|x_j| ||x||_1 + eps), written row-major and transposed
            for (int c = tid; c < CV * (D / EPC); c += 256) {
                const int i = c / (D / EPC);
                const int col = (c % (D / EPC)) * EPC;
                const int s = min(i / Wv, Ct - 1);
                const float et = sm.eta[s];
                const float l1 = sm.l1[i];
                T out[EPC];
#pragma unroll
                for (int u = 0; u < EPC; ++u) {
                    const float x = E::to_f(sm.X[i][col + u]);
                    const float den = fabsf(x) * l1 + eps;
                    const float uu = (i < NVR && den > 0.f) ? et * x / den : 0.f;
                    out[u] = E::from_f(uu);
                    sm.OmT[col + u][i] = out[u];
                }
                *reinterpret_cast<uint4*>(&sm.Om[i][col]) = *reinterpret_cast<const uint4*>(out);
            }
        }
        __syncthreads();

        // ---------------- (G) Gram blocks, masked and decayed ----------------
        {
            const T(*OmSrc)[D + ChunkSmem<E, D, CV>::PADE] = colnorm ? sm.Om : sm.X;
            const int NBQ = (Ct + 15) / 16;
            int q = 0;
            if (DELTA) {
                for (int bi = 0; bi < NB; ++bi) {
                    for (int bj = 0; bj <= bi; ++bj, ++q) {
                        if ((q & 3) != wave) continue;
                        f32x4 acc = zero4();
#pragma unroll
                        for (int m = 0; m < D / 32; ++m) {
                            const Frag a0 = E::load(&sm.X[16 * bi + lr][32 * m + 4 * grp]);
                            const Frag a1 = E::load(&sm.X[16 * bi + lr][32 * m + 16 + 4 * grp]);
                            const Frag b0 = E::load(&OmSrc[16 * bj + lr][32 * m + 4 * grp]);
                            const Frag b1 = E::load(&OmSrc[16 * bj + lr][32 * m + 16 + 4 * grp]);
                            acc = E::mma32(a0, a1, b0, b1, acc);
                        }
                        const int j = 16 * bj + lr;
                        const int sj = sm.step[j];
                        const float gj = sm.g[sj];
                        const float rj = sm.rs[j];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = 16 * bi + 4 * grp + r;
                            const int si = sm.step[i];
                            const float val = (sj < si) ? __expf(sm.g[si] - gj) * acc[r] * rj : 0.f;
                            sm.An[i][j] = E::from_f(-val);
                            if (bi == bj) sm.Adg[bi][4 * grp + r][lr] = val;
                        }
                    }
                }
            }
            for (int bt = 0; bt < NBQ; ++bt) {
                for (int bj = 0; bj < NB; ++bj) {
                    if ((16 * bj) / Wv > 16 * bt + 15) continue;
                    const int qq = q++;
                    if ((qq & 3) != wave) continue;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int m = 0; m < D / 32; ++m) {
                        const Frag a0 = E::load(&sm.Q[16 * bt + lr][32 * m + 4 * grp]);
                        const Frag a1 = E::load(&sm.Q[16 * bt + lr][32 * m + 16 + 4 * grp]);
                        const Frag b0 = E::load(&OmSrc[16 * bj + lr][32 * m + 4 * grp]);
                        const Frag b1 = E::load(&OmSrc[16 * bj + lr][32 * m + 16 + 4 * grp]);
                        acc = E::mma32(a0, a1, b0, b1, acc);
                    }
                    const int j = 16 * bj + lr;
                    const int sj = sm.step[j];
                    const float gj = sm.g[sj];
                    const float rj = sm.rs[j];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * bt + 4 * grp + r;
                        const float val =
                            (sj <= t && t < Ct) ? __expf(sm.g[t] - gj) * acc[r] * rj : 0.f;
                        sm.P[t][j] = E::from_f(val);
                    }
                }
            }
        }
        __syncthreads();

        // ---------------- (I) inverses of the diagonal blocks of I + A ----------------
        if (DELTA) {
            if (wave < NB && lane < 16) {
                const int bi = wave, c = lane;
                float tcol[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
                    for (int j = 0; j < i; ++j) acc -= sm.Adg[bi][i][j] * tcol[j];
                    tcol[i] = acc;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) sm.Td[bi][i][c] = E::from_f(tcol[i]);
            }
            __syncthreads();
        }

        // ---------------- (C) sequential part for this wave's 16 value columns ----------------
        {
            const int NBQ = (Ct + 15) / 16;
            Frag SB[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) SB[kb] = E::pack(Sacc[kb]);

            f32x4 Dl[NB];
            Frag DB[NB];
            if (DELTA) {
                // residuals R = Y - diag(gam) X S0^T
                f32x4 R[NB];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int m = 0; m < D / 32; ++m) {
                        const Frag a0 = E::load(&sm.X[16 * rb + lr][32 * m + 4 * grp]);
                        const Frag a1 = E::load(&sm.X[16 * rb + lr][32 * m + 16 + 4 * grp]);
                        acc = E::mma32(a0, a1, SB[2 * m], SB[2 * m + 1], acc);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * rb + 4 * grp + r;
                        R[rb][r] = E::to_f(sm.Y[i][16 * wave + lr]) - sm.gam[i] * acc[r];
                    }
                }
                // block forward substitution: Delta_b = T_bb (R_b - sum_{c<b} A_bc Delta_c)
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    f32x4 acc = R[rb];
#pragma unroll
                    for (int cb = 0; cb < rb; ++cb)
                        acc = E::mma16(E::load(&sm.An[16 * rb + lr][16 * cb + 4 * grp]), DB[cb],
                                       acc);
                    Dl[rb] = E::mma16(E::load(&sm.Td[rb][lr][4 * grp]), E::pack(acc), zero4());
                    DB[rb] = E::pack(Dl[rb]);
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
                if (tb >= NBQ) break;
                f32x4 acc = zero4();
#pragma unroll
                for (int m = 0; m < D / 32; ++m) {
                    const Frag a0 = E::load(&sm.Q[16 * tb + lr][32 * m + 4 * grp]);
                    const Frag a1 = E::load(&sm.Q[16 * tb + lr][32 * m + 16 + 4 * grp]);
                    acc = E::mma32(a0, a1, SB[2 * m], SB[2 * m + 1], acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= sm.gq[16 * tb + 4 * grp + r];
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) {
                    if ((16 * cb) / Wv > 16 * tb + 15) continue;
                    acc = E::mma16(E::load(&sm.P[16 * tb + lr][16 * cb + 4 * grp]), DB[cb], acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tb + 4 * grp + r;
                    if (t < Ct && t0 + t < T_) og[(size_t)(t0 + t) * D + vcol] = E::from_f(acc[r]);
                }
            }

            // state update S^T = exp(g_last) S0^T + Omega^T diag(hrow) Delta
            Frag HB[NB];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                f32x4 h;
#pragma unroll
                for (int r = 0; r < 4; ++r) h[r] = sm.hrow[16 * cb + 4 * grp + r] * Dl[cb][r];
                HB[cb] = E::pack(h);
            }
            const float glq = sm.gq[Ct - 1];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x4 acc = Sacc[kb] * glq;
                if constexpr (NB == 1) {
                    acc = E::mma16(E::load(&sm.OmT[16 * kb + lr][4 * grp]), HB[0], acc);
                } else {
#pragma unroll
                    for (int m = 0; m < NB / 2; ++m) {
                        const Frag a0 = E::load(&sm.OmT[16 * kb + lr][32 * m + 4 * grp]);
                        const Frag a1 = E::load(&sm.OmT[16 * kb + lr][32 * m + 16 + 4 * grp]);
                        acc = E::mma32(a0, a1, HB[2 * m], HB[2 * m + 1], acc);
                    }
                }
                Sacc[kb] = acc;
            }
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

template <class E, int D, int CV, bool DELTA>
static hipError_t launch_one(const ChunkArgs& a, hipStream_t stream) {
    const int nvs = D / 64;
    const int bh8 = (a.BH + 7) / 8 * 8;
    dim3 grid(bh8 * nvs), block(256);
    hipLaunchKernelGGL((chunk_fwd_kernel<E, D, CV, DELTA>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <class E, int D, bool DELTA>
static hipError_t launch_cv(const ChunkArgs& a, int chunk, hipStream_t stream) {
    switch (chunk) {
        case 16: return launch_one<E, D, 16, DELTA>(a, stream);
        case 32: return launch_one<E, D, 32, DELTA>(a, stream);
        case 64:
            if constexpr (chunk_smem_bytes<E, D, 64>() <= 160 * 1024)
                return launch_one<E, D, 64, DELTA>(a, stream);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <class E, bool DELTA>
static hipError_t launch_d(const ChunkArgs& a, int D, int chunk, hipStream_t stream) {
    if (D == 64) return launch_cv<E, 64, DELTA>(a, chunk, stream);
    if (D == 128) return launch_cv<E, 128, DELTA>(a, chunk, stream);
    return hipErrorInvalidValue;
}

bool chunk_supported(int dt, int D, int chunk) {
    if (D != 64 && D != 128) return false;
    if (chunk != 16 && chunk != 32 && chunk != 64) return false;
    if (chunk == 64 && dt == 0 && D == 128)
        return chunk_smem_bytes<EFp32, 128, 64>() <= 160 * 1024;
    return true;
}

hipError_t launch_chunk(const ChunkArgs& a, int dt, int D, int chunk, bool delta,
                        hipStream_t stream) {
    if (dt == 1)
        return delta ? launch_d<EBf16, true>(a, D, chunk, stream)
                     : launch_d<EBf16, false>(a, D, chunk, stream);
    return delta ? launch_d<EFp32, true>(a, D, chunk, stream)
                 : launch_d<EFp32, false>(a, D, chunk, stream);
}

}  // namespace falcon
