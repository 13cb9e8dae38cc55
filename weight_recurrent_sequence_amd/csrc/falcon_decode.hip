// falcon_decode.hip -- one decode step of the Falcon recurrence for many
// independent heads (gfx950).
//
// One step of the recurrence ("Fast Weight Attention for Continual Learning",
// authors' abstract: prefix-aligned example (k_{t-1}, v_t), read after the
// write; KLA abstract: normalized step, decay then delta write), for
// Falcon-1/1A (u = eta x / (||x||^2 + eps)) and Falcon-2/2A (per-column
// normalizer u_j = eta x_j / (|x_j| ||x||_1 + eps)):
//     x = k_cache (same-step pairs: x = k),  S' = alpha S,  r = v - S'x  (A forms: r = v)
//     S = S' + r u^T,  o = S q = alpha S q + (u . q) r,  k_cache <- k
// S is read once and written once: Sx and Sq come from the same pass over
// the registers, and o is formed without a second read of S.
//
// Work decomposition: one 256-thread workgroup per head; the d_v x d_k fp32
// state (64 KiB at d = 128) sits in registers, 64 floats per lane.  Lane
// groups of d/16 consecutive lanes share a row, each lane holding 16 columns
// as four 16-byte pieces spaced so that one load instruction of a wave
// covers whole 128-byte row segments.  Row dot products and the norms of x
// are reduced within the lane group with DPP lane permutations.  The kernel
// is bound by HBM: 2 * d_v * d_k * 4 bytes of state traffic per head-step.
#include "falcon_device.h"
#include "falcon_internal.h"

namespace falcon {

// Feature map on one row held as 16 entries per lane by a group of G lanes:
// L2 normalization (the row norm a DPP sum over the group; 0 for a zero row)
// or SiLU elementwise.  phi 0 leaves the row as it is.
template <int G>
__device__ __forceinline__ void phi_row(int phi, float (&x)[16]) {
    if (phi == 1) {
        float n2 = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) n2 += x[c] * x[c];
        n2 = group_sum_dpp<G>(n2);
        const float sc = n2 > 0.f ? rsqrtf(n2) : 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) x[c] *= sc;
    } else if (phi == 2) {
#pragma unroll
        for (int c = 0; c < 16; ++c) x[c] = x[c] / (1.f + __expf(-x[c]));
    }
}

// An empty asm statement that takes two values as register inputs: every
// load whose data feeds them has returned that data (so it is complete)
// before the statement, and the statement, being volatile, stays on its side
// of a barrier that follows it.
__device__ __forceinline__ void consumed(float a, float b) {
    asm volatile("" ::"v"(a), "v"(b));
}

template <class E, int D>
__global__ __launch_bounds__(256, 2) void decode_step_kernel(DecodeArgs a) {
    using T = typename E::T;
    constexpr int LPR = D / 16;               // lanes per row
    constexpr int ROWS_PER_PASS = 256 / LPR;
    constexpr int RPT = D / ROWS_PER_PASS;    // rows per thread
    const int tid = threadIdx.x;
    const int seg = tid % LPR;
    const int row0 = tid / LPR;
    const size_t head = blockIdx.x;

    float* S = a.S + head * D * D;
    T* kc = static_cast<T*>(a.k_cache) + head * D;
    const T* qh = static_cast<const T*>(a.q) + head * D;
    const T* kh = static_cast<const T*>(a.k) + head * D;
    const T* vh = static_cast<const T*>(a.v) + head * D;
    T* oh = static_cast<T*>(a.o) + head * D;
    const float al = a.alpha[head];
    const float et = a.eta[head];
    // Everything this thread reads is requested up front (targets and the new
    // key too), so no wait further down has a load queued behind a store.
    const T knew = kh[tid < D ? tid : 0];
    T vraw[RPT];  // converted where used, so the load stays in flight meanwhile
#pragma unroll
    for (int p = 0; p < RPT; ++p) vraw[p] = vh[row0 + ROWS_PER_PASS * p];

    // columns of this lane: 4*seg + 4*LPR*j + e, j, e in 0..3
    const T* xh = a.lag ? kc : kh;
    float x[16], qv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = 4 * seg + 4 * LPR * j;
        const typename E::Frag xf = E::load(xh + c), qf = E::load(qh + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[4 * j + e] = E::to_f((T)xf[e]);
            qv[4 * j + e] = E::to_f((T)qf[e]);
        }
    }
    f32x4 s[RPT][4];
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const int row = row0 + ROWS_PER_PASS * p;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s[p][j] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(S + (size_t)row * D + 4 * seg + 4 * LPR * j));
    }
    phi_row<LPR>(a.phi, x);
    phi_row<LPR>(a.phi, qv);

    float n2 = 0.f, n1 = 0.f, xq = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        n2 += x[c] * x[c];
        n1 += fabsf(x[c]);
        xq += x[c] * qv[c];
    }
    n2 = group_sum_dpp<LPR>(n2);
    n1 = group_sum_dpp<LPR>(n1);
    // Every lane has now consumed the previous key: its x values entered the
    // norms, and the empty asm below takes n2 and n1 as register inputs, so
    // the loads of the cached key have returned their data (they are
    // complete) before this wave reaches the barrier; neither the asm nor the
    // barrier can be moved across the other.  After the barrier k_cache may be
    // overwritten.  The barrier orders no memory besides that, so it waits for
    // no other load in flight (the state's).
    consumed(n2, n1);
    __builtin_amdgcn_s_barrier();
    if (tid < D) kc[tid] = knew;
    float u[16];
    float uq = 0.f;
    if (a.norm == kNormScalar) {
        const float den = n2 + a.eps;
        const float b = den > 0.f ? et / den : 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) u[c] = b * x[c];
        uq = b * group_sum_dpp<LPR>(xq);
    } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const float den = fabsf(x[c]) * n1 + a.eps;
            u[c] = den > 0.f ? et * x[c] / den : 0.f;
            uq += u[c] * qv[c];
        }
        uq = group_sum_dpp<LPR>(uq);
    }

#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const int row = row0 + ROWS_PER_PASS * p;
        float sx = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sx += s[p][j][e] * x[4 * j + e];
                sq += s[p][j][e] * qv[4 * j + e];
            }
        sx = group_sum_dpp<LPR>(sx);
        sq = group_sum_dpp<LPR>(sq);
        const float vr = E::to_f(vraw[p]);
        const float r = a.delta ? vr - al * sx : vr;
        if (seg == 0) oh[row] = E::from_f(al * sq + uq * r);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 nv;
#pragma unroll
            for (int e = 0; e < 4; ++e) nv[e] = al * s[p][j][e] + r * u[4 * j + e];
            __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + (size_t)row * D + 4 * seg + 4 * LPR * j));
        }
    }
}

bool decode_supported(int dt, int D) { return (dt == 0 || dt == 1) && (D == 64 || D == 128); }

template <class E, int D>
static hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_step_kernel<E, D>), dim3(a.NH), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dt, int D, hipStream_t stream) {
    if (dt == 1) {
        if (D == 64) return launch_dec<EBf16, 64>(a, stream);
        if (D == 128) return launch_dec<EBf16, 128>(a, stream);
    } else {
        if (D == 64) return launch_dec<EFp32, 64>(a, stream);
        if (D == 128) return launch_dec<EFp32, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace falcon

namespace falcon {

// ---------------------------------------------------------------------------
// Falcon-3 / Falcon-3A decode step: a window of W prefix-aligned pairs
// ("Fast Weight Attention for Continual Learning", authors' abstract: the
// sliding-window mini-batch variant).  With x_w = k_{t-1-w} (k_cache slot w;
// same-step pairs: x_w = k_{t-w}, the new key for w = 0 and slot w-1 after)
// and y_w = v_{t-w} (y_0 = v, y_w = v_cache slot w-1):
//     S' = alpha S,  b = eta / (sum_w ||x_w||^2 + eps)
//     S  = S' + b sum_w r_w x_w^T,  r_w = y_w - S' x_w  (3A: r_w = y_w)
//     o  = S q = alpha S q + b sum_w r_w (x_w . q)
// then both caches move one slot (the new key and value enter at slot 0).
// One workgroup per head, as in the single-pair step: the state rows and the
// W keys' column slices sit in registers, S is read and written once.  Every
// thread shifts only its own column of the caches, after a barrier that every
// wave reaches only once its own reads of the caches have returned their
// data, so no thread overwrites a cache element another thread still has to
// read.
// ---------------------------------------------------------------------------
template <class E, int D, int W>
__global__ __launch_bounds__(256, 2) void decode_window_kernel(DecodeWinArgs a) {
    using T = typename E::T;
    constexpr int LPR = D / 16;
    constexpr int ROWS_PER_PASS = 256 / LPR;
    constexpr int RPT = D / ROWS_PER_PASS;
    __shared__ float ys[W][D];  // targets y_w of every row
    const int tid = threadIdx.x;
    const int seg = tid % LPR;
    const int row0 = tid / LPR;
    const size_t head = blockIdx.x;

    float* S = a.S + head * D * D;
    T* kc = static_cast<T*>(a.k_cache) + head * W * D;
    T* vc = W > 1 ? static_cast<T*>(a.v_cache) + head * (W - 1) * D : nullptr;
    const T* qh = static_cast<const T*>(a.q) + head * D;
    const T* kh = static_cast<const T*>(a.k) + head * D;
    const T* vh = static_cast<const T*>(a.v) + head * D;
    T* oh = static_cast<T*>(a.o) + head * D;
    const float al = a.alpha[head];
    const float et = a.eta[head];

    // ---- every read is requested first ----
    // this thread's column of both caches and of the new key and value
    const int col = tid < D ? tid : 0;
    T kcol[W], vcol[W];  // kcol[w] = k_cache[w][col]; vcol[0] = v[col], vcol[w] = v_cache[w-1][col]
#pragma unroll
    for (int w = 0; w < W; ++w) kcol[w] = kc[(size_t)w * D + col];
    vcol[0] = vh[col];
#pragma unroll
    for (int w = 1; w < W; ++w) vcol[w] = vc[(size_t)(w - 1) * D + col];
    const T knew = kh[col];
    // columns of this lane: 4*seg + 4*LPR*j + e, j, e in 0..3
    float x[W][16], qv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = 4 * seg + 4 * LPR * j;
        const typename E::Frag qf = E::load(qh + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[4 * j + e] = E::to_f((T)qf[e]);
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const T* xw = (w + a.lag == 0) ? kh : kc + (size_t)(w + a.lag - 1) * D;
            const typename E::Frag xf = E::load(xw + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[w][4 * j + e] = E::to_f((T)xf[e]);
        }
    }
    f32x4 s[RPT][4];
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const int row = row0 + ROWS_PER_PASS * p;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s[p][j] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(S + (size_t)row * D + 4 * seg + 4 * LPR * j));
    }

    phi_row<LPR>(a.phi, qv);
#pragma unroll
    for (int w = 0; w < W; ++w) phi_row<LPR>(a.phi, x[w]);

    // ---- targets to LDS; window norm and x_w . q ----
    if (tid < D) {
#pragma unroll
        for (int w = 0; w < W; ++w) ys[w][tid] = E::to_f(vcol[w]);
    }
    float n2 = 0.f, xq[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            n2 += x[w][c] * x[w][c];
            d += x[w][c] * qv[c];
        }
        xq[w] = group_sum_dpp<LPR>(d);
    }
    n2 = group_sum_dpp<LPR>(n2);
    const float den = n2 + a.eps;
    const float bw = den > 0.f ? et / den : 0.f;
    // Every lane has consumed its cache reads (they entered the sums above,
    // and the empty asm takes the sums as register inputs, so those loads
    // have returned their data before the wave reaches the barrier) and the
    // targets are in LDS: the caches may now move.  The barrier orders LDS
    // only, so no other load in flight (the state's) is waited for.
    consumed(n2, xq[0]);
    lds_barrier();
    if (tid < D) {
#pragma unroll
        for (int w = W - 1; w >= 1; --w) kc[(size_t)w * D + tid] = kcol[w - 1];
        kc[tid] = knew;
#pragma unroll
        for (int w = W - 1; w >= 2; --w) vc[(size_t)(w - 1) * D + tid] = vcol[w - 1];
        if (W > 1) vc[tid] = vcol[0];
    }

#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const int row = row0 + ROWS_PER_PASS * p;
        float sq = 0.f, sx[W];
#pragma unroll
        for (int w = 0; w < W; ++w) sx[w] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sv = s[p][j][e];
                sq += sv * qv[4 * j + e];
                if (a.delta) {
#pragma unroll
                    for (int w = 0; w < W; ++w) sx[w] += sv * x[w][4 * j + e];
                }
            }
        sq = group_sum_dpp<LPR>(sq);
        float r[W], orow = al * sq;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float y = ys[w][row];
            r[w] = bw * (a.delta ? y - al * group_sum_dpp<LPR>(sx[w]) : y);  // b r_w
            orow += r[w] * xq[w];
        }
        if (seg == 0) oh[row] = E::from_f(orow);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 nv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float acc = al * s[p][j][e];
#pragma unroll
                for (int w = 0; w < W; ++w) acc += r[w] * x[w][4 * j + e];
                nv[e] = acc;
            }
            __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + (size_t)row * D + 4 * seg + 4 * LPR * j));
        }
    }
}

template <class E, int D, int W>
static hipError_t launch_decw(const DecodeWinArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_window_kernel<E, D, W>), dim3(a.NH), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_decw_w(const DecodeWinArgs& a, hipStream_t stream) {
    switch (a.W) {
        case 1: return launch_decw<E, D, 1>(a, stream);
        case 2: return launch_decw<E, D, 2>(a, stream);
        case 3: return launch_decw<E, D, 3>(a, stream);
        case 4: return launch_decw<E, D, 4>(a, stream);
        case 5: return launch_decw<E, D, 5>(a, stream);
        case 6: return launch_decw<E, D, 6>(a, stream);
        case 7: return launch_decw<E, D, 7>(a, stream);
        case 8: return launch_decw<E, D, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_window(const DecodeWinArgs& a, int dt, int D, hipStream_t stream) {
    if (dt == 1) {
        if (D == 64) return launch_decw_w<EBf16, 64>(a, stream);
        if (D == 128) return launch_decw_w<EBf16, 128>(a, stream);
    } else {
        if (D == 64) return launch_decw_w<EFp32, 64>(a, stream);
        if (D == 128) return launch_decw_w<EFp32, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace falcon
