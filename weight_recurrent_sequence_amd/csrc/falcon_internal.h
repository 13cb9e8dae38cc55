// falcon_internal.h -- argument blocks and launchers shared by the host
// library's translation units (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace falcon {

// How the write vector of a step is normalized.
enum NormKind : int {
    kNormScalar = 1,  // Falcon-1/1A: u = eta x / (||x||^2 + eps)
    kNormColumn = 2,  // Falcon-2/2A: u_j = eta x_j / (|x_j| ||x||_1 + eps)
    kNormWindow = 3   // Falcon-3/3A: b = eta / (sum_w ||x_{t-w}||^2 + eps), writes b x_{t-w}
};

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* eta;
    const float* S0;
    const void* k_prev;
    const void* v_prev;
    void* o;
    float* S_final;
    int BH;      // batch * heads (packed: sequences * heads)
    int T;       // steps per sequence (packed: the longest sequence allowed)
    // Packed sequences: q, k, v, o are [H, Ttot, d] and alpha, eta [H, Ttot];
    // sequence n of head h covers rows cu[n] .. cu[n+1] of head h's plane and
    // is "batch row" n * H + h for S0, S_final, k_prev, v_prev.  cu is NULL
    // for the batched layout [B, H, T, d].
    const int* cu;
    int H;
    int Ttot;
    // Packed calls: workspace room for the schedule (N + N+1 ints): the
    // sequences longest first (`order`) and the prefix sums of their tile
    // counts (`toff`), both written on the device before the kernels run and
    // set by the launcher (NULL: natural order, every (row, tile) job).
    int* order_ws;
    const int* order;
    const int* toff;
    // Packed calls: the intra-chunk jobs, 4 ints each (row, tile, first row of
    // the sequence in its head's plane, its length), written with the
    // schedule; NULL: jobs are decoded from their index.
    const int* jobs;
    int W;       // window (1 unless kNormWindow)
    int lag;     // key of step t's pair w is k_{t-w-lag}: 1 prefix-aligned, 0 same-step
    int norm;    // NormKind
    float eps;
    // Feature map on keys and queries (0 identity, 1 L2, 2 SiLU).  With a map,
    // the intra-chunk kernel writes the mapped keys, queries and halo keys to
    // kphi, qphi (layout of k, q) and kpphi (layout of k_prev), and the state
    // pass reads those instead.
    int phi;
    void* kphi;
    void* qphi;
    void* kpphi;
    // Checkpoints for the backward pass (bf16 state pass): when ck_s is set,
    // the state pass also writes, for every (row, tile), the state at the tile
    // start rounded to bf16 (d_v x d_k) to ck_s and the tile's Delta (the
    // residuals at the decayed state; the targets for the inner-product
    // family, d_v x CV) to ck_d, both in 16-column blocks: entry (v, c) at
    // ((c / 16) * d_v + v) * 16 + c % 16.  o may then be NULL (not written).
    void* ck_s = nullptr;
    void* ck_d = nullptr;
    // Per-column rule, bf16: the write vectors u of every (row, tile), CV x d
    // bf16 rows, written by the intra-chunk kernel after the records and read
    // by the state pass (set by the launcher).
    void* uws = nullptr;
};

struct DecodeArgs {
    float* S;
    void* k_cache;
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* eta;
    void* o;
    int NH;      // sequences * heads
    int norm;    // kNormScalar or kNormColumn
    int delta;   // 1: regression (residual write), 0: inner-product write
    int lag;     // 1: x = k_cache (prefix-aligned), 0: x = k (same-step)
    int phi;     // feature map on x and q (0 identity, 1 L2, 2 SiLU); caches stay raw
    float eps;
};

struct DecodeWinArgs {
    float* S;
    void* k_cache;       // [NH, W, d]: slot w holds k_{t-1-w}
    void* v_cache;       // [NH, W-1, d]: slot w-1 holds v_{t-w} (unused when W = 1)
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* eta;
    void* o;
    int NH;
    int W;
    int delta;   // 1: Falcon-3 (residual writes), 0: Falcon-3A
    int lag;     // pair w's key is k_{t-w-lag}: slot w+lag-1 of k_cache, or k when w+lag = 0
    int phi;     // feature map on the keys and q (0 identity, 1 L2, 2 SiLU); caches stay raw
    float eps;
};

// Backward pass of the chunk form (bf16, batched layout).  The forward is
// re-run first with checkpoints (ChunkArgs::ck_s / ck_d); then a reverse scan
// over the tiles carries the state gradient and writes dv and the state
// gradient at every tile end (ck_ds); then one workgroup per tile forms dq,
// dk, dalpha and deta.
struct BwdArgs {
    const void* q;        // queries and keys the kernels contract with (the
    const void* k;        // mapped copies when a feature map is on)
    const void* k_prev;   // halo keys (mapped copy likewise), or NULL
    const void* q_raw;    // the caller's queries, keys and halo keys, for the
    const void* k_raw;    // feature map's own derivative
    const void* kp_raw;
    const float* alpha;
    const float* eta;
    const void* d_o;      // [BH, T, d]
    const float* dS_final;  // [BH, d, d] or NULL (zero)
    void* dq;
    void* dk;
    void* dv;
    float* dalpha;
    float* deta;
    float* dS0;           // or NULL
    void* dk_prev;        // or NULL
    const void* rec;      // records of the intra-chunk kernel
    // checkpoints, per (row, tile), in 16-column blocks ([c/16][v][16]):
    const void* ck_s;     // bf16 state at each tile start (d x d)
    const void* ck_d;     // bf16 Delta of each tile (d x CV)
    void* ck_ds;          // bf16 state gradient at each tile end (d x d)
    // windows above one: per-virtual-row gradients of the targets (ck_r) and
    // keys (ck_x, before the feature map), bf16 [BH][ntiles][CV][d], summed
    // into dv / dk by a gather (a key or value serves W rows, which can sit in
    // two tiles)
    void* ck_r;
    void* ck_x;
    void* dv_prev;        // [BH, W-1, d] or NULL (windows above one)
    int BH, T, ntiles, W, lag, phi;
    int norm;             // NormKind
    float eps;
    // packed sequences (as ChunkArgs): rows cu[n] .. cu[n+1] of head h's
    // plane are "batch row" n * H + h; T is the longest sequence allowed and
    // ntiles its tile count.  NULL for the batched layout.
    const int* cu;
    int H;
    int Ttot;
};
bool chunk_bwd_supported(int dt, int D, int chunk, int norm, int window);
hipError_t launch_chunk_bwd(const BwdArgs& a, int D, int chunk, bool delta, hipStream_t stream);

// Packed calls: orders the sequences longest first and lists the tiles of Ct
// steps that exist (b.order, b.toff, b.jobs); nothing for batched calls.
hipError_t launch_packed_schedule(const ChunkArgs& a, int Ct, int ntiles, ChunkArgs& b,
                                  hipStream_t stream);

// The window rules (W >= 2) at bf16 in the collapsed form: tiles of kWinC
// steps whose C + W - 1 distinct (key, value) pairs carry the state update.
constexpr int kWinC = 32;
size_t window_workspace_bytes(int BH, int T, bool delta, int D);
hipError_t launch_window(const ChunkArgs& a, int D, bool delta, void* ws, hipStream_t stream);

// The scalar inner-product rule (kNormScalar, or kNormWindow with W = 1) at
// bf16, 64-step tiles, no feature map and no checkpoints: intra-chunk work and
// state pass in one kernel (needs no workspace beyond a packed call's
// schedule).
bool fused_supported(const ChunkArgs& a, int dt, int D, int chunk, bool delta);
hipError_t launch_fused(const ChunkArgs& a, int D, bool delta, hipStream_t stream);

// True when launch_chunk runs a call without checkpoints (ck_s == NULL) on
// other kernels than the same call with them, so that a forward that keeps
// checkpoints takes its outputs from a separate run.
bool forward_kernel_differs(const ChunkArgs& a, int dt, int D, int chunk, bool delta);

// dt: 0 fp32, 1 bf16.  Return false when the combination is not built.
bool chunk_supported(int dt, int D, int chunk);
// Bytes of the per-tile records the intra-chunk kernel hands to the
// state-passing kernel (bf16 per-column rule: then its write vectors).
size_t chunk_workspace_bytes(int BH, int T, int dt, int chunk, int window, int norm, bool delta,
                             int D);
hipError_t launch_chunk(const ChunkArgs& a, int dt, int D, int chunk, bool delta, void* ws,
                        hipStream_t stream);
bool decode_supported(int dt, int D);
hipError_t launch_decode(const DecodeArgs& a, int dt, int D, hipStream_t stream);
hipError_t launch_decode_window(const DecodeWinArgs& a, int dt, int D, hipStream_t stream);

}  // namespace falcon
