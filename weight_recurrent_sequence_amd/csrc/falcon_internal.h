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

// dt: 0 fp32, 1 bf16.  Return false when the combination is not built.
bool chunk_supported(int dt, int D, int chunk);
// Bytes of the per-tile records the intra-chunk kernel hands to the
// state-passing kernel.
size_t chunk_workspace_bytes(int BH, int T, int dt, int chunk, int window, int norm, bool delta);
hipError_t launch_chunk(const ChunkArgs& a, int dt, int D, int chunk, bool delta, void* ws,
                        hipStream_t stream);
bool decode_supported(int dt, int D);
hipError_t launch_decode(const DecodeArgs& a, int dt, int D, hipStream_t stream);
hipError_t launch_decode_window(const DecodeWinArgs& a, int dt, int D, hipStream_t stream);

}  // namespace falcon
