// falcon_api.hip -- the C ABI declared in include/falcon.h: argument
// validation on the host (before any HIP call), then dispatch to the
// kernels on the caller's stream.  No allocation and no synchronization;
// the only global state is the per-device address of the built-in scratch
// buffer that falcon_chunk_fwd_noalloc uses.
#include <stdint.h>

#include <mutex>

#include "../../include/falcon.h"
#include "falcon_internal.h"

namespace {

// Scratch of falcon_chunk_fwd_noalloc: one buffer per device, a file-scope
// device array (every GPU the library runs on holds its own copy for the
// life of the process).  Host code never uses the array's name as an
// address: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// kept here.
__device__ __align__(256) unsigned char scratch[FALCON_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of the scratch array (looked up on the first
// call on that device).
int device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FALCON_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FALCON_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return FALCON_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FALCON_OK;
}

bool is_variant(int v) {
    return v == FALCON_F1 || v == FALCON_F2 || v == FALCON_F3 || v == FALCON_F1A ||
           v == FALCON_F2A || v == FALCON_F3A;
}

int norm_of(int v) {
    switch (v) {
        case FALCON_F1:
        case FALCON_F1A: return falcon::kNormScalar;
        case FALCON_F2:
        case FALCON_F2A: return falcon::kNormColumn;
        default: return falcon::kNormWindow;
    }
}

bool is_delta(int v) { return v == FALCON_F1 || v == FALCON_F2 || v == FALCON_F3; }

// The variant argument: a variant code, optionally OR-ed with FALCON_SAME_STEP
// and with one of FALCON_PHI_L2 / FALCON_PHI_SILU.  Splits it into the code,
// the key lag (1: pair (k_{t-1}, v_t), 0: (k_t, v_t)) and the feature map
// (0 identity, 1 L2, 2 SiLU); returns false for unknown or conflicting flags.
bool split_variant(int var, int* base, int* lag, int* phi = nullptr) {
    if (var & ~(0xFF | FALCON_SAME_STEP | FALCON_PHI_L2 | FALCON_PHI_SILU)) return false;
    if ((var & FALCON_PHI_L2) && (var & FALCON_PHI_SILU)) return false;
    *base = var & 0xFF;
    *lag = (var & FALCON_SAME_STEP) ? 0 : 1;
    if (phi) *phi = (var & FALCON_PHI_L2) ? 1 : ((var & FALCON_PHI_SILU) ? 2 : 0);
    return true;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of the mapped keys, queries and halo keys (a feature map is
// selected): `rows` rows of dk entries twice, then BH * W halo rows.
size_t phi_bytes(size_t rows, size_t BH, int W, int dk, int dt) {
    const size_t es = dt == FALCON_BF16 ? 2 : 4;
    return 2 * align256(rows * dk * es) + align256(BH * W * dk * es);
}

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_chunk(const void* q, const void* k, const void* v, const float* alpha,
                const float* eta, const float* S0, const void* k_prev, const void* v_prev,
                const void* o, const float* S_final, int B, int H, int T, int dk, int dv,
                int dt, int var_arg, int window, int chunk, float eps) {
    int var = 0, lag = 1;
    if (!split_variant(var_arg, &var, &lag) || !is_variant(var)) return FALCON_ERR_UNSUPPORTED;
    if (dt != FALCON_FP32 && dt != FALCON_BF16) return FALCON_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return FALCON_ERR_SHAPE;
    if ((long long)B * H > (1LL << 28) || (long long)T * dk > (1LL << 40)) return FALCON_ERR_SHAPE;
    if (window < 1) return FALCON_ERR_SHAPE;
    const bool win = (var == FALCON_F3 || var == FALCON_F3A);
    if (!win && window != 1) return FALCON_ERR_SHAPE;
    if (window > 8) return FALCON_ERR_UNSUPPORTED;
    if (chunk != 16 && chunk != 32 && chunk != 64) return FALCON_ERR_UNSUPPORTED;
    if (window > chunk) return FALCON_ERR_UNSUPPORTED;
    if (dk != dv) return FALCON_ERR_UNSUPPORTED;
    if (!falcon::chunk_supported(dt, dk, chunk)) return FALCON_ERR_UNSUPPORTED;
    if (!(eps >= 0.0f)) return FALCON_ERR_SHAPE;  // also rejects NaN
    if (T > 0 && (!q || !k || !v || !alpha || !eta || !o)) return FALCON_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(S0) ||
        !aligned16(S_final) || !aligned16(k_prev) || !aligned16(v_prev) || !aligned4(alpha) ||
        !aligned4(eta))
        return FALCON_ERR_UNSUPPORTED;
    return FALCON_OK;
}

// Workspace of a forward call.  full: room for the split kernels' records as
// well (the backward's checkpoint runs and the saving forward run them for
// every rule); otherwise the window rules at bf16 without a feature map get
// their collapsed form's bytes only, the kernels falcon_chunk_fwd runs.
size_t fwd_ws(int B, int H, int T, int dk, int dv, falcon_dtype dt, falcon_variant var, int window,
              int chunk, bool full) {
    // Sizes only: pointers are not needed to size the workspace.
    const void* p = reinterpret_cast<const void*>(uintptr_t(256));
    if (check_chunk(p, p, p, (const float*)p, (const float*)p, nullptr, nullptr, nullptr, p,
                    nullptr, B, H, T, dk, dv, dt, var, window, chunk, 0.0f) != FALCON_OK)
        return 0;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    // the window rules at bf16 without a feature map run their collapsed
    // form: its records (and group states) only; everything else the split
    // kernels' records
    const bool collapsed = !full && dt == FALCON_BF16 && norm_of(base) == falcon::kNormWindow && window >= 2 && phi == 0;
    const size_t rec = align256(collapsed ? falcon::window_workspace_bytes(B * H, T, is_delta(base), dk)
                                          : falcon::chunk_workspace_bytes(B * H, T, (int)dt, chunk, window,
                                                                          norm_of(base), is_delta(base), dk));
    if (rec == 0 || phi == 0) return rec;
    return rec + phi_bytes((size_t)B * H * T, (size_t)B * H, window, dk, dt);
}

size_t fwd_varlen_ws(int N, int H, int max_seqlen, int dk, int dv, falcon_dtype dt,
                     falcon_variant var, int window, int chunk, bool full) {
    // the records, laid out per (sequence, head) with the longest sequence's
    // tile count, then the schedule: 2N+1 ints (the sequences' order, the
    // prefix sums of their tile counts) and, 256-byte aligned, a job table of
    // 4 ints per record slot
    const size_t rec = fwd_ws(N, H, max_seqlen, dk, dv, dt, var, window, chunk, full);
    if (rec == 0) return 0;
    const int Wv = (var & 0xFF) == FALCON_F3 || (var & 0xFF) == FALCON_F3A ? window : 1;
    const size_t slots = (size_t)N * H * ((max_seqlen + chunk / Wv - 1) / (chunk / Wv));
    return rec + ((2 * (size_t)N + 1) * sizeof(int) + 255) / 256 * 256 + slots * 4 * sizeof(int);
}

}  // namespace

extern "C" {

size_t falcon_chunk_fwd_workspace(int B, int H, int T, int dk, int dv, falcon_dtype dt,
                                  falcon_variant var, int window, int chunk) {
    return fwd_ws(B, H, T, dk, dv, dt, var, window, chunk, false);
}

// Where the mapped keys, queries and halo keys go (after the records).
void set_phi_buffers(falcon::ChunkArgs& a, void* ws, size_t rows, int BH, int W, int dk, int dt,
                     size_t rec) {
    const size_t es = dt == FALCON_BF16 ? 2 : 4;
    char* p = static_cast<char*>(ws) + rec;
    a.kphi = p;
    a.qphi = p + align256(rows * dk * es);
    a.kpphi = p + 2 * align256(rows * dk * es);
    (void)BH;
    (void)W;
}

int falcon_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                     const float* eta, const float* S0, const void* k_prev, const void* v_prev,
                     void* o, float* S_final, int B, int H, int T, int dk, int dv,
                     falcon_dtype dt, falcon_variant var, int window, int chunk, float eps,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = check_chunk(q, k, v, alpha, eta, S0, k_prev, v_prev, o, S_final, B, H, T, dk, dv,
                         dt, var, window, chunk, eps);
    if (st != FALCON_OK) return st;
    const size_t need = falcon_chunk_fwd_workspace(B, H, T, dk, dv, dt, var, window, chunk);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FALCON_ERR_WORKSPACE;
    if (T == 0 && S_final == nullptr) return FALCON_OK;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    falcon::ChunkArgs a;
    a.phi = phi;
    a.kphi = a.qphi = a.kpphi = nullptr;
    if (phi && need > 0)
        set_phi_buffers(a, workspace, (size_t)B * H * T, B * H, window, dk, dt,
                        align256(falcon::chunk_workspace_bytes(B * H, T, (int)dt, chunk, window,
                                                               norm_of(base), is_delta(base), dk)));
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.eta = eta;
    a.S0 = S0;
    a.k_prev = k_prev;
    a.v_prev = v_prev;
    a.o = o;
    a.S_final = S_final;
    a.BH = B * H;
    a.T = T;
    a.cu = nullptr;
    a.H = H;
    a.Ttot = T;
    a.order_ws = nullptr;
    a.order = nullptr;
    a.toff = nullptr;
    a.jobs = nullptr;
    a.W = window;
    a.lag = lag;
    a.norm = norm_of(base);
    a.eps = eps;
    hipError_t e = falcon::launch_chunk(a, (int)dt, dk, chunk, is_delta(base), workspace, stream);
    return e == hipSuccess ? FALCON_OK : FALCON_ERR_HIP;
}

size_t falcon_chunk_fwd_varlen_workspace(int N, int H, int max_seqlen, int dk, int dv,
                                         falcon_dtype dt, falcon_variant var, int window,
                                         int chunk) {
    return fwd_varlen_ws(N, H, max_seqlen, dk, dv, dt, var, window, chunk, false);
}

int falcon_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* alpha,
                            const float* eta, const float* S0, const void* k_prev,
                            const void* v_prev, void* o, float* S_final, const int* cu_seqlens,
                            int N, int H, int total_T, int max_seqlen, int dk, int dv,
                            falcon_dtype dt, falcon_variant var, int window, int chunk, float eps,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    // per-sequence checks as for N sequences of max_seqlen steps
    int st = check_chunk(q, k, v, alpha, eta, S0, k_prev, v_prev, o, S_final, N, H, max_seqlen,
                         dk, dv, dt, var, window, chunk, eps);
    if (st != FALCON_OK) return st;
    if (total_T < 0 || (long long)H * total_T > (1LL << 40) / (dk > 0 ? dk : 1))
        return FALCON_ERR_SHAPE;
    if (!cu_seqlens || !aligned4(cu_seqlens)) return cu_seqlens ? FALCON_ERR_UNSUPPORTED : FALCON_ERR_NULL;
    if (total_T > 0 && max_seqlen > 0 && (!q || !k || !v || !alpha || !eta || !o))
        return FALCON_ERR_NULL;
    const size_t need = falcon_chunk_fwd_varlen_workspace(N, H, max_seqlen, dk, dv, dt, var,
                                                          window, chunk);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FALCON_ERR_WORKSPACE;
    if ((max_seqlen == 0 || total_T == 0) && S_final == nullptr) return FALCON_OK;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    falcon::ChunkArgs a;
    a.phi = phi;
    a.kphi = a.qphi = a.kpphi = nullptr;
    if (phi && need > 0)  // room for N * max_seqlen >= total_T rows per head
        set_phi_buffers(a, workspace, (size_t)N * H * max_seqlen, N * H, window, dk, dt,
                        align256(falcon::chunk_workspace_bytes(N * H, max_seqlen, (int)dt, chunk,
                                                               window, norm_of(base),
                                                               is_delta(base), dk)));
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.eta = eta;
    a.S0 = S0;
    a.k_prev = k_prev;
    a.v_prev = v_prev;
    a.o = o;
    a.S_final = S_final;
    a.BH = N * H;
    a.T = total_T == 0 ? 0 : max_seqlen;
    a.cu = cu_seqlens;
    a.H = H;
    a.Ttot = total_T;
    const size_t rec = falcon_chunk_fwd_workspace(N, H, max_seqlen, dk, dv, dt, var, window, chunk);
    a.order_ws = (need > 0 && workspace) ? reinterpret_cast<int*>(static_cast<char*>(workspace) + rec)
                                         : nullptr;
    a.order = nullptr;
    a.toff = nullptr;
    a.jobs = nullptr;
    a.W = window;
    a.lag = lag;
    a.norm = norm_of(base);
    a.eps = eps;
    hipError_t e = falcon::launch_chunk(a, (int)dt, dk, chunk, is_delta(base), workspace, stream);
    return e == hipSuccess ? FALCON_OK : FALCON_ERR_HIP;
}

int falcon_decode_step(float* S, void* k_cache, const void* q, const void* k, const void* v,
                       const float* alpha, const float* eta, void* o, int N, int H, int dk,
                       int dv, falcon_dtype dt, falcon_variant var_arg, int window, float eps,
                       hipStream_t stream) {
    int var = 0, lag = 1, phi = 0;
    if (!split_variant(var_arg, &var, &lag, &phi) || !is_variant(var)) return FALCON_ERR_UNSUPPORTED;
    // the window rules have their own entry point, falcon_decode_step_window
    if (var == FALCON_F3 || var == FALCON_F3A) return FALCON_ERR_UNSUPPORTED;
    if (dt != FALCON_FP32 && dt != FALCON_BF16) return FALCON_ERR_UNSUPPORTED;
    if (N < 1 || H < 1 || dk < 1 || dv < 1 || window < 1) return FALCON_ERR_SHAPE;
    if ((long long)N * H > (1LL << 30)) return FALCON_ERR_SHAPE;
    if (window != 1) return FALCON_ERR_UNSUPPORTED;
    if (dk != dv || !falcon::decode_supported((int)dt, dk)) return FALCON_ERR_UNSUPPORTED;
    if (!(eps >= 0.0f)) return FALCON_ERR_SHAPE;
    if (!S || !k_cache || !q || !k || !v || !alpha || !eta || !o) return FALCON_ERR_NULL;
    if (!aligned16(S) || !aligned4(alpha) || !aligned4(eta)) return FALCON_ERR_UNSUPPORTED;
    falcon::DecodeArgs a;
    a.S = S;
    a.k_cache = k_cache;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.eta = eta;
    a.o = o;
    a.NH = N * H;
    a.norm = norm_of(var);
    a.delta = is_delta(var) ? 1 : 0;
    a.lag = lag;
    a.phi = phi;
    a.eps = eps;
    hipError_t e = falcon::launch_decode(a, (int)dt, dk, stream);
    return e == hipSuccess ? FALCON_OK : FALCON_ERR_HIP;
}

int falcon_decode_step_window(float* S, void* k_cache, void* v_cache, const void* q,
                              const void* k, const void* v, const float* alpha,
                              const float* eta, void* o, int N, int H, int dk, int dv,
                              falcon_dtype dt, falcon_variant var_arg, int window, float eps,
                              hipStream_t stream) {
    int var = 0, lag = 1, phi = 0;
    if (!split_variant(var_arg, &var, &lag, &phi)) return FALCON_ERR_UNSUPPORTED;
    if (var != FALCON_F3 && var != FALCON_F3A) return FALCON_ERR_UNSUPPORTED;
    if (dt != FALCON_FP32 && dt != FALCON_BF16) return FALCON_ERR_UNSUPPORTED;
    if (N < 1 || H < 1 || dk < 1 || dv < 1 || window < 1) return FALCON_ERR_SHAPE;
    if ((long long)N * H > (1LL << 30)) return FALCON_ERR_SHAPE;
    if (window > 8) return FALCON_ERR_UNSUPPORTED;
    if (dk != dv || !falcon::decode_supported((int)dt, dk)) return FALCON_ERR_UNSUPPORTED;
    if (!(eps >= 0.0f)) return FALCON_ERR_SHAPE;
    if (!S || !k_cache || !q || !k || !v || !alpha || !eta || !o) return FALCON_ERR_NULL;
    if (window > 1 && !v_cache) return FALCON_ERR_NULL;
    if (!aligned16(S) || !aligned4(alpha) || !aligned4(eta)) return FALCON_ERR_UNSUPPORTED;
    falcon::DecodeWinArgs a;
    a.S = S;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.eta = eta;
    a.o = o;
    a.NH = N * H;
    a.W = window;
    a.delta = var == FALCON_F3 ? 1 : 0;
    a.lag = lag;
    a.phi = phi;
    a.eps = eps;
    hipError_t e = falcon::launch_decode_window(a, (int)dt, dk, stream);
    return e == hipSuccess ? FALCON_OK : FALCON_ERR_HIP;
}

size_t falcon_chunk_bwd_workspace(int B, int H, int T, int dk, int dv, falcon_dtype dt,
                                  falcon_variant var, int window, int chunk) {
    const size_t fwd = fwd_ws(B, H, T, dk, dv, dt, var, window, chunk, true);
    if (fwd == 0) return 0;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    if (!falcon::chunk_bwd_supported((int)dt, dk, chunk, norm_of(base), window)) return 0;
    const int Wv = norm_of(base) == falcon::kNormWindow ? window : 1;
    const size_t ntiles = (size_t)((T + chunk / Wv - 1) / (chunk / Wv));
    const size_t ck = (size_t)B * H * ntiles * dk * dk * 2;
    const size_t cd = (size_t)B * H * ntiles * dk * chunk * 2;
    // windows above one: per-virtual-row gradients of targets and keys
    const size_t cw = Wv > 1 ? 2 * align256(cd) : 0;
    return align256(fwd) + 2 * align256(ck) + align256(cd) + cw;
}

}  // extern "C"

namespace {

// Checkpoint and gradient-row room of a backward call, after the forward's
// workspace `fwd`: the state at every tile start and the state gradient at
// every tile end (bf16, dk x dk), Delta (bf16, dk x chunk), and for a window
// above one the per-row target and key gradients (bf16, chunk x dk each).
size_t bwd_extra_bytes(int BH, int T, int dk, int chunk, int Wv) {
    const size_t ntiles = (size_t)((T + chunk / Wv - 1) / (chunk / Wv));
    const size_t ck = (size_t)BH * ntiles * dk * dk * 2;
    const size_t cd = (size_t)BH * ntiles * dk * chunk * 2;
    return 2 * align256(ck) + align256(cd) + (Wv > 1 ? 2 * align256(cd) : 0);
}

// The backward of falcon_chunk_fwd (cu == NULL: batched, BH = B * H rows of
// T steps) or of falcon_chunk_fwd_varlen (cu: packed, T = max_seqlen),
// arguments already checked.  `fwd` is the forward's workspace size, whose
// layout (records, feature-map copies, packed schedule) the forward re-run
// uses as it stands.  mode 0: re-run the forward with checkpoints, then the
// backward; mode 1: only the forward, with its outputs o / S_final and the
// checkpoints kept in the workspace; mode 2: only the backward, from a
// workspace that a mode-1 call on the same inputs filled.
enum BwdMode { kRecompute = 0, kSaveOnly = 1, kFromSaved = 2 };
int chunk_bwd_run(const void* q, const void* k, const void* v, const float* alpha,
                  const float* eta, const float* S0, const void* k_prev, const void* v_prev,
                  const void* d_o, const float* dS_final, void* dq, void* dk, void* dv,
                  float* dalpha, float* deta, float* dS0, void* dk_prev, void* dv_prev,
                  const int* cu, int BH, int H, int Ttot, int T, int dk_, int dt, int var,
                  int window, int chunk, float eps, void* workspace, size_t fwd, size_t rec,
                  size_t phi_rows, size_t order_off, hipStream_t stream, int mode = kRecompute,
                  void* o = nullptr, float* S_final = nullptr) {
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    const int Wv = norm_of(base) == falcon::kNormWindow ? window : 1;
    const int ntiles = (T + chunk / Wv - 1) / (chunk / Wv);
    char* ws = static_cast<char*>(workspace);
    const size_t ck = align256((size_t)BH * ntiles * dk_ * dk_ * 2);
    char* ck_s = ws + align256(fwd);
    char* ck_ds = ck_s + ck;
    char* ck_d = ck_ds + ck;
    const size_t cdb = align256((size_t)BH * ntiles * dk_ * chunk * 2);
    char* ck_r = Wv > 1 ? ck_d + cdb : nullptr;
    char* ck_x = Wv > 1 ? ck_d + 2 * cdb : nullptr;

    falcon::ChunkArgs a;
    a.phi = phi;
    a.kphi = a.qphi = a.kpphi = nullptr;
    if (phi && T > 0) set_phi_buffers(a, workspace, phi_rows, BH, window, dk_, dt, rec);
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.eta = eta;
    a.S0 = S0;
    a.k_prev = k_prev;
    a.v_prev = v_prev;
    a.o = o;
    a.S_final = S_final;
    a.BH = BH;
    a.T = T;
    a.cu = cu;
    a.H = H;
    a.Ttot = Ttot;
    a.order_ws = (cu && T > 0) ? reinterpret_cast<int*>(ws + order_off) : nullptr;
    a.order = nullptr;
    a.toff = nullptr;
    a.jobs = nullptr;
    a.W = window;
    a.lag = lag;
    a.norm = norm_of(base);
    a.eps = eps;
    a.ck_s = ck_s;
    a.ck_d = ck_d;
    if (mode == kSaveOnly && (o || S_final) && falcon::forward_kernel_differs(a, dt, dk_, chunk, is_delta(base))) {
        // the forward runs other kernels (the window rules' collapsed form,
        // the fused scalar-rule kernel): o and S_final from them (so they
        // equal falcon_chunk_fwd's bit for bit), then the checkpoints from a
        // run of the split kernels without outputs
        // With S_final aliasing S0 that first run must leave S0 alone: the
        // checkpoint run still reads it, and writes S_final itself (each of
        // its workgroups reads its slice of S0 before writing it).
        falcon::ChunkArgs f = a;
        f.ck_s = f.ck_d = nullptr;
        const bool alias = S_final && static_cast<const void*>(S_final) == static_cast<const void*>(S0);
        if (alias) f.S_final = nullptr;
        hipError_t e = falcon::launch_chunk(f, dt, dk_, chunk, is_delta(base), workspace, stream);
        if (e != hipSuccess) return FALCON_ERR_HIP;
        a.o = nullptr;
        if (!alias) a.S_final = nullptr;
    }
    if (mode != kFromSaved && (T > 0 || a.S_final)) {
        hipError_t e = falcon::launch_chunk(a, dt, dk_, chunk, is_delta(base), workspace, stream);
        if (e != hipSuccess) return FALCON_ERR_HIP;
    }
    if (mode == kSaveOnly) return FALCON_OK;

    falcon::BwdArgs b;
    b.q = phi ? a.qphi : q;
    b.k = phi ? a.kphi : k;
    b.k_prev = k_prev ? (phi ? a.kpphi : k_prev) : nullptr;
    b.q_raw = q;
    b.k_raw = k;
    b.kp_raw = k_prev;
    b.alpha = alpha;
    b.eta = eta;
    b.d_o = d_o;
    b.dS_final = dS_final;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.dalpha = dalpha;
    b.deta = deta;
    b.dS0 = dS0;
    b.dk_prev = dk_prev;
    b.rec = workspace;
    b.ck_s = ck_s;
    b.ck_d = ck_d;
    b.ck_ds = ck_ds;
    b.ck_r = ck_r;
    b.ck_x = ck_x;
    b.dv_prev = Wv > 1 ? dv_prev : nullptr;  // a window of one reads no value before the sequence
    b.BH = BH;
    b.T = T;
    b.ntiles = ntiles;
    b.W = window;
    b.lag = lag;
    b.phi = phi;
    b.norm = norm_of(base);
    b.eps = eps;
    b.cu = cu;
    b.H = H;
    b.Ttot = Ttot;
    hipError_t e = falcon::launch_chunk_bwd(b, dk_, chunk, is_delta(base), stream);
    return e == hipSuccess ? FALCON_OK : FALCON_ERR_HIP;
}

int check_bwd_outputs(int dt, int dk_, int chunk, int var, int window, bool any_steps, void* dq,
                      void* dk, void* dv, float* dalpha, float* deta, float* dS0, void* dk_prev,
                      void* dv_prev) {
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    if (!falcon::chunk_bwd_supported(dt, dk_, chunk, norm_of(base), window)) return FALCON_ERR_UNSUPPORTED;
    if (any_steps && (!dq || !dk || !dv || !dalpha || !deta)) return FALCON_ERR_NULL;
    if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dS0) ||
        !aligned16(dk_prev) || !aligned16(dv_prev) || !aligned4(dalpha) || !aligned4(deta))
        return FALCON_ERR_UNSUPPORTED;
    return FALCON_OK;
}

}  // namespace

extern "C" {

int falcon_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                     const float* eta, const float* S0, const void* k_prev, const void* v_prev,
                     const void* d_o, const float* dS_final, void* dq, void* dk, void* dv,
                     float* dalpha, float* deta, float* dS0, void* dk_prev, void* dv_prev,
                     int B, int H, int T, int dk_, int dv_, falcon_dtype dt, falcon_variant var,
                     int window, int chunk, float eps, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    int st = check_chunk(q, k, v, alpha, eta, S0, k_prev, v_prev, d_o, dS_final, B, H, T, dk_,
                         dv_, dt, var, window, chunk, eps);
    if (st != FALCON_OK) return st;
    st = check_bwd_outputs((int)dt, dk_, chunk, var, window, T > 0, dq, dk, dv, dalpha, deta, dS0,
                           dk_prev, dv_prev);
    if (st != FALCON_OK) return st;
    const size_t need = falcon_chunk_bwd_workspace(B, H, T, dk_, dv_, dt, var, window, chunk);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FALCON_ERR_WORKSPACE;
    if (T == 0 && dS0 == nullptr && dk_prev == nullptr && dv_prev == nullptr) return FALCON_OK;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    const int BH = B * H;
    const size_t fwd = fwd_ws(B, H, T, dk_, dv_, dt, var, window, chunk, true);
    const size_t rec = align256(falcon::chunk_workspace_bytes(BH, T, (int)dt, chunk, window,
                                                              norm_of(base), is_delta(base), dk_));
    return chunk_bwd_run(q, k, v, alpha, eta, S0, k_prev, v_prev, d_o, dS_final, dq, dk, dv, dalpha,
                         deta, dS0, dk_prev, dv_prev, nullptr, BH, H, T, T, dk_, (int)dt, var, window,
                         chunk, eps, workspace, fwd, rec, (size_t)BH * T, 0, stream);
}

size_t falcon_chunk_bwd_varlen_workspace(int N, int H, int max_seqlen, int dk, int dv,
                                         falcon_dtype dt, falcon_variant var, int window,
                                         int chunk) {
    const size_t fwd = fwd_varlen_ws(N, H, max_seqlen, dk, dv, dt, var, window, chunk, true);
    if (fwd == 0) return 0;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    if (!falcon::chunk_bwd_supported((int)dt, dk, chunk, norm_of(base), window)) return 0;
    const int Wv = norm_of(base) == falcon::kNormWindow ? window : 1;
    return align256(fwd) + bwd_extra_bytes(N * H, max_seqlen, dk, chunk, Wv);
}

int falcon_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* alpha,
                            const float* eta, const float* S0, const void* k_prev,
                            const void* v_prev, const void* d_o, const float* dS_final, void* dq,
                            void* dk, void* dv, float* dalpha, float* deta, float* dS0,
                            void* dk_prev, void* dv_prev, const int* cu_seqlens, int N, int H,
                            int total_T, int max_seqlen, int dk_, int dv_, falcon_dtype dt,
                            falcon_variant var, int window, int chunk, float eps, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    int st = check_chunk(q, k, v, alpha, eta, S0, k_prev, v_prev, d_o, dS_final, N, H, max_seqlen,
                         dk_, dv_, dt, var, window, chunk, eps);
    if (st != FALCON_OK) return st;
    if (total_T < 0 || (long long)H * total_T > (1LL << 40) / (dk_ > 0 ? dk_ : 1))
        return FALCON_ERR_SHAPE;
    if (!cu_seqlens || !aligned4(cu_seqlens)) return cu_seqlens ? FALCON_ERR_UNSUPPORTED : FALCON_ERR_NULL;
    const bool any = total_T > 0 && max_seqlen > 0;
    if (any && (!q || !k || !v || !alpha || !eta || !d_o)) return FALCON_ERR_NULL;
    st = check_bwd_outputs((int)dt, dk_, chunk, var, window, any, dq, dk, dv, dalpha, deta, dS0,
                           dk_prev, dv_prev);
    if (st != FALCON_OK) return st;
    const size_t need = falcon_chunk_bwd_varlen_workspace(N, H, max_seqlen, dk_, dv_, dt, var,
                                                          window, chunk);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FALCON_ERR_WORKSPACE;
    if (!any && dS0 == nullptr && dk_prev == nullptr && dv_prev == nullptr) return FALCON_OK;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    const int T = any ? max_seqlen : 0;
    const size_t fwd = fwd_varlen_ws(N, H, max_seqlen, dk_, dv_, dt, var, window, chunk, true);
    const size_t rec = align256(falcon::chunk_workspace_bytes(N * H, max_seqlen, (int)dt, chunk, window,
                                                              norm_of(base), is_delta(base), dk_));
    return chunk_bwd_run(q, k, v, alpha, eta, S0, k_prev, v_prev, d_o, dS_final, dq, dk, dv, dalpha,
                         deta, dS0, dk_prev, dv_prev, cu_seqlens, N * H, H, total_T, T, dk_, (int)dt,
                         var, window, chunk, eps, workspace, fwd, rec, (size_t)N * H * max_seqlen,
                         fwd_ws(N, H, max_seqlen, dk_, dv_, dt, var, window, chunk, true),
                         stream);
}

int falcon_chunk_fwd_save(const void* q, const void* k, const void* v, const float* alpha,
                          const float* eta, const float* S0, const void* k_prev, const void* v_prev,
                          void* o, float* S_final, int B, int H, int T, int dk_, int dv_,
                          falcon_dtype dt, falcon_variant var, int window, int chunk, float eps,
                          void* saved, size_t saved_bytes, hipStream_t stream) {
    int st = check_chunk(q, k, v, alpha, eta, S0, k_prev, v_prev, o, S_final, B, H, T, dk_, dv_,
                         dt, var, window, chunk, eps);
    if (st != FALCON_OK) return st;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    if (!falcon::chunk_bwd_supported((int)dt, dk_, chunk, norm_of(base), window))
        return FALCON_ERR_UNSUPPORTED;
    const size_t need = falcon_chunk_bwd_workspace(B, H, T, dk_, dv_, dt, var, window, chunk);
    if (need > 0 && (saved == nullptr || saved_bytes < need)) return FALCON_ERR_WORKSPACE;
    if (T == 0 && S_final == nullptr) return FALCON_OK;
    const int BH = B * H;
    const size_t fwd = fwd_ws(B, H, T, dk_, dv_, dt, var, window, chunk, true);
    const size_t rec = align256(falcon::chunk_workspace_bytes(BH, T, (int)dt, chunk, window,
                                                              norm_of(base), is_delta(base), dk_));
    return chunk_bwd_run(q, k, v, alpha, eta, S0, k_prev, v_prev, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, BH, H, T, T,
                         dk_, (int)dt, var, window, chunk, eps, saved, fwd, rec, (size_t)BH * T, 0,
                         stream, kSaveOnly, o, S_final);
}

int falcon_chunk_bwd_saved(const void* q, const void* k, const void* v, const float* alpha,
                           const float* eta, const float* S0, const void* k_prev,
                           const void* v_prev, const void* d_o, const float* dS_final, void* dq,
                           void* dk, void* dv, float* dalpha, float* deta, float* dS0,
                           void* dk_prev, void* dv_prev, int B, int H, int T, int dk_, int dv_,
                           falcon_dtype dt, falcon_variant var, int window, int chunk, float eps,
                           void* saved, size_t saved_bytes, hipStream_t stream) {
    int st = check_chunk(q, k, v, alpha, eta, S0, k_prev, v_prev, d_o, dS_final, B, H, T, dk_,
                         dv_, dt, var, window, chunk, eps);
    if (st != FALCON_OK) return st;
    st = check_bwd_outputs((int)dt, dk_, chunk, var, window, T > 0, dq, dk, dv, dalpha, deta, dS0,
                           dk_prev, dv_prev);
    if (st != FALCON_OK) return st;
    const size_t need = falcon_chunk_bwd_workspace(B, H, T, dk_, dv_, dt, var, window, chunk);
    if (need > 0 && (saved == nullptr || saved_bytes < need)) return FALCON_ERR_WORKSPACE;
    if (T == 0 && dS0 == nullptr && dk_prev == nullptr && dv_prev == nullptr) return FALCON_OK;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    const int BH = B * H;
    const size_t fwd = fwd_ws(B, H, T, dk_, dv_, dt, var, window, chunk, true);
    const size_t rec = align256(falcon::chunk_workspace_bytes(BH, T, (int)dt, chunk, window,
                                                              norm_of(base), is_delta(base), dk_));
    return chunk_bwd_run(q, k, v, alpha, eta, S0, k_prev, v_prev, d_o, dS_final, dq, dk, dv, dalpha,
                         deta, dS0, dk_prev, dv_prev, nullptr, BH, H, T, T, dk_, (int)dt, var, window,
                         chunk, eps, saved, fwd, rec, (size_t)BH * T, 0, stream, kFromSaved);
}

int falcon_chunk_fwd_varlen_save(const void* q, const void* k, const void* v, const float* alpha,
                                 const float* eta, const float* S0, const void* k_prev,
                                 const void* v_prev, void* o, float* S_final,
                                 const int* cu_seqlens, int N, int H, int total_T, int max_seqlen,
                                 int dk_, int dv_, falcon_dtype dt, falcon_variant var, int window,
                                 int chunk, float eps, void* saved, size_t saved_bytes,
                                 hipStream_t stream) {
    int st = check_chunk(q, k, v, alpha, eta, S0, k_prev, v_prev, o, S_final, N, H, max_seqlen,
                         dk_, dv_, dt, var, window, chunk, eps);
    if (st != FALCON_OK) return st;
    if (total_T < 0 || (long long)H * total_T > (1LL << 40) / (dk_ > 0 ? dk_ : 1))
        return FALCON_ERR_SHAPE;
    if (!cu_seqlens || !aligned4(cu_seqlens)) return cu_seqlens ? FALCON_ERR_UNSUPPORTED : FALCON_ERR_NULL;
    const bool any = total_T > 0 && max_seqlen > 0;
    if (any && (!q || !k || !v || !alpha || !eta || !o)) return FALCON_ERR_NULL;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    if (!falcon::chunk_bwd_supported((int)dt, dk_, chunk, norm_of(base), window))
        return FALCON_ERR_UNSUPPORTED;
    const size_t need = falcon_chunk_bwd_varlen_workspace(N, H, max_seqlen, dk_, dv_, dt, var,
                                                          window, chunk);
    if (need > 0 && (saved == nullptr || saved_bytes < need)) return FALCON_ERR_WORKSPACE;
    if (!any && S_final == nullptr) return FALCON_OK;
    const int T = any ? max_seqlen : 0;
    const size_t fwd = fwd_varlen_ws(N, H, max_seqlen, dk_, dv_, dt, var, window, chunk, true);
    const size_t rec = align256(falcon::chunk_workspace_bytes(N * H, max_seqlen, (int)dt, chunk, window,
                                                              norm_of(base), is_delta(base), dk_));
    return chunk_bwd_run(q, k, v, alpha, eta, S0, k_prev, v_prev, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, cu_seqlens, N * H, H,
                         total_T, T, dk_, (int)dt, var, window, chunk, eps, saved, fwd, rec,
                         (size_t)N * H * max_seqlen,
                         fwd_ws(N, H, max_seqlen, dk_, dv_, dt, var, window, chunk, true),
                         stream, kSaveOnly, o, S_final);
}

int falcon_chunk_bwd_varlen_saved(const void* q, const void* k, const void* v, const float* alpha,
                                  const float* eta, const float* S0, const void* k_prev,
                                  const void* v_prev, const void* d_o, const float* dS_final,
                                  void* dq, void* dk, void* dv, float* dalpha, float* deta,
                                  float* dS0, void* dk_prev, void* dv_prev, const int* cu_seqlens,
                                  int N, int H, int total_T, int max_seqlen, int dk_, int dv_,
                                  falcon_dtype dt, falcon_variant var, int window, int chunk,
                                  float eps, void* saved, size_t saved_bytes, hipStream_t stream) {
    int st = check_chunk(q, k, v, alpha, eta, S0, k_prev, v_prev, d_o, dS_final, N, H, max_seqlen,
                         dk_, dv_, dt, var, window, chunk, eps);
    if (st != FALCON_OK) return st;
    if (total_T < 0 || (long long)H * total_T > (1LL << 40) / (dk_ > 0 ? dk_ : 1))
        return FALCON_ERR_SHAPE;
    if (!cu_seqlens || !aligned4(cu_seqlens)) return cu_seqlens ? FALCON_ERR_UNSUPPORTED : FALCON_ERR_NULL;
    const bool any = total_T > 0 && max_seqlen > 0;
    if (any && (!q || !k || !v || !alpha || !eta || !d_o)) return FALCON_ERR_NULL;
    st = check_bwd_outputs((int)dt, dk_, chunk, var, window, any, dq, dk, dv, dalpha, deta, dS0,
                           dk_prev, dv_prev);
    if (st != FALCON_OK) return st;
    const size_t need = falcon_chunk_bwd_varlen_workspace(N, H, max_seqlen, dk_, dv_, dt, var,
                                                          window, chunk);
    if (need > 0 && (saved == nullptr || saved_bytes < need)) return FALCON_ERR_WORKSPACE;
    if (!any && dS0 == nullptr && dk_prev == nullptr && dv_prev == nullptr) return FALCON_OK;
    int base = 0, lag = 1, phi = 0;
    split_variant(var, &base, &lag, &phi);
    const int T = any ? max_seqlen : 0;
    const size_t fwd = fwd_varlen_ws(N, H, max_seqlen, dk_, dv_, dt, var, window, chunk, true);
    const size_t rec = align256(falcon::chunk_workspace_bytes(N * H, max_seqlen, (int)dt, chunk, window,
                                                              norm_of(base), is_delta(base), dk_));
    return chunk_bwd_run(q, k, v, alpha, eta, S0, k_prev, v_prev, d_o, dS_final, dq, dk, dv, dalpha,
                         deta, dS0, dk_prev, dv_prev, cu_seqlens, N * H, H, total_T, T, dk_, (int)dt,
                         var, window, chunk, eps, saved, fwd, rec, (size_t)N * H * max_seqlen,
                         fwd_ws(N, H, max_seqlen, dk_, dv_, dt, var, window, chunk, true),
                         stream, kFromSaved);
}

int falcon_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* alpha,
                             const float* eta, const float* S0, const void* k_prev,
                             const void* v_prev, void* o, float* S_final, int B, int H, int T,
                             int dk, int dv, falcon_dtype dt, falcon_variant var, int window,
                             int chunk, float eps, hipStream_t stream) {
    int st = check_chunk(q, k, v, alpha, eta, S0, k_prev, v_prev, o, S_final, B, H, T, dk, dv,
                         dt, var, window, chunk, eps);
    if (st != FALCON_OK) return st;
    const size_t need = falcon_chunk_fwd_workspace(B, H, T, dk, dv, dt, var, window, chunk);
    if (need > FALCON_NOALLOC_SCRATCH_BYTES) return FALCON_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        st = device_scratch(&ws);
        if (st != FALCON_OK) return st;
    }
    return falcon_chunk_fwd(q, k, v, alpha, eta, S0, k_prev, v_prev, o, S_final, B, H, T, dk, dv,
                            dt, var, window, chunk, eps, ws, need, stream);
}

const char* falcon_status_string(int status) {
    switch (status) {
        case FALCON_OK: return "ok";
        case FALCON_ERR_NULL: return "a required pointer is NULL";
        case FALCON_ERR_SHAPE: return "a size is out of range or inconsistent";
        case FALCON_ERR_UNSUPPORTED: return "arguments outside the supported set";
        case FALCON_ERR_WORKSPACE: return "workspace missing or too small";
        case FALCON_ERR_HIP: return "HIP reported an error at launch";
        case FALCON_ERR_SCRATCH:
            return "the call needs more scratch than the built-in buffer of "
                   "FALCON_NOALLOC_SCRATCH_BYTES (128 MiB) holds";
        default: return "unknown status";
    }
}

}  // extern "C"
