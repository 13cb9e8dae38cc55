// falcon_device.h -- device-side building blocks for the gfx950 kernels:
// element policies (bf16 / fp32), MFMA fragment conventions and small
// wavefront utilities.
//
// Fragment conventions (wave64, lane l, group g = l / 16, lr = l % 16), for a
// 16 x 16 x 16 step of a matrix product C += A * B:
//   A fragment  lane holds A[m = lr][k = 4g + r],     r = 0..3
//   B fragment  lane holds B[k = 4g + r][n = lr],     r = 0..3
//   accumulator lane holds C[m = 4g + r][n = lr],     r = 0..3
// These are the operand layouts of v_mfma_f32_16x16x16_bf16 and, applied
// instruction by instruction, of four v_mfma_f32_16x16x4_f32.  Consequence
// used throughout: an accumulator tile is, as it stands, the B fragment of a
// product that contracts over the tile's row index.
//
// A K = 32 step concatenates two K = 16 fragments into the eight operand
// slots of v_mfma_f32_16x16x32_bf16.  The instruction sums over all 32 slot
// pairs and maps (lane group, slot) to the same K position for A and for B,
// so any consistent assignment of logical k to slots gives the same sum; the
// one used here is "slots 0..3 = first 16-block, slots 4..7 = second".
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace falcon {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16-byte staging vector (a native vector type: copies are loads and stores,
// never memcpy, so arrays of it stay in registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// One entry of the per-column rule's write vector, u = eta x / (|x| l1 + eps)
// with l1 = ||x||_1 of the entry's row, through the hardware reciprocal
// (about 1 ulp; every caller rounds u to bf16 next).  The bf16 kernels that
// form u (intra-chunk products, state update, backward) all use this one
// expression, so they see the same bits.
__device__ __forceinline__ float col_write(float x, float l1, float eta, float eps) {
    const float den = __builtin_fmaf(fabsf(x), l1, eps);
    return den > 0.f ? (eta * x) * __builtin_amdgcn_rcpf(den) : 0.f;
}
// Eight bf16 entries of one row (16 bytes) to their write-vector entries.
__device__ __forceinline__ u32x4 col_write8(u32x4 v, float l1, float eta, float eps) {
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
    u32x4 o;
    uint16_t* out = reinterpret_cast<uint16_t*>(&o);
#pragma unroll
    for (int u = 0; u < 8; ++u) out[u] = f2bf(col_write(bf2f(e[u]), l1, eta, eps));
    return o;
}

struct EBf16 {
    using T = uint16_t;   // storage element in HBM and LDS
    using Frag = s16x4;   // four operand values
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float to_f(T x) { return bf2f(x); }
    static __device__ __forceinline__ T from_f(float x) { return f2bf(x); }
    static __device__ __forceinline__ Frag pack(f32x4 v) {
        Frag f;
        f.x = (short)f2bf(v.x);
        f.y = (short)f2bf(v.y);
        f.z = (short)f2bf(v.z);
        f.w = (short)f2bf(v.w);
        return f;
    }
    // Four consecutive elements at p (8-byte aligned).
    static __device__ __forceinline__ Frag load(const T* p) {
        return *reinterpret_cast<const Frag*>(p);
    }
    // Four elements spaced `stride` apart (a column of a row-major tile).
    static __device__ __forceinline__ Frag gather4(const T* p, int stride) {
        Frag f;
        f.x = (short)p[0];
        f.y = (short)p[stride];
        f.z = (short)p[2 * stride];
        f.w = (short)p[3 * stride];
        return f;
    }
    // Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
    // lanes, lane i receives in slot s the element (i % 4) of the 8 bytes that
    // lane 4 s + i / 4 of the group addressed.  So if lane i of a group
    // addresses  row0 + i / 4,  column col0 + 4 (i % 4)  of a row-major tile,
    // lane i receives rows row0 .. row0 + 3 of column col0 + i: a column
    // fragment (B-fragment order of the tile, A-fragment order of its
    // transpose) in one instruction.
    static __device__ __forceinline__ Frag load_tr(const T* p) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p));
    }
    // K = 16 on the K = 32 instruction with a zero upper half.  Every bf16
    // product of the library then has one MFMA shape: a 16x16x16 bf16 MFMA
    // that takes its accumulator straight from a 16x16x32 one issued just
    // before it (no wait states in between, which the compiler allows for an
    // exactly overlapping accumulator) was seen to return wrong rows on gfx950.
    static __device__ __forceinline__ f32x4 mma16(Frag a, Frag b, f32x4 c) {
        const Frag z = {0, 0, 0, 0};
        return mma32(a, z, b, z, c);
    }
    // The 16x16x16 instruction itself (half the K = 32 issue cost), for
    // accumulation chains built from it alone; the assembly of every kernel is
    // checked for a 16x16x32 result feeding it as accumulator within a few
    // wait states.
    static __device__ __forceinline__ f32x4 mma16n(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma32(Frag a0, Frag a1, Frag b0, Frag b1, f32x4 c) {
        s16x8 a = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        s16x8 b = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                       0);
    }
    // Row products A B^T with both operands read along their rows: a lane
    // takes eight contiguous elements of the 32-wide contraction slice (one
    // 16-byte LDS read; at a 272-byte row stride the 8-byte pairs of the
    // split layout above hit each bank twice).  The contraction order only has
    // to agree between the two operands.
    static __device__ __forceinline__ s16x8 load8(const T* p) {
        return *reinterpret_cast<const s16x8*>(p);
    }
    static __device__ __forceinline__ f32x4 mma32r(s16x8 a, s16x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                       0);
    }
};

struct EFp32 {
    using T = float;
    using Frag = f32x4;
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ float to_f(T x) { return x; }
    static __device__ __forceinline__ T from_f(float x) { return x; }
    static __device__ __forceinline__ Frag pack(f32x4 v) { return v; }
    static __device__ __forceinline__ Frag load(const T* p) {
        return *reinterpret_cast<const Frag*>(p);
    }
    static __device__ __forceinline__ Frag gather4(const T* p, int stride) {
        return Frag{p[0], p[stride], p[2 * stride], p[3 * stride]};
    }
    static __device__ __forceinline__ f32x4 mma16(Frag a, Frag b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ f32x4 mma32(Frag a0, Frag a1, Frag b0, Frag b1, f32x4 c) {
        return mma16(a1, b1, mma16(a0, b0, c));
    }
};

// Unpadded LDS tiles of bf16 rows of N elements (N = 64 or 128): the 16-byte
// chunk j of row r sits at chunk j ^ swz_row<N>(r).  A wave's row reads (16
// rows, one 8- or 16-byte piece each) and its transposing column reads (four
// rows, two adjacent chunks per 16 lanes) then fall on distinct banks; for
// N = 64 two rows share a 256-byte bank line and the row's parity picks the
// half.
template <int N>
__device__ __forceinline__ int swz_row(int r) {
    static_assert(N == 64 || N == 128, "row length");
    return N == 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}
// element offset of (row r, column c) in such a tile
template <int N>
__device__ __forceinline__ int swz_off(int r, int c) {
    return r * N + ((((c >> 3) ^ swz_row<N>(r)) << 3) | (c & 7));
}

// Workgroup barrier that orders LDS only: global loads and stores in flight
// are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kRawBufferFlags = 0x00020000;  // descriptor word 3 of a raw gfx9 buffer
constexpr uint32_t kOob = 0x80000000u;       // an offset beyond every buffer size used here

// Descriptor words of a raw buffer (base, stride 0, size in bytes, flags),
// wave-uniform, for the direct-to-LDS fill below.
__device__ __forceinline__ u32x4 make_desc(const void* base, int64_t bytes) {
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7FFFFFF0 ? 0x7FFFFFF0u : (uint32_t)bytes);
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    u32x4 d;
    d[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
    d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xFFFFu);
    d[2] = __builtin_amdgcn_readfirstlane(n);
    d[3] = (uint32_t)kRawBufferFlags;
    return d;
}
// 16 bytes per lane from a buffer straight into LDS: lane l writes
// lds + 16 l (lds is wave-uniform); lanes whose exec bit is off write nothing,
// out-of-range offsets write zeros.  Completion is counted by vmcnt and the
// caller waits for it (wait_vm_all) before the barrier that publishes the
// tile.  The instruction is issued from inline assembly on purpose: the
// compiler cannot tell which LDS bytes such a fill writes, and for the
// builtin form it waits for every fill in flight before the wave's next LDS
// read, which would serialize each fill's latency with the arithmetic it is
// meant to overlap.  The asm has no outputs; the fills' targets are read only
// after the explicit wait and a barrier.
// `lds` is the wave's LDS byte address (it goes to M0).
__device__ __forceinline__ void buf_load16_lds(u32x4 d, uint32_t lds, uint32_t off) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(d), "{m0}"(m0)
                 : "memory");
}
// s_waitcnt vmcnt(0), leaving the other counters alone
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(2): all but the two most recent vector memory operations
__device__ __forceinline__ void wait_vm_2() { __builtin_amdgcn_s_waitcnt(0x0F72); }
// 4 bytes per lane from a buffer into LDS at lds + 4 l (as buf_load16_lds).
__device__ __forceinline__ void buf_load4_lds(u32x4 d, uint32_t lds, uint32_t off) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(d), "{m0}"(m0)
                 : "memory");
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1, so that
// register arrays are only ever indexed by constants.
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>());
        static_for_impl<I + 1, N>(f);
    }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl<0, N>(f);
}
// f(std::integral_constant<int, w>()) for a wave-uniform w in 0..3: one
// specialized copy of f per value, so that conditions on w are resolved at
// compile time and do not split the copy's instruction stream into branches.
template <class F>
__device__ __forceinline__ void with_const4(int w, F&& f) {
    switch (__builtin_amdgcn_readfirstlane(w)) {
        case 0: f(std::integral_constant<int, 0>()); break;
        case 1: f(std::integral_constant<int, 1>()); break;
        case 2: f(std::integral_constant<int, 2>()); break;
        default: f(std::integral_constant<int, 3>()); break;
    }
}

// Sum over aligned groups of `width` consecutive lanes, width in {2,4,8,16},
// with DPP lane permutations (VALU only, no LDS round trip): quad_perm swaps
// within quads, then the half-row and row mirrors fold 8 and 16 lanes.
template <int width>
__device__ __forceinline__ float group_sum_dpp(float x) {
    static_assert(width == 2 || width == 4 || width == 8 || width == 16, "dpp group width");
    auto dpp = [](float v, auto ctrl) {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                               0xF, 0xF, false));
    };
    x += dpp(x, std::integral_constant<int, 0xB1>());      // quad_perm [1,0,3,2]
    if constexpr (width >= 4) x += dpp(x, std::integral_constant<int, 0x4E>());   // [2,3,0,1]
    if constexpr (width >= 8) x += dpp(x, std::integral_constant<int, 0x141>());  // row_half_mirror
    if constexpr (width >= 16) x += dpp(x, std::integral_constant<int, 0x140>()); // row_mirror
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP (no LDS round
// trips): shifts by 1, 2, 4 and 8 within each 16-lane row (lanes shifted in
// from outside the row add zero), then the last lane of row 0 is added to
// row 1 and that of row 2 to row 3, then lane 31 (rows 0-1 in total) to
// rows 2 and 3.  Rows left out by the row mask add zero.
__device__ __forceinline__ float wave_scan_dpp(float x) {
    auto dpp = [](float v, auto ctrl, auto rows) {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                               decltype(rows)::value, 0xF, false));
    };
    using all = std::integral_constant<int, 0xF>;
    x += dpp(x, std::integral_constant<int, 0x111>(), all());  // row_shr:1
    x += dpp(x, std::integral_constant<int, 0x112>(), all());  // row_shr:2
    x += dpp(x, std::integral_constant<int, 0x114>(), all());  // row_shr:4
    x += dpp(x, std::integral_constant<int, 0x118>(), all());  // row_shr:8
    x += dpp(x, std::integral_constant<int, 0x142>(), std::integral_constant<int, 0xA>());  // row_bcast:15
    x += dpp(x, std::integral_constant<int, 0x143>(), std::integral_constant<int, 0xC>());  // row_bcast:31
    return x;
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < width; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Feature maps on keys and queries (0 identity, 1 L2 normalization x/||x||
// with 0 for x = 0, 2 SiLU x / (1 + e^-x)) applied to one 16-byte piece of a
// row held by G consecutive lanes, one piece each (the row norm is a sum over
// the lane group).  Every lane of the wave must call it.  The identity
// returns the piece unchanged (no rounding).
template <class E, int G>
__device__ __forceinline__ u32x4 phi_piece(int phi, u32x4 v) {
    using T = typename E::T;
    constexpr int EPP = 16 / E::kBytes;
    if (phi == 0) return v;
    const T* e = reinterpret_cast<const T*>(&v);
    float f[EPP];
#pragma unroll
    for (int u = 0; u < EPP; ++u) f[u] = E::to_f(e[u]);
    if (phi == 1) {
        float n2 = 0.f;
#pragma unroll
        for (int u = 0; u < EPP; ++u) n2 += f[u] * f[u];
        if constexpr (G <= 16) n2 = group_sum_dpp<G>(n2);
        else n2 = group_sum<G>(n2);
        const float sc = n2 > 0.f ? rsqrtf(n2) : 0.f;
#pragma unroll
        for (int u = 0; u < EPP; ++u) f[u] *= sc;
    } else {
#pragma unroll
        for (int u = 0; u < EPP; ++u) f[u] = f[u] / (1.f + __expf(-f[u]));
    }
    u32x4 out;
    T* o = reinterpret_cast<T*>(&out);
#pragma unroll
    for (int u = 0; u < EPP; ++u) o[u] = E::from_f(f[u]);
    return out;
}

}  // namespace falcon
