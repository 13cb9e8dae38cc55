// falcon_rows.h -- device helpers shared by the chunk-forward kernels: where
// a (batch*head) sequence's rows lie in the [rows, d] planes (batched and
// packed layouts), the order of the state pass's workgroups, the job list of
// the intra-chunk kernels, and raw buffer loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "falcon_device.h"
#include "falcon_internal.h"

namespace falcon {

// Rows of sequence bh in the [rows, d] planes: [row0, row0 + T).  Batched
// calls: row0 = bh * T.  Packed calls: the bounds come from cu, clamped to the
// plane and to the longest sequence allowed, so offsets outside the contract
// cannot move any access out of the buffers.
struct SeqRows {
    size_t row0;
    int T;
};
__device__ __forceinline__ SeqRows rows_of(const ChunkArgs& a, int h, int c0, int c1) {
    const int s0 = min(max(c0, 0), a.Ttot);
    const int s1 = min(min(max(c1, s0), a.Ttot), s0 + a.T);
    return {(size_t)h * a.Ttot + s0, s1 - s0};
}
__device__ __forceinline__ SeqRows seq_rows(const ChunkArgs& a, int bh) {
    if (!a.cu) return {(size_t)bh * a.T, a.T};
    const int n = bh / a.H;
    return rows_of(a, bh - n * a.H, a.cu[n], a.cu[n + 1]);
}

// First row of sequence bh in the feature-mapped copies of the keys and
// queries that the intra-chunk kernel writes to the workspace: each
// (sequence, head) has its own T rows (packed calls: max_seqlen rows), so the
// copies fit the workspace whatever the packed plane's length is.  Batched
// calls: the same row as in the inputs.
__device__ __forceinline__ size_t mapped_row0(const ChunkArgs& a, int bh) {
    return (size_t)bh * a.T;
}

// The (batch*head) row of state-pass workgroup rank r: the natural order, or
// for packed calls the sequences longest first (`order`), so the longest
// sequences are dispatched first and none is left to run alone at the end.
__device__ __forceinline__ int pass_bh(const ChunkArgs& a, int r) {
    if (!a.order) return r;
    const int i = r / a.H;
    return a.order[i] * a.H + (r - i * a.H);
}

// The (batch*head row, tile) of intra-chunk job j.  Batched calls: row-major
// over (row, tile).  Packed calls: only existing tiles, j = h * G + g with G
// the tile count of all sequences and g a tile index in sequence order (so
// consecutive jobs walk one head's plane in address order), the sequence of
// g found in toff by binary search.
struct Job {
    int bh, tile;
    SeqRows sr;
};
__device__ __forceinline__ Job job_of(const ChunkArgs& a, int j, int ntiles) {
    if (!a.jobs) {
        const int bh = j / ntiles;
        return {bh, j - bh * ntiles, seq_rows(a, bh)};
    }
    const int4 e = reinterpret_cast<const int4*>(a.jobs)[j];
    const int h = e.x - (e.x / a.H) * a.H;
    return {e.x, e.y, {(size_t)h * a.Ttot + e.z, e.w}};
}


typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFF0 ? 0x7FFFFFF0 : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRawBufferFlags);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ s16x4 buf_load8(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(s16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
// 16 (8) bytes per lane to a buffer; an offset past the buffer's size (kOob)
// writes nothing, so a lane's store is masked without a branch.
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, s16x4 v) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

}  // namespace falcon
