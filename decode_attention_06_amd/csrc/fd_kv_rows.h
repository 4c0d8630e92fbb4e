// Row addressing of a KV cache for the split-KV kernels: dense
// [B, Hkv, Lmax, D] or paged (pages of a power-of-two number of rows >= 16,
// a per-sequence table of page ids).  Internal.
//
// Pieces start at multiples of 16 rows and the kernels' tiles are 16-row
// aligned, so an aligned group of 16 rows never spans two pages: one page
// lookup (a wave-uniform, scalar load) serves every row of a group.  A tile
// whose rows run past the piece's last valid row clamps them to that row; the
// group of a clamped row is the group of the last row, so the lookup of group
// start min(tile start + 16 h, last) & ~15 covers every row a lane reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fd {

// The two halves of kv_row_offset<true>: the table entry of row t (a
// scalar load; issued early, its latency hides behind other work) and the
// element offset that entry gives, computed where it is used.
__device__ __forceinline__ int kv_page_id(const PartialParams& p, int b, int t) {
    return p.block_table[(int64_t)b * p.bt_stride + (t >> p.page_shift)];
}

template <int D>
__device__ __forceinline__ int64_t kv_page_offset(const PartialParams& p, int page, int kvh, int t) {
    page = min(max(page, 0), p.n_pages - 1);
    const int in_page = t & ((1 << p.page_shift) - 1);
    return (int64_t)page * p.page_stride + (int64_t)kvh * p.kv_stride_h + (int64_t)in_page * D;
}

// Element offset of row t (any row of its 16-row group) of (b, kvh).
template <bool PAGED, int D>
__device__ __forceinline__ int64_t kv_row_offset(const PartialParams& p, int b, int kvh, int t) {
    if constexpr (PAGED) {
        return kv_page_offset<D>(p, kv_page_id(p, b, t), kvh, t);
    } else {
        return (int64_t)b * p.kv_stride_b + (int64_t)kvh * p.kv_stride_h + (int64_t)t * p.kv_stride_t;
    }
}

// First row of the 16-row group that holds row min(t, last).
__device__ __forceinline__ int kv_group_start(int t, int last) { return min(t, last) & ~15; }

}  // namespace fd
