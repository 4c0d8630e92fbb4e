// Internal interface between the host layer (fd_api.cpp) and the kernels
// (fd_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "fd.h"

namespace fd {

// Records the thread-local text fd_last_error_message() returns and passes
// the status through (printf-style format).
fd_status set_error(fd_status s, const char* fmt, ...);

// Device-side validation (FD_VALIDATE=1 or fd_set_validation(1)): count the
// entries of a device array outside their range, synchronise, and return
// FD_ERR_INVALID_ARG naming the first; FD_OK at once when validation is off.
bool validation_on();
// lens[0 .. n) must lie in [lo, hi].
fd_status validate_lens(const int32_t* lens, int64_t n, int64_t lo, int64_t hi, const char* what, hipStream_t s);
// Entries of table [B, cols] that cover rows below lens[b] (or `rows`) must
// lie in [0, n_pages).
fd_status validate_table(const int32_t* table, const int32_t* lens, int32_t B, int32_t cols, int32_t page_size,
                         int64_t rows, int32_t n_pages, hipStream_t s);

// Most pieces one combine can merge per output row (LDS holds their weights).
#define FD_MAX_PARTS 4096

// One launch of the split-KV partial kernel.  A work unit is
// (sequence b, KV head, block of query rows, piece); every unit streams its
// piece of the KV rows once and keeps a running max / running sum per query
// row (the online softmax).
struct PartialParams {
    const void* q;          // [B, Hq, D]: element (b, h, d) at b*q_stride_b + h*q_stride_h + d
    const void* k;          // dense: element (b, kvh, t, d) at b*kv_stride_b + kvh*kv_stride_h + t*kv_stride_t + d
    const void* v;          // paged: see block_table
    const int32_t* lens;    // [B] valid rows per sequence, or nullptr = Lmax
    void* out;              // direct mode: final output [B, Hq, D] at b*out_stride_b + h*out_stride_h + d
    float* lse_out;         // direct mode: [B, Hq] natural-log lse, or nullptr
    float* o_part;          // partial mode: [B*Hq, part_stride, D]
    float* lse_part;        // partial mode: [B*Hq, part_stride]
    int64_t Lmax;           // rows available per (b, kv head)
    int64_t kv_stride_b;    // elements; 0 makes every sequence read the same KV
    int64_t kv_stride_h;    // elements
    int64_t kv_stride_t;    // elements between consecutive rows (dense caches; pages hold rows D apart)
    int64_t q_stride_b, q_stride_h;       // elements
    int64_t out_stride_b, out_stride_h;   // elements
    int32_t B, Hq, Hkv;
    int32_t n_splits;       // pieces per sequence in this launch
    int32_t row_blocks;     // query-row blocks per KV head (G / rows per block)
    int32_t part_stride;    // pieces per output row in o_part / lse_part
    int32_t part_offset;    // first piece slot written by this launch
    float scale_log2;       // softmax scale * log2(e)
    int32_t out_bf16;       // direct mode output dtype
    int32_t direct;         // 1: n_splits == 1, write the final output
    // Piece layout: 0 gives piece i the contiguous rows [i*c, (i+1)*c); 1
    // deals the kernel's workgroup steps (MFMA_TILE_ROWS or valu_tile_rows
    // rows) out round-robin, piece i taking steps i, i + n_splits, ...
    int32_t strided;
    // Paged cache (block_table != nullptr): row t of (b, kvh) is row
    // t & (page_size - 1) of page block_table[b * bt_stride + (t >> page_shift)],
    // at element page * page_stride + kvh * kv_stride_h + (t & (page_size - 1)) * D.
    // Page ids outside [0, n_pages) are clamped into it.
    const int32_t* block_table;
    int64_t bt_stride;      // table entries per sequence
    int64_t page_stride;    // elements per page (Hkv * page_size * D)
    int32_t page_shift;     // log2(page_size), page_size >= 16
    int32_t n_pages;
    // E4M3 cache: per-KV-head scales [Hkv] (cache value = code value *
    // scale), or nullptr = 1.  The query stays bf16.
    const float* k_scale;
    const float* v_scale;
};

// Context part of a bifurcated call on the matrix cores (bf16, head_dim
// 128): the S * G query rows of each KV head against that head's context,
// cut into n_pieces pieces; writes pieces [part_offset, part_offset +
// n_pieces) of every row.
struct BifContextParams {
    const void* q;          // [S, Hq, D] at s*q_stride_b + h*q_stride_h + d
    const void* k_ctx;      // [Hkv, Lc, D] at kvh*ctx_stride_h + t*ctx_stride_t + d
    const void* v_ctx;
    int64_t q_stride_b, q_stride_h;
    int64_t ctx_stride_h, ctx_stride_t;
    float* o_part;          // [S*Hq, part_stride, D]
    float* lse_part;        // [S*Hq, part_stride]
    int32_t S, Hq, Hkv, Lc;
    int32_t n_pieces;       // context pieces
    int32_t row_tiles;      // bif_context_row_tiles(S, G)
    int32_t part_stride, part_offset;
    float scale_log2;
};

// Causal prefill on the matrix cores (bf16, head_dim 128): work unit =
// (sequence b, KV head, tile of pos_per_tile positions); its rows are the
// pos_per_tile * G (position, head-in-group) pairs.  Position p of sequence
// b attends to cache rows [0, p]; positions at or beyond lens[b] are not
// written.
struct PrefillParams {
    const void* q;          // [B, Hq, Lmax, D]
    const void* k;          // [B, Hkv, Lmax, D]
    const void* v;
    const int32_t* lens;    // [B] or nullptr = Lmax
    void* out;              // [B, Hq, Lmax, D]
    float* lse_out;         // [B, Hq, Lmax] natural-log lse, or nullptr
    int64_t Lmax;
    int32_t B, Hq, Hkv;
    int32_t pos_per_tile;   // 128 / G
    int32_t n_ptiles;       // ceil(Lmax / pos_per_tile)
    float scale_log2;
    int32_t out_bf16;
};

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Tiles of 128 query rows (four waves of 32) over the S * G rows of a KV head.
int bif_context_row_tiles(int S, int G);

// Whole bifurcated partial stage in one launch: context units (c) and the
// decode part's split-KV units (d: 16-row matrix-core blocks, i.e.
// d.row_blocks = ceil(G / 16)) run side by side.
hipError_t launch_bifurcated(const BifContextParams& c, const PartialParams& d, hipStream_t stream);

// Query rows handled by one work unit of the vector-ALU partial kernel for a
// GQA group of G query heads: the largest of 8, 4, 2, 1 that divides G (at
// most 4 for an E4M3 cache, whose 16-element lane slices double the
// per-row registers).
inline int valu_rows_per_block(int G, bool fp8_cache = false) {
    const int r = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
    return (fp8_cache && r > 4) ? 4 : r;
}

// Cache rows per workgroup step of the vector-ALU partial kernel, for
// elements of elem_bytes, head_dim D and GB query rows per unit: 4 waves,
// each loading 64 / (D / (16 / elem_bytes)) rows per 16-byte-per-lane load
// with U loads in flight (8 for GB <= 2, else 4; halved for 1-byte
// elements).  The interleaved piece layout deals these steps out.
constexpr int valu_tile_rows(int elem_bytes, int D, int GB) {
    return 4 * (64 / (D / (16 / elem_bytes))) * (((GB <= 2) ? 8 : 4) / (elem_bytes == 1 ? 2 : 1));
}

// Cache rows per workgroup step of the matrix-core partial kernel: 4 waves
// of 32-row tiles.
constexpr int MFMA_TILE_ROWS = 128;

// Rows per work unit of the matrix-core kernel (16 or 32) for a group of G.
int mfma_rows_per_block(int G);

// Matrix-core partial kernel: bf16, head_dim 128, any G (row_blocks =
// ceil(G / mfma_rows_per_block(G))).
hipError_t launch_partial_mfma(const PartialParams& p, bool fp8_cache, hipStream_t stream);

// dtype: 0 fp32, 1 bf16, 2 E4M3 cache with a bf16 query.
hipError_t launch_partial_valu(const PartialParams& p, int dtype, int head_dim, int rows_per_block,
                               hipStream_t stream);

// Streams `bytes` (multiple of 16) with 16-byte loads and folds them into
// one word written to sink[0] only if it equals a sentinel.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// Where the combine writes output row r (= b * hq + h of a [B, hq, D]
// output): element (r / hq) * stride_b + (r % hq) * stride_h + d.  A dense
// [rows, D] output is {1, D, 0}.
struct OutRows {
    int32_t hq;
    int64_t stride_b, stride_h;
};

hipError_t launch_lse_combine(const float* o_part, const float* lse_part, int32_t rows,
                              int32_t n_parts, int32_t head_dim, void* out, OutRows out_rows, int32_t out_bf16,
                              float* lse_out, hipStream_t stream);

}  // namespace fd
