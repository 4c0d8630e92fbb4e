// Split-KV partial work unit on the matrix cores (gfx950, D = 128, bf16
// or OCP E4M3 cache with a bf16 query), shared by the split-KV kernel and
// the decode role of the bifurcated kernel.  Internal.  See fd_mfma.hip for
// the method and the layouts.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fd_device.h"
#include "fd_internal.h"
#include "fd_kv_rows.h"
#include "fd_mfma_common.h"

namespace fd {
namespace {

// Registers of one 32-token tile as loaded.
//  bf16 cache: K in score A-operand layout (token block blk, k-step s: lane
//  (g, i) holds token 8*(i/4) + 4*blk + i%4, d = 32s + 8g .. +8) and V as
//  the lane's 8x8 block (tokens 8g .. 8g+7, d = 8i .. 8i+7).
//  E4M3 cache: K as the lane's 32 contiguous codes of its token, d = 32g ..
//  32g+31 (k-step s takes d = 32g + 8s .. +8; the query fragments use the
//  same assignment, the contraction over d does not depend on it) and V as
//  the lane's 8x8 block of codes.  Codes become bf16 (exactly) only when the
//  tile is computed, so the loads stay in flight meanwhile.
struct Bf16Tile {
    u32x4_t k[2][4];
    u32x4_t v[8];
};
struct Fp8Tile {
    u32x4_t k[2][2];
    u32x2_t v[8];
};

// Loads one tile starting at row tb (tb < t1).  Every load is issued
// unconditionally; a row index at or beyond t1 is clamped to t1 - 1, a valid
// row whose score is masked to -inf later, so no row past the sequence
// length is ever read.  `kb`, `vb`: element offsets from the pool to row 0
// of the lane's K and V rows (dense: the (b, kvh) slice; paged: per group);
// `st`: elements from one row to the next, below 2^24.  Addresses are a
// wave-uniform base at row tbase = min(tb, last) plus a 32-bit lane offset
// of dt = min(tb - tbase + token, last - tbase) rows (0 <= dt <= 31), formed
// with a 24-bit multiply: row tbase + dt = min(tb + token, last), also for
// a paged prefetch whose tile starts past the last row (tb > last).
struct RowWindow {
    int tbase, shift, lim;   // wave-uniform: base row, tb - tbase, last - tbase (both >= 0)
};

__device__ __forceinline__ RowWindow row_window(int tb, int last) {
    const int tbase = min(tb, last);
    return RowWindow{tbase, tb - tbase, last - tbase};
}

__device__ __forceinline__ uint32_t row_off(const RowWindow& w, int token, uint32_t st32) {
    return __umul24((uint32_t)min(w.shift + token, w.lim), st32);
}

// KEEP: plain loads instead of read-once (non-temporal) ones, for rows that
// another workgroup of the same XCD reads right after (the other row blocks
// of a unit): they then come from L2.
template <bool KEEP = false>
__device__ __forceinline__ u32x4_t ld16_rows(const uint16_t* p) {
    if constexpr (KEEP) return ld16(p);
    else return ld16_kv(p);
}

template <bool KEEP = false>
__device__ __forceinline__ void load_rows(const uint16_t* kpool, const uint16_t* vpool, int64_t ko, int64_t vo,
                                          int64_t st, int tb, int last, int ktok0, int g, int i, Bf16Tile& r) {
    const RowWindow w = row_window(tb, last);
    const uint16_t* kt = kpool + ko + (int64_t)w.tbase * st;
    const uint16_t* vt = vpool + vo + (int64_t)w.tbase * st;
    const uint32_t st32 = (uint32_t)st;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const uint32_t off = row_off(w, ktok0 + 4 * blk, st32) + 8u * (uint32_t)g;
#pragma unroll
        for (int s = 0; s < 4; ++s) r.k[blk][s] = ld16_rows<KEEP>(kt + off + 32 * s);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) r.v[j] = ld16_rows<KEEP>(vt + (row_off(w, 8 * g + j, st32) + 8u * (uint32_t)i));
}

template <bool KEEP = false>
__device__ __forceinline__ void load_rows(const uint8_t* kpool, const uint8_t* vpool, int64_t ko, int64_t vo,
                                          int64_t st, int tb, int last, int ktok0, int g, int i, Fp8Tile& r) {
    static_assert(!KEEP, "E4M3 caches are read once");
    const RowWindow w = row_window(tb, last);
    const uint8_t* kt = kpool + ko + (int64_t)w.tbase * st;
    const uint8_t* vt = vpool + vo + (int64_t)w.tbase * st;
    const uint32_t st32 = (uint32_t)st;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const uint32_t off = row_off(w, ktok0 + 4 * blk, st32) + 32u * (uint32_t)g;
        r.k[blk][0] = ld16_kv(kt + off);
        r.k[blk][1] = ld16_kv(kt + off + 16);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) r.v[j] = ld8_kv(vt + (row_off(w, 8 * g + j, st32) + 8u * (uint32_t)i));
}

// Computes one loaded tile (see compute_tile).
template <int NRB, bool PACK>
__device__ __forceinline__ void compute_loaded(const Bf16Tile& r, const bf16x8_t (&qb)[NRB][4], int tb, int t1,
                                               int g, float sl2, float (&m)[NRB], SplitSum<PACK> (&lsum)[NRB],
                                               f32x4_t (&acc)[NRB][8]) {
    compute_tile<NRB, PACK>(r.k, r.v, qb, tb, t1, g, sl2, m, lsum, acc);
}

template <int NRB, bool PACK>
__device__ __forceinline__ void compute_loaded(const Fp8Tile& r, const bf16x8_t (&qb)[NRB][4], int tb, int t1,
                                               int g, float sl2, float (&m)[NRB], SplitSum<PACK> (&lsum)[NRB],
                                               f32x4_t (&acc)[NRB][8]) {
    u32x4_t kr[2][4], vr[8];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4_t& w = r.k[blk][s >> 1];
            const int d0 = (s & 1) * 2;
            kr[blk][s] = fp8x8_to_bf16(w[d0], w[d0 + 1]);
        }
#pragma unroll
    for (int j = 0; j < 8; ++j) vr[j] = fp8x8_to_bf16(r.v[j][0], r.v[j][1]);
    compute_tile<NRB, PACK>(kr, vr, qb, tb, t1, g, sl2, m, lsum, acc);
}

// Paged tiles.  A tile (16-row aligned) covers two 16-row groups, each
// inside one page: PagedTile holds their first rows and page ids (wave-
// uniform; the ids come from scalar loads, looked up two tile loads ahead
// so that their latency hides behind the tiles in between).  A lane's K rows lie
// in group i / 8 and its V rows in group g / 2; rows at or beyond t1 clamp
// to t1 - 1, and kv_group_start gives the group that then holds them.
struct PagedTile {
    int s0, s1;       // first rows of the two groups
    int id0, id1;     // their page ids (table entries)
};

__device__ __forceinline__ PagedTile paged_tile(const PartialParams& p, int b, int tb, int last) {
    PagedTile r;
    r.s0 = kv_group_start(tb, last);
    r.s1 = kv_group_start(tb + 16, last);
    r.id0 = kv_page_id(p, b, r.s0);
    r.id1 = kv_page_id(p, b, r.s1);
    return r;
}

// NRB blocks of 16 query rows per work unit share every K/V load; NW waves
// per workgroup take turns at the 32-token tiles of the unit's piece.  The
// waves' states meet in LDS: per-row max and sum first, then each wave's
// accumulators already scaled by its weight in the merged sum, at word
// row * MF_ACC_STRIDE + d.  Lane (g, i) stores d = 32g + 8ii + e0 .. +3 as
// one 16-byte write; with a row stride of 132 words the 16 lanes of a group
// (rows i = 0..15) cover all 64 banks.
constexpr int MF_ACC_STRIDE = MF_D + 4;

template <int NRB, int NW>
struct PartialLds {
    static constexpr int ROWS = 16 * NRB;
    alignas(16) float acc[NW][ROWS][MF_ACC_STRIDE];
    float m[NW][ROWS];
    float l[NW][ROWS];
};

// PACK: at most 8 query rows per unit (G <= 8, one 16-row block); the
// weights' remainders ride in the block's padding columns (compute_tile).
// KEEP: the unit's KV rows are also read by its other row blocks (see
// load_rows).
template <int NRB, int NW, bool PAGED = false, bool KV8 = false, bool PACK = false, bool KEEP = false>
__device__ __forceinline__ void partial_mfma_body(const PartialParams& p, int bid, PartialLds<NRB, NW>& sh) {
    using Elem = typename std::conditional<KV8, uint8_t, uint16_t>::type;
    using Tile = typename std::conditional<KV8, Fp8Tile, Bf16Tile>::type;
    constexpr int D = MF_D, ROWS = 16 * NRB;
    auto& s_acc = sh.acc;
    auto& s_m = sh.m;
    auto& s_l = sh.l;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop control
    const int g = lane >> 4, i = lane & 15;

    int idx = bid;
    const int split = idx % p.n_splits;
    idx /= p.n_splits;
    const int rblk = idx % p.row_blocks;
    idx /= p.row_blocks;
    const int kvh = idx % p.Hkv;
    const int b = idx / p.Hkv;
    const int G = p.Hq / p.Hkv;
    const int h0 = kvh * G + rblk * ROWS;
    const int nr = min(ROWS, G - rblk * ROWS);   // valid query rows in this unit

    int n = p.lens ? p.lens[b] : (int)p.Lmax;
    n = max(0, min(n, (int)p.Lmax));
    // This piece's rows: the contiguous chunk [t0, t1), read by the waves in
    // tiles t0 + (k * NW + wave) * 32; or, interleaved, the workgroup steps
    // split, split + n_splits, ... of NW * 32 rows of the whole sequence.
    // Interleaved, the whole grid sweeps one window of the cache at a time,
    // which the memory serves faster than every workgroup streaming its own
    // chunk.
    int t0, t1, step;
    if (p.strided) {
        t0 = (int)min((int64_t)split * NW * MF_TILE, (int64_t)n);
        t1 = n;
        step = p.n_splits * NW * MF_TILE;
    } else {
        const int chunk = ((n + p.n_splits - 1) / p.n_splits + 15) & ~15;
        t0 = (int)min((int64_t)split * chunk, (int64_t)n);
        t1 = min(t0 + chunk, n);
        step = NW * MF_TILE;
    }

    // Q^T fragments (B operand of the score product); rows >= nr are zero.
    // k-step s of lane group g covers d = 32s + 8g .. +8 (bf16 cache) or
    // d = 32g + 8s .. +8 (E4M3 cache), as the K fragments do.
    bf16x8_t qb[NRB][4];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        const int row = r * 16 + i;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            const int d0 = KV8 ? 32 * g + 8 * s : 32 * s + 8 * g;
            if (row < nr)
                v = ld16(static_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_stride_b +
                         (int64_t)(h0 + row) * p.q_stride_h + d0);
            qb[r][s] = as_bf16x8(v);
        }
    }

    const Elem* kpool = static_cast<const Elem*>(p.k);
    const Elem* vpool = static_cast<const Elem*>(p.v);
    const int64_t slice = PAGED ? 0 : kv_row_offset<false, D>(p, b, kvh, 0);
    // Token offsets inside a tile for this lane's K rows (one per token block).
    const int ktok0 = 8 * (i >> 2) + (i & 3);
    // Per-KV-head cache scales (E4M3): K's folds into the score scale, V's
    // into the piece's output.
    const float sl2 = p.scale_log2 * (p.k_scale ? p.k_scale[kvh] : 1.f);
    const float vsc = p.v_scale ? p.v_scale[kvh] : 1.f;

    f32x4_t acc[NRB][8];
    // lsum: the running sum; a float per row holding this lane's share
    // (summed over the lane groups at the end), or with PACK an f32x4 whose
    // components hold the whole row sum (columns 8..15: the remainders')
    float m[NRB];
    SplitSum<PACK> lsum[NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        m[r] = -INFINITY;
        lsum[r] = SplitSum<PACK>{};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Two register buffers, alternating: the next tile's loads are in
    // flight while the current tile is computed, and every wait covers
    // exactly one tile's loads.  Dense caches peel the last tile off, so
    // nothing is loaded past the piece's end: an unconditional prefetch
    // there, clamped to row t1 - 1, has every wave of an interleaved grid
    // read the sequence's last row at once at the end of the kernel, and the
    // merge waits for it (peeling measured 1% faster on the CodeLlama share,
    // 4-5% on the bifurcated calls).  Paged caches keep that prefetch: the
    // peeled form needs more than 256 registers there (spills, 12% slower).
    Tile ta, tn;
    // Paged: `ahead` holds the page ids of the next tile to load and
    // `ahead2` those of the one after: each lookup is issued two loads
    // before its use, so the prologue's two loads wait for one round trip.
    PagedTile ahead{}, ahead2{};
    auto load = [&](int at, Tile& r) {
        if constexpr (PAGED) {
            // Offsets to row 0 of each group's page (row t of the group
            // then sits at offset + t * D).
            const int64_t o0 = kv_page_offset<MF_D>(p, ahead.id0, kvh, ahead.s0) - (int64_t)ahead.s0 * MF_D;
            const int64_t o1 = kv_page_offset<MF_D>(p, ahead.id1, kvh, ahead.s1) - (int64_t)ahead.s1 * MF_D;
            load_rows<KEEP>(kpool, vpool, i >= 8 ? o1 : o0, g >= 2 ? o1 : o0, (int64_t)MF_D, at, t1 - 1, ktok0, g, i,
                            r);
            ahead = ahead2;
            ahead2 = paged_tile(p, b, at + 2 * step, t1 - 1);
        } else {
            load_rows<KEEP>(kpool, vpool, slice, slice, p.kv_stride_t, at, t1 - 1, ktok0, g, i, r);
        }
    };
    int tb = t0 + wave * MF_TILE;
    if (tb < t1) {
        if constexpr (PAGED) {
            ahead = paged_tile(p, b, tb, t1 - 1);
            ahead2 = paged_tile(p, b, tb + step, t1 - 1);
        }
        load(tb, ta);
        while (true) {
            if (!PAGED && tb + step >= t1) {
                compute_loaded<NRB, PACK>(ta, qb, tb, t1, g, sl2, m, lsum, acc);
                break;
            }
            load(tb + step, tn);
            compute_loaded<NRB, PACK>(ta, qb, tb, t1, g, sl2, m, lsum, acc);
            tb += step;
            if (PAGED && tb >= t1) break;
            if (!PAGED && tb + step >= t1) {
                compute_loaded<NRB, PACK>(tn, qb, tb, t1, g, sl2, m, lsum, acc);
                break;
            }
            load(tb + step, ta);
            compute_loaded<NRB, PACK>(tn, qb, tb, t1, g, sl2, m, lsum, acc);
            tb += step;
            if (PAGED && tb >= t1) break;
        }
    }

    // Merge of the waves' states.  A row's running sum is first completed
    // over its four lane groups (every lane of the row then holds it).
    // Every lane computes its rows' merged max M and sum L from the waves'
    // (m, l) and scales its own accumulators by exp2(m - M) / L in
    // registers; what is left per output element is a plain sum over waves.
    float lrow[NRB];   // each lane: its row's complete running sum
    if constexpr (PACK) {
        pack_fold(acc);
        lrow[0] = lsum[0][0] + dpp<0x108>(lsum[0][0]);
    } else {
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            lrow[r] = lsum[r] + __shfl_xor(lsum[r], 16);
            lrow[r] += __shfl_xor(lrow[r], 32);
        }
    }
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        const int row = r * 16 + i;
        if (g == 0 && row < nr) {
            s_m[wave][row] = m[r];
            s_l[wave][row] = lrow[r];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        const int row = r * 16 + i;
        if (row < nr) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][row]);
            float L = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int w = 0; w < NW; ++w) L = fmaf(s_l[w][row], fast_exp2(s_m[w][row] - M), L);
            }
            const float f = (L > 0.f) ? fast_exp2(m[r] - M) / L * vsc : 0.f;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
                for (int e0 = 0; e0 < 8; e0 += 4) {
                    f32x4_t o;
                    o[0] = acc[r][e0][ii] * f;
                    o[1] = acc[r][e0 + 1][ii] * f;
                    o[2] = acc[r][e0 + 2][ii] * f;
                    o[3] = acc[r][e0 + 3][ii] * f;
                    *reinterpret_cast<f32x4_t*>(&s_acc[wave][row][32 * g + 8 * ii + e0]) = o;
                }
            if (wave == 0 && g == 0) {
                const float lse = (L > 0.f) ? (M + __log2f(L)) * kLn2f : -INFINITY;
                const int64_t orow = (int64_t)b * p.Hq + h0 + row;
                if (p.direct) {
                    if (p.lse_out) p.lse_out[orow] = lse;
                } else {
                    p.lse_part[orow * p.part_stride + p.part_offset + split] = lse;
                }
            }
        }
    }
    __syncthreads();

    // Four consecutive outputs per thread: the sum of the waves' scaled
    // accumulators.  Vector stores where the destination allows them.
    const bool vec_f32 = (reinterpret_cast<uintptr_t>(p.direct ? p.out : p.o_part) & 15) == 0;
    const bool vec_bf16 = (reinterpret_cast<uintptr_t>(p.out) & 7) == 0;
    for (int x = tid; x < nr * (D / 4); x += NW * 64) {
        const int row = x / (D / 4), d0 = 4 * (x % (D / 4));
        f32x4_t a = *reinterpret_cast<const f32x4_t*>(&s_acc[0][row][d0]);
#pragma unroll
        for (int w = 1; w < NW; ++w) a += *reinterpret_cast<const f32x4_t*>(&s_acc[w][row][d0]);
        const int64_t orow = (int64_t)b * p.Hq + h0 + row;
        if (p.direct) {
            const int64_t o0 = (int64_t)b * p.out_stride_b + (int64_t)(h0 + row) * p.out_stride_h + d0;
            if (p.out_bf16 && vec_bf16) {
                const uint32_t lo = (uint32_t)to_bf16(a[0]) | ((uint32_t)to_bf16(a[1]) << 16);
                const uint32_t hi = (uint32_t)to_bf16(a[2]) | ((uint32_t)to_bf16(a[3]) << 16);
                *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.out) + o0) = u32x2_t{lo, hi};
            } else if (!p.out_bf16 && vec_f32) {
                *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + o0) = a;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) store_out(p.out, o0 + k, a[k], p.out_bf16);
            }
        } else {
            float* dst = p.o_part + (orow * p.part_stride + p.part_offset + split) * D + d0;
            if (vec_f32) {
                *reinterpret_cast<f32x4_t*>(dst) = a;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) dst[k] = a[k];
            }
        }
    }
}

}  // namespace
}  // namespace fd
