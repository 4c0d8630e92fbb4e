// Split-KV decode-attention kernels for gfx950 (CDNA4, wave64).
//
// Method: [FD] "¿Qué es Flash-Decoding y cuándo acelera los LLMs?"
// (slavadubrov.com), section "Por qué la decodificación necesita otra
// planificación": the cached history of each sequence is cut into pieces
// that run as independent work units; each produces a normalised partial
// output and its log-sum-exp, and a reduction renormalises them.  Inside a
// piece the scores never leave the chip: [FA] "In che modo Flash Attention
// riduce il traffico di memoria durante l'inferenza locale?"
// (shop.zimaspace.com), sections on tiling, on the online softmax (running
// max and running sum carried across tiles) and on kernel fusion.
//
// Vector-ALU kernel layout (one 64-lane wave):
//   Each KV row (one token, D elements) is split into 16-byte vectors; LPR
//   consecutive lanes hold one row, so a wave-wide load covers RPW = 64/LPR
//   consecutive rows = 1 KiB of contiguous cache.  A lane keeps the query
//   elements matching its 16-byte slice in registers, forms partial dot
//   products, and a DPP butterfly inside each LPR-lane row group completes
//   the score.  Each row group runs its own online softmax over the tokens it
//   sees (no cross-group max per tile); groups and waves are merged once per
//   piece.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fd_device.h"
#include "fd_internal.h"
#include "fd_kv_rows.h"

namespace fd {
namespace {

// Unpack one 16-byte vector of storage type T into floats.
template <typename T>
struct Vec16;

template <>
struct Vec16<float> {
    static constexpr int N = 4;
    static constexpr int BYTES = 4;
    __device__ static void unpack(const uint4& r, float* f) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
};

template <>
struct Vec16<uint16_t> {  // bf16 bits
    static constexpr int N = 8;
    static constexpr int BYTES = 2;
    __device__ static void unpack(const uint4& r, float* f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
        f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
        f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
};

// OCP E4M3 codes (the cache of the fp8 entry point; its query is bf16).
struct Fp8E4M3 {};

template <>
struct Vec16<Fp8E4M3> {
    static constexpr int N = 16;
    static constexpr int BYTES = 1;
    __device__ static void unpack(const uint4& r, float* f) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], true);
            f[4 * k + 0] = lo[0];
            f[4 * k + 1] = lo[1];
            f[4 * k + 2] = hi[0];
            f[4 * k + 3] = hi[1];
        }
    }
};

// Storage type of the query for a cache element type.
template <typename T>
struct QueryOf {
    using type = T;
};
template <>
struct QueryOf<Fp8E4M3> {
    using type = uint16_t;
};

// Sum over each aligned group of LPR lanes; every lane of the group ends
// with the same bits (each step adds a pair in both orders, and float
// addition commutes).  DPP: quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror; a 32-lane group adds one cross-row swap.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (LPR >= 2) x += dpp<0xB1>(x);
    if constexpr (LPR >= 4) x += dpp<0x4E>(x);
    if constexpr (LPR >= 8) x += dpp<0x141>(x);
    if constexpr (LPR >= 16) x += dpp<0x140>(x);
    if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
    return x;
}

// Merge running state (m2, l2) into (m, l); returns the weights applied to
// the old and the incoming accumulators.  -inf marks "no row seen yet".
__device__ __forceinline__ void merge_weights(float m, float m2, float& mn, float& w1, float& w2) {
    mn = fmaxf(m, m2);
    const float ref = (mn == -INFINITY) ? 0.f : mn;
    w1 = fast_exp2(m - ref);
    w2 = fast_exp2(m2 - ref);
}

template <typename T, int D, int GB, bool PAGED>
__global__ __launch_bounds__(256) void partial_valu_kernel(const PartialParams p) {
    constexpr int EPL = Vec16<T>::N;     // elements per lane per row
    constexpr int LPR = D / EPL;         // lanes per KV row
    constexpr int RPW = 64 / LPR;        // KV rows per wave-wide load
    // Loads in flight per lane, per K and V and buffer.  An E4M3 load holds
    // 16 elements, twice a bf16 load: half as many keep the registers (and
    // the load instructions in flight) the same.
    constexpr int U = ((GB <= 2) ? 8 : 4) / (EPL == 16 ? 2 : 1);
    constexpr int NW = 4;                // waves per workgroup
    constexpr int WAVE_TOK = RPW * U;
    constexpr int WG_TOK = NW * WAVE_TOK;
    static_assert(LPR * RPW == 64, "row groups must tile the wave");
    static_assert(WG_TOK == valu_tile_rows(16 / EPL, D, GB), "workgroup step as the host computes it");

    __shared__ float s_acc[NW][GB][D];
    __shared__ float s_m[NW][GB];
    __shared__ float s_l[NW][GB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop control
    const int r = lane / LPR, c = lane % LPR;

    int idx = blockIdx.x;
    const int split = idx % p.n_splits;
    idx /= p.n_splits;
    const int rb = idx % p.row_blocks;
    idx /= p.row_blocks;
    const int kvh = idx % p.Hkv;
    const int b = idx / p.Hkv;
    const int h0 = kvh * (GB * p.row_blocks) + rb * GB;

    // Valid rows of this sequence and this unit's piece: the contiguous
    // rows [t0, t1), ceil(n / n_splits) rounded up to 16 long, walked in
    // workgroup tiles of WG_TOK rows; or, interleaved, the workgroup tiles
    // split, split + n_splits, ... of the whole sequence (t1 = n), so that
    // the grid sweeps one window of the cache at a time.
    int n = p.lens ? p.lens[b] : (int)p.Lmax;
    n = max(0, min(n, (int)p.Lmax));
    int t0, t1, wg_step;
    if (p.strided) {
        t0 = (int)min((int64_t)split * WG_TOK, (int64_t)n);
        t1 = n;
        wg_step = p.n_splits * WG_TOK;
    } else {
        const int chunk = ((n + p.n_splits - 1) / p.n_splits + 15) & ~15;
        t0 = (int)min((int64_t)split * chunk, (int64_t)n);
        t1 = min(t0 + chunk, n);
        wg_step = WG_TOK;
    }

    // Query slice of this lane, pre-multiplied by scale*log2(e) (and the
    // KV head's K scale for an E4M3 cache) so that exp2 of a score
    // difference is the softmax weight ratio.
    using TQ = typename QueryOf<T>::type;
    const float sl2 = p.scale_log2 * (p.k_scale ? p.k_scale[kvh] : 1.f);
    const float vsc = p.v_scale ? p.v_scale[kvh] : 1.f;
    float qf[GB][EPL];
#pragma unroll
    for (int g = 0; g < GB; ++g) {
        const TQ* qp = static_cast<const TQ*>(p.q) + (int64_t)b * p.q_stride_b + (int64_t)(h0 + g) * p.q_stride_h +
                       c * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += Vec16<TQ>::N)
            Vec16<TQ>::unpack(*reinterpret_cast<const uint4*>(qp + e), &qf[g][e]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[g][e] *= sl2;
    }

    // Rows are addressed per 16-row group: a wave-uniform 64-bit base (the
    // dense slice's row, or the row's page) plus a 32-bit lane offset below
    // 16 rows (the host keeps 16 row strides below 2^31 bytes), so each load
    // takes one offset register.  A wave tile covers NG groups; the rows of
    // load u lie in group u * RPW / 16.  Pages hold their rows D apart.
    const char* kpool = static_cast<const char*>(p.k);
    const char* vpool = static_cast<const char*>(p.v);
    const int64_t slice = PAGED ? 0 : kv_row_offset<false, D>(p, b, kvh, 0);
    constexpr int SZ = Vec16<T>::BYTES;
    const uint32_t lane_off = c * EPL * (uint32_t)SZ;
    const int64_t row_st = PAGED ? (int64_t)D : p.kv_stride_t;      // elements between rows, below 2^24
    const uint32_t row_st32 = (uint32_t)row_st;
    constexpr int NG = WAVE_TOK >= 16 ? WAVE_TOK / 16 : 1;
    static_assert(16 % RPW == 0, "a load's rows must stay inside one 16-row group");

    float m[GB], l[GB], acc[GB][EPL];
#pragma unroll
    for (int g = 0; g < GB; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    // Paged: first rows and page ids of the 16-row groups of the next tile
    // to load (gs, gid) and of the one after (gs2, gid2): scalar loads issued
    // two tile loads ahead of their use, so the first two loads wait for one
    // round trip.
    int gs[NG], gid[NG], gs2[NG], gid2[NG];
    auto lookup = [&](int at, int (&s_out)[NG], int (&id_out)[NG]) {
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            s_out[h] = kv_group_start(at + 16 * h, t1 - 1);
            id_out[h] = kv_page_id(p, b, s_out[h]);
        }
    };
    auto lookup_first = [&](int at) {
        lookup(at, gs, gid);
        lookup(at + wg_step, gs2, gid2);
    };

    // Loads one wave tile starting at row tb.  Unconditional: rows at or
    // beyond t1 clamp to t1 - 1 (a valid row, masked in compute), so the
    // loads issue back to back and a prefetch past the piece's end only
    // re-reads that row.
    auto load = [&](int tb, uint4 (&kr)[U], uint4 (&vr)[U]) {
        int64_t gb[NG];   // bytes from the pool to row gs[h]
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            if constexpr (PAGED) {
                gb[h] = kv_page_offset<D>(p, gid[h], kvh, gs[h]) * (int64_t)SZ;
            } else {
                gs[h] = kv_group_start(tb + 16 * h, t1 - 1);
                gb[h] = (slice + (int64_t)gs[h] * row_st) * (int64_t)SZ;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int h = (NG > 1) ? (u * RPW) / 16 : 0;
            const int t = min(tb + u * RPW + r, t1 - 1);
            const uint32_t off = __umul24((uint32_t)(t - gs[h]), row_st32) * (uint32_t)SZ + lane_off;
            kr[u] = ld_stream16(kpool + gb[h] + off);
            vr[u] = ld_stream16(vpool + gb[h] + off);
        }
        if constexpr (PAGED) {
#pragma unroll
            for (int h = 0; h < NG; ++h) {
                gs[h] = gs2[h];
                gid[h] = gid2[h];
            }
            lookup(tb + 2 * wg_step, gs2, gid2);
        }
    };

    // Scores, online-softmax update and P.V for one loaded wave tile.
    auto compute = [&](int tb, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
        const bool full = tb + WAVE_TOK <= t1;
        // Scores (log2 domain).  All lanes take part in the DPP sums.
        float s[U][GB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[EPL];
            Vec16<T>::unpack(kr[u], kf);
#pragma unroll
            for (int g = 0; g < GB; ++g) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) d = fmaf(qf[g][e], kf[e], d);
                s[u][g] = group_sum<LPR>(d);
            }
        }
        if (!full) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (tb + u * RPW + r >= t1)
#pragma unroll
                    for (int g = 0; g < GB; ++g) s[u][g] = -INFINITY;
        }

        // Online softmax update, one rescale per tile.
        float pr[U][GB];
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            float mt = s[0][g];
#pragma unroll
            for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][g]);
            const float mn = fmaxf(m[g], mt);
            const float ref = (mn == -INFINITY) ? 0.f : mn;
            const float alpha = fast_exp2(m[g] - ref);
            float lsum = l[g] * alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pr[u][g] = fast_exp2(s[u][g] - ref);
                lsum += pr[u][g];
            }
            l[g] = lsum;
            m[g] = mn;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
            Vec16<T>::unpack(vr[u], vf);
#pragma unroll
            for (int g = 0; g < GB; ++g)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pr[u][g], vf[e], acc[g][e]);
        }
    };

    // Two register buffers, both in flight before the loop: each tile is
    // computed, then its buffer is refilled with the tile after next, so the
    // other buffer's loads stay in flight across every compute.  A counted
    // loop over tile pairs with one exit keeps each buffer in its registers
    // across the back edge; the scheduling barriers keep each refill after
    // the compute that frees its registers and ahead of the next compute's
    // waits.
    // Eight query rows per unit leave no registers for a second buffer.
    const int tb0 = t0 + wave * WAVE_TOK;
    if (GB >= 8) {
        if (tb0 < t1) {
            if constexpr (PAGED) lookup_first(tb0);
            uint4 ka[U], va[U];
            for (int tb = tb0; tb < t1; tb += wg_step) {
                load(tb, ka, va);
                compute(tb, ka, va);
            }
        }
    } else if (tb0 < t1) {
        const int ntiles = (t1 - tb0 + wg_step - 1) / wg_step;
        uint4 ka[U], va[U], kn[U], vn[U];
        if constexpr (PAGED) lookup_first(tb0);
        load(tb0, ka, va);
        load(tb0 + wg_step, kn, vn);
        int tb = tb0;
        for (int it = 0; it < ntiles / 2; ++it) {
            compute(tb, ka, va);
            __builtin_amdgcn_sched_barrier(0);
            load(tb + 2 * wg_step, ka, va);
            __builtin_amdgcn_sched_barrier(0);
            compute(tb + wg_step, kn, vn);
            __builtin_amdgcn_sched_barrier(0);
            load(tb + 3 * wg_step, kn, vn);
            __builtin_amdgcn_sched_barrier(0);
            tb += 2 * wg_step;
        }
        if (ntiles & 1) compute(tb, ka, va);
    }

    // Merge the RPW row groups of the wave (butterfly across lane offsets
    // LPR, 2*LPR, ...).  Afterwards group 0 holds the wave's state.
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            const float m2 = __shfl_xor(m[g], off);
            const float l2 = __shfl_xor(l[g], off);
            float mn, w1, w2;
            merge_weights(m[g], m2, mn, w1, w2);
            l[g] = l[g] * w1 + l2 * w2;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * w1 + __shfl_xor(acc[g][e], off) * w2;
            m[g] = mn;
        }
    }
    if (r == 0) {
#pragma unroll
        for (int g = 0; g < GB; ++g) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) s_acc[wave][g][c * EPL + e] = acc[g][e];
            if (c == 0) {
                s_m[wave][g] = m[g];
                s_l[wave][g] = l[g];
            }
        }
    }
    __syncthreads();

    // Merge the waves (fixed order) and write this piece's result.
    for (int i = tid; i < GB * D; i += NW * 64) {
        const int g = i / D, d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float a = fast_exp2(s_m[w][g] - M);
                L = fmaf(s_l[w][g], a, L);
                A = fmaf(s_acc[w][g][d], a, A);
            }
        }
        const float o = (L > 0.f) ? A / L * vsc : 0.f;
        const float lse = (L > 0.f) ? (M + __log2f(L)) * kLn2f : -INFINITY;
        const int64_t row = (int64_t)b * p.Hq + h0 + g;
        if (p.direct) {
            store_out(p.out, (int64_t)b * p.out_stride_b + (int64_t)(h0 + g) * p.out_stride_h + d, o, p.out_bf16);
            if (d == 0 && p.lse_out) p.lse_out[row] = lse;
        } else {
            const int64_t slot = row * p.part_stride + p.part_offset + split;
            p.o_part[slot * D + d] = o;
            if (d == 0) p.lse_part[slot] = lse;
        }
    }
}

// LSE combine ([FD] "Por qué la decodificación necesita otra
// planificación": the reduction that renormalises the pieces), general
// form for head dims that are not a multiple of 4 or an unaligned o_part
// (lse_combine_v4_kernel below serves the rest).  One
// workgroup per (row, slice of CMB_SLICE columns); thread (part group pg,
// column vector dv) handles pieces pg, pg + GROUPS, ...  The first batch of
// partial outputs is requested together with the row's lse values, so a row
// with up to 8 * GROUPS pieces costs one memory round trip.  Piece weights are
// exp(lse_i - max lse); sums run in a fixed order (bitwise repeatable).
constexpr int CMB_THREADS = 256;
constexpr int CMB_SLICE = 16;                   // columns per workgroup
constexpr int CMB_BATCH = 8;                    // pieces in flight per thread

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int k = 1; k < CMB_THREADS / 64; ++k) r = fmaxf(r, red[k]);
    return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int k = 1; k < CMB_THREADS / 64; ++k) r += red[k];
    return r;
}

template <int VEC>
__device__ __forceinline__ void load_vec(const float* src, float (&v)[VEC]) {
    if constexpr (VEC == 4) {
        const float4 t = *reinterpret_cast<const float4*>(src);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] = src[e];
    }
}

// Element offset of output row `row` (see OutRows; rows stay below 2^30,
// so the division is a 32-bit one).
__device__ __forceinline__ int64_t out_row_offset(const OutRows& o, int64_t row) {
    const int32_t r = (int32_t)row;
    return (int64_t)(r / o.hq) * o.stride_b + (int64_t)(r % o.hq) * o.stride_h;
}

template <int VEC>
__global__ __launch_bounds__(CMB_THREADS) void lse_combine_kernel(const float* __restrict__ o_part,
                                                                  const float* __restrict__ lse_part,
                                                                  int32_t n_parts, int32_t D, void* out,
                                                                  OutRows orows, int32_t out_bf16, float* lse_out) {
    constexpr int DL = CMB_SLICE / VEC;         // threads across the slice
    constexpr int GROUPS = CMB_THREADS / DL;    // part groups
    __shared__ float s_red[CMB_THREADS / 64];
    __shared__ float s_acc[GROUPS][CMB_SLICE];

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const float* lrow = lse_part + row * n_parts;
    const int dv = tid % DL, pg = tid / DL;
    const int d0 = blockIdx.y * CMB_SLICE + dv * VEC;
    const bool col_ok = d0 < D;
    const float* obase = o_part + row * (int64_t)n_parts * D + d0;

    // Batch 0: partial outputs and their lse, requested together.
    float ov[CMB_BATCH][VEC], lv[CMB_BATCH];
#pragma unroll
    for (int u = 0; u < CMB_BATCH; ++u) {
        const int i = pg + u * GROUPS;
        lv[u] = (i < n_parts) ? lrow[i] : -INFINITY;
        if (i < n_parts && col_ok)
            load_vec<VEC>(obase + (int64_t)i * D, ov[u]);
        else
#pragma unroll
            for (int e = 0; e < VEC; ++e) ov[u][e] = 0.f;
    }
    // Row maximum and weight sum over all pieces.  With at most
    // CMB_BATCH * GROUPS pieces the lse values already in registers cover the
    // row (each piece is held by the DL threads of its group; only dv == 0
    // counts it in the sum); longer rows read the rest.
    const bool one_batch = n_parts <= CMB_BATCH * GROUPS;
    float M = -INFINITY;
    if (one_batch) {
#pragma unroll
        for (int u = 0; u < CMB_BATCH; ++u) M = fmaxf(M, lv[u]);
    } else {
        for (int i = tid; i < n_parts; i += CMB_THREADS) M = fmaxf(M, lrow[i]);
    }
    M = block_max(M, s_red);
    float z = 0.f;
    if (M != -INFINITY) {
        if (one_batch) {
            if (dv == 0)
#pragma unroll
                for (int u = 0; u < CMB_BATCH; ++u)
                    z += (lv[u] == -INFINITY) ? 0.f : fast_exp2((lv[u] - M) * kLog2ef);
        } else {
            for (int i = tid; i < n_parts; i += CMB_THREADS) {
                const float li = lrow[i];
                z += (li == -INFINITY) ? 0.f : fast_exp2((li - M) * kLog2ef);
            }
        }
    }
    const float Z = block_sum(z, s_red);

    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int u = 0; u < CMB_BATCH; ++u) {
            const float w = (lv[u] == -INFINITY) ? 0.f : fast_exp2((lv[u] - M) * kLog2ef);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = fmaf(w, ov[u][e], acc[e]);
        }
        for (int base = CMB_BATCH * GROUPS; base < n_parts; base += CMB_BATCH * GROUPS) {
#pragma unroll
            for (int u = 0; u < CMB_BATCH; ++u) {
                const int i = base + pg + u * GROUPS;
                lv[u] = (i < n_parts) ? lrow[i] : -INFINITY;
                if (i < n_parts && col_ok)
                    load_vec<VEC>(obase + (int64_t)i * D, ov[u]);
                else
#pragma unroll
                    for (int e = 0; e < VEC; ++e) ov[u][e] = 0.f;
            }
#pragma unroll
            for (int u = 0; u < CMB_BATCH; ++u) {
                const float w = (lv[u] == -INFINITY) ? 0.f : fast_exp2((lv[u] - M) * kLog2ef);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] = fmaf(w, ov[u][e], acc[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) s_acc[pg][dv * VEC + e] = acc[e];
    __syncthreads();
    if (tid < CMB_SLICE) {
        const int d = blockIdx.y * CMB_SLICE + tid;
        if (d < D) {
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < GROUPS; ++k) a += s_acc[k][tid];
            store_out(out, out_row_offset(orows, row) + d, (Z > 0.f) ? a / Z : 0.f, out_bf16);
            if (d == 0 && lse_out) lse_out[row] = (Z > 0.f) ? M + logf(Z) : -INFINITY;
        }
    }
}

// LSE combine with 16-byte columns (head_dim a multiple of 4, o_part
// 16-byte aligned): one workgroup per (row, 32 columns).  Thread (piece
// group pg = tid / 8, column vector cv = tid % 8) holds pieces pg, pg + 32,
// pg + 64, pg + 96 of the current batch of 128, their lse and their four
// columns, all requested in one round trip.  The row maximum takes one wave
// reduction and one barrier; the weighted sums reduce over the eight piece
// groups of a wave by three butterfly steps (lanes 8 apart) and over the
// four waves through LDS.  Every sum runs in a fixed order.
constexpr int CMB4_CV = 8;                      // float4 column vectors per workgroup
constexpr int CMB4_PG = 32;                     // piece groups
constexpr int CMB4_BATCH = 4;                   // pieces per thread per batch

__global__ __launch_bounds__(256) void lse_combine_v4_kernel(const float* __restrict__ o_part,
                                                             const float* __restrict__ lse_part, int32_t n_parts,
                                                             int32_t D, void* out, OutRows orows, int32_t out_bf16,
                                                             float* lse_out) {
    __shared__ float s_m[4], s_z[4];
    __shared__ float4 s_acc[4][CMB4_CV];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cv = tid % CMB4_CV, pg = tid / CMB4_CV;
    const int64_t row = blockIdx.x;
    const int c4 = blockIdx.y * CMB4_CV + cv;
    const bool col_ok = 4 * c4 < D;
    const float* lrow = lse_part + row * n_parts;
    const float* obase = o_part + row * (int64_t)n_parts * D + 4 * c4;
    constexpr int PER_BATCH = CMB4_PG * CMB4_BATCH;

    float lv[CMB4_BATCH];
    float4 ov[CMB4_BATCH];
    auto load_batch = [&](int base) {
#pragma unroll
        for (int u = 0; u < CMB4_BATCH; ++u) {
            const int i = base + pg + CMB4_PG * u;
            lv[u] = (i < n_parts) ? lrow[i] : -INFINITY;
            ov[u] = (i < n_parts && col_ok) ? *reinterpret_cast<const float4*>(obase + (int64_t)i * D)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    load_batch(0);

    // Row maximum over all pieces.
    float mloc = lv[0];
#pragma unroll
    for (int u = 1; u < CMB4_BATCH; ++u) mloc = fmaxf(mloc, lv[u]);
    for (int i = PER_BATCH + pg; i < n_parts; i += CMB4_PG) mloc = fmaxf(mloc, lrow[i]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    if (lane == 0) s_m[wave] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));

    // This thread's weighted sums, batch by batch.
    float z = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY) {
        for (int base = 0;;) {
#pragma unroll
            for (int u = 0; u < CMB4_BATCH; ++u) {
                const float w = (lv[u] == -INFINITY) ? 0.f : fast_exp2((lv[u] - M) * kLog2ef);
                z += w;
                a.x = fmaf(w, ov[u].x, a.x);
                a.y = fmaf(w, ov[u].y, a.y);
                a.z = fmaf(w, ov[u].z, a.z);
                a.w = fmaf(w, ov[u].w, a.w);
            }
            base += PER_BATCH;
            if (base >= n_parts) break;
            load_batch(base);
        }
    }
    // Sum over the wave's eight piece groups (lanes 8, 16, 32 apart), then
    // over the waves.  Each column vector's lanes carry every piece, so
    // their z is the wave's weight sum.
#pragma unroll
    for (int off = CMB4_CV; off < 64; off <<= 1) {
        z += __shfl_xor(z, off);
        a.x += __shfl_xor(a.x, off);
        a.y += __shfl_xor(a.y, off);
        a.z += __shfl_xor(a.z, off);
        a.w += __shfl_xor(a.w, off);
    }
    if (lane < CMB4_CV) s_acc[wave][lane] = a;
    if (lane == 0) s_z[wave] = z;
    __syncthreads();
    if (tid < CMB4_CV && col_ok) {
        const float Z = (s_z[0] + s_z[1]) + (s_z[2] + s_z[3]);
        float4 A = s_acc[0][tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            A.x += s_acc[w][tid].x;
            A.y += s_acc[w][tid].y;
            A.z += s_acc[w][tid].z;
            A.w += s_acc[w][tid].w;
        }
        const float inv = (Z > 0.f) ? 1.f / Z : 0.f;
        const int64_t o0 = out_row_offset(orows, row) + 4 * c4;
        store_out(out, o0, A.x * inv, out_bf16);
        store_out(out, o0 + 1, A.y * inv, out_bf16);
        store_out(out, o0 + 2, A.z * inv, out_bf16);
        store_out(out, o0 + 3, A.w * inv, out_bf16);
        if (c4 == 0 && lse_out) lse_out[row] = (Z > 0.f) ? M + logf(Z) : -INFINITY;
    }
}

// LSE combine for rows with at most 64 pieces (the bifurcated calls and
// short splits): one wave per row.  Lane j holds piece j's lse; the row
// maximum and the weight sum are butterfly reductions (every lane ends with
// the same bits); piece weights reach all lanes through v_readlane, and lane
// j accumulates columns j, j + 64, ...  The first batch of PB pieces is
// requested together with the lse values, so a row of up to that many pieces
// costs one memory round trip.  PB is the smallest multiple of 8 that covers
// the pieces (at most 64 loads in flight per lane): a batch past the last
// piece re-reads it, so a tight batch saves those loads.
constexpr int CMBW_ROWS = 4;                    // rows (waves) per workgroup
constexpr int CMBW_MAXV = 8;                    // columns per lane: D <= 512

template <int NV, int PB>
__global__ __launch_bounds__(64 * CMBW_ROWS) void lse_combine_rows_kernel(const float* __restrict__ o_part,
                                                                          const float* __restrict__ lse_part,
                                                                          int32_t rows, int32_t n_parts, int32_t D,
                                                                          void* out, OutRows orows, int32_t out_bf16,
                                                                          float* lse_out) {
    static_assert(PB * NV <= 64 && PB % 8 == 0, "pieces per batch");
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * CMBW_ROWS + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float* base = o_part + row * (int64_t)n_parts * D;
    float v[PB][NV];
    auto load = [&](int i0) {
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const int i = min(i0 + u, n_parts - 1);
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int d = lane + 64 * k;
                v[u][k] = (d < D) ? base[(int64_t)i * D + d] : 0.f;
            }
        }
    };
    const float li = (lane < n_parts) ? lse_part[row * n_parts + lane] : -INFINITY;
    load(0);
    float M = li;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = (li == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2((li - M) * kLog2ef);
    float Z = w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) Z += __shfl_xor(Z, off);

    float acc[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.f;
    for (int i0 = 0;;) {
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            if (i0 + u < n_parts) {
                const float wf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i0 + u));
#pragma unroll
                for (int k = 0; k < NV; ++k) acc[k] = fmaf(wf, v[u][k], acc[k]);
            }
        }
        i0 += PB;
        if (i0 >= n_parts) break;
        load(i0);
    }
    const float inv = (Z > 0.f) ? 1.f / Z : 0.f;
    const int64_t o0 = out_row_offset(orows, row);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int d = lane + 64 * k;
        if (d < D) store_out(out, o0 + d, acc[k] * inv, out_bf16);
    }
    if (lane == 0 && lse_out) lse_out[row] = (Z > 0.f) ? M + logf(Z) : -INFINITY;
}

// HBM read ceiling: each workgroup streams one contiguous chunk of the
// buffer with 16-byte loads (the KV loads' non-temporal hint), eight in
// flight per thread, and folds the data into a word so the loads cannot be
// dropped.
constexpr int PROBE_UNROLL = 8;
constexpr size_t PROBE_CHUNK = 16384;          // bytes per workgroup

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ buf, size_t n16,
                                                         uint32_t* sink) {
    const size_t per_wg = PROBE_CHUNK / 16;
    const size_t base = (size_t)blockIdx.x * per_wg;
    const size_t end = min(base + per_wg, n16);
    uint32_t acc = 0;
    for (size_t i = base + threadIdx.x; i < end; i += 256 * PROBE_UNROLL) {
        uint4 v[PROBE_UNROLL];
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) {
            const size_t j = min(i + (size_t)u * 256, end - 1);
            v[u] = ld_stream16(buf + j);
        }
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

template <typename T, int D, bool PAGED>
hipError_t launch_valu_rows(const PartialParams& p, int rows_per_block, hipStream_t stream) {
    const int64_t wgs = (int64_t)p.B * p.Hkv * p.row_blocks * p.n_splits;
    if (wgs >= (int64_t(1) << 30)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    const dim3 block(256);
    switch (rows_per_block) {
        case 1: hipLaunchKernelGGL((partial_valu_kernel<T, D, 1, PAGED>), grid, block, 0, stream, p); break;
        case 2: hipLaunchKernelGGL((partial_valu_kernel<T, D, 2, PAGED>), grid, block, 0, stream, p); break;
        case 4: hipLaunchKernelGGL((partial_valu_kernel<T, D, 4, PAGED>), grid, block, 0, stream, p); break;
        case 8:
            // An E4M3 cache uses at most 4 rows per unit (valu_rows_per_block).
            if constexpr (Vec16<T>::N == 16) return hipErrorInvalidValue;
            else hipLaunchKernelGGL((partial_valu_kernel<T, D, 8, PAGED>), grid, block, 0, stream, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu_layout(const PartialParams& p, int rows_per_block, hipStream_t stream) {
    return p.block_table ? launch_valu_rows<T, D, true>(p, rows_per_block, stream)
                         : launch_valu_rows<T, D, false>(p, rows_per_block, stream);
}

}  // namespace

hipError_t launch_partial_valu(const PartialParams& p, int dtype, int head_dim, int rows_per_block,
                               hipStream_t stream) {
    if (dtype == 0) {
        if (head_dim == 64) return launch_valu_layout<float, 64>(p, rows_per_block, stream);
        if (head_dim == 128) return launch_valu_layout<float, 128>(p, rows_per_block, stream);
    } else if (dtype == 2) {
        if (head_dim == 64) return launch_valu_layout<Fp8E4M3, 64>(p, rows_per_block, stream);
        if (head_dim == 128) return launch_valu_layout<Fp8E4M3, 128>(p, rows_per_block, stream);
    } else {
        if (head_dim == 64) return launch_valu_layout<uint16_t, 64>(p, rows_per_block, stream);
        if (head_dim == 128) return launch_valu_layout<uint16_t, 128>(p, rows_per_block, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const size_t wgs = (bytes + PROBE_CHUNK - 1) / PROBE_CHUNK;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)wgs), dim3(256), 0, stream,
                       static_cast<const uint4*>(buf), n16, sink);
    return hipGetLastError();
}

hipError_t launch_lse_combine(const float* o_part, const float* lse_part, int32_t rows,
                              int32_t n_parts, int32_t head_dim, void* out, OutRows orows, int32_t out_bf16,
                              float* lse_out, hipStream_t stream) {
    // One wave per row when rows are plentiful and pieces few; otherwise a
    // row spreads over several workgroups: 32 columns each with 16-byte
    // loads, or 16 columns each (scalar loads) for other head dims or an
    // unaligned o_part.
    if (n_parts <= 64 && rows >= 1024) {
        const dim3 grid((unsigned)((rows + CMBW_ROWS - 1) / CMBW_ROWS));
        const dim3 block(64 * CMBW_ROWS);
        const int nv = (head_dim + 63) / 64;
        const int pb8 = (n_parts + 7) / 8;   // batch of pieces, in eights
#define FD_CMBW(NV_, PB_) hipLaunchKernelGGL((lse_combine_rows_kernel<NV_, PB_>), grid, block, 0, stream, o_part, \
                                             lse_part, rows, n_parts, head_dim, out, orows, out_bf16, lse_out)
        if (nv <= 2) {
            if (pb8 <= 1) {
                if (nv <= 1) FD_CMBW(1, 8);
                else FD_CMBW(2, 8);
            } else if (pb8 == 2) {
                if (nv <= 1) FD_CMBW(1, 16);
                else FD_CMBW(2, 16);
            } else if (pb8 == 3) {
                if (nv <= 1) FD_CMBW(1, 24);
                else FD_CMBW(2, 24);
            } else {
                if (nv <= 1) FD_CMBW(1, 32);
                else FD_CMBW(2, 32);
            }
        } else if (nv <= 4) {
            if (pb8 <= 1) FD_CMBW(4, 8);
            else FD_CMBW(4, 16);
        } else {
            FD_CMBW(CMBW_MAXV, 8);
        }
#undef FD_CMBW
        return hipGetLastError();
    }
    const bool vec4 = (head_dim % 4 == 0) && (reinterpret_cast<uintptr_t>(o_part) % 16 == 0);
    if (vec4) {
        const dim3 grid4((unsigned)rows, (unsigned)((head_dim / 4 + CMB4_CV - 1) / CMB4_CV));
        hipLaunchKernelGGL(lse_combine_v4_kernel, grid4, dim3(256), 0, stream, o_part, lse_part, n_parts, head_dim,
                           out, orows, out_bf16, lse_out);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)rows, (unsigned)((head_dim + CMB_SLICE - 1) / CMB_SLICE));
    hipLaunchKernelGGL(lse_combine_kernel<1>, grid, dim3(CMB_THREADS), 0, stream, o_part, lse_part,
                           n_parts, head_dim, out, orows, out_bf16, lse_out);
    return hipGetLastError();
}

}  // namespace fd
