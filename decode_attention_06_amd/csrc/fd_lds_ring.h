// LDS tile ring shared by the kernels that stream one KV range for many
// query rows (bifurcated context part, prefill): 32-token K/V tiles go
// straight from global memory into a ring of LDS stages
// (global_load_lds_dwordx4), every wave of the workgroup reads each tile
// with the matrix-core operand layouts.  Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_device.h"
#include "fd_mfma_common.h"

namespace fd {
namespace {

constexpr int CTX_TILE = MF_TILE;         // tokens per LDS tile (32)
constexpr int CTX_STAGES = 4;             // LDS ring: three tiles in flight
constexpr int CTX_TILE_BYTES = CTX_TILE * 256;
constexpr int XCDS = 8;

// LDS byte offset of 16-byte chunk c (0..15) of token row t (0..31) in a
// tile: the chunk index is XORed with a linear function of the row bits,
// 2 t0 ^ 4 t1 ^ 8 t3 ^ 4 t4.  Bit 2 of the row never varies within one read
// instruction (it is the token block of a K read, the half h of a V read).
// The function was chosen against the bank behaviour measured with the
// SQ_LDS_BANK_CONFLICT counter on gfx950: 64 four-byte banks; the
// transposing 8-byte V reads serve 32 consecutive lanes per cycle, the
// 16-byte K reads the 16 lanes of one residue mod 4.  With it neither read
// conflicts (counter zero on the prefill kernel; the former XOR of
// (t & 3) | (t >> 3 & 3) << 2 left every V read two cycles of conflicts).
__device__ __forceinline__ int swz(int t) {
    return ((t & 3) << 1) ^ (((t >> 3) & 1) << 3) ^ (((t >> 4) & 1) << 2);
}
__device__ __forceinline__ int lds_off(int t, int c) { return t * 256 + ((c ^ swz(t)) << 4); }

// Issue the loads of one 32-token tile straight into LDS
// (global_load_lds_dwordx4: lane L of a wave instruction lands at the
// instruction's LDS base + 16 L).  Wave w fills K and V bytes
// [2048 w, 2048 w + 2048) of the stage: rows 8w .. 8w+7; lane L of part k
// writes row 8w + 4k + L/16 at chunk position L%16, so it fetches chunk
// (L%16) ^ swz(row) of that row.  Rows at or beyond c1 clamp to c1 - 1
// (c1 > t0 is not required: a tile past the end re-reads row c1 - 1).
// The loads keep the default cache policy, unlike the split-KV kernels'
// read-once KV loads: several workgroups read each tile (the row tiles of a
// bifurcated context piece, every later position tile in prefill), and the
// non-temporal hint measured slower on both (bifurcated 1-3%, prefill
// 2-11%).
// Addresses are a wave-uniform base (row min(t0, c1 - 1)) plus a 32-bit
// lane offset below 32 row strides (`st` elements from one row to the next;
// the host keeps it below 2^24, so a 24-bit multiply forms it), shared by K
// and V.  Four vector-memory
// instructions per wave.
// Offset registers of one wave's loads for a tile (one per KiB per
// operand: 4 waves use both, 8 waves the first).
struct TileAddrs {
    uint32_t off[2];
};

template <int NW>
__device__ __forceinline__ TileAddrs issue_tile(const uint16_t* kbase, const uint16_t* vbase, int st, int t0, int c1,
                                                    int wave, int lane, char* kst, char* vst) {
    typedef __attribute__((address_space(3))) void* lds_ptr;
    constexpr int IPW = 8 / NW;             // 1 KiB loads per wave per operand
    const int tbase = min(t0, c1 - 1);
    const uint16_t* kt = kbase + (int64_t)tbase * st;
    const uint16_t* vt = vbase + (int64_t)tbase * st;
    TileAddrs a;
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
        const int row = 4 * IPW * wave + 4 * k + (lane >> 4);
        const int chunk = (lane & 15) ^ swz(row);
        const int t = min(t0 + row, c1 - 1);
        const int base = 1024 * (IPW * wave + k);
        a.off[k] = __umul24((uint32_t)(t - tbase), (uint32_t)st) + 8 * chunk;
        __builtin_amdgcn_global_load_lds(kt + a.off[k], (lds_ptr)(kst + base), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + a.off[k], (lds_ptr)(vst + base), 16, 0, 0);
    }
    return a;
}

// Keeps the offset registers of the last issued tile alive up to this
// point (no instruction is emitted), so the registers of the LDS reads that
// follow the issue are never the in-flight loads' address registers and the
// compiler needs no wait for them.
template <int NW>
__device__ __forceinline__ void keep_addrs(const TileAddrs& a) {
    if constexpr (NW == 4)
        asm volatile("" ::"v"(a.off[0]), "v"(a.off[1]));
    else
        asm volatile("" ::"v"(a.off[0]));
}

// V^T operand of output block e (d = 16e .. 16e+15) for lane (g, i): the
// eight values V[8g + j][16e + i], j = 0..7, from two transposing LDS reads
// (ds_read_b64_tr_b16: within a 16-lane group, lane 4a + c receives element
// c of the 64-bit rows addressed by lanes a, a+4, a+8, a+12).  For read h,
// lane i of group g addresses token 8g + 4h + i/4, columns 16e + 4 (i%4) ..
// +3, so lane i gets tokens 8g + 4h .. +3 of column 16e + i.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16;

__device__ __forceinline__ u32x4_t v_operand(const char* __restrict__ rv, int e, int g, int i) {
    u32x4_t r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t = 8 * g + 4 * h + (i >> 2);
        const int chunk = 2 * e + ((i & 3) >> 1);
        const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16)(rv + lds_off(t, chunk) + 8 * (i & 1)));
        const u32x2_t w = __builtin_bit_cast(u32x2_t, x);
        r[2 * h] = w[0];
        r[2 * h + 1] = w[1];
    }
    return r;
}

// One ring step: issue the loads of a later tile into stage (wk, wv) and
// read the next tile's operands from stage (rk, rv).  The restrict
// qualifiers state that the stages are disjoint, which lets the compiler
// read one stage while the other is still being filled.
template <int NW>
__device__ __forceinline__ TileAddrs ring_step(const uint16_t* kbase, const uint16_t* vbase, int st, int t_issue, int c1,
                                                   int wave, int lane, char* __restrict__ wk, char* __restrict__ wv,
                                                   const char* __restrict__ rk, const char* __restrict__ rv, int ktok0,
                                                   int g, int i, u32x4_t (&kr)[2][4], u32x4_t (&vt)[8]) {
    const TileAddrs a = issue_tile<NW>(kbase, vbase, st, t_issue, c1, wave, lane, wk, wv);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int tt = ktok0 + 4 * blk;
#pragma unroll
        for (int s = 0; s < 4; ++s) kr[blk][s] = *reinterpret_cast<const u32x4_t*>(rk + lds_off(tt, 4 * s + g));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[e] = v_operand(rv, e, g, i);
    return a;
}

// Online-softmax state of a wave's two 16-row blocks in the ring kernels.
// `m` is the lazily raised reference (log2 domain, see tile_softmax); the
// two derived values change only when it does, so they are kept instead of
// being formed on every tile: `nref`, the weights' offset (-m, or 0 while
// no score has been seen), and `thr`, the raw score above which the
// reference must rise ((m + MF_RESCALE_SLACK) / sl2, or -inf while m is).
struct RingRows {
    float m[2];
    float nref[2];
    float thr[2];
};

__device__ __forceinline__ void ring_rows_init(RingRows& s) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        s.m[r] = -INFINITY;
        s.nref[r] = 0.f;
        s.thr[r] = -INFINITY;
    }
}

// Largest of eight scores in three v_max3_f32 and one v_max_f32.  Through
// fmaxf the compiler first canonicalises two of the inputs (the scores come
// straight from the matrix cores), two more instructions per row block;
// the scores are never signalling NaNs, so the plain maxima are exact.
__device__ __forceinline__ float max8(const float (&t)[8]) {
    float a, b, c, d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(a) : "v"(t[0]), "v"(t[1]), "v"(t[2]));
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(b) : "v"(a), "v"(t[3]), "v"(t[4]));
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(c) : "v"(b), "v"(t[5]), "v"(t[6]));
    asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(c), "v"(t[7]));
    return d;
}

// One ring tile for a wave's 32 query rows: scores, softmax step (masks,
// the lazily raised reference and bf16 weights as in tile_softmax, the row
// sums from the same weights on the matrix cores), then O^T += V^T P^T
// with the transposed V operands (output row m of block e is d = 16e + m).
__device__ __forceinline__ void ring_tile(const u32x4_t (&kr)[2][4], const u32x4_t (&vt)[8],
                                          const bf16x8_t (&qb)[2][4], int tb, int tmask, const int (&lim)[2], int g,
                                          float sl2, RingRows& st, f32x4_t (&lacc)[2], f32x4_t (&acc)[2][8]) {
    const bf16x8_t ones = as_bf16x8(u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    f32x4_t sc[2][2];
    tile_scores<2>(kr, qb, sc);
    float t[2][8];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) t[r][j] = sc[r][j >> 2][j & 3];
    // Masked tokens only in the tiles that reach tmask; the empty asm
    // statements keep this a branch (see tile_softmax).
    if (tb + MF_TILE > tmask) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (tb + 8 * g + j >= lim[r]) t[r][j] = -INFINITY;
                asm volatile("" : "+v"(t[r][j]));
            }
    }
    float mx[2];
    bool raise = false;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        mx[r] = max8(t[r]);
        raise = raise || (mx[r] > st.thr[r]);
    }
    if (__any(raise)) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            float x = fmaxf(mx[r], __shfl_xor(mx[r], 16));
            x = fmaxf(x, __shfl_xor(x, 32));
            const float mn = fmaxf(st.m[r], x * sl2);
            const float alpha = fast_exp2(st.m[r] - ((mn == -INFINITY) ? 0.f : mn));
            lacc[r] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
            st.m[r] = mn;
            st.nref[r] = (mn == -INFINITY) ? 0.f : -mn;
            st.thr[r] = (mn == -INFINITY) ? -INFINITY : (mn + MF_RESCALE_SLACK) / sl2;
        }
    }
    bf16x8_t pb[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[r][j] = (__bf16)fast_exp2(fmaf(t[r][j], sl2, st.nref[r]));
        lacc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[r], lacc[r], 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int r = 0; r < 2; ++r)
            acc[r][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vt[e]), pb[r], acc[r][e], 0, 0, 0);
}

// s_waitcnt with only the vector-memory count constrained (expcnt and
// lgkmcnt at their maxima): wait until at most N loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the fence __syncthreads() carries: that fence
// waits for every outstanding vector-memory load, the tiles still in flight
// included.  The ring needs no more than the barrier itself: each wave has
// waited for its own loads of the tile about to be read (wait_vm) and has
// consumed its LDS reads of the tile whose stage is refilled next.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

constexpr int CTX_LDS_BYTES = CTX_STAGES * 2 * CTX_TILE_BYTES;   // 64 KiB

}  // namespace
}  // namespace fd
