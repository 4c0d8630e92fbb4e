// Bifurcated attention, context part, on the matrix cores (gfx950, bf16,
// head_dim 128).
//
// Method: [BA] "Effiziente Verarbeitung und Analyse von Inhalten durch
// bifurkierte Aufmerksamkeit für Single-Context-Batch-Sampling" (linnk.ai),
// section "Tiivistelmä": all samples drawn from one context attend to the same
// context K/V, so the context part is one contraction of every sample's query
// rows against that KV, read once; the per-sample decode part is separate;
// the result is exact.  Here the context rows are cut into pieces ([FD]
// "¿Qué es Flash-Decoding y cuándo acelera los LLMs?", section "Por qué la
// decodificación necesita otra planificación") whose partial outputs and
// log-sum-exps join the decode pieces in the LSE combine.
//
// Work unit: (KV head, context piece, tile of 32 * CTX_NW query rows).  The
// query rows of a KV head are the (sample, head-in-group) pairs that read it,
// S * G of them.  A workgroup streams 32-token K/V tiles straight from global
// memory into a ring of LDS stages (XOR-swizzled 16-byte chunks, three tiles
// in flight) and every wave contracts them
// against its own 32 rows with the same register layout as the split-KV
// matrix-core kernel, so each wave owns its rows for the whole piece and no
// cross-wave merge is needed.  Workgroup ids are arranged so that all row
// tiles of one (KV head, piece) land on the same XCD and share its L2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fd_device.h"
#include "fd_internal.h"
#include "fd_mfma_common.h"

namespace fd {
namespace {

constexpr int CTX_NW = 4;                 // waves per workgroup
constexpr int CTX_ROWS = 32 * CTX_NW;     // query rows per workgroup
constexpr int CTX_TILE = MF_TILE;         // tokens per LDS tile (32)
constexpr int CTX_STAGES = 4;             // LDS ring: three tiles in flight
constexpr int CTX_TILE_BYTES = CTX_TILE * 256;
constexpr int XCDS = 8;

// LDS byte offset of 16-byte chunk c (0..15) of token row t (0..31) in a
// tile.  The chunk index is XORed with (t & 3) | (bits 3-4 of t) << 2, which
// makes the K-operand reads (16 lanes: tokens {0..3, 8..11, 16..19, 24..27}
// + const, one chunk) and the V-block reads (16 lanes: one token, chunks
// 0..15) touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int t) { return (t & 3) | (((t >> 3) & 3) << 2); }
__device__ __forceinline__ int lds_off(int t, int c) { return t * 256 + ((c ^ swz(t)) << 4); }

// Issue the loads of one 32-token tile straight into LDS
// (global_load_lds_dwordx4: lane L of a wave instruction lands at the
// instruction's LDS base + 16 L).  Wave w fills K and V bytes
// [2048 w, 2048 w + 2048) of the stage: rows 8w .. 8w+7; lane L of part k
// writes row 8w + 4k + L/16 at chunk position L%16, so it fetches chunk
// (L%16) ^ swz(row) of that row.  Rows at or beyond c1 clamp to c1 - 1.
// Four vector-memory instructions per wave.
__device__ __forceinline__ void issue_tile(const uint16_t* kbase, const uint16_t* vbase, int t0, int c1,
                                           int wave, int lane, char* kst, char* vst) {
    typedef __attribute__((address_space(3))) void* lds_ptr;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int row = 8 * wave + 4 * k + (lane >> 4);
        const int chunk = (lane & 15) ^ swz(row);
        const int t = min(t0 + row, c1 - 1);
        const int base = 1024 * (2 * wave + k);
        __builtin_amdgcn_global_load_lds(kbase + (int64_t)t * MF_D + 8 * chunk, (lds_ptr)(kst + base), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vbase + (int64_t)t * MF_D + 8 * chunk, (lds_ptr)(vst + base), 16, 0, 0);
    }
}

// s_waitcnt with only the vector-memory count constrained (expcnt and
// lgkmcnt at their maxima): wait until at most N loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__global__ __launch_bounds__(64 * CTX_NW, 2) void bif_context_kernel(const BifContextParams p) {
    // One LDS object per stage and per operand, addressed with constant stage
    // numbers only, so the compiler can tell the tile being read from the
    // tiles still being written by in-flight loads.
    __shared__ __attribute__((aligned(16))) char s_k0[CTX_TILE_BYTES], s_k1[CTX_TILE_BYTES],
        s_k2[CTX_TILE_BYTES], s_k3[CTX_TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char s_v0[CTX_TILE_BYTES], s_v1[CTX_TILE_BYTES],
        s_v2[CTX_TILE_BYTES], s_v3[CTX_TILE_BYTES];
    char* const ks[CTX_STAGES] = {s_k0, s_k1, s_k2, s_k3};
    char* const vs[CTX_STAGES] = {s_v0, s_v1, s_v2, s_v3};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;

    // XCD-aware id: ids congruent mod 8 run on one XCD; the row tiles of one
    // unit (KV head, piece) share u_lo and therefore an XCD.
    const int bid = blockIdx.x;
    const int u_lo = bid % XCDS;
    const int rest = bid / XCDS;
    const int rtile = rest % p.row_tiles;
    const int unit = (rest / p.row_tiles) * XCDS + u_lo;
    if (unit >= p.Hkv * p.n_pieces) return;
    const int kvh = unit / p.n_pieces;
    const int piece = unit % p.n_pieces;

    const int G = p.Hq / p.Hkv;
    const int nrows = p.S * G;
    const int chunk = ((p.Lc + p.n_pieces - 1) / p.n_pieces + CTX_TILE - 1) / CTX_TILE * CTX_TILE;
    const int c0 = min(piece * chunk, p.Lc);
    const int c1 = min(c0 + chunk, p.Lc);

    // This wave's 32 query rows: row rho -> sample rho / G, head kvh*G + rho % G.
    const int rho0 = rtile * CTX_ROWS + wave * 32;
    bf16x8_t qb[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int rho = rho0 + 16 * r + i;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (rho < nrows) {
                const int64_t row = (int64_t)(rho / G) * p.Hq + kvh * G + rho % G;
                v = ld16(static_cast<const uint16_t*>(p.q) + row * MF_D + 32 * s + 8 * g);
            }
            qb[r][s] = as_bf16x8(v);
        }
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(p.k_ctx) + (int64_t)kvh * p.Lc * MF_D;
    const uint16_t* vbase = static_cast<const uint16_t*>(p.v_ctx) + (int64_t)kvh * p.Lc * MF_D;
    const int ktok0 = 8 * (i >> 2) + (i & 3);
    const float sl2 = p.scale_log2;

    f32x4_t acc[2][8], lacc[2];
    float m[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        m[r] = -INFINITY;
        lacc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Ring of CTX_STAGES LDS tiles: tile t lives in stage t % CTX_STAGES and
    // its loads are issued three tiles ahead.  Before tile t is used, each
    // wave waits for its own loads of tile t (the later tiles' loads may
    // stay in flight) and the barrier makes every wave's part visible; the
    // same barrier tells that all waves are done with tile t - 1, whose
    // stage the loads of tile t + 3 then overwrite.
    const int n_tiles = (c1 - c0 + CTX_TILE - 1) / CTX_TILE;
#pragma unroll
    for (int t = 0; t < CTX_STAGES - 1; ++t)
        if (t < n_tiles) issue_tile(kbase, vbase, c0 + t * CTX_TILE, c1, wave, lane, ks[t], vs[t]);
    for (int t4 = 0; t4 < n_tiles; t4 += CTX_STAGES) {
#pragma unroll
        for (int st = 0; st < CTX_STAGES; ++st) {
            const int t = t4 + st;
            if (t < n_tiles) {
                if (t + 2 < n_tiles)
                    wait_vm<8>();
                else if (t + 1 < n_tiles)
                    wait_vm<4>();
                else
                    wait_vm<0>();
                __syncthreads();
                if (t + CTX_STAGES - 1 < n_tiles) {
                    const int nst = (st + CTX_STAGES - 1) % CTX_STAGES;
                    issue_tile(kbase, vbase, c0 + (t + CTX_STAGES - 1) * CTX_TILE, c1, wave, lane, ks[nst], vs[nst]);
                }
                const char* kl = ks[st];
                const char* vl = vs[st];
                u32x4_t kr[2][4], vr[8];
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const int tt = ktok0 + 4 * blk;
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        kr[blk][s] = *reinterpret_cast<const u32x4_t*>(kl + lds_off(tt, 4 * s + g));
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) vr[j] = *reinterpret_cast<const u32x4_t*>(vl + lds_off(8 * g + j, i));
                compute_tile<2>(kr, vr, qb, c0 + t * CTX_TILE, c1, g, sl2, m, lacc, acc);
            }
        }
    }

    // Each wave owns its rows (sums complete in lacc): write this piece.
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const float lr = lacc[r][0];
        const int rho = rho0 + 16 * r + i;
        if (rho < nrows) {
            const int64_t row = (int64_t)(rho / G) * p.Hq + kvh * G + rho % G;
            const int64_t slot = row * p.part_stride + p.part_offset + piece;
            const float inv = (lr > 0.f) ? 1.f / lr : 0.f;
            float* dst = p.o_part + slot * MF_D;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                float4 lo, hi;
                lo.x = acc[r][0][ii] * inv; lo.y = acc[r][1][ii] * inv;
                lo.z = acc[r][2][ii] * inv; lo.w = acc[r][3][ii] * inv;
                hi.x = acc[r][4][ii] * inv; hi.y = acc[r][5][ii] * inv;
                hi.z = acc[r][6][ii] * inv; hi.w = acc[r][7][ii] * inv;
                // d = 8 * (4g + ii) + e for e = 0..7: eight consecutive floats.
                *reinterpret_cast<float4*>(dst + 8 * (4 * g + ii)) = lo;
                *reinterpret_cast<float4*>(dst + 8 * (4 * g + ii) + 4) = hi;
            }
            if (g == 0) p.lse_part[slot] = (lr > 0.f) ? (m[r] + __log2f(lr)) * kLn2f : -INFINITY;
        }
    }
}

}  // namespace

int bif_context_row_tiles(int S, int G) { return (S * G + CTX_ROWS - 1) / CTX_ROWS; }

hipError_t launch_bif_context(const BifContextParams& p, hipStream_t stream) {
    const int units = p.Hkv * p.n_pieces;
    const int64_t wgs = (int64_t)((units + XCDS - 1) / XCDS) * XCDS * p.row_tiles;
    hipLaunchKernelGGL(bif_context_kernel, dim3((unsigned)wgs), dim3(64 * CTX_NW), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fd
