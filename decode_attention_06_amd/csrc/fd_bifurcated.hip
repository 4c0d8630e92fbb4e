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
// S * G of them.  A workgroup stages 64-token K/V tiles in LDS (double
// buffered, XOR-swizzled 16-byte chunks) and every wave contracts them
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
constexpr int CTX_TILE = 64;              // tokens per LDS tile
constexpr int XCDS = 8;

// LDS byte offset of 16-byte chunk c (0..15) of token row t in a tile.  The
// chunk index is XORed with (t & 3) | (bit 3 of t) << 2, which makes the
// K-operand reads (8 lanes: tokens {0..3, 8..11} + const, same chunk), the
// V-block reads (8 lanes: one token, chunks 0..7) and the tile writes
// (8 threads: one token, 8 consecutive chunks) hit 8 distinct bank groups.
__device__ __forceinline__ int lds_off(int t, int c) {
    const int f = (t & 3) | (((t >> 3) & 1) << 2);
    return t * 256 + ((c ^ f) << 4);
}

struct TileStage {
    u32x4_t k[4], v[4];
};

// Global -> registers for one 64-token tile: thread th covers rows
// th / 16 + 16u, chunk th % 16.  Rows at or beyond c1 clamp to c1 - 1.
__device__ __forceinline__ void fetch_tile(const uint16_t* kbase, const uint16_t* vbase, int t0, int c1, int th,
                                           TileStage& st) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int t = min(t0 + th / 16 + 16 * u, c1 - 1);
        st.k[u] = ld16(kbase + (int64_t)t * MF_D + 8 * (th % 16));
        st.v[u] = ld16(vbase + (int64_t)t * MF_D + 8 * (th % 16));
    }
}

__device__ __forceinline__ void store_tile(char* kl, char* vl, int th, const TileStage& st) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int off = lds_off(th / 16 + 16 * u, th % 16);
        *reinterpret_cast<u32x4_t*>(kl + off) = st.k[u];
        *reinterpret_cast<u32x4_t*>(vl + off) = st.v[u];
    }
}

__global__ __launch_bounds__(64 * CTX_NW, 2) void bif_context_kernel(const BifContextParams p) {
    __shared__ __attribute__((aligned(16))) char s_k[2][CTX_TILE * 256];
    __shared__ __attribute__((aligned(16))) char s_v[2][CTX_TILE * 256];

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

    if (c0 < c1) {
        TileStage st;
        fetch_tile(kbase, vbase, c0, c1, tid, st);
        store_tile(s_k[0], s_v[0], tid, st);
        __syncthreads();
        int buf = 0;
        for (int t0 = c0; t0 < c1; t0 += CTX_TILE) {
            const bool more = t0 + CTX_TILE < c1;
            if (more) fetch_tile(kbase, vbase, t0 + CTX_TILE, c1, tid, st);
            const char* kl = s_k[buf];
            const char* vl = s_v[buf];
#pragma unroll
            for (int sub = 0; sub < CTX_TILE / MF_TILE; ++sub) {
                u32x4_t kr[2][4], vr[8];
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const int t = sub * MF_TILE + ktok0 + 4 * blk;
#pragma unroll
                    for (int s = 0; s < 4; ++s) kr[blk][s] = *reinterpret_cast<const u32x4_t*>(kl + lds_off(t, 4 * s + g));
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    vr[j] = *reinterpret_cast<const u32x4_t*>(vl + lds_off(sub * MF_TILE + 8 * g + j, i));
                compute_tile<2>(kr, vr, qb, t0 + sub * MF_TILE, c1, g, sl2, m, lacc, acc);
            }
            if (more) store_tile(s_k[buf ^ 1], s_v[buf ^ 1], tid, st);
            __syncthreads();
            buf ^= 1;
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
