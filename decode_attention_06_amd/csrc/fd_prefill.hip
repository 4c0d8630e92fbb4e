// Causal prefill attention on the matrix cores (gfx950, bf16, head_dim 128).
//
// Method: [FD] "¿Qué es Flash-Decoding y cuándo acelera los LLMs?"
// (slavadubrov.com), section "Por qué la decodificación necesita otra
// planificación": during prefill many query positions run in parallel; [MW]
// (gyaansetu.com, memory-wall article), section on why prompts are fast and
// generation slow: prefill is matrix-matrix work; [FA] "In che modo Flash
// Attention riduce il traffico di memoria durante l'inferenza locale?"
// (shop.zimaspace.com), sections on on-chip working sets of query, key and
// value blocks and on the online softmax.  Position p of a sequence attends
// to cache rows [0, p].
//
// Work unit: (sequence, KV head, tile of 128 / G positions).  Its 128 query
// rows (position, head of the group) are split over four waves of 32; the
// unit streams K/V rows [0, end of its last position] through the LDS ring
// (fd_lds_ring.h), every wave contracting each tile against its own rows.  A
// wave skips the tiles past its last row and masks only the tiles that reach
// its first row's position (the causal diagonal).  Units are dispatched so
// that the position tiles of one (sequence, KV head) pair share an XCD and
// run together where the pair count allows it, longest first (see below).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fd_device.h"
#include "fd_internal.h"
#include "fd_lds_ring.h"
#include "fd_mfma_common.h"

namespace fd {
namespace {

constexpr int PF_NW = 4;
constexpr int PF_ROWS = 32 * PF_NW;

__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillParams p) {
    __shared__ __attribute__((aligned(16))) char lds[CTX_LDS_BYTES];
    char* const ks[CTX_STAGES] = {lds, lds + 2 * CTX_TILE_BYTES, lds + 4 * CTX_TILE_BYTES, lds + 6 * CTX_TILE_BYTES};
    char* const vs[CTX_STAGES] = {lds + CTX_TILE_BYTES, lds + 3 * CTX_TILE_BYTES, lds + 5 * CTX_TILE_BYTES,
                                  lds + 7 * CTX_TILE_BYTES};
    constexpr int TWO_TILES = 2 * 2 * (8 / PF_NW);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;

    // Units in dispatch order.  Ids congruent mod 8 run on one XCD.  With
    // the (sequence, KV head) pairs a multiple of 8, each XCD takes its
    // pairs one after another, every pair's position tiles longest first:
    // the units of one pair then run side by side and read the same KV
    // rows through that XCD's L2.  Otherwise all pairs of one position tile
    // go together, longest first, so every XCD gets the same mix.
    const int units = p.B * p.Hkv * p.n_ptiles;
    const int u = (int)blockIdx.x;
    if (u >= units) return;
    const int nbh = p.B * p.Hkv;
    int ptile, bh;
    if (nbh % XCDS == 0) {
        const int xcd = u % XCDS, idx = u / XCDS;
        ptile = p.n_ptiles - 1 - idx % p.n_ptiles;
        bh = (idx / p.n_ptiles) * XCDS + xcd;
    } else {
        ptile = p.n_ptiles - 1 - u / nbh;
        bh = u % nbh;
    }
    const int kvh = bh % p.Hkv, b = bh / p.Hkv;
    const int G = p.Hq / p.Hkv;
    const int PT = p.pos_per_tile;
    int n = p.lens ? p.lens[b] : (int)p.Lmax;
    n = max(0, min(n, (int)p.Lmax));
    const int p0 = ptile * PT;
    if (p0 >= n) return;                          // the whole workgroup leaves
    const int p_end = min(p0 + PT, n);            // KV rows [0, p_end)

    // This wave's rows: rho -> position p0 + rho / G, head kvh * G + rho % G.
    const int rho0 = wave * 32;
    const int nvalid = min(PT * G, (p_end - p0) * G);   // valid rows of the unit
    bf16x8_t qb[2][4];
    int lim[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int rho = rho0 + 16 * r + i;
        const bool ok = rho < nvalid;
        const int pos = p0 + rho / G;
        lim[r] = ok ? pos + 1 : 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (ok) {
                const int64_t row = ((int64_t)b * p.Hq + kvh * G + rho % G) * p.Lmax + pos;
                v = ld16(static_cast<const uint16_t*>(p.q) + row * MF_D + 32 * s + 8 * g);
            }
            qb[r][s] = as_bf16x8(v);
        }
    }
    // Wave-uniform range: rows start at position w_first and end at w_last.
    const bool wave_rows = rho0 < nvalid;
    const int w_first = p0 + rho0 / G;
    const int w_last = p0 + (min(rho0 + 31, nvalid - 1)) / G;

    const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.Hkv + kvh) * p.Lmax * MF_D;
    const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.Hkv + kvh) * p.Lmax * MF_D;
    const int ktok0 = 8 * (i >> 2) + (i & 3);
    const float sl2 = p.scale_log2;

    f32x4_t acc[2][8], lacc[2];
    RingRows rows;
    ring_rows_init(rows);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        lacc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // The ring as in the bifurcated context part, over rows [0, p_end).
    const int c1 = p_end;
    const int n_tiles = (c1 + CTX_TILE - 1) / CTX_TILE;
    // The query loads complete before the first tiles' (loads return in
    // order): the first wait below covers them too.
    u32x4_t kr[2][4], vt[8];
#pragma unroll
    for (int t = 0; t < CTX_STAGES - 1; ++t) issue_tile<PF_NW>(kbase, vbase, MF_D, t * CTX_TILE, c1, wave, lane, ks[t], vs[t]);
    wait_vm<TWO_TILES>();
    ring_barrier();
    const TileAddrs a0 = ring_step<PF_NW>(kbase, vbase, MF_D, (CTX_STAGES - 1) * CTX_TILE, c1, wave, lane,
                                          ks[CTX_STAGES - 1], vs[CTX_STAGES - 1], ks[0], vs[0], ktok0, g, i, kr, vt);
    keep_addrs<PF_NW>(a0);
    for (int t4 = 0; t4 < n_tiles; t4 += CTX_STAGES) {
#pragma unroll
        for (int st = 0; st < CTX_STAGES; ++st) {
            const int t = t4 + st;
            const int tb = t * CTX_TILE;
            if (wave_rows && tb <= w_last) ring_tile(kr, vt, qb, tb, w_first + 1, lim, g, sl2, rows, lacc, acc);
            if (t + 1 >= n_tiles) break;
            wait_vm<TWO_TILES>();
            ring_barrier();
            const TileAddrs an = ring_step<PF_NW>(kbase, vbase, MF_D, (t + CTX_STAGES) * CTX_TILE, c1, wave, lane, ks[st],
                                                  vs[st], ks[(st + 1) % CTX_STAGES], vs[(st + 1) % CTX_STAGES], ktok0, g,
                                                  i, kr, vt);
            keep_addrs<PF_NW>(an);
        }
    }
    // No load into this workgroup's LDS may outlive it.
    wait_vm<0>();

    // Each wave owns its rows (sums complete in lacc): write the outputs.
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int rho = rho0 + 16 * r + i;
        if (rho < nvalid) {
            const float lr = lacc[r][0];
            const int pos = p0 + rho / G;
            const int64_t row = ((int64_t)b * p.Hq + kvh * G + rho % G) * p.Lmax + pos;
            const float inv = (lr > 0.f) ? 1.f / lr : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)   // d = 16e + 4g + ii
                    store_out(p.out, row * MF_D + 16 * e + 4 * g + ii, acc[r][e][ii] * inv, p.out_bf16);
            if (g == 0 && p.lse_out) p.lse_out[row] = (lr > 0.f) ? (rows.m[r] + __log2f(lr)) * kLn2f : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
    const int G = p.Hq / p.Hkv;
    if (G < 1 || G > PF_ROWS || p.pos_per_tile != PF_ROWS / G) return hipErrorInvalidValue;
    const int64_t units = (int64_t)p.B * p.Hkv * p.n_ptiles;
    if (units >= (1 << 30)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)units), dim3(64 * PF_NW), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fd
