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
// Work unit: (KV head, context piece, tile of 128 query rows over four
// waves).  The query rows of a KV head are the (sample, head-in-group)
// pairs that read it, S * G of them.  A workgroup streams 32-token K/V
// tiles straight from global memory into a ring of LDS stages (16-byte
// chunks permuted against bank conflicts, three tiles in flight) and every
// wave contracts them
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
#include "fd_lds_ring.h"
#include "fd_mfma_partial.h"

namespace fd {
namespace {

// Context role: one work unit (KV head, piece, row tile) given by bid.
template <int NW>
__device__ __forceinline__ void context_body(const BifContextParams& p, int bid, char* lds) {
    constexpr int CTX_ROWS = 32 * NW;
    // Loads outstanding per wave for two tiles.
    constexpr int TWO_TILES = 2 * 2 * (8 / NW);
    // Stage st holds the K tile at lds + 2 st TILE and the V tile after it;
    // stages are addressed with constant numbers only.
    char* const ks[CTX_STAGES] = {lds, lds + 2 * CTX_TILE_BYTES, lds + 4 * CTX_TILE_BYTES, lds + 6 * CTX_TILE_BYTES};
    char* const vs[CTX_STAGES] = {lds + CTX_TILE_BYTES, lds + 3 * CTX_TILE_BYTES, lds + 5 * CTX_TILE_BYTES,
                                  lds + 7 * CTX_TILE_BYTES};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;

    // XCD-aware id: ids congruent mod 8 run on one XCD; the row tiles of one
    // unit (KV head, piece) share u_lo and therefore an XCD.
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
            if (rho < nrows)
                v = ld16(static_cast<const uint16_t*>(p.q) + (int64_t)(rho / G) * p.q_stride_b +
                         (int64_t)(kvh * G + rho % G) * p.q_stride_h + 32 * s + 8 * g);
            qb[r][s] = as_bf16x8(v);
        }
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(p.k_ctx) + (int64_t)kvh * p.ctx_stride_h;
    const uint16_t* vbase = static_cast<const uint16_t*>(p.v_ctx) + (int64_t)kvh * p.ctx_stride_h;
    const int rs = (int)p.ctx_stride_t;   // elements from one context row to the next
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

    // Ring of CTX_STAGES LDS tiles: tile t lives in stage t % CTX_STAGES.
    // Every step issues exactly four loads per wave (tiles past the end
    // re-read the piece's last row into a stage nobody reads again), so
    // the wait for all but two tiles' loads before reading tile t + 1 leaves it complete on every path
    // (tiles t + 2 and t + 3 may stay in flight); the barrier after it makes
    // all waves' parts visible and tells that all waves are done with tile
    // t, whose stage the loads of tile t + 4 then refill.  The LDS reads of
    // the next tile sit at the end of each step, after that step's issue, so
    // the compiler sees which stages are still being filled.
    if (c0 < c1) {
        const int n_tiles = (c1 - c0 + CTX_TILE - 1) / CTX_TILE;
        const int lim[2] = {c1, c1};
        // The query loads were issued before the first tiles' and complete
        // before them (loads return in order), so the first wait below also
        // covers them; their latency overlaps the tiles'.
        u32x4_t kr[2][4], vt[8];
#pragma unroll
        for (int t = 0; t < CTX_STAGES - 1; ++t)
            issue_tile<NW>(kbase, vbase, rs, c0 + t * CTX_TILE, c1, wave, lane, ks[t], vs[t]);
        wait_vm<TWO_TILES>();
        ring_barrier();
        const TileAddrs a0 = ring_step<NW>(kbase, vbase, rs, c0 + (CTX_STAGES - 1) * CTX_TILE, c1, wave, lane,
                                       ks[CTX_STAGES - 1], vs[CTX_STAGES - 1], ks[0], vs[0], ktok0, g, i, kr, vt);
        keep_addrs<NW>(a0);
        for (int t4 = 0; t4 < n_tiles; t4 += CTX_STAGES) {
#pragma unroll
            for (int st = 0; st < CTX_STAGES; ++st) {
                const int t = t4 + st;
                ring_tile(kr, vt, qb, c0 + t * CTX_TILE, c1, lim, g, sl2, rows, lacc, acc);
                if (t + 1 >= n_tiles) break;
                wait_vm<TWO_TILES>();
                ring_barrier();
                const TileAddrs an = ring_step<NW>(kbase, vbase, rs, c0 + (t + CTX_STAGES) * CTX_TILE, c1, wave, lane,
                                               ks[st], vs[st], ks[(st + 1) % CTX_STAGES], vs[(st + 1) % CTX_STAGES],
                                               ktok0, g, i, kr, vt);
                keep_addrs<NW>(an);
            }
        }
        // No load into this workgroup's LDS may outlive it.
        wait_vm<0>();
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
            for (int e = 0; e < 8; ++e) {
                // d = 16e + 4g + ii for ii = 0..3: four consecutive floats.
                float4 o;
                o.x = acc[r][e][0] * inv; o.y = acc[r][e][1] * inv;
                o.z = acc[r][e][2] * inv; o.w = acc[r][e][3] * inv;
                *reinterpret_cast<float4*>(dst + 16 * e + 4 * g) = o;
            }
            if (g == 0) p.lse_part[slot] = (lr > 0.f) ? (rows.m[r] + __log2f(lr)) * kLn2f : -INFINITY;
        }
    }
}

// The bifurcated call as one launch with two workgroup roles: context
// units (above) and the decode part's split-KV units (16-row matrix-core
// blocks, one piece per unit; dense or paged decode cache).  Workgroup ids
// come in blocks of eight (consecutive ids go to the eight XCDs in turn).
// The context blocks come first, the decode blocks after them: with at most
// one context workgroup per CU planned, every decode workgroup that fits
// starts at once beside one, streaming its own KV from HBM while the context
// part keeps the matrix cores busy; with more, the long context units all
// start first and the short decode units fill the CUs after them.  A
// context unit's row tiles share one XCD, and so do the row blocks of one
// decode unit (sample, KV head), which also start together: the second
// reads the decode rows the first brings into that XCD's L2 instead of
// fetching them again.
template <bool PAGED, bool PACK, bool KEEP>
__global__ __launch_bounds__(256, 2) void bifurcated_kernel(const BifContextParams c, const PartialParams d,
                                                            int n_ctx, int n_dec) {
    __shared__ __attribute__((aligned(16))) char lds[CTX_LDS_BYTES];
    static_assert(sizeof(PartialLds<1, 4>) <= CTX_LDS_BYTES, "decode role LDS");
    const int blk = blockIdx.x / XCDS, lane8 = blockIdx.x % XCDS;
    const int nb_ctx = (n_ctx + XCDS - 1) / XCDS;
    if (blk < nb_ctx) {
        const int cid = blk * XCDS + lane8;
        if (cid < n_ctx) context_body<4>(c, cid, lds);
    } else {
        // Decode id -> (unit, row block): ids congruent mod 8 share an XCD;
        // the row blocks of a unit take consecutive ids of one residue.
        const int did = (blk - nb_ctx) * XCDS + lane8;
        const int rb = d.row_blocks;
        const int q = did / XCDS;
        const int unit = (q / rb) * XCDS + did % XCDS;
        if (did < n_dec && unit < d.B * d.Hkv)
            partial_mfma_body<1, 4, PAGED, false, PACK, KEEP>(d, unit * rb + q % rb,
                                                       *reinterpret_cast<PartialLds<1, 4>*>(lds));
    }
}

}  // namespace

int bif_context_row_tiles(int S, int G) {
    constexpr int rows = 32 * 4;   // four waves of 32 rows
    return (S * G + rows - 1) / rows;
}

hipError_t launch_bifurcated(const BifContextParams& c, const PartialParams& d, hipStream_t stream) {
    // The decode role takes one piece per (sample, KV head); its ids are
    // padded to whole groups of eight units.
    if (d.n_splits != 1) return hipErrorInvalidValue;
    const int units = c.Hkv * c.n_pieces;
    const int64_t n_ctx = (int64_t)((units + XCDS - 1) / XCDS) * XCDS * c.row_tiles;
    const int64_t dec_units = (int64_t)d.B * d.Hkv;
    const int64_t n_dec = (dec_units + XCDS - 1) / XCDS * XCDS * d.row_blocks;
    const int64_t wgs = ((n_ctx + XCDS - 1) / XCDS + (n_dec + XCDS - 1) / XCDS) * XCDS;
    if (n_ctx >= (1 << 30) || n_dec >= (1 << 30)) return hipErrorInvalidValue;
    // Groups of at most 8 query heads on a dense decode cache: the decode
    // role packs its weight remainders into the 16-row block's padding
    // columns (the paged form keeps two products per block: packing there
    // needs more registers than two workgroups per CU leave).
    // With more than one row block per unit (groups above 16 heads), the
    // blocks after the first read the unit's decode rows from L2, so those
    // loads keep the default cache policy (read-once loads left the MQA
    // workload fetching its decode rows twice).
    const bool pack = d.Hq / d.Hkv <= 8 && !d.block_table;
    const bool keep = d.row_blocks > 1;
#define FD_BIF(PG, PK, KP) hipLaunchKernelGGL((bifurcated_kernel<PG, PK, KP>), dim3((unsigned)wgs), dim3(256), 0, stream, \
                                              c, d, (int)n_ctx, (int)n_dec)
    if (d.block_table) {
        if (keep) FD_BIF(true, false, true);
        else FD_BIF(true, false, false);
    } else if (pack) {
        FD_BIF(false, true, false);
    } else {
        if (keep) FD_BIF(false, false, true);
        else FD_BIF(false, false, false);
    }
#undef FD_BIF
    return hipGetLastError();
}

}  // namespace fd
