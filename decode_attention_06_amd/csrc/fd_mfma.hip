// Split-KV partial kernel on the MFMA matrix cores (gfx950, bf16, D = 128).
//
// Method: [FD] "¿Qué es Flash-Decoding y cuándo acelera los LLMs?"
// (slavadubrov.com), section "Por qué la decodificación necesita otra
// planificación" (pieces of the history -> partial output + log-sum-exp);
// [FA] "In che modo Flash Attention riduce il traffico di memoria durante
// l'inferenza locale?" (shop.zimaspace.com), sections on tiling and on the
// online softmax.  [BA] "Effiziente Verarbeitung ... bifurkierte
// Aufmerksamkeit ..." (linnk.ai), section "Tilastot": the G query heads of a
// KV head share its K/V rows, so the rows are read once and contracted
// against all G queries: a small dense product, which is what the matrix
// cores are for.
//
// Layout of one wave's 32-token tile (v_mfma_f32_16x16x32_bf16; lane l,
// g = l / 16, i = l % 16):
//  * Scores S^T = K Q^T, tokens on M, query rows on N, d on K.  A-operand
//    lane (g, i) of token block blk, k-step s holds K[token tau][32s + 8g ..
//    +8) with tau = 8*(i/4) + 4*blk + i%4; B-operand holds q[row i][same d].
//    The accumulator then gives lane (g, i) the scores of query row i for
//    tokens 8g .. 8g+7 (blk 0: +0..3, blk 1: +4..7).
//  * Those eight scores, as bf16 weights, are exactly the lane's B operand of
//    O^T += V^T P^T (k-slot 8g + j <-> token 8g + j).
//  * V^T A operand for output block e holds, in lane (g, i),
//    V[token 8g + j][8i + e] for j = 0..7: the lane loads V rows 8g .. 8g+7,
//    columns 8i .. 8i+7 (eight coalesced 16-byte loads) and transposes that
//    8x8 block in registers.  Output row m of block e is d = 8m + e.
//  No LDS is needed inside the token loop; each KV byte is loaded once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "fd_device.h"
#include "fd_internal.h"
#include "fd_mfma_common.h"
#include "fd_mfma_partial.h"

namespace fd {
namespace {

template <int NRB, int NW, bool PAGED, bool KV8, bool PACK>
__global__ __launch_bounds__(64 * NW, (NRB == 1 && NW == 4) ? 2 : 1) void partial_mfma_kernel(const PartialParams p) {
    static_assert(NW * MF_TILE == MFMA_TILE_ROWS, "workgroup step as the host computes it");
    __shared__ PartialLds<NRB, NW> sh;
    partial_mfma_body<NRB, NW, PAGED, KV8, PACK>(p, blockIdx.x, sh);
}

template <bool PAGED, bool KV8>
hipError_t launch_mfma_layout(const PartialParams& p, dim3 grid, int rows, hipStream_t stream) {
    if (rows == 16 && p.Hq / p.Hkv <= 8) {
        hipLaunchKernelGGL((partial_mfma_kernel<1, 4, PAGED, KV8, true>), grid, dim3(256), 0, stream, p);
    } else if (rows == 16) {
        hipLaunchKernelGGL((partial_mfma_kernel<1, 4, PAGED, KV8, false>), grid, dim3(256), 0, stream, p);
    } else {
        hipLaunchKernelGGL((partial_mfma_kernel<2, 4, PAGED, KV8, false>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

int mfma_rows_per_block(int G) { return G > 16 ? 32 : 16; }

hipError_t launch_partial_mfma(const PartialParams& p, bool fp8_cache, hipStream_t stream) {
    const int G = p.Hq / p.Hkv;
    const int rows = mfma_rows_per_block(G);
    if (p.row_blocks != (G + rows - 1) / rows) return hipErrorInvalidValue;
    const int64_t units = (int64_t)p.B * p.Hkv * p.row_blocks;
    if (units * p.n_splits >= (int64_t(1) << 30)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(units * p.n_splits));
    if (fp8_cache)
        return p.block_table ? launch_mfma_layout<true, true>(p, grid, rows, stream)
                             : launch_mfma_layout<false, true>(p, grid, rows, stream);
    return p.block_table ? launch_mfma_layout<true, false>(p, grid, rows, stream)
                         : launch_mfma_layout<false, false>(p, grid, rows, stream);
}

}  // namespace fd
