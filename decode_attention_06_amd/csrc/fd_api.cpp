// Host side of the C ABI declared in include/fd.h: argument validation,
// split planning, workspace sizing and kernel launches.  Every check runs
// before the first HIP call; no entry point allocates device memory or
// synchronises a stream.
#include "fd.h"
#include "fd_testing.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "fd_internal.h"

namespace {

thread_local char g_err[512] = "";

fd_status fail(fd_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

fd_status hip_fail(hipError_t e, const char* what) {
    return fail(FD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int32_t kWgPerCu = 2;        // partial-kernel workgroups to keep per CU
constexpr int64_t kFewMfmaUnits = 8;   // at most this many units: one workgroup per CU
constexpr int64_t kBalanceLen = 8192;  // several sequences at least this long (vector-ALU kernel):
constexpr int64_t kBalancePieces = 4;  //   at least this many pieces each
constexpr int64_t kMinChunk = 256;     // shortest vector-ALU piece where no kernel step applies
constexpr int64_t kMinChunkMfma = 128; // matrix-core kernel: one 32-token tile per wave
constexpr int64_t kMaxLen = int64_t(1) << 30;
constexpr int64_t kMaxUnits = int64_t(1) << 30;   // workgroups or output rows of one launch
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks shared by decode and bifurcated calls.
fd_status check_heads(int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype) {
    if (Hq <= 0 || Hkv <= 0) return fail(FD_ERR_INVALID_ARG, "head counts must be positive (Hq=%d, Hkv=%d)", Hq, Hkv);
    if (Hq % Hkv != 0) return fail(FD_ERR_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (D != 64 && D != 128) return fail(FD_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", D);
    if (dtype != FD_F32 && dtype != FD_BF16 && dtype != FD_FP8_E4M3)
        return fail(FD_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
    return FD_OK;
}

fd_status check_out_dtype(int32_t out_dtype) {
    if (out_dtype != FD_F32 && out_dtype != FD_BF16)
        return fail(FD_ERR_UNSUPPORTED, "out dtype %d not supported", out_dtype);
    return FD_OK;
}

fd_status check_ptr(const void* p, size_t align, const char* name) {
    if (!p) return fail(FD_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, align)) return fail(FD_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
    return FD_OK;
}

#define FD_TRY(expr)                  \
    do {                              \
        fd_status _s = (expr);        \
        if (_s != FD_OK) return _s;   \
    } while (0)

std::mutex g_cu_mutex;
std::vector<int32_t> g_cu_cache;

struct PartialLayout {
    size_t lse_bytes;   // [rows, parts] fp32, padded to kAlign
    size_t o_bytes;     // [rows, parts, D] fp32
    size_t total() const { return lse_bytes + o_bytes; }
};

PartialLayout partial_layout(int64_t rows, int64_t parts, int32_t D) {
    PartialLayout L;
    L.lse_bytes = align_up(size_t(rows * parts) * sizeof(float));
    L.o_bytes = size_t(rows * parts * D) * sizeof(float);
    return L;
}

float resolve_scale(float scale, int32_t D) {
    return scale > 0.f ? scale : 1.0f / std::sqrt(float(D));
}

constexpr float kLog2e = 1.4426950408889634f;

// Smallest GQA group that goes to the matrix-core kernel (bf16, D = 128).
constexpr int kMfmaMinGroup = 4;

// Which partial kernel serves a (dtype, D, G) call, and how many query-row
// blocks each KV head is cut into.  The choice depends on the shapes only;
// `force` (the test entry point fd_testing_decode_attn alone passes it)
// picks a kernel where both support the shape.
struct Path {
    bool mfma;
    int rows_per_block;
    int row_blocks;
};

bool mfma_supported(int32_t dtype, int32_t D) { return (dtype == FD_BF16 || dtype == FD_FP8_E4M3) && D == 128; }

Path choose_path(int32_t dtype, int32_t D, int G, int32_t force = FD_TESTING_KERNEL_AUTO) {
    bool mfma = mfma_supported(dtype, D) && G >= kMfmaMinGroup;
    if (force == FD_TESTING_KERNEL_VALU) mfma = false;
    if (force == FD_TESTING_KERNEL_MFMA) mfma = true;
    Path path;
    path.mfma = mfma;
    path.rows_per_block = mfma ? fd::mfma_rows_per_block(G) : fd::valu_rows_per_block(G, dtype == FD_FP8_E4M3);
    path.row_blocks = (G + path.rows_per_block - 1) / path.rows_per_block;
    return path;
}

hipError_t launch_partial(const fd::PartialParams& p, const Path& path, int32_t dtype, int32_t D,
                          hipStream_t s) {
    return path.mfma ? fd::launch_partial_mfma(p, dtype == FD_FP8_E4M3, s)
                     : fd::launch_partial_valu(p, dtype, D, path.rows_per_block, s);
}

constexpr int64_t kMinContextPiece = 256;   // shortest context piece planned

// Pieces for the context and for the decode part of a bifurcated call.  The
// matrix-core context kernel (bf16, D 128) works on tiles of query rows and
// shares its launch with the decode units (one piece each).  When the
// decode workgroups fit in one of the two workgroup slots per CU, the
// context units take one slot on every CU: a context workgroup alone on a
// CU runs its tiles about 13% faster than two side by side, and the
// HBM-bound decode workgroups share CUs with them.  Otherwise the context
// units take what the decode units leave but at least three quarters of the
// slots: the decode units then stream their rows from HBM beside the
// context units from the start, and the context pieces stay long enough
// that their partials (one per row and piece, written and read back by the
// combine) cost little.  Without the matrix-core context kernel the context
// goes through the split-KV kernel like a batch of S sequences.
struct BifPlan {
    bool mfma_ctx;
    int32_t row_tiles;
    int32_t pc, pd;
};

BifPlan plan_bifurcated(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int64_t Lc, int64_t Ld,
                        int32_t dtype, int32_t n_cu) {
    BifPlan b{};
    b.mfma_ctx = dtype == FD_BF16 && D == 128;
    if (b.mfma_ctx) {
        b.row_tiles = fd::bif_context_row_tiles(S, Hq / Hkv);
        const int64_t units = int64_t(Hkv) * b.row_tiles;
        const int64_t slots = int64_t(n_cu) * kWgPerCu;
        const int64_t dec_units = int64_t(S) * Hkv * ((Hq / Hkv + 15) / 16);
        const int64_t ctx_wgs =
            dec_units <= n_cu ? int64_t(n_cu) : std::max<int64_t>(slots * 3 / 4, slots - dec_units);
        int64_t pc = (ctx_wgs + units - 1) / units;
        pc = std::min<int64_t>(pc, std::max<int64_t>(1, Lc / kMinContextPiece));
        b.pc = int32_t(std::max<int64_t>(1, std::min<int64_t>(pc, FD_MAX_SPLITS)));
        // The decode units run beside the context units in the same launch:
        // one piece each keeps the partials to combine few.
        b.pd = 1;
    } else {
        b.pc = fd_plan_splits(S, Hq, Hkv, D, Lc, dtype, n_cu);
        b.pd = fd_plan_splits(S, Hq, Hkv, D, Ld, dtype, n_cu);
    }
    return b;
}

// Element strides of the query and output tensors [B, Hq, D] (D
// contiguous).  The KV cache's strides travel in PartialParams.
struct IoStrides {
    int64_t q_b, q_h;
    int64_t out_b, out_h;
};

IoStrides dense_io(int32_t Hq, int32_t D) { return {int64_t(Hq) * D, D, int64_t(Hq) * D, D}; }

size_t elem_bytes(int32_t dtype) { return dtype == FD_F32 ? 4 : dtype == FD_BF16 ? 2 : 1; }

// Rows of one KV head are read with 32-bit offsets inside 16- and 32-row
// groups, formed by 24-bit multiplies: a row stride below 2^24 elements and
// 2^27 bytes keeps them exact.
constexpr int64_t kMaxRowStride = (int64_t(1) << 24) - 1;
constexpr int64_t kMaxRowStrideBytes = int64_t(1) << 27;

// One fd_tensor argument: present, ndim dimensions of positive extent, the
// last contiguous, every other stride non-negative and a multiple of 16
// bytes (the kernels read 16-byte vectors), data 16-byte aligned.
fd_status check_tensor(const fd_tensor* t, int32_t ndim, const char* name) {
    if (!t) return fail(FD_ERR_INVALID_ARG, "%s descriptor is NULL", name);
    if (t->ndim != ndim) return fail(FD_ERR_INVALID_ARG, "%s has %d dimensions, %d expected", name, t->ndim, ndim);
    if (t->dtype != FD_F32 && t->dtype != FD_BF16 && t->dtype != FD_FP8_E4M3)
        return fail(FD_ERR_UNSUPPORTED, "%s dtype %d not supported", name, t->dtype);
    FD_TRY(check_ptr(t->data, 16, name));
    const int64_t esz = int64_t(elem_bytes(t->dtype));
    for (int i = 0; i < ndim; ++i)
        if (t->shape[i] <= 0)
            return fail(FD_ERR_INVALID_ARG, "%s shape[%d] = %lld is not positive", name, i, (long long)t->shape[i]);
    if (t->stride[ndim - 1] != 1)
        return fail(FD_ERR_UNSUPPORTED, "%s: the last dimension must be contiguous (stride %lld)", name,
                    (long long)t->stride[ndim - 1]);
    for (int i = 0; i < ndim - 1; ++i) {
        if (t->stride[i] < 0)
            return fail(FD_ERR_UNSUPPORTED, "%s stride[%d] = %lld is negative", name, i, (long long)t->stride[i]);
        if ((t->stride[i] * esz) % 16 != 0)
            return fail(FD_ERR_INVALID_ARG, "%s stride[%d] = %lld elements is not a multiple of 16 bytes", name, i,
                        (long long)t->stride[i]);
    }
    return FD_OK;
}

bool same_layout(const fd_tensor* a, const fd_tensor* b) {
    for (int i = 0; i < a->ndim; ++i)
        if (a->shape[i] != b->shape[i] || a->stride[i] != b->stride[i]) return false;
    return a->ndim == b->ndim && a->dtype == b->dtype;
}

// An output [B, H, D] whose rows do not overlap: the row dimensions,
// ordered by stride, each step past everything the smaller ones span.
bool rows_disjoint(const fd_tensor* o) {
    int64_t s[2] = {o->stride[0], o->stride[1]}, n[2] = {o->shape[0], o->shape[1]};
    if (s[0] > s[1]) {
        std::swap(s[0], s[1]);
        std::swap(n[0], n[1]);
    }
    int64_t span = o->shape[2];
    for (int i = 0; i < 2; ++i) {
        if (n[i] == 1) continue;
        if (s[i] < span) return false;
        span = s[i] * n[i];
    }
    return true;
}

// Row stride of a KV cache (token dimension `dim`) within what the
// kernels' 32-bit row offsets reach.
fd_status check_row_stride(const fd_tensor* t, int dim, const char* name) {
    const int64_t st = t->stride[dim];
    if (st > kMaxRowStride || st * int64_t(elem_bytes(t->dtype)) > kMaxRowStrideBytes)
        return fail(FD_ERR_UNSUPPORTED, "%s row stride %lld is not below 2^24 elements and 2^27 bytes", name,
                    (long long)st);
    return FD_OK;
}

}  // namespace

fd_status fd::set_error(fd_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

extern "C" {

const char* fd_status_string(fd_status s) {
    switch (s) {
        case FD_OK: return "FD_OK";
        case FD_ERR_INVALID_ARG: return "FD_ERR_INVALID_ARG";
        case FD_ERR_UNSUPPORTED: return "FD_ERR_UNSUPPORTED";
        case FD_ERR_WORKSPACE: return "FD_ERR_WORKSPACE";
        case FD_ERR_HIP: return "FD_ERR_HIP";
    }
    return "FD_ERR_UNKNOWN";
}

const char* fd_last_error_message(void) { return g_err; }

int32_t fd_version(void) { return 200; }

int32_t fd_plan_splits(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int64_t max_len, int32_t dtype, int32_t n_cu) {
    if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_len <= 0 ||
        n_cu <= 0 || num_q_heads % num_kv_heads != 0 ||
        (dtype != FD_F32 && dtype != FD_BF16 && dtype != FD_FP8_E4M3))
        return -1;
    const int G = num_q_heads / num_kv_heads;
    const Path path = choose_path(dtype, head_dim, G);
    const int64_t units = int64_t(batch) * num_kv_heads * path.row_blocks;
    // Very few units (long single sequences) on the matrix-core kernel: one
    // workgroup per CU, which halves the pieces to combine and reads as fast.
    const int64_t wg_per_cu = (path.mfma && units <= kFewMfmaUnits) ? 1 : kWgPerCu;
    const int64_t target = int64_t(n_cu) * wg_per_cu;
    // Shortest piece: one workgroup step of the kernel's rows, so every wave
    // of a piece has rows to load (vector-ALU kernel: 64 or 128 rows for the
    // supported shapes).  On MHA at batch 1 with 512 and 2K tokens, pieces of
    // one step measured 5-20% faster than pieces of 256 rows.
    const int64_t valu_step = fd::valu_tile_rows(dtype == FD_F32 ? 4 : dtype == FD_BF16 ? 2 : 1, head_dim,
                                                 path.rows_per_block);
    const int64_t min_piece = path.mfma ? kMinChunkMfma * wg_per_cu : (valu_step > 0 ? valu_step : kMinChunk);
    const int64_t by_len = std::max<int64_t>(1, max_len / min_piece);
    int64_t s = (units >= target) ? 1 : std::min<int64_t>((target + units - 1) / units, by_len);
    // Several sequences with long histories on the vector-ALU kernel: their
    // lengths may differ (they are not known here), and one piece each
    // would leave the longest to finish alone at the end; a few pieces each
    // keep that tail short.
    if (!path.mfma && batch > 1 && max_len >= kBalanceLen)
        s = std::max<int64_t>(s, std::min<int64_t>(kBalancePieces, by_len));
    s = std::min<int64_t>(s, FD_MAX_SPLITS);
    return int32_t(std::max<int64_t>(s, 1));
}

fd_status fd_device_cu_count(int32_t* n_cu) {
    if (!n_cu) return fail(FD_ERR_INVALID_ARG, "n_cu is NULL");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if (dev >= int(g_cu_cache.size())) g_cu_cache.resize(dev + 1, 0);
    if (g_cu_cache[dev] == 0) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
        if (cus <= 0) return fail(FD_ERR_HIP, "device reports %d compute units", cus);
        g_cu_cache[dev] = cus;
    }
    *n_cu = g_cu_cache[dev];
    return FD_OK;
}

static fd_status check_decode_shapes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t Lmax,
                                     int32_t dtype, int32_t n_splits) {
    if (B <= 0) return fail(FD_ERR_INVALID_ARG, "batch must be positive (got %d)", B);
    if (Lmax <= 0 || Lmax > kMaxLen)
        return fail(FD_ERR_INVALID_ARG, "max_len %lld outside [1, 2^30]", (long long)Lmax);
    if (n_splits > FD_MAX_SPLITS)
        return fail(FD_ERR_INVALID_ARG, "n_splits %d above FD_MAX_SPLITS", n_splits);
    return check_heads(Hq, Hkv, D, dtype);
}

static fd_status resolve_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t Lmax,
                                int32_t dtype, int32_t n_splits, int32_t* out) {
    if (n_splits > 0) {
        *out = n_splits;
        return FD_OK;
    }
    int32_t cus = 0;
    FD_TRY(fd_device_cu_count(&cus));
    *out = fd_plan_splits(B, Hq, Hkv, D, Lmax, dtype, cus);
    return FD_OK;
}

// Work units (one workgroup each) and output rows of one decode call must
// stay below 2^30: the kernels index them with 32-bit integers.
static fd_status check_grid(int32_t B, int32_t Hq, int32_t Hkv, int row_blocks, int32_t ns) {
    const int64_t units = int64_t(B) * Hkv * row_blocks * ns;
    if (units >= kMaxUnits)
        return fail(FD_ERR_UNSUPPORTED, "%lld work units (batch %d x %d KV heads x %d row blocks x %d pieces) "
                    "reach the 2^30 limit", (long long)units, B, Hkv, row_blocks, ns);
    if (int64_t(B) * Hq >= kMaxUnits)
        return fail(FD_ERR_UNSUPPORTED, "batch %d x %d query heads reach the 2^30 row limit", B, Hq);
    return FD_OK;
}

fd_status fd_decode_attn_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t Lmax,
                                        int32_t dtype, int32_t n_splits, size_t* bytes) {
    if (!bytes) return fail(FD_ERR_INVALID_ARG, "bytes is NULL");
    FD_TRY(check_decode_shapes(B, Hq, Hkv, D, Lmax, dtype, n_splits));
    int32_t ns = 0;
    FD_TRY(resolve_splits(B, Hq, Hkv, D, Lmax, dtype, n_splits, &ns));
    *bytes = (ns == 1) ? 0 : partial_layout(int64_t(B) * Hq, ns, D).total();
    return FD_OK;
}

// Shared tail of fd_decode_attn and fd_decode_attn_paged: `p` carries the
// cache addressing (dense strides or the page table); this fills in the
// rest, launches the partial kernel and, for several pieces, the combine.
static fd_status run_decode(fd::PartialParams p, const void* q, const int32_t* lens, int32_t B, int32_t Hq,
                            int32_t Hkv, int32_t D, int64_t Lmax, int32_t dtype, int32_t n_splits,
                            void* out, int32_t out_dtype, float* lse_out, float scale, void* workspace,
                            size_t workspace_bytes, void* stream, const IoStrides& io,
                            int32_t force = FD_TESTING_KERNEL_AUTO) {
    FD_TRY(check_out_dtype(out_dtype));
    FD_TRY(check_ptr(q, 16, "q"));
    FD_TRY(check_ptr(out, 16, "out"));
    if (lens && !aligned(lens, 4)) return fail(FD_ERR_INVALID_ARG, "lens is not 4-byte aligned");
    if (lse_out && !aligned(lse_out, 4)) return fail(FD_ERR_INVALID_ARG, "lse_out is not 4-byte aligned");
    if (!std::isfinite(scale)) return fail(FD_ERR_INVALID_ARG, "scale is not finite");

    int32_t ns = 0;
    FD_TRY(resolve_splits(B, Hq, Hkv, D, Lmax, dtype, n_splits, &ns));
    const int64_t rows = int64_t(B) * Hq;
    const PartialLayout L = partial_layout(rows, ns, D);
    if (ns > 1) {
        if (!workspace) return fail(FD_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", L.total());
        if (!aligned(workspace, 16)) return fail(FD_ERR_WORKSPACE, "workspace is not 16-byte aligned");
        if (workspace_bytes < L.total())
            return fail(FD_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total());
    }

    const Path path = choose_path(dtype, D, Hq / Hkv, force);
    FD_TRY(check_grid(B, Hq, Hkv, path.row_blocks, ns));
    p.q = q;
    p.q_stride_b = io.q_b;
    p.q_stride_h = io.q_h;
    p.out_stride_b = io.out_b;
    p.out_stride_h = io.out_h;
    p.lens = lens;
    p.out = out;
    p.lse_out = lse_out;
    p.Lmax = Lmax;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.n_splits = ns;
    p.row_blocks = path.row_blocks;
    p.scale_log2 = resolve_scale(scale, D) * kLog2e;
    p.out_bf16 = out_dtype == FD_BF16;
    p.direct = ns == 1;
    // Several pieces on the matrix-core kernel: interleaved workgroup steps
    // (the combine does not depend on which rows a piece holds).  The
    // vector-ALU kernel streams long contiguous pieces faster.
    p.strided = path.mfma && ns > 1;
    float* lse_part = nullptr;
    float* o_part = nullptr;
    if (ns > 1) {
        lse_part = static_cast<float*>(workspace);
        o_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse_bytes);
        p.o_part = o_part;
        p.lse_part = lse_part;
        p.part_stride = ns;
        p.part_offset = 0;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    FD_TRY(fd::validate_lens(lens, B, 1, Lmax, "lens (each in [1, max_len])", s));
    if (p.block_table)
        FD_TRY(fd::validate_table(p.block_table, lens, B, int32_t(p.bt_stride), 1 << p.page_shift, Lmax, p.n_pages, s));
    hipError_t e = launch_partial(p, path, dtype, D, s);
    if (e != hipSuccess) return hip_fail(e, "split-KV partial kernel launch");
    if (ns > 1) {
        e = fd::launch_lse_combine(o_part, lse_part, int32_t(rows), ns, D, out, fd::OutRows{Hq, io.out_b, io.out_h},
                                   p.out_bf16, lse_out, s);
        if (e != hipSuccess) return hip_fail(e, "lse combine kernel launch");
    }
    return FD_OK;
}

fd_status fd_decode_attn(const void* q, const void* k, const void* v, const int32_t* lens, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t D, int64_t Lmax, int32_t dtype,
                         int32_t n_splits, void* out, int32_t out_dtype, float* lse_out, float scale,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype == FD_FP8_E4M3)
        return fail(FD_ERR_UNSUPPORTED, "an E4M3 cache goes through fd_decode_attn_fp8 (it needs the scales)");
    FD_TRY(check_decode_shapes(B, Hq, Hkv, D, Lmax, dtype, n_splits));
    FD_TRY(check_ptr(k, 16, "k"));
    FD_TRY(check_ptr(v, 16, "v"));
    fd::PartialParams p{};
    p.k = k;
    p.v = v;
    p.kv_stride_t = D;
    p.kv_stride_h = Lmax * D;
    p.kv_stride_b = int64_t(Hkv) * Lmax * D;
    return run_decode(p, q, lens, B, Hq, Hkv, D, Lmax, dtype, n_splits, out, out_dtype, lse_out, scale,
                      workspace, workspace_bytes, stream, dense_io(Hq, D));
}

fd_status fd_decode_attn_fp8(const void* q, const void* k, const void* v, const float* k_scale,
                             const float* v_scale, const int32_t* lens, int32_t B, int32_t Hq, int32_t Hkv,
                             int32_t D, int64_t Lmax, int32_t n_splits, void* out, int32_t out_dtype,
                             float* lse_out, float scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
    FD_TRY(check_decode_shapes(B, Hq, Hkv, D, Lmax, FD_FP8_E4M3, n_splits));
    FD_TRY(check_ptr(k, 16, "k"));
    FD_TRY(check_ptr(v, 16, "v"));
    if (k_scale && !aligned(k_scale, 4)) return fail(FD_ERR_INVALID_ARG, "k_scale is not 4-byte aligned");
    if (v_scale && !aligned(v_scale, 4)) return fail(FD_ERR_INVALID_ARG, "v_scale is not 4-byte aligned");
    fd::PartialParams p{};
    p.k = k;
    p.v = v;
    p.kv_stride_t = D;
    p.kv_stride_h = Lmax * D;
    p.kv_stride_b = int64_t(Hkv) * Lmax * D;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    return run_decode(p, q, lens, B, Hq, Hkv, D, Lmax, FD_FP8_E4M3, n_splits, out, out_dtype, lse_out, scale,
                      workspace, workspace_bytes, stream, dense_io(Hq, D));
}

// Page-pool addressing shared by the paged entry points ([MW] PagedAttention
// paragraph): pool [num_pages, Hkv, page_size, D], table [B, max_pages].
static fd_status paged_addressing(const void* k_pages, const void* v_pages, const int32_t* block_table,
                                  int32_t Hkv, int32_t D, int32_t page_size, int64_t num_pages, int32_t max_pages,
                                  fd::PartialParams* p) {
    if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
        return fail(FD_ERR_UNSUPPORTED, "page_size %d is not a power of two in [16, 2^20]", page_size);
    if (num_pages <= 0 || num_pages > INT32_MAX)
        return fail(FD_ERR_INVALID_ARG, "num_pages %lld outside [1, 2^31 - 1]", (long long)num_pages);
    if (max_pages <= 0) return fail(FD_ERR_INVALID_ARG, "max_pages_per_seq must be positive (got %d)", max_pages);
    FD_TRY(check_ptr(k_pages, 16, "k_pages"));
    FD_TRY(check_ptr(v_pages, 16, "v_pages"));
    FD_TRY(check_ptr(block_table, 4, "block_table"));
    p->k = k_pages;
    p->v = v_pages;
    p->block_table = block_table;
    p->bt_stride = max_pages;
    p->kv_stride_t = D;
    p->kv_stride_h = int64_t(page_size) * D;
    p->page_stride = int64_t(Hkv) * page_size * D;
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    p->page_shift = shift;
    p->n_pages = int32_t(num_pages);
    return FD_OK;
}

fd_status fd_decode_attn_paged(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* lens, int32_t B, int32_t Hq,
                               int32_t Hkv, int32_t D, int32_t page_size, int64_t num_pages,
                               int32_t max_pages, int32_t dtype, int32_t n_splits, void* out,
                               int32_t out_dtype, float* lse_out, float scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (dtype == FD_FP8_E4M3) return fail(FD_ERR_UNSUPPORTED, "paged calls take fp32 or bf16 caches");
    fd::PartialParams p{};
    FD_TRY(paged_addressing(k_pages, v_pages, block_table, Hkv, D, page_size, num_pages, max_pages, &p));
    const int64_t Lmax = int64_t(max_pages) * page_size;
    FD_TRY(check_decode_shapes(B, Hq, Hkv, D, Lmax, dtype, n_splits));
    return run_decode(p, q, lens, B, Hq, Hkv, D, Lmax, dtype, n_splits, out, out_dtype, lse_out, scale,
                      workspace, workspace_bytes, stream, dense_io(Hq, D));
}

int32_t fd_piece_tile_rows(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
        (head_dim != 64 && head_dim != 128) || (dtype != FD_F32 && dtype != FD_BF16 && dtype != FD_FP8_E4M3))
        return -1;
    const Path path = choose_path(dtype, head_dim, num_q_heads / num_kv_heads);
    if (path.mfma) return fd::MFMA_TILE_ROWS;
    const int elem = dtype == FD_F32 ? 4 : dtype == FD_BF16 ? 2 : 1;
    return fd::valu_tile_rows(elem, head_dim, path.rows_per_block);
}

fd_status fd_decode_attn_partials(const void* q, const void* k, const void* v, const int32_t* lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t Lmax,
                                  int32_t dtype, int32_t n_splits, int32_t piece_layout, float* o_part,
                                  float* lse_part, float scale, void* stream) {
    if (dtype == FD_FP8_E4M3) return fail(FD_ERR_UNSUPPORTED, "the partial stage takes fp32 or bf16 caches");
    FD_TRY(check_decode_shapes(B, Hq, Hkv, D, Lmax, dtype, n_splits));
    if (n_splits <= 0) return fail(FD_ERR_INVALID_ARG, "n_splits must be given (> 0) for the partial stage");
    if (piece_layout != FD_PIECES_CONTIGUOUS && piece_layout != FD_PIECES_INTERLEAVED)
        return fail(FD_ERR_INVALID_ARG, "piece_layout %d is neither contiguous (0) nor interleaved (1)", piece_layout);
    FD_TRY(check_ptr(q, 16, "q"));
    FD_TRY(check_ptr(k, 16, "k"));
    FD_TRY(check_ptr(v, 16, "v"));
    FD_TRY(check_ptr(o_part, 16, "o_part"));
    FD_TRY(check_ptr(lse_part, 4, "lse_part"));
    if (lens && !aligned(lens, 4)) return fail(FD_ERR_INVALID_ARG, "lens is not 4-byte aligned");
    if (!std::isfinite(scale)) return fail(FD_ERR_INVALID_ARG, "scale is not finite");

    const Path path = choose_path(dtype, D, Hq / Hkv);
    FD_TRY(check_grid(B, Hq, Hkv, path.row_blocks, n_splits));
    fd::PartialParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.q_stride_b = int64_t(Hq) * D;
    p.q_stride_h = D;
    p.lens = lens;
    p.Lmax = Lmax;
    p.kv_stride_t = D;
    p.kv_stride_h = Lmax * D;
    p.kv_stride_b = int64_t(Hkv) * Lmax * D;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.n_splits = n_splits;
    p.row_blocks = path.row_blocks;
    p.scale_log2 = resolve_scale(scale, D) * kLog2e;
    p.direct = 0;
    p.strided = piece_layout == FD_PIECES_INTERLEAVED;
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.part_stride = n_splits;
    p.part_offset = 0;
    FD_TRY(fd::validate_lens(lens, B, 1, Lmax, "lens (each in [1, max_len])", static_cast<hipStream_t>(stream)));
    hipError_t e = launch_partial(p, path, dtype, D, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "split-KV partial kernel launch");
    return FD_OK;
}

fd_status fd_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    FD_TRY(check_ptr(buf, 16, "buf"));
    FD_TRY(check_ptr(sink, 4, "sink"));
    if (bytes == 0 || bytes % 16 != 0) return fail(FD_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
    hipError_t e = fd::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "read probe kernel launch");
    return FD_OK;
}

static fd_status check_bifurcated_shapes(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int64_t Lc,
                                         int64_t Ld, int32_t dtype) {
    if (S <= 0) return fail(FD_ERR_INVALID_ARG, "samples must be positive (got %d)", S);
    if (Lc <= 0 || Lc > kMaxLen)
        return fail(FD_ERR_INVALID_ARG, "ctx_len %lld outside [1, 2^30]", (long long)Lc);
    if (Ld <= 0 || Ld > kMaxLen)
        return fail(FD_ERR_INVALID_ARG, "dec_max_len %lld outside [1, 2^30]", (long long)Ld);
    if (dtype == FD_FP8_E4M3) return fail(FD_ERR_UNSUPPORTED, "bifurcated calls take fp32 or bf16 inputs");
    return check_heads(Hq, Hkv, D, dtype);
}

fd_status fd_bifurcated_attn_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int64_t Lc,
                                            int64_t Ld, int32_t dtype, size_t* bytes) {
    if (!bytes) return fail(FD_ERR_INVALID_ARG, "bytes is NULL");
    FD_TRY(check_bifurcated_shapes(S, Hq, Hkv, D, Lc, Ld, dtype));
    int32_t cus = 0;
    FD_TRY(fd_device_cu_count(&cus));
    const BifPlan plan = plan_bifurcated(S, Hq, Hkv, D, Lc, Ld, dtype, cus);
    *bytes = partial_layout(int64_t(S) * Hq, plan.pc + plan.pd, D).total();
    return FD_OK;
}

// Shared body of the bifurcated entry points.  `dk` carries the decode
// cache's addressing (k, v and dense strides, or the page pool and table);
// the context is [Hkv, Lc, D] with row stride ctx_t and head stride ctx_h.
static fd_status run_bifurcated(const void* q, const IoStrides& io, const void* k_ctx, const void* v_ctx,
                                int64_t ctx_h, int64_t ctx_t, fd::PartialParams dk, const int32_t* dec_lens,
                                int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int64_t Lc, int64_t Ld,
                                int32_t dtype, void* out, int32_t out_dtype, float* lse_out, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
    FD_TRY(check_bifurcated_shapes(S, Hq, Hkv, D, Lc, Ld, dtype));
    FD_TRY(check_out_dtype(out_dtype));
    FD_TRY(check_ptr(q, 16, "q"));
    FD_TRY(check_ptr(k_ctx, 16, "k_ctx"));
    FD_TRY(check_ptr(v_ctx, 16, "v_ctx"));
    FD_TRY(check_ptr(dk.k, 16, "k_dec"));
    FD_TRY(check_ptr(dk.v, 16, "v_dec"));
    FD_TRY(check_ptr(out, 16, "out"));
    if (dec_lens && !aligned(dec_lens, 4)) return fail(FD_ERR_INVALID_ARG, "dec_lens is not 4-byte aligned");
    if (lse_out && !aligned(lse_out, 4)) return fail(FD_ERR_INVALID_ARG, "lse_out is not 4-byte aligned");
    if (!std::isfinite(scale)) return fail(FD_ERR_INVALID_ARG, "scale is not finite");
    if (!workspace) return fail(FD_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 16)) return fail(FD_ERR_WORKSPACE, "workspace is not 16-byte aligned");

    int32_t cus = 0;
    FD_TRY(fd_device_cu_count(&cus));
    const BifPlan plan = plan_bifurcated(S, Hq, Hkv, D, Lc, Ld, dtype, cus);
    const int32_t pc = plan.pc, pd = plan.pd;
    const int32_t P = pc + pd;
    if (P > FD_MAX_PARTS) return fail(FD_ERR_UNSUPPORTED, "%d pieces exceed the combine limit %d", P, FD_MAX_PARTS);
    const int64_t rows = int64_t(S) * Hq;
    if (rows >= kMaxUnits) return fail(FD_ERR_UNSUPPORTED, "samples %d x %d query heads reach the 2^30 row limit", S, Hq);
    const PartialLayout L = partial_layout(rows, P, D);
    if (workspace_bytes < L.total())
        return fail(FD_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total());
    float* lse_part = static_cast<float*>(workspace);
    float* o_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse_bytes);

    const Path path = choose_path(dtype, D, Hq / Hkv);
    FD_TRY(check_grid(S, Hq, Hkv, path.row_blocks, std::max(pc, pd)));
    hipStream_t s = static_cast<hipStream_t>(stream);

    FD_TRY(fd::validate_lens(dec_lens, S, 0, Ld, "dec_lens (each in [0, dec_max_len])", s));
    if (dk.block_table)
        FD_TRY(fd::validate_table(dk.block_table, dec_lens, S, int32_t(dk.bt_stride), 1 << dk.page_shift, Ld,
                                  dk.n_pages, s));
    fd::PartialParams p = dk;   // decode cache addressing
    p.q = q;
    p.q_stride_b = io.q_b;
    p.q_stride_h = io.q_h;
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.B = S;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.row_blocks = path.row_blocks;
    p.part_stride = P;
    p.scale_log2 = resolve_scale(scale, D) * kLog2e;
    p.direct = 0;
    hipError_t e;
    if (plan.mfma_ctx) {
        // One launch: the context part on the matrix cores (every KV head's
        // context rows read once per tile of query rows = samples x heads of
        // the group) and, beside it, each sample's decode rows through the
        // split-KV unit with 16-row blocks.
        fd::BifContextParams c{};
        c.q = q;
        c.q_stride_b = io.q_b;
        c.q_stride_h = io.q_h;
        c.k_ctx = k_ctx;
        c.v_ctx = v_ctx;
        c.ctx_stride_h = ctx_h;
        c.ctx_stride_t = ctx_t;
        c.o_part = o_part;
        c.lse_part = lse_part;
        c.S = S;
        c.Hq = Hq;
        c.Hkv = Hkv;
        c.Lc = int32_t(Lc);
        c.n_pieces = pc;
        c.row_tiles = plan.row_tiles;
        c.part_stride = P;
        c.part_offset = 0;
        c.scale_log2 = p.scale_log2;
        p.lens = dec_lens;
        p.Lmax = Ld;
        p.n_splits = pd;
        p.part_offset = pc;
        p.row_blocks = (Hq / Hkv + 15) / 16;
        e = fd::launch_bifurcated(c, p, s);
        if (e != hipSuccess) return hip_fail(e, "bifurcated kernel launch");
    } else {
        // Context part through the split-KV kernel: every sample reads the
        // same [Hkv, Lc, D] rows (batch stride 0); all Lc rows are valid.
        fd::PartialParams pcx = p;
        pcx.k = k_ctx;
        pcx.v = v_ctx;
        pcx.block_table = nullptr;
        pcx.lens = nullptr;
        pcx.Lmax = Lc;
        pcx.kv_stride_b = 0;
        pcx.kv_stride_h = ctx_h;
        pcx.kv_stride_t = ctx_t;
        pcx.n_splits = pc;
        pcx.part_offset = 0;
        e = launch_partial(pcx, path, dtype, D, s);
        if (e != hipSuccess) return hip_fail(e, "bifurcated context kernel launch");
        // Decode part: each sample's own rows, dec_lens[s] of them (0 allowed).
        p.lens = dec_lens;
        p.Lmax = Ld;
        p.n_splits = pd;
        p.part_offset = pc;
        e = launch_partial(p, path, dtype, D, s);
        if (e != hipSuccess) return hip_fail(e, "bifurcated decode kernel launch");
    }

    e = fd::launch_lse_combine(o_part, lse_part, int32_t(rows), P, D, out, fd::OutRows{Hq, io.out_b, io.out_h},
                               out_dtype == FD_BF16, lse_out, s);
    if (e != hipSuccess) return hip_fail(e, "bifurcated combine kernel launch");
    return FD_OK;
}

fd_status fd_bifurcated_attn(const void* q, const void* k_ctx, const void* v_ctx, const void* k_dec,
                             const void* v_dec, const int32_t* dec_lens, int32_t S, int32_t Hq,
                             int32_t Hkv, int32_t D, int64_t Lc, int64_t Ld, int32_t dtype, void* out,
                             int32_t out_dtype, float* lse_out, float scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
    fd::PartialParams dk{};
    dk.k = k_dec;
    dk.v = v_dec;
    dk.kv_stride_t = D;
    dk.kv_stride_h = Ld * D;
    dk.kv_stride_b = int64_t(Hkv) * Ld * D;
    return run_bifurcated(q, dense_io(Hq, D), k_ctx, v_ctx, Lc * D, D, dk, dec_lens, S, Hq, Hkv, D, Lc, Ld, dtype,
                          out, out_dtype, lse_out, scale, workspace, workspace_bytes, stream);
}

fd_status fd_bifurcated_attn_paged(const void* q, const void* k_ctx, const void* v_ctx, const void* k_pages,
                                   const void* v_pages, const int32_t* block_table, const int32_t* dec_lens,
                                   int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int64_t Lc, int32_t page_size,
                                   int64_t num_pages, int32_t max_pages_per_seq, int32_t dtype, void* out,
                                   int32_t out_dtype, float* lse_out, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    fd::PartialParams dk{};
    FD_TRY(paged_addressing(k_pages, v_pages, block_table, Hkv, D, page_size, num_pages, max_pages_per_seq, &dk));
    const int64_t Ld = int64_t(max_pages_per_seq) * page_size;
    return run_bifurcated(q, dense_io(Hq, D), k_ctx, v_ctx, Lc * D, D, dk, dec_lens, S, Hq, Hkv, D, Lc, Ld, dtype,
                          out, out_dtype, lse_out, scale, workspace, workspace_bytes, stream);
}

fd_status fd_prefill_attn(const void* q, const void* k, const void* v, const int32_t* lens, int32_t B,
                          int32_t Hq, int32_t Hkv, int32_t D, int64_t Lmax, int32_t dtype, void* out,
                          int32_t out_dtype, float* lse_out, float scale, void* stream) {
    FD_TRY(check_decode_shapes(B, Hq, Hkv, D, Lmax, dtype, 0));
    if (dtype != FD_BF16 || D != 128)
        return fail(FD_ERR_UNSUPPORTED, "prefill supports bf16 with head_dim 128 (got dtype %d, D %d)", dtype, D);
    if (Hq / Hkv > 128) return fail(FD_ERR_UNSUPPORTED, "prefill supports up to 128 query heads per KV head");
    FD_TRY(check_out_dtype(out_dtype));
    FD_TRY(check_ptr(q, 16, "q"));
    FD_TRY(check_ptr(k, 16, "k"));
    FD_TRY(check_ptr(v, 16, "v"));
    FD_TRY(check_ptr(out, out_dtype == FD_BF16 ? 2 : 4, "out"));
    if (lens && !aligned(lens, 4)) return fail(FD_ERR_INVALID_ARG, "lens is not 4-byte aligned");
    if (lse_out && !aligned(lse_out, 4)) return fail(FD_ERR_INVALID_ARG, "lse_out is not 4-byte aligned");
    if (!std::isfinite(scale)) return fail(FD_ERR_INVALID_ARG, "scale is not finite");
    fd::PrefillParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.lens = lens;
    p.out = out;
    p.lse_out = lse_out;
    p.Lmax = Lmax;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.pos_per_tile = 128 / (Hq / Hkv);
    p.n_ptiles = int32_t((Lmax + p.pos_per_tile - 1) / p.pos_per_tile);
    p.scale_log2 = resolve_scale(scale, D) * kLog2e;
    p.out_bf16 = out_dtype == FD_BF16;
    if (int64_t(B) * Hkv * p.n_ptiles >= (int64_t(1) << 30))
        return fail(FD_ERR_UNSUPPORTED, "too many prefill work units");
    FD_TRY(fd::validate_lens(lens, B, 1, Lmax, "lens (each in [1, max_len])", static_cast<hipStream_t>(stream)));
    hipError_t e = fd::launch_prefill(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
    return FD_OK;
}

fd_status fd_lse_combine(const float* o_part, const float* lse_part, int32_t rows, int32_t n_parts,
                         int32_t D, void* out, int32_t out_dtype, float* lse_out, void* stream) {
    if (rows <= 0 || n_parts <= 0) return fail(FD_ERR_INVALID_ARG, "rows and n_parts must be positive");
    if (D <= 0 || D > 512) return fail(FD_ERR_UNSUPPORTED, "head_dim %d outside [1, 512]", D);
    if (n_parts > FD_MAX_PARTS) return fail(FD_ERR_UNSUPPORTED, "n_parts %d above %d", n_parts, FD_MAX_PARTS);
    FD_TRY(check_out_dtype(out_dtype));
    FD_TRY(check_ptr(o_part, 4, "o_part"));
    FD_TRY(check_ptr(lse_part, 4, "lse_part"));
    FD_TRY(check_ptr(out, out_dtype == FD_BF16 ? 2 : 4, "out"));
    if (lse_out && !aligned(lse_out, 4)) return fail(FD_ERR_INVALID_ARG, "lse_out is not 4-byte aligned");
    hipError_t e = fd::launch_lse_combine(o_part, lse_part, rows, n_parts, D, out, fd::OutRows{1, D, 0},
                                          out_dtype == FD_BF16,
                                          lse_out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "lse combine kernel launch");
    return FD_OK;
}

fd_status fd_testing_decode_attn(const void* q, const void* k, const void* v, const float* k_scale,
                                 const float* v_scale, const int32_t* lens, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t D, int64_t Lmax, int32_t dtype, int32_t n_splits, void* out,
                                 int32_t out_dtype, float* lse_out, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream, int32_t partial_kernel) {
    if (partial_kernel != FD_TESTING_KERNEL_AUTO && partial_kernel != FD_TESTING_KERNEL_VALU &&
        partial_kernel != FD_TESTING_KERNEL_MFMA)
        return fail(FD_ERR_INVALID_ARG, "partial_kernel %d is not 0, 1 or 2", partial_kernel);
    FD_TRY(check_decode_shapes(B, Hq, Hkv, D, Lmax, dtype, n_splits));
    if (partial_kernel == FD_TESTING_KERNEL_MFMA && !mfma_supported(dtype, D))
        return fail(FD_ERR_UNSUPPORTED, "the matrix-core kernel takes bf16 or E4M3 caches with head_dim 128");
    FD_TRY(check_ptr(k, 16, "k"));
    FD_TRY(check_ptr(v, 16, "v"));
    if (k_scale && !aligned(k_scale, 4)) return fail(FD_ERR_INVALID_ARG, "k_scale is not 4-byte aligned");
    if (v_scale && !aligned(v_scale, 4)) return fail(FD_ERR_INVALID_ARG, "v_scale is not 4-byte aligned");
    fd::PartialParams p{};
    p.k = k;
    p.v = v;
    p.kv_stride_t = D;
    p.kv_stride_h = Lmax * D;
    p.kv_stride_b = int64_t(Hkv) * Lmax * D;
    if (dtype == FD_FP8_E4M3) {
        p.k_scale = k_scale;
        p.v_scale = v_scale;
    }
    return run_decode(p, q, lens, B, Hq, Hkv, D, Lmax, dtype, n_splits, out, out_dtype, lse_out, scale,
                      workspace, workspace_bytes, stream, dense_io(Hq, D), partial_kernel);
}

fd_status fd_decode_attn_strided(const fd_tensor* q, const fd_tensor* k, const fd_tensor* v, const float* k_scale,
                                 const float* v_scale, const int32_t* lens, int32_t n_splits, const fd_tensor* out,
                                 float* lse_out, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    FD_TRY(check_tensor(q, 3, "q"));
    FD_TRY(check_tensor(k, 4, "k"));
    FD_TRY(check_tensor(v, 4, "v"));
    FD_TRY(check_tensor(out, 3, "out"));
    const int64_t B = q->shape[0], Hq = q->shape[1], D = q->shape[2];
    const int64_t Hkv = k->shape[1], Lmax = k->shape[2];
    if (k->shape[0] != B || k->shape[3] != D)
        return fail(FD_ERR_INVALID_ARG, "k [%lld, %lld, %lld, %lld] does not match q [%lld, %lld, %lld]",
                    (long long)k->shape[0], (long long)Hkv, (long long)Lmax, (long long)k->shape[3], (long long)B,
                    (long long)Hq, (long long)D);
    if (!same_layout(k, v)) return fail(FD_ERR_UNSUPPORTED, "k and v must share shape, strides and dtype");
    if (out->shape[0] != B || out->shape[1] != Hq || out->shape[2] != D)
        return fail(FD_ERR_INVALID_ARG, "out must be [B, Hq, D] like q");
    if (!rows_disjoint(out)) return fail(FD_ERR_INVALID_ARG, "out strides make output rows overlap");
    if (B > INT32_MAX || Hq > INT32_MAX || Hkv > INT32_MAX || D > INT32_MAX)
        return fail(FD_ERR_INVALID_ARG, "dimension beyond int32");
    const int32_t dtype = k->dtype;
    if (dtype == FD_FP8_E4M3 ? q->dtype != FD_BF16 : q->dtype != dtype)
        return fail(FD_ERR_UNSUPPORTED, "q dtype %d with a cache of dtype %d (same dtype, or bf16 q for E4M3)",
                    q->dtype, dtype);
    FD_TRY(check_decode_shapes(int32_t(B), int32_t(Hq), int32_t(Hkv), int32_t(D), Lmax, dtype, n_splits));
    FD_TRY(check_row_stride(k, 2, "k"));
    if (k_scale && !aligned(k_scale, 4)) return fail(FD_ERR_INVALID_ARG, "k_scale is not 4-byte aligned");
    if (v_scale && !aligned(v_scale, 4)) return fail(FD_ERR_INVALID_ARG, "v_scale is not 4-byte aligned");
    fd::PartialParams p{};
    p.k = k->data;
    p.v = v->data;
    p.kv_stride_b = k->stride[0];
    p.kv_stride_h = k->stride[1];
    p.kv_stride_t = k->stride[2];
    if (dtype == FD_FP8_E4M3) {
        p.k_scale = k_scale;
        p.v_scale = v_scale;
    }
    const IoStrides io{q->stride[0], q->stride[1], out->stride[0], out->stride[1]};
    return run_decode(p, q->data, lens, int32_t(B), int32_t(Hq), int32_t(Hkv), int32_t(D), Lmax, dtype, n_splits,
                      out->data, out->dtype, lse_out, scale, workspace, workspace_bytes, stream, io);
}

fd_status fd_bifurcated_attn_strided(const fd_tensor* q, const fd_tensor* k_ctx, const fd_tensor* v_ctx,
                                     const fd_tensor* k_dec, const fd_tensor* v_dec, const int32_t* dec_lens,
                                     const fd_tensor* out, float* lse_out, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    FD_TRY(check_tensor(q, 3, "q"));
    FD_TRY(check_tensor(k_ctx, 3, "k_ctx"));
    FD_TRY(check_tensor(v_ctx, 3, "v_ctx"));
    FD_TRY(check_tensor(k_dec, 4, "k_dec"));
    FD_TRY(check_tensor(v_dec, 4, "v_dec"));
    FD_TRY(check_tensor(out, 3, "out"));
    const int64_t S = q->shape[0], Hq = q->shape[1], D = q->shape[2];
    const int64_t Hkv = k_ctx->shape[0], Lc = k_ctx->shape[1], Ld = k_dec->shape[2];
    if (k_ctx->shape[2] != D || k_dec->shape[0] != S || k_dec->shape[1] != Hkv || k_dec->shape[3] != D)
        return fail(FD_ERR_INVALID_ARG, "k_ctx [Hkv, Lc, D] and k_dec [S, Hkv, Ldmax, D] do not match q [S, Hq, D]");
    if (!same_layout(k_ctx, v_ctx) || !same_layout(k_dec, v_dec))
        return fail(FD_ERR_UNSUPPORTED, "k and v of the context (and of the decode part) must share shape, strides "
                    "and dtype");
    if (out->shape[0] != S || out->shape[1] != Hq || out->shape[2] != D)
        return fail(FD_ERR_INVALID_ARG, "out must be [S, Hq, D] like q");
    if (!rows_disjoint(out)) return fail(FD_ERR_INVALID_ARG, "out strides make output rows overlap");
    if (S > INT32_MAX || Hq > INT32_MAX || Hkv > INT32_MAX || D > INT32_MAX)
        return fail(FD_ERR_INVALID_ARG, "dimension beyond int32");
    const int32_t dtype = q->dtype;
    if (k_ctx->dtype != dtype || k_dec->dtype != dtype)
        return fail(FD_ERR_UNSUPPORTED, "q, context and decode caches must share one dtype");
    FD_TRY(check_row_stride(k_ctx, 1, "k_ctx"));
    FD_TRY(check_row_stride(k_dec, 2, "k_dec"));
    fd::PartialParams dk{};
    dk.k = k_dec->data;
    dk.v = v_dec->data;
    dk.kv_stride_b = k_dec->stride[0];
    dk.kv_stride_h = k_dec->stride[1];
    dk.kv_stride_t = k_dec->stride[2];
    const IoStrides io{q->stride[0], q->stride[1], out->stride[0], out->stride[1]};
    return run_bifurcated(q->data, io, k_ctx->data, v_ctx->data, k_ctx->stride[0], k_ctx->stride[1], dk, dec_lens,
                          int32_t(S), int32_t(Hq), int32_t(Hkv), int32_t(D), Lc, Ld, dtype, out->data, out->dtype,
                          lse_out, scale, workspace, workspace_bytes, stream);
}

}  // extern "C"
