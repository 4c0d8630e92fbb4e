/*
 * fd.h - C ABI of the MI355X (gfx950) decode-attention library.
 *
 * Exact single-query (decode-step) attention over a long KV cache, built as
 * split-KV partials plus a log-sum-exp combine, and a bifurcated variant
 * for many samples that share one context.
 *
 * Sources (pages cited by title and section):
 *  [FD] "¿Qué es Flash-Decoding y cuándo acelera los LLMs?" (slavadubrov.com),
 *       section "Por qué la decodificación necesita otra planificación":
 *       decode attention is parallelised along the cached sequence; every
 *       piece produces a partial output and a log-sum-exp; a reduction
 *       renormalises them into the full-history result.
 *  [FA] "In che modo Flash Attention riduce il traffico di memoria durante
 *       l'inferenza locale?" (shop.zimaspace.com), sections on tiling, on
 *       the online softmax and on kernel fusion; and "Il supporto hardware e
 *       la forma dei dati determinano l'uso del percorso rapido": fast paths
 *       are specialised by head size, dtype and shape.
 *  [BA] "Effiziente Verarbeitung und Analyse von Inhalten durch bifurkierte
 *       Aufmerksamkeit für Single-Context-Batch-Sampling" (linnk.ai),
 *       sections "Tiivistelmä" and "Tilastot": attention over a shared
 *       context KV plus per-sample decode KV, exact, with the context KV
 *       read once; GQA/MQA heads share KV heads.
 *  [MW] gyaansetu.com article on the memory wall of LLM decoding (Kannada),
 *       section "ಮೆಮೊರಿ ವಾಲ್ (Memory Wall) ವಿರುದ್ಧ ಹೋರಾಟ", paragraph on
 *       PagedAttention: KV cache entries kept in fixed-size blocks that are
 *       allocated non-contiguously and found through an indirection table.
 *
 * Conventions shared by every entry point
 *  - Every data pointer is a device pointer owned by the caller.  The
 *    library never allocates or frees device memory and never synchronises
 *    the stream; work is enqueued on `stream` (a hipStream_t, NULL = the
 *    default stream) and faults inside kernels surface at the caller's next
 *    synchronisation.
 *  - Tensors are dense and row-major, last index fastest (the *_strided
 *    entry points take fd_tensor descriptors with strides instead):
 *        q    [B, Hq, D]            (bifurcated: [S, Hq, D])
 *        k, v [B, Hkv, Lmax, D]     (context: [Hkv, Lc, D];
 *                                    decode: [S, Hkv, Ldmax, D])
 *        out  [B, Hq, D]
 *    q, k, v and out must be 16-byte aligned; lens, lse buffers 4-byte.
 *  - Query head h reads KV head h / (Hq / Hkv) (contiguous groups).
 *  - Supported: q/k/v dtype FD_F32 or FD_BF16 (all three the same), or,
 *    for fd_decode_attn_fp8 only, FD_FP8_E4M3 (E4M3 cache, bf16 query); out
 *    dtype FD_F32 or FD_BF16 (bf16 is rounded to nearest even), head_dim
 *    64 or 128, Hq a multiple of Hkv.  Anything else returns
 *    FD_ERR_UNSUPPORTED; there is no silent fallback.
 *  - Every shape, pointer, alignment and workspace check runs before the
 *    first HIP call; a failing check returns its status and leaves the
 *    stream untouched.  Device-resident lengths and block tables cannot be
 *    checked without a synchronisation and are preconditions, checked only
 *    when validation is on (fd_set_validation, FD_VALIDATE=1).
 *  - Errors are returned as fd_status; fd_last_error_message() gives a
 *    thread-local description of the most recent failure.  No entry point
 *    aborts or throws.
 *  - scale <= 0 selects 1/sqrt(head_dim).  lse values are natural-log
 *    log-sum-exps of the scaled scores.
 */
#ifndef FD_H
#define FD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fd_status {
    FD_OK = 0,
    FD_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size          */
    FD_ERR_UNSUPPORTED = 2,   /* valid request the kernels do not implement */
    FD_ERR_WORKSPACE = 3,     /* workspace missing or too small             */
    FD_ERR_HIP = 4            /* the HIP runtime reported an error          */
} fd_status;

typedef enum fd_dtype {
    FD_F32 = 0,
    FD_BF16 = 1,
    /* K/V cache of OCP 8-bit floating point E4M3 codes (1 byte each) with a
     * bf16 query; for fd_decode_attn_fp8, fd_plan_splits and
     * fd_decode_attn_workspace_size. */
    FD_FP8_E4M3 = 2
} fd_dtype;

/* A tensor passed by descriptor (the *_strided entry points): a device
 * pointer, its element type (fd_dtype), and `ndim` dimensions in the
 * logical order the entry point names, outermost first, with the element
 * stride of each.  The last dimension (the head dim) must be contiguous
 * (stride 1); every other stride must be >= 0 and a multiple of 16 bytes,
 * and data 16-byte aligned.  A token-major cache [B, L, Hkv, D] is passed as
 * the logical [B, Hkv, L, D] with strides {L*Hkv*D, D, Hkv*D, 1}.  Unused
 * shape / stride entries are ignored. */
typedef struct fd_tensor {
    void* data;
    int32_t dtype;
    int32_t ndim;
    int64_t shape[4];
    int64_t stride[4];
} fd_tensor;

/* Largest split count accepted (per sequence for decode; context plus
 * decode pieces for the bifurcated call). */
#define FD_MAX_SPLITS 4096

/* Which cache rows make up piece i of a sequence of n valid rows cut into
 * P pieces ([FD] "Por qué la decodificación necesita otra planificación"
 * leaves the cut open: any partition of the rows combines to the same
 * attention).
 *   FD_PIECES_CONTIGUOUS: rows [i*c, min((i+1)*c, n)), c = ceil(n / P)
 *     rounded up to a multiple of 16.
 *   FD_PIECES_INTERLEAVED: the tiles of T rows (T = fd_piece_tile_rows())
 *     numbered i, i + P, i + 2P, ..., each clipped to [0, n); at any moment
 *     all pieces then read one window of the cache.
 * fd_decode_attn (and its paged and E4M3 forms) cuts interleaved where the
 * matrix-core kernel runs (bf16 or E4M3 cache, head_dim 128, G >= 4) and
 * contiguous elsewhere: the faster of the two for each kernel. */
typedef enum fd_piece_layout {
    FD_PIECES_CONTIGUOUS = 0,
    FD_PIECES_INTERLEAVED = 1
} fd_piece_layout;

/* Human-readable name of a status code (static string). */
const char* fd_status_string(fd_status status);

/* Thread-local text describing the last non-OK status returned on this
 * thread ("" if none). */
const char* fd_last_error_message(void);

/* Library version, as major*10000 + minor*100 + patch. */
int32_t fd_version(void);

/*
 * fd_plan_splits - split count for one decode call ([FD] section "Por qué
 * la decodificación necesita otra planificación": split only when batch x
 * heads alone leaves the GPU short of independent work, and not so far that
 * the pieces become too short to pay for the partial results).
 *
 * Pure host function; reads no device state.  n_cu is the number of
 * compute units to fill (256 on MI355X).  Returns a count in
 * [1, FD_MAX_SPLITS], or -1 for invalid arguments.  It depends only on
 * shapes, never on the device-resident lengths.
 */
int32_t fd_plan_splits(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int64_t max_len, int32_t dtype, int32_t n_cu);

/*
 * fd_device_cu_count - compute units of the current HIP device (cached per
 * device).  Returns FD_ERR_HIP when no device is usable.
 */
fd_status fd_device_cu_count(int32_t* n_cu);

/*
 * fd_decode_attn_workspace_size - bytes of device workspace fd_decode_attn
 * needs for these shapes and this n_splits (<= 0: the planner's count for
 * the current device, which needs a visible device).  The workspace holds
 * the per-piece partial outputs [B, Hq, n_splits, D] fp32 and their lse
 * [B, Hq, n_splits] fp32; it is 0 bytes when one piece suffices.
 */
fd_status fd_decode_attn_workspace_size(int32_t batch, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int64_t max_len, int32_t dtype,
                                        int32_t n_splits, size_t* bytes);

/*
 * fd_decode_attn - split-KV decode attention ([FD] "Por qué la
 * decodificación necesita otra planificación"; [FA] online softmax and
 * fusion; [BA] "Tilastot" for the KV-head sharing).
 *
 *   q        [B, Hq, D]        one query position per sequence
 *   k, v     [B, Hkv, Lmax, D] KV cache; row t of sequence b is valid for
 *                              t < lens[b]; other rows are never read
 *   lens     device int32 [B], each in [1, Lmax]; NULL = all Lmax
 *   n_splits pieces per sequence, <= 0 = fd_plan_splits() for the current
 *            device; a forced count above what the length needs yields
 *            empty pieces, which are legal
 *   out      [B, Hq, D] in out_dtype
 *   lse_out  device fp32 [B, Hq] (natural log) or NULL
 *   scale    softmax temperature; <= 0 selects 1/sqrt(D)
 *   workspace, workspace_bytes: device scratch of at least
 *            fd_decode_attn_workspace_size() bytes (may be NULL when that
 *            size is 0); 256-byte alignment recommended
 *   stream   hipStream_t or NULL
 *
 * Pieces are cut as fd_piece_layout describes.  The result for fixed
 * inputs and a fixed n_splits is bitwise repeatable
 * (fixed reduction order, no float atomics).
 */
fd_status fd_decode_attn(const void* q, const void* k, const void* v, const int32_t* lens,
                         int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int64_t max_len, int32_t dtype,
                         int32_t n_splits, void* out, int32_t out_dtype, float* lse_out,
                         float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of partials fd_decode_attn_noalloc can hold (16 MiB): that many per
 * GPU stay reserved inside the library until the process ends. */
#define FD_NOALLOC_MAX_WORKSPACE (16u << 20)

/*
 * fd_decode_attn_noalloc - fd_decode_attn for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  It calls no allocating routine of any kind.
 *
 * Arguments, results and errors are those of fd_decode_attn without the
 * workspace: the partials live in a fixed array of FD_NOALLOC_MAX_WORKSPACE
 * bytes inside the library, one per GPU, held until the process ends.  A
 * call whose partials need more (fd_decode_attn_workspace_size with the
 * same shapes and split count) returns FD_ERR_WORKSPACE before any launch.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind; calls that overlap on one GPU (two streams, two threads) race
 * and must be serialised by the caller.  The first call on each device
 * looks up that device's copy of the array (hipGetSymbolAddress).
 */
fd_status fd_decode_attn_noalloc(const void* q, const void* k, const void* v, const int32_t* lens,
                                 int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int64_t max_len, int32_t dtype, int32_t n_splits,
                                 void* out, int32_t out_dtype, float* lse_out, float scale, void* stream);

/*
 * fd_decode_attn_strided - fd_decode_attn (or, for an E4M3 cache,
 * fd_decode_attn_fp8) on tensors given by descriptors with arbitrary
 * strides, so that views and other cache layouts (token-major, a slice of a
 * larger pool) need no copy ([FA] "Il supporto hardware e la forma dei dati
 * determinano l'uso del percorso rapido": a fast path states exactly which
 * layouts it takes and checks them).
 *
 *   q    logical [B, Hq, D], dtype FD_F32 / FD_BF16 (FD_BF16 for an E4M3 cache)
 *   k, v logical [B, Hkv, Lmax, D], the same shape, strides and dtype
 *        (FD_F32, FD_BF16 or FD_FP8_E4M3); the token stride below 2^24
 *        elements and at most 2^27 bytes
 *   k_scale, v_scale  E4M3 cache only: as in fd_decode_attn_fp8
 *   out  logical [B, Hq, D], FD_F32 or FD_BF16, rows must not overlap
 *   everything else   as in fd_decode_attn; the workspace size is
 *                     fd_decode_attn_workspace_size() of the same shapes
 * Results equal fd_decode_attn's on the same values bit for bit, for the
 * same n_splits.
 */
fd_status fd_decode_attn_strided(const fd_tensor* q, const fd_tensor* k, const fd_tensor* v, const float* k_scale,
                                 const float* v_scale, const int32_t* lens, int32_t n_splits, const fd_tensor* out,
                                 float* lse_out, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * fd_decode_attn_fp8 - fd_decode_attn over a KV cache of 8-bit floating
 * point codes ([MW] "ಮೆಮೊರಿ ವಾಲ್ (Memory Wall) ವಿರುದ್ಧ ಹೋರಾಟ", quantisation
 * paragraph: fewer bits per stored value, fewer bytes over the memory bus).
 * Codes are OCP E4M3 ("fn": bias 7, no infinities, 0x7F/0xFF NaN, largest
 * finite 448); cache value = code value * the KV head's scale.  Every code
 * is exact in bf16; products run on bf16 with fp32 accumulation.
 *
 *   q                bf16 [B, Hq, D]
 *   k, v             uint8 codes [B, Hkv, Lmax, D]
 *   k_scale, v_scale device fp32 [Hkv], positive and finite, or NULL = 1
 *   everything else  as in fd_decode_attn; the workspace size is
 *                    fd_decode_attn_workspace_size(..., FD_FP8_E4M3, ...)
 */
fd_status fd_decode_attn_fp8(const void* q, const void* k, const void* v, const float* k_scale,
                             const float* v_scale, const int32_t* lens, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int64_t max_len, int32_t n_splits, void* out, int32_t out_dtype,
                             float* lse_out, float scale, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * fd_decode_attn_paged - fd_decode_attn over a paged KV cache ([MW] "ಮೆಮೊರಿ
 * ವಾಲ್ (Memory Wall) ವಿರುದ್ಧ ಹೋರಾಟ", PagedAttention: fixed-size blocks found
 * through an indirection table).  The result is the result of
 * fd_decode_attn on the gathered cache, bit for bit, for the same n_splits.
 *
 *   k_pages, v_pages  [num_pages, Hkv, page_size, D]: page p holds, for each
 *                     KV head, page_size consecutive rows
 *   block_table       device int32 [B, max_pages_per_seq]: row t of sequence
 *                     b is row t % page_size of page
 *                     block_table[b][t / page_size]; only entries that cover
 *                     rows < lens[b] are read.  Entries must lie in
 *                     [0, num_pages); an entry outside is clamped into it (a
 *                     wrong result, never a read outside the pool)
 *   page_size         power of two, 16 <= page_size <= 2^20
 *   num_pages         pages in the pool, 1 .. 2^31 - 1
 *   max_pages_per_seq table columns; rows per sequence are at most
 *                     max_len = max_pages_per_seq * page_size (<= 2^30)
 *   lens              device int32 [B], each in [1, max_len]; NULL = max_len
 *   everything else   as in fd_decode_attn; the workspace size is
 *                     fd_decode_attn_workspace_size(..., max_len, ...)
 */
fd_status fd_decode_attn_paged(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* lens, int32_t batch,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t page_size, int64_t num_pages, int32_t max_pages_per_seq,
                               int32_t dtype, int32_t n_splits, void* out, int32_t out_dtype,
                               float* lse_out, float scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * fd_piece_tile_rows - rows per tile T of the FD_PIECES_INTERLEAVED layout
 * for these shapes (the partial kernel's rows per workgroup step: 128 on
 * the matrix-core path; 32 to 256 on the vector-ALU path, depending on the
 * element size, head_dim and the query rows per unit).  Pure host
 * function; -1 for invalid or unsupported arguments.
 */
int32_t fd_piece_tile_rows(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype);

/*
 * fd_decode_attn_partials - the partial stage of fd_decode_attn on its own
 * ([FD] "Por qué la decodificación necesita otra planificación": every piece
 * yields a partial output and its log-sum-exp).  Together with
 * fd_lse_combine(o_part, lse_part, B*Hq, n_splits, D, ...) it computes
 * exactly what fd_decode_attn computes; callers that split one sequence's
 * history across several devices combine the pieces of all of them.
 *
 *   q, k, v, lens, shapes, dtype, scale: as in fd_decode_attn
 *   n_splits      pieces per sequence, > 0 (no planner here)
 *   piece_layout  fd_piece_layout: which rows each piece covers
 *   o_part        device fp32 [B*Hq, n_splits, D], 16-byte aligned
 *   lse_part      device fp32 [B*Hq, n_splits]; -inf (with o_part = 0)
 *                 marks an empty piece
 */
fd_status fd_decode_attn_partials(const void* q, const void* k, const void* v, const int32_t* lens,
                                  int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int64_t max_len, int32_t dtype, int32_t n_splits,
                                  int32_t piece_layout, float* o_part, float* lse_part, float scale,
                                  void* stream);

/*
 * fd_bifurcated_attn_workspace_size - bytes of workspace fd_bifurcated_attn
 * needs: partials of every context piece and every decode piece,
 * [S, Hq, P, D] fp32 plus [S, Hq, P] fp32.
 */
fd_status fd_bifurcated_attn_workspace_size(int32_t samples, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int64_t ctx_len, int64_t dec_max_len,
                                            int32_t dtype, size_t* bytes);

/*
 * fd_bifurcated_attn - single-context batch-sampling attention ([BA]
 * "Tiivistelmä"): S samples share one context KV; each also has its own
 * decode KV.  The result equals standard attention of every sample over
 * [context rows ; its own valid decode rows].
 *
 *   q             [S, Hq, D]
 *   k_ctx, v_ctx  [Hkv, Lc, D], Lc >= 1 (all rows valid)
 *   k_dec, v_dec  [S, Hkv, Ldmax, D], Ldmax >= 1
 *   dec_lens      device int32 [S], each in [0, Ldmax]; NULL = all Ldmax
 *   out, lse_out, scale, workspace, stream: as in fd_decode_attn
 */
fd_status fd_bifurcated_attn(const void* q, const void* k_ctx, const void* v_ctx,
                             const void* k_dec, const void* v_dec, const int32_t* dec_lens,
                             int32_t samples, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int64_t ctx_len, int64_t dec_max_len,
                             int32_t dtype, void* out, int32_t out_dtype, float* lse_out,
                             float scale, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * fd_bifurcated_attn_paged - fd_bifurcated_attn with each sample's decode
 * rows in a paged pool ([MW] "ಮೆಮೊರಿ ವಾಲ್ (Memory Wall) ವಿರುದ್ಧ ಹೋರಾಟ",
 * PagedAttention paragraph: fixed-size blocks found through an indirection
 * table), as a serving cache keeps the rows every sample appends; the shared
 * context stays dense.  The result equals fd_bifurcated_attn on the gathered
 * decode cache: bit for bit for fp32 inputs and for more than 8 query heads
 * per KV head; otherwise to within fp32 rounding of the row sums (with at
 * most 8 query heads per KV head the dense decode part carries each weight's
 * bf16 remainder in the padding columns of its matrix-core tile, which the
 * paged form, short of registers, does not).
 *
 *   q, k_ctx, v_ctx, dec_lens, out, lse_out, scale: as in fd_bifurcated_attn
 *   k_pages, v_pages   [num_pages, Hkv, page_size, D]
 *   block_table        device int32 [S, max_pages_per_seq]: decode row t of
 *                      sample s is row t % page_size of page
 *                      block_table[s][t / page_size]; only entries covering
 *                      rows < dec_lens[s] are read; ids outside
 *                      [0, num_pages) are clamped into it
 *   page_size, num_pages, max_pages_per_seq: as in fd_decode_attn_paged;
 *                      Ldmax = max_pages_per_seq * page_size
 *   workspace          fd_bifurcated_attn_workspace_size(..., Ldmax, ...)
 */
fd_status fd_bifurcated_attn_paged(const void* q, const void* k_ctx, const void* v_ctx, const void* k_pages,
                                   const void* v_pages, const int32_t* block_table, const int32_t* dec_lens,
                                   int32_t samples, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int64_t ctx_len, int32_t page_size, int64_t num_pages,
                                   int32_t max_pages_per_seq, int32_t dtype, void* out, int32_t out_dtype,
                                   float* lse_out, float scale, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * fd_bifurcated_attn_strided - fd_bifurcated_attn on tensors given by
 * descriptors (see fd_tensor and fd_decode_attn_strided).
 *
 *   q             logical [S, Hq, D]
 *   k_ctx, v_ctx  logical [Hkv, Lc, D], the same shape, strides and dtype
 *   k_dec, v_dec  logical [S, Hkv, Ldmax, D], the same shape, strides, dtype
 *   out           logical [S, Hq, D], rows must not overlap
 *   q and both caches share one dtype (FD_F32 or FD_BF16); token strides
 *   below 2^24 elements and at most 2^27 bytes.  Everything else as in
 *   fd_bifurcated_attn.
 */
fd_status fd_bifurcated_attn_strided(const fd_tensor* q, const fd_tensor* k_ctx, const fd_tensor* v_ctx,
                                     const fd_tensor* k_dec, const fd_tensor* v_dec, const int32_t* dec_lens,
                                     const fd_tensor* out, float* lse_out, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * fd_prefill_attn - causal many-query (prefill) attention over a whole
 * sequence ([FD] "Por qué la decodificación necesita otra planificación":
 * during prefill many query positions run in parallel; [MW] section on why
 * prompts are fast and generation slow: matrix-matrix work; [FA] on-chip
 * blocks of queries, keys and values with the online softmax).  Position p
 * of sequence b attends to cache rows [0, p].
 *
 *   q        bf16 [B, Hq, Lmax, D]  one query per position
 *   k, v     bf16 [B, Hkv, Lmax, D]
 *   lens     device int32 [B], each in [1, Lmax]; NULL = all Lmax
 *   out      [B, Hq, Lmax, D] in out_dtype; positions at or beyond lens[b]
 *            are not written
 *   lse_out  device fp32 [B, Hq, Lmax] (natural log) or NULL
 *   scale    softmax temperature; <= 0 selects 1/sqrt(D)
 * Supported: bf16, head_dim 128, G = Hq / Hkv <= 128.  No workspace.
 */
fd_status fd_prefill_attn(const void* q, const void* k, const void* v, const int32_t* lens,
                          int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int64_t max_len, int32_t dtype, void* out,
                          int32_t out_dtype, float* lse_out, float scale, void* stream);

/*
 * fd_lse_combine - the reduction of [FD] on its own: merges per-piece
 * normalised outputs and their natural-log lse into the full result.
 *
 *   o_part    device fp32 [rows, n_parts, D]
 *   lse_part  device fp32 [rows, n_parts]; -inf marks an empty piece, which
 *             carries zero weight; every row needs one finite entry (a row
 *             with none gets out = 0 and lse = -inf)
 *   head_dim  D, any value in [1, 512] (the combine does not need 64/128)
 *   out       [rows, D] in out_dtype;  lse_out fp32 [rows] or NULL
 *
 * Piece weights are exp(lse_i - max_j lse_j); out = sum w_i O_i / sum w_i;
 * lse = max_j lse_j + ln(sum w_i).  Fixed summation order.
 */
fd_status fd_lse_combine(const float* o_part, const float* lse_part, int32_t rows,
                         int32_t n_parts, int32_t head_dim, void* out, int32_t out_dtype,
                         float* lse_out, void* stream);

/*
 * fd_set_validation - turn device-side argument validation on (1) or off
 * (0) for every later call in the process; FD_VALIDATE=1 in the environment
 * turns it on when the library is first used.  With validation on, each
 * entry point first checks the device-resident arrays it is about to read
 * (lens / dec_lens against their documented ranges, and the block-table
 * entries that cover valid rows against [0, num_pages)), synchronises the
 * stream, and returns FD_ERR_INVALID_ARG naming the first bad entry before
 * any attention kernel runs.  It costs a synchronisation per call and
 * returns FD_ERR_UNSUPPORTED under stream capture: a debugging aid.
 * fd_validation_enabled() reports the current setting.
 */
fd_status fd_set_validation(int32_t on);
int32_t fd_validation_enabled(void);

/*
 * fd_read_probe - measurement aid, not part of the attention path: streams
 * `bytes` (a positive multiple of 16, buf 16-byte aligned) once with the
 * 16-byte coalesced loads the partial kernels use (non-temporal hint
 * included) and folds them into one
 * word (sink, 4 bytes of device memory, is written only in a
 * data-dependent corner case).  Timing it gives the HBM read rate this
 * device actually sustains, the ceiling for the KV stream.
 */
fd_status fd_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FD_H */
