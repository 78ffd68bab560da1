/*
 * ttl.h — tensor-parallel sharded linear layers, one rank's share on one MI355X (gfx950).
 *
 * The library runs the data-parallel hot path of Megatron-style tensor parallelism for a
 * Llama-style decoder with t tensor-parallel ranks simulated inside one GPU's HBM:
 *
 *   column-parallel GEMM   Y_r = X · W[:, C_r]              (gate_up_proj, head-sliced qkv_proj)
 *   fused SiLU·up          act_r = silu(gate_r) · up_r     (epilogue of the gate_up column GEMM)
 *   row-parallel GEMM      P_r = X_r · W[r·k/t:(r+1)·k/t, :]  (down_proj, o_proj: a partial sum)
 *   reduce + norm          h = Σ_r P_r + residual;  y = h / sqrt(mean(h²) + eps) · gamma
 *
 * The statement of the problem follows the vLLM tensor-parallel walkthrough
 * "vLLM 源码完全拆解（十一）：模型并行与 Worker 层" (pinghaoyang.com.cn), section
 * "一个矩阵乘法如何被切开": a dense layer computes Y = X·W with X[b,k] (b tokens, k input features),
 * W[k,n] and Y[b,n]; t ranks either cut W along n (column split, input replicated, outputs
 * concatenate) or cut W along k and X along its last dimension (row split, partial outputs that
 * must be summed).  Llama's projections carry no bias, so none is taken here.
 *
 * Conventions shared by every entry point
 *   - Tensors are bf16 (raw bits in uint16_t), row-major, dense: X[b,k] has row stride k, W[k,n]
 *     has row stride n, partials are [t,b,n].  Every tensor pointer is a DEVICE pointer.
 *   - W is always the full, unsharded weight; the rank's slice is addressed in place by offsets
 *     (the analogue of weight_loader's narrow() in section "ColumnParallelLinear"), never copied.
 *   - Arithmetic: bf16 × bf16 products accumulated in fp32 on the matrix cores; elementwise math in
 *     fp32; every output is rounded to bf16, nearest-even.
 *   - Ownership: the caller allocates and owns every buffer; the library keeps no pointer after a
 *     call returns and frees nothing of the caller's.  Calls are asynchronous: they validate, then
 *     enqueue kernels on `stream` (a hipStream_t; NULL = the default stream) and return.  Buffers
 *     must stay alive until the stream has run the work.
 *   - Workspace: GEMMs with few token rows (decode batches, small shards) are cut along k and need
 *     fp32 partial sums.  The library keeps one device buffer per (GPU, stream) for them, allocated
 *     on the first such call on that stream and replaced by a larger one when a later call needs
 *     more (the outgrown buffer is kept, so work already enqueued or captured in a graph stays
 *     valid); buffers live until the process ends.  Calls on different streams therefore never
 *     share a buffer and may overlap in time.  The allocation cannot run inside a stream capture:
 *     make one eager call of the shape on the capturing stream before capturing it (a capture that
 *     would need a new or larger buffer fails with TTL_ERR_HIP and enqueues nothing).  A failed
 *     allocation is TTL_ERR_HIP.
 *   - Errors: every call returns a ttl_status.  Arguments are validated synchronously before any
 *     launch; on a non-OK status nothing has been enqueued and ttl_last_error() returns a message
 *     (thread-local).  A launch failure reported by the runtime is TTL_ERR_HIP.  A fault inside a
 *     kernel surfaces at the caller's next synchronisation, as with any HIP kernel.
 *   - Alignment: every pointer 16-byte aligned and every row stride and every slice width a
 *     multiple of 8 elements (16 bytes), else TTL_ERR_ALIGN.
 */
#ifndef TTL_H
#define TTL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ttl_status;
#define TTL_OK 0
#define TTL_ERR_NULL 1          /* a required pointer is NULL */
#define TTL_ERR_SHAPE 2         /* a size is <= 0 or out of the supported range */
#define TTL_ERR_NOT_DIVISIBLE 3 /* a shard width is not an exact division (vLLM's divide() asserts) */
#define TTL_ERR_RANK 4          /* t < 1 or rank outside [0, t) */
#define TTL_ERR_ALIGN 5         /* pointer not 16-byte aligned or stride/width not a multiple of 8 */
#define TTL_ERR_UNSUPPORTED 6   /* a combination the library does not implement */
#define TTL_ERR_HIP 7           /* the HIP runtime reported an error */

typedef int32_t ttl_epilogue;
#define TTL_EPI_NONE 0
#define TTL_EPI_SILU_MUL 1

/* Storage of the weight W[k,n] (the logical operand is always W[k,n]):
 *   TTL_W_KN: row-major [k][n], row stride n — the statement's own layout;
 *   TTL_W_NK: the transpose stored row-major, [n][k], row stride k — how PyTorch-style Linear
 *             weights ([out_features, in_features]) are kept; the matrix cores read it without a
 *             transpose.  The rows one call reads (from the rank's first to its last weight
 *             column; for the row-parallel call all n rows) must span less than 2 GiB.
 *   TTL_W_BLOCKED: [k][n] cut into blocks of 64 k-rows x 128 columns, each block row-major (its 128
 *             columns contiguous), the blocks of one 128-column strip stored one after another
 *             down k, the strips one after another along n: element (i, j) lives at
 *             ((j/128)·(k/64) + i/64)·8192 + (i%64)·128 + j%128.  Needs k % 64 == 0 and
 *             n % 128 == 0 (and, for the row-parallel call, (k/t) % 64 == 0); ttl_pack_weight_blocked
 *             converts a [k][n] weight.  Each 128-column strip is one contiguous range, which the
 *             weight-bound decode GEMMs stream faster than rows of [k][n] or [n][k] (HBM reads whole
 *             DRAM pages instead of 128-256-byte pieces of many rows).  The strips one call reads
 *             must span less than 2 GiB. */
typedef int32_t ttl_weight_layout;
#define TTL_W_KN 0
#define TTL_W_NK 1
#define TTL_W_BLOCKED 2

#define TTL_MAX_SEGMENTS 3
#define TTL_MAX_PEERS 16   /* partial buffers reduce_partials_rmsnorm_peers accepts */

/*
 * Column split of the full W[k,n] ("MergedColumnParallelLinear / QkvParallelLinear" on the vLLM
 * walkthrough): W is nseg segments packed side by side along n — one for a plain layer, two for
 * gate_up (output_sizes = [I, I]), three for qkv (q | k | v).  seg_n[i] is segment i's width in the
 * full W (the widths sum to n); seg_parts[i] is how many distinct slices segment i is cut into:
 * t for a plain, gate, up or q segment and for k/v when t <= n_kv_heads; n_kv_heads for k/v when
 * t > n_kv_heads (each kv head then replicated on t / n_kv_heads ranks).  Rank r takes slice
 * floor(r · seg_parts[i] / t) of each segment; its output concatenates the slices in segment order.
 */
typedef struct {
  int32_t nseg;
  int64_t seg_n[TTL_MAX_SEGMENTS];
  int32_t seg_parts[TTL_MAX_SEGMENTS];
} ttl_col_split;

/*
 * shard_linear_col — ColumnParallelLinear forward of rank `rank` of `t`, with gather_output=False
 * (vLLM walkthrough, section "ColumnParallelLinear": the rank keeps its own n/t columns).
 *
 *   X      [b, k]  bf16, the full (replicated) input.
 *   W      the full weight W[k, n], row-major [k][n] (row stride n), the statement's own storage;
 *          only the rank's columns are read.
 *   split  column split (see ttl_col_split); NULL means one segment cut into t slices.
 *   epi    TTL_EPI_NONE: Y[b, n_r] = X · W[:, C_r], n_r = Σ_i seg_n[i] / seg_parts[i].
 *          TTL_EPI_SILU_MUL: the split must have two equal segments (gate | up) with equal part
 *          counts; Y[b, n_r/2] = silu(X·W_gate_r) · (X·W_up_r) with silu(x) = x / (1 + e^-x),
 *          computed in fp32 from the fp32 accumulators — the activation "on the local shard" of
 *          section 14 of "vLLM Code Reading (Section 5)" (jeremyguo.space).  gate and up never
 *          reach memory.
 *   Y      output, row stride n_r (or n_r/2), caller-allocated; must not overlap X or W.
 * Errors: NULL X/W/Y -> NULL; b,k,n <= 0 -> SHAPE; bad t/rank -> RANK; a segment width not
 * divisible by its part count, part count neither t nor a divisor of t, or widths not summing to n
 * -> NOT_DIVISIBLE; misalignment -> ALIGN; SILU_MUL with an unsuitable split, nseg outside 1..3,
 * or Y overlapping X or W -> UNSUPPORTED.
 */
ttl_status shard_linear_col(const uint16_t* X, int64_t b, int64_t k,
                            const uint16_t* W, int64_t n,
                            int32_t t, int32_t rank,
                            const ttl_col_split* split,
                            ttl_epilogue epi,
                            uint16_t* Y,
                            void* stream);

/*
 * shard_linear_col_stored — shard_linear_col with the weight in any of the storages above
 * (`w_layout`); the logical operand is still W[k, n] and the results are bit for bit those of
 * shard_linear_col on the same logical weight.  TTL_W_KN is exactly shard_linear_col.
 * Errors: as shard_linear_col; TTL_W_BLOCKED with k % 64 != 0 or n % 128 != 0 -> ALIGN; an
 * unknown w_layout, or TTL_W_NK rows (TTL_W_BLOCKED strips) read spanning 2 GiB or more ->
 * UNSUPPORTED.
 */
ttl_status shard_linear_col_stored(const uint16_t* X, int64_t b, int64_t k,
                                   const uint16_t* W, int64_t n, ttl_weight_layout w_layout,
                                   int32_t t, int32_t rank,
                                   const ttl_col_split* split,
                                   ttl_epilogue epi,
                                   uint16_t* Y,
                                   void* stream);

/*
 * shard_linear_col_noalloc — shard_linear_col_stored for callers that cannot allocate device memory:
 * code recorded under HIP graph capture, tight serving loops, and harnesses that forbid allocation
 * after start-up.  Same arguments, same kernels and bit for bit the same results as
 * shard_linear_col_stored; the only difference is where split-K launches (decode batches, few
 * tiles with a long k) keep their fp32 partial sums: a 64-MiB array inside the library's device
 * code (TTL_NOALLOC_SCRATCH_BYTES), one per GPU, held until the process ends, instead of the
 * per-stream buffers the other entry points allocate on first use.  The call allocates and frees
 * nothing (the array's device address is looked up on the first call on each GPU).
 * Every call on one GPU shares that GPU's array, which keeps the last call's partials (nothing in
 * it needs to start at zero: each call writes every partial it reads): calls whose work overlaps
 * in time on one GPU (different streams) race and must be serialised, e.g. on one stream.
 * Errors: as shard_linear_col_stored; a call whose split-K partials would need more than
 * TTL_NOALLOC_SCRATCH_BYTES -> UNSUPPORTED, before anything is enqueued; the array's address not
 * obtainable -> HIP.
 */
#define TTL_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
ttl_status shard_linear_col_noalloc(const uint16_t* X, int64_t b, int64_t k,
                                    const uint16_t* W, int64_t n, ttl_weight_layout w_layout,
                                    int32_t t, int32_t rank,
                                    const ttl_col_split* split,
                                    ttl_epilogue epi,
                                    uint16_t* Y,
                                    void* stream);

/*
 * shard_linear_col_gathered — ColumnParallelLinear forward with gather_output=True (vLLM
 * walkthrough, sections "ColumnParallelLinear" and "all-gather"): the rank's output is placed in its
 * block of the all-gathered tensor, the concatenation of the t rank outputs along the last dimension
 * in rank order.  On one GPU the simulated ranks fill the whole gathered tensor; with a plain split
 * it equals X · W (and with SILU_MUL the full silu(X·W_gate)·(X·W_up)).  Used, for one, by a
 * vocab-parallel LM head (the "Tensor Parallelism" manual, section "Vocab Parallel": each rank owns
 * a contiguous vocabulary slice, and the logits are all-gathered).
 *
 *   W      stored as `w_layout` says (as shard_linear_col_stored).
 *   Y_all  [b, t·w] bf16, w = the rank output width of shard_linear_col (n_r, or n_r/2 with
 *          SILU_MUL); this call writes columns [rank·w, (rank+1)·w) and nothing else.
 * Every other argument, and every error, as shard_linear_col_stored.
 */
ttl_status shard_linear_col_gathered(const uint16_t* X, int64_t b, int64_t k,
                                     const uint16_t* W, int64_t n, ttl_weight_layout w_layout,
                                     int32_t t, int32_t rank,
                                     const ttl_col_split* split,
                                     ttl_epilogue epi,
                                     uint16_t* Y_all,
                                     void* stream);

/*
 * shard_linear_row — RowParallelLinear forward of rank `rank` of `t` with reduce_results=False:
 * the rank's partial sum, which a later reduction adds up (vLLM walkthrough, section
 * "RowParallelLinear"; section 12 of "vLLM Code Reading (Section 5)": Y_i = X_i A_i, Y = Σ_i Y_i).
 *
 *   X      x_is_parallel != 0: the rank's input slice [b, k/t] (input_is_parallel=True, e.g. the
 *          act of shard_linear_col);  x_is_parallel == 0: the full input [b, k], whose columns
 *          [r·k/t, (r+1)·k/t) are used (split along the last dimension).
 *   k      the FULL input dimension of W.
 *   W      the full weight W[k, n], row-major [k][n]; W's rows [r·k/t, (r+1)·k/t) are read.
 *   P      [b, n] bf16 partial for this rank (for simulated ranks, the caller passes P + r·b·n of
 *          a [t, b, n] buffer); must not overlap X or W.
 * Errors: as shard_linear_col; k not divisible by t -> NOT_DIVISIBLE; P overlapping X or W ->
 * UNSUPPORTED.
 */
ttl_status shard_linear_row(const uint16_t* X, int64_t b, int64_t k,
                            int32_t x_is_parallel,
                            const uint16_t* W, int64_t n,
                            int32_t t, int32_t rank,
                            uint16_t* P,
                            void* stream);

/*
 * shard_linear_row_stored — shard_linear_row with the weight in any of the storages above
 * (`w_layout`); bit for bit the results of shard_linear_row on the same logical weight.
 * Errors: as shard_linear_row; TTL_W_BLOCKED with k % 64, (k/t) % 64 or n % 128 != 0 -> ALIGN; an
 * unknown w_layout, or a TTL_W_NK / TTL_W_BLOCKED weight of 2 GiB or more -> UNSUPPORTED.
 */
ttl_status shard_linear_row_stored(const uint16_t* X, int64_t b, int64_t k,
                                   int32_t x_is_parallel,
                                   const uint16_t* W, int64_t n, ttl_weight_layout w_layout,
                                   int32_t t, int32_t rank,
                                   uint16_t* P,
                                   void* stream);

/*
 * reduce_partials_rmsnorm — the row-parallel reduction of t rank partials held in one HBM,
 * followed by the residual add and RMSNorm of post_attention_layernorm(hidden, residual)
 * ("Tensor & pipeline parallelism", Undercurrent docs, sections "Row-parallel layers all-reduce
 * inside forward()", "residual_stream" and "final_norm": the norm is over the full, unsharded
 * hidden dimension).
 *
 *   P         [t, b, n] bf16 partials.
 *   residual  [b, n] bf16 or NULL (then h = Σ_r P_r).
 *   gamma     [n] bf16 RMSNorm gain (replicated on every rank).
 *   eps       added to the mean square inside the square root.
 *   residual_out [b, n] bf16: the updated residual stream h = Σ_r P_r + residual (the sum in fp32,
 *             ascending r, then the residual); may alias `residual`.
 *   Y         [b, n] bf16: h / sqrt(mean_j h_j² + eps) · gamma, from the fp32 h.
 * The summation order is fixed, so results are bitwise reproducible run to run.
 * Errors: NULL P/gamma/residual_out/Y -> NULL; t < 1 -> RANK; b, n <= 0 or n > 65536 -> SHAPE;
 * misalignment -> ALIGN; Y aliasing an input -> UNSUPPORTED.
 */
ttl_status reduce_partials_rmsnorm(const uint16_t* P, int32_t t, int64_t b, int64_t n,
                                   const uint16_t* residual,
                                   const uint16_t* gamma, float eps,
                                   uint16_t* residual_out,
                                   uint16_t* Y,
                                   void* stream);

/*
 * reduce_scatter_partials_rmsnorm — the sequence-parallel form of reduce_partials_rmsnorm: the
 * partial sums are reduce-scattered over the token rows, so rank `rank` reduces, adds its residual
 * shard to and normalises only its chunk of b/t rows, [rank·b/t, (rank+1)·b/t) ("Tensor
 * Parallelism" manual, section "Communication Patterns": after reduce-scatter each rank holds one
 * reduced chunk; "vLLM Code Reading (Section 5)", section 4, "PP + SP 下的 all_gather_tensors":
 * under sequence parallelism the residual is kept scattered over the ranks, the token count padded
 * for it).
 *
 *   P         [t, b, n] bf16 partials of all t ranks over all b rows.
 *   residual  [b/t, n] bf16, this rank's shard of the residual stream, or NULL.
 *   residual_out, Y  [b/t, n] bf16, this rank's shards of the outputs (as reduce_partials_rmsnorm).
 * The t calls rank = 0..t-1 together produce exactly reduce_partials_rmsnorm's outputs, row chunk
 * by row chunk (the all-gather that follows is their concatenation).
 * Errors: as reduce_partials_rmsnorm; rank outside [0, t) -> RANK; b not divisible by t ->
 * NOT_DIVISIBLE (the caller pads the token count).
 */
ttl_status reduce_scatter_partials_rmsnorm(const uint16_t* P, int32_t t, int64_t b, int64_t n,
                                           int32_t rank,
                                           const uint16_t* residual,
                                           const uint16_t* gamma, float eps,
                                           uint16_t* residual_out,
                                           uint16_t* Y,
                                           void* stream);

/*
 * reduce_partials_rmsnorm_peers — reduce_partials_rmsnorm over rows [row0, row0 + rows) of t
 * partials held in t separate buffers, one pointer per rank: the compute half of an all-reduce
 * that reads the other ranks' buffers in place (on several GPUs, buffers mapped from the peers;
 * "vLLM 源码完全拆解（十一）", section "RowParallelLinear": the row layer's output is the sum of
 * the ranks' partials; "Tensor Parallelism" manual, section "Communication Patterns": a
 * reduce-scatter leaves each rank one reduced chunk, which an all-gather then shares).  With
 * row0 = 0 and rows = b every row is reduced (one-shot); with row0 = rank·b/t and rows = b/t,
 * rank `rank` reduces its chunk (two-shot, the reduce-scatter half).
 *
 *   P_ranks   HOST array of t DEVICE pointers; P_ranks[r] is rank r's partial [b, n] bf16.
 *             1 <= t <= TTL_MAX_PEERS.  The array is read during the call only.
 *   residual  [rows, n] bf16 (the residual rows of the range) or NULL.
 *   residual_out, Y  [rows, n] bf16, as reduce_partials_rmsnorm, for the rows of the range.
 * Same arithmetic as reduce_partials_rmsnorm.  With the partials as one [t, b, n] slab, a call
 * over the same number of rows returns the same bits: reduce_partials_rmsnorm for all rows,
 * reduce_scatter_partials_rmsnorm for a rank's chunk.  (residual_out is a per-element sum; y also
 * depends on the order in which a row's mean square is reduced across threads, which is fixed for
 * a given row count and n.)
 * Errors: b, n, or the row range empty or out of [0, b) -> SHAPE; t < 1 -> RANK;
 * t > TTL_MAX_PEERS -> UNSUPPORTED; NULL P_ranks, an entry of it, gamma, residual_out or Y -> NULL;
 * misalignment -> ALIGN; outputs overlapping a partial or each other -> UNSUPPORTED.
 */
ttl_status reduce_partials_rmsnorm_peers(const uint16_t* const* P_ranks, int32_t t, int64_t b, int64_t n,
                                         int64_t row0, int64_t rows,
                                         const uint16_t* residual,
                                         const uint16_t* gamma, float eps,
                                         uint16_t* residual_out,
                                         uint16_t* Y,
                                         void* stream);

/*
 * ttl_pack_weight_blocked — W_blk = W stored as TTL_W_BLOCKED (see above), from W[k][n] row-major.
 * Set-up work for a weight that is used many times; not on the hot path.
 *
 *   W      [k, n] bf16, row-major.      W_blk  k·n bf16, caller-allocated, must not overlap W.
 * Errors: NULL W/W_blk -> NULL; k, n <= 0 or k·n >= 2^31 -> SHAPE; k % 64, n % 128 or 16-byte
 * alignment -> ALIGN; overlapping buffers -> UNSUPPORTED.  Enqueued on `stream`.
 */
ttl_status ttl_pack_weight_blocked(const uint16_t* W, int64_t k, int64_t n, uint16_t* W_blk, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ttl_last_error(void);

/*
 * ttl_set_gemm_override — for tests and measurements only: force the GEMM kernel family that every
 * later shard_linear_* call in the process uses, whatever the shape, instead of the library's
 * choice by shape.  Every kernel family computes the same products in the same k order within a
 * tile, so results differ only by the summation order of k-splits (bit-equal where the split
 * count is equal).  Process-wide; not for concurrent use with GEMM calls on other threads.
 *
 *   kernel    TTL_GEMM_AUTO restores the choice by shape; the others name a family (below).
 *   splits    > 0: the k-split count of the split-K kernel and of tiles cut along k; 0 = by shape.
 *   plan_cus  > 0: compute units the 256-row / 192-row cut (TTL_GEMM_MIXED) is planned for; 0 = the
 *             device's.
 *   trace     != 0: print each 256-row / 192-row cut and each launch with appended rows to stderr.
 * Errors: an unknown kernel, or a negative splits/plan_cus -> UNSUPPORTED.
 */
#define TTL_GEMM_AUTO 0
#define TTL_GEMM_TILED 1        /* 256 x 256 tiles: the four-wave kernel where K % 64 == 0 */
#define TTL_GEMM_SPLITK 2       /* the split-K kernel (32..128-row tiles, k cut into splits) */
#define TTL_GEMM_EIGHTWAVE 3    /* 256 x 256 tiles by the eight-wave kernel (any K) */
#define TTL_GEMM_TILESPLIT 4    /* 256 x 256 tiles cut along k */
#define TTL_GEMM_NARROW 5       /* 256 x 128 tiles */
#define TTL_GEMM_NARROWSPLIT 6  /* 256 x 128 tiles cut along k */
#define TTL_GEMM_SHORT 7        /* 192 x 256 tiles */
#define TTL_GEMM_MIXED 8        /* the 256-row / 192-row cut wherever one exists */
#define TTL_GEMM_PERSIST 9      /* 256 x 256 tiles by a persistent grid (up to two tiles per CU) */
#define TTL_GEMM_TILED16 10     /* 256 x 256 tiles fed to 16 x 16 x 32 products */
#define TTL_GEMM_APPENDED 11    /* 256 x 256 tiles (16 x 16 x 32) over the whole row-tiles, the rows
                                   below them appended to the tiles, at most 16 per row-tile (plain
                                   columns, K % 64 == 0); otherwise the choice by shape */
#define TTL_GEMM_STREAM_NK 12   /* the split-free kernel for weights stored [n][k] and at most 64
                                   rows (K % 32 == 0); otherwise the choice by shape */
ttl_status ttl_set_gemm_override(int32_t kernel, int32_t splits, int32_t plan_cus, int32_t trace);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t ttl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TTL_H */
