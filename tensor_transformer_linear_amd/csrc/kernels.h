// Internal declarations shared by the HIP sources of libttl (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttl {

// Parameters of one tiled bf16 GEMM launch: C[M, N] = A[M, K] · B_map[K, N].
// A rows have stride lda (elements); A already points at the first column the rank uses.
// B is the weight: w_nk = 0 stores it as W[k][n] (row stride ldb, B at the first k row the rank
// uses); w_nk = 1 stores W^T[n][k] (row stride ldb, b_rows rows, B at the first k column the rank
// uses).  Output column j reads weight column wcol(j) given by the column map below.
struct GemmParams {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* C;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;        // N = output columns (act columns in SiLU·up mode)
  int32_t mode;           // 0: plain / segmented columns, 1: SiLU(gate)·up
  int32_t nseg;           // mode 0: 1..3 segments
  int32_t seg_out0[4];    // mode 0: first output column of segment s; seg_out0[nseg] = N
  int64_t seg_w0[3];      // mode 0: weight column of segment s's first output column
  int64_t gate_w0, up_w0; // mode 1: weight columns of act column 0's gate and up inputs
  int32_t tiles_m, tiles_n;
  int32_t narrow;         // four-wave kernel: 1 = tiles of 256 rows x 128 weight columns, 0 = 256 x 256
  int32_t w_nk;           // weight stored transposed ([n][k])
  // w_blk: weight stored in 64 x 128 blocks, 128-column strips (TTL_W_BLOCKED).  B is the first
  // block of the first strip the call reads (at its first k row), column 0 the strip's first
  // column; ldb is the strip stride in elements (k_full * 128); element (k, j) of the call is at
  // B + (j / 128) * ldb + (k / 64) * 8192 + (k % 64) * 128 + j % 128.
  int32_t w_blk;
  int64_t b_rows;         // w_nk: rows of W^T reachable from B; w_blk: elements reachable from B
  // Split-K launches (splits > 1): fp32 partial sums [splits][M][ws_ld], split s covering k-tiles
  // [s * kt_per_split, (s + 1) * kt_per_split).
  float* ws;
  int64_t ws_ld;
  int32_t splits, kt_per_split;
  // Four-wave kernel: tile_rows = 256 (0 means 256) or 192.  192-row tiles run only as a tile set.
  // Tile sets (rects = 1 or 2, no splits): the launch covers rectangle 0 then rectangle 1, rectangle
  // i being rect_tmc[i] row-tiles of tile_rows rows from row rect_row0[i], by rect_tnc[i] tile
  // columns from tile column rect_tn0[i], walked in groups of rect_group[i] row-tiles (0: 4); rects
  // = 0 is tiles_m x tiles_n tiles from (0, 0).
  int32_t tile_rows;
  int32_t rects;
  int32_t rect_tn0[2], rect_tnc[2], rect_row0[2], rect_tmc[2], rect_group[2];
  // Four-wave kernel, 256 x 256 tiles, no splits and no tile set: persist = 1 launches fewer
  // workgroups than tiles; workgroup b then computes tiles b, b + grid, b + 2 grid, ... in turn,
  // fetching the next tile's first k-tiles while it finishes the current one.
  int32_t persist;
  // 16 x 16 x 32 kernel, plain columns, whole launches of 256 x 256 tiles, no splits: xr_row0 > 0
  // appends 16 rows to every tile, row-tile i taking rows xr_row0 + 16 i .. + 15 (those below M) as
  // its rows 256 .. 271, so that the rows past the launch's whole 256-row tiles are computed in the
  // same round instead of by a launch of their own.  0: none.
  int32_t xr_row0;
};

// SiLU·up as a plain GEMM over the gate columns followed by the up columns (2N outputs, two column
// segments), for split-K partial sums: output j and output N + j are the gate and up inputs of act
// column j, which the finalize kernel pairs.
inline GemmParams silu_as_plain_halves(const GemmParams& p) {
  GemmParams q = p;
  q.mode = 0;
  q.N = 2 * p.N;
  q.nseg = 2;
  q.seg_out0[0] = 0;
  q.seg_out0[1] = p.N;
  q.seg_out0[2] = q.seg_out0[3] = 2 * p.N;
  q.seg_w0[0] = p.gate_w0;
  q.seg_w0[1] = p.up_w0;
  q.seg_w0[2] = 0;
  return q;
}

// Picks the kernel for the shape and launches it: the 256 x 256-tile kernel when its tiles fill the
// chip, otherwise the split-K kernel (short M: decode batches, small shards).  Sets the tiling
// fields of p.  May allocate the split-K workspace of (device, stream) on first use.
hipError_t launch_gemm(GemmParams& p, hipStream_t stream);

// Bytes of split-K workspace launch_gemm would use for p (0 when no launch of its plan splits k):
// the plan walked without launching or allocating anything.
size_t gemm_workspace_bytes(const GemmParams& p);

// launch_gemm with every split-K launch writing its partials to `ws` (ws_bytes, at least
// gemm_workspace_bytes(p)) instead of the library's per-stream buffers; allocates nothing.
hipError_t launch_gemm_fixed_workspace(GemmParams& p, void* ws, size_t ws_bytes, hipStream_t stream);

// Process-wide test and measurement overrides of launch_gemm's choice (ttl_set_gemm_override):
// kernel family (0 = by shape), split count (0 = by shape), CUs the row cut is planned for (0 =
// the device's), and a trace of each cut on stderr.
void set_gemm_override(int kernel, int splits, int plan_cus, bool trace);

// 256 x 256 tiles (tiles_m, tiles_n set by the caller from the two functions below), by either of
// two kernels with identical results: eight waves (two per SIMD, any K), or four waves of 128 x 128
// outputs (one per SIMD, faster; K a multiple of 64).
int gemm_tile_rows();
int gemm_tile_cols(int mode);
hipError_t launch_gemm_tiled(const GemmParams& p, hipStream_t stream);
bool gemm_bigwave_supports(const GemmParams& p);
// Output columns of one four-wave tile: 256 (128 act columns in SiLU·up mode), or with p.narrow
// 128 (64).
int gemm_bigwave_tile_cols(int mode, bool narrow);
// The four-wave kernel also takes split-K launches (plain mode only): splits * tiles_m * tiles_n
// workgroups, each writing its fp32 partial tile; launch_splitk_finalize then sums them.
hipError_t launch_gemm_bigwave(const GemmParams& p, hipStream_t stream);

// The tiles of the four-wave kernel fed to 16 x 16 x 32 products (gemm_bigwave16.hip), every
// weight storage, K a multiple of 64: whole launches of 256 x 256 tiles, or of 256 x 128 tiles
// (p.narrow), tile sets of 256-row or 192-row tiles, (plain columns) 256 x 256 or 256 x 128 tiles
// cut along k into fp32 partials for launch_splitk_finalize (not persistent), or (plain columns)
// whole launches of 256 x 256 tiles with 16 appended rows (xr_row0).  Same results as
// launch_gemm_bigwave, bit for bit.
bool gemm_bigwave16_supports(const GemmParams& p);
hipError_t launch_gemm_bigwave16(const GemmParams& p, hipStream_t stream);

// Split-K kernel with 32*mb-row tiles (mb = 1, 2 or 4) of 128 weight columns, followed (splits > 1)
// by the kernel that sums the splits; tiles_m, tiles_n, splits, kt_per_split, ws and ws_ld set by
// the caller.
constexpr int kSkinnyCols = 128;  // weight columns per tile (64 act columns in SiLU·up mode)
constexpr int kSkinnyK = 64;      // k per pipeline stage
hipError_t launch_gemm_skinny(const GemmParams& p, int mb, hipStream_t stream);

// Split-free GEMM for at most 64 token rows with the weight stored [n][k] (p.w_nk), K a multiple of
// 32: one workgroup per 32 weight columns over the whole of k (its four waves cut k into quarters
// and add their sums through LDS), fragments loaded straight into registers; no workspace.
bool gemm_stream_nk_supports(const GemmParams& p);
int64_t gemm_stream_nk_workgroups(const GemmParams& p);
hipError_t launch_gemm_stream_nk(const GemmParams& p, hipStream_t stream);

// Sum of the p.splits fp32 partials in p.ws (ascending split order), then the epilogue of p.mode
// (SiLU·up: gate at workspace column j, up at column N + j), into p.C.
hipError_t launch_splitk_finalize(const GemmParams& p, hipStream_t stream);

// Rows [0, b) of the outputs; row i reads the partials at P + i*n + r*plane, r = 0..t-1.
constexpr int kMaxPeers = 16;  // partials passed as separate pointers (one per rank)

struct ReduceNormParams {
  const uint16_t* P;
  const uint16_t* residual;  // may be null
  const uint16_t* gamma;
  uint16_t* residual_out;
  uint16_t* Y;
  int64_t b, n;
  int64_t plane;             // elements between consecutive ranks' partials
  int32_t t;
  float eps;
  // peers != 0: rank r's partial of the call's row i is at peer[r] + i * n (t <= kMaxPeers), in
  // place of P + r * plane + i * n.
  int32_t peers;
  const uint16_t* peer[kMaxPeers];
};

hipError_t launch_reduce_rmsnorm(const ReduceNormParams& p, hipStream_t stream);

// W[k][n] row-major -> the blocked layout (64 x 128 blocks, 128-column strips); k % 64 == 0,
// n % 128 == 0, k * n < 2^31.
hipError_t launch_pack_blocked(const uint16_t* W, int64_t k, int64_t n, uint16_t* W_blk, hipStream_t stream);

}  // namespace ttl
