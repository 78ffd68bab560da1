// Tiled bf16 GEMM with one wave64 per SIMD and 256 x 256 tiles, fed to v_mfma_f32_16x16x32_bf16.
//
// Tiles, direct-to-LDS copies and the per-k-tile schedule are those of the four-wave kernel in
// gemm_bigwave.hip (32 x 32 x 16 products); a wave still owns 128 x 128 outputs, now as 8 x 8
// blocks of 16 x 16 (64 accumulators of four registers).  A slice is half a k32 step: slice s of a
// k-tile multiplies the k32 step s / 2 of the wave's row blocks 4 (s % 2) .. 4 (s % 2) + 3 by all
// eight column blocks, 32 products of 16 cycles, the length of a slice of the other kernel.  Each
// output sums the same products in the same k order as the 32 x 32 x 16 kernel, and the results
// agree with it bit for bit (tested).
//
// Both kernels keep the matrix cores equally busy per cycle (70B TP=8 row GEMM at 4096 tokens:
// 2.81-2.87 M active cycles per launch for either kernel and storage), but under the board's power
// cap this one runs at a higher clock: the 16 x 16 x 32 product moves fewer accumulator bytes per
// flop.  Measured on one box against the 32 x 32 x 16 kernel's best launch: 8 % faster on that row
// GEMM and on the SiLU·up column GEMM, with [k][n] or [n][k] weights.
//
// Weights stored [n][k] reach the products with plain 16-byte LDS reads, as the activations do.
// Weights stored [k][n] (plain or in 64 x 128 blocks) are staged [k][n] and read with
// ds_read_b64_tr_b16, two transposed half reads per fragment, joined at the product; their products
// (and, in the instances with appended rows, every storage's) are written out as asm with the
// accumulator tied in place (see mfma_one).
//
// Per k-tile t and wave (order pinned with scheduling barriers):
//   slice 0: 32 MFMAs, with the LDS reads of slice 2 of tile t (its row blocks and the weight
//            fragments of k32 step 1), and in the instances whose products are asm also those of
//            slice 3, so that no read is still in flight at the barrier;
//   slice 1: 32 MFMAs, with (builtin products) the reads of slice 3 (its row blocks); with asm
//            products, a workgroup barrier after the eighth MFMA (every wave's reads of tile t have
//            returned, so its stage is free) and then the first direct-to-LDS copies of tile t+2;
//   barrier: the wave waits for its own copies of tile t+1; the workgroup barrier publishes tile
//            t+1 (and, with builtin products, certifies that every wave's reads of tile t returned);
//   slice 2: 32 MFMAs, reads of slice 0 of tile t+1 (row-block and weight fragments of its first
//            k32 step), and copies of tile t+2: spread evenly from the first barrier to the end of
//            slice 3 with asm products, otherwise half of them, one after every fourth MFMA;
//   slice 3: 32 MFMAs, reads of slice 1 of tile t+1, the other copies.
// Lane layouts (weight fragment as the first operand, so each lane ends with four consecutive
// output columns of one output row): first operand lane l holds weight column l % 16 of the block
// and k = 8 (l / 16) .. + 7 of the k32 step; second operand lane l holds activation row l % 16 and
// the same k; accumulator register r of lane l is output row l % 16, column 4 (l / 16) + r.
//
// K must be a multiple of 64.  Whole launches of 256 x 256 tiles, tile sets of 256-row or 192-row
// tiles (the planner's cut of a launch whose last round is partly idle), 256 x 256 tiles with 16
// appended rows, or 256 x 256 tiles cut along k (plain columns: fp32 partial tiles for the split-K
// finalize kernel).  Narrow tiles (256 x 128, a wave owning 128 x 64 outputs as 8 x 4 blocks, 16
// products per slice) serve launches whose 256 x 256 tiles would fill too few CUs, whole or cut
// along k.
#include <type_traits>

#include "gemm_common.h"

namespace ttl {
namespace {

using namespace gemm;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 64;
constexpr int kChunks = kBK / 8;         // 16-B chunks per staged [rows][k] row
constexpr int kRowsPer256 = 256 / (2 * kBK);
constexpr int kRowsPerCopy = 1024 / (2 * kBK);
constexpr int kStages = 2;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPartials = 2;  // kernel mode: plain columns, fp32 partial tile of a k split to the workspace

// Slot permutation of a staged [k][n] row (32 chunks of 16 bytes, or 16 for narrow tiles; either
// row is a whole number of bank cycles): chunk c of k row r sits at slot c ^ kn_swizzle(r).  A transposed weight read covers 4 consecutive k rows in each 16-lane group,
// and the two groups of a half-wave are 8 rows apart at the same columns: 4 (r % 4) spreads the 4
// rows of a group over the banks, 2 ((r / 8) % 2) puts the other group on the other half of them,
// so that the 32 lanes of a half-wave read 256 distinct bytes (without the second term every read
// was a two-way bank conflict: 15x the conflict cycles of the [n][k] reads, 70B TP=8 row GEMM).
__host__ __device__ constexpr int kn_swizzle(int r) { return (4 * (r % 4)) ^ (2 * ((r >> 3) & 1)); }

// MODE: kPlain (bf16 outputs), kSiluMul, or kPartials (plain columns; workgroup split * tiles + tile
// runs k-tiles [split * kt_per_split, ...) of its tile and writes the fp32 partial tile to workspace
// slice `split`, which the split-K finalize kernel sums in split order).  WNK: weights stored
// [n][k]; otherwise [k][n], in 64 x 128 blocks when BLK.  BM rows per tile: 256, or 192 (96 per
// wave) for the last round of a launch whose 256-row tiles would leave that round partly idle.
// XR (plain 256-row tiles): 16 appended rows per tile, from row p.xr_row0 + 16 tile_m (see below).
// WN weight columns per wave: 128 (256-column tiles), or 64 (narrow: 256 x 128 tiles, 256-row).
template <int MODE, bool WNK, bool BLK, int BM, bool XR, int WN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_bigwave16_kernel(const GemmParams p) {
  static_assert(!(WNK && BLK), "blocked storage is a [k][n] storage");
  static_assert(BM == 256 || BM == 192, "tile heights built: 256 and 192");
  static_assert(MODE != kPartials || BM == 256, "k splits: 256-row tiles");
  static_assert(!XR || (MODE == kPlain && BM == 256 && WN == 128), "appended rows: plain 256 x 256 tiles");
  static_assert(WN == 128 || (WN == 64 && BM == 256), "narrow tiles: 256 rows");
  constexpr int kWN = WN, kBN = 2 * WN;
  constexpr int kNB = kWN / 16;                          // 16-column blocks per wave: 8 or 4
  constexpr int kBElems = kBK * kBN;
  constexpr int kBCopies = kBElems * 2 / 1024 / kWaves;  // 8 or 4
  constexpr int kBChunks = kBN / 8;                      // 16-B chunks per staged [k][n] row: 32 or 16
  constexpr int kKRowsPerCopy = 64 / kBChunks;           // k rows per 1-KiB copy of a [k][n] stage: 2 or 4
  constexpr int kBM = BM, kWM = BM / 2;
  constexpr int kMB = kWM / 16;                          // 16-row blocks per wave: 8 or 6
  constexpr int kMpsl = (kMB / 2) * kNB;                 // MFMAs per slice: 32, 24 or 16
  constexpr int kAMain = kBM * kBK;                      // the tile's own A rows in a stage
  constexpr int kAElems = kAMain + (XR ? 16 * kBK : 0), kStageElems = kAElems + kBElems;
  constexpr int kACopies = kAMain * 2 / 1024 / kWaves;   // 8 or 6
  constexpr int kCopies = kACopies + kBCopies;
  // Products written as asm with the accumulator tied in place (see mfma_one): [k][n] weights, and
  // every storage with appended rows.
  constexpr bool kAsm = !WNK || XR;
  // Where a k-tile's copies go.  With asm products every read of tile t's stage is issued by the end
  // of slice 0, so a second barrier, kB1 products into slice 1, frees that stage for tile t+2's
  // copies, and they spread over the rest of slices 1-3 (about 2.5 % fewer active cycles than in
  // slices 2-3 alone for the 70B TP=8 [k][n] GEMMs at 4096 tokens; the barrier's position measured
  // best at 8 of 2-20); otherwise they follow the barrier after slice 1.
  constexpr bool kSplitBarrier = kAsm;
  constexpr int kB1 = 8;
  static_assert(kB1 < kMpsl, "the first barrier sits inside slice 1");
  constexpr int kCopy0 = kSplitBarrier ? kMpsl + kB1 + 1 : 2 * kMpsl, kCopySpan = 4 * kMpsl - kCopy0;
  constexpr int kCopiesS1 = [] {
    int n = 0;
    for (int c = 0; c < kCopies; ++c) n += kCopy0 + (c + 1) * kCopySpan / kCopies - 1 < 2 * kMpsl;
    return n;
  }();
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kStages * kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / 2, wn = wave % 2;

  // Tile sets (p.rects > 0): block b < rect_tmc[0] * rect_tnc[0] is a tile of rectangle 0, the
  // rest of rectangle 1; rectangle i is rect_tmc[i] row-tiles from row rect_row0[i] by rect_tnc[i]
  // tile columns from tile column rect_tn0[i], walked in groups of rect_group[i] row-tiles.
  const int tiles = p.tiles_m * p.tiles_n;
  const int split = MODE == kPartials ? (int)blockIdx.x / tiles : 0;
  int tile_m, tile_n, row0 = 0;
  {
    const int bid = (int)blockIdx.x - split * tiles;
    if (p.rects > 0) {
      const int c0 = p.rect_tmc[0] * p.rect_tnc[0];
      const bool second = p.rects > 1 && bid >= c0;
      const int tmc = second ? p.rect_tmc[1] : p.rect_tmc[0];
      const int tnc = second ? p.rect_tnc[1] : p.rect_tnc[0];
      const int group = second ? p.rect_group[1] : p.rect_group[0];
      tile_coords(bid - (second ? c0 : 0), tmc, tnc, tile_m, tile_n, group > 0 ? group : 4);
      tile_n += second ? p.rect_tn0[1] : p.rect_tn0[0];
      row0 = second ? p.rect_row0[1] : p.rect_row0[0];
    } else {
      tile_coords(bid, p.tiles_m, p.tiles_n, tile_m, tile_n);
    }
  }
  const int m0 = row0 + tile_m * kBM;
  const int n0 = tile_n * (MODE == kSiluMul ? kBN / 2 : kBN);
  // Appended rows (XR): staged below the tile's 256 A rows as rows 256 .. 271; rows at or past M read
  // zeros (a tile may have none).  The wave in row half wm computes them against its column blocks
  // 2 wm, 2 wm + 1, 2 wm + 4, 2 wm + 5: with XR a wave holds its weight fragments in the order
  // ni ^ nperm, so that these are its fragments 0, 1, 4 and 5 in every wave.
  const int xm0 = XR ? p.xr_row0 + tile_m * 16 : 0;
  const int nperm = XR ? 2 * wm : 0;
  const int kt0 = split * p.kt_per_split;
  const int nk = MODE == kPartials ? min(p.kt_per_split, p.K / kBK - kt0) : p.K / kBK;  // >= 1
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds);

  // ---- Copy offsets.  Copy i < kACopies (8, or 6 for 192-row tiles) of this wave moves block
  // kACopies*wave + i of the A stage: rows 8 (kACopies wave + i) + l/8, whose swizzle depends on i
  // only through i % 2, so two offset registers serve all of them (the rest, 16 (i / 2) rows, goes
  // in the copy's scalar offset; rows past M lie beyond the descriptor's range and read zeros).
  // Copy kACopies + i moves block 8*wave + i of the B stage: with [n][k] weights the weight rows
  // (output columns) 8 (8 wave + i) + l/8, through the column map, which may jump between
  // segments, so each has its own offset register.
  uint32_t a_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int row = (kACopies * wave + par) * kRowsPerCopy + lane / kChunks;
    const int chunk = (lane % kChunks) ^ ((row / kRowsPer256) % kChunks);
    a_off[par] = (uint32_t)(((int64_t)row * p.lda + chunk * 8) * 2);
  }
  uint32_t b_off[kBCopies];
#pragma unroll
  for (int i = 0; i < kBCopies; ++i) {
    const int q = kBCopies * wave + i;
    bool ok;
    if constexpr (WNK) {
      const int n = q * kRowsPerCopy + lane / kChunks;
      const int chunk = (lane % kChunks) ^ ((n / kRowsPer256) % kChunks);
      const int64_t wrow = weight_column<MODE, kWN>(p, n0, n & ~7, ok) + (n & 7);
      b_off[i] = ok ? (uint32_t)((wrow * p.ldb + chunk * 8) * 2) : kOob;
    } else {
      // [64 k][256 n]: block q holds k rows 2q, 2q + 1; lane l lands in row 2q + l/32 at slot l%32,
      // which holds n-chunk slot ^ kn_swizzle(row).
      const int krow = kKRowsPerCopy * q + lane / kBChunks;
      const int chunk = (lane % kBChunks) ^ kn_swizzle(krow);
      const int64_t wcol = weight_column<MODE, kWN>(p, n0, chunk * 8, ok);
      b_off[i] = !ok ? kOob
                 : BLK ? blocked_offset(krow, wcol, p.ldb)
                           : (uint32_t)(((int64_t)krow * p.ldb + wcol) * 2);
    }
  }
  // A copy i sits 16 (i / 2) rows past copy i % 2.
  const uint32_t a_step2 = (uint32_t)(2 * kRowsPerCopy * p.lda * 2);
  auto a_desc = [&](int t) {
    const int k0 = (kt0 + t) * kBK;
    return buffer_desc(p.A + (int64_t)m0 * p.lda + k0, ((int64_t)(p.M - m0 - 1) * p.lda + (p.K - k0)) * 2);
  };
  // Appended rows: waves 0 and 1 each copy 8 of the 16 (one 1-KiB copy per k-tile), laid out as A.
  uint32_t x_off = 0;
  if constexpr (XR) {
    const int row = kRowsPerCopy * (wave & 1) + lane / kChunks;
    const int chunk = (lane % kChunks) ^ ((row / kRowsPer256) % kChunks);
    x_off = (uint32_t)(((int64_t)row * p.lda + chunk * 8) * 2);
  }
  auto x_desc = [&](int t) {
    const int k0 = (kt0 + t) * kBK;
    return buffer_desc(p.A + (int64_t)xm0 * p.lda + k0, ((int64_t)(p.M - xm0 - 1) * p.lda + (p.K - k0)) * 2);
  };
  auto b_desc = [&](int t) {
    const int k0 = (kt0 + t) * kBK;
    return WNK ? buffer_desc(p.B + k0, ((int64_t)(p.b_rows - 1) * p.ldb + (p.K - k0)) * 2)
           : BLK ? blocked_desc(p.B, p.b_rows, k0)
                     : buffer_desc(p.B + (int64_t)k0 * p.ldb, (int64_t)(p.K - k0) * p.ldb * 2);
  };
  const uint32_t wave_lds_a = lds0 + (uint32_t)(wave * kACopies * 1024);
  const uint32_t wave_lds_b = lds0 + (uint32_t)(kAElems * 2 + wave * kBCopies * 1024);
  auto copy_one = [&](int t, int i, i32x4_t ad, i32x4_t bd) {
    const uint32_t so = (uint32_t)(((unsigned)t % kStages) * kStageElems * 2);
    if (i < kACopies) {
      copy16_to_lds_so(ad, a_off[i % 2], (uint32_t)(i / 2) * a_step2, wave_lds_a + so, i * 1024);
    } else {
      copy16_to_lds_at(bd, b_off[i - kACopies], wave_lds_b + so, (i - kACopies) * 1024);
    }
  };
  const bool x_copier = XR && wave < 2;
  auto copy_x = [&](int t, i32x4_t xd) {
    const uint32_t so = (uint32_t)(((unsigned)t % kStages) * kStageElems * 2);
    copy16_to_lds_at(xd, x_off, lds0 + so + (uint32_t)(kAMain * 2 + (wave & 1) * 1024), 0);
  };
  auto copy_tile = [&](int t) {
    const i32x4_t ad = a_desc(t), bd = b_desc(t);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy_one(t, i, ad, bd);
    if (x_copier) copy_x(t, x_desc(t));
  };

  // ---- Fragment offsets (elements within a stage).
  // [rows][64 k] staging (A, and B: weight rows): row r, k-chunk c at slot c ^ ((r/2) % 8).
  // Lane l reads row (l % 16) of its block at k-chunk 4 * step + l / 16.
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int rsw = (r16 / kRowsPer256) % kChunks;  // the row's swizzle term (blocks start at multiples of 16 rows)
  int ra_off[2], rb_off[2][2], rx_off[2];
#pragma unroll
  for (int step = 0; step < 2; ++step) {
    const int slot = (4 * step + g4) ^ rsw;
    ra_off[step] = (wm * kWM + r16) * kBK + slot * 8;
    rx_off[step] = kAMain + r16 * kBK + slot * 8;
    // fragment ni reads block ni ^ nperm: ni + nperm where bit 1 of ni is clear, ni - nperm where set
    rb_off[step][0] = kAElems + (wn * kWN + r16) * kBK + slot * 8 + nperm * 16 * kBK;
    rb_off[step][1] = kAElems + (wn * kWN + r16) * kBK + slot * 8 - nperm * 16 * kBK;
  }
  // [64 k][256 n] staging, read with ds_read_b64_tr_b16 (each 16-lane group receives the transpose
  // of a 4 (k) x 16 (n) block): group g = lane/16 reads k row 32 step + 8 g + 4 h + (lane%16)/4 of
  // half h at n = 128 wn + 16 ni + 4 (lane%4), i.e. chunk 16 wn + 2 ni + (lane%4)/2, stored at slot
  // chunk ^ kn_swizzle(k) = chunk ^ 4 ((lane%16)/4) ^ 2 (g%2).
  int rt_off[kNB];
  {
    const int krow = 8 * g4 + (r16 >> 2);
    const int x = kn_swizzle(krow);
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni)
      rt_off[ni] = kAElems + krow * kBN + (((kWN / 8) * wn + 2 * (ni ^ nperm) + ((lane & 3) >> 1)) ^ x) * 8 + 4 * (lane & 1);
  }
  bf16x8_t af[4][kMB / 2], bv[2][kNB], afx[2];
  i16x4_t bl[2][kNB], bh[2][kNB];
  // Reads of slice s: j < 4 are its row-block fragments; an even slice also reads its step's eight
  // weight fragments and (XR) the appended rows' fragment.
  constexpr int kBReads = kNB + (XR ? 1 : 0);
  auto reads_of = [](int s) { return kMB / 2 + (s % 2 == 0 ? kBReads : 0); };
  auto read_one = [&](int t, int s, int j) {
    const uint16_t* st = lds + ((unsigned)t % kStages) * kStageElems;
    const int step = s / 2;
    if (j < kMB / 2) {
      const int mb = (s % 2) * (kMB / 2) + j;
      af[s][j] = *reinterpret_cast<const bf16x8_t*>(st + ra_off[step] + mb * 16 * kBK);
    } else if (XR && j == kMB / 2 + kNB) {
      afx[step] = *reinterpret_cast<const bf16x8_t*>(st + rx_off[step]);
    } else if constexpr (WNK) {
      const int ni = j - kMB / 2;
      bv[step][ni] = *reinterpret_cast<const bf16x8_t*>(st + rb_off[step][(ni >> 1) & 1] + ni * 16 * kBK);
    } else {
      // the two transposed halves (k 8 g .. + 3 and + 4 .. + 7), joined at once into the fragment
      const int ni = j - kMB / 2;
      const uint16_t* b = st + rt_off[ni] + step * 32 * kBN;
      bl[step][ni] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b));
      bh[step][ni] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + 4 * kBN));
    }
  };

  f32x4_t acc[kMB][kNB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mb][ni][r] = 0.0f;
  // Appended rows' accumulators (XR), in vector registers (the accumulation registers are full):
  // accx[e] is that row block against fragment 4 (e / 2) + e % 2.
  f32x4_t accx[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) accx[e][r] = 0.0f;
  if constexpr (kAsm) {
    // The zeros are placed in the accumulation registers here (the empty statements take them as
    // operands), and a vector write of a register read as a product's accumulator must lead it by
    // two wait states: the nops give several.
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni) asm volatile("" : "+a"(acc[mb][ni]));
    if constexpr (XR) {
#pragma unroll
      for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(accx[e]));
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7");
    __builtin_amdgcn_sched_barrier(0);
  }


  // MFMA j (0 .. 31) of slice s: row block 4 (s % 2) + j / 8, column block j % 8.
  auto mfma_one = [&](int s, int j) {
    const int ml = j / kNB, ni = j % kNB, mb = (s % 2) * (kMB / 2) + ml, step = s / 2;
    bf16x8_t b;
    if constexpr (WNK) b = bv[step][ni];
    else b = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(bl[step][ni], bh[step][ni], 0, 1, 2, 3, 4, 5, 6, 7));
    if constexpr (!kAsm) {
      acc[mb][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, af[s][ml], acc[mb][ni], 0, 0, 0);
    } else {
      // Written out, with the accumulator as one read-write operand: through the builtin, the
      // register allocator gave some products' accumulator input and output different registers
      // and moved those accumulators through other registers every k-tile (the two-read weight
      // fragments, or the appended rows' registers, leave it less room).  The compiler does not see this as a matrix instruction,
      // so the waits it would insert around one are made explicit (before the first product and
      // after the last); the products' operands come from LDS reads, whose waits it does insert.
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[mb][ni]) : "v"(b), "v"(af[s][ml]));
    }
  };
  // Appended rows (XR): product e2 (0, 1) of slice s, the k32 step s / 2 of the appended row block
  // against fragment 4 (s % 2) + e2 (two per slice, after the slice's own).
  auto mfma_x = [&](int s, int e2) {
    const int e = 2 * (s % 2) + e2, ni = 4 * (s % 2) + e2, step = s / 2;
    bf16x8_t b;
    if constexpr (WNK) b = bv[step][ni];
    else b = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(bl[step][ni], bh[step][ni], 0, 1, 2, 3, 4, 5, 6, 7));
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(accx[e]) : "v"(b), "v"(afx[step]));
  };
  auto slice_x = [&](int s) {
    if constexpr (XR) {
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        mfma_x(s, e2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- Prologue: tiles 0 and 1 in flight, tile 0 landed, slices 0 and 1 of tile 0 read.
  copy_tile(0);
  if (nk >= 2) {
    copy_tile(1);
    if (x_copier) wait_vmcnt<kCopies + 1>();
    else wait_vmcnt<kCopies>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
#pragma unroll
  for (int j = 0; j < reads_of(0); ++j) read_one(0, 0, j);
#pragma unroll
  for (int j = 0; j < reads_of(1); ++j) read_one(0, 1, j);
  __builtin_amdgcn_sched_barrier(0);

  // One k-tile (NEXT: tile t+1 exists; COPY: tile t+2 exists); reads spread evenly over the slots.
  auto k_tile = [&](int t, auto next_c, auto copy_c) {
    constexpr bool NEXT = decltype(next_c)::value, COPY = decltype(copy_c)::value;
    // slice 0: reads of slice 2 of tile t (its row blocks and the weight fragments of step 1);
    // slice 1: reads of slice 3 (row blocks only).  With asm products the reads of slice 3 are
    // issued in slice 0 too: the barrier after slice 1 waits for every read of the wave, and the
    // last of them no longer trails the slice (70B TP=8 at 4096 tokens, [k][n] weights, medians of
    // 8 alternating runs: SiLU·up 358.3 -> 355.6 us, row GEMM 179.8 -> 176.6 us; with the builtin
    // products the longer-lived fragments made the allocator move accumulators: [n][k] 447.7 us).
    constexpr int kR0 = kMB / 2 + kBReads, kR1 = kMB / 2;
    constexpr int kRS0 = kAsm ? kR0 + kR1 : kR0, kRS1 = kAsm ? 0 : kR1;
#pragma unroll
    for (int j = 0; j < kMpsl; ++j) {
      mfma_one(0, j);
#pragma unroll
      for (int r = j * kRS0 / kMpsl; r < (j + 1) * kRS0 / kMpsl; ++r) {
        if (r < kR0) read_one(t, 2, r);
        else read_one(t, 3, r - kR0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    slice_x(0);
    // The descriptors of tile t+2's copies are built between slice 1's first products.  Copy c
    // follows slot kCopy0 + (c + 1) kCopySpan / kCopies - 1 of the k-tile's 4 kMpsl product slots.
    i32x4_t ad = {0, 0, 0, 0}, bd = {0, 0, 0, 0}, xd = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kMpsl; ++j) {
      mfma_one(1, j);
#pragma unroll
      for (int r = j * kRS1 / kMpsl; r < (j + 1) * kRS1 / kMpsl; ++r) read_one(t, 3, r);
      if (COPY) {
        if (j == 0) ad = a_desc(t + kStages);
        if (j == 1) bd = b_desc(t + kStages);
        if (XR && j == 2) xd = x_desc(t + kStages);
        // every read of tile t's stage was issued in slice 0: once all have returned, in every
        // wave, tile t+2's copies may overwrite it
        if (kSplitBarrier && j == kB1) lds_barrier();
#pragma unroll
        for (int c = 0; c < kCopies; ++c)
          if (kCopy0 + (c + 1) * kCopySpan / kCopies - 1 == kMpsl + j) copy_one(t + kStages, c, ad, bd);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    slice_x(1);
    if (NEXT) {
      // this wave's copies of tile t+1 landed (those of tile t+2 issued in slice 1 are the last
      // kCopiesS1 copies), then everyone's; and every wave's reads of tile t returned
      if (COPY) wait_vmcnt<kCopiesS1>();
      else wait_vmcnt<0>();
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // slice 2: reads of slice 0 of tile t+1 and copies
    constexpr int kR2 = kMB / 2 + kBReads;
#pragma unroll
    for (int j = 0; j < kMpsl; ++j) {
      mfma_one(2, j);
      if (COPY) {
#pragma unroll
        for (int c = 0; c < kCopies; ++c)
          if (kCopy0 + (c + 1) * kCopySpan / kCopies - 1 == 2 * kMpsl + j) copy_one(t + kStages, c, ad, bd);
        if (j == kMpsl - 1 && x_copier) copy_x(t + kStages, xd);
      }
      if (NEXT) {
#pragma unroll
        for (int r = j * kR2 / kMpsl; r < (j + 1) * kR2 / kMpsl; ++r) read_one(t + 1, 0, r);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    slice_x(2);
    // slice 3: reads of slice 1 of tile t+1, the other copies
    constexpr int kR3 = kMB / 2;
#pragma unroll
    for (int j = 0; j < kMpsl; ++j) {
      mfma_one(3, j);
      if (COPY) {
#pragma unroll
        for (int c = 0; c < kCopies; ++c)
          if (kCopy0 + (c + 1) * kCopySpan / kCopies - 1 == 3 * kMpsl + j) copy_one(t + kStages, c, ad, bd);
      }
      if (NEXT) {
#pragma unroll
        for (int r = j * kR3 / kMpsl; r < (j + 1) * kR3 / kMpsl; ++r) read_one(t + 1, 1, r);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    slice_x(3);
  };
  int t = 0;
  for (; t + kStages < nk; ++t) k_tile(t, std::true_type{}, std::true_type{});
  if (t + 1 < nk) k_tile(t++, std::true_type{}, std::false_type{});
  k_tile(t, std::false_type{}, std::false_type{});
  if constexpr (kAsm) {
    // A product's results may be read by other vector instructions only some wait states after
    // it (about its pass count plus two; 8 passes here): 32 before the epilogue reads.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 15\n\ts_nop 15");
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- Epilogue: lane l holds output row 16 mb + l % 16 and columns 16 ni + 4 (l / 16) .. + 3, so
  // direct stores would write 32-byte pieces of 16 rows per instruction.  Instead each wave writes
  // 32 rows (two row blocks) at a time into its own quarter of the free ring stage and reads them
  // back as whole rows: each store instruction then covers 4 rows of 256 bytes (8 of 128 bytes
  // for SiLU·up).  The stage of the k-tile before the last is free (every read of it returned
  // before that k-tile's barrier; with one k-tile, stage 1 was never used); the quarter is the
  // wave's alone and its LDS accesses complete in order, so no barrier is needed.  Chunk c (16
  // bytes) of staged row r sits at slot c ^ (r % chunks per row).  Output stores carry the
  // non-temporal hint (written once, for a later launch); fp32 partial tiles do not, as the split-K
  // finalize reads them right after (70B TP=8 layer qkv, 5 k splits: 61.5 -> 60.1 us).
  uint16_t* stg = lds + ((unsigned)(t + 1) % kStages) * kStageElems + wave * (kStageElems / kWaves);
  const int wrow0 = m0 + wm * kWM;
  auto drain = [&](auto ch_c, int pass, int col0) {
    constexpr int CH = decltype(ch_c)::value;
    constexpr int kRowsPerRead = 64 / CH;
#pragma unroll
    for (int i = 0; i < 32 / kRowsPerRead; ++i) {
      const int r = i * kRowsPerRead + lane / CH, c = lane % CH;
      const i32x4_t v = *reinterpret_cast<const i32x4_t*>(stg + r * CH * 8 + ((c ^ (r % CH)) * 8));
      const int row = wrow0 + pass * 32 + r, col = col0 + c * 8;
      if (row < p.M && col < p.N) __builtin_nontemporal_store(v, reinterpret_cast<i32x4_t*>(p.C + (int64_t)row * p.ldc + col));
    }
  };
#pragma unroll
  for (int pass = 0; pass < kMB / 2; ++pass) {
    if constexpr (MODE == kPartials) {
      // fp32 partial tile: chunk c (16 bytes) of a staged row holds columns 4c .. 4c+3; lane l holds
      // columns 16 ni + 4 (l / 16) .. + 3, chunk 4 ni + l / 16.
      constexpr int CH = kWN / 4;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ni = 0; ni < kNB; ++ni) {
          const int mb = 2 * pass + h, r = 16 * h + r16, c = 4 * ni + g4;
          *reinterpret_cast<f32x4_t*>(stg + r * CH * 8 + ((c ^ (r % CH)) * 8)) = acc[mb][ni];
        }
      float* wbase = p.ws + (int64_t)split * p.M * p.ws_ld + n0 + wn * kWN;
      constexpr int kRowsPerRead = 64 / CH;
#pragma unroll
      for (int i = 0; i < 32 / kRowsPerRead; ++i) {
        const int r = i * kRowsPerRead + lane / CH, c = lane % CH;
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(stg + r * CH * 8 + ((c ^ (r % CH)) * 8));
        const int row = wrow0 + pass * 32 + r;
        if (row < p.M) *reinterpret_cast<i32x4_t*>(wbase + (int64_t)row * p.ws_ld + c * 4) = v;
      }
    } else if (MODE == kPlain) {
      constexpr int CH = kWN / 8;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ni = 0; ni < kNB; ++ni) {
          const int mb = 2 * pass + h, r = 16 * h + r16, c = 2 * (ni ^ nperm) + g4 / 2;
          u32x2_t v;
          v.x = pack_bf16x2(acc[mb][ni][0], acc[mb][ni][1]);
          v.y = pack_bf16x2(acc[mb][ni][2], acc[mb][ni][3]);
          *reinterpret_cast<u32x2_t*>(stg + r * CH * 8 + ((c ^ (r % CH)) * 8) + 4 * (g4 % 2)) = v;
        }
      drain(std::integral_constant<int, CH>{}, pass, n0 + wn * kWN);
    } else {
      // column blocks 0..3 are the gate columns and 4..7 the up columns of the same act columns
      constexpr int CH = kWN / 16;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ni = 0; ni < kNB / 2; ++ni) {
          const int mb = 2 * pass + h, r = 16 * h + r16, c = 2 * ni + g4 / 2;
          float a[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = silu_mul(acc[mb][ni][e], acc[mb][ni + kNB / 2][e]);
          u32x2_t v;
          v.x = pack_bf16x2(a[0], a[1]);
          v.y = pack_bf16x2(a[2], a[3]);
          *reinterpret_cast<u32x2_t*>(stg + r * CH * 8 + ((c ^ (r % CH)) * 8) + 4 * (g4 % 2)) = v;
        }
      drain(std::integral_constant<int, CH>{}, pass, n0 + wn * (kWN / 2));
    }
  }
  if constexpr (XR) {
    // Appended rows, straight from the registers: lane l holds row xm0 + l % 16 and, for accx[e],
    // the four columns from 16 ((4 (e / 2) + e % 2) ^ nperm) + 4 (l / 16) of the wave's 128.
    const int row = xm0 + r16;
    if (row < p.M) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = n0 + wn * kWN + 16 * ((4 * (e / 2) + e % 2) ^ nperm) + 4 * g4;
        if (col < p.N) {
          u32x2_t v;
          v.x = pack_bf16x2(accx[e][0], accx[e][1]);
          v.y = pack_bf16x2(accx[e][2], accx[e][3]);
          *reinterpret_cast<u32x2_t*>(p.C + (int64_t)row * p.ldc + col) = v;
        }
      }
    }
  }
}

template <int MODE, int BM, bool XR = false, int WN = 128>
void launch_one16(const GemmParams& p, hipStream_t stream) {
  const int blocks = p.rects > 0 ? p.rect_tmc[0] * p.rect_tnc[0] + (p.rects > 1 ? p.rect_tmc[1] * p.rect_tnc[1] : 0)
                                 : (p.splits > 1 ? p.splits : 1) * p.tiles_m * p.tiles_n;
  const dim3 grid((unsigned)blocks);
  if (p.w_nk) hipLaunchKernelGGL((gemm_bigwave16_kernel<MODE, true, false, BM, XR, WN>), grid, dim3(kThreads), 0, stream, p);
  else if (p.w_blk) hipLaunchKernelGGL((gemm_bigwave16_kernel<MODE, false, true, BM, XR, WN>), grid, dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL((gemm_bigwave16_kernel<MODE, false, false, BM, XR, WN>), grid, dim3(kThreads), 0, stream, p);
}

template <int BM, int WN = 128>
void launch_rows16(const GemmParams& p, hipStream_t stream) {
  if (p.mode == kSiluMul) launch_one16<kSiluMul, BM, false, WN>(p, stream);
  else launch_one16<kPlain, BM, false, WN>(p, stream);
}

}  // namespace

bool gemm_bigwave16_supports(const GemmParams& p) {
  // Tile sets with 256-row or 192-row tiles, or whole launches of 256-row tiles, or (plain columns)
  // 256-row tiles cut along k, or (plain columns) whole launches of 256-row tiles with appended rows;
  // narrow (256 x 128) tiles as whole launches, or (plain columns) cut along k.
  const bool rows_ok = p.rects > 0 ? (p.tile_rows == 256 || p.tile_rows == 192) : (p.tile_rows == 0 || p.tile_rows == 256);
  const bool splits_ok = p.splits <= 1 || (p.rects == 0 && p.mode == kPlain && p.kt_per_split > 0);
  const bool xr_ok = p.xr_row0 == 0 || (p.xr_row0 > 0 && p.mode == kPlain && p.rects == 0 && p.splits <= 1);
  const bool narrow_ok = !p.narrow || (p.rects == 0 && p.xr_row0 == 0);
  return p.K % kBK == 0 && p.K > 0 && splits_ok && xr_ok && narrow_ok && p.persist == 0 && rows_ok;
}

hipError_t launch_gemm_bigwave16(const GemmParams& p, hipStream_t stream) {
  if (!gemm_bigwave16_supports(p)) return hipErrorInvalidValue;
  if (p.splits > 1) {
    if (p.ws == nullptr || p.ws_ld < (int64_t)p.tiles_n * (p.narrow ? 128 : 256)) return hipErrorInvalidValue;
    if (p.narrow) launch_one16<kPartials, 256, false, 64>(p, stream);
    else launch_one16<kPartials, 256>(p, stream);
  }
  else if (p.narrow) launch_rows16<256, 64>(p, stream);
  else if (p.xr_row0 > 0) launch_one16<kPlain, 256, true>(p, stream);
  else if (p.tile_rows == 192) launch_rows16<192>(p, stream);
  else launch_rows16<256>(p, stream);
  return hipGetLastError();
}

}  // namespace ttl
