// Tiled bf16 GEMM with one wave64 per SIMD: 256 x 256 tiles, four waves of 128 x 128 outputs each
// (WN = 128), or 256 x 128 tiles of 128 x 64 per wave (WN = 64) for launches whose wide tiles
// would leave much of the chip idle.
//
// C[M, N] = A[M, K] · B[K, map(N)] with the operands, column maps, LDS layouts and M/N tails of the
// eight-wave kernel in gemm_bf16.hip; what differs is how the matrix cores are fed.  A wave owning
// 128 x 128 outputs keeps 16 v_mfma_f32_32x32x16_bf16 accumulators (256 registers, in the
// accumulation registers) and reads 4 A + 4 B fragments per 16 MFMAs: a third fewer LDS bytes per
// product than the 128 x 64 waves of the eight-wave kernel.  With one wave per SIMD its
// 512-register budget also holds the fragments of all four k16 slices of a k-tile, so LDS reads
// can run two slices (~1000 cycles) ahead of their MFMAs.
//
// With no second wave on the SIMD to hide stalls, everything is placed explicitly (the order below
// is pinned with scheduling barriers).  Per k-tile t and wave (4 slices of 16 MFMAs):
//   slice 0: MFMAs of slice 0, with the LDS reads of slices 2 and 3 of tile t;
//   slice 1: MFMAs of slice 1;
//   barrier: the wave waits for its own copies of tile t+1, then the workgroup barrier publishes
//            tile t+1 and certifies that every wave's reads of tile t have returned;
//   slice 2: MFMAs, reads of slice 0 of tile t+1, and half of the direct-to-LDS copies of tile
//            t+kStages (into tile t's stage, now free), one after every second MFMA;
//   slice 3: MFMAs, reads of slice 1 of tile t+1, the other half of the copies.
// With two stages (WN = 128) the copies of a tile have until the next barrier (two slices and
// more) to land; the WN = 64 tiles' k-tiles take half as long, so they use three stages.  Measured
// alternatives: a copy after every MFMA of one slice starves the wave's matrix core (the copies'
// issue blocks it); copies spread over all four slices (B staged three-deep to allow it) or moved
// before the barrier were slower; k-tiles of 32 with a five-stage ring were slower still (twice the
// L2 requests for the same bytes).
//
// K must be a multiple of 64 (no k tail); the eight-wave kernel serves the other shapes.
//
// Split-K launches (few tiles, long K: the qkv and o_proj shards at prefill sizes): workgroup
// split * tiles + tile runs k-tiles [split * kt_per_split, ...) of its tile and writes the fp32
// partial tile to the workspace (the kPartials mode: plain columns; SiLU·up runs as the gate
// columns then the up columns), which the split-K finalize kernel sums in split order.
//
// Outputs leave through LDS: each wave stages 32 rows at a time in a free ring stage and stores
// whole rows (see the epilogue below), which took about 5 us off every launch of 256 tiles against
// storing straight from the accumulators (70B TP=8 row GEMM, [n][k] weights: 169 -> 162 us).
#include <type_traits>

#include "gemm_common.h"

namespace ttl {
namespace {

using namespace gemm;

constexpr int kPartials = 2;  // kernel mode: plain columns, fp32 partial tile to the split-K workspace

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 64;
constexpr int kKK = kBK / 16;            // k16 slices per k-tile
constexpr int kChunks = kBK / 8;         // 16-B chunks per staged [rows][k] row
constexpr int kRowsPer256 = 256 / (2 * kBK);
constexpr int kRowsPerCopy = 1024 / (2 * kBK);

static_assert(kKK == 4, "the slice schedule assumes four k16 slices per k-tile");

// WN output columns per wave: 128 (256 x 256 tiles) or 64 (256 x 128 tiles, for launches that
// have too few 256 x 256 tiles to fill the chip).  The B stage holds 64 k rows of the tile's
// 2 * WN weight columns.  BM rows per tile: 256, or 192 (96 per wave) for the last round of a
// launch whose 256-row tiles would leave that round partly idle.
// MODE: kPlain (bf16 outputs), kSiluMul, or kPartials (plain columns whose fp32 partial tile goes to
// the split-K workspace).  PERSIST: a persistent launch (at most two tiles per workgroup; 256 x 256
// tiles, bf16 outputs only).
template <int MODE, bool WNK, int WN, int BM, bool PERSIST>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_bigwave_kernel(const GemmParams p) {
  static_assert(WN == 128 || WN == 64, "wave widths built: 128 and 64 columns");
  static_assert(BM == 256 || (BM == 192 && WN == 128), "tile heights built: 256, and 192 at WN = 128");
  static_assert(!PERSIST || (WN == 128 && BM == 256 && MODE != kPartials), "persistent launches: 256 x 256 bf16 tiles");
  constexpr int kBM = BM;
  constexpr int kWM = BM / 2;                    // output rows per wave (2 x 2 wave grid)
  constexpr int kMI = kWM / 32;
  constexpr int kAElems = kBM * kBK;
  constexpr int kACopies = kAElems * 2 / 1024 / kWaves;  // 1-KiB copies per wave per k-tile: 8 or 6
  constexpr int kBN = 2 * WN;                    // weight columns per tile
  constexpr int kNI = WN / 32;
  constexpr int kMps = kMI * kNI;                // MFMAs per k16 slice: 16 or 8
  constexpr int kBElems = kBK * kBN, kStageElems = kAElems + kBElems;
  constexpr int kBCopies = kBElems * 2 / 1024 / kWaves;  // 8 or 4
  constexpr int kCopies = kACopies + kBCopies;
  constexpr int kBChunks = kBN / 8;              // 16-B chunks per staged [k][n] row: 32 or 16
  constexpr int kKRowsPerCopy = 64 / kBChunks;   // k rows per 1-KiB copy of a [k][n] stage: 2 or 4
  // Ring depth: two stages of 64 KiB for 256 x 256 tiles; three of 48 KiB for 256 x 128 tiles,
  // whose k-tiles take half as long, so that their copies still have about two k-tiles to land.
  constexpr int kStages = WN == 128 ? 2 : 3;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kStages * kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / 2, wn = wave % 2;

  // Split-K launches: block = split * tiles + tile; split s runs k-tiles [s * kt_per_split, ...).
  // Tile sets (p.rects > 0, no splits): block b < rect_tmc[0] * rect_tnc[0] is a tile of
  // rectangle 0, the rest of rectangle 1; rectangle i is rect_tmc[i] row-tiles from row
  // rect_row0[i] by rect_tnc[i] tile columns from tile column rect_tn0[i], walked in groups of
  // rect_group[i] row-tiles.  Persistent launches (p.persist): tiles blockIdx.x + j * gridDim.x.
  const int tiles = p.tiles_m * p.tiles_n;
  const int split = p.splits > 1 ? (int)blockIdx.x / tiles : 0;
  auto tile_origin = [&](int bid, int& tm0, int& tn0) {
    int tile_m, tile_n, row0 = 0;
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
      tile_coords(bid - split * tiles, p.tiles_m, p.tiles_n, tile_m, tile_n);
    }
    tm0 = row0 + tile_m * kBM;
    tn0 = tile_n * (MODE == kSiluMul ? kBN / 2 : kBN);  // first output column of the tile
  };
  int m0, n0;
  tile_origin((int)blockIdx.x, m0, n0);
  const int kt0 = split * p.kt_per_split;
  const int nk = p.splits > 1 ? min(p.kt_per_split, p.K / kBK - kt0) : p.K / kBK;  // >= 1
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds);
  const bool persist = PERSIST && p.persist != 0;

  // ---- Copy offsets, fixed for a tile's whole k loop (the descriptors move with k0).  Copy i < 8
  // of this wave moves block 8*wave + i of the A stage, copy 8 + i block 8*wave + i of the B stage.
  uint32_t c_off[kCopies];
  auto set_copy_offsets = [&](int tm0, int tn0) {
#pragma unroll
    for (int i = 0; i < kACopies; ++i) {
      // [256 rows][64 k]: block q holds rows 8q .. 8q+7; lane l lands in row 8q + l/8 at slot l%8,
      // which holds k-chunk slot ^ ((row/2) % 8).
      const int row = (kACopies * wave + i) * kRowsPerCopy + lane / kChunks;
      const int chunk = (lane % kChunks) ^ ((row / kRowsPer256) % kChunks);
      c_off[i] = (tm0 + row < p.M) ? (uint32_t)(((int64_t)row * p.lda + chunk * 8) * 2) : kOob;
    }
#pragma unroll
    for (int i = 0; i < kBCopies; ++i) {
      const int q = kBCopies * wave + i;
      bool ok;
      if (WNK) {
        const int n = q * kRowsPerCopy + lane / kChunks;  // tile column = staged row
        const int chunk = (lane % kChunks) ^ ((n / kRowsPer256) % kChunks);
        const int64_t wrow = weight_column<MODE, WN>(p, tn0, n & ~7, ok) + (n & 7);
        c_off[kACopies + i] = ok ? (uint32_t)((wrow * p.ldb + chunk * 8) * 2) : kOob;
      } else {
        // [64 k][kBN n]: block q holds k rows kKRowsPerCopy*q ..; lane l lands in row
        // kKRowsPerCopy*q + l/kBChunks at slot l%kBChunks, which holds n-chunk slot ^ (4 * (row % 4)).
        const int krow = kKRowsPerCopy * q + lane / kBChunks;
        const int chunk = (lane % kBChunks) ^ (4 * (krow % 4));
        const int64_t wcol = weight_column<MODE, WN>(p, tn0, chunk * 8, ok);
        c_off[kACopies + i] = !ok ? kOob
                            : p.w_blk ? blocked_offset(krow, wcol, p.ldb)
                                      : (uint32_t)(((int64_t)krow * p.ldb + wcol) * 2);
      }
    }
  };
  set_copy_offsets(m0, n0);
  // cm0: first row of the tile whose copies are being issued (the next tile's in the last k-tiles
  // of a persistent workgroup's current tile).
  int cm0 = m0;
  auto a_desc = [&](int t) {
    const int k0 = (kt0 + t) * kBK;
    return buffer_desc(p.A + (int64_t)cm0 * p.lda + k0, ((int64_t)(p.M - cm0 - 1) * p.lda + (p.K - k0)) * 2);
  };
  auto b_desc = [&](int t) {
    const int k0 = (kt0 + t) * kBK;
    return WNK ? buffer_desc(p.B + k0, ((int64_t)(p.b_rows - 1) * p.ldb + (p.K - k0)) * 2)
           : p.w_blk ? blocked_desc(p.B, p.b_rows, k0)
                     : buffer_desc(p.B + (int64_t)k0 * p.ldb, (int64_t)(p.K - k0) * p.ldb * 2);
  };
  // Copy i of k-tile t into stage (t + sb) % kStages: the wave's block of the A or B half plus a
  // constant.  sb moves by the k-tile count from one tile of a persistent workgroup to the next, so
  // that the next tile's first k-tiles land in the stages its own loop expects.
  int sb = 0;
  const uint32_t wave_lds_a = lds0 + (uint32_t)(wave * kACopies * 1024);
  const uint32_t wave_lds_b = lds0 + (uint32_t)(kAElems * 2 + wave * kBCopies * 1024);
  auto copy_one = [&](int t, int i, i32x4_t ad, i32x4_t bd) {
    const uint32_t so = (uint32_t)(((unsigned)(t + sb) % kStages) * kStageElems * 2);
    if (i < kACopies) copy16_to_lds_at(ad, c_off[i], wave_lds_a + so, i * 1024);
    else copy16_to_lds_at(bd, c_off[i], wave_lds_b + so, (i - kACopies) * 1024);
  };
  auto copy_tile = [&](int t) {
    const i32x4_t ad = a_desc(t), bd = b_desc(t);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy_one(t, i, ad, bd);
  };

  // ---- Fragment offsets (elements within a stage).  [rows][64 k] staging: row r, k-chunk
  // 2*kk + lane/32 at slot chunk ^ ((r/2) % 8); for the rows a wave reads the swizzle term is
  // ((lane%32) / 2) % 8.
  const int a_r = lane & 31;
  const int a_half = lane >> 5;
  const int rs = (a_r / kRowsPer256) % kChunks;
  int ra_off[kKK], rb_off[kKK];
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    const int slot = (kk * 2 + a_half) ^ rs;
    ra_off[kk] = (wm * kWM + a_r) * kBK + slot * 8;
    rb_off[kk] = kAElems + (wn * WN + a_r) * kBK + slot * 8;  // W^T: B rows are weight columns
  }
  // [64 k][kBN n] staging, read with ds_read_b64_tr_b16 (each 16-lane group receives the transpose
  // of a 4 (k) x 16 (n) block): group g = lane/16 reads k row 16*kk + 8*(g/2) + 4*h + (lane%16)/4 at
  // n = WN*wn + 32*ni + 16*(g%2) + 4*(lane%4), i.e. chunk (WN/8)*wn + 4*ni + 2*(g%2) + (lane%4)/2,
  // stored at slot chunk ^ (4 * (k%4)) with k%4 = (lane%16)/4.
  int rt_off[kNI];
  {
    const int krow = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int x = 4 * ((lane & 15) >> 2);
    const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
      rt_off[ni] = kAElems + krow * kBN + (((WN / 8) * wn + 4 * ni + c) ^ x) * 8 + 4 * (lane & 1);
  }

  // Fragments of the four slices (buffer = slice index).  [k][n] weights: the two halves of each B
  // fragment are read separately and joined at the MFMA.
  bf16x8_t af[kKK][kMI], bv[kKK][kNI];
  i16x4_t bl[kKK][kNI], bh[kKK][kNI];
  // LDS read j of slice kk of tile t: j < 4 are the A fragments, then the B fragments (one read
  // each when W is stored [n][k], two half reads each when stored [k][n]).
  constexpr int kReadsPerSlice = kMI + (WNK ? 1 : 2) * kNI;
  auto read_one = [&](int t, int kk, int j) {
    const uint16_t* st = lds + ((unsigned)(t + sb) % kStages) * kStageElems;
    if (j < kMI) {
      af[kk][j] = *reinterpret_cast<const bf16x8_t*>(st + ra_off[kk] + j * 32 * kBK);
    } else if constexpr (WNK) {
      const int ni = j - kMI;
      bv[kk][ni] = *reinterpret_cast<const bf16x8_t*>(st + rb_off[kk] + ni * 32 * kBK);
    } else {
      const int ni = (j - kMI) / 2, h = (j - kMI) % 2;
      const uint16_t* b = st + rt_off[ni] + kk * 16 * kBN + h * 4 * kBN;
      const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b));
      if (h == 0) bl[kk][ni] = v;
      else bh[kk][ni] = v;
    }
  };

  f32x16_t acc[kMI][kNI];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // MFMA j (0 .. kMps-1) of slice kk: the weight fragment as the first operand, so lane l holds output
  // row (l & 31) and, in accumulator register r, column 8*(r/4) + 4*(l/32) + r%4 of the 32 x 32 block.
  auto mfma_one = [&](int kk, int j) {
    const int mi = j / kNI, ni = j % kNI;
    bf16x8_t b;
    if constexpr (WNK) b = bv[kk][ni];
    else b = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(bl[kk][ni], bh[kk][ni], 0, 1, 2, 3, 4, 5, 6, 7));
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, af[kk][mi], acc[mi][ni], 0, 0, 0);
  };

  // ---- Prologue: tiles 0 .. kStages-1 in flight, tile 0 landed, slices 0 and 1 of tile 0 read.
  copy_tile(0);
  if (nk >= kStages) {
#pragma unroll
    for (int s = 1; s < kStages; ++s) copy_tile(s);
    wait_vmcnt<(kStages - 1) * kCopies>();
  } else if (nk > 1) {  // three stages, two k-tiles
    copy_tile(1);
    wait_vmcnt<kCopies>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
#pragma unroll
  for (int j = 0; j < kReadsPerSlice; ++j) read_one(0, 0, j);
#pragma unroll
  for (int j = 0; j < kReadsPerSlice; ++j) read_one(0, 1, j);
  __builtin_amdgcn_sched_barrier(0);

  // One k-tile.  NEXT: tile t+1 exists (barrier, and its reads); COPY: tile t+kStages exists (its
  // copies, into tile t's stage); WAITN: this wave's copies of the tiles after t+1 that are in
  // flight at the barrier (kStages-2 tiles in the main loop, fewer near the end).  The main loop
  // runs with NEXT and COPY; the last kStages tiles are peeled, so the loop has no branches.
  //
  // Copies go into tile t's stage; ckt is the k-tile they fetch: t + kStages of the same tile, or,
  // in the last two k-tiles of a persistent workgroup's tile, k-tile 0 or 1 of its next tile (cm0
  // and c_off then describe that tile).  Without NEXT but with COPY (the last k-tile, prefetching),
  // the barrier still runs: it certifies that every wave's reads of tile t have returned.
  // rcopy: COPY decided at run time (a uniform branch), for the last two k-tiles, which copy only
  // when a persistent workgroup has a next tile; one code path keeps the registers as in the loop.
  auto k_tile = [&](int t, auto next_c, auto copy_c, auto waitn_c, int ckt, bool rcopy) {
    constexpr bool NEXT = decltype(next_c)::value, CCOPY = decltype(copy_c)::value;
    constexpr int WAITN = decltype(waitn_c)::value;
    const bool COPY = CCOPY || rcopy;
#pragma unroll
    for (int j = 0; j < kMps; ++j) {
      mfma_one(0, j);
#pragma unroll
      for (int r = j * 2 * kReadsPerSlice / kMps; r < (j + 1) * 2 * kReadsPerSlice / kMps; ++r)
        read_one(t, 2 + r / kReadsPerSlice, r % kReadsPerSlice);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < kMps; ++j) {
      mfma_one(1, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (NEXT || COPY) {
      if constexpr (NEXT) wait_vmcnt<WAITN>();  // this wave's copies of tile t+1 landed
      lds_barrier();        // ... everyone's; and every wave's reads of tile t returned
      __builtin_amdgcn_sched_barrier(0);
    }
    i32x4_t ad = {0, 0, 0, 0}, bd = {0, 0, 0, 0};
    if (COPY) {
      ad = a_desc(ckt);
      bd = b_desc(ckt);
    }
    // Copy c of the tile's kCopies follows MFMA slot c * 2*kMps / kCopies of slices 2-3 (slots
    // kMps.. are slice 3's): at 16 MFMAs per slice, the A copies after every second MFMA of slice
    // 2 and the B copies after every second MFMA of slice 3.
#pragma unroll
    for (int j = 0; j < kMps; ++j) {
      mfma_one(2, j);
      if (COPY) {
#pragma unroll
        for (int c = 0; c < kCopies; ++c)
          if (c * 2 * kMps / kCopies == j) copy_one(t + kStages, c, ad, bd);
      }
      if (NEXT) {
#pragma unroll
        for (int r = j * kReadsPerSlice / kMps; r < (j + 1) * kReadsPerSlice / kMps; ++r) read_one(t + 1, 0, r);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < kMps; ++j) {
      mfma_one(3, j);
      if (COPY) {
#pragma unroll
        for (int c = 0; c < kCopies; ++c)
          if (c * 2 * kMps / kCopies == kMps + j) copy_one(t + kStages, c, ad, bd);
      }
      if (NEXT) {
#pragma unroll
        for (int r = j * kReadsPerSlice / kMps; r < (j + 1) * kReadsPerSlice / kMps; ++r) read_one(t + 1, 1, r);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using W0 = std::integral_constant<int, 0>;
  using WMain = std::integral_constant<int, (kStages - 2) * kCopies>;
  using W1 = std::integral_constant<int, kCopies>;
  using T = std::true_type;
  using F = std::false_type;

  auto epilogue = [&](int em0, int en0) {
    const int row_base = em0 + wm * kWM + a_r;
    // ---- Epilogue straight from the accumulators: each lane owns 4 consecutive columns of one row
    // per register group, stored as one 8-byte bf16 piece, or (split-K, plain mode) as one 16-byte
    // fp32 piece of the partial tile in workspace slice `split`.
    constexpr bool partial = MODE == kPartials;
    float* wbase = partial ? p.ws + (int64_t)split * p.M * p.ws_ld : nullptr;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
      const int row = row_base + mi * 32;
      if (row >= p.M) continue;
      uint16_t* crow = p.C + (int64_t)row * p.ldc;
      if (MODE != kSiluMul) {
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = en0 + wn * WN + ni * 32 + g * 8 + a_half * 4;
            if constexpr (partial) {
              const float4 v = {acc[mi][ni][4 * g], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]};
              *reinterpret_cast<float4*>(wbase + (int64_t)row * p.ws_ld + col) = v;
            } else if (col < p.N) {
              u32x2_t v;
              v.x = pack_bf16x2(acc[mi][ni][4 * g + 0], acc[mi][ni][4 * g + 1]);
              v.y = pack_bf16x2(acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]);
              *reinterpret_cast<u32x2_t*>(crow + col) = v;
            }
          }
      } else {
#pragma unroll
        for (int ni = 0; ni < kNI / 2; ++ni)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = en0 + wn * (WN / 2) + ni * 32 + g * 8 + a_half * 4;
            if (col < p.N) {
              float a[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                a[e] = silu_mul(acc[mi][ni][4 * g + e], acc[mi][ni + kNI / 2][4 * g + e]);
              u32x2_t v;
              v.x = pack_bf16x2(a[0], a[1]);
              v.y = pack_bf16x2(a[2], a[3]);
              *reinterpret_cast<u32x2_t*>(crow + col) = v;
            }
          }
      }
    }
  };

  // ---- Epilogue through LDS.  The accumulator layout gives each lane 4 columns of one row per
  // register group, so direct stores write 16-byte pieces of 32 rows per instruction; here each wave
  // instead writes one 32-row block at a time into its own quarter of a free ring stage and reads it
  // back as whole rows, so that every store instruction covers whole rows (256 bytes of 4 rows, or
  // of 2 fp32 rows).  The stage after the last k-tile's is free: its last tile's reads all returned
  // before the barrier of the k-tile before the last, and no copy targets it.  The quarter is the
  // wave's alone, and a wave's LDS accesses complete in order, so no barrier is needed.  Staged
  // rows: chunk c (16 bytes) of row r at slot c ^ (r % chunks per row), so that both the column-wise
  // writes and the row-wise reads spread over the banks.  The global stores carry the non-temporal
  // hint: outputs are written once and read by a later launch (measured 1.3-2.4 us less per launch
  // of 256 tiles).
  constexpr int kWaveStage = kStageElems / kWaves;  // elements of one wave's staging quarter
  constexpr bool kF32Staged = 32 * WN * 4 <= kWaveStage * 2;
  auto epilogue_staged = [&](int em0, int en0, int t_last) {
    uint16_t* stg = lds + ((unsigned)(t_last + 1 + sb) % kStages) * kStageElems + wave * kWaveStage;
    const int wrow0 = em0 + wm * kWM;  // the wave's first output row
    // Read the 32 staged rows of chunks CH back and store them: row r to dst_row(r), chunk c at
    // element offset c * (16 / ES) of it; rows at or past M are skipped, as (plain outputs) are
    // chunks at or past N.
    auto drain = [&](auto ch_c, int mi, auto&& dst) {
      constexpr int CH = decltype(ch_c)::value;
      constexpr int kRowsPerRead = 64 / CH;
#pragma unroll
      for (int i = 0; i < 32 / kRowsPerRead; ++i) {
        const int r = i * kRowsPerRead + lane / CH, c = lane % CH;
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(stg + r * CH * 8 + ((c ^ (r % CH)) * 8));
        const int row = wrow0 + mi * 32 + r;
        if (row < p.M) dst(row, c, v);
      }
    };
    if (MODE == kSiluMul) {
      constexpr int CH = WN / 16;  // WN / 2 act columns per row
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < kNI / 2; ++ni)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float a[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = silu_mul(acc[mi][ni][4 * g + e], acc[mi][ni + kNI / 2][4 * g + e]);
            u32x2_t v;
            v.x = pack_bf16x2(a[0], a[1]);
            v.y = pack_bf16x2(a[2], a[3]);
            const int c = ni * 4 + g;
            *reinterpret_cast<u32x2_t*>(stg + a_r * CH * 8 + ((c ^ (a_r % CH)) * 8) + a_half * 4) = v;
          }
        drain(std::integral_constant<int, CH>{}, mi, [&](int row, int c, i32x4_t v) {
          const int col = en0 + wn * (WN / 2) + c * 8;
          if (col < p.N) __builtin_nontemporal_store(v, reinterpret_cast<i32x4_t*>(p.C + (int64_t)row * p.ldc + col));
        });
      }
    } else if constexpr (MODE == kPlain) {
      constexpr int CH = WN / 8;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2_t v;
            v.x = pack_bf16x2(acc[mi][ni][4 * g + 0], acc[mi][ni][4 * g + 1]);
            v.y = pack_bf16x2(acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]);
            const int c = ni * 4 + g;
            *reinterpret_cast<u32x2_t*>(stg + a_r * CH * 8 + ((c ^ (a_r % CH)) * 8) + a_half * 4) = v;
          }
        drain(std::integral_constant<int, CH>{}, mi, [&](int row, int c, i32x4_t v) {
          const int col = en0 + wn * WN + c * 8;
          if (col < p.N) __builtin_nontemporal_store(v, reinterpret_cast<i32x4_t*>(p.C + (int64_t)row * p.ldc + col));
        });
      }
    } else if constexpr (kF32Staged) {
      // fp32 partial tile: chunk c of a staged row holds columns 4c .. 4c+3.
      constexpr int CH = WN / 4;
      float* wbase = p.ws + (int64_t)split * p.M * p.ws_ld + en0 + wn * WN;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 v = {acc[mi][ni][4 * g], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]};
            const int c = ni * 8 + g * 2 + a_half;
            *reinterpret_cast<float4*>(stg + a_r * CH * 8 + ((c ^ (a_r % CH)) * 8)) = v;
          }
        drain(std::integral_constant<int, CH>{}, mi, [&](int row, int c, i32x4_t v) {
          __builtin_nontemporal_store(v, reinterpret_cast<i32x4_t*>(wbase + (int64_t)row * p.ws_ld + c * 4));
        });
      }
    } else {
      epilogue(em0, en0);
    }
  };

  // ---- The tiles of this workgroup: one, or (persistent launches) blockIdx.x and, where it exists,
  // blockIdx.x + gridDim.x (a persistent launch has at most twice as many tiles as workgroups).
  int bid = (int)blockIdx.x;
  int last_m0 = m0, last_n0 = n0, last_t = 0;  // the tile whose outputs the staged epilogue stores
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int em0 = m0, en0 = n0;
    int t = 0;
    for (; t + kStages < nk; ++t) k_tile(t, T{}, T{}, WMain{}, t + kStages, false);
    bool has_next = false;
    if constexpr (PERSIST) {
      if (jt == 0 && persist && nk >= 2 && bid + (int)gridDim.x < tiles) {
        has_next = true;
        bid += (int)gridDim.x;
        tile_origin(bid, m0, n0);
        set_copy_offsets(m0, n0);
        cm0 = m0;
      }
    }
    // The last k-tiles; with a next tile they copy its k-tiles 0 and 1 into the stages they free,
    // and this wave's copies of k-tile 0 must have landed before the stores join the vmcnt queue.
    if constexpr (kStages == 3) {
      if (t + 2 < nk) k_tile(t++, T{}, F{}, W1{}, 0, false);  // tile t+2 in flight
    }
    if (t + 1 < nk) {
      k_tile(t, T{}, F{}, W0{}, 0, has_next);
      ++t;
    }
    k_tile(t, F{}, F{}, W0{}, 1, has_next);
    if constexpr (!PERSIST) {
      last_m0 = em0;
      last_n0 = en0;
      last_t = t;
      break;
    }
    // Persistent instances store directly (the ring holds the next tile's first k-tiles).
    if (has_next) wait_vmcnt<kCopies>();
    epilogue(em0, en0);
    if (!has_next) break;
    // Next tile: accumulators cleared, its k-tile 0 published, slices 0 and 1 read.
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
    sb = (sb + nk) % kStages;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kReadsPerSlice; ++j) read_one(0, 0, j);
#pragma unroll
    for (int j = 0; j < kReadsPerSlice; ++j) read_one(0, 1, j);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!PERSIST) epilogue_staged(last_m0, last_n0, last_t);
}

template <int MODE, bool WNK, int WN, int BM, bool PERSIST>
void launch_one(const GemmParams& p, hipStream_t stream) {
  const int splits = p.splits > 1 ? p.splits : 1;
  int blocks = p.rects > 0 ? p.rect_tmc[0] * p.rect_tnc[0] + (p.rects > 1 ? p.rect_tmc[1] * p.rect_tnc[1] : 0)
                           : splits * p.tiles_m * p.tiles_n;
  if (PERSIST && p.persist < blocks) blocks = p.persist;  // persistent: p.persist workgroups
  hipLaunchKernelGGL((gemm_bigwave_kernel<MODE, WNK, WN, BM, PERSIST>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, p);
}

template <int MODE, int WN, int BM, bool PERSIST>
void launch_layout(const GemmParams& p, hipStream_t stream) {
  p.w_nk ? launch_one<MODE, true, WN, BM, PERSIST>(p, stream) : launch_one<MODE, false, WN, BM, PERSIST>(p, stream);
}

template <int WN, int BM>
void launch_width(const GemmParams& p, hipStream_t stream) {
  if (p.mode == kSiluMul) launch_layout<kSiluMul, WN, BM, false>(p, stream);
  else if (p.splits > 1) launch_layout<kPartials, WN, BM, false>(p, stream);
  else launch_layout<kPlain, WN, BM, false>(p, stream);
}

}  // namespace

bool gemm_bigwave_supports(const GemmParams& p) { return p.K % kBK == 0 && p.K > 0; }

int gemm_bigwave_tile_cols(int mode, bool narrow) {
  const int cols = narrow ? 128 : 256;
  return mode == kSiluMul ? cols / 2 : cols;
}

hipError_t launch_gemm_bigwave(const GemmParams& p, hipStream_t stream) {
  if (p.mode == kSiluMul && p.splits > 1) return hipErrorInvalidValue;  // split SiLU·up runs as halves
  if (p.tile_rows == 192) {
    // Short tiles: wide columns only, no k splits, rows given by a tile set.
    if (p.narrow || p.splits > 1 || p.rects < 1 || p.persist > 0) return hipErrorInvalidValue;
    launch_width<128, 192>(p, stream);
  } else if (p.tile_rows == 256 || p.tile_rows == 0) {
    if (p.rects > 0 && p.splits > 1) return hipErrorInvalidValue;
    if (p.persist > 0 && (p.rects > 0 || p.splits > 1 || p.narrow)) return hipErrorInvalidValue;
    if (p.persist > 0) {
      if (p.mode == kSiluMul) launch_layout<kSiluMul, 128, 256, true>(p, stream);
      else launch_layout<kPlain, 128, 256, true>(p, stream);
    } else {
      p.narrow ? launch_width<64, 256>(p, stream) : launch_width<128, 256>(p, stream);
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ttl
