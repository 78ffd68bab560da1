// Tiled bf16 GEMM on the CDNA4 matrix cores for the column- and row-parallel shards.
//
// C[M, N] = A[M, K] · B[K, map(N)]: A = the rank's input rows (k contiguous), B = the unsharded
// weight, addressed in place.  The weight is stored either as W[k][n] (n contiguous, the layout of
// the statement Y = X·W) or transposed as W^T[n][k] (k contiguous, the layout PyTorch-style Linear
// weights are kept in).  The rank's columns are chosen by a column map (plain slice, up to three
// q|k|v segments, or paired gate|up columns for the fused SiLU·up epilogue) and the rank's rows by
// the B base pointer.
//
// Workgroup tile 256 x 256 weight columns, k-tiles of 64 (each A row and W^T row then contributes
// one whole 128-B line per k-tile).  Eight wave64s (two per SIMD, so one
// wave's LDS reads, waits and barrier overlap the other's matrix work) in a 2 x 4 grid, each owning
// 128 x 64 outputs as 4 x 2 v_mfma_f32_32x32x16_bf16 accumulators.  This kernel takes any K; where
// K is a multiple of 64 the four-wave kernel (gemm_bigwave.hip) is used instead, as it is faster.
//
// Data movement (gfx950):
//  * Global -> LDS without registers: buffer_load_dwordx4 ... lds moves 64 lanes x 16 B = 1 KiB per
//    instruction, lane i landing at byte 16*i of the instruction's block.  Each lane picks the global
//    piece that must land there, which is how the LDS layouts below get their XOR swizzles.
//  * A ring of two 64-KiB k-tile stages in LDS, refilled as the ping-pong schedule below describes.
//  * LDS has 64 banks of 4 B; 16 lanes reading 16 B each (or 32 lanes reading 8 B each) are
//    conflict-free when they cover 256 distinct bytes modulo 256.
//  * A (and B when stored [n][k]) is staged as [256 rows][64 k]: eight 16-B chunks per 128-B row,
//    chunk c of row m at slot c ^ ((m / 2) % 8), so the 16 rows one ds_read_b128 touches at one
//    k-chunk fall on distinct banks.
//  * B stored [k][n] is staged as loaded, [64 k][256 n]: 32 chunks per 512-B row, chunk c of row k at
//    slot c ^ (4 * (k % 4)).  The matrix cores want 8 consecutive k of one n per lane;
//    ds_read_b64_tr_b16 returns, in each 16-lane group, the transpose of a 4 (k) x 16 (n) block —
//    lane j of the group addresses row k0 + j/4 at n0 + 4*(j%4) and receives k0..k0+3 at n0 + j — so
//    two such reads build one operand without a transpose in registers.
//  * Tiles are ordered for the L2 of each XCD: consecutive workgroups go to different XCDs, so the
//    block index is remapped so that each XCD works on a compact group of tiles (4 row-tiles tall)
//    that share A rows and weight columns in its L2.
//
// Tails in M, N and K: copies whose offsets are pushed past the buffer's record count read zeros, so
// the k-tail contributes exact zeros and the steady-state loop has no bounds logic; stores are masked.
#include "gemm_common.h"

namespace ttl {
namespace {

using namespace gemm;

constexpr int kBM = 256;                   // output rows per tile
constexpr int kBN = 256;                   // weight columns per tile
constexpr int kBK = 64;                    // k per stage (128-B global row pieces)
constexpr int kWaves = 8;                  // two per SIMD, 128 x 64 outputs each
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 2;                 // two 64-KiB stages
constexpr int kWM = 128;                   // rows per wave
constexpr int kWavesN = kWaves / (kBM / kWM);
constexpr int kWN = kBN / kWavesN;         // weight columns per wave (2 x kWavesN wave grid)
constexpr int kNI = kWN / 32;              // 32-wide accumulator blocks per wave along n
constexpr int kAElems = kBM * kBK;         // A stage (bf16 elements)
constexpr int kBElems = kBK * kBN;         // B stage
constexpr int kStageElems = kAElems + kBElems;
constexpr int kACopies = kAElems * 2 / 1024 / kWaves;   // 1-KiB copies per wave per tile
constexpr int kBCopies = kBElems * 2 / 1024 / kWaves;
constexpr int kLoads = kACopies + kBCopies;             // vmcnt increments per wave per tile

constexpr int kChunks = kBK / 8;           // 16-B chunks per [rows][k] staged row
constexpr int kRowsPer256 = 256 / (2 * kBK);  // staged rows per 256 B of LDS
constexpr int kRowsPerCopy = 1024 / (2 * kBK);
constexpr int kKK = kBK / 16;              // k16 slices per stage

static_assert(kStages * kStageElems * 2 <= 160 * 1024, "LDS ring");

// ---- Ping-pong schedule.
//
// The two row halves of the tile (waves 0-3: rows 0..127, waves 4-7: rows 128..255; one wave of
// each half per SIMD) alternate between two phases, offset by one phase, with a workgroup barrier
// between phases:
//   X(t): LDS reads of all four k16 slices of tile t into registers, plus this half's share of the
//         global -> LDS copies of a later tile;
//   Y(t): the 32 MFMAs of tile t from those registers.
// While one half runs Y on a SIMD the other runs X, so the matrix core of every SIMD is fed by one
// wave while the other fetches, instead of both waves competing for it and then idling together at
// the barrier.  Phase p: waves 0-3 do step p (X(p/2) for even p, Y otherwise), waves 4-7 step p-1.
//
// Copies: waves 0-3 move A and waves 4-7 move B (eight 1-KiB copies per wave per tile).  With two
// stages (tile u in stage u%2):
//   * waves 0-3 issue A(t+1) in X(t) (phase 2t); the stage's previous tile t-1 was last read by
//     waves 4-7 in phase 2t-1; A(t+1) must land before phase 2t+2, so they wait at the end of Y(t);
//   * waves 4-7 issue B(t+2) in X(t) (phase 2t+1), after their own reads of tile t from the same
//     stage have returned (waves 0-3 read tile t in phase 2t); B(t+2) must land before phase 2t+4,
//     so at the end of X(t+1) they wait until only B(t+3) is outstanding.
template <int MODE, bool WNK>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void gemm_pingpong_kernel(const GemmParams p) {
  static_assert(kWaves == 8 && kStages == 2 && kBK == 64 && kWM == 128, "ping-pong layout");
  constexpr int kCopies = 8;  // per wave per tile
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kStages * kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWavesN;  // row half = schedule group
  const int wn = wave % kWavesN;

  int tile_m, tile_n;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tile_m, tile_n);
  const int m0 = tile_m * kBM;
  const int n0 = tile_n * (MODE == kSiluMul ? kBN / 2 : kBN);
  const int nk = (p.K + kBK - 1) / kBK;
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds);

  // ---- This wave's copies: block q = 8*wn + i of A (group 0) or of B (group 1).
  uint32_t c_off[kCopies];
  int c_k[kCopies];  // k offset within the tile that each lane's piece starts at (k-tail test)
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int q = kCopies * wn + i;
    if (wm == 0) {
      const int row = q * kRowsPerCopy + lane / kChunks;
      const int chunk = (lane % kChunks) ^ ((row / kRowsPer256) % kChunks);
      c_k[i] = chunk * 8;
      c_off[i] = (m0 + row < p.M) ? (uint32_t)(((int64_t)row * p.lda + chunk * 8) * 2) : kOob;
    } else {
      bool ok;
      if (WNK) {
        const int n = q * kRowsPerCopy + lane / kChunks;
        const int chunk = (lane % kChunks) ^ ((n / kRowsPer256) % kChunks);
        const int64_t wrow = weight_column<MODE, kWN>(p, n0, n & ~7, ok) + (n & 7);
        c_off[i] = ok ? (uint32_t)((wrow * p.ldb + chunk * 8) * 2) : kOob;
        c_k[i] = chunk * 8;
      } else {
        const int krow = 2 * q + (lane >> 5);
        const int chunk = (lane & 31) ^ (4 * (krow % 4));
        const int64_t wcol = weight_column<MODE, kWN>(p, n0, chunk * 8, ok);
        c_off[i] = !ok ? kOob
                 : p.w_blk ? blocked_offset(krow, wcol, p.ldb)
                           : (uint32_t)(((int64_t)krow * p.ldb + wcol) * 2);
        c_k[i] = krow;
      }
    }
  }
  const bool ktail = (p.K % kBK) != 0;
  auto copy_tile = [&](int t) {
    const int k0 = t * kBK;
    const bool tail = ktail && t == nk - 1;
    const i32x4_t d =
        wm == 0 ? buffer_desc(p.A + (int64_t)m0 * p.lda + k0, ((int64_t)(p.M - m0 - 1) * p.lda + (p.K - k0)) * 2)
                : (WNK       ? buffer_desc(p.B + k0, ((int64_t)(p.b_rows - 1) * p.ldb + (p.K - k0)) * 2)
                   : p.w_blk ? blocked_desc(p.B, p.b_rows, k0)
                             : buffer_desc(p.B + (int64_t)k0 * p.ldb, (int64_t)(p.K - k0) * p.ldb * 2));
    const uint32_t st = lds0 + (uint32_t)((t % kStages) * kStageElems * 2) + (wm == 0 ? 0u : kAElems * 2u);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const uint32_t off = (tail && k0 + c_k[i] >= p.K) ? kOob : c_off[i];
      copy16_to_lds(d, off, st + (kCopies * wn + i) * 1024);
    }
  };

  // ---- Fragment reads of a whole tile.  [rows][64 k] staging: row r, k-chunk 2*kk + lane/32 at
  // slot chunk ^ ((r/2) % 8); for the rows a wave reads the swizzle term is ((lane%32) / 2) % 8.
  // [64 k][256 n] staging, read with ds_read_b64_tr_b16: 16-lane group g = lane/16 reads k row
  // 16*kk + 8*(g/2) + 4*h + (lane%16)/4 at n = 64*wn + 32*ni + 16*(g%2) + 4*(lane%4), i.e. chunk
  // 8*wn + 4*ni + 2*(g%2) + (lane%4)/2, stored at slot chunk ^ (4 * (k%4)), k%4 = (lane%16)/4.
  const int a_r = lane & 31;
  const int a_half = lane >> 5;
  const int rs = (a_r / kRowsPer256) % kChunks;
  int ra_off[kKK], rb_off[kKK];
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    const int slot = (kk * 2 + a_half) ^ rs;
    ra_off[kk] = (wm * kWM + a_r) * kBK + slot * 8;
    rb_off[kk] = kAElems + (wn * kWN + a_r) * kBK + slot * 8;
  }
  int rt_off[kNI];
  {
    const int krow = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int x = 4 * ((lane & 15) >> 2);
    const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
      rt_off[ni] = kAElems + krow * kBN + (((kWN / 8) * wn + 4 * ni + c) ^ x) * 8 + 4 * (lane & 1);
  }

  bf16x8_t af[kKK][4], bv[kKK][kNI];
  auto read_tile = [&](int t) {
    const uint16_t* st = lds + (t % kStages) * kStageElems;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[kk][mi] = *reinterpret_cast<const bf16x8_t*>(st + ra_off[kk] + mi * 32 * kBK);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        if (WNK) {
          bv[kk][ni] = *reinterpret_cast<const bf16x8_t*>(st + rb_off[kk] + ni * 32 * kBK);
        } else {
          const uint16_t* b = st + rt_off[ni] + kk * 16 * kBN;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + 4 * kBN));
          bv[kk][ni] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    }
  };

  f32x16_t acc[4][kNI];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  auto mfma_tile = [&]() {
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[kk][ni], af[kk][mi], acc[mi][ni], 0, 0, 0);
  };
  auto phase_end = [&]() { lds_barrier(); __builtin_amdgcn_sched_barrier(0); };

  // Prologue: A(0) by group 0; B(0) and B(1) by group 1; tile 0 complete before phase 0.
  if (wm == 0) {
    copy_tile(0);
    wait_vmcnt<0>();
  } else {
    copy_tile(0);
    if (nk > 1) {
      copy_tile(1);
      wait_vmcnt<kCopies>();
    } else {
      wait_vmcnt<0>();
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  phase_end();
  if (wm == 1) phase_end();  // group 1 runs one phase behind

  for (int t = 0; t < nk; ++t) {
    // X(t)
    if (wm == 0) {
      if (t + 1 < nk) copy_tile(t + 1);
      __builtin_amdgcn_sched_barrier(0);
      read_tile(t);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else {
      read_tile(t);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of this stage done before refilling it
      __builtin_amdgcn_sched_barrier(0);
      if (t + 2 < nk) {
        copy_tile(t + 2);
        wait_vmcnt<kCopies>();  // B(t+1) landed; B(t+2) may still be in flight
      } else {
        wait_vmcnt<0>();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    phase_end();
    // Y(t)
    mfma_tile();
    __builtin_amdgcn_sched_barrier(0);
    if (wm == 0) wait_vmcnt<0>();  // A(t+1) landed
    phase_end();
  }
  if (wm == 0) phase_end();  // matches group 1's last phase

  // Epilogue straight from the accumulators: each lane owns 4 consecutive columns of one row per
  // register group, stored as one 8-byte piece.
  const int row_base = m0 + wm * kWM + a_r;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int row = row_base + mi * 32;
    if (row >= p.M) continue;
    uint16_t* crow = p.C + (int64_t)row * p.ldc;
    if (MODE == kPlain) {
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn * kWN + ni * 32 + g * 8 + a_half * 4;
          if (col < p.N) {
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
          const int col = n0 + wn * (kWN / 2) + ni * 32 + g * 8 + a_half * 4;
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
}

template <int MODE, bool WNK>
void launch_one(const GemmParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_pingpong_kernel<MODE, WNK>), dim3((unsigned)(p.tiles_m * p.tiles_n)),
                     dim3(kThreads), 0, stream, p);
}

}  // namespace

int gemm_tile_rows() { return kBM; }
int gemm_tile_cols(int mode) { return mode == kSiluMul ? kBN / 2 : kBN; }

hipError_t launch_gemm_tiled(const GemmParams& p, hipStream_t stream) {
  if (p.mode == kSiluMul)
    p.w_nk ? launch_one<kSiluMul, true>(p, stream) : launch_one<kSiluMul, false>(p, stream);
  else
    p.w_nk ? launch_one<kPlain, true>(p, stream) : launch_one<kPlain, false>(p, stream);
  return hipGetLastError();
}

}  // namespace ttl
