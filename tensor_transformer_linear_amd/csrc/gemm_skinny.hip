// Split-K bf16 GEMM for short M (decode batches and shards too small to fill the chip with
// 256 x 256 tiles).
//
// With few token rows the weight slice is the only large operand: the work is bound by streaming
// W once from HBM, and the grid must cover all 256 CUs even when M / 256 * N / 256 tiles would not.
// So each workgroup takes a 32*MB-row x 128-weight-column tile over one range of k-tiles (a split),
// streams its weight slab through a ring of LDS stages with direct global -> LDS copies, multiplies
// on the matrix cores, and writes its fp32 partial tile to a workspace.  A second, fully parallel
// kernel then sums the splits of every output in ascending split order, applies the epilogue
// (plain bf16, or SiLU(gate)·up) and stores the bf16 output.  (Reducing inside the first kernel,
// in the last workgroup of each tile to arrive, needs device-scope fences that write back and
// invalidate each XCD's L2, and serialises the reduction's loads behind one workgroup: both are
// far slower than the extra launch.)
//
// When one split covers all of k, the workgroup stores its output straight from the accumulators
// and no workspace is involved.
//
// Tile layout: 4 wave64s, wave w owns weight columns 32w .. 32w+31 of the tile and all 32*MB rows
// (MB accumulators of v_mfma_f32_32x32x16_bf16).  SiLU·up with one split (the epilogue in the
// kernel): wave w's columns 0..15 are the gate columns and 16..31 the up columns of act columns
// 16w .. 16w+15, so that gate and up of one output land in the same lane (accumulator registers r
// and r + 8).  SiLU·up with several splits: the main kernel runs over the gate columns and then the
// up columns as plain outputs, 128 consecutive weight columns per tile (with weights stored [k][n]
// each k row is then read in 256-byte runs: measured ~30% faster at 70B decode sizes than the
// paired tiles' 128-byte runs), and the finalize kernel pairs them.
//
// LDS staging per stage (k-tiles of 64):
//  * A as [32*MB rows][64 k], eight 16-B chunks per 128-B row, chunk c of row m at slot
//    c ^ ((m / 2) % 8): the 16 rows one ds_read_b128 phase touches fall on distinct banks.
//  * W stored [n][k]: the same [128 rows][64 k] layout.
//  * W stored [k][n]: [64 k][128 n], sixteen chunks per 256-B row, chunk c of row k at slot
//    c ^ (4 * (k % 4)), read with ds_read_b64_tr_b16 (4 k x 16 n blocks transposed on the way out);
//    the four k rows one read phase touches then sit in four different 64-B bank groups.
// k tails and rows past M read zeros through the buffer descriptors' range checks.
#include "gemm_common.h"

namespace ttl {
namespace {

using namespace gemm;

constexpr int kBN = kSkinnyCols;
constexpr int kBK = kSkinnyK;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBElems = kBK * kBN;
constexpr int kBCopies = kBElems * 2 / 1024 / kWaves;  // 1-KiB copies per wave per k-tile
constexpr int kKK = kBK / 16;

static_assert(kBN == 128 && kBK == 64, "the copy and read layouts below assume 128 x 64 tiles");

// Weight column of tile column c (the first of 8 consecutive ones) and whether it is in range.
template <int MODE>
__device__ inline int64_t tile_weight_column(const GemmParams& p, int tile_n, int c, bool& ok) {
  if (MODE == kSiluMul) {
    const int act = tile_n * (kBN / 2) + 16 * (c / 32) + (c & 15);
    ok = act < p.N;
    return ((c & 16) == 0 ? p.gate_w0 : p.up_w0) + act;
  }
  const int oc = tile_n * kBN + c;
  ok = oc < p.N;
  int64_t w0 = p.seg_w0[0];
  int s0 = p.seg_out0[0];
  if (p.nseg > 1 && oc >= p.seg_out0[1]) { w0 = p.seg_w0[1]; s0 = p.seg_out0[1]; }
  if (p.nseg > 2 && oc >= p.seg_out0[2]) { w0 = p.seg_w0[2]; s0 = p.seg_out0[2]; }
  return w0 + (oc - s0);
}

template <int MODE, bool WNK, int MB, int STAGES>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void gemm_skinny_kernel(const GemmParams p) {
  constexpr int kBM = 32 * MB;
  constexpr int kAElems = kBM * kBK;
  constexpr int kStageElems = kAElems + kBElems;
  constexpr int kACopies = kAElems * 2 / 1024 / kWaves;
  constexpr int kLoads = kACopies + kBCopies;
  static_assert(kACopies >= 1 && STAGES >= 2 && STAGES * kStageElems * 2 <= 160 * 1024, "LDS ring");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Block -> (split, tile_m, tile_n).  Consecutive blocks go to different XCDs, each with its own
  // L2: the XCD-aware map gives each XCD a compact run of columns (split, tile_n), every row tile of
  // each, so that the row tiles reading one weight block [k range, columns] share an L2 (numbering
  // tile_n fastest split them over XCDs whenever the column count was not a multiple of 8: 8B TP=8
  // SiLU·up at 256 tokens fetched 90 MB for 32 MB of operands).
  int tile_m = 0, col = 0;
  tile_coords((int)blockIdx.x, p.tiles_m, p.tiles_n * p.splits, tile_m, col, p.tiles_m);
  const int split = col / p.tiles_n;
  const int tile_n = col % p.tiles_n;
  const int m0 = tile_m * kBM;
  const int nk_all = (p.K + kBK - 1) / kBK;
  const int kt0 = split * p.kt_per_split;
  const int nk = min(p.kt_per_split, nk_all - kt0);  // >= 1: the host sizes the splits
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds);

  // ---- Copy offsets (the descriptors move with k0).
  // A: copy q covers rows 8q .. 8q+7; lane l lands in row 8q + l/8 at slot l%8.
  uint32_t a_off[kACopies];
  int a_kc[kACopies];
#pragma unroll
  for (int i = 0; i < kACopies; ++i) {
    const int row = (kACopies * wave + i) * 8 + lane / 8;
    const int chunk = (lane % 8) ^ ((row / 2) % 8);
    a_kc[i] = chunk * 8;
    a_off[i] = (m0 + row < p.M) ? (uint32_t)(((int64_t)row * p.lda + chunk * 8) * 2) : kOob;
  }
  uint32_t b_off[kBCopies];
  int b_kc[kBCopies];
#pragma unroll
  for (int i = 0; i < kBCopies; ++i) {
    const int q = kBCopies * wave + i;
    bool ok;
    if (WNK) {
      const int n = q * 8 + lane / 8;  // tile column = staged row
      const int chunk = (lane % 8) ^ ((n / 2) % 8);
      const int64_t wrow = tile_weight_column<MODE>(p, tile_n, n & ~7, ok) + (n & 7);
      b_off[i] = ok ? (uint32_t)((wrow * p.ldb + chunk * 8) * 2) : kOob;
      b_kc[i] = chunk * 8;
    } else {
      // copy q covers k rows 4q .. 4q+3: lane l lands in row 4q + l/16 at slot l%16, which holds
      // chunk (l%16) ^ (4 * (l/16)).
      const int krow = 4 * q + (lane >> 4);
      const int chunk = (lane & 15) ^ (4 * (lane >> 4));
      const int64_t wcol = tile_weight_column<MODE>(p, tile_n, chunk * 8, ok);
      b_off[i] = !ok ? kOob
               : p.w_blk ? blocked_offset(krow, wcol, p.ldb)
                         : (uint32_t)(((int64_t)krow * p.ldb + wcol) * 2);
      b_kc[i] = krow;
    }
  }

  auto copy_tile = [&](int t) {
    const int k0 = (kt0 + t) * kBK;
    const bool ktail = k0 + kBK > p.K;
    const uint32_t st = lds0 + (uint32_t)((t % STAGES) * kStageElems * 2);
    const i32x4_t ad =
        buffer_desc(p.A + (int64_t)m0 * p.lda + k0, ((int64_t)(p.M - m0 - 1) * p.lda + (p.K - k0)) * 2);
#pragma unroll
    for (int i = 0; i < kACopies; ++i) {
      const uint32_t off = (ktail && k0 + a_kc[i] >= p.K) ? kOob : a_off[i];
      copy16_to_lds(ad, off, st + (kACopies * wave + i) * 1024);
    }
    const i32x4_t bd =
        WNK       ? buffer_desc(p.B + k0, ((int64_t)(p.b_rows - 1) * p.ldb + (p.K - k0)) * 2)
        : p.w_blk ? blocked_desc(p.B, p.b_rows, k0)
                  : buffer_desc(p.B + (int64_t)k0 * p.ldb, (int64_t)(p.K - k0) * p.ldb * 2);
#pragma unroll
    for (int i = 0; i < kBCopies; ++i) {
      const uint32_t off = (ktail && k0 + b_kc[i] >= p.K) ? kOob : b_off[i];
      copy16_to_lds(bd, off, st + kAElems * 2 + (kBCopies * wave + i) * 1024);
    }
  };

  // ---- Fragment reads (element offsets within a stage).
  const int a_r = lane & 31;
  const int a_half = lane >> 5;
  int ra_off[kKK], rb_off[kKK];
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    const int slot = (kk * 2 + a_half) ^ ((a_r / 2) % 8);
    ra_off[kk] = a_r * kBK + slot * 8;
    rb_off[kk] = kAElems + (wave * 32 + a_r) * kBK + slot * 8;
  }
  // [k][n]: 16-lane group g = lane/16 reads k row 8*(lane/32) + (lane%16)/4 (+4 for the second
  // read) at n = 32*wave + 16*(g%2) + 4*(lane%4): chunk 4*wave + 2*(g%2) + (lane%4)/2, stored at
  // slot chunk ^ (4 * (k%4)), k%4 = (lane%16)/4.
  int rt_off;
  {
    const int krow = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int x = 4 * ((lane & 15) >> 2);
    const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    rt_off = kAElems + krow * kBN + ((4 * wave + c) ^ x) * 8 + 4 * (lane & 1);
  }

  bf16x8_t af[2][MB], bv[2];
  auto read_frags = [&](int t, int kk, int buf) {
    const uint16_t* st = lds + (t % STAGES) * kStageElems;
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
      af[buf][mi] = *reinterpret_cast<const bf16x8_t*>(st + ra_off[kk] + mi * 32 * kBK);
    if (WNK) {
      bv[buf] = *reinterpret_cast<const bf16x8_t*>(st + rb_off[kk]);
    } else {
      const uint16_t* b = st + rt_off + kk * 16 * kBN;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + 4 * kBN));
      bv[buf] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  f32x16_t acc[MB];
#pragma unroll
  for (int mi = 0; mi < MB; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mi][r] = 0.0f;

  auto mfma_block = [&](int buf) {
    // Weight fragment as the first operand: lane l holds output row (l & 31) and, in accumulator
    // register r, tile column 32*wave + 8*(r/4) + 4*(l/32) + r%4.
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
      acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[buf], af[buf][mi], acc[mi], 0, 0, 0);
  };

  auto compute_tile = [&](int t, auto wait) {
#pragma unroll
    for (int kk = 0; kk + 1 < kKK; ++kk) {
      read_frags(t, kk + 1, (kk + 1) & 1);
      mfma_block(kk & 1);
    }
    wait();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < nk) read_frags(t + 1, 0, 0);
    mfma_block((kKK - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Prologue: tiles 0 .. STAGES-2 in flight, tile 0 landed and its first fragments read.
  for (int t = 0; t < STAGES - 1 && t < nk; ++t) copy_tile(t);
  if (nk >= STAGES - 1) wait_vmcnt<(STAGES - 2) * kLoads>();
  else wait_vmcnt<0>();
  lds_barrier();
  read_frags(0, 0, 0);

  int t = 0;
  // Steady state: the copy of tile t + STAGES - 1 refills the stage that every wave left at the
  // barrier of step t - 1; before the barrier of step t, tile t+1 must have landed.
  for (; t + STAGES - 1 < nk; ++t) {
    copy_tile(t + STAGES - 1);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile(t, [] { wait_vmcnt<(STAGES - 2) * kLoads>(); });
  }
  for (; t < nk; ++t) {
    const int newer = nk - 1 - (t + 1);  // tiles after t+1 still in flight
    compute_tile(t, [&] {
      if (newer >= 3) wait_vmcnt<(STAGES >= 5 ? 3 * kLoads : 0)>();
      else if (newer == 2) wait_vmcnt<(STAGES >= 4 ? 2 * kLoads : 0)>();
      else if (newer == 1) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
    });
  }

  // ---- One split: the output straight from the accumulators.  Lane l holds row (l & 31) and,
  // in register r, tile column 32*wave + 8*(r/4) + 4*(l/32) + r%4.
  if (p.splits == 1) {
#pragma unroll
    for (int mi = 0; mi < MB; ++mi) {
      const int row = m0 + mi * 32 + a_r;
      if (row >= p.M) continue;
      uint16_t* crow = p.C + (int64_t)row * p.ldc;
      if (MODE == kPlain) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = tile_n * kBN + wave * 32 + g * 8 + a_half * 4;
          if (col < p.N) {
            u32x2_t v;
            v.x = pack_bf16x2(acc[mi][4 * g + 0], acc[mi][4 * g + 1]);
            v.y = pack_bf16x2(acc[mi][4 * g + 2], acc[mi][4 * g + 3]);
            *reinterpret_cast<u32x2_t*>(crow + col) = v;
          }
        }
      } else {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int act = tile_n * (kBN / 2) + wave * 16 + g * 8 + a_half * 4;
          if (act < p.N) {
            float a[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = silu_mul(acc[mi][4 * g + e], acc[mi][8 + 4 * g + e]);
            u32x2_t v;
            v.x = pack_bf16x2(a[0], a[1]);
            v.y = pack_bf16x2(a[2], a[3]);
            *reinterpret_cast<u32x2_t*>(crow + act) = v;
          }
        }
      }
    }
    return;
  }

  // ---- Several splits: this split's fp32 partial tile -> workspace slice `split`.
  const int64_t slice = (int64_t)p.M * p.ws_ld;
  float* wtile = p.ws + tile_n * kBN;
#pragma unroll
  for (int mi = 0; mi < MB; ++mi) {
    const int row = m0 + mi * 32 + a_r;
    if (row < p.M) {
      float* dst = wtile + split * slice + (int64_t)row * p.ws_ld + wave * 32 + a_half * 4;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v = {acc[mi][4 * g], acc[mi][4 * g + 1], acc[mi][4 * g + 2], acc[mi][4 * g + 3]};
        *reinterpret_cast<float4*>(dst + g * 8) = v;
      }
    }
  }

}

// Sum of the splits' fp32 partials in ascending split order, then the epilogue.  One thread per 4
// consecutive outputs of one row; the loads of up to 8 splits are issued together.
template <int MODE>
__global__ __launch_bounds__(256) void splitk_finalize_kernel(const GemmParams p) {
  const int64_t groups_per_row = p.N / 4;  // N is a multiple of 8
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)p.M * groups_per_row) return;
  const int row = (int)(gid / groups_per_row);
  const int col = (int)(gid % groups_per_row) * 4;  // output (act) column
  const int64_t slice = (int64_t)p.M * p.ws_ld;
  // Workspace column of the first of the 4 outputs; in SiLU·up mode that of the gate input, the up
  // input being N columns further (the main kernel ran over the gate and up columns as two plain
  // column segments).
  const float* src = p.ws + (int64_t)row * p.ws_ld + col;
  float4 g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.splits; s0 += 8) {
    float4 vg[8], vu[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = s0 + j < p.splits;
      const float* q = src + (int64_t)(in ? s0 + j : 0) * slice;
      vg[j] = in ? *reinterpret_cast<const float4*>(q) : float4{0.f, 0.f, 0.f, 0.f};
      if (MODE == kSiluMul) vu[j] = in ? *reinterpret_cast<const float4*>(q + p.N) : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      g.x += vg[j].x; g.y += vg[j].y; g.z += vg[j].z; g.w += vg[j].w;
      if (MODE == kSiluMul) { u.x += vu[j].x; u.y += vu[j].y; u.z += vu[j].z; u.w += vu[j].w; }
    }
  }
  u32x2_t o;
  if (MODE == kSiluMul) {
    o.x = pack_bf16x2(silu_mul(g.x, u.x), silu_mul(g.y, u.y));
    o.y = pack_bf16x2(silu_mul(g.z, u.z), silu_mul(g.w, u.w));
  } else {
    o.x = pack_bf16x2(g.x, g.y);
    o.y = pack_bf16x2(g.z, g.w);
  }
  *reinterpret_cast<u32x2_t*>(p.C + (int64_t)row * p.ldc + col) = o;
}

template <int MODE, bool WNK, int MB>
void launch_one(const GemmParams& p, hipStream_t stream) {
  // LDS ring: MB 1, four stages (80 KiB: two workgroups per CU; three stages in flight, 8B TP=8 row
  // GEMM at 256 tokens 16.9 -> 14.9 us); MB 2, three (72 KiB, two per CU); MB 4, three (96 KiB).
  constexpr int kStages = MB == 1 ? 4 : 3;
  const unsigned grid = (unsigned)(p.splits * p.tiles_m * p.tiles_n);
  if (MODE == kSiluMul && p.splits > 1) {
    // Partial sums only: the gate and up columns run as two plain column segments of 2N outputs
    // (tile column c of tile j = output j*128 + c; the same tile count as the paired layout), so
    // that each k row of a [k][n] weight is read in 256-byte runs rather than 128-byte gate and up
    // halves; the finalize kernel pairs output j with output N + j.
    const GemmParams q = silu_as_plain_halves(p);
    hipLaunchKernelGGL((gemm_skinny_kernel<kPlain, WNK, MB, kStages>), dim3(grid), dim3(kThreads), 0,
                       stream, q);
  } else {
    hipLaunchKernelGGL((gemm_skinny_kernel<MODE, WNK, MB, kStages>), dim3(grid), dim3(kThreads), 0,
                       stream, p);
  }
  if (p.splits > 1) {
    const int64_t threads = (int64_t)p.M * (p.N / 4);
    hipLaunchKernelGGL((splitk_finalize_kernel<MODE>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, stream, p);
  }
}

template <int MODE, bool WNK>
void launch_mb(const GemmParams& p, int mb, hipStream_t stream) {
  if (mb == 1) launch_one<MODE, WNK, 1>(p, stream);
  else if (mb == 2) launch_one<MODE, WNK, 2>(p, stream);
  else launch_one<MODE, WNK, 4>(p, stream);
}

}  // namespace

hipError_t launch_splitk_finalize(const GemmParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.M * (p.N / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (p.mode == kSiluMul) hipLaunchKernelGGL((splitk_finalize_kernel<kSiluMul>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((splitk_finalize_kernel<kPlain>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const GemmParams& p, int mb, hipStream_t stream) {
  if (p.mode == kSiluMul)
    p.w_nk ? launch_mb<kSiluMul, true>(p, mb, stream) : launch_mb<kSiluMul, false>(p, mb, stream);
  else
    p.w_nk ? launch_mb<kPlain, true>(p, mb, stream) : launch_mb<kPlain, false>(p, mb, stream);
  return hipGetLastError();
}

}  // namespace ttl
