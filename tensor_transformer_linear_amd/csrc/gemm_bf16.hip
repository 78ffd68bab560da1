// Tiled bf16 GEMM on the CDNA4 matrix cores for the column- and row-parallel shards.
//
// C[M, N] = A[M, K] · B[K, map(N)] with A = the rank's input rows (k contiguous) and B = the
// unsharded weight W[k, n] (n contiguous), addressed in place: the rank's columns are chosen by a
// column map (plain slice, up to three q|k|v segments, or paired gate|up columns for the fused
// SiLU·up epilogue) and the rank's rows by the B base pointer.
//
// Workgroup tile 256 x 256 x 64, 256 threads = 4 wave64s in a 2 x 2 grid, each wave owning a
// 128 x 128 block as 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per lane, held in the
// accumulation registers).
//
// Data movement (gfx950):
//  * Global -> LDS without passing through registers: buffer_load_dwordx4 ... lds, 64 lanes x 16 B
//    = 1 KiB of LDS per instruction, lane i landing at byte 16*i of the instruction's block.  Each
//    lane picks the global piece that must land there, which is how the LDS layouts below get their
//    XOR swizzles.
//  * Two LDS stages (distinct __shared__ objects, so the compiler can tell the stage being read from
//    the one being filled): the copy of k-tile kt+1 is in flight while the matrix cores consume
//    k-tile kt; one wait + barrier per k-tile.
//  * A (X rows) is staged as [256 m][64 k]: 8 chunks of 16 B per 128-B row, chunk c stored at slot
//    c ^ (m % 8), so the 32 rows a 32 x 32 block reads at one k-chunk spread over all banks.
//  * B (W rows) is staged as loaded, [64 k][256 n]: 32 chunks per 512-B row, chunk c stored at slot
//    c ^ (2 * (k % 4)).  The matrix cores want 8 consecutive k of one n per lane; ds_read_b64_tr_b16
//    returns, in each 16-lane group, the transpose of a 4 (k) x 16 (n) block — lane j of the group
//    addresses row k0 + j/4 at n0 + 4*(j%4) and receives k0..k0+3 at n0 + j — so two such reads
//    build one operand with no transpose in registers.  The swizzle puts the 4 rows x 32 B of one
//    group read on distinct banks.
//  * Tiles are ordered for the L2 of each XCD: consecutive workgroups go to different XCDs, so the
//    block index is remapped so that each XCD works on a compact group of tiles (4 row-tiles wide)
//    that share A rows and W columns in its L2.
//
// Tails in M, N and K: buffer loads whose offsets are pushed past the record count return zeros, so
// the k-tail contributes exact zeros and no branch sits in the main loop; stores are masked.
#include "kernels.h"

namespace ttl {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

constexpr int kBM = 256;
constexpr int kBN = 256;                  // weight columns per tile
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kTileElems = kBM * kBK;     // A or B stage, bf16 elements (32 KiB)
constexpr int kLoadsPerOperand = kTileElems * 2 / (kThreads * 16);  // 16-B pieces per thread = 8
constexpr int kXcds = 8;                  // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kGroupM = 4;                // row-tiles per L2 group
constexpr uint32_t kOob = 0x80000000u;    // beyond every record count used below
constexpr int32_t kMaxRecords = 0x7FFFFFF0;

enum { kPlain = 0, kSiluMul = 1 };

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t rec = bytes <= 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : (int32_t)bytes);
  // dword3 = 0x00020000: 32-bit data format, the raw (untyped) buffer setting for gfx9 parts.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, rec, 0x00020000);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));  // round to nearest even
}

__device__ inline float silu_mul(float g, float u) {
  // silu(g) * u with silu(g) = g / (1 + exp(-g)); exp overflow gives rcp(inf) = 0, i.e. silu -> -0.
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// The LDS stages: one distinct object per (stage, operand).
template <int S> __device__ inline uint16_t* stage_a() {
  __shared__ __attribute__((aligned(1024))) uint16_t buf[kTileElems];
  return buf;
}
template <int S> __device__ inline uint16_t* stage_b() {
  __shared__ __attribute__((aligned(1024))) uint16_t buf[kTileElems];
  return buf;
}

// Remap the block index so that the tiles one XCD runs form compact groups, then walk tiles in
// groups of kGroupM row-tiles.  Both maps are bijections on [0, tiles).
__device__ inline void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int tiles = tiles_m * tiles_n;
  const int q = tiles / kXcds, r = tiles % kXcds;
  const int x = bid % kXcds, local = bid / kXcds;
  const int L = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
  const int per_group = kGroupM * tiles_n;
  const int g = L / per_group;
  const int first = g * kGroupM;
  const int gsize = min(tiles_m - first, kGroupM);
  const int inner = L - g * per_group;
  tm = first + inner % gsize;
  tn = inner / gsize;
}

template <int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const GemmParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  int tile_m, tile_n;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tile_m, tile_n);
  const int m0 = tile_m * kBM;
  const int n0 = tile_n * (MODE == kSiluMul ? kBN / 2 : kBN);  // first output column of the tile

  // ---- A copy: piece i of this thread is instruction q = wave*8 + i, rows 8q + lane/8, and the
  // slot lane%8 of the row holds k-chunk (lane%8) ^ (row%8) = (lane%8) ^ (lane/8).
  const int a_row0 = wave * 64 + (lane >> 3);               // + 8*i
  const int a_chunk = (lane & 7) ^ (lane >> 3);
  uint32_t a_rowmask = 0;
#pragma unroll
  for (int i = 0; i < kLoadsPerOperand; ++i)
    if (m0 + a_row0 + 8 * i < p.M) a_rowmask |= 1u << i;

  // ---- B copy: instruction q = wave*8 + i covers k rows 2q, 2q+1; lane -> row 2q + lane/32,
  // slot lane%32, which holds chunk (lane%32) ^ (2*(row%4)).  row%4 = 2*(i%2) + lane/32.
  int64_t b_wcol[2];
  uint32_t b_colok = 0;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int krow4 = 2 * par + (lane >> 5);
    const int chunk = (lane & 31) ^ (2 * krow4);
    const int c = chunk * 8;  // tile column of the chunk's first element
    int64_t wcol;
    bool ok;
    if (MODE == kSiluMul) {
      // Tile column c = w*128 + nb*32 + j: blocks nb = 0,1 are gate columns and nb = 2,3 the up
      // columns of the same act columns, so gate and up of one output meet in one lane.
      const int w = c >> 7, nb = (c & 127) >> 5, j = c & 31;
      const int act = n0 + w * 64 + (nb & 1) * 32 + j;
      ok = act < p.N;
      wcol = (nb < 2 ? p.gate_w0 : p.up_w0) + act;
    } else {
      const int oc = n0 + c;
      ok = oc < p.N;
      int64_t w0 = p.seg_w0[0];
      int s0 = p.seg_out0[0];
      if (p.nseg > 1 && oc >= p.seg_out0[1]) { w0 = p.seg_w0[1]; s0 = p.seg_out0[1]; }
      if (p.nseg > 2 && oc >= p.seg_out0[2]) { w0 = p.seg_w0[2]; s0 = p.seg_out0[2]; }
      wcol = w0 + (oc - s0);
    }
    b_wcol[par] = wcol;
    if (ok) b_colok |= 1u << par;
  }

  const int nk = (p.K + kBK - 1) / kBK;

  auto copy_tile = [&](int kt, uint16_t* sa, uint16_t* sb) {
    const int k0 = kt * kBK;
    const __amdgpu_buffer_rsrc_t ar =
        make_rsrc(p.A + (int64_t)m0 * p.lda + k0, ((int64_t)(p.M - m0 - 1) * p.lda + (p.K - k0)) * 2);
    const bool a_kok = k0 + a_chunk * 8 < p.K;
#pragma unroll
    for (int i = 0; i < kLoadsPerOperand; ++i) {
      const uint32_t off = (uint32_t)(((int64_t)(a_row0 + 8 * i) * p.lda + a_chunk * 8) * 2);
      const uint32_t ok = (uint32_t)a_kok & (a_rowmask >> i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void*)(sa + (wave * 8 + i) * 512), 16,
                                               off | (((ok & 1u) - 1u) & kOob), 0, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t br =
        make_rsrc(p.B + (int64_t)k0 * p.ldb, (int64_t)(p.K - k0) * p.ldb * 2);
#pragma unroll
    for (int i = 0; i < kLoadsPerOperand; ++i) {
      const int q = wave * 8 + i;
      const int krow = 2 * q + (lane >> 5);
      const int par = i & 1;
      const uint32_t off = (uint32_t)(((int64_t)krow * p.ldb + b_wcol[par]) * 2);
      const uint32_t ok = ((b_colok >> par) & 1u) & (uint32_t)(k0 + krow < p.K);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void*)(sb + q * 512), 16,
                                               off | ((ok - 1u) & kOob), 0, 0, 0);
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // Per-lane LDS read offsets (elements), split into a per-lane part and compile-time constants.
  // A: row wm*128 + mi*32 + lane%32, k-chunk kk*2 + lane/32, stored at slot chunk ^ (row % 8);
  //    row % 8 = lane % 8, so slot = ((kk ^ s1) << 1) | (lane/32 ^ s0) with s = lane % 8.
  // B: 16-lane group g = lane/16 reads k row kk*16 + 8*(g/2) + 4*h + (lane%16)/4 at
  //    n = wn*128 + ni*32 + 16*(g%2) + 4*(lane%4); its chunk n/8 = 16*wn + 4*ni + c with
  //    c = 2*(g%2) + (lane%4)/2 is stored at slot chunk ^ (2*(k%4)), k%4 = (lane%16)/4, and only
  //    the parity of ni reaches the XOR.
  const int a_r = lane & 31;
  const int a_half = lane >> 5;
  int a_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int slot = (((kk ^ ((a_r & 7) >> 1)) << 1) | (a_half ^ (a_r & 1)));
    a_off[kk] = (wm * 128 + a_r) * kBK + slot * 8;
  }
  int b_off[2];
  {
    const int krow = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int x = 2 * ((lane & 15) >> 2);
    const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int slot = (16 * wn + 4 * par + c) ^ x;
      b_off[par] = krow * kBN + slot * 8 + 4 * (lane & 1);
    }
  }

  auto read_frags = [&](const uint16_t* sa, const uint16_t* sb, int kk, bf16x8_t* af, bf16x8_t* bv) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      af[mi] = *reinterpret_cast<const bf16x8_t*>(sa + a_off[kk] + mi * 32 * kBK);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const uint16_t* base = sb + b_off[ni & 1] + kk * 16 * kBN + (ni >> 1) * 64;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 4 * kBN));
      bv[ni] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  auto compute = [&](const uint16_t* sa, const uint16_t* sb) {
    bf16x8_t af[2][4], bv[2][4];
    read_frags(sa, sb, 0, af[0], bv[0]);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < kBK / 16) read_frags(sa, sb, kk + 1, af[cur ^ 1], bv[cur ^ 1]);
      // Weight block as the first operand: lane l then holds output row (l & 31) and, in
      // accumulator register r, output column 8*(r/4) + 4*(l/32) + r%4 of the 32 x 32 block.
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[cur][ni], af[cur][mi], acc[mi][ni], 0, 0, 0);
    }
  };

  // Two-stage pipeline, unrolled by two so that every access names its stage object statically;
  // an odd last k-tile is peeled so that the loop has a single exit.
  copy_tile(0, stage_a<0>(), stage_b<0>());
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    copy_tile(kt + 1, stage_a<1>(), stage_b<1>());
    __builtin_amdgcn_sched_barrier(0);
    compute(stage_a<0>(), stage_b<0>());
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 2 < nk) copy_tile(kt + 2, stage_a<0>(), stage_b<0>());
    __builtin_amdgcn_sched_barrier(0);
    compute(stage_a<1>(), stage_b<1>());
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (kt < nk) compute(stage_a<0>(), stage_b<0>());

  // Epilogue straight from the accumulators: each lane owns 4 consecutive columns of one row per
  // register group, stored as one 8-byte piece.
  const int row_base = m0 + wm * 128 + a_r;
  if (MODE == kPlain) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int row = row_base + mi * 32;
      if (row >= p.M) continue;
      uint16_t* crow = p.C + (int64_t)row * p.ldc;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn * 128 + ni * 32 + g * 8 + a_half * 4;
          if (col < p.N) {
            u32x2_t v;
            v.x = pack_bf16x2(acc[mi][ni][4 * g + 0], acc[mi][ni][4 * g + 1]);
            v.y = pack_bf16x2(acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]);
            *reinterpret_cast<u32x2_t*>(crow + col) = v;
          }
        }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int row = row_base + mi * 32;
      if (row >= p.M) continue;
      uint16_t* crow = p.C + (int64_t)row * p.ldc;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn * 64 + ni * 32 + g * 8 + a_half * 4;
          if (col < p.N) {
            float a[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = silu_mul(acc[mi][ni][4 * g + e], acc[mi][ni + 2][4 * g + e]);
            u32x2_t v;
            v.x = pack_bf16x2(a[0], a[1]);
            v.y = pack_bf16x2(a[2], a[3]);
            *reinterpret_cast<u32x2_t*>(crow + col) = v;
          }
        }
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
  const dim3 block(kThreads);
  if (p.mode == kSiluMul)
    hipLaunchKernelGGL(gemm_bf16_kernel<kSiluMul>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<kPlain>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace ttl
