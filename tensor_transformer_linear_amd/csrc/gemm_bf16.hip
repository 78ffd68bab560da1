// Tiled bf16 GEMM on the CDNA4 matrix cores for the column- and row-parallel shards.
//
// C[M, N] = A[M, K] · B[K, map(N)] with A = the rank's input rows (k contiguous) and B = the
// unsharded weight W[k, n] (n contiguous), addressed in place: the rank's columns are chosen by a
// column map (plain slice, up to three q|k|v segments, or paired gate|up columns for the fused
// SiLU·up epilogue) and the rank's rows by the B base pointer.
//
// Workgroup tile 256 x 256 x 64, 256 threads = 4 wave64s in a 2 x 2 grid, each wave owning a
// 128 x 128 block as 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per lane).
// Global -> register -> LDS staging with two LDS stages: the loads of k-tile kt+1 are in flight
// while the matrix cores consume k-tile kt, and one barrier per k-tile separates the stages.
//
// The matrix cores want, per lane, 8 consecutive k values of one row of each operand.  X rows
// already are k-contiguous; W is n-contiguous, so each thread loads an 8(k) x 8(n) block of W as
// eight 16-byte row pieces and transposes it in registers before its LDS store, leaving both
// staged operands as [row][k] with a 144-byte row pitch (64 k + 8 pad), which keeps the 16-byte LDS
// reads and writes of a wave on distinct banks.
//
// Tails in M, N and K are handled by buffer loads whose offsets are pushed past the record count
// (the hardware returns zeros), so the k-tail contributes exact zeros and no branch sits in the
// inner loop; stores are masked per 16-byte piece.
#include "kernels.h"

namespace ttl {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 256;
constexpr int kBN = 256;                          // weight columns per tile
constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;                   // bf16 per staged row (144 bytes)
constexpr int kStage = (kBM + kBN) * kPitch;      // elements of one A+B stage
constexpr int kThreads = 256;
constexpr uint32_t kOob = 0x80000000u;            // beyond every record count used below
constexpr int32_t kMaxRecords = 0x7FFFFFF0;       // records are clamped below kOob

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

__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const int tile_n = blockIdx.x % p.tiles_n;
  const int tile_m = blockIdx.x / p.tiles_n;
  const bool silu = p.mode == 1;
  const int m0 = tile_m * kBM;
  const int n0 = tile_n * (silu ? kBN / 2 : kBN);  // first output column of the tile

  // A loader: 8 rows (a_row + 32 i) x one 16-byte k piece per thread per k-tile.
  const int a_row = tid >> 3;
  const int a_kc = (tid & 7) * 8;
  uint32_t a_rowmask = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (m0 + a_row + 32 * i < p.M) a_rowmask |= 1u << i;

  // B loader: rows b_kg*8 .. +7 of the k-tile, tile columns b_cg .. b_cg+7.
  const int b_kg = tid & 7;
  const int b_cg = (tid >> 3) * 8;
  int64_t wcol;
  bool col_ok;
  if (silu) {
    // Tile column c = wn*128 + ni*32 + w: blocks ni = 0,1 are gate columns and ni = 2,3 the up
    // columns of the same act columns, so gate and up of one output land in the same lane.
    const int wq = b_cg >> 7, ni = (b_cg & 127) >> 5, w = b_cg & 31;
    const int act = n0 + wq * 64 + (ni & 1) * 32 + w;
    col_ok = act < p.N;
    wcol = (ni < 2 ? p.gate_w0 : p.up_w0) + act;
  } else {
    const int oc = n0 + b_cg;
    col_ok = oc < p.N;
    int64_t w0 = p.seg_w0[0];
    int s0 = p.seg_out0[0];
    if (p.nseg > 1 && oc >= p.seg_out0[1]) { w0 = p.seg_w0[1]; s0 = p.seg_out0[1]; }
    if (p.nseg > 2 && oc >= p.seg_out0[2]) { w0 = p.seg_w0[2]; s0 = p.seg_out0[2]; }
    wcol = w0 + (oc - s0);
  }

  const int nk = (p.K + kBK - 1) / kBK;
  u32x4_t ra[8], rb[8];

  auto gload = [&](int kt) {
    const int k0 = kt * kBK;
    const uint16_t* abase = p.A + (int64_t)m0 * p.lda + k0;
    const __amdgpu_buffer_rsrc_t ar =
        make_rsrc(abase, ((int64_t)(p.M - m0 - 1) * p.lda + (p.K - k0)) * 2);
    const bool kok = k0 + a_kc < p.K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = (uint32_t)(((int64_t)(a_row + 32 * i) * p.lda + a_kc) * 2);
      const uint32_t ok = (uint32_t)kok & (a_rowmask >> i);
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, off | ((ok & 1u) - 1u & kOob), 0, 0);
    }
    const uint16_t* bbase = p.B + (int64_t)k0 * p.ldb;
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bbase, (int64_t)(p.K - k0) * p.ldb * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kr = b_kg * 8 + i;
      const uint32_t off = (uint32_t)(((int64_t)kr * p.ldb + wcol) * 2);
      const uint32_t ok = (uint32_t)col_ok & (uint32_t)(k0 + kr < p.K);
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(br, off | ((ok - 1u) & kOob), 0, 0);
    }
  };

  auto swrite = [&](int stage) {
    uint16_t* As = lds + stage * kStage;
    uint16_t* Bs = As + kBM * kPitch;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4_t*>(&As[(a_row + 32 * i) * kPitch + a_kc]) = ra[i];
    // 8 x 8 transpose: output column j gathers element j of the eight k rows.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = j >> 1;
      u32x4_t o;
      if ((j & 1) == 0) {
        o.x = (rb[0][d] & 0xFFFFu) | (rb[1][d] << 16);
        o.y = (rb[2][d] & 0xFFFFu) | (rb[3][d] << 16);
        o.z = (rb[4][d] & 0xFFFFu) | (rb[5][d] << 16);
        o.w = (rb[6][d] & 0xFFFFu) | (rb[7][d] << 16);
      } else {
        o.x = (rb[0][d] >> 16) | (rb[1][d] & 0xFFFF0000u);
        o.y = (rb[2][d] >> 16) | (rb[3][d] & 0xFFFF0000u);
        o.z = (rb[4][d] >> 16) | (rb[5][d] & 0xFFFF0000u);
        o.w = (rb[6][d] >> 16) | (rb[7][d] & 0xFFFF0000u);
      }
      *reinterpret_cast<u32x4_t*>(&Bs[(b_cg + j) * kPitch + b_kg * 8]) = o;
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int r32 = lane & 31;
  const int kh = (lane >> 5) * 8;
  auto compute = [&](int stage) {
    const uint16_t* As = lds + stage * kStage;
    const uint16_t* Bs = As + kBM * kPitch;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8_t af[4], bv[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 128 + mi * 32 + r32) * kPitch + kk * 16 + kh]);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bv[ni] = *reinterpret_cast<const bf16x8_t*>(&Bs[(wn * 128 + ni * 32 + r32) * kPitch + kk * 16 + kh]);
      // Weight block as the first operand: lane l then holds output row (l & 31) and, in
      // accumulator register r, output column 8*(r/4) + 4*(l/32) + r%4 of the 32 x 32 block.
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[ni], af[mi], acc[mi][ni], 0, 0, 0);
    }
  };

  gload(0);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    compute(kt & 1);
    if (more) swrite((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue: convert to bf16 through LDS so that global stores are whole 16-byte row pieces.
  uint16_t* Cs = lds;
  const int half = lane >> 5;
  if (!silu) {
    constexpr int kCp = kBN + 8;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = wm * 128 + mi * 32 + r32;
          const int col = wn * 128 + ni * 32 + g * 8 + half * 4;
          u32x2_t v;
          v.x = pack_bf16x2(acc[mi][ni][4 * g + 0], acc[mi][ni][4 * g + 1]);
          v.y = pack_bf16x2(acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]);
          *reinterpret_cast<u32x2_t*>(&Cs[row * kCp + col]) = v;
        }
    __syncthreads();
    for (int idx = tid; idx < kBM * (kBN / 8); idx += kThreads) {
      const int row = idx / (kBN / 8), ch = idx % (kBN / 8);
      const int gr = m0 + row, gc = n0 + ch * 8;
      if (gr < p.M && gc < p.N)
        *reinterpret_cast<u32x4_t*>(&p.C[(int64_t)gr * p.ldc + gc]) =
            *reinterpret_cast<const u32x4_t*>(&Cs[row * kCp + ch * 8]);
    }
  } else {
    constexpr int kCp = kBN / 2 + 8;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = wm * 128 + mi * 32 + r32;
          const int col = wn * 64 + ni * 32 + g * 8 + half * 4;
          float a[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = silu_mul(acc[mi][ni][4 * g + e], acc[mi][ni + 2][4 * g + e]);
          u32x2_t v;
          v.x = pack_bf16x2(a[0], a[1]);
          v.y = pack_bf16x2(a[2], a[3]);
          *reinterpret_cast<u32x2_t*>(&Cs[row * kCp + col]) = v;
        }
    __syncthreads();
    for (int idx = tid; idx < kBM * (kBN / 16); idx += kThreads) {
      const int row = idx / (kBN / 16), ch = idx % (kBN / 16);
      const int gr = m0 + row, gc = n0 + ch * 8;
      if (gr < p.M && gc < p.N)
        *reinterpret_cast<u32x4_t*>(&p.C[(int64_t)gr * p.ldc + gc]) =
            *reinterpret_cast<const u32x4_t*>(&Cs[row * kCp + ch * 8]);
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
  const dim3 block(kThreads);
  hipLaunchKernelGGL(gemm_bf16_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace ttl
