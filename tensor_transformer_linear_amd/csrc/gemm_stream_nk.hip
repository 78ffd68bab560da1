// Split-free GEMM for few token rows with the weight stored [n][k] (decode batches of at most 64
// rows): no k splits across workgroups, so no fp32 partials in HBM and no second kernel.
//
// Decode is bound by reading the weight slice once from HBM.  With [n][k] storage, the 16 bytes a
// lane needs for one 16 x 16 x 32 product (8 consecutive k of one weight column) are contiguous in
// memory, so fragments load straight into registers: no LDS staging.  A workgroup owns 32 weight
// columns (rows of the stored W^T) over the whole of k: 32 output columns, or in SiLU·up mode 16
// act columns with their gate and up columns.  Its four waves cut k into four contiguous quarters
// and keep kDepth k32 steps of loads in flight each (every load of step s + kDepth is issued as
// step s is multiplied); the four partial sums are then added through LDS in wave order, so every
// output is reproducible bit for bit.  Each workgroup reads all of X (at most 64 rows), which the
// L2 of its XCD serves after the first.
//
// Lane layouts (the 16 x 16 x 32 kernel's): the weight fragment is the first operand, lane l
// holding weight column l % 16 of the block and k = 8 (l / 16) .. + 7 of the k32 step; the
// activation fragment is the second, lane l holding token row l % 16 and the same k; accumulator
// register r of lane l is token row l % 16, output column 4 (l / 16) + r of the block.  Fragment j
// of a workgroup is weight columns 16 j .. 16 j + 15 of its 32 (SiLU·up: j = 0 the gate, j = 1
// the up columns of the same act columns, which then meet in one lane and register).
//
// Token rows past M read zeros through the activation descriptor's range; weight columns past N
// read zeros through an out-of-range offset.  K must be a multiple of 32, and at least 2048 (each
// wave at least 2 kDepth k32 steps).
#include "gemm_common.h"

namespace ttl {
namespace {

using namespace gemm;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = 32;   // weight columns per workgroup
constexpr int kDepth = 8;   // k32 steps of loads in flight per wave

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int32_t rec = bytes <= 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, rec, 0x00020000);
}

__device__ inline bf16x8_t load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// RB: 16-row blocks of tokens (1, 2 or 4: M <= 16, 32, 64).
template <int MODE, int RB>
__global__ __launch_bounds__(kThreads) void gemm_stream_nk_kernel(const GemmParams p) {
  __shared__ f32x4_t red[kWaves][RB][2][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  constexpr int kOut = MODE == kSiluMul ? kCols / 2 : kCols;  // output columns per workgroup
  const int c0 = (int)blockIdx.x * kOut;

  // This lane's weight column (row of W^T) in fragments 0 and 1.
  uint32_t woff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bool ok;
    int64_t wrow;
    if constexpr (MODE == kSiluMul) {
      const int act = c0 + r16;
      ok = act < p.N;
      wrow = (j == 0 ? p.gate_w0 : p.up_w0) + act;
    } else {
      const int oc = c0 + 16 * j + r16;
      ok = oc < p.N;
      int64_t w0 = p.seg_w0[0];
      int s0 = p.seg_out0[0];
      if (p.nseg > 1 && oc >= p.seg_out0[1]) { w0 = p.seg_w0[1]; s0 = p.seg_out0[1]; }
      if (p.nseg > 2 && oc >= p.seg_out0[2]) { w0 = p.seg_w0[2]; s0 = p.seg_out0[2]; }
      wrow = w0 + (oc - s0);
    }
    woff[j] = ok ? (uint32_t)((wrow * p.ldb + 8 * g4) * 2) : kOob;
  }
  uint32_t xoff[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) xoff[i] = (uint32_t)(((int64_t)(16 * i + r16) * p.lda + 8 * g4) * 2);
  const __amdgpu_buffer_rsrc_t wd = rsrc(p.B, ((int64_t)(p.b_rows - 1) * p.ldb + p.K) * 2);
  const __amdgpu_buffer_rsrc_t xd = rsrc(p.A, ((int64_t)(p.M - 1) * p.lda + p.K) * 2);

  // This wave's k32 steps.
  const int steps = p.K / 32;
  const int s0 = wave * steps / kWaves, ns = (wave + 1) * steps / kWaves - s0;

  f32x4_t acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  bf16x8_t wf[kDepth][2], xf[kDepth][RB];
  auto load = [&](int d, int s) {
    const uint32_t kb = (uint32_t)(s0 + s) * 64u;
#pragma unroll
    for (int j = 0; j < 2; ++j) wf[d][j] = load16(wd, woff[j] + kb);
#pragma unroll
    for (int i = 0; i < RB; ++i) xf[d][i] = load16(xd, xoff[i] + kb);
  };
  auto mfma = [&](int d) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[d][j], xf[d][i], acc[i][j], 0, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load(d, d);  // ns >= 2 kDepth (the host checks K)
  // Steady state, without branches, so that the compiler's waits keep the ring full (step d's
  // fragments are waited for with the loads of the kDepth - 1 later steps still in flight).
  int s = 0;
  for (; s + 2 * kDepth <= ns; s += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      mfma(d);
      load(d, s + d + kDepth);
    }
  }
  // The last kDepth .. 2 kDepth - 1 steps.
#pragma unroll
  for (int d = 0; d < 2 * kDepth; ++d) {
    if (s + d < ns) {
      mfma(d % kDepth);
      if (s + d + kDepth < ns) load(d % kDepth, s + d + kDepth);
    }
  }

  // The four waves' partial sums, added in wave order; wave w finishes token-row block w.
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) red[wave][i][j][lane] = acc[i][j];
  __syncthreads();
  if (wave >= RB) return;
  const int i = wave;
  f32x4_t v[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    v[j] = red[0][i][j][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v[j] += red[w][i][j][lane];
  }
  const int row = 16 * i + r16;
  if (row >= p.M) return;
  uint16_t* crow = p.C + (int64_t)row * p.ldc;
  if constexpr (MODE == kSiluMul) {
    const int col = c0 + 4 * g4;
    if (col < p.N) {
      u32x2_t o;
      o.x = pack_bf16x2(silu_mul(v[0][0], v[1][0]), silu_mul(v[0][1], v[1][1]));
      o.y = pack_bf16x2(silu_mul(v[0][2], v[1][2]), silu_mul(v[0][3], v[1][3]));
      *reinterpret_cast<u32x2_t*>(crow + col) = o;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = c0 + 16 * j + 4 * g4;
      if (col < p.N) {
        u32x2_t o;
        o.x = pack_bf16x2(v[j][0], v[j][1]);
        o.y = pack_bf16x2(v[j][2], v[j][3]);
        *reinterpret_cast<u32x2_t*>(crow + col) = o;
      }
    }
  }
}

template <int MODE>
void launch_mode(const GemmParams& p, unsigned grid, hipStream_t stream) {
  if (p.M <= 16) hipLaunchKernelGGL((gemm_stream_nk_kernel<MODE, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
  else if (p.M <= 32) hipLaunchKernelGGL((gemm_stream_nk_kernel<MODE, 2>), dim3(grid), dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL((gemm_stream_nk_kernel<MODE, 4>), dim3(grid), dim3(kThreads), 0, stream, p);
}

}  // namespace

int64_t gemm_stream_nk_workgroups(const GemmParams& p) {
  const int out = p.mode == kSiluMul ? kCols / 2 : kCols;
  return ((int64_t)p.N + out - 1) / out;
}

bool gemm_stream_nk_supports(const GemmParams& p) {
  // every wave takes at least 2 kDepth k32 steps
  return p.w_nk != 0 && p.M >= 1 && p.M <= 64 && p.K % 32 == 0 && p.K >= 32 * kWaves * 2 * kDepth &&
         p.N > 0;
}

hipError_t launch_gemm_stream_nk(const GemmParams& p, hipStream_t stream) {
  if (!gemm_stream_nk_supports(p)) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)gemm_stream_nk_workgroups(p);
  if (p.mode == kSiluMul) launch_mode<kSiluMul>(p, grid, stream);
  else launch_mode<kPlain>(p, grid, stream);
  return hipGetLastError();
}

}  // namespace ttl
