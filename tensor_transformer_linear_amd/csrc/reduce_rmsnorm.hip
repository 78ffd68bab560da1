// Sum of t simulated-rank partials + residual add + RMSNorm, one pass over HBM.  The partials are
// either t slabs of one [t][b][n] buffer or t separate [b][n] buffers (one pointer per rank, as a
// reduction over peers' buffers would see them).
//
// One workgroup per token row.  Each thread owns CPT pieces of 8 consecutive bf16 columns
// (piece c = tid + THREADS*j), read with 16-byte loads so that a wave covers 1 KiB of a row per
// load instruction.  The loads of RANKS partials are issued together before any of them is added,
// so a thread has up to RANKS*CPT 16-byte loads in flight and a row needs about t/RANKS memory
// round trips instead of t + 1.  The row's fp32 sum h stays in registers from the partial-sum pass
// to the normalisation pass, so every byte is read once and written once:
//   s = P_0 + P_1 + ... + P_{t-1}   (fp32, ascending rank: fixed order, bitwise reproducible)
//   h = s + residual                 (fp32); residual_out = bf16(h)
//   y = bf16(h * rsqrt(mean(h^2) + eps) * gamma)
// The mean square is reduced within each wave by butterfly shuffles and across waves through LDS
// in wave order, again a fixed order.
#include "kernels.h"

namespace ttl {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// The partials, the residual and both outputs are touched once: their loads and stores carry the
// non-temporal hint (measured: ~80% of HBM bandwidth with it against ~66% without, at t = 8,
// b = 4096, n = 8192).  gamma, read by every row, is loaded normally.
__device__ inline u32x4_t load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ inline void store_stream(uint16_t* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

__device__ inline void add_piece(float* h, u32x4_t v) {
  h[0] += lo_bf16(v.x); h[1] += hi_bf16(v.x);
  h[2] += lo_bf16(v.y); h[3] += hi_bf16(v.y);
  h[4] += lo_bf16(v.z); h[5] += hi_bf16(v.z);
  h[6] += lo_bf16(v.w); h[7] += hi_bf16(v.w);
}

template <int CPT, int THREADS, int RANKS, bool RES_JOIN>
__global__ __launch_bounds__(THREADS) void reduce_rmsnorm_kernel(const ReduceNormParams p) {
  constexpr int kWaves = THREADS / 64;
  __shared__ float wave_sums[kWaves];

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t n = p.n;
  const int pieces = (int)(n >> 3);
  const int64_t plane = p.plane;  // elements between consecutive ranks' partials

  float h[CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) h[j][e] = 0.0f;

  const uint16_t* prow = p.P + row * n;
  const uint16_t* rrow = p.residual != nullptr ? p.residual + row * n : nullptr;
  for (int r0 = 0; r0 < p.t; r0 += RANKS) {
    u32x4_t v[RANKS][CPT];
#pragma unroll
    for (int rr = 0; rr < RANKS; ++rr) {
      const int r = r0 + rr < p.t ? r0 + rr : p.t - 1;  // loads past t are skipped below
      const uint16_t* src = p.peers ? p.peer[r] + row * n : prow + (int64_t)r * plane;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = tid + THREADS * j;
        if (r0 + rr < p.t && c < pieces) v[rr][j] = load_stream(src + (int64_t)c * 8);
      }
    }
    // The residual joins the last group's loads (when registers allow); it is added after every
    // partial.
    u32x4_t res[CPT];
    const bool last = RES_JOIN && r0 + RANKS >= p.t;
    if (last && rrow != nullptr) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = tid + THREADS * j;
        if (c < pieces) res[j] = load_stream(rrow + (int64_t)c * 8);
      }
    }
#pragma unroll
    for (int rr = 0; rr < RANKS; ++rr)
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = tid + THREADS * j;
        if (r0 + rr < p.t && c < pieces) add_piece(h[j], v[rr][j]);
      }
    if (last && rrow != nullptr) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = tid + THREADS * j;
        if (c < pieces) add_piece(h[j], res[j]);
      }
    }
  }
  if (!RES_JOIN && rrow != nullptr) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + THREADS * j;
      if (c < pieces) add_piece(h[j], load_stream(rrow + (int64_t)c * 8));
    }
  }

  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += h[j][e] * h[j][e];  // pieces past n hold zeros
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((tid & 63) == 0) wave_sums[tid >> 6] = ss;
  __syncthreads();
  float total = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += wave_sums[w];
  const float inv = __frsqrt_rn(total / (float)n + p.eps);

  uint16_t* rout = p.residual_out + row * n;
  uint16_t* yrow = p.Y + row * n;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = tid + THREADS * j;
    if (c < pieces) {
      const u32x4_t g = *reinterpret_cast<const u32x4_t*>(p.gamma + (int64_t)c * 8);
      u32x4_t ro, yo;
      ro.x = pack_bf16x2(h[j][0], h[j][1]);
      ro.y = pack_bf16x2(h[j][2], h[j][3]);
      ro.z = pack_bf16x2(h[j][4], h[j][5]);
      ro.w = pack_bf16x2(h[j][6], h[j][7]);
      yo.x = pack_bf16x2(h[j][0] * inv * lo_bf16(g.x), h[j][1] * inv * hi_bf16(g.x));
      yo.y = pack_bf16x2(h[j][2] * inv * lo_bf16(g.y), h[j][3] * inv * hi_bf16(g.y));
      yo.z = pack_bf16x2(h[j][4] * inv * lo_bf16(g.z), h[j][5] * inv * hi_bf16(g.z));
      yo.w = pack_bf16x2(h[j][6] * inv * lo_bf16(g.w), h[j][7] * inv * hi_bf16(g.w));
      store_stream(rout + (int64_t)c * 8, ro);
      store_stream(yrow + (int64_t)c * 8, yo);
    }
  }
}

template <int CPT, int THREADS, int RANKS>
hipError_t launch(const ReduceNormParams& p, hipStream_t stream) {
  // The residual joins the last group of partial loads when the registers allow it.
  constexpr int kLoadBudget = THREADS >= 1024 ? 12 : 32;
  constexpr bool kResJoin = (RANKS + 1) * CPT <= kLoadBudget;
  hipLaunchKernelGGL((reduce_rmsnorm_kernel<CPT, THREADS, RANKS, kResJoin>), dim3((unsigned)p.b),
                     dim3(THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce_rmsnorm(const ReduceNormParams& p, hipStream_t stream) {
  const int64_t pieces = p.n / 8;  // n <= 65536, checked by the caller
  if (p.b >= 1024) {
    // Many rows (prefill): a few hundred threads per row; the rows in flight per CU keep HBM busy.
    // How many rows fit on the chip at once depends on the shape (pieces per thread, threads per
    // row, loads in flight), and a row count just above a whole number of such rounds leaves a slow
    // last round.  The shapes for n = 4096 and 8192 were measured at the rows of the workloads with
    // operands rotated through more than 512 MB (HBM, not the Infinity Cache): one partial's loads
    // in flight per thread (the residual joining the last) gives more rows in flight than several,
    // n = 4096, t = 4, b = 2048: 20.3 against 23.7-24.2 us (5.8 TB/s); n = 8192, t = 8: 67.8 and
    // 121.9 us at b = 2176 and 4096, against 68.8 and 124.0.
    if (pieces <= 64) return launch<1, 64, 4>(p, stream);
    if (pieces <= 128) return launch<1, 128, 4>(p, stream);
    if (pieces <= 256) return launch<1, 256, 4>(p, stream);
    if (pieces <= 512) return p.b <= 2560 ? launch<4, 128, 1>(p, stream) : launch<1, 512, 2>(p, stream);
    if (pieces <= 1024) return launch<2, 512, 1>(p, stream);
    if (pieces <= 2048) return launch<8, 256, 2>(p, stream);
    if (pieces <= 4096) return launch<4, 1024, 2>(p, stream);
    return launch<8, 1024, 1>(p, stream);
  }
  // Few rows (decode): each row spread over up to 1024 threads with all of a thread's partial loads
  // in flight, since only b of the CUs have work.
  if (pieces <= 64) return launch<1, 64, 8>(p, stream);
  if (pieces <= 128) return launch<1, 128, 8>(p, stream);
  if (pieces <= 256) return launch<1, 256, 8>(p, stream);
  if (pieces <= 512) return launch<1, 512, 8>(p, stream);
  if (pieces <= 1024) return launch<1, 1024, 8>(p, stream);
  if (pieces <= 2048) return launch<2, 1024, 4>(p, stream);
  if (pieces <= 4096) return launch<4, 1024, 2>(p, stream);
  return launch<8, 1024, 1>(p, stream);
}

}  // namespace ttl
