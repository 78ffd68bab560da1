// Weight re-layout for TTL_W_BLOCKED: W[k][n] row-major -> blocks of 64 k-rows x 128 columns, each
// block row-major, the blocks of a 128-column strip one after another down k, the strips one after
// another along n.  One thread moves 16 bytes (8 columns): output piece e holds block e / 1024,
// row (e % 1024) / 16 of the block, columns 8 * (e % 16) .. +7.
#include "kernels.h"

namespace ttl {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void pack_blocked_kernel(const uint16_t* W, int64_t k, int64_t n,
                                                           uint16_t* W_blk) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= k * n / 8) return;
  const int64_t block = e / 1024, within = e % 1024;
  const int64_t kblocks = k / 64;
  const int64_t strip = block / kblocks, kb = block % kblocks;
  const int64_t row = kb * 64 + within / 16, col = strip * 128 + (within % 16) * 8;
  *reinterpret_cast<u32x4_t*>(W_blk + e * 8) = *reinterpret_cast<const u32x4_t*>(W + row * n + col);
}

}  // namespace

hipError_t launch_pack_blocked(const uint16_t* W, int64_t k, int64_t n, uint16_t* W_blk, hipStream_t stream) {
  const int64_t pieces = k * n / 8;
  hipLaunchKernelGGL(pack_blocked_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, W, k, n,
                     W_blk);
  return hipGetLastError();
}

}  // namespace ttl
