// Device helpers shared by the GEMM kernels of libttl (gfx950): vector types, bf16 packing, the
// SiLU·up epilogue, raw buffer descriptors and the direct global -> LDS copy with its explicit waits.
#pragma once

#include "kernels.h"

namespace ttl {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

constexpr uint32_t kOob = 0x80000000u;     // buffer offset beyond every record count used
constexpr int32_t kMaxRecords = 0x7FFFFFF0;

enum { kPlain = 0, kSiluMul = 1 };

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));  // round to nearest even
}

__device__ inline float silu_mul(float g, float u) {
  // silu(g) * u with silu(g) = g / (1 + exp(-g)); exp overflow gives rcp(inf) = 0, i.e. silu -> -0.
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Raw buffer descriptor (gfx9): 48-bit base, stride 0, record count in bytes, dword3 = 0x00020000
// (32-bit data format, the raw untyped setting).  Accesses at offsets >= the record count read 0.
__device__ inline i32x4_t buffer_desc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int32_t rec = bytes <= 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : (int32_t)bytes);
  i32x4_t d;
  d.x = (int32_t)(uint32_t)a;
  d.y = (int32_t)((uint32_t)(a >> 32) & 0xFFFFu);
  d.z = rec;
  d.w = 0x00020000;
  return d;
}

// One 16-byte-per-lane copy from global memory straight into LDS (buffer_load_dwordx4 ... lds):
// lane i's 16 bytes land at lds_base + 16*i.  Written as asm so that the compiler's wait insertion,
// which cannot follow the ring's stage ownership across the loop, does not drain the ring; every
// wait for these copies is explicit (wait_vmcnt).  M0 holds the LDS base; one wait state must
// separate its write from the copy.
__device__ inline void copy16_to_lds(i32x4_t desc, uint32_t voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(desc), "s"(lds_base) : "memory");
}

// The same copy with the LDS destination lds_base + lds_imm (a compile-time constant) summed
// straight into M0 (one scalar instruction fewer per copy; the add writes SCC).  The descriptor and
// base are wave-uniform; reading them through readfirstlane states so to the compiler, which
// otherwise may keep a uniform value in a vector register where the instruction needs a scalar one.
__device__ inline void copy16_to_lds_at(i32x4_t desc, uint32_t voffset, uint32_t lds_base, uint32_t lds_imm) {
  desc.x = __builtin_amdgcn_readfirstlane(desc.x);
  desc.y = __builtin_amdgcn_readfirstlane(desc.y);
  desc.z = __builtin_amdgcn_readfirstlane(desc.z);
  desc.w = __builtin_amdgcn_readfirstlane(desc.w);
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(desc), "s"(lds_base), "n"(lds_imm) : "memory", "scc");
}

// The same copy with a uniform byte offset (an SGPR) added to the global address: copies whose
// per-lane offsets differ only by a per-copy constant share one offset register.
__device__ inline void copy16_to_lds_so(i32x4_t desc, uint32_t voffset, uint32_t soffset, uint32_t lds_base,
                                        uint32_t lds_imm) {
  asm volatile("s_add_u32 m0, %3, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voffset), "s"(desc), "s"(soffset), "s"(lds_base), "n"(lds_imm) : "memory", "scc");
}

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroup barrier for the ring.  __syncthreads() carries a release fence, which would make the
// compiler drain every outstanding copy (vmcnt(0)) before it; the waits this kernel needs are
// explicit (wait_vmcnt for this wave's copies, lgkmcnt(0) for its LDS reads), and the memory clobber
// keeps the compiler from moving LDS accesses across the barrier.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Byte offset of element (krow, wcol) of a k-tile of 64 rows in a blocked weight (64 x 128 blocks,
// 128-column strips `strip` elements apart), from the k-tile's first block of strip 0.
__device__ inline uint32_t blocked_offset(int krow, int64_t wcol, int64_t strip) {
  return (uint32_t)(((wcol >> 7) * strip + krow * 128 + (wcol & 127)) * 2);
}

// Buffer descriptor of k-tile k0 / 64 of a blocked weight: from its block in strip 0 to the end of
// the strips the call reads.
__device__ inline i32x4_t blocked_desc(const uint16_t* B, int64_t b_elems, int k0) {
  const int64_t e0 = (int64_t)(k0 / 64) * 8192;
  return buffer_desc(B + e0, (b_elems - e0) * 2);
}

// Tile order of the 256 x 256-tile kernels.  Consecutive workgroups are dealt to different XCDs
// (8 on MI355X), each with its own L2: the block index is remapped so that each XCD runs a compact
// run of tiles, and tiles are walked in groups of `group` row-tiles (all columns of a group before
// the next), so that one XCD's tiles share A rows and weight columns in its L2.  Both maps are
// bijections on [0, tiles_m * tiles_n) for any group >= 1.  Also compiled for the host, where the
// launch planner scores candidate group heights with it.
__host__ __device__ inline void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn, int group = 4) {
  constexpr int kXcds = 8;
  const int tiles = tiles_m * tiles_n;
  const int q = tiles / kXcds, r = tiles % kXcds;
  const int x = bid % kXcds, local = bid / kXcds;
  const int L = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
  const int per_group = group * tiles_n;
  const int g = L / per_group;
  const int first = g * group;
  const int gsize = tiles_m - first < group ? tiles_m - first : group;
  const int inner = L - g * per_group;
  tm = first + inner % gsize;
  tn = inner / gsize;
}

// Weight column of tile column c (the first of 8 consecutive ones) of the tile whose first output
// column is n0, and whether it is in range, for waves owning WN tile columns each as WN/32 blocks of
// 32.  SiLU·up: tile column c = w*WN + nb*32 + j; a wave's blocks nb < WN/64 hold gate columns and
// the others the up columns of the same act columns, so gate and up of one output meet in one lane.
// Plain: output column n0 + c through the (up to three) segments of the column map.
template <int MODE, int WN>
__device__ inline int64_t weight_column(const GemmParams& p, int n0, int c, bool& ok) {
  constexpr int NI = WN / 32;
  if (MODE == kSiluMul) {
    const int w = c / WN, nb = (c % WN) / 32, j = c % 32;
    const int act = n0 + w * (WN / 2) + (nb % (NI / 2)) * 32 + j;
    ok = act < p.N;
    return (nb < NI / 2 ? p.gate_w0 : p.up_w0) + act;
  }
  const int oc = n0 + c;
  ok = oc < p.N;
  int64_t w0 = p.seg_w0[0];
  int s0 = p.seg_out0[0];
  if (p.nseg > 1 && oc >= p.seg_out0[1]) { w0 = p.seg_w0[1]; s0 = p.seg_out0[1]; }
  if (p.nseg > 2 && oc >= p.seg_out0[2]) { w0 = p.seg_w0[2]; s0 = p.seg_out0[2]; }
  return w0 + (oc - s0);
}

}  // namespace gemm
}  // namespace ttl
