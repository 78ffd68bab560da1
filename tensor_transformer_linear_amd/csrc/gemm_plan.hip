// Kernel choice for one GEMM launch, split-K sizing, and the library's split-K workspace.
//
// 256 x 256 tiles keep the matrix cores busiest per byte staged, but a launch needs about one tile
// per CU to fill the chip; decode batches (a few dozen rows) and small shards give far fewer.
// Those go to the split-K kernel, whose 32..128-row x 128-column tiles are additionally cut along
// k into as many ranges as keep the grid within one workgroup per CU: a CU streams at its full
// rate with one workgroup, and a grid that does not divide evenly over the CUs leaves a slow tail.
// A launch of whole rounds of 256 x 256 tiles plus a short last round (e.g. 288 tiles: 2176 rows
// x 8192 columns) runs the whole rounds' tiles with the rows below them appended (at most 16 per
// row-tile, plain columns), or else is cut by rows: the whole rounds to the tiled kernel, the last
// few row-tiles to the split-K kernel.  One whose last round is more than half full (e.g. 448
// tiles: 4096 rows x 3584 SiLU·up columns) is cut per column strip into 256-row tiles that fill
// the whole rounds and 192-row tiles that fill one more round, which then takes three quarters of
// a round's time.  Launches with few 256 x 256 tiles take 256 x 128 tiles, whole or cut along k
// (at least 512 rows; or one row-tile of 129..256 rows with a long k).  Every tiled launch runs
// on the 16 x 16 x 32 kernel, for every weight storage.
//
// Workspace: split-K launches with more than one split write fp32 partial tiles that a second
// kernel reduces.  The library keeps one device buffer per (GPU, stream) for them, allocated (or
// grown) on first need by the calling thread, so launches on different streams never share one.
// Allocation cannot happen inside a stream capture: a graph that captures such launches must be
// recorded after one eager call of the same (or a larger) shape on the capturing stream.
//
// Overrides for tests and measurements (ttl_set_gemm_override): a forced kernel family, a forced
// split count, the CU count the 256-row / 192-row cut is planned for, and a trace of each cut,
// appended-rows or persistent launch.
// They are process-wide atomics read once per launch; nothing here reads the environment.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "gemm_common.h"

namespace ttl {
namespace {

constexpr int kDefaultCUs = 256;        // MI355X compute units (a whole-chip device)
constexpr int kMinKTilesPerSplit = 4;   // keep each split's copy pipeline full
constexpr int kTileSplitMinRows = 512;  // 256 x 256 tiles cut along k from this many rows
constexpr int kMinKTilesPerTileSplit = 16;
constexpr int kNarrowSplitMinKTiles = 8;  // one row-tile of 129..256 rows: k-tiles per split, at least
constexpr int kShortK = 2048;           // split-K kernel: k up to this takes its smallest row tiles

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;  // (device, stream) -> buffer

// Device buffer of at least `bytes` for this GPU and `stream`.  A buffer that is outgrown is
// retired, not freed: work already enqueued, or captured into a graph, keeps using it safely.
// Growth at least doubles the size, so few buffers are ever retired; all of them live until the
// process ends.  A stream that is being captured cannot allocate: such a launch fails instead.
hipError_t get_workspace(size_t bytes, hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[{dev, reinterpret_cast<uintptr_t>(stream)}];
  if (w.bytes < bytes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(stream, &cs)) != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    const size_t mib = (size_t)1 << 20;
    size_t nb = (bytes + mib - 1) / mib * mib;
    if (nb < 2 * w.bytes) nb = 2 * w.bytes;
    void* ptr = nullptr;
    if ((e = hipMalloc(&ptr, nb)) != hipSuccess) return e;
    w.ptr = ptr;  // the previous buffer, if any, stays allocated
    w.bytes = nb;
  }
  *out = w.ptr;
  return hipSuccess;
}

// One call's launch context: its stream, where split-K partials go, and whether anything launches.
// A dry pass (dry = true) walks the same plan, launches nothing and allocates nothing, and records
// in `need` the largest workspace any of the call's launches would use; a call with a fixed
// workspace (the caller's or the library's static scratch) uses that buffer for every split-K
// launch instead of the per-stream buffers.
struct Ctx {
  hipStream_t stream = nullptr;
  void* fixed_ws = nullptr;
  size_t fixed_bytes = 0;
  bool dry = false;
  size_t need = 0;
};

hipError_t workspace(Ctx& c, size_t bytes, void** out) {
  c.need = bytes > c.need ? bytes : c.need;
  *out = nullptr;
  if (c.dry) return hipSuccess;
  if (c.fixed_ws != nullptr) {
    if (bytes > c.fixed_bytes) return hipErrorInvalidValue;  // callers check the dry pass first
    *out = c.fixed_ws;
    return hipSuccess;
  }
  return get_workspace(bytes, c.stream, out);
}

hipError_t run_bigwave(Ctx& c, const GemmParams& p) { return c.dry ? hipSuccess : launch_gemm_bigwave(p, c.stream); }
hipError_t run_tiled(Ctx& c, const GemmParams& p) { return c.dry ? hipSuccess : launch_gemm_tiled(p, c.stream); }
hipError_t run_tiled16(Ctx& c, const GemmParams& p) { return c.dry ? hipSuccess : launch_gemm_bigwave16(p, c.stream); }
// A tile set (256-row or 192-row tiles): the 16 x 16 x 32 kernel where it applies, else the 32 x 32 x 16 one.
hipError_t run_tileset(Ctx& c, const GemmParams& p) {
  return gemm_bigwave16_supports(p) ? run_tiled16(c, p) : run_bigwave(c, p);
}
hipError_t run_skinny(Ctx& c, const GemmParams& p, int mb) {
  return c.dry ? hipSuccess : launch_gemm_skinny(p, mb, c.stream);
}
hipError_t run_stream_nk(Ctx& c, const GemmParams& p) { return c.dry ? hipSuccess : launch_gemm_stream_nk(p, c.stream); }
hipError_t run_finalize(Ctx& c, const GemmParams& p) { return c.dry ? hipSuccess : launch_splitk_finalize(p, c.stream); }

// Test and measurement overrides (see ttl_set_gemm_override).
std::atomic<int> g_force_kernel{0}, g_force_splits{0}, g_force_plan_cus{0}, g_trace{0};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (256 on a whole MI355X; fewer on a compute partition), read
// once per device: every launch shape below is sized against it.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int64_t device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = kDefaultCUs;
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The forced kernel family: 0 by shape, 1 256 x 256 tiles, 2 split-K, 3 256 x 256 tiles by the
// eight-wave kernel, 4 256 x 256 tiles cut along k, 5 256 x 128 tiles, 6 256 x 128 tiles cut along
// k, 7 192 x 256 tiles, 8 the 256-row / 192-row cut planned for the override's CU count, 9 256 x 256
// tiles by a persistent grid (at most two tiles per workgroup), 10 256 x 256 tiles by the 16 x 16 x 32
// kernel, 11 the same over the whole row-tiles with the rows below them appended (where those are at
// most 16 per row-tile; otherwise the choice by shape), 12 the split-free kernel for [n][k] weights
// and at most 64 rows (otherwise the choice by shape).
int forced_kernel() { return g_force_kernel.load(std::memory_order_relaxed); }
int64_t forced_splits() { return g_force_splits.load(std::memory_order_relaxed); }

// 256 x 256 tiles over all of p: the four-wave kernel where it applies, unless force == 3.
hipError_t launch_tiles(GemmParams& p, int force, Ctx& c) {
  p.tiles_m = (int32_t)cdiv(p.M, gemm_tile_rows());
  p.tiles_n = (int32_t)cdiv(p.N, gemm_tile_cols(p.mode));
  p.splits = 1;
  p.narrow = 0;
  if (force != 3 && gemm_bigwave_supports(p)) return run_bigwave(c, p);
  return run_tiled(c, p);
}

// 256 x 256 tiles of the four-wave kernel over all of p by a persistent grid (K a multiple of 64, at
// least two k-tiles): with more tiles than CUs and at most twice as many, one workgroup per CU,
// each computing tile b and then tile b + CUs, whose first k-tiles it fetches while it finishes the
// first.  Otherwise as launch_tiles.  The override's CU count, if set, stands in for the device's.
hipError_t launch_persist(GemmParams& p, Ctx& c) {
  p.tiles_m = (int32_t)cdiv(p.M, gemm_tile_rows());
  p.tiles_n = (int32_t)cdiv(p.N, gemm_tile_cols(p.mode));
  const int64_t pc = g_force_plan_cus.load(std::memory_order_relaxed);
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n, cus = pc > 0 ? pc : device_cus();
  if (!gemm_bigwave_supports(p) || p.K < 128 || tiles <= cus || tiles > 2 * cus) return launch_tiles(p, 0, c);
  p.splits = 1;
  p.narrow = 0;
  p.rects = 0;
  p.persist = (int32_t)cus;
  if (!c.dry && g_trace.load(std::memory_order_relaxed))
    std::fprintf(stderr, "ttl gemm persist: M=%d N=%d K=%d, %lld tiles on %lld workgroups\n", p.M, p.N, p.K,
                 (long long)tiles, (long long)cus);
  return run_bigwave(c, p);
}

// 256 x 256 tiles over all of p by the 16 x 16 x 32 four-wave kernel where it applies (K a multiple
// of 64), else as launch_tiles.
hipError_t launch_tiles16(GemmParams& p, Ctx& c) {
  p.tiles_m = (int32_t)cdiv(p.M, gemm_tile_rows());
  p.tiles_n = (int32_t)cdiv(p.N, gemm_tile_cols(p.mode));
  p.splits = 1;
  p.narrow = 0;
  p.rects = 0;
  p.persist = 0;
  if (gemm_bigwave16_supports(p)) return run_tiled16(c, p);
  return launch_tiles(p, 0, c);
}

// 256 x 256 tiles of the 16 x 16 x 32 kernel over rows [0, 256 head) of p, each row-tile with 16
// appended rows from row 256 head on (the rows below the whole tiles, at most 16 per row-tile):
// one launch instead of whole tiles plus a launch for the rest.  False if the kernel does not take
// p that way (then nothing is launched).
bool launch_tiles16_xr(GemmParams& p, int64_t head, int64_t tn, Ctx& c, hipError_t& e) {
  GemmParams q = p;
  q.tiles_m = (int32_t)head;
  q.tiles_n = (int32_t)tn;
  q.splits = 1;
  q.narrow = 0;
  q.rects = 0;
  q.persist = 0;
  q.tile_rows = 256;
  q.xr_row0 = (int32_t)(head * 256);
  if (q.mode != 0 || p.M - q.xr_row0 > 16 * head || !gemm_bigwave16_supports(q)) return false;
  if (!c.dry && g_trace.load(std::memory_order_relaxed))
    std::fprintf(stderr, "ttl gemm appended rows: M=%d N=%d K=%d, %lld row-tiles of 256 + 16 rows from row %d\n",
                 p.M, p.N, p.K, (long long)head, q.xr_row0);
  e = run_tiled16(c, q);
  return true;
}

// 256 x 128 tiles of the four-wave kernels over all of p (K a multiple of 64): the 16 x 16 x 32
// kernel's narrow instance where it applies.
hipError_t launch_narrow(GemmParams& p, Ctx& c) {
  p.tiles_m = (int32_t)cdiv(p.M, gemm_tile_rows());
  p.tiles_n = (int32_t)cdiv(p.N, gemm_bigwave_tile_cols(p.mode, true));
  p.splits = 1;
  p.narrow = 1;
  return gemm_bigwave16_supports(p) ? run_tiled16(c, p) : run_bigwave(c, p);
}

// Row cut of one launch into 256-row and 192-row tiles (four-wave kernel, 256 weight columns per
// tile): column strips [0, S) take a[0] 256-row tiles from row 0 and b[0] 192-row tiles for the
// rows below them, strips [S, tiles_n) take a[1] and b[1].
struct MixedRows {
  int64_t S, a[2], b[2];
};

// A launch of `full` whole rounds of 256-row tiles plus a last round more than half full: find a
// cut whose 256-row tiles fit in `full` rounds and whose 192-row tiles fit in one.  A 192-row tile
// holds three quarters of a 256-row tile's work, so the launch takes full + 3/4 rounds instead of
// full + 1; a cut exists only where the last round holds at most about three quarters of a round
// of 256-row tiles (e.g. 448 tiles on 256 CUs), and none is returned otherwise.  Among the cuts that fit, the one with the most 256-row tiles (the more efficient
// ones).  Strip classes: for a[0] > a[1], the 256-row count full(S) = S*(a0-a1) + tn*a1 grows with
// S and the 192-row count short(S) = S*(b0-b1) + tn*b1 shrinks, so each pair (a0, a1) admits an
// interval of S, whose largest member is taken.
bool plan_mixed_rows(int64_t M, int64_t tn, int64_t cus, MixedRows& out) {
  if (cus < 1) return false;
  const int64_t tm = cdiv(M, 256);
  const int64_t full = (tm * tn) / cus;
  if (full < 1 || tm > 256 || 2 * ((tm * tn) % cus) <= cus) return false;
  const int64_t cap_full = full * cus;
  int64_t best_full = -1;
  auto shorts = [&](int64_t a) { return M > 256 * a ? cdiv(M - 256 * a, 192) : 0; };
  for (int64_t a0 = 1; a0 <= tm; ++a0)
    for (int64_t a1 = 0; a1 <= a0; ++a1) {
      const int64_t b0 = shorts(a0), b1 = shorts(a1);
      int64_t lo = 1, hi = tn;  // S in [lo, hi]; S = tn leaves class 1 empty
      if (a0 == a1) {
        if (tn * a0 > cap_full || tn * b0 > cus) continue;
      } else {
        // S*(a0-a1) + tn*a1 <= cap_full
        if (tn * a1 > cap_full) continue;
        hi = std::min(tn - 1, (cap_full - tn * a1) / (a0 - a1));
        // S*(b1-b0) >= tn*b1 - cus (b1 >= b0)
        const int64_t need = tn * b1 - cus;
        if (need > 0) {
          if (b1 == b0) continue;
          lo = std::max(lo, cdiv(need, b1 - b0));
        }
      }
      if (lo > hi) continue;
      const int64_t S = a0 == a1 ? tn : hi;
      const int64_t nf = S * a0 + (tn - S) * a1, ns = S * b0 + (tn - S) * b1;
      if (ns == 0 || ns > cus || nf > cap_full) continue;
      if (nf > best_full) {
        best_full = nf;
        out.S = S;
        out.a[0] = a0;
        out.a[1] = a1;
        out.b[0] = b0;
        out.b[1] = S < tn ? b1 : 0;
        if (S == tn) out.a[1] = 0;
      }
    }
  return best_full >= 0;
}

// Bytes that the 8 XCDs' L2s fetch per k-tile for a tile-set launch of at most one round (its
// tiles run concurrently, one per CU, in step along k), if each XCD fetches every A row-block and
// weight strip its tiles use once per k-tile.  With 4-MB L2s this matches the FETCH_SIZE counter
// of these launches.  a_seen / b_seen: scratch of 8 * ceil(M / 64) and 8 * tn entries.
int64_t tile_set_fetch(const GemmParams& q, int64_t M, int64_t tn, std::vector<int>& a_seen,
                       std::vector<int>& b_seen) {
  constexpr int kXcds = 8;
  const int64_t rblocks = cdiv(M, 64);
  std::fill(a_seen.begin(), a_seen.end(), 0);
  std::fill(b_seen.begin(), b_seen.end(), 0);
  int64_t a_count = 0, b_count = 0;
  int bid = 0;
  for (int r = 0; r < q.rects; ++r)
    for (int b = 0; b < q.rect_tmc[r] * q.rect_tnc[r]; ++b, ++bid) {
      int tm = 0, tc = 0;
      gemm::tile_coords(b, q.rect_tmc[r], q.rect_tnc[r], tm, tc, q.rect_group[r]);
      const int x = bid % kXcds;
      const int64_t rb = (q.rect_row0[r] + (int64_t)tm * q.tile_rows) / 64;
      const int64_t st = q.rect_tn0[r] + tc;
      if (rb < rblocks && !a_seen[(size_t)(x * rblocks + rb)]++) ++a_count;
      if (st < tn && !b_seen[(size_t)(x * tn + st)]++) ++b_count;
    }
  return a_count * q.tile_rows * 128 + b_count * 256 * 128;
}

// Group heights (1..32 row-tiles) for the rectangles of a tile-set launch that minimise
// tile_set_fetch.  Launches of more than one round keep groups of 4: their rounds do not run
// concurrently, which the count assumes.
void choose_groups(GemmParams& q, int64_t M, int64_t tn, int64_t cus) {
  q.rect_group[0] = q.rect_group[1] = 4;
  int64_t tiles = 0;
  for (int r = 0; r < q.rects; ++r) tiles += (int64_t)q.rect_tmc[r] * q.rect_tnc[r];
  if (tiles > cus) return;
  std::vector<int> a_seen((size_t)(cdiv(M, 64) * 8)), b_seen((size_t)(tn * 8));
  int best[2] = {4, 4};
  int64_t best_bytes = -1;
  const int g0max = std::min(q.rect_tmc[0], 32);
  const int g1max = q.rects > 1 ? std::min(q.rect_tmc[1], 32) : 1;
  for (int g0 = 1; g0 <= g0max; ++g0)
    for (int g1 = 1; g1 <= g1max; ++g1) {
      q.rect_group[0] = g0;
      q.rect_group[1] = g1;
      const int64_t bytes = tile_set_fetch(q, M, tn, a_seen, b_seen);
      if (best_bytes < 0 || bytes < best_bytes) {
        best_bytes = bytes;
        best[0] = g0;
        best[1] = g1;
      }
    }
  q.rect_group[0] = best[0];
  q.rect_group[1] = best[1];
}

// The cut's two launches of the four-wave kernel: the 256-row tiles of both strip classes, then
// the 192-row tiles below them, each with the group heights that keep its L2 fetches lowest.
// Plans are cached per (M, N, K, mode, CU count), most recently used first, up to kPlanCache of
// them: the group search costs up to a few milliseconds.
struct MixedLaunch {
  int64_t M, N, K, cus;
  int32_t mode;
  GemmParams q[2];  // tiling fields only
};
constexpr size_t kPlanCache = 64;
std::mutex g_plan_mutex;
std::vector<MixedLaunch> g_plans;

void build_mixed(const GemmParams& p, const MixedRows& m, int64_t tn, int64_t cus, GemmParams q[2]) {
  for (int pass = 0; pass < 2; ++pass) {
    GemmParams& t = q[pass];
    t = p;
    t.splits = 1;
    t.narrow = 0;
    t.tiles_m = t.tiles_n = 0;
    t.tile_rows = pass == 0 ? 256 : 192;
    t.rects = 0;
    for (int c = 0; c < 2; ++c) {
      const int64_t width = c == 0 ? m.S : tn - m.S;
      const int64_t count = pass == 0 ? m.a[c] : m.b[c];
      if (width <= 0 || count <= 0) continue;
      const int r = t.rects++;
      t.rect_tn0[r] = (int32_t)(c == 0 ? 0 : m.S);
      t.rect_tnc[r] = (int32_t)width;
      t.rect_row0[r] = (int32_t)(pass == 0 ? 0 : 256 * m.a[c]);
      t.rect_tmc[r] = (int32_t)count;
      t.rect_group[r] = 4;
    }
    if (t.rects > 0) choose_groups(t, p.M, tn, cus);
  }
}

hipError_t launch_mixed(GemmParams& p, const MixedRows& m, int64_t cus, Ctx& c) {
  const int64_t tn = cdiv(p.N, gemm_tile_cols(p.mode));
  GemmParams q[2];
  bool cached = false;
  {
    std::lock_guard<std::mutex> lock(g_plan_mutex);
    for (size_t i = 0; i < g_plans.size(); ++i) {
      const MixedLaunch& c = g_plans[i];
      if (c.M == p.M && c.N == p.N && c.K == p.K && c.mode == p.mode && c.cus == cus) {
        q[0] = c.q[0];
        q[1] = c.q[1];
        cached = true;
        std::rotate(g_plans.begin(), g_plans.begin() + i, g_plans.begin() + i + 1);  // most recent first
        break;
      }
    }
  }
  if (!cached) {
    build_mixed(p, m, tn, cus, q);
    std::lock_guard<std::mutex> lock(g_plan_mutex);
    // Least recently used plans make room once the cache is full.
    if (g_plans.size() >= kPlanCache) g_plans.pop_back();
    g_plans.insert(g_plans.begin(), {p.M, p.N, p.K, cus, p.mode, {q[0], q[1]}});
  }
  if (!c.dry && g_trace.load(std::memory_order_relaxed))
    std::fprintf(stderr, "ttl gemm cut: M=%d N=%d K=%d strips [0,%lld) %lld x 256 + %lld x 192, "
                 "[%lld,%lld) %lld x 256 + %lld x 192, groups %d/%d and %d/%d\n", p.M, p.N, p.K,
                 (long long)m.S, (long long)m.a[0], (long long)m.b[0], (long long)m.S, (long long)tn,
                 (long long)m.a[1], (long long)m.b[1], q[0].rect_group[0], q[0].rect_group[1],
                 q[1].rect_group[0], q[1].rect_group[1]);
  for (int pass = 0; pass < 2; ++pass) {
    if (q[pass].rects == 0) continue;
    // The cached tiling fields with this call's pointers and strides.
    GemmParams t = p;
    t.splits = 1;
    t.narrow = 0;
    t.tiles_m = t.tiles_n = 0;
    t.tile_rows = q[pass].tile_rows;
    t.rects = q[pass].rects;
    for (int r = 0; r < 2; ++r) {
      t.rect_tn0[r] = q[pass].rect_tn0[r];
      t.rect_tnc[r] = q[pass].rect_tnc[r];
      t.rect_row0[r] = q[pass].rect_row0[r];
      t.rect_tmc[r] = q[pass].rect_tmc[r];
      t.rect_group[r] = q[pass].rect_group[r];
    }
    const hipError_t e = run_tileset(c, t);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// 192 x 256 tiles of the four-wave kernels over all of p, as one tile set.
hipError_t launch_short(GemmParams& p, Ctx& c) {
  GemmParams q = p;
  q.splits = 1;
  q.narrow = 0;
  q.tiles_m = q.tiles_n = 0;
  q.tile_rows = 192;
  q.rects = 1;
  q.rect_tn0[0] = 0;
  q.rect_tnc[0] = (int32_t)cdiv(p.N, gemm_tile_cols(p.mode));
  q.rect_row0[0] = 0;
  q.rect_tmc[0] = (int32_t)cdiv(p.M, 192);
  return run_tileset(c, q);
}

// 256 x 256 (or, narrow, 256 x 128) tiles of the four-wave kernel cut into `splits` k ranges
// (plain mode; SiLU·up as the gate columns then the up columns), then the split-K finalize kernel.
hipError_t launch_tiles_splitk(GemmParams& p, int64_t splits, bool narrow, Ctx& c) {
  GemmParams q = p.mode == 1 ? silu_as_plain_halves(p) : p;
  q.narrow = narrow ? 1 : 0;
  q.tiles_m = (int32_t)cdiv(q.M, gemm_tile_rows());
  q.tiles_n = (int32_t)cdiv(q.N, gemm_bigwave_tile_cols(0, narrow));
  const int64_t nk = q.K / 64;
  if (splits > nk) splits = nk;
  const int64_t kt_per = cdiv(nk, splits);
  splits = cdiv(nk, kt_per);  // every split gets at least one k-tile
  if (splits < 2) return narrow ? launch_narrow(p, c) : launch_tiles(p, 0, c);
  q.splits = (int32_t)splits;
  q.kt_per_split = (int32_t)kt_per;
  q.ws_ld = (int64_t)q.tiles_n * gemm_bigwave_tile_cols(0, narrow);
  void* base = nullptr;
  hipError_t e = workspace(c, (size_t)splits * q.M * q.ws_ld * sizeof(float), &base);
  if (e != hipSuccess) return e;
  q.ws = static_cast<float*>(base);
  // 256 x 256 or 256 x 128 tiles on the 16 x 16 x 32 kernel (else the 32 x 32 x 16 one).
  if ((e = gemm_bigwave16_supports(q) ? run_tiled16(c, q) : run_bigwave(c, q)) != hipSuccess) return e;
  GemmParams f = p;
  f.ws = q.ws;
  f.ws_ld = q.ws_ld;
  f.splits = q.splits;
  return run_finalize(c, f);
}

hipError_t launch_splitk(GemmParams& p, Ctx& c) {
  // Row blocks per tile: 32 * mb rows.  With a short k (at most kShortK), batches of 65..512 rows
  // take 32-row tiles (64-row above 256 rows): the grid then fills the CUs with few or no k splits,
  // whose fp32 partials would cost more than the extra passes over the weight (served from L2).
  // Measured (graph replay, splits as planned): 8B TP=8 row GEMM at 256 tokens 16.8 against 19.9 us
  // with 128-row tiles; a 128-row 70B o_proj tail (k = 1024) 10.4-11.2 against 19.1 us.  A long k
  // keeps the larger tiles, whose fewer passes over the weight win there.
  int mb = p.M <= 32 ? 1 : (p.M <= 64 ? 2 : 4);
  if (p.M > 64 && p.K <= kShortK) mb = p.M <= 256 ? 1 : 2;
  const int64_t tiles_m = cdiv(p.M, 32 * mb);
  const int64_t tiles_n = cdiv(p.N, p.mode == 1 ? kSkinnyCols / 2 : kSkinnyCols);
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t nk = cdiv(p.K, kSkinnyK);
  int64_t splits = device_cus() / tiles;  // split-K grid: at most one workgroup per CU
  const int64_t max_splits = nk / kMinKTilesPerSplit > 1 ? nk / kMinKTilesPerSplit : 1;
  if (splits > max_splits) splits = max_splits;
  const int64_t fs = forced_splits();
  if (fs > 0) splits = fs < nk ? fs : nk;
  if (splits < 1) splits = 1;
  const int64_t kt_per = cdiv(nk, splits);
  splits = cdiv(nk, kt_per);  // every split gets at least one k-tile
  p.tiles_m = (int32_t)tiles_m;
  p.tiles_n = (int32_t)tiles_n;
  p.splits = (int32_t)splits;
  p.kt_per_split = (int32_t)kt_per;
  p.ws_ld = tiles_n * kSkinnyCols;
  p.ws = nullptr;
  if (splits > 1) {
    void* base = nullptr;
    const hipError_t e = workspace(c, (size_t)splits * p.M * p.ws_ld * sizeof(float), &base);
    if (e != hipSuccess) return e;
    p.ws = static_cast<float*>(base);
  }
  return run_skinny(c, p, mb);
}

// The kernel choice for one call (see the notes at the top), launched through the call's context.
hipError_t plan_and_launch(GemmParams& p, Ctx& c) {
  const int force = forced_kernel();
  const int64_t n_cu = device_cus();
  const int64_t min_tiled = n_cu * 3 / 4;  // 256 x 256 tiles when they occupy >= 3/4 of the CUs
  if (force == 1 || force == 3) return launch_tiles(p, force, c);
  if (force == 12 && gemm_stream_nk_supports(p)) return run_stream_nk(c, p);
  if (force == 9) return launch_persist(p, c);
  if (force == 10) return launch_tiles16(p, c);
  if (force == 11 && p.M > 256 && p.M % 256 != 0) {
    hipError_t xe = hipSuccess;
    if (launch_tiles16_xr(p, p.M / 256, cdiv(p.N, gemm_tile_cols(p.mode)), c, xe)) return xe;
  }
  if (force == 7 && gemm_bigwave_supports(p)) return launch_short(p, c);
  if (force == 8 && gemm_bigwave_supports(p)) {
    MixedRows m;
    const int64_t pc = g_force_plan_cus.load(std::memory_order_relaxed);
    const int64_t cus = pc > 0 ? pc : device_cus();
    if (plan_mixed_rows(p.M, cdiv(p.N, gemm_tile_cols(p.mode)), cus, m)) return launch_mixed(p, m, cus, c);
    return launch_tiles(p, 0, c);
  }
  if (force == 5) return gemm_bigwave_supports(p) ? launch_narrow(p, c) : launch_tiles(p, 3, c);
  if (force == 2 || ((force == 4 || force == 6) && !gemm_bigwave_supports(p))) return launch_splitk(p, c);
  const int64_t tiled_m = cdiv(p.M, gemm_tile_rows());
  const int64_t tiled_n = cdiv(p.N, gemm_tile_cols(p.mode));
  const int64_t tiles = tiled_m * tiled_n;
  const int64_t narrow_tiles = tiled_m * cdiv(p.N, gemm_bigwave_tile_cols(p.mode, true));
  if (force == 4 || force == 6) {
    const int64_t fs = forced_splits();
    const int64_t auto_splits = n_cu / (force == 4 ? tiles : narrow_tiles);
    return launch_tiles_splitk(p, fs > 0 ? fs : (auto_splits > 2 ? auto_splits : 2), force == 6, c);
  }
  // Decode batches of at most 16 rows with [n][k] weights: the split-free kernel where its workgroups
  // (one per 32 weight columns) occupy at least 3/4 of the CUs; it writes no fp32 partials and needs
  // no second kernel (70B TP=8 at 1 token, ranks cycled, graph replay: SiLU·up 32.8 -> 31.0 us, row
  // GEMM 16.0 -> 14.3 us).  With more rows every workgroup's pass over all of X costs more than
  // the split-K kernel's partials (at 32 and 64 tokens: SiLU·up 28.4 -> 40.4 and 31-34 -> 54.7 us).
  if (force == 0 && p.M <= 16 && gemm_stream_nk_supports(p) && gemm_stream_nk_workgroups(p) >= min_tiled)
    return run_stream_nk(c, p);
  if (tiles < min_tiled) {
    // Few 256 x 256 tiles.  With many rows and a long k, 256 x 256 tiles cut along k into about
    // one workgroup per CU keep the matrix cores busier than the split-K kernel's 128-row tiles;
    // each split takes at least kMinKTilesPerTileSplit k-tiles, as the fp32 partial tiles cost HBM
    // traffic (k = 1024 with 2 splits measured slower than the split-K kernel).  Decode-sized
    // launches stay on the split-K kernel, which is built to stream the weight.
    // Where 256 x 128 tiles fill at least as much of the chip in one round, they run whole.
    if (p.M >= kTileSplitMinRows && gemm_bigwave_supports(p) && narrow_tiles >= min_tiled &&
        narrow_tiles <= n_cu)
      return launch_narrow(p, c);
    // Otherwise tiles cut along k: 256 x 256 tiles, or 256 x 128 tiles where those occupy at
    // least as many CUs (then with half the partial bytes per output).
    const int64_t by_k = (p.K / 64) / kMinKTilesPerTileSplit;
    const int64_t splits = n_cu / tiles < by_k ? n_cu / tiles : by_k;
    const int64_t nsplits = n_cu / narrow_tiles < by_k ? n_cu / narrow_tiles : by_k;
    if (p.M >= kTileSplitMinRows && gemm_bigwave_supports(p)) {
      if (nsplits >= 2 && narrow_tiles * nsplits >= tiles * splits)
        return launch_tiles_splitk(p, nsplits, true, c);
      if (splits >= 2) return launch_tiles_splitk(p, splits, false, c);
    }
    // One row-tile of 129..256 rows: 256 x 128 tiles cut along k into as many splits as fit one
    // round, each of at least kNarrowSplitMinKTiles k-tiles, where that makes 4 splits or more
    // (graph replay, [k][n] / [n][k] weights: 70B TP=8 SiLU·up at 256 tokens 64.2 -> 46.7 / 53.8 ->
    // 48.5 us, at 192 tokens 56.4 -> 43.4 / 50.0 -> 45.7; 70B row GEMM at 256 tokens 36.3 -> 30.2 /
    // 31.1 -> 28.4; 8B SiLU·up at 160-256 tokens 9-12 % / 4-5 %; 8B TP=4 qkv at 256 tokens 20.3 ->
    // 18.3 / 20.0 -> 18.1).  Below: a k too short for 4 such splits (8B row GEMM, k = 1792: the
    // split-K kernel's 15.1 against 20.0 us) and launches of 128 rows or fewer (half-empty tiles;
    // the split-K kernel wins at 128, 96 and 64 rows) stay on the split-K kernel.
    if (p.M > 128 && p.M <= 256 && gemm_bigwave_supports(p)) {
      const int64_t by_cu = n_cu / narrow_tiles, by_kt = (p.K / 64) / kNarrowSplitMinKTiles;
      const int64_t ns = by_cu < by_kt ? by_cu : by_kt;
      if (ns >= 4) return launch_tiles_splitk(p, ns, true, c);
    }
    return launch_splitk(p, c);
  }
  const int64_t rounds = tiles / n_cu, rem = tiles % n_cu;
  // The 16 x 16 x 32 kernel, for every weight storage, wherever the last round is full or more than
  // half full (measured faster than the persistent grid and every launch of the 32 x 32 x 16
  // kernel, 70B TP=8 at 4096 tokens: [n][k] weights, row GEMM 171-177 against 186 us, SiLU·up column
  // GEMM 341-343 against 350 us; [k][n] weights, same box, 172.9 against 188.5 us and 346.9 against
  // 377.9 us): whole tiles, or, for whole rounds plus a last round more than half full, 256-row
  // tiles for the whole rounds and 192-row tiles for the last one, which then takes about 3/4 of a
  // round's time (SiLU·up column GEMM 345.1 -> 342.1 us with [k][n] weights, 335.7 -> 329.0 us with
  // [n][k]).  Whole rounds (e.g. 512 tiles: 4096 x 8192 row-parallel outputs) run as whole tiles:
  // with the epilogue staged through LDS they beat the persistent grid of the 32 x 32 x 16 kernel,
  // whose first tile must store directly while the ring holds its next tile's first k-tiles.  A
  // short last round still goes to the split-K kernel below.
  bool use16 = false;
  {
    GemmParams q = p;
    q.splits = 1;
    q.narrow = 0;
    q.rects = 0;
    q.persist = 0;
    use16 = gemm_bigwave16_supports(q);
  }
  if (use16 && (rounds == 0 || rem == 0 || 2 * rem > n_cu)) {
    MixedRows m;
    if (rounds >= 1 && rem > 0 && plan_mixed_rows(p.M, tiled_n, n_cu, m)) return launch_mixed(p, m, n_cu, c);
    return launch_tiles16(p, c);
  }
  // Whole rounds plus a short last round (at most half the CUs): that round would take a whole
  // tile's time with most of the chip idle.  The row-tiles that fill the whole rounds go to the
  // tiled kernel, the remaining rows (a few row-tiles) to the split-K kernel, which spreads them
  // over all CUs; or, plain columns with at most 16 remaining rows per whole row-tile, the tiles
  // take those rows as appended rows in the same launch (70B TP=8 layer at 2048 + 128 tokens: each
  // tile's products grow by 1/16 in place of a split-K launch over the 128 rows).
  if (rounds >= 1 && rem > 0 && 2 * rem <= n_cu) {
    const int64_t head_row_tiles = rounds * n_cu / tiled_n;
    hipError_t xe = hipSuccess;
    if (use16 && head_row_tiles >= 1 && head_row_tiles < tiled_m &&
        launch_tiles16_xr(p, head_row_tiles, tiled_n, c, xe))
      return xe;
    if (head_row_tiles >= 1 && head_row_tiles < tiled_m) {
      GemmParams head = p;
      head.M = (int32_t)(head_row_tiles * gemm_tile_rows());
      hipError_t e = use16 ? launch_tiles16(head, c) : launch_tiles(head, 0, c);
      if (e != hipSuccess) return e;
      GemmParams tail = p;
      tail.A = p.A + (int64_t)head.M * p.lda;
      tail.C = p.C + (int64_t)head.M * p.ldc;
      tail.M = p.M - head.M;
      return launch_splitk(tail, c);
    }
  }
  return use16 ? launch_tiles16(p, c) : launch_tiles(p, 0, c);
}

}  // namespace

void set_gemm_override(int kernel, int splits, int plan_cus, bool trace) {
  g_force_kernel.store(kernel, std::memory_order_relaxed);
  g_force_splits.store(splits, std::memory_order_relaxed);
  g_force_plan_cus.store(plan_cus, std::memory_order_relaxed);
  g_trace.store(trace ? 1 : 0, std::memory_order_relaxed);
}

hipError_t launch_gemm(GemmParams& p, hipStream_t stream) {
  Ctx c;
  c.stream = stream;
  return plan_and_launch(p, c);
}

size_t gemm_workspace_bytes(const GemmParams& p) {
  GemmParams q = p;
  Ctx c;
  c.dry = true;
  (void)plan_and_launch(q, c);  // the dry pass launches nothing and fails only on an invalid plan
  return c.need;
}

hipError_t launch_gemm_fixed_workspace(GemmParams& p, void* ws, size_t ws_bytes, hipStream_t stream) {
  Ctx c;
  c.stream = stream;
  c.fixed_ws = ws;
  c.fixed_bytes = ws_bytes;
  return plan_and_launch(p, c);
}

}  // namespace ttl
