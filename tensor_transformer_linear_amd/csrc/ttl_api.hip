// C ABI of libttl: argument validation, shard addressing and kernel launch.
//
// Every entry point validates synchronously and returns a status before anything is enqueued; on
// success it enqueues its kernel on the caller's stream and returns without waiting.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.h"
#include "ttl.h"

// Split-K partial sums of shard_linear_col_noalloc: this array, not a buffer the library allocates.
// Each GPU the library runs on holds its own copy until the process ends.  In host code the name
// stands for a host-side placeholder, not the device memory: the device address is looked up once
// per device (scratch_address below) and only that address reaches a kernel.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static_assert(kScratchBytes == (size_t)TTL_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

// Device address of `scratch` on the current device, looked up on the first call on that device.
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

ttl_status fail(ttl_status status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// A GEMM output of out_elems bf16 elements overlapping its input (x_elems) or weight (w_elems).
bool output_overlaps(const uint16_t* out, int64_t out_elems, const uint16_t* x, int64_t x_elems,
                     const uint16_t* w, int64_t w_elems) {
  return overlaps(out, out_elems * 2, x, x_elems * 2) || overlaps(out, out_elems * 2, w, w_elems * 2);
}

constexpr int64_t kMaxDim = 0x7FFFFFFF;
// Per-tile buffer offsets are 32-bit: 256 input rows and 65 weight rows of pitch must stay < 2^31 B.
constexpr int64_t kMaxLda = (int64_t)1 << 21;
constexpr int64_t kMaxLdb = (int64_t)1 << 23;
// Output elements of one GEMM (keeps every tile and workgroup count far inside 32 bits).
constexpr int64_t kMaxOutput = (int64_t)1 << 40;
// [n][k] weight rows are addressed with 32-bit byte offsets from the first row read.
constexpr int64_t kMaxNkBytes = (int64_t)0x7FFFFFF0 - 16;

ttl_status launch_status(hipError_t e, const char* who) {
  if (e != hipSuccess) return fail(TTL_ERR_HIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
  return TTL_OK;
}


// Validation and GEMM parameters shared by the column entry points; the output placement (C, ldc)
// is left to the caller.  `width` receives the rank's output width (act columns with SILU_MUL).
ttl_status col_setup(const char* who, const uint16_t* X, int64_t b, int64_t k, const uint16_t* W,
                     int64_t n, ttl_weight_layout w_layout, int32_t t, int32_t rank,
                     const ttl_col_split* split, ttl_epilogue epi, const uint16_t* Y,
                     ttl::GemmParams& p, int64_t& out_width) {
  // Sizes first: an empty tensor (a size of 0) is a shape error even where its pointer is NULL.
  if (b <= 0 || k <= 0 || n <= 0 || b > kMaxDim || k > kMaxDim || n > kMaxDim)
    return fail(TTL_ERR_SHAPE, "%s: b=%lld k=%lld n=%lld must be in [1, 2^31)", who, (long long)b,
                (long long)k, (long long)n);
  if (X == nullptr || W == nullptr || Y == nullptr)
    return fail(TTL_ERR_NULL, "%s: X, W and Y must be non-NULL", who);
  if (t < 1 || rank < 0 || rank >= t)
    return fail(TTL_ERR_RANK, "%s: need t >= 1 and 0 <= rank < t (t=%d rank=%d)", who, t, rank);
  if (epi != TTL_EPI_NONE && epi != TTL_EPI_SILU_MUL)
    return fail(TTL_ERR_UNSUPPORTED, "%s: unknown epilogue %d", who, epi);
  if (w_layout != TTL_W_KN && w_layout != TTL_W_NK && w_layout != TTL_W_BLOCKED)
    return fail(TTL_ERR_UNSUPPORTED, "%s: unknown weight layout %d", who, w_layout);

  ttl_col_split sp;
  if (split != nullptr) {
    sp = *split;
  } else {
    sp.nseg = 1;
    sp.seg_n[0] = n;
    sp.seg_parts[0] = t;
  }
  if (sp.nseg < 1 || sp.nseg > TTL_MAX_SEGMENTS)
    return fail(TTL_ERR_UNSUPPORTED, "%s: nseg=%d must be 1..%d", who, sp.nseg, TTL_MAX_SEGMENTS);

  p = {};
  int64_t sum = 0, n_r = 0, wcol0[TTL_MAX_SEGMENTS], width[TTL_MAX_SEGMENTS];
  for (int s = 0; s < sp.nseg; ++s) {
    const int64_t ns = sp.seg_n[s];
    const int32_t parts = sp.seg_parts[s];
    if (ns <= 0) return fail(TTL_ERR_SHAPE, "%s: segment %d has width %lld", who, s, (long long)ns);
    if (parts < 1 || parts > t || t % parts != 0)
      return fail(TTL_ERR_NOT_DIVISIBLE, "%s: segment %d is cut into %d parts; need a divisor of t=%d",
                  who, s, parts, t);
    if (ns % parts != 0)
      return fail(TTL_ERR_NOT_DIVISIBLE, "%s: segment %d width %lld is not divisible by %d", who, s,
                  (long long)ns, parts);
    width[s] = ns / parts;
    const int64_t q = (int64_t)rank * parts / t;  // which slice of the segment this rank owns
    wcol0[s] = sum + q * width[s];
    sum += ns;
    n_r += width[s];
  }
  if (sum != n)
    return fail(TTL_ERR_NOT_DIVISIBLE, "%s: segment widths sum to %lld but W has n=%lld columns", who,
                (long long)sum, (long long)n);
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y))
    return fail(TTL_ERR_ALIGN, "%s: X, W and Y must be 16-byte aligned", who);
  if (k % 8 != 0 || n % 8 != 0)
    return fail(TTL_ERR_ALIGN, "%s: k=%lld and n=%lld must be multiples of 8", who, (long long)k,
                (long long)n);
  for (int s = 0; s < sp.nseg; ++s)
    if (width[s] % 8 != 0)
      return fail(TTL_ERR_ALIGN, "%s: slice width %lld of segment %d is not a multiple of 8", who,
                  (long long)width[s], s);
  if (k > kMaxLda || n > kMaxLdb)
    return fail(TTL_ERR_SHAPE, "%s: k=%lld or n=%lld exceeds the supported row pitch", who,
                (long long)k, (long long)n);
  // A [n][k] weight is addressed from the first row the rank reads, with 32-bit byte offsets: the
  // rows between the rank's first and last weight column must span less than 2 GiB (the whole
  // weight may be larger, e.g. a vocabulary-sized LM head).
  int64_t row_lo = 0, row_hi = n;
  if (w_layout == TTL_W_NK) {
    row_lo = wcol0[0];
    row_hi = wcol0[0] + width[0];
    for (int s = 1; s < sp.nseg; ++s) {
      row_lo = wcol0[s] < row_lo ? wcol0[s] : row_lo;
      row_hi = wcol0[s] + width[s] > row_hi ? wcol0[s] + width[s] : row_hi;
    }
    if ((row_hi - row_lo) * k * 2 >= kMaxNkBytes)
      return fail(TTL_ERR_UNSUPPORTED,
                  "%s: the [n][k] rows this rank reads must span less than 2 GiB", who);
    for (int s = 0; s < sp.nseg; ++s) wcol0[s] -= row_lo;
  }
  // A blocked weight is addressed from the first 128-column strip the rank reads; the strips up to
  // its last column must span less than 2 GiB.
  int64_t strip_lo = 0, strip_hi = 0;
  if (w_layout == TTL_W_BLOCKED) {
    if (k % 64 != 0 || n % 128 != 0)
      return fail(TTL_ERR_ALIGN, "%s: a blocked weight needs k %% 64 == 0 and n %% 128 == 0 (k=%lld n=%lld)",
                  who, (long long)k, (long long)n);
    int64_t lo = wcol0[0], hi = wcol0[0] + width[0];
    for (int s = 1; s < sp.nseg; ++s) {
      lo = wcol0[s] < lo ? wcol0[s] : lo;
      hi = wcol0[s] + width[s] > hi ? wcol0[s] + width[s] : hi;
    }
    strip_lo = lo / 128;
    strip_hi = (hi + 127) / 128;
    if ((strip_hi - strip_lo) * k * 128 * 2 >= kMaxNkBytes)
      return fail(TTL_ERR_UNSUPPORTED, "%s: the blocked strips this rank reads must span less than 2 GiB",
                  who);
    for (int s = 0; s < sp.nseg; ++s) wcol0[s] -= strip_lo * 128;
  }

  p.A = X;
  p.lda = k;
  p.w_nk = w_layout == TTL_W_NK;
  p.B = p.w_nk ? W + row_lo * k : W;
  p.ldb = p.w_nk ? k : n;
  p.b_rows = row_hi - row_lo;
  if (w_layout == TTL_W_BLOCKED) {
    p.w_blk = 1;
    p.B = W + strip_lo * k * 128;
    p.ldb = k * 128;
    p.b_rows = (strip_hi - strip_lo) * k * 128;
  }
  p.M = (int32_t)b;
  p.K = (int32_t)k;
  if (epi == TTL_EPI_SILU_MUL) {
    if (sp.nseg != 2 || sp.seg_n[0] != sp.seg_n[1] || sp.seg_parts[0] != sp.seg_parts[1])
      return fail(TTL_ERR_UNSUPPORTED,
                  "%s: SiLU*up needs two equal segments (gate | up) with equal part counts", who);
    p.mode = 1;
    p.N = (int32_t)width[0];
    p.gate_w0 = wcol0[0];
    p.up_w0 = wcol0[1];
  } else {
    p.mode = 0;
    p.N = (int32_t)n_r;
    p.nseg = sp.nseg;
    int64_t out0 = 0;
    for (int s = 0; s < sp.nseg; ++s) {
      p.seg_out0[s] = (int32_t)out0;
      p.seg_w0[s] = wcol0[s];
      out0 += width[s];
    }
    p.seg_out0[sp.nseg] = (int32_t)out0;
  }
  if (b * (int64_t)p.N * t > kMaxOutput)
    return fail(TTL_ERR_SHAPE, "%s: output of %lld x %d elements is too large", who, (long long)b, p.N);
  out_width = p.N;
  return TTL_OK;
}


// Validation, shard addressing and launch of the column-parallel GEMM (both column entry points).
ttl_status col_entry(const char* who, const uint16_t* X, int64_t b, int64_t k, const uint16_t* W,
                     int64_t n, ttl_weight_layout w_layout, int32_t t, int32_t rank,
                     const ttl_col_split* split, ttl_epilogue epi, uint16_t* Y, void* stream) {
  ttl::GemmParams p;
  int64_t width = 0;
  const ttl_status st = col_setup(who, X, b, k, W, n, w_layout, t, rank, split, epi, Y, p, width);
  if (st != TTL_OK) return st;
  if (output_overlaps(Y, b * width, X, b * k, W, k * n))
    return fail(TTL_ERR_UNSUPPORTED, "%s: Y must not overlap X or W", who);
  p.C = Y;
  p.ldc = width;
  return launch_status(ttl::launch_gemm(p, static_cast<hipStream_t>(stream)), who);
}

// Validation, shard addressing and launch of the row-parallel GEMM (both row entry points).
ttl_status row_entry(const char* who, const uint16_t* X, int64_t b, int64_t k, int32_t x_is_parallel,
                     const uint16_t* W, int64_t n, ttl_weight_layout w_layout, int32_t t, int32_t rank,
                     uint16_t* P, void* stream) {
  if (b <= 0 || k <= 0 || n <= 0 || b > kMaxDim || k > kMaxDim || n > kMaxDim)
    return fail(TTL_ERR_SHAPE, "%s: b=%lld k=%lld n=%lld must be in [1, 2^31)", who, (long long)b,
                (long long)k, (long long)n);
  if (X == nullptr || W == nullptr || P == nullptr)
    return fail(TTL_ERR_NULL, "%s: X, W and P must be non-NULL", who);
  if (t < 1 || rank < 0 || rank >= t)
    return fail(TTL_ERR_RANK, "%s: need t >= 1 and 0 <= rank < t (t=%d rank=%d)", who, t, rank);
  if (w_layout != TTL_W_KN && w_layout != TTL_W_NK && w_layout != TTL_W_BLOCKED)
    return fail(TTL_ERR_UNSUPPORTED, "%s: unknown weight layout %d", who, w_layout);
  if (k % t != 0)
    return fail(TTL_ERR_NOT_DIVISIBLE, "%s: k=%lld is not divisible by t=%d", who, (long long)k, t);
  const int64_t kr = k / t;
  if (!aligned16(X) || !aligned16(W) || !aligned16(P))
    return fail(TTL_ERR_ALIGN, "%s: X, W and P must be 16-byte aligned", who);
  if (kr % 8 != 0 || n % 8 != 0 || k % 8 != 0)
    return fail(TTL_ERR_ALIGN, "%s: k/t=%lld and n=%lld must be multiples of 8", who,
                (long long)kr, (long long)n);
  const int64_t lda = x_is_parallel ? kr : k;
  if (lda > kMaxLda || n > kMaxLdb || k > kMaxLdb)
    return fail(TTL_ERR_SHAPE, "%s: row pitch of X or W exceeds the supported range", who);
  if (w_layout == TTL_W_NK && n * k * 2 >= kMaxNkBytes)
    return fail(TTL_ERR_UNSUPPORTED, "%s: a [n][k] weight must stay below 2 GiB", who);
  if (w_layout == TTL_W_BLOCKED) {
    if (k % 64 != 0 || kr % 64 != 0 || n % 128 != 0)
      return fail(TTL_ERR_ALIGN, "%s: a blocked weight needs k %% 64, (k/t) %% 64 and n %% 128 == 0", who);
    if (n * k * 2 >= kMaxNkBytes)
      return fail(TTL_ERR_UNSUPPORTED, "%s: a blocked weight must stay below 2 GiB", who);
  }

  ttl::GemmParams p = {};
  p.A = x_is_parallel ? X : X + (int64_t)rank * kr;
  p.lda = lda;
  p.w_nk = w_layout == TTL_W_NK;
  // W[k][n]: the rank's k rows start at row r*k/t.  W^T[n][k]: they are columns r*k/t.. of each row.
  p.B = p.w_nk ? W + (int64_t)rank * kr : W + (int64_t)rank * kr * n;
  p.ldb = p.w_nk ? k : n;
  p.b_rows = n;
  if (w_layout == TTL_W_BLOCKED) {
    // the rank's k rows start at block row r*(k/t)/64 of every strip
    const int64_t e0 = (int64_t)rank * kr / 64 * 8192;
    p.w_blk = 1;
    p.B = W + e0;
    p.ldb = k * 128;
    p.b_rows = n / 128 * k * 128 - e0;
  }
  p.C = P;
  p.ldc = n;
  p.M = (int32_t)b;
  p.N = (int32_t)n;
  p.K = (int32_t)kr;
  p.mode = 0;
  p.nseg = 1;
  p.seg_out0[0] = 0;
  p.seg_out0[1] = (int32_t)n;
  p.seg_w0[0] = 0;
  if (b * n > kMaxOutput)
    return fail(TTL_ERR_SHAPE, "%s: output of %lld x %lld elements is too large", who, (long long)b,
                (long long)n);
  if (output_overlaps(P, b * n, X, b * lda, W, k * n))
    return fail(TTL_ERR_UNSUPPORTED, "%s: P must not overlap X or W", who);
  return launch_status(ttl::launch_gemm(p, static_cast<hipStream_t>(stream)), who);
}

// Validation and parameters of the reduction over rows [row0, row0 + rows) of P[t][b][n]; the
// residual and the outputs hold exactly those rows.
ttl_status reduce_setup(const char* who, const uint16_t* P, int32_t t, int64_t b, int64_t n,
                        int64_t row0, int64_t rows, const uint16_t* residual, const uint16_t* gamma,
                        float eps, uint16_t* residual_out, uint16_t* Y, ttl::ReduceNormParams& p) {
  if (b <= 0 || n <= 0 || b > kMaxDim || n > 65536)
    return fail(TTL_ERR_SHAPE, "%s: need 1 <= b < 2^31 and 1 <= n <= 65536 (b=%lld n=%lld)", who,
                (long long)b, (long long)n);
  if (P == nullptr || gamma == nullptr || residual_out == nullptr || Y == nullptr)
    return fail(TTL_ERR_NULL, "%s: P, gamma, residual_out and Y must be non-NULL", who);
  if (t < 1) return fail(TTL_ERR_RANK, "%s: t=%d must be >= 1", who, t);
  if (!(eps >= 0.0f)) return fail(TTL_ERR_SHAPE, "%s: eps must be >= 0", who);
  if (n % 8 != 0) return fail(TTL_ERR_ALIGN, "%s: n=%lld must be a multiple of 8", who, (long long)n);
  if (!aligned16(P) || !aligned16(gamma) || !aligned16(residual_out) || !aligned16(Y) ||
      (residual != nullptr && !aligned16(residual)))
    return fail(TTL_ERR_ALIGN, "%s: all tensors must be 16-byte aligned", who);
  const int64_t out_bytes = rows * n * 2;
  const int64_t p_bytes = b * n * 2 * t;
  if (overlaps(Y, out_bytes, P, p_bytes) || overlaps(Y, out_bytes, gamma, n * 2) ||
      overlaps(Y, out_bytes, residual_out, out_bytes) ||
      (residual != nullptr && overlaps(Y, out_bytes, residual, out_bytes)))
    return fail(TTL_ERR_UNSUPPORTED, "%s: Y must not overlap any other tensor", who);
  if (overlaps(residual_out, out_bytes, P, p_bytes) || overlaps(residual_out, out_bytes, gamma, n * 2) ||
      (residual != nullptr && residual != residual_out &&
       overlaps(residual_out, out_bytes, residual, out_bytes)))
    return fail(TTL_ERR_UNSUPPORTED,
                "%s: residual_out may alias residual exactly but must not overlap anything else", who);
  p = {};
  p.P = P + row0 * n;
  p.residual = residual;
  p.gamma = gamma;
  p.residual_out = residual_out;
  p.Y = Y;
  p.b = rows;
  p.n = n;
  p.plane = b * n;
  p.t = t;
  p.eps = eps;
  return TTL_OK;
}

}  // namespace

extern "C" {

const char* ttl_last_error(void) { return g_last_error.c_str(); }

ttl_status ttl_pack_weight_blocked(const uint16_t* W, int64_t k, int64_t n, uint16_t* W_blk, void* stream) {
  static const char* who = "ttl_pack_weight_blocked";
  if (k <= 0 || n <= 0 || k * n >= ((int64_t)1 << 31))
    return fail(TTL_ERR_SHAPE, "%s: need k, n >= 1 and k*n < 2^31 (k=%lld n=%lld)", who, (long long)k,
                (long long)n);
  if (W == nullptr || W_blk == nullptr) return fail(TTL_ERR_NULL, "%s: W and W_blk must be non-NULL", who);
  if (k % 64 != 0 || n % 128 != 0 || !aligned16(W) || !aligned16(W_blk))
    return fail(TTL_ERR_ALIGN, "%s: need k %% 64 == 0, n %% 128 == 0 and 16-byte aligned buffers", who);
  if (overlaps(W, k * n * 2, W_blk, k * n * 2))
    return fail(TTL_ERR_UNSUPPORTED, "%s: W and W_blk must not overlap", who);
  return launch_status(ttl::launch_pack_blocked(W, k, n, W_blk, static_cast<hipStream_t>(stream)), who);
}

int32_t ttl_version(void) { return 100; }  // 0.1.0

ttl_status shard_linear_col_stored(const uint16_t* X, int64_t b, int64_t k, const uint16_t* W, int64_t n,
                                   ttl_weight_layout w_layout, int32_t t, int32_t rank,
                                   const ttl_col_split* split, ttl_epilogue epi, uint16_t* Y, void* stream) {
  return col_entry("shard_linear_col_stored", X, b, k, W, n, w_layout, t, rank, split, epi, Y, stream);
}

ttl_status shard_linear_col(const uint16_t* X, int64_t b, int64_t k, const uint16_t* W, int64_t n,
                            int32_t t, int32_t rank, const ttl_col_split* split, ttl_epilogue epi,
                            uint16_t* Y, void* stream) {
  return col_entry("shard_linear_col", X, b, k, W, n, TTL_W_KN, t, rank, split, epi, Y, stream);
}

ttl_status shard_linear_col_noalloc(const uint16_t* X, int64_t b, int64_t k, const uint16_t* W, int64_t n,
                                    ttl_weight_layout w_layout, int32_t t, int32_t rank,
                                    const ttl_col_split* split, ttl_epilogue epi, uint16_t* Y,
                                    void* stream) {
  static const char* who = "shard_linear_col_noalloc";
  ttl::GemmParams p;
  int64_t width = 0;
  const ttl_status st = col_setup(who, X, b, k, W, n, w_layout, t, rank, split, epi, Y, p, width);
  if (st != TTL_OK) return st;
  if (output_overlaps(Y, b * width, X, b * k, W, k * n))
    return fail(TTL_ERR_UNSUPPORTED, "%s: Y must not overlap X or W", who);
  p.C = Y;
  p.ldc = width;
  // The plan is walked once without launching to size its split-K partials: a call that needs more
  // than the static scratch is refused before anything is enqueued.
  const size_t need = ttl::gemm_workspace_bytes(p);
  if (need > kScratchBytes)
    return fail(TTL_ERR_UNSUPPORTED,
                "%s: this call's split-K partials need %zu bytes, more than the %zu-byte static scratch "
                "(shard_linear_col_stored serves it with an allocated workspace)", who, need, kScratchBytes);
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess)
    return fail(TTL_ERR_HIP, "%s: no device address for the static scratch: %s", who, hipGetErrorString(e));
  return launch_status(ttl::launch_gemm_fixed_workspace(p, ws, kScratchBytes, static_cast<hipStream_t>(stream)),
                       who);
}

ttl_status shard_linear_col_gathered(const uint16_t* X, int64_t b, int64_t k, const uint16_t* W,
                                     int64_t n, ttl_weight_layout w_layout, int32_t t, int32_t rank,
                                     const ttl_col_split* split, ttl_epilogue epi, uint16_t* Y_all,
                                     void* stream) {
  static const char* who = "shard_linear_col_gathered";
  ttl::GemmParams p;
  int64_t width = 0;
  const ttl_status st = col_setup(who, X, b, k, W, n, w_layout, t, rank, split, epi, Y_all, p, width);
  if (st != TTL_OK) return st;
  if (width * t > kMaxLda)
    return fail(TTL_ERR_SHAPE, "%s: gathered row of %lld columns exceeds the supported pitch", who,
                (long long)(width * t));
  if (output_overlaps(Y_all, b * width * t, X, b * k, W, k * n))
    return fail(TTL_ERR_UNSUPPORTED, "%s: Y_all must not overlap X or W", who);
  p.C = Y_all + (int64_t)rank * width;  // this rank's block of the gathered row
  p.ldc = width * t;
  return launch_status(ttl::launch_gemm(p, static_cast<hipStream_t>(stream)), who);
}

ttl_status shard_linear_row_stored(const uint16_t* X, int64_t b, int64_t k, int32_t x_is_parallel,
                                   const uint16_t* W, int64_t n, ttl_weight_layout w_layout, int32_t t,
                                   int32_t rank, uint16_t* P, void* stream) {
  return row_entry("shard_linear_row_stored", X, b, k, x_is_parallel, W, n, w_layout, t, rank, P, stream);
}

ttl_status shard_linear_row(const uint16_t* X, int64_t b, int64_t k, int32_t x_is_parallel,
                            const uint16_t* W, int64_t n, int32_t t, int32_t rank, uint16_t* P,
                            void* stream) {
  return row_entry("shard_linear_row", X, b, k, x_is_parallel, W, n, TTL_W_KN, t, rank, P, stream);
}

ttl_status ttl_set_gemm_override(int32_t kernel, int32_t splits, int32_t plan_cus, int32_t trace) {
  static const char* who = "ttl_set_gemm_override";
  if (kernel < TTL_GEMM_AUTO || kernel > TTL_GEMM_STREAM_NK)
    return fail(TTL_ERR_UNSUPPORTED, "%s: unknown kernel family %d", who, kernel);
  if (splits < 0 || plan_cus < 0)
    return fail(TTL_ERR_UNSUPPORTED, "%s: splits=%d and plan_cus=%d must be >= 0", who, splits, plan_cus);
  ttl::set_gemm_override(kernel, splits, plan_cus, trace != 0);
  return TTL_OK;
}

ttl_status reduce_partials_rmsnorm(const uint16_t* P, int32_t t, int64_t b, int64_t n,
                                   const uint16_t* residual, const uint16_t* gamma, float eps,
                                   uint16_t* residual_out, uint16_t* Y, void* stream) {
  static const char* who = "reduce_partials_rmsnorm";
  ttl::ReduceNormParams p;
  const ttl_status st =
      reduce_setup(who, P, t, b, n, 0, b, residual, gamma, eps, residual_out, Y, p);
  if (st != TTL_OK) return st;
  return launch_status(ttl::launch_reduce_rmsnorm(p, static_cast<hipStream_t>(stream)), who);
}

ttl_status reduce_partials_rmsnorm_peers(const uint16_t* const* P_ranks, int32_t t, int64_t b, int64_t n,
                                         int64_t row0, int64_t rows, const uint16_t* residual,
                                         const uint16_t* gamma, float eps, uint16_t* residual_out,
                                         uint16_t* Y, void* stream) {
  static const char* who = "reduce_partials_rmsnorm_peers";
  if (b <= 0 || n <= 0 || b > kMaxDim || n > 65536)
    return fail(TTL_ERR_SHAPE, "%s: need 1 <= b < 2^31 and 1 <= n <= 65536 (b=%lld n=%lld)", who,
                (long long)b, (long long)n);
  if (row0 < 0 || rows <= 0 || row0 + rows > b)
    return fail(TTL_ERR_SHAPE, "%s: rows [%lld, %lld) must be a non-empty range inside [0, %lld)", who,
                (long long)row0, (long long)(row0 + rows), (long long)b);
  if (t < 1) return fail(TTL_ERR_RANK, "%s: t=%d must be >= 1", who, t);
  if (t > TTL_MAX_PEERS)
    return fail(TTL_ERR_UNSUPPORTED, "%s: t=%d partial buffers exceed the %d supported", who, t, TTL_MAX_PEERS);
  if (P_ranks == nullptr) return fail(TTL_ERR_NULL, "%s: P_ranks must be non-NULL", who);
  for (int r = 0; r < t; ++r) {
    if (P_ranks[r] == nullptr) return fail(TTL_ERR_NULL, "%s: P_ranks[%d] is NULL", who, r);
    if (!aligned16(P_ranks[r])) return fail(TTL_ERR_ALIGN, "%s: P_ranks[%d] is not 16-byte aligned", who, r);
  }
  // Shape, eps, alignment and aliasing of the residual, gamma and outputs, with rank 0's buffer as
  // the partial; then the outputs against every other rank's buffer.
  ttl::ReduceNormParams p;
  const ttl_status st = reduce_setup(who, P_ranks[0] + row0 * n, 1, rows, n, 0, rows, residual, gamma, eps,
                                     residual_out, Y, p);
  if (st != TTL_OK) return st;
  const int64_t out_bytes = rows * n * 2, slab = b * n * 2;
  for (int r = 0; r < t; ++r)
    if (overlaps(Y, out_bytes, P_ranks[r], slab) || overlaps(residual_out, out_bytes, P_ranks[r], slab))
      return fail(TTL_ERR_UNSUPPORTED, "%s: the outputs must not overlap P_ranks[%d]", who, r);
  p.t = t;
  p.peers = 1;
  for (int r = 0; r < t; ++r) p.peer[r] = P_ranks[r] + row0 * n;
  return launch_status(ttl::launch_reduce_rmsnorm(p, static_cast<hipStream_t>(stream)), who);
}

ttl_status reduce_scatter_partials_rmsnorm(const uint16_t* P, int32_t t, int64_t b, int64_t n,
                                           int32_t rank, const uint16_t* residual,
                                           const uint16_t* gamma, float eps, uint16_t* residual_out,
                                           uint16_t* Y, void* stream) {
  static const char* who = "reduce_scatter_partials_rmsnorm";
  if (t < 1 || rank < 0 || rank >= t)
    return fail(TTL_ERR_RANK, "%s: need t >= 1 and 0 <= rank < t (t=%d rank=%d)", who, t, rank);
  if (b > 0 && b % t != 0)
    return fail(TTL_ERR_NOT_DIVISIBLE, "%s: b=%lld rows are not divisible by t=%d", who,
                (long long)b, t);
  const int64_t rows = b / t;
  ttl::ReduceNormParams p;
  const ttl_status st = reduce_setup(who, P, t, b, n, (int64_t)rank * rows, rows, residual, gamma, eps,
                                     residual_out, Y, p);
  if (st != TTL_OK) return st;
  return launch_status(ttl::launch_reduce_rmsnorm(p, static_cast<hipStream_t>(stream)), who);
}

}  // extern "C"
