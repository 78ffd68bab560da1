/* The C ABI from plain C: ttl.h compiles as C99, libttl.so links, and every entry point rejects
 * invalid arguments with the documented status before touching the device.  Every pointer below is
 * a fake, aligned address that is never dereferenced: each call fails validation, so no HIP call is
 * made and no GPU is needed.  Exit status 0 when every check passes. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ttl.h"

static int failures = 0;

static void expect(const char* what, ttl_status got, ttl_status want) {
  if (got != want) {
    printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, ttl_last_error());
    ++failures;
  } else {
    printf("ok   %s: %s\n", what, ttl_last_error());
  }
}

int main(void) {
  const uint16_t* X = (const uint16_t*)(uintptr_t)0x10000;
  const uint16_t* W = (const uint16_t*)(uintptr_t)0x20000;
  uint16_t* Y = (uint16_t*)(uintptr_t)0x30000;
  const uint16_t* gamma = (const uint16_t*)(uintptr_t)0x40000;
  ttl_col_split split;
  memset(&split, 0, sizeof split);
  split.nseg = 2;
  split.seg_n[0] = 688;
  split.seg_n[1] = 688;
  split.seg_parts[0] = 2;
  split.seg_parts[1] = 2;

  if (ttl_version() < 100) {
    printf("FAIL version %d\n", ttl_version());
    ++failures;
  }
  /* the statement's form: X[b,k], W[k,n], t, rank */
  expect("col: NULL X", shard_linear_col(NULL, 16, 256, W, 1376, 2, 0, &split, TTL_EPI_SILU_MUL, Y, NULL),
         TTL_ERR_NULL);
  expect("col: rank >= t", shard_linear_col(X, 16, 256, W, 1376, 2, 2, &split, TTL_EPI_SILU_MUL, Y, NULL),
         TTL_ERR_RANK);
  expect("col: Y overlapping W",
         shard_linear_col(X, 16, 256, W, 1376, 2, 0, &split, TTL_EPI_SILU_MUL, (uint16_t*)(uintptr_t)0x20400, NULL),
         TTL_ERR_UNSUPPORTED);
  expect("col (stored): unknown layout",
         shard_linear_col_stored(X, 16, 256, W, 1376, 7, 2, 0, &split, TTL_EPI_SILU_MUL, Y, NULL),
         TTL_ERR_UNSUPPORTED);
  expect("gathered: b = 0",
         shard_linear_col_gathered(X, 0, 256, W, 1376, TTL_W_KN, 2, 0, &split, TTL_EPI_NONE, Y, NULL),
         TTL_ERR_SHAPE);
  expect("row: k not divisible by t", shard_linear_row(X, 16, 689, 1, W, 256, 2, 0, Y, NULL),
         TTL_ERR_NOT_DIVISIBLE);
  expect("row (stored): blocked with (k/t) % 64", shard_linear_row_stored(X, 16, 1024, 1, W, 256, TTL_W_BLOCKED, 32, 0, Y, NULL),
         TTL_ERR_ALIGN);
  expect("override: unknown kernel", ttl_set_gemm_override(TTL_GEMM_STREAM_NK + 1, 0, 0, 0), TTL_ERR_UNSUPPORTED);
  expect("reduce: misaligned Y", reduce_partials_rmsnorm(X, 2, 16, 256, NULL, gamma, 1e-5f, Y, Y + 2, NULL),
         TTL_ERR_ALIGN);
  expect("reduce-scatter: b not divisible by t",
         reduce_scatter_partials_rmsnorm(X, 2, 15, 256, 0, NULL, gamma, 1e-5f, Y, Y + 4096, NULL),
         TTL_ERR_NOT_DIVISIBLE);
  {
    const uint16_t* peers[2] = {X, W};
    expect("peers: t > TTL_MAX_PEERS",
           reduce_partials_rmsnorm_peers(peers, TTL_MAX_PEERS + 1, 16, 256, 0, 16, NULL, gamma, 1e-5f, Y,
                                         Y + 4096, NULL),
           TTL_ERR_UNSUPPORTED);
  }
  expect("pack: n % 128", ttl_pack_weight_blocked(W, 256, 1000, Y, NULL), TTL_ERR_ALIGN);
  printf("%s\n", failures == 0 ? "ALL OK" : "FAILURES");
  return failures == 0 ? 0 : 1;
}
