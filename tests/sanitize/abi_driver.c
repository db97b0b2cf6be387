/*
 * Host-side driver of the C ABI for the AddressSanitizer / UndefinedBehaviorSanitizer build: the
 * library's host code (argument checks, plans, workspace arithmetic, error strings) runs here
 * with sanitizers on and no GPU work. Every compute call below is rejected before anything is
 * enqueued, so pointers are fake addresses that are never dereferenced.
 * Exit status 0 when every call returns the expected status; a sanitizer report aborts.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssm.h"

static int failures = 0;

#define EXPECT(call, want)                                                                   \
  do {                                                                                       \
    ssm_status s_ = (call);                                                                  \
    if (s_ != (want)) {                                                                      \
      fprintf(stderr, "%s:%d: got %s, want %s (%s)\n", __FILE__, __LINE__,                   \
              ssm_status_string(s_), ssm_status_string(want), ssm_last_error_detail());      \
      ++failures;                                                                            \
    } else if (s_ != SSM_OK && ssm_last_error_detail()[0] == 0) {                            \
      fprintf(stderr, "%s:%d: no error detail\n", __FILE__, __LINE__);                       \
      ++failures;                                                                            \
    }                                                                                        \
  } while (0)

/* fake device addresses: 16-byte aligned and 1 TiB apart, so no two ranges overlap */
#define P(k) ((void*)(uintptr_t)((uint64_t)(k) << 40))
#define F(k) ((float*)P(k))

int main(void) {
  if (ssm_abi_version() != 1) { fprintf(stderr, "abi version\n"); return 1; }
  for (int s = -1; s <= 6; ++s) {
    const char* t = ssm_status_string((ssm_status)s);
    if (!t || !t[0]) { fprintf(stderr, "status string %d\n", s); return 1; }
  }

  /* workspace queries over a sweep of shapes (plan and size arithmetic) */
  size_t acc = 0;
  const int64_t Ns[] = {1, 2, 4, 8, 16, 3};
  for (int64_t B = 0; B <= 64; B = B ? B * 4 : 1)
    for (int64_t L = 0; L <= ((int64_t)1 << 24); L = L ? L * 8 : 1)
      for (int64_t D = 4; D <= 16384; D *= 8)
        for (int i = 0; i < 6; ++i) {
          acc += ssm_scan_fwd_workspace_bytes(B, L, D, Ns[i], SSM_F32);
          acc += ssm_scan_fwd_segmented_workspace_bytes(B, L, D, Ns[i], 256);
          acc += ssm_scan_fwd_conv_workspace_bytes(B, L, D, Ns[i], 0);
          acc += ssm_scan_bwd_workspace_bytes(B, L, D, Ns[i], SSM_BF16);
          acc += ssm_scan_bwd_segmented_workspace_bytes(B, L, D, Ns[i], 48);
        }
  for (int64_t L = 0; L <= 65536; L = L ? L * 4 : 1)
    for (int64_t q = 64; q <= 256; q *= 2) {
      acc += ssd_chunk_fwd_workspace_bytes(2, L, 80, 64, 128, q, SSM_BF16);
      acc += ssd_chunk_fwd_workspace_bytes(2, L, 80, 64, 128, q, SSM_F32);
      acc += ssd_chunk_fwd_grouped_workspace_bytes(2, L, 80, 64, 64, 8, q, SSM_BF16);
      acc += ssd_chunk_fwd_grouped_workspace_bytes(2, L, 80, 64, 64, 8, q, SSM_F32);
      acc += ssd_chunk_bwd_workspace_bytes(2, L, 80, 64, 128, 1, SSM_BF16);
    }
  for (int64_t M = 1; M <= 128; M *= 2) {
    acc += ssm_linear_workspace_bytes(M, 2048, 50288);
    acc += ssm_linear_workspace_bytes(M, 4096, 2048);
    acc += ssm_block_step_workspace_bytes(M, 2048, 4096, 16, 4, 128);
  }
  if (acc == 0) { fprintf(stderr, "all workspace queries returned 0\n"); return 1; }

  /* selective scan: rejected arguments */
  const int64_t ws_big = (int64_t)1 << 40;
  EXPECT(ssm_scan_fwd(1, 16, 64, 3, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                      P(6), NULL, NULL, 0, NULL), SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_scan_fwd(1, 16, 6, 16, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                      P(6), NULL, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT);
  EXPECT(ssm_scan_fwd(-1, 16, 64, 16, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                      P(6), NULL, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT);
  EXPECT(ssm_scan_fwd(1, 16, 64, 16, (ssm_dtype)7, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL,
                      NULL, P(6), NULL, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT);
  EXPECT(ssm_scan_fwd(1, 16, 64, 16, SSM_F32, NULL, P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                      P(6), NULL, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT);
  EXPECT(ssm_scan_fwd(1, 16, 64, 16, SSM_F32, (char*)P(1) + 4, P(2), NULL, 0, F(3), P(4), P(5), NULL,
                      NULL, NULL, P(6), NULL, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT);
  EXPECT(ssm_scan_fwd(1, 16, 64, 16, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                      (char*)P(1) + 64, NULL, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT);   /* y overlaps x */
  EXPECT(ssm_scan_fwd(1, 16, 64, 16, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, F(7),
                      P(6), (float*)((char*)P(7) + 16), NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT);
  EXPECT(ssm_scan_fwd(65536, 1, 4, 1, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                      P(6), NULL, NULL, 0, NULL), SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_scan_fwd(1, 4096, 256, 16, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                      P(6), NULL, NULL, 0, NULL), SSM_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(ssm_scan_fwd_segmented(1, 4096, 256, 16, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL,
                                NULL, NULL, P(6), NULL, 0, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT);
  EXPECT(ssm_scan_fwd_segmented(1, 4096, 256, 16, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL,
                                NULL, NULL, P(6), NULL, 256, P(9), 100, NULL), SSM_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(ssm_scan_fwd_noalloc(1, 16, 64, 32, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL,
                              NULL, P(6), NULL, NULL), SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_scan_fwd_conv(1, 16, 64, 16, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                           4, NULL, NULL, NULL, P(6), NULL, 0, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT);
  EXPECT(ssm_scan_fwd_conv(1, 16, 64, 16, SSM_F32, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                           5, F(8), NULL, NULL, P(6), NULL, 0, NULL, 0, NULL), SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_scan_bwd(1, 16, 64, 3, SSM_BF16, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                      P(6), NULL, P(7), P(8), F(9), F(10), F(11), NULL, NULL, NULL, NULL, P(12),
                      (size_t)ws_big, NULL), SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_scan_bwd(1, 16, 64, 16, SSM_BF16, P(1), P(2), NULL, 0, F(3), P(4), P(5), NULL, NULL, NULL,
                      P(6), NULL, P(1), P(8), F(9), F(10), F(11), NULL, NULL, NULL, NULL, P(12),
                      (size_t)ws_big, NULL), SSM_ERR_INVALID_ARGUMENT);   /* dx overlaps x */

  /* decode step */
  EXPECT(ssm_state_update(4, 64, 16, 4, SSM_BF16, P(1), P(2), NULL, 1, F(3), P(4), P(5), NULL, NULL,
                          P(6), NULL, NULL, F(7), P(8), NULL), SSM_ERR_INVALID_ARGUMENT);   /* no conv_w */
  EXPECT(ssm_state_update(4, 64, 5, 0, SSM_BF16, P(1), P(2), NULL, 1, F(3), P(4), P(5), NULL, NULL,
                          NULL, NULL, NULL, F(7), P(8), NULL), SSM_ERR_UNSUPPORTED);

  /* SSD */
  EXPECT(ssd_chunk_fwd(2, 512, 8, 32, 128, 256, SSM_BF16, P(1), P(2), NULL, 1, F(3), P(4), P(5), NULL,
                       NULL, NULL, P(6), NULL, P(9), (size_t)ws_big, NULL), SSM_ERR_UNSUPPORTED);
  EXPECT(ssd_chunk_fwd(2, 512, 8, 64, 128, 100, SSM_BF16, P(1), P(2), NULL, 1, F(3), P(4), P(5), NULL,
                       NULL, NULL, P(6), NULL, P(9), (size_t)ws_big, NULL), SSM_ERR_UNSUPPORTED);
  EXPECT(ssd_chunk_fwd(2, 512, 8, 64, 128, 256, SSM_F32, P(1), P(2), NULL, 1, F(3), P(4), P(5), NULL,
                       NULL, NULL, P(6), NULL, P(9), 16, NULL), SSM_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(ssd_chunk_bwd(2, 512, 8, 64, 128, 1, SSM_F32, P(1), P(2), NULL, 1, F(3), P(4), P(5), NULL, 0,
                       NULL, NULL, P(6), NULL, P(7), P(8), F(9), F(10), F(11), NULL, NULL, NULL, NULL, P(12),
                       (size_t)ws_big, NULL), SSM_ERR_UNSUPPORTED);   /* backward: bf16 only */
  EXPECT(ssd_chunk_fwd(2, 512, 8, 64, 128, 256, SSM_BF16, P(1), P(2), NULL, 1, F(3), P(4), P(5), NULL,
                       NULL, NULL, P(6), NULL, P(9), 16, NULL), SSM_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(ssd_chunk_fwd_grouped(2, 512, 8, 64, 128, 3, 256, SSM_BF16, P(1), P(2), NULL, 1, F(3), P(4), P(5),
                               NULL, 0, NULL, NULL, P(6), NULL, P(9), (size_t)ws_big, NULL),
         SSM_ERR_INVALID_ARGUMENT);   /* G does not divide H */
  EXPECT(ssd_chunk_bwd(2, 512, 8, 64, 128, 1, SSM_BF16, P(1), P(2), NULL, 1, F(3), P(4), P(5), NULL, 0,
                       NULL, NULL, P(6), NULL, P(2), P(8), F(9), F(10), F(11), NULL, NULL, NULL, NULL, P(12),
                       (size_t)ws_big, NULL), SSM_ERR_INVALID_ARGUMENT);   /* ddelta overlaps delta */

  /* model pieces */
  EXPECT(ssm_linear(128, 100, 2048, P(1), P(2), NULL, P(3), NULL, 0, NULL), SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_layernorm(4, 12, P(1), F(2), F(3), 1e-5f, P(4), NULL), SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_layernorm(4, 2048, P(1), F(2), F(3), 0.0f, P(4), NULL), SSM_ERR_INVALID_ARGUMENT);
  EXPECT(ssm_block_step(129, 2048, 4096, 16, 4, 128, P(1), F(2), F(3), 1e-5f, P(4), F(5), NULL, P(6), P(7),
                        F(8), F(9), NULL, P(10), P(11), F(12), P(13), (size_t)ws_big, NULL),
         SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_block_step(128, 2000, 4096, 16, 4, 128, P(1), F(2), F(3), 1e-5f, P(4), F(5), NULL, P(6), P(7),
                        F(8), F(9), NULL, P(10), P(11), F(12), P(13), (size_t)ws_big, NULL),
         SSM_ERR_UNSUPPORTED);

  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("abi driver ok (%zu workspace bytes summed)\n", acc);
  return 0;
}
