/* abi_sanitize.c -- drives the host-side checks of every libkda entry point
 * (include/kda.h) through their error paths, for a build of the library's host
 * code with the address and undefined-behaviour sanitizers and without device
 * code: every call here must return before its first HIP call (argument,
 * size, grid and workspace checks), so no GPU is needed.  Test infrastructure;
 * exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int fails = 0;
#define EXPECT(call, want)                                                            \
  do {                                                                                \
    const long got_ = (long)(call);                                                   \
    if (got_ != (long)(want)) {                                                       \
      fprintf(stderr, "FAIL line %d: %s = %ld, want %ld\n", __LINE__, #call, got_, (long)(want)); \
      ++fails;                                                                        \
    }                                                                                 \
  } while (0)

int main(void) {
  void* p = (void*)16;  /* never dereferenced: the checks fail first */
  const float* fp = (const float*)p;
  const int32_t* ip = (const int32_t*)p;
  float* wfp = (float*)p;
  const size_t bad = (size_t)-1, big = (size_t)-1;

  for (int s = -1; s <= 5; ++s) EXPECT(kda_status_string(s) != NULL && strlen(kda_status_string(s)) > 0, 1);

  /* workspace queries */
  size_t prev = 0;
  for (int64_t T = 1; T <= 1 << 20; T *= 4) {
    const size_t w = kda_chunk_fwd_workspace_bytes(T, 3, 64, 128, 0);
    EXPECT(w != bad && w % 256 == 0 && w >= prev, 1);
    prev = w;
    EXPECT(kda_chunk_bwd_workspace_bytes(T, 3, 64, 128, 1) % 256, 0);
    EXPECT(kda_chunk_bwd_conv_workspace_bytes(T, 3, 64, 128, 1) > kda_chunk_bwd_workspace_bytes(T, 3, 64, 128, 1), 1);
    EXPECT(kda_chunk_fwd_workspace_bytes(T, 3, 64, 128, KDA_MODE_WINDOWED) != bad, 1);
  }
  EXPECT(kda_chunk_fwd_workspace_bytes(0, 1, 64, 128, 0), 0);
  EXPECT(kda_chunk_fwd_workspace_bytes(10, 1, 64, 96, 0), bad);
  EXPECT(kda_chunk_fwd_workspace_bytes(10, 0, 64, 128, 0), bad);
  EXPECT(kda_chunk_fwd_workspace_bytes(-1, 1, 64, 128, 0), bad);
  EXPECT(kda_chunk_fwd_workspace_bytes(10, 1, 64, 128, 0x20), bad);
  EXPECT(kda_chunk_bwd_workspace_bytes(10, 1, 64, 96, 1), bad);
  EXPECT(kda_chunk_bwd_conv_workspace_bytes(10, 1, 0, 128, 1), bad);
  EXPECT(kda_chunk_fwd_num_stages(100, 1, 64, 0), 3);
  EXPECT(kda_chunk_fwd_num_stages(100, 1, 64, KDA_MODE_WINDOWED), 2);
  EXPECT(kda_chunk_fwd_num_stages(100, 0, 64, 0), -1);

  /* forward entry points: null pointer, mode, head dimension, workspace, grid */
  EXPECT(kda_chunk_fwd(NULL, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 0, p, p, big, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 0x20, p, p, big, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd(p, p, p, p, p, fp, fp, ip, 0, 10, 4, 128, 0, p, p, big, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 96, 0, p, p, big, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_chunk_fwd(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 0, p, p, 1, NULL), KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd(p, p, p, p, p, fp, fp, ip, 1, 1, (1 << 24) + 1, 128, 0, p, p, big, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_chunk_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 0, 4, 128, 0, NULL, NULL, 0, NULL), KDA_OK);
  EXPECT(kda_chunk_fwd_state(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 0, p, p, 1, NULL, NULL, NULL), KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd_state(p, p, p, p, p, fp, fp, NULL, 1, 10, 4, 128, 0, p, p, big, NULL, NULL, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd_conv(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 0, NULL, NULL, 1, p, p, big, NULL, NULL, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd_conv(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 0, fp, NULL, 1, p, p, 1, NULL, NULL, NULL), KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd_rect(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 16, 200, 0, p, p, big, NULL, NULL, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_chunk_fwd_rect(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 0, 24, 0, p, p, big, NULL, NULL, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd_rect(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 16, 24, 0, p, p, 1, NULL, NULL, NULL), KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd_noalloc(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, KDA_MODE_CHECK_CU, p, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_chunk_fwd_noalloc(p, p, p, p, p, fp, fp, ip, 1, 1 << 20, 64, 128, KDA_MODE_FP32_INTERMEDIATE, p, NULL), KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd_noalloc(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 96, 0, p, NULL), KDA_ERR_UNSUPPORTED);
  {
    void* ev[4] = {p, p, p, p};
    EXPECT(kda_chunk_fwd_timed(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 0, p, p, big, NULL, ev, 3), KDA_ERR_INVALID_ARG);
  }
  /* token-serial */
  EXPECT(kda_recurrent_fwd(NULL, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 0, p, NULL, NULL, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_recurrent_fwd(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, KDA_MODE_CHECK_CU, p, NULL, NULL, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_recurrent_fwd_rect(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 48, 24, 0, p, NULL, NULL, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_recurrent_fwd_rect(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 200, 0, p, NULL, NULL, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_recurrent_fwd(p, p, p, p, p, fp, fp, ip, 1, 0, 4, 128, 0, p, NULL, NULL, NULL), KDA_OK);
  /* backward */
  EXPECT(kda_chunk_bwd(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 1, NULL, p, NULL, p, p, p, p, p, NULL, wfp, NULL, p, big, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_bwd(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 1, NULL, p, NULL, p, p, p, p, p, wfp, wfp, NULL, p, 1, NULL), KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_bwd(p, p, p, p, p, fp, fp, ip, 1 << 24, 1 << 24, 1, 128, 1, NULL, p, NULL, p, p, p, p, p, wfp, wfp, NULL, p, big, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_chunk_bwd_conv(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 1, fp, NULL, 1, NULL, p, NULL, p, p, p, p, p, wfp, wfp, NULL, NULL, NULL, p, big, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_bwd_conv(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 1, NULL, NULL, 1, NULL, p, NULL, p, p, p, p, p, wfp, wfp, NULL, wfp, NULL, p, big, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_bwd_conv(p, p, p, p, p, fp, fp, ip, 1, 10, 4, 128, 1, fp, NULL, 1, NULL, p, NULL, p, p, p, p, p, wfp, wfp, NULL, wfp, NULL, p, 1, NULL), KDA_ERR_WORKSPACE);
  if (fails) return 1;
  printf("libkda host checks under the sanitizers: all clean\n");
  return 0;
}
