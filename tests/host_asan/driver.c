/*
 * Host-side driver for the AddressSanitizer build of libla (CPU only): runs
 * every entry point's host code -- argument validation, workspace sizes,
 * error strings, dispatch order of long batches, argument packing -- with
 * fake device addresses that no kernel ever touches.  Calls that pass
 * validation reach the HIP launch, which fails without a GPU (LA_ERR_HIP) or
 * enqueues nothing.  Exit status 0 when every status matches; ASan aborts the
 * run on any memory error in the library's host code.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "la.h"

static int failures = 0;

static void expect(const char* what, la_status got, la_status want) {
  const char* msg = la_last_error();
  if (got != want) {
    printf("FAIL %s: %s (%s), expected %s\n", what, la_status_str(got), msg, la_status_str(want));
    ++failures;
  }
  if (got != LA_OK && strlen(msg) == 0 && got != LA_ERR_HIP) {
    printf("FAIL %s: no error text\n", what);
    ++failures;
  }
}

static void expect_not(const char* what, la_status got, la_status bad) {
  if (got == bad) {
    printf("FAIL %s: %s (%s)\n", what, la_status_str(got), la_last_error());
    ++failures;
  }
}

#define Q ((void*)0x10000000)
#define K ((void*)0x20000000)
#define V ((void*)0x30000000)
#define O ((void*)0x40000000)
#define KVF ((float*)0x50000000)
#define KVI ((float*)0x60000000)
#define CUD ((int32_t*)0x70000000)
#define WS ((void*)0x90000000)
#define DO ((void*)0xA0000000)
#define DQ ((void*)0xB0000000)
#define DK ((void*)0xC0000000)
#define DV ((void*)0xD0000000)

int main(void) {
  const int H = 4, D = 128;
  float decay[LA_MAX_HEADS + 1];
  for (int i = 0; i <= LA_MAX_HEADS; ++i) decay[i] = 0.9f;
  int32_t cu[3] = {0, 40, 100};

  /* prefill: invalid arguments */
  expect("prefill negative seqs",
         la_prefill(Q, K, V, CUD, cu, -1, 100, H, D, LA_BF16, LA_BF16, decay, NULL, O, KVF, NULL),
         LA_ERR_INVALID_ARG);
  expect("prefill too many heads",
         la_prefill(Q, K, V, CUD, cu, 2, 100, LA_MAX_HEADS + 1, D, LA_BF16, LA_BF16, decay, NULL, O,
                    KVF, NULL),
         LA_ERR_UNSUPPORTED);
  expect("prefill head_dim 96",
         la_prefill(Q, K, V, CUD, cu, 2, 100, H, 96, LA_BF16, LA_BF16, decay, NULL, O, KVF, NULL),
         LA_ERR_UNSUPPORTED);
  expect("prefill NULL host cu",
         la_prefill(Q, K, V, CUD, NULL, 2, 100, H, D, LA_BF16, LA_BF16, decay, NULL, O, KVF, NULL),
         LA_ERR_INVALID_ARG);
  expect("prefill o overlaps k",
         la_prefill(Q, K, V, CUD, cu, 2, 100, H, D, LA_BF16, LA_BF16, decay, NULL,
                    (char*)K + 64, KVF, NULL),
         LA_ERR_INVALID_ARG);
  float bad_decay[4] = {0.9f, 1.5f, 0.9f, 0.9f};
  expect("prefill decay > 1",
         la_prefill(Q, K, V, CUD, cu, 2, 100, H, D, LA_BF16, LA_BF16, bad_decay, NULL, O, KVF, NULL),
         LA_ERR_INVALID_ARG);
  /* prefill: valid arguments reach the launch (no GPU here: a HIP error) */
  expect_not("prefill valid",
             la_prefill(Q, K, V, CUD, cu, 2, 100, H, D, LA_BF16, LA_BF16, decay, KVI, O, KVF,
                        NULL),
             LA_ERR_INVALID_ARG);

  /* a batch of 512 sequences: the longest-first dispatch order is built */
  {
    const int S = 512;
    int32_t* cub = (int32_t*)malloc(sizeof(int32_t) * (S + 1));
    cub[0] = 0;
    for (int s = 0; s < S; ++s) cub[s + 1] = cub[s] + (s * 37) % 101;
    expect_not("prefill 512 sequences",
               la_prefill(Q, K, V, CUD, cub, S, cub[S], 2, 64, LA_BF16, LA_BF16, decay, NULL, O,
                          NULL, NULL),
               LA_ERR_INVALID_ARG);
    size_t bytes = 0;
    expect("segmented workspace 512 sequences",
           la_prefill_segmented_workspace_size(S, cub, 2, 128, 64, &bytes), LA_OK);
    expect("segmented workspace d = 64",
           la_prefill_segmented_workspace_size(S, cub, 2, 64, 64, &bytes), LA_OK);
    expect("backward segmented workspace",
           la_prefill_backward_segmented_workspace_size(S, cub, 2, 128, 64, &bytes), LA_OK);
    expect("segmented workspace, library's segment length",
           la_prefill_segmented_workspace_size(S, cub, 2, 128, 0, &bytes), LA_OK);
    expect("backward segmented workspace, library's segment length",
           la_prefill_backward_segmented_workspace_size(S, cub, 2, 64, 0, &bytes), LA_OK);
    free(cub);
  }

  /* segmented */
  size_t ws_bytes = 0;
  expect("segmented workspace size", la_prefill_segmented_workspace_size(2, cu, H, D, 64, &ws_bytes),
         LA_OK);
  size_t bad_bytes = 1;
  expect("segmented bad segment_len",
         la_prefill_segmented_workspace_size(2, cu, H, D, 100, &bad_bytes), LA_ERR_INVALID_ARG);
  if (bad_bytes != 0) {
    printf("FAIL segmented bad segment_len: bytes not zeroed\n");
    ++failures;
  }
  expect("segmented workspace too small",
         la_prefill_segmented(Q, K, V, CUD, cu, 2, 100, H, D, LA_BF16, LA_BF16, decay, NULL, O,
                              KVF, 64, WS, 16, NULL),
         LA_ERR_INVALID_ARG);
  expect_not("segmented valid",
             la_prefill_segmented(Q, K, V, CUD, cu, 2, 100, H, D, LA_BF16, LA_BF16, decay, KVI, O,
                                  KVF, 64, WS, ws_bytes, NULL),
             LA_ERR_INVALID_ARG);
  expect("segmented noalloc fp32 input",
         la_prefill_segmented_noalloc(Q, K, V, CUD, cu, 2, 100, H, D, LA_FP32, LA_FP32, decay, NULL,
                                      O, KVF, 64, NULL),
         LA_ERR_UNSUPPORTED);

  /* backward */
  size_t bw = 0;
  expect("backward workspace size", la_prefill_backward_workspace_size(2, H, D, &bw), LA_OK);
  expect("backward fp32 input",
         la_prefill_backward(Q, K, V, DO, CUD, cu, 2, 100, H, D, LA_FP32, LA_BF16, decay, NULL, NULL,
                             DQ, DK, DV, NULL, NULL, 0, NULL),
         LA_ERR_UNSUPPORTED);
  expect("backward dq overlaps dk",
         la_prefill_backward(Q, K, V, DO, CUD, cu, 2, 100, H, D, LA_BF16, LA_BF16, decay, NULL,
                             NULL, DQ, (char*)DQ + 128, DV, NULL, NULL, 0, NULL),
         LA_ERR_INVALID_ARG);
  expect_not("backward valid",
             la_prefill_backward(Q, K, V, DO, CUD, cu, 2, 100, H, D, LA_BF16, LA_BF16, decay, KVI,
                                 KVF, DQ, DK, DV, (float*)0xE0000000, WS, bw, NULL),
             LA_ERR_INVALID_ARG);

  /* decode and the pools */
  int32_t slots[3] = {3, 0, 7}, dup[3] = {3, 3, 7};
  expect("decode negative batch",
         la_decode(Q, K, V, KVF, decay, -1, H, D, LA_BF16, O, NULL), LA_ERR_INVALID_ARG);
  expect_not("decode valid", la_decode(Q, K, V, KVF, decay, 3, H, D, LA_BF16, O, NULL),
             LA_ERR_INVALID_ARG);
  expect("decode pool repeated slot",
         la_decode_pool(Q, K, V, KVF, 10, CUD, dup, decay, 3, H, D, LA_BF16, O, NULL),
         LA_ERR_INVALID_ARG);
  expect("decode pool slot out of range",
         la_decode_pool(Q, K, V, KVF, 5, CUD, slots, decay, 3, H, D, LA_BF16, O, NULL),
         LA_ERR_INVALID_ARG);
  expect("prefill pool repeated slot",
         la_prefill_pool(Q, K, V, CUD, cu, 2, 100, H, D, LA_BF16, LA_BF16, decay, KVF, 10, CUD, dup,
                         O, NULL),
         LA_ERR_INVALID_ARG);
  /* the repeated-slot check sorts a copy of the slots: its memory follows
     the batch, not a pool of 2^31 - 1 states */
  int32_t far_dup[3] = {5, 2147483646, 5}, last_twice[2] = {2147483646, 2147483646};
  expect("decode pool repeated slot, largest pool",
         la_decode_pool(Q, K, V, KVF, 2147483647, CUD, far_dup, decay, 3, H, D, LA_BF16, O, NULL),
         LA_ERR_INVALID_ARG);
  expect("decode pool last slot of the largest pool twice",
         la_decode_pool(Q, K, V, KVF, 2147483647, CUD, last_twice, decay, 2, H, D, LA_BF16, O,
                        NULL),
         LA_ERR_INVALID_ARG);

  /* dtype arguments outside the enumerators (a C caller may pass any int):
     rejected, and never read as the enum type before they are checked */
  const la_dtype bad_dtypes[2] = {(la_dtype)7, (la_dtype)-1};
  la_norm nrm = {(const float*)0xF0000000, 1e-6f, NULL};
  int32_t ok_slots[2] = {0, 1};
  for (int i = 0; i < 2; ++i) {
    const la_dtype bd = bad_dtypes[i];
    expect("prefill bad in_dtype",
           la_prefill(Q, K, V, CUD, cu, 2, 100, H, D, bd, LA_BF16, decay, NULL, O, KVF, NULL),
           LA_ERR_INVALID_ARG);
    expect("prefill bad out_dtype",
           la_prefill(Q, K, V, CUD, cu, 2, 100, H, D, LA_BF16, bd, decay, NULL, O, KVF, NULL),
           LA_ERR_INVALID_ARG);
    expect("segmented bad in_dtype",
           la_prefill_segmented(Q, K, V, CUD, cu, 2, 100, H, D, bd, LA_BF16, decay, NULL, O, KVF,
                                64, WS, 1 << 20, NULL),
           LA_ERR_INVALID_ARG);
    expect("segmented noalloc bad out_dtype",
           la_prefill_segmented_noalloc(Q, K, V, CUD, cu, 2, 100, H, D, LA_BF16, bd, decay, NULL,
                                        O, KVF, 64, NULL),
           LA_ERR_INVALID_ARG);
    expect("pool prefill bad in_dtype",
           la_prefill_pool(Q, K, V, CUD, cu, 2, 100, H, D, bd, LA_BF16, decay, KVF, 4, CUD,
                           ok_slots, O, NULL),
           LA_ERR_INVALID_ARG);
    expect("normed bad in_dtype",
           la_prefill_normed(Q, K, V, CUD, cu, 2, 100, H, D, bd, LA_BF16, decay, NULL, &nrm, O,
                             KVF, WS, 1 << 20, NULL),
           LA_ERR_INVALID_ARG);
    expect("backward bad grad_dtype",
           la_prefill_backward(Q, K, V, DO, CUD, cu, 2, 100, H, D, LA_BF16, bd, decay, NULL, NULL,
                               DQ, DK, DV, NULL, NULL, 0, NULL),
           LA_ERR_INVALID_ARG);
    expect("backward segmented bad in_dtype",
           la_prefill_backward_segmented(Q, K, V, DO, CUD, cu, 2, 100, H, D, bd, LA_BF16, decay,
                                         NULL, NULL, DQ, DK, DV, NULL, 64, WS, 1 << 20, NULL),
           LA_ERR_INVALID_ARG);
    expect("decode bad in_dtype", la_decode(Q, K, V, KVF, decay, 3, H, D, bd, O, NULL),
           LA_ERR_INVALID_ARG);
    expect("decode pool bad in_dtype",
           la_decode_pool(Q, K, V, KVF, 4, CUD, ok_slots, decay, 2, H, D, bd, O, NULL),
           LA_ERR_INVALID_ARG);
    expect("decode normed bad in_dtype",
           la_decode_normed(Q, K, V, KVF, decay, 3, H, D, bd, &nrm, O, NULL), LA_ERR_INVALID_ARG);
  }

  /* kernel plan: every branch of the planner on the host (256 compute units) */
  {
    static int32_t cuv[130], order[129];
    int32_t n = -1;
    for (int S = 0; S <= 129; S += 1) {
      cuv[0] = 0;  /* mixed lengths, some empty */
      for (int i = 1; i <= S; ++i) cuv[i] = cuv[i - 1] + (i % 7 == 0 ? 0 : 64 + 911 * (i % 5));
      for (int h = 1; h <= 64; h *= 4) {
        expect("plan mixed", la_prefill_kernel_plan(S, cuv, h, 128, 256, &n, order), LA_OK);
        if (n < 0 || n > S) {
          printf("FAIL plan range S=%d H=%d: %d\n", S, h, n);
          ++failures;
        }
      }
      for (int i = 0; i <= S; ++i) cuv[i] = i * 640;  /* equal lengths */
      expect("plan equal", la_prefill_kernel_plan(S, cuv, 64, 128, 256, &n, NULL), LA_OK);
      expect("plan d64", la_prefill_kernel_plan(S, cuv, 64, 64, 256, &n, order), LA_OK);
      if (n != 0) {
        printf("FAIL plan d64 S=%d: %d\n", S, n);
        ++failures;
      }
    }
    expect("plan NULL out", la_prefill_kernel_plan(2, cu, 64, 128, 256, NULL, NULL),
           LA_ERR_INVALID_ARG);
    expect("plan negative units", la_prefill_kernel_plan(2, cu, 64, 128, -5, &n, NULL),
           LA_ERR_INVALID_ARG);
    expect("plan bad head_dim", la_prefill_kernel_plan(2, cu, 64, 80, 256, &n, NULL),
           LA_ERR_UNSUPPORTED);
  }

  /* status strings */
  for (int s = -1; s < 6; ++s) {
    const char* name = la_status_str((la_status)s);
    if (!name || !*name) {
      printf("FAIL status string %d\n", s);
      ++failures;
    }
  }
  printf("%s: %d failure(s)\n", failures ? "FAILED" : "OK", failures);
  return failures ? 1 : 0;
}
