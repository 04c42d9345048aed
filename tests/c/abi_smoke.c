/*
 * A plain C program against include/linattn.h: it links liblinattn.so and
 * makes calls that need no GPU (every forward/backward call below fails its
 * argument checks before anything is enqueued, so the fake pointers are
 * never dereferenced).  Exit status 0 when every result is as documented.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "linattn.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main(void) {
  void* A = (void*)(uintptr_t)(1u << 20); /* 16-byte aligned, never touched */
  void* B = (void*)(uintptr_t)(2u << 20);
  void* C = (void*)(uintptr_t)(3u << 20);
  float* S = (float*)(uintptr_t)(4u << 20);
  void* O = (void*)(uintptr_t)(5u << 20);
  float* S2 = (float*)(uintptr_t)(6u << 20);
  size_t bytes = 0;
  la_launch_opts opts;
  memset(&opts, 0, sizeof opts);

  expect("abi version", la_abi_version(), 13);
  expect("status string", strcmp(la_status_string(LA_E_ALIAS), "illegal buffer overlap"), 0);
  expect("chunk d=48", la_chunk_forward(A, B, C, S, O, S2, 1, 2, 64, 48, LA_BF16, LA_F32, 1e-6f, 0),
         LA_E_UNSUPPORTED);
  expect("chunk misaligned",
         la_chunk_forward((char*)A + 8, B, C, S, O, S2, 1, 2, 64, 64, LA_BF16, LA_F32, 1e-6f, 0),
         LA_E_ALIGN);
  expect("global out == q", la_global_forward(A, B, C, A, S2, 1, 2, 64, 64, LA_BF16, LA_F32, 1e-6f, 0),
         LA_E_ALIAS);
  expect("blockcausal T=0",
         la_blockcausal_forward_ex(A, B, C, S, O, S2, 1, 2, 640, 0, 64, LA_BF16, LA_F32, 1e-6f,
                                   &opts, 0),
         LA_E_INVAL);
  expect("rope grid 0", la_chunk_forward_rope(A, B, C, S, O, S2, 1, 2, 64, 64, LA_BF16, LA_F32,
                                              1e-6f, 0, 0, 4, 10000.0f, 0),
         LA_E_INVAL);
  expect("workspace size", la_backward_workspace_size(1, 32, 75600, 75600, 64, LA_BF16, &bytes),
         LA_OK);
  if (bytes == 0) {
    fprintf(stderr, "workspace size is zero\n");
    ++failures;
  }
  expect("backward without workspace",
         la_chunk_backward(A, B, C, S, O, NULL, (void*)S2, (char*)O + (64 << 20), (char*)O + (96 << 20),
                           NULL, 1, 2, 64, 64, LA_BF16, LA_F32, 1e-6f, NULL, 0, 0),
         LA_E_INVAL);
  expect("tconv C % 8", la_temporal_conv_chunk(A, NULL, S, NULL, O, NULL, 1, 3, 10, 12, LA_BF16,
                                               LA_BF16, 0),
         LA_E_UNSUPPORTED);
  {
    int splits = -1, wgs = -1;
    expect("plan", la_plan(1, 32, 75600, 64, LA_BF16, LA_F32, 0, 0, &splits, &wgs), LA_OK);
    expect("plan splits", splits, 16);
    expect("plan readout", wgs, 512);
  }
  {
    la_backward_shape sh;
    memset(&sh, 0xff, sizeof sh);
    expect("backward plan", la_backward_plan(1, 32, 75600, 75600, 64, LA_BF16, 0, 0, 0, 0, &sh),
           LA_OK);
    expect("backward plan blocks", sh.blocks, 1);
    expect("backward plan query splits", sh.query_splits, 16);
    expect("backward plan query grid", sh.query_workgroups, 512);
    expect("backward plan key items", sh.key_items, 0);
    expect("backward plan key grid", sh.key_workgroups, 512);
    expect("backward plan sweep units", sh.key_sweep_units, 591);
    expect("backward plan no output",
           la_backward_plan(1, 32, 75600, 75600, 64, LA_BF16, 0, 0, 0, 0, NULL), LA_E_INVAL);
  }
  if (failures == 0) printf("abi_smoke ok\n");
  return failures == 0 ? 0 : 1;
}
