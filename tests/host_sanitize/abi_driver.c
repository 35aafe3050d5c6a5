/*
 * Host-side check of libqlora's C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every entry point of qlora.h is called with
 * arguments that its validation must turn into a status before any device
 * work (null, misaligned or short buffers, bad sizes, enums and ranks, shapes
 * at the edge of the index range), and the host-only size queries run over
 * the layer shapes of the benchmark workloads and at the range limit. Built
 * from the library's sources with the sanitizers on the host code only (no
 * device code is compiled: nothing here may launch a kernel) and run on a
 * machine with or without a GPU. Plain C, so it also checks that qlora.h is a
 * C header. Exit status 0 when every status matches; a sanitizer report
 * aborts the run.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qlora.h"

static int failures = 0, checks = 0;

static void expect(int got, int want, const char* what) {
  ++checks;
  if (got != want) {
    ++failures;
    printf("FAIL %s: status %d (%s), expected %d (%s)\n", what, got, qlora_status_str(got),
           want, qlora_status_str(want));
  }
}

/* Stand-ins for device buffers: aligned addresses that the validation only
 * compares and never dereferences. */
static _Alignas(256) unsigned char arena[1 << 20];
#define P(off) ((void*)(arena + (off)))

static qlora_linear layer(int K, int N, int r, int fmt) {
  qlora_linear L;
  memset(&L, 0, sizeof L);
  L.K = K; L.N = N; L.r = r; L.alpha = 16.f; L.fmt = fmt;
  L.codes = P(0); L.scales = P(256); L.A = (const float*)P(512); L.B = (const float*)P(768);
  L.heads = 0;
  return L;
}

static void size_queries(void) {
  /* the benchmark workloads' layers, with their row counts */
  static const int shapes[][5] = {
      /* M, K, N, r, fmt */
      {64, 256, 256, 4, QLORA_W8},       {1024, 784, 1024, 8, QLORA_W8},
      {1024, 1024, 1024, 8, QLORA_W8},   {4096, 768, 2304, 4, QLORA_W8},
      {4096, 768, 768, 4, QLORA_W8},     {4096, 768, 3072, 4, QLORA_W8},
      {4096, 3072, 768, 4, QLORA_W8},    {512, 2048, 16384, 8, QLORA_W8},
      {512, 16384, 2048, 8, QLORA_W8},   {512, 2048, 16384, 8, QLORA_W8O},
      {2048, 4096, 4096, 4, QLORA_W4G128}, {33, 512, 80, 16, QLORA_W8},
      {5, 256, 144, 32, QLORA_W8},       {1, 16, 16, 1, QLORA_W8},
  };
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
    const int M = shapes[i][0], K = shapes[i][1], N = shapes[i][2], r = shapes[i][3];
    const int fmt = shapes[i][4];
    qlora_linear L = layer(K, N, r, fmt);
    size_t cb = 0, sb = 0, fw = 0, bw = 0, pb = 0;
    for (int dt = QLORA_F32; dt <= QLORA_BF16; ++dt) {
      const int want = (fmt != QLORA_W8 && dt == QLORA_F32) ? QLORA_EUNSUPPORTED : QLORA_OK;
      expect(qlora_fwd_workspace(&L, M, dt, &fw), want, "fwd_workspace");
      expect(qlora_bwd_workspace(&L, M, dt, &bw), want, "bwd_workspace");
      expect(qlora_bwd_partials_bytes(&L, M, dt, &pb), want, "partials_bytes");
      if (want == QLORA_OK) {
        ++checks;
        if (pb > bw || pb % 256) { ++failures; printf("FAIL partials %zu of %zu\n", pb, bw); }
        ++checks;
        if (qlora_bwd_main_kernel(&L, M, dt) == NULL) { ++failures; printf("FAIL kernel name\n"); }
      } else {
        ++checks;
        if (qlora_bwd_main_kernel(&L, M, dt) != NULL) { ++failures; printf("FAIL kernel name\n"); }
      }
    }
    expect(qlora_weight_bytes(K, N, fmt, &cb, &sb), QLORA_OK, "weight_bytes");
  }
  /* at the edge of the 2^31 index range and past it */
  qlora_linear L = layer(1 << 16, 1 << 15, 8, QLORA_W8);
  size_t b = 0;
  expect(qlora_fwd_workspace(&L, 1, QLORA_BF16, &b), QLORA_ERANGE, "K N = 2^31");
  L = layer(1 << 14, 1 << 16, 8, QLORA_W8);
  expect(qlora_bwd_workspace(&L, 1, QLORA_BF16, &b), QLORA_OK, "K N = 2^30");
  L = layer(32768, 32752, 8, QLORA_W8);
  expect(qlora_bwd_workspace(&L, 65535, QLORA_BF16, &b), QLORA_OK, "M K just below 2^31");
  expect(qlora_bwd_workspace(&L, 65536, QLORA_BF16, &b), QLORA_ERANGE, "M K = 2^31");
  L = layer(16384, 16384, 32, QLORA_W8);
  expect(qlora_bwd_workspace(&L, 131071, QLORA_BF16, &b), QLORA_OK, "M K just below 2^31");
  expect(qlora_fwd_workspace(&L, 131071, QLORA_BF16, &b), QLORA_OK, "fwd M K just below 2^31");
  expect(qlora_bwd_workspace(&L, 131072, QLORA_BF16, &b), QLORA_ERANGE, "M K = 2^31");
  L = layer(16384, 16384, 32, QLORA_W4G128);
  expect(qlora_bwd_workspace(&L, 131071, QLORA_BF16, &b), QLORA_OK, "4-bit at the range edge");
  L = layer(16384 + 128, 1024, 8, QLORA_W4G128);
  expect(qlora_fwd_workspace(&L, 64, QLORA_BF16, &b), QLORA_EUNSUPPORTED, "4-bit past 128 groups");
  int32_t cap = 0;
  size_t o1, o2, o3;
  expect(qlora_outlier_layout(16384, 2048, &o1, &o2, &o3, &cap), QLORA_OK, "outlier layout");
  expect(qlora_outlier_layout(1 << 16, 1 << 15, &o1, &o2, &o3, &cap), QLORA_ERANGE, "outlier range");
  expect(qlora_outlier_layout(16, 16, NULL, &o2, &o3, &cap), QLORA_EINVAL, "outlier null");
}

static void bad_layers(void) {
  size_t b = 0;
  qlora_linear L;
  expect(qlora_fwd_workspace(NULL, 16, QLORA_BF16, &b), QLORA_EINVAL, "null layer");
  L = layer(256, 256, 4, QLORA_W8);
  expect(qlora_fwd_workspace(&L, 16, QLORA_BF16, NULL), QLORA_EINVAL, "null size");
  expect(qlora_fwd_workspace(&L, 0, QLORA_BF16, &b), QLORA_EINVAL, "M = 0");
  expect(qlora_fwd_workspace(&L, -5, QLORA_BF16, &b), QLORA_EINVAL, "M < 0");
  expect(qlora_fwd_workspace(&L, 16, 7, &b), QLORA_EINVAL, "dtype");
  L = layer(250, 256, 4, QLORA_W8);
  expect(qlora_fwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "K % 16");
  L = layer(256, 8, 4, QLORA_W8);
  expect(qlora_fwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "N < 16");
  L = layer(256, 256, 0, QLORA_W8);
  expect(qlora_fwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "r = 0");
  L = layer(256, 256, 33, QLORA_W8);
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "r = 33");
  L = layer(256, 256, 4, 9);
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "fmt");
  L = layer(192, 256, 4, QLORA_W4G128);
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "4-bit K % 128");
  L = layer(256, 256, 4, QLORA_W8);
  L.A = (const float*)P(4);
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "misaligned A");
  L = layer(256, 256, 4, QLORA_W8);
  L.codes = NULL;
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "null codes");
  L = layer(256, 384, 4, QLORA_W8);
  L.heads = 5;
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "heads do not divide N");
  L.heads = 3;
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_OK, "head width 128");
  L.heads = 4;
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EUNSUPPORTED, "head width 96");
  L = layer(256, 384, 4, QLORA_W8);
  L.heads = 6;
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_OK, "head width 64");
  L.heads = -1;
  expect(qlora_bwd_workspace(&L, 16, QLORA_BF16, &b), QLORA_EINVAL, "heads < 0");
}

static void bad_calls(void) {
  qlora_linear L = layer(256, 256, 4, QLORA_W8);
  size_t fw = 0, bw = 0;
  expect(qlora_fwd_workspace(&L, 64, QLORA_BF16, &fw), QLORA_OK, "fwd ws");
  expect(qlora_bwd_workspace(&L, 64, QLORA_BF16, &bw), QLORA_OK, "bwd ws");
  void *x = P(1024), *y = P(2048), *ws = P(4096);
  float *t = (float*)P(3072), *dA = (float*)P(3328), *dB = (float*)P(3584);
  /* forward */
  expect(qlora_fwd(&L, 64, QLORA_BF16, NULL, y, t, ws, fw, NULL), QLORA_EINVAL, "fwd null x");
  expect(qlora_fwd(&L, 64, QLORA_BF16, P(1025), y, t, ws, fw, NULL), QLORA_EINVAL, "fwd misaligned x");
  expect(qlora_fwd(&L, 64, QLORA_BF16, x, NULL, t, ws, fw, NULL), QLORA_EINVAL, "fwd null y");
  expect(qlora_fwd(&L, 64, QLORA_BF16, x, y, (float*)P(3076), ws, fw, NULL), QLORA_EINVAL,
         "fwd misaligned t");
  expect(qlora_fwd(&L, 64, QLORA_BF16, x, y, t, ws, fw - 1, NULL), QLORA_EWORKSPACE, "fwd short ws");
  expect(qlora_fwd(&L, 64, QLORA_BF16, x, y, t, NULL, fw, NULL), QLORA_EWORKSPACE, "fwd null ws");
  expect(qlora_fwd_timed(&L, 64, QLORA_BF16, x, y, t, ws, fw, NULL, 0, NULL, NULL), QLORA_EINVAL,
         "fwd repeats 0");
  expect(qlora_fwd_a8w4(&L, 64, QLORA_BF16, x, y, t, ws, fw, NULL), QLORA_EUNSUPPORTED, "a8w4 on int8");
  expect(qlora_fwd_acc(&L, 64, QLORA_BF16, x, NULL, ws, fw, NULL), QLORA_EINVAL, "acc null");
  /* backward */
  expect(qlora_bwd(&L, 64, QLORA_BF16, NULL, y, t, x, dA, dB, ws, bw, NULL), QLORA_EINVAL, "bwd null x");
  expect(qlora_bwd(&L, 64, QLORA_BF16, x, NULL, t, x, dA, dB, ws, bw, NULL), QLORA_EINVAL, "bwd null dy");
  expect(qlora_bwd(&L, 64, QLORA_BF16, x, y, t, x, NULL, dB, ws, bw, NULL), QLORA_EINVAL, "bwd null dA");
  expect(qlora_bwd(&L, 64, QLORA_BF16, x, y, t, x, dA, (float*)P(3592), ws, bw, NULL), QLORA_EINVAL,
         "bwd misaligned dB");
  expect(qlora_bwd(&L, 64, QLORA_BF16, x, y, t, P(8), dA, dB, ws, bw, NULL), QLORA_EINVAL,
         "bwd misaligned dx");
  expect(qlora_bwd(&L, 64, QLORA_BF16, x, y, t, x, dA, dB, ws, bw - 16, NULL), QLORA_EWORKSPACE,
         "bwd short ws");
  expect(qlora_bwd_timed(&L, 64, QLORA_BF16, x, y, t, x, dA, dB, ws, bw, NULL, -1, NULL, NULL),
         QLORA_EINVAL, "bwd repeats < 1");
  expect(qlora_bwd_partial(&L, 64, QLORA_BF16, x, y, t, x, P(8), bw, NULL), QLORA_EWORKSPACE,
         "partial misaligned ws");
  expect(qlora_bwd_finish(&L, 64, QLORA_BF16, dA, dB, ws, 0, NULL), QLORA_EWORKSPACE, "finish ws 0");
  /* the allocation-free backward: a layer whose scratch is past the static array */
  qlora_linear G = layer(2048, 16384, 8, QLORA_W8);
  expect(qlora_bwd_noalloc(&G, 512, QLORA_BF16, x, y, t, x, dA, dB, NULL), QLORA_EWORKSPACE,
         "noalloc too large");
  expect(qlora_bwd_noalloc(NULL, 512, QLORA_BF16, x, y, t, x, dA, dB, NULL), QLORA_EINVAL,
         "noalloc null layer");
  /* batched combine */
  qlora_finish_item items[3];
  for (int i = 0; i < 3; ++i) {
    items[i].L = &L; items[i].M = 64; items[i].dtype = QLORA_BF16;
    items[i].dA = dA; items[i].dB = dB; items[i].ws = ws; items[i].ws_bytes = bw;
  }
  expect(qlora_bwd_finish_batch(NULL, 3, NULL), QLORA_EINVAL, "batch null");
  expect(qlora_bwd_finish_batch(items, 0, NULL), QLORA_EINVAL, "batch empty");
  items[2].ws_bytes = 0;
  expect(qlora_bwd_finish_batch(items, 3, NULL), QLORA_EWORKSPACE, "batch item 2 short");
  items[2].ws_bytes = bw;
  items[1].L = NULL;
  expect(qlora_bwd_finish_batch(items, 3, NULL), QLORA_EINVAL, "batch item 1 null");
  /* quantizers and merge */
  expect(qlora_quantize(NULL, 256, 256, QLORA_W8, P(0), P(256), NULL), QLORA_EINVAL, "quantize null W");
  expect(qlora_quantize((const float*)P(0), 256, 250, QLORA_W8, P(0), P(256), NULL), QLORA_EINVAL,
         "quantize N % 16");
  expect(qlora_quantize((const float*)P(0), 256, 256, 5, P(0), P(256), NULL), QLORA_EINVAL,
         "quantize fmt");
  expect(qlora_quantize_heads((const float*)P(0), 4, 256, 384, QLORA_W8, P(0), P(256), NULL),
         QLORA_EUNSUPPORTED, "quantize head width 96");
  expect(qlora_quantize_heads((const float*)P(0), 2, 256, 256, QLORA_W8O, P(0), P(256), NULL),
         QLORA_EUNSUPPORTED, "quantize w8o heads");
  expect(qlora_quantize_heads((const float*)P(0), 0, 256, 256, QLORA_W8, P(0), P(256), NULL),
         QLORA_EINVAL, "quantize heads 0");
  qlora_linear W4 = layer(256, 256, 4, QLORA_W4G128);
  expect(qlora_merge(&W4, P(8192), P(16384), NULL), QLORA_EUNSUPPORTED, "merge 4-bit");
  expect(qlora_merge(&L, P(0), P(16384), NULL), QLORA_EINVAL, "merge onto the codes");
  expect(qlora_merge(&L, P(1 << 18), P((1 << 18) + 1024), NULL), QLORA_EINVAL, "merge outputs overlap");
  expect(qlora_quantize_rows(P(0), 0, 256, QLORA_BF16, (int8_t*)P(256), (float*)P(512), NULL),
         QLORA_EINVAL, "rows M = 0");
  expect(qlora_quantize_rows(P(0), 1 << 16, 1 << 15, QLORA_BF16, (int8_t*)P(256), (float*)P(512), NULL),
         QLORA_ERANGE, "rows range");
  size_t cb, sb;
  expect(qlora_weight_bytes(256, 256, QLORA_W8, NULL, &sb), QLORA_EINVAL, "weight_bytes null");
  expect(qlora_weight_bytes(256, 256, 3, &cb, &sb), QLORA_EINVAL, "weight_bytes fmt");
  for (int s = -1; s <= 6; ++s)
    if (qlora_status_str(s) == NULL) { ++failures; printf("FAIL status_str(%d)\n", s); }
}

int main(void) {
  size_queries();
  bad_layers();
  bad_calls();
  printf("%d checks, %d failures\n", checks, failures);
  return failures ? 1 : 0;
}
