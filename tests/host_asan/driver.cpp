// Host-side checks of the C-ABI library under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built from the library's own sources with host code instrumented (device code is not
// compiled: no kernel is launched here, and the machine needs no GPU).  Every size query is
// swept over edge values of its arguments (zero, one, the limits the header states, one past
// them, the largest int32 values, negatives), and every entry point is called with the
// argument errors it must turn into a status code before any device work.  A sanitizer
// report or a wrong status ends the program with a non-zero exit code.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "smla.h"

static int failures = 0;

#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
      fprintf(stderr, __VA_ARGS__);                         \
      fprintf(stderr, "\n");                                \
      failures++;                                           \
    }                                                       \
  } while (0)

static const int32_t kInts[] = {INT32_MIN, -65536, -17, -1, 0, 1, 2, 3, 4, 5, 7, 15, 16, 17, 31, 32, 48, 63,
                                64, 65, 128, 255, 256, 1000, 1024, 2047, 2048, 2049, 4096, 8192, 65535,
                                65536, 65537, 1 << 20, 1 << 24, 1 << 30, INT32_MAX - 1, INT32_MAX};
static const int64_t kLongs[] = {INT64_MIN, -1, 0, 1, 4, 31, 32, 8192, 140000, 146000, 1 << 20,
                                 (int64_t)1 << 31, (int64_t)1 << 32, (int64_t)1 << 40, INT64_MAX};
#define N(a) (int)(sizeof(a) / sizeof((a)[0]))

// A 16-byte aligned stand-in for a device pointer: never dereferenced by the host code.
static void* const D = (void*)(uintptr_t)0x10000;

static void size_queries() {
  long calls = 0;
  for (int a = 0; a < N(kInts); a++)
    for (int b = 0; b < N(kInts); b++)
      for (int c = 0; c < N(kInts); c++) {
        const int32_t T = kInts[a], H = kInts[b], topk = kInts[c];
        const int32_t S = smla_choose_num_splits(T, H, topk);
        EXPECT(S >= 0, "choose_num_splits(%d, %d, %d) = %d", T, H, topk, S);
        if (T <= 0 || H <= 0 || H % 16 != 0 || topk <= 0) EXPECT(S == 0, "splits for a rejected shape");
        for (int d = 0; d < N(kInts); d += 3) {
          const size_t w = smla_decode_workspace_bytes(T, H, topk, kInts[d]);
          if (T <= 0 || H <= 0 || H % 16 != 0 || topk <= 0 || kInts[d] < 0)
            EXPECT(w == 0, "workspace for a rejected shape (%d, %d, %d, %d) = %zu", T, H, topk, kInts[d], w);
          calls++;
        }
        for (int tpg = 0; tpg <= 5; tpg++) {
          const size_t w = smla_decode_grouped_workspace_bytes(T, H, tpg, topk, c % 3 == 0 ? 0 : kInts[c]);
          if (T <= 0 || H <= 0 || tpg < 1 || tpg > 4 || topk <= 0) EXPECT(w == 0, "grouped workspace, rejected shape");
          calls++;
        }
      }
  for (int a = 0; a < N(kInts); a++)
    for (int b = 0; b < N(kLongs); b++)
      for (int c = 0; c < N(kInts); c++)
        for (int d = 0; d < N(kInts); d += 4) {
          const size_t w = smla_indexer_workspace_bytes(kInts[a], kLongs[b], kInts[c], kInts[d]);
          if (kInts[a] <= 0 || kLongs[b] < 0 || kInts[c] < 1 || kInts[d] < 0)
            EXPECT(w == 0, "indexer workspace, rejected arguments");
          calls++;
        }
  printf("size queries: %ld calls\n", calls);
}

static void status_strings() {
  for (int s = -10; s <= 10; s++) EXPECT(smla_status_string(s) != nullptr, "status string %d", s);
  EXPECT(smla_status_string(INT32_MIN) != nullptr, "status string min");
}

// Argument errors of every entry point: a status below zero, before any device work.
static void argument_errors() {
  const float nan = NAN, inf = INFINITY;
  const float scales[] = {0.0f, -1.0f, nan, inf, -inf};
  int calls = 0;
  auto bad = [&](int st, const char* what) {
    EXPECT(st < 0, "%s returned %d", what, st);
    calls++;
  };
  // null / misaligned pointers, negative or out-of-range sizes
  bad(nvfp4_pack_rows(nullptr, (const int32_t*)D, 4, D, 100, nullptr), "pack null src");
  bad(nvfp4_pack_rows(D, (const int32_t*)D, -1, D, 100, nullptr), "pack n < 0");
  bad(nvfp4_pack_rows(D, (const int32_t*)D, 4, (char*)D + 1, 100, nullptr), "pack misaligned pool");
  bad(nvfp4_pack_rows(D, (const int32_t*)D, 4, D, -5, nullptr), "pack pool_rows < 0");
  bad(fp8_pack_rows(nullptr, (const int32_t*)D, 4, D, 100, nullptr), "fp8 pack null src");
  bad(fp8_pack_rows(D, (const int32_t*)D, -3, D, 100, nullptr), "fp8 pack n < 0");
  bad(nvfp4_unpack_rows_f16(nullptr, 100, (const int32_t*)D, 4, D, nullptr), "unpack null pool");
  bad(nvfp4_unpack_rows_f16(D, 100, (const int32_t*)D, -2, D, nullptr), "unpack n < 0");
  bad(nvfp4_stage_fp8(nullptr, 100, (const int32_t*)D, 2, 64, D, nullptr), "stage null pool");
  bad(nvfp4_stage_fp8(D, 100, (const int32_t*)D, -2, 64, D, nullptr), "stage T < 0");
  bad(nvfp4_stage_fp8(D, 100, (const int32_t*)D, 2, 0, D, nullptr), "stage topk 0");
  for (float sc : scales) {
    bad(sparse_mla_decode(D, D, 100, (const int32_t*)D, 2, 16, 64, sc, D, (float*)D, 0, D, 1 << 20, nullptr),
        "decode scale");
    bad(sparse_mla_decode_noalloc(D, D, 100, (const int32_t*)D, 2, 16, 64, sc, D, (float*)D, 0, nullptr),
        "noalloc scale");
    bad(sparse_mla_decode_fp8rows(D, D, (const int32_t*)D, 100, 2, 16, 64, sc, D, (float*)D, 0, D, 1 << 20, nullptr),
        "fp8rows scale");
    bad(sparse_mla_decode_fp8pool(D, D, 100, (const int32_t*)D, 2, 16, 64, sc, D, (float*)D, 0, D, 1 << 20,
                                  nullptr),
        "fp8pool scale");
    bad(sparse_mla_decode_grouped(D, D, 100, (const int32_t*)D, 4, 16, 4, 64, sc, D, (float*)D, 0, D, 1 << 20,
                                  nullptr),
        "grouped scale");
    bad(sparse_mla_decode_blhnc(D, D, 10, 2, 0, 16, (const int32_t*)D, 2, 16, 64, sc, D, (float*)D, 0, D, 1 << 20,
                                nullptr),
        "blhnc scale");
  }
  for (int a = 0; a < N(kInts); a++) {
    const int32_t v = kInts[a];
    if (v < 0) {
      bad(sparse_mla_decode(D, D, 100, (const int32_t*)D, v, 16, 64, 0.1f, D, (float*)D, 0, D, 1 << 20, nullptr),
          "decode T < 0");
      bad(sparse_mla_decode(D, D, 100, (const int32_t*)D, 2, 16, 64, 0.1f, D, (float*)D, v, D, 1 << 20, nullptr),
          "decode splits < 0");
      bad(sparse_indexer_topk((const float*)D, 64, nullptr, nullptr, v, 8, (int32_t*)D, 0, nullptr, 0, nullptr),
          "indexer T < 0");
      bad(sparse_mla_combine((const float*)D, (const float*)D, v, 2, 16, D, (float*)D, nullptr), "combine T < 0");
      bad(smla_group_union((const int32_t*)D, v, 64, 2, 100, 128, (int32_t*)D, (int32_t*)D, nullptr),
          "union T < 0");
      bad(blhnc_copy_blocks(D, 10, (const int32_t*)D, D, 10, (const int32_t*)D, v, 1024, nullptr), "copy n < 0");
    }
    if (v <= 0 || v > 65536) {
      bad(sparse_mla_decode(D, D, 100, (const int32_t*)D, 2, 16, v, 0.1f, D, (float*)D, 0, D, 1 << 20, nullptr),
          "decode topk out of range");
      bad(sparse_mla_decode_fp8pool(D, D, 100, (const int32_t*)D, 2, 16, v, 0.1f, D, (float*)D, 0, D, 1 << 20,
                                    nullptr),
          "fp8pool topk out of range");
    }
    if (v <= 0 || v % 16 != 0) {
      bad(sparse_mla_decode(D, D, 100, (const int32_t*)D, 2, v, 64, 0.1f, D, (float*)D, 0, D, 1 << 20, nullptr),
          "decode H");
      bad(sparse_mla_combine((const float*)D, (const float*)D, 2, 2, v, D, (float*)D, nullptr), "combine H");
    }
    if (v <= 0 || (v & (v - 1)) != 0 || v > 65536) {
      bad(nvfp4_pack_rows_blhnc(D, (const int32_t*)D, 4, D, 10, 2, 0, v, nullptr), "blhnc pack block_rows");
      bad(sparse_mla_decode_blhnc(D, D, 10, 2, 0, v, (const int32_t*)D, 2, 16, 64, 0.1f, D, (float*)D, 0, D,
                                  1 << 20, nullptr),
          "blhnc decode block_rows");
    }
    if (v < 0 || v >= 2) {   // layer outside 0 .. layers-1 with 2 layers
      bad(sparse_mla_decode_blhnc(D, D, 10, 2, v, 16, (const int32_t*)D, 2, 16, 64, 0.1f, D, (float*)D, 0, D,
                                  1 << 20, nullptr),
          "blhnc decode layer");
    }
    if (v < 1 || v > 4) {
      bad(smla_group_union((const int32_t*)D, 8, 64, v, 100, 128, (int32_t*)D, (int32_t*)D, nullptr), "union tpg");
      bad(sparse_mla_decode_grouped(D, D, 100, (const int32_t*)D, 8, 16, v, 64, 0.1f, D, (float*)D, 0, D,
                                    1 << 20, nullptr),
          "grouped tpg");
    }
  }
  // workspace missing or too small
  EXPECT(sparse_mla_decode(D, D, 100, (const int32_t*)D, 2, 16, 64, 0.1f, D, (float*)D, 0, nullptr, 0, nullptr) ==
             SMLA_ERR_WORKSPACE,
         "decode without workspace");
  EXPECT(sparse_mla_decode(D, D, 100, (const int32_t*)D, 2, 16, 64, 0.1f, D, (float*)D, 0, D, 8, nullptr) ==
             SMLA_ERR_WORKSPACE,
         "decode with a small workspace");
  // nothing to do
  EXPECT(sparse_mla_decode(nullptr, nullptr, 0, nullptr, 0, 16, 64, 0.1f, nullptr, nullptr, 0, nullptr, 0,
                           nullptr) == SMLA_OK,
         "decode of no token");
  EXPECT(nvfp4_pack_rows(nullptr, nullptr, 0, nullptr, 0, nullptr) == SMLA_OK, "pack of no row");
  printf("argument errors: %d calls\n", calls);
}

int main() {
  status_strings();
  size_queries();
  argument_errors();
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
