/* Host-side checks of the C ABI, run against the library's sources built
 * with AddressSanitizer on the host side only (the device code is compiled as
 * usual but never launched, so no GPU is needed): every call below is refused
 * or answered by the host validation and sizing code before any kernel, so
 * ASan sees the whole host path of each entry point (argument checks,
 * workspace planning, error formatting).  Exits 0 and prints "ok" when every
 * status is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "hsa_attn.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, hsa_attn_last_error());
    ++failures;
  }
}

static hsa_attn_dims_t dims(int B, int Hq, int Hkv, int D, int S, int k, int64_t T, int dtype) {
  hsa_attn_dims_t d;
  memset(&d, 0, sizeof(d));
  d.batch = B;
  d.num_q_heads = Hq;
  d.num_kv_heads = Hkv;
  d.head_dim = D;
  d.chunk_size = S;
  d.top_k = k;
  d.seq_len = T;
  d.dtype = (hsa_attn_dtype_t)dtype;
  return d;
}

int main(void) {
  void* p = (void*)(uintptr_t)0x1000; /* aligned, never dereferenced on the host */
  void* mis = (void*)(uintptr_t)0x1004;
  float* pf = (float*)p;
  int32_t* pi = (int32_t*)p;
  int64_t* pl = (int64_t*)p;
  hsa_attn_dims_t d = dims(1, 32, 8, 128, 64, 16, 262144, HSA_ATTN_BF16);
  size_t bytes = 0;
  int64_t rows = 0;
  int kind;

  /* sizes of every call kind, and the slab planning they imply */
  for (kind = 0; kind <= 4; ++kind) {
    hsa_attn_dims_t dk = dims(2, 32, 8, 128, 64, kind == 4 ? 16 : 32, 64 * 1000 + 17, HSA_ATTN_BF16);
    bytes = 0;
    expect(hsa_attn_workspace_size(&dk, kind, &bytes), HSA_ATTN_OK, "workspace size");
    if (bytes == 0 || bytes % 256 != 0) {
      fprintf(stderr, "workspace size %zu for kind %d\n", bytes, kind);
      ++failures;
    }
  }
  expect(hsa_attn_workspace_size(&d, 5, &bytes), HSA_ATTN_INVALID_ARGUMENT, "unknown kind");
  expect(hsa_attn_workspace_size(NULL, 0, &bytes), HSA_ATTN_INVALID_ARGUMENT, "NULL dims");
  expect(hsa_attn_workspace_size(&d, 0, NULL), HSA_ATTN_INVALID_ARGUMENT, "NULL bytes");
  expect(hsa_attn_prefill_slab_rows(&d, 0, 0, (size_t)16 << 30, &rows), HSA_ATTN_OK, "slab rows");
  if (rows <= 0 || rows % 64 != 0) {
    fprintf(stderr, "slab rows %lld\n", (long long)rows);
    ++failures;
  }
  expect(hsa_attn_prefill_slab_rows(&d, 0, 0, 1024, &rows), HSA_ATTN_OK, "slab rows, tiny workspace");
  if (rows != 0) ++failures;

  /* dimension checks */
  {
    hsa_attn_dims_t bad = dims(1, 6, 4, 128, 64, 16, 4096, HSA_ATTN_BF16); /* Hq % Hkv != 0 */
    expect(hsa_forward_prefill(&bad, p, p, p, p, pf, NULL, NULL, p, 1 << 30, NULL), HSA_ATTN_INVALID_ARGUMENT,
           "Hq % Hkv");
    bad = dims(1, 32, 8, 96, 64, 16, 4096, HSA_ATTN_BF16);
    expect(hsa_forward_decode(&bad, p, p, p, p, pf, NULL, NULL, p, 1 << 30, NULL), HSA_ATTN_UNSUPPORTED, "D = 96");
    bad = dims(1, 32, 8, 128, 64, 65, 4096, HSA_ATTN_BF16);
    expect(hsa_forward_prefill(&bad, p, p, p, p, pf, NULL, NULL, p, 1 << 30, NULL), HSA_ATTN_UNSUPPORTED, "k = 65");
    bad = dims(1, 32, 8, 128, 64, 16, -1, HSA_ATTN_BF16);
    expect(hsa_forward_decode(&bad, p, p, p, p, pf, NULL, NULL, p, 1 << 30, NULL), HSA_ATTN_INVALID_ARGUMENT,
           "negative seq_len");
    bad = dims(1, 32, 8, 128, 64, 16, 4096, 7);
    expect(hsa_forward_prefill(&bad, p, p, p, p, pf, NULL, NULL, p, 1 << 30, NULL), HSA_ATTN_INVALID_ARGUMENT,
           "dtype");
  }

  /* pointers: NULL, misaligned, one selection output, ranges */
  expect(hsa_forward_prefill(&d, NULL, p, p, p, pf, NULL, NULL, p, (size_t)1 << 40, NULL), HSA_ATTN_INVALID_ARGUMENT,
         "NULL q");
  expect(hsa_forward_prefill(&d, mis, p, p, p, pf, NULL, NULL, p, (size_t)1 << 40, NULL), HSA_ATTN_INVALID_ARGUMENT,
         "misaligned q");
  expect(hsa_forward_prefill(&d, p, p, p, p, pf, pi, NULL, p, (size_t)1 << 40, NULL), HSA_ATTN_INVALID_ARGUMENT,
         "one selection output");
  expect(hsa_forward_prefill_cached(&d, 65, p, p, p, p, pf, NULL, NULL, p, (size_t)1 << 40, NULL),
         HSA_ATTN_INVALID_ARGUMENT, "q_offset not a multiple of S");
  expect(hsa_forward_prefill_adaptive(&d, -1.0f, p, p, p, p, pf, NULL, NULL, p, (size_t)1 << 40, NULL),
         HSA_ATTN_INVALID_ARGUMENT, "negative gap threshold");
  expect(hsa_build_landmarks(&d, p, p, 3, 2, NULL), HSA_ATTN_INVALID_ARGUMENT, "reversed chunk range");
  expect(hsa_build_landmarks(&d, p, p, 0, 4097, NULL), HSA_ATTN_INVALID_ARGUMENT, "chunk range past Nc");
  expect(hsa_build_landmarks(&d, NULL, NULL, 5, 5, NULL), HSA_ATTN_OK, "empty chunk range");
  {
    /* empty work: OK before any pointer is looked at */
    hsa_attn_dims_t e = d;
    e.seq_len = 0;
    expect(hsa_forward_prefill(&e, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), HSA_ATTN_OK,
           "prefill over no tokens");
    expect(hsa_forward_prefill_adaptive(&e, 0.5f, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL),
           HSA_ATTN_OK, "adaptive prefill over no tokens");
    expect(hsa_backward_prefill(&e, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL),
           HSA_ATTN_OK, "backward over no tokens");
    expect(hsa_forward_prefill_cached(&d, d.seq_len, NULL, p, p, p, NULL, NULL, NULL, NULL, 0, NULL), HSA_ATTN_OK,
           "cached prefill with no new rows");
    size_t eb = 0;
    expect(hsa_attn_workspace_size(&e, 0, &eb), HSA_ATTN_OK, "workspace size, no tokens");
    if (eb > ((size_t)1 << 30)) {
      fprintf(stderr, "empty prefill plans %zu workspace bytes\n", eb);
      ++failures;
    }
  }
  expect(hsa_forward_decode_varlen(&d, p, p, p, p, NULL, pf, NULL, NULL, p, (size_t)1 << 40, NULL),
         HSA_ATTN_INVALID_ARGUMENT, "NULL cache_lens");
  expect(hsa_append_kv(&d, p, p, p, p, p, (int64_t*)(uintptr_t)0x1004, NULL), HSA_ATTN_INVALID_ARGUMENT,
         "misaligned cache_lens");
  expect(hsa_backward_prefill(&d, p, p, p, p, pf, pf, pi, NULL, pf, pf, pf, p, (size_t)1 << 40, NULL),
         HSA_ATTN_INVALID_ARGUMENT, "backward without sel_score");

  /* workspaces too small: refused with the size that is needed */
  expect(hsa_forward_prefill(&d, p, p, p, p, pf, NULL, NULL, p, 4096, NULL), HSA_ATTN_WORKSPACE_TOO_SMALL,
         "small prefill workspace");
  if (!strstr(hsa_attn_last_error(), "workspace")) ++failures;
  expect(hsa_forward_decode(&d, p, p, p, p, pf, NULL, NULL, p, 64, NULL), HSA_ATTN_WORKSPACE_TOO_SMALL,
         "small decode workspace");
  expect(hsa_backward_prefill(&d, p, p, p, p, pf, pf, pi, pf, pf, pf, pf, p, 64, NULL), HSA_ATTN_WORKSPACE_TOO_SMALL,
         "small backward workspace");
  {
    hsa_attn_dims_t big = dims(64, 32, 8, 128, 64, 64, (int64_t)1 << 22, HSA_ATTN_BF16);
    expect(hsa_forward_decode_noalloc(&big, p, p, p, p, pf, NULL, NULL, NULL), HSA_ATTN_WORKSPACE_TOO_SMALL,
           "no-allocation decode beyond its scratch");
  }

  /* timing events, status strings, the debug-only call */
  expect(hsa_attn_set_timing_events(NULL, 1), HSA_ATTN_INVALID_ARGUMENT, "events NULL");
  expect(hsa_attn_set_timing_events(NULL, 0), HSA_ATTN_OK, "events off");
  for (kind = 0; kind <= 5; ++kind)
    if (!hsa_attn_status_string((hsa_attn_status_t)kind) || !*hsa_attn_status_string((hsa_attn_status_t)kind))
      ++failures;
  {
    uint32_t flags = 0;
    expect(hsa_attn_debug_flags(NULL, &flags), HSA_ATTN_UNSUPPORTED, "debug flags in the release build");
  }
  (void)pl;
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
