// Calls the C ABI of libhils.so built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code (tests/test_sanitize.py): workspace sizes for a sweep of shapes and
// every validation path of every entry point with arguments it must reject, so nothing
// reaches the device (no GPU is needed).  Any out-of-bounds access or undefined operation
// in the host code aborts the run; every call must return its documented error code.
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "../../include/hils.h"

static int g_fail = 0;
#define EXPECT(cond)                                            \
  do {                                                          \
    if (!(cond)) {                                              \
      printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, hils_last_error()); \
      g_fail = 1;                                               \
    }                                                           \
  } while (0)

static hils_dims_t dims(int B, int Hq, int Hkv, int Hl, int d, int N, int K, int r, int io, int W) {
  hils_dims_t x = {B, Hq, Hkv, Hl, d, 64, K, N, r, io, W};
  return x;
}

int main() {
  void* f = (void*)0x1000;  // never dereferenced: validation fails first
  // workspace sizes over a sweep of shapes, valid and invalid
  const int Ns[] = {1, 63, 64, 65, 1000, 4096, 262144, 524288, 1 << 20, 1 << 21};
  const int Ks[] = {0, 1, 16, 32, 33};
  for (int n : Ns)
    for (int k : Ks)
      for (int op = -1; op <= 5; ++op)
        for (int W : {0, 64, 512, 2048, 4096}) {
          hils_dims_t d = dims(2, 16, 4, 16, 128, n, k, 8, HILS_BF16, W);
          (void)hils_workspace_bytes(&d, op);
          d.Hlmk = 4;
          (void)hils_workspace_bytes(&d, op);
        }
  EXPECT(hils_workspace_bytes(nullptr, HILS_OP_PREFILL) == (size_t)-1);
  hils_dims_t ok = dims(1, 4, 2, 4, 64, 1024, 8, 0, HILS_BF16, 0);
  hils_dims_t bad = ok;
  bad.d = 96;
  EXPECT(hils_landmark_compress(&bad, f, f, 0, 1, (float*)f, (float*)f, nullptr) == HILS_E_UNSUPPORTED);
  EXPECT(hils_landmark_compress(&ok, f, f, 3, 2, (float*)f, (float*)f, nullptr) == HILS_E_INVAL);
  EXPECT(hils_landmark_compress(&ok, nullptr, f, 0, 1, (float*)f, (float*)f, nullptr) == HILS_E_INVAL);
  EXPECT(hils_landmark_compress(&ok, nullptr, nullptr, 2, 2, nullptr, nullptr, nullptr) == HILS_OK);
  EXPECT(hils_chunk_score_topk(&ok, 1025, f, nullptr, nullptr, nullptr, (float*)f, (float*)f, (int32_t*)f, (float*)f,
                               f, 1u << 30, nullptr) == HILS_E_INVAL);
  EXPECT(hils_chunk_score_topk(&ok, 10, f, nullptr, nullptr, nullptr, (float*)f, (float*)f, (int32_t*)f, (float*)f,
                               f, 1, nullptr) == HILS_E_WORKSPACE);
  EXPECT(hils_attn_prefill(&ok, f, f, f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, f, f,
                           (size_t)1 << 40, nullptr) == HILS_E_INVAL);
  EXPECT(hils_attn_prefill(&ok, f, f, f, f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, f, f, 16,
                           nullptr) == HILS_E_WORKSPACE);
  float stages[HILS_PREFILL_STAGES];
  EXPECT(hils_attn_prefill_timed(&bad, f, f, f, f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, f, f, 16,
                                 nullptr, stages) == HILS_E_UNSUPPORTED);
  EXPECT(hils_attn_decode(&ok, f, f, f, nullptr, (float*)f, (float*)f, nullptr, nullptr, nullptr, f, f, 1u << 30,
                          nullptr) == HILS_E_INVAL);
  EXPECT(hils_attn_decode(&ok, f, f, f, (int32_t*)f, (float*)f, (float*)f, nullptr, nullptr, nullptr, f, f, 1,
                          nullptr) == HILS_E_WORKSPACE);
  hils_dims_t big = dims(64, 64, 8, 64, 128, 1 << 20, 32, 0, HILS_BF16, 0);
  EXPECT(hils_attn_decode_noalloc(&big, f, f, f, (int32_t*)f, (float*)f, (float*)f, nullptr, nullptr, nullptr, f,
                                  nullptr) == HILS_E_UNSUPPORTED);
  EXPECT(hils_landmark_compress_paged(&ok, f, (int32_t*)f, 15, 40, f, 0, 1, (float*)f, (float*)f, nullptr) ==
         HILS_E_INVAL);
  EXPECT(hils_attn_decode_paged(&ok, f, f, f, nullptr, 16, 40, (int32_t*)f, (float*)f, (float*)f, nullptr, nullptr,
                                nullptr, f, f, 1u << 30, nullptr) == HILS_E_INVAL);
  EXPECT(hils_dense_attention(&bad, f, f, f, f, nullptr) == HILS_E_UNSUPPORTED);
  hils_dims_t f32 = ok;
  f32.io = HILS_F32;
  EXPECT(hils_attn_prefill_backward(&f32, f, f, f, f, (float*)f, nullptr, nullptr, (int32_t*)f, (float*)f, f, f, f, f,
                                    f, f, nullptr, nullptr, f, (size_t)1 << 40, nullptr) == HILS_E_UNSUPPORTED);
  hils_dims_t shared = ok;  // landmark heads shared by query heads: valid, stopped at the workspace check
  shared.Hlmk = 2;
  EXPECT(hils_attn_prefill_backward(&shared, f, f, f, f, (float*)f, nullptr, nullptr, (int32_t*)f, (float*)f, f, f, f,
                                    f, f, f, nullptr, nullptr, nullptr, 0, nullptr) == HILS_E_WORKSPACE);
  EXPECT(hils_last_error()[0] != 0);
  // the dense decode baseline: bf16 and Hq/Hkv in {1, 2, 4, 8}, a workspace of the reported size
  const size_t dd = hils_workspace_bytes(&ok, HILS_OP_DENSE_DECODE);
  EXPECT(dd != (size_t)-1 && dd > 0);
  EXPECT(hils_dense_decode(&ok, f, f, f, (const int32_t*)f, f, nullptr, 0, nullptr) == HILS_E_WORKSPACE);
  EXPECT(hils_dense_decode(&ok, nullptr, f, f, (const int32_t*)f, f, f, dd, nullptr) == HILS_E_INVAL);
  EXPECT(hils_dense_decode(&f32, f, f, f, (const int32_t*)f, f, f, (size_t)1 << 40, nullptr) == HILS_E_UNSUPPORTED);
  if (!g_fail) printf("host ABI sanitizer run: ok\n");
  return g_fail;
}
