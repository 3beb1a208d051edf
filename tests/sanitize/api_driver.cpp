// Drives the host-side argument validation of the C ABI (csrc/gqa_attn_api.cpp) under the address
// and undefined-behaviour sanitizers (built and run by tests/test_sanitizers.py, on a machine
// without a GPU): every entry point with arguments that fail each check, the workspace queries
// over many shapes, and the status strings. Pointers are fake, 16-byte aligned, non-overlapping
// addresses: validation never dereferences them, and every call here is refused before anything
// is enqueued.
#include <stdint.h>
#include <stdio.h>

#include <limits>

#include "gqa_attn.h"

static int failures = 0;
#define EXPECT(call, code)                                                             \
  do {                                                                                 \
    const int got_ = static_cast<int>(call);                                           \
    if (got_ != (code)) {                                                              \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, \
              static_cast<int>(code));                                                 \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

static void* P(uintptr_t i) { return reinterpret_cast<void*>(i * 0x10000000ull); }

int main() {
  void *Q = P(1), *K = P(2), *V = P(3), *O = P(4), *W = P(5);
  const gqa_dtype_t BF = GQA_DTYPE_BF16, F32 = GQA_DTYPE_F32;
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();

  // prefill
  EXPECT(gqa_attn_prefill(nullptr, K, V, O, 1, 8, 8, 8, 2, 128, 0.1f, 0, nullptr, 0, BF, nullptr),
         GQA_ERR_NULL_PTR);
  EXPECT(gqa_attn_prefill(Q, K, V, O, 0, 8, 8, 8, 2, 128, 0.1f, 0, nullptr, 0, BF, nullptr),
         GQA_ERR_SHAPE);
  EXPECT(gqa_attn_prefill(Q, K, V, O, 1, 8, 8, 8, 3, 128, 0.1f, 0, nullptr, 0, BF, nullptr),
         GQA_ERR_GROUPING);
  EXPECT(gqa_attn_prefill(Q, K, V, O, 1, 8, 8, 8, 2, 96, 0.1f, 0, nullptr, 0, BF, nullptr),
         GQA_ERR_UNSUPPORTED);
  EXPECT(gqa_attn_prefill(Q, K, V, O, 1, 9, 8, 8, 2, 128, 0.1f, 1, nullptr, 0, BF, nullptr),
         GQA_ERR_SHAPE);
  for (float bad : {nan, inf, -0.5f})
    EXPECT(gqa_attn_prefill(Q, K, V, O, 1, 8, 8, 8, 2, 128, bad, 0, nullptr, 0, BF, nullptr),
           GQA_ERR_SHAPE);
  EXPECT(gqa_attn_prefill(Q, K, V, Q, 1, 8, 8, 8, 2, 128, GQA_SCALE_DEFAULT, 0, nullptr, 0, BF,
                          nullptr),
         GQA_ERR_ALIAS);
  EXPECT(gqa_attn_prefill(Q, K, V, O, 1, 8, 8, 8, 2, 128, 0.1f, 1,
                          static_cast<const int32_t*>(W), 0, BF, nullptr),
         GQA_ERR_SHAPE);  // packed without a longest length
  EXPECT(gqa_attn_prefill(Q, K, V, O, 70000, 8, 8, 8, 8, 16, 0.1f, 0, nullptr, 0, F32, nullptr),
         GQA_ERR_UNSUPPORTED);
  EXPECT(gqa_attn_prefill(Q, K, V, O, 1, 1 << 22, 1 << 22, 8, 8, 128, 0.1f, 0, nullptr, 0, BF,
                          nullptr),
         GQA_ERR_UNSUPPORTED);  // one item's keys beyond 32-bit offsets

  // options
  gqa_attn_options_t opt = {};
  opt.rope_cos = static_cast<const float*>(P(6));
  EXPECT(gqa_attn_prefill_ex(Q, K, V, O, 1, 8, 8, 8, 2, 128, 0.1f, 1, nullptr, 0, &opt, BF,
                             nullptr),
         GQA_ERR_NULL_PTR);
  opt = {};
  opt.window = 4;
  EXPECT(gqa_attn_prefill_ex(Q, K, V, O, 1, 8, 8, 8, 2, 128, 0.1f, 0, nullptr, 0, &opt, BF,
                             nullptr),
         GQA_ERR_SHAPE);  // windows are causal
  opt = {};
  opt.q_norm_w = static_cast<const float*>(P(7));
  opt.k_norm_w = static_cast<const float*>(P(8));
  opt.norm_eps = 0.f;
  EXPECT(gqa_attn_prefill_ex(Q, K, V, O, 1, 8, 8, 8, 2, 128, 0.1f, 1, nullptr, 0, &opt, BF,
                             nullptr),
         GQA_ERR_SHAPE);
  EXPECT(gqa_attn_prefill_window(Q, K, V, O, 1, 8, 8, 8, 2, 128, 0.1f, -1, 0, nullptr, 0, BF,
                                 nullptr),
         GQA_ERR_SHAPE);
  EXPECT(gqa_prepare_keys(K, O, 1, 8, 2, 128, nullptr, 0, 0, nullptr, BF, nullptr),
         GQA_ERR_NULL_PTR);
  EXPECT(gqa_attn_prefill_gva(Q, K, V, O, 1, 8, 8, 2, 7, 128, 0.1f, 1, nullptr, 0, nullptr, BF,
                              nullptr),
         GQA_ERR_GROUPING);

  // decode and its workspace queries
  for (int B : {1, 3, 64, 1000})
    for (int Tkv : {1, 31, 256, 8192, 131072})
      for (int Hq : {1, 7, 32, 64, 96})
        for (int d : {64, 128}) {
          const size_t bound = gqa_attn_decode_workspace_bytes(B, Tkv, Hq, d);
          size_t most = 0;
          for (int hkv = 1; hkv <= Hq; ++hkv) {
            const size_t e = gqa_attn_decode_workspace_bytes_hkv(B, Tkv, Hq, hkv, d);
            if (Hq % hkv != 0) {
              if (e != 0) ++failures;
              continue;
            }
            if (e == 0 || e > bound) ++failures;
            most = e > most ? e : most;
          }
          if (most != bound) ++failures;
        }
  EXPECT(gqa_attn_decode_workspace_bytes(-1, 8, 8, 128), 0);
  const size_t need = gqa_attn_decode_workspace_bytes_hkv(4, 1024, 32, 8, 128);
  EXPECT(gqa_attn_decode(Q, K, V, O, 4, 1024, 32, 8, 128, 0.1f, 0, nullptr, need, BF, nullptr),
         GQA_ERR_WORKSPACE);
  EXPECT(gqa_attn_decode(Q, K, V, O, 4, 1024, 32, 8, 128, 0.1f, 0, W, need - 1, BF, nullptr),
         GQA_ERR_WORKSPACE);
  EXPECT(gqa_attn_decode(Q, K, V, O, 4, 1024, 32, 5, 128, 0.1f, 0, W, need, BF, nullptr),
         GQA_ERR_GROUPING);
  EXPECT(gqa_attn_decode(Q, K, V, Q, 4, 1024, 32, 8, 128, 0.1f, 0, W, need, BF, nullptr),
         GQA_ERR_ALIAS);
  EXPECT(gqa_attn_decode_ragged(Q, K, V, O, 4, 1024, 32, 8, 128, 0.1f, nullptr, -3, 0, W, need, BF,
                                nullptr),
         GQA_ERR_SHAPE);
  {
    // decode against caches bounded to the window
    gqa_attn_options_t wo = {};
    wo.window = 64;
    wo.n_sink = 4;
    const int32_t* lens = static_cast<const int32_t*>(P(6));
    const size_t wneed = gqa_attn_decode_workspace_bytes_hkv(4, 68, 32, 8, 128);
    EXPECT(gqa_attn_decode_window_cache(Q, K, V, O, 4, 32, 8, 128, 0.1f, nullptr, &wo, W, wneed,
                                        BF, nullptr),
           GQA_ERR_NULL_PTR);
    EXPECT(gqa_attn_decode_window_cache(Q, K, V, O, 4, 32, 8, 128, 0.1f, lens, nullptr, W, wneed,
                                        BF, nullptr),
           GQA_ERR_NULL_PTR);
    EXPECT(gqa_attn_decode_window_cache(Q, K, V, O, 4, 32, 8, 128, 0.1f, lens, &wo, W, wneed - 1,
                                        BF, nullptr),
           GQA_ERR_WORKSPACE);
    EXPECT(gqa_attn_decode_window_cache(Q, K, V, O, 4, 32, 8, 16, 0.1f, lens, &wo, W, wneed, F32,
                                        nullptr),
           GQA_ERR_UNSUPPORTED);
    EXPECT(gqa_attn_decode_window_cache(Q, K, V, O, 4, 32, 5, 128, 0.1f, lens, &wo, W, wneed, BF,
                                        nullptr),
           GQA_ERR_GROUPING);
    wo.window = 0;
    EXPECT(gqa_attn_decode_window_cache(Q, K, V, O, 4, 32, 8, 128, 0.1f, lens, &wo, W, wneed, BF,
                                        nullptr),
           GQA_ERR_SHAPE);
    wo.window = std::numeric_limits<int>::max();
    EXPECT(gqa_attn_decode_window_cache(Q, K, V, O, 4, 32, 8, 128, 0.1f, lens, &wo, W, wneed, BF,
                                        nullptr),
           GQA_ERR_SHAPE);  // n_sink + window beyond int
    wo.window = 64;
    wo.n_sink = -1;
    EXPECT(gqa_attn_decode_window_cache(Q, K, V, O, 4, 32, 8, 128, 0.1f, lens, &wo, W, wneed, BF,
                                        nullptr),
           GQA_ERR_SHAPE);
  }
  EXPECT(gqa_attn_decode_noalloc(Q, K, V, O, 1024, 1, 32, 8, 128, 0.1f, 0, BF, nullptr),
         GQA_ERR_WORKSPACE);  // partials beyond the fixed scratch: refused first
  EXPECT(gqa_attn_decode_noalloc(nullptr, K, V, O, 4, 1024, 32, 8, 128, 0.1f, 0, F32, nullptr),
         GQA_ERR_NULL_PTR);

  // backward
  const size_t bw = gqa_attn_backward_workspace_bytes(2, 8, 8);
  if (bw < 2 * 8 * 8 * 4 || bw % 16) ++failures;
  EXPECT(gqa_attn_backward(Q, K, V, O, P(9), static_cast<const float*>(P(10)), P(11), P(12),
                           P(13), 2, 8, 8, 8, 3, 128, 0.1f, 0, W, bw, BF, nullptr),
         GQA_ERR_GROUPING);
  EXPECT(gqa_attn_backward(Q, K, V, O, P(9), static_cast<const float*>(P(10)), Q, P(12), P(13),
                           2, 8, 8, 8, 2, 128, 0.1f, 0, W, bw, BF, nullptr),
         GQA_ERR_ALIAS);

  // fold
  EXPECT(gqa_fold_kv(Q, O, 1, 4, 8, 3, 16, F32, nullptr), GQA_ERR_GROUPING);
  EXPECT(gqa_fold_kv(Q, O, 1, 4, 8, 2, 6, F32, nullptr), GQA_ERR_UNSUPPORTED);
  EXPECT(gqa_fold_kv(Q, static_cast<char*>(Q) + 16, 1, 4, 8, 2, 16, F32, nullptr),
         GQA_ERR_ALIAS);

  for (int s = 0; s <= 7; ++s)
    if (!gqa_status_string(static_cast<gqa_status_t>(s))[0]) ++failures;
  if (gqa_attn_abi_version() != GQA_ATTN_ABI_VERSION) ++failures;

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("api driver ok\n");
  return 0;
}
