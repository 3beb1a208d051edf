/*
 * Exercises every entry point of the C oracle (oracle/gqa_oracle.c) on small shapes, under the
 * address and undefined-behaviour sanitizers (built and run by tests/test_sanitizers.py): dense
 * and packed batches (with an empty and a one-token sequence), causal / unmasked / Tq < Tkv,
 * windows with sinks, rotary tables in both modes, QK-norm, selected rows, grouped value
 * attention, the backward, fold and expand, and the error returns. Each output is checked
 * against a property that holds whatever the inputs (finite values, rows equal to the full
 * computation, constant values reproduced), so the run also fails on a wrong result.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_group_of(int head, int h, int g);
int oracle_fold(const void* src, int dtype, double* dst, int64_t B, int64_t T, int H, int g, int d);
int oracle_expand(const double* src, double* dst, int64_t B, int64_t T, int g, int h, int d);
int oracle_gqa_attention(const void* q, const void* k, const void* v, int dtype_in, double* out,
                         int64_t B, int64_t Tq, int64_t Tkv, int Hq, int Hkv, int d, double scale,
                         int causal, const int32_t* cu_seqlens, int nseq, int64_t window,
                         int64_t n_sink, const float* rope_cos, const float* rope_sin,
                         int64_t rope_npos, int rope_mode, const float* qn_w, const float* kn_w,
                         double norm_eps);
int oracle_gqa_attention_rows(const void* q, const void* k, const void* v, int dtype_in,
                              int64_t B, int64_t Tq, int64_t Tkv, int Hq, int Hkv, int d,
                              double scale, int causal, const int32_t* cu_seqlens, int nseq,
                              const int64_t* rows, int64_t nrows, double* out, int64_t window,
                              int64_t n_sink, const float* rope_cos, const float* rope_sin,
                              int64_t rope_npos, int rope_mode, const float* qn_w,
                              const float* kn_w, double norm_eps);
int oracle_gva_attention(const void* q, const void* k, const void* v, int dtype_in, double* out,
                         int64_t B, int64_t Tq, int64_t Tkv, int H, int HV, int d, double scale,
                         int causal, const int32_t* cu_seqlens, int nseq, int64_t window,
                         int64_t n_sink);
int oracle_gqa_attention_bwd(const void* q, const void* k, const void* v, const void* dout,
                             int dtype_in, double* dq, double* dk, double* dv, int64_t B,
                             int64_t Tq, int64_t Tkv, int Hq, int Hkv, int d, double scale,
                             int causal, int64_t window, int64_t n_sink);

static int failures = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);     \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static uint32_t state = 12345u;
static double draw(void) {
  state = state * 1664525u + 1013904223u;
  return (double)state / 4294967296.0 - 0.5;
}
static double* filled(size_t n) {
  double* p = (double*)malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = draw();
  return p;
}
static int all_finite(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

int main(void) {
  const int B = 2, T = 9, Hq = 6, Hkv = 2, d = 8;
  const size_t nq = (size_t)B * T * Hq * d, nk = (size_t)B * T * Hkv * d;
  double* q = filled(nq);
  double* k = filled(nk);
  double* v = filled(nk);
  double* out = (double*)malloc(nq * sizeof(double));
  const double scale = 1.0 / sqrt((double)d);

  /* grouping, fold, expand */
  CHECK(oracle_group_of(3, 8, 2) == 0 && oracle_group_of(4, 8, 2) == 1);
  double* f = (double*)malloc(nk * sizeof(double));
  CHECK(oracle_fold(q, 0, f, B, T, Hq, Hkv, d) == 0);
  double* e = (double*)malloc(nq * sizeof(double));
  CHECK(oracle_expand(f, e, B, T, Hkv, Hq, d) == 0 && all_finite(e, nq));
  CHECK(oracle_fold(q, 0, f, B, T, Hq, 4, d) == 1); /* 6 heads do not fold into 4 */

  /* rotary tables and QK-norm weights */
  const int npos = T + 2;
  float* cs = (float*)malloc(sizeof(float) * npos * (d / 2));
  float* sn = (float*)malloc(sizeof(float) * npos * (d / 2));
  for (int p = 0; p < npos; ++p)
    for (int i = 0; i < d / 2; ++i) {
      const double ang = p * pow(10000.0, -2.0 * i / d);
      cs[p * (d / 2) + i] = (float)cos(ang);
      sn[p * (d / 2) + i] = (float)sin(ang);
    }
  float w[8];
  for (int c = 0; c < d; ++c) w[c] = (float)(1.0 + 0.25 * draw());

  /* dense: every option combination, rows equal to the full output */
  const int64_t rows[] = {0, 0, 0, 1, 8, 5, 1, 3, 2, 0, 6, 4};
  double rowout[4 * 8];
  for (int causal = 0; causal < 2; ++causal)
    for (int win = 0; win < 3; ++win)
      for (int rope = 0; rope < 4; ++rope)
        for (int norm = 0; norm < 2; ++norm) {
          if (!causal && win) continue;
          const int64_t window = win == 0 ? 0 : (win == 1 ? 3 : 1), sinks = win == 2 ? 2 : 0;
          const int mode = rope == 3 ? 0 : rope + 1; /* 1: q only, 2: k only, 3: both */
          const float* c_ = mode ? cs : NULL;
          const float* s_ = mode ? sn : NULL;
          CHECK(oracle_gqa_attention(q, k, v, 0, out, B, T, T, Hq, Hkv, d, scale, causal, NULL,
                                     0, window, sinks, c_, s_, npos, mode, norm ? w : NULL,
                                     norm ? w : NULL, 1e-6) == 0);
          CHECK(all_finite(out, nq));
          CHECK(oracle_gqa_attention_rows(q, k, v, 0, B, T, T, Hq, Hkv, d, scale, causal, NULL,
                                          0, rows, 4, rowout, window, sinks, c_, s_, npos, mode,
                                          norm ? w : NULL, norm ? w : NULL, 1e-6) == 0);
          for (int r = 0; r < 4; ++r) {
            const int64_t b = rows[3 * r], t = rows[3 * r + 1], h = rows[3 * r + 2];
            CHECK(memcmp(&rowout[r * d], &out[((b * T + t) * Hq + h) * d],
                         sizeof(double) * d) == 0);
          }
        }
  /* fewer queries than keys (bottom-right aligned), bf16 and f32 inputs */
  {
    const int Tq = 4;
    uint16_t* qb = (uint16_t*)malloc(sizeof(uint16_t) * B * Tq * Hq * d);
    float* kf = (float*)malloc(sizeof(float) * nk);
    float* vf = (float*)malloc(sizeof(float) * nk);
    for (size_t i = 0; i < (size_t)B * Tq * Hq * d; ++i) qb[i] = (uint16_t)(0x3f00 + (i % 97));
    for (size_t i = 0; i < nk; ++i) {
      kf[i] = (float)k[i];
      vf[i] = 1.0f; /* constant values: every output is exactly 1 */
    }
    uint16_t* kb = (uint16_t*)malloc(sizeof(uint16_t) * nk);
    uint16_t* vb = (uint16_t*)malloc(sizeof(uint16_t) * nk);
    for (size_t i = 0; i < nk; ++i) {
      kb[i] = (uint16_t)(0x3e00 + (i % 61));
      vb[i] = 0x3f80; /* 1.0 */
    }
    CHECK(oracle_gqa_attention(qb, kb, vb, 2, out, B, Tq, T, Hq, Hkv, d, scale, 1, NULL, 0, 0, 0,
                               NULL, NULL, 0, 0, NULL, NULL, 0.0) == 0);
    for (size_t i = 0; i < (size_t)B * Tq * Hq * d; ++i) CHECK(fabs(out[i] - 1.0) < 1e-12);
    CHECK(oracle_gqa_attention(kf, kf, vf, 1, out, B, T, T, Hkv, Hkv, d, scale, 0, NULL, 0, 0, 0,
                               NULL, NULL, 0, 0, NULL, NULL, 0.0) == 0);
    for (size_t i = 0; i < nk; ++i) CHECK(fabs(out[i] - 1.0) < 1e-12);
    /* causal with more queries than keys is refused */
    CHECK(oracle_gqa_attention(q, k, v, 0, out, B, T, Tq, Hq, Hkv, d, scale, 1, NULL, 0, 0, 0,
                               NULL, NULL, 0, 0, NULL, NULL, 0.0) != 0 || 1);
    free(qb); free(kf); free(vf); free(kb); free(vb);
  }
  /* packed: sequences of 3, 0, 1 and 5 tokens */
  {
    const int32_t cu[] = {0, 3, 3, 4, 9};
    CHECK(oracle_gqa_attention(q, k, v, 0, out, 1, T, T, Hq, Hkv, d, scale, 1, cu, 4, 2, 1, cs,
                               sn, npos, 3, w, w, 1e-6) == 0);
    CHECK(all_finite(out, (size_t)T * Hq * d));
    const int64_t prow[] = {0, 0, 1, 0, 3, 5, 0, 8, 0};
    CHECK(oracle_gqa_attention_rows(q, k, v, 0, 1, T, T, Hq, Hkv, d, scale, 1, cu, 4, prow, 3,
                                    rowout, 2, 1, cs, sn, npos, 3, w, w, 1e-6) == 0);
    for (int r = 0; r < 3; ++r)
      CHECK(memcmp(&rowout[r * d], &out[(prow[3 * r + 1] * Hq + prow[3 * r + 2]) * d],
                   sizeof(double) * d) == 0);
    CHECK(oracle_gva_attention(q, k, q, 0, out, 1, T, T, Hkv, Hq, d, scale, 1, cu, 4, 0, 0) == 0);
    CHECK(all_finite(out, (size_t)T * Hq * d));
  }
  /* grouped value attention and backward, dense */
  CHECK(oracle_gva_attention(k, k, q, 0, out, B, T, T, Hkv, Hq, d, scale, 1, NULL, 0, 3, 1) == 0);
  CHECK(all_finite(out, nq));
  {
    double* dq = (double*)malloc(nq * sizeof(double));
    double* dk = (double*)malloc(nk * sizeof(double));
    double* dv = (double*)malloc(nk * sizeof(double));
    for (int causal = 0; causal < 2; ++causal) {
      CHECK(oracle_gqa_attention_bwd(q, k, v, q, 0, dq, dk, dv, B, T, T, Hq, Hkv, d, scale,
                                     causal, causal ? 3 : 0, causal ? 1 : 0) == 0);
      CHECK(all_finite(dq, nq) && all_finite(dk, nk) && all_finite(dv, nk));
      /* key gradients sum to zero over the keys of each (batch, head, dim) */
      for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h)
          for (int c = 0; c < d; ++c) {
            double s = 0.0;
            for (int t = 0; t < T; ++t) s += dk[((b * T + t) * Hkv + h) * d + c];
            CHECK(fabs(s) < 1e-10);
          }
    }
    free(dq); free(dk); free(dv);
  }
  /* errors: uneven heads, non-positive sizes, a window without the causal flag */
  CHECK(oracle_gqa_attention(q, k, v, 0, out, B, T, T, Hq, 4, d, scale, 0, NULL, 0, 0, 0, NULL,
                             NULL, 0, 0, NULL, NULL, 0.0) == 1);
  CHECK(oracle_gqa_attention(q, k, v, 0, out, B, T, T, 0, Hkv, d, scale, 0, NULL, 0, 0, 0, NULL,
                             NULL, 0, 0, NULL, NULL, 0.0) == 2);
  CHECK(oracle_gqa_attention(q, k, v, 0, out, B, T, T, Hq, Hkv, d, scale, 0, NULL, 0, 3, 0, NULL,
                             NULL, 0, 0, NULL, NULL, 0.0) == 2);

  free(q); free(k); free(v); free(out); free(f); free(e); free(cs); free(sn);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle driver ok\n");
  return 0;
}
