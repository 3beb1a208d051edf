/*
 * gqa_oracle.c -- plain, slow, fp64 CPU oracle for grouped-query attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU-baseline leg are
 * its only users; the product path (the HIP library) never links, loads or calls it, and this file
 * includes nothing from that library.
 *
 * What it computes follows the pages' own definitions, written out directly:
 *   - grouping: query head i belongs to group i / (h / g), the contiguous rule of the GQA lab page
 *     ("Transformer -- attention by hand: reducing only the key/value heads", step 1 note
 *     "split the query heads into groups"); a head count that does not divide is an error;
 *   - fold: position-wise mean of the key/value heads inside each contiguous group (lab step 2);
 *   - expand: adjacent repetition of the folded heads back to h heads, [A,B] -> [A,A,B,B]
 *     (lab step 3), materialised as a copy;
 *   - attend: for every query row, dot with every visible key row, multiply by the scale
 *     (1/sqrt(head dim), lab step 4 and the course page "Week 7. Attention", step 1), subtract the
 *     row maximum, exponentiate, normalise, and take the weighted average of the value rows;
 *   - causal mask: keys after the query's position are excluded before the softmax (course page,
 *     step 1: -inf before softmax). Alignment when Tq < Tkv is bottom-right: query t sits at
 *     position t + (Tkv - Tq). The pages only show the square case; this is the plainest reading
 *     that keeps the square case and makes a one-token decode see the whole cache.
 *   - heads_out: fold and expand K, fold and expand V, then one attend per query head (lab step 5).
 *
 * Everything is computed in double precision. Inputs may be fp64, fp32 or bf16 bit patterns;
 * widening any of them to double is exact. Two-pass softmax: first the maximum, then the
 * exponentials and their sum; dot products are summed sequentially in index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };

/* rotary embedding modes: which of q and k are rotated */
enum { ROPE_Q = 1, ROPE_K = 2 };

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_GROUPING = 1, /* head count not divisible by the group count */
  ORACLE_ERR_SHAPE = 2,    /* non-positive sizes, bad index, causal rows with no visible key */
  ORACLE_ERR_ALLOC = 3
};

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Exact widening of one element to double. */
static double widen(const void* base, int dtype, int64_t idx) {
  if (dtype == ORACLE_F64) return ((const double*)base)[idx];
  if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Group index of query head `head` when h heads are split into g contiguous groups.
 * Returns -1 when h is not divisible by g or the arguments are out of range. */
int oracle_group_of(int head, int h, int g) {
  if (h <= 0 || g <= 0 || h % g != 0 || head < 0 || head >= h) return -1;
  return head / (h / g);
}

/* fold: src[B,T,H,d] (any input dtype) -> dst[B,T,g,d] fp64.
 * dst[b,t,j,:] = (sum over the s = H/g heads j*s .. j*s+s-1 of src[b,t,head,:]) / s. */
int oracle_fold(const void* src, int dtype, double* dst, int64_t B, int64_t T, int H, int g,
                int d) {
  if (B <= 0 || T <= 0 || H <= 0 || g <= 0 || d <= 0) return ORACLE_ERR_SHAPE;
  if (H % g != 0) return ORACLE_ERR_GROUPING;
  const int s = H / g;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t = 0; t < T; ++t)
      for (int j = 0; j < g; ++j) {
        const int start = j * s;
        for (int c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int i = 0; i < s; ++i)
            acc += widen(src, dtype, ((b * T + t) * H + (start + i)) * (int64_t)d + c);
          dst[((b * T + t) * g + j) * (int64_t)d + c] = acc / (double)s;
        }
      }
  return ORACLE_OK;
}

/* expand: src[B,T,g,d] fp64 -> dst[B,T,h,d] fp64 by adjacent repetition: the outer loop runs
 * over the folded heads, the inner loop repeats each one h/g times, so [A,B] -> [A,A,B,B]. */
int oracle_expand(const double* src, double* dst, int64_t B, int64_t T, int g, int h, int d) {
  if (B <= 0 || T <= 0 || h <= 0 || g <= 0 || d <= 0) return ORACLE_ERR_SHAPE;
  if (h % g != 0) return ORACLE_ERR_GROUPING;
  const int rep = h / g;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t = 0; t < T; ++t) {
      int out_head = 0;
      for (int j = 0; j < g; ++j)
        for (int r = 0; r < rep; ++r) {
          memcpy(&dst[((b * T + t) * h + out_head) * (int64_t)d],
                 &src[((b * T + t) * g + j) * (int64_t)d], sizeof(double) * (size_t)d);
          ++out_head;
        }
    }
  return ORACLE_OK;
}

/* One output row of single-head attention.
 * q: d values; key j's row starts at k + j*kstride (likewise v); out: d values.
 * Keys 0 .. nvis-1 are candidates; candidate j is visible unless lo <= j is false and j is not
 * a sink (j >= n_sink), i.e. visible iff j >= lo or j < n_sink (lo = 0: every candidate).
 * Scores s_j = scale * sum_c q[c] k[j][c]; two-pass softmax over the visible keys;
 * out = sum_j p_j v_j / sum_j p_j. A row that sees no key is defined as zeros. */
static void attend_row(const double* q, const double* k, const double* v, int64_t kstride,
                       int64_t nvis, int64_t lo, int64_t n_sink, int d, double scale, double* s,
                       double* out) {
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  double m = -INFINITY;
  int64_t seen = 0;
  for (int64_t j = 0; j < nvis; ++j) {
    if (j < lo && j >= n_sink) continue;
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += q[c] * k[j * kstride + c];
    s[j] = scale * dot;
    if (s[j] > m) m = s[j];
    ++seen;
  }
  if (seen == 0) return;
  double l = 0.0;
  for (int64_t j = 0; j < nvis; ++j) {
    if (j < lo && j >= n_sink) continue;
    const double p = exp(s[j] - m);
    s[j] = p;
    l += p;
  }
  for (int64_t j = 0; j < nvis; ++j) {
    if (j < lo && j >= n_sink) continue;
    for (int c = 0; c < d; ++c) out[c] += s[j] * v[j * kstride + c];
  }
  for (int c = 0; c < d; ++c) out[c] /= l;
}

/* First key of the sliding window of query t (bottom-right aligned): with a window of W keys
 * the query at position p = t + (Tkv - Tq) sees keys p - W + 1 .. p, plus the sink keys
 * 0 .. n_sink-1 (course page "Week 7. Attention", step 3: sliding window and attention sinks).
 * window <= 0 means no window (returns 0). */
static int64_t window_lo(int64_t t, int64_t Tq, int64_t Tkv, int64_t window) {
  if (window <= 0) return 0;
  return t + (Tkv - Tq) - window + 1;
}

/* Number of keys query t of a (Tq, Tkv) item sees. */
static int64_t visible_keys(int64_t t, int64_t Tq, int64_t Tkv, int causal) {
  if (!causal) return Tkv;
  int64_t n = t + (Tkv - Tq) + 1;
  if (n < 0) n = 0;
  if (n > Tkv) n = Tkv;
  return n;
}

/* Rotary position embedding of one head row in place (course page "Week 7. Attention", step 3:
 * each pair of coordinates is turned by the angle pos * theta_i; in complex form the pair
 * (x[2i], x[2i+1]) is the number x[2i] + i x[2i+1] multiplied by e^{i pos theta_i}).
 * cos_t / sin_t: tables [n_pos][d/2] (fp32, as the caller passes them) holding cos and sin of
 * pos * theta_i. */
static void rope_row(double* x, int d, const float* cos_t, const float* sin_t, int64_t pos) {
  for (int i = 0; i < d / 2; ++i) {
    const double c = (double)cos_t[pos * (d / 2) + i];
    const double s = (double)sin_t[pos * (d / 2) + i];
    const double re = x[2 * i], im = x[2 * i + 1];
    x[2 * i] = re * c - im * s;
    x[2 * i + 1] = re * s + im * c;
  }
}

/* QK-norm of one head row in place (course page "Week 7. Attention", step 3: RMSNorm applied to
 * q and k before the dot product): x * w / sqrt(mean(x^2) + eps), the mean over the d
 * coordinates of the row, w the caller's per-coordinate weights (fp32 [d]). */
static void rms_row(double* x, int d, const float* w, double eps) {
  double ss = 0.0;
  for (int c = 0; c < d; ++c) ss += x[c] * x[c];
  const double inv = 1.0 / sqrt(ss / d + eps);
  for (int c = 0; c < d; ++c) x[c] = x[c] * inv * (double)w[c];
}

/* Item table: a dense batch has B items of (Tq, Tkv); a packed batch (cu_seqlens) has nseq items
 * of equal query and key length, laid out back to back in a single [1, total, H, d] tensor. */
typedef struct {
  int64_t q_row0, k_row0; /* first row of the item in the [rows, H, d] view */
  int64_t Tq, Tkv;
} item_t;

static int make_items(int64_t B, int64_t Tq, int64_t Tkv, const int32_t* cu, int nseq,
                      item_t** items, int* nitems) {
  if (cu) {
    if (nseq <= 0 || cu[0] != 0) return ORACLE_ERR_SHAPE;
    *items = (item_t*)malloc(sizeof(item_t) * (size_t)nseq);
    if (!*items) return ORACLE_ERR_ALLOC;
    for (int s = 0; s < nseq; ++s) {
      const int64_t len = (int64_t)cu[s + 1] - cu[s];
      if (len < 0) { free(*items); return ORACLE_ERR_SHAPE; }
      (*items)[s].q_row0 = cu[s];
      (*items)[s].k_row0 = cu[s];
      (*items)[s].Tq = len;
      (*items)[s].Tkv = len;
    }
    *nitems = nseq;
  } else {
    *items = (item_t*)malloc(sizeof(item_t) * (size_t)B);
    if (!*items) return ORACLE_ERR_ALLOC;
    for (int64_t b = 0; b < B; ++b) {
      (*items)[b].q_row0 = b * Tq;
      (*items)[b].k_row0 = b * Tkv;
      (*items)[b].Tq = Tq;
      (*items)[b].Tkv = Tkv;
    }
    *nitems = (int)B;
  }
  return ORACLE_OK;
}

/* heads_out: full grouped-query attention.
 *   q   [B, Tq, Hq, d]   (dtype_in)       or [1, total, Hq, d] with cu_seqlens
 *   k,v [B, Tkv, Hkv, d] (dtype_in)       or [1, total, Hkv, d]
 *   out [B, Tq, Hq, d]   fp64
 * Steps: widen K and V to fp64; expand both to Hq heads (materialised copies, adjacent
 * repetition); for every item, query head and query row, attend over the visible keys of the
 * expanded head. Hkv == Hq reproduces per-head multi-head attention exactly. */
int oracle_gqa_attention(const void* q, const void* k, const void* v, int dtype_in, double* out,
                         int64_t B, int64_t Tq, int64_t Tkv, int Hq, int Hkv, int d, double scale,
                         int causal, const int32_t* cu_seqlens, int nseq, int64_t window,
                         int64_t n_sink, const float* rope_cos, const float* rope_sin,
                         int64_t rope_npos, int rope_mode, const float* qn_w, const float* kn_w,
                         double norm_eps) {
  if (Hq <= 0 || Hkv <= 0 || d <= 0) return ORACLE_ERR_SHAPE;
  if ((window > 0 || n_sink > 0) && !causal) return ORACLE_ERR_SHAPE;  /* windows are causal */
  if (rope_mode && (!rope_cos || !rope_sin || d % 2 != 0)) return ORACLE_ERR_SHAPE;
  if (Hq % Hkv != 0) return ORACLE_ERR_GROUPING;
  item_t* items = NULL;
  int nitems = 0;
  int rc = make_items(B, Tq, Tkv, cu_seqlens, nseq, &items, &nitems);
  if (rc) return rc;
  const int64_t qrows = cu_seqlens ? cu_seqlens[nseq] : B * Tq;
  const int64_t krows = cu_seqlens ? cu_seqlens[nseq] : B * Tkv;

  double* kw = (double*)malloc(sizeof(double) * (size_t)(krows * Hkv * d));
  double* vw = (double*)malloc(sizeof(double) * (size_t)(krows * Hkv * d));
  double* ke = (double*)malloc(sizeof(double) * (size_t)(krows * Hq * d));
  double* ve = (double*)malloc(sizeof(double) * (size_t)(krows * Hq * d));
  if (!kw || !vw || !ke || !ve) {
    free(kw); free(vw); free(ke); free(ve); free(items);
    return ORACLE_ERR_ALLOC;
  }
  for (int64_t i = 0; i < krows * Hkv * d; ++i) {
    kw[i] = widen(k, dtype_in, i);
    vw[i] = widen(v, dtype_in, i);
  }
  /* QK-norm of the keys first, then their rotation (the norm acts on the raw head row) */
  if (kn_w)
    for (int64_t r = 0; r < krows * Hkv; ++r) rms_row(&kw[r * (int64_t)d], d, kn_w, norm_eps);
  if (rope_mode & ROPE_K) {
    /* key j of an item sits at position j */
    for (int it = 0; it < nitems; ++it)
      for (int64_t j = 0; j < items[it].Tkv; ++j) {
        if (j >= rope_npos) {
          free(kw); free(vw); free(ke); free(ve); free(items);
          return ORACLE_ERR_SHAPE;
        }
        for (int h = 0; h < Hkv; ++h)
          rope_row(&kw[((items[it].k_row0 + j) * Hkv + h) * (int64_t)d], d, rope_cos, rope_sin, j);
      }
  }
  oracle_expand(kw, ke, 1, krows, Hkv, Hq, d);
  oracle_expand(vw, ve, 1, krows, Hkv, Hq, d);
  free(kw);
  free(vw);

  int64_t max_tkv = 0;
  for (int it = 0; it < nitems; ++it)
    if (items[it].Tkv > max_tkv) max_tkv = items[it].Tkv;
  /* item of every query row, so the work can be spread over (row, head) pairs */
  int* row_item = (int*)malloc(sizeof(int) * (size_t)(qrows > 0 ? qrows : 1));
  if (!row_item) {
    free(ke); free(ve); free(items);
    return ORACLE_ERR_ALLOC;
  }
  for (int it = 0; it < nitems; ++it)
    for (int64_t t = 0; t < items[it].Tq; ++t) row_item[items[it].q_row0 + t] = it;

  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* qh = (double*)malloc(sizeof(double) * (size_t)d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)(max_tkv + 1));
    if (!qh || !sc) {
#pragma omp atomic write
      err = ORACLE_ERR_ALLOC;
    } else {
#pragma omp for schedule(dynamic, 8)
      for (int64_t r = 0; r < qrows * Hq; ++r) {
        const int64_t row = r / Hq;
        const int h = (int)(r % Hq);
        const item_t I = items[row_item[row]];
        const int64_t t = row - I.q_row0;
        for (int c = 0; c < d; ++c) qh[c] = widen(q, dtype_in, (row * Hq + h) * (int64_t)d + c);
        if (qn_w) rms_row(qh, d, qn_w, norm_eps);
        if (rope_mode & ROPE_Q) {
          /* query t sits at position t + (Tkv - Tq), the same alignment as the causal mask */
          const int64_t qpos = t + (I.Tkv - I.Tq);
          if (qpos < 0 || qpos >= rope_npos) {
#pragma omp atomic write
            err = ORACLE_ERR_SHAPE;
            continue;
          }
          rope_row(qh, d, rope_cos, rope_sin, qpos);
        }
        /* head h of the expanded K/V: rows k_row0.. of the [krows][Hq][d] tables */
        const double* kh = &ke[(I.k_row0 * Hq + h) * (int64_t)d];
        const double* vh = &ve[(I.k_row0 * Hq + h) * (int64_t)d];
        attend_row(qh, kh, vh, (int64_t)Hq * d, visible_keys(t, I.Tq, I.Tkv, causal),
                   window_lo(t, I.Tq, I.Tkv, window), n_sink, d, scale, sc,
                   &out[(row * Hq + h) * (int64_t)d]);
      }
    }
    free(qh); free(sc);
  }
  free(row_item);
  free(ke);
  free(ve);
  free(items);
  return err;
}

/* The same attention for a chosen set of output rows only (rows are independent, so this is
 * exact for those rows). rows: nrows triples (b, t, head) where for a packed batch b == 0 and t
 * is the packed row. out: nrows x d fp64. For each row the expanded head is materialised by
 * copying the K/V rows of the item for the group's key/value head, found with the same
 * contiguous rule the expansion above realises: head / (Hq / Hkv). */
int oracle_gqa_attention_rows(const void* q, const void* k, const void* v, int dtype_in,
                              int64_t B, int64_t Tq, int64_t Tkv, int Hq, int Hkv, int d,
                              double scale, int causal, const int32_t* cu_seqlens, int nseq,
                              const int64_t* rows, int64_t nrows, double* out, int64_t window,
                              int64_t n_sink, const float* rope_cos, const float* rope_sin,
                              int64_t rope_npos, int rope_mode, const float* qn_w,
                              const float* kn_w, double norm_eps) {
  if (Hq <= 0 || Hkv <= 0 || d <= 0) return ORACLE_ERR_SHAPE;
  if ((window > 0 || n_sink > 0) && !causal) return ORACLE_ERR_SHAPE;  /* windows are causal */
  if (rope_mode && (!rope_cos || !rope_sin || d % 2 != 0)) return ORACLE_ERR_SHAPE;
  if (Hq % Hkv != 0) return ORACLE_ERR_GROUPING;
  item_t* items = NULL;
  int nitems = 0;
  int rc = make_items(B, Tq, Tkv, cu_seqlens, nseq, &items, &nitems);
  if (rc) return rc;
  int64_t max_tkv = 0;
  for (int it = 0; it < nitems; ++it)
    if (items[it].Tkv > max_tkv) max_tkv = items[it].Tkv;
  /* validate and locate every row first */
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t b = rows[3 * r], t = rows[3 * r + 1], h = rows[3 * r + 2];
    if (h < 0 || h >= Hq) { free(items); return ORACLE_ERR_SHAPE; }
    if (cu_seqlens) {
      if (b != 0 || t < 0 || t >= cu_seqlens[nseq]) { free(items); return ORACLE_ERR_SHAPE; }
    } else if (b < 0 || b >= B || t < 0 || t >= Tq) {
      free(items);
      return ORACLE_ERR_SHAPE;
    }
  }
  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* qh = (double*)malloc(sizeof(double) * (size_t)d);
    double* kh = (double*)malloc(sizeof(double) * (size_t)(max_tkv * d + 1));
    double* vh = (double*)malloc(sizeof(double) * (size_t)(max_tkv * d + 1));
    double* sc = (double*)malloc(sizeof(double) * (size_t)(max_tkv + 1));
    if (!qh || !kh || !vh || !sc) {
#pragma omp atomic write
      err = ORACLE_ERR_ALLOC;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows[3 * r], tglob = rows[3 * r + 1];
        const int h = (int)rows[3 * r + 2];
        item_t I;
        int64_t t;
        if (cu_seqlens) {
          int s = 0;
          while (!(tglob >= cu_seqlens[s] && tglob < cu_seqlens[s + 1])) ++s;
          I = items[s];
          t = tglob - I.q_row0;
        } else {
          I = items[b];
          t = tglob;
        }
        const int kvh = oracle_group_of(h, Hq, Hkv);
        const int64_t qpos = t + (I.Tkv - I.Tq);
        if (rope_mode && (I.Tkv > rope_npos || qpos < 0 || qpos >= rope_npos)) {
#pragma omp atomic write
          err = ORACLE_ERR_SHAPE;
          continue;
        }
        for (int64_t j = 0; j < I.Tkv; ++j) {
          for (int c = 0; c < d; ++c) {
            const int64_t src = ((I.k_row0 + j) * Hkv + kvh) * (int64_t)d + c;
            kh[j * d + c] = widen(k, dtype_in, src);
            vh[j * d + c] = widen(v, dtype_in, src);
          }
          if (kn_w) rms_row(&kh[j * d], d, kn_w, norm_eps);
          if (rope_mode & ROPE_K) rope_row(&kh[j * d], d, rope_cos, rope_sin, j);
        }
        const int64_t row = I.q_row0 + t;
        for (int c = 0; c < d; ++c) qh[c] = widen(q, dtype_in, (row * Hq + h) * (int64_t)d + c);
        if (qn_w) rms_row(qh, d, qn_w, norm_eps);
        if (rope_mode & ROPE_Q) rope_row(qh, d, rope_cos, rope_sin, qpos);
        attend_row(qh, kh, vh, d, visible_keys(t, I.Tq, I.Tkv, causal),
                   window_lo(t, I.Tq, I.Tkv, window), n_sink, d, scale, sc, &out[r * d]);
      }
    }
    free(qh); free(kh); free(vh); free(sc);
  }
  free(items);
  return err;
}

/* Grouped value attention (K3 notes, section 4, GVA: the inverse sharing). H query/key heads
 * serve HV = G*H value heads; before attending, q and k are repeated from H to HV heads with
 * adjacent copies (the notes' forward: repeat_interleave over the head axis), so value head j
 * is attended with query/key head j / G, and every value head keeps its own values.
 *   q [B, Tq, H, d], k [B, Tkv, H, d], v [B, Tkv, HV, d] (dtype_in)   (or packed, cu_seqlens)
 *   out [B, Tq, HV, d] fp64
 * Steps: widen; expand q and k to HV heads (materialised copies, oracle_expand); for every
 * item, value head j and query row, attend the expanded query row over the expanded keys of
 * head j and the values of head j. Mask, window and sinks as for oracle_gqa_attention. */
int oracle_gva_attention(const void* q, const void* k, const void* v, int dtype_in, double* out,
                         int64_t B, int64_t Tq, int64_t Tkv, int H, int HV, int d, double scale,
                         int causal, const int32_t* cu_seqlens, int nseq, int64_t window,
                         int64_t n_sink) {
  if (H <= 0 || HV <= 0 || d <= 0) return ORACLE_ERR_SHAPE;
  if ((window > 0 || n_sink > 0) && !causal) return ORACLE_ERR_SHAPE;
  if (HV % H != 0) return ORACLE_ERR_GROUPING;
  item_t* items = NULL;
  int nitems = 0;
  int rc = make_items(B, Tq, Tkv, cu_seqlens, nseq, &items, &nitems);
  if (rc) return rc;
  const int64_t qrows = cu_seqlens ? cu_seqlens[nseq] : B * Tq;
  const int64_t krows = cu_seqlens ? cu_seqlens[nseq] : B * Tkv;

  double* qw = (double*)malloc(sizeof(double) * (size_t)(qrows * H * d));
  double* kw = (double*)malloc(sizeof(double) * (size_t)(krows * H * d));
  double* qe = (double*)malloc(sizeof(double) * (size_t)(qrows * HV * d));
  double* ke = (double*)malloc(sizeof(double) * (size_t)(krows * HV * d));
  double* vw = (double*)malloc(sizeof(double) * (size_t)(krows * HV * d));
  int* row_item = (int*)malloc(sizeof(int) * (size_t)(qrows > 0 ? qrows : 1));
  if (!qw || !kw || !qe || !ke || !vw || !row_item) {
    free(qw); free(kw); free(qe); free(ke); free(vw); free(row_item); free(items);
    return ORACLE_ERR_ALLOC;
  }
  for (int64_t i = 0; i < qrows * H * d; ++i) qw[i] = widen(q, dtype_in, i);
  for (int64_t i = 0; i < krows * H * d; ++i) kw[i] = widen(k, dtype_in, i);
  for (int64_t i = 0; i < krows * HV * d; ++i) vw[i] = widen(v, dtype_in, i);
  oracle_expand(qw, qe, 1, qrows, H, HV, d);
  oracle_expand(kw, ke, 1, krows, H, HV, d);
  free(qw);
  free(kw);

  int64_t max_tkv = 0;
  for (int it = 0; it < nitems; ++it)
    if (items[it].Tkv > max_tkv) max_tkv = items[it].Tkv;
  for (int it = 0; it < nitems; ++it)
    for (int64_t t = 0; t < items[it].Tq; ++t) row_item[items[it].q_row0 + t] = it;

  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)(max_tkv + 1));
    if (!sc) {
#pragma omp atomic write
      err = ORACLE_ERR_ALLOC;
    } else {
#pragma omp for schedule(dynamic, 8)
      for (int64_t r = 0; r < qrows * HV; ++r) {
        const int64_t row = r / HV;
        const int j = (int)(r % HV);
        const item_t I = items[row_item[row]];
        const int64_t t = row - I.q_row0;
        const double* qh = &qe[(row * HV + j) * (int64_t)d];
        const double* kh = &ke[(I.k_row0 * HV + j) * (int64_t)d];
        const double* vh = &vw[(I.k_row0 * HV + j) * (int64_t)d];
        attend_row(qh, kh, vh, (int64_t)HV * d, visible_keys(t, I.Tq, I.Tkv, causal),
                   window_lo(t, I.Tq, I.Tkv, window), n_sink, d, scale, sc,
                   &out[(row * HV + j) * (int64_t)d]);
      }
    }
    free(sc);
  }
  free(row_item);
  free(qe);
  free(ke);
  free(vw);
  free(items);
  return err;
}

/* Backward of grouped-query attention, written out from the chain rule in fp64.
 *   q, dout [B, Tq, Hq, d]; k, v [B, Tkv, Hkv, d] (dtype_in); dq [B, Tq, Hq, d] and
 *   dk, dv [B, Tkv, Hkv, d] fp64 outputs (dense batches).
 * For every query row (b, t, head h) with visible keys J (the forward's rule, incl. window):
 *   s_j = scale q.k_j, P_j = exp(s_j - max) / sum (two-pass, as the forward),
 *   dP_j = dout.v_j, D = sum_j P_j dP_j, dS_j = P_j (dP_j - D),
 *   dq = scale sum_j dS_j k_j;  expanded head h: dk_e[j] += scale dS_j q, dv_e[j] += P_j dout.
 * The key/value heads were replicated G = Hq/Hkv times into the expanded heads (adjacent
 * copies), so their gradients are the SUM over the G copies (K3 notes, section 4, backward:
 * the backward of a replication sums, it does not average). */
int oracle_gqa_attention_bwd(const void* q, const void* k, const void* v, const void* dout,
                             int dtype_in, double* dq, double* dk, double* dv, int64_t B,
                             int64_t Tq, int64_t Tkv, int Hq, int Hkv, int d, double scale,
                             int causal, int64_t window, int64_t n_sink) {
  if (B <= 0 || Tq <= 0 || Tkv <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return ORACLE_ERR_SHAPE;
  if (Hq % Hkv != 0) return ORACLE_ERR_GROUPING;
  if ((window > 0 || n_sink > 0) && !causal) return ORACLE_ERR_SHAPE;
  const int G = Hq / Hkv;
  const int64_t krows = B * Tkv;
  double* kw = (double*)malloc(sizeof(double) * (size_t)(krows * Hkv * d));
  double* vw = (double*)malloc(sizeof(double) * (size_t)(krows * Hkv * d));
  double* ke = (double*)malloc(sizeof(double) * (size_t)(krows * Hq * d));
  double* ve = (double*)malloc(sizeof(double) * (size_t)(krows * Hq * d));
  double* dke = (double*)calloc((size_t)(krows * Hq * d), sizeof(double));
  double* dve = (double*)calloc((size_t)(krows * Hq * d), sizeof(double));
  if (!kw || !vw || !ke || !ve || !dke || !dve) {
    free(kw); free(vw); free(ke); free(ve); free(dke); free(dve);
    return ORACLE_ERR_ALLOC;
  }
  for (int64_t i = 0; i < krows * Hkv * d; ++i) {
    kw[i] = widen(k, dtype_in, i);
    vw[i] = widen(v, dtype_in, i);
  }
  oracle_expand(kw, ke, 1, krows, Hkv, Hq, d);
  oracle_expand(vw, ve, 1, krows, Hkv, Hq, d);
  free(kw);
  free(vw);

  int err = ORACLE_OK;
  /* one (batch item, expanded head) per task: each task owns its dk_e / dv_e head slice */
#pragma omp parallel
  {
    double* qh = (double*)malloc(sizeof(double) * (size_t)d);
    double* gh = (double*)malloc(sizeof(double) * (size_t)d);
    double* p = (double*)malloc(sizeof(double) * (size_t)Tkv);
    double* dp = (double*)malloc(sizeof(double) * (size_t)Tkv);
    if (!qh || !gh || !p || !dp) {
#pragma omp atomic write
      err = ORACLE_ERR_ALLOC;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t task = 0; task < B * Hq; ++task) {
        const int64_t b = task / Hq;
        const int h = (int)(task % Hq);
        const int64_t kstride = (int64_t)Hq * d;
        const double* kh = &ke[(b * Tkv * Hq + h) * (int64_t)d];
        const double* vh = &ve[(b * Tkv * Hq + h) * (int64_t)d];
        double* dkh = &dke[(b * Tkv * Hq + h) * (int64_t)d];
        double* dvh = &dve[(b * Tkv * Hq + h) * (int64_t)d];
        for (int64_t t = 0; t < Tq; ++t) {
          const int64_t row = (b * Tq + t) * Hq + h;
          for (int c = 0; c < d; ++c) {
            qh[c] = widen(q, dtype_in, row * (int64_t)d + c);
            gh[c] = widen(dout, dtype_in, row * (int64_t)d + c);
          }
          const int64_t nvis = visible_keys(t, Tq, Tkv, causal);
          const int64_t lo = window_lo(t, Tq, Tkv, window);
          double* dqr = &dq[row * (int64_t)d];
          for (int c = 0; c < d; ++c) dqr[c] = 0.0;
          /* forward probabilities, two-pass */
          double m = -INFINITY;
          for (int64_t j = 0; j < nvis; ++j) {
            if (j < lo && j >= n_sink) continue;
            double dot = 0.0;
            for (int c = 0; c < d; ++c) dot += qh[c] * kh[j * kstride + c];
            p[j] = scale * dot;
            if (p[j] > m) m = p[j];
          }
          if (m == -INFINITY) continue; /* no visible key: no gradient */
          double l = 0.0;
          for (int64_t j = 0; j < nvis; ++j) {
            if (j < lo && j >= n_sink) continue;
            p[j] = exp(p[j] - m);
            l += p[j];
          }
          double D = 0.0;
          for (int64_t j = 0; j < nvis; ++j) {
            if (j < lo && j >= n_sink) continue;
            p[j] /= l;
            double dot = 0.0;
            for (int c = 0; c < d; ++c) dot += gh[c] * vh[j * kstride + c];
            dp[j] = dot;
            D += p[j] * dp[j];
          }
          for (int64_t j = 0; j < nvis; ++j) {
            if (j < lo && j >= n_sink) continue;
            const double ds = p[j] * (dp[j] - D);
            for (int c = 0; c < d; ++c) {
              dqr[c] += scale * ds * kh[j * kstride + c];
              dkh[j * kstride + c] += scale * ds * qh[c];
              dvh[j * kstride + c] += p[j] * gh[c];
            }
          }
        }
      }
    }
    free(qh); free(gh); free(p); free(dp);
  }
  /* fold the expanded-head gradients back: sum over the G copies of each key/value head */
  for (int64_t r = 0; r < krows; ++r)
    for (int j = 0; j < Hkv; ++j)
      for (int c = 0; c < d; ++c) {
        double sk = 0.0, sv = 0.0;
        for (int g = 0; g < G; ++g) {
          sk += dke[(r * Hq + j * G + g) * (int64_t)d + c];
          sv += dve[(r * Hq + j * G + g) * (int64_t)d + c];
        }
        dk[(r * Hkv + j) * (int64_t)d + c] = sk;
        dv[(r * Hkv + j) * (int64_t)d + c] = sv;
      }
  free(ke); free(ve); free(dke); free(dve);
  return err;
}
