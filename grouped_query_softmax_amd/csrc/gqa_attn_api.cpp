// gqa_attn_api.cpp -- the extern "C" boundary: argument validation and kernel dispatch.
//
// Every check runs before anything is enqueued, so an error status means nothing was written.
// The error convention follows the GQA lab page ("Transformer -- attention by hand: reducing only
// the key/value heads", steps 1-3 and 6-7): head counts that do not split evenly are an error
// (GQA_ERR_GROUPING), never silently truncated.
#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "gqa_attn.h"
#include "common.hpp"
#include "backward.hpp"
#include "decode.hpp"

static_assert(GQA_DECODE_SCRATCH_BYTES == gqa::kDecodeScratchBytes,
              "the header's scratch limit is the size of the library's array");

namespace {

constexpr int kMaxGridYZ = 65535;
// a flat grid must keep blockIdx.x * blockDim.x below 2^32
constexpr int64_t kMaxFlatWorkgroups512 = (int64_t{1} << 32) / 512 - 1;
constexpr int64_t kMaxFlatWorkgroups256 = (int64_t{1} << 32) / 256 - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t esize(gqa_dtype_t t) { return t == GQA_DTYPE_BF16 ? 2 : 4; }

bool dtype_ok(gqa_dtype_t t) { return t == GQA_DTYPE_F32 || t == GQA_DTYPE_BF16; }

bool attn_d_supported(gqa_dtype_t t, int d) {
  if (t == GQA_DTYPE_BF16) return d == 64 || d == 128;
  if (t == GQA_DTYPE_F32) return d == 16 || d == 32 || d == 64 || d == 128;
  return false;
}

// Rows-per-workgroup geometry must match the launchers (f32: 256 rows).
int cols_per_wg(gqa_dtype_t t) { return t == GQA_DTYPE_BF16 ? gqa::prefill_bf16_cols() : 256; }
int64_t prefill_tiles(gqa_dtype_t t, int G, int max_tq) {
  const int cols = cols_per_wg(t);
  const int hpw = G < cols ? G : cols;
  const int ppw = cols / hpw;
  return (static_cast<int64_t>(max_tq) + ppw - 1) / ppw;
}
int64_t head_tiles(gqa_dtype_t t, int G) {
  const int cols = cols_per_wg(t);
  const int hpw = G < cols ? G : cols;
  return (G + hpw - 1) / hpw;
}

gqa_status_t from_hip(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_HIP; }

// The score factor: the caller's, or 1/sqrt(d) for GQA_SCALE_DEFAULT (GQA lab page, step 4:
// scores are divided by the square root of the head dimension). False for a negative or
// non-finite scale.
bool resolve_scale(float& scale, int d) {
  if (scale == GQA_SCALE_DEFAULT) scale = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
  return isfinite(scale) && scale > 0.f;
}

// Value/output geometry of grouped-query attention: one value row of d columns per key/value
// head, one output row per query head.
void set_gqa_geometry(gqa::PrefillArgs& a) {
  a.dv = a.d;
  a.vslices = 1;
  a.v_row = a.Hkv * a.d;
  a.v_head = a.d;
  a.o_row = a.Hq * a.d;
  a.o_head = a.d;
}

}  // namespace

extern "C" {

int gqa_attn_abi_version(void) { return GQA_ATTN_ABI_VERSION; }

const char* gqa_status_string(gqa_status_t s) {
  switch (s) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL_PTR: return "a required pointer is NULL";
    case GQA_ERR_SHAPE: return "invalid or inconsistent sizes (or causal with Tq > Tkv)";
    case GQA_ERR_GROUPING: return "head count does not split evenly into groups";
    case GQA_ERR_UNSUPPORTED: return "unsupported dtype / head dim, or pointer not 16-byte aligned";
    case GQA_ERR_WORKSPACE: return "decode workspace missing or too small";
    case GQA_ERR_ALIAS: return "output overlaps an input";
    case GQA_ERR_HIP: return "HIP runtime error while enqueueing";
  }
  return "unknown status";
}

// Options shared by the extended entry points; a null pointer means none of them.
// keys_ready: the call reads keys that were normalised / turned beforehand (decode caches, or
// prefill with keys_prepared), so only the query weights are needed.
static gqa_status_t check_options(const gqa_attn_options_t* o, gqa_dtype_t dtype, int rows_needed,
                                  bool keys_ready = false) {
  if (!o) return GQA_OK;
  if (o->window < 0 || o->n_sink < 0) return GQA_ERR_SHAPE;
  const bool rope = o->rope_cos || o->rope_sin;
  if (rope && (!o->rope_cos || !o->rope_sin)) return GQA_ERR_NULL_PTR;
  if ((o->window > 0 || o->n_sink > 0 || rope) && dtype != GQA_DTYPE_BF16)
    return GQA_ERR_UNSUPPORTED;
  if (rope) {
    if (!aligned16(o->rope_cos) || !aligned16(o->rope_sin)) return GQA_ERR_UNSUPPORTED;
    if (o->rope_rows < rows_needed) return GQA_ERR_SHAPE;
  }
  if (o->lse && dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  keys_ready = keys_ready || o->keys_prepared;
  const bool norm = o->q_norm_w || o->k_norm_w;
  if (norm) {
    if (!o->q_norm_w || (!keys_ready && !o->k_norm_w)) return GQA_ERR_NULL_PTR;
    if (dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
    if (!aligned16(o->q_norm_w) || (o->k_norm_w && !aligned16(o->k_norm_w)))
      return GQA_ERR_UNSUPPORTED;
    if (!isfinite(o->norm_eps) || !(o->norm_eps > 0.f)) return GQA_ERR_SHAPE;
  }
  return GQA_OK;
}

static gqa_status_t prefill_impl(const void* q, const void* k, const void* v, void* out, int B,
                                 int Tq, int Tkv, int Hq, int Hkv, int d, float scale, int causal,
                                 const gqa_attn_options_t* opt, const int32_t* cu_seqlens,
                                 int max_seqlen, gqa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !out) return GQA_ERR_NULL_PTR;
  if (B <= 0 || Tq <= 0 || Tkv <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return GQA_ERR_SHAPE;
  if (!resolve_scale(scale, d)) return GQA_ERR_SHAPE;
  if (Hq % Hkv != 0) return GQA_ERR_GROUPING;
  if (!dtype_ok(dtype) || !attn_d_supported(dtype, d)) return GQA_ERR_UNSUPPORTED;
  if (const gqa_status_t st = check_options(opt, dtype, cu_seqlens ? max_seqlen : Tkv))
    return st;
  const int window = opt ? opt->window : 0;
  const int n_sink = opt ? opt->n_sink : 0;
  if ((window > 0 || n_sink > 0) && !causal) return GQA_ERR_SHAPE;  // windows are causal
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return GQA_ERR_UNSUPPORTED;
  int nitems, max_tq;
  if (cu_seqlens) {
    if (Tq != Tkv || max_seqlen <= 0 || max_seqlen > Tq) return GQA_ERR_SHAPE;
    nitems = B;
    max_tq = max_seqlen;
  } else {
    if (causal && Tq > Tkv) return GQA_ERR_SHAPE;
    nitems = B;
    max_tq = Tq;
  }
  const int G = Hq / Hkv;
  const size_t es = esize(dtype);
  if (dtype == GQA_DTYPE_BF16) {
    // one flat grid of 512-thread workgroups; key/value offsets inside an item are 32-bit
    const int64_t tiles = prefill_tiles(dtype, G, max_tq);
    const int64_t wgs = static_cast<int64_t>(Hkv) * head_tiles(dtype, G) * nitems *
                        (causal ? (tiles + 1) / 2 : tiles);
    const int64_t item_kv_bytes =
        static_cast<int64_t>(cu_seqlens ? max_tq : Tkv) * Hkv * d * static_cast<int64_t>(es);
    if (wgs > kMaxFlatWorkgroups512 || item_kv_bytes > INT32_MAX) return GQA_ERR_UNSUPPORTED;
  } else if (nitems > kMaxGridYZ || prefill_tiles(dtype, G, max_tq) > INT32_MAX ||
             static_cast<int64_t>(Hkv) * head_tiles(dtype, G) > kMaxGridYZ) {
    return GQA_ERR_UNSUPPORTED;
  }
  const size_t rows_q = cu_seqlens ? static_cast<size_t>(Tq) : static_cast<size_t>(B) * Tq;
  const size_t rows_k = cu_seqlens ? static_cast<size_t>(Tkv) : static_cast<size_t>(B) * Tkv;
  const size_t nq = rows_q * Hq * d * es, nk = rows_k * Hkv * d * es;
  if (overlap(out, nq, q, nq) || overlap(out, nq, k, nk) || overlap(out, nq, v, nk))
    return GQA_ERR_ALIAS;

  gqa::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.nitems = nitems;
  a.max_tq = max_tq;
  a.items.cu = cu_seqlens;
  a.items.Tq = Tq;
  a.items.Tkv = Tkv;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.window = window;
  a.n_sink = window > 0 ? n_sink : 0;  // without a window every past key is visible anyway
  a.rope_cos = opt ? opt->rope_cos : nullptr;
  a.rope_sin = opt ? opt->rope_sin : nullptr;
  a.rope_rows = opt ? opt->rope_rows : 0;
  a.lse = opt ? opt->lse : nullptr;
  a.qn_w = opt ? opt->q_norm_w : nullptr;
  a.kn_w = opt ? opt->k_norm_w : nullptr;
  a.norm_eps = opt ? opt->norm_eps : 0.f;
  a.keys_prepared = opt ? opt->keys_prepared : 0;
  set_gqa_geometry(a);
  if (a.lse && overlap(a.lse, rows_q * Hq * sizeof(float), q, nq)) return GQA_ERR_ALIAS;
  return from_hip(dtype == GQA_DTYPE_BF16 ? gqa::launch_prefill_bf16(a, stream)
                                          : gqa::launch_prefill_f32(a, stream));
}

gqa_status_t gqa_attn_prefill(const void* q, const void* k, const void* v, void* out, int B,
                              int Tq, int Tkv, int Hq, int Hkv, int d, float scale, int causal,
                              const int32_t* cu_seqlens, int max_seqlen, gqa_dtype_t dtype,
                              hipStream_t stream) {
  return prefill_impl(q, k, v, out, B, Tq, Tkv, Hq, Hkv, d, scale, causal, nullptr, cu_seqlens,
                      max_seqlen, dtype, stream);
}

gqa_status_t gqa_attn_prefill_window(const void* q, const void* k, const void* v, void* out,
                                     int B, int Tq, int Tkv, int Hq, int Hkv, int d, float scale,
                                     int window, int n_sink, const int32_t* cu_seqlens,
                                     int max_seqlen, gqa_dtype_t dtype, hipStream_t stream) {
  gqa_attn_options_t o = {window, n_sink, nullptr, nullptr, 0, nullptr};
  return prefill_impl(q, k, v, out, B, Tq, Tkv, Hq, Hkv, d, scale, 1, &o, cu_seqlens, max_seqlen,
                      dtype, stream);
}

gqa_status_t gqa_attn_prefill_ex(const void* q, const void* k, const void* v, void* out, int B,
                                 int Tq, int Tkv, int Hq, int Hkv, int d, float scale, int causal,
                                 const int32_t* cu_seqlens, int max_seqlen,
                                 const gqa_attn_options_t* options, gqa_dtype_t dtype,
                                 hipStream_t stream) {
  return prefill_impl(q, k, v, out, B, Tq, Tkv, Hq, Hkv, d, scale, causal, options, cu_seqlens,
                      max_seqlen, dtype, stream);
}

gqa_status_t gqa_attn_prefill_gva(const void* q, const void* k, const void* v, void* out, int B,
                                  int Tq, int Tkv, int H, int HV, int d, float scale, int causal,
                                  const int32_t* cu_seqlens, int max_seqlen,
                                  const gqa_attn_options_t* opt, gqa_dtype_t dtype,
                                  hipStream_t stream) {
  if (!q || !k || !v || !out) return GQA_ERR_NULL_PTR;
  if (B <= 0 || Tq <= 0 || Tkv <= 0 || H <= 0 || HV <= 0 || d <= 0) return GQA_ERR_SHAPE;
  if (!resolve_scale(scale, d)) return GQA_ERR_SHAPE;
  if (HV % H != 0) return GQA_ERR_GROUPING;
  if (dtype != GQA_DTYPE_BF16 || !attn_d_supported(dtype, d)) return GQA_ERR_UNSUPPORTED;
  if (const gqa_status_t st = check_options(opt, dtype, cu_seqlens ? max_seqlen : Tkv)) return st;
  if (opt && (opt->rope_cos || opt->rope_sin || opt->q_norm_w || opt->k_norm_w))
    return GQA_ERR_UNSUPPORTED;
  const int window = opt ? opt->window : 0;
  const int n_sink = opt ? opt->n_sink : 0;
  if ((window > 0 || n_sink > 0) && !causal) return GQA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return GQA_ERR_UNSUPPORTED;
  int max_tq;
  if (cu_seqlens) {
    if (Tq != Tkv || max_seqlen <= 0 || max_seqlen > Tq) return GQA_ERR_SHAPE;
    max_tq = max_seqlen;
  } else {
    if (causal && Tq > Tkv) return GQA_ERR_SHAPE;
    max_tq = Tq;
  }
  const int G = HV / H;
  // a workgroup produces dv value columns of one query/key head: 128 when the head's value row
  // (G*d columns) splits into 128-column slices, else d (then one slice per value head)
  const int dv = (G * d) % 128 == 0 ? 128 : d;
  const int vslices = G * d / dv;
  const int64_t tiles = prefill_tiles(dtype, 1, max_tq);
  const int64_t wgs = static_cast<int64_t>(H) * vslices * B * (causal ? (tiles + 1) / 2 : tiles);
  const int64_t item_v_bytes = static_cast<int64_t>(cu_seqlens ? max_tq : Tkv) * HV * d * 2;
  if (wgs > kMaxFlatWorkgroups512 || item_v_bytes > INT32_MAX) return GQA_ERR_UNSUPPORTED;
  const size_t rows_q = cu_seqlens ? static_cast<size_t>(Tq) : static_cast<size_t>(B) * Tq;
  const size_t rows_k = cu_seqlens ? static_cast<size_t>(Tkv) : static_cast<size_t>(B) * Tkv;
  const size_t nq = rows_q * H * d * 2, nk = rows_k * H * d * 2, nv = rows_k * HV * d * 2;
  const size_t no = rows_q * HV * d * 2;
  if (overlap(out, no, q, nq) || overlap(out, no, k, nk) || overlap(out, no, v, nv))
    return GQA_ERR_ALIAS;

  gqa::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.nitems = B;
  a.max_tq = max_tq;
  a.items.cu = cu_seqlens;
  a.items.Tq = Tq;
  a.items.Tkv = Tkv;
  a.Hq = H;  // one query per query/key head: the kernel's grouped-query view with G = 1
  a.Hkv = H;
  a.d = d;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.window = window;
  a.n_sink = window > 0 ? n_sink : 0;
  a.rope_cos = a.rope_sin = nullptr;
  a.rope_rows = 0;
  a.lse = opt ? opt->lse : nullptr;
  a.qn_w = a.kn_w = nullptr;
  a.norm_eps = 0.f;
  a.keys_prepared = 0;
  a.dv = dv;
  a.vslices = vslices;
  a.v_row = HV * d;
  a.v_head = G * d;
  a.o_row = HV * d;
  a.o_head = G * d;
  if (a.lse && (overlap(a.lse, rows_q * H * sizeof(float), q, nq) ||
                overlap(a.lse, rows_q * H * sizeof(float), out, no)))
    return GQA_ERR_ALIAS;
  return from_hip(gqa::launch_prefill_bf16(a, stream));
}

size_t gqa_attn_decode_workspace_bytes_hkv(int B, int Tkv, int Hq, int Hkv, int d) {
  if (B <= 0 || Tkv <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0) return 0;
  return gqa::decode_workspace_bytes(B, Tkv, Hq, Hkv, d);
}

size_t gqa_attn_decode_workspace_bytes(int B, int Tkv, int Hq, int d) {
  if (B <= 0 || Tkv <= 0 || Hq <= 0 || d <= 0) return 0;
  // the largest requirement over every key/value head count that divides Hq
  size_t most = 0;
  for (int hkv = 1; hkv <= Hq; ++hkv)
    if (Hq % hkv == 0) most = std::max(most, gqa::decode_workspace_bytes(B, Tkv, Hq, hkv, d));
  return most;
}

// ring: k_cache / v_cache are bounded to the window (Tkv = n_sink + window slots per sequence,
// cache_lens counting every entry a sequence has had); see gqa_attn_decode_window_cache.
static gqa_status_t decode_impl(const void* q, const void* k_cache, const void* v_cache,
                                void* out, int B, int Tkv, int Hq, int Hkv, int d, float scale,
                                const int32_t* cache_lens, const gqa_attn_options_t* opt,
                                void* workspace, size_t workspace_bytes, gqa_dtype_t dtype,
                                hipStream_t stream, bool ring = false) {
  if (!q || !k_cache || !v_cache || !out) return GQA_ERR_NULL_PTR;
  if (ring && (!cache_lens || !opt)) return GQA_ERR_NULL_PTR;
  if (B <= 0 || Tkv <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return GQA_ERR_SHAPE;
  if (!resolve_scale(scale, d)) return GQA_ERR_SHAPE;
  if (Hq % Hkv != 0) return GQA_ERR_GROUPING;
  if (!dtype_ok(dtype) || !attn_d_supported(dtype, d)) return GQA_ERR_UNSUPPORTED;
  // the query's table row of a bounded cache is clamped to the tables (its length is on the
  // device and unbounded): one row is the least they need
  if (const gqa_status_t st = check_options(opt, dtype, ring ? 1 : Tkv, true)) return st;
  if (cache_lens && dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  const int window = opt ? opt->window : 0;
  const int n_sink = opt ? opt->n_sink : 0;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return GQA_ERR_UNSUPPORTED;
  if (dtype == GQA_DTYPE_F32 && B > kMaxGridYZ) return GQA_ERR_UNSUPPORTED;
  if (dtype == GQA_DTYPE_BF16) {
    // one flat grid of 256-thread workgroups; cache offsets inside a sequence are 32-bit
    const int G = Hq / Hkv;
    const int64_t wgs = static_cast<int64_t>(gqa::decode_num_splits(B, Tkv, Hq, Hkv, d)) * Hkv *
                        ((G + 15) / 16) * B;
    const int64_t cache_item_bytes = static_cast<int64_t>(Tkv) * Hkv * d * 2;
    if (wgs > kMaxFlatWorkgroups256 || cache_item_bytes > INT32_MAX ||
        static_cast<int64_t>(B) * Hq > INT32_MAX)
      return GQA_ERR_UNSUPPORTED;
  }
  const size_t es = esize(dtype);
  const size_t nq = static_cast<size_t>(B) * Hq * d * es;
  const size_t nk = static_cast<size_t>(B) * Tkv * Hkv * d * es;
  if (overlap(out, nq, q, nq) || overlap(out, nq, k_cache, nk) || overlap(out, nq, v_cache, nk))
    return GQA_ERR_ALIAS;

  if (dtype == GQA_DTYPE_F32) {
    // fp32: the vector-ALU prefill kernel with one query row per sequence; no workspace.
    if (workspace && overlap(workspace, workspace_bytes, out, nq)) return GQA_ERR_ALIAS;
    gqa::PrefillArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.nitems = B;
    a.max_tq = 1;
    a.items.cu = nullptr;
    a.items.Tq = 1;
    a.items.Tkv = Tkv;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.d = d;
    a.scale = scale;
    a.causal = 0;
    a.window = 0;
    a.n_sink = 0;
    a.rope_cos = a.rope_sin = nullptr;
    a.rope_rows = 0;
    a.lse = nullptr;
    a.qn_w = a.kn_w = nullptr;
    a.norm_eps = 0.f;
    a.keys_prepared = 0;
    set_gqa_geometry(a);
    return from_hip(gqa::launch_prefill_f32(a, stream));
  }
  const size_t need = gqa::decode_workspace_bytes(B, Tkv, Hq, Hkv, d);
  if (!workspace || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GQA_ERR_UNSUPPORTED;
  if (overlap(workspace, need, q, nq) || overlap(workspace, need, k_cache, nk) ||
      overlap(workspace, need, v_cache, nk) || overlap(workspace, need, out, nq))
    return GQA_ERR_ALIAS;
  gqa::DecodeArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.B = B;
  a.Tkv = Tkv;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.scale = scale;
  a.ws = static_cast<float*>(workspace);
  a.nsplit = gqa::decode_num_splits(B, Tkv, Hq, Hkv, d);
  a.per = gqa::decode_split_len(Tkv, a.nsplit);
  a.lens = cache_lens;
  a.window = window;
  a.n_sink = window > 0 ? n_sink : 0;
  a.rope_cos = opt ? opt->rope_cos : nullptr;
  a.rope_sin = opt ? opt->rope_sin : nullptr;
  a.rope_rows = opt ? opt->rope_rows : 0;
  a.qn_w = opt ? opt->q_norm_w : nullptr;  // the cache holds normalised keys
  a.norm_eps = opt ? opt->norm_eps : 0.f;
  return from_hip(ring ? gqa::launch_decode_window_cache_bf16(a, stream)
                       : gqa::launch_decode_bf16(a, stream));
}

gqa_status_t gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                             int B, int Tkv, int Hq, int Hkv, int d, float scale, int causal,
                             void* workspace, size_t workspace_bytes, gqa_dtype_t dtype,
                             hipStream_t stream) {
  (void)causal;  // a single query at the last position sees the whole cache
  return decode_impl(q, k_cache, v_cache, out, B, Tkv, Hq, Hkv, d, scale, nullptr, nullptr,
                     workspace, workspace_bytes, dtype, stream);
}

gqa_status_t gqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     void* out, int B, int Tkv, int Hq, int Hkv, int d,
                                     float scale, int causal, gqa_dtype_t dtype,
                                     hipStream_t stream) {
  (void)causal;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (dtype == GQA_DTYPE_BF16 && B > 0 && Tkv > 0 && Hq > 0 && Hkv > 0 && d > 0 &&
      Hq % Hkv == 0) {
    // the sizes decide the partials' footprint; past the fixed scratch the call is refused
    // before the scratch is even looked up
    if (gqa::decode_workspace_bytes(B, Tkv, Hq, Hkv, d) > GQA_DECODE_SCRATCH_BYTES)
      return GQA_ERR_WORKSPACE;
    if (gqa::decode_scratch(&ws) != hipSuccess) return GQA_ERR_HIP;
    ws_bytes = GQA_DECODE_SCRATCH_BYTES;
  }
  return decode_impl(q, k_cache, v_cache, out, B, Tkv, Hq, Hkv, d, scale, nullptr, nullptr, ws,
                     ws_bytes, dtype, stream);
}

gqa_status_t gqa_attn_decode_ragged(const void* q, const void* k_cache, const void* v_cache,
                                    void* out, int B, int Tmax, int Hq, int Hkv, int d,
                                    float scale, const int32_t* cache_lens, int window,
                                    int n_sink, void* workspace, size_t workspace_bytes,
                                    gqa_dtype_t dtype, hipStream_t stream) {
  gqa_attn_options_t o = {window, n_sink, nullptr, nullptr, 0, nullptr};
  return decode_impl(q, k_cache, v_cache, out, B, Tmax, Hq, Hkv, d, scale, cache_lens, &o,
                     workspace, workspace_bytes, dtype, stream);
}

gqa_status_t gqa_attn_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                                void* out, int B, int Tmax, int Hq, int Hkv, int d, float scale,
                                const int32_t* cache_lens, const gqa_attn_options_t* options,
                                void* workspace, size_t workspace_bytes, gqa_dtype_t dtype,
                                hipStream_t stream) {
  return decode_impl(q, k_cache, v_cache, out, B, Tmax, Hq, Hkv, d, scale, cache_lens, options,
                     workspace, workspace_bytes, dtype, stream);
}

gqa_status_t gqa_attn_decode_window_cache(const void* q, const void* k_cache, const void* v_cache,
                                          void* out, int B, int Hq, int Hkv, int d, float scale,
                                          const int32_t* cache_lens,
                                          const gqa_attn_options_t* options, void* workspace,
                                          size_t workspace_bytes, gqa_dtype_t dtype,
                                          hipStream_t stream) {
  if (!options || !cache_lens) return GQA_ERR_NULL_PTR;
  if (options->window < 1 || options->n_sink < 0 ||
      static_cast<int64_t>(options->window) + options->n_sink > INT32_MAX)
    return GQA_ERR_SHAPE;
  if (dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  return decode_impl(q, k_cache, v_cache, out, B, options->window + options->n_sink, Hq, Hkv, d,
                     scale, cache_lens, options, workspace, workspace_bytes, dtype, stream, true);
}

size_t gqa_attn_backward_workspace_bytes(int B, int Tq, int Hq) {
  if (B <= 0 || Tq <= 0 || Hq <= 0) return 0;
  return 2 * gqa::backward_row_array_floats(static_cast<size_t>(B) * Tq * Hq) * sizeof(float);
}

static gqa_status_t backward_impl(const void* q, const void* k, const void* v, const void* out,
                                  const void* dout, const float* lse, void* dq, void* dk,
                                  void* dv, int B, int Tq, int Tkv, int Hq, int Hkv, int d,
                                  float scale, int causal, const int32_t* cu_seqlens,
                                  int max_seqlen, const gqa_attn_options_t* opt, void* workspace,
                                  size_t workspace_bytes, gqa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv) return GQA_ERR_NULL_PTR;
  if (B <= 0 || Tq <= 0 || Tkv <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return GQA_ERR_SHAPE;
  if (!resolve_scale(scale, d)) return GQA_ERR_SHAPE;
  if (Hq % Hkv != 0) return GQA_ERR_GROUPING;
  if (dtype != GQA_DTYPE_BF16 || !attn_d_supported(dtype, d)) return GQA_ERR_UNSUPPORTED;
  if (opt) {
    // the backward of the rotary embedding and of QK-norm is not built
    if (opt->rope_cos || opt->rope_sin || opt->q_norm_w || opt->k_norm_w || opt->keys_prepared)
      return GQA_ERR_UNSUPPORTED;
    if (opt->window < 0 || opt->n_sink < 0) return GQA_ERR_SHAPE;
  }
  const int window = opt ? opt->window : 0;
  const int n_sink = opt ? opt->n_sink : 0;
  if ((window > 0 || n_sink > 0) && !causal) return GQA_ERR_SHAPE;  // windows are causal
  int max_len;
  if (cu_seqlens) {
    if (Tq != Tkv || max_seqlen <= 0 || max_seqlen > Tq) return GQA_ERR_SHAPE;
    max_len = max_seqlen;
  } else {
    if (causal && Tq > Tkv) return GQA_ERR_SHAPE;
    max_len = Tq > Tkv ? Tq : Tkv;
  }
  const void* ptrs[] = {q, k, v, out, dout, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GQA_ERR_UNSUPPORTED;
  // packed: one [1, total, ., d] batch; its rows and keys count once
  const int64_t qrows = cu_seqlens ? static_cast<int64_t>(Tq) : static_cast<int64_t>(B) * Tq;
  const int64_t krows = cu_seqlens ? static_cast<int64_t>(Tkv) : static_cast<int64_t>(B) * Tkv;
  const size_t need = gqa_attn_backward_workspace_bytes(1, static_cast<int>(qrows), Hq);
  if (!workspace || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GQA_ERR_UNSUPPORTED;
  // the largest of the three launches: rows / (256 / (d / 8)), key tiles of 32, query tiles
  const int64_t rows = qrows * Hq;
  const int64_t wgs = std::max({rows * (d / 8) / 256 + 1,
                                static_cast<int64_t>(B) * Hkv * ((max_len + 31) / 32),
                                static_cast<int64_t>(B) * max_len * Hq / 128 +
                                    static_cast<int64_t>(B) * Hkv + 1});
  // one sequence's q / dout and k / v rows are addressed with 32-bit byte offsets
  const int64_t tq_item = cu_seqlens ? max_len : Tq, tkv_item = cu_seqlens ? max_len : Tkv;
  const bool seq_fits = tq_item * Hq * d * 2 < (1LL << 31) && tkv_item * Hkv * d * 2 < (1LL << 31);
  if (wgs > kMaxFlatWorkgroups256 || rows * d > INT32_MAX * 8LL || !seq_fits)
    return GQA_ERR_UNSUPPORTED;
  const size_t nq = static_cast<size_t>(qrows) * Hq * d * 2;
  const size_t nk = static_cast<size_t>(krows) * Hkv * d * 2;
  const size_t nl = static_cast<size_t>(qrows) * Hq * sizeof(float);
  // every output (and the workspace) must be disjoint from every input and from each other
  const void* outs[] = {dq, dk, dv, workspace};
  const size_t outn[] = {nq, nk, nk, need};
  const void* ins[] = {q, k, v, out, dout, lse};
  const size_t inn[] = {nq, nk, nk, nq, nq, nl};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], outn[i], ins[j], inn[j])) return GQA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outn[i], outs[j], outn[j])) return GQA_ERR_ALIAS;
  }
  gqa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.Drow = static_cast<float*>(workspace);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.Tq = Tq;
  a.Tkv = Tkv;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.items.cu = cu_seqlens;
  a.items.Tq = Tq;
  a.items.Tkv = Tkv;
  a.max_len = max_len;
  a.window = window;
  a.n_sink = window > 0 ? n_sink : 0;  // without a window every past key is visible anyway
  return from_hip(gqa::launch_backward_bf16(a, stream));
}

gqa_status_t gqa_attn_backward(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               int B, int Tq, int Tkv, int Hq, int Hkv, int d, float scale,
                               int causal, void* workspace, size_t workspace_bytes,
                               gqa_dtype_t dtype, hipStream_t stream) {
  return backward_impl(q, k, v, out, dout, lse, dq, dk, dv, B, Tq, Tkv, Hq, Hkv, d, scale, causal,
                       nullptr, 0, nullptr, workspace, workspace_bytes, dtype, stream);
}

gqa_status_t gqa_attn_backward_ex(const void* q, const void* k, const void* v, const void* out,
                                  const void* dout, const float* lse, void* dq, void* dk,
                                  void* dv, int B, int Tq, int Tkv, int Hq, int Hkv, int d,
                                  float scale, int causal, const int32_t* cu_seqlens,
                                  int max_seqlen, const gqa_attn_options_t* options,
                                  void* workspace, size_t workspace_bytes, gqa_dtype_t dtype,
                                  hipStream_t stream) {
  return backward_impl(q, k, v, out, dout, lse, dq, dk, dv, B, Tq, Tkv, Hq, Hkv, d, scale, causal,
                       cu_seqlens, max_seqlen, options, workspace, workspace_bytes, dtype, stream);
}

gqa_status_t gqa_prepare_keys(const void* k, void* k_out, int B, int T, int Hkv, int d,
                              const int32_t* cu_seqlens, int max_seqlen, int pos0,
                              const gqa_attn_options_t* opt, gqa_dtype_t dtype,
                              hipStream_t stream) {
  if (!k || !k_out || !opt) return GQA_ERR_NULL_PTR;
  if (B <= 0 || T <= 0 || Hkv <= 0 || d <= 0 || pos0 < 0) return GQA_ERR_SHAPE;
  if (dtype != GQA_DTYPE_BF16 || !attn_d_supported(dtype, d)) return GQA_ERR_UNSUPPORTED;
  const bool rope = opt->rope_cos || opt->rope_sin;
  if (rope && (!opt->rope_cos || !opt->rope_sin)) return GQA_ERR_NULL_PTR;
  if (!rope && !opt->k_norm_w) return GQA_ERR_SHAPE;  // nothing to apply
  const int longest = cu_seqlens ? max_seqlen : T;
  if (cu_seqlens && (max_seqlen <= 0 || max_seqlen > T)) return GQA_ERR_SHAPE;
  if (rope) {
    if (!aligned16(opt->rope_cos) || !aligned16(opt->rope_sin)) return GQA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(opt->rope_rows) < static_cast<int64_t>(pos0) + longest)
      return GQA_ERR_SHAPE;
  }
  if (opt->k_norm_w) {
    if (!aligned16(opt->k_norm_w)) return GQA_ERR_UNSUPPORTED;
    if (!isfinite(opt->norm_eps) || !(opt->norm_eps > 0.f)) return GQA_ERR_SHAPE;
  }
  if (!aligned16(k) || !aligned16(k_out)) return GQA_ERR_UNSUPPORTED;
  // packed: [1, T = total, Hkv, d] with B + 1 offsets; dense: [B, T, Hkv, d]
  const int64_t rows = static_cast<int64_t>(cu_seqlens ? 1 : B) * T * Hkv;
  const size_t bytes = static_cast<size_t>(rows) * d * 2;
  if (k_out != k && overlap(k_out, bytes, k, bytes)) return GQA_ERR_ALIAS;
  if ((rows * (d / 8) + 255) / 256 > kMaxFlatWorkgroups256) return GQA_ERR_UNSUPPORTED;
  gqa::KeyPrepArgs a;
  a.k = k;
  a.out = k_out;
  a.rows = rows;
  a.T = T;
  a.H = Hkv;
  a.d = d;
  a.cu = cu_seqlens;
  a.nseq = cu_seqlens ? B : 0;
  a.pos0 = pos0;
  a.w = opt->k_norm_w;
  a.eps = opt->norm_eps;
  a.rope_cos = rope ? opt->rope_cos : nullptr;
  a.rope_sin = rope ? opt->rope_sin : nullptr;
  return from_hip(gqa::launch_prepare_keys(a, stream));
}

gqa_status_t gqa_fold_kv(const void* src, void* dst, int B, int T, int H, int g, int d,
                         gqa_dtype_t dtype, hipStream_t stream) {
  if (!src || !dst) return GQA_ERR_NULL_PTR;
  if (B <= 0 || T <= 0 || H <= 0 || g <= 0 || d <= 0) return GQA_ERR_SHAPE;
  if (H % g != 0) return GQA_ERR_GROUPING;
  if (!dtype_ok(dtype)) return GQA_ERR_UNSUPPORTED;
  const size_t es = esize(dtype);
  if ((static_cast<size_t>(d) * es) % 16 != 0) return GQA_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(dst)) return GQA_ERR_UNSUPPORTED;
  const size_t ns = static_cast<size_t>(B) * T * H * d * es;
  const size_t nd = static_cast<size_t>(B) * T * g * d * es;
  if (overlap(src, ns, dst, nd)) return GQA_ERR_ALIAS;
  return from_hip(gqa::launch_fold(src, dst, static_cast<int64_t>(B) * T, H, g, d,
                                   dtype == GQA_DTYPE_BF16 ? 1 : 0, stream));
}

}  // extern "C"
