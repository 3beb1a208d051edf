// common.hpp -- device helpers and launcher declarations shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// log2(e): exponentials are evaluated as 2^(x * log2 e) on the hardware base-2 exponential.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round-to-nearest-even float -> bf16 bits (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
// Two floats -> packed bf16 pair (lo in bits 0-15), one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one held by lane l ^ 32 without going through LDS:
// v_permlane32_swap leaves the lower half's value in result[0] and the upper half's in
// result[1] of every lane, so both halves compute from the same operands in the same order.
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource word 3 for unformatted buffer loads: loads at or past num_records bytes
// return zeros. Only the VGPR offset takes part in that range check (the SGPR offset does not),
// so every offset goes in the VGPR operand; kOutside is past any buffer used here.
constexpr int kBufWord3 = 0x00020000;
constexpr unsigned kOutside = 0x80000000u;
// s_waitcnt immediate for vmcnt(0) with the other counters left alone (expcnt 7, lgkmcnt 15)
constexpr int kVmcnt0 = 0x0F70;

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read (ds_read_b64_tr_b16): with lane 4r + t of a 16-lane group pointing at 4
// consecutive bf16 of row r (columns 4t .. 4t+3), lane j of the group receives column j of rows
// 0..3.
__device__ __forceinline__ u32x2 lds_read_tr(const char* base, int byte_off) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((__attribute__((address_space(3))) const char*)base + byte_off));
  return __builtin_bit_cast(u32x2, r);
}

// Keeps the compiler from moving LDS accesses across this point. For an LDS region written and
// read back only by one wave, whose LDS instructions execute in program order, this is all the
// ordering needed (no wait, no workgroup barrier).
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// Element type traits for the kernels that take either dtype.
struct F32 {
  typedef float T;
  static constexpr int kBytes = 4;
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static float to_f32(float x) { return x; }
  __device__ static float from_f32(float x) { return x; }
};
struct BF16 {
  typedef uint16_t T;
  static constexpr int kBytes = 2;
  __device__ static float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
  __device__ static uint16_t from_f32(float x) { return f32_to_bf16(x); }
};

// Item geometry of a launch: a dense batch of B items of (Tq, Tkv), or a packed batch whose
// item s spans rows cu[s] .. cu[s+1]-1 of both q and k/v.
struct Items {
  const int32_t* cu;  // device offsets or nullptr
  int Tq, Tkv;        // dense item sizes (ignored when cu != nullptr)
  __device__ __forceinline__ void get(int item, int64_t& q0, int64_t& k0, int& tq,
                                      int& tkv) const {
    if (cu) {
      const int a = cu[item], b = cu[item + 1];
      q0 = a;
      k0 = a;
      tq = b - a;
      tkv = b - a;
    } else {
      q0 = static_cast<int64_t>(item) * Tq;
      k0 = static_cast<int64_t>(item) * Tkv;
      tq = Tq;
      tkv = Tkv;
    }
  }
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int nitems;     // B, or number of packed sequences
  int max_tq;     // longest query length of any item (grid size)
  Items items;
  int Hq, Hkv, d;
  float scale;
  int causal;
  int window;  // > 0: causal sliding window of this many keys (0: none)
  int n_sink;  // keys 0 .. n_sink-1 stay visible below the window
  const float* rope_cos;  // rotary tables [rope_rows][d/2] (device), or nullptr
  const float* rope_sin;
  int rope_rows;
  float* lse;  // optional output: natural-log log-sum-exp of each row's scaled scores
  const float* qn_w;  // QK-norm weights [d] of queries and keys (device), or nullptr
  const float* kn_w;
  float norm_eps;
  int keys_prepared;  // keys already normalised / turned: process the queries only
  // Value and output geometry, in elements. Grouped-query attention: dv = d, vslices = 1,
  // v_row = Hkv*d, v_head = d, o_row = Hq*d, o_head = d. Grouped value attention hands in the
  // G value heads of a query/key head as one value row of G*d columns, produced in vslices
  // slices of dv columns each.
  int dv, vslices;
  int v_row, v_head;  // between value rows of consecutive positions / key-value heads
  int o_row, o_head;  // between output rows of consecutive positions / query heads
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int B, Tkv, Hq, Hkv, d;
  float scale;
  float* ws;      // partial results
  int nsplit;     // splits of the cache
  int per;        // keys per split (a multiple of the kernel's key tile)
  const int32_t* lens;  // device per-sequence cache lengths, or nullptr (all Tkv)
  int window;     // > 0: the query sees only the last `window` cache entries (plus sinks)
  int n_sink;     // cache entries 0 .. n_sink-1 stay visible below the window
  const float* rope_cos;  // rotary tables for the query [rope_rows][d/2] (device), or nullptr
  const float* rope_sin;
  int rope_rows;
  const float* qn_w;  // QK-norm weights [d] of the query (device), or nullptr
  float norm_eps;
};
// Rotary embedding of one 16-byte chunk of a head row in place: 4 pairs (2i, 2i+1), each turned
// by the angle whose cos / sin are given (the pair is one complex number times e^{i angle}).
__device__ __forceinline__ u32x4 rope_chunk(u32x4 w, f32x4 c, f32x4 s) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float re = bf16_lo(w[e]), im = bf16_hi(w[e]);
    w[e] = pack_bf16x2(fmaf(re, c[e], -im * s[e]), fmaf(re, s[e], im * c[e]));
  }
  return w;
}

// The same arithmetic on 8 fp32 values (one 16-byte chunk of a head row, 4 pairs).
__device__ __forceinline__ void rope8(float* x, f32x4 c, f32x4 s) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float re = x[2 * e], im = x[2 * e + 1];
    x[2 * e] = fmaf(re, c[e], -im * s[e]);
    x[2 * e + 1] = fmaf(re, s[e], im * c[e]);
  }
}
__device__ __forceinline__ void unpack8(u32x4 w, float* x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(w[e]);
    x[2 * e + 1] = bf16_hi(w[e]);
  }
}
__device__ __forceinline__ u32x4 pack8(const float* x) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
  return w;
}
__device__ __forceinline__ float sumsq8(u32x4 w) {
  float x[8], s = 0.f;
  unpack8(w, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf(x[e], x[e], s);
  return s;
}
// QK-norm of one 16-byte chunk: x * inv * w, with inv = 1/sqrt(mean(x^2) + eps) of the whole
// head row and w the chunk's 8 weights (two fp32 vectors).
__device__ __forceinline__ void norm8(float* x, float inv, f32x4 w0, f32x4 w1) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] *= inv * w0[e];
    x[4 + e] *= inv * w1[e];
  }
}
// Sum over aligned groups of N = 8 or 16 consecutive lanes, left in every lane of the group, with
// DPP moves inside a 16-lane row (no LDS crossbar): swap neighbours, swap pairs, mirror the
// 8-lane halves (quad sums meet), and for 16 also mirror the row. DPP controls: quad_perm
// [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(N == 8 || N == 16, "DPP row reductions over 8 or 16 lanes");
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
  if constexpr (N == 16)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}
__device__ __forceinline__ float rms_inv(float sumsq, int d, float eps) {
  return __builtin_amdgcn_rsqf(sumsq / static_cast<float>(d) + eps);
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;  // [B, Tq, Hq] natural-log log-sum-exp of the forward rows
  float* Drow;       // workspace [B, Tq, Hq]: dout . out
  void* dq;
  void* dk;
  void* dv;
  int B, Tq, Tkv, Hq, Hkv, d;
  float scale;
  int causal;
  // packed batch: B sequences at the device offsets items.cu (Tq == Tkv == total tokens), the
  // longest max_len tokens; dense: items.cu == nullptr, items.Tq / items.Tkv == Tq / Tkv
  Items items;
  int max_len;
  int window;  // > 0: causal sliding window of this many keys (0: none)
  int n_sink;  // keys 0 .. n_sink-1 stay visible below the window
};

// Launchers (return hipSuccess or the launch error). Shapes have been validated by the caller.
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
int prefill_bf16_cols();  // (position, head) columns per bf16 prefill workgroup
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_backward_bf16(const BwdArgs& a, hipStream_t s);
// Key preparation (QK-norm and rotary embedding of key rows, once per key).
struct KeyPrepArgs {
  const void* k;
  void* out;
  int64_t rows;       // B*T*H key rows (dense) or total*H (packed)
  int T, H, d;        // dense sequence length, heads, head dim
  const int32_t* cu;  // packed sequence offsets (device) or nullptr
  int nseq;
  int pos0;           // position of each sequence's first key
  const float* w;     // QK-norm weights [d] or nullptr
  float eps;
  const float* rope_cos;  // rotary tables [rows][d/2] or nullptr
  const float* rope_sin;
};
hipError_t launch_prepare_keys(const KeyPrepArgs& a, hipStream_t s);

hipError_t launch_fold(const void* src, void* dst, int64_t BT, int H, int g, int d, int is_bf16,
                       hipStream_t s);

// Decode split planning (host): shared by the workspace query and the launcher.
int decode_num_splits(int B, int Tkv, int Hq, int Hkv, int d);
int decode_split_len(int Tkv, int nsplit);
size_t decode_workspace_bytes(int B, int Tkv, int Hq, int Hkv, int d);
// The library's own decode scratch (for callers that cannot allocate): its size, and its device
// address on the current device (taken once per device).
constexpr size_t kDecodeScratchBytes = size_t{16} << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace gqa
