// decode.hip -- split-KV grouped-query attention for one query token per sequence.
//
// A decode step is bound by streaming the key/value cache from HBM: every cached element is read
// once and used for a handful of flops (G query heads share it). Grouped-query attention is what
// makes the stream small: the cache holds Hkv heads, not Hq (course page "Week 7. Attention",
// step 2: 32 query / 8 key-value heads is a 4x smaller cache; GQA lab page "Transformer --
// attention by hand: reducing only the key/value heads", step 6: the cache element count has no
// query-head term).
//
// Kernel 1 (split): one workgroup per (sequence, key/value head, head chunk, split of the cache).
//   Every 16-lane group (8 for d = 64) reads one whole key row with 16-byte loads (256 contiguous
//   bytes per row), so each cache element leaves HBM exactly once for all query heads of the
//   group. The group dots its 8 dims with each query head, sums across its lanes, and keeps an
//   online max-subtracted softmax per head in fp32. Groups are merged inside the workgroup and
//   the split's partial (running max m, running sum l, unnormalised output o) goes to the
//   workspace.
// Kernel 2 (combine): out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s with M = max_s m_s.
#include <math.h>

#include "common.hpp"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr int kTargetBlocks = 2048;  // split count aims at this many workgroups

__device__ __forceinline__ void merge(float& m, float& l, float* o, float m2, float l2,
                                      const float* o2, int n) {
  const float M = fmaxf(m, m2);
  const float a1 = (M == -INFINITY) ? 0.f : fast_exp2(m - M);
  const float a2 = (M == -INFINITY) ? 0.f : fast_exp2(m2 - M);
  l = l * a1 + l2 * a2;
  for (int i = 0; i < n; ++i) o[i] = o[i] * a1 + o2[i] * a2;
  m = M;
}

template <int D, int GC>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a, int head_chunks) {
  constexpr int LPK = D / 8;               // lanes per key row
  constexpr int SLOTS = kThreads / LPK;    // key rows in flight per workgroup step
  __shared__ float sm[4][GC], sl[4][GC];
  __shared__ float so[4][GC][D];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y / head_chunks;
  const int hc = blockIdx.y % head_chunks;
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int slot = tid / LPK;
  const int lc = tid % LPK;
  const int per = (a.Tkv + a.nsplit - 1) / a.nsplit;
  const int kb = split * per;
  const int ke = min(a.Tkv, kb + per);

  const uint16_t* __restrict__ Qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ Kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ Vp = static_cast<const uint16_t*>(a.v);

  float qv[GC][8], o[GC][8], m[GC], l[GC];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const int hi = hc * GC + g;
    u32x4 w = {0, 0, 0, 0};
    if (hi < G)
      w = *reinterpret_cast<const u32x4*>(Qp + (static_cast<int64_t>(b) * a.Hq + kvh * G + hi) * D +
                                          8 * lc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[g][2 * e] = bf16_lo(w[e]);
      qv[g][2 * e + 1] = bf16_hi(w[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
    m[g] = -INFINITY;
    l[g] = 0.f;
  }
  const float sl2 = a.scale * kLog2e;
  const int64_t kstride = static_cast<int64_t>(a.Hkv) * D;
  const int64_t base = (static_cast<int64_t>(b) * a.Tkv * a.Hkv + kvh) * D + 8 * lc;

#pragma unroll 2
  for (int key = kb + slot; key < ke; key += SLOTS) {
    const u32x4 kw = *reinterpret_cast<const u32x4*>(Kp + base + key * kstride);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(Vp + base + key * kstride);
    float kf[8], vf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf[2 * e] = bf16_lo(kw[e]);
      kf[2 * e + 1] = bf16_hi(kw[e]);
      vf[2 * e] = bf16_lo(vw[e]);
      vf[2 * e + 1] = bf16_hi(vw[e]);
    }
    float s[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(qv[g][e], kf[e], acc);
      s[g] = acc;
    }
#pragma unroll
    for (int off = LPK / 2; off > 0; off >>= 1)
#pragma unroll
      for (int g = 0; g < GC; ++g) s[g] += __shfl_xor(s[g], off);
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const float t = s[g] * sl2;
      const float mn = fmaxf(m[g], t);
      const float al = fast_exp2(m[g] - mn);
      const float p = fast_exp2(t - mn);
      l[g] = l[g] * al + p;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = fmaf(p, vf[e], o[g][e] * al);
      m[g] = mn;
    }
  }

  // merge the key slots of this wave (lanes lc, lc+LPK, ...)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const float m2 = __shfl_xor(m[g], off);
      const float l2 = __shfl_xor(l[g], off);
      float o2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[g][e], off);
      merge(m[g], l[g], o[g], m2, l2, o2, 8);
    }
  }
  if (lane < LPK) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      if (lane == 0) {
        sm[wave][g] = m[g];
        sl[wave][g] = l[g];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) so[wave][g][8 * lc + e] = o[g][e];
    }
  }
  __syncthreads();
  if (wave == 0 && lane < LPK) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float mm = sm[0][g], ll = sl[0][g];
      float oo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) oo[e] = so[0][g][8 * lc + e];
      for (int w = 1; w < 4; ++w) {
        float o2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o2[e] = so[w][g][8 * lc + e];
        merge(mm, ll, oo, sm[w][g], sl[w][g], o2, 8);
      }
      const int hi = hc * GC + g;
      if (hi < G) {
        const int64_t idx = (static_cast<int64_t>(b) * a.Hq + kvh * G + hi) * a.nsplit + split;
        float* wo = a.ws + idx * D + 8 * lc;
#pragma unroll
        for (int e = 0; e < 8; ++e) wo[e] = oo[e];
        if (lc == 0) {
          const int64_t nbh = static_cast<int64_t>(a.B) * a.Hq * a.nsplit;
          a.ws[nbh * D + idx] = mm;
          a.ws[nbh * D + nbh + idx] = ll;
        }
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ ws,
                                                           uint16_t* __restrict__ out, int nbh,
                                                           int nsplit) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  const int64_t ntot = static_cast<int64_t>(nbh) * nsplit;
  const float* wm = ws + ntot * D + static_cast<int64_t>(bh) * nsplit;
  const float* wl = ws + ntot * D + ntot + static_cast<int64_t>(bh) * nsplit;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, wm[s]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float w = (wm[s] == -INFINITY) ? 0.f : fast_exp2(wm[s] - M);
    num = fmaf(w, ws[(static_cast<int64_t>(bh) * nsplit + s) * D + d], num);
    den = fmaf(w, wl[s], den);
  }
  out[static_cast<int64_t>(bh) * D + d] = f32_to_bf16(num / den);
}

int head_chunk_size(int G) { return G >= 8 ? 8 : (G >= 4 ? 4 : (G >= 2 ? 2 : 1)); }

template <int D, int GC>
hipError_t launch_split(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int head_chunks = (G + GC - 1) / GC;
  dim3 grid(a.nsplit, a.Hkv * head_chunks, a.B);
  hipLaunchKernelGGL((decode_split_kernel<D, GC>), grid, dim3(kThreads), 0, s, a, head_chunks);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  hipError_t e;
  switch (head_chunk_size(G)) {
    case 8: e = launch_split<D, 8>(a, s); break;
    case 4: e = launch_split<D, 4>(a, s); break;
    case 2: e = launch_split<D, 2>(a, s); break;
    default: e = launch_split<D, 1>(a, s); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.B * a.Hq), dim3(D), 0, s, a.ws,
                     static_cast<uint16_t*>(a.out), a.B * a.Hq, a.nsplit);
  return hipGetLastError();
}

}  // namespace

int decode_num_splits(int B, int Tkv, int Hq, int Hkv, int d) {
  (void)d;
  const int G = Hq / Hkv;
  const int gc = head_chunk_size(G);
  const int64_t units = static_cast<int64_t>(B) * Hkv * ((G + gc - 1) / gc);
  int64_t s = (kTargetBlocks + units - 1) / units;
  const int64_t max_s = Tkv / 256 > 1 ? Tkv / 256 : 1;  // at least 256 keys per split
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

size_t decode_workspace_bytes(int B, int Tkv, int Hq, int Hkv, int d) {
  const int64_t S = decode_num_splits(B, Tkv, Hq, Hkv, d);
  return static_cast<size_t>(static_cast<int64_t>(B) * Hq * S * (d + 2)) * sizeof(float);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
