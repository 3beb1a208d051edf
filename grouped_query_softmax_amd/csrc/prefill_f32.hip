// prefill_f32.hip -- fp32 grouped-query attention forward on the vector ALUs.
//
// The fp32 path serves small head dims and exactness checks, where the matrix cores' bf16
// rounding is not wanted. Structure (same decomposition as the bf16 matrix-core kernel):
//   * a workgroup owns one key/value head `kvh` of one batch item and a tile of query positions,
//     and takes ALL query heads of that group (query head i reads key/value head i / G, the
//     contiguous grouping of the GQA lab page, steps 1 and 3); its 256 threads are
//     (position, head) rows, so each K/V tile is loaded into LDS once and read by every head;
//   * each thread keeps its query row and output accumulator in registers and runs the
//     max-subtracted softmax online: for every key, m' = max(m, s), the running sum and output
//     are rescaled by e^(m - m'), and the key adds e^(s - m') (lab step 4: subtract the maximum
//     before exponentiating; course page "Week 7. Attention", step 1: scale 1/sqrt(d) and causal
//     keys removed before the softmax).
// Exponentials use the hardware base-2 exponential on (s - m') * log2(e), with s already scaled,
// which keeps the argument error proportional to |s - m'| rather than to |s|.
#include <math.h>

#include "common.hpp"

namespace gqa {
namespace {

constexpr int kRows = 256;  // (position, head) rows per workgroup
constexpr int kKeys = 32;   // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void prefill_f32_kernel(PrefillArgs a, int heads_per_wg,
                                                            int pos_per_wg, int head_tiles) {
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];
  const int tile = blockIdx.x;
  const int kvh = blockIdx.y / head_tiles;
  const int ht = blockIdx.y % head_tiles;
  const int item = blockIdx.z;
  int64_t q0, k0;
  int tq, tkv;
  a.items.get(item, q0, k0, tq, tkv);
  const int p0 = tile * pos_per_wg;
  if (p0 >= tq) return;  // whole workgroup: tile past this item's length

  const int G = a.Hq / a.Hkv;
  const int r = threadIdx.x;
  const int pl = r / heads_per_wg;
  const int hi = ht * heads_per_wg + r % heads_per_wg;
  const int pos = p0 + pl;
  const bool active = pl < pos_per_wg && pos < tq && hi < G;
  const int hq = kvh * G + hi;
  const int off = tkv - tq;  // bottom-right alignment of the causal mask

  const float* __restrict__ Q = static_cast<const float*>(a.q);
  const float* __restrict__ K = static_cast<const float*>(a.k);
  const float* __restrict__ V = static_cast<const float*>(a.v);
  float* __restrict__ O = static_cast<float*>(a.out);

  float qv[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = active ? Q[((q0 + pos) * a.Hq + hq) * D + c] : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int last = min(p0 + pos_per_wg, tq) - 1;
  const int kmax = a.causal ? min(tkv, last + off + 1) : tkv;  // keys any row here can see
  const int my_kmax = a.causal ? min(tkv, pos + off + 1) : tkv;

  for (int kt = 0; kt < kmax; kt += kKeys) {
    __syncthreads();
    for (int i = threadIdx.x; i < kKeys * D; i += kRows) {
      const int j = i / D, c = i % D;
      const int key = kt + j;
      const bool in = key < kmax;
      const int64_t src = ((k0 + key) * a.Hkv + kvh) * D + c;
      ks[j][c] = in ? K[src] : 0.f;
      vs[j][c] = in ? V[src] : 0.f;
    }
    __syncthreads();
    if (active) {
      const int jn = min(kKeys, my_kmax - kt);
      for (int j = 0; j < jn; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) dot = fmaf(qv[c], ks[j][c], dot);
        const float s = dot * a.scale;
        const float mn = fmaxf(m, s);
        const float alpha = fast_exp2((m - mn) * kLog2e);
        const float p = fast_exp2((s - mn) * kLog2e);
        l = l * alpha + p;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = fmaf(p, vs[j][c], o[c] * alpha);
        m = mn;
      }
    }
  }
  if (active) {
#pragma unroll
    for (int c = 0; c < D; ++c) O[((q0 + pos) * a.Hq + hq) * D + c] = o[c] / l;
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int heads_per_wg = G < kRows ? G : kRows;
  const int pos_per_wg = kRows / heads_per_wg;
  const int head_tiles = (G + heads_per_wg - 1) / heads_per_wg;
  const int ntiles = (a.max_tq + pos_per_wg - 1) / pos_per_wg;
  dim3 grid(ntiles, a.Hkv * head_tiles, a.nitems);
  hipLaunchKernelGGL(prefill_f32_kernel<D>, grid, dim3(kRows), 0, s, a, heads_per_wg, pos_per_wg,
                     head_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_d<16>(a, s);
    case 32: return launch_d<32>(a, s);
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
