// fold.hip -- key/value head folding: mean over each contiguous group of H/g heads.
//
// GQA lab page ("Transformer -- attention by hand: reducing only the key/value heads"), step 2:
// the key/value heads inside a group are averaged position by position, leaving g heads; the
// group of a head is the contiguous block of step 1. This is a pure streaming kernel (HBM bound):
// each thread owns 16 bytes of one output row, reads the s = H/g matching 16-byte pieces of the
// input heads, sums them in fp32 in head order, divides by s in fp32 and rounds once. The output
// is written with non-temporal stores: nothing reads it back in this kernel, and kept out of the
// caches it leaves them to the streamed input (one 32-head to 8-head fold of 336 MB: 61 -> 48 us).
#include "common.hpp"

namespace gqa {
namespace {

template <typename E>
__global__ __launch_bounds__(256) void fold_kernel(const typename E::T* __restrict__ src,
                                                   typename E::T* __restrict__ dst, int64_t nvec,
                                                   int H, int g, int d) {
  constexpr int VEC = 16 / E::kBytes;
  const int s = H / g;
  const int dv = d / VEC;
  const float fs = static_cast<float>(s);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int cv = static_cast<int>(i % dv);
    const int64_t row = i / dv;  // (b*T + t) * g + j
    const int j = static_cast<int>(row % g);
    const int64_t bt = row / g;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    const typename E::T* base = src + (bt * H + static_cast<int64_t>(j) * s) * d + cv * VEC;
    for (int h = 0; h < s; ++h) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(base + static_cast<int64_t>(h) * d);
      if constexpr (E::kBytes == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16_lo(w[e]);
          acc[2 * e + 1] += bf16_hi(w[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
      }
    }
    u32x4 o;
    if constexpr (E::kBytes == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e] / fs, acc[2 * e + 1] / fs);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(acc[e] / fs);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst + row * d + cv * VEC));
  }
}

}  // namespace

hipError_t launch_fold(const void* src, void* dst, int64_t BT, int H, int g, int d, int is_bf16,
                       hipStream_t s) {
  const int vec = is_bf16 ? 8 : 4;
  const int64_t nvec = BT * g * (d / vec);
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 4096) blocks = 4096;  // grid-stride beyond this (16 workgroups per CU)
  if (blocks < 1) blocks = 1;
  if (is_bf16)
    hipLaunchKernelGGL(fold_kernel<BF16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), nvec, H, g,
                       d);
  else
    hipLaunchKernelGGL(fold_kernel<F32>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const float*>(src), static_cast<float*>(dst), nvec, H, g, d);
  return hipGetLastError();
}

}  // namespace gqa
