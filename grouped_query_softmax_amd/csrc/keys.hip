// keys.hip -- key preparation: QK-norm and rotary embedding of key rows, once per key.
//
// The course page ("Week 7. Attention", step 3) applies RMSNorm to q and k before their dot
// product and turns both by the rotary embedding. Queries are processed inside the attention
// kernels as they are loaded (each query row is read by one workgroup), but each key tile is
// staged by every workgroup of its key/value head; processing the keys once here, into the
// caller's buffer (typically the key cache), and running the attention with keys_prepared is
// the cheaper order on this chip. The arithmetic is the in-kernel one: fp32 from the bf16 row,
// x * w / sqrt(mean(x^2) + eps), then each pair (2i, 2i+1) turned by the table's angle at the
// key's position, rounded once to bf16.
//
// One key row of d bf16 is d/8 lanes holding 16 bytes each; the row's sum of squares is a DPP
// reduction over those lanes. Key j of a sequence sits at position pos0 + j.
#include "common.hpp"

namespace gqa {
namespace {

template <int D, bool NORM, bool ROPE>
__global__ __launch_bounds__(256) void prepare_keys_kernel(const uint16_t* __restrict__ k,
                                                           uint16_t* __restrict__ out,
                                                           int64_t rows, int T, int H,
                                                           const int32_t* cu, int nseq, int pos0,
                                                           const float* __restrict__ w,
                                                           float eps, const float* __restrict__ ct,
                                                           const float* __restrict__ st) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (256 / LPR) + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  const bool ok = row < rows;  // every lane takes part in the row reduction
  const int64_t r = ok ? row : rows - 1;
  u32x4 v = *reinterpret_cast<const u32x4*>(k + r * D + 8 * c);
  float x[8];
  unpack8(v, x);
  if constexpr (NORM) {
    const float inv = rms_inv(lane_group_sum<LPR>(sumsq8(v)), D, eps);
    norm8(x, inv, *reinterpret_cast<const f32x4*>(w + 8 * c),
          *reinterpret_cast<const f32x4*>(w + 8 * c + 4));
  }
  if constexpr (ROPE) {
    const int64_t tok = r / H;  // token row of the [rows / H, H, D] view
    int j;
    if (cu) {  // packed: position inside its sequence
      int lo = 0, hi = nseq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= tok) lo = mid; else hi = mid - 1;
      }
      j = static_cast<int>(tok - cu[lo]);
    } else {
      j = static_cast<int>(tok % T);
    }
    const int64_t ti = static_cast<int64_t>(pos0 + j) * (D / 2) + 4 * c;
    rope8(x, *reinterpret_cast<const f32x4*>(ct + ti), *reinterpret_cast<const f32x4*>(st + ti));
  }
  if (ok) *reinterpret_cast<u32x4*>(out + r * D + 8 * c) = pack8(x);
}

template <int D, bool NORM, bool ROPE>
hipError_t launch_d(const KeyPrepArgs& a, hipStream_t s) {
  constexpr int kRowsPerBlock = 256 / (D / 8);
  const int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((prepare_keys_kernel<D, NORM, ROPE>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, s, static_cast<const uint16_t*>(a.k),
                     static_cast<uint16_t*>(a.out), a.rows, a.T, a.H, a.cu, a.nseq, a.pos0, a.w,
                     a.eps, a.rope_cos, a.rope_sin);
  return hipGetLastError();
}

template <int D>
hipError_t launch_flags(const KeyPrepArgs& a, hipStream_t s) {
  const bool norm = a.w != nullptr, rope = a.rope_cos != nullptr;
  if (norm && rope) return launch_d<D, true, true>(a, s);
  if (norm) return launch_d<D, true, false>(a, s);
  if (rope) return launch_d<D, false, true>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prepare_keys(const KeyPrepArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_flags<64>(a, s);
    case 128: return launch_flags<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
