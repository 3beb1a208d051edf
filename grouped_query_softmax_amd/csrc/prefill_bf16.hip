// prefill_bf16.hip -- bf16 grouped-query attention forward on the gfx950 matrix cores.
//
// What is computed: for every query row, scores = scale * q.k over the visible keys of its
// group's key/value head (query head i reads head i / G: contiguous groups, GQA lab page
// "Transformer -- attention by hand: reducing only the key/value heads", steps 1 and 3), the
// row maximum subtracted before exponentiating (lab step 4), causal keys removed before the
// softmax (course page "Week 7. Attention", step 1), and the normalised weighted sum of value rows.
//
// How (one workgroup = 4 waves = one key/value head x a tile of 128 (position, head) columns):
//   * All G query heads of a group are packed into the workgroup's columns, so every K/V tile is
//     read from HBM into LDS once and consumed by every query head of the group -- the reuse that
//     grouped-query attention exists for.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: keys are the
//     MFMA rows, queries the columns, so each lane owns one query column and the softmax row
//     statistics are lane-local (one exchange with the partner lane l^32 per tile).
//   * Output is accumulated transposed as well, O^T += V^T P^T: P^T comes straight from the score
//     accumulators rounded to bf16 (the key order inside the contraction is permuted to match the
//     accumulator layout), V^T is read from an LDS copy of the V tile stored transposed.
//   * Online softmax in fp32 in the base-2 domain: scale*log2(e) is folded into one multiply,
//     m' = max(m, tile max), O and the running sum are rescaled by 2^(m - m').
//   * Causal: key tiles beyond the workgroup's last visible key are never loaded; the tiles that
//     cross the diagonal are masked per element with bottom-right alignment.
//   * Launch order: query tiles with the most keys first (tile index reversed, and slowest in the
//     grid), key/value heads fastest, so consecutive workgroups -- which the dispatcher spreads
//     round-robin over the 8 XCDs -- keep one key/value head per XCD L2 when Hkv * items is 8.
#include <math.h>

#include "common.hpp"

namespace gqa {
namespace {

constexpr int kWaves = 4;
constexpr int kCols = 32 * kWaves;  // (position, head) columns per workgroup
constexpr int kKT = 64;             // keys per tile

// K tile in LDS: [64 keys][D] bf16, 16-byte chunks XOR-swizzled by key so that 16 lanes reading
// the same chunk of 16 consecutive keys hit 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int key, int chunk) {
  if constexpr (D == 128) return chunk ^ (key & 15);
  else return chunk ^ ((key >> 1) & 7);
}
// V^T tile in LDS: [D][64 keys] bf16 (128 B per d row), 8-byte groups of 4 keys XOR-swizzled by d
// so that 32 lanes reading the same key group of 32 consecutive d rows are conflict-free.
__device__ __forceinline__ int v_swz(int d, int kg) { return kg ^ ((d >> 1) & 15); }

template <int D>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(PrefillArgs a, int heads_per_wg,
                                                           int pos_per_wg, int head_tiles,
                                                           int ntiles) {
  constexpr int NS = D / 16;   // MFMA k-steps over d for the scores
  constexpr int NMT = D / 32;  // 32-row d tiles of O^T
  __shared__ __attribute__((aligned(16))) uint16_t ks[kKT * D];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * kKT];

  const int kvh = blockIdx.x / head_tiles;
  const int ht = blockIdx.x % head_tiles;
  const int item = blockIdx.y;
  const int tile = ntiles - 1 - static_cast<int>(blockIdx.z);  // heaviest first
  int64_t q0, k0;
  int tq, tkv;
  a.items.get(item, q0, k0, tq, tkv);
  const int p0 = tile * pos_per_wg;
  if (p0 >= tq) return;

  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;   // query column inside the wave's MFMA tile
  const int hh = lane >> 5;  // which half of the k-slots / accumulator rows this lane holds
  const int col = wave * 32 + n;
  const int pl = col / heads_per_wg;
  const int hi = ht * heads_per_wg + col % heads_per_wg;
  const bool valid = pl < pos_per_wg && (p0 + pl) < tq && hi < G;
  const int pos = min(p0 + pl, tq - 1);  // clamped for masking of dead columns
  const int hq = kvh * G + min(hi, G - 1);
  const int off = tkv - tq;

  const uint16_t* __restrict__ Qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ Kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ Vp = static_cast<const uint16_t*>(a.v);
  uint16_t* __restrict__ Op = static_cast<uint16_t*>(a.out);

  // Q^T operand: lane holds q[col][16*s + 8*hh .. +8] for each k-step s.
  bf16x8 qf[NS];
  {
    const uint16_t* qrow = Qp + ((q0 + pos) * a.Hq + hq) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 w = valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * s) : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 acc_o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_o[mt][i] = 0.f;
  float m_run = -INFINITY;  // running max (log2 domain), shared by the lane pair
  float l_run = 0.f;        // this lane's part of the running sum
  const float sl2 = a.scale * kLog2e;

  const int last = min(p0 + pos_per_wg, tq) - 1;
  const int kend = a.causal ? min(tkv, last + off + 1) : tkv;  // keys this workgroup needs
  const int nkt = (kend + kKT - 1) / kKT;

  for (int kt = 0; kt < nkt; ++kt) {
    const int kbase = kt * kKT;
    __syncthreads();  // previous tile fully consumed
    // ---- stage K tile (row-major, swizzled) ----
    {
      constexpr int CH = D / 8;             // 16-byte chunks per key row
      constexpr int RPI = 256 / CH;         // rows per pass
#pragma unroll
      for (int it = 0; it < kKT / RPI; ++it) {
        const int j = it * RPI + tid / CH;
        const int c = tid % CH;
        const int key = kbase + j;
        u32x4 w = {0, 0, 0, 0};
        if (key < kend)
          w = *reinterpret_cast<const u32x4*>(Kp + ((k0 + key) * a.Hkv + kvh) * D + 8 * c);
        *reinterpret_cast<u32x4*>(&ks[j * D + 8 * k_swz<D>(j, c)]) = w;
      }
    }
    // ---- stage V tile transposed: thread takes 4 keys x 8 d, writes 8 rows of 4 keys ----
    {
      constexpr int CH = D / 8;
      constexpr int ITEMS = CH * (kKT / 4);
#pragma unroll
      for (int it = 0; it < (ITEMS + 255) / 256; ++it) {
        const int item2 = it * 256 + tid;
        if (item2 < ITEMS) {
          const int c = item2 % CH;
          const int kg = item2 / CH;
          u32x4 x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kbase + 4 * kg + r;
            x[r] = key < kend ? *reinterpret_cast<const u32x4*>(
                                    Vp + ((k0 + key) * a.Hkv + kvh) * D + 8 * c)
                              : u32x4{0, 0, 0, 0};
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            u32x2 w;
            w[0] = __builtin_amdgcn_perm(x[1][e >> 1], x[0][e >> 1], sel);
            w[1] = __builtin_amdgcn_perm(x[3][e >> 1], x[2][e >> 1], sel);
            const int dd = 8 * c + e;
            *reinterpret_cast<u32x2*>(&vt[dd * kKT + 4 * v_swz(dd, kg)]) = w;
          }
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for the 2 sub-tiles of 32 keys ----
    f32x16 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[t][i] = 0.f;
      const int j = t * 32 + n;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(&ks[j * D + 8 * k_swz<D>(j, 2 * s + hh)]);
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), qf[s],
                                                          sacc[t], 0, 0, 0);
      }
    }
    // ---- scale, mask, tile max ----
    const bool need_mask = (kbase + kKT > tkv) || (a.causal && kbase + kKT - 1 > p0 + off);
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = sacc[t][i] * sl2;
        if (need_mask) {
          const int key = kbase + t * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
          const bool vis = key < tkv && (!a.causal || key <= pos + off);
          x = vis ? x : -INFINITY;
        }
        sacc[t][i] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    // ---- P = 2^(x - m'), running sum, rescale O ----
    bf16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0v = fast_exp2(sacc[t][8 * h2 + 2 * e] - m_new);
          const float p1v = fast_exp2(sacc[t][8 * h2 + 2 * e + 1] - m_new);
          psum += p0v + p1v;
          w[e] = pack_bf16x2(p0v, p1v);
        }
        pb[2 * t + h2] = __builtin_bit_cast(bf16x8, w);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[mt][i] *= alpha;
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int dd = mt * 32 + n;
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2) {  // 16-key steps: (sub-tile t, half h2)
        const int kga = ks2 * 4 + hh;        // 4-key group index of the first 4 keys
        u32x4 w;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(&vt[dd * kKT + 4 * v_swz(dd, kga)]);
        const u32x2 hi2 = *reinterpret_cast<const u32x2*>(&vt[dd * kKT + 4 * v_swz(dd, kga + 2)]);
        w[0] = lo[0];
        w[1] = lo[1];
        w[2] = hi2[0];
        w[3] = hi2[1];
        acc_o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                            pb[ks2], acc_o[mt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: combine the lane pair's sums, normalise, round, store ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (valid) {
    uint16_t* orow = Op + ((q0 + pos) * a.Hq + hq) * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dd = mt * 32 + g4 * 8 + hh * 4;
        u32x2 w;
        w[0] = pack_bf16x2(acc_o[mt][4 * g4 + 0] / l_tot, acc_o[mt][4 * g4 + 1] / l_tot);
        w[1] = pack_bf16x2(acc_o[mt][4 * g4 + 2] / l_tot, acc_o[mt][4 * g4 + 3] / l_tot);
        *reinterpret_cast<u32x2*>(orow + dd) = w;
      }
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int heads_per_wg = G < kCols ? G : kCols;
  const int pos_per_wg = kCols / heads_per_wg;
  const int head_tiles = (G + heads_per_wg - 1) / heads_per_wg;
  const int ntiles = (a.max_tq + pos_per_wg - 1) / pos_per_wg;
  dim3 grid(a.Hkv * head_tiles, a.nitems, ntiles);
  hipLaunchKernelGGL(prefill_bf16_kernel<D>, grid, dim3(256), 0, s, a, heads_per_wg, pos_per_wg,
                     head_tiles, ntiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
