// prefill_bf16.hip -- bf16 grouped-query attention forward on the gfx950 matrix cores.
//
// What is computed: for every query row, scores = scale * q.k over the visible keys of its
// group's key/value head (query head i reads head i / G: contiguous groups, GQA lab page
// "Transformer -- attention by hand: reducing only the key/value heads", steps 1 and 3), the
// row maximum subtracted before exponentiating (lab step 4), causal keys removed before the
// softmax (course page "Week 7. Attention", step 1), and the normalised weighted sum of value rows.
//
// How. One workgroup = NW waves = one key/value head x one tile of NC = NW*32*QT (position, head)
// columns; all G query heads of the group sit in the same workgroup, so each K/V tile is read
// from HBM into LDS once and consumed by every query head of the group.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: keys are the MFMA
//     rows and queries the columns, so each lane owns one query column and the softmax row
//     statistics are lane-local (one exchange with the partner lane l^32 per tile).
//   * The output is accumulated transposed as well, O^T += V^T P^T. P^T is the score accumulator
//     rounded to bf16 in place; the contraction order of keys is permuted to follow the
//     accumulator layout, and V is stored in LDS transposed ([d][keys]) in that same permuted key
//     order, so both MFMA operands are single 16-byte LDS reads.
//   * K/V tiles of 64 keys are double-buffered in LDS: the global loads of tile t+1 are issued
//     into registers before tile t is computed and written to the other buffer afterwards, so one
//     barrier per tile suffices and HBM latency hides behind the matrix work.
//   * Online softmax in fp32 in the base-2 domain: x = s*scale*log2(e) - m in one FMA, p = 2^x.
//     The reference maximum m is only moved when a tile raises the row maximum by more than
//     kRescaleSlack (in log2 units); otherwise O and the running sum keep the old reference,
//     which is exact (the final O / l uses one reference throughout) and skips the O rescale.
//     p is then at most 2^kRescaleSlack, far inside fp32 and bf16 range.
//   * Causal: key tiles past the workgroup's last visible key are never loaded; tiles crossing
//     the diagonal are masked per element with bottom-right alignment. For balance each
//     workgroup takes the query tile pair (i, n-1-i), so every workgroup does the same number of
//     key tiles.
//   * Grid: key/value heads fastest, so consecutive workgroups -- spread round-robin over the 8
//     XCDs by the dispatcher -- keep one key/value head per XCD L2 when Hkv * items is 8.
#include <math.h>

#include "common.hpp"

namespace gqa {
namespace {

#ifndef GQA_PREFILL_ORDER
#define GQA_PREFILL_ORDER 1
#endif
#ifndef GQA_PREFILL_NW
#define GQA_PREFILL_NW 8  // waves per workgroup for d = 128
#endif
#ifndef GQA_PREFILL_QT
#define GQA_PREFILL_QT 1  // 32-column query tiles per wave for d = 128
#endif

constexpr int kKT = 64;                // keys per tile
constexpr float kRescaleSlack = 8.0f;  // log2 units

// Buffer resource word 3 for raw (unformatted) buffer loads on CDNA; loads at or beyond
// num_records bytes return zeros, which pads the last key tile without branches.
constexpr int kBufWord3 = 0x00020000;

template <int D, int NW, int QT>
struct Cfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kCols = NW * 32 * QT;
  static constexpr int kChunks = D / 8;                     // 16-byte chunks per key row
  static constexpr int kKLoads = kKT * kChunks / kThreads;  // 16-byte K loads per thread
  static constexpr int kVD = (kKT / 4) * D / kThreads;      // d values per V staging item
  // LDS pitches: one 16-byte pad per row makes 16 consecutive rows read at the same column
  // land in 16 distinct bank groups, and keeps every read address lane base + immediate.
  static constexpr int kKPitch = D * 2 + 16;        // bytes per key row of the K tile
  static constexpr int kVPitch = kKT * 2 + 16;      // bytes per d row of the V^T tile
  static constexpr int kKBytes = kKT * kKPitch;
  static constexpr int kVBytes = D * kVPitch;
  static constexpr int kStageBytes = kKBytes + kVBytes;
  static_assert(kKLoads >= 1 && kKT * kChunks % kThreads == 0, "K staging split");
  static_assert(kVD == 8 || kVD == 4 || kVD == 2, "V staging split");
};

// V^T rows hold the 64 keys of a tile permuted inside each group of 16: key 8a + 4h + r
// (a, h in {0,1}, r < 4) sits at position 8h + 4a + r. The 8 keys one lane feeds into one MFMA
// k-step (accumulator rows 4h..4h+3 and 8+4h..8+4h+3 of a 16-key step) are then 16 contiguous
// bytes. Returns the 4-key slot (8 bytes) of the group of keys 4kg .. 4kg+3.
__device__ __forceinline__ int vt_slot(int kg) {
  const int g16 = kg >> 2, a = (kg >> 1) & 1, h = kg & 1;
  return 4 * g16 + 2 * h + a;
}

template <typename T>
__device__ __forceinline__ T lds_read(const char* base, int byte_off) {
  return *reinterpret_cast<const T*>(base + byte_off);
}
template <typename T>
__device__ __forceinline__ void lds_write(char* base, int byte_off, T v) {
  *reinterpret_cast<T*>(base + byte_off) = v;
}

template <int D, int NW, int QT>
__global__ __launch_bounds__(NW * 64, 2) void prefill_bf16_kernel(PrefillArgs a, int heads_per_wg,
                                                                  int pos_per_wg, int head_tiles,
                                                                  int gz) {
  using C = Cfg<D, NW, QT>;
  constexpr int NS = D / 16;   // MFMA k-steps over d for the scores
  constexpr int NMT = D / 32;  // 32-row d tiles of O^T
  constexpr int VD = C::kVD;   // V staging: 4 keys x VD dims per thread
  constexpr int VW = VD / 2;   // dwords per key of one V item
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kStageBytes];

  // 1-D grid: (key/value head, head tile) fastest, then the order of GQA_PREFILL_ORDER
  const int gx = a.Hkv * head_tiles;
  const int lin = blockIdx.x;
  const int xi = lin % gx;
  const int rest = lin / gx;
#if GQA_PREFILL_ORDER == 0
  const int item = rest % a.nitems;  // items, then query tiles
  const int z = rest / a.nitems;
#else
  const int z = rest % gz;           // query tiles, then items
  const int item = rest / gz;
#endif
  const int kvh = xi / head_tiles;
  const int ht = xi % head_tiles;
  int64_t q0, k0;
  int tq, tkv;
  a.items.get(item, q0, k0, tq, tkv);
  const int ntiles = (tq + pos_per_wg - 1) / pos_per_wg;
  // causal: this workgroup takes the query tiles (ntiles-1-z, z); otherwise tile z alone
  int tiles[2];
  int ntile_here;
  if (a.causal) {
    if (2 * z >= ntiles) return;
    tiles[0] = ntiles - 1 - z;  // heavy tile first
    tiles[1] = z;
    ntile_here = (tiles[1] != tiles[0]) ? 2 : 1;
  } else {
    if (z >= ntiles) return;
    tiles[0] = z;
    ntile_here = 1;
  }

  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;   // query column inside a 32-column MFMA tile
  const int hh = lane >> 5;  // which half of the k-slots / accumulator rows this lane holds
  const int off = tkv - tq;  // bottom-right causal alignment
  const float sl2 = a.scale * kLog2e;

  const uint16_t* __restrict__ Qp = static_cast<const uint16_t*>(a.q);
  uint16_t* __restrict__ Op = static_cast<uint16_t*>(a.out);
  const int row_bytes = a.Hkv * D * 2;  // bytes between consecutive keys of one head
  const uint16_t* kbase_ptr = static_cast<const uint16_t*>(a.k) + (k0 * a.Hkv + kvh) * D;
  const uint16_t* vbase_ptr = static_cast<const uint16_t*>(a.v) + (k0 * a.Hkv + kvh) * D;

  // per-thread staging geometry (loop invariant)
  int k_src[C::kKLoads], k_dst[C::kKLoads];
#pragma unroll
  for (int i = 0; i < C::kKLoads; ++i) {
    const int idx = i * C::kThreads + tid;
    const int j = idx / C::kChunks, c = idx % C::kChunks;
    k_src[i] = j * row_bytes + 16 * c;
    k_dst[i] = j * C::kKPitch + 16 * c;
  }
  constexpr int NPR = D / VD;  // V items per key row
  const int v_c = tid % NPR, v_kg = tid / NPR;
  const int v_src = 4 * v_kg * row_bytes + 2 * VD * v_c;
  const int v_dst = C::kKBytes + (VD * v_c) * C::kVPitch + 8 * vt_slot(v_kg);
  // per-lane MFMA operand read bases
  const int k_rd = n * C::kKPitch + 16 * hh;
  const int v_rd = C::kKBytes + n * C::kVPitch + 16 * hh;

  for (int tt = 0; tt < ntile_here; ++tt) {
    const int tile = tiles[tt];
    const int p0 = tile * pos_per_wg;

    // ---- per-lane column geometry ----
    int pos[QT], hq[QT];
    bool valid[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int col = (wave * QT + qt) * 32 + n;
      const int pl = col / heads_per_wg;
      const int hi = ht * heads_per_wg + col % heads_per_wg;
      valid[qt] = pl < pos_per_wg && (p0 + pl) < tq && hi < G;
      pos[qt] = min(p0 + pl, tq - 1);
      hq[qt] = kvh * G + min(hi, G - 1);
    }

    // ---- Q^T operands: lane holds q[col][16*s + 8*hh .. +8] for each k-step s ----
    bf16x8 qf[QT][NS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const uint16_t* qrow = Qp + ((q0 + pos[qt]) * a.Hq + hq[qt]) * D + 8 * hh;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u32x4 w = valid[qt] ? *reinterpret_cast<const u32x4*>(qrow + 16 * s) : u32x4{0, 0, 0, 0};
        qf[qt][s] = __builtin_bit_cast(bf16x8, w);
      }
    }

    f32x16 acc_o[QT][NMT];
    float m_run[QT], l_run[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[qt][mt][i] = 0.f;
      m_run[qt] = -INFINITY;
      l_run[qt] = 0.f;
    }

    const int last = min(p0 + pos_per_wg, tq) - 1;
    const int kend = a.causal ? min(tkv, last + off + 1) : tkv;  // keys this tile needs
    const int nkt = (kend + kKT - 1) / kKT;
    // K/V rows past kend read as zeros
    const int nrec = (kend - 1) * row_bytes + D * 2;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kbase_ptr), 0, nrec, kBufWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vbase_ptr), 0, nrec, kBufWord3);

    u32x4 kreg[C::kKLoads];
    uint32_t vreg[4][VW];
    auto load_tile = [&](int kt) {
      const int soff = kt * kKT * row_bytes;
#pragma unroll
      for (int i = 0; i < C::kKLoads; ++i)
        kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, k_src[i], soff, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (VD == 8) {
          const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(vrs, v_src + r * row_bytes, soff, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) vreg[r][e] = w[e];
        } else if constexpr (VD == 4) {
          const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(vrs, v_src + r * row_bytes, soff, 0);
          vreg[r][0] = w[0];
          vreg[r][1] = w[1];
        } else {
          vreg[r][0] = __builtin_amdgcn_raw_buffer_load_b32(vrs, v_src + r * row_bytes, soff, 0);
        }
      }
    };
    auto store_tile = [&](int stage) {
      char* base = smem + stage * C::kStageBytes;
#pragma unroll
      for (int i = 0; i < C::kKLoads; ++i) lds_write<u32x4>(base, k_dst[i], kreg[i]);
#pragma unroll
      for (int e = 0; e < VD; ++e) {
        // keys 4kg..4kg+3 at dim VD*c+e: the low or high halves of the dwords holding that dim
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 w;
        w[0] = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
        w[1] = __builtin_amdgcn_perm(vreg[3][e >> 1], vreg[2][e >> 1], sel);
        lds_write<u32x2>(base, v_dst + e * C::kVPitch, w);
      }
    };

    __syncthreads();  // the previous query tile's readers are done with both stages
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
      const int stage = kt & 1;
      const int kbase = kt * kKT;
      if (kt + 1 < nkt) load_tile(kt + 1);
      const char* sm = smem + stage * C::kStageBytes;

      // ---- S^T = K Q^T: 2 sub-tiles of 32 keys x QT query tiles ----
      f32x16 sacc[QT][2];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 kop = __builtin_bit_cast(
              bf16x8, lds_read<u32x4>(sm, k_rd + t * 32 * C::kKPitch + 32 * s));
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            sacc[qt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                kop, qf[qt][s], s == 0 ? f32x16{} : sacc[qt][t], 0, 0, 0);
        }

      // ---- mask the tiles that cross the causal diagonal or the end of the keys ----
      const bool need_mask = (kbase + kKT > tkv) || (a.causal && kbase + kKT - 1 > p0 + off);
      if (need_mask) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int lim = a.causal ? min(tkv - 1, pos[qt] + off) : tkv - 1;  // last visible key
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kbase + t * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
              sacc[qt][t][i] = key <= lim ? sacc[qt][t][i] : -INFINITY;
            }
        }
      }

      // ---- online softmax (per query tile) ----
      bf16x8 pb[QT][4];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        // row max of the 32 scores this lane holds: a tree of three-input maxima
        float r3[11];
#pragma unroll
        for (int g = 0; g < 10; ++g) {
          const int i0 = 3 * g, i1 = 3 * g + 1, i2 = 3 * g + 2;
          r3[g] = fmaxf(fmaxf(sacc[qt][i0 >> 4][i0 & 15], sacc[qt][i1 >> 4][i1 & 15]),
                        sacc[qt][i2 >> 4][i2 & 15]);
        }
        r3[10] = fmaxf(sacc[qt][1][14], sacc[qt][1][15]);
        const float r4a = fmaxf(fmaxf(r3[0], r3[1]), r3[2]);
        const float r4b = fmaxf(fmaxf(r3[3], r3[4]), r3[5]);
        const float r4c = fmaxf(fmaxf(r3[6], r3[7]), r3[8]);
        const float r4d = fmaxf(r3[9], r3[10]);
        float tmax = fmaxf(fmaxf(r4a, r4b), fmaxf(r4c, r4d));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * sl2;  // both halves of the column agree
        // move the reference max only when it grows by more than the slack (or is unset)
        const bool move = tmax > m_run[qt] + kRescaleSlack;
        if (__any(move)) {
          const float m_new = move ? tmax : m_run[qt];
          const float alpha = fast_exp2(m_run[qt] - m_new);
          l_run[qt] *= alpha;
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc_o[qt][mt][i] *= alpha;
          m_run[qt] = m_new;
        }
        const float mref = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            uint32_t pw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0v = fast_exp2(fmaf(sacc[qt][t][8 * h2 + 2 * e], sl2, -mref));
              const float p1v = fast_exp2(fmaf(sacc[qt][t][8 * h2 + 2 * e + 1], sl2, -mref));
              pw[e] = pack_bf16x2(p0v, p1v);
            }
            // the row sum adds the rounded weights the MFMA consumes, so the weights used for
            // the output are exactly normalised by it
#pragma unroll
            for (int e = 0; e < 4; ++e)
              psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[e]),
                                                     __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                                     psum, false);
            const u32x4 w = {pw[0], pw[1], pw[2], pw[3]};
            pb[qt][2 * t + h2] = __builtin_bit_cast(bf16x8, w);
          }
        l_run[qt] += psum;
      }

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep) {  // 16-key steps: (sub-tile, half)
          const bf16x8 vop = __builtin_bit_cast(
              bf16x8, lds_read<u32x4>(sm, v_rd + mt * 32 * C::kVPitch + 32 * kstep));
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            acc_o[qt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[qt][kstep],
                                                                    acc_o[qt][mt], 0, 0, 0);
        }

      if (kt + 1 < nkt) store_tile(stage ^ 1);
      __syncthreads();
    }

    // ---- epilogue: combine the lane pair's sums, normalise, round, store ----
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float inv = 1.f / (l_run[qt] + __shfl_xor(l_run[qt], 32));
      if (valid[qt]) {
        uint16_t* orow = Op + ((q0 + pos[qt]) * a.Hq + hq[qt]) * D;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int dd = mt * 32 + g4 * 8 + hh * 4;
            u32x2 w;
            w[0] = pack_bf16x2(acc_o[qt][mt][4 * g4 + 0] * inv, acc_o[qt][mt][4 * g4 + 1] * inv);
            w[1] = pack_bf16x2(acc_o[qt][mt][4 * g4 + 2] * inv, acc_o[qt][mt][4 * g4 + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + dd) = w;
          }
      }
    }
  }
}

template <int D, int NW, int QT>
hipError_t launch_cfg(const PrefillArgs& a, hipStream_t s) {
  constexpr int kCols = Cfg<D, NW, QT>::kCols;
  const int G = a.Hq / a.Hkv;
  const int heads_per_wg = G < kCols ? G : kCols;
  const int pos_per_wg = kCols / heads_per_wg;
  const int head_tiles = (G + heads_per_wg - 1) / heads_per_wg;
  const int ntiles = (a.max_tq + pos_per_wg - 1) / pos_per_wg;
  const int gz = a.causal ? (ntiles + 1) / 2 : ntiles;
  const dim3 grid(a.Hkv * head_tiles * a.nitems * gz);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, QT>), grid, dim3(NW * 64), 0, s, a, heads_per_wg,
                     pos_per_wg, head_tiles, gz);
  return hipGetLastError();
}

}  // namespace

// Columns per workgroup of the launched configurations (the host validates the grid with it).
int prefill_bf16_cols() { return Cfg<128, GQA_PREFILL_NW, GQA_PREFILL_QT>::kCols; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_cfg<64, GQA_PREFILL_NW, GQA_PREFILL_QT>(a, s);
    case 128: return launch_cfg<128, GQA_PREFILL_NW, GQA_PREFILL_QT>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
