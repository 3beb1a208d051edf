// prefill_bf16.hip -- bf16 grouped-query attention forward on the gfx950 matrix cores.
//
// What is computed: for every query row, scores = scale * q.k over the visible keys of its
// group's key/value head (query head i reads head i / G: contiguous groups, GQA lab page
// "Transformer -- attention by hand: reducing only the key/value heads", steps 1 and 3), the
// row maximum subtracted before exponentiating (lab step 4), causal keys removed before the
// softmax (course page "Week 7. Attention", step 1), and the normalised weighted sum of value rows.
//
// How. One workgroup = 8 waves = one key/value head x one tile of 256 (position, head) columns;
// all G query heads of the group sit in the same workgroup, so each K/V tile is read from HBM
// into LDS once and consumed by every query head of the group.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: keys are the MFMA
//     rows and queries the columns, so each lane owns one query column and the softmax row
//     statistics are lane-local (one v_permlane32_swap with the partner lane l^32 per tile).
//   * The output is accumulated transposed as well, O^T += V^T P^T. P^T is the score accumulator
//     rounded to bf16 in place; the contraction order of keys is permuted to follow the
//     accumulator layout, and V is stored in LDS transposed ([d][keys]) in that same permuted key
//     order, so both MFMA operands are single 16-byte LDS reads.
//   * K/V tiles of 64 keys rotate through three LDS stages. Two groups of 4 waves share the
//     SIMDs and run half a step apart (ping-pong): while one group's waves issue the matrix-core
//     work of a tile, the other group's waves do the softmax of theirs on the vector ALUs.
//   * Online softmax in fp32 in the base-2 domain: x = s*scale*log2(e) - m in one FMA, p = 2^x.
//     The reference maximum m is only moved when a tile raises the row maximum by more than
//     kRescaleSlack (in log2 units); otherwise O and the running sum keep the old reference,
//     which is exact (the final O / l uses one reference throughout) and skips the O rescale.
//     p is then at most 2^kRescaleSlack, far inside fp32 and bf16 range.
//   * Causal: key tiles past the workgroup's last visible key are never loaded; tiles crossing
//     the diagonal are masked per element with bottom-right alignment. With a sliding window
//     (course page "Week 7. Attention", step 3) only the sink tiles and the tiles from the
//     window start of the workgroup's first row are visited, and the window edge is masked. For balance each
//     workgroup takes the query tile pair (i, n-1-i), so every workgroup does the same number of
//     key tiles.
//   * Launch order: key/value heads fastest, then query tiles, then batch items / packed
//     sequences. Consecutive workgroups are spread round-robin over the 8 XCDs, so with 8 key/
//     value heads each XCD L2 serves one head, and the workgroups running together on an XCD
//     stream the same head of the same sequence.
//   * The kernel assumes finite inputs: it is built without NaN semantics so row maxima of
//     matrix-core results compile to v_max3_f32 (infinities keep their meaning: masked scores
//     are -inf).
#include <math.h>

#include <type_traits>

#include "common.hpp"

namespace gqa {
namespace {

constexpr int kKT = 64;                // keys per tile
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr int kLdsAhead = 6;           // MFMA operand reads kept in flight
constexpr int kCols = 256;             // (position, head) columns per workgroup

// K/V tiles are read with raw buffer loads (kBufWord3): loads past the end of an item return
// zeros, which pads the last key tile without branches; tile offsets go in the range-checked
// VGPR offset.

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

// DQ: query/key head dim; DV: value columns a workgroup produces (DQ for grouped-query
// attention; a slice of the wider value row for grouped value attention).
template <int DQ, int DV>
struct PPCfg {
  static constexpr int kGroupThreads = 256;
  static constexpr int kChunks = DQ / 8;
  static constexpr int kKLoads = kKT * kChunks / kGroupThreads;  // 16-byte K loads per thread
  static constexpr int kVD = (kKT / 4) * DV / kGroupThreads;     // value columns per V item
  static constexpr int kKPitch = DQ * 2 + 16;
  static constexpr int kVPitch = kKT * 2 + 16;
  static constexpr int kKBytes = kKT * kKPitch;
  static constexpr int kVBytes = DV * kVPitch;
  static constexpr int kVBase = 3 * kKBytes;  // LDS: [K stage 0..2][V^T stage 0..2]
  static constexpr int kSmemBytes = 3 * (kKBytes + kVBytes);
  static_assert(kVD == 8 || kVD == 4, "V staging split");
  static_assert(kVBase < 65536 && 3 * kVBytes < 65536, "stage offsets fit LDS immediates");
};

template <int DQ, int DV, bool ROPE, bool NORM, bool KPROC>
__global__ __launch_bounds__(512) void prefill_pp_kernel(PrefillArgs a, int heads_per_wg,
                                                         int pos_per_wg, int head_tiles, int gz) {
  using C = PPCfg<DQ, DV>;
  constexpr int D = DQ;
  constexpr int NS = DQ / 16;   // MFMA k-steps over the head dim for the scores
  constexpr int NMT = DV / 32;  // 32-row value-column tiles of O^T
  constexpr int VD = C::kVD;
  constexpr int VW = VD / 2;
  // with QK-norm the key weights (read while staging K) and then the query weights (read in
  // each query tile's prologue) follow the stages in LDS
  constexpr int kNormOff = C::kSmemBytes;
  constexpr int kQNormOff = kNormOff + (KPROC ? 4 * DQ : 0);
  // epilogue: one region of 32 rows x 64 values (bf16) per wave; the 16-byte pad puts the 32
  // rows' 8-byte pieces in distinct bank pairs
  constexpr int kEpiPitch = 128 + 16;
  constexpr int kEpiBytes = 32 * kEpiPitch;
  constexpr bool kEpiBarrier = 8 * kEpiBytes > 3 * C::kKBytes;
  static_assert(4 * kEpiBytes <= 3 * C::kKBytes && 8 * kEpiBytes <= C::kSmemBytes,
                "epilogue regions must fit the K stages (group A) and the stages (both groups)");
  __shared__ __attribute__((aligned(16))) char smem[C::kSmemBytes + (NORM ? (KPROC ? 8 : 4) * DQ : 0)];

  const int gx = a.Hkv * head_tiles * a.vslices;
  const int lin = blockIdx.x;
  const int xi = lin % gx;
  const int rest = lin / gx;
  const int z = rest % gz;  // query tiles, then items
  const int item = rest / gz;
  const int vsl = xi % a.vslices;  // value slice
  const int kvh = xi / (head_tiles * a.vslices);
  const int ht = (xi / a.vslices) % head_tiles;
  int64_t q0, k0;
  int tq, tkv;
  a.items.get(item, q0, k0, tq, tkv);
  const int ntiles = (tq + pos_per_wg - 1) / pos_per_wg;
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
  const bool grp_a = wave < 4;
  const int gtid = tid & 255;  // thread index inside the group
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int off = tkv - tq;
  const float sl2 = a.scale * kLog2e;

  const uint16_t* __restrict__ Qp = static_cast<const uint16_t*>(a.q);
  uint16_t* __restrict__ Op = static_cast<uint16_t*>(a.out);
  const int row_bytes = a.Hkv * D * 2;  // between K rows
  const int vrow_bytes = a.v_row * 2;   // between V rows
  const uint16_t* kbase_ptr = static_cast<const uint16_t*>(a.k) + (k0 * a.Hkv + kvh) * D;
  const uint16_t* vbase_ptr = static_cast<const uint16_t*>(a.v) + k0 * a.v_row +
                              static_cast<int64_t>(kvh) * a.v_head + vsl * DV;

  // staging geometry of this thread inside its group (loop invariant)
  int k_src[C::kKLoads], k_dst[C::kKLoads];
#pragma unroll
  for (int i = 0; i < C::kKLoads; ++i) {
    const int idx = i * C::kGroupThreads + gtid;
    const int j = idx / C::kChunks, c = idx % C::kChunks;
    k_src[i] = j * row_bytes + 16 * c;
    k_dst[i] = j * C::kKPitch + 16 * c;
  }
  // V items: 4 keys x VD dims; the key group runs fastest across lanes so 16 lanes write one
  // V^T row (128 contiguous bytes) at once
  const int v_kg = gtid % 16, v_c = gtid / 16;
  const int v_src = 4 * v_kg * vrow_bytes + 2 * VD * v_c;
  const int v_dst = (VD * v_c) * C::kVPitch + 8 * vt_slot(v_kg);
  const int k_rd = n * C::kKPitch + 16 * hh;
  const int v_rd = n * C::kVPitch + 16 * hh;
  // QK-norm weights into LDS. Read from there, the query weights take no registers across the
  // prologue's table loads; 64 more live registers per lane would spill at this tile size.
  if constexpr (NORM) {
    if constexpr (KPROC) {
      if (tid < DQ / 4)
        lds_write<f32x4>(smem, kNormOff + 16 * tid,
                         *reinterpret_cast<const f32x4*>(a.kn_w + 4 * tid));
    }
    if (tid >= 64 && tid < 64 + DQ / 4)
      lds_write<f32x4>(smem, kQNormOff + 16 * (tid - 64),
                       *reinterpret_cast<const f32x4*>(a.qn_w + 4 * (tid - 64)));
    __syncthreads();
  }

  for (int tt = 0; tt < ntile_here; ++tt) {
    const int tile = tiles[tt];
    const int p0 = tile * pos_per_wg;

    const int col = wave * 32 + n;
    const int pl = col / heads_per_wg;
    const int hi = ht * heads_per_wg + col % heads_per_wg;
    const bool valid = pl < pos_per_wg && (p0 + pl) < tq && hi < G;
    const int pos = min(p0 + pl, tq - 1);
    const int hq = kvh * G + min(hi, G - 1);

    bf16x8 qf[NS];
    {
      const uint16_t* qrow = Qp + ((q0 + pos) * a.Hq + hq) * D + 8 * hh;
      u32x4 wq[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        wq[s] = valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * s) : u32x4{0, 0, 0, 0};
      // with QK-norm the table rows are loaded up front (in flight with the query), the chunks
      // below are then processed one at a time
      constexpr int kQTabs = NORM && ROPE ? NS : 1;
      [[maybe_unused]] f32x4 qc[kQTabs], qs[kQTabs];
      if constexpr (NORM && ROPE) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int ti = (pos + off) * (D / 2) + 8 * s + 4 * hh;
          qc[s] = *reinterpret_cast<const f32x4*>(a.rope_cos + ti);
          qs[s] = *reinterpret_cast<const f32x4*>(a.rope_sin + ti);
        }
      }
      [[maybe_unused]] float inv = 0.f;
      // this lane's query weights in LDS: a base computed here from the lane id (an opaque
      // instruction pair the compiler cannot move out of the loop), so that neither it nor the
      // per-chunk addresses (its constant offsets) occupy registers across the key loop
      [[maybe_unused]] int wbase = 0;
      if constexpr (NORM) {
        int l;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
        wbase = kQNormOff + 32 * (l >> 5);
      }
      if constexpr (NORM) {
        // the row's sum of squares: this lane's half plus its partner's (lane ^ 32), taken on the
        // packed words (bf16 squares are exact in fp32) so that no unpacked copy of the row
        // stays live until the per-chunk pass below
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // through a scalar: a bit cast of the vector element itself reads element 0 here
            const uint32_t x = wq[s][e];
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                                 __builtin_bit_cast(bf16x2, x), ss, false);
          }
        ss = pair_sum32(ss);
        inv = rms_inv(ss, D, a.norm_eps);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u32x4 w = wq[s];
        // query at position pos + off (the causal mask's alignment); pairs 8s + 4hh .. +3
        [[maybe_unused]] const int ti = (pos + off) * (D / 2) + 8 * s + 4 * hh;
        if constexpr (NORM) {
          float x[8];
          unpack8(w, x);
          norm8(x, inv, lds_read<f32x4>(smem, wbase + 64 * s),
                lds_read<f32x4>(smem, wbase + 64 * s + 16));
          if constexpr (ROPE) rope8(x, qc[s], qs[s]);
          w = pack8(x);
          // one chunk's weights in registers at a time
          __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (ROPE) {
          w = rope_chunk(w, *reinterpret_cast<const f32x4*>(a.rope_cos + ti),
                         *reinterpret_cast<const f32x4*>(a.rope_sin + ti));
        }
        qf[s] = __builtin_bit_cast(bf16x8, w);
      }
      // finish the query operands before anything of the tile loop is scheduled in between:
      // the norm's and rotation's temporaries then never overlap the loop's registers
      if constexpr (ROPE || NORM) __builtin_amdgcn_sched_barrier(0);
    }
    f32x16 acc_o[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[mt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int last = min(p0 + pos_per_wg, tq) - 1;
    const int kend = a.causal ? min(tkv, last + off + 1) : tkv;
    // Key tiles of this query tile: with a sliding window, the sink tiles [0, nst) and then the
    // window tiles from wt0 up; loop step t works on key tile ktile(t). Steps past the end map
    // past kend, where the loads return zeros.
    const int kt_end = (kend + kKT - 1) / kKT;
    int nst = 0, wt0 = 0;
    if (a.window > 0) {
      wt0 = max(0, p0 + off - a.window + 1) / kKT;
      nst = min((min(a.n_sink, kend) + kKT - 1) / kKT, wt0);
    }
    const int nkt = nst + (kt_end - wt0);
    auto ktile = [&](int t) { return t < nst ? t : t - nst + wt0; };
    const int nrec = (kend - 1) * row_bytes + D * 2;
    const int vnrec = (kend - 1) * vrow_bytes + DV * 2;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kbase_ptr), 0, nrec, kBufWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vbase_ptr), 0, vnrec, kBufWord3);

    // one staging register file per thread: group B stages K tiles, group A stages V tiles
    constexpr int kStageRegs = (4 * C::kKLoads > 4 * VW) ? 4 * C::kKLoads : 4 * VW;
    uint32_t stg[kStageRegs];
    // rotary embedding of the staged keys: key j of the item sits at position j; the tables are
    // read through a range-checked resource (rows past the table read as 0: those keys are the
    // zero padding of the last tile)
    constexpr int kRopeRegs = ROPE && KPROC ? C::kKLoads : 1;
    [[maybe_unused]] f32x4 rc[kRopeRegs], rs[kRopeRegs];
    [[maybe_unused]] __amdgpu_buffer_rsrc_t crs, srs;
    if constexpr (ROPE && KPROC) {
      const int tbytes = a.rope_rows * (D / 2) * 4;
      crs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.rope_cos), 0, tbytes,
                                              kBufWord3);
      srs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.rope_sin), 0, tbytes,
                                              kBufWord3);
    }
    auto load_k = [&](int t) {
      const int soff = ktile(t) * kKT * row_bytes;
#pragma unroll
      for (int i = 0; i < C::kKLoads; ++i) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(krs, k_src[i] + soff, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) stg[4 * i + e] = w[e];
      }
    };
    // the table rows of the keys staged next; issued at the start of a matrix phase so they
    // arrive by its end, where the keys are turned and written to LDS
    auto load_rope = [&](int t) {
      if constexpr (ROPE && KPROC) {
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
          const int idx = i * C::kGroupThreads + gtid;
          const int key = ktile(t) * kKT + idx / C::kChunks;
          const int toff = (key * (D / 2) + 4 * (idx % C::kChunks)) * 4;
          rc[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, toff, 0, 0));
          rs[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, toff, 0, 0));
        }
      }
    };
    auto store_k = [&](int stage) {
      char* base = smem + stage * C::kKBytes;
      [[maybe_unused]] float inv_k[C::kKLoads];
      if constexpr (NORM && KPROC) {
        // each key row is spread over kChunks consecutive lanes: sum their squares
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
          const float ss = lane_group_sum<C::kChunks>(
              sumsq8(u32x4{stg[4 * i], stg[4 * i + 1], stg[4 * i + 2], stg[4 * i + 3]}));
          inv_k[i] = rms_inv(ss, D, a.norm_eps);
        }
      }
#pragma unroll
      for (int i = 0; i < C::kKLoads; ++i) {
        u32x4 w = {stg[4 * i], stg[4 * i + 1], stg[4 * i + 2], stg[4 * i + 3]};
        if constexpr (NORM && KPROC) {
          float x[8];
          unpack8(w, x);
          // weights of this thread's pieces (piece gtid % kChunks of each row)
          const int woff = kNormOff + 32 * (gtid % C::kChunks);
          norm8(x, inv_k[i], lds_read<f32x4>(smem, woff), lds_read<f32x4>(smem, woff + 16));
          if constexpr (ROPE) rope8(x, rc[i], rs[i]);
          w = pack8(x);
        } else if constexpr (ROPE && KPROC) {
          w = rope_chunk(w, rc[i], rs[i]);
        }
        lds_write<u32x4>(base, k_dst[i], w);
      }
    };
    auto load_v = [&](int t) {
      const int soff = ktile(t) * kKT * vrow_bytes;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (VD == 8) {
          const u32x4 w =
              __builtin_amdgcn_raw_buffer_load_b128(vrs, v_src + r * vrow_bytes + soff, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) stg[VW * r + e] = w[e];
        } else {
          const u32x2 w =
              __builtin_amdgcn_raw_buffer_load_b64(vrs, v_src + r * vrow_bytes + soff, 0, 0);
          stg[VW * r] = w[0];
          stg[VW * r + 1] = w[1];
        }
      }
    };
    auto store_v = [&](int stage) {
      char* base = smem + C::kVBase + stage * C::kVBytes;
#pragma unroll
      for (int e = 0; e < VD; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 w;
        w[0] = __builtin_amdgcn_perm(stg[VW * 1 + (e >> 1)], stg[VW * 0 + (e >> 1)], sel);
        w[1] = __builtin_amdgcn_perm(stg[VW * 3 + (e >> 1)], stg[VW * 2 + (e >> 1)], sel);
        lds_write<u32x2>(base, v_dst + e * C::kVPitch, w);
      }
    };

    f32x16 sacc[2];
    bf16x8 pb[4];
    // M phase pieces: O += V(t-1) P(t-1) and S(t) = K(t) Q^T, operands read from LDS
    auto pv = [&](int t) {
      const char* sm = smem + C::kVBase + ((t + 2) % 3) * C::kVBytes;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep) {
          const bf16x8 vop = __builtin_bit_cast(
              bf16x8, lds_read<u32x4>(sm, v_rd + mt * 32 * C::kVPitch + 32 * kstep));
          acc_o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[kstep], acc_o[mt], 0, 0, 0);
        }
    };
    auto qk = [&](int t) {
      const char* sm = smem + (t % 3) * C::kKBytes;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 kop = __builtin_bit_cast(
              bf16x8, lds_read<u32x4>(sm, k_rd + h * 32 * C::kKPitch + 32 * s));
          sacc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[s], s == 0 ? f32x16{} : sacc[h],
                                                            0, 0, 0);
        }
    };
    // Ask the scheduler to keep kLdsAhead operand reads in flight ahead of the MFMAs that use
    // them instead of waiting on each read right before its MFMA.
    auto sched_stream = [&](auto nmfma_tag) {
      constexpr int NM = decltype(nmfma_tag)::value;
      constexpr int AHEAD = kLdsAhead < NM ? kLdsAhead : NM;
      __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
      for (int i = 0; i < NM - AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
    };
    auto m_full = [&](int t) {  // 1 <= t < nkt
      pv(t);
      qk(t);
      sched_stream(std::integral_constant<int, NMT * 4 + 2 * NS>{});
    };
    auto m_first = [&]() {
      qk(0);
      sched_stream(std::integral_constant<int, 2 * NS>{});
    };
    auto m_last = [&](int t) {
      pv(t);
      sched_stream(std::integral_constant<int, NMT * 4>{});
    };
    // V phase: softmax of S(t) into P(t)
    auto v_phase = [&](int t) {
      const int kbase = ktile(t) * kKT;
      const bool below_window =
          a.window > 0 && kbase < last + off - a.window + 1 && kbase + kKT > a.n_sink;
      const bool need_mask =
          (kbase + kKT > tkv) || (a.causal && kbase + kKT - 1 > p0 + off) || below_window;
      if (need_mask) {
        const int lim = a.causal ? min(tkv - 1, pos + off) : tkv - 1;
        // key of element (h, i) is kbase + 4*hh + c(h, i) with a compile-time c; compare c
        // against per-lane remainders so no per-element offsets stay live across tiles. The key
        // is visible if it is at most lim and (inside the window or a sink key).
        const int rem = lim - kbase - 4 * hh;
        const int rlo = a.window > 0 ? pos + off - a.window + 1 - kbase - 4 * hh : -kKT;
        const int rsk = a.n_sink - kbase - 4 * hh;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int c = h * 32 + (i >> 2) * 8 + (i & 3);
            sacc[h][i] = (c <= rem && (c >= rlo || c < rsk)) ? sacc[h][i] : -INFINITY;
          }
      }
      float r3[11];
#pragma unroll
      for (int g = 0; g < 10; ++g) {
        const int i0 = 3 * g, i1 = 3 * g + 1, i2 = 3 * g + 2;
        r3[g] = fmaxf(fmaxf(sacc[i0 >> 4][i0 & 15], sacc[i1 >> 4][i1 & 15]), sacc[i2 >> 4][i2 & 15]);
      }
      r3[10] = fmaxf(sacc[1][14], sacc[1][15]);
      const float r4a = fmaxf(fmaxf(r3[0], r3[1]), r3[2]);
      const float r4b = fmaxf(fmaxf(r3[3], r3[4]), r3[5]);
      const float r4c = fmaxf(fmaxf(r3[6], r3[7]), r3[8]);
      const float r4d = fmaxf(r3[9], r3[10]);
      float tmax = fmaxf(fmaxf(r4a, r4b), fmaxf(r4c, r4d));
      tmax = pair_max32(tmax) * sl2;
      // The new reference is chosen without a branch, so the exponentials follow the maximum in
      // one block; only the rare rescale of O and of the running sum sits in a branch, after
      // them. Lanes that keep their reference keep their sums (alpha = 1; their m may still be
      // -inf, since with a sliding window a row can see nothing in the first tiles).
      const bool move = tmax > m_run + kRescaleSlack;
      const float m_old = m_run;
      m_run = move ? tmax : m_run;
      const float mref = m_run == -INFINITY ? 0.f : m_run;
      // the row sum in four independent partial sums (a chain of 16 dependent dot products
      // would pace the phase)
      float psum4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float& psum = psum4[2 * h + h2];
          uint32_t pw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0v = fast_exp2(fmaf(sacc[h][8 * h2 + 2 * e], sl2, -mref));
            const float p1v = fast_exp2(fmaf(sacc[h][8 * h2 + 2 * e + 1], sl2, -mref));
            pw[e] = pack_bf16x2(p0v, p1v);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[e]),
                                                   __builtin_bit_cast(bf16x2, 0x3f803f80u), psum,
                                                   false);
          const u32x4 w = {pw[0], pw[1], pw[2], pw[3]};
          pb[2 * h + h2] = __builtin_bit_cast(bf16x8, w);
        }
      if (__any(move)) {
        const float alpha = move ? fast_exp2(m_old - m_run) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc_o[mt][i] *= alpha;
      }
      l_run += (psum4[0] + psum4[1]) + (psum4[2] + psum4[3]);
    };

    __syncthreads();  // the previous query tile's readers are done with every stage
    if (grp_a) {
      load_v(0);
      store_v(0);
      load_v(1);
    } else {
      load_k(0);
      load_rope(0);
      store_k(0);
      load_k(1);
    }
    __syncthreads();
    // Staging runs at the end of each group's matrix phase, which has slack, so waiting for
    // the global loads does not lengthen the vector-ALU (softmax) phase that paces the loop.
    // A writes V(t+1) in its M(t) at half-step 2t (V(t-2) is no longer read after 2t-1);
    // B writes K(t+1) in its M(t) at half-step 2t+1 (read first by A at 2t+2).
    // t = 0: only the scores of tile 0
    if (grp_a) {
      m_first();
      store_v(1);
      load_v(2);
    }
    __syncthreads();
    if (grp_a) {
      v_phase(0);
    } else {
      load_rope(1);
      m_first();
      store_k(1);
      load_k(2);
    }
    __syncthreads();
    for (int t = 1; t < nkt; ++t) {
      const int st_next = (t + 1) % 3;
      if (grp_a) {
        m_full(t);
        store_v(st_next);
        load_v(t + 2);
      } else {
        v_phase(t - 1);
      }
      __syncthreads();
      if (grp_a) {
        v_phase(t);
      } else {
        load_rope(t + 1);
        m_full(t);
        store_k(st_next);
        load_k(t + 2);
      }
      __syncthreads();
    }
    // Epilogue: O / l rounded to bf16. A lane holds 4 consecutive values of its column per
    // accumulator group, so a direct store would put 16 bytes into each of 32 rows per
    // instruction. Instead each wave passes its 32 columns through its own LDS region, 64 values
    // at a time, and reads them back as 16-byte pieces of rows: every store instruction then
    // writes 8 whole 128-byte row segments.
    auto epilogue = [&]() __attribute__((always_inline)) {
      const float l_tot = pair_sum32(l_run);
      const float inv = 1.f / l_tot;
      if (a.lse && valid && hh == 0 && vsl == 0)  // log-sum-exp of the scaled scores, natural log
        a.lse[(q0 + pos) * a.Hq + hq] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
      char* tb = smem + wave * kEpiBytes;
      // position (-1: no output) and head of the columns whose row pieces this lane moves, from
      // the lanes that own those columns
      int rpos[4], rhq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 8 * j + (lane >> 3);
        rpos[j] = __shfl(valid ? pos : -1, r);
        rhq[j] = __shfl(hq, r);
      }
#pragma unroll
      for (int h = 0; h < DV / 64; ++h) {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int mt = 2 * h + m2;
            u32x2 w;
            w[0] = pack_bf16x2(acc_o[mt][4 * g4 + 0] * inv, acc_o[mt][4 * g4 + 1] * inv);
            w[1] = pack_bf16x2(acc_o[mt][4 * g4 + 2] * inv, acc_o[mt][4 * g4 + 3] * inv);
            lds_write<u32x2>(tb, n * kEpiPitch + 2 * (32 * m2 + 8 * g4 + 4 * hh), w);
          }
        asm volatile("" ::: "memory");  // one wave's LDS accesses run in program order
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 8 * j + (lane >> 3);  // the wave's column whose row piece this lane moves
          const u32x4 x = lds_read<u32x4>(tb, r * kEpiPitch + 16 * (lane & 7));
          if (rpos[j] >= 0) {
            uint16_t* orow = Op + (q0 + rpos[j]) * a.o_row +
                             static_cast<int64_t>(rhq[j]) * a.o_head + vsl * DV;
            // non-temporal: nothing here reads the output back; kept out of the caches the
            // stores retire sooner, and the next query tile's first loads, which share the
            // memory counter with them, wait less
            __builtin_nontemporal_store(x,
                                        reinterpret_cast<u32x4*>(orow + 64 * h + 8 * (lane & 7)));
          }
        }
        asm volatile("" ::: "memory");
      }
    };
    // t = nkt: only O += V(nkt-1) P(nkt-1). Group A's epilogue regions lie in the K stages, which
    // nobody reads any more; group B's follow them and, when the K stages are too small for
    // eight regions, reach into the V stages, so B then waits until all of its waves are done
    // with them.
    if (grp_a) {
      m_last(nkt);
    } else {
      v_phase(nkt - 1);
    }
    __syncthreads();
    if (!grp_a) {
      m_last(nkt);
    } else {
      epilogue();
    }
    if constexpr (kEpiBarrier) __syncthreads();
    if (!grp_a) epilogue();
  }
}

template <int DQ, int DV, bool ROPE, bool NORM, bool KPROC>
hipError_t launch_pp(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int heads_per_wg = G < kCols ? G : kCols;
  const int pos_per_wg = kCols / heads_per_wg;
  const int head_tiles = (G + heads_per_wg - 1) / heads_per_wg;
  const int ntiles = (a.max_tq + pos_per_wg - 1) / pos_per_wg;
  const int gz = a.causal ? (ntiles + 1) / 2 : ntiles;
  const dim3 grid(a.Hkv * head_tiles * a.vslices * a.nitems * gz);
  hipLaunchKernelGGL((prefill_pp_kernel<DQ, DV, ROPE, NORM, KPROC>), grid, dim3(512), 0, s, a,
                     heads_per_wg, pos_per_wg, head_tiles, gz);
  return hipGetLastError();
}

template <int D, bool KPROC>
hipError_t launch_processed(const PrefillArgs& a, hipStream_t s) {
  const bool rope = a.rope_cos != nullptr, norm = a.qn_w != nullptr;
  if (norm && rope) return launch_pp<D, D, true, true, KPROC>(a, s);
  if (norm) return launch_pp<D, D, false, true, KPROC>(a, s);
  return launch_pp<D, D, true, false, KPROC>(a, s);
}

template <int D>
hipError_t launch_same_width(const PrefillArgs& a, hipStream_t s) {
  if (!a.rope_cos && !a.qn_w) return launch_pp<D, D, false, false, false>(a, s);
  // keys_prepared: the keys were normalised / turned beforehand; only the queries are here
  return a.keys_prepared ? launch_processed<D, false>(a, s) : launch_processed<D, true>(a, s);
}

}  // namespace

int prefill_bf16_cols() { return kCols; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  if (a.d == 64 && a.dv == 64) return launch_same_width<64>(a, s);
  if (a.d == 128 && a.dv == 128) return launch_same_width<128>(a, s);
  if (a.d == 64 && a.dv == 128 && !a.rope_cos && !a.qn_w)
    return launch_pp<64, 128, false, false, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gqa
