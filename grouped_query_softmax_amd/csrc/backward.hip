// backward.hip -- gradients of grouped-query attention (bf16 in, bf16 gradients, fp32 math).
//
// From the chain rule for one query row (softmax probabilities P recomputed from the forward's
// row log-sum-exp L):  P_j = exp(s_j - L), dP_j = dout.v_j, D = dout.out (= sum_j P_j dP_j),
// dS_j = P_j (dP_j - D);  dq = scale sum_j dS_j k_j,  dk_j = scale sum_i dS_ij q_i,
// dv_j = sum_i P_ij dout_i. The key/value heads are shared by G query heads (copies of one
// head), so their gradients are the sum over the G heads of the group (K3 notes, section 4,
// backward: the backward of a replication is a sum over the copies).
//
// Three kernels:
//   * bwd_rowdot: D = dout.out per query row (fp32).
//   * bwd_dkdv: one workgroup of 4 waves per (sequence, key/value head, 64-key tile; causal: a
//     pair of tiles, heavy and light). Waves 0 and 2 own the tile's first 32 keys, waves 1 and 3
//     the other 32, each with the keys' K^T, V^T operands and its own dK^T, dV^T accumulators in
//     registers. The 32-row chunks of (q, dout, L, D) of all query heads of the group stream
//     through two LDS stages two at a time (the next pair's loads in flight): waves 0, 1 take the
//     first chunk of a pair, waves 2, 3 the second, so every chunk read from memory feeds 64
//     keys. Waves 2, 3 hand their partial sums to waves 0, 1 through LDS at the end of a tile.
//     Per chunk: S = Q K^T and dP = dO V^T with the keys as MFMA columns, P and dS in fp32,
//     then dV^T += dO^T P and dK^T += Q^T dS with dO^T / Q^T read transposed from LDS
//     (ds_read_b64_tr_b16) in the key order of the accumulators.
//   * bwd_dq: one workgroup of 4 waves per (sequence, key/value head, 128 (position, head) query
//     columns; causal: a pair of such tiles, heavy and light); 32-key chunks of K and V stream
//     through two LDS buffers with the next chunk's loads in flight. Per chunk: S^T = K Q^T and
//     dP^T = V dO^T with the queries as columns, dS^T, then dQ^T += K^T dS^T.
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
#include <math.h>

#include "common.hpp"

namespace gqa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32;  // rows of a streamed chunk
// LDS layout of a [rows][D] chunk: rows of 2*D bytes, the 16-byte pieces of row r stored at
// piece index c ^ swz(r). The two readers of a chunk -- 16-byte reads down a column of rows (an
// MFMA operand with the rows as its M index) and transposing 8-byte reads of 4 rows x 64 bytes --
// then both hit 64 distinct banks per pass, which no plain row padding achieves for both.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
}

template <int D>
struct BwdCfg {
  static constexpr int kPitch = 2 * D;             // bytes per LDS row of a [rows][D] chunk
  static constexpr int kChunkBytes = kRows * kPitch;
  static constexpr int kNS = D / 16;               // MFMA k-steps over d
  static constexpr int kNMT = D / 32;              // 32-row d tiles
  static constexpr int kLoadsPerRow = D / 8;       // 16-byte pieces per row
  static constexpr int kChunkLoads = kRows * kLoadsPerRow / kThreads;  // per thread
};

// The A operand (8 bf16) of an MFMA whose rows are the d values base .. base+31 and whose k
// values are the 16 chunk rows 16 ks .. 16 ks + 15 in the accumulator order
// (rows 16ks+4hh+0..3, then 16ks+8+4hh+0..3), read transposed from a [rows][D] LDS chunk.
template <int D>
__device__ __forceinline__ int chunk_off(int r, int c) {  // byte offset of piece c of row r
  return r * BwdCfg<D>::kPitch + 16 * (c ^ swz<D>(r));
}

template <int D>
__device__ __forceinline__ bf16x8 tr_operand(char* chunk, int lane, int base, int ks) {
  const int hh = lane >> 5, sub = (lane >> 4) & 1, j = lane & 15;
  const int row = 16 * ks + 4 * hh + (j >> 2);
  const int c = base / 8 + 2 * sub + ((j & 3) >> 1);  // 16-byte piece; 8-byte half (j & 1)
  const u32x2 lo = lds_read_tr(chunk, chunk_off<D>(row, c) + 8 * (j & 1));
  const u32x2 hi = lds_read_tr(chunk, chunk_off<D>(row + 8, c) + 8 * (j & 1));
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Packs accumulator values i = 8 ks .. 8 ks + 7 (rows 16ks+4hh+0..3 and 16ks+8+4hh+0..3 of the
// lane's column) into a B operand.
__device__ __forceinline__ bf16x8 pack_rows(const float* x, int ks) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[8 * ks + 2 * e], x[8 * ks + 2 * e + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

// D = dout . out per row; rows = B*Tq*Hq, one 64-lane wave per 4 rows (16 lanes per row).
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t* __restrict__ out,
                                                         const uint16_t* __restrict__ dout,
                                                         float* __restrict__ Dr, int64_t rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t row = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(out + row * D + 8 * c);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dout + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_lo(o[e]), bf16_lo(g[e]), acc);
      acc = fmaf(bf16_hi(o[e]), bf16_hi(g[e]), acc);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < rows && c == 0) Dr[row] = acc;
}


// WIN: a sliding window (with sinks) is on; the plain kernels carry none of its tests.
template <int D, bool WIN>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(BwdArgs a, int tile_wgs) {
  using C = BwdCfg<D>;
  constexpr int NS = C::kNS, NMT = C::kNMT;
  constexpr int kSlotBytes = 2 * C::kChunkBytes + 2 * kRows * 4;  // q, dout, L, D of a chunk
  constexpr int kStageBytes = 2 * kSlotBytes;                     // the two items of a step
  constexpr int kRedBytes = 2 * 2 * 32 * D * 4;                   // two waves' dK^T, dV^T
  constexpr int kSmem = 2 * kStageBytes > kRedBytes ? 2 * kStageBytes : kRedBytes;
  constexpr int kMatPieces = kRows * C::kLoadsPerRow;             // 16-byte pieces per matrix
  constexpr int kPieces = 2 * 2 * kMatPieces / kThreads;          // per thread and step
  static_assert(kMatPieces % kThreads == 0, "a piece index decides its matrix uniformly");
  __shared__ __attribute__((aligned(16))) char smem[kSmem];

  // key/value heads fastest: consecutive workgroups go round-robin to the XCDs, so with 8 heads
  // each XCD's L2 serves one head, whose query chunks its workgroups read in the same order
  const int lin = blockIdx.x;
  const int kvh = lin % a.Hkv;
  const int z = (lin / a.Hkv) % tile_wgs;
  const int b = lin / (tile_wgs * a.Hkv);  // batch item or packed sequence
  int64_t q0, k0;
  int tq, tkv;
  a.items.get(b, q0, k0, tq, tkv);
  const int key_tiles = (tkv + 63) / 64;
  if (z >= (a.causal ? (key_tiles + 1) / 2 : key_tiles)) return;  // past this item's keys
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave & 1;    // which 32 keys of the 64-key tile
  const int slot = wave >> 1;  // which item of each step (waves 0, 1: the first; 2, 3: the second)
  const int n = lane & 31, hh = lane >> 5;
  const int off = tkv - tq;
  const float sl2 = a.scale * kLog2e;
  const int W = WIN ? a.window : 0;

  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const uint16_t* GO = static_cast<const uint16_t*>(a.dout);
  // this sequence's q, dout, L and D (each below 2 GiB: checked by the entry point)
  const int64_t qe0 = q0 * a.Hq;
  const int qbytes = tq * a.Hq * D * 2, lbytes = tq * a.Hq * 4;
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Q + qe0 * D), 0, qbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(GO + qe0 * D), 0, qbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.lse + qe0), 0, lbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(a.Drow + qe0, 0, lbytes,
                                                                       kBufWord3);

  // causal: a workgroup takes the key tile pair (z, key_tiles-1-z), equal work per pair
  int tiles[2];
  int ntile_here = 1;
  tiles[0] = z;
  if (a.causal) {
    tiles[1] = key_tiles - 1 - z;
    ntile_here = tiles[1] != tiles[0] ? 2 : 1;
  }

  for (int tt = 0; tt < ntile_here; ++tt) {
    const int kb0 = tiles[tt] * 64;
    const int kfirst = kb0 + 32 * kh;  // first key of this wave
    const int key = kfirst + n;        // this lane's key column
    const bool key_ok = key < tkv;

    bf16x8 kop[NS], vop[NS];
    {
      const int64_t kr = ((k0 + (key_ok ? key : 0)) * a.Hkv + kvh) * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 wk = key_ok ? *reinterpret_cast<const u32x4*>(K + kr + 16 * s + 8 * hh)
                                : u32x4{0, 0, 0, 0};
        const u32x4 wv = key_ok ? *reinterpret_cast<const u32x4*>(V + kr + 16 * s + 8 * hh)
                                : u32x4{0, 0, 0, 0};
        kop[s] = __builtin_bit_cast(bf16x8, wk);
        vop[s] = __builtin_bit_cast(bf16x8, wv);
      }
    }
    f32x16 dk[NMT], dv[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dk[mt][i] = dv[mt][i] = 0.f;

    // items: (32-row chunk from the first row that can see the tile's first key, query head of
    // the group), chunks from the last one down and heads inner, so that every workgroup walks
    // the rows in the same order; step s holds items 2s (waves 0, 1) and 2s+1 (waves 2, 3)
    // With a sliding window (course page "Week 7. Attention", step 3) the rows end at the last
    // one whose window still reaches the tile's last key, unless the tile holds sink keys.
    const int qstart = a.causal ? max(0, kb0 - off) / kRows * kRows : 0;
    const int qlast = (WIN && kb0 >= a.n_sink) ? min(tq - 1, kb0 + 63 + W - 1 - off) : tq - 1;
    const int nchunk = qstart <= qlast ? (qlast - qstart) / kRows + 1 : 0;
    const int nitems = G * nchunk;
    const int nsteps = (nitems + 1) / 2;

    // the next step's loads: two chunks of q and dout (kPieces 16-byte pieces per thread), and
    // L and D of their rows (threads 0..63). Buffer loads with the range check doing the
    // padding: rows past the end get an offset past the buffer and read zeros.
    u32x4 pr_[kPieces];
    float pL = 0.f, pD = 0.f;
    bool pvalid = false;
    auto load = [&](int st) {
      int soff[2], srow[2], nrows[2];  // per slot: element offset / row index of the chunk's
                                       // first row (head h), rows present
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const int it = 2 * st + sl;
        const int h = it % G, ci = nchunk - 1 - it / G;
        const int p0 = qstart + ci * kRows;
        const bool ok = it < nitems;
        srow[sl] = ok ? p0 * a.Hq + kvh * G + h : 0;
        soff[sl] = srow[sl] * D;
        nrows[sl] = ok ? min(kRows, tq - p0) : 0;
      }
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        constexpr int kSlotPieces = 2 * kMatPieces;
        const int sl = (i * kThreads) / kSlotPieces;           // the same for the whole workgroup
        const int mat = ((i * kThreads) / kMatPieces) & 1;     // 0: q, 1: dout
        const int pc = (i * kThreads) % kMatPieces + tid;
        const int r = pc / C::kLoadsPerRow, c = pc % C::kLoadsPerRow;
        const unsigned vo =
            r < nrows[sl] ? static_cast<unsigned>(soff[sl] + r * a.Hq * D + 8 * c) * 2u : kOutside;
        pr_[i] = __builtin_amdgcn_raw_buffer_load_b128(mat ? grs : qrs, vo, 0, 0);
      }
      if (tid < 2 * kRows) {
        const int sl = tid / kRows, r = tid % kRows;
        pvalid = r < nrows[sl];
        const unsigned vo = pvalid ? static_cast<unsigned>(srow[sl] + r * a.Hq) * 4u : kOutside;
        pL = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, vo, 0, 0));
        pD = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(drs, vo, 0, 0));
      }
    };
    auto store = [&](int stage) {
      char* base = smem + stage * kStageBytes;
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        const int sl = (i * kThreads) / (2 * kMatPieces);
        const int mat = ((i * kThreads) / kMatPieces) & 1;
        const int pc = (i * kThreads) % kMatPieces + tid;
        const int r = pc / C::kLoadsPerRow, c = pc % C::kLoadsPerRow;
        *reinterpret_cast<u32x4*>(base + sl * kSlotBytes + mat * C::kChunkBytes +
                                  chunk_off<D>(r, c)) = pr_[i];
      }
      if (tid < 2 * kRows) {
        const int sl = tid / kRows, r = tid % kRows;
        float* ld = reinterpret_cast<float*>(base + sl * kSlotBytes + 2 * C::kChunkBytes);
        ld[r] = pvalid ? pL * kLog2e : INFINITY;  // rows past the end: P = 0
        ld[kRows + r] = pD;
      }
    };

    __syncthreads();  // the previous tile's reduction is done with the LDS
    if (nsteps > 0) {
      load(0);
      store(0);
    }
    // nothing in flight from here on (the K/V operands included), so that the loop below waits
    // only for its own loads
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      if (st + 1 < nsteps) load(st + 1);  // in flight during this step
      const int it = 2 * st + slot;
      const int ci = nchunk - 1 - it / G;
      const int qc = qstart + ci * kRows;
      // a chunk whose last row cannot see this wave's first key, or whose first row's window
      // starts past this wave's keys (none of them a sink), contributes nothing
      const bool work = it < nitems && (!a.causal || qc + kRows - 1 + off >= kfirst) &&
                        (!WIN || kfirst < a.n_sink || kfirst + 31 > qc + off - W);
      if (work) {
        char* sq = smem + (st & 1) * kStageBytes + slot * kSlotBytes;
        char* sg = sq + C::kChunkBytes;
        const float* sl = reinterpret_cast<const float*>(sg + C::kChunkBytes);
        const float* sd = sl + kRows;
        f32x16 s_acc = {}, p_acc = {};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 qa = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(sq + chunk_off<D>(n, 2 * s + hh)));
          const bf16x8 ga = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(sg + chunk_off<D>(n, 2 * s + hh)));
          s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kop[s], s_acc, 0, 0, 0);
          p_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vop[s], p_acc, 0, 0, 0);
        }
        float lrow[16], drow[16], pr[16], ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = (i >> 2) * 8 + 4 * hh + (i & 3);
          lrow[i] = sl[r];
          drow[i] = sd[r];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int p = qc + (i >> 2) * 8 + 4 * hh + (i & 3);
          const bool vis = key_ok && (!a.causal || key <= p + off) &&
                           (!WIN || key > p + off - W || key < a.n_sink);
          const float e = fast_exp2(fmaf(s_acc[i], sl2, -lrow[i]));
          pr[i] = vis ? e : 0.f;
          ds[i] = pr[i] * (p_acc[i] - drow[i]);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 pb = pack_rows(pr, ks);
          const bf16x8 db = pack_rows(ds, ks);
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) {
            dv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(sg, lane, 32 * mt, ks),
                                                             pb, dv[mt], 0, 0, 0);
            dk[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(sq, lane, 32 * mt, ks),
                                                             db, dk[mt], 0, 0, 0);
          }
        }
      }
      // the other stage was last read in step st-1, before the previous barrier
      if (st + 1 < nsteps) store((st + 1) & 1);
      __syncthreads();
    }

    // waves 2, 3 hand their partial dK^T, dV^T to waves 0, 1 (same keys), which write them
    float* red = reinterpret_cast<float*>(smem);
    if (slot == 1) {
      float* base = red + kh * 2 * 32 * D;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          base[(mt * 16 + i) * 64 + lane] = dk[mt][i];
          base[32 * D + (mt * 16 + i) * 64 + lane] = dv[mt][i];
        }
    }
    __syncthreads();
    if (slot == 0) {
      const float* base = red + kh * 2 * 32 * D;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          dk[mt][i] += base[(mt * 16 + i) * 64 + lane];
          dv[mt][i] += base[32 * D + (mt * 16 + i) * 64 + lane];
        }
      if (key_ok) {
        uint16_t* DK = static_cast<uint16_t*>(a.dk);
        uint16_t* DV = static_cast<uint16_t*>(a.dv);
        const int64_t orow = ((k0 + key) * a.Hkv + kvh) * D;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int dd = mt * 32 + g4 * 8 + hh * 4;
            u32x2 wk, wv;
            wk[0] = pack_bf16x2(dk[mt][4 * g4] * a.scale, dk[mt][4 * g4 + 1] * a.scale);
            wk[1] = pack_bf16x2(dk[mt][4 * g4 + 2] * a.scale, dk[mt][4 * g4 + 3] * a.scale);
            wv[0] = pack_bf16x2(dv[mt][4 * g4], dv[mt][4 * g4 + 1]);
            wv[1] = pack_bf16x2(dv[mt][4 * g4 + 2], dv[mt][4 * g4 + 3]);
            *reinterpret_cast<u32x2*>(DK + orow + dd) = wk;
            *reinterpret_cast<u32x2*>(DV + orow + dd) = wv;
          }
      }
    }
  }
}

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdArgs a, int pos_per_wg,
                                                          int heads_per_wg, int head_tiles,
                                                          int gz) {
  using C = BwdCfg<D>;
  constexpr int NS = C::kNS, NMT = C::kNMT;
  __shared__ __attribute__((aligned(16))) char smem[4 * C::kChunkBytes];  // 2 x (K, V) chunks

  // key/value heads fastest (one head per XCD L2 with 8 heads: its K/V chunks are shared there)
  const int lin = blockIdx.x;
  const int kvh = lin % a.Hkv;
  const int rest = lin / a.Hkv;
  const int z = rest % gz;
  const int ht = (rest / gz) % head_tiles;
  const int b = rest / (gz * head_tiles);  // batch item or packed sequence
  int64_t q0, k0;
  int tq, tkv;
  a.items.get(b, q0, k0, tq, tkv);
  const int pos_tiles = (tq + pos_per_wg - 1) / pos_per_wg;
  if (a.causal ? 2 * z >= pos_tiles : z >= pos_tiles) return;  // past this item's rows
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int off = tkv - tq;
  const float sl2 = a.scale * kLog2e;
  const int W = WIN ? a.window : 0;
  // causal: each workgroup takes the query tile pair (pos_tiles-1-z, z), equal work per pair
  int tiles[2];
  int ntile_here;
  if (a.causal) {
    tiles[0] = pos_tiles - 1 - z;
    tiles[1] = z;
    ntile_here = tiles[1] != tiles[0] ? 2 : 1;
  } else {
    tiles[0] = z;
    ntile_here = 1;
  }

  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const uint16_t* GO = static_cast<const uint16_t*>(a.dout);
  // this sequence's K and V (below 2 GiB each: checked by the entry point)
  const int64_t ke0 = k0 * a.Hkv * D;
  const int kbytes = tkv * a.Hkv * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(K + ke0), 0, kbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(V + ke0), 0, kbytes, kBufWord3);

  for (int tt = 0; tt < ntile_here; ++tt) {
    // this lane's query column: 128 (position, head) columns per workgroup, heads fastest
    const int col = wave * 32 + n;
    const int p0 = tiles[tt] * pos_per_wg;
    const int pl = col / heads_per_wg;
    const int hi = ht * heads_per_wg + col % heads_per_wg;
    const bool valid = pl < pos_per_wg && p0 + pl < tq && hi < G;
    const int pos = min(p0 + pl, tq - 1);
    const int hq = kvh * G + min(hi, G - 1);
    const int64_t qrow = (q0 + pos) * a.Hq + hq;

    bf16x8 qop[NS], gop[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4 wq = valid ? *reinterpret_cast<const u32x4*>(Q + qrow * D + 16 * s + 8 * hh)
                             : u32x4{0, 0, 0, 0};
      const u32x4 wg = valid ? *reinterpret_cast<const u32x4*>(GO + qrow * D + 16 * s + 8 * hh)
                             : u32x4{0, 0, 0, 0};
      qop[s] = __builtin_bit_cast(bf16x8, wq);
      gop[s] = __builtin_bit_cast(bf16x8, wg);
    }
    const float Lr = valid ? a.lse[qrow] * kLog2e : INFINITY;
    const float Dq = valid ? a.Drow[qrow] : 0.f;
    f32x16 dq[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dq[mt][i] = 0.f;

    const int last = min(p0 + pos_per_wg, tq) - 1;
    const int kend = a.causal ? min(tkv, last + off + 1) : tkv;
    // key chunks: with a sliding window, the sink chunks [0, nsc) and then the chunks from the
    // window start of the tile's first row up; step ci works on chunk kchunk(ci)
    const int kc_end = (kend + kRows - 1) / kRows;
    int nsc = 0, wc0 = 0;
    if (WIN) {
      wc0 = max(0, p0 + off - W + 1) / kRows;
      nsc = min((min(a.n_sink, kend) + kRows - 1) / kRows, wc0);
    }
    const int nchunk = nsc + (kc_end - wc0);
    auto kchunk = [&](int ci) { return ci < nsc ? ci : ci - nsc + wc0; };

    u32x4 pk[C::kChunkLoads], pv[C::kChunkLoads];
    auto load = [&](int ci) {  // keys past the end read zeros (offset past the buffer)
#pragma unroll
      for (int i = 0; i < C::kChunkLoads; ++i) {
        const int idx = i * kThreads + tid;
        const int r = idx / C::kLoadsPerRow, c = idx % C::kLoadsPerRow;
        const int kk = kchunk(ci) * kRows + r;
        const unsigned vo =
            kk < tkv ? static_cast<unsigned>((kk * a.Hkv + kvh) * D + 8 * c) * 2u : kOutside;
        pk[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, vo, 0, 0);
        pv[i] = __builtin_amdgcn_raw_buffer_load_b128(vrs, vo, 0, 0);
      }
    };
    auto store = [&](int buf) {
      char* sk = smem + buf * 2 * C::kChunkBytes;
      char* sv = sk + C::kChunkBytes;
#pragma unroll
      for (int i = 0; i < C::kChunkLoads; ++i) {
        const int idx = i * kThreads + tid;
        const int r = idx / C::kLoadsPerRow, c = idx % C::kLoadsPerRow;
        *reinterpret_cast<u32x4*>(sk + chunk_off<D>(r, c)) = pk[i];
        *reinterpret_cast<u32x4*>(sv + chunk_off<D>(r, c)) = pv[i];
      }
    };

    __syncthreads();  // the previous query tile is done with both buffers
    load(0);
    store(0);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // nothing in flight: the loop waits only for its loads
    __syncthreads();
    for (int ci = 0; ci < nchunk; ++ci) {
      const int kc = kchunk(ci) * kRows;
      if (ci + 1 < nchunk) load(ci + 1);  // in flight during this chunk
      char* sk = smem + (ci & 1) * 2 * C::kChunkBytes;
      char* sv = sk + C::kChunkBytes;
      // S^T = K Q^T and dP^T = V dO^T: rows are the chunk's keys, columns the queries
      f32x16 s_acc = {}, p_acc = {};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 ka = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(sk + chunk_off<D>(n, 2 * s + hh)));
        const bf16x8 va = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(sv + chunk_off<D>(n, 2 * s + hh)));
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[s], s_acc, 0, 0, 0);
        p_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gop[s], p_acc, 0, 0, 0);
      }
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = kc + (i >> 2) * 8 + 4 * hh + (i & 3);
        const bool vis = kk < tkv && (!a.causal || kk <= pos + off) &&
                         (!WIN || kk > pos + off - W || kk < a.n_sink);
        const float pv2 = vis ? fast_exp2(fmaf(s_acc[i], sl2, -Lr)) : 0.f;
        ds[i] = pv2 * (p_acc[i] - Dq);
      }
      // dQ^T += K^T dS^T (K^T read transposed in the accumulator's key order)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 db = pack_rows(ds, ks);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
          dq[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(sk, lane, 32 * mt, ks),
                                                           db, dq[mt], 0, 0, 0);
      }
      // the other buffer was last read in chunk ci-1, before the previous barrier
      if (ci + 1 < nchunk) store((ci + 1) & 1);
      __syncthreads();
    }
    if (valid) {
      uint16_t* DQ = static_cast<uint16_t*>(a.dq) + qrow * D;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dd = mt * 32 + g4 * 8 + hh * 4;
          u32x2 w;
          w[0] = pack_bf16x2(dq[mt][4 * g4] * a.scale, dq[mt][4 * g4 + 1] * a.scale);
          w[1] = pack_bf16x2(dq[mt][4 * g4 + 2] * a.scale, dq[mt][4 * g4 + 3] * a.scale);
          *reinterpret_cast<u32x2*>(DQ + dd) = w;
        }
    }
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  // one row per (query position, head): all items back to back, dense or packed
  const int64_t rows =
      (a.items.cu ? static_cast<int64_t>(a.Tq) : static_cast<int64_t>(a.B) * a.Tq) * a.Hq;
  const int64_t rblocks = (rows * (D / 8) + 255) / 256;
  hipLaunchKernelGGL(bwd_rowdot_kernel<D>, dim3(static_cast<unsigned>(rblocks)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(a.out), static_cast<const uint16_t*>(a.dout),
                     a.Drow, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the grid covers the longest item; workgroups past a shorter item's tiles return at once
  const int max_tkv = a.items.cu ? a.max_len : a.Tkv;
  const int max_tq = a.items.cu ? a.max_len : a.Tq;
  const int key_tiles = (max_tkv + 63) / 64;
  const int tile_wgs = a.causal ? (key_tiles + 1) / 2 : key_tiles;
  if (a.window > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3(a.B * a.Hkv * tile_wgs), dim3(kThreads), 0,
                       s, a, tile_wgs);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3(a.B * a.Hkv * tile_wgs), dim3(kThreads),
                       0, s, a, tile_wgs);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.Hq / a.Hkv;
  constexpr int kCols = kWaves * 32;
  const int heads_per_wg = G < kCols ? G : kCols;
  const int pos_per_wg = kCols / heads_per_wg;
  const int head_tiles = (G + heads_per_wg - 1) / heads_per_wg;
  const int pos_tiles = (max_tq + pos_per_wg - 1) / pos_per_wg;
  const int gz = a.causal ? (pos_tiles + 1) / 2 : pos_tiles;
  const dim3 qgrid(a.B * a.Hkv * head_tiles * gz);
  if (a.window > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), qgrid, dim3(kThreads), 0, s, a, pos_per_wg,
                       heads_per_wg, head_tiles, gz);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), qgrid, dim3(kThreads), 0, s, a, pos_per_wg,
                       heads_per_wg, head_tiles, gz);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_bf16(const BwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_bwd_d<64>(a, s);
    case 128: return launch_bwd_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
