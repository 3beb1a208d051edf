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
//   * bwd_rowdot: per query row D = dout.out and L2 = L log2 e (fp32, into the workspace).
//   * bwd_dkdv: one workgroup of 8 waves (two per SIMD) per (sequence, key/value head, 64-key
//     tile; causal: a pair of tiles, heavy and light). Even waves own the tile's first 32 keys,
//     odd waves the other 32, each with its own dK^T, dV^T accumulators in registers; K (half
//     of it with d = 128) sits in registers as MFMA operands, V and the other half of K in
//     per-tile LDS tiles. The items -- 32-row chunks of q and dout with their rows' L2 and D,
//     for every query head of the group -- go four per step, one per wave pair, loaded straight
//     into double-buffered LDS stages a step ahead; every chunk read from memory feeds 64 keys.
//     Per item: S = Q K^T and dP = dO V^T with the keys as MFMA columns, P and dS in fp32, then
//     dV^T += dO^T P and dK^T += Q^T dS with dO^T / Q^T read transposed from LDS
//     (ds_read_b64_tr_b16) in the key order of the accumulators. The two halves of the wave
//     pairs run half a step apart (one's softmax beside the other's products), and the four
//     slots' partial sums are added through LDS at the end of a tile.
//   * bwd_dq: one workgroup of 4 waves per (sequence, key/value head, 128 (position, head) query
//     columns; causal: a pair of such tiles, heavy and light); 32-key chunks of K and V stream
//     through two LDS buffers with the next chunk's loads in flight. Per chunk: S^T = K Q^T and
//     dP^T = V dO^T with the queries as columns, dS^T, then dQ^T += K^T dS^T.
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "backward.hpp"

namespace gqa {
namespace {

// Buffer loads that write LDS directly (buffer_load ... lds): the wave's data goes to the
// (wave-uniform) LDS address `lds` plus the load size times the lane index; voff is the lane's
// byte offset in the buffer (range-checked: past num_records the lane writes zeros).
__device__ __forceinline__ __attribute__((address_space(3))) void* to_lds(char* p) {
  return (__attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, char* lds,
                                                  unsigned voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, to_lds(lds), 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t rs, char* lds,
                                                 unsigned voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, to_lds(lds), 4, voff, 0, 0, 0);
}

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32;  // rows of a streamed chunk
constexpr int kDkdvSlots = 4;  // query items per dK/dV step (two waves each)
// LDS layout of a [rows][D] chunk: rows of 2*D bytes, the 16-byte pieces of row r stored at
// piece index c ^ swz(r). The two readers of a chunk -- 16-byte reads down a column of rows (an
// MFMA operand with the rows as its M index) and transposing 8-byte reads of 4 rows x 64 bytes --
// then both hit 64 distinct banks per pass, which no plain row padding achieves for both.
template <int D>
__host__ __device__ constexpr int swz(int r) {
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

// Per row: D = dout . out and L2 = lse log2 e (the log-sum-exp in base 2); rows = B*Tq*Hq, one
// 64-lane wave per 4 rows (16 lanes per row).
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t* __restrict__ out,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         float* __restrict__ Dr,
                                                         float* __restrict__ L2r, int64_t rows) {
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
  if (row < rows && c == 0) {
    Dr[row] = acc;
    L2r[row] = lse[row] * kLog2e;
  }
}


// XOR pattern that the swizzle adds to the pieces of the rows i*R .. i*R+R-1 of a chunk relative
// to rows 0 .. R-1 (R rows per 1 KiB block), the same for every row of the block.
template <int D>
constexpr int block_xor(int i) {
  constexpr int R = 64 / BwdCfg<D>::kLoadsPerRow;
  return swz<D>(i * R) ^ swz<D>(0);
}
template <int D>
constexpr bool block_xor_is_uniform() {
  constexpr int R = 64 / BwdCfg<D>::kLoadsPerRow;
  for (int i = 0; i < kRows / R; ++i)
    for (int r = 0; r < R; ++r)
      if ((swz<D>(i * R + r) ^ swz<D>(r)) != block_xor<D>(i)) return false;
  return true;
}

// WIN: a sliding window (with sinks) is on; the plain kernels carry none of its tests.
// SL: query items per step (wave pairs); the workgroup has 2 SL waves.
template <int D, bool WIN, int SL>
__global__ __launch_bounds__(128 * SL) void bwd_dkdv_kernel(BwdArgs a, const float* L2row,
                                                            int tile_wgs) {
  using C = BwdCfg<D>;
  constexpr int NS = C::kNS, NMT = C::kNMT;
  constexpr int CB = C::kChunkBytes;
  // LDS: chunk (slot, matrix (0: q, 1: dout), stage) at ((slot * 2 + matrix) * 2 + stage) * CB,
  // so that a wave's chunks lie within the reach of a DS instruction's offset field; then the
  // rows' L2 (matrix 0) and D (matrix 1): 32 floats each, in 256-byte regions at
  // kRowsOff + ((stage * 2 + matrix) * SL + slot) * 256
  // (the tile's V rows follow at kVOff: [64][D], swizzled as a chunk)
  constexpr int kRowsOff = SL * 4 * CB;
  constexpr int kVOff = kRowsOff + 4 * SL * 256;
  // and with D = 128 the second half (d >= 64) of the tile's K rows at kKOff: [64][64], swizzled
  // as the rows of a d = 64 chunk; the first half (all of K with D = 64) stays in registers
  constexpr int NSR = D == 128 ? NS / 2 : NS;  // k-steps with K in registers
  constexpr int kKOff = kVOff + 2 * CB;
  constexpr int kStagesBytes = kKOff + (NSR < NS ? CB : 0);
  constexpr int kWaveRed = 2 * 32 * D * 4;  // one wave's dK^T, dV^T
  constexpr int kRedBytes = SL * kWaveRed;  // the upper half's waves
  constexpr int kSmem = kStagesBytes > kRedBytes ? kStagesBytes : kRedBytes;
  constexpr int kBlocks = C::kChunkBytes / 1024;      // 1 KiB blocks per chunk
  constexpr int kBlockRows = 64 / C::kLoadsPerRow;    // rows per block
  static_assert(C::kChunkBytes % 1024 == 0 && block_xor_is_uniform<D>(),
                "a block's loads differ from the first block's by one XOR pattern");
  static_assert(SL == 2 || SL == 4, "the cross-wave sums pair the slots");
  static_assert((2 * kBlocks) % (2 * SL) == 0, "the V tile's blocks split evenly over the waves");
  static_assert(3 * CB + CB <= 65536, "offset field reach");
  static_assert(swz<D>(32) == swz<D>(0) && swz<D>(kRows) == swz<D>(0),
                "the V tile's row 32 + n swizzles as chunk row n");
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
  const int kh = wave & 1;     // which 32 keys of the 64-key tile; also which matrix it loads
  const int slot = wave >> 1;  // which item of each step
  const int n = lane & 31, hh = lane >> 5;
  const int off = tkv - tq;
  const float sl2 = a.scale * kLog2e;
  const int W = WIN ? a.window : 0;

  // this sequence's q or dout (the wave's matrix) and its rows' L2 or D; K and V
  const int64_t qe0 = q0 * a.Hq;
  const uint16_t* mat = static_cast<const uint16_t*>(kh ? a.dout : a.q) + qe0 * D;
  const float* rowv = (kh ? a.Drow : L2row) + qe0;
  const int kbytes = tkv * a.Hkv * D * 2;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const uint16_t*>(a.k) + k0 * a.Hkv * D)),
      0, kbytes, kBufWord3);
  // (V, and half of K with D = 128, go through per-tile LDS tiles loaded by all waves)
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const uint16_t*>(a.v) + k0 * a.Hkv * D)),
      0, kbytes, kBufWord3);

  // lane constants of the LDS addresses (byte offsets into smem; stage and matrix are added as
  // multiples of the chunk size):
  //   row reads (A operands with the chunk rows as M): piece 2s + hh of row n lies at
  //   rb + ((s << 5) ^ x1) (the swizzle's upper bits move whole 32-byte pairs);
  //   transposed reads: rows 4 hh + (j >> 2) (+8), pieces 4 mt + 2 sub + ((j >> 1) & 1), half
  //   j & 1, at tb + ((mt << 6) ^ t6) (+ 16 rows per k-step: 16 row pitches)
  const int sw = swz<D>(n);
  int x1 = (sw >> 1) << 5;
  int rb = slot * 4 * CB + n * C::kPitch + 16 * (hh ^ (sw & 1));
  //   the V tile's row 32 kh + n (the lane's key) likewise at vb + ((s << 5) ^ x1)
  int vb = kVOff + (32 * kh + n) * C::kPitch + 16 * (hh ^ (sw & 1));
  //   the K half-tile's row 32 kh + n: piece 2 (s - NSR) + hh at kb + ((s - NSR) << 5 ^ xk)
  const int swk = swz<64>(32 * kh + n);
  int xk = (swk >> 1) << 5;
  int kb = kKOff + (32 * kh + n) * (C::kPitch / 2) + 16 * (hh ^ (swk & 1));
  const int j = lane & 15, sub = (lane >> 4) & 1;
  const int trow = 4 * hh + (j >> 2), tp = 2 * sub + ((j >> 1) & 1);
  const int swl = swz<D>(trow), swh = swz<D>(trow + 8);
  int tbl = slot * 4 * CB + trow * C::kPitch + 16 * (tp ^ (swl & 3)) + 8 * (j & 1);
  int tbh = slot * 4 * CB + (trow + 8) * C::kPitch + 16 * (tp ^ (swh & 3)) + 8 * (j & 1);
  int t6l = (swl >> 2) << 6, t6h = (swh >> 2) << 6;
  //   L2 / D of rows 8 g + 4 hh + 0..3 (the lane's accumulator rows): 16 bytes at lrow + 32 g
  int lrow = kRowsOff + slot * 256 + 16 * hh;
  // lane constants of the loads: piece i of the wave's chunk, 16-byte position 64 i + lane, holds
  // row i * kBlockRows + lane / kLoadsPerRow, piece (lane % kLoadsPerRow) ^ swz(row)
  const int lr = lane / C::kLoadsPerRow;
  const int v0 = lr * a.Hq * D * 2 + 16 * ((lane % C::kLoadsPerRow) ^ swz<D>(lr));
  const int vrow = (lane & 31) * a.Hq * 4;

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

    __syncthreads();  // the previous tile's cross-wave sums and V reads are done with the LDS
    bf16x8 kop[NSR];
    {  // keys past the end read zeros
      const unsigned kr = static_cast<unsigned>((key * a.Hkv + kvh) * D) * 2u;
#pragma unroll
      for (int s = 0; s < NSR; ++s) {
        const unsigned o = key_ok ? kr + 32 * s + 16 * hh : kOutside;
        kop[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, o, 0, 0));
      }
      // the K half-tile: rows of 8 pieces, kBlocks 1 KiB blocks
      constexpr int KL = 8;
#pragma unroll
      for (int i = 0; i < (NSR < NS ? (kBlocks + 2 * SL - 1) / (2 * SL) : 0); ++i) {
        const int blk = i * 2 * SL + wave;
        if (blk < kBlocks) {
          const int pos = blk * 64 + lane;
          const int r = pos / KL, c = (pos % KL) ^ swz<64>(r);
          const unsigned o =
              static_cast<unsigned>(((kb0 + r) * a.Hkv + kvh) * D + D / 2 + 8 * c) * 2u;
          buffer_load_lds16(krs, smem + kKOff + blk * 1024, o);
        }
      }
      // the V tile: 2 kBlocks 1 KiB blocks over the 2 SL waves, lane l at 16 l of its block
#pragma unroll
      for (int i = 0; i < 2 * kBlocks / (2 * SL); ++i) {
        const int blk = i * 2 * SL + wave;
        const int pos = blk * 64 + lane;
        const int r = pos / C::kLoadsPerRow, c = (pos % C::kLoadsPerRow) ^ swz<D>(r);
        const unsigned o = static_cast<unsigned>(((kb0 + r) * a.Hkv + kvh) * D + 8 * c) * 2u;
        buffer_load_lds16(vrs, smem + kVOff + blk * 1024, o);
      }
    }
    f32x16 dk[NMT], dv[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dk[mt][i] = dv[mt][i] = 0.f;

    // items: (32-row chunk from the first row that can see the tile's first key, query head of
    // the group), chunks from the last one down and heads inner, so that every workgroup walks
    // the rows in the same order; step s holds items SL s .. SL s + SL-1, item SL s + j on the
    // wave pair j
    // With a sliding window (course page "Week 7. Attention", step 3) the rows end at the last
    // one whose window still reaches the tile's last key, unless the tile holds sink keys.
    const int qstart = a.causal ? max(0, kb0 - off) / kRows * kRows : 0;
    const int qlast = (WIN && kb0 >= a.n_sink) ? min(tq - 1, kb0 + 63 + W - 1 - off) : tq - 1;
    const int nchunk = qstart <= qlast ? (qlast - qstart) / kRows + 1 : 0;
    const int nsteps = (G * nchunk + SL - 1) / SL;

    // (query head, chunk counted from the last one) of this wave pair's item: item it has head
    // it % G and chunk it / G, followed from step to step without divisions
    struct ItemPos {
      int h, c;
    };
    auto advance = [&](ItemPos p, int by) {
      for (int i = 0; i < by; ++i) {
        p.h = p.h + 1 == G ? 0 : p.h + 1;
        p.c += p.h == 0;
      }
      return p;
    };

    // a step's loads, straight into its LDS stage: the wave loads its pair's item's chunk of its
    // matrix (q for the tile's first 32 keys, dout for the others) and the rows' L2 or D. Each
    // 16-byte load fills 1 KiB of the chunk, lane l at 16 l, with the piece that the swizzle puts
    // there. The buffer starts at the chunk's first row and ends at the sequence's end, so rows
    // past the end read zeros (and add nothing below: their q and dout rows are zero); a step
    // without an item for the pair reads zeros only.
    auto load = [&](int stage, ItemPos ip) {
      const bool ok = ip.c < nchunk;
      const int p0 = qstart + (nchunk - 1 - ip.c) * kRows;
      const int srow = ok ? p0 * a.Hq + kvh * G + ip.h : 0;
      const int left = ok ? (tq - p0) * a.Hq - (kvh * G + ip.h) : 0;  // rows of the buffer
      const __amdgpu_buffer_rsrc_t ms = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(mat + static_cast<int64_t>(srow) * D), 0, left * D * 2,
          kBufWord3);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(rowv + srow), 0, left * 4, kBufWord3);
      char* chunk = smem + ((slot * 2 + kh) * 2 + stage) * CB;
#pragma unroll
      for (int i = 0; i < kBlocks; ++i) {
        const unsigned vo = static_cast<unsigned>((v0 ^ (16 * block_xor<D>(i))) +
                                                  i * kBlockRows * a.Hq * D * 2);
        buffer_load_lds16(ms, chunk + i * 1024, vo);
      }
      // 64 lanes write the 256-byte region: the 32 rows, then the same 32 rows again (unused)
      buffer_load_lds4(rs, smem + kRowsOff + ((stage * 2 + kh) * SL + slot) * 256,
                       static_cast<unsigned>(vrow));
    };

    // One item's work in two parts. m1v: S = Q K^T and dP = dO V^T (the chunk rows as M, the
    // wave's keys as N), then P = 2^(S scale log2 e - L2) and dS = P (dP - D), packed as the B
    // operands of the second part; returns whether the item contributes. m3: dV^T += dO^T P and
    // dK^T += Q^T dS, with dO^T and Q^T read transposed (k = the chunk rows in the accumulator
    // order). The lane constants are opaque to the compiler at each call: the addresses are
    // formed per call (one instruction each) instead of being held in registers.
    bf16x8 pk[2], dsk[2];
    auto m1v = [&](int stage, ItemPos ip) {
      const int qc = qstart + (nchunk - 1 - ip.c) * kRows;
      // a chunk whose last row cannot see this wave's first key, or whose first row's window
      // starts past this wave's keys (none of them a sink), contributes nothing
      const bool work = ip.c < nchunk && (!a.causal || qc + kRows - 1 + off >= kfirst) &&
                        (!WIN || kfirst < a.n_sink || kfirst + 31 > qc + off - W);
      if (!work) return false;
      asm volatile("" : "+v"(x1), "+v"(rb), "+v"(vb), "+v"(xk), "+v"(kb), "+v"(lrow));
      const int rbs = rb + stage * CB;
      f32x16 s_acc = {}, p_acc = {};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int o = ((s << 5) ^ x1) + rbs, ov = ((s << 5) ^ x1) + vb;
        const bf16x8 qa = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + o));
        const bf16x8 ga =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + o + 2 * CB));
        const bf16x8 vo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + ov));
        bf16x8 ko;
        if (s < NSR)
          ko = kop[s < NSR ? s : 0];
        else
          ko = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(smem + ((((s - NSR) & 7) << 5) ^ xk) + kb));
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, ko, s_acc, 0, 0, 0);
        p_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vo, p_acc, 0, 0, 0);
      }
      // the lane's rows are 8 g + 4 hh + t; the masks only in chunks where some (row, key) pair
      // is hidden. Keys past the end need none: each lane's accumulator column is its own key,
      // which is not written.
      const int lrs = lrow + stage * 2 * SL * 256;
      float pr[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(smem + lrs + 32 * g);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          pr[4 * g + t] = fast_exp2(fmaf(s_acc[4 * g + t], sl2, -l2[t]));
      }
      const bool hide_causal = a.causal && kfirst + 31 > qc + off;
      const bool hide_window =
          WIN && !(kfirst + 31 < a.n_sink || kfirst > qc + kRows - 1 + off - W);
      if (hide_causal || hide_window) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int p = qc + (i >> 2) * 8 + 4 * hh + (i & 3);
          const bool vis = (!a.causal || key <= p + off) &&
                           (!WIN || key > p + off - W || key < a.n_sink);
          pr[i] = vis ? pr[i] : 0.f;
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 dd = *reinterpret_cast<const f32x4*>(smem + lrs + SL * 256 + 32 * g);
#pragma unroll
        for (int t = 0; t < 4; ++t) ds[4 * g + t] = pr[4 * g + t] * (p_acc[4 * g + t] - dd[t]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pk[ks] = pack_rows(pr, ks);
        dsk[ks] = pack_rows(ds, ks);
      }
      return true;
    };
    auto m3 = [&](int stage) {
      asm volatile("" : "+v"(tbl), "+v"(tbh), "+v"(t6l), "+v"(t6h));
      const int tls = tbl + stage * CB, ths = tbh + stage * CB;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const int ol = ((mt << 6) ^ t6l) + tls + ks * 16 * C::kPitch;
          const int oh = ((mt << 6) ^ t6h) + ths + ks * 16 * C::kPitch;
          const u32x2 gl = lds_read_tr(smem, ol + 2 * CB), gh = lds_read_tr(smem, oh + 2 * CB);
          dv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, u32x4{gl[0], gl[1], gh[0], gh[1]}), pk[ks], dv[mt], 0, 0,
              0);
          const u32x2 ql = lds_read_tr(smem, ol), qh = lds_read_tr(smem, oh);
          dk[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, u32x4{ql[0], ql[1], qh[0], qh[1]}), dsk[ks], dk[mt], 0,
              0, 0);
        }
      }
    };

    // Two groups of wave pairs, half a step apart, so that on each SIMD (one wave of each group)
    // one wave's softmax runs beside the other's matrix products: group 0 (slots 0 .. SL/2-1)
    // does m1v of step st's item in the first half of step st and m3 in the second half; group 1
    // does m1v in the second half and m3 in the first half of step st+1. Each slot's two stages
    // are refilled one step ahead, at the start of the slot's m1v, into the stage that its m3 of
    // the previous step finished reading before the last barrier.
    // Every wave runs the same steps (m1v, barrier, m3, barrier); group 1 passes one barrier
    // before its first step and group 0 one after its last, so the groups' barriers pair up half
    // a step apart.
    const int lag = slot < SL / 2 ? 0 : 1;
    ItemPos cur = advance(ItemPos{0, 0}, slot);  // item `slot` of step 0
    if (nsteps > 0) load(0, cur);
    // nothing in flight from here on (the K/V operands included), so that the loop below waits
    // only for its own loads
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (lag) __builtin_amdgcn_s_barrier();
    for (int st = 0; st < nsteps; ++st) {
      const int stage = st & 1;
      const ItemPos nxt = advance(cur, SL);
      if (st + 1 < nsteps) load(stage ^ 1, nxt);
      const bool work = m1v(stage, cur);
      cur = nxt;
      // only pairs the groups' halves (no data passes here): a bare barrier, without the fence
      // that would wait for the loads just issued
      __builtin_amdgcn_s_barrier();
      if (work) m3(stage);
      __builtin_amdgcn_s_waitcnt(kVmcnt0);  // the next step's stage is in place
      __syncthreads();
    }
    if (!lag) __builtin_amdgcn_s_barrier();
    __syncthreads();  // every wave's m3 is done before the LDS is reused below

    // cross-wave sums over the slots (same keys): the upper half of the slots hands its partial
    // dK^T, dV^T to the lower half through LDS, halving until slot 0 holds the sum
    // (a wave's area: kWaveRed bytes at its lane's float, the values 256 bytes apart)
#pragma unroll
    for (int half = SL / 2; half > 0; half >>= 1) {
      // the area of wave pair (slot mod half), kept opaque so that the addresses stay one
      // register plus the instructions' offsets
      int area = ((slot & (half - 1)) * 2 + kh) * kWaveRed + 4 * lane;
      asm volatile("" : "+v"(area));
      if (slot >= half && slot < 2 * half) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            *reinterpret_cast<float*>(smem + area + (mt * 16 + i) * 256) = dk[mt][i];
            *reinterpret_cast<float*>(smem + area + 32 * D * 4 + (mt * 16 + i) * 256) = dv[mt][i];
          }
      }
      __syncthreads();
      if (slot < half) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            dk[mt][i] += *reinterpret_cast<const float*>(smem + area + (mt * 16 + i) * 256);
            dv[mt][i] +=
                *reinterpret_cast<const float*>(smem + area + 32 * D * 4 + (mt * 16 + i) * 256);
          }
      }
      if (half > 1) __syncthreads();  // read before the next round overwrites
    }
    if (slot == 0 && key_ok) {
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

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdArgs a, const float* L2row,
                                                          int pos_per_wg, int heads_per_wg,
                                                          int head_tiles, int gz) {
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
    const int pmin = p0 + (wave * 32) / heads_per_wg;  // the wave's first position
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
    const float Lr = valid ? L2row[qrow] : INFINITY;
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
      // P (in place of S) and dS; the masks only in chunks that cross the diagonal of some of the
      // wave's positions (or with a window). Keys past the end need none: their K and V rows
      // read zeros, so they add nothing to dQ.
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) s_acc[i] = fast_exp2(fmaf(s_acc[i], sl2, -Lr));
      if (WIN || (a.causal && kc + kRows - 1 > pmin + off)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = kc + (i >> 2) * 8 + 4 * hh + (i & 3);
          const bool vis = kk < tkv && (!a.causal || kk <= pos + off) &&
                           (!WIN || kk > pos + off - W || kk < a.n_sink);
          s_acc[i] = vis ? s_acc[i] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = s_acc[i] * (p_acc[i] - Dq);
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
  float* L2row = a.Drow + backward_row_array_floats(static_cast<size_t>(rows));
  hipLaunchKernelGGL(bwd_rowdot_kernel<D>, dim3(static_cast<unsigned>(rblocks)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(a.out), static_cast<const uint16_t*>(a.dout),
                     a.lse, a.Drow, L2row, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the grid covers the longest item; workgroups past a shorter item's tiles return at once
  const int max_tkv = a.items.cu ? a.max_len : a.Tkv;
  const int max_tq = a.items.cu ? a.max_len : a.Tq;
  const int key_tiles = (max_tkv + 63) / 64;
  const int tile_wgs = a.causal ? (key_tiles + 1) / 2 : key_tiles;
  if (a.window > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, kDkdvSlots>), dim3(a.B * a.Hkv * tile_wgs),
                       dim3(128 * kDkdvSlots), 0, s, a, L2row, tile_wgs);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, kDkdvSlots>), dim3(a.B * a.Hkv * tile_wgs),
                       dim3(128 * kDkdvSlots), 0, s, a, L2row, tile_wgs);
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
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), qgrid, dim3(kThreads), 0, s, a, L2row,
                       pos_per_wg, heads_per_wg, head_tiles, gz);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), qgrid, dim3(kThreads), 0, s, a, L2row,
                       pos_per_wg, heads_per_wg, head_tiles, gz);
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
