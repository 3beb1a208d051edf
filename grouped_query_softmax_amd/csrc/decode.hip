// decode.hip -- split-KV grouped-query attention for one query token per sequence.
//
// A decode step is bound by streaming the key/value cache from HBM: every cached element is read
// once and used for a handful of flops (G query heads share it). Grouped-query attention is what
// makes the stream small: the cache holds Hkv heads, not Hq (course page "Week 7. Attention",
// step 2: 32 query / 8 key-value heads is a 4x smaller cache; GQA lab page "Transformer --
// attention by hand: reducing only the key/value heads", step 6: the cache element count has no
// query-head term).
//
// Kernel 1 (split): one workgroup of 4 waves per (sequence, key/value head, chunk of up to 16
// query heads -- 32 when the group has more than 16 -- split of the cache). Each wave streams its own 32-key tiles of the split and keeps
// the next tile's loads in flight while it computes the current one, so the vector and matrix
// work hides under the HBM stream. Per tile, on the matrix cores (v_mfma_f32_16x16x32_bf16):
//   * the tile's K and V rows are loaded whole (each load instruction covers complete 128-byte
//     lines, with the non-temporal cache policy: every line is used exactly once) and written
//     to per-wave LDS tiles; every cache element leaves HBM exactly once for all query heads;
//   * scores S^T = K Q^T: K rows are the A operand read back from LDS, the query heads are the
//     16 columns of B (unused columns are zero);
//   * O^T += V^T P^T: V comes back from LDS transposed with ds_read_b64_tr_b16 (4 keys of one
//     dimension per lane), P^T is the score accumulator rounded to bf16 in place, with the
//     contraction order of keys following the accumulator layout.
// Ragged caches and sliding windows (course page "Week 7. Attention", step 3): sequence b uses
// its first lens[b] cache entries; with a window it sees only the last `window` of them plus the
// first n_sink (sink) entries. The visible entries form one list (sinks, then window) over which
// the splits and tiles run, so nothing outside it is read. A cache bounded to the window (the
// same page: the window bounds the cache to its size) holds n_sink + window slots per sequence:
// the sinks in their own slots, and entry e >= n_sink in slot n_sink + (e - n_sink) mod window,
// where it replaced the entry that left the window; the list is then mapped to those slots.
// With up to 512 sequences, each workgroup takes its sequence from a balanced order (longest and
// shortest sequences paired on the compute units) that it works out itself at its start.
// Each lane owns one query head (one accumulator column), so the softmax reference and the
// rescale factor are per lane; the row maximum of a tile is combined over the 4 lane groups that
// hold that head's keys. Online softmax in the base-2 domain with a lazily moved reference
// (moved only when a tile raises the maximum by more than 8 in log2 units; exact, since one
// reference is used for both the output and the running sum). The 4 waves are merged in LDS and
// the split's partial (reference m, running sum l, unnormalised output o) goes to the workspace,
// or, when the cache is not split, the normalised output goes straight to `out`.
// Kernel 2 (combine, only with more than one split), one workgroup per (sequence, query head):
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s with M = max_s m_s.
#include <math.h>

#include <algorithm>

#include <mutex>

#include "decode.hpp"

// Scratch for callers that cannot allocate: the fp32 split partials of gqa_attn_decode_noalloc
// live in this fixed device array (one copy per GPU, for the life of the process) instead of a
// caller workspace. Every call on a GPU shares that GPU's copy, so calls that overlap in time on
// one GPU race. Nothing in it needs clearing between calls: each split writes every partial the
// combine pass reads.
static __device__ __align__(256) char scratch[gqa::kDecodeScratchBytes];

namespace gqa {
namespace {

// The device address of `scratch` on each GPU, taken once per device with that device current
// (host code must never pass the array's own name to a kernel: on the host it stands for a
// host-side shadow, not device memory).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTK = 32;              // keys per tile
constexpr int kHeadCols = 16;        // query heads per workgroup (MFMA columns)
// Splits are added only until the grid has this many workgroups: one per CU. Fewer, longer
// splits stream faster than two resident per CU with half the keys each (measured: one
// 131072-entry sequence 106 -> 98 us, 8 x 32768 entries 175 -> 170 us): a workgroup's fixed
// cost (query load, merge, partial write) is spread over more keys, and 4 waves with two tiles
// in flight each already cover the memory latency.
constexpr int kTargetBlocks = 256;
// Cache policy of the key/value loads: non-temporal (each cache line is read exactly once).
constexpr int kStreamLoad = 2;
constexpr int kMinSplitKeys = 256;
constexpr float kRescaleSlack = 8.0f;

template <int D>
struct DecCfg {
  static constexpr int kSteps = D / 32;   // MFMA k-steps over d for the scores
  static constexpr int kDT = D / 16;      // 16-dimension tiles of O^T
  // LDS row pitches (bytes), chosen so that the reads are free of bank conflicts: 16-byte K
  // operand reads of 16 rows, and transposing 8-byte V reads of 8 rows per half wave
  static constexpr int kPitch = 2 * D + 32;   // V tile
  static constexpr int kKPitch = 2 * D + 16;  // K tile
  static constexpr int kTileBytes = kTK * (kPitch + kKPitch);
  static constexpr int kLPR = D / 8;          // lanes per key row in the full-row loads
  static constexpr int kRPI = 64 / kLPR;      // key rows per load instruction
  static constexpr int kVBytes = kWaves * kTileBytes;
  static constexpr int kMergeBytes = kWaves * kHeadCols * (D + 2) * 4;
  static constexpr int kSmemBytes = kVBytes > kMergeBytes ? kVBytes : kMergeBytes;
};


// Ragged caches: a balanced order of the sequences. With equal splits a sequence's work grows with
// its visible entries, and the workgroups go out in rows of about one per compute unit, the rows
// that fit at once all resident together: a unit that gets two long sequences finishes last.
// Ranked longest first (ties by index), the sequences are laid out in rows of `row` with every
// other row reversed (a snake), so the unit that holds a row's longest also holds the next row's
// shortest. Each split workgroup finds the sequence at its position of that layout itself (up to
// kMaxOrdered sequences, ranked in LDS: B^2 / 256 comparisons per thread).
constexpr int kMaxOrdered = 512;
template <bool RING>
__device__ int balanced_sequence(const DecodeArgs& a, int pos, int row, int* vis) {
  for (int j = threadIdx.x; j < a.B; j += kThreads) {
    const int L = RING ? max(a.lens[j], 0) : min(max(a.lens[j], 0), a.Tkv);
    const int w_start = a.window > 0 ? max(0, L - a.window) : 0;
    vis[j] = min(a.n_sink, w_start) + (L - w_start);
  }
  __syncthreads();
  // the rank that the snake layout puts at this position (the last row may be short)
  const int r = pos / row, c = pos % row;
  const int len = min(row, a.B - r * row);
  const int k = r * row + ((r & 1) ? len - 1 - c : c);
  for (int j = threadIdx.x; j < a.B; j += kThreads) {
    const int v = vis[j];
    int rank = 0;
    for (int i = 0; i < a.B; ++i) rank += (vis[i] > v) || (vis[i] == v && i < j);
    if (rank == k) vis[kMaxOrdered] = j;  // each rank belongs to exactly one sequence
  }
  __syncthreads();
  const int b = vis[kMaxOrdered];
  __syncthreads();  // the LDS is the key/value tiles' from here on
  return b;
}

// NCH: 16-head chunks of query heads per workgroup (1, or 2 when a group has more than 16 heads:
// every K/V operand read from LDS then feeds both chunks' MFMAs, and the cache is read once for
// up to 32 heads). RING: the cache is bounded to the window (launch_decode_window_cache_bf16).
template <int D, int NCH, bool RING>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a, int head_chunks,
                                                                int order_row) {
  using C = DecCfg<D>;
  constexpr int NS = C::kSteps;
  constexpr int NDT = C::kDT;
  __shared__ __attribute__((aligned(16))) char smem[C::kSmemBytes];
  static_assert(C::kSmemBytes >= (kMaxOrdered + 1) * 4, "the ragged order's ranks fit the LDS");

  const int S = a.nsplit;
  const int lin = blockIdx.x;
  const int split = lin % S;
  const int rest = lin / S;
  const int y = rest % (a.Hkv * head_chunks);
  // sequence: in launch order, or from the balanced order of a ragged cache (rows of order_row)
  const int pos = rest / (a.Hkv * head_chunks);
  const int b = order_row > 0
                    ? balanced_sequence<RING>(a, pos, order_row, reinterpret_cast<int*>(smem))
                    : pos;
  const int kvh = y / head_chunks;
  const int hc = y % head_chunks;
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int r16 = lane & 15;
  const int g = lane >> 4;
  // The visible cache entries of this sequence, as one list: the sink entries below the window
  // [0, a_end) followed by the window [w_start, L). Splits and tiles run over list positions.
  // L = 0 (an empty cache) leaves nothing visible: the output row is zero. A bounded cache's
  // length counts every entry the sequence has had.
  const int L = RING ? max(a.lens[b], 0) : a.lens ? min(max(a.lens[b], 0), a.Tkv) : a.Tkv;
  const int w_start = a.window > 0 ? max(0, L - a.window) : 0;
  const int a_end = min(a.n_sink, w_start);
  const int nvis = a_end + (L - w_start);
  const int kb = split * a.per;
  const int nkeys = min(nvis, kb + a.per) - kb;  // <= 0: nothing of this sequence in the split
  // a split past the sequence's visible entries has nothing to contribute: the combine reads
  // only the splits a sequence has (with a single split the output must still be written)
  if (S > 1 && nkeys <= 0) return;
  const int ntile = nkeys > 0 ? (nkeys + kTK - 1) / kTK : 0;
  const int row_bytes = a.Hkv * D * 2;
  const float sl2 = a.scale * kLog2e;

  // this lane's query head (accumulator column) of each chunk and its B operand, loaded once
  bf16x8 qop[NCH][NS];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = (hc * NCH + c) * kHeadCols + r16;
    const bool col_ok = col < G;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<int64_t>(b) * a.Hq + kvh * G + (col_ok ? col : 0)) * D +
                           8 * g;
    u32x4 wq[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
      wq[s] = col_ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * s) : u32x4{0, 0, 0, 0};
    float inv = 0.f;
    if (a.qn_w) {
      // QK-norm of the query (the cache holds normalised keys): the row is spread over the
      // lanes r16 + 16 g, g = 0..3
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) ss += sumsq8(wq[s]);
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      inv = rms_inv(ss, D, a.norm_eps);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 w = wq[s];
      // rotary embedding of the query at its position L - 1 (the cache holds turned keys);
      // this lane's dimensions 32s + 8g .. +7 are the pairs 16s + 4g .. +3. A bounded cache's
      // length is not bounded by the tables: past their last row the query takes that row.
      const int qpos = RING ? min(L, a.rope_rows) - 1 : L - 1;
      const int ti = max(qpos, 0) * (D / 2) + 16 * s + 4 * g;
      if (a.qn_w) {
        float x[8];
        unpack8(w, x);
        norm8(x, inv, *reinterpret_cast<const f32x4*>(a.qn_w + 32 * s + 8 * g),
              *reinterpret_cast<const f32x4*>(a.qn_w + 32 * s + 8 * g + 4));
        if (a.rope_cos)
          rope8(x, *reinterpret_cast<const f32x4*>(a.rope_cos + ti),
                *reinterpret_cast<const f32x4*>(a.rope_sin + ti));
        w = pack8(x);
      } else if (a.rope_cos) {
        w = rope_chunk(w, *reinterpret_cast<const f32x4*>(a.rope_cos + ti),
                       *reinterpret_cast<const f32x4*>(a.rope_sin + ti));
      }
      qop[c][s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int64_t seq_elem = (static_cast<int64_t>(b) * a.Tkv * a.Hkv + kvh) * D;
  // bytes from the head's first entry to the end of its last visible one (0 for an empty cache,
  // so every load of that sequence is out of range and reads zeros); a bounded cache uses at
  // most its Tkv slots
  const int nslot = RING ? min(L, a.Tkv) : L;
  const int nrec = nslot > 0 ? (nslot - 1) * row_bytes + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(static_cast<const uint16_t*>(a.k) + seq_elem), 0, nrec, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(static_cast<const uint16_t*>(a.v) + seq_elem), 0, nrec, kBufWord3);
  const int vend = kb + max(nkeys, 0);    // list positions of this split: [kb, vend)
  const int shift = w_start - a_end;      // list position -> cache entry, past the sinks
  // bounded cache: the window's entries e >= e0 = max(w_start, n_sink) sit in slot
  // n_sink + (r0 + e - e0) mod window with r0 = (e0 - n_sink) mod window; they span fewer than
  // `window` entries, so the sum wraps at most once
  [[maybe_unused]] const int e0 = max(w_start, a.n_sink);
  [[maybe_unused]] const int r0 = RING ? (e0 - a.n_sink) % a.window : 0;

  // Loads: kLPR lanes cover one whole key row (16 bytes each), so every load instruction reads
  // whole 128-byte lines; K and V go to this wave's LDS tiles as they arrived. The K operand is
  // read back as lane (g, r16) <- row r16, bytes 64s + 16g (dimensions 32s + 8g .. +7, the A
  // operand slice of lane group g at k-step s); V is read back transposed.
  char* vt = smem + wave * C::kTileBytes;
  char* kt = vt + kTK * C::kPitch;
  const int lrow = lane / C::kLPR, lcol = lane % C::kLPR;
  const int k_wr = lrow * C::kKPitch + 16 * lcol;
  const int v_wr = lrow * C::kPitch + 16 * lcol;
  const int k_rd = r16 * C::kKPitch + 16 * g;
  const int v_rd = (4 * g + (r16 >> 2)) * C::kPitch + 8 * (r16 & 3);

  f32x4 acc_o[NCH][NDT];
  float m_run[NCH], l_run[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt) acc_o[c][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
  }

  // Rows past the split's list positions are pointed past num_records and read as zeros; tiles
  // at or past ntile are never processed.
  auto load = [&](u32x4 (&kr)[2][NS], u32x4 (&vr)[2][NS], int t) {
    const int v0 = kb + t * kTK + lrow;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int vpos = v0 + (blk * NS + s) * C::kRPI;
        int entry = vpos < a_end ? vpos : vpos + shift;
        if constexpr (RING) {
          // (rows past the list read zeros below whatever their entry)
          if (vpos < vend && entry >= a.n_sink) {
            const int r = r0 + (entry - e0);
            entry = a.n_sink + (r >= a.window ? r - a.window : r);
          }
        }
        const int off = vpos < vend
                            ? static_cast<int>(static_cast<unsigned>(entry) * row_bytes) + 16 * lcol
                            : nrec;
        kr[blk][s] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, kStreamLoad);
        vr[blk][s] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kStreamLoad);
      }
  };

  auto process = [&](const u32x4 (&kr)[2][NS], const u32x4 (&vr)[2][NS], int t) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int row = (blk * NS + s) * C::kRPI;
        *reinterpret_cast<u32x4*>(kt + k_wr + row * C::kKPitch) = kr[blk][s];
        *reinterpret_cast<u32x4*>(vt + v_wr + row * C::kPitch) = vr[blk][s];
      }
    lds_order();
    // S^T for the 2 blocks of 16 keys: lane (g, r16) gets keys 16 blk + 4g + i of head r16 of
    // each chunk; every K operand read feeds the MFMAs of all chunks
    f32x4 sc[NCH][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) sc[c][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 kw =
            *reinterpret_cast<const u32x4*>(kt + k_rd + blk * 16 * C::kKPitch + 64 * s);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          sc[c][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw),
                                                               qop[c][s], sc[c][blk], 0, 0, 0);
      }
    }
    const int k0 = t * kTK;
    bf16x8 pop[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (k0 + kTK > nkeys) {
        const int rem = nkeys - 1 - k0 - 4 * g;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[c][blk][i] = (16 * blk + i <= rem) ? sc[c][blk][i] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(sc[c][0][0], sc[c][0][1]), fmaxf(sc[c][0][2], sc[c][0][3])),
                       fmaxf(fmaxf(sc[c][1][0], sc[c][1][1]), fmaxf(sc[c][1][2], sc[c][1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = pair_max32(mx) * sl2;
      const bool move = mx > m_run[c] + kRescaleSlack;
      if (__any(move)) {
        const float m_new = move ? mx : m_run[c];
        const float alpha = move ? fast_exp2(m_run[c] - m_new) : 1.f;
        l_run[c] *= alpha;
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_o[c][nt][i] *= alpha;
        m_run[c] = m_new;
      }
      uint32_t pw[4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          pw[2 * blk + e] = pack_bf16x2(fast_exp2(fmaf(sc[c][blk][2 * e], sl2, -m_run[c])),
                                        fast_exp2(fmaf(sc[c][blk][2 * e + 1], sl2, -m_run[c])));
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[e]),
                                               __builtin_bit_cast(bf16x2, 0x3f803f80u), psum,
                                               false);
      l_run[c] += psum;
      pop[c] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    }
    lds_order();
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt) {
      const u32x2 lo = lds_read_tr(vt, v_rd + 32 * nt);                  // keys 4g .. 4g+3
      const u32x2 hi = lds_read_tr(vt, v_rd + 16 * C::kPitch + 32 * nt);  // keys 16+4g ..
      const bf16x8 vop = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        acc_o[c][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[c], acc_o[c][nt], 0, 0, 0);
    }
    lds_order();
  };

  {
    // two register sets: the loads of the next tile are in flight while a tile is processed
    // (a fixed trip count and no early exit, so the compiler's wait analysis sees only the
    // other set's loads in flight at the top of the loop)
    u32x4 ka[2][NS], va[2][NS], kbuf[2][NS], vbuf[2][NS];
    const int mine = wave < ntile ? (ntile - wave + kWaves - 1) / kWaves : 0;
    load(ka, va, wave);
    int t = wave;
    for (int i = 0; i < mine / 2; ++i) {
      load(kbuf, vbuf, t + kWaves);
      process(ka, va, t);
      load(ka, va, t + 2 * kWaves);
      process(kbuf, vbuf, t + kWaves);
      t += 2 * kWaves;
    }
    if (mine & 1) process(ka, va, t);
  }

  // this wave's running sums: the 4 lane groups hold different keys of the same head
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    l_run[c] += __shfl_xor(l_run[c], 16);
    l_run[c] = pair_sum32(l_run[c]);
  }

  // merge the 4 waves in LDS, one chunk at a time: m, l per head, then o[head][dim]
  float* mm = reinterpret_cast<float*>(smem);
  float* ll = mm + kWaves * kHeadCols;
  float* oo = ll + kWaves * kHeadCols;
  constexpr int kDimsPerThread = kHeadCols * D / kThreads;  // 8 at d = 128, 4 at d = 64
  const int h = tid / (D / kDimsPerThread);
  const int d0 = (tid % (D / kDimsPerThread)) * kDimsPerThread;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    __syncthreads();  // every wave is done with its V tile (c = 0) or the previous chunk's merge
    if (g == 0) {
      mm[wave * kHeadCols + r16] = m_run[c];
      ll[wave * kHeadCols + r16] = l_run[c];
    }
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt)
      *reinterpret_cast<f32x4*>(oo + (wave * kHeadCols + r16) * D + 16 * nt + 4 * g) =
          acc_o[c][nt];
    __syncthreads();
    const int hq_in = (hc * NCH + c) * kHeadCols + h;
    if (hq_in < G) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mm[w * kHeadCols + h]);
      float L = 0.f, o[kDimsPerThread];
#pragma unroll
      for (int e = 0; e < kDimsPerThread; ++e) o[e] = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = mm[w * kHeadCols + h];
        const float aw = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        L = fmaf(aw, ll[w * kHeadCols + h], L);
#pragma unroll
        for (int e = 0; e < kDimsPerThread; ++e)
          o[e] = fmaf(aw, oo[(w * kHeadCols + h) * D + d0 + e], o[e]);
      }
      const int64_t idx = (static_cast<int64_t>(b) * a.Hq + kvh * G + hq_in) * S + split;
      if (S == 1) {  // the whole cache in one split: finish here, no combine pass
        uint16_t* orow = static_cast<uint16_t*>(a.out) + idx * D + d0;
#pragma unroll
        for (int e = 0; e < kDimsPerThread; e += 4) {
          u32x2 w;
          // an empty cache (L = 0, o = 0) gives the zero row
          const float r = L > 0.f ? L : 1.f;
          w[0] = pack_bf16x2(o[e] / r, o[e + 1] / r);
          w[1] = pack_bf16x2(o[e + 2] / r, o[e + 3] / r);
          *reinterpret_cast<u32x2*>(orow + e) = w;
        }
      } else {
        float* wo = a.ws + idx * D + d0;
#pragma unroll
        for (int e = 0; e < kDimsPerThread; e += 4)
          *reinterpret_cast<f32x4*>(wo + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
        if (d0 == 0) {
          const int64_t nbh = static_cast<int64_t>(a.B) * a.Hq * S;
          a.ws[nbh * D + idx] = M;
          a.ws[nbh * D + nbh + idx] = L;
        }
      }
    }
  }
}

// Largest number of splits a launch uses (decode_num_splits aims at kTargetBlocks workgroups).
constexpr int kMaxSplits = kTargetBlocks;

// Reductions over the D threads of a combine workgroup (D / 64 waves), through LDS.
template <int D>
__device__ __forceinline__ float block_max(float x, float* red) {
  for (int m = 32; m > 0; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < D / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}
template <int D>
__device__ __forceinline__ float block_sum(float x, float* red) {
  for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < D / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

// One workgroup of D threads per (sequence, query head): the splits' (m, l) pairs are reduced by
// the whole workgroup and their weights kept in LDS, then each thread forms one output column
// from four independent partial sums, so that the split partials' loads overlap instead of
// following one another.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float wsh[kMaxSplits];
  __shared__ float red[D / 64];
  const float* __restrict__ ws = a.ws;
  const int nsplit = a.nsplit;
  const int nbh = a.B * a.Hq;
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  // the splits this sequence has: its visible entries (as in the split kernel) over a.per
  const int b = bh / a.Hq;
  const int L = a.lens ? min(max(a.lens[b], 0), a.Tkv) : a.Tkv;
  const int w_start = a.window > 0 ? max(0, L - a.window) : 0;
  const int nvis = min(a.n_sink, w_start) + (L - w_start);
  const int nvalid = min(nsplit, (nvis + a.per - 1) / a.per);
  if (nvalid == 0) {  // an empty cache: no split wrote a partial, the row is zero
    static_cast<uint16_t*>(a.out)[static_cast<int64_t>(bh) * D + d] = 0;
    return;
  }
  const int64_t ntot = static_cast<int64_t>(nbh) * nsplit;
  const float* wm = ws + ntot * D + static_cast<int64_t>(bh) * nsplit;
  const float* wl = ws + ntot * D + ntot + static_cast<int64_t>(bh) * nsplit;
  float m = -INFINITY;
  for (int s = d; s < nvalid; s += D) m = fmaxf(m, wm[s]);
  const float M = block_max<D>(m, red);
  float dl = 0.f;
  for (int s = d; s < nvalid; s += D) {
    const float w = (wm[s] == -INFINITY) ? 0.f : fast_exp2(wm[s] - M);
    wsh[s] = w;
    dl = fmaf(w, wl[s], dl);
  }
  const float den = block_sum<D>(dl, red);  // its barriers also publish wsh
  const float* o = ws + static_cast<int64_t>(bh) * nsplit * D + d;
  float n4[4] = {0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 4 <= nvalid; s += 4)
#pragma unroll
    for (int j = 0; j < 4; ++j) n4[j] = fmaf(wsh[s + j], o[static_cast<int64_t>(s + j) * D], n4[j]);
  for (; s < nvalid; ++s) n4[0] = fmaf(wsh[s], o[static_cast<int64_t>(s) * D], n4[0]);
  const float num = (n4[0] + n4[1]) + (n4[2] + n4[3]);
  static_cast<uint16_t*>(a.out)[static_cast<int64_t>(bh) * D + d] = f32_to_bf16(num / den);
}

// floats of the split partials in the workspace
int64_t partial_floats(int B, int Hq, int S, int d) {
  return static_cast<int64_t>(B) * Hq * S * (d + 2);
}

// compute units of the current device (cached per device)
int g_units[kMaxDevices] = {};
int device_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_units[dev]) {
    int n = 0;
    g_units[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                               hipSuccess && n > 0 ? n : 256;
  }
  return g_units[dev];
}

// 16-head chunks per workgroup: two when a group has more than 16 query heads
int chunks_per_wg(int G) { return G > kHeadCols ? 2 : 1; }
int head_chunks_of(int G) {
  const int per = kHeadCols * chunks_per_wg(G);
  return (G + per - 1) / per;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s, bool ring) {
  if (a.nsplit < 1 || a.nsplit > kMaxSplits) return hipErrorInvalidValue;  // the combine's LDS
  const int G = a.Hq / a.Hkv;
  const int hcs = head_chunks_of(G);
  const dim3 grid(a.nsplit * a.Hkv * hcs * a.B);
  // a ragged cache's balanced order: rows of the sequences whose workgroups take about one per
  // compute unit (0: launch order)
  const int order_row = (a.lens && a.B > 1 && a.B <= kMaxOrdered)
                            ? std::max(1, device_units() / (a.nsplit * a.Hkv * hcs))
                            : 0;
  if (ring) {
    if (chunks_per_wg(G) == 2)
      hipLaunchKernelGGL((decode_split_kernel<D, 2, true>), grid, dim3(kThreads), 0, s, a, hcs,
                         order_row);
    else
      hipLaunchKernelGGL((decode_split_kernel<D, 1, true>), grid, dim3(kThreads), 0, s, a, hcs,
                         order_row);
  } else if (chunks_per_wg(G) == 2) {
    hipLaunchKernelGGL((decode_split_kernel<D, 2, false>), grid, dim3(kThreads), 0, s, a, hcs,
                       order_row);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<D, 1, false>), grid, dim3(kThreads), 0, s, a, hcs,
                       order_row);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.B * a.Hq), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int decode_split_len(int Tkv, int nsplit) {
  const int per = (Tkv + nsplit - 1) / nsplit;
  return (per + kTK - 1) / kTK * kTK;
}

int decode_num_splits(int B, int Tkv, int Hq, int Hkv, int d) {
  (void)d;
  const int64_t units = static_cast<int64_t>(B) * Hkv * head_chunks_of(Hq / Hkv);
  int64_t s = (kTargetBlocks + units - 1) / units;
  const int64_t max_s = Tkv / kMinSplitKeys > 1 ? Tkv / kMinSplitKeys : 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  // splits are whole tiles; recount so that every split holds at least one key
  const int per = decode_split_len(Tkv, static_cast<int>(s));
  return (Tkv + per - 1) / per;
}

size_t decode_workspace_bytes(int B, int Tkv, int Hq, int Hkv, int d) {
  const int S = decode_num_splits(B, Tkv, Hq, Hkv, d);
  // the split partials
  return static_cast<size_t>(partial_floats(B, Hq, S, d)) * sizeof(float);
}

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_d<64>(a, s, false);
    case 128: return launch_d<128>(a, s, false);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_window_cache_bf16(const DecodeArgs& a, hipStream_t s) {
  if (!a.lens || a.window < 1) return hipErrorInvalidValue;
  switch (a.d) {
    case 64: return launch_d<64>(a, s, true);
    case 128: return launch_d<128>(a, s, true);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
