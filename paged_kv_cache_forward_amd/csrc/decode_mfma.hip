// Decode attention for bf16 K/V with head_dim 128: scores on the matrix cores,
// P.V on the vector ALUs.  Two launches share the per-tile fold below:
//   * the balanced kernel (decode_balanced_kernel, further down; the default
//     up to 1024 sequences): a fixed grid of waves cuts each KV head's
//     concatenated tiles into equal ranges, stages them through LDS, and
//     writes partial results for its own merge kernel;
//   * the partitioned kernel (decode_mfma_kernel): one work-group per
//     (sequence, KV head, partition), partials merged by the merge kernel of
//     decode.hip.
//
// What is computed: "PagedAttention et vLLM" (aiunderstanding.org), section
// "Plongée profonde": the new token of each sequence attends to all of its
// cached keys/values, which sit in fixed-size blocks anywhere in memory and are
// found through a table from logical positions to physical blocks.
// "Внутреннее устройство vLLM" (artificials.ru), forward-pass paragraph: each
// sequence of the super-batch sees only its own tokens.  Decode is bound by
// memory bandwidth ("vLLM PagedAttention: eine Revolution ..."
// (de.news.hada.io), bullet on disaggregation), so every choice below serves
// the K/V stream: each (block, KV head) tile is read from HBM exactly once, by
// the work-group that owns its KV head, for all G query heads of that head.
//
// Why the scores go to MFMA: G query heads sharing a KV head make Q.K^T a real
// (G x 128) . (128 x 16) product per tile.  On the vector ALUs it costs ~130
// instructions per 8 KiB tile (dot2 + cross-lane reductions), which together
// with softmax and P.V left no VALU headroom at the HBM rate.  One
// v_mfma_f32_16x16x32_bf16 per 32 dims does it in 4 instructions, reading the
// K tile in its stored layout as the A operand.
//
// Partitioned kernel's work item: one work-group of NW waves per (sequence i,
// KV head g, partition p of `part_tokens` tokens).  Wave w folds tiles w, w+NW, ... of the partition.
// Launch order is g fastest, so consecutive work-groups (which the dispatcher
// spreads over the 8 XCDs) of one sequence and partition run on different XCDs
// while every work-group of one KV head lands on the same XCD.
//
// Lane layout (lane = 16 r + j, r = 0..3, j = 0..15), per 16-token tile:
//   K (A operand of S^T = K Q^T): lane reads key row j, dims 32 ks + 8 r .. +8
//     for ks = 0..3 (four 16-byte loads; each load instruction covers 64
//     contiguous bytes of all 16 rows).
//   Q (B operand): column j is query head g*G + j % G (heads repeat across the
//     16 columns), dims as for K; loaded once.
//   S^T (C): lane holds the scores of keys 4r .. 4r+3 for head j % G.
//   V: lane reads keys 4r .. 4r+3, dims 8j .. 8j+7 (each load instruction
//     covers 4 whole 256-byte rows), i.e. exactly the keys whose scores it
//     holds, for the head-dim chunk j.
// Row group r keeps its own online-softmax state per head: the running max and
// sum live in lane (r, h) (and its copies j = h mod G), the fp32 accumulator
// for chunk j of every head in lane (r, j).  P.V takes each weight from lane
// (r, h) with a DPP row broadcast, so no LDS or shuffles are needed per tile.
// Scores are kept in base-2 units (scale * log2 e) so exponentials are v_exp_f32.
//
// Masking selects, never multiplies: keys past the sequence end get score
// -inf and their V rows are zeroed, so stale or NaN slots never reach an
// accumulator.
//
// Partitioned finish: the row groups are combined with the log-sum-exp rule,
// then the NW waves through LDS.  A sequence with one partition writes its output;
// otherwise each partition writes (max, sum, acc) to the workspace and the
// merge kernel, launched next on the same stream, combines the partitions in
// ascending order.  (Merging inside this kernel -- the last partition to finish
// merging the rest -- needs an agent-scope release per partition, i.e. an L2
// write-back per work-group; measured on MI355X that serialises at roughly
// 0.5 us per partition per XCD and cost more than the separate launch.)
//
// Partitioned start-up: the block-table entries of a wave's first tiles are requested
// together with the sequence length (the index is clamped to the table, so
// the speculative read is always in bounds), which removes one dependent
// memory round trip from every work-group.
#include <cstdlib>
#include <cstring>

#include "device.h"
#include "ops.h"
#include "status.h"

namespace pa {
namespace {

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;                 // one bf16 token row of one KV head
constexpr int kTileBytes = kBlock * kRowBytes;    // one (block, KV head) tile: 4 KiB

struct MfmaDecodeArgs {
  AttnArgs a;
  int32_t part_tokens;
  int32_t max_parts;
  float* p_acc;        // [num_seqs][Hq][max_parts][D]
  float* p_ml;         // [num_seqs][Hq][max_parts][2]  (max in base-2 units, sum)
};

// Broadcast lane h (< 16) of each row; h is a compile-time constant after unrolling.
__device__ __forceinline__ float bcast(float x, int h) {
  switch (h) {
    case 0: return row_bcast<0>(x);
    case 1: return row_bcast<1>(x);
    case 2: return row_bcast<2>(x);
    case 3: return row_bcast<3>(x);
    case 4: return row_bcast<4>(x);
    case 5: return row_bcast<5>(x);
    case 6: return row_bcast<6>(x);
    case 7: return row_bcast<7>(x);
    case 8: return row_bcast<8>(x);
    case 9: return row_bcast<9>(x);
    case 10: return row_bcast<10>(x);
    case 11: return row_bcast<11>(x);
    case 12: return row_bcast<12>(x);
    case 13: return row_bcast<13>(x);
    case 14: return row_bcast<14>(x);
    default: return row_bcast<15>(x);
  }
}

template <int G>
struct WaveState {
  float m;           // running max (base 2) of row group r for head j % G
  float l;           // running sum of weights, same owner
  float acc[G][8];   // row group r's accumulator, dims 8j..8j+7 of every head
};

// Fold one tile (tokens tok0 .. tok0+15, of which those < t_end are valid).
template <int G>
__device__ __forceinline__ void fold(const uint4 (&kq)[4], uint4 (&vq)[4], const bf16x8_t (&qf)[4], int tok0,
                                     int t_end, int r, float scale_log2, WaveState<G>& st) {
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[ks]), qf[ks], s, 0, 0, 0);
  float sc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sc[e] = s[e] * scale_log2;
  if (tok0 + kBlock > t_end) {  // wave-uniform: only a sequence's last tile is partial
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool valid = tok0 + 4 * r + e < t_end;
      sc[e] = valid ? sc[e] : -INFINITY;
      if (!valid) vq[e] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  const bool need = mx > st.m + kRescaleSlack;
  if (__any(need)) {
    const float mn = need ? mx : st.m;
    const float alpha = fast_exp2(st.m - mn);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ah = bcast(alpha, h);
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[h][e] *= ah;
    }
  }
  float pr[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) pr[e] = fast_exp2(sc[e] - st.m);
  st.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float vf[8];
    widen_bf16x8(vq[u], vf);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pb = bcast(pr[u], h);
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[h][e] = fmaf(pb, vf[e], st.acc[h][e]);
    }
  }
}

template <int G, int NW>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(MfmaDecodeArgs k) {
  static_assert(16 % G == 0, "query heads per KV head must divide 16");
  __shared__ float s_ml[NW][G][2];
  __shared__ __attribute__((aligned(16))) float s_acc[NW][G][kD];

  const AttnArgs& a = k.a;
  const int Hkv = a.num_kv_heads;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int p = rest % k.max_parts;
  const int i = rest / k.max_parts;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int t0 = p * k.part_tokens;
  const int b_first = t0 / kBlock;
  const int32_t* bt_row = a.block_tables + (size_t)i * a.bt_stride;
  // Speculative: table entries of this wave's first 64 tiles, issued before the
  // length is known (clamped index, always inside the table row).
  const int bt_first = bt_row[min(b_first + w + lane * NW, a.bt_stride - 1)];
  const int q0 = a.qsl[i];
  if (a.qsl[i + 1] - q0 != 1 || q0 < 0 || q0 >= a.num_tokens) return;
  const int L = min(a.seq_lens[i], a.bt_stride * kBlock);
  if (t0 >= L) return;
  const int t1 = min(t0 + k.part_tokens, L);
  const int nparts = min((L + k.part_tokens - 1) / k.part_tokens, k.max_parts);

  const int j = lane & 15, r = lane >> 4;
  const int hq0 = g * G;

  bf16x8_t qf[4];
  {
    const uint8_t* qrow = (const uint8_t*)a.q + ((size_t)q0 * a.num_q_heads + hq0 + (j % G)) * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8_t, ld16(qrow + (4 * ks + r) * 16));
  }
  WaveState<G> st;
  st.m = kNegBig;
  st.l = 0.0f;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.0f;

  const uint8_t* kc = (const uint8_t*)a.k_cache + (size_t)g * kTileBytes;
  const uint8_t* vc = (const uint8_t*)a.v_cache + (size_t)g * kTileBytes;
  const size_t block_stride = (size_t)Hkv * kTileBytes;
  const int koff = j * kRowBytes + r * 16;        // + 64 ks
  const int voff = 4 * r * kRowBytes + j * 16;    // + kRowBytes u
  const int nbt = (t1 - 1) / kBlock - b_first + 1;
  const int cnt = nbt > w ? (nbt - w + NW - 1) / NW : 0;

  for (int cb = 0; cb < cnt; cb += 64) {
    const int nb = min(64, cnt - cb);
    const int entry = cb == 0 ? bt_first : bt_row[min(b_first + w + (cb + lane) * NW, a.bt_stride - 1)];
    const int my_bid = lane < nb ? clamp_block(entry, a.num_blocks) : 0;
    uint4 ka[4], va[4], kb[4], vb[4];
    // A prefetch past the last block (jj >= nb) reads an empty range: zeros, no memory traffic.
    auto issue = [&](int jj, uint4 (&kq)[4], uint4 (&vq)[4]) {
      const int bytes = jj < nb ? kTileBytes : 0;
      const size_t off = (size_t)__builtin_amdgcn_readlane(my_bid, min(jj, nb - 1)) * block_stride;
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc + off, bytes);
      const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc + off, bytes);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kq[ks] = buf_ld16(rk, koff + ks * 64);
#pragma unroll
      for (int u = 0; u < 4; ++u) vq[u] = buf_ld16(rv, voff + u * kRowBytes);
      // Keep the loads ahead of the fold that follows, so the wait before
      // the fold covers only the tile it consumes.
      __builtin_amdgcn_sched_barrier(0);
    };
    const int tok_base = (b_first + w + cb * NW) * kBlock;
    issue(0, ka, va);
    for (int jj = 0; jj < nb; jj += 2) {
      issue(jj + 1, kb, vb);
      fold<G>(ka, va, qf, tok_base + jj * NW * kBlock, t1, r, a.scale_log2, st);
      if (jj + 1 >= nb) break;
      issue(jj + 2, ka, va);
      fold<G>(kb, vb, qf, tok_base + (jj + 1) * NW * kBlock, t1, r, a.scale_log2, st);
    }
  }

  // Combine the four row groups of this wave (lanes j, j+16, j+32, j+48).
  float M = fmaxf(st.m, __shfl_xor(st.m, 16));
  M = fmaxf(M, __shfl_xor(M, 32));
  const float f = fast_exp2(st.m - M);
  float lt = st.l * f;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float fh = bcast(f, h);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = st.acc[h][e] * fh;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      st.acc[h][e] = x;
    }
  }
  if (r == 0 && j < G) {
    s_ml[w][j][0] = M;
    s_ml[w][j][1] = lt;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if ((h & 3) == r) {
      float4* dst = reinterpret_cast<float4*>(&s_acc[w][h][8 * j]);
      dst[0] = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
      dst[1] = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
    }
  }
  __syncthreads();

  // Combine the waves; item = (head h, four dims 4 d4 .. 4 d4 + 3).
  const int Hq = a.num_q_heads;
  for (int it = tid; it < G * (kD / 4); it += 64 * NW) {
    const int h = it / (kD / 4), d4 = it % (kD / 4);
    float Ms = s_ml[0][h][0];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) Ms = fmaxf(Ms, s_ml[ww][h][0]);
    float den = 0.0f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float fw = fast_exp2(s_ml[ww][h][0] - Ms);
      den = fmaf(fw, s_ml[ww][h][1], den);
      const float4 x = *reinterpret_cast<const float4*>(&s_acc[ww][h][4 * d4]);
      num.x = fmaf(fw, x.x, num.x); num.y = fmaf(fw, x.y, num.y);
      num.z = fmaf(fw, x.z, num.z); num.w = fmaf(fw, x.w, num.w);
    }
    if (nparts == 1) {
      const float inv = 1.0f / den;
      uint8_t* op = (uint8_t*)a.out + ((size_t)q0 * Hq + hq0 + h) * kRowBytes + d4 * 8;
      *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(num.x * inv, num.y * inv),
                                                 pack_bf16x2(num.z * inv, num.w * inv));
    } else {
      const size_t item = ((size_t)i * Hq + hq0 + h) * k.max_parts + p;
      *reinterpret_cast<float4*>(k.p_acc + item * kD + 4 * d4) = num;
      if (d4 == 0) *reinterpret_cast<float2*>(k.p_ml + item * 2) = make_float2(Ms, den);
    }
  }
}

// ---------------------------------------------------------------------------
// Balanced one-round decode.
//
// A fixed grid of W = Hkv * Wg single-wave work-groups, every one of which
// has work: for KV head g, the decode tiles of all sequences are concatenated
// in batch order into one stream of `total` tiles, and wave rank r of that
// head takes tiles [r*total/Wg, (r+1)*total/Wg).  Every wave therefore moves
// the same bytes, all waves are resident at once and each CU holds the same
// number of them (no early-exiting work-groups to skew the dispatcher), and
// each wave pays the start-up latency chain once.  A wave whose range crosses
// sequence boundaries folds each sequence's part separately: a sequence it
// covers whole is written out directly; otherwise its part goes to partial
// slot i + r (unique: ranges are disjoint and ordered) and the merge kernel
// combines a sequence's parts in rank order.  The wave holding a sequence's
// first tile records (first rank, parts) for the merge.
constexpr int kMaxBalancedSeqs = 1024;   // prefix sums kept in LDS per wave

struct BalancedArgs {
  AttnArgs a;
  int32_t waves_per_head;   // Wg
  int32_t slots;            // partial slots per KV head: num_seqs + Wg
  float* p_acc;             // [Hkv][slots][G][D]
  float* p_ml;              // [Hkv][slots][G][2]  (max in base-2 units, sum)
  int2* seqinfo;            // [num_seqs]: (first rank, parts) of each decode sequence
};

inline size_t balanced_lds_bytes(int num_seqs) { return (size_t)(2 * num_seqs + 1) * sizeof(int); }


// Combine the four row groups (lanes j, j+16, j+32, j+48): afterwards every
// lane (r, j) holds the wave's max M and sum lt of head j % G and, for every
// head h, the accumulator of dims 8j .. 8j+7.
template <int G>
__device__ __forceinline__ void combine_row_groups(WaveState<G>& st, float& M, float& lt) {
  M = fmaxf(st.m, __shfl_xor(st.m, 16));
  M = fmaxf(M, __shfl_xor(M, 32));
  const float f = fast_exp2(st.m - M);
  lt = st.l * f;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float fh = bcast(f, h);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = st.acc[h][e] * fh;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      st.acc[h][e] = x;
    }
  }
}

// Write one finished segment of sequence i: the output when the segment is
// the whole sequence, else a partial in slot i + rank of this KV head.
template <int G>
__device__ __forceinline__ void finish_segment(const BalancedArgs& k, int i, int g, int rank, bool whole, int q0,
                                              WaveState<G>& st) {
  const AttnArgs& a = k.a;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, r = lane >> 4;
  float M, lt;
  combine_row_groups<G>(st, M, lt);
  const size_t slot = (size_t)g * k.slots + (size_t)(i + rank);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if ((h & 3) != r) continue;   // row group r writes heads r, r+4, ...
    if (whole) {
      const float inv = 1.0f / bcast(lt, h);
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = st.acc[h][e] * inv;
      uint8_t* op = (uint8_t*)a.out + ((size_t)q0 * a.num_q_heads + g * G + h) * kRowBytes + j * 16;
      st16(op, make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                          pack_bf16x2(f[6], f[7])));
    } else {
      float* dst = k.p_acc + (slot * G + h) * kD + 8 * j;
      *reinterpret_cast<float4*>(dst) = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
    }
  }
  if (!whole && r == 0 && j < G) *reinterpret_cast<float2*>(k.p_ml + (slot * G + j) * 2) = make_float2(M, lt);
}

// One wave streams its range of the KV head's concatenated tiles, NS tiles
// deep, through LDS: each tile is copied global -> LDS by the buffer unit
// (no registers hold data in flight), into one of NS stage buffers that are
// separate LDS arrays so that the wait before reading a stage covers only the
// copies into that stage.  Each lane copies, and later reads back, exactly
// the 16-byte pieces of the K and V tiles it uses, in the lane layout above.
// Block-table entries are looked up 64 tiles at a time, one tile per lane
// (sequence by binary search over the prefix sums), well ahead of use.  The
// query rows of the next segment's sequence are copied to LDS one segment
// ahead, so a sequence boundary only flushes the fold state: nothing issued
// there is waited on by the next fold.
//
// FW (a fused cache write, k_new / v_new set): the step's new token is not in
// the cache yet.  Its K and V rows are copied to LDS with the query rows, and
// the lanes of its row in the sequence's last tile take them instead of the
// cache's; merge_balanced_kernel then stores the rows into the cache.  A
// separate instantiation, so that the plain kernel's registers are untouched.
template <int G, int NS, bool FW>
__global__ __launch_bounds__(64) void decode_balanced_kernel(BalancedArgs k) {
  static_assert(16 % G == 0, "query heads per KV head must divide 16");
  static_assert(NS >= 2 && NS <= 4, "tiles in flight");
  // Per-sequence tables in dynamic LDS, sized by the batch (balanced_lds_bytes):
  // prefix sums of decode tiles [num_seqs + 1], then query row << 5 | (valid
  // keys of the last tile - 1) [num_seqs].
  extern __shared__ int s_dyn[];
  int* s_cum = s_dyn;
  int* s_meta = s_dyn + k.a.num_seqs + 1;
  __shared__ int s_raw[2][64];                   // lookup windows: block-table entry (copied), sequence, logical block
  __shared__ int s_sj[2][2][64];
  __shared__ __attribute__((aligned(16))) uint4 s_q[4 * 4 * G];    // next segment's query rows: [ks][r][h]
  __shared__ __attribute__((aligned(16))) uint4 s_new[2][32];      // fused write: new K row, then V row, by segment parity
  __shared__ __attribute__((aligned(16))) uint4 s_t0[512];         // tile stages: K [ks][lane], V [e][lane]
  __shared__ __attribute__((aligned(16))) uint4 s_t1[512];
  __shared__ __attribute__((aligned(16))) uint4 s_t2[512];
  __shared__ __attribute__((aligned(16))) uint4 s_t3[512];
  const AttnArgs& a = k.a;
  const int Hkv = a.num_kv_heads;
  const int g = blockIdx.x % Hkv, rank = blockIdx.x / Hkv;
  const int lane = threadIdx.x;
  const int S = a.num_seqs;

  // Decode tiles of every sequence (0 for sequences with other than one query
  // token), four chunks of 64 per batch so their loads overlap, then exclusive
  // prefix sums in place.
  for (int c0 = 0; c0 < S; c0 += 256) {
    int T[4], M[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = c0 + 64 * u + lane;
      T[u] = 0;
      M[u] = 0;
      if (i < S) {
        const int q0 = a.qsl[i], n = a.qsl[i + 1] - q0;
        const int len = min(a.seq_lens[i], a.bt_stride * kBlock);
        if (n == 1 && q0 >= 0 && q0 < a.num_tokens && len > 0) {
          T[u] = (len + kBlock - 1) / kBlock;
          M[u] = (q0 << 5) | (len - 1 - (T[u] - 1) * kBlock);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = c0 + 64 * u + lane;
      if (i < S) {
        s_cum[i] = T[u];
        s_meta[i] = M[u];
      }
    }
  }
  int carry = 0;
  for (int c0 = 0; c0 < S; c0 += 64) {
    const int i = c0 + lane;
    const int T = i < S ? s_cum[i] : 0;
    int x = T;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (i < S) s_cum[i] = carry + x - T;
    carry += __shfl(x, 63);
  }
  if (lane == 0) s_cum[S] = carry;
  __syncthreads();
  const int64_t total = carry;
  // With fewer tiles than waves, the first `total` ranks take one tile each,
  // so every rank that runs has a non-empty range and a sequence's parts sit
  // in consecutive ranks.
  const int Wg = (int)min((int64_t)k.waves_per_head, total);
  if (rank >= Wg) return;
  const int tb = (int)stream_start(rank, total, Wg);
  const int n = (int)(stream_start(rank + 1, total, Wg) - tb);

  // Lookup window w: tile 64 w + lane -> sequence and logical block (binary
  // search over the prefix sums) and its block-table entry, copied to LDS.
  const u32x4_t rbt = rsrc_words((const uint8_t*)a.block_tables,
                                 (int)min((int64_t)S * a.bt_stride * 4, (int64_t)0x7fffffff));
  auto lookup = [&](int window) {
    const int u = window * 64 + lane;
    int seq = 0, jt = 0;
    if (u < n) {
      const int t = tb + u;
      int lo = 0, hi = S - 1;   // largest i with s_cum[i] <= t (that sequence has tiles)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_cum[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      seq = lo;
      jt = t - s_cum[lo];
      lds_copy4(rbt, &s_raw[window & 1][0], (seq * a.bt_stride + jt) * 4);
    }
    s_sj[window & 1][0][lane] = seq;
    s_sj[window & 1][1][lane] = jt;
  };
  lookup(0);
  lookup(1);
  PA_VM_WAIT(0);
  int window = 0;

  const int j = lane & 15, r = lane >> 4;
  const int hq0 = g * G;
  // Query rows of sequence `seq` -> s_q, lane r * G + h copying dims 32 ks + 8 r .. +8 of head h.
  // With a fused cache write (k_new set), also the sequence's new K and V rows
  // -> s_new[par] when this range folds its last tile.
  constexpr bool fused = FW;
  auto copy_q = [&](int seq, int par) {
    const int q0 = __builtin_amdgcn_readfirstlane(s_meta[seq] >> 5);
    const u32x4_t rq = rsrc_words((const uint8_t*)a.q + ((size_t)q0 * a.num_q_heads + hq0) * kRowBytes, G * kRowBytes);
    if (lane < 4 * G) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) lds_copy16(rq, s_q + ks * 4 * G, (lane % G) * kRowBytes + (lane / G) * 16 + ks * 64);
    }
    if (fused && __builtin_amdgcn_readfirstlane(s_cum[seq + 1]) <= tb + n && lane < 32) {
      // lanes 0..15: the K row's 16-byte chunks; lanes 16..31: the V row's
      const uint8_t* src = (const uint8_t*)(lane < 16 ? a.k_new : a.v_new) +
                           ((size_t)q0 * Hkv + g) * kRowBytes + (lane & 15) * 16;
      lds_copy16_global(src, &s_new[par][0]);
    }
  };
  copy_q(__builtin_amdgcn_readfirstlane(s_sj[0][0][0]), 0);
  int seg = -1;             // this range's segment count - 1: s_new[seg & 1] holds the current one's rows
  int q_tile = -(NS - 1);   // tile whose issue followed the last query copy

  const uint8_t* kc = (const uint8_t*)a.k_cache + (size_t)g * kTileBytes;
  const uint8_t* vc = (const uint8_t*)a.v_cache + (size_t)g * kTileBytes;
  const size_t block_stride = (size_t)Hkv * kTileBytes;
  const int koff = j * kRowBytes + r * 16;
  const int voff = 4 * r * kRowBytes + j * 16;
  auto stage = [&](int sI) -> uint4* { return sI == 0 ? s_t0 : sI == 1 ? s_t1 : sI == 2 ? s_t2 : s_t3; };
  // A prefetch past the range (uu >= n) still issues its eight copies, so
  // that every wait counts the same operations, but through an empty range:
  // they read nothing and write zeros into a stage no later fold reads.
  auto issue = [&](int uu, int sI) {
    const int u = min(uu, n - 1);
    const int bytes = uu < n ? kTileBytes : 0;
    const int bid = clamp_block(__builtin_amdgcn_readfirstlane(s_raw[(u >> 6) & 1][u & 63]), a.num_blocks);
    const size_t off = (size_t)bid * block_stride;
    const u32x4_t rk = rsrc_words(kc + off, bytes);
    const u32x4_t rv = rsrc_words(vc + off, bytes);
    uint4* dst = stage(sI);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) lds_copy16_nt(rk, dst + ks * 64, koff + ks * 64);
#pragma unroll
    for (int e = 0; e < 4; ++e) lds_copy16_nt(rv, dst + 256 + e * 64, voff + e * kRowBytes);
  };
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0) issue(s0, s0);

  WaveState<G> st;
  bf16x8_t qf[4];
  int cur = -1, cur_end = 0, cur_j0 = 0, cur_jl = 0;
  for (int u0 = 0; u0 < n; u0 += NS) {
#pragma unroll
    for (int sI = 0; sI < NS; ++sI) {
      const int u = u0 + sI;
      if (u >= n) break;
      if ((u >> 6) != window) {
        // Window w begins: look up window w + 1 into the slot window w - 1
        // used.  Its first tile is issued NS - 1 tiles before window w + 1
        // begins; by then the per-tile waits below have covered the copies.
        ++window;
        lookup(window + 1);
      }
      const int seq = __builtin_amdgcn_readfirstlane(s_sj[window & 1][0][u & 63]);
      const int jt = __builtin_amdgcn_readfirstlane(s_sj[window & 1][1][u & 63]);
      if (seq != cur) {
        if (cur >= 0) {
          const int T = s_cum[cur + 1] - s_cum[cur];
          finish_segment<G>(k, cur, g, rank, cur_j0 == 0 && cur_jl + 1 == T, s_meta[cur] >> 5, st);
        }
        cur = seq;
        ++seg;
        const int meta = s_meta[seq];
        cur_end = (s_cum[seq + 1] - s_cum[seq] - 1) * kBlock + (meta & 31) + 1;   // sequence length
        cur_j0 = jt;
        if (jt == 0 && g == 0 && lane == 0) {
          const int last = stream_owner((int64_t)s_cum[seq + 1] - 1, total, Wg);
          k.seqinfo[seq] = make_int2(rank, last - rank + 1);
        }
        // This sequence's query copy was followed by the issues of tiles
        // q_tile .. u - 1 (eight copies each; at least one tile).
        __builtin_amdgcn_sched_barrier(0);
        wait_tiles(min(u - q_tile, NS - 1));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qf[ks] = __builtin_bit_cast(bf16x8_t, s_q[ks * 4 * G + r * G + j % G]);
        // The copy of the next sequence's rows overwrites s_q: the reads above come first.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        int nx = seq + 1;                      // next sequence with tiles, if this range reaches it
        while (nx < S && s_cum[nx + 1] == s_cum[nx]) ++nx;
        if (nx < S && s_cum[nx] < tb + n) {
          copy_q(nx, (seg + 1) & 1);
          q_tile = u;
        }
        st.m = kNegBig;
        st.l = 0.0f;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.0f;
      }
      // The stage refilled here was read by the previous fold; the copies
      // stay after those reads and ahead of the reads of this tile's stage,
      // which wait for this tile's copies: NS - 1 tiles were issued after them.
      __builtin_amdgcn_sched_barrier(0);
      issue(u + NS - 1, (sI + NS - 1) % NS);
      __builtin_amdgcn_sched_barrier(0);
      wait_tiles(NS - 1);
      cur_jl = jt;
      const lds_u32x4_t* src = (const lds_u32x4_t*)stage(sI);
      uint4 kq[4], vq[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kq[ks] = __builtin_bit_cast(uint4, src[ks * 64 + lane]);
#pragma unroll
      for (int e = 0; e < 4; ++e) vq[e] = __builtin_bit_cast(uint4, src[256 + e * 64 + lane]);
      if (fused && (jt + 1) * kBlock >= cur_end) {
        // The sequence's last tile: row rho = (L - 1) % 16 is the new token.
        // Its lanes take the new row (copied to s_new with the query rows)
        // instead of the cache's; the merge kernel stores it into the cache.
        const int rho = (cur_end - 1) & (kBlock - 1);
        const uint4* nr = s_new[seg & 1];
        if (j == rho) {   // K piece ks: lane (r, j) holds bytes 64 ks + 16 r of row j
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) kq[ks] = nr[ks * 4 + r];
        }
        if (r == (rho >> 2)) {   // V piece e: lane (r, j) holds bytes 16 j of row 4 r + e
          const uint4 nv = nr[16 + j];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e == (rho & 3)) vq[e] = nv;
        }
      }
      fold<G>(kq, vq, qf, jt * kBlock, cur_end, r, a.scale_log2, st);
    }
  }
  const int T = s_cum[cur + 1] - s_cum[cur];
  finish_segment<G>(k, cur, g, rank, cur_j0 == 0 && cur_jl + 1 == T, s_meta[cur] >> 5, st);
}

// Merge of the balanced decode's parts: one work-group of TPW threads per
// (sequence, KV head), for all G query heads of that head.  A part's G x D
// partial block is contiguous, so reading a part is one coalesced load of
// DPL floats per thread (thread = head * TPW/G + chunk).  The parts are
// folded in order with the log-sum-exp rule, U parts' loads in flight per
// round trip, and the output written.  One wave and eight parts in flight
// when the batch has a work-group per CU or more (its sequences have a few
// parts); with fewer (a few long sequences, each cut into many parts), up to
// four waves and sixteen parts in flight, so that each sequence costs one
// round trip (measured on MI355X on eight 32K-128K sequences cut into ~16
// parts each: the step 389.6 -> 388.8 us).
template <int G, int TPW, int U>
__global__ __launch_bounds__(TPW) void merge_balanced_kernel(BalancedArgs k) {
  constexpr int LPH = TPW / G;         // threads per head
  constexpr int DPL = kD / LPH;        // dims per thread
  static_assert(DPL == 2 || DPL % 4 == 0, "dims per thread");
  const AttnArgs& a = k.a;
  const int i = blockIdx.x / a.num_kv_heads, g = blockIdx.x % a.num_kv_heads;
  const int lane = threadIdx.x, h = lane / LPH, c = lane % LPH;
  // Two memory round trips: first everything that depends on i alone (this
  // call's decode kernel wrote seqinfo for every sequence it took), then the
  // new rows, their table entry and the parts' partials together.
  const int q0 = a.qsl[i], q1 = a.qsl[i + 1];
  const int len = a.seq_lens[i];
  const int2 si = k.seqinfo[i];
  // (An empty asm reading all four values keeps the compiler from sinking the
  // later loads below the checks, which would make them serial round trips.)
  asm volatile("" ::"s"(q0), "s"(q1), "s"(len), "s"(si.x), "s"(si.y));
  if (q1 - q0 != 1 || q0 < 0 || q0 >= a.num_tokens) return;
  const int L = min(len, a.bt_stride * kBlock);
  if (L <= 0) return;
  // Fused cache write: the new token's K (lanes 0..15) and V (16..31) row
  // into its slot, position L - 1, stored after the partials' loads are
  // issued.  The decode kernel, which ran before, took this row from k_new /
  // v_new, not from the cache.
  // Each of those lanes loads the table entry itself, so nothing waits for
  // it before the partials' loads are issued.
  const bool fw = a.k_new != nullptr;
  uint4 x_new = make_uint4(0u, 0u, 0u, 0u);
  int bid_new = 0;
  if (fw && lane < 32) {
    bid_new = a.block_tables[(size_t)i * a.bt_stride + (L - 1) / kBlock];
    x_new = ld16((const uint8_t*)(lane < 16 ? a.k_new : a.v_new) + ((size_t)q0 * a.num_kv_heads + g) * kRowBytes +
                 (lane & 15) * 16);
  }
  auto store_new = [&]() {
    if (!fw || lane >= 32) return;
    const size_t dst = ((size_t)clamp_block(bid_new, a.num_blocks) * a.num_kv_heads + g) * kTileBytes +
                       ((L - 1) % kBlock) * kRowBytes + (lane & 15) * 16;
    st16((uint8_t*)(lane < 16 ? a.k_cache : a.v_cache) + dst, x_new);
  };
  const int P = si.y;
  if (P <= 1) {                          // written out by the decode kernel
    store_new();
    return;
  }
  const size_t slot0 = (size_t)g * k.slots + (size_t)(i + si.x);
  float Mx = -INFINITY, den = 0.0f;
  float num[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) num[e] = 0.0f;
  // Parts p0 .. p0 + U - 1.  All U parts' loads are issued unconditionally
  // (past the last part they re-read it, unused), so that they are in flight
  // together; the first batch is straight-line code, so nothing before it
  // (the new rows' loads) is waited for at a loop head.
  auto batch = [&](int p0) {
    float2 ml[U];
    float x[U][DPL];   // this thread's DPL dims of part p0 + u
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t e = (slot0 + min(p0 + u, P - 1)) * G + h;
      ml[u] = reinterpret_cast<const float2*>(k.p_ml)[e];
      const float* src = k.p_acc + e * kD + c * DPL;
      if constexpr (DPL % 4 == 0) {
#pragma unroll
        for (int v = 0; v < DPL / 4; ++v) {
          const float4 t = reinterpret_cast<const float4*>(src)[v];
          x[u][4 * v] = t.x; x[u][4 * v + 1] = t.y; x[u][4 * v + 2] = t.z; x[u][4 * v + 3] = t.w;
        }
      } else {
        const float2 t = *reinterpret_cast<const float2*>(src);
        x[u][0] = t.x; x[u][1] = t.y;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (p0 + u < P) {
        const float Mn = fmaxf(Mx, ml[u].x);
        const float sa = fast_exp2(Mx - Mn), sb = fast_exp2(ml[u].x - Mn);
        den = fmaf(den, sa, ml[u].y * sb);
#pragma unroll
        for (int e = 0; e < DPL; ++e) num[e] = fmaf(num[e], sa, x[u][e] * sb);
        Mx = Mn;
      }
    }
  };
  batch(0);
  for (int p0 = U; p0 < P; p0 += U) batch(p0);
  store_new();
  const float inv = 1.0f / den;
  uint32_t wd[DPL / 2];
#pragma unroll
  for (int e = 0; e < DPL / 2; ++e) wd[e] = pack_bf16x2(num[2 * e] * inv, num[2 * e + 1] * inv);
  uint8_t* op = (uint8_t*)a.out + ((size_t)q0 * a.num_q_heads + g * G + h) * kRowBytes + c * DPL * 2;
  if constexpr (DPL == 2) {
    *reinterpret_cast<uint32_t*>(op) = wd[0];
  } else if constexpr (DPL == 4) {
    *reinterpret_cast<uint2*>(op) = make_uint2(wd[0], wd[1]);
  } else {
#pragma unroll
    for (int v = 0; v < DPL / 8; ++v)
      *reinterpret_cast<uint4*>(op + 16 * v) = make_uint4(wd[4 * v], wd[4 * v + 1], wd[4 * v + 2], wd[4 * v + 3]);
  }
}

template <int NW>
pa_status launch_nw(const MfmaDecodeArgs& k, int G, dim3 grid, hipStream_t s) {
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: %d query heads per KV head", G);
  const int mark = trace_begin(s);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_mfma_kernel<1, NW>), grid, dim3(64 * NW), 0, s, k); break;
    case 2: hipLaunchKernelGGL((decode_mfma_kernel<2, NW>), grid, dim3(64 * NW), 0, s, k); break;
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<4, NW>), grid, dim3(64 * NW), 0, s, k); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<8, NW>), grid, dim3(64 * NW), 0, s, k); break;
    default: return fail(PA_ERR_UNSUPPORTED, "pa_forward: %d query heads per KV head", G);
  }
  trace_end(s, mark, "decode_mfma");
  return launch_status("pa_forward (decode, matrix cores)");
}

template <int G>
pa_status launch_balanced_g(const BalancedArgs& k, int depth, hipStream_t s) {
  const int W = k.waves_per_head * k.a.num_kv_heads;
  const size_t lds = balanced_lds_bytes(k.a.num_seqs);
  int mark = trace_begin(s);
  // the fused cache write is its own instantiation: the plain kernel keeps its registers
  if (k.a.k_new != nullptr) {
    if (depth == 4) hipLaunchKernelGGL((decode_balanced_kernel<G, 4, true>), dim3(W), dim3(64), lds, s, k);
    else if (depth == 3) hipLaunchKernelGGL((decode_balanced_kernel<G, 3, true>), dim3(W), dim3(64), lds, s, k);
    else hipLaunchKernelGGL((decode_balanced_kernel<G, 2, true>), dim3(W), dim3(64), lds, s, k);
  } else {
    if (depth == 4) hipLaunchKernelGGL((decode_balanced_kernel<G, 4, false>), dim3(W), dim3(64), lds, s, k);
    else if (depth == 3) hipLaunchKernelGGL((decode_balanced_kernel<G, 3, false>), dim3(W), dim3(64), lds, s, k);
    else hipLaunchKernelGGL((decode_balanced_kernel<G, 2, false>), dim3(W), dim3(64), lds, s, k);
  }
  trace_end(s, mark, "decode_mfma");
  pa_status st = launch_status("pa_forward (decode, balanced)");
  if (st != PA_OK) return st;
  mark = trace_begin(s);
  const dim3 mgrid(k.a.num_seqs * k.a.num_kv_heads);
  constexpr int kWide = 64 * (G < 4 ? G : 4);
  if (k.a.num_seqs * k.a.num_kv_heads < 256 && G > 1)
    hipLaunchKernelGGL((merge_balanced_kernel<G, kWide, 16>), mgrid, dim3(kWide), 0, s, k);
  else
    hipLaunchKernelGGL((merge_balanced_kernel<G, 64, 8>), mgrid, dim3(64), 0, s, k);
  trace_end(s, mark, "merge");
  return launch_status("pa_forward (decode merge, balanced)");
}

}  // namespace

bool decode_balanced_supported(int32_t num_seqs) { return num_seqs >= 1 && num_seqs <= kMaxBalancedSeqs; }

pa_status launch_decode_balanced(const AttnArgs& a, const DecodePlan& plan, float* p_acc, float* p_ml,
                                 int32_t* part_table, hipStream_t s) {
  BalancedArgs k{a, plan.waves_per_head, a.num_seqs + plan.waves_per_head, p_acc, p_ml, (int2*)part_table};
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_balanced_g<1>(k, plan.depth, s);
    case 2: return launch_balanced_g<2>(k, plan.depth, s);
    case 4: return launch_balanced_g<4>(k, plan.depth, s);
    case 8: return launch_balanced_g<8>(k, plan.depth, s);
    default: return fail(PA_ERR_UNSUPPORTED, "pa_forward: %d query heads per KV head", a.num_q_heads / a.num_kv_heads);
  }
}

bool decode_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  return dtype == PA_BF16 && head_dim == kD && (group == 1 || group == 2 || group == 4 || group == 8);
}

pa_status launch_decode_mfma(const AttnArgs& a, const DecodePlan& plan, float* p_acc, float* p_ml,
                             hipStream_t s) {
  MfmaDecodeArgs k{a, plan.part_tokens, plan.max_parts, p_acc, p_ml};
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t wgs = (int64_t)a.num_kv_heads * plan.max_parts * a.num_seqs;
  if (wgs > 0x7fffffff / 256) return fail(PA_ERR_UNSUPPORTED, "pa_forward: decode grid of %lld work-groups", (long long)wgs);
  dim3 grid((unsigned)wgs);
  switch (plan.waves) {
    case 1: return launch_nw<1>(k, G, grid, s);
    case 2: return launch_nw<2>(k, G, grid, s);
    case 4: return launch_nw<4>(k, G, grid, s);
    default: return fail(PA_ERR_ARG, "pa_forward: %d waves per decode work-group", plan.waves);
  }
}

}  // namespace pa
