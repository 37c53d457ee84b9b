// Single-token decode for a batch whose sequences share prefix blocks, each
// shared block read once for all the sequences that share it.
//
// "Was ändert PagedAttention an der KV-Speicherzuweisung für LLMs?"
// (slavadubrov.com), section "Gemeinsame Nutzung erfordert mehr als
// Speicherzuweisung", and "PagedAttention et vLLM" (aiunderstanding.org), FAQ
// on sharing: several requests point at the same physical blocks (a common
// prompt, parallel samples of one prompt).  Attention itself is unchanged --
// each sequence's query attends to its own tokens ("Внутреннее устройство vLLM"
// (artificials.ru), forward-pass paragraph) -- but a block that G query heads
// of P sequences all read can be streamed once and multiplied by all P x G
// query rows together: the (sequence, query head) pairs become the columns of
// the matrix-core products, exactly as the (token, query head) pairs of a
// multi-token decode do.
//
// Sharing is given by the caller: shared_blocks[i] = the number of leading
// block-table entries sequence i has in common with sequence i - 1 (the host
// allocator reports it, pa_alloc_shared_blocks).  Sequences are grouped in
// fixed runs of P = 16 CG / G consecutive batch entries; group [kP, kP + P)
// has a shared prefix of F full tiles, F = the minimum over its members of
// floor(L / 16) and over all but its first member of shared_blocks (0 unless
// every member is a single-token sequence and there are two or more).  Per KV
// head, the tile stream holds, for each sequence i in batch order:
//   item 2i     -- when i starts a group with F > 0: the group's prefix,
//                  tiles 0 .. F-1 of i's table, columns (member m, head h) ->
//                  c = m G + h, queries = the members' rows (consecutive);
//   item 2i + 1 -- i's own tiles F .. T_i - 1, columns h (its query row).
// The balanced one-round scheme of the single- and multi-token decodes then
// applies unchanged: the stream is cut into equal ranges, one single-wave
// work-group per range; tiles are copied global -> LDS by the buffer unit NS
// deep; the fold is the multi-token decode's (S^T = K Q^T and O^T += V^T P^T
// on the matrix cores, per-column online softmax, P rounded to bf16).  Each
// segment of an item writes an fp32 partial (max, sum, acc per column); a
// sequence with no prefix item whose own tiles sit in one segment is written
// out directly.  merge_shared_kernel then folds, for every sequence and KV
// head, the parts of its group's prefix item (its columns) and of its own item
// by the log-sum-exp rule, in a fixed order.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "device.h"
#include "ops.h"
#include "status.h"

namespace pa {
namespace {

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;                 // one bf16 token row of one KV head
constexpr int kTileBytes = kBlock * kRowBytes;    // one (block, KV head) tile: 4 KiB
constexpr int kMaxSharedSeqs = 512;               // per-sequence tables kept in LDS

struct SharedArgs {
  AttnArgs a;
  const int32_t* shared_blocks;   // [num_seqs]
  int32_t waves_per_head;         // Wg
  int32_t slots;                  // partial slots per KV head: 2 num_seqs + Wg
  uint16_t* p_acc;                // [Hkv][slots][CG][8 db][64 lanes][4] fp16: fragment order
  float* p_ml;                    // [Hkv][slots][16 CG][4]  (max in base-2 units, sum, e, 0)
  int2* item_info;                // [2 num_seqs]: (first rank, parts) of each item
  int32_t* seq_prefix;            // [num_seqs]: F of the sequence's group (0: none)
};

// Dynamic LDS: tile prefix sums [S + 1], then per sequence its length (0 when
// it is not a single-token sequence), query row and group prefix F.
inline size_t shared_dyn_lds(int num_seqs) { return (size_t)(4 * num_seqs + 1) * sizeof(int); }
inline size_t shared_static_lds(int cg, int ns) { return 3 * 512 + 1024 + (size_t)cg * 4096 + (size_t)ns * 8192; }

// Sequences per group: the 16 CG columns hold G query heads of each.
template <int G, int CG>
constexpr int members() { return 16 * CG / G; }

// A single-token sequence the kernel handles: its query row and length.
__device__ __forceinline__ bool shared_item(const AttnArgs& a, int i, int& q0, int& len) {
  q0 = a.qsl[i];
  const int n = a.qsl[i + 1] - q0;
  len = min(a.seq_lens[i], a.bt_stride * kBlock);
  return n == 1 && q0 >= 0 && q0 < a.num_tokens && len > 0;
}

// Wait until at most 8 t vector memory operations (t tiles' copies) are outstanding.
__device__ __forceinline__ void wait_copies(int t) {
  if (t <= 1) PA_VM_WAIT(8);
  else if (t == 2) PA_VM_WAIT(16);
  else PA_VM_WAIT(24);
}

template <int CG>
struct ColsState {
  float m[CG];          // running max (base 2) of the lane's column, the same in its four lanes
  float l[CG];          // this lane's share of the column's weight sum
  f32x4_t acc[CG][8];   // O^T: column j, dims 16 db + 4 r .. +3
};

// FW (a fused cache write, k_new / v_new set): the step's new token is not in
// the cache yet.  A sequence's new K and V rows are copied to LDS with the
// query rows of its own item, and in that item's last tile the lanes of row
// (L - 1) mod 16 take them instead of the cache's (K in registers, V patched
// into the stage before the transpose reads); merge_shared_kernel stores the
// rows into the cache.  A separate instantiation.
template <int G, int CG, int NS, bool FW>
__global__ __launch_bounds__(64) void decode_shared_kernel(SharedArgs k) {
  static_assert(16 % G == 0, "query heads per KV head must divide 16");
  static_assert(NS >= 2 && NS <= 3, "tiles in flight");
  constexpr int P = members<G, CG>();
  static_assert(64 % P == 0, "a group of sequences sits in one chunk of 64");
  constexpr int C = 16 * CG;
  extern __shared__ int s_dyn[];
  const AttnArgs& a = k.a;
  const int S = a.num_seqs;
  int* s_cum = s_dyn;
  int* s_len = s_dyn + S + 1;
  int* s_q0 = s_len + S;
  int* s_F = s_q0 + S;
  __shared__ int s_raw[2][64];      // lookup windows: block-table entry (copied), sequence, packed tile
  __shared__ int s_sj[2][2][64];
  __shared__ __attribute__((aligned(16))) uint4 s_q[CG * 4 * 64];    // query rows: [cg][ks][lane]
  __shared__ __attribute__((aligned(16))) uint4 s_st[NS][512];       // K [ks][lane], V [db][16 keys][16 dims]
  __shared__ __attribute__((aligned(16))) uint4 s_new[FW ? 2 : 1][32]; // FW: new K row, then V row, by item parity
  const int Hkv = a.num_kv_heads;
  const int g = blockIdx.x % Hkv, rank = blockIdx.x / Hkv;
  const int lane = threadIdx.x;

  // Per sequence: length, query row, and its group's prefix F (a minimum
  // over the group's P lanes: P divides 64, so a group never straddles a
  // chunk of 64); then tile counts and their exclusive prefix sums.
  int carry = 0;
  for (int c0 = 0; c0 < S; c0 += 64) {
    const int i = c0 + lane;
    int q0 = 0, len = 0;
    const bool dec = i < S && shared_item(a, i, q0, len);
    if (!dec) len = 0;
    const int first = i - i % P;
    int v = 0x7fffffff;                           // lanes past the batch do not limit their group
    if (i < S) {
      v = dec ? len / kBlock : 0;
      if (i != first) v = min(v, max(k.shared_blocks[i], 0));
    }
#pragma unroll
    for (int off = 1; off < P; off <<= 1) v = min(v, __shfl_xor(v, off));
    const int F = min(S - first, P) >= 2 ? v : 0;
    const int T = (len + kBlock - 1) / kBlock;
    const int cnt = i < S ? (i == first ? F : 0) + (dec ? T - F : 0) : 0;
    int x = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (i < S) {
      s_cum[i] = carry + x - cnt;
      s_len[i] = len;
      s_q0[i] = q0;
      s_F[i] = F;
      if (g == 0 && rank == 0) k.seq_prefix[i] = F;
    }
    carry += __shfl(x, 63);
  }
  if (lane == 0) s_cum[S] = carry;
  __syncthreads();
  const int64_t total = carry;
  const int Wg = (int)min((int64_t)k.waves_per_head, total);
  if (rank >= Wg) return;
  const int tb = (int)stream_start(rank, total, Wg);
  const int cnt = (int)(stream_start(rank + 1, total, Wg) - tb);

  // Lookup window w: tile 64 w + lane -> sequence i, item kind (0: its
  // group's prefix, 1: its own tiles) and logical block jt, with the rows of
  // the block that the item's columns see; its block-table entry is copied
  // to LDS.  s_sj[w][1] = jt | kind << 15 | rows << 16.
  const u32x4_t rbt = rsrc_words((const uint8_t*)a.block_tables,
                                 (int)min((int64_t)S * a.bt_stride * 4, (int64_t)0x7fffffff));
  auto lookup = [&](int window) {
    const int u = window * 64 + lane;
    int seq = 0, packed = kBlock << 16;
    if (u < cnt) {
      const int t = tb + u;
      int lo = 0, hi = S - 1;   // largest i with s_cum[i] <= t (that sequence has tiles)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_cum[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      seq = lo;
      const int F = s_F[lo];
      const int tp = lo % P == 0 ? F : 0;
      const int off = t - s_cum[lo];
      int jt, kind, rows = kBlock;
      if (off < tp) {
        jt = off;
        kind = 0;
      } else {
        jt = F + off - tp;
        kind = 1;
        rows = min(s_len[lo] - jt * kBlock, kBlock);
      }
      packed = jt | (kind << 15) | (rows << 16);
      lds_copy4(rbt, &s_raw[window & 1][0], (seq * a.bt_stride + jt) * 4);
    }
    s_sj[window & 1][0][lane] = seq;
    s_sj[window & 1][1][lane] = packed;
  };
  lookup(0);
  lookup(1);
  PA_VM_WAIT(0);
  int window = 0;

  const int j = lane & 15, r = lane >> 4;
  const int hq0 = g * G;
  // Query rows of an item -> s_q: copy (cg, ks) has lane (r, j) fetch the
  // eight dims of column 16 cg + j (member c / G, head c % G) that k-step ks
  // pairs with this lane's K operand.  The buffer range ends at the item's
  // last query row, so columns past its members read zeros.
  auto copy_q = [&](int seq_in, int kind_in, int par) {
    const int seq = __builtin_amdgcn_readfirstlane(seq_in), kind = __builtin_amdgcn_readfirstlane(kind_in);
    const int q0 = __builtin_amdgcn_readfirstlane(s_q0[seq]);
    // FW: the sequence's new K / V rows (lanes 0..15 / 16..31) when this range
    // folds its last tile, which is its own item's (the block holding the new
    // token is the sequence's own).
    if (FW && kind == 1 && __builtin_amdgcn_readfirstlane(s_cum[seq + 1]) <= tb + cnt && lane < 32) {
      const uint8_t* src = (const uint8_t*)(lane < 16 ? a.k_new : a.v_new) +
                           ((size_t)q0 * Hkv + g) * kRowBytes + (lane & 15) * 16;
      lds_copy16_global(src, &s_new[FW ? par : 0][0]);
    }
    const int nq = kind == 0 ? min(P, S - seq) : 1;
    const u32x4_t rq = rsrc_words((const uint8_t*)a.q + (size_t)q0 * a.num_q_heads * kRowBytes,
                                  nq * a.num_q_heads * kRowBytes);
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      const int col = 16 * cg + j;
      const int off = ((col / G) * a.num_q_heads + hq0 + col % G) * kRowBytes + r * 16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) lds_copy16(rq, s_q + (cg * 4 + ks) * 64, off + ks * 64);
    }
  };
  {
    const int p0 = __builtin_amdgcn_readfirstlane(s_sj[0][1][0]);
    copy_q(__builtin_amdgcn_readfirstlane(s_sj[0][0][0]), (p0 >> 15) & 1, 0);
  }
  int itm = -1;             // this range's item count - 1: s_new[itm & 1] holds the current item's rows
  int q_tile = -(NS - 1);   // tile whose issue followed the last query copy

  const uint8_t* kc = (const uint8_t*)a.k_cache + (size_t)g * kTileBytes;
  const uint8_t* vc = (const uint8_t*)a.v_cache + (size_t)g * kTileBytes;
  const size_t block_stride = (size_t)Hkv * kTileBytes;
  // K piece ks: lane (r, j) copies key j, dims 32 ks + 8 r .. +8.  V piece p
  // (dim blocks 2p, 2p+1): lane 32 dsel + 2 key + half copies key `key`, dims
  // 16 (2p + dsel) + 8 half .. +8, landing in row `key` of the [16 keys][16
  // dims] sub-tile of dim block 2p + dsel.
  const int koff = j * kRowBytes + r * 16;
  const int voff = ((lane & 31) >> 1) * kRowBytes + (lane >> 5) * 32 + (lane & 1) * 16;
  // A prefetch past the range (uu >= cnt) still issues its eight copies, so
  // that every wait counts the same operations, but through an empty range:
  // they read nothing and write zeros into a stage no later fold reads.
  auto issue = [&](int uu, int sI) {
    const int u = min(uu, cnt - 1);
    const int w = (u >> 6) & 1, e = u & 63;
    const int bid = clamp_block(__builtin_amdgcn_readfirstlane(s_raw[w][e]), a.num_blocks);
    const size_t off = (size_t)bid * block_stride;
    // Rows the item does not see (past a sequence's last token) read as zero.
    const int bytes = uu < cnt ? __builtin_amdgcn_readfirstlane(s_sj[w][1][e] >> 16) * kRowBytes : 0;
    const u32x4_t rk = rsrc_words(kc + off, bytes);
    const u32x4_t rv = rsrc_words(vc + off, bytes);
    uint4* dst = s_st[sI];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) lds_copy16_nt(rk, dst + ks * 64, koff + ks * 64);
#pragma unroll
    for (int p = 0; p < 4; ++p) lds_copy16_nt(rv, dst + 256 + p * 64, voff + p * 64);
  };
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0) issue(s0, s0);

  // Transposed-read address of this lane inside a [16 keys][16 dims] sub-tile:
  // row group r points at key rows 4r .. 4r+3, four lanes per row, four dims each.
  const int tr_off = (4 * r + j / 4) * 32 + (j & 3) * 8;

  ColsState<CG> st;
  bf16x8_t qf[CG][4];
  // Current segment: item (2 seq + kind), its query row and rows, active
  // column groups, key limit, and the first and last logical block it folded.
  int cur = -1, cur_seq = 0, cur_kind = 0, cur_q0 = 0, cur_nq = 1, cga = 1, key_end = 0, cur_j0 = 0, cur_jl = 0;

  // The item's whole tile range sits in this segment?
  auto whole = [&]() -> bool {
    const int F = s_F[cur_seq];
    if (cur_kind == 0) return cur_j0 == 0 && cur_jl == F - 1;
    const int T = (s_len[cur_seq] + kBlock - 1) / kBlock;
    return cur_j0 == F && cur_jl == T - 1;
  };
  auto finish = [&]() {
    const bool direct = cur_kind == 1 && s_F[cur_seq] == 0 && whole();
    const size_t slot = (size_t)g * k.slots + (size_t)(cur + rank);
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      if (cg > 0 && cg >= cga) break;   // group 0 is always active
      float lt = st.l[cg];
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
      const int col = 16 * cg + j;
      if (col / G >= cur_nq) continue;
      if (direct) {
        const float inv = 1.0f / lt;
        uint8_t* op = (uint8_t*)a.out + ((size_t)cur_q0 * a.num_q_heads + hq0 + col) * kRowBytes + r * 8;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const f32x4_t x = st.acc[cg][db];
          *reinterpret_cast<uint2*>(op + db * 32) =
              make_uint2(pack_bf16x2(x[0] * inv, x[1] * inv), pack_bf16x2(x[2] * inv, x[3] * inv));
        }
      } else {
        // The column's output normalised by its weight sum, times 2^-e in
        // fp16 (e from the column's largest magnitude over its four lanes:
        // values in [2^14, 2^15), exact power-of-two scalings), in fragment
        // order, with (max, sum, e); sum 0 (no key seen) weighs 0 in the merge.
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        float amax = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(st.acc[cg][db][e] * inv));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int ex = amax > 0.0f ? max(ilogbf(amax) - 14, -100) : 0;
        uint16_t* dst = k.p_acc + ((slot * CG + cg) * 8 * 64 + lane) * 4;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          uint32_t w[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const _Float16 lo = static_cast<_Float16>(ldexpf(st.acc[cg][db][2 * hh] * inv, -ex));
            const _Float16 hi = static_cast<_Float16>(ldexpf(st.acc[cg][db][2 * hh + 1] * inv, -ex));
            w[hh] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
          *reinterpret_cast<uint2*>(dst + db * 256) = make_uint2(w[0], w[1]);
        }
        if (r == 0)
          *reinterpret_cast<float4*>(k.p_ml + (slot * C + col) * 4) = make_float4(st.m[cg], lt, (float)ex, 0.0f);
      }
    }
  };

  for (int u0 = 0; u0 < cnt; u0 += NS) {
#pragma unroll
    for (int sI = 0; sI < NS; ++sI) {
      const int u = u0 + sI;
      if (u >= cnt) break;
      if ((u >> 6) != window) {
        // Window w begins: look up window w + 1 into the slot window w - 1 used.
        ++window;
        lookup(window + 1);
      }
      const int seq = __builtin_amdgcn_readfirstlane(s_sj[window & 1][0][u & 63]);
      const int packed = __builtin_amdgcn_readfirstlane(s_sj[window & 1][1][u & 63]);
      const int jt = packed & 0x7fff, kind = (packed >> 15) & 1;
      const int item = 2 * seq + kind;
      if (item != cur) {
        if (cur >= 0) finish();
        cur = item;
        ++itm;
        cur_seq = seq;
        cur_kind = kind;
        cur_q0 = __builtin_amdgcn_readfirstlane(s_q0[seq]);
        cur_nq = kind == 0 ? min(P, S - seq) : 1;
        cga = min(CG, (cur_nq * G + 15) / 16);
        key_end = kind == 0 ? s_F[seq] * kBlock : s_len[seq];
        cur_j0 = jt;
        if (g == 0 && lane == 0 && jt == (kind == 0 ? 0 : s_F[seq])) {
          // This wave holds the item's first tile: record (first rank, parts).
          const int tp = seq % P == 0 ? s_F[seq] : 0;
          const int64_t last_tile = kind == 0 ? (int64_t)s_cum[seq] + tp - 1 : (int64_t)s_cum[seq + 1] - 1;
          const int last = stream_owner(last_tile, total, Wg);
          k.item_info[item] = make_int2(rank, last - rank + 1);
        }
        // This item's query copy was followed by the issues of tiles
        // q_tile .. u - 1 (eight copies each; at least one tile).
        __builtin_amdgcn_sched_barrier(0);
        wait_copies(min(u - q_tile, NS - 1));
        const lds_u32x4_t* qs = (const lds_u32x4_t*)s_q;
#pragma unroll
        for (int cg = 0; cg < CG; ++cg)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) qf[cg][ks] = __builtin_bit_cast(bf16x8_t, qs[(cg * 4 + ks) * 64 + lane]);
        // The copy of the next item's rows overwrites s_q: the reads above come first.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // The next item with tiles, if this range reaches it.
        int nseq = seq, nkind = kind;
        {
          int ns_ = seq, nk = kind;
          while (true) {
            if (nk == 0) {
              nk = 1;                                   // the same sequence's own tiles
            } else {
              ++ns_;
              nk = 0;
            }
            if (ns_ >= S) break;
            const int tp = ns_ % P == 0 ? s_F[ns_] : 0;
            const int first_tile = s_cum[ns_] + (nk == 0 ? 0 : tp);
            const int n_tiles = nk == 0 ? tp : s_cum[ns_ + 1] - s_cum[ns_] - tp;
            if (n_tiles > 0) {
              if (first_tile < tb + cnt) {
                nseq = ns_;
                nkind = nk;
              }
              break;
            }
          }
        }
        if (nseq != seq || nkind != kind) {
          copy_q(nseq, nkind, (itm + 1) & 1);
          q_tile = u;
        }
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) {
          st.m[cg] = kNegBig;
          st.l[cg] = 0.0f;
#pragma unroll
          for (int db = 0; db < 8; ++db) st.acc[cg][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
      // The stage refilled here was read by the previous fold; the copies
      // stay after those reads and ahead of the reads of this tile's stage,
      // which wait for this tile's copies: NS - 1 tiles were issued after them.
      __builtin_amdgcn_sched_barrier(0);
      issue(u + NS - 1, (sI + NS - 1) % NS);
      __builtin_amdgcn_sched_barrier(0);
      wait_copies(NS - 1);
      cur_jl = jt;
      const lds_u32x4_t* src = (const lds_u32x4_t*)s_st[sI];
      const uint8_t* sb = (const uint8_t*)s_st[sI];
      const int tok0 = jt * kBlock;
      uint4 kq[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kq[ks] = __builtin_bit_cast(uint4, src[ks * 64 + lane]);
      if (FW && cur_kind == 1 && tok0 + kBlock >= key_end) {
        // The sequence's last tile: row rho = (L - 1) % 16 is the new token.
        const int rho = (key_end - 1) & (kBlock - 1);
        const uint4* nr = s_new[FW ? (itm & 1) : 0];
        if (j == rho) {   // K piece ks: lane (r, j) holds bytes 64 ks + 16 r of row j
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) kq[ks] = nr[ks * 4 + r];
        }
        if (lane < 16)    // V: chunk `lane` (dims 8 lane .. +8) into row rho of sub-tile lane / 2
          s_st[sI][256 + (lane >> 1) * 32 + rho * 2 + (lane & 1)] = nr[16 + lane];
        asm volatile("" ::: "memory");   // the transpose reads below come after the patch
      }

      // Scores of the active column groups, base-2 units, masked past the item's keys.
      float sc[CG][4];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (cg > 0 && cg >= cga) break;   // group 0 is always active
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ks += 2) {
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[ks]), qf[cg][ks], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[ks + 1]), qf[cg][ks + 1], s1,
                                                        0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[cg][e] = (s0[e] + s1[e]) * a.scale_log2;
        if (tok0 + kBlock > key_end) {   // wave-uniform: only an item's last tile can be partial
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[cg][e] = tok0 + 4 * r + e < key_end ? sc[cg][e] : -INFINITY;
        }
      }
      // Lazy rescale, per column: only when some lane's scores beat its
      // column's reference by the slack are the column's four lanes reduced
      // to its tile max and the reference moved.
      bool need = false;
      float mx[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (cg > 0 && cg >= cga) break;
        mx[cg] = fmaxf(fmaxf(sc[cg][0], sc[cg][1]), fmaxf(sc[cg][2], sc[cg][3]));
        need |= mx[cg] > st.m[cg] + kRescaleSlack;
      }
      if (__any(need)) {
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) {
          if (cg > 0 && cg >= cga) break;
          float x = fmaxf(mx[cg], __shfl_xor(mx[cg], 16));
          x = fmaxf(x, __shfl_xor(x, 32));
          const float mn = x > st.m[cg] + kRescaleSlack ? x : st.m[cg];
          const float alpha = fast_exp2(st.m[cg] - mn);
          st.m[cg] = mn;
          st.l[cg] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) st.acc[cg][db] *= alpha;
        }
      }
      // Weights (bf16, as the product uses them), their sums, and O^T += V^T P^T.
      s16x4_t pb[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (cg > 0 && cg >= cga) break;
        f32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = fast_exp2(sc[cg][e] - st.m[cg]);
        const bf16x4_t wb = __builtin_convertvector(w, bf16x4_t);   // nearest even
        const f32x4_t wr = __builtin_convertvector(wb, f32x4_t);    // exact
        st.l[cg] += (wr[0] + wr[1]) + (wr[2] + wr[3]);
        pb[cg] = __builtin_bit_cast(s16x4_t, wb);
      }
      // All eight V^T operands are read before the first product, so their
      // LDS latencies overlap.
      s16x4_t vt[8];
#pragma unroll
      for (int db = 0; db < 8; ++db) vt[db] = lds_read_tr(sb + 4096 + tr_off + db * 512);
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (cg > 0 && cg >= cga) break;
#pragma unroll
        for (int db = 0; db < 8; ++db)
          st.acc[cg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[db], pb[cg], st.acc[cg][db], 0, 0, 0);
      }
    }
  }
  finish();
}

// Merge: one work-group per (sequence, KV head); thread (h, db, r) folds the
// parts of the sequence's group-prefix item (column m G + h, m = its place in
// the group) and then of its own item (column h), in rank order, by the
// log-sum-exp rule, four dims 16 db + 4 r .. +3 each, and writes the output.
// A sequence with no prefix item whose own item is one part was written out
// by the decode kernel.
template <int G, int CG>
__global__ __launch_bounds__(256) void merge_shared_kernel(SharedArgs k) {
  constexpr int P = members<G, CG>();
  constexpr int C = 16 * CG, U = 8;
  const AttnArgs& a = k.a;
  const int Hkv = a.num_kv_heads;
  const int i = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int t = threadIdx.x;
  if (t >= G * 32) return;
  int q0, len;
  if (!shared_item(a, i, q0, len)) return;
  if (a.k_new != nullptr && t < 32) {
    // Fused cache write: the new token's K (threads 0..15) and V (16..31) row
    // into its slot, position len - 1; the decode kernel took it from k_new / v_new.
    const int bid = clamp_block(a.block_tables[(size_t)i * a.bt_stride + (len - 1) / kBlock], a.num_blocks);
    const size_t src = ((size_t)q0 * Hkv + g) * kRowBytes + (t & 15) * 16;
    const size_t dst = ((size_t)bid * Hkv + g) * kTileBytes + ((len - 1) % kBlock) * kRowBytes + (t & 15) * 16;
    const uint4 x = ld16((const uint8_t*)(t < 16 ? a.k_new : a.v_new) + src);
    st16((uint8_t*)(t < 16 ? a.k_cache : a.v_cache) + dst, x);
  }
  const int F = k.seq_prefix[i];                  // written by this call's decode kernel
  const int T = (len + kBlock - 1) / kBlock;
  const int h = t / 32, db = (t / 4) % 8, r = t % 4;
  const int first = i - i % P, m = i - first;
  int2 own = make_int2(0, 0);
  if (T > F) own = k.item_info[2 * i + 1];
  if (F == 0 && own.y <= 1) return;               // written out by the decode kernel
  float M = -INFINITY, den = 0.0f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int pass = 0; pass < 2; ++pass) {
    int2 info;
    int col;
    size_t item;
    if (pass == 0) {
      if (F == 0) continue;
      item = 2 * (size_t)first;
      info = k.item_info[item];
      col = m * G + h;
    } else {
      if (T <= F) continue;
      item = 2 * (size_t)i + 1;
      info = own;
      col = h;
    }
    const size_t slot0 = (size_t)g * k.slots + item + info.x;
    const int cg = col / 16, ln = 16 * r + col % 16;
    const float4* ml = reinterpret_cast<const float4*>(k.p_ml) + slot0 * C + col;
    const uint16_t* acc = k.p_acc + (((slot0 * CG + cg) * 8 + db) * 64 + ln) * 4;
    for (int p0 = 0; p0 < info.y; p0 += U) {
      float4 v[U];
      uint2 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p0 + u < info.y) {
          v[u] = ml[(size_t)(p0 + u) * C];
          x[u] = *reinterpret_cast<const uint2*>(acc + (size_t)(p0 + u) * C * kD);   // one slot = C x D values
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p0 + u >= info.y) break;
        // Part u's output is sum * 2^e * (the stored values).
        const float Mn = fmaxf(M, v[u].x);
        const float sa = fast_exp2(M - Mn), sb = fast_exp2(v[u].x - Mn);
        den = fmaf(den, sa, v[u].y * sb);
        const float wv = ldexpf(v[u].y * sb, (int)v[u].z);
        auto h16 = [](uint32_t w, int hi) {
          return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(hi ? w >> 16 : w & 0xffffu)));
        };
        num.x = fmaf(num.x, sa, h16(x[u].x, 0) * wv);
        num.y = fmaf(num.y, sa, h16(x[u].x, 1) * wv);
        num.z = fmaf(num.z, sa, h16(x[u].y, 0) * wv);
        num.w = fmaf(num.w, sa, h16(x[u].y, 1) * wv);
        M = Mn;
      }
    }
  }
  const float inv = 1.0f / den;
  uint8_t* op = (uint8_t*)a.out + ((size_t)q0 * a.num_q_heads + g * G + h) * kRowBytes + (16 * db + 4 * r) * 2;
  *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(num.x * inv, num.y * inv),
                                             pack_bf16x2(num.z * inv, num.w * inv));
}

template <int G, int CG, int NS>
pa_status launch_shared_gn(const SharedArgs& k, hipStream_t s) {
  const int W = k.waves_per_head * k.a.num_kv_heads;
  int mark = trace_begin(s);
  if (k.a.k_new != nullptr)
    hipLaunchKernelGGL((decode_shared_kernel<G, CG, NS, true>), dim3(W), dim3(64), shared_dyn_lds(k.a.num_seqs), s, k);
  else
    hipLaunchKernelGGL((decode_shared_kernel<G, CG, NS, false>), dim3(W), dim3(64), shared_dyn_lds(k.a.num_seqs), s, k);
  trace_end(s, mark, "decode_shared");
  pa_status st = launch_status("pa_forward_shared (decode)");
  if (st != PA_OK) return st;
  mark = trace_begin(s);
  hipLaunchKernelGGL((merge_shared_kernel<G, CG>), dim3(k.a.num_seqs * k.a.num_kv_heads), dim3(256), 0, s, k);
  trace_end(s, mark, "merge_shared");
  return launch_status("pa_forward_shared (merge)");
}

template <int G>
pa_status launch_shared_g(const SharedArgs& k, int cg, int depth, hipStream_t s) {
  if (cg == 4) return depth >= 3 ? launch_shared_gn<G, 4, 3>(k, s) : launch_shared_gn<G, 4, 2>(k, s);
  return depth >= 3 ? launch_shared_gn<G, 2, 3>(k, s) : launch_shared_gn<G, 2, 2>(k, s);
}

size_t round256s(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

SharedPlan make_shared_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t dtype, int32_t max_seq_len, int32_t max_query_len) {
  SharedPlan sp{};
  const int32_t G = num_kv_heads > 0 ? num_q_heads / num_kv_heads : 0;
  if (!decode_mfma_supported(dtype, head_dim, G) || num_seqs < 1 || num_seqs > kMaxSharedSeqs ||
      max_query_len != 1 || max_seq_len <= 0)
    return sp;
  sp.on = true;
  // As the other balanced decodes: 1024 single-wave work-groups in all (one
  // per SIMD), never more than the tiles there can be.  PA_SHARED_TOTAL_WAVES overrides.
  int64_t target = 1024;
  if (const char* tw = std::getenv("PA_SHARED_TOTAL_WAVES")) {
    const int v = std::atoi(tw);
    if (v >= 1 && v <= 65536) target = v;
  }
  const int64_t whole_tiles = ((int64_t)max_seq_len + kBlock - 1) / kBlock;
  const int64_t wg = std::max<int64_t>(1, std::min<int64_t>(target / num_kv_heads, (int64_t)num_seqs * whole_tiles));
  sp.waves_per_head = (int32_t)wg;
  // Column groups of 16 (sequences per group: 16 CG / G); PA_SHARED_CG=2|4 overrides.
  sp.col_groups = 2;
  if (const char* e = std::getenv("PA_SHARED_CG")) sp.col_groups = std::atoi(e) == 4 ? 4 : 2;
  // Three tiles in flight while four work-groups still fit a CU's LDS, else two.
  sp.depth = shared_static_lds(sp.col_groups, 3) + shared_dyn_lds(num_seqs) <= 40 * 1024 ? 3 : 2;
  const size_t slots = 2 * (size_t)num_seqs + (size_t)wg;
  sp.prefix_bytes = round256s((size_t)num_seqs * sizeof(int32_t));
  sp.info_bytes = round256s((size_t)num_seqs * 2 * sizeof(int2));
  sp.acc_bytes = round256s((size_t)num_kv_heads * slots * 16 * sp.col_groups * head_dim * sizeof(uint16_t));
  sp.ml_bytes = round256s((size_t)num_kv_heads * slots * 16 * sp.col_groups * 4 * sizeof(float));
  return sp;
}

pa_status launch_decode_shared(const AttnArgs& a, const SharedPlan& sp, const int32_t* shared_blocks,
                               void* workspace, hipStream_t s) {
  uint8_t* base = (uint8_t*)workspace;
  SharedArgs k{a,
               shared_blocks,
               sp.waves_per_head,
               2 * a.num_seqs + sp.waves_per_head,
               (uint16_t*)(base + sp.prefix_bytes + sp.info_bytes),
               (float*)(base + sp.prefix_bytes + sp.info_bytes + sp.acc_bytes),
               (int2*)(base + sp.prefix_bytes),
               (int32_t*)base};
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_shared_g<1>(k, sp.col_groups, sp.depth, s);
    case 2: return launch_shared_g<2>(k, sp.col_groups, sp.depth, s);
    case 4: return launch_shared_g<4>(k, sp.col_groups, sp.depth, s);
    case 8: return launch_shared_g<8>(k, sp.col_groups, sp.depth, s);
    default:
      return fail(PA_ERR_UNSUPPORTED, "pa_forward_shared: %d query heads per KV head", a.num_q_heads / a.num_kv_heads);
  }
}

}  // namespace pa
