// Multi-token decode on the matrix cores: sequences that add a few query
// tokens in one step, as a speculative-decoding step does when it scores the
// tokens a smaller draft model proposed ("vLLM PagedAttention: eine
// Revolution ..." (de.news.hada.io), bullet "Guided and Speculative
// Decoding"; "Внутреннее устройство vLLM" (artificials.ru), closing paragraph:
// several tokens predicted at once).  Query token jq of a sequence holding L
// tokens after this step's write sits at position L - n + jq and, causally,
// sees keys 0 .. L - n + jq (same page, forward-pass paragraph: attention
// masks and exact positional indices keep each row on its own sequence).
//
// Such a step reads a sequence's whole cache for a handful of query rows, so
// it is bound by memory bandwidth like single-token decode, and it reuses the
// balanced one-round scheme of the single-token kernel: per KV head, the
// 16-token tiles of all these sequences form one stream cut into equal ranges,
// one single-wave work-group per range; tiles are staged through LDS by the
// buffer unit NS deep; the parts of a sequence split between waves are merged
// afterwards in rank order by merge_verify_kernel.
//
// What differs is the work per tile.  The MFMA columns are (token, query head)
// pairs -- column c -> token c / G, query head g G + c % G -- in CG groups of
// 16, so up to 16 CG / G tokens of a sequence share every K/V tile read:
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16 per 32 dims: A = K rows from
//                   LDS (lane l: key l % 16, dims 8 (l / 16) of the step), B =
//                   the column group's query rows; lane (r, j) receives the
//                   scores of keys 4r .. 4r+3 for column j.
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16 per 16 dims: B = P^T is exactly
//                   the lane's own four weights (rounded to bf16); A = V^T is
//                   read from a row-major [16 keys][16 dims] sub-tile with
//                   ds_read_b64_tr_b16, which hands lane (r, m) keys 4r .. 4r+3
//                   of dim m when the 16 lanes of row group r point at those
//                   four key rows (four lanes per row, four dims each).
// A column's softmax state is kept by its four lanes together: one running
// max (equal in all four; moved, after a reduction across them, only when a
// score beats it by the rescale slack) and a partial sum each, so a rescale
// touches only the lane's own accumulators and the common tile needs no
// cross-lane traffic.
// The sum adds the same bf16-rounded weights the P.V product uses.
//
// Keys past a column's visible end get weight 0 (select, on the tiles that
// need it); the copies of a sequence's last tile go through a buffer range
// that ends at its last token, so stale slots arrive as zeros and nothing
// past the sequence reaches an MFMA.
#include <algorithm>
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
// fp8 pools: a plane of code tiles, per (block, KV head) 16 x 128 E4M3 codes
// (K row-major, V transposed: byte d * 16 + row), 128-byte aligned; then a
// plane of row exponents, 16 bytes per tile (E8M0, 2^(c - 127)).
constexpr int kTileBytesF8 = kBlock * kD;
constexpr int kMaxVerifySeqs = 1024;              // per-sequence tables kept in LDS
constexpr int kMaxColGroups = 4;
constexpr int kMaxVerifyTokens = 16;


struct VerifyArgs {
  AttnArgs a;
  int32_t min_q;            // sequences with min_q .. max_q query tokens
  int32_t max_q;
  int32_t waves_per_head;   // Wg
  int32_t slots;            // partial slots per KV head: num_seqs + Wg
  uint16_t* p_acc;          // [Hkv][slots][CG][8 db][64 lanes][4] fp16: fragment order (see finish)
  float* p_ml;              // [Hkv][slots][16 CG][4]  (max in base-2 units, sum, e, 0)
  int2* seqinfo;            // [num_seqs]: (first rank, parts)
  int32_t first_ranks;      // ranks dispatched first on their SIMD (the lowest work-group ids) ...
  int32_t first_weight;     // ... take this many tiles per 1000 of the others' (see make_verify_plan)
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Weighted split of a head's tile stream: ranks below h weigh wa, the others
// wb, and rank r takes tiles [start(r), start(r + 1)), its share of `total` in
// proportion to the weights before it.  wa = wb gives stream_start's ranges.
// Every range is non-empty when total * min(wa, wb) >= the weight sum.
struct StreamSplit {
  int64_t total;
  int Wg, h, wa, wb;
  __device__ int64_t cum(int r) const {
    return r <= h ? (int64_t)r * wa : (int64_t)h * wa + (int64_t)(r - h) * wb;
  }
  __device__ int64_t start(int r) const { return total * cum(r) / cum(Wg); }
  // The largest r with start(r) <= t, for 0 <= t < total.
  __device__ int owner(int64_t t) const {
    const int64_t x = ((t + 1) * cum(Wg) - 1) / total;   // largest weight prefix with start <= t
    const int64_t hx = (int64_t)h * wa;
    return x < hx ? (int)(x / wa) : h + (int)((x - hx) / wb);
  }
};

// Dynamic LDS: tile prefix sums [S + 1], query row << 5 | (tokens - 1) [S], length [S].
inline size_t verify_dyn_lds(int num_seqs) { return (size_t)(3 * num_seqs + 1) * sizeof(int); }
// Static LDS of one instantiation: lookup windows, query rows, NS stages.
inline size_t verify_static_lds(int cg, int ns) { return 3 * 512 + (size_t)cg * 4096 + (size_t)ns * 8192; }

// True for the sequences this kernel and its merge handle (the same test in
// both), from query_start_loc[i], [i + 1] and seq_lens[i].
__device__ __forceinline__ bool verify_item_of(const VerifyArgs& k, int qa, int qb, int sl, int& q0, int& n,
                                               int& len) {
  q0 = qa;
  n = qb - qa;
  len = min(sl, k.a.bt_stride * kBlock);
  return n >= k.min_q && n <= k.max_q && q0 >= 0 && q0 + n <= k.a.num_tokens && len >= n;
}
__device__ __forceinline__ bool verify_item(const VerifyArgs& k, int i, int& q0, int& n, int& len) {
  return verify_item_of(k, k.a.qsl[i], k.a.qsl[i + 1], k.a.seq_lens[i], q0, n, len);
}

// Wait until at most OPS * t vector memory operations (t tiles' copies) are outstanding.
template <int OPS>
__device__ __forceinline__ void wait_ops(int t) {
  if (t <= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OPS) : "memory");
  else if (t == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * OPS) : "memory");
  else if (t == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * OPS) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * OPS) : "memory");
}

// E8M0 exponent code -> 2^(c - 127) (codes 1..254; 255 gives inf, masked by the callers).
__device__ __forceinline__ float e8m0(uint32_t c) { return __uint_as_float(c << 23); }

// Eight E4M3 codes (memory order, two dwords) -> eight bf16, each times `scale`
// (a power of two, so exact).
__device__ __forceinline__ uint4 cvt8_fp8(uint32_t w0, uint32_t w1, float scale) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true)));
}

template <int CG>
struct VerifyState {
  float m[CG];          // running max (base 2) of the lane's column, the same in its four lanes
  float l[CG];          // this lane's share of the column's weight sum
  f32x4_t acc[CG][8];   // O^T: column j, dims 16 db + 4 r .. +3
};

template <int G, int CG, int NS, bool F8>
__global__ __launch_bounds__(64) void decode_verify_kernel(VerifyArgs k) {
  static_assert(16 % G == 0, "query heads per KV head must divide 16");
  static_assert(NS >= 2 && NS <= 5, "tiles in flight");
  constexpr int C = 16 * CG;
  constexpr int TILE = F8 ? kTileBytesF8 : kTileBytes;   // bytes of one (block, KV head) code tile
  constexpr int OPS = F8 ? 5 : 8;                        // copies per tile
  constexpr int STAGE_U4 = F8 ? 260 : 512;               // one LDS stage, in 16-byte units
  extern __shared__ int s_dyn[];
  const AttnArgs& a = k.a;
  const int S = a.num_seqs;
  int* s_cum = s_dyn;
  int* s_meta = s_dyn + S + 1;
  int* s_len = s_meta + S;
  __shared__ int s_raw[2][64];                   // lookup windows: block-table entry (copied), sequence, logical block
  __shared__ int s_sj[2][2][64];
  __shared__ __attribute__((aligned(16))) uint4 s_q[CG * 4 * 64];   // query rows: [cg][ks][lane]
  // Tile stages.  bf16: K [ks][lane], V [db][16 keys][16 dims].  fp8: K codes
  // [piece][lane], V codes [dim][16 keys], then 16 K and 16 V row exponents.
  __shared__ __attribute__((aligned(16))) uint4 s_st[NS][STAGE_U4];
  const int Hkv = a.num_kv_heads;
  // Work-group -> (KV head, rank).  Work-groups go to the eight XCDs round
  // robin (blockIdx % 8).  fp8: the row exponents of all KV heads of a block
  // share one 128-byte line (16 bytes per head), so the KV heads of one rank
  // -- the same blocks -- are put on one XCD, where the line is fetched once
  // into that XCD's L2 instead of once per XCD.  Otherwise KV head fastest.
  int g, rank;
  if (F8 && k.waves_per_head % 8 == 0) {
    const int y = blockIdx.x >> 3;
    g = y % Hkv;
    rank = (y / Hkv) * 8 + (blockIdx.x & 7);
  } else {
    g = blockIdx.x % Hkv;
    rank = blockIdx.x / Hkv;
  }
  const int lane = threadIdx.x;

  // Tiles of every sequence this kernel handles (0 for the others), then
  // exclusive prefix sums in place.
  for (int c0 = 0; c0 < S; c0 += 256) {
    int T[4], M[4], Ln[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = c0 + 64 * u + lane;
      T[u] = 0;
      M[u] = 0;
      Ln[u] = 0;
      int q0, n, len;
      if (i < S && verify_item(k, i, q0, n, len)) {
        T[u] = (len + kBlock - 1) / kBlock;
        M[u] = (q0 << 5) | (n - 1);
        Ln[u] = len;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = c0 + 64 * u + lane;
      if (i < S) {
        s_cum[i] = T[u];
        s_meta[i] = M[u];
        s_len[i] = Ln[u];
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
  const int Wg = (int)min((int64_t)k.waves_per_head, total);
  if (rank >= Wg) return;
  // Ranks split the head's tile stream by weight: those of the first-dispatched
  // waves on each SIMD take first_weight / 1000 times the others' share,
  // whenever that leaves every range non-empty (else equal ranges).
  StreamSplit sp{total, Wg, min(k.first_ranks, Wg), k.first_weight, 1000};
  if (sp.h >= Wg || total * 1000 < 2 * (int64_t)Wg * max(sp.wa, 1000)) sp.wa = sp.wb = 1;
  const int tb = (int)sp.start(rank);
  const int cnt = (int)(sp.start(rank + 1) - tb);

  const u32x4_t rbt = rsrc_words((const uint8_t*)a.block_tables,
                                 (int)min((int64_t)S * a.bt_stride * 4, (int64_t)0x7fffffff));
  auto lookup = [&](int window) {
    const int u = window * 64 + lane;
    int seq = 0, jt = 0;
    if (u < cnt) {
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
  // Query rows of sequence `seq` -> s_q: copy (cg, ks) has lane (r, j) fetch
  // the eight dims of column 16 cg + j that k-step ks pairs with this lane's
  // K operand: 32 ks + 8 r .. +8 (bf16 cache), 64 (ks / 2) + 16 r + 8 (ks % 2)
  // .. +8 (fp8 cache, whose K codes arrive 16 per lane).  The buffer range ends
  // at the sequence's last query row, so columns past its tokens read zeros.
  auto copy_q = [&](int seq) {
    const int meta = __builtin_amdgcn_readfirstlane(s_meta[seq]);
    const int q0 = meta >> 5, nq = (meta & 31) + 1;
    const u32x4_t rq = rsrc_words((const uint8_t*)a.q + (size_t)q0 * a.num_q_heads * kRowBytes,
                                  nq * a.num_q_heads * kRowBytes);
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      const int col = 16 * cg + j;
      const int off = ((col / G) * a.num_q_heads + hq0 + col % G) * kRowBytes + r * 16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        lds_copy16(rq, s_q + (cg * 4 + ks) * 64, F8 ? off + r * 16 + (ks / 2) * 128 + (ks % 2) * 16 : off + ks * 64);
    }
  };
  copy_q(__builtin_amdgcn_readfirstlane(s_sj[0][0][0]));
  int q_tile = -(NS - 1);   // tile whose issue followed the last query copy

  const uint8_t* kc = (const uint8_t*)a.k_cache + (size_t)g * TILE;
  const uint8_t* vc = (const uint8_t*)a.v_cache + (size_t)g * TILE;
  const size_t block_stride = (size_t)Hkv * TILE;
  // fp8: the exponent plane follows all code tiles.
  const uint8_t* kx = (const uint8_t*)a.k_cache + (size_t)a.num_blocks * block_stride + (size_t)g * kBlock;
  const uint8_t* vx = (const uint8_t*)a.v_cache + (size_t)a.num_blocks * block_stride + (size_t)g * kBlock;
  // K piece ks: lane (r, j) copies key j, dims 32 ks + 8 r .. +8.
  const int koff = j * kRowBytes + r * 16;
  // V piece e (dim blocks 2e, 2e+1): lane 32 dsel + 2 key + half copies key
  // `key`, dims 16 (2e + dsel) + 8 half .. +8, landing in row `key` of the
  // [16 keys][16 dims] sub-tile of dim block 2e + dsel.
  const int voff = ((lane & 31) >> 1) * kRowBytes + (lane >> 5) * 32 + (lane & 1) * 16;
  auto stage = [&](int sI) -> uint4* { return s_st[sI]; };
  // A prefetch past the range (uu >= cnt) still issues its copies, so that
  // every wait counts the same operations, but through empty ranges: they
  // read nothing and write zeros into a stage no later fold reads.
  auto issue = [&](int uu, int sI) {
    const int u = min(uu, cnt - 1);
    const bool real = uu < cnt;
    const int w = (u >> 6) & 1, e = u & 63;
    const int bid = clamp_block(__builtin_amdgcn_readfirstlane(s_raw[w][e]), a.num_blocks);
    const size_t off = (size_t)bid * block_stride;
    uint4* dst = stage(sI);
    if constexpr (F8) {
      // K codes: piece p, lane (r, j) = key j's dims 64 p + 16 r .. +16.  V codes
      // (stored transposed): piece p, lane l = dim 64 p + l, all 16 keys.  Then
      // lanes 0..3 copy the 16 K and the 16 V row exponents.  Keys past the
      // sequence are masked where they are used.
      const u32x4_t rk = rsrc_words(kc + off, real ? TILE : 0);
      const u32x4_t rv = rsrc_words(vc + off, real ? TILE : 0);
#pragma unroll
      for (int p = 0; p < 2; ++p) lds_copy16_nt(rk, dst + p * 64, j * kD + r * 16 + p * 64);
#pragma unroll
      for (int p = 0; p < 2; ++p) lds_copy16_nt(rv, dst + 128 + p * 64, (p * 64 + lane) * kBlock);
      // One copy for both: lanes 0..3 the K row exponents, lanes 4..7 the V
      // ones, by address (a prefetch past the range reads the clamped
      // tile's, into a stage no fold reads).
      if (lane < 8) {
        const size_t xoff = (size_t)bid * Hkv * kBlock + 4 * (lane & 3);
        lds_copy4_global((lane < 4 ? kx : vx) + xoff, dst + 256);
      }
    } else {
      const int seq = __builtin_amdgcn_readfirstlane(s_sj[w][0][e]);
      const int jt = __builtin_amdgcn_readfirstlane(s_sj[w][1][e]);
      // Rows past the sequence read as zero.
      const int bytes = real ? __builtin_amdgcn_readfirstlane(min(s_len[seq] - jt * kBlock, kBlock) * kRowBytes) : 0;
      const u32x4_t rk = rsrc_words(kc + off, bytes);
      const u32x4_t rv = rsrc_words(vc + off, bytes);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) lds_copy16_nt(rk, dst + ks * 64, koff + ks * 64);
#pragma unroll
      for (int p = 0; p < 4; ++p) lds_copy16_nt(rv, dst + 256 + p * 64, voff + p * 64);
    }
  };
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0) issue(s0, s0);

  // Transpose-read address of this lane inside a [16 keys][16 dims] sub-tile:
  // row group r points at key rows 4r .. 4r+3, four lanes per row, four dims each.
  const int tr_off = (4 * r + j / 4) * 32 + (j & 3) * 8;

  VerifyState<CG> st;
  bf16x8_t qf[CG][4];
  int cur = -1, cur_j0 = 0, cur_jl = 0, cur_q0 = 0, cur_n = 0, cga = 0, first_end = 0, cur_len = 0;
  int col_end[CG];

  auto finish = [&](int seq, bool whole) {
    const size_t slot = (size_t)g * k.slots + (size_t)(seq + rank);
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      if (cg > 0 && cg >= cga) break;   // group 0 is always active
      float lt = st.l[cg];
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
      const int col = 16 * cg + j;
      const int jq = col / G;
      if (jq >= cur_n) continue;
      if (whole) {
        const float inv = 1.0f / lt;
        uint8_t* op = (uint8_t*)a.out + ((size_t)(cur_q0 + jq) * a.num_q_heads + hq0 + col % G) * kRowBytes + r * 8;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const f32x4_t x = st.acc[cg][db];
          *reinterpret_cast<uint2*>(op + db * 32) =
              make_uint2(pack_bf16x2(x[0] * inv, x[1] * inv), pack_bf16x2(x[2] * inv, x[3] * inv));
        }
      } else {
        // Partials: the column's output normalised by its weight sum, times
        // 2^-e in fp16, e set by the column's largest magnitude (over its four
        // lanes) so that it lands in [2^14, 2^15): full fp16 precision through
        // exact power-of-two scalings, half the bytes of fp32.  Fragment order:
        // dim block db of column group cg is one contiguous 512-byte piece,
        // lane l's four values at 8 l.  Beside them (max, sum, e); a column
        // that sees no key of this part has sum 0 and weight 0 in the merge.
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
          for (int h = 0; h < 2; ++h) {
            const _Float16 lo = static_cast<_Float16>(ldexpf(st.acc[cg][db][2 * h] * inv, -ex));
            const _Float16 hi = static_cast<_Float16>(ldexpf(st.acc[cg][db][2 * h + 1] * inv, -ex));
            w[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
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
      const int jt = __builtin_amdgcn_readfirstlane(s_sj[window & 1][1][u & 63]);
      if (seq != cur) {
        if (cur >= 0) finish(cur, cur_j0 == 0 && cur_jl + 1 == s_cum[cur + 1] - s_cum[cur]);
        cur = seq;
        // Per-segment values are wave-uniform: kept in scalar registers so the
        // per-tile branches on them are scalar branches.
        const int meta = __builtin_amdgcn_readfirstlane(s_meta[seq]);
        const int L = __builtin_amdgcn_readfirstlane(s_len[seq]);
        cur_q0 = meta >> 5;
        cur_n = (meta & 31) + 1;
        cur_len = L;
        cga = min(CG, (cur_n * G + 15) / 16);
        first_end = a.causal ? L - cur_n + 1 : L;
#pragma unroll
        for (int cg = 0; cg < CG; ++cg)
          col_end[cg] = a.causal ? min(L, L - cur_n + (16 * cg + j) / G + 1) : L;
        cur_j0 = jt;
        if (jt == 0 && g == 0 && lane == 0) {
          const int last = sp.owner((int64_t)s_cum[seq + 1] - 1);
          k.seqinfo[seq] = make_int2(rank, last - rank + 1);
        }
        // This sequence's query copy was followed by the issues of tiles
        // q_tile .. u - 1 (eight copies each; at least one tile).
        __builtin_amdgcn_sched_barrier(0);
        wait_ops<OPS>(min(u - q_tile, NS - 1));
        const lds_u32x4_t* qs = (const lds_u32x4_t*)s_q;
#pragma unroll
        for (int cg = 0; cg < CG; ++cg)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) qf[cg][ks] = __builtin_bit_cast(bf16x8_t, qs[(cg * 4 + ks) * 64 + lane]);
        // The copy of the next sequence's rows overwrites s_q: the reads above come first.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        int nx = seq + 1;                      // next sequence with tiles, if this range reaches it
        while (nx < S && s_cum[nx + 1] == s_cum[nx]) ++nx;
        if (nx < S && s_cum[nx] < tb + cnt) {
          copy_q(nx);
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
      wait_ops<OPS>(NS - 1);
      cur_jl = jt;
      const lds_u32x4_t* src = (const lds_u32x4_t*)stage(sI);
      const uint8_t* sb = (const uint8_t*)stage(sI);
      const int tok0 = jt * kBlock;
      uint4 kq[4];
      uint32_t vexp = 0;
      if constexpr (F8) {
        // k-step ks = 2 p + h takes half h of piece p, converted exactly to bf16
        // with key j's exponent.
        const uint4 k0 = __builtin_bit_cast(uint4, src[lane]), k1 = __builtin_bit_cast(uint4, src[64 + lane]);
        const float ks_scale = e8m0(sb[4096 + j]);
        vexp = *reinterpret_cast<const uint32_t*>(sb + 4112 + 4 * r);   // V exponents of keys 4r .. 4r+3
        kq[0] = cvt8_fp8(k0.x, k0.y, ks_scale);
        kq[1] = cvt8_fp8(k0.z, k0.w, ks_scale);
        kq[2] = cvt8_fp8(k1.x, k1.y, ks_scale);
        kq[3] = cvt8_fp8(k1.z, k1.w, ks_scale);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kq[ks] = __builtin_bit_cast(uint4, src[ks * 64 + lane]);
      }

      // Scores of the active column groups, base-2 units, masked past each column's end.
      float sc[CG][4];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (cg > 0 && cg >= cga) break;   // group 0 is always active
        // Two independent accumulation chains (k-steps 0, 2 and 1, 3), added at the end.
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ks += 2) {
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[ks]), qf[cg][ks], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[ks + 1]), qf[cg][ks + 1], s1,
                                                        0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[cg][e] = (s0[e] + s1[e]) * a.scale_log2;
        if (tok0 + kBlock > first_end) {   // wave-uniform: only a sequence's last tiles reach a column's end
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[cg][e] = tok0 + 4 * r + e < col_end[cg] ? sc[cg][e] : -INFINITY;
        }
      }
      // Lazy rescale: only when some lane's scores beat its column's reference
      // by the slack (rare after a segment's first tile) are the four lanes of
      // each column reduced to the column's tile max and the reference moved.
      bool need = false;
      float mx[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (cg > 0 && cg >= cga) break;   // group 0 is always active
        mx[cg] = fmaxf(fmaxf(sc[cg][0], sc[cg][1]), fmaxf(sc[cg][2], sc[cg][3]));
        need |= mx[cg] > st.m[cg] + kRescaleSlack;
      }
      if (__any(need)) {
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) {
          if (cg > 0 && cg >= cga) break;   // group 0 is always active
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
      // fp8: the product takes each weight times its key's V exponent (exact),
      // the sum the weight alone; keys past the sequence get weight 0 and
      // their (stale) codes are zeroed.
      f32x4_t vsc = {1.0f, 1.0f, 1.0f, 1.0f};
      uint32_t vkeep = 0xffffffffu;
      if constexpr (F8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) vsc[e] = e8m0((vexp >> (8 * e)) & 0xffu);
        if (tok0 + kBlock > cur_len) {   // wave-uniform: the sequence's last tile
          const int live = min(max(cur_len - tok0 - 4 * r, 0), 4);   // valid keys among 4r .. 4r+3
#pragma unroll
          for (int e = 0; e < 4; ++e) vsc[e] = e < live ? vsc[e] : 0.0f;
          vkeep = live >= 4 ? 0xffffffffu : live == 0 ? 0u : (1u << (8 * live)) - 1u;
        }
      }
      s16x4_t pb[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (cg > 0 && cg >= cga) break;   // group 0 is always active
        f32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = fast_exp2(sc[cg][e] - st.m[cg]);
        const bf16x4_t wb = __builtin_convertvector(w, bf16x4_t);   // nearest even
        f32x4_t wr = __builtin_convertvector(wb, f32x4_t);          // exact
        st.l[cg] += (wr[0] + wr[1]) + (wr[2] + wr[3]);
        if constexpr (F8) pb[cg] = __builtin_bit_cast(s16x4_t, __builtin_convertvector(wr * vsc, bf16x4_t));
        else pb[cg] = __builtin_bit_cast(s16x4_t, wb);
      }
      // All eight V^T operands are read before the first product, so their LDS
      // latencies overlap.
      const uint8_t* vst = F8 ? sb + 2048 + 16 * j + 4 * r : sb + 4096 + tr_off;
      s16x4_t vt[8];
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        if constexpr (F8) {
          // Lane (r, m): dim 16 db + m, keys 4r .. 4r+3 -- four codes of one transposed row.
          const uint32_t w = *reinterpret_cast<const uint32_t*>(vst + 256 * db) & vkeep;
          const uint2 h = make_uint2(
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
          vt[db] = __builtin_bit_cast(s16x4_t, h);
        } else {
          vt[db] = lds_read_tr(vst + db * 512);
        }
      }
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (cg > 0 && cg >= cga) break;   // group 0 is always active
#pragma unroll
        for (int db = 0; db < 8; ++db)
          st.acc[cg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[db], pb[cg], st.acc[cg][db], 0, 0, 0);
      }
    }
  }
  finish(cur, cur_j0 == 0 && cur_jl + 1 == s_cum[cur + 1] - s_cum[cur]);
}

// Merge of the parts of split sequences: one work-group per (sequence, KV
// head, column group), one thread per float4 of the fragment-ordered partials
// (dim block db, lane (r, j): column 16 cg + j, dims 16 db + 4 r .. +3), so
// consecutive threads read consecutive 16 bytes; the parts are folded in
// rank order by the log-sum-exp rule in one pass, eight parts' loads in
// flight -- a sequence split into up to eight parts costs one memory round
// trip.
template <int CG>
__global__ __launch_bounds__(512) void merge_verify_kernel(VerifyArgs k) {
  constexpr int C = 16 * CG, U = 8;
  const AttnArgs& a = k.a;
  const int Hkv = a.num_kv_heads, G = a.num_q_heads / Hkv;
  const int i = blockIdx.x / Hkv, g = blockIdx.x % Hkv, cg = blockIdx.y;
  // The part table is read with the sequence's metadata, in one memory round
  // trip (this call's verify kernel wrote it for every sequence it took); the
  // empty asm keeps the compiler from sinking that load below the checks.
  const int2 si = k.seqinfo[i];
  const int qa = a.qsl[i], qb = a.qsl[i + 1], sl = a.seq_lens[i];
  asm volatile("" ::"s"(si.x), "s"(si.y), "s"(qa), "s"(qb), "s"(sl));
  int q0, n, len;
  if (!verify_item_of(k, qa, qb, sl, q0, n, len)) return;
  if (cg * 16 >= n * G) return;          // column group beyond this sequence's rows
  const int P = si.y;
  if (P <= 1) return;                    // written out by the verify kernel
  const size_t slot0 = (size_t)g * k.slots + (size_t)(i + si.x);
  {
    const int it = cg * 512 + threadIdx.x;
    const int ln = it & 63, db = (it >> 6) & 7;
    const int col = 16 * cg + (ln & 15);
    if (col >= n * G) return;
    const float4* ml = reinterpret_cast<const float4*>(k.p_ml) + slot0 * C + col;
    const uint16_t* acc = k.p_acc + (slot0 * CG * 8 * 64 + it) * 4;
    float M = -INFINITY, den = 0.0f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < P; p0 += U) {
      float4 v[U];
      uint2 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p0 + u < P) {
          v[u] = ml[(size_t)(p0 + u) * C];
          x[u] = *reinterpret_cast<const uint2*>(acc + (size_t)(p0 + u) * C * kD);   // one slot = C x D values
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p0 + u >= P) break;
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
    const float inv = 1.0f / den;
    uint8_t* op = (uint8_t*)a.out + ((size_t)(q0 + col / G) * a.num_q_heads + g * G + col % G) * kRowBytes +
                  (16 * db + 4 * (ln >> 4)) * 2;
    *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(num.x * inv, num.y * inv),
                                               pack_bf16x2(num.z * inv, num.w * inv));
  }
}

template <int G, int CG, int NS, bool F8>
pa_status launch_verify_gc(const VerifyArgs& k, hipStream_t s) {
  const int W = k.waves_per_head * k.a.num_kv_heads;
  int mark = trace_begin(s);
  hipLaunchKernelGGL((decode_verify_kernel<G, CG, NS, F8>), dim3(W), dim3(64), verify_dyn_lds(k.a.num_seqs), s, k);
  trace_end(s, mark, "decode_verify");
  pa_status st = launch_status("pa_forward (multi-token decode)");
  if (st != PA_OK) return st;
  mark = trace_begin(s);
  hipLaunchKernelGGL((merge_verify_kernel<CG>), dim3(k.a.num_seqs * k.a.num_kv_heads, CG), dim3(512), 0, s, k);
  trace_end(s, mark, "merge_verify");
  return launch_status("pa_forward (multi-token decode merge)");
}

template <int G, int CG>
pa_status launch_verify_g(const VerifyArgs& k, int depth, bool f8, hipStream_t s) {
  if (f8) return depth >= 5 ? launch_verify_gc<G, CG, 5, true>(k, s) : launch_verify_gc<G, CG, 3, true>(k, s);
  if (depth >= 4) return launch_verify_gc<G, CG, 4, false>(k, s);
  if (depth == 3) return launch_verify_gc<G, CG, 3, false>(k, s);
  return launch_verify_gc<G, CG, 2, false>(k, s);
}

}  // namespace

bool verify_fp8_supported(int32_t head_dim, int32_t group) {
  return head_dim == kD && (group == 1 || group == 2 || group == 4 || group == 8);
}

VerifyPlan make_verify_plan(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t dtype, int32_t max_seq_len, int32_t max_query_len) {
  VerifyPlan vp{};
  const int32_t G = num_kv_heads > 0 ? num_q_heads / num_kv_heads : 0;
  // Whenever a batch may hold sequences of more than one query token, this
  // launch takes the single-token sequences too, so a step launches one
  // decode-like kernel and one merge instead of two of each (either of which
  // may find nothing to do: the host cannot see the per-sequence counts).  A
  // batch of single-token sequences only keeps the single-token decode.  A
  // quantised (fp8) cache always comes here.  PA_VERIFY=prefill sends the
  // multi-token sequences to the chunked-prefill kernel; PA_VERIFY=all routes
  // single-token sequences here even then; PA_VERIFY=split keeps them apart.
  const bool fp8 = dtype == PA_FP8;
  const char* env = std::getenv("PA_VERIFY");
  if (!fp8 && env != nullptr && std::strcmp(env, "prefill") == 0) return vp;
  const bool all = env != nullptr && std::strcmp(env, "all") == 0;
  const bool split = env != nullptr && std::strcmp(env, "split") == 0;
  const int32_t min_q = fp8 || all || (max_query_len >= 2 && !split) ? 1 : 2;
  const bool shape_ok = fp8 ? verify_fp8_supported(head_dim, G) : decode_mfma_supported(dtype, head_dim, G);
  if (!shape_ok || num_seqs < 1 || num_seqs > kMaxVerifySeqs || max_query_len < min_q || max_seq_len <= 0 ||
      num_tokens >= (1 << 26))
    return vp;
  // Columns (token, query head) in groups of 16: enough groups for the
  // longest multi-token sequence up to 16 tokens and 4 groups.
  const int cap = std::min(kMaxVerifyTokens, 16 * kMaxColGroups / G);
  const int want = std::min<int>(max_query_len, cap);
  int cg = (want * G + 15) / 16;
  if (cg == 3) cg = 4;
  vp.on = true;
  vp.fp8 = fp8;
  vp.min_q = min_q;
  vp.col_groups = cg;
  vp.max_q = std::min(cap, 16 * cg / G);
  // As the single-token decode: 1024 single-wave work-groups in all (one per
  // SIMD).  fp8 with one column group: 2048 (two per SIMD fit its registers
  // and LDS, and measured on MI355X they hide more of its per-tile latency).
  int64_t target = fp8 && cg == 1 ? 2048 : 1024;
  if (const char* tw = std::getenv("PA_VERIFY_TOTAL_WAVES")) {
    const int v = std::atoi(tw);
    if (v >= 1 && v <= 65536) target = v;
  }
  const int64_t whole_tiles = ((int64_t)max_seq_len + kBlock - 1) / kBlock;
  const int64_t wg = std::max<int64_t>(1, std::min<int64_t>(target / num_kv_heads, (int64_t)num_seqs * whole_tiles));
  vp.waves_per_head = (int32_t)wg;
  // With more waves than SIMDs (up to two per SIMD: 256 CUs x 4), the
  // work-groups dispatched first -- the lowest ids, one per SIMD -- keep the
  // older wave's issue priority over the second wave on their SIMD for the
  // whole launch.  Measured on MI355X (fp8 batched decode, 2048 waves, equal
  // ranges): the first 1024 stream their tiles 1.18x as fast as the others
  // and finish 7.5 us earlier.  Their ranks (ids below 1024 are the ranks
  // below 1024 / Hkv in either work-group mapping, for Hkv dividing 128) take
  // 1.35x the tiles: swept from 1.0 to 2.0, the kernel was fastest at
  // 1.35-1.5 (54.8 -> 52.5 us).  PA_VERIFY_FIRST_WEIGHT=<500..2000> (per
  // 1000) overrides the ratio.
  constexpr int64_t kSimds = 1024;
  const int64_t waves = wg * num_kv_heads;
  vp.first_ranks = (int32_t)wg;
  vp.first_weight = 1000;
  if (waves > kSimds && waves <= 2 * kSimds) {
    vp.first_ranks = (int32_t)(kSimds / num_kv_heads);
    vp.first_weight = 1350;
  }
  if (const char* fw = std::getenv("PA_VERIFY_FIRST_WEIGHT")) {
    const int v = std::atoi(fw);
    if (v >= 500 && v <= 2000) vp.first_weight = v;
  }
  // bf16: three tiles in flight while four work-groups still fit in a CU's
  // LDS, else two.  fp8: three (measured on MI355X: deeper rings of the
  // half-size fp8 tiles were slower).  PA_VERIFY_DEPTH=2..5 overrides (fp8: 3 or 5).
  vp.depth = fp8 ? 3 : verify_static_lds(cg, 3) + verify_dyn_lds(num_seqs) <= 40 * 1024 ? 3 : 2;
  if (const char* dp = std::getenv("PA_VERIFY_DEPTH")) {
    const int v = std::atoi(dp);
    if (v >= 2 && v <= 5) vp.depth = v;
  }
  const size_t slots = (size_t)num_seqs + (size_t)wg;
  vp.info_bytes = round256((size_t)num_seqs * 2 * sizeof(int32_t));
  vp.acc_bytes = round256((size_t)num_kv_heads * slots * 16 * cg * head_dim * sizeof(uint16_t));
  vp.ml_bytes = round256((size_t)num_kv_heads * slots * 16 * cg * 4 * sizeof(float));
  return vp;
}

pa_status launch_decode_verify(const AttnArgs& a, const VerifyPlan& vp, uint16_t* p_acc, float* p_ml,
                               int32_t* part_table, hipStream_t s) {
  VerifyArgs k{a, vp.min_q, vp.max_q, vp.waves_per_head, a.num_seqs + vp.waves_per_head, p_acc, p_ml,
               (int2*)part_table, vp.first_ranks, vp.first_weight};
  const int G = a.num_q_heads / a.num_kv_heads;
  const bool f8 = vp.fp8;
  switch (G * 16 + vp.col_groups) {
    case 1 * 16 + 1: return launch_verify_g<1, 1>(k, vp.depth, f8, s);
    case 2 * 16 + 1: return launch_verify_g<2, 1>(k, vp.depth, f8, s);
    case 2 * 16 + 2: return launch_verify_g<2, 2>(k, vp.depth, f8, s);
    case 4 * 16 + 1: return launch_verify_g<4, 1>(k, vp.depth, f8, s);
    case 4 * 16 + 2: return launch_verify_g<4, 2>(k, vp.depth, f8, s);
    case 4 * 16 + 4: return launch_verify_g<4, 4>(k, vp.depth, f8, s);
    case 8 * 16 + 1: return launch_verify_g<8, 1>(k, vp.depth, f8, s);
    case 8 * 16 + 2: return launch_verify_g<8, 2>(k, vp.depth, f8, s);
    case 8 * 16 + 4: return launch_verify_g<8, 4>(k, vp.depth, f8, s);
    default:
      return fail(PA_ERR_UNSUPPORTED, "pa_forward: multi-token decode with %d query heads per KV head, %d column groups",
                  G, vp.col_groups);
  }
}

}  // namespace pa
