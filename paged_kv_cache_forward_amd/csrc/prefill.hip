// Chunked-prefill attention over paged K/V on the gfx950 matrix cores.
//
// What is computed: "Внутреннее устройство vLLM" (artificials.ru), chunked-
// prefill paragraph, and "vLLM PagedAttention: eine Revolution ..."
// (de.news.hada.io), bullet "Chunked Prefill": a prompt's prefill is cut into
// chunks that run in later steps on top of the tokens already cached.  Query
// row j of a chunk sits at absolute position c + j (c = tokens cached before
// the chunk) and sees keys 0 .. c + j (causal) -- the positional indices and
// masks of the same page's forward-pass paragraph.  The K/V of the prefix and
// of the chunk itself (written before this call) are read through the block
// table like any other cached token.  Prefill is compute-bound (same page as
// above, bullet on disaggregation), so both contractions run on MFMA.
//
// Work-group: 4 waves owning 128 query rows of one KV head g (or 8 waves and
// 256 rows, chosen on the host), a row being a (token, query head) pair:
// row r -> token r / G, head g*G + r % G, so the G heads sharing g share
// every K/V tile; each wave owns 32 rows (two 16-row MFMA tiles).  Launch
// order: KV head fastest (every work-group of one KV head runs on one XCD and
// shares that XCD's L2 for the K/V it re-reads), then the query tile, latest
// tiles (most keys) first, then the sequence (last in the batch first), then
// the key piece (highest first).
//
// K/V tiles of 64 keys (four 16-token cache blocks) are copied global -> LDS
// by the buffer unit, one tile ahead, into a double-buffered LDS stage (no
// registers hold data in flight).  Each copy goes through a buffer resource
// for one cache block whose range ends at the sequence's last token, so slots
// past it (stale, possibly NaN) read as zero and never reach an MFMA.  The
// block table of the work-group's key range is staged in LDS, a window at a
// time.
//
// Contractions, v_mfma_f32_16x16x32_bf16 (A 16x32, B 32x16, C 16x16 fp32):
//   S^T = K Q^T     A = K rows from LDS (lane: key row l % 16, dims 8 (l / 16)
//                   of each 32-dim step), B = Q^T held in registers; the C
//                   fragment gives lane l keys 4q .. 4q+3 (q = l / 16) of
//                   query row l % 16.
//   O^T += V^T P^T  B = P^T straight from two S^T fragments (keys 4q..4q+3 and
//                   16+4q..16+4q+3 of a 32-key step); A = V^T read from the
//                   row-major V tile with ds_read_b64_tr_b16, which hands lane
//                   l four consecutive keys of head-dim column l % 16 when the
//                   16 lanes of its group point at the four key rows (four
//                   lanes per row, four dims each).  No transposing copy.
// Softmax state is per query row, spread over the four lanes holding its
// keys; scores are in base-2 units; the running max only moves when a score
// beats it by 2^8 (kRescaleSlack), so accumulators are rarely rescaled.  P is
// rounded to bf16 (nearest even) for the second MFMA; accumulation is fp32.
// Keys past a row's visible end are masked by select on the tiles that need
// it; tiles past every row of a wave are skipped.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "device.h"
#include "ops.h"
#include "status.h"

namespace pa {
namespace {

// (token, query head) rows per work-group: 16 RT per wave, RT = row tiles per
// wave, NW = waves per work-group (4 or 8).
template <int NW, int RT> constexpr int rows_per_wg() { return 16 * RT * NW; }
constexpr int kKeys = 64;         // keys per tile: four 16-token cache blocks
constexpr int kBtCache = 1024;    // block-table entries staged in LDS (16384 tokens)

// LDS stage of one 64-key tile, filled by buffer-unit copies (16 bytes per
// lane, lane l of a copy landing at its piece base + 16 l), one 1 KiB piece
// per copy, laid out so that every fragment read is conflict-free:
//   K piece (block b, k-step ks): lane (lr, lq) = lq * 16 + lr holds key row
//     16 b + lr, dims 32 ks + 8 lq .. +8 -- exactly the A fragment that lane
//     reads for S^T = K Q^T, so it reads its own 16 bytes back.
//   V piece (block b, dim pair dp): lane dsel * 32 + 2 r + h holds key row
//     16 b + r, dims 16 (2 dp + dsel) + 8 h .. +8; a transpose read for
//     output columns dt = 2 dp + dsel then has each 16-lane group reading
//     128 contiguous bytes.
// Each of the tile's four cache blocks is copied by NW / 4 waves: with
// four waves, wave b copies block b's KS K pieces and DT/2 V pieces; with
// eight, waves 2b and 2b + 1 split them.
template <int D>
struct PCfg {
  static constexpr int ROW = D * 2;                       // bytes of one key row (one KV head)
  static constexpr int TILE = kBlock * ROW;               // bytes of one (block, KV head) tile
  static constexpr int KS = D / 32;                       // MFMA k-steps over the head dim; K pieces per block
  static constexpr int DT = D / 16;                       // 16-column output tiles; DT / 2 V pieces per block
  static constexpr int KBUF = kKeys * ROW;                // K part of a stage
  static constexpr int BUF = 2 * KBUF;                    // one stage: K pieces, then V pieces
  static_assert(KBUF == 4 * KS * 1024 && KBUF == 4 * (DT / 2) * 1024, "1 KiB pieces");
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;   // LDS byte pointer (no generic-pointer checks)


__device__ __forceinline__ u32x4_t buf_ld16v(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}

// fp8 caches (head_dim 128): a plane of code tiles, 16 x 128 E4M3 codes per
// (block, KV head) -- K row-major, V transposed (byte d * 16 + row) -- then a
// plane of row exponents (E8M0, 16 bytes per tile).  A stage holds a tile's
// raw codes and exponents; fragments are converted to bf16 as they are read
// (exactly: power-of-two scales).  Stage layout: K codes of the four blocks
// (2 KiB each, piece p of block b at b * 2048 + p * 1024: lane (lq, lr) = key
// lr, dims 64 p + 16 lq .. +16), V codes (2 KiB each, as stored), then the K
// and the V exponents (16 bytes per block).
constexpr int kF8Tile = kBlock * 128;
constexpr int kF8V = 4 * kF8Tile, kF8KX = 8 * kF8Tile, kF8VX = kF8KX + 4 * kBlock;
constexpr int kF8Stage = kF8VX + 4 * kBlock;

__device__ __forceinline__ float e8m0f(uint32_t c) { return __uint_as_float(c << 23); }
template <bool HI>
__device__ __forceinline__ uint32_t cvt2_fp8(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI));
}
// Eight E4M3 codes (two dwords, memory order) -> eight bf16, times `scale`.
__device__ __forceinline__ bf16x8_t cvt8_fp8(uint32_t w0, uint32_t w1, float scale) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(cvt2_fp8<false>(w0, scale), cvt2_fp8<true>(w0, scale),
                                                 cvt2_fp8<false>(w1, scale), cvt2_fp8<true>(w1, scale)));
}

__device__ __forceinline__ s16x4_t lds_read_tr(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
}

struct PrefillArgs {
  AttnArgs a;
  int32_t tok;          // tokens per query tile (rows per work-group / G)
  int32_t mtok;         // tokens per merge tile (divides tok)
  int32_t mqtiles;      // merge tiles of the longest chunk
  int32_t qtiles;       // query tiles of the longest chunk
  int32_t piece_keys;   // keys per split piece (multiple of kKeys)
  int32_t pieces;       // pieces of the longest key range
  uint16_t* p_o;        // [num_tokens][Hq][pieces][D] partial outputs: fp16, normalised, scaled by 2^-e
  float* p_ml;          // [num_tokens][Hq][pieces][4] partial (max in base-2 units, sum, e, 0)
  int32_t seq_major;    // work-group order: sequences slowest (else pieces slowest)
};

// Which (KV head, query tile, sequence, piece) a work-group handles.  KV head
// fastest (every work-group of one KV head on one XCD), then query tiles.
// Sequences go in descending batch order: a super-batch lists its decode
// sequences before the prefill chunks, and the work-groups of a decode
// sequence find no rows and exit, but each holds an LDS slot for a memory
// round trip first; dispatched after the chunks' work-groups, they fill the
// tail instead of delaying real work.
//  - Pieces slowest (descending; the default): the work-groups in flight
//    together read the same piece of every chunk's key range, a working set
//    that the L2 of each XCD holds.  But every piece level has the decode
//    sequences' empty work-groups after its chunks.
//  - Sequences slowest (seq_major, for batches where most of the grid is
//    empty): all of a chunk's pieces (ascending) before the next chunk, so
//    the empty work-groups of a decode-first batch all come last.
struct PrefillItem {
  int g, p, qt, i;
};
__device__ __forceinline__ PrefillItem prefill_item(int wg, int Hkv, int pieces, int qtiles, int num_seqs,
                                                    bool seq_major) {
  PrefillItem it;
  it.g = wg % Hkv;
  int r = wg / Hkv;
  it.qt = qtiles - 1 - r % qtiles;
  r /= qtiles;
  if (seq_major) {
    it.p = r % pieces;
    it.i = num_seqs - 1 - r / pieces;
  } else {
    it.i = num_seqs - 1 - r % num_seqs;
    it.p = pieces - 1 - r / num_seqs;
  }
  return it;
}

// RT = 2: 32 rows per wave, two waves per SIMD.  RT = 4: 64 rows per wave --
// each K/V fragment read from LDS feeds twice the MFMAs -- with the output
// accumulators in AGPRs at one wave per SIMD.  NW = 8: 256 rows per
// work-group (one per CU), so each K/V tile is copied once for twice the rows
// and a batch's query tiles are half as many.
template <int D, bool F8, int RT, int NW>
__global__ __launch_bounds__(64 * NW, RT >= 4 || NW >= 8 ? 1 : 2) void prefill_kernel(PrefillArgs pk) {
  using C = PCfg<D>;
  constexpr int kThreads = 64 * NW;
  constexpr int kWavesPerBlock = NW / 4;   // waves copying each of a tile's four cache blocks
  constexpr int kRowsPerWG = rows_per_wg<NW, RT>();
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(!F8 || (D == 128 && kWavesPerBlock == 1), "fp8: head_dim 128, one wave per block");
  constexpr int SBUF = F8 ? kF8Stage : C::BUF;   // bytes of one LDS stage
  __shared__ __attribute__((aligned(1024))) uint8_t lds_stage[2 * SBUF];
  __shared__ int s_bt[kBtCache];
  lds_u8* const lds = (lds_u8*)lds_stage;

  const AttnArgs& a = pk.a;
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int TOK = kRowsPerWG / G;
  const PrefillItem it = prefill_item(blockIdx.x, Hkv, pk.pieces, pk.qtiles, a.num_seqs, pk.seq_major);
  const int g = it.g, qt = it.qt, i = it.i;
  const int tid = threadIdx.x, lane = tid & 63;

  // The block table of the work-group's key range passes through LDS in
  // windows of kBtCache entries; a window is refilled (behind a barrier) when
  // the loads reach it, so no global load sits inside the tile loop.  The
  // entries of the first window depend only on the sequence and the piece:
  // one per thread, from the piece's first block, is loaded together with the
  // sequence's lengths, in one memory round trip (entries past the piece's
  // range, still inside the table's row, are loaded and not used).
  const int32_t* bt_row = a.block_tables + (size_t)i * a.bt_stride;
  const int kt0 = it.p * (pk.piece_keys / kKeys);
  int cur_win = kt0 * (kKeys / kBlock) / kBtCache;
  const int bt_spec = kt0 * (kKeys / kBlock) - cur_win * kBtCache + tid;   // this thread's entry of the window
  const int bt_val =
      bt_spec < kBtCache && cur_win * kBtCache + bt_spec < a.bt_stride ? bt_row[cur_win * kBtCache + bt_spec] : 0;
  const int c = a.cached_lens[i];
  const int L_raw = a.seq_lens[i];
  const int q0 = a.qsl[i];
  const int q1 = a.qsl[i + 1];
  asm volatile("" ::"s"(c), "s"(L_raw), "s"(q0), "s"(q1), "v"(bt_val));   // all five loads issued before the checks
  const int n = q1 - q0;
  if (n < max(a.prefill_min_q, 2) || q0 < 0 || q0 + n > a.num_tokens) return;
  const int tok0 = qt * TOK;
  if (tok0 >= n) return;
  const int L = min(L_raw, a.bt_stride * kBlock);
  const int tok_last = min(tok0 + TOK, n) - 1;
  const int kv_end = a.causal ? min(L, c + tok_last + 1) : L;
  if (kv_end <= 0) return;
  // This work-group's piece of the key range; the last piece takes whatever
  // remains, so every key is covered whatever the lengths.
  const int k_lo = it.p * pk.piece_keys;
  if (k_lo >= kv_end) return;
  const int k_hi = it.p == pk.pieces - 1 ? kv_end : min(k_lo + pk.piece_keys, kv_end);
  const bool split = kv_end > pk.piece_keys && pk.pieces > 1;   // partials instead of the output
  const int kt_end = (k_hi + kKeys - 1) / kKeys;
  const int nblk = (k_hi + kBlock - 1) / kBlock;

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;

  auto fill_window = [&](int win) {
    const int b0 = win * kBtCache;
    for (int b = tid; b < min(nblk - b0, kBtCache); b += kThreads) s_bt[b] = clamp_block(bt_row[b0 + b], a.num_blocks);
  };

  // Query fragments (B operand of S^T = K Q^T): lane holds 8 head-dim values of
  // its row: dims 32 ks + 8 lq (bf16 cache); 64 (ks / 2) + 16 lq + 8 (ks % 2)
  // (fp8 cache, matching the K fragments it converts 16 codes at a time).
  bf16x8_t qf[RT][C::KS];
  int row_tok[RT], row_head[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = w * 16 * RT + rt * 16 + lr;
    row_tok[rt] = tok0 + r / G;
    row_head[rt] = g * G + r % G;
    const bool ok = row_tok[rt] < n;
    const uint8_t* qp =
        (const uint8_t*)a.q + ((size_t)(q0 + row_tok[rt]) * a.num_q_heads + row_head[rt]) * C::ROW;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int qoff = F8 ? (ks / 2) * 128 + lq * 32 + (ks % 2) * 16 : ks * 64 + lq * 16;
      const uint4 v = ok ? ld16(qp + qoff) : make_uint4(0u, 0u, 0u, 0u);
      qf[rt][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // The first window's entries, behind the query loads (still in flight): the
  // one already loaded, then any further ones of a range of more than
  // kThreads blocks.
  {
    const int win_end = min(nblk - cur_win * kBtCache, kBtCache);
    if (bt_spec < win_end) s_bt[bt_spec] = clamp_block(bt_val, a.num_blocks);
    for (int b = bt_spec + kThreads; b < win_end; b += kThreads)
      s_bt[b] = clamp_block(bt_row[cur_win * kBtCache + b], a.num_blocks);
  }

  // Exponent arguments are cs * s - m in base-2 units (cs = |scale| log2 e),
  // one fma per score; a negative scale is folded into Q by exact sign flips,
  // so the running max can be taken over raw scores.
  // cs >= 1e-30 so that a masked score (-inf) always gives a -inf argument;
  // at scale 0 the arguments stay 0 to fp32 precision (uniform weights).
  const float cs = fmaxf(fabsf(a.scale_log2), 1e-30f);
  if (a.scale_log2 < 0.0f) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        uint4 u = __builtin_bit_cast(uint4, qf[rt][ks]);
        u.x ^= 0x80008000u; u.y ^= 0x80008000u; u.z ^= 0x80008000u; u.w ^= 0x80008000u;
        qf[rt][ks] = __builtin_bit_cast(bf16x8_t, u);
      }
  }
  // A operand of all ones: the extra output tile o[rt][DT] accumulates each
  // row's sum of the (bf16) weights on the matrix cores, in every element.
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

  float m[RT];
  f32x4_t o[RT][C::DT + 1];
  int lim[RT];   // keys visible to row tile rt's row of this lane: t < lim
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kNegBig;
    lim[rt] = a.causal ? min(L, c + row_tok[rt] + 1) : L;
#pragma unroll
    for (int dt = 0; dt <= C::DT; ++dt) o[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int wave_tok_last = min(tok0 + (w * 16 * RT + 16 * RT - 1) / G, n - 1);

  constexpr int CTILE = F8 ? kF8Tile : C::TILE;      // bytes of one (block, KV head) code tile
  const size_t block_stride = (size_t)Hkv * CTILE;
  const uint8_t* kc = (const uint8_t*)a.k_cache + (size_t)g * CTILE;
  const uint8_t* vc = (const uint8_t*)a.v_cache + (size_t)g * CTILE;
  // fp8: the exponent plane after all code tiles, 16 bytes per tile.
  const uint8_t* kx = (const uint8_t*)a.k_cache + (size_t)a.num_blocks * block_stride + (size_t)g * kBlock;
  const uint8_t* vx = (const uint8_t*)a.v_cache + (size_t)a.num_blocks * block_stride + (size_t)g * kBlock;

  auto block_id = [&](int b) -> int {   // b < nblk, inside the current window, wave-uniform
    return __builtin_amdgcn_readfirstlane(s_bt[b - cur_win * kBtCache]);
  };

  // Copy tile kt of the key range into LDS stage `buf` (this wave: block w of
  // the tile).  Each copy goes through a buffer resource for one cache block
  // whose range ends at the sequence's last token, so rows past it read as
  // zero.  A tile past the end is not copied (it is never computed).
  const int dsel = lane >> 5, vr2 = (lane & 31) >> 1, vh = lane & 1;
  auto dma_tile = [&](int kt, int buf) {
    if (kt >= kt_end) return;
    const int win = kt * (kKeys / kBlock) / kBtCache;   // a tile never straddles two windows
    if (win != cur_win) {
      cur_win = win;
      fill_window(win);
      __syncthreads();
    }
    const int blk = kt * (kKeys / kBlock) + w / kWavesPerBlock;
    const int part = w % kWavesPerBlock;   // with two waves per block: 0 copies K, 1 copies V
    const int rows = __builtin_amdgcn_readfirstlane(blk < nblk ? min(max(L - blk * kBlock, 0), kBlock) : 0);
    const int bid = rows > 0 ? block_id(blk) : 0;
    const size_t off = (size_t)bid * block_stride;
    const int b = w / kWavesPerBlock;
    if constexpr (F8) {
      // K codes (rows past the sequence read as zero), V codes (masked where
      // read), and lanes 0..3 copy the block's 16 K and 16 V exponents.
      const u32x4_t rk = rsrc_words(kc + off, rows * 128);
      const u32x4_t rv = rsrc_words(vc + off, kF8Tile);
      const u32x4_t rkx = rsrc_words(kx + (size_t)bid * Hkv * kBlock, kBlock);
      const u32x4_t rvx = rsrc_words(vx + (size_t)bid * Hkv * kBlock, kBlock);
      uint8_t* st8 = lds_stage + buf * SBUF;
#pragma unroll
      for (int p = 0; p < 2; ++p) lds_copy16(rk, st8 + b * kF8Tile + p * 1024, lr * 128 + p * 64 + lq * 16);
#pragma unroll
      for (int p = 0; p < 2; ++p) lds_copy16(rv, st8 + kF8V + b * kF8Tile + p * 1024, p * 1024 + lane * 16);
      if (lane < 4) {
        lds_copy4(rkx, st8 + kF8KX + b * kBlock, 4 * lane);
        lds_copy4(rvx, st8 + kF8VX + b * kBlock, 4 * lane);
      }
      return;
    }
    const u32x4_t rk = rsrc_words(kc + off, rows * C::ROW);
    const u32x4_t rv = rsrc_words(vc + off, rows * C::ROW);
    if (kWavesPerBlock == 1 || part == 0) {   // the block's K pieces
      uint8_t* kdst = lds_stage + buf * SBUF + b * C::KS * 1024;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) lds_copy16(rk, kdst + ks * 1024, lr * C::ROW + ks * 64 + lq * 16);
    }
    if (kWavesPerBlock == 1 || part == 1) {   // its V pieces
      uint8_t* vdst = lds_stage + buf * SBUF + C::KBUF + b * (C::DT / 2) * 1024;
#pragma unroll
      for (int dp = 0; dp < C::DT / 2; ++dp)
        lds_copy16(rv, vdst + dp * 1024, vr2 * C::ROW + (2 * dp + dsel) * 32 + vh * 16);
    }
  };

  // Per-lane LDS addresses of the K and V fragments; every fragment read is
  // one of these plus an immediate offset.
  // (Both stages' offsets fit the 16-bit immediate: at most 65024 bytes at D = 128.)
  const lds_u8* k_lane = lds + lane * 16;
  const lds_u8* v_lane = lds + C::KBUF + (4 * lq + (lr >> 2)) * 32 + (lr & 3) * 8;

  // Online softmax of one tile's scores s (raw), weights to bf16 P^T
  // fragments.  Keys at or past a row's visible limit get score -inf, by one
  // compare against a per-row threshold and one select per score, only in
  // lanes that hold such keys (one code path: the register allocation stays
  // tight).
  auto softmax_tile = [&](f32x4_t (&s)[RT][4], int key0, bf16x8_t (&pb)[RT][2]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int t = lim[rt] - key0 - lq * 4;   // key kt16 * 16 + e of this lane is visible iff < t
      if (t < 3 * 16 + 4) {   // some key of this lane is not visible (diagonal and last tiles)
#pragma unroll
        for (int kt16 = 0; kt16 < 4; ++kt16)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[rt][kt16][e] = kt16 * 16 + e < t ? s[rt][kt16][e] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt16 = 0; kt16 < 4; ++kt16)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[rt][kt16][e]);
      const float mxs = mx * cs;   // -inf when this lane sees no key of the tile
      if (__any(mxs > m[rt] + kRescaleSlack)) {   // rare after a row's first tile
        float rm = fmaxf(mxs, __shfl_xor(mxs, 16));
        rm = fmaxf(rm, __shfl_xor(rm, 32));
        const float mn = fmaxf(m[rt], rm);
        const float alpha = fast_exp2(m[rt] - mn);
        m[rt] = mn;
#pragma unroll
        for (int dt = 0; dt <= C::DT; ++dt) o[rt][dt] *= alpha;
      }
      auto weight = [&](int kt16, int e) { return fast_exp2(fmaf(s[rt][kt16][e], cs, -m[rt])); };
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[rt][ks2][e] = static_cast<__bf16>(weight(2 * ks2, e));
          pb[rt][ks2][4 + e] = static_cast<__bf16>(weight(2 * ks2 + 1, e));
        }
    }
  };

  auto compute = [&](int kt, int buf) {
    const int key0 = kt * kKeys;
    if (a.causal && key0 > c + wave_tok_last) return;   // past every row of this wave
    const lds_u8* kl = k_lane + buf * SBUF;
    const lds_u8* vl = v_lane + buf * SBUF;
    const lds_u8* st8 = lds + buf * SBUF;
    // Wave priority: raised over the two MFMA phases, lowered over the
    // softmax, so of the two waves sharing a SIMD the one with products to
    // issue goes first (measured on MI355X: 148.7 -> 147.0 us bf16, 212 -> 208
    // us fp8, same box, alternating runs).
    __builtin_amdgcn_s_setprio(2);
    f32x4_t s[RT][4];
    // bf16: the K fragments of 16-key block kt16 + 1 are read while block
    // kt16's MFMAs run (two register sets), so each block's LDS reads are in
    // flight behind the previous block's products instead of in front of
    // their own.
    typedef const __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
    bf16x8_t kfr[2][C::KS];
    if constexpr (!F8) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) kfr[0][ks] = *reinterpret_cast<lds_bf16x8*>(kl + ks * 1024);
    }
#pragma unroll
    for (int kt16 = 0; kt16 < 4; ++kt16) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s[rt][kt16] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (F8) {
        // Block kt16: each 16-code piece gives two k-steps, converted with key lr's scale.
        const float ksc = e8m0f(st8[kF8KX + kt16 * kBlock + lr]);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint4 raw = __builtin_bit_cast(
              uint4, *reinterpret_cast<const lds_u32x4_t*>(st8 + kt16 * kF8Tile + p * 1024 + lane * 16));
          const bf16x8_t k0 = cvt8_fp8(raw.x, raw.y, ksc), k1 = cvt8_fp8(raw.z, raw.w, ksc);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            s[rt][kt16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[rt][2 * p], s[rt][kt16], 0, 0, 0);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            s[rt][kt16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[rt][2 * p + 1], s[rt][kt16], 0, 0, 0);
        }
      } else {
        if (kt16 + 1 < 4) {
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks)
            kfr[(kt16 + 1) & 1][ks] = *reinterpret_cast<lds_bf16x8*>(kl + ((kt16 + 1) * C::KS + ks) * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);   // the next block's reads stay ahead of these products
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            s[rt][kt16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr[kt16 & 1][ks], qf[rt][ks], s[rt][kt16], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (F8 && kt16 == 1) __builtin_amdgcn_sched_barrier(0);   // bound how far fragment reads are hoisted
    }
    bf16x8_t pb[RT][2];
    __builtin_amdgcn_s_setprio(0);
    softmax_tile(s, key0, pb);
    __builtin_amdgcn_s_setprio(2);
    if constexpr (F8) {
      // P.V on the fp8 codes: the product takes each weight times its key's V
      // exponent (exact), the row sums (ones tile) the weights alone.  Keys
      // past the sequence: weight 0 and codes zeroed (stale bytes may be NaN codes).
      bf16x8_t pv[RT][2];
      uint32_t keep[2][2];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int blk = 2 * ks2 + h;
          const uint32_t xw = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(
              st8 + kF8VX + blk * kBlock + 4 * lq);
          int live = 4;
          if (key0 + kKeys > L) live = min(max(L - key0 - 16 * blk - 4 * lq, 0), 4);   // wave-uniform test
          keep[ks2][h] = live >= 4 ? 0xffffffffu : live == 0 ? 0u : (1u << (8 * live)) - 1u;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sv = e < live ? e8m0f((xw >> (8 * e)) & 0xffu) : 0.0f;
              pv[rt][ks2][4 * h + e] = static_cast<__bf16>(static_cast<float>(pb[rt][ks2][4 * h + e]) * sv);
            }
        }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          // keys 4 lq .. +3 of blocks 2 ks2 and 2 ks2 + 1, dim 16 dt + lr: one dword of each block's row
          const lds_u8* vp = st8 + kF8V + (16 * dt + lr) * kBlock + 4 * lq;
          const uint32_t w0 = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(
                                  vp + (2 * ks2) * kF8Tile) & keep[ks2][0];
          const uint32_t w1 = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(
                                  vp + (2 * ks2 + 1) * kF8Tile) & keep[ks2][1];
          const bf16x8_t vf = cvt8_fp8(w0, w1, 1.0f);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pv[rt][ks2], o[rt][dt], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          // keys 32 ks2 + 4 lq + lr / 4 (block 2 ks2) and 16 further (block 2 ks2 + 1)
          const lds_u8* vp = vl + (2 * ks2 * (C::DT / 2) + dt / 2) * 1024 + (dt & 1) * 512;
          const s16x4_t v0 = lds_read_tr(vp);
          const s16x4_t v1 = lds_read_tr(vp + (C::DT / 2) * 1024);
          const bf16x8_t vf = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[rt][ks2], o[rt][dt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        o[rt][C::DT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[rt][ks2], o[rt][C::DT], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Pipeline: tile kt+1 is copied into the other LDS stage while tile kt is
  // computed; each wave then waits for its own copies, and the barrier makes
  // every wave's copies visible (and frees the stage just read for refill).
  __syncthreads();   // first block-table window ready
  dma_tile(kt0, 0);
  // The query fragments are loaded by ordinary global loads, which the
  // compiler tracks: without a wait it can see here, it waits for them
  // (vmcnt(0)) at their first use inside the tile loop, on every iteration,
  // and that wait also drains the untracked copies of the next tile issued
  // just before -- serialising copy and compute.  s_waitcnt vmcnt(0)
  // (simm16 0x0F70: expcnt and lgkmcnt left at their maxima) retires them
  // here, together with the first tile's copies: one round trip for both.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int kt = kt0; kt < kt_end; kt += 2) {
    dma_tile(kt + 1, 1);
    compute(kt, 0);
    PA_VM_WAIT(0);
    __syncthreads();
    if (kt + 1 >= kt_end) break;
    dma_tile(kt + 2, 0);
    compute(kt + 1, 1);
    PA_VM_WAIT(0);
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lt = o[rt][C::DT][0];   // the row's weight sum (ones tile)
    if (row_tok[rt] >= n) continue;
    if (split) {
      // Piece it.p of this row: its output normalised by its own weight sum,
      // times 2^-e in fp16, with e set by the row's largest magnitude so that
      // it lands in [2^14, 2^15): full fp16 precision whatever the range of
      // V, through exact power-of-two scalings; beside it the max (base 2),
      // the sum and e.  Half the bytes of fp32 partials, to write here and
      // read in the merge.  A piece past a row's causal limit (sum 0) stores
      // zeros and (kNegBig, 0, 0): weight 0 in the merge.
      const size_t item = ((size_t)(q0 + row_tok[rt]) * a.num_q_heads + row_head[rt]) * pk.pieces + it.p;
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      float amax = 0.0f;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(o[rt][dt][e] * inv));
      amax = fmaxf(amax, __shfl_xor(amax, 16));   // the row's four lanes (lq)
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const int ex = amax > 0.0f ? max(ilogbf(amax) - 14, -100) : 0;
      uint16_t* po = pk.p_o + item * D;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const _Float16 lo = static_cast<_Float16>(ldexpf(o[rt][dt][2 * h] * inv, -ex));
          const _Float16 hi = static_cast<_Float16>(ldexpf(o[rt][dt][2 * h + 1] * inv, -ex));
          w[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *reinterpret_cast<uint2*>(po + dt * 16 + lq * 4) = make_uint2(w[0], w[1]);
      }
      if (lq == 0) *reinterpret_cast<float4*>(pk.p_ml + item * 4) = make_float4(m[rt], lt, (float)ex, 0.0f);
      continue;
    }
    const float inv = 1.0f / lt;
    uint8_t* op = (uint8_t*)a.out + ((size_t)(q0 + row_tok[rt]) * a.num_q_heads + row_head[rt]) * C::ROW;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const f32x4_t v = o[rt][dt] * inv;
      *reinterpret_cast<uint2*>(op + (dt * 16 + lq * 4) * 2) =
          make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

// Prefill split-KV merge: one work-group per (KV head, query tile, sequence)
// whose key range was split; eight threads per (token, head) row, each owning
// 16 dims (D / 8), so a merge tile's 128 rows take 1024 threads, each one row
// slice: one memory round trip for up to four pieces.  Measured on MI355X on
// the mixed super-batch's four chunks: 14.5 us with fp32 partials, 12.4 us
// with fp16 ones, 11.6 us with a thread per slice instead of 256 threads
// looping over four slices each.  Pieces are folded four at a time with their
// loads issued together, in ascending order with the log-sum-exp rule, so the
// result is deterministic.
constexpr int kMergeThreads = 1024;
template <int D>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(PrefillArgs pk) {
  constexpr int SL = D / 8;            // dims per thread
  constexpr int NV = SL / 8;           // 16-byte (eight fp16) loads per piece per thread
  constexpr int U = 4;                 // pieces per round trip
  const AttnArgs& a = pk.a;
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const PrefillItem it = prefill_item(blockIdx.x, Hkv, 1, pk.mqtiles, a.num_seqs, false);
  const int q0 = a.qsl[it.i];
  const int n = a.qsl[it.i + 1] - q0;
  if (n < max(a.prefill_min_q, 2) || q0 < 0 || q0 + n > a.num_tokens) return;
  const int tok0 = it.qt * pk.mtok;   // this merge tile's tokens
  if (tok0 >= n) return;
  // The prefill tile holding these tokens decided whether its rows went to
  // partials, and how many pieces it wrote.
  const int ptok0 = tok0 / pk.tok * pk.tok;
  const int L = min(a.seq_lens[it.i], a.bt_stride * kBlock);
  const int c = a.cached_lens[it.i];
  const int ptok_last = min(ptok0 + pk.tok, n) - 1;
  const int kv_end = a.causal ? min(L, c + ptok_last + 1) : L;
  if (kv_end <= pk.piece_keys || pk.pieces <= 1) return;   // written by the prefill kernel itself
  const int np = min((kv_end + pk.piece_keys - 1) / pk.piece_keys, pk.pieces);
  const int tok_last = min(tok0 + pk.mtok, n) - 1;
  const int rows = (tok_last - tok0 + 1) * G;   // rows are token-major: the first `rows` are valid
  for (int idx = threadIdx.x; idx < rows * 8; idx += kMergeThreads) {
    const int r = idx >> 3, sl = idx & 7;
    const int tok = tok0 + r / G, head = it.g * G + r % G;
    const size_t item0 = ((size_t)(q0 + tok) * a.num_q_heads + head) * pk.pieces;
    const float4* ml = reinterpret_cast<const float4*>(pk.p_ml) + item0;
    float Mx = -INFINITY, den = 0.0f;
    float acc[SL];
#pragma unroll
    for (int e = 0; e < SL; ++e) acc[e] = 0.0f;
    for (int p0 = 0; p0 < np; p0 += U) {
      float4 v[U];
      uint4 x[U][NV];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p0 + u < np) {
          v[u] = ml[p0 + u];
          const uint4* src = reinterpret_cast<const uint4*>(pk.p_o + (item0 + p0 + u) * D + sl * SL);
#pragma unroll
          for (int q = 0; q < NV; ++q) x[u][q] = src[q];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p0 + u >= np) break;
        // Piece u's output is sum * 2^e * (the stored values); a piece past
        // the row's causal limit holds (kNegBig, 0, 0): weight 0.
        const float Mn = fmaxf(Mx, v[u].x);
        const float sa = fast_exp2(Mx - Mn), sb = fast_exp2(v[u].x - Mn);
        den = fmaf(den, sa, v[u].y * sb);
        const float wv = ldexpf(v[u].y * sb, (int)v[u].z);
#pragma unroll
        for (int q = 0; q < NV; ++q) {
          const uint32_t wq[4] = {x[u][q].x, x[u][q].y, x[u][q].z, x[u][q].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const float lo = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(wq[h] & 0xffffu)));
            const float hi = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(wq[h] >> 16)));
            acc[8 * q + 2 * h] = fmaf(acc[8 * q + 2 * h], sa, lo * wv);
            acc[8 * q + 2 * h + 1] = fmaf(acc[8 * q + 2 * h + 1], sa, hi * wv);
          }
        }
        Mx = Mn;
      }
    }
    const float inv = 1.0f / den;
    uint8_t* op = (uint8_t*)a.out + ((size_t)(q0 + tok) * a.num_q_heads + head) * (D * 2) + sl * SL * 2;
#pragma unroll
    for (int q = 0; q < SL / 8; ++q)
      *reinterpret_cast<uint4*>(op + q * 16) = make_uint4(
          pack_bf16x2(acc[8 * q] * inv, acc[8 * q + 1] * inv), pack_bf16x2(acc[8 * q + 2] * inv, acc[8 * q + 3] * inv),
          pack_bf16x2(acc[8 * q + 4] * inv, acc[8 * q + 5] * inv), pack_bf16x2(acc[8 * q + 6] * inv, acc[8 * q + 7] * inv));
  }
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool prefill_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  if (group < 1 || rows_per_wg<4, 2>() % group != 0) return false;
  if (dtype == PA_FP8) return head_dim == 128;
  return dtype == PA_BF16 && (head_dim == 64 || head_dim == 128);
}

PrefillPlan make_prefill_plan(int32_t num_tokens, int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                              int32_t max_query_len, bool mfma) {
  PrefillPlan pp{};
  pp.piece_keys = 1 << 30;
  pp.pieces = 1;
  if (!mfma || max_query_len <= 1 || max_seq_len <= 0) return pp;
  // A work-group's key range is cut into at most four pieces of at least
  // 1024 keys, so the longest chunk is spread over more CUs and every CU keeps
  // two work-groups busy; PA_PREFILL_SPLIT=off|<keys> overrides.
  int64_t keys = std::max<int64_t>(1024, ((int64_t)(max_seq_len + 3) / 4 + kKeys - 1) / kKeys * kKeys);
  if (const char* env = std::getenv("PA_PREFILL_SPLIT")) {
    if (std::strcmp(env, "off") == 0) keys = (int64_t)1 << 30;
    else if (std::atoi(env) >= kKeys) keys = (std::atoi(env) + kKeys - 1) / kKeys * kKeys;
  }
  pp.piece_keys = (int32_t)std::min<int64_t>(keys, (int64_t)1 << 30);
  pp.pieces = (int32_t)std::max<int64_t>(1, ((int64_t)max_seq_len + pp.piece_keys - 1) / pp.piece_keys);
  if (pp.pieces > 1) {
    const size_t items = (size_t)num_tokens * num_q_heads * pp.pieces;
    pp.o_bytes = round256(items * head_dim * sizeof(uint16_t));
    pp.ml_bytes = round256(items * 4 * sizeof(float));
  }
  return pp;
}

pa_status launch_prefill(const AttnArgs& a, int32_t max_query_len, const PrefillPlan& pp, uint16_t* p_o, float* p_ml,
                         bool fp8, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  // Row tiles per wave: 2 (32 rows, two waves per SIMD).  PA_PREFILL_ROWS=64
  // selects 64 rows per wave at one wave per SIMD (head_dim 128): half the LDS
  // bytes per MFMA, but measured on MI355X 1.5x slower -- one wave per SIMD
  // does not hide the LDS and MFMA latencies.
  int rt = 2;
  if (const char* env = std::getenv("PA_PREFILL_ROWS")) {
    if (std::strcmp(env, "64") == 0 && a.head_dim == 128) rt = 4;
  }
  // Waves per work-group (bf16, head_dim 128, 32 rows per wave): four (128
  // rows, two work-groups per CU).  The grid holds a work-group per (query
  // tile, KV head, piece) for every sequence of the batch, and those of
  // sequences that are not chunks find no rows and exit; eight waves (256
  // rows, one work-group per CU) halve those, but measured on MI355X four
  // waves are faster on both shapes: 16 decode sequences + 4 chunks of 512,
  // 139.3-139.7 us vs 141.4-141.9 us; the 4 chunks alone, 141-150 us vs
  // 150-156 us (without the clocks settled first).  PA_PREFILL_WAVES=8
  // selects eight.
  int nw = 4;
  if (!fp8 && a.head_dim == 128 && rt == 2) {
    if (const char* env = std::getenv("PA_PREFILL_WAVES")) nw = std::atoi(env) == 8 ? 8 : 4;
  }
  const int TOK = 16 * rt * nw / G;
  const int qtiles = (max_query_len + TOK - 1) / TOK;
  const int64_t tiles = (int64_t)qtiles * a.num_kv_heads * a.num_seqs;
  const int64_t wgs = tiles * pp.pieces;
  if (a.head_dim != 64 && a.head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: prefill head_dim %d", a.head_dim);
  if (wgs > 0x7fffffff / (64 * nw))
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: prefill grid of %lld work-groups", (long long)wgs);
  if (pp.pieces > 1 && (p_o == nullptr || p_ml == nullptr))
    return fail(PA_ERR_ARG, "pa_forward: prefill split needs workspace");
  // The merge works on tiles of at most 128 rows, whatever the prefill tile:
  // with 256-row prefill tiles that doubles its work-groups.
  const int MTOK = TOK * G > 128 && TOK % 2 == 0 ? TOK / 2 : TOK;
  const int mqtiles = (max_query_len + MTOK - 1) / MTOK;
  // Sequences-slowest order where most of the (sequence, query tile) grid
  // has no rows (the query tokens would fill fewer than half of it).
  // Measured on MI355X, 16 decode sequences + 4 chunks of 512 tokens: 154.8
  // -> 148.7 us (the four chunks alone: 142.8 us in the default order, 149.0
  // in this one).  PA_PREFILL_ORDER=pieces|sequences overrides.
  int seq_major = (int64_t)a.num_seqs * max_query_len > 2 * (int64_t)a.num_tokens;
  if (const char* env = std::getenv("PA_PREFILL_ORDER")) {
    if (std::strcmp(env, "sequences") == 0) seq_major = 1;
    else if (std::strcmp(env, "pieces") == 0) seq_major = 0;
  }
  PrefillArgs k{a, TOK, MTOK, mqtiles, qtiles, pp.piece_keys, pp.pieces, p_o, p_ml, seq_major};
  if (fp8 && a.head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "pa_forward: fp8 prefill head_dim %d", a.head_dim);
  int mark = trace_begin(s);
  const dim3 grid((unsigned)wgs), block(64 * nw);
  if (fp8 && rt == 4) hipLaunchKernelGGL((prefill_kernel<128, true, 4, 4>), grid, block, 0, s, k);
  else if (fp8) hipLaunchKernelGGL((prefill_kernel<128, true, 2, 4>), grid, block, 0, s, k);
  else if (a.head_dim == 128 && rt == 4) hipLaunchKernelGGL((prefill_kernel<128, false, 4, 4>), grid, block, 0, s, k);
  else if (a.head_dim == 128 && nw == 8) hipLaunchKernelGGL((prefill_kernel<128, false, 2, 8>), grid, block, 0, s, k);
  else if (a.head_dim == 128) hipLaunchKernelGGL((prefill_kernel<128, false, 2, 4>), grid, block, 0, s, k);
  else hipLaunchKernelGGL((prefill_kernel<64, false, 2, 4>), grid, block, 0, s, k);
  trace_end(s, mark, "prefill");
  pa_status st = launch_status("pa_forward (prefill)");
  if (st != PA_OK || pp.pieces <= 1) return st;
  mark = trace_begin(s);
  const dim3 mgrid((unsigned)((int64_t)mqtiles * a.num_kv_heads * a.num_seqs));
  if (a.head_dim == 128) hipLaunchKernelGGL((prefill_merge_kernel<128>), mgrid, dim3(kMergeThreads), 0, s, k);
  else hipLaunchKernelGGL((prefill_merge_kernel<64>), mgrid, dim3(kMergeThreads), 0, s, k);
  trace_end(s, mark, "prefill_merge");
  return launch_status("pa_forward (prefill merge)");
}

}  // namespace pa
