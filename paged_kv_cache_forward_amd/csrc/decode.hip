// Decode attention over paged K/V (one query token per sequence), split-KV.
//
// What is computed: "PagedAttention et vLLM" (aiunderstanding.org), section
// "Plongée profonde": the new token attends to every cached key/value of its
// sequence, and those live in fixed-size blocks anywhere in memory, found
// through a table from logical positions to physical blocks.  "Внутреннее
// устройство vLLM" (artificials.ru), forward-pass paragraph: each sequence of
// the super-batch sees only its own tokens.  "vLLM PagedAttention: eine
// Revolution ..." (de.news.hada.io), bullet on disaggregation: decode is bound
// by memory bandwidth, so this kernel is built around the K/V stream.
//
// Work item = one wavefront for (partition p of sequence i, KV head g), serving
// all G query heads of that KV head, so each K/V byte is read once per KV head.
// A partition is `part_tokens` consecutive logical tokens (a multiple of 16).
//
// Lane layout for one 16-token block tile of one KV head (16 rows x D elems,
// contiguous): the tile is CPL consecutive 1 KiB (for bf16 D128) runs; run u
// is loaded by all 64 lanes with one 16-byte load each (fully coalesced).  Lane
// l holds chunk `col = l % CPR` (E elements of the head dim) of token row
// `u * R + rg`, rg = l / CPR.  So the R lane groups ("row groups") each own a
// fixed subset of every block's tokens.
//
// Scores: per-lane partial dot products (bf16 pairs through v_dot2_f32_bf16, or
// fp32 FMAs) summed across the CPR lanes of a row group with DPP row ops.
// Each row group keeps its own online-softmax state (running max m, sum l,
// fp32 accumulator for its E output columns per query head); the R states are
// combined once at the end of the item with the log-sum-exp rule, so no
// cross-row-group traffic happens per block.  Scores are in base-2 units
// (scale * log2 e folded in) so the exponentials are single v_exp_f32.
//
// Masking selects (never multiplies): keys past the partition end get score
// -inf and their V chunks are zeroed, so stale or NaN slots in a sequence's
// last block never reach an accumulator.
//
// Output: a sequence with one partition writes its normalised result directly;
// otherwise each partition writes (m, l, acc) to the workspace and the merge
// kernel below combines them in ascending partition order.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "device.h"
#include "ops.h"
#include "status.h"

namespace pa {

constexpr int kMaxParts = 4096;   // bound on partitions per sequence

struct DecodeKernelArgs {
  AttnArgs a;
  int32_t part_tokens;
  int32_t max_parts;
  float* p_acc;   // [num_seqs][Hq][max_parts][D]
  float* p_ml;    // [num_seqs][Hq][max_parts][2]  (m in base-2 units, l)
  int32_t rows_mode;
};

template <typename T, int D>
struct Tile {
  static constexpr int E = Elem<T>::per16;   // elements per 16-byte chunk
  static constexpr int CPR = D / E;          // chunks per token row
  static constexpr int R = 64 / CPR;         // row groups
  static constexpr int CPL = kBlock / R;     // chunks each lane loads per block tile
  static constexpr int ROW_BYTES = D * Elem<T>::bytes;
  static_assert(CPR == 8 || CPR == 16 || CPR == 32, "head_dim / dtype combination");
};

// Widen one 16-byte chunk to E floats.
template <typename T>
__device__ __forceinline__ void widen(uint4 w, float* f);
template <>
__device__ __forceinline__ void widen<float>(uint4 w, float* f) {
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}
template <>
__device__ __forceinline__ void widen<uint16_t>(uint4 w, float* f) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// Partial dot product of one query chunk with one key chunk.
template <typename T>
__device__ __forceinline__ float chunk_dot(uint4 q, uint4 k);
template <>
__device__ __forceinline__ float chunk_dot<uint16_t>(uint4 q, uint4 k) {
  float d = dot2_bf16(q.x, k.x, 0.0f);
  d = dot2_bf16(q.y, k.y, d);
  d = dot2_bf16(q.z, k.z, d);
  return dot2_bf16(q.w, k.w, d);
}
template <>
__device__ __forceinline__ float chunk_dot<float>(uint4 q, uint4 k) {
  float d = __uint_as_float(q.x) * __uint_as_float(k.x);
  d = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), d);
  d = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), d);
  return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), d);
}

// Store E floats as one 16-byte chunk of T.
template <typename T>
__device__ __forceinline__ void store_chunk(void* p, const float* f);
template <>
__device__ __forceinline__ void store_chunk<float>(void* p, const float* f) {
  st16(p, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                     __float_as_uint(f[3])));
}
template <>
__device__ __forceinline__ void store_chunk<uint16_t>(void* p, const float* f) {
  st16(p, make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7])));
}

// Online-softmax state of one row group for the G query heads.
template <int G, int E>
struct RowState {
  float m[G];
  float l[G];
  float acc[G][E];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegBig;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
    }
  }
};

// One (block, KV head) tile: 16 rows of ROW_BYTES, addressed through a buffer
// descriptor built in SGPRs from the block's base pointer, so each lane's
// offset inside the tile is a constant and no per-block vector address math is
// needed.  The descriptor's range is exactly the tile.
template <typename T, int D>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int lane_off,
                                          uint4 (&kq)[Tile<T, D>::CPL], uint4 (&vq)[Tile<T, D>::CPL]) {
  using TL = Tile<T, D>;
#pragma unroll
  for (int u = 0; u < TL::CPL; ++u) kq[u] = buf_ld16(rk, lane_off + u * TL::R * TL::ROW_BYTES);
#pragma unroll
  for (int u = 0; u < TL::CPL; ++u) vq[u] = buf_ld16(rv, lane_off + u * TL::R * TL::ROW_BYTES);
}

// Fold one block tile (tokens tok0 .. tok0+15) into the row group's state.
template <typename T, int D, int G>
__device__ __forceinline__ void fold_tile(const uint4 (&kq)[Tile<T, D>::CPL], uint4 (&vq)[Tile<T, D>::CPL],
                                          const uint4 (&qv)[G], int tok0, int t_end, int rg,
                                          float scale_log2, RowState<G, Tile<T, D>::E>& st) {
  using TL = Tile<T, D>;
  constexpr int CPL = TL::CPL, E = TL::E;
  float s[CPL][G];
#pragma unroll
  for (int u = 0; u < CPL; ++u)
#pragma unroll
    for (int h = 0; h < G; ++h) s[u][h] = group_sum<TL::CPR>(chunk_dot<T>(qv[h], kq[u])) * scale_log2;

  if (tok0 + kBlock > t_end) {  // wave-uniform: only a range's last block is partial
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const bool valid = tok0 + u * TL::R + rg < t_end;
#pragma unroll
      for (int h = 0; h < G; ++h) s[u][h] = valid ? s[u][h] : -INFINITY;
      if (!valid) vq[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  float vf[CPL][E];
#pragma unroll
  for (int u = 0; u < CPL; ++u) widen<T>(vq[u], vf[u]);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float bm = s[0][h];
#pragma unroll
    for (int u = 1; u < CPL; ++u) bm = fmaxf(bm, s[u][h]);
    const bool need = bm > st.m[h] + kRescaleSlack;
    if (__any(need)) {  // wave-uniform branch; rare after a range's first block
      const float mn = need ? bm : st.m[h];
      const float alpha = fast_exp2(st.m[h] - mn);
      st.m[h] = mn;
      st.l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) st.acc[h][e] *= alpha;
    }
    float p[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      p[u] = fast_exp2(s[u][h] - st.m[h]);
      st.l[h] += p[u];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float a = st.acc[h][e];
#pragma unroll
      for (int u = 0; u < CPL; ++u) a = fmaf(p[u], vf[u][e], a);
      st.acc[h][e] = a;
    }
  }
}

// Attend query row `row` of sequence i (KV head g) over logical tokens [t0, t1);
// t0 is a multiple of 16 and t1 > t0.
//
// Blocks stream through two register buffers: while one block is folded the
// next one's loads are in flight.  The prefetch is issued unconditionally
// (past the last block it reads an empty range: zeros, no memory traffic) so
// the compiler's wait counts only ever wait for the buffer being folded,
// never for the one in flight.
//
// With `fw` (a fused cache write; [t0, t1) ends at the sequence's last token,
// the step's new one), the row of token t1 - 1 is taken from the step's new
// K/V rows instead of the cache and stored into the cache at its place.
template <typename T, int D, int G>
__device__ __forceinline__ void attend_range(const AttnArgs& a, int i, int g, int row, int t0, int t1,
                                             RowState<G, Tile<T, D>::E>& st, bool fw = false) {
  using TL = Tile<T, D>;
  constexpr int CPL = TL::CPL;
  const int lane = threadIdx.x;
  const int col = lane % TL::CPR;
  const int rg = lane / TL::CPR;
  const int lane_off = rg * TL::ROW_BYTES + col * 16;

  uint4 qv[G];
  const uint8_t* qrow = (const uint8_t*)a.q + ((size_t)row * a.num_q_heads + (size_t)g * G) * TL::ROW_BYTES;
#pragma unroll
  for (int h = 0; h < G; ++h) qv[h] = ld16(qrow + h * TL::ROW_BYTES + col * 16);

  const int32_t* bt_row = a.block_tables + (size_t)i * a.bt_stride;
  constexpr int tile_bytes = kBlock * TL::ROW_BYTES;
  const uint8_t* kc = (const uint8_t*)a.k_cache + (size_t)g * tile_bytes;
  const uint8_t* vc = (const uint8_t*)a.v_cache + (size_t)g * tile_bytes;
  const size_t block_stride = (size_t)a.num_kv_heads * tile_bytes;

  uint4 kn = make_uint4(0u, 0u, 0u, 0u), vn = kn;
  if (fw) {   // the new token's K/V chunk of this lane's column
    const size_t nrow = ((size_t)row * a.num_kv_heads + g) * TL::ROW_BYTES + col * 16;
    kn = ld16((const uint8_t*)a.k_new + nrow);
    vn = ld16((const uint8_t*)a.v_new + nrow);
  }

  const int b_first = t0 / kBlock;
  const int nbt = (t1 - 1) / kBlock - b_first + 1;
  for (int bb = 0; bb < nbt; bb += 64) {
    const int nb = min(64, nbt - bb);
    const int my_bid = lane < nb ? clamp_block(bt_row[b_first + bb + lane], a.num_blocks) : 0;
    const int tok_base = (b_first + bb) * kBlock;
    uint4 ka[CPL], va[CPL], kb[CPL], vb[CPL];
    // A prefetch past the last block (j >= nb) reads an empty range: zeros, no memory traffic.
    auto issue = [&](int j, uint4 (&kq)[CPL], uint4 (&vq)[CPL]) {
      const int bytes = j < nb ? tile_bytes : 0;
      const size_t off = (size_t)__builtin_amdgcn_readlane(my_bid, min(j, nb - 1)) * block_stride;
      load_tile<T, D>(tile_rsrc(kc + off, bytes), tile_rsrc(vc + off, bytes), lane_off, kq, vq);
    };
    // Fused write: in the block holding token t1 - 1, the lanes of its row
    // take the new chunks and store them into the cache.
    auto patch = [&](int j, uint4 (&kq)[CPL], uint4 (&vq)[CPL]) {
      const int tok0 = tok_base + j * kBlock;
      if (!fw || tok0 + kBlock < t1) return;   // wave-uniform
      const int rho = t1 - 1 - tok0;
      if (rg != rho % TL::R) return;
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        if (u == rho / TL::R) {
          kq[u] = kn;
          vq[u] = vn;
        }
      }
      const size_t off = (size_t)__builtin_amdgcn_readlane(my_bid, j) * block_stride + rho * TL::ROW_BYTES + col * 16;
      st16((uint8_t*)a.k_cache + (size_t)g * tile_bytes + off, kn);
      st16((uint8_t*)a.v_cache + (size_t)g * tile_bytes + off, vn);
    };
    issue(0, ka, va);
    for (int j = 0; j < nb; j += 2) {
      issue(j + 1, kb, vb);
      patch(j, ka, va);
      fold_tile<T, D, G>(ka, va, qv, tok_base + j * kBlock, t1, rg, a.scale_log2, st);
      if (j + 1 >= nb) break;
      issue(j + 2, ka, va);
      patch(j + 1, kb, vb);
      fold_tile<T, D, G>(kb, vb, qv, tok_base + (j + 1) * kBlock, t1, rg, a.scale_log2, st);
    }
  }
}

// Combine the R row-group states; lanes of row group 0 end up with the totals
// for their columns.  Returns per head: M (base-2 max), Lsum, and acc in `out`.
template <typename T, int D, int G>
__device__ __forceinline__ void combine_row_groups(RowState<G, Tile<T, D>::E>& st) {
  using TL = Tile<T, D>;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = cross_group_max<TL::CPR>(st.m[h]);
    const float f = fast_exp2(st.m[h] - M);
    st.l[h] = cross_group_sum<TL::CPR>(st.l[h] * f);
#pragma unroll
    for (int e = 0; e < TL::E; ++e) st.acc[h][e] = cross_group_sum<TL::CPR>(st.acc[h][e] * f);
    st.m[h] = M;
  }
}

template <typename T, int D, int G>
__device__ __forceinline__ void write_final(const AttnArgs& a, int row, int g, const RowState<G, Tile<T, D>::E>& st) {
  using TL = Tile<T, D>;
  const int lane = threadIdx.x;
  if (lane >= TL::CPR) return;
  uint8_t* orow = (uint8_t*)a.out + ((size_t)row * a.num_q_heads + (size_t)g * G) * TL::ROW_BYTES;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float inv = 1.0f / st.l[h];
    float f[TL::E];
#pragma unroll
    for (int e = 0; e < TL::E; ++e) f[e] = st.acc[h][e] * inv;
    store_chunk<T>(orow + h * TL::ROW_BYTES + lane * 16, f);
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(64) void decode_kernel(DecodeKernelArgs k) {
  using TL = Tile<T, D>;
  const AttnArgs& a = k.a;
  const int p = blockIdx.x, g = blockIdx.y, i = blockIdx.z;
  const int q0 = a.qsl[i];
  const int n = a.qsl[i + 1] - q0;
  if (n <= 0 || q0 < 0 || q0 + n > a.num_tokens) return;  // rows outside q/out: nothing to do
  const int L = min(a.seq_lens[i], a.bt_stride * kBlock);
  RowState<G, TL::E> st;

  if (n == 1) {
    const int t0 = p * k.part_tokens;
    if (t0 >= L) return;
    const int t1 = min(t0 + k.part_tokens, L);
    st.init();
    attend_range<T, D, G>(a, i, g, q0, t0, t1, st, a.k_new != nullptr && t1 == L);
    combine_row_groups<T, D, G>(st);
    if (k.max_parts == 1 || L <= k.part_tokens) {
      write_final<T, D, G>(a, q0, g, st);
      return;
    }
    const int lane = threadIdx.x;
    if (lane >= TL::CPR) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const size_t item = ((size_t)i * a.num_q_heads + (size_t)g * G + h) * k.max_parts + p;
      float* dst = k.p_acc + item * D + lane * TL::E;
#pragma unroll
      for (int e = 0; e < TL::E; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(st.acc[h][e], st.acc[h][e + 1], st.acc[h][e + 2], st.acc[h][e + 3]);
      if (lane == 0) *reinterpret_cast<float2*>(k.p_ml + item * 2) = make_float2(st.m[h], st.l[h]);
    }
    return;
  }

  // Multi-token sequence on the vector path: one query row at a time, unsplit.
  if (!k.rows_mode || p != 0) return;
  const int c = a.cached_lens[i];
  for (int j = 0; j < n; ++j) {
    const int t1 = a.causal ? min(c + j + 1, L) : L;
    if (t1 <= 0) continue;
    st.init();
    attend_range<T, D, G>(a, i, g, q0 + j, 0, t1, st);
    combine_row_groups<T, D, G>(st);
    write_final<T, D, G>(a, q0 + j, g, st);
  }
}

// Split-KV merge: one work-group of 256 threads per (sequence, query head).
// The threads form R = 256 / (D/4) row groups of D/4 lanes (four output
// columns per lane); row group r folds partitions r, r+R, r+2R, ... in that
// order with the log-sum-exp rule, U partitions at a time so their loads are
// in flight together, and the R row groups are then combined in ascending
// order through LDS.  The order is fixed, so the result is deterministic.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int32_t part_tokens, int32_t max_parts,
                                                    const float* __restrict__ p_acc,
                                                    const float* __restrict__ p_ml) {
  constexpr int TPR = D / 4;      // lanes per partition row
  constexpr int R = 256 / TPR;    // row groups
  constexpr int U = 4;            // partitions per row group per batch
  __shared__ float s_m[R], s_l[R];
  __shared__ float4 s_acc[R][TPR];
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int q0 = a.qsl[i];
  if (a.qsl[i + 1] - q0 != 1 || q0 < 0 || q0 >= a.num_tokens) return;
  const int L = min(a.seq_lens[i], a.bt_stride * kBlock);
  // The decode kernel wrote at most max_parts partitions (grid width).
  const int P = min((L + part_tokens - 1) / part_tokens, max_parts);
  if (P <= 1) return;
  const size_t item0 = ((size_t)i * a.num_q_heads + h) * max_parts;
  const float2* ml = reinterpret_cast<const float2*>(p_ml) + item0;
  const float4* acc = reinterpret_cast<const float4*>(p_acc + item0 * D);
  const int d4 = tid % TPR, r = tid / TPR;

  float M = -INFINITY, den = 0.0f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = r; p0 < P; p0 += R * U) {
    float2 v[U];
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pp = p0 + u * R;
      if (pp < P) {
        v[u] = ml[pp];
        x[u] = acc[(size_t)pp * TPR + d4];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (p0 + u * R >= P) break;
      const float Mn = fmaxf(M, v[u].x);       // partition maxima are finite
      const float sa = fast_exp2(M - Mn);      // 0 on the first partition (M = -inf)
      const float sb = fast_exp2(v[u].x - Mn);
      den = fmaf(den, sa, v[u].y * sb);
      num.x = fmaf(num.x, sa, x[u].x * sb);
      num.y = fmaf(num.y, sa, x[u].y * sb);
      num.z = fmaf(num.z, sa, x[u].z * sb);
      num.w = fmaf(num.w, sa, x[u].w * sb);
      M = Mn;
    }
  }
  s_acc[r][d4] = num;
  if (d4 == 0) {
    s_m[r] = M;
    s_l[r] = den;
  }
  __syncthreads();
  if (r != 0) return;
  float Mt = s_m[0];
#pragma unroll
  for (int q = 1; q < R; ++q) Mt = fmaxf(Mt, s_m[q]);
  float dt = 0.0f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const float f = fast_exp2(s_m[q] - Mt);   // row groups without partitions: -inf -> 0
    const float4 y = s_acc[q][d4];
    dt = fmaf(f, s_l[q], dt);
    o.x = fmaf(f, y.x, o.x); o.y = fmaf(f, y.y, o.y); o.z = fmaf(f, y.z, o.z); o.w = fmaf(f, y.w, o.w);
  }
  const float inv = 1.0f / dt;
  float f4[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
  uint8_t* orow = (uint8_t*)a.out + ((size_t)q0 * a.num_q_heads + h) * D * Elem<T>::bytes;
  if constexpr (Elem<T>::bytes == 2) {
    *reinterpret_cast<uint2*>(orow + d4 * 8) = make_uint2(pack_bf16x2(f4[0], f4[1]), pack_bf16x2(f4[2], f4[3]));
  } else {
    *reinterpret_cast<float4*>(orow + d4 * 16) = make_float4(f4[0], f4[1], f4[2], f4[3]);
  }
}

// ---------------------------------------------------------------------------

static size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

DecodePlan make_decode_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t dtype, int32_t max_seq_len) {
  DecodePlan pl{};
  const int32_t group = num_kv_heads > 0 ? num_q_heads / num_kv_heads : 0;
  const char* kind = std::getenv("PA_DECODE");
  pl.mfma = decode_mfma_supported(dtype, head_dim, group) && !(kind != nullptr && std::strcmp(kind, "valu") == 0);
  const int32_t whole = max_seq_len > 0 ? ((max_seq_len + kBlock - 1) / kBlock) * kBlock : kBlock;
  int32_t part = whole;
  const char* env = std::getenv("PA_SPLIT");
  if (env != nullptr && std::strcmp(env, "off") == 0) {
    part = whole;
  } else if (env != nullptr && std::strcmp(env, "auto") != 0 && env[0] != '\0') {
    part = std::atoi(env);
    if (part < kBlock || part % kBlock != 0 || part > 8192) part = 512;
  } else if (max_seq_len > 256) {
    // Size partitions so that (sequence, KV head, partition) work-groups number
    // about 4096 (several per CU, so the dispatcher balances ragged lengths),
    // at least 128 tokens each: part ~ S * Hkv * max_seq_len / 4096, rounded
    // to the nearest power of two in [128, 2048].  Measured on MI355X.
    const double want = (double)num_seqs * num_kv_heads * max_seq_len / 4096.0;
    part = 128;
    while (part < 2048 && want > 1.5 * part) part *= 2;
  }
  // Long partitions are shared by four waves of one work-group.
  pl.waves = part >= 2048 ? 4 : 1;
  if (const char* wv = std::getenv("PA_DECODE_WAVES")) {
    const int v = std::atoi(wv);
    if (v == 1 || v == 2 || v == 4) pl.waves = v;
  }
  while ((whole + part - 1) / part > kMaxParts) part *= 2;
  pl.part_tokens = part;
  pl.max_parts = (whole + part - 1) / part;
  pl.balanced = pl.mfma && decode_balanced_supported(num_seqs) &&
                !(kind != nullptr && std::strcmp(kind, "partition") == 0);
  if (pl.balanced) {
    // 1024 single-wave work-groups in all: one per SIMD, every one resident
    // at once, never more than the tiles there can be; two tiles in flight.
    // Measured on MI355X with the non-temporal tile copies (same box, two
    // runs each, us of decode): batched decode 87.5-88.2 at depth 2 against
    // 89.1-89.5 at depth 3 and 90.0-90.1 at depth 4; long context equal;
    // a shared prefix 245-246 against 255-256.  768, 1280 or 1536 waves are
    // slower.  PA_DECODE_TOTAL_WAVES and PA_DECODE_DEPTH override.
    int64_t target = 1024;
    if (const char* tw = std::getenv("PA_DECODE_TOTAL_WAVES")) {
      const int v = std::atoi(tw);
      if (v >= 1 && v <= 65536) target = v;
    }
    const int64_t max_tiles = (int64_t)num_seqs * (whole / kBlock);
    const int64_t wg = std::max<int64_t>(1, std::min<int64_t>(target / num_kv_heads, max_tiles));
    pl.waves_per_head = (int32_t)wg;
    pl.depth = 2;
    if (const char* dp = std::getenv("PA_DECODE_DEPTH")) {
      const int v = std::atoi(dp);
      if (v >= 2 && v <= 4) pl.depth = v;
    }
    pl.part_tokens = whole;
    pl.max_parts = 1;
    const size_t slots = (size_t)num_seqs + (size_t)wg;
    pl.info_bytes = round256((size_t)num_seqs * 2 * sizeof(int32_t));
    pl.acc_bytes = round256(slots * num_q_heads * head_dim * sizeof(float));
    pl.ml_bytes = round256(slots * num_q_heads * 2 * sizeof(float));
  } else if (pl.max_parts > 1) {
    const size_t items = (size_t)num_seqs * num_q_heads * pl.max_parts;
    pl.acc_bytes = round256(items * head_dim * sizeof(float));
    pl.ml_bytes = round256(items * 2 * sizeof(float));
  }
  return pl;
}

template <typename T, int D>
static pa_status launch_decode_d(const DecodeKernelArgs& k, int G, dim3 grid, hipStream_t s) {
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: query heads per KV head %d", G);
  const int mark = trace_begin(s);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_kernel<T, D, 1>), grid, dim3(64), 0, s, k); break;
    case 2: hipLaunchKernelGGL((decode_kernel<T, D, 2>), grid, dim3(64), 0, s, k); break;
    case 4: hipLaunchKernelGGL((decode_kernel<T, D, 4>), grid, dim3(64), 0, s, k); break;
    case 8: hipLaunchKernelGGL((decode_kernel<T, D, 8>), grid, dim3(64), 0, s, k); break;
    default: return fail(PA_ERR_UNSUPPORTED, "pa_forward: query heads per KV head %d", G);
  }
  trace_end(s, mark, "decode_valu");
  return launch_status("pa_forward (decode)");
}

pa_status launch_decode(const AttnArgs& a, int32_t dtype, const DecodePlan& plan, float* partial_acc,
                        float* partial_ml, bool rows_mode, hipStream_t s) {
  DecodeKernelArgs k{a, plan.part_tokens, plan.max_parts, partial_acc, partial_ml, rows_mode ? 1 : 0};
  const int G = a.num_q_heads / a.num_kv_heads;
  dim3 grid(plan.max_parts, a.num_kv_heads, a.num_seqs);
  if (dtype == PA_BF16 && a.head_dim == 128) return launch_decode_d<uint16_t, 128>(k, G, grid, s);
  if (dtype == PA_BF16 && a.head_dim == 64) return launch_decode_d<uint16_t, 64>(k, G, grid, s);
  if (dtype == PA_F32 && a.head_dim == 128) return launch_decode_d<float, 128>(k, G, grid, s);
  if (dtype == PA_F32 && a.head_dim == 64) return launch_decode_d<float, 64>(k, G, grid, s);
  return fail(PA_ERR_UNSUPPORTED, "pa_forward: head_dim %d", a.head_dim);
}

pa_status launch_merge(const AttnArgs& a, int32_t dtype, const DecodePlan& plan,
                       const float* partial_acc, const float* partial_ml, hipStream_t s) {
  if (a.head_dim != 64 && a.head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "pa_forward: head_dim %d", a.head_dim);
  dim3 grid(a.num_seqs, a.num_q_heads);
  const int mark = trace_begin(s);
  if (dtype == PA_BF16 && a.head_dim == 128)
    hipLaunchKernelGGL((merge_kernel<uint16_t, 128>), grid, dim3(256), 0, s, a, plan.part_tokens,
                       plan.max_parts, partial_acc, partial_ml);
  else if (dtype == PA_BF16 && a.head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<uint16_t, 64>), grid, dim3(256), 0, s, a, plan.part_tokens,
                       plan.max_parts, partial_acc, partial_ml);
  else if (dtype == PA_F32 && a.head_dim == 128)
    hipLaunchKernelGGL((merge_kernel<float, 128>), grid, dim3(256), 0, s, a, plan.part_tokens,
                       plan.max_parts, partial_acc, partial_ml);
  else if (dtype == PA_F32 && a.head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<float, 64>), grid, dim3(256), 0, s, a, plan.part_tokens,
                       plan.max_parts, partial_acc, partial_ml);
  else
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: head_dim %d", a.head_dim);
  trace_end(s, mark, "merge");
  return launch_status("pa_forward (merge)");
}

}  // namespace pa
