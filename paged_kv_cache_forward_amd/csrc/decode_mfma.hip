// Decode attention for bf16 K/V with head_dim 128: scores on the matrix cores,
// P.V on the vector ALUs, split-KV partitions written for the merge kernel.
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
// Work item: one work-group of NW waves per (sequence i, KV head g, partition
// p of `part_tokens` tokens).  Wave w folds tiles w, w+NW, ... of the partition.
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
// Finish: the row groups are combined with the log-sum-exp rule, then the NW
// waves through LDS.  A sequence with one partition writes its output;
// otherwise each partition writes (max, sum, acc) to the workspace and the
// merge kernel, launched next on the same stream, combines the partitions in
// ascending order.  (Merging inside this kernel -- the last partition to finish
// merging the rest -- needs an agent-scope release per partition, i.e. an L2
// write-back per work-group; measured on MI355X that serialises at roughly
// 0.5 us per partition per XCD and cost more than the separate launch.)
//
// Start-up: the block-table entries of a wave's first tiles are requested
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
    auto issue = [&](int jj, uint4 (&kq)[4], uint4 (&vq)[4]) {
      const size_t off = (size_t)__builtin_amdgcn_readlane(my_bid, jj) * block_stride;
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc + off, kTileBytes);
      const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc + off, kTileBytes);
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
      issue(min(jj + 1, nb - 1), kb, vb);
      fold<G>(ka, va, qf, tok_base + jj * NW * kBlock, t1, r, a.scale_log2, st);
      if (jj + 1 >= nb) break;
      issue(min(jj + 2, nb - 1), ka, va);
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

}  // namespace

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
