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
// Tiling: a workgroup (4 waves) owns 128 query rows of one KV head g, a row
// being a (token, query head) pair: row r -> token r / G, head g*G + r % G,
// so the G heads sharing g share every K/V tile.  Each wave owns 32 rows
// (two 16-row MFMA tiles).  Keys stream in tiles of 64 (four 16-token cache
// blocks) through double-buffered LDS.
//
// Contractions use v_mfma_f32_16x16x32_bf16 (A 16x32, B 32x16, C 16x16 fp32):
//   S^T = K Q^T   A = K tile rows (keys) from LDS, B = Q^T from registers;
//                 the C fragment leaves lane l with four consecutive keys of
//                 one query row (row = l % 16);
//   O^T += V^T P^T  B = P^T taken straight from two S^T fragments (keys
//                 4q..4q+3 and 16+4q..16+4q+3 of a 32-key step, q = l / 16),
//                 A = V^T read from a transposed LDS copy of the V tile with
//                 the same key order, so no shuffles are needed; the C
//                 fragment leaves lane l with four head-dim columns of its own
//                 query row, so the softmax rescale is per lane.
// Softmax statistics are per query row, reduced across the four lanes sharing
// it; scores are in base-2 units.  P is rounded to bf16 for the second MFMA;
// accumulation stays fp32.  Keys past the visible end are masked by select
// and V rows past it are zeroed in LDS, so stale or NaN slots never reach an
// accumulator.
#include "device.h"
#include "ops.h"
#include "status.h"

namespace pa {

constexpr int kRowsPerWG = 128;
constexpr int kKeysPerTile = 64;

template <int D>
struct PCfg {
  static constexpr int KS = D / 32;                       // MFMA k-steps over the head dim
  static constexpr int DT = D / 16;                       // 16-column output tiles
  static constexpr int CPK = D / 8;                       // 16-byte chunks per key row
  static constexpr int KC = kKeysPerTile * CPK / 256;     // K chunks per thread per tile
  static constexpr int VK = D / 32;                       // V keys per thread per tile
  static constexpr int K_STRIDE = D * 2 + 16;             // LDS bytes per key row (padded)
  static constexpr int V_STRIDE = kKeysPerTile * 2 + 8;   // LDS bytes per head-dim row of V^T
  static constexpr int K_BYTES = kKeysPerTile * K_STRIDE;
  static constexpr int V_BYTES = D * V_STRIDE;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
  static_assert(KC * 256 == kKeysPerTile * CPK, "K tile split");
  static_assert((256 / CPK) * VK == kKeysPerTile && kBlock % VK == 0, "V tile split");
};

// Element x (0..7) of a chunk of eight bf16, as the low 16 bits of a dword.
__device__ __forceinline__ uint32_t bf16_at(const uint4& w, int x) {
  const uint32_t word = (x >> 1) == 0 ? w.x : (x >> 1) == 1 ? w.y : (x >> 1) == 2 ? w.z : w.w;
  return (x & 1) ? (word >> 16) : (word & 0xffffu);
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(AttnArgs a) {
  using C = PCfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::BUF_BYTES];

  const int G = a.num_q_heads / a.num_kv_heads;
  const int TOK = kRowsPerWG / G;
  const int i = blockIdx.z, g = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;   // later query tiles see more keys: start them first
  const int q0 = a.qsl[i];
  const int n = a.qsl[i + 1] - q0;
  if (n <= 1 || q0 < 0 || q0 + n > a.num_tokens) return;
  const int tok0 = qt * TOK;
  if (tok0 >= n) return;
  const int L = min(a.seq_lens[i], a.bt_stride * kBlock);
  const int c = a.cached_lens[i];
  const int tok_last = min(tok0 + TOK, n) - 1;
  const int kv_end = a.causal ? min(L, c + tok_last + 1) : L;
  if (kv_end <= 0) return;
  const int ntiles = (kv_end + kKeysPerTile - 1) / kKeysPerTile;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const size_t row_bytes = (size_t)D * 2;

  // Query fragments (B operand of S^T = K Q^T): lane holds 8 head-dim values of its row.
  bf16x8_t qf[2][C::KS];
  int row_tok[2], row_head[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = w * 32 + rt * 16 + lr;
    row_tok[rt] = tok0 + r / G;
    row_head[rt] = g * G + r % G;
    const bool ok = row_tok[rt] < n;
    const uint8_t* qp = (const uint8_t*)a.q + ((size_t)(q0 + row_tok[rt]) * a.num_q_heads + row_head[rt]) * row_bytes;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 v = ok ? ld16(qp + ks * 64 + lq * 16) : make_uint4(0u, 0u, 0u, 0u);
      qf[rt][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  float m[2] = {kNegBig, kNegBig};
  float l[2] = {0.0f, 0.0f};
  f32x4_t o[2][C::DT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) o[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wave_tok_first = tok0 + (w * 32) / G;
  const int wave_tok_last = min(tok0 + (w * 32 + 31) / G, n - 1);
  const int vis_min = a.causal ? min(L, c + wave_tok_first + 1) : L;  // keys every row of the wave sees

  const int32_t* bt_row = a.block_tables + (size_t)i * a.bt_stride;
  const size_t tile_bytes = (size_t)kBlock * row_bytes;            // one (block, head) tile
  const size_t block_stride = (size_t)a.num_kv_heads * tile_bytes;
  const uint8_t* kc = (const uint8_t*)a.k_cache + (size_t)g * tile_bytes;
  const uint8_t* vc = (const uint8_t*)a.v_cache + (size_t)g * tile_bytes;

  // Staging registers: K chunk (key kc_key, 16B column kc_col) and V keys vk0..vk0+VK-1 at column v_col.
  uint4 kst[C::KC];
  uint4 vst[C::VK];
  const int v_col = tid % C::CPK;
  const int v_kg = tid / C::CPK;

  auto load_tile = [&](int kt) {
    const int key0 = kt * kKeysPerTile;
#pragma unroll
    for (int u = 0; u < C::KC; ++u) {
      const int ch = tid + 256 * u;
      const int key = ch / C::CPK, col = ch % C::CPK;
      const int kabs = key0 + key;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (kabs < kv_end) {
        const int bid = clamp_block(bt_row[kabs / kBlock], a.num_blocks);
        v = ld16(kc + bid * block_stride + (kabs % kBlock) * row_bytes + col * 16);
      }
      kst[u] = v;
    }
    const int vkey0 = key0 + v_kg * C::VK;   // VK consecutive keys, all inside one cache block
    const int bid = vkey0 < kv_end ? clamp_block(bt_row[vkey0 / kBlock], a.num_blocks) : 0;
#pragma unroll
    for (int e = 0; e < C::VK; ++e) {
      const int kabs = vkey0 + e;
      vst[e] = kabs < kv_end ? ld16(vc + bid * block_stride + (kabs % kBlock) * row_bytes + v_col * 16)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  auto store_tile = [&](int buf) {
    uint8_t* kl = lds + buf * C::BUF_BYTES;
    uint8_t* vl = kl + C::K_BYTES;
#pragma unroll
    for (int u = 0; u < C::KC; ++u) {
      const int ch = tid + 256 * u;
      const int key = ch / C::CPK, col = ch % C::CPK;
      *reinterpret_cast<uint4*>(kl + key * C::K_STRIDE + col * 16) = kst[u];
    }
    // V^T: head-dim row d = v_col*8 + x gets this thread's VK keys, consecutive.
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      uint8_t* dst = vl + (v_col * 8 + x) * C::V_STRIDE + v_kg * C::VK * 2;
      if constexpr (C::VK == 4) {
        const uint32_t lo = bf16_at(vst[0], x) | (bf16_at(vst[1], x) << 16);
        const uint32_t hi = bf16_at(vst[2], x) | (bf16_at(vst[3], x) << 16);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<uint32_t*>(dst) = bf16_at(vst[0], x) | (bf16_at(vst[1], x) << 16);
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) load_tile(kt + 1);
    const int key0 = kt * kKeysPerTile;
    const bool skip = a.causal && key0 > c + wave_tok_last;   // every row of this wave is past it
    if (!skip) {
      const uint8_t* kl = lds + buf * C::BUF_BYTES;
      const uint8_t* vl = kl + C::K_BYTES;
      f32x4_t s[2][4];
#pragma unroll
      for (int kt16 = 0; kt16 < 4; ++kt16) {
        s[0][kt16] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        s[1][kt16] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kl + (kt16 * 16 + lr) * C::K_STRIDE + ks * 64 + lq * 16);
          s[0][kt16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], s[0][kt16], 0, 0, 0);
          s[1][kt16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][ks], s[1][kt16], 0, 0, 0);
        }
      }
      const bool full = key0 + kKeysPerTile <= vis_min;
      bf16x8_t pb[2][2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int lim = a.causal ? min(L, c + row_tok[rt] + 1) : L;
        float mx = -INFINITY;
#pragma unroll
        for (int kt16 = 0; kt16 < 4; ++kt16)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v = s[rt][kt16][e] * a.scale_log2;
            if (!full) v = (key0 + kt16 * 16 + lq * 4 + e) < lim ? v : -INFINITY;
            s[rt][kt16][e] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m[rt], mx);
        const float alpha = fast_exp2(m[rt] - mn);
        m[rt] = mn;
        float ls = 0.0f;
#pragma unroll
        for (int kt16 = 0; kt16 < 4; ++kt16)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = fast_exp2(s[rt][kt16][e] - mn);
            s[rt][kt16][e] = p;
            ls += p;
          }
        l[rt] = fmaf(l[rt], alpha, ls);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) o[rt][dt] *= alpha;
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pb[rt][ks2][e] = static_cast<__bf16>(s[rt][2 * ks2][e]);
            pb[rt][ks2][4 + e] = static_cast<__bf16>(s[rt][2 * ks2 + 1][e]);
          }
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          const uint8_t* vp = vl + (dt * 16 + lr) * C::V_STRIDE + (ks2 * 32 + lq * 4) * 2;
          const uint2 v0 = *reinterpret_cast<const uint2*>(vp);
          const uint2 v1 = *reinterpret_cast<const uint2*>(vp + 32);
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
          o[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[0][ks2], o[0][dt], 0, 0, 0);
          o[1][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[1][ks2], o[1][dt], 0, 0, 0);
        }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float lt = l[rt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (row_tok[rt] >= n) continue;
    const float inv = 1.0f / lt;
    uint8_t* op = (uint8_t*)a.out + ((size_t)(q0 + row_tok[rt]) * a.num_q_heads + row_head[rt]) * row_bytes;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const f32x4_t v = o[rt][dt] * inv;
      *reinterpret_cast<uint2*>(op + (dt * 16 + lq * 4) * 2) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

bool prefill_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  return dtype == PA_BF16 && (head_dim == 64 || head_dim == 128) && group >= 1 &&
         kRowsPerWG % group == 0;
}

pa_status launch_prefill(const AttnArgs& a, int32_t max_query_len, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int TOK = kRowsPerWG / G;
  dim3 grid((max_query_len + TOK - 1) / TOK, a.num_kv_heads, a.num_seqs);
  if (a.head_dim != 64 && a.head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: prefill head_dim %d", a.head_dim);
  const int mark = trace_begin(s);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(256), 0, s, a);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(256), 0, s, a);
  else
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: prefill head_dim %d", a.head_dim);
  trace_end(s, mark, "prefill");
  return launch_status("pa_forward (prefill)");
}

}  // namespace pa
