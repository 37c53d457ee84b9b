// Cache write through a slot mapping, and whole-block copies for copy-on-write.
//
// Write: "Was ändert PagedAttention an der KV-Speicherzuweisung für LLMs?"
// (slavadubrov.com), lead paragraph: a block table sends each logical position
// of a request to a physical block; the per-token slot flattens that mapping.
// Copy: same page, section "Gemeinsame Nutzung erfordert mehr als
// Speicherzuweisung", and "PagedAttention et vLLM" (aiunderstanding.org), FAQ on
// sharing: a shared block is copied only when a request diverges.
//
// Both kernels move 16-byte chunks: one lane per chunk, consecutive lanes on
// consecutive source bytes, so every wave reads and writes whole 1 KiB runs
// (a token's row for one KV head is head_dim * elem bytes, 256 B for bf16 D128).
//
// Quantised (fp8) pools: "Was ändert PagedAttention ..." section "Gemeinsame
// Nutzung erfordert mehr als Speicherzuweisung" (cache quantisation) and
// "PagedAttention et vLLM" section "L'avenir de PagedAttention et vLLM".  The
// write quantises each (token, KV head) row with its own power-of-two scale:
// one wave per row, two dims per lane (head_dim 128).
#include <vector>

#include "device.h"
#include "ops.h"
#include "status.h"

namespace pa {

// grid.x covers tokens * chunks_per_token chunks, grid.y = 0 for K, 1 for V.
__global__ __launch_bounds__(256) void write_kv_kernel(const uint8_t* __restrict__ k,
                                                       const uint8_t* __restrict__ v,
                                                       uint8_t* __restrict__ k_cache,
                                                       uint8_t* __restrict__ v_cache,
                                                       const int64_t* __restrict__ slots,
                                                       int64_t total_chunks, int chunks_per_token,
                                                       int chunks_per_row, int64_t num_slots) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  const uint8_t* src = blockIdx.y == 0 ? k : v;
  uint8_t* dst = blockIdx.y == 0 ? k_cache : v_cache;
  const int64_t t = idx / chunks_per_token;
  const int c = (int)(idx - t * chunks_per_token);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;  // padding token, or a slot outside the pool
  const int h = c / chunks_per_row;           // KV head
  const int cc = c - h * chunks_per_row;      // 16-byte chunk inside the row
  const int64_t blk = slot / kBlock;
  const int row = (int)(slot - blk * kBlock);
  const int num_kv_heads = chunks_per_token / chunks_per_row;
  const int64_t dst_chunk = ((blk * num_kv_heads + h) * kBlock + row) * chunks_per_row + cc;
  st16(dst + dst_chunk * 16, ld16(src + idx * 16));
}

// grid.x = pair, grid.y = 0 for K, 1 for V (and, for fp8 pools, 2 / 3 for the
// K / V exponent planes, which start at plane2 bytes and hold chunks2 16-byte
// chunks per block); each work-group copies one block's region.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int chunks_per_block, int num_blocks, int64_t plane2,
                                                          int chunks2) {
  const int src = pairs[2 * blockIdx.x];
  const int dst = pairs[2 * blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  uint8_t* cache = (blockIdx.y & 1) == 0 ? k_cache : v_cache;
  const int per = blockIdx.y < 2 ? chunks_per_block : chunks2;
  if (blockIdx.y >= 2) cache += plane2;
  const uint8_t* s = cache + (int64_t)src * per * 16;
  uint8_t* d = cache + (int64_t)dst * per * 16;
  for (int c = threadIdx.x; c < per; c += blockDim.x) st16(d + c * 16, ld16(s + c * 16));
}

// Smallest e in [-126, 127] with amax <= 448 * 2^e (0 for amax = 0).  amax =
// f * 2^E with f in [1, 2): 448 = 1.75 * 2^8, so e = E - 8, plus one when f > 1.75.
// A subnormal amax (below 2^-126) takes the lower limit.
__device__ __forceinline__ int fp8_row_exponent(float amax) {
  if (amax == 0.0f) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)(b >> 23) - 127;
  const int e = E - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return min(max(e, -126), 127);
}

// E4M3 (OCP, FN) code of x * 2^-e, which lies in [-448, 448] for a finite x:
// nearest value, ties to an even mantissa; the sign of zero is kept.  Below
// 2^-6 the code counts steps of 2^-9 (eight steps are the smallest normal,
// code 0x08); above, mantissa (f - 1) * 8 of y = f * 2^E, a carry moving to
// the next binade.  E4M3 FN has no infinity: a NaN or infinite x is stored as
// the NaN code 0x7f with x's sign bit.
__device__ __forceinline__ uint32_t fp8_code(float x, int e) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  if (!__builtin_isfinite(x)) return sign | 0x7fu;
  const float a = fabsf(ldexpf(x, -e));
  if (a < 0x1p-6f) return sign | (uint32_t)(int)rintf(a * 512.0f);
  int E = (int)(__float_as_uint(a) >> 23) - 127;
  uint32_t q = (uint32_t)(int)rintf((ldexpf(a, -E) - 1.0f) * 8.0f);
  if (q == 8u) {
    q = 0u;
    ++E;
  }
  return sign | ((uint32_t)(E + 7) << 3) | q;
}

// grid.x covers (token, KV head) rows four waves per block, grid.y = 0 for K, 1 for V.
// A pool is a plane of code tiles (kBlock * 128 bytes per (block, KV head))
// followed by a plane of row exponents (kBlock bytes per tile).
__global__ __launch_bounds__(256) void write_kv_fp8_kernel(const uint32_t* __restrict__ k,
                                                           const uint32_t* __restrict__ v,
                                                           uint8_t* __restrict__ k_cache,
                                                           uint8_t* __restrict__ v_cache,
                                                           const int64_t* __restrict__ slots, int64_t rows,
                                                           int num_kv_heads, int64_t num_slots) {
  constexpr int D = 128, TILE = kBlock * D;
  const int64_t rw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (token, KV head) row, wave-uniform
  const int lane = threadIdx.x & 63;
  if (rw >= rows) return;
  const int64_t t = rw / num_kv_heads;
  const int h = (int)(rw - t * num_kv_heads);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;  // padding token, or a slot outside the pool
  const bool is_v = blockIdx.y != 0;
  const uint32_t w = (is_v ? v : k)[rw * (D / 2) + lane];   // dims 2 lane, 2 lane + 1 (bf16)
  const float x0 = bf16_lo(w), x1 = bf16_hi(w);
  // The scale comes from the row's finite elements only.
  const float a0 = __builtin_isfinite(x0) ? fabsf(x0) : 0.0f;
  const float a1 = __builtin_isfinite(x1) ? fabsf(x1) : 0.0f;
  const int e = fp8_row_exponent(wave_max(fmaxf(a0, a1)));
  const uint32_t c0 = fp8_code(x0, e), c1 = fp8_code(x1, e);
  const int64_t blk = slot / kBlock;
  const int row = (int)(slot - blk * kBlock);
  uint8_t* pool = is_v ? v_cache : k_cache;
  uint8_t* tile = pool + (blk * num_kv_heads + h) * TILE;
  if (is_v) {                                  // transposed: byte d * 16 + row
    tile[(2 * lane) * kBlock + row] = (uint8_t)c0;
    tile[(2 * lane + 1) * kBlock + row] = (uint8_t)c1;
  } else {
    *reinterpret_cast<uint16_t*>(tile + row * D + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  }
  const int64_t exps = (num_slots / kBlock) * num_kv_heads * TILE;   // exponent plane
  if (lane == 0) pool[exps + (blk * num_kv_heads + h) * kBlock + row] = (uint8_t)(e + 127);
}

pa_status check_desc(const pa_cache_desc* c, const char* who) {
  if (c == nullptr) return fail(PA_ERR_ARG, "%s: cache descriptor is NULL", who);
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return fail(PA_ERR_ARG, "%s: descriptor sizes must be > 0 (blocks %d, kv heads %d, head_dim %d)",
                who, c->num_blocks, c->num_kv_heads, c->head_dim);
  if (c->block_size != kBlock)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (device path is built for 16)", who, c->block_size);
  if (c->dtype != PA_F32 && c->dtype != PA_BF16 && c->dtype != PA_FP8)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", who, c->dtype);
  if (c->dtype == PA_FP8 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: fp8 cache with head_dim %d (built for 128)", who, c->head_dim);
  if ((c->head_dim * elem_bytes(c->dtype)) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d x elem not a multiple of 16 bytes", who, c->head_dim);
  return PA_OK;
}

pa_status launch_status(const char* who) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_write_kv(const void* k, const void* v, void* k_cache, void* v_cache,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 const pa_cache_desc* c, void* stream) {
  pa_status st = check_desc(c, "pa_write_kv");
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_ARG, "pa_write_kv: num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_ARG, "pa_write_kv: NULL device pointer");
  hipStream_t s = (hipStream_t)stream;
  const int64_t num_slots = (int64_t)c->num_blocks * kBlock;
  if (check_mode()) {
    if (stream_capturing(s)) return fail(PA_ERR_ARG, "pa_write_kv: PA_CHECK=1 cannot run on a stream being captured");
    std::vector<int64_t> h(num_tokens);
    if (hipMemcpyAsync(h.data(), slot_mapping, sizeof(int64_t) * num_tokens, hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(PA_ERR_HIP, "pa_write_kv: check-mode copy failed");
    std::vector<char> seen(num_slots, 0);
    for (int32_t t = 0; t < num_tokens; ++t) {
      if (h[t] < 0) continue;
      if (h[t] >= num_slots) return fail(PA_ERR_RANGE, "pa_write_kv: token %d slot %lld outside the pool", t, (long long)h[t]);
      if (seen[h[t]]) return fail(PA_ERR_RANGE, "pa_write_kv: token %d repeats slot %lld", t, (long long)h[t]);
      seen[h[t]] = 1;
    }
  }
  if (c->dtype == PA_FP8) {
    const int64_t rows = (int64_t)num_tokens * c->num_kv_heads;
    const int64_t nblk = (rows + 3) / 4;
    if (nblk > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: too many tokens in one call");
    const int mark = trace_begin(s);
    hipLaunchKernelGGL(write_kv_fp8_kernel, dim3((unsigned)nblk, 2), dim3(256), 0, s, (const uint32_t*)k,
                       (const uint32_t*)v, (uint8_t*)k_cache, (uint8_t*)v_cache, slot_mapping, rows,
                       c->num_kv_heads, num_slots);
    trace_end(s, mark, "write_kv");
    return launch_status("pa_write_kv");
  }
  const int row_bytes = c->head_dim * elem_bytes(c->dtype);
  const int chunks_per_row = row_bytes / 16;
  const int chunks_per_token = chunks_per_row * c->num_kv_heads;
  const int64_t total = (int64_t)num_tokens * chunks_per_token;
  const int64_t nblk = (total + 255) / 256;
  if (nblk > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: too many tokens in one call");
  const int mark = trace_begin(s);
  hipLaunchKernelGGL(write_kv_kernel, dim3((unsigned)nblk, 2), dim3(256), 0, s,
                     (const uint8_t*)k, (const uint8_t*)v, (uint8_t*)k_cache, (uint8_t*)v_cache,
                     slot_mapping, total, chunks_per_token, chunks_per_row, num_slots);
  trace_end(s, mark, "write_kv");
  return launch_status("pa_write_kv");
}

extern "C" pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                                    const pa_cache_desc* c, void* stream) {
  pa_status st = check_desc(c, "pa_copy_blocks");
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_ARG, "pa_copy_blocks: num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return fail(PA_ERR_ARG, "pa_copy_blocks: NULL device pointer");
  hipStream_t s = (hipStream_t)stream;
  if (check_mode()) {
    if (stream_capturing(s)) return fail(PA_ERR_ARG, "pa_copy_blocks: PA_CHECK=1 cannot run on a stream being captured");
    std::vector<int32_t> h(2 * (size_t)num_pairs);
    if (hipMemcpyAsync(h.data(), pairs, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(PA_ERR_HIP, "pa_copy_blocks: check-mode copy failed");
    std::vector<char> src(c->num_blocks, 0), dst(c->num_blocks, 0);
    for (int32_t p = 0; p < num_pairs; ++p) {
      int32_t a = h[2 * p], b = h[2 * p + 1];
      if (a < 0 || a >= c->num_blocks || b < 0 || b >= c->num_blocks)
        return fail(PA_ERR_RANGE, "pa_copy_blocks: pair %d (%d, %d) outside the pool", p, a, b);
      src[a] = 1;
    }
    for (int32_t p = 0; p < num_pairs; ++p) {
      int32_t b = h[2 * p + 1];
      if (dst[b] || src[b]) return fail(PA_ERR_RANGE, "pa_copy_blocks: block %d is written twice or also read", b);
      dst[b] = 1;
    }
  }
  // fp8 pools: the code plane (tiles of 16 x head_dim bytes), then the exponent plane (16 bytes per tile).
  const bool f8 = c->dtype == PA_FP8;
  const int64_t code_block = (int64_t)c->num_kv_heads * kBlock * c->head_dim * elem_bytes(c->dtype);
  const int chunks_per_block = (int)(code_block / 16);
  const int64_t plane2 = f8 ? code_block * c->num_blocks : 0;
  const int chunks2 = f8 ? c->num_kv_heads * kBlock / 16 : 0;
  const int mark = trace_begin(s);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, f8 ? 4 : 2), dim3(256), 0, s, (uint8_t*)k_cache,
                     (uint8_t*)v_cache, pairs, chunks_per_block, c->num_blocks, plane2, chunks2);
  trace_end(s, mark, "copy_blocks");
  return launch_status("pa_copy_blocks");
}
