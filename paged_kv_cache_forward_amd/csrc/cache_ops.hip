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

// grid.x = pair, grid.y = 0 for K, 1 for V; each block copies one block tile.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int chunks_per_block, int num_blocks) {
  const int src = pairs[2 * blockIdx.x];
  const int dst = pairs[2 * blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  uint8_t* cache = blockIdx.y == 0 ? k_cache : v_cache;
  const uint8_t* s = cache + (int64_t)src * chunks_per_block * 16;
  uint8_t* d = cache + (int64_t)dst * chunks_per_block * 16;
  for (int c = threadIdx.x; c < chunks_per_block; c += blockDim.x) st16(d + c * 16, ld16(s + c * 16));
}

pa_status check_desc(const pa_cache_desc* c, const char* who) {
  if (c == nullptr) return fail(PA_ERR_ARG, "%s: cache descriptor is NULL", who);
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return fail(PA_ERR_ARG, "%s: descriptor sizes must be > 0 (blocks %d, kv heads %d, head_dim %d)",
                who, c->num_blocks, c->num_kv_heads, c->head_dim);
  if (c->block_size != kBlock)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (device path is built for 16)", who, c->block_size);
  if (c->dtype != PA_F32 && c->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", who, c->dtype);
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
  const int chunks_per_block = c->num_kv_heads * kBlock * c->head_dim * elem_bytes(c->dtype) / 16;
  const int mark = trace_begin(s);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, s, (uint8_t*)k_cache,
                     (uint8_t*)v_cache, pairs, chunks_per_block, c->num_blocks);
  trace_end(s, mark, "copy_blocks");
  return launch_status("pa_copy_blocks");
}
