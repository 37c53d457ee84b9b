// pa_forward: the super-batch dispatcher.
//
// "Внутреннее устройство vLLM" (artificials.ru), forward-pass and engine
// paragraphs: one step carries decode rows and prefill chunks together in a
// single unpadded batch, each row restricted to its own sequence.  Rows of
// sequences with one query token go to the split-KV decode kernel (plus the
// log-sum-exp merge when a sequence spans several partitions); sequences with
// a few query tokens (2 .. the verify plan's max_q: a speculative-decoding
// step) to the multi-token decode kernel; longer ones to the chunked-prefill
// kernel.  Grids are sized from the host scalars max_seq_len / max_query_len,
// so nothing waits on the device.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "device.h"
#include "ops.h"
#include "status.h"

namespace pa {

struct ForwardShape {
  int32_t group;
  DecodePlan plan;
  VerifyPlan vplan;
  PrefillPlan pplan;
  bool use_mfma_prefill;
  bool any_prefill;
  size_t workspace_bytes() const { return plan.workspace_bytes() + vplan.workspace_bytes() + pplan.workspace_bytes(); }
};

static pa_status shape_of(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                          int32_t max_query_len, const pa_cache_desc* c, const char* who, ForwardShape* fs) {
  pa_status st = check_desc(c, who);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || max_seq_len < 0 || max_query_len < 0)
    return fail(PA_ERR_ARG, "%s: negative size (seqs %d, tokens %d, max_seq_len %d, max_query_len %d)", who,
                num_seqs, num_tokens, max_seq_len, max_query_len);
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0)
    return fail(PA_ERR_ARG, "%s: num_q_heads %d is not a positive multiple of num_kv_heads %d", who,
                num_q_heads, c->num_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (built for 64 and 128)", who, c->head_dim);
  fs->group = num_q_heads / c->num_kv_heads;
  if (fs->group != 1 && fs->group != 2 && fs->group != 4 && fs->group != 8)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d query heads per KV head (built for 1, 2, 4, 8)", who, fs->group);
  fs->vplan = make_verify_plan(num_seqs, num_tokens, num_q_heads, c->num_kv_heads, c->head_dim, c->dtype,
                               max_seq_len, max_query_len);
  if (c->dtype == PA_FP8) {
    // Quantised cache: sequences of up to max_q query tokens go through the
    // multi-token decode kernel, longer ones through the chunked-prefill
    // kernel; both read fp8 tiles.
    fs->plan = DecodePlan{};
    if (!verify_fp8_supported(c->head_dim, fs->group))
      return fail(PA_ERR_UNSUPPORTED, "%s: fp8 cache with head_dim %d", who, c->head_dim);
    if (num_seqs > 1024)
      return fail(PA_ERR_UNSUPPORTED, "%s: fp8 cache with %d sequences (built for up to 1024)", who, num_seqs);
    if (!fs->vplan.on && num_seqs > 0 && num_tokens > 0 && max_seq_len > 0 && max_query_len > 0)
      return fail(PA_ERR_UNSUPPORTED, "%s: fp8 cache with %d tokens in one call", who, num_tokens);
    fs->any_prefill = fs->use_mfma_prefill = fs->vplan.on && max_query_len > fs->vplan.max_q;
    fs->pplan = make_prefill_plan(num_tokens, num_q_heads, c->head_dim, max_seq_len, max_query_len,
                                  fs->use_mfma_prefill);
    return PA_OK;
  }
  // When the multi-token decode launch also takes the single-token
  // sequences, no single-token decode runs (and needs no workspace).
  if (fs->vplan.on && fs->vplan.min_q <= 1)
    fs->plan = DecodePlan{};
  else
    fs->plan = make_decode_plan(num_seqs, num_q_heads, c->num_kv_heads, c->head_dim, c->dtype, max_seq_len);
  fs->any_prefill = max_query_len > 1 && !(fs->vplan.on && max_query_len <= fs->vplan.max_q);
  fs->use_mfma_prefill = fs->any_prefill && prefill_mfma_supported(c->dtype, c->head_dim, fs->group);
  fs->pplan = make_prefill_plan(num_tokens, num_q_heads, c->head_dim, max_seq_len, max_query_len,
                                fs->use_mfma_prefill);
  return PA_OK;
}

// Check mode: copy the device metadata back and validate every precondition.
static pa_status validate_metadata(const int32_t* block_tables, int32_t stride, const int32_t* seq_lens,
                                   const int32_t* qsl, const int32_t* cached_lens, int32_t num_seqs,
                                   int32_t num_tokens, int32_t max_seq_len, int32_t max_query_len,
                                   int32_t num_blocks, hipStream_t s) {
  std::vector<int32_t> L(num_seqs), C(num_seqs), Q(num_seqs + 1), BT((size_t)num_seqs * stride);
  bool ok = hipMemcpyAsync(L.data(), seq_lens, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(C.data(), cached_lens, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(Q.data(), qsl, sizeof(int32_t) * (num_seqs + 1), hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(BT.data(), block_tables, sizeof(int32_t) * BT.size(), hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipStreamSynchronize(s) == hipSuccess;
  if (!ok) return fail(PA_ERR_HIP, "pa_forward: check-mode copy failed");
  if (Q[0] != 0 || Q[num_seqs] != num_tokens)
    return fail(PA_ERR_RANGE, "pa_forward: query_start_loc[0]=%d, [num_seqs]=%d, num_tokens=%d", Q[0], Q[num_seqs],
                num_tokens);
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t n = Q[i + 1] - Q[i];
    if (n < 0) return fail(PA_ERR_RANGE, "pa_forward: query_start_loc decreases at %d", i);
    if (n > max_query_len) return fail(PA_ERR_RANGE, "pa_forward: sequence %d has %d query tokens > max_query_len %d", i, n, max_query_len);
    if (L[i] != C[i] + n) return fail(PA_ERR_RANGE, "pa_forward: sequence %d: seq_len %d != cached %d + new %d", i, L[i], C[i], n);
    if (C[i] < 0) return fail(PA_ERR_RANGE, "pa_forward: sequence %d: cached_len %d < 0", i, C[i]);
    if (L[i] > max_seq_len) return fail(PA_ERR_RANGE, "pa_forward: sequence %d: seq_len %d > max_seq_len %d", i, L[i], max_seq_len);
    const int64_t nb = ((int64_t)L[i] + kBlock - 1) / kBlock;
    if (nb > stride) return fail(PA_ERR_RANGE, "pa_forward: sequence %d needs %lld blocks > table stride %d", i, (long long)nb, stride);
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t b = BT[(size_t)i * stride + j];
      if (b < 0 || b >= num_blocks) return fail(PA_ERR_RANGE, "pa_forward: sequence %d block %lld = %d outside the pool", i, (long long)j, b);
    }
  }
  return PA_OK;
}

// Check mode for the fused write: every single-token sequence's new token is
// stored at its position L - 1 as its block table gives it.
static pa_status validate_fused_slots(const int32_t* block_tables, int32_t stride, const int32_t* seq_lens,
                                      const int32_t* qsl, const int64_t* slots, int32_t num_seqs,
                                      int32_t num_tokens, hipStream_t s) {
  std::vector<int32_t> L(num_seqs), Q(num_seqs + 1), BT((size_t)num_seqs * stride);
  std::vector<int64_t> SL(num_tokens);
  bool ok = hipMemcpyAsync(L.data(), seq_lens, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(Q.data(), qsl, sizeof(int32_t) * (num_seqs + 1), hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(BT.data(), block_tables, sizeof(int32_t) * BT.size(), hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(SL.data(), slots, sizeof(int64_t) * num_tokens, hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipStreamSynchronize(s) == hipSuccess;
  if (!ok) return fail(PA_ERR_HIP, "pa_write_kv_forward: check-mode copy failed");
  std::vector<int64_t> seen;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (Q[i] < 0 || Q[i + 1] - Q[i] != 1 || Q[i] >= num_tokens || L[i] < 1 || (L[i] - 1) / kBlock >= stride)
      continue;                                       // the metadata check reports these
    const int64_t p = (int64_t)L[i] - 1;
    const int64_t want = (int64_t)BT[(size_t)i * stride + p / kBlock] * kBlock + p % kBlock;
    if (SL[Q[i]] != want)
      return fail(PA_ERR_RANGE, "pa_write_kv_forward: sequence %d's new token has slot %lld, its position %lld is "
                  "slot %lld", i, (long long)SL[Q[i]], (long long)p, (long long)want);
    seen.push_back(want);
  }
  std::sort(seen.begin(), seen.end());
  for (size_t j = 1; j < seen.size(); ++j)
    if (seen[j] == seen[j - 1])
      return fail(PA_ERR_RANGE, "pa_write_kv_forward: two sequences write slot %lld", (long long)seen[j]);
  return PA_OK;
}

// Check mode for pa_forward_shared: sequence i's first shared_blocks[i] table
// entries equal sequence i - 1's, within both sequences' blocks.
static pa_status validate_shared(const int32_t* block_tables, int32_t stride, const int32_t* seq_lens,
                                 const int32_t* shared_blocks, int32_t num_seqs, hipStream_t s) {
  std::vector<int32_t> L(num_seqs), SB(num_seqs), BT((size_t)num_seqs * stride);
  bool ok = hipMemcpyAsync(L.data(), seq_lens, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(SB.data(), shared_blocks, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(BT.data(), block_tables, sizeof(int32_t) * BT.size(), hipMemcpyDeviceToHost, s) == hipSuccess;
  ok = ok && hipStreamSynchronize(s) == hipSuccess;
  if (!ok) return fail(PA_ERR_HIP, "pa_forward_shared: check-mode copy failed");
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (SB[i] < 0) return fail(PA_ERR_RANGE, "pa_forward_shared: shared_blocks[%d] = %d < 0", i, SB[i]);
    if (i == 0 || SB[i] == 0) continue;
    const int64_t nb = std::min(((int64_t)L[i] + kBlock - 1) / kBlock, ((int64_t)L[i - 1] + kBlock - 1) / kBlock);
    if (SB[i] > nb)
      return fail(PA_ERR_RANGE, "pa_forward_shared: shared_blocks[%d] = %d exceeds the sequences' blocks (%lld)", i,
                  SB[i], (long long)nb);
    for (int32_t b = 0; b < SB[i]; ++b)
      if (BT[(size_t)i * stride + b] != BT[(size_t)(i - 1) * stride + b])
        return fail(PA_ERR_RANGE, "pa_forward_shared: sequence %d block %d differs from sequence %d's", i, b, i - 1);
  }
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_forward_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                            int32_t max_seq_len, int32_t max_query_len, const pa_cache_desc* c) {
  ForwardShape fs;
  if (shape_of(num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, "pa_forward_workspace_size",
               &fs) != PA_OK)
    return 0;
  return fs.workspace_bytes();
}

namespace pa {
namespace {

// Scratch of pa_forward_noalloc: one array per GPU, held for the life of the
// process.  Host code never uses the array's name as an address: on each
// device it takes the array's device address once, with that device current,
// and passes that address to the kernels.
constexpr size_t kNoallocScratchBytes = PA_FORWARD_NOALLOC_MAX_SCRATCH;
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `s`.
pa_status scratch_for_stream(hipStream_t s, void** out) {
  hipDevice_t dev = 0;
  if (s == nullptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return fail(PA_ERR_HIP, "pa_forward_noalloc: hipGetDevice failed");
    dev = cur;
  } else if (hipStreamGetDevice(s, &dev) != hipSuccess) {
    return fail(PA_ERR_HIP, "pa_forward_noalloc: hipStreamGetDevice failed");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "pa_forward_noalloc: device %d", (int)dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return fail(PA_ERR_HIP, "pa_forward_noalloc: hipGetDevice failed");
    if (prev != dev && hipSetDevice(dev) != hipSuccess)
      return fail(PA_ERR_HIP, "pa_forward_noalloc: hipSetDevice(%d) failed", (int)dev);
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != dev) (void)hipSetDevice(prev);
    if (e != hipSuccess || p == nullptr)
      return fail(PA_ERR_HIP, "pa_forward_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

// The body of pa_forward and pa_forward_noalloc: `workspace` holds at least
// fs.workspace_bytes() (checked by the callers).
static pa_status forward_impl(const ForwardShape& fs, void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* seq_lens, const int32_t* query_start_loc, const int32_t* cached_lens,
                              int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                              int32_t max_query_len, const pa_cache_desc* c, float scale, int32_t causal,
                              void* workspace, hipStream_t s, const void* k_new = nullptr,
                              const void* v_new = nullptr) {
  pa_status st;
  const size_t ws_need = fs.workspace_bytes();
  if (check_mode()) {
    if (stream_capturing(s)) return fail(PA_ERR_ARG, "pa_forward: PA_CHECK=1 cannot run on a stream being captured");
    st = validate_metadata(block_tables, block_table_stride, seq_lens, query_start_loc, cached_lens, num_seqs,
                           num_tokens, max_seq_len, max_query_len, c->num_blocks, s);
    if (st != PA_OK) return st;
  }

  AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.bt_stride = block_table_stride;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.cached_lens = cached_lens;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = c->num_kv_heads;
  a.num_blocks = c->num_blocks;
  a.head_dim = c->head_dim;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal;
  a.prefill_min_q = fs.vplan.on ? fs.vplan.max_q + 1 : 2;
  a.k_new = k_new;
  a.v_new = v_new;

  int32_t* p_info = nullptr;
  float* p_acc = nullptr;
  float* p_ml = nullptr;
  int32_t* v_info = nullptr;
  uint16_t* v_acc = nullptr;
  float* v_ml = nullptr;
  uint16_t* pre_o = nullptr;
  float* pre_ml = nullptr;
  if (ws_need > 0) {
    uint8_t* base = (uint8_t*)workspace;
    p_info = (int32_t*)base;
    p_acc = (float*)(base + fs.plan.info_bytes);
    p_ml = (float*)(base + fs.plan.info_bytes + fs.plan.acc_bytes);
    uint8_t* vbase = base + fs.plan.workspace_bytes();
    v_info = (int32_t*)vbase;
    v_acc = (uint16_t*)(vbase + fs.vplan.info_bytes);
    v_ml = (float*)(vbase + fs.vplan.info_bytes + fs.vplan.acc_bytes);
    uint8_t* pbase = vbase + fs.vplan.workspace_bytes();
    pre_o = (uint16_t*)pbase;
    pre_ml = (float*)(pbase + fs.pplan.o_bytes);
  }
  if (fs.use_mfma_prefill) {
    st = launch_prefill(a, max_query_len, fs.pplan, pre_o, pre_ml, c->dtype == PA_FP8, s);
    if (st != PA_OK) return st;
  }
  if (fs.vplan.on) {
    st = launch_decode_verify(a, fs.vplan, v_acc, v_ml, v_info, s);
    if (st != PA_OK) return st;
  }
  if (fs.vplan.on && fs.vplan.min_q <= 1) return PA_OK;   // single-token sequences taken by the launch above
  if (fs.plan.balanced) return launch_decode_balanced(a, fs.plan, p_acc, p_ml, p_info, s);
  if (fs.plan.mfma)
    st = launch_decode_mfma(a, fs.plan, p_acc, p_ml, s);
  else
    st = launch_decode(a, c->dtype, fs.plan, p_acc, p_ml, fs.any_prefill && !fs.use_mfma_prefill, s);
  if (st != PA_OK) return st;
  if (fs.plan.max_parts > 1) st = launch_merge(a, c->dtype, fs.plan, p_acc, p_ml, s);
  return st;
}

// Host-argument checks shared by both entry points.
static pa_status check_forward_args(void* out, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, int32_t block_table_stride,
                                    const int32_t* seq_lens, const int32_t* query_start_loc,
                                    const int32_t* cached_lens, float scale, int32_t causal, const char* who) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start_loc || !cached_lens)
    return fail(PA_ERR_ARG, "%s: NULL device pointer", who);
  if (block_table_stride <= 0) return fail(PA_ERR_ARG, "%s: block_table_stride %d", who, block_table_stride);
  if (!std::isfinite(scale)) return fail(PA_ERR_ARG, "%s: scale is not finite", who);
  if (causal != 0 && causal != 1) return fail(PA_ERR_ARG, "%s: causal must be 0 or 1", who);
  return PA_OK;
}

}  // namespace pa

extern "C" pa_status pa_forward(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int32_t block_table_stride, const int32_t* seq_lens,
                                const int32_t* query_start_loc, const int32_t* cached_lens, int32_t num_seqs,
                                int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                                int32_t max_query_len, const pa_cache_desc* c, float scale, int32_t causal,
                                void* workspace, size_t workspace_bytes, void* stream) {
  ForwardShape fs;
  pa_status st = shape_of(num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, "pa_forward", &fs);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || num_tokens == 0 || max_seq_len == 0 || max_query_len == 0) return PA_OK;
  st = check_forward_args(out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                          cached_lens, scale, causal, "pa_forward");
  if (st != PA_OK) return st;
  const size_t ws_need = fs.workspace_bytes();
  if (ws_need > 0 && (workspace == nullptr || workspace_bytes < ws_need))
    return fail(PA_ERR_ARG, "pa_forward: workspace of %zu bytes needed, %zu given", ws_need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  return forward_impl(fs, out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                      cached_lens, num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, scale, causal,
                      workspace, (hipStream_t)stream);
}

extern "C" pa_status pa_forward_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t block_table_stride,
                                        const int32_t* seq_lens, const int32_t* query_start_loc,
                                        const int32_t* cached_lens, int32_t num_seqs, int32_t num_tokens,
                                        int32_t num_q_heads, int32_t max_seq_len, int32_t max_query_len,
                                        const pa_cache_desc* c, float scale, int32_t causal, void* stream) {
  ForwardShape fs;
  pa_status st =
      shape_of(num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, "pa_forward_noalloc", &fs);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || num_tokens == 0 || max_seq_len == 0 || max_query_len == 0) return PA_OK;
  st = check_forward_args(out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                          cached_lens, scale, causal, "pa_forward_noalloc");
  if (st != PA_OK) return st;
  const size_t ws_need = fs.workspace_bytes();
  if (ws_need > kNoallocScratchBytes)
    return fail(PA_ERR_UNSUPPORTED, "pa_forward_noalloc: this batch needs %zu bytes of scratch, more than the %zu "
                "bytes the library holds per GPU (use pa_forward with a workspace)", ws_need, kNoallocScratchBytes);
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  if (ws_need > 0) {
    st = scratch_for_stream(s, &ws);
    if (st != PA_OK) return st;
  }
  return forward_impl(fs, out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                      cached_lens, num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, scale, causal,
                      ws, s);
}

static SharedPlan shared_plan_of(int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len, int32_t max_query_len,
                                 const pa_cache_desc* c) {
  return make_shared_plan(num_seqs, num_q_heads, c->num_kv_heads, c->head_dim, c->dtype, max_seq_len, max_query_len);
}

extern "C" size_t pa_forward_shared_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                                   int32_t max_seq_len, int32_t max_query_len,
                                                   const pa_cache_desc* c) {
  ForwardShape fs;
  if (shape_of(num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, "pa_forward_shared_workspace_size",
               &fs) != PA_OK)
    return 0;
  const SharedPlan sp = shared_plan_of(num_seqs, num_q_heads, max_seq_len, max_query_len, c);
  return sp.on ? sp.workspace_bytes() : fs.workspace_bytes();
}

// pa_forward_shared, optionally with the fused cache write (k_new / v_new set;
// only when the shared-prefix decode takes the batch).
static pa_status forward_shared_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t block_table_stride,
                                     const int32_t* seq_lens, const int32_t* query_start_loc,
                                     const int32_t* cached_lens, const int32_t* shared_blocks, int32_t num_seqs,
                                     int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                                     int32_t max_query_len, const pa_cache_desc* c, float scale, int32_t causal,
                                     void* workspace, size_t workspace_bytes, hipStream_t s, const char* who,
                                     const void* k_new, const void* v_new, const int64_t* slots) {
  ForwardShape fs;
  pa_status st = shape_of(num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, who, &fs);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || num_tokens == 0 || max_seq_len == 0 || max_query_len == 0) return PA_OK;
  st = check_forward_args(out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                          cached_lens, scale, causal, who);
  if (st != PA_OK) return st;
  if (shared_blocks == nullptr) return fail(PA_ERR_ARG, "%s: shared_blocks is NULL", who);
  const SharedPlan sp = shared_plan_of(num_seqs, num_q_heads, max_seq_len, max_query_len, c);
  const size_t ws_need = sp.on ? sp.workspace_bytes() : fs.workspace_bytes();
  if (ws_need > 0 && (workspace == nullptr || workspace_bytes < ws_need))
    return fail(PA_ERR_ARG, "%s: workspace of %zu bytes needed, %zu given", who, ws_need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!sp.on)   // not a batch of single-token bf16 head_dim-128 sequences: pa_forward's paths
    return forward_impl(fs, out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                        cached_lens, num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, scale,
                        causal, workspace, s);
  if (check_mode()) {
    if (stream_capturing(s)) return fail(PA_ERR_ARG, "%s: PA_CHECK=1 cannot run on a stream being captured", who);
    st = validate_metadata(block_tables, block_table_stride, seq_lens, query_start_loc, cached_lens, num_seqs,
                           num_tokens, max_seq_len, max_query_len, c->num_blocks, s);
    if (st != PA_OK) return st;
    st = validate_shared(block_tables, block_table_stride, seq_lens, shared_blocks, num_seqs, s);
    if (st != PA_OK) return st;
    if (k_new != nullptr) {
      st = validate_fused_slots(block_tables, block_table_stride, seq_lens, query_start_loc, slots, num_seqs,
                                num_tokens, s);
      if (st != PA_OK) return st;
    }
  }
  AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.bt_stride = block_table_stride;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.cached_lens = cached_lens;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = c->num_kv_heads;
  a.num_blocks = c->num_blocks;
  a.head_dim = c->head_dim;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal;
  a.prefill_min_q = 2;
  a.k_new = k_new;
  a.v_new = v_new;
  return launch_decode_shared(a, sp, shared_blocks, workspace, s);
}

extern "C" pa_status pa_forward_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int32_t block_table_stride,
                                       const int32_t* seq_lens, const int32_t* query_start_loc,
                                       const int32_t* cached_lens, const int32_t* shared_blocks, int32_t num_seqs,
                                       int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                                       int32_t max_query_len, const pa_cache_desc* c, float scale, int32_t causal,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  return forward_shared_impl(out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                             cached_lens, shared_blocks, num_seqs, num_tokens, num_q_heads, max_seq_len,
                             max_query_len, c, scale, causal, workspace, workspace_bytes, (hipStream_t)stream,
                             "pa_forward_shared", nullptr, nullptr, nullptr);
}

extern "C" pa_status pa_write_kv_forward_shared(const void* k, const void* v, const int64_t* slot_mapping,
                                                void* out, const void* q, void* k_cache, void* v_cache,
                                                const int32_t* block_tables, int32_t block_table_stride,
                                                const int32_t* seq_lens, const int32_t* query_start_loc,
                                                const int32_t* cached_lens, const int32_t* shared_blocks,
                                                int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                                int32_t max_seq_len, int32_t max_query_len, const pa_cache_desc* c,
                                                float scale, int32_t causal, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  ForwardShape fs;
  pa_status st = shape_of(num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c,
                          "pa_write_kv_forward_shared", &fs);
  if (st != PA_OK) return st;
  const SharedPlan sp = shared_plan_of(num_seqs, num_q_heads, max_seq_len, max_query_len, c);
  hipStream_t s = (hipStream_t)stream;
  if (!sp.on || num_tokens == 0) {   // the shared-prefix decode does not take the batch: the two calls
    st = pa_write_kv(k, v, k_cache, v_cache, slot_mapping, num_tokens, c, stream);
    if (st != PA_OK) return st;
    return pa_forward_shared(out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                             cached_lens, shared_blocks, num_seqs, num_tokens, num_q_heads, max_seq_len,
                             max_query_len, c, scale, causal, workspace, workspace_bytes, stream);
  }
  if (!k || !v || !slot_mapping) return fail(PA_ERR_ARG, "pa_write_kv_forward_shared: NULL device pointer");
  return forward_shared_impl(out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                             cached_lens, shared_blocks, num_seqs, num_tokens, num_q_heads, max_seq_len,
                             max_query_len, c, scale, causal, workspace, workspace_bytes, s,
                             "pa_write_kv_forward_shared", k, v, slot_mapping);
}

extern "C" pa_status pa_write_kv_forward(const void* k, const void* v, const int64_t* slot_mapping, void* out,
                                         const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
                                         int32_t block_table_stride, const int32_t* seq_lens,
                                         const int32_t* query_start_loc, const int32_t* cached_lens,
                                         int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                         int32_t max_seq_len, int32_t max_query_len, const pa_cache_desc* c,
                                         float scale, int32_t causal, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  ForwardShape fs;
  pa_status st =
      shape_of(num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, "pa_write_kv_forward", &fs);
  if (st != PA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // A batch of single-token sequences whose decode runs the balanced matrix-core
  // kernel or the vector kernel takes the fused write; anything else writes first.
  const bool fuse = num_seqs > 0 && num_tokens > 0 && max_seq_len > 0 && max_query_len == 1 &&
                    c->dtype != PA_FP8 && !fs.vplan.on && (fs.plan.balanced || !fs.plan.mfma);
  if (!fuse) {
    st = pa_write_kv(k, v, k_cache, v_cache, slot_mapping, num_tokens, c, stream);
    if (st != PA_OK) return st;
    return pa_forward(out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                      cached_lens, num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, scale, causal,
                      workspace, workspace_bytes, stream);
  }
  st = check_forward_args(out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                          cached_lens, scale, causal, "pa_write_kv_forward");
  if (st != PA_OK) return st;
  if (!k || !v || !slot_mapping) return fail(PA_ERR_ARG, "pa_write_kv_forward: NULL device pointer");
  if ((c->head_dim * elem_bytes(c->dtype)) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "pa_write_kv_forward: head_dim %d", c->head_dim);
  const size_t ws_need = fs.workspace_bytes();
  if (ws_need > 0 && (workspace == nullptr || workspace_bytes < ws_need))
    return fail(PA_ERR_ARG, "pa_write_kv_forward: workspace of %zu bytes needed, %zu given", ws_need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (check_mode()) {
    if (stream_capturing(s)) return fail(PA_ERR_ARG, "pa_write_kv_forward: PA_CHECK=1 cannot run on a stream being captured");
    st = validate_fused_slots(block_tables, block_table_stride, seq_lens, query_start_loc, slot_mapping, num_seqs,
                              num_tokens, s);
    if (st != PA_OK) return st;
  }
  return forward_impl(fs, out, q, k_cache, v_cache, block_tables, block_table_stride, seq_lens, query_start_loc,
                      cached_lens, num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, c, scale, causal,
                      workspace, s, k, v);
}
