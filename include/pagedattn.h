/*
 * libpagedattn — paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; no C++ or framework types cross it.
 *
 * Pages whose description of the method these calls follow (cited by title
 * and section):
 *   [SLAVA] "Was ändert PagedAttention an der KV-Speicherzuweisung für LLMs?"
 *           (slavadubrov.com): lead paragraph; section "Ungenutzten Platz in
 *           Blöcken berechnen"; section "Gemeinsame Nutzung erfordert mehr als
 *           Speicherzuweisung".
 *   [AIU]   "PagedAttention et vLLM" (aiunderstanding.org): section "Plongée
 *           profonde"; "Questions fréquemment posées".
 *   [ART]   "Внутреннее устройство vLLM: как работает высокопроизводительный
 *           инференс LLM" (artificials.ru): paragraphs on paged attention,
 *           chunked prefill and the forward pass.
 *   [HADA]  "vLLM PagedAttention: eine Revolution für den Durchsatz bei der
 *           LLM-Inferenz" (de.news.hada.io): bullet "Chunked Prefill".
 *
 * Conventions for every call:
 *   - Every call returns pa_status; no exception or abort crosses the ABI.
 *     After a non-OK status, pa_last_error() gives a message (per thread).
 *   - Device calls take device pointers owned by the caller and a HIP stream
 *     (hipStream_t passed as void*, NULL = the null stream).  They enqueue
 *     work and return without synchronising (except in check mode, below).
 *     The library never allocates device memory: split-KV scratch is the
 *     caller's `workspace`.
 *   - Host arguments (sizes, descriptors, null pointers, supported shapes)
 *     are checked before anything is enqueued: PA_ERR_ARG / PA_ERR_UNSUPPORTED.
 *   - Device-resident metadata (slots, block tables, lengths) is not read by
 *     the host on the fast path.  Out-of-range block ids and slots are made
 *     harmless on the device (a slot outside the pool is skipped; a block id
 *     outside the pool is clamped into it), so a bad table gives wrong values,
 *     never a fault.  With the environment variable PA_CHECK=1 the host copies
 *     the metadata back, synchronises the stream and validates every
 *     precondition first, returning PA_ERR_RANGE on a violation.
 *   - HIP launch failures return PA_ERR_HIP with the runtime's message.
 *
 * Cache layout ([SLAVA] section "Ungenutzten Platz in Blöcken berechnen":
 * block size and layout are the runtime's choice; [ART] paged-attention
 * paragraph: blocks of 16 tokens): separate K and V pools, each
 *     [num_blocks][num_kv_heads][block_size = 16][head_dim]   row-major,
 * so one (block, KV head) tile of 16 tokens is contiguous.  Slot s of the
 * pool is row s % 16 of block s / 16.
 *
 * Quantised pools (dtype PA_FP8, head_dim 128).  [SLAVA] section "Gemeinsame
 * Nutzung erfordert mehr als Speicherzuweisung" names cache quantisation as
 * the remedy when the K/V data itself does not fit; [AIU] "L'avenir de
 * PagedAttention et vLLM" expects paged K/V combined with quantisation.  Each
 * (token, KV head) row of head_dim values is stored as E4M3 codes (the FN
 * encoding of the OCP 8-bit floating point specification) with one
 * power-of-two scale 2^e, e = the smallest integer in [-126, 127] with
 * max|x| <= 448 * 2^e (0 for a zero row), kept as an E8M0 byte e + 127; the
 * codes are x * 2^-e rounded to nearest, ties to even mantissa.  A pool is
 * num_blocks * num_kv_heads * (16 * head_dim + 16) bytes in two planes:
 *     codes      [num_blocks][num_kv_heads][16 * head_dim]   (tiles 128-byte aligned)
 *     exponents  [num_blocks][num_kv_heads][16]              (one byte per row)
 * K codes are row-major in their tile (byte row * head_dim + d); V codes are
 * stored transposed (byte d * 16 + row), the layout the P.V product reads.
 * The value a cached element stands for is decode(code) * 2^e, exactly.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_ARG = 1,          /* bad host argument (null pointer, size, descriptor) */
  PA_ERR_UNSUPPORTED = 2,  /* valid but not built: dtype / head_dim / group size / block size */
  PA_ERR_OOM = 3,          /* allocator: not enough free blocks (state unchanged) */
  PA_ERR_RANGE = 4,        /* check mode: device metadata violates a precondition */
  PA_ERR_HIP = 5           /* HIP runtime error */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8 = 2 } pa_dtype;

/* Shape of one K (or V) pool.  block_size must be 16 for device calls. */
typedef struct {
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t dtype;           /* pa_dtype: element type of pools, k/v, q and out;
                              PA_FP8: quantised pools, k/v/q/out bf16 */
} pa_cache_desc;

/* Library version string (static storage). */
const char* pa_version(void);

/* Message for the last non-OK status returned on this thread (static storage). */
const char* pa_last_error(void);

/* ------------------------------------------------------------------------ */
/* Device operations                                                         */
/* ------------------------------------------------------------------------ */

/*
 * pa_write_kv — store new tokens' keys and values into their cache slots.
 *
 * [SLAVA] lead paragraph: a block table maps a request's logical positions to
 * physical blocks; the per-token slot is that mapping, flattened.  The new
 * tokens are written before attention reads them.
 *
 *   k, v          device, [num_tokens][num_kv_heads][head_dim], contiguous, c->dtype
 *                 (bf16 for a PA_FP8 cache, which this call quantises row by row)
 *   k_cache,
 *   v_cache       device pools (layout above), modified in place
 *   slot_mapping  device int64 [num_tokens]; slot < 0 means "skip this token"
 *                 (padding); a slot >= num_blocks*16 is also skipped.
 *                 Precondition: no two tokens name the same slot.
 *   num_tokens    >= 0 (0 is a no-op)
 *
 * A bit copy: the stored bytes equal the input bytes exactly (PA_FP8: the
 * quantisation above, exactly; a row's codes and scale are written together).
 * Errors: PA_ERR_ARG, PA_ERR_UNSUPPORTED (block_size != 16 or head_dim*elem
 * not a multiple of 16 bytes), PA_ERR_RANGE (check mode: duplicate or
 * out-of-pool slot), PA_ERR_HIP.
 */
pa_status pa_write_kv(const void* k, const void* v, void* k_cache, void* v_cache,
                      const int64_t* slot_mapping, int32_t num_tokens,
                      const pa_cache_desc* c, void* stream);

/*
 * pa_copy_blocks — whole-block copies for copy-on-write.
 *
 * [SLAVA] section "Gemeinsame Nutzung erfordert mehr als Speicherzuweisung"
 * and [AIU] FAQ (sharing question): a block several requests share is copied
 * only when one of them diverges, so the shared original stays intact.
 *
 *   pairs      device int32 [num_pairs][2] = (src block, dst block); each
 *              copy moves the block's K and V, all KV heads, all 16 rows.
 *              Precondition: no dst appears twice or as any pair's src.
 *              Pairs naming a block outside [0, num_blocks) are skipped.
 *   num_pairs  >= 0 (0 is a no-op)
 *
 * Enqueue it before the pa_write_kv that writes into the copies (same stream).
 * Errors: PA_ERR_ARG, PA_ERR_RANGE (check mode), PA_ERR_HIP.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                         int32_t num_pairs, const pa_cache_desc* c, void* stream);

/*
 * pa_forward_workspace_size — bytes of device scratch pa_forward needs for the
 * same host arguments (0 when the call needs none).  Depends only on its
 * arguments and on the tuning variables that choose the route or the split
 * (see pa_forward): PA_DECODE, PA_DECODE_TOTAL_WAVES, PA_SPLIT, PA_VERIFY,
 * PA_VERIFY_TOTAL_WAVES and PA_PREFILL_SPLIT.
 */
size_t pa_forward_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                 int32_t max_seq_len, int32_t max_query_len,
                                 const pa_cache_desc* c);

/*
 * pa_forward — attention for a flattened variable-length super-batch.
 *
 * [ART] forward-pass paragraph: every sequence of the step sits in one batch
 * with no padding; masks and exact positions keep each to its own tokens.
 * [AIU] "Plongée profonde": each query attends to its sequence's whole cached
 * context, read through the block table from blocks anywhere in memory.
 * [HADA] "Chunked Prefill" / [ART] chunked-prefill paragraph: a prompt's
 * prefill may arrive in chunks on top of tokens already cached.
 *
 * For sequence i (rows query_start_loc[i] .. query_start_loc[i+1]-1, n_i of
 * them), query row j (absolute position cached_lens[i] + j) and query head h,
 * with KV head g = h / (num_q_heads / num_kv_heads):
 *   visible keys t:  t <= cached_lens[i] + j   if causal, else t < seq_lens[i]
 *   out = sum_t softmax_t(scale * <q, K_t>) V_t
 * where K_t / V_t is token t of sequence i, in block block_tables[i][t / 16]
 * at row t % 16.  Accumulation is fp32; out is rounded once (nearest-even for
 * bf16).  Sequences with n_i = 1 run the split-KV decode path (their keys cut
 * into parts whose partial results are merged by log-sum-exp); with bf16 and
 * head_dim 128, sequences with a few query tokens (2 .. 16, 2 .. 8 when eight
 * query heads share a KV head, bounded also by max_query_len: a speculative-
 * decoding step, "vLLM PagedAttention: eine Revolution ..." (de.news.hada.io),
 * bullet "Guided and Speculative Decoding") run a multi-token decode path of
 * the same split-KV kind; longer ones run the chunked-prefill path (bf16:
 * matrix cores; long key ranges likewise cut into pieces and merged).  On a
 * PA_FP8 cache (head_dim 128) single-token sequences take the multi-token
 * path too, and every path reads the exact dequantised values.
 *
 *   out, q           device, [num_tokens][num_q_heads][head_dim], c->dtype
 *   k_cache, v_cache device pools (read only)
 *   block_tables     device int32 [num_seqs][block_table_stride]
 *   seq_lens         device int32 [num_seqs]   L_i: tokens in cache after this step's write
 *   query_start_loc  device int32 [num_seqs+1] non-decreasing, [0] = 0, [num_seqs] = num_tokens
 *   cached_lens      device int32 [num_seqs]   c_i; precondition L_i = c_i + n_i
 *   max_seq_len      host, >= every L_i       (sizes the grid without a device->host sync)
 *   max_query_len    host, >= every n_i
 *   scale            softmax scale (typically 1/sqrt(head_dim))
 *   causal           0 or 1
 *   workspace        device scratch of >= pa_forward_workspace_size(...) bytes
 *                    (may be NULL when that size is 0); contents need no init
 *
 * Supported: dtype f32 or bf16; head_dim 64 or 128; num_q_heads/num_kv_heads
 * in {1, 2, 4, 8}; block_size 16.  bf16 with head_dim 128 runs the scores of
 * the decode rows on the matrix cores; other combinations use the vector path.
 * Decode on the matrix cores, up to 1024 sequences: a fixed grid of waves
 * cuts each KV head's concatenated decode tiles into equal ranges (balanced);
 * otherwise per-sequence partitions.  Results are deterministic: the same
 * inputs give the same bits.  With the balanced decode, where a sequence is
 * cut depends on the other sequences of the batch, so a reordered batch may
 * differ in the last bits (within the stated tolerance).
 * Tuning knobs (environment, read on every call; results stay within the
 * stated tolerance under every setting):
 *   PA_DECODE=partition     per-sequence partitions instead of the balanced decode
 *   PA_DECODE=valu          force the vector decode kernel (partitioned)
 *   PA_DECODE_TOTAL_WAVES=<1..65536>  balanced decode: waves in all (default
 *            1024, one per SIMD), divided evenly among the KV heads
 *   PA_DECODE_DEPTH=2|3|4   balanced decode: K/V tiles in flight per wave (default 2)
 *   PA_SPLIT=auto (default) | off | <tokens>   partitioned decode: partition
 *            size (a multiple of 16, <= 8192); auto aims at ~4096 (sequence,
 *            KV head, partition) work-groups with partitions of 128..2048 tokens
 *   PA_DECODE_WAVES=1|2|4   partitioned decode: waves per work-group
 *   PA_VERIFY=prefill       send the multi-token sequences to the chunked-prefill path
 *   PA_VERIFY=all           send single-token sequences through the multi-token
 *            decode path too (one launch for both kinds)
 *   PA_VERIFY_TOTAL_WAVES=<1..65536>  multi-token decode: waves in all (default 1024)
 *   PA_VERIFY_FIRST_WEIGHT=<500..2000>  multi-token decode with more waves
 *            than SIMDs (up to two per SIMD): tiles taken by the waves
 *            dispatched first on each SIMD, per 1000 taken by the others
 *            (default 1350; 1000 = equal ranges)
 *   PA_VERIFY_DEPTH=2..5    multi-token decode: K/V tiles in flight per wave
 *            (bf16: default 3, or 2 when four work-groups would not fit a
 *            CU's LDS; 4 and 5 both run 4.  fp8 cache: default 3; 5 runs 5,
 *            any other value 3)
 *   PA_PREFILL_ROWS=32 (default) | 64   chunked prefill: (token, head) rows per
 *            wave (64: head_dim 128 only)
 *   PA_PREFILL_WAVES=4|8    chunked prefill (bf16, head_dim 128, 32 rows per
 *            wave): waves per work-group (default 4)
 *   PA_PREFILL_SPLIT=auto (default) | off | <keys>   chunked prefill: keys per
 *            piece of a query tile's key range (rounded up to a multiple of 64); auto uses
 *            max(1024, a quarter of the longest sequence)
 *   PA_PREFILL_ORDER=auto (default) | pieces | sequences   chunked prefill:
 *            order of the work-groups -- key-range pieces slowest, or
 *            sequences slowest (the last sequence of the batch first, so a
 *            batch that lists its decode sequences before its chunks
 *            dispatches the chunks' work first); auto: sequences when
 *            num_seqs * max_query_len > 2 * num_tokens
 * Errors: PA_ERR_ARG (incl. a workspace smaller than required),
 * PA_ERR_UNSUPPORTED, PA_ERR_RANGE (check mode), PA_ERR_HIP.
 */
pa_status pa_forward(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t block_table_stride,
                     const int32_t* seq_lens, const int32_t* query_start_loc,
                     const int32_t* cached_lens, int32_t num_seqs, int32_t num_tokens,
                     int32_t num_q_heads, int32_t max_seq_len, int32_t max_query_len,
                     const pa_cache_desc* c, float scale, int32_t causal,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_forward_noalloc — pa_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments and results as pa_forward, without
 * the workspace.  The split-KV scratch is instead a device array the library
 * holds, PA_FORWARD_NOALLOC_MAX_SCRATCH bytes on each GPU it runs on, kept
 * until the process ends; its address is looked up once per device, on the
 * first call there.  The call allocates nothing.
 *   - A batch whose pa_forward_workspace_size exceeds the limit returns
 *     PA_ERR_UNSUPPORTED with nothing enqueued (use pa_forward).
 *   - Every call on one GPU shares that GPU's array, and the array keeps the
 *     last call's contents (no call needs it cleared).  Calls that may overlap
 *     on one GPU -- on different streams without ordering between them, or
 *     from several threads -- race on it and give wrong results; order them.
 * Other errors as pa_forward.
 */
#define PA_FORWARD_NOALLOC_MAX_SCRATCH ((size_t)64 << 20)
pa_status pa_forward_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int32_t block_table_stride,
                             const int32_t* seq_lens, const int32_t* query_start_loc,
                             const int32_t* cached_lens, int32_t num_seqs, int32_t num_tokens,
                             int32_t num_q_heads, int32_t max_seq_len, int32_t max_query_len,
                             const pa_cache_desc* c, float scale, int32_t causal, void* stream);

/*
 * pa_write_kv_forward — pa_write_kv followed by pa_forward, in one call.
 *
 * [SLAVA] lead paragraph and [ART] forward-pass paragraph: a step stores its
 * new tokens' keys and values in their slots, then attends over the cache.
 * Arguments: pa_write_kv's (k, v, slot_mapping; num_tokens is the batch's)
 * and pa_forward's; the results -- the cache bytes and `out` -- are those of
 * the two calls in that order, bit for bit.
 *
 * A batch of single-token sequences (max_query_len == 1) with a bf16 or fp32
 * cache whose decode runs the balanced split-KV kernel or the vector kernel
 * (the defaults) takes a fused path: the decode reads each new token's row
 * from k / v instead of the cache and stores it into the cache itself, so no
 * separate write launch runs.  Every other batch runs the two calls.
 * Precondition of the fused path: each sequence's new token goes to its own
 * position seq_lens[i] - 1 as its block table maps it (slot_mapping[
 * query_start_loc[i]] = table[i][(L-1)/16]*16 + (L-1)%16), no two sequences
 * name the same slot, and that block is not read by another sequence of the
 * batch (the allocator's copy-on-write gives this).  Check mode (PA_CHECK=1)
 * validates the slots.  Errors as pa_write_kv and pa_forward.
 */
pa_status pa_write_kv_forward(const void* k, const void* v, const int64_t* slot_mapping, void* out,
                              const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
                              int32_t block_table_stride, const int32_t* seq_lens,
                              const int32_t* query_start_loc, const int32_t* cached_lens, int32_t num_seqs,
                              int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                              int32_t max_query_len, const pa_cache_desc* c, float scale, int32_t causal,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_forward_shared — pa_forward for a batch whose sequences share prefix
 * blocks, reading each shared block once for all of them.
 *
 * [SLAVA] section "Gemeinsame Nutzung erfordert mehr als Speicherzuweisung"
 * and [AIU] FAQ (sharing question): requests that fork from one prompt point
 * at the same physical blocks.  The result is pa_forward's (the same
 * definition, tolerances and supported shapes); only the work changes.
 *
 *   shared_blocks  device int32 [num_seqs]: shared_blocks[i] = the number of
 *                  leading block-table entries sequence i has in common with
 *                  sequence i - 1 (shared_blocks[0] is ignored); fewer than
 *                  the true count is allowed (less is shared), more is not.
 *                  pa_alloc_shared_blocks computes it on the host.
 *   other arguments as pa_forward; workspace of at least
 *   pa_forward_shared_workspace_size(...) bytes.
 *
 * A batch of single-token sequences (max_query_len == 1), bf16, head_dim 128,
 * up to 512 sequences, runs the shared-prefix decode: consecutive batch
 * entries are taken in fixed groups of P = 32 / (num_q_heads / num_kv_heads)
 * (4 at eight query heads per KV head, 32 at one); a group's leading blocks
 * that every member shares (and sees whole) are streamed once, with every
 * member's query heads as the columns of the matrix-core products; each
 * sequence's remaining blocks are its own; a log-sum-exp merge combines the
 * two parts per sequence.  Every other batch runs pa_forward's paths, and
 * shared_blocks is not read.  Results are deterministic; they are not bit
 * for bit pa_forward's (another order of accumulation).  Check mode
 * (PA_CHECK=1) also validates shared_blocks against the tables.
 * PA_SHARED_TOTAL_WAVES=<1..65536> sets the waves in all (default 1024).
 * Errors as pa_forward (PA_ERR_ARG also for a NULL shared_blocks).
 */
size_t pa_forward_shared_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                        int32_t max_seq_len, int32_t max_query_len, const pa_cache_desc* c);
pa_status pa_forward_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t block_table_stride,
                            const int32_t* seq_lens, const int32_t* query_start_loc,
                            const int32_t* cached_lens, const int32_t* shared_blocks, int32_t num_seqs,
                            int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len, int32_t max_query_len,
                            const pa_cache_desc* c, float scale, int32_t causal, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * pa_write_kv_forward_shared — pa_write_kv followed by pa_forward_shared, in
 * one call.
 *
 * As pa_write_kv_forward ([SLAVA] lead paragraph, [ART] forward-pass
 * paragraph: the step's write comes before its attention) for the batches
 * pa_forward_shared takes: when its shared-prefix decode runs the batch, the
 * decode takes each new token's row from k / v and its merge stores the row
 * into its slot; otherwise the two calls run.  The cache bytes are those of
 * pa_write_kv, and the output that of pa_forward_shared, bit for bit.
 * Preconditions: pa_write_kv_forward's (each new token at its sequence's
 * position L - 1, no slot twice, that block read by no other sequence) and
 * pa_forward_shared's (shared_blocks not above the true counts); check mode
 * validates both.  Arguments: pa_write_kv_forward's plus shared_blocks;
 * workspace as pa_forward_shared.  Errors as pa_write_kv and pa_forward_shared.
 */
pa_status pa_write_kv_forward_shared(const void* k, const void* v, const int64_t* slot_mapping, void* out,
                                     const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
                                     int32_t block_table_stride, const int32_t* seq_lens,
                                     const int32_t* query_start_loc, const int32_t* cached_lens,
                                     const int32_t* shared_blocks, int32_t num_seqs, int32_t num_tokens,
                                     int32_t num_q_heads, int32_t max_seq_len, int32_t max_query_len,
                                     const pa_cache_desc* c, float scale, int32_t causal, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * HIP graphs.  pa_write_kv, pa_copy_blocks, pa_forward and pa_write_kv_forward
 * (and pa_forward_noalloc, pa_forward_shared, pa_write_kv_forward_shared) may be recorded into
 * a HIP graph (stream capture on `stream`), so that a whole serving step
 * replays as one launch ([ART] forward-pass paragraph: the step's kernels are
 * replayed from a captured graph to save launch overhead).  On the fast path
 * none of them allocates, synchronises, writes memory with a memset or reads
 * device memory on the host.  A captured call keeps its host arguments
 * (pointers, sizes, max_seq_len, max_query_len, scale, causal, and the
 * environment knobs as read at capture); device data -- q, the caches, block
 * tables, slot mappings, seq_lens, query_start_loc, cached_lens -- are read
 * at each replay, so a step may be replayed after its inputs are updated in
 * place within the captured sizes (e.g. lengths that grew, up to the captured
 * max_seq_len).  While the stream is being captured, tracing records nothing
 * and check mode (PA_CHECK=1) returns PA_ERR_ARG.
 */

/* ------------------------------------------------------------------------ */
/* Tracing (instrumentation; not part of the method)                         */
/* ------------------------------------------------------------------------ */

/* One timed kernel launch: `kernel` names it (static storage); `ms` is the
 * time between HIP events recorded just before and just after the launch on
 * the caller's stream, or -1 if the events could not be read. */
typedef struct {
  const char* kernel;
  float ms;
} pa_trace_record;

/* Turn per-kernel timing on (on != 0) or off for every later device call of
 * this process.  While on, each kernel launch records two HIP events on the
 * caller's stream (no synchronisation); at most 4096 records are kept, the
 * oldest dropped first.  Always PA_OK. */
pa_status pa_trace_enable(int32_t on);

/* Waits for the recorded events, copies up to `cap` records (launch order)
 * into host array `out`, sets *n to the number copied, and clears the list.
 * Errors: PA_ERR_ARG (n NULL, cap < 0, out NULL with cap > 0), PA_ERR_HIP. */
pa_status pa_trace_read(pa_trace_record* out, int32_t cap, int32_t* n);

/* Measures the shader clock the GPU runs at now: launches a short probe (256
 * one-wave work-groups, about a millisecond, on `stream`), waits for it, and
 * sets *mhz to the median over the waves of (shader-clock ticks / real-time
 * ticks) * 100 MHz.  Meant right after timed work, to record the clock it ran
 * at.  Allocates nothing.  Errors: PA_ERR_ARG (mhz NULL, or the stream is
 * being captured), PA_ERR_HIP. */
pa_status pa_trace_clock(void* stream, float* mhz);

/* ------------------------------------------------------------------------ */
/* Host block allocator (no GPU calls; one thread at a time per allocator)   */
/* ------------------------------------------------------------------------ */

/*
 * [SLAVA] section "Ungenutzten Platz in Blöcken berechnen": blocks are added
 * as a sequence grows and returned when the request ends; only the last one
 * is partly filled.  [SLAVA] section "Gemeinsame Nutzung ..." / [AIU] FAQ:
 * requests may share blocks; a shared block is copied only on divergence.
 * [ART] paged-attention paragraph: 16-token blocks; exhausting them is the
 * signal for preemption (here PA_ERR_OOM, with nothing changed).
 *
 * Rules (exact; the same op sequence always yields the same tables, slots
 * and copy pairs):
 *   - Free blocks are taken from the head of a free list whose initial order
 *     the caller gives; a block whose refcount falls to 0 joins its tail.
 *   - Sequence ids are 0, 1, 2, ... in creation order, never reused.
 *   - fork(parent, k): the child shares the parent's first ceil(k/B) blocks
 *     (refcount + 1 each) and has length k (k <= parent length).
 *   - append(seq, n): positions p = len .. len+n-1 in order; at p % B == 0 a
 *     fresh block is appended; otherwise, the first time the append writes
 *     into a block with refcount > 1, that block is copied: a fresh block
 *     replaces it in the table, the pair (old, fresh) is emitted and the old
 *     refcount drops by one.  slot(p) = table[p / B] * B + p % B.
 *     All-or-nothing: PA_ERR_OOM (not enough free blocks) and PA_ERR_ARG
 *     (cow_cap too small) leave every table, refcount and list unchanged.
 *   - free(seq): refcount - 1 for each of its blocks in table order; blocks
 *     reaching 0 go to the free-list tail.
 */
typedef struct pa_alloc pa_alloc;

typedef struct {
  int64_t blocks_total;
  int64_t blocks_free;
  int64_t blocks_used;     /* refcount > 0 */
  int64_t blocks_shared;   /* refcount > 1 */
  int64_t tokens_logical;  /* sum of sequence lengths */
  int64_t slots_logical;   /* sum over sequences of table length * block_size */
  int64_t slots_physical;  /* blocks_used * block_size */
} pa_alloc_stats_t;

/* free_order: host int32 permutation of 0..num_blocks-1, or NULL for 0..num_blocks-1.
 * *out receives a handle owned by the caller, released with pa_alloc_destroy. */
pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                          pa_alloc** out);
void pa_alloc_destroy(pa_alloc* a);

pa_status pa_seq_create(pa_alloc* a, int32_t* seq_id);
pa_status pa_seq_fork(pa_alloc* a, int32_t parent, int32_t share_tokens, int32_t* child);

/* slots_out: host int64 [n_tokens]; cow_pairs_out: host int32 [2*cow_cap] (src, dst) pairs;
 * *n_cow receives the number of pairs written.  n_tokens == 0 is a no-op. */
pa_status pa_seq_append(pa_alloc* a, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                        int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow);
pa_status pa_seq_free(pa_alloc* a, int32_t seq);

/* Copies up to cap block ids (logical order) into out; *n_blocks and *len
 * always receive the table length and token count.  out may be NULL to query
 * the size; a non-NULL out with cap < table length is PA_ERR_ARG. */
pa_status pa_seq_block_table(const pa_alloc* a, int32_t seq, int32_t* out, int32_t cap,
                             int32_t* n_blocks, int32_t* len);
pa_status pa_alloc_stats(const pa_alloc* a, pa_alloc_stats_t* s);

/* Blocks each sequence shares with the one before it in a batch: for
 * seq_ids[0..n-1] (host int32, batch order), out[i] (host int32) = the number
 * of leading block-table entries sequence seq_ids[i] has in common with
 * seq_ids[i-1] (the length of their common prefix of block ids), out[0] = 0.
 * The argument pa_forward_shared takes ([SLAVA] section "Gemeinsame Nutzung
 * ...": forked requests point at the same blocks).  Errors: PA_ERR_ARG (NULL
 * arguments, n < 0, unknown sequence). */
pa_status pa_alloc_shared_blocks(const pa_alloc* a, const int32_t* seq_ids, int32_t n, int32_t* out);

/* Refcount of one block, or -1 for an id outside the pool. */
int32_t pa_block_refcount(const pa_alloc* a, int32_t block);

/* Free list, head first: copies up to cap ids into out; *n receives its length. */
pa_status pa_alloc_free_list(const pa_alloc* a, int32_t* out, int32_t cap, int32_t* n);

/*
 * Prefix caching.  [ART] prefix-caching paragraph: the engine hashes blocks
 * of tokens and keeps them; a request that starts with the same tokens finds
 * the matching blocks and reuses their K/V instead of recomputing them.
 * [HADA] bullet "Prefix Caching".  Host-side only: a hit gives the new
 * sequence the existing physical blocks, and the caller's prefill then runs
 * with cached_lens = *n_cached.
 *
 * Rules (exact; both the library and its reference follow them):
 *   - Chained block hash: for full block b of a token sequence (tokens
 *     B*b .. B*b+B-1), h(b) = FNV-1a 64 of the 8 little-endian bytes of
 *     h(b-1) followed by the 4 little-endian bytes of each token id, with
 *     h(-1) = 0xcbf29ce484222325 (the FNV-1a 64 offset basis; FNV prime
 *     0x100000001b3).  A block's hash thus names the whole prefix it ends.
 *   - A registered block carries its hash, its parent's hash and its B
 *     tokens; the cache maps a hash to at most one registered block.  A
 *     lookup hits only when the hash, the parent hash and every token match.
 *   - pa_prefix_register(seq, tokens, n): for each full block b of the first
 *     n tokens of seq (n <= the sequence's length), in order, that is not
 *     registered yet: if no block is registered under h(b), register it;
 *     otherwise leave it unregistered (the sequence keeps its own copy).
 *   - pa_prefix_lookup(tokens, n): creates a sequence (the next id) holding
 *     the longest run of full blocks b = 0, 1, ... that hit, leaving at least
 *     one token uncached (b < (n - 1) / B).  Each hit block's refcount rises
 *     by one; a hit block with refcount 0 is taken out of the free list.
 *     *n_cached = B * hits is the sequence's length; the caller appends the
 *     other n - *n_cached tokens (pa_seq_append) and runs their prefill.
 *   - A registered block whose refcount falls to 0 stays registered at the
 *     free-list tail; when the free list hands it out again it is first
 *     unregistered (evicted).  Blocks registered after it stay: a lookup
 *     reaches them only through a block registered under the same hash,
 *     i.e. after the same tokens, so their K/V stay valid.
 *   - A registered block is never written while registered: an append that
 *     would write into one without copying it (a fork shared it part-way and
 *     the other holders have let go) unregisters it first (an eviction).
 * tokens: host int32 [n_tokens].  Errors: PA_ERR_ARG (NULL arguments,
 * unknown sequence, n_tokens outside [0, length] for register, < 0 for lookup).
 */
pa_status pa_prefix_register(pa_alloc* a, int32_t seq, const int32_t* tokens, int32_t n_tokens);
pa_status pa_prefix_lookup(pa_alloc* a, const int32_t* tokens, int32_t n_tokens, int32_t* seq_id,
                           int32_t* n_cached);

typedef struct {
  int64_t blocks_registered;  /* blocks currently in the cache */
  int64_t registered_free;    /* of those, refcount 0 (on the free list) */
  int64_t lookups;            /* pa_prefix_lookup calls */
  int64_t hit_blocks;         /* blocks reused by them */
  int64_t evictions;          /* registered blocks dropped from the cache */
} pa_prefix_stats_t;
pa_status pa_prefix_stats(const pa_alloc* a, pa_prefix_stats_t* s);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
