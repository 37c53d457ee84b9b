// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

inline int elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : dtype == PA_FP8 ? 1 : 2; }


pa_status check_desc(const pa_cache_desc* c, const char* who);
pa_status launch_status(const char* who);

// True while `s` is being captured into a HIP graph (calls that would
// synchronise or read device memory on the host refuse to run then).
bool stream_capturing(hipStream_t s);

// Tracing: bracket a kernel launch with trace_begin / trace_end on its stream
// (no-ops unless pa_trace_enable(1), and while the stream is being captured);
// `kernel` must have static storage.
int trace_begin(hipStream_t s);
void trace_end(hipStream_t s, int mark, const char* kernel);

// Arguments shared by the attention kernels (device pointers, host scalars).
struct AttnArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;          // query_start_loc
  const int32_t* cached_lens;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t head_dim;
  float scale_log2;            // softmax scale * log2(e): scores are kept in base-2 units
  int32_t causal;
  int32_t prefill_min_q;       // the prefill kernel takes sequences with at least this many query tokens
  // Fused cache write (pa_write_kv_forward on a batch of single-token
  // sequences; both NULL otherwise): the step's new K and V rows,
  // [num_tokens][num_kv_heads][head_dim].  The decode kernel that folds a
  // sequence's last block takes the new token's row (position L - 1) from
  // these and stores it into the cache there.
  const void* k_new;
  const void* v_new;
};

// Plan for the decode path (sequences with one query token).
//
// Balanced (decode_mfma, at most 1024 sequences): `waves_per_head` waves per KV
// head split that head's concatenated decode tiles into equal ranges.
// Workspace (offsets 256-byte aligned):
//   [part table: int32 [num_seqs][2]]
//   [partial acc: fp32 [Hkv][num_seqs + waves_per_head][G][head_dim]]
//   [partial (max, sum): fp32 [Hkv][num_seqs + waves_per_head][G][2]]
// Partitioned (otherwise): sequences are cut into partitions of part_tokens.
// Workspace when max_parts > 1:
//   [partial acc: fp32 [num_seqs][Hq][max_parts][head_dim]]
//   [partial (max, sum): fp32 [num_seqs][Hq][max_parts][2]]
struct DecodePlan {
  bool mfma;               // decode on the matrix cores (bf16, head_dim 128), else the VALU kernel
  bool balanced;           // balanced one-round decode_mfma launch
  int32_t waves_per_head;  // balanced: waves per KV head
  int32_t depth;           // balanced: K/V tiles in flight per wave (2..4)
  int32_t waves;           // partitioned decode_mfma: waves per work-group
  int32_t part_tokens;     // partitioned: tokens per partition (multiple of 16)
  int32_t max_parts;       // partitioned: partitions of the longest sequence; 1 = no split
  size_t info_bytes;       // balanced: part table
  size_t acc_bytes;        // partial accumulators
  size_t ml_bytes;         // partial (max, sum) pairs
  size_t workspace_bytes() const { return info_bytes + acc_bytes + ml_bytes; }
};

DecodePlan make_decode_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t dtype, int32_t max_seq_len);

// Decode (VALU) kernel: sequences with one query token; with `rows_mode` it
// also handles multi-token sequences one query row at a time (no split).
pa_status launch_decode(const AttnArgs& a, int32_t dtype, const DecodePlan& plan, float* partial_acc,
                        float* partial_ml, bool rows_mode, hipStream_t s);
pa_status launch_merge(const AttnArgs& a, int32_t dtype, const DecodePlan& plan,
                       const float* partial_acc, const float* partial_ml, hipStream_t s);

// Decode on the matrix cores (bf16, head_dim 128); partials go to launch_merge.
bool decode_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group);
pa_status launch_decode_mfma(const AttnArgs& a, const DecodePlan& plan, float* p_acc, float* p_ml,
                             hipStream_t s);
// Balanced decode_mfma and its merge (both launched here).
bool decode_balanced_supported(int32_t num_seqs);
pa_status launch_decode_balanced(const AttnArgs& a, const DecodePlan& plan, float* p_acc, float* p_ml,
                                 int32_t* part_table, hipStream_t s);

// Plan for the multi-token decode path (sequences with 2 .. max_q query
// tokens, bf16, head_dim 128, at most 1024 sequences): balanced like the
// single-token decode, columns = (token, query head) pairs in col_groups
// groups of 16.  Workspace (offsets 256-byte aligned):
//   [part table: int32 [num_seqs][2]]
//   [partial acc: fp16 [Hkv][num_seqs + waves_per_head][16 col_groups][head_dim], each
//    column normalised by its weight sum and scaled by 2^-e]
//   [partial (max, sum, e, 0): fp32 [Hkv][num_seqs + waves_per_head][16 col_groups][4]]
struct VerifyPlan {
  bool on;
  bool fp8;                // quantised pools (then it takes every sequence it can)
  int32_t min_q;           // 2, or 1 when it also takes the single-token sequences
  int32_t col_groups;      // 1, 2 or 4
  int32_t max_q;           // longest sequence (query tokens) it takes; longer ones go to prefill
  int32_t waves_per_head;
  int32_t depth;           // K/V tiles in flight per wave (2 or 3)
  int32_t first_ranks;     // ranks of each head whose work-groups are dispatched first on their SIMD
  int32_t first_weight;    // their share of tiles per 1000 of the other ranks'
  size_t info_bytes, acc_bytes, ml_bytes;
  size_t workspace_bytes() const { return info_bytes + acc_bytes + ml_bytes; }
};

bool verify_fp8_supported(int32_t head_dim, int32_t group);
VerifyPlan make_verify_plan(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t dtype, int32_t max_seq_len, int32_t max_query_len);
pa_status launch_decode_verify(const AttnArgs& a, const VerifyPlan& vp, uint16_t* p_acc, float* p_ml,
                               int32_t* part_table, hipStream_t s);

// Plan for the shared-prefix decode (pa_forward_shared): single-token
// sequences only, bf16, head_dim 128, at most 512 sequences.  Workspace
// (offsets 256-byte aligned):
//   [group prefix F per sequence: int32 [num_seqs]]
//   [item (first rank, parts): int2 [2 num_seqs]]
//   [partial acc: fp16 [Hkv][2 num_seqs + waves_per_head][col_groups][8][64][4], each column
//    normalised by its weight sum and scaled by 2^-e]
//   [partial (max, sum, e, 0): fp32 [Hkv][2 num_seqs + waves_per_head][16 col_groups][4]]
struct SharedPlan {
  bool on;
  int32_t col_groups;      // 2 or 4 groups of 16 MFMA columns
  int32_t waves_per_head;
  int32_t depth;           // K/V tiles in flight per wave (2 or 3)
  size_t prefix_bytes, info_bytes, acc_bytes, ml_bytes;
  size_t workspace_bytes() const { return prefix_bytes + info_bytes + acc_bytes + ml_bytes; }
};

SharedPlan make_shared_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t dtype, int32_t max_seq_len, int32_t max_query_len);
pa_status launch_decode_shared(const AttnArgs& a, const SharedPlan& sp, const int32_t* shared_blocks,
                               void* workspace, hipStream_t s);

// Split-KV plan for the chunked-prefill kernel: the key range of every
// (sequence, query tile, KV head) work-group is cut into pieces of piece_keys
// keys (a multiple of 64); work-groups whose range spans more than one piece
// write partials per piece and the prefill merge kernel combines them.
// Workspace (after the decode partials, 256-byte aligned):
//   [partial O: fp16 [num_tokens][Hq][pieces][head_dim], each row normalised
//    by its piece's weight sum and scaled by 2^-e]
//   [partial (max, sum, e, 0): fp32 [num_tokens][Hq][pieces][4]]
struct PrefillPlan {
  int32_t piece_keys;
  int32_t pieces;      // pieces of the longest key range; 1 = no split
  size_t o_bytes;
  size_t ml_bytes;
  size_t workspace_bytes() const { return o_bytes + ml_bytes; }
};

PrefillPlan make_prefill_plan(int32_t num_tokens, int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                              int32_t max_query_len, bool mfma);

// Chunked-prefill (MFMA) kernel for bf16 (or fp8-cache) sequences with more
// than one query token, followed by its merge when the plan splits key ranges.
bool prefill_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group);
pa_status launch_prefill(const AttnArgs& a, int32_t max_query_len, const PrefillPlan& pp, uint16_t* p_o, float* p_ml,
                         bool fp8, hipStream_t s);

}  // namespace pa
