// Host-side interfaces between the C ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Tokens of one sequence handled by one decode work unit (a "partition").  A multiple of 32 so
// partitions start on block boundaries for both block sizes; at most 64 blocks per partition.
int decode_partition_tokens();

struct DecodeParams {
  uint16_t* out;
  const uint16_t* query;
  const uint16_t* kpool;
  const uint16_t* vpool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_ml;   // [B][Hq][P] (m, l) pairs
  float* ws_acc;  // [B][Hq][P][D]
  int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  int part_tokens, max_parts;
  // Lengths are clamped to this (min of max_parts*part_tokens and the table width) so a length
  // beyond the caller's bound cannot take a kernel outside the table or the workspace.
  int len_cap;
  float scale_log2;  // softmax scale times log2(e)
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

struct ReshapeParams {
  const uint16_t* key;
  const uint16_t* value;
  int64_t token_stride;
  uint16_t* kpool;
  uint16_t* vpool;
  const int64_t* slots;
  int num_tokens, num_kv_heads, head_dim, block_size;
  int64_t num_blocks;
};

hipError_t launch_reshape(const ReshapeParams& p, hipStream_t stream);

struct PrefillParams {
  uint16_t* out;
  const uint16_t* query;
  const uint16_t* kpool;
  const uint16_t* vpool;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  const int32_t* seq_lens;
  float* ws_ml;   // [total_q][Hq][splits] (m, l)
  float* ws_acc;  // [total_q][Hq][splits][D]
  int num_seqs, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size;
  int max_blocks_per_seq, max_seq_len, splits;
  float scale_log2;
};

int prefill_splits(int num_seqs, int max_q_len, int num_kv_heads, int group, int max_seq_len);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Kernel timing: when tracing is on, launches are bracketed by events on their stream.
struct TraceScope {
  TraceScope(const char* name, hipStream_t stream);
  ~TraceScope();
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;

 private:
  int slot_;
  hipStream_t stream_;
};

}  // namespace pa
