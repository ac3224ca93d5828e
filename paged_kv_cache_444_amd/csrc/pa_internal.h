// Host-side interfaces between the C ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Launch tunables (for sweeps and tests).  Each starts from its default, or from the environment
// variable of the same name if that holds an in-range value; the environment is read once, on
// first use.  pa_set_tunable / pa_get_tunable change and read them afterwards.
enum Tunable {
  kTuneDecodePrefetch,     // PA_DECODE_PREFETCH: K/V steps in flight per wave, vector step (0-2)
  kTuneDecodePrefetchFp8,  // PA_DECODE_PREFETCH_FP8: the same for FP8 pools (1-2)
  kTuneDecodeMfma,         // PA_DECODE_MFMA: bf16 steps on the matrix cores (1) or vector ALUs (0)
  kTuneDecodeQuad,         // PA_DECODE_QUAD: workgroup workers over units of four KV heads (0-1)
  kTuneDecodePieceCost,    // PA_DECODE_PIECE_COST: steps charged per unit a worker starts (0-64)
  kTuneDecodeWorkers,      // PA_DECODE_WORKERS: worker waves (0: one workgroup per CU)
  kTuneDecodeStaticQ10,    // PA_DECODE_STATIC_Q10: share of steps split statically (512-1024)
  kTuneDecodeChunk,        // PA_DECODE_CHUNK: smallest dynamic chunk, in steps (1-256)
  kTunePrefillSplits,      // PA_PREFILL_SPLITS: forced context split of a prefill (0: automatic)
  kTuneDecodeTailQ10,      // PA_DECODE_TAIL_Q10: share of head-quad steps left to the dynamic tail
  kTuneDecodeTailQ10Fp8,   // PA_DECODE_TAIL_Q10_FP8: the same for FP8 pools
  kTuneDecodeTailChunk,    // PA_DECODE_TAIL_CHUNK: steps per dynamic tail chunk (1-256)
  kNumTunables
};
int tunable(Tunable t);

// Decode work is cut into "steps" of 16 tokens of one (sequence, KV head) pair.  The pairs
// ("units", numbered s*num_kv_heads + h) are laid end to end and every worker wave takes an equal
// contiguous range of the concatenated steps, so the load is balanced whatever the length mix.
// A unit finished inside one wave is written to the output directly; the pieces of a unit that
// spans several waves go to per-piece partial slots and decode_merge combines them.
struct DecodeParams {
  uint16_t* out;
  const uint16_t* query;
  const uint16_t* kpool;
  const uint16_t* vpool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  unsigned* counter;  // dynamic chunks handed out so far; zero between calls
  int2* unit_info;    // [num_seqs*num_kv_heads] (first worker, last worker) of each unit
  float* partials;    // [num_workers + dyn_cap + units][G][2 + D]: m[G], l[G], acc[G][D]
  int64_t num_blocks;
  int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  int num_workers;     // waves launched (grid size * waves per workgroup)
  int dyn_cap;         // most dynamic chunks the workspace holds (0: static split only)
  int chunk_steps;     // smallest dynamic chunk, in steps
  int static_frac_q10; // share of the steps split statically, in 1/1024
  // Nonzero: workgroup-level workers over units of four consecutive KV heads (wave r takes head
  // 4*unit + r), so the four waves of a CU read neighbouring 4 KB tiles of the same block
  // together.  Static split only; num_kv_heads a multiple of four.
  int quad;
  // Cost of starting a piece, in steps: the static split balances steps plus this much per unit
  // a worker starts, since each piece begins with dependent loads that nothing overlaps.
  int piece_cost;
  // Dynamic tail of the head-quad split (matrix-core steps): the last tail_q10/1024 of the steps
  // are cut into chunks of about tail_chunk steps that workgroups claim from `counter` once their
  // static range is done, so workgroups served faster take more.  0: static split only.
  int tail_q10, tail_chunk;
  // Lengths are clamped to this (min of max_seq_len and the table width) so a length beyond the
  // caller's bound cannot take a kernel outside the table.
  int len_cap;
  float scale_log2;  // softmax scale times log2(e) (times the K scale for an FP8 cache)
  // Nonzero: the pools hold FP8 E4M3 codes (one byte per element, same element order) and
  // every output is multiplied by v_scale; for bf16 pools v_scale is 1.
  int kv_fp8;
  float v_scale;
  // Shared-prefix (cascade) use.  skip_lens non-null: int32 [num_seqs], leading tokens of each
  // sequence left out (whole blocks: rounded down to a multiple of block_size), so the sequence
  // is attended from table entry skip / block_size on.  state_ml non-null: each (sequence, query
  // head) row's final (m in the log2 domain, l) and unnormalised acc go to split state_split of
  // the prefill workspace layout (state_ml[2u], state_ml[2u+1], state_acc[u*D..],
  // u = row*state_stride + state_split) instead of the output.
  // state_final nonzero: splits 0 .. state_split-1 of every row already hold states (the shared
  // prompt's), and the merge combines them with this call's tail and writes the output, so no
  // separate pass over the states is needed.
  const int32_t* skip_lens;
  float* state_ml;
  float* state_acc;
  int state_stride, state_split, state_final;
};

// Waves the decode kernel is launched with for this shape and pool type on the current device.
int decode_workers(int head_dim, int group, bool fp8);
// Workspace layout of pa_decode: the chunk counter, then unit_info, then the partial slots.
// With chunk_slots, `bytes` also holds the dynamic chunks' slots and covers both pool types (one
// size query serves pa_decode and pa_decode_fp8); without, it is the static split's layout of
// this launch only (no dynamic chunks: dyn_cap = 0).
struct DecodeWorkspace {
  size_t counter_off, info_off, partials_off, bytes;
  int workers, dyn_cap;
};
DecodeWorkspace decode_workspace(int num_seqs, int num_kv_heads, int head_dim, int group, bool fp8,
                                 bool chunk_slots = true);
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
  // FP8 pools: write E4M3 codes of value / scale (kpool and vpool then point at bytes).
  int kv_fp8;
  float k_scale, v_scale;
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
  float* ws_ml;   // [total_q][Hq][splits] (m, l), m in the log2 domain
  float* ws_acc;  // [total_q][Hq][splits][D]
  int64_t num_blocks;
  int num_seqs, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size;
  int max_blocks_per_seq, max_seq_len;
  int splits, split_keys;  // context split: `splits` key ranges of split_keys keys (multiple of 32)
  float scale_log2;
  // Shared-prefix (cascade) use.  noncausal: every row sees all L keys.  from_first_row: sequence
  // i's block-table row and length are those of row query_start_loc[i] (its first query row's
  // sequence): block_tables and seq_lens are then indexed by query row.  ws_splits: split count
  // of the workspace layout (>= splits; split j of row u is slot u * ws_splits + j).
  // defer_merge: always write split states, never the output; the caller merges later.
  int noncausal, from_first_row, ws_splits, defer_merge;
  // FP8 pools (E4M3 codes, same element order, one byte each); outputs and split states are
  // multiplied by v_scale (1 for bf16 pools).
  int kv_fp8;
  float v_scale;
  // Nonzero when another kernel runs beside this one on the same CUs (the mixed step's decode on
  // its side stream).  Otherwise each wave raises its issue priority over its softmax and second
  // product, which a concurrent kernel's waves would then wait behind.
  int concurrent;
};

// Context split chosen for a prefill launch (it sizes the workspace).
struct PrefillSplit {
  int splits, split_keys;
};
PrefillSplit prefill_split(int num_seqs, int max_q_len, int num_kv_heads, int group, int head_dim,
                           int max_seq_len);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
// Combine p.ws_splits split states of each of p.total_q rows into p.out.
hipError_t launch_prefill_merge(const PrefillParams& p, hipStream_t stream);

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
