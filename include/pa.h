/*
 * pa.h — C ABI of libpagedattn: paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * The KV cache lives in fixed-size physical blocks of `block_size` tokens (16 or 32) that may sit
 * anywhere in a pool; each sequence reaches its blocks through a block table that maps logical
 * token positions to physical block ids ("Serving engine internals" lesson, section
 * "PagedAttention as a virtual memory system"; "Inference optimization" lesson, section "Paged
 * attention"; vLLM-on-H100 article, section "PagedAttention borrows from operating systems").
 * Attention itself is max-subtracted softmax(q·kᵀ·scale)·v ("Inference optimization", Build it,
 * Step 2: attention with a KV cache), with grouped-query heads (exercises of the same lesson).
 *
 * Conventions for every entry point
 *   - All arrays are device pointers owned by the caller; the library allocates no device memory,
 *     keeps no device state between calls (except pa_decode_no_alloc's fixed scratch array, see
 *     there), and never synchronises the stream (pa_mixed_step keeps two host-side events per
 *     thread and device, see there).
 *   - bf16 tensors are raw 16-bit bfloat16 bit patterns, contiguous, 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call enqueues its kernels on
 *     that stream and returns immediately.
 *   - Errors that can be seen from host-side scalars and pointer values are returned before any
 *     launch, with no buffer touched: PA_ERR_NULL_POINTER, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED,
 *     PA_ERR_WORKSPACE.  PA_ERR_HIP means a launch failed.  pa_last_error() then holds a message
 *     for the calling thread.
 *   - Contents of device arrays (lengths, table entries, slots) are preconditions, not checked on
 *     the host.  Kernels clamp what they must to stay inside the buffers they were given (a slot
 *     past the pool is skipped), but results for inputs that break a precondition are unspecified.
 *
 * Pool layout (the library's own; the pages fix only that blocks are fixed-size and placed
 * anywhere).  key_cache and value_cache are each [num_blocks][num_kv_heads][block_size*head_dim]
 * bf16.  A block is cut into sub-blocks of 16 tokens; inside a sub-block
 *   K is [head_dim/32][16][32]: per 32-wide slice of the head dimension, 16 tokens x 32 values;
 *   V is [head_dim][16]:         per head-dimension index, the 16 tokens' values.
 * Element (token o of the block, dim d) therefore sits at, counting from the (block, head) tile,
 *   K: (o/16)*16*head_dim + (d/32)*512 + (o%16)*32 + d%32
 *   V: (o/16)*16*head_dim + d*16 + o%16
 * Callers write the pools only through pa_reshape_and_cache, so the layout is opaque to them.
 */
#ifndef PAGEDATTN_PA_H
#define PAGEDATTN_PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status_t;

#define PA_OK 0
#define PA_ERR_NULL_POINTER 1 /* a required pointer is NULL */
#define PA_ERR_INVALID_ARG 2  /* negative size, Hq % Hkv != 0, misaligned pointer, bad stride ... */
#define PA_ERR_UNSUPPORTED 3  /* head_dim not in {64,128,256}, block_size not in {16,32}, group too wide */
#define PA_ERR_WORKSPACE 4    /* workspace NULL or smaller than the *_workspace_bytes query */
#define PA_ERR_HIP 5          /* a kernel launch failed; see pa_last_error() */

/* Library version, major*10000 + minor*100 + patch. */
int32_t pa_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* pa_last_error(void);

/*
 * Launch tunables, for sweeps and tests: they change how work is spread over the GPU, never what
 * is computed beyond fp32 rounding order.  Each starts from its default, or from the environment
 * variable of the same name if that holds an in-range integer; the environment is read once, at
 * the first call that needs a tunable.  Values are process-wide (all threads and devices); a call
 * uses the values current when it is made.
 *   PA_DECODE_PREFETCH      0-2, default 1: K/V steps in flight per wave on the vector step
 *   PA_DECODE_PREFETCH_FP8  1-2, default 1: the same for FP8 pools
 *   PA_DECODE_MFMA          0-1, default 1: bf16 decode steps on the matrix cores (0: vector ALUs)
 *   PA_DECODE_QUAD          0-1, default 1: workgroup workers over units of four KV heads
 *   PA_DECODE_PIECE_COST    0-64, default 4: steps' worth of cost per unit a decode worker starts
 *   PA_DECODE_WORKERS       default 0 (one workgroup of four waves per CU): total decode worker
 *                           waves, rounded down to a multiple of 4 and capped at what can be
 *                           resident; values below 4 mean the default
 *   PA_DECODE_STATIC_Q10    512-1024, default 1024: share (in 1/1024) of decode steps split
 *                           statically; the rest is handed out in dynamic chunks
 *   PA_DECODE_CHUNK         1-256, default 4: smallest dynamic chunk, in steps
 *   PA_PREFILL_SPLITS       0-16, default 0 (automatic): forced context split of a prefill chunk
 *   PA_DECODE_TAIL_Q10      0-512, default 0: share (in 1/1024) of the head-quad split's steps
 *                           left to a dynamic tail of chunks that workgroups claim once their
 *                           static range is done (results stay bitwise reproducible)
 *   PA_DECODE_TAIL_Q10_FP8  the same for FP8 pools, default 0
 *   PA_DECODE_TAIL_CHUNK    1-256, default 12: steps per dynamic tail chunk
 * The decode workspace size depends on PA_DECODE_WORKERS: query it after setting that.
 * pa_set_tunable returns PA_ERR_INVALID_ARG for an unknown name or an out-of-range value (the
 * value is then unchanged); pa_get_tunable writes the current value to *value.
 */
pa_status_t pa_set_tunable(const char* name, int32_t value);
pa_status_t pa_get_tunable(const char* name, int32_t* value);

/*
 * pa_reshape_and_cache — write the K/V rows of new tokens into their cache slots.
 *
 * Source: blocks fill as tokens arrive and a sequence that outgrows its blocks gets one more
 * ("Serving engine internals", PagedAttention section); the slot of logical position p of a
 * sequence is  block_table[p / block_size] * block_size + p % block_size.
 *
 *   key, value     bf16 [num_tokens] rows; token t, head h, dim d at t*kv_token_stride + h*head_dim + d
 *   kv_token_stride elements between consecutive tokens (>= num_kv_heads*head_dim, multiple of 8)
 *   key_cache, value_cache  pools as described above, modified in place
 *   slot_mapping   int64 [num_tokens]; negative = skip this token; slots past the pool are skipped
 *   num_blocks     physical blocks in each pool
 * Slots must be pairwise distinct within one call (otherwise which row lands is unspecified).
 * The copy is bit-exact.  num_tokens == 0 is a no-op.
 */
pa_status_t pa_reshape_and_cache(const void* key, const void* value, int64_t kv_token_stride,
                                 void* key_cache, void* value_cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, void* stream);

/*
 * FP8 KV cache.  The pages name FP8 as a serving precision (the "Serving engine internals" lesson
 * quotes Llama 3.3 70B in FP8; the "Inference optimization" lesson lists FP8 quantization among
 * kernel optimizations; the vLLM-on-H100 article names FP8 precision as a further lever) without
 * fixing a format.  Here it is the OCP 8-bit E4M3 format (sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, largest finite 448, no infinities) with one scale per pool: a cached value is
 * k_scale * (value of its code) for K and v_scale * (value of its code) for V.  FP8 pools have the
 * layout above with one byte per element, so a block is num_kv_heads*block_size*head_dim bytes.
 */

/*
 * pa_reshape_and_cache_fp8 — pa_reshape_and_cache into FP8 pools.  Each bf16 value x of a new
 * token is stored as the E4M3 code of fp32(x) / scale (the correctly rounded fp32 quotient,
 * rounded to the nearest E4M3 value with ties to even, magnitudes above 448 saturating to 448,
 * NaN stored as 0x7F with x's sign).  key_cache / value_cache are byte pools; k_scale and v_scale
 * must be finite and positive (PA_ERR_INVALID_ARG otherwise).  Other arguments, preconditions and
 * errors as pa_reshape_and_cache.
 */
pa_status_t pa_reshape_and_cache_fp8(const void* key, const void* value, int64_t kv_token_stride,
                                     void* key_cache, void* value_cache,
                                     const int64_t* slot_mapping, int32_t num_tokens,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int64_t num_blocks, float k_scale, float v_scale,
                                     void* stream);

/*
 * pa_copy_blocks — copy whole physical blocks (K and V, every KV head) for copy-on-write.
 *
 * Source: sequences that share a prompt reference the prompt's physical blocks, and a sequence
 * receives a block of its own only where it diverges ("Inference optimization" lesson, section
 * "Paged attention"; vLLM-on-H100 article, PagedAttention section: rollouts of one prompt share
 * its pages and copy only where their completions diverge).  Before a sequence writes into a
 * block that others still reference, the caller allocates a fresh block, points that sequence's
 * table entry at it and copies the shared block there with this call; pa_reshape_and_cache then
 * writes the new token into the copy.
 *
 *   key_cache, value_cache  pools of num_blocks blocks (layout above), modified in place
 *   block_mapping  int64 [num_pairs][2]: (source, destination) block ids; a pair with an id
 *                  outside [0, num_blocks) is skipped
 *   num_kv_heads, head_dim, block_size  the pools' shape (a block is
 *                  num_kv_heads*block_size*head_dim bf16 values in each pool)
 * Destinations must be pairwise distinct and no destination may also be a source within one call
 * (otherwise the result is unspecified); each destination then holds the bytes its source held
 * before the call.  The copy is bit-exact.  num_pairs == 0 is a no-op.
 */
pa_status_t pa_copy_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                           const int64_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, void* stream);

/*
 * Bytes of workspace pa_decode needs for this batch shape on the current device (0 if the shape is
 * unsupported or num_seqs <= 0).  The workspace holds partial softmax states of sequences whose
 * context is split over several waves and a counter that hands out work; it must be filled with
 * zeros before its first use, and every pa_decode call leaves it ready for the next one (reuse it
 * across calls on one stream).  Calls that may run concurrently (different streams) need
 * separate workspaces.  The size depends on num_seqs, num_kv_heads, head_dim, the group size and
 * the device, not on the lengths; max_seq_len is accepted for symmetry with pa_decode.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len);

/*
 * pa_decode — one query token per sequence against that sequence's whole paged context.
 *
 * Source: decode produces one token per step and re-reads the accumulated KV cache each time
 * ("Inference optimization", section "Prefill vs decode"; vLLM-on-H100 article, section "Decode is
 * a memory problem"); the attention is Step 2 of the same lesson with a single query row.
 * Query head h reads KV head h / (num_q_heads/num_kv_heads).
 *
 *   out            bf16 [num_seqs][num_q_heads][head_dim] (written; must not alias inputs)
 *   query          bf16 [num_seqs][num_q_heads][head_dim]
 *   key_cache, value_cache  pools of num_blocks blocks (layout above)
 *   num_blocks     blocks in each pool; table entries are clamped into [0, num_blocks) so a bad
 *                  entry cannot read outside the pool (its result is then unspecified)
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]; only the first ceil(L/block_size)
 *                  entries of a row are read
 *   seq_lens       int32 [num_seqs]; L = cached tokens including the query's own K/V
 *                  (0 <= L <= max_seq_len; larger values are clamped to max_seq_len);
 *                  L == 0 yields a zero output row
 *   max_seq_len    an upper bound of every seq_lens entry, known on the host
 *                  (<= max_blocks_per_seq*block_size)
 *   scale          softmax scale (> 0), normally 1/sqrt(head_dim)
 *   workspace      device buffer of at least pa_decode_workspace_bytes(...) bytes (never NULL
 *                  when num_seqs > 0), zero-filled before its first use; a workspace that was
 *                  not gives unspecified results (never an access outside the buffers)
 * Output is fp32-accumulated and rounded to bf16 (nearest even); results are bitwise
 * reproducible for the same inputs and do not depend on which physical blocks hold the context.
 * Supported: head_dim 64 with group size <= 16, head_dim 128 with group <= 8, head_dim 256 with
 * group <= 4; group sizes are powers of two.
 */
pa_status_t pa_decode(void* out, const void* query, const void* key_cache,
                      const void* value_cache, int64_t num_blocks, const int32_t* block_tables,
                      const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_fp8 — pa_decode over FP8 pools written by pa_reshape_and_cache_fp8, with the same
 * k_scale and v_scale.  The attention is that of pa_decode on the dequantised cache: scores are
 * scale * k_scale * (q · codes' values), outputs v_scale * (softmax-weighted codes' values); each
 * code is widened to bf16 exactly and accumulated in fp32.  scale * k_scale must stay finite.
 * Workspace, preconditions, limits and errors as pa_decode (same workspace size query).
 */
pa_status_t pa_decode_fp8(void* out, const void* query, const void* key_cache,
                          const void* value_cache, int64_t num_blocks,
                          const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                          float scale, float k_scale, float v_scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * pa_decode_no_alloc — pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It takes no workspace
 * and allocates nothing; its scratch (the unit table and partial softmax states of sequences
 * split over several waves) is a fixed array of PA_DECODE_NO_ALLOC_SCRATCH_BYTES inside the
 * library, one per device, held from the device's first call until the process ends.
 *
 *   arguments      as pa_decode (bf16 pools), without the workspace
 * Limit: the batch's scratch (about (num_seqs*num_kv_heads + 4 * CUs) * G * (head_dim + 2) * 4
 * bytes: 8.5 MB for 128 sequences of 8 KV heads, G 8, head_dim 128 on 256 CUs) must fit the
 * array; a larger batch returns PA_ERR_WORKSPACE before anything is launched (use pa_decode).
 * The whole batch is split statically (no dynamic chunks, no dynamic tail), so results equal
 * pa_decode's bit for bit when pa_decode's dynamic tail is off (PA_DECODE_TAIL_Q10 = 0), and
 * agree with them within fp32 rounding otherwise.
 * Every call on a device uses that device's one array, and nothing in it has to start at a set
 * value: calls that overlap in time on one device (different streams, or threads) race on it and
 * give unspecified results; calls ordered on one stream are safe.  Other errors as pa_decode.
 */
#define PA_DECODE_NO_ALLOC_SCRATCH_BYTES (32u << 20)
pa_status_t pa_decode_no_alloc(void* out, const void* query, const void* key_cache,
                               const void* value_cache, int64_t num_blocks,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                               int32_t max_seq_len, float scale, void* stream);

/*
 * Cascade decode for sequences that share a prompt (copy-on-write rollouts).
 *
 * Source: sequences continuing one prompt reference the same physical blocks for it ("Inference
 * optimization" lesson, section "Paged attention"; vLLM-on-H100 article, PagedAttention section:
 * 8 or 16 rollouts of one prompt share its pages).  The result is exactly pa_decode's; only the
 * order of the work changes: the shared prompt's keys are read once per group, as one matrix-core
 * chunk of all the group's query rows (the chunked-prefill kernel, non-causal), each sequence's
 * own later tokens are attended by the decode kernel, and the two softmax states of every row are
 * combined.
 *
 *   group_start    int32 [num_groups+1]: group i is sequences group_start[i] .. group_start[i+1]-1,
 *                  group_start[0] == 0, group_start[num_groups] == num_seqs, non-decreasing
 *   prefix_lens    int32 [num_seqs]: tokens a sequence shares with its group, a multiple of
 *                  block_size (0: nothing shared), the same for every member of a group and
 *                  <= that sequence's seq_lens entry; members' first prefix_len / block_size table
 *                  entries must be those of the group's first member (otherwise results are
 *                  unspecified, never an access outside the buffers)
 *   max_group_size host-side bound of every group's size (1 <= max_group_size <= num_seqs)
 *   max_prefix_len host-side bound of prefix_lens (0 <= max_prefix_len <= max_seq_len)
 *   workspace      at least pa_decode_cascade_workspace_bytes(...) bytes, 256-byte aligned,
 *                  zero-filled before its first use and reusable by later calls on one stream
 * Other arguments, limits and errors as pa_decode (bf16 pools).  Outputs are fp32-accumulated and
 * rounded to bf16 once.
 */
size_t pa_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_groups,
                                         int32_t max_group_size, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_prefix_len);
pa_status_t pa_decode_cascade(void* out, const void* query, const void* key_cache,
                              const void* value_cache, int64_t num_blocks,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              const int32_t* group_start, const int32_t* prefix_lens,
                              int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                              int32_t max_prefix_len, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, float scale, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * pa_decode_cascade_fp8 — pa_decode_cascade over FP8 pools (pa_reshape_and_cache_fp8, same
 * k_scale and v_scale): the result of pa_decode_fp8.  Same workspace size query.
 */
pa_status_t pa_decode_cascade_fp8(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, int64_t num_blocks,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens,
                                  int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                                  int32_t max_prefix_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                                  float k_scale, float v_scale, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace pa_prefill_chunk needs for this batch shape on the current device; 0 means
 * none (workspace may then be NULL).  Long contexts are split into key ranges whose partial softmax
 * states are combined afterwards; the workspace holds those states.  It needs no initialisation.
 */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seq_len);

/*
 * pa_prefill_chunk — causal attention of a chunk of query tokens per sequence over the
 * sequence's paged context (chunked prefill).
 *
 * Source: long prompts are processed in fixed-size chunks (512 tokens by default) that attend to
 * everything cached before them and are batched with decode tokens ("Serving engine internals",
 * section "Chunked prefill protects the TTFT tail"); the mask is Step 2's causal mask aligned to
 * the end of the key range ("Inference optimization", Build it, Step 2), so chunk row t (0-based)
 * of a sequence of L cached tokens with q_len chunk rows sees keys 0 .. L - q_len + t.
 *
 *   out            bf16 [total_q][num_q_heads][head_dim] (written; must not alias inputs)
 *   query          bf16 [total_q][num_q_heads][head_dim]; sequence i owns rows
 *                  query_start_loc[i] .. query_start_loc[i+1]-1
 *   key_cache, value_cache, num_blocks  as for pa_decode (ids are clamped into the pool)
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]; entries for keys < L are read
 *   query_start_loc int32 [num_seqs+1], non-decreasing, query_start_loc[num_seqs] == total_q
 *   seq_lens       int32 [num_seqs]; L_i = prior context + chunk length; the chunk's own K/V must
 *                  already be in the cache (pa_reshape_and_cache first); q_len_i <= L_i <=
 *                  max_seq_len (other values give unspecified results, never an access outside
 *                  the buffers)
 *   max_q_len      host-side upper bound of the chunk lengths (<= max_seq_len)
 *   max_seq_len    host-side upper bound of seq_lens (<= max_blocks_per_seq*block_size)
 *   scale          softmax scale (> 0)
 *   workspace      at least pa_prefill_workspace_bytes(...) bytes
 * Both contractions run on bf16 matrix cores with fp32 accumulation; output rounded to bf16
 * (nearest even).  Same head_dim / group limits as pa_decode.
 */
pa_status_t pa_prefill_chunk(void* out, const void* query, const void* key_cache,
                             const void* value_cache, int64_t num_blocks,
                             const int32_t* block_tables, const int32_t* query_start_loc,
                             const int32_t* seq_lens, int32_t num_seqs, int32_t total_q,
                             int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                             int32_t max_seq_len, float scale, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * pa_prefill_chunk_fp8 — pa_prefill_chunk over FP8 pools written by pa_reshape_and_cache_fp8
 * (the chunk's own K/V included), with the same k_scale and v_scale.  The attention is that of
 * pa_prefill_chunk on the dequantised cache; codes are widened to bf16 exactly before both
 * matrix-core products.  Workspace (same size query), limits and errors as pa_prefill_chunk;
 * k_scale and v_scale must be finite and positive.
 */
pa_status_t pa_prefill_chunk_fp8(void* out, const void* query, const void* key_cache,
                                 const void* value_cache, int64_t num_blocks,
                                 const int32_t* block_tables, const int32_t* query_start_loc,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t total_q,
                                 int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                 int32_t max_seq_len, float scale, float k_scale, float v_scale,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_mixed_step — one chunked-prefill batch step: a prefill-chunk call and a decode call run side
 * by side, the decode on `side_stream`, so decode's HBM-bound work overlaps the matrix-core-bound
 * chunk.
 *
 * Source: a serving step batches the slices of a long prompt with the decode tokens of the other
 * requests ("Serving engine internals" lesson, chunked-prefill section: the batch is one GPU
 * call).  Write every new token's K/V first (pa_reshape_and_cache on `stream`).
 *
 *   prefill, decode  the arguments of pa_prefill_chunk / pa_decode (or their FP8 forms when
 *                    kv_fp8 is nonzero, with k_scale and v_scale).  The two outputs and the
 *                    workspace bytes each half uses (its *_workspace_bytes query) must not
 *                    overlap one another: PA_ERR_INVALID_ARG otherwise.  A half with no sequences
 *                    launches nothing and may pass null pointers, as the single calls allow
 *   stream           the caller's stream: both halves start after the work already on it, and
 *                    later work on it waits for both
 *   side_stream      a second stream of the same device at default priority; NULL or `stream`
 *                    runs the two calls one after the other on `stream`
 * Both halves are validated before either is launched; errors as the two calls.  Results are
 * those of the two calls made one after the other, bit for bit.  The library keeps one pair of
 * events per thread and device for the fork and the join (created on first use).
 */
typedef struct pa_prefill_args {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  int64_t num_blocks;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  const int32_t* seq_lens;
  int32_t num_seqs, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size;
  int32_t max_blocks_per_seq, max_seq_len;
  float scale;
  int32_t kv_fp8;
  float k_scale, v_scale;
  void* workspace;
  size_t workspace_bytes;
} pa_prefill_args;

typedef struct pa_decode_args {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  int64_t num_blocks;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  int32_t max_seq_len;
  float scale;
  int32_t kv_fp8;
  float k_scale, v_scale;
  void* workspace;
  size_t workspace_bytes;
} pa_decode_args;

pa_status_t pa_mixed_step(const pa_prefill_args* prefill, const pa_decode_args* decode,
                          void* stream, void* side_stream);

/*
 * Measurement: a plain streaming read, the HBM read ceiling the decode kernel is compared
 * against.  pa_stream_read reads `bytes` of `src` (a multiple of 16, 16-byte aligned) once, in
 * order, with 16-byte non-temporal loads, and writes one XOR word per workgroup to `sink`
 * (at least pa_stream_read_sink_words() words; 0 means the device could not be queried).
 * Errors as elsewhere; PA_ERR_WORKSPACE for a short sink.  Kernel name for tracing: "stream_read".
 */
int32_t pa_stream_read_sink_words(void);
pa_status_t pa_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                           void* stream);

/*
 * Kernel timing (tracing).  While enabled, every kernel the library launches is bracketed by a
 * pair of HIP events recorded on its stream.  pa_trace_read synchronises on the recorded events,
 * returns the number of launches and their summed duration (milliseconds) for one kernel name, and
 * forgets those records.  Kernel names: "reshape_and_cache", "copy_blocks", "decode_partition",
 * "decode_merge", "prefill_chunk", "prefill_merge", "stream_read".  Events are host-side driver objects; no
 * device memory is used.
 */
pa_status_t pa_trace_enable(int32_t enable);
pa_status_t pa_trace_read(const char* kernel_name, int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_PA_H */
