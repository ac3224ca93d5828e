// C ABI of libpagedattn: argument validation, launch geometry, workspace sizing, kernel tracing.
// Every check that host scalars allow happens here, before any launch.

#include "../../include/pa.h"
#include "cascade.h"
#include "copy_blocks.h"
#include "stream_read.h"
#include "pa_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

namespace {

thread_local std::string g_last_error;

pa_status_t fail(pa_status_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status_t fail(pa_status_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

pa_status_t ok() {
  g_last_error.clear();
  return PA_OK;
}

pa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256; }
bool supported_block(int bs) { return bs == 16 || bs == 32; }

// Group size (query heads per KV head) must be a power of two with group*head_dim <= 1024.
bool supported_group(int g, int d) { return g >= 1 && g <= 16 && (g & (g - 1)) == 0 && g * d <= 1024; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Common validation of the attention entry points.
pa_status_t check_attention_shape(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_blocks_per_seq,
                                  int32_t max_seq_len, float scale) {
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "head counts must be positive (got %d query, %d kv)",
                num_q_heads, num_kv_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", head_dim);
  if (!supported_block(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not in {16,32}", block_size);
  const int g = num_q_heads / num_kv_heads;
  if (!supported_group(g, head_dim))
    return fail(PA_ERR_UNSUPPORTED, "group size %d with head_dim %d not supported", g, head_dim);
  if (max_blocks_per_seq <= 0 || max_seq_len < 0)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d / max_seq_len %d out of range",
                max_blocks_per_seq, max_seq_len);
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID_ARG, "max_seq_len %d exceeds max_blocks_per_seq*block_size %lld",
                max_seq_len, (long long)max_blocks_per_seq * block_size);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "scale must be finite and positive");
  return PA_OK;
}

// ---------------------------------------------------------------------------------------------
// Tracing
std::atomic<bool> g_trace_on{false};
std::mutex g_trace_mu;
struct TraceRec {
  std::string name;
  hipEvent_t start, stop;
};
std::vector<TraceRec> g_trace_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  // Trace events only time kernels, so they skip the system-scope release (an L2 write-back)
  // that a default event performs when it is recorded between two launches.
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace pa {

TraceScope::TraceScope(const char* name, hipStream_t stream) : slot_(-1), stream_(stream) {
  if (!g_trace_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_trace_mu);
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return;
  if (hipEventRecord(a, stream) != hipSuccess) return;
  g_trace_recs.push_back({name, a, b});
  slot_ = (int)g_trace_recs.size() - 1;
}

TraceScope::~TraceScope() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lk(g_trace_mu);
  (void)hipEventRecord(g_trace_recs[slot_].stop, stream_);
}

}  // namespace pa

namespace {

// Launch tunables: name, default, allowed range.  The environment is read once, when the table is
// first used; pa_set_tunable changes a value afterwards.
struct TunableDef {
  const char* name;
  int dflt, lo, hi;
};
constexpr TunableDef kTunableDefs[pa::kNumTunables] = {
    {"PA_DECODE_PREFETCH", 1, 0, 2},    {"PA_DECODE_PREFETCH_FP8", 1, 1, 2},
    {"PA_DECODE_MFMA", 1, 0, 1},        {"PA_DECODE_QUAD", 1, 0, 1},
    {"PA_DECODE_PIECE_COST", 4, 0, 64}, {"PA_DECODE_WORKERS", 0, 0, 1 << 20},
    {"PA_DECODE_STATIC_Q10", 1024, 512, 1024}, {"PA_DECODE_CHUNK", 4, 1, 256},
    {"PA_PREFILL_SPLITS", 0, 0, 16},    {"PA_DECODE_TAIL_Q10", 0, 0, 512},
    {"PA_DECODE_TAIL_Q10_FP8", 0, 0, 512}, {"PA_DECODE_TAIL_CHUNK", 12, 1, 256},
};

std::atomic<int>* tunable_values() {
  static std::atomic<int> values[pa::kNumTunables];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int i = 0; i < pa::kNumTunables; ++i) {
      const TunableDef& d = kTunableDefs[i];
      int v = d.dflt;
      if (const char* e = std::getenv(d.name); e && *e) {
        char* end = nullptr;
        const long x = std::strtol(e, &end, 10);
        if (end && *end == '\0' && x >= d.lo && x <= d.hi) v = (int)x;
      }
      values[i].store(v);
    }
  });
  return values;
}

int tunable_index(const char* name) {
  for (int i = 0; i < pa::kNumTunables; ++i)
    if (std::strcmp(kTunableDefs[i].name, name) == 0) return i;
  return -1;
}

}  // namespace

namespace pa {
int tunable(Tunable t) { return tunable_values()[t].load(std::memory_order_relaxed); }
}  // namespace pa

extern "C" {

pa_status_t pa_set_tunable(const char* name, int32_t value) {
  if (!name) return fail(PA_ERR_NULL_POINTER, "null tunable name");
  const int i = tunable_index(name);
  if (i < 0) return fail(PA_ERR_INVALID_ARG, "unknown tunable %s", name);
  const TunableDef& d = kTunableDefs[i];
  if (value < d.lo || value > d.hi)
    return fail(PA_ERR_INVALID_ARG, "%s must be in [%d, %d] (got %d)", name, d.lo, d.hi, value);
  tunable_values()[i].store(value);
  return ok();
}

pa_status_t pa_get_tunable(const char* name, int32_t* value) {
  if (!name || !value) return fail(PA_ERR_NULL_POINTER, "null argument");
  const int i = tunable_index(name);
  if (i < 0) return fail(PA_ERR_INVALID_ARG, "unknown tunable %s", name);
  *value = tunable_values()[i].load();
  return ok();
}

int32_t pa_version(void) { return 200; }

const char* pa_last_error(void) { return g_last_error.c_str(); }

pa_status_t pa_trace_enable(int32_t enable) {
  g_trace_on.store(enable != 0);
  return ok();
}

pa_status_t pa_trace_read(const char* kernel_name, int32_t* launches, double* total_ms) {
  if (!kernel_name || !launches || !total_ms) return fail(PA_ERR_NULL_POINTER, "null argument");
  std::lock_guard<std::mutex> lk(g_trace_mu);
  int n = 0;
  double ms = 0.0;
  std::vector<TraceRec> keep;
  for (auto& r : g_trace_recs) {
    if (r.name != kernel_name) {
      keep.push_back(r);
      continue;
    }
    hipError_t e = hipEventSynchronize(r.stop);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess) return hip_status(e, "pa_trace_read");
    ms += t;
    ++n;
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_trace_recs.swap(keep);
  *launches = n;
  *total_ms = ms;
  return ok();
}

}  // extern "C"

namespace {

bool valid_kv_scale(float s) { return std::isfinite(s) && s > 0.f; }

pa_status_t reshape_impl(const void* key, const void* value, int64_t kv_token_stride,
                         void* key_cache, void* value_cache, const int64_t* slot_mapping,
                         int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, bool fp8, float k_scale,
                         float v_scale, void* stream) {
  if (fp8 && (!valid_kv_scale(k_scale) || !valid_kv_scale(v_scale)))
    return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d <= 0", num_kv_heads);
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", head_dim);
  if (!supported_block(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not in {16,32}", block_size);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks %lld <= 0", (long long)num_blocks);
  if (kv_token_stride < (int64_t)num_kv_heads * head_dim || kv_token_stride % 8 != 0)
    return fail(PA_ERR_INVALID_ARG, "kv_token_stride %lld must be >= %d and a multiple of 8",
                (long long)kv_token_stride, num_kv_heads * head_dim);
  if (num_tokens == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_NULL_POINTER, "null pointer argument");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer (need 16 bytes for bf16 arrays)");
  pa::ReshapeParams p{};
  p.kv_fp8 = fp8;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.key = static_cast<const uint16_t*>(key);
  p.value = static_cast<const uint16_t*>(value);
  p.token_stride = kv_token_stride;
  p.kpool = static_cast<uint16_t*>(key_cache);
  p.vpool = static_cast<uint16_t*>(value_cache);
  p.slots = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  return hip_status(pa::launch_reshape(p, static_cast<hipStream_t>(stream)), "reshape_and_cache");
}

}  // namespace

extern "C" {

pa_status_t pa_reshape_and_cache(const void* key, const void* value, int64_t kv_token_stride,
                                 void* key_cache, void* value_cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, void* stream) {
  return reshape_impl(key, value, kv_token_stride, key_cache, value_cache, slot_mapping,
                      num_tokens, num_kv_heads, head_dim, block_size, num_blocks, false, 1.f, 1.f,
                      stream);
}

pa_status_t pa_reshape_and_cache_fp8(const void* key, const void* value, int64_t kv_token_stride,
                                     void* key_cache, void* value_cache,
                                     const int64_t* slot_mapping, int32_t num_tokens,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int64_t num_blocks, float k_scale, float v_scale,
                                     void* stream) {
  return reshape_impl(key, value, kv_token_stride, key_cache, value_cache, slot_mapping,
                      num_tokens, num_kv_heads, head_dim, block_size, num_blocks, true, k_scale,
                      v_scale, stream);
}

pa_status_t pa_copy_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                           const int64_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, void* stream) {
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs %d < 0", num_pairs);
  if (num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d <= 0", num_kv_heads);
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", head_dim);
  if (!supported_block(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not in {16,32}", block_size);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks %lld <= 0", (long long)num_blocks);
  if (num_pairs == 0) return ok();
  if (!key_cache || !value_cache || !block_mapping)
    return fail(PA_ERR_NULL_POINTER, "null pointer argument");
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(block_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer (need 16 bytes for the pools)");
  pa::CopyBlocksParams p{};
  p.kpool = static_cast<uint16_t*>(key_cache);
  p.vpool = static_cast<uint16_t*>(value_cache);
  p.mapping = block_mapping;
  p.num_blocks = num_blocks;
  p.block_vec16 = (int64_t)num_kv_heads * block_size * head_dim / 8;
  p.num_pairs = num_pairs;
  return hip_status(pa::launch_copy_blocks(p, static_cast<hipStream_t>(stream)), "copy_blocks");
}

int32_t pa_stream_read_sink_words(void) { return pa::stream_read_grid(); }

pa_status_t pa_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                           void* stream) {
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(PA_ERR_NULL_POINTER, "null pointer argument");
  if (bytes % 16 || !aligned(src, 16) || !aligned(sink, 4))
    return fail(PA_ERR_INVALID_ARG, "bytes must be a multiple of 16 and src 16-byte aligned");
  const int grid = pa::stream_read_grid();
  if (grid <= 0) return fail(PA_ERR_HIP, "cannot query the device");
  if (sink_words < (size_t)grid)
    return fail(PA_ERR_WORKSPACE, "sink of %zu words given, %d needed", sink_words, grid);
  return hip_status(pa::launch_stream_read(src, bytes, sink, grid, static_cast<hipStream_t>(stream)),
                    "stream_read");
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len) {
  (void)max_seq_len;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return 0;
  const int g = num_q_heads / num_kv_heads;
  if (!supported_head_dim(head_dim) || !supported_group(g, head_dim)) return 0;
  return pa::decode_workspace(num_seqs, num_kv_heads, head_dim, g, false).bytes;
}

}  // extern "C"

namespace {

pa_status_t decode_impl(void* out, const void* query, const void* key_cache,
                        const void* value_cache, int64_t num_blocks, const int32_t* block_tables,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                        bool fp8, float k_scale, float v_scale, void* workspace,
                        size_t workspace_bytes, void* stream,
                        const int32_t* skip_lens = nullptr, float* state_ml = nullptr,
                        float* state_acc = nullptr, int state_stride = 0, int state_split = 0,
                        bool validate_only = false, bool static_layout = false,
                        bool state_final = false) {
  if (fp8 && (!valid_kv_scale(k_scale) || !valid_kv_scale(v_scale)))
    return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (fp8 && !std::isfinite(scale * k_scale))
    return fail(PA_ERR_INVALID_ARG, "scale * k_scale overflows");
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
  pa_status_t st = check_attention_shape(num_q_heads, num_kv_heads, head_dim, block_size,
                                         max_blocks_per_seq, max_seq_len, scale);
  if (st != PA_OK) return st;
  if (num_blocks <= 0 || num_blocks > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_blocks %lld out of range", (long long)num_blocks);
  if (num_seqs == 0) return ok();
  if (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens)
    return fail(PA_ERR_NULL_POINTER, "null pointer argument");
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer (need 16 bytes for bf16 arrays)");
  if (out == query) return fail(PA_ERR_INVALID_ARG, "out must not alias query");
  const int g = num_q_heads / num_kv_heads;
  // static_layout: no dynamic-chunk slots (the whole batch is split statically).
  const pa::DecodeWorkspace wl =
      pa::decode_workspace(num_seqs, num_kv_heads, head_dim, g, fp8, !static_layout);
  if (wl.workers <= 0)
    return fail(PA_ERR_HIP, "cannot query the device for the decode launch shape");
  if (static_layout && workspace_bytes < wl.bytes)
    return fail(PA_ERR_WORKSPACE,
                "this batch needs %zu bytes of decode scratch, more than the %zu the library "
                "holds for pa_decode_no_alloc (use pa_decode with a workspace)",
                wl.bytes, workspace_bytes);
  if (!workspace || workspace_bytes < wl.bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                wl.bytes);
  if (!aligned(workspace, 16)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  pa::DecodeParams p{};
  p.out = static_cast<uint16_t*>(out);
  p.query = static_cast<const uint16_t*>(query);
  p.kpool = static_cast<const uint16_t*>(key_cache);
  p.vpool = static_cast<const uint16_t*>(value_cache);
  p.block_tables = block_tables;
  p.skip_lens = skip_lens;  // per-sequence prefix left out (cascade), or none
  p.state_ml = state_ml;
  p.state_acc = state_acc;
  p.state_stride = state_stride;
  p.state_split = state_split;
  p.state_final = state_final;
  p.seq_lens = seq_lens;
  p.num_blocks = num_blocks;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_workers = wl.workers;
  p.dyn_cap = wl.dyn_cap;
  p.chunk_steps = pa::tunable(pa::kTuneDecodeChunk);
  p.static_frac_q10 = static_layout ? 1024 : pa::tunable(pa::kTuneDecodeStaticQ10);
  // Head quads (four KV heads per workgroup worker) need a multiple of four KV heads.
  p.quad = p.static_frac_q10 == 1024 && num_kv_heads % 4 == 0 &&
           pa::tunable(pa::kTuneDecodeQuad) != 0;
  p.piece_cost = pa::tunable(pa::kTuneDecodePieceCost);
  // The dynamic tail needs the workspace's chunk counter, so the fixed-scratch entry point (which
  // leaves nothing in its scratch to start at zero) keeps the static split.
  p.tail_q10 = (p.quad && !static_layout)
                   ? pa::tunable(fp8 ? pa::kTuneDecodeTailQ10Fp8 : pa::kTuneDecodeTailQ10)
                   : 0;
  p.tail_chunk = pa::tunable(pa::kTuneDecodeTailChunk);
  p.len_cap = max_seq_len;
  // FP8: the K scale joins the softmax scale and the V scale multiplies the outputs.
  p.scale_log2 = (fp8 ? scale * k_scale : scale) * 1.4426950408889634f;
  p.kv_fp8 = fp8;
  p.v_scale = fp8 ? v_scale : 1.f;
  char* base = static_cast<char*>(workspace);
  p.counter = reinterpret_cast<unsigned*>(base + wl.counter_off);
  p.unit_info = reinterpret_cast<int2*>(base + wl.info_off);
  p.partials = reinterpret_cast<float*>(base + wl.partials_off);
  if (validate_only) return ok();
  return hip_status(pa::launch_decode(p, static_cast<hipStream_t>(stream)), "decode");
}

}  // namespace

extern "C" {

pa_status_t pa_decode(void* out, const void* query, const void* key_cache,
                      const void* value_cache, int64_t num_blocks, const int32_t* block_tables,
                      const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, query, key_cache, value_cache, num_blocks, block_tables, seq_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, max_seq_len, scale, false, 1.f, 1.f, workspace,
                     workspace_bytes, stream);
}

pa_status_t pa_decode_fp8(void* out, const void* query, const void* key_cache,
                          const void* value_cache, int64_t num_blocks,
                          const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                          float scale, float k_scale, float v_scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_impl(out, query, key_cache, value_cache, num_blocks, block_tables, seq_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, max_seq_len, scale, true, k_scale, v_scale, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// pa_decode_no_alloc: pa_decode whose scratch (unit table, partial states, chunk counter) is a
// fixed device array of the library instead of a caller workspace.  Each device holds its own
// copy of the array for as long as the process runs; host code reaches a device's copy only
// through the address hipGetSymbolAddress returns for it with that device current (the array's
// name on the host is a stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[PA_DECODE_NO_ALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up on the first call that device
// makes and kept.
pa_status_t scratch_on_current_device(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "decode_no_alloc (device)");
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "decode_no_alloc (scratch address)");
    if (!p) return fail(PA_ERR_HIP, "decode_no_alloc: no scratch address on device %d", dev);
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_decode_no_alloc(void* out, const void* query, const void* key_cache,
                               const void* value_cache, int64_t num_blocks,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                               int32_t max_seq_len, float scale, void* stream) {
  // Host-side checks first (the scratch stands in as a 256-byte aligned placeholder of its full
  // size), so a rejected call touches no device state.
  const size_t cap = PA_DECODE_NO_ALLOC_SCRATCH_BYTES;
  void* ws = reinterpret_cast<void*>(uintptr_t{256});
  pa_status_t st = decode_impl(out, query, key_cache, value_cache, num_blocks, block_tables,
                               seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                               block_size, max_blocks_per_seq, max_seq_len, scale, false, 1.f, 1.f,
                               ws, cap, stream, nullptr, nullptr, nullptr, 0, 0,
                               /*validate_only=*/true, /*static_layout=*/true);
  if (st != PA_OK || num_seqs == 0) return st;
  if ((st = scratch_on_current_device(&ws)) != PA_OK) return st;
  // Nothing in the scratch has to start at zero: with the static split every unit's table entry
  // and every partial slot is written before it is read, and the chunk counter is unused.
  return decode_impl(out, query, key_cache, value_cache, num_blocks, block_tables, seq_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, max_seq_len, scale, false, 1.f, 1.f, ws, cap, stream,
                     nullptr, nullptr, nullptr, 0, 0, /*validate_only=*/false,
                     /*static_layout=*/true);
}

}  // extern "C"

namespace {

// Workspace of pa_decode_cascade: split states in the prefill layout (prompt splits plus one for
// the tails) for every (sequence, query head) row, then the decode workspace.
struct CascadeLayout {
  pa::PrefillSplit split;
  size_t ml_bytes, acc_off, dec_off, bytes;
};

CascadeLayout cascade_layout(int num_seqs, int num_groups, int max_group_size, int num_q_heads,
                             int num_kv_heads, int head_dim, int prefix_len) {
  CascadeLayout c{};
  const int g = num_q_heads / num_kv_heads;
  // The shared prompt is read by few query rows per group, so its chunk is bandwidth-bound: one
  // workgroup per CU (4 ranges at 8 groups of 16 rollouts: 95.8 us against 100.7 us with the
  // two-per-CU split, whose merge reads twice the states).
  c.split = pa::prompt_split(num_groups, max_group_size, num_kv_heads, g, head_dim, prefix_len);
  const size_t slots = (size_t)num_seqs * num_q_heads * (c.split.splits + 1);
  c.ml_bytes = align_up(slots * 2 * sizeof(float), 256);
  c.acc_off = c.ml_bytes;
  c.dec_off = align_up(c.acc_off + slots * head_dim * sizeof(float), 256);
  const size_t dec = pa::decode_workspace(num_seqs, num_kv_heads, head_dim, g, false).bytes;
  c.bytes = dec ? c.dec_off + dec : 0;
  return c;
}

}  // namespace

extern "C" {

size_t pa_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_groups,
                                         int32_t max_group_size, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_prefix_len) {
  if (num_seqs <= 0 || num_groups <= 0 || max_group_size <= 0 || max_prefix_len < 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return 0;
  const int g = num_q_heads / num_kv_heads;
  if (!supported_head_dim(head_dim) || !supported_group(g, head_dim)) return 0;
  return cascade_layout(num_seqs, num_groups, max_group_size, num_q_heads, num_kv_heads, head_dim,
                        max_prefix_len).bytes;
}

}  // extern "C"

namespace {

pa_status_t cascade_impl(void* out, const void* query, const void* key_cache,
                         const void* value_cache, int64_t num_blocks, const int32_t* block_tables,
                         const int32_t* seq_lens, const int32_t* group_start,
                         const int32_t* prefix_lens, int32_t num_seqs, int32_t num_groups,
                         int32_t max_group_size, int32_t max_prefix_len, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, int32_t max_seq_len, float scale, bool fp8,
                         float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (num_seqs < 0 || num_groups < 0 || max_group_size < 0)
    return fail(PA_ERR_INVALID_ARG, "negative size (num_seqs %d, num_groups %d, max_group_size %d)",
                num_seqs, num_groups, max_group_size);
  pa_status_t st = check_attention_shape(num_q_heads, num_kv_heads, head_dim, block_size,
                                         max_blocks_per_seq, max_seq_len, scale);
  if (st != PA_OK) return st;
  if (fp8 && (!valid_kv_scale(k_scale) || !valid_kv_scale(v_scale)))
    return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (fp8 && !std::isfinite(scale * k_scale))
    return fail(PA_ERR_INVALID_ARG, "scale * k_scale overflows");
  if (num_blocks <= 0 || num_blocks > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_blocks %lld out of range", (long long)num_blocks);
  if (max_prefix_len < 0 || max_prefix_len > max_seq_len)
    return fail(PA_ERR_INVALID_ARG, "max_prefix_len %d must be in [0, max_seq_len %d]",
                max_prefix_len, max_seq_len);
  if (num_seqs == 0) return ok();
  if (num_groups == 0 || max_group_size == 0 || max_group_size > num_seqs)
    return fail(PA_ERR_INVALID_ARG, "num_groups %d / max_group_size %d do not cover %d sequences",
                num_groups, max_group_size, num_seqs);
  if (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens || !group_start ||
      !prefix_lens)
    return fail(PA_ERR_NULL_POINTER, "null pointer argument");
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(block_tables, 4) || !aligned(seq_lens, 4) ||
      !aligned(group_start, 4) || !aligned(prefix_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer (need 16 bytes for the bf16 arrays)");
  if (out == query) return fail(PA_ERR_INVALID_ARG, "out must not alias query");
  const CascadeLayout c = cascade_layout(num_seqs, num_groups, max_group_size, num_q_heads,
                                         num_kv_heads, head_dim, max_prefix_len);
  if (c.bytes == 0) return fail(PA_ERR_HIP, "cannot query the device for the launch shapes");
  if (!workspace || workspace_bytes < c.bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                c.bytes);
  if (!aligned(workspace, 256)) return fail(PA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  float* ml = reinterpret_cast<float*>(ws);
  float* acc = reinterpret_cast<float*>(ws + c.acc_off);
  const int S = c.split.splits;
  hipStream_t hs = static_cast<hipStream_t>(stream);

  // 1. Each group's shared prompt, once: the group's decode queries are one non-causal chunk over
  //    its first prefix_lens[first member] tokens, read through its first member's table row.
  pa::PrefillParams a{};
  a.out = static_cast<uint16_t*>(out);
  a.query = static_cast<const uint16_t*>(query);
  a.kpool = static_cast<const uint16_t*>(key_cache);
  a.vpool = static_cast<const uint16_t*>(value_cache);
  a.block_tables = block_tables;
  a.query_start_loc = group_start;
  a.seq_lens = prefix_lens;
  a.ws_ml = ml;
  a.ws_acc = acc;
  a.num_blocks = num_blocks;
  a.num_seqs = num_groups;
  a.total_q = num_seqs;
  a.max_q_len = max_group_size;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seq_len = max_prefix_len;
  a.splits = S;
  a.split_keys = S > 1 ? c.split.split_keys : std::max(max_prefix_len, 1);
  a.scale_log2 = (fp8 ? scale * k_scale : scale) * 1.4426950408889634f;
  a.noncausal = 1;
  a.from_first_row = 1;
  a.ws_splits = S + 1;
  a.defer_merge = 1;
  a.kv_fp8 = fp8;
  a.v_scale = fp8 ? v_scale : 1.f;
  if (S > 1 && a.split_keys % 32)
    return fail(PA_ERR_HIP, "internal: prompt split of %d keys", a.split_keys);
  // The tails' decode is checked before anything is launched.
  st = decode_impl(out, query, key_cache, value_cache, num_blocks, block_tables, seq_lens,
                   num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                   max_seq_len, scale, fp8, k_scale, v_scale, ws + c.dec_off,
                   workspace_bytes - c.dec_off, stream, prefix_lens, ml, acc, S + 1, S, true);
  if (st != PA_OK) return st;
  hipError_t e = pa::launch_prefill(a, hs);
  if (e != hipSuccess) return hip_status(e, "decode_cascade (prompt)");
  // 2. Each sequence's own tokens past its prompt, as decode with the prompt's blocks skipped.
  //    A tail taken whole by one wave leaves its state in the last split; the decode's merge
  //    then combines the prompt splits with each row's tail and writes the output.
  return decode_impl(out, query, key_cache, value_cache, num_blocks, block_tables, seq_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, max_seq_len, scale, fp8, k_scale, v_scale,
                     ws + c.dec_off, workspace_bytes - c.dec_off, stream, prefix_lens, ml, acc,
                     S + 1, S, false, false, true);
}

}  // namespace

extern "C" {

pa_status_t pa_decode_cascade(void* out, const void* query, const void* key_cache,
                              const void* value_cache, int64_t num_blocks,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              const int32_t* group_start, const int32_t* prefix_lens,
                              int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                              int32_t max_prefix_len, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return cascade_impl(out, query, key_cache, value_cache, num_blocks, block_tables, seq_lens,
                      group_start, prefix_lens, num_seqs, num_groups, max_group_size,
                      max_prefix_len, num_q_heads, num_kv_heads, head_dim, block_size,
                      max_blocks_per_seq, max_seq_len, scale, false, 1.f, 1.f, workspace,
                      workspace_bytes, stream);
}

pa_status_t pa_decode_cascade_fp8(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, int64_t num_blocks,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens,
                                  int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                                  int32_t max_prefix_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                                  float k_scale, float v_scale, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return cascade_impl(out, query, key_cache, value_cache, num_blocks, block_tables, seq_lens,
                      group_start, prefix_lens, num_seqs, num_groups, max_group_size,
                      max_prefix_len, num_q_heads, num_kv_heads, head_dim, block_size,
                      max_blocks_per_seq, max_seq_len, scale, true, k_scale, v_scale, workspace,
                      workspace_bytes, stream);
}

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seq_len) {
  if (num_seqs <= 0 || total_q <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads)
    return 0;
  const int g = num_q_heads / num_kv_heads;
  if (!supported_head_dim(head_dim) || !supported_group(g, head_dim)) return 0;
  const pa::PrefillSplit sp =
      pa::prefill_split(num_seqs, max_q_len, num_kv_heads, g, head_dim, max_seq_len);
  if (sp.splits <= 1) return 0;
  const size_t rows = (size_t)total_q * num_q_heads * sp.splits;
  return align_up(rows * 2 * sizeof(float), 256) + rows * head_dim * sizeof(float);
}

}  // extern "C"

namespace {

pa_status_t prefill_impl(void* out, const void* query, const void* key_cache,
                         const void* value_cache, int64_t num_blocks,
                         const int32_t* block_tables, const int32_t* query_start_loc,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t total_q,
                         int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                         int32_t max_seq_len, float scale, bool fp8, float k_scale,
                         float v_scale, void* workspace, size_t workspace_bytes, void* stream,
                         bool validate_only = false, bool concurrent = false) {
  if (fp8 && (!valid_kv_scale(k_scale) || !valid_kv_scale(v_scale)))
    return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (fp8 && !std::isfinite(scale * k_scale))
    return fail(PA_ERR_INVALID_ARG, "scale * k_scale overflows");
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0)
    return fail(PA_ERR_INVALID_ARG, "negative size (num_seqs %d, total_q %d, max_q_len %d)",
                num_seqs, total_q, max_q_len);
  pa_status_t st = check_attention_shape(num_q_heads, num_kv_heads, head_dim, block_size,
                                         max_blocks_per_seq, max_seq_len, scale);
  if (st != PA_OK) return st;
  if (num_blocks <= 0 || num_blocks > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_blocks %lld out of range", (long long)num_blocks);
  if (max_q_len > max_seq_len)
    return fail(PA_ERR_INVALID_ARG, "max_q_len %d exceeds max_seq_len %d", max_q_len, max_seq_len);
  if (num_seqs == 0 || total_q == 0) return ok();
  if (!out || !query || !key_cache || !value_cache || !block_tables || !query_start_loc ||
      !seq_lens)
    return fail(PA_ERR_NULL_POINTER, "null pointer argument");
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(block_tables, 4) || !aligned(query_start_loc, 4) ||
      !aligned(seq_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer (need 16 bytes for bf16 arrays)");
  if (out == query) return fail(PA_ERR_INVALID_ARG, "out must not alias query");
  const int g = num_q_heads / num_kv_heads;
  const size_t need = pa_prefill_workspace_bytes(num_seqs, total_q, max_q_len, num_q_heads,
                                                 num_kv_heads, head_dim, max_seq_len);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (need > 0 && !aligned(workspace, 16))
    return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  const pa::PrefillSplit sp =
      pa::prefill_split(num_seqs, max_q_len, num_kv_heads, g, head_dim, max_seq_len);
  pa::PrefillParams p{};
  p.out = static_cast<uint16_t*>(out);
  p.query = static_cast<const uint16_t*>(query);
  p.kpool = static_cast<const uint16_t*>(key_cache);
  p.vpool = static_cast<const uint16_t*>(value_cache);
  p.block_tables = block_tables;
  p.query_start_loc = query_start_loc;
  p.seq_lens = seq_lens;
  p.num_blocks = num_blocks;
  p.num_seqs = num_seqs;
  p.total_q = total_q;
  p.max_q_len = max_q_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.splits = need > 0 ? sp.splits : 1;
  p.split_keys = need > 0 ? sp.split_keys : max_seq_len;
  p.ws_splits = p.splits;
  // lengths from seq_lens, causal, merged here
  // FP8: the K scale joins the softmax scale and the V scale multiplies the outputs.
  p.scale_log2 = (fp8 ? scale * k_scale : scale) * 1.4426950408889634f;
  p.kv_fp8 = fp8;
  p.v_scale = fp8 ? v_scale : 1.f;
  p.concurrent = concurrent;
  if (need > 0) {
    const size_t rows = (size_t)total_q * num_q_heads * p.splits;
    p.ws_ml = static_cast<float*>(workspace);
    p.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align_up(rows * 2 * sizeof(float), 256));
  }
  if (validate_only) return ok();
  return hip_status(pa::launch_prefill(p, static_cast<hipStream_t>(stream)), "prefill_chunk");
}

}  // namespace

extern "C" {

pa_status_t pa_prefill_chunk(void* out, const void* query, const void* key_cache,
                             const void* value_cache, int64_t num_blocks,
                             const int32_t* block_tables, const int32_t* query_start_loc,
                             const int32_t* seq_lens, int32_t num_seqs, int32_t total_q,
                             int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                             int32_t max_seq_len, float scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return prefill_impl(out, query, key_cache, value_cache, num_blocks, block_tables,
                      query_start_loc, seq_lens, num_seqs, total_q, max_q_len, num_q_heads,
                      num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len, scale,
                      false, 1.f, 1.f, workspace, workspace_bytes, stream);
}

pa_status_t pa_prefill_chunk_fp8(void* out, const void* query, const void* key_cache,
                                 const void* value_cache, int64_t num_blocks,
                                 const int32_t* block_tables, const int32_t* query_start_loc,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t total_q,
                                 int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                 int32_t max_seq_len, float scale, float k_scale, float v_scale,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(out, query, key_cache, value_cache, num_blocks, block_tables,
                      query_start_loc, seq_lens, num_seqs, total_q, max_q_len, num_q_heads,
                      num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len, scale,
                      true, k_scale, v_scale, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------------------------
// Mixed step: decode beside the prefill chunk on a second stream.

}  // extern "C"

namespace {

// concurrent: another kernel (the mixed step's decode) runs beside the chunk on the same CUs.
pa_status_t prefill_call(const pa_prefill_args& a, void* stream, bool validate_only,
                         bool concurrent = false) {
  return prefill_impl(a.out, a.query, a.key_cache, a.value_cache, a.num_blocks, a.block_tables,
                      a.query_start_loc, a.seq_lens, a.num_seqs, a.total_q, a.max_q_len,
                      a.num_q_heads, a.num_kv_heads, a.head_dim, a.block_size,
                      a.max_blocks_per_seq, a.max_seq_len, a.scale, a.kv_fp8 != 0, a.k_scale,
                      a.v_scale, a.workspace, a.workspace_bytes, stream, validate_only,
                      concurrent);
}

pa_status_t decode_call(const pa_decode_args& a, void* stream, bool validate_only) {
  return decode_impl(a.out, a.query, a.key_cache, a.value_cache, a.num_blocks, a.block_tables,
                     a.seq_lens, a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim,
                     a.block_size, a.max_blocks_per_seq, a.max_seq_len, a.scale, a.kv_fp8 != 0,
                     a.k_scale, a.v_scale, a.workspace, a.workspace_bytes, stream, nullptr,
                     nullptr, nullptr, 0, 0, validate_only);
}

// A byte range one half of a mixed step writes.
struct Span {
  const char* what;
  const void* ptr;
  size_t bytes;
  bool overlaps(const Span& o) const {
    if (!ptr || !o.ptr || !bytes || !o.bytes) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(ptr), b = reinterpret_cast<uintptr_t>(o.ptr);
    return a < b + o.bytes && b < a + bytes;
  }
};

// Fork and join events of the calling thread on the current device (created on first use, kept
// until the process ends).  They keep the default release on record: the other stream's kernels
// consume what was written before the event (workspaces, inputs copied in), and without that
// release those writes need not be visible to another queue's kernels.
hipError_t fork_join_events(hipEvent_t* fork, hipEvent_t* join) {
  thread_local std::map<int, std::pair<hipEvent_t, hipEvent_t>> per_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto& ev = per_device[dev];
  if (!ev.first) {
    const unsigned f = hipEventDisableTiming;
    if ((e = hipEventCreateWithFlags(&ev.first, f)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ev.second, f)) != hipSuccess) return e;
  }
  *fork = ev.first;
  *join = ev.second;
  return hipSuccess;
}

}  // namespace

extern "C" {

pa_status_t pa_mixed_step(const pa_prefill_args* prefill, const pa_decode_args* decode,
                          void* stream, void* side_stream) {
  if (!prefill || !decode) return fail(PA_ERR_NULL_POINTER, "null argument struct");
  // Both halves are validated before either is launched.
  pa_status_t st = prefill_call(*prefill, stream, true);
  if (st != PA_OK) return st;
  // The halves run at the same time: nothing one writes may overlap what the other writes.  The
  // byte ranges are the outputs and the workspace bytes each call uses (an empty half writes
  // nothing).
  const pa_prefill_args& pf = *prefill;
  const pa_decode_args& dc = *decode;
  std::vector<Span> spans;
  if (pf.num_seqs > 0 && pf.total_q > 0) {
    spans.push_back({"the prefill output", pf.out,
                     (size_t)pf.total_q * pf.num_q_heads * pf.head_dim * 2});
    spans.push_back({"the prefill workspace", pf.workspace,
                     pa_prefill_workspace_bytes(pf.num_seqs, pf.total_q, pf.max_q_len,
                                                pf.num_q_heads, pf.num_kv_heads, pf.head_dim,
                                                pf.max_seq_len)});
  }
  if (dc.num_seqs > 0 && dc.num_q_heads > 0 && dc.num_kv_heads > 0 && dc.head_dim > 0) {
    spans.push_back({"the decode output", dc.out,
                     (size_t)dc.num_seqs * dc.num_q_heads * dc.head_dim * 2});
    spans.push_back({"the decode workspace", dc.workspace,
                     pa::decode_workspace(dc.num_seqs, dc.num_kv_heads, dc.head_dim,
                                          dc.num_q_heads / dc.num_kv_heads, dc.kv_fp8 != 0)
                         .bytes});
  }
  for (size_t i = 0; i < spans.size(); ++i)
    for (size_t j = i + 1; j < spans.size(); ++j)
      if (spans[i].overlaps(spans[j]))
        return fail(PA_ERR_INVALID_ARG, "%s overlaps %s", spans[i].what, spans[j].what);
  if ((st = decode_call(*decode, side_stream, true)) != PA_OK) return st;
  if (!side_stream || side_stream == stream) {  // one stream: the two calls in order
    if ((st = decode_call(*decode, stream, false)) != PA_OK) return st;
    return prefill_call(*prefill, stream, false);
  }
  hipEvent_t fork = nullptr, join = nullptr;
  hipError_t e = fork_join_events(&fork, &join);
  if (e != hipSuccess) return hip_status(e, "mixed_step (events)");
  hipStream_t hs = static_cast<hipStream_t>(stream), side = static_cast<hipStream_t>(side_stream);
  if ((e = hipEventRecord(fork, hs)) != hipSuccess ||
      (e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess)
    return hip_status(e, "mixed_step (fork)");
  // Decode first, so its persistent workgroups are resident before the chunk's fill the rest.
  // Once the fork is recorded the join is always made, so later work on `stream` waits for
  // whatever was launched on the side stream even when a launch fails.
  st = decode_call(*decode, side_stream, false);
  if (st == PA_OK) st = prefill_call(*prefill, stream, false, true);
  if ((e = hipEventRecord(join, side)) != hipSuccess ||
      (e = hipStreamWaitEvent(hs, join, 0)) != hipSuccess)
    return st != PA_OK ? st : hip_status(e, "mixed_step (join)");
  return st;
}

}  // extern "C"
