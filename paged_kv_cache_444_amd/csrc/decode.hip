// Paged decode attention for gfx950: one query token per sequence against its whole paged
// context.
//
// What is computed: the attention of the "Inference optimization" lesson (Build it, Step 2:
// attention with a KV cache) with a single query row, max-subtracted softmax(q·kᵀ·scale)·v, where
// the sequence's keys and values are reached through its block table ("Serving engine internals"
// lesson, PagedAttention section).  Decode re-reads the whole KV cache every step and does about
// one multiply-add per byte per query head, so it is bound by HBM bandwidth ("Inference
// optimization", Prefill vs decode; vLLM-on-H100 article, "Decode is a memory problem").  The
// contraction therefore runs on the vector ALUs (v_dot2_f32_bf16) with DPP / swizzle reductions;
// matrix cores would sit idle waiting for memory.
//
// Work decomposition (balanced split-K).  A "step" is 16 tokens of one (sequence, KV head)
// "unit"; units are numbered s * num_kv_heads + h and laid end to end.  The T steps of the whole
// batch are cut into contiguous ranges ("virtual workers"): equal static ranges, one per resident
// wave, optionally followed by small dynamic chunks that idle waves take from an atomic counter
// (see Plan).  A wave keeps an online-softmax state (running max m, running sum l, accumulator
// acc) per query head; when a worker's range ends or leaves a unit it finishes that piece: a unit
// wholly inside one worker is normalised and written to the output; otherwise the piece's
// (m, l, acc) goes to its partial slot (worker + unit, unique per piece) and decode_merge
// combines the pieces of the unit in worker order.  Which wave runs which worker never changes
// the arithmetic, so results are bitwise reproducible and independent of where blocks sit.
//
// Lane roles within a step (one 16-token sub-block of one physical block, one KV head; the pool
// layout puts K as [D/32][16][32] and V as [D][16] inside the sub-block):
//   K side: lane l holds tokens l/8 and 8 + l/8 and the head-dim values 8c + 64x + [0, 8),
//           c = l % 8, x < D/64, so that each load instruction of the wave reads whole 64-byte
//           token rows of two 32-wide slices; the same values of the G query rows stay in
//           registers for the whole piece (G*D/16 registers, at most 64), and three DPP adds
//           finish each score.
//   softmax: online in the log2 domain with one running max per head for the whole wave; lane
//           l computes the probabilities of its own head(s) c + 8j.  The max is only raised (and
//           acc rescaled) when a score exceeds it by more than kRescaleSlack, which after the
//           first step almost never happens.
//   V side: lane l holds head-dim rows l%32 (+32k) of octet l/32, and P·V is v_dot2 over token
//           pairs with the probabilities read back from LDS as bf16 pairs.
// The next step's K and V are loaded into a second register set while the current step is
// computed.
//
// FP8 cache.  Pools of E4M3 codes keep the bf16 element order with one byte per element; their
// steps run on the matrix cores (see the matrix-core step below), widening the codes to bf16
// pairs (v_cvt_scalef32_pk_bf16_fp8 with scale 1, exact: every E4M3 value is a bf16 value).  The
// K scale is folded into the softmax scale and the V scale multiplies each output row, so the
// codes are never rescaled one by one.

#include "pa_device.h"
#include "pa_internal.h"

#include <algorithm>
#include <type_traits>
#include <map>
#include <mutex>
#include <utility>

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Fewer steps than this per worker would make partial slots and their merge outweigh the work
// (at 8, a batch of 128 sequences on one KV head used every wave and spent 1.1 us more per call),
// unless there are as many units as workers: a unit alone on its worker needs no partial.
constexpr int kMinStepsPerWave = 16;
// log2-domain slack before the running max is raised: probabilities stay below 2^8.
constexpr float kRescaleSlack = 8.0f;
// Dynamic chunks: batches of at most kMaxPrefixSeqs sequences keep their prefix sums in LDS; the
// workspace holds kDynSlotsPerWorker chunk slots per worker wave.
constexpr int kMaxPrefixSeqs = 4096;
constexpr int kPrefixLdsBytes = (kMaxPrefixSeqs + 1) * 4;
constexpr int kDynSlotsPerWorker = 2;
constexpr int kBlocksPerCU = 1;

// Whole blocks of sequence s left out at the front (a shared prefix attended elsewhere).
__device__ __forceinline__ int skip_blocks(const DecodeParams& p, int s) {
  if (!p.skip_lens) return 0;
  return min(max(p.skip_lens[s], 0) / p.block_size, p.max_blocks_per_seq);
}

// Tokens of sequence s this call attends: its length, clamped, less the skipped prefix.
__device__ __forceinline__ int clamped_len(const DecodeParams& p, int s) {
  return max(min(max(p.seq_lens[s], 0), p.len_cap) - skip_blocks(p, s) * p.block_size, 0);
}

// Slot of (sequence, query head) row `row` in the prefill-layout state workspace.
__device__ __forceinline__ size_t state_slot(const DecodeParams& p, size_t row) {
  return row * p.state_stride + p.state_split;
}

__device__ __forceinline__ int steps_of(const DecodeParams& p, int s) {
  return (clamped_len(p, s) + kSub - 1) / kSub;
}

// Inclusive prefix sum over the wave's 64 lanes with DPP moves: shifts by 1, 2, 4 and 8 within
// each 16-lane row (lanes without a source read 0), then row 0's and row 2's totals broadcast
// into rows 1 and 3, then lane 31's prefix into rows 2 and 3.  Six dependent adds, where the
// shuffle form took six LDS permutes.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return x;
}

// How the T steps of a call are split over "virtual workers".  Workers [0, ns) are static: worker
// v takes steps [v*S/ns, (v+1)*S/ns) and runs on wave v.  Workers [ns, ns+nd) are dynamic chunks
// of C steps covering [S, T), taken by whichever wave is free (an atomic counter hands them out).
// Which wave runs a worker never changes what the worker computes, and every piece of work has a
// fixed partial slot (worker + unit), so results do not depend on the dynamic order.
//
// The static split balances cost, not steps: every piece a worker starts costs A steps' worth of
// time (the block-id window and the first K/V tile are dependent loads that nothing overlaps), so
// step x of the batch's j-th non-empty unit costs position x + A*(j+1) on a line of length
// CT = S + A * (non-empty units).  Worker v starts at the first step whose cost position reaches
// v*CT/ns; A = 0 gives the even split of steps.  Dynamic chunks keep A = 0.
// floor(n / d) for 0 <= n < 2^53 and d > 0.  The correctly rounded double quotient is at most one
// above the exact floor (rounding is monotone and every integer below 2^53 is a double), so one
// exact integer check finishes it.  It replaces the long 64-bit integer division sequence on the
// partition's critical path at the start of every launch.
__device__ __forceinline__ long long div_nonneg(long long n, long long d) {
  long long q = (long long)((double)n / (double)d);
  if (q * d > n) --q;
  return q;
}

struct Plan {
  long long T, S, ns, C, nd, A, CT;
  __device__ long long start(long long v) const {  // A = 0 only
    return v <= ns ? div_nonneg(v * S, ns) : min(T, S + (v - ns) * C);
  }
  __device__ long long target(long long v) const { return div_nonneg(v * CT, ns); }
  // Worker holding step x, which lies in non-empty unit j.
  __device__ long long owner(long long x, long long j) const {
    return x < S ? div_nonneg((x + A * (j + 1) + 1) * ns - 1, CT) : ns + div_nonneg(x - S, C);
  }
};

// K-side lane roles: lane l holds token 8p + l/8 of the step's two octets (p = 0, 1) and the
// D/8 head-dim values 8c + 64x + [0, 8) with c = l % 8; the 8 lanes of a token finish its scores
// with three DPP adds.  Load (p, x) of the wave covers rows 8p .. 8p+7 of slices 2x and 2x+1:
// two 512-byte runs of whole cache lines.  V-side: lane l holds head-dim rows l%32 + 32x of
// octet l/32, so load x is 1 KB contiguous.
template <int D>
struct StepRegs {
  uint4 k[2][D / 64];
  uint4 v[D / kSlice];
};

// Eight E4M3 codes -> eight bf16 values, same order (two per conversion).
template <bool Hi>
__device__ __forceinline__ uint32_t fp8_pair_to_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, Hi));
}
__device__ __forceinline__ uint4 widen8(const uint2& w) {
  return make_uint4(fp8_pair_to_bf16<false>(w.x), fp8_pair_to_bf16<true>(w.x),
                    fp8_pair_to_bf16<false>(w.y), fp8_pair_to_bf16<true>(w.y));
}

// Query heads a lane computes probabilities for: heads c + 8j (j < kOwn) of the G sharing the
// KV head, where c = lane % 8; for G < 8 only lanes with c < G own a head.
template <int G>
constexpr int kOwn = (G + 7) / 8;

// Online-softmax state of one piece.  Scores are kept unscaled: m[g] is the running maximum of
// raw scores of head g (the same in every lane), nmc = -m * scale * log2(e) (0 while m is -inf),
// thr = m + slack / (scale * log2(e)).  The own_* copies hold those of the lane's own heads, l the
// lane's partial sums of its own heads' probabilities.
template <int D, int G>
struct PieceState {
  float m[G], nmc[G], thr[G];
  float own_nmc[kOwn<G>], own_thr[kOwn<G>], l[kOwn<G>];
  float acc[G][D / kSlice];
};

__device__ __forceinline__ float uniform_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// Partial slot of the piece of unit u (s * num_kv_heads + h) held by worker w.  Later workers
// hold later units, so w + u is unique among pieces; with head quads the worker is a workgroup
// and the order is over quad units u / kWaves, so the slot is (w + u / kWaves) * kWaves + u % kWaves.
__device__ __forceinline__ size_t slot_of(const DecodeParams& p, long long w, int u) {
  return p.quad ? (size_t)(w + u / kWaves) * kWaves + u % kWaves : (size_t)(w + u);
}

// Head owned by this lane in slot j, or -1.
template <int G>
__device__ __forceinline__ int own_head(int c, int j) {
  const int g = c + 8 * j;
  return g < G ? g : -1;
}

// Issue the loads of step i of the current unit.  `win`/`ids` hold up to 64 physical block ids
// of the unit, one per lane, starting at logical block `win`.
// 16-byte global load.  Stream = read-once data: the non-temporal hint keeps it from displacing
// lines in L2 and the last-level cache, which the 70B-shaped batch measured 9 % faster.
template <bool Stream>
__device__ __forceinline__ uint4 load16(const uint16_t* ptr) {
  if constexpr (Stream) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)ptr);
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *(const uint4*)ptr;
  }
}
// 8-byte load of eight E4M3 codes (FP8 pools).
template <bool Stream>
__device__ __forceinline__ uint2 load8(const uint8_t* ptr) {
  if constexpr (Stream) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)ptr);
    return make_uint2(v.x, v.y);
  } else {
    return *(const uint2*)ptr;
  }
}
// Eight elements at element offset `off` of a pool: 16 bytes of bf16 or 8 bytes of codes.
template <bool Stream, bool Fp8>
__device__ __forceinline__ std::conditional_t<Fp8, uint2, uint4> load_elems(const uint16_t* pool,
                                                                            size_t off) {
  if constexpr (Fp8) return load8<Stream>(reinterpret_cast<const uint8_t*>(pool) + off);
  else return load16<Stream>(pool + off);
}

template <int D, bool Stream>
__device__ __forceinline__ void load_step(StepRegs<D>& r, int i, const DecodeParams& p,
                                          const int* bt, int cols, int& win, int& ids,
                                          size_t head_off, size_t block_elems) {
  constexpr int R = D / kSlice;
  const int lane = threadIdx.x & 63;
  const int bs = p.block_size;
  const int t0 = i * kSub;
  const int b = t0 >> (bs == 32 ? 5 : 4);
  if (b - win >= 64) {  // rare: refill the block-id window
    win = b;
    const int id = (win + lane < cols) ? bt[win + lane] : 0;
    ids = min(max(id, 0), (int)(p.num_blocks - 1));
  }
  const int id = __builtin_amdgcn_readlane(ids, b - win);
  const size_t off = (size_t)id * block_elems + head_off + (size_t)(t0 & (bs - 1)) * D;
  const int c = lane & 7, tt = lane >> 3;
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int x = 0; x < D / 64; ++x) {
      const int d = 8 * c + 64 * x;
      r.k[pp][x] = load16<Stream>(p.kpool + off + (d >> 5) * (kSub * kSlice) +
                                  (8 * pp + tt) * kSlice + (d & 31));
    }
  const int vd = lane & 31, vo = lane >> 5;
#pragma unroll
  for (int x = 0; x < R; ++x)
    r.v[x] = load16<Stream>(p.vpool + off + (vd + 32 * x) * kSub + 8 * vo);
}

// One 16-token step: scores, online softmax, P·V.  nvalid = tokens of the step inside the piece
// (>= 1); only the last step of a piece can have fewer than 16.
template <int D, int G>
__device__ __forceinline__ void compute_step(const StepRegs<D>& r, const uint4 (&q)[G][D / 64],
                                             int nvalid, float c, float slack_raw,
                                             uint16_t (*p_sh)[G][8], PieceState<D, G>& st) {
  constexpr int R = D / kSlice;
  constexpr int O = kOwn<G>;
  const int lane = threadIdx.x & 63;
  const int lc = lane & 7, tt = lane >> 3;
  const int vo = lane >> 5;
  const bool tail = nvalid < kSub;  // wave-uniform

  // Raw scores q·k of tokens tt and 8 + tt for every head.
  float sc[2][G];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a = 0.f;
#pragma unroll
      for (int x = 0; x < D / 64; ++x) a = dot8(q[g][x], r.k[pp][x], a);
      a += dpp_f32<kDppQuadXor1>(a);
      a += dpp_f32<kDppQuadXor2>(a);
      a += dpp_f32<kDppRowHalfMirror>(a);
      sc[pp][g] = a;
    }
  if (tail) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int g = 0; g < G; ++g) sc[pp][g] = (8 * pp + tt < nvalid) ? sc[pp][g] : kNegInf;
  }
  float own[2][O];
#pragma unroll
  for (int j = 0; j < O; ++j) {
    const int mine = own_head<G>(lc, j);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      float v = kNegInf;
#pragma unroll
      for (int g = 0; g < G; ++g) v = (g == mine) ? sc[pp][g] : v;
      own[pp][j] = v;
    }
  }

  // The running max is raised only when some score exceeds it by the slack; otherwise the
  // probabilities below stay under 2^slack and nothing is rescaled.
  bool raise = false;
#pragma unroll
  for (int j = 0; j < O; ++j) raise |= fmaxf(own[0][j], own[1][j]) > st.own_thr[j];
  if (__builtin_expect(__ballot(raise) != 0, 0)) {  // rare: kept out of line
    float alpha[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x = fmaxf(sc[0][g], sc[1][g]);
      x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
      x = fmaxf(x, xor16_f32(x));
      x = fmaxf(x, __shfl_xor(x, 32, 64));
      const float mn = uniform_f(fmaxf(st.m[g], x));
      alpha[g] = 1.f;
      if (mn != kNegInf && mn != st.m[g]) {
        alpha[g] = fast_exp2((st.m[g] - mn) * c);  // 0 when the old max is -inf
#pragma unroll
        for (int y = 0; y < R; ++y) st.acc[g][y] *= alpha[g];
        st.m[g] = mn;
        st.nmc[g] = -mn * c;
        st.thr[g] = mn + slack_raw;
      }
    }
#pragma unroll
    for (int j = 0; j < O; ++j) {
      const int mine = own_head<G>(lc, j);
      float a = 1.f, n = 0.f, t = kNegInf;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        a = (g == mine) ? alpha[g] : a;
        n = (g == mine) ? st.nmc[g] : n;
        t = (g == mine) ? st.thr[g] : t;
      }
      st.l[j] *= a;
      st.own_nmc[j] = n;
      st.own_thr[j] = (mine < 0) ? __builtin_inff() : t;
    }
  }
#pragma unroll
  for (int j = 0; j < O; ++j) {
    const int mine = own_head<G>(lc, j);
    const float p0 = fast_exp2(__builtin_fmaf(own[0][j], c, st.own_nmc[j]));
    const float p1 = fast_exp2(__builtin_fmaf(own[1][j], c, st.own_nmc[j]));
    st.l[j] += p0 + p1;
    if (mine >= 0) {
      p_sh[0][mine][tt] = to_bf16(p0);
      p_sh[1][mine][tt] = to_bf16(p1);
    }
  }
  wave_lds_sync();

  uint4 v[R];
#pragma unroll
  for (int x = 0; x < R; ++x) v[x] = r.v[x];
  if (tail) {  // zero V of tokens past the end: 0 * NaN must not reach acc
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 8 * vo + 2 * e;
      const uint32_t keep = (t + 1 < nvalid) ? 0xFFFFFFFFu : ((t < nvalid) ? 0xFFFFu : 0u);
#pragma unroll
      for (int x = 0; x < R; ++x) {
        if (e == 0) v[x].x &= keep;
        if (e == 1) v[x].y &= keep;
        if (e == 2) v[x].z &= keep;
        if (e == 3) v[x].w &= keep;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 pp = *(const uint4*)&p_sh[vo][g][0];
#pragma unroll
    for (int x = 0; x < R; ++x) st.acc[g][x] = dot8(pp, v[x], st.acc[g][x]);
  }
  wave_lds_sync();
}

// Steps j0 .. j0+take-1 of unit (s, h) by virtual worker w.  x is the global index of step j0.
// Depth is the number of steps whose loads are in flight while one step is computed.  With
// `coop` set the wave's (m, l, acc) always goes to `coop` (its slot in LDS) and the workgroup
// combines the slots; otherwise the piece is finished here.
template <int D, int G, int Depth, bool Stream>
__device__ __forceinline__ void decode_piece(const DecodeParams& p, int s, int h, int j0, int take,
                                             int n_s, long long w, long long x, long long jn,
                                             const Plan& plan, uint16_t (*p_sh)[G][8],
                                             float* coop = nullptr) {
  constexpr int R = D / kSlice;
  constexpr int O = kOwn<G>;
  const int lane = threadIdx.x & 63;
  const int lc = lane & 7;
  const int Hq = p.num_q_heads;
  const int L = uniform(clamped_len(p, s));
  const int u = s * p.num_kv_heads + h;
  const bool whole = !coop && (j0 == 0) && (take == n_s);
  if (!coop && j0 == 0 && lane == 0)
    p.unit_info[u] = make_int2((int)w, (int)plan.owner(x + n_s - 1, jn));

  // This lane's head-dim slice of the G query rows sharing KV head h.
  uint4 q[G][D / 64];
  {
    const uint16_t* qg = p.query + ((size_t)s * Hq + (size_t)h * G) * D + 8 * lc;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int y = 0; y < D / 64; ++y) q[g][y] = *(const uint4*)(qg + g * D + 64 * y);
  }

  const int bs = p.block_size;
  // Table entries of the sequence from its first attended block on (after a skipped prefix).
  const int skip_b = skip_blocks(p, s);
  const int* bt = p.block_tables + (size_t)s * p.max_blocks_per_seq + skip_b;
  const int cols = p.max_blocks_per_seq - skip_b;
  const int tok_end = min(L, (j0 + take) * kSub);
  int win = (j0 * kSub) / bs;
  int ids;
  {
    // Read without waiting for the length: entries past the sequence's blocks are padding, and
    // the steps below only ever use the sequence's own blocks.
    const int id = (win + lane < cols) ? bt[win + lane] : 0;
    ids = min(max(id, 0), (int)(p.num_blocks - 1));
  }
  const size_t tile = (size_t)bs * D;
  const size_t block_elems = (size_t)p.num_kv_heads * tile;
  const size_t head_off = (size_t)h * tile;

  PieceState<D, G> st;
  const float c = p.scale_log2;
  const float slack_raw = kRescaleSlack / c;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = kNegInf;
    st.nmc[g] = 0.f;
    st.thr[g] = kNegInf;
#pragma unroll
    for (int y = 0; y < R; ++y) st.acc[g][y] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < O; ++j) {
    st.own_nmc[j] = 0.f;
    st.own_thr[j] = own_head<G>(lc, j) >= 0 ? kNegInf : __builtin_inff();
    st.l[j] = 0.f;
  }

  // Prefetch loads are issued unconditionally (past the last step they repeat the last step's
  // addresses, which hit in cache): a load issued on only some paths would make the compiler
  // wait for every outstanding load before each step.
  auto ld = [&](StepRegs<D>& r, int step) __attribute__((always_inline)) {
    load_step<D, Stream>(r, step, p, bt, cols, win, ids, head_off, block_elems);
  };
  const int iend = j0 + take;
  const int ilast = iend - 1;
  int i = j0;
  if constexpr (Depth == 0) {  // no prefetch: fewer registers, more resident waves
    while (true) {
      StepRegs<D> ra;
      ld(ra, i);
      compute_step<D, G>(ra, q, tok_end - i * kSub, c, slack_raw, p_sh, st);
      if (++i >= iend) break;
    }
  } else if constexpr (Depth == 1) {
    StepRegs<D> ra, rb;
    ld(ra, i);
    while (true) {
      ld(rb, min(i + 1, ilast));
      compute_step<D, G>(ra, q, tok_end - i * kSub, c, slack_raw, p_sh, st);
      if (++i >= iend) break;
      ld(ra, min(i + 1, ilast));
      compute_step<D, G>(rb, q, tok_end - i * kSub, c, slack_raw, p_sh, st);
      if (++i >= iend) break;
    }
  } else {  // two steps in flight while one is computed
    StepRegs<D> r0, r1, r2;
    ld(r0, i);
    ld(r1, min(i + 1, ilast));
    while (true) {
      ld(r2, min(i + 2, ilast));
      compute_step<D, G>(r0, q, tok_end - i * kSub, c, slack_raw, p_sh, st);
      if (++i >= iend) break;
      ld(r0, min(i + 2, ilast));
      compute_step<D, G>(r1, q, tok_end - i * kSub, c, slack_raw, p_sh, st);
      if (++i >= iend) break;
      ld(r1, min(i + 2, ilast));
      compute_step<D, G>(r2, q, tok_end - i * kSub, c, slack_raw, p_sh, st);
      if (++i >= iend) break;
    }
  }

  // Finish the piece.  l: sum each own head's partial over the eight token groups; lane g % 8
  // then holds head g's total.  acc: both octet halves share m, so they simply add.
  const int vd = lane & 31, vo = lane >> 5;
  float lsum[O];
#pragma unroll
  for (int j = 0; j < O; ++j) {
    float y = st.l[j];
    y += dpp_f32<kDppRowRor8>(y);
    y += xor16_f32(y);
    y += __shfl_xor(y, 32, 64);
    lsum[j] = y;
  }
  float* slot = coop ? coop : p.partials + slot_of(p, w, u) * (G * (2 + D));
  uint16_t* orow = p.out + ((size_t)s * Hq + (size_t)h * G) * D;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float lt = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lsum[g / 8]), g % 8));
    if (!whole && lane == 0) {
      slot[g] = st.m[g] * c;  // the merge works in the log2 domain
      slot[G + g] = lt;
    }
    if (whole && p.state_ml && lane == 0) {
      const size_t u = state_slot(p, (size_t)s * Hq + (size_t)h * G + g);
      p.state_ml[2 * u] = st.m[g] * c;
      p.state_ml[2 * u + 1] = lt;
    }
    // Half 0 finishes rows vd + 32k for k < R/2, half 1 the rest; each sends the other half's.
#pragma unroll
    for (int k = 0; k < R / 2; ++k) {
      const float mine = vo ? st.acc[g][k + R / 2] : st.acc[g][k];
      const float send = vo ? st.acc[g][k] : st.acc[g][k + R / 2];
      const float a = mine + __shfl_xor(send, 32, 64);
      const int d = vd + 32 * (k + (vo ? R / 2 : 0));
      if (whole && p.state_ml)
        p.state_acc[state_slot(p, (size_t)s * Hq + (size_t)h * G + g) * D + d] = a * p.v_scale;
      else if (whole) orow[g * D + d] = to_bf16(a * p.v_scale / lt);
      else slot[2 * G + g * D + d] = a;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Matrix-core step (FP8 pools).  With an FP8 cache a step carries half the bytes, and the vector
// step above (about 430 instructions per 16-token step of one KV head with the conversions)
// becomes the limit, not HBM.  The G query heads sharing a KV head make the step a small dense
// contraction, so it runs on the matrix cores instead:
//   S[token][head] = K·Qᵀ    v_mfma_f32_16x16x32_bf16 per 32-dim slice: A = K (row = token
//                          lane%16, dims 8*(lane/16) .. +7 of the slice: 8 contiguous elements of
//                          the K sub-block layout), B = Q (column = head lane%16, zero past G);
//                          lane l ends up with tokens 4*(l/16) + i of head l%16.
//   Oᵀ[dim][head] += Vᵀ·P   v_mfma_f32_16x16x16_bf16 per 16-dim tile: A = V (row = dim
//                          16m + lane%16, tokens 4*(lane/16) .. +3: 4 contiguous elements of the
//                          V sub-block layout), B = P, which the score product left in exactly
//                          this operand layout, so probabilities never leave registers.
// Each lane owns one head (column lane%16); its online-softmax state is a scalar, the same in
// the four lanes of a column, and its accumulators hold dims 16m + 4*(lane/16) + i of that head.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D, bool Fp8>
struct MStepRegs {
  std::conditional_t<Fp8, uint2, uint4> k[D / kSlice];     // 8 elements per 32-dim slice
  std::conditional_t<Fp8, uint32_t, uint2> v[D / kSub];    // 4 elements per 16-dim tile
};

template <int D>
struct MState {
  float m, nmc, thr, l;
  f32x4_t acc[D / kSub];
};

template <bool Stream>
__device__ __forceinline__ uint32_t load4(const uint8_t* ptr) {
  if constexpr (Stream) return __builtin_nontemporal_load((const uint32_t*)ptr);
  else return *(const uint32_t*)ptr;
}
template <bool Stream>
__device__ __forceinline__ uint2 load8_u16(const uint16_t* ptr) {
  return load8<Stream>(reinterpret_cast<const uint8_t*>(ptr));
}

template <int D, bool Stream, bool Fp8>
__device__ __forceinline__ void load_mstep(MStepRegs<D, Fp8>& r, int i, const DecodeParams& p,
                                           const int* bt, int cols, int& win, int& ids,
                                           size_t head_off, size_t block_elems) {
  const int lane = threadIdx.x & 63;
  const int bs = p.block_size;
  const int t0 = i * kSub;
  const int b = t0 >> (bs == 32 ? 5 : 4);
  if (b - win >= 64) {  // rare: refill the block-id window
    win = b;
    const int id = (win + lane < cols) ? bt[win + lane] : 0;
    ids = min(max(id, 0), (int)(p.num_blocks - 1));
  }
  const int id = __builtin_amdgcn_readlane(ids, b - win);
  const size_t off = (size_t)id * block_elems + head_off + (size_t)(t0 & (bs - 1)) * D;
  const int r16 = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int sl = 0; sl < D / kSlice; ++sl)
    r.k[sl] =
        load_elems<Stream, Fp8>(p.kpool, off + sl * (kSub * kSlice) + r16 * kSlice + 8 * q4);
#pragma unroll
  for (int m = 0; m < D / kSub; ++m) {
    const size_t e = off + (size_t)(kSub * m + r16) * kSub + 4 * q4;
    if constexpr (Fp8) r.v[m] = load4<Stream>(reinterpret_cast<const uint8_t*>(p.vpool) + e);
    else r.v[m] = load8_u16<Stream>(p.vpool + e);
  }
}

__device__ __forceinline__ uint4 k_operand(const uint4& k) { return k; }
__device__ __forceinline__ uint4 k_operand(const uint2& k) { return widen8(k); }
// V operand (4 elements) with tokens at or past nvalid zeroed, so 0 * NaN cannot reach acc.
__device__ __forceinline__ uint2 v_operand(const uint2& v, int t, int nvalid, bool tail) {
  if (!tail) return v;
  const uint32_t k0 = (t + 1 < nvalid) ? 0xFFFFFFFFu : ((t < nvalid) ? 0xFFFFu : 0u);
  const uint32_t k1 = (t + 3 < nvalid) ? 0xFFFFFFFFu : ((t + 2 < nvalid) ? 0xFFFFu : 0u);
  return make_uint2(v.x & k0, v.y & k1);
}
__device__ __forceinline__ uint2 v_operand(uint32_t v, int t, int nvalid, bool tail) {
  if (tail) {  // one code per token; code 0 is +0
    const int n = min(max(nvalid - t, 0), 4);
    v &= (n >= 4) ? 0xFFFFFFFFu : ((1u << (8 * n)) - 1u);
  }
  return make_uint2(fp8_pair_to_bf16<false>(v), fp8_pair_to_bf16<true>(v));
}

template <int D, bool Fp8>
__device__ __forceinline__ void compute_mstep(const MStepRegs<D, Fp8>& r,
                                              const uint4 (&qb)[D / kSlice], int nvalid, float c,
                                              float slack_raw, MState<D>& st) {
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4;
  const bool tail = nvalid < kSub;  // wave-uniform
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sl = 0; sl < D / kSlice; ++sl)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k_operand(r.k[sl])),
                                                 __builtin_bit_cast(bf16x8_t, qb[sl]), sc, 0, 0, 0);
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (!tail || 4 * q4 + i < nvalid) ? sc[i] : kNegInf;
  const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  // Raising the maximum is rare: its code is kept out of line, so the step's common path has no
  // taken branch.
  if (__builtin_expect(__ballot(mx > st.thr) != 0, 0)) {
    float cm = fmaxf(mx, xor16_f32(mx));
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));  // the column's max over its 16 tokens
    const float mn = fmaxf(st.m, cm);
    if (mn != kNegInf && mn != st.m) {
      const float alpha = fast_exp2((st.m - mn) * c);  // 0 when the old max is -inf
      st.l *= alpha;
#pragma unroll
      for (int m = 0; m < D / kSub; ++m) st.acc[m] *= alpha;
      st.m = mn;
      st.nmc = -mn * c;
      st.thr = mn + slack_raw;
    }
  }
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(__builtin_fmaf(x[i], c, st.nmc));
  st.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  const uint2 pb = make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
#pragma unroll
  for (int m = 0; m < D / kSub; ++m)
    st.acc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(s16x4_t, v_operand(r.v[m], 4 * q4, nvalid, tail)),
        __builtin_bit_cast(s16x4_t, pb), st.acc[m], 0, 0, 0);
}

// End of a matrix-core piece of unit u = (s, h): normalise and write the output (the unit lies
// wholly in the piece), or hand the unnormalised state to the cascade's state slot, or write the
// piece's partial slot (or `coop`, the wave's LDS slot of a shared piece).
template <int D, int G>
__device__ __forceinline__ void finish_mpiece(const DecodeParams& p, const MState<D>& st, int s,
                                              int h, int u, long long w, bool whole,
                                              float* coop) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int Hq = p.num_q_heads;
  const float c = p.scale_log2;
  // The column's sum over its four lanes; lane (r16, q4) holds dims 16m + 4*q4 + i.
  float lt = st.l + xor16_f32(st.l);
  lt += __shfl_xor(lt, 32, 64);
  if (r16 >= G) return;
  const int g = r16;
  float* slot = coop ? coop : p.partials + slot_of(p, w, u) * (G * (2 + D));
  uint16_t* orow = p.out + ((size_t)s * Hq + (size_t)h * G + g) * D;
  if (whole && p.state_ml) {
    const size_t su = state_slot(p, (size_t)s * Hq + (size_t)h * G + g);
    if (q4 == 0) {
      p.state_ml[2 * su] = st.m * c;
      p.state_ml[2 * su + 1] = lt;
    }
#pragma unroll
    for (int m = 0; m < D / kSub; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.state_acc[su * D + kSub * m + 4 * q4 + e] = st.acc[m][e] * p.v_scale;
    return;
  }
  if (whole) {
#pragma unroll
    for (int m = 0; m < D / kSub; ++m) {
      const f32x4_t a = st.acc[m];
      *(uint2*)(orow + kSub * m + 4 * q4) =
          make_uint2(pack_bf16x2(a[0] * p.v_scale / lt, a[1] * p.v_scale / lt),
                     pack_bf16x2(a[2] * p.v_scale / lt, a[3] * p.v_scale / lt));
    }
    return;
  }
  if (q4 == 0) {
    slot[g] = st.m * c;  // the merge works in the log2 domain
    slot[G + g] = lt;
  }
  // Scalar stores: a slot holds G*(2+D) floats, so it is only 4-byte aligned when G is odd.
#pragma unroll
  for (int m = 0; m < D / kSub; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) slot[2 * G + g * D + kSub * m + 4 * q4 + e] = st.acc[m][e];
}

// B operand of the score product for the G query heads of (sequence s, KV head h): head r16
// (zero past G), dims 8*q4 .. +7 of each 32-dim slice.
template <int D, int G>
__device__ __forceinline__ void load_qb(uint4 (&qb)[D / kSlice], const DecodeParams& p, int s,
                                        int h) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, q4 = lane >> 4;
  const uint16_t* qg =
      p.query + ((size_t)s * p.num_q_heads + (size_t)h * G + min(r16, G - 1)) * D + 8 * q4;
#pragma unroll
  for (int sl = 0; sl < D / kSlice; ++sl) {
    const uint4 v = *(const uint4*)(qg + kSlice * sl);
    qb[sl] = r16 < G ? v : make_uint4(0u, 0u, 0u, 0u);
  }
}

// decode_piece on the matrix cores (same contract and partial-slot format).
template <int D, int G, int Depth, bool Stream, bool Fp8>
__device__ __forceinline__ void decode_piece_mfma(const DecodeParams& p, int s, int h, int j0,
                                                  int take, int n_s, long long w, long long x,
                                                  long long jn, const Plan& plan,
                                                  float* coop = nullptr) {
  static_assert(G <= 16, "one matrix-core column per query head");
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int Hq = p.num_q_heads;
  const int L = uniform(clamped_len(p, s));
  const int u = s * p.num_kv_heads + h;
  const bool whole = !coop && (j0 == 0) && (take == n_s);
  if (!coop && j0 == 0 && lane == 0)
    p.unit_info[u] = make_int2((int)w, (int)plan.owner(x + n_s - 1, jn));

  // B operand of the score product: head r16 (zero past G), dims 8*q4 .. +7 of each slice.
  uint4 qb[D / kSlice];
  {
    const uint16_t* qg = p.query + ((size_t)s * Hq + (size_t)h * G + min(r16, G - 1)) * D + 8 * q4;
#pragma unroll
    for (int sl = 0; sl < D / kSlice; ++sl) {
      const uint4 v = *(const uint4*)(qg + kSlice * sl);
      qb[sl] = r16 < G ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  const int bs = p.block_size;
  // Table entries of the sequence from its first attended block on (after a skipped prefix).
  const int skip_b = skip_blocks(p, s);
  const int* bt = p.block_tables + (size_t)s * p.max_blocks_per_seq + skip_b;
  const int cols = p.max_blocks_per_seq - skip_b;
  const int tok_end = min(L, (j0 + take) * kSub);
  int win = (j0 * kSub) / bs;
  int ids;
  {
    const int id = (win + lane < cols) ? bt[win + lane] : 0;
    ids = min(max(id, 0), (int)(p.num_blocks - 1));
  }
  const size_t tile = (size_t)bs * D;
  const size_t block_elems = (size_t)p.num_kv_heads * tile;
  const size_t head_off = (size_t)h * tile;

  MState<D> st;
  const float c = p.scale_log2;
  const float slack_raw = kRescaleSlack / c;
  st.m = kNegInf;
  st.nmc = 0.f;
  st.thr = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int m = 0; m < D / kSub; ++m) st.acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Prefetch loads are issued unconditionally (past the last step they repeat its addresses).
  auto ld = [&](MStepRegs<D, Fp8>& r, int step) __attribute__((always_inline)) {
    load_mstep<D, Stream, Fp8>(r, step, p, bt, cols, win, ids, head_off, block_elems);
  };
  const int iend = j0 + take;
  const int ilast = iend - 1;
  int i = j0;
  if constexpr (Depth <= 1) {
    MStepRegs<D, Fp8> ra, rb;
    ld(ra, i);
    while (true) {
      ld(rb, min(i + 1, ilast));
      compute_mstep<D, Fp8>(ra, qb, tok_end - i * kSub, c, slack_raw, st);
      if (++i >= iend) break;
      ld(ra, min(i + 1, ilast));
      compute_mstep<D, Fp8>(rb, qb, tok_end - i * kSub, c, slack_raw, st);
      if (++i >= iend) break;
    }
  } else {
    MStepRegs<D, Fp8> r0, r1, r2;
    ld(r0, i);
    ld(r1, min(i + 1, ilast));
    while (true) {
      ld(r2, min(i + 2, ilast));
      compute_mstep<D, Fp8>(r0, qb, tok_end - i * kSub, c, slack_raw, st);
      if (++i >= iend) break;
      ld(r0, min(i + 2, ilast));
      compute_mstep<D, Fp8>(r1, qb, tok_end - i * kSub, c, slack_raw, st);
      if (++i >= iend) break;
      ld(r1, min(i + 2, ilast));
      compute_mstep<D, Fp8>(r2, qb, tok_end - i * kSub, c, slack_raw, st);
      if (++i >= iend) break;
    }
  }

  finish_mpiece<D, G>(p, st, s, h, u, w, whole, coop);
}

// Where a piece's K/V come from: its sequence's table row (after a skipped prefix), a window of
// 64 block ids of that row starting at logical block `win` (one per lane), and its KV head.
struct MPieceSrc {
  const int* bt;
  int cols, win, ids;
  size_t head_off;
};

// The static range [x, x1) of worker v on the matrix cores, piece after piece, with the next
// piece's loads started early: its query operand and block-id window when the current piece
// starts, and its first K/V step in the prefetch slot of the current piece's last step (where a
// single piece would load nothing new).  A piece boundary then costs no dependent round trip.
// Same pieces, partial slots and arithmetic as run_worker with decode_piece_mfma.
//
// Dynamic tail (quad workers, `tail` set): after its static range the workgroup takes the chunks
// [S + d*C, S + (d+1)*C) of the step line in claim order (d from the workspace counter; chunk d is
// worker ns + d, with its own partial slots).  Each claim is made inside the walk of the range's
// last piece, kClaimLead steps before its end: late enough that the workgroups which run ahead
// take the chunks, early enough that the chunk's block ids, query and first step are loading while
// the piece finishes.  The claims travel through two LDS slots in turn; every wave of the
// workgroup makes the same decisions, so all reach the same barriers.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// bf16 matrix-core steps keep register loads: staged through LDS they measured about 0.7 us
// slower at the 70B shape, where the bf16 walk is bound by HBM rather than by its loads in flight.
constexpr bool kStageBf16 = false;
// Steps before the end of a range's last piece at which the workgroup claims its next tail chunk
// (2, 4 and 8 measured alike at the 70B shape).
constexpr int kClaimLead = 2;
// Matrix-core steps stage each step's K and V in LDS: the K tile and the V tile of one 16-token
// sub-block of one KV head are each kSub * D contiguous elements of the pool, so a wave fetches
// them with 16-byte direct global->LDS loads (1 KB per instruction) and then reads its operands
// from LDS.  A step then takes D/32 (FP8) or D/16 (bf16) load instructions instead of 3*D/32
// register loads of 4 to 16 bytes; the number of loads a wave keeps in flight, not their bytes,
// was what bounded the step rate.
template <int D, bool Fp8>
constexpr int kStageBytes = 2 * kSub * D * (Fp8 ? 1 : 2);
template <int D, bool Fp8>
constexpr int kDmaPerStep = kStageBytes<D, Fp8> / 1024;

// One direct global->LDS load of 16 bytes per lane: lane l's bytes land at LDS byte address
// m0 + 16*l (m0 wave-uniform).  Written as inline assembly so the compiler does not treat the
// walk's LDS reads as dependent on it (it would wait for every such load before each read); the
// walk waits for these loads itself.  The load has no register result.  It first waits for this
// wave's LDS reads issued before it, so a slot is never refilled while its last reads are still
// pending.
template <bool Stream>
__device__ __forceinline__ void lds_dma_16(const uint8_t* src, unsigned m0) {
  if constexpr (Stream)
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off nt"
        :
        : "v"(src), "s"(m0)
        : "memory", "m0");
  else
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(src), "s"(m0)
        : "memory", "m0");
}

template <int D, int G, int Dep, bool Stream, bool Fp8>
__device__ __forceinline__ void run_worker_mfma(const DecodeParams& p, const Plan& plan,
                                                long long v, int s, long long off, long long jn,
                                                long long x, long long x1, bool quad,
                                                lds_u8* stage, bool tail = false,
                                                const int* seq_prefix = nullptr,
                                                unsigned* sh_claim = nullptr) {
  // Steps staged through LDS (FP8 pools always, bf16 pools with kStageBf16).
  constexpr bool kStaged = Fp8 || kStageBf16;
  const int B = p.num_seqs;
  const int U = quad ? p.num_kv_heads / kWaves : p.num_kv_heads;
  // Sequence and step offset (within its U * n_s steps) of global step x0 of a dynamic chunk:
  // the last sequence whose per-head prefix is <= x0 / U.
  auto locate = [&](long long x0, int& so, long long& oo) {
    const long long xh = x0 / U;
    int lo = 0, hi = B;  // invariant: seq_prefix[lo] <= xh < seq_prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seq_prefix[mid] <= xh) lo = mid;
      else hi = mid;
    }
    so = lo;
    oo = x0 - (long long)seq_prefix[lo] * U;
  };
  int par = 0;  // LDS slot of the next claim
  // Claims the next chunk (-1: none left).  One counter increment per workgroup, published in
  // LDS; the slots alternate, so the barrier of the claim between two writes of one slot orders
  // the later write after every wave's read of the earlier one.
  auto claim = [&]() -> long long {
    if (threadIdx.x == 0) sh_claim[par] = atomicAdd(p.counter, 1u);
    __syncthreads();
    const unsigned d = sh_claim[par];
    par ^= 1;
    return ((long long)d < plan.nd) ? (long long)d : -1;
  };
  long long w = v;
  if (x >= x1 || s < 0 || s >= B) {  // no static range: start with the first claimed chunk
    if (!tail) return;
    const long long d = claim();
    if (d < 0) return;
    w = plan.ns + d;
    x = plan.start(w);
    x1 = plan.start(w + 1);
    locate(x, s, off);
  }
  int n_s = steps_of(p, s);
  if (n_s == 0) return;  // unreachable: every step lies in a sequence with steps
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int bs = p.block_size;
  const int shift = (bs == 32) ? 5 : 4;
  const size_t tile = (size_t)bs * D;
  const size_t block_elems = (size_t)p.num_kv_heads * tile;
  const float c = p.scale_log2;
  const float slack_raw = kRescaleSlack / c;
  auto head_of = [&](int unit) { return quad ? unit * kWaves + wave : unit; };
  // Source of a piece of unit (ss, hh) starting at step j0: issues its block-id window load.
  auto src_of = [&](int ss, int hh, int j0) __attribute__((always_inline)) {
    MPieceSrc r;
    const int skip_b = skip_blocks(p, ss);
    r.bt = p.block_tables + (size_t)ss * p.max_blocks_per_seq + skip_b;
    r.cols = p.max_blocks_per_seq - skip_b;
    r.win = (j0 * kSub) / bs;
    const int id = (r.win + lane < r.cols) ? r.bt[r.win + lane] : 0;
    r.ids = min(max(id, 0), (int)(p.num_blocks - 1));
    r.head_off = (size_t)hh * tile;
    return r;
  };
  // K/V loads of one 16-token step at element offset `o` of the pools: into the registers `r`,
  // or (FP8) into LDS stage slot `slot` of this wave.
  constexpr int kEl = Fp8 ? 1 : 2;  // bytes per pool element
  auto issue = [&](MStepRegs<D, Fp8>& r, int slot, size_t o) __attribute__((always_inline)) {
    if constexpr (kStaged) {
      const uint8_t* kb = reinterpret_cast<const uint8_t*>(p.kpool) + o * kEl + 16 * lane;
      const uint8_t* vb = reinterpret_cast<const uint8_t*>(p.vpool) + o * kEl + 16 * lane;
      const unsigned dst = __builtin_amdgcn_readfirstlane(
          (unsigned)(uintptr_t)(stage + slot * kStageBytes<D, Fp8>));
#pragma unroll
      for (int c = 0; c < kDmaPerStep<D, Fp8> / 2; ++c)
        lds_dma_16<Stream>(kb + 1024 * c, dst + 1024 * c);
#pragma unroll
      for (int c = 0; c < kDmaPerStep<D, Fp8> / 2; ++c)
        lds_dma_16<Stream>(vb + 1024 * c, dst + kSub * D * kEl + 1024 * c);
      (void)r;
    } else {
      const int r16 = lane & 15, q4 = lane >> 4;
#pragma unroll
      for (int sl = 0; sl < D / kSlice; ++sl)
        r.k[sl] = load_elems<Stream, Fp8>(p.kpool, o + sl * (kSub * kSlice) + r16 * kSlice + 8 * q4);
#pragma unroll
      for (int m = 0; m < D / kSub; ++m)
        r.v[m] = load8_u16<Stream>(p.vpool + o + (size_t)(kSub * m + r16) * kSub + 4 * q4);
    }
    // Staged: keep the compiler from moving the current step's products, which wait for their
    // own loads, ahead of these, so the next step's loads leave as early as the source issues
    // them.
    if constexpr (kStaged) __builtin_amdgcn_sched_barrier(0);
  };

  int hu = (int)div_nonneg(off, n_s);
  int j = (int)(off - (long long)hu * n_s);
  int h = head_of(hu);
  MPieceSrc cs = src_of(s, h, j);
  uint4 qb[D / kSlice];
  load_qb<D, G>(qb, p, s, h);
  // Dep + 1 register sets rotate over the steps; Dep steps' loads are in flight while one is
  // computed.
  static_assert(Dep == 1 || Dep == 2, "prefetch depth");
  MStepRegs<D, Fp8> ra, rb, rc;
  {
    // The first Dep steps of the first piece (a step past the unit repeats its last one: it is
    // then computed fully masked, or not at all).
    auto first = [&](MStepRegs<D, Fp8>& r, int slot, int jj) __attribute__((always_inline)) {
      jj = min(jj, n_s - 1);
      const int b = (jj * kSub) >> shift;  // inside the window just loaded (b - win <= 1)
      const int id = __builtin_amdgcn_readlane(cs.ids, b - cs.win);
      issue(r, slot, (size_t)id * block_elems + cs.head_off + (size_t)((jj * kSub) & (bs - 1)) * D);
    };
    first(ra, 0, j);
    if constexpr (Dep == 2) first(rb, 1, j + 1);
  }
  bool in_a = true;  // register steps: the current piece's first step is in ra
  while (true) {  // each piece starts with its first Dep steps' loads in flight (ra, then rb)
    const int take = (int)min((long long)(n_s - j), x1 - x);
    // The next piece of this worker: the next unit with steps, if the range goes on, else (with
    // the dynamic tail) the first piece of the next claimed chunk.
    int s2 = s, hu2 = hu, n2 = n_s, j2 = 0;
    long long w2 = w, x2 = x + take, x1n = x1;
    bool more = x + take < x1;
    if (more && ++hu2 == U) {
      hu2 = 0;
      do {
        ++s2;
        n2 = (s2 < B) ? steps_of(p, s2) : 0;
      } while (s2 < B && n2 == 0);
      more = s2 < B;
    }
    // The range ends with this piece: the next chunk is claimed inside its walk.
    bool pend = !more && tail;
    if (!more) {  // nothing follows: the "next" source is this piece (its loads hit in cache)
      s2 = s;
      hu2 = hu;
      n2 = n_s;
      j2 = j;
    }
    int h2 = head_of(hu2);
    MPieceSrc ns = src_of(s2, h2, j2);
    uint4 qn[D / kSlice];
    load_qb<D, G>(qn, p, s2, h2);
    // Claims the next chunk and makes it the next piece (its block-id window and query start
    // loading); with none left the next source stays this piece.
    auto resolve = [&]() __attribute__((always_inline)) {
      pend = false;
      const long long d = claim();
      if (d < 0) return;
      w2 = plan.ns + d;
      x2 = plan.start(w2);
      x1n = plan.start(w2 + 1);
      long long off2;
      locate(x2, s2, off2);
      n2 = steps_of(p, s2);
      hu2 = (int)div_nonneg(off2, n2);
      j2 = (int)(off2 - (long long)hu2 * n2);
      more = true;
      h2 = head_of(hu2);
      ns = src_of(s2, h2, j2);
      load_qb<D, G>(qn, p, s2, h2);
    };

    // This piece.
    const int L = uniform(clamped_len(p, s));
    const int u = s * p.num_kv_heads + h;
    const bool whole = (j == 0) && (take == n_s);
    if (j == 0 && lane == 0) p.unit_info[u] = make_int2((int)w, (int)plan.owner(x + n_s - 1, jn));
    const int tok_end = min(L, (j + take) * kSub);
    const int iend = j + take, ilast = iend - 1;
    // The staged walk covers a multiple of Dep + 1 steps; the ones past the piece are fully
    // masked.  The register walk ends with the piece.
    const int iwalk = kStaged ? j + (take + Dep) / (Dep + 1) * (Dep + 1) : iend;
    // The walk's first step at which a pending claim is made (the first loads past the walk need
    // its answer).
    const int icl = max(j, iwalk - max(kClaimLead, kStaged ? Dep + 1 : 1));
    MState<D> st;
    st.m = kNegInf;
    st.nmc = 0.f;
    st.thr = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int m = 0; m < D / kSub; ++m) st.acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Loads of step `step`: inside the piece (a masked step past its end repeats the last one),
    // or, from iwalk on, the next piece's steps (the last step again when nothing follows).  One
    // load path for all, so the compiler's counter waits stay exact.
    auto ld = [&](MStepRegs<D, Fp8>& r, int slot, int step) __attribute__((always_inline)) {
      const bool here = step < iwalk || !more;  // wave-uniform
      int id;
      size_t hoff, tin;
      if (here) {
        const int t0 = min(step, ilast) * kSub;
        const int b = t0 >> shift;
        if (b - cs.win >= 64) {  // rare: refill the block-id window
          cs.win = b;
          const int i2 = (cs.win + lane < cs.cols) ? cs.bt[cs.win + lane] : 0;
          cs.ids = min(max(i2, 0), (int)(p.num_blocks - 1));
        }
        id = __builtin_amdgcn_readlane(cs.ids, b - cs.win);
        hoff = cs.head_off;
        tin = (size_t)(t0 & (bs - 1)) * D;
      } else {  // the next piece's step j2 + (step - iwalk), at the start of its id window
        const int jj = min(j2 + (step - iwalk), n2 - 1);
        id = __builtin_amdgcn_readlane(ns.ids, ((jj * kSub) >> shift) - ns.win);
        hoff = ns.head_off;
        tin = (size_t)((jj * kSub) & (bs - 1)) * D;
      }
      issue(r, slot, (size_t)id * block_elems + hoff + tin);
    };
    // One step: from the registers `r`, or (FP8) from LDS slot `slot` once its loads, and so
    // every older vector-memory operation, are done (the Dep later steps' loads may still fly).
    auto cstep = [&](MStepRegs<D, Fp8>& r, int slot, int i) __attribute__((always_inline)) {
      if constexpr (kStaged) {
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(kDmaPerStep<D, Fp8> * Dep) : "memory");
        const lds_u8* src = stage + slot * kStageBytes<D, Fp8>;
        const int r16 = lane & 15, q4 = lane >> 4;
        MStepRegs<D, Fp8> t;
        // The same elements the register loads take: K slice sl, token r16, elements 8*q4 ..;
        // V row 16m + r16, tokens 4*q4 .. .
#pragma unroll
        for (int sl = 0; sl < D / kSlice; ++sl) {
          const lds_u8* a = src + (sl * (kSub * kSlice) + r16 * kSlice + 8 * q4) * kEl;
          if constexpr (Fp8) {
            const u32x2_t k = *(const __attribute__((address_space(3))) u32x2_t*)a;
            t.k[sl] = make_uint2(k.x, k.y);
          } else {
            const u32x4_t k = *(const __attribute__((address_space(3))) u32x4_t*)a;
            t.k[sl] = make_uint4(k.x, k.y, k.z, k.w);
          }
        }
#pragma unroll
        for (int m = 0; m < D / kSub; ++m) {
          const lds_u8* a = src + (kSub * D + (kSub * m + r16) * kSub + 4 * q4) * kEl;
          if constexpr (Fp8) {
            t.v[m] = *(const __attribute__((address_space(3))) uint32_t*)a;
          } else {
            const u32x2_t v = *(const __attribute__((address_space(3))) u32x2_t*)a;
            t.v[m] = make_uint2(v.x, v.y);
          }
        }
        compute_mstep<D, Fp8>(t, qb, tok_end - i * kSub, c, slack_raw, st);
        (void)r;
      } else {
        compute_mstep<D, Fp8>(r, qb, tok_end - i * kSub, c, slack_raw, st);
      }
    };
    if constexpr (kStaged) {
      // Staged steps rotate through the LDS slots, Dep + 1 per iteration, each slot refilled Dep
      // steps ahead as soon as it is free.  The walk is padded with fully masked steps (they add
      // nothing) to whole rotations, so the next piece's first steps always land in slots 0
      // (and 1), and the walk exists once in the compiled code.
      // A step past the piece only keeps the loads regular (each wait counts a fixed number of
      // loads per step); its product is skipped.  The compiler does not track the staged loads,
      // so the branch costs no extra counter waits.
      for (int i = j; i < iwalk; i += Dep + 1) {
        if (pend && i >= icl) resolve();
        if constexpr (Dep == 1) {
          ld(rb, 1, i + 1);
          cstep(ra, 0, i);
          ld(ra, 0, i + 2);
          if (i + 1 < iend) cstep(rb, 1, i + 1);
        } else {
          ld(rc, 2, i + 2);
          cstep(ra, 0, i);
          ld(ra, 0, i + 3);
          if (i + 1 < iend) cstep(rb, 1, i + 1);
          ld(rb, 1, i + 4);
          if (i + 2 < iend) cstep(rc, 2, i + 2);
        }
      }
    } else {
      static_assert(kStaged || Dep == 1, "register steps prefetch one step");
      // Register steps alternate between the two register sets; returns true when the last step
      // was in `first` (the next piece's first step then sits in `second`).  Both orders are
      // compiled, so no step past the piece is computed.
      auto walk = [&](MStepRegs<D, Fp8>& first, MStepRegs<D, Fp8>& second)
                      __attribute__((always_inline)) {
        int i = j;
        while (true) {
          if (pend && i >= icl) resolve();
          ld(second, 1, i + 1);
          cstep(first, 0, i);
          if (++i >= iend) return true;
          if (pend && i >= icl) resolve();
          ld(first, 0, i + 1);
          cstep(second, 1, i);
          if (++i >= iend) return false;
        }
      };
      const bool swap = in_a ? walk(ra, rb) : walk(rb, ra);
      in_a = swap ? !in_a : in_a;
    }
    finish_mpiece<D, G>(p, st, s, h, u, w, whole, nullptr);
    if (!more) break;
    x = x2;
    x1 = x1n;
    w = w2;
    ++jn;
    s = s2;
    hu = hu2;
    n_s = n2;
    h = h2;
    j = j2;
    cs = ns;
#pragma unroll
    for (int sl = 0; sl < D / kSlice; ++sl) qb[sl] = qn[sl];
  }
}

// A piece taken by the whole workgroup: wave r runs steps [j0 + take*r/kWaves,
// j0 + take*(r+1)/kWaves) into its LDS slot, then the workgroup combines the slots in wave order
// and writes the output (unit wholly inside the piece) or the piece's partial slot.  Contains
// barriers: every wave of the block must call it with the same arguments.
template <int D, int G, int Depth, bool Stream, bool Fp8, bool Mfma>
__device__ __forceinline__ void coop_piece(const DecodeParams& p, int s, int h, int j0, int take,
                                           int n_s, long long w, long long x, long long jn,
                                           const Plan& plan, uint16_t (*p_sh)[G][8],
                                           float (*st)[G * (2 + D)]) {
  constexpr int PER = (G * D + kThreads - 1) / kThreads;
  const int wave = threadIdx.x >> 6;
  auto lo_of = [&](int r) { return j0 + (int)((long long)take * r / kWaves); };
  const int a = lo_of(wave), b = lo_of(wave + 1);
  if (b > a) {
    if constexpr (Mfma)
      decode_piece_mfma<D, G, Depth, Stream, Fp8>(p, s, h, a, b - a, n_s, w, x + (a - j0), jn,
                                                  plan, st[wave]);
    else
      decode_piece<D, G, Depth, Stream>(p, s, h, a, b - a, n_s, w, x + (a - j0), jn, plan, p_sh,
                                        st[wave]);
  }
  __syncthreads();
  const int u = s * p.num_kv_heads + h;
  const bool whole = (j0 == 0) && (take == n_s);
  if (j0 == 0 && threadIdx.x == 0)
    p.unit_info[u] = make_int2((int)w, (int)plan.owner(x + n_s - 1, jn));
  float* slot = p.partials + slot_of(p, w, u) * (G * (2 + D));
  uint16_t* orow = p.out + ((size_t)s * p.num_q_heads + (size_t)h * G) * D;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + kThreads * k;
    if (i >= G * D) break;
    const int g = i / D;
    float M = kNegInf;
#pragma unroll
    for (int r = 0; r < kWaves; ++r)
      if (lo_of(r + 1) > lo_of(r)) M = fmaxf(M, st[r][g]);
    float lt = 0.f, acc = 0.f;
#pragma unroll
    for (int r = 0; r < kWaves; ++r) {
      if (lo_of(r + 1) > lo_of(r)) {
        const float e = fast_exp2(st[r][g] - M);
        lt += e * st[r][G + g];
        acc += e * st[r][2 * G + i];
      }
    }
    if (whole && p.state_ml) {
      const size_t su = state_slot(p, (size_t)s * p.num_q_heads + (size_t)h * G + g);
      if (i % D == 0) {
        p.state_ml[2 * su] = M;
        p.state_ml[2 * su + 1] = lt;
      }
      p.state_acc[su * D + i % D] = acc * p.v_scale;
    } else if (whole) {
      orow[i] = to_bf16(acc * p.v_scale / lt);
    } else {
      if (i % D == 0) {
        slot[g] = M;
        slot[G + g] = lt;
      }
      slot[2 * G + i] = acc;
    }
  }
  __syncthreads();  // the slots are rewritten by the next piece
}

// Steps [x, x1) of virtual worker v, unit by unit.  (s, off) locate its first step: sequence s
// and offset within that sequence's U * n_s steps, U = num_kv_heads units per sequence, or with
// `quad` num_kv_heads / kWaves units of kWaves consecutive KV heads, wave r taking head
// kWaves*unit + r (the workgroup is the worker); jn is that unit's index among the non-empty
// units.  Coop: each piece is shared by the workgroup.
template <int D, int G, int Depth, bool Stream, bool Fp8, bool Mfma, bool Coop = false>
__device__ __forceinline__ void run_worker(const DecodeParams& p, const Plan& plan, long long v,
                                           int s, long long off, long long jn, long long x,
                                           long long x1, uint16_t (*p_sh)[G][8],
                                           float (*st)[G * (2 + D)] = nullptr, bool quad = false,
                                           lds_u8* stage = nullptr) {
  if constexpr (Mfma && !Coop) {
    run_worker_mfma<D, G, (Depth >= 2 ? 2 : 1), Stream, Fp8>(p, plan, v, s, off, jn, x, x1, quad,
                                                             stage);
    return;
  }
  const int B = p.num_seqs;
  const int Hkv = quad ? p.num_kv_heads / kWaves : p.num_kv_heads;
  if (x >= x1 || s < 0 || s >= B) return;
  int n_s = steps_of(p, s);
  if (n_s == 0) return;  // unreachable: every step lies in a sequence with steps
  int h = (int)(off / n_s);
  int j = (int)(off % n_s);
  while (true) {
    const int take = (int)min((long long)(n_s - j), x1 - x);
    if constexpr (Coop)
      coop_piece<D, G, Depth, Stream, Fp8, Mfma>(p, s, h, j, take, n_s, v, x, jn, plan, p_sh, st);
    else if constexpr (Mfma)
      decode_piece_mfma<D, G, Depth, Stream, Fp8>(
          p, s, quad ? h * kWaves + (int)(threadIdx.x >> 6) : h, j, take, n_s, v, x, jn, plan);
    else
      decode_piece<D, G, Depth, Stream>(p, s, quad ? h * kWaves + (int)(threadIdx.x >> 6) : h, j,
                                        take, n_s, v, x, jn, plan, p_sh);
    x += take;
    if (x >= x1) break;
    j = 0;
    ++jn;
    if (++h == Hkv) {
      h = 0;
      do {
        ++s;
        n_s = (s < B) ? steps_of(p, s) : 0;
      } while (s < B && n_s == 0);
      if (s >= B) break;
    }
  }
}

// Fp8: the pools hold E4M3 codes (always on the matrix cores).  Mfma: matrix-core steps.
template <int D, int G, int Depth, bool Fp8, bool Mfma = Fp8>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  // Alone on the chip the decode has one wave per SIMD and its priority changes nothing.  Beside
  // a prefill chunk (the mixed step) a raised priority lets the bf16 decode's waves issue their
  // loads ahead of the chunk's vector work: 551 against 558 us a step.  The FP8 step measured
  // 10 us slower with it, so FP8 decode keeps the normal priority.
  if constexpr (!Fp8) __builtin_amdgcn_s_setprio(1);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int B = p.num_seqs;
  const int Hkv = p.num_kv_heads;

  __shared__ long long sh_sum[kWaves];
  __shared__ int sh_nonempty[kWaves];
  __shared__ int sh_shares[kWaves];
  __shared__ int sh_scan[kWaves];
  __shared__ int sh_scan_ne[kWaves];
  // Start of each of this block's workers and of the next block's first one: sequence, offset
  // within the sequence's steps, non-empty unit index, global step.
  __shared__ int sh_start_s[kWaves + 1];
  __shared__ long long sh_start_off[kWaves + 1];
  __shared__ long long sh_start_j[kWaves + 1];
  __shared__ long long sh_start_x[kWaves + 1];
  __shared__ __attribute__((aligned(16))) uint16_t p_lds[kWaves][2][G][8];
  __shared__ unsigned sh_chunk;
  __shared__ unsigned sh_claim[2];  // dynamic-tail claims, in turn
  __shared__ float coop_st[kWaves][G * (2 + D)];  // per-wave (m, l, acc) of a shared piece
  // Per-wave ring of staged steps (FP8 matrix-core steps; a placeholder otherwise).
  constexpr bool kStagedK = Mfma && (Fp8 || kStageBf16);
  constexpr int kSlots = kStagedK ? (Depth >= 2 ? 3 : 2) : 1;
  __shared__ __attribute__((aligned(16))) uint8_t
      stage_lds[kWaves][kSlots][kStagedK ? kStageBytes<D, Fp8> : 16];
  extern __shared__ int seq_prefix[];  // [B+1] steps per KV head before each sequence (dynamic mode)

  // Prefix sharing (several sequences reading the same physical blocks, as when many samples
  // continue one prompt) shows as a sequence starting at the same block as the next one.  Such a
  // batch re-reads blocks, so its K/V loads stay ordinary; any other batch streams them.
  int shares = 0;
  const size_t row = (size_t)p.max_blocks_per_seq;
  // Total steps of the batch.  The first kThreads sequences' step counts stay in a register for
  // the prefix sums below, so small batches read their lengths once.
  int n_first = 0;
  if (!p.skip_lens && B > 0 && row > 0) {
    // Nothing skipped: the first probe compares first table entries, which do not depend on the
    // lengths, so its two loads go out with the length load and the three share one round trip
    // (taken one after the other they cost two at the start of every launch).  The loads are
    // unconditional, at indices clamped into the batch, so that no branch holds a wait.
    const int t = threadIdx.x;
    const int len = p.seq_lens[min(t, B - 1)];
    const int e0 = p.block_tables[(size_t)min(t, B - 1) * row];
    const int e1 = p.block_tables[(size_t)min(t + 1, B - 1) * row];
    n_first = t < B ? (max(min(max(len, 0), p.len_cap), 0) + kSub - 1) / kSub : 0;  // steps_of
    shares = t + 1 < B && e0 == e1;
  } else if ((int)threadIdx.x < B) {
    n_first = steps_of(p, threadIdx.x);
  }
  long long mine = n_first;
  int nonempty = n_first > 0;
  for (int s = threadIdx.x + kThreads; s < B; s += kThreads) {
    const int n = steps_of(p, s);
    mine += n;
    nonempty += n > 0;
  }
  // With leading blocks skipped (the cascade's tails) the shared prefix has been taken out and
  // attended once elsewhere, so no probe is made and the tails stream: probing their first
  // attended entries would wait for the skips first.
  for (int s = threadIdx.x + kThreads; !p.skip_lens && row > 0 && s + 1 < B; s += kThreads)
    shares |= p.block_tables[(size_t)s * row] == p.block_tables[(size_t)(s + 1) * row];
  shares = __any(shares);
  // When every per-head step count of the batch fits an int (it does unless the batch holds 2^35
  // tokens per head), DPP scans serve; otherwise 64-bit shuffles give the wave totals.
  const bool int_sums = (long long)B * ((p.len_cap + kSub - 1) / kSub) < (1LL << 31);
  // One pass (a batch of at most kThreads sequences, one per thread): the wave scans of the step
  // counts give the totals and the prefix sums at once, so a single barrier publishes both and a
  // second one the workers' starts (four barriers in the general form).
  const bool one_pass = B <= kThreads && int_sums;
  int incl0 = 0, ne_incl0 = 0;
  if (one_pass) {
    incl0 = wave_inclusive_scan(n_first);
    ne_incl0 = wave_inclusive_scan(nonempty);  // n_first > 0: no second chunk added to it
    if (lane == 63) {
      sh_scan[wave] = incl0;
      sh_scan_ne[wave] = ne_incl0;
      sh_shares[wave] = shares;
    }
  } else {
    nonempty = __builtin_amdgcn_readlane(wave_inclusive_scan(nonempty), 63);
    if (int_sums) {
      mine = __builtin_amdgcn_readlane(wave_inclusive_scan((int)mine), 63);
    } else {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o, 64);
    }
    if (lane == 0) {
      sh_sum[wave] = mine;
      sh_nonempty[wave] = nonempty;
      sh_shares[wave] = shares;
    }
  }
  __syncthreads();
  long long per_head = 0;
  long long seqs_nonempty = 0;
  bool shared = false;
  int before0 = 0, ne_before0 = 0;  // one pass: the waves before this one
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    if (one_pass) {
      per_head += sh_scan[k];
      seqs_nonempty += sh_scan_ne[k];
      before0 += (k < wave) ? sh_scan[k] : 0;
      ne_before0 += (k < wave) ? sh_scan_ne[k] : 0;
    } else {
      per_head += sh_sum[k];
      seqs_nonempty += sh_nonempty[k];
    }
    shared |= sh_shares[k] != 0;
  }
  // quad: the workgroup is one worker over units of kWaves consecutive KV heads.
  const bool quad = p.quad != 0;
  const int U = quad ? Hkv / kWaves : Hkv;  // units per sequence
  Plan plan;
  plan.T = per_head * U;
  if (plan.T == 0) return;  // block-uniform
  const long long workers = quad ? (long long)gridDim.x : (long long)p.num_workers;
  plan.ns = min(workers, max(seqs_nonempty * U, (plan.T + kMinStepsPerWave - 1) / kMinStepsPerWave));
  // Dynamic chunks only when a share of the steps is left to them: with the whole batch split
  // statically the plan (piece cost included) does not depend on the workspace's chunk slots.
  const bool dynamic =
      !quad && p.dyn_cap > 0 && p.static_frac_q10 < 1024 && plan.ns == p.num_workers;
  // Dynamic tail of the head-quad split: chunk d is worker ns + d, whose partial slots
  // (ns + d + u/kWaves)*kWaves + u%kWaves stay inside the workspace for d < dyn_cap/kWaves.
  const bool tail = Mfma && Depth <= 1 && quad && p.tail_q10 > 0 && p.dyn_cap > 0;
  if (tail) {
    plan.S = max(plan.ns, plan.T - plan.T * p.tail_q10 / 1024);
    const long long rest = plan.T - plan.S;
    const long long cap = p.dyn_cap / kWaves;
    plan.C = max((long long)max(p.tail_chunk, 1), (rest + cap - 1) / cap);
    plan.nd = (rest + plan.C - 1) / plan.C;
  } else if (dynamic) {
    plan.S = max(plan.ns, plan.T * p.static_frac_q10 / 1024);
    const long long rest = plan.T - plan.S;
    plan.C = max((long long)p.chunk_steps, (rest + p.dyn_cap - 1) / p.dyn_cap);
    plan.nd = (rest + plan.C - 1) / plan.C;
  } else {
    plan.S = plan.T;
    plan.C = 1;
    plan.nd = 0;
  }
  // Piece cost, kept below half a worker's share of steps so that no static worker's cost range
  // falls inside one piece's overhead (every static worker gets at least one step).
  plan.A = (dynamic || tail) ? 0 : min((long long)p.piece_cost, div_nonneg(plan.T, plan.ns) / 2);
  plan.CT = plan.S + plan.A * seqs_nonempty * U;
  const long long wbase = (long long)blockIdx.x * kWaves;
  // Workers whose starts this block needs: its own (1 with quads, else kWaves) and the next one.
  const int n_own = quad ? 1 : kWaves;
  const long long wfirst = quad ? (long long)blockIdx.x : wbase;
  // Sequence s has n steps per head, excl steps per head before it and ne_excl non-empty
  // sequences before it: record it as the start of every worker of this block whose target
  // falls in its cost range.  The ranges of the non-empty sequences tile [0, CT), so each static
  // worker's start is written by exactly one thread.
  auto place = [&](int s, int n, long long excl, long long ne_excl) {
    if ((dynamic || tail) && s < B) seq_prefix[s] = (int)excl;
    if (n <= 0) return;
    // The sequence's U units cover cost positions [c_lo, c_lo + U*(n + A)).
    const long long lo = excl * U;
    const long long j0 = ne_excl * U;
    const long long c_lo = lo + plan.A * j0;
    const long long per_unit = n + plan.A;
    for (int k = 0; k <= n_own; ++k) {
      const long long wk = wfirst + k;
      if (wk >= plan.ns) break;
      const long long t = plan.target(wk);
      if (t >= c_lo && t < c_lo + U * per_unit) {
        const long long kk = div_nonneg(t - c_lo, per_unit);
        const long long o = max(0LL, t - c_lo - kk * per_unit - plan.A);
        sh_start_s[k] = s;
        sh_start_off[k] = kk * n + o;
        sh_start_j[k] = j0 + kk;
        sh_start_x[k] = lo + kk * n + o;
      }
    }
  };
  // Workers at or past ns start (and end) at S.  In one pass only they take the defaults, so no
  // barrier has to order the defaults before the placements.
  if ((int)threadIdx.x <= n_own && (!one_pass || wfirst + (int)threadIdx.x >= plan.ns)) {
    sh_start_s[threadIdx.x] = -1;
    sh_start_off[threadIdx.x] = 0;
    sh_start_j[threadIdx.x] = 0;
    sh_start_x[threadIdx.x] = plan.S;
  }
  long long base = 0;
  if (one_pass) {
    place(threadIdx.x, n_first, before0 + incl0 - n_first, ne_before0 + ne_incl0 - (n_first > 0));
    base = per_head;
  } else {
    __syncthreads();
    // Prefix sums over sequences, kThreads at a time: locate where each static worker of this
    // block starts, and keep the prefix in LDS for the dynamic chunks.
    long long ne_base = 0;
    for (int c = 0; c < B; c += kThreads) {
      const int s = c + threadIdx.x;
      const int n = (c == 0) ? n_first : (s < B ? steps_of(p, s) : 0);
      const int ne = n > 0;
      const int incl = wave_inclusive_scan(n);
      const int ne_incl = wave_inclusive_scan(ne);
      if (lane == 63) {
        sh_scan[wave] = incl;
        sh_scan_ne[wave] = ne_incl;
      }
      __syncthreads();
      int before = 0, chunk = 0, ne_before = 0, ne_chunk = 0;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        before += (k < wave) ? sh_scan[k] : 0;
        chunk += sh_scan[k];
        ne_before += (k < wave) ? sh_scan_ne[k] : 0;
        ne_chunk += sh_scan_ne[k];
      }
      place(s, n, base + before + incl - n, ne_base + ne_before + ne_incl - ne);
      base += chunk;
      ne_base += ne_chunk;
      if (c + kThreads < B) __syncthreads();  // the next chunk rewrites sh_scan
    }
  }
  if ((dynamic || tail) && threadIdx.x == 0) seq_prefix[B] = (int)base;
  __syncthreads();  // publishes sh_start_* and seq_prefix

  const long long w = quad ? (long long)blockIdx.x : wbase + wave;
  // One instantiation of the worker per load kind (the choice is uniform over the grid).
  auto body = [&](auto stream) {
    constexpr bool S = decltype(stream)::value;
    const int k = quad ? 0 : wave;
    if constexpr (Mfma && Depth <= 1) {
      if (tail) {  // every workgroup: its static range (possibly empty), then claimed chunks
        const bool own = w < plan.ns;
        run_worker_mfma<D, G, 1, S, Fp8>(p, plan, w, own ? sh_start_s[k] : -1,
                                      sh_start_off[k], sh_start_j[k],
                                      own ? sh_start_x[k] : plan.S,
                                      own ? sh_start_x[k + 1] : plan.S, quad,
                                      (lds_u8*)&stage_lds[wave][0][0], true, seq_prefix,
                                      sh_claim);
        return;
      }
    }
    if (w < plan.ns)
      run_worker<D, G, Depth, S, Fp8, Mfma>(p, plan, w, sh_start_s[k], sh_start_off[k],
                                            sh_start_j[k], sh_start_x[k], sh_start_x[k + 1],
                                            p_lds[wave], nullptr, quad,
                                            (lds_u8*)&stage_lds[wave][0][0]);
    if (!dynamic) return;  // block-uniform

    // Dynamic chunks, each shared by the whole workgroup (one counter increment per chunk; the
    // next chunk is claimed while the current one runs).  In dynamic mode every wave has a static
    // range (plan.ns == num_workers), so all waves reach these barriers.
    if (threadIdx.x == 0) sh_chunk = atomicAdd(p.counter, 1u);
    __syncthreads();
    while (true) {
      const unsigned d = sh_chunk;  // block-uniform
      if ((long long)d >= plan.nd) break;
      unsigned nxt = 0;
      if (threadIdx.x == 0) nxt = atomicAdd(p.counter, 1u);
      // Locate the chunk's first step: the last sequence whose prefix is <= x / Hkv.
      const long long x0 = plan.start(plan.ns + d);
      const long long xh = x0 / Hkv;
      int lo = 0, hi = B;  // invariant: seq_prefix[lo] <= xh < seq_prefix[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seq_prefix[mid] <= xh) lo = mid;
        else hi = mid;
      }
      run_worker<D, G, Depth, S, Fp8, Mfma, true>(p, plan, plan.ns + d, lo,
                                       x0 - (long long)seq_prefix[lo] * Hkv, 0, x0,
                                       plan.start(plan.ns + d + 1), p_lds[wave], coop_st);
      __syncthreads();  // every thread has read sh_chunk
      if (threadIdx.x == 0) sh_chunk = nxt;
      __syncthreads();
    }
  };
  if (shared) body(std::false_type{});
  else body(std::true_type{});
}

// Merge thread layout: thread t owns chunks c = t + 256*k of four consecutive head-dim values,
// row (4c)/D of the unit's G query heads, so each source of a chunk is one (m, l) pair and one
// 16-byte acc load.  A partial slot holds G*(2+D) floats, so with G odd a slot's acc is only
// 8-byte aligned: the acc loads assume 4-byte alignment.
typedef float f32x4u_t __attribute__((ext_vector_type(4), aligned(4)));

template <int D, int G>
struct MergeLayout {
  static constexpr int kChunks = G * D / 4;
  static constexpr int kPer = (kChunks + 255) / 256;  // chunks per thread
  // Chunk k of this thread, clamped to the last so every thread's loads stay inside the unit.
  __device__ static int chunk(int k) { return min((int)threadIdx.x + 256 * k, kChunks - 1); }
  __device__ static bool owns(int k) { return (int)threadIdx.x + 256 * k < kChunks; }
};

// Fold one (m, l, acc) source into a running state, in the log2 domain; an empty source (m =
// -inf) changes nothing.
__device__ __forceinline__ void merge_fold(float& M, float& lt, f32x4_t& a, float mv, float lv,
                                           f32x4_t av) {
  if (mv == kNegInf) return;
  const float mn = fmaxf(M, mv);
  const float c_old = fast_exp2(M - mn);  // M = -inf on the first source: c_old = 0
  const float c_new = fast_exp2(mv - mn);
  lt = lt * c_old + lv * c_new;
  a = a * c_old + av * c_new;
  M = mn;
}

// Combine the pieces of every unit that spans several waves; write zeros for empty sequences.
// One pass over the pieces with an online rescale, four pieces' loads issued together.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
  using L = MergeLayout<D, G>;
  constexpr int PER = L::kPer;
  const int u = blockIdx.x;
  const int s = u / p.num_kv_heads;
  const int h = u % p.num_kv_heads;
  if (u == 0 && threadIdx.x == 0) *p.counter = 0u;  // ready for the next call
  uint16_t* orow = p.out + ((size_t)s * p.num_q_heads + (size_t)h * G) * D;
  const size_t row0 = (size_t)s * p.num_q_heads + (size_t)h * G;
  // The unit's worker range is loaded with the length, before the branch on it, so the two
  // share one round trip.  (An empty sequence's range is stale and never read.)
  int2 info = p.unit_info[u];
  if (clamped_len(p, s) == 0) {
    if (p.state_ml) {  // no keys here: an empty state
      for (int i = threadIdx.x; i < G * D; i += 256) {
        const size_t su = state_slot(p, row0 + i / D);
        if (i % D == 0) {
          p.state_ml[2 * su] = kNegInf;
          p.state_ml[2 * su + 1] = 0.f;
        }
        p.state_acc[su * D + i % D] = 0.f;
      }
      return;
    }
    for (int i = threadIdx.x; i < G * D; i += 256) orow[i] = 0;
    return;
  }
  info.x = max(info.x, 0);
  info.y = min(info.y, p.num_workers + p.dyn_cap - 1);
  if (info.x >= info.y) return;  // written by its only wave
  float M[PER], lt[PER];
  f32x4_t a[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    M[k] = kNegInf;
    lt[k] = 0.f;
    a[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // Rounds of four pieces' loads, or eight when the unit has more than four pieces (units split
  // over many waves, as with one KV head): a unit's pieces then arrive in one round trip.  The
  // fold order is the same either way.
  auto fold_all = [&](auto round_c) __attribute__((always_inline)) {
    constexpr int kRound = decltype(round_c)::value;
    for (int w0 = info.x; w0 <= info.y; w0 += kRound) {
      float mv[kRound][PER], lv[kRound][PER];
      f32x4_t av[kRound][PER];
#pragma unroll
      for (int r = 0; r < kRound; ++r) {
        const int w = min(w0 + r, info.y);
        const float* slot = p.partials + slot_of(p, w, u) * (G * (2 + D));
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const int c = L::chunk(k);
          mv[r][k] = slot[4 * c / D];
          lv[r][k] = slot[G + 4 * c / D];
          av[r][k] = *(const f32x4u_t*)(slot + 2 * G + 4 * c);
        }
      }
#pragma unroll
      for (int r = 0; r < kRound; ++r) {
        if (w0 + r > info.y) break;
#pragma unroll
        for (int k = 0; k < PER; ++k)
          merge_fold(M[k], lt[k], a[k], mv[r][k], lv[r][k], av[r][k]);
      }
    }
  };
  if (info.y - info.x >= 4)  // block-uniform
    fold_all(std::integral_constant<int, 8>{});
  else
    fold_all(std::integral_constant<int, 4>{});
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (!L::owns(k)) continue;
    const int c = L::chunk(k);
    const f32x4_t o = a[k] * p.v_scale;
    if (p.state_ml) {
      const size_t su = state_slot(p, row0 + 4 * c / D);
      if ((4 * c) % D == 0) {
        p.state_ml[2 * su] = M[k];
        p.state_ml[2 * su + 1] = lt[k];
      }
      *(f32x4_t*)(p.state_acc + su * D + (4 * c) % D) = o;
    } else {
      *(uint2*)(orow + 4 * c) = make_uint2(pack_bf16x2(o[0] / lt[k], o[1] / lt[k]),
                                           pack_bf16x2(o[2] / lt[k], o[3] / lt[k]));
    }
  }
}

// The final merge of a cascade call: every (sequence, query head) row combines the shared
// prompt's states (splits 0 .. state_split-1 of the state workspace, in split order) with its
// own tail, taken from the tail's pieces when several waves shared it, from the tail state the
// decode kernel wrote when one wave took it whole, and left out when the row has no tail, then
// writes the normalised output.
template <int D, int G>
__global__ __launch_bounds__(256) void cascade_merge_kernel(DecodeParams p) {
  using L = MergeLayout<D, G>;
  constexpr int PER = L::kPer;
  const int u = blockIdx.x;
  const int s = u / p.num_kv_heads;
  const int h = u % p.num_kv_heads;
  if (u == 0 && threadIdx.x == 0) *p.counter = 0u;  // ready for the next call
  const size_t row0 = (size_t)s * p.num_q_heads + (size_t)h * G;
  int2 info = p.unit_info[u];
  info.x = max(info.x, 0);
  info.y = min(info.y, p.num_workers + p.dyn_cap - 1);
  const bool tail = clamped_len(p, s) > 0;
  const bool pieces = tail && info.x < info.y;
  // Sources in combination order: the workspace states (the prompt's splits, then the tail's
  // when it was written whole), then the tail's pieces in worker order.
  const int nstates = p.state_split + ((tail && !pieces) ? 1 : 0);
  const int nsrc = nstates + (pieces ? info.y - info.x + 1 : 0);
  float M[PER], lt[PER];
  f32x4_t a[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    M[k] = kNegInf;
    lt[k] = 0.f;
    a[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // Eight sources per round: their loads are issued together, then folded in order.  The source
  // of each load is picked by selecting its address, not by branching, so no wait for earlier
  // loads separates them.  A piece's acc still lacks the V scale, which the workspace states
  // carry.
  constexpr int kRound = 8;
  for (int q0 = 0; q0 < nsrc; q0 += kRound) {
    float mv[kRound][PER], lv[kRound][PER], sc[kRound];
    f32x4_t av[kRound][PER];
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const int q = min(q0 + r, nsrc - 1);
      const bool is_state = q < nstates;  // block-uniform
      const float* slot =
          p.partials + slot_of(p, info.x + max(q - nstates, 0), u) * (G * (2 + D));
      sc[r] = is_state ? 1.f : p.v_scale;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int c = L::chunk(k);
        const size_t su = (row0 + 4 * c / D) * p.state_stride + q;
        const float* pm = is_state ? p.state_ml + 2 * su : slot + 4 * c / D;
        const float* pl = is_state ? p.state_ml + 2 * su + 1 : slot + G + 4 * c / D;
        const float* pv = is_state ? p.state_acc + su * D + (4 * c) % D : slot + 2 * G + 4 * c;
        mv[r][k] = *pm;
        lv[r][k] = *pl;
        av[r][k] = *(const f32x4u_t*)pv;
      }
    }
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      if (q0 + r >= nsrc) break;
#pragma unroll
      for (int k = 0; k < PER; ++k)
        merge_fold(M[k], lt[k], a[k], mv[r][k], lv[r][k], av[r][k] * sc[r]);
    }
  }
  uint16_t* orow = p.out + row0 * D;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (!L::owns(k)) continue;
    const int c = L::chunk(k);
    const float inv = lt[k] > 0.f ? 1.f / lt[k] : 0.f;
    const f32x4_t o = a[k] * inv;
    *(uint2*)(orow + 4 * c) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
  }
}

// Which decode_kernel instantiation a call launches.  FP8 pools always run on the matrix-core
// step, with prefetch depth 1 or 2.  bf16 pools run on the matrix-core step by default:
// offloading the products frees the vector issue slots the bf16 step spends most of its time
// in, which at the 70B shape makes the kernel about 2 % faster; the vector step (prefetch depth
// 0, 1 or 2) stays selectable.
enum class Variant { kFp8Depth1, kFp8Depth2, kBf16Mfma, kVecDepth0, kVecDepth1, kVecDepth2 };

Variant variant(bool fp8) {
  if (fp8) return tunable(kTuneDecodePrefetchFp8) == 2 ? Variant::kFp8Depth2 : Variant::kFp8Depth1;
  if (tunable(kTuneDecodeMfma)) return Variant::kBf16Mfma;
  switch (tunable(kTuneDecodePrefetch)) {
    case 0: return Variant::kVecDepth0;
    case 2: return Variant::kVecDepth2;
    default: return Variant::kVecDepth1;
  }
}

template <int D, int G>
const void* kernel_of(Variant v) {
  switch (v) {
    case Variant::kFp8Depth1: return reinterpret_cast<const void*>(&decode_kernel<D, G, 1, true>);
    case Variant::kFp8Depth2: return reinterpret_cast<const void*>(&decode_kernel<D, G, 2, true>);
    case Variant::kBf16Mfma:
      return reinterpret_cast<const void*>(&decode_kernel<D, G, 1, false, true>);
    case Variant::kVecDepth0: return reinterpret_cast<const void*>(&decode_kernel<D, G, 0, false>);
    case Variant::kVecDepth2: return reinterpret_cast<const void*>(&decode_kernel<D, G, 2, false>);
    default: return reinterpret_cast<const void*>(&decode_kernel<D, G, 1, false>);
  }
}

template <int D, int G>
hipError_t launch_dg(const DecodeParams& p, hipStream_t stream) {
  {
    TraceScope t("decode_partition", stream);
    const dim3 grid(p.num_workers / kWaves), block(kThreads);
    // The per-sequence prefix of the dynamic chunks (either kind).
    const size_t lds = (p.dyn_cap > 0 && (p.static_frac_q10 < 1024 || p.tail_q10 > 0))
                           ? (size_t)(p.num_seqs + 1) * 4
                           : 0;
    switch (variant(p.kv_fp8 != 0)) {
      case Variant::kFp8Depth1:
        hipLaunchKernelGGL((decode_kernel<D, G, 1, true>), grid, block, lds, stream, p);
        break;
      case Variant::kFp8Depth2:
        hipLaunchKernelGGL((decode_kernel<D, G, 2, true>), grid, block, lds, stream, p);
        break;
      case Variant::kBf16Mfma:
        hipLaunchKernelGGL((decode_kernel<D, G, 1, false, true>), grid, block, lds, stream, p);
        break;
      case Variant::kVecDepth0:
        hipLaunchKernelGGL((decode_kernel<D, G, 0, false>), grid, block, lds, stream, p);
        break;
      case Variant::kVecDepth2:
        hipLaunchKernelGGL((decode_kernel<D, G, 2, false>), grid, block, lds, stream, p);
        break;
      default:
        hipLaunchKernelGGL((decode_kernel<D, G, 1, false>), grid, block, lds, stream, p);
        break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.state_final) {
    TraceScope t("cascade_merge", stream);
    hipLaunchKernelGGL((cascade_merge_kernel<D, G>), dim3(p.num_seqs * p.num_kv_heads),
                       dim3(256), 0, stream, p);
  } else {
    TraceScope t("decode_merge", stream);
    hipLaunchKernelGGL((decode_merge_kernel<D, G>), dim3(p.num_seqs * p.num_kv_heads), dim3(256),
                       0, stream, p);
  }
  return hipGetLastError();
}

// Dispatch over the supported (head_dim, group) pairs; `fallback` for any other pair.
template <typename Ret, typename F>
Ret dispatch(int D, int G, Ret fallback, F&& f) {
  switch (D) {
    case 64:
      switch (G) {
        case 1: return f.template operator()<64, 1>();
        case 2: return f.template operator()<64, 2>();
        case 4: return f.template operator()<64, 4>();
        case 8: return f.template operator()<64, 8>();
        case 16: return f.template operator()<64, 16>();
      }
      break;
    case 128:
      switch (G) {
        case 1: return f.template operator()<128, 1>();
        case 2: return f.template operator()<128, 2>();
        case 4: return f.template operator()<128, 4>();
        case 8: return f.template operator()<128, 8>();
      }
      break;
    case 256:
      switch (G) {
        case 1: return f.template operator()<256, 1>();
        case 2: return f.template operator()<256, 2>();
        case 4: return f.template operator()<256, 4>();
      }
      break;
  }
  return fallback;
}

}  // namespace

int decode_workers(int head_dim, int group, bool fp8) {
  static std::mutex mu;
  // (device, shape, launched variant) -> (default workgroups, resident workgroups)
  static std::map<std::pair<int, int>, std::pair<int, int>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const Variant v = variant(fp8);
  std::pair<int, int> blocks{0, 0};
  {
    std::lock_guard<std::mutex> lk(mu);
    const auto key = std::make_pair(dev, (head_dim * 64 + group) * 8 + (int)v);
    auto it = cache.find(key);
    if (it != cache.end()) {
      blocks = it->second;
    } else {
      int cus = 0, per_cu = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
      // Residency of the instantiation this call launches.
      const void* fn = dispatch(head_dim, group, (const void*)nullptr,
                                [v]<int D, int G>() { return kernel_of<D, G>(v); });
      if (!fn || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads,
                                                              kPrefixLdsBytes) != hipSuccess)
        return 0;
      per_cu = std::max(per_cu, 1);
      // One workgroup (one wave per SIMD) per CU by default: the kernel is bound by HBM
      // bandwidth, and on the 70B-shaped batch a second resident wave per SIMD measured no
      // more bytes moved, only more partial slots and merge work.
      blocks = {cus * std::min(per_cu, kBlocksPerCU), cus * per_cu};
      cache[key] = blocks;
    }
  }
  // Tuning and test override: the total number of worker waves, at most what can be resident.
  if (const int w = tunable(kTuneDecodeWorkers); w >= kWaves)
    return std::min(w / kWaves, blocks.second) * kWaves;
  return blocks.first * kWaves;
}

DecodeWorkspace decode_workspace(int num_seqs, int num_kv_heads, int head_dim, int group, bool fp8,
                                 bool chunk_slots) {
  DecodeWorkspace ws{};
  ws.workers = decode_workers(head_dim, group, fp8);
  // With chunk slots the size covers the worker count of either pool type, so one query serves
  // both; without them it is exactly this launch's static layout.
  const int most =
      chunk_slots ? std::max(decode_workers(head_dim, group, !fp8), ws.workers) : ws.workers;
  if (ws.workers <= 0 || most <= 0 || num_seqs <= 0) {
    ws.workers = 0;
    return ws;
  }
  // Dynamic chunks need the per-sequence prefix in LDS: batches up to kMaxPrefixSeqs.
  const bool dyn = chunk_slots && num_seqs <= kMaxPrefixSeqs;
  ws.dyn_cap = dyn ? kDynSlotsPerWorker * ws.workers : 0;
  const int most_dyn = dyn ? kDynSlotsPerWorker * most : 0;
  const size_t units = (size_t)num_seqs * num_kv_heads;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  ws.counter_off = 0;
  ws.info_off = 256;
  ws.partials_off = ws.info_off + up(units * sizeof(int2));
  ws.bytes = ws.partials_off +
             ((size_t)most + most_dyn + units) * group * (2 + head_dim) * sizeof(float);
  return ws;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.num_workers < kWaves || p.num_workers % kWaves) return hipErrorInvalidConfiguration;
  if (p.dyn_cap > 0 && (p.num_seqs > kMaxPrefixSeqs || p.chunk_steps < 1 ||
                        p.static_frac_q10 < 512 || p.static_frac_q10 > 1024))
    return hipErrorInvalidConfiguration;
  const int G = p.num_q_heads / p.num_kv_heads;
  return dispatch(p.head_dim, G, hipErrorInvalidValue,
                  [&]<int D, int GG>() { return launch_dg<D, GG>(p, stream); });
}

}  // namespace pa
