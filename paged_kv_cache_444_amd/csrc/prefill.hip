// Chunked-prefill attention for gfx950 on matrix cores.
//
// What is computed: a chunk of q_len query tokens of a sequence attends causally to the
// sequence's whole paged context, including the chunk's own keys, which pa_reshape_and_cache has
// already written ("Serving engine internals" lesson, section on chunked prefill: long prompts are
// processed as fixed-size chunks batched with decode tokens).  The attention is the "Inference
// optimization" lesson's Build it, Step 2: max-subtracted softmax(q·kᵀ·scale)·v with the causal
// mask aligned to the end of the key range, so chunk row t (0-based) of a sequence of L cached
// tokens sees keys 0 .. L - q_len + t.  Prefill is compute-bound (same lesson, "Prefill vs
// decode"), so both contractions run on v_mfma_f32_16x16x32_bf16.
//
// Tiling.  A workgroup of four waves owns 64*RT query rows of one KV head, where a row is a
// (query token, head-in-group) pair: the G query heads that share a KV head share every K/V tile,
// so they are packed into the rows of one tile (row r = token r / G, head r % G).  Each wave owns
// RT tiles of 16 rows.  The keys are walked in tiles of 32 (two 16-token sub-blocks); each tile's
// K and V are copied into LDS in MFMA operand order (see the tile pipeline below) and every wave
// computes
//   Sᵀ[key][row] = K·Qᵀ      A = K from LDS (16 keys x 32 dims per instruction), B = Q rows kept
//                            in registers for the whole walk;
//   Oᵀ[dim][row] += Vᵀ·Pᵀ    A = V from LDS, B = the bf16 probabilities;
//   lsum[row]    += 1·Pᵀ     the running row sum, on the matrix cores as well.
// With the transposed product the score tile comes out of the matrix core exactly in the lane
// layout the second product needs as its B operand (lane l holds keys 8*(l/16) .. +7 of row l%16),
// so probabilities never leave registers.  The softmax is online per row in the log2 domain;
// masking is applied only on tiles that reach past the first token's diagonal, by selection
// (NaN-safe), and V rows of keys at or past L are zeroed in LDS so that 0 * NaN cannot enter the
// accumulator.

// Context split.  Long contexts are cut into `splits` key ranges (multiples of 32 keys) so the
// launch has enough workgroups; each range's (m, l, acc) per row goes to the workspace and
// prefill_merge combines them in split order.  With one split the output is written directly.

#include "pa_device.h"
#include "cascade.h"
#include "pa_internal.h"

#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kKeyTile = 32;
// log2-domain slack before the running max is raised: probabilities stay below 2^8.
constexpr float kRescaleSlack = 8.0f;

// 16-row MFMA tiles per wave: two, except for head_dim 256 whose accumulators need the room.
template <int D>
constexpr int kRowTiles = (D == 256) ? 1 : 2;

__device__ __forceinline__ f32x4_t mfma(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float xor32_f32(float x) { return __shfl_xor(x, 32, 64); }

// K/V tile pipeline.  kStages LDS stages each hold one 32-key tile in operand order: the K
// pieces [kt][ks] of the score product, then the V pieces [dt] of the second product, each 1 KB
// piece holding the 16-byte MFMA operand of lane l at 16*l, so every operand read is one linear
// ds_read_b128.  Wave 0 fetches the K pieces of product kt = 0, wave 1 those of kt = 1, waves 2
// and 3 half of the V pieces each, with D/32 direct global->LDS loads of 1 KB (lane l's 16 bytes
// land at 16*l); each lane's source address picks its own key's physical block.  Every wave
// issues the same number of loads per tile, so a vmcnt wait releases exactly one tile without
// touching registers.  Physical block ids come from an LDS copy of the table slice, so no other
// vector-memory load is in flight inside the walk.
//
// FP8 pools (E4M3 codes, one byte per element): an operand is 8 bytes, and the operands of lanes
// l and l+16 (l/16 even) are contiguous in the pool: the two 8-dim halves of one 32-byte K row
// of a slice, or the two 8-key halves of one 16-byte V row.  So one 16-byte direct load fetches
// a lane pair's operands, a wave's load covers two 512-byte pieces, and each wave issues half as
// many loads per tile.  In LDS pair q of a piece sits at 16*q (q = l%16 + 16*(l/32) for the
// reading lane l, which takes the half (l/16)%2); the reads are 8 bytes, widened to bf16 by
// v_cvt_scalef32_pk_bf16_fp8 (exact).
#ifndef PA_PREFILL_STAGES
#define PA_PREFILL_STAGES 3
#endif
// FP8 walks take their tiles in pairs: four stages, and the workgroup's barrier (with the loads
// it releases) comes once per two tiles, which measured 3 % faster for them and 1 % slower for
// bf16 walks; bf16 walks keep PA_PREFILL_STAGES stages and a barrier per tile.
template <bool Fp8>
constexpr bool kPairs = Fp8;
template <bool Fp8>
constexpr int kStages = kPairs<Fp8> ? 4 : PA_PREFILL_STAGES;
constexpr int kMaxTableLds = 2048;  // block ids of one workgroup's key range
constexpr unsigned kXcds = 8;       // accelerator dies (each with its own L2) of the GPU

// s_waitcnt with vmcnt(n) and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// One direct global->LDS load of 16 bytes per lane: lane l's bytes land at LDS byte address
// m0 + 16*l (m0 wave-uniform).  No immediate offset: on these loads it would move the LDS
// destination as well as the source.  Written as inline assembly so the compiler does not treat
// every later LDS access as dependent on it; the walk below waits for these loads explicitly.
__device__ __forceinline__ void lds_dma_16(const uint16_t* src, unsigned m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

// Where this wave's tile loads come from and go to; everything but `pool`, `pool8` and `sb` is
// wave-uniform.
struct TileSrc {
  const uint16_t* pool;    // K or V pool + KV head h + this lane's offset inside a piece
  const uint8_t* pool8;    // the same for FP8 pools (byte addressing)
  unsigned lds;            // LDS byte address of this wave's first piece in stage 0
  int sb;                  // sub-block (0: keys 0-15 of the tile, 1: keys 16-31) of this lane
  int piece_step;          // source elements between this wave's consecutive pieces
};

// Lane l of K piece (kt, ks): key kappa = 8*((l%16)/4) + l%4 + 4*kt of the tile, dims
// 32*ks + 8*(l/16) .. +7.  Lane l of V piece dt: dim 16*dt + l%16, keys 8*(l/16) .. +7.
template <int D, bool Fp8>
__device__ __forceinline__ TileSrc tile_src(const PrefillParams& p, int h, const void* lds0) {
  constexpr int KS = D / 32, DT = D / 16;
  const int lane = threadIdx.x & 63;
  const int r = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  TileSrc ts;
  int off, first_piece;
  if constexpr (Fp8) {
    // Fetching lane j: piece (j/32) of the load's two, lane pair q = j%32, whose first lane is
    // l = q%16 + 32*(q/16).
    const int q = lane & 31, half_piece = lane >> 5;
    const int l = (q & 15) + 32 * (q >> 4);
    if (r < 2) {  // K pieces (kt = r, ks = 2*load + half_piece): 16 bytes of key kappa's row
      const int key = 8 * ((l & 15) >> 2) + (l & 3) + 4 * r;
      ts.sb = key >> 4;
      off = half_piece * 512 + (key & 15) * 32 + 8 * (l >> 4);
      ts.piece_step = 1024;  // bytes between a wave's loads: two 32-dim slices
      first_piece = r * KS;
    } else {  // V pieces dt = (r-2)*DT/2 + 2*load + half_piece: the 16-byte row of dim 16dt + l%16
      ts.sb = l >> 5;
      off = ((r - 2) * (DT / 2) * 16 + half_piece * 16 + (l & 15)) * 16;
      ts.piece_step = 512;  // two pieces of 16 dims x 16 keys
      first_piece = 2 * KS + (r - 2) * (DT / 2);
    }
    ts.pool = nullptr;
    ts.pool8 = reinterpret_cast<const uint8_t*>((r < 2) ? p.kpool : p.vpool) +
               (size_t)h * p.block_size * D + off;
    const unsigned l0 = (unsigned)(uintptr_t)(const lds_u16*)lds0;
    ts.lds = __builtin_amdgcn_readfirstlane(l0 + (unsigned)first_piece * 512);
    return ts;
  }
  if (r < 2) {  // K of product kt = r; the pool sub-block layout is [D/32][16 keys][32 dims]
    const int key = 8 * ((lane & 15) >> 2) + (lane & 3) + 4 * r;
    ts.sb = key >> 4;
    off = (key & 15) * 32 + 8 * (lane >> 4);
    ts.piece_step = 512;
    first_piece = r * KS;
  } else {  // V pieces dt = (r-2)*DT/2 ..; the pool sub-block layout is [D dims][16 keys]
    const int g = lane >> 4;
    ts.sb = g >> 1;
    off = ((r - 2) * (DT / 2) * 16 + (lane & 15)) * 16 + 8 * (g & 1);
    ts.piece_step = 256;
    first_piece = 2 * KS + (r - 2) * (DT / 2);
  }
  ts.pool = ((r < 2) ? p.kpool : p.vpool) + (size_t)h * p.block_size * D + off;
  ts.pool8 = nullptr;
  const unsigned l0 = (unsigned)(uintptr_t)(const lds_u16*)lds0;
  ts.lds = __builtin_amdgcn_readfirstlane(l0 + (unsigned)first_piece * 1024);
  return ts;
}

// Issue this wave's loads of one tile into LDS stage `stage`.  `off` is the element offset in the
// pool of the 16-key sub-block this lane's key lies in (its block's start plus the sub-block's
// place in the block), from the workgroup's offset table.
template <int D, bool Fp8>
__device__ __forceinline__ void issue_tile(const TileSrc& ts, long long off, int stage) {
  constexpr int NP = Fp8 ? D / 64 : D / 32;  // loads per wave
  const unsigned m0 = ts.lds + (unsigned)stage * (4 * 16 * D * 2);
  if constexpr (Fp8) {
    const uint8_t* src = ts.pool8 + off;  // one byte per element
#pragma unroll
    for (int pc = 0; pc < NP; ++pc)
      lds_dma_16(reinterpret_cast<const uint16_t*>(src + pc * ts.piece_step), m0 + pc * 1024);
  } else {
    const uint16_t* src = ts.pool + off;
#pragma unroll
    for (int pc = 0; pc < NP; ++pc) lds_dma_16(src + pc * ts.piece_step, m0 + pc * 1024);
  }
}

// Eight E4M3 codes -> eight bf16 values, same order.
template <bool Hi>
__device__ __forceinline__ uint32_t fp8_pair_to_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, Hi));
}
__device__ __forceinline__ uint4 widen8(const uint2& w) {
  return make_uint4(fp8_pair_to_bf16<false>(w.x), fp8_pair_to_bf16<true>(w.x),
                    fp8_pair_to_bf16<false>(w.y), fp8_pair_to_bf16<true>(w.y));
}

// Prio: each wave takes a raised issue priority over its softmax and second products, and the
// normal one for the score products.  The two waves of a SIMD then settle into alternating
// phases, one wave's exponentials and probability products issuing ahead of the other wave's
// score products: about 6 % (bf16) and 7 % (FP8) off the chunk.  Off when another kernel shares
// the CUs, whose waves would wait behind the raised ones.
template <int D, int G, bool Fp8, bool Prio>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillParams p) {
  constexpr int RT = kRowTiles<D>;
  constexpr int KS = D / 32;       // k-steps of the score product
  constexpr int DT = D / 16;       // 16-dim tiles of the output
  constexpr int ROWS = kPWaves * 16 * RT;
  constexpr int TQ = ROWS / G;     // query tokens per workgroup
  constexpr int TILE_ELEMS = 4 * 16 * D;
  constexpr int kStages = pa::kStages<Fp8>;
  constexpr bool kPairs = pa::kPairs<Fp8>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kStages][TILE_ELEMS];
  // Pool element offset of every 16-key sub-block of this workgroup's key range, in key order.
  __shared__ long long off_lds[kMaxTableLds];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Workgroups are handed to the XCDs in turn (linear id n to XCD n % 8), and each XCD has its own
  // L2.  The query tiles of one (sequence, head, key range) read the same K/V tiles, so the
  // linear id is remapped to give every XCD a contiguous run of logical ids: one XCD then holds
  // all the query tiles of its (head, range) pairs and fetches their K/V from HBM once.
  int bx, by, bz;
  {
    const unsigned nx = gridDim.x, ny = gridDim.y;
    const unsigned n = nx * ny * gridDim.z;
    const unsigned lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const unsigned xcd = lin % kXcds, per = n / kXcds, extra = n % kXcds;
    const unsigned logical = xcd * per + min(xcd, extra) + lin / kXcds;
    bx = logical % nx;
    by = (logical / nx) % ny;
    bz = logical / (nx * ny);
  }
  const int s = bz;
  const int h = by / p.splits;
  const int split = by % p.splits;
  const int qs = p.query_start_loc[s];
  const int q_len = p.query_start_loc[s + 1] - qs;
  const int q0 = bx * TQ;
  if (q_len <= 0 || q0 >= q_len) return;  // block-uniform
  // With from_first_row the table row and length are those of the first query row, clamped into
  // the table (whose rows are then the total_q query rows) so a malformed query_start_loc cannot
  // leave it.
  const int trow = p.from_first_row ? min(max(qs, 0), p.total_q - 1) : s;
  const int L = min(max(p.seq_lens[trow], 0), p.max_seq_len);
  // Non-causal rows see every key: ctx = L makes each row's last visible key L - 1.
  const int ctx = p.noncausal ? L : max(L - q_len, 0);
  const int tq = min(TQ, q_len - q0);
  const int kv_end = min(L, ctx + q0 + tq);
  const int kb = split * p.split_keys;
  const int ke = min(kv_end, kb + p.split_keys);
  const int Hq = p.num_q_heads;
  const float c = p.scale_log2;

  // Rows of this lane: column n = lane % 16 of each of the wave's row tiles.
  int row_tok[RT], row_lim[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = wave * 16 * RT + 16 * rt + (lane & 15);
    row_tok[rt] = q0 + r / G;
    // Rows past the chunk, or past the query array if query_start_loc is malformed, are skipped.
    row_ok[rt] = (r / G) < tq && qs + row_tok[rt] < p.total_q && qs >= 0;
    row_lim[rt] = min(ctx + row_tok[rt], L - 1);  // last visible key
  }

  // Q operand: rows as B, 32 dims per k-step, lane holds dims 8*(lane/16) .. +7.  The softmax
  // scale times log2(e) is applied here, once (fp32 product rounded to bf16, nearest even), so
  // the score product yields log2-domain scores y = q·k·scale·log2(e) directly.
  uint4 qb[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = wave * 16 * RT + 16 * rt + (lane & 15);
    // Rows past the chunk read its last row (always inside the query array) and are zeroed.
    const int tok = min(min(qs + q0 + r / G, qs + q_len - 1), p.total_q - 1);
    const size_t qrow = (size_t)max(tok, 0) * Hq + (size_t)h * G + r % G;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = *(const uint4*)(p.query + qrow * D + 32 * ks + 8 * (lane >> 4));
      const uint4 sv = make_uint4(pack_bf16x2(bf16_lo(v.x) * c, bf16_hi(v.x) * c),
                                  pack_bf16x2(bf16_lo(v.y) * c, bf16_hi(v.y) * c),
                                  pack_bf16x2(bf16_lo(v.z) * c, bf16_hi(v.z) * c),
                                  pack_bf16x2(bf16_lo(v.w) * c, bf16_hi(v.w) * c));
      qb[rt][ks] = row_ok[rt] ? sv : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // Online-softmax state per row (the same in the four lanes sharing a row), in the log2
  // domain: M is the running maximum of the row's scores y (-inf before its first key), and
  // cz = -M (0 while M is -inf) is the initial accumulator of every score product, so the
  // products yield z = y - M and the probabilities are exp2(z) with no further vector work.
  // thr bounds z: -inf until M is set, then the slack; a z above it raises M (and rescales).
  // The running sum of the row's probabilities is accumulated on the matrix cores as one more
  // product, an all-ones A operand times the bf16 probabilities, so every element of lsum[rt]
  // holds the sum of the row the lane's column belongs to (the same rounded probabilities that
  // weight V).
  f32x4_t acc[DT][RT], lsum[RT], cz[RT];
  float M[RT], thr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    M[rt] = kNegInf;
    thr[rt] = kNegInf;
    cz[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lsum[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int* bt = p.block_tables + (size_t)trow * p.max_blocks_per_seq;
  const int t_first = kb / kKeyTile;
  const int t_end = (ke + kKeyTile - 1) / kKeyTile;  // empty range: t_end <= t_first
  // Keys above this need a per-row mask (non-causal: only keys at or past L, in the last tile).
  const int diag = p.noncausal ? L - 1 : ctx + q0;
  // Offset table of this workgroup's keys [32*t_first, 32*t_end): for 16-key sub-block j (keys
  // 32*t_first + 16j ..), its physical block (clamped into the pool) times the block's size plus
  // the sub-block's place in the block.  Sub-blocks at or past L point at block 0, always inside
  // the pool: their V rows are zeroed before use and their scores are masked.
  const int bs = p.block_size;
  {
    const int shift = (bs == 32) ? 5 : 4;
    const long long block_stride = (long long)p.num_kv_heads * bs * D;
    const int nsb = (t_first < t_end) ? min(2 * (t_end - t_first), kMaxTableLds) : 0;
    constexpr int kPer = kMaxTableLds / kPThreads;
    int v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + kPThreads * k;
      const int key = (2 * t_first + i) * 16;
      v[k] = (i < nsb && key < L) ? bt[key >> shift] : 0;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + kPThreads * k;
      const int key = (2 * t_first + i) * 16;
      const int id = min(max(v[k], 0), (int)(p.num_blocks - 1));
      off_lds[i] = (i < nsb) ? (long long)id * block_stride + (long long)(key & (bs - 1)) * D : 0;
    }
  }
  // Every ordinary vector-memory load (query rows, table slice) is complete before the walk, so
  // the only loads in flight inside it are the tile loads counted by wait_vmcnt.
  wait_vmcnt<0>();
  __syncthreads();
  if (t_first < t_end) {
    constexpr int NP = Fp8 ? D / 64 : D / 32;  // tile loads per wave
    const TileSrc ts = tile_src<D, Fp8>(p, h, &lds[0][0]);
    // The all-ones A operand of the row-sum product.  Passed through an empty asm statement it is
    // opaque to the compiler, which then keeps it in four registers instead of rebuilding it in
    // every tile.
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    constexpr uint32_t kOnes = 0x3F803F80u;  // two bf16 1.0
    u32x4_t ones_v = {kOnes, kOnes, kOnes, kOnes};
    asm volatile("" : "+v"(ones_v));
    const uint4 ones = __builtin_bit_cast(uint4, ones_v);
    // This lane's sub-block offset for tile t (clamped to the range's last tile).
    auto tile_off = [&](int t) __attribute__((always_inline)) {
      return off_lds[min(2 * (min(t, t_end - 1) - t_first) + ts.sb, kMaxTableLds - 1)];
    };
    constexpr int kAhead = kPairs ? 2 : kStages - 1;  // tiles loaded before the walk
#pragma unroll
    for (int k = 0; k < kAhead; ++k) issue_tile<D, Fp8>(ts, tile_off(t_first + k), k);
    // One key tile.  kMasked: the tile reaches past the first row's diagonal and the causal mask
    // is applied per score; those tiles are the last ones of the walk, so the two variants run
    // as two loops and the other tiles carry no per-score selects.
    // cur is tile t's stage, (t - t_first) % kStages, kept as a rotating counter.
    int cur = 0;
    auto walk_tile = [&](int t, auto masked_c) __attribute__((always_inline)) {
      constexpr bool kMasked = decltype(masked_c)::value;
      if constexpr (kPairs) {
        if (((t - t_first) & 1) == 0) {  // block-uniform: the first tile of a pair
          const long long off2 = tile_off(t + 2), off3 = tile_off(t + 3);
          wait_vmcnt<0>();   // this wave's parts of tiles t and t+1 have landed
          __syncthreads();   // all parts landed; every wave is done with tiles t-2 and t-1
          issue_tile<D, Fp8>(ts, off2, (cur + 2) & 3);
          issue_tile<D, Fp8>(ts, off3, (cur + 3) & 3);
        }
      } else {
        const int prev = (cur == 0) ? kStages - 1 : cur - 1;  // tile t-1's stage, free below
        const long long next_off = tile_off(t + kStages - 1);  // read while the barrier waits
        wait_vmcnt<NP * (kStages - 2)>();  // this wave's part of tile t has landed
        __syncthreads();                   // all parts landed; every wave is done with tile t-1
        issue_tile<D, Fp8>(ts, next_off, prev);
      }
      if (t * kKeyTile + kKeyTile > L) {  // block-uniform: zero V rows of keys at or past L
        if constexpr (Fp8) {
          uint8_t* vz = reinterpret_cast<uint8_t*>(&lds[cur][0]) + 32 * D;
          for (int i = threadIdx.x; i < 32 * D; i += kPThreads) {
            // byte i of piece i / 512: pair (i % 512) / 16, half (i / 8) % 2, code i % 8, which
            // is key 16 * ((i / 256) % 2) + i % 16 of the tile
            const int key = t * kKeyTile + 16 * ((i >> 8) & 1) + (i & 15);
            if (key >= L) vz[i] = 0;  // code 0 is +0
          }
        } else {
          uint16_t* vz = &lds[cur][2 * 16 * D];
          for (int i = threadIdx.x; i < 2 * 16 * D; i += kPThreads) {
            // piece i / 512, lane (i % 512) / 8 holding keys 8 * (lane / 16) .., element i % 8
            const int key = t * kKeyTile + 8 * ((i >> 7) & 3) + (i & 7);
            if (key >= L) vz[i] = 0;
          }
        }
        __syncthreads();
      }
      const uint16_t* kl = lds[cur];
      const uint16_t* vl = lds[cur] + 2 * 16 * D;
      const uint8_t* kl8 = reinterpret_cast<const uint8_t*>(lds[cur]);
      const uint8_t* vl8 = kl8 + 32 * D;
      // FP8: this lane's operand in a 512-byte piece: pair q, half (lane/16)%2.
      const int op8 = 16 * ((lane & 15) + 16 * (lane >> 5)) + 8 * ((lane >> 4) & 1);

      // K fragments, the A operands of the score product, shared by the row tiles.  Row m of
      // product kt is key 8*(m/4) + m%4 + 4*kt of the tile, so lane l gets keys
      // 8*(l/16) + 4*kt + i: eight consecutive keys of one sub-block, the B operand layout the
      // second product needs.
      uint4 kf[2][KS];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kf[kt][ks] = Fp8 ? widen8(*(const uint2*)(kl8 + (kt * KS + ks) * 512 + op8))
                           : *(const uint4*)(kl + ((kt * KS + ks) * 64 + lane) * 8);
      // V fragments, the A operands of the second product: dim 16dt + lane%16, keys 8g .. 8g+7
      // (g = lane/16).
      auto v_frag = [&](int dt) __attribute__((always_inline)) {
        if constexpr (Fp8) return widen8(*(const uint2*)(vl8 + dt * 512 + op8));
        else return *(const uint4*)(vl + (dt * 64 + lane) * 8);
      };
      auto scores = [&](int rt, f32x4_t (&sc)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          sc[kt] = cz[rt];  // z = y - M
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) sc[kt] = mfma(kf[kt][ks], qb[rt][ks], sc[kt]);
        }
      };
      // Online softmax of row tile rt, then its second product with the V fragments vf.
      auto softmax_pv = [&](int rt, const f32x4_t (&sc)[2], auto&& vf)
                            __attribute__((always_inline)) {
        float x[8];  // z = y - M; -inf where masked
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = sc[kt][i];
            if constexpr (kMasked) {
              const int key = t * kKeyTile + 8 * (lane >> 4) + 4 * kt + i;
              v = (key <= row_lim[rt]) ? v : kNegInf;
            }
            x[4 * kt + i] = v;
          }
        // The running max is raised (and acc rescaled) only when a score exceeds it by the
        // slack, so probabilities stay below 2^slack and the accumulators are rarely touched.
        bool raise = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) raise |= x[i] > thr[rt];
        // The bf16 walk keeps the rare branch out of line (its common path then has no taken
        // branch: 0.4 % faster); the FP8 walk measured slower that way.
        const bool any_raise = __ballot(raise) != 0;
        if (Fp8 ? any_raise : __builtin_expect(any_raise, 0)) {
          float mx = x[0];
#pragma unroll
          for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
          mx = fmaxf(mx, xor16_f32(mx));
          mx = fmaxf(mx, xor32_f32(mx));
          const float cz0 = cz[rt][0];
          const float mn = fmaxf(M[rt], mx - cz0);  // the row's new maximum of y
          if (mn != kNegInf && mn != M[rt]) {
            const float alpha = fast_exp2(M[rt] - mn);  // 0 when the old max is -inf
            lsum[rt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt][rt] *= alpha;
            M[rt] = mn;
            thr[rt] = kRescaleSlack;
            // this tile's scores were taken against the old maximum: move them to the new one
            const float shift = cz0 + mn;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] -= shift;
            cz[rt] = f32x4_t{-mn, -mn, -mn, -mn};
          }
        }
        float pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = fast_exp2(x[i]);
        // B operand of the second product: item j is key 8*(lane/16) + j of the tile (the V
        // fragments use the same order).
        const uint4 pb = make_uint4(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                    pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7]));
        lsum[rt] = mfma(ones, pb, lsum[rt]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt][rt] = mfma(vf(dt), pb, acc[dt][rt]);
      };
      if constexpr (RT == 2) {
        // Row tile 1's scores are issued before row tile 0's softmax and row tile 0's second
        // product before row tile 1's softmax, so the matrix cores run while the vector ALUs do.
        uint4 vf[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vf[dt] = v_frag(dt);
        auto vreg = [&](int dt) __attribute__((always_inline)) { return vf[dt]; };
        f32x4_t s0[2], s1[2];
        // bf16 drops the raised priority only for the score products (it stays up over the next
        // tile's barrier and fragment reads); FP8 drops it as soon as the second products are
        // issued (kept up until the scores, FP8 measured 8 % slower; bf16 1.6 % faster).
        if constexpr (Prio && !Fp8) __builtin_amdgcn_s_setprio(0);
        scores(0, s0);
        scores(1, s1);
        if constexpr (Prio) __builtin_amdgcn_s_setprio(1);
        softmax_pv(0, s0, vreg);
        softmax_pv(1, s1, vreg);
        if constexpr (Prio && Fp8) __builtin_amdgcn_s_setprio(0);
      } else {
        f32x4_t s0[2];
        scores(0, s0);
        if constexpr (Prio) __builtin_amdgcn_s_setprio(1);
        softmax_pv(0, s0, v_frag);
        if constexpr (Prio) __builtin_amdgcn_s_setprio(0);
      }
      cur = (cur == kStages - 1) ? 0 : cur + 1;
    };
    // Tile t needs the mask iff 32t + 31 > diag.
    const int t_mask = min(max((diag + 1) / kKeyTile, t_first), t_end);
    int t = t_first;
    for (; t < t_mask; ++t) walk_tile(t, std::false_type{});
    for (; t < t_end; ++t) walk_tile(t, std::true_type{});
    wait_vmcnt<0>();  // no tile load may still be writing LDS when the workgroup ends
    if constexpr (Prio) __builtin_amdgcn_s_setprio(0);
  }

  // Finish: normalise or hand the split's state over.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lt = lsum[rt][0];
    if (!row_ok[rt]) continue;
    const int r = wave * 16 * RT + 16 * rt + (lane & 15);
    const size_t orow = (size_t)(qs + row_tok[rt]) * Hq + (size_t)h * G + r % G;
    if (p.splits == 1 && !p.defer_merge) {
      const float inv = lt > 0.f ? p.v_scale / lt : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t a = acc[dt][rt];
        const uint2 o = make_uint2(pack_bf16x2(a[0] * inv, a[1] * inv),
                                   pack_bf16x2(a[2] * inv, a[3] * inv));
        *(uint2*)(p.out + orow * D + 16 * dt + 4 * (lane >> 4)) = o;
      }
    } else {
      const size_t u = orow * p.ws_splits + split;
      if (lane < 16) {
        p.ws_ml[2 * u] = M[rt];  // log2 domain; -inf for an empty or fully masked range
        p.ws_ml[2 * u + 1] = lt;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *(f32x4_t*)(p.ws_acc + u * D + 16 * dt + 4 * (lane >> 4)) = acc[dt][rt] * p.v_scale;
    }
  }
}

// Combine the context splits of every (query row, head) in split order.  A thread owns four
// head-dim values of one (row, head); the split maxima are loaded first, then the sums.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams p) {
  constexpr int TPH = D / 4;  // threads per (row, head)
  const size_t unit = (size_t)blockIdx.x * (256 / TPH) + threadIdx.x / TPH;  // row * Hq + head
  if (unit >= (size_t)p.total_q * p.num_q_heads) return;
  const int d = 4 * (threadIdx.x % TPH);
  const size_t u0 = unit * p.ws_splits;
  // One pass with an online rescale, four splits' (m, l, acc) loads issued together per round
  // (indices clamped to the last split), so a row with at most four splits costs one round trip
  // where a pass for the maximum and then one for the sums cost two.  An empty range (m = -inf)
  // adds nothing.
  constexpr int kRound = 4;
  float M = kNegInf, lt = 0.f;
  f32x4_t a = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < p.ws_splits; j0 += kRound) {
    float mv[kRound], lv[kRound];
    f32x4_t av[kRound];
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const size_t u = u0 + min(j0 + r, p.ws_splits - 1);
      mv[r] = p.ws_ml[2 * u];
      lv[r] = p.ws_ml[2 * u + 1];
      av[r] = *(const f32x4_t*)(p.ws_acc + u * D + d);
    }
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      if (j0 + r >= p.ws_splits || mv[r] == kNegInf) continue;
      const float mn = fmaxf(M, mv[r]);
      const float c_old = fast_exp2(M - mn);  // 0 while M is -inf
      const float c_new = fast_exp2(mv[r] - mn);
      lt = lt * c_old + lv[r] * c_new;
      a = a * c_old + av[r] * c_new;
      M = mn;
    }
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  *(uint2*)(p.out + unit * D + d) =
      make_uint2(pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv));
}

template <int D>
hipError_t merge_d(const PrefillParams& p, hipStream_t stream) {
  TraceScope t("prefill_merge", stream);
  constexpr int UPB = 256 / (D / 4);  // (row, head) units per block
  const size_t units = (size_t)p.total_q * p.num_q_heads;
  const dim3 grid((unsigned)((units + UPB - 1) / UPB));
  hipLaunchKernelGGL((prefill_merge_kernel<D>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_dg(const PrefillParams& p, hipStream_t stream) {
  constexpr int TQ = kPWaves * 16 * kRowTiles<D> / G;
  {
    TraceScope t("prefill_chunk", stream);
    const dim3 grid((p.max_q_len + TQ - 1) / TQ, p.num_kv_heads * p.splits, p.num_seqs);
    if (p.kv_fp8 && !p.concurrent)
      hipLaunchKernelGGL((prefill_kernel<D, G, true, true>), grid, dim3(kPThreads), 0, stream, p);
    else if (p.kv_fp8)
      hipLaunchKernelGGL((prefill_kernel<D, G, true, false>), grid, dim3(kPThreads), 0, stream, p);
    else if (!p.concurrent)
      hipLaunchKernelGGL((prefill_kernel<D, G, false, true>), grid, dim3(kPThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((prefill_kernel<D, G, false, false>), grid, dim3(kPThreads), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1 || p.defer_merge) return e;
  return merge_d<D>(p, stream);
}

template <int D>
hipError_t launch_d(const PrefillParams& p, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_dg<D, 1>(p, stream);
    case 2: return launch_dg<D, 2>(p, stream);
    case 4: return launch_dg<D, 4>(p, stream);
    case 8: if constexpr (D <= 128) return launch_dg<D, 8>(p, stream); break;
    case 16: if constexpr (D <= 64) return launch_dg<D, 16>(p, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return cus > 0 ? cus : 256;
}

template <int D>
const void* kernel_of(int G) {
  switch (G) {
    case 1: return reinterpret_cast<const void*>(&prefill_kernel<D, 1, false, true>);
    case 2: return reinterpret_cast<const void*>(&prefill_kernel<D, 2, false, true>);
    case 4: return reinterpret_cast<const void*>(&prefill_kernel<D, 4, false, true>);
    case 8:
      if constexpr (D <= 128)
        return reinterpret_cast<const void*>(&prefill_kernel<D, 8, false, true>);
      break;
    case 16:
      if constexpr (D <= 64)
        return reinterpret_cast<const void*>(&prefill_kernel<D, 16, false, true>);
      break;
    default: break;
  }
  return nullptr;
}

// Workgroups of the (head_dim, group) variant resident on one CU at once (at least 1).
int resident_per_cu(int head_dim, int group) {
  static std::mutex mu;
  static std::map<std::pair<int, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_pair(dev, head_dim * 64 + group);
  if (auto it = cache.find(key); it != cache.end()) return it->second;
  const void* fn = head_dim == 64    ? kernel_of<64>(group)
                   : head_dim == 128 ? kernel_of<128>(group)
                   : head_dim == 256 ? kernel_of<256>(group)
                                     : nullptr;
  int n = 0;
  if (!fn || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kPThreads, 0) != hipSuccess)
    n = 1;
  n = std::max(n, 1);
  cache[key] = n;
  return n;
}

}  // namespace

namespace {

PrefillSplit split_for(int num_seqs, int max_q_len, int num_kv_heads, int group, int head_dim,
                       int max_seq_len, bool one_per_cu) {
  PrefillSplit r{1, std::max(max_seq_len, 1)};
  if (num_seqs <= 0 || max_q_len <= 0 || max_seq_len <= 0) return r;
  // One range's table slice must fit the LDS copy (kMaxTableLds entries of 16-token blocks).
  const int max_keys = (kMaxTableLds - 2) * 16 / kKeyTile * kKeyTile;
  const long long need = (max_seq_len + max_keys - 1) / max_keys;
  const int rows = kPWaves * 16 * (head_dim == 256 ? 1 : 2);
  const int tq = rows / group;
  const long long base = (long long)((max_q_len + tq - 1) / tq) * num_kv_heads * num_seqs;
  // Enough workgroups for one round of every CU's resident slots (more rounds only add merge
  // work), each range at least 256 keys, at most 16 ranges.
  // one_per_cu: a bandwidth-bound chunk (few query rows over a long context) gains nothing from a
  // second resident round, and every extra range adds merge traffic.
  const long long slots = (long long)(one_per_cu ? 1 : resident_per_cu(head_dim, group)) * cu_count();
  long long want = (slots + base - 1) / base;
  if (const int forced = tunable(kTunePrefillSplits); forced > 0) want = forced;
  want = std::min<long long>(std::max<long long>(want, 1), 16);
  want = std::min<long long>(want, std::max(1, max_seq_len / 256));
  want = std::max(want, need);
  if (want <= 1) return r;
  int keys = (int)((max_seq_len + want - 1) / want);
  keys = (keys + kKeyTile - 1) / kKeyTile * kKeyTile;
  r.split_keys = keys;
  r.splits = (max_seq_len + keys - 1) / keys;
  return r;
}

}  // namespace

PrefillSplit prefill_split(int num_seqs, int max_q_len, int num_kv_heads, int group, int head_dim,
                           int max_seq_len) {
  return split_for(num_seqs, max_q_len, num_kv_heads, group, head_dim, max_seq_len, false);
}

PrefillSplit prompt_split(int num_groups, int max_group_size, int num_kv_heads, int group,
                          int head_dim, int prefix_len) {
  return split_for(num_groups, max_group_size, num_kv_heads, group, head_dim, prefix_len, true);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.splits < 1 || (p.splits > 1 && p.split_keys % kKeyTile) || p.ws_splits < p.splits)
    return hipErrorInvalidValue;
  const int G = p.num_q_heads / p.num_kv_heads;
  switch (p.head_dim) {
    case 64: return launch_d<64>(p, G, stream);
    case 128: return launch_d<128>(p, G, stream);
    case 256: return launch_d<256>(p, G, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_merge(const PrefillParams& p, hipStream_t stream) {
  if (p.ws_splits < 1) return hipErrorInvalidValue;
  switch (p.head_dim) {
    case 64: return merge_d<64>(p, stream);
    case 128: return merge_d<128>(p, stream);
    case 256: return merge_d<256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
