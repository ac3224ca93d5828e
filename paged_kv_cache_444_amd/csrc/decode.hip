// Split-K paged decode attention for gfx950.
//
// One query token per sequence attends to the sequence's whole paged context ("Inference
// optimization" lesson, Step 2 with one query row; decode re-reads the KV cache every step, which
// makes it a bandwidth-bound matrix-vector product — same lesson, "Prefill vs decode", and the
// vLLM-on-H100 article, "Decode is a memory problem").  No matrix cores: the contraction per KV
// head is an [G x D] by [D x 16] product per 16-token step, far below the MFMA ridge.
//
// Work unit: (sequence s, KV head h, partition p of `part` tokens).  A 256-thread workgroup (four
// waves) owns one unit; the waves take the unit's 16-token steps round-robin.  Per step a wave
// loads the step's K tile (16 tokens x D) and V tile (D x 16 tokens) with 16-byte loads, each
// instruction covering 1 KiB of contiguous pool memory, and
//   K side: lane l holds token l/4 and head-dim chunk l%4 of every 32-wide slice, so the G scores
//           of a token are finished with two quad DPP adds;
//   softmax: online (running max and sum) per octet of tokens — tokens 0..7 live in lanes 0..31,
//           8..15 in lanes 32..63 — in the log2 domain;
//   V side: lane l holds head-dim rows l%32 (+32k) for the 8 tokens of octet l/32, so P·V is
//           v_dot2 over token pairs with the probabilities read back from LDS as bf16 pairs.
// Each (wave, octet) keeps its own (m, l, acc) state; the eight states of a workgroup are merged
// through LDS at the end.  A sequence that fits in one partition is written straight to the
// output; otherwise the unit's state goes to the workspace and decode_merge combines partitions.

#include "pa_device.h"
#include "pa_internal.h"

#include <cstdlib>

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void decode_partition_kernel(DecodeParams p) {
  constexpr int R = D / kSlice;  // 16-byte K loads per lane per step, and V loads
  const int part_idx = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);

  const int L = min(max(p.seq_lens[s], 0), p.len_cap);
  const int tok0 = part_idx * p.part_tokens;
  const int Hq = p.num_q_heads;
  if (tok0 >= L) {
    if (part_idx == 0) {  // empty sequence: zero output
      for (int i = threadIdx.x; i < G * D; i += kThreads)
        p.out[((size_t)s * Hq + h * G) * D + i] = 0;
    }
    return;
  }
  const int tok1 = min(L, tok0 + p.part_tokens);
  const int nsteps = (tok1 - tok0 + kSub - 1) / kSub;
  const int n_parts = (L + p.part_tokens - 1) / p.part_tokens;
  const int bs = p.block_size;

  __shared__ uint16_t p_lds[kWaves][2][G][8];
  __shared__ float st_m[kWaves][2][G];
  __shared__ float st_l[kWaves][2][G];
  __shared__ float st_acc[kWaves][2][G][D];

  // K-side and V-side lane roles.
  const int kt = lane >> 2;   // token within the step
  const int kj = lane & 3;    // 8-wide chunk within each 32-wide slice
  const int vd = lane & 31;   // head-dim row (plus 32*k)
  const int vo = lane >> 5;   // token octet

  // Query of the G heads sharing KV head h, restricted to this lane's head-dim chunks.
  uint4 q[G][R];
  {
    const uint16_t* qb = p.query + ((size_t)s * Hq + (size_t)h * G) * D + 8 * kj;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int r = 0; r < R; ++r) q[g][r] = *(const uint4*)(qb + g * D + r * kSlice);
  }

  // Physical ids of the unit's blocks, one per lane (a partition spans at most 64 blocks).
  const int first_blk = tok0 / bs;
  const int nblk = (tok1 - 1) / bs - first_blk + 1;
  const int* bt = p.block_tables + (size_t)s * p.max_blocks_per_seq + first_blk;
  const int blk_id = lane < nblk ? bt[lane] : 0;

  const size_t tile = (size_t)bs * D;                   // elements per (block, head)
  const size_t block_elems = (size_t)p.num_kv_heads * tile;
  const size_t head_off = (size_t)h * tile;

  float m[G], l[G], acc[G][R];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[g][r] = 0.f;
  }

  for (int i = wave; i < nsteps; i += kWaves) {
    const int t0 = tok0 + i * kSub;
    const int id = __builtin_amdgcn_readlane(blk_id, t0 / bs - first_blk);
    const size_t off = (size_t)id * block_elems + head_off + (size_t)((t0 % bs) / kSub) * kSub * D;
    const uint16_t* kp = p.kpool + off;
    const uint16_t* vp = p.vpool + off;
    uint4 kr[R], vr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) kr[r] = *(const uint4*)(kp + r * (kSub * kSlice) + 8 * lane);
#pragma unroll
    for (int k = 0; k < R; ++k) vr[k] = *(const uint4*)(vp + (vd + 32 * k) * kSub + 8 * vo);

    // Scores of token kt for the G heads.
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) a = dot8(q[g][r], kr[r], a);
      a += dpp_f32<kDppQuadXor1>(a);
      a += dpp_f32<kDppQuadXor2>(a);
      sc[g] = a;
    }
    const int nvalid = tok1 - t0;  // tokens of this step inside the unit (>= 1)
    const bool tail = nvalid < kSub;
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = (kt < nvalid) ? sc[g] * p.scale_log2 : kNegInf;

    // Online softmax per octet.
    float alpha[G], pr[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x = sc[g];
      x = fmaxf(x, dpp_f32<kDppRowRor4>(x));
      x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
      x = fmaxf(x, xor16_f32(x));
      const float mn = fmaxf(m[g], x);
      const float ms = (mn == kNegInf) ? 0.f : mn;
      alpha[g] = fast_exp2(m[g] - ms);
      pr[g] = fast_exp2(sc[g] - ms);
      m[g] = mn;
      l[g] = l[g] * alpha[g] + pr[g];
    }
    if (kj == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) p_lds[wave][kt >> 3][g][kt & 7] = to_bf16(pr[g]);
    }
    wave_lds_sync();

    if (tail) {  // zero V of tokens past the end: 0 * NaN must not reach the accumulators
#pragma unroll
      for (int k = 0; k < R; ++k) {
        uint32_t w[4] = {vr[k].x, vr[k].y, vr[k].z, vr[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int u = 8 * vo + 2 * e;
          if (u >= nvalid) w[e] = 0u;
          else if (u + 1 >= nvalid) w[e] &= 0xFFFFu;
        }
        vr[k] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 pp = *(const uint4*)&p_lds[wave][vo][g][0];
#pragma unroll
      for (int k = 0; k < R; ++k) acc[g][k] = dot8(pp, vr[k], acc[g][k] * alpha[g]);
    }
    wave_lds_sync();
  }

  // Sum l over the quads of each octet (every lane of a quad holds the same partial).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = l[g];
    x += dpp_f32<kDppRowRor4>(x);
    x += dpp_f32<kDppRowRor8>(x);
    x += xor16_f32(x);
    l[g] = x;
  }
  if (vd == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      st_m[wave][vo][g] = m[g];
      st_l[wave][vo][g] = l[g];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int k = 0; k < R; ++k) st_acc[wave][vo][g][vd + 32 * k] = acc[g][k];
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int o = 0; o < 2; ++o) M = fmaxf(M, st_m[w][o][g]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float Lt = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const float c = fast_exp2(st_m[w][o][g] - Ms);
        Lt += st_l[w][o][g] * c;
        A += st_acc[w][o][g][d] * c;
      }
    const size_t row = (size_t)s * Hq + (size_t)h * G + g;
    if (n_parts == 1) {
      p.out[row * D + d] = to_bf16(Lt > 0.f ? A / Lt : 0.f);
    } else {
      const size_t u = row * p.max_parts + part_idx;
      p.ws_acc[u * D + d] = A;
      if (d == 0) {
        p.ws_ml[2 * u] = M;
        p.ws_ml[2 * u + 1] = Lt;
      }
    }
  }
}

// Combine the partitions of each (sequence, query head): rescale every partition's partial sums
// to the common maximum and divide once.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
  constexpr int HPB = 256 / D;  // heads per block
  const int s = blockIdx.x;
  const int hq = blockIdx.y * HPB + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (hq >= p.num_q_heads) return;
  const int L = min(max(p.seq_lens[s], 0), p.len_cap);
  const int n_parts = (L + p.part_tokens - 1) / p.part_tokens;
  if (n_parts <= 1) return;  // written directly by the partition kernel
  const size_t row = (size_t)s * p.num_q_heads + hq;
  const float* ml = p.ws_ml + 2 * row * p.max_parts;
  const float* acc = p.ws_acc + row * p.max_parts * D + d;
  float M = kNegInf;
  for (int j = 0; j < n_parts; ++j) M = fmaxf(M, ml[2 * j]);
  float Lt = 0.f, A = 0.f;
  for (int j = 0; j < n_parts; ++j) {
    const float c = fast_exp2(ml[2 * j] - M);
    Lt += ml[2 * j + 1] * c;
    A += acc[(size_t)j * D] * c;
  }
  p.out[row * D + d] = to_bf16(A / Lt);
}

template <int D, int G>
hipError_t launch_dg(const DecodeParams& p, hipStream_t stream) {
  {
    TraceScope t("decode_partition", stream);
    dim3 grid(p.max_parts, p.num_kv_heads, p.num_seqs);
    hipLaunchKernelGGL((decode_partition_kernel<D, G>), grid, dim3(kThreads), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_parts <= 1) return e;
  {
    TraceScope t("decode_merge", stream);
    constexpr int HPB = 256 / D;
    dim3 grid(p.num_seqs, (p.num_q_heads + HPB - 1) / HPB);
    hipLaunchKernelGGL((decode_merge_kernel<D>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, int G, hipStream_t stream) {
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

}  // namespace

int decode_partition_tokens() {
  static const int part = [] {
    int v = 512;
    if (const char* e = std::getenv("PA_DECODE_PART")) {
      const int x = std::atoi(e);
      if (x >= 64 && x <= 1024 && x % 32 == 0) v = x;
    }
    return v;
  }();
  return part;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const int G = p.num_q_heads / p.num_kv_heads;
  switch (p.head_dim) {
    case 64: return launch_d<64>(p, G, stream);
    case 128: return launch_d<128>(p, G, stream);
    case 256: return launch_d<256>(p, G, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
