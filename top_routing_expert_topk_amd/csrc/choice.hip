// Expert Choice routing: each expert takes a fixed number of tokens (page
// "MoE混合专家模型路由机制原理与稀疏激活实现", section "Expert Choice路由策略与容量因子调优":
// the direction of selection is reversed, every expert processes the same
// number of tokens, capacity = tokens / E * factor, and tokens no expert
// takes keep only the residual).
//
// Scores: p[t,e] = softmax over experts of token t's router logits (the gate
// equation of the same page without its top-k mask). Expert e takes the
// min(C, T) tokens of largest p[t,e], ties to the lower token index, lists
// them in ascending token order as rows [e*C, (e+1)*C) of the permutation,
// and gates each chosen pair with p[t,e]. The outputs have the shapes the
// grouped FFN and the combine already take: offsets / sorted_token for the
// FFN, and per token E slots (dest_row [T][E], -1 where not chosen; gate
// [T][E]) for the combine, which sums them in ascending expert order.
//
// Kernels:
//   ec_scores  one wave per token: softmax of its E logits (max, then a
//              fixed-order sum), written transposed through LDS as scores
//              [E][T] so each expert's column is contiguous; also clears the
//              token's dest_row / gate slots
//   ec_select  one block per expert: the column staged in LDS, radix select
//              of the C-th largest score (four 8-bit digit passes, histograms
//              in LDS), then one ordered block scan over per-thread token
//              segments that keeps every score above it and the lowest-index
//              ties at it, writing rows in token order
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kEcTokens = 16;  // tokens per ec_scores block (4 waves x 4)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(256) void ec_scores(const float* __restrict__ logits, int T, int E,
                                                 float* __restrict__ scores,
                                                 int32_t* __restrict__ dest,
                                                 float* __restrict__ gate) {
  __shared__ float tile[kMaxE][kEcTokens + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kEcTokens;
  constexpr int PER = kMaxE / 64;  // experts per lane, lane l holds l, l+64, ...
#pragma unroll 1
  for (int u = 0; u < kEcTokens / 4; ++u) {
    const int tl = wave * (kEcTokens / 4) + u, t = t0 + tl;
    if (t >= T) break;
    const float* row = logits + (size_t)t * E;
    float v[PER];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? row[e] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      v[i] = lane + 64 * i < E ? expf(v[i] - m) : 0.0f;
      s += v[i];
    }
    s = wave_sum(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        tile[e][tl] = v[i] * inv;
        dest[(size_t)t * E + e] = -1;
        gate[(size_t)t * E + e] = 0.0f;
      }
    }
  }
  __syncthreads();
  // scores[e][t0 .. t0+15]: 16 consecutive floats per expert
  for (int i = threadIdx.x; i < E * kEcTokens; i += blockDim.x) {
    const int e = i / kEcTokens, tl = i % kEcTokens;
    if (t0 + tl < T) scores[(size_t)e * T + t0 + tl] = tile[e][tl];
  }
}

constexpr int kSelThreads = 1024;
constexpr int kSelLds = 16384;  // columns up to this many tokens are staged in LDS

// Inclusive prefix sum over the block (threads in order) of one int per
// thread; `total` gets the block sum. ws holds one int per wave.
__device__ __forceinline__ int block_incl_sum(int v, int* ws, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  __syncthreads();
  if (lane == 63) ws[wave] = v;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int x = ws[w];
    if (w < wave) before += x;
    total += x;
  }
  return before + v;
}

__global__ __launch_bounds__(kSelThreads) void ec_select(const float* __restrict__ scores, int T,
                                                         int E, int C,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_token,
                                                         int32_t* __restrict__ dest,
                                                         float* __restrict__ gate) {
  __shared__ uint32_t skeys[kSelLds];
  __shared__ int hist[256];
  __shared__ int wsum[kSelThreads / 64];
  __shared__ int sh_digit, sh_need;
  const int e = blockIdx.x, tid = threadIdx.x;
  const uint32_t* key = (const uint32_t*)(scores + (size_t)e * T);  // p >= 0: bits order as values
  if (tid == 0) {
    offsets[e] = e * C;
    if (e == 0) offsets[E] = E * C;
  }
  if (C == 0) return;
  // stage the column (all loads in flight at once) so the passes below read LDS
  const bool in_lds = T <= kSelLds;
  if (in_lds) {
#pragma unroll 4
    for (int t = tid; t < T; t += kSelThreads) skeys[t] = key[t];
    __syncthreads();
  }
  auto K = [&](int t) { return in_lds ? skeys[t] : key[t]; };

  // radix select: the C-th largest key, prefix/mask over the digits fixed so far
  uint32_t prefix = 0, mask = 0;
  int need = C;  // how many keys still to take among those matching the prefix
  if (C < T) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += kSelThreads) hist[b] = 0;
      __syncthreads();
#pragma unroll 4
      for (int t = tid; t < T; t += kSelThreads) {
        const uint32_t k = K(t);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      // digit holding the need-th largest key: thread i looks at digit 255 - i;
      // a prefix sum in that (descending) order gives the keys above each digit
      {
        const int dg = 255 - tid;
        const int v = tid < 256 ? hist[dg] : 0;
        int tot;
        const int incl = block_incl_sum(v, wsum, tot);
        if (tid < 256 && incl - v < need && need <= incl) {
          sh_digit = dg;
          sh_need = need - (incl - v);
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh_digit << shift;
      mask |= 255u << shift;
      need = sh_need;
    }
  }
  // Keep keys above the threshold and the first `need` keys equal to it
  // (every key when C == T). Thread i owns tokens [i*S, (i+1)*S): one scan of
  // its counts gives how many kept keys precede each of its tokens.
  const bool all = C >= T;
  const int S = (T + kSelThreads - 1) / kSelThreads;
  const int tb = tid * S, te = min(T, tb + S);
  int ngt = 0, neq = 0;
  for (int t = tb; t < te; ++t) {
    const uint32_t k = K(t);
    ngt += (all || k > prefix) ? 1 : 0;
    neq += (!all && k == prefix) ? 1 : 0;
  }
  int tot;
  const int gt_before = block_incl_sum(ngt, wsum, tot) - ngt;
  const int eq_before = block_incl_sum(neq, wsum, tot) - neq;
  int g = gt_before, q = eq_before;
  for (int t = tb; t < te; ++t) {
    const uint32_t k = K(t);
    const bool gt = all || k > prefix;
    const bool eq = !all && k == prefix;
    const bool keep = gt || (eq && q < need);
    const int pos = g + min(q, need);
    if (keep && pos < C) {  // exactly C keys are kept; the bound only guards the store
      const int r = e * C + pos;
      sorted_token[r] = t;
      dest[(size_t)t * E + e] = r;
      gate[(size_t)t * E + e] = __uint_as_float(k);
    }
    g += gt ? 1 : 0;
    q += eq ? 1 : 0;
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_expert_choice(const float* logits, int T, int E, int C, float* scores,
                                 int32_t* offsets, int32_t* sorted_token, int32_t* dest_row,
                                 float* gate, moe_stream_t stream) {
  if (T < 0 || E < 1 || C < 0) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if ((long)T * E >= (1L << 31)) return MOE_ERR_UNSUPPORTED;
  if (!offsets) return MOE_ERR_INVALID;
  const int Cc = C < T ? C : T;
  if (T > 0 && (!logits || !scores || !dest_row || !gate || (Cc > 0 && !sorted_token)))
    return MOE_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  if (T > 0)
    hipLaunchKernelGGL(ec_scores, dim3(ceil_div(T, kEcTokens)), dim3(256), 0, s, logits, T, E,
                       scores, dest_row, gate);
  hipLaunchKernelGGL(ec_select, dim3(E), dim3(kSelThreads), 0, s, scores, T, E, Cc, offsets,
                     sorted_token, dest_row, gate);
  return launch_status();
}
