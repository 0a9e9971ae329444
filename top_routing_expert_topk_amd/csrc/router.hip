// Router: skinny GEMM x . W_g^T on bf16 MFMA (or fp32 FMA), fused with the
// full softmax, a wavefront top-k with lowest-index tie-break, the gates and
// per-block probability partial sums.
//
// What it computes: the gate equation G(x) = softmax(TopK(x . W_g)) and the
// TopKRouter of page "MoE混合专家模型路由机制原理与稀疏激活实现" (sections
// "门控路由原理" and "Top-K门控路由的PyTorch实现"): a bias-free linear gate,
// softmax over all experts, top-k, renormalisation over the selected k; the
// optional per-expert router bias of "MoE 架构完整指南" section 5.2.
// The selection is made on the fp32 logits (the same order as selecting on
// the probabilities) so that no tie is created by rounding in exp.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int RT = kRouterTokens;  // tokens per block
constexpr int KC = 64;             // bf16 elements of K staged per step
constexpr int kWaves = 4;

// Total order for selection: larger value first, then lower expert index.
// +0 and -0 map to the same key.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = (v == 0.0f) ? 0u : __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// LDS byte layout of one block: [GEMM staging | logits tile] (aliased) then
// the per-wave probability partials.
__host__ __device__ inline int pad16(int E) { return (E + 15) & ~15; }
__host__ __device__ inline size_t stage_bytes(int E) { return (size_t)(RT + pad16(E)) * KC * 2; }
__host__ __device__ inline size_t logit_bytes(int E) { return (size_t)RT * pad16(E) * 4; }
__host__ __device__ inline size_t union_bytes(int E) {
  size_t a = stage_bytes(E), b = logit_bytes(E);
  return a > b ? a : b;
}
__host__ __device__ inline size_t router_lds(int E) {
  return union_bytes(E) + (size_t)kWaves * E * 4;
}

// Logits of the block's RT tokens into lg[RT][Ep] (bias added), bf16 MFMA.
// v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 k, B = 32 k x 16 experts;
// lane l supplies row (l%16) and k-octet (l/16) of each operand and receives
// D[4*(l/16)+v][l%16], v = 0..3.
__device__ void logits_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                            const float* __restrict__ gbias, int T, int d, int E, int t0,
                            unsigned char* smem, float* lg) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Ep = pad16(E);
  const int NT = Ep / 16;
  const int P = 2 * NT;  // (token tile, expert tile) pairs
  uint16_t* sX = (uint16_t*)smem;
  uint16_t* sW = sX + RT * KC;
  f32x4 acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < d; k0 += KC) {
    {  // x tile: RT rows x 8 chunks of 16 B, one chunk per thread
      int row = tid >> 3, ch = tid & 7;
      int t = t0 + row, kk = k0 + ch * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (t < T && kk < d) v = *(const u32x4*)(x + (size_t)t * d + kk);
      *(u32x4*)(sX + row * KC + ((ch ^ (row & 7)) * 8)) = v;
    }
    for (int c = tid; c < Ep * 8; c += 256) {
      int row = c >> 3, ch = c & 7;
      int kk = k0 + ch * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (row < E && kk < d) v = *(const u32x4*)(w + (size_t)row * d + kk);
      *(u32x4*)(sW + row * KC + ((ch ^ (row & 7)) * 8)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int ch = kh * 4 + (lane >> 4);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int p = wave + kWaves * q;
        if (p < P) {
          const int mt = p / NT, nt = p % NT;
          const int ra = mt * 16 + (lane & 15), rb = nt * 16 + (lane & 15);
          bf16x8 a = *(const bf16x8*)(sX + ra * KC + ((ch ^ (ra & 7)) * 8));
          bf16x8 b = *(const bf16x8*)(sW + rb * KC + ((ch ^ (rb & 7)) * 8));
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[q], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  // staging is dead now; lg aliases it
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int p = wave + kWaves * q;
    if (p < P) {
      const int mt = p / NT, nt = p % NT;
      const int e = nt * 16 + (lane & 15);
      const float b = (gbias && e < E) ? gbias[e] : 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tl = mt * 16 + 4 * (lane >> 4) + v;
        lg[tl * Ep + e] = acc[q][v] + b;
      }
    }
  }
}

// fp32 logits by plain FMA dot products (the small fp32 workloads).
__device__ void logits_f32(const float* __restrict__ x, const float* __restrict__ w,
                           const float* __restrict__ gbias, int T, int d, int E, int t0,
                           float* lg) {
  const int Ep = pad16(E);
  for (int pi = threadIdx.x; pi < RT * E; pi += 256) {
    const int tl = pi / E, e = pi % E, t = t0 + tl;
    float s = 0.0f;
    if (t < T) {
      const float* xr = x + (size_t)t * d;
      const float* wr = w + (size_t)e * d;
      for (int i = 0; i < d; ++i) s = fmaf(xr[i], wr[i], s);
    }
    lg[tl * Ep + e] = s + (gbias ? gbias[e] : 0.0f);
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void router_kernel(
    const void* __restrict__ x, const void* __restrict__ w, const float* __restrict__ gbias,
    int T, int d, int E, int k, int renorm, float* __restrict__ logits_out,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out, float* __restrict__ partial) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int t0 = blockIdx.x * RT;
  const int Ep = pad16(E);
  float* lg = (float*)smem;
  float* part = (float*)(smem + union_bytes(E));  // [kWaves][E]

  if (BF16)
    logits_bf16((const uint16_t*)x, (const uint16_t*)w, gbias, T, d, E, t0, smem, lg);
  else
    logits_f32((const float*)x, (const float*)w, gbias, T, d, E, t0, lg);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int EPL = (E + 63) >> 6;  // experts per lane (<= 8)
  float pacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pacc[i] = 0.0f;

  for (int tl = wave; tl < RT; tl += kWaves) {
    const int t = t0 + tl;
    if (t >= T) break;
    float v[8], ex[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = lane + 64 * i;
      v[i] = (i < EPL && e < E) ? lg[tl * Ep + e] : 0.0f;
      if (logits_out && i < EPL && e < E) logits_out[(size_t)t * E + e] = v[i];
    }
    uint32_t taken = 0;
    float selv[kMaxK];
    int sele[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = lane + 64 * i;
          if (i < EPL && e < E && !((taken >> i) & 1u)) {
            uint64_t key = ((uint64_t)ordered_bits(v[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
            best = key > best ? key : best;
          }
        }
        best = wave_max_u64(best);
        const int ej = (int)(0xFFFFFFFFu - (uint32_t)best);
        if ((ej & 63) == lane) taken |= 1u << (ej >> 6);
        sele[j] = ej;
        selv[j] = from_ordered_bits((uint32_t)(best >> 32));
      }
    }
    const float m = selv[0];
    float zl = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = lane + 64 * i;
      ex[i] = (i < EPL && e < E) ? expf(v[i] - m) : 0.0f;
      zl += ex[i];
    }
    const float z = wave_sum_f32(zl);
    float zs = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) zs += expf(selv[j] - m);
    const float denom = renorm ? zs : z;
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
          idx_out[(size_t)t * k + j] = sele[j];
          gate_out[(size_t)t * k + j] = expf(selv[j] - m) / denom;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) pacc[i] += ex[i] / z;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = lane + 64 * i;
    if (i < EPL && e < E) part[wave * E + e] = pacc[i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    partial[(size_t)blockIdx.x * E + e] = ((part[e] + part[E + e]) + part[2 * E + e]) + part[3 * E + e];
}

// prob_sum[e] = sum over blocks of partial[b][e]: fixed-order tree in double.
__global__ __launch_bounds__(256) void router_reduce(const float* __restrict__ partial, int nb,
                                                      int E, float* __restrict__ prob_sum) {
  __shared__ double s[256];
  const int e = blockIdx.x;
  double a = 0.0;
  for (int b = threadIdx.x; b < nb; b += 256) a += (double)partial[(size_t)b * E + e];
  s[threadIdx.x] = a;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) prob_sum[e] = (float)s[0];
}

__global__ void fill_zero_f32(float* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_router_topk(const void* x, int dtype, int T, int d, const void* w_gate,
                               const float* gate_bias, int E, int k, int renorm,
                               float* logits_out, int32_t* topk_idx, float* topk_gate,
                               float* prob_sum, void* ws, size_t ws_bytes,
                               moe_stream_t stream) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (renorm != 0 && renorm != 1) return MOE_ERR_INVALID;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_BF16 && (d % 8) != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) {
    if (prob_sum) {
      hipLaunchKernelGGL(fill_zero_f32, dim3(ceil_div(E, 256)), dim3(256), 0,
                         (hipStream_t)stream, prob_sum, E);
      return launch_status();
    }
    return MOE_OK;
  }
  if (!x || !w_gate || !topk_idx || !topk_gate) return MOE_ERR_INVALID;
  if (!ws || ws_bytes < router_ws(T, E)) return MOE_ERR_WORKSPACE;
  const int nb = router_blocks(T);
  const size_t lds = router_lds(E);
  hipStream_t s = (hipStream_t)stream;
  float* partial = (float*)ws;
  if (lds > 65536 &&
      hipFuncSetAttribute(
          (const void*)(dtype == MOE_BF16 ? router_kernel<true> : router_kernel<false>),
          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return MOE_ERR_LAUNCH;
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(router_kernel<true>, dim3(nb), dim3(256), lds, s, x, w_gate, gate_bias, T,
                       d, E, k, renorm, logits_out, topk_idx, topk_gate, partial);
  else
    hipLaunchKernelGGL(router_kernel<false>, dim3(nb), dim3(256), lds, s, x, w_gate, gate_bias,
                       T, d, E, k, renorm, logits_out, topk_idx, topk_gate, partial);
  if (prob_sum)
    hipLaunchKernelGGL(router_reduce, dim3(E), dim3(256), 0, s, partial, nb, E, prob_sum);
  return launch_status();
}
