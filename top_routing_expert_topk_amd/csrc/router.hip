// Router: logits x . W_g^T (+ router bias), full softmax, a wavefront top-k
// with lowest-index tie-break, gates and per-block probability partial sums.
//
// What it computes: the gate equation G(x) = softmax(TopK(x . W_g)) and the
// TopKRouter of page "MoE混合专家模型路由机制原理与稀疏激活实现" (sections
// "门控路由原理" and "Top-K门控路由的PyTorch实现"): a bias-free linear gate,
// softmax over all experts, top-k, renormalisation over the selected k; the
// optional per-expert router bias of "MoE 架构完整指南" section 5.2.
// The selection is made on the fp32 logits (the same order as selecting on
// the probabilities) so that no tie is created by rounding in exp.
//
// bf16 layers run two kernels:
//   router_logits_bf16  a skinny MFMA GEMM split over (token tile, K range)
//                       blocks so that even a handful of tokens (decode) or
//                       a long K (d = 7168) spreads over every CU; operands
//                       reach LDS by direct global->LDS DMA, double-buffered;
//                       each block writes fp32 partial logits [split][T][E].
//   router_select       one wave per token: partial logits summed in split
//                       order (+ bias), then softmax / top-k / gates.
// fp32 layers (small) use one fused kernel with FMA dot products.
// router_reduce sums the per-block probability partials in a fixed order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RT = kRouterTokens;  // tokens per selection block
constexpr int kWaves = 4;
constexpr int RT32 = 32;  // tokens per fp32 fused block (a multiple of RT)
constexpr int RKS = 32;  // K columns per LDS stage (64-byte rows)

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

// One token, one wave. Lane l holds v[i] = logit of expert l + 64 i (i < 8).
// Writes the k selected experts (descending, lower index first on ties) and
// their gates, and adds this token's softmax probabilities to pacc.
__device__ __forceinline__ void select_token(const float (&v)[8], int E, int k, int renorm,
                                             int lane, int32_t* __restrict__ idx_row,
                                             float* __restrict__ gate_row, float (&pacc)[8]) {
  const int EPL = (E + 63) >> 6;
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
          const uint64_t key =
              ((uint64_t)ordered_bits(v[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
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
  float ex[8], zl = 0.0f;
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
        idx_row[j] = sele[j];
        gate_row[j] = expf(selv[j] - m) / denom;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) pacc[i] += ex[i] / z;
}

// Per-block probability partials: the four waves' sums added in wave order.
__device__ __forceinline__ void write_prob_partial(const float (&pacc)[8], int E, float* part,
                                                   float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int EPL = (E + 63) >> 6;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = lane + 64 * i;
    if (i < EPL && e < E) part[wave * E + e] = pacc[i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    out[(size_t)blockIdx.x * E + e] =
        ((part[e] + part[E + e]) + part[2 * E + e]) + part[3 * E + e];
}

// ---------------------------------------------------- bf16 partial logits --
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// 16 consecutive 64-byte rows at one chunk land in 16 distinct bank groups.
__device__ __forceinline__ int rswz(int r, int c) { return c ^ ((r >> 2) & 3); }

// Block: TT tokens (64 * MTW) x EP experts (16 * NTE) over the 32-wide K
// chunks [c0, c1) of its split. LDS stage = TT token rows then EP expert rows,
// 64 bytes each, chunk c of row r at slot c ^ ((r >> 2) & 3); each DMA
// instruction fills 16 rows, lane l writing slot l%4 of row l/4. Wave w owns
// token tiles w, w+4, ... and every expert tile, so a token fragment is read
// once per chunk and reused across all expert tiles. A ring of NS stages
// (as many as fit in 80 KB, so two blocks share a CU) keeps NS - 1 chunks
// in flight: a chunk is a few MFMAs per wave, far shorter than a load.
template <int MTW, int NTE>
struct LogitsCfg {
  static constexpr int ROWS = 64 * MTW + 16 * NTE;
  static constexpr int STAGE = ROWS * RKS;  // bf16 elements
  static constexpr int NS0 = 81920 / (STAGE * 2);
  static constexpr int NS = NS0 < 2 ? 2 : NS0 > 4 ? 4 : NS0;
  static constexpr size_t LDS = (size_t)NS * STAGE * 2;
};
// v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 k, B = 32 k x 16 experts; lane
// l supplies row l%16, k-octet l/16 and receives D[4*(l/16)+v][l%16].
template <int MTW, int NTE>
__global__ __launch_bounds__(256) void router_logits_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int d, int E, int nch,
    int split, float* __restrict__ part) {
  constexpr int TT = 64 * MTW, EP = 16 * NTE;
  constexpr int ROWS = TT + EP;
  constexpr int STAGE = ROWS * RKS;
  constexpr int NS = LogitsCfg<MTW, NTE>::NS;
  constexpr int NI = ROWS / 16;  // DMA instructions per stage (multiple of 4)
  constexpr int IPC = NI / 4;    // of them per wave
  extern __shared__ __align__(1024) uint16_t rs[];
  const int tile = blockIdx.x / split, p = blockIdx.x % split;
  const int t0 = tile * TT;
  const int c0 = p * nch / split, c1 = (p + 1) * nch / split;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  const uint16_t* src[NI / 4];
#pragma unroll
  for (int q = 0; q < NI / 4; ++q) {
    const int r = (q * 4 + wave) * 16 + (lane >> 2);
    const uint16_t* base;
    if (r < TT) {
      const int t = min(t0 + r, T - 1);
      base = x + (size_t)t * d;
    } else {
      const int e = min(r - TT, E - 1);
      base = w + (size_t)e * d;
    }
    src[q] = base + rswz(r, lane & 3) * 8;
  }
  auto issue = [&](int buf, int c) {
#pragma unroll
    for (int q = 0; q < NI / 4; ++q)
      dma16(src[q] + c * RKS, &rs[buf * STAGE + (q * 4 + wave) * 16 * RKS]);
  };

  f32x4 acc[MTW][NTE];
#pragma unroll
  for (int j = 0; j < MTW; ++j)
#pragma unroll
    for (int n = 0; n < NTE; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ch = lane >> 4;
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (c0 + i < c1) issue(i, c0 + i);
  for (int c = c0; c < c1; ++c) {
    const int buf = (c - c0) % NS;
    // this wave's DMA of chunk c has landed (the up to NS - 2 later chunks
    // issued may not have); after the barrier every wave's has, and every
    // wave is done reading the stage of chunk c - 1, which takes chunk
    // c + NS - 1
    const int later = min(c1 - 1 - c, NS - 2);
    if (NS > 3 && later >= 2) wait_vm<(NS > 3 ? 2 : 0) * IPC>();
    else if (NS > 2 && later >= 1) wait_vm<(NS > 2 ? 1 : 0) * IPC>();
    else wait_vm<0>();
    lds_barrier();
    if (c + NS - 1 < c1) issue((c - c0 + NS - 1) % NS, c + NS - 1);
    const uint16_t* sx = rs + buf * STAGE;
    const uint16_t* sw = sx + TT * RKS;
    bf16x8 a[MTW];
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      const int r = (wave + 4 * j) * 16 + (lane & 15);
      a[j] = *(const bf16x8*)(sx + r * RKS + rswz(r, ch) * 8);
    }
#pragma unroll
    for (int n = 0; n < NTE; ++n) {
      const int r = n * 16 + (lane & 15);
      const bf16x8 b = *(const bf16x8*)(sw + r * RKS + rswz(r, ch) * 8);
#pragma unroll
      for (int j = 0; j < MTW; ++j)
        acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b, acc[j][n], 0, 0, 0);
    }
  }
  float* pp = part + (size_t)p * T * E;
#pragma unroll
  for (int j = 0; j < MTW; ++j)
#pragma unroll
    for (int n = 0; n < NTE; ++n) {
      const int e = n * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + (wave + 4 * j) * 16 + 4 * (lane >> 4) + v;
        if (t < T && e < E) pp[(size_t)t * E + e] = acc[j][n][v];
      }
    }
}

__global__ __launch_bounds__(256) void router_select(
    const float* __restrict__ part, int split, const float* __restrict__ gbias, int T, int E,
    int k, int renorm, float* __restrict__ logits_out, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, float* __restrict__ probpart) {
  __shared__ float wpart[kWaves * kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int EPL = (E + 63) >> 6;
  float pacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pacc[i] = 0.0f;
  const int t = blockIdx.x * RT + wave;
  if (t < T) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = lane + 64 * i;
      float s = 0.0f;
      if (i < EPL && e < E) {
        // partials in split order; loads issued 8 at a time
        const float* src = part + (size_t)t * E + e;
        const size_t stride = (size_t)T * E;
        int p = 0;
        for (; p + 8 <= split; p += 8) {
          float q[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) q[u] = src[(size_t)(p + u) * stride];
#pragma unroll
          for (int u = 0; u < 8; ++u) s += q[u];
        }
        for (; p < split; ++p) s += src[(size_t)p * stride];
        if (gbias) s += gbias[e];
        if (logits_out) logits_out[(size_t)t * E + e] = s;
      }
      v[i] = s;
    }
    select_token(v, E, k, renorm, lane, idx_out + (size_t)t * k, gate_out + (size_t)t * k, pacc);
  }
  write_prob_partial(pacc, E, wpart, probpart);
}

// ----------------------------------------------------------- fp32 fused --
// RT tokens per block: logits by FMA dot products into LDS, then selection.
__global__ __launch_bounds__(256) void router_f32(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ gbias,
    int T, int d, int E, int k, int renorm, float* __restrict__ logits_out,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out, float* __restrict__ probpart) {
  extern __shared__ float lg[];  // [RT32][E] then [kWaves][E]
  const int t0 = blockIdx.x * RT32;
  for (int pi = threadIdx.x; pi < RT32 * E; pi += 256) {
    const int tl = pi / E, e = pi % E, t = t0 + tl;
    float s = 0.0f;
    if (t < T) {
      const float* xr = x + (size_t)t * d;
      const float* wr = w + (size_t)e * d;
      for (int i = 0; i < d; ++i) s = fmaf(xr[i], wr[i], s);
    }
    lg[pi] = s + (gbias ? gbias[e] : 0.0f);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int EPL = (E + 63) >> 6;
  float pacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pacc[i] = 0.0f;
  for (int tl = wave; tl < RT32; tl += kWaves) {
    const int t = t0 + tl;
    if (t >= T) break;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = lane + 64 * i;
      v[i] = (i < EPL && e < E) ? lg[tl * E + e] : 0.0f;
      if (logits_out && i < EPL && e < E) logits_out[(size_t)t * E + e] = v[i];
    }
    select_token(v, E, k, renorm, lane, idx_out + (size_t)t * k, gate_out + (size_t)t * k, pacc);
  }
  write_prob_partial(pacc, E, lg + RT32 * E, probpart);
}

// prob_sum[e] = sum over blocks of probpart[b][e]: fixed-order tree in double.
__global__ __launch_bounds__(256) void router_reduce(const float* __restrict__ probpart, int nb,
                                                      int E, float* __restrict__ prob_sum) {
  __shared__ double s[256];
  const int e = blockIdx.x;
  double a = 0.0;
  for (int b = threadIdx.x; b < nb; b += 256) a += (double)probpart[(size_t)b * E + e];
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

template <int MTW, int NTE>
bool launch_logits(const RouterPlan& pl, const void* x, const void* w, int T, int d, int E,
                   float* part, hipStream_t s) {
  const size_t lds = LogitsCfg<MTW, NTE>::LDS;
  if (lds > 65536 &&
      hipFuncSetAttribute((const void*)router_logits_bf16<MTW, NTE>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return false;
  hipLaunchKernelGGL((router_logits_bf16<MTW, NTE>), dim3(pl.ntt * pl.split), dim3(256), lds, s,
                     (const uint16_t*)x, (const uint16_t*)w, T, d, E, pl.nch, pl.split, part);
  return true;
}

bool dispatch_logits(const RouterPlan& pl, const void* x, const void* w, int T, int d, int E,
                     float* part, hipStream_t s) {
  const int mtw = pl.tt / 64, nte = pl.ep / 16;
#define MOE_CASE(A, B)                               \
  if (mtw == A && nte == B) return launch_logits<A, B>(pl, x, w, T, d, E, part, s);
  MOE_CASE(4, 4)
  MOE_CASE(4, 8)
  MOE_CASE(2, 12)
  MOE_CASE(2, 16)
  MOE_CASE(1, 20)
  MOE_CASE(1, 24)
  MOE_CASE(1, 28)
  MOE_CASE(1, 32)
#undef MOE_CASE
  return false;
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
  if (dtype == MOE_BF16 && (d % RKS) != 0) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    if (prob_sum) {
      hipLaunchKernelGGL(fill_zero_f32, dim3(ceil_div(E, 256)), dim3(256), 0, s, prob_sum, E);
      return launch_status();
    }
    return MOE_OK;
  }
  if (!x || !w_gate || !topk_idx || !topk_gate) return MOE_ERR_INVALID;
  if (!ws || ws_bytes < router_ws(T, d, E)) return MOE_ERR_WORKSPACE;
  int nb = router_blocks(T);
  float* logit_part = (float*)ws;
  float* probpart = (float*)((unsigned char*)ws + router_partial_bytes(T, d, E));
  if (dtype == MOE_BF16) {
    const RouterPlan pl = router_plan(T, d, E);
    if (!dispatch_logits(pl, x, w_gate, T, d, E, logit_part, s)) return MOE_ERR_LAUNCH;
    hipLaunchKernelGGL(router_select, dim3(nb), dim3(256), 0, s, logit_part, pl.split, gate_bias,
                       T, E, k, renorm, logits_out, topk_idx, topk_gate, probpart);
  } else {
    const size_t lds = (size_t)(RT32 + kWaves) * E * sizeof(float);
    if (lds > 65536 &&
        hipFuncSetAttribute((const void*)router_f32, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return MOE_ERR_LAUNCH;
    nb = ceil_div(T, RT32);
    hipLaunchKernelGGL(router_f32, dim3(nb), dim3(256), lds, s, (const float*)x,
                       (const float*)w_gate, gate_bias, T, d, E, k, renorm, logits_out, topk_idx,
                       topk_gate, probpart);
  }
  if (prob_sum)
    hipLaunchKernelGGL(router_reduce, dim3(E), dim3(256), 0, s, probpart, nb, E, prob_sum);
  return launch_status();
}
