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
//   router_logits_wide  a skinny MFMA GEMM split over (token tile, K range)
//                       blocks so that even a handful of tokens (decode) or
//                       a long K (d = 7168) spreads over every CU; operands
//                       reach LDS by direct global->LDS DMA through a ring of
//                       stages; each block writes fp32 partial logits
//                       [split][T][E]. router_logits_bf16 is the same product
//                       on 16x16x32 tiles for d not a multiple of 64.
//   router_select       S lanes per token (8 experts each): partial logits
//                       summed in split order (+ bias), each lane's top-k
//                       merged across the S lanes, softmax, gates and the
//                       block's probability column sums.
// fp32 layers (small) compute the logits by FMA dot products
// (router_logits_f32) and run the same selection over them.
// router_reduce sums the per-block probability partials in a fixed order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RT32 = 32;            // tokens per fp32 logits block
constexpr int kF32Chunk = 32;       // K columns staged per step (fp32 logits)
constexpr int kF32Row = kF32Chunk + 1;  // their LDS row stride (no bank conflicts)
constexpr int RKS = 32;             // K columns per LDS stage (64-byte rows)
constexpr int kSelectPerLane = 8;   // experts per lane in the selection

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

// Insert key into top[0..KK) (descending), dropping the smallest.
template <int KK>
__device__ __forceinline__ void topk_insert(uint64_t (&top)[KK], uint64_t key) {
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    const uint64_t hi = top[j] > key ? top[j] : key;
    key = top[j] > key ? key : top[j];
    top[j] = hi;
  }
}
// top (descending) becomes the KK largest of top and o (both descending):
// the larger of top[j] and o[KK-1-j] are those KK and form a bitonic
// sequence, which half-cleaners of width KK/2 .. 1 sort.
template <int KK>
__device__ __forceinline__ void topk_merge(uint64_t (&top)[KK], const uint64_t (&o)[KK]) {
#pragma unroll
  for (int j = 0; j < KK; ++j) top[j] = top[j] > o[KK - 1 - j] ? top[j] : o[KK - 1 - j];
#pragma unroll
  for (int h = KK / 2; h >= 1; h >>= 1)
#pragma unroll
    for (int j = 0; j < KK; ++j)
      if ((j & h) == 0) {
        const uint64_t a = top[j], b = top[j + h];
        top[j] = a > b ? a : b;
        top[j + h] = a > b ? b : a;
      }
}

// Selection over the partial logits: S lanes per token (a power of two),
// each holding NPL = 8 of its experts (consecutive ones, e = sg * 8 + i, when
// rows split into 16-byte pieces; else e = sg + S * i), so a block of 4 waves
// takes 256 / S tokens. A lane sums its experts' partials in split order
// (+ bias), keeps its KK largest keys (logit, then lower index first), and
// the S lanes merge their lists by xor butterflies, after which every lane
// of the token holds the token's top KK. The softmax denominator is the
// xor-butterfly sum of the lanes' sums (the same bits on every lane), and
// the block's probability column sums run over its tokens in order.
template <int S, int KK>
__global__ __launch_bounds__(256) void router_select(
    const float* __restrict__ part, int split, const float* __restrict__ gbias, int T, int E,
    int k, int renorm, float* __restrict__ logits_out, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, float* __restrict__ probpart) {
  constexpr int NPL = kSelectPerLane;
  constexpr int TPW = 64 / S, TB = 4 * TPW;  // tokens per wave, per block
  __shared__ float sp[TB * S * NPL];         // [TB][E] logits, then probabilities (E <= S * NPL)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tl = wave * TPW + lane / S, sg = lane % S;
  const int t = blockIdx.x * TB + tl;
  const bool valid = t < T;
  const bool vec = (NPL % 4) == 0 && (E % 4) == 0;
  auto expert = [&](int i) { return vec ? sg * NPL + i : sg + S * i; };
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = 0.0f;
  if (valid) {
    const size_t plane = (size_t)T * E;
    const float* src = part + (size_t)t * E;
    // PB planes per batch, so that about 16 loads per lane are in flight
    if (vec) {
      constexpr int NQ = NPL / 4 > 0 ? NPL / 4 : 1, PB = 16 / NQ > 0 ? 16 / NQ : 1;
      for (int p0 = 0; p0 < split; p0 += PB) {
        f32x4 a[PB][NQ];
#pragma unroll
        for (int u = 0; u < PB; ++u)
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            if (p0 + u < split && sg * NPL + 4 * q < E)
              a[u][q] = *(const f32x4*)(src + (size_t)(p0 + u) * plane + sg * NPL + 4 * q);
#pragma unroll
        for (int u = 0; u < PB; ++u)
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            if (p0 + u < split && sg * NPL + 4 * q < E)
#pragma unroll
              for (int w = 0; w < 4; ++w) v[4 * q + w] += a[u][q][w];
      }
    } else {
      constexpr int PB = 16 / NPL > 0 ? 16 / NPL : 1;
      for (int p0 = 0; p0 < split; p0 += PB) {
        float a[PB][NPL];
#pragma unroll
        for (int u = 0; u < PB; ++u)
#pragma unroll
          for (int i = 0; i < NPL; ++i)
            if (p0 + u < split && expert(i) < E) a[u][i] = src[(size_t)(p0 + u) * plane + expert(i)];
#pragma unroll
        for (int u = 0; u < PB; ++u)
#pragma unroll
          for (int i = 0; i < NPL; ++i)
            if (p0 + u < split && expert(i) < E) v[i] += a[u][i];
      }
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = expert(i);
      if (e < E) {
        if (gbias) v[i] += gbias[e];
        if (logits_out) logits_out[(size_t)t * E + e] = v[i];
      }
    }
  }
  auto key = [](float x, int e) {
    return ((uint64_t)ordered_bits(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
  };
  uint64_t top[KK];
#pragma unroll
  for (int j = 0; j < KK; ++j) top[j] = 0;
  if constexpr (KK <= 2) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = expert(i);
      topk_insert(top, (valid && e < E) ? key(v[i], e) : 0ull);
    }
  } else {
    // With k <= S, a logit below the smallest of the S lanes' largest has at
    // least S larger ones, so only logits at or above it are inserted; they
    // are read back from LDS in a loop that runs as often as the lane with
    // the most of them needs.
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = expert(i);
      if (e < E) {
        lm = fmaxf(lm, v[i]);
        sp[tl * E + e] = v[i];
      }
    }
    float tau = lm;
#pragma unroll
    for (int off = 1; off < S; off <<= 1) tau = fminf(tau, __shfl_xor(tau, off, 64));
    if (k > S) tau = -INFINITY;
    uint32_t cand = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (valid && expert(i) < E && v[i] >= tau) cand |= 1u << i;
    while (cand) {
      const int i = __builtin_ctz(cand);
      cand &= cand - 1;
      const int e = expert(i);
      topk_insert(top, key(sp[tl * E + e], e));
    }
  }
#pragma unroll
  for (int off = 1; off < S; off <<= 1) {
    uint64_t o[KK];
#pragma unroll
    for (int j = 0; j < KK; ++j) o[j] = __shfl_xor(top[j], off, 64);
    topk_merge(top, o);
  }
  const float m = from_ordered_bits((uint32_t)(top[0] >> 32));
  float ex[NPL], zl = 0.0f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    ex[i] = (valid && expert(i) < E) ? expf(v[i] - m) : 0.0f;
    zl += ex[i];
  }
  float z = zl;
#pragma unroll
  for (int off = 1; off < S; off <<= 1) z += __shfl_xor(z, off, 64);
  if (valid && sg == 0) {
    float selv[KK], zs = 0.0f;
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      selv[j] = from_ordered_bits((uint32_t)(top[j] >> 32));
      if (j < k) zs += expf(selv[j] - m);
    }
    const float denom = renorm ? zs : z;
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      if (j < k) {
        idx_out[(size_t)t * k + j] = (int)(0xFFFFFFFFu - (uint32_t)top[j]);
        gate_out[(size_t)t * k + j] = expf(selv[j] - m) / denom;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = expert(i);
    if (e < E) sp[tl * E + e] = valid ? ex[i] / z : 0.0f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    float s = 0.0f;
    for (int r = 0; r < TB; ++r) s += sp[r * E + e];
    probpart[(size_t)blockIdx.x * E + e] = s;
  }
}

// ------------------------------------------- bf16 logits, 32x32x16 tiles --
// The same split-K product for d a multiple of 64, with 64-column stages
// (128-byte LDS rows, chunk c of row r at c ^ ((r >> 1) & 7), which puts the
// 16 rows a ds_read_b128 serves at once on distinct bank groups) and the
// waves in a 2 x NWN grid (NWN = 4, two waves per SIMD, when the expert
// tiles split evenly; else 2), each owning (TT/2) tokens x (EP/NWN) experts
// as TM x TNW v_mfma_f32_32x32x16_bf16 tiles: per 16 k a wave reads TM + TNW
// fragments for TM * TNW MFMAs. Lane l supplies row l%32 and k-octet l/32 of
// both operands (A = 32 experts, B = 32 tokens) and receives expert
// 8*(v/4) + 4*(l/32) + v%4 of token l%32 in accumulator v.
constexpr int RK2 = 64;  // K columns per stage
constexpr int kWideNWN = 4;  // waves along the experts when a block has an even TN
__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int TM, int TN, int NWN>
struct WideCfg {
  static constexpr int TT = 64 * TM, EP = 64 * TN, ROWS = TT + EP;
  static constexpr int STAGE = ROWS * RK2;  // bf16 elements
  static constexpr int NS0 = 163840 / (STAGE * 2);
  static constexpr int NS = NS0 < 2 ? 2 : NS0 > 4 ? 4 : NS0;
  static constexpr size_t LDS = (size_t)NS * STAGE * 2;
};

template <int TM, int TN, int NWN>
__global__ __launch_bounds__(128 * NWN) void router_logits_wide(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int d, int E, int nch,
    int split, float* __restrict__ part) {
  using C = WideCfg<TM, TN, NWN>;
  constexpr int TT = C::TT, EP = C::EP, ROWS = C::ROWS, STAGE = C::STAGE, NS = C::NS;
  constexpr int NW = 2 * NWN;         // waves: 2 along tokens x NWN along experts
  constexpr int TNW = 2 * TN / NWN;   // expert tiles per wave
  constexpr int IPW = ROWS / 8 / NW;  // DMA instructions (8 rows each) per wave per stage
  static_assert((ROWS / 8) % NW == 0 && TNW >= 1, "wave layout");
  extern __shared__ __align__(1024) uint16_t rs[];
  const int tile = blockIdx.x / split, p = blockIdx.x % split;
  const int t0 = tile * TT;
  const int c0 = p * nch / split, c1 = (p + 1) * nch / split;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / NWN, wn = wave % NWN;

  const uint16_t* src[IPW];
#pragma unroll
  for (int q = 0; q < IPW; ++q) {
    const int r = (q * NW + wave) * 8 + (lane >> 3);
    const uint16_t* base = r < TT ? x + (size_t)min(t0 + r, T - 1) * d
                                  : w + (size_t)min(r - TT, E - 1) * d;
    src[q] = base + swz8(r, lane & 7) * 8;
  }
  auto issue = [&](int buf, int c) {
#pragma unroll
    for (int q = 0; q < IPW; ++q)
      dma16(src[q] + (size_t)c * RK2, &rs[buf * STAGE + (q * NW + wave) * 8 * RK2]);
  };
  // part p of P of a stage's DMA instructions
  auto issue_part = [&](int buf, int c, int p, int P) {
#pragma unroll
    for (int q = 0; q < IPW; ++q)
      if (q * P / IPW == p)
        dma16(src[q] + (size_t)c * RK2, &rs[buf * STAGE + (q * NW + wave) * 8 * RK2]);
  };

  f32x16 acc[TM][TNW];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j) acc[i][j] = f32x16{};

  const int ch = lane >> 5;
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (c0 + i < c1) issue(i, c0 + i);
  for (int c = c0; c < c1; ++c) {
    const int buf = (c - c0) % NS;
    // as in router_logits_bf16: chunk c has landed for this wave, and after
    // the barrier for every wave, whose reads of chunk c - 1 are done
    const int later = min(c1 - 1 - c, NS - 2);
    if (NS > 3 && later >= 2) wait_vm<(NS > 3 ? 2 : 0) * IPW>();
    else if (NS > 2 && later >= 1) wait_vm<(NS > 2 ? 1 : 0) * IPW>();
    else wait_vm<0>();
    lds_barrier();
    // the refill of chunk c - 1's buffer goes out in three parts, before each
    // of the first three 16-column sub-steps, so no wave issues all of it
    // behind the barrier before its first MFMA (router call 80 -> 77 us on
    // the DeepSeek shape, 22 -> 21 us on the Switch shape, in an A/B on one
    // box); all of it is issued before the next wait, whose counts hold
    const bool refill = c + NS - 1 < c1;
    const int rbuf = (c - c0 + NS - 1) % NS;
    const uint16_t* st = rs + buf * STAGE;
#pragma unroll
    for (int s = 0; s < RK2 / 16; ++s) {
      if (refill && s < 3) issue_part(rbuf, c + NS - 1, s, 3);
      bf16x8 a[TNW], b[TM];
#pragma unroll
      for (int j = 0; j < TNW; ++j) {
        const int r = TT + wn * (EP / NWN) + 32 * j + (lane & 31);
        a[j] = *(const bf16x8*)(st + r * RK2 + swz8(r, 2 * s + ch) * 8);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (TT / 2) + 32 * i + (lane & 31);
        b[i] = *(const bf16x8*)(st + r * RK2 + swz8(r, 2 * s + ch) * 8);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[i], acc[i][j], 0, 0, 0);
    }
  }
  float* pp = part + (size_t)p * T * E;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int t = t0 + wm * (TT / 2) + 32 * i + (lane & 31);
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < TNW; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = wn * (EP / NWN) + 32 * j + 8 * g + 4 * ch;
        float* dst = pp + (size_t)t * E + e;
        if ((E & 3) == 0) {
          if (e < E)
            *(f32x4*)dst = f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                 acc[i][j][4 * g + 3]};
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (e + u < E) dst[u] = acc[i][j][4 * g + u];
        }
      }
  }
}

// ------------------------------------------------------------ fp32 logits --
// RT32 tokens x E experts per block by FMA dot products, each over
// i = 0 .. d-1 in order, a chunk of columns at a time from rows staged in LDS
// by coalesced loads; the logits (without bias) go to part [T][E], which the
// selection then reads as a single K range.
__global__ __launch_bounds__(256) void router_logits_f32(
    const float* __restrict__ x, const float* __restrict__ w, int T, int d, int E,
    float* __restrict__ part) {
  // [RT32][E] sums, then RT32 token rows and E expert rows of a chunk
  extern __shared__ float lg[];
  float* xs = lg + RT32 * E;
  float* ws = xs + RT32 * kF32Row;
  const int t0 = blockIdx.x * RT32;
  for (int pi = threadIdx.x; pi < RT32 * E; pi += 256) lg[pi] = 0.0f;
  for (int c0 = 0; c0 < d; c0 += kF32Chunk) {
    const int nc = min(kF32Chunk, d - c0);
    __syncthreads();  // the previous chunk's reads are done
    for (int q = threadIdx.x; q < (RT32 + E) * kF32Chunk; q += 256) {
      const int r = q / kF32Chunk, c = q % kF32Chunk;
      float val = 0.0f;
      if (c < nc) {
        if (r < RT32) {
          if (t0 + r < T) val = x[(size_t)(t0 + r) * d + c0 + c];
        } else {
          val = w[(size_t)(r - RT32) * d + c0 + c];
        }
      }
      (r < RT32 ? xs + r * kF32Row : ws + (r - RT32) * kF32Row)[c] = val;
    }
    __syncthreads();
    for (int pi = threadIdx.x; pi < RT32 * E; pi += 256) {
      const int tl = pi / E, e = pi % E;
      const float* xr = xs + tl * kF32Row;
      const float* wr = ws + e * kF32Row;
      float s = lg[pi];
      for (int i = 0; i < nc; ++i) s = fmaf(xr[i], wr[i], s);
      lg[pi] = s;
    }
  }
  __syncthreads();
  for (int pi = threadIdx.x; pi < RT32 * E; pi += 256)
    if (t0 + pi / E < T) part[(size_t)t0 * E + pi] = lg[pi];
}

// Logits only: the partials summed in split order (+ bias), as the
// selection sums them, four logits per thread when E % 4 == 0.
__global__ __launch_bounds__(256) void router_sum(const float* __restrict__ part, int split,
                                                  const float* __restrict__ gbias, int T, int E,
                                                  float* __restrict__ logits_out) {
  const size_t plane = (size_t)T * E;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= plane) return;
  if ((E & 3) == 0) {
    f32x4 s = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int p = 0; p < split; ++p) s += *(const f32x4*)(part + (size_t)p * plane + i);
    if (gbias) {
      const int e = (int)(i % (size_t)E);
      s += f32x4{gbias[e], gbias[e + 1], gbias[e + 2], gbias[e + 3]};
    }
    *(f32x4*)(logits_out + i) = s;
  } else {
    for (size_t j = i; j < i + 4 && j < plane; ++j) {
      float s = 0.0f;
      for (int p = 0; p < split; ++p) s += part[(size_t)p * plane + j];
      if (gbias) s += gbias[j % (size_t)E];
      logits_out[j] = s;
    }
  }
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

// Lanes per token for E experts: the power of two S with S * kSelectPerLane
// >= E (so 64 / S tokens per wave, 4 waves per block).
inline int select_lanes(int E) {
  int s = 1;
  while (s * kSelectPerLane < E) s <<= 1;
  return s;
}
inline int select_tokens(int E) { return 4 * (64 / select_lanes(E)); }

template <int S>
bool launch_select_k(int k, int nb, hipStream_t s, const float* part, int split, const float* gbias,
                     int T, int E, int renorm, float* logits_out, int32_t* idx, float* gate,
                     float* probpart) {
#define MOE_SEL(KK)                                                                            \
  hipLaunchKernelGGL((router_select<S, KK>), dim3(nb), dim3(256), 0, s, part, split, gbias, T, E, \
                     k, renorm, logits_out, idx, gate, probpart)
  if (k == 1) MOE_SEL(1);
  else if (k == 2) MOE_SEL(2);
  else if (k <= 4) MOE_SEL(4);
  else if (k <= 8) MOE_SEL(8);
  else if (k <= 16) MOE_SEL(16);
  else return false;
#undef MOE_SEL
  return true;
}

bool launch_select(int k, hipStream_t s, const float* part, int split, const float* gbias, int T,
                   int E, int renorm, float* logits_out, int32_t* idx, float* gate,
                   float* probpart) {
  const int nb = ceil_div(T, select_tokens(E));
  switch (select_lanes(E)) {
#define MOE_S(S)                                                                             \
  case S:                                                                                    \
    return launch_select_k<S>(k, nb, s, part, split, gbias, T, E, renorm, logits_out, idx, \
                              gate, probpart);
    MOE_S(1)
    MOE_S(2)
    MOE_S(4)
    MOE_S(8)
    MOE_S(16)
    MOE_S(32)
    MOE_S(64)
#undef MOE_S
    default:
      return false;
  }
}

template <int TM, int TN>
bool launch_wide(const RouterPlan& pl, const void* x, const void* w, int T, int d, int E,
                 float* part, hipStream_t s) {
  constexpr int NWN = (TN % 2 == 0) ? kWideNWN : 2;
  const size_t lds = WideCfg<TM, TN, NWN>::LDS;
  if (lds > 65536 &&
      hipFuncSetAttribute((const void*)router_logits_wide<TM, TN, NWN>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return false;
  hipLaunchKernelGGL((router_logits_wide<TM, TN, NWN>), dim3(pl.ntt * pl.split), dim3(128 * NWN), lds, s,
                     (const uint16_t*)x, (const uint16_t*)w, T, d, E, d / RK2, pl.split, part);
  return true;
}

bool dispatch_logits(const RouterPlan& pl, const void* x, const void* w, int T, int d, int E,
                     float* part, hipStream_t s) {
  const int mtw = pl.tt / 64, nte = pl.ep / 16;
  if (d % RK2 == 0 && pl.split <= d / RK2) {
#define MOE_WIDE(A, B)                                                                 \
  if (mtw == A && nte == 4 * B) return launch_wide<A, B>(pl, x, w, T, d, E, part, s);
    MOE_WIDE(2, 1)
    MOE_WIDE(1, 2)
    MOE_WIDE(1, 3)
    MOE_WIDE(2, 4)
    MOE_WIDE(1, 5)
    MOE_WIDE(1, 6)
    MOE_WIDE(1, 7)
    MOE_WIDE(1, 8)
#undef MOE_WIDE
  }
#define MOE_CASE(A, B)                               \
  if (mtw == A && nte == B) return launch_logits<A, B>(pl, x, w, T, d, E, part, s);
  MOE_CASE(2, 4)
  MOE_CASE(1, 8)
  MOE_CASE(1, 12)
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
  // logits only: no selection, gates or probability sums asked for
  const bool only_logits = !topk_idx && !topk_gate && !prob_sum;
  if (!x || !w_gate) return MOE_ERR_INVALID;
  if (only_logits ? !logits_out : (!topk_idx || !topk_gate)) return MOE_ERR_INVALID;
  if (!ws || ws_bytes < router_ws(T, d, E)) return MOE_ERR_WORKSPACE;
  float* logit_part = (float*)ws;
  float* probpart = (float*)((unsigned char*)ws + router_partial_bytes(T, d, E));
  if (dtype == MOE_BF16) {
    const RouterPlan pl = router_plan(T, d, E);
    if (!dispatch_logits(pl, x, w_gate, T, d, E, logit_part, s)) return MOE_ERR_LAUNCH;
    if (only_logits) {
      hipLaunchKernelGGL(router_sum, dim3((unsigned)ceil_div((long)T * E, 1024)), dim3(256), 0, s,
                         logit_part, pl.split, gate_bias, T, E, logits_out);
      return launch_status();
    }
    if (!launch_select(k, s, logit_part, pl.split, gate_bias, T, E, renorm, logits_out, topk_idx,
                       topk_gate, probpart))
      return MOE_ERR_LAUNCH;
  } else {
    const size_t lds = ((size_t)RT32 * E + (size_t)(RT32 + E) * kF32Row) * sizeof(float);
    if (lds > 65536 &&
        hipFuncSetAttribute((const void*)router_logits_f32,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return MOE_ERR_LAUNCH;
    hipLaunchKernelGGL(router_logits_f32, dim3(ceil_div(T, RT32)), dim3(256), lds, s,
                       (const float*)x, (const float*)w_gate, T, d, E, logit_part);
    if (only_logits) {
      hipLaunchKernelGGL(router_sum, dim3((unsigned)ceil_div((long)T * E, 1024)), dim3(256), 0, s,
                         logit_part, 1, gate_bias, T, E, logits_out);
      return launch_status();
    }
    if (!launch_select(k, s, logit_part, 1, gate_bias, T, E, renorm, logits_out, topk_idx,
                       topk_gate, probpart))
      return MOE_ERR_LAUNCH;
  }
  const int nb = ceil_div(T, select_tokens(E));
  if (prob_sum)
    hipLaunchKernelGGL(router_reduce, dim3(E), dim3(256), 0, s, probpart, nb, E, prob_sum);
  return launch_status();
}
