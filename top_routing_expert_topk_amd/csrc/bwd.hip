// Backward of the router, combine and gather steps of one MoE layer: the
// gradients of L = <dout, out> + daux * aux_loss through
//   out[t] = (residual ? x[t] : 0) + sum_j g[t,j] y[dest[t,j]]
//     (output equation of page "MoE混合专家模型路由机制原理与稀疏激活实现",
//      section "门控路由原理", slot-by-slot as its MoELayer accumulates);
//   g = softmax over the top-k logits (renorm) or p[t, S_j] (no renorm),
//     p = softmax of the logits over all experts (gate equation, TopKRouter);
//   aux_loss = E * sum_e (sum_t p[t,e] / T) (counts_e / T)
//     (load_balancing_loss of the same page; the counts carry no gradient);
//   logits = x W_g^T (+ b_g).
// Selection, counts and capacity drops are piecewise constant: gradients
// flow through the gate values, the probabilities and the products only.
//
// Kernels:
//   combine_bwd     per token: dY[row] = g * dout[t] for each kept slot and
//                   dg[t,j] = <dout[t], y[row]> (fp32, fixed-order reduction)
//   router_bwd      one wave per token: dlogits from dg (renormalised top-k
//                   softmax or full-softmax backward) plus the aux term
//   gather_bwd_mfma dx[t] = sum_e dlogits[t,e] W_g[e] (on the matrix cores,
//                   dlogits split into bf16 hi + lo) + dout[t] (residual)
//                   + sum_j dXp[dest[t,j]], 64 tokens x 128 columns per
//                   block, kept slots listed in LDS (bf16, d % 128 == 0)
//   gather_bwd      the same sum in fp32 FMA, 16 tokens per block (fp32
//                   layers and other widths)
//   wgate_mfma      dW_g partial sums over token ranges on the matrix cores
//                   (128 x 128 tiles, both operands K-major)
//   wgate_partial   the same in fp32 FMA (64 x 64 tiles, up to 64 ranges so
//                   that small E still fills the chip)
//   wgate_reduce    partials summed in range order; db_g over all tokens
#include <type_traits>

#include "moe_internal.h"
#include "ring_gemm.h"

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  const u32x4 r = *(const u32x4*)p;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = bf16lo(r[q]);
    v[2 * q + 1] = bf16hi(r[q]);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = a[q];
    v[4 + q] = b[q];
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float* v) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
  *(u32x4*)p = o;
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
template <typename T>
__device__ __forceinline__ float ld1(const T* p) {
  if constexpr (std::is_same<T, uint16_t>::value) return bf16_to_f32(*p);
  else return *p;
}
template <typename T>
__device__ __forceinline__ void st1(T* p, float v) {
  if constexpr (std::is_same<T, uint16_t>::value) *p = (uint16_t)f32_to_bf16(v);
  else *p = v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sum of one float per thread over a 256-thread block, same order every run;
// every thread gets the result.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// ------------------------------------------------------------- combine ---
// One block per token. The block first lists the token's kept slots in
// slot order (a ballot per wave, 256 slots at a time) and writes dgate = 0
// for the dropped ones, so a layer with many slots per token (Expert Choice:
// one per expert, most of them empty) pays one coalesced read of its dest
// row instead of a dependent read per slot. vec: d % 8 == 0 (8 elements per
// thread per pass). y holds the forward's expert outputs: fp32 rows for an
// fp32 layer, the grouped FFN's block fixed point for a bf16 one (T =
// uint16_t, d % 8 == 0); dout and dy are the layer's dtype T.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd(const void* __restrict__ y,
                                                   const int32_t* __restrict__ dest,
                                                   const float* __restrict__ gate, int k, int d,
                                                   const T* __restrict__ dout, T* __restrict__ dy,
                                                   float* __restrict__ dgate, bool vec) {
  __shared__ float red[4];
  __shared__ int kept[kMaxE];  // slot indices, then their rows
  __shared__ int krow[kMaxE];
  __shared__ int wcnt[4];
  __shared__ int nkept;
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* go = dout + (size_t)t * d;
  constexpr bool kYQ = std::is_same<T, uint16_t>::value;
  const size_t yrb = kYQ ? yq_row_bytes(d) : (size_t)d * sizeof(float);
  auto yload8 = [&](long r, int c, float* v) __attribute__((always_inline)) {
    if constexpr (kYQ) yq_load8((const unsigned char*)y, yrb, d, r, c, v);
    else load8<float>((const float*)y + (size_t)r * d + c, v);
  };
  int base = 0;
  for (int j0 = 0; j0 < k; j0 += 256) {
    const int j = j0 + tid;
    const int r = j < k ? dest[(size_t)t * k + j] : -1;
    if (j < k && r < 0) dgate[(size_t)t * k + j] = 0.0f;  // dropped: no output, no gradient
    const uint64_t m = __ballot(r >= 0);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w2 = 0; w2 < wave; ++w2) off += wcnt[w2];
    if (r >= 0) {
      const int pos = off + __popcll(m & ((1ull << lane) - 1));
      kept[pos] = j;
      krow[pos] = r;
    }
    base += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();
  }
  if (tid == 0) nkept = base;
  __syncthreads();
  const int nk = nkept;
  int q = 0;
  if (vec) {
    // eight kept slots per pass over the row: dout is read once per pass and
    // their eight y rows are in flight together; each dot product is summed
    // per thread in column order and reduced as block_sum256 does
    __shared__ float red8[4][8];
    for (; q + 8 <= nk; q += 8) {
      float dot[8], g[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        dot[u] = 0.0f;
        g[u] = gate[(size_t)t * k + kept[q + u]];
      }
      for (int c = tid * 8; c < d; c += 256 * 8) {
        float a[8], b[8][8];
        load8<T>(go + c, a);
#pragma unroll
        for (int u = 0; u < 8; ++u) yload8(krow[q + u], c, b[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float o[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            dot[u] = fmaf(a[v], b[u][v], dot[u]);
            o[v] = g[u] * a[v];
          }
          store8<T>(dy + (size_t)krow[q + u] * d + c, o);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) dot[u] = wave_sum(dot[u]);
      __syncthreads();
      if (lane == 0)
#pragma unroll
        for (int u = 0; u < 8; ++u) red8[wave][u] = dot[u];
      __syncthreads();
      if (tid < 8)
        dgate[(size_t)t * k + kept[q + tid]] =
            (red8[0][tid] + red8[1][tid]) + (red8[2][tid] + red8[3][tid]);
    }
  }
  for (; q < nk; ++q) {  // one slot per pass
    const int j = kept[q], r = krow[q];
    const float g = gate[(size_t)t * k + j];
    T* dr = dy + (size_t)r * d;
    float dot = 0.0f;
    if (vec) {
      for (int c = tid * 8; c < d; c += 256 * 8) {
        float a[8], b[8], o[8];
        load8<T>(go + c, a);
        yload8(r, c, b);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          dot = fmaf(a[u], b[u], dot);
          o[u] = g * a[u];
        }
        store8<T>(dr + c, o);
      }
    } else {
      for (int c = tid; c < d; c += 256) {
        const float a = ld1<T>(go + c);
        if constexpr (!kYQ) dot = fmaf(a, ((const float*)y)[(size_t)r * d + c], dot);
        st1<T>(dr + c, g * a);
      }
    }
    dot = block_sum256(dot, red);
    if (tid == 0) dgate[(size_t)t * k + j] = dot;
  }
}

// -------------------------------------------------------------- router ---
constexpr int kRbTokens = 4;  // tokens per block, one wave each
constexpr int kPer = kMaxE / 64;

__global__ __launch_bounds__(256) void router_bwd(const float* __restrict__ logits,
                                                  const int32_t* __restrict__ idx,
                                                  const float* __restrict__ gate,
                                                  const float* __restrict__ dgate,
                                                  const int32_t* __restrict__ counts, int T, int E,
                                                  int k, int renorm, float aux_scale,
                                                  float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRbTokens + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  float p[kPer], dl[kPer], dp[kPer];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    p[i] = e < E ? l[e] : -INFINITY;
    m = fmaxf(m, p[i]);
    dl[i] = 0.0f;
    dp[i] = 0.0f;
  }
  m = wave_max(m);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    p[i] = lane + 64 * i < E ? expf(p[i] - m) : 0.0f;
    s += p[i];
  }
  s = wave_sum(s);
  const float inv = 1.0f / s;
#pragma unroll
  for (int i = 0; i < kPer; ++i) p[i] *= inv;

  const int32_t* it = idx + (size_t)t * k;
  const float* gt = gate + (size_t)t * k;
  const float* dgt = dgate + (size_t)t * k;
  if (renorm) {
    // dl[S_j] = g_j (dg_j - sum_i g_i dg_i)
    float inner = 0.0f;
    for (int j = 0; j < k; ++j) inner = fmaf(gt[j], dgt[j], inner);
    for (int j = 0; j < k; ++j) {
      const int e = idx ? it[j] : j;
      const float v = gt[j] * (dgt[j] - inner);
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (e == lane + 64 * i) dl[i] += v;
    }
  } else if (idx) {
    // g_j = p[S_j]: dp[S_j] += dg_j, then the softmax backward
    for (int j = 0; j < k; ++j) {
      const int e = it[j];
      const float v = dgt[j];
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (e == lane + 64 * i) dp[i] += v;
    }
  } else {
    // no index table: slot j is expert j (Expert Choice, k == E)
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (lane + 64 * i < E) dp[i] += dgt[lane + 64 * i];
  }
  // aux: d/dp[t,e] = daux E counts_e / T^2
  if (aux_scale != 0.0f) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      if (e < E) dp[i] += aux_scale * (float)counts[e];
    }
  }
  float pdp = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) pdp = fmaf(p[i], dp[i], pdp);
  pdp = wave_sum(pdp);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    if (e < E) dlogits[(size_t)t * E + e] = dl[i] + p[i] * (dp[i] - pdp);
  }
}

// -------------------------------------------------------------- gather ---
constexpr int kGbTokens = 16;  // tokens per block
constexpr int kGbCols = 256 * 8;

// Grid (ceil(T / 16), ceil(d / 2048)); d % 8 == 0. Each thread owns 8
// columns of the block's 16 tokens.
template <typename T>
__global__ __launch_bounds__(256) void gather_bwd(const T* __restrict__ dxp,
                                                  const int32_t* __restrict__ dest, int Tn, int k,
                                                  int d, const T* __restrict__ dres,
                                                  const float* __restrict__ dlogits,
                                                  const T* __restrict__ wg, int E,
                                                  T* __restrict__ dx) {
  __shared__ float sdl[kGbTokens][kMaxE];
  const int t0 = blockIdx.x * kGbTokens;
  const int nt = min(kGbTokens, Tn - t0);
  if (dlogits) {
    for (int i = threadIdx.x; i < nt * E; i += 256) sdl[i / E][i % E] = dlogits[(size_t)t0 * E + i];
    __syncthreads();
  }
  const int c = blockIdx.y * kGbCols + threadIdx.x * 8;
  if (c >= d) return;
  float acc[kGbTokens][8];
#pragma unroll
  for (int tt = 0; tt < kGbTokens; ++tt)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[tt][q] = 0.0f;
  // router term first, experts in ascending order
  if (dlogits) {
    for (int e = 0; e < E; ++e) {
      float w[8];
      load8<T>(wg + (size_t)e * d + c, w);
#pragma unroll
      for (int tt = 0; tt < kGbTokens; ++tt) {
        const float a = sdl[tt][e];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[tt][q] = fmaf(a, w[q], acc[tt][q]);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < kGbTokens; ++tt) {
    if (tt < nt) {
      const int t = t0 + tt;
      float v[8];
      if (dres) {
        load8<T>(dres + (size_t)t * d + c, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[tt][q] += v[q];
      }
      for (int j = 0; j < k; ++j) {
        const int r = dest[(size_t)t * k + j];
        if (r >= 0) {
          load8<T>(dxp + (size_t)r * d + c, v);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[tt][q] += v[q];
        }
      }
      store8<T>(dx + (size_t)t * d + c, acc[tt]);
    }
  }
}

// bf16 layers with d % 128 == 0: the router term on the MFMA units. Grid
// (ceil(T / 64), d / 128), four waves; a block owns 64 tokens x 128 columns.
// 1. The kept slots of each token are listed in LDS in slot order (a ballot
//    per 64 slots, four tokens' dest rows in flight per wave); past
//    kGmSlots a token resumes reading its dest row in the gather.
// 2. R = dlogits . W_g over 64-expert chunks: dlogits (fp32) is split into
//    bf16 hi + lo (hi = bf16(v), lo = bf16(v - hi), so hi + lo keeps 16
//    significant bits) and both halves multiply the bf16 W_g on
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulation. Operands are staged in
//    LDS per chunk: [64 tokens][64 experts] hi and lo (128-byte rows,
//    swizzled as the ring's) and W_g's [64 experts][128 columns] K-major
//    block read by transpose loads; experts past E are zero on the dlogits
//    side (W_g rows clamped to E - 1). Wave w owns columns 32 w .. +31 of
//    all 64 tokens (two 32 x 32 tiles; lane = column, registers = tokens).
// 3. R goes through LDS (fp32, rows of 136 floats: the two half-waves, four
//    tokens apart, land on disjoint banks), and each thread then sums 8
//    columns of a token in the order of gather_bwd: router term, residual,
//    the kept slots in slot order.
constexpr int kGmTok = 64, kGmCols = 128, kGmSlots = 16, kGmStr = 136;
struct GmOps {
  uint16_t wgs[64 * 128];      // W_g chunk, K-major transpose layout
  uint16_t dls[2][64 * 64];    // dlogits chunk, hi and lo
};
union GmLds {
  GmOps ops;
  float racc[kGmTok * kGmStr];
};

__global__ __launch_bounds__(256) void gather_bwd_mfma(const uint16_t* __restrict__ dxp,
                                                       const int32_t* __restrict__ dest, int Tn,
                                                       int k, int d,
                                                       const uint16_t* __restrict__ dres,
                                                       const float* __restrict__ dlogits,
                                                       const uint16_t* __restrict__ wg, int E,
                                                       uint16_t* __restrict__ dx) {
  __shared__ __align__(16) GmLds sm;
  __shared__ int list[kGmTok][kGmSlots];
  __shared__ int nlist[kGmTok], resume[kGmTok];
  const int t0 = blockIdx.x * kGmTok, c0 = blockIdx.y * kGmCols;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // 1. kept slots: wave w lists tokens 16 w .. 16 w + 15, four at a time
  for (int tq = 0; tq < 16; tq += 4) {
    int cnt[4] = {0, 0, 0, 0}, res[4] = {k, k, k, k};
    for (int j0 = 0; j0 < k; j0 += 64) {
      int r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + wave * 16 + tq + u, j = j0 + lane;
        r[u] = (t < Tn && j < k) ? dest[(size_t)t * k + j] : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t m = __ballot(r[u] >= 0);
        const int pos = cnt[u] + __popcll(m & ((1ull << lane) - 1));
        const int tt = wave * 16 + tq + u;
        if (r[u] >= 0 && pos < kGmSlots) list[tt][pos] = r[u];
        if (r[u] >= 0 && pos == kGmSlots) res[u] = j0 + lane;  // the first slot not listed
        cnt[u] += __popcll(m);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tt = wave * 16 + tq + u;
      // the lane that saw the first unlisted slot holds it; others hold k
      int rs = res[u];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) rs = min(rs, __shfl_xor(rs, o));
      if (lane == 0) {
        nlist[tt] = min(cnt[u], kGmSlots);
        resume[tt] = rs;
      }
    }
  }

  // 2. router term; a chunk's global loads are issued a chunk ahead, into
  // registers, so their latency hides behind the previous chunk's MFMAs
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  if (dlogits) {
    u32x4 wr[4];
    float dv[16];
    auto load_chunk = [&](int e0) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = tid + 256 * i, r = q >> 4, c = q & 15;
        wr[i] = *(const u32x4*)(wg + (size_t)min(e0 + r, E - 1) * d + c0 + c * 8);
      }
      const int r = tid >> 2, qd = tid & 3, t = t0 + r;
      const int eb = e0 + qd * 16;
      if (t < Tn && eb + 16 <= E && (E & 3) == 0) {
#pragma unroll
        for (int u4 = 0; u4 < 4; ++u4) {
          const f32x4 a = *(const f32x4*)(dlogits + (size_t)t * E + eb + 4 * u4);
#pragma unroll
          for (int u = 0; u < 4; ++u) dv[4 * u4 + u] = a[u];
        }
      } else {
#pragma unroll
        for (int u = 0; u < 16; ++u)
          dv[u] = (t < Tn && eb + u < E) ? dlogits[(size_t)t * E + eb + u] : 0.0f;
      }
    };
    load_chunk(0);
    for (int e0 = 0; e0 < E; e0 += 64) {
      __syncthreads();  // the previous chunk's reads are done
      // W_g rows e0 .. e0 + 63 (clamped), columns c0 .. c0 + 127: 16-byte
      // chunk c of row r at c ^ 4 (r % 4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = tid + 256 * i, r = q >> 4, c = q & 15;
        *(u32x4*)(sm.ops.wgs + r * 128 + ((c ^ (4 * (r & 3))) << 3)) = wr[i];
      }
      // dlogits rows t0 .. t0 + 63, experts e0 .. e0 + 63: thread (row tid / 4,
      // experts 16 (tid % 4) .. +15) -> hi and lo chunks 2 (tid % 4), +1
      {
        const int r = tid >> 2, qd = tid & 3;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          u32x4 hi, lo;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float a = dv[h2 * 8 + 2 * u], b = dv[h2 * 8 + 2 * u + 1];
            const uint32_t ph = pack_bf16x2(a, b);
            hi[u] = ph;
            lo[u] = pack_bf16x2(a - bf16lo(ph), b - bf16hi(ph));
          }
          const int ck = swz128(r, 2 * qd + h2);
          *(u32x4*)(sm.ops.dls[0] + r * 64 + ck * 8) = hi;
          *(u32x4*)(sm.ops.dls[1] + r * 64 + ck * 8) = lo;
        }
      }
      __syncthreads();
      if (e0 + 64 < E) load_chunk(e0 + 64);
      const int nsub = min(4, (E - e0 + 15) / 16);
      for (int sub = 0; sub < nsub; ++sub) {
        const bf16x8 b = tr_frag(sm.ops.wgs, sub, wave, lane);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const int r = mi * 32 + (lane & 31);
          const int ck = swz128(r, 2 * sub + (lane >> 5));
          const bf16x8 ah = *(const bf16x8*)(sm.ops.dls[0] + r * 64 + ck * 8);
          const bf16x8 al = *(const bf16x8*)(sm.ops.dls[1] + r * 64 + ck * 8);
          acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b, acc[mi], 0, 0, 0);
          acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b, acc[mi], 0, 0, 0);
        }
      }
    }
  }
  // 3. router term through LDS, then the sums
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tt = mi * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v & 3);
      sm.racc[tt * kGmStr + wave * 32 + (lane & 31)] = acc[mi][v];
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = (tid >> 4) + 16 * i, cc = tid & 15, t = t0 + tt;
    if (t >= Tn) continue;
    const int c = c0 + cc * 8;
    float a[8], v[8];
    const f32x4 lo = *(const f32x4*)(sm.racc + tt * kGmStr + cc * 8);
    const f32x4 hi = *(const f32x4*)(sm.racc + tt * kGmStr + cc * 8 + 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = lo[u];
      a[4 + u] = hi[u];
    }
    if (dres) {
      load8<uint16_t>(dres + (size_t)t * d + c, v);
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] += v[u];
    }
    const int n = nlist[tt];
    int j = 0;
    for (; j + 8 <= n; j += 8) {  // eight rows in flight, added in slot order
      u32x4 rv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) rv[q] = *(const u32x4*)(dxp + (size_t)list[tt][j + q] * d + c);
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[2 * u] += bf16lo(rv[q][u]);
          a[2 * u + 1] += bf16hi(rv[q][u]);
        }
    }
    for (; j + 4 <= n; j += 4) {  // four rows in flight, added in slot order
      u32x4 rv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) rv[q] = *(const u32x4*)(dxp + (size_t)list[tt][j + q] * d + c);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[2 * u] += bf16lo(rv[q][u]);
          a[2 * u + 1] += bf16hi(rv[q][u]);
        }
    }
    for (; j < n; ++j) {
      load8<uint16_t>(dxp + (size_t)list[tt][j] * d + c, v);
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] += v[u];
    }
    for (int j = resume[tt]; j < k; ++j) {  // slots past the listed ones (rare)
      const int r = dest[(size_t)t * k + j];
      if (r >= 0) {
        load8<uint16_t>(dxp + (size_t)r * d + c, v);
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] += v[u];
      }
    }
    store8<uint16_t>(dx + (size_t)t * d + c, a);
  }
}

// Any d: one thread per (token, column), same sum order as gather_bwd.
template <typename T>
__global__ __launch_bounds__(256) void gather_bwd_scalar(const T* __restrict__ dxp,
                                                         const int32_t* __restrict__ dest, int Tn,
                                                         int k, int d, const T* __restrict__ dres,
                                                         const float* __restrict__ dlogits,
                                                         const T* __restrict__ wg, int E,
                                                         T* __restrict__ dx) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)Tn * d) return;
  const int t = (int)(i / d), c = (int)(i % d);
  float a = 0.0f;
  if (dlogits)
    for (int e = 0; e < E; ++e) a = fmaf(dlogits[(size_t)t * E + e], ld1<T>(wg + (size_t)e * d + c), a);
  if (dres) a += ld1<T>(dres + i);
  for (int j = 0; j < k; ++j) {
    const int r = dest[(size_t)t * k + j];
    if (r >= 0) a += ld1<T>(dxp + (size_t)r * d + c);
  }
  st1<T>(dx + i, a);
}

// ------------------------------------------------------- router weights ---
constexpr int kWgTile = 64;
constexpr int kWgTok = 16;

// part[s][e][c] = sum over tokens t of range s (in order) of dl[t][e] x[t][c].
// Grid (ceil(E/64), ceil(d/64), S); thread (ty, tx) owns experts 4ty..4ty+3
// and columns 4tx..4tx+3 of the tile.
template <typename T>
__global__ __launch_bounds__(256) void wgate_partial(const T* __restrict__ x,
                                                     const float* __restrict__ dl, int Tn, int d,
                                                     int E, int S, float* __restrict__ part) {
  __shared__ float sx[kWgTok][kWgTile + 4];
  __shared__ float se[kWgTok][kWgTile + 4];
  const int e0 = blockIdx.x * kWgTile, c0 = blockIdx.y * kWgTile, s = blockIdx.z;
  const int tb = (int)((long)s * Tn / S), te = (int)((long)(s + 1) * Tn / S);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int t0 = tb; t0 < te; t0 += kWgTok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, tt = q / kWgTile, col = q % kWgTile, t = t0 + tt;
      const bool live = t < te;
      sx[tt][col] = (live && c0 + col < d) ? ld1<T>(x + (size_t)t * d + c0 + col) : 0.0f;
      se[tt][col] = (live && e0 + col < E) ? dl[(size_t)t * E + e0 + col] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < kWgTok; ++tt) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = se[tt][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sx[tt][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + ty * 4 + i;
    if (e >= E) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + tx * 4 + j;
      if (c < d) part[((size_t)s * E + e) * d + c] = acc[i][j];
    }
  }
}

// dW_g[e][c] = sum_s part[s][e][c] (s ascending); grid (ceil(E*d / 256)).
// bf16 layers with d % 128 == 0: the same partial sums on the MFMA units.
// Grid ceil(E / 128) * (d / 128) * S; four waves, each 64 experts x 64 columns
// of the block's 128 x 128 tile (2 x 2 32x32 MFMA tiles; lane = column,
// registers = experts). Both operands contract over tokens, their leading
// index, so each 64-token chunk is staged K-major ([64 tokens][128
// features], 16-byte chunk c of row r at c ^ 4 (r % 4)) and read by
// transpose loads: x as bf16, dlogits split into bf16 hi + lo (hi =
// bf16(v), lo = bf16(v - hi)), both multiplied with fp32 accumulation.
// Tokens past the range and experts past E are zero on the dlogits side (x
// rows clamped to the range's last).
__global__ __launch_bounds__(256) void wgate_mfma(const uint16_t* __restrict__ x,
                                                  const float* __restrict__ dl, int Tn, int d,
                                                  int E, int S, float* __restrict__ part) {
  __shared__ __align__(16) uint16_t sdl[2][64 * 128];
  __shared__ __align__(16) uint16_t sx[64 * 128];
  // Block -> (token range s, column tile, expert tile). With S a multiple of
  // 8, range s runs on XCD s % 8 (blocks are dealt to the 8 XCDs in turn),
  // all its tiles in a row with the expert tiles of a column adjacent, so
  // its dlogits rows and x columns are fetched from HBM about once and
  // re-read from that XCD's L2.
  const int ne = (E + 127) / 128, per = ne * (d / 128);
  int s, rem;
  if ((S & 7) == 0) {
    const int j = blockIdx.x >> 3;
    s = (blockIdx.x & 7) + 8 * (j / per);
    rem = j % per;
  } else {
    s = blockIdx.x / per;
    rem = blockIdx.x % per;
  }
  const int e0 = (rem % ne) * 128, c0 = (rem / ne) * 128;
  const int tb = (int)((long)s * Tn / S), te = (int)((long)(s + 1) * Tn / S);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};
  // A chunk's global loads are issued a chunk ahead, into registers, so
  // their latency hides behind the previous chunk's MFMAs.
  u32x4 xr[4];
  float dv[4][8];
  auto load_chunk = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, r = q >> 4, c = q & 15;
      xr[i] = *(const u32x4*)(x + (size_t)min(t + r, te - 1) * d + c0 + c * 8);
    }
    const int r = tid >> 2, qd = tid & 3, tr = t + r;
    const bool vec = tr < te && e0 + 128 <= E && (E & 3) == 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int eb = e0 + qd * 32 + q * 8;
      if (vec) {
        const f32x4 a = *(const f32x4*)(dl + (size_t)tr * E + eb);
        const f32x4 b = *(const f32x4*)(dl + (size_t)tr * E + eb + 4);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          dv[q][u] = a[u];
          dv[q][4 + u] = b[u];
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          dv[q][u] = (tr < te && eb + u < E) ? dl[(size_t)tr * E + eb + u] : 0.0f;
      }
    }
  };
  if (tb < te) load_chunk(tb);
  for (int t = tb; t < te; t += 64) {
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, r = q >> 4, c = q & 15;
      *(u32x4*)(sx + r * 128 + ((c ^ (4 * (r & 3))) << 3)) = xr[i];
    }
    {
      const int r = tid >> 2, qd = tid & 3;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 hi, lo;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t ph = pack_bf16x2(dv[q][2 * u], dv[q][2 * u + 1]);
          hi[u] = ph;
          lo[u] = pack_bf16x2(dv[q][2 * u] - bf16lo(ph), dv[q][2 * u + 1] - bf16hi(ph));
        }
        const int pos = r * 128 + (((qd * 4 + q) ^ (4 * (r & 3))) << 3);
        *(u32x4*)(sdl[0] + pos) = hi;
        *(u32x4*)(sdl[1] + pos) = lo;
      }
    }
    __syncthreads();
    if (t + 64 < te) load_chunk(t + 64);
    const int nsub = min(4, (te - t + 15) / 16);
    for (int sub = 0; sub < nsub; ++sub) {
      bf16x8 b[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) b[ni] = tr_frag(sx, sub, wn * 2 + ni, lane);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const bf16x8 ah = tr_frag(sdl[0], sub, wm * 2 + mi, lane);
        const bf16x8 al = tr_frag(sdl[1], sub, wm * 2 + mi, lane);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b[ni], acc[mi][ni], 0, 0, 0);
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b[ni], acc[mi][ni], 0, 0, 0);
        }
      }
    }
  }
  float* ps = part + (size_t)s * E * d;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int e = e0 + wm * 64 + mi * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v & 3);
      if (e < E) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          ps[(size_t)e * d + c0 + wn * 64 + ni * 32 + (lane & 31)] = acc[mi][ni][v];
      }
    }
}

// Token ranges of the MFMA form: about 1024 blocks, at most 64 ranges and
// at least 64 tokens per range (never more ranges than router_bwd_splits,
// whose workspace holds the partials); from 8 on a multiple of 8, one group
// of ranges per XCD.
inline int wgate_mfma_splits(int T, int d, int E) {
  const int tiles = ceil_div(E, 128) * (d / 128);
  int s = ceil_div(1024, tiles);
  if (s > 64) s = 64;
  if (s > T / 64) s = T / 64;
  const int cap = router_bwd_splits(T, d, E);
  if (s > cap) s = cap;
  if (s >= 8) s = s / 8 * 8;
  return s < 1 ? 1 : s;
}

template <typename T>
__global__ __launch_bounds__(256) void wgate_reduce(const float* __restrict__ part, int E, int d,
                                                    int S, T* __restrict__ dwg) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)E * d) return;
  float a = 0.0f;
  for (int s = 0; s < S; ++s) a += part[(size_t)s * E * d + i];
  st1<T>(dwg + i, a);
}

// db_g[e] = sum_t dl[t][e]: one block per expert, fixed-order tree.
__global__ __launch_bounds__(256) void gate_bias_grad(const float* __restrict__ dl, int Tn, int E,
                                                      float* __restrict__ dbg) {
  __shared__ float red[4];
  const int e = blockIdx.x;
  float a = 0.0f;
  for (int t = threadIdx.x; t < Tn; t += 256) a += dl[(size_t)t * E + e];
  a = block_sum256(a, red);
  if (threadIdx.x == 0) dbg[e] = a;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_combine_backward(const void* y_perm, int dtype, const int32_t* dest_row,
                                    const float* topk_gate, int T, int k, int d, const void* dout,
                                    void* dy_perm, float* dgate, moe_stream_t stream) {
  if (T < 0 || k < 1 || d < 1) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (k > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_BF16 && (d % 8) != 0) return MOE_ERR_UNSUPPORTED;  // whole blocks of 8
  if (T == 0) return MOE_OK;
  if (!y_perm || !dest_row || !topk_gate || !dout || !dy_perm || !dgate) return MOE_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  MOE_DEBUG_CHECK(s, nullptr, 1, nullptr, dest_row, T, k);
  const bool vec = (d % 8) == 0;
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_bwd<uint16_t>, dim3(T), dim3(256), 0, s, y_perm,
                       dest_row, topk_gate, k, d, (const uint16_t*)dout, (uint16_t*)dy_perm, dgate,
                       vec);
  else
    hipLaunchKernelGGL(combine_bwd<float>, dim3(T), dim3(256), 0, s, y_perm, dest_row,
                       topk_gate, k, d, (const float*)dout, (float*)dy_perm, dgate, vec);
  return launch_status();
}

extern "C" int moe_router_backward(const float* logits, const int32_t* topk_idx,
                                   const float* topk_gate, const float* dgate,
                                   const int32_t* counts, int T, int E, int k, int renorm,
                                   float daux, float* dlogits, moe_stream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_gate || !dgate || !dlogits) return MOE_ERR_INVALID;
  if (!topk_idx && k != E) return MOE_ERR_INVALID;
  if (daux != 0.0f && !counts) return MOE_ERR_INVALID;
  const float aux_scale = daux * (float)E / ((float)T * (float)T);
  hipLaunchKernelGGL(router_bwd, dim3(ceil_div(T, kRbTokens)), dim3(256), 0, (hipStream_t)stream,
                     logits, topk_idx, topk_gate, dgate, counts, T, E, k, renorm ? 1 : 0, aux_scale,
                     dlogits);
  return launch_status();
}

extern "C" int moe_gather_backward(const void* dx_perm, int dtype, const int32_t* dest_row, int T,
                                   int k, int d, const void* dout_residual,
                                   const float* dlogits, const void* w_gate, int E, void* dx,
                                   moe_stream_t stream) {
  if (T < 0 || k < 1 || d < 1 || E < 1) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (E > kMaxE || k > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!dx_perm || !dest_row || !dx || (dlogits && !w_gate)) return MOE_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  MOE_DEBUG_CHECK(s, nullptr, 1, nullptr, dest_row, T, k);
  if (dtype == MOE_BF16 && (d % kGmCols) == 0) {
    hipLaunchKernelGGL(gather_bwd_mfma, dim3(ceil_div(T, kGmTok), d / kGmCols), dim3(256), 0, s,
                       (const uint16_t*)dx_perm, dest_row, T, k, d,
                       (const uint16_t*)dout_residual, dlogits, (const uint16_t*)w_gate, E,
                       (uint16_t*)dx);
  } else if ((d % 8) == 0) {
    const dim3 g(ceil_div(T, kGbTokens), ceil_div(d, kGbCols));
    if (dtype == MOE_BF16)
      hipLaunchKernelGGL(gather_bwd<uint16_t>, g, dim3(256), 0, s, (const uint16_t*)dx_perm,
                         dest_row, T, k, d, (const uint16_t*)dout_residual, dlogits,
                         (const uint16_t*)w_gate, E, (uint16_t*)dx);
    else
      hipLaunchKernelGGL(gather_bwd<float>, g, dim3(256), 0, s, (const float*)dx_perm, dest_row, T,
                         k, d, (const float*)dout_residual, dlogits, (const float*)w_gate, E,
                         (float*)dx);
  } else {
    const dim3 g(ceil_div((long)T * d, 256));
    if (dtype == MOE_BF16)
      hipLaunchKernelGGL(gather_bwd_scalar<uint16_t>, g, dim3(256), 0, s, (const uint16_t*)dx_perm,
                         dest_row, T, k, d, (const uint16_t*)dout_residual, dlogits,
                         (const uint16_t*)w_gate, E, (uint16_t*)dx);
    else
      hipLaunchKernelGGL(gather_bwd_scalar<float>, g, dim3(256), 0, s, (const float*)dx_perm,
                         dest_row, T, k, d, (const float*)dout_residual, dlogits,
                         (const float*)w_gate, E, (float*)dx);
  }
  return launch_status();
}

extern "C" int moe_router_weight_backward(const void* x, int dtype, int T, int d, int E,
                                          const float* dlogits, void* dw_gate, float* dgate_bias,
                                          void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (T < 0 || d < 1 || E < 1) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (!dw_gate || (T > 0 && (!x || !dlogits))) return MOE_ERR_INVALID;
  if (!ws || ws_bytes < router_bwd_ws(T, d, E)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool mfma = dtype == MOE_BF16 && (d % 128) == 0;
  const int S = mfma ? wgate_mfma_splits(T, d, E) : router_bwd_splits(T, d, E);
  float* part = (float*)ws;
  const dim3 g(ceil_div(E, kWgTile), ceil_div(d, kWgTile), S);
  if (mfma && T > 0)
    hipLaunchKernelGGL(wgate_mfma, dim3(ceil_div(E, 128) * (d / 128) * S), dim3(256), 0, s,
                       (const uint16_t*)x, dlogits, T, d, E, S, part);
  else if (dtype == MOE_BF16)
    hipLaunchKernelGGL(wgate_partial<uint16_t>, g, dim3(256), 0, s, (const uint16_t*)x, dlogits, T,
                       d, E, S, part);
  else
    hipLaunchKernelGGL(wgate_partial<float>, g, dim3(256), 0, s, (const float*)x, dlogits, T, d, E,
                       S, part);
  const dim3 gr(ceil_div((long)E * d, 256));
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(wgate_reduce<uint16_t>, gr, dim3(256), 0, s, (const float*)part, E, d, S,
                       (uint16_t*)dw_gate);
  else
    hipLaunchKernelGGL(wgate_reduce<float>, gr, dim3(256), 0, s, (const float*)part, E, d, S,
                       (float*)dw_gate);
  if (dgate_bias)
    hipLaunchKernelGGL(gate_bias_grad, dim3(E), dim3(256), 0, s, dlogits, T, E, dgate_bias);
  return launch_status();
}
