// Combine and aux loss.
//
// Combine: out[t] = residual[t] + sum_j gate[t,j] * y_perm[dest_row[t,j]], the
// output equation y = sum_i G(x)_i E_i(x) of page "MoE混合专家模型路由机制原理与稀疏激活实现"
// (section "门控路由原理") with the MoELayer's slot-by-slot accumulation
// (section "Top-K门控路由的PyTorch实现"); dropped slots (dest_row = -1)
// contribute nothing and the token keeps its residual (capacity section).
// The "weighted scatter" is done as a per-token gather: each output element
// is owned by one lane, which sums its k terms in fp32 in ascending j, so
// the result is deterministic and needs no atomics. The expert outputs
// y_perm of a bf16 layer are in the block fixed point the grouped FFN writes
// (moe_internal.h: int16 mantissas, one exponent per 8 features of a row,
// rows of yq_row_bytes(d) bytes) and are decoded exactly to fp32 here; an
// fp32 layer's are fp32. A bf16 layer's residual is bf16. Expert Choice gives a
// token one slot per expert (k = E, dest_row -1 where the expert did not
// take it); the same sum then runs over its choosing experts in order.
//
// Aux loss: load_balancing_loss of the same page: f = mean probability per
// expert, P = assignments per token per expert (before drops), loss = E *
// sum f*P, summed in a fixed-order tree.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCombineWaves = 4;  // tokens per block, one wave each

template <typename OutT>
__device__ __forceinline__ void store8(OutT* p, const float* v);
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

// acc[0..7] += g * features c..c+7 of expert-output row r
__device__ __forceinline__ void fma8(float g, const unsigned char* __restrict__ y, size_t rb, int d,
                                     long r, int c, float* acc) {
  float v[8];
  yq_load8(y, rb, d, r, c, v);
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = fmaf(g, v[q], acc[q]);
}

// KK slots per token (k rounded up to 1, 2, 4, 8 or 16). A token's slot rows
// are wave-uniform, so their bases sit in scalar registers and every row's
// load of a column chunk is issued before the first is used (the loads carry
// no branch). A dropped slot, or one past k, reads the token's first live
// row with gate 0: it adds a zero, which changes no sum except a -0 to +0.
template <int KK, typename OutT>
__global__ __launch_bounds__(256) void combine_bf16(
    const unsigned char* __restrict__ y, const int32_t* __restrict__ dest,
    const float* __restrict__ gate, int T, int k, int d, const uint16_t* __restrict__ resid,
    OutT* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kCombineWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  const size_t rb = yq_row_bytes(d);
  int dj[KK];
  float gj[KK];
  int first = -1;
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    dj[j] = j < k ? __builtin_amdgcn_readfirstlane(dest[(size_t)t * k + j]) : -1;
    gj[j] = j < k ? __int_as_float(__builtin_amdgcn_readfirstlane(
                        __float_as_int(gate[(size_t)t * k + j])))
                  : 0.0f;
    if (first < 0 && dj[j] >= 0) first = dj[j];
  }
  const bool any = first >= 0;
  const unsigned char* rowp[KK];
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    if (dj[j] < 0) gj[j] = 0.0f;
    rowp[j] = y + (size_t)(dj[j] >= 0 ? dj[j] : (any ? first : 0)) * rb;
  }
  for (int c = lane * 8; c < d; c += 64 * 8) {
    float acc[8];
    if (resid) {
      const u32x4 r = *(const u32x4*)(resid + (size_t)t * d + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = bf16lo(r[q]);
        acc[2 * q + 1] = bf16hi(r[q]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    }
    if (any) {
      u32x4 mant[KK];
      int ex[KK];
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        mant[j] = *(const u32x4*)(rowp[j] + (uint32_t)(2 * c));
        ex[j] = (int)(signed char)rowp[j][(uint32_t)(2 * d + c / kYBlock)];
      }
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        float v[8];
        yq_decode8(mant[j], ex[j], v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(gj[j], v[q], acc[q]);
      }
    }
    store8<OutT>(out + (size_t)t * d + c, acc);
  }
}

// Any number of slots (Expert Choice gives a token one slot per expert): per
// 16-byte column chunk, the wave reads 64 slots at a time, ballots the live
// ones and adds them in ascending slot order.
template <typename OutT>
__global__ __launch_bounds__(256) void combine_bf16_many(
    const unsigned char* __restrict__ y, const int32_t* __restrict__ dest,
    const float* __restrict__ gate, int T, int k, int d, const uint16_t* __restrict__ resid,
    OutT* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t rb = yq_row_bytes(d);
  for (int c0 = 0; c0 < d; c0 += 64 * 8) {
    const int c = c0 + lane * 8;
    const bool mine = c < d;
    float acc[8];
    if (resid && mine) {
      const u32x4 r = *(const u32x4*)(resid + (size_t)t * d + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = bf16lo(r[q]);
        acc[2 * q + 1] = bf16hi(r[q]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    }
    for (int j0 = 0; j0 < k; j0 += 64) {
      const int j = j0 + lane;
      const int dj = j < k ? dest[(size_t)t * k + j] : -1;
      const float gj = j < k ? gate[(size_t)t * k + j] : 0.0f;
      uint64_t live = __ballot(dj >= 0);
      while (live) {
        const int b = __ffsll((long long)live) - 1;
        live &= live - 1;
        const int r = __builtin_amdgcn_readlane(dj, b);
        const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gj), b));
        if (mine) fma8(g, y, rb, d, r, c, acc);
      }
    }
    if (mine) store8<OutT>(out + (size_t)t * d + c, acc);
  }
}

__global__ __launch_bounds__(256) void combine_f32(
    const float* __restrict__ y, const int32_t* __restrict__ dest, const float* __restrict__ gate,
    int T, int k, int d, const float* __restrict__ resid, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  for (int c = lane; c < d; c += 64) {
    float acc = resid ? resid[(size_t)t * d + c] : 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = dest[(size_t)t * k + j];
      if (r >= 0) acc = fmaf(gate[(size_t)t * k + j], y[(size_t)r * d + c], acc);
    }
    out[(size_t)t * d + c] = acc;
  }
}

__global__ __launch_bounds__(512) void aux_kernel(const float* __restrict__ prob_sum,
                                                  const int32_t* __restrict__ counts, int T, int E,
                                                  float* __restrict__ f, float* __restrict__ P,
                                                  float* __restrict__ loss) {
  __shared__ double s[512];
  const int e = threadIdx.x;
  double term = 0.0;
  if (e < E) {
    const double fe = (double)prob_sum[e] / (double)T;
    const double pe = (double)counts[e] / (double)T;
    if (f) f[e] = (float)fe;
    if (P) P[e] = (float)pe;
    term = fe * pe;
  }
  s[e] = term;
  __syncthreads();
  for (int w = 256; w >= 1; w >>= 1) {
    if (e < w) s[e] += s[e + w];
    __syncthreads();
  }
  if (e == 0) *loss = (float)((double)E * s[0]);
}

template <int KK, typename OutT>
void launch_kk(int nb, hipStream_t s, const unsigned char* y, const int32_t* dest,
               const float* gate, int T, int k, int d, const uint16_t* resid, OutT* out) {
  hipLaunchKernelGGL((combine_bf16<KK, OutT>), dim3(nb), dim3(256), 0, s, y, dest, gate,
                     T, k, d, resid, out);
}
template <typename OutT>
bool launch_combine(int k, int nb, hipStream_t s, const unsigned char* y, const int32_t* dest,
                    const float* gate, int T, int d, const uint16_t* resid, OutT* out) {
  if (k == 1) launch_kk<1>(nb, s, y, dest, gate, T, k, d, resid, out);
  else if (k == 2) launch_kk<2>(nb, s, y, dest, gate, T, k, d, resid, out);
  else if (k <= 4) launch_kk<4>(nb, s, y, dest, gate, T, k, d, resid, out);
  else if (k <= 8) launch_kk<8>(nb, s, y, dest, gate, T, k, d, resid, out);
  else if (k <= kMaxK) launch_kk<kMaxK>(nb, s, y, dest, gate, T, k, d, resid, out);
  else return false;
  return true;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_combine(const void* y_perm, int dtype, const int32_t* dest_row,
                           const float* topk_gate, int T, int k, int d, const void* residual,
                           void* out, int out_dtype, moe_stream_t stream) {
  if (T < 0 || k < 1 || d < 1) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (dtype == MOE_F32 && out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (k > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_BF16 && (d % 8) != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_perm || !dest_row || !topk_gate || !out) return MOE_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  MOE_DEBUG_CHECK(s, nullptr, 1, nullptr, dest_row, T, k);
  const int nb = ceil_div(T, kCombineWaves);
  if (dtype == MOE_BF16 && k > kMaxK) {
    if (out_dtype == MOE_BF16)
      hipLaunchKernelGGL(combine_bf16_many<uint16_t>, dim3(nb), dim3(256), 0, s,
                         (const unsigned char*)y_perm, dest_row, topk_gate, T, k, d,
                         (const uint16_t*)residual, (uint16_t*)out);
    else
      hipLaunchKernelGGL(combine_bf16_many<float>, dim3(nb), dim3(256), 0, s,
                         (const unsigned char*)y_perm, dest_row, topk_gate, T, k, d,
                         (const uint16_t*)residual, (float*)out);
  } else if (dtype == MOE_BF16) {
    const unsigned char* yq = (const unsigned char*)y_perm;
    const uint16_t* res = (const uint16_t*)residual;
    if (out_dtype == MOE_BF16) {
      if (!launch_combine<uint16_t>(k, nb, s, yq, dest_row, topk_gate, T, d, res, (uint16_t*)out))
        return MOE_ERR_UNSUPPORTED;
    } else if (!launch_combine<float>(k, nb, s, yq, dest_row, topk_gate, T, d, res, (float*)out)) {
      return MOE_ERR_UNSUPPORTED;
    }
  } else {
    hipLaunchKernelGGL(combine_f32, dim3(nb), dim3(256), 0, s, (const float*)y_perm, dest_row,
                       topk_gate, T, k, d, (const float*)residual, (float*)out);
  }
  return launch_status();
}

extern "C" int moe_aux_loss(const float* prob_sum, const int32_t* counts, int T, int E, float* f,
                            float* P, float* loss, moe_stream_t stream) {
  if (T < 1 || E < 1) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (!prob_sum || !counts || !loss) return MOE_ERR_INVALID;
  hipLaunchKernelGGL(aux_kernel, dim3(1), dim3(512), 0, (hipStream_t)stream, prob_sum, counts, T,
                     E, f, P, loss);
  return launch_status();
}
