// Tile map of expert row blocks and the fp32 FMA grouped GEMM. Used by the
// grouped FFN (ffn.hip) and its backward pass (ffn_bwd.hip).
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- tile map --
__global__ __launch_bounds__(512) void build_tile_map(const int32_t* __restrict__ offsets, int E,
                                                      int BM, int32_t* __restrict__ tile_start) {
  __shared__ int sc[2][kMaxE];
  const int e = threadIdx.x;
  int v = 0;
  if (e < E) v = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
  int cur = 0;
  sc[0][e] = v;
  __syncthreads();
  for (int off = 1; off < kMaxE; off <<= 1) {
    const int s = sc[cur][e] + (e >= off ? sc[cur][e - off] : 0);
    sc[cur ^ 1][e] = s;
    cur ^= 1;
    __syncthreads();
  }
  if (e < E) tile_start[e + 1] = sc[cur][e];
  if (e == 0) tile_start[0] = 0;
}

// Expert e with tile_start[e] <= ms < tile_start[e+1] (ms < tile_start[E]).
__device__ __forceinline__ int find_expert(const int32_t* __restrict__ tile_start, int E, int ms) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= ms) lo = mid; else hi = mid;
  }
  return lo;
}



// ---------------------------------------------------------------- fp32 ----
constexpr int FB = 64;   // tile edge
constexpr int FKC = 16;  // K step

template <bool GATHER, bool SILU>
__global__ __launch_bounds__(256) void gemm_f32(
    const float* __restrict__ act, const int32_t* __restrict__ sorted_token,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_start,
    const float* __restrict__ w, const float* __restrict__ bias, float* __restrict__ out, int E,
    int N, int K, int mslots, float* __restrict__ zout) {
  __shared__ float sW[FKC][FB + 4];
  __shared__ float sX[FKC][FB + 4];
  const int ms = blockIdx.x % mslots, nt = blockIdx.x / mslots;
  const int total = tile_start[E];
  if (ms >= total) return;
  const int e = find_expert(tile_start, E, ms);
  const int row0 = offsets[e] + (ms - tile_start[e]) * FB;
  const int rows = min(FB, offsets[e + 1] - row0);
  const int n0 = nt * FB;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

  size_t xsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid + 256 * i) / FKC;
    const int rr = row0 + (r < rows ? r : rows - 1);
    xsrc[i] = GATHER ? (size_t)sorted_token[rr] : (size_t)rr;
  }
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += FKC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c / FKC, kk = c % FKC;
      const int n = n0 + r, kg = k0 + kk;
      sW[kk][r] = (n < N && kg < K) ? w[((size_t)e * N + n) * K + kg] : 0.0f;
      sX[kk][r] = (r < rows && kg < K) ? act[xsrc[i] * K + kg] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FKC; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sW[kk][tx * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sX[kk][ty * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + tx * 4 + i;
    if (n >= N) continue;
    const float b = bias ? bias[(size_t)e * N + n] : 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = ty * 4 + j;
      if (m < rows) {
        float v = acc[i][j] + b;
        if (SILU && zout) zout[(size_t)(row0 + m) * N + n] = v;
        if (SILU) v = silu(v);
        out[(size_t)(row0 + m) * N + n] = v;
      }
    }
  }
}


}  // namespace
}  // namespace moe
