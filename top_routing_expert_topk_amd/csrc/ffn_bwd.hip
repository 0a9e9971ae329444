// Backward pass of the grouped expert FFN (the Expert module of page
// "MoE混合专家模型路由机制原理与稀疏激活实现", section "Top-K门控路由的PyTorch实现",
// y = W2 SiLU(W1 x + b1) + b2, run over each expert's rows of the
// permutation). Given dY (the gradient of the permuted outputs) it returns
//   dZ  = (dY W2[e]) * SiLU'(Z),   Z = W1[e] x[sorted_token] + b1[e]
//   dXp = dZ W1[e]                 (per permuted row, summed into dx later)
//   dW2[e] = dY_e^T SiLU(Z_e),  db2[e] = sum of dY_e rows
//   dW1[e] = dZ_e^T X_e,        db1[e] = sum of dZ_e rows
// Z and SiLU(Z) come from a forward that kept them (moe_grouped_ffn_train);
// without them Z is recomputed from x here.
//
// bf16 data path: the data gradients run on the 256 x 256 DMA-ring MFMA
// GEMM of the forward; they contract over the weights' leading index, so
// the ring reads the weights in place, K-major, through LDS transpose
// loads. The weight gradients contract over the rows of an expert: both
// operands (dY and H, dZ and the gathered x rows) are read K-major in place
// the same way by gemm_bf16_wgrad, one 256 x 128 tile per (expert, output
// block) over the expert's row range, two blocks per CU.
//
// fp32 data path: FMA tiles read the operands in place.
#include "moe_internal.h"
#include "ring_gemm.h"
#include "tile_map.h"

namespace moe {
namespace {

// Xp[r] = x[sorted_token[r]] for the kept rows (bf16, d % 8 == 0): the
// gathered input rows the dW1 product reads K-major. Grid (ceil(R_max / 4)),
// a wave per row; rows past offsets[E] exit.
__global__ __launch_bounds__(256) void gather_rows(const uint16_t* __restrict__ x,
                                                   const int32_t* __restrict__ sorted_token,
                                                   const int32_t* __restrict__ offsets, int E,
                                                   int d, uint16_t* __restrict__ xp) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= offsets[E]) return;
  const uint16_t* src = x + (size_t)sorted_token[r] * d;
  uint16_t* dst = xp + (size_t)r * d;
  for (int c = (threadIdx.x & 63) * 8; c < d; c += 64 * 8) *(u32x4*)(dst + c) = *(const u32x4*)(src + c);
}

// z <- SiLU(z) in place over the kept rows (bf16), when the backward had to
// recompute Z: the dW2 product then reads these hidden rows.
__global__ __launch_bounds__(256) void silu_rows(uint16_t* __restrict__ z,
                                                 const int32_t* __restrict__ offsets, int E,
                                                 int h) {
  const long n = (long)offsets[E] * h / 8;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    u32x4 v = *(u32x4*)(z + i * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(silu_bf16(bf16lo(v[q])), silu_bf16(bf16hi(v[q])));
    *(u32x4*)(z + i * 8) = v;
  }
}

constexpr int kWgBM = 128;             // m rows of a weight-gradient tile
constexpr int kWgRows = 32;            // K rows per step
constexpr int kWgBlk = kWgRows * 128;  // bf16 elements per block (8 KB)
constexpr int kWgSlots = 10;

// Work list of a weight-gradient GEMM: one whole tile per (expert, 128-row
// block of the M output rows, 256 output features), K range = the expert's
// rows [offsets[e], offsets[e+1]) (empty for an expert with no rows: the
// tile stores zeros).
// Tile order as in big_plan (expert-major, groups of kGroupN feature tiles,
// row blocks inside a group); when the count allows, hardware block b (on
// XCD b % 8) takes tile (b % 8) * tiles/8 + b / 8, so each XCD works through
// one contiguous range.
__global__ __launch_bounds__(256) void wgrad_plan(const int32_t* __restrict__ offsets, int E,
                                                  int mt, int nt, BigWork* __restrict__ list) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  const int tiles = E * mt * nt;
  if (b >= tiles) return;
  const int t = (tiles & 7) == 0 ? (b & 7) * (tiles >> 3) + (b >> 3) : b;
  const int e = t / (mt * nt), l = t % (mt * nt);
  const int g = l / (mt * kGroupN);
  const int gs = min(kGroupN, nt - g * kGroupN);
  const int l2 = l - g * mt * kGroupN;
  BigWork w;
  w.e = e;
  w.row0 = (l2 / gs) * kWgBM;
  w.rows = kWgBM;
  w.n0 = (g * kGroupN + l2 % gs) * kBigBN;
  w.kbeg = offsets[e];
  w.kend = offsets[e + 1];
  w.unit = -1;
  w.ms = 0;
  list[b] = w;
}

// Weight-gradient GEMM: out[e * ores + m0 + m][n0 + n] = sum over the rows r
// of expert e ([kbeg, kend) of a wgrad_plan entry) of act[r][m0 + m] *
// w[r][n0 + n], both operands K-major (rows of K and N elements). An expert
// holds a few hundred rows or fewer, so a tile is a handful of K steps, and
// a block alone on its CU would spend much of its time filling its pipeline
// and draining its output tile with the MFMAs idle. Tiles are therefore
// 256 n x 128 m on four waves (each 128 n x 64 m, 4 x 2 MFMA tiles) with
// 80 KB of LDS, so two blocks share a CU and one's fill and stores overlap
// the other's MFMAs (vmcnt is per wave, so neither waits on the other's
// stores).
// Data path: 32-row K steps of three 8 KB blocks (w features 0-127 and
// 128-255, act features 0-127; 32 k-rows x 128 features, 256-byte rows,
// chunk c of row k at c ^ 4 (k % 4)) in a ring of ten slots: block b of the
// tile's sequence (step b / 3, part b % 3) in slot b % 10, so 3.3 steps are
// resident and at the end of step j the blocks of step j+1 have landed while
// up to four later ones are in flight. Fragments come from LDS transpose
// loads (tr_frag). In the ragged last step the w rows past kend re-read row
// kend - 1 and the act rows past it are fetched from a row of zeros, so those
// k add nothing and the loop needs no mask; an expert without rows stores a
// zero tile. The tile leaves through LDS as whole 512-byte rows.
__device__ __align__(256) uint16_t g_zero_k[128];  // never written: zeros

__global__ __launch_bounds__(256, 2) void gemm_bf16_wgrad(const uint16_t* __restrict__ act,
                                                          const uint16_t* __restrict__ w,
                                                          const BigWork* __restrict__ work,
                                                          uint16_t* __restrict__ out, int N, int K,
                                                          int ores) {
  constexpr int NW = 4, P = 3, S = kWgSlots, AHEAD = S - 2 * P, IPB = 8 / NW;
  constexpr int TN = 4, TM = 2, WTM = 32 * TM;
  constexpr int OSTR = kBigBN + 8;  // staging row stride (bf16), padded for the banks
  __shared__ __align__(1024) uint16_t ring[S * kWgBlk];
  static_assert((size_t)kWgBM * OSTR * 2 <= sizeof(ring), "output tile must fit the ring");
  const BigWork wk = work[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % 2, wm = wave / 2;  // wave w runs on SIMD w
  const int ch = lane >> 5;
  // DMA: instruction (i, wave) moves k-rows 4 (i NW + wave) .. +3; this lane
  // row lane / 16 of them, chunk slot lane % 16, which holds feature chunk
  // (lane % 16) ^ 4 ((lane / 16) % 4)
  const int tchunk = (((lane & 15) ^ (4 * (lane >> 4))) << 3);
  const int ns = (wk.kend - wk.kbeg + kWgRows - 1) / kWgRows;
  const int nblk = ns * P;
  auto issue = [&](int bi) __attribute__((always_inline)) {
    const int g = bi / P, q = bi - g * P;
    uint16_t* dst = ring + (bi % S) * kWgBlk;
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int r = wk.kbeg + g * kWgRows + (i * NW + wave) * 4 + (lane >> 4);
      const uint16_t* src = q < 2 ? w + (size_t)min(r, wk.kend - 1) * N + wk.n0 + q * 128 + tchunk
                          : r < wk.kend ? act + (size_t)r * K + wk.row0 + tchunk
                                        : g_zero_k + tchunk;
      dma16(src, dst + (i * NW + wave) * 4 * 128);
    }
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x16{};

  if (ns > 0) {
    for (int bi = 0; bi < S && bi < nblk; ++bi) issue(bi);
    bf16x8 f0a[TN], f0b[TM], f1a[TN], f1b[TM];
    int sa, sb;
#define MOE_SLOTS(step)                                    \
  do {                                                     \
    const int b_ = (P * (step)) % S;                       \
    const int a_ = b_ + wn, c_ = b_ + 2;                   \
    sa = a_ < S ? a_ : a_ - S;                             \
    sb = c_ < S ? c_ : c_ - S;                             \
  } while (0)
#define MOE_RD(sub, FA, FB)                                                              \
  do {                                                                                   \
    const uint16_t* sa_ = ring + sa * kWgBlk;                                            \
    const uint16_t* sb_ = ring + sb * kWgBlk;                                            \
    _Pragma("unroll") for (int i = 0; i < TN; ++i) FA[i] = tr_frag(sa_, (sub), i, lane); \
    _Pragma("unroll") for (int j = 0; j < TM; ++j)                                       \
      FB[j] = tr_frag(sb_, (sub), wm * TM + j, lane);                                    \
  } while (0)
#define MOE_MM(FA, FB)                                                                   \
  do {                                                                                   \
    _Pragma("unroll") for (int i = 0; i < TN; ++i)                                       \
    _Pragma("unroll") for (int j = 0; j < TM; ++j)                                       \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i], FB[j], acc[i][j], 0, 0, 0); \
  } while (0)
    // step 0 landed: up to S - P later blocks may be in flight
    static_assert((S - P) * IPB == 14 && S < 4 * P, "prologue wait counts");
    if (nblk >= S) wait_vmcnt<(S - P) * IPB>();
    else if (nblk == 3 * P) wait_vmcnt<2 * P * IPB>();
    else if (nblk == 2 * P) wait_vmcnt<P * IPB>();
    else wait_vmcnt<0>();
    lds_barrier();
    MOE_SLOTS(0);
    MOE_RD(0, f0a, f0b);
    for (int j = 0; j < ns; ++j) {
      MOE_RD(1, f1a, f1b);
      MOE_MM(f0a, f0b);
      interleave_mfma_reads<TN * TM, TN * TM>();
      if (j + 1 < ns) {
        // step j+1 landed (only later blocks may be in flight), and this
        // wave's reads of step j are done before its slots are refilled
        const int issued = min(S + P * j, nblk), need = P * (j + 2) - 1;
        wait_vmcnt_le<0>(min(issued - 1 - need, AHEAD) * IPB);
        wait_lgkmcnt0();
        lds_barrier();
#pragma unroll
        for (int u = 0; u < P; ++u)
          if (S + P * j + u < nblk) issue(S + P * j + u);
        MOE_SLOTS(j + 1);
        MOE_RD(0, f0a, f0b);
      }
      MOE_MM(f1a, f1b);
      interleave_mfma_reads<TN * TM, TN * TM>();
    }
#undef MOE_SLOTS
#undef MOE_RD
#undef MOE_MM
  }

  // epilogue: bf16 into the idle ring, then whole rows out
  wait_lgkmcnt0();
  lds_barrier();
  uint16_t* ot = ring;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = wn * 128 + i * 32 + 8 * q + 4 * ch;
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = wm * WTM + j * 32 + (lane & 31);
        u32x2 o;
        o[0] = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
        o[1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        *(u32x2*)(ot + m * OSTR + nl) = o;
      }
    }
  __syncthreads();
  constexpr int CPR = kBigBN / 8;  // 16-byte chunks per row
#pragma unroll 4
  for (int c = tid; c < kWgBM * CPR; c += NW * 64) {
    const int m = c / CPR, cc = c % CPR;
    *(u32x4*)(out + ((size_t)wk.e * ores + wk.row0 + m) * N + wk.n0 + cc * 8) =
        *(const u32x4*)(ot + m * OSTR + cc * 8);
  }
}

// db[e][c] = sum of g[row][c] over expert e's rows: bf16 rows, grid
// (C / 128, E). Thread (p, c2) owns features 2 c2, 2 c2 + 1 of the block's
// 128 and sums rows p, p + 4, p + 8, ... of the expert (four loads in
// flight); the four partial sums are then added in order p = 0..3.
__global__ __launch_bounds__(256) void bias_grad_bf16(const uint16_t* __restrict__ g,
                                                      const int32_t* __restrict__ offsets, int C,
                                                      uint16_t* __restrict__ db) {
  __shared__ float part[4][128];
  const int e = blockIdx.y, cp = threadIdx.x & 63, ph = threadIdx.x >> 6;
  const int c = blockIdx.x * 128 + 2 * cp;
  const int r1 = offsets[e + 1];
  float a0 = 0.0f, a1 = 0.0f;
  int r = offsets[e] + ph;
  for (; r + 12 < r1; r += 16) {
    uint32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *(const uint32_t*)(g + (size_t)(r + 4 * u) * C + c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a0 += bf16lo(v[u]);
      a1 += bf16hi(v[u]);
    }
  }
  for (; r < r1; r += 4) {
    const uint32_t v = *(const uint32_t*)(g + (size_t)r * C + c);
    a0 += bf16lo(v);
    a1 += bf16hi(v);
  }
  part[ph][2 * cp] = a0;
  part[ph][2 * cp + 1] = a1;
  __syncthreads();
  if (ph == 0) {
    const float s0 = ((part[0][2 * cp] + part[1][2 * cp]) + part[2][2 * cp]) + part[3][2 * cp];
    const float s1 =
        ((part[0][2 * cp + 1] + part[1][2 * cp + 1]) + part[2][2 * cp + 1]) + part[3][2 * cp + 1];
    *(uint32_t*)(db + (size_t)e * C + c) = pack_bf16x2(s0, s1);
  }
}

// fp32 rows, any C: grid (ceil(C / 256), E), one feature per thread.
__global__ __launch_bounds__(256) void bias_grad_f32(const float* __restrict__ g,
                                                     const int32_t* __restrict__ offsets, int C,
                                                     float* __restrict__ db) {
  const int e = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  float a = 0.0f;
  for (int r = offsets[e]; r < offsets[e + 1]; ++r) a += g[(size_t)r * C + c];
  db[(size_t)e * C + c] = a;
}

// fp32: d/dz SiLU(z) with the library exp.
__device__ __forceinline__ float silu_grad_f32(float z) {
  const float s = 1.0f / (1.0f + expf(-z));
  return s * (1.0f + z * (1.0f - s));
}

// fp32 data gradient: out[r][n] = (sum_k a[r][k] w[e][k][n]) (* SiLU'(z[r][n])
// when DSILU) over expert e's rows (64-row tiles of the tile map), w [E][K][N].
template <bool DSILU>
__global__ __launch_bounds__(256) void gemm_f32_dgrad(
    const float* __restrict__ a, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_start, const float* __restrict__ w,
    const float* __restrict__ z, float* __restrict__ out, int E, int N, int K, int mslots) {
  __shared__ float sW[FKC][FB + 4];
  __shared__ float sA[FKC][FB + 4];
  const int ms = blockIdx.x % mslots, nt = blockIdx.x / mslots;
  if (ms >= tile_start[E]) return;
  const int e = find_expert(tile_start, E, ms);
  const int row0 = offsets[e] + (ms - tile_start[e]) * FB;
  const int rows = min(FB, offsets[e + 1] - row0);
  const int n0 = nt * FB;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FKC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      {  // weights: consecutive threads along n
        const int r = c % FB, kk = c / FB, n = n0 + r, kg = k0 + kk;
        sW[kk][r] = (n < N && kg < K) ? w[((size_t)e * K + kg) * N + n] : 0.0f;
      }
      {  // rows: consecutive threads along k
        const int r = c / FKC, kk = c % FKC, kg = k0 + kk;
        sA[kk][r] = (r < rows && kg < K) ? a[(size_t)(row0 + r) * K + kg] : 0.0f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FKC; ++kk) {
      float wv[4], av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] = sW[kk][tx * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = sA[kk][ty * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(wv[i], av[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + tx * 4 + i;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = ty * 4 + j;
      if (m < rows) {
        const size_t o = (size_t)(row0 + m) * N + n;
        out[o] = DSILU ? acc[i][j] * silu_grad_f32(z[o]) : acc[i][j];
      }
    }
  }
}

// fp32 weight gradient: out[e][m][n] = sum over expert e's rows r (in
// order) of a[r][m] * f(b[src(r)][n]), src(r) = sorted_token[r] when GATHER,
// f = SiLU when SILU. Grid (ceil(M/64) * ceil(N/64), E).
template <bool GATHER, bool SILU>
__global__ __launch_bounds__(256) void gemm_f32_wgrad(const float* __restrict__ a,
                                                      const float* __restrict__ b,
                                                      const int32_t* __restrict__ sorted_token,
                                                      const int32_t* __restrict__ offsets, int M,
                                                      int N, float* __restrict__ out) {
  __shared__ float sA[FKC][FB + 4];
  __shared__ float sB[FKC][FB + 4];
  const int nmt = (M + FB - 1) / FB;
  const int m0 = (blockIdx.x % nmt) * FB, n0 = (blockIdx.x / nmt) * FB, e = blockIdx.y;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = r0; k0 < r1; k0 += FKC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, col = c % FB, kk = c / FB, r = k0 + kk;
      const bool live = r < r1;
      const int m = m0 + col, n = n0 + col;
      sA[kk][col] = (live && m < M) ? a[(size_t)r * M + m] : 0.0f;
      float v = 0.0f;
      if (live && n < N) {
        const size_t src = GATHER ? (size_t)sorted_token[r] : (size_t)r;
        v = b[src * N + n];
        if (SILU) v = silu(v);
      }
      sB[kk][col] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FKC; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sA[kk][tx * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = sB[kk][ty * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tx * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + ty * 4 + j;
      if (n < N) out[((size_t)e * M + m) * N + n] = acc[i][j];
    }
  }
}

int ffn_backward_f32(const float* x, int T, int d, int h, int E, int k, const int32_t* offsets,
                     const int32_t* sorted_token, const float* w1, const float* b1,
                     const float* w2, const float* dy, const float* zin, const float* hin,
                     float* dxp, float* dw1, float* db1, float* dw2, float* db2, void* ws,
                     hipStream_t s) {
  const FfnBwdLayout L = ffn_bwd_layout(T, d, h, E, k);
  unsigned char* base = (unsigned char*)ws;
  int32_t* tile_start = (int32_t*)base;
  float* Zw = (float*)(base + L.z);
  const float* Z = zin ? zin : Zw;
  float* dZ = (float*)(base + L.dz);
  const long rows = (long)T * k;
  const int nonempty = (int)(rows < E ? rows : E);
  const int mslots = ceil_div(rows, FB) + nonempty;
  hipLaunchKernelGGL(build_tile_map, dim3(1), dim3(512), 0, s, offsets, E, FB, tile_start);
  if (rows > 0) {
    if (!zin)
      hipLaunchKernelGGL((gemm_f32<true, false>), dim3(mslots * ceil_div(h, FB)), dim3(256), 0, s,
                         x, sorted_token, offsets, tile_start, w1, b1, Zw, E, h, d, mslots,
                         (float*)nullptr);
    // dZ = (dY W2[e]) * SiLU'(Z): W2[e] is [d][h] = [K][N]
    hipLaunchKernelGGL((gemm_f32_dgrad<true>), dim3(mslots * ceil_div(h, FB)), dim3(256), 0, s, dy,
                       offsets, tile_start, w2, Z, dZ, E, h, d, mslots);
    // dXp = dZ W1[e]: W1[e] is [h][d] = [K][N]
    hipLaunchKernelGGL((gemm_f32_dgrad<false>), dim3(mslots * ceil_div(d, FB)), dim3(256), 0, s, dZ,
                       offsets, tile_start, w1, (const float*)nullptr, dxp, E, d, h, mslots);
  }
  const dim3 g2(ceil_div(d, FB) * ceil_div(h, FB), E);
  if (hin)
    hipLaunchKernelGGL((gemm_f32_wgrad<false, false>), g2, dim3(256), 0, s, dy, hin, sorted_token,
                       offsets, d, h, dw2);
  else
    hipLaunchKernelGGL((gemm_f32_wgrad<false, true>), g2, dim3(256), 0, s, dy, Z, sorted_token,
                       offsets, d, h, dw2);
  hipLaunchKernelGGL((gemm_f32_wgrad<true, false>), g2, dim3(256), 0, s, (const float*)dZ, x,
                     sorted_token, offsets, h, d, dw1);
  if (db2)
    hipLaunchKernelGGL(bias_grad_f32, dim3(ceil_div(d, 256), E), dim3(256), 0, s, dy, offsets, d,
                       db2);
  if (db1)
    hipLaunchKernelGGL(bias_grad_f32, dim3(ceil_div(h, 256), E), dim3(256), 0, s,
                       (const float*)dZ, offsets, h, db1);
  return launch_status();
}

int ffn_backward_bf16(const uint16_t* x, int T, int d, int h, int E, int k,
                      const int32_t* offsets, const int32_t* sorted_token, const uint16_t* w1,
                      const uint16_t* b1, const uint16_t* w2, const uint16_t* dy,
                      const uint16_t* zin, const uint16_t* hin, uint16_t* dxp, uint16_t* dw1,
                      uint16_t* db1, uint16_t* dw2, uint16_t* db2, void* ws, hipStream_t s) {
  const FfnBwdLayout L = ffn_bwd_layout(T, d, h, E, k);
  unsigned char* base = (unsigned char*)ws;
  const long rows = (long)T * k;
  BigHdr* hdr = (BigHdr*)base;
  const int g1 = ffn_big_grid(rows, E, h, kBigBM), g2 = ffn_big_grid(rows, E, d, kBigBM);
  BigWork* list1 = (BigWork*)(base + 256);
  BigWork* list2 = list1 + g1;
  const int md = d / kBigBN, mh = h / kBigBN;
  const int nw2 = E * (d / kWgBM) * mh, nw1 = E * (h / kWgBM) * md;
  BigWork* wl2 = (BigWork*)(base + L.wl);  // dW2: M = d, N = h
  BigWork* wl1 = wl2 + nw2;                // dW1: M = h, N = d
  uint16_t* Zw = (uint16_t*)(base + L.z);
  const uint16_t* Z = zin ? zin : Zw;
  uint16_t* dZ = (uint16_t*)(base + L.dz);
  uint16_t* xp = (uint16_t*)(base + L.xp);
  uint16_t* const nz = nullptr;
  float* part = (float*)(base + L.part);
  const uint16_t* none = nullptr;
  const dim3 gr(kTailSlots * kReduceSlices), rb(kRingWaves * 64);

  // the data-gradient products (K-major weights) run on the forward's tiles
  hipLaunchKernelGGL((big_plan<kBigBM, true>), dim3(ceil_div(g1 + g2, kMaxE)), dim3(kMaxE), 0, s,
                     offsets, E, big_xr(E), mh, d / kRS, g1, md, h / kRS, g2, hdr, list1, list2, sorted_token,
                     (int32_t*)nullptr);
  hipLaunchKernelGGL(wgrad_plan, dim3(ceil_div(nw2, 256)), dim3(256), 0, s, offsets, E, d / kWgBM, mh,
                     wl2);
  hipLaunchKernelGGL(wgrad_plan, dim3(ceil_div(nw1, 256)), dim3(256), 0, s, offsets, E, h / kWgBM, md,
                     wl1);
  if (rows > 0)
    hipLaunchKernelGGL(gather_rows, dim3(ceil_div(rows, 4)), dim3(256), 0, s, x, sorted_token,
                       offsets, E, d, xp);
  if (!zin) {
    // Z = W1[e] x + b1 (the forward's first product without the activation),
    // on the forward's tiles (taller last tiles included), so that it equals
    // the Z a training forward keeps bit for bit
    BigHdr* hdr_r = (BigHdr*)(base + L.zr);
    BigWork* list_r = (BigWork*)(base + L.zr + 256);
    hipLaunchKernelGGL((big_plan<kBigBM, true>), dim3(ceil_div(g1, kMaxE)), dim3(kMaxE), 0,
                       s, offsets, E, big_xr(E), mh, d / kRS, g1, md, h / kRS, 0, hdr_r, list_r,
                       (BigWork*)nullptr, sorted_token, (int32_t*)nullptr);
    hipLaunchKernelGGL((gemm_bf16_ring<kRingWaves, true, kEpiBias>), dim3(g1), rb, 0, s, x,
                       sorted_token, list_r, w1, b1, Zw, part, h, d, (size_t)h * d, 0, none, nz);
    hipLaunchKernelGGL((big_tail_reduce<kBigRowsMax, kEpiBias>), gr, dim3(256), 0, s, hdr_r,
                       list_r, b1, part, Zw, h, none, nz);
  }
  // dZ = (dY W2[e]) * SiLU'(Z): W2[e] is [d][h], K-major for this product
  hipLaunchKernelGGL((gemm_bf16_ring<kRingWaves, false, kEpiDSilu, true>), dim3(g1), rb, 0, s, dy,
                     (const int32_t*)nullptr, list1, w2, none, dZ, part, h, d, (size_t)h * d, 0,
                     Z, nz);
  hipLaunchKernelGGL((big_tail_reduce<kBigRowsMax, kEpiDSilu>), gr, dim3(256), 0, s, hdr, list1, none,
                     part, dZ, h, Z, nz);
  // H: the forward's, or SiLU of the recomputed Z (in place, Z is no longer read)
  const uint16_t* H = hin;
  if (!hin) {
    hipLaunchKernelGGL(silu_rows, dim3(2048), dim3(256), 0, s, Zw, offsets, E, h);
    H = Zw;
  }
  // dW2[e] = dY_e^T H_e, dW1[e] = dZ_e^T X_e: both operands K-major
  hipLaunchKernelGGL(gemm_bf16_wgrad, dim3(nw2), dim3(256), 0, s, dy, H, (const BigWork*)wl2, dw2,
                     h, d, d);
  hipLaunchKernelGGL(gemm_bf16_wgrad, dim3(nw1), dim3(256), 0, s, (const uint16_t*)dZ,
                     (const uint16_t*)xp, (const BigWork*)wl1, dw1, d, h, h);
  // dXp = dZ W1[e]: W1[e] is [h][d], K-major for this product
  hipLaunchKernelGGL((gemm_bf16_ring<kRingWaves, false, kEpiBias, true>), dim3(g2), rb, 0, s,
                     (const uint16_t*)dZ, (const int32_t*)nullptr, list2, w1, none, dxp, part, d, h,
                     (size_t)d * h, 0, none, nz);
  hipLaunchKernelGGL((big_tail_reduce<kBigRowsMax, kEpiBias>), gr, dim3(256), 0, s, hdr + 1, list2, none,
                     part, dxp, d, none, nz);
  if (db2)
    hipLaunchKernelGGL(bias_grad_bf16, dim3(d / 128, E), dim3(256), 0, s, dy, offsets, d, db2);
  if (db1)
    hipLaunchKernelGGL(bias_grad_bf16, dim3(h / 128, E), dim3(256), 0, s, (const uint16_t*)dZ,
                       offsets, h, db1);
  return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_grouped_ffn_backward(const void* x, int dtype, int T, int d, int h, int E, int k,
                                        const int32_t* offsets, const int32_t* sorted_token,
                                        const void* w1, const void* b1, const void* w2,
                                        const void* dy_perm, const void* z_perm,
                                        const void* h_perm, void* dx_perm, void* dw1, void* db1,
                                        void* dw2, void* db2, void* ws, size_t ws_bytes,
                                        moe_stream_t stream) {
  if (T < 0 || d < 1 || h < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  const long rows = (long)T * k;
  if (rows > 0x7FFFFFFFL) return MOE_ERR_UNSUPPORTED;
  if (!offsets || !w1 || !w2 || !dw1 || !dw2) return MOE_ERR_INVALID;
  if (rows > 0 && (!x || !sorted_token || !dy_perm || !dx_perm)) return MOE_ERR_INVALID;
  if ((z_perm == nullptr) != (h_perm == nullptr)) return MOE_ERR_INVALID;
  if (!ws || ws_bytes < ffn_bwd_layout(T, d, h, E, k).total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  MOE_DEBUG_CHECK(s, offsets, E, rows > 0 ? sorted_token : nullptr, nullptr, T, k);
  if (dtype == MOE_F32)
    return ffn_backward_f32((const float*)x, T, d, h, E, k, offsets, sorted_token,
                            (const float*)w1, (const float*)b1, (const float*)w2,
                            (const float*)dy_perm, (const float*)z_perm, (const float*)h_perm,
                            (float*)dx_perm, (float*)dw1, (float*)db1, (float*)dw2, (float*)db2,
                            ws, s);
  // bf16: 256-wide tiles on both widths; 32-bit element offsets of the
  // gathered x rows and the permuted rows in the ring's DMA
  if ((d % kBigBN) != 0 || (h % kBigBN) != 0) return MOE_ERR_UNSUPPORTED;
  if ((long)T * d >= (1L << 31) || rows * d >= (1L << 31) || rows * h >= (1L << 31))
    return MOE_ERR_UNSUPPORTED;
  return ffn_backward_bf16((const uint16_t*)x, T, d, h, E, k, offsets, sorted_token,
                           (const uint16_t*)w1, (const uint16_t*)b1, (const uint16_t*)w2,
                           (const uint16_t*)dy_perm, (const uint16_t*)z_perm,
                           (const uint16_t*)h_perm, (uint16_t*)dx_perm, (uint16_t*)dw1,
                           (uint16_t*)db1, (uint16_t*)dw2, (uint16_t*)db2, ws, s);
}
