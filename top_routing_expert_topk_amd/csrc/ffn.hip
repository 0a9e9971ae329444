// Grouped expert FFN: for each expert e, over its rows of the permutation,
//   H = SiLU(W1[e] . x[sorted_token] + b1[e]),   Y = W2[e] . H + b2[e]
// (the Expert module of page "MoE混合专家模型路由机制原理与稀疏激活实现", section
// "Top-K门控路由的PyTorch实现"; one grouped kernel per layer of the FFN
// rather than a loop over experts, as section 3.3 of
// "MoE三难困境破解：按需加载+路由解耦+显存精控" asks of its _grouped_ffn).
//
// Kernels:
//   build_tile_map  prefix sum of ceil(kept_e / BM) -> tile_start[E+1], so a
//                   gemm_bf16 / gemm_f32 block finds its (expert, row block)
//                   with no host read
//   big_plan        work lists (tile, K range) of both GEMMs of the DMA-ring
//                   paths and the token table of their row blocks, built
//                   from offsets on the device
//   gemm_bf16_ring  256 x 256 MFMA tiles fed by a global->LDS DMA ring of
//                   64-column steps; tail tiles split along K
//   gemm_bf16_pring persistent 256 x 128 variant for experts of fewer rows:
//                   one block per CU, the ring running across its tiles
//   big_tail_reduce sums the K-range partials of split tail tiles in order
//   gemm_bf16       128 x 128 MFMA tiles, LDS double-buffered 64-deep K
//                   steps, for widths that are not multiples of 256
//   decode_bf16     weight-streaming path for few rows per expert: each
//                   touched expert's weights are read once per 4 rows, rows
//                   of untouched experts cost one offsets read
//   gemm_f32        FMA tiles for fp32 layers
// In every kernel the gather of x rows is fused into the activation load and
// bias (+SiLU) into the epilogue. H leaves in bf16 (the second product's
// MFMA operand); Y leaves in the block fixed point of moe_internal.h (YQ: 8
// features of a row share a power-of-two exponent, int16 mantissas), whose
// error is a 2^-15 fraction of each block's largest value.
#include <type_traits>

#include "moe_internal.h"
#include "ring_gemm.h"
#include "tile_map.h"

namespace moe {
namespace {

constexpr int KC = 64;  // bf16 K elements per LDS stage (128 bytes per row)

// The tile map (build_tile_map, find_expert) and the fp32 FMA GEMM live in
// tile_map.h (shared with the backward pass).

// ------------------------------------------------------------- MFMA GEMM --
// Block tile: BN weight rows (output features) x BM permuted rows. Four waves
// in a 2 x 2 grid, each (BN/2) x (BM/2) of 16x16 MFMA tiles.
// v_mfma_f32_16x16x32_bf16 operands: A = weight rows (16 n x 32 k), B =
// activation rows (32 k x 16 rows); lane l gives row (l%16), k-octet (l/16)
// and receives D[n = 4*(l/16)+v][row = l%16], i.e. 4 consecutive output
// features of one row -> one 8-byte store.
// LDS rows are 64 bf16 (8 chunks of 16 B); chunk c of row r sits at
// c ^ ((r >> 1) & 7), so the 16 lanes of one ds_read_b128 pass, reading 16
// rows at one chunk, spread over all 16 bank groups of 16 bytes.
template <int BN, int BM, bool GATHER, bool SILU, bool YQ = false>
__global__ __launch_bounds__(256) void gemm_bf16(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ sorted_token,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_start,
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
    void* __restrict__ out, int E, int N, int K, int mslots, uint16_t* __restrict__ zout) {
  constexpr int TN = BN / 32, TM = BM / 32;  // 16-wide tiles per wave
  constexpr int AL = BN * 8 / 256, BL = BM * 8 / 256;  // 16-byte chunks per thread
  __shared__ __align__(16) uint16_t sA[2][BN * KC];
  __shared__ __align__(16) uint16_t sB[2][BM * KC];

  const int ms = blockIdx.x % mslots, nt = blockIdx.x / mslots;
  const int total = tile_start[E];
  if (ms >= total) return;
  const int e = find_expert(tile_start, E, ms);
  const int row0 = offsets[e] + (ms - tile_start[e]) * BM;
  const int rows = min(BM, offsets[e + 1] - row0);
  const int n0 = nt * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;

  const uint16_t* asrc[AL];
  const uint16_t* bsrc[BL];
  int aoff[AL], boff[BL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int c = tid + 256 * i, r = c >> 3, ch = c & 7;
    asrc[i] = w + ((size_t)e * N + n0 + r) * K + ch * 8;
    aoff[i] = r * KC + ((ch ^ ((r >> 1) & 7)) * 8);
  }
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    const int c = tid + 256 * i, r = c >> 3, ch = c & 7;
    const int rr = row0 + (r < rows ? r : rows - 1);
    const size_t src = GATHER ? (size_t)sorted_token[rr] : (size_t)rr;
    bsrc[i] = act + src * K + ch * 8;
    boff[i] = r * KC + ((ch ^ ((r >> 1) & 7)) * 8);
  }

  f32x4 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[AL], rb[BL];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AL; ++i) ra[i] = *(const u32x4*)(asrc[i] + k0);
#pragma unroll
    for (int i = 0; i < BL; ++i) rb[i] = *(const u32x4*)(bsrc[i] + k0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AL; ++i) *(u32x4*)(&sA[buf][aoff[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < BL; ++i) *(u32x4*)(&sB[buf][boff[i]]) = rb[i];
  };

  const int nk = K / KC;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * KC);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int ch = kh * 4 + (lane >> 4);
      bf16x8 a[TN], b[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int r = wn * (BN / 2) + i * 16 + (lane & 15);
        a[i] = *(const bf16x8*)(&sA[cur][r * KC + ((ch ^ ((r >> 1) & 7)) * 8)]);
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int r = wm * (BM / 2) + j * 16 + (lane & 15);
        b[j] = *(const bf16x8*)(&sB[cur][r * KC + ((ch ^ ((r >> 1) & 7)) * 8)]);
      }
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int n = n0 + wn * (BN / 2) + i * 16 + 4 * (lane >> 4);
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
      const u32x2 bb = *(const u32x2*)(bias + (size_t)e * N + n);
      bv[0] = bf16lo(bb[0]);
      bv[1] = bf16hi(bb[0]);
      bv[2] = bf16lo(bb[1]);
      bv[3] = bf16hi(bb[1]);
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = wm * (BM / 2) + j * 16 + (lane & 15);
      if constexpr (YQ) {
        // lanes l and l ^ 16 hold features 0-3 and 4-7 of one block of a row
        float v[4], mx = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = acc[i][j][q] + bv[q];
          mx = fmaxf(mx, fabsf(v[q]));
        }
        const int ex = yq_exponent(fmaxf(mx, __shfl_xor(mx, 16, 64)));
        if (m < rows) {
          unsigned char* row = (unsigned char*)out + (size_t)(row0 + m) * yq_row_bytes(N);
          u32x2 o;
          o[0] = ((uint32_t)yq_encode(v[0], ex) & 0xFFFFu) | ((uint32_t)yq_encode(v[1], ex) << 16);
          o[1] = ((uint32_t)yq_encode(v[2], ex) & 0xFFFFu) | ((uint32_t)yq_encode(v[3], ex) << 16);
          *(u32x2*)(row + (size_t)2 * n) = o;
          if (((lane >> 4) & 1) == 0) row[(size_t)2 * N + n / kYBlock] = (unsigned char)(signed char)ex;
        }
        continue;
      }
      if (m < rows) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[i][j][q] + bv[q];
        if (SILU && zout) {
          u32x2 z;
          z[0] = pack_bf16x2(v[0], v[1]);
          z[1] = pack_bf16x2(v[2], v[3]);
          *(u32x2*)(zout + (size_t)(row0 + m) * N + n) = z;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (SILU) v[q] = silu_bf16(v[q]);
        u32x2 o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        *(u32x2*)((uint16_t*)out + (size_t)(row0 + m) * N + n) = o;
      }
    }
  }
}

// The 256 x 256 DMA-ring GEMM, its work lists, epilogue and tail reduction
// live in ring_gemm.h (shared with the backward pass).

// ------------------------------------------------ persistent DMA-ring GEMM --
// One block per CU walks its share of the launch's tiles with a single DMA
// ring that runs across tile boundaries: the first steps of the next tile are
// already in flight while the current one finishes, and each finished tile
// leaves straight from the accumulators (8-byte stores of 4 features of one
// row; the ring holds the next tile's data), so no tile pays a pipeline fill
// or drain. Whole tiles are dealt in the tile order, each XCD's 32 blocks
// taking one contiguous range 32 tiles at a time; the K ranges of split tail
// tiles follow, one per block.
// Used for BM = 128 (experts of fewer rows, where the weight stream from HBM
// is the bound): 3 blocks per step (two weight halves, one row block), 9
// slots, so two more steps are in flight; waves 4 x 2 of 64 x 64. The BM =
// 256 shape (gemm_bf16_ring's tile and waves, 4 blocks per step, 10 slots)
// measures slower than gemm_bf16_ring, whose LDS-staged epilogue writes
// whole rows: there the MFMA work per tile dwarfs the pipeline fill.
template <int BM>
struct PRing {
  static constexpr int P = 2 + BM / 128;        // 16 KB blocks per 64-column step
  static constexpr int S = BM == 256 ? 10 : 9;  // ring slots
  static constexpr int AHEAD = S - 2 * P;       // blocks past step j+1 in flight at the end of step j
  static constexpr int WN = BM == 256 ? 2 : 4;  // waves along the weight rows
  static constexpr int WM = 8 / WN;
  static constexpr int WTN = kBigBN / WN, WTM = BM / WM;
  static constexpr int TN = WTN / 32, TM = WTM / 32;
  static constexpr int NBQ = BM / 128;          // permuted-row blocks per step
};

template <int BM, bool GATHER, bool SILU, bool YQ = false>
__global__ __launch_bounds__(512) void gemm_bf16_pring(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ tok_tab,
    const BigHdr* __restrict__ hdr, const BigWork* __restrict__ units,
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
    void* __restrict__ out, float* __restrict__ part, int N, int K,
    uint16_t* __restrict__ zout) {
  using C = PRing<BM>;
  constexpr int P = C::P, S = C::S, AHEAD = C::AHEAD, NBQ = C::NBQ;
  constexpr int TN = C::TN, TM = C::TM, WM = C::WM, WTN = C::WTN, WTM = C::WTM;
  constexpr int NW = 8, IPB = 2;
  __shared__ __align__(1024) uint16_t ring[S * kRBlk];

  cu32* hp = (cu32*)hdr;
  const int full = __builtin_amdgcn_readfirstlane((int)hp[0]);
  const int tail = __builtin_amdgcn_readfirstlane((int)hp[1]);
  const int split = __builtin_amdgcn_readfirstlane((int)hp[2]);
  const int b = blockIdx.x;  // gridDim.x == kTailSlots, one block per CU
  const int nf = full / kTailSlots;
  const bool has_tail = b < tail * split;
  const int nu = nf + (has_tail ? 1 : 0);
  if (nu == 0) return;
  const int per_xcd = full >> 3;
  // unit i of this block: whole tiles walk the XCD's contiguous range 32 at a
  // time, then this block's K range of a split tail tile
  auto unit_of = [&](int i) { return i < nf ? (b & 7) * per_xcd + (b >> 3) + 32 * i : full + b; };
  const int nsf = K / kRS;
  int tlen = 0;
  if (has_tail) {
    const WorkS t = load_work(units, full + b);
    tlen = t.kend - t.kbeg;
  }
  const int total = nf * nsf + tlen;  // 64-column steps of this block
  const int nblk = total * P;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / WM, wm = wave % WM;
  const int r0 = wave * 8 + (lane >> 3);
  const int c0 = swz128(r0, lane & 7) * 8;

  // ---- issue side: the unit whose blocks are being issued.
  // Activation rows are 32-bit element offsets. Gathered rows take their
  // token from the token table with scalar loads (8 consecutive rows per
  // wave and DMA instruction, lane l using row l/8), so no vector load sits
  // in the DMA queue that the ring's vmcnt waits count.
  uint32_t bo[NBQ][IPB];
  auto row_offsets = [&](int row0, int rows, int ms) {
#pragma unroll
    for (int q = 0; q < NBQ; ++q)
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        uint32_t tok;
        if (GATHER) {
          cu32* tp = (cu32*)(tok_tab + (size_t)ms * BM + q * 128 + i * 64 + wave * 8);
          uint32_t t8[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) t8[v] = tp[v];
          const int sel = lane >> 3;
          tok = t8[0];
#pragma unroll
          for (int v = 1; v < 8; ++v) tok = sel == v ? t8[v] : tok;
        } else {
          const int pr = q * 128 + i * 64 + r0;
          tok = (uint32_t)(row0 + (pr < rows ? pr : rows - 1));
        }
        bo[q][i] = tok * (uint32_t)K + c0;
      }
  };
  int iu = 0, ig0 = 0, ilen, ikbeg;
  const uint16_t* wb;
  auto enter_unit = [&](int i) {
    const WorkS u = load_work(units, unit_of(i));
    ilen = u.kend - u.kbeg;
    ikbeg = u.kbeg;
    wb = w + ((size_t)u.e * N + u.n0 + r0) * K + c0;
    row_offsets(u.row0, u.rows, u.ms);
  };
  enter_unit(0);
  auto issue_block = [&](int bi) {
    const int g = bi / P, q = bi - g * P;
    if (g == ig0 + ilen) {  // first block of the next unit
      ++iu;
      ig0 += ilen;
      enter_unit(iu);
    }
    const int koff = (ikbeg + g - ig0) * kRS;
    uint16_t* dst = ring + (bi % S) * kRBlk;
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const uint16_t* src;
      // weights non-temporal: with at most a few row blocks per expert they
      // are read about once, and the hint measured faster here (it slows
      // the 256-row ring, whose tile order reuses weight panels from L2)
      if (q < 2) {
        src = wb + (size_t)(q * 128 + i * 64) * K + koff;
        dma16_nt(src, dst + (i * NW + wave) * 8 * kRS);
      } else {
        src = act + (q == 2 ? bo[0][i] : bo[NBQ - 1][i]) + koff;
        dma16(src, dst + (i * NW + wave) * 8 * kRS);
      }
    }
  };

  // ---- compute side
  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x16{};

#pragma unroll
  for (int bi = 0; bi < S; ++bi)
    if (bi < nblk) issue_block(bi);

  const int ch = lane >> 5;
  const int aq = (wn * WTN) >> 7, ar = (wn * WTN) & 127;  // this wave's weight block, first row
  const int bq = (wm * WTM) >> 7, br = (wm * WTM) & 127;  // its permuted-row block, first row
  bf16x8 f0a[TN], f0b[TM], f1a[TN], f1b[TM];
  int sa, sb;
#define MOE_SLOTS(step)                                    \
  do {                                                     \
    const int b_ = (P * (step)) % S;                       \
    const int a_ = b_ + aq, c_ = b_ + 2 + bq;              \
    sa = a_ < S ? a_ : a_ - S;                             \
    sb = c_ < S ? c_ : c_ - S;                             \
  } while (0)
#define MOE_RD(sub, FA, FB)                                                            \
  do {                                                                                 \
    const uint16_t* sa_ = ring + sa * kRBlk;                                           \
    const uint16_t* sb_ = ring + sb * kRBlk;                                           \
    _Pragma("unroll") for (int i = 0; i < TN; ++i) {                                   \
      const int r = ar + i * 32 + (lane & 31);                                         \
      FA[i] = *(const bf16x8*)(sa_ + r * kRS + swz128(r, 2 * (sub) + ch) * 8);         \
    }                                                                                  \
    _Pragma("unroll") for (int j = 0; j < TM; ++j) {                                   \
      const int r = br + j * 32 + (lane & 31);                                         \
      FB[j] = *(const bf16x8*)(sb_ + r * kRS + swz128(r, 2 * (sub) + ch) * 8);         \
    }                                                                                  \
  } while (0)
#define MOE_MM(FA, FB)                                                                 \
  do {                                                                                 \
    _Pragma("unroll") for (int i = 0; i < TN; ++i)                                     \
    _Pragma("unroll") for (int j = 0; j < TM; ++j)                                     \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i], FB[j], acc[i][j], 0, 0, 0); \
  } while (0)

  // step 0 landed: the blocks of the next steps may still be in flight
  if (nblk >= S) wait_vmcnt<(S - P) * IPB>(); else wait_vmcnt<0>();
  lds_barrier();
  MOE_SLOTS(0);
  MOE_RD(0, f0a, f0b);
  int cu = 0, cend = nf > 0 ? nsf : tlen;  // compute unit, its end step
  for (int g = 0; g < total; ++g) {
    MOE_RD(1, f1a, f1b);
    MOE_MM(f0a, f0b);
    MOE_RD(2, f0a, f0b);
    MOE_MM(f1a, f1b);
    MOE_RD(3, f1a, f1b);
    MOE_MM(f0a, f0b);
    if (g + 1 < total) {
      // step g+1 landed (only later blocks may be in flight), and this wave's
      // reads of step g are done before its slots are refilled
      const int newest = min(S + P * g, nblk) - 1, need = P * (g + 2) - 1;
      if (newest - need >= AHEAD) wait_vmcnt<AHEAD * IPB>(); else wait_vmcnt<0>();
      wait_lgkmcnt0();
      lds_barrier();
#pragma unroll
      for (int u = 0; u < P; ++u)
        if (S + P * g + u < nblk) issue_block(S + P * g + u);
      MOE_SLOTS(g + 1);
      MOE_RD(0, f0a, f0b);
    }
    MOE_MM(f1a, f1b);
    if (g + 1 == cend) {
      // the unit is done: partial or finished tile straight from the accumulators
      const WorkS uc = load_work(units, unit_of(cu));
      if (uc.unit >= 0) {
        float* pp = part + (size_t)uc.unit * (BM * kBigBN);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nl = wn * WTN + i * 32 + 8 * q + 4 * ch;
#pragma unroll
            for (int j = 0; j < TM; ++j) {
              const int m = wm * WTM + j * 32 + (lane & 31);
              *(f32x4*)(pp + m * kBigBN + nl) = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                      acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            }
          }
      } else {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nb = wn * WTN + i * 32 + 8 * q;  // uniform: 8 features, 4 per half-wave
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (bias) {
              cu32* bp = (cu32*)(bias + (size_t)uc.e * N + uc.n0 + nb);
              const uint32_t p0 = bp[0], p1 = bp[1], p2 = bp[2], p3 = bp[3];
              const uint32_t lo = ch ? p2 : p0, hi = ch ? p3 : p1;
              bv[0] = bf16lo(lo);
              bv[1] = bf16hi(lo);
              bv[2] = bf16lo(hi);
              bv[3] = bf16hi(hi);
            }
            const int nl = nb + 4 * ch;
#pragma unroll
            for (int j = 0; j < TM; ++j) {
              const int m = wm * WTM + j * 32 + (lane & 31);
              float v[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * q + t] + bv[t];
              if (SILU && zout && m < uc.rows) {
                u32x2 z;
                z[0] = pack_bf16x2(v[0], v[1]);
                z[1] = pack_bf16x2(v[2], v[3]);
                *(u32x2*)(zout + (size_t)(uc.row0 + m) * N + uc.n0 + nl) = z;
              }
#pragma unroll
              for (int t = 0; t < 4; ++t)
                if (SILU) v[t] = silu_bf16(v[t]);
              if constexpr (YQ) {
                // lanes l and l ^ 32 hold features nb..nb+3 and nb+4..nb+7
                float mx = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
                const int ex = yq_exponent(fmaxf(mx, __shfl_xor(mx, 32, 64)));
                if (m < uc.rows) {
                  unsigned char* row = (unsigned char*)out + (size_t)(uc.row0 + m) * yq_row_bytes(N);
                  u32x2 o;
                  o[0] = ((uint32_t)yq_encode(v[0], ex) & 0xFFFFu) |
                         ((uint32_t)yq_encode(v[1], ex) << 16);
                  o[1] = ((uint32_t)yq_encode(v[2], ex) & 0xFFFFu) |
                         ((uint32_t)yq_encode(v[3], ex) << 16);
                  *(u32x2*)(row + (size_t)2 * (uc.n0 + nl)) = o;
                  if (ch == 0)
                    row[(size_t)2 * N + (uc.n0 + nb) / kYBlock] = (unsigned char)(signed char)ex;
                }
              } else if (m < uc.rows) {
                u32x2 o;
                o[0] = pack_bf16x2(v[0], v[1]);
                o[1] = pack_bf16x2(v[2], v[3]);
                *(u32x2*)((uint16_t*)out + (size_t)(uc.row0 + m) * N + uc.n0 + nl) = o;
              }
            }
          }
      }
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x16{};
      ++cu;
      cend += cu < nf ? nsf : tlen;
    }
  }
#undef MOE_SLOTS
#undef MOE_RD
#undef MOE_MM
}

// ------------------------------------------------------ decode streaming --
// Grid (ceil(N / 16), E). Each wave owns 4 consecutive output features and
// computes them for up to G rows of expert e at a time; the rows' activations
// sit in LDS, the weights stream straight from HBM with 16-byte loads (8
// loads per row in flight per lane for K = 4096), and each dot product ends
// in a wave butterfly sum.
constexpr int DG = 4;    // rows per pass
constexpr int DRPW = 4;  // output features per wave
constexpr int DRPB = 4 * DRPW;

__device__ __forceinline__ float dot8(const u32x4 a, const u32x4 b) {
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s = fmaf(bf16lo(a[q]), bf16lo(b[q]), s);
    s = fmaf(bf16hi(a[q]), bf16hi(b[q]), s);
  }
  return s;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// With an expert cache (slot_of != NULL) expert e's weights sit in device slot
// slot_of[e] of the weight arrays, and only experts with phase_of[e] == phase
// run, so a launch can cover the resident experts while others are copied in.
// YQ: the outputs leave in the block fixed point (the second product); a
// block of 8 features is the 4 of wave w and the 4 of wave w ^ 1, so the
// waves leave their sums in LDS and lane 0 of each encodes its 4 against the
// largest magnitude of the 8. Otherwise bf16 (H).
template <bool GATHER, bool SILU, bool YQ>
__global__ __launch_bounds__(256) void decode_bf16(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ sorted_token,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ bias, void* __restrict__ out, int E, int N, int K,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ phase_of, int phase,
    uint16_t* __restrict__ zout) {
  extern __shared__ __align__(16) uint16_t sx[];  // [DG][K]
  __shared__ float sy[4][DRPW][DG];               // YQ: every wave's outputs of the pass
  const int e = blockIdx.y;
  const int r0 = offsets[e];
  const int cnt = offsets[e + 1] - r0;
  if (cnt <= 0) return;
  if (phase_of && phase_of[e] != phase) return;
  const int ew = slot_of ? slot_of[e] : e;  // where expert e's weights are
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockIdx.x * DRPB + wave * DRPW;
  const int kchunks = K / 8;

  for (int g0 = 0; g0 < cnt; g0 += DG) {
    const int ng = min(DG, cnt - g0);
    for (int c = tid; c < ng * kchunks; c += 256) {
      const int g = c / kchunks, kc = c - g * kchunks;
      const int rr = r0 + g0 + g;
      const size_t src = GATHER ? (size_t)sorted_token[rr] : (size_t)rr;
      *(u32x4*)(sx + g * K + kc * 8) = *(const u32x4*)(act + src * K + kc * 8);
    }
    __syncthreads();
    // not unrolled: two passes' weight loads in flight at once would cost a
    // wave per SIMD of occupancy, which this HBM-bound loop needs more
#pragma unroll 1
    for (int rp = 0; rp < DRPW; rp += 2) {
      const int n = nw + rp;
      float acc[2][DG];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int g = 0; g < DG; ++g) acc[a][g] = 0.0f;
      const uint16_t* w0 = w + ((size_t)ew * N + (n < N ? n : N - 1)) * K;
      const uint16_t* w1 = w + ((size_t)ew * N + (n + 1 < N ? n + 1 : N - 1)) * K;
      for (int kb = 0; kb < K; kb += 8 * 512) {
        u32x4 wa[8], wb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int kk = kb + u * 512 + lane * 8;
          if (kk < K) {
            // each weight is read once per call: non-temporal loads
            wa[u] = __builtin_nontemporal_load((const u32x4*)(w0 + kk));
            wb[u] = __builtin_nontemporal_load((const u32x4*)(w1 + kk));
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int kk = kb + u * 512 + lane * 8;
          if (kk < K) {
#pragma unroll
            for (int g = 0; g < DG; ++g) {
              if (g < ng) {
                const u32x4 xv = *(const u32x4*)(sx + g * K + kk);
                acc[0][g] += dot8(wa[u], xv);
                acc[1][g] += dot8(wb[u], xv);
              }
            }
          }
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int na = n + a;
        const float b = (bias && na < N) ? bf16_to_f32(bias[(size_t)ew * N + na]) : 0.0f;
#pragma unroll
        for (int g = 0; g < DG; ++g) {
          if (g < ng) {
            float v = wave_sum(acc[a][g]) + b;
            if (SILU && zout && lane == 0 && na < N)
              zout[(size_t)(r0 + g0 + g) * N + na] = (uint16_t)f32_to_bf16(v);
            if (SILU) v = silu_bf16(v);
            if constexpr (YQ) {
              if (lane == 0) sy[wave][rp + a][g] = v;
            } else if (lane == 0 && na < N)
              ((uint16_t*)out)[(size_t)(r0 + g0 + g) * N + na] = (uint16_t)f32_to_bf16(v);
          }
        }
      }
    }
    if constexpr (YQ) {
      // N is a multiple of 16 here, so all 4 features of every wave exist
      __syncthreads();
      if (lane == 0) {
        const size_t rb = yq_row_bytes(N);
#pragma unroll
        for (int g = 0; g < DG; ++g) {
          if (g < ng) {
            float mx = 0.0f;
#pragma unroll
            for (int f = 0; f < DRPW; ++f)
              mx = fmaxf(mx, fmaxf(fabsf(sy[wave][f][g]), fabsf(sy[wave ^ 1][f][g])));
            const int ex = yq_exponent(mx);
            unsigned char* row = (unsigned char*)out + (size_t)(r0 + g0 + g) * rb;
            u32x2 o;
            o[0] = ((uint32_t)yq_encode(sy[wave][0][g], ex) & 0xFFFFu) |
                   ((uint32_t)yq_encode(sy[wave][1][g], ex) << 16);
            o[1] = ((uint32_t)yq_encode(sy[wave][2][g], ex) & 0xFFFFu) |
                   ((uint32_t)yq_encode(sy[wave][3][g], ex) << 16);
            *(u32x2*)(row + (size_t)2 * nw) = o;
            if ((wave & 1) == 0) row[(size_t)2 * N + nw / kYBlock] = (unsigned char)(signed char)ex;
          }
        }
      }
    }
    __syncthreads();
  }
}
// ------------------------------------------------------------ dispatch ----
constexpr int kBM = 128;

template <int BN>
int launch_gemms_bf16(const uint16_t* x, const int32_t* sorted_token, const int32_t* offsets,
                      const int32_t* tile_start, const uint16_t* w1, const uint16_t* b1,
                      const uint16_t* w2, const uint16_t* b2, uint16_t* H, unsigned char* y, int E,
                      int d, int h, int mslots, uint16_t* zout, hipStream_t s) {
  hipLaunchKernelGGL((gemm_bf16<BN, kBM, true, true>), dim3(mslots * (h / BN)), dim3(256), 0, s, x,
                     sorted_token, offsets, tile_start, w1, b1, H, E, h, d, mslots, zout);
  hipLaunchKernelGGL((gemm_bf16<BN, kBM, false, false, true>), dim3(mslots * (d / BN)), dim3(256), 0, s,
                     H, sorted_token, offsets, tile_start, w2, b2, y, E, d, h, mslots,
                     (uint16_t*)nullptr);
  return launch_status();
}

bool use_decode(long rows, int E) { return rows <= 4L * E && rows <= 1024; }

// 256 x 256 DMA-ring tiles when experts average at least 192 rows, both
// widths tile by 256 and activation element offsets fit 31 bits.
bool ring_shapes(long rows, int T, int d, int h) {
  return (d % kBigBN) == 0 && (h % kBigBN) == 0 && (long)T * d < (1L << 31) &&
         rows * h < (1L << 31);
}
bool use_ring(long rows, int E, int T, int d, int h) {
  return rows >= 192L * E && ring_shapes(rows, T, d, h);
}
// 128-row persistent tiles for experts of fewer rows (above the decode range).
bool use_ring128(long rows, int E, int T, int d, int h) {
  return rows < 192L * E && ring_shapes(rows, T, d, h);
}

int launch_ring(const uint16_t* x, const int32_t* sorted_token, const int32_t* offsets, void* plan,
                const uint16_t* w1, const uint16_t* b1, const uint16_t* w2, const uint16_t* b2,
                uint16_t* H, unsigned char* y, float* part, uint16_t* zout, int E, int d, int h,
                long rows, hipStream_t s) {
  const int g1 = ffn_big_grid(rows, E, h, kBigBM), g2 = ffn_big_grid(rows, E, d, kBigBM);
  BigHdr* hdr = (BigHdr*)plan;
  BigWork* list1 = (BigWork*)((unsigned char*)plan + 256);
  BigWork* list2 = list1 + g1;
  const dim3 gr(kTailSlots * kReduceSlices);
  hipLaunchKernelGGL((big_plan<kBigBM, true>), dim3(ceil_div(g1 + g2, kMaxE)), dim3(kMaxE), 0, s,
                     offsets, E, big_xr(E), h / kBigBN, d / kRS, g1, d / kBigBN, h / kRS, g2, hdr,
                     list1, list2, sorted_token, (int32_t*)nullptr);
  hipLaunchKernelGGL((gemm_bf16_ring<kRingWaves, true, kEpiSilu>), dim3(g1), dim3(kRingWaves * 64),
                     0, s, x, sorted_token, list1, w1, b1, H, part, h, d, (size_t)h * d, 0,
                     (const uint16_t*)nullptr, zout);
  hipLaunchKernelGGL((big_tail_reduce<kBigRowsMax, kEpiSilu>), gr, dim3(256), 0, s, hdr, list1, b1, part,
                     H, h, (const uint16_t*)nullptr, zout);
  hipLaunchKernelGGL((gemm_bf16_ring<kRingWaves, false, kEpiBiasQ>), dim3(g2),
                     dim3(kRingWaves * 64), 0, s, H, sorted_token, list2, w2, b2, y, part, d, h,
                     (size_t)d * h, 0, (const uint16_t*)nullptr, (uint16_t*)nullptr);
  hipLaunchKernelGGL((big_tail_reduce<kBigRowsMax, kEpiBiasQ>), gr, dim3(256), 0, s, hdr + 1,
                     list2, b2, part, y, d, (const uint16_t*)nullptr, (uint16_t*)nullptr);
  return launch_status();
}

// Persistent DMA-ring GEMMs with BM-row tiles: one block per CU.
template <int BM>
int launch_pring(const uint16_t* x, const int32_t* sorted_token, const int32_t* offsets,
                 void* plan, const uint16_t* w1, const uint16_t* b1, const uint16_t* w2,
                 const uint16_t* b2, uint16_t* H, unsigned char* y, float* part, uint16_t* zout, int E,
                 int d, int h, int T, int k, long rows, hipStream_t s) {
  const int g1 = ffn_big_grid(rows, E, h, BM), g2 = ffn_big_grid(rows, E, d, BM);
  BigHdr* hdr = (BigHdr*)plan;
  BigWork* list1 = (BigWork*)((unsigned char*)plan + 256);
  BigWork* list2 = list1 + g1;
  const size_t tok_off = align_up(ffn_lists_bytes(rows, E, d, h), 256);
  int32_t* tok = (int32_t*)((unsigned char*)plan + tok_off);
  const long ntok = ffn_tok_entries(rows, E, BM);
  // the plan region must hold the lists and the table (H follows it)
  if ((size_t)(g1 + g2) * kWorkBytes + 256 > tok_off ||
      tok_off + (size_t)ntok * sizeof(int32_t) > ffn_plan_bytes(T, d, h, E, k))
    return MOE_ERR_WORKSPACE;
  const dim3 gr(kTailSlots * kReduceSlices);
  hipLaunchKernelGGL((big_plan<BM, false>), dim3(ceil_div(g1 + g2 + ntok, kMaxE)), dim3(kMaxE), 0,
                     s, offsets, E, 0, h / kBigBN, d / kRS, g1, d / kBigBN, h / kRS, g2, hdr, list1,
                     list2, sorted_token, tok);
  hipLaunchKernelGGL((gemm_bf16_pring<BM, true, true>), dim3(kTailSlots), dim3(512), 0, s, x, tok,
                     hdr, list1, w1, b1, H, part, h, d, zout);
  hipLaunchKernelGGL((big_tail_reduce<BM, kEpiSilu>), gr, dim3(256), 0, s, hdr, list1, b1, part, H, h,
                     (const uint16_t*)nullptr, zout);
  hipLaunchKernelGGL((gemm_bf16_pring<BM, false, false, true>), dim3(kTailSlots), dim3(512), 0, s,
                     H, (const int32_t*)nullptr, hdr + 1, list2, w2, b2, y, part, d, h,
                     (uint16_t*)nullptr);
  hipLaunchKernelGGL((big_tail_reduce<BM, kEpiBiasQ>), gr, dim3(256), 0, s, hdr + 1, list2, b2,
                     part, y, d, (const uint16_t*)nullptr, (uint16_t*)nullptr);
  return launch_status();
}

// Both FFN GEMMs through the weight-streaming kernel (H in the workspace).
int launch_decode(const uint16_t* x, const int32_t* sorted_token, const int32_t* offsets,
                  const uint16_t* w1, const uint16_t* b1, const uint16_t* w2, const uint16_t* b2,
                  uint16_t* H, unsigned char* y, int E, int d, int h, const int32_t* slot_of,
                  const int32_t* phase_of, int phase, uint16_t* zout, hipStream_t s) {
  const size_t lds1 = (size_t)DG * d * 2, lds2 = (size_t)DG * h * 2;
  const size_t lds_static = sizeof(float) * 4 * DRPW * DG;  // the kernel's sy
  if (lds1 + lds_static > 160 * 1024 || lds2 + lds_static > 160 * 1024) return MOE_ERR_UNSUPPORTED;
  if (lds1 > 65536 &&
      hipFuncSetAttribute((const void*)decode_bf16<true, true, false>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1) != hipSuccess)
    return MOE_ERR_LAUNCH;
  if (lds2 > 65536 &&
      hipFuncSetAttribute((const void*)decode_bf16<false, false, true>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2) != hipSuccess)
    return MOE_ERR_LAUNCH;
  hipLaunchKernelGGL((decode_bf16<true, true, false>), dim3(ceil_div(h, DRPB), E), dim3(256), lds1, s, x,
                     sorted_token, offsets, w1, b1, H, E, h, d, slot_of, phase_of, phase, zout);
  hipLaunchKernelGGL((decode_bf16<false, false, true>), dim3(ceil_div(d, DRPB), E), dim3(256), lds2, s,
                     (const uint16_t*)H, sorted_token, offsets, w2, b2, y, E, d, h, slot_of,
                     phase_of, phase, (uint16_t*)nullptr);
  return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace moe {
namespace {

// The grouped FFN with its hidden rows H at `hidden` (the workspace, or a
// caller buffer) and, when zout is not NULL, the pre-activations Z = W1 x +
// b1 written there too. Sizes and pointers are checked by the callers.
int grouped_ffn(const void* x, int dtype, int T, int d, int h, int E, int k,
                const int32_t* offsets, const int32_t* sorted_token, const void* w1,
                const void* b1, const void* w2, const void* b2, void* y_perm, void* ws,
                void* hidden, void* zout, hipStream_t s) {
  const long rows = (long)T * k;
  int32_t* tile_start = (int32_t*)ws;
  void* H = hidden;
  float* part = (float*)((unsigned char*)ws + ffn_plan_bytes(T, d, h, E, k) +
                         ffn_hidden_bytes(T, h, k));
  const int nonempty = (int)(rows < E ? rows : E);

  if (dtype == MOE_F32) {
    const int mslots = ceil_div(rows, FB) + nonempty;
    hipLaunchKernelGGL(build_tile_map, dim3(1), dim3(512), 0, s, offsets, E, FB, tile_start);
    hipLaunchKernelGGL((gemm_f32<true, true>), dim3(mslots * ceil_div(h, FB)), dim3(256), 0, s,
                       (const float*)x, sorted_token, offsets, tile_start, (const float*)w1,
                       (const float*)b1, (float*)H, E, h, d, mslots, (float*)zout);
    hipLaunchKernelGGL((gemm_f32<false, false>), dim3(mslots * ceil_div(d, FB)), dim3(256), 0, s,
                       (const float*)H, sorted_token, offsets, tile_start, (const float*)w2,
                       (const float*)b2, (float*)y_perm, E, d, h, mslots, (float*)nullptr);
    return launch_status();
  }

  const uint16_t* xb = (const uint16_t*)x;
  uint16_t* zb = (uint16_t*)zout;
  if (use_decode(rows, E)) {
    return launch_decode(xb, sorted_token, offsets, (const uint16_t*)w1, (const uint16_t*)b1,
                         (const uint16_t*)w2, (const uint16_t*)b2, (uint16_t*)H,
                         (unsigned char*)y_perm, E, d, h, nullptr, nullptr, 0, zb, s);
  }

  if (use_ring(rows, E, T, d, h))
    return launch_ring(xb, sorted_token, offsets, ws, (const uint16_t*)w1, (const uint16_t*)b1,
                       (const uint16_t*)w2, (const uint16_t*)b2, (uint16_t*)H, (unsigned char*)y_perm,
                       part, zb, E, d, h, rows, s);
  if (use_ring128(rows, E, T, d, h))
    return launch_pring<128>(xb, sorted_token, offsets, ws, (const uint16_t*)w1,
                             (const uint16_t*)b1, (const uint16_t*)w2, (const uint16_t*)b2,
                             (uint16_t*)H, (unsigned char*)y_perm, part, zb, E, d, h, T, k, rows, s);
  const int mslots = ceil_div(rows, kBM) + nonempty;
  hipLaunchKernelGGL(build_tile_map, dim3(1), dim3(512), 0, s, offsets, E, kBM, tile_start);
  if ((d % 128) == 0 && (h % 128) == 0)
    return launch_gemms_bf16<128>(xb, sorted_token, offsets, tile_start, (const uint16_t*)w1,
                                  (const uint16_t*)b1, (const uint16_t*)w2, (const uint16_t*)b2,
                                  (uint16_t*)H, (unsigned char*)y_perm, E, d, h, mslots, zb, s);
  return launch_gemms_bf16<64>(xb, sorted_token, offsets, tile_start, (const uint16_t*)w1,
                               (const uint16_t*)b1, (const uint16_t*)w2, (const uint16_t*)b2,
                               (uint16_t*)H, (unsigned char*)y_perm, E, d, h, mslots, zb, s);
}

int ffn_check(const void* x, int dtype, int T, int d, int h, int E, int k,
              const int32_t* offsets, const int32_t* sorted_token, const void* w1,
              const void* w2, const void* y_perm, const void* ws, size_t ws_bytes) {
  if (T < 0 || d < 1 || h < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  const long rows = (long)T * k;
  if (rows > 0x7FFFFFFFL) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_BF16 && ((d % 64) != 0 || (h % 64) != 0)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !offsets || !sorted_token || !w1 || !w2 || !y_perm) return MOE_ERR_INVALID;
  if (!ws || ws_bytes < ffn_ws(T, d, h, E, k)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_grouped_ffn(const void* x, int dtype, int T, int d, int h, int E, int k,
                               const int32_t* offsets, const int32_t* sorted_token, const void* w1,
                               const void* b1, const void* w2, const void* b2, void* y_perm,
                               void* ws, size_t ws_bytes, moe_stream_t stream) {
  const int st = ffn_check(x, dtype, T, d, h, E, k, offsets, sorted_token, w1, w2, y_perm, ws,
                           ws_bytes);
  if (st != MOE_OK || (long)T * k == 0) return st;
  MOE_DEBUG_CHECK((hipStream_t)stream, offsets, E, sorted_token, nullptr, T, k);
  void* H = (unsigned char*)ws + ffn_plan_bytes(T, d, h, E, k);
  return grouped_ffn(x, dtype, T, d, h, E, k, offsets, sorted_token, w1, b1, w2, b2, y_perm, ws,
                     H, nullptr, (hipStream_t)stream);
}

extern "C" int moe_grouped_ffn_train(const void* x, int dtype, int T, int d, int h, int E, int k,
                                     const int32_t* offsets, const int32_t* sorted_token,
                                     const void* w1, const void* b1, const void* w2,
                                     const void* b2, void* y_perm, void* z_perm, void* h_perm,
                                     void* ws, size_t ws_bytes, moe_stream_t stream) {
  const int st = ffn_check(x, dtype, T, d, h, E, k, offsets, sorted_token, w1, w2, y_perm, ws,
                           ws_bytes);
  if (st != MOE_OK || (long)T * k == 0) return st;
  if (!z_perm || !h_perm) return MOE_ERR_INVALID;
  MOE_DEBUG_CHECK((hipStream_t)stream, offsets, E, sorted_token, nullptr, T, k);
  return grouped_ffn(x, dtype, T, d, h, E, k, offsets, sorted_token, w1, b1, w2, b2, y_perm, ws,
                     h_perm, z_perm, (hipStream_t)stream);
}

extern "C" int moe_grouped_ffn_cached(const void* x, int dtype, int T, int d, int h, int E, int k,
                                      const int32_t* offsets, const int32_t* sorted_token,
                                      const int32_t* slot_of, const int32_t* phase_of, int phase,
                                      const void* w1, const void* b1, const void* w2,
                                      const void* b2, void* y_perm, void* ws, size_t ws_bytes,
                                      moe_stream_t stream) {
  if (T < 0 || d < 1 || h < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (dtype != MOE_BF16) return dtype == MOE_F32 ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  const long rows = (long)T * k;
  if (!use_decode(rows, E) && rows > 0) return MOE_ERR_UNSUPPORTED;
  if ((d % 64) != 0 || (h % 64) != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !offsets || !sorted_token || !slot_of || !phase_of || !w1 || !w2 || !y_perm)
    return MOE_ERR_INVALID;
  if (!ws || ws_bytes < ffn_ws(T, d, h, E, k)) return MOE_ERR_WORKSPACE;
  MOE_DEBUG_CHECK((hipStream_t)stream, offsets, E, sorted_token, nullptr, T, k);
  void* H = (unsigned char*)ws + ffn_plan_bytes(T, d, h, E, k);
  return launch_decode((const uint16_t*)x, sorted_token, offsets, (const uint16_t*)w1,
                       (const uint16_t*)b1, (const uint16_t*)w2, (const uint16_t*)b2,
                       (uint16_t*)H, (unsigned char*)y_perm, E, d, h, slot_of, phase_of, phase,
                       (uint16_t*)nullptr, (hipStream_t)stream);
}
