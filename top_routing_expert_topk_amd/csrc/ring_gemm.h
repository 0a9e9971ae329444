// 256 x 256 bf16 MFMA GEMM tiles fed by a global->LDS DMA ring, with the
// device-built work lists and the split-K tail reduction it runs on. Used
// by the grouped FFN (ffn.hip) and its backward pass (ffn_bwd.hip).
#pragma once

#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

// ---------------------------------- MFMA GEMM, 256 x 256 tiles, DMA ring --
// For experts with a few hundred rows or more. Block tile 256 weight rows x
// 256 permuted rows, eight waves (two per SIMD, so one wave's MFMAs cover the
// other's waits) in a 2 x 4 grid, each owning 128 x 64 of the tile as 4 x 2
// v_mfma_f32_32x32x16_bf16 tiles (128 accumulator floats per lane).
//
// v_mfma_f32_32x32x16_bf16: lane l supplies row l%32 and k-octet l/32 of each
// operand (A = 32 weight rows x 16 k, B = 16 k x 32 permuted rows) and
// receives D[n = 8*(v/4) + 4*(l/32) + v%4][row = l%32], v = 0..15, i.e. four
// runs of 4 consecutive output features of one row.
//
// Data path: direct global->LDS DMA (16 bytes per lane, no VGPR round trip)
// of full 128-byte row segments: one DMA instruction moves 8 rows x 64
// columns, touching 8 cache lines (32-column segments would touch 16 half
// lines for the same bytes, and the L1/L2 path serves requests, not bytes).
// A 64-column step of a tile needs four 16 KB blocks (weight rows 0-127 and
// 128-255, permuted rows 0-127 and 128-255), held in a ring of ten block slots
// (all 160 KB of LDS): block b of the tile's sequence (step b/4, part b%4)
// lives in slot b % 10. While step j is computed, step j+1 is landing and
// half of step j+2 is in flight. At the end of step j, once every wave's
// fragment reads of it have completed, two of its slots take the second
// half of step j+2 (the permuted rows); the other two take the first half of
// step j+3 (the weights), issued one block after each of the first two
// sub-steps of step j+1 rather than together at the step boundary, so the
// waves reach their MFMAs sooner after the barrier (DeepSeek-shaped FFN
// 4.52 -> 4.45 ms, Mixtral-shaped 1.88 -> 1.76-1.86 ms, same results bit
// for bit). Up to 1.5 steps (96 KB) are in flight.
// The ring barrier is an s_barrier with a compiler memory clobber: it keeps
// LDS accesses on their side without draining the DMA queue, which a
// workgroup fence would do.
//
// LDS rows are 128 bytes (8 chunks of 16 B); chunk c of row r sits at
// c ^ ((r >> 1) & 7). A ds_read_b128 is served 16 lanes (256 bytes) at a
// time, and 16 consecutive rows at one chunk then hit 16 distinct 16-byte
// bank groups. Lane l of a DMA instruction writes chunk slot l%8 of row l/8,
// so it fetches chunk (l%8) ^ swizzle(row).
constexpr int kBigBM = 256;          // permuted rows per tile
constexpr int kBigXR = kBigRowsMax - kBigBM;  // more rows an expert's last tile may take
// Taller last tiles are planned for layers of at least 32 experts. There each
// XCD's contiguous range of tiles spans several experts, and an expert's
// taller tiles replace tiles that would stream a whole weight panel for a few
// rows. With fewer experts an XCD's range is one or two experts, so all taller
// tiles of one expert (which keep one K step in flight instead of one and a
// half) land on the same XCD, and its CUs finish last.
constexpr int kBigXRMinExperts = 32;
inline int big_xr(int E) { return E >= kBigXRMinExperts ? kBigXR : 0; }
constexpr int kBigBN = kBigBNTile;   // weight rows (output features) per tile
constexpr int kRS = 64;              // K columns per step
constexpr int kRBlk = 128 * kRS;     // bf16 elements per block (16 KB)
constexpr int kRSlots = 10;
constexpr int kMaxSplit = 8;         // K ranges per tail tile
constexpr int kReduceSlices = 8;     // row slices per tail tile in the reduction
constexpr int kGroupN = 4;           // weight-row tiles per group of the tile order
constexpr int kRingWaves = 8;        // waves per 256 x 256 tile
static_assert(kBigBN == 256, "tile");

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// At most BASE + n vector memory operations outstanding, n in 0..8 (uniform).
template <int BASE>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n) {
    case 0: wait_vmcnt<BASE>(); break;
    case 1: wait_vmcnt<BASE + 1>(); break;
    case 2: wait_vmcnt<BASE + 2>(); break;
    case 3: wait_vmcnt<BASE + 3>(); break;
    case 4: wait_vmcnt<BASE + 4>(); break;
    case 5: wait_vmcnt<BASE + 5>(); break;
    case 6: wait_vmcnt<BASE + 6>(); break;
    case 7: wait_vmcnt<BASE + 7>(); break;
    default: wait_vmcnt<BASE + 8>(); break;
  }
}
// Workgroup barrier that the compiler may not move memory accesses across.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One 16-byte direct global->LDS load per lane; the LDS address is the
// wave-uniform base plus 16 * lane.
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
// The same with the non-temporal cache policy, for data read once per call.
__device__ __forceinline__ void dma16_nt(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 2);
}

__device__ __forceinline__ int swz128(int r, int c) { return c ^ ((r >> 1) & 7); }

// Scheduling hint for a sub-step: alternate one MFMA with one LDS fragment
// read NR times, then the remaining MFMAs, so the reads for the next
// sub-step hide behind this one's MFMAs instead of queueing up behind a
// single lgkmcnt(0) wait.
template <int NM, int NR>
__device__ __forceinline__ void interleave_mfma_reads() {
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
}

// Epilogues of a tile: out = acc + bias, SiLU(acc + bias), or acc * SiLU'(z)
// with z read from a second [rows][N] array (the backward of the activation),
// all three stored as bf16; kEpiBiasQ stores acc + bias in the block fixed
// point of moe_internal.h (the expert outputs Y of the forward: 2^-15 of the
// largest of every 8 consecutive features instead of bf16's 2^-9 of each).
constexpr int kEpiBias = 0;
constexpr int kEpiSilu = 1;
constexpr int kEpiDSilu = 2;
constexpr int kEpiBiasQ = 3;

// MFMA operand fragment of a K-major weight block in LDS (64 k-rows x 128
// features, 256-byte rows, chunk c of row k at c ^ 4 (k % 4)): lane l gets
// the 8 consecutive k (16 sub .. +15, octet l / 32) of feature 32 i + l % 32
// from two transpose loads of 4 k each. The block pointer is restrict: the
// ring's own waits order these reads after the DMA that filled the block, as
// for the plain fragment reads, and without alias information the compiler
// would drain every DMA in flight before each transpose load.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* __restrict__ blk, int sub, int i,
                                          int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int row = sub * 16 + 8 * (g >> 1) + (j >> 2);
  const int col = i * 32 + 16 * (g & 1) + 4 * (j & 3);
  const int off = row * 128 + (((col >> 3) ^ (4 * (j >> 2))) << 3) + (col & 4);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(blk + off));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(blk + off + 4 * 128));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One entry of a launch's work list: the block's tile and K range. The
// lists are built on the device by big_plan, so a GEMM block starts with one
// uniform load instead of searching the tile map.
struct alignas(16) BigWork {
  int e;           // expert, -1: no work for this block
  int row0, rows;  // permuted rows of the tile
  int n0;          // first output feature
  int kbeg, kend;  // K range in kRS-column steps
  int unit;        // fp32 partial slot of a split tail tile, -1 for a whole tile
  int ms;          // row block (index into the token table of the tile's rows)
};
static_assert(sizeof(BigWork) == kWorkBytes, "work entry size");
typedef const __attribute__((address_space(4))) uint32_t cu32;  // scalar-cache reads

// A work-list entry read through the scalar cache (its index is uniform).
struct WorkS {
  int e, row0, rows, n0, kbeg, kend, unit, ms;
};
__device__ __forceinline__ WorkS load_work(const BigWork* __restrict__ units, int idx) {
  cu32* p = (cu32*)(units + idx);
  WorkS u;
  u.e = __builtin_amdgcn_readfirstlane((int)p[0]);
  u.row0 = __builtin_amdgcn_readfirstlane((int)p[1]);
  u.rows = __builtin_amdgcn_readfirstlane((int)p[2]);
  u.n0 = __builtin_amdgcn_readfirstlane((int)p[3]);
  u.kbeg = __builtin_amdgcn_readfirstlane((int)p[4]);
  u.kend = __builtin_amdgcn_readfirstlane((int)p[5]);
  u.unit = __builtin_amdgcn_readfirstlane((int)p[6]);
  u.ms = __builtin_amdgcn_readfirstlane((int)p[7]);
  return u;
}

// Per launch: tiles = whole tiles + tail tiles; the `full` first tiles (a
// whole number of rounds over the kTailSlots resident blocks) run whole, the
// `tail` remaining ones are each cut into `split` K ranges so that the last
// round fills every CU.
struct BigHdr {
  int full, tail, split, tiles;
};

// Largest e with ts[e] <= v (ts in LDS, ts[0] = 0 <= v).
__device__ __forceinline__ int find_le(const int* ts, int E, int v) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] <= v) lo = mid; else hi = mid;
  }
  return lo;
}

// Work lists of both GEMMs of the FFN (N = nt * kBigBN features, nk K steps,
// BM permuted rows per tile; with xr > 0 an expert's last row block takes up
// to BM + xr rows, so an expert of BM + r rows, r <= xr, runs as one tile
// instead of a full one plus one of r rows that would stream the same
// weights for almost no work). Tile order: expert-major; inside an expert,
// groups of kGroupN weight-row tiles, inside a group the expert's row blocks.
// REMAP: entry b is the work of hardware block b, whole tiles dealt to the
// XCDs in contiguous ranges of that order (block b runs on XCD b % 8), so each
// XCD's L2 sees a few weight and row panels at a time. Otherwise entries are
// in that order (whole tiles, then the K ranges of the tail tiles) and the
// persistent kernel deals them out itself.
template <int BM, bool REMAP>
__global__ __launch_bounds__(512) void big_plan(const int32_t* __restrict__ offsets, int E, int xr,
                                                int nt1, int nk1, int g1, int nt2, int nk2,
                                                int g2, BigHdr* __restrict__ hdr,
                                                BigWork* __restrict__ list1,
                                                BigWork* __restrict__ list2,
                                                const int32_t* __restrict__ sorted_token,
                                                int32_t* __restrict__ tok_tab) {
  __shared__ int sc[2][kMaxE];
  __shared__ int ts[kMaxE + 1];
  const int x = threadIdx.x;  // blockDim == kMaxE
  int cur = 0;
  if (x < E) {
    const int c = offsets[x + 1] - offsets[x];
    sc[0][x] = c <= 0 ? 0 : max(1, (c - xr + BM - 1) / BM);
  } else {
    sc[0][x] = 0;
  }
  __syncthreads();
  for (int off = 1; off < kMaxE; off <<= 1) {
    const int v = sc[cur][x] + (x >= off ? sc[cur][x - off] : 0);
    sc[cur ^ 1][x] = v;
    cur ^= 1;
    __syncthreads();
  }
  ts[x + 1] = sc[cur][x];
  if (x == 0) ts[0] = 0;
  __syncthreads();

  const int i = blockIdx.x * kMaxE + x;
  if (i >= g1 + g2) {
    // token table: entry ms * BM + r = the token of row r of row block ms,
    // rows past the block's last one repeating it
    if (xr > 0 || !tok_tab) return;
    const int j = i - g1 - g2, ms = j / BM, r = j % BM;
    if (ms >= ts[E]) return;
    const int e = find_le(ts, E, ms);
    const int row0 = offsets[e] + (ms - ts[e]) * BM;
    const int rows = min(BM, offsets[e + 1] - row0);
    tok_tab[j] = sorted_token[row0 + (r < rows ? r : rows - 1)];
    return;
  }
  const bool second = i >= g1;
  const int b = second ? i - g1 : i;
  if (second && b >= g2) return;
  const int nt = second ? nt2 : nt1, nk = second ? nk2 : nk1;
  BigWork* list = second ? list2 : list1;

  BigHdr sp;
  sp.tiles = ts[E] * nt;
  sp.tail = sp.tiles % kTailSlots;
  sp.full = sp.tiles - sp.tail;
  sp.split = 1;
  if (sp.tail > 0) sp.split = max(1, min(min(kTailSlots / sp.tail, kMaxSplit), nk));
  if (b == 0) hdr[second ? 1 : 0] = sp;

  BigWork w;
  w.e = -1;
  w.row0 = w.rows = w.n0 = w.kbeg = w.kend = 0;
  w.unit = -1;
  w.ms = 0;
  int t = -1, p = 0, split = 1;
  if (b < sp.full) {
    const int per = sp.full >> 3;
    t = REMAP ? (b & 7) * per + (b >> 3) : b;
  } else if (b - sp.full < sp.tail * sp.split) {
    const int u = b - sp.full;
    split = sp.split;
    t = sp.full + u / split;
    p = u % split;
  }
  if (t >= 0) {
    const int e = find_le(ts, E, t / nt);  // experts own nt * (ts[e+1] - ts[e]) tiles
    const int mt = ts[e + 1] - ts[e];
    const int l = t - ts[e] * nt;
    const int g = l / (mt * kGroupN);
    const int gs = min(kGroupN, nt - g * kGroupN);
    const int l2 = l - g * mt * kGroupN;
    const int mi = l2 / gs, ni = g * kGroupN + l2 % gs;
    w.e = e;
    w.row0 = offsets[e] + mi * BM;
    w.rows = mi == mt - 1 ? offsets[e + 1] - w.row0 : BM;
    w.n0 = ni * kBigBN;
    w.kbeg = p * nk / split;
    w.kend = (p + 1) * nk / split;
    w.unit = split > 1 ? (t - sp.full) * split + p : -1;
    w.ms = ts[e] + mi;
  }
  list[b] = w;
}

// Epilogue of a 256 x 256 tile, each of NW waves holding 128 x (32 TM) of it
// as 4 x TM 32x32 MFMA accumulators; a taller last tile (rows > 256) adds
// rows 256..287, wave (wn, wm) holding features 128 wn + 32 wm .. +31 of them
// in accx. A split tail tile stores its fp32 partial [288 rows][256
// features] for big_tail_reduce; a whole tile adds the bias,
// applies SiLU if asked, rounds to bf16 into LDS (ot, the idle ring), and
// leaves with 16-byte stores of whole rows: 32 lanes write one 512-byte row.
// LDS rows are padded by 16 bytes so the 32 rows a wave writes at one feature
// offset spread over the banks. kEpiDSilu multiplies by SiLU'(z) in that last
// pass, where z arrives in the same 16-byte row chunks as the output leaves
// (the product is taken of the bf16-rounded accumulator). Output row of tile
// row m: e * ores + row0 + m. kEpiSilu with zout: the pre-activation
// acc + bias also leaves, to zout, in a first pass through the same staging.
// kEpiBiasQ (block fixed point) stages fp32 sums instead, in passes of 128
// rows, and adds the bias as the rows leave (see there).
template <int NW, int TM, int EPI>
__device__ __forceinline__ void big_store(f32x16 (&acc)[4][TM], const f32x16& accx,
                                          uint16_t* ot, size_t ot_bytes,
                                          const BigWork& wk, const uint16_t* __restrict__ bias,
                                          void* __restrict__ outv, float* __restrict__ part,
                                          int N, int ores, const uint16_t* __restrict__ zin,
                                          uint16_t* __restrict__ zout, int wn, int wm, int lane,
                                          int tid) {
  constexpr int BM = kBigBM, BN = kBigBN, TN = 4, WTN = 128, WTM = 32 * TM;
  const int ch = lane >> 5;
  const bool ext = wk.rows > BM;
  const int mx = BM + (lane & 31);  // the extra tile's row, and its features:
  auto nlx = [&](int q) { return wn * WTN + wm * 32 + 8 * q + 4 * ch; };
  if (wk.unit >= 0) {
    float* pp = part + (size_t)wk.unit * (kBigRowsMax * BN);
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * WTN + i * 32 + 8 * q + 4 * ch;
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const int m = wm * WTM + j * 32 + (lane & 31);
          *(f32x4*)(pp + m * BN + nl) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
      }
    if (ext)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4*)(pp + mx * BN + nlx(q)) =
            f32x4{accx[4 * q], accx[4 * q + 1], accx[4 * q + 2], accx[4 * q + 3]};
    return;
  }
  // The tile's 256 biases go to LDS once, at the start of the epilogue
  // (32 lanes, one 16-byte load each, behind the staging area): reading
  // them from global memory where each piece is used cost one round trip
  // per piece (and, after the first stores, a wait for those stores, which
  // share the vector memory counter), about 4 us per half tile.
  uint16_t* sbias = ot + ot_bytes / 2 - kBigBN;
  static_assert((size_t)kBigRowsMax * (BN + 8) * 2 <= (size_t)kRSlots * kRBlk * 2 - kBigBN * 2 &&
                    (size_t)kBigRowsMax * (BN / 2 + 4) * 4 <= (size_t)kRSlots * kRBlk * 2 - kBigBN * 2,
                "the staged tile and the biases must not overlap");
  auto load_bias = [&]() __attribute__((always_inline)) {
    if (tid < kBigBN / 8) {
      const u32x4 b = bias ? *(const u32x4*)(bias + (size_t)wk.e * N + wk.n0 + tid * 8)
                           : u32x4{0u, 0u, 0u, 0u};
      *(u32x4*)(sbias + tid * 8) = b;
    }
    __syncthreads();
  };
  auto bias4 = [&](int nl, float* bv) __attribute__((always_inline)) {
    const u32x2 bb = *(const u32x2*)(sbias + nl);
    bv[0] = bf16lo(bb[0]);
    bv[1] = bf16hi(bb[0]);
    bv[2] = bf16lo(bb[1]);
    bv[3] = bf16hi(bb[1]);
  };
  if constexpr (EPI == kEpiBiasQ) {
    // rows leave through LDS (the idle ring) in passes of 128 rows x all 256
    // features (then the up to 32 rows of a taller tile): the four waves that
    // hold a pass's rows, one per SIMD, stage them in fp32 (rows padded by 16
    // bytes, so the 32 rows a wave writes at one feature offset spread over
    // the banks), then 32 lanes per row add the bias, encode its 32 blocks
    // of 8 features and store its 512 bytes of mantissas and 32 exponent
    // bytes. Staging by weight halves instead (the four waves of a half sit
    // on two SIMDs) made each staging pass about 1 us longer. The staging
    // loop has no reads: with one (a bias read per run) each of its LDS waits
    // also waited for the previous run's writes.
    unsigned char* out = (unsigned char*)outv;
    const size_t rb = yq_row_bytes(N);
    float* st = (float*)ot;
    constexpr int FSTR = BN + 4;  // LDS row stride in floats
    static_assert(128 * FSTR * 4 <= (size_t)kRSlots * kRBlk * 2 - kBigBN * 2,
                  "a staged pass and the biases must not overlap");
    static_assert(NW == 8 && WTM == 64, "a pass is the rows of two 64-row wave groups");
    lds_barrier();  // every wave is done reading the ring
    load_bias();
    const int bl = tid & 31;  // this thread's block of 8 features
    const u32x4 bb = *(const u32x4*)(sbias + bl * 8);
    const long r0 = (long)wk.e * ores + wk.row0;
    const int npass = ext ? 3 : 2;
#pragma unroll 1
    for (int pp = 0; pp < npass; ++pp) {
      if (pp < 2) {
        if ((wm >> 1) == pp) {
#pragma unroll
          for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int nl = wn * WTN + i * 32 + 8 * q + 4 * ch;
#pragma unroll
              for (int j = 0; j < TM; ++j) {
                const int m = (wm & 1) * WTM + j * 32 + (lane & 31);  // row within the pass
                *(f32x4*)(st + m * FSTR + nl) =
                    f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                          acc[i][j][4 * q + 3]};
              }
            }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(f32x4*)(st + (lane & 31) * FSTR + nlx(q)) =
              f32x4{accx[4 * q], accx[4 * q + 1], accx[4 * q + 2], accx[4 * q + 3]};
      }
      __syncthreads();
      const int prow0 = pp * 128, prows = min(pp < 2 ? 128 : kBigXR, wk.rows - prow0);
#pragma unroll 2
      for (int m = tid >> 5; m < prows; m += NW * 2) {
        const f32x4 a = *(const f32x4*)(st + m * FSTR + bl * 8);
        const f32x4 b = *(const f32x4*)(st + m * FSTR + bl * 8 + 4);
        const float v[8] = {a[0] + bf16lo(bb[0]), a[1] + bf16hi(bb[0]), a[2] + bf16lo(bb[1]),
                            a[3] + bf16hi(bb[1]), b[0] + bf16lo(bb[2]), b[1] + bf16hi(bb[2]),
                            b[2] + bf16lo(bb[3]), b[3] + bf16hi(bb[3])};
        yq_store8(out, rb, N, r0 + prow0 + m, wk.n0 + bl * 8, v);
      }
      __syncthreads();
    }
    return;
  }
  uint16_t* out = (uint16_t*)outv;
  constexpr int OSTR = BN + 8;  // LDS row stride in bf16 elements
  constexpr int CPR = BN / 8;   // 16-byte chunks per row
  lds_barrier();  // every wave is done reading the ring
  load_bias();
  if (EPI == kEpiSilu && zout) {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * WTN + i * 32 + 8 * q + 4 * ch;
        float bv[4];
        bias4(wn * WTN + i * 32 + 8 * q + 4 * ch, bv);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const int m = wm * WTM + j * 32 + (lane & 31);
          u32x2 o;
          o[0] = pack_bf16x2(acc[i][j][4 * q] + bv[0], acc[i][j][4 * q + 1] + bv[1]);
          o[1] = pack_bf16x2(acc[i][j][4 * q + 2] + bv[2], acc[i][j][4 * q + 3] + bv[3]);
          *(u32x2*)(ot + m * OSTR + nl) = o;
        }
      }
    }
    if (ext)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float bv[4];
        bias4(nlx(q), bv);
        u32x2 o;
        o[0] = pack_bf16x2(accx[4 * q] + bv[0], accx[4 * q + 1] + bv[1]);
        o[1] = pack_bf16x2(accx[4 * q + 2] + bv[2], accx[4 * q + 3] + bv[3]);
        *(u32x2*)(ot + mx * OSTR + nlx(q)) = o;
      }
    __syncthreads();
    auto zrow = [&](int c) __attribute__((always_inline)) {
      const int m = c / CPR, cc = c % CPR;
      if (m < wk.rows)
        *(u32x4*)(zout + (size_t)(wk.row0 + m) * N + wk.n0 + cc * 8) =
            *(const u32x4*)(ot + m * OSTR + cc * 8);
    };
#pragma unroll 4
    for (int c = tid; c < BM * CPR; c += NW * 64) zrow(c);
    if (ext)
      for (int c = BM * CPR + tid; c < kBigRowsMax * CPR; c += NW * 64) zrow(c);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TN; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = wn * WTN + i * 32 + 8 * q + 4 * ch;
      float bv[4];
      bias4(wn * WTN + i * 32 + 8 * q + 4 * ch, bv);
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = wm * WTM + j * 32 + (lane & 31);
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[u] = acc[i][j][4 * q + u] + bv[u];
          if (EPI == kEpiSilu) v[u] = silu_bf16(v[u]);
        }
        u32x2 o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        *(u32x2*)(ot + m * OSTR + nl) = o;
      }
    }
  }
  if (ext)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float bv[4], v[4];
      bias4(nlx(q), bv);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = accx[4 * q + u] + bv[u];
        if (EPI == kEpiSilu) v[u] = silu_bf16(v[u]);
      }
      u32x2 o;
      o[0] = pack_bf16x2(v[0], v[1]);
      o[1] = pack_bf16x2(v[2], v[3]);
      *(u32x2*)(ot + mx * OSTR + nlx(q)) = o;
    }
  __syncthreads();
  auto orow = [&](int c) __attribute__((always_inline)) {
    const int m = c / CPR, cc = c % CPR;
    if (m < wk.rows) {
      u32x4 o = *(const u32x4*)(ot + m * OSTR + cc * 8);
      if (EPI == kEpiDSilu) {
        const u32x4 z = *(const u32x4*)(zin + (size_t)(wk.row0 + m) * N + wk.n0 + cc * 8);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[u] = pack_bf16x2(bf16lo(o[u]) * silu_grad(bf16lo(z[u])),
                             bf16hi(o[u]) * silu_grad(bf16hi(z[u])));
      }
      *(u32x4*)(out + ((size_t)wk.e * ores + wk.row0 + m) * N + wk.n0 + cc * 8) = o;
    }
  };
#pragma unroll 4
  for (int c = tid; c < BM * CPR; c += NW * 64) orow(c);
  if (ext)
    for (int c = BM * CPR + tid; c < kBigRowsMax * CPR; c += NW * 64) orow(c);
}

// out[row][n] = epilogue(sum_k act[src(row)][k] w[e][n][k]): act rows and
// weight rows are K-contiguous with row stride K (the work item's K range
// may be a part of it); src(row) = sorted_token[row] (GATHER) or row; expert
// e's weights start at w + e * wes; output rows as in big_store.
//
// WT: the weights are stored K-major instead, w[e][k][n] with rows of N
// features, as when a product runs through a weight matrix in the direction
// opposite to the forward's. The DMA then moves 64 k-rows x 128 features
// per 16 KB block (256-byte LDS rows, 16-byte chunk c of row k at
// c ^ 4 (k % 4)), and the weight fragments come from LDS transpose loads:
// ds_read_b64_tr_b16 gives each lane of a 16-lane group one feature of a 4 k
// x 16 feature tile (lane j of the group addresses row j / 4, features
// 4 (j % 4) .. +3, and receives the 4 k of feature j), so two of them make
// the 8 consecutive k an MFMA operand lane holds. The 32 lanes of a half
// wave read 64 bytes of each of four rows, which the swizzle spreads over
// all 256 bytes of the LDS banks (the plain layout would put the four rows
// on the same banks).
template <int NW, bool GATHER, int EPI, bool WT = false>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_ring(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ sorted_token,
    const BigWork* __restrict__ work, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ bias, void* __restrict__ out, float* __restrict__ part, int N,
    int K, size_t wes, int ores, const uint16_t* __restrict__ zin, uint16_t* __restrict__ zout) {
  constexpr int BM = kBigBM, BN = kBigBN;
  constexpr int WM = NW / 2;          // waves along the permuted rows (2 along the weight rows)
  constexpr int TN = 4, TM = 8 / WM;  // 32x32 MFMA tiles per wave
  constexpr int WTM = 32 * TM;        // permuted rows per wave
  constexpr int IPB = 16 / NW;        // DMA instructions per wave per 16 KB block
  static_assert(NW == 4 || NW == 8, "waves");
  __shared__ __align__(1024) uint16_t ring[kRSlots * kRBlk];
  static_assert((size_t)kBigRowsMax * (BN + 8) * 2 <= sizeof(ring), "output tile must fit the ring");
  static_assert((size_t)kBigRowsMax * (BN / 2 + 4) * 4 <= sizeof(ring),
                "half an output tile in fp32 must fit the ring");

  const BigWork wk = work[blockIdx.x];
  if (wk.e < 0) return;
  const int e = wk.e, row0 = wk.row0, rows = wk.rows, n0 = wk.n0, kbeg = wk.kbeg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Waves alternate along the weight rows, so the waves holding the first
  // permuted rows sit on different SIMDs (wave w runs on SIMD w % 4).
  const int wn = wave % 2, wm = wave / 2;
  // Tiles with few rows (an expert's last row block) skip the work of rows
  // past the last: a wave whose permuted rows are all past it issues no
  // MFMAs, and DMA instructions whose 8 rows are all past it are not issued.
  const bool active = wm * WTM < rows;
  auto b_live = [&](int q, int i) { return (q - 2) * 128 + i * NW * 8 + wave * 8 < rows; };
  int nbi = 0;  // activation DMA instructions this wave issues per step
#pragma unroll
  for (int q = 2; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < IPB; ++i) nbi += b_live(q, i) ? 1 : 0;

  // part q of a step: 0/1 weight rows 0-127 / 128-255, 2/3 permuted rows 0-127 /
  // 128-255; each wave moves row groups (i * NW + wave) * 8 .. +7, i < IPB.
  // Weight rows are one per-lane base plus a uniform row offset; activation
  // rows are gathered, kept as 32-bit element offsets (R * K < 2^31 is
  // checked on the host). The swizzle depends on r only through (r >> 1) & 7,
  // which the uniform offsets (multiples of 8 rows) leave unchanged.
  const int r0 = wave * 8 + (lane >> 3);
  const int c0 = swz128(r0, lane & 7) * 8;
  // WT: this lane moves k-row (lane / 16) of each 4-row DMA group, chunk
  // slot lane % 16, which holds feature chunk (lane % 16) ^ 4 ((lane / 16) % 4)
  const int tchunk = (((lane & 15) ^ (4 * (lane >> 4))) << 3);
  const uint16_t* wbase =
      WT ? w + (size_t)e * wes + (size_t)(lane >> 4) * N + n0 + tchunk
         : w + (size_t)e * wes + (size_t)(n0 + r0) * K + c0;
  uint32_t boff[2][IPB];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int pr = q * 128 + i * NW * 8 + r0;
      const int rr = row0 + (pr < rows ? pr : rows - 1);
      const uint32_t tok = GATHER ? (uint32_t)sorted_token[rr] : (uint32_t)rr;
      boff[q][i] = tok * (uint32_t)K + c0;
    }
  auto issue = [&](auto qc, int step, int slot) {
    constexpr int q = decltype(qc)::value;
    const int koff = (kbeg + step) * kRS;
    uint16_t* dst = ring + slot * kRBlk;
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      if (q >= 2 && !b_live(q, i)) continue;
      const uint16_t* g;
      if constexpr (WT)
        g = q < 2 ? wbase + (size_t)(koff + (i * NW + wave) * 4) * N + q * 128
                  : act + boff[q & 1][i] + koff;
      else
        g = q < 2 ? wbase + (size_t)(q * 128 + i * NW * 8) * K + koff
                  : act + boff[q & 1][i] + koff;
      dma16(g, dst + (i * NW + wave) * 8 * kRS);
    }
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x16{};

  const int ns = wk.kend - kbeg;
  if (rows > BM) {
    // A taller last tile: rows 256 .. rows-1 (at most 32) ride along in the
    // same weight stream. The ring becomes two step buffers of four parts
    // (weights 0-127, 128-255: 16 KB each; rows 0-127: 16 KB; rows 128-287:
    // 20 KB, 160 LDS rows), i.e. 136 KB, so a step is in flight while one is
    // computed; part p of a step always lands in the same place, which lets
    // the parts differ in size. Each wave adds one 32x32 MFMA tile: the extra
    // rows x its weight slice 128 wn + 32 wm .. +31, whose A fragment is one
    // more LDS read (two transpose reads for K-major weights).
    constexpr int kPW = 128 * kRS;              // elements of a 128-row part
    constexpr int kP3 = (128 + kBigXR) * kRS;   // elements of the tall part
    constexpr int kBuf = 3 * kPW + kP3;
    constexpr int kN3 = (128 + kBigXR) / 8;     // DMA instructions of the tall part
    static_assert(2 * kBuf * 2 <= (int)sizeof(ring), "two step buffers must fit");
    static_assert(NW == 8 && kN3 <= 3 * NW, "tall-part DMA mapping");
    uint32_t b3[3];  // this lane's rows of the tall part (clamped to the tile)
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int pr = 128 + (i * NW + wave) * 8 + (lane >> 3);
      const int rr = row0 + (pr < rows ? pr : rows - 1);
      const uint32_t tok = GATHER ? (uint32_t)sorted_token[rr] : (uint32_t)rr;
      b3[i] = tok * (uint32_t)K + c0;
    }
    // this wave's DMA instructions per step: 2 IPB (weights) + IPB (rows
    // 0-127) + its share of the kN3 instructions of the tall part
    const int n3 = (wave < kN3 - 2 * NW) ? 3 : 2;
    auto issue_step = [&](int step) __attribute__((always_inline)) {
      const int koff = (kbeg + step) * kRS;
      uint16_t* buf = ring + (step & 1) * kBuf;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < IPB; ++i)
          dma16(WT ? wbase + (size_t)(koff + (i * NW + wave) * 4) * N + q * 128
                   : wbase + (size_t)(q * 128 + i * NW * 8) * K + koff,
                buf + q * kPW + (i * NW + wave) * 8 * kRS);
#pragma unroll
      for (int i = 0; i < IPB; ++i)
        dma16(act + boff[0][i] + koff, buf + 2 * kPW + (i * NW + wave) * 8 * kRS);
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (i < n3) dma16(act + b3[i] + koff, buf + 3 * kPW + (i * NW + wave) * 8 * kRS);
    };
    const int ch = lane >> 5;
    // this wave's row fragments: rows wm*64 + 32 j + lane%32, in part 2 or 3
    const int bpart = (wm * WTM) >= 128 ? 3 : 2, brow = (wm * WTM) & 127;
    // FX[0]: rows 256 + lane%32 (B); FX[1]: weight rows 32 wm + lane%32 of
    // this wave's half (A)
    bf16x8 fa0[4], fb0[2], fx0[2], fa1[4], fb1[2], fx1[2];
    f32x16 accx = f32x16{};
#define MOE_XRD(step, sub, FA, FB, FX)                                                     \
    do {                                                                                   \
      const uint16_t* bb_ = ring + ((step) & 1) * kBuf;                                    \
      const uint16_t* wb_ = bb_ + wn * kPW;                                                \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
        if constexpr (WT) {                                                                \
          FA[i] = tr_frag(wb_, (sub), i, lane);                                            \
        } else {                                                                           \
          const int r = i * 32 + (lane & 31);                                              \
          FA[i] = *(const bf16x8*)(wb_ + r * kRS + swz128(r, 2 * (sub) + ch) * 8);         \
        }                                                                                  \
      }                                                                                    \
      _Pragma("unroll") for (int jj = 0; jj < 2; ++jj) {                                   \
        const int r = brow + jj * 32 + (lane & 31);                                        \
        FB[jj] = *(const bf16x8*)(bb_ + bpart * kPW + r * kRS + swz128(r, 2 * (sub) + ch) * 8); \
      }                                                                                    \
      {                                                                                    \
        const int r = 128 + (lane & 31);                                                   \
        FX[0] = *(const bf16x8*)(bb_ + 3 * kPW + r * kRS + swz128(r, 2 * (sub) + ch) * 8); \
      }                                                                                    \
      if constexpr (WT) {                                                                  \
        FX[1] = tr_frag(wb_, (sub), wm, lane);                                             \
      } else {                                                                             \
        const int r = wm * 32 + (lane & 31);                                               \
        FX[1] = *(const bf16x8*)(wb_ + r * kRS + swz128(r, 2 * (sub) + ch) * 8);           \
      }                                                                                    \
    } while (0)
#define MOE_XMM(FA, FB, FX)                                                                \
    do {                                                                                   \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                        \
      _Pragma("unroll") for (int jj = 0; jj < 2; ++jj)                                     \
        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i], FB[jj], acc[i][jj], 0, 0, 0); \
      accx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FX[1], FX[0], accx, 0, 0, 0);         \
    } while (0)
    issue_step(0);
    if (ns > 1) issue_step(1);
    // step 0 landed: step 1 may be in flight
    if (ns > 1) wait_vmcnt_le<3 * IPB>(n3); else wait_vmcnt<0>();
    lds_barrier();
    MOE_XRD(0, 0, fa0, fb0, fx0);
    // LDS reads paired with the 9 MFMAs of a sub-step by the scheduling hint
    constexpr int kXR = WT ? 9 : 8;
    for (int j = 0; j < ns; ++j) {
      MOE_XRD(j, 1, fa1, fb1, fx1);
      MOE_XMM(fa0, fb0, fx0);
      interleave_mfma_reads<9, kXR>();
      MOE_XRD(j, 2, fa0, fb0, fx0);
      MOE_XMM(fa1, fb1, fx1);
      interleave_mfma_reads<9, kXR>();
      MOE_XRD(j, 3, fa1, fb1, fx1);
      MOE_XMM(fa0, fb0, fx0);
      interleave_mfma_reads<9, kXR>();
      if (j + 1 < ns) {
        // step j+1 landed, and this wave's reads of step j are done before
        // its buffer takes step j+2
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        lds_barrier();
        if (j + 2 < ns) issue_step(j + 2);
        MOE_XRD(j + 1, 0, fa0, fb0, fx0);
      }
      MOE_XMM(fa1, fb1, fx1);
      interleave_mfma_reads<9, kXR>();
    }
#undef MOE_XRD
#undef MOE_XMM
    big_store<NW, TM, EPI>(acc, accx, ring, sizeof(ring), wk, bias, out, part, N, ores, zin,
                           zout, wn, wm, lane, tid);
    return;
  }
  // blocks 0..9: steps 0 and 1, and the weight half of step 2
#pragma unroll
  for (int st = 0; st < 2; ++st)
    if (st < ns) {
      issue(Q0{}, st, 4 * st);
      issue(Q1{}, st, 4 * st + 1);
      issue(Q2{}, st, 4 * st + 2);
      issue(Q3{}, st, 4 * st + 3);
    }
  if (2 < ns) {
    issue(Q0{}, 2, 8);
    issue(Q1{}, 2, 9);
  }

  const int ch = lane >> 5;
  // LDS fragment reads paired with MFMAs by the scheduling hint (the
  // transpose path issues two reads per weight fragment)
  constexpr int kNR = WT ? TN * TM : TN + TM;
  const int bq = (wm * WTM) >> 7;      // the permuted-row block this wave reads
  const int br = (wm * WTM) & 127;     // its first row inside that block
  bf16x8 f0a[TN], f0b[TM], f1a[TN], f1b[TM];
  int sa, sb;  // slots of this wave's weight block and permuted-row block in the current step
#define MOE_SLOTS(step)                                    \
  do {                                                     \
    const int b_ = (4 * (step)) % kRSlots;                 \
    const int a_ = b_ + wn, c_ = b_ + 2 + bq;              \
    sa = a_ < kRSlots ? a_ : a_ - kRSlots;                 \
    sb = c_ < kRSlots ? c_ : c_ - kRSlots;                 \
  } while (0)
#define MOE_RD(sub, FA, FB)                                                            \
  if constexpr (ACT) {                                                                 \
    const uint16_t* sa_ = ring + sa * kRBlk;                                           \
    const uint16_t* sb_ = ring + sb * kRBlk;                                           \
    _Pragma("unroll") for (int i = 0; i < TN; ++i) {                                   \
      if constexpr (WT) {                                                              \
        FA[i] = tr_frag(sa_, (sub), i, lane);                                          \
      } else {                                                                         \
        const int r = i * 32 + (lane & 31);                                            \
        FA[i] = *(const bf16x8*)(sa_ + r * kRS + swz128(r, 2 * (sub) + ch) * 8);       \
      }                                                                                \
    }                                                                                  \
    _Pragma("unroll") for (int j = 0; j < TM; ++j) {                                   \
      const int r = br + j * 32 + (lane & 31);                                         \
      FB[j] = *(const bf16x8*)(sb_ + r * kRS + swz128(r, 2 * (sub) + ch) * 8);         \
    }                                                                                  \
  }
#define MOE_MM(FA, FB)                                                                 \
  do {                                                                                 \
    if constexpr (ACT)                                                                 \
    _Pragma("unroll") for (int i = 0; i < TN; ++i)                                     \
    _Pragma("unroll") for (int j = 0; j < TM; ++j)                                     \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i], FB[j], acc[i][j], 0, 0, 0); \
  } while (0)

  // step 0 landed: the blocks of steps 1 and 2 may still be in flight, i.e.
  // this wave's DMAs of step 1 (both weight halves and its nbi activation
  // instructions) and of the weight half of step 2
  if (ns > 2) wait_vmcnt_le<4 * IPB>(nbi); else if (ns > 1) wait_vmcnt_le<2 * IPB>(nbi); else wait_vmcnt<0>();
  lds_barrier();
  // the loop twice over: with MFMAs for waves that own live rows, without
  // for the others (barriers and DMA issue are the same)
  auto main_loop = [&](auto act_c) {
  constexpr bool ACT = decltype(act_c)::value;
  MOE_SLOTS(0);
  MOE_RD(0, f0a, f0b);
  for (int j = 0; j < ns; ++j) {
    // the weight half of step j+2 goes into two of step j-1's slots, one
    // 16 KB block after each of the first two sub-steps (see the issue order
    // above the kernel)
    const int pb = (4 * (j + kRSlots - 1)) % kRSlots;
    const int pb2 = pb + 2 < kRSlots ? pb + 2 : pb + 2 - kRSlots;
    const int pb3 = pb + 3 < kRSlots ? pb + 3 : pb + 3 - kRSlots;
    MOE_RD(1, f1a, f1b);
    MOE_MM(f0a, f0b);
    if constexpr (ACT) interleave_mfma_reads<TN * TM, kNR>();
    if (j >= 1 && j + 2 < ns) issue(Q0{}, j + 2, pb2);
    MOE_RD(2, f0a, f0b);
    MOE_MM(f1a, f1b);
    if constexpr (ACT) interleave_mfma_reads<TN * TM, kNR>();
    if (j >= 1 && j + 2 < ns) issue(Q1{}, j + 2, pb3);
    MOE_RD(3, f1a, f1b);
    MOE_MM(f0a, f0b);
    if constexpr (ACT) interleave_mfma_reads<TN * TM, kNR>();
    if (j + 1 < ns) {
      // step j+1 landed (only the weight half of step j+2, issued during
      // this step, may be in flight), and this wave's reads of step j are
      // done before its slots are refilled
      if (j + 2 < ns) wait_vmcnt<2 * IPB>(); else wait_vmcnt<0>();
      wait_lgkmcnt0();
      lds_barrier();
      const int b0 = (4 * j) % kRSlots;
      const int b1 = b0 + 1 < kRSlots ? b0 + 1 : b0 + 1 - kRSlots;
      if (j + 2 < ns) {
        issue(Q2{}, j + 2, b0);
        issue(Q3{}, j + 2, b1);
      }
    }
    // the first fragments of step j+1 (after the last step these read stale
    // slots into registers nobody uses)
    MOE_SLOTS(j + 1);
    MOE_RD(0, f0a, f0b);
    MOE_MM(f1a, f1b);
    if constexpr (ACT) interleave_mfma_reads<TN * TM, kNR>();
  }
  };
  if (active) main_loop(std::true_type{});
  else main_loop(std::false_type{});
#undef MOE_SLOTS
#undef MOE_RD
#undef MOE_MM

  const f32x16 accx = f32x16{};  // no extra rows on this path
  big_store<NW, TM, EPI>(acc, accx, ring, sizeof(ring), wk, bias, out, part, N, ores, zin, zout, wn, wm,
                         lane, tid);
}


// Tail tiles: out = epilogue(sum_p partial[p] + bias), partials summed in
// order of their K-range, so the result does not depend on timing.
// kReduceSlices blocks per tail tile, each over BM/8 rows; a thread owns 8
// consecutive features of every 8th row of its slice.
template <int BM, int EPI>
__global__ __launch_bounds__(256) void big_tail_reduce(const BigHdr* __restrict__ hdr,
                                                       const BigWork* __restrict__ work,
                                                       const uint16_t* __restrict__ bias,
                                                       const float* __restrict__ part,
                                                       void* __restrict__ out, int N,
                                                       const uint16_t* __restrict__ zin,
                                                       uint16_t* __restrict__ zout) {
  const BigHdr sp = *hdr;
  const int tt = blockIdx.x / kReduceSlices, slice = blockIdx.x % kReduceSlices;
  if (tt >= sp.tail || sp.split < 2) return;
  const BigWork tile = work[sp.full + tt * sp.split];  // the tile's first K range
  const int nl = (threadIdx.x & 31) * 8;
  float bv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    bv[u] = bias ? bf16_to_f32(bias[(size_t)tile.e * N + tile.n0 + nl + u]) : 0.0f;
  constexpr int RS = BM / kReduceSlices;
  const float* base = part + (size_t)tt * sp.split * (BM * kBigBN);
  const int mend = min(tile.rows, (slice + 1) * RS);
  for (int m = slice * RS + (threadIdx.x >> 5); m < mend; m += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = 0.0f;
    for (int p = 0; p < sp.split; ++p) {
      const float* src = base + (size_t)p * (BM * kBigBN) + m * kBigBN + nl;
      const f32x4 lo = *(const f32x4*)src, hi = *(const f32x4*)(src + 4);
      v[0] += lo[0]; v[1] += lo[1]; v[2] += lo[2]; v[3] += lo[3];
      v[4] += hi[0]; v[5] += hi[1]; v[6] += hi[2]; v[7] += hi[3];
    }
    if constexpr (EPI == kEpiBiasQ) {
      float y8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) y8[u] = v[u] + bv[u];
      yq_store8((unsigned char*)out, yq_row_bytes(N), N, tile.row0 + m, tile.n0 + nl, y8);
      continue;
    }
    u32x4 o, z, pre;
    if (EPI == kEpiDSilu) z = *(const u32x4*)(zin + (size_t)(tile.row0 + m) * N + tile.n0 + nl);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a = v[2 * q] + bv[2 * q], c = v[2 * q + 1] + bv[2 * q + 1];
      pre[q] = pack_bf16x2(a, c);
      if (EPI == kEpiSilu) {
        a = silu_bf16(a);
        c = silu_bf16(c);
      } else if (EPI == kEpiDSilu) {
        a *= silu_grad(bf16lo(z[q]));
        c *= silu_grad(bf16hi(z[q]));
      }
      o[q] = pack_bf16x2(a, c);
    }
    *(u32x4*)((uint16_t*)out + (size_t)(tile.row0 + m) * N + tile.n0 + nl) = o;
    if (EPI == kEpiSilu && zout) *(u32x4*)(zout + (size_t)(tile.row0 + m) * N + tile.n0 + nl) = pre;
  }
}


}  // namespace
}  // namespace moe
