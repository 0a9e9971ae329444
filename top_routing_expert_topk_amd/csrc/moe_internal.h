// Internal helpers shared by the libmoe.so translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- limits of this build --------------------------------------------------
constexpr int kMaxE = 512;  // experts per layer
constexpr int kMaxK = 16;   // top-k

// ---- vector types ----------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));  // MFMA bf16 operand
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Low and high bf16 of a packed pair.
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (inputs are finite by contract): the
// conversion lowers to gfx950's v_cvt_pk_bf16_f32, two values per
// instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// SiLU from the hardware exp2 and reciprocal (about 1e-7 relative error), for
// results that are rounded to bf16 right after.
__device__ __forceinline__ float silu_bf16(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// d/dz SiLU(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z); same hardware exp2
// and reciprocal as silu_bf16.
__device__ __forceinline__ float silu_grad(float z) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
  return s * (1.0f + z * (1.0f - s));
}

// ---- expert outputs of bf16 layers (block fixed point) ----------------------
// Row r of y_perm takes moe_yq_row_bytes(d) bytes: d int16 mantissas, then
// one int8 exponent per block of 8 consecutive features (padded to 16
// bytes). A block with largest magnitude m, 2^e <= m < 2^(e+1), stores each
// value as round(v 2^(14-e)) (|.| <= 32767) with exponent e, and reads back
// exactly q 2^(e-14): the error is at most 2^(e-15) <= m 2^-15 (2^-14 m for a
// value clamped at the top), against 2^-9 |v| for a bf16 value, in 2.125
// bytes per element instead of fp32's 4. Blocks below the normal range use
// e = -127.
constexpr int kYBlock = 8;
__host__ __device__ inline size_t yq_row_bytes(int d) { return MOE_YQ_ROW_BYTES(d); }
__device__ __forceinline__ int yq_exponent(float maxabs) {
  if (!(maxabs >= 1.17549435e-38f)) return -127;  // zero, or below the normal range
  return (int)((__float_as_uint(maxabs) >> 23) & 0xFFu) - 127;
}
__device__ __forceinline__ int yq_encode(float v, int e) {
  const float s = __builtin_rintf(__builtin_ldexpf(v, 14 - e));
  return (int)fminf(fmaxf(s, -32767.0f), 32767.0f);
}
__device__ __forceinline__ float yq_decode(int q, int e) {
  return __builtin_ldexpf((float)q, e - 14);
}
// Eight features of one row: mantissas as 16 bytes and the block exponent.
__device__ __forceinline__ void yq_encode8(const float* v, u32x4& mant, int& e) {
  float m = 0.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf(v[u]));
  e = yq_exponent(m);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    mant[u] = ((uint32_t)yq_encode(v[2 * u], e) & 0xFFFFu) |
              ((uint32_t)yq_encode(v[2 * u + 1], e) << 16);
}
__device__ __forceinline__ void yq_decode8(const u32x4 mant, int e, float* v) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v[2 * u] = yq_decode((int)(int16_t)(mant[u] & 0xFFFFu), e);
    v[2 * u + 1] = yq_decode((int)(int16_t)(mant[u] >> 16), e);
  }
}
// Features c..c+7 (c a multiple of 8) of row r of a y_perm with rows of
// `rb` bytes.
__device__ __forceinline__ void yq_load8(const unsigned char* __restrict__ y, size_t rb, int d,
                                         long r, int c, float* v) {
  const unsigned char* row = y + (size_t)r * rb;
  const u32x4 mant = *(const u32x4*)(row + (size_t)2 * c);
  const int e = (int)(signed char)row[(size_t)2 * d + c / kYBlock];
  yq_decode8(mant, e, v);
}
__device__ __forceinline__ void yq_store8(unsigned char* __restrict__ y, size_t rb, int d, long r,
                                          int c, const float* v) {
  unsigned char* row = y + (size_t)r * rb;
  u32x4 mant;
  int e;
  yq_encode8(v, mant, e);
  *(u32x4*)(row + (size_t)2 * c) = mant;
  row[(size_t)2 * d + c / kYBlock] = (unsigned char)(signed char)e;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << __lane_id()) - 1ull;
}

// ---- host helpers ----------------------------------------------------------
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Debug builds (MOE_HOST_BOUNDS_CHECK): copy the permutation arrays a call
// is about to index with to the host (synchronising `s`) and check them with
// moe_check_permutation; any of the device pointers may be NULL. Returns
// the status the entry point gives back (MOE_ERR_INVALID for bad arrays).
int debug_check(hipStream_t s, const int32_t* offsets, int E, const int32_t* sorted_token,
                const int32_t* dest_row, int T, int k);
#ifdef MOE_HOST_BOUNDS_CHECK
#define MOE_DEBUG_CHECK(...)                  \
  do {                                        \
    const int st_ = moe::debug_check(__VA_ARGS__); \
    if (st_ != MOE_OK) return st_;            \
  } while (0)
#else
#define MOE_DEBUG_CHECK(...) \
  do {                       \
  } while (0)
#endif
inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// Workspace layouts; each op's size function is the single source of truth
// for both moe_workspace_size() and the call that consumes the workspace.
constexpr int kRouterTokens = 4;  // fewest tokens per selection block (sizes the partials)
constexpr int kPermuteChunk = 1024;  // assignments per permute block

// bf16 router logits: blocks of tt tokens x ep (E padded to 64) experts, each
// over one of `split` ranges of the 32-wide K chunks; fp32 partial logits
// [split][T][E] are summed in order by the selection kernel.
constexpr int kRouterMinChunks = 8;
struct RouterPlan {
  int ep, tt, ntt, nch, split;
};
inline RouterPlan router_plan(int T, int d, int E) {
  RouterPlan p;
  p.ep = (E + 63) / 64 * 64;
  // token rows per tile: 128 x 256 for E = 256, where every token tile
  // re-reads the 3.7 MB W_g; smaller tiles (less K splitting, fewer partial
  // logits) for E <= 192
  int tt = (p.ep >= 256 ? 32768 : 8192) / p.ep / 64 * 64;
  if (tt > 256) tt = 256;
  if (tt < 64) tt = 64;
  p.tt = tt;  // 128 or 64
  p.ntt = ceil_div(T > 0 ? T : 1, tt);
  p.nch = ceil_div(d, 32);
  // about one block per CU, but each K range at least kRouterMinChunks chunks:
  // a shorter one costs more partial-logit traffic than it saves
  int s = 256 / p.ntt;
  if (s > p.nch / kRouterMinChunks) s = p.nch / kRouterMinChunks;
  if (s < 1) s = 1;
  p.split = s;
  return p;
}
inline int router_blocks(int T) { return ceil_div(T, kRouterTokens); }
inline size_t router_partial_bytes(int T, int d, int E) {
  return align_up((size_t)router_plan(T, d, E).split * T * E * sizeof(float), 256);
}
inline size_t router_ws(int T, int d, int E) {
  return router_partial_bytes(T, d, E) + align_up((size_t)router_blocks(T) * E * sizeof(float), 256);
}
inline int permute_blocks(long n) { return n > 0 ? ceil_div(n, kPermuteChunk) : 0; }
inline size_t permute_ws(int T, int k, int E) {
  long n = (long)T * k;
  return align_up((size_t)2 * E * permute_blocks(n) * sizeof(int32_t), 256);
}
// FFN: [plan: tile map (2*(E+1) int32) or the DMA-ring kernels' work lists]
//      [hidden H: T*k*h elements of 4 bytes max]
//      [tail partials: kTailSlots tiles of 256 x 256 fp32]
constexpr int kBigBNTile = 256;  // weight rows per DMA-ring tile
constexpr int kTailSlots = 256;  // DMA-ring blocks resident at once (one per CU)
// Work-list entries of one DMA-ring GEMM launch (256 x BM tiles over N output
// features): every tile once plus at most kTailSlots split units, rounded to
// the 8 XCDs.
inline int ffn_big_grid(long rows, int E, int N, int BM) {
  const long nonempty = rows < E ? rows : E;
  const long mslots = (rows + BM - 1) / BM + nonempty;
  return ceil_div(mslots * (N / kBigBNTile) + kTailSlots, 8) * 8;
}
constexpr int kWorkBytes = 32;  // one work-list entry
// Plan region of the DMA-ring path: [2 headers][work lists of both GEMMs]
// [token table: the token of each row of each BM-row block, padded rows
// repeating the block's last]. The lists are longest for 128-row tiles; the
// table's padding grows with BM, so it is sized for the larger of the two.
inline long ffn_tok_entries(long rows, int E, int BM) {
  const long nonempty = rows < E ? rows : E;
  return ((rows + BM - 1) / BM + nonempty) * BM;
}
inline size_t ffn_lists_bytes(long rows, int E, int d, int h) {
  return 256 + (size_t)(ffn_big_grid(rows, E, h, 128) + ffn_big_grid(rows, E, d, 128)) * kWorkBytes;
}
inline size_t ffn_tok_bytes(long rows, int E) {
  const long a = ffn_tok_entries(rows, E, 128), b = ffn_tok_entries(rows, E, 256);
  return align_up((size_t)(a > b ? a : b) * sizeof(int32_t), 256);
}
inline size_t ffn_plan_bytes(int T, int d, int h, int E, int k) {
  const long rows = (long)T * k;
  const size_t tmap = align_up((size_t)2 * (E + 1) * sizeof(int32_t), 256);
  const size_t ring = align_up(ffn_lists_bytes(rows, E, d, h), 256) + ffn_tok_bytes(rows, E);
  return align_up(tmap > ring ? tmap : ring, 256);
}
inline size_t ffn_hidden_bytes(int T, int h, int k) { return align_up((size_t)T * k * h * 4, 256); }
// A DMA-ring tile holds up to 256 + 32 permuted rows (an expert's last row
// block takes up to 32 more rows rather than leaving them to a nearly empty
// tile); its fp32 partial is [288][256].
constexpr int kBigRowsMax = 288;
inline size_t ffn_partial_bytes() {
  return (size_t)kTailSlots * kBigRowsMax * 256 * sizeof(float);
}
inline size_t ffn_ws(int T, int d, int h, int E, int k) {
  return ffn_plan_bytes(T, d, h, E, k) + ffn_hidden_bytes(T, h, k) + ffn_partial_bytes();
}

// Router weight backward: fp32 partial dW_g over S token ranges [S][E][d],
// S chosen so that the 64 x 64 tiles times S make about 4096 blocks, with
// at least 16 tokens per range and at most 64 ranges.
inline int router_bwd_splits(int T, int d, int E) {
  const int tiles = ceil_div(E, 64) * ceil_div(d, 64);
  int s = ceil_div(4096, tiles);
  if (s > 64) s = 64;
  if (s > T / 16) s = T / 16;
  return s < 1 ? 1 : s;
}
inline size_t router_bwd_ws(int T, int d, int E) {
  return align_up((size_t)router_bwd_splits(T, d, E) * E * d * sizeof(float), 256);
}

// FFN backward: [plan of the forward-shaped GEMMs (ffn_plan_bytes)]
//   [weight-gradient work lists: 2 x E x (d/128)(h/256) entries]
//   [header + work list of the Z recompute (the forward's taller last tiles)]
//   [Z: T*k*h x 4 B] [dZ: T*k*h x 4 B] [tail partials]
//   [gathered input rows: T*k*d bf16]
struct FfnBwdLayout {
  size_t wl, zr, z, dz, part, xp, total;
};
inline FfnBwdLayout ffn_bwd_layout(int T, int d, int h, int E, int k) {
  FfnBwdLayout L;
  const size_t rows = (size_t)T * k;
  size_t o = ffn_plan_bytes(T, d, h, E, k);
  L.wl = o;
  o += align_up((size_t)4 * E * (d / kBigBNTile) * (h / kBigBNTile) * kWorkBytes, 256);
  L.zr = o;
  o += align_up(256 + (size_t)ffn_big_grid(rows, E, h, kBigBNTile) * kWorkBytes, 256);
  L.z = o;
  o += align_up(rows * h * 4, 256);
  L.dz = o;
  o += align_up(rows * h * 4, 256);
  L.part = o;
  o += ffn_partial_bytes();
  L.xp = o;
  o += align_up(rows * d * 2, 256);
  L.total = o;
  return L;
}

}  // namespace moe
