// Host-side checks of the permutation arrays that the FFN, the combine and
// their backward index with: offsets, sorted_token and dest_row (the
// counting sort of page "MoE混合专家模型路由机制原理与稀疏激活实现", section
// "Top-K门控路由的PyTorch实现", with the capacity drop of section "Expert
// Choice路由策略与容量因子调优"). A kernel trusts these arrays for every
// gather and scatter address, so a debug build (MOE_HOST_BOUNDS_CHECK)
// copies them to the host and runs these checks before each such launch.
//
// This file holds host code only; it is compiled into libmoe.so with the
// kernels, and on its own by the host-only builds of the tests.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

extern "C" int moe_check_permutation(const int32_t* offsets, int E, const int32_t* sorted_token,
                                     const int32_t* dest_row, int T, int k) {
  if (T < 0 || k < 1 || E < 1) return MOE_ERR_INVALID;
  const long slots = (long)T * k;
  long R = slots;  // rows the permuted arrays may hold
  if (offsets) {
    if (offsets[0] != 0) return MOE_ERR_INVALID;
    for (int e = 0; e < E; ++e)
      if (offsets[e + 1] < offsets[e]) return MOE_ERR_INVALID;
    if (offsets[E] > slots) return MOE_ERR_INVALID;
    R = offsets[E];
  }
  if (sorted_token) {
    if (!offsets) return MOE_ERR_INVALID;  // its length is offsets[E]
    for (long r = 0; r < R; ++r)
      if (sorted_token[r] < 0 || sorted_token[r] >= T) return MOE_ERR_INVALID;
  }
  if (!dest_row) return MOE_OK;
  for (long i = 0; i < slots; ++i)
    if (dest_row[i] < -1 || dest_row[i] >= R) return MOE_ERR_INVALID;
  if (!offsets || !sorted_token) return MOE_OK;
  // every row is the row of exactly one kept slot, and holds that slot's token
  unsigned char* seen = (unsigned char*)calloc(R > 0 ? (size_t)R : 1, 1);
  if (!seen) return MOE_ERR_INVALID;
  int st = MOE_OK;
  long kept = 0;
  for (long i = 0; i < slots && st == MOE_OK; ++i) {
    const int32_t r = dest_row[i];
    if (r < 0) continue;
    if (seen[r] || sorted_token[r] != (int32_t)(i / k)) st = MOE_ERR_INVALID;
    seen[r] = 1;
    ++kept;
  }
  if (st == MOE_OK && kept != R) st = MOE_ERR_INVALID;
  free(seen);
  return st;
}

extern "C" int moe_debug_checks(void) {
#ifdef MOE_HOST_BOUNDS_CHECK
  return 1;
#else
  return 0;
#endif
}
