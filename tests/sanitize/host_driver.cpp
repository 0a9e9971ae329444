// Drives the host code of libmoe (argument validation, workspace sizes, the
// expert-cache policy and the permutation check) for a build whose host
// code runs under AddressSanitizer and UndefinedBehaviorSanitizer. No call
// here reaches the GPU: every entry point is given arguments that its host
// validation refuses before any launch, the cache steps copy nothing (no
// tensors, no device tables), and the permutation check reads host arrays.
// Every result is compared with the status the header documents; the run
// must end with status 0 and no sanitizer report.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "moe.h"

static int failures = 0;
#define EXPECT(cond)                                             \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                \
    }                                                            \
  } while (0)

// a pointer value that validation must refuse before it is ever read
static void* const BAD = (void*)(uintptr_t)0x1000;

static uint64_t rng = 12345;
static uint32_t next_u32() {
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(rng >> 33);
}

static void status_and_sizes() {
  for (int s = -1; s <= 6; ++s) EXPECT(moe_status_string(s) != nullptr);
  EXPECT(moe_version() > 0);
  EXPECT(moe_debug_checks() == 0 || moe_debug_checks() == 1);
  const int Ts[] = {0, 1, 7, 300, 4096, 8192, 1 << 17};
  const int Es[] = {1, 8, 64, 256, 512, 513};
  const int ks[] = {1, 2, 8, 16};
  const int ds[] = {64, 768, 4096, 7168};
  for (int op = -1; op <= 5; ++op)
    for (int T : Ts)
      for (int E : Es)
        for (int k : ks)
          for (int d : ds) {
            const size_t n = moe_workspace_size(op, T, d, 2 * d, E, k);
            if (op < 0 || op > 4) EXPECT(n == 0);
          }
}

static void cache_policy() {
  EXPECT(moe_cache_state_bytes(0, 4) == 0);
  EXPECT(moe_cache_state_bytes(8, 0) == 0);
  EXPECT(moe_cache_state_bytes(600, 4) == 0);
  EXPECT(moe_cache_init(nullptr, 8, 4) == MOE_ERR_INVALID);
  const int shapes[][2] = {{8, 4}, {64, 56}, {512, 300}, {5, 5}, {3, 1}};
  for (const auto& sh : shapes) {
    const int E = sh[0], S = sh[1];
    const size_t nb = moe_cache_state_bytes(E, S);
    EXPECT(nb > 0);
    std::vector<unsigned char> state(nb);
    EXPECT(moe_cache_init(state.data(), E, S) == MOE_OK);
    std::vector<int32_t> counts(E), slot(E), phase(E);
    for (int step = 0; step < 40; ++step) {
      int need = 0;
      for (int e = 0; e < E; ++e) {
        counts[e] = (next_u32() % 5 == 0) ? (int)(next_u32() % 7) : 0;
        need += counts[e] > 0;
      }
      int loaded = -1;
      const int st = moe_cache_step(state.data(), counts.data(), 0, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, &loaded, nullptr, nullptr);
      if (need > S) {
        EXPECT(st == MOE_ERR_UNSUPPORTED);
        continue;
      }
      EXPECT(st == MOE_OK);
      EXPECT(moe_cache_slot_of(state.data(), slot.data(), phase.data()) == MOE_OK);
      int misses = 0;
      for (int e = 0; e < E; ++e) {
        if (counts[e] > 0) EXPECT(slot[e] >= 0 && slot[e] < S && phase[e] >= 0);
        else EXPECT(phase[e] == -1);
        misses += phase[e] == 1;
      }
      EXPECT(loaded == misses);
    }
    EXPECT(moe_cache_step(state.data(), nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr, nullptr) == MOE_ERR_INVALID);
  }
}

// A valid counting-sort permutation of random top-k indices, then one
// mutation at a time, each of which the check must refuse.
static void permutation_check() {
  for (int trial = 0; trial < 200; ++trial) {
    const int T = 1 + (int)(next_u32() % 40), E = 1 + (int)(next_u32() % 12);
    const int k = 1 + (int)(next_u32() % (E < 4 ? E : 4));
    const int cap = (next_u32() % 3 == 0) ? (int)(next_u32() % 5) : -1;
    std::vector<int32_t> idx((size_t)T * k);
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j) {  // k distinct experts per token
        int e;
        bool dup;
        do {
          e = (int)(next_u32() % E);
          dup = false;
          for (int i = 0; i < j; ++i) dup = dup || idx[(size_t)t * k + i] == e;
        } while (dup);
        idx[(size_t)t * k + j] = e;
      }
    std::vector<int32_t> cnt(E, 0), offsets(E + 1, 0), dest((size_t)T * k, -1), st;
    std::vector<int32_t> kept(E, 0);
    for (size_t i = 0; i < idx.size(); ++i) {
      const int e = idx[i];
      if (cap < 0 || kept[e] < cap) {
        dest[i] = -2 - e;  // kept; its row is set below
        ++kept[e];
      }
    }
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + kept[e];
    st.assign((size_t)offsets[E] + 1, -7);
    std::vector<int32_t> fill(offsets.begin(), offsets.end() - 1);
    for (size_t i = 0; i < idx.size(); ++i)
      if (dest[i] <= -2) {
        const int r = fill[idx[i]]++;
        dest[i] = r;
        st[r] = (int32_t)(i / k);
      }
    const int R = offsets[E];
    EXPECT(moe_check_permutation(offsets.data(), E, st.data(), dest.data(), T, k) == MOE_OK);
    EXPECT(moe_check_permutation(offsets.data(), E, st.data(), nullptr, T, k) == MOE_OK);
    EXPECT(moe_check_permutation(nullptr, E, nullptr, dest.data(), T, k) == MOE_OK);
    EXPECT(moe_check_permutation(offsets.data(), E, nullptr, nullptr, T, k) == MOE_OK);
    EXPECT(moe_check_permutation(nullptr, E, st.data(), nullptr, T, k) == MOE_ERR_INVALID);
    auto bad = [&](std::vector<int32_t> o, std::vector<int32_t> s, std::vector<int32_t> d) {
      return moe_check_permutation(o.data(), E, s.data(), d.data(), T, k) == MOE_ERR_INVALID;
    };
    {
      auto o = offsets;
      o[0] = 1;
      EXPECT(bad(o, st, dest));
    }
    if (E > 1 && R > 0) {
      auto o = offsets;
      const int e = (int)(next_u32() % (E - 1)) + 1;
      o[e] = o[e + 1] + 1;  // decreasing step
      EXPECT(bad(o, st, dest));
    }
    {
      auto o = offsets;
      o[E] = T * k + 1;  // more rows than slots
      std::vector<int32_t> s2(st);
      s2.resize((size_t)T * k + 2, 0);
      EXPECT(bad(o, s2, dest));
    }
    if (R > 0) {
      const int r = (int)(next_u32() % R);
      auto s = st;
      s[r] = T;  // token out of range
      EXPECT(bad(offsets, s, dest));
      s[r] = -1;
      EXPECT(bad(offsets, s, dest));
      auto d = dest;
      size_t i = next_u32() % d.size();
      d[i] = R;  // row out of range
      EXPECT(bad(offsets, st, d));
      d[i] = -2;
      EXPECT(bad(offsets, st, d));
      // a kept slot dropped: row left without its slot
      d = dest;
      for (size_t j = 0; j < d.size(); ++j)
        if (d[j] >= 0) {
          d[j] = -1;
          break;
        }
      EXPECT(bad(offsets, st, d));
    }
    if (R > 1) {
      // two slots on one row
      auto d = dest;
      int first = -1;
      for (size_t j = 0; j < d.size(); ++j)
        if (d[j] >= 0) {
          if (first < 0) first = (int)j;
          else {
            d[j] = d[first];
            break;
          }
        }
      EXPECT(bad(offsets, st, d));
    }
  }
  EXPECT(moe_check_permutation(nullptr, 4, nullptr, nullptr, -1, 2) == MOE_ERR_INVALID);
  EXPECT(moe_check_permutation(nullptr, 0, nullptr, nullptr, 4, 2) == MOE_ERR_INVALID);
}

static void refused_arguments() {
  int32_t* I = (int32_t*)BAD;
  float* F = (float*)BAD;
  EXPECT(moe_router_topk(BAD, 1, -1, 64, BAD, nullptr, 8, 2, 1, nullptr, I, F, nullptr, BAD,
                         1 << 30, nullptr) == MOE_ERR_INVALID);
  EXPECT(moe_router_topk(BAD, 1, 4, 60, BAD, nullptr, 8, 2, 1, nullptr, I, F, nullptr, BAD,
                         1 << 30, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_permute(I, -1, 2, 8, -1, I, I, I, I, BAD, 1 << 20, nullptr) == MOE_ERR_INVALID);
  EXPECT(moe_permute(I, 10, 2, 513, -1, I, I, I, I, BAD, 1 << 20, nullptr) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_permute(I, 10, 2, 8, -1, I, I, I, I, BAD, 4, nullptr) == MOE_ERR_WORKSPACE);
  EXPECT(moe_permute_noalloc(I, (1 << 17) + 1, 8, 512, -1, I, I, I, I, nullptr) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_grouped_ffn(BAD, 1, 10, 100, 256, 8, 2, I, I, BAD, nullptr, BAD, nullptr, BAD, BAD,
                         1 << 30, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_grouped_ffn(BAD, 1, 10, 128, 256, 8, 2, I, I, BAD, nullptr, BAD, nullptr, BAD, BAD,
                         100, nullptr) == MOE_ERR_WORKSPACE);
  EXPECT(moe_combine(BAD, 2, I, F, 4, 2, 64, nullptr, BAD, 0, nullptr) == MOE_ERR_INVALID);
  EXPECT(moe_combine(BAD, 1, I, F, 4, 513, 64, nullptr, BAD, 0, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_aux_loss(F, I, 4, 600, nullptr, nullptr, F, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_choice(F, -1, 8, 4, F, I, I, I, F, nullptr) == MOE_ERR_INVALID);
  EXPECT(moe_expert_choice(F, 1 << 23, 512, 4, F, I, I, I, F, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_combine_backward(BAD, 1, I, F, 4, 513, 64, BAD, BAD, F, nullptr) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_router_backward(F, I, F, F, I, 4, 600, 2, 1, 0.0f, F, nullptr) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_grouped_ffn_backward(BAD, 1, 10, 192, 512, 8, 2, I, I, BAD, nullptr, BAD, BAD,
                                  nullptr, nullptr, BAD, BAD, nullptr, BAD, nullptr, BAD,
                                  (size_t)1 << 40, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_grouped_ffn_train(BAD, 1, 10, 128, 256, 8, 2, I, I, BAD, nullptr, BAD, nullptr, BAD,
                               nullptr, BAD, BAD, (size_t)1 << 40, nullptr) == MOE_ERR_INVALID);
  EXPECT(moe_gather_backward(BAD, 1, I, 4, 2, 64, nullptr, nullptr, nullptr, 600, BAD, nullptr) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_router_weight_backward(BAD, 1, -1, 64, 8, F, F, nullptr, BAD, 1 << 30, nullptr) ==
         MOE_ERR_INVALID);
  EXPECT(moe_grouped_ffn_cached(BAD, 0, 4, 64, 64, 8, 2, I, I, I, I, 0, BAD, nullptr, BAD,
                                nullptr, BAD, BAD, 1 << 30, nullptr) == MOE_ERR_UNSUPPORTED);
}

int main() {
  status_and_sizes();
  cache_policy();
  permutation_check();
  refused_arguments();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host driver: all expectations met\n");
  return 0;
}
