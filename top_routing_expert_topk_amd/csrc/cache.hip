// Expert cache for host-resident experts: a least-recently-used set of S
// device slots over E experts whose weights live in pinned host memory,
// loaded on demand (page "MoE三难困境破解：按需加载+路由解耦+显存精控", section
// 3.1: an expert container that keeps only metadata and an LRU of loaded
// experts, loading an expert when routing selects it; section 3.2: routing
// only returns indices, the executor loads the active experts and then runs
// the grouped FFN; page "MoE 架构完整指南", section 5.3: hot experts resident,
// cold ones fetched into an LRU cache).
//
// One step: the host reads the per-expert counts of the routing, and
// moe_cache_step marks each needed expert as a hit (already in a slot) or a
// miss. A miss takes the least recently used slot that this step does not
// need and is copied host->device on the copy stream; the slot table and the
// phase of every expert (0 hit, 1 miss, -1 not needed) go to the device on
// the compute stream. The FFN then runs the hits (phase 0) while the misses
// are still being copied, and the misses (phase 1) once the copy stream's
// work is done, so the copies overlap the hits' compute.
//
// The state is a caller-owned host block (moe_cache_state_bytes); the
// library keeps nothing between calls.
#include <string.h>

#include "moe_internal.h"

namespace moe {
namespace {

struct CacheHeader {
  int32_t E, S;
  int64_t clock;
};

// [header][slot_of E][phase_of E][expert_in S][last_use S (int64)]
struct CacheView {
  CacheHeader* hdr;
  int32_t* slot_of;
  int32_t* phase_of;
  int32_t* expert_in;
  int64_t* last_use;
};

size_t cache_bytes(int E, int S) {
  return align_up(sizeof(CacheHeader), 8) + align_up((size_t)2 * E * sizeof(int32_t), 8) +
         align_up((size_t)S * sizeof(int32_t), 8) + (size_t)S * sizeof(int64_t);
}

CacheView view(void* state, int E, int S) {
  unsigned char* p = (unsigned char*)state;
  CacheView v;
  v.hdr = (CacheHeader*)p;
  p += align_up(sizeof(CacheHeader), 8);
  v.slot_of = (int32_t*)p;
  v.phase_of = v.slot_of + E;
  p += align_up((size_t)2 * E * sizeof(int32_t), 8);
  v.expert_in = (int32_t*)p;
  p += align_up((size_t)S * sizeof(int32_t), 8);
  v.last_use = (int64_t*)p;
  return v;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_cache_state_bytes(int E, int S) {
  if (E < 1 || S < 1 || E > kMaxE) return 0;
  return cache_bytes(E, S);
}

extern "C" int moe_cache_init(void* state, int E, int S) {
  if (!state || E < 1 || S < 1) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  CacheView v = view(state, E, S);
  v.hdr->E = E;
  v.hdr->S = S;
  v.hdr->clock = 0;
  for (int e = 0; e < E; ++e) {
    v.slot_of[e] = -1;
    v.phase_of[e] = -1;
  }
  for (int s = 0; s < S; ++s) {
    v.expert_in[s] = -1;
    v.last_use[s] = -1;
  }
  return MOE_OK;
}

extern "C" int moe_cache_step(void* state, const int32_t* counts, int ntensors,
                              const void* const* host_base, void* const* dev_base,
                              const size_t* bytes_per_expert, int32_t* slot_of_dev,
                              int32_t* phase_of_dev, int* n_loaded, moe_stream_t compute_stream,
                              moe_stream_t copy_stream) {
  if (!state || !counts || ntensors < 0) return MOE_ERR_INVALID;
  if (ntensors > 0 && (!host_base || !dev_base || !bytes_per_expert)) return MOE_ERR_INVALID;
  const CacheHeader* h0 = (const CacheHeader*)state;
  const int E = h0->E, S = h0->S;
  if (E < 1 || S < 1 || E > kMaxE) return MOE_ERR_INVALID;
  CacheView v = view(state, E, S);
  int need = 0;
  for (int e = 0; e < E; ++e) need += counts[e] > 0 ? 1 : 0;
  if (need > S) return MOE_ERR_UNSUPPORTED;  // more experts in one step than slots
  const int64_t now = ++v.hdr->clock;
  // hits first, so every slot this step needs is marked before any eviction
  for (int e = 0; e < E; ++e) {
    v.phase_of[e] = -1;
    if (counts[e] > 0 && v.slot_of[e] >= 0) {
      v.phase_of[e] = 0;
      v.last_use[v.slot_of[e]] = now;
    }
  }
  int loaded = 0;
  for (int e = 0; e < E; ++e) {
    if (counts[e] <= 0 || v.slot_of[e] >= 0) continue;
    // least recently used slot not needed by this step (empty slots first)
    int victim = -1;
    for (int s = 0; s < S; ++s)
      if (v.last_use[s] < now && (victim < 0 || v.last_use[s] < v.last_use[victim])) victim = s;
    if (victim < 0) return MOE_ERR_UNSUPPORTED;  // cannot happen: need <= S
    if (v.expert_in[victim] >= 0) v.slot_of[v.expert_in[victim]] = -1;
    v.expert_in[victim] = e;
    v.slot_of[e] = victim;
    v.last_use[victim] = now;
    v.phase_of[e] = 1;
    for (int i = 0; i < ntensors; ++i) {
      if (!host_base[i] || !dev_base[i] || bytes_per_expert[i] == 0) continue;
      const size_t nb = bytes_per_expert[i];
      if (hipMemcpyAsync((unsigned char*)dev_base[i] + (size_t)victim * nb,
                         (const unsigned char*)host_base[i] + (size_t)e * nb, nb,
                         hipMemcpyHostToDevice, (hipStream_t)copy_stream) != hipSuccess)
        return MOE_ERR_LAUNCH;
    }
    ++loaded;
  }
  if (n_loaded) *n_loaded = loaded;
  // the tables the FFN reads, ordered before it on the compute stream
  if (slot_of_dev &&
      hipMemcpyAsync(slot_of_dev, v.slot_of, (size_t)E * sizeof(int32_t), hipMemcpyHostToDevice,
                     (hipStream_t)compute_stream) != hipSuccess)
    return MOE_ERR_LAUNCH;
  if (phase_of_dev &&
      hipMemcpyAsync(phase_of_dev, v.phase_of, (size_t)E * sizeof(int32_t),
                     hipMemcpyHostToDevice, (hipStream_t)compute_stream) != hipSuccess)
    return MOE_ERR_LAUNCH;
  return MOE_OK;
}

extern "C" int moe_cache_slot_of(const void* state, int32_t* slot_of, int32_t* phase_of) {
  if (!state) return MOE_ERR_INVALID;
  const CacheHeader* h0 = (const CacheHeader*)state;
  const int E = h0->E, S = h0->S;
  if (E < 1 || S < 1) return MOE_ERR_INVALID;
  CacheView v = view((void*)state, E, S);
  if (slot_of) memcpy(slot_of, v.slot_of, (size_t)E * sizeof(int32_t));
  if (phase_of) memcpy(phase_of, v.phase_of, (size_t)E * sizeof(int32_t));
  return MOE_OK;
}
