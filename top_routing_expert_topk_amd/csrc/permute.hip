// Permute: stable counting sort of the T*k (token, slot) assignments by
// expert, with per-expert capacity.
//
// The executor of page "MoE三难困境破解：按需加载+路由解耦+显存精控" (section 3.3)
// counts tokens per expert and groups them so each expert runs one matmul
// over its group; the capacity section of "MoE混合专家模型路由机制原理与稀疏激活实现"
// caps each expert at capacity = tokens/experts * factor and lets rejected
// tokens pass on the residual. Which assignments are kept when an expert
// overflows is not stated there; here the first `capacity` in flat order
// f = t*k + j are kept (first come, first served by token).
//
// Three kernels, all integer and exact (a few assignments take one block,
// permute_small, through the same steps):
//   1. hist:    one block per chunk of kPermuteChunk assignments; LDS
//               histogram; counts per (expert, chunk).
//   2. scan:    one block; per expert, exclusive prefix over chunks (block
//               bases), totals -> counts, kept -> offsets (exclusive scan).
//   3. scatter: one block per chunk; the rank of an assignment inside its
//               chunk comes from wave ballots (lanes with the same expert),
//               prefix over earlier waves and earlier rounds, so the order is
//               stable in f; then dest_row / sorted_token.
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int CH = kPermuteChunk;
constexpr int NTH = 256;
constexpr int ROUNDS = CH / NTH;

__global__ __launch_bounds__(NTH) void permute_hist(const int32_t* __restrict__ idx, long n, int E,
                                                    int nb, int32_t* __restrict__ blk_hist) {
  __shared__ int hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += NTH) hist[e] = 0;
  __syncthreads();
  const long base = (long)blockIdx.x * CH;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const long f = base + r * NTH + threadIdx.x;
    if (f < n) atomicAdd(&hist[idx[f]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += NTH) blk_hist[(size_t)e * nb + blockIdx.x] = hist[e];
}

// One block of 512 threads (>= kMaxE): thread e walks the chunks of expert e.
__global__ __launch_bounds__(512) void permute_scan(const int32_t* __restrict__ blk_hist, int nb,
                                                   int E, int capacity,
                                                   int32_t* __restrict__ blk_base,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets) {
  __shared__ int sc[2][kMaxE];
  const int e = threadIdx.x;
  int kept = 0;
  if (e < E) {
    const int32_t* hrow = blk_hist + (size_t)e * nb;
    int32_t* brow = blk_base + (size_t)e * nb;
    int run = 0;
    int b = 0;
    for (; b + 8 <= nb; b += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = hrow[b + i];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        brow[b + i] = run;
        run += v[i];
      }
    }
    for (; b < nb; ++b) {
      const int v = hrow[b];
      brow[b] = run;
      run += v;
    }
    counts[e] = run;
    kept = (capacity >= 0 && run > capacity) ? capacity : run;
  }
  // inclusive Hillis-Steele scan of kept over experts
  int cur = 0;
  sc[0][e] = kept;
  __syncthreads();
  for (int off = 1; off < kMaxE; off <<= 1) {
    const int v = sc[cur][e] + (e >= off ? sc[cur][e - off] : 0);
    sc[cur ^ 1][e] = v;
    cur ^= 1;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = sc[cur][e];
  if (e == 0) offsets[0] = 0;
}

__global__ __launch_bounds__(NTH) void permute_scatter(
    const int32_t* __restrict__ idx, long n, int k, int E, int nb,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ dest_row, int32_t* __restrict__ sorted_token) {
  __shared__ int run[kMaxE];         // assignments of expert e seen before this round
  __shared__ int off[kMaxE + 1];     // offsets
  __shared__ int wcnt[NTH / 64][kMaxE];  // this round's count per (wave, expert)
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int e = tid; e < E; e += NTH) {
    run[e] = blk_base[(size_t)e * nb + blockIdx.x];
    off[e] = offsets[e];
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) wcnt[w][e] = 0;
  }
  if (tid == 0) off[E] = offsets[E];
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  __syncthreads();

  const long base = (long)blockIdx.x * CH;
  for (int r = 0; r < ROUNDS; ++r) {
    const long f = base + r * NTH + tid;
    const bool valid = f < n;
    const int e = valid ? idx[f] : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lanemask_lt());
    const int cnt = __popcll(peers);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave][e] = cnt;
    __syncthreads();
    if (valid) {
      int pos = run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      const int kept = off[e + 1] - off[e];
      int dst = -1;
      if (pos < kept) {
        dst = off[e] + pos;
        sorted_token[dst] = (int32_t)(f / k);
      }
      dest_row[f] = dst;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&run[e], cnt);
      wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

// Up to kSmallN assignments: the same three steps in one block of 1024
// threads (histogram, kept counts and their scan, then rounds of 1024
// assignments ranked as permute_scatter ranks them), one launch instead of
// three and no workspace; each thread loads its assignments once, up front.
// (At 8192 assignments the one block is slower than the three kernels.)
constexpr int kSmallN = 2048;
constexpr int STH = 1024;
__global__ __launch_bounds__(STH) void permute_small(const int32_t* __restrict__ idx, int n, int k,
                                                     int E, int capacity,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ dest_row,
                                                     int32_t* __restrict__ sorted_token) {
  __shared__ int hist[kMaxE];
  __shared__ int run[kMaxE];
  __shared__ int off[kMaxE + 1];
  __shared__ int sc[2][kMaxE];
  __shared__ int wcnt[STH / 64][kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int e = tid; e < kMaxE; e += STH) {
    hist[e] = 0;
    run[e] = 0;
#pragma unroll
    for (int w = 0; w < STH / 64; ++w) wcnt[w][e] = 0;
  }
  // every assignment this thread ranks, loaded once up front
  int ev[kSmallN / STH];
#pragma unroll
  for (int r = 0; r < kSmallN / STH; ++r) {
    const int f = r * STH + tid;
    ev[r] = f < n ? idx[f] : 0;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSmallN / STH; ++r)
    if (r * STH + tid < n) atomicAdd(&hist[ev[r]], 1);
  __syncthreads();
  // kept per expert, inclusive scan over experts (threads 0 .. kMaxE-1)
  int cur = 0;
  if (tid < kMaxE) {
    const int c = tid < E ? hist[tid] : 0;
    if (tid < E) counts[tid] = c;
    sc[0][tid] = (capacity >= 0 && c > capacity) ? capacity : c;
  }
  __syncthreads();
  for (int o = 1; o < kMaxE; o <<= 1) {
    if (tid < kMaxE) sc[cur ^ 1][tid] = sc[cur][tid] + (tid >= o ? sc[cur][tid - o] : 0);
    cur ^= 1;
    __syncthreads();
  }
  if (tid < E) {
    off[tid + 1] = sc[cur][tid];
    offsets[tid + 1] = sc[cur][tid];
  }
  if (tid == 0) {
    off[0] = 0;
    offsets[0] = 0;
  }
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < kSmallN / STH; ++rr) {
    const int r0 = rr * STH;
    if (r0 >= n) break;
    const int f = r0 + tid;
    const bool valid = f < n;
    const int e = ev[rr];
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lanemask_lt());
    const int cnt = __popcll(peers);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave][e] = cnt;
    __syncthreads();
    if (valid) {
      int pos = run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      const int kept = off[e + 1] - off[e];
      int dst = -1;
      if (pos < kept) {
        dst = off[e] + pos;
        sorted_token[dst] = f / k;
      }
      dest_row[f] = dst;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&run[e], cnt);
      wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

// The three kernels over a caller's workspace (per-chunk histograms and
// bases, 2 E nb int32, every entry written before it is read), or the
// one-block kernel for a few assignments.
int permute_run(const int32_t* topk_idx, int T, int k, int E, int capacity, int32_t* counts,
                int32_t* offsets, int32_t* dest_row, int32_t* sorted_token, int32_t* blk_hist,
                hipStream_t s) {
  const long n = (long)T * k;
  if (n <= kSmallN) {
    hipLaunchKernelGGL(permute_small, dim3(1), dim3(STH), 0, s, topk_idx, (int)n, k, E, capacity,
                       counts, offsets, dest_row, sorted_token);
    return launch_status();
  }
  const int nb = permute_blocks(n);
  int32_t* blk_base = blk_hist + (size_t)E * nb;
  if (nb > 0) hipLaunchKernelGGL(permute_hist, dim3(nb), dim3(NTH), 0, s, topk_idx, n, E, nb, blk_hist);
  // with n == 0 the scan still writes zero counts and offsets (nb == 0)
  hipLaunchKernelGGL(permute_scan, dim3(1), dim3(512), 0, s, blk_hist, nb, E, capacity, blk_base,
                     counts, offsets);
  if (nb > 0)
    hipLaunchKernelGGL(permute_scatter, dim3(nb), dim3(NTH), 0, s, topk_idx, n, k, E, nb, blk_base,
                       offsets, dest_row, sorted_token);
  return launch_status();
}

int permute_check(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                  int32_t* offsets, int32_t* dest_row, int32_t* sorted_token) {
  if (T < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID;
  const long n = (long)T * k;
  if (n > 0x7FFFFFFFL) return MOE_ERR_UNSUPPORTED;
  if (n > 0 && (!topk_idx || !dest_row || !sorted_token)) return MOE_ERR_INVALID;
  return MOE_OK;
}

// The allocation-free variant's histograms: a file-scope device array, one
// copy per GPU, sized for MOE_PERMUTE_NOALLOC_MAX_ASSIGN assignments at the
// largest E. Host code never passes the array's name to a kernel (in host
// code it is a stand-in, not a device address): each device's address is
// looked up once, with that device current, and kept.
constexpr long kNoallocAssign = MOE_PERMUTE_NOALLOC_MAX_ASSIGN;
constexpr size_t kNoallocInts = (size_t)2 * kMaxE * (kNoallocAssign / kPermuteChunk);
static_assert(kNoallocAssign % kPermuteChunk == 0, "whole chunks");
__device__ __align__(256) int32_t scratch[kNoallocInts];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch[kMaxDevices] = {};

// This device's copy of scratch, or nullptr if it cannot be found.
int32_t* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return nullptr;
    g_scratch[dev] = (int32_t*)p;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_permute(const int32_t* topk_idx, int T, int k, int E, int capacity,
                           int32_t* counts, int32_t* offsets, int32_t* dest_row,
                           int32_t* sorted_token, void* ws, size_t ws_bytes,
                           moe_stream_t stream) {
  const int st = permute_check(topk_idx, T, k, E, counts, offsets, dest_row, sorted_token);
  if (st != MOE_OK) return st;
  const int nb = permute_blocks((long)T * k);
  if (nb > 0 && (!ws || ws_bytes < permute_ws(T, k, E))) return MOE_ERR_WORKSPACE;
  return permute_run(topk_idx, T, k, E, capacity, counts, offsets, dest_row, sorted_token,
                     (int32_t*)ws, (hipStream_t)stream);
}

extern "C" int moe_permute_noalloc(const int32_t* topk_idx, int T, int k, int E, int capacity,
                                   int32_t* counts, int32_t* offsets, int32_t* dest_row,
                                   int32_t* sorted_token, moe_stream_t stream) {
  const int st = permute_check(topk_idx, T, k, E, counts, offsets, dest_row, sorted_token);
  if (st != MOE_OK) return st;
  if ((long)T * k > kNoallocAssign) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  int dev = -1;
  if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return MOE_ERR_LAUNCH;
  int32_t* hist = scratch_on(dev);
  if (!hist) return MOE_ERR_LAUNCH;
  return permute_run(topk_idx, T, k, E, capacity, counts, offsets, dest_row, sorted_token, hist,
                     s);
}
