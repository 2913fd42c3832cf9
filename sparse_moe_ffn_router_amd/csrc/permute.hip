// Token -> expert permutation: a stable counting sort of the T*k
// token-expert assignments a = t*k + j by expert id.  Counts use LDS
// atomics; positions never depend on atomic return order: inside a
// wavefront a lane's rank is the number of lower lanes holding the same
// expert (ballot + popcount), and wavefront steps run in assignment order,
// so the result is deterministic and ascending in a inside each segment.
//
// The pages only imply this step ("qwen35moe - Forward-Pass Design",
// section "K80 GPU decode": grouped expert launches; section "Batched
// prefill": tokens sharing an expert stream its weights once).
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kSmallThreads = 1024;

// Places one wavefront's 64 assignments [a0, a0+64) given the running
// per-expert fill pointers `fill` (LDS); returns nothing, writes outputs.
__device__ __forceinline__ void place_wave(const int32_t* __restrict__ topk_idx, int64_t n, int64_t a0,
                                           int32_t* fill, int32_t* __restrict__ sorted_assign,
                                           int32_t* __restrict__ assign_pos) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t a = a0 + lane;
  const int e = a < n ? topk_idx[a] : -1;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t pending = __ballot(e >= 0);
  int rank = 0, base = 0;
  bool leader = false;
  int group = 0;
  while (pending) {
    const int src = __ffsll((unsigned long long)pending) - 1;
    const int v = __shfl(e, src, kWave);
    const uint64_t m = __ballot(e == v);
    if (e == v) {
      rank = __popcll(m & lower);
      group = __popcll(m);
      leader = lane == src;
      base = fill[v];
    }
    pending &= ~m;
  }
  if (e >= 0) {
    const int pos = base + rank;
    sorted_assign[pos] = (int32_t)a;
    assign_pos[a] = pos;
  }
  // all lanes read `fill` above before any leader advances it
  __builtin_amdgcn_s_waitcnt(0);
  if (e >= 0 && leader) fill[e] = base + group;
  __builtin_amdgcn_s_waitcnt(0);
}

// Whole permutation in one workgroup (n = T*k small): LDS histogram,
// exclusive scan, then wave 0 places the assignments in order.
__global__ __launch_bounds__(kSmallThreads) void k_permute_small(const int32_t* __restrict__ topk_idx, int32_t T,
                                                                 int32_t k, int32_t E, int32_t shared,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ sorted_assign,
                                                                 int32_t* __restrict__ assign_pos) {
  __shared__ int32_t cnt[kMaxExperts + 2];
  __shared__ int32_t wsum[kSmallThreads / kWave];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)T * k;
  for (int e = tid; e <= E; e += kSmallThreads) cnt[e] = 0;
  __syncthreads();
  for (int64_t a = tid; a < n; a += kSmallThreads) atomicAdd(&cnt[topk_idx[a]], 1);
  __syncthreads();
  // exclusive scan over E entries (E <= 1024: one per thread)
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  int v = tid < E ? cnt[tid] : 0;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) wsum[wid] = incl;
  __syncthreads();
  int before = 0;
  for (int w2 = 0; w2 < wid; ++w2) before += wsum[w2];
  const int excl = before + incl - v;
  __syncthreads();
  if (tid < E) {
    cnt[tid] = excl;
    offsets[tid] = excl;
  }
  if (tid == 0) {
    offsets[E] = (int32_t)n;
    if (shared) offsets[E + 1] = (int32_t)(n + T);
  }
  __syncthreads();
  if (wid == 0)
    for (int64_t a0 = 0; a0 < n; a0 += kWave) place_wave(topk_idx, n, a0, cnt, sorted_assign, assign_pos);
  if (shared)
    for (int t = tid; t < T; t += kSmallThreads) {
      sorted_assign[n + t] = (int32_t)(n + t);
      assign_pos[n + t] = (int32_t)(n + t);
    }
}

// Large n, pass 1: per-chunk histograms counts[g][e].
__global__ __launch_bounds__(256) void k_perm_count(const int32_t* __restrict__ topk_idx, int64_t n, int32_t E,
                                                    int32_t* __restrict__ counts) {
  __shared__ int32_t h[kMaxExperts];
  const int g = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t a = (int64_t)g * kPermChunk + threadIdx.x;
  if (threadIdx.x < kPermChunk && a < n) atomicAdd(&h[topk_idx[a]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) counts[(size_t)g * E + e] = h[e];
}

// Large n, pass 2 (one workgroup): column prefix over chunks (turns counts
// into each chunk's start inside its expert segment), expert offsets.
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ counts, int32_t G, int32_t T, int32_t k,
                                                    int32_t E, int32_t shared, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ sorted_assign,
                                                    int32_t* __restrict__ assign_pos) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  int total = 0;
  if (tid < E)
    for (int g = 0; g < G; ++g) {
      const int c = counts[(size_t)g * E + tid];
      counts[(size_t)g * E + tid] = total;
      total += c;
    }
  int incl = total;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) wsum[wid] = incl;
  __syncthreads();
  int before = 0;
  for (int w2 = 0; w2 < wid; ++w2) before += wsum[w2];
  const int64_t n = (int64_t)T * k;
  if (tid < E) offsets[tid] = before + incl - total;
  if (tid == 0) {
    offsets[E] = (int32_t)n;
    if (shared) offsets[E + 1] = (int32_t)(n + T);
  }
  if (shared)
    for (int t = tid; t < T; t += 1024) {
      sorted_assign[n + t] = (int32_t)(n + t);
      assign_pos[n + t] = (int32_t)(n + t);
    }
}

// Large n, pass 3: one wave per chunk places its assignments in order.
__global__ __launch_bounds__(kWave) void k_perm_scatter(const int32_t* __restrict__ topk_idx, int64_t n, int32_t E,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_assign,
                                                        int32_t* __restrict__ assign_pos) {
  __shared__ int32_t fill[kMaxExperts];
  const int g = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kWave) fill[e] = offsets[e] + counts[(size_t)g * E + e];
  __syncthreads();
  const int64_t a_end = min<int64_t>(n, (int64_t)(g + 1) * kPermChunk);
  for (int64_t a0 = (int64_t)g * kPermChunk; a0 < a_end; a0 += kWave)
    place_wave(topk_idx, a_end, a0, fill, sorted_assign, assign_pos);
}

}  // namespace

hipError_t launch_permute(const moe_config* c, const int32_t* topk_idx, int32_t T, int32_t* offsets,
                          int32_t* sorted_assign, int32_t* assign_pos, int32_t* scratch, hipStream_t s) {
  const int E = c->n_expert, k = c->top_k, shared = c->shared_ff > 0;
  const int64_t n = (int64_t)T * k;
  if (n <= kPermSmallMax) {
    k_permute_small<<<1, kSmallThreads, 0, s>>>(topk_idx, T, k, E, shared, offsets, sorted_assign, assign_pos);
    return hipGetLastError();
  }
  const int G = (int)((n + kPermChunk - 1) / kPermChunk);
  k_perm_count<<<G, 256, 0, s>>>(topk_idx, n, E, scratch);
  k_perm_scan<<<1, 1024, 0, s>>>(scratch, G, T, k, E, shared, offsets, sorted_assign, assign_pos);
  k_perm_scatter<<<G, kWave, 0, s>>>(topk_idx, n, E, scratch, offsets, sorted_assign, assign_pos);
  return hipGetLastError();
}

}  // namespace moe
