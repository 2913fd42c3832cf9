// Token -> expert permutation: a stable counting sort of the T*k
// token-expert assignments a = t*k + j by expert id.
//
// A token picks each expert at most once, so inside an expert's segment
// ascending a is ascending token.  For every expert the kernels build a
// bitmask over a block of tokens (bit t set when token t picked the expert)
// with LDS atomic ORs, whose result does not depend on their order; an
// assignment's rank in its segment is then the popcount of the mask below
// its token plus the counts of earlier blocks.  Positions are therefore
// deterministic and need no serial pass.
//
// The pages only imply this step ("qwen35moe - Forward-Pass Design",
// section "K80 GPU decode": grouped expert launches; section "Batched
// prefill": tokens sharing an expert stream its weights once).
#include "gating.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kThreadsBig = 1024;
constexpr int kBlockTokens = 256;             // tokens per mask block
constexpr int kWords = kBlockTokens / 64;     // 64-bit words per expert mask

__device__ __forceinline__ uint64_t lower_bits(int t) { return t ? (~0ull >> (64 - t)) : 0ull; }

// The k picks of one token, made distinct and in range, in place (one
// thread per token).  The contract asks each token for k distinct experts
// in [0, E), which the gating always gives; a caller's picks that break it
// (an id out of range, or one repeating an earlier pick of the token) are
// replaced, in slot order, by the lowest experts the token's valid picks
// leave free (k <= E, so there are enough).  The permutation is then always
// a bijection with full segments, so no later kernel reads or writes past a
// buffer, whatever the picks held.
__device__ void make_picks_distinct(int32_t* p, int k, int E) {
  int v[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) v[j] = j < k ? p[j] : 0;
  uint32_t bad = 0;  // slots to replace
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      bool b = (unsigned)v[j] >= (unsigned)E;
#pragma unroll
      for (int i = 0; i < j; ++i) b = b || (((bad >> i) & 1u) == 0 && v[i] == v[j]);
      bad |= (uint32_t)b << j;
    }
  }
  if (!bad) return;  // the contract holds (always, after the gating)
  int cand = 0;
  for (int j = 0; j < k; ++j) {
    if (!((bad >> j) & 1u)) continue;
    for (;; ++cand) {
      bool used = false;
      for (int i = 0; i < k && !used; ++i) used = ((bad >> i) & 1u) == 0 && p[i] == cand;
      if (!used) break;
    }
    p[j] = cand++;
  }
}

// Exclusive scan of v over the first n threads of a 1024-thread block
// (n <= 1024); returns the exclusive prefix, *total gets the sum.
__device__ int block_excl_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) wsum[wid] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w2 = 0; w2 < kThreadsBig / kWave; ++w2) {
    const int s = wsum[w2];
    before += w2 < wid ? s : 0;
    all += s;
  }
  *total = all;
  return before + incl - v;
}

// Permutation of up to kBlockTokens tokens inside one workgroup, from the
// picks in LDS (idx_s, T*k entries); with segtab, also the segment-slot
// table of nslots entries {expert, first sorted position, rows, 0}: slot 0
// the shared expert when there is one, then the non-empty routed segments
// in expert order, then {-1, 0, 0, 0}.
__device__ void permute_one_block(const int32_t* idx_s, int32_t T, int32_t k, int32_t E, int32_t shared,
                                  uint64_t* mask, int* base, int* wsum, int32_t* __restrict__ offsets,
                                  int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos,
                                  int32_t* __restrict__ segtab = nullptr, int nslots = 0) {
  const int tid = threadIdx.x;
  const int n = T * k;
  const int W = (T + 63) / 64;
  for (int i = tid; i < E * W; i += kThreadsBig) mask[i] = 0ull;
  __syncthreads();
  for (int a = tid; a < n; a += kThreadsBig) {
    const int t = a / k;
    atomicOr((unsigned long long*)&mask[idx_s[a] * W + t / 64], 1ull << (t & 63));
  }
  __syncthreads();
  int cnt = 0;
  if (tid < E)
    for (int w = 0; w < W; ++w) cnt += __popcll(mask[tid * W + w]);
  // one scan gives both the segment starts (low 20 bits: n = T*k <= 256*32
  // here) and each non-empty segment's slot (the count of non-empty ones
  // before it, high bits: E <= 1024)
  int total;
  const int packed = block_excl_scan(tid < E ? cnt + (cnt > 0 ? 1 << 20 : 0) : 0, wsum, &total);
  const int excl = packed & 0xFFFFF;
  if (tid < E) {
    base[tid] = excl;
    offsets[tid] = excl;
  }
  if (tid == 0) {
    offsets[E] = n;
    if (shared) offsets[E + 1] = n + T;
  }
  __syncthreads();
  if (segtab) {
    const int nact = total >> 20, r = packed >> 20;
    int4* tab = reinterpret_cast<int4*>(segtab);
    if (tid < E && cnt > 0 && shared + r < nslots) tab[shared + r] = make_int4(tid, excl, cnt, 0);
    if (tid == 0 && shared) tab[0] = make_int4(E, n, T, 0);
    for (int q = shared + nact + tid; q < nslots; q += kThreadsBig) tab[q] = make_int4(-1, 0, 0, 0);
  }
  for (int a = tid; a < n; a += kThreadsBig) {
    const int t = a / k, e = idx_s[a];
    int r = __popcll(mask[e * W + t / 64] & lower_bits(t & 63));
    for (int w = 0; w < t / 64; ++w) r += __popcll(mask[e * W + w]);
    const int pos = base[e] + r;
    sorted_assign[pos] = a;
    assign_pos[a] = pos;
  }
  if (shared)
    for (int t = tid; t < T; t += kThreadsBig) {
      sorted_assign[n + t] = n + t;
      assign_pos[n + t] = n + t;
    }
}

// Up to kBlockTokens tokens: the whole permutation in one workgroup.
__global__ __launch_bounds__(kThreadsBig) void k_permute_small(const int32_t* __restrict__ topk_idx, int32_t T,
                                                               int32_t k, int32_t E, int32_t shared,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_assign,
                                                               int32_t* __restrict__ assign_pos) {
  __shared__ uint64_t mask[kMaxExperts * kWords];
  __shared__ int32_t idx_s[kBlockTokens * kMaxTopK];
  __shared__ int base[kMaxExperts];
  __shared__ int wsum[kThreadsBig / kWave];
  for (int a = threadIdx.x; a < T * k; a += kThreadsBig) idx_s[a] = topk_idx[a];
  __syncthreads();
  if (threadIdx.x < T) make_picks_distinct(idx_s + threadIdx.x * k, k, E);
  __syncthreads();
  permute_one_block(idx_s, T, k, E, shared, mask, base, wsum, offsets, sorted_assign, assign_pos);
}

// Gating and permutation of a small batch (T <= 16) in one workgroup: wave t
// gates token t, then the block permutes.
__global__ __launch_bounds__(kThreadsBig) void k_gate_permute_small(
    const float* __restrict__ logits, const float* __restrict__ sgate_pre, int32_t T, int32_t E, int32_t k,
    int32_t softmax_first, int32_t renorm, float scale, int32_t shared, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ sgate, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos, int32_t* __restrict__ segtab,
    int32_t nslots) {
  __shared__ uint64_t mask[kMaxExperts];
  __shared__ int32_t idx_s[16 * kMaxTopK];
  __shared__ int base[kMaxExperts];
  __shared__ int wsum[kThreadsBig / kWave];
  const int lane = threadIdx.x & (kWave - 1), t = threadIdx.x / kWave;
  if (t < T) {
    const int e = gate_token(logits + (size_t)t * E, E, k, softmax_first, renorm, scale, topk_idx + (size_t)t * k,
                             topk_w + (size_t)t * k);
    if (lane < k) idx_s[t * k + lane] = e;
    if (shared && lane == 0) sgate[t] = 1.f / (1.f + expf(-sgate_pre[t]));
  }
  __syncthreads();
  permute_one_block(idx_s, T, k, E, shared, mask, base, wsum, offsets, sorted_assign, assign_pos, segtab, nslots);
}

// Large batches, pass 1: masks and counts of one block of kBlockTokens
// tokens, stored to scratch (masks [G][E][kWords], counts [G][E]); the
// block's picks, made distinct per token, go to picks [T][k] for pass 3.
__global__ __launch_bounds__(kThreadsBig) void k_perm_masks(const int32_t* __restrict__ topk_idx, int32_t T,
                                                            int32_t k, int32_t E, uint64_t* __restrict__ gmask,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ picks) {
  __shared__ uint64_t mask[kMaxExperts * kWords];
  __shared__ int32_t idx_s[kBlockTokens * kMaxTopK];
  const int g = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < E * kWords; i += kThreadsBig) mask[i] = 0ull;
  const int t0 = g * kBlockTokens;
  const int nt = min(kBlockTokens, T - t0);
  for (int i = tid; i < nt * k; i += kThreadsBig) idx_s[i] = topk_idx[(size_t)t0 * k + i];
  __syncthreads();
  if (tid < nt) make_picks_distinct(idx_s + tid * k, k, E);
  __syncthreads();
  for (int i = tid; i < nt * k; i += kThreadsBig) {
    const int tl = i / k;
    const int e = idx_s[i];
    picks[(size_t)t0 * k + i] = e;
    atomicOr((unsigned long long*)&mask[e * kWords + tl / 64], 1ull << (tl & 63));
  }
  __syncthreads();
  for (int i = tid; i < E * kWords; i += kThreadsBig) gmask[(size_t)g * E * kWords + i] = mask[i];
  if (tid < E) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) c += __popcll(mask[tid * kWords + w]);
    counts[(size_t)g * E + tid] = c;
  }
}

// Pass 2 (one workgroup): expert offsets and each block's start inside each
// segment (counts[g][e] becomes that start).
__global__ __launch_bounds__(kThreadsBig) void k_perm_scan(int32_t* __restrict__ counts, int32_t G, int32_t T,
                                                           int32_t k, int32_t E, int32_t shared,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_assign,
                                                           int32_t* __restrict__ assign_pos) {
  __shared__ int wsum[kThreadsBig / kWave];
  constexpr int kU = 8;  // block counts loaded per round trip
  const int tid = threadIdx.x;
  int tot = 0;
  if (tid < E)
    for (int g0 = 0; g0 < G; g0 += kU) {
      int c[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) c[u] = g0 + u < G ? counts[(size_t)(g0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < kU; ++u) tot += c[u];
    }
  int all;
  const int excl = block_excl_scan(tid < E ? tot : 0, wsum, &all);
  if (tid < E) {
    offsets[tid] = excl;
    int run = excl;
    for (int g0 = 0; g0 < G; g0 += kU) {
      int c[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) c[u] = g0 + u < G ? counts[(size_t)(g0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (g0 + u < G) counts[(size_t)(g0 + u) * E + tid] = run;
        run += c[u];
      }
    }
  }
  const int n = T * k;
  if (tid == 0) {
    offsets[E] = n;
    if (shared) offsets[E + 1] = n + T;
  }
  if (shared)
    for (int t = tid; t < T; t += kThreadsBig) {
      sorted_assign[n + t] = n + t;
      assign_pos[n + t] = n + t;
    }
}

// Pass 3: every assignment's position from its block's masks and start.
__global__ __launch_bounds__(256) void k_perm_place(const int32_t* __restrict__ topk_idx, int32_t T, int32_t k,
                                                    int32_t E, const uint64_t* __restrict__ gmask,
                                                    const int32_t* __restrict__ start,
                                                    int32_t* __restrict__ sorted_assign,
                                                    int32_t* __restrict__ assign_pos) {
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a >= T * k) return;
  const int t = a / k, e = topk_idx[a];
  const int g = t / kBlockTokens, tl = t % kBlockTokens;
  const uint64_t* m = gmask + ((size_t)g * E + e) * kWords;
  int r = __popcll(m[tl / 64] & lower_bits(tl & 63));
  for (int w = 0; w < tl / 64; ++w) r += __popcll(m[w]);
  const int pos = start[(size_t)g * E + e] + r;
  sorted_assign[pos] = a;
  assign_pos[a] = pos;
}

}  // namespace

size_t permute_scratch_bytes(int32_t T, int32_t E, int32_t k) {
  const size_t G = (size_t)(T + kBlockTokens - 1) / kBlockTokens;
  return G * E * kWords * sizeof(uint64_t) + G * E * sizeof(int32_t) + (size_t)T * k * sizeof(int32_t);
}

hipError_t launch_permute(const moe_config* c, const int32_t* topk_idx, int32_t T, int32_t* offsets,
                          int32_t* sorted_assign, int32_t* assign_pos, int32_t* scratch, hipStream_t s) {
  const int E = c->n_expert, k = c->top_k, shared = c->shared_ff > 0;
  if (T == 0) return hipSuccess;
  if (T <= kBlockTokens) {
    k_permute_small<<<1, kThreadsBig, 0, s>>>(topk_idx, T, k, E, shared, offsets, sorted_assign, assign_pos);
    return hipGetLastError();
  }
  const int G = (T + kBlockTokens - 1) / kBlockTokens;
  uint64_t* gmask = reinterpret_cast<uint64_t*>(scratch);
  int32_t* counts = reinterpret_cast<int32_t*>(gmask + (size_t)G * E * kWords);
  int32_t* picks = counts + (size_t)G * E;
  k_perm_masks<<<G, kThreadsBig, 0, s>>>(topk_idx, T, k, E, gmask, counts, picks);
  k_perm_scan<<<1, kThreadsBig, 0, s>>>(counts, G, T, k, E, shared, offsets, sorted_assign, assign_pos);
  k_perm_place<<<(T * k + 255) / 256, 256, 0, s>>>(picks, T, k, E, gmask, counts, sorted_assign, assign_pos);
  return hipGetLastError();
}

bool can_fuse_gate_permute(int32_t T) { return T > 0 && T <= 16; }

hipError_t launch_gate_permute(const moe_config* c, const float* logits, const float* sgate_pre, int32_t T,
                               int32_t* topk_idx, float* topk_w, float* sgate, int32_t* offsets,
                               int32_t* sorted_assign, int32_t* assign_pos, hipStream_t s, int32_t* segtab,
                               int nslots) {
  const int softmax_first = c->gating == MOE_GATING_SOFTMAX_TOPK;
  const int shared = c->shared_ff > 0;
  k_gate_permute_small<<<1, kThreadsBig, 0, s>>>(logits, sgate_pre, T, c->n_expert, c->top_k, softmax_first,
                                                 c->norm_topk_prob, c->weights_scale, shared, topk_idx, topk_w,
                                                 shared ? sgate : nullptr, offsets, sorted_assign, assign_pos,
                                                 segtab, segtab ? nslots : 0);
  return hipGetLastError();
}

}  // namespace moe
