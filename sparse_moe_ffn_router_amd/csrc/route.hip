// Routing kernels: router product (fp32 logits plus the shared-expert gate
// dot) and gating (softmax / top-k with the first-seen tie-break / weights /
// sigmoid gate), one wavefront per token.
//
// Sources: "qwen35moe - Forward-Pass Design (Pantheon port)", section
// "Shared-expert MoE FFN" (router logits, softmax gating with
// norm_topk_prob and expert_weights_scale, sigmoid shared gate);
// "qwen35moe CPU-reference golden vectors", Kernel 4 (selection order and
// first-seen tie-break); "Phase 19: MoE - gpt-oss-20b", section 2 Router
// (router bias, top-k then softmax over the selected).
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kRouterTokens = 8;   // tokens per wave pass
constexpr int kRouterWaves = 4;    // rows per workgroup (one per wave)

// Element loads: 16 bytes per lane per step (8 bf16 or 4 fp32).
template <typename XT> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* v) {
    uint4 q = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16lo(q.x); v[1] = bf16hi(q.x); v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
    v[4] = bf16lo(q.z); v[5] = bf16hi(q.z); v[6] = bf16lo(q.w); v[7] = bf16hi(q.w);
  }
  __device__ static float scalar(const uint16_t* p, int i) { return __uint_as_float((uint32_t)p[i] << 16); }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* v) {
    float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  __device__ static float scalar(const float* p, int i) { return p[i]; }
};

// Extended router rows: r < E is router_w[r] (written to logits[t][r] with
// the bias), r == E is the shared-expert gate row (written to sgate_pre[t]).
// One wave per row and kRouterTokens tokens; lanes split the hidden dim in
// 16-byte pieces.  Every row is reduced in the same order, so bit-equal
// router rows give bit-equal logits.
template <typename XT>
__global__ __launch_bounds__(kRouterWaves * kWave) void k_router_logits(
    const XT* __restrict__ x, const XT* __restrict__ wr, const XT* __restrict__ br,
    const XT* __restrict__ wsg, int32_t T, int32_t H, int32_t E, int32_t row0, int32_t row1,
    float* __restrict__ logits, float* __restrict__ sgate_pre) {
  constexpr int N = Vec<XT>::N;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = row0 + blockIdx.x * kRouterWaves + (threadIdx.x / kWave);
  const int t0 = blockIdx.y * kRouterTokens;
  if (r >= row1) return;
  const XT* wrow = r < E ? wr + (size_t)r * H : wsg;
  const int nt = min(kRouterTokens, T - t0);
  float acc[kRouterTokens];
#pragma unroll
  for (int i = 0; i < kRouterTokens; ++i) acc[i] = 0.f;
  for (int c = lane * N; c < H; c += kWave * N) {
    float wv[N];
    Vec<XT>::load(wrow + c, wv);
#pragma unroll
    for (int i = 0; i < kRouterTokens; ++i) {
      if (i < nt) {
        float xv[N];
        Vec<XT>::load(x + (size_t)(t0 + i) * H + c, xv);
#pragma unroll
        for (int q = 0; q < N; ++q) acc[i] = fmaf(wv[q], xv[q], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRouterTokens; ++i) acc[i] = wave_sum(acc[i]);
  if (lane < nt) {
    float v = acc[0];
#pragma unroll
    for (int i = 1; i < kRouterTokens; ++i) v = lane == i ? acc[i] : v;
    if (r < E) {
      if (br) v += Vec<XT>::scalar(br, r);
      logits[(size_t)(t0 + lane) * E + r] = v;
    } else {
      sgate_pre[t0 + lane] = v;
    }
  }
}

constexpr int kGateWaves = 4;  // tokens per workgroup
constexpr int kMaxPerLane = kMaxExperts / kWave;

// One wave per token.  Top-k runs k rounds of a wave-wide maximum over
// 64-bit keys (order_key(logit) << 32 | ~expert): the largest logit wins,
// and among bit-equal logits the lowest expert id -- the first one a
// left-to-right selection sort would keep.
__global__ __launch_bounds__(kGateWaves * kWave) void k_gating(
    const float* __restrict__ logits, const float* __restrict__ sgate_pre, int32_t T, int32_t E, int32_t k,
    int32_t softmax_first, int32_t renorm, float scale, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ sgate) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kGateWaves + threadIdx.x / kWave;
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  uint64_t key[kMaxPerLane];
  float val[kMaxPerLane];
  const int nper = (E + kWave - 1) / kWave;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = i * kWave + lane;
    const bool ok = i < nper && e < E;
    val[i] = ok ? l[e] : -INFINITY;
    key[i] = ok ? (((uint64_t)order_key(val[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0ull;
  }
  uint32_t used = 0;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (!((used >> i) & 1u) && key[i] > best) best = key[i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      uint64_t other = __shfl_xor(best, o, kWave);
      best = other > best ? other : best;
    }
    const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
    if ((e & (kWave - 1)) == lane) used |= 1u << (e / kWave);
    if (lane == j) my_idx = e;
  }
  // pick 0 holds the largest logit, the softmax shift for both gatings
  const float m = l[__shfl(my_idx, 0, kWave)];
  const float ej = lane < k ? expf(l[my_idx] - m) : 0.f;
  float denom;
  if (!softmax_first || renorm) {
    denom = wave_sum(ej);
  } else {
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) z += (i < nper && i * kWave + lane < E) ? expf(val[i] - m) : 0.f;
    denom = wave_sum(z);
  }
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_idx;
    topk_w[(size_t)t * k + lane] = ej / denom * scale;
  }
  if (sgate && lane == 0) sgate[t] = 1.f / (1.f + expf(-sgate_pre[t]));
}

}  // namespace

hipError_t launch_router_logits(const moe_config* c, const moe_weights* w, const void* x, int32_t T,
                                float* logits, float* sgate_pre, hipStream_t s) {
  const int E = c->n_expert;
  const int row0 = w->router_w ? 0 : E;
  const int row1 = c->shared_ff > 0 ? E + 1 : E;
  if (row1 <= row0 || T == 0) return hipSuccess;
  dim3 grid((row1 - row0 + kRouterWaves - 1) / kRouterWaves, (T + kRouterTokens - 1) / kRouterTokens);
  if (c->x_dtype == MOE_DTYPE_BF16)
    k_router_logits<uint16_t><<<grid, kRouterWaves * kWave, 0, s>>>(
        (const uint16_t*)x, (const uint16_t*)w->router_w, (const uint16_t*)w->router_b,
        (const uint16_t*)w->sh_gate_inp, T, c->hidden, E, row0, row1, logits, sgate_pre);
  else
    k_router_logits<float><<<grid, kRouterWaves * kWave, 0, s>>>(
        (const float*)x, (const float*)w->router_w, (const float*)w->router_b, (const float*)w->sh_gate_inp, T,
        c->hidden, E, row0, row1, logits, sgate_pre);
  return hipGetLastError();
}

hipError_t launch_gating(const moe_config* c, const float* logits, const float* sgate_pre, int32_t T,
                         int32_t* topk_idx, float* topk_w, float* sgate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int softmax_first = c->gating == MOE_GATING_SOFTMAX_TOPK;
  k_gating<<<(T + kGateWaves - 1) / kGateWaves, kGateWaves * kWave, 0, s>>>(
      logits, sgate_pre, T, c->n_expert, c->top_k, softmax_first, c->norm_topk_prob, c->weights_scale, topk_idx,
      topk_w, c->shared_ff > 0 ? sgate : nullptr);
  return hipGetLastError();
}

}  // namespace moe
