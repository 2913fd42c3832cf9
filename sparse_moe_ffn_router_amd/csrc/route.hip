// Routing kernels: the router product for few tokens (one wavefront per
// router row) and the gating kernel (one wavefront per token).
//
// Sources: "qwen35moe - Forward-Pass Design (Pantheon port)", section
// "Shared-expert MoE FFN" (router logits = ffn_gate_inp . x, sigmoid shared
// gate); "Phase 19: MoE - gpt-oss-20b", section 2 Router (router bias).
#include "gating.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kRouterWaves = 1;   // router rows per workgroup (one per wave)

// Extended router rows: r < E is router_w[r] (written to logits[t][r] with
// the bias), r == E the shared-expert gate row (written to sgate_pre[t]).
// One wave per (row, group of TG tokens): blockIdx.y is the token group.
// PIECES 16-byte pieces per lane and token are loaded at once (the whole
// row when PIECES * 64 covers it), so a wave waits for memory once per
// chunk; a lane's pieces are summed in the same order whatever PIECES is.
template <typename XT, int PIECES, int TG>
__global__ __launch_bounds__(kRouterWaves * kWave) void k_router_gemv(
    const XT* __restrict__ x, const XT* __restrict__ wr, const XT* __restrict__ br,
    const XT* __restrict__ wsg, int32_t T, int32_t H, int32_t E, int32_t row0, int32_t row1,
    float* __restrict__ logits, float* __restrict__ sgate_pre) {
  const int r = row0 + blockIdx.x * kRouterWaves + (threadIdx.x / kWave);
  if (r >= row1) return;
  const int t0 = blockIdx.y * TG;
  router_row<XT, PIECES, TG>(x, wr, br, wsg, T, H, E, r, logits, sgate_pre, t0, min(T, t0 + TG));
}

// The same rows with the pre-norm block's prologue for few tokens: x is the
// residual stream, normalised on the fly by every wave (router_row_norm with
// P pieces per lane, sized to the row on the host), and the waves also write
// the normalised rows to xn for the expert kernels -- no separate
// normalisation launch.
template <typename XT, int P, int TG, bool PF>
__global__ __launch_bounds__(kRouterWaves * kWave) void k_router_gemv_norm(
    const XT* __restrict__ x, const XT* __restrict__ wr, const XT* __restrict__ br,
    const XT* __restrict__ wsg, int32_t T, int32_t H, int32_t E, int32_t row0, int32_t row1,
    float* __restrict__ logits, float* __restrict__ sgate_pre, const XT* __restrict__ g, float eps,
    XT* __restrict__ xn) {
  const int wave = blockIdx.x * kRouterWaves + (threadIdx.x / kWave);
  const int r = row0 + wave;
  if (r >= row1) return;
  router_row_norm<XT, P, TG, PF>(x, wr, br, wsg, g, eps, T, H, E, r, logits, sgate_pre, xn, wave, row1 - row0);
}

constexpr int kGateWaves = 4;  // tokens per workgroup

// sg_mode: 0 no shared expert; 1 sigmoid of the dot staged in sgate_pre;
// 2 the wave computes the dot itself from x and wsg.
// part / nsplit > 1: the router product came as nsplit partial sums over
// K ranges; the logits are their sum in range order plus the router bias,
// written to logits before the gating reads them back.
template <typename XT>
__global__ __launch_bounds__(kGateWaves * kWave) void k_gating(
    float* __restrict__ logits, const float* __restrict__ sgate_pre, const XT* __restrict__ x,
    const XT* __restrict__ wsg, int32_t H, int32_t sg_mode, int32_t T, int32_t E, int32_t k,
    int32_t softmax_first, int32_t renorm, float scale, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ sgate, const float* __restrict__ part, int32_t nsplit,
    const XT* __restrict__ br) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kGateWaves + threadIdx.x / kWave;
  if (t >= T) return;
  if (nsplit > 1) {
    // the ranges' partial sums, added in range order; the loads of up to 8
    // ranges of 4 chunks of 64 experts go out together
    constexpr int kC = 4, kU = 8;
    for (int e0 = 0; e0 < E; e0 += kC * kWave) {
      float v[kC];
#pragma unroll
      for (int c = 0; c < kC; ++c) v[c] = 0.f;
      for (int s0 = 0; s0 < nsplit; s0 += kU) {
        float pv[kC][kU];
#pragma unroll
        for (int c = 0; c < kC; ++c)
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int e = e0 + c * kWave + lane, sp = s0 + u;
            pv[c][u] = e < E && sp < nsplit ? part[((size_t)sp * T + t) * E + e] : 0.f;
          }
#pragma unroll
        for (int c = 0; c < kC; ++c)
#pragma unroll
          for (int u = 0; u < kU; ++u)
            if (s0 + u < nsplit) v[c] = s0 + u == 0 ? pv[c][u] : v[c] + pv[c][u];
      }
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const int e = e0 + c * kWave + lane;
        if (e < E) logits[(size_t)t * E + e] = br ? v[c] + RouterVec<XT>::scalar(br, e) : v[c];
      }
    }
  }
  gate_token(logits + (size_t)t * E, E, k, softmax_first, renorm, scale, topk_idx + (size_t)t * k,
             topk_w + (size_t)t * k);
  if (sg_mode == 2) {
    const float s = shared_gate_dot<XT>(x + (size_t)t * H, wsg, H);
    if (lane == 0) sgate[t] = 1.f / (1.f + expf(-s));
  } else if (sg_mode == 1 && lane == 0) {
    sgate[t] = 1.f / (1.f + expf(-sgate_pre[t]));
  }
}

}  // namespace

hipError_t launch_router_mfma(const moe_config* c, const moe_weights* w, const void* x, int32_t T, float* logits,
                              float* sgate_pre, hipStream_t s, float* part);  // ffn_mfma.hip
bool mfma_shapes_ok(const moe_config* c);

bool sgate_in_router(const moe_config* c, int32_t T) { return !(T > kGemvMaxT && mfma_shapes_ok(c)); }

bool router_norm_fusable(const moe_config* c, const moe_weights* w, int32_t T) {
  return w->router_w != nullptr && T <= kGemvMaxT && sgate_in_router(c, T);
}

hipError_t launch_router_logits(const moe_config* c, const moe_weights* w, const void* x, int32_t T,
                                float* logits, float* sgate_pre, hipStream_t s, float* part) {
  const int E = c->n_expert;
  const bool mfma = !sgate_in_router(c, T);
  const int row0 = w->router_w ? 0 : E;
  // with the MFMA router the shared-gate dot moves to the gating kernel
  const int row1 = (c->shared_ff > 0 && !mfma) ? E + 1 : E;
  if (row1 <= row0 || T == 0) return hipSuccess;
  if (mfma) return launch_router_mfma(c, w, x, T, logits, sgate_pre, s, part);
  const unsigned rows = (unsigned)((row1 - row0 + kRouterWaves - 1) / kRouterWaves);
  // rows of up to 256 pieces per lane set: 8 tokens per wave; longer rows
  // (whole row in flight, 6 or 8 pieces per lane): 4 tokens per wave
  const int pieces = c->hidden / (c->x_dtype == MOE_DTYPE_BF16 ? 8 : 4);
  if (c->x_dtype == MOE_DTYPE_BF16) {
    const uint16_t *xx = (const uint16_t*)x, *wr = (const uint16_t*)w->router_w, *br = (const uint16_t*)w->router_b,
                   *wg = (const uint16_t*)w->sh_gate_inp;
    if (pieces <= 4 * kWave)
      k_router_gemv<uint16_t, 4, 8><<<dim3(rows, (T + 7) / 8), kRouterWaves * kWave, 0, s>>>(
          xx, wr, br, wg, T, c->hidden, E, row0, row1, logits, sgate_pre);
    else if (pieces <= 6 * kWave)
      k_router_gemv<uint16_t, 6, 4><<<dim3(rows, (T + 3) / 4), kRouterWaves * kWave, 0, s>>>(
          xx, wr, br, wg, T, c->hidden, E, row0, row1, logits, sgate_pre);
    else
      k_router_gemv<uint16_t, 8, 4><<<dim3(rows, (T + 3) / 4), kRouterWaves * kWave, 0, s>>>(
          xx, wr, br, wg, T, c->hidden, E, row0, row1, logits, sgate_pre);
  } else {
    k_router_gemv<float, 4, 8><<<dim3(rows, (T + 7) / 8), kRouterWaves * kWave, 0, s>>>(
        (const float*)x, (const float*)w->router_w, (const float*)w->router_b, (const float*)w->sh_gate_inp, T,
        c->hidden, E, row0, row1, logits, sgate_pre);
  }
  return hipGetLastError();
}

template <typename XT, int P, int TG, bool PF>
static void router_norm_launch(const moe_config* c, const moe_weights* w, const void* resid, const void* g,
                               float eps, int32_t T, void* xn, float* logits, float* sgate_pre, hipStream_t s,
                               int row0, int row1) {
  dim3 grid((row1 - row0 + kRouterWaves - 1) / kRouterWaves);
  k_router_gemv_norm<XT, P, TG, PF><<<grid, kRouterWaves * kWave, 0, s>>>(
      (const XT*)resid, (const XT*)w->router_w, (const XT*)w->router_b, (const XT*)w->sh_gate_inp, T, c->hidden,
      c->n_expert, row0, row1, logits, sgate_pre, (const XT*)g, eps, (XT*)xn);
}

template <typename XT>
static void router_norm_dispatch(const moe_config* c, const moe_weights* w, const void* resid, const void* g,
                                 float eps, int32_t T, void* xn, float* logits, float* sgate_pre, hipStream_t s,
                                 int row0, int row1) {
  const int np = c->hidden / (16 / (int)sizeof(XT));  // 16-byte pieces per row (<= 512)
  if (np <= 64)
    router_norm_launch<XT, 1, 8, true>(c, w, resid, g, eps, T, xn, logits, sgate_pre, s, row0, row1);
  else if (np <= 128)
    router_norm_launch<XT, 2, 8, true>(c, w, resid, g, eps, T, xn, logits, sgate_pre, s, row0, row1);
  else if (np <= 256)
    router_norm_launch<XT, 4, 8, false>(c, w, resid, g, eps, T, xn, logits, sgate_pre, s, row0, row1);
  else if (np <= 384)
    router_norm_launch<XT, 6, 4, false>(c, w, resid, g, eps, T, xn, logits, sgate_pre, s, row0, row1);
  else
    router_norm_launch<XT, 8, 2, false>(c, w, resid, g, eps, T, xn, logits, sgate_pre, s, row0, row1);
}

hipError_t launch_router_logits_norm(const moe_config* c, const moe_weights* w, const void* resid, const void* g,
                                     float eps, int32_t T, void* xn, float* logits, float* sgate_pre, hipStream_t s) {
  // router_norm_fusable: router_w given and few tokens, so rows [0, E (+1)) run here
  const int row1 = c->shared_ff > 0 ? c->n_expert + 1 : c->n_expert;
  if (T == 0) return hipSuccess;
  if (c->x_dtype == MOE_DTYPE_BF16)
    router_norm_dispatch<uint16_t>(c, w, resid, g, eps, T, xn, logits, sgate_pre, s, 0, row1);
  else
    router_norm_dispatch<float>(c, w, resid, g, eps, T, xn, logits, sgate_pre, s, 0, row1);
  return hipGetLastError();
}

hipError_t launch_gating(const moe_config* c, const moe_weights* w, const void* x, float* logits,
                         const float* sgate_pre, int32_t T, int32_t* topk_idx, float* topk_w, float* sgate,
                         hipStream_t s, const float* part, int32_t nsplit) {
  if (T == 0) return hipSuccess;
  const int softmax_first = c->gating == MOE_GATING_SOFTMAX_TOPK;
  const int sg_mode = c->shared_ff <= 0 ? 0 : sgate_in_router(c, T) ? 1 : 2;
  const dim3 grid((T + kGateWaves - 1) / kGateWaves);
  if (c->x_dtype == MOE_DTYPE_BF16)
    k_gating<uint16_t><<<grid, kGateWaves * kWave, 0, s>>>(
        logits, sgate_pre, (const uint16_t*)x, (const uint16_t*)w->sh_gate_inp, c->hidden, sg_mode, T, c->n_expert,
        c->top_k, softmax_first, c->norm_topk_prob, c->weights_scale, topk_idx, topk_w, sgate, part, nsplit,
        (const uint16_t*)w->router_b);
  else
    k_gating<float><<<grid, kGateWaves * kWave, 0, s>>>(
        logits, sgate_pre, (const float*)x, (const float*)w->sh_gate_inp, c->hidden, sg_mode, T, c->n_expert,
        c->top_k, softmax_first, c->norm_topk_prob, c->weights_scale, topk_idx, topk_w, sgate, part, nsplit,
        (const float*)w->router_b);
  return hipGetLastError();
}

}  // namespace moe
