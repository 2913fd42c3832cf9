// Gating of one token by one wavefront, shared by the gating kernels.
//
// "qwen35moe - Forward-Pass Design", section "Shared-expert MoE FFN":
// softmax over all experts, keep the top-k, renormalise them
// (norm_topk_prob) and multiply by expert_weights_scale.  "qwen35moe
// CPU-reference golden vectors", Kernel 4: selection sort with first-seen
// tie-break, picks in selection order.  "Phase 19: MoE - gpt-oss-20b",
// section 2 Router: top-k of the biased logits, softmax over the k picks.
#pragma once
#include "moe_internal.hpp"

namespace moe {

// Returns, in lane j < k, the expert of pick j; writes topk_idx / topk_w of
// the token.  The top-k runs k rounds of a wave-wide maximum of 64-bit keys
// order_key(logit) << 32 | (2^32 - 1 - expert): the largest logit wins, and
// among bit-equal logits the lowest expert id, as a left-to-right selection
// sort with strict comparison keeps the first one it sees.
// NPER = experts held per lane (E <= 64 * NPER).
template <int NPER>
__device__ __forceinline__ int gate_token_n(const float* __restrict__ l, int E, int k, int softmax_first, int renorm,
                                            float scale, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t key[NPER];
  float val[NPER];
  const int nper = NPER;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = i * kWave + lane;
    const bool ok = i < nper && e < E;
    val[i] = ok ? l[e] : -INFINITY;
    key[i] = ok ? (((uint64_t)order_key(val[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0ull;
  }
  uint32_t used = 0;
  int my_idx = 0;
  uint32_t my_key = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (!((used >> i) & 1u) && key[i] > best) best = key[i];
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
    if ((e & (kWave - 1)) == lane) used |= 1u << (e / kWave);
    if (lane == j) {
      my_idx = e;
      my_key = (uint32_t)(best >> 32);
    }
  }
  // the pick's logit back from its key (order_key is invertible; a -0 logit
  // comes back as +0, which exp() treats the same)
  const float my_val = __uint_as_float((my_key & 0x80000000u) ? (my_key & 0x7FFFFFFFu) : ~my_key);
  // pick 0 holds the largest logit, the softmax shift for both gatings
  const float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_val), 0));
  const float ej = lane < k ? expf(my_val - m) : 0.f;
  float denom;
  if (!softmax_first || renorm) {
    denom = wave_sum(ej);
  } else {
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < NPER; ++i) z += (i * kWave + lane < E) ? expf(val[i] - m) : 0.f;
    denom = wave_sum(z);
  }
  if (lane < k) {
    topk_idx[lane] = my_idx;
    topk_w[lane] = ej / denom * scale;
  }
  return my_idx;
}

__device__ __forceinline__ int gate_token(const float* __restrict__ l, int E, int k, int softmax_first, int renorm,
                                          float scale, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  if (E <= 64) return gate_token_n<1>(l, E, k, softmax_first, renorm, scale, topk_idx, topk_w);
  if (E <= 128) return gate_token_n<2>(l, E, k, softmax_first, renorm, scale, topk_idx, topk_w);
  if (E <= 256) return gate_token_n<4>(l, E, k, softmax_first, renorm, scale, topk_idx, topk_w);
  if (E <= 512) return gate_token_n<8>(l, E, k, softmax_first, renorm, scale, topk_idx, topk_w);
  return gate_token_n<16>(l, E, k, softmax_first, renorm, scale, topk_idx, topk_w);
}

// Shared-expert gate of token t computed by one wave: sigmoid(wsg . x[t]).
template <typename XT>
__device__ __forceinline__ float shared_gate_dot(const XT* __restrict__ xrow, const XT* __restrict__ wsg, int H);
template <>
__device__ __forceinline__ float shared_gate_dot<uint16_t>(const uint16_t* __restrict__ xrow,
                                                           const uint16_t* __restrict__ wsg, int H) {
  const int lane = threadIdx.x & (kWave - 1);
  float acc = 0.f;
  for (int c = lane * 8; c < H; c += kWave * 8) {
    const uint4 a = *reinterpret_cast<const uint4*>(xrow + c);
    const uint4 b = *reinterpret_cast<const uint4*>(wsg + c);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, b.x), __builtin_bit_cast(bf16x2_t, a.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, b.y), __builtin_bit_cast(bf16x2_t, a.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, b.z), __builtin_bit_cast(bf16x2_t, a.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, b.w), __builtin_bit_cast(bf16x2_t, a.w), acc, false);
  }
  return wave_sum(acc);
}
template <>
__device__ __forceinline__ float shared_gate_dot<float>(const float* __restrict__ xrow, const float* __restrict__ wsg,
                                                        int H) {
  const int lane = threadIdx.x & (kWave - 1);
  float acc = 0.f;
  for (int c = lane * 4; c < H; c += kWave * 4) {
    const float4 a = *reinterpret_cast<const float4*>(xrow + c);
    const float4 b = *reinterpret_cast<const float4*>(wsg + c);
    acc = fmaf(b.x, a.x, acc);
    acc = fmaf(b.y, a.y, acc);
    acc = fmaf(b.z, a.z, acc);
    acc = fmaf(b.w, a.w, acc);
  }
  return wave_sum(acc);
}

}  // namespace moe
