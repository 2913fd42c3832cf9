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

// Wave-wide maximum / minimum of a 32-bit value, wave-uniform result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppHalfMirror>(v));
  v = max(v, dpp_u32<kDppMirror>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kDppXor1>(v));
  v = min(v, dpp_u32<kDppXor2>(v));
  v = min(v, dpp_u32<kDppHalfMirror>(v));
  v = min(v, dpp_u32<kDppMirror>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(a, b), min(c, d));
}

// Returns, in lane j < k, the expert of pick j; writes topk_idx / topk_w of
// the token.  The top-k runs k rounds of: each lane's largest unpicked
// order_key(logit) (order_key is monotone in the logit and folds -0 into
// +0; expert e = i * 64 + lane sits in slot i of its lane, and a lane keeps
// its lowest slot among equal keys), the wave-wide maximum of those, and,
// among the lanes holding that maximum, the lowest expert id -- so the
// largest logit wins and bit-equal logits go to the lowest index, as a
// left-to-right selection sort with strict comparison keeps the first one
// it sees.  A picked slot's key becomes 0, below every valid key.
// NPER = experts held per lane (E <= 64 * NPER).
template <int NPER>
__device__ __forceinline__ int gate_token_n(const float* __restrict__ l, int E, int k, int softmax_first, int renorm,
                                            float scale, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t key[NPER];
  float val[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = i * kWave + lane;
    const bool ok = e < E;
    val[i] = ok ? l[e] : -INFINITY;
    key[i] = ok ? order_key(val[i]) : 0u;
  }
  int my_idx = 0;
  uint32_t my_key = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t best = key[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < NPER; ++i)
      if (key[i] > best) {
        best = key[i];
        bi = i;
      }
    const uint32_t wmax = wave_max_u32(best);
    const uint64_t tied = __ballot(best == wmax);
    int e;
    if (__popcll(tied) == 1) {
      const int wl = __ffsll((unsigned long long)tied) - 1;
      e = __builtin_amdgcn_readlane(bi, wl) * kWave + wl;
    } else {
      e = (int)wave_min_u32(best == wmax ? (uint32_t)(bi * kWave + lane) : 0xFFFFFFFFu);
    }
    if ((e & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (i == e / kWave) key[i] = 0u;
    }
    if (lane == j) {
      my_idx = e;
      my_key = wmax;
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

constexpr int kRouterTokens = 8;  // tokens per pass of a wave

// RMSNorm element helpers (the pre-norm block's prologue): sum of squares
// of one 16-byte piece, and a piece scaled by the row factor r and the norm
// weight, rounded to the activation type (x * r first, then * weight).
__device__ __forceinline__ float sumsq4(uint4 v, uint16_t) {
  float s = 0.f;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(bf16lo(w[i]), bf16lo(w[i]), s);
    s = fmaf(bf16hi(w[i]), bf16hi(w[i]), s);
  }
  return s;
}
__device__ __forceinline__ float sumsq4(uint4 v, float) {
  float s = 0.f;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) s = fmaf(__uint_as_float(w[i]), __uint_as_float(w[i]), s);
  return s;
}

__device__ __forceinline__ uint4 scale4(uint4 v, uint4 g, float r, uint16_t) {
  const uint32_t a[4] = {v.x, v.y, v.z, v.w}, b[4] = {g.x, g.y, g.z, g.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // gfx950 converts a pair to bf16 in one instruction, nearest-even
    const bf16x2_t p = {(__bf16)(bf16lo(a[i]) * r * bf16lo(b[i])), (__bf16)(bf16hi(a[i]) * r * bf16hi(b[i]))};
    o[i] = __builtin_bit_cast(uint32_t, p);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
__device__ __forceinline__ uint4 scale4(uint4 v, uint4 g, float r, float) {
  return make_uint4(__float_as_uint(__uint_as_float(v.x) * r * __uint_as_float(g.x)),
                    __float_as_uint(__uint_as_float(v.y) * r * __uint_as_float(g.y)),
                    __float_as_uint(__uint_as_float(v.z) * r * __uint_as_float(g.z)),
                    __float_as_uint(__uint_as_float(v.w) * r * __uint_as_float(g.w)));
}


template <typename XT> struct RouterVec;
template <> struct RouterVec<uint16_t> {
  static constexpr int N = 8;
  __device__ static float dot(uint4 w, uint4 x, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), acc, false);
    return acc;
  }
  __device__ static float scalar(const uint16_t* p, int i) { return __uint_as_float((uint32_t)p[i] << 16); }
};
template <> struct RouterVec<float> {
  static constexpr int N = 4;
  __device__ static float dot(uint4 w, uint4 x, float acc) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
    return acc;
  }
  __device__ static float scalar(const float* p, int i) { return p[i]; }
};

// One extended router row by one wavefront: r < E is router_w[r] (written,
// with the bias, to logits[t][r]), r == E the shared-expert gate row
// (written to sgate_pre[t]).  Lane l holds 16-byte pieces l, l+64, ... of
// the row and multiplies them with the same pieces of up to 8 tokens at a
// time; every row is reduced in the same order, so bit-equal router rows
// give bit-equal logits.  PIECES: 16-byte pieces per lane and token held at
// once; all of a chunk's loads are issued before its first product.
// The wave takes tokens [t_begin, t_end) in groups of TG.
template <typename XT, int PIECES, int TG = kRouterTokens>
__device__ __forceinline__ void router_row(const XT* __restrict__ x, const XT* __restrict__ wr,
                                           const XT* __restrict__ br, const XT* __restrict__ wsg, int T, int H,
                                           int E, int r, float* __restrict__ logits, float* __restrict__ sgate_pre,
                                           int t_begin = 0, int t_end = -1) {
  constexpr int N = RouterVec<XT>::N;
  const int lane = threadIdx.x & (kWave - 1);
  const uint4* wrow = reinterpret_cast<const uint4*>(r < E ? wr + (size_t)r * H : wsg);
  const int npieces = H / N;
  const float bias = (r < E && br) ? RouterVec<XT>::scalar(br, r) : 0.f;
  if (t_end < 0) t_end = T;
  for (int t0 = t_begin; t0 < t_end; t0 += TG) {
    float acc[TG];
#pragma unroll
    for (int j = 0; j < TG; ++j) acc[j] = 0.f;
    for (int p0 = 0; p0 < npieces; p0 += PIECES * kWave) {
      // every load of the chunk (row pieces and the tokens' pieces) is
      // issued before the first product, so the wave waits once per chunk
      uint4 w[PIECES], xv[TG][PIECES];
#pragma unroll
      for (int i = 0; i < PIECES; ++i) {
        const int pc = p0 + i * kWave + lane;
        w[i] = pc < npieces ? wrow[pc] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < TG; ++j) {
        const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + j, T - 1) * H);
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
          const int pc = p0 + i * kWave + lane;
          xv[j][i] = pc < npieces ? xr[pc] : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < TG; ++j)
#pragma unroll
        for (int i = 0; i < PIECES; ++i) acc[j] = RouterVec<XT>::dot(w[i], xv[j][i], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < TG; ++j) acc[j] = wave_sum(acc[j]);
    if (lane < TG && t0 + lane < t_end) {
      float v = acc[0];
#pragma unroll
      for (int j = 1; j < TG; ++j) v = lane == j ? acc[j] : v;
      if (r < E)
        logits[(size_t)(t0 + lane) * E + r] = v + bias;
      else
        sgate_pre[t0 + lane] = v;
    }
  }
}

// router_row with the pre-norm block's RMSNorm folded in: x holds the
// un-normalised rows, g the norm weight.  A whole row (P 16-byte pieces per
// lane, P * 64 >= H / (16 / sizeof(XT))) is held in registers, so each
// token's factor 1 / sqrt(mean(x^2) + eps) comes from the pieces already
// loaded for the product, and each piece is normalised and rounded to the
// activation type before it is multiplied -- the same values, sums and
// order as the RMSNorm kernel followed by router_row, so the logits are
// bit-equal to those.  The weight row and g stay in registers over all
// tokens; tokens go in groups of TG (PF: the next group's rows load while
// the current group's sums are reduced, for widths where the registers
// allow it).  Wave `wave` of `nwaves` also
// stores the normalised rows t with t % nwaves == wave to xn for the expert
// kernels.
template <typename XT, int P, int TG, bool PF>
__device__ __forceinline__ void router_row_norm(const XT* __restrict__ x, const XT* __restrict__ wr,
                                                const XT* __restrict__ br, const XT* __restrict__ wsg,
                                                const XT* __restrict__ g, float eps, int T, int H, int E, int r,
                                                float* __restrict__ logits, float* __restrict__ sgate_pre,
                                                XT* __restrict__ xn, int wave, int nwaves) {
  constexpr int N = RouterVec<XT>::N;
  const int lane = threadIdx.x & (kWave - 1);
  const int np = H / N;
  const uint4* wrow = reinterpret_cast<const uint4*>(r < E ? wr + (size_t)r * H : wsg);
  const uint4* grow = reinterpret_cast<const uint4*>(g);
  uint4 w[P], gv[P], xv[TG][P];
  auto load_group = [&](int t0) {
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + j, T - 1) * H);
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int pc = lane + i * kWave;
        xv[j][i] = pc < np ? xr[pc] : make_uint4(0, 0, 0, 0);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int pc = lane + i * kWave;
    w[i] = pc < np ? wrow[pc] : make_uint4(0, 0, 0, 0);
    gv[i] = pc < np ? grow[pc] : make_uint4(0, 0, 0, 0);
  }
  load_group(0);
  // after the row loads, so that its wait (layers with a router bias) comes
  // with theirs at the loop entry
  const float bias = (r < E && br) ? RouterVec<XT>::scalar(br, r) : 0.f;
  for (int t0 = 0; t0 < T; t0 += TG) {
    if constexpr (!PF) {
      if (t0 > 0) load_group(t0);
    }
    float acc[TG];
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < P; ++i) ss += sumsq4(xv[j][i], XT());
      ss = wave_sum(ss);
      const float rj = 1.f / sqrtf(ss / (float)H + eps);
      acc[j] = 0.f;
#pragma unroll
      for (int i = 0; i < P; ++i) {
        xv[j][i] = scale4(xv[j][i], gv[i], rj, XT());
        acc[j] = RouterVec<XT>::dot(w[i], xv[j][i], acc[j]);
      }
      const int t = t0 + j;
      if (t < T && t % nwaves == wave) {
        uint4* yr = reinterpret_cast<uint4*>(xn + (size_t)t * H);
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int pc = lane + i * kWave;
          if (pc < np) yr[pc] = xv[j][i];
        }
      }
    }
    if constexpr (PF) {
      if (t0 + TG < T) load_group(t0 + TG);
    }
#pragma unroll
    for (int j = 0; j < TG; ++j) acc[j] = wave_sum(acc[j]);
    if (lane < TG && t0 + lane < T) {
      float v = acc[0];
#pragma unroll
      for (int j = 1; j < TG; ++j) v = lane == j ? acc[j] : v;
      if (r < E)
        logits[(size_t)(t0 + lane) * E + r] = v + bias;
      else
        sgate_pre[t0 + lane] = v;
    }
  }
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
