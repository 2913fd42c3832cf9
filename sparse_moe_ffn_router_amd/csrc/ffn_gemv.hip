// Expert kernels for few tokens per expert (decode-sized batches): each
// weight row is streamed from HBM once per expert and applied to every token
// routed to that expert.  Work unit: (active expert segment, tile of output
// rows).  A group of 8 lanes owns one output row pair and splits its input
// dimension in 16-byte pieces, so a wavefront keeps 8 rows streaming with
// 128-byte contiguous segments each.
//
// Sources: "qwen35moe - Forward-Pass Design", section "Shared-expert MoE
// FFN" (SwiGLU experts, shared expert); "Phase 19: MoE - gpt-oss-20b",
// section 2 Experts (interleaved gate_up with bias, clamps, (up+1) * gate *
// sigmoid(alpha gate), down + bias) and section 3 (MXFP4 decode).
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 8;                      // lanes per output row
constexpr int kRowsPerBlock = kThreads / kGroup;  // 32
constexpr int kTG = 16;                        // tokens per pass

enum { W_F32 = 0, W_BF16 = 1, W_MXFP4 = 2 };

// s-th non-empty segment among nseg (offsets has nseg + 1 entries), or -1.
__device__ int find_segment(const int32_t* __restrict__ offsets, int nseg, int s) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int base = 0; base < nseg; base += kWave) {
    const int e = base + lane;
    const bool ne = e < nseg && offsets[e + 1] > offsets[e];
    const uint64_t m = __ballot(ne);
    const int c = __popcll(m);
    if (s < c) {
      const uint64_t lower = lane ? (~0ull >> (64 - lane)) : 0ull;
      const bool hit = ne && __popcll(m & lower) == s;
      const uint64_t h = __ballot(hit);
      return base + __ffsll((unsigned long long)h) - 1;
    }
    s -= c;
  }
  return -1;
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

// Dot of one 16-byte weight piece with the matching activations of one
// token, accumulated into acc.  `xp` points at the piece's first element.
template <int WK> struct Piece;

template <> struct Piece<W_BF16> {
  static constexpr int kElems = 8;     // elements per lane piece
  typedef uint4 W;
  __device__ static W load(const void* row, int piece) { return reinterpret_cast<const uint4*>(row)[piece]; }
  __device__ static float dot(const W& w, const uint16_t* xp, float acc, float) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xp);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, xv.w), acc, false);
    return acc;
  }
};

template <> struct Piece<W_F32> {
  static constexpr int kElems = 4;
  typedef float4 W;
  __device__ static W load(const void* row, int piece) { return reinterpret_cast<const float4*>(row)[piece]; }
  __device__ static float dot(const W& w, const float* xp, float acc, float) {
    const float4 xv = *reinterpret_cast<const float4*>(xp);
    acc = fmaf(w.x, xv.x, acc);
    acc = fmaf(w.y, xv.y, acc);
    acc = fmaf(w.z, xv.z, acc);
    acc = fmaf(w.w, xv.w, acc);
    return acc;
  }
};

// MXFP4: a piece is one 32-element block (16 code bytes); the block's E8M0
// exponent is applied while converting the codes to bf16 (exact for the
// E2M1 values times 2^(e-127) that bf16 represents).
template <> struct Piece<W_MXFP4> {
  static constexpr int kElems = 32;
  typedef uint4 W;
  __device__ static W load(const void* row, int piece) { return reinterpret_cast<const uint4*>(row)[piece]; }
  __device__ static float dot(const W& w, const uint16_t* xp, float acc, float scale) {
    const uint4* xq = reinterpret_cast<const uint4*>(xp);
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 xv = xq[q];
      const uint32_t cw = words[q];
      const bf16x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scale, 0);
      const bf16x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scale, 1);
      const bf16x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scale, 2);
      const bf16x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scale, 3);
      acc = __builtin_amdgcn_fdot2_f32_bf16(w0, __builtin_bit_cast(bf16x2_t, xv.x), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(w1, __builtin_bit_cast(bf16x2_t, xv.y), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(w2, __builtin_bit_cast(bf16x2_t, xv.z), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(w3, __builtin_bit_cast(bf16x2_t, xv.w), acc, false);
    }
    return acc;
  }
};

template <typename XT> __device__ __forceinline__ float xscalar(const XT* p, int i);
template <> __device__ __forceinline__ float xscalar<float>(const float* p, int i) { return p[i]; }
template <> __device__ __forceinline__ float xscalar<uint16_t>(const uint16_t* p, int i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
template <typename XT> __device__ __forceinline__ void xstore(XT* p, size_t i, float v);
template <> __device__ __forceinline__ void xstore<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void xstore<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = (uint16_t)f32_to_bf16(v);
}

// Row byte pitch of a weight matrix with `cols` inputs.
template <int WK> __device__ __forceinline__ size_t row_bytes(int cols) {
  return WK == W_F32 ? (size_t)cols * 4 : WK == W_BF16 ? (size_t)cols * 2 : (size_t)cols / 2;
}

struct GateUpArgs {
  const void* x;
  const void* gate_w;      // SWIGLU [E][F][H]  | OAI gate_up [E][2F][H]
  const void* up_w;        // SWIGLU [E][F][H]  | unused
  const uint8_t* scales;   // MXFP4 gate_up scales [E][2F][H/32]
  const void* gate_up_b;   // OAI [E][2F]
  const void* sh_gate_w;   // [Fs][H]
  const void* sh_up_w;     // [Fs][H]
  const int32_t* offsets;
  const int32_t* sorted_assign;
  void* h;
  int32_t T, k, H, E, F, Fs, shared, oai;
  float alpha, limit;
};

// h[p][f] = act(gate row f . x_t, up row f . x_t) for every sorted position
// p of the block's expert segment.  Grid: (segment slot, row tile).
template <typename XT, int WK>
__global__ __launch_bounds__(kThreads) void k_gateup_gemv(GateUpArgs a) {
  using P = Piece<WK>;
  const int nseg = a.E + a.shared;
  const int e = find_segment(a.offsets, nseg, blockIdx.x);
  if (e < 0) return;
  const bool sh = e == a.E;
  const int Fe = sh ? a.Fs : a.F;
  const int grp = threadIdx.x / kGroup, lig = threadIdx.x & (kGroup - 1);
  const int f = blockIdx.y * kRowsPerBlock + grp;
  if (blockIdx.y * kRowsPerBlock >= Fe) return;
  const bool active = f < Fe;
  const int fr = active ? f : Fe - 1;   // inactive groups still join the shuffles
  // the two input rows of feature fr
  const uint8_t *rg, *ru;
  const uint8_t *sg = nullptr, *su = nullptr;
  const int rb = (int)row_bytes<WK>(a.H);
  if (sh) {
    rg = (const uint8_t*)a.sh_gate_w + (size_t)fr * row_bytes<(WK == W_MXFP4 ? W_BF16 : WK)>(a.H);
    ru = (const uint8_t*)a.sh_up_w + (size_t)fr * row_bytes<(WK == W_MXFP4 ? W_BF16 : WK)>(a.H);
  } else if (a.oai) {
    rg = (const uint8_t*)a.gate_w + ((size_t)e * 2 * a.F + 2 * fr) * rb;
    ru = rg + rb;
    if (WK == W_MXFP4) {
      sg = a.scales + ((size_t)e * 2 * a.F + 2 * fr) * (a.H / 32);
      su = sg + a.H / 32;
    }
  } else {
    rg = (const uint8_t*)a.gate_w + ((size_t)e * a.F + fr) * rb;
    ru = (const uint8_t*)a.up_w + ((size_t)e * a.F + fr) * rb;
  }
  const int p0 = a.offsets[e];
  const int n = a.offsets[e + 1] - p0;
  const int64_t nas = (int64_t)a.T * a.k;
  const XT* x = (const XT*)a.x;
  float bg = 0.f, bu = 0.f;
  if (a.oai && !sh && a.gate_up_b) {
    bg = xscalar<XT>((const XT*)a.gate_up_b, e * 2 * a.F + 2 * fr);
    bu = xscalar<XT>((const XT*)a.gate_up_b, e * 2 * a.F + 2 * fr + 1);
  }
  for (int tb = 0; tb < n; tb += kTG) {
    const int nt = min(kTG, n - tb);
    int tok[kTG];
#pragma unroll
    for (int i = 0; i < kTG; ++i) {
      const int sa = i < nt ? a.sorted_assign[p0 + tb + i] : 0;
      tok[i] = sa < nas ? sa / a.k : (int)(sa - nas);
    }
    float ag[kTG], au[kTG];
#pragma unroll
    for (int i = 0; i < kTG; ++i) ag[i] = au[i] = 0.f;
    if (sh && WK == W_MXFP4) {
      // shared expert rows are bf16 even when routed experts are MXFP4
      using PB = Piece<W_BF16>;
      const int npieces = a.H / PB::kElems;
      for (int pc = lig; pc < npieces; pc += kGroup) {
        const uint4 wg = PB::load(rg, pc), wu = PB::load(ru, pc);
#pragma unroll
        for (int i = 0; i < kTG; ++i)
          if (i < nt) {
            const uint16_t* xp = (const uint16_t*)x + (size_t)tok[i] * a.H + pc * PB::kElems;
            ag[i] = PB::dot(wg, xp, ag[i], 1.f);
            au[i] = PB::dot(wu, xp, au[i], 1.f);
          }
      }
    } else {
      const int npieces = a.H / P::kElems;
      int pc = lig;
      // four pieces per row in flight per lane
      for (; pc + 3 * kGroup < npieces; pc += 4 * kGroup) {
        typename P::W wg[4], wu[4];
        float sgv[4] = {1.f, 1.f, 1.f, 1.f}, suv[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          wg[u] = P::load(rg, pc + u * kGroup);
          wu[u] = P::load(ru, pc + u * kGroup);
          if (WK == W_MXFP4) {
            sgv[u] = e8m0_to_f32(sg[pc + u * kGroup]);
            suv[u] = e8m0_to_f32(su[pc + u * kGroup]);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < kTG; ++i)
            if (i < nt) {
              const XT* xp = x + (size_t)tok[i] * a.H + (size_t)(pc + u * kGroup) * P::kElems;
              ag[i] = P::dot(wg[u], xp, ag[i], sgv[u]);
              au[i] = P::dot(wu[u], xp, au[i], suv[u]);
            }
      }
      for (; pc < npieces; pc += kGroup) {
        const typename P::W wg = P::load(rg, pc), wu = P::load(ru, pc);
        const float sgv = WK == W_MXFP4 ? e8m0_to_f32(sg[pc]) : 1.f;
        const float suv = WK == W_MXFP4 ? e8m0_to_f32(su[pc]) : 1.f;
#pragma unroll
        for (int i = 0; i < kTG; ++i)
          if (i < nt) {
            const XT* xp = x + (size_t)tok[i] * a.H + (size_t)pc * P::kElems;
            ag[i] = P::dot(wg, xp, ag[i], sgv);
            au[i] = P::dot(wu, xp, au[i], suv);
          }
      }
    }
#pragma unroll
    for (int i = 0; i < kTG; ++i) {
#pragma unroll
      for (int o = 1; o < kGroup; o <<= 1) {
        ag[i] += __shfl_xor(ag[i], o, kWave);
        au[i] += __shfl_xor(au[i], o, kWave);
      }
    }
    if (active) {
#pragma unroll
      for (int i = 0; i < kTG; ++i) {
        if (i < nt && (i & (kGroup - 1)) == lig) {
          float hv;
          if (a.oai && !sh) {
            float g = fminf(ag[i] + bg, a.limit);
            float u = fminf(fmaxf(au[i] + bu, -a.limit), a.limit);
            hv = (u + 1.f) * (g / (1.f + expf(-a.alpha * g)));
          } else {
            hv = silu(ag[i]) * au[i];
          }
          const int p = p0 + tb + i;
          const size_t row = p < nas ? (size_t)p * a.F : (size_t)nas * a.F + (size_t)(p - nas) * a.Fs;
          xstore<XT>((XT*)a.h, row + f, hv);
        }
      }
    }
  }
}

struct DownArgs {
  const void* h;
  const void* down_w;       // [E][H][F]
  const uint8_t* scales;    // MXFP4 [E][H][F/32]
  const void* down_b;       // [E][H] or null
  const void* sh_down_w;    // [H][Fs]
  const int32_t* offsets;
  const int32_t* sorted_assign;
  float* y;                 // [T*k (+T)][H], row = assignment id
  int32_t T, k, H, E, F, Fs, shared;
};

// y[a][o] = down row o . h[p] (+ bias) for every sorted position p of the
// segment, written at the row of its assignment id a.
template <typename XT, int WK>
__global__ __launch_bounds__(kThreads) void k_down_gemv(DownArgs a) {
  const int nseg = a.E + a.shared;
  const int e = find_segment(a.offsets, nseg, blockIdx.x);
  if (e < 0) return;
  const bool sh = e == a.E;
  const int Fe = sh ? a.Fs : a.F;
  const int grp = threadIdx.x / kGroup, lig = threadIdx.x & (kGroup - 1);
  const int o = blockIdx.y * kRowsPerBlock + grp;
  if (blockIdx.y * kRowsPerBlock >= a.H) return;
  const bool active = o < a.H;
  const int orow = active ? o : a.H - 1;
  const int p0 = a.offsets[e];
  const int n = a.offsets[e + 1] - p0;
  const int64_t nas = (int64_t)a.T * a.k;
  const XT* hb = (const XT*)a.h;
  const XT* hbase = sh ? hb + (size_t)nas * a.F : hb;  // shared rows follow the routed rows
  const int prow0 = sh ? p0 - (int)nas : p0;
  float bias = 0.f;
  if (!sh && a.down_b) bias = xscalar<XT>((const XT*)a.down_b, e * a.H + orow);
  for (int tb = 0; tb < n; tb += kTG) {
    const int nt = min(kTG, n - tb);
    float acc[kTG];
#pragma unroll
    for (int i = 0; i < kTG; ++i) acc[i] = 0.f;
    if (sh || WK != W_MXFP4) {
      constexpr int WB = WK == W_F32 ? W_F32 : W_BF16;
      using P = Piece<WB>;
      const uint8_t* row = sh ? (const uint8_t*)a.sh_down_w + (size_t)orow * row_bytes<WB>(a.Fs)
                              : (const uint8_t*)a.down_w + ((size_t)e * a.H + orow) * row_bytes<WB>(a.F);
      const int npieces = Fe / P::kElems;
      for (int pc = lig; pc < npieces; pc += kGroup) {
        const typename P::W w = P::load(row, pc);
#pragma unroll
        for (int i = 0; i < kTG; ++i)
          if (i < nt) acc[i] = P::dot(w, hbase + (size_t)(prow0 + tb + i) * Fe + (size_t)pc * P::kElems, acc[i], 1.f);
      }
    } else {
      using P = Piece<W_MXFP4>;
      const uint8_t* row = (const uint8_t*)a.down_w + ((size_t)e * a.H + orow) * row_bytes<W_MXFP4>(a.F);
      const uint8_t* srow = a.scales + ((size_t)e * a.H + orow) * (a.F / 32);
      const int npieces = a.F / P::kElems;
      for (int pc = lig; pc < npieces; pc += kGroup) {
        const uint4 w = P::load(row, pc);
        const float sc = e8m0_to_f32(srow[pc]);
#pragma unroll
        for (int i = 0; i < kTG; ++i)
          if (i < nt)
            acc[i] = P::dot(w, (const uint16_t*)hbase + (size_t)(prow0 + tb + i) * Fe + (size_t)pc * P::kElems, acc[i], sc);
      }
    }
#pragma unroll
    for (int i = 0; i < kTG; ++i)
#pragma unroll
      for (int q = 1; q < kGroup; q <<= 1) acc[i] += __shfl_xor(acc[i], q, kWave);
    if (active) {
#pragma unroll
      for (int i = 0; i < kTG; ++i)
        if (i < nt && (i & (kGroup - 1)) == lig) {
          const int asg = a.sorted_assign[p0 + tb + i];
          a.y[(size_t)asg * a.H + o] = acc[i] + bias;
        }
    }
  }
}

// out[t][o] = sum_j w[t][j] y[t*k + j][o] (+ sgate[t] y[T*k + t][o]), the
// picks summed in pick order.
__global__ __launch_bounds__(256) void k_combine_gather(const float* __restrict__ y, const float* __restrict__ topk_w,
                                                        const float* __restrict__ sgate, int32_t T, int32_t k,
                                                        int32_t H, float* __restrict__ out) {
  const int t = blockIdx.y;
  const int o4 = blockIdx.x * 256 + threadIdx.x;  // float4 index
  if (o4 * 4 >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = topk_w[(size_t)t * k + j];
    const float4 v = reinterpret_cast<const float4*>(y + ((size_t)t * k + j) * H)[o4];
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  if (sgate) {
    const float g = sgate[t];
    const float4 v = reinterpret_cast<const float4*>(y + ((size_t)T * k + t) * H)[o4];
    acc.x = fmaf(g, v.x, acc.x);
    acc.y = fmaf(g, v.y, acc.y);
    acc.z = fmaf(g, v.z, acc.z);
    acc.w = fmaf(g, v.w, acc.w);
  }
  reinterpret_cast<float4*>(out + (size_t)t * H)[o4] = acc;
}

}  // namespace

// Defined in ffn_mfma.hip.
hipError_t launch_gateup_mfma(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                              const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s);
hipError_t launch_down_mfma(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                            const int32_t* sorted_assign, int32_t T, float* y, hipStream_t s);

bool mfma_shapes_ok(const moe_config* c);

static int max_segments(const moe_config* c, int32_t T) {
  const int64_t nk = (int64_t)T * c->top_k;
  return (int)(nk < c->n_expert ? nk : c->n_expert) + (c->shared_ff > 0 ? 1 : 0);
}

hipError_t launch_expert_ffn(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                             const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T > kGemvMaxT && mfma_shapes_ok(c))
    return launch_gateup_mfma(c, w, x, offsets, sorted_assign, T, h, s);
  GateUpArgs a;
  const bool oai = c->act == MOE_ACT_SWIGLU_OAI;
  a.x = x;
  a.gate_w = oai ? w->gate_up_w : w->gate_w;
  a.up_w = w->up_w;
  a.scales = w->gate_up_scales;
  a.gate_up_b = w->gate_up_b;
  a.sh_gate_w = w->sh_gate_w;
  a.sh_up_w = w->sh_up_w;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.h = h;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.shared = c->shared_ff > 0; a.oai = oai; a.alpha = c->act_alpha; a.limit = c->act_limit;
  const int fmax = c->expert_ff > c->shared_ff ? c->expert_ff : c->shared_ff;
  dim3 grid(max_segments(c, T), (fmax + kRowsPerBlock - 1) / kRowsPerBlock);
  if (c->x_dtype == MOE_DTYPE_F32)
    k_gateup_gemv<float, W_F32><<<grid, kThreads, 0, s>>>(a);
  else if (c->w_dtype == MOE_DTYPE_BF16)
    k_gateup_gemv<uint16_t, W_BF16><<<grid, kThreads, 0, s>>>(a);
  else
    k_gateup_gemv<uint16_t, W_MXFP4><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                       const int32_t* sorted_assign, int32_t T, float* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T > kGemvMaxT && mfma_shapes_ok(c))
    return launch_down_mfma(c, w, h, offsets, sorted_assign, T, y, s);
  DownArgs a;
  a.h = h;
  a.down_w = w->down_w;
  a.scales = w->down_scales;
  a.down_b = c->act == MOE_ACT_SWIGLU_OAI ? w->down_b : nullptr;
  a.sh_down_w = w->sh_down_w;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.y = y;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.shared = c->shared_ff > 0;
  dim3 grid(max_segments(c, T), (c->hidden + kRowsPerBlock - 1) / kRowsPerBlock);
  if (c->x_dtype == MOE_DTYPE_F32)
    k_down_gemv<float, W_F32><<<grid, kThreads, 0, s>>>(a);
  else if (c->w_dtype == MOE_DTYPE_BF16)
    k_down_gemv<uint16_t, W_BF16><<<grid, kThreads, 0, s>>>(a);
  else
    k_down_gemv<uint16_t, W_MXFP4><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine_gather(const moe_config* c, const float* y, const float* topk_w, const float* sgate,
                                 int32_t T, float* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((c->hidden / 4 + 255) / 256, T);
  k_combine_gather<<<grid, 256, 0, s>>>(y, topk_w, c->shared_ff > 0 ? sgate : nullptr, T, c->top_k, c->hidden,
                                         out);
  return hipGetLastError();
}

}  // namespace moe
