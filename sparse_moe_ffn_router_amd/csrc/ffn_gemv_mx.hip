// Few-token expert kernels for MXFP4 experts (bf16 activations).
//
// MXFP4 rows are a quarter of the bytes of the bf16 activation rows they
// multiply, so here a workgroup owns many rows of one expert segment (64 row
// pairs, or 128 output rows) and stages the segment's activation rows in LDS
// once, up to 8 at a time; a group of 4 lanes streams one row (pair) in
// 16-byte pieces (one 32-element block with its E8M0 exponent each), 4
// pieces in flight plus the next 4 prefetched (the first 4 issued before
// the activations are staged), decoding each block to bf16 in registers
// with the scaled fp4 conversion.  The shared expert, when a
// layer has one, keeps bf16 weights and runs through the same kernels.
//
// Sources: "Phase 19: MoE - gpt-oss-20b", section 2 Experts (interleaved
// gate_up with bias, clamps, (up+1) * gate * sigmoid(alpha gate), down +
// bias) and section 3 (MXFP4 decode); "qwen35moe - Forward-Pass Design",
// section "Shared-expert MoE FFN" (shared expert).
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
// Lanes per row pair: 4 (64 row pairs per workgroup) measured fastest
// against 2, 8 and 16 at the gpt-oss MXFP4 T = 16 shape -- fewer, larger
// workgroups spread the activation staging over more weight bytes.
constexpr int kGroup = 4;
constexpr int kPairsPerBlock = kThreads / kGroup;  // 64
// Sum over each group of kGroup lanes, result in every lane of the group.
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  return v;
}
constexpr int kStage = 8;                          // activation rows staged at once
constexpr int kU = 2;                              // pieces per row per pipeline step

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
      const bool hit = ne && __popcll(m & (lane ? (~0ull >> (64 - lane)) : 0ull)) == s;
      return base + __ffsll((unsigned long long)__ballot(hit)) - 1;
    }
    s -= c;
  }
  return -1;
}

// Segment of a workgroup: the grid is (row tile, segment slot), so each
// segment's row tiles are dispatched together; slot 0 is the shared expert
// (the segment with the most tokens, started first), slot s > 0 the
// (s-1)-th non-empty routed segment (the s-th without a shared expert).
__device__ __forceinline__ int slot_segment(const int32_t* __restrict__ offsets, int E, int shared) {
  const int slot = blockIdx.y;
  if (shared) return slot == 0 ? E : find_segment(offsets, E, slot - 1);
  return find_segment(offsets, E, slot);
}

template <int WK> struct Piece;

// bf16 weights: 8 elements per 16-byte piece, products summed in pairs.
template <> struct Piece<W_BF16> {
  static constexpr int kElems = 8;
  __device__ static float dot(uint4 w, const uint16_t* xp, float acc, float) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xp);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, xv.w), acc, false);
    return acc;
  }
};

// MXFP4: a piece is one 32-element block (16 code bytes); the block's E8M0
// exponent is applied while converting the codes to bf16 (exact for the
// E2M1 values times 2^(e-127) that bf16 represents).
template <> struct Piece<W_MXFP4> {
  static constexpr int kElems = 32;
  __device__ static float dot(uint4 w, const uint16_t* xp, float acc, float scale) {
    const uint4* xq = reinterpret_cast<const uint4*>(xp);
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 xv = xq[q];
      const uint32_t cw = words[q];
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scale, 0),
                                            __builtin_bit_cast(bf16x2_t, xv.x), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scale, 1),
                                            __builtin_bit_cast(bf16x2_t, xv.y), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scale, 2),
                                            __builtin_bit_cast(bf16x2_t, xv.z), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, scale, 3),
                                            __builtin_bit_cast(bf16x2_t, xv.w), acc, false);
    }
    return acc;
  }
};

template <typename XT> __device__ __forceinline__ float xscalar(const XT* p, size_t i);
template <> __device__ __forceinline__ float xscalar<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
template <typename XT> __device__ __forceinline__ void xstore(XT* p, size_t i, float v);
template <> __device__ __forceinline__ void xstore<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = (uint16_t)f32_to_bf16(v);
}

// The first kU pieces of a row pair (and their exponents), this lane's share.
struct First {
  uint4 w0[kU], w1[kU];
  uint8_t c0[kU], c1[kU];
};
template <int WK>
__device__ __forceinline__ void fetch_pieces(const uint4* r0, const uint4* r1, const uint8_t* s0, const uint8_t* s1,
                                             int npieces, int pc, uint4 (&a)[kU], uint4 (&b)[kU], uint8_t (&sa)[kU],
                                             uint8_t (&sb)[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int q = pc + u * kGroup;
    const bool ok = q < npieces;
    a[u] = ok ? r0[q] : make_uint4(0, 0, 0, 0);
    b[u] = ok ? r1[q] : make_uint4(0, 0, 0, 0);
    if (WK == W_MXFP4) {
      sa[u] = ok ? s0[q] : 0;
      sb[u] = ok ? s1[q] : 0;
    }
  }
}

// acc[r][i] += row r . xs[i] over K inputs, this lane's share (pieces
// lig, lig+8, ...).  Rows are streamed with the next kU pieces prefetched;
// the first kU pieces come in `first` (loaded before the activations were
// staged, so their latency overlaps the staging).
template <typename XT, int WK, int NT>
__device__ __forceinline__ void rows2_dot(const uint4* r0, const uint4* r1, const uint8_t* s0, const uint8_t* s1,
                                          const XT* xs, int K, int lig, const First& first,
                                          float (&acc)[2][kStage]) {
  using P = Piece<WK>;
  const int npieces = K / P::kElems;
  uint4 w0[kU], w1[kU];
  uint8_t c0[kU], c1[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    w0[u] = first.w0[u];
    w1[u] = first.w1[u];
    c0[u] = first.c0[u];
    c1[u] = first.c1[u];
  }
  for (int pc = lig; pc < npieces; pc += kU * kGroup) {
    uint4 n0[kU], n1[kU];
    uint8_t d0[kU], d1[kU];
    fetch_pieces<WK>(r0, r1, s0, s1, npieces, pc + kU * kGroup, n0, n1, d0, d1);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int q = pc + u * kGroup;
      if (q < npieces) {
        const float sc0 = WK == W_MXFP4 ? e8m0_to_f32(c0[u]) : 1.f;
        const float sc1 = WK == W_MXFP4 ? e8m0_to_f32(c1[u]) : 1.f;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const XT* xp = xs + (size_t)i * K + (size_t)q * P::kElems;
          acc[0][i] = P::dot(w0[u], xp, acc[0][i], sc0);
          acc[1][i] = P::dot(w1[u], xp, acc[1][i], sc1);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      w0[u] = n0[u];
      w1[u] = n1[u];
      c0[u] = d0[u];
      c1[u] = d1[u];
    }
  }
}

template <typename XT, int WK>
__device__ __forceinline__ void rows2_dot_n(int nt, const uint4* r0, const uint4* r1, const uint8_t* s0,
                                            const uint8_t* s1, const XT* xs, int K, int lig, const First& f,
                                            float (&acc)[2][kStage]) {
  switch (nt) {
    case 1: rows2_dot<XT, WK, 1>(r0, r1, s0, s1, xs, K, lig, f, acc); break;
    case 2: rows2_dot<XT, WK, 2>(r0, r1, s0, s1, xs, K, lig, f, acc); break;
    case 3: rows2_dot<XT, WK, 3>(r0, r1, s0, s1, xs, K, lig, f, acc); break;
    case 4: rows2_dot<XT, WK, 4>(r0, r1, s0, s1, xs, K, lig, f, acc); break;
    case 5: rows2_dot<XT, WK, 5>(r0, r1, s0, s1, xs, K, lig, f, acc); break;
    case 6: rows2_dot<XT, WK, 6>(r0, r1, s0, s1, xs, K, lig, f, acc); break;
    case 7: rows2_dot<XT, WK, 7>(r0, r1, s0, s1, xs, K, lig, f, acc); break;
    default: rows2_dot<XT, WK, 8>(r0, r1, s0, s1, xs, K, lig, f, acc); break;
  }
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
// p of the block's expert segment.  Grid: (tile of kPairsPerBlock features, segment slot).
template <typename XT, int WK>
__global__ __launch_bounds__(kThreads) void k_gateup_gemv_mx(GateUpArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  const int e = slot_segment(a.offsets, a.E, a.shared);
  if (e < 0) return;
  const bool sh = e == a.E;
  const int Fe = sh ? a.Fs : a.F;
  if (blockIdx.x * kPairsPerBlock >= Fe) return;
  const int grp = threadIdx.x / kGroup, lig = threadIdx.x & (kGroup - 1);
  const int f = blockIdx.x * kPairsPerBlock + grp;
  const bool active = f < Fe;
  const int fr = active ? f : Fe - 1;
  const uint8_t *rg, *ru, *sg = nullptr, *su = nullptr;
  constexpr int WS = WK == W_MXFP4 ? W_BF16 : WK;  // shared-expert element kind
  if (sh) {
    rg = (const uint8_t*)a.sh_gate_w + (size_t)fr * row_bytes<WS>(a.H);
    ru = (const uint8_t*)a.sh_up_w + (size_t)fr * row_bytes<WS>(a.H);
  } else if (a.oai) {
    const size_t rb = row_bytes<WK>(a.H);
    rg = (const uint8_t*)a.gate_w + ((size_t)e * 2 * a.F + 2 * fr) * rb;
    ru = rg + rb;
    if (WK == W_MXFP4) {
      sg = a.scales + ((size_t)e * 2 * a.F + 2 * fr) * (a.H / 32);
      su = sg + a.H / 32;
    }
  } else {
    const size_t rb = row_bytes<WK>(a.H);
    rg = (const uint8_t*)a.gate_w + ((size_t)e * a.F + fr) * rb;
    ru = (const uint8_t*)a.up_w + ((size_t)e * a.F + fr) * rb;
  }
  const int p0 = a.offsets[e];
  const int n = a.offsets[e + 1] - p0;
  const int64_t nas = (int64_t)a.T * a.k;
  float bg = 0.f, bu = 0.f;
  if (a.oai && !sh && a.gate_up_b) {
    bg = xscalar<XT>((const XT*)a.gate_up_b, (size_t)e * 2 * a.F + 2 * fr);
    bu = xscalar<XT>((const XT*)a.gate_up_b, (size_t)e * 2 * a.F + 2 * fr + 1);
  }
  const int xpieces = a.H * (int)sizeof(XT) / 16;  // 16-byte pieces per x row
  // the first weight pieces go out before the activations are staged
  const bool plain = sh || WK != W_MXFP4;  // bf16 (or fp32) rows
  const int npc = plain ? a.H / Piece<WS>::kElems : a.H / Piece<WK>::kElems;
  First first;
  if (plain)
    fetch_pieces<WS>((const uint4*)rg, (const uint4*)ru, sg, su, npc, lig, first.w0, first.w1, first.c0, first.c1);
  else
    fetch_pieces<WK>((const uint4*)rg, (const uint4*)ru, sg, su, npc, lig, first.w0, first.w1, first.c0, first.c1);
  for (int tb = 0; tb < n; tb += kStage) {
    const int nt = min(kStage, n - tb);
    if (tb) {
      __syncthreads();
      if (plain)
        fetch_pieces<WS>((const uint4*)rg, (const uint4*)ru, sg, su, npc, lig, first.w0, first.w1, first.c0, first.c1);
      else
        fetch_pieces<WK>((const uint4*)rg, (const uint4*)ru, sg, su, npc, lig, first.w0, first.w1, first.c0, first.c1);
    }
    for (int i = threadIdx.x; i < nt * xpieces; i += kThreads) {
      const int j = i / xpieces, q = i - j * xpieces;
      const int sa = a.sorted_assign[p0 + tb + j];
      const int t = sa < nas ? sa / a.k : (int)(sa - nas);
      reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>((const XT*)a.x + (size_t)t * a.H)[q];
    }
    __syncthreads();
    float acc[2][kStage];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < kStage; ++i) acc[r][i] = 0.f;
    if (plain)
      rows2_dot_n<XT, WS>(nt, (const uint4*)rg, (const uint4*)ru, sg, su, xs, a.H, lig, first, acc);
    else
      rows2_dot_n<XT, WK>(nt, (const uint4*)rg, (const uint4*)ru, sg, su, xs, a.H, lig, first, acc);
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      acc[0][i] = group_sum(acc[0][i]);
      acc[1][i] = group_sum(acc[1][i]);
    }
    if (active) {
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        if (i < nt && i % kGroup == lig) {
          float hv;
          if (a.oai && !sh) {
            const float g = fminf(acc[0][i] + bg, a.limit);
            const float u = fminf(fmaxf(acc[1][i] + bu, -a.limit), a.limit);
            hv = (u + 1.f) * (g / (1.f + expf(-a.alpha * g)));
          } else {
            const float g = acc[0][i];
            hv = g / (1.f + expf(-g)) * acc[1][i];
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
// segment, written at the row of its assignment id a.  Grid: (tile of
// 2 * kPairsPerBlock output rows, segment slot); a group of kGroup lanes owns rows
// o and o + kPairsPerBlock.
template <typename XT, int WK>
__global__ __launch_bounds__(kThreads) void k_down_gemv_mx(DownArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  XT* hs = reinterpret_cast<XT*>(smem);
  const int e = slot_segment(a.offsets, a.E, a.shared);
  if (e < 0) return;
  const bool sh = e == a.E;
  const int Fe = sh ? a.Fs : a.F;
  const int obase = blockIdx.x * 2 * kPairsPerBlock;
  if (obase >= a.H) return;
  const int grp = threadIdx.x / kGroup, lig = threadIdx.x & (kGroup - 1);
  const int o0 = obase + grp, o1 = obase + kPairsPerBlock + grp;
  const int q0 = min(o0, a.H - 1), q1 = min(o1, a.H - 1);
  constexpr int WS = WK == W_MXFP4 ? W_BF16 : WK;
  const uint8_t *r0, *r1, *s0 = nullptr, *s1 = nullptr;
  if (sh) {
    r0 = (const uint8_t*)a.sh_down_w + (size_t)q0 * row_bytes<WS>(a.Fs);
    r1 = (const uint8_t*)a.sh_down_w + (size_t)q1 * row_bytes<WS>(a.Fs);
  } else {
    const size_t rb = row_bytes<WK>(a.F);
    r0 = (const uint8_t*)a.down_w + ((size_t)e * a.H + q0) * rb;
    r1 = (const uint8_t*)a.down_w + ((size_t)e * a.H + q1) * rb;
    if (WK == W_MXFP4) {
      s0 = a.scales + ((size_t)e * a.H + q0) * (a.F / 32);
      s1 = a.scales + ((size_t)e * a.H + q1) * (a.F / 32);
    }
  }
  const int p0 = a.offsets[e];
  const int n = a.offsets[e + 1] - p0;
  const int64_t nas = (int64_t)a.T * a.k;
  const XT* hb = (const XT*)a.h;
  const XT* hbase = sh ? hb + (size_t)nas * a.F + (size_t)(p0 - nas) * a.Fs : hb + (size_t)p0 * a.F;
  float b0 = 0.f, b1 = 0.f;
  if (!sh && a.down_b) {
    b0 = xscalar<XT>((const XT*)a.down_b, (size_t)e * a.H + q0);
    b1 = xscalar<XT>((const XT*)a.down_b, (size_t)e * a.H + q1);
  }
  const int hpieces = Fe * (int)sizeof(XT) / 16;
  // the first weight pieces go out before the activations are staged
  const bool plain = sh || WK != W_MXFP4;
  const int npc = plain ? Fe / Piece<WS>::kElems : Fe / Piece<WK>::kElems;
  First first;
  if (plain)
    fetch_pieces<WS>((const uint4*)r0, (const uint4*)r1, s0, s1, npc, lig, first.w0, first.w1, first.c0, first.c1);
  else
    fetch_pieces<WK>((const uint4*)r0, (const uint4*)r1, s0, s1, npc, lig, first.w0, first.w1, first.c0, first.c1);
  for (int tb = 0; tb < n; tb += kStage) {
    const int nt = min(kStage, n - tb);
    if (tb) {
      __syncthreads();
      if (plain)
        fetch_pieces<WS>((const uint4*)r0, (const uint4*)r1, s0, s1, npc, lig, first.w0, first.w1, first.c0, first.c1);
      else
        fetch_pieces<WK>((const uint4*)r0, (const uint4*)r1, s0, s1, npc, lig, first.w0, first.w1, first.c0, first.c1);
    }
    for (int i = threadIdx.x; i < nt * hpieces; i += kThreads)
      reinterpret_cast<uint4*>(hs)[i] = reinterpret_cast<const uint4*>(hbase + (size_t)tb * Fe)[i];
    __syncthreads();
    float acc[2][kStage];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < kStage; ++i) acc[r][i] = 0.f;
    if (sh || WK != W_MXFP4)
      rows2_dot_n<XT, WS>(nt, (const uint4*)r0, (const uint4*)r1, s0, s1, hs, Fe, lig, first, acc);
    else
      rows2_dot_n<XT, WK>(nt, (const uint4*)r0, (const uint4*)r1, s0, s1, hs, Fe, lig, first, acc);
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      acc[0][i] = group_sum(acc[0][i]);
      acc[1][i] = group_sum(acc[1][i]);
    }
#pragma unroll
    for (int i = 0; i < kStage; ++i)
      if (i < nt && i % kGroup == lig) {
        const int asg = a.sorted_assign[p0 + tb + i];
        if (o0 < a.H) a.y[(size_t)asg * a.H + o0] = acc[0][i] + b0;
        if (o1 < a.H) a.y[(size_t)asg * a.H + o1] = acc[1][i] + b1;
      }
  }
}

}  // namespace

static int max_segments_mx(const moe_config* c, int32_t T) {
  const int64_t nk = (int64_t)T * c->top_k;
  return (int)(nk < c->n_expert ? nk : c->n_expert) + (c->shared_ff > 0 ? 1 : 0);
}

static size_t stage_rows_mx(int32_t T) { return (size_t)(T < kStage ? T : kStage); }

hipError_t launch_expert_ffn_mx(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                                const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s) {
  GateUpArgs a;
  a.x = x;
  a.gate_w = w->gate_up_w;
  a.up_w = nullptr;
  a.scales = w->gate_up_scales;
  a.gate_up_b = w->gate_up_b;
  a.sh_gate_w = w->sh_gate_w;
  a.sh_up_w = w->sh_up_w;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.h = h;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.shared = c->shared_ff > 0; a.oai = 1; a.alpha = c->act_alpha; a.limit = c->act_limit;
  const int fmax = c->expert_ff > c->shared_ff ? c->expert_ff : c->shared_ff;
  dim3 grid((fmax + kPairsPerBlock - 1) / kPairsPerBlock, max_segments_mx(c, T));
  const size_t lds = stage_rows_mx(T) * c->hidden * 2;
  k_gateup_gemv_mx<uint16_t, W_MXFP4><<<grid, kThreads, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_mx(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                          const int32_t* sorted_assign, int32_t T, float* y, hipStream_t s) {
  DownArgs a;
  a.h = h;
  a.down_w = w->down_w;
  a.scales = w->down_scales;
  a.down_b = w->down_b;
  a.sh_down_w = w->sh_down_w;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.y = y;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.shared = c->shared_ff > 0;
  dim3 grid((c->hidden + 2 * kPairsPerBlock - 1) / (2 * kPairsPerBlock), max_segments_mx(c, T));
  const int fmax = c->expert_ff > c->shared_ff ? c->expert_ff : c->shared_ff;
  const size_t lds = stage_rows_mx(T) * fmax * 2;
  k_down_gemv_mx<uint16_t, W_MXFP4><<<grid, kThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
