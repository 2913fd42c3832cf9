// Few-token expert kernels for MXFP4 experts (bf16 activations).
//
// Routed segments run through the burst kernels (k_gateup_mx_burst,
// k_down_mx_burst): a wavefront owns 4 row pairs of one segment, 16 lanes
// per pair, and issues the loads of all its pieces (16 bytes = one
// 32-element block, with its E8M0 exponent) at once, right after those of
// the first activation rows the workgroup stages in LDS; every piece is
// decoded to bf16 once, with the scaled fp4 conversion, and multiplied with
// each staged token.  The shared expert, when a layer has one, keeps bf16
// weights and runs through the streaming kernels (k_gateup_gemv_mx,
// k_down_gemv_mx): 64 row pairs per workgroup, a group of 4 lanes streams
// one row pair with two 16-byte pieces per row in flight.
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
            hv = oai_act(acc[0][i] + bg, acc[1][i] + bu, a.alpha, a.limit);
          } else {
            hv = swiglu_act(acc[0][i], acc[1][i]);
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

// ---------------------------------------------------------------------------
// Routed MXFP4 segments: burst kernels.  A wavefront owns 4 row pairs of one
// segment, 16 lanes per pair; a lane issues the loads of all its pieces of
// both rows at once (pieces l, l + 16, ... of a row; 6 per row at K = 2880,
// i.e. 11.5 KiB in flight per wavefront), like the bf16 decode kernels.
// The first kBStage activation rows of the segment (and the rows' biases)
// are loaded just before the weights, so they arrive while the weights are
// in flight, and go to LDS once the weight loads are out; later groups of
// kBStage rows are staged the plain way (the weights stay in registers for
// every group).  Loaded after the weights, as before, the rows' loads and
// an early use of the biases waited for every weight load first
// (gpt-oss MXFP4 T = 16: gate/up 68.3 -> 57.6 us, down 36.8 -> 32.4 us).  Each
// piece is decoded once and multiplied with every staged token; the (row,
// token) sums are reduced over the pair's 16 lanes with DPP.  Against the
// streaming kernels above this keeps about three times the weight bytes in
// flight per CU.
constexpr int kBWaves = 4;
constexpr int kBThreads = kBWaves * kWave;
constexpr int kBLanes = 16;                   // lanes per row pair
constexpr int kBPairs = kBThreads / kBLanes;  // row pairs per workgroup
constexpr int kBStage = 2;                    // tokens staged per pass (126 VGPRs, 4 waves per SIMD; 4 tokens: 164, 3 waves, 6% slower)

// The s-th non-empty routed segment (s = blockIdx.y): expert (-1: none),
// first sorted position and rows.  With segtab (the permutation's slot
// table, the routed segments after the shared expert's slot) one scalar
// load; without, a search of the offsets and the segment's bounds.
struct BSeg {
  int e, p0, n;
};
__device__ __forceinline__ BSeg routed_segment(const int32_t* __restrict__ offsets, int E, int shared,
                                               const int32_t* __restrict__ segtab) {
  if (segtab) {
    const int4 v = reinterpret_cast<const int4*>(segtab)[shared + (int)blockIdx.y];
    return BSeg{__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                __builtin_amdgcn_readfirstlane(v.z)};
  }
  const int e = __builtin_amdgcn_readfirstlane(find_segment(offsets, E, blockIdx.y));
  if (e < 0) return BSeg{-1, 0, 0};
  const int p0 = offsets[e];
  return BSeg{e, p0, offsets[e + 1] - p0};
}

// Both rows' pieces of this lane (codes and E8M0 exponents).  The buffer
// descriptors are wave-uniform (they span the wavefront's rows; a
// per-lane descriptor would make every load a loop over the distinct
// descriptors); row r of this lane's pair starts at byte co[r] of rc and at
// byte so[r] of rs (kOutOfRange: no such row).  Pieces past P read zeros.
template <int NPL>
__device__ __forceinline__ void burst_load(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, const uint32_t (&co)[2],
                                           const uint32_t (&so)[2], int P, int l, uint4 (&w)[2][NPL],
                                           uint32_t (&sc)[2][NPL]) {
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int p = l + kBLanes * j;
      const bool ok = p < P && co[r] != kOutOfRange;
      w[r][j] = buf_load16_once(rc, ok ? co[r] + (uint32_t)p * 16 : kOutOfRange, 0);
      sc[r][j] = buf_load_u8(rs, ok ? so[r] + (uint32_t)p : kOutOfRange, 0);
    }
}

// acc[r][i] += row r . xs[i], this lane's pieces, NT staged tokens of K inputs.
template <int NPL, int NT>
__device__ __forceinline__ void burst_dot(const uint4 (&w)[2][NPL], const uint32_t (&sc)[2][NPL],
                                          const uint16_t* xs, int K, int P, int l, float (&acc)[2][kBStage]) {
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int p = l + kBLanes * j;
    if (p < P) {
      const float s0 = e8m0_to_f32(sc[0][j]), s1 = e8m0_to_f32(sc[1][j]);
      const uint32_t c0[4] = {w[0][j].x, w[0][j].y, w[0][j].z, w[0][j].w};
      const uint32_t c1[4] = {w[1][j].x, w[1][j].y, w[1][j].z, w[1][j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2_t g0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c0[q], s0, 0);
        const bf16x2_t g1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c0[q], s0, 1);
        const bf16x2_t g2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c0[q], s0, 2);
        const bf16x2_t g3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c0[q], s0, 3);
        const bf16x2_t u0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c1[q], s1, 0);
        const bf16x2_t u1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c1[q], s1, 1);
        const bf16x2_t u2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c1[q], s1, 2);
        const bf16x2_t u3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c1[q], s1, 3);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const uint4 xv = reinterpret_cast<const uint4*>(xs + (size_t)i * K)[q * P + p];
          const bf16x2_t x0 = __builtin_bit_cast(bf16x2_t, xv.x), x1 = __builtin_bit_cast(bf16x2_t, xv.y);
          const bf16x2_t x2 = __builtin_bit_cast(bf16x2_t, xv.z), x3 = __builtin_bit_cast(bf16x2_t, xv.w);
          float a0 = acc[0][i], a1 = acc[1][i];
          a0 = __builtin_amdgcn_fdot2_f32_bf16(g0, x0, a0, false);
          a1 = __builtin_amdgcn_fdot2_f32_bf16(u0, x0, a1, false);
          a0 = __builtin_amdgcn_fdot2_f32_bf16(g1, x1, a0, false);
          a1 = __builtin_amdgcn_fdot2_f32_bf16(u1, x1, a1, false);
          a0 = __builtin_amdgcn_fdot2_f32_bf16(g2, x2, a0, false);
          a1 = __builtin_amdgcn_fdot2_f32_bf16(u2, x2, a1, false);
          a0 = __builtin_amdgcn_fdot2_f32_bf16(g3, x3, a0, false);
          a1 = __builtin_amdgcn_fdot2_f32_bf16(u3, x3, a1, false);
          acc[0][i] = a0;
          acc[1][i] = a1;
        }
      }
    }
  }
}

template <int NPL>
__device__ __forceinline__ void burst_dot_n(int nt, const uint4 (&w)[2][NPL], const uint32_t (&sc)[2][NPL],
                                            const uint16_t* xs, int K, int P, int l, float (&acc)[2][kBStage]) {
  static_assert(kBStage == 2, "one case per staged token count");
  switch (nt) {
    case 1: burst_dot<NPL, 1>(w, sc, xs, K, P, l, acc); break;
    default: burst_dot<NPL, 2>(w, sc, xs, K, P, l, acc); break;
  }
}

// Stage activation rows [tb, tb + nt) of the segment (row i of src_row(i))
// into xs, 16 bytes per thread per step.  A row's 16-byte chunk g (quarter
// g % 4 of 32-element piece g / 4) goes to chunk (g % 4) * P + g / 4: the 16
// lanes of a row pair, which read one quarter of 16 consecutive pieces at a
// time, then read 256 contiguous bytes, one 16-byte group of banks each (at
// the piece-major layout their 64-byte stride was a 4-way bank conflict).
template <typename RowOf>
__device__ __forceinline__ void stage_rows(uint16_t* xs, int nt, int K, RowOf src_row) {
  const int chunks = K / 8;  // 16-byte chunks per row
  const int P = K / 32;
  for (int j = 0; j < nt; ++j) {
    const uint4* src = reinterpret_cast<const uint4*>(src_row(j));
    uint4* dst = reinterpret_cast<uint4*>(xs + (size_t)j * K);
    for (int g = threadIdx.x; g < chunks; g += kBThreads) dst[(g & 3) * P + (g >> 2)] = src[g];
  }
}

// The first staged group's rows loaded into registers (before the weights,
// so their data arrives while the weight loads are still in flight), then
// written to LDS in stage_rows' layout.  Rows of at most 2 * kBThreads
// 16-byte chunks (K <= 4096).
template <typename RowOf>
__device__ __forceinline__ void pre_stage(uint4 (&xr)[kBStage][2], int nt, int K, RowOf src_row) {
  const int chunks = K / 8;
#pragma unroll
  for (int j = 0; j < kBStage; ++j) {
    const uint4* src = reinterpret_cast<const uint4*>(src_row(j < nt ? j : 0));
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int g = (int)threadIdx.x + c * kBThreads;
      xr[j][c] = j < nt && g < chunks ? src[g] : make_uint4(0, 0, 0, 0);
    }
  }
}
__device__ __forceinline__ void put_stage(uint16_t* xs, const uint4 (&xr)[kBStage][2], int nt, int K) {
  const int chunks = K / 8;
  const int P = K / 32;
#pragma unroll
  for (int j = 0; j < kBStage; ++j)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int g = (int)threadIdx.x + c * kBThreads;
      if (j < nt && g < chunks) reinterpret_cast<uint4*>(xs + (size_t)j * K)[(g & 3) * P + (g >> 2)] = xr[j][c];
    }
}

// Gate/up of the routed segments (interleaved gate_up rows 2f, 2f + 1, bias
// and clamped activation).  Grid: (groups of kBPairs features, routed
// segment slot).
template <int NPL>
__global__ __launch_bounds__(kBThreads) void k_gateup_mx_burst(GateUpArgs a, const int32_t* __restrict__ segtab) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  const BSeg sg = routed_segment(a.offsets, a.E, a.shared, segtab);
  const int e = sg.e;
  if (e < 0) return;
  const int l = threadIdx.x & (kBLanes - 1);
  const int f = blockIdx.x * kBPairs + threadIdx.x / kBLanes;
  if (blockIdx.x * kBPairs >= a.F) return;
  const bool active = f < a.F;
  const int fr = active ? f : a.F - 1;
  const int P = a.H / 32;
  const uint32_t rb = (uint32_t)a.H / 2;
  // the wavefront's rows: fused rows 2 fw .. 2 F - 1 of the expert
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int fw = min((int)(blockIdx.x * kBPairs) + wv * (kWave / kBLanes), a.F - 1);
  const size_t wrow = (size_t)e * 2 * a.F + 2 * (size_t)fw;
  const uint32_t nrows = (uint32_t)(2 * (a.F - fw));
  const __amdgpu_buffer_rsrc_t rc = make_rsrc((const uint8_t*)a.gate_w + wrow * rb, nrows * rb);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + wrow * P, nrows * (uint32_t)P);
  const uint32_t lr = (uint32_t)(2 * (fr - fw));  // this lane's first row in the wavefront's span
  const uint32_t co[2] = {lr * rb, (lr + 1) * rb}, so[2] = {lr * (uint32_t)P, (lr + 1) * (uint32_t)P};
  const int p0 = sg.p0, n = sg.n;
  uint4 xr[kBStage][2];
  pre_stage(xr, min(kBStage, n), a.H, [&](int j) {
    const int sa = a.sorted_assign[p0 + j];
    return (const uint16_t*)a.x + (size_t)(sa / a.k) * a.H;
  });
  // the (gate, up) bias pair as one word, loaded ahead of the weights and
  // unpacked after them: a use right after the weight loads would wait for
  // all of them
  const size_t row0 = (size_t)e * 2 * a.F + 2 * (size_t)fr;
  const uint32_t braw = a.gate_up_b ? *reinterpret_cast<const uint32_t*>((const uint16_t*)a.gate_up_b + row0) : 0u;
  uint4 w[2][NPL];
  uint32_t sc[2][NPL];
  burst_load<NPL>(rc, rs, co, so, P, l, w, sc);
  __builtin_amdgcn_sched_barrier(0);
  const float bg = __uint_as_float(braw << 16), bu = __uint_as_float(braw & 0xFFFF0000u);
  put_stage(xs, xr, min(kBStage, n), a.H);
  for (int tb = 0; tb < n; tb += kBStage) {
    const int nt = min(kBStage, n - tb);
    if (tb) {
      __syncthreads();
      stage_rows(xs, nt, a.H, [&](int j) {
        const int sa = a.sorted_assign[p0 + tb + j];
        return (const uint16_t*)a.x + (size_t)(sa / a.k) * a.H;
      });
    }
    __syncthreads();
    float acc[2][kBStage];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < kBStage; ++i) acc[r][i] = 0.f;
    burst_dot_n<NPL>(nt, w, sc, xs, a.H, P, l, acc);
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int i = 0; i < kBStage; ++i) {
      if (i < nt) {
        const float gi = row16_sum(acc[0][i]), ui = row16_sum(acc[1][i]);
        gs = l == i ? gi : gs;
        us = l == i ? ui : us;
      }
    }
    if (active && l < nt) {
      const float hv = oai_act(gs + bg, us + bu, a.alpha, a.limit);
      xstore<uint16_t>((uint16_t*)a.h, (size_t)(p0 + tb + l) * a.F + f, hv);
    }
  }
}

// Down of the routed segments: a pair is output rows 2o', 2o' + 1.  Grid:
// (groups of kBPairs row pairs, routed segment slot).
template <int NPL>
__global__ __launch_bounds__(kBThreads) void k_down_mx_burst(DownArgs a, const int32_t* __restrict__ segtab) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
  const BSeg sg = routed_segment(a.offsets, a.E, a.shared, segtab);
  const int e = sg.e;
  if (e < 0) return;
  const int l = threadIdx.x & (kBLanes - 1);
  const int npairs = (a.H + 1) / 2;
  const int pr = blockIdx.x * kBPairs + threadIdx.x / kBLanes;
  if (blockIdx.x * kBPairs >= npairs) return;
  const int o0 = 2 * min(pr, npairs - 1);
  const bool two = o0 + 1 < a.H;  // H odd: the last pair has one row
  const int P = a.F / 32;
  const uint32_t rb = (uint32_t)a.F / 2;
  // the wavefront's rows: output rows ow .. H - 1 of the expert
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int ow = 2 * min((int)(blockIdx.x * kBPairs) + wv * (kWave / kBLanes), npairs - 1);
  const size_t wrow = (size_t)e * a.H + ow;
  const uint32_t nrows = (uint32_t)(a.H - ow);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc((const uint8_t*)a.down_w + wrow * rb, nrows * rb);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + wrow * P, nrows * (uint32_t)P);
  const uint32_t lr = (uint32_t)(o0 - ow);
  const uint32_t co[2] = {lr * rb, two ? (lr + 1) * rb : kOutOfRange};
  const uint32_t so[2] = {lr * (uint32_t)P, two ? (lr + 1) * (uint32_t)P : kOutOfRange};
  const int p0 = sg.p0, n = sg.n;
  const uint16_t* hseg = (const uint16_t*)a.h + (size_t)p0 * a.F;
  uint4 xr[kBStage][2];
  pre_stage(xr, min(kBStage, n), a.F, [&](int j) { return hseg + (size_t)j * a.F; });
  // the pair's two biases as one word (the second half unused when H is
  // odd and the pair has one row), loaded ahead of the weights and unpacked
  // after them
  const size_t row0 = (size_t)e * a.H + o0;
  const uint32_t braw = a.down_b ? (two ? *reinterpret_cast<const uint32_t*>((const uint16_t*)a.down_b + row0)
                                        : (uint32_t)((const uint16_t*)a.down_b)[row0])
                                 : 0u;
  uint4 w[2][NPL];
  uint32_t sc[2][NPL];
  burst_load<NPL>(rc, rs, co, so, P, l, w, sc);
  __builtin_amdgcn_sched_barrier(0);
  const float b0 = __uint_as_float(braw << 16), b1 = __uint_as_float(braw & 0xFFFF0000u);
  put_stage(hs, xr, min(kBStage, n), a.F);
  for (int tb = 0; tb < n; tb += kBStage) {
    const int nt = min(kBStage, n - tb);
    if (tb) {
      __syncthreads();
      stage_rows(hs, nt, a.F, [&](int j) { return hseg + (size_t)(tb + j) * a.F; });
    }
    __syncthreads();
    float acc[2][kBStage];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < kBStage; ++i) acc[r][i] = 0.f;
    burst_dot_n<NPL>(nt, w, sc, hs, a.F, P, l, acc);
    float y0 = 0.f, y1 = 0.f;
#pragma unroll
    for (int i = 0; i < kBStage; ++i) {
      if (i < nt) {
        const float v0 = row16_sum(acc[0][i]), v1 = row16_sum(acc[1][i]);
        y0 = l == i ? v0 : y0;
        y1 = l == i ? v1 : y1;
      }
    }
    if (pr < npairs && l < nt) {
      const int asg = a.sorted_assign[p0 + tb + l];
      a.y[(size_t)asg * a.H + o0] = y0 + b0;
      if (two) a.y[(size_t)asg * a.H + o0 + 1] = y1 + b1;
    }
  }
}

}  // namespace

static int max_routed_mx(const moe_config* c, int32_t T) {
  const int64_t nk = (int64_t)T * c->top_k;
  return (int)(nk < c->n_expert ? nk : c->n_expert);
}

static size_t stage_rows_mx(int32_t T) { return (size_t)(T < kStage ? T : kStage); }
static size_t stage_rows_burst(int32_t T) { return (size_t)(T < kBStage ? T : kBStage); }

// Pieces per lane per row for rows of K inputs (K / 32 pieces over 16 lanes;
// K <= 4096 gives at most 8).
static int burst_npl(int K) {
  const int np = (K / 32 + kBLanes - 1) / kBLanes;
  return np <= 1 ? 1 : np <= 2 ? 2 : np <= 4 ? 4 : np <= 6 ? 6 : 8;
}

#define MOE_NPL_SWITCH(KERNEL, npl, grid, lds, s, ...)                    \
  switch (npl) {                                                          \
    case 1: KERNEL<1><<<grid, kBThreads, lds, s>>>(__VA_ARGS__); break;          \
    case 2: KERNEL<2><<<grid, kBThreads, lds, s>>>(__VA_ARGS__); break;          \
    case 4: KERNEL<4><<<grid, kBThreads, lds, s>>>(__VA_ARGS__); break;          \
    case 6: KERNEL<6><<<grid, kBThreads, lds, s>>>(__VA_ARGS__); break;          \
    default: KERNEL<8><<<grid, kBThreads, lds, s>>>(__VA_ARGS__); break;         \
  }

// Routed segments through the burst kernel; the shared expert (bf16 rows),
// if any, through the streaming kernel with a single segment slot (slot 0
// is the shared expert there).
hipError_t launch_expert_ffn_mx(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                                const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s,
                                const int32_t* segtab) {
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
  {
    const dim3 grid((c->expert_ff + kBPairs - 1) / kBPairs, max_routed_mx(c, T));
    const size_t lds = stage_rows_burst(T) * c->hidden * 2;
    MOE_NPL_SWITCH(k_gateup_mx_burst, burst_npl(c->hidden), grid, lds, s, a, segtab)
  }
  if (a.shared) {
    const dim3 grid((c->shared_ff + kPairsPerBlock - 1) / kPairsPerBlock, 1);
    const size_t lds = stage_rows_mx(T) * c->hidden * 2;
    k_gateup_gemv_mx<uint16_t, W_MXFP4><<<grid, kThreads, lds, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_down_mx(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                          const int32_t* sorted_assign, int32_t T, float* y, hipStream_t s, const int32_t* segtab) {
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
  {
    const dim3 grid(((c->hidden + 1) / 2 + kBPairs - 1) / kBPairs, max_routed_mx(c, T));
    const size_t lds = stage_rows_burst(T) * c->expert_ff * 2;
    MOE_NPL_SWITCH(k_down_mx_burst, burst_npl(c->expert_ff), grid, lds, s, a, segtab)
  }
  if (a.shared) {
    const dim3 grid((c->hidden + 2 * kPairsPerBlock - 1) / (2 * kPairsPerBlock), 1);
    const size_t lds = stage_rows_mx(T) * c->shared_ff * 2;
    k_down_gemv_mx<uint16_t, W_MXFP4><<<grid, kThreads, lds, s>>>(a);
  }
  return hipGetLastError();
}
#undef MOE_NPL_SWITCH

}  // namespace moe
