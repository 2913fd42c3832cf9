// Expert kernels for few tokens per expert (decode-sized batches): each
// weight row is streamed from HBM once and applied to every token routed to
// its expert.
//
// Work unit: one wavefront owns RPW consecutive weight rows of one non-empty
// expert segment (gate/up: RPW feature row pairs; down: RPW output rows).
// It issues every load of its rows at once -- a 64-lane load instruction
// reads 1 KiB of one row, 16 bytes per lane -- then loads the segment's
// activation rows (L2-resident) while the weights are in flight, and reduces
// each (row, token) dot product across the wavefront.  Many short
// wavefronts, each with one burst of loads, keep HBM busier than long
// software-pipelined ones for this access pattern; there is no LDS and no
// barrier.  Activation rows are processed one token at a time, the next
// one prefetched while the current one is reduced.  Weight loads carry the
// streaming cache policy (each byte is read once).
//
// These kernels serve fp32 and bf16 experts; MXFP4 experts have their own
// (ffn_gemv_mx.hip).
//
// Sources: "qwen35moe - Forward-Pass Design", section "Shared-expert MoE
// FFN" (SwiGLU experts, shared expert); "Phase 19: MoE - gpt-oss-20b",
// section 2 Experts (interleaved gate_up with bias, clamps, (up+1) * gate *
// sigmoid(alpha gate), down + bias).
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;  // wavefronts per workgroup

enum { W_F32 = 0, W_BF16 = 1 };

// Bytes of one weight row with `cols` inputs.
template <int WK> __host__ __device__ constexpr size_t row_bytes(int cols) {
  return WK == W_F32 ? (size_t)cols * 4 : (size_t)cols * 2;
}

// A 16-byte weight piece and the activation bytes it multiplies.
template <int WK> struct Wp;
template <> struct Wp<W_BF16> {
  static constexpr int kElems = 8, kXq = 1;  // elements; 16-byte activation words
  __device__ static float dot(uint4 w, const uint4* x, float acc, uint32_t) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x[0].x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x[0].y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x[0].z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x[0].w), acc, false);
    return acc;
  }
};
template <> struct Wp<W_F32> {
  static constexpr int kElems = 4, kXq = 1;
  __device__ static float dot(uint4 w, const uint4* x, float acc, uint32_t) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(x[0].x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(x[0].y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(x[0].z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(x[0].w), acc);
    return acc;
  }
};
// Weight rows per wavefront for NP 16-byte pieces per lane per row: about
// 8-16 KiB of weights each.
__host__ __device__ constexpr int rows_per_wave(int np) { return np >= 6 ? 1 : 8 / np; }
// gate/up: a row pair per feature
__host__ __device__ constexpr int gateup_rows_per_wave(int np) { return np >= 6 ? 1 : np == 4 ? 2 : 4; }
// tokens per register chunk: one keeps the gate/up kernel at 117 VGPRs (4
// waves per SIMD) and the down kernel at 61 (8), so more weight bytes are in
// flight per CU (two: 3 and 7 waves, 1.5% slower layer)
constexpr int kCh = 1;

struct Seg {
  int e, p0, n;
};

// The s-th non-empty segment of offsets[0 .. nseg] with its first sorted
// position and row count (one wavefront; the offsets of 512 segments are
// loaded per round trip), or e = -1.
__device__ Seg find_segment(const int32_t* __restrict__ off, int nseg, int s) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int base = 0; base < nseg; base += 8 * kWave) {
    int lo[8], hi[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int e = base + c * kWave + lane;
      lo[c] = e < nseg ? off[e] : 0;
      hi[c] = e < nseg ? off[e + 1] : 0;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bool ne = hi[c] > lo[c];
      const uint64_t m = __ballot(ne);
      const int cnt = __popcll(m);
      if (s < cnt) {
        const bool hit = ne && __popcll(m & ((1ull << lane) - 1ull)) == s;
        const int l = __ffsll((unsigned long long)__ballot(hit)) - 1;
        const int p0 = __builtin_amdgcn_readlane(lo[c], l);
        return Seg{base + c * kWave + l, p0, __builtin_amdgcn_readlane(hi[c], l) - p0};
      }
      s -= cnt;
    }
  }
  return Seg{-1, 0, 0};
}

// The segment a workgroup works on.  Workgroups are dispatched in blockIdx
// order, x fastest, so with the segment slot in blockIdx.y each segment's
// row groups go out together, and slot 0 is the shared expert (the segment
// with the most tokens, hence the longest compute), so it starts first and
// does not trail at the end; slot s > 0 is the (s-1)-th non-empty routed
// segment (the s-th without a shared expert).
// With segtab (the permutation's slot table) the segment is one scalar load
// that never queues behind other workgroups' weight loads; without it, a
// search of the offsets.
__device__ __forceinline__ Seg block_segment(const int32_t* off, int E, int shared,
                                             const int32_t* __restrict__ segtab) {
  const int slot = blockIdx.y;
  if (segtab) {
    const int4 v = reinterpret_cast<const int4*>(segtab)[slot];
    return Seg{__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
               __builtin_amdgcn_readfirstlane(v.z)};
  }
  Seg s;
  if (shared && slot == 0) {
    const int p0 = off[E];
    s = Seg{E, p0, off[E + 1] - p0};
  } else {
    s = find_segment(off, E, slot - shared);
  }
  return Seg{__builtin_amdgcn_readfirstlane(s.e), __builtin_amdgcn_readfirstlane(s.p0),
             __builtin_amdgcn_readfirstlane(s.n)};
}

// Activation pieces of one token: NP pieces of the row starting at byte
// `base` (kOutOfRange: zeros), matching the weight pieces of this lane.
template <typename XT, int WK, int NP>
__device__ __forceinline__ void load_act(__amdgpu_buffer_rsrc_t r, uint32_t base, bool valid, int P,
                                         uint4 (&xv)[NP][Wp<WK>::kXq]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int q = lane + p * kWave;
    const bool ok = valid && q < P;
#pragma unroll
    for (int j = 0; j < Wp<WK>::kXq; ++j)
      xv[p][j] = buf_load16(r, ok ? base + (uint32_t)(q * Wp<WK>::kElems * sizeof(XT) + j * 16) : kOutOfRange, 0);
  }
}

template <typename XT> __device__ __forceinline__ void store_elem(void* p, size_t i, float v) {
  if (sizeof(XT) == 4)
    reinterpret_cast<float*>(p)[i] = v;
  else
    reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16(v);
}

// Element i of a bias row held as raw words (bf16: two per word).
template <typename XT> __device__ __forceinline__ float bias_elem(uint32_t word, int i) {
  if (sizeof(XT) == 4) return __uint_as_float(word);
  return __uint_as_float((i & 1) ? (word & 0xFFFF0000u) : (word << 16));
}

struct GateUpArgs {
  const void* x;
  const void* gate_w;      // SWIGLU [E][F][H]  | OAI gate_up [E][2F][H]
  const void* up_w;        // SWIGLU [E][F][H]  | unused
  const void* gate_up_b;   // OAI [E][2F]
  const void* sh_gate_w;   // [Fs][H]
  const void* sh_up_w;     // [Fs][H]
  const int32_t* offsets;
  const int32_t* sorted_assign;
  void* h;
  const int32_t* segtab;    // the permutation's slot table, or NULL
  int32_t T, k, H, E, F, Fs, shared, oai;
  float alpha, limit;
};

// h[p][f] = act(gate row f . x_t, up row f . x_t) for every sorted position
// p of the workgroup's segment.  Grid: (groups of kWaves * RPW features,
// segment slot).
// sorted_assign is passed on its own, read-only and unaliased, so the
// uniform reads of it are scalar loads that never wait behind weight loads.
template <typename XT, int WK, int NP>
__global__ __launch_bounds__(kWaves * kWave) void k_gateup_gemv(GateUpArgs a, const int32_t* __restrict__ sorted,
                                                                const int32_t* __restrict__ segtab) {
  constexpr int RPW = gateup_rows_per_wave(NP);
  constexpr int XQ = Wp<WK>::kXq;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const Seg sg = block_segment(a.offsets, a.E, a.shared, segtab);
  if (sg.e < 0) return;
  const bool sh = sg.e == a.E;
  const int Fe = sh ? a.Fs : a.F;
  const int f0 = (blockIdx.x * kWaves + wv) * RPW;
  if (f0 >= Fe) return;
  const int nr = min(RPW, Fe - f0);
  const size_t rb = row_bytes<WK>(a.H);
  const int P = (int)(rb / 16);
  const bool oai = a.oai && !sh;
  const size_t e = (size_t)sg.e;
  // rows of feature f0 + r: gate at gb + r * stride, up at ub + r * stride
  const uint8_t *gb, *ub;
  size_t stride = rb;
  if (sh) {
    gb = (const uint8_t*)a.sh_gate_w + (size_t)f0 * rb;
    ub = (const uint8_t*)a.sh_up_w + (size_t)f0 * rb;
  } else if (oai) {
    gb = (const uint8_t*)a.gate_w + (e * 2 * a.F + 2 * f0) * rb;
    ub = gb + rb;
    stride = 2 * rb;
  } else {
    gb = (const uint8_t*)a.gate_w + (e * a.F + f0) * rb;
    ub = (const uint8_t*)a.up_w + (e * a.F + f0) * rb;
  }
  const uint32_t span = (uint32_t)((nr - 1) * stride + rb);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gb, span), ru = make_rsrc(ub, span);
  const int nas = a.T * a.k;
  // gate/up biases of the rows: one word per row (bf16 pair) or two (fp32)
  uint32_t bw[RPW][2];
  {
    const void* bb = oai && a.gate_up_b ? (const void*)((const XT*)a.gate_up_b + e * 2 * a.F + 2 * f0) : a.x;
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(bb, oai && a.gate_up_b ? (uint32_t)(nr * 2 * sizeof(XT)) : 0u);
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bw[r][j] = (sizeof(XT) == 4 || j == 0)
                       ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rbias, (int)(r * 2 * sizeof(XT) + j * 4), 0, 0)
                       : 0u;
  }
  uint4 G[RPW][NP], U[RPW][NP];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int q = lane + p * kWave;
      const uint32_t off = q < P ? (uint32_t)(r * stride + q * 16) : kOutOfRange;
      G[r][p] = buf_load16_once(rg, off, 0);
      U[r][p] = buf_load16_once(ru, off, 0);
    }
  const size_t xrb = (size_t)a.H * sizeof(XT);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((size_t)a.T * xrb));
  uint4 X0[kCh][NP][XQ], X1[kCh][NP][XQ];
  auto load_chunk = [&](int i0, uint4 (&X)[kCh][NP][XQ]) {
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      const int ii = i0 + i;
      const int as = ii < sg.n ? sorted[sg.p0 + ii] : 0;
      const int t = as < nas ? as / a.k : as - nas;
      load_act<XT, WK, NP>(rx, (uint32_t)(t * xrb), ii < sg.n, P, X[i]);
    }
  };
  auto compute_chunk = [&](int i0, const uint4 (&X)[kCh][NP][XQ]) {
    float ag[RPW][kCh], au[RPW][kCh];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int i = 0; i < kCh; ++i) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          g = Wp<WK>::dot(G[r][p], X[i][p], g, 0u);
          u = Wp<WK>::dot(U[r][p], X[i][p], u, 0u);
        }
        ag[r][i] = g;
        au[r][i] = u;
      }
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      const int p = sg.p0 + i0 + i;
      if (i0 + i < sg.n) {
        float hv = 0.f;
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          float gs = wave_sum(ag[r][i]), us = wave_sum(au[r][i]);
          float v;
          if (oai) {
            gs += bias_elem<XT>(bw[r][0], 0);
            us += sizeof(XT) == 4 ? __uint_as_float(bw[r][1]) : bias_elem<XT>(bw[r][0], 1);
            v = oai_act(gs, us, a.alpha, a.limit);
          } else {
            v = swiglu_act(gs, us);
          }
          hv = lane == r ? v : hv;
        }
        const size_t row = p < nas ? (size_t)p * a.F : (size_t)nas * a.F + (size_t)(p - nas) * a.Fs;
        if (lane < nr) store_elem<XT>(a.h, row + f0 + lane, hv);
      }
    }
  };
  load_chunk(0, X0);
  for (int i0 = 0; i0 < sg.n; i0 += 2 * kCh) {
    if (i0 + kCh < sg.n) load_chunk(i0 + kCh, X1);
    compute_chunk(i0, X0);
    if (i0 + kCh < sg.n) {
      if (i0 + 2 * kCh < sg.n) load_chunk(i0 + 2 * kCh, X0);
      compute_chunk(i0 + kCh, X1);
    }
  }
}

struct DownArgs {
  const void* h;
  const void* down_w;       // [E][H][F]
  const void* down_b;       // [E][H] or null
  const void* sh_down_w;    // [H][Fs]
  const int32_t* offsets;
  const int32_t* sorted_assign;
  float* y;                 // [T*k (+T)][H], row = assignment id
  const int32_t* segtab;    // the permutation's slot table, or NULL
  int32_t T, k, H, E, F, Fs, shared;
};

// y[a][o] = down row o . h[p] (+ bias) for every sorted position p of the
// segment, written at the row of its assignment id a.  Grid: (groups of
// kWaves * RPW output rows, segment slot).
template <typename XT, int WK, int NP>
__global__ __launch_bounds__(kWaves * kWave) void k_down_gemv(DownArgs a, const int32_t* __restrict__ sorted,
                                                              const int32_t* __restrict__ segtab) {
  constexpr int RPW = rows_per_wave(NP);
  constexpr int XQ = Wp<WK>::kXq;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const Seg sg = block_segment(a.offsets, a.E, a.shared, segtab);
  if (sg.e < 0) return;
  const bool sh = sg.e == a.E;
  const int Fe = sh ? a.Fs : a.F;
  const int o0 = (blockIdx.x * kWaves + wv) * RPW;
  if (o0 >= a.H) return;
  const int nr = min(RPW, a.H - o0);
  const size_t rb = row_bytes<WK>(Fe);
  const int P = (int)(rb / 16);
  const size_t e = (size_t)sg.e;
  const uint8_t* wb = sh ? (const uint8_t*)a.sh_down_w + (size_t)o0 * rb
                         : (const uint8_t*)a.down_w + (e * a.H + o0) * rb;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wb, (uint32_t)(nr * rb));
  const int nas = a.T * a.k;
  // bias words of the rows (bf16: element o0 + r in word (o0 + r) / 2)
  uint32_t bw[RPW];
  {
    const bool hb = !sh && a.down_b;
    const size_t first = hb ? (e * a.H + o0) & ~(size_t)(sizeof(XT) == 4 ? 0 : 1) : 0;
    const void* bb = hb ? (const void*)((const XT*)a.down_b + first) : a.h;
    const uint32_t bbytes = sizeof(XT) == 4 ? (uint32_t)nr * 4 : (uint32_t)(((o0 & 1) + nr - 1) / 2 * 4 + 4);
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(bb, hb ? bbytes : 0u);
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      bw[r] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
          rbias, (int)(sizeof(XT) == 4 ? r * 4 : ((o0 & 1) + r) / 2 * 4), 0, 0);
  }
  uint4 W[RPW][NP];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int q = lane + p * kWave;
      W[r][p] = buf_load16_once(rw, q < P ? (uint32_t)(r * rb + q * 16) : kOutOfRange, 0);
    }
  const size_t hrb = (size_t)Fe * sizeof(XT);
  const XT* hseg = sh ? (const XT*)a.h + (size_t)nas * a.F + (size_t)(sg.p0 - nas) * a.Fs
                      : (const XT*)a.h + (size_t)sg.p0 * a.F;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(hseg, (uint32_t)((size_t)sg.n * hrb));
  uint4 X0[kCh][NP][XQ], X1[kCh][NP][XQ];
  auto load_chunk = [&](int i0, uint4 (&X)[kCh][NP][XQ]) {
#pragma unroll
    for (int i = 0; i < kCh; ++i)
      load_act<XT, WK, NP>(rh, (uint32_t)((i0 + i) * hrb), i0 + i < sg.n, P, X[i]);
  };
  auto compute_chunk = [&](int i0, const uint4 (&X)[kCh][NP][XQ]) {
    float acc[RPW][kCh];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int i = 0; i < kCh; ++i) {
        float v = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) v = Wp<WK>::dot(W[r][p], X[i][p], v, 0u);
        acc[r][i] = v;
      }
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      if (i0 + i < sg.n) {
        float yv = 0.f;
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const float v = wave_sum(acc[r][i]) + bias_elem<XT>(bw[r], o0 + r);
          yv = lane == r ? v : yv;
        }
        const int as = sorted[sg.p0 + i0 + i];
        if (lane < nr) a.y[(size_t)as * a.H + o0 + lane] = yv;
      }
    }
  };
  load_chunk(0, X0);
  for (int i0 = 0; i0 < sg.n; i0 += 2 * kCh) {
    if (i0 + kCh < sg.n) load_chunk(i0 + kCh, X1);
    compute_chunk(i0, X0);
    if (i0 + kCh < sg.n) {
      if (i0 + 2 * kCh < sg.n) load_chunk(i0 + 2 * kCh, X0);
      compute_chunk(i0 + kCh, X1);
    }
  }
}

// out[t][o] = sum_j w[t][j] y[t*k + j][o] (+ sgate[t] y[T*k + t][o]), the
// picks summed in pick order, in fp32.  The y rows of up to 8 picks are
// loaded together before the sums, so the loads overlap.  This form takes
// the few-token kernels' fp32 y, 4 outputs per thread.
__device__ __forceinline__ float4 load_y4(const float* y, size_t row, int o4, int H) {
  return reinterpret_cast<const float4*>(y + row * H)[o4];
}

// RD: residual rows added last (the decoder block's residual): 0 none,
// 1 bf16, 2 fp32 (a template parameter: a runtime choice between two
// loads made the wave wait for one before issuing the y loads).
// SH: a shared expert (its row and gate), likewise a template parameter.
template <int RD, bool SH>
__global__ __launch_bounds__(256) void k_combine_gather(const float* __restrict__ y, const float* __restrict__ topk_w,
                                                        const float* __restrict__ sgate, int32_t T, int32_t k,
                                                        int32_t H, float* __restrict__ out,
                                                        const void* __restrict__ resid) {
  constexpr int kBatch = 8;
  const int t = blockIdx.y;
  const int o4 = blockIdx.x * blockDim.x + threadIdx.x;  // index of 4 outputs
  if (o4 * 4 >= H) return;
  // the shared expert's row is loaded with the first batch of picks (one
  // round trip for k <= 8) and added last
  float g = 0.f;
  float4 vs = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (SH) {
    g = sgate[t];
    vs = load_y4(y, (size_t)T * k + t, o4, H);
  }
  // raw residual bits, converted only where they are added: a conversion
  // right after the load would make the wave wait for it before the y loads
  uint4 rraw = make_uint4(0, 0, 0, 0);
  if constexpr (RD == 1) {
    const uint2 v = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(resid) + (size_t)t * H)[o4];
    rraw = make_uint4(v.x, v.y, 0, 0);
  } else if constexpr (RD == 2) {
    rraw = reinterpret_cast<const uint4*>(static_cast<const float*>(resid) + (size_t)t * H)[o4];
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += kBatch) {
    float4 v[kBatch];
    float wj[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool ok = j0 + j < k;
      wj[j] = ok ? topk_w[(size_t)t * k + j0 + j] : 0.f;
      v[j] = ok ? load_y4(y, (size_t)t * k + j0 + j, o4, H) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j0 + j < k) {
        acc.x = fmaf(wj[j], v[j].x, acc.x);
        acc.y = fmaf(wj[j], v[j].y, acc.y);
        acc.z = fmaf(wj[j], v[j].z, acc.z);
        acc.w = fmaf(wj[j], v[j].w, acc.w);
      }
    }
  }
  if constexpr (SH) {
    acc.x = fmaf(g, vs.x, acc.x);
    acc.y = fmaf(g, vs.y, acc.y);
    acc.z = fmaf(g, vs.z, acc.z);
    acc.w = fmaf(g, vs.w, acc.w);
  }
  if constexpr (RD != 0) {
    const float4 res = RD == 1 ? make_float4(bf16lo(rraw.x), bf16hi(rraw.x), bf16lo(rraw.y), bf16hi(rraw.y))
                               : make_float4(__uint_as_float(rraw.x), __uint_as_float(rraw.y),
                                             __uint_as_float(rraw.z), __uint_as_float(rraw.w));
    acc.x = res.x + acc.x;
    acc.y = res.y + acc.y;
    acc.z = res.z + acc.z;
    acc.w = res.w + acc.w;
  }
  reinterpret_cast<float4*>(out + (size_t)t * H)[o4] = acc;
}

// The same sum for bf16 y (the grouped GEMMs' output): 8 outputs per thread,
// so each y row piece is one 16-byte load.  Same operations in the same
// order per output.  Its layers have bf16 x, so a residual is bf16 (RD 0/1).
template <int RD, bool SH>
__global__ __launch_bounds__(256) void k_combine_gather8(const uint16_t* __restrict__ y,
                                                         const float* __restrict__ topk_w,
                                                         const float* __restrict__ sgate, int32_t T, int32_t k,
                                                         int32_t H, float* __restrict__ out,
                                                         const void* __restrict__ resid) {
  constexpr int kBatch = 8;
  const int t = blockIdx.y;
  const int o8 = blockIdx.x * blockDim.x + threadIdx.x;  // index of 8 outputs
  static_assert(RD == 0 || RD == 1, "bf16 residual rows only");
  if (o8 * 8 >= H) return;
  float g = 0.f;
  uint4 sraw = make_uint4(0, 0, 0, 0);
  if constexpr (SH) {
    g = sgate[t];
    sraw = reinterpret_cast<const uint4*>(y + ((size_t)T * k + t) * H)[o8];
  }
  uint4 rraw = make_uint4(0, 0, 0, 0);
  if constexpr (RD == 1) rraw = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(resid) + (size_t)t * H)[o8];
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < k; j0 += kBatch) {
    uint4 q[kBatch];
    float wj[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool ok = j0 + j < k;
      wj[j] = ok ? topk_w[(size_t)t * k + j0 + j] : 0.f;
      q[j] = ok ? reinterpret_cast<const uint4*>(y + ((size_t)t * k + j0 + j) * H)[o8] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j0 + j < k) {
        const uint32_t w4[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(wj[j], bf16lo(w4[i]), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wj[j], bf16hi(w4[i]), acc[2 * i + 1]);
        }
      }
    }
  }
  if constexpr (SH) {
    const uint32_t w4[4] = {sraw.x, sraw.y, sraw.z, sraw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(g, bf16lo(w4[i]), acc[2 * i]);
      acc[2 * i + 1] = fmaf(g, bf16hi(w4[i]), acc[2 * i + 1]);
    }
  }
  if constexpr (RD == 1) {
    const uint32_t w4[4] = {rraw.x, rraw.y, rraw.z, rraw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = bf16lo(w4[i]) + acc[2 * i];
      acc[2 * i + 1] = bf16hi(w4[i]) + acc[2 * i + 1];
    }
  }
  float4* dst = reinterpret_cast<float4*>(out + (size_t)t * H) + 2 * o8;
  dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

}  // namespace

// Defined in ffn_mfma.hip.
hipError_t launch_gateup_mfma(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                              const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s);
hipError_t launch_down_mfma(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                            const int32_t* sorted_assign, int32_t T, uint16_t* y, hipStream_t s);
bool mfma_shapes_ok(const moe_config* c);
// Defined in ffn_gemv_mx.hip (MXFP4 experts).
hipError_t launch_expert_ffn_mx(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                                const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s,
                                const int32_t* segtab);
hipError_t launch_down_mx(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                          const int32_t* sorted_assign, int32_t T, float* y, hipStream_t s, const int32_t* segtab);

static int max_routed_segments(const moe_config* c, int32_t T) {
  const int64_t nk = (int64_t)T * c->top_k;
  return (int)(nk < c->n_expert ? nk : c->n_expert);
}

// 16-byte pieces per lane for rows of `cols` inputs: 1, 2, 4, 6 or 8.
static int pieces_per_lane(size_t row_bytes) {
  const size_t np = (row_bytes / 16 + kWave - 1) / kWave;
  return np <= 1 ? 1 : np <= 2 ? 2 : np <= 4 ? 4 : np <= 6 ? 6 : 8;
}
static size_t row_bytes_of(int wdt, int cols) {
  return wdt == MOE_DTYPE_F32 ? (size_t)cols * 4 : wdt == MOE_DTYPE_BF16 ? (size_t)cols * 2 : (size_t)cols / 2;
}

template <typename XT, int WK, int NP> static void gateup_launch(dim3 g, const GateUpArgs& a, hipStream_t s) {
  k_gateup_gemv<XT, WK, NP><<<g, kWaves * kWave, 0, s>>>(a, a.sorted_assign, a.segtab);
}
template <typename XT, int WK, int NP> static void down_launch(dim3 g, const DownArgs& a, hipStream_t s) {
  k_down_gemv<XT, WK, NP><<<g, kWaves * kWave, 0, s>>>(a, a.sorted_assign, a.segtab);
}

#define MOE_NP_SWITCH(FN, XT, WK, np, grid, args, s) \
  switch (np) {                                      \
    case 1: FN<XT, WK, 1>(grid, args, s); break;     \
    case 2: FN<XT, WK, 2>(grid, args, s); break;     \
    case 4: FN<XT, WK, 4>(grid, args, s); break;     \
    case 6: FN<XT, WK, 6>(grid, args, s); break;     \
    default: FN<XT, WK, 8>(grid, args, s); break;    \
  }

// One gate/up launch over every segment slot.
static void gateup_dispatch(const moe_config* c, const GateUpArgs& a, int wdt, int nslots, int fe, hipStream_t s) {
  const int np = pieces_per_lane(row_bytes_of(wdt, c->hidden));
  const int rpw = gateup_rows_per_wave(np);
  const dim3 grid((fe + kWaves * rpw - 1) / (kWaves * rpw), nslots);
  if (c->x_dtype == MOE_DTYPE_F32) {
    MOE_NP_SWITCH(gateup_launch, float, W_F32, np, grid, a, s)
  } else {
    MOE_NP_SWITCH(gateup_launch, uint16_t, W_BF16, np, grid, a, s)
  }
}

static void down_dispatch(const moe_config* c, const DownArgs& a, int wdt, int nslots, int cols, hipStream_t s) {
  const int np = pieces_per_lane(row_bytes_of(wdt, cols));
  const int rpw = rows_per_wave(np);
  const dim3 grid((c->hidden + kWaves * rpw - 1) / (kWaves * rpw), nslots);
  if (c->x_dtype == MOE_DTYPE_F32) {
    MOE_NP_SWITCH(down_launch, float, W_F32, np, grid, a, s)
  } else {
    MOE_NP_SWITCH(down_launch, uint16_t, W_BF16, np, grid, a, s)
  }
}
#undef MOE_NP_SWITCH

int gemv_slots(const moe_config* c, int32_t T) { return max_routed_segments(c, T) + (c->shared_ff > 0); }

hipError_t launch_expert_ffn(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                             const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s,
                             const int32_t* segtab) {
  if (T == 0) return hipSuccess;
  if (T > kGemvMaxT && mfma_shapes_ok(c)) return launch_gateup_mfma(c, w, x, offsets, sorted_assign, T, h, s);
  if (c->w_dtype == MOE_DTYPE_MXFP4) return launch_expert_ffn_mx(c, w, x, offsets, sorted_assign, T, h, s, segtab);
  GateUpArgs a;
  const bool oai = c->act == MOE_ACT_SWIGLU_OAI;
  a.x = x;
  a.gate_w = oai ? w->gate_up_w : w->gate_w;
  a.up_w = w->up_w;
  a.gate_up_b = w->gate_up_b;
  a.sh_gate_w = w->sh_gate_w;
  a.sh_up_w = w->sh_up_w;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.h = h;
  a.segtab = segtab;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.shared = c->shared_ff > 0; a.oai = oai; a.alpha = c->act_alpha; a.limit = c->act_limit;
  const int fmax = c->expert_ff > c->shared_ff ? c->expert_ff : c->shared_ff;
  gateup_dispatch(c, a, c->w_dtype, gemv_slots(c, T), fmax, s);
  return hipGetLastError();
}

bool y_is_bf16(const moe_config* c, int32_t T) { return T > kGemvMaxT && mfma_shapes_ok(c); }

hipError_t launch_down(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                       const int32_t* sorted_assign, int32_t T, void* yv, hipStream_t s, const int32_t* segtab) {
  if (T == 0) return hipSuccess;
  if (y_is_bf16(c, T)) return launch_down_mfma(c, w, h, offsets, sorted_assign, T, (uint16_t*)yv, s);
  float* y = (float*)yv;
  if (c->w_dtype == MOE_DTYPE_MXFP4) return launch_down_mx(c, w, h, offsets, sorted_assign, T, y, s, segtab);
  DownArgs a;
  a.h = h;
  a.down_w = w->down_w;
  a.down_b = c->act == MOE_ACT_SWIGLU_OAI ? w->down_b : nullptr;
  a.sh_down_w = w->sh_down_w;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.y = y;
  a.segtab = segtab;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.shared = c->shared_ff > 0;
  // one piece count for both: the wider of the routed and shared rows
  const int cols = c->expert_ff >= c->shared_ff ? c->expert_ff : c->shared_ff;
  down_dispatch(c, a, c->w_dtype, gemv_slots(c, T), cols, s);
  return hipGetLastError();
}

template <bool SH>
static void combine_launch_sh(int rd, dim3 grid, int threads, hipStream_t s, const float* y, const float* topk_w,
                              const float* sg, int32_t T, int32_t k, int32_t H, float* out, const void* resid) {
  if (rd == 1)
    k_combine_gather<1, SH><<<grid, threads, 0, s>>>(y, topk_w, sg, T, k, H, out, resid);
  else if (rd == 2)
    k_combine_gather<2, SH><<<grid, threads, 0, s>>>(y, topk_w, sg, T, k, H, out, resid);
  else
    k_combine_gather<0, SH><<<grid, threads, 0, s>>>(y, topk_w, sg, T, k, H, out, resid);
}

hipError_t launch_combine_gather(const moe_config* c, const void* y, const float* topk_w, const float* sgate,
                                 int32_t T, float* out, hipStream_t s, const void* resid) {
  if (T == 0) return hipSuccess;
  // few tokens: 64-thread workgroups, so the loads spread over more CUs
  const int threads = T <= kGemvMaxT ? 64 : 256;
  dim3 grid((c->hidden / 4 + threads - 1) / threads, T);
  const float* sg = c->shared_ff > 0 ? sgate : nullptr;
  const int rd = !resid ? 0 : c->x_dtype == MOE_DTYPE_BF16 ? 1 : 2;
  if (y_is_bf16(c, T)) {
    // bf16 y comes from the MFMA path: x (so any residual) is bf16 and the
    // hidden size a multiple of 32, so every row splits into 8-output pieces
    const dim3 g8((c->hidden / 8 + threads - 1) / threads, T);
    const uint16_t* yb = (const uint16_t*)y;
#define MOE_C8(RD, SH) k_combine_gather8<RD, SH><<<g8, threads, 0, s>>>(yb, topk_w, sg, T, c->top_k, c->hidden, out, resid)
    if (sg) {
      if (rd) MOE_C8(1, true); else MOE_C8(0, true);
    } else {
      if (rd) MOE_C8(1, false); else MOE_C8(0, false);
    }
#undef MOE_C8
  } else if (sg) {
    combine_launch_sh<true>(rd, grid, threads, s, (const float*)y, topk_w, sg, T, c->top_k, c->hidden, out, resid);
  } else {
    combine_launch_sh<false>(rd, grid, threads, s, (const float*)y, topk_w, sg, T, c->top_k, c->hidden, out, resid);
  }
  return hipGetLastError();
}

}  // namespace moe
