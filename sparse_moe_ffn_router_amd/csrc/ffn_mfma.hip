// Grouped expert GEMMs (and the router product) on bf16 MFMA for
// prefill-sized batches.
//
// One workgroup of 8 waves computes a 128 x 256 tile: 128 sorted rows of one
// expert segment (the rows of a segment are contiguous after the
// permutation) by 256 weight rows.  K advances in steps of 64; global loads
// run two steps ahead through registers into a double-buffered LDS tile
// (rows padded by 16 bytes).  Waves sit 2 (rows) x 4 (columns), each 64 x 64
// as 2 x 2 v_mfma_f32_32x32x16_bf16 blocks.
//
//  gate/up: A = x rows gathered by token; the 256 weight rows are 128 gate
//           rows and the 128 matching up rows (for the interleaved gpt-oss
//           gate_up, the even and odd rows of the tile's 256 fused rows), so
//           a lane holds gate and up of the same (row, feature) in two
//           accumulators and the activation runs in registers; h is bf16.
//  down:    A = h rows; the 256 weight rows are output columns; the result
//           (+ bias) is written as fp32 at the row of the assignment id,
//           ready for the gather-combine.
//  router:  A = x rows; weight rows = router rows; fp32 logits (+ bias).
// MXFP4 weights are decoded to bf16 while staging (one 16-byte piece is one
// 32-element block with its E8M0 exponent).
//
// Sources: "qwen35moe - Forward-Pass Design", section "Shared-expert MoE
// FFN"; "Phase 19: MoE - gpt-oss-20b", section 2 Router and Experts, and
// section 3.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements)
constexpr int kThreads = 512;
constexpr int kAChunks = BM * BK / 8 / kThreads;  // 16-byte A pieces per thread per step (2)
constexpr int kBChunks = BN * BK / 8 / kThreads;  // 16-byte B pieces per thread per step (4)

enum { MODE_GATEUP = 0, MODE_DOWN = 1, MODE_ROUTER = 2 };

struct GemmArgs {
  const uint16_t* a_src;     // gate/up, router: x [T][H]; down: h
  const void* w0;            // gate/up SWIGLU gate_w | OAI gate_up_w ; down: down_w ; router: router_w
  const void* w1;            // gate/up SWIGLU up_w
  const uint8_t* scales;     // MXFP4 scales of w0
  const uint16_t* bias;      // OAI gate_up_b [E][2F] | down_b [E][H] | router_b [E]
  const uint16_t* sh0;       // shared gate_w [Fs][H] | shared down [H][Fs]
  const uint16_t* sh1;       // shared up_w
  const int32_t* offsets;
  const int32_t* sorted_assign;
  void* out;                 // h (bf16) | y (fp32) | router logits (fp32)
  int32_t T, k, H, E, F, Fs, shared, oai;
  int32_t n_tiles;           // column tiles per segment (max over segments)
  int32_t m_tiles_max;       // grid bound on row tiles
  float alpha, limit;
};

// Row tile mt -> (segment, first sorted position); -1 if past the last tile.
__device__ int tile_lookup(const int32_t* __restrict__ offsets, int nseg, int mt, int* row0) {
  const int lane = threadIdx.x & (kWave - 1);
  int acc = 0;
  for (int base = 0; base < nseg; base += kWave) {
    const int e = base + lane;
    const int cnt = e < nseg ? (offsets[e + 1] - offsets[e] + BM - 1) / BM : 0;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += u;
    }
    const int total = __shfl(incl, kWave - 1, kWave);
    if (mt < acc + total) {
      const bool hit = (mt >= acc + incl - cnt) && (mt < acc + incl);
      const uint64_t m = __ballot(hit);
      const int src = __ffsll((unsigned long long)m) - 1;
      const int excl = __shfl(acc + incl - cnt, src, kWave);
      const int seg = base + src;
      *row0 = offsets[seg] + (mt - excl) * BM;
      return seg;
    }
    acc += total;
  }
  return -1;
}

__device__ __forceinline__ void store_u4(uint16_t* lds, int row, int col8, uint4 v) {
  *reinterpret_cast<uint4*>(lds + row * LDK + col8 * 8) = v;
}

// One 32-element MXFP4 block (16 code bytes, E8M0 exponent) to 32 bf16.
__device__ __forceinline__ void mxfp4_block_to_bf16(uint4 codes, uint32_t e8m0, uint4 out[4]) {
  const float sc = e8m0_to_f32(e8m0);
  const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 0);
    const bf16x2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 1);
    const bf16x2_t b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 2);
    const bf16x2_t b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 3);
    out[q] = make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                        __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3));
  }
}

// Staging registers of one K step.
struct Stage {
  uint4 a[kAChunks];
  uint4 b[kBChunks];   // bf16 pieces, or in b[0] the MXFP4 block
  uint32_t sc;         // MXFP4 block exponent
};

template <int MODE, bool MX>
__global__ __launch_bounds__(kThreads, 1) void k_grouped_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][BN * LDK];

  // XCD-aware order: the hardware deals workgroups round-robin over 8 XCDs;
  // give each XCD a contiguous run of (column tile, row tiles) so the row
  // tiles sharing one weight tile meet in the same L2.
  const int nblk = gridDim.x;
  const int per_xcd = nblk / 8;
  const int lin = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int nt = lin / a.m_tiles_max;
  const int mt = lin % a.m_tiles_max;
  const int nseg = a.E + a.shared;
  int p0, seg, rows;
  if (MODE == MODE_ROUTER) {
    seg = 0;
    p0 = mt * BM;
    rows = min(BM, a.T - p0);
    if (rows <= 0) return;
  } else {
    seg = tile_lookup(a.offsets, nseg, mt, &p0);
    if (seg < 0) return;
    rows = min(BM, a.offsets[seg + 1] - p0);
  }
  const bool sh = MODE != MODE_ROUTER && seg == a.E;
  const int64_t nas = (int64_t)a.T * a.k;
  const int Fe = sh ? a.Fs : a.F;
  const int ncols = MODE == MODE_GATEUP ? Fe : MODE == MODE_DOWN ? a.H : a.E;
  const int col_tile = MODE == MODE_GATEUP ? BN / 2 : BN;  // features | outputs per tile
  const int c0 = nt * col_tile;
  if (c0 >= ncols) return;
  const int K = MODE == MODE_DOWN ? Fe : a.H;
  const bool mx = MX && !sh && MODE != MODE_ROUTER;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const int wm = wid >> 2, wn = wid & 3;

  // ---- per-thread staging sources (fixed over K).  Piece q = tid + i*512
  // covers row q/8, 16-byte column q%8 of the step.
  const uint16_t* a_ptr[kAChunks];
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int q = tid + i * kThreads;
    const int r = min(q / 8, rows - 1);
    const int p = p0 + r;
    const uint16_t* base;
    if (MODE == MODE_ROUTER) {
      base = a.a_src + (size_t)p * a.H;
    } else if (MODE == MODE_GATEUP) {
      const int asg = a.sorted_assign[p];
      const int t = asg < nas ? asg / a.k : (int)(asg - nas);
      base = a.a_src + (size_t)t * a.H;
    } else {
      base = p < nas ? a.a_src + (size_t)p * a.F : a.a_src + (size_t)nas * a.F + (size_t)(p - nas) * a.Fs;
    }
    a_ptr[i] = base + (q % 8) * 8;
  }
  auto wrow = [&](int r) -> int {  // row of the segment's weight matrix for tile row r
    if (MODE == MODE_GATEUP) {
      const int f = min(c0 + (r & (BN / 2 - 1)), Fe - 1);
      if (a.oai && !sh) return 2 * f + (r >= BN / 2);
      return f;  // gate (r < BN/2) or up (r >= BN/2) matrix row f
    }
    if (MODE == MODE_ROUTER) return min(c0 + r, a.E - 1);
    return min(c0 + r, a.H - 1);
  };
  const uint16_t* b_ptr[kBChunks];
  const uint8_t* b_code = nullptr;
  const uint8_t* b_sc = nullptr;
  if (!mx) {
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / 8;
      const int wr = wrow(r);
      const uint16_t* base;
      if (MODE == MODE_ROUTER) {
        base = (const uint16_t*)a.w0 + (size_t)wr * a.H;
      } else if (MODE == MODE_GATEUP) {
        if (sh)
          base = (r < BN / 2 ? a.sh0 : a.sh1) + (size_t)wr * a.H;
        else if (a.oai)
          base = (const uint16_t*)a.w0 + ((size_t)seg * 2 * a.F + wr) * a.H;
        else
          base = (const uint16_t*)(r < BN / 2 ? a.w0 : a.w1) + ((size_t)seg * a.F + wr) * a.H;
      } else {
        base = sh ? a.sh0 + (size_t)wr * a.Fs : (const uint16_t*)a.w0 + ((size_t)seg * a.H + wr) * a.F;
      }
      b_ptr[i] = base + (q % 8) * 8;
    }
  } else {
    // one 32-element block per thread per step: tile row tid/2, block tid%2
    const int r = tid / 2;
    const int wr = wrow(r);
    const size_t row = MODE == MODE_GATEUP ? (size_t)seg * 2 * a.F + wr : (size_t)seg * a.H + wr;
    b_code = (const uint8_t*)a.w0 + row * (K / 2) + (tid % 2) * 16;
    b_sc = a.scales + row * (K / 32) + (tid % 2);
  }

  auto g_load = [&](Stage& st, int k0) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) st.a[i] = *reinterpret_cast<const uint4*>(a_ptr[i] + k0);
    if (!mx) {
#pragma unroll
      for (int i = 0; i < kBChunks; ++i) st.b[i] = *reinterpret_cast<const uint4*>(b_ptr[i] + k0);
    } else {
      st.b[0] = *reinterpret_cast<const uint4*>(b_code + k0 / 2);
      st.sc = b_sc[k0 / 32];
    }
  };
  auto s_store = [&](const Stage& st, int buf) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int q = tid + i * kThreads;
      store_u4(lds_a[buf], q / 8, q % 8, st.a[i]);
    }
    if (!mx) {
#pragma unroll
      for (int i = 0; i < kBChunks; ++i) {
        const int q = tid + i * kThreads;
        store_u4(lds_b[buf], q / 8, q % 8, st.b[i]);
      }
    } else {
      uint4 d[4];
      mxfp4_block_to_bf16(st.b[0], st.sc, d);
      const int r = tid / 2, blk = tid % 2;
#pragma unroll
      for (int q = 0; q < 4; ++q) store_u4(lds_b[buf], r, blk * 4 + q, d[q]);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // LDS rows of this wave's operands
  const int arow = wm * 64 + (lane & 31);
  int brow[2];
  if (MODE == MODE_GATEUP) {
    brow[0] = wn * 32 + (lane & 31);           // gate rows
    brow[1] = BN / 2 + wn * 32 + (lane & 31);  // matching up rows
  } else {
    brow[0] = wn * 64 + (lane & 31);
    brow[1] = wn * 64 + 32 + (lane & 31);
  }
  const int kofs = (lane >> 5) * 8;

  const int nk = K / BK;
  Stage s0, s1;
  g_load(s0, 0);
  if (nk > 1) g_load(s1, BK);
  s_store(s0, 0);
  __syncthreads();
  // step kt computes LDS buffer kt&1 while the loads of step kt+2 land in
  // `nxt` (whose previous content was already stored) and step kt+1 (in
  // `pend`) goes to the other buffer at the end
  auto step = [&](int kt, Stage& nxt, Stage& pend, int buf) {
    if (kt + 2 < nk) g_load(nxt, (kt + 2) * BK);
    const uint16_t* la = lds_a[buf];
    const uint16_t* lb = lds_b[buf];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const bf16x8_t*>(la + (arow + i * 32) * LDK + kk + kofs);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const bf16x8_t*>(lb + brow[j] * LDK + kk + kofs);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) s_store(pend, buf ^ 1);
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, s0, s1, 0);
    if (kt + 1 < nk) step(kt + 1, s1, s0, 1);
  }

  // ---- epilogue.  Lane l of a 32x32 block holds column (l & 31) and rows
  // (q / 4) * 8 + (l / 32) * 4 + (q % 4), q = 0..15.
  const int colin = lane & 31;
  if (MODE == MODE_GATEUP) {
    const int f = c0 + wn * 32 + colin;
    if (f < Fe) {
      float bg = 0.f, bu = 0.f;
      if (a.oai && !sh && a.bias) {
        bg = __uint_as_float((uint32_t)a.bias[(size_t)seg * 2 * a.F + 2 * f] << 16);
        bu = __uint_as_float((uint32_t)a.bias[(size_t)seg * 2 * a.F + 2 * f + 1] << 16);
      }
      uint16_t* h = (uint16_t*)a.out;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm * 64 + i * 32 + (q / 4) * 8 + (lane >> 5) * 4 + (q & 3);
          if (r < rows) {
            float hv;
            if (a.oai && !sh) {
              const float g = fminf(acc[i][0][q] + bg, a.limit);
              const float u = fminf(fmaxf(acc[i][1][q] + bu, -a.limit), a.limit);
              hv = (u + 1.f) * (g / (1.f + expf(-a.alpha * g)));
            } else {
              const float g = acc[i][0][q];
              hv = g / (1.f + expf(-g)) * acc[i][1][q];
            }
            const int p = p0 + r;
            const size_t rowoff = p < nas ? (size_t)p * a.F : (size_t)nas * a.F + (size_t)(p - nas) * a.Fs;
            h[rowoff + f] = (uint16_t)f32_to_bf16(hv);
          }
        }
    }
  } else {
    float* y = (float*)a.out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = c0 + wn * 64 + j * 32 + colin;
      if (o < ncols) {
        float bias = 0.f;
        if (MODE == MODE_ROUTER && a.bias) bias = __uint_as_float((uint32_t)a.bias[o] << 16);
        if (MODE == MODE_DOWN && !sh && a.bias) bias = __uint_as_float((uint32_t)a.bias[(size_t)seg * a.H + o] << 16);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = wm * 64 + i * 32 + (q / 4) * 8 + (lane >> 5) * 4 + (q & 3);
            if (r < rows) {
              const size_t orow = MODE == MODE_ROUTER ? (size_t)(p0 + r) : (size_t)a.sorted_assign[p0 + r];
              y[orow * ncols + o] = acc[i][j][q] + bias;
            }
          }
      }
    }
  }
}

int row_tiles_bound(const moe_config* c, int32_t T) {
  const int64_t nk = (int64_t)T * c->top_k;
  const int64_t nonempty = nk < c->n_expert ? nk : c->n_expert;
  int64_t b = (nk + (int64_t)(BM - 1) * nonempty) / BM;
  if (c->shared_ff > 0) b += (T + BM - 1) / BM;
  return (int)b;
}

template <int MODE>
hipError_t launch(const GemmArgs& a, bool mx, hipStream_t s) {
  int64_t blocks = (int64_t)a.n_tiles * a.m_tiles_max;
  blocks = (blocks + 7) / 8 * 8;
  if (mx)
    k_grouped_gemm<MODE, true><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  else
    k_grouped_gemm<MODE, false><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_mfma(const moe_config* c, const moe_weights* w, const void* x, int32_t T, float* logits,
                              float* sgate_pre, hipStream_t s) {
  (void)sgate_pre;  // the shared-gate dot is taken by the gating kernel
  GemmArgs a = {};
  a.a_src = (const uint16_t*)x;
  a.w0 = w->router_w;
  a.bias = (const uint16_t*)w->router_b;
  a.out = logits;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.n_tiles = (c->n_expert + BN - 1) / BN;
  a.m_tiles_max = (T + BM - 1) / BM;
  return launch<MODE_ROUTER>(a, false, s);
}

bool mfma_shapes_ok(const moe_config* c) {
  return c->x_dtype == MOE_DTYPE_BF16 && c->hidden % BK == 0 && c->expert_ff % BK == 0 && c->shared_ff % BK == 0;
}

hipError_t launch_gateup_mfma(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                              const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s) {
  GemmArgs a = {};
  const bool oai = c->act == MOE_ACT_SWIGLU_OAI;
  a.a_src = (const uint16_t*)x;
  a.w0 = oai ? w->gate_up_w : w->gate_w;
  a.w1 = w->up_w;
  a.scales = w->gate_up_scales;
  a.bias = (const uint16_t*)w->gate_up_b;
  a.sh0 = (const uint16_t*)w->sh_gate_w;
  a.sh1 = (const uint16_t*)w->sh_up_w;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.out = h;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.shared = c->shared_ff > 0; a.oai = oai; a.alpha = c->act_alpha; a.limit = c->act_limit;
  const int fmax = c->expert_ff > c->shared_ff ? c->expert_ff : c->shared_ff;
  a.n_tiles = (fmax + BN / 2 - 1) / (BN / 2);
  a.m_tiles_max = row_tiles_bound(c, T);
  return launch<MODE_GATEUP>(a, c->w_dtype == MOE_DTYPE_MXFP4, s);
}

hipError_t launch_down_mfma(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                            const int32_t* sorted_assign, int32_t T, float* y, hipStream_t s) {
  GemmArgs a = {};
  a.a_src = (const uint16_t*)h;
  a.w0 = w->down_w;
  a.scales = w->down_scales;
  a.bias = c->act == MOE_ACT_SWIGLU_OAI ? (const uint16_t*)w->down_b : nullptr;
  a.sh0 = (const uint16_t*)w->sh_down_w;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.out = y;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.shared = c->shared_ff > 0; a.oai = c->act == MOE_ACT_SWIGLU_OAI;
  a.n_tiles = (c->hidden + BN - 1) / BN;
  a.m_tiles_max = row_tiles_bound(c, T);
  return launch<MODE_DOWN>(a, c->w_dtype == MOE_DTYPE_MXFP4, s);
}

}  // namespace moe
