// Grouped expert GEMMs (and the router product) on bf16 MFMA for
// prefill-sized batches.
//
// One workgroup of 8 waves computes a 128 x 256 tile: 128 sorted rows of one
// expert segment (the rows of a segment are contiguous after the
// permutation) by 256 weight rows.  K advances in steps of 64 through a ring
// of three LDS stages filled by direct buffer-to-LDS loads issued two steps
// ahead; each 128-byte LDS row holds its eight 16-byte pieces in XOR-swizzled
// order (piece c of row r at slot c ^ ((r >> 1) & 7)) so MFMA operand reads
// spread over the banks.  Waves sit 2 (rows) x 4 (columns), each 64 x 64 as 2 x 2
// v_mfma_f32_32x32x16_bf16 blocks.
//
//  gate/up: A = x rows gathered by token; the 256 weight rows are 128 gate
//           rows and the 128 matching up rows (for the interleaved gpt-oss
//           gate_up, the even and odd rows of the tile's 256 fused rows), so
//           a lane holds gate and up of the same (row, feature) in two
//           accumulators and the activation runs in registers; h is bf16.
//  down:    A = h rows; the 256 weight rows are output columns; the result
//           (+ bias, fp32 accumulate) is written as bf16 at the row of the
//           assignment id, ready for the gather-combine (which sums in fp32).
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
constexpr int kThreads = 512;
constexpr int kStages = 3;
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
  void* out;                 // h (bf16) | y (bf16) | router logits (fp32)
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

// Number of BM-row tiles over all segments (wave-uniform).
__device__ int count_row_tiles(const int32_t* __restrict__ offsets, int nseg) {
  const int lane = threadIdx.x & (kWave - 1);
  int acc = 0;
  for (int base = 0; base < nseg; base += kWave) {
    const int e = base + lane;
    acc += e < nseg ? (offsets[e + 1] - offsets[e] + BM - 1) / BM : 0;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  return acc;
}

// Byte offset of 16-byte piece c (of 8) in row r of a swizzled 128-byte-row
// tile.  Two 128-byte rows span the 64 four-byte banks, so 16 consecutive
// rows read at one logical piece (what 16 lanes of an MFMA operand read do)
// hit 16 distinct 16-byte bank groups when the slot is c ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz_slot(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + (swz_slot(r, c) << 4); }

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

// MXFP4 weight block of one K step held in registers until converted.
struct CodeRegs {
  uint4 codes;
  uint32_t sc;
};

// Per-thread state of the K pipeline.
struct Pipe {
  __amdgpu_buffer_rsrc_t ra, rw0, rw1, rsc;
  uint32_t a_off[kAChunks], b_off[kBChunks], sc_off;
  bool two_mats, mx;
  int nk, wid, tid, arow0, brow0, brow1, khalf;
};

// Issue the loads of step s into stage (la, lb) (all lanes, always: a step
// past the end reads at an out-of-range offset, i.e. zeros, so every step
// has the same number of outstanding loads).
__device__ __forceinline__ void pipe_issue(const Pipe& p, int s, uint8_t* __restrict__ la, uint8_t* __restrict__ lb,
                                           CodeRegs& cr) {
  const uint32_t kb = s < p.nk ? (uint32_t)s * BK * 2 : kOutOfRange;  // byte offset of the step in a bf16 row
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) dma16(p.ra, la + (i * kThreads + p.wid * kWave) * 16, p.a_off[i] + kb);
  if (!p.mx) {
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const bool up = p.two_mats && i >= kBChunks / 2;  // pieces i >= 2 are tile rows >= 128
      dma16(up ? p.rw1 : p.rw0, lb + (i * kThreads + p.wid * kWave) * 16, p.b_off[i] + kb);
    }
  } else {
    cr.codes = buf_load16(p.rw0, p.b_off[0], s < p.nk ? (uint32_t)s * BK / 2 : kOutOfRange);
    cr.sc = buf_load_u8(p.rsc, p.sc_off, s < p.nk ? (uint32_t)s * BK / 32 : kOutOfRange);
  }
}

// MXFP4: decode a step's block to bf16 and write it (swizzled) to lb.
__device__ __forceinline__ void pipe_put_codes(const Pipe& p, const CodeRegs& cr, uint8_t* __restrict__ lb) {
  uint4 d[4];
  mxfp4_block_to_bf16(cr.codes, cr.sc, d);
  const int r = p.tid / 2, blk = p.tid % 2;
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(lb + swz(r, blk * 4 + q)) = d[q];
}

__device__ __forceinline__ void pipe_compute(const Pipe& p, f32x16_t (&acc)[2][2], const uint8_t* __restrict__ la,
                                             const uint8_t* __restrict__ lb) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int c = kk * 2 + p.khalf;  // logical 16-byte piece of the row
    bf16x8_t fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(la + swz(p.arow0 + i * 32, c));
    fb[0] = *reinterpret_cast<const bf16x8_t*>(lb + swz(p.brow0, c));
    fb[1] = *reinterpret_cast<const bf16x8_t*>(lb + swz(p.brow1, c));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }
}

// The K loop over a ring of three LDS stages; the six stage buffers are
// distinct restrict pointers so the loads landing in one stage are known
// not to alias the reads of another.  Step s lives in stage s % 3 and its
// loads are issued during step s - 2.  Per step: wait for this thread's
// loads of step kt, barrier (all threads' loads landed; everyone finished
// step kt - 1, whose stage the next loads reuse), issue step kt + 2,
// compute step kt.
__device__ __forceinline__ void mainloop(const Pipe& p, f32x16_t (&acc)[2][2], uint8_t* __restrict__ a0,
                                         uint8_t* __restrict__ a1, uint8_t* __restrict__ a2,
                                         uint8_t* __restrict__ b0, uint8_t* __restrict__ b1,
                                         uint8_t* __restrict__ b2) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  // step s's MXFP4 block sits in code registers cr[s % 3] until converted
  CodeRegs cr0 = {}, cr1 = {}, cr2 = {};
  pipe_issue(p, 0, a0, b0, cr0);
  pipe_issue(p, 1, a1, b1, cr1);
  if (p.mx) {
    wait_vm<2>();  // step 0's block (step 1's code and scale loads may remain)
    pipe_put_codes(p, cr0, b0);
  }
  // loads per thread per step: 6 (bf16) or 4 (MXFP4: 2 DMA + codes + scale)
#define MOE_STEP(KT, LA, LB, LA2, LB2, LB1, CRN, CRP) \
  {                                                   \
    if (p.mx)                                         \
      wait_vm<4>();                                   \
    else                                              \
      wait_vm<6>();                                   \
    lds_barrier();                                    \
    pipe_issue(p, (KT) + 2, LA2, LB2, CRN);           \
    pipe_compute(p, acc, LA, LB);                     \
    if (p.mx) {                                       \
      wait_vm<4>();                                   \
      pipe_put_codes(p, CRP, LB1);                    \
    }                                                 \
  }
  for (int kt = 0; kt < p.nk; kt += 3) {
    MOE_STEP(kt, a0, b0, a2, b2, b1, cr2, cr1)
    if (kt + 1 < p.nk) MOE_STEP(kt + 1, a1, b1, a0, b0, b2, cr0, cr2)
    if (kt + 2 < p.nk) MOE_STEP(kt + 2, a2, b2, a1, b1, b0, cr1, cr0)
  }
#undef MOE_STEP
  wait_vm<0>();
}

template <int MODE, bool MX>
__global__ __launch_bounds__(kThreads, 1) void k_grouped_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[BM * 128], lds_a1[BM * 128], lds_a2[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b0[BN * 128], lds_b1[BN * 128], lds_b2[BN * 128];

  // XCD-aware order: the hardware deals workgroups round-robin over 8 XCDs;
  // give each XCD a contiguous run of (column tile, row tiles) so the row
  // tiles sharing one weight tile meet in the same L2.  The grid is sized
  // for the worst-case number of row tiles; the real tiles (counted from the
  // segment offsets) are dealt evenly over the XCDs, so none of them ends
  // up with most of the empty slots.
  const int nseg = a.E + a.shared;
  int p0, seg, rows, nt, mt;
  if (MODE == MODE_ROUTER) {
    const int per_xcd = gridDim.x / 8;
    const int lin = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    nt = lin / a.m_tiles_max;
    mt = lin % a.m_tiles_max;
    seg = 0;
    p0 = mt * BM;
    rows = min(BM, a.T - p0);
    if (rows <= 0) return;
  } else {
    const int total_m = __builtin_amdgcn_readfirstlane(count_row_tiles(a.offsets, nseg));
    const int total = total_m * a.n_tiles;
    const int per_xcd = (total + 7) / 8;
    const int slot = blockIdx.x / 8;
    const int lin = (blockIdx.x % 8) * per_xcd + slot;
    if (slot >= per_xcd || lin >= total) return;
    nt = lin / total_m;
    mt = lin % total_m;
    seg = tile_lookup(a.offsets, nseg, mt, &p0);
    // the lookup is wave-uniform: keep it in scalar registers so buffer
    // descriptors built from it stay scalar
    seg = __builtin_amdgcn_readfirstlane(seg);
    p0 = __builtin_amdgcn_readfirstlane(p0);
    if (seg < 0) return;
    rows = min(BM, __builtin_amdgcn_readfirstlane(a.offsets[seg + 1]) - p0);
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
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wid >> 2, wn = wid & 3;

  // ---- staging sources.  Piece q = tid + i*512 of a step lands at LDS
  // byte 16 q = row q/8, slot q%8; it must hold the logical piece whose
  // swizzled slot that is (the XOR is its own inverse).  Rows past the
  // tile's end read zeros.
  __amdgpu_buffer_rsrc_t ra;
  uint32_t a_off[kAChunks];
  {
    const uint16_t* abase;
    uint32_t abytes;
    if (MODE == MODE_DOWN) {
      abase = sh ? a.a_src + (size_t)nas * a.F + (size_t)(p0 - nas) * a.Fs : a.a_src + (size_t)p0 * a.F;
      abytes = (uint32_t)((size_t)rows * K * 2);
    } else {
      abase = a.a_src;
      abytes = (uint32_t)((size_t)a.T * a.H * 2);
    }
    ra = make_rsrc(abase, abytes);
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / 8;
      uint32_t off = kOutOfRange;
      if (r < rows) {
        if (MODE == MODE_ROUTER) {
          off = (uint32_t)((size_t)(p0 + r) * a.H * 2);
        } else if (MODE == MODE_GATEUP) {
          const int asg = a.sorted_assign[p0 + r];
          const int t = asg < nas ? asg / a.k : (int)(asg - nas);
          off = (uint32_t)((size_t)t * a.H * 2);
        } else {
          off = (uint32_t)((size_t)r * K * 2);
        }
        off += swz_slot(r, q % 8) << 4;
      }
      a_off[i] = off;
    }
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
  // weights: rw0 = the segment's first matrix (gate / fused gate_up / down /
  // router), rw1 = its up matrix (separate SwiGLU layout)
  __amdgpu_buffer_rsrc_t rw0, rw1, rsc;
  uint32_t b_off[kBChunks];
  uint32_t sc_off = 0;
  {
    const uint8_t *w0, *w1 = nullptr;
    size_t wbytes;
    const size_t pack = mx ? 4 : 1;  // MXFP4 holds 4 bits per element instead of 16
    if (MODE == MODE_ROUTER) {
      w0 = (const uint8_t*)a.w0;
      wbytes = (size_t)a.E * a.H * 2;
    } else if (MODE == MODE_GATEUP) {
      if (sh) {
        w0 = (const uint8_t*)a.sh0;
        w1 = (const uint8_t*)a.sh1;
        wbytes = (size_t)a.Fs * a.H * 2;
      } else if (a.oai) {
        wbytes = (size_t)2 * a.F * a.H * 2 / pack;
        w0 = (const uint8_t*)a.w0 + (size_t)seg * wbytes;
      } else {
        wbytes = (size_t)a.F * a.H * 2;
        w0 = (const uint8_t*)a.w0 + (size_t)seg * wbytes;
        w1 = (const uint8_t*)a.w1 + (size_t)seg * wbytes;
      }
    } else {
      if (sh) {
        w0 = (const uint8_t*)a.sh0;
        wbytes = (size_t)a.H * a.Fs * 2;
      } else {
        wbytes = (size_t)a.H * a.F * 2 / pack;
        w0 = (const uint8_t*)a.w0 + (size_t)seg * wbytes;
      }
    }
    rw0 = make_rsrc(w0, (uint32_t)wbytes);
    rw1 = make_rsrc(w1 ? w1 : w0, (uint32_t)wbytes);
    rsc = rw0;
    if (!mx) {
#pragma unroll
      for (int i = 0; i < kBChunks; ++i) {
        const int q = tid + i * kThreads;
        const int r = q / 8;
        b_off[i] = (uint32_t)((size_t)wrow(r) * K * 2) + (swz_slot(r, q % 8) << 4);
      }
    } else {
      // one 32-element block per thread per step: tile row tid/2, block tid%2
      const size_t row = wrow(tid / 2);
      b_off[0] = (uint32_t)(row * (K / 2)) + (tid % 2) * 16;
      const size_t srow0 = MODE == MODE_GATEUP ? (size_t)seg * 2 * a.F : (size_t)seg * a.H;
      const size_t nrows = MODE == MODE_GATEUP ? (size_t)2 * a.F : (size_t)a.H;
      rsc = make_rsrc(a.scales + srow0 * (K / 32), (uint32_t)(nrows * (K / 32)));
      sc_off = (uint32_t)(row * (K / 32)) + (tid % 2);
    }
  }
  // SwiGLU with separate gate and up matrices: B rows >= BN/2 read the up matrix
  const bool two_mats = MODE == MODE_GATEUP && (sh || !a.oai);
  const int nk = K / BK;

  const int arow0 = wm * 64 + (lane & 31);
  int brow[2];
  if (MODE == MODE_GATEUP) {
    brow[0] = wn * 32 + (lane & 31);           // gate rows
    brow[1] = BN / 2 + wn * 32 + (lane & 31);  // matching up rows
  } else {
    brow[0] = wn * 64 + (lane & 31);
    brow[1] = wn * 64 + 32 + (lane & 31);
  }
  Pipe p;
  p.ra = ra; p.rw0 = rw0; p.rw1 = rw1; p.rsc = rsc;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) p.a_off[i] = a_off[i];
#pragma unroll
  for (int i = 0; i < kBChunks; ++i) p.b_off[i] = b_off[i];
  p.sc_off = sc_off;
  p.two_mats = two_mats;
  p.mx = mx;
  p.nk = nk;
  p.wid = wid;
  p.tid = tid;
  p.arow0 = arow0;
  p.brow0 = brow[0];
  p.brow1 = brow[1];
  p.khalf = lane >> 5;
  f32x16_t acc[2][2];
  mainloop(p, acc, lds_a0, lds_a1, lds_a2, lds_b0, lds_b1, lds_b2);

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
    float* lg = (float*)a.out;
    uint16_t* y = (uint16_t*)a.out;
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
              if (MODE == MODE_ROUTER)
                lg[(size_t)(p0 + r) * ncols + o] = acc[i][j][q] + bias;
              else
                y[(size_t)a.sorted_assign[p0 + r] * ncols + o] = (uint16_t)f32_to_bf16(acc[i][j][q] + bias);
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
                            const int32_t* sorted_assign, int32_t T, uint16_t* y, hipStream_t s) {
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
