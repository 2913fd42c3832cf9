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
// v_mfma_f32_32x32x16_bf16 blocks.  The MFMAs take the weight rows as their
// first operand and the activation rows as their second, so a lane ends with
// one activation row and runs of four consecutive outputs of it, which the
// epilogue writes as 8-byte (bf16) or 16-byte (fp32) pieces.
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
  int32_t n_tiles;           // column tiles per segment (max over segments); router: times ksplit
  int32_t ksplit;            // router: K split into ksplit ranges of split_steps steps (1: no split)
  int32_t split_steps;
  int32_t col_tiles;         // router: column tiles of one K range
  float* part;               // router with ksplit > 1: partial logits [ksplit][T][E]
  int32_t m_tiles_max;       // grid bound on row tiles
  float alpha, limit;
  const uint8_t* a8;         // MXFP8 path: E4M3 activation codes [rows][K]
  const uint8_t* a8s;        // and their E8M0 scales [rows][a8s_stride]
  int32_t a8s_stride;
};


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

// One output tile: row tile of a segment (or of the tokens, router) by a
// column tile.
struct Tile {
  int seg, p0, rows, c0, Fe, ncols, K;
  int ks, k0, nk;  // K range (router split-K): index, first step, steps
  bool sh;
};

// Per-thread state of the K pipeline of one tile.
struct Pipe {
  __amdgpu_buffer_rsrc_t ra, rw0, rw1, rsc;
  uint32_t a_off[kAChunks], b_off[kBChunks], sc_off;
  bool a_ok[kAChunks];      // gate/up: the staged row is a row of the tile
  int32_t* ids;             // the tile's assignment ids in LDS (gate/up, down)
  uint32_t* bias;           // the tile's bias words in LDS (gate/up, down)
  int k0;                   // first K step of the tile
  bool two_mats, mx;
  int nk;
};

// Issue the loads of step s into stage (la, lb) (all lanes, always: a step
// past the end reads at an out-of-range offset, i.e. zeros, so every step
// has the same number of outstanding loads).
__device__ __forceinline__ void pipe_issue(const Pipe& p, int s, int wid, uint8_t* __restrict__ la,
                                           uint8_t* __restrict__ lb, CodeRegs& cr) {
  const uint32_t kb = s < p.nk ? (uint32_t)(p.k0 + s) * BK * 2 : kOutOfRange;  // byte offset of the step in a bf16 row
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) dma16(p.ra, la + (i * kThreads + wid * kWave) * 16, p.a_off[i] + kb);
  if (!p.mx) {
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const bool up = p.two_mats && i >= kBChunks / 2;  // pieces i >= 2 are tile rows >= 128
      dma16(up ? p.rw1 : p.rw0, lb + (i * kThreads + wid * kWave) * 16, p.b_off[i] + kb);
    }
  } else {
    cr.codes = buf_load16(p.rw0, p.b_off[0], s < p.nk ? (uint32_t)(p.k0 + s) * BK / 2 : kOutOfRange);
    cr.sc = buf_load_u8(p.rsc, p.sc_off, s < p.nk ? (uint32_t)(p.k0 + s) * BK / 32 : kOutOfRange);
  }
}

// The pipe whose step s2 comes next: p while s2 < p.nk, else q (its step
// s2 - p.nk).  Every field is chosen with a select on a wave-uniform
// condition, so a single copy of the loads is emitted.
__device__ __forceinline__ Pipe pipe_pick(const Pipe& p, const Pipe& q, bool uq) {
  Pipe x;
  x.ra = uq ? q.ra : p.ra;
  x.rw0 = uq ? q.rw0 : p.rw0;
  x.rw1 = uq ? q.rw1 : p.rw1;
  x.rsc = uq ? q.rsc : p.rsc;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) x.a_off[i] = uq ? q.a_off[i] : p.a_off[i];
#pragma unroll
  for (int i = 0; i < kBChunks; ++i) x.b_off[i] = uq ? q.b_off[i] : p.b_off[i];
  x.sc_off = uq ? q.sc_off : p.sc_off;
  x.two_mats = uq ? q.two_mats : p.two_mats;
  x.mx = uq ? q.mx : p.mx;
  x.nk = uq ? q.nk : p.nk;
  x.k0 = uq ? q.k0 : p.k0;
  return x;
}

// Issue step s2 of the pair (p, q) all at once (MXFP4 kernels).
__device__ __forceinline__ void pipe_issue_pq(const Pipe& p, const Pipe& q, int s2, int wid, uint8_t* __restrict__ la,
                                              uint8_t* __restrict__ lb, CodeRegs& cr) {
  const bool uq = s2 >= p.nk;
  pipe_issue(pipe_pick(p, q, uq), uq ? s2 - p.nk : s2, wid, la, lb, cr);
}

// MXFP4 staging: thread t decodes 32-element block mx_blk(t) of tile row
// mx_row(t).  Each 16-lane quarter of a wave takes 16 rows, the even ones
// first: two rows r, r + 1 share a swizzle pattern, so taking them in
// different halves of the quarter makes the rows written by 8 consecutive
// lanes fall in 8 different swizzle classes and their 16-byte stores hit
// distinct banks (two lanes per row made every store a 2-way bank conflict).
__device__ __forceinline__ int mx_row(int t) {
  const int lane = t & (kWave - 1), l = lane & 15;
  return (t / kWave) * 32 + ((lane >> 5) << 4) + (l < 8 ? 2 * l : 2 * (l - 8) + 1);
}
__device__ __forceinline__ int mx_blk(int t) { return (t >> 4) & 1; }

// MXFP4: decode a step's block to bf16 and write it (swizzled) to lb.
__device__ __forceinline__ void pipe_put_codes(const CodeRegs& cr, uint8_t* __restrict__ lb) {
  uint4 d[4];
  mxfp4_block_to_bf16(cr.codes, cr.sc, d);
  const int r = mx_row(threadIdx.x), blk = mx_blk(threadIdx.x);
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(lb + swz(r, blk * 4 + q)) = d[q];
}

// Fragment rows of this thread: A rows arow0 (+32), B rows brow0 / brow1;
// khalf = which 8-element half of each 16-element K slice the lane holds.
struct Frag {
  int arow0, brow0, brow1, khalf;
};

// Operand reads from LDS go through inline asm: the compiler then does not
// see LDS reads that might alias the buffer->LDS loads in flight (which
// target other stages) and adds no wait for those loads; lds_wait ties the
// fragment registers to the wait for the reads themselves, so no MFMA can
// use them earlier.
__device__ __forceinline__ bf16x8_t ds_read16(const uint8_t* p) {
  bf16x8_t r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"((uint32_t)(uintptr_t)p) : "memory");
  return r;
}
// 4-byte LDS read through inline asm, completed by the s_waitcnt inside.
__device__ __forceinline__ int32_t ds_read4_sync(const int32_t* p) {
  int32_t r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"((uint32_t)(uintptr_t)p) : "memory");
  return r;
}
// Wait for every vector memory operation of the wave, as an s_waitcnt the
// compiler's own wait placement knows about (bias words loaded in uniform
// control flow are then complete before the per-row branches that use them,
// and are not taken as pending where the tile loop comes round again).
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// Epilogue staging through LDS (inline asm, like the operand reads): an
// 8-byte write, and a 16-byte read whose wait is tied to its registers.
__device__ __forceinline__ void ds_write8(uint32_t addr, uint32_t lo, uint32_t hi) {
  const uint64_t v = (uint64_t)hi << 32 | lo;
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ u32x4_t ds_read16u(uint32_t addr) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
  return r;
}
__device__ __forceinline__ void lds_wait4(u32x4_t (&v)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t ds_read8u(uint32_t addr) {
  u32x2_t r;
  asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(addr) : "memory");
  return r;
}
__device__ __forceinline__ void lds_wait8(u32x2_t (&v)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}
__device__ __forceinline__ int32_t ds_read4(const int32_t* p) {
  int32_t r;
  asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"((uint32_t)(uintptr_t)p) : "memory");
  return r;
}

struct KFrag {
  bf16x8_t a[2], b[2];
};
__device__ __forceinline__ void read_kfrag(const Frag& f, int kk, const uint8_t* la, const uint8_t* lb, KFrag& o) {
  const int c = kk * 2 + f.khalf;  // logical 16-byte piece of the row
  o.a[0] = ds_read16(la + swz(f.arow0, c));
  o.a[1] = ds_read16(la + swz(f.arow0 + 32, c));
  o.b[0] = ds_read16(lb + swz(f.brow0, c));
  o.b[1] = ds_read16(lb + swz(f.brow1, c));
}
template <int N> __device__ __forceinline__ void lds_wait(KFrag& o) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(o.a[0]), "+v"(o.a[1]), "+v"(o.b[0]), "+v"(o.b[1]) : "n"(N));
}
__device__ __forceinline__ void mfma4(f32x16_t (&acc)[2][2], const KFrag& o) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.b[j], o.a[i], acc[i][j], 0, 0, 0);
}

// One K step: four 16-deep sub-steps, the operand reads of sub-step kk + 1
// in flight during the MFMAs of kk.
__device__ __forceinline__ void pipe_compute(const Frag& f, f32x16_t (&acc)[2][2], const uint8_t* la,
                                             const uint8_t* lb) {
  KFrag k0, k1, k2, k3;
  read_kfrag(f, 0, la, lb, k0);
  read_kfrag(f, 1, la, lb, k1);
  lds_wait<4>(k0);
  read_kfrag(f, 2, la, lb, k2);
  mfma4(acc, k0);
  lds_wait<4>(k1);
  read_kfrag(f, 3, la, lb, k3);
  mfma4(acc, k1);
  lds_wait<4>(k2);
  mfma4(acc, k2);
  lds_wait<0>(k3);
  mfma4(acc, k3);
}

__device__ __forceinline__ void mfma1(f32x16_t (&acc)[2][2], const KFrag& o, int i, int j) {
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.b[j], o.a[i], acc[i][j], 0, 0, 0);
}

// The same K step for bf16 weights, with the six buffer->LDS loads of step s
// of pipe x (into stage la2 / lb2) issued one at a time between the MFMAs of
// the first two sub-steps.  Issued as a burst at the step's start, a load
// that waits for room in the address queue holds the wave before its first
// MFMA; spread out, the MFMAs already issued keep the matrix pipe busy
// meanwhile (7-9% faster grouped GEMMs).  The next step's wait and barrier
// come before this step's last sub-step: kn holds this step's sub-step-0
// fragments (read after the previous barrier) and, when `next`, receives the
// next step's (from stage nla / nlb) right after the barrier, so they arrive
// while this step's last four MFMAs run instead of after the next barrier
// (gpt-oss bf16 layer 3% faster).  The barrier still comes after every
// operand read of this step's stage, which the loads it lets go reuse.  The
// scheduling barriers keep this order.
__device__ __forceinline__ void pipe_compute_issue(const Frag& f, f32x16_t (&acc)[2][2], const uint8_t* la,
                                                      const uint8_t* lb, const Pipe& x, int s, int wid,
                                                      uint8_t* __restrict__ la2, uint8_t* __restrict__ lb2,
                                                      KFrag& kn, bool next, const uint8_t* nla,
                                                      const uint8_t* nlb) {
  const uint32_t kb = s < x.nk ? (uint32_t)(x.k0 + s) * BK * 2 : kOutOfRange;
  auto ld_a = [&](int i) { dma16(x.ra, la2 + (i * kThreads + wid * kWave) * 16, x.a_off[i] + kb); };
  auto ld_b = [&](int i) {
    const bool up = x.two_mats && i >= kBChunks / 2;
    dma16(up ? x.rw1 : x.rw0, lb2 + (i * kThreads + wid * kWave) * 16, x.b_off[i] + kb);
  };
  KFrag k1, k2, k3;
  read_kfrag(f, 1, la, lb, k1);
  lds_wait<4>(kn);
  read_kfrag(f, 2, la, lb, k2);
  __builtin_amdgcn_sched_barrier(0);
  mfma1(acc, kn, 0, 0); __builtin_amdgcn_sched_barrier(0); ld_a(0); __builtin_amdgcn_sched_barrier(0);
  mfma1(acc, kn, 0, 1); __builtin_amdgcn_sched_barrier(0); ld_a(1); __builtin_amdgcn_sched_barrier(0);
  mfma1(acc, kn, 1, 0); __builtin_amdgcn_sched_barrier(0); ld_b(0); __builtin_amdgcn_sched_barrier(0);
  mfma1(acc, kn, 1, 1); __builtin_amdgcn_sched_barrier(0);
  lds_wait<4>(k1);
  read_kfrag(f, 3, la, lb, k3);
  __builtin_amdgcn_sched_barrier(0);
  mfma1(acc, k1, 0, 0); __builtin_amdgcn_sched_barrier(0); ld_b(1); __builtin_amdgcn_sched_barrier(0);
  mfma1(acc, k1, 0, 1); __builtin_amdgcn_sched_barrier(0); ld_b(2); __builtin_amdgcn_sched_barrier(0);
  mfma1(acc, k1, 1, 0); __builtin_amdgcn_sched_barrier(0); ld_b(3); __builtin_amdgcn_sched_barrier(0);
  mfma1(acc, k1, 1, 1); __builtin_amdgcn_sched_barrier(0);
  lds_wait<4>(k2);
  __builtin_amdgcn_sched_barrier(0);
  mfma4(acc, k2);
  __builtin_amdgcn_sched_barrier(0);
  lds_wait<0>(k3);
  if (next) {
    wait_vm<6>();
    lds_barrier();
    read_kfrag(f, 0, nla, nlb, kn);
  }
  __builtin_amdgcn_sched_barrier(0);
  mfma4(acc, k3);
  __builtin_amdgcn_sched_barrier(0);
}

// Segment tables in LDS: offsets[0..nseg] and the exclusive prefix of the
// BM-row tiles per segment (tpre[nseg] = all row tiles).
struct SegTables {
  int off[kMaxExperts + 2];
  int tpre[kMaxExperts + 2];
  int wsum[kThreads / kWave];
};

__device__ __forceinline__ int row_tiles(int n) { return (n + BM - 1) / BM; }

// Fill the tables from the offsets in HBM; returns the number of row tiles.
__device__ int build_tables(const int32_t* __restrict__ offsets, int nseg, SegTables& t) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  for (int e = tid; e <= nseg; e += kThreads) t.off[e] = offsets[e];
  __syncthreads();
  const int per = (nseg + kThreads - 1) / kThreads;  // consecutive segments per thread
  int loc = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < nseg) loc += row_tiles(t.off[e + 1] - t.off[e]);
  }
  int incl = loc;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) t.wsum[wid] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    const int s = t.wsum[w];
    before += w < wid ? s : 0;
    all += s;
  }
  int run = before + incl - loc;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < nseg) {
      t.tpre[e] = run;
      run += row_tiles(t.off[e + 1] - t.off[e]);
    }
  }
  if (tid == 0) t.tpre[nseg] = all;
  __syncthreads();
  return all;
}

// Segment holding tile lin when each segment's tiles are contiguous in lin
// (scale = column tiles per row tile), searched from segment `from` on (a
// workgroup's tiles only move forward, so the previous tile's segment is a
// lower bound): 64 segments per LDS read, no per-lane branches.
__device__ int find_segment(const SegTables& t, int nseg, int lin, int scale, int from) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int base = from; base < nseg; base += kWave) {
    const int e = min(base + lane, nseg - 1);
    const int lo = t.tpre[e] * scale, hi = t.tpre[e + 1] * scale;
    const uint64_t m = __ballot((base + lane < nseg) & (lo <= lin) & (lin < hi));
    if (m) return base + __ffsll((unsigned long long)m) - 1;
  }
  return -1;
}

// Tile lin of the (column tile, row tile) space; false if its column tile
// lies past the segment's columns (shared expert narrower than the routed).
// Expert GEMMs: the tiles of one segment are contiguous in lin, column-tile
// major inside it (nt, then row tile), so the row tiles sharing a weight
// tile run side by side and a small segment's column tiles, which share its
// gathered activation rows, follow each other (same XCD, same L2).
// Router: column tiles (and K ranges) outermost.
template <int MODE>
__device__ bool tile_at(const GemmArgs& a, const SegTables& st, int lin, int total_m, Tile& t, int from) {
  int nt = lin / total_m;
  const int mt = lin % total_m;  // router row tile
  const int nseg = a.E + a.shared;
  t.ks = 0;
  if (MODE == MODE_ROUTER) {
    t.ks = nt / a.col_tiles;
    nt = nt % a.col_tiles;
    t.seg = 0;
    t.p0 = mt * BM;
    t.rows = min(BM, a.T - t.p0);
  } else {
    const int seg = __builtin_amdgcn_readfirstlane(find_segment(st, nseg, lin, a.n_tiles, from));
    const int r0 = __builtin_amdgcn_readfirstlane(st.tpre[seg]);
    const int nr = __builtin_amdgcn_readfirstlane(st.tpre[seg + 1]) - r0;  // row tiles of the segment
    const int local = lin - r0 * a.n_tiles;
    nt = local / nr;
    t.seg = seg;
    t.p0 = __builtin_amdgcn_readfirstlane(st.off[seg]) + (local % nr) * BM;
    t.rows = min(BM, __builtin_amdgcn_readfirstlane(st.off[seg + 1]) - t.p0);
  }
  t.sh = MODE != MODE_ROUTER && t.seg == a.E;
  t.Fe = t.sh ? a.Fs : a.F;
  t.ncols = MODE == MODE_GATEUP ? t.Fe : MODE == MODE_DOWN ? a.H : a.E;
  const int col_tile = MODE == MODE_GATEUP ? BN / 2 : BN;  // features | outputs per tile
  t.c0 = nt * col_tile;
  t.K = MODE == MODE_DOWN ? t.Fe : a.H;
  t.k0 = t.ks * a.split_steps;
  t.nk = min(t.K / BK - t.k0, a.split_steps);
  return t.c0 < t.ncols;
}

// Buffer descriptors and per-thread source offsets of a tile.  Piece
// q = tid + i*512 of a step lands at LDS byte 16 q = row q/8, slot q%8; it
// must hold the logical piece whose swizzled slot that is (the XOR is its
// own inverse).  Rows past the tile's end read zeros.  Gate/up A rows are
// gathered by token: the assignment ids are loaded here and turned into
// offsets by finish_pipe, so the loads can be in flight meanwhile.
template <int MODE, bool MX>
__device__ void make_pipe(const GemmArgs& a, const Tile& t, int32_t* ids, uint32_t* bias, Pipe& p) {
  const int tid = threadIdx.x;
  const int64_t nas = (int64_t)a.T * a.k;
  const bool mx = MX && !t.sh && MODE != MODE_ROUTER;
  {
    const uint16_t* abase;
    uint32_t abytes;
    if (MODE == MODE_DOWN) {
      abase = t.sh ? a.a_src + (size_t)nas * a.F + (size_t)(t.p0 - nas) * a.Fs : a.a_src + (size_t)t.p0 * a.F;
      abytes = (uint32_t)((size_t)t.rows * t.K * 2);
    } else {
      abase = a.a_src;
      abytes = (uint32_t)((size_t)a.T * a.H * 2);
    }
    p.ra = make_rsrc(abase, abytes);
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / 8;
      uint32_t off = kOutOfRange;
      p.a_ok[i] = r < t.rows;
      if (MODE != MODE_GATEUP && r < t.rows) {
        if (MODE == MODE_ROUTER)
          off = (uint32_t)((size_t)(t.p0 + r) * a.H * 2) + (swz_slot(r, q % 8) << 4);
        else
          off = (uint32_t)((size_t)r * t.K * 2) + (swz_slot(r, q % 8) << 4);
      }
      p.a_off[i] = off;
    }
  }
  // The assignment ids of the tile's rows (gate/up: which token each row
  // gathers; down: which y row each row writes) go to LDS through
  // buffer->LDS loads of waves 0 and 1, and the tile's 512 bias bytes
  // (gate/up: a gate | up word per feature; down: the 256 outputs) through
  // those of waves 2 and 3 — columns past the matrix, a shared-expert tile
  // or a layer without biases read zeros — so the epilogue has no global
  // load to wait for (such a wait would also wait for the next tile's first
  // loads).  The K loop's waits and barriers cover both before finish_pipe
  // and the epilogue read them.
  p.ids = ids;
  p.bias = bias;
  // (branches on the wave index, so each load's descriptor is wave-uniform
  // in scalar registers)
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  if (MODE != MODE_ROUTER && wv < BM / kWave) {
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(a.sorted_assign + t.p0, (uint32_t)t.rows * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ri, (lds_ptr_t)(ids + (tid & ~(kWave - 1))), 4, (int)(tid * 4), 0, 0, 0);
  } else if (MODE != MODE_ROUTER && wv < 2 * BM / kWave && a.bias) {
    const bool hb = !t.sh && (MODE == MODE_DOWN || a.oai);
    const size_t e0 = MODE == MODE_GATEUP ? (size_t)t.seg * 2 * a.F + 2 * t.c0 : (size_t)t.seg * a.H + t.c0;
    const int n = MODE == MODE_GATEUP ? 2 * (a.F - t.c0) : a.H - t.c0;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(hb ? a.bias + e0 : a.bias, hb ? (uint32_t)n * 2 : 0u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(bias + ((tid - BM) & ~(kWave - 1))), 4,
                                             (int)((tid - BM) * 4), 0, 0, 0);
  }
  auto wrow = [&](int r) -> int {  // row of the segment's weight matrix for tile row r
    if (MODE == MODE_GATEUP) {
      const int f = min(t.c0 + (r & (BN / 2 - 1)), t.Fe - 1);
      if (a.oai && !t.sh) return 2 * f + (r >= BN / 2);
      return f;  // gate (r < BN/2) or up (r >= BN/2) matrix row f
    }
    if (MODE == MODE_ROUTER) return min(t.c0 + r, a.E - 1);
    return min(t.c0 + r, a.H - 1);
  };
  // weights: rw0 = the segment's first matrix (gate / fused gate_up / down /
  // router), rw1 = its up matrix (separate SwiGLU layout)
  const uint8_t *w0, *w1 = nullptr;
  size_t wbytes;
  const size_t pack = mx ? 4 : 1;  // MXFP4 holds 4 bits per element instead of 16
  if (MODE == MODE_ROUTER) {
    w0 = (const uint8_t*)a.w0;
    wbytes = (size_t)a.E * a.H * 2;
  } else if (MODE == MODE_GATEUP) {
    if (t.sh) {
      w0 = (const uint8_t*)a.sh0;
      w1 = (const uint8_t*)a.sh1;
      wbytes = (size_t)a.Fs * a.H * 2;
    } else if (a.oai) {
      wbytes = (size_t)2 * a.F * a.H * 2 / pack;
      w0 = (const uint8_t*)a.w0 + (size_t)t.seg * wbytes;
    } else {
      wbytes = (size_t)a.F * a.H * 2;
      w0 = (const uint8_t*)a.w0 + (size_t)t.seg * wbytes;
      w1 = (const uint8_t*)a.w1 + (size_t)t.seg * wbytes;
    }
  } else {
    if (t.sh) {
      w0 = (const uint8_t*)a.sh0;
      wbytes = (size_t)a.H * a.Fs * 2;
    } else {
      wbytes = (size_t)a.H * a.F * 2 / pack;
      w0 = (const uint8_t*)a.w0 + (size_t)t.seg * wbytes;
    }
  }
  p.rw0 = make_rsrc(w0, (uint32_t)wbytes);
  p.rw1 = make_rsrc(w1 ? w1 : w0, (uint32_t)wbytes);
  p.rsc = p.rw0;
  p.sc_off = 0;
  if (!mx) {
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / 8;
      p.b_off[i] = (uint32_t)((size_t)wrow(r) * t.K * 2) + (swz_slot(r, q % 8) << 4);
    }
  } else {
    // one 32-element block per thread per step: tile row mx_row(tid), block mx_blk(tid)
    const size_t row = wrow(mx_row(tid));
    p.b_off[0] = (uint32_t)(row * (t.K / 2)) + mx_blk(tid) * 16;
#pragma unroll
    for (int i = 1; i < kBChunks; ++i) p.b_off[i] = 0;
    const size_t srow0 = MODE == MODE_GATEUP ? (size_t)t.seg * 2 * a.F : (size_t)t.seg * a.H;
    const size_t nrows = MODE == MODE_GATEUP ? (size_t)2 * a.F : (size_t)a.H;
    p.rsc = make_rsrc(a.scales + srow0 * (t.K / 32), (uint32_t)(nrows * (t.K / 32)));
    p.sc_off = (uint32_t)(row * (t.K / 32)) + mx_blk(tid);
  }
  // SwiGLU with separate gate and up matrices: B rows >= BN/2 read the up matrix
  p.two_mats = MODE == MODE_GATEUP && (t.sh || !a.oai);
  p.mx = mx;
  p.nk = t.nk;
  p.k0 = t.k0;
}

// Gate/up: token row offsets from the assignment ids that make_pipe sent to
// LDS (the caller has waited for those loads and passed a barrier).
template <int MODE>
__device__ __forceinline__ void finish_pipe(const GemmArgs& a, Pipe& p) {
  if (MODE != MODE_GATEUP) return;
  const int64_t nas = (int64_t)a.T * a.k;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int q = threadIdx.x + i * kThreads;
    const int asg = ds_read4_sync(p.ids + q / 8);
    if (p.a_ok[i]) {
      const int t = asg < nas ? asg / a.k : (int)(asg - nas);
      p.a_off[i] = (uint32_t)((size_t)t * a.H * 2) + (swz_slot(q / 8, q % 8) << 4);
    }
  }
}

// Field by field (a whole-struct copy left never-read slices of the
// structs in scratch memory, whose copies waited for every load in flight).
__device__ __forceinline__ void pipe_copy(Pipe& d, const Pipe& s) {
  d.ra = s.ra;
  d.rw0 = s.rw0;
  d.rw1 = s.rw1;
  d.rsc = s.rsc;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    d.a_off[i] = s.a_off[i];
    d.a_ok[i] = s.a_ok[i];
  }
#pragma unroll
  for (int i = 0; i < kBChunks; ++i) d.b_off[i] = s.b_off[i];
  d.sc_off = s.sc_off;
  d.ids = s.ids;
  d.bias = s.bias;
  d.k0 = s.k0;
  d.two_mats = s.two_mats;
  d.mx = s.mx;
  d.nk = s.nk;
}

// A pipe with no steps: its loads all read zeros.
__device__ __forceinline__ void null_pipe(const Pipe& like, Pipe& p) {
  pipe_copy(p, like);
  p.nk = 0;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    p.a_ok[i] = false;
    p.a_off[i] = kOutOfRange;
  }
}

// The K loop of one tile over a ring of three LDS stages; the six stage
// buffers are distinct restrict pointers so the loads landing in one stage
// are known not to alias the reads of another.  Step s of the tile lives in
// stage s % 3 of (a0, a1, a2) and its loads were issued during step s - 2;
// the steps 0 and 1 were issued before the call (by the previous tile's
// loop or the prologue), and the last two steps issue steps 0 and 1 of the
// next tile q, so the ring runs on across tiles.  Per step: wait for this
// thread's loads of step kt, barrier (all threads' loads landed; everyone
// finished step kt - 1, whose stage the next loads reuse), issue step
// kt + 2, compute step kt.  With bf16 weights the wait and barrier of step
// kt + 1 sit in front of step kt's last sub-step (those of the tile's first
// step here, before the loop), and the epilogue has its own barrier.
template <int MODE, bool MX>
__device__ __forceinline__ void tile_loop(const GemmArgs& a, const Pipe& p, Pipe& q, const Frag& fr, int wid,
                                          f32x16_t (&acc)[2][2], CodeRegs& c0, CodeRegs& c1, CodeRegs& c2,
                                          uint8_t* __restrict__ a0,
                                          uint8_t* __restrict__ a1, uint8_t* __restrict__ a2,
                                          uint8_t* __restrict__ b0, uint8_t* __restrict__ b1,
                                          uint8_t* __restrict__ b2) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // Loads per thread per step: 6 (bf16) or 4 (MXFP4: 2 DMA + codes + scale).
  // A step's loads are complete once at most the next step's are in
  // flight; kernels with MXFP4 experts wait down to 4, which also covers a
  // bf16 step (the shared expert's) on either side.  An MXFP4 step's block
  // is decoded into its stage during the step before it, from the codes
  // loaded two steps before that (the next tile's first block during this
  // tile's last step).  Steps 0 and 1 of the next tile q are issued by the
  // last two steps; q's ids went out before this tile's step 2 loads, so
  // with three or more steps (persistent launches) the wait and barrier of
  // step nk - 2 covered them, and otherwise q is the empty pipe.  The issue
  // picks p's or q's fields with selects, not branches, so the code
  // registers are written by a single load.
#define MOE_STEP(KT, LA, LB, LA2, LB2, LA1, LB1, CRN, CRP)              \
  {                                                                     \
    if (MX) {                                                           \
      wait_vm<4>();                                                     \
      lds_barrier();                                                    \
    }                                                                   \
    const int s2 = (KT) + 2;                                            \
    if (s2 == p.nk) finish_pipe<MODE>(a, q);                            \
    if (MX) {                                                           \
      pipe_issue_pq(p, q, s2, wid, LA2, LB2, CRN);                      \
      pipe_compute(fr, acc, LA, LB);                                    \
    } else {                                                            \
      const bool uq = s2 >= p.nk;                                       \
      pipe_compute_issue(fr, acc, LA, LB, pipe_pick(p, q, uq), uq ? s2 - p.nk : s2, wid, LA2, LB2, kn, \
                         (KT) + 1 < p.nk, LA1, LB1);                    \
    }                                                                   \
    if (MX && ((KT) + 1 < p.nk ? p.mx : q.mx)) {                        \
      wait_vm<4>();                                                     \
      pipe_put_codes(CRP, LB1);                                         \
    }                                                                   \
  }
  KFrag kn;  // sub-step 0 fragments of the step about to run (bf16 weights)
  if (!MX) {
    wait_vm<6>();
    lds_barrier();
    read_kfrag(fr, 0, a0, b0, kn);
  }
  for (int kt = 0; kt < p.nk; kt += 3) {
    MOE_STEP(kt, a0, b0, a2, b2, a1, b1, c2, c1)
    if (kt + 1 < p.nk) MOE_STEP(kt + 1, a1, b1, a0, b0, a2, b2, c0, c2)
    if (kt + 2 < p.nk) MOE_STEP(kt + 2, a2, b2, a1, b1, a0, b0, c1, c0)
  }
  // (a tile has at least one step, whose reads complete kn; this wait only
  // spells that out for the compiler, whose register reuse sees no load)
  if (!MX) lds_wait<0>(kn);
#undef MOE_STEP
}

// Epilogue.  acc[i][j] is the product of weight block j (first MFMA
// operand) and activation block i (second): lane l holds activation row
// i * 32 + (l & 31) of the wave's 64 and weight rows
// (q / 4) * 8 + (l / 32) * 4 + (q % 4), q = 0..15, of block j; group
// g = q / 4 is a run of four consecutive outputs of that row.  BIAS: 0 none,
// 1 from LDS (the tile's, staged when the tile was set up), 2 from HBM, all
// of the lane's bias words requested at once from in-range addresses (a load
// under a branch would make the compiler wait for every load in flight
// where the branches meet, on the path without it too).
//
// STG (gate/up and down): the results go through the LDS stage that the
// tile's last K step read, idle until the next tile's step 2 loads refill it
// (behind the next tile's first barrier): after a barrier (every wave is
// done with that step's operand reads), each wave writes its block as bf16
// to its own 4 KiB there (`stage`: 16-byte pieces XOR-swizzled by row, so
// the 8-byte writes of a wave hit every bank equally), reads it back row-
// major and stores whole 64- (h) or 128-byte (y) row segments — a store
// instruction then covers 16 or 8 rows instead of 32 partial ones.
template <int MODE, int BIAS, bool STG>
__device__ __forceinline__ void epilogue_b(const GemmArgs& a, const Tile& t, const f32x16_t (&acc)[2][2], int wm,
                                           int wn, const int32_t* ids, const uint32_t* bias_lds, uint8_t* stage) {
  const int lane = threadIdx.x & (kWave - 1);
  const int rl = lane & 31, hq = lane >> 5;
  const int64_t nas = (int64_t)a.T * a.k;
  if (MODE == MODE_GATEUP) {
    // feature of group g, element e: fb + g * 8 + e; gate and up biases as
    // one word per feature (gate in the low half, up in the high half)
    const int fb = t.c0 + wn * 32 + hq * 4;
    const bool oai = a.oai && !t.sh;
    uint4 bw[4];
    if (BIAS == 1) {  // the four reads in flight together, one wait
      u32x4_t bq[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) bq[g] = ds_read16u((uint32_t)(uintptr_t)(bias_lds + wn * 32 + g * 8 + hq * 4));
      lds_wait4(bq);
#pragma unroll
      for (int g = 0; g < 4; ++g) bw[g] = make_uint4(bq[g].x, bq[g].y, bq[g].z, bq[g].w);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (BIAS == 2)
        bw[g] = *reinterpret_cast<const uint4*>(a.bias + (size_t)t.seg * 2 * a.F + 2 * min(fb + g * 8, t.Fe - 4));
      else if (BIAS == 0)
        bw[g] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (BIAS == 2) vm_wait_all();
    uint16_t* h = (uint16_t*)a.out;
    if (STG) {
      lds_barrier();
      if (t.c0 + wn * 32 >= t.Fe) return;  // the wave's 32 features lie past a narrower segment
      const uint32_t R = (uint32_t)(uintptr_t)stage;  // 64 rows x 64 bytes
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = i * 32 + rl;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t bb[4] = {bw[g].x, bw[g].y, bw[g].z, bw[g].w};
          float hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int q = g * 4 + e;
            float v;
            if (oai) {
              v = oai_act(acc[i][0][q] + bf16lo(bb[e]), acc[i][1][q] + bf16hi(bb[e]), a.alpha, a.limit);
            } else {
              v = swiglu_act(acc[i][0][q], acc[i][1][q]);
            }
            hv[e] = v;
          }
          ds_write8(R + r * 64 + ((g ^ ((r >> 1) & 3)) << 4) + hq * 8, pack_bf16(hv[0], hv[1]), pack_bf16(hv[2], hv[3]));
        }
      }
      u32x4_t v[4];
      const int c = lane & 3;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 16 + (lane >> 2);
        v[it] = ds_read16u(R + r * 64 + ((c ^ ((r >> 1) & 3)) << 4));
      }
      lds_wait4(v);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = wm * 64 + it * 16 + (lane >> 2);
        if (r < t.rows) {
          const int p = t.p0 + r;
          uint16_t* hrow = h + (p < nas ? (size_t)p * a.F : (size_t)nas * a.F + (size_t)(p - nas) * a.Fs);
          *reinterpret_cast<u32x4_t*>(hrow + t.c0 + wn * 32 + c * 8) = v[it];
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + rl;
      if (r < t.rows) {
        const int p = t.p0 + r;
        uint16_t* hrow = h + (p < nas ? (size_t)p * a.F : (size_t)nas * a.F + (size_t)(p - nas) * a.Fs);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = fb + g * 8;
          if (f < t.Fe) {
            const uint32_t bb[4] = {bw[g].x, bw[g].y, bw[g].z, bw[g].w};
            float hv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int q = g * 4 + e;
              float v;
              if (oai) {
                v = oai_act(acc[i][0][q] + bf16lo(bb[e]), acc[i][1][q] + bf16hi(bb[e]), a.alpha, a.limit);
              } else {
                v = swiglu_act(acc[i][0][q], acc[i][1][q]);
              }
              hv[e] = v;
            }
            *reinterpret_cast<uint2*>(hrow + f) = make_uint2(pack_bf16(hv[0], hv[1]), pack_bf16(hv[2], hv[3]));
          }
        }
      }
    }
  } else {
    // output column of (j, g, e): ob + j * 32 + g * 8 + e; router rows of a
    // width that is not a multiple of four are written element by element
    const int ob = t.c0 + wn * 64 + hq * 4;
    const bool split = MODE == MODE_ROUTER && a.ksplit > 1;  // partial sums: no bias
    const bool vec = MODE != MODE_ROUTER || t.ncols % 4 == 0;
    uint2 bb[2][4];
    if (BIAS == 1) {  // the eight reads in flight together, one wait
      u32x2_t bq[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          bq[j * 4 + g] = ds_read8u((uint32_t)(uintptr_t)(bias_lds + (ob + j * 32 + g * 8 - t.c0) / 2));
      lds_wait8(bq);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) bb[j][g] = make_uint2(bq[j * 4 + g].x, bq[j * 4 + g].y);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int o = ob + j * 32 + g * 8;
        if (BIAS == 2 && vec)
          bb[j][g] = *reinterpret_cast<const uint2*>(a.bias + (MODE == MODE_DOWN ? (size_t)t.seg * a.H : 0) +
                                                     min(o, t.ncols - 4));
        else if (BIAS != 1)
          bb[j][g] = make_uint2(0u, 0u);
      }
    if (BIAS == 2) vm_wait_all();
    if (STG && MODE == MODE_DOWN) {
      lds_barrier();
      if (t.c0 + wn * 64 >= t.ncols) return;
      const uint32_t R = (uint32_t)(uintptr_t)stage;  // 32 rows x 128 bytes
      const int c = lane & 7;
      int32_t id[2][4];  // y rows (assignment ids) of the rows this lane stores
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int it = 0; it < 4; ++it) id[i][it] = ds_read4(ids + min(wm * 64 + i * 32 + it * 8 + (lane >> 3), BM - 1));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            // (without a bias the sums go out as they are: no +0 per output)
            const float v0 = BIAS ? acc[i][j][g * 4] + bf16lo(bb[j][g].x) : acc[i][j][g * 4];
            const float v1 = BIAS ? acc[i][j][g * 4 + 1] + bf16hi(bb[j][g].x) : acc[i][j][g * 4 + 1];
            const float v2 = BIAS ? acc[i][j][g * 4 + 2] + bf16lo(bb[j][g].y) : acc[i][j][g * 4 + 2];
            const float v3 = BIAS ? acc[i][j][g * 4 + 3] + bf16hi(bb[j][g].y) : acc[i][j][g * 4 + 3];
            const uint32_t y01 = pack_bf16(v0, v1), y23 = pack_bf16(v2, v3);
            ds_write8(R + rl * 128 + (((j * 4 + g) ^ (rl & 7)) << 4) + hq * 8, y01, y23);
          }
        u32x4_t v[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int r = it * 8 + (lane >> 3);
          v[it] = ds_read16u(R + r * 128 + ((c ^ (r & 7)) << 4));
        }
        lds_wait4(v);
        asm volatile("" : "+v"(id[i][0]), "+v"(id[i][1]), "+v"(id[i][2]), "+v"(id[i][3]));
#pragma unroll
        for (int it = 0; it < 4; ++it)
          if (wm * 64 + i * 32 + it * 8 + (lane >> 3) < t.rows)
            *reinterpret_cast<u32x4_t*>((uint16_t*)a.out + (size_t)id[i][it] * t.ncols + t.c0 + wn * 64 + c * 8) =
                v[it];
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + rl;
      if (r >= t.rows) continue;
      size_t row;
      if (MODE == MODE_DOWN)
        row = (size_t)ds_read4_sync(ids + r);  // y row = the assignment id
      else if (split)
        row = (size_t)t.ks * a.T + t.p0 + r;
      else
        row = (size_t)(t.p0 + r);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int o = ob + j * 32 + g * 8;
          if (o >= t.ncols) continue;
          const float v[4] = {acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]};
          // + bias (+0 without one), as the few-token kernels do
          const float v0 = v[0] + bf16lo(bb[j][g].x), v1 = v[1] + bf16hi(bb[j][g].x);
          const float v2 = v[2] + bf16lo(bb[j][g].y), v3 = v[3] + bf16hi(bb[j][g].y);
          if (MODE == MODE_DOWN) {
            *reinterpret_cast<uint2*>((uint16_t*)a.out + row * t.ncols + o) =
                make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
          } else if (split) {
            float* dst = a.part + row * t.ncols + o;
            if (vec)
              *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            else
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (o + e < t.ncols) dst[e] = v[e];
          } else {
            float* dst = (float*)a.out + row * t.ncols + o;
            if (vec)
              *reinterpret_cast<float4*>(dst) = make_float4(v0, v1, v2, v3);
            else
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (o + e < t.ncols)
                  dst[e] = v[e] + (BIAS == 2 ? __uint_as_float((uint32_t)a.bias[o + e] << 16) : 0.f);
          }
        }
    }
  }
}

template <int MODE, bool BIAS_LDS = false, bool STG = false>
__device__ __forceinline__ void epilogue(const GemmArgs& a, const Tile& t, const f32x16_t (&acc)[2][2], int wm,
                                         int wn, const int32_t* ids, const uint32_t* bias_lds = nullptr,
                                         uint8_t* stage = nullptr) {
  constexpr bool S = STG && MODE != MODE_ROUTER;
  if (BIAS_LDS) {
    epilogue_b<MODE, 1, S>(a, t, acc, wm, wn, ids, bias_lds, stage);
    return;
  }
  const bool hb = a.bias && (MODE == MODE_GATEUP   ? a.oai && !t.sh
                             : MODE == MODE_DOWN ? !t.sh
                                                 : a.ksplit == 1);
  if (hb)
    epilogue_b<MODE, 2, S>(a, t, acc, wm, wn, ids, bias_lds, stage);
  else
    epilogue_b<MODE, 0, S>(a, t, acc, wm, wn, ids, bias_lds, stage);
}

// Next tile of this workgroup's run at or after lin (skipping column tiles
// past a narrower segment); false when the run is done.  `from` is a
// segment at or before the tile's (the previous tile's).
template <int MODE>
__device__ bool next_tile(const GemmArgs& a, const SegTables& st, int& lin, int lin_end, int step, int total_m,
                          Tile& t, int from) {
  for (; lin < lin_end; lin += step)
    if (tile_at<MODE>(a, st, lin, total_m, t, from)) return true;
  return false;
}

// Field-by-field copy (a whole-struct copy leaves slices in scratch memory).
__device__ __forceinline__ void tile_copy(Tile& d, const Tile& s) {
  d.seg = s.seg, d.p0 = s.p0, d.rows = s.rows, d.c0 = s.c0, d.Fe = s.Fe, d.ncols = s.ncols, d.K = s.K;
  d.ks = s.ks, d.k0 = s.k0, d.nk = s.nk, d.sh = s.sh;
}

template <int MODE, bool MX>
__global__ __launch_bounds__(kThreads, 1) void k_grouped_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[BM * 128], lds_a1[BM * 128], lds_a2[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b0[BN * 128], lds_b1[BN * 128], lds_b2[BN * 128];
  __shared__ SegTables st;
  __shared__ int32_t ids_s[3][BM];  // assignment ids of three consecutive tiles
  __shared__ __attribute__((aligned(16))) uint32_t bias_s[3][BM];  // and their bias words

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wid >> 2, wn = wid & 3;

  // The run of tiles of this workgroup.  The hardware deals workgroups
  // round-robin over the 8 XCDs; each XCD gets a contiguous range of the
  // (column tile, row tile) space, column-tile-major, so the row tiles
  // sharing one weight tile meet in the same L2, and its workgroups take
  // the range's tiles in turn.  The range is cut from the real number of
  // tiles (counted from the segment offsets), so the XCDs get equal shares.
  // With one workgroup per CU a workgroup runs several tiles back to back.
  const int total_m = MODE == MODE_ROUTER ? (a.T + BM - 1) / BM
                                          : __builtin_amdgcn_readfirstlane(build_tables(a.offsets, a.E + a.shared, st));
  const int total = total_m * a.n_tiles;
  const int per_xcd = (total + 7) / 8;
  const int nslots = gridDim.x / 8;
  const int xcd = blockIdx.x % 8;
  int lin = xcd * per_xcd + blockIdx.x / 8;
  const int lin_end = min((xcd + 1) * per_xcd, total);
  Tile tc, tn;
  if (!next_tile<MODE>(a, st, lin, lin_end, nslots, total_m, tc, 0)) return;

  Frag fr;
  fr.arow0 = wm * 64 + (lane & 31);
  if (MODE == MODE_GATEUP) {
    fr.brow0 = wn * 32 + (lane & 31);           // gate rows
    fr.brow1 = BN / 2 + wn * 32 + (lane & 31);  // matching up rows
  } else {
    fr.brow0 = wn * 64 + (lane & 31);
    fr.brow1 = wn * 64 + 32 + (lane & 31);
  }
  fr.khalf = lane >> 5;

  Pipe pc, pn;
  int ntile = 0;  // tiles made so far; tile n's ids live in ids_s[n % 3]
  make_pipe<MODE, MX>(a, tc, ids_s[ntile % 3], bias_s[ntile % 3], pc);
  ++ntile;
  wait_vm<0>();
  __syncthreads();
  finish_pipe<MODE>(a, pc);
  // step s's MXFP4 block sits in code registers cr[s % 3] (s counted over
  // the workgroup's whole run of tiles) until converted
  CodeRegs cr[3] = {};
  pipe_issue(pc, 0, wid, lds_a0, lds_b0, cr[0]);
  pipe_issue(pc, 1, wid, lds_a1, lds_b1, cr[1]);
  if (MX && pc.mx) {
    wait_vm<2>();  // step 0's block (step 1's code and scale loads may remain)
    pipe_put_codes(cr[0], lds_b0);
  }
  lin += nslots;
  bool more = next_tile<MODE>(a, st, lin, lin_end, nslots, total_m, tn, tc.seg);
  if (more) {
    make_pipe<MODE, MX>(a, tn, ids_s[ntile % 3], bias_s[ntile % 3], pn);
    ++ntile;
  } else {
    null_pipe(pc, pn);
  }

  int phase = 0;  // stage of the current tile's step 0
  f32x16_t acc[2][2];
  for (;;) {
    // stages and code registers rotate with the global step index
    if (phase == 0)
      tile_loop<MODE, MX>(a, pc, pn, fr, wid, acc, cr[0], cr[1], cr[2], lds_a0, lds_a1, lds_a2, lds_b0, lds_b1,
                          lds_b2);
    else if (phase == 1)
      tile_loop<MODE, MX>(a, pc, pn, fr, wid, acc, cr[1], cr[2], cr[0], lds_a1, lds_a2, lds_a0, lds_b1, lds_b2,
                          lds_b0);
    else
      tile_loop<MODE, MX>(a, pc, pn, fr, wid, acc, cr[2], cr[0], cr[1], lds_a2, lds_a0, lds_a1, lds_b2, lds_b0,
                          lds_b1);
    {
      // the stage the tile's last step read (idle until the next tile's step 0)
      const int ls = (phase + pc.nk + 2) % 3;
      uint8_t* const stage = (ls == 0 ? lds_b0 : ls == 1 ? lds_b1 : lds_b2) + wid * 4096;  // this wave's 4 KiB
      if (MODE != MODE_ROUTER && a.bias)
        epilogue<MODE, true, true>(a, tc, acc, wm, wn, pc.ids, pc.bias, stage);
      else
        epilogue<MODE, false, true>(a, tc, acc, wm, wn, pc.ids, nullptr, stage);
    }
    if (!more) break;
    phase = (phase + pc.nk) % 3;
    tile_copy(tc, tn);  // the tile of pn
    pipe_copy(pc, pn);
    lin += nslots;
    more = next_tile<MODE>(a, st, lin, lin_end, nslots, total_m, tn, tc.seg);
    if (more) {
      make_pipe<MODE, MX>(a, tn, ids_s[ntile % 3], bias_s[ntile % 3], pn);
      ++ntile;
    } else {
      null_pipe(pc, pn);
    }
  }
  wait_vm<0>();  // the zero-reading loads of the steps past the last tile
}


// ---------------------------------------------------------------------------
// MXFP8 activations x MXFP4 weights on the scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 A, E2M1 B, one E8M0 scale per
// 32-deep block of each operand row), with fp32 accumulation.  Same tiles,
// wave layout, segment walk and epilogues as the bf16 kernel above; a K
// step is 128 deep (two MFMA slices of 64; a last step of 64 when K is an
// odd multiple of 64).  Per step the LDS ring stage holds 128 activation
// rows of 128 code bytes (XOR-swizzled like the bf16 rows), 256 weight rows
// of 64 code bytes (slot p ^ ((n >> 2) & 3) of a row n: 16 consecutive rows
// read at one logical piece fall in 16 distinct 16-byte bank groups) and the
// activation rows' scale words; the tile's weight scales, contiguous in the
// caller's [rows][K/32] layout, sit in LDS as one block per tile (the next
// tile's block streams in while the current tile runs).
//
// Lane layout of the scaled MFMA (measured on gfx950): lane l holds operand
// row l % 32; for the E4M3 operand, K elements 16h..16h+15 of the slice's
// first 32-block and 32+16h..32+16h+15 of its second (h = l / 32); for the
// E2M1 operand, the 32 elements of block h, as stored (low nibble = even
// index); the scale of lane l applies to block l / 32 of its row.  The
// result layout is the 32x32 one of the bf16 MFMA.

constexpr int BK8 = 128;
constexpr int kLoads8 = 6;  // loads per thread per step: 2 A, 2 B, 1 activation scale word, 1 scale block chunk

__device__ __forceinline__ int swz_slot4(int n, int p) { return p ^ ((n >> 2) & 3); }

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t ds_read_u8a(const uint8_t* p) {
  uint32_t r;
  asm volatile("ds_read_u8 %0, %1" : "=v"(r) : "v"((uint32_t)(uintptr_t)p) : "memory");
  return r;
}
__device__ __forceinline__ uint32_t ds_read_b32a(const void* p) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"((uint32_t)(uintptr_t)p) : "memory");
  return r;
}

// Fragments and scales of one K step (two slices).
struct Mx8Frag {
  bf16x8_t a[2][2][2];  // [slice][row block][piece]
  bf16x8_t b[2][2];     // [slice][column block]
  uint32_t sa[2];       // scale word of each row block
  uint32_t sb[2][2];    // [slice][column block] scale byte
};
// Wait until at most N LDS reads are outstanding; ties the fragments of
// slice S (and the activation scale words) to that wait.
template <int N, int S> __device__ __forceinline__ void mx8_wait(Mx8Frag& f) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(f.a[S][0][0]), "+v"(f.a[S][0][1]), "+v"(f.a[S][1][0]), "+v"(f.a[S][1][1]), "+v"(f.b[S][0]),
                 "+v"(f.b[S][1]), "+v"(f.sb[S][0]), "+v"(f.sb[S][1])
               : "n"(N), "v"(f.sa[0]), "v"(f.sa[1]));
  asm volatile("" : "+v"(f.sa[0]), "+v"(f.sa[1]));
}

// Bytes of a tile's weight scale block in LDS: 256 weight rows of K/32
// bytes, contiguous in the caller's layout, copied as the aligned dwords
// that cover them.
__host__ __device__ constexpr int mx8_block_bytes(int K) { return BN * (K / 32) + 256; }

// Load state of one tile of the MXFP8 kernel: the segment's weight
// descriptor and this thread's source offsets of step 0 (a step adds
// s * 128 to the activation offset, s * 64 to the weight offset, s * 4 to
// the activation scale offset).
struct Mx8Pipe {
  __amdgpu_buffer_rsrc_t rw;
  uint32_t aoff[2], boff[2], soff;
  uint32_t sc_start;  // first byte of the tile's weight scale block
  bool a_ok[2], s_ok;
  int32_t* ids;
  uint32_t* bias;  // the tile's bias in LDS (gate/up: 128 (gate, up) bf16 pairs; down: 256 bf16)
  int nk;
  int seg, c0;
};

// Weight row (in the segment's matrix) of tile row n.
template <int MODE>
__device__ __forceinline__ int mx8_wrow(const GemmArgs& a, int c0, int n) {
  if (MODE == MODE_GATEUP) return 2 * min(c0 + (n & (BN / 2 - 1)), a.F - 1) + (n >= BN / 2);
  return min(c0 + n, a.H - 1);
}

// Set up tile t: descriptors and the offsets that do not need the tile's
// assignment ids; the ids themselves go to LDS through buffer->LDS loads of
// waves 0 and 1 (gate/up takes its activation rows from them in
// mx8_finish_pipe, once a wait and a barrier have covered those loads).
template <int MODE>
__device__ void mx8_make_pipe(const GemmArgs& a, const Tile& t, int K, int32_t* ids, uint32_t* bias, Mx8Pipe& p) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int rows_e = MODE == MODE_GATEUP ? 2 * a.F : a.H;
  const size_t wbytes = (size_t)rows_e * (K / 2);
  p.rw = make_rsrc((const uint8_t*)a.w0 + (size_t)t.seg * wbytes, (uint32_t)wbytes);
  p.ids = ids;
  p.nk = (K + BK8 - 1) / BK8;
  p.seg = t.seg;
  p.c0 = t.c0;
  p.bias = bias;
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform descriptors
  if (wv < BM / kWave) {
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(a.sorted_assign + t.p0, (uint32_t)t.rows * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ri, (lds_ptr_t)(ids + (tid & ~(kWave - 1))), 4, (int)(tid * 4), 0, 0, 0);
  } else if (wv < 2 * BM / kWave) {
    // the tile's bias, 512 bytes from dword-aligned offsets (columns past
    // the matrix read zeros), so the epilogue has no global load to wait for
    const size_t e0 = MODE == MODE_GATEUP ? (size_t)t.seg * 2 * a.F + 2 * t.c0 : (size_t)t.seg * a.H + t.c0;
    const int n = MODE == MODE_GATEUP ? 2 * (a.F - t.c0) : a.H - t.c0;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.bias ? a.bias + e0 : a.bias, a.bias ? (uint32_t)n * 2 : 0u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(bias + ((tid - BM) & ~(kWave - 1))), 4,
                                             (int)((tid - BM) * 4), 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + i * kThreads;
    const int r = q / 8;
    p.a_ok[i] = r < t.rows;
    p.aoff[i] = MODE == MODE_DOWN && r < t.rows ? (uint32_t)((size_t)(t.p0 + r) * K) + (swz_slot(r, q % 8) << 4)
                                                : kOutOfRange;
  }
  {
    const int r = (tid / kWave) * 16 + (lane & 15);  // lanes 0..15 of each wave: one activation row's scale word
    p.s_ok = lane < 16 && r < t.rows;
    p.soff = MODE == MODE_DOWN && p.s_ok ? (uint32_t)((size_t)(t.p0 + r) * a.a8s_stride) : kOutOfRange;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + i * kThreads;
    const int n = q / 4;
    p.boff[i] = (uint32_t)((size_t)mx8_wrow<MODE>(a, t.c0, n) * (K / 2)) + (swz_slot4(n, q % 4) << 4);
  }
  const int rb0 = MODE == MODE_GATEUP ? 2 * t.c0 : t.c0;
  p.sc_start = (uint32_t)(((size_t)t.seg * rows_e + rb0) * (K / 32));
}

template <int MODE>
__device__ __forceinline__ void mx8_finish_pipe(const GemmArgs& a, int K, Mx8Pipe& p) {
  if (MODE != MODE_GATEUP) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + i * kThreads;
    const int id = ds_read4_sync(p.ids + q / 8);
    if (p.a_ok[i]) p.aoff[i] = (uint32_t)((size_t)(id / a.k) * K) + (swz_slot(q / 8, q % 8) << 4);
  }
  const int id = ds_read4_sync(p.ids + (tid / kWave) * 16 + (lane & 15));
  if (p.s_ok) p.soff = (uint32_t)((size_t)(id / a.k) * a.a8s_stride);
}

__device__ __forceinline__ void mx8_pipe_copy(Mx8Pipe& d, const Mx8Pipe& s) {
  d.rw = s.rw;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    d.aoff[i] = s.aoff[i];
    d.boff[i] = s.boff[i];
    d.a_ok[i] = s.a_ok[i];
  }
  d.soff = s.soff;
  d.sc_start = s.sc_start;
  d.s_ok = s.s_ok;
  d.ids = s.ids;
  d.bias = s.bias;
  d.nk = s.nk;
  d.seg = s.seg;
  d.c0 = s.c0;
}

// A pipe with no steps and no tile: all its loads read zeros.
__device__ __forceinline__ void mx8_null_pipe(const Mx8Pipe& like, Mx8Pipe& p) {
  mx8_pipe_copy(p, like);
  p.nk = 0;
  p.s_ok = false;
  p.soff = kOutOfRange;
  p.sc_start = kOutOfRange;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    p.a_ok[i] = false;
    p.aoff[i] = kOutOfRange;
  }
}

// One workgroup runs a contiguous share of the tiles, as the bf16 kernel
// does: the LDS ring runs on across tiles (the last two K steps of a tile
// issue the first two of the next), the next tile's assignment ids go out
// when it is set up, and its weight scale block streams into the second
// block buffer during the current tile, one 256-byte chunk per wave per
// step.  A launch with fewer than three K steps per tile gives every
// workgroup one tile and has a single block buffer.
template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_mx8_gemm(GemmArgs a, int persistent) {
  __shared__ __attribute__((aligned(1024))) uint8_t la[3][BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lb[3][BN * 64];
  __shared__ __attribute__((aligned(16))) uint32_t lsa[3][(kThreads / kWave) * kWave];
  __shared__ SegTables st;
  __shared__ int32_t ids_s[3][BM];
  __shared__ __attribute__((aligned(16))) uint32_t bias_s[3][BM];
  __shared__ __attribute__((aligned(16))) uint32_t dump[kWave];  // target of the chunk loads with no block to fill
  extern __shared__ __attribute__((aligned(16))) uint8_t lsb_dyn[];  // one or two weight scale blocks

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wid >> 2, wn = wid & 3;
  const int hh = lane >> 5;

  const int total_m = __builtin_amdgcn_readfirstlane(build_tables(a.offsets, a.E, st));
  const int total = total_m * a.n_tiles;
  const int per_xcd = (total + 7) / 8;
  const int nslots = gridDim.x / 8;
  const int xcd = blockIdx.x % 8;
  int lin = xcd * per_xcd + blockIdx.x / 8;
  const int lin_end = min((xcd + 1) * per_xcd, total);
  Tile tc, tn;
  if (!next_tile<MODE>(a, st, lin, lin_end, nslots, total_m, tc, 0)) return;
  const int K = MODE == MODE_GATEUP ? a.H : a.F;
  const int kb = K / 32;  // scale bytes per row
  const int bbytes = mx8_block_bytes(K);

  const int64_t nas = (int64_t)a.T * a.k;
  const size_t arows = MODE == MODE_GATEUP ? (size_t)a.T : (size_t)nas;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.a8, (uint32_t)(arows * K));
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(a.a8s, (uint32_t)(arows * a.a8s_stride));
  const int rows_e = MODE == MODE_GATEUP ? 2 * a.F : a.H;
  // the scale blocks are read as whole dwords from a 4-byte aligned base
  const uint32_t smis = (uint32_t)((uintptr_t)a.scales & 3u);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(a.scales - smis, (uint32_t)((smis + (size_t)a.E * rows_e * kb + 3) & ~(size_t)3));
  const int nchunk = (BN * kb + 3 + 3) / 4 / kWave + 1;  // 256-byte chunks covering a block
  // chunk c of the block starting at byte sc (relative to the aligned base)
  auto chunk_off = [&](uint32_t sc, int c) -> uint32_t {
    return sc == kOutOfRange || c >= nchunk ? kOutOfRange : ((sc + smis) & ~3u) + (uint32_t)(c * 256 + lane * 4);
  };

  // fragment rows of this lane
  const int ar0 = wm * 64 + (lane & 31);
  int bn[2];
  if (MODE == MODE_GATEUP) {
    bn[0] = wn * 32 + (lane & 31);
    bn[1] = BN / 2 + wn * 32 + (lane & 31);
  } else {
    bn[0] = wn * 64 + (lane & 31);
    bn[1] = wn * 64 + 32 + (lane & 31);
  }
  int li[2];  // row of each column row in the tile's scale block
#pragma unroll
  for (int j = 0; j < 2; ++j)
    li[j] = MODE == MODE_GATEUP ? (bn[j] < BN / 2 ? 2 * bn[j] : 2 * (bn[j] - BN / 2) + 1) : bn[j];

  auto issue = [&](const Mx8Pipe& x, int s, int sg) {
    const bool ok = s < x.nk;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16(ra, la[sg] + (i * kThreads + wid * kWave) * 16,
            ok && x.aoff[i] != kOutOfRange ? x.aoff[i] + s * BK8 : kOutOfRange);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16(x.rw, lb[sg] + (i * kThreads + wid * kWave) * 16, ok ? x.boff[i] + s * (BK8 / 2) : kOutOfRange);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, (lds_ptr_t)(lsa[sg] + wid * kWave), 4,
                                             (int)(ok && x.soff != kOutOfRange ? x.soff + s * 4 : kOutOfRange), 0, 0,
                                             0);
  };

  Mx8Pipe pc, pn;
  int ntile = 0;  // tiles set up so far; tile n's ids and bias live in slot n % 3, its block in buffer n % 2
  mx8_make_pipe<MODE>(a, tc, K, ids_s[ntile % 3], bias_s[ntile % 3], pc);
  ++ntile;
  // the first tile's scale block, whole
  for (int c = wid; c < nchunk; c += kThreads / kWave)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lsb_dyn + c * 256), 4, (int)chunk_off(pc.sc_start, c), 0,
                                             0, 0);
  wait_vm<0>();
  __syncthreads();
  mx8_finish_pipe<MODE>(a, K, pc);
  issue(pc, 0, 0);
  issue(pc, 1, 1);
  lin += nslots;
  bool more = persistent && next_tile<MODE>(a, st, lin, lin_end, nslots, total_m, tn, tc.seg);
  if (more)
    mx8_make_pipe<MODE>(a, tn, K, ids_s[ntile % 3], bias_s[ntile % 3], pn), ++ntile;
  else
    mx8_null_pipe(pc, pn);

  int sg = 0;   // stage of the next step to compute
  int cur = 0;  // block buffer of the current tile
  f32x16_t acc[2][2];
  for (;;) {
    const uint8_t* lsb = lsb_dyn + cur * bbytes;
    uint8_t* lsb_next = lsb_dyn + (cur ^ 1) * bbytes;
    const int shift = (int)((pc.sc_start + smis) & 3u);
    int bsc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) bsc[j] = shift + li[j] * kb + hh;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Per step: wait for this thread's loads of step kt (at most the next
    // step's remain), barrier (all threads' loads landed; everyone finished
    // step kt - 1, whose stage the next loads reuse), issue step kt + 2 of
    // this tile or, past its end, of the next, and one chunk of the next
    // tile's scale block, then compute step kt.  The next tile's ids went
    // out before this tile's step 2 loads, so the wait and barrier of step
    // nk - 2 (nk >= 3 in persistent launches) covered them.
    for (int kt = 0; kt < pc.nk; ++kt) {
      wait_vm<kLoads8>();
      lds_barrier();
      const int s2 = kt + 2;
      if (s2 == pc.nk) mx8_finish_pipe<MODE>(a, K, pn);
      const bool uq = s2 >= pc.nk;
      Mx8Pipe x;
      x.rw = uq ? pn.rw : pc.rw;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        x.aoff[i] = uq ? pn.aoff[i] : pc.aoff[i];
        x.boff[i] = uq ? pn.boff[i] : pc.boff[i];
      }
      x.soff = uq ? pn.soff : pc.soff;
      x.nk = uq ? pn.nk : pc.nk;
      issue(x, uq ? s2 - pc.nk : s2, sg == 0 ? 2 : sg - 1);
      {
        // chunk c of the next tile's block (a launch with one tile per
        // workgroup has no second buffer: its chunk loads read zeros into dump)
        const int c = kt * (kThreads / kWave) + wid;
        const bool fill = persistent && c < nchunk;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(fill ? (void*)(lsb_next + c * 256) : (void*)dump), 4,
                                                 (int)(fill ? chunk_off(pn.sc_start, c) : kOutOfRange), 0, 0, 0);
      }

      const uint8_t* A = la[sg];
      const uint8_t* B = lb[sg];
      Mx8Frag f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = ar0 + 32 * i;
        f.sa[i] = ds_read_b32a(lsa[sg] + (r / 16) * kWave + (r % 16));
      }
      // slice 1's reads are in flight during slice 0's MFMAs
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          f.a[s][i][0] = ds_read16(A + swz(ar0 + 32 * i, 4 * s + hh));
          f.a[s][i][1] = ds_read16(A + swz(ar0 + 32 * i, 4 * s + 2 + hh));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int p = 2 * s + hh;
          f.b[s][j] = ds_read16(B + bn[j] * 64 + (swz_slot4(bn[j], p) << 4));
          f.sb[s][j] = ds_read_u8a(lsb + bsc[j] + 4 * kt + 2 * s);
        }
      }
      const int nsl = K - kt * BK8 >= BK8 ? 2 : 1;
      auto slice = [&](int s) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t* p0 = reinterpret_cast<const uint32_t*>(&f.a[s][i][0]);
          const uint32_t* p1 = reinterpret_cast<const uint32_t*>(&f.a[s][i][1]);
          const i32x8_t av = {(int)p0[0], (int)p0[1], (int)p0[2], (int)p0[3],
                              (int)p1[0], (int)p1[1], (int)p1[2], (int)p1[3]};
          const int sa = (int)((f.sa[i] >> (8 * (2 * s + hh))) & 0xFFu);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint32_t* pb = reinterpret_cast<const uint32_t*>(&f.b[s][j]);
            const i32x8_t bv = {(int)pb[0], (int)pb[1], (int)pb[2], (int)pb[3], 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], 4, 0, 0,
                                                                         (int)f.sb[s][j], 0, sa);
          }
        }
      };
      mx8_wait<8, 0>(f);
      slice(0);
      mx8_wait<0, 1>(f);
      if (nsl == 2) slice(1);
      sg = sg == 2 ? 0 : sg + 1;
    }
    {
      // the stage the tile's last step read (two 16 KiB halves: waves 0-3
      // take the activation half, 4-7 the weight half)
      const int ls = sg == 0 ? 2 : sg - 1;
      uint8_t* const stage = (wid < 4 ? la[ls] : lb[ls]) + (wid & 3) * 4096;
      epilogue<MODE, true, true>(a, tc, acc, wm, wn, pc.ids, pc.bias, stage);
    }
    if (!more) break;
    tile_copy(tc, tn);  // the tile of pn
    mx8_pipe_copy(pc, pn);
    cur ^= 1;
    lin += nslots;
    more = next_tile<MODE>(a, st, lin, lin_end, nslots, total_m, tn, tc.seg);
    if (more)
      mx8_make_pipe<MODE>(a, tn, K, ids_s[ntile % 3], bias_s[ntile % 3], pn), ++ntile;
    else
      mx8_null_pipe(pc, pn);
  }
  wait_vm<0>();  // the zero-reading loads of the steps past the last tile
}

int row_tiles_bound(const moe_config* c, int32_t T) {
  const int64_t nk = (int64_t)T * c->top_k;
  const int64_t nonempty = nk < c->n_expert ? nk : c->n_expert;
  int64_t b = (nk + (int64_t)(BM - 1) * nonempty) / BM;
  if (c->shared_ff > 0) b += (T + BM - 1) / BM;
  return (int)b;
}

// Workgroups of a launch: one per tile, or, when every tile has at least
// three K steps (the ring hands steps 0 and 1 of the next tile over from the
// previous one, and the next tile's ids must have landed two steps before
// its end), at most one per CU, each running its share of the tiles.
int grid_size(int64_t tiles, bool persistent) {
  int64_t blocks = tiles;
  if (persistent) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
      ncu = 256;
    if (blocks > ncu) blocks = ncu;
  }
  return (int)((blocks + 7) / 8 * 8);
}

template <int MODE>
hipError_t launch(const GemmArgs& a, bool mx, int min_k, hipStream_t s) {
  const int64_t tiles = (int64_t)a.n_tiles * a.m_tiles_max;
  const unsigned blocks = (unsigned)grid_size(tiles, min_k >= 3 * BK);
  if (mx)
    k_grouped_gemm<MODE, true><<<blocks, kThreads, 0, s>>>(a);
  else
    k_grouped_gemm<MODE, false><<<blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

// Static LDS of k_mx8_gemm besides the scale block buffers (the ring, the
// segment tables, the ids and biases of three tiles, the dump target).
constexpr int kMx8StaticLds =
    3 * BM * 128 + 3 * BN * 64 + 3 * kThreads * 4 + (int)sizeof(SegTables) + 2 * 3 * BM * 4 + kWave * 4;
constexpr int kLdsBytes = 160 * 1024;

// Persistent (two scale block buffers) when a tile has at least three K
// steps and two blocks fit in LDS; otherwise one tile per workgroup.
template <int MODE>
hipError_t launch_mx8(const GemmArgs& a, int K, hipStream_t s) {
  const int64_t tiles = (int64_t)a.n_tiles * a.m_tiles_max;
  const int nk = (K + BK8 - 1) / BK8;
  const bool persistent = nk >= 3 && kMx8StaticLds + 2 * mx8_block_bytes(K) + 1024 <= kLdsBytes;
  const size_t dyn = (size_t)(persistent ? 2 : 1) * mx8_block_bytes(K);
  if (kMx8StaticLds + dyn + 1024 > (size_t)kLdsBytes) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)grid_size(tiles, persistent);
  k_mx8_gemm<MODE><<<blocks, kThreads, dyn, s>>>(a, persistent ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

// Router split of the K steps: about one tile per two CUs over all splits
// (measured against one per CU: qwen35moe T = 4096 router product and
// gating 31.0 -> 27.4 us, gpt-oss T = 2048 15.3 -> 14.6 us; each more split
// writes and reads back another [T][E] fp32 partial), at least three steps
// per range (persistent launches), ranges of equal length but the last.
void router_split(const moe_config* c, int32_t T, int* ksplit, int* steps) {
  const int nk = c->hidden / BK;
  const int tiles = ((c->n_expert + BN - 1) / BN) * ((T + BM - 1) / BM);
  int ks = 128 / (tiles > 0 ? tiles : 1);
  if (ks > nk / 3) ks = nk / 3;
  if (ks < 1) ks = 1;
  const int spp = (nk + ks - 1) / ks;
  *steps = spp;
  *ksplit = (nk + spp - 1) / spp;
}

hipError_t launch_router_mfma(const moe_config* c, const moe_weights* w, const void* x, int32_t T, float* logits,
                              float* sgate_pre, hipStream_t s, float* part) {
  (void)sgate_pre;  // the shared-gate dot is taken by the gating kernel
  GemmArgs a = {};
  a.a_src = (const uint16_t*)x;
  a.w0 = w->router_w;
  a.bias = (const uint16_t*)w->router_b;
  a.out = logits;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = c->shared_ff;
  a.col_tiles = (c->n_expert + BN - 1) / BN;
  a.m_tiles_max = (T + BM - 1) / BM;
  a.ksplit = 1;
  a.split_steps = c->hidden / BK;
  if (part) router_split(c, T, &a.ksplit, &a.split_steps);
  a.part = part;
  a.n_tiles = a.col_tiles * a.ksplit;
  const int nk = c->hidden / BK;
  const int last = nk - (a.ksplit - 1) * a.split_steps;  // steps of the last range
  return launch<MODE_ROUTER>(a, false, (last < a.split_steps ? last : a.split_steps) * BK, s);
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
  a.ksplit = 1;
  a.split_steps = c->hidden / BK;
  return launch<MODE_GATEUP>(a, c->w_dtype == MOE_DTYPE_MXFP4, c->hidden, s);
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
  a.ksplit = 1;
  a.split_steps = (c->expert_ff > c->shared_ff ? c->expert_ff : c->shared_ff) / BK;
  const int min_k = c->shared_ff > 0 && c->shared_ff < c->expert_ff ? c->shared_ff : c->expert_ff;
  return launch<MODE_DOWN>(a, c->w_dtype == MOE_DTYPE_MXFP4, min_k, s);
}


// MXFP8 x MXFP4 expert products (routed experts only, no shared expert).
hipError_t launch_gateup_mx8(const moe_config* c, const moe_weights* w, const uint8_t* xq, const uint8_t* xs,
                             const int32_t* offsets, const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s) {
  GemmArgs a = {};
  a.a8 = xq;
  a.a8s = xs;
  a.a8s_stride = ((c->hidden + BK8 - 1) / BK8) * 4;
  a.w0 = w->gate_up_w;
  a.scales = w->gate_up_scales;
  a.bias = (const uint16_t*)w->gate_up_b;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.out = h;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = 0;
  a.shared = 0; a.oai = 1; a.alpha = c->act_alpha; a.limit = c->act_limit;
  a.n_tiles = (c->expert_ff + BN / 2 - 1) / (BN / 2);
  a.m_tiles_max = row_tiles_bound(c, T);
  a.ksplit = 1;
  a.split_steps = c->hidden / BK;
  return launch_mx8<MODE_GATEUP>(a, c->hidden, s);
}

hipError_t launch_down_mx8(const moe_config* c, const moe_weights* w, const uint8_t* hq, const uint8_t* hs,
                           const int32_t* offsets, const int32_t* sorted_assign, int32_t T, uint16_t* y, hipStream_t s) {
  GemmArgs a = {};
  a.a8 = hq;
  a.a8s = hs;
  a.a8s_stride = ((c->expert_ff + BK8 - 1) / BK8) * 4;
  a.w0 = w->down_w;
  a.scales = w->down_scales;
  a.bias = (const uint16_t*)w->down_b;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.out = y;
  a.T = T; a.k = c->top_k; a.H = c->hidden; a.E = c->n_expert; a.F = c->expert_ff; a.Fs = 0;
  a.shared = 0; a.oai = 1;
  a.n_tiles = (c->hidden + BN - 1) / BN;
  a.m_tiles_max = row_tiles_bound(c, T);
  a.ksplit = 1;
  a.split_steps = c->expert_ff / BK;
  return launch_mx8<MODE_DOWN>(a, c->expert_ff, s);
}

}  // namespace moe
