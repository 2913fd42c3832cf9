// Internal declarations shared by the HIP translation units of libmoe.
// Device helpers for bf16 / MXFP4 element handling, the workspace plan and
// the host-side launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
// GEMV-style expert kernels (one weight stream, few tokens per expert) are
// used while T <= this; above it bf16 layers go to the MFMA grouped GEMM.
constexpr int kGemvMaxT = 64;
// Permutation: up to this many tokens one workgroup does everything.
constexpr int kPermSmallTokens = 256;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- device

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 values -> packed bf16 (lo in the low half), round to nearest
// even, one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

// Logistic sigma(x) = 1 / (1 + e^-x) on the hardware base-2 exponential and
// reciprocal (v_exp_f32, v_rcp_f32: about one ulp each in fp32; e^-x = 2^(-x
// log2 e), whose product rounding grows the relative error to ~|x| 2^-24).
// The expert activations x sigma(x) and the gpt-oss form use it: their
// results are rounded to bf16 (2^-9) or summed at that tolerance, so five
// instructions replace the ~25 of a full-precision exponential and IEEE
// divide.  Large |x|: 2^(+inf) -> sigma = 0, 2^(-inf) -> sigma = 1.
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504088896341f * x));
}
// SwiGLU's x sigma(x) * up and the clamped gpt-oss activation
// (up + 1) * g sigma(alpha g) (g clamped above, up to [-limit, limit]).
__device__ __forceinline__ float swiglu_act(float g, float u) { return g * sigmoid_fast(g) * u; }
__device__ __forceinline__ float oai_act(float g, float u, float alpha, float limit) {
  g = fminf(g, limit);
  u = fminf(fmaxf(u, -limit), limit);
  return (u + 1.f) * (g * sigmoid_fast(alpha * g));
}

// Order-preserving map of an fp32 value to uint32 with -0 folded into +0:
// a > b (as floats, NaN excluded) <=> key(a) > key(b); -0 and +0 tie.  The
// key is never 0 (the top-k's mark for a picked or absent expert): the one
// pattern that would map there, the NaN 0xFFFFFFFF, gets key 1, below -Inf
// like every NaN with the sign bit set.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  const uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return k ? k : 1u;
}

// DPP lane exchanges (gfx9 encodings): quad permutes, mirrors within a
// 16-lane row.  Used for the butterfly steps xor 1, xor 2, then half-row and
// row swaps, which leave the full reduction of each 8- or 16-lane group in
// every lane of the group.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i inside each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i inside each 16 lanes

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Sum over each group of 8 consecutive lanes, result in all 8 lanes.
__device__ __forceinline__ float group8_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v;
}
// Sum over each 16-lane row, result in all 16 lanes.
__device__ __forceinline__ float row16_sum(float v) {
  v = group8_sum(v);
  v += dpp<kDppMirror>(v);
  return v;
}
// Wave-wide sum, wave-uniform result; the same order for every call.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (a + b) + (c + d);
}
// Raw buffer resource over [base, base + bytes): loads at offsets past the
// end return zero (gfx9 descriptor word 3: 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// Weight rows that a decode-sized layer reads once carry the streaming
// cache policy (non-temporal, sc0): 6-8% more read bandwidth than the
// default policy on a pure weight stream.
constexpr int kStreamPolicy = 3;  // cache-policy bits: sc0 | nt
__device__ __forceinline__ uint4 buf_load16_once(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kStreamPolicy));
}
__device__ __forceinline__ uint32_t buf_load_u8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past every buffer: loads give 0

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct buffer -> LDS load of 16 bytes per lane: lane l of the wave writes
// LDS bytes [lds + 16 l, lds + 16 l + 16) (lds must be wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, (int)voff, 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the K pipeline: LDS writes of this wave complete,
// then s_barrier.  Unlike __syncthreads it is not a release fence, so the
// buffer->LDS loads still in flight for later steps are not waited for; the
// loads of the step about to be read are waited for explicitly (wait_vm).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// E8M0 exponent byte -> 2^(s-127) as fp32 (s = 0 gives 2^-127, subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// ---------------------------------------------------------------- host

// Scratch layout of moe_forward inside the caller's workspace (bytes).
struct Plan {
  int32_t T, H, E, k, F, Fs;
  int shared;
  int64_t n_assign;   // T*k
  int64_t n_rows;     // T*k (+T)
  int nseg;           // E (+1)
  size_t elem_x;      // bytes per activation / h element
  size_t off_logits, off_idx, off_w, off_sgate, off_offsets, off_sorted, off_pos;
  size_t off_perm, off_h, off_y, off_part, off_aqx, off_aqh, off_xn, total;
  // few tokens: the segment-slot table the permutation writes for the
  // decode expert kernels (nslots entries of {expert, first row, rows, 0})
  size_t off_segtab;
  int nslots;
  int32_t nsplit;     // router split-K ranges (1: none)
  size_t perm_bytes, y_bytes;  // scratch needed by moe_permute / moe_combine alone
  // act_quant: rounded x (moe_expert_ffn's scratch) and rounded h (after y in
  // moe_combine's scratch); each is the bf16 values or the E4M3 codes, then
  // the E8M0 scales at aqx_scales / aqh_scales bytes in
  size_t aqx_bytes, aqh_bytes, aqx_scales, aqh_scales;
  bool mx8;           // act_quant and the MFMA path: codes + scales, else bf16 values
};

int make_plan(const moe_config* c, int32_t T, Plan* p);
int check_config(const moe_config* c);

// Launchers (return hipError_t of the last launch).
// part: when the router product runs on MFMA (sgate_in_router false) and
// part is given, it is split over K ranges (router_split) with the partial
// sums in part [nsplit][T][E], which launch_gating then adds up into logits.
hipError_t launch_router_logits(const moe_config* c, const moe_weights* w, const void* x, int32_t T,
                                float* logits, float* sgate_pre, hipStream_t s, float* part = nullptr);
void router_split(const moe_config* c, int32_t T, int* nsplit, int* steps);
hipError_t launch_gating(const moe_config* c, const moe_weights* w, const void* x, float* logits,
                         const float* sgate_pre, int32_t T, int32_t* topk_idx, float* topk_w, float* sgate,
                         hipStream_t s, const float* part = nullptr, int32_t nsplit = 1);
// Whether the shared-gate dot is computed by the router-product kernel
// (few tokens) rather than by the gating kernel.
bool sgate_in_router(const moe_config* c, int32_t T);
hipError_t launch_permute(const moe_config* c, const int32_t* topk_idx, int32_t T, int32_t* offsets,
                          int32_t* sorted_assign, int32_t* assign_pos, int32_t* scratch, hipStream_t s);
size_t permute_scratch_bytes(int32_t T, int32_t E, int32_t k);
// Gating + permutation in one launch for small batches.
bool can_fuse_gate_permute(int32_t T);
// segtab (or NULL): also write the segment-slot table, slot 0 the shared
// expert when there is one, then the non-empty routed segments in expert
// order, then {-1, 0, 0, 0} up to nslots.
hipError_t launch_gate_permute(const moe_config* c, const float* logits, const float* sgate_pre, int32_t T,
                               int32_t* topk_idx, float* topk_w, float* sgate, int32_t* offsets,
                               int32_t* sorted_assign, int32_t* assign_pos, hipStream_t s, int32_t* segtab = nullptr,
                               int nslots = 0);
// Segment slots of the few-token expert launches (routed ones + shared).
int gemv_slots(const moe_config* c, int32_t T);
// segtab: the permutation's slot table (the kernels take their segment
// from it with one scalar load) or NULL (they search the offsets).
hipError_t launch_expert_ffn(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                             const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s,
                             const int32_t* segtab = nullptr);
// y rows are indexed by assignment id a (routed a = t*k + j, shared a = T*k + t);
// y is bf16 when the MFMA grouped GEMM computes it (y_is_bf16), fp32 otherwise.
bool y_is_bf16(const moe_config* c, int32_t T);
hipError_t launch_down(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                       const int32_t* sorted_assign, int32_t T, void* y, hipStream_t s,
                       const int32_t* segtab = nullptr);
// resid: NULL, or [T][H] x_dtype rows added to out (the block's residual).
hipError_t launch_combine_gather(const moe_config* c, const void* y, const float* topk_w, const float* sgate,
                                 int32_t T, float* out, hipStream_t s, const void* resid = nullptr);
// The few-token router product with the RMSNorm prologue folded in: resid
// rows are normalised on the fly (weight g) and also written to xn
// (route.hip); usable when router_norm_fusable.
bool router_norm_fusable(const moe_config* c, const moe_weights* w, int32_t T);
hipError_t launch_router_logits_norm(const moe_config* c, const moe_weights* w, const void* resid, const void* g,
                                     float eps, int32_t T, void* xn, float* logits, float* sgate_pre, hipStream_t s);
// RMSNorm of T rows of x ([T][H] x_dtype) with weight g [H] into y (norm.hip).
hipError_t launch_rmsnorm(const moe_config* c, const void* x, const void* g, float eps, int32_t T, void* y,
                          hipStream_t s);
// MXFP8 rounding of bf16 rows [rows][K] (mxfp8.hip): E4M3 codes + E8M0
// scales (row stride mx8_scale_stride(K) bytes), or the rounded bf16 values.
int mx8_scale_stride(int K);
hipError_t launch_mxfp8_codes(const uint16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);
hipError_t launch_mxfp8_values(const uint16_t* src, int64_t rows, int K, uint16_t* dst, hipStream_t s);
// MXFP8 x MXFP4 grouped expert products on the scaled MFMA (ffn_mfma.hip).
hipError_t launch_gateup_mx8(const moe_config* c, const moe_weights* w, const uint8_t* xq, const uint8_t* xs,
                             const int32_t* offsets, const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s);
hipError_t launch_down_mx8(const moe_config* c, const moe_weights* w, const uint8_t* hq, const uint8_t* hs,
                           const int32_t* offsets, const int32_t* sorted_assign, int32_t T, uint16_t* y, hipStream_t s);

}  // namespace moe
