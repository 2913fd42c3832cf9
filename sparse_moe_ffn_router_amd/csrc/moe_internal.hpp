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
// Permutation: up to this many assignments one workgroup does everything.
constexpr int kPermSmallMax = 2048;
constexpr int kPermChunk = 256;

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

// Order-preserving map of an fp32 value to uint32 with -0 folded into +0:
// a > b (as floats, NaN excluded) <=> key(a) > key(b); -0 and +0 tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

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
  size_t off_perm, off_h, off_y, total;
  size_t perm_bytes, y_bytes;  // scratch needed by moe_permute / moe_combine alone
};

int make_plan(const moe_config* c, int32_t T, Plan* p);
int check_config(const moe_config* c);

// Launchers (return hipError_t of the last launch).
hipError_t launch_router_logits(const moe_config* c, const moe_weights* w, const void* x, int32_t T,
                                float* logits, float* sgate_pre, hipStream_t s);
hipError_t launch_gating(const moe_config* c, const float* logits, const float* sgate_pre, int32_t T,
                         int32_t* topk_idx, float* topk_w, float* sgate, hipStream_t s);
hipError_t launch_permute(const moe_config* c, const int32_t* topk_idx, int32_t T, int32_t* offsets,
                          int32_t* sorted_assign, int32_t* assign_pos, int32_t* scratch, hipStream_t s);
hipError_t launch_expert_ffn(const moe_config* c, const moe_weights* w, const void* x, const int32_t* offsets,
                             const int32_t* sorted_assign, int32_t T, void* h, hipStream_t s);
hipError_t launch_down(const moe_config* c, const moe_weights* w, const void* h, const int32_t* offsets,
                       const int32_t* sorted_assign, int32_t T, float* y, hipStream_t s);
// y rows are indexed by assignment id a (routed a = t*k + j, shared a = T*k + t).
hipError_t launch_combine_gather(const moe_config* c, const float* y, const float* topk_w, const float* sgate,
                                 int32_t T, float* out, hipStream_t s);

}  // namespace moe
