// RMSNorm prologue of the layer inside its decoder block.
//
// The block is pre-norm with a residual: the layer's input is the residual
// stream normalised by its root mean square and scaled by the norm weight,
// and the layer's output is added to the un-normalised stream
// ("qwen35moe - Forward-Pass Design (Pantheon port)", section "Block
// scaffold"; "Phase 19: MoE - gpt-oss-20b", section 2, RMSNorm and decoder
// layer).  Per token row:
//   y[h] = x[h] * g[h] / sqrt(mean(x^2) + eps)
// with the statistics in fp32 (the gpt-oss page fixes the variance in fp32)
// and y rounded once to the activation type that the router and the experts
// then read.  The residual add sits in the combine kernel (ffn_gemv.hip).
//
// One wavefront per row: a row of up to 4096 bf16 (2048 fp32) values is at
// most 8 16-byte pieces per lane, held in registers between the sum of
// squares and the scaling, so x is read once.
#include "gating.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kNormWaves = 4;    // rows per workgroup
constexpr int kNormPieces = 8;   // 16-byte pieces per lane at most

template <typename XT>
__global__ __launch_bounds__(kNormWaves * kWave) void k_rmsnorm(const XT* __restrict__ x, const XT* __restrict__ g,
                                                               float eps, int32_t T, int32_t H,
                                                               XT* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kNormWaves + threadIdx.x / kWave;
  if (t >= T) return;
  constexpr int N = 16 / sizeof(XT);
  const int np = H / N;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  uint4 v[kNormPieces];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormPieces; ++i) {
    const int pc = lane + i * kWave;
    v[i] = pc < np ? xr[pc] : make_uint4(0, 0, 0, 0);
    ss += sumsq4(v[i], XT());
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)H + eps);
  const uint4* gr = reinterpret_cast<const uint4*>(g);
  uint4* yr = reinterpret_cast<uint4*>(y + (size_t)t * H);
#pragma unroll
  for (int i = 0; i < kNormPieces; ++i) {
    const int pc = lane + i * kWave;
    if (pc < np) yr[pc] = scale4(v[i], gr[pc], r, XT());
  }
}

}  // namespace

hipError_t launch_rmsnorm(const moe_config* c, const void* x, const void* g, float eps, int32_t T, void* y,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kNormWaves - 1) / kNormWaves);
  if (c->x_dtype == MOE_DTYPE_BF16)
    k_rmsnorm<uint16_t><<<grid, kNormWaves * kWave, 0, s>>>((const uint16_t*)x, (const uint16_t*)g, eps, T,
                                                            c->hidden, (uint16_t*)y);
  else
    k_rmsnorm<float><<<grid, kNormWaves * kWave, 0, s>>>((const float*)x, (const float*)g, eps, T, c->hidden,
                                                         (float*)y);
  return hipGetLastError();
}

}  // namespace moe
