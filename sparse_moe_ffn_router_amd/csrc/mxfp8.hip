// MXFP8 rounding of expert GEMM inputs (activations rounded to E4M3
// elements with one E8M0 scale per 32 along the input dimension, before a
// routed expert's product consumes them).
//
// The rule is the OCP Microscaling Formats spec v1.0, section 6.3: per block
// of 32 values the shared exponent is floor(log2(max |v|)) minus 8 (the
// largest E4M3 exponent), kept in [-127, 127]; each element is v / 2^shared
// rounded to the nearest E4M3 value, ties to the even mantissa, magnitudes
// beyond 448 saturated.  Every step is exact in fp32 for bf16 inputs (a
// power-of-two scaling and one round-to-nearest-even), so the codes do not
// depend on evaluation order.
//
// Two outputs: E4M3 codes [rows][K] with scales [rows][Kp/32] (Kp = K
// rounded up to 128, so one 4-byte word per row holds a 128-deep K step's
// four scales) for the MFMA path, or the rounded values themselves as bf16
// (every E4M3 value times a power of two is exact in bf16) for the
// few-token kernels, which take bf16 activations.
//
// MXFP4 is the pages' native weight format ("Phase 19: MoE - gpt-oss-20b",
// section 3); computing the expert products on MX MFMA with MXFP8 inputs is
// this library's reading of running those weights natively.
#include "moe_internal.hpp"

namespace moe {
namespace {

// E4M3 code of v = x / 2^shared (|v| < 512).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = v < 0.f ? 0x80u : 0u;  // -0 encodes as +0
  const float a = fabsf(v);
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.f);  // step 2^-9; 8 is 2^-6
  const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  uint32_t m = (uint32_t)(__builtin_rintf(__builtin_ldexpf(a, 3 - e)) - 8.f);  // 0..8
  int ex = e + 7;
  if (m == 8u) {
    m = 0u;
    ++ex;
  }
  return sign | ((uint32_t)ex << 3) | m;
}

// Value of an E4M3 code (no NaN codes are produced above).
__device__ __forceinline__ float e4m3_float(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, m = c & 7u;
  const float mag = ex ? __builtin_ldexpf(1.f + (float)m * 0.125f, (int)ex - 7) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// One thread per 32-element block of a bf16 [rows][K] matrix.
template <bool CODES>
__global__ __launch_bounds__(256) void k_mxfp8_round(const uint16_t* __restrict__ src, int64_t nblk, int K,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                     int sstride, uint16_t* __restrict__ dst) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblk) return;
  const int bpr = K / 32;
  const int64_t row = b / bpr;
  const int col = (int)(b - row * bpr) * 32;
  const uint4* s = reinterpret_cast<const uint4*>(src + row * K + col);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = s[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(w[i])), fabsf(bf16hi(w[i]))));
  int sh = -127;
  if (amax > 0.f) {
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
    sh = ef == 0 ? -127 : ef - 127 - 8;
    sh = sh < -127 ? -127 : (sh > 127 ? 127 : sh);
  }
  uint32_t c[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    c[2 * i] = e4m3_code(__builtin_ldexpf(bf16lo(w[i]), -sh));
    c[2 * i + 1] = e4m3_code(__builtin_ldexpf(bf16hi(w[i]), -sh));
  }
  if (CODES) {
    uint4* d = reinterpret_cast<uint4*>(codes + row * K + col);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 16 * i + 4 * j;
        q[j] = c[e] | (c[e + 1] << 8) | (c[e + 2] << 16) | (c[e + 3] << 24);
      }
      d[i] = make_uint4(q[0], q[1], q[2], q[3]);
    }
    scales[row * sstride + col / 32] = (uint8_t)(sh + 127);
  } else {
    uint4* d = reinterpret_cast<uint4*>(dst + row * K + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 8 * i + 2 * j;
        const uint32_t lo = __float_as_uint(__builtin_ldexpf(e4m3_float(c[e]), sh)) >> 16;
        const uint32_t hi = __float_as_uint(__builtin_ldexpf(e4m3_float(c[e + 1]), sh)) >> 16;
        q[j] = lo | (hi << 16);
      }
      d[i] = make_uint4(q[0], q[1], q[2], q[3]);
    }
  }
}

}  // namespace

int mx8_scale_stride(int K) { return ((K + 127) / 128) * 4; }

hipError_t launch_mxfp8_codes(const uint16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const int64_t nblk = rows * (K / 32);
  if (nblk == 0) return hipSuccess;
  k_mxfp8_round<true><<<(unsigned)((nblk + 255) / 256), 256, 0, s>>>(src, nblk, K, codes, scales,
                                                                     mx8_scale_stride(K), nullptr);
  return hipGetLastError();
}

hipError_t launch_mxfp8_values(const uint16_t* src, int64_t rows, int K, uint16_t* dst, hipStream_t s) {
  const int64_t nblk = rows * (K / 32);
  if (nblk == 0) return hipSuccess;
  k_mxfp8_round<false><<<(unsigned)((nblk + 255) / 256), 256, 0, s>>>(src, nblk, K, nullptr, nullptr, 0, dst);
  return hipGetLastError();
}

}  // namespace moe
