/*
 * moe_abi_check.c -- the layer driven from plain C through include/moe.h.
 *
 * TEST PROGRAM.  It shows the boundary without Python or torch: device
 * buffers come from the HIP runtime, inputs from the seeded generator
 * (synth/libsynth.so), and every output is checked against the CPU oracle
 * (oracle/libmoe_ref.so, test infrastructure) on the same host copies.
 *
 * Two layers ("qwen35moe - Forward-Pass Design", section "Shared-expert MoE
 * FFN"; "Phase 19: MoE - gpt-oss-20b", sections 2 and 3):
 *   bf16   -- softmax -> top-k -> renormalise gating, SwiGLU experts and a
 *             shared expert behind a sigmoid gate;
 *   mxfp4  -- biased router, top-k -> softmax gating, MXFP4 interleaved
 *             gate_up and down with biases, clamped activation.
 * For each: moe_forward on the GPU; the oracle on the GPU's picks (a token
 * whose logits sit within rounding of a tie may pick differently, which is
 * counted and bounded); max|gpu - oracle| <= tol * max|oracle| over the
 * whole output.  Then the argument checks that run before any launch.
 *
 * Usage: moe_abi_check T_bf16 T_mxfp4   (prints one line per check; exit 0 on
 * success, 1 on a mismatch, 2 on a runtime error).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"
#include "moe_ref.h"

/* generator entry points (synth/synth.c) */
void synth_normal_bf16(uint32_t base, uint64_t stream0, double stddev, int64_t rows, int64_t cols, uint16_t* out);
void synth_bytes(uint32_t base, uint64_t stream0, int64_t rows, int64_t cols, uint8_t* out);
void synth_range_bytes(uint32_t base, uint64_t stream0, int64_t rows, int64_t cols, uint32_t lo, uint32_t span,
                       uint8_t* out);

#define SEED 0x9E3779B9u

static int g_fail = 0;

#define HIP_OK(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) {                                                            \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(2);                                                                         \
    }                                                                                  \
  } while (0)

/* a host buffer and its device copy */
typedef struct {
  void* h;
  void* d;
  size_t bytes;
} buf;

static buf buf_new(size_t bytes) {
  buf b;
  b.bytes = bytes;
  b.h = calloc(bytes ? bytes : 1, 1);
  if (!b.h) exit(2);
  HIP_OK(hipMalloc(&b.d, bytes ? bytes : 16));
  return b;
}
static void buf_up(buf* b) { HIP_OK(hipMemcpy(b->d, b->h, b->bytes, hipMemcpyHostToDevice)); }
static void buf_down(buf* b) { HIP_OK(hipMemcpy(b->h, b->d, b->bytes, hipMemcpyDeviceToHost)); }
static void buf_free(buf* b) {
  free(b->h);
  HIP_OK(hipFree(b->d));
}

/* bf16 normal draws: tensor id tid, rows x cols, stddev 1/sqrt(fan_in) */
static buf bf16_tensor(uint64_t tid, int64_t rows, int64_t cols, double stddev) {
  buf b = buf_new((size_t)rows * cols * 2);
  synth_normal_bf16(SEED, tid << 32, stddev, rows, cols, (uint16_t*)b.h);
  buf_up(&b);
  return b;
}

static ref_mat mat(int32_t dtype, const void* data, const uint8_t* scales) {
  ref_mat m;
  m.dtype = dtype;
  m.data = data;
  m.scales = scales;
  return m;
}

/* GPU layer against the oracle on the GPU's picks */
static void check_layer(const char* name, const moe_config* mc, const moe_weights* mw, const ref_cfg* rc,
                        const ref_weights* rw, buf* x, int32_t T, double tol) {
  const int32_t H = mc->hidden, k = mc->top_k;
  buf out = buf_new((size_t)T * H * 4), idx = buf_new((size_t)T * k * 4);
  const size_t wsb = moe_workspace_bytes(mc, T);
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, wsb ? wsb : 256));
  int st = moe_forward(mc, mw, x->d, T, (float*)out.d, NULL, (int32_t*)idx.d, NULL, NULL, ws, wsb, NULL);
  if (st != MOE_OK) {
    printf("%s T=%d: moe_forward returned %d (%s)\n", name, T, st, moe_status_string(st));
    g_fail = 1;
    return;
  }
  HIP_OK(hipDeviceSynchronize());
  buf_down(&out);
  buf_down(&idx);

  const ref_mat rx = mat(mc->x_dtype == MOE_DTYPE_BF16 ? REF_BF16 : REF_F32, x->h, NULL);
  float* ref = (float*)malloc((size_t)T * H * 4);
  int32_t* ref_idx = (int32_t*)malloc((size_t)T * k * 4);
  ref_forward(rc, rw, &rx, T, NULL, NULL, NULL, 0, ref, ref_idx, NULL, NULL);
  int moved = 0;
  for (int32_t t = 0; t < T; ++t)
    if (memcmp(ref_idx + (size_t)t * k, (const int32_t*)idx.h + (size_t)t * k, (size_t)k * 4)) ++moved;
  if (moved) /* the oracle on the GPU's picks, for every token */
    ref_forward(rc, rw, &rx, T, NULL, (const int32_t*)idx.h, NULL, 0, ref, NULL, NULL, NULL);
  double err = 0.0, scale = 0.0;
  const float* g = (const float*)out.h;
  for (size_t i = 0; i < (size_t)T * H; ++i) {
    const double d = fabs((double)g[i] - (double)ref[i]);
    if (!(d <= err)) err = d; /* NaN propagates as a failure */
    if (fabs((double)ref[i]) > scale) scale = fabs((double)ref[i]);
  }
  const int ok = err <= tol * scale && moved <= T / 20;
  printf("%s T=%d: max|err|/max|ref| = %.3e (tol %.0e), %d of %d tokens picked differently -> %s\n", name, T,
         scale > 0 ? err / scale : err, tol, moved, T, ok ? "ok" : "MISMATCH");
  if (!ok) g_fail = 1;
  free(ref);
  free(ref_idx);
  buf_free(&out);
  buf_free(&idx);
  HIP_OK(hipFree(ws));
}

/* qwen35moe-shaped (small): bf16, softmax-topk + renorm, SwiGLU, shared expert */
static void run_bf16(int32_t T) {
  const int32_t E = 16, H = 256, F = 128, Fs = 128, k = 4;
  buf x = bf16_tensor(1, T, H, 1.0), rw = bf16_tensor(2, E, H, 1.0 / sqrt(H));
  buf gw = bf16_tensor(4, (int64_t)E * F, H, 1.0 / sqrt(H)), uw = bf16_tensor(5, (int64_t)E * F, H, 1.0 / sqrt(H));
  buf dw = bf16_tensor(8, (int64_t)E * H, F, 1.0 / sqrt(F));
  buf sg = bf16_tensor(10, Fs, H, 1.0 / sqrt(H)), su = bf16_tensor(11, Fs, H, 1.0 / sqrt(H));
  buf sd = bf16_tensor(12, H, Fs, 1.0 / sqrt(Fs)), si = bf16_tensor(13, 1, H, 1.0 / sqrt(H));

  moe_config mc;
  memset(&mc, 0, sizeof mc);
  mc.hidden = H; mc.n_expert = E; mc.top_k = k; mc.expert_ff = F; mc.shared_ff = Fs;
  mc.gating = MOE_GATING_SOFTMAX_TOPK; mc.norm_topk_prob = 1; mc.weights_scale = 1.0f;
  mc.act = MOE_ACT_SWIGLU; mc.x_dtype = MOE_DTYPE_BF16; mc.w_dtype = MOE_DTYPE_BF16;
  mc.act_quant = MOE_ACT_QUANT_NONE;
  moe_weights mw;
  memset(&mw, 0, sizeof mw);
  mw.router_w = rw.d; mw.gate_w = gw.d; mw.up_w = uw.d; mw.down_w = dw.d;
  mw.sh_gate_w = sg.d; mw.sh_up_w = su.d; mw.sh_down_w = sd.d; mw.sh_gate_inp = si.d;

  ref_cfg rc;
  memset(&rc, 0, sizeof rc);
  rc.H = H; rc.E = E; rc.k = k; rc.F = F; rc.Fs = Fs; rc.gating = REF_SOFTMAX_TOPK; rc.norm_topk_prob = 1;
  rc.weights_scale = 1.0f; rc.act = REF_SWIGLU; rc.act_quant = REF_AQ_NONE;
  ref_weights rwt;
  memset(&rwt, 0, sizeof rwt);
  rwt.router_w = mat(REF_BF16, rw.h, NULL); rwt.gate_w = mat(REF_BF16, gw.h, NULL);
  rwt.up_w = mat(REF_BF16, uw.h, NULL); rwt.down_w = mat(REF_BF16, dw.h, NULL);
  rwt.sh_gate_w = mat(REF_BF16, sg.h, NULL); rwt.sh_up_w = mat(REF_BF16, su.h, NULL);
  rwt.sh_down_w = mat(REF_BF16, sd.h, NULL); rwt.sh_gate_inp = mat(REF_BF16, si.h, NULL);

  check_layer("bf16 (softmax-topk, SwiGLU, shared expert)", &mc, &mw, &rc, &rwt, &x, T, 2e-2);

  /* argument checks: nothing is launched */
  int st = moe_forward(NULL, &mw, x.d, T, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  int ok = st == MOE_EINVAL;
  moe_config bad = mc;
  bad.top_k = E + 1;
  ok = ok && moe_workspace_bytes(&bad, T) == 0;
  const size_t wsb = moe_workspace_bytes(&mc, T);
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, wsb + 512));
  buf out = buf_new((size_t)T * H * 4);
  st = moe_forward(&mc, &mw, x.d, T, (float*)out.d, NULL, NULL, NULL, NULL, ws, wsb - 256, NULL);
  ok = ok && st == MOE_EWORKSPACE;
  st = moe_forward(&mc, &mw, x.d, T, (float*)out.d, NULL, NULL, NULL, NULL, (char*)ws + 4, wsb, NULL);
  ok = ok && st == MOE_EWORKSPACE;
  st = moe_forward(&mc, &mw, (const char*)x.d + 2, T, (float*)out.d, NULL, NULL, NULL, NULL, ws, wsb, NULL);
  ok = ok && st == MOE_EINVAL;
  printf("argument checks (null config, k > E, short and misaligned workspace, misaligned x) -> %s\n",
         ok ? "ok" : "MISMATCH");
  if (!ok) g_fail = 1;
  HIP_OK(hipFree(ws));
  buf_free(&out);
  buf* all[] = {&x, &rw, &gw, &uw, &dw, &sg, &su, &sd, &si};
  for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i) buf_free(all[i]);
}

/* gpt-oss-shaped (small): MXFP4 experts, biased router, top-k -> softmax */
static void run_mxfp4(int32_t T) {
  const int32_t E = 8, H = 256, F = 128, k = 2;
  buf x = bf16_tensor(1, T, H, 1.0), rw = bf16_tensor(2, E, H, 1.0 / sqrt(H));
  buf rb = bf16_tensor(3, 1, E, 1.0 / sqrt(H));
  buf gub = bf16_tensor(7, E, 2 * F, 1.0 / sqrt(H)), db = bf16_tensor(9, E, H, 1.0 / sqrt(F));
  buf guc = buf_new((size_t)E * 2 * F * (H / 32) * 16), gus = buf_new((size_t)E * 2 * F * (H / 32));
  buf dc = buf_new((size_t)E * H * (F / 32) * 16), ds = buf_new((size_t)E * H * (F / 32));
  synth_bytes(SEED, (uint64_t)14 << 32, (int64_t)E * 2 * F * (H / 32), 16, (uint8_t*)guc.h);
  synth_range_bytes(SEED, (uint64_t)15 << 32, (int64_t)E * 2 * F, H / 32, 118, 13, (uint8_t*)gus.h);
  synth_bytes(SEED, (uint64_t)16 << 32, (int64_t)E * H * (F / 32), 16, (uint8_t*)dc.h);
  synth_range_bytes(SEED, (uint64_t)17 << 32, (int64_t)E * H, F / 32, 118, 13, (uint8_t*)ds.h);
  buf_up(&guc);
  buf_up(&gus);
  buf_up(&dc);
  buf_up(&ds);

  moe_config mc;
  memset(&mc, 0, sizeof mc);
  mc.hidden = H; mc.n_expert = E; mc.top_k = k; mc.expert_ff = F; mc.shared_ff = 0;
  mc.gating = MOE_GATING_TOPK_SOFTMAX; mc.norm_topk_prob = 0; mc.weights_scale = 1.0f;
  mc.act = MOE_ACT_SWIGLU_OAI; mc.act_alpha = 1.702f; mc.act_limit = 7.0f;
  mc.x_dtype = MOE_DTYPE_BF16; mc.w_dtype = MOE_DTYPE_MXFP4; mc.act_quant = MOE_ACT_QUANT_NONE;
  moe_weights mw;
  memset(&mw, 0, sizeof mw);
  mw.router_w = rw.d; mw.router_b = rb.d; mw.gate_up_w = guc.d; mw.gate_up_scales = (const uint8_t*)gus.d;
  mw.gate_up_b = gub.d; mw.down_w = dc.d; mw.down_scales = (const uint8_t*)ds.d; mw.down_b = db.d;

  ref_cfg rc;
  memset(&rc, 0, sizeof rc);
  rc.H = H; rc.E = E; rc.k = k; rc.F = F; rc.Fs = 0; rc.gating = REF_TOPK_SOFTMAX; rc.norm_topk_prob = 0;
  rc.weights_scale = 1.0f; rc.act = REF_SWIGLU_OAI; rc.alpha = 1.702f; rc.limit = 7.0f; rc.act_quant = REF_AQ_NONE;
  ref_weights rwt;
  memset(&rwt, 0, sizeof rwt);
  rwt.router_w = mat(REF_BF16, rw.h, NULL); rwt.router_b = mat(REF_BF16, rb.h, NULL);
  rwt.gate_up_w = mat(REF_MXFP4, guc.h, (const uint8_t*)gus.h); rwt.gate_up_b = mat(REF_BF16, gub.h, NULL);
  rwt.down_w = mat(REF_MXFP4, dc.h, (const uint8_t*)ds.h); rwt.down_b = mat(REF_BF16, db.h, NULL);

  check_layer("mxfp4 (biased router, topk-softmax, clamped interleaved SwiGLU)", &mc, &mw, &rc, &rwt, &x, T, 3e-2);
  buf* all[] = {&x, &rw, &rb, &gub, &db, &guc, &gus, &dc, &ds};
  for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i) buf_free(all[i]);
}

int main(int argc, char** argv) {
  const int32_t tb = argc > 1 ? atoi(argv[1]) : 37, tm = argc > 2 ? atoi(argv[2]) : 150;
  int n = 0;
  HIP_OK(hipGetDeviceCount(&n));
  if (n < 1) {
    fprintf(stderr, "no GPU\n");
    return 2;
  }
  HIP_OK(hipSetDevice(0));
  run_bf16(tb);
  run_mxfp4(tm);
  printf("%s\n", g_fail ? "FAILED" : "all checks passed");
  return g_fail ? 1 : 0;
}
