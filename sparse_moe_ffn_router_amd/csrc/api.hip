// C entry points of libmoe: host-side argument checks, the workspace plan
// and the launch sequence of each step.  No allocation, no synchronisation.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moe_internal.hpp"

namespace moe {

bool mfma_shapes_ok(const moe_config* c);  // ffn_mfma.hip

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_config(const moe_config* c) {
  if (!c) return MOE_EINVAL;
  if (c->hidden <= 0 || c->n_expert <= 0 || c->top_k <= 0 || c->expert_ff <= 0 || c->shared_ff < 0)
    return MOE_EINVAL;
  if (c->n_expert > kMaxExperts || c->top_k > kMaxTopK || c->top_k > c->n_expert) return MOE_EINVAL;
  if (c->gating != MOE_GATING_SOFTMAX_TOPK && c->gating != MOE_GATING_TOPK_SOFTMAX) return MOE_EINVAL;
  if (c->act != MOE_ACT_SWIGLU && c->act != MOE_ACT_SWIGLU_OAI) return MOE_EINVAL;
  if (c->x_dtype != MOE_DTYPE_F32 && c->x_dtype != MOE_DTYPE_BF16) return MOE_EINVAL;
  if (c->w_dtype != MOE_DTYPE_F32 && c->w_dtype != MOE_DTYPE_BF16 && c->w_dtype != MOE_DTYPE_MXFP4)
    return MOE_EINVAL;
  if (c->hidden % 32 || c->expert_ff % 32 || c->shared_ff % 32) return MOE_EUNSUPPORTED;
  // rows of at most 8 x 64 16-byte pieces per lane set in the few-token kernels
  const int dmax = c->x_dtype == MOE_DTYPE_F32 ? 2048 : 4096;
  if (c->hidden > dmax || c->expert_ff > dmax || c->shared_ff > dmax) return MOE_EUNSUPPORTED;
  if (c->x_dtype == MOE_DTYPE_F32 && c->w_dtype != MOE_DTYPE_F32) return MOE_EUNSUPPORTED;
  if (c->x_dtype == MOE_DTYPE_BF16 && c->w_dtype == MOE_DTYPE_F32) return MOE_EUNSUPPORTED;
  // MXFP4 experts come in the fused interleaved gate_up layout only
  if (c->w_dtype == MOE_DTYPE_MXFP4 && c->act != MOE_ACT_SWIGLU_OAI) return MOE_EUNSUPPORTED;
  if (c->act_quant != MOE_ACT_QUANT_NONE && c->act_quant != MOE_ACT_QUANT_MXFP8) return MOE_EINVAL;
  if (c->act_quant == MOE_ACT_QUANT_MXFP8 &&
      (c->w_dtype != MOE_DTYPE_MXFP4 || c->x_dtype != MOE_DTYPE_BF16 || c->shared_ff != 0 || c->hidden % 64 ||
       c->expert_ff % 64))
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

static size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

int make_plan(const moe_config* c, int32_t T, Plan* p) {
  int st = check_config(c);
  if (st) return st;
  if (T < 0) return MOE_EINVAL;
  memset(p, 0, sizeof(*p));
  p->T = T; p->H = c->hidden; p->E = c->n_expert; p->k = c->top_k; p->F = c->expert_ff; p->Fs = c->shared_ff;
  p->shared = c->shared_ff > 0;
  p->n_assign = (int64_t)T * c->top_k;
  p->n_rows = p->n_assign + (p->shared ? T : 0);
  p->nseg = c->n_expert + p->shared;
  p->elem_x = c->x_dtype == MOE_DTYPE_BF16 ? 2 : 4;
  p->perm_bytes = up256(permute_scratch_bytes(T, c->n_expert, c->top_k));
  p->y_bytes = up256((size_t)p->n_rows * c->hidden * 4);
  size_t o = 0;
  p->off_logits = o; o += up256((size_t)T * c->n_expert * 4);
  p->off_idx = o; o += up256((size_t)p->n_assign * 4);
  p->off_w = o; o += up256((size_t)p->n_assign * 4);
  p->off_sgate = o; o += up256((size_t)T * 4);
  p->off_offsets = o; o += up256((size_t)(p->nseg + 1) * 4);
  p->off_sorted = o; o += up256((size_t)p->n_rows * 4);
  p->off_pos = o; o += up256((size_t)p->n_rows * 4);
  p->nslots = can_fuse_gate_permute(T) ? gemv_slots(c, T) : 0;
  p->off_segtab = o; o += up256((size_t)p->nslots * 16);
  p->off_perm = o; o += p->perm_bytes;
  p->off_h = o; o += up256((size_t)(p->n_assign * c->expert_ff + (p->shared ? (int64_t)T * c->shared_ff : 0)) * p->elem_x);
  p->off_y = o; o += p->y_bytes;
  p->nsplit = 1;
  if (T > kGemvMaxT && mfma_shapes_ok(c)) {
    int steps;
    router_split(c, T, &p->nsplit, &steps);
  }
  p->off_part = o; o += p->nsplit > 1 ? up256((size_t)p->nsplit * T * c->n_expert * 4) : 0;
  if (c->act_quant == MOE_ACT_QUANT_MXFP8) {
    // bf16 values (2 bytes per element) cover the E4M3 codes (1 byte) too
    p->mx8 = T > kGemvMaxT && mfma_shapes_ok(c);
    p->aqx_scales = up256((size_t)T * c->hidden * 2);
    p->aqx_bytes = p->aqx_scales + up256((size_t)T * mx8_scale_stride(c->hidden));
    p->aqh_scales = up256((size_t)p->n_assign * c->expert_ff * 2);
    p->aqh_bytes = p->aqh_scales + up256((size_t)p->n_assign * mx8_scale_stride(c->expert_ff));
  }
  p->off_aqx = o; o += p->aqx_bytes;
  p->off_aqh = o; o += p->aqh_bytes;
  // moe_forward_prenorm: the normalised rows when the caller does not take them
  p->off_xn = o; o += up256((size_t)T * c->hidden * p->elem_x);
  p->total = o;
  // Buffer descriptors hold 32-bit extents: every kernel addresses the
  // token rows x through one (router product, gate/up); the few-token
  // kernels address all of h through one; the MX MFMA path addresses the
  // MXFP8 codes of h ([T*k][F] bytes) through one.  Larger batches are
  // rejected here rather than wrapped on the device.
  const size_t lim = (size_t)1 << 31;
  const size_t act_bytes = (size_t)(p->n_assign * c->expert_ff + (p->shared ? (int64_t)T * c->shared_ff : 0)) * p->elem_x;
  if ((size_t)T * c->hidden * p->elem_x >= lim) return MOE_EUNSUPPORTED;
  if (!(T > kGemvMaxT && mfma_shapes_ok(c)) && act_bytes >= lim) return MOE_EUNSUPPORTED;
  if (p->mx8 && (size_t)p->n_assign * c->expert_ff >= lim) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

static int weights_ok(const moe_config* c, const moe_weights* w, bool need_router, bool need_experts) {
  if (!w) return MOE_EINVAL;
  const void* ptrs[14] = {w->router_w, w->router_b, w->gate_w, w->up_w, w->gate_up_w, w->gate_up_scales,
                          w->gate_up_b, w->down_w, w->down_scales, w->down_b, w->sh_gate_w, w->sh_up_w,
                          w->sh_down_w, w->sh_gate_inp};
  for (int i = 0; i < 14; ++i)
    if (ptrs[i] && !aligned16(ptrs[i])) return MOE_EINVAL;
  if (need_router && c->shared_ff > 0 && !w->sh_gate_inp) return MOE_EINVAL;
  if (need_experts) {
    if (c->act == MOE_ACT_SWIGLU && (!w->gate_w || !w->up_w || !w->down_w)) return MOE_EINVAL;
    if (c->act == MOE_ACT_SWIGLU_OAI && (!w->gate_up_w || !w->down_w)) return MOE_EINVAL;
    if (c->w_dtype == MOE_DTYPE_MXFP4 && (!w->gate_up_scales || !w->down_scales)) return MOE_EINVAL;
    if (c->shared_ff > 0 && (!w->sh_gate_w || !w->sh_up_w || !w->sh_down_w)) return MOE_EINVAL;
  }
  return MOE_OK;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Gate/up with the routed experts' input x rounded to MXFP8 in aq (aqx_bytes).
static hipError_t expert_ffn_aq(const moe_config* c, const moe_weights* w, const Plan& p, const void* x,
                                const int32_t* offsets, const int32_t* sorted, int32_t T, void* h, char* aq,
                                hipStream_t s) {
  hipError_t e;
  if (p.mx8) {
    uint8_t* codes = (uint8_t*)aq;
    uint8_t* scales = (uint8_t*)(aq + p.aqx_scales);
    if ((e = launch_mxfp8_codes((const uint16_t*)x, T, c->hidden, codes, scales, s)) != hipSuccess) return e;
    return launch_gateup_mx8(c, w, codes, scales, offsets, sorted, T, h, s);
  }
  if ((e = launch_mxfp8_values((const uint16_t*)x, T, c->hidden, (uint16_t*)aq, s)) != hipSuccess) return e;
  return launch_expert_ffn(c, w, aq, offsets, sorted, T, h, s);
}

// Down with h rounded to MXFP8 in aq (aqh_bytes); y as launch_down writes it.
static hipError_t down_aq(const moe_config* c, const moe_weights* w, const Plan& p, const void* h,
                          const int32_t* offsets, const int32_t* sorted, int32_t T, void* y, char* aq, hipStream_t s) {
  hipError_t e;
  if (p.mx8) {
    uint8_t* codes = (uint8_t*)aq;
    uint8_t* scales = (uint8_t*)(aq + p.aqh_scales);
    if ((e = launch_mxfp8_codes((const uint16_t*)h, p.n_assign, c->expert_ff, codes, scales, s)) != hipSuccess)
      return e;
    return launch_down_mx8(c, w, codes, scales, offsets, sorted, T, (uint16_t*)y, s);
  }
  if ((e = launch_mxfp8_values((const uint16_t*)h, p.n_assign, c->expert_ff, (uint16_t*)aq, s)) != hipSuccess)
    return e;
  return launch_down(c, w, aq, offsets, sorted, T, y, s);
}

// The pre-norm block's prologue and epilogue: norm weight, eps and the
// residual rows (which the layer's input x is normalised from).
struct PreNorm {
  const void* g;
  float eps;
  const void* resid;
};

// The layer's launch sequence on checked arguments: route, permute, expert
// FFN, down, combine.  With pn, x is where the normalised rows go: few
// tokens normalise inside the router-product kernel, larger batches in an
// RMSNorm launch of their own; the combine adds pn->resid.
static int forward_steps(const moe_config* cfg, const moe_weights* w, const Plan& p, const void* x,
                         const PreNorm* pn, int32_t T, float* out, float* logits, int32_t* topk_idx, float* topk_w,
                         float* sgate, char* b, hipStream_t stream) {
  float* lg = logits ? logits : (float*)(b + p.off_logits);
  int32_t* idx = topk_idx ? topk_idx : (int32_t*)(b + p.off_idx);
  float* wt = topk_w ? topk_w : (float*)(b + p.off_w);
  float* sg = p.shared ? (sgate ? sgate : (float*)(b + p.off_sgate)) : nullptr;
  int32_t* offsets = (int32_t*)(b + p.off_offsets);
  int32_t* sorted = (int32_t*)(b + p.off_sorted);
  int32_t* pos = (int32_t*)(b + p.off_pos);
  int32_t* perm = (int32_t*)(b + p.off_perm);
  void* h = b + p.off_h;
  void* y = b + p.off_y;
  // MFMA router product split over K ranges, summed by the gating kernel
  float* part = (p.nsplit > 1 && w->router_w) ? (float*)(b + p.off_part) : nullptr;
  hipError_t e;
  if (pn && router_norm_fusable(cfg, w, T)) {
    e = launch_router_logits_norm(cfg, w, pn->resid, pn->g, pn->eps, T, const_cast<void*>(x), lg, sg, stream);
  } else {
    if (pn && (e = launch_rmsnorm(cfg, pn->resid, pn->g, pn->eps, T, const_cast<void*>(x), stream)) != hipSuccess)
      return MOE_EHIP;
    e = launch_router_logits(cfg, w, x, T, lg, sg, stream, part);
  }
  if (e != hipSuccess) return MOE_EHIP;
  int32_t* segtab = nullptr;
  if (can_fuse_gate_permute(T)) {
    if (p.nslots) segtab = (int32_t*)(b + p.off_segtab);
    if ((e = launch_gate_permute(cfg, lg, sg, T, idx, wt, sg, offsets, sorted, pos, stream, segtab, p.nslots)) !=
        hipSuccess)
      return MOE_EHIP;
  } else {
    if ((e = launch_gating(cfg, w, x, lg, sg, T, idx, wt, sg, stream, part, part ? p.nsplit : 1)) != hipSuccess)
      return MOE_EHIP;
    if ((e = launch_permute(cfg, idx, T, offsets, sorted, pos, perm, stream)) != hipSuccess) return MOE_EHIP;
  }
  if (cfg->act_quant == MOE_ACT_QUANT_MXFP8) {
    if ((e = expert_ffn_aq(cfg, w, p, x, offsets, sorted, T, h, b + p.off_aqx, stream)) != hipSuccess) return MOE_EHIP;
    if ((e = down_aq(cfg, w, p, h, offsets, sorted, T, y, b + p.off_aqh, stream)) != hipSuccess) return MOE_EHIP;
  } else {
    if ((e = launch_expert_ffn(cfg, w, x, offsets, sorted, T, h, stream, segtab)) != hipSuccess) return MOE_EHIP;
    if ((e = launch_down(cfg, w, h, offsets, sorted, T, y, stream, segtab)) != hipSuccess) return MOE_EHIP;
  }
  return hip_status(launch_combine_gather(cfg, y, wt, sg, T, out, stream, pn ? pn->resid : nullptr));
}

// Scratch of moe_forward_noalloc: one file-scope device array, which every
// GPU the library runs on holds (its own copy, at its own address) until
// the process ends.  In host code the array's name is only a stand-in for
// that address: each device's address is taken once, with the device
// current, through hipGetSymbolAddress and kept in scratch_ptr; host code
// passes only that pointer on.  Nothing in the forward pass needs its
// scratch to start at zero (every workspace area is written before it is
// read), so the contents the previous call left do not matter.
static __device__ __attribute__((aligned(256))) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void* scratch_ptr[kMaxDevices];

static int scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    scratch_ptr[dev] = p;
  }
  *out = (char*)scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_config* cfg, int32_t T) {
  Plan p;
  if (make_plan(cfg, T, &p)) return 0;
  return p.total;
}

int moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)) return MOE_EINVAL;
  return hip_status(launch_mxfp8_codes((const uint16_t*)x, rows, K, codes, scales, stream));
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null or misaligned pointer, bad shape or enum)";
    case MOE_EUNSUPPORTED: return "unsupported dtype or shape combination";
    case MOE_EWORKSPACE: return "workspace too small or misaligned";
    case MOE_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int moe_route(const moe_config* cfg, const moe_weights* w, const void* x, float* logits, int32_t* topk_idx,
              float* topk_w, float* sgate, int32_t T, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_config(cfg);
  if (st) return st;
  if (T < 0) return MOE_EINVAL;
  if ((st = weights_ok(cfg, w, true, false))) return st;
  if (T == 0) return MOE_OK;
  const bool shared = cfg->shared_ff > 0;
  if (!logits || !topk_idx || !topk_w || !aligned16(logits)) return MOE_EINVAL;
  if ((w->router_w || shared) && (!x || !aligned16(x))) return MOE_EINVAL;
  if (shared && !sgate) return MOE_EINVAL;
  Plan p = {};
  p.nsplit = 1;
  if (ws) {
    if ((st = make_plan(cfg, T, &p))) return st;
    if (ws_bytes < p.total || ((uintptr_t)ws & 255u)) return MOE_EWORKSPACE;
  }
  // split router product: partial sums in the workspace's partials area
  float* part = (ws && p.nsplit > 1 && w->router_w) ? (float*)((char*)ws + p.off_part) : nullptr;
  // the pre-sigmoid shared-gate dot is staged in sgate itself
  hipError_t e = launch_router_logits(cfg, w, x, T, logits, sgate, stream, part);
  if (e != hipSuccess) return MOE_EHIP;
  return hip_status(
      launch_gating(cfg, w, x, logits, sgate, T, topk_idx, topk_w, sgate, stream, part, part ? p.nsplit : 1));
}

int moe_permute(const moe_config* cfg, const int32_t* topk_idx, int32_t T, int32_t* offsets, int32_t* sorted_assign,
                int32_t* assign_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, T, &p);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (!offsets || !topk_idx || !sorted_assign || !assign_pos) return MOE_EINVAL;
  if (T > kPermSmallTokens && (!ws || ws_bytes < p.perm_bytes || ((uintptr_t)ws & 255u))) return MOE_EWORKSPACE;
  return hip_status(launch_permute(cfg, topk_idx, T, offsets, sorted_assign, assign_pos, (int32_t*)ws, stream));
}

int moe_expert_ffn(const moe_config* cfg, const moe_weights* w, const void* x, const int32_t* offsets,
                   const int32_t* sorted_assign, int32_t T, void* h, void* ws, size_t ws_bytes, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, T, &p);
  if (st) return st;
  if ((st = weights_ok(cfg, w, false, true))) return st;
  if (T == 0) return MOE_OK;
  if (!x || !offsets || !sorted_assign || !h || !aligned16(x) || !aligned16(h)) return MOE_EINVAL;
  if (cfg->act_quant == MOE_ACT_QUANT_MXFP8) {
    if (!ws || ws_bytes < p.aqx_bytes || ((uintptr_t)ws & 255u)) return MOE_EWORKSPACE;
    return hip_status(expert_ffn_aq(cfg, w, p, x, offsets, sorted_assign, T, h, (char*)ws, stream));
  }
  return hip_status(launch_expert_ffn(cfg, w, x, offsets, sorted_assign, T, h, stream));
}

int moe_combine(const moe_config* cfg, const moe_weights* w, const void* h, const int32_t* offsets,
                const int32_t* sorted_assign, const float* topk_w, const float* sgate, int32_t T, float* out, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, T, &p);
  if (st) return st;
  if ((st = weights_ok(cfg, w, false, true))) return st;
  if (T == 0) return MOE_OK;
  if (!h || !offsets || !sorted_assign || !topk_w || !out || !aligned16(h) || !aligned16(out)) return MOE_EINVAL;
  if (p.shared && !sgate) return MOE_EINVAL;
  if (!ws || ws_bytes < p.y_bytes + p.aqh_bytes || ((uintptr_t)ws & 255u)) return MOE_EWORKSPACE;
  void* y = ws;
  hipError_t e = cfg->act_quant == MOE_ACT_QUANT_MXFP8
                     ? down_aq(cfg, w, p, h, offsets, sorted_assign, T, y, (char*)ws + p.y_bytes, stream)
                     : launch_down(cfg, w, h, offsets, sorted_assign, T, y, stream);
  if (e != hipSuccess) return MOE_EHIP;
  return hip_status(launch_combine_gather(cfg, y, topk_w, sgate, T, out, stream));
}

int moe_forward(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T, float* out, float* logits,
                int32_t* topk_idx, float* topk_w, float* sgate, void* ws, size_t ws_bytes, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, T, &p);
  if (st) return st;
  if ((st = weights_ok(cfg, w, true, true))) return st;
  if (T == 0) return MOE_OK;
  if (!x || !out || !aligned16(x) || !aligned16(out)) return MOE_EINVAL;
  if (!w->router_w && !logits) return MOE_EINVAL;
  if (logits && !aligned16(logits)) return MOE_EINVAL;
  if (!ws || ws_bytes < p.total || ((uintptr_t)ws & 255u)) return MOE_EWORKSPACE;
  return forward_steps(cfg, w, p, x, nullptr, T, out, logits, topk_idx, topk_w, sgate, (char*)ws, stream);
}

int moe_forward_prenorm(const moe_config* cfg, const moe_weights* w, const void* norm_w, float norm_eps,
                        const void* resid, int32_t T, float* out, void* xn, float* logits, int32_t* topk_idx,
                        float* topk_w, float* sgate, void* ws, size_t ws_bytes, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, T, &p);
  if (st) return st;
  if ((st = weights_ok(cfg, w, true, true))) return st;
  if (!(norm_eps >= 0.f) || norm_eps > 1.f) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!norm_w || !resid || !out || !aligned16(norm_w) || !aligned16(resid) || !aligned16(out)) return MOE_EINVAL;
  if (xn && !aligned16(xn)) return MOE_EINVAL;
  if (!w->router_w && !logits) return MOE_EINVAL;
  if (logits && !aligned16(logits)) return MOE_EINVAL;
  if (!ws || ws_bytes < p.total || ((uintptr_t)ws & 255u)) return MOE_EWORKSPACE;
  char* b = (char*)ws;
  const PreNorm pn = {norm_w, norm_eps, resid};
  return forward_steps(cfg, w, p, xn ? xn : b + p.off_xn, &pn, T, out, logits, topk_idx, topk_w, sgate, b, stream);
}

int moe_forward_noalloc(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T, float* out,
                        float* logits, int32_t* topk_idx, float* topk_w, float* sgate, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, T, &p);
  if (st) return st;
  if ((st = weights_ok(cfg, w, true, true))) return st;
  if (T == 0) return MOE_OK;
  if (!x || !out || !aligned16(x) || !aligned16(out)) return MOE_EINVAL;
  if (!w->router_w && !logits) return MOE_EINVAL;
  if (logits && !aligned16(logits)) return MOE_EINVAL;
  if (p.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  char* b = nullptr;
  if ((st = scratch_of_current_device(&b))) return st;
  return forward_steps(cfg, w, p, x, nullptr, T, out, logits, topk_idx, topk_w, sgate, b, stream);
}

}  // extern "C"
