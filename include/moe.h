/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts FFN layer.
 *
 * The layer, as stated in "qwen35moe - Forward-Pass Design (Pantheon port)",
 * section "Shared-expert MoE FFN (every layer)", and in "Phase 19: MoE -
 * gpt-oss-20b", section 2 (Router, Experts):
 *
 *   logits[t][e] = x[t] . router_w[e] (+ router_b[e])                 (fp32)
 *   gating       = softmax over all experts -> top-k -> renormalise -> * scale
 *                  (qwen35moe), or top-k -> softmax over the k picks (gpt-oss);
 *                  top-k keeps the first-seen (lowest-index) expert on ties
 *                  ("qwen35moe CPU-reference golden vectors", Kernel 4)
 *   h            = silu(gate_w[e] x) * (up_w[e] x)                    (SwiGLU)
 *                  or, with fused interleaved gate_up rows and bias,
 *                  (clamp(up,-L,L) + 1) * min(gate,L) * sigmoid(a*min(gate,L))
 *   out[t]       = sum_j w[t][j] (down_w[e_j] h + down_b[e_j])
 *                  + sigmoid(sh_gate_inp . x[t]) * SwiGLU_shared(x[t])
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or synchronises.  Each call enqueues
 *     its kernels on `stream` (NULL = the default stream) and returns
 *     before they run.  Calls are reentrant; the library holds no state.
 *   - Matrices are row-major [out][in] ("y = x W^T"), experts outermost.
 *   - Scratch memory is the caller's `ws` buffer of `ws_bytes` bytes
 *     (size from moe_workspace_bytes); it must be 256-byte aligned.
 *   - Every argument is checked on the host before any launch.  A non-zero
 *     return means nothing was enqueued (except MOE_EHIP, a launch error
 *     reported by the HIP runtime after enqueueing).
 *   - Shapes: hidden, expert_ff and shared_ff must be multiples of 32;
 *     1 <= top_k <= min(n_expert, 32); n_expert <= 1024; T >= 0 (T = 0 is a
 *     no-op that returns MOE_OK).  Tensor pointers must be 16-byte aligned.
 *     A batch whose token rows x pass 2 GiB (T * hidden * element size),
 *     or, with act_quant, whose MXFP8 codes of h pass 2 GiB (T * top_k *
 *     expert_ff bytes), is refused with MOE_EUNSUPPORTED (the kernels
 *     address them through 32-bit buffer extents).
 *   - Dtypes: x, router, biases and the shared expert share `x_dtype`
 *     (F32 or BF16); routed expert matrices use `w_dtype`: F32 with F32 x,
 *     BF16 or MXFP4 with BF16 x.  Logits, routing weights, the shared gate
 *     and `out` are fp32.
 *   - act_quant = MOE_ACT_QUANT_MXFP8 (MXFP4 experts only): the routed
 *     experts' GEMM inputs (x for gate/up, h for down) are rounded to MXFP8
 *     before each product, which then runs on the scaled MX MFMA.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK 0
#define MOE_EINVAL (-1)      /* null or misaligned pointer, bad shape or enum */
#define MOE_EUNSUPPORTED (-2) /* valid but unsupported dtype/shape combination */
#define MOE_EWORKSPACE (-3)  /* ws too small or misaligned */
#define MOE_EHIP (-4)        /* the HIP runtime reported a launch error */

/* Element types. */
#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1
/* MXFP4 (OCP MX v1.0): E2M1 codes, two per byte, low nibble = even index,
 * 32-element blocks along the input dim stored as [rows][in/32][16] bytes,
 * plus one E8M0 exponent byte per block [rows][in/32]; value =
 * e2m1(code) * 2^(e8m0 - 127) ("Phase 19: MoE - gpt-oss-20b", section 3 and
 * the tensor-layout listing).  E8M0 = 255 (NaN) is outside the contract. */
#define MOE_DTYPE_MXFP4 2

/* Precision of the routed experts' GEMM inputs.  MXFP8 (OCP MX v1.0):
 * E4M3 elements with one E8M0 scale per 32 along the input dimension, the
 * scale 2^(floor(log2(max|v|)) - 8), elements rounded to nearest (ties to
 * even) and saturated at 448.  Requires w_dtype MXFP4, x_dtype BF16, no
 * shared expert, and hidden, expert_ff multiples of 64 (MOE_EUNSUPPORTED
 * otherwise).  MXFP4 is the weight format the gpt-oss page ("Phase 19: MoE -
 * gpt-oss-20b", section 3) ships; this mode runs those weights natively. */
#define MOE_ACT_QUANT_NONE 0
#define MOE_ACT_QUANT_MXFP8 1

/* Gating ("qwen35moe - Forward-Pass Design", Shared-expert MoE FFN;
 * "Phase 19: MoE - gpt-oss-20b", section 2 Router). */
#define MOE_GATING_SOFTMAX_TOPK 0 /* softmax over E, top-k, optional renorm, * scale */
#define MOE_GATING_TOPK_SOFTMAX 1 /* top-k of the (biased) logits, softmax of the k, * scale */

/* Expert activation. */
#define MOE_ACT_SWIGLU 0     /* separate gate_w / up_w, no biases */
#define MOE_ACT_SWIGLU_OAI 1 /* fused gate_up_w, rows interleaved (even = gate,
                                odd = up), gate_up_b and down_b biases, gate
                                clamped above at act_limit, up clamped to
                                [-act_limit, act_limit], h = (up + 1) * gate *
                                sigmoid(act_alpha * gate) */

typedef struct {
  int32_t hidden;         /* H */
  int32_t n_expert;       /* E */
  int32_t top_k;          /* k */
  int32_t expert_ff;      /* F */
  int32_t shared_ff;      /* Fs; 0 = no shared expert */
  int32_t gating;         /* MOE_GATING_* */
  int32_t norm_topk_prob; /* softmax-topk only: renormalise the k weights */
  float weights_scale;    /* multiplies the final routing weights (1.0) */
  int32_t act;            /* MOE_ACT_* */
  float act_alpha;        /* 1.702 for gpt-oss */
  float act_limit;        /* 7.0 for gpt-oss */
  int32_t x_dtype;        /* MOE_DTYPE_F32 | MOE_DTYPE_BF16 */
  int32_t w_dtype;        /* MOE_DTYPE_F32 | MOE_DTYPE_BF16 | MOE_DTYPE_MXFP4 */
  int32_t act_quant;      /* MOE_ACT_QUANT_*: 0 for every layer the pages define */
} moe_config;

/* Weight tensors (device pointers; names follow the pages' GGUF and
 * safetensors names).  Unused fields may be NULL. */
typedef struct {
  const void* router_w;          /* ffn_gate_inp [E][H] x_dtype; NULL: logits are an input */
  const void* router_b;          /* [E] x_dtype or NULL (gpt-oss router bias) */
  const void* gate_w;            /* SWIGLU: ffn_gate_exps [E][F][H] */
  const void* up_w;              /* SWIGLU: ffn_up_exps   [E][F][H] */
  const void* gate_up_w;         /* SWIGLU_OAI: [E][2F][H] (MXFP4: codes [E][2F][H/32][16]) */
  const uint8_t* gate_up_scales; /* MXFP4: [E][2F][H/32] */
  const void* gate_up_b;         /* SWIGLU_OAI: [E][2F] x_dtype, interleaved like the rows */
  const void* down_w;            /* ffn_down_exps [E][H][F] (MXFP4: codes [E][H][F/32][16]) */
  const uint8_t* down_scales;    /* MXFP4: [E][H][F/32] */
  const void* down_b;            /* SWIGLU_OAI: [E][H] x_dtype */
  const void* sh_gate_w;         /* ffn_gate_shexp [Fs][H] x_dtype */
  const void* sh_up_w;           /* ffn_up_shexp   [Fs][H] */
  const void* sh_down_w;         /* ffn_down_shexp [H][Fs] */
  const void* sh_gate_inp;       /* ffn_gate_inp_shexp [H] */
} moe_weights;

/* Bytes of workspace that moe_forward and moe_forward_prenorm (the largest
 * users) need for T tokens; it also covers moe_permute, moe_expert_ffn and
 * moe_combine.  Returns 0 for an invalid config. */
size_t moe_workspace_bytes(const moe_config* cfg, int32_t T);

/* Routing: router product (when w->router_w != NULL) and gating.
 * Defined by "qwen35moe - Forward-Pass Design (Pantheon port)", section
 * "Shared-expert MoE FFN (every layer)" (softmax over the router logits,
 * top-k, norm_topk_prob, expert_weights_scale, sigmoid shared gate),
 * "qwen35moe CPU-reference golden vectors", section "Kernel 4 - MoE
 * routing" (selection order, first-seen ties) and "Phase 19: MoE -
 * gpt-oss-20b", section 2 "Router" (biased logits, top-k, softmax of the k).
 *   x        [T][H] x_dtype; may be NULL only when router_w == NULL and there
 *            is no shared expert
 *   logits   [T][E] fp32: written when router_w != NULL (bias included),
 *            read when router_w == NULL
 *   topk_idx [T][k] int32, expert ids in pick order (descending logit,
 *            lowest index first among bit-equal logits; -0 == +0)
 *   topk_w   [T][k] fp32 routing weights
 *   sgate    [T] fp32 sigmoid shared-expert gate; required iff shared_ff > 0
 *   ws       NULL, or scratch of ws_bytes >= moe_workspace_bytes(cfg, T)
 *            bytes: with it, a large batch's router product is split over
 *            ranges of the hidden dimension (more workgroups) whose partial
 *            sums the gating adds up in a fixed order
 * Same logits in => bit-identical topk_idx, on every call.  Logits that
 * are NaN or infinite are outside the contract; the picks are still k
 * distinct experts in [0, E) for every token. */
int moe_route(const moe_config* cfg, const moe_weights* w, const void* x, float* logits,
              int32_t* topk_idx, float* topk_w, float* sgate, int32_t T, void* ws, size_t ws_bytes,
              hipStream_t stream);

/* Token -> expert permutation: a stable counting sort of the T*k
 * assignments a = t*k + j by expert id (ascending a inside each segment).
 * With a shared expert a last segment E holds a = T*k + t for every token.
 * The pages only imply this step: expert-grouped launches in "qwen35moe -
 * Forward-Pass Design (Pantheon port)", sections "K80 GPU decode - status
 * & performance" and "Batched prefill" (tokens that share an expert stream
 * its weights once).
 *   offsets       [E + 1 (+1 if shared)] int32, exclusive prefix of the counts
 *   sorted_assign [T*k (+T)] int32, assignment id at each sorted position
 *   assign_pos    [T*k (+T)] int32, its inverse
 * Contract: each token's k picks are distinct experts in [0, E) (what
 * moe_route writes); the result is then bit-exact and deterministic.  Picks
 * that break it (an id out of range, or one repeating an earlier pick of
 * the same token) are replaced, in slot order, by the lowest experts the
 * token's valid picks leave free, so the permutation is always a bijection
 * and no later step indexes past a buffer; the layer's output for such a
 * token is then that of the replaced picks. */
int moe_permute(const moe_config* cfg, const int32_t* topk_idx, int32_t T, int32_t* offsets,
                int32_t* sorted_assign, int32_t* assign_pos, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* Expert gate/up products with the activation applied, one row per sorted
 * position: h rows [0, T*k) have F columns, the shared rows [T*k, T*k+T)
 * follow with Fs columns.  Defined by "qwen35moe - Forward-Pass Design
 * (Pantheon port)", section "Shared-expert MoE FFN" (SwiGLU experts and
 * the shared SwiGLU expert) and "Phase 19: MoE - gpt-oss-20b", section 2
 * "Experts" (interleaved gate_up with bias, clamps, (up+1)*gate*
 * sigmoid(alpha*gate)) and section 3 (MXFP4 blocks and scales).  h is bf16 when x_dtype is BF16, fp32 otherwise.
 * ws is used only with act_quant (the rounded x); then it must be 256-byte
 * aligned and at least moe_workspace_bytes(cfg, T) bytes (MOE_EWORKSPACE). */
int moe_expert_ffn(const moe_config* cfg, const moe_weights* w, const void* x,
                   const int32_t* offsets, const int32_t* sorted_assign, int32_t T, void* h,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Down projection (+ bias), weighted combine over each token's k picks in
 * pick order, plus sgate * the shared expert's down projection.  Defined by
 * "qwen35moe - Forward-Pass Design (Pantheon port)", section "Shared-expert
 * MoE FFN" (weighted sum of the picked experts plus the gated shared
 * expert) and "Phase 19: MoE - gpt-oss-20b", section 2 "Experts" (the down
 * bias inside each expert's weighted term).
 *   h as written by moe_expert_ffn (with act_quant, rounded to MXFP8 here,
 *   into ws); topk_w [T][k]; sgate [T] (shared only);
 *   out [T][H] fp32 (fully overwritten). */
int moe_combine(const moe_config* cfg, const moe_weights* w, const void* h,
                const int32_t* offsets, const int32_t* sorted_assign, const float* topk_w,
                const float* sgate, int32_t T, float* out, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* The whole layer: route, permute, expert FFN, combine, as the layer
 * statement at the top of this header gives it ("qwen35moe - Forward-Pass
 * Design (Pantheon port)", section "Shared-expert MoE FFN (every layer)";
 * "Phase 19: MoE - gpt-oss-20b", section 2 "Router" and "Experts").
 *   logits: NULL or [T][E] fp32 -- an output when router_w != NULL, the
 *   required input when router_w == NULL.  topk_idx, topk_w, sgate: NULL or
 *   outputs as in moe_route.  Intermediates live in ws. */
int moe_forward(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T, float* out,
                float* logits, int32_t* topk_idx, float* topk_w, float* sgate, void* ws,
                size_t ws_bytes, hipStream_t stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same layer and arguments, but the intermediates live in a scratch
 * array of MOE_NOALLOC_SCRATCH_BYTES built into the library instead of a
 * caller's workspace.  Each GPU the library runs on holds its own copy of
 * that array until the process ends.  The call allocates nothing (no
 * hipMalloc, no library allocation); its first call on a device looks up
 * that device's copy.  A batch whose moe_workspace_bytes(cfg, T) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES is refused with MOE_EWORKSPACE (for the
 * qwen35moe-shaped decode layer, T <= 256 fits).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, or two host threads) race and must be ordered by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_forward_noalloc(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T, float* out,
                        float* logits, int32_t* topk_idx, float* topk_w, float* sgate, hipStream_t stream);

/* The layer inside its pre-norm decoder block, with the norm in front and
 * the residual add behind it ("qwen35moe - Forward-Pass Design (Pantheon
 * port)", section "Block scaffold": every norm is an RMS norm and the
 * residual adds the un-normalised input; "Phase 19: MoE - gpt-oss-20b",
 * section 2: RMSNorm with the variance in fp32, out = h + moe(post_norm(h))):
 *   xn[t]  = resid[t] * norm_w / sqrt(mean(resid[t]^2) + norm_eps)
 *            (fp32 statistics, rounded once to x_dtype)
 *   out[t] = resid[t] + layer(xn)[t]          (fp32; the layer as moe_forward)
 *   norm_w   [H] x_dtype (post_attention_norm / ffn_norm weight)
 *   norm_eps 1e-6 (qwen35moe), 1e-5 (gpt-oss); 0 <= norm_eps <= 1
 *   resid    [T][H] x_dtype, the un-normalised residual stream
 *   xn       NULL, or [T][H] x_dtype output: the normalised rows the layer
 *            read; must not overlap resid (else they live in ws)
 *   out      [T][H] fp32, fully overwritten; must not overlap resid or xn
 *   logits, topk_idx, topk_w, sgate, ws: as in moe_forward. */
int moe_forward_prenorm(const moe_config* cfg, const moe_weights* w, const void* norm_w, float norm_eps,
                        const void* resid, int32_t T, float* out, void* xn, float* logits, int32_t* topk_idx,
                        float* topk_w, float* sgate, void* ws, size_t ws_bytes, hipStream_t stream);

/* MXFP8 rounding as act_quant applies it (OCP MX v1.0, section 6.3):
 *   x      [rows][K] bf16, K a multiple of 32
 *   codes  [rows][K] uint8 E4M3 codes
 *   scales [rows][scale_stride] uint8 E8M0 bytes, scale_stride =
 *          4 * ceil(K / 128) (block b of a row at byte b; the bytes past
 *          K / 32 are left as they are)
 * Bit-exact and deterministic: every step is exact in fp32. */
int moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream);

/* Text for a status code (static storage). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
