/*
 * moe_ref.h -- CPU oracle of the sparse mixture-of-experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, double-precision C
 * statement of what the layer computes, written from the pages that define
 * it.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load it.  It shares no code, header or constant table with the
 * GPU library, and the GPU library never calls it.
 *
 * Sources (cited per function in moe_ref.c):
 *   [Q]  "qwen35moe - Forward-Pass Design (Pantheon port)", section
 *        "Shared-expert MoE FFN (every layer)" and the "Correctness
 *        watch-list" (norm_topk_prob).
 *   [G]  "qwen35moe CPU-reference golden vectors", section "Kernel 4 - MoE
 *        routing" (selection sort with first-seen tie-break, slot order,
 *        renormalise then scale, sigmoid shared gate) and the config table
 *        (expert_weights_scale 1.0).
 *   [X]  "Phase 19: MoE - gpt-oss-20b", section 2 "Router" and "Experts"
 *        (biased top-k then softmax over the selected; fused interleaved
 *        gate_up with bias; clamps; (up+1)*gate*sigmoid(alpha*gate); down +
 *        bias; weighted sum) and section 3 plus the tensor-layout listing
 *        (MXFP4: 32-element blocks along the input dim, low nibble = even
 *        index, value = lut[code] * 2^(e8m0-127)).
 *   [B]  The decoder block around the layer: "qwen35moe - Forward-Pass
 *        Design (Pantheon port)", section "Block scaffold" (pre-norm
 *        sandwich, every norm an RMS norm, the residual adds the
 *        un-normalised input) and its config table (rms_norm_eps 1e-6);
 *        "Phase 19: MoE - gpt-oss-20b", section 2 (standard RMSNorm with
 *        the variance in fp32, eps 1e-5; decoder layer out = h +
 *        moe(post_norm(h))); "qwen35moe CPU-reference golden vectors",
 *        section "Kernel 3" (y = x * w / sqrt(mean(x^2) + eps)).
 *
 * Every dot product accumulates in double.  Values the pages fix as fp32
 * (router logits, routing weights, the shared gate scalar) are rounded to
 * fp32 where they are stored; expert activations are kept in double inside
 * ref_forward and rounded to fp32 only where a function hands them out.
 *
 * All pointers are host pointers owned by the caller.  Layouts are row-major
 * [out][in] ("y = x W^T"), experts outermost.
 */
#ifndef MOE_REF_H
#define MOE_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { REF_F32 = 0, REF_BF16 = 1, REF_MXFP4 = 2 };
enum { REF_SOFTMAX_TOPK = 0, REF_TOPK_SOFTMAX = 1 };
enum { REF_SWIGLU = 0, REF_SWIGLU_OAI = 1 };
/* Precision of the routed experts' GEMM inputs: as given, or rounded to
 * MXFP8 (E4M3 elements, one E8M0 scale per 32 along the input dimension)
 * before each routed gate/up and down product. */
enum { REF_AQ_NONE = 0, REF_AQ_MXFP8 = 1 };

/* A matrix operand: f32 / bf16 elements, or MXFP4 codes [rows][cols/32][16]
 * with E8M0 scales [rows][cols/32]. */
typedef struct {
  int32_t dtype;
  const void* data;
  const uint8_t* scales;
} ref_mat;

typedef struct {
  int32_t H, E, k, F, Fs;        /* Fs = 0: no shared expert */
  int32_t gating;                /* REF_SOFTMAX_TOPK | REF_TOPK_SOFTMAX */
  int32_t norm_topk_prob;
  float weights_scale;
  int32_t act;                   /* REF_SWIGLU | REF_SWIGLU_OAI */
  float alpha, limit;
  int32_t act_quant;             /* REF_AQ_NONE | REF_AQ_MXFP8 (routed experts only) */
} ref_cfg;

typedef struct {
  ref_mat router_w;              /* [E][H] */
  ref_mat router_b;              /* [E] or data == NULL */
  ref_mat gate_w, up_w;          /* SWIGLU: [E][F][H] */
  ref_mat gate_up_w;             /* SWIGLU_OAI: [E][2F][H], rows interleaved gate/up */
  ref_mat gate_up_b;             /* [E][2F] or NULL */
  ref_mat down_w;                /* [E][H][F] */
  ref_mat down_b;                /* [E][H] or NULL */
  ref_mat sh_gate_w, sh_up_w;    /* [Fs][H] */
  ref_mat sh_down_w;             /* [H][Fs] */
  ref_mat sh_gate_inp;           /* [H] */
} ref_weights;

/* Exact value of element (row, col) of a matrix with `cols` columns. */
double ref_elem(const ref_mat* m, int64_t row, int64_t col, int64_t cols);
/* One E2M1 code (0..15) and one E8M0 exponent byte, exactly. */
double ref_mxfp4_value(uint32_t code, uint32_t e8m0);
/* One E4M3 code (0..255; 0x7F and 0xFF are NaN) and one E8M0 byte, exactly. */
double ref_e4m3_value(uint32_t code, uint32_t e8m0);
/* MXFP8 (E4M3) quantisation of n values (n a multiple of 32): codes[n] and
 * one scale byte per 32 consecutive values. */
void ref_mxfp8_quantize(const double* v, int64_t n, uint8_t* codes, uint8_t* scales);
/* v -> the MXFP8 value it quantises to, in place-safe form (out may be v). */
void ref_mxfp8_round(const double* v, int64_t n, double* out);

/* [B] RMSNorm of T rows of H values:
 *   y[t][h] = x[t][h] * g[h] / sqrt(mean_h x[t][h]^2 + eps)
 * in double, rounded once to out_dtype (REF_F32: float; REF_BF16: bf16 bits,
 * nearest even).  x and g are F32 or BF16 matrices ([T][H] and [1][H]). */
void ref_rmsnorm(const ref_mat* x, int32_t T, int32_t H, const ref_mat* g, double eps, int32_t out_dtype,
                 void* out);

/* logits[t][e] = fp32(sum_h x[t][h] Wr[e][h] (+ br[e])) */
void ref_router_logits(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T, float* logits);
/* s[t] = fp32(sum_h wsg[h] x[t][h]) (pre-sigmoid) */
void ref_shared_gate_logit(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T, float* s);
/* Selection sort, k passes, first-seen wins ties; idx in pick order. */
void ref_topk(int32_t E, int32_t k, const float* key, int32_t* idx);
/* Gating from logits: indices (pick order) and fp32 weights per token. */
void ref_route(const ref_cfg* c, const float* logits, int32_t T, int32_t* topk_idx, float* topk_w);
/* The same gating, but the selection compares fp32 probabilities (literal
 * softmax-then-select reading); returns the number of tokens whose index
 * list differs from ref_route's. */
int32_t ref_route_prob_key_disagreements(const ref_cfg* c, const float* logits, int32_t T);
/* sgate = fp32(1 / (1 + exp(-s))) */
void ref_sigmoid(const float* s, int32_t n, float* out);

/* Stable counting sort of the T*k assignments a = t*k + j by expert.
 * offsets [E+1] (+1 when shared: segment E holds a = T*k + t, t ascending),
 * sorted_assign[pos] = a, assign_pos[a] = pos. */
void ref_permute(int32_t E, int32_t k, int32_t T, int32_t shared, const int32_t* topk_idx,
                 int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos);

/* Activation vector of one token row through expert e (e == E: shared
 * expert) -> h[F] (or h[Fs]), double. */
void ref_expert_act(const ref_cfg* c, const ref_weights* w, int32_t e, const double* xrow, double* h);
/* y[H] = Wd[e] h (+ bd[e]); e == E: shared down. */
void ref_expert_down(const ref_cfg* c, const ref_weights* w, int32_t e, const double* h, double* y);

/* h rows in permuted order: h[pos][:] = act(expert of pos, token of pos), fp32. */
void ref_expert_ffn(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T,
                    const int32_t* offsets, const int32_t* sorted_assign, float* h);
/* out[t] = sum_j w[t][j] y(t,j) + sgate[t] y_shared(t), from given h rows (fp32). */
void ref_combine(const ref_cfg* c, const ref_weights* w, const float* h, const int32_t* offsets,
                 const int32_t* sorted_assign, const float* topk_w, const float* sgate,
                 int32_t T, float* out);

/* Whole layer, token by token.  logits_in != NULL: those logits are used and
 * the router product is skipped.  tokens != NULL: only those n_tokens rows of
 * out (and of the optional outputs) are written.  idx_in != NULL forces the
 * expert choice (its weights are still computed from the logits by the same
 * softmax). */
void ref_forward(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T,
                 const float* logits_in, const int32_t* idx_in,
                 const int32_t* tokens, int32_t n_tokens,
                 float* out, int32_t* topk_idx, float* topk_w, float* sgate);

/* Dense brute force: every expert evaluated for every token, masked by the
 * scattered top-k weights; output in double. */
void ref_forward_dense(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T,
                       const float* logits_in, double* out);

/* Threads used by the parallel-over-tokens loops (n <= 0 leaves the count
 * unchanged); returns the current count. */
int32_t ref_set_threads(int32_t n);

#ifdef __cplusplus
}
#endif
#endif
