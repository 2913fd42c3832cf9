/*
 * moe_ref.c -- CPU oracle of the sparse MoE FFN layer (test infrastructure).
 * See moe_ref.h for the sources [Q], [G], [X] and the precision rules.
 */
#include "moe_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- inputs */

/* E2M1 (OCP Microscaling Formats spec v1.0, section 5.3.3): sign bit 3,
 * exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is subnormal
 * (0 or 0.5).  E8M0 scale = 2^(e - 127) [X, section 3]. */
double ref_mxfp4_value(uint32_t code, uint32_t e8m0) {
  uint32_t ex = (code >> 1) & 3u, m = code & 1u;
  double mag = ex == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)ex - 1);
  if (code & 8u) mag = -mag;
  return mag * ldexp(1.0, (int)e8m0 - 127);
}

/* E4M3 (OCP Microscaling Formats spec v1.0, section 5.3.3, and the OCP 8-bit
 * floating point spec): sign bit 7, exponent bits 6..3 with bias 7, mantissa
 * bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with
 * mantissa 7 is NaN, so the largest magnitude is 1.75 * 2^8 = 448. */
double ref_e4m3_value(uint32_t code, uint32_t e8m0) {
  uint32_t ex = (code >> 3) & 15u, m = code & 7u;
  if (ex == 15u && m == 7u) return NAN;
  double mag = ex == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)ex - 7);
  if (code & 0x80u) mag = -mag;
  return mag * ldexp(1.0, (int)e8m0 - 127);
}

/* E4M3 code of a value already divided by its block scale: nearest
 * representable value, ties to the even mantissa, magnitudes beyond 448
 * saturated to 448 (OCP MX v1.0, section 6.3, conversion with saturation). */
static uint8_t e4m3_encode(double v) {
  uint8_t sign = v < 0.0 ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {                 /* subnormal grid, step 2^-9 */
    double m = rint(ldexp(a, 9));            /* 0..8; 8 is the smallest normal */
    return sign | (uint8_t)m;                /* m = 8 encodes exponent 1, mantissa 0 */
  }
  int e;
  double f = frexp(a, &e);                   /* a = f * 2^e, f in [0.5, 1) */
  double m = rint((2.0 * f - 1.0) * 8.0);    /* mantissa of 1.m * 2^(e-1), 0..8 */
  int ex = e - 1 + 7;
  if (m == 8.0) { m = 0.0; ++ex; }
  if (ex > 15 || (ex == 15 && m == 7.0)) return sign | 0x7E;
  return sign | (uint8_t)((ex << 3) | (int)m);
}

/* OCP MX v1.0, section 6.3: per block of 32, the shared exponent is
 * floor(log2(max |v|)) minus the largest E4M3 exponent (8), kept in the E8M0
 * range [-127, 127]; every element is v / 2^shared rounded by e4m3_encode.
 * An all-zero block gets scale byte 0 and zero codes. */
void ref_mxfp8_quantize(const double* v, int64_t n, uint8_t* codes, uint8_t* scales) {
  for (int64_t b = 0; b < n / 32; ++b) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[b * 32 + i]));
    int sh = -127;
    if (amax > 0.0) {
      int e;
      frexp(amax, &e);                       /* amax in [2^(e-1), 2^e) */
      sh = e - 1 - 8;
      if (sh < -127) sh = -127;
      if (sh > 127) sh = 127;
    }
    scales[b] = (uint8_t)(sh + 127);
    for (int i = 0; i < 32; ++i) codes[b * 32 + i] = e4m3_encode(ldexp(v[b * 32 + i], -sh));
  }
}

void ref_mxfp8_round(const double* v, int64_t n, double* out) {
  uint8_t* c = malloc((size_t)n);
  uint8_t* s = malloc((size_t)(n / 32 + 1));
  ref_mxfp8_quantize(v, n, c, s);
  for (int64_t i = 0; i < n; ++i) out[i] = ref_e4m3_value(c[i], s[i / 32]);
  free(c);
  free(s);
}

static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

double ref_elem(const ref_mat* m, int64_t row, int64_t col, int64_t cols) {
  switch (m->dtype) {
    case REF_F32: return (double)((const float*)m->data)[row * cols + col];
    case REF_BF16: return bf16_value(((const uint16_t*)m->data)[row * cols + col]);
    default: {
      /* [X] tensor layout: 16 bytes hold one 32-element block, low nibble =
       * even index; one scale byte per block, blocks along the input dim. */
      const uint8_t* codes = (const uint8_t*)m->data;
      uint8_t byte = codes[row * (cols / 2) + col / 2];
      uint32_t code = (col & 1) ? (byte >> 4) : (byte & 15u);
      return ref_mxfp4_value(code, m->scales[row * (cols / 32) + col / 32]);
    }
  }
}

/* Row `row` of an [rows][cols] matrix, widened exactly to double. */
static void load_row(const ref_mat* m, int64_t row, int64_t cols, double* dst) {
  for (int64_t j = 0; j < cols; ++j) dst[j] = ref_elem(m, row, j, cols);
}

static double dot(const double* a, const double* b, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

/* ---------------------------------------------------------------- block */

/* fp32 -> bf16 bits, round to nearest even (finite values). */
static uint16_t bf16_round(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* [B] RMSNorm: the mean of squares over the row, plus eps, its inverse
 * square root, times the element and its weight, all in double; the result
 * is rounded to the nearest float and, for bf16 output, that float to the
 * nearest bf16 (the storage type the layer then reads). */
void ref_rmsnorm(const ref_mat* x, int32_t T, int32_t H, const ref_mat* g, double eps, int32_t out_dtype,
                 void* out) {
  double* v = malloc(sizeof(double) * (size_t)H);
  for (int64_t t = 0; t < T; ++t) {
    load_row(x, t, H, v);
    double ms = dot(v, v, H) / (double)H;
    double r = 1.0 / sqrt(ms + eps);
    for (int64_t h = 0; h < H; ++h) {
      double y = v[h] * r * ref_elem(g, 0, h, H);
      if (out_dtype == REF_BF16)
        ((uint16_t*)out)[t * H + h] = bf16_round((float)y);
      else
        ((float*)out)[t * H + h] = (float)y;
    }
  }
  free(v);
}

/* ---------------------------------------------------------------- router */

/* [Q] router logits = ffn_gate_inp . x (no bias); [X] Router: x W^T + b. */
void ref_router_logits(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T, float* logits) {
  const int64_t H = c->H, E = c->E;
  double* xr = malloc(sizeof(double) * H);
  double* wr = malloc(sizeof(double) * H);
  for (int64_t t = 0; t < T; ++t) {
    load_row(x, t, H, xr);
    for (int64_t e = 0; e < E; ++e) {
      load_row(&w->router_w, e, H, wr);
      double s = dot(xr, wr, H);
      if (w->router_b.data) s += ref_elem(&w->router_b, 0, e, E);
      logits[t * E + e] = (float)s;
    }
  }
  free(xr);
  free(wr);
}

/* [Q] sgate = sigmoid(ffn_gate_inp_shexp . x); this is the pre-sigmoid dot. */
void ref_shared_gate_logit(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T, float* s) {
  const int64_t H = c->H;
  double* xr = malloc(sizeof(double) * H);
  double* g = malloc(sizeof(double) * H);
  load_row(&w->sh_gate_inp, 0, H, g);
  for (int64_t t = 0; t < T; ++t) {
    load_row(x, t, H, xr);
    s[t] = (float)dot(g, xr, H);
  }
  free(xr);
  free(g);
}

/* [G] Kernel 4: selection sort; each pass scans the experts in index order
 * and keeps the first one seen among equal keys (strict greater-than).
 * -0 and +0 compare equal, so they tie.  Indices come out in pick order. */
void ref_topk(int32_t E, int32_t k, const float* key, int32_t* idx) {
  unsigned char* used = calloc((size_t)E, 1);
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (used[e]) continue;
      if (best < 0 || key[e] > key[best]) best = e;
    }
    idx[j] = best;
    used[best] = 1;
  }
  free(used);
}

/* Gating of one token.  Selection key is the fp32 logit: softmax is
 * monotone, so the chosen set and order equal those of the probabilities.
 * qwen35moe [Q][G]: p = softmax over all E (max-subtracted), keep top-k,
 * renormalise over the kept (norm_topk_prob) and then multiply by
 * expert_weights_scale.  gpt-oss [X]: softmax over the k selected logits. */
static void route_token(const ref_cfg* c, const float* l, const int32_t* idx_forced, int32_t* idx, float* wt) {
  const int32_t E = c->E, k = c->k;
  if (idx_forced)
    memcpy(idx, idx_forced, sizeof(int32_t) * (size_t)k);
  else
    ref_topk(E, k, l, idx);
  if (c->gating == REF_SOFTMAX_TOPK) {
    double m = l[0];
    for (int32_t e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    double z = 0.0;
    for (int32_t e = 0; e < E; ++e) z += exp((double)l[e] - m);
    double sel = 0.0;
    for (int32_t j = 0; j < k; ++j) sel += exp((double)l[idx[j]] - m) / z;
    for (int32_t j = 0; j < k; ++j) {
      double p = exp((double)l[idx[j]] - m) / z;
      double v = c->norm_topk_prob ? p / sel : p;
      wt[j] = (float)(v * (double)c->weights_scale);
    }
  } else {
    double m = l[idx[0]];
    for (int32_t j = 1; j < k; ++j) m = l[idx[j]] > m ? l[idx[j]] : m;
    double z = 0.0;
    for (int32_t j = 0; j < k; ++j) z += exp((double)l[idx[j]] - m);
    for (int32_t j = 0; j < k; ++j) wt[j] = (float)(exp((double)l[idx[j]] - m) / z * (double)c->weights_scale);
  }
}

void ref_route(const ref_cfg* c, const float* logits, int32_t T, int32_t* topk_idx, float* topk_w) {
  for (int64_t t = 0; t < T; ++t)
    route_token(c, logits + t * c->E, NULL, topk_idx + t * c->k, topk_w + t * c->k);
}

int32_t ref_route_prob_key_disagreements(const ref_cfg* c, const float* logits, int32_t T) {
  const int32_t E = c->E, k = c->k;
  float* p = malloc(sizeof(float) * (size_t)E);
  int32_t* a = malloc(sizeof(int32_t) * (size_t)k);
  int32_t* b = malloc(sizeof(int32_t) * (size_t)k);
  int32_t bad = 0;
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    double m = l[0];
    for (int32_t e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    double z = 0.0;
    for (int32_t e = 0; e < E; ++e) z += exp((double)l[e] - m);
    for (int32_t e = 0; e < E; ++e) p[e] = (float)(exp((double)l[e] - m) / z);
    ref_topk(E, k, l, a);
    ref_topk(E, k, p, b);
    if (memcmp(a, b, sizeof(int32_t) * (size_t)k)) ++bad;
  }
  free(p);
  free(a);
  free(b);
  return bad;
}

/* [Q] sigmoid of the shared-gate dot. */
void ref_sigmoid(const float* s, int32_t n, float* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = (float)(1.0 / (1.0 + exp(-(double)s[i])));
}

/* ----------------------------------------------------------- permutation */

/* Grouping the token-expert assignments by expert: a counting sort that
 * keeps assignments in ascending a = t*k + j inside each expert's segment. */
void ref_permute(int32_t E, int32_t k, int32_t T, int32_t shared, const int32_t* topk_idx,
                 int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos) {
  const int64_t n = (int64_t)T * k;
  const int32_t nseg = E + (shared ? 1 : 0);
  int64_t* cnt = calloc((size_t)nseg + 1, sizeof(int64_t));
  for (int64_t a = 0; a < n; ++a) cnt[topk_idx[a]]++;
  if (shared) cnt[E] = T;
  offsets[0] = 0;
  for (int32_t e = 0; e < nseg; ++e) offsets[e + 1] = offsets[e] + (int32_t)cnt[e];
  int64_t* fill = calloc((size_t)nseg, sizeof(int64_t));
  for (int32_t e = 0; e < nseg; ++e) fill[e] = offsets[e];
  for (int64_t a = 0; a < n; ++a) {
    int64_t pos = fill[topk_idx[a]]++;
    sorted_assign[pos] = (int32_t)a;
    assign_pos[a] = (int32_t)pos;
  }
  if (shared)
    for (int64_t t = 0; t < T; ++t) {
      int64_t pos = fill[E]++;
      sorted_assign[pos] = (int32_t)(n + t);
      assign_pos[n + t] = (int32_t)pos;
    }
  free(cnt);
  free(fill);
}

/* ---------------------------------------------------------------- experts */

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Input row of a routed expert product (e < E) at the layer's activation
 * precision: copied, or rounded to MXFP8 when act_quant is set.  The shared
 * expert (e == E) always takes its input as given. */
static void expert_input(const ref_cfg* c, int32_t e, const double* v, int64_t n, double* out) {
  if (c->act_quant == REF_AQ_MXFP8 && e < c->E)
    ref_mxfp8_round(v, n, out);
  else
    memcpy(out, v, sizeof(double) * (size_t)n);
}

/* SwiGLU expert [Q]: h = silu(W_gate x) * (W_up x), silu(g) = g sigmoid(g)
 * (Shazeer 2020, "GLU Variants Improve Transformer").
 * gpt-oss expert [X] Experts: gu = W_gate_up x + b (2F outputs); gate = the
 * even entries, up = the odd ones; gate clamped above at limit, up clamped
 * to [-limit, limit]; h = (up + 1) * gate * sigmoid(alpha * gate).
 * e == E selects the shared expert, which is a plain SwiGLU [Q].
 * With act_quant the routed experts see x rounded to MXFP8 (expert_input). */
void ref_expert_act(const ref_cfg* c, const ref_weights* w, int32_t e, const double* xin, double* h) {
  const int64_t H = c->H;
  double* wr = malloc(sizeof(double) * H);
  double* xrow = malloc(sizeof(double) * H);
  expert_input(c, e, xin, H, xrow);
  if (e == c->E) {
    for (int64_t f = 0; f < c->Fs; ++f) {
      load_row(&w->sh_gate_w, f, H, wr);
      double g = dot(wr, xrow, H);
      load_row(&w->sh_up_w, f, H, wr);
      double u = dot(wr, xrow, H);
      h[f] = g * sigmoid(g) * u;
    }
  } else if (c->act == REF_SWIGLU) {
    const int64_t F = c->F;
    for (int64_t f = 0; f < F; ++f) {
      load_row(&w->gate_w, (int64_t)e * F + f, H, wr);
      double g = dot(wr, xrow, H);
      load_row(&w->up_w, (int64_t)e * F + f, H, wr);
      double u = dot(wr, xrow, H);
      h[f] = g * sigmoid(g) * u;
    }
  } else {
    const int64_t F = c->F;
    const double lim = (double)c->limit, alpha = (double)c->alpha;
    double* gu = malloc(sizeof(double) * 2 * F);
    for (int64_t r = 0; r < 2 * F; ++r) {
      load_row(&w->gate_up_w, (int64_t)e * 2 * F + r, H, wr);
      gu[r] = dot(wr, xrow, H);
      if (w->gate_up_b.data) gu[r] += ref_elem(&w->gate_up_b, e, r, 2 * F);
    }
    for (int64_t f = 0; f < F; ++f) {
      double g = gu[2 * f], u = gu[2 * f + 1];
      g = g > lim ? lim : g;
      u = u > lim ? lim : (u < -lim ? -lim : u);
      h[f] = (u + 1.0) * (g * sigmoid(alpha * g));
    }
    free(gu);
  }
  free(wr);
  free(xrow);
}

/* Down projection [Q][X]: y = W_down h (+ b_down for gpt-oss); with
 * act_quant the routed experts see h rounded to MXFP8 (expert_input). */
void ref_expert_down(const ref_cfg* c, const ref_weights* w, int32_t e, const double* hin, double* y) {
  const int64_t H = c->H;
  const int shared = e == c->E;
  const int64_t F = shared ? c->Fs : c->F;
  double* wr = malloc(sizeof(double) * F);
  double* h = malloc(sizeof(double) * F);
  expert_input(c, e, hin, F, h);
  for (int64_t o = 0; o < H; ++o) {
    if (shared)
      load_row(&w->sh_down_w, o, F, wr);
    else
      load_row(&w->down_w, (int64_t)e * H + o, F, wr);
    y[o] = dot(wr, h, F);
    if (!shared && w->down_b.data) y[o] += ref_elem(&w->down_b, e, o, H);
  }
  free(wr);
  free(h);
}

static int32_t token_of(const ref_cfg* c, int32_t T, int32_t a) {
  int64_t n = (int64_t)T * c->k;
  return a < n ? a / c->k : (int32_t)(a - n);
}

/* Offset of the h row at sorted position pos: the T*k routed rows of F
 * values come first, then the T shared rows of Fs values (the layout the
 * GPU library's moe_expert_ffn writes). */
static int64_t h_row_offset(const ref_cfg* c, int32_t T, int64_t pos) {
  const int64_t n = (int64_t)T * c->k;
  return pos < n ? pos * c->F : n * c->F + (pos - n) * c->Fs;
}

static int32_t expert_of_pos(const int32_t* offsets, int32_t nseg, int32_t pos) {
  int32_t e = 0;
  while (e + 1 < nseg && offsets[e + 1] <= pos) ++e;
  return e;
}

void ref_expert_ffn(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T,
                    const int32_t* offsets, const int32_t* sorted_assign, float* h) {
  const int32_t nseg = c->E + (c->Fs > 0 ? 1 : 0);
  const int64_t rows = offsets[nseg];
  const int64_t H = c->H, F = c->F > c->Fs ? c->F : c->Fs;
#pragma omp parallel
  {
    double* xr = malloc(sizeof(double) * H);
    double* hv = malloc(sizeof(double) * F);
#pragma omp for schedule(dynamic, 1)
    for (int64_t pos = 0; pos < rows; ++pos) {
      int32_t e = expert_of_pos(offsets, nseg, (int32_t)pos);
      int32_t t = token_of(c, T, sorted_assign[pos]);
      int64_t Fe = e == c->E ? c->Fs : c->F;
      load_row(x, t, H, xr);
      ref_expert_act(c, w, e, xr, hv);
      for (int64_t f = 0; f < Fe; ++f) h[h_row_offset(c, T, pos) + f] = (float)hv[f];
    }
    free(xr);
    free(hv);
  }
}

/* [Q] out = sum over the k picks of w * y + sgate * y_shared; [X] the
 * bias of each routed down projection sits inside the weighted sum. */
void ref_combine(const ref_cfg* c, const ref_weights* w, const float* h, const int32_t* offsets,
                 const int32_t* sorted_assign, const float* topk_w, const float* sgate,
                 int32_t T, float* out) {
  const int32_t nseg = c->E + (c->Fs > 0 ? 1 : 0);
  const int64_t H = c->H, n = (int64_t)T * c->k;
  int32_t* pos_of = malloc(sizeof(int32_t) * (size_t)(offsets[nseg] + 1));
  for (int32_t p = 0; p < offsets[nseg]; ++p) pos_of[sorted_assign[p]] = p;
#pragma omp parallel
  {
    double* acc = malloc(sizeof(double) * H);
    double* y = malloc(sizeof(double) * H);
    double* hv = malloc(sizeof(double) * (c->F > c->Fs ? c->F : c->Fs));
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t o = 0; o < H; ++o) acc[o] = 0.0;
      for (int32_t j = 0; j < c->k; ++j) {
        int32_t p = pos_of[t * c->k + j];
        int32_t e = expert_of_pos(offsets, nseg, p);
        for (int64_t f = 0; f < c->F; ++f) hv[f] = (double)h[h_row_offset(c, T, p) + f];
        ref_expert_down(c, w, e, hv, y);
        for (int64_t o = 0; o < H; ++o) acc[o] += (double)topk_w[t * c->k + j] * y[o];
      }
      if (c->Fs > 0) {
        int32_t p = pos_of[n + t];
        for (int64_t f = 0; f < c->Fs; ++f) hv[f] = (double)h[h_row_offset(c, T, p) + f];
        ref_expert_down(c, w, c->E, hv, y);
        for (int64_t o = 0; o < H; ++o) acc[o] += (double)sgate[t] * y[o];
      }
      for (int64_t o = 0; o < H; ++o) out[t * H + o] = (float)acc[o];
    }
    free(acc);
    free(y);
    free(hv);
  }
  free(pos_of);
}

/* ---------------------------------------------------------------- layer */

/* One token through the whole layer [Q][X]; returns out[H] in double. */
static void forward_token(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t t,
                          const float* logits_in, const int32_t* idx_in,
                          double* out, int32_t* idx, float* wt, float* sg) {
  const int64_t H = c->H, E = c->E;
  const int64_t Fm = c->F > c->Fs ? c->F : c->Fs;
  double* xr = malloc(sizeof(double) * H);
  double* wr = malloc(sizeof(double) * H);
  double* hv = malloc(sizeof(double) * Fm);
  double* y = malloc(sizeof(double) * H);
  float* l = malloc(sizeof(float) * E);
  load_row(x, t, H, xr);
  if (logits_in) {
    memcpy(l, logits_in + (int64_t)t * E, sizeof(float) * E);
  } else {
    for (int64_t e = 0; e < E; ++e) {
      load_row(&w->router_w, e, H, wr);
      double s = dot(xr, wr, H);
      if (w->router_b.data) s += ref_elem(&w->router_b, 0, e, E);
      l[e] = (float)s;
    }
  }
  route_token(c, l, idx_in ? idx_in + (int64_t)t * c->k : NULL, idx, wt);
  for (int64_t o = 0; o < H; ++o) out[o] = 0.0;
  for (int32_t j = 0; j < c->k; ++j) {
    ref_expert_act(c, w, idx[j], xr, hv);
    ref_expert_down(c, w, idx[j], hv, y);
    for (int64_t o = 0; o < H; ++o) out[o] += (double)wt[j] * y[o];
  }
  *sg = 0.0f;
  if (c->Fs > 0) {
    load_row(&w->sh_gate_inp, 0, H, wr);
    float s = (float)dot(wr, xr, H);
    ref_sigmoid(&s, 1, sg);
    ref_expert_act(c, w, c->E, xr, hv);
    ref_expert_down(c, w, c->E, hv, y);
    for (int64_t o = 0; o < H; ++o) out[o] += (double)(*sg) * y[o];
  }
  free(xr);
  free(wr);
  free(hv);
  free(y);
  free(l);
}

void ref_forward(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T,
                 const float* logits_in, const int32_t* idx_in,
                 const int32_t* tokens, int32_t n_tokens,
                 float* out, int32_t* topk_idx, float* topk_w, float* sgate) {
  const int32_t n = tokens ? n_tokens : T;
  const int64_t H = c->H;
#pragma omp parallel
  {
    double* o = malloc(sizeof(double) * H);
    int32_t* idx = malloc(sizeof(int32_t) * (size_t)c->k);
    float* wt = malloc(sizeof(float) * (size_t)c->k);
#pragma omp for schedule(dynamic, 1)
    for (int32_t i = 0; i < n; ++i) {
      int32_t t = tokens ? tokens[i] : i;
      float sg;
      forward_token(c, w, x, t, logits_in, idx_in, o, idx, wt, &sg);
      for (int64_t h = 0; h < H; ++h) out[(int64_t)t * H + h] = (float)o[h];
      if (topk_idx) memcpy(topk_idx + (int64_t)t * c->k, idx, sizeof(int32_t) * (size_t)c->k);
      if (topk_w) memcpy(topk_w + (int64_t)t * c->k, wt, sizeof(float) * (size_t)c->k);
      if (sgate) sgate[t] = sg;
    }
    free(o);
    free(idx);
    free(wt);
  }
}

/* [X] Router: scores = zeros[T, E].scatter(idx, weights); out = sum over all
 * E experts of scores[t, e] * y_e(x_t), every expert evaluated. */
void ref_forward_dense(const ref_cfg* c, const ref_weights* w, const ref_mat* x, int32_t T,
                       const float* logits_in, double* out) {
  const int64_t H = c->H, E = c->E, k = c->k;
  const int64_t Fm = c->F > c->Fs ? c->F : c->Fs;
  float* logits = malloc(sizeof(float) * (size_t)(T * E));
  int32_t* idx = malloc(sizeof(int32_t) * (size_t)(T * k));
  float* wt = malloc(sizeof(float) * (size_t)(T * k));
  double* scores = calloc((size_t)(T * E), sizeof(double));
  float* s = malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
  float* sg = malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
  double* xr = malloc(sizeof(double) * H);
  double* hv = malloc(sizeof(double) * Fm);
  double* y = malloc(sizeof(double) * H);
  if (logits_in)
    memcpy(logits, logits_in, sizeof(float) * (size_t)(T * E));
  else
    ref_router_logits(c, w, x, T, logits);
  ref_route(c, logits, T, idx, wt);
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < k; ++j) scores[t * E + idx[t * k + j]] = (double)wt[t * k + j];
  if (c->Fs > 0) {
    ref_shared_gate_logit(c, w, x, T, s);
    ref_sigmoid(s, T, sg);
  }
  for (int64_t t = 0; t < T; ++t) {
    load_row(x, t, H, xr);
    for (int64_t o = 0; o < H; ++o) out[t * H + o] = 0.0;
    for (int32_t e = 0; e < E; ++e) {
      ref_expert_act(c, w, e, xr, hv);
      ref_expert_down(c, w, e, hv, y);
      for (int64_t o = 0; o < H; ++o) out[t * H + o] += scores[t * E + e] * y[o];
    }
    if (c->Fs > 0) {
      ref_expert_act(c, w, c->E, xr, hv);
      ref_expert_down(c, w, c->E, hv, y);
      for (int64_t o = 0; o < H; ++o) out[t * H + o] += (double)sg[t] * y[o];
    }
  }
  free(logits); free(idx); free(wt); free(scores); free(s); free(sg);
  free(xr); free(hv); free(y);
}

/* Threads of the parallel-over-tokens loops (the CPU baseline times the
 * oracle with one thread and with all of them); returns the count set. */
int32_t ref_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return (int32_t)omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}
