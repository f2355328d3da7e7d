/*
 * pmk_oracle.c -- the CPU oracle for one LLM decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code with the GPU library: no headers, no tables, no
 * helpers.
 *
 * What it computes: the plain definition of one decode step of a decoder stack,
 * as run by the Event Tensor megakernel ("Event Tensor: A Unified Abstraction
 * for Compiling Dynamic Megakernel", summary page, Experiments: the end-to-end
 * decode step covers attention, RoPE, KV cache, norm, MLP and MoE; Key
 * observations, observation 2: the MoE chain is attention -> TopK -> grouping ->
 * grouped GEMM; Core method, two kinds of dynamism: per-expert counts from topk
 * and the exp_indptr prefix sum). The pages give no formula for the layer maths,
 * so each function below is the standard textbook definition; the readings the
 * pages leave open are listed next to the function that takes them.
 *
 * Precision: every intermediate is a double. The only roundings are the ones
 * the method itself performs: new K/V entries are stored in the cache's dtype
 * (float32 or bfloat16, round-to-nearest-even), and router logits are rounded to
 * float32 before the top-k decision because the GPU takes that decision on
 * float32 logits.
 *
 * Layout (shared with the GPU library by specification, not by code): weights
 * are row-major [out][in]; the fused QKV matrix holds the q rows, then k, then v;
 * the KV cache is [L][2][max_batch][Hkv][max_seq][d]; hidden is [batch][H].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

typedef struct {
  int32_t dtype;                 /* storage of projection weights and KV cache */
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim;
  int32_t n_experts, top_k, expert_ffn_dim;
  int32_t max_batch, max_seq;
  double rms_eps, rope_theta;
} orc_desc;

typedef struct {
  const float* attn_norm;        /* [H] */
  const void* w_qkv;             /* [(Hq+2Hkv)d][H] */
  const void* w_o;               /* [H][Hq d] */
  const float* ffn_norm;         /* [H] */
  const void* w_gate;            /* [F][H] */
  const void* w_up;              /* [F][H] */
  const void* w_down;            /* [H][F] */
  const void* w_router;          /* [E][H] */
  const void* w_exp_gate;        /* [E][Fe][H] */
  const void* w_exp_up;          /* [E][Fe][H] */
  const void* w_exp_down;        /* [E][H][Fe] */
} orc_layer;

/* ---------------------------------------------------------------- storage -- */

/* Read element i of a float32 or bfloat16 array as a double (exact). */
static double ld(const void* p, int dt, size_t i) {
  if (dt == ORC_BF16) {
    uint32_t b = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
  }
  return (double)((const float*)p)[i];
}

/* Round a double to the nearest bfloat16 value, ties to even, returned as a
 * double. bfloat16 keeps 8 significant bits and float32's exponent range, so in
 * the binade [2^e, 2^(e+1)) its spacing is 2^(e-7) (2^-133 below 2^-126). */
double orc_round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e2;
  frexp(v, &e2);               /* |v| in [2^(e2-1), 2^e2) */
  int lead = e2 - 1;
  if (lead < -126) lead = -126;
  double q = ldexp(1.0, lead - 7);
  double r = nearbyint(v / q) * q;   /* default rounding mode: half to even */
  if (fabs(r) >= ldexp(1.0, 128)) r = copysign(INFINITY, v);
  return r;
}

/* Store v into element i of a float32 or bfloat16 array, rounding to nearest
 * even in that dtype. */
static void st(void* p, int dt, size_t i, double v) {
  if (dt == ORC_BF16) {
    float f = (float)orc_round_bf16(v);   /* exact: at most 8 significant bits */
    uint32_t b;
    memcpy(&b, &f, 4);
    ((uint16_t*)p)[i] = (uint16_t)(b >> 16);
  } else {
    ((float*)p)[i] = (float)v;
  }
}

/* ------------------------------------------------------------------- ops -- */

/* RMSNorm: out_i = x_i * g_i / sqrt(mean_j x_j^2 + eps). The pages name the
 * norm (Experiments, decode step op list) without a formula; eps sits inside
 * the square root, as in the standard definition. */
void orc_rmsnorm(const double* x, const float* g, int n, double eps, double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * r * (double)g[i];
}

/* Matrix-vector product y_j = sum_i W[j][i] x_i with W row-major [rows][cols]
 * (a projection of the decode step). */
void orc_matvec(const void* W, int dt, int rows, int cols, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int j = 0; j < rows; ++j) {
    size_t base = (size_t)j * (size_t)cols;
    double s = 0.0;
    for (int i = 0; i < cols; ++i) s += ld(W, dt, base + (size_t)i) * x[i];
    y[j] = s;
  }
}

/* Rotary position embedding at position pos, rotate-half pairing: for
 * i < d/2 the pair (z_i, z_{i+d/2}) turns by phi_i = pos * theta^(-2i/d).
 * The pages list RoPE in the decode step without fixing the pairing; the
 * rotate-half form is the reading taken (interleaved pairs would serve equally
 * for random weights). */
void orc_rope(double* z, int d, long pos, double theta) {
  int h = d / 2;
  for (int i = 0; i < h; ++i) {
    double phi = (double)pos * pow(theta, -2.0 * (double)i / (double)d);
    double c = cos(phi), s = sin(phi);
    double a = z[i], b = z[i + h];
    z[i] = a * c - b * s;
    z[i + h] = b * c + a * s;
  }
}

/* SiLU(z) = z / (1 + e^-z). */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Decode attention of one request against its cache, grouped-query form:
 * query head h reads KV head g = floor(h / (Hq/Hkv)); scores q_h . K_j / sqrt(d)
 * over the n cached entries, max-subtracted softmax, o_h = sum_j p_j V_j.
 * K and V point at the [Hkv][max_seq][d] slices of this request and layer. */
void orc_attention(const double* q, const void* K, const void* V, int dt, int Hq, int Hkv, int d,
                   int max_seq, int n, double* o) {
  int grp = Hq / Hkv;
  double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(static)
  for (int h = 0; h < Hq; ++h) {
    int g = h / grp;
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    size_t kb = (size_t)g * (size_t)max_seq * (size_t)d;
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int t = 0; t < d; ++t) acc += q[(size_t)h * d + t] * ld(K, dt, kb + (size_t)j * d + t);
      s[j] = acc * scale;
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) { s[j] = exp(s[j] - m); l += s[j]; }
    for (int t = 0; t < d; ++t) {
      double acc = 0.0;
      for (int j = 0; j < n; ++j) acc += s[j] * ld(V, dt, kb + (size_t)j * d + t);
      o[(size_t)h * d + t] = acc / l;
    }
    free(s);
  }
}

/* Top-k of one token's logits, ordered by (logit descending, index ascending):
 * ties go to the lower expert index. Gates are the softmax over the k selected
 * logits, which equals the full softmax renormalised over the selection. The
 * decision is taken on the float32 logits given. */
void orc_topk(const float* z, int E, int k, int32_t* idx, double* w) {
  char* taken = (char*)calloc((size_t)E, 1);
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || z[e] > z[best])) best = e;
    taken[best] = 1;
    idx[j] = best;
  }
  free(taken);
  double zmax = (double)z[idx[0]], sum = 0.0;
  for (int j = 0; j < k; ++j) { w[j] = exp((double)z[idx[j]] - zmax); sum += w[j]; }
  for (int j = 0; j < k; ++j) w[j] /= sum;
}

/* Expert grouping of T tokens' top-k choices (Core method, two kinds of
 * dynamism: the per-expert counter starts at the number of routed tokens, and
 * exp_indptr is the per-expert prefix sum that decides which grouped-GEMM tiles
 * an expert triggers).
 *   counts[e]        = number of (t, j) with idx[t][j] == e
 *   exp_indptr[e+1]  = exp_indptr[e] + counts[e]        (token-row granularity)
 *   tile_indptr[e+1] = tile_indptr[e] + ceil(counts[e] / bm)   (tile granularity)
 *   sorted_tok/slot  = the (t, j) pairs ordered by expert, then token (stable)
 * The pages call exp_indptr a prefix sum over grouped-GEMM tiles; both
 * granularities are produced (reading recorded with the GPU library). */
void orc_group(const int32_t* idx, int T, int k, int E, int bm, int32_t* exp_indptr, int32_t* tile_indptr,
               int32_t* sorted_tok, int32_t* sorted_slot) {
  int32_t* cnt = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  int32_t* pos = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int i = 0; i < T * k; ++i) cnt[idx[i]]++;
  exp_indptr[0] = 0;
  tile_indptr[0] = 0;
  for (int e = 0; e < E; ++e) {
    exp_indptr[e + 1] = exp_indptr[e] + cnt[e];
    tile_indptr[e + 1] = tile_indptr[e] + (cnt[e] + bm - 1) / bm;
    pos[e] = exp_indptr[e];
  }
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int e = idx[t * k + j];
      sorted_tok[pos[e]] = t;
      sorted_slot[pos[e]] = j;
      pos[e]++;
    }
  free(cnt);
  free(pos);
}

/* ------------------------------------------------------------ the layers -- */

static size_t kv_layer_elems(const orc_desc* D) {
  return (size_t)2 * D->max_batch * D->n_kv_heads * (size_t)D->max_seq * D->head_dim;
}

/* Attention half of a decoder layer for request b at position pos = seq_len:
 *   u = RMSNorm(x; attn_norm); [q|k|v] = W_qkv u; q, k rotated at pos;
 *   K[b][g][pos] <- rnd(k_g), V[b][g][pos] <- rnd(v_g)   (append, cache dtype);
 *   o = attention over the pos+1 cached entries (the new token attends to itself);
 *   h1 = x + W_o o.
 * kv points at this layer's [2][max_batch][Hkv][max_seq][d] block. With
 * given_append, the entry at slot pos is taken as it already stands in kv
 * (another implementation's append, whose rounding to the cache dtype may fall
 * on the other side of a rounding boundary) instead of being written. */
static void attn_half(const orc_desc* D, const orc_layer* W, void* kv, int b, int pos, const double* x, double* h1,
                      int given_append) {
  int H = D->hidden, Hq = D->n_q_heads, Hkv = D->n_kv_heads, d = D->head_dim, dt = D->dtype;
  int nq = Hq * d, nkv = Hkv * d;
  double* u = (double*)malloc(sizeof(double) * H);
  double* qkv = (double*)malloc(sizeof(double) * (size_t)(nq + 2 * nkv));
  double* o = (double*)malloc(sizeof(double) * nq);
  orc_rmsnorm(x, W->attn_norm, H, D->rms_eps, u);
  orc_matvec(W->w_qkv, dt, nq + 2 * nkv, H, u, qkv);
  for (int h = 0; h < Hq; ++h) orc_rope(qkv + (size_t)h * d, d, pos, D->rope_theta);
  for (int g = 0; g < Hkv; ++g) orc_rope(qkv + nq + (size_t)g * d, d, pos, D->rope_theta);
  size_t half = (size_t)D->max_batch * Hkv * (size_t)D->max_seq * d;   /* K block, then V block */
  char* base = (char*)kv;
  size_t eb = dt == ORC_BF16 ? 2 : 4;
  void* K = base + eb * ((size_t)b * Hkv * (size_t)D->max_seq * d);
  void* V = base + eb * (half + (size_t)b * Hkv * (size_t)D->max_seq * d);
  for (int g = 0; g < Hkv && !given_append; ++g)
    for (int t = 0; t < d; ++t) {
      size_t off = ((size_t)g * D->max_seq + (size_t)pos) * d + t;
      st(K, dt, off, qkv[nq + (size_t)g * d + t]);
      st(V, dt, off, qkv[nq + nkv + (size_t)g * d + t]);
    }
  orc_attention(qkv, K, V, dt, Hq, Hkv, d, D->max_seq, pos + 1, o);
  orc_matvec(W->w_o, dt, H, nq, o, h1);
  for (int i = 0; i < H; ++i) h1[i] += x[i];
  free(u);
  free(qkv);
  free(o);
}

/* SwiGLU FFN: out = W_down (silu(W_gate u) * (W_up u)). */
static void swiglu_ffn(const void* Wg, const void* Wu, const void* Wd, int dt, int H, int F, const double* u, double* out) {
  double* g = (double*)malloc(sizeof(double) * F);
  double* v = (double*)malloc(sizeof(double) * F);
  orc_matvec(Wg, dt, F, H, u, g);
  orc_matvec(Wu, dt, F, H, u, v);
  for (int j = 0; j < F; ++j) g[j] = orc_silu(g[j]) * v[j];
  orc_matvec(Wd, dt, H, F, g, out);
  free(g);
  free(v);
}

static int check_desc(const orc_desc* D) {
  if (D->n_q_heads <= 0 || D->n_kv_heads <= 0 || D->n_q_heads % D->n_kv_heads) return -1;
  if (D->head_dim <= 0 || D->head_dim % 2) return -1;
  if (D->hidden <= 0 || D->max_batch <= 0 || D->max_seq <= 0) return -1;
  if (D->dtype != ORC_F32 && D->dtype != ORC_BF16) return -1;
  return 0;
}

/* One dense decoder layer over a batch: for each request b (independently),
 * h1 = attention half; x' = h1 + FFN(RMSNorm(h1; ffn_norm)). hidden is
 * [batch][H] doubles, updated in place; kv is this layer's cache block. */
static int decode_layer_impl(const orc_desc* D, const orc_layer* W, void* kv, const int32_t* seq_lens, int batch,
                             double* hidden, int given_append) {
  if (check_desc(D) || batch < 0 || batch > D->max_batch || D->ffn_dim <= 0) return -1;
  for (int b = 0; b < batch; ++b)
    if (seq_lens[b] < 0 || seq_lens[b] >= D->max_seq) return -2;
  int H = D->hidden;
  double* h1 = (double*)malloc(sizeof(double) * H);
  double* u2 = (double*)malloc(sizeof(double) * H);
  double* f = (double*)malloc(sizeof(double) * H);
  for (int b = 0; b < batch; ++b) {
    double* x = hidden + (size_t)b * H;
    attn_half(D, W, kv, b, seq_lens[b], x, h1, given_append);
    orc_rmsnorm(h1, W->ffn_norm, H, D->rms_eps, u2);
    swiglu_ffn(W->w_gate, W->w_up, W->w_down, D->dtype, H, D->ffn_dim, u2, f);
    for (int i = 0; i < H; ++i) x[i] = h1[i] + f[i];
  }
  free(h1);
  free(u2);
  free(f);
  return 0;
}

int orc_decode_layer(const orc_desc* D, const orc_layer* W, void* kv, const int32_t* seq_lens, int batch, double* hidden) {
  return decode_layer_impl(D, W, kv, seq_lens, batch, hidden, 0);
}

/* The same layer with each request's new K/V entry read from slot seq_len of
 * kv as given, not appended (see attn_half). */
int orc_decode_layer_given_append(const orc_desc* D, const orc_layer* W, void* kv, const int32_t* seq_lens, int batch,
                                  double* hidden) {
  return decode_layer_impl(D, W, kv, seq_lens, batch, hidden, 1);
}

/* The stack: layer l's output is layer l+1's input; no final norm. */
int orc_decode_stack(const orc_desc* D, const orc_layer* layers, void* kv, const int32_t* seq_lens, int batch, double* hidden) {
  size_t eb = D->dtype == ORC_BF16 ? 2 : 4;
  for (int l = 0; l < D->n_layers; ++l) {
    int rc = orc_decode_layer(D, &layers[l], (char*)kv + eb * kv_layer_elems(D) * (size_t)l, seq_lens, batch, hidden);
    if (rc) return rc;
  }
  return 0;
}

/* Gates for a given selection: the softmax over the selected logits, taken
 * in selection order (the renormalised full softmax restricted to idx). */
static void sel_gates(const float* z, const int32_t* idx, int k, double* w) {
  double zmax = (double)z[idx[0]], sum = 0.0;
  for (int j = 0; j < k; ++j) { w[j] = exp((double)z[idx[j]] - zmax); sum += w[j]; }
  for (int j = 0; j < k; ++j) w[j] /= sum;
}

/* One MoE decoder layer over T tokens, each token its own request:
 *   h1 = attention half; u2 = RMSNorm(h1; ffn_norm);
 *   z = W_router u2 (rounded to float32: the decision precision);
 *   (idx, w) = top-k of z with renormalised softmax gates;
 *   x' = h1 + sum_j w_j * SwiGLU_{idx_j}(u2)      (summed in slot order j = 0..k-1);
 * and the grouping of all tokens' choices (orc_group). Each routing output is
 * optional (NULL skips it). With force_idx (T x k), the selection is taken
 * from there instead of from top-k (gates: the softmax over this layer's own
 * logits at the given experts), for comparing a token that another
 * implementation routed differently at a near tie. */
static int moe_layer_impl(const orc_desc* D, const orc_layer* W, void* kv, const int32_t* seq_lens, int T, int bm,
                          double* hidden, float* logits, int32_t* topk_idx, double* topk_w, int32_t* exp_indptr,
                          int32_t* tile_indptr, int32_t* sorted_tok, int32_t* sorted_slot,
                          const int32_t* force_idx) {
  if (check_desc(D) || T < 0 || T > D->max_batch || D->n_experts <= 0 || D->top_k <= 0 ||
      D->top_k > D->n_experts || D->expert_ffn_dim <= 0 || bm <= 0)
    return -1;
  for (int t = 0; t < T; ++t)
    if (seq_lens[t] < 0 || seq_lens[t] >= D->max_seq) return -2;
  int H = D->hidden, E = D->n_experts, k = D->top_k, Fe = D->expert_ffn_dim, dt = D->dtype;
  size_t eb = dt == ORC_BF16 ? 2 : 4;
  double* h1 = (double*)malloc(sizeof(double) * H);
  double* u2 = (double*)malloc(sizeof(double) * H);
  double* f = (double*)malloc(sizeof(double) * H);
  double* zd = (double*)malloc(sizeof(double) * E);
  float* z = (float*)malloc(sizeof(float) * E);
  int32_t* all_idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * k);
  double* w = (double*)malloc(sizeof(double) * k);
  for (int t = 0; t < T; ++t) {
    double* x = hidden + (size_t)t * H;
    attn_half(D, W, kv, t, seq_lens[t], x, h1, 0);
    orc_rmsnorm(h1, W->ffn_norm, H, D->rms_eps, u2);
    orc_matvec(W->w_router, dt, E, H, u2, zd);
    for (int e = 0; e < E; ++e) z[e] = (float)zd[e];
    int32_t* idx = all_idx + (size_t)t * k;
    if (force_idx) {
      for (int j = 0; j < k; ++j) {
        idx[j] = force_idx[(size_t)t * k + j];
        if (idx[j] < 0 || idx[j] >= E) { free(h1); free(u2); free(f); free(zd); free(z); free(all_idx); free(w); return -3; }
      }
      sel_gates(z, idx, k, w);
    } else {
      orc_topk(z, E, k, idx, w);
    }
    for (int i = 0; i < H; ++i) x[i] = h1[i];
    for (int j = 0; j < k; ++j) {
      int e = idx[j];
      const char* wg = (const char*)W->w_exp_gate + eb * (size_t)e * Fe * H;
      const char* wu = (const char*)W->w_exp_up + eb * (size_t)e * Fe * H;
      const char* wd = (const char*)W->w_exp_down + eb * (size_t)e * H * Fe;
      swiglu_ffn(wg, wu, wd, dt, H, Fe, u2, f);
      for (int i = 0; i < H; ++i) x[i] += w[j] * f[i];
    }
    if (logits) memcpy(logits + (size_t)t * E, z, sizeof(float) * E);
    if (topk_idx) memcpy(topk_idx + (size_t)t * k, idx, sizeof(int32_t) * k);
    if (topk_w) memcpy(topk_w + (size_t)t * k, w, sizeof(double) * k);
  }
  if (exp_indptr && tile_indptr && sorted_tok && sorted_slot)
    orc_group(all_idx, T, k, E, bm, exp_indptr, tile_indptr, sorted_tok, sorted_slot);
  free(h1); free(u2); free(f); free(zd); free(z); free(all_idx); free(w);
  return 0;
}

int orc_moe_layer(const orc_desc* D, const orc_layer* W, void* kv, const int32_t* seq_lens, int T, int bm,
                  double* hidden, float* logits, int32_t* topk_idx, double* topk_w, int32_t* exp_indptr,
                  int32_t* tile_indptr, int32_t* sorted_tok, int32_t* sorted_slot) {
  return moe_layer_impl(D, W, kv, seq_lens, T, bm, hidden, logits, topk_idx, topk_w, exp_indptr, tile_indptr,
                        sorted_tok, sorted_slot, NULL);
}

/* The same layer with the experts of every token given (force_idx, T x k). */
int orc_moe_layer_routed(const orc_desc* D, const orc_layer* W, void* kv, const int32_t* seq_lens, int T,
                         const int32_t* force_idx, double* hidden, double* topk_w) {
  if (!force_idx) return -1;
  return moe_layer_impl(D, W, kv, seq_lens, T, 1, hidden, NULL, NULL, topk_w, NULL, NULL, NULL, NULL, force_idx);
}
