/*
 * CPU oracle for the batched decode step — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The GPU product path neither links nor calls it, and it
 * shares no code with the GPU path.
 *
 * What it computes: the plain definition of one decode step of a dense Llama
 * decoder, lane by lane, in f32 with fixed-order scalar arithmetic.  The
 * method ("MODEL-BATCHING-RESULTS — multi-user batched decode, measured",
 * sections "The lever" and "Correctness — proven, not asserted") stacks one
 * token from each of B users into a [B, *] panel, runs the seven projections
 * and the LM head once over that panel, and keeps attention per user over the
 * user's own cache; it states that this is bit-for-bit the serial per-user
 * step because every output is the same dot product in the same order.  So the
 * oracle is the serial step (orc_step), plus a panel mode (orc_step_batch,
 * weight rows outer, lanes inner) that must equal it bitwise.
 *
 * Layer math (the pages name only "dense-Llama" and "SwiGLU"; the standard
 * pre-norm Llama decoder is taken as the plainest reading):
 *   x  = E[token]
 *   per layer:  xn = rmsnorm(x, g_attn);  q,k,v = Wq xn, Wk xn, Wv xn
 *               rotate q and k at the lane's position p (rotate-half pairs)
 *               append k, v at slot p;  o_h = softmax_t(q_h.K_t / sqrt(hd)) V
 *               over t = 0..p, KV head of query head h = h / (Hq / Hkv)
 *               x += Wo o;  xn = rmsnorm(x, g_ffn)
 *               x += Wd (silu(Wg xn) * (Wu xn))
 *   logits = Wlm rmsnorm(x, g_final)   (Wlm = E when tied)
 * The per-lane rotary position is the lane's own pre-write position, used for
 * both q and k ("parallel-slots.md", section "S1b decode: design traps",
 * trap 2, and "The one genuinely hard problem: per-sequence position").
 *
 * Precision modes (wtype): f32 weights — all f32.  bf16 weights ("bf16
 * weights/activations, f32 accumulate"): weights are upcast exactly, the
 * inputs of every projection (xn, o, the SwiGLU output, the final xn) and the
 * stored K/V are rounded to bf16; accumulation, residual stream, norm
 * statistics, softmax and logits stay f32.  Q8_0 weights: each weight is
 * q * f32(scale) of its block of 32 along K; activations and KV f32.
 *
 * Build: -O2 -fno-fast-math -ffp-contract=off; OpenMP splits output rows (or
 * attention heads) across threads, which does not change any value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_Q8_0 = 2 };

/* Accumulator of every sum (dot products, sums of squares, softmax sums, the
 * weighted value sum): the sums are computed exactly up to double rounding and
 * rounded to f32 where the definition stores a value. */
#ifndef ORC_ACC
#define ORC_ACC double
#endif
typedef ORC_ACC acc_t;

typedef struct {
  int d, n_layers, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps, rope_theta;
  int tied;
  int wtype;
} orc_config;

/* One weight matrix [N, K] row-major.  data: float (f32), uint16 bf16 bits
 * (bf16) or int8 (Q8_0); scale: binary16 bits [N, K/32] for Q8_0, else NULL. */
typedef struct {
  const void* data;
  const uint16_t* scale;
} orc_mat;

typedef struct {
  orc_mat embed, lm_head;
  const float* final_norm;
  const float* const* attn_norm; /* [L] of [d] */
  const float* const* ffn_norm;  /* [L] of [d] */
  const orc_mat* w_qkv;          /* [L]: [(Hq+2Hkv)*hd, d], q rows then k rows then v rows */
  const orc_mat* w_o;            /* [L]: [d, Hq*hd] */
  const orc_mat* w_gu;           /* [L]: [2F, d], gate rows then up rows */
  const orc_mat* w_down;         /* [L]: [d, F] */
} orc_weights;

typedef struct {
  orc_config c;
  orc_mat embed, head;
  const float* final_norm;
  const float** attn_norm;
  const float** ffn_norm;
  orc_mat *w_qkv, *w_o, *w_gu, *w_down;
} orc_model;

typedef struct {
  int max_seq, length;
  int L, kvd; /* layers, Hkv*hd */
  float* K;   /* [L][max_seq][Hkv*hd] (rotated keys) */
  float* V;   /* [L][max_seq][Hkv*hd] */
} orc_lane;

/* ---- number formats ------------------------------------------------------- */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round an f32 to the nearest bf16 value (ties to even), returned as f32. */
float orc_round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return f;
  u += 0x7fffu + ((u >> 16) & 1u);
  u &= 0xffff0000u;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE binary16 bits -> f32 (exact). */
float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  float v;
  if (ex == 0) {
    v = ldexpf((float)man, -24);
  } else if (ex == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexpf((float)(man | 0x400), ex - 25);
  }
  return sign ? -v : v;
}

/* Weight element W[r][i] as f32: plain value, exact bf16 upcast, or the Q8_0
 * dequantised value q * scale (an exact product: 8-bit times 11-bit). */
static inline float wval(const orc_mat* W, int wtype, int64_t K, int64_t r, int64_t i) {
  if (wtype == ORC_F32) return ((const float*)W->data)[r * K + i];
  if (wtype == ORC_BF16) return bf16_to_f32(((const uint16_t*)W->data)[r * K + i]);
  float q = (float)((const int8_t*)W->data)[r * K + i];
  return q * orc_f16_to_f32(W->scale[r * (K / 32) + i / 32]);
}

/* The one dot product every projection uses: sum_{i=0}^{K-1} W[r][i] * x[i]
 * in ascending i, products and sum in the accumulator type, the result
 * rounded to f32. */
static float dot_row(const orc_mat* W, int wtype, int64_t K, int64_t r, const float* x) {
  acc_t acc = 0;
  for (int64_t i = 0; i < K; ++i) acc += (acc_t)wval(W, wtype, K, r, i) * (acc_t)x[i];
  return (float)acc;
}

/* ---- pieces, exported so tests can pin them one by one ------------------- */

/* y[r] = dot_row(W, row0 + r, x) for r in [0, nrows). */
void orc_matvec(const orc_mat* W, int wtype, int row0, int nrows, int K, const float* x, float* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < nrows; ++r) y[r] = dot_row(W, wtype, K, (int64_t)row0 + r, x);
}

/* out_i = (x_i * r) * g_i with r = 1 / sqrt(mean(x^2) + eps); the sum of
 * squares runs in ascending i in the accumulator type; the mean is rounded to
 * f32 and r computed in f32. */
void orc_rmsnorm(const float* x, const float* g, int n, float eps, float* out) {
  acc_t ss = 0;
  for (int i = 0; i < n; ++i) ss += (acc_t)x[i] * (acc_t)x[i];
  float ms = (float)(ss / (acc_t)n);
  float r = 1.0f / sqrtf(ms + eps);
  for (int i = 0; i < n; ++i) out[i] = (x[i] * r) * g[i];
}

/* Rotary angles of position pos: theta_j = theta^(-2j/hd), a = pos * theta_j,
 * all in double; cos and sin rounded to f32.  j in [0, hd/2). */
void orc_rope_cs(int hd, int pos, float theta, float* c, float* s) {
  for (int j = 0; j < hd / 2; ++j) {
    double th = pow((double)theta, -(2.0 * (double)j) / (double)hd);
    double a = (double)pos * th;
    c[j] = (float)cos(a);
    s[j] = (float)sin(a);
  }
}

/* Rotate one head vector in place, rotate-half pairing (j, j + hd/2). */
void orc_rope(float* v, int hd, int pos, float theta) {
  float c[512], s[512];
  int h = hd / 2;
  orc_rope_cs(hd, pos, theta, c, s);
  for (int j = 0; j < h; ++j) {
    float a = v[j], b = v[j + h];
    v[j] = a * c[j] - b * s[j];
    v[j + h] = b * c[j] + a * s[j];
  }
}

float orc_silu(float u) { return u / (1.0f + expf(-u)); }

/* Attention of one lane over its n_keys cached positions (the new one
 * included).  q: [Hq*hd]; Kc, Vc: rows of Hkv*hd floats, row stride kv_stride;
 * out: [Hq*hd].  Query head h reads KV head h / (Hq/Hkv). */
void orc_attention(const float* q, const float* Kc, const float* Vc, int64_t kv_stride, int n_keys, int Hq,
                   int Hkv, int hd, float* out) {
  int grp = Hq / Hkv;
  float inv = 1.0f / sqrtf((float)hd);
#pragma omp parallel for schedule(static)
  for (int h = 0; h < Hq; ++h) {
    int g = h / grp;
    const float* qh = q + (int64_t)h * hd;
    float* sc = (float*)malloc(sizeof(float) * (size_t)n_keys);
    acc_t* oa = (acc_t*)malloc(sizeof(acc_t) * (size_t)hd);
    float m = -INFINITY;
    for (int t = 0; t < n_keys; ++t) {
      const float* kt = Kc + (int64_t)t * kv_stride + (int64_t)g * hd;
      acc_t dot = 0;
      for (int i = 0; i < hd; ++i) dot += (acc_t)qh[i] * (acc_t)kt[i];
      sc[t] = (float)dot * inv;
      if (sc[t] > m) m = sc[t];
    }
    acc_t Z = 0;
    for (int t = 0; t < n_keys; ++t) {
      sc[t] = expf(sc[t] - m);
      Z += sc[t];
    }
    for (int i = 0; i < hd; ++i) oa[i] = 0;
    for (int t = 0; t < n_keys; ++t) {
      const float* vt = Vc + (int64_t)t * kv_stride + (int64_t)g * hd;
      for (int i = 0; i < hd; ++i) oa[i] += (acc_t)sc[t] * (acc_t)vt[i];
    }
    float* oh = out + (int64_t)h * hd;
    for (int i = 0; i < hd; ++i) oh[i] = (float)(oa[i] / Z);
    free(oa);
    free(sc);
  }
}

int orc_argmax(const float* x, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (x[i] > x[best]) best = i; /* strict: the lowest index wins ties */
  return best;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- model and lanes ----------------------------------------------------- */

orc_model* orc_model_create(const orc_config* c, const orc_weights* w) {
  if (c->n_heads % c->n_kv_heads != 0 || c->head_dim % 2 != 0 || c->head_dim > 1024) return NULL;
  if (c->wtype == ORC_Q8_0 && (c->d % 32 != 0 || c->ffn % 32 != 0 || (c->n_heads * c->head_dim) % 32 != 0))
    return NULL;
  orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
  int L = c->n_layers;
  m->c = *c;
  m->embed = w->embed;
  m->head = c->tied ? w->embed : w->lm_head;
  m->final_norm = w->final_norm;
  m->attn_norm = (const float**)malloc(sizeof(float*) * L);
  m->ffn_norm = (const float**)malloc(sizeof(float*) * L);
  m->w_qkv = (orc_mat*)malloc(sizeof(orc_mat) * L);
  m->w_o = (orc_mat*)malloc(sizeof(orc_mat) * L);
  m->w_gu = (orc_mat*)malloc(sizeof(orc_mat) * L);
  m->w_down = (orc_mat*)malloc(sizeof(orc_mat) * L);
  for (int l = 0; l < L; ++l) {
    m->attn_norm[l] = w->attn_norm[l];
    m->ffn_norm[l] = w->ffn_norm[l];
    m->w_qkv[l] = w->w_qkv[l];
    m->w_o[l] = w->w_o[l];
    m->w_gu[l] = w->w_gu[l];
    m->w_down[l] = w->w_down[l];
  }
  return m;
}

void orc_model_destroy(orc_model* m) {
  if (!m) return;
  free(m->attn_norm); free(m->ffn_norm);
  free(m->w_qkv); free(m->w_o); free(m->w_gu); free(m->w_down);
  free(m);
}

orc_lane* orc_lane_create(const orc_model* m, int max_seq) {
  orc_lane* ln = (orc_lane*)calloc(1, sizeof(orc_lane));
  ln->max_seq = max_seq;
  ln->L = m->c.n_layers;
  ln->kvd = m->c.n_kv_heads * m->c.head_dim;
  size_t n = (size_t)ln->L * max_seq * ln->kvd;
  ln->K = (float*)calloc(n, sizeof(float));
  ln->V = (float*)calloc(n, sizeof(float));
  if (!ln->K || !ln->V) { free(ln->K); free(ln->V); free(ln); return NULL; }
  return ln;
}

void orc_lane_destroy(orc_lane* ln) {
  if (!ln) return;
  free(ln->K); free(ln->V); free(ln);
}

void orc_lane_clear(orc_lane* ln) { ln->length = 0; }
int orc_lane_length(const orc_lane* ln) { return ln->length; }

/* KV exchange layout: [L][Hkv][length][hd]. */
int orc_lane_set_kv(orc_lane* ln, int length, int hd, const float* k, const float* v) {
  if (length < 0 || length > ln->max_seq) return -1;
  int hkv = ln->kvd / hd;
  for (int l = 0; l < ln->L; ++l)
    for (int g = 0; g < hkv; ++g)
      for (int t = 0; t < length; ++t)
        for (int i = 0; i < hd; ++i) {
          int64_t src = (((int64_t)l * hkv + g) * length + t) * hd + i;
          int64_t dst = ((int64_t)l * ln->max_seq + t) * ln->kvd + (int64_t)g * hd + i;
          ln->K[dst] = k[src];
          ln->V[dst] = v[src];
        }
  ln->length = length;
  return 0;
}

int orc_lane_get_kv(const orc_lane* ln, int hd, float* k, float* v) {
  int hkv = ln->kvd / hd, length = ln->length;
  for (int l = 0; l < ln->L; ++l)
    for (int g = 0; g < hkv; ++g)
      for (int t = 0; t < length; ++t)
        for (int i = 0; i < hd; ++i) {
          int64_t dst = (((int64_t)l * hkv + g) * length + t) * hd + i;
          int64_t src = ((int64_t)l * ln->max_seq + t) * ln->kvd + (int64_t)g * hd + i;
          k[dst] = ln->K[src];
          v[dst] = ln->V[src];
        }
  return length;
}

/* Rounding applied to projection inputs and to stored K/V in bf16 mode. */
static void round_act(const orc_model* m, float* x, int n) {
  if (m->c.wtype != ORC_BF16) return;
  for (int i = 0; i < n; ++i) x[i] = orc_round_bf16(x[i]);
}

/* Evict the span [begin, end) of a lane: the per-user Evict ("quarantine a
 * poisoned span") of "MODEL-BATCHING-RESULTS — multi-user batched decode,
 * measured" (section "Why in-kernel batching, not vLLM").  The page keeps
 * each user's raw keys beside the rotated ones for it; this cache stores keys
 * rotated at their own positions only, so the reading taken is: entries at
 * t >= end move to t - d (d = end - begin), their stored keys rotated by the
 * rotary angle of -d positions (orc_rope at position -d: the composition of
 * rotations by p and by -d is the rotation by p - d) and rounded to the KV
 * format; values move unchanged; the length drops by d.  Returns -1 for a
 * span outside [0, length]. */
int orc_lane_evict_span(const orc_model* m, orc_lane* ln, int begin, int end) {
  const orc_config* c = &m->c;
  if (begin < 0 || end < begin || end > ln->length) return -1;
  int d = end - begin, hd = c->head_dim, kvd = ln->kvd;
  if (d == 0) return 0;
  for (int l = 0; l < ln->L; ++l) {
    float* Kl = ln->K + (int64_t)l * ln->max_seq * kvd;
    float* Vl = ln->V + (int64_t)l * ln->max_seq * kvd;
    for (int t = end; t < ln->length; ++t) {
      float* kd = Kl + (int64_t)(t - d) * kvd;
      memcpy(kd, Kl + (int64_t)t * kvd, sizeof(float) * kvd);
      memcpy(Vl + (int64_t)(t - d) * kvd, Vl + (int64_t)t * kvd, sizeof(float) * kvd);
      for (int g = 0; g < c->n_kv_heads; ++g) orc_rope(kd + (int64_t)g * hd, hd, -d, c->rope_theta);
      round_act(m, kd, kvd);
    }
  }
  ln->length -= d;
  return 0;
}

static void embed_row(const orc_model* m, int token, float* x) {
  for (int i = 0; i < m->c.d; ++i) x[i] = wval(&m->embed, m->c.wtype, m->c.d, token, i);
}

/* Everything of one layer that follows the q/k/v projection, for one lane:
 * rotary, append, attention; the o projection is done by the caller. */
static void rope_append_attend(const orc_model* m, orc_lane* ln, int l, float* q, float* k, const float* v,
                               float* o) {
  const orc_config* c = &m->c;
  int hd = c->head_dim, p = ln->length;
  for (int h = 0; h < c->n_heads; ++h) orc_rope(q + (int64_t)h * hd, hd, p, c->rope_theta);
  for (int g = 0; g < c->n_kv_heads; ++g) orc_rope(k + (int64_t)g * hd, hd, p, c->rope_theta);
  int kvd = ln->kvd;
  float* Kl = ln->K + (int64_t)l * ln->max_seq * kvd;
  float* Vl = ln->V + (int64_t)l * ln->max_seq * kvd;
  memcpy(Kl + (int64_t)p * kvd, k, sizeof(float) * kvd);
  memcpy(Vl + (int64_t)p * kvd, v, sizeof(float) * kvd);
  round_act(m, Kl + (int64_t)p * kvd, kvd);
  round_act(m, Vl + (int64_t)p * kvd, kvd);
  orc_attention(q, Kl, Vl, kvd, p + 1, c->n_heads, c->n_kv_heads, hd, o);
}

/* One serial decode step of one lane: token in, f32 logits [vocab] out. */
int orc_step(const orc_model* m, orc_lane* ln, int token, float* logits) {
  const orc_config* c = &m->c;
  if (token < 0 || token >= c->vocab || ln->length >= ln->max_seq) return -1;
  int d = c->d, hd = c->head_dim, F = c->ffn, wt = c->wtype;
  int qd = c->n_heads * hd, kvd = c->n_kv_heads * hd;
  float* x = (float*)malloc(sizeof(float) * d);
  float* xn = (float*)malloc(sizeof(float) * d);
  float* q = (float*)malloc(sizeof(float) * qd);
  float* k = (float*)malloc(sizeof(float) * kvd);
  float* v = (float*)malloc(sizeof(float) * kvd);
  float* o = (float*)malloc(sizeof(float) * qd);
  float* y = (float*)malloc(sizeof(float) * (d > F ? d : F));
  float* gt = (float*)malloc(sizeof(float) * F);
  float* up = (float*)malloc(sizeof(float) * F);
  embed_row(m, token, x);
  for (int l = 0; l < c->n_layers; ++l) {
    orc_rmsnorm(x, m->attn_norm[l], d, c->rms_eps, xn);
    round_act(m, xn, d);
    orc_matvec(&m->w_qkv[l], wt, 0, qd, d, xn, q);
    orc_matvec(&m->w_qkv[l], wt, qd, kvd, d, xn, k);
    orc_matvec(&m->w_qkv[l], wt, qd + kvd, kvd, d, xn, v);
    rope_append_attend(m, ln, l, q, k, v, o);
    round_act(m, o, qd);
    orc_matvec(&m->w_o[l], wt, 0, d, qd, o, y);
    for (int i = 0; i < d; ++i) x[i] = x[i] + y[i];
    orc_rmsnorm(x, m->ffn_norm[l], d, c->rms_eps, xn);
    round_act(m, xn, d);
    orc_matvec(&m->w_gu[l], wt, 0, F, d, xn, gt);
    orc_matvec(&m->w_gu[l], wt, F, F, d, xn, up);
    for (int i = 0; i < F; ++i) gt[i] = orc_silu(gt[i]) * up[i];
    round_act(m, gt, F);
    orc_matvec(&m->w_down[l], wt, 0, d, F, gt, y);
    for (int i = 0; i < d; ++i) x[i] = x[i] + y[i];
  }
  orc_rmsnorm(x, m->final_norm, d, c->rms_eps, xn);
  round_act(m, xn, d);
  orc_matvec(&m->head, wt, 0, c->vocab, d, xn, logits);
  ln->length += 1;
  free(x); free(xn); free(q); free(k); free(v); free(o); free(y); free(gt); free(up);
  return 0;
}

/* Panel product: Y[b][r] = dot_row(W, row0 + r, X[b]) for every lane b,
 * weight rows outer (each row is visited once for the whole panel), lanes
 * inner.  Y has row stride ldy, X row stride K. */
static void panel(const orc_mat* W, int wtype, int row0, int nrows, int K, int B, const float* X, float* Y,
                  int ldy) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < nrows; ++r)
    for (int b = 0; b < B; ++b) Y[(int64_t)b * ldy + r] = dot_row(W, wtype, K, (int64_t)row0 + r, X + (int64_t)b * K);
}

/* One batched decode step over B lanes (distinct lanes, one token each):
 * logits [B][vocab].  Every projection and the head run once over the panel;
 * attention stays per lane. */
int orc_step_batch(const orc_model* m, orc_lane* const* lanes, int B, const int* tokens, float* logits) {
  const orc_config* c = &m->c;
  for (int b = 0; b < B; ++b) {
    if (tokens[b] < 0 || tokens[b] >= c->vocab || lanes[b]->length >= lanes[b]->max_seq) return -1;
    for (int b2 = 0; b2 < b; ++b2)
      if (lanes[b2] == lanes[b]) return -2;
  }
  int d = c->d, hd = c->head_dim, F = c->ffn, wt = c->wtype;
  int qd = c->n_heads * hd, kvd = c->n_kv_heads * hd;
  float* x = (float*)malloc(sizeof(float) * (size_t)B * d);
  float* xn = (float*)malloc(sizeof(float) * (size_t)B * d);
  float* q = (float*)malloc(sizeof(float) * (size_t)B * qd);
  float* k = (float*)malloc(sizeof(float) * (size_t)B * kvd);
  float* v = (float*)malloc(sizeof(float) * (size_t)B * kvd);
  float* o = (float*)malloc(sizeof(float) * (size_t)B * qd);
  float* y = (float*)malloc(sizeof(float) * (size_t)B * d);
  float* gt = (float*)malloc(sizeof(float) * (size_t)B * F);
  float* up = (float*)malloc(sizeof(float) * (size_t)B * F);
  for (int b = 0; b < B; ++b) embed_row(m, tokens[b], x + (int64_t)b * d);
  for (int l = 0; l < c->n_layers; ++l) {
    for (int b = 0; b < B; ++b) {
      orc_rmsnorm(x + (int64_t)b * d, m->attn_norm[l], d, c->rms_eps, xn + (int64_t)b * d);
      round_act(m, xn + (int64_t)b * d, d);
    }
    panel(&m->w_qkv[l], wt, 0, qd, d, B, xn, q, qd);
    panel(&m->w_qkv[l], wt, qd, kvd, d, B, xn, k, kvd);
    panel(&m->w_qkv[l], wt, qd + kvd, kvd, d, B, xn, v, kvd);
    for (int b = 0; b < B; ++b) {
      rope_append_attend(m, lanes[b], l, q + (int64_t)b * qd, k + (int64_t)b * kvd, v + (int64_t)b * kvd,
                         o + (int64_t)b * qd);
      round_act(m, o + (int64_t)b * qd, qd);
    }
    panel(&m->w_o[l], wt, 0, d, qd, B, o, y, d);
    for (int64_t i = 0; i < (int64_t)B * d; ++i) x[i] = x[i] + y[i];
    for (int b = 0; b < B; ++b) {
      orc_rmsnorm(x + (int64_t)b * d, m->ffn_norm[l], d, c->rms_eps, xn + (int64_t)b * d);
      round_act(m, xn + (int64_t)b * d, d);
    }
    panel(&m->w_gu[l], wt, 0, F, d, B, xn, gt, F);
    panel(&m->w_gu[l], wt, F, F, d, B, xn, up, F);
    for (int64_t i = 0; i < (int64_t)B * F; ++i) gt[i] = orc_silu(gt[i]) * up[i];
    for (int b = 0; b < B; ++b) round_act(m, gt + (int64_t)b * F, F);
    panel(&m->w_down[l], wt, 0, d, F, B, gt, y, d);
    for (int64_t i = 0; i < (int64_t)B * d; ++i) x[i] = x[i] + y[i];
  }
  /* every layer wrote slot `length` of each lane; the lengths advance once per step */
  for (int b = 0; b < B; ++b) lanes[b]->length += 1;
  for (int b = 0; b < B; ++b) {
    orc_rmsnorm(x + (int64_t)b * d, m->final_norm, d, c->rms_eps, xn + (int64_t)b * d);
    round_act(m, xn + (int64_t)b * d, d);
  }
  panel(&m->head, wt, 0, c->vocab, d, B, xn, logits, c->vocab);
  free(x); free(xn); free(q); free(k); free(v); free(o); free(y); free(gt); free(up);
  return 0;
}
