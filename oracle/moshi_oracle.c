/*
 * moshi_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded fp64 CPU reference of one Moshi/PersonaPlex
 * RQ-Transformer frame step. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it. The HIP library shares no code,
 * header, table or helper with it.
 *
 * What it computes, and where the pages say so:
 *  - 17-channel token column (text, 8 agent codes, 8 user codes), one
 *    embedding per channel, summed ("vLLM-Omni recipe: PersonaPlex",
 *    section "Architecture (Moshi RQ-Transformer, all native)").
 *  - Temporal transformer: 4096-d, 32 layers, RoPE, sliding-window causal
 *    attention, SwiGLU via a fused gate/up projection, RMSNorm eps 1e-8
 *    (mobius PR #368, commit "P2 - Moshi LM", the models/moshi.py bullet and
 *    the PR summary list); a 3000-frame window kept in a ring KV cache (recipe,
 *    "Architecture"; "Notes", last bullet).
 *  - Text head on the temporal output, greedy (recipe, "Notes": greedy only).
 *  - Depformer: 1024-d, 6 layers, no RoPE, full causal over substeps,
 *    weights_per_step = 16 per-substep linears, one substep consuming the
 *    previous substep's token, text token first (mobius PR #368, "P2 - Moshi
 *    LM" and "P3 - ONNX Runtime example"); reset every frame (recipe,
 *    "Architecture").
 *
 * Readings taken where the pages leave a step open (each is listed with its
 * reason in the design notes of the repository):
 *  - window: the keys attended at position p are positions max(0, p-W+1)..p
 *    (W keys including the current one); with mask_oldest, once p >= W-1 the
 *    oldest of them is masked too (W-1 keys) -- the SGLang cookbook's
 *    "Known limitations" mentions a masked oldest slot once the ring fills;
 *  - RoPE position = number of frames the session has consumed; pairs are
 *    interleaved (2i, 2i+1), inverse frequency theta^(-2i/hd), theta = 1e4;
 *  - one final RMSNorm on the temporal output (its result is the hidden state
 *    handed to both the text head and the depformer); none in the depformer;
 *  - per substep: input projection, every linear of every layer, the head and
 *    the previous-token embedding; RMSNorm gains shared across substeps;
 *  - no biases; attention scale 1/sqrt(head_dim); MHA (K/V heads = heads);
 *  - the fused gate/up matrix holds gate rows first, then up rows;
 *  - argmax ties go to the lowest index;
 *  - bf16 model: every linear's input vector is rounded to bf16 (the normed
 *    vector before each projection, the attention output, the SwiGLU output,
 *    the temporal hidden state, the depformer residual before its head), and
 *    K/V are stored as bf16; everything else is fp64 here. fp32 model: no
 *    rounding points.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t dim, n_layers, n_heads, ffn_hidden, window;
  int32_t dep_dim, dep_layers, dep_heads, dep_ffn_hidden, n_substeps;
  int32_t text_vocab, audio_card;
  double rope_theta, norm_eps;
  int32_t bf16;        /* 1: bf16 weights, K/V and rounding points; 0: fp32, none */
  int32_t mask_oldest; /* window reading flag (see header) */
  int32_t dep_q;          /* depformer substeps run per frame; 0 = all n_substeps */
  int32_t dep_final_norm; /* RMSNorm (gain dep.out_norm) on the residual before each head */
  int32_t dep_ref_ring;   /* mask substep K/V entry 0 at the last substep run */
} orc_config;

typedef struct {
  orc_config c;
  /* temporal */
  const void* emb_text;
  const void** emb_audio; /* [S] */
  const void **attn_norm, **qkv, **wo, **mlp_norm, **gate_up, **down; /* [L] */
  const void* out_norm;
  const void* text_head;
  /* depformer */
  const void** dep_in;  /* [S] */
  const void** dep_emb; /* [S]; 0 = text table */
  const void **dep_attn_norm, **dep_mlp_norm; /* [Ld] */
  const void **dep_qkv, **dep_o, **dep_gate_up, **dep_down; /* [S*Ld] */
  const void** dep_head; /* [S] */
  const void* dep_out_norm; /* [Dd], with dep_final_norm only */
} orc_model;

typedef struct {
  const orc_model* m;
  int64_t pos;
  void* k_ring; /* [L][W][D]: uint16 bf16 bits (bf16 model) or double (fp32 model) */
  void* v_ring;
} orc_session;

/* ------------------------------------------------------------------ */
/* numeric primitives                                                  */
/* ------------------------------------------------------------------ */

/* The bf16 value nearest to v, ties to even (8 significant bits). */
double orc_bf16_round(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  double mant = frexp(v, &e);             /* v = mant * 2^e, 0.5 <= |mant| < 1 */
  if (e - 1 < -126) {                     /* below the smallest normal: fixed step 2^-133 */
    return nearbyint(ldexp(v, 133)) * ldexp(1.0, -133);
  }
  return ldexp(nearbyint(ldexp(mant, 8)), e - 8); /* nearbyint rounds half to even */
}

static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static uint16_t double_to_bf16_bits(double v) {
  float f = (float)orc_bf16_round(v); /* exact: a bf16 value is representable in fp32 */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static inline double rnd(const orc_model* m, double v) { return m->c.bf16 ? orc_bf16_round(v) : v; }

/* Element i of a weight tensor stored in the model's type. */
static inline double wget(const orc_model* m, const void* p, size_t i) {
  return m->c.bf16 ? bf16_bits_to_double(((const uint16_t*)p)[i]) : (double)((const float*)p)[i];
}

/* y = W x, W row-major [N, K] (row n produces output n); no bias. */
static void linear(const orc_model* m, const void* W, int N, int K, const double* x, double* y) {
  for (int n = 0; n < N; ++n) {
    double acc = 0.0;
    size_t base = (size_t)n * (size_t)K;
    if (m->c.bf16) {
      const uint16_t* row = (const uint16_t*)W + base;
      for (int k = 0; k < K; ++k) acc += bf16_bits_to_double(row[k]) * x[k];
    } else {
      const float* row = (const float*)W + base;
      for (int k = 0; k < K; ++k) acc += (double)row[k] * x[k];
    }
    y[n] = acc;
  }
}

/* RMSNorm (mobius PR #368, models/moshi.py bullet: pre-norm, eps 1e-8):
 * out_i = x_i / sqrt(mean(x^2) + eps) * g_i. */
void orc_rmsnorm(const double* x, const double* g, int n, double eps, double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * r * g[i];
}

static void rmsnorm_w(const orc_model* m, const double* x, const void* g, int n, double* out) {
  double* gd = (double*)malloc(sizeof(double) * n);
  for (int i = 0; i < n; ++i) gd[i] = wget(m, g, i);
  orc_rmsnorm(x, gd, n, m->c.norm_eps, out);
  free(gd);
}

/* Rotary position embedding at position pos, in place, for n_heads heads of
 * head_dim each (mobius PR #368: RoPE theta 1e4, offset from the cache length).
 * Interleaved pairs: (v[2i], v[2i+1]) rotates by pos * theta^(-2i/head_dim). */
void orc_rope(double* v, int n_heads, int head_dim, int64_t pos, double theta) {
  for (int h = 0; h < n_heads; ++h) {
    double* x = v + (size_t)h * head_dim;
    for (int i = 0; i < head_dim / 2; ++i) {
      double ang = (double)pos * pow(theta, -2.0 * i / head_dim);
      double c = cos(ang), s = sin(ang);
      double a = x[2 * i], b = x[2 * i + 1];
      x[2 * i] = a * c - b * s;
      x[2 * i + 1] = a * s + b * c;
    }
  }
}

/* One attention head over n keys: o = sum_j softmax_j(q.k_j / sqrt(hd)) v_j.
 * keys/vals are n rows of hd (row stride `stride`). Softmax subtracts the max. */
void orc_attend(const double* q, const double* keys, const double* vals, int n, int hd,
                int stride, double* o) {
  for (int d = 0; d < hd; ++d) o[d] = 0.0;
  if (n <= 0) return;
  double* s = (double*)malloc(sizeof(double) * n);
  double scale = 1.0 / sqrt((double)hd);
  double mx = -INFINITY;
  for (int j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int d = 0; d < hd; ++d) acc += q[d] * keys[(size_t)j * stride + d];
    s[j] = acc * scale;
    if (s[j] > mx) mx = s[j];
  }
  double den = 0.0;
  for (int j = 0; j < n; ++j) {
    s[j] = exp(s[j] - mx);
    den += s[j];
  }
  for (int j = 0; j < n; ++j) {
    double p = s[j] / den;
    for (int d = 0; d < hd; ++d) o[d] += p * vals[(size_t)j * stride + d];
  }
  free(s);
}

/* SiLU(z) = z / (1 + e^-z). */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Greedy choice: the index of the largest value, lowest index on ties.
 * *margin = top1 - top2 (0 on a tie). */
int32_t orc_argmax(const double* v, int n, double* margin) {
  int32_t best = 0;
  for (int i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  double second = -INFINITY;
  for (int i = 0; i < n; ++i)
    if (i != best && v[i] > second) second = v[i];
  if (margin) *margin = (n > 1) ? v[best] - second : INFINITY;
  return best;
}

/* ------------------------------------------------------------------ */
/* sampling (SGLang-Omni cookbook "PersonaPlex", "Request parameters":  */
/* text temperature/top-k 0.7/25, audio 0.8/250, a seed that makes both */
/* draws reproducible with a child seed each; mobius PR #368's sampling  */
/* commit: temperature + top-k instead of greedy)                        */
/* ------------------------------------------------------------------ */

/* splitmix64's output function (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", 2014): the generator adds the golden
 * gamma to its state and returns this mix of the new state. */
static uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

/* Output n (n >= 1) of a splitmix64 generator seeded with `seed`. */
uint64_t orc_splitmix64(uint64_t seed, uint64_t n) { return sm64_mix(seed + n * SM64_GAMMA); }

/* The uniform draw in [0, 1) of a session's stream at one frame: the
 * stream's child seed is output stream+1 of the session seed's generator
 * (stream 0: text; 1 + s: depformer substep s), the draw is output pos+1 of
 * the child's generator (pos: frames the session consumed before this one),
 * keeping its top 53 bits. */
double orc_uniform(uint64_t seed, int32_t stream, int64_t pos) {
  uint64_t child = orc_splitmix64(seed, (uint64_t)stream + 1);
  return (double)(orc_splitmix64(child, (uint64_t)pos + 1) >> 11) * (1.0 / 9007199254740992.0);
}

typedef struct {
  float v;
  int32_t i;
} orc_cand;

/* Order of the candidates: larger fp32 value first (IEEE total order: -0
 * below +0), lower index first on equal bits. */
static uint32_t f32_order_key(float v) {
  uint32_t b;
  memcpy(&b, &v, 4);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
static int cand_cmp(const void* a, const void* b) {
  const orc_cand* x = (const orc_cand*)a;
  const orc_cand* y = (const orc_cand*)b;
  uint32_t kx = f32_order_key(x->v), ky = f32_order_key(y->v);
  if (kx != ky) return kx > ky ? -1 : 1;
  return x->i < y->i ? -1 : (x->i > y->i);
}

/* Temperature + top-k draw from n logits, decided on their fp32 values:
 * the top_k largest (all of them when top_k <= 0 or >= n) are the
 * candidates; weight w_i = exp((l_i - l_max) / temperature) in fp64; the
 * draw is the first candidate, in ascending index order, whose running sum
 * of weights exceeds u * (sum of all weights); the last candidate if none
 * does. *margin (optional): distance of u * sum to the nearest running sum
 * around the choice, divided by the sum (how far the draw is from choosing
 * a neighbour). temperature must be > 0. */
int32_t orc_sample(const double* logits, int n, double temperature, int top_k, double u,
                   double* margin) {
  int k = (top_k <= 0 || top_k >= n) ? n : top_k;
  orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * n);
  for (int i = 0; i < n; ++i) {
    c[i].v = (float)logits[i];
    c[i].i = i;
  }
  qsort(c, n, sizeof(orc_cand), cand_cmp);
  double lmax = (double)c[0].v;
  char* member = (char*)calloc(n, 1);
  for (int j = 0; j < k; ++j) member[c[j].i] = 1;
  double total = 0.0;
  for (int i = 0; i < n; ++i)
    if (member[i]) total += exp(((double)(float)logits[i] - lmax) / temperature);
  double target = u * total, run = 0.0, before = 0.0;
  int32_t pick = -1, last = -1;
  for (int i = 0; i < n; ++i) {
    if (!member[i]) continue;
    last = i;
    before = run;
    run += exp(((double)(float)logits[i] - lmax) / temperature);
    if (run > target) {
      pick = i;
      break;
    }
  }
  if (pick < 0) {
    pick = last;
    before = run;
  }
  if (margin) {
    double a = fabs(target - before), b = fabs(run - target);
    *margin = (a < b ? a : b) / total;
  }
  free(c);
  free(member);
  return pick;
}

/* ------------------------------------------------------------------ */
/* model                                                               */
/* ------------------------------------------------------------------ */

int32_t orc_n_tensors(const orc_config* c) {
  int S = c->n_substeps, L = c->n_layers, Ld = c->dep_layers;
  return 1 + S + 6 * L + 2 + S + S + 2 * Ld + 4 * S * Ld + S + (c->dep_final_norm ? 1 : 0);
}

/* Substeps the depformer runs per frame. */
static int dep_run(const orc_config* c) {
  return (c->dep_q > 0 && c->dep_q < c->n_substeps) ? c->dep_q : c->n_substeps;
}

void orc_model_free(orc_model* m) {
  if (!m) return;
  free(m->emb_audio);
  free(m->attn_norm); free(m->qkv); free(m->wo); free(m->mlp_norm); free(m->gate_up); free(m->down);
  free(m->dep_in); free(m->dep_emb); free(m->dep_attn_norm); free(m->dep_mlp_norm);
  free(m->dep_qkv); free(m->dep_o); free(m->dep_gate_up); free(m->dep_down); free(m->dep_head);
  free(m);
}

/* Binds the weight pointers (host arrays, list order of the weight layout
 * contract); the arrays must outlive the model. NULL on a bad config. */
orc_model* orc_model_new(const orc_config* c, const void* const* t, int32_t n) {
  if (!c || !t) return NULL;
  if (c->dim <= 0 || c->n_heads <= 0 || c->dim % c->n_heads || (c->dim / c->n_heads) % 2) return NULL;
  if (c->dep_dim <= 0 || c->dep_heads <= 0 || c->dep_dim % c->dep_heads) return NULL;
  if (c->window < 1 || (c->mask_oldest && c->window < 2)) return NULL;
  if (c->n_substeps < 1 || c->text_vocab < 2 || c->audio_card < 2) return NULL;
  if (c->dep_q < 0 || c->dep_q > c->n_substeps) return NULL;
  if (c->dep_ref_ring && dep_run(c) < 2) return NULL;
  if (n != orc_n_tensors(c)) return NULL;
  orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
  m->c = *c;
  int S = c->n_substeps, L = c->n_layers, Ld = c->dep_layers;
  int i = 0;
  m->emb_text = t[i++];
  m->emb_audio = (const void**)malloc(sizeof(void*) * S);
  for (int k = 0; k < S; ++k) m->emb_audio[k] = t[i++];
#define ARR(name, cnt) m->name = (const void**)malloc(sizeof(void*) * (cnt) + 1)
  ARR(attn_norm, L); ARR(qkv, L); ARR(wo, L); ARR(mlp_norm, L); ARR(gate_up, L); ARR(down, L);
  for (int l = 0; l < L; ++l) {
    m->attn_norm[l] = t[i++];
    m->qkv[l] = t[i++];
    m->wo[l] = t[i++];
    m->mlp_norm[l] = t[i++];
    m->gate_up[l] = t[i++];
    m->down[l] = t[i++];
  }
  m->out_norm = t[i++];
  m->text_head = t[i++];
  ARR(dep_in, S);
  for (int s = 0; s < S; ++s) m->dep_in[s] = t[i++];
  ARR(dep_emb, S);
  for (int s = 0; s < S; ++s) m->dep_emb[s] = t[i++];
  ARR(dep_attn_norm, Ld); ARR(dep_mlp_norm, Ld);
  for (int l = 0; l < Ld; ++l) {
    m->dep_attn_norm[l] = t[i++];
    m->dep_mlp_norm[l] = t[i++];
  }
  ARR(dep_qkv, S * Ld); ARR(dep_o, S * Ld); ARR(dep_gate_up, S * Ld); ARR(dep_down, S * Ld);
  for (int s = 0; s < S; ++s)
    for (int l = 0; l < Ld; ++l) {
      m->dep_qkv[s * Ld + l] = t[i++];
      m->dep_o[s * Ld + l] = t[i++];
      m->dep_gate_up[s * Ld + l] = t[i++];
      m->dep_down[s * Ld + l] = t[i++];
    }
  ARR(dep_head, S);
  for (int s = 0; s < S; ++s) m->dep_head[s] = t[i++];
  if (c->dep_final_norm) m->dep_out_norm = t[i++];
#undef ARR
  return m;
}

/* ------------------------------------------------------------------ */
/* session: ring KV cache (recipe "Architecture": 3000-frame sliding    */
/* window held in a ring KV cache with per-slot recycle)                */
/* ------------------------------------------------------------------ */

static size_t ring_elems(const orc_model* m) {
  return (size_t)m->c.n_layers * (size_t)m->c.window * (size_t)m->c.dim;
}

orc_session* orc_session_new(const orc_model* m) {
  if (!m) return NULL;
  orc_session* s = (orc_session*)calloc(1, sizeof(orc_session));
  s->m = m;
  size_t esz = m->c.bf16 ? sizeof(uint16_t) : sizeof(double);
  s->k_ring = calloc(ring_elems(m), esz);
  s->v_ring = calloc(ring_elems(m), esz);
  if (!s->k_ring || !s->v_ring) {
    free(s->k_ring); free(s->v_ring); free(s);
    return NULL;
  }
  return s;
}

void orc_session_free(orc_session* s) {
  if (!s) return;
  free(s->k_ring);
  free(s->v_ring);
  free(s);
}

static size_t ring_index(const orc_model* m, int l, int64_t slot, int i) {
  return ((size_t)l * m->c.window + (size_t)slot) * m->c.dim + (size_t)i;
}

static void ring_put(orc_session* s, void* ring, int l, int64_t slot, const double* vec) {
  const orc_model* m = s->m;
  for (int i = 0; i < m->c.dim; ++i) {
    size_t at = ring_index(m, l, slot, i);
    if (m->c.bf16) ((uint16_t*)ring)[at] = double_to_bf16_bits(vec[i]);
    else ((double*)ring)[at] = vec[i];
  }
}

static double ring_get(const orc_session* s, const void* ring, int l, int64_t slot, int i) {
  size_t at = ring_index(s->m, l, slot, i);
  return s->m->c.bf16 ? bf16_bits_to_double(((const uint16_t*)ring)[at]) : ((const double*)ring)[at];
}

/* Forgets the session's history: position 0, nothing attended. */
void orc_session_reset(orc_session* s) { s->pos = 0; }

/* Loads K and V for positions 0..n-1 (layout [L][n][D], model storage type)
 * and sets the position to n. Returns -1 if n is outside [0, W]. */
int orc_session_prefill(orc_session* s, int32_t n, const void* k, const void* v) {
  const orc_model* m = s->m;
  if (n < 0 || n > m->c.window) return -1;
  int D = m->c.dim;
  double* kv = (double*)malloc(sizeof(double) * D);
  double* vv = (double*)malloc(sizeof(double) * D);
  for (int l = 0; l < m->c.n_layers; ++l)
    for (int j = 0; j < n; ++j) {
      size_t base = ((size_t)l * n + j) * D;
      for (int i = 0; i < D; ++i) {
        kv[i] = wget(m, k, base + i);
        vv[i] = wget(m, v, base + i);
      }
      ring_put(s, s->k_ring, l, j % m->c.window, kv);
      ring_put(s, s->v_ring, l, j % m->c.window, vv);
    }
  free(kv);
  free(vv);
  s->pos = n;
  return 0;
}

/* Test-only state transfer (no model arithmetic): replaces the whole ring,
 * k, v [L][W][D] in the model storage type with row j = ring slot j, and sets
 * the position. Lets a test check one step at any position starting from
 * another implementation's cache. Returns -1 on a negative position. */
int orc_session_load_ring(orc_session* s, int64_t pos, const void* k, const void* v) {
  const orc_model* m = s->m;
  if (pos < 0) return -1;
  int D = m->c.dim, W = m->c.window;
  double* kv = (double*)malloc(sizeof(double) * D);
  double* vv = (double*)malloc(sizeof(double) * D);
  for (int l = 0; l < m->c.n_layers; ++l)
    for (int j = 0; j < W; ++j) {
      size_t base = ((size_t)l * W + j) * D;
      for (int i = 0; i < D; ++i) {
        kv[i] = wget(m, k, base + i);
        vv[i] = wget(m, v, base + i);
      }
      ring_put(s, s->k_ring, l, j, kv);
      ring_put(s, s->v_ring, l, j, vv);
    }
  free(kv);
  free(vv);
  s->pos = pos;
  return 0;
}

/* Test-only: copies the ring out (k, v [L][W][D], model storage type, row j =
 * ring slot j). */
void orc_session_read_ring(const orc_session* s, void* k, void* v) {
  const orc_model* m = s->m;
  int D = m->c.dim, W = m->c.window;
  for (int l = 0; l < m->c.n_layers; ++l)
    for (int j = 0; j < W; ++j)
      for (int i = 0; i < D; ++i) {
        size_t at = ((size_t)l * W + j) * D + i;
        double kv = ring_get(s, s->k_ring, l, j, i), vv = ring_get(s, s->v_ring, l, j, i);
        if (m->c.bf16) {
          ((uint16_t*)k)[at] = double_to_bf16_bits(kv);
          ((uint16_t*)v)[at] = double_to_bf16_bits(vv);
        } else {
          ((float*)k)[at] = (float)kv;
          ((float*)v)[at] = (float)vv;
        }
      }
}

/* Ring bookkeeping of the next step: its write index and how many keys it
 * will attend (window reading in the header). */
void orc_session_info(const orc_session* s, int64_t* pos, int32_t* fill, int32_t* write_idx) {
  int64_t W = s->m->c.window;
  if (pos) *pos = s->pos;
  if (fill) *fill = (int32_t)(s->pos < W ? s->pos : W);
  if (write_idx) *write_idx = (int32_t)(s->pos % W);
}

/* First position attended at position p (window reading in the header). */
static int64_t first_key(const orc_model* m, int64_t p) {
  int64_t W = m->c.window;
  int64_t first = p - W + 1;
  if (m->c.mask_oldest && p >= W - 1) first = p - W + 2;
  return first < 0 ? 0 : first;
}

/* ------------------------------------------------------------------ */
/* temporal step                                                       */
/* ------------------------------------------------------------------ */

static int check_frame(const orc_model* m, const int32_t* f) {
  if (f[0] < 0 || f[0] > m->c.text_vocab) return -1;
  for (int k = 1; k <= m->c.n_substeps; ++k)
    if (f[k] < 0 || f[k] > m->c.audio_card) return -1;
  return 0;
}

/* One temporal step of a session: embed the frame, run every layer at the
 * session's position (writing that position's K/V into the ring), the final
 * norm and the text head. hidden_out [D] (optional) receives the normed,
 * rounded hidden state; logits_out [Vt] (optional) the text logits. */
int orc_temporal(orc_session* s, const int32_t* frame, double* hidden_out, double* logits_out,
                 int32_t* token_out, double* margin_out) {
  const orc_model* m = s->m;
  const orc_config* c = &m->c;
  if (check_frame(m, frame)) return -1;
  int D = c->dim, H = c->n_heads, hd = D / H, F = c->ffn_hidden, W = c->window;
  int64_t p = s->pos;
  double* x = (double*)calloc(D, sizeof(double));
  double* h = (double*)malloc(sizeof(double) * D);
  double* qkv = (double*)malloc(sizeof(double) * 3 * D);
  double* o = (double*)malloc(sizeof(double) * D);
  double* y = (double*)malloc(sizeof(double) * D);
  double* gu = (double*)malloc(sizeof(double) * 2 * F);
  double* a = (double*)malloc(sizeof(double) * F);
  int nk_max = W;
  double* keys = (double*)malloc(sizeof(double) * (size_t)nk_max * hd);
  double* vals = (double*)malloc(sizeof(double) * (size_t)nk_max * hd);

  /* summed 17-channel embedding, channel order 0..16 */
  for (int i = 0; i < D; ++i) x[i] += wget(m, m->emb_text, (size_t)frame[0] * D + i);
  for (int k = 0; k < c->n_substeps; ++k)
    for (int i = 0; i < D; ++i) x[i] += wget(m, m->emb_audio[k], (size_t)frame[1 + k] * D + i);

  int64_t first = first_key(m, p);
  int nk = (int)(p - first + 1);
  for (int l = 0; l < c->n_layers; ++l) {
    /* attention block: pre-norm, q|k|v projection, RoPE, ring write, window attention */
    rmsnorm_w(m, x, m->attn_norm[l], D, h);
    for (int i = 0; i < D; ++i) h[i] = rnd(m, h[i]);
    linear(m, m->qkv[l], 3 * D, D, h, qkv);
    double *q = qkv, *k = qkv + D, *v = qkv + 2 * D;
    orc_rope(q, H, hd, p, c->rope_theta);
    orc_rope(k, H, hd, p, c->rope_theta);
    ring_put(s, s->k_ring, l, p % W, k);
    ring_put(s, s->v_ring, l, p % W, v);
    for (int hh = 0; hh < H; ++hh) {
      for (int j = 0; j < nk; ++j) {
        int64_t slot = (first + j) % W;
        for (int d = 0; d < hd; ++d) {
          keys[(size_t)j * hd + d] = ring_get(s, s->k_ring, l, slot, hh * hd + d);
          vals[(size_t)j * hd + d] = ring_get(s, s->v_ring, l, slot, hh * hd + d);
        }
      }
      orc_attend(q + hh * hd, keys, vals, nk, hd, hd, o + hh * hd);
    }
    for (int i = 0; i < D; ++i) o[i] = rnd(m, o[i]);
    linear(m, m->wo[l], D, D, o, y);
    for (int i = 0; i < D; ++i) x[i] += y[i];
    /* MLP block: pre-norm, fused gate|up, SiLU(gate) * up, down */
    rmsnorm_w(m, x, m->mlp_norm[l], D, h);
    for (int i = 0; i < D; ++i) h[i] = rnd(m, h[i]);
    linear(m, m->gate_up[l], 2 * F, D, h, gu);
    for (int i = 0; i < F; ++i) a[i] = rnd(m, orc_silu(gu[i]) * gu[F + i]);
    linear(m, m->down[l], D, F, a, y);
    for (int i = 0; i < D; ++i) x[i] += y[i];
  }
  rmsnorm_w(m, x, m->out_norm, D, h);
  for (int i = 0; i < D; ++i) h[i] = rnd(m, h[i]);
  double* logits = logits_out ? logits_out : (double*)malloc(sizeof(double) * c->text_vocab);
  linear(m, m->text_head, c->text_vocab, D, h, logits);
  double margin;
  int32_t tok = orc_argmax(logits, c->text_vocab, &margin);
  if (token_out) *token_out = tok;
  if (margin_out) *margin_out = margin;
  if (hidden_out) memcpy(hidden_out, h, sizeof(double) * D);
  if (!logits_out) free(logits);
  s->pos = p + 1;
  free(x); free(h); free(qkv); free(o); free(y); free(gu); free(a); free(keys); free(vals);
  return 0;
}

/* ------------------------------------------------------------------ */
/* depformer                                                           */
/* ------------------------------------------------------------------ */

/* The 16 autoregressive substeps of one frame from the temporal hidden state
 * `hid` [D] and the frame's text token. Substep s embeds the previous token
 * (the text token at s = 0, else code s-1) with its own table, adds its own
 * projection of `hid`, runs every depformer layer with substep s's linears
 * over the substep K/V entries 0..s (cleared at s = 0), and its own head picks
 * code s. forced (optional, [S]) replaces code s as the next substep's input
 * (teacher forcing) where it is >= 0; the returned codes are always the
 * oracle's own argmax. logits (optional) [S][Va]; margins (optional) [S].
 *
 * Variants (config flags; readings of the SGLang-Omni cookbook, "Known
 * limitations": only 8 depformer steps run there, and "Reference parity":
 * the last depformer step matches the reference only with its ring
 * behaviour emulated):
 *  - dep_q > 0: only substeps 0..dep_q-1 run (the agent's codebooks); codes
 *    of the others are -1, their margins +inf and logits 0;
 *  - dep_ref_ring: the substep K/V is a ring whose capacity is the number of
 *    substeps run; once it is full (the last substep) its oldest entry,
 *    entry 0, is masked, as the temporal ring masks its oldest key;
 *  - dep_final_norm: each head reads RMSNorm(y) * dep.out_norm (rounded)
 *    instead of the rounded residual y. */
int orc_depformer(const orc_model* m, const double* hid, int32_t text_in, const int32_t* forced,
                  double* logits, int32_t* codes, double* margins) {
  const orc_config* c = &m->c;
  int D = c->dim, Dd = c->dep_dim, Hd = c->dep_heads, hdd = Dd / Hd, Fd = c->dep_ffn_hidden;
  int S = c->n_substeps, Ld = c->dep_layers, Va = c->audio_card;
  if (text_in < 0 || text_in > c->text_vocab) return -1;
  if (forced)
    for (int s = 0; s < S; ++s)
      if (forced[s] < -1 || forced[s] > Va) return -1;
  double* y = (double*)malloc(sizeof(double) * Dd);
  double* h = (double*)malloc(sizeof(double) * Dd);
  double* qkv = (double*)malloc(sizeof(double) * 3 * Dd);
  double* o = (double*)malloc(sizeof(double) * Dd);
  double* t = (double*)malloc(sizeof(double) * (Dd > D ? Dd : D));
  double* gu = (double*)malloc(sizeof(double) * 2 * Fd);
  double* a = (double*)malloc(sizeof(double) * Fd);
  double* kc = (double*)calloc((size_t)Ld * S * Dd, sizeof(double)); /* [Ld][S][Dd] */
  double* vc = (double*)calloc((size_t)Ld * S * Dd, sizeof(double));
  double* lg = (double*)malloc(sizeof(double) * Va);
  double* hid_r = (double*)malloc(sizeof(double) * D);
  for (int i = 0; i < D; ++i) hid_r[i] = rnd(m, hid[i]);

  int S_run = dep_run(c);
  for (int s = S_run; s < S; ++s) {
    if (codes) codes[s] = -1;
    if (margins) margins[s] = INFINITY;
    if (logits) memset(logits + (size_t)s * Va, 0, sizeof(double) * Va);
  }
  int32_t prev = text_in;
  for (int s = 0; s < S_run; ++s) {
    linear(m, m->dep_in[s], Dd, D, hid_r, y);
    for (int i = 0; i < Dd; ++i) y[i] += wget(m, m->dep_emb[s], (size_t)prev * Dd + i);
    for (int l = 0; l < Ld; ++l) {
      int wi = s * Ld + l;
      rmsnorm_w(m, y, m->dep_attn_norm[l], Dd, h);
      for (int i = 0; i < Dd; ++i) h[i] = rnd(m, h[i]);
      linear(m, m->dep_qkv[wi], 3 * Dd, Dd, h, qkv);
      double* kr = kc + ((size_t)l * S + s) * Dd;
      double* vr = vc + ((size_t)l * S + s) * Dd;
      for (int i = 0; i < Dd; ++i) {
        kr[i] = rnd(m, qkv[Dd + i]);
        vr[i] = rnd(m, qkv[2 * Dd + i]);
      }
      /* entries first..s; the ring reading masks entry 0 at the last substep */
      int first = (c->dep_ref_ring && s == S_run - 1) ? 1 : 0;
      for (int hh = 0; hh < Hd; ++hh)
        orc_attend(qkv + hh * hdd, kc + ((size_t)l * S + first) * Dd + hh * hdd,
                   vc + ((size_t)l * S + first) * Dd + hh * hdd, s + 1 - first, hdd, Dd,
                   o + hh * hdd);
      for (int i = 0; i < Dd; ++i) o[i] = rnd(m, o[i]);
      linear(m, m->dep_o[wi], Dd, Dd, o, t);
      for (int i = 0; i < Dd; ++i) y[i] += t[i];
      rmsnorm_w(m, y, m->dep_mlp_norm[l], Dd, h);
      for (int i = 0; i < Dd; ++i) h[i] = rnd(m, h[i]);
      linear(m, m->dep_gate_up[wi], 2 * Fd, Dd, h, gu);
      for (int i = 0; i < Fd; ++i) a[i] = rnd(m, orc_silu(gu[i]) * gu[Fd + i]);
      linear(m, m->dep_down[wi], Dd, Fd, a, t);
      for (int i = 0; i < Dd; ++i) y[i] += t[i];
    }
    if (c->dep_final_norm) {
      rmsnorm_w(m, y, m->dep_out_norm, Dd, h);
      for (int i = 0; i < Dd; ++i) h[i] = rnd(m, h[i]);
    } else {
      for (int i = 0; i < Dd; ++i) h[i] = rnd(m, y[i]);
    }
    linear(m, m->dep_head[s], Va, Dd, h, lg);
    double mg;
    int32_t code = orc_argmax(lg, Va, &mg);
    if (codes) codes[s] = code;
    if (margins) margins[s] = mg;
    if (logits) memcpy(logits + (size_t)s * Va, lg, sizeof(double) * Va);
    prev = (forced && forced[s] >= 0) ? forced[s] : code;
  }
  free(y); free(h); free(qkv); free(o); free(t); free(gu); free(a); free(kc); free(vc); free(lg);
  free(hid_r);
  return 0;
}

/* One full frame step: temporal then depformer (one user frame in, one text
 * token and one set of codes out). forced_text < 0 means "use the oracle's own
 * text token"; forced_codes NULL means no forcing. */
int orc_step(orc_session* s, const int32_t* frame, int32_t forced_text, const int32_t* forced_codes,
             int32_t* text_token, int32_t* codes, double* text_logits, double* audio_logits,
             double* text_margin, double* audio_margins, double* hidden_out) {
  const orc_model* m = s->m;
  double* hid = (double*)malloc(sizeof(double) * m->c.dim);
  int32_t tok;
  int rc = orc_temporal(s, frame, hid, text_logits, &tok, text_margin);
  if (rc == 0) {
    if (text_token) *text_token = tok;
    if (hidden_out) memcpy(hidden_out, hid, sizeof(double) * m->c.dim);
    rc = orc_depformer(m, hid, forced_text >= 0 ? forced_text : tok, forced_codes, audio_logits,
                       codes, audio_margins);
  }
  free(hid);
  return rc;
}
