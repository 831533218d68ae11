/* CPU check of the test oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_sanitize.py): every entry
 * point on small fp32 and bf16 models -- prefill, ring wrap-around, ring
 * transfer, teacher forcing, the depformer variants -- must run clean and
 * return finite logits. The oracle's source is compiled into this file. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/moshi_oracle.c"

static int failures = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);  \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

/* A small linear congruential generator for test weights (values only need
 * to be finite and varied). */
static uint64_t lcg = 12345;
static double next_unit(void) {
  lcg = lcg * 6364136223846793005ULL + 1442695040888963407ULL;
  return (double)(lcg >> 11) * (1.0 / 9007199254740992.0) - 0.5;
}

static size_t tensor_elems(const orc_config* c, int idx, int* is_gain) {
  /* walk the weight list in order and return element count of tensor idx */
  int S = c->n_substeps, L = c->n_layers, Ld = c->dep_layers;
  size_t D = c->dim, F = c->ffn_hidden, Dd = c->dep_dim, Fd = c->dep_ffn_hidden;
  size_t Vt = c->text_vocab, Va = c->audio_card;
  int i = 0;
  *is_gain = 0;
  if (idx == i++) return (Vt + 1) * D;
  for (int k = 0; k < S; ++k)
    if (idx == i++) return (Va + 1) * D;
  for (int l = 0; l < L; ++l) {
    size_t sizes[6] = {D, 3 * D * D, D * D, D, 2 * F * D, D * F};
    for (int j = 0; j < 6; ++j)
      if (idx == i++) {
        *is_gain = (j == 0 || j == 3);
        return sizes[j];
      }
  }
  if (idx == i++) { *is_gain = 1; return D; }
  if (idx == i++) return Vt * D;
  for (int s = 0; s < S; ++s)
    if (idx == i++) return Dd * D;
  for (int s = 0; s < S; ++s)
    if (idx == i++) return ((s == 0 ? Vt : Va) + 1) * Dd;
  for (int l = 0; l < 2 * Ld; ++l)
    if (idx == i++) { *is_gain = 1; return Dd; }
  for (int s = 0; s < S * Ld; ++s) {
    size_t sizes[4] = {3 * Dd * Dd, Dd * Dd, 2 * Fd * Dd, Dd * Fd};
    for (int j = 0; j < 4; ++j)
      if (idx == i++) return sizes[j];
  }
  for (int s = 0; s < S; ++s)
    if (idx == i++) return Va * Dd;
  if (c->dep_final_norm && idx == i++) { *is_gain = 1; return Dd; }
  return 0;
}

static void run_model(orc_config cfg) {
  const int n = orc_n_tensors(&cfg);
  void** t = (void**)calloc((size_t)n, sizeof(void*));
  for (int i = 0; i < n; ++i) {
    int gain = 0;
    size_t ne = tensor_elems(&cfg, i, &gain);
    EXPECT(ne > 0);
    if (cfg.bf16) {
      uint16_t* a = (uint16_t*)malloc(ne * sizeof(uint16_t));
      for (size_t j = 0; j < ne; ++j) a[j] = double_to_bf16_bits(gain ? 1.0 + 0.2 * next_unit() : 0.5 * next_unit());
      t[i] = a;
    } else {
      float* a = (float*)malloc(ne * sizeof(float));
      for (size_t j = 0; j < ne; ++j) a[j] = (float)(gain ? 1.0 + 0.2 * next_unit() : 0.5 * next_unit());
      t[i] = a;
    }
  }
  orc_model* m = orc_model_new(&cfg, (const void* const*)t, n);
  EXPECT(m != NULL);
  if (!m) return;
  const int S = cfg.n_substeps, D = cfg.dim, L = cfg.n_layers, W = cfg.window;
  const size_t esz = cfg.bf16 ? 2 : 4;
  orc_session* a = orc_session_new(m);
  /* prefill W-1 positions of small values */
  const int npre = W - 1;
  void* pk = calloc((size_t)L * npre * D, esz);
  void* pv = calloc((size_t)L * npre * D, esz);
  EXPECT(orc_session_prefill(a, npre, pk, pv) == 0);
  EXPECT(orc_session_prefill(a, W + 1, pk, pv) == -1);
  int32_t frame[65], codes[64], forced[64], tok;
  double* tl = (double*)malloc(sizeof(double) * cfg.text_vocab);
  double* al = (double*)malloc(sizeof(double) * S * cfg.audio_card);
  double* hid = (double*)malloc(sizeof(double) * D);
  double tm, am[64];
  for (int step = 0; step < 2 * W + 3; ++step) {
    frame[0] = (int32_t)((step * 7) % (cfg.text_vocab + 1));
    for (int k = 1; k <= S; ++k) frame[k] = (int32_t)((step * 13 + k) % (cfg.audio_card + 1));
    for (int s = 0; s < S; ++s) forced[s] = (step % 3 == 0 && s % 2) ? s % cfg.audio_card : -1;
    EXPECT(orc_step(a, frame, step % 4 == 0 ? 3 : -1, step % 2 ? forced : NULL, &tok, codes, tl,
                    al, &tm, am, hid) == 0);
    for (int i = 0; i < cfg.text_vocab; ++i) EXPECT(isfinite(tl[i]));
    for (int i = 0; i < S * cfg.audio_card; ++i) EXPECT(isfinite(al[i]));
  }
  int64_t pos;
  int32_t fill, widx;
  orc_session_info(a, &pos, &fill, &widx);
  EXPECT(pos == npre + 2 * W + 3 && fill == W && widx == (int32_t)(pos % W));
  /* ring transfer */
  void* rk = malloc((size_t)L * W * D * esz);
  void* rv = malloc((size_t)L * W * D * esz);
  orc_session_read_ring(a, rk, rv);
  orc_session* b = orc_session_new(m);
  EXPECT(orc_session_load_ring(b, pos, rk, rv) == 0);
  EXPECT(orc_session_load_ring(b, -1, rk, rv) == -1);
  EXPECT(orc_temporal(b, frame, hid, tl, &tok, &tm) == 0);
  frame[3] = cfg.audio_card + 1;
  EXPECT(orc_temporal(b, frame, hid, tl, &tok, &tm) == -1); /* bad code */
  forced[0] = cfg.audio_card + 2;
  EXPECT(orc_depformer(m, hid, 0, forced, al, codes, am) == -1);
  EXPECT(orc_depformer(m, hid, cfg.text_vocab + 1, NULL, al, codes, am) == -1);
  orc_session_reset(b);
  orc_session_free(a);
  orc_session_free(b);
  free(rk); free(rv); free(pk); free(pv); free(tl); free(al); free(hid);
  orc_model_free(m);
  for (int i = 0; i < n; ++i) free(t[i]);
  free(t);
}

int main(void) {
  orc_config c;
  memset(&c, 0, sizeof(c));
  c.dim = 32; c.n_layers = 2; c.n_heads = 2; c.ffn_hidden = 40; c.window = 5;
  c.dep_dim = 16; c.dep_layers = 2; c.dep_heads = 2; c.dep_ffn_hidden = 24; c.n_substeps = 6;
  c.text_vocab = 11; c.audio_card = 9; c.rope_theta = 1e4; c.norm_eps = 1e-8;
  run_model(c);                        /* fp32, wrap-around */
  c.bf16 = 1;
  c.mask_oldest = 1;
  run_model(c);                        /* bf16, masked oldest key */
  c.dep_q = 4;
  c.dep_ref_ring = 1;
  c.dep_final_norm = 1;
  run_model(c);                        /* depformer variants */
  c.window = 1;
  c.mask_oldest = 0;
  c.dep_q = 0;
  run_model(c);                        /* window of one key */
  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("oracle checks ok\n");
  return 0;
}
