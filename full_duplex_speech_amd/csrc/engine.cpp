// engine.cpp -- host side of libmoshi.so: the C ABI of include/moshi.h, the
// session slot table, device buffers, and the two captured HIP graphs (the
// temporal step and the 16 depformer substeps) that run a frame.
//
// One user frame in, one text token and one set of codes out per live slot
// per call ("vLLM-Omni recipe: PersonaPlex", "Why it is different"); sessions
// join and leave between calls, a full engine refuses joins, and a recycled
// slot starts exactly like a fresh one ("Notes"). Per-slot state that changes
// between calls (liveness, position, the frame) lives in device buffers the
// graphs read, so joins and leaves never re-capture a graph.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <utility>
#include <vector>

#include "../../include/moshi.h"
#include "engine_internal.h"
#include "host.h"
#include "kernels.h"

using namespace moshi;
using moshi_host::SlotTable;

namespace {

// Kernel classes reported by moshi_time_kernels.
enum KClass {
  KC_EMBED = 0,
  KC_T_QKV,
  KC_T_ATTN,
  KC_T_O,
  KC_T_GATEUP,
  KC_T_DOWN,
  KC_T_HEAD,
  KC_D_INPROJ,
  KC_D_ENTRY,
  KC_D_QKV,
  KC_D_ATTN,
  KC_D_O,
  KC_D_GATEUP,
  KC_D_DOWN,
  KC_D_HEAD,
  KC_T_COMBINE,
  KC_ARGMAX,
  KC_SAMPLE,
  KC_COUNT
};
const char* kClassNames[KC_COUNT] = {
    "embed",      "temporal_qkv",  "temporal_attn", "temporal_o",    "temporal_gateup",
    "temporal_down", "text_head",  "dep_inproj",    "dep_entry",     "dep_qkv",
    "dep_attn",   "dep_o",         "dep_gateup",    "dep_down",      "dep_head",
    "temporal_attn_combine", "argmax_reduce", "sample"};

int32_t tensor_count(const moshi_config* c) { return moshi_host::tensor_count(c); }
const char* config_error(const moshi_config* c) { return moshi_host::config_error(c); }

}  // namespace

// Workspace of the multi-frame prefill (up to 64 frames per chunk).
struct PrefillWs {
  bool ready = false;
  int rows = 0, spans = 1;
  double *x = nullptr, *ssq = nullptr, *q = nullptr, *part = nullptr;
  void *hn = nullptr, *o = nullptr, *act = nullptr, *hid = nullptr, *wk = nullptr, *wv = nullptr;
  float* logits = nullptr;
  moshi::ArgPart* apart = nullptr;
  int *tok = nullptr, *live = nullptr, *frames = nullptr, *key0 = nullptr, *nkeys = nullptr;
  int64_t* pos = nullptr;
};

struct moshi_ctx {
  moshi_config c{};
  int B = 0, dtype = 0, esz = 0, device = 0;
  int D = 0, H = 0, hd = 0, F = 0, W = 0, L = 0;
  int Dd = 0, Hd = 0, hdd = 0, Fd = 0, Ld = 0, S = 0, Vt = 0, Va = 0, NCH = 0;
  int S_run = 0;  // depformer substeps run per frame
  hipStream_t stream = nullptr;
  bool own_stream = false;
  bool failed = false;
  std::string err;

  // weights (device)
  std::vector<void*> dev_alloc;  // every hipMalloc, freed at destroy
  const void* emb_text = nullptr;
  std::vector<const void*> emb_audio, attn_norm, qkv, wo, mlp_norm, gate_up, down;
  const void* out_norm = nullptr;
  const void* text_head = nullptr;
  const void* dep_in = nullptr;  // [S*Dd][D], contiguous
  std::vector<const void*> dep_emb, dep_attn_norm, dep_mlp_norm, dep_qkv, dep_o, dep_gate_up,
      dep_down, dep_head;
  const void* dep_out_norm = nullptr;  // MOSHI_FLAG_DEP_FINAL_NORM only

  // state and activations (device)
  void *ring_k = nullptr, *ring_v = nullptr;  // [B][L][H][W][hd]
  void *dkv_k = nullptr, *dkv_v = nullptr;    // [B][Ld][Hd][S][hdd]
  double *x = nullptr, *ssq = nullptr, *q = nullptr;     // fp64 arithmetic state
  void *o = nullptr, *act = nullptr, *hid = nullptr;      // model dtype
  double *pre = nullptr, *y = nullptr, *ssq_d = nullptr, *qd = nullptr;
  void *od = nullptr, *actd = nullptr;
  void *hn = nullptr, *hnd = nullptr;  // rounded norm outputs (two or more sessions)
  float *text_logits = nullptr, *audio_logits = nullptr;
  int *tokens = nullptr, *codes = nullptr;
  ArgPart* apart = nullptr;  // per-tile argmax partials of the last head
  double* attn_part = nullptr;
  double* kpart = nullptr;  // K-segment sums of split projections (GemmArgs::kpart)
  int* kcnt = nullptr;      // their counters
  int *d_frames = nullptr, *d_live = nullptr;
  int64_t* d_pos = nullptr;
  int* d_err = nullptr;  // set by the embedding when a live code was out of range
  int* d_forced = nullptr;  // [B][1+S] forced text / codes, -1 = not forced
  SampleParams* d_samp = nullptr;  // [B] sampling parameters (MOSHI_FLAG_SAMPLING)
  bool sampling = false;
  double *d_inv_freq = nullptr;
  void* staging = nullptr;  // one layer of prefill K or V
  int max_spans = 0;  // temporal attention spans per (slot, head)
  int ncu = 1;        // compute units of the device

  // host state: the slot table (the device copies of live / pos are
  // refreshed only when it is dirty; the step itself advances the device
  // positions)
  SlotTable slots;
  int* h_frames = nullptr;  // pinned
  int* h_live = nullptr;
  int64_t* h_pos = nullptr;
  int* h_forced = nullptr;
  bool forced_on_device = false;  // d_forced holds a forced step's values
  std::vector<SampleParams> samp;  // per slot
  bool samp_dirty = false;
  SampleParams* h_samp = nullptr;  // pinned staging
  // recorded after the last copy out of h_live / h_pos / h_forced: those
  // pinned buffers are rewritten only once it has completed, so a step
  // enqueued earlier still reads its own metadata
  hipEvent_t meta_ev = nullptr;
  bool meta_ev_pending = false;
  int* h_tokens = nullptr;
  int* h_codes = nullptr;

  // graphs
  hipGraphExec_t g_temporal = nullptr, g_dep = nullptr;
  bool use_graphs = true;

  // persistent one-session step kernel (capacity 1 and an instantiated shape)
  bool persistent = false;
  StepArgs* d_step = nullptr;
  unsigned* d_bar = nullptr;
  int* d_abort = nullptr;
  int step_grid = 0;
  size_t step_lds = 0;
  int step_parity = 0;
  uint32_t step_seq = 0;  // sequence number of the last step kernel launch
  StepArgs step_host{};   // host copy of *d_step
  PrefillWs pf;
  // the same step with its synchronisation scratch in the static scratch of
  // static_step.hip (moshi_step_enqueue_noalloc); null when it does not fit
  StepArgs* d_step_static = nullptr;
  std::string static_why;  // why there is no static variant

  // persistent multi-session depformer kernel (capacity 2..64, an
  // instantiated shape, no sampling); it shares d_abort's role
  bool dep_multi = false;
  DepMultiArgs* d_dm = nullptr;
  DepMultiArgs dm_host{};
  int dm_grid = 0;
  size_t dm_lds = 0;
  int dm_parity = 0;

  // kernel timing (eager launches bracketed by events); `dry` only records
  // the (class, bytes) sequence of a step without launching anything
  bool timing = false;
  bool dry = false;
  std::vector<hipEvent_t> ev;
  std::vector<int> ev_class;
  std::vector<double> ev_bytes;
  size_t ev_used = 0;
};

namespace {

int fail(moshi_ctx* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  return code;
}

int device_fail(moshi_ctx* c, hipError_t e, const char* where) {
  if (c) {
    c->failed = true;
    c->err = std::string(where) + ": " + hipGetErrorString(e);
  }
  return MOSHI_E_DEVICE;
}

#define CKD(ctx, expr)                                        \
  do {                                                        \
    hipError_t e_ = (expr);                                   \
    if (e_ != hipSuccess) return device_fail(ctx, e_, #expr); \
  } while (0)

hipError_t dalloc(moshi_ctx* c, void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) bytes = 256;
  hipError_t e = hipMalloc(p, bytes);
  if (e == hipSuccess) c->dev_alloc.push_back(*p);
  return e;
}

// ---- launch helpers (each kernel launch goes through `run`) ----

template <typename F>
hipError_t run(moshi_ctx* c, int kclass, double bytes, F&& launch) {
  if (c->dry) {
    c->ev_class.push_back(kclass);
    c->ev_bytes.push_back(bytes);
    return hipSuccess;
  }
  if (!c->timing) return launch();
  if (c->ev_used + 2 > c->ev.size()) {
    for (int i = 0; i < 64; ++i) {
      hipEvent_t e;
      hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) return r;
      c->ev.push_back(e);
    }
  }
  hipError_t r = hipEventRecord(c->ev[c->ev_used], c->stream);
  if (r != hipSuccess) return r;
  r = launch();
  if (r != hipSuccess) return r;
  r = hipEventRecord(c->ev[c->ev_used + 1], c->stream);
  if (r != hipSuccess) return r;
  c->ev_class.push_back(kclass);
  c->ev_bytes.push_back(bytes);
  c->ev_used += 2;
  return hipSuccess;
}

int live_count(const moshi_ctx* c) { return c->slots.live_count(); }

GemmArgs gemm_base(const moshi_ctx* c) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.B = c->B;
  a.eps = c->c.norm_eps;
  a.live = c->d_live;
  return a;
}

hipError_t gemm(moshi_ctx* c, int pro, int epi, const GemmArgs& a) {
  return launch_gemm(c->dtype, gemm_kw(c->dtype, a.B, a.K, gemm_tiles(epi, a.N)), pro, epi, a,
                     c->stream);
}

// ---- argument blocks of every operation (shared by the per-operation
// kernels and the persistent step kernel) ----

// Rows per sum-of-squares partial of a residual stream, and their count.
int ssq_rows(const moshi_ctx* c) { return c->B == 1 ? GEMV_SSQ_ROWS : 16; }
int n_ssq(const moshi_ctx* c, int n) { return (n + ssq_rows(c) - 1) / ssq_rows(c); }

EmbedArgs embed_args(const moshi_ctx* c) {
  EmbedArgs a;
  memset(&a, 0, sizeof(a));
  a.tables[0] = c->emb_text;
  for (int k = 0; k < c->S; ++k) a.tables[1 + k] = c->emb_audio[k];
  a.frames = c->d_frames; a.live = c->d_live; a.n_ch = c->NCH; a.D = c->D; a.B = c->B;
  a.rows_text = c->Vt + 1; a.rows_audio = c->Va + 1; a.bad_code = c->d_err;
  a.x = c->x; a.ssq_out = c->ssq; a.ssq_rows = ssq_rows(c);
  return a;
}

int64_t t_slot_stride(const moshi_ctx* c) { return (int64_t)c->L * c->H * c->W * c->hd; }
int64_t t_layer_elems(const moshi_ctx* c) { return (int64_t)c->H * c->W * c->hd; }
int64_t d_slot_stride(const moshi_ctx* c) { return (int64_t)c->Ld * c->Hd * c->S * c->hdd; }
int64_t d_layer_elems(const moshi_ctx* c) { return (int64_t)c->Hd * c->S * c->hdd; }

// RMSNorm -> q|k|v -> RoPE -> ring write
GemmArgs t_qkv_args(const moshi_ctx* c, int l) {
  GemmArgs a = gemm_base(c);
  a.vec_cols = 1;  // two to four sessions: VALU tiles
  a.W = c->qkv[l]; a.N = 3 * c->D; a.K = c->D;
  a.X = c->x; a.ldx = c->D; a.ssq = c->ssq; a.n_ssq = n_ssq(c, c->D); a.gain = c->attn_norm[l];
  a.xn_out = c->B > 1 ? c->hn : nullptr;
  a.q_out = c->q; a.dq = c->D; a.hd = c->hd; a.inv_freq = c->d_inv_freq; a.pos = c->d_pos;
  a.ring_k = c->ring_k; a.ring_v = c->ring_v; a.slot_stride = t_slot_stride(c);
  a.layer_off = (int64_t)l * t_layer_elems(c); a.head_stride = (int64_t)c->W * c->hd;
  a.cap = c->W;
  return a;
}

// window attention over the ring
AttnArgs t_attn_args(const moshi_ctx* c, int l) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = c->q; a.ldq = c->D; a.ring_k = c->ring_k; a.ring_v = c->ring_v;
  a.slot_stride = t_slot_stride(c); a.layer_off = (int64_t)l * t_layer_elems(c);
  a.head_stride = (int64_t)c->W * c->hd; a.cap = c->W; a.pos = c->d_pos; a.live = c->d_live;
  a.mask_oldest = (c->c.flags & MOSHI_FLAG_MASK_OLDEST) ? 1 : 0;
  a.n_heads = c->H; a.max_spans = c->max_spans; a.part = c->attn_part;
  a.o_out = c->o; a.ldo = c->D;
  return a;
}

// o-projection + residual
GemmArgs t_o_args(const moshi_ctx* c, int l) {
  GemmArgs a = gemm_base(c);
  a.vec_cols = 1;  // two to four sessions: VALU tiles
  a.W = c->wo[l]; a.N = c->D; a.K = c->D; a.X = c->o; a.ldx = c->D;
  a.resid = c->x; a.ldr = c->D; a.ssq_out = c->ssq;
  return a;
}

// RMSNorm -> gate|up -> SiLU(gate)*up
GemmArgs t_gu_args(const moshi_ctx* c, int l) {
  GemmArgs a = gemm_base(c);
  a.vec_cols = 1;  // two to four sessions: VALU tiles
  a.W = c->gate_up[l]; a.N = c->F; a.K = c->D;
  a.X = c->x; a.ldx = c->D; a.ssq = c->ssq; a.n_ssq = n_ssq(c, c->D); a.gain = c->mlp_norm[l];
  a.xn_out = c->B > 1 ? c->hn : nullptr;
  a.act = c->act; a.lda = c->F;
  return a;
}

// down + residual
GemmArgs t_dn_args(const moshi_ctx* c, int l) {
  GemmArgs a = gemm_base(c);
  a.vec_cols = 1;  // two to four sessions: VALU tiles
  a.W = c->down[l]; a.N = c->D; a.K = c->F; a.X = c->act; a.ldx = c->F;
  a.resid = c->x; a.ldr = c->D; a.ssq_out = c->ssq;
  return a;
}

// final norm -> hidden (kept for the depformer) -> text head logits + argmax partials
GemmArgs t_head_args(const moshi_ctx* c) {
  GemmArgs a = gemm_base(c);
  a.vec_cols = 1;  // two to four sessions: VALU tiles
  a.W = c->text_head; a.N = c->Vt; a.K = c->D;
  a.X = c->x; a.ldx = c->D; a.ssq = c->ssq; a.n_ssq = n_ssq(c, c->D); a.gain = c->out_norm;
  a.xn_out = c->hid;
  a.logits = c->text_logits; a.ldo = c->Vt; a.apart = c->apart;
  return a;
}

// y_pre[s] = W_in[s] . hidden for every substep run, at once (the input
// projections of all substeps are one [S * Dd, D] matrix)
GemmArgs d_in_args(const moshi_ctx* c) {
  GemmArgs a = gemm_base(c);
  a.W = c->dep_in; a.N = c->S_run * c->Dd; a.K = c->D; a.X = c->hid; a.ldx = c->D;
  a.out64 = c->pre; a.ldo = c->S * c->Dd;
  return a;
}

GemmArgs d_qkv_args(const moshi_ctx* c, int s, int l) {
  GemmArgs a = gemm_base(c);
  a.W = c->dep_qkv[s * c->Ld + l]; a.N = 3 * c->Dd; a.K = c->Dd;
  a.X = c->y; a.ldx = c->Dd; a.ssq = c->ssq_d; a.n_ssq = n_ssq(c, c->Dd);
  a.gain = c->dep_attn_norm[l];
  a.xn_out = c->B > 1 ? c->hnd : nullptr;
  a.q_out = c->qd; a.dq = c->Dd; a.hd = c->hdd; a.inv_freq = nullptr; a.pos = nullptr;
  a.scalar_widx = s; a.ring_k = c->dkv_k; a.ring_v = c->dkv_v; a.slot_stride = d_slot_stride(c);
  a.layer_off = (int64_t)l * d_layer_elems(c); a.head_stride = (int64_t)c->S * c->hdd; a.cap = c->S;
  return a;
}

AttnArgs d_attn_args(const moshi_ctx* c, int s, int l) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = c->qd; a.ldq = c->Dd; a.ring_k = c->dkv_k; a.ring_v = c->dkv_v;
  a.slot_stride = d_slot_stride(c); a.layer_off = (int64_t)l * d_layer_elems(c);
  a.head_stride = (int64_t)c->S * c->hdd;
  a.cap = c->S; a.pos = nullptr; a.scalar_nvalid = s + 1; a.live = c->d_live;
  // the depformer ring reading masks entry 0 at the last substep run
  a.scalar_excl = ((c->c.flags & MOSHI_FLAG_DEP_REF_RING) && s == c->S_run - 1) ? 0 : -1;
  a.n_heads = c->Hd; a.max_spans = 1; a.part = c->attn_part;  // S <= 64: one span
  a.o_out = c->od; a.ldo = c->Dd;
  return a;
}

GemmArgs d_o_args(const moshi_ctx* c, int s, int l) {
  GemmArgs a = gemm_base(c);
  a.W = c->dep_o[s * c->Ld + l]; a.N = c->Dd; a.K = c->Dd; a.X = c->od; a.ldx = c->Dd;
  a.resid = c->y; a.ldr = c->Dd; a.ssq_out = c->ssq_d;
  return a;
}

GemmArgs d_gu_args(const moshi_ctx* c, int s, int l) {
  GemmArgs a = gemm_base(c);
  a.W = c->dep_gate_up[s * c->Ld + l]; a.N = c->Fd; a.K = c->Dd;
  a.X = c->y; a.ldx = c->Dd; a.ssq = c->ssq_d; a.n_ssq = n_ssq(c, c->Dd);
  a.gain = c->dep_mlp_norm[l];
  a.xn_out = c->B > 1 ? c->hnd : nullptr;
  a.act = c->actd; a.lda = c->Fd;
  return a;
}

GemmArgs d_dn_args(const moshi_ctx* c, int s, int l) {
  GemmArgs a = gemm_base(c);
  a.W = c->dep_down[s * c->Ld + l]; a.N = c->Dd; a.K = c->Fd; a.X = c->actd; a.ldx = c->Fd;
  a.resid = c->y; a.ldr = c->Dd; a.ssq_out = c->ssq_d;
  a.ksplit = gemm_ksplit(c->B, a.K, gemm_tiles(EPI_RESID, a.N));
  a.kpart = c->kpart; a.kcnt = c->kcnt;
  return a;
}

// head s on the rounded residual (or, with the final-norm reading, on its
// RMSNorm) -> logits + argmax partials
bool dep_final_norm(const moshi_ctx* c) { return (c->c.flags & MOSHI_FLAG_DEP_FINAL_NORM) != 0; }
GemmArgs d_head_args(const moshi_ctx* c, int s) {
  GemmArgs a = gemm_base(c);
  a.W = c->dep_head[s]; a.N = c->Va; a.K = c->Dd; a.X = c->y; a.ldx = c->Dd;
  if (dep_final_norm(c)) {
    a.ssq = c->ssq_d; a.n_ssq = n_ssq(c, c->Dd); a.gain = c->dep_out_norm;
  }
  a.xn_out = c->B > 1 ? c->hnd : nullptr;
  a.logits = c->audio_logits + (size_t)s * c->Va; a.ldo = c->S * c->Va;
  a.apart = c->apart;
  return a;
}

// Draws of head `stream` (0 text, 1 + s substep s) for the sessions that
// sample; the others keep the argmax (or forced token) already in `out`.
SampleArgs sample_args(const moshi_ctx* c, const float* logits, int ld, int n, int which, int stream,
                       int pos_off, int* out, int out_stride, int forced_col) {
  SampleArgs a;
  memset(&a, 0, sizeof(a));
  a.logits = logits; a.ld = ld; a.n = n; a.params = c->d_samp; a.which = which;
  a.stream = stream; a.pos = c->d_pos; a.pos_off = pos_off; a.live = c->d_live;
  a.forced = c->d_forced; a.forced_stride = c->NCH; a.forced_col = forced_col;
  a.out = out; a.out_stride = out_stride; a.B = c->B;
  return a;
}

// ---- the temporal step: embed, L layers, final norm + text head ----

hipError_t enqueue_temporal(moshi_ctx* c) {
  const int dt = c->dtype, B = c->B, D = c->D, F = c->F, es = c->esz;
  const double nlive = live_count(c);
  hipError_t e;
  {
    EmbedArgs a = embed_args(c);
    e = run(c, KC_EMBED, nlive * c->NCH * D * es, [&] { return launch_embed(dt, a, c->stream); });
    if (e != hipSuccess) return e;
  }
  for (int l = 0; l < c->L; ++l) {
    {
      GemmArgs a = t_qkv_args(c, l);
      double bytes = 3.0 * D * D * es + D * es + nlive * 2.0 * D * es;
      e = run(c, KC_T_QKV, bytes, [&] { return gemm(c, PRO_NORM, EPI_QKV, a); });
      if (e != hipSuccess) return e;
    }
    {
      AttnArgs a = t_attn_args(c, l);
      double keys = 0;
      for (int b = 0; b < B; ++b)
        if (c->slots.live[b]) {
          int64_t p = c->slots.pos[b];
          int64_t n = p + 1 < c->W ? p + 1 : c->W;
          if (a.mask_oldest && p >= c->W - 1) n -= 1;
          keys += (double)n;
        }
      e = run(c, KC_T_ATTN, keys * 2.0 * D * es,
              [&] { return launch_attn(dt, c->hd, a, B, c->stream); });
      if (e != hipSuccess) return e;
      if (c->max_spans > 1) {
        e = run(c, KC_T_COMBINE, 0.0, [&] { return launch_attn_combine(dt, c->hd, a, B, c->stream); });
        if (e != hipSuccess) return e;
      }
    }
    {
      GemmArgs a = t_o_args(c, l);
      e = run(c, KC_T_O, (double)D * D * es, [&] { return gemm(c, PRO_DIRECT, EPI_RESID, a); });
      if (e != hipSuccess) return e;
    }
    {
      GemmArgs a = t_gu_args(c, l);
      e = run(c, KC_T_GATEUP, 2.0 * F * D * es + D * es,
              [&] { return gemm(c, PRO_NORM, EPI_SWIGLU, a); });
      if (e != hipSuccess) return e;
    }
    {
      GemmArgs a = t_dn_args(c, l);
      e = run(c, KC_T_DOWN, (double)D * F * es, [&] { return gemm(c, PRO_DIRECT, EPI_RESID, a); });
      if (e != hipSuccess) return e;
    }
  }
  {
    GemmArgs a = t_head_args(c);
    e = run(c, KC_T_HEAD, (double)c->Vt * D * es + D * es,
            [&] { return gemm(c, PRO_NORM, EPI_ARGMAX, a); });
    if (e != hipSuccess) return e;
    e = run(c, KC_ARGMAX, 0.0, [&] {
      return launch_argmax_reduce(c->apart, (c->Vt + 15) / 16, c->Vt, B, c->tokens, 1, c->d_forced,
                                  c->NCH, 0, c->stream);
    });
    if (e != hipSuccess) return e;
    if (c->sampling) {  // sessions that sample replace the argmax by a draw
      const SampleArgs sa = sample_args(c, c->text_logits, c->Vt, c->Vt, 0, 0, 0, c->tokens, 1, 0);
      e = run(c, KC_SAMPLE, 0.0, [&] { return launch_sample(sa, c->stream); });
      if (e != hipSuccess) return e;
    }
  }
  return c->dry ? hipSuccess : launch_advance(c->d_pos, c->d_live, B, c->stream);
}

// ---- the depformer: all substep input projections, then 16 substeps ----

hipError_t enqueue_depformer(moshi_ctx* c) {
  const int dt = c->dtype, B = c->B, D = c->D, Dd = c->Dd, Fd = c->Fd, S = c->S, es = c->esz;
  const double nlive = live_count(c);
  hipError_t e;
  {
    // the depformer's wave split (8 / 4) also for its 4096-wide input
    // projections: the multi-session depformer kernel computes the same bits
    GemmArgs a = d_in_args(c);
    const int kw = B == 1 ? GEMV_KW : (B <= 32 ? 8 : 4);
    e = run(c, KC_D_INPROJ, (double)c->S_run * Dd * D * es,
            [&] { return launch_gemm(dt, kw, PRO_DIRECT, EPI_STORE, a, c->stream); });
    if (e != hipSuccess) return e;
  }
  for (int s = 0; s < c->S_run; ++s) {
    {  // entry: y = pre[s] + E_s[previous token]; for s >= 1 the previous
       // head's partials are reduced here (or the forced code taken) and
       // code s-1 is stored
      EntryArgs a;
      memset(&a, 0, sizeof(a));
      a.pre = c->pre; a.ldpre = S * Dd; a.s = s; a.table = c->dep_emb[s];
      a.prev = s == 0 ? c->tokens : c->codes + (s - 1); a.prev_stride = s == 0 ? 1 : S;
      // with sampling every code is settled (argmax, draw or forced) right
      // after its head; otherwise the entry reduces the previous head's
      // partials itself
      a.prev_part = (s == 0 || c->sampling) ? nullptr : c->apart; a.prev_tiles = (c->Va + 15) / 16;
      a.prev_n = c->Va; a.D = Dd; a.B = B; a.y = c->y; a.ssq_out = c->ssq_d;
      if (s > 0 && !c->sampling) {
        a.forced = c->d_forced; a.forced_stride = c->NCH; a.forced_col = s;
      }
      a.ssq_rows = ssq_rows(c);
      e = run(c, KC_D_ENTRY, nlive * Dd * es, [&] { return launch_entry(dt, a, c->stream); });
      if (e != hipSuccess) return e;
    }
    for (int l = 0; l < c->Ld; ++l) {
      {
        GemmArgs a = d_qkv_args(c, s, l);
        e = run(c, KC_D_QKV, 3.0 * Dd * Dd * es + Dd * es + nlive * 2.0 * Dd * es,
                [&] { return gemm(c, PRO_NORM, EPI_QKV, a); });
        if (e != hipSuccess) return e;
      }
      {
        AttnArgs a = d_attn_args(c, s, l);
        e = run(c, KC_D_ATTN, nlive * (s + 1) * 2.0 * Dd * es, [&] {
          return S <= DEP_MAX_KEYS_HOST ? launch_dep_attn(dt, c->hdd, a, B, c->stream)
                                        : launch_attn(dt, c->hdd, a, B, c->stream);
        });
        if (e != hipSuccess) return e;
      }
      {
        GemmArgs a = d_o_args(c, s, l);
        e = run(c, KC_D_O, (double)Dd * Dd * es, [&] { return gemm(c, PRO_DIRECT, EPI_RESID, a); });
        if (e != hipSuccess) return e;
      }
      {
        GemmArgs a = d_gu_args(c, s, l);
        e = run(c, KC_D_GATEUP, 2.0 * Fd * Dd * es + Dd * es,
                [&] { return gemm(c, PRO_NORM, EPI_SWIGLU, a); });
        if (e != hipSuccess) return e;
      }
      {
        GemmArgs a = d_dn_args(c, s, l);
        e = run(c, KC_D_DOWN, (double)Dd * Fd * es, [&] { return gemm(c, PRO_DIRECT, EPI_RESID, a); });
        if (e != hipSuccess) return e;
      }
    }
    {
      GemmArgs a = d_head_args(c, s);
      const int pro = dep_final_norm(c) ? PRO_NORM : PRO_CAST;
      e = run(c, KC_D_HEAD, (double)c->Va * Dd * es + (dep_final_norm(c) ? Dd * es : 0.0),
              [&] { return gemm(c, pro, EPI_ARGMAX, a); });
      if (e != hipSuccess) return e;
    }
    if (c->sampling && s + 1 < c->S_run) {
      // code s now: argmax or forced, then the draws (the last code below)
      e = run(c, KC_ARGMAX, 0.0, [&] {
        return launch_argmax_reduce(c->apart, (c->Va + 15) / 16, c->Va, B, c->codes + s, S,
                                    c->d_forced, c->NCH, s + 1, c->stream);
      });
      if (e != hipSuccess) return e;
      // the temporal step advanced the positions: this frame's is pos - 1
      const SampleArgs sa = sample_args(c, c->audio_logits + (size_t)s * c->Va, S * c->Va, c->Va, 1,
                                        1 + s, -1, c->codes + s, S, s + 1);
      e = run(c, KC_SAMPLE, 0.0, [&] { return launch_sample(sa, c->stream); });
      if (e != hipSuccess) return e;
    }
  }
  // the last substep's code (earlier ones are stored by the next entry)
  const int sl = c->S_run - 1;
  e = run(c, KC_ARGMAX, 0.0, [&] {
    return launch_argmax_reduce(c->apart, (c->Va + 15) / 16, c->Va, B, c->codes + sl, S,
                                c->d_forced, c->NCH, sl + 1, c->stream);
  });
  if (e != hipSuccess) return e;
  if (c->sampling) {
    const SampleArgs sa = sample_args(c, c->audio_logits + (size_t)sl * c->Va, S * c->Va, c->Va, 1,
                                      1 + sl, -1, c->codes + sl, S, sl + 1);
    e = run(c, KC_SAMPLE, 0.0, [&] { return launch_sample(sa, c->stream); });
    if (e != hipSuccess) return e;
  }
  // free slots and substeps not run read -1
  return run(c, KC_ARGMAX, 0.0, [&] {
    return launch_finish_outputs(c->tokens, c->codes, c->d_live, B, S, c->S_run, c->stream);
  });
}

// ---- multi-frame prefill of one session (moshi_session_prefill_frames) ----

constexpr int PF_COLS = 64;  // frames per chunk: the MFMA kernels' widest column tile set

// The chunk workspace, allocated at the first prefill.
int ensure_prefill(moshi_ctx* c) {
  if (c->pf.ready) return MOSHI_OK;
  PrefillWs& p = c->pf;
  const size_t NC = PF_COLS, D = c->D, F = c->F, es = c->esz;
  const size_t rows = (size_t)c->W - 1 + NC;  // window rows: W - 1 earlier positions + the chunk
  p.spans = (c->W + ATTN_CHUNK - 1) / ATTN_CHUNK;
  if (p.spans > 4) p.spans = 4;
  const size_t nssq = (D + 1) / 2 > ((D + 15) / 16) * NC ? (D + 1) / 2 : ((D + 15) / 16) * NC;
  struct Req {
    void** ptr;
    size_t bytes;
  } reqs[] = {
      {(void**)&p.x, NC * D * 8},
      {(void**)&p.ssq, nssq * 8},
      {(void**)&p.q, NC * D * 8},
      {&p.hn, NC * D * es},
      {&p.o, NC * D * es},
      {&p.act, NC * F * es},
      {&p.hid, NC * D * es},
      {(void**)&p.logits, NC * c->Vt * 4},
      {(void**)&p.apart, (size_t)((c->Vt + 15) / 16) * NC * sizeof(ArgPart)},
      {(void**)&p.tok, NC * 4},
      {(void**)&p.pos, NC * 8},
      {(void**)&p.live, NC * 4},
      {(void**)&p.frames, NC * c->NCH * 4},
      {(void**)&p.key0, NC * 4},
      {(void**)&p.nkeys, NC * 4},
      {(void**)&p.part, NC * c->H * p.spans * (size_t)(c->hd + 2) * 8},
      {&p.wk, (size_t)c->H * rows * c->hd * es},
      {&p.wv, (size_t)c->H * rows * c->hd * es},
  };
  for (auto& r : reqs) {
    hipError_t e = dalloc(c, r.ptr, r.bytes);
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
      return fail(c, MOSHI_E_OOM, "prefill workspace: out of device memory");
    if (e != hipSuccess) return device_fail(c, e, "hipMalloc(prefill)");
  }
  for (size_t i = 0; i < 11; ++i) CKD(c, hipMemsetAsync(*reqs[i].ptr, 0, reqs[i].bytes, c->stream));
  std::vector<int> ones(NC, 1);
  CKD(c, hipMemcpyAsync(p.live, ones.data(), NC * 4, hipMemcpyHostToDevice, c->stream));
  CKD(c, hipStreamSynchronize(c->stream));
  p.rows = (int)rows;
  p.ready = true;
  return MOSHI_OK;
}

// One chunk of m frames (positions p0 .. p0 + m - 1) of slot `slot`.
hipError_t prefill_chunk(moshi_ctx* c, int slot, int64_t p0, int m) {
  PrefillWs& p = c->pf;
  const int dt = c->dtype, D = c->D, F = c->F, H = c->H, hd = c->hd, W = c->W;
  const int sr = m == 1 ? GEMV_SSQ_ROWS : 16;  // rows per sum-of-squares partial
  const int nss_D = (D + sr - 1) / sr;
  // window rows: row i holds position s0 + i; the chunk starts at row p0 - s0
  const int64_t s0 = p0 - (W - 1) > 0 ? p0 - (W - 1) : 0;
  const int c0 = (int)(p0 - s0);
  auto base = [&](GemmArgs a) {
    a.B = m;
    a.live = p.live;
    return a;
  };
  hipError_t e;
  {
    EmbedArgs a = embed_args(c);
    a.frames = p.frames; a.live = p.live; a.B = m; a.x = p.x; a.ssq_out = p.ssq; a.ssq_rows = sr;
    if ((e = launch_embed(dt, a, c->stream)) != hipSuccess) return e;
  }
  const int64_t ring_slot = (int64_t)slot * t_slot_stride(c);
  const int64_t ring_head = (int64_t)W * hd, win_head = (int64_t)p.rows * hd;
  for (int l = 0; l < c->L; ++l) {
    char* rk = (char*)c->ring_k + (ring_slot + l * t_layer_elems(c)) * c->esz;
    char* rv = (char*)c->ring_v + (ring_slot + l * t_layer_elems(c)) * c->esz;
    // the ring's earlier positions into the window's first rows
    if ((e = launch_window_copy(dt, p.wk, rk, 0, c0, s0, W, H, hd, win_head, ring_head, 0,
                                c->stream)) != hipSuccess ||
        (e = launch_window_copy(dt, p.wv, rv, 0, c0, s0, W, H, hd, win_head, ring_head, 0,
                                c->stream)) != hipSuccess)
      return e;
    {  // RMSNorm -> q|k|v -> RoPE(pos) -> the chunk's rows of the window
      GemmArgs a = base(t_qkv_args(c, l));
      a.X = p.x; a.ssq = p.ssq; a.n_ssq = nss_D; a.xn_out = m > 1 ? p.hn : nullptr;
      a.q_out = p.q; a.pos = p.pos;
      a.ring_k = (char*)p.wk + (size_t)c0 * hd * c->esz;
      a.ring_v = (char*)p.wv + (size_t)c0 * hd * c->esz;
      a.slot_stride = hd; a.layer_off = 0; a.head_stride = win_head; a.cap = 1;
      if ((e = gemm(c, PRO_NORM, EPI_QKV, a)) != hipSuccess) return e;
    }
    {
      PrefillAttnArgs pa;
      memset(&pa, 0, sizeof(pa));
      pa.a.q = p.q; pa.a.ldq = D; pa.a.ring_k = p.wk; pa.a.ring_v = p.wv;
      pa.a.head_stride = win_head; pa.a.cap = p.rows; pa.a.n_heads = H;
      pa.a.max_spans = p.spans; pa.a.part = p.part; pa.a.o_out = p.o; pa.a.ldo = D;
      pa.a.scalar_excl = -1;
      pa.key0 = p.key0; pa.nkeys = p.nkeys; pa.m = m;
      if ((e = launch_prefill_attn(dt, hd, pa, c->stream)) != hipSuccess) return e;
    }
    // the chunk's rows into the ring (the last W of them, later rows win)
    const int first = c0 + (m > W ? m - W : 0);
    if ((e = launch_window_copy(dt, p.wk, rk, first, c0 + m, s0, W, H, hd, win_head, ring_head, 1,
                                c->stream)) != hipSuccess ||
        (e = launch_window_copy(dt, p.wv, rv, first, c0 + m, s0, W, H, hd, win_head, ring_head, 1,
                                c->stream)) != hipSuccess)
      return e;
    {
      GemmArgs a = base(t_o_args(c, l));
      a.X = p.o; a.resid = p.x; a.ssq_out = p.ssq;
      if ((e = gemm(c, PRO_DIRECT, EPI_RESID, a)) != hipSuccess) return e;
    }
    {
      GemmArgs a = base(t_gu_args(c, l));
      a.X = p.x; a.ssq = p.ssq; a.n_ssq = nss_D; a.xn_out = m > 1 ? p.hn : nullptr; a.act = p.act;
      if ((e = gemm(c, PRO_NORM, EPI_SWIGLU, a)) != hipSuccess) return e;
    }
    {
      GemmArgs a = base(t_dn_args(c, l));
      a.X = p.act; a.resid = p.x; a.ssq_out = p.ssq;
      if ((e = gemm(c, PRO_DIRECT, EPI_RESID, a)) != hipSuccess) return e;
    }
  }
  {
    GemmArgs a = base(t_head_args(c));
    a.X = p.x; a.ssq = p.ssq; a.n_ssq = nss_D; a.xn_out = p.hid; a.logits = p.logits;
    a.ldo = c->Vt; a.apart = p.apart;
    if ((e = gemm(c, PRO_NORM, EPI_ARGMAX, a)) != hipSuccess) return e;
    if ((e = launch_argmax_reduce(p.apart, (c->Vt + 15) / 16, c->Vt, m, p.tok, 1, nullptr, 0, 0,
                                  c->stream)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

// ---- the persistent step kernel (one session) ----

// Builds the kernel's argument block and weight-pointer tables in device
// memory. Leaves c->persistent false when the shape or device does not allow
// it (the per-operation kernels are used then).
// The depformer's sections of a weight pointer table: [S * Ld][4] qkv, o,
// gate_up, down of (substep, layer); [Ld][2] attn_norm, mlp_norm; [S]
// previous-token tables; [S] heads.
void append_dep_tables(const moshi_ctx* c, std::vector<const void*>& tab, int* o_dw, int* o_dn,
                       int* o_de, int* o_dh) {
  *o_dw = (int)tab.size();
  for (int s = 0; s < c->S; ++s)
    for (int l = 0; l < c->Ld; ++l) {
      const int wi = s * c->Ld + l;
      for (const void* p : {c->dep_qkv[wi], c->dep_o[wi], c->dep_gate_up[wi], c->dep_down[wi]})
        tab.push_back(p);
    }
  *o_dn = (int)tab.size();
  for (int l = 0; l < c->Ld; ++l) {
    tab.push_back(c->dep_attn_norm[l]);
    tab.push_back(c->dep_mlp_norm[l]);
  }
  *o_de = (int)tab.size();
  for (int s = 0; s < c->S; ++s) tab.push_back(c->dep_emb[s]);
  *o_dh = (int)tab.size();
  for (int s = 0; s < c->S; ++s) tab.push_back(c->dep_head[s]);
}

// The multi-session depformer kernel: used at capacity 2..64 for an
// instantiated shape unless sampling is on (the draws run per operation) or
// MOSHI_DEP_MULTI=0 (the per-operation graph instead).
int setup_dep_multi(moshi_ctx* c) {
  const char* env = getenv("MOSHI_DEP_MULTI");
  if (c->B < 2 || (env && env[0] == '0') || !dep_multi_supported(c->dtype, c->hdd) ||
      c->S > DEP_MAX_KEYS_HOST || c->sampling)
    return MOSHI_OK;
  std::vector<const void*> tab;
  int o_dw, o_dn, o_de, o_dh;
  append_dep_tables(c, tab, &o_dw, &o_dn, &o_de, &o_dh);
  const size_t lds = tab.size() * sizeof(void*);  // the pointer table
  const int grid = dep_multi_grid(c->dtype, c->hdd, c->B, lds);
  if (grid < 1) return MOSHI_OK;
  void* d_tab = nullptr;
  CKD(c, dalloc(c, &d_tab, tab.size() * sizeof(void*)));
  CKD(c, hipMemcpy(d_tab, tab.data(), tab.size() * sizeof(void*), hipMemcpyHostToDevice));

  DepMultiArgs A;
  memset(&A, 0, sizeof(A));
  A.d_in = d_in_args(c); A.d_qkv = d_qkv_args(c, 0, 0); A.d_o = d_o_args(c, 0, 0);
  A.d_gu = d_gu_args(c, 0, 0); A.d_dn = d_dn_args(c, 0, 0); A.d_head = d_head_args(c, 0);
  A.d_attn = d_attn_args(c, 0, 0);
  EntryArgs& e = A.entry;
  e.pre = c->pre; e.ldpre = c->S * c->Dd; e.prev_tiles = (c->Va + 15) / 16; e.prev_n = c->Va;
  e.D = c->Dd; e.B = c->B; e.y = c->y; e.ssq_out = c->ssq_d; e.ssq_rows = ssq_rows(c);
  A.S = c->S; A.S_run = c->S_run; A.Ld = c->Ld; A.Dd = c->Dd; A.Va = c->Va; A.B = c->B;
  A.nch = c->NCH;
  A.d_layer_elems = d_layer_elems(c);
  A.dep_final_norm = dep_final_norm(c) ? 1 : 0;
  A.ref_excl_at = (c->c.flags & MOSHI_FLAG_DEP_REF_RING) ? c->S_run - 1 : -1;
  A.forced = c->d_forced; A.tokens = c->tokens; A.codes = c->codes; A.live = c->d_live;
  A.apart = c->apart;
  A.tab = (const void* const*)d_tab; A.n_tab = (int)tab.size();
  A.o_dw = o_dw; A.o_dn = o_dn; A.o_de = o_de; A.o_dh = o_dh;
  CKD(c, dalloc(c, (void**)&A.bar, 2 * STEP_BAR_WORDS * sizeof(unsigned)));
  CKD(c, hipMemset(A.bar, 0, 2 * STEP_BAR_WORDS * sizeof(unsigned)));
  if (!c->d_abort) {
    CKD(c, dalloc(c, (void**)&c->d_abort, sizeof(int)));
    CKD(c, hipMemset(c->d_abort, 0, sizeof(int)));
  }
  A.abort = c->d_abort;
  A.spin_limit = STEP_SPIN_LIMIT;
  CKD(c, dalloc(c, (void**)&c->d_dm, sizeof(DepMultiArgs)));
  CKD(c, hipMemcpy(c->d_dm, &A, sizeof(DepMultiArgs), hipMemcpyHostToDevice));
  c->dm_host = A;
  c->dm_grid = grid;
  c->dm_lds = lds;
  c->dep_multi = true;
  return MOSHI_OK;
}

int setup_step(moshi_ctx* c) {
  const char* env = getenv("MOSHI_STEP_KERNEL");
  if (c->B != 1 || (env && env[0] == '0') || !step_supported(c->dtype, c->hd, c->hdd) ||
      c->S > DEP_MAX_KEYS_HOST || c->sampling)
    return MOSHI_OK;
  // the flagged depformer inputs: a normed input pair per thread, at most 4
  // two-value lines per thread for a model-dtype input, whole lines
  if (c->Dd % 2 || c->Fd % 2 || c->Dd > 2 * STEP_THREADS || c->Fd > 8 * STEP_THREADS ||
      c->D % 2 || c->D > 8 * STEP_THREADS || c->max_spans > 8 ||
      step_ll_words(c->S, c->Ld, c->Dd, c->Fd, c->Va, c->L, c->H, c->hd, c->max_spans, c->D) * 8 >=
          (1LL << 31))
    return MOSHI_OK;
  const size_t es = c->esz, vec = es == 2 ? 8 : 4;
  // attention span scratch: per wave, 64 / (hd / vec) key rows of hd + 1 doubles, and a maximum
  auto attn_lds = [&](int hd) {
    return ((STEP_THREADS / (hd / vec)) * (size_t)(hd + 1) + STEP_THREADS / 64 + 1) * 8;
  };
  size_t kmax = c->D;
  for (int k : {c->F, c->Dd, c->Fd}) kmax = (size_t)k > kmax ? (size_t)k : kmax;
  size_t lds = kmax * es;
  lds = attn_lds(c->hd) > lds ? attn_lds(c->hd) : lds;
  lds = attn_lds(c->hdd) > lds ? attn_lds(c->hdd) : lds;
  const int grid = step_max_grid(c->dtype, c->hd, c->hdd, lds);
  if (grid < 1) return MOSHI_OK;
  // the depformer projections stage their weight slices in LDS, after the
  // largest depformer input vector
  const size_t wbuf = ((size_t)(c->Dd > c->Fd ? c->Dd : c->Fd) * es + 1023) / 1024 * 1024;
  if ((int64_t)grid * (3 * c->Dd > c->Fd ? 3 * c->Dd : c->Fd) >= (1LL << 31)) return MOSHI_OK;
  int64_t staged = 0;
  {
    const GemmArgs q = d_qkv_args(c, 0, 0), o = d_o_args(c, 0, 0), gu = d_gu_args(c, 0, 0),
                   dn = d_dn_args(c, 0, 0), hd = d_head_args(c, 0);
    const std::pair<int, const GemmArgs*> ops[] = {
        {EPI_QKV, &q}, {EPI_RESID, &o}, {EPI_SWIGLU, &gu}, {EPI_RESID, &dn}, {EPI_ARGMAX, &hd}};
    // the kernel's register copies of each wave's slice are sized per operation
    const int max_i[] = {LLR_QKV_I, LLR_O_I, LLR_GU_I, LLR_DN_I, LLR_HD_I};
    const int max_c[] = {LLR_QKV_C, LLR_O_C, LLR_GU_C, LLR_DN_C, LLR_HD_C};
    int k = 0;
    for (const auto& op : ops) {
      const int64_t b = staged_slice_bytes((int)vec, op.first, op.second->N, op.second->K, grid);
      staged = b > staged ? b : staged;
      const int cpl = (int)((op.second->K / (int)vec + 63) / 64);
      if (staged_items_per_wave(op.first, op.second->N, grid) > max_i[k] || cpl > max_c[k])
        return MOSHI_OK;
      ++k;
    }
  }
  lds = wbuf + staged > lds ? wbuf + staged : lds;

  std::vector<const void*> tab;
  const size_t o_tw = tab.size();
  for (int l = 0; l < c->L; ++l)
    for (const void* p : {c->attn_norm[l], c->qkv[l], c->wo[l], c->mlp_norm[l], c->gate_up[l],
                          c->down[l]})
      tab.push_back(p);
  int o_dw, o_dn, o_de, o_dh;
  append_dep_tables(c, tab, &o_dw, &o_dn, &o_de, &o_dh);

  void* d_tab = nullptr;
  CKD(c, dalloc(c, &d_tab, tab.size() * sizeof(void*)));
  CKD(c, hipMemcpy(d_tab, tab.data(), tab.size() * sizeof(void*), hipMemcpyHostToDevice));
  const void* const* dt = (const void* const*)d_tab;

  StepArgs A;
  memset(&A, 0, sizeof(A));
  A.emb = embed_args(c);
  A.t_qkv = t_qkv_args(c, 0); A.t_o = t_o_args(c, 0); A.t_gu = t_gu_args(c, 0);
  A.t_dn = t_dn_args(c, 0); A.t_head = t_head_args(c); A.t_attn = t_attn_args(c, 0);
  A.L = c->L; A.H = c->H; A.t_layer_elems = t_layer_elems(c);
  A.d_in = d_in_args(c); A.d_qkv = d_qkv_args(c, 0, 0); A.d_o = d_o_args(c, 0, 0);
  A.d_gu = d_gu_args(c, 0, 0); A.d_dn = d_dn_args(c, 0, 0); A.d_head = d_head_args(c, 0);
  A.d_attn = d_attn_args(c, 0, 0);
  A.tab = dt; A.n_tab = (int)tab.size();
  A.o_tw = (int)o_tw; A.o_dw = o_dw; A.o_dn = o_dn; A.o_de = o_de; A.o_dh = o_dh;
  A.wbuf_lds = (int)wbuf;
  // the pointer table goes to LDS after the scratch region
  lds = (lds + 15) / 16 * 16;
  A.tab_lds = (int)lds;
  lds += tab.size() * sizeof(void*);
  A.S = c->S; A.Ld = c->Ld; A.Hd = c->Hd; A.Dd = c->Dd; A.Vt = c->Vt; A.Va = c->Va;
  A.S_run = c->S_run;
  A.dep_final_norm = dep_final_norm(c) ? 1 : 0;
  A.d_attn.scalar_excl = (c->c.flags & MOSHI_FLAG_DEP_REF_RING) ? 0 : -1;  // on / off
  A.forced = c->d_forced;
  A.spin_limit = STEP_SPIN_LIMIT;
  A.ll_spin_limit = STEP_LL_SPIN_LIMIT;
  A.d_layer_elems = d_layer_elems(c);
  A.pre = c->pre; A.y = c->y; A.ssq_d = c->ssq_d; A.apart = c->apart;
  A.audio_logits = c->audio_logits;
  A.pos = c->d_pos; A.live = c->d_live;
  CKD(c, dalloc(c, (void**)&c->d_bar, 2 * STEP_BAR_WORDS * sizeof(unsigned)));
  CKD(c, dalloc(c, (void**)&c->d_abort, sizeof(int)));
  CKD(c, hipMemset(c->d_bar, 0, 2 * STEP_BAR_WORDS * sizeof(unsigned)));
  CKD(c, hipMemset(c->d_abort, 0, sizeof(int)));
  A.bar = c->d_bar; A.abort = c->d_abort;
  {
    const size_t ll_bytes =
        (size_t)step_ll_words(c->S, c->Ld, c->Dd, c->Fd, c->Va, c->L, c->H, c->hd, c->max_spans,
                              c->D) *
        sizeof(uint64_t);
    CKD(c, dalloc(c, (void**)&A.ll, ll_bytes));
    CKD(c, hipMemset(A.ll, 0, ll_bytes));
  }
  CKD(c, dalloc(c, (void**)&c->d_step, sizeof(StepArgs)));
  CKD(c, hipMemcpy(c->d_step, &A, sizeof(StepArgs), hipMemcpyHostToDevice));
  c->step_host = A;
  {
    // the allocation-free variant: barrier counters at the start of the
    // static scratch, the flagged arena after them; the abort flag stays the
    // context's (it reports back to this context's host calls)
    size_t sbytes = 0;
    void* sp = moshi_internal::static_scratch_setup(c->device, &sbytes);
    const size_t bar_bytes = 2 * (size_t)STEP_BAR_WORDS * sizeof(unsigned);
    const size_t arena_off = (bar_bytes + 65535) / 65536 * 65536;
    const size_t ll_bytes =
        (size_t)step_ll_words(c->S, c->Ld, c->Dd, c->Fd, c->Va, c->L, c->H, c->hd, c->max_spans,
                              c->D) *
        sizeof(uint64_t);
    if (sp == nullptr) {
      c->static_why = "the static scratch's address could not be found on this device";
    } else if (arena_off + ll_bytes > sbytes) {
      c->static_why = "this model's step needs " + std::to_string(arena_off + ll_bytes) +
                      " bytes of scratch; the static scratch holds " + std::to_string(sbytes);
    } else {
      StepArgs As = A;
      As.bar = (unsigned*)sp;
      As.ll = (uint64_t*)((char*)sp + arena_off);
      CKD(c, dalloc(c, (void**)&c->d_step_static, sizeof(StepArgs)));
      CKD(c, hipMemcpy(c->d_step_static, &As, sizeof(StepArgs), hipMemcpyHostToDevice));
    }
  }
  c->step_grid = step_max_grid(c->dtype, c->hd, c->hdd, lds);  // with the final LDS size
  if (c->step_grid != grid) return MOSHI_OK;  // the staged slices are sized for `grid`
  c->step_lds = lds;
  c->persistent = true;
  return MOSHI_OK;
}

// One full step of slot 0 on the stream; outputs to text_out [1], codes_out [S].
int launch_persistent(moshi_ctx* c, const int* frames, int* text_out, int* codes_out,
                      uint64_t* trace = nullptr) {
  if (++c->step_seq == 0) c->step_seq = 1;  // 0 is the arena's initial flag
  CKD(c, launch_step(c->dtype, c->hd, c->hdd, c->d_step, frames, text_out, codes_out,
                     c->step_parity, c->step_seq, c->step_grid, c->step_lds, c->stream, trace));
  c->step_parity ^= 1;
  return MOSHI_OK;
}

// A barrier wait ran out of time in an earlier launch: the context is lost.
int check_abort(moshi_ctx* c, int flag) {
  if (flag) {
    c->failed = true;
    c->err = "persistent kernel: a grid barrier or flagged wait timed out";
    return MOSHI_E_DEVICE;
  }
  return MOSHI_OK;
}

hipError_t capture(moshi_ctx* c, hipError_t (*fn)(moshi_ctx*), hipGraphExec_t* out) {
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return e;
  hipError_t e2 = fn(c);
  e = hipStreamEndCapture(c->stream, &g);
  if (e2 != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return e2;
  }
  if (e != hipSuccess) return e;
  e = hipGraphInstantiate(out, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  return e;
}

int ensure_graphs(moshi_ctx* c, bool temporal, bool dep) {
  if (!c->use_graphs || c->timing) return MOSHI_OK;
  if (temporal && !c->g_temporal) CKD(c, capture(c, enqueue_temporal, &c->g_temporal));
  if (dep && !c->g_dep && !c->dep_multi) CKD(c, capture(c, enqueue_depformer, &c->g_dep));
  return MOSHI_OK;
}

int launch_part(moshi_ctx* c, bool temporal) {
  if (!temporal && c->dep_multi && !c->timing) {
    CKD(c, launch_dep_multi(c->dtype, c->hdd, c->B, c->d_dm, c->dm_parity, c->dm_grid, c->dm_lds,
                            c->stream));
    c->dm_parity ^= 1;
    return MOSHI_OK;
  }
  if (c->use_graphs && !c->timing) {
    CKD(c, hipGraphLaunch(temporal ? c->g_temporal : c->g_dep, c->stream));
  } else {
    CKD(c, temporal ? enqueue_temporal(c) : enqueue_depformer(c));
  }
  return MOSHI_OK;
}

int check_ctx(moshi_ctx* c) {
  if (!c) return MOSHI_E_INVALID;
  if (c->failed) return MOSHI_E_DEVICE;
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return device_fail(c, e, "hipSetDevice");
  return MOSHI_OK;
}

int validate_frames(moshi_ctx* c, const int32_t* frames) {
  const char* e = moshi_host::frames_error(c->slots, frames, c->NCH, c->Vt, c->Va);
  return e ? fail(c, MOSHI_E_INVALID, e) : MOSHI_OK;
}

// The pinned metadata buffers may be rewritten: every copy out of them that
// an earlier call enqueued has completed.
int wait_meta(moshi_ctx* c) {
  if (c->meta_ev_pending) {
    CKD(c, hipEventSynchronize(c->meta_ev));
    c->meta_ev_pending = false;
  }
  return MOSHI_OK;
}

int record_meta(moshi_ctx* c) {
  CKD(c, hipEventRecord(c->meta_ev, c->stream));
  c->meta_ev_pending = true;
  return MOSHI_OK;
}

// Refresh the device copies of liveness and positions after a join, leave or
// prefill (the step advances the device positions itself). Stream-ordered:
// steps enqueued before keep the metadata they were enqueued with.
int upload_meta(moshi_ctx* c) {
  if (!c->slots.dirty && !c->samp_dirty) return MOSHI_OK;
  int rc = wait_meta(c);
  if (rc) return rc;
  if (c->slots.dirty) {
    for (int b = 0; b < c->B; ++b) {
      c->h_live[b] = c->slots.live[b];
      c->h_pos[b] = c->slots.pos[b];
    }
    CKD(c, hipMemcpyAsync(c->d_live, c->h_live, sizeof(int) * c->B, hipMemcpyHostToDevice, c->stream));
    CKD(c, hipMemcpyAsync(c->d_pos, c->h_pos, sizeof(int64_t) * c->B, hipMemcpyHostToDevice, c->stream));
    c->slots.dirty = false;
  }
  if (c->samp_dirty) {
    for (int b = 0; b < c->B; ++b) c->h_samp[b] = c->samp[b];
    CKD(c, hipMemcpyAsync(c->d_samp, c->h_samp, sizeof(SampleParams) * c->B, hipMemcpyHostToDevice,
                          c->stream));
    c->samp_dirty = false;
  }
  return record_meta(c);
}

// The forced tokens of the next step ([B][1+S], -1 = not forced; NULL = none
// forced), copied to the device only when they change.
int upload_forced(moshi_ctx* c, const int32_t* forced) {
  if (!forced && !c->forced_on_device) return MOSHI_OK;
  int rc = wait_meta(c);
  if (rc) return rc;
  const size_t n = (size_t)c->B * c->NCH;
  for (size_t i = 0; i < n; ++i)
    c->h_forced[i] = (forced && c->slots.live[i / c->NCH]) ? forced[i] : -1;
  CKD(c, hipMemcpyAsync(c->d_forced, c->h_forced, sizeof(int) * n, hipMemcpyHostToDevice,
                        c->stream));
  c->forced_on_device = forced != nullptr;
  return record_meta(c);
}

// Stage the host frames (zeros for free slots) and the slot metadata.
int upload_step_inputs(moshi_ctx* c, const int32_t* frames) {
  int rc = upload_meta(c);
  if (rc) return rc;
  if (!frames) return MOSHI_OK;
  for (int b = 0; b < c->B; ++b)
    for (int k = 0; k < c->NCH; ++k)
      c->h_frames[(size_t)b * c->NCH + k] = c->slots.live[b] ? frames[(size_t)b * c->NCH + k] : 0;
  CKD(c, hipMemcpyAsync(c->d_frames, c->h_frames, sizeof(int) * c->B * c->NCH,
                        hipMemcpyHostToDevice, c->stream));
  return MOSHI_OK;
}

int run_step(moshi_ctx* c, const int32_t* frames, int32_t* text_token, int32_t* audio_codes,
             bool with_dep, const int32_t* forced = nullptr) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if ((rc = validate_frames(c, frames))) return rc;
  if (const char* e = moshi_host::forced_error(c->slots, forced, c->NCH, c->Vt, c->Va))
    return fail(c, MOSHI_E_INVALID, e);
  const bool pers = c->persistent && with_dep && !c->timing;
  if (!pers && (rc = ensure_graphs(c, true, with_dep))) return rc;
  if ((rc = upload_step_inputs(c, frames))) return rc;
  if ((rc = upload_forced(c, forced))) return rc;
  int abort_flag = 0;
  if (pers) {
    if (live_count(c) > 0 && (rc = launch_persistent(c, c->d_frames, c->tokens, c->codes)))
      return rc;
    CKD(c, hipMemcpyAsync(&abort_flag, c->d_abort, sizeof(int), hipMemcpyDeviceToHost, c->stream));
  } else {
    if ((rc = launch_part(c, true))) return rc;
    if (with_dep && (rc = launch_part(c, false))) return rc;
    if (with_dep && c->dep_multi && !c->timing)
      CKD(c, hipMemcpyAsync(&abort_flag, c->d_abort, sizeof(int), hipMemcpyDeviceToHost,
                            c->stream));
  }
  CKD(c, hipMemcpyAsync(c->h_tokens, c->tokens, sizeof(int) * c->B, hipMemcpyDeviceToHost, c->stream));
  if (with_dep)
    CKD(c, hipMemcpyAsync(c->h_codes, c->codes, sizeof(int) * c->B * c->S, hipMemcpyDeviceToHost,
                          c->stream));
  CKD(c, hipStreamSynchronize(c->stream));
  c->meta_ev_pending = false;
  if ((rc = check_abort(c, abort_flag))) return rc;
  c->slots.advance();
  for (int b = 0; b < c->B; ++b) {
    if (text_token) text_token[b] = c->slots.live[b] ? c->h_tokens[b] : -1;
    if (with_dep && audio_codes)
      for (int s = 0; s < c->S; ++s)
        audio_codes[(size_t)b * c->S + s] =
            (c->slots.live[b] && s < c->S_run) ? c->h_codes[(size_t)b * c->S + s] : -1;
  }
  return MOSHI_OK;
}

int upload_weights(moshi_ctx* c, const void* const* t) {
  const moshi_config& k = c->c;
  const size_t es = c->esz;
  const int D = c->D, F = c->F, Dd = c->Dd, Fd = c->Fd, S = c->S, Vt = c->Vt, Va = c->Va;
  int i = 0;
  auto put = [&](const void* src, size_t elems, const void** dst) -> int {
    void* p;
    hipError_t e = dalloc(c, &p, elems * es);
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return fail(c, MOSHI_E_OOM, "weights: out of device memory");
    if (e != hipSuccess) return device_fail(c, e, "hipMalloc(weights)");
    if (!src) return fail(c, MOSHI_E_INVALID, "NULL weight tensor");
    e = hipMemcpy(p, src, elems * es, hipMemcpyHostToDevice);
    if (e != hipSuccess) return device_fail(c, e, "hipMemcpy(weights)");
    *dst = p;
    return MOSHI_OK;
  };
  int rc;
  (void)k;
  if ((rc = put(t[i++], (size_t)(Vt + 1) * D, &c->emb_text))) return rc;
  c->emb_audio.resize(S);
  for (int s = 0; s < S; ++s)
    if ((rc = put(t[i++], (size_t)(Va + 1) * D, &c->emb_audio[s]))) return rc;
  c->attn_norm.resize(c->L); c->qkv.resize(c->L); c->wo.resize(c->L);
  c->mlp_norm.resize(c->L); c->gate_up.resize(c->L); c->down.resize(c->L);
  for (int l = 0; l < c->L; ++l) {
    if ((rc = put(t[i++], D, &c->attn_norm[l]))) return rc;
    if ((rc = put(t[i++], (size_t)3 * D * D, &c->qkv[l]))) return rc;
    if ((rc = put(t[i++], (size_t)D * D, &c->wo[l]))) return rc;
    if ((rc = put(t[i++], D, &c->mlp_norm[l]))) return rc;
    if ((rc = put(t[i++], (size_t)2 * F * D, &c->gate_up[l]))) return rc;
    if ((rc = put(t[i++], (size_t)D * F, &c->down[l]))) return rc;
  }
  if ((rc = put(t[i++], D, &c->out_norm))) return rc;
  if ((rc = put(t[i++], (size_t)Vt * D, &c->text_head))) return rc;
  {  // the S input projections, contiguous: one [S*Dd, D] matrix
    void* p;
    const size_t one = (size_t)Dd * D;
    hipError_t e = dalloc(c, &p, one * S * es);
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return fail(c, MOSHI_E_OOM, "weights: out of device memory");
    if (e != hipSuccess) return device_fail(c, e, "hipMalloc(dep_in)");
    for (int s = 0; s < S; ++s) {
      const void* src = t[i++];
      if (!src) return fail(c, MOSHI_E_INVALID, "NULL weight tensor");
      CKD(c, hipMemcpy((char*)p + one * s * es, src, one * es, hipMemcpyHostToDevice));
    }
    c->dep_in = p;
  }
  c->dep_emb.resize(S);
  for (int s = 0; s < S; ++s)
    if ((rc = put(t[i++], (size_t)((s == 0 ? Vt : Va) + 1) * Dd, &c->dep_emb[s]))) return rc;
  c->dep_attn_norm.resize(c->Ld); c->dep_mlp_norm.resize(c->Ld);
  for (int l = 0; l < c->Ld; ++l) {
    if ((rc = put(t[i++], Dd, &c->dep_attn_norm[l]))) return rc;
    if ((rc = put(t[i++], Dd, &c->dep_mlp_norm[l]))) return rc;
  }
  const int n = S * c->Ld;
  c->dep_qkv.resize(n); c->dep_o.resize(n); c->dep_gate_up.resize(n); c->dep_down.resize(n);
  for (int s = 0; s < S; ++s)
    for (int l = 0; l < c->Ld; ++l) {
      const int wi = s * c->Ld + l;
      if ((rc = put(t[i++], (size_t)3 * Dd * Dd, &c->dep_qkv[wi]))) return rc;
      if ((rc = put(t[i++], (size_t)Dd * Dd, &c->dep_o[wi]))) return rc;
      if ((rc = put(t[i++], (size_t)2 * Fd * Dd, &c->dep_gate_up[wi]))) return rc;
      if ((rc = put(t[i++], (size_t)Dd * Fd, &c->dep_down[wi]))) return rc;
    }
  c->dep_head.resize(S);
  for (int s = 0; s < S; ++s)
    if ((rc = put(t[i++], (size_t)Va * Dd, &c->dep_head[s]))) return rc;
  if (dep_final_norm(c) && (rc = put(t[i++], Dd, &c->dep_out_norm))) return rc;
  return MOSHI_OK;
}

int alloc_buffers(moshi_ctx* c) {
  const size_t B = c->B, es = c->esz;
  const size_t D = c->D, F = c->F, Dd = c->Dd, Fd = c->Fd, S = c->S;
  struct Req {
    void** p;
    size_t bytes;
  };
  // temporal attention: one workgroup per (slot, head, key span); with one
  // session the spans of all heads fill the CUs once
  {
    const int by_len = (c->W + ATTN_CHUNK - 1) / ATTN_CHUNK;
    int n = c->ncu / c->H;
    n = n < 1 ? 1 : n;
    c->max_spans = n < by_len ? n : by_len;
    if (c->max_spans > 8) c->max_spans = 8;  // the step kernel merges at most 8 span partials
    // five or more sessions: (slot, head) pairs fill the CUs already; 4
    // longer spans per head measured faster than 8 (B=16: 3.42 -> 3.25 ms of
    // attention and merge per step, B=64: 16.96 -> 16.60) and than 2 or ~23;
    // up to four sessions 8 stay (full rings: B=3 10.23 -> 10.08 ms per step
    // with 8, B=4 10.44 -> 10.35)
    if (c->B > 4 && c->max_spans > 4) c->max_spans = 4;
  }
  const size_t hmax = c->H > c->Hd ? c->H : c->Hd;
  const size_t hdmax = c->hd > c->hdd ? c->hd : c->hdd;
  const size_t ntile_max = ((size_t)(c->Vt > c->Va ? c->Vt : c->Va) + 15) / 16;  // argmax tiles
  Req reqs[] = {
      {&c->ring_k, B * c->L * c->H * c->W * c->hd * es},
      {&c->ring_v, B * c->L * c->H * c->W * c->hd * es},
      {&c->dkv_k, B * c->Ld * c->Hd * S * c->hdd * es},
      {&c->dkv_v, B * c->Ld * c->Hd * S * c->hdd * es},
      {(void**)&c->x, B * D * 8},
      {(void**)&c->ssq, ((D + 1) / 2) * B * 8},
      {(void**)&c->q, B * D * 8},
      {&c->o, B * D * es},
      {&c->act, B * F * es},
      {&c->hid, B * D * es},
      {&c->hn, B * D * es},
      {(void**)&c->pre, B * S * Dd * 8},
      {(void**)&c->y, B * Dd * 8},
      {(void**)&c->ssq_d, ((Dd + 1) / 2) * B * 8},
      {(void**)&c->qd, B * Dd * 8},
      {&c->od, B * Dd * es},
      {&c->actd, B * Fd * es},
      {&c->hnd, B * Dd * es},
      {(void**)&c->text_logits, B * c->Vt * 4},
      {(void**)&c->audio_logits, B * S * c->Va * 4},
      {(void**)&c->tokens, B * 4},
      {(void**)&c->codes, B * S * 4},
      {(void**)&c->apart, ntile_max * B * sizeof(ArgPart)},
      {(void**)&c->attn_part, B * hmax * c->max_spans * (hdmax + 2) * 8},
      {(void**)&c->d_frames, B * c->NCH * 4},
      {(void**)&c->d_live, B * 4},
      {(void**)&c->d_pos, B * 8},
      {(void**)&c->d_err, 4},
      {(void**)&c->d_forced, B * c->NCH * 4},
      {(void**)&c->d_samp, B * sizeof(SampleParams)},
      {(void**)&c->d_inv_freq, (size_t)(c->hd / 2) * 8},
      {&c->staging, (size_t)c->W * D * es},
      // K-segment sums and counters of split MFMA projections (zeroed here;
      // each counter is reset by the segment that completes it)
      {(void**)&c->kpart, (size_t)(Dd + 15) / 16 * 4 * GEMM_KSPLIT_MAX * 64 * 4 * 8},
      {(void**)&c->kcnt, (size_t)(Dd + 15) / 16 * 4 * 4},
  };
  for (auto& r : reqs) {
    hipError_t e = dalloc(c, r.p, r.bytes);
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return fail(c, MOSHI_E_OOM, "buffers: out of device memory");
    if (e != hipSuccess) return device_fail(c, e, "hipMalloc(buffers)");
  }
  // Zero everything but the rings (activations of free slots then hold finite
  // values). The rings need no clearing: only positions a session has written
  // are ever attended.
  for (size_t i = 4; i < sizeof(reqs) / sizeof(reqs[0]); ++i)
    CKD(c, hipMemsetAsync(*reqs[i].p, 0, reqs[i].bytes, c->stream));
  CKD(c, hipMemsetAsync(c->d_forced, 0xff, B * c->NCH * 4, c->stream));  // -1: nothing forced
  std::vector<double> inv(c->hd / 2);
  for (int i = 0; i < c->hd / 2; ++i) inv[i] = pow((double)c->c.rope_theta, -2.0 * i / c->hd);
  CKD(c, hipMemcpyAsync(c->d_inv_freq, inv.data(), sizeof(double) * inv.size(), hipMemcpyHostToDevice,
                        c->stream));
  CKD(c, hipStreamSynchronize(c->stream));
  // pinned host staging
  CKD(c, hipHostMalloc((void**)&c->h_frames, sizeof(int) * B * c->NCH, hipHostMallocDefault));
  CKD(c, hipHostMalloc((void**)&c->h_live, sizeof(int) * B, hipHostMallocDefault));
  CKD(c, hipHostMalloc((void**)&c->h_pos, sizeof(int64_t) * B, hipHostMallocDefault));
  CKD(c, hipHostMalloc((void**)&c->h_tokens, sizeof(int) * B, hipHostMallocDefault));
  CKD(c, hipHostMalloc((void**)&c->h_codes, sizeof(int) * B * S, hipHostMallocDefault));
  CKD(c, hipHostMalloc((void**)&c->h_forced, sizeof(int) * B * c->NCH, hipHostMallocDefault));
  CKD(c, hipHostMalloc((void**)&c->h_samp, sizeof(SampleParams) * B, hipHostMallocDefault));
  CKD(c, hipEventCreateWithFlags(&c->meta_ev, hipEventDisableTiming));
  return MOSHI_OK;
}

void release(moshi_ctx* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  if (c->stream) (void)hipStreamSynchronize(c->stream);
  if (c->g_temporal) (void)hipGraphExecDestroy(c->g_temporal);
  if (c->g_dep) (void)hipGraphExecDestroy(c->g_dep);
  for (hipEvent_t e : c->ev) (void)hipEventDestroy(e);
  for (void* p : c->dev_alloc) (void)hipFree(p);
  if (c->h_frames) (void)hipHostFree(c->h_frames);
  if (c->h_live) (void)hipHostFree(c->h_live);
  if (c->h_pos) (void)hipHostFree(c->h_pos);
  if (c->h_tokens) (void)hipHostFree(c->h_tokens);
  if (c->h_codes) (void)hipHostFree(c->h_codes);
  if (c->h_forced) (void)hipHostFree(c->h_forced);
  if (c->h_samp) (void)hipHostFree(c->h_samp);
  if (c->meta_ev) (void)hipEventDestroy(c->meta_ev);
  if (c->own_stream && c->stream) (void)hipStreamDestroy(c->stream);
  delete c;
}

// Per-operation timing of the persistent step kernel: workgroup 0 stamps the
// wall clock after every grid barrier; the interval that ends at barrier k is
// charged to operation k (its work plus the barrier). The operation sequence
// is the per-operation path's, without its argmax-reduce launches and
// depformer substep entries (folded into the next operation) and its
// attention span merges (done inside the attention operation).
int time_step_phases(moshi_ctx* c, const int32_t* frames, int n_steps, std::vector<double>& acc_ms,
                     std::vector<double>& acc_b, std::vector<int64_t>& acc_n) {
  int rate_khz = 0;
  CKD(c, hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, c->device));
  if (rate_khz <= 0) return fail(c, MOSHI_E_DEVICE, "no wall clock rate");
  void* d_trace = nullptr;
  CKD(c, hipMalloc(&d_trace, STEP_TRACE_MAX * sizeof(uint64_t)));
  std::vector<uint64_t> tr(STEP_TRACE_MAX);
  int rc = MOSHI_OK;
  for (int it = 0; it < n_steps && rc == MOSHI_OK; ++it) {
    c->dry = true;
    c->ev_class.clear();
    c->ev_bytes.clear();
    (void)enqueue_temporal(c);
    (void)enqueue_depformer(c);
    c->dry = false;
    std::vector<int> cls;
    std::vector<double> by;
    double carry = 0.0;  // bytes of an operation folded into the next one
    for (size_t i = 0; i < c->ev_class.size(); ++i) {
      const int k = c->ev_class[i];
      if (k == KC_D_ATTN && !by.empty()) {
        by.back() += c->ev_bytes[i];  // the depformer attention ends the q/k/v phase
        continue;
      }
      if (k == KC_ARGMAX || k == KC_T_COMBINE || k == KC_D_ENTRY) {
        carry += c->ev_bytes[i];
        continue;
      }
      cls.push_back(k);
      by.push_back(c->ev_bytes[i] + carry);
      carry = 0.0;
    }
    const size_t nb = cls.size();
    if (nb + 2 > (size_t)STEP_TRACE_MAX || live_count(c) == 0) {
      rc = fail(c, MOSHI_E_INVALID, "step too long to trace, or no live session");
      break;
    }
    if ((rc = upload_step_inputs(c, frames))) break;
    if ((rc = launch_persistent(c, c->d_frames, c->tokens, c->codes, (uint64_t*)d_trace))) break;
    int abort_flag = 0;
    hipError_t e = hipMemcpyAsync(tr.data(), d_trace, (nb + 2) * sizeof(uint64_t),
                                  hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(&abort_flag, c->d_abort, sizeof(int), hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) {
      rc = device_fail(c, e, "step trace");
      break;
    }
    if ((rc = check_abort(c, abort_flag))) break;
    c->slots.advance();
    const double ms_per_tick = 1.0 / (double)rate_khz;
    for (size_t k = 0; k < nb; ++k) {
      acc_ms[cls[k]] += (double)(tr[k + 1] - tr[k]) * ms_per_tick;
      acc_b[cls[k]] += by[k];
      acc_n[cls[k]] += 1;
    }
    acc_ms[KC_ARGMAX] += (double)(tr[nb + 1] - tr[nb]) * ms_per_tick;
    acc_n[KC_ARGMAX] += 1;
  }
  (void)hipFree(d_trace);
  return rc;
}

// Kernel timing with the multi-session depformer kernel: the temporal
// step's kernels bracketed by events, the depformer kernel's phases from its
// trace, each under the class of the per-operation kernel it replaces (a norm
// phase under the projection it feeds, the last code under argmax_reduce),
// with that path's byte counts.
int time_dep_multi(moshi_ctx* c, const int32_t* frames, int n_steps, std::vector<double>& acc_ms,
                   std::vector<double>& acc_b, std::vector<int64_t>& acc_n) {
  int rate_khz = 0;
  CKD(c, hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, c->device));
  if (rate_khz <= 0) return fail(c, MOSHI_E_DEVICE, "no wall clock rate");
  std::vector<int> phases{KC_D_INPROJ};
  for (int s = 0; s < c->S_run; ++s) {
    phases.push_back(KC_D_ENTRY);
    for (int l = 0; l < c->Ld; ++l)
      for (int k : {KC_D_QKV, KC_D_QKV, KC_D_ATTN, KC_D_O, KC_D_GATEUP, KC_D_GATEUP, KC_D_DOWN})
        phases.push_back(k);
    phases.push_back(KC_D_HEAD);
    phases.push_back(KC_D_HEAD);
  }
  phases.push_back(KC_ARGMAX);
  if (phases.size() + 1 > (size_t)STEP_TRACE_MAX) return fail(c, MOSHI_E_INVALID, "step too long to trace");
  std::vector<double> dep_bytes(KC_COUNT, 0.0);
  c->dry = true;
  c->ev_class.clear();
  c->ev_bytes.clear();
  (void)enqueue_depformer(c);
  c->dry = false;
  for (size_t i = 0; i < c->ev_class.size(); ++i) dep_bytes[c->ev_class[i]] += c->ev_bytes[i];
  void* d_trace = nullptr;
  CKD(c, hipMalloc(&d_trace, STEP_TRACE_MAX * sizeof(uint64_t)));
  std::vector<uint64_t> tr(phases.size() + 1);
  int rc = MOSHI_OK;
  for (int it = 0; it < n_steps && rc == MOSHI_OK; ++it) {
    c->ev_used = 0;
    c->ev_class.clear();
    c->ev_bytes.clear();
    if ((rc = upload_step_inputs(c, frames)) || (rc = upload_forced(c, nullptr))) break;
    c->timing = true;
    hipError_t e = enqueue_temporal(c);
    c->timing = false;
    if (e == hipSuccess)
      e = launch_dep_multi(c->dtype, c->hdd, c->B, c->d_dm, c->dm_parity, c->dm_grid, c->dm_lds,
                           c->stream, (uint64_t*)d_trace);
    c->dm_parity ^= 1;
    int abort_flag = 0;
    if (e == hipSuccess)
      e = hipMemcpyAsync(tr.data(), d_trace, tr.size() * sizeof(uint64_t), hipMemcpyDeviceToHost,
                         c->stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(&abort_flag, c->d_abort, sizeof(int), hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) {
      rc = device_fail(c, e, "depformer kernel trace");
      break;
    }
    c->meta_ev_pending = false;
    if ((rc = check_abort(c, abort_flag))) break;
    c->slots.advance();
    for (size_t i = 0; i < c->ev_class.size(); ++i) {
      float t = 0.f;
      if ((e = hipEventElapsedTime(&t, c->ev[2 * i], c->ev[2 * i + 1])) != hipSuccess) {
        rc = device_fail(c, e, "hipEventElapsedTime");
        break;
      }
      acc_ms[c->ev_class[i]] += t;
      acc_b[c->ev_class[i]] += c->ev_bytes[i];
      acc_n[c->ev_class[i]] += 1;
    }
    const double ms_per_tick = 1.0 / (double)rate_khz;
    for (size_t k = 0; k < phases.size(); ++k) {
      acc_ms[phases[k]] += (double)(tr[k + 1] - tr[k]) * ms_per_tick;
      acc_n[phases[k]] += 1;
    }
    for (int k = 0; k < KC_COUNT; ++k) acc_b[k] += dep_bytes[k];
  }
  (void)hipFree(d_trace);
  return rc;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================

extern "C" {

int32_t moshi_n_tensors(const moshi_config* cfg) {
  if (config_error(cfg)) return MOSHI_E_INVALID;
  return tensor_count(cfg);
}

const char* moshi_strerror(int status) {
  switch (status) {
    case MOSHI_OK: return "ok";
    case MOSHI_E_INVALID: return "invalid argument";
    case MOSHI_E_FULL: return "all session slots are taken";
    case MOSHI_E_NOSESSION: return "no live session in that slot";
    case MOSHI_E_DEVICE: return "device error";
    case MOSHI_E_OOM: return "out of device memory";
  }
  return "unknown status";
}

const char* moshi_last_error(const moshi_ctx* ctx) { return ctx ? ctx->err.c_str() : ""; }

int32_t moshi_uses_step_kernel(const moshi_ctx* ctx) {
  if (!ctx) return MOSHI_E_INVALID;
  return ctx->persistent ? 1 : 0;
}

int32_t moshi_uses_dep_kernel(const moshi_ctx* ctx) {
  if (!ctx) return MOSHI_E_INVALID;
  return ctx->dep_multi ? 1 : 0;
}

const char* moshi_kernel_class_name(int32_t c) {
  return (c >= 0 && c < KC_COUNT) ? kClassNames[c] : "";
}

int moshi_create(const moshi_config* cfg, const void* const* tensors, int32_t n_tensors,
                 void* hip_stream, moshi_ctx** out) {
  if (!out) return MOSHI_E_INVALID;
  *out = nullptr;
  if (config_error(cfg) || !tensors) return MOSHI_E_INVALID;
  if (n_tensors != tensor_count(cfg)) return MOSHI_E_INVALID;
  for (int i = 0; i < n_tensors; ++i)
    if (!tensors[i]) return MOSHI_E_INVALID;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return MOSHI_E_DEVICE;

  moshi_ctx* c = new moshi_ctx();
  c->c = *cfg;
  c->B = cfg->max_sessions;
  c->dtype = cfg->dtype == MOSHI_BF16 ? DT_BF16 : DT_F32;
  c->esz = cfg->dtype == MOSHI_BF16 ? 2 : 4;
  c->D = cfg->dim; c->H = cfg->n_heads; c->hd = cfg->dim / cfg->n_heads; c->F = cfg->ffn_hidden;
  c->W = cfg->window; c->L = cfg->n_layers;
  c->Dd = cfg->dep_dim; c->Hd = cfg->dep_heads; c->hdd = cfg->dep_dim / cfg->dep_heads;
  c->Fd = cfg->dep_ffn_hidden; c->Ld = cfg->dep_layers; c->S = cfg->n_substeps;
  c->Vt = cfg->text_vocab; c->Va = cfg->audio_card; c->NCH = 1 + cfg->n_substeps;
  c->slots.init(c->B);
  c->S_run = moshi_host::dep_steps(cfg);
  c->sampling = (cfg->flags & MOSHI_FLAG_SAMPLING) != 0;
  c->samp.assign(c->B, SampleParams{});  // temperature 0: greedy
  const char* ng = getenv("MOSHI_NO_GRAPH");
  c->use_graphs = !(ng && ng[0] == '1');
  if (hipGetDevice(&c->device) != hipSuccess) {
    release(c);
    return MOSHI_E_DEVICE;
  }
  {
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, c->device) == hipSuccess)
      set_gemv_grid(ncu);
    c->ncu = ncu > 0 ? ncu : 1;
  }
  int rc = MOSHI_OK;
  if (hip_stream) {
    c->stream = (hipStream_t)hip_stream;
  } else {
    if (hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking) != hipSuccess) {
      release(c);
      return MOSHI_E_DEVICE;
    }
    c->own_stream = true;
  }
  if ((rc = alloc_buffers(c)) || (rc = upload_weights(c, tensors)) || (rc = setup_step(c)) ||
      (rc = setup_dep_multi(c))) {
    release(c);
    return rc;
  }
  *out = c;
  return MOSHI_OK;
}

int moshi_get_config(const moshi_ctx* ctx, moshi_config* out) {
  if (!ctx || !out) return MOSHI_E_INVALID;
  *out = ctx->c;
  return MOSHI_OK;
}

int moshi_destroy(moshi_ctx* ctx) {
  release(ctx);
  return MOSHI_OK;
}

int moshi_session_join(moshi_ctx* ctx, int32_t* slot_out) {
  if (!ctx || !slot_out) return MOSHI_E_INVALID;
  if (ctx->failed) return MOSHI_E_DEVICE;
  const int b = ctx->slots.join();
  if (b < 0) return fail(ctx, MOSHI_E_FULL, "every slot is live");
  if (ctx->sampling) {
    ctx->samp[b] = SampleParams{};  // a new session is greedy until told otherwise
    ctx->samp_dirty = true;
  }
  *slot_out = b;
  return MOSHI_OK;
}

int moshi_session_set_sampling(moshi_ctx* ctx, int32_t slot, const moshi_sampling* p) {
  if (!ctx) return MOSHI_E_INVALID;
  if (ctx->failed) return MOSHI_E_DEVICE;
  if (!ctx->slots.is_live(slot)) return fail(ctx, MOSHI_E_NOSESSION, "slot not live");
  SampleParams q{};
  if (p) {
    q.temperature[0] = p->text_temperature > 0.0 ? p->text_temperature : 0.0;
    q.temperature[1] = p->audio_temperature > 0.0 ? p->audio_temperature : 0.0;
    q.top_k[0] = p->text_top_k;
    q.top_k[1] = p->audio_top_k;
    q.seed = p->seed;
    if (!(p->text_temperature == p->text_temperature) ||
        !(p->audio_temperature == p->audio_temperature))
      return fail(ctx, MOSHI_E_INVALID, "temperature is NaN");
  }
  const bool draws = q.temperature[0] > 0.0 || q.temperature[1] > 0.0;
  if (draws && !ctx->sampling)
    return fail(ctx, MOSHI_E_INVALID, "the context was created without MOSHI_FLAG_SAMPLING");
  if (!ctx->sampling) return MOSHI_OK;  // greedy is all it does
  ctx->samp[slot] = q;
  ctx->samp_dirty = true;
  return MOSHI_OK;
}

int moshi_session_leave(moshi_ctx* ctx, int32_t slot) {
  if (!ctx) return MOSHI_E_INVALID;
  if (ctx->failed) return MOSHI_E_DEVICE;
  if (!ctx->slots.leave(slot)) return fail(ctx, MOSHI_E_NOSESSION, "slot not live");
  return MOSHI_OK;
}

int moshi_step(moshi_ctx* ctx, const int32_t* frames, int32_t* text_token, int32_t* audio_codes) {
  return run_step(ctx, frames, text_token, audio_codes, true);
}

int moshi_step_forced(moshi_ctx* ctx, const int32_t* frames, const int32_t* forced,
                      int32_t* text_token, int32_t* audio_codes) {
  return run_step(ctx, frames, text_token, audio_codes, true, forced);
}

int moshi_test_set_spin_limit(moshi_ctx* c, int32_t limit) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (limit < 1) return fail(c, MOSHI_E_INVALID, "spin limit must be >= 1");
  if (!c->persistent && !c->dep_multi)
    return fail(c, MOSHI_E_INVALID, "no persistent kernel on this context");
  CKD(c, hipStreamSynchronize(c->stream));
  if (c->persistent) {
    c->step_host.spin_limit = limit;
    c->step_host.ll_spin_limit = limit;
    CKD(c, hipMemcpy(c->d_step, &c->step_host, sizeof(StepArgs), hipMemcpyHostToDevice));
  }
  if (c->dep_multi) {
    c->dm_host.spin_limit = limit;
    CKD(c, hipMemcpy(c->d_dm, &c->dm_host, sizeof(DepMultiArgs), hipMemcpyHostToDevice));
  }
  return MOSHI_OK;
}

int moshi_step_enqueue(moshi_ctx* c, const int32_t* d_frames, int32_t* d_text_token,
                       int32_t* d_audio_codes) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!d_frames) return fail(c, MOSHI_E_INVALID, "frames is NULL");
  if ((rc = upload_forced(c, nullptr))) return rc;
  if (c->persistent) {
    if ((rc = upload_meta(c))) return rc;
    if (live_count(c) > 0) {
      if ((rc = launch_persistent(c, d_frames, d_text_token ? d_text_token : c->tokens,
                                  d_audio_codes ? d_audio_codes : c->codes)))
        return rc;
    } else {
      if (d_text_token) CKD(c, hipMemsetAsync(d_text_token, 0xff, sizeof(int) * c->B, c->stream));
      if (d_audio_codes)
        CKD(c, hipMemsetAsync(d_audio_codes, 0xff, sizeof(int) * c->B * c->S, c->stream));
    }
  } else {
    if ((rc = ensure_graphs(c, true, true))) return rc;
    if ((rc = upload_meta(c))) return rc;
    CKD(c, hipMemcpyAsync(c->d_frames, d_frames, sizeof(int) * c->B * c->NCH,
                          hipMemcpyDeviceToDevice, c->stream));
    if ((rc = launch_part(c, true))) return rc;
    if ((rc = launch_part(c, false))) return rc;
    if (d_text_token)
      CKD(c, hipMemcpyAsync(d_text_token, c->tokens, sizeof(int) * c->B, hipMemcpyDeviceToDevice,
                            c->stream));
    if (d_audio_codes)
      CKD(c, hipMemcpyAsync(d_audio_codes, c->codes, sizeof(int) * c->B * c->S,
                            hipMemcpyDeviceToDevice, c->stream));
  }
  c->slots.advance();
  return MOSHI_OK;
}

int moshi_sync(moshi_ctx* c) {
  int rc = check_ctx(c);
  if (rc) return rc;
  int bad = 0, abort_flag = 0;
  CKD(c, hipMemcpyAsync(&bad, c->d_err, sizeof(int), hipMemcpyDeviceToHost, c->stream));
  if (c->persistent || c->dep_multi)
    CKD(c, hipMemcpyAsync(&abort_flag, c->d_abort, sizeof(int), hipMemcpyDeviceToHost, c->stream));
  CKD(c, hipStreamSynchronize(c->stream));
  if ((rc = check_abort(c, abort_flag))) return rc;
  if (bad) {
    CKD(c, hipMemsetAsync(c->d_err, 0, sizeof(int), c->stream));
    CKD(c, hipStreamSynchronize(c->stream));
    return fail(c, MOSHI_E_INVALID, "a live frame code was out of range (clamped)");
  }
  return MOSHI_OK;
}

int moshi_temporal_step(moshi_ctx* ctx, const int32_t* frames, int32_t* text_token) {
  return run_step(ctx, frames, text_token, nullptr, false);
}

int moshi_depformer_step(moshi_ctx* c, const void* hidden, const int32_t* text_in,
                         int32_t* audio_codes) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!hidden || !text_in) return fail(c, MOSHI_E_INVALID, "NULL argument");
  for (int b = 0; b < c->B; ++b)
    if (c->slots.live[b] && (text_in[b] < 0 || text_in[b] > c->Vt))
      return fail(c, MOSHI_E_INVALID, "text token out of range");
  if ((rc = ensure_graphs(c, false, true))) return rc;
  if ((rc = upload_step_inputs(c, nullptr))) return rc;
  if ((rc = upload_forced(c, nullptr))) return rc;
  for (int b = 0; b < c->B; ++b) c->h_tokens[b] = c->slots.live[b] ? text_in[b] : 0;
  CKD(c, hipMemcpyAsync(c->tokens, c->h_tokens, sizeof(int) * c->B, hipMemcpyHostToDevice, c->stream));
  CKD(c, hipMemcpyAsync(c->hid, hidden, (size_t)c->B * c->D * c->esz, hipMemcpyHostToDevice, c->stream));
  if ((rc = launch_part(c, false))) return rc;
  int abort_flag = 0;
  if (c->dep_multi && !c->timing)
    CKD(c, hipMemcpyAsync(&abort_flag, c->d_abort, sizeof(int), hipMemcpyDeviceToHost, c->stream));
  CKD(c, hipMemcpyAsync(c->h_codes, c->codes, sizeof(int) * c->B * c->S, hipMemcpyDeviceToHost, c->stream));
  CKD(c, hipStreamSynchronize(c->stream));
  c->meta_ev_pending = false;
  if ((rc = check_abort(c, abort_flag))) return rc;
  if (audio_codes)
    for (int b = 0; b < c->B; ++b)
      for (int s = 0; s < c->S; ++s)
        audio_codes[(size_t)b * c->S + s] =
            (c->slots.live[b] && s < c->S_run) ? c->h_codes[(size_t)b * c->S + s] : -1;
  return MOSHI_OK;
}

int moshi_session_prefill_kv(moshi_ctx* c, int32_t slot, int32_t n, const void* k, const void* v) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->slots.is_live(slot)) return fail(c, MOSHI_E_NOSESSION, "slot not live");
  if (n < 0 || n > c->W) return fail(c, MOSHI_E_INVALID, "prefill length outside [0, window]");
  if (n > 0 && (!k || !v)) return fail(c, MOSHI_E_INVALID, "NULL prefill data");
  const size_t layer_elems = (size_t)n * c->D;
  const int64_t slot_stride = (int64_t)c->L * c->H * c->W * c->hd;
  for (int l = 0; l < c->L && n > 0; ++l) {
    for (int kv = 0; kv < 2; ++kv) {
      const char* src = (const char*)(kv == 0 ? k : v) + (size_t)l * layer_elems * c->esz;
      char* ring = (char*)(kv == 0 ? c->ring_k : c->ring_v) +
                   ((size_t)slot * slot_stride + (size_t)l * c->H * c->W * c->hd) * c->esz;
      CKD(c, hipMemcpyAsync(c->staging, src, layer_elems * c->esz, hipMemcpyHostToDevice, c->stream));
      CKD(c, launch_scatter_prefill(c->dtype, c->staging, ring, n, c->H, c->hd,
                                    (int64_t)c->W * c->hd, c->stream));
    }
  }
  CKD(c, hipStreamSynchronize(c->stream));
  c->slots.set_pos(slot, n);
  return MOSHI_OK;
}

int moshi_session_prefill_frames(moshi_ctx* c, int32_t slot, int32_t n, const int32_t* frames,
                                 int32_t* text_tokens, float* text_logits) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->slots.is_live(slot)) return fail(c, MOSHI_E_NOSESSION, "slot not live");
  if (n < 0) return fail(c, MOSHI_E_INVALID, "negative frame count");
  if (n == 0) return MOSHI_OK;
  if (!frames) return fail(c, MOSHI_E_INVALID, "frames is NULL");
  for (int64_t i = 0; i < (int64_t)n * c->NCH; ++i) {
    const int k = (int)(i % c->NCH);
    if (frames[i] < 0 || frames[i] > (k == 0 ? c->Vt : c->Va))
      return fail(c, MOSHI_E_INVALID, "frame code out of range");
  }
  if ((rc = ensure_prefill(c))) return rc;
  PrefillWs& p = c->pf;
  const int64_t p0 = c->slots.pos[slot];
  const int W = c->W;
  const bool mo = (c->c.flags & MOSHI_FLAG_MASK_OLDEST) != 0;
  std::vector<int64_t> pos(PF_COLS);
  std::vector<int> key0(PF_COLS), nkeys(PF_COLS), tok(PF_COLS);
  for (int j0 = 0; j0 < n; j0 += PF_COLS) {
    const int m = n - j0 < PF_COLS ? n - j0 : PF_COLS;
    const int64_t P0 = p0 + j0;
    const int64_t s0 = P0 - (W - 1) > 0 ? P0 - (W - 1) : 0;
    for (int j = 0; j < m; ++j) {
      const int64_t P = P0 + j;
      int64_t lo = P - W + 1;
      if (mo && P >= W - 1) lo = P - W + 2;
      if (lo < 0) lo = 0;
      pos[j] = P;
      key0[j] = (int)(lo - s0);
      nkeys[j] = (int)(P - lo + 1);
    }
    CKD(c, hipMemcpyAsync(p.frames, frames + (size_t)j0 * c->NCH, sizeof(int) * m * c->NCH,
                          hipMemcpyHostToDevice, c->stream));
    CKD(c, hipMemcpyAsync(p.pos, pos.data(), sizeof(int64_t) * m, hipMemcpyHostToDevice, c->stream));
    CKD(c, hipMemcpyAsync(p.key0, key0.data(), sizeof(int) * m, hipMemcpyHostToDevice, c->stream));
    CKD(c, hipMemcpyAsync(p.nkeys, nkeys.data(), sizeof(int) * m, hipMemcpyHostToDevice, c->stream));
    CKD(c, prefill_chunk(c, slot, P0, m));
    CKD(c, hipMemcpyAsync(tok.data(), p.tok, sizeof(int) * m, hipMemcpyDeviceToHost, c->stream));
    if (text_logits)
      CKD(c, hipMemcpyAsync(text_logits + (size_t)j0 * c->Vt, p.logits, sizeof(float) * m * c->Vt,
                            hipMemcpyDeviceToHost, c->stream));
    CKD(c, hipStreamSynchronize(c->stream));
    if (text_tokens)
      for (int j = 0; j < m; ++j) text_tokens[j0 + j] = tok[j];
  }
  c->meta_ev_pending = false;
  c->slots.set_pos(slot, p0 + n);
  return MOSHI_OK;
}

int moshi_session_read_kv(moshi_ctx* c, int32_t slot, void* k, void* v) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!c->slots.is_live(slot)) return fail(c, MOSHI_E_NOSESSION, "slot not live");
  if (!k || !v) return fail(c, MOSHI_E_INVALID, "NULL output");
  const size_t layer_elems = (size_t)c->W * c->D;
  const int64_t slot_stride = (int64_t)c->L * c->H * c->W * c->hd;
  for (int l = 0; l < c->L; ++l) {
    for (int kv = 0; kv < 2; ++kv) {
      char* dst = (char*)(kv == 0 ? k : v) + (size_t)l * layer_elems * c->esz;
      const char* ring = (const char*)(kv == 0 ? c->ring_k : c->ring_v) +
                         ((size_t)slot * slot_stride + (size_t)l * c->H * c->W * c->hd) * c->esz;
      CKD(c, launch_gather_ring(c->dtype, ring, c->staging, c->W, c->H, c->hd,
                                (int64_t)c->W * c->hd, c->stream));
      CKD(c, hipMemcpyAsync(dst, c->staging, layer_elems * c->esz, hipMemcpyDeviceToHost, c->stream));
      CKD(c, hipStreamSynchronize(c->stream));
    }
  }
  return MOSHI_OK;
}

int moshi_session_info(moshi_ctx* c, int32_t slot, int64_t* pos, int32_t* fill, int32_t* write_idx) {
  if (!c) return MOSHI_E_INVALID;
  if (!c->slots.is_live(slot)) return fail(c, MOSHI_E_NOSESSION, "slot not live");
  c->slots.info(slot, c->W, pos, fill, write_idx);
  return MOSHI_OK;
}

// Copies of the last step's outputs are ordered after every step enqueued on
// the context's stream.
int moshi_read_logits(moshi_ctx* c, float* text, float* audio) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (text)
    CKD(c, hipMemcpyAsync(text, c->text_logits, sizeof(float) * c->B * c->Vt,
                          hipMemcpyDeviceToHost, c->stream));
  if (audio)
    CKD(c, hipMemcpyAsync(audio, c->audio_logits, sizeof(float) * c->B * c->S * c->Va,
                          hipMemcpyDeviceToHost, c->stream));
  CKD(c, hipStreamSynchronize(c->stream));
  return MOSHI_OK;
}

int moshi_read_hidden(moshi_ctx* c, float* hidden) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!hidden) return fail(c, MOSHI_E_INVALID, "NULL argument");
  const size_t n = (size_t)c->B * c->D;
  if (c->dtype == DT_F32) {
    CKD(c, hipMemcpyAsync(hidden, c->hid, n * 4, hipMemcpyDeviceToHost, c->stream));
    CKD(c, hipStreamSynchronize(c->stream));
  } else {
    std::vector<uint16_t> tmp(n);
    CKD(c, hipMemcpyAsync(tmp.data(), c->hid, n * 2, hipMemcpyDeviceToHost, c->stream));
    CKD(c, hipStreamSynchronize(c->stream));
    for (size_t i = 0; i < n; ++i) {
      uint32_t u = (uint32_t)tmp[i] << 16;
      memcpy(&hidden[i], &u, 4);
    }
  }
  return MOSHI_OK;
}

int moshi_time_kernels(moshi_ctx* c, const int32_t* frames, int32_t n_steps, double* ms,
                       int64_t* launches, double* bytes, int32_t n_classes) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (n_steps < 0 || n_classes < 0) return fail(c, MOSHI_E_INVALID, "negative count");
  if ((rc = validate_frames(c, frames))) return rc;
  std::vector<double> acc_ms(KC_COUNT, 0.0), acc_b(KC_COUNT, 0.0);
  std::vector<int64_t> acc_n(KC_COUNT, 0);
  if (c->persistent || c->dep_multi) {
    rc = c->persistent ? time_step_phases(c, frames, n_steps, acc_ms, acc_b, acc_n)
                       : time_dep_multi(c, frames, n_steps, acc_ms, acc_b, acc_n);
    if (rc) return rc;
    for (int k = 0; k < n_classes && k < KC_COUNT; ++k) {
      if (ms) ms[k] = acc_ms[k];
      if (launches) launches[k] = acc_n[k];
      if (bytes) bytes[k] = acc_b[k];
    }
    return KC_COUNT;
  }
  c->timing = true;
  for (int it = 0; it < n_steps; ++it) {
    c->ev_used = 0;
    c->ev_class.clear();
    c->ev_bytes.clear();
    rc = run_step(c, frames, nullptr, nullptr, true);
    if (rc) break;
    for (size_t i = 0; i < c->ev_class.size(); ++i) {
      float t = 0.f;
      hipError_t e = hipEventElapsedTime(&t, c->ev[2 * i], c->ev[2 * i + 1]);
      if (e != hipSuccess) {
        rc = device_fail(c, e, "hipEventElapsedTime");
        break;
      }
      acc_ms[c->ev_class[i]] += t;
      acc_b[c->ev_class[i]] += c->ev_bytes[i];
      acc_n[c->ev_class[i]] += 1;
    }
    if (rc) break;
  }
  c->timing = false;
  if (rc) return rc;
  for (int k = 0; k < n_classes && k < KC_COUNT; ++k) {
    if (ms) ms[k] = acc_ms[k];
    if (launches) launches[k] = acc_n[k];
    if (bytes) bytes[k] = acc_b[k];
  }
  return KC_COUNT;
}

}  // extern "C"

int moshi_internal::ctx_device(const moshi_ctx* c) { return c ? c->device : -1; }

int moshi_internal::enqueue_static(moshi_ctx* c, const int32_t* d_frames, int32_t* d_text_token,
                                   int32_t* d_audio_codes) {
  int rc = check_ctx(c);
  if (rc) return rc;
  if (!d_frames) return fail(c, MOSHI_E_INVALID, "frames is NULL");
  if (!c->persistent)
    return fail(c, MOSHI_E_INVALID, "the allocation-free step needs the one-session step kernel");
  if (!c->d_step_static) return fail(c, MOSHI_E_INVALID, c->static_why);
  if ((rc = upload_forced(c, nullptr))) return rc;
  if ((rc = upload_meta(c))) return rc;
  int* tok = d_text_token ? d_text_token : c->tokens;
  int* codes = d_audio_codes ? d_audio_codes : c->codes;
  if (live_count(c) > 0) {
    uint32_t seq = 0;
    int parity = 0;
    moshi_internal::static_launch_ids(c->device, &seq, &parity);
    CKD(c, launch_step(c->dtype, c->hd, c->hdd, c->d_step_static, d_frames, tok, codes, parity, seq,
                       c->step_grid, c->step_lds, c->stream, nullptr));
    moshi_internal::static_launch_done(c->device);
  } else {
    // no live session: every output reads -1 (a fill kernel, no memset)
    CKD(c, launch_finish_outputs(tok, codes, c->d_live, c->B, c->S, c->S_run, c->stream));
  }
  c->slots.advance();
  return MOSHI_OK;
}
