// kernels.h -- argument blocks and launchers of the gfx950 kernels of the
// Moshi frame step (internal to libmoshi.so).
//
// Storage is the model dtype (bf16 or fp32) for weights, embeddings, the K/V
// rings and every vector that feeds a projection; all arithmetic is fp64
// (residual stream, norms, projections, RoPE, attention, SiLU, logits), so the
// rounding of each stored bf16 value is decided from an fp64 result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moshi {

enum Dtype { DT_F32 = 0, DT_BF16 = 1 };

// How a projection kernel builds its input vector.
enum Prologue {
  PRO_DIRECT = 0,  // X already stored in the model dtype [B][ldx]
  PRO_NORM = 1,    // X = round(x * rms_scale * gain): x fp64 [B][ldx] + per-tile sums of squares
  PRO_CAST = 2,    // X = round(x): x fp64 [B][ldx], no scaling
};

// What a projection kernel does with its 16-row output tile.
enum Epilogue {
  EPI_STORE = 0,   // out64[b][row] = y
  EPI_RESID = 1,   // resid[b][row] += y; per-tile sums of squares of the new residual
  EPI_QKV = 2,     // q rows -> RoPE -> q buffer; k,v rows -> (RoPE on k) -> ring cache
  EPI_SWIGLU = 3,  // tile rows interleave gate/up units: act[b][u] = round(silu(g) * u)
  EPI_ARGMAX = 4,  // logits (fp32 copy) + per-tile (max, index) partials of the fp64 values
};

struct ArgPart {
  double v;
  int i;
  int pad;
};

struct GemmArgs {
  const void* W;  // weight rows [.., K], model dtype
  int N;          // output rows (EPI_SWIGLU: number of units F; W has 2F rows: gate | up)
  int K;
  int B;          // columns = slot capacity
  // prologue
  const void* X;  // PRO_DIRECT: model dtype; PRO_NORM / PRO_CAST: fp64
  int ldx;
  const double* ssq;  // PRO_NORM: [n_ssq][B] partial sums of squares of x
  int n_ssq;
  const void* gain;  // PRO_NORM: [K] model dtype
  double eps;
  void* xn_out;      // PRO_NORM / PRO_CAST: if set, workgroup 0 stores the rounded input [B][K]
  // EPI_STORE
  double* out64;
  int ldo;
  // EPI_ARGMAX
  float* logits;     // [B][ldo]
  ArgPart* apart;    // [n_tiles][B]
  // EPI_RESID
  double* resid;
  int ldr;
  double* ssq_out;   // one session: [ceil(N/GEMV_SSQ_ROWS)]; more: [n_tiles][B]
  // EPI_SWIGLU
  void* act;
  int lda;
  // EPI_QKV
  double* q_out;
  int dq;                  // rows per part (q | k | v), = n_heads * head_dim
  int hd;                  // head dim
  const double* inv_freq;  // RoPE inverse frequencies [hd/2]; null = no RoPE
  const int64_t* pos;      // per-slot absolute position; null = use scalar_widx
  int scalar_widx;
  const int* live;         // per-slot liveness (ring writes only for live slots)
  void* ring_k;
  void* ring_v;
  int64_t slot_stride, layer_off, head_stride;  // ring strides, elements
  int cap;                                      // ring capacity
  // two to four sessions: VALU tiles instead of MFMA (the temporal projections)
  int vec_cols;
  // K split over workgroups (MFMA path; gemm_ksplit): ksplit > 1 segments of
  // the k-steps, each summed by its own workgroup into kpart [tile][4][ksplit]
  // [64 lanes] (f64x4); the last segment of a (tile, 16-column block group)
  // to finish (counter kcnt [tile][4], back to 0 after) adds the segments in
  // order and runs the epilogue
  int ksplit;
  double* kpart;
  int* kcnt;
};

struct AttnArgs {
  const double* q;  // [B][ldq], head h at h*HD
  int ldq;
  const void* ring_k;
  const void* ring_v;
  int64_t slot_stride, layer_off, head_stride;
  int cap;
  const int64_t* pos;  // per-slot position (temporal); null = all slots use scalar_nvalid
  int scalar_nvalid;
  int scalar_excl;     // with pos null: a key index masked out (-1: none)
  const int* live;
  int mask_oldest;
  int n_heads;
  int max_spans;  // key spans per (slot, head): one workgroup each (see n_spans)
  double* part;   // [B][H][max_spans][HD + 2]: (max, sum, p.V) of each span
  void* o_out;   // [B][ldo] model dtype
  int ldo;
};

constexpr int MAX_CHANNELS = 65;

struct EmbedArgs {
  const void* tables[MAX_CHANNELS];  // n_ch table pointers, each [rows][D]
  const int* frames;                 // [B][n_ch]
  const int* live;                   // [B]
  int n_ch;
  int D;
  int B;
  int rows_text, rows_audio;  // table rows (codes are clamped into range)
  int* bad_code;              // set to 1 when a live code was out of range
  double* x;                  // [B][D]
  double* ssq_out;            // [ceil(D/ssq_rows)][B]
  int ssq_rows;               // rows per sum-of-squares partial (2 or 16)
};

struct EntryArgs {
  const double* pre;  // [B][ldpre]; substep s block at s*D
  int ldpre;
  int s;
  const void* table;  // [rows][D]
  // previous token: either read (prev[b*prev_stride]) or, when prev_part is
  // set, reduced from the previous head's per-tile argmax partials and stored
  // to prev[b*prev_stride] by the workgroups of the first row tile
  int* prev;
  int prev_stride;
  const ArgPart* prev_part;  // [prev_tiles][B] or null
  int prev_tiles;
  int prev_n;  // rows of the previous head (index bound)
  // teacher forcing: where forced[b*forced_stride + forced_col] >= 0 it is
  // the previous token instead (and is what gets stored to prev); null = none
  const int* forced;
  int forced_stride, forced_col;
  int D;
  int B;
  double* y;        // [B][D]
  double* ssq_out;  // [ceil(D/ssq_rows)][B]
  int ssq_rows;     // rows per sum-of-squares partial (2 or 16)
};

// Per-slot sampling parameters (moshi_session_set_sampling).
struct SampleParams {
  double temperature[2];  // [0] text, [1] audio codes; <= 0: greedy (the argmax stands)
  int top_k[2];           // <= 0 or >= the vocabulary: every token is a candidate
  uint64_t seed;          // the session's seed (child streams per head)
};

// One temperature + top-k draw per live column b (see sample_kernel).
struct SampleArgs {
  const float* logits;  // column b at logits + b * ld, n values
  int ld, n;
  const SampleParams* params;  // [B]
  int which;                   // 0 text, 1 audio
  int stream;                  // the draw's stream: 0 text, 1 + s depformer substep s
  const int64_t* pos;          // [B] positions; the draw uses pos[b] + pos_off
  int pos_off;
  const int* live;             // [B]
  const int* forced;           // [B][forced_stride]; a forced column keeps its token
  int forced_stride, forced_col;
  int* out;                    // out[b * out_stride]: the drawn token
  int out_stride;
  int B;
};
// Attention of a multi-frame prefill chunk (prefill_attn_kernel): query
// column b attends rows [key0[b], key0[b] + nkeys[b]) of a window buffer whose
// head h starts at a.ring_k / a.ring_v + h * a.head_stride; q [m][a.ldq],
// outputs a.o_out [m][a.ldo], span partials a.part [m][H][max_spans][HD + 2].
struct PrefillAttnArgs {
  AttnArgs a;
  const int* key0;
  const int* nkeys;
  int m;
};
hipError_t launch_prefill_attn(int dtype, int hd, const PrefillAttnArgs& p, hipStream_t st);
// Rows [i0, i1) of a window buffer (head stride win_head_stride) <-> one
// layer of a session's ring (head stride ring_head_stride; row i is ring
// slot (s0 + i) mod W); to_ring picks the direction.
hipError_t launch_window_copy(int dtype, void* win, void* ring, int i0, int i1, int64_t s0, int W,
                              int H, int hd, int64_t win_head_stride, int64_t ring_head_stride,
                              int to_ring, hipStream_t st);

constexpr int SAMPLE_THREADS = 1024;
constexpr int SAMPLE_MAX_PER_THREAD = 32;  // vocabularies up to 32768

// Attention spans hold about ATTN_CHUNK keys or more; the window is at most
// ATTN_CHUNK * ATTN_MAX_CHUNKS keys.
constexpr int ATTN_CHUNK = 64;
constexpr int ATTN_MAX_CHUNKS = 512;

// Argument block of the persistent one-session step kernel (step.hip), kept in
// device memory. The GemmArgs / AttnArgs are templates: the kernel fills in
// the per-layer weights, gains and ring offsets from the pointer tables.
struct StepArgs {
  // temporal
  EmbedArgs emb;  // frames come with each launch
  GemmArgs t_qkv, t_o, t_gu, t_dn, t_head;
  AttnArgs t_attn;
  int L, H;
  int64_t t_layer_elems;   // ring elements per layer of one slot (H * W * hd)
  // depformer
  GemmArgs d_in, d_qkv, d_o, d_gu, d_dn, d_head;
  AttnArgs d_attn;
  int S, Ld, Hd, Dd, Vt, Va;
  int64_t d_layer_elems;       // depformer K/V elements per layer (Hd * S * hdd)
  const double* pre;           // [S * Dd] input projections of the hidden state
  double* y;                   // depformer residual [Dd]
  double* ssq_d;               // its per-tile sums of squares
  ArgPart* apart;              // argmax partials of the last head
  float* audio_logits;         // [S][Va]
  int S_run;                   // substeps run per frame (<= S)
  int dep_final_norm;          // heads read RMSNorm(y) * gain (d_head.gain) instead of y
  const int* forced;           // [1 + S] forced text / codes of slot 0 (-1: not forced)
  int spin_limit;              // polls before a grid-barrier wait gives up
  int ll_spin_limit;           // polls before a flagged-vector wait gives up
  // bookkeeping
  int64_t* pos;                // slot 0 position (advanced at the end)
  const int* live;
  // weight pointers, one table (copied to LDS at tab_lds bytes into the
  // dynamic LDS when the kernel starts), with these sections:
  //   o_tw: [L][6] attn_norm, qkv, o, mlp_norm, gate_up, down
  //   o_dw: [S * Ld][4] qkv, o, gate_up, down of (substep, layer)
  //   o_dn: [Ld][2] depformer attn_norm, mlp_norm
  //   o_de: [S] previous-token tables;  o_dh: [S] heads
  const void* const* tab;
  int n_tab, tab_lds;
  // depformer projections: the workgroup's weight slice is staged in the
  // dynamic LDS at wbuf_lds bytes (see staged_slice_bytes)
  int wbuf_lds;
  int o_tw, o_dw, o_dn, o_de, o_dh;
  unsigned* bar;               // 2 sets of STEP_BAR_WORDS barrier counters
  int* abort;                  // set when a barrier or flag wait times out
  // flagged vectors the depformer operations hand on (step.hip); zeroed at
  // creation, step_ll_words() words of 8 bytes
  uint64_t* ll;
};
// Argument block of the multi-session depformer kernel (step.hip; capacity
// 2..64): the per-operation argument blocks of substep 0, layer 0 (for B
// columns) as templates, completed per (substep, layer) from the pointer
// table, whose sections are as in StepArgs: o_dw [S * Ld][4] qkv, o, gate_up,
// down; o_dn [Ld][2] attn_norm, mlp_norm; o_de [S] previous-token tables;
// o_dh [S] heads.
struct DepMultiArgs {
  GemmArgs d_in, d_qkv, d_o, d_gu, d_dn, d_head;
  AttnArgs d_attn;
  EntryArgs entry;
  int S, S_run, Ld, Dd, Va, B, nch;
  int64_t d_layer_elems;
  int dep_final_norm;
  int ref_excl_at;      // substep whose depformer attention masks entry 0 (-1: none)
  const int* forced;    // [B][nch]
  int* tokens;          // [B] the text tokens (substep 0's input)
  int* codes;           // [B][S]
  const int* live;
  ArgPart* apart;
  const void* const* tab;
  int n_tab, o_dw, o_dn, o_de, o_dh;
  unsigned* bar;        // 2 sets of STEP_BAR_WORDS barrier counters
  int* abort;
  int spin_limit;
};
bool dep_multi_supported(int dtype, int hdd);
// Workgroups of the multi-session depformer kernel resident at once (one per
// CU), 0 if it cannot run.
int dep_multi_grid(int dtype, int hdd, int B, size_t lds_bytes);
// One cooperative launch of the depformer of every live slot (B columns).
// `trace`, if set, receives the wall clock (100 MHz) when the grid has
// started, after every grid barrier, and when workgroup 0 ends, as seen by
// workgroup 0: one entry per phase boundary (the phases: the input
// projections; per substep run its entry, per layer the q/k/v norm, q/k/v,
// attention, output projection, gate/up norm, gate/up, down; its head's
// norm and head; then the last code).
hipError_t launch_dep_multi(int dtype, int hdd, int B, const DepMultiArgs* dP, int parity, int nwg,
                            size_t lds_bytes, hipStream_t st, uint64_t* trace = nullptr);

// One-session projections run 8 waves per workgroup; each wave owns 2 rows
// of a 16-row tile, and the residual epilogue writes one sum-of-squares
// partial per wave (every 2 rows). With two or more sessions the partials are
// per 16-row tile.
constexpr int GEMV_KW = 8;
constexpr int GEMV_SSQ_ROWS = 16 / GEMV_KW;
constexpr int STEP_THREADS = 512;
// Default bounds of the step kernel's waits (polls; one memory round trip,
// ~0.5 us, each): a wait that runs out raises the abort flag.
constexpr int STEP_SPIN_LIMIT = 1 << 21;
constexpr int STEP_LL_SPIN_LIMIT = 1 << 20;
constexpr int STEP_BAR_WORDS = 17 * 1024;  // one barrier counter set (17 pages of 4 KB)

// Whether step.hip has an instantiation for (dtype, temporal head dim,
// depformer head dim).
bool step_supported(int dtype, int hd, int hdd);
// Workgroups the step kernel can keep resident on the device (0 = none).
int step_max_grid(int dtype, int hd, int hdd, size_t lds_bytes);
// One cooperative launch of the whole step for slot 0. `parity` alternates
// between launches (it picks the barrier counter set). `trace`, if set,
// receives the wall clock (100 MHz) at the start, after every grid barrier
// and at the end, as seen by workgroup 0 (STEP_TRACE_MAX entries at most).
// `seq` is the launch's sequence number (nonzero, different from the previous
// launch's): the flag of the vectors it writes.
hipError_t launch_step(int dtype, int hd, int hdd, const StepArgs* dP, const int* frames,
                       int* text_out, int* codes_out, int parity, uint32_t seq, int nwg,
                       size_t lds_bytes, hipStream_t st, uint64_t* trace);
// Words of the flagged vectors of the step kernel (step.hip's layout): per
// depformer substep and layer 11 Dd + Fd, then per substep 2 Dd + 32
// ceil(Va / 16); then per temporal layer, head and key span 2 (hd + 2), then
// per temporal layer D.
inline int64_t step_ll_words(int S, int Ld, int Dd, int Fd, int Va, int L, int H, int hd, int nsp,
                             int D) {
  return (int64_t)S * Ld * (11LL * Dd + Fd) + (int64_t)S * (2LL * Dd + 32LL * ((Va + 15) / 16)) +
         (int64_t)L * H * nsp * 2LL * (hd + 2) + (int64_t)L * D;
}
// Register copies of the depformer weight slices in the step kernel: at most
// I items (row pairs) per wave and C column passes (ceil(K / vec / 64)) for
// the q/k/v, output, gate/up, down and head projections.
constexpr int LLR_QKV_I = 1, LLR_QKV_C = 2;
constexpr int LLR_O_I = 1, LLR_O_C = 2;
constexpr int LLR_GU_I = 2, LLR_GU_C = 2;
constexpr int LLR_DN_I = 1, LLR_DN_C = 6;
constexpr int LLR_HD_I = 1, LLR_HD_C = 2;
// Items per wave of a one-session staged projection on nwg workgroups (the
// split of gemv_stage).
inline int staged_items_per_wave(int epi, int N, int nwg) {
  if (epi == EPI_QKV || epi == EPI_ARGMAX) return ((N + 15) / 16 + nwg - 1) / nwg;
  const int64_t pairs = epi == EPI_SWIGLU ? N : (N + 1) / 2;
  return (int)(((pairs + nwg - 1) / nwg + GEMV_KW - 1) / GEMV_KW);
}
constexpr int STEP_TRACE_MAX = 4096;
// LDS bytes of one workgroup's staged weight slice in the step kernel: the
// most row pairs one of its GEMV_KW waves takes (q/k/v and argmax: one per
// 16-row tile of the workgroup; others: row pairs spread evenly over nwg
// workgroups, then over the waves) x column passes (ceil(K / vec / 64)) x
// 16 KB (2 rows x GEMV_KW waves x 64 lanes x 16 bytes). vec = elements per
// 16 bytes.
inline int64_t staged_slice_bytes(int vec, int epi, int N, int K, int nwg) {
  int64_t items;
  if (epi == EPI_QKV || epi == EPI_ARGMAX) {
    items = ((N + 15) / 16 + nwg - 1) / nwg;
  } else {
    const int64_t pairs = epi == EPI_SWIGLU ? N : (N + 1) / 2;
    items = ((pairs + nwg - 1) / nwg + GEMV_KW - 1) / GEMV_KW;
  }
  return items * ((K / vec + 63) / 64) * 16 * 1024;
}

int gemm_tiles(int epi, int N);  // row tiles of a projection
// Workgroups launched for a one-session projection (the number of CUs).
void set_gemv_grid(int n);
// Waves per workgroup for a projection of `tiles` row tiles with K inputs
// and B sessions: one session 8; more: 16 (up to 32 sessions) or 12 / 4
// (33..64, at most / more than 512 tiles) for inputs of 4096 or wider, 8 / 4
// for narrower ones (up to 32 / 33..64 sessions).
int gemm_kw(int dtype, int B, int K, int tiles);
// K segments of an MFMA projection (1: none); see GemmArgs::ksplit.
int gemm_ksplit(int B, int K, int tiles);
constexpr int GEMM_KSPLIT_MAX = 4;
// kw from gemm_kw (B > 1: 16 or 8 up to 32 sessions, 12 or 4 above). With
// B > 1 and PRO_NORM / PRO_CAST, xn_out must be a [B][K] buffer: the rounded
// input vectors are written there first.
hipError_t launch_gemm(int dtype, int kw, int pro, int epi, const GemmArgs& a, hipStream_t st);
hipError_t launch_attn(int dtype, int hd, const AttnArgs& a, int B, hipStream_t st);
// Depformer attention over a.scalar_nvalid <= DEP_MAX_KEYS entries, one
// workgroup per slot, every head.
hipError_t launch_dep_attn(int dtype, int hd, const AttnArgs& a, int B, hipStream_t st);
constexpr int DEP_MAX_KEYS_HOST = 16;  // equals DEP_MAX_KEYS in dev.h
// Merges the per-chunk partials of every (slot, head) with more than one chunk.
hipError_t launch_attn_combine(int dtype, int hd, const AttnArgs& a, int B, hipStream_t st);
// tok[b*stride] = argmax over the per-tile partials of column b (lowest index
// on ties), or forced[b*forced_stride + forced_col] where that is >= 0
// (forced may be null).
hipError_t launch_argmax_reduce(const ArgPart* part, int n_tiles, int n_rows, int B, int* tok,
                                int stride, const int* forced, int forced_stride, int forced_col,
                                hipStream_t st);
// Temperature + top-k draws of every live column that samples (one workgroup
// of SAMPLE_THREADS per column; greedy and forced columns keep their token).
hipError_t launch_sample(const SampleArgs& a, hipStream_t st);
// Outputs of free slots become -1, and codes of substeps past s_run too.
hipError_t launch_finish_outputs(int* tokens, int* codes, const int* live, int B, int S, int s_run,
                                 hipStream_t st);
hipError_t launch_embed(int dtype, const EmbedArgs& a, hipStream_t st);
hipError_t launch_entry(int dtype, const EntryArgs& a, hipStream_t st);
hipError_t launch_advance(int64_t* pos, const int* live, int B, hipStream_t st);
hipError_t launch_gather_ring(int dtype, const void* ring, void* dst, int n, int n_heads, int hd,
                              int64_t head_stride, hipStream_t st);
hipError_t launch_scatter_prefill(int dtype, const void* src, void* ring, int n, int n_heads,
                                  int hd, int64_t head_stride, hipStream_t st);

}  // namespace moshi
