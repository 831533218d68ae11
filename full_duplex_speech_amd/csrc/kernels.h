// kernels.h -- argument blocks and launchers of the gfx950 kernels of the
// Moshi frame step (internal to libmoshi.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moshi {

enum Dtype { DT_F32 = 0, DT_BF16 = 1 };

// How a projection kernel builds its input vector (the MFMA B operand).
enum Prologue {
  PRO_DIRECT = 0,  // X already in the model dtype [B][ldx]
  PRO_NORM = 1,    // X = round(x * rms_scale * gain): x fp32 [B][ldx] + per-tile sums of squares
  PRO_CAST = 2,    // X = round(x): x fp32 [B][ldx], no scaling
};

// What a projection kernel does with its 16-row output tile.
enum Epilogue {
  EPI_STORE = 0,   // out[b][row] = y (fp32)
  EPI_RESID = 1,   // resid[b][row] += y; per-tile sums of squares of the new residual
  EPI_QKV = 2,     // q rows -> RoPE -> q buffer; k,v rows -> (RoPE on k) -> ring cache
  EPI_SWIGLU = 3,  // tile rows interleave gate/up units: act[b][u] = round(silu(g) * u)
  EPI_ARGMAX = 4,  // logits out + per-tile (max, index); the last workgroup picks the token
};

struct ArgPart {
  float v;
  int i;
};

struct GemmArgs {
  const void* W;  // weight rows [.., K], model dtype
  int N;          // output rows (EPI_SWIGLU: number of units F; W has 2F rows: gate | up)
  int K;
  int B;          // columns = slot capacity
  // prologue
  const void* X;  // PRO_DIRECT: model dtype; PRO_NORM / PRO_CAST: fp32
  int ldx;
  const float* ssq;  // PRO_NORM: [n_ssq][B] partial sums of squares of x
  int n_ssq;
  const void* gain;  // PRO_NORM: [K] model dtype
  float eps;
  void* xn_out;      // PRO_NORM / PRO_CAST: if set, workgroup 0 stores the rounded input [B][K]
  // EPI_STORE / EPI_ARGMAX
  float* out;
  int ldo;
  // EPI_RESID
  float* resid;
  int ldr;
  float* ssq_out;  // [n_tiles][B]
  // EPI_SWIGLU
  void* act;
  int lda;
  // EPI_QKV
  float* q_out;
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
  // EPI_ARGMAX
  ArgPart* apart;      // [n_tiles][B]
  unsigned* ticket;    // zero on entry, reset to zero by the last workgroup
  int* tok_out;
  int tok_stride;
};

struct AttnArgs {
  const float* q;   // [B][ldq], head h at h*HD
  int ldq;
  const void* ring_k;
  const void* ring_v;
  int64_t slot_stride, layer_off, head_stride;
  int cap;
  const int64_t* pos;  // per-slot position (temporal); null = all slots use scalar_nvalid
  int scalar_nvalid;
  const int* live;
  int mask_oldest;
  int n_heads;
  int max_chunks;
  float* part;        // [B][H][max_chunks][HD + 2]
  unsigned* ticket;   // [B][H]
  void* o_out;        // [B][ldo] model dtype
  int ldo;
};

struct EmbedArgs {
  const void* const* tables;  // device array of n_ch table pointers, each [rows][D]
  const int* frames;          // [B][n_ch]
  const int* live;            // [B]
  int n_ch;
  int D;
  int B;
  int rows_text, rows_audio;  // table rows (codes are clamped into range)
  int* bad_code;              // set to 1 when a live code was out of range
  float* x;        // [B][D]
  float* ssq_out;  // [ceil(D/16)][B]
};

struct EntryArgs {
  const float* pre;  // [B][ldpre]; substep s block at s*D
  int ldpre;
  int s;
  const void* table;  // [rows][D]
  const int* prev;    // token of column b at prev[b*prev_stride]
  int prev_stride;
  int D;
  int B;
  float* y;        // [B][D]
  float* ssq_out;  // [ceil(D/16)][B]
};

// Keys per attention workgroup.
constexpr int ATTN_CHUNK = 64;

int gemm_nb(int B);            // 16-column tiles for capacity B (1, 2 or 4)
int gemm_tiles(int epi, int N);  // grid size of a projection
// kw = waves per workgroup (K split), 4 or 8.
hipError_t launch_gemm(int dtype, int kw, int pro, int epi, const GemmArgs& a, hipStream_t st);
hipError_t launch_attn(int dtype, int hd, const AttnArgs& a, int B, hipStream_t st);
hipError_t launch_embed(int dtype, const EmbedArgs& a, hipStream_t st);
hipError_t launch_entry(int dtype, const EntryArgs& a, hipStream_t st);
hipError_t launch_advance(int64_t* pos, const int* live, int B, hipStream_t st);
hipError_t launch_scatter_prefill(int dtype, const void* src, void* ring, int n, int n_heads,
                                  int hd, int64_t head_stride, hipStream_t st);

}  // namespace moshi
