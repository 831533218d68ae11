// step.hip -- the whole frame step of one session as ONE persistent kernel.
//
// Model and numerics are those of kernels.hip (same device functions from
// dev.h, so results are bit-identical to the per-operation kernels): the
// summed embedding, the temporal layers (q/k/v + RoPE + ring write, windowed
// attention, output projection, SwiGLU MLP), the text head and its greedy
// token, the depformer input projections and the 16 substeps with their
// heads ("vLLM-Omni recipe: PersonaPlex", "Architecture"; mobius PR #368,
// "P2 - Moshi LM").
//
// Why one kernel: at one session every operation is a GEMV of a few to a few
// hundred MB, and a dependent kernel launch costs about 4-5 us of ramp-up and
// drain on MI355X; the depformer alone is ~500 dependent operations. Here one
// workgroup runs per CU for the whole step and the operations are separated
// by grid barriers instead of launches.
//
// Grid barrier: two levels, because 256 workgroups incrementing one counter
// serialise at the memory side. Each workgroup counts into the counter of its
// XCD; the last arrival of an XCD increments the global counter; the last of
// those writes a release word that everyone polls. Cross-workgroup data use agent-scope relaxed
// atomics (sc1 loads and stores, see dev.h), each thread waits for its own
// stores (s_waitcnt 0) before the workgroup arrives, so no cache write-back
// or invalidate is needed. Every wait is bounded: after SPIN_LIMIT polls a
// workgroup raises the abort flag, and every waiter that sees it leaves, so
// the grid always drains; the host then reports a device error.
// The launch is cooperative (every workgroup resident or the launch fails).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dev.h"
#include "kernels.h"

namespace moshi {
namespace {

constexpr int NT = STEP_THREADS;
constexpr int KW = NT / 64;
static_assert(KW == GEMV_KW, "the step kernel's projections use the one-session layout");
// Weight groups per lane and row in flight in the temporal projections (long
// streams). The depformer projections instead stage their whole weight slice
// in LDS during the barrier before them (gemv_stage / gemv_staged).
constexpr int GU = 4;
constexpr int SPIN_LIMIT = 1 << 21;  // polls (one memory round trip each, ~0.5 us) before giving up

// Barrier words of one set (32-bit words): one 4 KB page per XCD holding its
// arrival counter, its registration count and its release word (each on a
// 128-byte line of its own), then a page with the grid-wide counters. The
// pages keep different XCDs' counters, and the release words every
// workgroup polls, in different memory channels: 256 workgroups polling one
// word would queue every other access to that word's channel behind them.
constexpr int MAX_XCC = 16;
constexpr int BW_PAGE = 1024;
constexpr int BW_LOCAL = 0, BW_REG = 32, BW_RELEASE = 64;  // within an XCD's page
constexpr int BW_FLAT = MAX_XCC * BW_PAGE, BW_GLOBAL = BW_FLAT + 32;
static_assert(STEP_BAR_WORDS >= (MAX_XCC + 1) * BW_PAGE, "barrier words");

__device__ __forceinline__ unsigned xcc_id() {
  // hardware register XCC_ID (id 20), bits [3:0]
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (MAX_XCC - 1);
}

struct Grid {
  unsigned* set;
  int* abort;
  uint64_t* trace;  // optional: barrier exit times of workgroup 0
  unsigned idx;    // barriers passed
  unsigned xcc;    // this workgroup's XCD
  unsigned xcc_n;  // workgroups on it
  unsigned n_xcc;  // XCDs with at least one workgroup
};

// A value every lane holds equally (read from LDS), as a wave-uniform (scalar)
// value.
template <typename X>
__device__ __forceinline__ X uni(const X& v) {
  static_assert(sizeof(X) % 4 == 0, "word-sized fields");
  struct Words {
    uint32_t w[sizeof(X) / 4];
  };
  const Words in = __builtin_bit_cast(Words, v);
  Words out;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(X) / 4); ++i) out.w[i] = __builtin_amdgcn_readfirstlane(in.w[i]);
  return __builtin_bit_cast(X, out);
}

// Make this thread's stores visible at agent scope before arriving.
__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Thread 0 polls `ctr` until it reaches `target` (wrap-safe) or the abort
// flag rises. Returns nonzero when the grid must leave.
__device__ __forceinline__ int poll_until(unsigned* ctr, unsigned target, int* abort) {
  int spins = 0;
  while ((int)(__hip_atomic_load((MOSHI_GLB unsigned*)ctr, MOSHI_RLX, MOSHI_AGT) - target) < 0) {
    if (++spins > SPIN_LIMIT) {
      __hip_atomic_store((MOSHI_GLB int*)abort, 1, MOSHI_RLX, MOSHI_AGT);
      return 1;
    }
    if ((spins & 15) == 0 && __hip_atomic_load((MOSHI_GLB int*)abort, MOSHI_RLX, MOSHI_AGT)) return 1;
  }
  return 0;
}

// Grid barrier in two halves, so that loads can be issued in between:
// grid_arrive (after drain_stores() and a workgroup barrier) counts this
// workgroup in; grid_wait completes the count and waits. Loads issued between
// the two are younger than the arrival atomic, so reading its result does not
// wait for them; the polls do, but those loads (a weight prefetch) land well
// before the grid does. Every thread of every workgroup calls both; true =
// abort.
__device__ __forceinline__ unsigned grid_arrive(Grid& g) {
  g.idx += 1;
  unsigned old = 0;
  if (threadIdx.x == 0)
    old = __hip_atomic_fetch_add((MOSHI_GLB unsigned*)g.set + g.xcc * BW_PAGE + BW_LOCAL, 1u,
                                 MOSHI_RLX, MOSHI_AGT);
  return old;
}

__device__ __forceinline__ bool grid_wait(Grid& g, unsigned old) {
  __shared__ int s_leave;
  if (threadIdx.x == 0) {
    // the last arrival of the last XCD releases everyone through the release
    // words, one per XCD (polling the counters themselves slows their
    // increments)
    if (old + 1 == g.idx * g.xcc_n) {
      const unsigned og =
          __hip_atomic_fetch_add((MOSHI_GLB unsigned*)g.set + BW_GLOBAL, 1u, MOSHI_RLX, MOSHI_AGT);
      if (og + 1 == g.idx * g.n_xcc)
        for (int x = 0; x < MAX_XCC; ++x)
          __hip_atomic_store((MOSHI_GLB unsigned*)g.set + x * BW_PAGE + BW_RELEASE, g.idx, MOSHI_RLX,
                             MOSHI_AGT);
    }
    s_leave = poll_until(g.set + g.xcc * BW_PAGE + BW_RELEASE, g.idx, g.abort);
    if (g.trace != nullptr && blockIdx.x == 0) *(MOSHI_GLB uint64_t*)(g.trace + g.idx) = wall_clock64();
  }
  __syncthreads();
  return s_leave != 0;
}

__device__ __forceinline__ bool grid_sync(Grid& g) {
  drain_stores();
  __syncthreads();
  const unsigned old = grid_arrive(g);
  return grid_wait(g, old);
}

// Start of a launch: clear the other counter set (used by the next launch;
// the previous launch, which used it, has finished), count the workgroups of
// every XCD, and wait for all of them (flat barrier).
__device__ __forceinline__ bool grid_init(Grid& g, unsigned* bar, unsigned* attn_ctr, int n_heads,
                                          int parity, int* abort, uint64_t* trace) {
  __shared__ int s_leave;
  __shared__ unsigned s_cnt[MAX_XCC];
  g.set = bar + parity * STEP_BAR_WORDS;
  g.abort = abort;
  g.trace = trace;
  g.idx = 0;
  g.xcc = xcc_id();
  unsigned* other = bar + (parity ^ 1) * STEP_BAR_WORDS;
  if (blockIdx.x == 0 && threadIdx.x < MAX_XCC) {
    unsigned* page = other + threadIdx.x * BW_PAGE;
    __hip_atomic_store((MOSHI_GLB unsigned*)page + BW_LOCAL, 0u, MOSHI_RLX, MOSHI_AGT);
    __hip_atomic_store((MOSHI_GLB unsigned*)page + BW_REG, 0u, MOSHI_RLX, MOSHI_AGT);
    __hip_atomic_store((MOSHI_GLB unsigned*)page + BW_RELEASE, 0u, MOSHI_RLX, MOSHI_AGT);
    if (threadIdx.x == 0) {
      __hip_atomic_store((MOSHI_GLB unsigned*)other + BW_FLAT, 0u, MOSHI_RLX, MOSHI_AGT);
      __hip_atomic_store((MOSHI_GLB unsigned*)other + BW_GLOBAL, 0u, MOSHI_RLX, MOSHI_AGT);
    }
  }
  if (blockIdx.x == 0)
    for (int h = threadIdx.x; h < n_heads; h += NT)
      __hip_atomic_store((MOSHI_GLB unsigned*)attn_ctr + ((parity ^ 1) * n_heads + h) * 16, 0u,
                         MOSHI_RLX, MOSHI_AGT);
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add((MOSHI_GLB unsigned*)g.set + g.xcc * BW_PAGE + BW_REG, 1u, MOSHI_RLX,
                           MOSHI_AGT);
    __hip_atomic_fetch_add((MOSHI_GLB unsigned*)g.set + BW_FLAT, 1u, MOSHI_RLX, MOSHI_AGT);
    s_leave = poll_until(g.set + BW_FLAT, gridDim.x, abort);
    if (trace != nullptr && blockIdx.x == 0) *(MOSHI_GLB uint64_t*)trace = wall_clock64();
  }
  __syncthreads();
  if (s_leave) return true;
  if (threadIdx.x < MAX_XCC)
    s_cnt[threadIdx.x] = __hip_atomic_load((MOSHI_GLB unsigned*)g.set + threadIdx.x * BW_PAGE + BW_REG,
                                           MOSHI_RLX, MOSHI_AGT);
  __syncthreads();
  g.n_xcc = 0;
  for (int i = 0; i < MAX_XCC; ++i) g.n_xcc += s_cnt[i] ? 1u : 0u;
  g.xcc_n = s_cnt[g.xcc];
  __syncthreads();
  return false;
}

// Sum of squares of GEMV_SSQ_ROWS consecutive rows held by consecutive lanes;
// the first lane of each group stores it as the group's partial (the layout
// the one-session residual epilogue writes).
template <bool C>
__device__ __forceinline__ void store_tile_ssq(double v, int row, int n_rows, double* ssq_out) {
  const double ss = group_reduce<GEMV_SSQ_ROWS>(v * v);
  if (row % GEMV_SSQ_ROWS == 0 && row < n_rows) st_f64<C>(ssq_out + row / GEMV_SSQ_ROWS, ss);
}

// x = E_text[c0] + sum_k E_audio_k[c_k] for slot 0; NT rows per item.
// A code outside its table is clamped into range and flagged for the host.
// `a` is the LDS copy; its fields are read one by one (the table array is
// indexed by channel and must not be copied into registers).
template <typename T>
__device__ __forceinline__ void embed_phase(const EmbedArgs& a, const int* frames, int wg,
                                            int nwg) {
  const int D = uni(a.D), n_ch = uni(a.n_ch);
  const int rows_text = uni(a.rows_text), rows_audio = uni(a.rows_audio);
  double* x = uni(a.x);
  double* ssq_out = uni(a.ssq_out);
  int* bad_code = uni(a.bad_code);
  for (int item = wg; item * NT < D; item += nwg) {
    const int row = item * NT + tid();
    double acc = 0.0;
    if (row < D) {
      for (int c0 = 0; c0 < n_ch; c0 += 8) {
        double v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = c0 + j;
          v[j] = 0.0;
          if (c < n_ch) {
            int code = ldg(frames + c);
            const int rows = (c == 0) ? rows_text : rows_audio;
            if (code < 0 || code >= rows) {
              if (row == 0) atomicOr(bad_code, 1);
              code = code < 0 ? 0 : rows - 1;
            }
            const T* table = (const T*)uni(a.tables[c]);
            v[j] = to_d(ldg(table + (size_t)code * D + row));
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (c0 + j < n_ch) acc += v[j];
      }
      st_f64<true>(x + row, acc);
    }
    store_tile_ssq<true>(acc, row, D, ssq_out);
  }
}

// Depformer substep entry for slot 0: the previous head's token (the text
// token at s = 0), stored as an output by workgroup 0, then
// y = W_in[s] hidden + E_s[token].
template <typename T, int HD, int HDD>
__global__ __launch_bounds__(NT) void step_kernel(const StepArgs* P,
                                                  const int* __restrict__ frames, int* text_out,
                                                  int* codes_out, int parity, uint64_t* trace) {
  static_assert(HDD % 16 == 0, "a depformer q/k/v tile holds rows of one head");
  constexpr int DEP_TILES_PER_HEAD = 3 * HDD / 16;  // q, k and v tiles
  extern __shared__ __align__(16) unsigned char s_dyn[];  // GEMV input or attention scratch
  T* xs = (T*)s_dyn;
  double* s_o = (double*)s_dyn;
  // The argument block and the weight pointers live in LDS for the whole
  // launch: every operation reads its arguments there (as wave-uniform
  // values) instead of from global memory after each barrier.
  __shared__ __align__(16) StepArgs sA;
  {
    const uint32_t* src = (const uint32_t*)P;
    uint32_t* dst = (uint32_t*)&sA;
    for (int i = tid(); i < (int)(sizeof(StepArgs) / 4); i += NT) dst[i] = ldg(src + i);
  }
  __syncthreads();
  const StepArgs& A = sA;
  const void** s_tab = (const void**)(s_dyn + uni(A.tab_lds));
  {
    const void* const* tab = uni(A.tab);
    const int n_tab = uni(A.n_tab);
    for (int i = tid(); i < n_tab; i += NT) s_tab[i] = ldg(tab + i);
  }
  __syncthreads();
  auto tab = [&](int i) { return uni(s_tab[i]); };
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int L = uni(A.L), H = uni(A.H), S = uni(A.S), Ld = uni(A.Ld), Hd = uni(A.Hd);
  const int Va = uni(A.Va), Dd = uni(A.Dd);
  const int o_tw = uni(A.o_tw), o_dw = uni(A.o_dw), o_dn = uni(A.o_dn), o_de = uni(A.o_de),
            o_dh = uni(A.o_dh);
  const int64_t t_lel = uni(A.t_layer_elems), d_lel = uni(A.d_layer_elems);
  Grid g;
  // attention tickets of this launch: temporal heads, then depformer heads
  if (grid_init(g, uni(A.bar), uni(A.attn_ctr), H + Hd, parity, uni(A.abort), trace)) return;
  unsigned* const tickets = uni(A.attn_ctr) + (size_t)parity * (H + Hd) * 16;
  // first weight batch of the next projection, requested before each barrier
  u32x4 pf[GU][16 / KW];
  unsigned char* const wbuf = s_dyn + uni(A.wbuf_lds);
#define PREFETCH_SYNC_G(EPI_, args_, GU_, PF_)             \
  do {                                                     \
    const GemmArgs na_ = (args_);                          \
    drain_stores();                                        \
    __syncthreads();                                       \
    const unsigned old_ = grid_arrive(g);                  \
    gemv_prefetch<T, KW, EPI_, GU_>(na_, wg, PF_);         \
    if (grid_wait(g, old_)) return;                        \
  } while (0)
#define PREFETCH_SYNC(EPI_, args_) PREFETCH_SYNC_G(EPI_, args_, GU, pf)
#define GEMV(PRO_, EPI_, args_) \
  gemv_core<T, KW, PRO_, EPI_, true, GU, true>((args_), wg, nwg, xs, pf, s_rope)
  // depformer: the next projection's weight slice goes to LDS during the barrier
#define STAGE_SYNC(EPI_, args_)                            \
  do {                                                     \
    const GemmArgs na_ = (args_);                          \
    drain_stores();                                        \
    __syncthreads();                                       \
    const unsigned old_ = grid_arrive(g);                  \
    gemv_stage<T, KW, EPI_>(na_, wg, nwg, wbuf);           \
    if (grid_wait(g, old_)) return;                        \
  } while (0)
#define GEMV_S(PRO_, EPI_, args_) gemv_staged<T, KW, PRO_, EPI_, true>((args_), wg, nwg, xs, wbuf)

  // per-layer argument blocks
  auto t_qkv = [&](int l) {
    GemmArgs a = uni(A.t_qkv);
    a.gain = tab(o_tw + l * 6 + 0);
    a.W = tab(o_tw + l * 6 + 1);
    a.layer_off = (int64_t)l * t_lel;
    return a;
  };
  auto t_o = [&](int l) {
    GemmArgs a = uni(A.t_o);
    a.W = tab(o_tw + l * 6 + 2);
    return a;
  };
  auto t_gu = [&](int l) {
    GemmArgs a = uni(A.t_gu);
    a.gain = tab(o_tw + l * 6 + 3);
    a.W = tab(o_tw + l * 6 + 4);
    return a;
  };
  auto t_dn = [&](int l) {
    GemmArgs a = uni(A.t_dn);
    a.W = tab(o_tw + l * 6 + 5);
    return a;
  };
  auto d_qkv = [&](int s, int l) {
    GemmArgs a = uni(A.d_qkv);
    a.W = tab(o_dw + (s * Ld + l) * 4 + 0);
    a.gain = tab(o_dn + l * 2 + 0);
    a.scalar_widx = s;
    a.layer_off = (int64_t)l * d_lel;
    return a;
  };
  auto d_o = [&](int s, int l) {
    GemmArgs a = uni(A.d_o);
    a.W = tab(o_dw + (s * Ld + l) * 4 + 1);
    return a;
  };
  auto d_gu = [&](int s, int l) {
    GemmArgs a = uni(A.d_gu);
    a.W = tab(o_dw + (s * Ld + l) * 4 + 2);
    a.gain = tab(o_dn + l * 2 + 1);
    return a;
  };
  auto d_dn = [&](int s, int l) {
    GemmArgs a = uni(A.d_dn);
    a.W = tab(o_dw + (s * Ld + l) * 4 + 3);
    return a;
  };
  auto d_head = [&](int s) {
    GemmArgs a = uni(A.d_head);
    a.W = tab(o_dh + s);
    a.logits = uni(A.audio_logits) + (size_t)s * Va;
    return a;
  };

  // RoPE cos/sin at this step's position, for every temporal q/k/v epilogue
  __shared__ double s_rope[HD / 2][2];
  {
    const GemmArgs q0 = uni(A.t_qkv);
    if (q0.inv_freq != nullptr) rope_table(q0, s_rope, NT);
  }
  // ---- summed embedding ----
  embed_phase<T>(A.emb, frames, wg, nwg);
  PREFETCH_SYNC(EPI_QKV, t_qkv(0));

  // ---- temporal layers ----
  int nvalid, excl;
  window_of(uni(A.t_attn), 0, nvalid, excl);
  const int nspan = n_spans(uni(A.t_attn), nvalid);
  for (int l = 0; l < L; ++l) {
    GEMV(PRO_NORM, EPI_QKV, t_qkv(l));
    if (grid_sync(g)) return;
    {
      // each head's window split into nspan key spans, one per workgroup
      // (the per-operation kernel's split); the workgroup finishing a
      // head's last span merges the span partials
      AttnArgs at = uni(A.t_attn);
      at.layer_off = (int64_t)l * t_lel;
      for (int item = wg; item < H * nspan; item += nwg) {
        const int h = item / nspan, j = item % nspan;
        double* part = at.part + ((size_t)h * at.max_spans + j) * (HD + 2);
        attn_span<T, HD, NT, true>(at, h, 0, j * nvalid / nspan, (j + 1) * nvalid / nspan, nvalid,
                                   excl, s_o, part, nspan == 1);
        if (nspan > 1) {
          __shared__ int s_last;
          drain_stores();
          __syncthreads();
          if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add((MOSHI_GLB unsigned*)tickets + h * 16, 1u,
                                                        MOSHI_RLX, MOSHI_AGT);
            s_last = (old + 1 == (unsigned)((l + 1) * nspan));
          }
          __syncthreads();
          if (s_last) combine_direct<T, HD, true>(at, h, 0, nspan);
        }
      }
    }
    PREFETCH_SYNC(EPI_RESID, t_o(l));
    GEMV(PRO_DIRECT, EPI_RESID, t_o(l));
    PREFETCH_SYNC(EPI_SWIGLU, t_gu(l));
    GEMV(PRO_NORM, EPI_SWIGLU, t_gu(l));
    PREFETCH_SYNC(EPI_RESID, t_dn(l));
    GEMV(PRO_DIRECT, EPI_RESID, t_dn(l));
    if (l + 1 < L)
      PREFETCH_SYNC(EPI_QKV, t_qkv(l + 1));
    else
      PREFETCH_SYNC(EPI_ARGMAX, uni(A.t_head));
  }
  // ---- final norm -> hidden, text head (argmax partials) ----
  GEMV(PRO_NORM, EPI_ARGMAX, uni(A.t_head));
  PREFETCH_SYNC(EPI_STORE, uni(A.d_in));
  // ---- depformer input projections of all substeps ----
  GEMV(PRO_DIRECT, EPI_STORE, uni(A.d_in));
  STAGE_SYNC(EPI_QKV, d_qkv(0, 0));

  // ---- 16 substeps ----
  for (int s = 0; s < S; ++s) {
    for (int l = 0; l < Ld; ++l) {
      if (l == 0) {
        // The substep's entry (previous token -> residual) is folded into its
        // first q/k/v projection: every workgroup forms the normed input from
        // the previous head's partials itself; workgroup 0 stores the
        // residual and the token.
        EntryIn E;
        E.apart = uni(A.apart);
        E.prev_rows = s == 0 ? uni(A.Vt) : Va;
        E.pre = uni(A.pre) + (size_t)s * Dd;
        E.table = tab(o_de + s);
        E.y = uni(A.y);
        E.tok_out = s == 0 ? text_out : codes_out + (s - 1);
        gemv_staged<T, KW, PRO_NORM, EPI_QKV, true, true>(d_qkv(s, 0), wg, nwg, xs, wbuf, nullptr, &E);
      } else {
        GEMV_S(PRO_NORM, EPI_QKV, d_qkv(s, l));
      }
      {
        // A q/k/v tile holds 16 rows of one head. The workgroup that stores
        // the last of a head's tiles computes that head's attention.
        AttnArgs at = uni(A.d_attn);
        at.layer_off = (int64_t)l * d_lel;
        const unsigned goal = (unsigned)((s * Ld + l + 1) * DEP_TILES_PER_HEAD);
        __shared__ int s_last;
        drain_stores();
        __syncthreads();
        for (int tile = wg; tile * 16 < 3 * Dd; tile += nwg) {
          const int h = (tile * 16 % Dd) / HDD;
          if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add((MOSHI_GLB unsigned*)tickets + (H + h) * 16, 1u,
                                                        MOSHI_RLX, MOSHI_AGT);
            s_last = old + 1 == goal;
          }
          __syncthreads();
          if (s_last) dep_attention<T, HDD, NT, true, 1>(at, 0, h, 1, s + 1);
          __syncthreads();
        }
      }
      STAGE_SYNC(EPI_RESID, d_o(s, l));
      GEMV_S(PRO_DIRECT, EPI_RESID, d_o(s, l));
      STAGE_SYNC(EPI_SWIGLU, d_gu(s, l));
      GEMV_S(PRO_NORM, EPI_SWIGLU, d_gu(s, l));
      STAGE_SYNC(EPI_RESID, d_dn(s, l));
      GEMV_S(PRO_DIRECT, EPI_RESID, d_dn(s, l));
      if (l + 1 < Ld)
        STAGE_SYNC(EPI_QKV, d_qkv(s, l + 1));
      else
        STAGE_SYNC(EPI_ARGMAX, d_head(s));
    }
    GEMV_S(PRO_CAST, EPI_ARGMAX, d_head(s));
    if (s + 1 < S)
      STAGE_SYNC(EPI_QKV, d_qkv(s + 1, 0));
    else if (grid_sync(g))
      return;
  }
#undef GEMV
#undef GEMV_S
#undef PREFETCH_SYNC
#undef STAGE_SYNC
#undef PREFETCH_SYNC_G
  // ---- last code, next position ----
  if (wg == 0) {
    const int tok = reduce_token<NT>(uni(A.apart), (Va + 15) / 16, Va);
    if (threadIdx.x == 0) {
      *(MOSHI_GLB int*)(codes_out + S - 1) = tok;
      int64_t* pos = uni(A.pos);
      if (ldg(uni(A.live))) *(MOSHI_GLB int64_t*)pos += 1;
    }
  }
  if (trace != nullptr && wg == 0 && threadIdx.x == 0) *(MOSHI_GLB uint64_t*)(trace + g.idx + 1) = wall_clock64();
}

template <typename T, int HD, int HDD>
hipError_t launch_t(const StepArgs* dP, const int* frames, int* text_out, int* codes_out,
                    int parity, int nwg, size_t lds, hipStream_t st, uint64_t* trace) {
  void* args[] = {(void*)&dP,     (void*)&frames, (void*)&text_out, (void*)&codes_out,
                  (void*)&parity, (void*)&trace};
  return hipLaunchCooperativeKernel((const void*)step_kernel<T, HD, HDD>, dim3(nwg), dim3(NT), args,
                                    (unsigned)lds, st);
}

template <typename T, int HD, int HDD>
int max_grid_t(size_t lds) {
  int per_cu = 0, dev = 0, ncu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, step_kernel<T, HD, HDD>, NT, lds) !=
      hipSuccess)
    return 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return per_cu > 0 ? ncu : 0;  // one workgroup per CU
}

}  // namespace

// Instantiated shapes: bf16 with head dims 128 / 64 (PersonaPlex), fp32 with
// 64 / 32 (the small fp32 test model). Other shapes use the per-operation
// kernels.
bool step_supported(int dtype, int hd, int hdd) {
  return (dtype == DT_BF16 && hd == 128 && hdd == 64) || (dtype == DT_F32 && hd == 64 && hdd == 32);
}

int step_max_grid(int dtype, int hd, int hdd, size_t lds) {
  if (dtype == DT_BF16 && hd == 128 && hdd == 64) return max_grid_t<__bf16, 128, 64>(lds);
  if (dtype == DT_F32 && hd == 64 && hdd == 32) return max_grid_t<float, 64, 32>(lds);
  return 0;
}

hipError_t launch_step(int dtype, int hd, int hdd, const StepArgs* dP, const int* frames,
                       int* text_out, int* codes_out, int parity, int nwg, size_t lds,
                       hipStream_t st, uint64_t* trace) {
  if (dtype == DT_BF16 && hd == 128 && hdd == 64)
    return launch_t<__bf16, 128, 64>(dP, frames, text_out, codes_out, parity, nwg, lds, st, trace);
  if (dtype == DT_F32 && hd == 64 && hdd == 32)
    return launch_t<float, 64, 32>(dP, frames, text_out, codes_out, parity, nwg, lds, st, trace);
  return hipErrorInvalidValue;
}

}  // namespace moshi
