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
// Grid barrier (grid_arrive / grid_wait below): no single counter that every
// workgroup increments (those serialise at the memory side); each XCD's
// workgroups poll words in a page of their own, written either by every
// workgroup (arrival words) or by each XCD's last arrival (done words).
// Cross-workgroup data use agent-scope relaxed
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

// Barrier words of one set (32-bit words): one 4 KB page per XCD holding its
// arrival counter, its registration count, its done words (one per XCD, on
// one 128-byte line) and a copy of every workgroup's arrival word (each group
// on lines of its own), then a page with the grid-wide start counter. Each
// XCD's workgroups poll only their own page, so the polled lines of
// different XCDs sit in different memory channels: 256 workgroups polling
// one word would queue every other access to that word's channel behind
// them.
constexpr int MAX_XCC = 16;
constexpr int BW_PAGE = 1024;
constexpr int BW_LOCAL = 0, BW_REG = 32, BW_DONE = 64, BW_ARRIVE = 256;  // within an XCD's page
constexpr int BW_MAXWG = BW_PAGE - BW_ARRIVE;  // workgroups a grid barrier supports
constexpr int BW_FLAT = MAX_XCC * BW_PAGE;
static_assert(STEP_BAR_WORDS >= (MAX_XCC + 1) * BW_PAGE, "barrier words");

__device__ __forceinline__ unsigned xcc_id() {
  // hardware register XCC_ID (id 20), bits [3:0]
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (MAX_XCC - 1);
}

struct Grid {
  unsigned* set;
  int* abort;
  int limit;        // polls before a wait gives up (STEP_SPIN_LIMIT unless a test lowers it)
  uint64_t* trace;  // optional: barrier exit times of workgroup 0
  unsigned idx;    // barriers passed
  unsigned tshift; // trace entries written at flagged hand-offs (no barrier)
  unsigned xcc;    // this workgroup's XCD
  unsigned xcc_n;  // workgroups on it
  unsigned xmask;  // XCDs with at least one workgroup (bit x: XCD x)
  bool words;      // barrier form: per-workgroup arrival words (else XCD counters)
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
// flag rises, at most `limit` times. Returns nonzero when the grid must leave.
__device__ __forceinline__ int poll_until(unsigned* ctr, unsigned target, int* abort, int limit) {
  int spins = 0;
  while ((int)(__hip_atomic_load((MOSHI_GLB unsigned*)ctr, MOSHI_RLX, MOSHI_AGT) - target) < 0) {
    if (++spins > limit) {
      __hip_atomic_store((MOSHI_GLB int*)abort, 1, MOSHI_RLX, MOSHI_AGT);
      return 1;
    }
    if ((spins & 15) == 0 && __hip_atomic_load((MOSHI_GLB int*)abort, MOSHI_RLX, MOSHI_AGT)) return 1;
  }
  return 0;
}

// Grid barrier in two halves, so that loads can be issued in between:
// grid_arrive (after drain_stores() and a workgroup barrier) posts this
// workgroup's arrival; grid_wait waits for every other workgroup's. Loads
// issued between the two do not delay the arrival; the polls wait for them,
// but those loads (a weight prefetch) land well before the grid does. Every
// thread of every workgroup calls both; true = abort. A workgroup's stores
// landed before it arrived (drain_stores), its arrival before anything a
// poll can see, so its stores are visible once the polls let a workgroup go.
//
// Two forms (chosen per kernel at grid_init, measured):
// - arrival words: threads x < 16 store the barrier's number into this
//   workgroup's arrival word in XCD x's page (one store per XCD with
//   workgroups, issued together; no atomic round trip); wave 0 reads its own
//   XCD's copy of all arrival words (16 bytes per lane per load) until every
//   one has reached this barrier. Shortest path (one store, one poll), but
//   every poll reads 4 bytes per workgroup: used by the one-session step
//   kernel (256 workgroups, long phases).
// - XCD counters: thread 0 counts the workgroup into its XCD's counter; the
//   last arrival of an XCD (the returned count tells) writes the barrier's
//   number into that XCD's done word of every XCD's page, and wave 0 polls
//   the done words of its own page (one lane per XCD; one line). One atomic
//   round trip more, but polls read one line: used by the multi-session
//   depformer kernel (up to 512 workgroups, short phases).
// Arrival words and done words only grow, so a workgroup already past this
// barrier still counts as arrived.
__device__ __forceinline__ unsigned grid_arrive(Grid& g) {
  g.idx += 1;
  unsigned old = 0;
  if (g.words) {
    if (threadIdx.x < MAX_XCC && ((g.xmask >> threadIdx.x) & 1u))
      __hip_atomic_store((MOSHI_GLB unsigned*)g.set + threadIdx.x * BW_PAGE + BW_ARRIVE + blockIdx.x,
                         g.idx, MOSHI_RLX, MOSHI_AGT);
  } else if (threadIdx.x == 0) {
    old = __hip_atomic_fetch_add((MOSHI_GLB unsigned*)g.set + g.xcc * BW_PAGE + BW_LOCAL, 1u,
                                 MOSHI_RLX, MOSHI_AGT);
  }
  return old;
}

__device__ __forceinline__ bool grid_wait(Grid& g, unsigned old) {
  __shared__ int s_leave;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const unsigned* page = g.set + g.xcc * BW_PAGE;
    const int n = gridDim.x;
    const bool mine = lane < MAX_XCC && ((g.xmask >> lane) & 1u);
    if (!g.words) {
      old = __builtin_amdgcn_readfirstlane(old);  // thread 0's arrival count
      if (old + 1 == g.idx * g.xcc_n && mine)
        __hip_atomic_store((MOSHI_GLB unsigned*)g.set + lane * BW_PAGE + BW_DONE + g.xcc, g.idx,
                           MOSHI_RLX, MOSHI_AGT);
    }
    int spins = 0, leave = 0;
    while (true) {
      bool ok = true;
      if (g.words) {
        for (int base = 0; base < n; base += 256) {
          const int w0 = base + lane * 4;
          if (w0 < n) {
            const u32x4 q = ld16_coh(page + BW_ARRIVE, (uint32_t)w0 * 4u);
#pragma unroll
            for (int i = 0; i < 4; ++i) ok = ok && (w0 + i >= n || (int)(q[i] - g.idx) >= 0);
          }
        }
      } else if (mine) {
        ok = (int)(__hip_atomic_load((MOSHI_GLB unsigned*)page + BW_DONE + lane, MOSHI_RLX,
                                     MOSHI_AGT) - g.idx) >= 0;
      }
      if (__all(ok)) break;
      if (++spins > g.limit) {
        if (lane == 0) __hip_atomic_store((MOSHI_GLB int*)g.abort, 1, MOSHI_RLX, MOSHI_AGT);
        leave = 1;
        break;
      }
      if ((spins & 15) == 0 &&
          __builtin_amdgcn_readfirstlane(
              __hip_atomic_load((MOSHI_GLB int*)g.abort, MOSHI_RLX, MOSHI_AGT))) {
        leave = 1;
        break;
      }
    }
    if (lane == 0) {
      s_leave = leave;
      if (g.trace != nullptr && blockIdx.x == 0)
        *(MOSHI_GLB uint64_t*)(g.trace + g.idx + g.tshift) = wall_clock64();
    }
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
__device__ __forceinline__ bool grid_init(Grid& g, unsigned* bar, int parity, int* abort, int limit,
                                          uint64_t* trace, bool words) {
  __shared__ int s_leave;
  __shared__ unsigned s_cnt[MAX_XCC];
  g.set = bar + parity * STEP_BAR_WORDS;
  g.abort = abort;
  g.limit = limit;
  g.trace = trace;
  g.idx = 0;
  g.tshift = 0;
  g.xcc = xcc_id();
  g.words = words;
  if (gridDim.x > (unsigned)BW_MAXWG) {  // the launchers never ask for more; leave, reported as an abort
    if (threadIdx.x == 0) __hip_atomic_store((MOSHI_GLB int*)abort, 1, MOSHI_RLX, MOSHI_AGT);
    return true;
  }
  unsigned* other = bar + (parity ^ 1) * STEP_BAR_WORDS;
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < MAX_XCC * BW_MAXWG; i += blockDim.x)
      __hip_atomic_store((MOSHI_GLB unsigned*)other + (i / BW_MAXWG) * BW_PAGE + BW_ARRIVE + i % BW_MAXWG,
                         0u, MOSHI_RLX, MOSHI_AGT);
    if (threadIdx.x < MAX_XCC) {
      unsigned* page = other + threadIdx.x * BW_PAGE;
      __hip_atomic_store((MOSHI_GLB unsigned*)page + BW_LOCAL, 0u, MOSHI_RLX, MOSHI_AGT);
      __hip_atomic_store((MOSHI_GLB unsigned*)page + BW_REG, 0u, MOSHI_RLX, MOSHI_AGT);
      for (int x = 0; x < MAX_XCC; ++x)
        __hip_atomic_store((MOSHI_GLB unsigned*)page + BW_DONE + x, 0u, MOSHI_RLX, MOSHI_AGT);
    }
    if (threadIdx.x == 0) __hip_atomic_store((MOSHI_GLB unsigned*)other + BW_FLAT, 0u, MOSHI_RLX, MOSHI_AGT);
  }
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add((MOSHI_GLB unsigned*)g.set + g.xcc * BW_PAGE + BW_REG, 1u, MOSHI_RLX,
                           MOSHI_AGT);
    __hip_atomic_fetch_add((MOSHI_GLB unsigned*)g.set + BW_FLAT, 1u, MOSHI_RLX, MOSHI_AGT);
    s_leave = poll_until(g.set + BW_FLAT, gridDim.x, abort, limit);
    if (trace != nullptr && blockIdx.x == 0) *(MOSHI_GLB uint64_t*)trace = wall_clock64();
  }
  __syncthreads();
  if (s_leave) return true;
  if (threadIdx.x < MAX_XCC)
    s_cnt[threadIdx.x] = __hip_atomic_load((MOSHI_GLB unsigned*)g.set + threadIdx.x * BW_PAGE + BW_REG,
                                           MOSHI_RLX, MOSHI_AGT);
  __syncthreads();
  g.xmask = 0;
  for (int i = 0; i < MAX_XCC; ++i) g.xmask |= s_cnt[i] ? (1u << i) : 0u;
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

// ---- flagged vectors: the depformer's exchange between workgroups ---------
//
// The 16 substeps are ~400 dependent projections of a few MB each; a grid
// barrier between them costs several memory round trips (store
// acknowledgement, the arrival, the polls). Instead each
// vector a projection hands on is written as flagged 8-byte words
// {payload, flag}, flag = the launch's sequence number, and its readers poll
// the words themselves until every flag is current: one round trip after
// the last producer's store lands. Every flagged vector is written once per
// launch (one buffer per substep and layer), so a word never needs clearing
// and a reader never races a later write of the same word; the sequence
// number differs from the previous launch's, and the buffers start zeroed
// with sequence numbers starting at 1.
//
// fp64 element i of a vector: words 2i (low half) and 2i+1 (high half), one
// 16-byte line. Model-dtype element i: word i (the value's stored bits).
// Writers use one 8-byte store per word, readers 16-byte sc1 loads of whole
// lines (two words, each read whole), so a word is never seen half written.
//
// Layout (in words) of the flagged arena: for each (substep s, layer l), in
// order s * Ld + l, a block of 11 Dd + Fd words
//   R1 [2 Dd] residual after the output projection, S1 [Dd] its sums of
//   squares per row pair, R2 [2 Dd] residual after the down projection, S2
//   [Dd], Q [2 Dd] queries, K [Dd], V [Dd] (rounded), O [Dd] attention
//   output (rounded), A [Fd] SwiGLU output (rounded);
// then for each substep, Y [2 Dd] (the substep's input residual) and AP
// [32 ceil(Va / 16)] (argmax partials of its head, one per row pair: value
// low, value high, index, 0); then the temporal attention's: for each layer,
// head and key span, the span partial [2 (hd + 2)] (M, L, O[hd]); then for
// each layer the merged attention output O [D] (rounded).

struct LLCtx {
  uint64_t* w;     // the flagged arena
  uint32_t flag;   // this launch's sequence number
  int* abort;
  int limit;       // polls before a wait gives up
};

struct LLMap {
  int Dd, Fd, Ld, nta;
  // word indices (the host keeps the arena under 2 GB, so they fit 32 bits)
  __device__ uint32_t layer(int s, int l) const { return (uint32_t)(s * Ld + l) * (11 * Dd + Fd); }
  __device__ uint32_t R1(int s, int l) const { return layer(s, l); }
  __device__ uint32_t S1(int s, int l) const { return layer(s, l) + 2 * Dd; }
  __device__ uint32_t R2(int s, int l) const { return layer(s, l) + 3 * Dd; }
  __device__ uint32_t S2(int s, int l) const { return layer(s, l) + 5 * Dd; }
  __device__ uint32_t Q(int s, int l) const { return layer(s, l) + 6 * Dd; }
  __device__ uint32_t K(int s, int l) const { return layer(s, l) + 8 * Dd; }
  __device__ uint32_t V(int s, int l) const { return layer(s, l) + 9 * Dd; }
  __device__ uint32_t O(int s, int l) const { return layer(s, l) + 10 * Dd; }
  __device__ uint32_t A(int s, int l) const { return layer(s, l) + 11 * Dd; }
  __device__ uint32_t sub(int s, int S) const {
    return layer(S, 0) + (uint32_t)s * (2 * Dd + 32 * nta);
  }
  __device__ uint32_t Y(int s, int S) const { return sub(s, S); }
  __device__ uint32_t AP(int s, int S) const { return sub(s, S) + 2 * Dd; }
  // temporal attention, after the depformer's vectors: per layer, the span
  // partials of every head (M, L, O[hd], fp64) and the merged output [D]
  int S, H, HD, NSP, L, D;
  __device__ uint32_t tbase() const { return sub(S, S); }
  __device__ uint32_t TP(int l, int h, int j) const {
    return tbase() + (uint32_t)((l * H + h) * NSP + j) * (2 * (HD + 2));
  }
  __device__ uint32_t TO(int l) const {
    return tbase() + (uint32_t)(L * H * NSP) * (2 * (HD + 2)) + (uint32_t)l * D;
  }
};

__device__ __forceinline__ void ll_put(const LLCtx& c, uint32_t word, uint32_t payload) {
  st_u64<true>(c.w + word, (uint64_t)payload | ((uint64_t)c.flag << 32));
}
__device__ __forceinline__ void ll_put_f64(const LLCtx& c, uint32_t word, double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  ll_put(c, word, (uint32_t)b);
  ll_put(c, word + 1, (uint32_t)(b >> 32));
}
// the line holding words `word` (even) and word + 1
__device__ __forceinline__ u32x4 ll_ld(const LLCtx& c, uint32_t word) {
  return ld16_coh(c.w, word * 8u);
}
__device__ __forceinline__ bool ll_fresh(const u32x4& q, uint32_t flag) {
  return (q[1] == flag) & (q[3] == flag);
}
__device__ __forceinline__ double ll_f64(const u32x4& q) {
  return __hiloint2double((int)q[2], (int)q[0]);
}

// Waits until the N lines starting at the even words addr(j) are current,
// re-reading stale ones (LOADED: the first reads are already in q). False
// when the wait timed out or another workgroup gave up (the abort flag).
// Addresses are recomputed for each re-read rather than held in registers.
template <int N, bool LOADED = false, typename F>
__device__ __forceinline__ bool ll_wait(const LLCtx& c, F addr, u32x4 (&q)[N]) {
  if (!LOADED) {
#pragma unroll
    for (int j = 0; j < N; ++j) q[j] = ll_ld(c, addr(j));
  }
  for (int spins = 0;; ++spins) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < N; ++j) ok = ok & ll_fresh(q[j], c.flag);
    if (ok) return true;
    if (spins > c.limit) {
      __hip_atomic_store((MOSHI_GLB int*)c.abort, 1, MOSHI_RLX, MOSHI_AGT);
      return false;
    }
    if ((spins & 15) == 15 && __hip_atomic_load((MOSHI_GLB int*)c.abort, MOSHI_RLX, MOSHI_AGT))
      return false;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (!ll_fresh(q[j], c.flag)) q[j] = ll_ld(c, addr(j));
  }
}

// The same for N single words (8-byte loads) at words addr(j).
template <int N, bool LOADED = false, typename F>
__device__ __forceinline__ bool ll_wait_words(const LLCtx& c, F addr, uint64_t (&q)[N]) {
  if (!LOADED) {
#pragma unroll
    for (int j = 0; j < N; ++j) q[j] = ld_u64<true>(c.w + addr(j));
  }
  for (int spins = 0;; ++spins) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < N; ++j) ok = ok & ((uint32_t)(q[j] >> 32) == c.flag);
    if (ok) return true;
    if (spins > c.limit) {
      __hip_atomic_store((MOSHI_GLB int*)c.abort, 1, MOSHI_RLX, MOSHI_AGT);
      return false;
    }
    if ((spins & 15) == 15 && __hip_atomic_load((MOSHI_GLB int*)c.abort, MOSHI_RLX, MOSHI_AGT))
      return false;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < N; ++j)
      if ((uint32_t)(q[j] >> 32) != c.flag) q[j] = ld_u64<true>(c.w + addr(j));
  }
}

// Stored bits of a model-dtype value in a word's payload, as a double.
template <typename T>
__device__ __forceinline__ double ll_val(uint32_t payload) {
  return sizeof(T) == 2 ? (double)__uint_as_float(payload << 16) : (double)__uint_as_float(payload);
}

// PRO_NORM / PRO_CAST input from a flagged fp64 vector at word ox (PRO_NORM:
// sums of squares per pair at word os), in build_input's arithmetic: pair
// p = t (K / 2 <= NTH), partial t, the scale from rms_finish. False = leave.
template <typename T, int PRO, int NTH>
__device__ __forceinline__ bool ll_input_x(const GemmArgs& a, const LLCtx& c, uint32_t ox, uint32_t os,
                                           T* xs, double* red) {
  const int t = tid();
  const int np = a.K / 2;
  const int p = t < np ? t : np - 1;
  double g0 = 1.0, g1 = 1.0;
  if constexpr (PRO == PRO_NORM) ld_pair_d((const T*)a.gain, p, g0, g1);
  const int n = a.n_ssq;
  const int pn = t < n ? t : n - 1;
  auto wd = [&](int j) {
    return j < 2 ? ox + 4 * (uint32_t)p + 2 * j : (PRO == PRO_NORM ? os + 2 * (uint32_t)pn : ox);
  };
  u32x4 q[3];
  const bool ok = ll_wait<3>(c, wd, q);
  if (__syncthreads_or(!ok)) return false;
  const double x0 = ll_f64(q[0]), x1 = ll_f64(q[1]);
  double rs = 1.0;
  if constexpr (PRO == PRO_NORM) {
    double sum = 0.0;
    if (t < n) sum += ll_f64(q[2]);
    rs = rms_finish(sum, a, red, NTH);
  }
  if (t < np) {
    const double v0 = PRO == PRO_NORM ? x0 * rs * g0 : x0;
    const double v1 = PRO == PRO_NORM ? x1 * rs * g1 : x1;
    put_pair<T, false>(xs, nullptr, t, v0, v1);
  }
  return true;
}

// PRO_DIRECT input from a flagged model-dtype vector at word ov (K <= 8 NTH).
template <typename T, int NTH>
__device__ __forceinline__ bool ll_input_direct(const GemmArgs& a, const LLCtx& c, uint32_t ov,
                                                T* xs) {
  constexpr int ML = 4;
  const int t = tid();
  const int nl = a.K / 2;  // lines, two values each
  auto wd = [&](int j) {
    const int i = t + j * NTH;
    return ov + 2 * (uint32_t)(i < nl ? i : nl - 1);
  };
  u32x4 q[ML];
  const bool ok = ll_wait<ML>(c, wd, q);
#pragma unroll
  for (int j = 0; j < ML; ++j) {
    const int i = t + j * NTH;
    if (i < nl) {
      if constexpr (sizeof(T) == 2) {
        *(uint32_t*)(xs + 2 * i) = (q[j][0] & 0xffffu) | (q[j][2] << 16);
      } else {
        *(uint64_t*)(xs + 2 * i) = (uint64_t)q[j][0] | ((uint64_t)q[j][2] << 32);
      }
    }
  }
  return !__syncthreads_or(!ok);
}

// Greedy token from flagged argmax partials at word ap (n_part of them, one
// per row pair), in reduce_token's arithmetic: the comparison is exact and
// ties go to the lowest index, so the winner does not depend on how rows
// were grouped into partials. ok = false when a wait gave up.
template <int NTH>
__device__ __forceinline__ int ll_reduce_token(const LLCtx& c, uint32_t ap, int n_part, int n_rows,
                                               bool& ok) {
  constexpr int NW = NTH / 64;
  __shared__ double s_v[NW];
  __shared__ int s_i[NW];
  const int t = tid();
  double bv = -INFINITY;
  int bi = 0x7fffffff;
  // partials t and t + NTH in one wait (clamped; duplicates are harmless)
  {
    auto wd = [&](int j) {
      const int i = t + (j >> 1) * NTH;
      return ap + 4 * (uint32_t)(i < n_part ? i : n_part - 1) + 2 * (j & 1);
    };
    u32x4 q[4];
    ok = ll_wait<4>(c, wd, q);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const double v = ll_f64(q[2 * k]);
      const int idx = (int)q[2 * k + 1][0];
      if (t + k * NTH < n_part && arg_better(v, idx, bv, bi)) {
        bv = v;
        bi = idx;
      }
    }
  }
  for (int i = t + 2 * NTH; i < n_part; i += NTH) {
    u32x4 q[2];
    ok = ok & ll_wait<2>(c, [&](int j) { return ap + 4 * (uint32_t)i + 2 * j; }, q);
    const double v = ll_f64(q[0]);
    const int idx = (int)q[1][0];
    if (arg_better(v, idx, bv, bi)) {
      bv = v;
      bi = idx;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double ov = shfl_xor_d(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (arg_better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if ((t & 63) == 0) {
    s_v[t >> 6] = bv;
    s_i[t >> 6] = bi;
  }
  __syncthreads();
  bv = s_v[0];
  bi = s_i[0];
  for (int w = 1; w < NW; ++w)
    if (arg_better(s_v[w], s_i[w], bv, bi)) {
      bv = s_v[w];
      bi = s_i[w];
    }
  __syncthreads();
  return bi < n_rows ? bi : 0;
}

// Input of a substep's first q/k/v projection (build_entry_input's
// arithmetic): the previous token (from the text head's partials at s = 0,
// else from the previous substep's flagged head partials), y = pre + E[tok];
// the `first` workgroup stores y as the flagged vector Y and the token.
struct EntryLL {
  const ArgPart* text_part;  // s = 0: the text head's partials (plain)
  uint32_t ap;               // s > 0: word of the previous head's flagged partials
  int prev_rows;
  const double* pre;
  const void* table;
  uint32_t y;                // word of Y[s]
  int* tok_out;
  const int* forced;         // teacher forcing: the token when forced[0] >= 0 (null: none)
};

template <typename T, int NTH>
__device__ __forceinline__ bool ll_input_entry(const GemmArgs& a, const LLCtx& c, const EntryLL& E,
                                               T* xs, double* red, bool first) {
  const int t = tid();
  const int np = a.K / 2;  // <= NTH
  const T* g = (const T*)a.gain;
  const int p0 = t < np ? t : np - 1;
  double pv[2], gv[2];
  ld_pair_f64<true>(E.pre, p0, pv[0], pv[1]);
  ld_pair_d(g, p0, gv[0], gv[1]);
  const int n_tiles = (E.prev_rows + 15) / 16;
  bool ok = true;
  const int tok = E.text_part != nullptr
                      ? reduce_token<NTH>(E.text_part, n_tiles, E.prev_rows)
                      : ll_reduce_token<NTH>(c, E.ap, 8 * n_tiles, E.prev_rows, ok);
  if (__syncthreads_or(!ok)) return false;
  int tk = tok;
  if (E.forced != nullptr) {
    const int f = ldg(E.forced);
    tk = f >= 0 ? f : tk;
  }
  if (first && t == 0) st_i32<true>(E.tok_out, tk);
  const T* row = (const T*)E.table + (uint32_t)tk * a.K;
  double ev[2];
  ld_pair_d(row, p0, ev[0], ev[1]);
  const double y0 = pv[0] + ev[0], y1 = pv[1] + ev[1];
  double sum = 0.0;
  if (t < np) {
    if (first) {
      ll_put_f64(c, E.y + 4 * (uint32_t)t, y0);
      ll_put_f64(c, E.y + 4 * (uint32_t)t + 2, y1);
    }
    sum += sq_pair(y0, y1);
  }
  const double rs = rms_finish(sum, a, red, NTH);
  if (t < np) put_pair<T, false>(xs, nullptr, t, y0 * rs * gv[0], y1 * rs * gv[1]);
  return true;
}

// Where a flagged projection reads and writes (word offsets in the arena).
struct LLIo {
  uint32_t x, ss;      // PRO_NORM / PRO_CAST input (fp64), its sums of squares; PRO_DIRECT: x
  uint32_t resid;      // EPI_RESID: residual rows (fp64)
  uint32_t out, out_ss;  // EPI_RESID: new residual, its sums of squares; EPI_SWIGLU: act;
                         // EPI_ARGMAX: partials
  uint32_t q, k, v;    // EPI_QKV
};

// Epilogue of the R = 2 rows a wave owns (lane 0), flagged outputs:
// wave_epilogue's arithmetic. rv: the residual rows (EPI_RESID).
template <typename T, int EPI>
__device__ __forceinline__ void ll_wave_epilogue(const GemmArgs& a, const LLCtx& c, const LLIo& io,
                                                 int tile, int w, const double* v,
                                                 const double* rv) {
  constexpr int R = 2;
  if constexpr (EPI == EPI_RESID) {
    const int row0 = tile * 16 + w * R;
    if (row0 >= a.N) return;
    double xn[R];
#pragma unroll
    for (int r = 0; r < R; ++r) xn[r] = rv[r] + v[r];
    double ss = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (row0 + r < a.N) {
        ll_put_f64(c, io.out + 2 * (uint32_t)(row0 + r), xn[r]);
        ss += xn[r] * xn[r];
      }
    }
    ll_put_f64(c, io.out_ss + 2 * (uint32_t)(row0 / R), ss);
  } else if constexpr (EPI == EPI_QKV) {
    const int row0 = tile * 16 + w * R;
    if (row0 >= a.N) return;
    const int part = row0 / a.dq;
    const int din = row0 - part * a.dq;
    if (part == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) ll_put_f64(c, io.q + 2 * (uint32_t)(din + r), v[r]);
    } else {
      const uint32_t base = (part == 1 ? io.k : io.v) + din;
#pragma unroll
      for (int r = 0; r < R; ++r) ll_put(c, base + r, stored_bits<T>(v[r]));
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int u0 = tile * 8 + w;
    if (u0 < a.N) {
      const double gt = v[0], up = v[1];
      const double r_ = gt / (1.0 + exp(-gt)) * up;
      ll_put(c, io.out + u0, stored_bits<T>(r_));
    }
  }
}

// Argmax partial of the row pair of wave w in tile `tile` (lane 0): the
// logits of its rows (fp32 copy for the host) and (max, lowest index) of the
// pair, NaN counting as -inf; partial number tile * 8 + w. A pair past the
// last row still writes its partial (index INT_MAX, never chosen).
template <typename T>
__device__ __forceinline__ void ll_argmax_pair(const GemmArgs& a, const LLCtx& c, const LLIo& io,
                                               int tile, int w, const double* v) {
  double bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = tile * 16 + w * 2 + r;
    if (row < a.N) {
      *(MOSHI_GLB float*)(a.logits + row) = (float)v[r];  // host reads
      const double val = (v[r] != v[r]) ? -INFINITY : v[r];
      if (bi == 0x7fffffff || val > bv) {
        bv = val;
        bi = row;
      }
    }
  }
  const uint32_t pw = io.out + 4 * (uint32_t)(tile * 8 + w);
  ll_put_f64(c, pw, bv);
  ll_put(c, pw + 2, (uint32_t)bi);
  ll_put(c, pw + 3, 0u);
}

// A projection from a weight slice staged by gemv_stage (gemv_staged's
// arithmetic and work split) whose input and outputs are flagged vectors.
// Once the input has arrived, each wave copies its weight slots (at most MI
// items x MC column passes) and its input groups from LDS to registers, then
// requests the next operation's slice into LDS (stage_next): before computing
// (EARLY: the slice has the longest time to land before the next operation
// needs it) or after its outputs are stored (issuing it then does not delay
// them). Either way it streams while the next input is awaited; a wave's
// loads complete in issue order, so that first poll returns once the slice
// has landed. Which is faster depends on the sizes of the next slices
// (measured per operation).
// Workgroups without rows skip the projection (but still stage the next
// one), except workgroup 0, which always waits for the input (its trace
// stamp marks the end of the previous operation). False = leave (a wait gave
// up). Argmax projections write one partial per row pair.
template <typename T, int KW, int PRO, int EPI, int MI, int MC, bool EARLY, bool ENTRY = false,
          typename FN>
__device__ __forceinline__ bool ll_gemv(const GemmArgs& a, const LLCtx& c, const LLIo& io, int wg,
                                        int nwg, T* xs, const unsigned char* wbuf,
                                        const EntryLL* ent, uint64_t* stamp, FN stage_next) {
  constexpr int VEC = VecOf<T>::N;
  constexpr int R = 16 / KW;
  constexpr int NTH = 64 * KW;
  static_assert(R == 2, "row pairs");
  const int t = tid();
  const int lane = t & 63, wave = t >> 6;
  __shared__ double s_tmp[KW];
  const int ngroups = a.K / VEC;
  const int cpl = staged_cpl<T>(a.K);
  bool wg_any;
  if constexpr (staged_by_tile<EPI>()) {
    wg_any = wg < n_tiles_of(EPI, a.N);
  } else {
    const int P = EPI == EPI_SWIGLU ? a.N : (a.N + 1) / 2;
    wg_any = wg * P / nwg < (wg + 1) * P / nwg;
  }
  if (!wg_any && wg != 0) {
    stage_next();
    return true;
  }
  // this wave's items (staged_item is false from the first missing one on)
  int te[MI], we[MI], nit = 0;
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    te[j] = 0;
    we[j] = 0;
    if (staged_item<EPI, KW>(a, wg, nwg, wave, j, te[j], we[j])) nit = j + 1;
  }
  // residual rows of the wave's first item, requested before the input
  u32x4 rq[2];
  const int rrow0 = nit > 0 ? te[0] * 16 + we[0] * R : 0;
  auto rw = [&](int r) { return io.resid + 2 * (uint32_t)(rrow0 + r < a.N ? rrow0 + r : rrow0); };
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int r = 0; r < 2; ++r) rq[r] = ll_ld(c, rw(r));
  }
  bool ok;
  if constexpr (ENTRY)
    ok = ll_input_entry<T, NTH>(a, c, *ent, xs, s_tmp, wg == 0);
  else if constexpr (PRO == PRO_DIRECT)
    ok = ll_input_direct<T, NTH>(a, c, io.x, xs);
  else
    ok = ll_input_x<T, PRO, NTH>(a, c, io.x, io.ss, xs, s_tmp);
  if (!ok) return false;
  if constexpr (EPI == EPI_RESID) {
    const bool rok = ll_wait<2, true>(c, rw, rq);
    if (__syncthreads_or(!rok)) return false;
  }
  if (stamp != nullptr && wg == 0 && t == 0) *(MOSHI_GLB uint64_t*)stamp = wall_clock64();
  __syncthreads();
  if (!wg_any) {
    stage_next();
    return true;
  }
  // this wave's LDS-direct loads have landed (the input waits above already
  // waited for them)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const MOSHI_LDS unsigned char* base = (const MOSHI_LDS unsigned char*)wbuf;
  u32x4 wr[MI][MC][2], xr[MC];
#pragma unroll
  for (int cc = 0; cc < MC; ++cc) {
    const int gi = cc * 64 + lane;
    xr[cc] = *(const u32x4*)(xs + (uint32_t)(gi < ngroups ? gi : 0) * VEC);
  }
#pragma unroll
  for (int j = 0; j < MI; ++j)
#pragma unroll
    for (int cc = 0; cc < MC; ++cc)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        // slot (j * cpl + cc) * 2 + r of gemv_stage's layout (clamped to slot 0 when unused)
        const int slot = (j < nit && cc < cpl) ? (j * cpl + cc) * 2 + r : 0;
        wr[j][cc][r] = *(const MOSHI_LDS u32x4*)(base + ((slot * KW + wave) * 64 + lane) * 16);
      }
  // every read of this wave's slots and of xs has returned before the next
  // slice overwrites them; the workgroup barrier covers the other waves' reads of xs
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __syncthreads();
  if constexpr (EARLY) stage_next();
  // every item's row sums, then the items' epilogues in parallel lanes
  // (lane j takes item j; the reduction leaves the sums in every lane)
  double acc[MI][R];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    acc[j][0] = 0.0;
    acc[j][1] = 0.0;
    if (j < nit) {
#pragma unroll
      for (int cc = 0; cc < MC; ++cc) {
        const int gi = cc * 64 + lane;
        if (cc < cpl && gi < ngroups) {
          double xv[VEC];
          widen<T>(xr[cc], xv);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            double wd[VEC];
            widen<T>(wr[j][cc][r], wd);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[j][r] = fma(wd[e], xv[e], acc[j][r]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MI; ++j)
    if (j < nit) {
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = group_reduce<64>(acc[j][r]);
    }
  if (lane < nit) {
    const int j = lane;
    double v[R] = {acc[0][0], acc[0][1]};
    int tj = te[0], wj = we[0];
#pragma unroll
    for (int i = 1; i < MI; ++i)
      if (j == i) {
        v[0] = acc[i][0];
        v[1] = acc[i][1];
        tj = te[i];
        wj = we[i];
      }
    if constexpr (EPI == EPI_ARGMAX) {
      ll_argmax_pair<T>(a, c, io, tj, wj, v);
    } else {
      double rv[R] = {0.0, 0.0};
      if constexpr (EPI == EPI_RESID) {
        if (j == 0) {
          rv[0] = ll_f64(rq[0]);
          rv[1] = ll_f64(rq[1]);
        } else {
          // later items (only with many rows per workgroup): wait here
          const int row0 = tj * 16 + wj * R;
          u32x4 q2[2];
          (void)ll_wait<2>(  // a timeout raises the abort flag; the host fails the step
              c, [&](int r) { return io.resid + 2 * (uint32_t)(row0 + r < a.N ? row0 + r : row0); },
              q2);
          rv[0] = ll_f64(q2[0]);
          rv[1] = ll_f64(q2[1]);
        }
      }
      ll_wave_epilogue<T, EPI>(a, c, io, tj, wj, v, rv);
    }
  }
  if constexpr (!EARLY) stage_next();
  __syncthreads();  // xs may be rewritten by the next operation
  return true;
}

// Merge of the flagged span partials of temporal head h (layer l) for the
// output dims [d0, d1) this workgroup takes: combine_direct's arithmetic
// (span weights e^{m_c - M}, sums in span order), by wave 0 (lane i: dim
// d0 + i; every lane takes part so that lanes 0..7 form the span weights).
// The rounded outputs go to the flagged O[l]. False = a wait gave up.
template <typename T, int HD>
__device__ __forceinline__ bool ll_span_merge(const LLCtx& c, const LLMap& M, int l, int h,
                                              int nspans, int d0, int d1) {
  constexpr int NS = 8;  // spans per head at most (the grid's split)
  bool ok = true;
  if (tid() < 64) {
    const int lane = tid();
    const int d = d0 + lane < d1 ? d0 + lane : d0;
    const int lc = lane & (NS - 1);  // lanes c < NS also fetch span c's M and L
    // lines: M and L of span lc, then O[d] of spans 0..NS-1 (spans past
    // nspans read span 0)
    auto wd = [&](int i) {
      const int cc = i < 2 ? (lc < nspans ? lc : 0) : (i - 2 < nspans ? i - 2 : 0);
      const uint32_t pw = M.TP(l, h, cc);
      return i == 0 ? pw : i == 1 ? pw + 2 : pw + 4 + 2 * (uint32_t)d;
    };
    u32x4 q[2 + NS];
    ok = ll_wait<2 + NS>(c, wd, q);
    const double mine = ll_f64(q[0]), lmine = ll_f64(q[1]);
    double Mx = -INFINITY;
#pragma unroll
    for (int cc = 0; cc < NS; ++cc)
      if (cc < nspans) Mx = fmax(Mx, readlane_d(mine, cc));
    const double emine = (mine == -INFINITY) ? 0.0 : exp(mine - Mx);
    double Ls = 0.0, Os = 0.0;
#pragma unroll
    for (int cc = 0; cc < NS; ++cc) {
      if (cc < nspans) {
        const double w = readlane_d(emine, cc);
        Ls = fma(readlane_d(lmine, cc), w, Ls);
        Os = fma(ll_f64(q[2 + cc]), w, Os);
      }
    }
    if (d0 + lane < d1) {
      const double o = Ls > 0.0 ? Os / Ls : 0.0;
      ll_put(c, M.TO(l) + (uint32_t)(h * HD + d), stored_bits<T>(o));
    }
  }
  return ok;
}

// Attention of depformer head h at substep s (keys: entries 0..s of this
// layer except entry `excl`, -1 = none), by wave 0 of one workgroup, from the
// flagged q, K and V: the arithmetic of dep_attention for one head. The
// output goes to the flagged O[s][l]. False = leave.
template <typename T, int HD, int NTH>
__device__ __forceinline__ bool ll_dep_attention(const LLCtx& c, const LLMap& M, int s, int l,
                                                 int h, int excl) {
  constexpr int VEC = VecOf<T>::N;
  constexpr int TK = HD / VEC;
  constexpr int KPW = 64 / TK;
  constexpr int NP = (DEP_MAX_KEYS + KPW - 1) / KPW;
  constexpr int DPL = HD > 64 ? HD / 64 : 1;
  constexpr int KL = NP * VEC / 2;  // K lines per lane
  __shared__ double s_sc[64];
  __shared__ int s_bad;
  const int t = tid();
  const int lane = t & 63;
  const int kd = lane % TK, kq = lane / TK;
  const int nvalid = s + 1;
  if (t == 0) s_bad = 0;
  __syncthreads();
  if (t < 64) {
    const double scale = 1.0 / sqrt((double)HD);
    // q (VEC fp64 lines), K (VEC/2 lines per key pass) and V (one word per
    // entry j and dim lane + 64 i), all requested before any is waited for
    const uint32_t qb = M.Q(s, l) + 2 * (uint32_t)(h * HD + kd * VEC);
    uint32_t kb[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int j = p * KPW + kq;
      kb[p] = M.K(j < nvalid ? j : 0, l) + (uint32_t)(h * HD + kd * VEC);
    }
    const uint32_t vstep = M.V(1, l) - M.V(0, l);  // words between entries
    const uint32_t vb = M.V(0, l) + (uint32_t)(h * HD);
    auto wv = [&](int n) {
      const int j = n / DPL, i = n % DPL;
      const int dd = (lane + 64 * i) < HD ? lane + 64 * i : 0;
      return vb + (uint32_t)(j < nvalid ? j : 0) * vstep + (uint32_t)dd;
    };
    constexpr int NV = DEP_MAX_KEYS * DPL;
    uint64_t vq[NV];
    auto wq = [&](int e) { return qb + 2 * e; };
    auto wk = [&](int i) { return kb[i / (VEC / 2)] + 2 * (i % (VEC / 2)); };
    bool ok;
    {
      u32x4 qq[VEC], kk[KL];
#pragma unroll
      for (int e = 0; e < VEC; ++e) qq[e] = ll_ld(c, wq(e));
#pragma unroll
      for (int i = 0; i < KL; ++i) kk[i] = ll_ld(c, wk(i));
#pragma unroll
      for (int n = 0; n < NV; ++n) vq[n] = ld_u64<true>(c.w + wv(n));
      ok = ll_wait<VEC, true>(c, wq, qq);
      ok = ok & ll_wait<KL, true>(c, wk, kk);
      double qv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) qv[e] = ll_f64(qq[e]);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        double d = 0.0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const u32x4& q = kk[p * (VEC / 2) + e / 2];
          d = fma(qv[e], ll_val<T>(q[2 * (e & 1)]), d);
        }
        d = group_reduce<TK>(d);
        const int j = p * KPW + kq;
        if (kd == 0 && j < DEP_MAX_KEYS) s_sc[j] = d * scale;
      }
    }
    ok = ok & ll_wait_words<NV, true>(c, wv, vq);
    // softmax over the valid keys
    const double sv = (lane < nvalid && lane != excl) ? s_sc[lane] : -INFINITY;
    const double m = group_reduce<64, true>(sv);
    const double pj = (sv == -INFINITY) ? 0.0 : exp(sv - m);
    const double lsum = group_reduce<64>(pj);
    s_sc[lane] = pj;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int dd = lane + 64 * i;
      double od = 0.0;
#pragma unroll
      for (int j = 0; j < DEP_MAX_KEYS; ++j) {
        if (j < nvalid) od = fma(s_sc[j], ll_val<T>((uint32_t)vq[j * DPL + i]), od);
      }
      if (dd < HD) {
        const double ov = lsum > 0.0 ? od / lsum : 0.0;
        ll_put(c, M.O(s, l) + (uint32_t)(h * HD + dd), stored_bits<T>(ov));
      }
    }
    if (!ok) s_bad = 1;
  }
  __syncthreads();
  return s_bad == 0;
}

template <typename T, int HD, int HDD>
__global__ __launch_bounds__(NT) void step_kernel(const StepArgs* P,
                                                  const int* __restrict__ frames, int* text_out,
                                                  int* codes_out, int parity, uint32_t seq,
                                                  uint64_t* trace) {
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
  if (grid_init(g, uni(A.bar), parity, uni(A.abort), uni(A.spin_limit), trace, true)) return;
  // first weight batch of the next projection, requested before each barrier
  u32x4 pf[GU][16 / KW];
  unsigned char* const wbuf = s_dyn + uni(A.wbuf_lds);
#define PREFETCH_SYNC_G(EPI_, args_, GU_, PF_)             \
  do {                                                     \
    const GemmArgs na_ = (args_);                          \
    drain_stores();                                        \
    __syncthreads();                                       \
    const unsigned old_ = grid_arrive(g);                  \
    gemv_prefetch<T, KW, EPI_, GU_>(na_, wg, nwg, PF_);         \
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
    GemmArgs a = uni(A.d_head);  // with the final norm: its gain and sums of squares set
    a.W = tab(o_dh + s);
    a.logits = uni(A.audio_logits) + (size_t)s * Va;
    return a;
  };
  const int S_run = uni(A.S_run);
  const bool dep_final_norm = uni(A.dep_final_norm) != 0;
  const int* const forced = uni(A.forced);
  // the depformer ring reading masks entry 0 at the last substep (-1 = off)
  const int ref_excl_at = uni(A.d_attn.scalar_excl) >= 0 ? S_run - 1 : -1;

  // RoPE cos/sin at this step's position, for every temporal q/k/v epilogue
  __shared__ double s_rope[HD / 2][2];
  {
    const GemmArgs q0 = uni(A.t_qkv);
    if (q0.inv_freq != nullptr) rope_table(q0, s_rope, NT);
  }
  // ---- summed embedding ----
  embed_phase<T>(A.emb, frames, wg, nwg);
  PREFETCH_SYNC(EPI_QKV, t_qkv(0));

  // flagged vectors (the temporal attention's outputs, the depformer's hand-offs)
  LLCtx c;
  c.w = uni(A.ll);
  c.flag = seq;
  c.abort = uni(A.abort);
  c.limit = uni(A.ll_spin_limit);
  LLMap M;
  M.Dd = Dd;
  M.Fd = uni(A.d_gu.N);
  M.Ld = Ld;
  M.nta = (Va + 15) / 16;
  M.S = S;
  M.H = H;
  M.HD = HD;
  M.NSP = uni(A.t_attn.max_spans);
  M.L = L;
  M.D = uni(A.emb.D);

  // ---- temporal layers ----
  int nvalid, excl;
  window_of(uni(A.t_attn), 0, nvalid, excl);
  const int nspan = n_spans(uni(A.t_attn), nvalid);
  for (int l = 0; l < L; ++l) {
    GEMV(PRO_NORM, EPI_QKV, t_qkv(l));
    if (grid_sync(g)) return;
    {
      // each head's window split into nspan key spans, one per workgroup
      // (the per-operation kernel's split); the span partials (or, with one
      // span, the output) are flagged vectors
      AttnArgs at = uni(A.t_attn);
      at.layer_off = (int64_t)l * t_lel;
      for (int item = wg; item < H * nspan; item += nwg) {
        const int h = item / nspan, j = item % nspan;
        auto put = [&](int t, double Mv, double Lv, double Ov, bool direct) {
          if (direct) {
            const double o = Lv > 0.0 ? Ov / Lv : 0.0;
            ll_put(c, M.TO(l) + (uint32_t)(h * HD + t), stored_bits<T>(o));
          } else {
            const uint32_t pw = M.TP(l, h, j);
            ll_put_f64(c, pw + 4 + 2 * (uint32_t)t, Ov);
            if (t == 0) {
              ll_put_f64(c, pw, Mv);
              ll_put_f64(c, pw + 2, Lv);
            }
          }
        };
        attn_span<T, HD, NT, true>(at, h, 0, j * nvalid / nspan, (j + 1) * nvalid / nspan, nvalid,
                                   excl, s_o, nullptr, nspan == 1, put);
      }
    }
    // the workgroups of a head's spans merge its partials, each for its
    // share of the output dims; then the output projection's first batch
    if (nspan > 1)
      for (int item = wg; item < H * nspan; item += nwg) {
        const int h = item / nspan, j = item % nspan;
        (void)ll_span_merge<T, HD>(c, M, l, h, nspan, j * HD / nspan, (j + 1) * HD / nspan);
      }
    gemv_prefetch<T, KW, EPI_RESID, GU>(t_o(l), wg, nwg, pf);
    {
      // output projection, its input polled from the flagged O[l] (no grid
      // barrier after the attention; a timed-out wait raises the abort flag,
      // which ends the launch at the next barrier)
      ++g.tshift;
      auto ib = [&](T* xs_) {
        (void)ll_input_direct<T, NT>(t_o(l), c, M.TO(l), xs_);
        if (trace != nullptr && wg == 0 && tid() == 0)
          *(MOSHI_GLB uint64_t*)(trace + g.idx + g.tshift) = wall_clock64();
      };
      gemv_core<T, KW, PRO_DIRECT, EPI_RESID, true, GU, true, 4>(t_o(l), wg, nwg, xs, pf, s_rope, ib);
    }
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

  // ---- 16 substeps: the operations hand on flagged vectors, no grid barriers ----
  const int nqkv = 3 * Dd / 16;  // q/k/v tiles; head h's attention runs on workgroup (nqkv + h) % nwg
  unsigned tix = g.idx + g.tshift;  // trace entry of the last operation's end
  auto stamp = [&]() -> uint64_t* {
    ++tix;
    return trace != nullptr ? trace + tix : nullptr;
  };
  // the next operation's weight slice, requested by each projection once its
  // own slice is in registers
  auto st_qkv = [&](int s_, int l_) {
    return [&, s_, l_]() { gemv_stage<T, KW, EPI_QKV>(d_qkv(s_, l_), wg, nwg, wbuf); };
  };
  auto st_o = [&](int s_, int l_) {
    return [&, s_, l_]() { gemv_stage<T, KW, EPI_RESID>(d_o(s_, l_), wg, nwg, wbuf); };
  };
  auto st_gu = [&](int s_, int l_) {
    return [&, s_, l_]() { gemv_stage<T, KW, EPI_SWIGLU>(d_gu(s_, l_), wg, nwg, wbuf); };
  };
  auto st_dn = [&](int s_, int l_) {
    return [&, s_, l_]() { gemv_stage<T, KW, EPI_RESID>(d_dn(s_, l_), wg, nwg, wbuf); };
  };
  auto st_head = [&](int s_) {
    return [&, s_]() { gemv_stage<T, KW, EPI_ARGMAX>(d_head(s_), wg, nwg, wbuf); };
  };
  for (int s = 0; s < S_run; ++s) {
    for (int l = 0; l < Ld; ++l) {
      LLIo io{};
      io.q = M.Q(s, l);
      io.k = M.K(s, l);
      io.v = M.V(s, l);
      if (l == 0) {
        // the substep's entry (previous token -> residual) is folded into its
        // first q/k/v projection: every workgroup forms the normed input
        // itself; workgroup 0 stores the residual Y and the token
        EntryLL E;
        E.text_part = s == 0 ? uni(A.apart) : nullptr;
        E.ap = s == 0 ? 0 : M.AP(s - 1, S);
        E.prev_rows = s == 0 ? uni(A.Vt) : Va;
        E.pre = uni(A.pre) + (size_t)s * Dd;
        E.table = tab(o_de + s);
        E.y = M.Y(s, S);
        E.tok_out = s == 0 ? text_out : codes_out + (s - 1);
        E.forced = forced != nullptr ? forced + s : nullptr;
        // at s = 0 the grid barrier after the input projections ended the
        // previous operation
        if (!ll_gemv<T, KW, PRO_NORM, EPI_QKV, LLR_QKV_I, LLR_QKV_C, false, true>(
                d_qkv(s, 0), c, io, wg, nwg, xs, wbuf, &E, s == 0 ? nullptr : stamp(), st_o(s, 0)))
          return;
      } else {
        io.x = M.R2(s, l - 1);
        io.ss = M.S2(s, l - 1);
        if (!ll_gemv<T, KW, PRO_NORM, EPI_QKV, LLR_QKV_I, LLR_QKV_C, false>(
                d_qkv(s, l), c, io, wg, nwg, xs, wbuf, nullptr, stamp(), st_o(s, l)))
          return;
      }
      for (int h = 0; h < Hd; ++h)
        if ((nqkv + h) % nwg == wg &&
            !ll_dep_attention<T, HDD, NT>(c, M, s, l, h, s == ref_excl_at ? 0 : -1))
          return;
      io = LLIo{};
      io.x = M.O(s, l);
      io.resid = l == 0 ? M.Y(s, S) : M.R2(s, l - 1);
      io.out = M.R1(s, l);
      io.out_ss = M.S1(s, l);
      if (!ll_gemv<T, KW, PRO_DIRECT, EPI_RESID, LLR_O_I, LLR_O_C, false>(
              d_o(s, l), c, io, wg, nwg, xs, wbuf, nullptr, stamp(), st_gu(s, l)))
        return;
      io = LLIo{};
      io.x = M.R1(s, l);
      io.ss = M.S1(s, l);
      io.out = M.A(s, l);
      if (!ll_gemv<T, KW, PRO_NORM, EPI_SWIGLU, LLR_GU_I, LLR_GU_C, false>(
              d_gu(s, l), c, io, wg, nwg, xs, wbuf, nullptr, stamp(), st_dn(s, l)))
        return;
      io = LLIo{};
      io.x = M.A(s, l);
      io.resid = M.R1(s, l);
      io.out = M.R2(s, l);
      io.out_ss = M.S2(s, l);
      bool ok;
      if (l + 1 < Ld)
        ok = ll_gemv<T, KW, PRO_DIRECT, EPI_RESID, LLR_DN_I, LLR_DN_C, false>(
            d_dn(s, l), c, io, wg, nwg, xs, wbuf, nullptr, stamp(), st_qkv(s, l + 1));
      else
        ok = ll_gemv<T, KW, PRO_DIRECT, EPI_RESID, LLR_DN_I, LLR_DN_C, false>(
            d_dn(s, l), c, io, wg, nwg, xs, wbuf, nullptr, stamp(), st_head(s));
      if (!ok) return;
    }
    LLIo io{};
    io.x = M.R2(s, Ld - 1);
    io.ss = M.S2(s, Ld - 1);
    io.out = M.AP(s, S);
    // the head reads the rounded residual, or with the final norm its
    // RMSNorm (same input path as a normed projection)
    auto head = [&](auto next) {
      if (dep_final_norm)
        return ll_gemv<T, KW, PRO_NORM, EPI_ARGMAX, LLR_HD_I, LLR_HD_C, true>(
            d_head(s), c, io, wg, nwg, xs, wbuf, nullptr, stamp(), next);
      return ll_gemv<T, KW, PRO_CAST, EPI_ARGMAX, LLR_HD_I, LLR_HD_C, true>(
          d_head(s), c, io, wg, nwg, xs, wbuf, nullptr, stamp(), next);
    };
    const bool ok = s + 1 < S_run ? head(st_qkv(s + 1, 0)) : head([]() {});
    if (!ok) return;
  }
#undef GEMV
#undef GEMV_S
#undef PREFETCH_SYNC
#undef STAGE_SYNC
#undef PREFETCH_SYNC_G
  // ---- last code (forced if asked), codes of substeps not run, next position ----
  if (wg == 0) {
    bool ok;
    int tok = ll_reduce_token<NT>(c, M.AP(S_run - 1, S), 8 * M.nta, Va, ok);
    if (forced != nullptr) {
      const int f = ldg(forced + S_run);
      tok = f >= 0 ? f : tok;
    }
    uint64_t* st = stamp();
    for (int k = S_run + (int)threadIdx.x; k < S; k += NT) *(MOSHI_GLB int*)(codes_out + k) = -1;
    if (threadIdx.x == 0) {
      if (st != nullptr) *(MOSHI_GLB uint64_t*)st = wall_clock64();
      *(MOSHI_GLB int*)(codes_out + S_run - 1) = tok;
      int64_t* pos = uni(A.pos);
      if (ldg(uni(A.live))) *(MOSHI_GLB int64_t*)pos += 1;
      if (trace != nullptr) *(MOSHI_GLB uint64_t*)(trace + tix + 1) = wall_clock64();
    }
  }
}

template <typename T, int HD, int HDD>
hipError_t launch_t(const StepArgs* dP, const int* frames, int* text_out, int* codes_out,
                    int parity, uint32_t seq, int nwg, size_t lds, hipStream_t st,
                    uint64_t* trace) {
  void* args[] = {(void*)&dP,     (void*)&frames, (void*)&text_out, (void*)&codes_out,
                  (void*)&parity, (void*)&seq,    (void*)&trace};
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
  // one workgroup per CU (a grid barrier takes at most BW_MAXWG workgroups)
  return per_cu > 0 ? (ncu < BW_MAXWG ? ncu : 0) : 0;
}

// ===========================================================================
// The depformer of two or more sessions as one persistent kernel
// ===========================================================================
// At 2..64 sessions every depformer operation is a small MFMA product (a few
// MB of weights, 16-64 columns), and the ~45 dependent operations per substep
// cost a kernel launch each (~700 per frame). Here they are grid-stride
// phases of one cooperative launch, separated by the grid barrier above. Each
// phase runs the per-operation kernels' device code (gemm_tile, entry_item,
// dep_attention) with the thread counts its arithmetic depends on (KW waves
// per projection tile), so every value is bit-identical to the per-operation
// path. Data written in one phase and read in a later one use coherent
// accesses (C = true). (Building each tile's normed input itself instead of
// a norm phase was measured slower: every workgroup then re-reads its
// columns' fp64 residual, ~24 MB of coherent loads per phase at 16 sessions.)

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <typename T, int HDD, int KW>
__global__ __launch_bounds__(64 * KW) void dep_multi_kernel(const DepMultiArgs* P, int parity,
                                                            uint64_t* trace) {
  constexpr int NTH = 64 * KW;
  constexpr int NW = KW;
  extern __shared__ __align__(16) unsigned char s_dyn[];  // the weight pointer table
  __shared__ __align__(16) DepMultiArgs sA;
  __shared__ f64x4 s_acc[KW * 2 * 64];  // two row tiles per wave: the gate/up
  __shared__ double s_red[NW];
  __shared__ double s_v[NW];
  __shared__ int s_i[NW];
  {
    const uint32_t* src = (const uint32_t*)P;
    uint32_t* dst = (uint32_t*)&sA;
    for (int i = tid(); i < (int)(sizeof(DepMultiArgs) / 4); i += NTH) dst[i] = ldg(src + i);
  }
  __syncthreads();
  const DepMultiArgs& A = sA;
  const void** s_tab = (const void**)s_dyn;
  {
    const void* const* tab = uni(A.tab);
    const int n_tab = uni(A.n_tab);
    for (int i = tid(); i < n_tab; i += NTH) s_tab[i] = ldg(tab + i);
  }
  __syncthreads();
  auto tab = [&](int i) { return uni(s_tab[i]); };
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int S = uni(A.S), S_run = uni(A.S_run), Ld = uni(A.Ld), Va = uni(A.Va), B = uni(A.B);
  const int o_dw = uni(A.o_dw), o_dn = uni(A.o_dn), o_de = uni(A.o_de), o_dh = uni(A.o_dh);
  const int64_t d_lel = uni(A.d_layer_elems);
  const int* const live = uni(A.live);
  const int* const forced = uni(A.forced);
  const int nch = uni(A.nch);
  // the input projections' first weight batch, requested before the start barrier
  u32x4 wpf[GEMM_U];
  {
    const GemmArgs a = uni(A.d_in);
    int tl, c0, ksg;
    gemm_item(a, EPI_STORE, wg, tl, c0, ksg);
    if (wg < gemm_items(a, EPI_STORE)) gemm_tile_weights<T, KW, EPI_STORE>(a, tl, 0, wpf, ksg);
  }
  Grid g;
  if (grid_init(g, uni(A.bar), parity, uni(A.abort), uni(A.spin_limit), trace, false)) return;
#define DM_SYNC()               \
  do {                          \
    if (grid_sync(g)) return;   \
  } while (0)

  // projection items: (row tile, 16-column block, K segment) (gemm_item);
  // the blocks of one tile are nt items apart, so with nt a multiple of 8
  // they run on the same XCD and share its L2 copy of the tile's weights.
  // The first item's first weight batch was requested during the barrier
  // before the phase (sync_pf).
  auto gemm_phase = [&](auto epi_c, const GemmArgs& a) {
    constexpr int EPI = decltype(epi_c)::value;
    const int n = gemm_items(a, EPI);
    for (int item = wg; item < n; item += nwg) {
      int tl, c0, ksg;
      gemm_item(a, EPI, item, tl, c0, ksg);
      gemm_tile<T, 1, KW, EPI, true, true>(a, tl, c0, s_acc, item == wg ? wpf : nullptr, ksg);
      __syncthreads();
    }
  };
  // A gate/up with more items than workgroups: items of two row tiles (each
  // wave sums both over its k-steps, sharing every input group's conversion;
  // the values are those of one tile per item), so no workgroup runs two
  // items one after the other. Single batches: no prefetched first batch.
  auto gu_pairs = [&](const GemmArgs& a) {
    const int nt = n_tiles_of(EPI_SWIGLU, a.N), ncb = (a.B + 15) / 16;
    return a.ksplit <= 1 && nt * ncb > nwg;
  };
  auto gemm_phase_gu = [&](const GemmArgs& a) {
    if (!gu_pairs(a)) {
      gemm_phase(IntC<EPI_SWIGLU>{}, a);
      return;
    }
    const int nt = n_tiles_of(EPI_SWIGLU, a.N), nt2 = (nt + 1) / 2, ncb = (a.B + 15) / 16;
    for (int item = wg; item < nt2 * ncb; item += nwg) {
      gemm_tile<T, 1, KW, EPI_SWIGLU, false, true, 2>(a, (item % nt2) * 2, (item / nt2) * 16, s_acc);
      __syncthreads();
    }
  };
  // grid barrier; in between its two halves this workgroup requests the first
  // weight batch of its first tile of the projection `next` (weights do not
  // depend on the phase that ends). True: leave (abort).
  auto sync_pf = [&](auto epi_c, const GemmArgs& next) {
    constexpr int EPI = decltype(epi_c)::value;
    drain_stores();
    __syncthreads();
    const unsigned old = grid_arrive(g);
    int tl, c0, ksg;
    gemm_item(next, EPI, wg, tl, c0, ksg);
    if (wg < gemm_items(next, EPI)) gemm_tile_weights<T, KW, EPI>(next, tl, 0, wpf, ksg);
    return grid_wait(g, old);
  };
  // rounded (normed) input vectors, one column per workgroup; the projection
  // then reads them as its input
  auto norm_phase = [&](auto pro_c, const GemmArgs& a) {
    constexpr int PRO = decltype(pro_c)::value;
    for (int b = wg; b < a.B; b += nwg) norm_column<T, PRO, true, NTH>(a, b, s_red);
  };
  auto normed = [&](GemmArgs a) {
    a.X = a.xn_out;
    a.ldx = a.K;
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
    GemmArgs a = uni(A.d_head);  // with the final norm: its gain and sums of squares set
    a.W = tab(o_dh + s);
    a.logits += (size_t)s * Va;
    return a;
  };
  const bool final_norm = uni(A.dep_final_norm) != 0;
  const int ref_excl_at = uni(A.ref_excl_at);

  // ---- input projections of every substep run ----
  gemm_phase(IntC<EPI_STORE>{}, uni(A.d_in));
  DM_SYNC();
  for (int s = 0; s < S_run; ++s) {
    {  // entry: y = pre[s] + E_s[previous token]; from s = 1 on the previous
       // head's partials are reduced here (or the forced code taken) and code
       // s - 1 is stored
      EntryArgs e = uni(A.entry);
      e.s = s;
      e.table = tab(o_de + s);
      e.prev = s == 0 ? uni(A.tokens) : uni(A.codes) + (s - 1);
      e.prev_stride = s == 0 ? 1 : S;
      e.prev_part = s == 0 ? nullptr : uni(A.apart);
      e.forced = s == 0 ? nullptr : forced;
      e.forced_stride = nch;
      e.forced_col = s;
      const int nbx = (e.D + 15) / 16, nby = (e.B + 3) / 4;
      for (int item = wg * NW + (tid() >> 6); item < nbx * nby; item += nwg * NW)
        entry_item<T, true>(e, item % nbx, item / nbx, tid() & 63);
    }
    DM_SYNC();
    for (int l = 0; l < Ld; ++l) {
      norm_phase(IntC<PRO_NORM>{}, d_qkv(s, l));
      if (sync_pf(IntC<EPI_QKV>{}, d_qkv(s, l))) return;
      gemm_phase(IntC<EPI_QKV>{}, normed(d_qkv(s, l)));
      DM_SYNC();
      {  // causal attention over substeps 0..s, NW heads of one slot per item
        AttnArgs at = uni(A.d_attn);
        at.layer_off = (int64_t)l * d_lel;
        const int Hd = at.n_heads;
        const int nhc = (Hd + NW - 1) / NW;
        for (int item = wg; item < B * nhc; item += nwg) {
          const int b = item / nhc, h0 = (item % nhc) * NW;
          if (!ldg(live + b)) continue;
          dep_attention<T, HDD, NTH, true, 1>(at, b, h0, Hd - h0 < NW ? Hd - h0 : NW, s + 1,
                                              s == ref_excl_at ? 0 : -1);
        }
      }
      if (sync_pf(IntC<EPI_RESID>{}, d_o(s, l))) return;
      gemm_phase(IntC<EPI_RESID>{}, d_o(s, l));
      DM_SYNC();
      norm_phase(IntC<PRO_NORM>{}, d_gu(s, l));
      if (gu_pairs(d_gu(s, l)) ? grid_sync(g) : sync_pf(IntC<EPI_SWIGLU>{}, d_gu(s, l))) return;
      gemm_phase_gu(normed(d_gu(s, l)));
      if (sync_pf(IntC<EPI_RESID>{}, d_dn(s, l))) return;
      gemm_phase(IntC<EPI_RESID>{}, d_dn(s, l));
      DM_SYNC();
    }
    // head s on the rounded residual, or with the final-norm reading on its RMSNorm
    if (final_norm)
      norm_phase(IntC<PRO_NORM>{}, d_head(s));
    else
      norm_phase(IntC<PRO_CAST>{}, d_head(s));
    if (sync_pf(IntC<EPI_ARGMAX>{}, d_head(s))) return;
    gemm_phase(IntC<EPI_ARGMAX>{}, normed(d_head(s)));
    DM_SYNC();
  }
#undef DM_SYNC
  // ---- the last code (forced if asked); free slots and substeps not run read -1 ----
  {
    const ArgPart* ap = uni(A.apart);
    int* codes = uni(A.codes);
    int* tokens = uni(A.tokens);
    const int nt = (Va + 15) / 16;
    for (int b = wg; b < B; b += nwg) {
      double bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int i = tid(); i < nt; i += NTH) {
        const ArgPart p = unpack_part(ld_grp<true>(ap + (size_t)i * B + b));
        if (arg_better(p.v, p.i, bv, bi)) {
          bv = p.v;
          bi = p.i;
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double ov = shfl_xor_d(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (arg_better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((tid() & 63) == 0) {
        s_v[tid() >> 6] = bv;
        s_i[tid() >> 6] = bi;
      }
      __syncthreads();
      const bool lv = ldg(live + b) != 0;
      if (tid() == 0) {
        for (int w = 1; w < NW; ++w)
          if (arg_better(s_v[w], s_i[w], bv, bi)) {
            bv = s_v[w];
            bi = s_i[w];
          }
        int r = bi < Va ? bi : 0;
        if (forced != nullptr) {
          const int f = ldg(forced + (size_t)b * nch + S_run);
          if (f >= 0) r = f;
        }
        *(MOSHI_GLB int*)(codes + (size_t)b * S + S_run - 1) = lv ? r : -1;
        if (!lv) *(MOSHI_GLB int*)(tokens + b) = -1;
      }
      for (int k = tid(); k < S; k += NTH)
        if (!lv || k >= S_run) *(MOSHI_GLB int*)(codes + (size_t)b * S + k) = -1;
      __syncthreads();
    }
  }
  if (trace != nullptr && wg == 0 && tid() == 0)
    *(MOSHI_GLB uint64_t*)(trace + g.idx + 1) = wall_clock64();
}

template <typename T, int HDD, int KW>
int dep_multi_grid_t(size_t lds) {
  int per_cu = 0, dev = 0, ncu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dep_multi_kernel<T, HDD, KW>, 64 * KW,
                                                   lds) != hipSuccess)
    return 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  // one workgroup of 8 waves per CU; two of 4 waves where they fit
  const int want = KW == 4 ? 2 : 1;
  const int n = per_cu < 1 ? 0 : ncu * (per_cu < want ? per_cu : want);
  return n <= BW_MAXWG ? n : 0;  // a grid barrier takes at most BW_MAXWG workgroups
}

template <typename T, int HDD, int KW>
hipError_t launch_dep_multi_t(const DepMultiArgs* dP, int parity, int nwg, size_t lds,
                              hipStream_t st, uint64_t* trace) {
  void* args[] = {(void*)&dP, (void*)&parity, (void*)&trace};
  return hipLaunchCooperativeKernel((const void*)dep_multi_kernel<T, HDD, KW>, dim3(nwg),
                                    dim3(64 * KW), args, (unsigned)lds, st);
}

// Waves per projection tile: the per-operation path's (8 up to 32 sessions,
// 4 at 33..64; see launch_gemm).
int dep_multi_kw(int B) { return B <= 32 ? 8 : 4; }

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
                       int* text_out, int* codes_out, int parity, uint32_t seq, int nwg,
                       size_t lds, hipStream_t st, uint64_t* trace) {
  if (dtype == DT_BF16 && hd == 128 && hdd == 64)
    return launch_t<__bf16, 128, 64>(dP, frames, text_out, codes_out, parity, seq, nwg, lds, st,
                                      trace);
  if (dtype == DT_F32 && hd == 64 && hdd == 32)
    return launch_t<float, 64, 32>(dP, frames, text_out, codes_out, parity, seq, nwg, lds, st,
                                     trace);
  return hipErrorInvalidValue;
}

// Instantiated: bf16 with depformer head dim 64, fp32 with 32.
bool dep_multi_supported(int dtype, int hdd) {
  return (dtype == DT_BF16 && hdd == 64) || (dtype == DT_F32 && hdd == 32);
}

int dep_multi_grid(int dtype, int hdd, int B, size_t lds) {
  const int kw = dep_multi_kw(B);
  if (dtype == DT_BF16 && hdd == 64)
    return kw == 8 ? dep_multi_grid_t<__bf16, 64, 8>(lds) : dep_multi_grid_t<__bf16, 64, 4>(lds);
  if (dtype == DT_F32 && hdd == 32)
    return kw == 8 ? dep_multi_grid_t<float, 32, 8>(lds) : dep_multi_grid_t<float, 32, 4>(lds);
  return 0;
}

hipError_t launch_dep_multi(int dtype, int hdd, int B, const DepMultiArgs* dP, int parity, int nwg,
                            size_t lds, hipStream_t st, uint64_t* trace) {
  const int kw = dep_multi_kw(B);
  if (dtype == DT_BF16 && hdd == 64)
    return kw == 8 ? launch_dep_multi_t<__bf16, 64, 8>(dP, parity, nwg, lds, st, trace)
                   : launch_dep_multi_t<__bf16, 64, 4>(dP, parity, nwg, lds, st, trace);
  if (dtype == DT_F32 && hdd == 32)
    return kw == 8 ? launch_dep_multi_t<float, 32, 8>(dP, parity, nwg, lds, st, trace)
                   : launch_dep_multi_t<float, 32, 4>(dP, parity, nwg, lds, st, trace);
  return hipErrorInvalidValue;
}

}  // namespace moshi
