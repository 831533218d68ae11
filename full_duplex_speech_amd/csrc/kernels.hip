// kernels.hip -- gfx950 kernels of the Moshi/PersonaPlex frame step.
//
// Model (pages): mobius PR #368 "P2 - Moshi LM" (RMSNorm eps 1e-8, RoPE theta
// 1e4, sliding-window causal attention, fused gate/up SwiGLU, depformer with
// per-substep linears, no RoPE, causal over substeps); vLLM-Omni recipe
// "PersonaPlex", "Architecture" (3000-frame ring window, 17-row token column).
//
// Numerics: weights, embeddings, K/V and every vector that feeds a projection
// are stored in the model dtype (bf16 or fp32); all arithmetic is fp64, and a
// stored bf16 value is the nearest-even rounding of the fp64 result. This is
// what keeps every rounding decision equal to an fp64 evaluation of the
// model: with fp32 accumulation a single flipped bf16 rounding spreads through
// the next dense projection into many more flips, and after 32 layers the
// logits drift by several 1e-2.
//
// Kernels:
//  * gemv_kernel (one session): every projection. Weights stream from HBM
//    once in 16-byte loads; a workgroup owns 16 output rows, its waves split K,
//    each lane keeps its slice of the input vector in registers and
//    accumulates in fp64; lanes and waves reduce in a fixed order. The
//    prologue fuses the RMSNorm (from per-tile sums of squares written by the
//    producer of the residual) and the bf16 rounding of the input.
//  * gemm_kernel (two or more sessions): the same projections as fp64 MFMA
//    16x16x4 tiles (16 weight rows x 16 session columns), input vectors
//    pre-normalised by norm_kernel.
//  * epilogues shared by both: RoPE + ring write, residual add + sums of
//    squares, SiLU(gate)*up, argmax partials.
//  * attn_kernel / attn_combine_kernel: sliding-window decode attention over
//    the per-slot ring, one workgroup per (64-key chunk, head, slot), chunks
//    merged in a fixed order.
//  * embed_kernel / entry_kernel: summed channel embedding and depformer
//    substep entry.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dev.h"
#include "kernels.h"

namespace moshi {

// One session: every projection (see gemv_body).
template <typename T, int KW, int PRO, int EPI>
__global__ __launch_bounds__(64 * KW) void gemv_kernel(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char s_dyn[];  // rounded input, K elements
  gemv_body<T, KW, PRO, EPI, false>(a, blockIdx.x, gridDim.x, (T*)s_dyn);
}

// ---------------------------------------------------------------------------
// Two to four sessions, temporal projections: fp64 FMA over 16-row tiles
// ---------------------------------------------------------------------------

// A 16-column MFMA tile with two to four live columns spends most of its
// matrix work on empty columns; here each weight group is read once and
// multiplied into every session's rounded input (LDS, model dtype, columns
// past B zero) on the VALU. One workgroup of 8 waves takes row tiles
// blockIdx.x, + gridDim.x, ... (the MFMA path's row mapping, tile_row), up
// to MT of them per pass over K: wave w holds tile rows 2w, 2w + 1 of each,
// one group per lane and row per batch, double-buffered, and widens each
// input group once for all of them. Each row's sums are reduced over the 64
// lanes (a lane sums its groups in K order); the tiles' 16 x NC sums go
// through LDS to wave 0, which runs the MFMA path's epilogue in its lane
// layout (lane 16 g + c: rows 4g..4g+3 of column c), so every output,
// partial and ring write has that path's layout. (Inputs kept as fp64 in
// LDS instead measured slower: LDS bound.)
template <typename T, int NC, int EPI, int MT>
__global__ __launch_bounds__(512) void gemv_cols_kernel(GemmArgs a) {
  constexpr int VEC = VecOf<T>::N, R = 2;
  extern __shared__ __align__(16) unsigned char s_dyn[];
  T* xs = (T*)s_dyn;  // [NC][K]
  __shared__ double s_sum[MT][16][NC];
  const int t = tid(), lane = t & 63, wave = t >> 6;
  const int ngroups = a.K / VEC;  // K is a multiple of VEC
  const int ntiles = n_tiles_of(EPI, a.N);
  const int nb = (ngroups + 63) / 64;  // batches: group b * 64 + lane
  // the pass starting at tile t0 takes tiles t0 + m * gridDim.x, m < nm
  auto n_in_pass = [&](int t0) {
    const int n = (ntiles - t0 + (int)gridDim.x - 1) / (int)gridDim.x;
    return n < MT ? n : MT;
  };
  // Every batch loads all MT x R rows with no branch around the loads (a
  // tile past the end, m >= nm, re-reads tile t0's rows; a batch past K the
  // row's last group; neither sum is used), so the compiler knows how many
  // loads are younger than the batch being consumed and waits for that
  // batch only: with branches around them (or a break between the two
  // batches of a loop trip) it waited for all of them, the next batch
  // included, and batches cost a full memory round trip each.
  const T* wr[MT][R];
  auto set_rows = [&](int t0, int nm) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        bool ok;
        const int row = tile_row<EPI>(m < nm ? t0 + m * (int)gridDim.x : t0, 2 * wave + r, a.N, ok);
        wr[m][r] = (const T*)a.W + (size_t)(ok ? row : 0) * a.K;
      }
  };
  auto load = [&](int b, u32x4 (&w)[MT][R]) {
    const int gi = b * 64 + lane;
    const int gc = gi < ngroups ? gi : ngroups - 1;  // past K: the row's last group, unused
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) w[m][r] = ld16_stream(wr[m][r] + (size_t)gc * VEC);
  };
  // The first pass's first weight batch is requested before the inputs are
  // staged (the grid is at most the tile count, so every workgroup has a
  // tile), and the staging requests SU groups per thread before it stores
  // any: one memory round trip before the products instead of one per
  // staging round plus one for the weights.
  u32x4 wa[MT][R], wb[MT][R];
  int t0 = blockIdx.x;
  int nm = n_in_pass(t0);
  set_rows(t0, nm);
  load(0, wa);
  {
    constexpr int SU = 4;
    const int nx = NC * ngroups;
    for (int i0 = t; i0 < nx; i0 += SU * 512) {
      u32x4 v[SU];
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        const int i = i0 + u * 512 < nx ? i0 + u * 512 : nx - 1;
        const int c = i / ngroups, gi = i - c * ngroups;
        v[u] = c < a.B ? ld16((const T*)a.X + (size_t)c * a.ldx + (size_t)gi * VEC)
                       : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        const int i = i0 + u * 512;
        if (i < nx) {
          const int c = i / ngroups, gi = i - c * ngroups;
          *(u32x4*)(xs + (size_t)c * a.K + (size_t)gi * VEC) = v[u];
        }
      }
    }
  }
  __syncthreads();
  for (; t0 < ntiles; t0 += MT * gridDim.x) {
    if (t0 != (int)blockIdx.x) {
      nm = n_in_pass(t0);
      set_rows(t0, nm);
      load(0, wa);
    }
    double acc[MT][R][NC];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[m][r][c] = 0.0;
    auto consume = [&](int b, const u32x4 (&w)[MT][R]) {
      const int gi = b * 64 + lane;
      if (gi < ngroups) {
        double xv[NC][VEC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
          widen<T>(*(const u32x4*)(xs + (size_t)c * a.K + (size_t)gi * VEC), xv[c]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < nm)
#pragma unroll
            for (int r = 0; r < R; ++r) {
              double wd[VEC];
              widen<T>(w[m][r], wd);
#pragma unroll
              for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[m][r][c] = fma(wd[e], xv[c][e], acc[m][r][c]);
            }
      }
    };
    // whole pairs of batches, without a break between them (a batch past the
    // last consumes nothing: every lane's group is past K)
    for (int b = 0; b < nb; b += 2) {
      load(b + 1, wb);
      consume(b, wa);
      load(b + 2, wa);
      consume(b + 1, wb);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < nm)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const double v = group_reduce<64>(acc[m][r][c]);
            if (lane == 0) s_sum[m][2 * wave + r][c] = v;
          }
    __syncthreads();
    if (wave == 0) {
      const int g = lane >> 4, c = lane & 15;
      for (int m = 0; m < nm; ++m) {
        double v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = c < NC ? s_sum[m][4 * g + i][c] : 0.0;
        epilogue<T, EPI, false>(a, t0 + m * (int)gridDim.x, g, c, v);  // columns past B store nothing
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Two or more sessions: fp64 MFMA 16x16x4 tiles
// ---------------------------------------------------------------------------

// 16 RT weight rows x 16 NB session columns per workgroup (see gemm_tile);
// K segment blockIdx.y of a.ksplit.
template <typename T, int NB, int KW, int EPI, bool DB, int RT = 1, int U = GEMM_U>
__global__ __launch_bounds__(64 * KW) void gemm_kernel(GemmArgs a) {
  __shared__ f64x4 s_acc[KW * RT * NB * 64];
  gemm_tile<T, NB, KW, EPI, DB, false, RT, U>(a, blockIdx.x * RT, 0, s_acc, nullptr, blockIdx.y);
}

// Input vectors for the MFMA path: xn[b][k] = round(x[b][k] * scale_b * g[k])
// (PRO_NORM) or round(x[b][k]) (PRO_CAST); one workgroup per column.
// (column blockIdx.x, elements [1024 blockIdx.y, 1024 blockIdx.y + 1024))
template <typename T, int PRO>
__global__ __launch_bounds__(256) void norm_kernel(GemmArgs a) {
  __shared__ double s_tmp[4];
  norm_column<T, PRO, false, 256>(a, blockIdx.x, s_tmp, blockIdx.y * 1024, blockIdx.y * 1024 + 1024);
}

// Greedy token of column blockIdx.x from per-tile (max, index) partials.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const ArgPart* part, int n_tiles,
                                                            int n_rows, int B, int* tok,
                                                            int stride, const int* forced,
                                                            int forced_stride, int forced_col) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ double s_v[4];
  __shared__ int s_i[4];
  double bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = t; i < n_tiles; i += 256) {
    const ArgPart p = part[(size_t)i * B + b];
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
  if ((t & 63) == 0) {
    s_v[t >> 6] = bv;
    s_i[t >> 6] = bi;
  }
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < 4; ++w)
      if (arg_better(s_v[w], s_i[w], bv, bi)) {
        bv = s_v[w];
        bi = s_i[w];
      }
    int r = (bi < n_rows) ? bi : 0;
    if (forced != nullptr) {
      const int f = forced[(size_t)b * forced_stride + forced_col];
      if (f >= 0) r = f;
    }
    tok[(size_t)b * stride] = r;
  }
}

// ---------------------------------------------------------------------------
// Temperature + top-k sampling (SGLang-Omni cookbook "PersonaPlex", "Request
// parameters": text 0.7 / 25, audio 0.8 / 250, a seed with a child stream per
// head; mobius PR #368's sampling commit)
// ---------------------------------------------------------------------------

// splitmix64 (Steele, Lea and Flood, OOPSLA 2014): output n of a generator
// seeded with `seed` is this mix of seed + n * gamma.
__device__ __forceinline__ uint64_t sm64(uint64_t seed, uint64_t n) {
  uint64_t z = seed + n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The draw in [0, 1) of stream `stream` at position pos: output pos+1 of the
// generator seeded with the stream's child seed (output stream+1 of the
// session seed's generator), top 53 bits.
__device__ __forceinline__ double draw_uniform(uint64_t seed, int stream, int64_t pos) {
  const uint64_t child = sm64(seed, (uint64_t)stream + 1);
  return (double)(sm64(child, (uint64_t)pos + 1) >> 11) * 0x1.0p-53;
}

// fp32 value -> unsigned key with the same order (IEEE total order: -0
// below +0).
__device__ __forceinline__ uint32_t f32_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ double shfl_up_d(double v, int d) {
  return __hiloint2double(__shfl_up(__double2hiint(v), d), __shfl_up(__double2loint(v), d));
}

// Exclusive prefix of x over the workgroup's threads in thread order (waves
// scanned with shuffles, wave totals in order by thread 0); `total` gets the
// sum. Every thread calls it.
template <typename V, int NT>
__device__ __forceinline__ V block_exclusive(V x, V& total) {
  constexpr int NW = NT / 64;
  __shared__ V s_w[NW + 1];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  V inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    V y;
    if constexpr (sizeof(V) == 8) y = shfl_up_d(inc, off);
    else y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  V ex;
  if constexpr (sizeof(V) == 8) ex = shfl_up_d(inc, 1);
  else ex = __shfl_up(inc, 1);
  if (lane == 0) ex = V(0);
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  if (t == 0) {
    V acc = V(0);
    for (int i = 0; i < NW; ++i) {
      const V v = s_w[i];
      s_w[i] = acc;
      acc += v;
    }
    s_w[NW] = acc;
  }
  __syncthreads();
  const V r = s_w[w] + ex;
  total = s_w[NW];
  __syncthreads();
  return r;
}

// One workgroup per column b. The candidates are the top_k largest fp32
// logits (lowest index first among equal values), found by a 4-pass radix
// select of the k-th largest key and a prefix count of the keys equal to it;
// weights w_i = exp((l_i - l_max) / T) in fp64; each thread holds a
// contiguous run of indices, so an exclusive scan of the threads' sums in
// thread order gives every candidate's running sum in index order; the draw
// is the lowest index whose running sum exceeds u * (the total), or the last
// candidate if none does (the oracle's definition; only the rounding of the
// sums differs).
__global__ __launch_bounds__(SAMPLE_THREADS) void sample_kernel(SampleArgs a) {
  constexpr int NT = SAMPLE_THREADS, MC = SAMPLE_MAX_PER_THREAD;
  const int b = blockIdx.x, t = threadIdx.x;
  if (b >= a.B || !a.live[b]) return;
  if (a.forced != nullptr && a.forced[(size_t)b * a.forced_stride + a.forced_col] >= 0) return;
  const SampleParams& P = a.params[b];
  const double T = P.temperature[a.which];
  if (!(T > 0.0)) return;  // greedy: the argmax already written stands
  const int n = a.n;
  int k = P.top_k[a.which];
  if (k <= 0 || k >= n) k = n;
  const float* L = a.logits + (size_t)b * a.ld;
  const int c = (n + NT - 1) / NT;
  const int i0 = t * c;
  float val[MC];
#pragma unroll
  for (int j = 0; j < MC; ++j) val[j] = (j < c && i0 + j < n) ? L[i0 + j] : 0.0f;
  auto valid = [&](int j) { return j < c && i0 + j < n; };

  // the k-th largest key and how many keys equal to it are candidates
  __shared__ unsigned hist[256];
  __shared__ unsigned s_sel[2];
  uint32_t kth = 0, need_eq = 0;
  if (k < n) {
    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = t; i < 256; i += NT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < MC; ++j) {
        if (!valid(j)) continue;
        const uint32_t key = f32_key(val[j]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (t == 0) {
        uint32_t acc = 0;
        int bin = 255;
        for (; bin > 0; --bin) {
          if (acc + hist[bin] >= krem) break;
          acc += hist[bin];
        }
        s_sel[0] = (uint32_t)bin;
        s_sel[1] = krem - acc;
      }
      __syncthreads();
      prefix |= s_sel[0] << shift;
      pmask |= 0xffu << shift;
      krem = s_sel[1];
      __syncthreads();
    }
    kth = prefix;
    need_eq = krem;
  }
  // candidates: keys above kth, and the first need_eq keys equal to it
  unsigned my_eq = 0;
#pragma unroll
  for (int j = 0; j < MC; ++j)
    if (valid(j) && k < n && f32_key(val[j]) == kth) ++my_eq;
  unsigned eq_total;
  const unsigned eq_base = block_exclusive<unsigned, NT>(my_eq, eq_total);
  uint32_t member = 0;  // bit j: element j is a candidate
  {
    unsigned r = eq_base;
#pragma unroll
    for (int j = 0; j < MC; ++j) {
      if (!valid(j)) continue;
      const uint32_t key = f32_key(val[j]);
      bool m = true;
      if (k < n) {
        m = key > kth;
        if (key == kth) {
          m = r < need_eq;
          ++r;
        }
      }
      if (m) member |= 1u << j;
    }
  }
  // the largest value (always a candidate)
  __shared__ uint32_t s_kmax[NT / 64];
  uint32_t km = 0;
#pragma unroll
  for (int j = 0; j < MC; ++j)
    if (valid(j)) km = max(km, f32_key(val[j]));
  for (int off = 32; off > 0; off >>= 1) km = max(km, (uint32_t)__shfl_xor((int)km, off));
  if ((t & 63) == 0) s_kmax[t >> 6] = km;
  __syncthreads();
  km = s_kmax[0];
  for (int w = 1; w < NT / 64; ++w) km = max(km, s_kmax[w]);
  const double lmax = (double)key_f32(km);
  // weights, the threads' sums in index order, the draw
  double mine = 0.0;
#pragma unroll
  for (int j = 0; j < MC; ++j)
    if (member & (1u << j)) mine += exp(((double)val[j] - lmax) / T);
  double total;
  const double before = block_exclusive<double, NT>(mine, total);
  const double target = draw_uniform(P.seed, a.stream, ldg(a.pos + b) + a.pos_off) * total;
  int cand = 0x7fffffff, last = -1;
  double run = before;
#pragma unroll
  for (int j = 0; j < MC; ++j) {
    if (!(member & (1u << j))) continue;
    last = i0 + j;
    run += exp(((double)val[j] - lmax) / T);
    if (cand == 0x7fffffff && run > target) cand = i0 + j;
  }
  __shared__ int s_c[NT / 64], s_l[NT / 64];
  for (int off = 32; off > 0; off >>= 1) {
    cand = min(cand, __shfl_xor(cand, off));
    last = max(last, __shfl_xor(last, off));
  }
  if ((t & 63) == 0) {
    s_c[t >> 6] = cand;
    s_l[t >> 6] = last;
  }
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < NT / 64; ++w) {
      cand = min(cand, s_c[w]);
      last = max(last, s_l[w]);
    }
    a.out[(size_t)b * a.out_stride] = cand != 0x7fffffff ? cand : last;
  }
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t st) {
  if (a.n < 1 || a.n > SAMPLE_THREADS * SAMPLE_MAX_PER_THREAD) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_kernel, dim3(a.B), dim3(SAMPLE_THREADS), 0, st, a);
  return hipGetLastError();
}

// Outputs of free slots read -1, and so do the codes of substeps not run.
__global__ __launch_bounds__(64) void finish_outputs_kernel(int* tokens, int* codes,
                                                            const int* live, int B, int S,
                                                            int s_run) {
  const int b = blockIdx.x;
  const int s = threadIdx.x;
  if (b >= B) return;
  const bool lv = live[b] != 0;
  if (s == 0 && !lv) tokens[b] = -1;
  for (int k = s; k < S; k += 64)
    if (!lv || k >= s_run) codes[(size_t)b * S + k] = -1;
}

// ---------------------------------------------------------------------------
// Sliding-window decode attention over a ring of K/V
// ---------------------------------------------------------------------------

// One workgroup per (key span, head, slot); see attn_span. NTH = 512 with one
// session (the step kernel's workgroup shape, so both give identical bits);
// 256 with several, so that a few workgroups share a CU and hide each
// other's first-block latency.
template <typename T, int HD, int NTH>
__global__ __launch_bounds__(NTH) void attn_kernel(AttnArgs a) {
  __shared__ double s_w[span_lds_doubles<T, HD, NTH>()];
  const int span = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (!a.live[b]) return;
  int nvalid, excl;
  window_of(a, b, nvalid, excl);
  const int ns = n_spans(a, nvalid);
  if (span >= ns) return;
  double* part = a.part + (((size_t)b * a.n_heads + h) * a.max_spans + span) * (HD + 2);
  attn_span<T, HD, NTH, false>(a, h, b, span * nvalid / ns, (span + 1) * nvalid / ns, nvalid, excl,
                               s_w, part, ns == 1);
}

// Depformer attention of slot blockIdx.x, every head (see dep_attention).
template <typename T, int HD>
__global__ __launch_bounds__(512) void dep_attn_kernel(AttnArgs a) {
  const int b = blockIdx.x;
  if (!ldg(a.live + b)) return;
  dep_attention<T, HD, 512, false, 2>(a, b, 0, a.n_heads, a.scalar_nvalid, a.scalar_excl);
}

// Span merge of (slot blockIdx.y, head blockIdx.x); see combine_item.
template <typename T, int HD>
__global__ __launch_bounds__(HD) void attn_combine_kernel(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  if (!a.live[b]) return;
  int nvalid, excl;
  window_of(a, b, nvalid, excl);
  const int ns = n_spans(a, nvalid);
  if (ns <= 1) return;  // written directly by attn_kernel
  combine_item<T, HD, false>(a, h, b, ns);
}

// ---------------------------------------------------------------------------
// Summed channel embedding and depformer substep entry
// ---------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(64) void embed_kernel(EmbedArgs a) {
  const int r = threadIdx.x & 15;
  const int b = blockIdx.y * 4 + (threadIdx.x >> 4);
  const int row = blockIdx.x * 16 + r;
  double acc = 0.0;
  if (b < a.B && row < a.D) {
    const bool live = a.live[b] != 0;
    // rows requested 8 channels at a time; the sum runs in channel order
    for (int c0 = 0; c0 < a.n_ch; c0 += 8) {
      double v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = c0 + j;
        v[j] = 0.0;
        if (c < a.n_ch) {
          // Free slots embed code 0. A live code outside the table is clamped
          // to a valid row (never read out of bounds) and flagged for the host.
          int code = live ? a.frames[(size_t)b * a.n_ch + c] : 0;
          const int rows = (c == 0) ? a.rows_text : a.rows_audio;
          if (code < 0 || code >= rows) {
            if (row == 0) atomicOr(a.bad_code, 1);
            code = code < 0 ? 0 : rows - 1;
          }
          v[j] = to_d(((const T*)a.tables[c])[(size_t)code * a.D + row]);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + j < a.n_ch) acc += v[j];
    }
    a.x[(size_t)b * a.D + row] = acc;
  }
  double ss = acc * acc;
  for (int off = a.ssq_rows / 2; off > 0; off >>= 1) ss += shfl_xor_d(ss, off);
  if (r % a.ssq_rows == 0 && b < a.B && row < a.D) a.ssq_out[(size_t)(row / a.ssq_rows) * a.B + b] = ss;
}

// Depformer substep entry (see entry_item): one wave per 16 rows x 4 columns.
template <typename T>
__global__ __launch_bounds__(64) void entry_kernel(EntryArgs a) {
  entry_item<T, false>(a, blockIdx.x, blockIdx.y, threadIdx.x);
}

// End of a temporal step: every live slot moves to its next position.
__global__ __launch_bounds__(64) void advance_kernel(int64_t* pos, const int* live, int B) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b < B && live[b]) pos[b] += 1;
}

// Prefill copy: src [n][H*hd] (one layer) -> ring [H][cap][hd] of one slot.
template <typename T>
__global__ __launch_bounds__(256) void scatter_kernel(const T* src, T* ring, int n, int H, int hd,
                                                      int64_t head_stride) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t D = (int64_t)H * hd;
  if (e >= (int64_t)n * D) return;
  const int64_t j = e / D;
  const int64_t c = e - j * D;
  const int64_t h = c / hd;
  const int64_t d = c - h * hd;
  ring[h * head_stride + j * hd + d] = src[e];
}

// Ring read-back: ring [H][cap][hd] of one slot and layer -> dst [n][H*hd].
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* ring, T* dst, int n, int H, int hd,
                                                     int64_t head_stride) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t D = (int64_t)H * hd;
  if (e >= (int64_t)n * D) return;
  const int64_t j = e / D;
  const int64_t c = e - j * D;
  const int64_t h = c / hd;
  const int64_t d = c - h * hd;
  dst[e] = ring[h * head_stride + j * hd + d];
}

// ---------------------------------------------------------------------------
// Multi-frame prefill of one session (mobius PR #368, "P2 - Moshi LM": the
// temporal task takes input_frame[B, 17, S] with S > 1; priming runs whole
// prompts through it): the frames are the columns of the projections, and
// each layer's keys and values sit in a window buffer, per head
// [rows][HD], row i holding position s0 + i (the ring's rows of earlier
// positions gathered in front, the chunk's own rows written after them by
// the q/k/v epilogue), so every query column attends a contiguous run.
// ---------------------------------------------------------------------------

// Rows [i0, i1) of the window buffer <-> the session's ring (ring slot of
// position s0 + i is (s0 + i) mod W): to_ring = 0 copies ring -> window,
// 1 copies window -> ring. One thread per element.
template <typename T>
__global__ __launch_bounds__(256) void window_copy_kernel(T* win, T* ring, int i0, int i1, int64_t s0,
                                                          int W, int H, int hd,
                                                          int64_t win_head_stride,
                                                          int64_t ring_head_stride, int to_ring) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_head = (int64_t)(i1 - i0) * hd;
  if (e >= per_head * H) return;
  const int64_t h = e / per_head;
  const int64_t r = e - h * per_head;
  const int64_t i = i0 + r / hd;
  const int64_t d = r - (r / hd) * hd;
  T* w = win + h * win_head_stride + i * hd + d;
  T* g = ring + h * ring_head_stride + ((s0 + i) % W) * hd + d;
  if (to_ring) *g = *w;
  else *w = *g;
}

// Attention of query column b = blockIdx.z, head blockIdx.y, key span
// blockIdx.x over window rows [key0[b], key0[b] + nkeys[b]) (attn_span's
// arithmetic; spans merged by prefill_combine_kernel in span order).
template <typename T, int HD>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillAttnArgs p) {
  __shared__ double s_w[span_lds_doubles<T, HD, 256>()];
  const int span = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nvalid = p.nkeys[b];
  const int ns = n_spans(p.a, nvalid);
  if (span >= ns) return;
  AttnArgs a = p.a;
  a.slot_stride = 0;  // the column's window starts key0[b] rows into the buffer
  a.ring_k = (const T*)p.a.ring_k + (size_t)p.key0[b] * HD;
  a.ring_v = (const T*)p.a.ring_v + (size_t)p.key0[b] * HD;
  double* part = a.part + (((size_t)b * a.n_heads + h) * a.max_spans + span) * (HD + 2);
  attn_span<T, HD, 256, false>(a, h, b, span * nvalid / ns, (span + 1) * nvalid / ns, nvalid, -1,
                               s_w, part, ns == 1);
}

template <typename T, int HD>
__global__ __launch_bounds__(HD) void prefill_combine_kernel(PrefillAttnArgs p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int ns = n_spans(p.a, p.nkeys[b]);
  if (ns <= 1) return;  // written directly
  combine_item<T, HD, false>(p.a, h, b, ns);
}

template <typename T>
static hipError_t launch_prefill_attn_t(int hd, const PrefillAttnArgs& p, hipStream_t st) {
  const dim3 grid(p.a.max_spans, p.a.n_heads, p.m), cgrid(p.a.n_heads, p.m);
#define MOSHI_PF(HDV)                                                                 \
  case HDV:                                                                           \
    hipLaunchKernelGGL((prefill_attn_kernel<T, HDV>), grid, dim3(256), 0, st, p);     \
    hipLaunchKernelGGL((prefill_combine_kernel<T, HDV>), cgrid, dim3(HDV), 0, st, p); \
    break;
  switch (hd) {
    MOSHI_PF(32)
    MOSHI_PF(64)
    MOSHI_PF(128)
    default: return hipErrorInvalidValue;
  }
#undef MOSHI_PF
  return hipGetLastError();
}

hipError_t launch_prefill_attn(int dtype, int hd, const PrefillAttnArgs& p, hipStream_t st) {
  if (p.m < 1 || p.a.max_spans < 1) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? launch_prefill_attn_t<__bf16>(hd, p, st)
                          : launch_prefill_attn_t<float>(hd, p, st);
}

hipError_t launch_window_copy(int dtype, void* win, void* ring, int i0, int i1, int64_t s0, int W,
                              int H, int hd, int64_t win_head_stride, int64_t ring_head_stride,
                              int to_ring, hipStream_t st) {
  const int64_t total = (int64_t)(i1 - i0) * hd * H;
  if (total <= 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(window_copy_kernel<__bf16>, grid, block, 0, st, (__bf16*)win, (__bf16*)ring,
                       i0, i1, s0, W, H, hd, win_head_stride, ring_head_stride, to_ring);
  else
    hipLaunchKernelGGL(window_copy_kernel<float>, grid, block, 0, st, (float*)win, (float*)ring, i0,
                       i1, s0, W, H, hd, win_head_stride, ring_head_stride, to_ring);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

int gemm_tiles(int epi, int N) { return epi == EPI_SWIGLU ? (N + 7) / 8 : (N + 15) / 16; }

int gemm_kw(int dtype, int B, int K, int tiles) {
  (void)dtype;
  // one session: 8 waves (the sum-of-squares partials assume 2 rows per
  // wave). More sessions, inputs of 4096 or wider (the temporal projections):
  // up to 32 sessions 16 waves; at 33..64, 12 waves for projections of at
  // most 512 row tiles (three 4-wave workgroups fit a CU, so fewer tiles
  // would leave SIMDs with one wave) and 4 above (measured). Narrower inputs
  // (the depformer's) take 8 waves up to 32 sessions and 4 at 33..64.
  if (B == 1) return GEMV_KW;
  if (K >= 4096) return B <= 32 ? 16 : (tiles <= 512 ? 12 : 4);
  return B <= 32 ? 8 : 4;
}

int gemm_ksplit(int B, int K, int tiles) {
  // long inputs with few row tiles (the depformer's down projection: 64
  // tiles, K = 2816) up to 32 sessions: a whole-K tile per workgroup left
  // most CUs idle and each wave with ~44 dependent k-steps (16 sessions: the
  // down phases 1.33 -> 0.86 ms per step, the step 15.02 -> 14.51 ms). At 33+
  // sessions the multi-session depformer already spreads 4 column blocks
  // per tile (2 or 4 segments: within noise of none); the temporal
  // projections (256+ tiles) measured no faster split in a probe.
  if (B < 2 || K < 2048 || tiles > 64) return 1;
  const char* env = getenv("MOSHI_KSPLIT");  // segments override (measurement)
  if (env && env[0] >= '1' && env[0] <= '4' && env[1] == 0) return env[0] - '0';
  return B <= 32 ? 4 : 1;
}

// Workgroups of the one-session projection: at most one per CU (the kernel
// loops over row tiles), never more than there are tiles.
static int g_gemv_grid = 256;
void set_gemv_grid(int n) { g_gemv_grid = n > 0 ? n : 256; }

template <typename T, int KW>
static hipError_t launch_gemv_kw(int pro, int epi, const GemmArgs& a, hipStream_t st) {
  const int ntiles = gemm_tiles(epi, a.N);
  dim3 grid(ntiles < g_gemv_grid ? ntiles : g_gemv_grid), block(64 * KW);
  const size_t lds = (size_t)a.K * sizeof(T);
#define MOSHI_GEMV_CASE(P, E)                                                  \
  if (pro == P && epi == E) {                                                 \
    hipLaunchKernelGGL((gemv_kernel<T, KW, P, E>), grid, block, lds, st, a); \
    return hipGetLastError();                                                 \
  }
  MOSHI_GEMV_CASE(PRO_NORM, EPI_QKV)
  MOSHI_GEMV_CASE(PRO_DIRECT, EPI_RESID)
  MOSHI_GEMV_CASE(PRO_NORM, EPI_SWIGLU)
  MOSHI_GEMV_CASE(PRO_NORM, EPI_ARGMAX)
  MOSHI_GEMV_CASE(PRO_DIRECT, EPI_STORE)
  MOSHI_GEMV_CASE(PRO_CAST, EPI_ARGMAX)
#undef MOSHI_GEMV_CASE
  return hipErrorInvalidValue;
}

template <typename T, int NB, int KW, bool DB, int RT = 1, int U = GEMM_U>
static hipError_t launch_gemm_db(int epi, const GemmArgs& a, hipStream_t st) {
  if (a.ksplit > GEMM_KSPLIT_MAX || (a.ksplit > 1 && (RT != 1 || a.kpart == nullptr || a.kcnt == nullptr)))
    return hipErrorInvalidValue;
  dim3 grid((gemm_tiles(epi, a.N) + RT - 1) / RT, a.ksplit > 1 ? a.ksplit : 1), block(64 * KW);
  switch (epi) {
    case EPI_STORE:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_STORE, DB, RT, U>), grid, block, 0, st, a);
      break;
    case EPI_RESID:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_RESID, DB, RT, U>), grid, block, 0, st, a);
      break;
    case EPI_QKV:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_QKV, DB, RT, U>), grid, block, 0, st, a);
      break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_SWIGLU, DB, RT, U>), grid, block, 0, st, a);
      break;
    case EPI_ARGMAX:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_ARGMAX, DB, RT, U>), grid, block, 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Double-buffered batches (the next batch requested before this one is
// used) where the registers allow it.
template <typename T, int NB, int KW>
static hipError_t launch_gemm_kw(int epi, const GemmArgs& a, hipStream_t st) {
  // double-buffered batches only for narrow inputs at 8 or fewer waves: the
  // wide ones need every wave slot (single batches: 54 VGPRs, two 16-wave
  // workgroups per CU; double-buffered ones lose half of that, or spill;
  // measured slower)
  if constexpr (NB <= 2 && KW <= 8)
    if (a.K < 4096) return launch_gemm_db<T, NB, KW, true>(epi, a, st);
  // wide inputs with four column blocks and many row tiles: two row tiles
  // per workgroup share each input group's conversion (fewer VALU
  // instructions per MFMA; measured faster for the 1408-tile gate/up and the
  // 2000-tile text head at 64 sessions, slower wherever it halves the
  // workgroups of a projection with fewer tiles or, with one column block,
  // the workgroups per CU)
  if constexpr (NB == 4 && KW <= 8)  // (LDS: KW x 2 x NB x 2 KB)
    if (gemm_tiles(epi, a.N) >= 1024 && a.ksplit <= 1)
      return launch_gemm_db<T, NB, KW, false, 2>(epi, a, st);
  // up to 16 sessions, the 1408-tile gate/up: two row tiles per wave with
  // two k-steps per batch (58 VGPRs: still two 16-wave workgroups per CU);
  // 70.3 -> 65.2 us in a probe of its tiles, slower for the 256-tile
  // projections (half the workgroups)
  if constexpr (NB == 1 && KW == 16)
    if (epi == EPI_SWIGLU && gemm_tiles(epi, a.N) >= 1024 && a.ksplit <= 1)
      return launch_gemm_db<T, 1, 16, false, 2, 2>(epi, a, st);
  return launch_gemm_db<T, NB, KW, false>(epi, a, st);
}

template <typename T>
static hipError_t launch_gemm_t(int kw, int pro, int epi, const GemmArgs& a, hipStream_t st) {
  if (a.B == 1) {
    if (kw == 8) return launch_gemv_kw<T, 8>(pro, epi, a, st);
    if (kw == 4) return launch_gemv_kw<T, 4>(pro, epi, a, st);
    if (kw == 2) return launch_gemv_kw<T, 2>(pro, epi, a, st);
    return hipErrorInvalidValue;
  }
  // more than one session: input vectors rounded first, then MFMA tiles
  GemmArgs b = a;
  if (pro != PRO_DIRECT) {
    if (a.xn_out == nullptr) return hipErrorInvalidValue;  // the caller provides the buffer
    const dim3 ng(a.B, (a.K + 1023) / 1024);
    if (pro == PRO_NORM)
      hipLaunchKernelGGL((norm_kernel<T, PRO_NORM>), ng, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((norm_kernel<T, PRO_CAST>), ng, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    b.X = a.xn_out;
    b.ldx = a.K;
  }
  // temporal projections of two to four sessions: VALU tiles (gemv_cols_kernel)
  // where every session's input fits the workgroup's LDS beside the tiles'
  // sums (wider inputs take the MFMA tiles below)
  const size_t cols_lds = (size_t)(a.B <= 2 ? 2 : 4) * a.K * sizeof(T) + 3 * 16 * 4 * sizeof(double);
  if (a.vec_cols && a.B <= 4 && cols_lds <= 160 * 1024 && a.K % VecOf<T>::N == 0) {
    const int ntiles = gemm_tiles(epi, a.N);
    const int grid = ntiles < g_gemv_grid ? ntiles : g_gemv_grid;
#define MOSHI_COLS(NC_, E_)                                                                    \
  hipLaunchKernelGGL((gemv_cols_kernel<T, NC_, E_, 3>), dim3(grid), dim3(512),                 \
                     (NC_) * a.K * sizeof(T), st, b)
    const bool two = a.B <= 2;
    switch (epi) {
      case EPI_STORE: if (two) MOSHI_COLS(2, EPI_STORE); else MOSHI_COLS(4, EPI_STORE); break;
      case EPI_RESID: if (two) MOSHI_COLS(2, EPI_RESID); else MOSHI_COLS(4, EPI_RESID); break;
      case EPI_QKV: if (two) MOSHI_COLS(2, EPI_QKV); else MOSHI_COLS(4, EPI_QKV); break;
      case EPI_SWIGLU: if (two) MOSHI_COLS(2, EPI_SWIGLU); else MOSHI_COLS(4, EPI_SWIGLU); break;
      case EPI_ARGMAX: if (two) MOSHI_COLS(2, EPI_ARGMAX); else MOSHI_COLS(4, EPI_ARGMAX); break;
      default: return hipErrorInvalidValue;
    }
#undef MOSHI_COLS
    return hipGetLastError();
  }
  // waves per tile: 16 or 8 (up to 32 sessions), 12 or 4 (33..64)
  const int nb = a.B <= 16 ? 1 : (a.B <= 32 ? 2 : 4);
  if (nb == 1) {
    if (kw == 16) return launch_gemm_kw<T, 1, 16>(epi, b, st);
    if (kw == 8) return launch_gemm_kw<T, 1, 8>(epi, b, st);
  } else if (nb == 2) {
    if (kw == 16) return launch_gemm_kw<T, 2, 16>(epi, b, st);
    if (kw == 8) return launch_gemm_kw<T, 2, 8>(epi, b, st);
  } else {
    if (kw == 12) return launch_gemm_kw<T, 4, 12>(epi, b, st);
    if (kw == 4) return launch_gemm_kw<T, 4, 4>(epi, b, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int dtype, int kw, int pro, int epi, const GemmArgs& a, hipStream_t st) {
  if (a.B < 1 || a.B > 64 || a.N < 1 || a.K < 1) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? launch_gemm_t<__bf16>(kw, pro, epi, a, st)
                          : launch_gemm_t<float>(kw, pro, epi, a, st);
}

template <typename T>
static hipError_t launch_attn_t(int hd, const AttnArgs& a, int B, hipStream_t st) {
  const dim3 grid(a.max_spans, a.n_heads, B);
  if (B == 1) {
    switch (hd) {
      case 32: hipLaunchKernelGGL((attn_kernel<T, 32, 512>), grid, dim3(512), 0, st, a); break;
      case 64: hipLaunchKernelGGL((attn_kernel<T, 64, 512>), grid, dim3(512), 0, st, a); break;
      case 128: hipLaunchKernelGGL((attn_kernel<T, 128, 512>), grid, dim3(512), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (hd) {
      case 32: hipLaunchKernelGGL((attn_kernel<T, 32, 256>), grid, dim3(256), 0, st, a); break;
      case 64: hipLaunchKernelGGL((attn_kernel<T, 64, 256>), grid, dim3(256), 0, st, a); break;
      case 128: hipLaunchKernelGGL((attn_kernel<T, 128, 256>), grid, dim3(256), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_attn(int dtype, int hd, const AttnArgs& a, int B, hipStream_t st) {
  return dtype == DT_BF16 ? launch_attn_t<__bf16>(hd, a, B, st) : launch_attn_t<float>(hd, a, B, st);
}

template <typename T>
static hipError_t launch_dep_attn_t(int hd, const AttnArgs& a, int B, hipStream_t st) {
  if (a.scalar_nvalid < 1 || a.scalar_nvalid > DEP_MAX_KEYS) return hipErrorInvalidValue;
  switch (hd) {
    case 32: hipLaunchKernelGGL((dep_attn_kernel<T, 32>), dim3(B), dim3(512), 0, st, a); break;
    case 64: hipLaunchKernelGGL((dep_attn_kernel<T, 64>), dim3(B), dim3(512), 0, st, a); break;
    case 128: hipLaunchKernelGGL((dep_attn_kernel<T, 128>), dim3(B), dim3(512), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dep_attn(int dtype, int hd, const AttnArgs& a, int B, hipStream_t st) {
  return dtype == DT_BF16 ? launch_dep_attn_t<__bf16>(hd, a, B, st)
                          : launch_dep_attn_t<float>(hd, a, B, st);
}

template <typename T>
static hipError_t launch_combine_t(int hd, const AttnArgs& a, int B, hipStream_t st) {
  dim3 grid(a.n_heads, B);
  switch (hd) {
    case 32: hipLaunchKernelGGL((attn_combine_kernel<T, 32>), grid, dim3(32), 0, st, a); break;
    case 64: hipLaunchKernelGGL((attn_combine_kernel<T, 64>), grid, dim3(64), 0, st, a); break;
    case 128: hipLaunchKernelGGL((attn_combine_kernel<T, 128>), grid, dim3(128), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(int dtype, int hd, const AttnArgs& a, int B, hipStream_t st) {
  return dtype == DT_BF16 ? launch_combine_t<__bf16>(hd, a, B, st)
                          : launch_combine_t<float>(hd, a, B, st);
}

hipError_t launch_argmax_reduce(const ArgPart* part, int n_tiles, int n_rows, int B, int* tok,
                                int stride, const int* forced, int forced_stride, int forced_col,
                                hipStream_t st) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(B), dim3(256), 0, st, part, n_tiles, n_rows, B,
                     tok, stride, forced, forced_stride, forced_col);
  return hipGetLastError();
}

hipError_t launch_finish_outputs(int* tokens, int* codes, const int* live, int B, int S, int s_run,
                                 hipStream_t st) {
  hipLaunchKernelGGL(finish_outputs_kernel, dim3(B), dim3(64), 0, st, tokens, codes, live, B, S,
                     s_run);
  return hipGetLastError();
}

hipError_t launch_embed(int dtype, const EmbedArgs& a, hipStream_t st) {
  dim3 grid((a.D + 15) / 16, (a.B + 3) / 4), block(64);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(embed_kernel<__bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(embed_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_entry(int dtype, const EntryArgs& a, hipStream_t st) {
  dim3 grid((a.D + 15) / 16, (a.B + 3) / 4), block(64);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(entry_kernel<__bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(entry_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_advance(int64_t* pos, const int* live, int B, hipStream_t st) {
  hipLaunchKernelGGL(advance_kernel, dim3((B + 63) / 64), dim3(64), 0, st, pos, live, B);
  return hipGetLastError();
}

hipError_t launch_scatter_prefill(int dtype, const void* src, void* ring, int n, int n_heads,
                                  int hd, int64_t head_stride, hipStream_t st) {
  const int64_t total = (int64_t)n * n_heads * hd;
  if (total == 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(scatter_kernel<__bf16>, grid, block, 0, st, (const __bf16*)src,
                       (__bf16*)ring, n, n_heads, hd, head_stride);
  else
    hipLaunchKernelGGL(scatter_kernel<float>, grid, block, 0, st, (const float*)src, (float*)ring,
                       n, n_heads, hd, head_stride);
  return hipGetLastError();
}

hipError_t launch_gather_ring(int dtype, const void* ring, void* dst, int n, int n_heads, int hd,
                              int64_t head_stride, hipStream_t st) {
  const int64_t total = (int64_t)n * n_heads * hd;
  if (total == 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(gather_kernel<__bf16>, grid, block, 0, st, (const __bf16*)ring,
                       (__bf16*)dst, n, n_heads, hd, head_stride);
  else
    hipLaunchKernelGGL(gather_kernel<float>, grid, block, 0, st, (const float*)ring, (float*)dst,
                       n, n_heads, hd, head_stride);
  return hipGetLastError();
}

}  // namespace moshi
