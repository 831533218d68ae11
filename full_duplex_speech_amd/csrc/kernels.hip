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

#include "kernels.h"

namespace moshi {

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte group

template <typename T>
struct VecOf;
template <>
struct VecOf<__bf16> {
  static constexpr int N = 8;  // elements per 16-byte group
};
template <>
struct VecOf<float> {
  static constexpr int N = 4;
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
// Weights are read once per step: stream them past the caches.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// ---- conversions -----------------------------------------------------------

template <typename T>
__device__ __forceinline__ void widen(u32x4 w, double* out);
template <>
__device__ __forceinline__ void widen<__bf16>(u32x4 w, double* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = (double)__uint_as_float(w[i] << 16);
    out[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void widen<float>(u32x4 w, double* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = (double)__uint_as_float(w[i]);
}

__device__ __forceinline__ double to_d(__bf16 v) { return (double)(float)v; }
__device__ __forceinline__ double to_d(float v) { return (double)v; }

// bf16 bits of the value nearest to d (ties to even). Rounding d to fp32 first
// is exact enough except when that lands exactly on a bf16 midpoint while d
// itself is not on it; then d decides the direction.
__device__ __forceinline__ unsigned short bf16_bits_rne(double d) {
  const float f = (float)d;
  unsigned int u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u)
    return (unsigned short)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  if ((u & 0xffffu) == 0x8000u && (double)f != d) {
    const bool up = fabs(d) > fabs((double)f);
    return (unsigned short)((u >> 16) + (up ? 1u : 0u));
  }
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

template <typename T>
__device__ __forceinline__ T round_to(double d);
template <>
__device__ __forceinline__ __bf16 round_to<__bf16>(double d) {
  return __builtin_bit_cast(__bf16, bf16_bits_rne(d));
}
template <>
__device__ __forceinline__ float round_to<float>(double d) {
  return (float)d;
}

// The rounded input vector: VEC values k0.. of column col as doubles (the
// values the stored dtype holds), and the same values packed for storing.
template <typename T, int PRO>
__device__ __forceinline__ void load_x(const GemmArgs& a, int col, int k0, double rs, double* xv,
                                       u32x4* packed) {
  constexpr int VEC = VecOf<T>::N;
  if constexpr (PRO == PRO_DIRECT) {
    const u32x4 w = ld16((const T*)a.X + (size_t)col * a.ldx + k0);
    widen<T>(w, xv);
    *packed = w;
  } else {
    const double* xp = (const double*)a.X + (size_t)col * a.ldx + k0;
    double gv[VEC];
    if constexpr (PRO == PRO_NORM) widen<T>(ld16((const T*)a.gain + k0), gv);
    u32x4 r;
    T* rv = (T*)&r;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const double v = (PRO == PRO_NORM) ? xp[e] * rs * gv[e] : xp[e];
      rv[e] = round_to<T>(v);
      xv[e] = to_d(rv[e]);
    }
    *packed = r;
  }
}

// Weight row read by tile row t of tile `tile`. EPI_SWIGLU interleaves units:
// even tile rows are gate rows, odd tile rows the matching up rows.
template <int EPI>
__device__ __forceinline__ int tile_row(int tile, int t, int N, bool& ok) {
  if constexpr (EPI == EPI_SWIGLU) {
    const int u = tile * 8 + (t >> 1);
    ok = u < N;
    return (t & 1) ? N + u : u;
  } else {
    const int r = tile * 16 + t;
    ok = r < N;
    return r;
  }
}

__device__ __forceinline__ bool arg_better(double v, int i, double bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ double shfl_xor_d(double v, int m) {
  return __hiloint2double(__shfl_xor(__double2hiint(v), m), __shfl_xor(__double2loint(v), m));
}

// RMSNorm scale 1/sqrt(mean(x^2) + eps) of column col from the producer's
// per-tile sums of squares; every thread of the workgroup gets the same value.
// Threads [0, nthr) split the tiles; fixed-order reduction through `red`.
__device__ __forceinline__ double rms_scale(const GemmArgs& a, int col, double* red, int nthr) {
  const int t = threadIdx.x;
  double s = 0.0;
  for (int i = t; i < a.n_ssq; i += nthr) s += a.ssq[(size_t)i * a.B + col];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += shfl_xor_d(s, off);
  if ((t & 63) == 0) red[t >> 6] = s;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < nthr / 64; ++w) tot += red[w];
  return 1.0 / sqrt(tot / (double)a.K + a.eps);
}

// ---- epilogue: tile rows 4g..4g+3 of column col, values v -----------------

template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& a, int tile, int g, int col,
                                         const double* v) {
  const bool cok = col < a.B;
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tile * 16 + 4 * g + i;
      if (cok && row < a.N) a.out64[(size_t)col * a.ldo + row] = v[i];
    }
  } else if constexpr (EPI == EPI_RESID) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tile * 16 + 4 * g + i;
      if (cok && row < a.N) {
        double* p = a.resid + (size_t)col * a.ldr + row;
        const double xn = *p + v[i];
        *p = xn;
        ss += xn * xn;
      }
    }
    // the 4 lanes of this column (g = 0..3) combine in a fixed order
    ss += shfl_xor_d(ss, 16);
    ss += shfl_xor_d(ss, 32);
    if (g == 0 && cok) a.ssq_out[(size_t)tile * a.B + col] = ss;
  } else if constexpr (EPI == EPI_QKV) {
    const int row0 = tile * 16 + 4 * g;  // 16-row tiles never straddle a part or a head
    const int part = row0 / a.dq;
    const int din = row0 - part * a.dq;
    const int head = din / a.hd;
    const int d0 = din - head * a.hd;
    double vals[4] = {v[0], v[1], v[2], v[3]};
    if (!cok || row0 >= a.N) return;
    if (a.inv_freq != nullptr && part < 2) {
      const double p = (double)a.pos[col];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const double ang = p * a.inv_freq[(d0 >> 1) + j];
        double sn, cs;
        sincos(ang, &sn, &cs);
        const double x0 = vals[2 * j], x1 = vals[2 * j + 1];
        vals[2 * j] = x0 * cs - x1 * sn;
        vals[2 * j + 1] = x0 * sn + x1 * cs;
      }
    }
    if (part == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a.q_out[(size_t)col * a.dq + din + i] = vals[i];
    } else if (a.live[col]) {
      const int widx = a.pos ? (int)(a.pos[col] % a.cap) : a.scalar_widx;
      T* dst = (T*)(part == 1 ? a.ring_k : a.ring_v) + (size_t)col * a.slot_stride + a.layer_off +
               (size_t)head * a.head_stride + (size_t)widx * a.hd + d0;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = round_to<T>(vals[i]);
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int u = tile * 8 + 2 * g + j;
      if (cok && u < a.N) {
        const double gt = v[2 * j], up = v[2 * j + 1];
        ((T*)a.act)[(size_t)col * a.lda + u] = round_to<T>(gt / (1.0 + exp(-gt)) * up);
      }
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    // NaN never wins: it compares as -inf; rows past N carry index INT_MAX.
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tile * 16 + 4 * g + i;
      if (row < a.N) {
        if (cok) a.logits[(size_t)col * a.ldo + row] = (float)v[i];
        const double val = (v[i] != v[i]) ? -INFINITY : v[i];
        if (bi == 0x7fffffff || val > bv) {
          bv = val;
          bi = row;
        }
      }
    }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const double ov = shfl_xor_d(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (arg_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (g == 0 && cok) a.apart[(size_t)tile * a.B + col] = ArgPart{bv, bi, 0};
  }
}

// ---------------------------------------------------------------------------
// One session: fp64 VALU GEMV
// ---------------------------------------------------------------------------

// A workgroup of KW waves walks row tiles blockIdx.x, +gridDim.x, ... (16
// output rows each); wave w owns rows w*R .. w*R+R-1 (R = 16/KW) of a tile
// over the whole of K. The rounded input vector is built once per workgroup in
// LDS (model dtype). Lane l covers the 16-byte groups l, l+64, ... of a row, so
// a wave reads each row in contiguous 1 KB pieces. Weights stream in batches
// of U groups per lane and row, double-buffered: the next batch (possibly of
// the next tile) is requested before the current one is used. Each finished
// row is reduced over the 64 lanes by a butterfly; wave 0 applies the
// epilogue to the tile's 16 rows.
template <typename T, int KW, int PRO, int EPI>
__global__ __launch_bounds__(64 * KW) void gemv_kernel(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char s_dyn[];  // rounded input, K elements
  constexpr int VEC = VecOf<T>::N;
  constexpr int R = 16 / KW;                 // rows per wave
  constexpr int U = (R <= 2) ? 8 : 4;        // groups per lane and row per batch
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  T* xs = (T*)s_dyn;
  __shared__ double s_red[2][16];
  __shared__ double s_tmp[KW];

  const int ntiles = (EPI == EPI_SWIGLU) ? (a.N + 7) / 8 : (a.N + 15) / 16;
  const int ngroups = a.K / VEC;  // K is a multiple of VEC
  const int nbatch = (ngroups + U * 64 - 1) / (U * 64);

  auto load_batch = [&](u32x4 (&w)[U][R], int tile, int bt) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      bool ok;
      const int rr = tile_row<EPI>(tile, wave * R + r, a.N, ok);
      const T* wr = (const T*)a.W + (size_t)(ok ? rr : 0) * a.K;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int gi = bt * U * 64 + u * 64 + lane;
        w[u][r] = (ok && gi < ngroups) ? ld16_stream(wr + (size_t)gi * VEC) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  int tile = blockIdx.x;
  u32x4 wa[U][R], wb[U][R];
  if (tile < ntiles) load_batch(wa, tile, 0);  // in flight while the input is built

  // input vector -> LDS (rounded to the model dtype)
  double rs = 1.0;
  if constexpr (PRO == PRO_NORM) rs = rms_scale(a, 0, s_tmp, 64 * KW);
  const bool write_xn = (PRO != PRO_DIRECT) && a.xn_out != nullptr && blockIdx.x == 0;
  for (int gi = threadIdx.x; gi < ngroups; gi += 64 * KW) {
    double xv[VEC];
    u32x4 packed;
    load_x<T, PRO>(a, 0, gi * VEC, rs, xv, &packed);
    *(u32x4*)(xs + (size_t)gi * VEC) = packed;
    if (write_xn) *(u32x4*)((T*)a.xn_out + (size_t)gi * VEC) = packed;
  }
  __syncthreads();
  if (tile >= ntiles) return;

  double acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0;
  int bt = 0, parity = 0;

  // consume batch (tile, bt) held in w; finish the tile after its last batch
  auto consume = [&](const u32x4 (&w)[U][R]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gi = bt * U * 64 + u * 64 + lane;
      if (gi < ngroups) {
        double xv[VEC];
        widen<T>(*(const u32x4*)(xs + (size_t)gi * VEC), xv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          double wd[VEC];
          widen<T>(w[u][r], wd);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[r] = fma(wd[e], xv[e], acc[r]);
        }
      }
    }
    if (bt == nbatch - 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc[r] += shfl_xor_d(acc[r], off);
      }
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) s_red[parity][wave * R + r] = acc[r];
      }
      __syncthreads();
      if (wave == 0 && (lane & 15) == 0) {
        // g = lane / 16 holds rows 4g..4g+3 of column 0
        const int g = lane >> 4;
        const double v[4] = {s_red[parity][4 * g], s_red[parity][4 * g + 1],
                             s_red[parity][4 * g + 2], s_red[parity][4 * g + 3]};
        epilogue<T, EPI>(a, tile, g, 0, v);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.0;
      parity ^= 1;
    }
  };
  // the batch after (tile, bt)
  auto advance = [&](int& t, int& b) {
    if (++b == nbatch) {
      b = 0;
      t += gridDim.x;
    }
  };

  for (;;) {
    int nt = tile, nb = bt;
    advance(nt, nb);
    if (nt < ntiles) load_batch(wb, nt, nb);
    consume(wa);
    if (nt >= ntiles) break;
    tile = nt;
    bt = nb;
    advance(nt, nb);
    if (nt < ntiles) load_batch(wa, nt, nb);
    consume(wb);
    if (nt >= ntiles) break;
    tile = nt;
    bt = nb;
  }
}

// ---------------------------------------------------------------------------
// Two or more sessions: fp64 MFMA 16x16x4 tiles
// ---------------------------------------------------------------------------

// A = 16 weight rows x 4 k (lane: row lane%16, k-slot lane/16), B = 4 k x 16
// session columns (lane: column lane%16, same k-slot). A lane loads 16 bytes of
// its row (VEC consecutive k) and of its column's input; element e of every
// lane feeds MFMA e, so both operands map k-slot g to k0 + VEC*g + e.
// The fp64 16x16 result puts row (lane/16) + 4i in element i of a lane, so A
// row m carries tile row 4*(m%4) + m/4: element i of lane group g is then tile
// row 4g + i, the layout the epilogues use.
template <typename T, int NB, int KW, int EPI>
__global__ __launch_bounds__(64 * KW) void gemm_kernel(GemmArgs a) {
  constexpr int VEC = VecOf<T>::N;
  constexpr int KSTEP = 4 * VEC;
  constexpr int U = 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x;
  __shared__ f64x4 s_acc[KW][NB][64];

  bool rok;
  const int wrow = tile_row<EPI>(tile, 4 * (r16 & 3) + (r16 >> 2), a.N, rok);
  const T* wbase = (const T*)a.W + (size_t)(rok ? wrow : 0) * a.K + g * VEC;
  const int nsteps = (a.K + KSTEP - 1) / KSTEP;
  const int s0 = (wave * nsteps) / KW;
  const int s1 = ((wave + 1) * nsteps) / KW;

  f64x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int st = s0; st < s1; st += U) {
    u32x4 wv[U];
    u32x4 xw[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (st + u) * KSTEP + g * VEC;
      const bool kok = (st + u < s1) && (k0 < a.K);
      wv[u] = (kok && rok) ? ld16_stream(wbase + (size_t)(st + u) * KSTEP) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = nb * 16 + r16;
        xw[u][nb] = (kok && col < a.B) ? ld16((const T*)a.X + (size_t)col * a.ldx + k0)
                                       : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      double wd[VEC];
      widen<T>(wv[u], wd);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        double xd[VEC];
        widen<T>(xw[u][nb], xd);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          acc[nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(wd[e], xd[e], acc[nb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) s_acc[wave][nb][lane] = acc[nb];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f64x4 s = s_acc[0][nb][lane];
    for (int w = 1; w < KW; ++w) s += s_acc[w][nb][lane];
    const double v[4] = {s[0], s[1], s[2], s[3]};
    epilogue<T, EPI>(a, tile, g, nb * 16 + r16, v);
  }
}

// Input vectors for the MFMA path: xn[b][k] = round(x[b][k] * scale_b * g[k])
// (PRO_NORM) or round(x[b][k]) (PRO_CAST); one workgroup per column.
template <typename T, int PRO>
__global__ __launch_bounds__(256) void norm_kernel(GemmArgs a) {
  const int b = blockIdx.x;
  __shared__ double s_tmp[4];
  double rs = 1.0;
  if constexpr (PRO == PRO_NORM) rs = rms_scale(a, b, s_tmp, 256);
  const double* x = (const double*)a.X + (size_t)b * a.ldx;
  T* out = (T*)a.xn_out + (size_t)b * a.K;
  for (int k = threadIdx.x; k < a.K; k += 256) {
    const double v = (PRO == PRO_NORM) ? x[k] * rs * to_d(((const T*)a.gain)[k]) : x[k];
    out[k] = round_to<T>(v);
  }
}

// Greedy token of column blockIdx.x from per-tile (max, index) partials.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const ArgPart* part, int n_tiles,
                                                            int n_rows, int B, int* tok,
                                                            int stride) {
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
    tok[(size_t)b * stride] = (bi < n_rows) ? bi : 0;
  }
}

// ---------------------------------------------------------------------------
// Sliding-window decode attention over a ring of K/V
// ---------------------------------------------------------------------------

// Keys of slot b visible at its current position: ring slots [0, nvalid),
// minus `excl` (the oldest key, under the mask-oldest reading).
__device__ __forceinline__ void window_of(const AttnArgs& a, int b, int& nvalid, int& excl) {
  excl = -1;
  if (a.pos != nullptr) {
    const int64_t p = a.pos[b];
    nvalid = (int)(p + 1 < (int64_t)a.cap ? p + 1 : (int64_t)a.cap);
    if (a.mask_oldest && p >= (int64_t)a.cap - 1) excl = (int)((p + 1) % a.cap);
  } else {
    nvalid = a.scalar_nvalid;
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int VEC = VecOf<T>::N;
  constexpr int TK = HD / VEC;   // threads per key (one 16-byte group each)
  constexpr int KP = 256 / TK;   // keys per pass
  constexpr int C = ATTN_CHUNK;
  constexpr int PASSES = C / KP;
  static_assert(TK <= 64 && (64 % TK) == 0 && PASSES >= 1, "head dim / chunk layout");

  const int chunk = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int t = threadIdx.x;
  if (!a.live[b]) return;
  int nvalid, excl;
  window_of(a, b, nvalid, excl);
  const int nchunks = (nvalid + C - 1) / C;
  if (chunk >= nchunks) return;

  __shared__ double s_p[C];
  __shared__ double s_o[KP][HD + 1];
  __shared__ double s_ml[2];

  const int kd = t % TK;
  const int kk = t / TK;
  const size_t base = (size_t)b * a.slot_stride + a.layer_off + (size_t)h * a.head_stride;
  const T* kbase = (const T*)a.ring_k + base;
  const T* vbase = (const T*)a.ring_v + base;

  // every K and V group of this chunk is requested up front
  u32x4 kw[PASSES], vw[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int j = chunk * C + ps * KP + kk;
    const bool ok = j < nvalid;
    kw[ps] = ok ? ld16(kbase + (size_t)j * HD + kd * VEC) : u32x4{0u, 0u, 0u, 0u};
    vw[ps] = ok ? ld16(vbase + (size_t)j * HD + kd * VEC) : u32x4{0u, 0u, 0u, 0u};
  }
  const double scale = 1.0 / sqrt((double)HD);
  double qv[VEC];
  const double* qp = a.q + (size_t)b * a.ldq + h * HD + kd * VEC;
#pragma unroll
  for (int e = 0; e < VEC; ++e) qv[e] = qp[e];

  // scores s_j = q.k_j / sqrt(HD)
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int j = chunk * C + ps * KP + kk;
    const bool ok = j < nvalid && j != excl;
    double kd_[VEC];
    widen<T>(kw[ps], kd_);
    double d = 0.0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) d = fma(qv[e], kd_[e], d);
#pragma unroll
    for (int off = TK / 2; off > 0; off >>= 1) d += shfl_xor_d(d, off);
    if (kd == 0) s_p[ps * KP + kk] = ok ? d * scale : -INFINITY;
  }
  __syncthreads();
  if (t < 64) {
    const double sv = (t < C) ? s_p[t] : -INFINITY;
    double m = sv;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmax(m, shfl_xor_d(m, off));
    const double pj = (m == -INFINITY || sv == -INFINITY) ? 0.0 : exp(sv - m);
    double l = pj;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += shfl_xor_d(l, off);
    if (t < C) s_p[t] = pj;
    if (t == 0) {
      s_ml[0] = m;
      s_ml[1] = l;
    }
  }
  __syncthreads();

  // p . V
  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const double pj = s_p[ps * KP + kk];
    double vd[VEC];
    widen<T>(vw[ps], vd);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = fma(pj, vd[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) s_o[kk][kd * VEC + e] = acc[e];
  __syncthreads();
  if (t >= HD) return;
  double od = 0.0;
  for (int r = 0; r < KP; ++r) od += s_o[r][t];

  if (nchunks == 1) {
    const double l = s_ml[1];
    ((T*)a.o_out)[(size_t)b * a.ldo + h * HD + t] = round_to<T>(l > 0.0 ? od / l : 0.0);
    return;
  }
  double* mypart = a.part + (((size_t)b * a.n_heads + h) * a.max_chunks + chunk) * (HD + 2);
  mypart[2 + t] = od;
  if (t == 0) {
    mypart[0] = s_ml[0];
    mypart[1] = s_ml[1];
  }
}

// Merge the chunk partials of (slot blockIdx.y, head blockIdx.x) in chunk
// order: o = sum_c e^{m_c - M} (p.V)_c / sum_c e^{m_c - M} l_c.
template <typename T, int HD>
__global__ __launch_bounds__(HD) void attn_combine_kernel(AttnArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  if (!a.live[b]) return;
  int nvalid, excl;
  window_of(a, b, nvalid, excl);
  const int nchunks = (nvalid + ATTN_CHUNK - 1) / ATTN_CHUNK;
  if (nchunks <= 1) return;  // written directly by attn_kernel
  const double* parts = a.part + ((size_t)b * a.n_heads + h) * a.max_chunks * (HD + 2);
  __shared__ double s_m[HD / 64 > 0 ? HD / 64 : 1];
  __shared__ double s_w[ATTN_MAX_CHUNKS];
  // M = max over the chunk maxima (exact, so any reduction order gives the same M)
  double mloc = -INFINITY;
  for (int c = t; c < nchunks; c += HD) mloc = fmax(mloc, parts[(size_t)c * (HD + 2)]);
#pragma unroll
  for (int off = (HD < 64 ? HD : 64) / 2; off > 0; off >>= 1)
    mloc = fmax(mloc, shfl_xor_d(mloc, off));
  if ((t & 63) == 0) s_m[t >> 6] = mloc;
  __syncthreads();
  double M = s_m[0];
  for (int w = 1; w < HD / 64; ++w) M = fmax(M, s_m[w]);
  // chunk weights e^{m_c - M}, one exp per chunk
  for (int c = t; c < nchunks; c += HD) {
    const double mc = parts[(size_t)c * (HD + 2)];
    s_w[c] = (mc == -INFINITY) ? 0.0 : exp(mc - M);
  }
  __syncthreads();
  double L = 0.0, O = 0.0;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) {
    const double* pc = parts + (size_t)c * (HD + 2);
    const double w = s_w[c];
    L = fma(pc[1], w, L);
    O = fma(pc[2 + t], w, O);
  }
  ((T*)a.o_out)[(size_t)b * a.ldo + h * HD + t] = round_to<T>(L > 0.0 ? O / L : 0.0);
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
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) ss += shfl_xor_d(ss, off);
  if (r == 0 && b < a.B) a.ssq_out[(size_t)blockIdx.x * a.B + b] = ss;
}

// Depformer substep entry: y = (W_in[s] hidden) + E_s[previous token].
template <typename T>
__global__ __launch_bounds__(64) void entry_kernel(EntryArgs a) {
  const int r = threadIdx.x & 15;
  const int b = blockIdx.y * 4 + (threadIdx.x >> 4);
  const int row = blockIdx.x * 16 + r;
  int tok = 0;
  if (a.prev_part != nullptr) {
    // reduce the previous head's partials of column b over the 16 lanes of this column
    double bv = -INFINITY;
    int bi = 0x7fffffff;
    if (b < a.B)
      for (int i = r; i < a.prev_tiles; i += 16) {
        const ArgPart p = a.prev_part[(size_t)i * a.B + b];
        if (arg_better(p.v, p.i, bv, bi)) {
          bv = p.v;
          bi = p.i;
        }
      }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      const double ov = shfl_xor_d(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (arg_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    tok = (bi < a.prev_n) ? bi : 0;
    if (blockIdx.x == 0 && r == 0 && b < a.B) a.prev[(size_t)b * a.prev_stride] = tok;
  } else if (b < a.B) {
    tok = a.prev[(size_t)b * a.prev_stride];
  }
  double acc = 0.0;
  if (b < a.B && row < a.D) {
    acc = a.pre[(size_t)b * a.ldpre + (size_t)a.s * a.D + row] +
          to_d(((const T*)a.table)[(size_t)tok * a.D + row]);
    a.y[(size_t)b * a.D + row] = acc;
  }
  double ss = acc * acc;
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) ss += shfl_xor_d(ss, off);
  if (r == 0 && b < a.B) a.ssq_out[(size_t)blockIdx.x * a.B + b] = ss;
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
// Launchers
// ---------------------------------------------------------------------------

int gemm_tiles(int epi, int N) { return epi == EPI_SWIGLU ? (N + 7) / 8 : (N + 15) / 16; }

int gemm_kw(int dtype, int B, int K) {
  (void)dtype;
  // temporal projections (K >= 4096): 8 waves; depformer ones: 4 waves
  return K >= 4096 ? 8 : 4;
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

template <typename T, int NB, int KW>
static hipError_t launch_gemm_kw(int epi, const GemmArgs& a, hipStream_t st) {
  dim3 grid(gemm_tiles(epi, a.N)), block(64 * KW);
  switch (epi) {
    case EPI_STORE:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_STORE>), grid, block, 0, st, a);
      break;
    case EPI_RESID:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_RESID>), grid, block, 0, st, a);
      break;
    case EPI_QKV:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_QKV>), grid, block, 0, st, a);
      break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_SWIGLU>), grid, block, 0, st, a);
      break;
    case EPI_ARGMAX:
      hipLaunchKernelGGL((gemm_kernel<T, NB, KW, EPI_ARGMAX>), grid, block, 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
    if (pro == PRO_NORM)
      hipLaunchKernelGGL((norm_kernel<T, PRO_NORM>), dim3(a.B), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((norm_kernel<T, PRO_CAST>), dim3(a.B), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    b.X = a.xn_out;
    b.ldx = a.K;
  }
  const int nb = a.B <= 16 ? 1 : (a.B <= 32 ? 2 : 4);
  const int kwm = kw >= 8 ? 8 : 4;
  if (nb == 1)
    return kwm == 8 ? launch_gemm_kw<T, 1, 8>(epi, b, st) : launch_gemm_kw<T, 1, 4>(epi, b, st);
  if (nb == 2)
    return kwm == 8 ? launch_gemm_kw<T, 2, 8>(epi, b, st) : launch_gemm_kw<T, 2, 4>(epi, b, st);
  return launch_gemm_kw<T, 4, 4>(epi, b, st);
}

hipError_t launch_gemm(int dtype, int kw, int pro, int epi, const GemmArgs& a, hipStream_t st) {
  if (a.B < 1 || a.B > 64 || a.N < 1 || a.K < 1) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? launch_gemm_t<__bf16>(kw, pro, epi, a, st)
                          : launch_gemm_t<float>(kw, pro, epi, a, st);
}

template <typename T>
static hipError_t launch_attn_t(int hd, const AttnArgs& a, int B, hipStream_t st) {
  dim3 grid(a.max_chunks, a.n_heads, B), block(256);
  switch (hd) {
    case 32: hipLaunchKernelGGL((attn_kernel<T, 32>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((attn_kernel<T, 64>), grid, block, 0, st, a); break;
    case 128: hipLaunchKernelGGL((attn_kernel<T, 128>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn(int dtype, int hd, const AttnArgs& a, int B, hipStream_t st) {
  return dtype == DT_BF16 ? launch_attn_t<__bf16>(hd, a, B, st) : launch_attn_t<float>(hd, a, B, st);
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
                                int stride, hipStream_t st) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(B), dim3(256), 0, st, part, n_tiles, n_rows, B,
                     tok, stride);
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
