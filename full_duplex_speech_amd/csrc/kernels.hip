// kernels.hip -- gfx950 kernels of the Moshi/PersonaPlex frame step.
//
// Everything on the step's path runs here:
//  * gemm_kernel: every projection (q|k|v, o, gate|up, down, text head,
//    depformer input projections and heads). Weights stream from HBM once per
//    step in 16-byte loads; each 64-lane wave owns 16 weight rows and a slice
//    of K; the batch of session columns is the N side of a bf16 (or fp32)
//    MFMA 16x16 tile, so the same kernel serves one session (15 idle columns,
//    HBM-bound) and 64 sessions (weights read once for all).
//    Prologues fuse the RMSNorm (from per-tile sums of squares written by the
//    producer of the residual) and the bf16 rounding of the input vector;
//    epilogues fuse RoPE + ring-cache write, the residual add, SiLU(gate)*up,
//    and the greedy argmax (per-tile maxima, the last workgroup reduces).
//  * attn_kernel: sliding-window decode attention over the per-slot ring of
//    K/V; one workgroup per (64-key chunk, head, slot); partial softmax
//    statistics are combined in a fixed chunk order by the last workgroup of
//    each (slot, head).
//  * embed_kernel / entry_kernel: the summed 17-channel embedding and the
//    depformer substep entry (projection of the hidden state + embedding of
//    the previous token), both writing sums of squares for the next norm.
//
// Model (pages): mobius PR #368 "P2 - Moshi LM" (RMSNorm eps 1e-8, RoPE theta
// 1e4, sliding-window causal attention, fused gate/up SwiGLU, depformer with
// per-substep linears, no RoPE, causal over substeps); vLLM-Omni recipe
// "PersonaPlex", "Architecture" (3000-frame ring window, 17-row token column).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace moshi {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte group

template <typename T>
struct VecOf;
template <>
struct VecOf<__bf16> {
  static constexpr int N = 8;  // elements per 16-byte load
};
template <>
struct VecOf<float> {
  static constexpr int N = 4;
};

__device__ __forceinline__ float to_f(__bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f(float v) { return v; }
template <typename T>
__device__ __forceinline__ T from_f(float v);
template <>
__device__ __forceinline__ __bf16 from_f<__bf16>(float v) {
  return (__bf16)v;  // round to nearest even
}
template <>
__device__ __forceinline__ float from_f<float>(float v) {
  return v;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
// Weights are read once per step: stream them past the caches.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// ---------------------------------------------------------------------------
// Input-vector construction (MFMA B operand, one 16-byte group per lane)
// ---------------------------------------------------------------------------

// 8 (bf16) or 4 (fp32) consecutive input elements k0.. of column col, in the
// model dtype, packed as 16 bytes.
template <typename T, int PRO>
__device__ __forceinline__ u32x4 load_x(const GemmArgs& a, int col, int k0, float rs) {
  constexpr int VEC = VecOf<T>::N;
  if constexpr (PRO == PRO_DIRECT) {
    return ld16((const T*)a.X + (size_t)col * a.ldx + k0);
  } else {
    const float* xp = (const float*)a.X + (size_t)col * a.ldx + k0;
    float xv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      const f32x4 f = *(const f32x4*)(xp + e);
      xv[e] = f[0];
      xv[e + 1] = f[1];
      xv[e + 2] = f[2];
      xv[e + 3] = f[3];
    }
    if constexpr (PRO == PRO_NORM) {
      u32x4 gw = ld16((const T*)a.gain + k0);
      const T* gv = (const T*)&gw;
#pragma unroll
      for (int e = 0; e < VEC; ++e) xv[e] = xv[e] * rs * to_f(gv[e]);
    }
    u32x4 r;
    T* rv = (T*)&r;
#pragma unroll
    for (int e = 0; e < VEC; ++e) rv[e] = from_f<T>(xv[e]);
    return r;
  }
}

template <typename T>
__device__ __forceinline__ f32x4 mma(u32x4 w, u32x4 x, f32x4 acc);
template <>
__device__ __forceinline__ f32x4 mma<__bf16>(u32x4 w, u32x4 x, f32x4 acc) {
  // A = 16 weight rows x 32 k (lane: row lane%16, k 8*(lane/16)..+7);
  // B = 32 k x 16 columns (lane: column lane%16, same k).
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                  __builtin_bit_cast(bf16x8, x), acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mma<float>(u32x4 w, u32x4 x, f32x4 acc) {
  // Four 16x16x4 steps; step c pairs element c of every lane (k-slot lane/16).
  const f32x4 wf = __builtin_bit_cast(f32x4, w);
  const f32x4 xf = __builtin_bit_cast(f32x4, x);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[0], xf[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[1], xf[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[2], xf[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[3], xf[3], acc, 0, 0, 0);
  return acc;
}

// Weight row read by tile row t of tile `tile`. EPI_SWIGLU interleaves units:
// even tile rows are gate rows, odd tile rows the matching up rows.
template <int EPI>
__device__ __forceinline__ int tile_row(int tile, int t, int N, bool& ok) {
  if constexpr (EPI == EPI_SWIGLU) {
    int u = tile * 8 + (t >> 1);
    ok = u < N;
    return (t & 1) ? N + u : u;
  } else {
    int r = tile * 16 + t;
    ok = r < N;
    return r;
  }
}

__device__ __forceinline__ bool arg_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// ---------------------------------------------------------------------------
// Projection kernel
// ---------------------------------------------------------------------------

template <typename T, int NB, int KSPLIT, int PRO, int EPI>
__global__ __launch_bounds__(64 * KSPLIT) void gemm_kernel(GemmArgs a) {
  constexpr int VEC = VecOf<T>::N;
  constexpr int KSTEP = 4 * VEC;  // k covered by one 16-byte load per lane
  constexpr int U = 4;            // loads in flight per lane per operand
  constexpr int NCOL = 16 * NB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x;

  __shared__ float s_r[NCOL];
  __shared__ f32x4 s_acc[KSPLIT][NB][64];
  __shared__ int s_last;

  // RMSNorm scale of every column from the producer's per-tile sums of squares.
  if constexpr (PRO == PRO_NORM) {
    constexpr int TPC = 64 * KSPLIT / NCOL;  // threads per column (power of two <= 64)
    const int col = threadIdx.x / TPC;
    const int part = threadIdx.x % TPC;
    float s = 0.f;
    if (col < a.B)
      for (int t = part; t < a.n_ssq; t += TPC) s += a.ssq[(size_t)t * a.B + col];
#pragma unroll
    for (int off = TPC / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (part == 0) s_r[col] = (col < a.B) ? 1.0f / sqrtf(s / (float)a.K + a.eps) : 0.f;
    __syncthreads();
  }

  bool rok;
  const int wrow = tile_row<EPI>(tile, r16, a.N, rok);
  const T* wbase = (const T*)a.W + (size_t)(rok ? wrow : 0) * a.K + g * VEC;
  const int nsteps = (a.K + KSTEP - 1) / KSTEP;
  const int s0 = (wave * nsteps) / KSPLIT;
  const int s1 = ((wave + 1) * nsteps) / KSPLIT;
  const bool write_xn = (PRO != PRO_DIRECT) && a.xn_out != nullptr && tile == 0;

  float rs[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) rs[nb] = (PRO == PRO_NORM) ? s_r[nb * 16 + r16] : 1.f;

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = s0; st < s1; st += U) {
    u32x4 wv[U];
    u32x4 xv[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (st + u) * KSTEP + g * VEC;
      const bool kok = (st + u < s1) && (k0 < a.K);
      wv[u] = (kok && rok) ? ld16_stream(wbase + (size_t)(st + u) * KSTEP) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (st + u) * KSTEP + g * VEC;
      const bool kok = (st + u < s1) && (k0 < a.K);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = nb * 16 + r16;
        xv[u][nb] = (kok && col < a.B) ? load_x<T, PRO>(a, col, k0, rs[nb]) : u32x4{0u, 0u, 0u, 0u};
        if (write_xn && kok && col < a.B)
          *(u32x4*)((T*)a.xn_out + (size_t)col * a.K + k0) = xv[u][nb];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = mma<T>(wv[u], xv[u][nb], acc[nb]);
  }

  // Split-K reduction over the waves, fixed order.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) s_acc[wave][nb][lane] = acc[nb];
  __syncthreads();

  if (wave == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 v = s_acc[0][nb][lane];
#pragma unroll
      for (int w = 1; w < KSPLIT; ++w) v += s_acc[w][nb][lane];
      const int col = nb * 16 + r16;
      const bool cok = col < a.B;
      // lane holds tile rows 4g..4g+3 of column col
      if constexpr (EPI == EPI_STORE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = tile * 16 + 4 * g + i;
          if (cok && row < a.N) a.out[(size_t)col * a.ldo + row] = v[i];
        }
      } else if constexpr (EPI == EPI_RESID) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = tile * 16 + 4 * g + i;
          if (cok && row < a.N) {
            float* p = a.resid + (size_t)col * a.ldr + row;
            const float xn = *p + v[i];
            *p = xn;
            ss += xn * xn;
          }
        }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        if (g == 0 && cok) a.ssq_out[(size_t)tile * a.B + col] = ss;
      } else if constexpr (EPI == EPI_QKV) {
        const int row0 = tile * 16 + 4 * g;  // 16-row tiles never straddle a part or a head
        const int part = row0 / a.dq;
        const int din = row0 - part * a.dq;
        const int head = din / a.hd;
        const int d0 = din - head * a.hd;
        float vals[4] = {v[0], v[1], v[2], v[3]};
        if (cok && row0 < a.N) {
          if (a.inv_freq != nullptr && part < 2) {
            const double p = (double)a.pos[col];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const double ang = p * a.inv_freq[(d0 >> 1) + j];
              double sn, cs;
              sincos(ang, &sn, &cs);
              const float c = (float)cs, s = (float)sn;
              const float x0 = vals[2 * j], x1 = vals[2 * j + 1];
              vals[2 * j] = x0 * c - x1 * s;
              vals[2 * j + 1] = x0 * s + x1 * c;
            }
          }
          if (part == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a.q_out[(size_t)col * a.dq + din + i] = vals[i];
          } else if (a.live[col]) {
            const int widx = a.pos ? (int)(a.pos[col] % a.cap) : a.scalar_widx;
            T* dst = (T*)(part == 1 ? a.ring_k : a.ring_v) + (size_t)col * a.slot_stride +
                     a.layer_off + (size_t)head * a.head_stride + (size_t)widx * a.hd + d0;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = from_f<T>(vals[i]);
          }
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int u = tile * 8 + 2 * g + j;
          if (cok && u < a.N) {
            const float gt = v[2 * j], up = v[2 * j + 1];
            const float act = gt / (1.0f + expf(-gt)) * up;
            ((T*)a.act)[(size_t)col * a.lda + u] = from_f<T>(act);
          }
        }
      } else if constexpr (EPI == EPI_ARGMAX) {
        // NaN never wins: it compares as -inf; rows past N carry index INT_MAX.
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = tile * 16 + 4 * g + i;
          if (row < a.N) {
            if (cok) a.out[(size_t)col * a.ldo + row] = v[i];
            const float val = (v[i] != v[i]) ? -INFINITY : v[i];
            if (bi == 0x7fffffff || val > bv) {
              bv = val;
              bi = row;
            }
          }
        }
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
          const float ov = __shfl_xor(bv, off);
          const int oi = __shfl_xor(bi, off);
          if (arg_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
          }
        }
        if (g == 0 && cok) a.apart[(size_t)tile * a.B + col] = ArgPart{bv, bi};
      }
    }
  }

  if constexpr (EPI == EPI_ARGMAX) {
    // The last workgroup to finish reduces the per-tile maxima of every column.
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(a.ticket, 1u) == gridDim.x - 1) ? 1 : 0;
    __syncthreads();
    if (s_last) {
      __threadfence();
      constexpr int TPC = 64 * KSPLIT / NCOL;
      const int col = threadIdx.x / TPC;
      const int part = threadIdx.x % TPC;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      if (col < a.B) {
        for (int t = part; t < (int)gridDim.x; t += TPC) {
          const ArgPart p = a.apart[(size_t)t * a.B + col];
          if (arg_better(p.v, p.i, bv, bi)) {
            bv = p.v;
            bi = p.i;
          }
        }
      }
#pragma unroll
      for (int off = TPC / 2; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (arg_better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (part == 0 && col < a.B) a.tok_out[(size_t)col * a.tok_stride] = (bi < a.N) ? bi : 0;
      if (threadIdx.x == 0) atomicExch(a.ticket, 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// Sliding-window decode attention over a ring of K/V
// ---------------------------------------------------------------------------

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
  int nvalid, excl = -1;
  if (a.pos != nullptr) {
    const int64_t p = a.pos[b];
    nvalid = (int)(p + 1 < (int64_t)a.cap ? p + 1 : (int64_t)a.cap);
    if (a.mask_oldest && p >= (int64_t)a.cap - 1) excl = (int)((p + 1) % a.cap);
  } else {
    nvalid = a.scalar_nvalid;
  }
  const int nchunks = (nvalid + C - 1) / C;
  if (chunk >= nchunks) return;

  __shared__ float s_p[C];
  __shared__ float s_o[KP][HD + 1];
  __shared__ float s_ml[2];
  __shared__ int s_last;

  const int kd = t % TK;
  const int kk = t / TK;
  const float scale = 1.0f / sqrtf((float)HD);
  float qv[VEC];
  const float* qp = a.q + (size_t)b * a.ldq + h * HD + kd * VEC;
#pragma unroll
  for (int e = 0; e < VEC; ++e) qv[e] = qp[e] * scale;

  const size_t base = (size_t)b * a.slot_stride + a.layer_off + (size_t)h * a.head_stride;
  const T* kbase = (const T*)a.ring_k + base;
  const T* vbase = (const T*)a.ring_v + base;

  // scores
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int j = chunk * C + ps * KP + kk;
    const bool ok = j < nvalid && j != excl;
    float d = 0.f;
    if (ok) {
      u32x4 kw = ld16(kbase + (size_t)j * HD + kd * VEC);
      const T* kvp = (const T*)&kw;
#pragma unroll
      for (int e = 0; e < VEC; ++e) d += qv[e] * to_f(kvp[e]);
    }
#pragma unroll
    for (int off = TK / 2; off > 0; off >>= 1) d += __shfl_xor(d, off);
    if (kd == 0) s_p[ps * KP + kk] = ok ? d : -INFINITY;
  }
  __syncthreads();
  if (t < 64) {
    float sv = (t < C) ? s_p[t] : -INFINITY;
    float m = sv;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float pj = (m == -INFINITY || sv == -INFINITY) ? 0.f : expf(sv - m);
    float l = pj;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (t < C) s_p[t] = pj;
    if (t == 0) {
      s_ml[0] = m;
      s_ml[1] = l;
    }
  }
  __syncthreads();

  // p . V
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int j = chunk * C + ps * KP + kk;
    const float pj = s_p[ps * KP + kk];
    if (j < nvalid && pj != 0.f) {
      u32x4 vw = ld16(vbase + (size_t)j * HD + kd * VEC);
      const T* vvp = (const T*)&vw;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += pj * to_f(vvp[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) s_o[kk][kd * VEC + e] = acc[e];
  __syncthreads();
  float od = 0.f;
  if (t < HD) {
    for (int r = 0; r < KP; ++r) od += s_o[r][t];
  }

  T* optr = (T*)a.o_out + (size_t)b * a.ldo + h * HD;
  if (nchunks == 1) {
    if (t < HD) {
      const float l = s_ml[1];
      optr[t] = from_f<T>(l > 0.f ? od / l : 0.f);
    }
    return;
  }
  float* mypart = a.part + (((size_t)b * a.n_heads + h) * a.max_chunks + chunk) * (HD + 2);
  if (t < HD) mypart[2 + t] = od;
  if (t == 0) {
    mypart[0] = s_ml[0];
    mypart[1] = s_ml[1];
  }
  __threadfence();
  __syncthreads();
  unsigned* tk = a.ticket + (size_t)b * a.n_heads + h;
  if (t == 0) s_last = (atomicAdd(tk, 1u) == (unsigned)(nchunks - 1)) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // combine the chunks in order 0..nchunks-1
  const float* parts = a.part + ((size_t)b * a.n_heads + h) * a.max_chunks * (HD + 2);
  float M = -INFINITY;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, parts[(size_t)c * (HD + 2)]);
  if (t < HD) {
    float L = 0.f, O = 0.f;
    for (int c = 0; c < nchunks; ++c) {
      const float* pc = parts + (size_t)c * (HD + 2);
      const float mc = pc[0];
      if (mc == -INFINITY) continue;
      const float w = expf(mc - M);
      L += pc[1] * w;
      O += pc[2 + t] * w;
    }
    optr[t] = from_f<T>(L > 0.f ? O / L : 0.f);
  }
  if (t == 0) atomicExch(tk, 0u);
}

// ---------------------------------------------------------------------------
// Summed channel embedding and depformer substep entry
// ---------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(64) void embed_kernel(EmbedArgs a) {
  const int r = threadIdx.x & 15;
  const int b = blockIdx.y * 4 + (threadIdx.x >> 4);
  const int row = blockIdx.x * 16 + r;
  float acc = 0.f;
  if (b < a.B && row < a.D) {
    const bool live = a.live[b] != 0;
    for (int c = 0; c < a.n_ch; ++c) {
      // Free slots embed code 0. A live code outside the table is clamped to
      // a valid row (never read out of bounds) and flagged for the host.
      int code = live ? a.frames[(size_t)b * a.n_ch + c] : 0;
      const int rows = (c == 0) ? a.rows_text : a.rows_audio;
      if (code < 0 || code >= rows) {
        if (row == 0) atomicOr(a.bad_code, 1);
        code = code < 0 ? 0 : rows - 1;
      }
      acc += to_f(((const T*)a.tables[c])[(size_t)code * a.D + row]);
    }
    a.x[(size_t)b * a.D + row] = acc;
  }
  float ss = acc * acc;
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (r == 0 && b < a.B) a.ssq_out[(size_t)blockIdx.x * a.B + b] = ss;
}

template <typename T>
__global__ __launch_bounds__(64) void entry_kernel(EntryArgs a) {
  const int r = threadIdx.x & 15;
  const int b = blockIdx.y * 4 + (threadIdx.x >> 4);
  const int row = blockIdx.x * 16 + r;
  float acc = 0.f;
  if (b < a.B && row < a.D) {
    const int tok = a.prev[(size_t)b * a.prev_stride];
    acc = a.pre[(size_t)b * a.ldpre + (size_t)a.s * a.D + row] +
          to_f(((const T*)a.table)[(size_t)tok * a.D + row]);
    a.y[(size_t)b * a.D + row] = acc;
  }
  float ss = acc * acc;
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
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

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

int gemm_nb(int B) { return B <= 16 ? 1 : (B <= 32 ? 2 : 4); }

int gemm_tiles(int epi, int N) { return epi == EPI_SWIGLU ? (N + 7) / 8 : (N + 15) / 16; }

template <typename T, int NB, int KW>
static hipError_t launch_gemm_kw(int pro, int epi, const GemmArgs& a, hipStream_t st) {
  dim3 grid(gemm_tiles(epi, a.N)), block(64 * KW);
#define MOSHI_GEMM_CASE(P, E)                                                    \
  if (pro == P && epi == E) {                                                   \
    hipLaunchKernelGGL((gemm_kernel<T, NB, KW, P, E>), grid, block, 0, st, a); \
    return hipGetLastError();                                                   \
  }
  MOSHI_GEMM_CASE(PRO_NORM, EPI_QKV)
  MOSHI_GEMM_CASE(PRO_DIRECT, EPI_RESID)
  MOSHI_GEMM_CASE(PRO_NORM, EPI_SWIGLU)
  MOSHI_GEMM_CASE(PRO_NORM, EPI_ARGMAX)
  MOSHI_GEMM_CASE(PRO_DIRECT, EPI_STORE)
  MOSHI_GEMM_CASE(PRO_CAST, EPI_ARGMAX)
#undef MOSHI_GEMM_CASE
  return hipErrorInvalidValue;
}

template <typename T, int NB>
static hipError_t launch_gemm_nb(int kw, int pro, int epi, const GemmArgs& a, hipStream_t st) {
  if (kw == 8) return launch_gemm_kw<T, NB, 8>(pro, epi, a, st);
  if (kw == 4) return launch_gemm_kw<T, NB, 4>(pro, epi, a, st);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_gemm_t(int kw, int pro, int epi, const GemmArgs& a, hipStream_t st) {
  switch (gemm_nb(a.B)) {
    case 1: return launch_gemm_nb<T, 1>(kw, pro, epi, a, st);
    case 2: return launch_gemm_nb<T, 2>(kw, pro, epi, a, st);
    case 4: return launch_gemm_nb<T, 4>(kw, pro, epi, a, st);
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

hipError_t launch_embed(int dtype, const EmbedArgs& a, hipStream_t st) {
  dim3 grid((a.D + 15) / 16, (a.B + 3) / 4), block(64);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(embed_kernel<__bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(embed_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_advance(int64_t* pos, const int* live, int B, hipStream_t st) {
  hipLaunchKernelGGL(advance_kernel, dim3((B + 63) / 64), dim3(64), 0, st, pos, live, B);
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

}  // namespace moshi
