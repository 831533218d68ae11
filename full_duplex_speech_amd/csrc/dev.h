// dev.h -- device code shared by the per-operation kernels (kernels.hip) and
// the persistent one-session step kernel (step.hip): conversions, rounding,
// the projection (GEMV) loop with its prologues and epilogues, and the
// windowed-attention pieces.
//
// Template flag C ("coherent"): inside the persistent step kernel, vectors
// produced by one workgroup are read by others after a grid barrier, so every
// such load and store is an agent-scope relaxed atomic (global_load/store
// with sc1: it bypasses the non-coherent caches, so other XCDs see it).
// Weights, tables and anything not written during the kernel use ordinary
// loads. With C = false (one kernel per operation) kernel boundaries order
// everything and plain accesses are used.
#pragma once

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

// Every device pointer here is global memory; saying so makes the compiler
// emit global_* instead of flat_* instructions (flat ones also count against
// lgkmcnt, so every workgroup barrier would wait for loads in flight).
#define MOSHI_GLB __attribute__((address_space(1)))

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const MOSHI_GLB u32x4*)p; }
// Weights are read once per step: stream them past the caches (in the long
// projections this beats plain loads, which evict the rings and activations).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load((const MOSHI_GLB u32x4*)p);
}

// ---- activation accesses (see C above) -------------------------------------

#define MOSHI_RLX __ATOMIC_RELAXED
#define MOSHI_AGT __HIP_MEMORY_SCOPE_AGENT

template <bool C>
__device__ __forceinline__ uint64_t ld_u64(const void* p) {
  if constexpr (C) return __hip_atomic_load((MOSHI_GLB uint64_t*)p, MOSHI_RLX, MOSHI_AGT);
  else return *(const MOSHI_GLB uint64_t*)p;
}
template <bool C>
__device__ __forceinline__ void st_u64(void* p, uint64_t v) {
  if constexpr (C) __hip_atomic_store((MOSHI_GLB uint64_t*)p, v, MOSHI_RLX, MOSHI_AGT);
  else *(MOSHI_GLB uint64_t*)p = v;
}
template <bool C>
__device__ __forceinline__ void st_u32(void* p, uint32_t v) {
  if constexpr (C) __hip_atomic_store((MOSHI_GLB uint32_t*)p, v, MOSHI_RLX, MOSHI_AGT);
  else *(MOSHI_GLB uint32_t*)p = v;
}
template <bool C>
__device__ __forceinline__ void st_u16(void* p, uint16_t v) {
  if constexpr (C) __hip_atomic_store((MOSHI_GLB uint16_t*)p, v, MOSHI_RLX, MOSHI_AGT);
  else *(MOSHI_GLB uint16_t*)p = v;
}
template <bool C>
__device__ __forceinline__ int ld_i32(const int* p) {
  if constexpr (C) return __hip_atomic_load((MOSHI_GLB int*)p, MOSHI_RLX, MOSHI_AGT);
  else return *(const MOSHI_GLB int*)p;
}
template <bool C>
__device__ __forceinline__ void st_i32(int* p, int v) {
  if constexpr (C) __hip_atomic_store((MOSHI_GLB int*)p, v, MOSHI_RLX, MOSHI_AGT);
  else *(MOSHI_GLB int*)p = v;
}
// plain read-only loads of global memory (tables, positions, gains)
template <typename V>
__device__ __forceinline__ V ldg(const V* p) {
  return *(const MOSHI_GLB V*)p;
}
template <bool C>
__device__ __forceinline__ double ld_f64(const double* p) {
  return __builtin_bit_cast(double, ld_u64<C>(p));
}
template <bool C>
__device__ __forceinline__ void st_f64(double* p, double v) {
  st_u64<C>(p, __builtin_bit_cast(uint64_t, v));
}
// 16-byte coherent load at byte offset `off` from a workgroup-uniform base:
// one buffer_load_dwordx4 with sc1 (the same count of loads in flight as a
// plain 16-byte load, which keeps the compiler's wait counts exact).
__device__ __forceinline__ u32x4 ld16_coh(const void* base, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, /*sc1*/ 16);
}

// one 16-byte group
template <bool C>
__device__ __forceinline__ u32x4 ld_grp(const void* p) {
  if constexpr (C) {
    const uint64_t a = ld_u64<true>(p), b = ld_u64<true>((const char*)p + 8);
    return u32x4{(unsigned)a, (unsigned)(a >> 32), (unsigned)b, (unsigned)(b >> 32)};
  } else {
    return ld16(p);
  }
}
template <bool C>
__device__ __forceinline__ void st_grp(void* p, u32x4 v) {
  if constexpr (C) {
    st_u64<true>(p, (uint64_t)v[0] | ((uint64_t)v[1] << 32));
    st_u64<true>((char*)p + 8, (uint64_t)v[2] | ((uint64_t)v[3] << 32));
  } else {
    *(MOSHI_GLB u32x4*)p = v;
  }
}

// threadIdx.x, re-read at every use site: values derived from it are then not
// hoisted out of the layer loops of the step kernel, where they would stay
// live across every operation and exhaust the registers.
__device__ __forceinline__ int tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
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
// itself is not on it; then d decides the direction. Inf/NaN keep their
// class (a NaN stays quiet). All cases are computed and selected, so a wave
// does not branch per value.
__device__ __forceinline__ unsigned short bf16_bits_rne(double d) {
  const float f = (float)d;
  const unsigned int u = __float_as_uint(f);
  const unsigned int hi = u >> 16, lo = u & 0xffffu;
  const unsigned int special = hi | (lo ? 0x40u : 0u);
  const unsigned int tie = hi + (fabs(d) > fabs((double)f) ? 1u : 0u);
  const unsigned int rne = (u + 0x7fffu + (hi & 1u)) >> 16;
  unsigned int r = (lo == 0x8000u && (double)f != d) ? tie : rne;
  r = (u & 0x7f800000u) == 0x7f800000u ? special : r;
  return (unsigned short)r;
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

// Stored bits of round_to<T>(d), zero-extended.
template <typename T>
__device__ __forceinline__ uint32_t stored_bits(double d);
template <>
__device__ __forceinline__ uint32_t stored_bits<__bf16>(double d) {
  return bf16_bits_rne(d);
}
template <>
__device__ __forceinline__ uint32_t stored_bits<float>(double d) {
  return __float_as_uint((float)d);
}

// n consecutive rounded values (n = 1, 2 or 4) stored at p.
template <typename T, bool C>
__device__ __forceinline__ void store_rounded(T* p, const double* v, int n) {
  if constexpr (sizeof(T) == 2) {
    if (n == 4) {
      uint64_t w = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) w |= (uint64_t)stored_bits<T>(v[i]) << (16 * i);
      st_u64<C>(p, w);
    } else if (n == 2) {
      st_u32<C>(p, stored_bits<T>(v[0]) | (stored_bits<T>(v[1]) << 16));
    } else {
      st_u16<C>(p, (uint16_t)stored_bits<T>(v[0]));
    }
  } else {
    if (n == 4) {
      st_grp<C>(p, u32x4{stored_bits<T>(v[0]), stored_bits<T>(v[1]), stored_bits<T>(v[2]),
                         stored_bits<T>(v[3])});
    } else if (n == 2) {
      st_u64<C>(p, (uint64_t)stored_bits<T>(v[0]) | ((uint64_t)stored_bits<T>(v[1]) << 32));
    } else {
      st_u32<C>(p, stored_bits<T>(v[0]));
    }
  }
}

// ---- the one-session input vector (built in LDS, rounded to the model dtype)

// Elements 2p, 2p+1 of an fp64 vector: one 16-byte load (coherent: sc1).
template <bool C>
__device__ __forceinline__ void ld_pair_f64(const double* x, int p, double& v0, double& v1) {
  const u32x4 q = C ? ld16_coh(x, (uint32_t)p * 16u) : ld16(x + 2 * (size_t)p);
  v0 = __hiloint2double((int)q[1], (int)q[0]);
  v1 = __hiloint2double((int)q[3], (int)q[2]);
}
// Elements 2p, 2p+1 of a model-dtype vector (gains), as doubles.
__device__ __forceinline__ void ld_pair_d(const __bf16* g, int p, double& v0, double& v1) {
  const uint32_t u = ldg((const uint32_t*)g + p);
  v0 = (double)__uint_as_float(u << 16);
  v1 = (double)__uint_as_float(u & 0xffff0000u);
}
__device__ __forceinline__ void ld_pair_d(const float* g, int p, double& v0, double& v1) {
  const uint64_t u = ldg((const uint64_t*)g + p);
  v0 = (double)__uint_as_float((uint32_t)u);
  v1 = (double)__uint_as_float((uint32_t)(u >> 32));
}
// Rounded pair stored to LDS (and, if xn, to global memory).
template <typename T, bool C>
__device__ __forceinline__ void put_pair(T* xs, T* xn, int p, double v0, double v1) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t u = stored_bits<T>(v0) | (stored_bits<T>(v1) << 16);
    *(uint32_t*)(xs + 2 * p) = u;
    if (xn != nullptr) st_u32<C>(xn + 2 * p, u);
  } else {
    const uint64_t u = (uint64_t)stored_bits<T>(v0) | ((uint64_t)stored_bits<T>(v1) << 32);
    *(uint64_t*)(xs + 2 * p) = u;
    if (xn != nullptr) st_u64<C>(xn + 2 * p, u);
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

__device__ __forceinline__ int n_tiles_of(int epi, int N) {
  return epi == EPI_SWIGLU ? (N + 7) / 8 : (N + 15) / 16;
}

__device__ __forceinline__ bool arg_better(double v, int i, double bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ double shfl_xor_d(double v, int m) {
  return __hiloint2double(__shfl_xor(__double2hiint(v), m), __shfl_xor(__double2loint(v), m));
}

// ---- wave reductions on DPP lane moves (a few cycles each, where a shuffle
// through ds_bpermute costs ~100) ----

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_d(double v, int lane) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                          __builtin_amdgcn_readlane(__double2loint(v), lane));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within 16

// Sum (MAX = false) or maximum over aligned groups of N lanes (N = 1, 2, 4,
// 8, 16, 32, 64), the result in every lane of the group. The association is
// fixed: pairs, quads, eights, rows of 16, then rows combined in lane order.
// All 64 lanes must be active.
template <int N, bool MAX = false>
__device__ __forceinline__ double group_reduce(double v) {
  auto op = [](double x, double y) { return MAX ? fmax(x, y) : x + y; };
  if constexpr (N >= 2) v = op(v, dpp_d<DPP_XOR1>(v));
  if constexpr (N >= 4) v = op(v, dpp_d<DPP_XOR2>(v));
  if constexpr (N >= 8) v = op(v, dpp_d<DPP_HALF_MIRROR>(v));
  if constexpr (N >= 16) v = op(v, dpp_d<DPP_MIRROR>(v));
  if constexpr (N == 32) {
    const double a = op(readlane_d(v, 0), readlane_d(v, 16));
    const double b = op(readlane_d(v, 32), readlane_d(v, 48));
    v = (__lane_id() < 32) ? a : b;
  } else if constexpr (N == 64) {
    v = op(op(readlane_d(v, 0), readlane_d(v, 16)), op(readlane_d(v, 32), readlane_d(v, 48)));
  }
  return v;
}

// RMSNorm scale 1/sqrt(mean(x^2) + eps) of column col from the producer's
// per-tile sums of squares; every thread of the workgroup gets the same value.
// Threads [0, nthr) split the tiles; fixed-order reduction through `red`.
// rms_finish: the same from each thread's sum of its partials i = t, t +
// nthr, ... (summed in that order).
__device__ __forceinline__ double rms_finish(double s, const GemmArgs& a, double* red, int nthr) {
  const int t = tid();
  s = group_reduce<64>(s);
  if ((t & 63) == 0) red[t >> 6] = s;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < nthr / 64; ++w) tot += red[w];
  __syncthreads();  // `red` may be reused right after
  return 1.0 / sqrt(tot / (double)a.K + a.eps);
}
template <bool C>
__device__ __forceinline__ double rms_scale(const GemmArgs& a, int col, double* red, int nthr) {
  double s = 0.0;
  for (int i = tid(); i < a.n_ssq; i += nthr) s += ld_f64<C>(a.ssq + (size_t)i * a.B + col);
  return rms_finish(s, a, red, nthr);
}

// The one-session input vector -> LDS `xs`, rounded to the model dtype.
// Every thread requests its first XP items (16-byte groups for PRO_DIRECT;
// fp64 element pairs with their gains and the sum-of-squares partials
// otherwise) before it uses any; addresses are clamped, so every lane loads
// and a wave reads contiguous memory. Items past XP per thread are loaded a
// pass at a time. PRO_NORM / PRO_CAST with xn_out: the workgroup with
// `first` also stores the rounded vector there.
template <typename T, int PRO, bool C, int NTH, int XP>
__device__ __forceinline__ void build_input(const GemmArgs& a, T* xs, double* red, bool first) {
  constexpr int VEC = VecOf<T>::N;
  const int t = tid();
  if constexpr (PRO == PRO_DIRECT) {
    const int ng = a.K / VEC;
    auto ld_g = [&](int gi) {
      return C ? ld16_coh(a.X, (uint32_t)gi * 16u) : ld16((const T*)a.X + (size_t)gi * VEC);
    };
    u32x4 q[XP];
#pragma unroll
    for (int j = 0; j < XP; ++j) q[j] = ld_g(t + j * NTH < ng ? t + j * NTH : ng - 1);
#pragma unroll
    for (int j = 0; j < XP; ++j)
      if (t + j * NTH < ng) *(u32x4*)(xs + (size_t)(t + j * NTH) * VEC) = q[j];
    for (int gi = t + XP * NTH; gi < ng; gi += NTH) *(u32x4*)(xs + (size_t)gi * VEC) = ld_g(gi);
  } else {
    const int np = a.K / 2;
    const double* x = (const double*)a.X;
    const T* g = (const T*)a.gain;
    T* xn = first ? (T*)a.xn_out : nullptr;
    double xv[XP][2], gv[XP][2];
#pragma unroll
    for (int j = 0; j < XP; ++j) {
      const int p = t + j * NTH < np ? t + j * NTH : np - 1;
      ld_pair_f64<C>(x, p, xv[j][0], xv[j][1]);
      if constexpr (PRO == PRO_NORM) ld_pair_d(g, p, gv[j][0], gv[j][1]);
    }
    double rs = 1.0;
    if constexpr (PRO == PRO_NORM) {
      const int n = a.n_ssq;
      double sq[XP];
#pragma unroll
      for (int j = 0; j < XP; ++j)
        sq[j] = ld_f64<C>(a.ssq + (size_t)(t + j * NTH < n ? t + j * NTH : n - 1) * a.B);
      double sum = 0.0;
#pragma unroll
      for (int j = 0; j < XP; ++j)
        if (t + j * NTH < n) sum += sq[j];
      for (int i = t + XP * NTH; i < n; i += NTH) sum += ld_f64<C>(a.ssq + (size_t)i * a.B);
      rs = rms_finish(sum, a, red, NTH);
    }
    auto put = [&](int p, const double (&xp)[2], const double (&gp)[2]) {
      const double v0 = PRO == PRO_NORM ? xp[0] * rs * gp[0] : xp[0];
      const double v1 = PRO == PRO_NORM ? xp[1] * rs * gp[1] : xp[1];
      put_pair<T, C>(xs, xn, p, v0, v1);
    };
#pragma unroll
    for (int j = 0; j < XP; ++j)
      if (t + j * NTH < np) put(t + j * NTH, xv[j], gv[j]);
    for (int p = t + XP * NTH; p < np; p += NTH) {
      double xp[2], gp[2] = {1.0, 1.0};
      ld_pair_f64<C>(x, p, xp[0], xp[1]);
      if constexpr (PRO == PRO_NORM) ld_pair_d(g, p, gp[0], gp[1]);
      put(p, xp, gp);
    }
  }
}

// ---- epilogue: tile rows 4g..4g+3 of column col, values v -----------------

template <typename T, int EPI, bool C>
__device__ __forceinline__ void epilogue(const GemmArgs& a, int tile, int g, int col,
                                         const double* v) {
  const bool cok = col < a.B;
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tile * 16 + 4 * g + i;
      if (cok && row < a.N) st_f64<C>(a.out64 + (size_t)col * a.ldo + row, v[i]);
    }
  } else if constexpr (EPI == EPI_RESID) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tile * 16 + 4 * g + i;
      if (cok && row < a.N) {
        double* p = a.resid + (size_t)col * a.ldr + row;
        const double xn = ld_f64<C>(p) + v[i];
        st_f64<C>(p, xn);
        ss += xn * xn;
      }
    }
    // the 4 lanes of this column (g = 0..3) combine in a fixed order
    ss += shfl_xor_d(ss, 16);
    ss += shfl_xor_d(ss, 32);
    if (g == 0 && cok) st_f64<C>(a.ssq_out + (size_t)tile * a.B + col, ss);
  } else if constexpr (EPI == EPI_QKV) {
    const int row0 = tile * 16 + 4 * g;  // 16-row tiles never straddle a part or a head
    const int part = row0 / a.dq;
    const int din = row0 - part * a.dq;
    const int head = din / a.hd;
    const int d0 = din - head * a.hd;
    double vals[4] = {v[0], v[1], v[2], v[3]};
    if (!cok || row0 >= a.N) return;
    if (a.inv_freq != nullptr && part < 2) {
      const double p = (double)ldg(a.pos + col);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const double ang = p * ldg(a.inv_freq + (d0 >> 1) + j);
        double sn, cs;
        sincos(ang, &sn, &cs);
        const double x0 = vals[2 * j], x1 = vals[2 * j + 1];
        vals[2 * j] = x0 * cs - x1 * sn;
        vals[2 * j + 1] = x0 * sn + x1 * cs;
      }
    }
    if (part == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st_f64<C>(a.q_out + (size_t)col * a.dq + din + i, vals[i]);
    } else if (ldg(a.live + col)) {
      const int widx = a.pos ? (int)(ldg(a.pos + col) % a.cap) : a.scalar_widx;
      T* dst = (T*)(part == 1 ? a.ring_k : a.ring_v) + (size_t)col * a.slot_stride + a.layer_off +
               (size_t)head * a.head_stride + (size_t)widx * a.hd + d0;
      store_rounded<T, C>(dst, vals, 4);
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    double r[2];
    int n = 0;
    const int u0 = tile * 8 + 2 * g;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int u = u0 + j;
      if (cok && u < a.N) {
        const double gt = v[2 * j], up = v[2 * j + 1];
        r[j] = gt / (1.0 + exp(-gt)) * up;
        n = j + 1;
      }
    }
    if (n > 0) store_rounded<T, C>((T*)a.act + (size_t)col * a.lda + u0, r, n);
  } else if constexpr (EPI == EPI_ARGMAX) {
    // NaN never wins: it compares as -inf; rows past N carry index INT_MAX.
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tile * 16 + 4 * g + i;
      if (row < a.N) {
        if (cok) *(MOSHI_GLB float*)(a.logits + (size_t)col * a.ldo + row) = (float)v[i];  // host reads
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
    if (g == 0 && cok) {
      const uint64_t vb = __builtin_bit_cast(uint64_t, bv);
      st_grp<C>(a.apart + (size_t)tile * a.B + col,
                u32x4{(unsigned)vb, (unsigned)(vb >> 32), (unsigned)bi, 0u});
    }
  }
}

__device__ __forceinline__ ArgPart unpack_part(u32x4 w) {
  ArgPart p;
  p.v = __builtin_bit_cast(double, (uint64_t)w[0] | ((uint64_t)w[1] << 32));
  p.i = (int)w[2];
  p.pad = 0;
  return p;
}

// Greedy token from per-tile argmax partials [n_tiles] (one session), reduced
// by the whole workgroup of NTH threads (the comparison is exact, so the
// winner does not depend on the order). Indices past n_rows read as 0.
template <int NTH>
__device__ __forceinline__ int reduce_token(const ArgPart* part, int n_tiles, int n_rows) {
  constexpr int NW = NTH / 64;
  __shared__ double s_v[NW];
  __shared__ int s_i[NW];
  const int t = tid();
  double bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = t; i < n_tiles; i += NTH) {
    const ArgPart p = unpack_part(ld_grp<true>(part + i));
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

// Epilogue of the R consecutive rows tile*16 + w*R .. that one wave owns
// (one session, column 0), run by lane 0 with the finished sums v[0..R).
// EPI_RESID writes one sum-of-squares partial per R rows (index row0 / R).
// Inputs of the one-session q/k/v epilogue, read when the projection starts
// so that no tile's epilogue waits on memory (a wait for a load also waits
// for the weight batch in flight): whether the session is live, the ring
// slot written at this step, and with RoPE the cos/sin of position * each
// inverse frequency (LDS, [hd/2][2]; null without RoPE).
struct QkvIn {
  int live, widx;
  const double* cs;
};

// The RoPE table for QkvIn at the session's position: threads [0, nthr)
// compute entries t, t + nthr, ... (hd / 2 <= 64). The caller synchronises
// the workgroup before it is read.
__device__ __forceinline__ void rope_table(const GemmArgs& a, double (*cs)[2], int nthr) {
  const double p = (double)ldg(a.pos);
  for (int i = tid(); i < a.hd / 2; i += nthr) {
    double sn, c;
    sincos(p * ldg(a.inv_freq + i), &sn, &c);
    cs[i][0] = c;
    cs[i][1] = sn;
  }
}

__device__ __forceinline__ QkvIn qkv_in(const GemmArgs& a, const double (*rope)[2]) {
  QkvIn q;
  q.live = ldg(a.live);
  q.widx = a.pos ? (int)(ldg(a.pos) % a.cap) : a.scalar_widx;
  q.cs = a.inv_freq != nullptr ? &rope[0][0] : nullptr;
  return q;
}

// EPI_RESID: rpre holds the residual values of these rows if pre_ok (else
// they are loaded here). EPI_QKV: qin.
template <typename T, int EPI, bool C, int R>
__device__ __forceinline__ void wave_epilogue(const GemmArgs& a, int tile, int w, const double* v,
                                              const double (&rpre)[R], bool pre_ok,
                                              const QkvIn& qin) {
  static_assert(EPI != EPI_ARGMAX, "argmax partials are per tile");
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = tile * 16 + w * R + r;
      if (row < a.N) st_f64<C>(a.out64 + row, v[r]);
    }
  } else if constexpr (EPI == EPI_RESID) {
    const int row0 = tile * 16 + w * R;
    if (row0 >= a.N) return;
    // every load before the first store: a wait for a load also waits for
    // the stores issued before it
    double xn[R];
    if (pre_ok) {
#pragma unroll
      for (int r = 0; r < R; ++r) xn[r] = rpre[r] + v[r];
    } else {
      double rv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) rv[r] = ld_f64<C>(a.resid + (row0 + r < a.N ? row0 + r : row0));
#pragma unroll
      for (int r = 0; r < R; ++r) xn[r] = rv[r] + v[r];
    }
    double ss = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (row0 + r < a.N) {
        st_f64<C>(a.resid + row0 + r, xn[r]);
        ss += xn[r] * xn[r];
      }
    }
    st_f64<C>(a.ssq_out + row0 / R, ss);
  } else if constexpr (EPI == EPI_QKV) {
    const int row0 = tile * 16 + w * R;  // R-row groups never straddle a part or a head
    if (row0 >= a.N) return;
    const int part = row0 / a.dq;
    const int din = row0 - part * a.dq;
    const int head = din / a.hd;
    const int d0 = din - head * a.hd;
    double vals[R];
#pragma unroll
    for (int r = 0; r < R; ++r) vals[r] = v[r];
    if (qin.cs != nullptr && part < 2) {
#pragma unroll
      for (int j = 0; j < R / 2; ++j) {
        const double cs = qin.cs[2 * ((d0 >> 1) + j)], sn = qin.cs[2 * ((d0 >> 1) + j) + 1];
        const double x0 = vals[2 * j], x1 = vals[2 * j + 1];
        vals[2 * j] = x0 * cs - x1 * sn;
        vals[2 * j + 1] = x0 * sn + x1 * cs;
      }
    }
    if (part == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) st_f64<C>(a.q_out + din + r, vals[r]);
    } else if (qin.live) {
      T* dst = (T*)(part == 1 ? a.ring_k : a.ring_v) + a.layer_off + (size_t)head * a.head_stride +
               (size_t)qin.widx * a.hd + d0;
      store_rounded<T, C>(dst, vals, R);
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // rows alternate gate / up of units tile*8 + w*R/2 + k
    constexpr int NU = R / 2;
    const int u0 = tile * 8 + w * NU;
    double r_[NU];
    int n = 0;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      if (u0 + k < a.N) {
        const double gt = v[2 * k], up = v[2 * k + 1];
        r_[k] = gt / (1.0 + exp(-gt)) * up;
        n = k + 1;
      }
    }
    if (n > 0) store_rounded<T, C>((T*)a.act + u0, r_, n);
  }
}

// ---------------------------------------------------------------------------
// One session: fp64 VALU GEMV over row tiles
// ---------------------------------------------------------------------------

// One batch of weights for wave `wave`: U groups (lanes l, l+64, ...) of each
// of its R rows of tile `tile`, batch `bt` along K. Every lane loads: rows
// past the matrix read row 0 and groups past K read the row's last group
// (their sums are never used, and the consumer skips groups past K). No
// conditional zero-fill: writing a load's destination register twice would
// make the compiler wait for every load in flight.
// With live = false every lane reads the matrix's first group instead (one
// line, a placeholder that keeps the number of loads in flight the same on
// every path, so the compiler's wait counts stay exact).
template <typename T, int EPI, int U, int R>
__device__ __forceinline__ void load_wbatch(const GemmArgs& a, int tile, int bt, int lane, int wave,
                                            u32x4 (&w)[U][R], bool live = true) {
  constexpr int VEC = VecOf<T>::N;
  const int ngroups = a.K / VEC;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    bool ok;
    const int rr = tile_row<EPI>(tile, wave * R + r, a.N, ok);
    const T* wr = (const T*)a.W + (size_t)(ok ? rr : 0) * a.K;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gi = bt * U * 64 + u * 64 + lane;
      const T* p = wr + (size_t)(gi < ngroups ? gi : ngroups - 1) * VEC;
      w[u][r] = ld16_stream(live ? p : (const T*)a.W);
    }
  }
}

template <int KW, int U_>
struct GemvShape {
  static constexpr int R = 16 / KW;  // rows per wave
  static constexpr int U = U_ > 0 ? U_ : ((R <= 2) ? 8 : 4);  // groups per lane and row per batch
};

// The row pairs a wave of workgroup wg (of nwg) takes in gemv_core: item j
// (j < n) is pair `we` of tile tile0 + j * step. By default the workgroup
// walks tiles wg, wg + nwg, ... and wave w takes pair w of each. A SwiGLU
// projection with two rows per wave spreads its units evenly instead
// (workgroup wg: units [wg P / nwg, (wg + 1) P / nwg), P = N; wave w every
// 8th of them from the w-th; unit u is pair u % 8 of tile u / 8), so no
// workgroup streams a whole tile more than another (the temporal gate/up's
// 1408 tiles on 256 workgroups left half of them a sixth tile). Every row is
// still summed by one wave in the same order, so the values do not depend
// on the mapping.
struct GemvItems {
  int tile0, we, step, n;
};
template <int EPI, int R>
__device__ __forceinline__ GemvItems gemv_items(const GemmArgs& a, int wg, int nwg, int wave) {
  GemvItems it;
  if constexpr (EPI == EPI_SWIGLU && R == 2) {
    const int lo = (int)((int64_t)wg * a.N / nwg), hi = (int)((int64_t)(wg + 1) * a.N / nwg);
    const int u0 = lo + wave;
    it.tile0 = u0 / 8;
    it.we = u0 % 8;
    it.step = 1;
    it.n = u0 < hi ? (hi - u0 + 7) / 8 : 0;
  } else {
    const int ntiles = n_tiles_of(EPI, a.N);
    it.tile0 = wg;
    it.we = wave;
    it.step = nwg;
    it.n = wg < ntiles ? (ntiles - wg + nwg - 1) / nwg : 0;
  }
  return it;
}

// The first weight batch of workgroup `wg` (of nwg) for the projection `a`,
// requested ahead of time (while the grid barrier that precedes it completes).
template <typename T, int KW, int EPI, int U_>
__device__ __forceinline__ void gemv_prefetch(const GemmArgs& a, int wg, int nwg,
                                              u32x4 (&w)[GemvShape<KW, U_>::U][GemvShape<KW, U_>::R]) {
  constexpr int R = GemvShape<KW, U_>::R, U = GemvShape<KW, U_>::U;
  const int t = tid();
  const GemvItems it = gemv_items<EPI, R>(a, wg, nwg, t >> 6);
  load_wbatch<T, EPI, U, R>(a, it.tile0, 0, t & 63, it.we, w, it.n > 0);
}

// EPI_RESID: the residual values of wave `wave`'s rows of tile `tile`
// (rows past the matrix, or a tile past the last, read row 0; every lane of
// the wave reads the same address).
template <int EPI, bool C, int R>
__device__ __forceinline__ void load_rpre(const GemmArgs& a, int tile, int wave, double (&rpre)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rpre[r] = 0.0;
    if constexpr (EPI == EPI_RESID) {
      const int row = tile * 16 + wave * R + r;
      rpre[r] = ld_f64<C>(a.resid + (row < a.N ? row : 0));
    }
  }
}

// A finished tile: each of the wave's R row sums is reduced over the 64
// lanes; the wave applies the epilogue to its own rows (argmax partials:
// wave 0 combines the tile's 16 rows through s_red, double-buffered by
// `parity`). rpre: residual values of the rows, valid if pre_ok.
template <typename T, int EPI, bool C, int R>
__device__ __forceinline__ void finish_tile(const GemmArgs& a, int tile, int wave, int lane,
                                            double (&acc)[R], const double (&rpre)[R], bool pre_ok,
                                            const QkvIn& qin, double (&s_red)[2][16], int& parity) {
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = group_reduce<64>(acc[r]);
  if constexpr (EPI == EPI_ARGMAX) {
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) s_red[parity][wave * R + r] = acc[r];
    }
    __syncthreads();
    if (wave == 0 && (lane & 15) == 0) {
      // g = lane / 16 holds rows 4g..4g+3 of column 0
      const int g = lane >> 4;
      const double v[4] = {s_red[parity][4 * g], s_red[parity][4 * g + 1], s_red[parity][4 * g + 2],
                           s_red[parity][4 * g + 3]};
      epilogue<T, EPI, C>(a, tile, g, 0, v);
    }
    parity ^= 1;
  } else {
    // every wave finishes its own rows: no workgroup barrier per tile
    if (lane == 0) wave_epilogue<T, EPI, C, R>(a, tile, wave, acc, rpre, pre_ok, qin);
  }
}

// Workgroup `wg` of `nwg` (KW waves) walks row tiles wg, wg+nwg, ... (16
// output rows each); wave w owns rows w*R .. w*R+R-1 (R = 16/KW) of a tile
// over the whole of K. The rounded input vector is built once per workgroup in
// LDS `xs` (model dtype, K elements). Lane l covers the 16-byte groups l,
// l+64, ... of a row, so a wave reads each row in contiguous 1 KB pieces.
// Weights stream in batches of U groups per lane and row, double-buffered: the
// next batch (possibly of the next tile) is requested before the current one
// is used. Each finished row is reduced over the 64 lanes; the wave that owns
// it applies the epilogue (argmax partials: wave 0, per tile). PRE: the first
// batch is already in `pre` (gemv_prefetch). The residual rows of the first
// tile (EPI_RESID) and the first XP input items of every thread (see
// build_input) are requested before the norm scale is computed. Every thread
// of the workgroup must call this (it synchronises the workgroup).
// IB (optional): ib(xs) builds the input vector in place of build_input
// (every thread calls it).
template <typename T, int KW, int PRO, int EPI, bool C, int U_, bool PRE, int XP = 4,
          typename IB = decltype(nullptr)>
__device__ __forceinline__ void gemv_core(
    const GemmArgs& a, int wg, int nwg, T* xs,
    const u32x4 (&pre)[GemvShape<KW, U_>::U][GemvShape<KW, U_>::R],
    const double (*rope)[2] = nullptr, IB ib = nullptr) {
  constexpr int VEC = VecOf<T>::N;
  constexpr int R = GemvShape<KW, U_>::R;
  constexpr int U = GemvShape<KW, U_>::U;
  constexpr int NTH = 64 * KW;
  const int t = tid();
  const int lane = t & 63;
  const int wave = t >> 6;
  __shared__ double s_red[2][16];
  __shared__ double s_tmp[KW];

  const int ngroups = a.K / VEC;  // K is a multiple of VEC
  const int nbatch = (ngroups + U * 64 - 1) / (U * 64);
  const GemvItems it = gemv_items<EPI, R>(a, wg, nwg, wave);

  int tile = it.tile0;
  u32x4 wa[U][R], wb[U][R];
  if (PRE) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) wa[u][r] = pre[u][r];
  } else {
    // in flight while the input is built
    load_wbatch<T, EPI, U, R>(a, tile, 0, lane, it.we, wa, it.n > 0);
  }
  // residual rows of the first item (one address per wave; clamped, so
  // every wave loads)
  double rpre[R];
  load_rpre<EPI, C, R>(a, tile, it.we, rpre);
  QkvIn qin{};
  if constexpr (EPI == EPI_QKV) {
    __shared__ double s_rope[64][2];
    if (a.inv_freq != nullptr && rope == nullptr) {
      rope_table(a, s_rope, NTH);  // read after the barrier below
      rope = s_rope;
    }
    qin = qkv_in(a, rope);
  }
  if constexpr (!__is_same(IB, decltype(nullptr)))
    ib(xs);
  else
    build_input<T, PRO, C, NTH, XP>(a, xs, s_tmp, wg == 0);
  __syncthreads();
  // every wave of the workgroup has the same number of items unless they
  // are SwiGLU units, whose epilogue needs no workgroup barrier
  if (it.n > 0) {
    double acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0;
    int bt = 0, parity = 0, j = 0;

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
        finish_tile<T, EPI, C, R>(a, tile, it.we, lane, acc, rpre, j == 0, qin, s_red, parity);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0;
      }
    };
    // the batch after (item jj, batch b)
    auto advance = [&](int& jj, int& b) {
      if (++b == nbatch) {
        b = 0;
        ++jj;
      }
    };

    // the next batch is always requested (a placeholder past the last one)
    for (;;) {
      int nj = j, nb = bt;
      advance(nj, nb);
      load_wbatch<T, EPI, U, R>(a, it.tile0 + nj * it.step, nb, lane, it.we, wb, nj < it.n);
      consume(wa);
      if (nj >= it.n) break;
      j = nj;
      bt = nb;
      tile = it.tile0 + j * it.step;
      advance(nj, nb);
      load_wbatch<T, EPI, U, R>(a, it.tile0 + nj * it.step, nb, lane, it.we, wa, nj < it.n);
      consume(wb);
      if (nj >= it.n) break;
      j = nj;
      bt = nb;
      tile = it.tile0 + j * it.step;
    }
  }
  __syncthreads();  // xs and s_red may be reused by the caller
}

// Without a prefetched first batch.
template <typename T, int KW, int PRO, int EPI, bool C, int U_ = 0>
__device__ __forceinline__ void gemv_body(const GemmArgs& a, int wg, int nwg, T* xs) {
  u32x4 none[GemvShape<KW, U_>::U][GemvShape<KW, U_>::R];
  gemv_core<T, KW, PRO, EPI, C, U_, false>(a, wg, nwg, xs, none);
}

// ---- one session, weight slice staged in LDS ------------------------------
//
// For short projections whose whole per-workgroup slice fits in LDS: every
// weight group of the workgroup's rows is requested at once with LDS-direct
// loads (global_load_lds_dwordx4) while the preceding grid barrier completes,
// then the projection runs from LDS.
//
// Work items: a wave always owns row pairs (the rows one sum-of-squares
// partial or one SwiGLU unit covers). q/k/v and argmax projections keep the
// 16-row tiles of gemv_core (tile i of the workgroup: wave w takes pair w),
// because attention tickets and argmax partials are per tile. The others
// spread pairs evenly: workgroup wg takes pairs [wg*P/nwg, (wg+1)*P/nwg) and
// wave w every KW-th of them from the w-th. Each row is still summed by one
// wave in gemv_core's order (lane l: groups l, l+64, ...; then the 64-lane
// reduction), so results are bit-identical to it whatever the mapping.
//
// Slot layout: lane l of wave w puts its 16-byte group of (the wave's item j,
// column pass c, row r of the pair) at byte ((((j * CPL + c) * 2 + r) * KW +
// w) * 64 + l) * 16, CPL = column passes per row (ceil(K / VEC / 64)); the
// same lane reads it back, so the only wait needed is the wave's own. The
// host sizes the buffer with staged_slice_bytes.

#define MOSHI_LDS __attribute__((address_space(3)))

template <typename T>
__device__ __forceinline__ int staged_cpl(int K) {
  return (K / VecOf<T>::N + 63) / 64;
}

template <int EPI>
constexpr bool staged_by_tile() {
  return EPI == EPI_QKV || EPI == EPI_ARGMAX;
}

// Item j of wave `wave` as (tile, pair in tile) of gemv_core's numbering;
// false past the wave's last item.
template <int EPI, int KW>
__device__ __forceinline__ bool staged_item(const GemmArgs& a, int wg, int nwg, int wave, int j,
                                            int& te, int& we) {
  if constexpr (staged_by_tile<EPI>()) {
    te = wg + j * nwg;
    we = wave;
    return te < n_tiles_of(EPI, a.N);
  } else {
    const int P = EPI == EPI_SWIGLU ? a.N : (a.N + 1) / 2;
    const int lo = wg * P / nwg, hi = (wg + 1) * P / nwg;  // nwg * P < 2^31
    const int p = lo + wave + j * KW;
    te = p / KW;
    we = p % KW;
    return p < hi;
  }
}

template <typename T, int KW, int EPI>
__device__ __forceinline__ void gemv_stage(const GemmArgs& a, int wg, int nwg, unsigned char* wbuf) {
  constexpr int VEC = VecOf<T>::N;
  constexpr int R = 16 / KW;
  static_assert(R == 2, "staged projections work on row pairs");
  const int t = tid();
  const int lane = t & 63, wave = t >> 6;
  const int ngroups = a.K / VEC;
  const int cpl = staged_cpl<T>(a.K);
  MOSHI_LDS unsigned char* base = (MOSHI_LDS unsigned char*)wbuf;
  int slot = 0, te, we;
  for (int j = 0; staged_item<EPI, KW>(a, wg, nwg, wave, j, te, we); ++j) {
    for (int c = 0; c < cpl; ++c) {
      const int gi = c * 64 + lane;
      const int gic = gi < ngroups ? gi : ngroups - 1;
#pragma unroll
      for (int r = 0; r < R; ++r, ++slot) {
        bool ok;
        const int rr = tile_row<EPI>(te, we * R + r, a.N, ok);
        const T* src = (const T*)a.W + (size_t)(ok ? rr : 0) * a.K + (size_t)gic * VEC;
        __builtin_amdgcn_global_load_lds((const MOSHI_GLB void*)src,
                                         (MOSHI_LDS void*)(base + (slot * KW + wave) * 1024), 16, 0,
                                         0);
      }
    }
  }
}

// The projection from a slice staged by gemv_stage (same arguments). Every
// thread of the workgroup must call this (it synchronises the workgroup).
// Entry of a depformer substep (one session): the substep's residual starts
// as y = pre + E_prev[tok], its own projection of the temporal hidden state
// plus its own embedding of the previous substep's greedy token (the text
// token first; mobius PR #368, "P2 - Moshi LM" and "P3 - ONNX Runtime example").
struct EntryIn {
  const ArgPart* apart;  // previous head's per-tile argmax partials
  int prev_rows;         // rows of the previous head
  const double* pre;     // [K] the substep's projection of the temporal hidden state
  const void* table;     // [prev_rows][K] model dtype: embedding of the previous token
  double* y;             // [K] residual, stored by the `first` workgroup
  int* tok_out;          // previous token, stored by the `first` workgroup
};

// Sum of squares of a pair, each product rounded on its own before the sum
// (the order of two lanes that hold one element each and add their squares).
__device__ __forceinline__ double sq_pair(double v0, double v1) {
#pragma clang fp contract(off)
  return v0 * v0 + v1 * v1;
}

// PRO_NORM input of the substep's first q/k/v projection built straight from
// the entry: every workgroup forms y for its element pairs, their
// sums of squares in the layout the residual epilogue writes (one per pair,
// a.n_ssq == a.K / 2), and the norm scale in build_input's order, so the
// rounded input is the one build_input makes from the stored y.
template <typename T, bool C, int NTH>
__device__ __forceinline__ void build_entry_input(const GemmArgs& a, const EntryIn& E, T* xs,
                                                  double* red, bool first) {
  const int t = tid();
  const int np = a.K / 2;
  const T* g = (const T*)a.gain;
  T* xn = first ? (T*)a.xn_out : nullptr;
  // the token does not decide these: request them first
  const int p0 = t < np ? t : np - 1;
  double pv[2], gv[2];
  ld_pair_f64<C>(E.pre, p0, pv[0], pv[1]);
  ld_pair_d(g, p0, gv[0], gv[1]);
  const int tok = reduce_token<NTH>(E.apart, (E.prev_rows + 15) / 16, E.prev_rows);
  if (first && t == 0) st_i32<C>(E.tok_out, tok);
  const T* row = (const T*)E.table + (size_t)tok * a.K;
  double ev[2];
  ld_pair_d(row, p0, ev[0], ev[1]);
  double y0 = pv[0] + ev[0], y1 = pv[1] + ev[1];
  double sum = 0.0;
  if (t < np) {
    if (first) {
      st_f64<C>(E.y + 2 * t, y0);
      st_f64<C>(E.y + 2 * t + 1, y1);
    }
    sum += sq_pair(y0, y1);
  }
  for (int p = t + NTH; p < np; p += NTH) {  // pairs past the first pass
    double q0, q1, e0, e1;
    ld_pair_f64<C>(E.pre, p, q0, q1);
    ld_pair_d(row, p, e0, e1);
    q0 += e0;
    q1 += e1;
    if (first) {
      st_f64<C>(E.y + 2 * p, q0);
      st_f64<C>(E.y + 2 * p + 1, q1);
    }
    sum += sq_pair(q0, q1);
  }
  const double rs = rms_finish(sum, a, red, NTH);
  if (t < np) put_pair<T, C>(xs, xn, t, y0 * rs * gv[0], y1 * rs * gv[1]);
  for (int p = t + NTH; p < np; p += NTH) {
    double q0, q1, e0, e1, g0, g1;
    ld_pair_f64<C>(E.pre, p, q0, q1);
    ld_pair_d(row, p, e0, e1);
    ld_pair_d(g, p, g0, g1);
    put_pair<T, C>(xs, xn, p, (q0 + e0) * rs * g0, (q1 + e1) * rs * g1);
  }
}

template <typename T, int KW, int PRO, int EPI, bool C, bool ENTRY = false>
__device__ __forceinline__ void gemv_staged(const GemmArgs& a, int wg, int nwg, T* xs,
                                            const unsigned char* wbuf,
                                            const double (*rope)[2] = nullptr,
                                            const EntryIn* ent = nullptr) {
  static_assert(!ENTRY || PRO == PRO_NORM, "the substep entry feeds a normed projection");
  constexpr int VEC = VecOf<T>::N;
  constexpr int R = 16 / KW;
  constexpr int NTH = 64 * KW;
  const int t = tid();
  const int lane = t & 63, wave = t >> 6;
  __shared__ double s_red[2][16];
  const int ngroups = a.K / VEC;
  const int cpl = staged_cpl<T>(a.K);
  int te, we;
  // residual rows of the wave's first item (row 0 if it has none)
  const bool any = staged_item<EPI, KW>(a, wg, nwg, wave, 0, te, we);
  double rpre[R];
  load_rpre<EPI, C, R>(a, any ? te : 0, any ? we : 0, rpre);
  QkvIn qin{};
  if constexpr (EPI == EPI_QKV) {
    __shared__ double s_rope[64][2];
    if (a.inv_freq != nullptr && rope == nullptr) {
      rope_table(a, s_rope, NTH);  // read after the barrier below
      rope = s_rope;
    }
    qin = qkv_in(a, rope);
  }
  __shared__ double s_tmp[KW];
  if constexpr (ENTRY)
    build_entry_input<T, C, NTH>(a, *ent, xs, s_tmp, wg == 0);
  else
    build_input<T, PRO, C, NTH, 1>(a, xs, s_tmp, wg == 0);
  __syncthreads();
  // this wave's LDS-direct loads have landed (they were issued before its
  // input loads, which it has already waited for; this makes it explicit)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const MOSHI_LDS unsigned char* base = (const MOSHI_LDS unsigned char*)wbuf;
  int parity = 0, slot = 0;
  for (int j = 0; staged_item<EPI, KW>(a, wg, nwg, wave, j, te, we); ++j) {
    double acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0;
#pragma unroll 2
    for (int c = 0; c < cpl; ++c, slot += R) {
      const int gi = c * 64 + lane;
      if (gi < ngroups) {
        double xv[VEC];
        widen<T>(*(const u32x4*)(xs + (size_t)gi * VEC), xv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          double wd[VEC];
          widen<T>(*(const MOSHI_LDS u32x4*)(base + (((slot + r) * KW + wave) * 64 + lane) * 16), wd);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[r] = fma(wd[e], xv[e], acc[r]);
        }
      }
    }
    finish_tile<T, EPI, C, R>(a, te, we, lane, acc, rpre, j == 0, qin, s_red, parity);
  }
  __syncthreads();  // xs, s_red and the slots may be reused by the caller
}

// ---------------------------------------------------------------------------
// Sliding-window decode attention over a ring of K/V
// ---------------------------------------------------------------------------

// Keys of slot b visible at its current position: ring slots [0, nvalid),
// minus `excl` (the oldest key, under the mask-oldest reading). Without
// positions (the depformer's entries): scalar_nvalid keys minus scalar_excl.
__device__ __forceinline__ void window_of(const AttnArgs& a, int b, int& nvalid, int& excl) {
  excl = -1;
  if (a.pos != nullptr) {
    const int64_t p = ldg(a.pos + b);
    nvalid = (int)(p + 1 < (int64_t)a.cap ? p + 1 : (int64_t)a.cap);
    if (a.mask_oldest && p >= (int64_t)a.cap - 1) excl = (int)((p + 1) % a.cap);
  } else {
    nvalid = a.scalar_nvalid;
    excl = a.scalar_excl;
  }
}

// One workgroup of NTH threads computes the attention of (slot b, head h)
// over the keys [k0, k1) of its window (a "span"); the span partials of a
// head are merged afterwards (combine_item / combine_staged), or, for a
// single span, the output is written directly.
//
// Each wave takes a contiguous run of the span's keys: wave w of NW gets
// [k0 + w*(k1-k0)/NW, k0 + (w+1)*(k1-k0)/NW). A wave holds TK = HD/VEC lanes
// per key (one 16-byte group each, dims kd*VEC ..) and KPW = 64/TK keys per
// pass; KB passes make a block of BK keys, and the wave streams its blocks
// double-buffered (the next block's K and V are requested before the
// current one is used). Per block, in fp64: scores s_j = (q.k_j) / sqrt(HD)
// (lane dot products, then a TK-lane reduction), the block maximum over the
// wave, and the online-softmax update with the running maximum m:
//   m' = max(m, block max);  c = e^{m - m'};  l <- l*c + sum_j e^{s_j - m'};
//   acc <- acc*c + sum_j e^{s_j - m'} v_j      (per lane: its key row, dims)
// Masked keys (past nvalid, past the run, or the excluded oldest key) have
// s = -inf and p = 0. Then the workgroup merges its waves in a fixed order
// (threads t < HD, dim t):
//   M = max_w m_w;  e_w = e^{m_w - M};  L = sum_w sum_r e_w l_{w,r};
//   O = sum_w sum_r e_w acc_{w,r}   (r: the KPW key rows of wave w)
// giving the span partial (M, L, O), or O / L for a single span.
template <typename T, int HD>
struct SpanShape {
  static constexpr int VEC = VecOf<T>::N;
  static constexpr int TK = HD / VEC;   // lanes per key
  static constexpr int KPW = 64 / TK;   // keys per wave pass
  static constexpr int KB = KPW < 16 ? 16 / KPW : 1;  // passes per block
  static constexpr int BK = KB * KPW;                 // keys per block (16)
  static_assert(TK <= 64 && 64 % TK == 0, "head dim");
};
// LDS doubles attn_span needs (per-wave accumulators, sums and maxima).
template <typename T, int HD, int NTH>
constexpr int span_lds_doubles() {
  return (NTH / 64) * SpanShape<T, HD>::KPW * (HD + 1) + NTH / 64;
}

template <typename T, int HD>
struct KvBlock {
  u32x4 k[SpanShape<T, HD>::KB], v[SpanShape<T, HD>::KB];
};

// Requests block keys j0 + ps*KPW + kk (ps < KB) of this lane. Keys at or
// past nvalid read key 0 (always written; masked by the caller). COH: the
// ring was written during the running kernel (its newest row), so every
// load is coherent (sc1).
template <typename T, int HD, bool COH>
__device__ __forceinline__ void load_kv_block(const T* kbase, const T* vbase, int j0, int kk,
                                              int kd, int nvalid, KvBlock<T, HD>& kv) {
  using S = SpanShape<T, HD>;
#pragma unroll
  for (int ps = 0; ps < S::KB; ++ps) {
    const int j = j0 + ps * S::KPW + kk;
    const uint32_t off = (uint32_t)(((size_t)(j < nvalid ? j : 0) * HD + kd * S::VEC) * sizeof(T));
    if constexpr (COH) {
      kv.k[ps] = ld16_coh(kbase, off);
      kv.v[ps] = ld16_coh(vbase, off);
    } else {
      kv.k[ps] = ld16_stream((const char*)kbase + off);
      kv.v[ps] = ld16_stream((const char*)vbase + off);
    }
  }
}

// direct: write O / L to a.o_out (the only span); else the partial goes to
// part (HD + 2 doubles: M, L, O). s_w: LDS, span_lds_doubles() doubles.
// Every thread of the workgroup calls it.
// PUT (optional): put(t, M, L, O, direct) takes each thread t < HD's results
// instead of the stores to part / a.o_out.
template <typename T, int HD, int NTH, bool C, typename PUT = decltype(nullptr)>
__device__ __forceinline__ void attn_span(const AttnArgs& a, int h, int b, int k0, int k1,
                                          int nvalid, int excl, double* s_w, double* part,
                                          bool direct, PUT put = nullptr) {
  using S = SpanShape<T, HD>;
  constexpr int VEC = S::VEC, TK = S::TK, KPW = S::KPW, KB = S::KB, BK = S::BK;
  constexpr int NW = NTH / 64;
  const int t = tid();
  const int lane = t & 63, w = t >> 6;
  const int kd = lane % TK, kk = lane / TK;
  const int ws = k0 + w * (k1 - k0) / NW, we = k0 + (w + 1) * (k1 - k0) / NW;
  const int nb = (we - ws + BK - 1) / BK;
  const size_t base = (size_t)b * a.slot_stride + a.layer_off + (size_t)h * a.head_stride;
  const T* kbase = (const T*)a.ring_k + base;
  const T* vbase = (const T*)a.ring_v + base;
  const double scale = 1.0 / sqrt((double)HD);

  KvBlock<T, HD> ka, kb;
  load_kv_block<T, HD, C>(kbase, vbase, ws, kk, kd, nvalid, ka);
  double qv[VEC];
  {
    const double* qp = a.q + (size_t)b * a.ldq + h * HD + kd * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[e] = ld_f64<C>(qp + e);
  }
  double m = -INFINITY, l = 0.0, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;

  auto block = [&](const KvBlock<T, HD>& kv, int j0) {
    double sc[KB];
    double mloc = -INFINITY;
#pragma unroll
    for (int ps = 0; ps < KB; ++ps) {
      const int j = j0 + ps * KPW + kk;
      double kx[VEC];
      widen<T>(kv.k[ps], kx);
      double d = 0.0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) d = fma(qv[e], kx[e], d);
      d = group_reduce<TK>(d);
      sc[ps] = (j < we && j < nvalid && j != excl) ? d * scale : -INFINITY;
      mloc = fmax(mloc, sc[ps]);
    }
    const double mn = fmax(m, group_reduce<64, true>(mloc));
    if (mn != m) {  // wave-uniform; with m = mn the rescale is by e^0 = 1
      const double c = m == -INFINITY ? 0.0 : exp(m - mn);
      l *= c;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] *= c;
    }
    // softmax weights: with 16 lanes per key, lane ps of each 16-lane row
    // computes the weight of pass ps and the row shares it (one exp per lane)
    double pw[KB];
    if constexpr (TK == 16 && KB == 4) {
      const int mine = kd & 3;
      const double sm = mine == 0 ? sc[0] : mine == 1 ? sc[1] : mine == 2 ? sc[2] : sc[3];
      const double pm = sm == -INFINITY ? 0.0 : exp(sm - mn);
      pw[0] = dpp_d<0x150>(pm);  // row_newbcast: lane n of each row to the row
      pw[1] = dpp_d<0x151>(pm);
      pw[2] = dpp_d<0x152>(pm);
      pw[3] = dpp_d<0x153>(pm);
    } else {
#pragma unroll
      for (int ps = 0; ps < KB; ++ps) pw[ps] = sc[ps] == -INFINITY ? 0.0 : exp(sc[ps] - mn);
    }
#pragma unroll
    for (int ps = 0; ps < KB; ++ps) {
      const double p = pw[ps];
      l += p;
      double vx[VEC];
      widen<T>(kv.v[ps], vx);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fma(p, vx[e], acc[e]);
    }
    m = mn;
  };
  // the next block is always requested (past the run it re-reads key 0)
  for (int i = 0; i < nb; i += 2) {
    load_kv_block<T, HD, C>(kbase, vbase, ws + (i + 1) * BK, kk, kd, i + 1 < nb ? nvalid : 0, kb);
    block(ka, ws + i * BK);
    if (i + 1 >= nb) break;
    load_kv_block<T, HD, C>(kbase, vbase, ws + (i + 2) * BK, kk, kd, i + 2 < nb ? nvalid : 0, ka);
    block(kb, ws + (i + 1) * BK);
  }

  // workgroup merge of the waves (fixed order); lane v of each merging wave
  // forms the weight of wave v, read by the others with readlane
  static_assert(NW <= 64, "waves per workgroup");
  double* s_acc = s_w;                       // [NW][KPW][HD + 1]
  double* s_m = s_w + NW * KPW * (HD + 1);   // [NW]
  double* row = s_acc + (size_t)(w * KPW + kk) * (HD + 1);
#pragma unroll
  for (int e = 0; e < VEC; ++e) row[kd * VEC + e] = acc[e];
  if (kd == 0) row[HD] = l;
  if (lane == 0) s_m[w] = m;
  __syncthreads();
  if (t < HD) {
    double M = s_m[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) M = fmax(M, s_m[v]);
    const double mine = s_m[lane % NW];
    const double emine = mine == -INFINITY ? 0.0 : exp(mine - M);
    double L = 0.0, O = 0.0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const double ev = readlane_d(emine, v);
#pragma unroll
      for (int r = 0; r < KPW; ++r) {
        const double* rr = s_acc + (size_t)(v * KPW + r) * (HD + 1);
        L = fma(ev, rr[HD], L);
        O = fma(ev, rr[t], O);
      }
    }
    if constexpr (!__is_same(PUT, decltype(nullptr))) {
      put(t, M, L, O, direct);
    } else if (direct) {
      const double ov = L > 0.0 ? O / L : 0.0;
      store_rounded<T, C>((T*)a.o_out + (size_t)b * a.ldo + h * HD + t, &ov, 1);
    } else {
      st_f64<C>(part + 2 + t, O);
      if (t == 0) {
        st_f64<C>(part, M);
        st_f64<C>(part + 1, L);
      }
    }
  }
  __syncthreads();  // s_w is reused by the caller
}

// Spans of a slot's window: at most a.max_spans (the spans per head the
// grid provides), and about ATTN_CHUNK keys or more each. Span j covers keys
// [j*nvalid/n, (j+1)*nvalid/n).
__device__ __forceinline__ int n_spans(const AttnArgs& a, int nvalid) {
  const int by_len = (nvalid + ATTN_CHUNK - 1) / ATTN_CHUNK;
  const int n = a.max_spans < by_len ? a.max_spans : by_len;
  return n < 1 ? 1 : n;
}

// Merge the span partials of (slot b, head h) in span order:
// o = sum_c e^{m_c - M} O_c / sum_c e^{m_c - M} L_c. Threads [0, HD) work;
// every thread of the workgroup must call this.
template <typename T, int HD, bool C>
__device__ __forceinline__ void combine_item(const AttnArgs& a, int h, int b, int nchunks) {
  const int t = tid();
  const double* parts = a.part + ((size_t)b * a.n_heads + h) * a.max_spans * (HD + 2);
  constexpr int NW = HD / 64 > 0 ? HD / 64 : 1;
  __shared__ double s_m[NW];
  __shared__ double s_w[ATTN_MAX_CHUNKS];
  // M = max over the chunk maxima (exact, so any reduction order gives the same M)
  double mloc = -INFINITY;
  if (t < HD)
    for (int c = t; c < nchunks; c += HD) mloc = fmax(mloc, ld_f64<C>(parts + (size_t)c * (HD + 2)));
  mloc = group_reduce<(HD < 64 ? HD : 64), true>(mloc);
  if (t < HD && (t & 63) == 0) s_m[t >> 6] = mloc;
  __syncthreads();
  double M = s_m[0];
  for (int w = 1; w < NW; ++w) M = fmax(M, s_m[w]);
  // chunk weights e^{m_c - M}, one exp per chunk
  if (t < HD)
    for (int c = t; c < nchunks; c += HD) {
      const double mc = ld_f64<C>(parts + (size_t)c * (HD + 2));
      s_w[c] = (mc == -INFINITY) ? 0.0 : exp(mc - M);
    }
  __syncthreads();
  if (t < HD) {
    double L = 0.0, O = 0.0;
#pragma unroll 8
    for (int c = 0; c < nchunks; ++c) {
      const double* pc = parts + (size_t)c * (HD + 2);
      const double w = s_w[c];
      L = fma(ld_f64<C>(pc + 1), w, L);
      O = fma(ld_f64<C>(pc + 2 + t), w, O);
    }
    const double ov = L > 0.0 ? O / L : 0.0;
    store_rounded<T, C>((T*)a.o_out + (size_t)b * a.ldo + h * HD + t, &ov, 1);
  }
  __syncthreads();
}

// The same merge as combine_item (identical arithmetic and order) without
// LDS or workgroup barriers: threads [0, HD) request every partial they need
// at once and each forms the span weights itself. Every thread of the
// workgroup calls it.
template <typename T, int HD, bool C>
__device__ __forceinline__ void combine_direct(const AttnArgs& a, int h, int b, int nspans) {
  constexpr int NS = 8;  // spans whose partials are requested up front
  const int t = tid();
  if (t < HD) {
    const double* parts = a.part + ((size_t)b * a.n_heads + h) * a.max_spans * (HD + 2);
    double mv[NS], lv[NS], ov[NS];
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      const double* pc = parts + (size_t)(c < nspans ? c : 0) * (HD + 2);
      mv[c] = ld_f64<C>(pc);
      lv[c] = ld_f64<C>(pc + 1);
      ov[c] = ld_f64<C>(pc + 2 + t);
    }
    double M = -INFINITY;
#pragma unroll
    for (int c = 0; c < NS; ++c)
      if (c < nspans) M = fmax(M, mv[c]);
    for (int c = NS; c < nspans; ++c) M = fmax(M, ld_f64<C>(parts + (size_t)c * (HD + 2)));
    // lane c forms the weight of span c; the others read it with readlane
    const int lc = tid() & (NS - 1);
    double mine = mv[0];
#pragma unroll
    for (int c = 1; c < NS; ++c) mine = lc == c ? mv[c] : mine;
    const double emine = (mine == -INFINITY) ? 0.0 : exp(mine - M);
    double L = 0.0, O = 0.0;
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      if (c < nspans) {
        const double w = readlane_d(emine, c);
        L = fma(lv[c], w, L);
        O = fma(ov[c], w, O);
      }
    }
    for (int c = NS; c < nspans; ++c) {
      const double* pc = parts + (size_t)c * (HD + 2);
      const double mc = ld_f64<C>(pc);
      const double w = (mc == -INFINITY) ? 0.0 : exp(mc - M);
      L = fma(ld_f64<C>(pc + 1), w, L);
      O = fma(ld_f64<C>(pc + 2 + t), w, O);
    }
    const double ov_ = L > 0.0 ? O / L : 0.0;
    store_rounded<T, C>((T*)a.o_out + (size_t)b * a.ldo + h * HD + t, &ov_, 1);
  }
}

// Depformer attention of slot b, heads head0 .. head0+n_heads-1, keys 0 ..
// nvalid-1 except key `excl` (-1: none; nvalid <= DEP_MAX_KEYS), by one
// workgroup of NTH threads: wave w
// takes heads w, w + NW, ..., NH at a time (every load of those heads is
// requested before any is used). Scores: TK lanes per key, fp64 dot products
// reduced in the lanes; softmax over the keys in fp64; p.V: one lane per
// output dim, an fp64 fma chain over the keys in order. The rounded outputs
// go to a.o_out. The arithmetic of a head does not depend on NH or on which
// wave takes it. C: q/K/V were written during the running kernel (coherent
// loads). Every thread of the workgroup calls it.
constexpr int DEP_MAX_KEYS = DEP_MAX_KEYS_HOST;
template <typename T, int HD, int NTH, bool C, int NH>
__device__ __forceinline__ void dep_attention(const AttnArgs& a, int b, int head0, int n_heads,
                                              int nvalid, int excl) {
  constexpr int VEC = VecOf<T>::N;
  constexpr int TK = HD / VEC;        // lanes per key for the scores
  constexpr int KPW = 64 / TK;        // keys per wave pass
  constexpr int NP = (DEP_MAX_KEYS + KPW - 1) / KPW;
  constexpr int NW = NTH / 64;
  constexpr int DPL = HD > 64 ? HD / 64 : 1;  // output dims per lane
  static_assert(TK <= 64 && 64 % TK == 0, "head dim");
  __shared__ double s_sc[NW][NH][64];
  const int t = tid();
  const int lane = t & 63, w = t >> 6;
  const int kd = lane % TK, kq = lane / TK;
  const double scale = 1.0 / sqrt((double)HD);
  for (int h0 = w; h0 < n_heads; h0 += NH * NW) {
    u32x4 kw[NH][NP];
    uint32_t vr[NH][DEP_MAX_KEYS][DPL];
    double qv[NH][VEC];
    // every load of the NH heads first (heads past n_heads read head 0)
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      const int h = head0 + (h0 + k * NW < n_heads ? h0 + k * NW : 0);
      // the slot's layer (workgroup-uniform: the base of a coherent buffer
      // load) and the head within it
      const T* lbase = (const T*)a.ring_k + (size_t)b * a.slot_stride + a.layer_off;
      const size_t base = (size_t)b * a.slot_stride + a.layer_off + (size_t)h * a.head_stride;
      const T* kbase = (const T*)a.ring_k + base;
      const T* vbase = (const T*)a.ring_v + base;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int j = p * KPW + kq;
        const int jc = j < nvalid ? j : 0;
        const uint32_t off = (uint32_t)(((size_t)jc * HD + kd * VEC) * sizeof(T));
        if constexpr (C)
          kw[k][p] = ld16_coh(lbase, off + (uint32_t)((size_t)h * a.head_stride * sizeof(T)));
        else
          kw[k][p] = ld16((const char*)kbase + off);
      }
#pragma unroll
      for (int j = 0; j < DEP_MAX_KEYS; ++j) {
        const int jc = j < nvalid ? j : 0;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          const int dd = (lane + 64 * i) < HD ? lane + 64 * i : 0;
          const T* vp = vbase + (size_t)jc * HD + dd;
          if constexpr (sizeof(T) == 2) {
            vr[k][j][i] = C ? (uint32_t)__hip_atomic_load((MOSHI_GLB uint16_t*)vp, MOSHI_RLX, MOSHI_AGT)
                            : (uint32_t)ldg((const uint16_t*)vp);
          } else {
            vr[k][j][i] = C ? __hip_atomic_load((MOSHI_GLB uint32_t*)vp, MOSHI_RLX, MOSHI_AGT)
                            : ldg((const uint32_t*)vp);
          }
        }
      }
      const double* qp = a.q + (size_t)b * a.ldq + h * HD + kd * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) qv[k][e] = ld_f64<C>(qp + e);
    }
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      const int h = h0 + k * NW;
      double* sp = s_sc[w][k];
      // scores
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        double kv_[VEC];
        widen<T>(kw[k][p], kv_);
        double d = 0.0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = fma(qv[k][e], kv_[e], d);
        d = group_reduce<TK>(d);
        const int j = p * KPW + kq;
        if (kd == 0 && j < DEP_MAX_KEYS) sp[j] = d * scale;
      }
      // softmax over the valid keys (entry `excl` masked)
      const double sv = (lane < nvalid && lane != excl) ? sp[lane] : -INFINITY;
      const double m = group_reduce<64, true>(sv);
      const double pj = (sv == -INFINITY) ? 0.0 : exp(sv - m);
      const double l = group_reduce<64>(pj);
      sp[lane] = pj;
      // p.V
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        double od = 0.0;
#pragma unroll
        for (int j = 0; j < DEP_MAX_KEYS; ++j) {
          if (j < nvalid) {
            const double vv = sizeof(T) == 2 ? (double)__uint_as_float(vr[k][j][i] << 16)
                                             : (double)__uint_as_float(vr[k][j][i]);
            od = fma(sp[j], vv, od);
          }
        }
        const int dd = lane + 64 * i;
        if (h < n_heads && dd < HD) {
          const double ov = l > 0.0 ? od / l : 0.0;
          store_rounded<T, C>((T*)a.o_out + (size_t)b * a.ldo + (head0 + h) * HD + dd, &ov, 1);
        }
      }
    }
  }
  __syncthreads();
}

// EPI_RESID with the residual rows already loaded (r): the same arithmetic as
// epilogue<.., EPI_RESID, ..>.
template <bool C>
__device__ __forceinline__ void epilogue_resid(const GemmArgs& a, int tile, int g, int col,
                                               const double* v, const double* r) {
  const bool cok = col < a.B;
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tile * 16 + 4 * g + i;
    if (cok && row < a.N) {
      const double xn = r[i] + v[i];
      st_f64<C>(a.resid + (size_t)col * a.ldr + row, xn);
      ss += xn * xn;
    }
  }
  ss += shfl_xor_d(ss, 16);
  ss += shfl_xor_d(ss, 32);
  if (g == 0 && cok) st_f64<C>(a.ssq_out + (size_t)tile * a.B + col, ss);
}

// ---- operations of two or more sessions (per-operation kernels in
// kernels.hip, and the multi-session depformer kernel in step.hip) ----------

// One 16-row tile x NB 16-column blocks (columns col0 .. col0 + 16 NB - 1) of a
// projection as fp64 MFMA 16x16x4 products.
// A = 16 weight rows x 4 k (lane: row lane%16, k-slot lane/16), B = 4 k x 16
// session columns (lane: column lane%16, same k-slot). A lane loads 16 bytes of
// its row (VEC consecutive k) and of its column's input; element e of every
// lane feeds MFMA e, so both operands map k-slot g to k0 + VEC*g + e.
// The fp64 16x16 result puts row (lane/16) + 4i in element i of a lane, so A
// row m carries tile row 4*(m%4) + m/4: element i of lane group g is then tile
// row 4g + i, the layout the epilogues use.
// Wave w of KW sums k-steps [w n / KW, (w+1) n / KW) in order; the waves'
// sums are added in wave order by wave 0, which runs the epilogue. (Two
// accumulator chains per wave were measured slower.) A column's
// value therefore depends on KW and K only (not on NB, col0 or DB). DB:
// double-buffered batches. C: X was written during the running kernel
// (coherent loads). wpre (DB only; null = none): the wave's first batch of
// weights, already loaded by gemm_tile_weights for this tile. The residual
// epilogue's inputs are requested before the products (by wave 0, which runs
// it). s_acc: KW * NB * 64 f64x4 of LDS. Every thread of the 64 KW calls it;
// the caller synchronises before reusing s_acc.
constexpr int GEMM_U = 4;  // k-steps per batch

// A lane's weight groups of the U k-steps from st of tile `tile` (zero past
// its wave's k-range or the matrix; rows past N may read anything).
// The k-steps [first, first + count) of K segment kseg of a projection
// (all of them when it is not split).
__device__ __forceinline__ void gemm_segment(const GemmArgs& a, int nsteps, int kseg, int& first,
                                             int& count) {
  const int ks = a.ksplit > 1 ? a.ksplit : 1;
  first = (kseg * nsteps) / ks;
  count = ((kseg + 1) * nsteps) / ks - first;
}

// Item `item` of a projection's MFMA work: (row tile, first column, K
// segment); the 16-column blocks of a tile are nt items apart and its K
// segments nt * (column blocks) apart. Items: nt * ncb * ksplit.
__device__ __forceinline__ int gemm_items(const GemmArgs& a, int epi) {
  return n_tiles_of(epi, a.N) * ((a.B + 15) / 16) * (a.ksplit > 1 ? a.ksplit : 1);
}
__device__ __forceinline__ void gemm_item(const GemmArgs& a, int epi, int item, int& tile,
                                          int& col0, int& kseg) {
  const int nt = n_tiles_of(epi, a.N), ncb = (a.B + 15) / 16;
  tile = item % nt;
  col0 = ((item / nt) % ncb) * 16;
  kseg = item / (nt * ncb);
}

template <typename T, int KW, int EPI>
__device__ __forceinline__ void gemm_tile_weights(const GemmArgs& a, int tile, int st_off,
                                                  u32x4 (&wv)[GEMM_U], int kseg = 0) {
  constexpr int VEC = VecOf<T>::N;
  constexpr int KSTEP = 4 * VEC;
  const int lane = tid() & 63, wave = tid() >> 6, r16 = lane & 15, g = lane >> 4;
  bool rok;
  const int wrow = tile_row<EPI>(tile, 4 * (r16 & 3) + (r16 >> 2), a.N, rok);
  const T* wbase = (const T*)a.W + (size_t)(rok ? wrow : 0) * a.K + g * VEC;
  const int nsteps = (a.K + KSTEP - 1) / KSTEP;
  int g0, gn;
  gemm_segment(a, nsteps, kseg, g0, gn);
  const int s1 = g0 + ((wave + 1) * gn) / KW;
  const int st = g0 + (wave * gn) / KW + st_off;
#pragma unroll
  for (int u = 0; u < GEMM_U; ++u) {
    const int k0 = (st + u) * KSTEP + g * VEC;
    const bool kok = (st + u < s1) && (k0 < a.K);
    wv[u] = (kok && rok) ? ld16_stream(wbase + (size_t)(st + u) * KSTEP) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <typename T, int NB, int KW, int EPI, bool DB, bool C, int RT = 1, int U = GEMM_U>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int tile, int col0, f64x4* s_acc,
                                          const u32x4* wpre = nullptr, int kseg = 0) {
  // RT row tiles (tile .. tile + RT - 1) share each input group's conversion;
  // each tile's sums are those of RT = 1 (same order), so RT changes no value;
  // neither does U (k-steps per batch: a wave sums its k-steps in order)
  constexpr int VEC = VecOf<T>::N;
  constexpr int KSTEP = 4 * VEC;
  static_assert(RT == 1 || !DB, "several row tiles: single batches");
  static_assert(!DB || U == GEMM_U, "double-buffered batches take gemm_tile_weights' first batch");
  static_assert(RT <= KW, "one epilogue wave per row tile");
  const int lane = tid() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid() >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int ntiles = n_tiles_of(EPI, a.N);

  // Rows past N read row 0 and columns past B read column B - 1 (their sums
  // are never stored), so loads need no mask: a batch's loads are issued
  // together. k-steps past the wave's range re-read its last step and skip
  // their products (a wave-uniform branch); only when K is not a multiple of
  // KSTEP are the groups past K zeroed per lane.
  int wrow[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    bool rok;
    wrow[r] = tile_row<EPI>(tile + r, 4 * (r16 & 3) + (r16 >> 2), a.N, rok);
    wrow[r] = rok ? wrow[r] : 0;
  }
  const int nsteps = (a.K + KSTEP - 1) / KSTEP;
  int g0, gn;
  gemm_segment(a, nsteps, kseg, g0, gn);
  const int s0 = g0 + (wave * gn) / KW;
  const int s1 = g0 + ((wave + 1) * gn) / KW;
  const bool ktail = (a.K % KSTEP) != 0;

  f64x4 acc[RT][NB];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[r][nb] = f64x4{0.0, 0.0, 0.0, 0.0};
  // the residual rows this lane's epilogue adds to (written before this
  // operation): wave r runs tile r's epilogue
  double rpre[NB][4];
  if constexpr (EPI == EPI_RESID) {
    if (wave < RT)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = col0 + nb * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = (tile + wave) * 16 + 4 * g + i;
          rpre[nb][i] = (col < a.B && row < a.N) ? ld_f64<C>(a.resid + (size_t)col * a.ldr + row) : 0.0;
        }
      }
  }
  // batch of U k-steps starting at st: weights and input groups (the
  // weights only where `w`)
  auto load = [&](int st, u32x4 (&wv)[U][RT], u32x4 (&xw)[U][NB], bool w = true) {
    int k0[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = st + u < s1 ? st + u : s1 - 1;
      k0[u] = su * KSTEP + g * VEC;
      if (ktail) k0[u] = k0[u] < a.K ? k0[u] : 0;
      if (w)
#pragma unroll
        for (int r = 0; r < RT; ++r)
          wv[u][r] = ld16_stream((const T*)a.W + (size_t)wrow[r] * a.K + k0[u]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        int col = col0 + nb * 16 + r16;
        col = col < a.B ? col : a.B - 1;
        if constexpr (C)
          xw[u][nb] = ld16_coh(a.X, (uint32_t)(((size_t)col * a.ldx + k0[u]) * sizeof(T)));
        else
          xw[u][nb] = ld16((const T*)a.X + (size_t)col * a.ldx + k0[u]);
      }
    }
    if (ktail) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if ((st + u) * KSTEP + g * VEC >= a.K) {
          if (w)
#pragma unroll
            for (int r = 0; r < RT; ++r) wv[u][r] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) xw[u][nb] = u32x4{0u, 0u, 0u, 0u};
        }
    }
  };
  auto compute = [&](int st, const u32x4 (&wv)[U][RT], const u32x4 (&xw)[U][NB]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (st + u >= s1) break;  // wave-uniform: past the wave's k-range
      if constexpr (RT == 1) {
        double wd[VEC];
        widen<T>(wv[u][0], wd);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          double xd[VEC];
          widen<T>(xw[u][nb], xd);
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            acc[0][nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(wd[e], xd[e], acc[0][nb], 0, 0, 0);
        }
      } else {
        double wd[RT][VEC];
#pragma unroll
        for (int r = 0; r < RT; ++r) widen<T>(wv[u][r], wd[r]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          double xd[VEC];
          widen<T>(xw[u][nb], xd);
#pragma unroll
          for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int e = 0; e < VEC; ++e)
              acc[r][nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(wd[r][e], xd[e], acc[r][nb], 0, 0, 0);
        }
      }
    }
  };
  if constexpr (DB) {
    // the next batch is requested before this one is used
    u32x4 wa[U][1], xa[U][NB], wb[U][1], xb[U][NB];
    if (wpre != nullptr) {
#pragma unroll
      for (int u = 0; u < U; ++u) wa[u][0] = wpre[u];
    }
    if (s0 < s1) load(s0, wa, xa, wpre == nullptr);
    for (int st = s0; st < s1; st += 2 * U) {
      if (st + U < s1) load(st + U, wb, xb);
      compute(st, wa, xa);
      if (st + U >= s1) break;
      if (st + 2 * U < s1) load(st + 2 * U, wa, xa);
      compute(st + U, wb, xb);
    }
  } else {
    for (int st = s0; st < s1; st += U) {
      u32x4 wv[U][RT];
      u32x4 xw[U][NB];
      load(st, wv, xw);
      compute(st, wv, xw);
    }
  }
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s_acc[((wave * RT + r) * NB + nb) * 64 + lane] = acc[r][nb];
  __syncthreads();
  if (wave >= RT || tile + wave >= ntiles) return;
  f64x4 sms[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f64x4 sm = s_acc[(wave * NB + nb) * 64 + lane];
    for (int w = 1; w < KW; ++w) sm += s_acc[((w * RT + wave) * NB + nb) * 64 + lane];
    sms[nb] = sm;
  }
  if (a.ksplit > 1) {
    // K segments (RT == 1, wave 0): this segment's sums go out coherently;
    // once they have landed, the segment counts itself in; the last one
    // adds every segment's sums in segment order (its own from registers,
    // the same values it stored) and runs the epilogue
    const int ks = a.ksplit;
    const int pc = tile * 4 + col0 / 16;  // (tile, first column block)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      double* p = a.kpart + ((((size_t)tile * 4 + col0 / 16 + nb) * ks + kseg) * 64 + lane) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) st_f64<true>(p + i, sms[nb][i]);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add((MOSHI_GLB int*)(a.kcnt + pc), 1, MOSHI_RLX, MOSHI_AGT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != ks - 1) return;
    if (lane == 0) __hip_atomic_store((MOSHI_GLB int*)(a.kcnt + pc), 0, MOSHI_RLX, MOSHI_AGT);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const double* p = a.kpart + (((size_t)tile * 4 + col0 / 16 + nb) * ks * 64 + lane) * 4;
      f64x4 tot = {0.0, 0.0, 0.0, 0.0};
      for (int s = 0; s < ks; ++s) {
        f64x4 ps = sms[nb];
        if (s != kseg)
#pragma unroll
          for (int i = 0; i < 4; ++i) ps[i] = ld_f64<true>(p + (size_t)s * 256 + i);
        tot = s == 0 ? ps : tot + ps;
      }
      sms[nb] = tot;
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const double v[4] = {sms[nb][0], sms[nb][1], sms[nb][2], sms[nb][3]};
    if constexpr (EPI == EPI_RESID)
      epilogue_resid<C>(a, tile + wave, g, col0 + nb * 16 + r16, v, rpre[nb]);
    else
      epilogue<T, EPI, C>(a, tile + wave, g, col0 + nb * 16 + r16, v);
  }
}

// The MFMA path's input vector of column b, elements [k0, k1):
// xn[b][k] = round(x[b][k] * scale_b * g[k]) (PRO_NORM) or round(x[b][k])
// (PRO_CAST). The scale comes from threads [0, 256) exactly as rms_scale with
// 256 threads (the others add nothing), so any workgroup of 256 or more
// threads, for any range, gives the same bits. `red` holds NTH / 64 doubles.
// Every thread of the workgroup calls it.
template <typename T, int PRO, bool C, int NTH>
__device__ __forceinline__ void norm_column(const GemmArgs& a, int b, double* red, int k0 = 0,
                                            int k1 = 0x7fffffff) {
  static_assert(NTH >= 256, "the scale uses 256 threads");
  constexpr int PF = 4;  // elements per thread requested before the scale is formed
  const double* x = (const double*)a.X + (size_t)b * a.ldx;
  T* out = (T*)a.xn_out + (size_t)b * a.K;
  k1 = k1 < a.K ? k1 : a.K;
  double xp[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int k = k0 + tid() + j * NTH;
    xp[j] = k < k1 ? ld_f64<C>(x + k) : 0.0;
  }
  double rs = 1.0;
  if constexpr (PRO == PRO_NORM) {
    double s = 0.0;
    if (tid() < 256)
      for (int i = tid(); i < a.n_ssq; i += 256) s += ld_f64<C>(a.ssq + (size_t)i * a.B + b);
    rs = rms_finish(s, a, red, 256);
  }
  auto put = [&](int k, double xv) {
    const double v = (PRO == PRO_NORM) ? xv * rs * to_d(((const T*)a.gain)[k]) : xv;
    store_rounded<T, C>(out + k, &v, 1);
  };
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int k = k0 + tid() + j * NTH;
    if (k < k1) put(k, xp[j]);
  }
  for (int k = k0 + tid() + PF * NTH; k < k1; k += NTH) put(k, ld_f64<C>(x + k));
}

// Depformer substep entry of rows bx*16 .. bx*16+15 and columns by*4 ..
// by*4+3 by one wave (lane: row lane%16, column by*4 + lane/16):
// y = (W_in[s] hidden) + E_s[previous token]. With prev_part the previous
// head's per-tile argmax partials of the column are reduced over its 16 lanes
// (or the forced token taken) and stored to prev by the items of row tile 0.
// Sums of squares per ssq_rows rows, combined across lanes in a fixed order.
template <typename T, bool C>
__device__ __forceinline__ void entry_item(const EntryArgs& a, int bx, int by, int lane) {
  const int r = lane & 15;
  const int b = by * 4 + (lane >> 4);
  const int row = bx * 16 + r;
  int tok = 0;
  if (a.prev_part != nullptr) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
    if (b < a.B)
      for (int i = r; i < a.prev_tiles; i += 16) {
        const ArgPart p = unpack_part(ld_grp<C>(a.prev_part + (size_t)i * a.B + b));
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
    if (a.forced != nullptr && b < a.B) {
      const int f = a.forced[(size_t)b * a.forced_stride + a.forced_col];
      if (f >= 0) tok = f;
    }
    if (bx == 0 && r == 0 && b < a.B) st_i32<C>(a.prev + (size_t)b * a.prev_stride, tok);
  } else if (b < a.B) {
    tok = ld_i32<C>(a.prev + (size_t)b * a.prev_stride);
    tok = tok < 0 ? 0 : tok;  // a free slot's token (never used) may read -1
  }
  double acc = 0.0;
  if (b < a.B && row < a.D) {
    acc = ld_f64<C>(a.pre + (size_t)b * a.ldpre + (size_t)a.s * a.D + row) +
          to_d(((const T*)a.table)[(size_t)tok * a.D + row]);
    st_f64<C>(a.y + (size_t)b * a.D + row, acc);
  }
  double ss = acc * acc;
  for (int off = a.ssq_rows / 2; off > 0; off >>= 1) ss += shfl_xor_d(ss, off);
  if (r % a.ssq_rows == 0 && b < a.B && row < a.D)
    st_f64<C>(a.ssq_out + (size_t)(row / a.ssq_rows) * a.B + b, ss);
}

}  // namespace moshi
