/*
 * synth.c -- seeded synthetic inputs for the Moshi frame step.
 *
 * This module only draws numbers; it holds none of the model's arithmetic.
 * Both the CPU oracle and the HIP library consume the host arrays it fills.
 *
 * Generator (counter based, so any element is a pure function of
 * (seed, tensor id, element index)):
 *   key      = splitmix64_finalise(splitmix64_finalise(seed) ^ (tensor * 0xD1B54A32D192ED03))
 *   U(n)     = splitmix64 output n of a generator whose state starts at `key`,
 *              i.e. finalise(key + (n + 1) * 0x9E3779B97F4A7C15)
 *              (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *              generators", OOPSLA 2014).
 *   unit(x)  = ((x >> 11) + 1) * 2^-53, a double in (0, 1].
 *   normal element i: pair j = i / 2 draws u1 = unit(U(2j)), u2 = unit(U(2j+1));
 *              r = sqrt(-2 ln u1), t = 2 pi u2 (Box & Muller 1958);
 *              element 2j = r cos t, element 2j+1 = r sin t; scaled by `std`.
 *   integer element i in [0, n): (U(i) * n) >> 64 (Lemire multiply-shift).
 *   bf16 values: fp64 -> fp32 (round to nearest even) -> bf16 (round to
 *              nearest even on the upper 16 bits).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t finalise(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor) {
  return finalise(finalise(seed) ^ (tensor * 0xD1B54A32D192ED03ull));
}

static inline uint64_t draw(uint64_t key, uint64_t n) {
  return finalise(key + (n + 1) * 0x9E3779B97F4A7C15ull);
}

static inline double unit(uint64_t x) { return (double)((x >> 11) + 1) * 0x1.0p-53; }

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t j = i >> 1;
  double u1 = unit(draw(key, 2 * j));
  double u2 = unit(draw(key, 2 * j + 1));
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(t) : r * cos(t);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* ---- single-threaded kernels over [offset, offset+count) ---- */

/* Both draws of Box-Muller pair j (elements 2j and 2j+1). */
static inline void normal_pair(uint64_t key, uint64_t j, double* z0, double* z1) {
  double u1 = unit(draw(key, 2 * j));
  double u2 = unit(draw(key, 2 * j + 1));
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(t);
  *z1 = r * sin(t);
}

static void fill_normal_any(uint64_t key, uint64_t off, uint64_t cnt, double stdv, void* out,
                            int bf16) {
  uint64_t i = 0;
  while (i < cnt) {
    uint64_t e = off + i;
    double z[2];
    normal_pair(key, e >> 1, &z[0], &z[1]);
    for (int h = (int)(e & 1); h < 2 && i < cnt; ++h, ++i) {
      float f = (float)(stdv * z[h]);
      if (bf16)
        ((uint16_t*)out)[i] = f32_to_bf16_rne(f);
      else
        ((float*)out)[i] = f;
    }
  }
}

static void fill_normal_f32(uint64_t key, uint64_t off, uint64_t cnt, double stdv, float* out) {
  fill_normal_any(key, off, cnt, stdv, out, 0);
}

static void fill_normal_bf16(uint64_t key, uint64_t off, uint64_t cnt, double stdv, uint16_t* out) {
  fill_normal_any(key, off, cnt, stdv, out, 1);
}

/* ---- threaded front ends ---- */

typedef struct {
  uint64_t key, off, cnt;
  double stdv;
  void* out;
  int bf16;
} job_t;

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  if (j->bf16)
    fill_normal_bf16(j->key, j->off, j->cnt, j->stdv, (uint16_t*)j->out);
  else
    fill_normal_f32(j->key, j->off, j->cnt, j->stdv, (float*)j->out);
  return NULL;
}

static int fill_normal(uint64_t seed, uint64_t tensor, uint64_t off, uint64_t cnt, double stdv,
                       void* out, int bf16, int nthreads) {
  uint64_t key = stream_key(seed, tensor);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (cnt < (uint64_t)nthreads * 65536u) nthreads = 1;
  if (nthreads == 1) {
    job_t j = {key, off, cnt, stdv, out, bf16};
    run_job(&j);
    return 0;
  }
  pthread_t th[256];
  job_t jobs[256];
  uint64_t per = (cnt + nthreads - 1) / nthreads;
  per = (per + 1) & ~1ull; /* keep Box-Muller pairs inside one job (not required, tidy) */
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t b = (uint64_t)t * per;
    if (b >= cnt) break;
    uint64_t e = b + per < cnt ? b + per : cnt;
    size_t esz = bf16 ? 2 : 4;
    jobs[t] = (job_t){key, off + b, e - b, stdv, (char*)out + b * esz, bf16};
    if (pthread_create(&th[t], NULL, run_job, &jobs[t]) != 0) {
      run_job(&jobs[t]);
      th[t] = 0;
      jobs[t].cnt = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (th[t]) pthread_join(th[t], NULL);
  return 0;
}

/* Normal(0, std) draws, elements [offset, offset+count) of stream (seed, tensor), as fp32. */
int synth_normal_f32(uint64_t seed, uint64_t tensor, uint64_t offset, uint64_t count, double stdv,
                     float* out, int nthreads) {
  if (!out && count) return -1;
  return fill_normal(seed, tensor, offset, count, stdv, out, 0, nthreads);
}

/* The same draws, stored as bf16 bit patterns. */
int synth_normal_bf16(uint64_t seed, uint64_t tensor, uint64_t offset, uint64_t count, double stdv,
                      uint16_t* out, int nthreads) {
  if (!out && count) return -1;
  return fill_normal(seed, tensor, offset, count, stdv, out, 1, nthreads);
}

/* The same draws in fp64 (used by tests that need the unrounded values). */
int synth_normal_f64(uint64_t seed, uint64_t tensor, uint64_t offset, uint64_t count, double stdv,
                     double* out) {
  uint64_t key = stream_key(seed, tensor);
  for (uint64_t i = 0; i < count; ++i) out[i] = stdv * normal_at(key, offset + i);
  return 0;
}

/* Uniform integers: element i of stream (seed, tensor) lies in [0, bound[i % period]). */
int synth_uniform_int(uint64_t seed, uint64_t tensor, uint64_t offset, uint64_t count,
                      const int32_t* bound, int32_t period, int32_t* out) {
  if (period < 1) return -1;
  uint64_t key = stream_key(seed, tensor);
  for (uint64_t i = 0; i < count; ++i) {
    uint64_t idx = offset + i;
    uint64_t n = (uint64_t)(uint32_t)bound[idx % (uint64_t)period];
    unsigned __int128 m = (unsigned __int128)draw(key, idx) * n;
    out[i] = (int32_t)(uint64_t)(m >> 64);
  }
  return 0;
}

/* Raw 64-bit draws (for statistical tests of the generator itself). */
int synth_raw_u64(uint64_t seed, uint64_t tensor, uint64_t offset, uint64_t count, uint64_t* out) {
  uint64_t key = stream_key(seed, tensor);
  for (uint64_t i = 0; i < count; ++i) out[i] = draw(key, offset + i);
  return 0;
}
