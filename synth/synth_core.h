/*
 * synth_core.h -- seeded, counter-based synthetic input generator.
 *
 * Inputs only: this header holds none of the method's arithmetic (no layout,
 * flatten, norm or optimizer math).  It is compiled twice, into the host fill
 * and into the device fill of libsynth.so, so that a value depends only on
 * (seed, stream, step, element index) and both fills produce the same bits:
 * every step is integer arithmetic or a single IEEE-754 double/float
 * operation rounded to nearest-even, and the build disables contraction.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast Splittable Pseudorandom
 * Number Generators", OOPSLA 2014) evaluated at counter k as
 * mix(key + (k + 1)·γ), γ = 0x9E3779B97F4A7C15.  Element i of a field uses
 * counters 4i .. 4i+3.
 *
 * Approximately normal values: Irwin–Hall sum of twelve 16-bit uniforms
 * (three draws), centred: z = (Σu − 12·32767.5)·2^-16, so E[z] = 0 and
 * Var[z] = 1 − 2^-32, |z| < 6.  Exact in double.
 */
#ifndef ZERO_SYNTH_CORE_H
#define ZERO_SYNTH_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYN_HD __host__ __device__ static inline
#else
#define SYN_HD static inline
#endif

#define SYN_GAMMA 0x9E3779B97F4A7C15ull

typedef struct {
  uint64_t seed;
  uint32_t stream;               /* value stream: 1 grads, 2 master init, ... */
  uint32_t step;                 /* training step (0 for initial state) */
  double sigma;                  /* value = sigma·z ... */
  double scale;                  /* ... then ·scale (a loss scale; 1 otherwise) */
  uint32_t outlier_per_million;  /* elements replaced by outlier_sigma·z' */
  uint32_t kind;                 /* 0 = f32, 1 = bf16, 2 = fp16 */
  double outlier_sigma;
} syn_field;

enum { SYN_F32 = 0, SYN_BF16 = 1, SYN_FP16 = 2 };

/* One destination of a multi-buffer device fill: elements idx0 .. idx0+n-1
 * of the field, written to out[0 .. n). */
typedef struct {
  void* out;
  int64_t idx0;
  int64_t n;
} syn_piece;

SYN_HD uint64_t syn_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

SYN_HD uint64_t syn_key(uint64_t seed, uint32_t stream, uint32_t step) {
  uint64_t k = syn_mix64(seed + SYN_GAMMA);
  return syn_mix64(k ^ (((uint64_t)stream << 32) | (uint64_t)step));
}

SYN_HD uint64_t syn_draw(uint64_t key, uint64_t counter) {
  return syn_mix64(key + (counter + 1ull) * SYN_GAMMA);
}

SYN_HD uint32_t syn_sum4x16(uint64_t d) {
  return (uint32_t)(d & 0xFFFFu) + (uint32_t)((d >> 16) & 0xFFFFu) + (uint32_t)((d >> 32) & 0xFFFFu) +
         (uint32_t)(d >> 48);
}

/* Centred Irwin–Hall(12) value for element i of the field with this key. */
SYN_HD double syn_normal(uint64_t key, uint64_t i) {
  uint32_t s = syn_sum4x16(syn_draw(key, 4 * i)) + syn_sum4x16(syn_draw(key, 4 * i + 1)) +
               syn_sum4x16(syn_draw(key, 4 * i + 2));
  return (double)((int64_t)s - 393210) * 0x1p-16;
}

SYN_HD uint32_t syn_f32_bits(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  return c.u;
}

/* Input encodings (finite values only reach these). */
SYN_HD uint16_t syn_enc_bf16(float f) {
  uint32_t u = syn_f32_bits(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

SYN_HD uint16_t syn_enc_fp16(float f) {
  uint32_t x = syn_f32_bits(f);
  uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  uint32_t a = x & 0x7FFFFFFFu;
  if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520 rounds to inf */
  if (a >= 0x38800000u) {                                  /* normal fp16 */
    uint32_t r = ((a >> 23) - 112u) << 10 | ((a >> 13) & 0x3FFu);
    uint32_t rest = a & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (r & 1u))) r += 1u;
    return (uint16_t)(sign | r);
  }
  uint32_t e = a >> 23; /* subnormal fp16 (or zero): units of 2^-24 */
  if (e < 102u) return sign;
  uint32_t mant = (a & 0x7FFFFFu) | 0x800000u;
  uint32_t shift = 126u - e; /* 14 .. 24 */
  uint32_t r = mant >> shift;
  uint32_t rest = mant & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1u);
  if (rest > half || (rest == half && (r & 1u))) r += 1u;
  return (uint16_t)(sign | r);
}

/* The value of element i (global flat index) of the field, before encoding. */
SYN_HD float syn_value_f32(const syn_field* f, uint64_t key, uint64_t okey, uint64_t i) {
  double v;
  if (f->outlier_per_million != 0u &&
      (syn_draw(key, 4 * i + 3) >> 11) % 1000000ull < (uint64_t)f->outlier_per_million) {
    v = f->outlier_sigma * syn_normal(okey, i);
  } else {
    v = f->sigma * syn_normal(key, i);
  }
  v = v * f->scale;
  return (float)v;
}

#endif
