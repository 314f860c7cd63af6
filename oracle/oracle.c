/*
 * oracle.c -- plain, slow, single-threaded CPU oracle.  TEST INFRASTRUCTURE
 * ONLY (see oracle.h): no product code may use it.  Built with
 * -O2 -ffp-contract=off and no fast-math, so every float/double operation
 * below is one IEEE-754 operation rounded to nearest-even, in source order.
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

#define ORC_MAX_PSI (INT64_MAX / 32)

/* ---------------------------------------------------------------- codecs */

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
float orc_bf16_to_f32(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int frac = h & 0x3FF;
  double mag;
  if (e == 0) {
    mag = ldexp((double)frac, -24); /* zero or subnormal: frac * 2^-24 */
  } else if (e == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(frac + 1024), e - 25); /* (1 + frac/1024) * 2^(e-15) */
  }
  return (float)(sign ? -mag : mag);
}

/* Round a binary32 to the nearest bf16, ties to the even bf16 (RNE).
 * A NaN stays a NaN (quiet bit set); overflow carries into infinity. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) {
    return (uint16_t)((u >> 16) | 0x0040u);
  }
  uint32_t kept = u >> 16;       /* truncated bf16 pattern */
  uint32_t rest = u & 0xFFFFu;   /* discarded low half */
  int round_up;
  if (rest > 0x8000u) {
    round_up = 1;
  } else if (rest < 0x8000u) {
    round_up = 0;
  } else {
    round_up = (int)(kept & 1u); /* exact tie: go to the even neighbour */
  }
  return (uint16_t)(kept + (uint32_t)round_up);
}

/* Round a binary32 to the nearest IEEE binary16 value, ties to the value
 * with an even fraction; a magnitude that rounds past the largest finite
 * half (65504) becomes infinity.  Done on the exact value in double: for
 * 2^E <= |x| < 2^(E+1) with E >= -14 the binary16 values are spaced
 * q = 2^(E-10) apart, and below 2^-14 (subnormals) q = 2^-24; |x|/q is exact
 * in double and is rounded to an integer k, ties to even; the result is k·q.
 * A NaN stays a NaN (quiet bit set). */
uint16_t orc_f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7E00u | ((u >> 13) & 0x3FFu));
  if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);  /* 2^(e-1) <= a < 2^e */
  int E = e - 1;
  if (E < -14) E = -14;
  double q = ldexp(1.0, E - 10);
  double k = a / q;
  double r = floor(k);
  double rest = k - r;
  if (rest > 0.5 || (rest == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  double val = r * q;
  if (val > 65504.0) return (uint16_t)(sign | 0x7C00u);
  if (val < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)r); /* zero or subnormal: r·2^-24 */
  frexp(val, &e);
  E = e - 1;                                                          /* -14 <= E <= 15 */
  uint16_t fraction = (uint16_t)(ldexp(val, 10 - E) - 1024.0);        /* val = (1024 + fraction)·2^(E-10) */
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | fraction);
}

void orc_f32_to_f16_array(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_f16(x[i]);
}

static float orc_decode(uint16_t h, int32_t dtype) {
  return dtype == ORC_BF16 ? orc_bf16_to_f32(h) : orc_f16_to_f32(h);
}

/* ---------------------------------------------------------------- layout */

/* Partition rule: N_d equal partitions, partition i belongs to rank i
 * ([Z] section 四（一）; [Z] section 六（二） 8-parameter example, where
 * GPU i owns parameters 2i and 2i+1).  Reading: the pages assume N_d | Ψ;
 * for other Ψ we take S = ceil(Ψ/N) and pad the flat buffers to N·S with
 * zeros at the tail of the last shard(s).
 *
 * Per-rank model-state bytes with 2-byte params and grads and K = 12 bytes
 * of fp32 master/m/v ([O] opening equation; [Z] section 二（一）):
 *   DP     : every rank holds everything                  16·Ψ
 *   ZeRO-1 : full params + full grads, 1/N of optimizer    2·Ψp + 2·Ψp + 12·S
 *   ZeRO-2 : full params, 1/N of grads and optimizer       2·Ψp + (2+12)·S
 *   ZeRO-3 : 1/N of everything                             (2+2+12)·S
 * with Ψp = N·S the padded flat length ([X] section 三 lists the same four
 * rows as 16, 4+12/N, 2+14/N and 16/N bytes per parameter). */
int orc_layout_compute(const int64_t* numels, int32_t n_tensors, int32_t world, int32_t rank,
                       orc_layout* out, orc_segment* segs, int32_t segs_cap, int32_t* n_segs) {
  if (!out || !n_segs || n_tensors < 0 || (n_tensors > 0 && !numels) || world < 1 || rank < 0 ||
      rank >= world || segs_cap < 0 || (segs_cap > 0 && !segs)) {
    return ORC_ERR_INVALID;
  }
  int64_t psi = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    if (numels[t] < 0 || numels[t] > ORC_MAX_PSI - psi) return ORC_ERR_INVALID;
    psi += numels[t];
  }
  int64_t shard = psi / world + (psi % world != 0 ? 1 : 0);
  int64_t offset = (int64_t)rank * shard;
  int64_t valid = psi - offset;
  if (valid < 0) valid = 0;
  if (valid > shard) valid = shard;

  memset(out, 0, sizeof *out);
  out->psi = psi;
  out->padded_numel = (int64_t)world * shard;
  out->shard_numel = shard;
  out->shard_offset = offset;
  out->shard_valid = valid;
  out->world = world;
  out->rank = rank;
  out->bytes_dp = 16 * psi;
  out->bytes_zero1 = 2 * out->padded_numel + 2 * out->padded_numel + 12 * shard;
  out->bytes_zero2 = 2 * out->padded_numel + (2 + 12) * shard;
  out->bytes_zero3 = (2 + 2 + 12) * shard;

  /* Communication per step ([Z] section 六): a ring reduce-scatter over N
   * ranks takes N-1 rounds, each rank sending one 1/N chunk per round, and a
   * ring all-gather the same; so each moves (N-1)/N of the (padded) flat
   * space per rank.  Plain DP all-reduces the gradients (reduce-scatter +
   * all-gather); ZeRO-1/2 reduce-scatter the gradients and all-gather the
   * updated parameters; ZeRO-3 gathers the parameters for forward and again
   * for backward and reduce-scatters the gradients. */
  int64_t one_collective = (int64_t)(world - 1) * shard;
  out->comm_dp = one_collective + one_collective;
  out->comm_zero1 = one_collective + one_collective;
  out->comm_zero2 = one_collective + one_collective;
  out->comm_zero3 = one_collective + one_collective + one_collective;

  /* Tensors are laid end to end in list order; each contributes the part of
   * its flat range that falls inside [offset, offset + valid). */
  int32_t count = 0;
  int64_t start = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    int64_t lo = start > offset ? start : offset;
    int64_t end = start + numels[t];
    int64_t hi = end < offset + valid ? end : offset + valid;
    if (hi > lo) {
      if (count < segs_cap) {
        segs[count].tensor = t;
        segs[count].reserved = 0;
        segs[count].src_offset = lo - start;
        segs[count].dst_offset = lo - offset;
        segs[count].numel = hi - lo;
      }
      ++count;
    }
    start = end;
  }
  *n_segs = count;
  return count > segs_cap ? ORC_ERR_CAPACITY : ORC_OK;
}

/* ---------------------------------------------------------------- flatten */

/* The rank's contiguous gradient shard: element j is flat element
 * rank·S + j of the concatenated gradients, or +0 past Ψ ([Z] section 五（三）
 * pre-allocated contiguous gradient region; [Z] section 四（二） the rank keeps
 * only the reduced gradients of its own partition).  Tensors that do not
 * intersect the shard may be passed as NULL. */
int orc_flatten(const uint16_t* const* tensors, const int64_t* numels, int32_t n_tensors,
                int32_t world, int32_t rank, uint16_t* shard) {
  if (n_tensors < 0 || (n_tensors > 0 && (!tensors || !numels)) || world < 1 || rank < 0 ||
      rank >= world) {
    return ORC_ERR_INVALID;
  }
  int64_t psi = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    if (numels[t] < 0 || numels[t] > ORC_MAX_PSI - psi) return ORC_ERR_INVALID;
    psi += numels[t];
  }
  int64_t s = psi / world + (psi % world != 0 ? 1 : 0);
  if (s > 0 && !shard) return ORC_ERR_INVALID;
  int32_t t = 0;
  int64_t t_start = 0;
  for (int64_t j = 0; j < s; ++j) {
    int64_t k = (int64_t)rank * s + j;
    if (k >= psi) {
      shard[j] = 0;
      continue;
    }
    while (k >= t_start + numels[t]) {
      t_start += numels[t];
      ++t;
    }
    if (!tensors[t]) return ORC_ERR_INVALID;
    shard[j] = tensors[t][k - t_start];
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------- grad norm */

/* Local part of the global L2 grad norm that optimizer.step() reduces across
 * ranks before clipping ([G] table "AdamW全局grad_norm"; [Z] section 二（二）
 * gradients are flattened for the norm).  Reading: accumulate x² in fp64 in
 * index order (each square is exact in fp64 for 16-bit inputs); an element
 * whose exponent field is all ones (inf or NaN) sets the nonfinite flag. */
int orc_sqnorm(const uint16_t* x, int32_t dtype, int64_t n, double* sqnorm, int32_t* nonfinite) {
  if (n < 0 || (n > 0 && !x) || !sqnorm || !nonfinite || (dtype != ORC_BF16 && dtype != ORC_FP16)) {
    return ORC_ERR_INVALID;
  }
  uint16_t expmask = dtype == ORC_BF16 ? 0x7F80u : 0x7C00u;
  double acc = 0.0;
  int32_t flag = 0;
  for (int64_t i = 0; i < n; ++i) {
    double g = (double)orc_decode(x[i], dtype);
    double sq = g * g;
    acc = acc + sq;
    if ((x[i] & expmask) == expmask) flag = 1;
  }
  *sqnorm = acc;
  *nonfinite = flag;
  return ORC_OK;
}

/* Clip coefficient from the global norm ([G]: the norm gives clip_coeff).
 * Reading (torch.nn.utils.clip_grad_norm_ convention): coef =
 * max_norm / (||g|| + 1e-6), capped at 1; max_norm <= 0 disables clipping. */
double orc_clip_coef(double global_sqnorm, double max_norm) {
  if (!(max_norm > 0.0)) return 1.0;
  double norm = sqrt(global_sqnorm);
  double coef = max_norm / (norm + 1e-6);
  return coef < 1.0 ? coef : 1.0;
}

/* Dynamic loss scaling for fp16 training (the pages only enable fp16).
 * Reading (torch.amp.GradScaler convention): an overflow halves the scale and
 * resets the good-step count; growth_interval consecutive good steps double
 * it.  The caller skips the optimizer step when nonfinite is set. */
int orc_loss_scale_update(double* scale, int32_t nonfinite, int32_t* good_steps, int32_t growth_interval) {
  if (!scale || !good_steps || growth_interval < 1) return ORC_ERR_INVALID;
  if (nonfinite) {
    *scale = *scale * 0.5;
    *good_steps = 0;
  } else {
    *good_steps = *good_steps + 1;
    if (*good_steps >= growth_interval) {
      *scale = *scale * 2.0;
      *good_steps = 0;
    }
  }
  return ORC_OK;
}

/* One rank's host decision after the norm all-reduce, composed from the two
 * functions above.  The simulated all-reduce sums the ranks' fp64 partial
 * square-norms in rank order and ORs their flags.  The grads hold g times
 * the loss scale, so the unscaled square-norm is global / scale²; the update
 * multiplies each gradient by coef / scale.  Overflow skips the update.
 * Reading (the pages never reach it): a loss scale that is not a positive
 * finite number, or so small that scale² underflows and a step without
 * overflow has no finite unscaled norm, cannot give a decision: refused,
 * nothing written. */
int orc_step_decision(const double* rank_sqnorms, const int32_t* rank_flags, int32_t n_ranks, double max_norm,
                      double* loss_scale, int32_t* good_steps, int32_t growth_interval, double* grad_scale,
                      int32_t* skip, double* global_norm) {
  if (n_ranks < 1 || !rank_sqnorms || !rank_flags || !loss_scale || !good_steps || !grad_scale || !skip ||
      !global_norm || growth_interval < 1 || !(*loss_scale > 0.0)) {
    return ORC_ERR_INVALID;
  }
  double total = 0.0;
  int32_t flag = 0;
  for (int32_t r = 0; r < n_ranks; ++r) {
    total = total + rank_sqnorms[r];
    if (rank_flags[r]) flag = 1;
  }
  double scale = *loss_scale;
  if (!isfinite(scale)) return ORC_ERR_INVALID;
  if (!flag && !isfinite(total / (scale * scale))) return ORC_ERR_INVALID;
  if (flag) {
    *skip = 1;
    *grad_scale = 0.0;
    *global_norm = NAN;
  } else {
    double unscaled = total / (scale * scale);
    double coef = orc_clip_coef(unscaled, max_norm);
    *skip = 0;
    *grad_scale = coef / scale;
    *global_norm = sqrt(unscaled);
  }
  return orc_loss_scale_update(loss_scale, flag, good_steps, growth_interval);
}

/* Reading for a changing learning rate: half-cosine from lr_max at t=1 down
 * to lr_min at t=total. */
double orc_cosine_lr(int64_t t, int64_t total, double lr_max, double lr_min) {
  if (total <= 1) return lr_max;
  double frac = (double)(t - 1) / (double)(total - 1);
  return lr_min + 0.5 * (lr_max - lr_min) * (1.0 + cos(M_PI * frac));
}

/* ---------------------------------------------------------------- AdamW */

/* Host scalars, computed in fp64 and rounded once to fp32. */
int orc_adamw_scalars(const orc_hparams* hp, orc_scalars* s) {
  if (!hp || !s || hp->step < 1 || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
      !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !(hp->eps >= 0.0) || !(hp->lr >= 0.0) ||
      !(hp->weight_decay >= 0.0) || !isfinite(hp->grad_scale)) {
    return ORC_ERR_INVALID;
  }
  double bc1 = 1.0 - pow(hp->beta1, (double)hp->step);
  double bc2 = 1.0 - pow(hp->beta2, (double)hp->step);
  s->b1 = (float)hp->beta1;
  s->omb1 = (float)(1.0 - hp->beta1);
  s->b2 = (float)hp->beta2;
  s->omb2 = (float)(1.0 - hp->beta2);
  s->eps = (float)hp->eps;
  s->decay = (float)(1.0 - hp->lr * hp->weight_decay);
  s->step_size = (float)(hp->lr / bc1);
  s->bc2_sqrt = (float)sqrt(bc2);
  s->gscale = (float)hp->grad_scale;
  return ORC_OK;
}

/* One AdamW step on the rank's fp32 master / m / v shard, writing the bf16
 * parameter shard that the all-gather sends ([Z] section 四（一）: rank i
 * updates only partition i, then parameters are all-gathered; [O] opening
 * equation: bf16 weights and grads, fp32 m, v and master).  The pages name
 * AdamW but print no update equations.  Reading: bias-corrected Adam with
 * decoupled weight decay applied as p·(1 − lr·wd) (the torch.optim.AdamW
 * convention), evaluated per element in fp32 in exactly this order:
 *   g ← gscale·g            (unscale by the loss scale and clip)
 *   m ← β1·m + (1−β1)·g
 *   v ← β2·v + (1−β2)·(g·g)
 *   d ← sqrt(v) / sqrt(1−β2^t) + eps
 *   p ← p·(1 − lr·wd) − (lr/(1−β1^t))·(m/d)
 *   param ← rne16(p)
 * where rne16 rounds to bf16 or, for fp16 parameters ([Z] section 四（一）:
 * fp16 parameters and gradients stay whole on every process; [D]: fp16
 * enabled in the training configuration), to IEEE binary16.                */
int orc_adamw_step(const uint16_t* grad, int32_t dtype, float* master, float* m, float* v,
                   uint16_t* param16, int32_t param_dtype, int64_t n, const orc_hparams* hp) {
  orc_scalars s;
  if (n < 0 || (dtype != ORC_BF16 && dtype != ORC_FP16)) return ORC_ERR_INVALID;
  if (param_dtype != ORC_BF16 && param_dtype != ORC_FP16) return ORC_ERR_INVALID;
  if (n > 0 && (!grad || !master || !m || !v || !param16)) return ORC_ERR_INVALID;
  if (orc_adamw_scalars(hp, &s) != ORC_OK) return ORC_ERR_INVALID;
  for (int64_t i = 0; i < n; ++i) {
    float g = orc_decode(grad[i], dtype);
    g = g * s.gscale;

    float m_old = s.b1 * m[i];
    float m_new = s.omb1 * g;
    m_new = m_old + m_new;

    float gg = g * g;
    float v_old = s.b2 * v[i];
    float v_new = s.omb2 * gg;
    v_new = v_old + v_new;

    float d = sqrtf(v_new);
    d = d / s.bc2_sqrt;
    d = d + s.eps;

    float u = m_new / d;
    u = s.step_size * u;

    float p = master[i] * s.decay;
    p = p - u;

    m[i] = m_new;
    v[i] = v_new;
    master[i] = p;
    param16[i] = param_dtype == ORC_BF16 ? orc_f32_to_bf16(p) : orc_f32_to_f16(p);
  }
  return ORC_OK;
}

/* The same update with every quantity in fp64; the reference point for the
 * rounding error of the fp32 update above. */
int orc_adamw_step_f64(const double* grad, double* master, double* m, double* v, int64_t n,
                       const orc_hparams* hp) {
  if (n < 0 || !hp || hp->step < 1) return ORC_ERR_INVALID;
  if (n > 0 && (!grad || !master || !m || !v)) return ORC_ERR_INVALID;
  double bc1 = 1.0 - pow(hp->beta1, (double)hp->step);
  double bc2 = 1.0 - pow(hp->beta2, (double)hp->step);
  for (int64_t i = 0; i < n; ++i) {
    double g = grad[i] * hp->grad_scale;
    m[i] = hp->beta1 * m[i] + (1.0 - hp->beta1) * g;
    v[i] = hp->beta2 * v[i] + (1.0 - hp->beta2) * (g * g);
    double d = sqrt(v[i]) / sqrt(bc2) + hp->eps;
    master[i] = master[i] * (1.0 - hp->lr * hp->weight_decay) - (hp->lr / bc1) * (m[i] / d);
  }
  return ORC_OK;
}

/* Batch helpers so tests can sweep codecs without a call per element. */
void orc_f32_to_bf16_array(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_bf16(x[i]);
}

void orc_decode_array(const uint16_t* x, int32_t dtype, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_decode(x[i], dtype);
}
