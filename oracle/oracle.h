/*
 * oracle.h -- plain, slow, single-threaded CPU oracle for one data-parallel
 * rank's share of a ZeRO step (sharded mixed-precision AdamW).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library: every definition below is written out again
 * here from the pages' statement of the problem.
 *
 * Sources (web pages on ZeRO; cited by title and section):
 *   [Z]  "【论文解读】ZeRO" (wkq9411.github.io): section 二（一） model-state
 *        ledger, section 四 ZeRO-DP three partitioning stages, section 六（二）
 *        8-parameter / 4-GPU partition example, section 八 summary formulas.
 *   [X]  "ZeRO 显存优化：ZeRO-1、ZeRO-2 与 ZeRO-3" (xiangdong0520.pages.dev):
 *        section 三, per-card bytes for DP / ZeRO-1 / ZeRO-2 / ZeRO-3.
 *   [O]  operatorworld.com "ai-zero-optimizer-sharding": opening display
 *        equation, 16 bytes per parameter with bf16 weights and grads and
 *        fp32 m, v and master weights.
 *   [G]  gitcode.csdn.net Megatron distributed-optimizer note: table
 *        "AdamW全局grad_norm" -- the global L2 grad norm is reduced inside
 *        optimizer.step() before clipping and gives the clip coefficient.
 *
 * Parity status of each function is stated next to it.  "Reading" marks a
 * choice the pages leave open.
 */
#ifndef ZERO_ORACLE_H
#define ZERO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_ERR_INVALID = -1, ORC_ERR_CAPACITY = -2 };
enum { ORC_BF16 = 0, ORC_FP16 = 1 };

typedef struct {
  int64_t psi;           /* total parameters Ψ */
  int64_t padded_numel;  /* N·S */
  int64_t shard_numel;   /* S = ceil(Ψ/N) */
  int64_t shard_offset;  /* rank·S */
  int64_t shard_valid;   /* elements of this shard below Ψ */
  int32_t world, rank;
  int64_t bytes_dp, bytes_zero1, bytes_zero2, bytes_zero3;
  int64_t comm_dp, comm_zero1, comm_zero2, comm_zero3; /* elements sent per rank per step */
} orc_layout;

typedef struct {
  int32_t tensor;
  int32_t reserved;
  int64_t src_offset;  /* element offset inside the tensor */
  int64_t dst_offset;  /* element offset inside the shard */
  int64_t numel;
} orc_segment;

typedef struct {
  double lr, beta1, beta2, eps, weight_decay, grad_scale;
  int64_t step; /* 1-based Adam step counter */
} orc_hparams;

/* fp32 scalars handed to the per-element update, each rounded once from fp64. */
typedef struct {
  float b1, omb1, b2, omb2, eps, decay, step_size, bc2_sqrt, gscale;
} orc_scalars;

/* Layout of rank `rank` of `world` over the flat concatenation of the tensors.
 * Pinned to: the per-rank memory figures the pages print ([X] section 三,
 * [Z] section 八, [O]), their other algebraic forms, the 8-parameter /
 * 4-GPU example ([Z] section 六（二）), the communication volumes of [Z]
 * section 六, and brute-force coverage of every Ψ <= 64, N <= 9. */
int orc_layout_compute(const int64_t* numels, int32_t n_tensors, int32_t world, int32_t rank,
                       orc_layout* out, orc_segment* segs, int32_t segs_cap, int32_t* n_segs);

/* shard[j] = flat[rank·S + j] for flat index < Ψ, else +0 (bit copy).
 * Pinned to: numpy concatenation and slicing (the definition), the
 * 8-parameter example. */
int orc_flatten(const uint16_t* const* tensors, const int64_t* numels, int32_t n_tensors,
                int32_t world, int32_t rank, uint16_t* shard);

/* Σ x_j² accumulated in fp64 in index order; nonfinite = any all-ones exponent.
 * Pinned to: exact rational sums within the sequential rounding bound, hand
 * vectors, numpy and torch fp64, inf/NaN patterns of both formats. */
int orc_sqnorm(const uint16_t* x, int32_t dtype, int64_t n, double* sqnorm, int32_t* nonfinite);

/* Clip coefficient, loss-scale update and the decision that composes them
 * (reading of [G]: torch clip_grad_norm_ and GradScaler conventions).
 * Pinned to: torch clip_grad_norm_ and torch's loss-scale update on the CPU;
 * overflow skips and halves.  The cosine rate: pinned to torch's
 * CosineAnnealingLR closed form.  The policies themselves are readings the
 * pages do not fix (parity unpinned by the pages). */
double orc_clip_coef(double global_sqnorm, double max_norm);
int orc_loss_scale_update(double* scale, int32_t nonfinite, int32_t* good_steps, int32_t growth_interval);
int orc_step_decision(const double* rank_sqnorms, const int32_t* rank_flags, int32_t n_ranks, double max_norm,
                      double* loss_scale, int32_t* good_steps, int32_t growth_interval, double* grad_scale,
                      int32_t* skip, double* global_norm);
double orc_cosine_lr(int64_t t, int64_t total, double lr_max, double lr_min);

/* AdamW on the shard (reading: torch.optim.AdamW convention; the pages name
 * AdamW but print no equations).  Pinned to: torch.optim.AdamW in fp64 and
 * fp32, the fp64 variant within its rounding bound, the step-1 closed form,
 * a four-element two-step worked example, lr = 0 / beta = 0 / zero padding
 * special cases, the shard-concatenation invariance; fp16 parameters to
 * torch's binary16 conversion.  The update form itself is a reading (parity
 * unpinned by the pages). */
int orc_adamw_scalars(const orc_hparams* hp, orc_scalars* out);
int orc_adamw_step(const uint16_t* grad, int32_t dtype, float* master, float* m, float* v,
                   uint16_t* param16, int32_t param_dtype, int64_t n, const orc_hparams* hp);

/* Same update in fp64 throughout (no fp32 rounding of state or scalars);
 * used only to bound the fp32 oracle's rounding error. */
int orc_adamw_step_f64(const double* grad, double* master, double* m, double* v, int64_t n,
                       const orc_hparams* hp);

/* Number codecs.  Pinned to: all 65536 patterns of each 16-bit format
 * against torch / numpy; rounding to bf16 and to binary16 against torch and
 * numpy on every rounding boundary and millions of random patterns. */
float orc_bf16_to_f32(uint16_t h);
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);
void orc_f32_to_bf16_array(const float* x, uint16_t* y, int64_t n);
uint16_t orc_f32_to_f16(float f);
void orc_f32_to_f16_array(const float* x, uint16_t* y, int64_t n);
void orc_decode_array(const uint16_t* x, int32_t dtype, float* y, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
