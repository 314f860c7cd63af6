/*
 * zero_shard.h -- C ABI of libzero_shard.so: one data-parallel rank's share of
 * a ZeRO-1/2/3 mixed-precision AdamW step on an AMD Instinct MI355X (gfx950).
 *
 * What the step computes comes from these web pages on ZeRO (cited by title
 * and section):
 *   [Z] "【论文解读】ZeRO" (wkq9411.github.io)
 *   [X] "ZeRO 显存优化：ZeRO-1、ZeRO-2 与 ZeRO-3" (xiangdong0520.pages.dev)
 *   [O] operatorworld.com "ai-zero-optimizer-sharding"
 *   [D] "3、ZeRO技术概述：ZeRO三个阶段原理与对比" (5688vip.com DeepSpeed tutorial)
 *   [G] gitcode.csdn.net note on Megatron's distributed optimizer and ZeRO
 *
 * The rank's step, in call order:
 *   zero_shard_layout     which 1/N slice of the flat model state the rank owns
 *   zero_flatten_grads    per-tensor 16-bit grads -> the rank's contiguous shard
 *   zero_grad_sqnorm      local Σg² (fp64) and an inf/NaN flag over the shard
 *                         (zero_flatten_grads_sqnorm does both in one pass)
 *   zero_step_decision    global norm -> clip coefficient, loss scale, skip
 *   zero_adamw_step       fused AdamW on fp32 master/m/v + bf16 param writeback
 *
 * Conventions for every function:
 *   - Status: ZERO_OK (0) or a negative ZERO_ERR_*; zero_last_error() returns
 *     a message for the calling thread's last failure.  A status covers
 *     argument validation and kernel-launch errors only, not kernel results.
 *   - Memory: the caller allocates and frees every buffer (device buffers,
 *     workspace, segment tables).  The library never allocates or frees
 *     device memory.  Its only mutable global state is the per-thread error
 *     message and, for zero_flatten_grads_sqnorm_noalloc, one fixed-size
 *     scratch array per device (a static device variable) and its looked-up
 *     device addresses.
 *   - Device calls are asynchronous: they enqueue kernels on `stream` (a
 *     hipStream_t; NULL = the default stream) and return before completion.
 *   - Device buffers passed to one call must not overlap unless stated.
 *   - Sizes are element counts (int64); n = 0 is a valid no-op.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element counts are limited to 2^58 (ZERO_MAX_NUMEL): larger counts are
 * rejected with ZERO_ERR_INVALID, and the size queries return 0 for them. */
#define ZERO_MAX_NUMEL (INT64_MAX / 32)

enum {
  ZERO_OK = 0,
  ZERO_ERR_INVALID = -1,  /* bad argument (null pointer, negative or too large size, rank out of range, ...) */
  ZERO_ERR_CAPACITY = -2, /* caller-provided array too small; the required count is returned */
  ZERO_ERR_HIP = -3       /* the HIP runtime rejected a launch */
};

/* 16-bit floating-point formats.  Passed as a plain int32_t (an enum's size
 * and value range are implementation-defined across C and C++); any other
 * value is rejected with ZERO_ERR_INVALID. */
typedef int32_t zero_dtype;
enum { ZERO_BF16 = 0, ZERO_FP16 = 1 };

/* Message describing the calling thread's most recent failure ("" if none). */
const char* zero_last_error(void);

/* ------------------------------------------------------------------ layout
 *
 * [Z] section 四（一）: the optimizer state is split into N_d equal partitions
 * and rank i keeps and updates partition i; section 六（二） walks the same
 * rule on 8 parameters over 4 GPUs.  [Z] section 二（一） and [O]'s opening
 * equation give the ledger: 2 B param + 2 B grad (fp16/bf16) + 12 B fp32
 * master/m/v = 16 B per parameter; [X] section 三 and [Z] section 八 give the
 * per-rank bytes of DP / ZeRO-1 / ZeRO-2 / ZeRO-3.
 *
 * Reading where the pages assume N_d | Ψ: S = ceil(Ψ/N), every flat buffer
 * is padded with zeros to N·S, rank r owns flat elements [r·S, (r+1)·S).
 */
typedef struct zero_layout {
  int64_t psi;          /* Ψ: total parameters (sum of numels) */
  int64_t padded_numel; /* N·S */
  int64_t shard_numel;  /* S = ceil(Ψ/N) */
  int64_t shard_offset; /* r·S: first flat element of this rank's shard */
  int64_t shard_valid;  /* elements of the shard below Ψ; the rest is padding */
  int32_t world, rank;
  int64_t bytes_dp;     /* 16·Ψ */
  int64_t bytes_zero1;  /* 2·N·S + 2·N·S + 12·S */
  int64_t bytes_zero2;  /* 2·N·S + 14·S */
  int64_t bytes_zero3;  /* 16·S */
  /* Elements this rank sends per training step with ring collectives over the
   * padded flat space ([Z] section 六: a ring reduce-scatter or all-gather of
   * N·S elements sends (N-1)·S per rank; DP all-reduces the gradients (RS +
   * AG); ZeRO-1/2 reduce-scatter the gradients and all-gather the updated
   * parameters; ZeRO-3 also all-gathers the parameters once more, once for
   * forward and once for backward).  Multiply by the element size for bytes. */
  int64_t comm_dp;      /* 2·(N-1)·S */
  int64_t comm_zero1;   /* 2·(N-1)·S */
  int64_t comm_zero2;   /* 2·(N-1)·S */
  int64_t comm_zero3;   /* 3·(N-1)·S */
} zero_layout;

/* One piece of a tensor that lands in the shard. */
typedef struct zero_segment {
  int32_t tensor;     /* index into the tensor list */
  int32_t reserved;   /* 0 */
  int64_t src_offset; /* first element inside the tensor */
  int64_t dst_offset; /* first element inside the shard */
  int64_t numel;      /* > 0 */
} zero_segment;

/* Host only.  Tensors are laid end to end in list order (row-major each).
 * numels[n_tensors] >= 0; world >= 1; 0 <= rank < world; Σ numels <= 2^58.
 * Fills *out and up to segs_cap segments (sorted by dst_offset, contiguous,
 * covering [0, shard_valid)); *n_segs receives the full count.  If segs_cap
 * is too small, returns ZERO_ERR_CAPACITY after filling *out and *n_segs
 * (call again with a larger array).  segs may be NULL when segs_cap == 0. */
int zero_shard_layout(const int64_t* numels, int32_t n_tensors, int32_t world, int32_t rank, zero_layout* out,
                      zero_segment* segs, int32_t segs_cap, int32_t* n_segs);

/* ------------------------------------------------------------------ flatten
 *
 * [Z] section 五（三）: gradients are copied into a pre-allocated contiguous
 * region as they are produced; [Z] section 四（二）: a rank keeps only the
 * reduced gradients of its own partition (the buffer a reduce-scatter lands
 * in); [Z] section 二（二）: gradient norms flatten the gradients first.
 *
 * Device-side segment descriptor (32 bytes): element i of the piece is
 * src[src_offset + i] and goes to shard[dst_offset + i]. */
typedef struct zero_flat_seg {
  const void* src;    /* device address of the source tensor (16-bit elements) */
  int64_t src_offset;
  int64_t dst_offset;
  int64_t numel;
} zero_flat_seg;

/* Host only.  Packs layout segments and tensor base pointers into
 * descriptors: out[k] = {tensor_ptrs[segs[k].tensor], segs[k].src_offset,
 * segs[k].dst_offset, segs[k].numel}.  The caller copies `out` to device
 * memory for zero_flatten_grads. */
int zero_flatten_plan(const zero_segment* segs, int32_t n_segs, const void* const* tensor_ptrs, int32_t n_tensors,
                      zero_flat_seg* out);

/* Host only.  Constant-capacity buckets of the shard ([Z] section 五（二）:
 * fused buffers of a fixed capacity that does not grow with the model;
 * section 四（二）: gradients are bucketed and reduced bucket by bucket as
 * backward produces them).  Writes the parts of the layout's segments that
 * fall in the shard window [win_begin, win_begin + win_numel), with
 * dst_offset relative to the window, so that a bucket is flattened by
 * zero_flatten_grads[_sqnorm] on shard + win_begin with shard_numel =
 * win_numel.  Fills up to cap segments; *n_out receives the full count
 * (ZERO_ERR_CAPACITY when it exceeds cap).  Elements of the window past the
 * layout's shard_valid are padding (no segment covers them). */
int zero_bucket_segments(const zero_segment* segs, int32_t n_segs, int64_t win_begin, int64_t win_numel,
                         zero_segment* out, int32_t cap, int32_t* n_out);

/* Device.  segs_dev: n_segs descriptors in device memory, sorted by
 * dst_offset and non-overlapping, each inside [0, shard_numel).  Writes
 * shard[0, shard_numel): covered elements are bit copies of the source,
 * uncovered ones (padding) are +0.  Never writes outside the shard.  dt only
 * names the 16-bit format (the copy is bitwise).  The body of every piece
 * moves 16-byte vectors to 16-byte aligned destinations; when source and
 * destination differ in their position inside a 16-byte line, each vector is
 * assembled from the two aligned source lines it straddles (reads never leave
 * a 16-byte line that holds bytes of the piece).  Heads and tails shorter
 * than a vector are copied element by element. */
int zero_flatten_grads(const zero_flat_seg* segs_dev, int32_t n_segs, zero_dtype dt, void* shard_dev,
                       int64_t shard_numel, void* stream);

/* Device.  The same copy fused with the square-norm of the copied shard (one
 * pass over the gradients instead of two): writes the shard exactly as
 * zero_flatten_grads does and *sqnorm_dev / *nonfinite_dev exactly as
 * zero_grad_sqnorm would define them (padding contributes +0).  Deterministic
 * for a given shard_numel; the summation tree differs from
 * zero_grad_sqnorm's, so the two sums may differ in the last bits.  ws_dev
 * must hold zero_grad_sqnorm_workspace_bytes(shard_numel) bytes. */
int zero_flatten_grads_sqnorm(const zero_flat_seg* segs_dev, int32_t n_segs, zero_dtype dt, void* shard_dev,
                              int64_t shard_numel, void* ws_dev, size_t ws_bytes, double* sqnorm_dev,
                              int32_t* nonfinite_dev, void* stream);

/* Device.  For callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same fused flatten and norm as zero_flatten_grads_sqnorm, with the same
 * results bit for bit, but with its partials in a static scratch array of
 * ZERO_NOALLOC_SCRATCH_BYTES (6 MiB) per device instead of a caller
 * workspace.  That covers every shard size; a shard needing more scratch
 * than the array holds would be refused with ZERO_ERR_CAPACITY.  It calls no
 * allocating routine.  On its first call on a device the array's device
 * address is looked up (hipGetSymbolAddress) with that device current, so
 * call it with the stream's device current (a stream of another device is
 * refused with ZERO_ERR_INVALID).  Every call on one device shares that
 * device's array: calls that overlap in time on one device (two streams, two
 * threads) race on it and give wrong sums; serialize them.  The array keeps
 * the last call's partials; no call relies on its earlier contents (every
 * partial is written before it is read).  sqnorm_dev: 8-byte aligned;
 * nonfinite_dev: 4-byte aligned. */
#define ZERO_NOALLOC_SCRATCH_BYTES ((size_t)6 << 20)
int zero_flatten_grads_sqnorm_noalloc(const zero_flat_seg* segs_dev, int32_t n_segs, zero_dtype dt, void* shard_dev,
                                      int64_t shard_numel, double* sqnorm_dev, int32_t* nonfinite_dev, void* stream);

/* Bucketed norm.  With the shard split into constant-capacity windows
 * (zero_bucket_segments), each window is flattened as soon as its gradients
 * exist and leaves its per-workgroup partial square-sums and non-finite flags
 * side by side with the other windows'; one zero_sqnorm_reduce then folds
 * them all (fixed order: window by window, workgroup by workgroup), so a
 * bucket costs one launch.
 *
 * zero_flatten_partials_count: partials that zero_flatten_grads_partials
 * writes for a window of numel elements (0 for numel = 0).  Not monotone in
 * numel: size a shared partials buffer by summing the counts.
 *
 * zero_flatten_grads_partials (device): flattens the window exactly as
 * zero_flatten_grads does (dst_dev = the window's first shard element) and
 * writes the window's partials to part_sum_dev[0 .. count) (double, 8-byte
 * aligned) and part_flag_dev[0 .. count) (uint32, 4-byte aligned).  No final
 * reduction.
 *
 * zero_sqnorm_reduce (device): folds count partials into *sqnorm_dev and
 * *nonfinite_dev (0 or 1) in a fixed order (deterministic for a given
 * count), exactly as zero_flatten_grads_sqnorm folds its own.  Past 65536
 * partials the fold takes two levels and overwrites the partials: they are
 * scratch once reduced. */
int64_t zero_flatten_partials_count(int64_t numel);
int zero_flatten_grads_partials(const zero_flat_seg* segs_dev, int32_t n_segs, zero_dtype dt, void* dst_dev,
                                int64_t numel, double* part_sum_dev, uint32_t* part_flag_dev, void* stream);
int zero_sqnorm_reduce(double* part_sum_dev, uint32_t* part_flag_dev, int64_t count, double* sqnorm_dev,
                       int32_t* nonfinite_dev, void* stream);

/* ------------------------------------------------------------------ grad norm
 *
 * [G] table "AdamW全局grad_norm": inside optimizer.step() the global L2 norm
 * of the gradients is all-reduced before clipping and sets the clip
 * coefficient.  This call computes one rank's part: Σ g_j² over its shard,
 * accumulated in fp64 (each square is exact), and flags any element whose
 * exponent field is all ones (inf or NaN; bf16 0x7F80 mask, fp16 0x7C00).
 *
 * Deterministic: a fixed grid and fixed reduction tree give the same bits on
 * every run for the same n and pointer alignment.  The summation order is not
 * sequential, so results differ from a sequential fp64 sum by rounding only.
 * ws_dev: caller workspace of at least zero_grad_sqnorm_workspace_bytes(n)
 * bytes, 16-byte aligned.  Writes *sqnorm_dev (double) and *nonfinite_dev
 * (int32, 0 or 1); when the flag is set the sum is unspecified. */
size_t zero_grad_sqnorm_workspace_bytes(int64_t n);
int zero_grad_sqnorm(const void* shard_dev, zero_dtype dt, int64_t n, void* ws_dev, size_t ws_bytes,
                     double* sqnorm_dev, int32_t* nonfinite_dev, void* stream);

/* ------------------------------------------------------------------ host decision
 *
 * [G]: global norm -> clip coefficient.  The pages enable fp16 training
 * ([D] configuration) without describing loss scaling; readings:
 *   global = Σ_r rank_sqnorms[r] in rank order (the all-reduce's sum);
 *   nonfinite = OR of rank_flags;
 *   if nonfinite: *skip = 1, no update, *loss_scale halves, good steps reset;
 *   else: norm = sqrt(global / loss_scale²);
 *         coef = min(1, max_norm / (norm + 1e-6)) (max_norm <= 0: coef = 1);
 *         *grad_scale = coef / loss_scale; then growth_interval consecutive
 *         good steps double *loss_scale.
 * *global_norm receives the unscaled norm (NaN/inf when skipped).  For bf16
 * training pass loss_scale = 1 and growth_interval = INT32_MAX.
 * A loss scale that is not a positive finite number, or one so small that
 * loss_scale² underflows and the unscaled square-norm of a step without
 * overflow is not finite (after a long run of halvings), is refused with
 * ZERO_ERR_INVALID and nothing is written. */
int zero_step_decision(const double* rank_sqnorms, const int32_t* rank_flags, int32_t n_ranks, double max_norm,
                       double* loss_scale, int32_t* good_steps, int32_t growth_interval, double* grad_scale,
                       int32_t* skip, double* global_norm);

double zero_clip_coef(double global_sqnorm, double max_norm);
int zero_loss_scale_update(double* scale, int32_t nonfinite, int32_t* good_steps, int32_t growth_interval);
/* Half-cosine learning rate from lr_max at t = 1 to lr_min at t = total (reading). */
double zero_cosine_lr(int64_t t, int64_t total, double lr_max, double lr_min);

/* ------------------------------------------------------------------ AdamW
 *
 * [Z] section 四（一）: rank i updates only its partition of the optimizer
 * state and parameters, then parameters are all-gathered; [O] opening
 * equation and [Z] section 二（一）: bf16/fp16 weights and grads with fp32 m,
 * v and master weights.  The pages name AdamW ([O], [G]) but print no update
 * equations.  Reading: bias-corrected Adam with decoupled weight decay
 * p·(1 − lr·wd); host scalars are computed in fp64 and rounded once to fp32:
 *   b1 = β1, omb1 = 1−β1, b2 = β2, omb2 = 1−β2, eps, decay = 1 − lr·wd,
 *   step_size = lr / (1 − β1^t), bc2_sqrt = sqrt(1 − β2^t), gscale = grad_scale.
 * Per element, in fp32, round-to-nearest-even, no fused multiply-add, in
 * this order:
 *   g = gscale·g
 *   m = (b1·m) + (omb1·g)
 *   v = (b2·v) + (omb2·(g·g))
 *   d = ((sqrt(v) / bc2_sqrt) + eps)
 *   p = (p·decay) − (step_size·(m/d))
 *   param = p rounded to the parameter format pdt, nearest, ties to even:
 *           bf16, or IEEE binary16 for fp16 parameters ([Z] section 四（一）
 *           keeps fp16 parameters and gradients whole on every process; [D]
 *           trains with fp16 enabled); binary16 overflows to infinity and
 *           keeps subnormals.  NaN stays NaN.
 */
typedef struct zero_adamw_hparams {
  double lr;           /* >= 0 */
  double beta1, beta2; /* in [0, 1) */
  double eps;          /* >= 0 */
  double weight_decay; /* >= 0 */
  double grad_scale;   /* finite: clip coefficient / loss scale */
  int64_t step;        /* 1-based Adam step t */
} zero_adamw_hparams;

/* Device.  grad_dev: n gradients (bf16 or fp16, per gdt); master/m/v: n fp32
 * each, updated in place; param_dev: n 16-bit parameters in format pdt
 * (ZERO_BF16 or ZERO_FP16), written (never read).  Buffers
 * must be aligned to their element size.  When grad and param are 8-byte
 * aligned and master/m/v 16-byte aligned the kernel streams whole vectors;
 * otherwise (and for the last n mod 4 elements) it updates element by
 * element with identical results. */
int zero_adamw_step(const void* grad_dev, zero_dtype gdt, float* master_dev, float* m_dev, float* v_dev,
                    uint16_t* param_dev, zero_dtype pdt, int64_t n, const zero_adamw_hparams* hp, void* stream);

/* Tiled optimizer state: the same fp32 master / m / v, interleaved in tiles of
 * ZERO_STATE_TILE elements.  Tile k holds master[T·k .. T·k+T), then m[...],
 * then v[...] (T = ZERO_STATE_TILE, 12·T = 12 KiB per tile), so the update
 * streams three address ranges (grad, state, param) instead of five; on
 * MI355X the tiled update runs about 6% faster than the separate-array one
 * (6.66 against 6.27 TB/s on a 1.95e8-element shard).  A shard of n
 * elements needs zero_state_tiled_numel(n) floats (the last tile is padded).
 * zero_adamw_step_tiled computes exactly what zero_adamw_step computes (same
 * per-element operations, same bits); state_dev must be 16-byte aligned. */
#define ZERO_STATE_TILE 1024
int64_t zero_state_tiled_numel(int64_t n);
int zero_adamw_step_tiled(const void* grad_dev, zero_dtype gdt, float* state_dev, uint16_t* param_dev,
                          zero_dtype pdt, int64_t n, const zero_adamw_hparams* hp, void* stream);
/* Device bit copies between separate master/m/v arrays and the tiled state
 * (for initialisation and checkpoints); padding floats are left untouched.
 * All four buffers must be 4-byte aligned; NULL buffers (n > 0), n outside
 * [0, ZERO_MAX_NUMEL] or misalignment give ZERO_ERR_INVALID. */
int zero_state_tile(const float* master_dev, const float* m_dev, const float* v_dev, float* state_dev, int64_t n,
                    void* stream);
int zero_state_untile(const float* state_dev, float* master_dev, float* m_dev, float* v_dev, int64_t n, void* stream);

/* ------------------------------------------------------------------ device-resident decision
 *
 * The same decision (zero_step_decision) and scalar derivation (zero_adamw_step)
 * evaluated by one GPU thread, so a step needs no host round trip between the
 * norm and the update: flatten+norm -> zero_step_decision_dev ->
 * zero_adamw_step_[tiled_]dev, all enqueued back to back on one stream (and
 * capturable in a HIP graph: no memset, copy or host callback is involved).
 * The state lives in caller-allocated device memory; read it back at will.
 * The fp64 host arithmetic of the decision is repeated on the device with the
 * same IEEE operations (correctly rounded +, -, *, /, sqrt); beta^t uses the
 * device pow, which can differ from the host's in the last fp64 bit (then an
 * fp32 scalar may differ by one ulp, in about 1 of 10^9 steps). */
typedef struct zero_step_state {
  double loss_scale;      /* current dynamic loss scale */
  double global_norm;     /* unscaled global norm of the last decided step (NaN if skipped) */
  double grad_scale;      /* factor of the last decided step: coef / loss scale (0 if skipped) */
  int64_t adam_step;      /* Adam t of the last applied update */
  int64_t iteration;      /* steps decided so far, skipped or not */
  int32_t good_steps;     /* consecutive good steps since the last scale change */
  int32_t growth_interval;
  int32_t skip;           /* 1: the last decided step is skipped (the update kernels do nothing) */
  int32_t error;          /* 0, or ZERO_STEP_ERR_LOSS_SCALE for the last decided step */
  float scalars[12];      /* fp32 b1, 1-b1, b2, 1-b2, eps, 1-lr*wd, lr/(1-b1^t), sqrt(1-b2^t), gscale, 0, 0, 0 */
} zero_step_state;

/* The decision could not be taken: the loss scale is not a positive finite
 * number, or loss_scale² underflowed so that the unscaled square-norm of a
 * step without overflow is not finite (the cases zero_step_decision refuses
 * with ZERO_ERR_INVALID).  The step is skipped (skip = 1, grad_scale = 0,
 * global_norm = NaN); loss scale, good steps and Adam t are left as they
 * are.  The next decision sets error back to 0 if it can be taken. */
#define ZERO_STEP_ERR_LOSS_SCALE 1

/* Device.  Writes the initial state (loss scale, growth interval >= 1, t = 0,
 * error 0) with a one-thread kernel.  state_dev: 16-byte aligned. */
int zero_step_state_init(zero_step_state* state_dev, double loss_scale, int32_t growth_interval, void* stream);

/* Device.  rank_sqnorms_dev[n_ranks] (double) and rank_flags_dev[n_ranks]
 * (int32) as written by zero_grad_sqnorm / zero_flatten_grads_sqnorm; hp
 * supplies lr, beta1, beta2, eps and weight_decay (hp->step and
 * hp->grad_scale are ignored: t and the factor come from the state and the
 * decision).  Updates *state_dev as described above. */
int zero_step_decision_dev(const double* rank_sqnorms_dev, const int32_t* rank_flags_dev, int32_t n_ranks,
                           double max_norm, const zero_adamw_hparams* hp, zero_step_state* state_dev, void* stream);

/* Device.  zero_adamw_step / zero_adamw_step_tiled with the scalars taken
 * from the device state; when state_dev->skip is set the kernels return
 * without touching memory. */
int zero_adamw_step_dev(const void* grad_dev, zero_dtype gdt, float* master_dev, float* m_dev, float* v_dev,
                        uint16_t* param_dev, zero_dtype pdt, int64_t n, const zero_step_state* state_dev,
                        void* stream);
int zero_adamw_step_tiled_dev(const void* grad_dev, zero_dtype gdt, float* state_dev, uint16_t* param_dev,
                              zero_dtype pdt, int64_t n, const zero_step_state* step_state_dev, void* stream);

/* ------------------------------------------------------------------ measurement aid
 *
 * Not a step of the method: the read-modify-write ceiling of the tiled
 * update's own access pattern.  Device.  Exactly the loads and stores of
 * zero_adamw_step_tiled over n elements (same launches of at most 2^25
 * elements, same workgroup-to-tile mapping, same non-temporal hints: read 2 B
 * of gradient and 12 B of tiled state, write the 12 B of state back and 2 B
 * of parameter per element), with the arithmetic replaced by an XOR with key:
 * state words become state ^ key, each 32-bit pair of parameters becomes the
 * gradient pair ^ key.  With key = 0 the state keeps its bits and the
 * parameters receive the gradient bits.  Only whole groups of four elements
 * are touched (n mod 4 trailing elements are left alone).  Same alignment
 * rules as the vector path of zero_adamw_step_tiled (grad and param 8-byte,
 * state 16-byte aligned), otherwise ZERO_ERR_INVALID. */
int zero_calibrate_tiled_rmw(const void* grad_dev, float* state_dev, uint16_t* param_dev, int64_t n, uint32_t key,
                             void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_SHARD_H */
