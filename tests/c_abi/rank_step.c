/*
 * One data-parallel rank's ZeRO step driven through the C ABI from plain C:
 * device memory from hipMalloc, no PyTorch in the process.  Tensors of
 * ragged sizes (pieces out of phase with the shard's 16-byte lines), fp16
 * gradients under a dynamic loss scale, tiled optimizer state, two steps:
 * the first decided on the host after a 16-byte readback, the second on the
 * device.  Every result is compared with the CPU oracle (test
 * infrastructure, linked here only as the checker): layout and flattened
 * shard bit for bit, square-norm within the fp64 summation bound, decision
 * exactly, and master / m / v / parameters bit for bit given the factor the
 * library decided (several fp64 summation orders give correct factors; the
 * update given a factor is unique).  Inputs come from the seeded generator.
 * Exit status 0 when everything agrees.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "oracle.h"
#include "synth_core.h"
#include "zero_shard.h"

int syn_fill_host(const syn_field* f, int64_t idx0, int64_t n, void* out, int32_t threads);

#define NT 5
#define WORLD 3
#define RANK 2

static int failures = 0;
#define EXPECT(c, ...)                                     \
  do {                                                     \
    if (!(c)) {                                            \
      fprintf(stderr, "%s:%d: ", __FILE__, __LINE__);      \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
      ++failures;                                          \
    }                                                      \
  } while (0)
#define HIP_OK(x)                                                                  \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(2);                                                                     \
    }                                                                              \
  } while (0)
#define ZERO_OK_(x)                                                                \
  do {                                                                             \
    int s_ = (x);                                                                  \
    if (s_ != ZERO_OK) {                                                           \
      fprintf(stderr, "%s:%d: %s -> %d: %s\n", __FILE__, __LINE__, #x, s_, zero_last_error()); \
      exit(3);                                                                     \
    }                                                                              \
  } while (0)

static int bits_equal(const void* a, const void* b, size_t bytes) { return memcmp(a, b, bytes) == 0; }

int main(void) {
  const int64_t numels[NT] = {1000, 7, 40097, 20000, 4};  /* psi = 61108: two padding elements in rank 2 */
  int64_t starts[NT + 1] = {0};
  for (int t = 0; t < NT; ++t) starts[t + 1] = starts[t] + numels[t];
  const int64_t psi = starts[NT];

  /* a1: layout, against the oracle's */
  zero_layout lay;
  zero_segment segs[NT];
  int32_t n_segs = 0;
  ZERO_OK_(zero_shard_layout(numels, NT, WORLD, RANK, &lay, segs, NT, &n_segs));
  orc_layout olay;
  orc_segment osegs[NT];
  int32_t on_segs = 0;
  EXPECT(orc_layout_compute(numels, NT, WORLD, RANK, &olay, osegs, NT, &on_segs) == ORC_OK, "oracle layout");
  EXPECT(lay.psi == olay.psi && lay.shard_numel == olay.shard_numel && lay.shard_offset == olay.shard_offset &&
             lay.shard_valid == olay.shard_valid && lay.bytes_zero1 == olay.bytes_zero1 &&
             lay.bytes_zero3 == olay.bytes_zero3 && n_segs == on_segs,
         "layout differs from the oracle's");
  const int64_t S = lay.shard_numel;

  /* device buffers: per-tensor fp16 gradients, the shard, tiled state, params, workspace, results */
  void* src_dev[NT];
  uint16_t* src_host[NT];
  for (int t = 0; t < NT; ++t) {
    HIP_OK(hipMalloc(&src_dev[t], (size_t)numels[t] * 2));
    src_host[t] = (uint16_t*)malloc((size_t)numels[t] * 2);
  }
  void *shard, *state, *param, *ws, *table, *norm, *step_state;
  const int64_t state_numel = zero_state_tiled_numel(S);
  const size_t ws_bytes = zero_grad_sqnorm_workspace_bytes(S);
  HIP_OK(hipMalloc(&shard, (size_t)S * 2));
  HIP_OK(hipMalloc(&state, (size_t)state_numel * 4));
  HIP_OK(hipMalloc(&param, (size_t)S * 2));
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMalloc(&table, sizeof(zero_flat_seg) * NT));
  HIP_OK(hipMalloc(&norm, 16));       /* fp64 square-norm, then the int32 flag */
  HIP_OK(hipMalloc(&step_state, 128));

  const void* ptrs[NT];
  for (int t = 0; t < NT; ++t) ptrs[t] = src_dev[t];
  zero_flat_seg plan[NT];
  ZERO_OK_(zero_flatten_plan(segs, n_segs, ptrs, NT, plan));
  HIP_OK(hipMemcpy(table, plan, sizeof(zero_flat_seg) * (size_t)n_segs, hipMemcpyHostToDevice));

  /* initial state: master ~ N(0, 0.02) over the shard's flat elements, m = v = 0, tiled on the device */
  float* master = (float*)calloc((size_t)S, 4);
  float* m = (float*)calloc((size_t)S, 4);
  float* v = (float*)calloc((size_t)S, 4);
  uint16_t* q = (uint16_t*)calloc((size_t)S, 2);
  const syn_field mf = {0x5EED0C01ull, 2, 0, 0.02, 1.0, 0, SYN_F32, 0.0};
  syn_fill_host(&mf, lay.shard_offset, lay.shard_valid, master, 1);
  void *dm, *dz;
  HIP_OK(hipMalloc(&dm, (size_t)S * 4));
  HIP_OK(hipMalloc(&dz, (size_t)S * 4));
  HIP_OK(hipMemcpy(dm, master, (size_t)S * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(dz, 0, (size_t)S * 4));
  ZERO_OK_(zero_state_tile((const float*)dm, (const float*)dz, (const float*)dz, (float*)state, S, NULL));

  const double lr = 1e-3, b1 = 0.9, b2 = 0.999, eps = 1e-8, wd = 0.01, max_norm = 0.1;  /* clips */
  double scale = 1024.0, oscale = 1024.0;
  int32_t good = 0, ogood = 0;
  const int32_t growth = 1000;
  uint16_t* g_host = (uint16_t*)malloc((size_t)S * 2);
  uint16_t* got16 = (uint16_t*)malloc((size_t)S * 2);
  float* got = (float*)malloc((size_t)S * 4 * 3);

  for (int step = 1; step <= 2; ++step) {
    const syn_field gf = {0x5EED0C01ull, 1, (uint32_t)step, 1e-3, scale, 0, SYN_FP16, 0.0};
    for (int t = 0; t < NT; ++t) {
      syn_fill_host(&gf, starts[t], numels[t], src_host[t], 1);
      HIP_OK(hipMemcpy(src_dev[t], src_host[t], (size_t)numels[t] * 2, hipMemcpyHostToDevice));
    }
    /* a2 + a3 */
    ZERO_OK_(zero_flatten_grads_sqnorm((const zero_flat_seg*)table, n_segs, ZERO_FP16, shard, S, ws, ws_bytes,
                                       (double*)norm, (int32_t*)((char*)norm + 8), NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got16, shard, (size_t)S * 2, hipMemcpyDeviceToHost));
    EXPECT(orc_flatten((const uint16_t* const*)src_host, numels, NT, WORLD, RANK, g_host) == ORC_OK, "flatten");
    EXPECT(bits_equal(got16, g_host, (size_t)S * 2), "step %d: flattened shard differs", step);
    unsigned char nb[16];
    HIP_OK(hipMemcpy(nb, norm, 16, hipMemcpyDeviceToHost));
    double sq;
    int32_t flag;
    memcpy(&sq, nb, 8);
    memcpy(&flag, nb + 8, 4);
    double osq;
    int32_t oflag;
    EXPECT(orc_sqnorm(g_host, ORC_FP16, S, &osq, &oflag) == ORC_OK, "sqnorm");
    EXPECT(flag == oflag && flag == 0, "step %d: flag %d, oracle %d", step, flag, oflag);
    EXPECT(fabs(sq - osq) <= 2.0 * (double)S * ldexp(1.0, -53) * osq, "step %d: square-norm %.17g vs %.17g", step,
           sq, osq);

    /* a4: the oracle's own decision, then the library's (host at step 1, device at step 2) */
    double ogs, ogn;
    int32_t oskip;
    EXPECT(orc_step_decision(&osq, &oflag, 1, max_norm, &oscale, &ogood, growth, &ogs, &oskip, &ogn) == ORC_OK,
           "oracle decision");
    double gs;
    int32_t skip;
    int64_t t_adam = step;
    if (step == 1) {
      double gn;
      ZERO_OK_(zero_step_decision(&sq, &flag, 1, max_norm, &scale, &good, growth, &gs, &skip, &gn));
      zero_adamw_hparams hp = {lr, b1, b2, eps, wd, gs, t_adam};
      ZERO_OK_(zero_adamw_step_tiled(shard, ZERO_FP16, (float*)state, (uint16_t*)param, ZERO_BF16, S, &hp, NULL));
      ZERO_OK_(zero_step_state_init((zero_step_state*)step_state, scale, growth, NULL));
    } else {
      /* the device state carries Adam t = 0 from its init; t = 1 was taken on the host, so set it */
      zero_step_state st;
      HIP_OK(hipDeviceSynchronize());
      HIP_OK(hipMemcpy(&st, step_state, sizeof st, hipMemcpyDeviceToHost));
      st.adam_step = 1;
      st.good_steps = good;
      HIP_OK(hipMemcpy(step_state, &st, sizeof st, hipMemcpyHostToDevice));
      zero_adamw_hparams hp = {lr, b1, b2, eps, wd, 1.0, 1};
      ZERO_OK_(zero_step_decision_dev((const double*)norm, (const int32_t*)((char*)norm + 8), 1, max_norm, &hp,
                                      (zero_step_state*)step_state, NULL));
      ZERO_OK_(zero_adamw_step_tiled_dev(shard, ZERO_FP16, (float*)state, (uint16_t*)param, ZERO_BF16, S,
                                         (const zero_step_state*)step_state, NULL));
      HIP_OK(hipDeviceSynchronize());
      HIP_OK(hipMemcpy(&st, step_state, sizeof st, hipMemcpyDeviceToHost));
      gs = st.grad_scale;
      skip = st.skip;
      scale = st.loss_scale;
      EXPECT(st.adam_step == 2 && st.error == 0, "step 2: device state t=%lld error=%d", (long long)st.adam_step,
             st.error);
    }
    EXPECT(skip == oskip && skip == 0 && scale == oscale, "step %d: decision differs (skip %d, scale %g vs %g)",
           step, skip, scale, oscale);
    EXPECT(fabs(gs - ogs) <= 2.0 * (double)S * ldexp(1.0, -53) * ogs, "step %d: factor %.17g vs %.17g", step, gs,
           ogs);

    /* a5: the oracle applies the library's factor; the state must match bit for bit */
    orc_hparams ohp = {lr, b1, b2, eps, wd, gs, t_adam};
    EXPECT(orc_adamw_step(g_host, ORC_FP16, master, m, v, q, ORC_BF16, S, &ohp) == ORC_OK, "oracle update");
    HIP_OK(hipDeviceSynchronize());
    void *gm, *gmm, *gv;
    HIP_OK(hipMalloc(&gm, (size_t)S * 4));
    HIP_OK(hipMalloc(&gmm, (size_t)S * 4));
    HIP_OK(hipMalloc(&gv, (size_t)S * 4));
    ZERO_OK_(zero_state_untile((const float*)state, (float*)gm, (float*)gmm, (float*)gv, S, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got, gm, (size_t)S * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(got + S, gmm, (size_t)S * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(got + 2 * S, gv, (size_t)S * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(got16, param, (size_t)S * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipFree(gm));
    HIP_OK(hipFree(gmm));
    HIP_OK(hipFree(gv));
    EXPECT(bits_equal(got, master, (size_t)S * 4), "step %d: master differs", step);
    EXPECT(bits_equal(got + S, m, (size_t)S * 4), "step %d: m differs", step);
    EXPECT(bits_equal(got + 2 * S, v, (size_t)S * 4), "step %d: v differs", step);
    EXPECT(bits_equal(got16, q, (size_t)S * 2), "step %d: params differ", step);
  }

  for (int t = 0; t < NT; ++t) {
    HIP_OK(hipFree(src_dev[t]));
    free(src_host[t]);
  }
  HIP_OK(hipFree(shard));
  HIP_OK(hipFree(state));
  HIP_OK(hipFree(param));
  HIP_OK(hipFree(ws));
  HIP_OK(hipFree(table));
  HIP_OK(hipFree(norm));
  HIP_OK(hipFree(step_state));
  HIP_OK(hipFree(dm));
  HIP_OK(hipFree(dz));
  free(master);
  free(m);
  free(v);
  free(q);
  free(g_host);
  free(got16);
  free(got);
  printf("rank step through the C ABI: psi=%lld S=%lld pieces=%d, %s\n", (long long)psi, (long long)S, n_segs,
         failures ? "FAILED" : "all equal to the oracle");
  return failures ? 1 : 0;
}
