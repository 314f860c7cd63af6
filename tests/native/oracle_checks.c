/* Exercises every oracle entry point on small random and degenerate inputs so
 * that an AddressSanitizer / UndefinedBehaviorSanitizer build of the oracle
 * can see each memory access and integer operation.  Checks only invariants
 * that need no reference (coverage, bit copies, range of results); the
 * numerical pins live in the Python tests. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static int64_t below(int64_t n) { return n > 0 ? (int64_t)(next_u64() % (uint64_t)n) : 0; }

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      exit(1);                                                     \
    }                                                              \
  } while (0)

static void layout_and_flatten(void) {
  for (int trial = 0; trial < 3000; ++trial) {
    int32_t nt = (int32_t)below(7);
    int64_t numels[8];
    int64_t psi = 0;
    for (int32_t t = 0; t < nt; ++t) {
      numels[t] = below(5) == 0 ? 0 : below(200);
      psi += numels[t];
    }
    int32_t world = 1 + (int32_t)below(9);
    int32_t rank = (int32_t)below(world);
    orc_layout lay;
    int32_t need = -1;
    int rc = orc_layout_compute(numels, nt, world, rank, &lay, NULL, 0, &need);
    CHECK(rc == ORC_OK || rc == ORC_ERR_CAPACITY);
    orc_segment* segs = (orc_segment*)malloc(sizeof(orc_segment) * (size_t)(need > 0 ? need : 1));
    int32_t got = -1;
    CHECK(orc_layout_compute(numels, nt, world, rank, &lay, segs, need, &got) == ORC_OK && got == need);
    CHECK(lay.psi == psi && lay.shard_numel * world == lay.padded_numel);
    uint16_t* tensors[8];
    for (int32_t t = 0; t < nt; ++t) {
      tensors[t] = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(numels[t] > 0 ? numels[t] : 1));
      for (int64_t i = 0; i < numels[t]; ++i) tensors[t][i] = (uint16_t)next_u64();
    }
    uint16_t* shard = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(lay.shard_numel > 0 ? lay.shard_numel : 1));
    CHECK(orc_flatten((const uint16_t* const*)tensors, numels, nt, world, rank, shard) == ORC_OK);
    for (int32_t k = 0; k < got; ++k)
      CHECK(memcmp(shard + segs[k].dst_offset, tensors[segs[k].tensor] + segs[k].src_offset,
                   sizeof(uint16_t) * (size_t)segs[k].numel) == 0);
    for (int64_t j = lay.shard_valid; j < lay.shard_numel; ++j) CHECK(shard[j] == 0);
    double sq = -1.0;
    int32_t bad = -1;
    CHECK(orc_sqnorm(shard, (int32_t)below(2), lay.shard_numel, &sq, &bad) == ORC_OK && (bad == 0 || bad == 1));
    for (int32_t t = 0; t < nt; ++t) free(tensors[t]);
    free(shard);
    free(segs);
  }
  orc_layout lay;
  int32_t n = 0;
  int64_t bad_numel = -1;
  CHECK(orc_layout_compute(&bad_numel, 1, 2, 0, &lay, NULL, 0, &n) != ORC_OK);
  int64_t one = 4;
  CHECK(orc_layout_compute(&one, 1, 0, 0, &lay, NULL, 0, &n) != ORC_OK);
  CHECK(orc_layout_compute(&one, 1, 2, 2, &lay, NULL, 0, &n) != ORC_OK);
}

static void decision_and_update(void) {
  for (int trial = 0; trial < 2000; ++trial) {
    int32_t ranks = 1 + (int32_t)below(5);
    double sq[5];
    int32_t fl[5];
    for (int32_t r = 0; r < ranks; ++r) {
      sq[r] = (double)below(1000000) * 1e-3;
      fl[r] = below(10) == 0;
    }
    double scale = ldexp(1.0, (int)below(17)), gs = 0.0, norm = 0.0;
    int32_t good = (int32_t)below(3), skip = -1;
    CHECK(orc_step_decision(sq, fl, ranks, (double)below(3), &scale, &good, 1 + (int32_t)below(3), &gs, &skip,
                            &norm) == ORC_OK);
    CHECK(skip == 0 || skip == 1);
    CHECK(isfinite(orc_cosine_lr(1 + below(10), 10, 1e-4, 1e-5)));
    CHECK(orc_clip_coef(sq[0], 1.0) <= 1.0);
    int64_t n = below(70);
    uint16_t* g = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n + 1));
    uint16_t* q = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n + 1));
    float* p = (float*)malloc(sizeof(float) * (size_t)(n + 1));
    float* m = (float*)calloc((size_t)(n + 1), sizeof(float));
    float* v = (float*)calloc((size_t)(n + 1), sizeof(float));
    double* gd = (double*)malloc(sizeof(double) * (size_t)(n + 1));
    double* pd = (double*)malloc(sizeof(double) * (size_t)(n + 1));
    double* md = (double*)calloc((size_t)(n + 1), sizeof(double));
    double* vd = (double*)calloc((size_t)(n + 1), sizeof(double));
    for (int64_t i = 0; i < n; ++i) {
      g[i] = (uint16_t)next_u64();
      p[i] = (float)((double)below(2000) * 1e-3 - 1.0);
      gd[i] = (double)orc_bf16_to_f32(g[i]);
      pd[i] = p[i];
    }
    orc_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, 0.5, 1 + below(5)};
    CHECK(orc_adamw_step(g, (int32_t)below(2), p, m, v, q, (int32_t)below(2), n, &hp) == ORC_OK);
    CHECK(orc_adamw_step_f64(gd, pd, md, vd, n, &hp) == ORC_OK);
    orc_f32_to_bf16_array(p, q, n);
    orc_f32_to_f16_array(p, q, n);
    orc_decode_array(g, 1, p, n);
    free(g), free(q), free(p), free(m), free(v), free(gd), free(pd), free(md), free(vd);
  }
  orc_hparams bad = {1e-3, 1.0, 0.999, 1e-8, 0.01, 1.0, 1};
  orc_scalars s;
  CHECK(orc_adamw_scalars(&bad, &s) != ORC_OK);
  for (uint32_t h = 0; h < 65536; ++h) {
    (void)orc_bf16_to_f32((uint16_t)h);
    (void)orc_f16_to_f32((uint16_t)h);
  }
  for (int i = 0; i < 100000; ++i) {
    uint32_t u = (uint32_t)next_u64();
    float f;
    memcpy(&f, &u, sizeof f);
    (void)orc_f32_to_bf16(f);
    (void)orc_f32_to_f16(f);
  }
}

int main(void) {
  layout_and_flatten();
  decision_and_update();
  puts("oracle checks ok");
  return 0;
}
