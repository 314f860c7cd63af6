// Exercises every host-side path of libzero_shard (layout, bucket windows,
// flatten plans, the host decision and its helpers, size queries, and the
// argument checks of the device entry points, which return before any
// device work) so that a build with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code can see each access.  Checks
// only invariants that need no reference; the numerical comparisons with the
// oracle live in the Python tests.  Needs no GPU.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "zero_shard.h"

namespace {

uint64_t rng_state = 0x2545F4914F6CDD1Dull;
uint64_t next_u64() {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int64_t below(int64_t n) { return n > 0 ? static_cast<int64_t>(next_u64() % static_cast<uint64_t>(n)) : 0; }

#define CHECK(c)                                                                     \
  do {                                                                               \
    if (!(c)) {                                                                      \
      std::fprintf(stderr, "%s:%d: check failed: %s (%s)\n", __FILE__, __LINE__, #c, \
                   zero_last_error());                                               \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

void layout_windows_plans() {
  for (int trial = 0; trial < 3000; ++trial) {
    const int32_t nt = static_cast<int32_t>(below(9));
    std::vector<int64_t> numels(nt + 1);
    for (int32_t t = 0; t < nt; ++t) numels[t] = below(4) == 0 ? 0 : below(5000);
    const int32_t world = 1 + static_cast<int32_t>(below(12));
    const int32_t rank = static_cast<int32_t>(below(world));
    zero_layout lay;
    int32_t need = -1;
    const int rc = zero_shard_layout(numels.data(), nt, world, rank, &lay, nullptr, 0, &need);
    CHECK(rc == ZERO_OK || rc == ZERO_ERR_CAPACITY);
    std::vector<zero_segment> segs(need + 1);
    int32_t got = -1;
    if (need > 1) {  // capacity one short
      CHECK(zero_shard_layout(numels.data(), nt, world, rank, &lay, segs.data(), need - 1, &got) ==
            ZERO_ERR_CAPACITY);
      CHECK(got == need);
    }
    CHECK(zero_shard_layout(numels.data(), nt, world, rank, &lay, segs.data(), need, &got) == ZERO_OK);
    CHECK(got == need && lay.shard_numel * world == lay.padded_numel);
    // constant-capacity windows: every valid element once, offsets inside the window
    const int64_t cap = 8 * (1 + below(64));
    std::vector<int32_t> cover(lay.shard_numel + 1, 0);
    for (int64_t a = 0; a < lay.shard_numel; a += cap) {
      const int64_t len = std::min<int64_t>(cap, lay.shard_numel - a);
      int32_t cnt = -1;
      const int r0 = zero_bucket_segments(segs.data(), got, a, len, nullptr, 0, &cnt);
      CHECK(r0 == ZERO_OK || r0 == ZERO_ERR_CAPACITY);
      std::vector<zero_segment> w(cnt + 1);
      int32_t cnt2 = -1;
      CHECK(zero_bucket_segments(segs.data(), got, a, len, w.data(), cnt, &cnt2) == ZERO_OK && cnt2 == cnt);
      for (int32_t k = 0; k < cnt; ++k) {
        CHECK(w[k].dst_offset >= 0 && w[k].dst_offset + w[k].numel <= len && w[k].numel > 0);
        for (int64_t i = 0; i < w[k].numel; ++i) ++cover[a + w[k].dst_offset + i];
      }
    }
    for (int64_t j = 0; j < lay.shard_numel; ++j) CHECK(cover[j] == (j < lay.shard_valid ? 1 : 0));
    // descriptors from fake (never dereferenced) tensor addresses
    std::vector<const void*> ptrs(nt + 1);
    for (int32_t t = 0; t < nt; ++t) ptrs[t] = reinterpret_cast<const void*>(static_cast<uintptr_t>(0x1000 * (t + 1)));
    std::vector<zero_flat_seg> plan(got + 1);
    CHECK(zero_flatten_plan(segs.data(), got, ptrs.data(), nt, plan.data()) == ZERO_OK);
    for (int32_t k = 0; k < got; ++k) CHECK(plan[k].src == ptrs[segs[k].tensor]);
  }
  zero_layout lay;
  int32_t n = 0;
  const int64_t bad = -1, four = 4;
  CHECK(zero_shard_layout(&bad, 1, 2, 0, &lay, nullptr, 0, &n) == ZERO_ERR_INVALID);
  CHECK(zero_shard_layout(&four, 1, 0, 0, &lay, nullptr, 0, &n) == ZERO_ERR_INVALID);
  CHECK(zero_shard_layout(&four, 1, 2, 2, &lay, nullptr, 0, &n) == ZERO_ERR_INVALID);
  CHECK(zero_bucket_segments(nullptr, 0, -1, 4, nullptr, 0, &n) == ZERO_ERR_INVALID);
  CHECK(std::strlen(zero_last_error()) > 0);
}

void decisions_and_sizes() {
  for (int trial = 0; trial < 5000; ++trial) {
    const int32_t ranks = 1 + static_cast<int32_t>(below(6));
    double sq[6];
    int32_t fl[6];
    for (int32_t r = 0; r < ranks; ++r) {
      sq[r] = static_cast<double>(below(1000000)) * 1e-3;
      fl[r] = below(8) == 0;
    }
    double scale = std::ldexp(1.0, static_cast<int>(below(17))), gs = 0.0, norm = 0.0;
    int32_t good = static_cast<int32_t>(below(3)), skip = -1;
    CHECK(zero_step_decision(sq, fl, ranks, static_cast<double>(below(3)), &scale, &good,
                             1 + static_cast<int32_t>(below(3)), &gs, &skip, &norm) == ZERO_OK);
    CHECK(skip == 0 || skip == 1);
    CHECK(zero_clip_coef(sq[0], 1.0) <= 1.0);
    CHECK(std::isfinite(zero_cosine_lr(1 + below(10), 10, 1e-4, 1e-5)));
    double s2 = scale;
    int32_t g2 = 0;
    CHECK(zero_loss_scale_update(&s2, fl[0], &g2, 2) == ZERO_OK);
    const int64_t m = below(int64_t(1) << 40);
    CHECK(zero_state_tiled_numel(m) >= 3 * m);
    CHECK(zero_grad_sqnorm_workspace_bytes(m) >= 12u * static_cast<uint64_t>(zero_flatten_partials_count(m)));
  }
  CHECK(zero_grad_sqnorm_workspace_bytes(INT64_MAX) <= 12u * (1u << 19) + 256u);
  // loss scales down to the smallest subnormal: refused exactly when the scale is unusable or, without an
  // overflow, the unscaled square-norm is not finite; refused calls write nothing
  for (int trial = 0; trial < 5000; ++trial) {
    double sq = static_cast<double>(below(1000000)) * 1e-3;
    int32_t fl = below(4) == 0;
    double scale = std::ldexp(1.0, -static_cast<int>(below(1080)));
    if (below(50) == 0) scale = below(2) ? 0.0 : HUGE_VAL;
    const double scale0 = scale;
    double gs = -7.0, norm = -7.0;
    int32_t good = 5, skip = -7;
    const bool usable = std::isfinite(scale) && scale > 0.0 && (fl || std::isfinite(sq / (scale * scale)));
    const int rc = zero_step_decision(&sq, &fl, 1, 1.0, &scale, &good, 1000, &gs, &skip, &norm);
    CHECK(rc == (usable ? ZERO_OK : ZERO_ERR_INVALID));
    if (!usable) CHECK(scale == scale0 && good == 5 && skip == -7 && gs == -7.0 && norm == -7.0);
    if (usable && fl) CHECK(skip == 1 && scale == scale0 * 0.5 && good == 0);
    if (usable && !fl) CHECK(skip == 0 && std::isfinite(gs));
  }
}

void device_argument_checks() {
  zero_adamw_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1};
  alignas(16) static float f[16];
  alignas(16) static uint16_t h[16];
  CHECK(zero_adamw_step(nullptr, ZERO_BF16, f, f, f, h, ZERO_BF16, 8, &hp, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_adamw_step(h, static_cast<zero_dtype>(7), f, f, f, h, ZERO_BF16, 8, &hp, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_adamw_step(h, ZERO_BF16, f, f, f, h, static_cast<zero_dtype>(2), 8, &hp, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_adamw_step(h, ZERO_BF16, f, f, f, h, ZERO_BF16, -1, &hp, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_adamw_step(nullptr, ZERO_BF16, nullptr, nullptr, nullptr, nullptr, ZERO_BF16, 0, &hp, nullptr) ==
        ZERO_OK);
  hp.step = 0;
  CHECK(zero_adamw_step_tiled(h, ZERO_BF16, f, h, ZERO_BF16, 8, &hp, nullptr) == ZERO_ERR_INVALID);
  hp.step = 1;
  CHECK(zero_adamw_step_tiled(h, ZERO_BF16, f + 1, h, ZERO_BF16, 8, &hp, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_adamw_step_dev(h, ZERO_BF16, f, f, f, h, ZERO_BF16, 8, nullptr, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_adamw_step_tiled_dev(h, ZERO_BF16, f, h, ZERO_BF16, 8, nullptr, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_flatten_grads(nullptr, 1, ZERO_BF16, h, 8, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_flatten_grads(nullptr, 0, ZERO_BF16, nullptr, 0, nullptr) == ZERO_OK);
  CHECK(zero_flatten_grads_sqnorm(nullptr, 0, ZERO_BF16, h, 8, nullptr, 0, nullptr, nullptr, nullptr) ==
        ZERO_ERR_INVALID);
  CHECK(zero_flatten_grads_partials(nullptr, 0, ZERO_BF16, h, 8, nullptr, nullptr, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_sqnorm_reduce(nullptr, nullptr, 4, nullptr, nullptr, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_grad_sqnorm(h, ZERO_BF16, 8, nullptr, 0, nullptr, nullptr, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_step_state_init(nullptr, 1.0, 1, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_step_decision_dev(nullptr, nullptr, 1, 1.0, &hp, nullptr, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_state_tile(nullptr, nullptr, nullptr, nullptr, 8, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_state_untile(nullptr, nullptr, nullptr, nullptr, -1, nullptr) == ZERO_ERR_INVALID);
  alignas(16) static double d2[2];
  CHECK(zero_flatten_grads_sqnorm_noalloc(nullptr, 1, ZERO_BF16, h, 8, d2, reinterpret_cast<int32_t*>(d2 + 1),
                                          nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_flatten_grads_sqnorm_noalloc(nullptr, 0, ZERO_BF16, h, 8, nullptr, nullptr, nullptr) ==
        ZERO_ERR_INVALID);
  CHECK(zero_flatten_grads_sqnorm_noalloc(nullptr, 0, static_cast<zero_dtype>(9), h, 8, d2,
                                          reinterpret_cast<int32_t*>(d2 + 1), nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_flatten_grads_sqnorm_noalloc(nullptr, 0, ZERO_BF16, h, 8, reinterpret_cast<double*>(h + 1),
                                          reinterpret_cast<int32_t*>(d2 + 1), nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_calibrate_tiled_rmw(h, f, h, -1, 0u, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_calibrate_tiled_rmw(h, f + 1, h, 8, 0u, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_calibrate_tiled_rmw(nullptr, f, h, 8, 0u, nullptr) == ZERO_ERR_INVALID);
  CHECK(zero_calibrate_tiled_rmw(nullptr, nullptr, nullptr, 0, 0u, nullptr) == ZERO_OK);
}

}  // namespace

int main() {
  layout_windows_plans();
  decisions_and_sizes();
  device_argument_checks();
  std::puts("library host checks ok");
  return 0;
}
