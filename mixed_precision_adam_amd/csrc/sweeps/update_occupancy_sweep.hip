// update_occupancy_sweep.hip -- measurement program (not part of the library): the library's own tiled
// AdamW update (its source is included, so the same device code runs) instantiated under different
// occupancy caps, compared in one process at the Llama-13B rank shard's size (fp16 gradients, bf16
// parameters, host scalars).  Timed with HIP events, 8 calls per configuration after one warm-up call,
// three interleaved rounds.
//
// Build and run (repository root, one MI355X):
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -ffp-contract=off -fhip-fp32-correctly-rounded-divide-sqrt \
//     -fno-gpu-flush-denormals-to-zero -Xclang -target-feature -Xclang -packed-fp32-ops -I include \
//     -o /tmp/update_occupancy_sweep mixed_precision_adam_amd/csrc/sweeps/update_occupancy_sweep.hip && \
//     /tmp/update_occupancy_sweep
#include "../zero_shard.hip"

template <int W>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, W)))
void upd(const uint16_t* __restrict__ g, f32x4* __restrict__ state, uint16_t* __restrict__ q, int64_t n,
         int64_t tile0, AdamScalars s) {
  tiled_tile<ZERO_FP16, ZERO_BF16, false>(g, state, q, n, tile0, s, nullptr, 0u);
}
template <int W>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, W)))
void rmw(const uint16_t* __restrict__ g, f32x4* __restrict__ state, uint16_t* __restrict__ q, int64_t n,
         int64_t tile0, uint32_t key) {  // key at run time: a literal 0 would let the compiler drop the stores
  tiled_tile<ZERO_BF16, ZERO_BF16, true>(g, state, q, n, tile0, AdamScalars{}, nullptr, key);
}
__global__ void fill16(uint16_t* g, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    g[i] = (uint16_t)(0x3C00u | ((uint32_t)(i * 2654435761u) >> 22));  // fp16 values in [1, 2)
}
#define HIPCHK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP %s at %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)

int main() {
  const int64_t n = 3253966080;  // the Llama-13B rank shard
  const int64_t tiles = (n + 1023) / 1024;
  uint16_t *g, *q; f32x4* s;
  HIPCHK(hipMalloc(&g, n * 2)); HIPCHK(hipMalloc(&q, n * 2)); HIPCHK(hipMalloc(&s, tiles * 1024 * 12));
  HIPCHK(hipMemset(s, 0, tiles * 1024 * 12));
  hipLaunchKernelGGL(fill16, dim3(65536), dim3(256), 0, 0, g, n);
  HIPCHK(hipDeviceSynchronize());
  zero_adamw_hparams hp = {1e-4, 0.9, 0.999, 1e-8, 0.01, 1.0 / 65536 / 57.0, 1};
  AdamScalars sc;
  if (adam_args_ok("probe", g, ZERO_FP16, q, ZERO_BF16, n, &hp, &sc) != ZERO_OK) { printf("args\n"); return 1; }
  hipEvent_t a, b; HIPCHK(hipEventCreate(&a)); HIPCHK(hipEventCreate(&b));
  const int64_t tpl = kUpdateElemsPerLaunch / kTile;
  auto once = [&](int kind) {
    for (int64_t t0 = 0; t0 < tiles; t0 += tpl) {
      const dim3 grid((unsigned)std::min(tpl, tiles - t0));
      switch (kind) {
        case 0: hipLaunchKernelGGL((adamw_tiled_kernel<ZERO_FP16, ZERO_BF16>), grid, dim3(kBlock), 0, 0, g, s, q, n, t0, sc, nullptr); break;
        case 1: hipLaunchKernelGGL(upd<2>, grid, dim3(kBlock), 0, 0, g, s, q, n, t0, sc); break;
        case 2: hipLaunchKernelGGL(upd<3>, grid, dim3(kBlock), 0, 0, g, s, q, n, t0, sc); break;
        case 3: hipLaunchKernelGGL(upd<4>, grid, dim3(kBlock), 0, 0, g, s, q, n, t0, sc); break;
        case 4: hipLaunchKernelGGL(upd<5>, grid, dim3(kBlock), 0, 0, g, s, q, n, t0, sc); break;
        case 5: hipLaunchKernelGGL(rmw<2>, grid, dim3(kBlock), 0, 0, g, s, q, n, t0, 0u); break;
        default: hipLaunchKernelGGL(rmw<4>, grid, dim3(kBlock), 0, 0, g, s, q, n, t0, 0u); break;
      }
    }
  };
  const char* names[] = {"library update", "update w2", "update w3", "update w4", "update w5", "no-arith w2", "no-arith w4"};
  for (int round = 0; round < 3; ++round)
    for (int k = 0; k < 7; ++k) {
      once(k);
      HIPCHK(hipEventRecord(a, 0));
      for (int r = 0; r < 8; ++r) once(k);
      HIPCHK(hipEventRecord(b, 0));
      HIPCHK(hipEventSynchronize(b));
      float ms = 0;
      HIPCHK(hipEventElapsedTime(&ms, a, b));
      ms /= 8;
      printf("round %d %-15s %.4f ms  %.1f GB/s\n", round, names[k], ms, 28.0 * n / (ms * 1e-3) / 1e9);
      fflush(stdout);
    }
  HIPCHK(hipGetLastError());
  return 0;
}
