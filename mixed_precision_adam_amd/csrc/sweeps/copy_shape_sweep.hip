// copy_shape_sweep.hip -- measurement program (not part of the library): a bare contiguous 16-bit copy between
// two buffers of the Llama-13B rank shard's size (6.5 GB each), in one process, over the shapes the flatten's
// body can take: U 16-byte vectors in flight per thread, at most W wavefronts per SIMD, elements per 256-thread
// workgroup, non-temporal or ordinary stores.  Timed with HIP events (10 copies after a warm-up, three
// interleaved rounds); rates count read plus written bytes.
//
// Build and run (repository root, one MI355X):
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     -o /tmp/copy_shape_sweep mixed_precision_adam_amd/csrc/sweeps/copy_shape_sweep.hip && /tmp/copy_shape_sweep
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <algorithm>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define HIPCHK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP %s at %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)
typedef const u32x4 __attribute__((address_space(1)))* gptr;

template <int U, int W, bool NTS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, W)))
void copyk(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t nv, int64_t per_v) {
  const int64_t lo = (int64_t)blockIdx.x * per_v;
  const int64_t hi = lo + per_v < nv ? lo + per_v : nv;
  const gptr s = (gptr)src;
  int64_t j = lo + threadIdx.x;
  for (; j + (U - 1) * 256 < hi; j += U * 256) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = __builtin_nontemporal_load(s + j + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (NTS) __builtin_nontemporal_store(w[u], dst + j + u * 256); else dst[j + u * 256] = w[u];
    }
  }
  for (; j < hi; j += 256) {
    const u32x4 w = __builtin_nontemporal_load(s + j);
    if constexpr (NTS) __builtin_nontemporal_store(w, dst + j); else dst[j] = w;
  }
}
int main() {
  const int64_t n = 3253966080, nv = n / 8;  // 16-bit elements, 16-byte vectors
  u32x4 *a, *b;
  HIPCHK(hipMalloc(&a, n * 2)); HIPCHK(hipMalloc(&b, n * 2));
  HIPCHK(hipMemset(a, 1, n * 2));
  hipEvent_t e0, e1; HIPCHK(hipEventCreate(&e0)); HIPCHK(hipEventCreate(&e1));
  struct C { const char* name; int kind; int64_t per; };
  C cs[] = {{"U4 W4 8192 (flatten)", 0, 8192}, {"U2 W4 4096", 1, 4096}, {"U1 W4 2048", 9, 2048}, {"U4 W4 4096", 0, 4096},
            {"U2 W2 4096", 10, 4096}, {"U2 W3 4096", 11, 4096}, {"U4 W2 8192", 3, 8192}, {"U4 W3 8192", 4, 8192},
            {"U2 W4 4096 nt-store", 12, 4096}, {"U4 W4 8192 nt-store", 7, 8192}, {"U8 W4 16384", 2, 16384},
            {"U1 W8 2048", 13, 2048}};
  auto launch = [&](int kind, int64_t per) {
    const int64_t per_v = per / 8, blocks = (nv + per_v - 1) / per_v;
    const dim3 g((unsigned)blocks), t(256);
    switch (kind) {
      case 0: hipLaunchKernelGGL((copyk<4, 4, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 1: hipLaunchKernelGGL((copyk<2, 4, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 2: hipLaunchKernelGGL((copyk<8, 4, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 3: hipLaunchKernelGGL((copyk<4, 2, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 4: hipLaunchKernelGGL((copyk<4, 3, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 5: hipLaunchKernelGGL((copyk<4, 8, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 6: hipLaunchKernelGGL((copyk<8, 2, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 7: hipLaunchKernelGGL((copyk<4, 4, true>), g, t, 0, 0, a, b, nv, per_v); break;
      case 9: hipLaunchKernelGGL((copyk<1, 4, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 10: hipLaunchKernelGGL((copyk<2, 2, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 11: hipLaunchKernelGGL((copyk<2, 3, false>), g, t, 0, 0, a, b, nv, per_v); break;
      case 12: hipLaunchKernelGGL((copyk<2, 4, true>), g, t, 0, 0, a, b, nv, per_v); break;
      case 13: hipLaunchKernelGGL((copyk<1, 8, false>), g, t, 0, 0, a, b, nv, per_v); break;
      default: hipLaunchKernelGGL((copyk<2, 8, false>), g, t, 0, 0, a, b, nv, per_v); break;
    }
  };
  for (int round = 0; round < 3; ++round)
    for (const C& c : cs) {
      launch(c.kind, c.per);
      HIPCHK(hipEventRecord(e0, 0));
      for (int r = 0; r < 10; ++r) launch(c.kind, c.per);
      HIPCHK(hipEventRecord(e1, 0));
      HIPCHK(hipEventSynchronize(e1));
      float ms = 0;
      HIPCHK(hipEventElapsedTime(&ms, e0, e1));
      ms /= 10;
      printf("round %d %-22s %.4f ms  %.1f GB/s\n", round, c.name, ms, 4.0 * n / (ms * 1e-3) / 1e9);
      fflush(stdout);
    }
  HIPCHK(hipGetLastError());
  return 0;
}
