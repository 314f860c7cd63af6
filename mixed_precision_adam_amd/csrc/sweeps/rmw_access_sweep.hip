// rmw_access_sweep.hip -- measurement program (not part of the library): the read-modify-write traffic of
// the tiled AdamW update without its arithmetic, in one process on buffers of the Llama-13B rank shard's size
// (52 GB), for several access patterns and launch parameters.  Every kernel moves exactly 28 bytes per
// element: reads 2 B of gradient and 12 B of optimizer state, writes the 12 B of state (XOR a run-time key,
// 0, so the compiler cannot drop the stores) and 2 B of parameter.  Timed with HIP events, 8 passes per
// configuration after one warm-up pass, three interleaved rounds.
//
// Build and run (repository root, one MI355X):
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     -o /tmp/rmw_access_sweep mixed_precision_adam_amd/csrc/sweeps/rmw_access_sweep.hip && /tmp/rmw_access_sweep
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <algorithm>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define HIPCHK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP %s at %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)

template <bool NT, typename T> __device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p); else return *p;
}
template <bool NT, typename T> __device__ __forceinline__ void st(T* p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p); else *p = v;
}
__device__ __forceinline__ int64_t grp(int64_t b, int64_t n, int64_t G) {
  if (G <= 1) return b;
  const int64_t span = 8 * G;
  if (b >= n / span * span) return b;
  const int64_t x = b % 8, q = b / 8;
  return q / G * span + x * G + q % G;
}
// Layout variants moving the same bytes.  Sub-tiles of 256 elements: [master 256][m 256][v 256] four times
// per 1024 elements; wavefront w takes sub-tile w (3 KB contiguous).
template <int W = 4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, W)))
void lay_subtile256(const uint16_t* g16, u32x4* state, uint16_t* q16, int64_t tile0, uint32_t key, int64_t G) {
  const int64_t tile = tile0 + grp(blockIdx.x, gridDim.x, G);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  u32x4* b = state + tile * 768 + w * 192;
  const int64_t e = tile * 1024 + 4 * threadIdx.x;
  u32x2 g = ld<true>(reinterpret_cast<const u32x2*>(g16 + e));
  u32x4 p = ld<true>(b + l), m = ld<true>(b + 64 + l), v = ld<true>(b + 128 + l);
  const u32x4 k4 = {key, key, key, key};
  st<true>(b + l, p ^ k4); st<true>(b + 64 + l, m ^ k4); st<true>(b + 128 + l, v ^ k4);
  st<true>(reinterpret_cast<u32x2*>(q16 + e), g ^ u32x2{key, key});
}
// 8 elements per thread: 2048-element tiles ([master 2048][m 2048][v 2048]), 16-byte gradient and parameter
// vectors, two 16-byte state vectors per array and thread.
template <int W = 4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, W)))
void lay_8_per_thread(const uint16_t* g16, u32x4* state, uint16_t* q16, int64_t tile0, uint32_t key, int64_t G) {
  const int64_t tile = tile0 + grp(blockIdx.x, gridDim.x, G);
  u32x4* b = state + tile * 1536;
  const int j = threadIdx.x;
  const int64_t e = tile * 2048 + 8 * j;
  u32x4 g = ld<true>(reinterpret_cast<const u32x4*>(g16 + e));
  u32x4 p0 = ld<true>(b + 2 * j), p1 = ld<true>(b + 2 * j + 1), m0 = ld<true>(b + 512 + 2 * j), m1 = ld<true>(b + 512 + 2 * j + 1);
  u32x4 v0 = ld<true>(b + 1024 + 2 * j), v1 = ld<true>(b + 1024 + 2 * j + 1);
  const u32x4 k4 = {key, key, key, key};
  st<true>(b + 2 * j, p0 ^ k4); st<true>(b + 2 * j + 1, p1 ^ k4); st<true>(b + 512 + 2 * j, m0 ^ k4); st<true>(b + 512 + 2 * j + 1, m1 ^ k4);
  st<true>(b + 1024 + 2 * j, v0 ^ k4); st<true>(b + 1024 + 2 * j + 1, v1 ^ k4);
  st<true>(reinterpret_cast<u32x4*>(q16 + e), g ^ k4);
}
// State interleaved per thread: [master 4][m 4][v 4] = 48 contiguous bytes per thread, 12 KB per workgroup.
template <int W = 4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, W)))
void lay_aos48(const uint16_t* g16, u32x4* state, uint16_t* q16, int64_t tile0, uint32_t key, int64_t G) {
  const int64_t tile = tile0 + grp(blockIdx.x, gridDim.x, G);
  u32x4* b = state + tile * 768 + 3 * threadIdx.x;
  const int64_t e = tile * 1024 + 4 * threadIdx.x;
  u32x2 g = ld<true>(reinterpret_cast<const u32x2*>(g16 + e));
  u32x4 p = ld<true>(b), m = ld<true>(b + 1), v = ld<true>(b + 2);
  const u32x4 k4 = {key, key, key, key};
  st<true>(b, p ^ k4); st<true>(b + 1, m ^ k4); st<true>(b + 2, v ^ k4);
  st<true>(reinterpret_cast<u32x2*>(q16 + e), g ^ u32x2{key, key});
}

// The library's pattern: tiles of 1024 elements = [master 1024][m 1024][v 1024], one 256-thread
// workgroup per tile, 4 elements per thread, workgroups grouped G tiles per XCD.
template <int W, bool NTL, bool NTS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, W)))
void k0(const uint16_t* g16, u32x4* state, uint16_t* q16, int64_t tile0, uint32_t key, int64_t G) {
  const int64_t tile = tile0 + grp(blockIdx.x, gridDim.x, G);
  u32x4* b = state + tile * 768;
  const int j = threadIdx.x;
  const int64_t e = tile * 1024 + 4 * j;
  u32x2 g = ld<NTL>(reinterpret_cast<const u32x2*>(g16 + e));
  u32x4 p = ld<NTL>(b + j), m = ld<NTL>(b + 256 + j), v = ld<NTL>(b + 512 + j);
  const u32x4 k4 = {key, key, key, key};
  st<NTS>(b + j, p ^ k4); st<NTS>(b + 256 + j, m ^ k4); st<NTS>(b + 512 + j, v ^ k4);
  st<NTS>(reinterpret_cast<u32x2*>(q16 + e), g ^ u32x2{key, key});
}
struct Cfg { const char* name; int kind; int64_t G; int64_t launch; };
int main() {
  const int64_t n = 3253966848;  // 1,588,851 whole tiles of 2048 elements (just above the Llama-13B shard)
  uint16_t *g, *q; u32x4* s;
  HIPCHK(hipMalloc(&g, n * 2)); HIPCHK(hipMalloc(&q, n * 2)); HIPCHK(hipMalloc(&s, n * 12));
  HIPCHK(hipMemset(g, 0, n * 2)); HIPCHK(hipMemset(s, 0, n * 12));
  hipEvent_t a, b; HIPCHK(hipEventCreate(&a)); HIPCHK(hipEventCreate(&b));
  auto launch1 = [&](int kind, unsigned cnt, int64_t t0, int64_t G) {
    switch (kind) {
      case 0: hipLaunchKernelGGL((k0<4, true, true>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
      case 1: hipLaunchKernelGGL((k0<3, true, true>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
      case 2: hipLaunchKernelGGL((k0<5, true, true>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
      case 3: hipLaunchKernelGGL((k0<8, true, true>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
      case 4: hipLaunchKernelGGL((k0<4, false, true>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
      case 5: hipLaunchKernelGGL((k0<4, true, false>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
      case 6: hipLaunchKernelGGL((k0<2, true, true>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
      case 7: hipLaunchKernelGGL((lay_subtile256<4>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
      case 8: hipLaunchKernelGGL((lay_8_per_thread<4>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
      default: hipLaunchKernelGGL((lay_aos48<4>), dim3(cnt), dim3(256), 0, 0, g, s, q, t0, 0u, G); break;
    }
  };
  auto run = [&](const Cfg& c) -> float {
    const int64_t per_tile = c.kind == 8 ? 2048 : 1024;
    const int64_t tiles = n / per_tile, tpl = c.launch / per_tile;
    auto once = [&]() {
      for (int64_t t0 = 0; t0 < tiles; t0 += tpl) launch1(c.kind, (unsigned)std::min(tpl, tiles - t0), t0, c.G);
    };
    once();
    HIPCHK(hipEventRecord(a, 0));
    for (int r = 0; r < 8; ++r) once();
    HIPCHK(hipEventRecord(b, 0));
    HIPCHK(hipEventSynchronize(b));
    float ms = 0;
    HIPCHK(hipEventElapsedTime(&ms, a, b));
    return ms / 8;
  };
  const int64_t L = int64_t(1) << 25;
  Cfg cfgs[] = {
    {"library: w4 G24 2^25", 0, 24, L}, {"G1", 0, 1, L}, {"G8", 0, 8, L}, {"G16", 0, 16, L}, {"G32", 0, 32, L},
    {"G48", 0, 48, L}, {"G64", 0, 64, L}, {"w3", 1, 24, L}, {"w5", 2, 24, L}, {"w8", 3, 24, L}, {"w2", 6, 24, L},
    {"loads cached", 4, 24, L}, {"stores cached", 5, 24, L}, {"launch 2^24", 0, 24, L / 2},
    {"launch 2^26", 0, 24, L * 2}, {"launch 3*2^24", 0, 24, 3 * (L / 2)}, {"launch 2^27", 0, 24, L * 4},
    {"subtiles of 256", 7, 24, L}, {"8 per thread", 8, 12, L}, {"aos 48 B/thread", 9, 24, L},
  };
  const int nc = sizeof cfgs / sizeof cfgs[0];
  for (int round = 0; round < 3; ++round)
    for (int i = 0; i < nc; ++i) {
      float ms = run(cfgs[i]);
      if (ms <= 0) return 1;
      printf("round %d %-22s %.4f ms  %.1f GB/s\n", round, cfgs[i].name, ms, 28.0 * n / (ms * 1e-3) / 1e9);
      fflush(stdout);
    }
  HIPCHK(hipGetLastError());
  return 0;
}
