// update_staged_lds.hip -- measurement program (not part of the library): an LDS-staged, wavefront-
// specialised form of the tiled update against the library's update, in one process at the Llama-13B shard
// size (whole tiles).  Persistent 512-thread workgroups: threads 0..255 stream tile i+1 in and tile i-1 out
// through two LDS tile buffers while threads 256..511 update tile i with the library's own per-element code
// (its source is included).  The outputs are first compared word for word with the library's; then each
// configuration is timed with HIP events (8 calls after a warm-up, three interleaved rounds).
//
// Build and run (repository root, one MI355X):
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -ffp-contract=off -fhip-fp32-correctly-rounded-divide-sqrt \
//     -fno-gpu-flush-denormals-to-zero -Xclang -target-feature -Xclang -packed-fp32-ops -I include \
//     -o /tmp/update_staged_lds mixed_precision_adam_amd/csrc/sweeps/update_staged_lds.hip && /tmp/update_staged_lds
#include "../zero_shard.hip"

struct __align__(16) TileBuf { f32x4 st[768]; u32x2 g[256]; };

template <bool XCDMAP>
__global__ __launch_bounds__(512) void upd_staged(const uint16_t* __restrict__ g16, f32x4* __restrict__ state,
                                                  uint16_t* __restrict__ q16, int64_t tile0, int64_t ntiles,
                                                  AdamScalars s) {
  __shared__ TileBuf buf[2];
  const int tid = threadIdx.x, j = tid & 255;
  const bool mem = tid < 256;
  const int64_t stride = gridDim.x;
  int64_t first = blockIdx.x;
  if (XCDMAP) {  // XCD x (= b mod 8) takes a contiguous eighth of each stride block
    const int64_t per = stride / 8;
    first = (blockIdx.x % 8) * per + blockIdx.x / 8;
  }
  const int64_t iters = first < ntiles ? (ntiles - first + stride - 1) / stride : 0;
  if (iters == 0) return;  // uniform for the workgroup
  auto tile_of = [&](int64_t i) { return tile0 + first + i * stride; };
  if (mem) {
    const int64_t t = tile_of(0);
    const f32x4* b = state + t * 768;
    buf[0].g[j] = ld_stream(reinterpret_cast<const u32x2*>(g16 + t * 1024 + 4 * j));
    buf[0].st[j] = ld_stream(b + j);
    buf[0].st[256 + j] = ld_stream(b + 256 + j);
    buf[0].st[512 + j] = ld_stream(b + 512 + j);
  }
  __syncthreads();
  for (int64_t i = 0; i < iters; ++i) {
    TileBuf& cur = buf[i & 1];
    TileBuf& oth = buf[(i + 1) & 1];
    if (mem) {
      const bool prev = i > 0, next = i + 1 < iters;
      u32x2 rq = {0u, 0u}, ng = {0u, 0u};
      f32x4 rp = {}, rm = {}, rv = {}, np = {}, nm = {}, nv = {};
      if (prev) { rq = oth.g[j]; rp = oth.st[j]; rm = oth.st[256 + j]; rv = oth.st[512 + j]; }
      if (next) {
        const int64_t t = tile_of(i + 1);
        const f32x4* b = state + t * 768;
        ng = ld_stream(reinterpret_cast<const u32x2*>(g16 + t * 1024 + 4 * j));
        np = ld_stream(b + j); nm = ld_stream(b + 256 + j); nv = ld_stream(b + 512 + j);
      }
      if (prev) {
        const int64_t t = tile_of(i - 1);
        f32x4* b = state + t * 768;
        st_stream(b + j, rp); st_stream(b + 256 + j, rm); st_stream(b + 512 + j, rv);
        st_stream(reinterpret_cast<u32x2*>(q16 + t * 1024 + 4 * j), rq);
      }
      if (next) { oth.g[j] = ng; oth.st[j] = np; oth.st[256 + j] = nm; oth.st[512 + j] = nv; }
    } else {
      u32x2 g = cur.g[j];
      f32x4 p = cur.st[j], m = cur.st[256 + j], v = cur.st[512 + j];
      const u32x2 q = adam_unit4<ZERO_FP16, ZERO_BF16>(g, p, m, v, s);
      cur.st[j] = p; cur.st[256 + j] = m; cur.st[512 + j] = v; cur.g[j] = q;
    }
    __syncthreads();
  }
  if (mem) {
    const int64_t t = tile_of(iters - 1);
    TileBuf& last = buf[(iters - 1) & 1];
    f32x4* b = state + t * 768;
    st_stream(b + j, last.st[j]); st_stream(b + 256 + j, last.st[256 + j]); st_stream(b + 512 + j, last.st[512 + j]);
    st_stream(reinterpret_cast<u32x2*>(q16 + t * 1024 + 4 * j), last.g[j]);
  }
}

__global__ void fill16(uint16_t* g, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    g[i] = (uint16_t)(0x3C00u | ((uint32_t)(i * 2654435761u) >> 22));
}
__global__ void count_diff(const uint32_t* a, const uint32_t* b, int64_t n, unsigned long long* out) {
  unsigned long long c = 0;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) c += a[i] != b[i];
  if (c) atomicAdd(out, c);
}
#define HIPCHK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP %s at %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)

int main() {
  const int64_t tiles = 3177701, n = tiles * 1024;  // whole tiles of the Llama-13B shard
  uint16_t *g, *qa, *qb; f32x4 *sa, *sb; unsigned long long* cnt;
  HIPCHK(hipMalloc(&g, n * 2)); HIPCHK(hipMalloc(&qa, n * 2)); HIPCHK(hipMalloc(&qb, n * 2));
  HIPCHK(hipMalloc(&sa, n * 12)); HIPCHK(hipMalloc(&sb, n * 12)); HIPCHK(hipMalloc(&cnt, 8));
  HIPCHK(hipMemset(sa, 0, n * 12)); HIPCHK(hipMemset(sb, 0, n * 12));
  hipLaunchKernelGGL(fill16, dim3(65536), dim3(256), 0, 0, g, n);
  HIPCHK(hipDeviceSynchronize());
  zero_adamw_hparams hp = {1e-4, 0.9, 0.999, 1e-8, 0.01, 1.0 / 65536 / 57.0, 1};
  AdamScalars sc;
  if (adam_args_ok("probe", g, ZERO_FP16, qa, ZERO_BF16, n, &hp, &sc) != ZERO_OK) { printf("args\n"); return 1; }
  const int64_t tpl = 32768;
  auto lib = [&](f32x4* s, uint16_t* q) {
    for (int64_t t0 = 0; t0 < tiles; t0 += tpl)
      hipLaunchKernelGGL((adamw_tiled_kernel<ZERO_FP16, ZERO_BF16>), dim3((unsigned)std::min(tpl, tiles - t0)),
                         dim3(kBlock), 0, 0, g, s, q, n, t0, sc, nullptr);
  };
  auto staged = [&](f32x4* s, uint16_t* q, int wgs, bool xcd) {
    for (int64_t t0 = 0; t0 < tiles; t0 += tpl) {
      const int64_t nt = std::min(tpl, tiles - t0);
      const unsigned grid = (unsigned)std::min<int64_t>(wgs, nt);
      if (xcd) hipLaunchKernelGGL(upd_staged<true>, dim3(grid), dim3(512), 0, 0, g, s, q, t0, nt, sc);
      else hipLaunchKernelGGL(upd_staged<false>, dim3(grid), dim3(512), 0, 0, g, s, q, t0, nt, sc);
    }
  };
  // correctness: one pass each from the same zero state, every word compared
  lib(sa, qa); staged(sb, qb, 512, false);
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemset(cnt, 0, 8));
  hipLaunchKernelGGL(count_diff, dim3(65536), dim3(256), 0, 0, (const uint32_t*)sa, (const uint32_t*)sb, n * 3, cnt);
  hipLaunchKernelGGL(count_diff, dim3(65536), dim3(256), 0, 0, (const uint32_t*)qa, (const uint32_t*)qb, n / 2, cnt);
  unsigned long long diff = 0;
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemcpy(&diff, cnt, 8, hipMemcpyDeviceToHost));
  printf("staged vs library after one pass: %llu differing words\n", diff);
  staged(sb, qb, 1024, true);  // the XCD mapping too, one more pass on both
  lib(sa, qa);
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemset(cnt, 0, 8));
  hipLaunchKernelGGL(count_diff, dim3(65536), dim3(256), 0, 0, (const uint32_t*)sa, (const uint32_t*)sb, n * 3, cnt);
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemcpy(&diff, cnt, 8, hipMemcpyDeviceToHost));
  printf("after a second pass (xcd mapping, 4 workgroups per CU): %llu differing words\n", diff);
  fflush(stdout);
  hipEvent_t a, b; HIPCHK(hipEventCreate(&a)); HIPCHK(hipEventCreate(&b));
  struct C { const char* name; int wgs; bool xcd; bool libk; };
  C cs[] = {{"library update", 0, false, true}, {"staged 2/CU", 512, false, false}, {"staged 3/CU", 768, false, false},
            {"staged 4/CU", 1024, false, false}, {"staged 2/CU xcd", 512, true, false},
            {"staged 3/CU xcd", 768, true, false}, {"staged 4/CU xcd", 1024, true, false}};
  for (int round = 0; round < 3; ++round)
    for (const C& c : cs) {
      auto once = [&]() { if (c.libk) lib(sa, qa); else staged(sb, qb, c.wgs, c.xcd); };
      once();
      HIPCHK(hipEventRecord(a, 0));
      for (int r = 0; r < 8; ++r) once();
      HIPCHK(hipEventRecord(b, 0));
      HIPCHK(hipEventSynchronize(b));
      float ms = 0;
      HIPCHK(hipEventElapsedTime(&ms, a, b));
      ms /= 8;
      printf("round %d %-17s %.4f ms  %.1f GB/s\n", round, c.name, ms, 28.0 * n / (ms * 1e-3) / 1e9);
      fflush(stdout);
    }
  HIPCHK(hipGetLastError());
  return 0;
}
