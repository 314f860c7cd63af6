// synth.hip -- host and device fills of the counter-based input generator in
// synth_core.h.  Both fills evaluate the same inline functions, so element i
// gets the same bits whichever side made it.  Inputs only: no method
// arithmetic lives here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <thread>
#include <vector>

#include "synth_core.h"

#pragma clang fp contract(off)

namespace {

constexpr uint32_t kOutlierStreamOffset = 1000u;

__host__ __device__ inline void fill_one(const syn_field& f, uint64_t key, uint64_t okey, uint64_t i, void* out,
                                         int64_t j) {
  float v = syn_value_f32(&f, key, okey, i);
  if (f.kind == SYN_F32) {
    reinterpret_cast<float*>(out)[j] = v;
  } else if (f.kind == SYN_BF16) {
    reinterpret_cast<uint16_t*>(out)[j] = syn_enc_bf16(v);
  } else {
    reinterpret_cast<uint16_t*>(out)[j] = syn_enc_fp16(v);
  }
}

__global__ void fill_kernel(syn_field f, uint64_t key, uint64_t okey, int64_t idx0, int64_t n, void* out) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
    fill_one(f, key, okey, (uint64_t)(idx0 + j), out, j);
  }
}

bool field_ok(const syn_field* f) { return f && f->kind <= SYN_FP16 && f->outlier_per_million <= 1000000u; }

// One row of workgroups per piece: piece p = blockIdx.y writes its elements
// idx0 .. idx0+n-1 to its own buffer, grid-stride over blockIdx.x.
__global__ void fill_many_kernel(syn_field f, uint64_t key, uint64_t okey, const syn_piece* pieces) {
  const syn_piece pc = pieces[blockIdx.y];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < pc.n; j += stride) {
    fill_one(f, key, okey, (uint64_t)(pc.idx0 + j), pc.out, j);
  }
}

}  // namespace

extern "C" {

// Fill out[0..n) with elements idx0 .. idx0+n-1 of the field on the host.
int syn_fill_host(const syn_field* f, int64_t idx0, int64_t n, void* out, int32_t threads) {
  if (!field_ok(f) || n < 0 || idx0 < 0 || (n > 0 && !out)) return -1;
  const syn_field fv = *f;
  const uint64_t key = syn_key(fv.seed, fv.stream, fv.step);
  const uint64_t okey = syn_key(fv.seed, fv.stream + kOutlierStreamOffset, fv.step);
  int32_t nt = threads > 0 ? threads : (int32_t)std::max(1u, std::thread::hardware_concurrency());
  nt = std::min<int32_t>(nt, 64);
  if (n < (1 << 16)) nt = 1;
  auto work = [&](int64_t lo, int64_t hi) {
    for (int64_t j = lo; j < hi; ++j) fill_one(fv, key, okey, (uint64_t)(idx0 + j), out, j);
  };
  if (nt == 1) {
    work(0, n);
    return 0;
  }
  std::vector<std::thread> pool;
  int64_t chunk = (n + nt - 1) / nt;
  for (int32_t t = 0; t < nt; ++t) {
    int64_t lo = std::min<int64_t>(n, (int64_t)t * chunk), hi = std::min<int64_t>(n, lo + chunk);
    pool.emplace_back(work, lo, hi);
  }
  for (auto& th : pool) th.join();
  return 0;
}

// Same values written to device memory on `stream` (asynchronous).
int syn_fill_device(const syn_field* f, int64_t idx0, int64_t n, void* out_dev, void* stream) {
  if (!field_ok(f) || n < 0 || idx0 < 0 || (n > 0 && !out_dev)) return -1;
  if (n == 0) return 0;
  const uint64_t key = syn_key(f->seed, f->stream, f->step);
  const uint64_t okey = syn_key(f->seed, f->stream + kOutlierStreamOffset, f->step);
  int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, *f, key, okey, idx0, n,
                     out_dev);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Several buffers in one launch: pieces_dev is a device array of n_pieces
// syn_piece records (the longest holding max_n elements); each gets exactly
// what syn_fill_device would write for it.
int syn_fill_device_many(const syn_field* f, const syn_piece* pieces_dev, int32_t n_pieces, int64_t max_n,
                         void* stream) {
  if (!field_ok(f) || n_pieces < 0 || n_pieces > 65535 || max_n < 0 || (n_pieces > 0 && !pieces_dev)) return -1;
  if (n_pieces == 0 || max_n == 0) return 0;
  const uint64_t key = syn_key(f->seed, f->stream, f->step);
  const uint64_t okey = syn_key(f->seed, f->stream + kOutlierStreamOffset, f->step);
  const int64_t blocks = std::min<int64_t>((max_n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_many_kernel, dim3((unsigned)blocks, (unsigned)n_pieces), dim3(256), 0, (hipStream_t)stream,
                     *f, key, okey, pieces_dev);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
