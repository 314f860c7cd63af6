// zero_shard.hip -- libzero_shard.so: one data-parallel rank's share of a
// ZeRO-1/2/3 mixed-precision AdamW step, written for CDNA4 (gfx950).
//
// The operations and their sources are documented in include/zero_shard.h.
// Design for the MI355X: every device kernel here streams HBM (the AdamW step
// moves 28 bytes per parameter for 60-80 VALU instructions), so the kernels are
// built around 16-byte coalesced vector accesses, one tile per workgroup with
// all loads of a tile issued before any arithmetic, and no matrix cores --
// nothing on this path is a contraction.  The gradient norm is a fixed-grid,
// fixed-tree fp64 reduction (wavefront shuffles, then LDS) so its bits do not
// change from run to run.  Floating-point contraction is off for the whole
// file: the AdamW update is specified as a sequence of individually rounded
// fp32 operations.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <algorithm>
#include <cstdio>
#include <limits>
#include <mutex>

#include "zero_shard.h"

#pragma clang fp contract(off)

namespace {

// ------------------------------------------------------------------ errors

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return ZERO_OK;
}

constexpr int64_t kMaxPsi = ZERO_MAX_NUMEL;  // 2^58: keeps 16·Ψ and N·S in range
static_assert(kMaxPsi == std::numeric_limits<int64_t>::max() / 32, "element-count limit");

// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1 (which can overflow).
constexpr int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0 ? 1 : 0); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;  // 4 wavefronts of 64

// Streaming kernels capped at 4 wavefronts per SIMD (measurements at each
// kernel): the compiler reserves registers so that no more fit on a SIMD.
#define STREAMING_KERNEL __global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 4)))

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
inline bool fp32_aligned(const void* a, const void* b, const void* c, const void* d) {
  return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) | reinterpret_cast<uintptr_t>(c) |
           reinterpret_cast<uintptr_t>(d)) & 3u) == 0;
}

// ------------------------------------------------------------------ 16-bit formats

// Widen one 16-bit value (in the low half of h) to fp32; exact for both formats.
template <int DT>
__device__ __forceinline__ float widen(uint32_t h) {
  if constexpr (DT == ZERO_BF16) {
    return __uint_as_float(h << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
  }
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> the parameter format PT (bf16 or IEEE binary16), round to nearest,
// ties to even.  The binary16 conversion is the hardware's (v_cvt_f16_f32 in
// the default round-to-nearest-even mode, binary16 denormals kept): overflow
// gives infinity, tiny values become subnormals or zero.
template <int PT>
__device__ __forceinline__ uint32_t narrow(float f) {
  if constexpr (PT == ZERO_BF16) {
    return bf16_rne(f);
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  }
}

// ------------------------------------------------------------------ AdamW

struct AdamScalars {
  float b1, omb1, b2, omb2, eps, decay, step_size, bc2_sqrt, gscale;
};

// One element of the update, each line one rounded fp32 operation.
__device__ __forceinline__ void adam_element(float g, float& p, float& m, float& v, const AdamScalars& s) {
  g = g * s.gscale;
  const float m_keep = s.b1 * m;
  const float m_add = s.omb1 * g;
  m = m_keep + m_add;
  const float gg = g * g;
  const float v_keep = s.b2 * v;
  const float v_add = s.omb2 * gg;
  v = v_keep + v_add;
  float d = sqrtf(v);
  d = d / s.bc2_sqrt;
  d = d + s.eps;
  float u = m / d;
  u = s.step_size * u;
  const float p_dec = p * s.decay;
  p = p_dec - u;
}

// Scalars of the update: by value from the host, or from the device-resident
// step state when `dev` is given (then a skipped step leaves everything as is).
// Every lane reads the same few bytes, so they come through the scalar cache.
__device__ __forceinline__ bool take_scalars(const zero_step_state* dev, AdamScalars& s) {
  if (dev == nullptr) return true;
  if (dev->skip) return false;
  s.b1 = dev->scalars[0];
  s.omb1 = dev->scalars[1];
  s.b2 = dev->scalars[2];
  s.omb2 = dev->scalars[3];
  s.eps = dev->scalars[4];
  s.decay = dev->scalars[5];
  s.step_size = dev->scalars[6];
  s.bc2_sqrt = dev->scalars[7];
  s.gscale = dev->scalars[8];
  return true;
}

// Streaming accesses: every byte the update touches is used exactly once, so
// loads and stores carry the non-temporal hint (measured on MI355X: the
// stores are worth 13% to the tiled update, the loads a few percent more).
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

// Four consecutive elements: grads as two 32-bit words (2 x 16-bit each), the
// fp32 state as one 16-byte vector per array.  Returns the four 16-bit params.
template <int DT, int PT>
__device__ __forceinline__ u32x2 adam_unit4(u32x2 g, f32x4& p, f32x4& m, f32x4& v, const AdamScalars& s) {
  u32x2 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const int c = 2 * w;
    float p0 = p[c], p1 = p[c + 1], m0 = m[c], m1 = m[c + 1], v0 = v[c], v1 = v[c + 1];
    adam_element(widen<DT>(g[w] & 0xFFFFu), p0, m0, v0, s);
    adam_element(widen<DT>(g[w] >> 16), p1, m1, v1, s);
    p[c] = p0;
    p[c + 1] = p1;
    m[c] = m0;
    m[c + 1] = m1;
    v[c] = v0;
    v[c + 1] = v1;
    out[w] = narrow<PT>(p0) | (narrow<PT>(p1) << 16);
  }
  return out;
}

// The last, partial group of four elements (at most one per launch): element
// by element, touching nothing at or past n.
template <int DT, int PT>
__device__ __forceinline__ void adam_partial4(const uint16_t* __restrict__ grad, float* __restrict__ p,
                                              float* __restrict__ m, float* __restrict__ v,
                                              uint16_t* __restrict__ param, int64_t e, int64_t n,
                                              const AdamScalars& s) {
  for (int64_t i = e; i < n; ++i) {
    float pi = p[i - e], mi = m[i - e], vi = v[i - e];
    adam_element(widen<DT>(grad[i]), pi, mi, vi, s);
    p[i - e] = pi;
    m[i - e] = mi;
    v[i - e] = vi;
    param[i] = static_cast<uint16_t>(narrow<PT>(pi));
  }
}

// Separate master / m / v arrays.  Unit u of workgroup b (= block0 + the
// launch's blockIdx.x) covers elements
// 4·(b·U·256 + u·256 + t) .. +3 for thread t, so every load and store
// instruction of a wavefront touches one contiguous span (1 KiB for the fp32
// arrays, 512 B for grads and params).  All loads of the workgroup's U units
// are issued before the arithmetic.  The thread whose group straddles n
// finishes the ragged tail element by element.
// Capped at 4 wavefronts per SIMD like the tiled update: measured 2.3% faster
// on the GPT-2 rank shard than uncapped.
template <int DT, int PT, int U>
STREAMING_KERNEL void adamw_vec_kernel(const uint16_t* __restrict__ grad16, float* __restrict__ master,
                                       float* __restrict__ mom, float* __restrict__ var,
                                       uint16_t* __restrict__ param16, int64_t n, int64_t block0, AdamScalars s,
                                       const zero_step_state* dev) {
  const int64_t n4 = n >> 2;
  const int64_t first = (block0 + blockIdx.x) * (kBlock * U) + threadIdx.x;
  const u32x2* grad = reinterpret_cast<const u32x2*>(grad16);
  f32x4* p4 = reinterpret_cast<f32x4*>(master);
  f32x4* m4 = reinterpret_cast<f32x4*>(mom);
  f32x4* v4 = reinterpret_cast<f32x4*>(var);
  u32x2* param = reinterpret_cast<u32x2*>(param16);
  u32x2 g[U];
  f32x4 p[U], m[U], v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = first + static_cast<int64_t>(u) * kBlock;
    if (i < n4) {
      g[u] = ld_stream(grad + i);
      p[u] = ld_stream(p4 + i);
      m[u] = ld_stream(m4 + i);
      v[u] = ld_stream(v4 + i);
    }
  }
  if (!take_scalars(dev, s)) return;  // after the data loads: they overlap with the scalar fetch
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = first + static_cast<int64_t>(u) * kBlock;
    if (i < n4) {
      const u32x2 q = adam_unit4<DT, PT>(g[u], p[u], m[u], v[u], s);
      st_stream(p4 + i, p[u]);
      st_stream(m4 + i, m[u]);
      st_stream(v4 + i, v[u]);
      st_stream(param + i, q);
    } else if (i == n4 && 4 * n4 < n) {
      const int64_t e = 4 * n4;
      adam_partial4<DT, PT>(grad16, master + e, mom + e, var + e, param16, e, n, s);
    }
  }
}

// Groups of four elements per thread in the separate-array update: measured
// on MI355X, one beats two by 3% and four by 9% of the update's bandwidth.
constexpr int kAdamUnroll = 1;

// Tiled optimizer state (ZERO_STATE_TILE = 1024 elements per tile): tile k
// stores master, m and v of elements [1024k, 1024k+1024) back to back, so the
// update streams three address ranges (grad, state, param) instead of five.
// One 256-thread workgroup per tile (tile0 + an XCD-grouped blockIdx.x, see
// xcd_grouped); thread t owns the group of four elements 4t .. 4t+3
// (kTileUnits groups in general, issuing every load before any arithmetic).
// Measured on MI355X, one group per thread and 12 KiB of state per workgroup
// beats two groups / 24 KiB by 4%, provided every store carries the
// non-temporal hint (without it the update loses 13%).  In the last tile,
// groups past n are skipped and the group straddling n is updated element by
// element (the tile's padding floats keep their bits).
constexpr int64_t kTile = ZERO_STATE_TILE;
constexpr int kTileUnits = 1;

// The dispatcher deals a launch's workgroups to the eight XCDs in turn, so
// workgroup b runs on XCD b mod 8.  Remapping workgroups to tiles so that each
// XCD takes kXcdGroup adjacent tiles at a time (the first 8·kXcdGroup
// workgroups cover 8·kXcdGroup adjacent tiles, XCD x taking the x-th run of
// kXcdGroup) is faster on MI355X: groups of 8 gained 0.5-1.2% over no
// grouping, and with the occupancy cap below, update time on the GPT-2 rank
// shard relative to groups of 8 is: 16 -0.3%, 20 -0.6%, 24 -1.9%, 28 +0.5%,
// 32 -1.2%, 40 +0.8%, 48 -1.1%, 64 +0.2%; with 24 the Llama-7B, Llama-13B
// and 1T shards gain 1.7% too.  A whole contiguous range per XCD was 2-3%
// slower than no grouping.  A bijection on [0, n): workgroups past the last
// whole span of 8·kXcdGroup keep their own index.
constexpr int64_t kXcds = 8, kXcdGroup = 24;
__device__ __forceinline__ int64_t xcd_grouped(int64_t b, int64_t n) {
  constexpr int64_t kSpan = kXcds * kXcdGroup;
  if (b >= n / kSpan * kSpan) return b;
  const int64_t x = b % kXcds, q = b / kXcds;
  return q / kXcdGroup * kSpan + x * kXcdGroup + q % kXcdGroup;
}
constexpr int64_t kTile4 = kTile / 4;  // 16-byte vectors per array per tile
static_assert(kTile4 == kBlock * kTileUnits, "each thread owns kTileUnits groups of 4 elements of a tile");

// One tile of the tiled update, or (CALIB) the same loads and stores with the
// arithmetic replaced by an XOR with a run-time key: the read-modify-write
// ceiling of exactly this access pattern (zero_calibrate_tiled_rmw).
template <int DT, int PT, bool CALIB>
__device__ __forceinline__ void tiled_tile(const uint16_t* __restrict__ grad16, f32x4* __restrict__ state,
                                           uint16_t* __restrict__ param16, int64_t n, int64_t tile0, AdamScalars s,
                                           const zero_step_state* dev, uint32_t key) {
  const int64_t tile = tile0 + xcd_grouped(blockIdx.x, gridDim.x);
  f32x4* base = state + tile * (3 * kTile4);
  u32x2 g[kTileUnits];
  f32x4 p[kTileUnits], m[kTileUnits], v[kTileUnits];
#pragma unroll
  for (int u = 0; u < kTileUnits; ++u) {
    const int j = threadIdx.x + u * kBlock;
    const int64_t e = tile * kTile + 4 * static_cast<int64_t>(j);
    if (e + 4 <= n) {
      g[u] = ld_stream(reinterpret_cast<const u32x2*>(grad16 + e));
      p[u] = ld_stream(base + j);
      m[u] = ld_stream(base + kTile4 + j);
      v[u] = ld_stream(base + 2 * kTile4 + j);
    }
  }
  // The data loads above do not depend on the scalars, so they are in flight
  // while the (device-resident) scalars arrive.
  if (!CALIB && !take_scalars(dev, s)) return;
#pragma unroll
  for (int u = 0; u < kTileUnits; ++u) {
    const int j = threadIdx.x + u * kBlock;
    const int64_t e = tile * kTile + 4 * static_cast<int64_t>(j);
    if (e + 4 <= n) {
      u32x2 q;
      if constexpr (CALIB) {
        const u32x4 k4 = {key, key, key, key};
        p[u] = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, p[u]) ^ k4);
        m[u] = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, m[u]) ^ k4);
        v[u] = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, v[u]) ^ k4);
        q = g[u] ^ u32x2{key, key};
      } else {
        q = adam_unit4<DT, PT>(g[u], p[u], m[u], v[u], s);
      }
      st_stream(base + j, p[u]);
      st_stream(base + kTile4 + j, m[u]);
      st_stream(base + 2 * kTile4 + j, v[u]);
      st_stream(reinterpret_cast<u32x2*>(param16 + e), q);
    } else if (e < n && !CALIB) {
      float* f = reinterpret_cast<float*>(base + j);
      adam_partial4<DT, PT>(grad16, f, f + kTile, f + 2 * kTile, param16, e, n, s);
    }
  }
}

// At most 4 wavefronts per SIMD (4 tiles, 64 KiB in flight per CU): the
// compiler reserves registers so that no more fit.  Measured on MI355X: 1.7%
// faster than the 8 the kernel's 26 registers would allow (3: the same; 5:
// 0.6% slower than 4; 2: 7% slower), 1% faster on the Llama-13B shard.
template <int DT, int PT>
STREAMING_KERNEL void adamw_tiled_kernel(const uint16_t* __restrict__ grad16, f32x4* __restrict__ state,
                                         uint16_t* __restrict__ param16, int64_t n, int64_t tile0, AdamScalars s,
                                         const zero_step_state* dev) {
  tiled_tile<DT, PT, false>(grad16, state, param16, n, tile0, s, dev, 0u);
}

// The update's memory traffic without its arithmetic (whole groups of four
// only; a ragged tail is left alone).
STREAMING_KERNEL void tiled_rmw_calibration_kernel(const uint16_t* __restrict__ grad16, f32x4* __restrict__ state,
                                                   uint16_t* __restrict__ param16, int64_t n, int64_t tile0,
                                                   uint32_t key) {
  tiled_tile<ZERO_BF16, ZERO_BF16, true>(grad16, state, param16, n, tile0, AdamScalars{}, nullptr, key);
}

// Element paths for ragged tails and unaligned buffers: the same update, one
// element per thread, grid-stride.  TILED selects the state addressing.
template <int DT, int PT, bool TILED>
__global__ __launch_bounds__(kBlock) void adamw_element_kernel(const uint16_t* __restrict__ grad,
                                                               float* __restrict__ master, float* __restrict__ mom,
                                                               float* __restrict__ var, uint16_t* __restrict__ param,
                                                               int64_t begin, int64_t n, AdamScalars s,
                                                               const zero_step_state* dev) {
  if (!take_scalars(dev, s)) return;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = begin + static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
    int64_t ip = i, im = i, iv = i;
    if (TILED) {
      ip = (i / kTile) * (3 * kTile) + (i % kTile);
      im = ip + kTile;
      iv = ip + 2 * kTile;
    }
    float p = master[ip], m = mom[im], v = var[iv];
    adam_element(widen<DT>(grad[i]), p, m, v, s);
    master[ip] = p;
    mom[im] = m;
    var[iv] = v;
    param[i] = static_cast<uint16_t>(narrow<PT>(p));
  }
}

// Conversion between separate arrays and the tiled state (bit copies).
template <bool TO_TILED>
__global__ __launch_bounds__(kBlock) void retile_kernel(float* __restrict__ master, float* __restrict__ mom,
                                                        float* __restrict__ var, float* __restrict__ state, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
    const int64_t t = (i / kTile) * (3 * kTile) + (i % kTile);
    if (TO_TILED) {
      state[t] = master[i];
      state[t + kTile] = mom[i];
      state[t + 2 * kTile] = var[i];
    } else {
      master[i] = state[t];
      mom[i] = state[t + kTile];
      var[i] = state[t + 2 * kTile];
    }
  }
}

// ------------------------------------------------------------------ gradient square-norm

// One workgroup per 32768 elements (up to 2^19 workgroups, so the partials
// stay under 6 MiB).  Measured on MI355X over the 976.6M-element fp16 shard
// of the 1T configuration: 6.6 TB/s, against 6.2 TB/s with at most 4096
// workgroups of longer ranges (8192 and 16384 elements: 6.35 and 6.46).
constexpr int64_t kNormElemsPerPart = int64_t(1) << 15;
constexpr int64_t kNormMaxParts = int64_t(1) << 19;

int64_t norm_parts(int64_t n) {
  int64_t parts = ceil_div(n, kNormElemsPerPart);
  if (parts < 1) parts = 1;
  if (parts > kNormMaxParts) parts = kNormMaxParts;
  return parts;
}

template <int DT>
__device__ __forceinline__ void accumulate(uint32_t h, double& acc, uint32_t& bad) {
  constexpr uint32_t kExp = DT == ZERO_BF16 ? 0x7F80u : 0x7C00u;
  const double x = static_cast<double>(widen<DT>(h));
  const double sq = x * x;  // exact: at most 2·11 significant bits
  acc = acc + sq;
  bad |= ((h & kExp) == kExp) ? 1u : 0u;
}

template <int DT>
__device__ __forceinline__ void accumulate8(u32x4 w, double& acc, uint32_t& bad) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    accumulate<DT>(w[c] & 0xFFFFu, acc, bad);
    accumulate<DT>(w[c] >> 16, acc, bad);
  }
}

// Sum over a workgroup of NT threads in a fixed tree: butterfly inside each
// wavefront, then the NT/64 wavefront sums in order.  Result valid in thread 0.
template <int NT = kBlock>
__device__ __forceinline__ void block_reduce(double& acc, uint32_t& bad) {
  __shared__ double wsum[NT / 64];
  __shared__ uint32_t wbad[NT / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    acc = acc + __shfl_xor(acc, off, 64);
    bad |= __shfl_xor(bad, off, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    wsum[wave] = acc;
    wbad[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    acc = wsum[0];
    bad = wbad[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
      acc = acc + wsum[w];
      bad |= wbad[w];
    }
  }
}

// Stage 1: workgroup b reduces its contiguous range of 16-B vectors; the last
// workgroup also takes the unaligned head and ragged tail elements.
// Capped at 4 wavefronts per SIMD: measured 6% faster over the 1T shard's
// 976.6M fp16 gradients than uncapped (2: 40% slower).
template <int DT>
STREAMING_KERNEL void sqnorm_partial_kernel(const uint16_t* __restrict__ x, int64_t n, int64_t head, int64_t n8,
                                            int64_t per_block, double* __restrict__ part_sum,
                                            uint32_t* __restrict__ part_bad) {
  double acc = 0.0;
  uint32_t bad = 0;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x + head);
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per_block;
  const int64_t hi = lo + per_block < n8 ? lo + per_block : n8;
  constexpr int kU = 4;
  int64_t i = lo + threadIdx.x;
  for (; i + (kU - 1) * kBlock < hi; i += kU * kBlock) {
    u32x4 w[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) w[u] = ld_stream(xv + i + u * kBlock);
#pragma unroll
    for (int u = 0; u < kU; ++u) accumulate8<DT>(w[u], acc, bad);
  }
  for (; i < hi; i += kBlock) accumulate8<DT>(ld_stream(xv + i), acc, bad);
  if (blockIdx.x == gridDim.x - 1) {
    for (int64_t j = threadIdx.x; j < head; j += kBlock) accumulate<DT>(x[j], acc, bad);
    for (int64_t j = head + 8 * n8 + threadIdx.x; j < n; j += kBlock) accumulate<DT>(x[j], acc, bad);
  }
  block_reduce(acc, bad);
  if (threadIdx.x == 0) {
    part_sum[blockIdx.x] = acc;
    part_bad[blockIdx.x] = bad;
  }
}

// Stage 2: one workgroup of kFoldThreads folds `parts` partials, read at
// indices 0, stride, 2·stride, ..., in a fixed order: thread t adds partials
// t, t + kFoldThreads, ... in ascending order, then the workgroup tree.  It is
// bound by memory latency: loads are issued kR at a time ahead of the
// additions (which keep their order), and 16 wavefronts keep 16 times more
// of them in flight than one.
constexpr int kFoldThreads = 1024;
__global__ __launch_bounds__(kFoldThreads) void sqnorm_final_kernel(const double* __restrict__ part_sum,
                                                                    const uint32_t* __restrict__ part_bad,
                                                                    int64_t parts, int64_t stride,
                                                                    double* __restrict__ out_sum,
                                                                    int32_t* __restrict__ out_bad) {
  constexpr int kR = 8;
  double acc = 0.0;
  uint32_t bad = 0;
  int64_t j = threadIdx.x;
  for (; j + (kR - 1) * kFoldThreads < parts; j += kR * kFoldThreads) {
    double x[kR];
    uint32_t f[kR];
#pragma unroll
    for (int u = 0; u < kR; ++u) {
      x[u] = part_sum[(j + u * kFoldThreads) * stride];
      f[u] = part_bad[(j + u * kFoldThreads) * stride];
    }
#pragma unroll
    for (int u = 0; u < kR; ++u) {
      acc = acc + x[u];
      bad |= f[u];
    }
  }
  for (; j < parts; j += kFoldThreads) {
    acc = acc + part_sum[j * stride];
    bad |= part_bad[j * stride];
  }
  block_reduce<kFoldThreads>(acc, bad);
  if (threadIdx.x == 0) {
    *out_sum = acc;
    *out_bad = bad ? 1 : 0;
  }
}

// A single workgroup reads its partials at the bandwidth of one compute unit:
// 397,213 partials (the flatten of a 3.25e9-element shard) took 96 us.  Past
// kFoldTwoLevel partials the fold therefore takes two levels: workgroup g
// folds the chunk [g·kFoldChunk, (g+1)·kFoldChunk) in a fixed order (thread
// t adds the chunk's partials t, t + 256, ... in order, then the workgroup
// tree) and leaves the result in place of the chunk's first partial, which it
// has already read; stage 2 then folds those at stride kFoldChunk.  The
// partials buffer is scratch and is overwritten.
constexpr int64_t kFoldChunk = 4096, kFoldTwoLevel = 65536;
__global__ __launch_bounds__(kBlock) void sqnorm_fold_chunks_kernel(double* __restrict__ part_sum,
                                                                    uint32_t* __restrict__ part_bad, int64_t parts) {
  constexpr int kPer = static_cast<int>(kFoldChunk / kBlock);
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * kFoldChunk;
  double x[kPer];
  uint32_t f[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t j = lo + threadIdx.x + u * kBlock;
    x[u] = j < parts ? part_sum[j] : 0.0;  // adding +0.0 to a sum of non-negative terms changes nothing
    f[u] = j < parts ? part_bad[j] : 0u;
  }
  double acc = 0.0;
  uint32_t bad = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    acc = acc + x[u];
    bad |= f[u];
  }
  block_reduce(acc, bad);  // its barrier orders every read of the chunk before the write below
  if (threadIdx.x == 0) {
    part_sum[lo] = acc;
    part_bad[lo] = bad;
  }
}

// ------------------------------------------------------------------ flatten

// Source tensors are plain device allocations (global memory); saying so lets
// the compiler use global rather than flat loads for them.
typedef const u32x4 __attribute__((address_space(1)))* global_u32x4_ptr;
typedef const uint16_t __attribute__((address_space(1)))* global_u16_ptr;

// Bytes [SH, SH + 16) of the 32 bytes a, b (SH even, 2 .. 14): the 16 source
// bytes of one destination vector when source and destination differ in
// their position inside a 16-byte line.
template <int SH>
__device__ __forceinline__ u32x4 funnel16(u32x4 a, u32x4 b) {
  constexpr int q = SH / 4, r = SH % 4;
  const uint32_t c[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (r == 0) {
      out[i] = c[q + i];
    } else {
      out[i] = __builtin_amdgcn_alignbyte(c[q + i + 1], c[q + i], r);  // ({hi, lo} >> 8r), low 32 bits
    }
  }
  return out;
}

// The 16-byte body of a piece: nv destination vectors dv[0 .. nv).  SH = 0:
// source vector j is sv[j].  SH > 0: it straddles the aligned 16-byte source
// blocks sv[j] and sv[j + 1] (both hold bytes of the piece, so neither read
// leaves the source's pages); adjacent threads read the same blocks, so these
// loads keep the ordinary cache policy and the second read of a block is
// served by the cache.
template <int DT, bool ACC, int SH>
__device__ __forceinline__ void copy_body(const global_u32x4_ptr sv, u32x4* __restrict__ dv, int64_t nv, double& acc,
                                          uint32_t& bad) {
  constexpr int kU = 4;  // vectors in flight per thread (more than occupancy is worth here)
  auto load = [&](int64_t j) -> u32x4 {
    if constexpr (SH == 0) {
      return __builtin_nontemporal_load(sv + j);
    } else {
      return funnel16<SH>(sv[j], sv[j + 1]);
    }
  };
  int64_t j = threadIdx.x;
  for (; j + (kU - 1) * kBlock < nv; j += kU * kBlock) {
    u32x4 w[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) w[u] = load(j + u * kBlock);
#pragma unroll
    for (int u = 0; u < kU; ++u) dv[j + u * kBlock] = w[u];
    if (ACC) {
#pragma unroll
      for (int u = 0; u < kU; ++u) accumulate8<DT>(w[u], acc, bad);
    }
  }
  for (; j < nv; j += kBlock) {
    const u32x4 w = load(j);
    dv[j] = w;
    if (ACC) accumulate8<DT>(w, acc, bad);
  }
}

// A workgroup copies len 16-bit elements from s to d: a scalar head brings d
// to a 16-byte boundary, the body moves 16-byte vectors (copy_body), a scalar
// tail finishes.  When source and destination differ in their position
// inside a 16-byte line, each destination vector is assembled from the two
// aligned source blocks it straddles.  With ACC the copied values are also
// squared into acc (fp64) and checked for inf/NaN.  Source reads stream
// (non-temporal); the shard is stored with ordinary stores: the update reads
// part of it back from the Infinity Cache right away.  Measured on MI355X
// against non-temporal stores: the GPT-2 1.5B rank's whole step is 1.2%
// faster that way (its flatten 3.7%) and the Llama-13B one 0.8-1%, although a
// plain copy runs 1-2% slower.
template <int DT, bool ACC>
__device__ void copy_piece(const uint16_t* __restrict__ s_generic, uint16_t* __restrict__ d, int64_t len, double& acc,
                           uint32_t& bad) {
  const global_u16_ptr s = (global_u16_ptr)s_generic;
  const uintptr_t ds = reinterpret_cast<uintptr_t>(d), ss = reinterpret_cast<uintptr_t>(s_generic);
  int64_t head = static_cast<int64_t>(((16u - (ds & 15u)) & 15u) >> 1);
  if (head > len) head = len;
  const int64_t nv = (len - head) >> 3;
  for (int64_t j = threadIdx.x; j < head; j += kBlock) {
    const uint16_t x = s[j];
    d[j] = x;
    if (ACC) accumulate<DT>(x, acc, bad);
  }
  if (nv > 0) {
    // byte offset of the body's first source byte inside its 16-byte line:
    // 0 when the phases match, else even (both are 2-byte aligned)
    const uintptr_t sb = ss + 2 * static_cast<uintptr_t>(head);
    const int shift = static_cast<int>(sb & 15u);
    const global_u32x4_ptr sv = (global_u32x4_ptr)(s_generic + head - shift / 2);  // aligned: sb - shift
    u32x4* dv = reinterpret_cast<u32x4*>(d + head);
    switch (shift) {  // uniform across the workgroup
      case 0: copy_body<DT, ACC, 0>(sv, dv, nv, acc, bad); break;
      case 2: copy_body<DT, ACC, 2>(sv, dv, nv, acc, bad); break;
      case 4: copy_body<DT, ACC, 4>(sv, dv, nv, acc, bad); break;
      case 6: copy_body<DT, ACC, 6>(sv, dv, nv, acc, bad); break;
      case 8: copy_body<DT, ACC, 8>(sv, dv, nv, acc, bad); break;
      case 10: copy_body<DT, ACC, 10>(sv, dv, nv, acc, bad); break;
      case 12: copy_body<DT, ACC, 12>(sv, dv, nv, acc, bad); break;
      default: copy_body<DT, ACC, 14>(sv, dv, nv, acc, bad); break;
    }
  }
  for (int64_t t = head + 8 * nv + threadIdx.x; t < len; t += kBlock) {
    const uint16_t x = s[t];
    d[t] = x;
    if (ACC) accumulate<DT>(x, acc, bad);
  }
}

__device__ void zero_piece(uint16_t* __restrict__ d, int64_t len) {
  const uintptr_t ds = reinterpret_cast<uintptr_t>(d);
  int64_t head = static_cast<int64_t>(((16u - (ds & 15u)) & 15u) >> 1);
  if (head > len) head = len;
  const int64_t nv = (len - head) >> 3;
  for (int64_t j = threadIdx.x; j < head; j += kBlock) d[j] = 0;
  u32x4* dv = reinterpret_cast<u32x4*>(d + head);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t j = threadIdx.x; j < nv; j += kBlock) st_stream(dv + j, z);
  for (int64_t t = head + 8 * nv + threadIdx.x; t < len; t += kBlock) d[t] = 0;
}

// Workgroup b writes shard elements [b·per_block, (b+1)·per_block): it finds
// the first descriptor that ends past its start by binary search, then walks
// the descriptors in order, copying covered pieces and zero-filling gaps.
// With ACC it also leaves its partial square-sum and non-finite flag in
// part_sum[b] / part_bad[b] (padding contributes +0).
// Capped at 4 wavefronts per SIMD.  The fused form (ACC) holds no more by its
// registers anyway; the plain copy (44 registers, 8 wavefronts otherwise)
// copies 1 GiB and 4 GiB 3% and 5% faster with the cap on MI355X, and the
// unfused steps of the GPT-2 1.5B and Llama-7B rank shards run 0.2% and 0.7%
// faster.
template <int DT, bool ACC>
STREAMING_KERNEL void flatten_kernel(const zero_flat_seg* __restrict__ segs, int32_t n_segs,
                                     uint16_t* __restrict__ shard, int64_t shard_numel, int64_t per_block,
                                     double* __restrict__ part_sum, uint32_t* __restrict__ part_bad) {
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per_block;
  const int64_t hi = lo + per_block < shard_numel ? lo + per_block : shard_numel;
  int32_t a = 0, b = n_segs;
  while (a < b) {
    const int32_t mid = (a + b) >> 1;
    if (segs[mid].dst_offset + segs[mid].numel > lo) {
      b = mid;
    } else {
      a = mid + 1;
    }
  }
  double acc = 0.0;
  uint32_t bad = 0;
  int32_t k = a;
  int64_t pos = lo;
  while (pos < hi) {
    if (k < n_segs && segs[k].dst_offset <= pos) {
      const zero_flat_seg sg = segs[k];
      int64_t end = sg.dst_offset + sg.numel;
      if (end > hi) end = hi;
      if (end > pos) {
        const uint16_t* src = static_cast<const uint16_t*>(sg.src) + (sg.src_offset + (pos - sg.dst_offset));
        copy_piece<DT, ACC>(src, shard + pos, end - pos, acc, bad);
        pos = end;
      }
      ++k;
    } else {
      int64_t end = hi;
      if (k < n_segs && segs[k].dst_offset < end) end = segs[k].dst_offset;
      zero_piece(shard + pos, end - pos);
      pos = end;
    }
  }
  if (ACC) {
    block_reduce(acc, bad);
    if (threadIdx.x == 0) {
      part_sum[blockIdx.x] = acc;
      part_bad[blockIdx.x] = bad;
    }
  }
}

// Every flatten workgroup owns 8192 shard elements (one pass of four 16-byte
// vectors per thread).  Measured on MI355X against a fixed grid of 4096
// workgroups with longer ranges: the Llama-13B rank shard (3.25e9 elements)
// flattens at 5.6-5.7 instead of 5.1 TB/s, the GPT-2 1.5B one at the same
// rate, and the whole step gains 0.7-2%.  Past 2^19 workgroups (inputs above
// 4.3e9 elements) the ranges grow instead, which bounds the partials (the
// norm workspace) at 6 MiB.
constexpr int64_t kFlattenPer = 8192, kFlattenMaxBlocks = int64_t(1) << 19;
int64_t flatten_per_block(int64_t n) {
  int64_t per = ceil_div(n, kFlattenMaxBlocks);
  per = ceil_div(per, kFlattenPer) * kFlattenPer;
  return per < kFlattenPer ? kFlattenPer : per;
}

bool dtype_ok(int dt) { return dt == ZERO_BF16 || dt == ZERO_FP16; }

// Validates the arguments shared by both AdamW entry points and derives the
// fp32 scalars from fp64 host arithmetic (each rounded once).
int adam_args_ok(const char* fn, const void* grad_dev, int gdt, const void* param_dev, int pdt, int64_t n,
                 const zero_adamw_hparams* hp, AdamScalars* s) {
  if (!dtype_ok(gdt)) return fail(ZERO_ERR_INVALID, "%s: unknown dtype %d", fn, gdt);
  if (!dtype_ok(pdt)) return fail(ZERO_ERR_INVALID, "%s: unknown parameter dtype %d", fn, pdt);
  if (!hp) return fail(ZERO_ERR_INVALID, "%s: hparams NULL", fn);
  if (n < 0 || n > kMaxPsi) return fail(ZERO_ERR_INVALID, "%s: n = %lld out of range", fn, static_cast<long long>(n));
  if (n > 0 && (!grad_dev || !param_dev)) return fail(ZERO_ERR_INVALID, "%s: NULL grad or param", fn);
  if (hp->step < 1 || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) ||
      !(hp->eps >= 0.0) || !(hp->lr >= 0.0) || !(hp->weight_decay >= 0.0) || !std::isfinite(hp->grad_scale) ||
      !std::isfinite(hp->lr))
    return fail(ZERO_ERR_INVALID, "%s: hyper-parameters out of range", fn);
  if (((reinterpret_cast<uintptr_t>(grad_dev) | reinterpret_cast<uintptr_t>(param_dev)) & 1u) != 0)
    return fail(ZERO_ERR_INVALID, "%s: 16-bit buffers not 2-byte aligned", fn);
  const double t = static_cast<double>(hp->step);
  const double bc1 = 1.0 - std::pow(hp->beta1, t);
  const double bc2 = 1.0 - std::pow(hp->beta2, t);
  s->b1 = static_cast<float>(hp->beta1);
  s->omb1 = static_cast<float>(1.0 - hp->beta1);
  s->b2 = static_cast<float>(hp->beta2);
  s->omb2 = static_cast<float>(1.0 - hp->beta2);
  s->eps = static_cast<float>(hp->eps);
  s->decay = static_cast<float>(1.0 - hp->lr * hp->weight_decay);
  s->step_size = static_cast<float>(hp->lr / bc1);
  s->bc2_sqrt = static_cast<float>(std::sqrt(bc2));
  s->gscale = static_cast<float>(hp->grad_scale);
  return ZERO_OK;
}

// The update is issued in launches of at most 2^25 elements (32768 tiles).
// Measured on MI355X (tiled state, bf16): one launch over a 3.25e9-element
// shard sustains 5.58 TB/s and over a 1.95e8-element shard 6.10 TB/s, while
// launches of 2^24 / 2^25 / 2^26 / 2^27 elements give 6.32 / 6.39 / 6.33 /
// 6.20 TB/s at every shard size.  Over a long grid the workgroups of the
// eight XCDs drift apart in the address space; a launch boundary brings
// them back together at the cost of one drain.
constexpr int64_t kUpdateElemsPerLaunch = int64_t(1) << 25;
static_assert(kUpdateElemsPerLaunch % kTile == 0 && kUpdateElemsPerLaunch % (4 * kBlock * kAdamUnroll) == 0,
              "launches cover whole tiles / whole workgroups");

// Calls f(Formats<G, P>{}) for the run-time (gradient, parameter) format pair,
// so each launcher names its kernel template once.
template <int G, int P>
struct Formats {
  static constexpr int grad = G, param = P;
};
template <typename F>
void with_formats(int gdt, int pdt, F&& f) {
  if (gdt == ZERO_BF16) {
    if (pdt == ZERO_BF16) f(Formats<ZERO_BF16, ZERO_BF16>{}); else f(Formats<ZERO_BF16, ZERO_FP16>{});
  } else {
    if (pdt == ZERO_BF16) f(Formats<ZERO_FP16, ZERO_BF16>{}); else f(Formats<ZERO_FP16, ZERO_FP16>{});
  }
}

template <bool TILED>
int launch_elements(const uint16_t* grad, int gdt, float* master, float* m, float* v, uint16_t* param, int pdt,
                    int64_t begin, int64_t n, const AdamScalars& s, const zero_step_state* dev, hipStream_t st,
                    const char* what) {
  if (begin >= n) return ZERO_OK;
  const int64_t blocks = std::min<int64_t>(ceil_div(n - begin, kBlock), 65536);
  with_formats(gdt, pdt, [&](auto fm) {
    using FM = decltype(fm);
    hipLaunchKernelGGL((adamw_element_kernel<FM::grad, FM::param, TILED>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kBlock), 0, st, grad, master, m, v, param, begin, n, s, dev);
  });
  return launch_status(what);
}

int launch_adamw_arrays(const char* fn, const void* grad_dev, int gdt, float* master_dev, float* m_dev, float* v_dev,
                        uint16_t* param_dev, int pdt, int64_t n, const AdamScalars& s, const zero_step_state* dev,
                        hipStream_t st) {
  if (n > 0 && (!master_dev || !m_dev || !v_dev)) return fail(ZERO_ERR_INVALID, "%s: NULL state", fn);
  if (!fp32_aligned(master_dev, m_dev, v_dev, nullptr))
    return fail(ZERO_ERR_INVALID, "%s: fp32 buffers not 4-byte aligned", fn);
  if (n == 0) return ZERO_OK;
  const uint16_t* g = static_cast<const uint16_t*>(grad_dev);
  const bool vec = aligned8(grad_dev) && aligned8(param_dev) && aligned16(master_dev) && aligned16(m_dev) &&
                   aligned16(v_dev);
  if (!vec) return launch_elements<false>(g, gdt, master_dev, m_dev, v_dev, param_dev, pdt, 0, n, s, dev, st, fn);
  constexpr int64_t per = kBlock * kAdamUnroll;
  const int64_t groups = (n + 3) / 4;  // the last one may be partial
  const int64_t blocks = ceil_div(groups, per);
  constexpr int64_t kBlocksPerLaunch = kUpdateElemsPerLaunch / (4 * per);
  for (int64_t b0 = 0; b0 < blocks; b0 += kBlocksPerLaunch) {
    const int64_t cnt = std::min(kBlocksPerLaunch, blocks - b0);
    with_formats(gdt, pdt, [&](auto fm) {
      using FM = decltype(fm);
      hipLaunchKernelGGL((adamw_vec_kernel<FM::grad, FM::param, kAdamUnroll>), dim3(static_cast<unsigned>(cnt)),
                         dim3(kBlock), 0, st, g, master_dev, m_dev, v_dev, param_dev, n, b0, s, dev);
    });
    const int rc = launch_status(fn);
    if (rc != ZERO_OK) return rc;
  }
  return ZERO_OK;
}

// Issues launch(t0, count) for each launch of the tiled update over n
// elements: count tiles from tile t0, at most kUpdateElemsPerLaunch elements.
template <typename F>
int for_each_tiled_launch(int64_t n, const char* fn, F&& launch) {
  const int64_t tiles = ceil_div(n, kTile);
  constexpr int64_t kTilesPerLaunch = kUpdateElemsPerLaunch / kTile;
  for (int64_t t0 = 0; t0 < tiles; t0 += kTilesPerLaunch) {
    launch(t0, std::min(kTilesPerLaunch, tiles - t0));
    const int rc = launch_status(fn);
    if (rc != ZERO_OK) return rc;
  }
  return ZERO_OK;
}

int launch_adamw_tiled(const char* fn, const void* grad_dev, int gdt, float* state_dev, uint16_t* param_dev, int pdt,
                       int64_t n, const AdamScalars& s, const zero_step_state* dev, hipStream_t st) {
  if (n > 0 && !state_dev) return fail(ZERO_ERR_INVALID, "%s: NULL state", fn);
  if (!aligned16(state_dev)) return fail(ZERO_ERR_INVALID, "%s: state must be 16-byte aligned", fn);
  if (n == 0) return ZERO_OK;
  const uint16_t* g = static_cast<const uint16_t*>(grad_dev);
  if (!aligned8(grad_dev) || !aligned8(param_dev))
    return launch_elements<true>(g, gdt, state_dev, state_dev, state_dev, param_dev, pdt, 0, n, s, dev, st, fn);
  auto* state = reinterpret_cast<f32x4*>(state_dev);
  return for_each_tiled_launch(n, fn, [&](int64_t t0, int64_t cnt) {
    with_formats(gdt, pdt, [&](auto fm) {
      using FM = decltype(fm);
      hipLaunchKernelGGL((adamw_tiled_kernel<FM::grad, FM::param>), dim3(static_cast<unsigned>(cnt)), dim3(kBlock), 0,
                         st, g, state, param_dev, n, t0, s, dev);
    });
  });
}

int dev_args_ok(const char* fn, const void* grad_dev, int gdt, const void* param_dev, int pdt, int64_t n,
                const zero_step_state* dev) {
  if (!dtype_ok(gdt)) return fail(ZERO_ERR_INVALID, "%s: unknown dtype %d", fn, gdt);
  if (!dtype_ok(pdt)) return fail(ZERO_ERR_INVALID, "%s: unknown parameter dtype %d", fn, pdt);
  if (!dev || !aligned16(dev)) return fail(ZERO_ERR_INVALID, "%s: step state NULL or not 16-byte aligned", fn);
  if (n < 0 || n > kMaxPsi) return fail(ZERO_ERR_INVALID, "%s: n = %lld out of range", fn, static_cast<long long>(n));
  if (n > 0 && (!grad_dev || !param_dev)) return fail(ZERO_ERR_INVALID, "%s: NULL grad or param", fn);
  if (((reinterpret_cast<uintptr_t>(grad_dev) | reinterpret_cast<uintptr_t>(param_dev)) & 1u) != 0)
    return fail(ZERO_ERR_INVALID, "%s: 16-bit buffers not 2-byte aligned", fn);
  return ZERO_OK;
}

__global__ void step_state_init_kernel(zero_step_state* st, double loss_scale, int32_t growth_interval) {
  if (threadIdx.x != 0) return;
  st->loss_scale = loss_scale;
  st->global_norm = 0.0;
  st->grad_scale = 0.0;
  st->adam_step = 0;
  st->iteration = 0;
  st->good_steps = 0;
  st->growth_interval = growth_interval;
  st->skip = 1;  // nothing decided yet: an update launched now does nothing
  st->error = 0;
  for (int k = 0; k < 12; ++k) st->scalars[k] = 0.0f;
}

// The host decision (zero_step_decision) and scalar derivation (adam_args_ok)
// on one thread, operation for operation.
__global__ void step_decision_kernel(const double* __restrict__ sq, const int32_t* __restrict__ flags, int32_t n_ranks,
                                     double max_norm, double lr, double beta1, double beta2, double eps, double wd,
                                     zero_step_state* __restrict__ st) {
  if (threadIdx.x != 0) return;
  double global = 0.0;
  bool overflow = false;
  for (int32_t r = 0; r < n_ranks; ++r) {
    global += sq[r];
    overflow = overflow || flags[r] != 0;
  }
  const double scale = st->loss_scale;
  st->iteration += 1;
  // The host decision refuses these cases with ZERO_ERR_INVALID; here the
  // step is skipped, the error recorded, and the scale, good-step count and
  // Adam t are left as they are.
  const double unscaled = global / (scale * scale);
  if (!(scale > 0.0) || !isfinite(scale) || (!overflow && !isfinite(unscaled))) {
    st->skip = 1;
    st->error = ZERO_STEP_ERR_LOSS_SCALE;
    st->grad_scale = 0.0;
    st->global_norm = __builtin_nan("");
    return;
  }
  st->error = 0;
  if (overflow) {
    st->skip = 1;
    st->grad_scale = 0.0;
    st->global_norm = __builtin_nan("");
    st->loss_scale = scale * 0.5;
    st->good_steps = 0;
    return;
  }
  double coef = 1.0;
  if (max_norm > 0.0) {
    const double c = max_norm / (sqrt(unscaled) + 1e-6);
    coef = c < 1.0 ? c : 1.0;
  }
  const double gscale = coef / scale;
  int32_t good = st->good_steps + 1;
  double new_scale = scale;
  if (good >= st->growth_interval) {
    new_scale = scale * 2.0;
    good = 0;
  }
  const int64_t t = st->adam_step + 1;
  const double bc1 = 1.0 - pow(beta1, static_cast<double>(t));
  const double bc2 = 1.0 - pow(beta2, static_cast<double>(t));
  st->skip = 0;
  st->grad_scale = gscale;
  st->global_norm = sqrt(unscaled);
  st->loss_scale = new_scale;
  st->good_steps = good;
  st->adam_step = t;
  st->scalars[0] = static_cast<float>(beta1);
  st->scalars[1] = static_cast<float>(1.0 - beta1);
  st->scalars[2] = static_cast<float>(beta2);
  st->scalars[3] = static_cast<float>(1.0 - beta2);
  st->scalars[4] = static_cast<float>(eps);
  st->scalars[5] = static_cast<float>(1.0 - lr * wd);
  st->scalars[6] = static_cast<float>(lr / bc1);
  st->scalars[7] = static_cast<float>(sqrt(bc2));
  st->scalars[8] = static_cast<float>(gscale);
}

int flatten_args_ok(const char* fn, const zero_flat_seg* segs_dev, int32_t n_segs, int dt, const void* shard_dev,
                    int64_t shard_numel) {
  if (!dtype_ok(dt)) return fail(ZERO_ERR_INVALID, "%s: unknown dtype %d", fn, dt);
  if (n_segs < 0 || (n_segs > 0 && !segs_dev))
    return fail(ZERO_ERR_INVALID, "%s: bad segment table (n_segs=%d)", fn, n_segs);
  if (shard_numel < 0 || shard_numel > kMaxPsi || (shard_numel > 0 && !shard_dev))
    return fail(ZERO_ERR_INVALID, "%s: bad shard (numel=%lld)", fn, static_cast<long long>(shard_numel));
  if ((reinterpret_cast<uintptr_t>(shard_dev) & 1u) != 0)
    return fail(ZERO_ERR_INVALID, "%s: shard must be 2-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(segs_dev) & 7u) != 0)
    return fail(ZERO_ERR_INVALID, "%s: segment table must be 8-byte aligned", fn);
  return ZERO_OK;
}

// The fused flatten with its per-workgroup partial square-sums and flags
// written to part_sum[0 .. blocks) / part_bad[0 .. blocks).
int launch_flatten_partials(const char* fn, const zero_flat_seg* segs_dev, int32_t n_segs, int dt, void* dst_dev,
                            int64_t numel, double* part_sum, uint32_t* part_bad, hipStream_t st) {
  if (numel <= 0) return ZERO_OK;
  const int64_t per = flatten_per_block(numel);
  const int64_t blocks = ceil_div(numel, per);
  if (dt == ZERO_BF16) {
    hipLaunchKernelGGL((flatten_kernel<ZERO_BF16, true>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, st,
                       segs_dev, n_segs, static_cast<uint16_t*>(dst_dev), numel, per, part_sum, part_bad);
  } else {
    hipLaunchKernelGGL((flatten_kernel<ZERO_FP16, true>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, st,
                       segs_dev, n_segs, static_cast<uint16_t*>(dst_dev), numel, per, part_sum, part_bad);
  }
  return launch_status(fn);
}

// Folds `parts` partials (overwriting them when it takes two levels) into
// *out_sum and *out_bad.
int launch_fold(const char* fn, double* part_sum, uint32_t* part_bad, int64_t parts, double* out_sum,
                int32_t* out_bad, hipStream_t st) {
  int64_t count = parts, stride = 1;
  if (parts > kFoldTwoLevel) {
    const int64_t chunks = ceil_div(parts, kFoldChunk);
    hipLaunchKernelGGL(sqnorm_fold_chunks_kernel, dim3(static_cast<unsigned>(chunks)), dim3(kBlock), 0, st, part_sum,
                       part_bad, parts);
    const int rc = launch_status(fn);
    if (rc != ZERO_OK) return rc;
    count = chunks;
    stride = kFoldChunk;
  }
  hipLaunchKernelGGL(sqnorm_final_kernel, dim3(1), dim3(kFoldThreads), 0, st, part_sum, part_bad, count, stride,
                     out_sum, out_bad);
  return launch_status(fn);
}

int norm_outputs_ok(const char* fn, int64_t n, const void* ws_dev, size_t ws_bytes, const double* sqnorm_dev,
                    const int32_t* nonfinite_dev) {
  if (!sqnorm_dev || !nonfinite_dev || !ws_dev) return fail(ZERO_ERR_INVALID, "%s: NULL output or workspace", fn);
  if (!aligned16(ws_dev)) return fail(ZERO_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
  const size_t need = zero_grad_sqnorm_workspace_bytes(n);
  if (ws_bytes < need) return fail(ZERO_ERR_INVALID, "%s: workspace %zu bytes < %zu", fn, ws_bytes, need);
  return ZERO_OK;
}

// The fused flatten and its fold, with the partials in ws_dev (validated by
// the caller to hold zero_grad_sqnorm_workspace_bytes(shard_numel) bytes).
int flatten_sqnorm_into(const char* fn, const zero_flat_seg* segs_dev, int32_t n_segs, int dt, void* shard_dev,
                        int64_t shard_numel, void* ws_dev, double* sqnorm_dev, int32_t* nonfinite_dev,
                        hipStream_t st) {
  const int64_t blocks = zero_flatten_partials_count(shard_numel);
  double* part_sum = static_cast<double*>(ws_dev);
  uint32_t* part_bad = reinterpret_cast<uint32_t*>(part_sum + (blocks > 0 ? blocks : 1));
  int rc = launch_flatten_partials(fn, segs_dev, n_segs, dt, shard_dev, shard_numel, part_sum, part_bad, st);
  if (rc != ZERO_OK) return rc;
  return launch_fold(fn, part_sum, part_bad, blocks, sqnorm_dev, nonfinite_dev, st);
}

}  // namespace

// ------------------------------------------------------------------ static scratch
//
// For callers that cannot allocate: the partials of the fused flatten + norm
// live in this file-scope array instead of a caller workspace.  Its size is
// the largest workspace the fused flatten ever needs (2^19 partials of 12
// bytes), so every shard size fits.  Every GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` only names the
// variable: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
constexpr size_t kStaticScratchBytes = ZERO_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kScratchMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device.  The stream (if any) must belong to that device.
int static_scratch(const char* fn, hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ZERO_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchMaxDevices)
    return fail(ZERO_ERR_INVALID, "%s: device %d outside the %d devices the scratch table covers", fn, dev,
                kScratchMaxDevices);
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(ZERO_ERR_HIP, "%s: hipStreamGetDevice failed: %s", fn, hipGetErrorString(e));
    if (sdev != dev)
      return fail(ZERO_ERR_INVALID, "%s: the stream belongs to device %d, the current device is %d", fn,
                  static_cast<int>(sdev), dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(ZERO_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return ZERO_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

const char* zero_last_error(void) { return g_last_error; }

int zero_shard_layout(const int64_t* numels, int32_t n_tensors, int32_t world, int32_t rank, zero_layout* out,
                      zero_segment* segs, int32_t segs_cap, int32_t* n_segs) {
  if (!out || !n_segs) return fail(ZERO_ERR_INVALID, "zero_shard_layout: out and n_segs must not be NULL");
  if (n_tensors < 0 || (n_tensors > 0 && !numels))
    return fail(ZERO_ERR_INVALID, "zero_shard_layout: bad tensor list (n_tensors=%d)", n_tensors);
  if (world < 1 || rank < 0 || rank >= world)
    return fail(ZERO_ERR_INVALID, "zero_shard_layout: rank %d outside world %d", rank, world);
  if (segs_cap < 0 || (segs_cap > 0 && !segs))
    return fail(ZERO_ERR_INVALID, "zero_shard_layout: bad segment array (cap=%d)", segs_cap);
  int64_t psi = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    if (numels[t] < 0 || numels[t] > kMaxPsi - psi)
      return fail(ZERO_ERR_INVALID, "zero_shard_layout: tensor %d numel %lld invalid or total too large", t,
                  static_cast<long long>(numels[t]));
    psi += numels[t];
  }
  const int64_t shard = ceil_div(psi, world);
  const int64_t begin = static_cast<int64_t>(rank) * shard;
  const int64_t stop = begin + shard < psi ? begin + shard : psi;  // end of real (unpadded) elements
  zero_layout L{};
  L.psi = psi;
  L.padded_numel = static_cast<int64_t>(world) * shard;
  L.shard_numel = shard;
  L.shard_offset = begin;
  L.shard_valid = stop > begin ? stop - begin : 0;
  L.world = world;
  L.rank = rank;
  L.bytes_dp = 16 * psi;                                   // 2 param + 2 grad + 12 optimizer, all replicated
  L.bytes_zero1 = (2 + 2) * L.padded_numel + 12 * shard;   // optimizer state partitioned
  L.bytes_zero2 = 2 * L.padded_numel + (2 + 12) * shard;   // + gradients partitioned
  L.bytes_zero3 = (2 + 2 + 12) * shard;                    // + parameters partitioned
  const int64_t ring = static_cast<int64_t>(world - 1) * shard;  // one ring RS or AG, sent per rank
  L.comm_dp = 2 * ring;     // gradient all-reduce = RS + AG
  L.comm_zero1 = 2 * ring;  // gradient RS + parameter AG
  L.comm_zero2 = 2 * ring;
  L.comm_zero3 = 3 * ring;  // + a second parameter AG (forward and backward each gather)
  *out = L;

  int32_t count = 0;
  int64_t t_begin = 0;
  for (int32_t t = 0; t < n_tensors && t_begin < stop; ++t) {
    const int64_t t_end = t_begin + numels[t];
    const int64_t a = t_begin > begin ? t_begin : begin;
    const int64_t b = t_end < stop ? t_end : stop;
    if (b > a) {
      if (count < segs_cap) segs[count] = zero_segment{t, 0, a - t_begin, a - begin, b - a};
      ++count;
    }
    t_begin = t_end;
  }
  *n_segs = count;
  if (count > segs_cap)
    return fail(ZERO_ERR_CAPACITY, "zero_shard_layout: %d segments needed, capacity %d", count, segs_cap);
  return ZERO_OK;
}

int zero_flatten_plan(const zero_segment* segs, int32_t n_segs, const void* const* tensor_ptrs, int32_t n_tensors,
                      zero_flat_seg* out) {
  if (n_segs < 0 || (n_segs > 0 && (!segs || !tensor_ptrs || !out)))
    return fail(ZERO_ERR_INVALID, "zero_flatten_plan: NULL argument");
  for (int32_t k = 0; k < n_segs; ++k) {
    const zero_segment& s = segs[k];
    if (s.tensor < 0 || s.tensor >= n_tensors || !tensor_ptrs[s.tensor] || s.numel <= 0 || s.src_offset < 0 ||
        s.dst_offset < 0)
      return fail(ZERO_ERR_INVALID, "zero_flatten_plan: segment %d is invalid", k);
    out[k] = zero_flat_seg{tensor_ptrs[s.tensor], s.src_offset, s.dst_offset, s.numel};
  }
  return ZERO_OK;
}

int zero_bucket_segments(const zero_segment* segs, int32_t n_segs, int64_t win_begin, int64_t win_numel,
                         zero_segment* out, int32_t cap, int32_t* n_out) {
  if (n_segs < 0 || (n_segs > 0 && !segs) || win_begin < 0 || win_numel < 0 || cap < 0 || (cap > 0 && !out) ||
      !n_out || win_numel > kMaxPsi - win_begin)
    return fail(ZERO_ERR_INVALID, "zero_bucket_segments: bad arguments");
  const int64_t win_end = win_begin + win_numel;
  int32_t count = 0;
  for (int32_t k = 0; k < n_segs; ++k) {
    const zero_segment& sg = segs[k];
    const int64_t a = sg.dst_offset > win_begin ? sg.dst_offset : win_begin;
    const int64_t e = sg.dst_offset + sg.numel;
    const int64_t b = e < win_end ? e : win_end;
    if (b <= a) continue;
    if (count < cap) out[count] = zero_segment{sg.tensor, 0, sg.src_offset + (a - sg.dst_offset), a - win_begin, b - a};
    ++count;
  }
  *n_out = count;
  if (count > cap) return fail(ZERO_ERR_CAPACITY, "zero_bucket_segments: %d segments needed, capacity %d", count, cap);
  return ZERO_OK;
}

int zero_flatten_grads(const zero_flat_seg* segs_dev, int32_t n_segs, zero_dtype dt, void* shard_dev,
                       int64_t shard_numel, void* stream) {
  int rc = flatten_args_ok("zero_flatten_grads", segs_dev, n_segs, dt, shard_dev, shard_numel);
  if (rc != ZERO_OK || shard_numel == 0) return rc;
  const int64_t per = flatten_per_block(shard_numel);
  const int64_t blocks = ceil_div(shard_numel, per);
  hipLaunchKernelGGL((flatten_kernel<ZERO_BF16, false>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), segs_dev, n_segs, static_cast<uint16_t*>(shard_dev),
                     shard_numel, per, nullptr, nullptr);
  return launch_status("zero_flatten_grads");
}

int zero_flatten_grads_sqnorm(const zero_flat_seg* segs_dev, int32_t n_segs, zero_dtype dt, void* shard_dev,
                              int64_t shard_numel, void* ws_dev, size_t ws_bytes, double* sqnorm_dev,
                              int32_t* nonfinite_dev, void* stream) {
  int rc = flatten_args_ok("zero_flatten_grads_sqnorm", segs_dev, n_segs, dt, shard_dev, shard_numel);
  if (rc != ZERO_OK) return rc;
  rc = norm_outputs_ok("zero_flatten_grads_sqnorm", shard_numel, ws_dev, ws_bytes, sqnorm_dev, nonfinite_dev);
  if (rc != ZERO_OK) return rc;
  return flatten_sqnorm_into("zero_flatten_grads_sqnorm", segs_dev, n_segs, dt, shard_dev, shard_numel, ws_dev,
                             sqnorm_dev, nonfinite_dev, static_cast<hipStream_t>(stream));
}

int zero_flatten_grads_sqnorm_noalloc(const zero_flat_seg* segs_dev, int32_t n_segs, zero_dtype dt, void* shard_dev,
                                      int64_t shard_numel, double* sqnorm_dev, int32_t* nonfinite_dev, void* stream) {
  const char* fn = "zero_flatten_grads_sqnorm_noalloc";
  int rc = flatten_args_ok(fn, segs_dev, n_segs, dt, shard_dev, shard_numel);
  if (rc != ZERO_OK) return rc;
  if (!sqnorm_dev || !nonfinite_dev || !aligned8(sqnorm_dev) || (reinterpret_cast<uintptr_t>(nonfinite_dev) & 3u))
    return fail(ZERO_ERR_INVALID, "%s: outputs NULL or misaligned", fn);
  const size_t need = zero_grad_sqnorm_workspace_bytes(shard_numel);
  if (need > kStaticScratchBytes)
    return fail(ZERO_ERR_CAPACITY, "%s: a shard of %lld elements needs %zu bytes of scratch, the static scratch holds %zu",
                fn, static_cast<long long>(shard_numel), need, kStaticScratchBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  rc = static_scratch(fn, st, &ws);
  if (rc != ZERO_OK) return rc;
  return flatten_sqnorm_into(fn, segs_dev, n_segs, dt, shard_dev, shard_numel, ws, sqnorm_dev, nonfinite_dev, st);
}

int64_t zero_flatten_partials_count(int64_t numel) {
  if (numel <= 0) return 0;
  const int64_t per = flatten_per_block(numel);
  return ceil_div(numel, per);
}

int zero_flatten_grads_partials(const zero_flat_seg* segs_dev, int32_t n_segs, zero_dtype dt, void* dst_dev,
                                int64_t numel, double* part_sum_dev, uint32_t* part_flag_dev, void* stream) {
  int rc = flatten_args_ok("zero_flatten_grads_partials", segs_dev, n_segs, dt, dst_dev, numel);
  if (rc != ZERO_OK) return rc;
  if (numel > 0 && (!part_sum_dev || !part_flag_dev || !aligned8(part_sum_dev) ||
                    (reinterpret_cast<uintptr_t>(part_flag_dev) & 3u) != 0))
    return fail(ZERO_ERR_INVALID, "zero_flatten_grads_partials: partial outputs NULL or misaligned");
  return launch_flatten_partials("zero_flatten_grads_partials", segs_dev, n_segs, dt, dst_dev, numel, part_sum_dev,
                                 part_flag_dev, static_cast<hipStream_t>(stream));
}

int zero_sqnorm_reduce(double* part_sum_dev, uint32_t* part_flag_dev, int64_t count, double* sqnorm_dev,
                       int32_t* nonfinite_dev, void* stream) {
  if (count < 0 || count > kMaxPsi || (count > 0 && (!part_sum_dev || !part_flag_dev)) || !sqnorm_dev ||
      !nonfinite_dev || !aligned8(sqnorm_dev) || (reinterpret_cast<uintptr_t>(nonfinite_dev) & 3u) != 0 ||
      (count > 0 && (!aligned8(part_sum_dev) || (reinterpret_cast<uintptr_t>(part_flag_dev) & 3u) != 0)))
    return fail(ZERO_ERR_INVALID, "zero_sqnorm_reduce: bad arguments");
  return launch_fold("zero_sqnorm_reduce", part_sum_dev, part_flag_dev, count, sqnorm_dev, nonfinite_dev,
                     static_cast<hipStream_t>(stream));
}

size_t zero_grad_sqnorm_workspace_bytes(int64_t n) {
  if (n < 0) n = 0;
  int64_t parts = norm_parts(n);
  const int64_t fl = n > 0 ? ceil_div(n, flatten_per_block(n)) : 1;
  if (fl > parts) parts = fl;
  const size_t bytes = static_cast<size_t>(parts) * (sizeof(double) + sizeof(uint32_t));
  return (bytes + 255) / 256 * 256;
}

int zero_grad_sqnorm(const void* shard_dev, zero_dtype dt, int64_t n, void* ws_dev, size_t ws_bytes,
                     double* sqnorm_dev, int32_t* nonfinite_dev, void* stream) {
  if (!dtype_ok(dt)) return fail(ZERO_ERR_INVALID, "zero_grad_sqnorm: unknown dtype %d", static_cast<int>(dt));
  if (n < 0 || n > kMaxPsi || (n > 0 && !shard_dev)) return fail(ZERO_ERR_INVALID, "zero_grad_sqnorm: bad shard");
  if ((reinterpret_cast<uintptr_t>(shard_dev) & 1u) != 0)
    return fail(ZERO_ERR_INVALID, "zero_grad_sqnorm: shard must be 2-byte aligned");
  int rc = norm_outputs_ok("zero_grad_sqnorm", n, ws_dev, ws_bytes, sqnorm_dev, nonfinite_dev);
  if (rc != ZERO_OK) return rc;
  const int64_t parts = norm_parts(n);
  const uint16_t* x = static_cast<const uint16_t*>(shard_dev);
  int64_t head = static_cast<int64_t>(((16u - (reinterpret_cast<uintptr_t>(x) & 15u)) & 15u) >> 1);
  if (head > n) head = n;
  const int64_t n8 = (n - head) >> 3;
  int64_t per = ceil_div(n8, parts);
  if (per < 1) per = 1;
  double* part_sum = static_cast<double*>(ws_dev);
  uint32_t* part_bad = reinterpret_cast<uint32_t*>(part_sum + parts);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == ZERO_BF16) {
    hipLaunchKernelGGL(sqnorm_partial_kernel<ZERO_BF16>, dim3(static_cast<unsigned>(parts)), dim3(kBlock), 0, st, x,
                       n, head, n8, per, part_sum, part_bad);
  } else {
    hipLaunchKernelGGL(sqnorm_partial_kernel<ZERO_FP16>, dim3(static_cast<unsigned>(parts)), dim3(kBlock), 0, st, x,
                       n, head, n8, per, part_sum, part_bad);
  }
  rc = launch_status("zero_grad_sqnorm (partials)");
  if (rc != ZERO_OK) return rc;
  return launch_fold("zero_grad_sqnorm (fold)", part_sum, part_bad, parts, sqnorm_dev, nonfinite_dev, st);
}

double zero_clip_coef(double global_sqnorm, double max_norm) {
  if (!(max_norm > 0.0)) return 1.0;
  const double coef = max_norm / (std::sqrt(global_sqnorm) + 1e-6);
  return coef < 1.0 ? coef : 1.0;
}

int zero_loss_scale_update(double* scale, int32_t nonfinite, int32_t* good_steps, int32_t growth_interval) {
  if (!scale || !good_steps || growth_interval < 1)
    return fail(ZERO_ERR_INVALID, "zero_loss_scale_update: bad arguments");
  if (nonfinite) {
    *scale *= 0.5;
    *good_steps = 0;
    return ZERO_OK;
  }
  if (++*good_steps >= growth_interval) {
    *scale *= 2.0;
    *good_steps = 0;
  }
  return ZERO_OK;
}

int zero_step_decision(const double* rank_sqnorms, const int32_t* rank_flags, int32_t n_ranks, double max_norm,
                       double* loss_scale, int32_t* good_steps, int32_t growth_interval, double* grad_scale,
                       int32_t* skip, double* global_norm) {
  if (n_ranks < 1 || !rank_sqnorms || !rank_flags || !loss_scale || !good_steps || !grad_scale || !skip ||
      !global_norm || growth_interval < 1 || !(*loss_scale > 0.0))
    return fail(ZERO_ERR_INVALID, "zero_step_decision: bad arguments");
  double global = 0.0;
  bool overflow = false;
  for (int32_t r = 0; r < n_ranks; ++r) {  // the all-reduce, in rank order
    global += rank_sqnorms[r];
    overflow = overflow || rank_flags[r] != 0;
  }
  const double scale = *loss_scale;
  const double unscaled = global / (scale * scale);
  if (!std::isfinite(scale) || (!overflow && !std::isfinite(unscaled)))
    return fail(ZERO_ERR_INVALID, "zero_step_decision: loss scale %g is not usable (the unscaled square-norm is %g)",
                scale, unscaled);
  if (overflow) {
    *skip = 1;
    *grad_scale = 0.0;
    *global_norm = std::numeric_limits<double>::quiet_NaN();
  } else {
    *skip = 0;
    *grad_scale = zero_clip_coef(unscaled, max_norm) / scale;
    *global_norm = std::sqrt(unscaled);
  }
  return zero_loss_scale_update(loss_scale, overflow ? 1 : 0, good_steps, growth_interval);
}

double zero_cosine_lr(int64_t t, int64_t total, double lr_max, double lr_min) {
  if (total <= 1) return lr_max;
  const double frac = static_cast<double>(t - 1) / static_cast<double>(total - 1);
  return lr_min + 0.5 * (lr_max - lr_min) * (1.0 + std::cos(M_PI * frac));
}

int zero_adamw_step(const void* grad_dev, zero_dtype gdt, float* master_dev, float* m_dev, float* v_dev,
                    uint16_t* param_dev, zero_dtype pdt, int64_t n, const zero_adamw_hparams* hp, void* stream) {
  AdamScalars s;
  int rc = adam_args_ok("zero_adamw_step", grad_dev, gdt, param_dev, pdt, n, hp, &s);
  if (rc != ZERO_OK) return rc;
  return launch_adamw_arrays("zero_adamw_step", grad_dev, gdt, master_dev, m_dev, v_dev, param_dev, pdt, n, s,
                             nullptr, static_cast<hipStream_t>(stream));
}

int zero_adamw_step_dev(const void* grad_dev, zero_dtype gdt, float* master_dev, float* m_dev, float* v_dev,
                        uint16_t* param_dev, zero_dtype pdt, int64_t n, const zero_step_state* state_dev,
                        void* stream) {
  int rc = dev_args_ok("zero_adamw_step_dev", grad_dev, gdt, param_dev, pdt, n, state_dev);
  if (rc != ZERO_OK) return rc;
  return launch_adamw_arrays("zero_adamw_step_dev", grad_dev, gdt, master_dev, m_dev, v_dev, param_dev, pdt, n,
                             AdamScalars{}, state_dev, static_cast<hipStream_t>(stream));
}

int64_t zero_state_tiled_numel(int64_t n) {
  if (n <= 0 || n > kMaxPsi) return 0;
  return 3 * kTile * ceil_div(n, kTile);
}

int zero_adamw_step_tiled(const void* grad_dev, zero_dtype gdt, float* state_dev, uint16_t* param_dev,
                          zero_dtype pdt, int64_t n, const zero_adamw_hparams* hp, void* stream) {
  AdamScalars s;
  int rc = adam_args_ok("zero_adamw_step_tiled", grad_dev, gdt, param_dev, pdt, n, hp, &s);
  if (rc != ZERO_OK) return rc;
  return launch_adamw_tiled("zero_adamw_step_tiled", grad_dev, gdt, state_dev, param_dev, pdt, n, s, nullptr,
                            static_cast<hipStream_t>(stream));
}

int zero_adamw_step_tiled_dev(const void* grad_dev, zero_dtype gdt, float* state_dev, uint16_t* param_dev,
                              zero_dtype pdt, int64_t n, const zero_step_state* step_state_dev, void* stream) {
  int rc = dev_args_ok("zero_adamw_step_tiled_dev", grad_dev, gdt, param_dev, pdt, n, step_state_dev);
  if (rc != ZERO_OK) return rc;
  return launch_adamw_tiled("zero_adamw_step_tiled_dev", grad_dev, gdt, state_dev, param_dev, pdt, n, AdamScalars{},
                            step_state_dev, static_cast<hipStream_t>(stream));
}

int zero_step_state_init(zero_step_state* state_dev, double loss_scale, int32_t growth_interval, void* stream) {
  if (!state_dev || !aligned16(state_dev) || !(loss_scale > 0.0) || !std::isfinite(loss_scale) || growth_interval < 1)
    return fail(ZERO_ERR_INVALID, "zero_step_state_init: bad arguments");
  hipLaunchKernelGGL(step_state_init_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), state_dev,
                     loss_scale, growth_interval);
  return launch_status("zero_step_state_init");
}

int zero_step_decision_dev(const double* rank_sqnorms_dev, const int32_t* rank_flags_dev, int32_t n_ranks,
                           double max_norm, const zero_adamw_hparams* hp, zero_step_state* state_dev, void* stream) {
  if (n_ranks < 1 || !rank_sqnorms_dev || !rank_flags_dev || !hp || !state_dev || !aligned16(state_dev))
    return fail(ZERO_ERR_INVALID, "zero_step_decision_dev: bad arguments");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !(hp->eps >= 0.0) ||
      !(hp->lr >= 0.0) || !std::isfinite(hp->lr) || !(hp->weight_decay >= 0.0))
    return fail(ZERO_ERR_INVALID, "zero_step_decision_dev: hyper-parameters out of range");
  hipLaunchKernelGGL(step_decision_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), rank_sqnorms_dev,
                     rank_flags_dev, n_ranks, max_norm, hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay,
                     state_dev);
  return launch_status("zero_step_decision_dev");
}

int zero_state_tile(const float* master_dev, const float* m_dev, const float* v_dev, float* state_dev, int64_t n,
                    void* stream) {
  if (n < 0 || n > kMaxPsi || (n > 0 && (!master_dev || !m_dev || !v_dev || !state_dev)) ||
      !fp32_aligned(master_dev, m_dev, v_dev, state_dev))
    return fail(ZERO_ERR_INVALID, "zero_state_tile: bad arguments");
  if (n == 0) return ZERO_OK;
  const int64_t blocks = std::min<int64_t>(ceil_div(n, kBlock), 65536);
  hipLaunchKernelGGL(retile_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), const_cast<float*>(master_dev), const_cast<float*>(m_dev),
                     const_cast<float*>(v_dev), state_dev, n);
  return launch_status("zero_state_tile");
}

int zero_state_untile(const float* state_dev, float* master_dev, float* m_dev, float* v_dev, int64_t n, void* stream) {
  if (n < 0 || n > kMaxPsi || (n > 0 && (!master_dev || !m_dev || !v_dev || !state_dev)) ||
      !fp32_aligned(master_dev, m_dev, v_dev, state_dev))
    return fail(ZERO_ERR_INVALID, "zero_state_untile: bad arguments");
  if (n == 0) return ZERO_OK;
  const int64_t blocks = std::min<int64_t>(ceil_div(n, kBlock), 65536);
  hipLaunchKernelGGL(retile_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), master_dev, m_dev, v_dev, const_cast<float*>(state_dev), n);
  return launch_status("zero_state_untile");
}

int zero_calibrate_tiled_rmw(const void* grad_dev, float* state_dev, uint16_t* param_dev, int64_t n, uint32_t key,
                             void* stream) {
  const char* fn = "zero_calibrate_tiled_rmw";
  if (n < 0 || n > kMaxPsi || (n > 0 && (!grad_dev || !state_dev || !param_dev)) || !aligned8(grad_dev) ||
      !aligned8(param_dev) || !aligned16(state_dev))
    return fail(ZERO_ERR_INVALID, "%s: bad arguments", fn);
  if (n == 0) return ZERO_OK;
  const uint16_t* g = static_cast<const uint16_t*>(grad_dev);
  auto* state = reinterpret_cast<f32x4*>(state_dev);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return for_each_tiled_launch(n, fn, [&](int64_t t0, int64_t cnt) {
    hipLaunchKernelGGL(tiled_rmw_calibration_kernel, dim3(static_cast<unsigned>(cnt)), dim3(kBlock), 0, st, g, state,
                       param_dev, n, t0, key);
  });
}

}  // extern "C"
