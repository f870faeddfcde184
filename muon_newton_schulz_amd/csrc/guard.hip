// The safety net around the optimizer step (optimizer tutorial, section
// 5.4): the global gradient norm behind clip_grad_norm and the step guard,
// and statistics of an optimizer-state buffer for monitoring.
//
// Both are reductions over long flat buffers, bound by HBM.  They run on a
// fixed grid of kReduceBlocks workgroups with a fixed assignment of
// elements to threads and fixed reduction trees, accumulating in fp64, so
// the results are bitwise reproducible for a given input.
#include <cmath>

#include "muon.h"
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kThreads = 256;

// 8 consecutive elements as float (bf16: one 16-byte load; fp32: two).
template <typename T>
__device__ __forceinline__ void load8(const T* p, int64_t q, float* o);
template <>
__device__ __forceinline__ void load8<float>(const float* p, int64_t q, float* o) {
  const float4 a = reinterpret_cast<const float4*>(p)[2 * q];
  const float4 b = reinterpret_cast<const float4*>(p)[2 * q + 1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, int64_t q, float* o) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[q];
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(w[k] << 16);
    o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
template <typename T>
__device__ __forceinline__ float load1(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load1<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// Sum over the workgroup, fixed order: butterfly within each wave, then
// the four wave sums in order.  Every thread must call it; thread 0 gets
// the result.
__device__ __forceinline__ double block_sum(double v) {
  __shared__ double red[kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------- gradient norm

// Partial sums of squares: workgroup b writes partials[b].  vec: the
// buffer start is 16-byte aligned, so 8-element vectors are read and the
// n % 8 tail elements go to the first threads.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_sumsq(const T* __restrict__ g, int64_t n,
                                                   double* __restrict__ partials, int vec) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kThreads;
  double s = 0.0;
  if (vec) {
    const int64_t n8 = n >> 3;
    for (int64_t q = tid; q < n8; q += nthreads) {
      float x[8];
      load8<T>(g, q, x);
#pragma unroll
      for (int k = 0; k < 8; ++k) s = fma(static_cast<double>(x[k]), static_cast<double>(x[k]), s);
    }
    if (tid < (n & 7)) {
      const double x = load1<T>(g, (n8 << 3) + tid);
      s = fma(x, x, s);
    }
  } else {
    for (int64_t i = tid; i < n; i += nthreads) {
      const double x = load1<T>(g, i);
      s = fma(x, x, s);
    }
  }
  const double total = block_sum(s);
  if (threadIdx.x == 0) partials[blockIdx.x] = total;
}

// norm = sqrt(sum of all partials, in order); scale and skip from it.
__global__ __launch_bounds__(kThreads) void k_clip_finalize(const double* __restrict__ partials,
                                                           int n_parts, float max_norm, float eps,
                                                           ClipState* __restrict__ out) {
  double s = 0.0;
  for (int i = threadIdx.x; i < n_parts; i += kThreads) s += partials[i];
  const double total = block_sum(s);
  if (threadIdx.x == 0) {
    const double norm = sqrt(total);
    const bool skip = !isfinite(norm);
    double scale = 1.0;
    if (!skip && max_norm > 0.0f)
      scale = fmin(1.0, static_cast<double>(max_norm) / (norm + static_cast<double>(eps)));
    ClipState c;
    c.norm = static_cast<float>(norm);
    c.scale = static_cast<float>(scale);
    c.skip = skip ? 1 : 0;
    c.reserved = 0;
    *out = c;
  }
}

// ------------------------------------------------------- state statistics

// Running statistics of a set of finite values (Chan et al.'s pairwise
// update for the mean and the sum of squared deviations) plus the count
// of non-finite values.  64 bytes: the partials' stride in the workspace.
struct Stats {
  double n, mean, m2, mn, mx, amax, nonfinite, pad;
};
static_assert(sizeof(Stats) == kStatsPartialBytes, "partial stride");

__device__ __forceinline__ Stats stats_empty() {
  Stats s;
  s.n = 0.0; s.mean = 0.0; s.m2 = 0.0;
  s.mn = INFINITY; s.mx = -INFINITY; s.amax = 0.0;
  s.nonfinite = 0.0; s.pad = 0.0;
  return s;
}

__device__ __forceinline__ Stats stats_merge(const Stats& a, const Stats& b) {
  Stats r;
  r.n = a.n + b.n;
  if (a.n == 0.0) {
    r.mean = b.mean;
    r.m2 = b.m2;
  } else if (b.n == 0.0) {
    r.mean = a.mean;
    r.m2 = a.m2;
  } else {
    const double d = b.mean - a.mean;
    r.mean = a.mean + d * (b.n / r.n);
    r.m2 = a.m2 + b.m2 + d * d * (a.n * b.n / r.n);
  }
  r.mn = fmin(a.mn, b.mn);
  r.mx = fmax(a.mx, b.mx);
  r.amax = fmax(a.amax, b.amax);
  r.nonfinite = a.nonfinite + b.nonfinite;
  r.pad = 0.0;
  return r;
}

// One thread's values, accumulated about a shift (its first finite value)
// so that the sum of squared deviations does not cancel.
struct ThreadStats {
  double k, s1, s2, n, mn, mx, amax, nonf;
  __device__ __forceinline__ void init() {
    k = 0.0; s1 = 0.0; s2 = 0.0; n = 0.0;
    mn = INFINITY; mx = -INFINITY; amax = 0.0; nonf = 0.0;
  }
  __device__ __forceinline__ void add(float xf) {
    if (!isfinite(xf)) {
      nonf += 1.0;
      return;
    }
    const double x = xf;
    if (n == 0.0) k = x;
    const double d = x - k;
    s1 += d;
    s2 = fma(d, d, s2);
    n += 1.0;
    mn = fmin(mn, x);
    mx = fmax(mx, x);
    amax = fmax(amax, fabs(x));
  }
  __device__ __forceinline__ Stats finish() const {
    Stats s = stats_empty();
    s.n = n;
    s.nonfinite = nonf;
    if (n > 0.0) {
      s.mean = k + s1 / n;
      s.m2 = fmax(0.0, s2 - s1 * s1 / n);
      s.mn = mn;
      s.mx = mx;
      s.amax = amax;
    }
    return s;
  }
};

// Merge the workgroup's per-thread statistics in a fixed tree order;
// thread 0 returns the total.
__device__ __forceinline__ Stats block_stats(Stats s) {
  __shared__ Stats sh[kThreads];
  sh[threadIdx.x] = s;
  __syncthreads();
#pragma unroll
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) sh[threadIdx.x] = stats_merge(sh[threadIdx.x], sh[threadIdx.x + w]);
    __syncthreads();
  }
  return sh[0];
}

__global__ __launch_bounds__(kThreads) void k_stats_partial(const float* __restrict__ x,
                                                           int64_t n, Stats* __restrict__ parts,
                                                           int vec) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kThreads;
  ThreadStats t;
  t.init();
  if (vec) {
    const int64_t n4 = n >> 2;
    for (int64_t q = tid; q < n4; q += nthreads) {
      const float4 v = reinterpret_cast<const float4*>(x)[q];
      t.add(v.x);
      t.add(v.y);
      t.add(v.z);
      t.add(v.w);
    }
    if (tid < (n & 3)) t.add(x[(n4 << 2) + tid]);
  } else {
    for (int64_t i = tid; i < n; i += nthreads) t.add(x[i]);
  }
  const Stats total = block_stats(t.finish());
  if (threadIdx.x == 0) parts[blockIdx.x] = total;
}

__global__ __launch_bounds__(kThreads) void k_stats_finalize(const Stats* __restrict__ parts,
                                                            int n_parts,
                                                            muon_state_stats_t* __restrict__ out) {
  Stats s = stats_empty();
  for (int i = threadIdx.x; i < n_parts; i += kThreads) s = stats_merge(s, parts[i]);
  const Stats total = block_stats(s);
  if (threadIdx.x == 0) {
    muon_state_stats_t r;
    const bool any = total.n > 0.0;
    r.mean = any ? total.mean : 0.0;
    r.var = any ? total.m2 / total.n : 0.0;
    r.min = any ? total.mn : 0.0;
    r.max = any ? total.mx : 0.0;
    r.absmax = any ? total.amax : 0.0;
    r.count = static_cast<int64_t>(total.n);
    r.nonfinite = static_cast<int64_t>(total.nonfinite);
    *out = r;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_sumsq(const void* g, int dtype, int64_t n, double* partials, hipStream_t s) {
  const int vec = aligned16(g) ? 1 : 0;
  if (dtype == 1)
    hipLaunchKernelGGL(k_sumsq<uint16_t>, dim3(kReduceBlocks), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(g), n, partials, vec);
  else
    hipLaunchKernelGGL(k_sumsq<float>, dim3(kReduceBlocks), dim3(kThreads), 0, s,
                       static_cast<const float*>(g), n, partials, vec);
  return hipGetLastError();
}

hipError_t launch_clip_finalize(const double* partials, int n_parts, float max_norm, float eps,
                                ClipState* out, hipStream_t s) {
  hipLaunchKernelGGL(k_clip_finalize, dim3(1), dim3(kThreads), 0, s, partials, n_parts,
                     max_norm, eps, out);
  return hipGetLastError();
}

hipError_t launch_state_stats(const float* x, int64_t n, void* partials, void* out,
                              hipStream_t s) {
  Stats* parts = static_cast<Stats*>(partials);
  hipLaunchKernelGGL(k_stats_partial, dim3(kReduceBlocks), dim3(kThreads), 0, s, x, n, parts,
                     aligned16(x) ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_stats_finalize, dim3(1), dim3(kThreads), 0, s, parts, kReduceBlocks,
                     static_cast<muon_state_stats_t*>(out));
  return hipGetLastError();
}

}  // namespace muon
