// MuonClip (Kimi K2 answer by toothacher17, section 4): a scalar rescale of
// blocks of the flat parameter buffer (W_q / W_k, whole or one head's rows)
// after the optimizer step, either by the block's Frobenius norm (which
// bounds its spectral norm and so ||x W||_2) or by a supplied max attention
// logit (a head's logits are bilinear in its W_q and W_k rows).
//
// HBM-bound.  The blocks are cut into fixed chunks of kClipChunk elements,
// one workgroup per chunk:
//   k_clip_sumsq   (Frobenius mode) fp64 sum of squares of each chunk;
//   k_clip_scale   sums its block's chunk partials in a fixed order (every
//                  workgroup of the block gets the same norm, bit for bit),
//                  forms gamma and rescales its chunk, or returns at once
//                  when gamma is 1.
// Frobenius mode reads a block once (2 B/param bf16) and, when it is
// clipped, reads and writes it once more; max-logit mode is one launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "muon.h"
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kClipThreads = 256;
constexpr int kClipChunk = 32768;  // elements per workgroup, a multiple of 8
static_assert(kClipChunk % 8 == 0, "chunks keep 8-element vectors whole");

// One block as the device sees it.
struct ClipTarget {
  int64_t off;         // element offset of (0, 0) in the flat buffer
  int64_t ld;          // elements between rows
  int32_t cols;
  int32_t group;
  int32_t vec;         // offset, ld and cols are multiples of 8
  int32_t contiguous;  // ld == cols or one row: element e sits at off + e
  int32_t chunk_begin, chunk_end;
};

// One workgroup's share: elements [e0, e0 + n) of a block, row-major.
struct ClipChunk {
  int32_t target;
  int32_t e0;
  int32_t n;
  int32_t reserved;
};

__device__ __forceinline__ int64_t elem_addr(const ClipTarget& t, uint32_t e) {
  if (t.contiguous) return t.off + e;
  const uint32_t r = e / static_cast<uint32_t>(t.cols);
  const uint32_t c = e - r * static_cast<uint32_t>(t.cols);
  return t.off + static_cast<int64_t>(r) * t.ld + c;
}

// 8 consecutive elements at element index a (a multiple of 8, base 16-byte
// aligned) as float, and back.
__device__ __forceinline__ void load8(const uint16_t* p, int64_t a, float* o) {
  const uint4 v = *reinterpret_cast<const uint4*>(p + a);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(w[k] << 16);
    o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, int64_t a, float* o) {
  const float4 u = *reinterpret_cast<const float4*>(p + a);
  const float4 v = *reinterpret_cast<const float4*>(p + a + 4);
  o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
  o[4] = v.x; o[5] = v.y; o[6] = v.z; o[7] = v.w;
}
__device__ __forceinline__ void store8(uint16_t* p, int64_t a, const float* o) {
  uint4 v;
  v.x = static_cast<uint32_t>(f32_to_bf16(o[0])) | (static_cast<uint32_t>(f32_to_bf16(o[1])) << 16);
  v.y = static_cast<uint32_t>(f32_to_bf16(o[2])) | (static_cast<uint32_t>(f32_to_bf16(o[3])) << 16);
  v.z = static_cast<uint32_t>(f32_to_bf16(o[4])) | (static_cast<uint32_t>(f32_to_bf16(o[5])) << 16);
  v.w = static_cast<uint32_t>(f32_to_bf16(o[6])) | (static_cast<uint32_t>(f32_to_bf16(o[7])) << 16);
  *reinterpret_cast<uint4*>(p + a) = v;
}
__device__ __forceinline__ void store8(float* p, int64_t a, const float* o) {
  *reinterpret_cast<float4*>(p + a) = make_float4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<float4*>(p + a + 4) = make_float4(o[4], o[5], o[6], o[7]);
}
__device__ __forceinline__ float load1(const uint16_t* p, int64_t a) { return bf16_to_f32(p[a]); }
__device__ __forceinline__ float load1(const float* p, int64_t a) { return p[a]; }
__device__ __forceinline__ void store1(uint16_t* p, int64_t a, float x) { p[a] = f32_to_bf16(x); }
__device__ __forceinline__ void store1(float* p, int64_t a, float x) { p[a] = x; }

// gamma * w in fp64, rounded to fp32 (the storage cast rounds once more
// for bf16)
__device__ __forceinline__ float scaled(double gamma, float w) {
  return static_cast<float>(gamma * static_cast<double>(w));
}

// Sum over the workgroup in a fixed order (butterfly within each wave,
// then the four wave sums in order).  Every thread gets the result.
__device__ __forceinline__ double block_sum(double v) {
  __shared__ double red[kClipThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename T>
__global__ __launch_bounds__(kClipThreads) void k_clip_sumsq(
    const ClipTarget* __restrict__ targets, const ClipChunk* __restrict__ chunks,
    const T* __restrict__ w, int allow_vec, double* __restrict__ partials) {
  const ClipChunk ch = chunks[blockIdx.x];
  const ClipTarget t = targets[ch.target];
  double s = 0.0;
  if (allow_vec && t.vec) {
    for (int q = threadIdx.x; q < (ch.n >> 3); q += kClipThreads) {
      float x[8];
      load8(w, elem_addr(t, static_cast<uint32_t>(ch.e0 + 8 * q)), x);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        s = fma(static_cast<double>(x[k]), static_cast<double>(x[k]), s);
    }
  } else {
    for (int i = threadIdx.x; i < ch.n; i += kClipThreads) {
      const double x = load1(w, elem_addr(t, static_cast<uint32_t>(ch.e0 + i)));
      s = fma(x, x, s);
    }
  }
  const double total = block_sum(s);
  if (threadIdx.x == 0) partials[blockIdx.x] = total;
}

template <typename T>
__global__ __launch_bounds__(kClipThreads) void k_clip_scale(
    const ClipTarget* __restrict__ targets, const ClipChunk* __restrict__ chunks,
    T* __restrict__ w, int allow_vec, int mode, float tau, const double* __restrict__ partials,
    const float* __restrict__ max_logits, float* __restrict__ norms_out,
    float* __restrict__ scales_out) {
  const ClipChunk ch = chunks[blockIdx.x];
  const ClipTarget t = targets[ch.target];
  double gamma = 1.0, norm = 0.0;
  if (mode == MUON_CLIP_FROBENIUS) {
    double s = 0.0;
    for (int c = t.chunk_begin + static_cast<int>(threadIdx.x); c < t.chunk_end;
         c += kClipThreads)
      s += partials[c];
    norm = sqrt(block_sum(s));
    if (isfinite(norm) && norm > static_cast<double>(tau)) gamma = static_cast<double>(tau) / norm;
  } else {
    const float S = max_logits[t.group];
    if (isfinite(S) && S > tau) gamma = sqrt(static_cast<double>(tau) / static_cast<double>(S));
  }
  if (ch.e0 == 0 && threadIdx.x == 0) {
    if (norms_out) norms_out[ch.target] = static_cast<float>(norm);
    if (scales_out) scales_out[ch.target] = static_cast<float>(gamma);
  }
  if (gamma == 1.0) return;  // uniform over the workgroup
  if (allow_vec && t.vec) {
    for (int q = threadIdx.x; q < (ch.n >> 3); q += kClipThreads) {
      const int64_t a = elem_addr(t, static_cast<uint32_t>(ch.e0 + 8 * q));
      float x[8];
      load8(w, a, x);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = scaled(gamma, x[k]);
      store8(w, a, x);
    }
  } else {
    for (int i = threadIdx.x; i < ch.n; i += kClipThreads) {
      const int64_t a = elem_addr(t, static_cast<uint32_t>(ch.e0 + i));
      store1(w, a, scaled(gamma, load1(w, a)));
    }
  }
}

}  // namespace
}  // namespace muon

using muon::ClipChunk;
using muon::ClipTarget;

struct muon_clip_plan {
  int device = -1;       // set by muon_clip_plan_upload
  bool uploaded = false;
  int32_t n_targets = 0, n_groups = 0, param_dtype = 0;
  int64_t flat_numel = 0;
  int32_t n_chunks = 0;
  size_t ws_bytes = 0;
  // the block and chunk tables packed as the device sees them, and the
  // chunk table's byte offset
  std::vector<char> host_tables;
  size_t o_chunks = 0;
  // device copies, inside the caller's table buffer
  ClipTarget* d_targets = nullptr;
  ClipChunk* d_chunks = nullptr;
};

namespace {

using muon::set_error;
using muon::set_hip_error;

constexpr int64_t kMaxOverlapIntervals = int64_t(1) << 24;

int validate_targets(const muon_clip_target_t* tg, int32_t n, int64_t flat_numel,
                     int32_t n_groups) {
  std::vector<std::pair<int64_t, int64_t>> iv;  // [begin, end) element ranges
  for (int32_t i = 0; i < n; ++i) {
    const muon_clip_target_t& t = tg[i];
    const std::string who = "target " + std::to_string(i) + ": ";
    if (t.rows < 1 || t.cols < 1) return set_error(MUON_ERR_BAD_SHAPE, who + "rows, cols < 1");
    if (static_cast<int64_t>(t.rows) * t.cols > INT32_MAX)
      return set_error(MUON_ERR_BAD_SHAPE, who + "more than 2^31 - 1 elements");
    if (t.ld < t.cols) return set_error(MUON_ERR_BAD_SHAPE, who + "ld < cols");
    if (t.offset < 0 || t.ld > flat_numel || t.offset > flat_numel - t.cols ||
        (t.rows > 1 && (t.rows - 1) > (flat_numel - t.cols - t.offset) / t.ld))
      return set_error(MUON_ERR_BAD_SHAPE, who + "outside the flat buffer");
    if (t.group < 0 || t.group >= std::max<int32_t>(n_groups, 1))
      return set_error(MUON_ERR_INVALID_ARG, who + "group out of range");
    if (t.ld == t.cols || t.rows == 1) {
      iv.emplace_back(t.offset, t.offset + static_cast<int64_t>(t.rows) * t.cols);
    } else {
      if (static_cast<int64_t>(iv.size()) + t.rows > kMaxOverlapIntervals)
        return set_error(MUON_ERR_UNSUPPORTED, "too many strided rows to check for overlap");
      for (int32_t r = 0; r < t.rows; ++r)
        iv.emplace_back(t.offset + r * t.ld, t.offset + r * t.ld + t.cols);
    }
  }
  std::sort(iv.begin(), iv.end());
  for (size_t k = 1; k < iv.size(); ++k)
    if (iv[k].first < iv[k - 1].second)
      return set_error(MUON_ERR_OVERLAP, "two clip targets share elements");
  return MUON_OK;
}

}  // namespace

extern "C" {

int muon_clip_plan_create(const muon_clip_target_t* targets, int32_t n_targets,
                          int64_t flat_numel, int32_t param_dtype, int32_t n_groups,
                          muon_clip_plan_t** out, size_t* workspace_bytes) {
  if (out == nullptr) return set_error(MUON_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  if (n_targets < 0 || (n_targets > 0 && targets == nullptr))
    return set_error(MUON_ERR_INVALID_ARG, "bad target list");
  if (flat_numel < 0 || n_groups < 0)
    return set_error(MUON_ERR_INVALID_ARG, "flat_numel and n_groups must be >= 0");
  if (param_dtype != MUON_DTYPE_FP32 && param_dtype != MUON_DTYPE_BF16)
    return set_error(MUON_ERR_BAD_DTYPE, "params must be fp32 or bf16");
  int rc = validate_targets(targets, n_targets, flat_numel, n_groups);
  if (rc != MUON_OK) return rc;

  std::vector<ClipTarget> dt(n_targets);
  std::vector<ClipChunk> dc;
  for (int32_t i = 0; i < n_targets; ++i) {
    const muon_clip_target_t& t = targets[i];
    ClipTarget& d = dt[i];
    d.off = t.offset;
    d.ld = t.ld;
    d.cols = t.cols;
    d.group = t.group;
    d.vec = (t.offset % 8 == 0 && t.ld % 8 == 0 && t.cols % 8 == 0) ? 1 : 0;
    d.contiguous = (t.ld == t.cols || t.rows == 1) ? 1 : 0;
    d.chunk_begin = static_cast<int32_t>(dc.size());
    const int64_t total = static_cast<int64_t>(t.rows) * t.cols;
    for (int64_t e = 0; e < total; e += muon::kClipChunk) {
      ClipChunk c;
      c.target = i;
      c.e0 = static_cast<int32_t>(e);
      c.n = static_cast<int32_t>(std::min<int64_t>(muon::kClipChunk, total - e));
      c.reserved = 0;
      dc.push_back(c);
      if (dc.size() > static_cast<size_t>(INT32_MAX))
        return set_error(MUON_ERR_UNSUPPORTED, "too many chunks");
    }
    d.chunk_end = static_cast<int32_t>(dc.size());
  }

  muon_clip_plan* p = new (std::nothrow) muon_clip_plan;
  if (p == nullptr) return set_error(MUON_ERR_INVALID_ARG, "out of host memory");
  p->n_targets = n_targets;
  p->n_groups = n_groups;
  p->param_dtype = param_dtype;
  p->flat_numel = flat_numel;
  p->n_chunks = static_cast<int32_t>(dc.size());
  p->ws_bytes = (dc.size() * sizeof(double) + 255) / 256 * 256;
  if (n_targets > 0) {
    p->o_chunks = (dt.size() * sizeof(ClipTarget) + 255) / 256 * 256;
    p->host_tables.assign(p->o_chunks + dc.size() * sizeof(ClipChunk), 0);
    std::copy_n(reinterpret_cast<const char*>(dt.data()), dt.size() * sizeof(ClipTarget),
                p->host_tables.data());
    std::copy_n(reinterpret_cast<const char*>(dc.data()), dc.size() * sizeof(ClipChunk),
                p->host_tables.data() + p->o_chunks);
  }
  if (workspace_bytes) *workspace_bytes = p->ws_bytes;
  *out = p;
  return MUON_OK;
}

void muon_clip_plan_destroy(muon_clip_plan_t* plan) { delete plan; }

size_t muon_clip_plan_table_bytes(const muon_clip_plan_t* plan) {
  return plan == nullptr ? 0 : plan->host_tables.size();
}

int muon_clip_plan_upload(muon_clip_plan_t* plan, void* tables, size_t table_bytes,
                          hipStream_t stream) {
  if (plan == nullptr) return set_error(MUON_ERR_INVALID_ARG, "plan is null");
  const size_t need = plan->host_tables.size();
  if (need > 0) {
    if (tables == nullptr) return set_error(MUON_ERR_INVALID_ARG, "tables is null");
    if (reinterpret_cast<uintptr_t>(tables) % 256 != 0)
      return set_error(MUON_ERR_INVALID_ARG, "tables must be 256-byte aligned");
    if (table_bytes < need)
      return set_error(MUON_ERR_INVALID_ARG, "tables has " + std::to_string(table_bytes) +
                                                 " bytes, the plan needs " +
                                                 std::to_string(need));
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_hip_error(e, "hipGetDevice");
  if (need > 0) {
    e = hipMemcpyAsync(tables, plan->host_tables.data(), need, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return set_hip_error(e, "hipMemcpyAsync(clip tables)");
  }
  plan->d_targets = reinterpret_cast<ClipTarget*>(tables);
  plan->d_chunks = reinterpret_cast<ClipChunk*>(static_cast<char*>(tables) + plan->o_chunks);
  plan->device = dev;
  plan->uploaded = true;
  return MUON_OK;
}

int muon_clip(const muon_clip_plan_t* plan, void* params, int32_t mode, float tau,
              const float* max_logits, void* workspace, size_t workspace_bytes,
              float* norms_out, float* scales_out, hipStream_t stream) {
  if (plan == nullptr) return set_error(MUON_ERR_INVALID_ARG, "plan is null");
  if (mode != MUON_CLIP_FROBENIUS && mode != MUON_CLIP_MAX_LOGIT)
    return set_error(MUON_ERR_INVALID_ARG, "unknown clip mode");
  if (!std::isfinite(tau) || !(tau > 0.0f))
    return set_error(MUON_ERR_INVALID_ARG, "tau must be finite and > 0");
  if (plan->n_chunks == 0) return MUON_OK;
  if (!plan->uploaded)
    return set_error(MUON_ERR_INVALID_ARG, "plan tables are not on a device (muon_clip_plan_upload)");
  if (params == nullptr) return set_error(MUON_ERR_INVALID_ARG, "params is null");
  if (mode == MUON_CLIP_FROBENIUS) {
    if (workspace == nullptr || workspace_bytes < plan->ws_bytes ||
        reinterpret_cast<uintptr_t>(workspace) % alignof(double) != 0)
      return set_error(MUON_ERR_WORKSPACE_TOO_SMALL,
                       "muon_clip needs " + std::to_string(plan->ws_bytes) +
                           " bytes of workspace, 8-byte aligned");
  } else {
    if (max_logits == nullptr) return set_error(MUON_ERR_INVALID_ARG, "max_logits is null");
    if (plan->n_groups < 1)
      return set_error(MUON_ERR_INVALID_ARG, "max-logit mode needs a plan with n_groups >= 1");
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_hip_error(e, "hipGetDevice");
  if (dev != plan->device)
    return set_error(MUON_ERR_INVALID_ARG, "current device differs from the plan's device");

  const int allow_vec = (reinterpret_cast<uintptr_t>(params) % 16 == 0) ? 1 : 0;
  double* partials = static_cast<double*>(workspace);
  const dim3 grid(plan->n_chunks), block(muon::kClipThreads);
  if (plan->param_dtype == MUON_DTYPE_BF16) {
    uint16_t* w = static_cast<uint16_t*>(params);
    if (mode == MUON_CLIP_FROBENIUS)
      hipLaunchKernelGGL(muon::k_clip_sumsq<uint16_t>, grid, block, 0, stream, plan->d_targets,
                         plan->d_chunks, w, allow_vec, partials);
    hipLaunchKernelGGL(muon::k_clip_scale<uint16_t>, grid, block, 0, stream, plan->d_targets,
                       plan->d_chunks, w, allow_vec, mode, tau, partials, max_logits, norms_out,
                       scales_out);
  } else {
    float* w = static_cast<float*>(params);
    if (mode == MUON_CLIP_FROBENIUS)
      hipLaunchKernelGGL(muon::k_clip_sumsq<float>, grid, block, 0, stream, plan->d_targets,
                         plan->d_chunks, w, allow_vec, partials);
    hipLaunchKernelGGL(muon::k_clip_scale<float>, grid, block, 0, stream, plan->d_targets,
                       plan->d_chunks, w, allow_vec, mode, tau, partials, max_logits, norms_out,
                       scales_out);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "MuonClip kernel launch");
  return MUON_OK;
}

}  // extern "C"
