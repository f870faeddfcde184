// Elementwise and reduction kernels of the Muon and AdamW steps (gfx950).
//
//  k_momentum       momentum EMA (optimizer tutorial, section 2.1) and the
//                   Nesterov look-ahead U, written into the NS workspace in
//                   the oriented layout (tall matrices transposed through
//                   an LDS tile), plus one fixed-order partial sum of U^2
//                   per 64x64 tile.
//  k_norm_finalize  per-matrix ||U||_F and 1/(||U||_F + eps) (Zhihu answer
//                   on K2, section 4: the Frobenius norm bounds the
//                   spectral norm).
//  k_apply          W <- (1 - lr*wd) W - lr*s*O (optimizer tutorial,
//                   section 3.1, decoupled decay; scale s per the K2
//                   answer, sections 3.1 / 3.2).
//  k_export         copies the current NS iterate out (stepwise checks).
//  k_adamw          fused AdamW (optimizer tutorial, sections 2.3, 3.1,
//                   3.3) with an optional fp32 master copy.
//
// All kernels are HBM-bound; accesses are coalesced along the contiguous
// dimension and reductions use a fixed order, so results are bitwise
// reproducible run to run.
#include "muon_internal.h"

namespace muon {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Natural padded dims of a matrix: the oriented iterate is [m_pad][n_pad];
// for a tall matrix that is the transpose of the natural [rows][cols].
struct NatDims {
  int rp, cp;  // natural padded rows / cols
};
__device__ __forceinline__ NatDims nat_dims(const MatDev& md) {
  NatDims d;
  d.rp = md.trans ? md.n_pad : md.m_pad;
  d.cp = md.trans ? md.m_pad : md.n_pad;
  return d;
}

// One 64x64 tile (natural coordinates) of one matrix per block, covering
// the padded extent so the zero padding of the NS operand is (re)written
// every step.
template <typename GT, typename UT>
__global__ __launch_bounds__(256) void k_momentum(const MatDev* __restrict__ mats,
                                                  const Item* __restrict__ items,
                                                  const GT* __restrict__ grads,
                                                  float* __restrict__ mom, UT* __restrict__ ws,
                                                  float* __restrict__ partials, float mu,
                                                  int nesterov) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ float wsum[4];
  const Item it = items[blockIdx.x];
  const MatDev md = mats[it.mat];
  const int r0 = (it.rc >> 16) * kEwTile, c0 = (it.rc & 0xffff) * kEwTile;
  const NatDims nd = nat_dims(md);
  UT* X = ws + md.ws_x[0];
  const int lc = threadIdx.x & 63, lr = threadIdx.x >> 6;
  const float omm = 1.0f - mu;
  const int c = c0 + lc;
  float ss = 0.0f;
#pragma unroll 4
  for (int q = 0; q < 16; ++q) {
    const int rr = lr + 4 * q, r = r0 + rr;
    float u = 0.0f;
    if (r < md.rows && c < md.cols) {
      const int64_t e = md.off + static_cast<int64_t>(r) * md.cols + c;
      const float g = Elem<GT>::ld(grads, e);
      const float m = mu * mom[e] + omm * g;
      mom[e] = m;
      u = nesterov ? mu * m + omm * g : m;
    }
    ss = fmaf(u, u, ss);
    if (md.trans) tile[rr][lc] = u;
    else Elem<UT>::st(X, static_cast<int64_t>(r) * nd.cp + c, u);
  }
  if (md.trans) {
    // X = U^T: X[c][r], coalesced along r
    __syncthreads();
#pragma unroll 4
    for (int q = 0; q < 16; ++q) {
      const int cc = lr + 4 * q;
      Elem<UT>::st(X, static_cast<int64_t>(c0 + cc) * nd.rp + r0 + lc, tile[lc][cc]);
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

// Reads the 64x64 natural-coordinate tile (r0, c0) of the oriented iterate
// X into registers: o[q] = O[r0 + lr + 4q][c0 + lc] (natural layout).  For
// a tall matrix the tile is staged through LDS so that the HBM reads stay
// coalesced.  Every thread of the block must call it.
template <typename UT>
__device__ __forceinline__ f32x16_t load_nat_tile(const MatDev& md, const UT* X, int r0, int c0,
                                                  float (&tile)[kEwTile][kEwTile + 1]) {
  f32x16_t o;
  const NatDims nd = nat_dims(md);
  const int lc = threadIdx.x & 63, lr = threadIdx.x >> 6;
  if (!md.trans) {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      o[q] = Elem<UT>::ld(X, static_cast<int64_t>(r0 + lr + 4 * q) * nd.cp + c0 + lc);
  } else {
    // X[c][r]: read rows c0.. of X along r, transpose in LDS
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int cc = lr + 4 * q;
      tile[cc][lc] = Elem<UT>::ld(X, static_cast<int64_t>(c0 + cc) * nd.rp + r0 + lc);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) o[q] = tile[lc][lr + 4 * q];
  }
  return o;
}

__global__ __launch_bounds__(256) void k_norm_finalize(const MatDev* __restrict__ mats,
                                                       int mat_begin,
                                                       const float* __restrict__ partials,
                                                       float* __restrict__ norms,
                                                       float* __restrict__ inv, float eps) {
  __shared__ double red[256];
  const MatDev md = mats[mat_begin + blockIdx.x];
  double s = 0.0;
  for (int t = threadIdx.x; t < md.k1_count; t += 256) s += partials[md.k1_begin + t];
  red[threadIdx.x] = s;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double nrm = sqrt(red[0]);
    norms[md.widx] = static_cast<float>(nrm);
    inv[md.widx] = static_cast<float>(1.0 / (nrm + static_cast<double>(eps)));
  }
}

__device__ __forceinline__ float update_scale(int rows, int cols, int mode, float rms_target) {
  if (mode == 0) return rms_target * sqrtf(static_cast<float>(rows > cols ? rows : cols));
  if (mode == 1) return sqrtf(fmaxf(1.0f, static_cast<float>(rows) / static_cast<float>(cols)));
  return 1.0f;
}

template <typename PT, typename UT>
__global__ __launch_bounds__(256) void k_apply(const MatDev* __restrict__ mats,
                                               const Item* __restrict__ items,
                                               PT* __restrict__ params, const UT* __restrict__ ws,
                                               const float* __restrict__ inv, int use_inv,
                                               int x_final, float lr, float wd, int scale_mode,
                                               float rms_target, float* __restrict__ out_update) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  const Item it = items[blockIdx.x];
  const MatDev md = mats[it.mat];
  const int r0 = (it.rc >> 16) * kEwTile, c0 = (it.rc & 0xffff) * kEwTile;
  const f32x16_t o = load_nat_tile<UT>(md, ws + (x_final ? md.ws_x[1] : md.ws_x[0]), r0, c0, tile);
  const float osc = use_inv ? inv[md.widx] : 1.0f;
  const float decay = 1.0f - lr * wd;
  const float step = lr * update_scale(md.rows, md.cols, scale_mode, rms_target);
  const int c = c0 + (threadIdx.x & 63);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int r = r0 + (threadIdx.x >> 6) + 4 * q;
    if (r < md.rows && c < md.cols) {
      const int64_t e = md.off + static_cast<int64_t>(r) * md.cols + c;
      const float oo = o[q] * osc;
      const float w = Elem<PT>::ld(params, e);
      Elem<PT>::st(params, e, decay * w - step * oo);
      if (out_update) out_update[e] = oo;
    }
  }
}

template <typename UT>
__global__ __launch_bounds__(256) void k_export(const MatDev* __restrict__ mats,
                                                const Item* __restrict__ items,
                                                const UT* __restrict__ ws, int x_idx,
                                                float* __restrict__ out) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  const Item it = items[blockIdx.x];
  const MatDev md = mats[it.mat];
  const int r0 = (it.rc >> 16) * kEwTile, c0 = (it.rc & 0xffff) * kEwTile;
  const f32x16_t o = load_nat_tile<UT>(md, ws + (x_idx ? md.ws_x[1] : md.ws_x[0]), r0, c0, tile);
  const int c = c0 + (threadIdx.x & 63);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int r = r0 + (threadIdx.x >> 6) + 4 * q;
    if (r < md.rows && c < md.cols) out[md.off + static_cast<int64_t>(r) * md.cols + c] = o[q];
  }
}

// ---------------------------------------------------------------- AdamW

template <typename PT, typename GT, bool MASTER>
__device__ __forceinline__ void adamw_one(PT* params, float* master, const GT* grads, float* m,
                                          float* v, int64_t i, float b1, float b2, float eps,
                                          float lr_bc1, float rsqrt_bc2, float decay) {
  const float g = Elem<GT>::ld(grads, i);
  const float th = MASTER ? master[i] : Elem<PT>::ld(params, i);
  const float mm = b1 * m[i] + (1.0f - b1) * g;
  const float vv = b2 * v[i] + (1.0f - b2) * g * g;
  const float den = sqrtf(vv) * rsqrt_bc2 + eps;
  const float nt = th * decay - lr_bc1 * (mm / den);
  m[i] = mm;
  v[i] = vv;
  if (MASTER) master[i] = nt;
  Elem<PT>::st(params, i, nt);
}

// Scalar grid-stride variant: any alignment.
template <typename PT, typename GT, bool MASTER>
__global__ __launch_bounds__(256) void k_adamw_scalar(PT* __restrict__ params,
                                                      float* __restrict__ master,
                                                      const GT* __restrict__ grads,
                                                      float* __restrict__ m, float* __restrict__ v,
                                                      int64_t n, float b1, float b2, float eps,
                                                      float lr_bc1, float rsqrt_bc2,
                                                      float decay) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride)
    adamw_one<PT, GT, MASTER>(params, master, grads, m, v, i, b1, b2, eps, lr_bc1, rsqrt_bc2,
                              decay);
}

template <typename T> struct Vec4;
template <> struct Vec4<float> { using type = float4; };
template <> struct Vec4<uint16_t> { using type = ushort4; };

__device__ __forceinline__ void to_f4(const float4& a, float* o) {
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}
__device__ __forceinline__ void to_f4(const ushort4& a, float* o) {
  o[0] = bf16_to_f32(a.x); o[1] = bf16_to_f32(a.y);
  o[2] = bf16_to_f32(a.z); o[3] = bf16_to_f32(a.w);
}
__device__ __forceinline__ void from_f4(const float* o, float4& a) {
  a.x = o[0]; a.y = o[1]; a.z = o[2]; a.w = o[3];
}
__device__ __forceinline__ void from_f4(const float* o, ushort4& a) {
  a.x = f32_to_bf16(o[0]); a.y = f32_to_bf16(o[1]);
  a.z = f32_to_bf16(o[2]); a.w = f32_to_bf16(o[3]);
}

// Vector variant: 4 elements per thread per iteration; every pointer is
// aligned to 4 elements (checked on the host); the tail of n % 4 elements
// is done by the first threads of block 0.
template <typename PT, typename GT, bool MASTER>
__global__ __launch_bounds__(256) void k_adamw_vec4(PT* __restrict__ params,
                                                    float* __restrict__ master,
                                                    const GT* __restrict__ grads,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    int64_t n, float b1, float b2, float eps,
                                                    float lr_bc1, float rsqrt_bc2, float decay) {
  using PV = typename Vec4<PT>::type;
  using GV = typename Vec4<GT>::type;
  const int64_t n4 = n >> 2;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < n4;
       q += stride) {
    float g[4], th[4], mm[4], vv[4];
    to_f4(reinterpret_cast<const GV*>(grads)[q], g);
    if (MASTER) to_f4(reinterpret_cast<const float4*>(master)[q], th);
    else to_f4(reinterpret_cast<const PV*>(params)[q], th);
    to_f4(reinterpret_cast<const float4*>(m)[q], mm);
    to_f4(reinterpret_cast<const float4*>(v)[q], vv);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      mm[k] = b1 * mm[k] + (1.0f - b1) * g[k];
      vv[k] = b2 * vv[k] + (1.0f - b2) * g[k] * g[k];
      const float den = sqrtf(vv[k]) * rsqrt_bc2 + eps;
      th[k] = th[k] * decay - lr_bc1 * (mm[k] / den);
    }
    float4 o;
    from_f4(mm, o); reinterpret_cast<float4*>(m)[q] = o;
    from_f4(vv, o); reinterpret_cast<float4*>(v)[q] = o;
    if (MASTER) { from_f4(th, o); reinterpret_cast<float4*>(master)[q] = o; }
    PV pv;
    from_f4(th, pv);
    reinterpret_cast<PV*>(params)[q] = pv;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t i = (n4 << 2) + threadIdx.x;
    adamw_one<PT, GT, MASTER>(params, master, grads, m, v, i, b1, b2, eps, lr_bc1, rsqrt_bc2,
                              decay);
  }
}

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

template <typename PT, typename GT, bool MASTER>
hipError_t adamw_dispatch(void* params, float* master, const void* grads, float* m, float* v,
                          int64_t n, float b1, float b2, float eps, float lr_bc1,
                          float rsqrt_bc2, float decay, hipStream_t s) {
  PT* p = static_cast<PT*>(params);
  const GT* g = static_cast<const GT*>(grads);
  const bool vec = aligned(p, 4 * sizeof(PT)) && aligned(g, 4 * sizeof(GT)) &&
                   aligned(m, 16) && aligned(v, 16) && (!MASTER || aligned(master, 16));
  const int64_t work = vec ? (n >> 2) : n;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (vec)
    hipLaunchKernelGGL((k_adamw_vec4<PT, GT, MASTER>), dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, p, master, g, m, v, n, b1, b2, eps, lr_bc1, rsqrt_bc2,
                       decay);
  else
    hipLaunchKernelGGL((k_adamw_scalar<PT, GT, MASTER>), dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, p, master, g, m, v, n, b1, b2, eps, lr_bc1, rsqrt_bc2,
                       decay);
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------ launchers

hipError_t launch_momentum(const MatDev* mats, const Item* items, int n_items, int grad_dtype,
                           int ns_dtype, const void* grads, float* mom, void* ws,
                           float* partials, float mu, int nesterov, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(n_items), block(256);
#define MUON_K1(GT, UT)                                                                   \
  hipLaunchKernelGGL((k_momentum<GT, UT>), grid, block, 0, s, mats, items,                \
                     static_cast<const GT*>(grads), mom, static_cast<UT*>(ws), partials, mu, \
                     nesterov)
  if (grad_dtype == 1 && ns_dtype == 1) MUON_K1(uint16_t, uint16_t);
  else if (grad_dtype == 1 && ns_dtype == 0) MUON_K1(uint16_t, float);
  else if (grad_dtype == 0 && ns_dtype == 1) MUON_K1(float, uint16_t);
  else MUON_K1(float, float);
#undef MUON_K1
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const MatDev* mats, int mat_begin, int n_mats,
                                const float* partials, float* norms, float* inv, float eps,
                                hipStream_t s) {
  if (n_mats == 0) return hipSuccess;
  hipLaunchKernelGGL(k_norm_finalize, dim3(n_mats), dim3(256), 0, s, mats, mat_begin, partials,
                     norms, inv, eps);
  return hipGetLastError();
}

hipError_t launch_apply(const MatDev* mats, const Item* items, int n_items, int param_dtype,
                        int ns_dtype, void* params, const void* ws, const float* inv,
                        float o_scale_by_inv, int x_final, float lr, float wd, int scale_mode,
                        float rms_target, float* out_update, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(n_items), block(256);
  const int use_inv = o_scale_by_inv != 0.0f;
#define MUON_K7(PT, UT)                                                                       \
  hipLaunchKernelGGL((k_apply<PT, UT>), grid, block, 0, s, mats, items, static_cast<PT*>(params), \
                     static_cast<const UT*>(ws), inv, use_inv, x_final, lr, wd, scale_mode,     \
                     rms_target, out_update)
  if (param_dtype == 1 && ns_dtype == 1) MUON_K7(uint16_t, uint16_t);
  else if (param_dtype == 1 && ns_dtype == 0) MUON_K7(uint16_t, float);
  else if (param_dtype == 0 && ns_dtype == 1) MUON_K7(float, uint16_t);
  else MUON_K7(float, float);
#undef MUON_K7
  return hipGetLastError();
}

hipError_t launch_export(const MatDev* mats, const Item* items, int n_items, int ns_dtype,
                         const void* ws, int x_idx, float* out, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  if (ns_dtype == 1)
    hipLaunchKernelGGL((k_export<uint16_t>), dim3(n_items), dim3(256), 0, s, mats, items,
                       static_cast<const uint16_t*>(ws), x_idx, out);
  else
    hipLaunchKernelGGL((k_export<float>), dim3(n_items), dim3(256), 0, s, mats, items,
                       static_cast<const float*>(ws), x_idx, out);
  return hipGetLastError();
}

hipError_t launch_adamw(void* params, int param_dtype, float* master, const void* grads,
                        int grad_dtype, float* m, float* v, int64_t n, float lr, float beta1,
                        float beta2, float eps, float wd, float lr_bc1, float rsqrt_bc2,
                        hipStream_t s) {
  if (n == 0) return hipSuccess;
  const float decay = 1.0f - lr * wd;
  const bool ma = master != nullptr;
#define MUON_K8(PT, GT, MA)                                                                 \
  return adamw_dispatch<PT, GT, MA>(params, master, grads, m, v, n, beta1, beta2, eps, lr_bc1, \
                                    rsqrt_bc2, decay, s)
  if (param_dtype == 1) {
    // bf16 parameters always come with a fp32 master (checked by the caller)
    if (grad_dtype == 1) MUON_K8(uint16_t, uint16_t, true);
    MUON_K8(uint16_t, float, true);
  }
  if (ma) {
    if (grad_dtype == 1) MUON_K8(float, uint16_t, true);
    MUON_K8(float, float, true);
  }
  if (grad_dtype == 1) MUON_K8(float, uint16_t, false);
  MUON_K8(float, float, false);
#undef MUON_K8
}

}  // namespace muon
