// Elementwise and reduction kernels of the Muon and AdamW steps (gfx950).
//
//  k_momentum       momentum EMA (optimizer tutorial, section 2.1) and the
//                   Nesterov look-ahead U, written into the NS workspace in
//                   the oriented layout (tall matrices transposed through
//                   an LDS tile), plus one fixed-order partial sum of U^2
//                   per 64x64 tile.
//  k_norm_finalize  per-matrix ||U||_F and 1/(||U||_F + eps) (Zhihu answer
//                   on K2, section 4: the Frobenius norm bounds the
//                   spectral norm); rescales X0 by a power of two for a
//                   norm outside the folded normalisation's range.
//  k_apply          W <- (1 - lr*wd) W - lr*s*O (optimizer tutorial,
//                   section 3.1, decoupled decay; scale s per the K2
//                   answer, sections 3.1 / 3.2).
//  k_export         copies the current NS iterate out (stepwise checks).
//  k_adamw_vec8     fused AdamW (optimizer tutorial, sections 2.3, 3.1,
//                   3.3) with an optional fp32 master copy.
//
// All kernels are HBM-bound; accesses are coalesced along the contiguous
// dimension and reductions use a fixed order, so results are bitwise
// reproducible run to run.
#include <type_traits>

#include "muon_internal.h"

namespace muon {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

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
// IEEE binary16 (AdamW second moment only); the cast rounds to nearest even
template <> struct Elem<_Float16> {
  static __device__ __forceinline__ float ld(const _Float16* p, int64_t i) {
    return static_cast<float>(p[i]);
  }
  static __device__ __forceinline__ void st(_Float16* p, int64_t i, float v) {
    p[i] = static_cast<_Float16>(v);
  }
};

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}


// Index of element (row, col) of a matrix's oriented iterate X in the
// workspace: the bf16 workspace's 32-column panels (panel_off), or
// row-major [m_pad][n_pad] for fp32.  Four consecutive columns from a
// multiple of 4 stay contiguous either way.
template <typename UT>
__device__ __forceinline__ int64_t ws_idx(const MatDev& md, int row, int col) {
  if constexpr (std::is_same<UT, uint16_t>::value) return panel_off(row, col, md.m_pad);
  else return static_cast<int64_t>(row) * md.n_pad + col;
}

// 4 consecutive elements (bf16: 8 bytes, fp32: 16 bytes)
template <typename T> struct V4;
template <> struct V4<float> {
  using type = float4;
  static __device__ __forceinline__ f32x4v ld(const float* p, int64_t i) {
    const float4 v = *reinterpret_cast<const float4*>(p + i);
    return f32x4v{v.x, v.y, v.z, v.w};
  }
  static __device__ __forceinline__ void st(float* p, int64_t i, f32x4v v) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct V4<uint16_t> {
  static __device__ __forceinline__ f32x4v ld(const uint16_t* p, int64_t i) {
    const uint2 w = *reinterpret_cast<const uint2*>(p + i);
    return f32x4v{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
  }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, f32x4v v) {
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    *reinterpret_cast<uint2*>(p + i) = w;
  }
};

// A matrix can use 4-wide accesses when its rows start on 4-element
// boundaries of the flat buffers (the buffers themselves are checked on
// the host).
__device__ __forceinline__ bool vec4_ok(const MatDev& md, int bufs_aligned) {
  return bufs_aligned && (md.off & 3) == 0 && (md.cols & 3) == 0;
}

// Span path of the apply kernel for a matrix whose rows are off that grid
// (an odd offset or width in the flat concatenation): row rr of a 64x64
// tile is the flat span [a, b) of the parameter-side buffers.  Its whole aligned 4-element groups,
// [fs, fe), at most 16, are read and written 4-wide, 16 threads per row;
// the head [a, min(fs, b)) and the tail [max(fs, fe), b), at most 3
// elements each, one at a time, 4 threads per row, so that neither pass
// branches on the data.  The iterate side goes through the LDS tile.
struct Span {
  int64_t a, b;    // flat elements of the row in the tile: [a, b), empty past the matrix
  int64_t fs, fe;  // whole 4-element groups: [fs, fe) (empty if fe <= fs)
};
__device__ __forceinline__ Span tile_row_span(const MatDev& md, int r, int c0) {
  Span sp;
  const int w = (r < md.rows && c0 < md.cols) ? min(kEwTile, md.cols - c0) : 0;
  sp.a = md.off + static_cast<int64_t>(r) * md.cols + c0;
  sp.b = sp.a + w;
  sp.fs = (sp.a + 3) & ~int64_t{3};
  sp.fe = sp.b & ~int64_t{3};
  return sp;
}

// One 64x64 tile (natural coordinates) of one matrix per block, covering
// the padded extent so the zero padding of the NS operand is (re)written
// every step.  4-wide path: thread = 4 consecutive columns x 4 rows.
template <typename GT, typename UT>
__global__ __launch_bounds__(256) void k_momentum(const MatDev* __restrict__ mats,
                                                  const Item* __restrict__ items,
                                                  const GT* __restrict__ grads,
                                                  float* __restrict__ mom, UT* __restrict__ ws,
                                                  double* __restrict__ partials, float mu,
                                                  int nesterov, int bufs_aligned,
                                                  const ClipState* __restrict__ clip) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ double wsum[4];
  // guarded step: skip it whole, or scale the gradient (uniform branch)
  float gscale = 1.0f;
  if (clip != nullptr) {
    if (clip->skip) return;
    gscale = clip->scale;
  }
  const Item it = items[blockIdx.x];
  const MatDev md = mats[it.mat];
  const int r0 = (it.rc >> 16) * kEwTile, c0 = (it.rc & 0xffff) * kEwTile;
  UT* X = ws + md.ws_x[0];
  const float omm = 1.0f - mu;
  // the sum of squares in fp64 (fixed order), so the norm keeps full
  // precision over the tile
  double ss = 0.0;
  if (vec4_ok(md, bufs_aligned)) {
    const int cg = (threadIdx.x & 15) * 4, rg = threadIdx.x >> 4;
    const int c = c0 + cg;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = rg + 16 * q, r = r0 + rr;
      f32x4v u = {0.f, 0.f, 0.f, 0.f};
      if (r < md.rows && c < md.cols) {
        const int64_t e = md.off + static_cast<int64_t>(r) * md.cols + c;
        const f32x4v g = gscale * V4<GT>::ld(grads, e);
        f32x4v m = V4<float>::ld(mom, e);
        m = mu * m + omm * g;
        V4<float>::st(mom, e, m);
        u = nesterov ? mu * m + omm * g : m;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) ss = fma(static_cast<double>(u[k]), static_cast<double>(u[k]), ss);
      if (md.trans) {
#pragma unroll
        for (int k = 0; k < 4; ++k) tile[rr][cg + k] = u[k];
      } else {
        V4<UT>::st(X, ws_idx<UT>(md, r, c), u);
      }
    }
    if (md.trans) {
      // X = U^T: thread writes X[c][r..r+3] (4 consecutive rows of U)
      __syncthreads();
      const int rq = (threadIdx.x & 15) * 4, cc0 = threadIdx.x >> 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = cc0 + 16 * q;
        const f32x4v v = {tile[rq][cc], tile[rq + 1][cc], tile[rq + 2][cc], tile[rq + 3][cc]};
        V4<UT>::st(X, ws_idx<UT>(md, c0 + cc, r0 + rq), v);
      }
    }
  } else {
    const int lc = threadIdx.x & 63, lr = threadIdx.x >> 6;
    const int c = c0 + lc;
#pragma unroll 4
    for (int q = 0; q < 16; ++q) {
      const int rr = lr + 4 * q, r = r0 + rr;
      float u = 0.0f;
      if (r < md.rows && c < md.cols) {
        const int64_t e = md.off + static_cast<int64_t>(r) * md.cols + c;
        const float g = gscale * Elem<GT>::ld(grads, e);
        const float m = mu * mom[e] + omm * g;
        mom[e] = m;
        u = nesterov ? mu * m + omm * g : m;
      }
      ss = fma(static_cast<double>(u), static_cast<double>(u), ss);
      if (md.trans) tile[rr][lc] = u;
      else Elem<UT>::st(X, ws_idx<UT>(md, r, c), u);
    }
    if (md.trans) {
      // X = U^T: X[c][r], coalesced along r
      __syncthreads();
#pragma unroll 4
      for (int q = 0; q < 16; ++q) {
        const int cc = lr + 4 * q;
        Elem<UT>::st(X, ws_idx<UT>(md, c0 + cc, r0 + lc), tile[lc][cc]);
      }
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  // the partial's slot is the tile's place in its matrix's row-major tile
  // order (the launch order of the tiles is permuted over the XCDs)
  if (threadIdx.x == 0) {
    const int ctiles = (md.trans ? md.m_pad : md.n_pad) / kEwTile;
    partials[md.k1_begin + static_cast<int64_t>(it.rc >> 16) * ctiles + (it.rc & 0xffff)] =
        (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  }
}

// Reads the 64x64 natural-coordinate tile (r0, c0) of the oriented iterate
// X into registers: o[q] = O[r0 + lr + 4q][c0 + lc] (natural layout).  For
// a tall matrix the tile is staged through LDS so that the HBM reads stay
// coalesced.  Every thread of the block must call it.
template <typename UT>
__device__ __forceinline__ f32x16_t load_nat_tile(const MatDev& md, const UT* X, int r0, int c0,
                                                  float (&tile)[kEwTile][kEwTile + 1]) {
  f32x16_t o;
  const int lc = threadIdx.x & 63, lr = threadIdx.x >> 6;
  if (!md.trans) {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      o[q] = Elem<UT>::ld(X, ws_idx<UT>(md, r0 + lr + 4 * q, c0 + lc));
  } else {
    // X[c][r]: read rows c0.. of X along r, transpose in LDS
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int cc = lr + 4 * q;
      tile[cc][lc] = Elem<UT>::ld(X, ws_idx<UT>(md, c0 + cc, r0 + lc));
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) o[q] = tile[lc][lr + 4 * q];
  }
  return o;
}

// The first NS products accumulate the unnormalised U U^T in fp32 and
// scale it by inv^2 in the epilogue.  That is exact in range while
// ||U||_F lies in [2^-40, 2^40]: products of the entries that carry the
// norm stay normal fp32 numbers, and neither U U^T nor inv^2 can exceed
// 2^80.  A matrix whose norm lies outside (finite and nonzero) has its
// iterate X0 = U scaled in place by 2^k, with ||U||_F * 2^k in [0.5, 1),
// and inv divided by 2^k, so that inv * X0 is unchanged and every product
// is in range.  Scaling by a power of two is exact (bf16 and fp32 alike).
// Returns k (0 inside the range).
__device__ __forceinline__ int norm_rescale_exp(double nrm) {
  if (!(nrm > 0.0) || !(nrm < HUGE_VAL) || (nrm >= 0x1p-40 && nrm <= 0x1p40)) return 0;
  int e;
  (void)frexp(nrm, &e);  // nrm = f * 2^e, f in [0.5, 1)
  return -e;
}

template <typename UT>
__device__ __forceinline__ void scale_pow2(UT* x, int64_t n, int k);
template <>
__device__ __forceinline__ void scale_pow2<float>(float* x, int64_t n, int k) {
  for (int64_t i = threadIdx.x; i < n / 4; i += blockDim.x) {
    float4 v = reinterpret_cast<float4*>(x)[i];
    v.x = ldexpf(v.x, k); v.y = ldexpf(v.y, k); v.z = ldexpf(v.z, k); v.w = ldexpf(v.w, k);
    reinterpret_cast<float4*>(x)[i] = v;
  }
}
template <>
__device__ __forceinline__ void scale_pow2<uint16_t>(uint16_t* x, int64_t n, int k) {
  for (int64_t i = threadIdx.x; i < n / 8; i += blockDim.x) {
    uint4 v = reinterpret_cast<uint4*>(x)[i];
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = ldexpf(__uint_as_float(w[e] << 16), k);
      const float hi = ldexpf(__uint_as_float(w[e] & 0xffff0000u), k);
      w[e] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
    }
    reinterpret_cast<uint4*>(x)[i] = uint4{w[0], w[1], w[2], w[3]};
  }
}

// One block per matrix: ||U||_F from the fixed-order partials, inv =
// 1/(||U||_F + eps), and the power-of-two rescale of X0 for a norm out of
// the folded normalisation's range (the rare path: the whole block scales
// the matrix's iterate).
template <typename UT>
__global__ __launch_bounds__(256) void k_norm_finalize(const MatDev* __restrict__ mats,
                                                       int mat_begin,
                                                       const double* __restrict__ partials,
                                                       float* __restrict__ norms,
                                                       float* __restrict__ inv, float eps,
                                                       UT* __restrict__ ws) {
  __shared__ double red[256];
  const MatDev md = mats[mat_begin + blockIdx.x];
  double s = 0.0;
  for (int t = threadIdx.x; t < md.k1_count; t += 256) s += partials[md.k1_begin + t];
  red[threadIdx.x] = s;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double nrm = sqrt(red[0]);
  const int k = norm_rescale_exp(nrm);
  if (threadIdx.x == 0) {
    norms[md.widx] = static_cast<float>(nrm);
    inv[md.widx] = static_cast<float>(ldexp(1.0 / (nrm + static_cast<double>(eps)), -k));
  }
  if (k != 0)
    scale_pow2<UT>(ws + md.ws_x[0], static_cast<int64_t>(md.m_pad) * md.n_pad, k);
}

template <typename PT, typename UT>
__global__ __launch_bounds__(256) void k_apply(const MatDev* __restrict__ mats,
                                               const Item* __restrict__ items,
                                               PT* __restrict__ params, const UT* __restrict__ ws,
                                               const float* __restrict__ inv, int use_inv,
                                               int x_final, float lr, float wd, int scale_mode,
                                               float rms_target, float* __restrict__ out_update,
                                               int bufs_aligned,
                                               const ClipState* __restrict__ clip) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  if (clip != nullptr && clip->skip) return;  // guarded step: nothing changes
  const Item it = items[blockIdx.x];
  const MatDev md = mats[it.mat];
  const int r0 = (it.rc >> 16) * kEwTile, c0 = (it.rc & 0xffff) * kEwTile;
  const UT* X = ws + (x_final ? md.ws_x[1] : md.ws_x[0]);
  const float osc = use_inv ? inv[md.widx] : 1.0f;
  const ApplyConsts ak = apply_consts(md.rows, md.cols, lr, wd, scale_mode, rms_target);
  if (vec4_ok(md, bufs_aligned)) {
    // thread = 4 consecutive columns x 4 rows (16 elements)
      const int cg = (threadIdx.x & 15) * 4, rg = threadIdx.x >> 4;
    f32x4v o[4];
    if (!md.trans) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = V4<UT>::ld(X, ws_idx<UT>(md, r0 + rg + 16 * q, c0 + cg));
    } else {
      // X[c][r]: 4 consecutive r per thread, transposed through LDS
      const int rq = (threadIdx.x & 15) * 4, cc0 = threadIdx.x >> 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = cc0 + 16 * q;
        const f32x4v v = V4<UT>::ld(X, ws_idx<UT>(md, c0 + cc, r0 + rq));
#pragma unroll
        for (int k = 0; k < 4; ++k) tile[rq + k][cc] = v[k];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) o[q][k] = tile[rg + 16 * q][cg + k];
    }
    const int c = c0 + cg;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r0 + rg + 16 * q;
      if (r < md.rows && c < md.cols) {
        const int64_t e = md.off + static_cast<int64_t>(r) * md.cols + c;
        const f32x4v oo = o[q] * osc;
        const f32x4v w = V4<PT>::ld(params, e);
        f32x4v wn;
#pragma unroll
        for (int k = 0; k < 4; ++k) wn[k] = apply_one(ak, w[k], oo[k]);
        V4<PT>::st(params, e, wn);
        if (out_update) V4<float>::st(out_update, e, oo);
      }
    }
    return;
  }
  if (bufs_aligned) {
    // span path: O of the tile into LDS in natural coordinates, then the
    // parameter-side buffers in aligned groups
    {
      const int q4 = (threadIdx.x & 15) * 4, q16 = threadIdx.x >> 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!md.trans) {
          const int rr = q16 + 16 * q;
          const f32x4v v = V4<UT>::ld(X, ws_idx<UT>(md, r0 + rr, c0 + q4));
#pragma unroll
          for (int k = 0; k < 4; ++k) tile[rr][q4 + k] = v[k] * osc;
        } else {
          const int cc = q16 + 16 * q;
          const f32x4v v = V4<UT>::ld(X, ws_idx<UT>(md, c0 + cc, r0 + q4));
#pragma unroll
          for (int k = 0; k < 4; ++k) tile[q4 + k][cc] = v[k] * osc;
        }
      }
    }
    __syncthreads();
    {
      const int gi = threadIdx.x & 15, q16 = threadIdx.x >> 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = q16 + 16 * q;
        const Span sp = tile_row_span(md, r0 + rr, c0);
        const int64_t gs = sp.fs + 4 * gi;
        if (gs + 4 > sp.fe) continue;
        const int cc = static_cast<int>(gs - sp.a);
        f32x4v oo;
#pragma unroll
        for (int k = 0; k < 4; ++k) oo[k] = tile[rr][cc + k];
        const f32x4v w = V4<PT>::ld(params, gs);
        f32x4v wn;
#pragma unroll
        for (int k = 0; k < 4; ++k) wn[k] = apply_one(ak, w[k], oo[k]);
        V4<PT>::st(params, gs, wn);
        if (out_update) V4<float>::st(out_update, gs, oo);
      }
    }
    {
      const int rr = threadIdx.x >> 2, j = threadIdx.x & 3;
      const Span sp = tile_row_span(md, r0 + rr, c0);
      const int64_t eh = sp.a + j, et = (sp.fe > sp.fs ? sp.fe : sp.fs) + j;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t e = h == 0 ? eh : et;
        const bool mine = h == 0 ? (e < sp.fs && e < sp.b) : (e < sp.b);
        if (!mine) continue;
        const float oo = tile[rr][static_cast<int>(e - sp.a)];
        Elem<PT>::st(params, e, apply_one(ak, Elem<PT>::ld(params, e), oo));
        if (out_update) out_update[e] = oo;
      }
    }
    return;
  }
  const f32x16_t o = load_nat_tile<UT>(md, X, r0, c0, tile);
  const int c = c0 + (threadIdx.x & 63);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int r = r0 + (threadIdx.x >> 6) + 4 * q;
    if (r < md.rows && c < md.cols) {
      const int64_t e = md.off + static_cast<int64_t>(r) * md.cols + c;
      const float oo = o[q] * osc;
      const float w = Elem<PT>::ld(params, e);
      Elem<PT>::st(params, e, apply_one(ak, w, oo));
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
//
// Template parameters: PT parameter storage, GT gradient storage, MT / VT
// storage of the first / second moment (float; uint16_t = bf16; _Float16
// for the second moment), MASTER: a fp32 master copy is updated and the
// parameter receives its cast.  A step reads the states from their
// storage, computes in fp32 and stores them rounded to nearest even.

template <typename PT, typename GT, typename MT, typename VT, bool MASTER>
__device__ __forceinline__ void adamw_one(PT* params, float* master, const GT* grads, MT* m,
                                          VT* v, int64_t i, float b1, float b2, float eps,
                                          float lr_bc1, float rsqrt_bc2, float decay,
                                          float gscale) {
  const float g = gscale * Elem<GT>::ld(grads, i);
  const float th = MASTER ? master[i] : Elem<PT>::ld(params, i);
  const float mm = b1 * Elem<MT>::ld(m, i) + (1.0f - b1) * g;
  const float vv = b2 * Elem<VT>::ld(v, i) + (1.0f - b2) * g * g;
  const float den = sqrtf(vv) * rsqrt_bc2 + eps;
  const float nt = th * decay - lr_bc1 * (mm / den);
  Elem<MT>::st(m, i, mm);
  Elem<VT>::st(v, i, vv);
  if (MASTER) master[i] = nt;
  Elem<PT>::st(params, i, nt);
}

// Scalar grid-stride variant: any alignment.
template <typename PT, typename GT, typename MT, typename VT, bool MASTER>
__global__ __launch_bounds__(256) void k_adamw_scalar(PT* __restrict__ params,
                                                      float* __restrict__ master,
                                                      const GT* __restrict__ grads,
                                                      MT* __restrict__ m, VT* __restrict__ v,
                                                      int64_t n, float b1, float b2, float eps,
                                                      float lr_bc1, float rsqrt_bc2,
                                                      float decay,
                                                      const ClipState* __restrict__ clip) {
  float gscale = 1.0f;
  if (clip != nullptr) {
    if (clip->skip) return;  // guarded step: nothing changes
    gscale = clip->scale;
  }
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride)
    adamw_one<PT, GT, MT, VT, MASTER>(params, master, grads, m, v, i, b1, b2, eps, lr_bc1,
                                      rsqrt_bc2, decay, gscale);
}

// 8 consecutive elements per thread and iteration: 16-bit vectors are 16
// bytes, fp32 vectors two 16-byte loads.  Every pointer is aligned to 8
// elements (checked on the host); the tail of n % 8 elements is done by the
// first threads of block 0.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
template <typename T>
__device__ __forceinline__ void ld8(const T* p, int64_t q, float* o);
template <>
__device__ __forceinline__ void ld8<float>(const float* p, int64_t q, float* o) {
  const float4 a = reinterpret_cast<const float4*>(p)[2 * q];
  const float4 b = reinterpret_cast<const float4*>(p)[2 * q + 1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <>
__device__ __forceinline__ void ld8<uint16_t>(const uint16_t* p, int64_t q, float* o) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[q];
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(w[k] << 16);
    o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void ld8<_Float16>(const _Float16* p, int64_t q, float* o) {
  const f16x8_t h = reinterpret_cast<const f16x8_t*>(p)[q];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = static_cast<float>(h[k]);
}
template <typename T>
__device__ __forceinline__ void st8(T* p, int64_t q, const float* o);
template <>
__device__ __forceinline__ void st8<float>(float* p, int64_t q, const float* o) {
  reinterpret_cast<float4*>(p)[2 * q] = make_float4(o[0], o[1], o[2], o[3]);
  reinterpret_cast<float4*>(p)[2 * q + 1] = make_float4(o[4], o[5], o[6], o[7]);
}
template <>
__device__ __forceinline__ void st8<uint16_t>(uint16_t* p, int64_t q, const float* o) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = static_cast<uint32_t>(f32_to_bf16(o[2 * k])) |
           (static_cast<uint32_t>(f32_to_bf16(o[2 * k + 1])) << 16);
  reinterpret_cast<uint4*>(p)[q] = make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ void st8<_Float16>(_Float16* p, int64_t q, const float* o) {
  f16x8_t h;
#pragma unroll
  for (int k = 0; k < 8; ++k) h[k] = static_cast<_Float16>(o[k]);
  reinterpret_cast<f16x8_t*>(p)[q] = h;
}

template <typename PT, typename GT, typename MT, typename VT, bool MASTER>
__global__ __launch_bounds__(256) void k_adamw_vec8(PT* __restrict__ params,
                                                    float* __restrict__ master,
                                                    const GT* __restrict__ grads,
                                                    MT* __restrict__ m, VT* __restrict__ v,
                                                    int64_t n, float b1, float b2, float eps,
                                                    float lr_bc1, float rsqrt_bc2, float decay,
                                                    const ClipState* __restrict__ clip) {
  float gscale = 1.0f;
  if (clip != nullptr) {
    if (clip->skip) return;  // guarded step: nothing changes
    gscale = clip->scale;
  }
  const int64_t n8 = n >> 3;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < n8;
       q += stride) {
    float g[8], th[8], mm[8], vv[8];
    ld8<GT>(grads, q, g);
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] *= gscale;
    if (MASTER) ld8<float>(master, q, th);
    else ld8<PT>(params, q, th);
    ld8<MT>(m, q, mm);
    ld8<VT>(v, q, vv);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      mm[k] = b1 * mm[k] + (1.0f - b1) * g[k];
      vv[k] = b2 * vv[k] + (1.0f - b2) * g[k] * g[k];
      const float den = sqrtf(vv[k]) * rsqrt_bc2 + eps;
      th[k] = th[k] * decay - lr_bc1 * (mm[k] / den);
    }
    st8<MT>(m, q, mm);
    st8<VT>(v, q, vv);
    if (MASTER) st8<float>(master, q, th);
    st8<PT>(params, q, th);
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t i = (n8 << 3) + threadIdx.x;
    adamw_one<PT, GT, MT, VT, MASTER>(params, master, grads, m, v, i, b1, b2, eps, lr_bc1,
                                      rsqrt_bc2, decay, gscale);
  }
}

template <typename PT, typename GT, typename MT, typename VT, bool MASTER>
hipError_t adamw_dispatch(void* params, float* master, const void* grads, void* mv, void* vv,
                          int64_t n, float b1, float b2, float eps, float lr_bc1,
                          float rsqrt_bc2, float decay, const ClipState* clip, hipStream_t s) {
  PT* p = static_cast<PT*>(params);
  const GT* g = static_cast<const GT*>(grads);
  MT* m = static_cast<MT*>(mv);
  VT* v = static_cast<VT*>(vv);
  const bool vec = aligned(p, 8 * sizeof(PT)) && aligned(g, 8 * sizeof(GT)) &&
                   aligned(m, 8 * sizeof(MT)) && aligned(v, 8 * sizeof(VT)) &&
                   (!MASTER || aligned(master, 32));
  const int64_t work = vec ? (n >> 3) : n;
  int64_t blocks = (work + 255) / 256;
  // Up to 65536 blocks, one pass for groups of up to 1.3e8 elements.  A
  // thread's next loads wait behind its stores (they may alias), so a
  // grid-stride loop over few blocks keeps fewer bytes in flight: at 8192
  // blocks a 6.6e7-element group ran 5% slower.
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (vec)
    hipLaunchKernelGGL((k_adamw_vec8<PT, GT, MT, VT, MASTER>),
                       dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, master, g, m, v,
                       n, b1, b2, eps, lr_bc1, rsqrt_bc2, decay, clip);
  else
    hipLaunchKernelGGL((k_adamw_scalar<PT, GT, MT, VT, MASTER>),
                       dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, master, g, m, v,
                       n, b1, b2, eps, lr_bc1, rsqrt_bc2, decay, clip);
  return hipGetLastError();
}

// state storage: m fp32 / bf16, v fp32 / bf16 / fp16
template <typename PT, typename GT, bool MASTER>
hipError_t adamw_states(int m_dtype, int v_dtype, void* params, float* master, const void* grads,
                        void* m, void* v, int64_t n, float b1, float b2, float eps, float lr_bc1,
                        float rsqrt_bc2, float decay, const ClipState* clip, hipStream_t s) {
#define MUON_K8S(MT, VT)                                                                      \
  return adamw_dispatch<PT, GT, MT, VT, MASTER>(params, master, grads, m, v, n, b1, b2, eps,  \
                                                lr_bc1, rsqrt_bc2, decay, clip, s)
  if (m_dtype == 1) {
    if (v_dtype == 2) MUON_K8S(uint16_t, _Float16);
    if (v_dtype == 1) MUON_K8S(uint16_t, uint16_t);
    MUON_K8S(uint16_t, float);
  }
  if (v_dtype == 2) MUON_K8S(float, _Float16);
  if (v_dtype == 1) MUON_K8S(float, uint16_t);
  MUON_K8S(float, float);
#undef MUON_K8S
}

}  // namespace

// ------------------------------------------------------------ launchers

hipError_t launch_momentum(const MatDev* mats, const Item* items, int n_items, int grad_dtype,
                           int ns_dtype, const void* grads, float* mom, void* ws,
                           double* partials, float mu, int nesterov, const ClipState* clip,
                           hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(n_items), block(256);
  const int al = aligned(grads, 4 * (grad_dtype == 1 ? 2 : 4)) && aligned(mom, 16);
#define MUON_K1(GT, UT)                                                                   \
  hipLaunchKernelGGL((k_momentum<GT, UT>), grid, block, 0, s, mats, items,                \
                     static_cast<const GT*>(grads), mom, static_cast<UT*>(ws), partials, mu, \
                     nesterov, al, clip)
  if (grad_dtype == 1 && ns_dtype == 1) MUON_K1(uint16_t, uint16_t);
  else if (grad_dtype == 1 && ns_dtype == 0) MUON_K1(uint16_t, float);
  else if (grad_dtype == 0 && ns_dtype == 1) MUON_K1(float, uint16_t);
  else MUON_K1(float, float);
#undef MUON_K1
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const MatDev* mats, int mat_begin, int n_mats,
                                const double* partials, float* norms, float* inv, float eps,
                                int ns_dtype, void* ws, hipStream_t s) {
  if (n_mats == 0) return hipSuccess;
  if (ns_dtype == 1)
    hipLaunchKernelGGL(k_norm_finalize<uint16_t>, dim3(n_mats), dim3(256), 0, s, mats, mat_begin,
                       partials, norms, inv, eps, static_cast<uint16_t*>(ws));
  else
    hipLaunchKernelGGL(k_norm_finalize<float>, dim3(n_mats), dim3(256), 0, s, mats, mat_begin,
                       partials, norms, inv, eps, static_cast<float*>(ws));
  return hipGetLastError();
}

hipError_t launch_apply(const MatDev* mats, const Item* items, int n_items, int param_dtype,
                        int ns_dtype, void* params, const void* ws, const float* inv,
                        float o_scale_by_inv, int x_final, float lr, float wd, int scale_mode,
                        float rms_target, float* out_update, const ClipState* clip,
                        hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(n_items), block(256);
  const int use_inv = o_scale_by_inv != 0.0f;
  const int al = aligned(params, 4 * (param_dtype == 1 ? 2 : 4)) &&
                 (out_update == nullptr || aligned(out_update, 16));
#define MUON_K7(PT, UT)                                                                       \
  hipLaunchKernelGGL((k_apply<PT, UT>), grid, block, 0, s, mats, items, static_cast<PT*>(params), \
                     static_cast<const UT*>(ws), inv, use_inv, x_final, lr, wd, scale_mode,     \
                     rms_target, out_update, al, clip)
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
                        int grad_dtype, void* m, int m_dtype, void* v, int v_dtype, int64_t n,
                        float lr, float beta1, float beta2, float eps, float wd, float lr_bc1,
                        float rsqrt_bc2, const ClipState* clip, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const float decay = 1.0f - lr * wd;
  const bool ma = master != nullptr;
#define MUON_K8(PT, GT, MA)                                                                    \
  return adamw_states<PT, GT, MA>(m_dtype, v_dtype, params, master, grads, m, v, n, beta1,     \
                                  beta2, eps, lr_bc1, rsqrt_bc2, decay, clip, s)
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
