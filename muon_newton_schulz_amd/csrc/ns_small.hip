// Newton-Schulz for small matrices on gfx950: one workgroup runs one whole
// NS iteration (optimizer tutorial, section 4.2, generalised to
// X <- a X + (b A + c A A) X with A = X X^T) of one matrix in LDS.
//
// A matrix with m_k <= kSmallM and m_k * n_k <= kSmallElems is a single
// 256x256 tile of the tiled engine (ns_gemm.hip), which would run it on one
// CU as three dependent launches per iteration; here X, A and B stay in LDS
// between the phases and the iteration is one launch.  The MFMA chains
// (v_mfma_f32_32x32x16_bf16 over k in ascending order, operands in the same
// roles) and the epilogue arithmetic are the tiled engine's, so the iterate
// is bitwise the same.
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// LDS rows are padded by 8 elements (16 bytes): consecutive rows start 4
// banks apart, so the 16-byte fragment reads of 16 rows hit 64 distinct
// banks and the transpose reads and 2-byte epilogue writes at most 2-way.
constexpr int kPad = 8;

// two floats -> packed bf16 pair, round to nearest even (the tiled engine's
// conversion)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Work split: 32x32 output blocks, block b to wave b % 4; each lane holds
// element (i, j) = (bi*32 + lane%32, bj*32 + 8*(r/4) + 4*(lane/32) + r%4)
// of accumulator register r, as in the tiled engine.

// Fragment reads run one 16-wide k step ahead of the MFMAs (the k loop is
// unrolled by two, K being a multiple of 32), and every fragment read feeds
// several MFMAs.  Slots a wave does not own run on block 0's fragments and
// are discarded, so the k loop has no branches.

// C = sc * P P^T (+ bterm * A, phase 2) (+ dval on the diagonal of the
// diagonal blocks), rounded to bf16, for the blocks on and above the
// diagonal.  P: [rows][ld] bf16 in LDS, K-contiguous.
// Wave (wr, wc) = (wave / 2, wave % 2) owns the 2 x 2 blocks bi = 2 wr + u,
// bj = 2 wc + v (those inside the nb x nb grid): 2 P and 2 Q fragments per
// k step for 4 MFMAs.
template <bool ATERM>
__device__ __forceinline__ void small_nt(const uint16_t* P, int ld, int K, int nb, float sc,
                                         float bterm, const uint16_t* A, float dval,
                                         uint16_t* C, int ldc, int wave, int lane) {
  const int frow = lane & 31, kh = (lane >> 5) * 8;
  const int wr = wave >> 1, wc = wave & 1;
  int pa[2], qa[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int bi = 2 * wr + u < nb ? 2 * wr + u : 0;
    const int bj = 2 * wc + u < nb ? 2 * wc + u : 0;
    pa[u] = (bi * 32 + frow) * ld + kh;
    qa[u] = (bj * 32 + frow) * ld + kh;
  }
  f32x16_t acc[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) acc[u][v] = f32x16_t{};
  bf16x8_t p0[2], q0[2], p1[2], q1[2];
  auto load = [&](bf16x8_t (&pf)[2], bf16x8_t (&qf)[2], int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pf[u] = *reinterpret_cast<const bf16x8_t*>(P + pa[u] + k0);
      qf[u] = *reinterpret_cast<const bf16x8_t*>(P + qa[u] + k0);
    }
  };
  auto mma = [&](const bf16x8_t (&pf)[2], const bf16x8_t (&qf)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 2; ++v)
        acc[u][v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[v], pf[u], acc[u][v], 0, 0, 0);
  };
  load(p0, q0, 0);
  for (int k0 = 0; k0 < K; k0 += 32) {
    load(p1, q1, k0 + 16);
    mma(p0, q0);
    if (k0 + 32 < K) load(p0, q0, k0 + 32);
    mma(p1, q1);
  }
  // four consecutive columns per lane and register group: 8-byte accesses;
  // only the blocks on and above the diagonal (small_mirror fills the rest)
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int bi = 2 * wr + u, bj = 2 * wc + v;
      if (bi < nb && bj < nb && bi <= bj) {
        const int i = bi * 32 + frow;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // every rounding step as written, as in the tiled engine
#pragma clang fp contract(off)
          const int j0 = bj * 32 + 8 * q + 4 * (lane >> 5);
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = sc * acc[u][v][4 * q + e];
          if constexpr (ATERM) {
            // fma(b, a, c A A), as the tiled engine writes it out
            const u32x2_t a = *reinterpret_cast<const u32x2_t*>(A + i * ldc + j0);
            x[0] = fmaf(bterm, lo_bf(a[0]), x[0]);
            x[1] = fmaf(bterm, hi_bf(a[0]), x[1]);
            x[2] = fmaf(bterm, lo_bf(a[1]), x[2]);
            x[3] = fmaf(bterm, hi_bf(a[1]), x[3]);
          }
          if (bi == bj) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] += i == j0 + e ? dval : 0.0f;
          }
          *reinterpret_cast<u32x2_t*>(C + i * ldc + j0) =
              u32x2_t{pack2(x[0], x[1]), pack2(x[2], x[3])};
        }
      }
    }
}

// As in the tiled engine's diagonal tile, the 32x32 blocks below the
// diagonal are the transposes of those above it.  Every thread; between
// barriers (the upper blocks are final, the lower ones not yet read).
__device__ __forceinline__ void small_mirror(uint16_t* C, int ldc, int mk) {
  for (int e = threadIdx.x; e < mk * mk; e += 256) {
    const int i = e / mk, j = e - i * mk;
    if ((i >> 5) > (j >> 5)) C[i * ldc + j] = C[j * ldc + i];
  }
}

// X <- sc * (B X) in LDS: B [mk][ldb], X [mk][ldx], NU = mk / 32 row blocks.
// Wave w owns every row block and the column blocks bj = w + 4 t, t < NT:
// NU B fragments and NT X fragments per k step for NU * NT MFMAs.  The X
// fragments (8 consecutive k of one column) come from two
// ds_read_b64_tr_b16: each 16-lane group reads a 4 x 16 block (lane s: row
// s/4, columns 4*(s%4)..+3) and every lane receives one column's 4 rows.
template <int NU, int NT>
__device__ __forceinline__ void small_bx(const uint16_t* B, int ldb, uint16_t* X, int ldx, int mk,
                                         int nk, float sc, int wave, int lane) {
  const int frow = lane & 31, kh = (lane >> 5) * 8;
  const int ts = lane & 15;
  const int trow = kh + (ts >> 2), tcol = 16 * ((lane >> 4) & 1) + 4 * (ts & 3);
  const int nbn = nk >> 5;
  int ba[NU], xa[NT];
#pragma unroll
  for (int u = 0; u < NU; ++u) ba[u] = (u * 32 + frow) * ldb + kh;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int bj = wave + 4 * t < nbn ? wave + 4 * t : 0;
    xa[t] = trow * ldx + bj * 32 + tcol;
  }
  f32x16_t acc[NU][NT];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[u][t] = f32x16_t{};
  bf16x8_t p0[NU], q0[NT], p1[NU], q1[NT];
  auto load = [&](bf16x8_t (&pf)[NU], bf16x8_t (&qf)[NT], int k0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) pf[u] = *reinterpret_cast<const bf16x8_t*>(B + ba[u] + k0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint16_t* x = X + xa[t] + k0 * ldx;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(x));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(x + 4 * ldx));
      qf[t] = __builtin_bit_cast(bf16x8_t,
                                 __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mma = [&](const bf16x8_t (&pf)[NU], const bf16x8_t (&qf)[NT]) {
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[u][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t], pf[u], acc[u][t], 0, 0, 0);
  };
  load(p0, q0, 0);
  for (int k0 = 0; k0 < mk; k0 += 32) {
    load(p1, q1, k0 + 16);
    mma(p0, q0);
    if (k0 + 32 < mk) load(p0, q0, k0 + 32);
    mma(p1, q1);
  }
  __syncthreads();  // every wave is done reading X
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int bj = wave + 4 * t;
    if (bj < nbn) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int i = u * 32 + frow;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j0 = bj * 32 + 8 * q + 4 * (lane >> 5);
          *reinterpret_cast<u32x2_t*>(X + i * ldx + j0) =
              u32x2_t{pack2(sc * acc[u][t][4 * q], sc * acc[u][t][4 * q + 1]),
                      pack2(sc * acc[u][t][4 * q + 2], sc * acc[u][t][4 * q + 3])};
        }
      }
    }
  }
}

__device__ __forceinline__ void small_bx_any(const uint16_t* B, int ldb, uint16_t* X, int ldx,
                                             int mk, int nk, float sc, int wave, int lane) {
  switch (mk >> 5) {  // the host admits nb * ceil(nbn / 4) <= 8
    case 1: small_bx<1, 8>(B, ldb, X, ldx, mk, nk, sc, wave, lane); break;
    case 2: small_bx<2, 4>(B, ldb, X, ldx, mk, nk, sc, wave, lane); break;
    case 3: small_bx<3, 2>(B, ldb, X, ldx, mk, nk, sc, wave, lane); break;
    default: small_bx<4, 2>(B, ldb, X, ldx, mk, nk, sc, wave, lane); break;
  }
}

// n_iter iterations from the one g describes (g.first: iteration 0, whose
// epilogues fold in the normalisation; g.x_cur: the buffer holding X).
__global__ __launch_bounds__(256) void k_ns_small(GemmArgs g, const int32_t* __restrict__ list,
                                                  const MatDev* __restrict__ mats,
                                                  const float* __restrict__ invs, int n_iter) {
  // X [mk][nk + kPad], A and B [mk][mk + kPad]: at most 66 + 34 + 34 KiB
  __shared__ __attribute__((aligned(16))) uint16_t sx[kSmallElems + kSmallM * kPad];
  __shared__ __attribute__((aligned(16))) uint16_t sa[kSmallM * (kSmallM + kPad)];
  __shared__ __attribute__((aligned(16))) uint16_t sb[kSmallM * (kSmallM + kPad)];
  const MatDev md = mats[list[blockIdx.x]];
  const int mk = md.m_k, nk = md.n_k, c8 = nk >> 3;
  const int ldx = nk + kPad, lda = mk + kPad;
  const float inv0 = g.first ? invs[md.widx] : 1.0f;
  const uint16_t* Xin = static_cast<const uint16_t*>(g.ws) + (g.x_cur ? md.ws_x[1] : md.ws_x[0]);
  uint16_t* Xout = static_cast<uint16_t*>(g.ws) + (((g.x_cur + n_iter) & 1) ? md.ws_x[1] : md.ws_x[0]);
  // X in: every load of the thread in flight before the first LDS write
  // (at most kSmallElems / 8 / 256 = 16 per thread)
  {
    constexpr int kLoads = kSmallElems / 8 / 256;
    u32x4_t buf[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int v = threadIdx.x + 256 * u;
      if (v < mk * c8) {
        const int r = v / c8, c = (v - r * c8) * 8;
        buf[u] = *reinterpret_cast<const u32x4_t*>(Xin + panel_off(r, c, md.m_pad));
      }
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int v = threadIdx.x + 256 * u;
      if (v < mk * c8) {
        const int r = v / c8, c = (v - r * c8) * 8;
        *reinterpret_cast<u32x4_t*>(sx + r * ldx + c) = buf[u];
      }
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = mk >> 5;
  for (int it = 0; it < n_iter; ++it) {
    const float inv = it == 0 ? inv0 : 1.0f;
    const float s2 = inv * inv;
    if (g.c != 0.0f) {
      small_nt<false>(sx, ldx, nk, nb, g.e1_scale * s2, 0.0f, nullptr, g.e1_diag, sa, lda, wave,
                      lane);
      __syncthreads();
      small_mirror(sa, lda, mk);
      __syncthreads();
      small_nt<true>(sa, lda, mk, nb, g.e2_scale, g.b, sa, g.e2_diag, sb, lda, wave, lane);
    } else {
      small_nt<false>(sx, ldx, nk, nb, g.e1_scale * s2, 0.0f, nullptr, g.e1_diag, sb, lda, wave,
                      lane);
    }
    __syncthreads();
    small_mirror(sb, lda, mk);
    __syncthreads();
    small_bx_any(sb, lda, sx, ldx, mk, nk, inv, wave, lane);
    __syncthreads();
  }
  __syncthreads();
  for (int v = threadIdx.x; v < mk * c8; v += 256) {
    const int r = v / c8, c = (v - r * c8) * 8;
    *reinterpret_cast<u32x4_t*>(Xout + panel_off(r, c, md.m_pad)) =
        *reinterpret_cast<const u32x4_t*>(sx + r * ldx + c);
  }
}

}  // namespace

hipError_t launch_ns_small(int n_mats, const int32_t* list, int n_iter, const GemmArgs& args,
                           hipStream_t s) {
  if (n_mats == 0 || n_iter == 0) return hipSuccess;
  hipLaunchKernelGGL(k_ns_small, dim3(n_mats), dim3(256), 0, s, args, list, args.mats, args.inv,
                     n_iter);
  return hipGetLastError();
}

}  // namespace muon
