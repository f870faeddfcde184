// Grouped, ragged Newton-Schulz engine for gfx950.
//
// One NS iteration (optimizer tutorial, section 4.2, generalised to
// X <- a X + (b A + c A A) X with A = X X^T) is three grouped launches over
// every matrix of a wave:
//   phase 1  A = s2 * X X^T        symmetric: one triangle of tiles, each
//                                  tile written to (i,j) and mirrored to (j,i)
//   phase 2  B = b A + c A A       symmetric (A A = A A^T), same scheme
//   phase 3  X <- xs*(a X + B X)   (with c == 0 the product is b*(A X))
// On the first iteration s2 = inv^2 and xs = inv, which folds the
// Frobenius normalisation X0 = U/(||U||_F + eps) into the GEMM epilogues.
//
// Every product is computed in "NT" form, C[i][j] = sum_k P[i][k] Q[j][k],
// with both operands K-contiguous in HBM:
//   phase 1: P = Q = X (m x n);  phase 2: P = Q = A;
//   phase 3: P = B, Q = X^T (n x m), which is why the workspace keeps the
//   iterate in both layouts.  Phase 3 writes X in place (each X tile is
//   read only by the work item that rewrites it) and X^T into the other
//   ping-pong buffer.
//
// bf16 engine: 256x256 tiles, BK = 64, 256 threads = 4 waves in a 2x2
// grid, 128x128 per wave as 4x4 blocks of v_mfma_f32_32x32x16_bf16 with
// fp32 accumulation; operands double-buffered in LDS (2 x 64 KiB) with an
// XOR swizzle of the 16-byte chunks, so both the global->LDS stores and
// the per-lane fragment reads are free of bank conflicts.
// fp32 engine (tolerance path): 64x64 tiles of plain FMA.
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BT = kTileBf16;  // 256
constexpr int BK = 64;

struct Operands {
  const uint16_t* P;
  const uint16_t* Q;
  int ld;  // = K
};

template <int PHASE>
__device__ __forceinline__ void phase_operands(const GemmArgs& g, const MatDev& md, int ti,
                                               int tj, const uint16_t* ws, const uint16_t*& P,
                                               const uint16_t*& Q, int& ld) {
  if (PHASE == 1) {
    ld = md.n_pad;
    P = ws + md.ws_x + static_cast<int64_t>(ti) * BT * ld;
    Q = ws + md.ws_x + static_cast<int64_t>(tj) * BT * ld;
  } else if (PHASE == 2) {
    ld = md.m_pad;
    P = ws + md.ws_a + static_cast<int64_t>(ti) * BT * ld;
    Q = ws + md.ws_a + static_cast<int64_t>(tj) * BT * ld;
  } else {
    ld = md.m_pad;
    P = ws + (g.c != 0.0f ? md.ws_b : md.ws_a) + static_cast<int64_t>(ti) * BT * ld;
    Q = ws + md.ws_xt[g.xt_cur] + static_cast<int64_t>(tj) * BT * ld;
  }
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  uint2 r;
  r.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
  r.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
  return r;
}
__device__ __forceinline__ void unpack4(uint2 r, float* o) {
  o[0] = __uint_as_float(r.x << 16);
  o[1] = __uint_as_float(r.x & 0xffff0000u);
  o[2] = __uint_as_float(r.y << 16);
  o[3] = __uint_as_float(r.y & 0xffff0000u);
}

template <int PHASE>
__global__ __launch_bounds__(256, 1) void k_ns_bf16(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * BT * BK];  // 128 KiB
  const Item it = g.items[blockIdx.x];
  const MatDev md = g.mats[it.mat];
  const int ti = it.rc >> 16, tj = it.rc & 0xffff;
  const uint16_t* ws = static_cast<const uint16_t*>(g.ws);
  const uint16_t *P, *Q;
  int ld;
  phase_operands<PHASE>(g, md, ti, tj, ws, P, Q, ld);

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wi = wv & 1, wj = wv >> 1;

  // global -> LDS mapping: 8 threads per 128-byte row segment, 32 rows per
  // pass, 8 passes per operand
  const int lrow = t >> 3, lchunk = t & 7;
  const int swz_st = (lchunk ^ (lrow & 7)) << 3;
  const uint16_t* Pg = P + static_cast<int64_t>(lrow) * ld + lchunk * 8;
  const uint16_t* Qg = Q + static_cast<int64_t>(lrow) * ld + lchunk * 8;
  const int64_t row32 = static_cast<int64_t>(32) * ld;

  u32x4_t rp[8], rq[8];
  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

#pragma unroll
  for (int r = 0; r < 8; ++r) {
    rp[r] = *reinterpret_cast<const u32x4_t*>(Pg + r * row32);
    rq[r] = *reinterpret_cast<const u32x4_t*>(Qg + r * row32);
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    *reinterpret_cast<u32x4_t*>(smem + (lrow + 32 * r) * BK + swz_st) = rp[r];
    *reinterpret_cast<u32x4_t*>(smem + BT * BK + (lrow + 32 * r) * BK + swz_st) = rq[r];
  }
  __syncthreads();

  const int nk = ld / BK;
  const int frow = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = (kt + 1) * BK;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        rp[r] = *reinterpret_cast<const u32x4_t*>(Pg + r * row32 + k0);
        rq[r] = *reinterpret_cast<const u32x4_t*>(Qg + r * row32 + k0);
      }
    }
    const uint16_t* sp = smem + buf * 2 * BT * BK;
    const uint16_t* sq = sp + BT * BK;
    // fragments of k-substep ks+1 are read from LDS while the 16 MFMAs of
    // substep ks run
    bf16x8_t qf[2][4], pf[2][4];
    auto read_frags = [&](int ks, bf16x8_t* q, bf16x8_t* p) {
      const int kc = ks * 2 + (lane >> 5);
      const int sw = (kc ^ (lane & 7)) << 3;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        q[b] = *reinterpret_cast<const bf16x8_t*>(sq + (wj * 128 + b * 32 + frow) * BK + sw);
        p[b] = *reinterpret_cast<const bf16x8_t*>(sp + (wi * 128 + b * 32 + frow) * BK + sw);
      }
    };
    read_frags(0, qf[0], pf[0]);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) read_frags(ks + 1, qf[(ks + 1) & 1], pf[(ks + 1) & 1]);
      // keep the reads above ahead of this substep's MFMAs
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
          acc[bj][bi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks & 1][bj], pf[ks & 1][bi],
                                                                acc[bj][bi], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) {
      uint16_t* dp = smem + (buf ^ 1) * 2 * BT * BK;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        *reinterpret_cast<u32x4_t*>(dp + (lrow + 32 * r) * BK + swz_st) = rp[r];
        *reinterpret_cast<u32x4_t*>(dp + BT * BK + (lrow + 32 * r) * BK + swz_st) = rq[r];
      }
    }
    __syncthreads();
  }

  // ---- epilogue.  Accumulator layout of the 32x32 MFMA (A operand = Q
  // rows j, B operand = P rows i): lane holds column i = lane%32 and rows
  // j = 8*(v/4) + 4*(lane/32) + v%4, i.e. C[i][j..j+3] for each v/4.
  uint16_t* wsw = static_cast<uint16_t*>(g.ws);
  const int ib = ti * BT + wi * 128 + frow;
  const int jb = tj * BT + wj * 128 + 4 * (lane >> 5);
  const float inv = g.first ? g.inv[md.widx] : 1.0f;
  if (PHASE == 1 || PHASE == 2) {
    const int ldc = md.m_pad;
    uint16_t* C = wsw + (PHASE == 1 ? md.ws_a : md.ws_b);
    const uint16_t* Aold = wsw + md.ws_a;
    const float s2 = inv * inv;
    const bool mirror = ti != tj;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = ib + bi * 32;
          const int j = jb + bj * 32 + 8 * q;
          float v[4];
          if (PHASE == 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = s2 * acc[bj][bi][4 * q + e];
          } else {
            float a0[4];
            unpack4(*reinterpret_cast<const uint2*>(Aold + static_cast<int64_t>(i) * ldc + j), a0);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = g.b * a0[e] + g.c * acc[bj][bi][4 * q + e];
          }
          const uint2 pk = pack4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<uint2*>(C + static_cast<int64_t>(i) * ldc + j) = pk;
          if (mirror) {
            C[static_cast<int64_t>(j + 0) * ldc + i] = static_cast<uint16_t>(pk.x & 0xffffu);
            C[static_cast<int64_t>(j + 1) * ldc + i] = static_cast<uint16_t>(pk.x >> 16);
            C[static_cast<int64_t>(j + 2) * ldc + i] = static_cast<uint16_t>(pk.y & 0xffffu);
            C[static_cast<int64_t>(j + 3) * ldc + i] = static_cast<uint16_t>(pk.y >> 16);
          }
        }
  } else {
    const int ldx = md.n_pad, ldt = md.m_pad;
    uint16_t* X = wsw + md.ws_x;
    uint16_t* XT = wsw + md.ws_xt[g.xt_cur ^ 1];
    const float alpha = g.c != 0.0f ? 1.0f : g.b;
    const bool write_x = !(g.last && md.trans);
    const bool write_xt = !(g.last && !md.trans);
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = ib + bi * 32;
          const int j = jb + bj * 32 + 8 * q;
          float x0[4], v[4];
          uint16_t* xp = X + static_cast<int64_t>(i) * ldx + j;
          unpack4(*reinterpret_cast<const uint2*>(xp), x0);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = inv * (g.a * x0[e] + alpha * acc[bj][bi][4 * q + e]);
          const uint2 pk = pack4(v[0], v[1], v[2], v[3]);
          if (write_x) *reinterpret_cast<uint2*>(xp) = pk;
          if (write_xt) {
            XT[static_cast<int64_t>(j + 0) * ldt + i] = static_cast<uint16_t>(pk.x & 0xffffu);
            XT[static_cast<int64_t>(j + 1) * ldt + i] = static_cast<uint16_t>(pk.x >> 16);
            XT[static_cast<int64_t>(j + 2) * ldt + i] = static_cast<uint16_t>(pk.y & 0xffffu);
            XT[static_cast<int64_t>(j + 3) * ldt + i] = static_cast<uint16_t>(pk.y >> 16);
          }
        }
  }
}

// ------------------------------------------------------------ fp32 engine

constexpr int FT = kTileFp32;  // 64
constexpr int FK = 16;

template <int PHASE>
__global__ __launch_bounds__(256) void k_ns_f32(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) float Ps[FK][FT + 4];
  __shared__ __attribute__((aligned(16))) float Qs[FK][FT + 4];
  const Item it = g.items[blockIdx.x];
  const MatDev md = g.mats[it.mat];
  const int ti = it.rc >> 16, tj = it.rc & 0xffff;
  float* ws = static_cast<float*>(g.ws);
  const float *P, *Q;
  int ld;
  if (PHASE == 1) {
    ld = md.n_pad;
    P = ws + md.ws_x + static_cast<int64_t>(ti) * FT * ld;
    Q = ws + md.ws_x + static_cast<int64_t>(tj) * FT * ld;
  } else if (PHASE == 2) {
    ld = md.m_pad;
    P = ws + md.ws_a + static_cast<int64_t>(ti) * FT * ld;
    Q = ws + md.ws_a + static_cast<int64_t>(tj) * FT * ld;
  } else {
    ld = md.m_pad;
    P = ws + (g.c != 0.0f ? md.ws_b : md.ws_a) + static_cast<int64_t>(ti) * FT * ld;
    Q = ws + md.ws_xt[g.xt_cur] + static_cast<int64_t>(tj) * FT * ld;
  }
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  const int lrow = t >> 2, lk = (t & 3) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < ld; k0 += FK) {
    const float4 pv = *reinterpret_cast<const float4*>(P + static_cast<int64_t>(lrow) * ld + k0 + lk);
    const float4 qv = *reinterpret_cast<const float4*>(Q + static_cast<int64_t>(lrow) * ld + k0 + lk);
    __syncthreads();
    Ps[lk + 0][lrow] = pv.x; Ps[lk + 1][lrow] = pv.y; Ps[lk + 2][lrow] = pv.z; Ps[lk + 3][lrow] = pv.w;
    Qs[lk + 0][lrow] = qv.x; Qs[lk + 1][lrow] = qv.y; Qs[lk + 2][lrow] = qv.z; Qs[lk + 3][lrow] = qv.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FK; ++k) {
      const float4 pa = *reinterpret_cast<const float4*>(&Ps[k][ty * 4]);
      const float4 qa = *reinterpret_cast<const float4*>(&Qs[k][tx * 4]);
      const float p4[4] = {pa.x, pa.y, pa.z, pa.w};
      const float q4[4] = {qa.x, qa.y, qa.z, qa.w};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(p4[a], q4[b], acc[a][b]);
    }
  }
  const float inv = g.first ? g.inv[md.widx] : 1.0f;
  const int i0 = ti * FT + ty * 4, j0 = tj * FT + tx * 4;
  if (PHASE == 1 || PHASE == 2) {
    const int ldc = md.m_pad;
    float* C = ws + (PHASE == 1 ? md.ws_a : md.ws_b);
    const float* Aold = ws + md.ws_a;
    const float s2 = inv * inv;
    float v[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (PHASE == 2) a0 = *reinterpret_cast<const float4*>(Aold + static_cast<int64_t>(i0 + a) * ldc + j0);
      const float ao[4] = {a0.x, a0.y, a0.z, a0.w};
#pragma unroll
      for (int b = 0; b < 4; ++b)
        v[a][b] = PHASE == 1 ? s2 * acc[a][b] : g.b * ao[b] + g.c * acc[a][b];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<float4*>(C + static_cast<int64_t>(i0 + a) * ldc + j0) =
          make_float4(v[a][0], v[a][1], v[a][2], v[a][3]);
    if (ti != tj) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<float4*>(C + static_cast<int64_t>(j0 + b) * ldc + i0) =
            make_float4(v[0][b], v[1][b], v[2][b], v[3][b]);
    }
  } else {
    const int ldx = md.n_pad, ldt = md.m_pad;
    float* X = ws + md.ws_x;
    float* XT = ws + md.ws_xt[g.xt_cur ^ 1];
    const float alpha = g.c != 0.0f ? 1.0f : g.b;
    float v[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 x0 = *reinterpret_cast<const float4*>(X + static_cast<int64_t>(i0 + a) * ldx + j0);
      const float xo[4] = {x0.x, x0.y, x0.z, x0.w};
#pragma unroll
      for (int b = 0; b < 4; ++b) v[a][b] = inv * (g.a * xo[b] + alpha * acc[a][b]);
    }
    if (!(g.last && md.trans)) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(X + static_cast<int64_t>(i0 + a) * ldx + j0) =
            make_float4(v[a][0], v[a][1], v[a][2], v[a][3]);
    }
    if (!(g.last && !md.trans)) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<float4*>(XT + static_cast<int64_t>(j0 + b) * ldt + i0) =
            make_float4(v[0][b], v[1][b], v[2][b], v[3][b]);
    }
  }
}

}  // namespace

hipError_t launch_ns_phase(int ns_dtype, int phase, int n_items, const GemmArgs& args,
                           hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(n_items), block(256);
  if (ns_dtype == 1) {
    if (phase == 1) hipLaunchKernelGGL(k_ns_bf16<1>, grid, block, 0, s, args);
    else if (phase == 2) hipLaunchKernelGGL(k_ns_bf16<2>, grid, block, 0, s, args);
    else hipLaunchKernelGGL(k_ns_bf16<3>, grid, block, 0, s, args);
  } else {
    if (phase == 1) hipLaunchKernelGGL(k_ns_f32<1>, grid, block, 0, s, args);
    else if (phase == 2) hipLaunchKernelGGL(k_ns_f32<2>, grid, block, 0, s, args);
    else hipLaunchKernelGGL(k_ns_f32<3>, grid, block, 0, s, args);
  }
  return hipGetLastError();
}

}  // namespace muon
