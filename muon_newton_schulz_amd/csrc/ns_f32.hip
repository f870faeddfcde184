// fp32 Newton-Schulz engine for gfx950: the tolerance path of the NS
// phases (optimizer tutorial, section 4.2, generalised to
// X <- a X + (b A + c A A) X with A = X X^T), on the fp32 matrix cores.
// Same phases, workspace and tile lists as the bf16 engine (ns_gemm.hip),
// with 64x64 tiles over a row-major fp32 workspace ([m_pad][ld]):
//   phase 1  A = s2 X X^T, or B = a I + b s2 X X^T when c == 0
//            (upper-triangle tiles, each also written mirrored)
//   phase 2  B = a I + b A + c A A   (same scheme)
//   phase 3  X' = xs (B X)
// with s2 = inv^2 and xs = inv on the first iteration (the Frobenius
// normalisation folded in), 1 otherwise.
#include "muon_internal.h"

namespace muon {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// The fp32 NS path (the 1e-4 tolerance path) on the fp32 matrix cores:
// 64x64 tiles, 4 waves in a 2x2 grid, each wave one 32x32 block of
// v_mfma_f32_32x32x2_f32 (fp32 products, fp32 accumulation).  Operands
// go through LDS in chunks of FK k, double buffered: the next chunk's
// global loads are in flight while the current chunk's MFMAs run.
// Within a chunk a group of 8 k runs as four MFMAs, and lane l of MFMA s
// supplies k = 4 (l / 32) + s of the group in the instruction's k slot
// l / 32.  Both operands use that assignment, so each k of the group is
// summed exactly once, and one 16-byte LDS read of 4 consecutive k gives
// a lane its K-contiguous operand for all four MFMAs.
// Accumulator layout (A operand = P rows i, B operand = Q columns j): lane
// l holds column j = l % 32 of the block and rows
// i = 8 (v / 4) + 4 (l / 32) + v % 4, v = 0..15.

constexpr int FT = kTileFp32;  // 64
constexpr int FK = 32;         // k per chunk
// LDS row strides (floats): a K-contiguous [64 rows][FK] tile is padded to
// FK + 4, so that the 16-byte reads of 16 consecutive rows fall on distinct
// banks; phase 3's [FK k][64 j] tile to FT + 8, so that the single-float
// reads of k rows r and r + 4 (the two lane halves) are 32 banks apart.
constexpr int FPS = FK + 4;
constexpr int FQS = FT + 8;

template <int PHASE>
__global__ __launch_bounds__(256) void k_ns_f32(GemmArgs g) {
  constexpr int QSZ = PHASE == 3 ? FK * FQS : FT * FPS;
  __shared__ __attribute__((aligned(16))) float Ps[2][FT * FPS];
  __shared__ __attribute__((aligned(16))) float Qs[2][QSZ];
  const Item it = g.items[blockIdx.x];
  if (it.mat < 0) return;  // padding of the XCD-grouped order
  const MatDev md = g.mats[it.mat];
  const int ti = it.rc >> 16, tj = it.rc & 0xffff;
  float* ws = static_cast<float*>(g.ws);
  const float *P, *Q;
  int ldp, ldq, K;
  if (PHASE == 1) {
    ldp = ldq = K = md.n_pad;
    P = ws + (g.x_cur ? md.ws_x[1] : md.ws_x[0]) + static_cast<int64_t>(ti) * FT * ldp;
    Q = ws + (g.x_cur ? md.ws_x[1] : md.ws_x[0]) + static_cast<int64_t>(tj) * FT * ldq;
  } else if (PHASE == 2) {
    ldp = ldq = K = md.m_pad;
    P = ws + md.ws_a + static_cast<int64_t>(ti) * FT * ldp;
    Q = ws + md.ws_a + static_cast<int64_t>(tj) * FT * ldq;
  } else {
    ldp = K = md.m_pad;
    ldq = md.n_pad;
    P = ws + md.ws_b + static_cast<int64_t>(ti) * FT * ldp;
    Q = ws + (g.x_cur ? md.ws_x[1] : md.ws_x[0]) + static_cast<int64_t>(tj) * FT;  // [k][j] column block
  }
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wi = wave & 1, wj = wave >> 1;  // this wave's block: rows 32 wi, columns 32 wj
  // global -> LDS, FK / 16 pieces of 16 bytes per operand and thread;
  // piece p = t + 256 h: row p / (FK / 4), k 4 (p % (FK / 4)) of a
  // K-contiguous tile, or k row p / 16, columns 4 (p % 16) of phase 3's
  // [k][j] tile
  constexpr int NPC = FK / 16;
  static_assert(FK % 16 == 0 && FT % FK == 0, "a chunk is whole 16-byte pieces, K a multiple of it");
  f32x4_t pr[NPC], qr[NPC];
  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < NPC; ++h) {
      const int pc = t + 256 * h;
      const int r = pc / (FK / 4), kk = 4 * (pc % (FK / 4));
      pr[h] = *reinterpret_cast<const f32x4_t*>(P + static_cast<int64_t>(r) * ldp + k0 + kk);
      if (PHASE != 3)
        qr[h] = *reinterpret_cast<const f32x4_t*>(Q + static_cast<int64_t>(r) * ldq + k0 + kk);
      else
        qr[h] = *reinterpret_cast<const f32x4_t*>(Q + static_cast<int64_t>(k0 + (pc >> 4)) * ldq +
                                                  4 * (pc & 15));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int h = 0; h < NPC; ++h) {
      const int pc = t + 256 * h;
      const int r = pc / (FK / 4), kk = 4 * (pc % (FK / 4));
      *reinterpret_cast<f32x4_t*>(&Ps[buf][r * FPS + kk]) = pr[h];
      if (PHASE != 3)
        *reinterpret_cast<f32x4_t*>(&Qs[buf][r * FPS + kk]) = qr[h];
      else
        *reinterpret_cast<f32x4_t*>(&Qs[buf][(pc >> 4) * FQS + 4 * (pc & 15)]) = qr[h];
    }
  };
  // this lane's operand positions within a chunk (k 4 (lane / 32) of each
  // group of 8)
  const int row = lane & 31, kh = 4 * (lane >> 5);
  const int pa = (wi * 32 + row) * FPS + kh;
  const int qa = PHASE == 3 ? kh * FQS + wj * 32 + row : (wj * 32 + row) * FPS + kh;

  f32x16_t acc = {};
  const int nc = K / FK;
  load(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    const int buf = c & 1;
    if (c + 1 < nc) load((c + 1) * FK);  // in flight during this chunk's MFMAs
    const float* ps = &Ps[buf][pa];
    const float* qs = &Qs[buf][qa];
#pragma unroll
    for (int grp = 0; grp < FK / 8; ++grp) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(ps + 8 * grp);
      f32x4_t b;
      if (PHASE != 3) {
        b = *reinterpret_cast<const f32x4_t*>(qs + 8 * grp);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) b[s] = qs[(8 * grp + s) * FQS];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
    }
    if (c + 1 < nc) store(buf ^ 1);
    __syncthreads();
  }

  const float inv = g.first ? g.inv[md.widx] : 1.0f;
  // rows i0 + 8 (v / 4) + v % 4 of column j of the output
  const int i0 = ti * FT + wi * 32 + 4 * (lane >> 5), j = tj * FT + wj * 32 + row;
  if (PHASE == 3) {
    float* X = ws + (g.x_cur ? md.ws_x[0] : md.ws_x[1]);
#pragma unroll
    for (int v = 0; v < 16; ++v)
      X[static_cast<int64_t>(i0 + 8 * (v >> 2) + (v & 3)) * md.n_pad + j] = inv * acc[v];
    return;
  }
  const int ldc = md.m_pad;
  float* C = ws + ((PHASE == 1 && g.c != 0.0f) ? md.ws_a : md.ws_b);
  const float* Aold = ws + md.ws_a;
  const float s2 = inv * inv;
  f32x16_t x;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int i = i0 + 8 * (v >> 2) + (v & 3);
    float y;
    if (PHASE == 1) y = (g.c != 0.0f ? 1.0f : g.b) * s2 * acc[v];
    else y = g.b * Aold[static_cast<int64_t>(i) * ldc + j] + g.c * acc[v];
    if ((PHASE == 2 || g.c == 0.0f) && i == j) y += g.a;
    x[v] = y;
  }
  // phase 2 reads A and writes B, phase 1 (c != 0) writes A: distinct buffers
#pragma unroll
  for (int v = 0; v < 16; ++v)
    C[static_cast<int64_t>(i0 + 8 * (v >> 2) + (v & 3)) * ldc + j] = x[v];
  if (ti != tj) {
    // mirror: C[j][i..i+3] for each group of four rows
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4_t*>(C + static_cast<int64_t>(j) * ldc + i0 + 8 * q) =
          f32x4_t{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
  }
}

}  // namespace

hipError_t launch_ns_f32(int phase, int n_items, const GemmArgs& args, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(n_items), block(256);
  if (phase == 1) hipLaunchKernelGGL(k_ns_f32<1>, grid, block, 0, s, args);
  else if (phase == 2) hipLaunchKernelGGL(k_ns_f32<2>, grid, block, 0, s, args);
  else hipLaunchKernelGGL(k_ns_f32<3>, grid, block, 0, s, args);
  return hipGetLastError();
}

}  // namespace muon
