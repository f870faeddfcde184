// Grouped, ragged Newton-Schulz engine for gfx950.
//
// One NS iteration (optimizer tutorial, section 4.2, generalised to
// X <- a X + (b A + c A A) X with A = X X^T) runs as grouped launches over
// every matrix of a wave:
//   phase 1  A = s2 * X X^T          symmetric: upper-triangle tiles, each
//                                    written at (i,j) and mirrored to (j,i)
//   phase 2  B = a I + b A + c A A   symmetric (A A = A A^T), same scheme;
//                                    skipped when c == 0, in which case
//                                    phase 1 writes B = a I + b s2 X X^T
//   phase 3  X' = xs * (B X)         the a X term is folded into B's diagonal
// On the first iteration s2 = inv^2 and xs = inv, which folds the
// Frobenius normalisation X0 = U/(||U||_F + eps) into the epilogues.
// X lives in two ping-pong buffers (m x n, padded; the padding inside the
// contraction extents m_k, n_k is zero).  X, A and B are stored as panels
// of 32 columns (panel_off in muon_internal.h): one stage of 256 rows x 32
// k of an operand read along its rows is 16 KiB of contiguous memory, so
// the operand loads read whole 128-byte lines (row-major storage gave each
// load instruction 16 half lines).
// The last phase 3 of a step can instead apply the update to the
// parameters, W <- (1 - lr wd) W - lr s O with O the bf16 value X' would
// hold (k_ns_bf16_apply; optimizer tutorial 3.1, decoupled decay).
//
// Phases 1 and 2 are "NT" products, C[i][j] = sum_k P[i][k] Q[j][k], with
// both operands K-contiguous.  Phase 3 is "NN": P = B (K-contiguous rows),
// Q = X stored [k][j]; its MFMA fragments (8 consecutive k of one column)
// are read from LDS with ds_read_b64_tr_b16, so no transposed copy of X is
// ever written.
//
// bf16 engine: 256x256 tiles, 256 threads = 4 waves in a 2x2 grid,
// 128x128 per wave as 4x4 blocks of v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  Operands stream HBM -> LDS with global_load_lds (16 bytes
// per lane, no VGPR staging) through a ring of 4 slots of 32 K-columns
// (4 x 32 KiB), three stages in flight: the operand loads see L2 latencies
// of several hundred cycles and one stage in flight cannot cover them.
// LDS has 64 banks (256 bytes per cycle), and the layouts are swizzled so
// that the DMA writes, ds_read_b128 and the transpose reads are free of
// bank conflicts:
//   K-contiguous tile [256 rows][32 k]: 16-byte chunk c of row r at
//     position c ^ ((r >> 2) & 3);
//   [k][j] tile [32 k][256 j]: 32-column block q of row k at q ^ (k & 3).
// The epilogue stages each wave's 128x128 result in LDS (8-byte slot s of
// row i at s ^ g(i), g(i) = ((i & 3) << 3) | ((i >> 2) & 7)) and writes it
// with 16-byte row stores; the symmetric mirror is read back transposed
// with ds_read_b64_tr_b16 and also written in 16-byte pieces.
//
// The fp32 engine (the tolerance path) is in ns_f32.hip.
#include <type_traits>

#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* gbl_void_t;

constexpr int BT = kTileBf16;  // 256
constexpr int BK = kNsKStep;     // K per pipeline stage (32)
constexpr int NSLOT = 4;         // LDS ring slots (stages in flight: NSLOT - 1)
constexpr int DMA_PER_STAGE = 8;  // DMA instructions per wave per stage

// 16 bytes per lane, HBM -> LDS; lane l's data lands at lds + 16*l.  The
// source is a wave-uniform base plus a 32-bit per-lane byte offset, the
// instruction's SGPR-base + VGPR-offset form: advancing a stage is scalar
// arithmetic only.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint16_t* lds_wave_uniform) {
  // one opaque 64-bit scalar, so that the address is matched as
  // SGPR base + zero-extended VGPR offset
  uint64_t sbase = reinterpret_cast<uint64_t>(base);
  asm("" : "+s"(sbase));
  __builtin_amdgcn_global_load_lds((gbl_void_t)(reinterpret_cast<const char*>(sbase) + voff),
                                   (lds_void_t)lds_wave_uniform, 16, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t)p));
}

// LDS fragment reads are issued as inline asm: the compiler's wait-count
// pass would otherwise make every LDS read wait for all LDS DMA (and, for
// the transpose read, all global stores) in flight, which drains the
// pipelines.  Their completion is awaited explicitly (wait_frags,
// wait_lds16) before use.  OFF is the instruction's immediate byte offset.
// Transpose read: within each group of 16 lanes, lane l receives element
// (l % 4) of the 8-byte blocks addressed by lanes 4q + l/4, q = 0..3.
template <int OFF>
__device__ __forceinline__ s16x4_t ld_tr_async(uint32_t addr) {
  s16x4_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ bf16x8_t ld128_async(uint32_t addr) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
  return __builtin_bit_cast(bf16x8_t, r);
}

template <int N>
using Int = std::integral_constant<int, N>;

// f(Int<I>{}), ..., f(Int<N-1>{}): loop bodies that need the index as a
// compile-time constant (immediate offsets, register-array indices).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for<I + 1, N>(f);
  }
}
// Wait until this wave's DMA for stage `st` has landed, given that stages
// up to `newest` have been issued (DPS instructions each); the newer
// stages may stay in flight (vmcnt counts vector memory instructions,
// which complete in issue order).
template <int DPS>
__device__ __forceinline__ void wait_stage_landed(int st, int newest) {
  static_assert(NSLOT == 4, "wait counts below assume at most 3 newer stages");
  const int newer = newest - st;
  if (newer >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * DPS) : "memory");
  else if (newer == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DPS) : "memory");
  else if (newer == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DPS) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Bare workgroup barrier for the operand pipeline.  A fenced barrier
// (__syncthreads) makes the compiler wait for every vector memory
// instruction in flight first (vmcnt(0)), LDS DMA included, which would
// drain the pipeline.  Here nothing else is needed: each wave has waited
// for its own DMA of the stage (wait_stage_landed) and for its own
// fragment reads (wait_frags) before it arrives.
__device__ __forceinline__ void pipe_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most N LDS reads are outstanding; the fragments are tied
// to the wait so that their consumers cannot be scheduled above it.
template <int N>
__device__ __forceinline__ void wait_frags(bf16x8_t* q, bf16x8_t* p) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(p[0]), "+v"(p[1]),
                 "+v"(p[2]), "+v"(p[3])
               : "n"(N)
               : "memory");
}

// Same for the transposed halves of phase 3 (the Q fragments are
// assembled from them only after the wait).
template <int N>
__device__ __forceinline__ void wait_frags_tr(s16x4_t* t, bf16x8_t* p) {
  asm volatile("s_waitcnt lgkmcnt(%12)"
               : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]),
                 "+v"(t[6]), "+v"(t[7]), "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3])
               : "n"(N)
               : "memory");
}

// All LDS reads done, tied to the 16 results (epilogue transpose reads).
__device__ __forceinline__ void wait_lds16(s16x4_t* t) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]),
                 "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]),
                 "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               :
               : "memory");
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Fused update of 8 bf16 parameters: W' = decay W - step O, O the 8 bf16
// values phase 3 would store (the apply kernel's arithmetic, same bits).
__device__ __forceinline__ u32x4_t apply8(const ApplyConsts& k, u32x4_t w, u32x4_t o) {
  u32x4_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = pack2(apply_one(k, lo_bf(w[e]), lo_bf(o[e])), apply_one(k, hi_bf(w[e]), hi_bf(o[e])));
  return r;
}

// The lane id, hidden from the optimiser (see the epilogue).
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

// staging layout of a wave's 128x128 bf16 result: element offset of the
// 4-element (8-byte) slot holding (i, j..j+3), j % 4 == 0
__device__ __forceinline__ int stg(int i, int j) {
  const int g = ((i & 3) << 3) | ((i >> 2) & 7);
  return i * 128 + ((((j >> 2) ^ g) & 31) << 2);
}

// Eight consecutive staged values of row i from any column c (c <= 120):
// the three 4-element slots from c/4 on, shifted by c%4 elements.
__device__ __forceinline__ u32x4_t stg_read8(const uint16_t* S, int i, int c) {
  const int a = c & ~3, b = c & 3;
  const u32x2_t s0 = *reinterpret_cast<const u32x2_t*>(S + stg(i, a));
  const u32x2_t s1 = *reinterpret_cast<const u32x2_t*>(S + stg(i, a + 4));
  const u32x2_t s2 = *reinterpret_cast<const u32x2_t*>(S + stg(i, a + 8 < 128 ? a + 8 : 124));
  const uint32_t w[6] = {s0[0], s0[1], s1[0], s1[1], s2[0], s2[1]};
  const uint32_t sh = (b & 1) * 16;  // element b starts in word b/2 at bit 16 (b%2)
  u32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = (b >> 1) ? __builtin_amdgcn_alignbit(w[k + 2], w[k + 1], sh)
                    : __builtin_amdgcn_alignbit(w[k + 1], w[k], sh);
  return o;
}

// Split tiles.  Diagonal tiles of the symmetric products (phases 1, 2) need
// only the 36 upper 32x32 blocks of their 8x8.  ROLE 1, waves (0,0) and
// (1,1): the upper blocks of their quadrant (bi <= bj, 10 of 16).  ROLE 2:
// wave (0,1) the left half of quadrant (0,1) (bj < 2, 8 blocks), wave (1,0)
// the same on Q rows 64 further, i.e. that quadrant's right half.  Every
// wave writes its blocks and, mirrored, their transposes, so a diagonal tile
// costs 10 MFMA slots per substep instead of 16.
// Edge tiles whose last 128 rows (ROLE 3, phase 3: the m side) or columns
// (ROLE 4: the Q side) are all padding: the four waves split the two
// quadrants that hold data, 64 Q rows each, as ROLE 2 splits one, so the
// tile costs 8 MFMA slots per substep; only on matrices with at most
// kSplitEdgeMaxTiles tiles per side (on larger ones they measured
// slower).  ROLE 0: the whole quadrant.  Only matrices with MatDev::split
// take split tiles.
__device__ __forceinline__ int tile_role(int phase, const MatDev& md, int ti, int tj, int wave) {
  if (!md.split) return 0;
  if (phase != 3 && ti == tj) return (wave == 0 || wave == 3) ? 1 : 2;
  if (md.m_pad > kSplitEdgeMaxTiles * BT) return 0;
  const int m = md.rows < md.cols ? md.rows : md.cols;
  const int n = md.rows < md.cols ? md.cols : md.rows;
  if (phase == 3 && m - ti * BT <= BT / 2) return 3;
  if ((phase == 3 ? n : m) - tj * BT <= BT / 2) return 4;
  return 0;
}

// The fused update of a matrix whose W rows are off the flat buffer's
// 8-element grid (offset or cols not a multiple of 8).  A W row of the
// wave's sub-tile is a tile row (wide matrix) or a tile column (tall
// matrix): W row RB + r, r < 128 (64 rows of a tall matrix's split-role
// wave), columns CB .. CB + len - 1.  Its flat range splits into 16-byte
// pieces on the grid (piece t at column c0 + 8t) and at most 7 + 7
// parameters before and after them, written one by one (2-byte stores
// touch no parameter of a neighbouring tile).  Lane slot u takes row
// r = lane/16 + 4u: piece t = lane % 16, and the parameter t before the
// pieces (t < 8) or t - 8 after them.  After the staging, every W load
// goes out first (offgrid_load, then the single parameters'), and O is
// read at the same positions (offgrid_update); holding W in registers
// across the last K stage or the staging loop spilled.  A tall matrix's W
// row is a staged column, read one value per row.  Same arithmetic as the
// apply kernel:
// W' = fma(-step, O, decay W) rounded to bf16.  The 16-byte alignment of
// the parameter buffer is the caller's (the host checks it).
struct OffgridRow {
  const uint16_t* base;  // params + row0(u), wave-uniform
  int r, lo, c0, np, hn, ts, tn;
};
struct OffgridTile {
  int RB, CB, nrows, len;
};
template <int ROLE>
__device__ __forceinline__ OffgridTile offgrid_tile(const MatDev& md, int i0w, int j0w) {
  constexpr int WC = ROLE >= 2 ? 64 : 128;  // a split-role wave's tile columns
  OffgridTile tl;
  tl.RB = md.trans ? j0w : i0w;
  tl.CB = md.trans ? i0w : j0w;
  tl.nrows = md.trans ? WC : 128;
  tl.len = min(tl.CB + (md.trans ? 128 : WC), md.cols) - tl.CB;
  return tl;
}
// Row r = ln/16 + 4u starts at flat element row0(u) + lo, with the
// wave-uniform row0(u) = off + (RB + 4u) cols + CB and the lane part
// lo = (ln/16) cols; everything per lane is 32-bit.  s: the row's shift off
// the grid, c0 = (8 - s) % 8 its first piece, np pieces, hn parameters
// before them and tn after them from column ts.  Each pass derives ln from
// its own opaque copy of the lane id, so that these values are recomputed
// rather than kept live from one pass to the next.
__device__ __forceinline__ bool offgrid_row(const MatDev& md, const OffgridTile& tl,
                                            const uint16_t* params, int ln, int u,
                                            OffgridRow& q) {
  q.r = (ln >> 4) + 4 * u;
  if (tl.len <= 0 || q.r >= tl.nrows || tl.RB + q.r >= md.rows) return false;
  const int64_t row0 = md.off + static_cast<int64_t>(tl.RB + 4 * u) * md.cols + tl.CB;
  q.base = params + row0;
  q.lo = (ln >> 4) * md.cols;
  const int sft = (static_cast<int>(row0 & 7) + (q.lo & 7)) & 7;
  q.c0 = (8 - sft) & 7;
  q.hn = min(q.c0, tl.len);
  q.np = tl.len > q.c0 ? (tl.len - q.c0) >> 3 : 0;
  q.ts = q.c0 + 8 * q.np;
  q.tn = tl.len - q.ts;
  return true;
}
__device__ __forceinline__ bool offgrid_single(const OffgridRow& q, int t, int& c) {
  c = t < 8 ? t : q.ts + t - 8;
  return t < 8 ? t < q.hn : t - 8 < q.tn;
}
template <int ROLE>
__device__ __forceinline__ void offgrid_load(const MatDev& md, const uint16_t* params, int i0w,
                                             int j0w, int lane, u32x4_t* wv) {
  const OffgridTile tl = offgrid_tile<ROLE>(md, i0w, j0w);
  const int ln = opaque_lane(lane), t = ln & 15;
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    OffgridRow q;
    if (offgrid_row(md, tl, params, ln, u, q) && t < q.np)
      wv[u] = *reinterpret_cast<const u32x4_t*>(q.base + q.lo + q.c0 + 8 * t);
  }
}
// staged O of W row r, column c: tile element (r, c) of a wide matrix,
// (c, r) of a tall one
__device__ __forceinline__ uint16_t staged_o(const uint16_t* S, bool trans, int r, int c) {
  return trans ? S[stg(c, r) + (r & 3)] : S[stg(r, c) + (c & 3)];
}
template <int ROLE>
__device__ __forceinline__ void offgrid_update(uint16_t* S, const MatDev& md, uint16_t* params,
                                               const ApplyConsts& ak, int i0w, int j0w,
                                               int elane, const u32x4_t* wv) {
  const OffgridTile tl = offgrid_tile<ROLE>(md, i0w, j0w);
  // the single parameters' loads before the pieces' stores (a load issued
  // after a store waits for it); fully unrolled passes keep wv and w1 in
  // registers
  uint16_t w1[32];
  {
    const int ln = opaque_lane(elane), t = ln & 15;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      OffgridRow q;
      int c;
      if (offgrid_row(md, tl, params, ln, u, q) && offgrid_single(q, t, c)) w1[u] = q.base[q.lo + c];
    }
  }
  {
    const int ln = opaque_lane(elane), t = ln & 15;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      OffgridRow q;
      if (!offgrid_row(md, tl, params, ln, u, q) || t >= q.np) continue;
      const int c = q.c0 + 8 * t;
      u32x4_t o;
      if (!md.trans) {
        o = stg_read8(S, q.r, c);
      } else {
        // a W row of a tall matrix is a staged column: one value per row
#pragma unroll
        for (int k = 0; k < 4; ++k)
          o[k] = static_cast<uint32_t>(staged_o(S, true, q.r, c + 2 * k)) |
                 (static_cast<uint32_t>(staged_o(S, true, q.r, c + 2 * k + 1)) << 16);
      }
      *reinterpret_cast<u32x4_t*>(const_cast<uint16_t*>(q.base) + q.lo + c) = apply8(ak, wv[u], o);
      // one slot at a time: the scheduler would otherwise hoist the LDS
      // reads of every slot (up to 8 per piece) ahead of the first store
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  {
    const int ln = opaque_lane(elane), t = ln & 15;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      OffgridRow q;
      int c;
      if (!offgrid_row(md, tl, params, ln, u, q) || !offgrid_single(q, t, c)) continue;
      const float o = bf16_to_f32(staged_o(S, md.trans, q.r, c));
      const_cast<uint16_t*>(q.base)[q.lo + c] = f32_to_bf16(apply_one(ak, bf16_to_f32(w1[u]), o));
    }
  }
}

// One 256x256 output tile: operand pipeline, MFMA main loop, epilogue.
// APPLY (phase 3 only): a matrix with MatDev::fuse gets the update applied
// to its parameters instead of X' written.
template <int PHASE, int ROLE, bool APPLY = false>
__device__ __forceinline__ void ns_tile(const GemmArgs& g, const MatDev& md, const int ti,
                                        const int tj, const float inv, uint16_t* smem) {
  // MFMA m = 4 bj + bi runs iff bit m is set
  constexpr uint32_t MASK = ROLE == 0 ? 0xFFFFu : ROLE == 1 ? 0xF731u : 0x00FFu;
  static_assert(ROLE <= 2 || (ROLE == 3 ? PHASE == 3 : true), "half-height tiles are phase 3's");
  // A guarded step that is skipped leaves W untouched: a matrix whose
  // update this tile would apply needs none of the tile's work (it writes
  // no X').  The flag is uniform over the workgroup.
  if constexpr (APPLY)
    if (md.fuse && g.clip != nullptr && g.clip->skip) return;
  uint16_t* ws = static_cast<uint16_t*>(g.ws);

  // operands, in the panel layout of the workspace (panel_off): P and, in
  // phases 1 and 2, Q are read along their rows, one 32-column panel per
  // stage, so P (Q) points at row ti*256 (tj*256) of panel 0 and a stage
  // advances by one panel, PS elements.  Phase 3's Q = X is read as [k][j]:
  // Q points at panel 8*tj (column tj*256), row 0, and a stage advances by
  // 32 rows.
  const uint16_t *P, *Q;
  int K;
  const int64_t PS = static_cast<int64_t>(md.m_pad) * kPanelCols;  // elements per panel
  // K runs over the true extent rounded to the K step only: the rest of
  // the padded operands is zero
  if (PHASE == 1) {
    K = md.n_k;
    P = ws + (g.x_cur ? md.ws_x[1] : md.ws_x[0]) + static_cast<int64_t>(ti) * BT * kPanelCols;
    Q = ws + (g.x_cur ? md.ws_x[1] : md.ws_x[0]) + static_cast<int64_t>(tj) * BT * kPanelCols;
  } else if (PHASE == 2) {
    K = md.m_k;
    P = ws + md.ws_a + static_cast<int64_t>(ti) * BT * kPanelCols;
    Q = ws + md.ws_a + static_cast<int64_t>(tj) * BT * kPanelCols;
  } else {
    K = md.m_k;
    P = ws + md.ws_b + static_cast<int64_t>(ti) * BT * kPanelCols;
    Q = ws + (g.x_cur ? md.ws_x[1] : md.ws_x[0]) + static_cast<int64_t>(tj) * (BT / kPanelCols) * PS;
  }

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wi = wave & 1, wj = wave >> 1;
  const int frow = lane & 31;
  // quadrant this wave computes and the shift of its 64 Q rows: wave (1,0)
  // of a diagonal tile takes quadrant (0,1) shifted by 64; on a half-height
  // tile wave (wi, wj) takes quadrant (0, wj) shifted by 64 wi, on a
  // half-width tile quadrant (wi, 0) shifted by 64 wj
  const bool adopt = ROLE == 2 && wi == 1;
  // A diagonal tile's P and Q panels are the same rows (ti == tj): in phase
  // 2 it loads them once and reads its Q fragments from the P copy, with
  // half the DMA.
  constexpr bool SHARED_PQ = PHASE == 2 && (ROLE == 1 || ROLE == 2);
  constexpr int DPS = SHARED_PQ ? DMA_PER_STAGE / 2 : DMA_PER_STAGE;  // DMA per wave per stage
  // Half edge tiles: waves 2 and 3 load the padding half of P (half-height,
  // phase 3) or of Q (half-width, phases 1 and 2), which no MFMA reads, so
  // they skip those DMA and wait on half the count.
  constexpr bool HALF_DMA = ROLE == 3 || (ROLE == 4 && PHASE != 3);
  const bool dma_half = HALF_DMA && wave >= 2;
  const int wie = ROLE == 3 ? 0 : ROLE == 4 ? wi : adopt ? 0 : wi;
  const int wje = ROLE == 3 ? wj : ROLE == 4 ? 0 : adopt ? 1 : wj;
  const int qshift = ROLE == 3 ? 64 * wi : ROLE == 4 ? 64 * wj : adopt ? 64 : 0;

  // MFMA operand fragments.  A fragment set (one 16-wide k substep) is
  // NR LDS reads: 4 P fragments (ds_read_b128) then the Q fragments, 4
  // ds_read_b128 (phases 1, 2) or 8 transpose reads (phase 3, lo/hi halves
  // of 8 consecutive k).  Read R of a set is issued by issue_read so that
  // the reads can be interleaved one by one with MFMAs.  Addresses: a
  // per-lane byte offset within a ring slot (below) + the wave-uniform slot
  // base + an immediate.
  constexpr int NR = PHASE == 3 ? 12 : 8;
  constexpr uint32_t SLOT_BYTES = 2 * BT * BK * 2;
  const uint32_t lds0 = lds_addr(smem);
  uint32_t vp[2], vq[2];  // K-contiguous fragments of k substep ks
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int sw = ((ks * 2 + (lane >> 5)) ^ ((frow >> 2) & 3)) << 3;
    vp[ks] = ((wie * 128 + frow) * BK + sw) * 2;
    vq[ks] = (SHARED_PQ ? 0 : BT * BK * 2) + ((wje * 128 + qshift + frow) * BK + sw) * 2;
  }
  // phase 3: transposed reads of column block b.  Lane group of 16: k row
  // 8*(lane/32) + (lane%16)/4 (+4 for the hi half, +16 per substep), columns
  // wj*128 + 32b + 16*((lane/16)%2) + 4*(lane%4), whose 32-column block is
  // swizzled by (k & 3) = (lane%16)/4.
  uint32_t vt[4];
  {
    const int s = lane & 15, yy = (s >> 2) & 3;
    const int x = 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const int bq = qshift >> 5;  // 32-column blocks of the Q shift
#pragma unroll
    for (int b = 0; b < 4; ++b)
      vt[b] = BT * BK * 2 +
              ((8 * (lane >> 5) + (s >> 2)) * BT + wje * 128 + x + ((((b + bq) & 3) ^ yy) << 5)) * 2;
  }
  struct Frags {
    bf16x8_t p[4];
    bf16x8_t q[4];
    s16x4_t t[8];  // phase 3: transposed halves of q
  };
  auto issue_read = [&](Frags& f, uint32_t sb, auto ks_c, auto r_c) {
    constexpr int KS = decltype(ks_c)::value, R = decltype(r_c)::value;
    if constexpr (R < 4) {
      f.p[R] = ld128_async<R * 32 * BK * 2>(vp[KS] + sb);
    } else if constexpr (PHASE != 3) {
      // split roles use Q fragments 0 and 1 only (the others would lie
      // past the shifted wave's Q rows)
      if constexpr (ROLE < 2 || R - 4 < 2)
        f.q[R - 4] = ld128_async<(R - 4) * 32 * BK * 2>(vq[KS] + sb);
    } else {
      constexpr int B = (R - 4) >> 1, H = (R - 4) & 1;
      if constexpr (ROLE < 2 || B < 2)
        f.t[R - 4] = ld_tr_async<KS * 16 * BT * 2 + H * 4 * BT * 2>(vt[B] + sb);
    }
  };
  // all reads of a set have landed (no other LDS reads outstanding)
  auto settle = [&](Frags& f) {
    if constexpr (PHASE == 3) {
      wait_frags_tr<0>(f.t, f.p);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        f.q[b] = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(f.t[2 * b], f.t[2 * b + 1], 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      wait_frags<0>(f.q, f.p);
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  // DMA of one stage, one instruction at a time: instruction D (0..7) of
  // this wave; D < 4: 16 P rows of 64 bytes, 1 KiB contiguous in the
  // panel (16-byte chunk c of row r at LDS position c ^ ((r >> 2) & 3)),
  // D >= 4: the same for Q (phases 1, 2) or 2 k-rows of 512 bytes of Q
  // (phase 3: 32-column block q of k-row r, the 64-byte row r of panel q,
  // at LDS position q ^ (r & 3); rows r and r + 1 of a panel make one
  // 128-byte line).  The per-lane source offsets are fixed for the tile.
  const char* Pc = reinterpret_cast<const char*>(P);
  const char* Qc = reinterpret_cast<const char*>(Q);
  const int pc = (lane & 3) ^ ((lane >> 4) & 3);
  const uint32_t dPQ = ((lane >> 2) * kPanelCols + 8 * pc) * 2;
  uint32_t dQ3[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int jl = 8 * ((lane & 31) ^ (((2 * par + (lane >> 5)) & 3) << 2));  // column in the tile
    dQ3[par] = static_cast<uint32_t>(((jl >> 5) * PS + (lane >> 5) * kPanelCols + (jl & 31)) * 2);
  }
  auto issue_dma = [&](int kt, int slot, auto d_c) {
    constexpr int D = decltype(d_c)::value, U = D & 3;
    if constexpr (D >= DPS) return;  // shared P and Q: no Q copy
    if constexpr (HALF_DMA && ((ROLE == 3) == (D < 4)))
      if (dma_half) return;  // padding rows of P (ROLE 3) or Q (ROLE 4)
    uint16_t* sp = smem + slot * 2 * BT * BK;
    uint16_t* sq = sp + BT * BK;
    if constexpr (D < 4) {
      const int R0 = (wave * 4 + U) * 16;
      dma16(Pc + (kt * PS + R0 * kPanelCols) * 2, dPQ, sp + R0 * BK);
    } else if constexpr (PHASE != 3) {
      const int R0 = (wave * 4 + U) * 16;
      dma16(Qc + (kt * PS + R0 * kPanelCols) * 2, dPQ, sq + R0 * BK);
    } else {
      const int R0 = (wave * 4 + U) * 2;
      dma16(Qc + (static_cast<int64_t>(kt) * BK + R0) * kPanelCols * 2, dQ3[U & 1],
            sq + R0 * BT);
    }
  };

  // Pipeline: a ring of NSLOT stages, NSLOT - 1 in flight.  Per stage two
  // groups of 16 MFMAs (k substeps 0 and 1).  Group A runs on substep 0
  // while the reads of substep 1 are issued between its MFMAs.  Then this
  // wave waits for its DMA of stage kt+1 and the workgroup barrier makes
  // every wave's DMA visible and guarantees slot kt-1 is no longer read.
  // Group B runs on substep 1 while the DMA of stage kt+NSLOT-1 (into slot
  // kt-1) and the reads of stage kt+1's substep 0 are issued between its
  // MFMAs.  Every memory instruction sits next to an MFMA, so the matrix
  // pipe does not wait for instruction issue.
  const int nk = K / BK;
#pragma unroll
  for (int s0 = 0; s0 < NSLOT - 1; ++s0)
    if (s0 < nk) static_for<0, DMA_PER_STAGE>([&](auto d) { issue_dma(s0, s0, d); });
  auto wait_landed = [&](int st, int newest) {
    if (HALF_DMA && dma_half) wait_stage_landed<DPS / 2>(st, newest);
    else wait_stage_landed<DPS>(st, newest);
  };
  wait_landed(0, min(NSLOT - 2, nk - 1));
  pipe_barrier();

  Frags F[2];
  static_for<0, NR>([&](auto r) { issue_read(F[0], lds0, Int<0>{}, r); });

  // one stage; REFILL: issue the DMA of stage kt+NSLOT-1, NEXT: read the
  // first fragments of stage kt+1 (both true except in the last stages)
  auto stage = [&](int kt, auto refill_c, auto next_c) {
    constexpr bool REFILL = decltype(refill_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    const uint32_t sb = lds0 + (kt % NSLOT) * SLOT_BYTES;
    settle(F[0]);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 16>([&](auto m_c) {
      constexpr int m = decltype(m_c)::value;
      if constexpr ((MASK >> m) & 1u)
        acc[m >> 2][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            F[0].q[m >> 2], F[0].p[m & 3], acc[m >> 2][m & 3], 0, 0, 0);
      if constexpr (m < NR) issue_read(F[1], sb, Int<1>{}, Int<m>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (NEXT) {
      // (the last stage has no next stage to wait for, and no slot is
      // refilled after it)
      wait_landed(kt + 1, min(kt + NSLOT - 2, nk - 1));
      pipe_barrier();
    }
    settle(F[1]);
    __builtin_amdgcn_sched_barrier(0);
    const int rslot = (kt + NSLOT - 1) % NSLOT;
    const uint32_t nsb = lds0 + ((kt + 1) % NSLOT) * SLOT_BYTES;
    static_for<0, 16>([&](auto m_c) {
      constexpr int m = decltype(m_c)::value;
      if constexpr ((MASK >> m) & 1u)
        acc[m >> 2][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            F[1].q[m >> 2], F[1].p[m & 3], acc[m >> 2][m & 3], 0, 0, 0);
      // after MFMA m: DMA m/2 on even m, read m/2 on odd m, and reads
      // 8..NR-1 after MFMAs 8..NR-1
      if constexpr (REFILL && (m & 1) == 0) issue_dma(kt + NSLOT - 1, rslot, Int<(m >> 1)>{});
      if constexpr (NEXT && (m & 1) == 1) issue_read(F[0], nsb, Int<0>{}, Int<(m >> 1)>{});
      if constexpr (NEXT && m >= 8 && m < NR) issue_read(F[0], nsb, Int<0>{}, Int<m>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int kt = 0;
  for (; kt + NSLOT - 1 < nk; ++kt) stage(kt, T_{}, T_{});
  for (; kt + 1 < nk; ++kt) stage(kt, F_{}, T_{});
  // Phase 2's epilogue adds b*A: this wave's 128x128 sub-tile of A is
  // loaded into registers while the last stage computes (16-byte row
  // loads: row lane/16 + 4u, 16-byte chunk lane%16).
  const int i0w = ti * BT + wie * 128, j0w = tj * BT + wje * 128 + qshift;
  constexpr bool aterm = PHASE == 2;
  // Fused update (phase 3 of the last iteration): W instead of X' for this
  // matrix.  A natural row of W is a row of the tile (wide matrix) or a
  // column of it (tall matrix).  A wide matrix's W sub-tile is loaded like
  // phase 2's A, while the last stage computes, and updated in the staging
  // layout; a tall one is updated after the staging, through the
  // transposed pass.
  bool to_w = false;
  ApplyConsts ak{0.0f, 0.0f};
  uint16_t* Wm = nullptr;
  if constexpr (APPLY) {
    if (md.fuse) {
      to_w = true;
      ak = apply_consts(md.rows, md.cols, g.lr, g.wd, g.scale_mode, g.rms_target);
      Wm = g.params + md.off;
    }
  }
  // (md.fuse == 2: W off the 8-element grid, O is staged as for X')
  const bool w_rows = APPLY && to_w && md.fuse == 1 && !md.trans;
  u32x4_t apre[32];
  if constexpr (aterm) {
    const int pl = opaque_lane(lane);
    const uint16_t* Ao = ws + md.ws_a + panel_off(i0w + (pl >> 4), j0w + 8 * (pl & 15), md.m_pad);
#pragma unroll
    for (int u = 0; u < 32; ++u)
      apre[u] = *reinterpret_cast<const u32x4_t*>(Ao + 4 * u * kPanelCols);
  }
  if constexpr (APPLY) {
    if (w_rows) {
      // row i0w + lane/16 + 4u, 8 columns from j0w + 8*(lane%16); a piece
      // past W's rows or cols is not loaded (cols is a multiple of 8)
      const int pl = opaque_lane(lane);
      const int wc = j0w + 8 * (pl & 15);
      const bool wcol = wc < md.cols && (ROLE < 2 || (pl & 15) < 8);
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int wr = i0w + (pl >> 4) + 4 * u;
        if (wr < md.rows && wcol)
          apre[u] = *reinterpret_cast<const u32x4_t*>(Wm + static_cast<int64_t>(wr) * md.cols + wc);
      }
    }
  }
  stage(kt, F_{}, F_{});
  __syncthreads();

  // ---- epilogue.  Accumulator layout of the 32x32 MFMA (A operand = Q
  // rows j, B operand = P rows i): lane holds column i = lane%32 and rows
  // j = 8*(v/4) + 4*(lane/32) + v%4, i.e. C[i][j..j+3] for each v/4.
  // Wave sub-tile: rows i0w..i0w+127, columns j0w..j0w+127; LDS region of
  // this wave: 32 KiB (the operand buffers are no longer needed).
  // The epilogue's lane-dependent addresses are derived from an opaque
  // copy of the lane id, so the compiler cannot hoist them out of the
  // persistent tile loop, where they would stay live across the main loop
  // (and spill).
  const int elane = opaque_lane(lane);
  uint16_t* S = smem + wave * (128 * 128);
  uint16_t* C;  // result, panel layout with m_pad rows
  bool mirror;
  if (PHASE == 3) {
    C = ws + (g.x_cur ? md.ws_x[0] : md.ws_x[1]);
    mirror = false;
  } else {
    C = ws + ((PHASE == 1 && g.c != 0.0f) ? md.ws_a : md.ws_b);
    mirror = true;  // off-diagonal tiles whole, diagonal tiles block by block
  }

  // Staging-layout addressing.  For the accumulator positions of this
  // lane, row il = bi*32 + frow has g(il) = g(frow), and the 8-byte slot
  // of (il, bj*32 + 8q + 4*hl) is (bj*8 + 2q) ^ g(frow) ^ hl, so one base
  // address per (bj, q) serves all four bi (+ bi * 8 KiB).  For the
  // 16-byte row accesses (row r = lane/16 + 4u, chunk c = lane % 16) the
  // chunk's two slots are (2c, 2c+1) ^ g(r) with g(r) = gr ^ (u & 7): one
  // 16-byte access at the even slot, halves swapped when u is odd.
  const int efrow = elane & 31;
  const int hl = elane >> 5;
  const int gacc = (((efrow & 3) << 3) | ((efrow >> 2) & 7)) ^ hl;
  const int gr = ((elane >> 4) & 3) << 3;
  const int rc = elane & 15;
  auto row_slot16 = [&](int u) {  // element offset of the 16-byte chunk
    const int r = (elane >> 4) + 4 * u;
    return r * 128 + (((2 * rc) ^ (gr | (u & 6))) << 2);
  };

  // Fused update: this lane's 32 pieces of 8 parameters.  A wide matrix's
  // piece u is W[i][j..j+7] with i = i0w + lane/16 + 4u, j = j0w + 8*(lane%16)
  // (the row stores' chunks); a tall matrix's is W[j][i..i+7] with
  // j = j0w + 32*(u%4) + 16*((lane/16)%2) + lane%16, i = i0w + 16*(u/4) +
  // 8*(lane/32) (the transposed pass's pieces).  cols is a multiple of 8, so
  // a piece is inside W or outside it whole.
  auto w_piece = [&](int u, int64_t& e) {
    // a split-role wave computed staged columns 0..63 only
    if (ROLE >= 2 && (md.trans ? (u & 3) >= 2 : rc >= 8)) return false;
    int wr, wc;
    if (!md.trans) {
      wr = i0w + (elane >> 4) + 4 * u;
      wc = j0w + 8 * rc;
    } else {
      wr = j0w + 32 * (u & 3) + 16 * ((elane >> 4) & 1) + (elane & 15);
      wc = i0w + 16 * (u >> 2) + 8 * (elane >> 5);
    }
    e = static_cast<int64_t>(wr) * md.cols + wc;
    return wr < md.rows && wc < md.cols;
  };
  if (aterm || w_rows) {
    // b*A term, or the fused update of a wide matrix: the prefetched A or
    // W sub-tile into the staging layout
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      u32x4_t v = apre[u];
      if (u & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
      *reinterpret_cast<u32x4_t*>(S + row_slot16(u)) = v;
    }
    __syncthreads();
  }

  // values -> LDS staging (8-byte slots)
  const float s2 = inv * inv;
  const float sc = PHASE == 1 ? g.e1_scale * s2 : PHASE == 2 ? g.e2_scale : inv;
  // diagonal term: only a wave sub-tile on the diagonal (ti == tj,
  // wi == wj) has one, in its blocks bi == bj, where element (il, jl + e)
  // is diagonal iff frow == 8q + 4*hl + e
  const float dval =
      (PHASE != 3 && ti == tj && wi == wj) ? (PHASE == 1 ? g.e1_diag : g.e2_diag) : 0.0f;
#pragma unroll
  for (int bj = 0; bj < 4; ++bj)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint16_t* Sjq = S + efrow * 128 + ((((bj * 8 + 2 * q) ^ gacc) & 31) << 2);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        // every rounding step as written (the small-matrix kernel computes
        // the same expressions and must give the same bits)
#pragma clang fp contract(off)
        u32x2_t* slotp = reinterpret_cast<u32x2_t*>(Sjq + bi * 32 * 128);
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = sc * acc[bj][bi][4 * q + e];
        if constexpr (aterm) {
          // fma(b, a, c A A), as in the small-matrix kernel
          const u32x2_t a0 = *slotp;
          v[0] = fmaf(g.b, lo_bf(a0[0]), v[0]);
          v[1] = fmaf(g.b, hi_bf(a0[0]), v[1]);
          v[2] = fmaf(g.b, lo_bf(a0[1]), v[2]);
          v[3] = fmaf(g.b, hi_bf(a0[1]), v[3]);
        }
        if (PHASE != 3 && bi == bj) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += efrow == 8 * q + 4 * hl + e ? dval : 0.0f;
        }
        if (APPLY && w_rows) {
          // O rounded to bf16 as X' would hold it, then W' = decay W - step O
          const u32x2_t w0 = *slotp;
          const uint32_t o0 = pack2(v[0], v[1]), o1 = pack2(v[2], v[3]);
          *slotp = u32x2_t{pack2(apply_one(ak, lo_bf(w0[0]), lo_bf(o0)),
                                 apply_one(ak, hi_bf(w0[0]), hi_bf(o0))),
                           pack2(apply_one(ak, lo_bf(w0[1]), lo_bf(o1)),
                                 apply_one(ak, hi_bf(w0[1]), hi_bf(o1)))};
        } else {
          *slotp = u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])};
        }
      }
    }
  __syncthreads();

  if constexpr (APPLY) {
    if (to_w) {
      if (md.fuse == 2) {
        u32x4_t wv[32];
        offgrid_load<ROLE>(md, g.params, i0w, j0w, elane, wv);
        offgrid_update<ROLE>(S, md, g.params, ak, i0w, j0w, elane, wv);
      } else if (!md.trans) {
        // the staged tile holds W': row stores into W
#pragma unroll 8
        for (int u = 0; u < 32; ++u) {
          int64_t e;
          if (!w_piece(u, e)) continue;
          u32x4_t v = *reinterpret_cast<const u32x4_t*>(S + row_slot16(u));
          if (u & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
          *reinterpret_cast<u32x4_t*>(Wm + e) = v;
        }
      } else {
        // All 32 loads are issued first (the accumulators are staged and
        // their registers free), so one memory latency covers them: a wait
        // for loads would also wait for every store issued before it.
        u32x4_t wv[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          int64_t e;
          if (w_piece(u, e)) wv[u] = *reinterpret_cast<const u32x4_t*>(Wm + e);
        }
        // W' = decay W - step O for the 32 pieces, O read back transposed
        const int s = elane & 15, G = elane >> 4;
        const uint32_t sbase = lds_addr(S);
        static_for<0, 4>([&](auto b_c) {
          constexpr int u0 = 8 * decltype(b_c)::value;
          s16x4_t tr[16];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            const int u = u0 + v;
            const int jb = (u & 3) * 32, ib = (u >> 2) * 16;
            const int ir = ib + 8 * (G >> 1) + (s >> 2);
            const int jc = jb + 16 * (G & 1) + 4 * (s & 3);
            tr[2 * v] = ld_tr_async<0>(sbase + 2 * stg(ir, jc));
            tr[2 * v + 1] = ld_tr_async<0>(sbase + 2 * stg(ir + 4, jc));
          }
          wait_lds16(tr);
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            int64_t e;
            if (!w_piece(u0 + v, e)) continue;
            const u32x4_t o = __builtin_bit_cast(
                u32x4_t,
                __builtin_shufflevector(tr[2 * v], tr[2 * v + 1], 0, 1, 2, 3, 4, 5, 6, 7));
            *reinterpret_cast<u32x4_t*>(Wm + e) = apply8(ak, wv[u0 + v], o);
          }
        });
      }
      return;
    }
  }

  // row stores: 16 bytes per lane, 4 rows of 256 bytes per instruction;
  // ROLE 1 stores its upper blocks (block row r/32 <= block column rc/4),
  // ROLES 2-4 staged columns 0..63 (j0w includes the Q shift)
#pragma unroll 8
  for (int u = 0; u < 32; ++u) {
    const int r = (elane >> 4) + 4 * u;
    if (ROLE == 1 && (r >> 5) > (rc >> 2)) continue;
    if (ROLE >= 2 && rc >= 8) continue;
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(S + row_slot16(u));
    if (u & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
    *reinterpret_cast<u32x4_t*>(C + panel_off(i0w + r, j0w + 8 * rc, md.m_pad)) = v;
  }

  // mirror piece u (rows 16*(u/4).., columns 32*(u%4).. of the staged
  // tile: source block (u/8, u%4)) is written iff this wave computed it
  // and, on a diagonal quadrant, it lies strictly above the diagonal
  auto mirror_keep = [](int u) {
    return ROLE == 0 || (ROLE == 1 ? (u >> 3) < (u & 3) : (u & 3) < 2);
  };
  if (mirror) {
    // C^T[j][i..i+7] = C[i..i+7][j] via two transpose reads per lane:
    // group G = lane/16 covers columns jb + 16*(G&1) + (lane%16) and rows
    // ib + 8*(G>>1) .. +7 of the staged tile.  Eight rows of output per
    // batch: 16 reads in flight, one wait, 8 stores.
    const int s = elane & 15, G = elane >> 4;
    const uint32_t sbase = lds_addr(S);
    for (int u0 = 0; u0 < 32; u0 += 8) {
      s16x4_t tr[16];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int u = u0 + v;
        if (!mirror_keep(u)) continue;
        const int jb = (u & 3) * 32, ib = (u >> 2) * 16;
        const int ir = ib + 8 * (G >> 1) + (s >> 2);
        const int jc = jb + 16 * (G & 1) + 4 * (s & 3);
        tr[2 * v] = ld_tr_async<0>(sbase + 2 * stg(ir, jc));
        tr[2 * v + 1] = ld_tr_async<0>(sbase + 2 * stg(ir + 4, jc));
      }
      wait_lds16(tr);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int u = u0 + v;
        if (!mirror_keep(u)) continue;
        const int jb = (u & 3) * 32, ib = (u >> 2) * 16;
        const int jo = jb + 16 * (G & 1) + s;
        const int io = ib + 8 * (G >> 1);
        *reinterpret_cast<s16x8_t*>(C + panel_off(j0w + jo, i0w + io, md.m_pad)) =
            __builtin_shufflevector(tr[2 * v], tr[2 * v + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  }
}

// Persistent launch: one workgroup per CU walks the tile list with stride
// gridDim.x.  The list is in XCD-grouped order for a grid that is a
// multiple of 8, so the 32 workgroups of an XCD still work on one group of
// neighbouring tiles at a time; a tile's epilogue stores drain while the
// next tile's first operand stages load.
//
// The tile list, the matrix table and the inverse norms come in as
// __restrict__ parameters: they are read-only for the whole launch, so
// their uniform loads become scalar loads, which do not wait for the
// previous tile's stores (vector loads would: vmcnt counts loads and
// stores together).
//
// With GemmArgs::sync set (phases 1 and 2, where the planner finds that a
// round's tiles cost much the same) the walk also holds each XCD's
// workgroups together: a workgroup that starts round r (its items are
// idx = b + r * gridDim.x), r a multiple of GemmArgs::sync_every, first
// waits until the other workgroups of its XCD group have finished round
// r - 1.  Without it they drift apart by whole tiles over the rounds and
// read the shared operand panels at different times, from HBM instead of
// L2.  The wait is a timing device only and is bounded:
// after kSyncSpins polls the workgroup goes on (a member of the group may
// not be resident while other kernels hold CUs).
constexpr int kSyncSpins = 1024;
__device__ __forceinline__ void xcd_round_barrier(uint32_t* cnt, uint32_t target) {
  __syncthreads();  // every wave is done with the previous round
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = 0; i < kSyncSpins; ++i) {
      if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

template <int PHASE>
__global__ __launch_bounds__(256, 1) void k_ns_bf16(GemmArgs g, const Item* __restrict__ items,
                                                    const MatDev* __restrict__ mats,
                                                    const float* __restrict__ invs) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[NSLOT * 2 * BT * BK];  // 128 KiB
  bool busy = false;
  // round holds (phases 1 and 2 only): a countdown of the rounds to the
  // next hold, and the holds passed so far
  uint32_t* const cnt = PHASE != 3 && g.sync != nullptr
                            ? g.sync + (blockIdx.x % kSyncGroups) * kSyncStride
                            : nullptr;
  int left = g.sync_every;
  uint32_t holds = 0;
  for (int idx = blockIdx.x; idx < g.n_items; idx += gridDim.x) {
    if constexpr (PHASE != 3) {
      if (cnt != nullptr && idx != static_cast<int>(blockIdx.x) && --left == 0) {
        left = g.sync_every;
        xcd_round_barrier(cnt, (gridDim.x / kSyncGroups) * ++holds);
      }
    }
    const Item it = items[idx];
    if (it.mat < 0) continue;  // padding of the XCD-grouped order
    const MatDev md = mats[it.mat];
    const float inv = g.first ? invs[md.widx] : 1.0f;
    if (busy) __syncthreads();  // the previous tile's epilogue is done with LDS
    busy = true;
    const int ti = it.rc >> 16, tj = it.rc & 0xffff;
    const int role = tile_role(PHASE, md, ti, tj, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    if (PHASE != 3 && role == 1) ns_tile<PHASE, 1>(g, md, ti, tj, inv, smem);
    else if (PHASE != 3 && role == 2) ns_tile<PHASE, 2>(g, md, ti, tj, inv, smem);
    else if (PHASE == 3 && role == 3) ns_tile<3, 3>(g, md, ti, tj, inv, smem);
    else if (role == 4) ns_tile<PHASE, 4>(g, md, ti, tj, inv, smem);
    else ns_tile<PHASE, 0>(g, md, ti, tj, inv, smem);
  }
}

// Phase 3 of the last iteration with the update applied in the epilogue
// (GemmArgs::params): the same tile walk as k_ns_bf16<3>.
__global__ __launch_bounds__(256, 1) void k_ns_bf16_apply(GemmArgs g, const Item* __restrict__ items,
                                                          const MatDev* __restrict__ mats,
                                                          const float* __restrict__ invs) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[NSLOT * 2 * BT * BK];  // 128 KiB
  bool busy = false;
  for (int idx = blockIdx.x; idx < g.n_items; idx += gridDim.x) {
    const Item it = items[idx];
    if (it.mat < 0) continue;  // padding of the XCD-grouped order
    const MatDev md = mats[it.mat];
    const float inv = g.first ? invs[md.widx] : 1.0f;
    if (busy) __syncthreads();  // the previous tile's epilogue is done with LDS
    busy = true;
    const int ti = it.rc >> 16, tj = it.rc & 0xffff;
    const int role = tile_role(3, md, ti, tj, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    if (role == 3) ns_tile<3, 3, true>(g, md, ti, tj, inv, smem);
    else if (role == 4) ns_tile<3, 4, true>(g, md, ti, tj, inv, smem);
    else ns_tile<3, 0, true>(g, md, ti, tj, inv, smem);
  }
}

__global__ void k_zero_u32(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_ns_phase(int ns_dtype, int phase, int n_items, int n_cu,
                           const GemmArgs& args, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 block(256);
  if (ns_dtype == 1) {
    const dim3 grid(n_items < n_cu ? n_items : n_cu);
    // round counters (phases 1, 2): on a grid of whole 32-workgroup XCD
    // groups with every workgroup walking the same number of rounds
    GemmArgs a = args;
    const bool sync = (phase == 1 || phase == 2) && a.sync != nullptr && a.sync_every > 0 &&
                      static_cast<int>(grid.x) == kSyncGroups * 32 && n_items > static_cast<int>(grid.x) &&
                      n_items % static_cast<int>(grid.x) == 0;
    if (sync) {
      hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(kSyncGroups * kSyncStride), 0, s, a.sync,
                         kSyncGroups * kSyncStride);
    } else {
      a.sync = nullptr;
    }
    if (phase == 3 && a.params != nullptr)
      hipLaunchKernelGGL(k_ns_bf16_apply, grid, block, 0, s, a, a.items, a.mats, a.inv);
    else if (phase == 1)
      hipLaunchKernelGGL(k_ns_bf16<1>, grid, block, 0, s, a, a.items, a.mats, a.inv);
    else if (phase == 2)
      hipLaunchKernelGGL(k_ns_bf16<2>, grid, block, 0, s, a, a.items, a.mats, a.inv);
    else
      hipLaunchKernelGGL(k_ns_bf16<3>, grid, block, 0, s, a, a.items, a.mats, a.inv);
  } else {
    return launch_ns_f32(phase, n_items, args, s);
  }
  return hipGetLastError();
}

}  // namespace muon
