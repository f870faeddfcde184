// Internal types shared by the host planner and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace muon {

// Edge of the elementwise tiles used by the momentum and apply kernels.
constexpr int kEwTile = 64;
// GEMM tile edges: bf16 MFMA engine and fp32 engine.
constexpr int kTileBf16 = 256;
constexpr int kTileFp32 = 64;
constexpr int kNsKStep = 32;  // bf16 engine: K per pipeline stage
// Small matrices (bf16 NS): m_k <= kSmallM and m_k * n_k <= kSmallElems run
// one NS iteration per launch in one workgroup, entirely in LDS.
constexpr int kSmallM = 128;
constexpr int kSmallElems = 32768;
// Tiled bf16 NS: the diagonal tiles of A = X X^T and A A split their upper
// blocks between the waves, and a matrix with at most this many tiles per
// side of A (m_pad / kTileBf16) also splits its half-empty edge tiles.
constexpr int kSplitEdgeMaxTiles = 8;

// Workspace area for the round counters of the persistent NS kernels: one
// 32-bit counter per XCD group, 256 bytes apart.
constexpr int kSyncGroups = 8;
constexpr int kSyncStride = 64;  // uint32 elements
constexpr size_t kSyncBytes = kSyncGroups * kSyncStride * 4;
// rounds between two holds: the plan takes the shortest of 4, 8, 16 and 32
// that costs little idle time (each hold costs a device-scope atomic and
// polling; a longer period lets more drift build up between holds)
constexpr int kSyncEveryMin = 4, kSyncEveryMax = 32;

// Layout of the bf16 NS workspace.  Every matrix there (the iterates X,
// A and B; all have m_pad rows) is stored as panels of 32 columns: panel q
// holds columns 32q..32q+31 of every row, row-major, so element (r, c) is at
// ((c / 32) * m_pad + r) * 32 + c % 32.  A pipeline stage of the NS GEMMs
// (256 rows x 32 k of an operand read along its rows) is then 16 KiB of
// contiguous memory and its loads read whole 128-byte lines.  The fp32
// workspace stays row-major ([m_pad][ld]).
constexpr int kPanelCols = 32;
__host__ __device__ __forceinline__ int64_t panel_off(int64_t r, int64_t c, int64_t rows) {
  return ((c >> 5) * rows + r) * kPanelCols + (c & 31);
}

// One matrix of a plan, as the device sees it.  "Oriented" dims put the
// short side first (m = min(rows, cols), n = max(rows, cols)); tall
// matrices (rows > cols) are iterated transposed.  The NS iterate X is
// kept oriented ([m_pad][n_pad], row-major, zero padded) in two ping-pong
// buffers.
struct MatDev {
  int64_t off;      // element offset in the flat params/grads/momentum
  int32_t rows, cols;
  int32_t m_pad, n_pad;  // oriented, padded to the GEMM tile
  int32_t m_k, n_k;      // m, n rounded up to the bf16 engine's K step: the
                         // contraction extents (the padding beyond is zero)
  int32_t trans;         // 1 if rows > cols
  int32_t widx;          // index of the matrix within its wave
  int32_t k1_begin;      // first elementwise tile of this matrix (wave-local)
  int32_t k1_count;      // number of elementwise tiles of this matrix
  int32_t small;         // 1: NS runs in the fused one-workgroup kernel
  int32_t split;         // 1: split tiles (diagonal tiles of the symmetric
                         // products, half-empty edge tiles) share their
                         // work out over the waves
  int32_t fuse;          // the last phase 3 can apply the update to W in
                         // its epilogue (tiled bf16 NS, bf16 params): 1 when
                         // offset and cols are multiples of 8, 2 otherwise
                         // (W rows realigned onto the 8-element grid)
  int32_t reserved;
  // element offsets (in NS elements) into the workspace
  int64_t ws_x[2];       // X : m_pad x n_pad, ping-pong
  int64_t ws_a;          // A : m_pad x m_pad
  int64_t ws_b;          // B : m_pad x m_pad
};

// A tile work item: matrix index (plan-global) and packed tile coords.
// Unsigned, so that a row tile of 32768 or more (a natural side of more
// than 2^21 elements in 64-element tiles) decodes with a logical shift.
struct Item {
  int32_t mat;
  uint32_t rc;  // (row_tile << 16) | col_tile, each < 2^16
};

// Device view of muon_clip_state_t (same layout): the gradient scale and
// the skip flag of a guarded step.  A null pointer means scale 1, no skip.
struct ClipState {
  float norm;
  float scale;
  int32_t skip;
  int32_t reserved;
};

struct GemmArgs {
  const MatDev* mats;
  const Item* items;
  void* ws;           // workspace base (NS element type)
  const float* inv;   // wave-local 1/(||U||_F + eps)
  float a, b, c;
  // bf16 engine epilogue constants (host-computed from a, b, c):
  //   phase 1 writes e1_scale * s2 * X X^T + e1_diag * I
  //   phase 2 writes e2_scale * A A + b * A + e2_diag * I
  float e1_scale, e1_diag, e2_scale, e2_diag;
  int32_t first;      // first NS iteration: fold the normalisation in
  int32_t x_cur;      // X buffer read by phases 1 and 3 (phase 3 writes 1 - x_cur)
  int32_t n_items;    // tile-list length (the persistent grid walks it)
  // Phase 3 of the last iteration with the update applied in the epilogue
  // (bf16 engine): for matrices with MatDev::fuse, W <- decay W - step O
  // with O the bf16 value X' would hold; X' is not written for them.
  // params == nullptr: plain phase 3.
  uint16_t* params;   // flat bf16 parameters
  const ClipState* clip;  // guarded step (skip: W untouched), or null
  float lr, wd, rms_target;
  int32_t scale_mode;
  // Round counters of the persistent bf16 kernels of phases 1 and 2, one
  // per XCD group, kSyncStride apart; zeroed on the stream before each
  // launch that uses them.
  uint32_t* sync;
  int32_t sync_every;  // rounds between holds (with sync)
};

// kernel launchers (defined in the .hip files)
hipError_t launch_momentum(const MatDev* mats, const Item* items, int n_items,
                           int grad_dtype, int ns_dtype, const void* grads, float* mom,
                           void* ws, double* partials, float mu, int nesterov,
                           const ClipState* clip, hipStream_t s);
// Also rescales X0 (in the workspace ws, NS dtype ns_dtype) by a power of
// two, folded into inv, for a matrix whose norm lies outside [2^-40, 2^40].
hipError_t launch_norm_finalize(const MatDev* mats, int mat_begin, int n_mats,
                                const double* partials, float* norms, float* inv,
                                float eps, int ns_dtype, void* ws, hipStream_t s);
hipError_t launch_apply(const MatDev* mats, const Item* items, int n_items, int param_dtype,
                        int ns_dtype, void* params, const void* ws, const float* inv,
                        float o_scale_by_inv, int x_final, float lr, float wd,
                        int scale_mode, float rms_target, float* out_update,
                        const ClipState* clip, hipStream_t s);
hipError_t launch_export(const MatDev* mats, const Item* items, int n_items, int ns_dtype,
                         const void* ws, int x_idx, float* out, hipStream_t s);
hipError_t launch_ns_phase(int ns_dtype, int phase, int n_items, int n_cu,
                           const GemmArgs& args, hipStream_t s);
// the fp32 engine's phases (one workgroup per tile item; ns_f32.hip)
hipError_t launch_ns_f32(int phase, int n_items, const GemmArgs& args, hipStream_t s);
// n_iter NS iterations (all phases) of each listed small matrix, starting
// at the iteration args describes
hipError_t launch_ns_small(int n_mats, const int32_t* list, int n_iter, const GemmArgs& args,
                           hipStream_t s);
// m_dtype: 0 fp32, 1 bf16; v_dtype: 0 fp32, 1 bf16, 2 fp16
hipError_t launch_adamw(void* params, int param_dtype, float* master, const void* grads,
                        int grad_dtype, void* m, int m_dtype, void* v, int v_dtype, int64_t n,
                        float lr, float beta1, float beta2, float eps, float wd, float lr_bc1,
                        float rsqrt_bc2, const ClipState* clip, hipStream_t s);
// Global gradient norm: one launch per buffer writes kReduceBlocks fp64
// partial sums of squares at partials + index * kReduceBlocks; the
// finalize launch reduces n_bufs * kReduceBlocks partials in order.
constexpr int kReduceBlocks = 1024;
hipError_t launch_sumsq(const void* g, int dtype, int64_t n, double* partials, hipStream_t s);
hipError_t launch_clip_finalize(const double* partials, int n_parts, float max_norm, float eps,
                                ClipState* out, hipStream_t s);
// State statistics: kReduceBlocks partials of kStatsPartialBytes each.
constexpr int kStatsPartialBytes = 64;
hipError_t launch_state_stats(const float* x, int64_t n, void* partials, void* out,
                              hipStream_t s);

// Error reporting shared by the host sources: record the message for
// muon_last_error() on the calling thread and return the status code.
int set_error(int code, const std::string& msg);
int set_hip_error(hipError_t e, const char* what);

// The update of one parameter, shared by the apply kernel and the fused
// phase-3 epilogue so that both give the same bits: with
// decay = 1 - lr*wd and step = lr * s (s the matrix's update scale),
// W' = decay*W - step*O, written with explicit fmas.
__device__ __forceinline__ float update_scale(int rows, int cols, int mode, float rms_target) {
  if (mode == 0) return rms_target * sqrtf(static_cast<float>(rows > cols ? rows : cols));
  if (mode == 1) return sqrtf(fmaxf(1.0f, static_cast<float>(rows) / static_cast<float>(cols)));
  return 1.0f;
}
struct ApplyConsts {
  float decay, step;
};
__device__ __forceinline__ ApplyConsts apply_consts(int rows, int cols, float lr, float wd,
                                                    int mode, float rms_target) {
  return ApplyConsts{fmaf(-lr, wd, 1.0f), lr * update_scale(rows, cols, mode, rms_target)};
}
__device__ __forceinline__ float apply_one(const ApplyConsts& k, float w, float o) {
  return fmaf(-k.step, o, k.decay * w);
}

// bf16 <-> fp32 (bf16 stored as its 16-bit pattern)
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// round-to-nearest-even, NaN stays NaN (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

}  // namespace muon
