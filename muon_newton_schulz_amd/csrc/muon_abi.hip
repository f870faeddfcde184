// Host side of the library: validation, planning (orientation, padding,
// workspace layout, tile lists, waves) and the C ABI declared in muon.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "muon.h"
#include "muon_internal.h"

using muon::Item;
using muon::MatDev;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return MUON_ERR_HIP;
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Wave {
  int mat_begin = 0, mat_end = 0;
  int64_t k1_begin = 0, k1_count = 0;      // into the k1 item table
  int64_t syrk_begin = 0, syrk_count = 0;  // phase 1's tiles (X X^T)
  int64_t aa_begin = 0, aa_count = 0;      // phase 2's: the same tiles (A A),
                                           // dealt out for phase 2's costs
  int64_t bx_begin = 0, bx_count = 0;
  int64_t small_begin = 0, small_count = 0;  // into the small-matrix table
  int64_t k7_begin = 0, k7_count = 0;  // elementwise tiles of the matrices whose
                                       // update is not fused into phase 3
  size_t partial_off = 0, norm_off = 0, inv_off = 0, sync_off = 0;  // byte offsets in the workspace
  // NS phases 1, 2: rounds between two holds of each XCD's workgroups (0: no hold)
  int32_t sync_every[2] = {0, 0};
  size_t bytes = 0;
};

}  // namespace

// The workspace of muon_step_noalloc: one file-scope device array, which the
// runtime places on every GPU that loads this library and keeps until the
// process ends.  In host code its name is a host-side stand-in, not a device
// address: kernels get the per-device address that hipGetSymbolAddress
// returns (static_ws_ptr).
static __device__ __align__(256) unsigned char scratch[MUON_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (which must be current),
// looked up once per device.
int static_ws_ptr(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MUON_ERR_UNSUPPORTED, "device index beyond the static workspace table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(static workspace)");
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % kAlign != 0)
      return fail(MUON_ERR_HIP, "static workspace address is null or not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MUON_OK;
}

}  // namespace

int muon::set_error(int code, const std::string& msg) { return fail(code, msg); }
int muon::set_hip_error(hipError_t e, const char* what) { return hip_fail(e, what); }

struct muon_plan {
  // set by muon_plan_upload: the device the tables live on, its compute
  // units (the persistent grid size)
  int device = -1;
  int n_cu = 0;
  bool uploaded = false;
  int32_t n_mats = 0;
  int64_t flat_numel = 0;
  int32_t param_dtype = 0, grad_dtype = 0, ns_dtype = 0;
  int tile = 0;
  size_t ws_bytes = 0;
  std::vector<MatDev> mats;
  std::vector<Item> k1_items, syrk_items, aa_items, bx_items, k7_items;
  std::vector<int32_t> small_list;  // matrices run by the fused small-matrix kernel
  std::vector<Wave> waves;
  // the tables packed as the device sees them (built at creation; copied
  // into the caller's buffer by muon_plan_upload) and their byte offsets
  std::vector<char> host_tables;
  size_t o_k1 = 0, o_syrk = 0, o_aa = 0, o_bx = 0, o_small = 0, o_k7 = 0;
  // device copies, inside the caller's table buffer
  MatDev* d_mats = nullptr;
  Item* d_k1 = nullptr;
  Item* d_syrk = nullptr;
  Item* d_aa = nullptr;
  Item* d_bx = nullptr;
  Item* d_k7 = nullptr;
  int32_t* d_small = nullptr;
  double flops_per_iter = 0.0;
};

namespace {

size_t ns_elem_bytes(int ns_dtype) { return ns_dtype == MUON_DTYPE_BF16 ? 2 : 4; }

bool dtype_ok(int32_t d) { return d == MUON_DTYPE_FP32 || d == MUON_DTYPE_BF16; }

// Per-matrix workspace elements (NS dtype): X ping-pong, A, B.
int64_t matrix_ws_elems(const MatDev& m) {
  const int64_t mn = static_cast<int64_t>(m.m_pad) * m.n_pad;
  const int64_t mm = static_cast<int64_t>(m.m_pad) * m.m_pad;
  return 2 * mn + 2 * mm;
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on
// XCD b % 8), and each XCD has its own L2.  Tiles that share operand
// panels should therefore run on the same XCD at the same time: the
// logical list is cut into groups of kGroup tiles (one group ~ the 32 CUs
// of an XCD), group s goes to XCD s % 8, and within an XCD the groups run
// in logical order, one per round of the persistent tile walk (workgroup
// b takes items b, b + 256, ...).  The list is padded with empty items
// (mat = -1) to a multiple of 8 * kGroup; those workgroups skip them.
//
// Tiles differ in cost (K, split diagonal and half edge tiles), and with a
// fixed lane per workgroup the differences would add up over the rounds:
// the workgroups of an XCD would drift apart by whole tiles, each would
// read its operand panels alone, and the panels would no longer be shared
// in L2.  So each group's tiles are dealt out longest first to the
// workgroups of its XCD that have the least estimated work so far (stable
// in both orders, so that tiles of equal cost keep the plain mapping).
constexpr int kXcds = 8;
constexpr int kGroup = 32;
constexpr int kSuperRows = 4, kSuperCols = 8;

template <typename Cost>
std::vector<Item> xcd_dispatch_order(const std::vector<Item>& logical, Cost cost) {
  const int64_t n = static_cast<int64_t>(logical.size());
  if (n == 0) return {};
  const int64_t round = static_cast<int64_t>(kXcds) * kGroup;
  const int64_t padded = (n + round - 1) / round * round;
  std::vector<Item> out(static_cast<size_t>(padded), Item{-1, 0});
  std::vector<double> work(static_cast<size_t>(kXcds) * kGroup, 0.0);
  int tile_of[kGroup], lane_of[kGroup];
  double c[kGroup];
  for (int64_t g = 0; g * kGroup < n; ++g) {
    const int64_t x = g % kXcds, rr = g / kXcds;
    const int nt = static_cast<int>(std::min<int64_t>(kGroup, n - g * kGroup));
    double* wx = work.data() + x * kGroup;
    for (int t = 0; t < nt; ++t) {
      tile_of[t] = t;
      c[t] = cost(logical[static_cast<size_t>(g * kGroup + t)]);
    }
    for (int l = 0; l < kGroup; ++l) lane_of[l] = l;
    std::stable_sort(tile_of, tile_of + nt, [&](int a, int b) { return c[a] > c[b]; });
    std::stable_sort(lane_of, lane_of + kGroup, [&](int a, int b) { return wx[a] < wx[b]; });
    for (int k = 0; k < nt; ++k) {
      const int t = tile_of[k], l = lane_of[k];
      out[static_cast<size_t>((rr * kGroup + l) * kXcds + x)] =
          logical[static_cast<size_t>(g * kGroup + t)];
      wx[l] += c[t];
    }
  }
  return out;
}

// Whether the round barrier pays for a dispatched list: the relative
// increase of the estimated makespan when every `every`-th round of an
// XCD starts only after the slowest of its workgroups has finished the
// previous one.
// The barrier keeps the workgroups that share operand panels in step (they
// then read them from L2); it is worth its idle time only where a round's
// tiles cost much the same.
template <typename Cost>
double barrier_idle(const std::vector<Item>& dispatched, Cost cost, int every) {
  const int64_t n = static_cast<int64_t>(dispatched.size());
  const int64_t round = static_cast<int64_t>(kXcds) * kGroup;
  if (n <= round) return 0.0;
  std::vector<double> free_run(static_cast<size_t>(round), 0.0), synced(free_run);
  for (int64_t r = 0; r * round < n; ++r) {
    for (int x = 0; x < kXcds && r % every == 0; ++x) {
      double mx = 0.0;
      for (int l = 0; l < kGroup; ++l) mx = std::max(mx, synced[static_cast<size_t>(l * kXcds + x)]);
      for (int l = 0; l < kGroup; ++l) synced[static_cast<size_t>(l * kXcds + x)] = mx;
    }
    for (int64_t b = 0; b < round && r * round + b < n; ++b) {
      const Item& it = dispatched[static_cast<size_t>(r * round + b)];
      if (it.mat < 0) continue;
      const double c = cost(it);
      free_run[static_cast<size_t>(b)] += c;
      synced[static_cast<size_t>(b)] += c;
    }
  }
  const double a = *std::max_element(free_run.begin(), free_run.end());
  const double s = *std::max_element(synced.begin(), synced.end());
  return a > 0.0 ? s / a - 1.0 : 0.0;
}
constexpr double kBarrierMaxIdle = 0.01;

// Estimated cost of a tile of NS phase `phase`, in K stages: the stages of
// its main loop, scaled for the split roles (a split diagonal tile's
// busiest wave does 10 of 16 MFMA blocks, a half edge tile 8), plus the
// prologue and epilogue (about 13, 17 and 8 stages in phases 1, 2 and 3).
// It only orders work: any value gives the same results.
double tile_cost(const MatDev& d, int phase, const Item& it, int T) {
  const int ti = static_cast<int>(it.rc >> 16), tj = static_cast<int>(it.rc & 0xffffu);
  const double stages = (phase == 1 ? d.n_k : d.m_k) / static_cast<double>(muon::kNsKStep);
  double f = 1.0;
  if (d.split) {
    const int m = std::min(d.rows, d.cols), n = std::max(d.rows, d.cols);
    if (phase != 3 && ti == tj) f = 0.625;
    else if (d.m_pad <= muon::kSplitEdgeMaxTiles * T &&
             ((phase == 3 && m - ti * T <= T / 2) || (phase == 3 ? n : m) - tj * T <= T / 2))
      f = 0.5;
  }
  return stages * f + (phase == 1 ? 13.0 : phase == 2 ? 17.0 : 8.0);
}

// Launch order of an elementwise tile list: workgroup b runs on XCD b % 8,
// and XCD x receives a contiguous run of the list, in order.  Neighbouring
// tiles of a row band share the cache lines at their boundary when a
// matrix's rows are off the line grid (ragged offsets and widths); in this
// order both tiles go through the same L2, close in time, instead of two.
std::vector<Item> xcd_contiguous_order(const std::vector<Item>& logical) {
  const int64_t n = static_cast<int64_t>(logical.size());
  std::vector<Item> out(logical.size());
  const int64_t q = n / kXcds, rem = n % kXcds;
  int64_t start[kXcds];
  for (int64_t x = 0, s = 0; x < kXcds; ++x) {
    start[x] = s;
    s += q + (x < rem ? 1 : 0);
  }
  for (int64_t b = 0; b < n; ++b) out[static_cast<size_t>(b)] = logical[static_cast<size_t>(start[b % kXcds] + b / kXcds)];
  return out;
}

// Tiles of one matrix (rows x cols tiles; upper triangle only if tri) in
// super-tile order: kSuperRows x kSuperCols blocks, row-major, so that
// consecutive tiles share their row and column operand panels.
void emit_super_tiles(int mat, int rows, int cols, bool tri, std::vector<Item>& out) {
  for (int R = 0; R < rows; R += kSuperRows)
    for (int C = tri ? (R / kSuperCols) * kSuperCols : 0; C < cols; C += kSuperCols)
      for (int a = R; a < std::min(rows, R + kSuperRows); ++a)
        for (int b = C; b < std::min(cols, C + kSuperCols); ++b)
          if (!tri || a <= b)
            out.push_back(Item{mat, (static_cast<uint32_t>(a) << 16) | static_cast<uint32_t>(b)});
}

// Build every host-side table; no HIP call.
int build_plan(const muon_matrix_t* mats, int32_t n_mats, int64_t flat_numel,
               int32_t param_dtype, int32_t grad_dtype, int32_t ns_dtype, size_t workspace_cap,
               uint32_t flags, muon_plan& p) {
  if ((flags & ~static_cast<uint32_t>(MUON_PLAN_TILED_ONLY | MUON_PLAN_WHOLE_TILES |
                                      MUON_PLAN_FREE_ROUNDS)) != 0)
    return fail(MUON_ERR_INVALID_ARG, "unknown plan flags");
  if (n_mats < 0) return fail(MUON_ERR_INVALID_ARG, "n_mats < 0");
  if (n_mats > 0 && mats == nullptr) return fail(MUON_ERR_INVALID_ARG, "mats is null");
  if (flat_numel < 0) return fail(MUON_ERR_INVALID_ARG, "flat_numel < 0");
  if (!dtype_ok(param_dtype) || !dtype_ok(grad_dtype) || !dtype_ok(ns_dtype))
    return fail(MUON_ERR_BAD_DTYPE, "dtype must be MUON_DTYPE_FP32 or MUON_DTYPE_BF16");
  p.n_mats = n_mats;
  p.flat_numel = flat_numel;
  p.param_dtype = param_dtype;
  p.grad_dtype = grad_dtype;
  p.ns_dtype = ns_dtype;
  p.tile = ns_dtype == MUON_DTYPE_BF16 ? muon::kTileBf16 : muon::kTileFp32;
  const int T = p.tile;

  // shape checks
  for (int32_t i = 0; i < n_mats; ++i) {
    const muon_matrix_t& m = mats[i];
    if (m.rows < 1 || m.cols < 1)
      return fail(MUON_ERR_BAD_SHAPE, "matrix " + std::to_string(i) + ": rows and cols must be >= 1");
    if (m.offset < 0)
      return fail(MUON_ERR_BAD_SHAPE, "matrix " + std::to_string(i) + ": negative offset");
    const int64_t numel = static_cast<int64_t>(m.rows) * m.cols;
    if (m.offset > flat_numel || numel > flat_numel - m.offset)
      return fail(MUON_ERR_BAD_SHAPE,
                  "matrix " + std::to_string(i) + ": extends past the flat buffer");
    // tile coordinates are packed in 16 bits
    if (round_up(std::max(m.rows, m.cols), T) / muon::kEwTile > 0xffff)
      return fail(MUON_ERR_BAD_SHAPE, "matrix " + std::to_string(i) + ": dimension too large");
  }
  // overlap check
  {
    std::vector<int32_t> order(n_mats);
    for (int32_t i = 0; i < n_mats; ++i) order[i] = i;
    std::sort(order.begin(), order.end(),
              [&](int32_t a, int32_t b) { return mats[a].offset < mats[b].offset; });
    for (int32_t k = 1; k < n_mats; ++k) {
      const muon_matrix_t& a = mats[order[k - 1]];
      const muon_matrix_t& b = mats[order[k]];
      if (a.offset + static_cast<int64_t>(a.rows) * a.cols > b.offset)
        return fail(MUON_ERR_OVERLAP, "matrices " + std::to_string(order[k - 1]) + " and " +
                                          std::to_string(order[k]) + " overlap");
    }
  }

  // orientation and padding
  p.mats.resize(n_mats);
  for (int32_t i = 0; i < n_mats; ++i) {
    MatDev& d = p.mats[i];
    std::memset(&d, 0, sizeof(d));
    d.off = mats[i].offset;
    d.rows = mats[i].rows;
    d.cols = mats[i].cols;
    d.trans = d.rows > d.cols ? 1 : 0;
    d.m_pad = static_cast<int32_t>(round_up(std::min(d.rows, d.cols), T));
    d.n_pad = static_cast<int32_t>(round_up(std::max(d.rows, d.cols), T));
    d.m_k = static_cast<int32_t>(round_up(std::min(d.rows, d.cols), muon::kNsKStep));
    d.n_k = static_cast<int32_t>(round_up(std::max(d.rows, d.cols), muon::kNsKStep));
    // small: m_k <= 128 and (m_k / 32) * ceil(n_k / 128) <= 8 (the fused
    // kernel's register tiling; implies m_k * n_k <= 32768)
    d.small = (ns_dtype == MUON_DTYPE_BF16 && !(flags & MUON_PLAN_TILED_ONLY) &&
               d.m_k <= muon::kSmallM && (d.m_k / 32) * ((d.n_k + 127) / 128) <= 8)
                  ? 1
                  : 0;
    d.split = (ns_dtype == MUON_DTYPE_BF16 && !d.small && !(flags & MUON_PLAN_WHOLE_TILES)) ? 1 : 0;
    // the fused update writes 16-byte pieces of 8 parameters along a
    // natural row: from the staged tile when the rows are on the flat
    // buffer's 8-element grid (1), realigned per row otherwise (2)
    const bool fusable =
        ns_dtype == MUON_DTYPE_BF16 && param_dtype == MUON_DTYPE_BF16 && !d.small;
    d.fuse = !fusable ? 0 : (d.off % 8 == 0 && d.cols % 8 == 0) ? 1 : 2;
    const double m = std::min(d.rows, d.cols), n = std::max(d.rows, d.cols);
    p.flops_per_iter += m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n;
  }

  // waves: consecutive matrices while the wave's workspace fits the cap
  const size_t eb = ns_elem_bytes(ns_dtype);
  auto k1_tiles_of = [&](const MatDev& d) {
    const int64_t rp = d.trans ? d.n_pad : d.m_pad, cp = d.trans ? d.m_pad : d.n_pad;
    return (rp / muon::kEwTile) * (cp / muon::kEwTile);
  };
  auto fixed_bytes = [&](int64_t k1, int64_t nm) {
    // fp64 partial sums (one per k1 tile), fp32 norms and inverse norms
    // (one per matrix), the NS kernels' round counters
    return align_up(static_cast<size_t>(k1) * 8, kAlign) +
           2 * align_up(static_cast<size_t>(nm) * 4, kAlign) + muon::kSyncBytes;
  };
  {
    int32_t i = 0;
    while (i < n_mats) {
      Wave w;
      w.mat_begin = i;
      size_t mat_bytes = 0;
      int64_t k1 = 0;
      int32_t j = i;
      while (j < n_mats) {
        const size_t mb = align_up(static_cast<size_t>(matrix_ws_elems(p.mats[j])) * eb, kAlign);
        const int64_t k1j = k1_tiles_of(p.mats[j]);
        const size_t total = mat_bytes + mb + fixed_bytes(k1 + k1j, j - i + 1);
        if (workspace_cap != 0 && total > workspace_cap) break;
        mat_bytes += mb;
        k1 += k1j;
        ++j;
      }
      if (j == i)
        return fail(MUON_ERR_WORKSPACE_TOO_SMALL,
                    "matrix " + std::to_string(i) + " alone needs more workspace than the cap");
      w.mat_end = j;
      p.waves.push_back(w);
      i = j;
    }
  }

  // per-wave layout and tile lists
  size_t ws_max = 0;
  for (Wave& w : p.waves) {
    const int nm = w.mat_end - w.mat_begin;
    int64_t k1 = 0;
    for (int m = w.mat_begin; m < w.mat_end; ++m) k1 += k1_tiles_of(p.mats[m]);
    size_t off = 0;
    w.partial_off = off;
    off += align_up(static_cast<size_t>(k1) * 8, kAlign);
    w.norm_off = off;
    off += align_up(static_cast<size_t>(nm) * 4, kAlign);
    w.inv_off = off;
    off += align_up(static_cast<size_t>(nm) * 4, kAlign);
    // matrices: offsets in NS elements from the workspace base
    w.k1_begin = static_cast<int64_t>(p.k1_items.size());
    for (int m = w.mat_begin; m < w.mat_end; ++m) {
      MatDev& d = p.mats[m];
      d.widx = m - w.mat_begin;
      const int64_t mn = static_cast<int64_t>(d.m_pad) * d.n_pad;
      const int64_t mm = static_cast<int64_t>(d.m_pad) * d.m_pad;
      const int64_t base = static_cast<int64_t>(off / eb);
      d.ws_x[0] = base;
      d.ws_x[1] = base + mn;
      d.ws_a = base + 2 * mn;
      d.ws_b = base + 2 * mn + mm;
      off += align_up(static_cast<size_t>(matrix_ws_elems(d)) * eb, kAlign);
      // elementwise tiles over the natural padded extent, row-major
      const int64_t rp = d.trans ? d.n_pad : d.m_pad, cp = d.trans ? d.m_pad : d.n_pad;
      d.k1_begin = static_cast<int32_t>(static_cast<int64_t>(p.k1_items.size()) - w.k1_begin);
      d.k1_count = static_cast<int32_t>((rp / muon::kEwTile) * (cp / muon::kEwTile));
      for (int64_t r = 0; r < rp / muon::kEwTile; ++r)
        for (int64_t c = 0; c < cp / muon::kEwTile; ++c)
          p.k1_items.push_back(
              Item{m, (static_cast<uint32_t>(r) << 16) | static_cast<uint32_t>(c)});
    }
    w.k1_count = static_cast<int64_t>(p.k1_items.size()) - w.k1_begin;
    w.k7_begin = static_cast<int64_t>(p.k7_items.size());
    std::vector<Item> k7_l;
    for (int64_t k = w.k1_begin; k < w.k1_begin + w.k1_count; ++k)
      if (!p.mats[p.k1_items[k].mat].fuse) k7_l.push_back(p.k1_items[k]);
    const std::vector<Item> k7 = xcd_contiguous_order(k7_l);
    p.k7_items.insert(p.k7_items.end(), k7.begin(), k7.end());
    w.k7_count = static_cast<int64_t>(p.k7_items.size()) - w.k7_begin;
    {
      const std::vector<Item> k1_l(p.k1_items.begin() + w.k1_begin, p.k1_items.end());
      const std::vector<Item> k1 = xcd_contiguous_order(k1_l);
      std::copy(k1.begin(), k1.end(), p.k1_items.begin() + w.k1_begin);
    }
    // the NS kernels' round counters, after the matrices (which keep the
    // same addresses with or without them)
    w.sync_off = off;
    off += muon::kSyncBytes;
    w.bytes = off;
    ws_max = std::max(ws_max, off);

    // GEMM tile lists: each matrix's tiles in super-tile order, then
    // permuted so that every XCD receives whole groups of neighbouring
    // tiles (see xcd_dispatch_order).  Phases 1 and 2 cover the upper
    // triangle of m x m with K = n and K = m; each takes the matrices by
    // its own K, then the other side, so that a round's tiles cost much
    // the same.  Matrices with more than kSplitEdgeMaxTiles tiles per side
    // run their split diagonal tiles after all off-diagonal tiles; smaller
    // ones keep them in place, next to the tiles that share their panels.
    // Phase 3 takes the matrices by m (its K).  Large tiles first, small
    // ones last, for the tail.
    std::vector<int> order;
    w.small_begin = static_cast<int64_t>(p.small_list.size());
    for (int m = w.mat_begin; m < w.mat_end; ++m) {
      if (p.mats[m].small) p.small_list.push_back(m);
      else order.push_back(m);
    }
    w.small_count = static_cast<int64_t>(p.small_list.size()) - w.small_begin;
    auto triangle_list = [&](bool by_n) {
      std::vector<int> o = order;
      std::stable_sort(o.begin(), o.end(), [&](int x, int y) {
        const MatDev &a = p.mats[x], &b = p.mats[y];
        const int ka = by_n ? a.n_k : a.m_k, kb = by_n ? b.n_k : b.m_k;
        if (ka != kb) return ka > kb;
        return by_n ? a.m_pad > b.m_pad : a.n_pad > b.n_pad;
      });
      std::vector<Item> l;
      for (int m : o) emit_super_tiles(m, p.mats[m].m_pad / T, p.mats[m].m_pad / T, true, l);
      std::stable_partition(l.begin(), l.end(), [&](const Item& it) {
        const MatDev& d = p.mats[it.mat];
        return !(d.split && d.m_pad / T > muon::kSplitEdgeMaxTiles &&
                 (it.rc >> 16) == (it.rc & 0xffffu));
      });
      return l;
    };
    const std::vector<Item> syrk_l = triangle_list(true), aa_l = triangle_list(false);
    std::vector<Item> bx_l;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
      return p.mats[x].m_pad > p.mats[y].m_pad;
    });
    for (int m : order) emit_super_tiles(m, p.mats[m].m_pad / T, p.mats[m].n_pad / T, false, bx_l);
    auto cost_of = [&](int phase) {
      return [&p, phase, T](const Item& it) { return tile_cost(p.mats[it.mat], phase, it, T); };
    };
    const std::vector<Item> syrk = xcd_dispatch_order(syrk_l, cost_of(1));
    const std::vector<Item> aa = xcd_dispatch_order(aa_l, cost_of(2));
    const std::vector<Item> bx = xcd_dispatch_order(bx_l, [](const Item&) { return 1.0; });
    // Phases 1 and 2 hold their rounds together where it costs little
    // idle time: every `every` rounds, the shortest period that does
    // (a list of at most `every` rounds has no hold).
    // Phase 3 never does: its workgroups stay within a few tens of K
    // stages of each other without it (a workgroup that runs ahead takes
    // the L2 misses), and the hold measured 0.5-2% slower there.
    if (ns_dtype == MUON_DTYPE_BF16 && !(flags & MUON_PLAN_FREE_ROUNDS)) {
      auto period = [&](const std::vector<Item>& l, int phase) {
        const int64_t rounds = static_cast<int64_t>(l.size()) / (int64_t{kXcds} * kGroup);
        for (int e = muon::kSyncEveryMin; e <= muon::kSyncEveryMax; e *= 2)
          if (rounds > e && barrier_idle(l, cost_of(phase), e) <= kBarrierMaxIdle) return e;
        return 0;
      };
      w.sync_every[0] = period(syrk, 1);
      w.sync_every[1] = period(aa, 2);
    }
    w.syrk_begin = static_cast<int64_t>(p.syrk_items.size());
    w.syrk_count = static_cast<int64_t>(syrk.size());
    p.syrk_items.insert(p.syrk_items.end(), syrk.begin(), syrk.end());
    w.aa_begin = static_cast<int64_t>(p.aa_items.size());
    w.aa_count = static_cast<int64_t>(aa.size());
    p.aa_items.insert(p.aa_items.end(), aa.begin(), aa.end());
    w.bx_begin = static_cast<int64_t>(p.bx_items.size());
    w.bx_count = static_cast<int64_t>(bx.size());
    p.bx_items.insert(p.bx_items.end(), bx.begin(), bx.end());
    if (w.k1_count > 0x7fffffff || w.syrk_count > 0x7fffffff || w.aa_count > 0x7fffffff ||
        w.bx_count > 0x7fffffff)
      return fail(MUON_ERR_BAD_SHAPE, "too many tiles in one wave");
  }
  p.ws_bytes = ws_max;
  return MUON_OK;
}

// Pack the tables into one host buffer laid out as the device copy will be
// (each table 256-byte aligned).  No HIP call.
void pack_tables(muon_plan& p) {
  const size_t b_mats = align_up(p.mats.size() * sizeof(MatDev), kAlign);
  const size_t b_k1 = align_up(p.k1_items.size() * sizeof(Item), kAlign);
  const size_t b_syrk = align_up(p.syrk_items.size() * sizeof(Item), kAlign);
  const size_t b_aa = align_up(p.aa_items.size() * sizeof(Item), kAlign);
  const size_t b_bx = align_up(p.bx_items.size() * sizeof(Item), kAlign);
  const size_t b_small = align_up(p.small_list.size() * sizeof(int32_t), kAlign);
  const size_t b_k7 = align_up(p.k7_items.size() * sizeof(Item), kAlign);
  p.o_k1 = b_mats;
  p.o_syrk = p.o_k1 + b_k1;
  p.o_aa = p.o_syrk + b_syrk;
  p.o_bx = p.o_aa + b_aa;
  p.o_small = p.o_bx + b_bx;
  p.o_k7 = p.o_small + b_small;
  p.host_tables.assign(p.o_k7 + b_k7, 0);
  char* h = p.host_tables.data();
  auto put = [&](size_t off, const void* src, size_t n) {
    if (n) std::memcpy(h + off, src, n);
  };
  put(0, p.mats.data(), p.mats.size() * sizeof(MatDev));
  put(p.o_k1, p.k1_items.data(), p.k1_items.size() * sizeof(Item));
  put(p.o_syrk, p.syrk_items.data(), p.syrk_items.size() * sizeof(Item));
  put(p.o_aa, p.aa_items.data(), p.aa_items.size() * sizeof(Item));
  put(p.o_bx, p.bx_items.data(), p.bx_items.size() * sizeof(Item));
  put(p.o_small, p.small_list.data(), p.small_list.size() * sizeof(int32_t));
  put(p.o_k7, p.k7_items.data(), p.k7_items.size() * sizeof(Item));
}

int check_step_common(const muon_plan_t* plan, int32_t wave, const void* workspace,
                      size_t workspace_bytes) {
  if (plan == nullptr) return fail(MUON_ERR_INVALID_ARG, "plan is null");
  if (!plan->uploaded)
    return fail(MUON_ERR_INVALID_ARG, "plan tables are not on a device (muon_plan_upload)");
  if (wave < 0 || wave >= static_cast<int32_t>(plan->waves.size()))
    return fail(MUON_ERR_INVALID_ARG, "wave index out of range");
  if (workspace == nullptr) return fail(MUON_ERR_INVALID_ARG, "workspace is null");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(MUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan->ws_bytes)
    return fail(MUON_ERR_WORKSPACE_TOO_SMALL,
                "workspace has " + std::to_string(workspace_bytes) + " bytes, plan needs " +
                    std::to_string(plan->ws_bytes));
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(MUON_ERR_INVALID_ARG, "current device differs from the plan's device");
  return MUON_OK;
}

int check_hparams(const muon_hparams_t* hp) {
  if (hp == nullptr) return fail(MUON_ERR_INVALID_ARG, "hparams is null");
  const float vals[] = {hp->lr, hp->weight_decay, hp->momentum, hp->ns_a, hp->ns_b,
                        hp->ns_c, hp->eps, hp->rms_target};
  for (float v : vals)
    if (!std::isfinite(v)) return fail(MUON_ERR_INVALID_ARG, "non-finite hyperparameter");
  if (hp->ns_steps < 0 || hp->ns_steps > 1000)
    return fail(MUON_ERR_INVALID_ARG, "ns_steps must be in [0, 1000]");
  if (hp->scale_mode < 0 || hp->scale_mode > 2)
    return fail(MUON_ERR_INVALID_ARG, "scale_mode must be 0, 1 or 2");
  if (hp->eps < 0.0f) return fail(MUON_ERR_INVALID_ARG, "eps must be >= 0");
  return MUON_OK;
}

inline char* ws_bytes_ptr(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

static_assert(sizeof(muon_clip_state_t) == sizeof(muon::ClipState) &&
                  offsetof(muon_clip_state_t, scale) == offsetof(muon::ClipState, scale) &&
                  offsetof(muon_clip_state_t, skip) == offsetof(muon::ClipState, skip),
              "muon_clip_state_t and its device view must agree");
inline const muon::ClipState* clip_of(const muon_clip_state_t* c) {
  return reinterpret_cast<const muon::ClipState*>(c);
}

muon::GemmArgs gemm_args(const muon_plan_t* p, const Wave& w, void* ws, const muon_hparams_t* hp,
                         int iter, const Item* items) {
  muon::GemmArgs g;
  g.mats = p->d_mats;
  g.items = items;
  g.ws = ws;
  g.inv = reinterpret_cast<const float*>(ws_bytes_ptr(ws, w.inv_off));
  g.sync = nullptr;  // set per phase by run_ns_phase
  g.sync_every = 0;
  g.a = hp->ns_a;
  g.b = hp->ns_b;
  g.c = hp->ns_c;
  // The bf16 engine's form of B = a I + b A + c A^2 (A = X X^T): with
  // c == 0 phase 1 writes B = b A + a I directly (phase 2 is skipped);
  // otherwise phase 1 writes A and phase 2 adds b A + a I to c A A.  (A
  // shifted Gram matrix sqrt(c) A + beta I, whose square plus a multiple
  // of I is B, would spare phase 2 its read of A, but its diagonal is
  // dominated by beta and bf16 rounding then erases the Gram diagonal.)
  const bool direct = hp->ns_c == 0.0f;
  g.e1_scale = direct ? hp->ns_b : 1.0f;
  g.e1_diag = direct ? hp->ns_a : 0.0f;
  g.e2_scale = hp->ns_c;
  g.e2_diag = hp->ns_a;
  g.first = iter == 0;
  g.x_cur = iter & 1;
  g.params = nullptr;
  g.clip = nullptr;
  g.lr = hp->lr;
  g.wd = hp->weight_decay;
  g.rms_target = hp->rms_target;
  g.scale_mode = hp->scale_mode;
  return g;
}

}  // namespace

extern "C" {

const char* muon_status_string(int32_t status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_ERR_INVALID_ARG: return "invalid argument";
    case MUON_ERR_BAD_SHAPE: return "bad shape";
    case MUON_ERR_OVERLAP: return "matrices overlap";
    case MUON_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MUON_ERR_BAD_DTYPE: return "bad dtype";
    case MUON_ERR_HIP: return "HIP runtime error";
    case MUON_ERR_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
  }
}

const char* muon_last_error(void) { return g_last_error.c_str(); }

int muon_workspace_size(const muon_matrix_t* mats, int32_t n_mats, int64_t flat_numel,
                        int32_t param_dtype, int32_t grad_dtype, int32_t ns_dtype,
                        size_t workspace_cap, size_t* workspace_bytes) {
  if (workspace_bytes == nullptr) return fail(MUON_ERR_INVALID_ARG, "workspace_bytes is null");
  muon_plan p;
  const int rc = build_plan(mats, n_mats, flat_numel, param_dtype, grad_dtype, ns_dtype,
                            workspace_cap, 0u, p);
  if (rc != MUON_OK) return rc;
  *workspace_bytes = p.ws_bytes;
  return MUON_OK;
}

int muon_plan_create_ex(const muon_matrix_t* mats, int32_t n_mats, int64_t flat_numel,
                        int32_t param_dtype, int32_t grad_dtype, int32_t ns_dtype,
                        size_t workspace_cap, uint32_t flags, muon_plan_t** out,
                        size_t* workspace_bytes) {
  if (out == nullptr) return fail(MUON_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  muon_plan* p = new (std::nothrow) muon_plan();
  if (p == nullptr) return fail(MUON_ERR_INVALID_ARG, "out of host memory");
  const int rc = build_plan(mats, n_mats, flat_numel, param_dtype, grad_dtype, ns_dtype,
                            workspace_cap, flags, *p);
  if (rc != MUON_OK) {
    muon_plan_destroy(p);
    return rc;
  }
  pack_tables(*p);
  if (workspace_bytes) *workspace_bytes = p->ws_bytes;
  *out = p;
  return MUON_OK;
}

int muon_plan_create(const muon_matrix_t* mats, int32_t n_mats, int64_t flat_numel,
                     int32_t param_dtype, int32_t grad_dtype, int32_t ns_dtype,
                     size_t workspace_cap, muon_plan_t** out, size_t* workspace_bytes) {
  return muon_plan_create_ex(mats, n_mats, flat_numel, param_dtype, grad_dtype, ns_dtype,
                             workspace_cap, 0u, out, workspace_bytes);
}

void muon_plan_destroy(muon_plan_t* plan) { delete plan; }

size_t muon_plan_table_bytes(const muon_plan_t* plan) {
  return plan == nullptr ? 0 : plan->host_tables.size();
}

int muon_plan_upload(muon_plan_t* plan, void* tables, size_t table_bytes, hipStream_t stream) {
  if (plan == nullptr) return fail(MUON_ERR_INVALID_ARG, "plan is null");
  const size_t need = plan->host_tables.size();
  if (need > 0) {
    if (tables == nullptr) return fail(MUON_ERR_INVALID_ARG, "tables is null");
    if (reinterpret_cast<uintptr_t>(tables) % kAlign != 0)
      return fail(MUON_ERR_INVALID_ARG, "tables must be 256-byte aligned");
    if (table_bytes < need)
      return fail(MUON_ERR_INVALID_ARG, "tables has " + std::to_string(table_bytes) +
                                            " bytes, the plan needs " + std::to_string(need));
  }
  int dev = -1, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
  if (need > 0) {
    e = hipMemcpyAsync(tables, plan->host_tables.data(), need, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan tables)");
  }
  char* base = static_cast<char*>(tables);
  plan->d_mats = reinterpret_cast<MatDev*>(base);
  plan->d_k1 = reinterpret_cast<Item*>(base + plan->o_k1);
  plan->d_syrk = reinterpret_cast<Item*>(base + plan->o_syrk);
  plan->d_aa = reinterpret_cast<Item*>(base + plan->o_aa);
  plan->d_bx = reinterpret_cast<Item*>(base + plan->o_bx);
  plan->d_small = reinterpret_cast<int32_t*>(base + plan->o_small);
  plan->d_k7 = reinterpret_cast<Item*>(base + plan->o_k7);
  plan->device = dev;
  // the XCD-grouped tile order assumes a grid that is a multiple of the XCD count
  plan->n_cu = n_cu >= 8 ? n_cu / 8 * 8 : (n_cu > 0 ? n_cu : 1);
  plan->uploaded = true;
  // set-up of muon_step_noalloc on this device: its static workspace's address
  void* ws = nullptr;
  return static_ws_ptr(dev, &ws);
}

int muon_plan_get_info(const muon_plan_t* plan, muon_plan_info_t* info) {
  if (plan == nullptr || info == nullptr) return fail(MUON_ERR_INVALID_ARG, "null argument");
  info->n_mats = plan->n_mats;
  info->n_waves = static_cast<int32_t>(plan->waves.size());
  info->tile = plan->tile;
  info->ns_dtype = plan->ns_dtype;
  info->k1_tiles = static_cast<int64_t>(plan->k1_items.size());
  info->syrk_tiles = static_cast<int64_t>(plan->syrk_items.size());
  info->bx_tiles = static_cast<int64_t>(plan->bx_items.size());
  info->workspace_bytes = plan->ws_bytes;
  info->ns_flops_per_iter_alg = plan->flops_per_iter;
  info->small_mats = static_cast<int32_t>(plan->small_list.size());
  info->split_tile_mats = 0;
  info->fused_apply_mats = 0;
  for (const muon::MatDev& d : plan->mats) {
    info->split_tile_mats += d.split;
    info->fused_apply_mats += d.fuse != 0;
  }
  info->round_sync_phases = 0;
  for (const Wave& w : plan->waves)
    for (int ph = 0; ph < 2; ++ph) info->round_sync_phases |= w.sync_every[ph] > 0 ? 1 << ph : 0;
  return MUON_OK;
}

int muon_stage_momentum(const muon_plan_t* plan, int32_t wave, const void* grads,
                        float* momentum, void* workspace, size_t workspace_bytes,
                        const muon_hparams_t* hp, hipStream_t stream) {
  int rc = check_step_common(plan, wave, workspace, workspace_bytes);
  if (rc != MUON_OK) return rc;
  if ((rc = check_hparams(hp)) != MUON_OK) return rc;
  if (grads == nullptr || momentum == nullptr)
    return fail(MUON_ERR_INVALID_ARG, "grads or momentum is null");
  const Wave& w = plan->waves[wave];
  double* partials = reinterpret_cast<double*>(ws_bytes_ptr(workspace, w.partial_off));
  hipError_t e = muon::launch_momentum(plan->d_mats, plan->d_k1 + w.k1_begin,
                                       static_cast<int>(w.k1_count), plan->grad_dtype,
                                       plan->ns_dtype, grads, momentum, workspace, partials,
                                       hp->momentum, hp->nesterov, clip_of(hp->clip), stream);
  if (e != hipSuccess) return hip_fail(e, "momentum kernel launch");
  e = muon::launch_norm_finalize(plan->d_mats, w.mat_begin, w.mat_end - w.mat_begin, partials,
                                 reinterpret_cast<float*>(ws_bytes_ptr(workspace, w.norm_off)),
                                 reinterpret_cast<float*>(ws_bytes_ptr(workspace, w.inv_off)),
                                 hp->eps, plan->ns_dtype, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "norm kernel launch");
  return MUON_OK;
}

namespace {

// Phase `phase` of NS iteration `iter` for the wave's tiled matrices; with
// small_iters > 0 (phase 3 only) also small_iters whole iterations of its
// small matrices, starting at `iter`.  fused_params (phase 3 of the last
// iteration, bf16 engine): apply the update of the matrices with
// MatDev::fuse in the epilogue.
int run_ns_phase(const muon_plan_t* plan, int32_t wave, void* workspace,
                 const muon_hparams_t* hp, int32_t iter, int32_t phase, int32_t small_iters,
                 hipStream_t stream, void* fused_params = nullptr) {
  const Wave& w = plan->waves[wave];
  const Item* items = phase == 3   ? plan->d_bx + w.bx_begin
                      : phase == 2 ? plan->d_aa + w.aa_begin
                                   : plan->d_syrk + w.syrk_begin;
  const int n = static_cast<int>(phase == 3 ? w.bx_count : phase == 2 ? w.aa_count : w.syrk_count);
  muon::GemmArgs g = gemm_args(plan, w, workspace, hp, iter, items);
  g.n_items = n;
  if (phase != 3 && w.sync_every[phase - 1] > 0) {
    g.sync = reinterpret_cast<uint32_t*>(ws_bytes_ptr(workspace, w.sync_off));
    g.sync_every = w.sync_every[phase - 1];
  }
  if (fused_params != nullptr) {
    g.params = static_cast<uint16_t*>(fused_params);
    g.clip = clip_of(hp->clip);
  }
  hipError_t e = muon::launch_ns_phase(plan->ns_dtype, phase, n, plan->n_cu, g, stream);
  if (e != hipSuccess) return hip_fail(e, "NS kernel launch");
  if (small_iters > 0 && w.small_count > 0) {
    e = muon::launch_ns_small(static_cast<int>(w.small_count), plan->d_small + w.small_begin,
                              small_iters, g, stream);
    if (e != hipSuccess) return hip_fail(e, "small-matrix NS kernel launch");
  }
  return MUON_OK;
}

}  // namespace

int muon_stage_ns_phase(const muon_plan_t* plan, int32_t wave, void* workspace,
                        size_t workspace_bytes, const muon_hparams_t* hp, int32_t iter,
                        int32_t phase, hipStream_t stream) {
  int rc = check_step_common(plan, wave, workspace, workspace_bytes);
  if (rc != MUON_OK) return rc;
  if ((rc = check_hparams(hp)) != MUON_OK) return rc;
  if (iter < 0 || iter >= hp->ns_steps) return fail(MUON_ERR_INVALID_ARG, "iter out of range");
  if (phase < 1 || phase > 3) return fail(MUON_ERR_INVALID_ARG, "phase must be 1, 2 or 3");
  if (phase == 2 && hp->ns_c == 0.0f)
    return fail(MUON_ERR_INVALID_ARG, "phase 2 is skipped when ns_c == 0");
  // the small matrices run their whole iteration with phase 3
  return run_ns_phase(plan, wave, workspace, hp, iter, phase, phase == 3 ? 1 : 0, stream);
}

namespace {

// The apply kernel over `count` elementwise tiles of the wave.
int run_apply(const muon_plan_t* plan, const Wave& w, const Item* items, int64_t count,
              void* params, void* workspace, const muon_hparams_t* hp, float* out_update,
              hipStream_t stream) {
  const hipError_t e = muon::launch_apply(
      plan->d_mats, items, static_cast<int>(count), plan->param_dtype, plan->ns_dtype, params,
      workspace, reinterpret_cast<const float*>(ws_bytes_ptr(workspace, w.inv_off)),
      hp->ns_steps == 0 ? 1.0f : 0.0f, hp->ns_steps & 1, hp->lr, hp->weight_decay,
      hp->scale_mode, hp->rms_target, out_update, clip_of(hp->clip), stream);
  if (e != hipSuccess) return hip_fail(e, "apply kernel launch");
  return MUON_OK;
}

// Phase 3 of the last iteration and the update: fused into phase 3's
// epilogue for the matrices that allow it (bf16 engine and parameters, a
// 16-byte aligned parameter buffer), the apply kernel for the others.
int run_ns_apply(const muon_plan_t* plan, int32_t wave, void* params, void* workspace,
                 const muon_hparams_t* hp, int32_t small_iters, hipStream_t stream) {
  const Wave& w = plan->waves[wave];
  const int32_t last = hp->ns_steps - 1;
  const bool fused = plan->ns_dtype == MUON_DTYPE_BF16 &&
                     plan->param_dtype == MUON_DTYPE_BF16 &&
                     reinterpret_cast<uintptr_t>(params) % 16 == 0;
  int rc = run_ns_phase(plan, wave, workspace, hp, last, 3, small_iters, stream,
                        fused ? params : nullptr);
  if (rc != MUON_OK) return rc;
  if (!fused)
    return run_apply(plan, w, plan->d_k1 + w.k1_begin, w.k1_count, params, workspace, hp,
                     nullptr, stream);
  if (w.k7_count == 0) return MUON_OK;
  return run_apply(plan, w, plan->d_k7 + w.k7_begin, w.k7_count, params, workspace, hp,
                   nullptr, stream);
}

}  // namespace

int muon_stage_apply(const muon_plan_t* plan, int32_t wave, void* params, void* workspace,
                     size_t workspace_bytes, const muon_hparams_t* hp, float* out_update,
                     hipStream_t stream) {
  int rc = check_step_common(plan, wave, workspace, workspace_bytes);
  if (rc != MUON_OK) return rc;
  if ((rc = check_hparams(hp)) != MUON_OK) return rc;
  if (params == nullptr) return fail(MUON_ERR_INVALID_ARG, "params is null");
  const Wave& w = plan->waves[wave];
  return run_apply(plan, w, plan->d_k1 + w.k1_begin, w.k1_count, params, workspace, hp,
                   out_update, stream);
}

int muon_stage_ns_apply(const muon_plan_t* plan, int32_t wave, void* params, void* workspace,
                        size_t workspace_bytes, const muon_hparams_t* hp, hipStream_t stream) {
  int rc = check_step_common(plan, wave, workspace, workspace_bytes);
  if (rc != MUON_OK) return rc;
  if ((rc = check_hparams(hp)) != MUON_OK) return rc;
  if (params == nullptr) return fail(MUON_ERR_INVALID_ARG, "params is null");
  if (hp->ns_steps < 1) return fail(MUON_ERR_INVALID_ARG, "ns_steps must be >= 1");
  // like muon_stage_ns_phase, the small matrices run one iteration
  return run_ns_apply(plan, wave, params, workspace, hp, 1, stream);
}

int muon_stage_export_x(const muon_plan_t* plan, int32_t wave, const void* workspace,
                        size_t workspace_bytes, int32_t iter_done, float* out,
                        hipStream_t stream) {
  int rc = check_step_common(plan, wave, workspace, workspace_bytes);
  if (rc != MUON_OK) return rc;
  if (out == nullptr) return fail(MUON_ERR_INVALID_ARG, "out is null");
  if (iter_done < 0) return fail(MUON_ERR_INVALID_ARG, "iter_done < 0");
  const Wave& w = plan->waves[wave];
  const hipError_t e =
      muon::launch_export(plan->d_mats, plan->d_k1 + w.k1_begin, static_cast<int>(w.k1_count),
                          plan->ns_dtype, workspace, iter_done & 1, out, stream);
  if (e != hipSuccess) return hip_fail(e, "export kernel launch");
  return MUON_OK;
}

int muon_stage_export_norms(const muon_plan_t* plan, int32_t wave, const void* workspace,
                            size_t workspace_bytes, float* out, hipStream_t stream) {
  int rc = check_step_common(plan, wave, workspace, workspace_bytes);
  if (rc != MUON_OK) return rc;
  if (out == nullptr) return fail(MUON_ERR_INVALID_ARG, "out is null");
  const Wave& w = plan->waves[wave];
  const hipError_t e = hipMemcpyAsync(
      out, static_cast<const char*>(workspace) + w.norm_off,
      static_cast<size_t>(w.mat_end - w.mat_begin) * sizeof(float), hipMemcpyDeviceToDevice,
      stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(norms)");
  return MUON_OK;
}

int muon_step(const muon_plan_t* plan, void* params, const void* grads, float* momentum,
              void* workspace, size_t workspace_bytes, const muon_hparams_t* hp,
              float* out_update, hipStream_t stream) {
  if (plan == nullptr) return fail(MUON_ERR_INVALID_ARG, "plan is null");
  int rc = check_hparams(hp);
  if (rc != MUON_OK) return rc;
  if (plan->waves.empty()) return MUON_OK;
  if (params == nullptr || grads == nullptr || momentum == nullptr)
    return fail(MUON_ERR_INVALID_ARG, "params, grads or momentum is null");
  for (int32_t w = 0; w < static_cast<int32_t>(plan->waves.size()); ++w) {
    rc = muon_stage_momentum(plan, w, grads, momentum, workspace, workspace_bytes, hp, stream);
    if (rc != MUON_OK) return rc;
    // tiled matrices phase by phase; the small matrices run all their
    // iterations in one launch (bitwise the same as one per iteration).
    // Without out_update, the last phase 3 applies the update itself.
    const bool fuse = out_update == nullptr && hp->ns_steps >= 1;
    for (int32_t it = 0; it < hp->ns_steps; ++it) {
      const int32_t small_iters = it == 0 ? hp->ns_steps : 0;
      rc = run_ns_phase(plan, w, workspace, hp, it, 1, 0, stream);
      if (rc == MUON_OK && hp->ns_c != 0.0f)
        rc = run_ns_phase(plan, w, workspace, hp, it, 2, 0, stream);
      if (rc == MUON_OK) {
        if (fuse && it == hp->ns_steps - 1)
          rc = run_ns_apply(plan, w, params, workspace, hp, small_iters, stream);
        else
          rc = run_ns_phase(plan, w, workspace, hp, it, 3, small_iters, stream);
      }
      if (rc != MUON_OK) return rc;
    }
    if (!fuse) {
      rc = muon_stage_apply(plan, w, params, workspace, workspace_bytes, hp, out_update, stream);
      if (rc != MUON_OK) return rc;
    }
  }
  return MUON_OK;
}

int muon_step_noalloc(const muon_plan_t* plan, void* params, const void* grads,
                      float* momentum, const muon_hparams_t* hp, float* out_update,
                      hipStream_t stream) {
  if (plan == nullptr) return fail(MUON_ERR_INVALID_ARG, "plan is null");
  if (plan->ws_bytes > MUON_NOALLOC_WORKSPACE_BYTES)
    return fail(MUON_ERR_WORKSPACE_TOO_SMALL,
                "plan needs " + std::to_string(plan->ws_bytes) +
                    " bytes of workspace; the static workspace holds " +
                    std::to_string(static_cast<size_t>(MUON_NOALLOC_WORKSPACE_BYTES)) +
                    " (create the plan with workspace_cap <= MUON_NOALLOC_WORKSPACE_BYTES)");
  if (plan->waves.empty()) return muon_step(plan, params, grads, momentum, nullptr, 0, hp,
                                            out_update, stream);
  if (!plan->uploaded)
    return fail(MUON_ERR_INVALID_ARG, "plan tables are not on a device (muon_plan_upload)");
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(MUON_ERR_INVALID_ARG, "current device differs from the plan's device");
  void* ws = nullptr;
  const int rc = static_ws_ptr(dev, &ws);
  if (rc != MUON_OK) return rc;
  return muon_step(plan, params, grads, momentum, ws, MUON_NOALLOC_WORKSPACE_BYTES, hp,
                   out_update, stream);
}

int adamw_step_ex(void* params, int32_t param_dtype, float* master, const void* grads,
                  int32_t grad_dtype, void* exp_avg, int32_t exp_avg_dtype, void* exp_avg_sq,
                  int32_t exp_avg_sq_dtype, int64_t n, const adamw_hparams_t* hp, int64_t step,
                  hipStream_t stream) {
  if (hp == nullptr) return fail(MUON_ERR_INVALID_ARG, "hparams is null");
  if (!dtype_ok(param_dtype) || !dtype_ok(grad_dtype))
    return fail(MUON_ERR_BAD_DTYPE, "dtype must be MUON_DTYPE_FP32 or MUON_DTYPE_BF16");
  if (!dtype_ok(exp_avg_dtype))
    return fail(MUON_ERR_BAD_DTYPE, "exp_avg must be MUON_DTYPE_FP32 or MUON_DTYPE_BF16");
  if (!dtype_ok(exp_avg_sq_dtype) && exp_avg_sq_dtype != MUON_DTYPE_FP16)
    return fail(MUON_ERR_BAD_DTYPE, "exp_avg_sq must be MUON_DTYPE_FP32, _BF16 or _FP16");
  if (param_dtype == MUON_DTYPE_BF16 && master == nullptr)
    return fail(MUON_ERR_INVALID_ARG, "bf16 parameters need a fp32 master copy");
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "n < 0");
  if (step < 1) return fail(MUON_ERR_INVALID_ARG, "step must be >= 1 (t starts at 1)");
  const float vals[] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
  for (float v : vals)
    if (!std::isfinite(v)) return fail(MUON_ERR_INVALID_ARG, "non-finite hyperparameter");
  if (hp->beta1 < 0.0f || hp->beta1 >= 1.0f || hp->beta2 < 0.0f || hp->beta2 >= 1.0f)
    return fail(MUON_ERR_INVALID_ARG, "betas must be in [0, 1)");
  if (n == 0) return MUON_OK;
  if (params == nullptr || grads == nullptr || exp_avg == nullptr || exp_avg_sq == nullptr)
    return fail(MUON_ERR_INVALID_ARG, "null buffer");
  // bias corrections in fp64 on the host
  const double bc1 = 1.0 - std::pow(static_cast<double>(hp->beta1), static_cast<double>(step));
  const double bc2 = 1.0 - std::pow(static_cast<double>(hp->beta2), static_cast<double>(step));
  const float lr_bc1 = static_cast<float>(static_cast<double>(hp->lr) / bc1);
  const float rsqrt_bc2 = static_cast<float>(1.0 / std::sqrt(bc2));
  const hipError_t e = muon::launch_adamw(
      params, param_dtype, master, grads, grad_dtype, exp_avg, exp_avg_dtype, exp_avg_sq,
      exp_avg_sq_dtype, n, hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, lr_bc1,
      rsqrt_bc2, clip_of(hp->clip), stream);
  if (e != hipSuccess) return hip_fail(e, "AdamW kernel launch");
  return MUON_OK;
}

int adamw_step(void* params, int32_t param_dtype, float* master, const void* grads,
               int32_t grad_dtype, float* exp_avg, float* exp_avg_sq, int64_t n,
               const adamw_hparams_t* hp, int64_t step, hipStream_t stream) {
  return adamw_step_ex(params, param_dtype, master, grads, grad_dtype, exp_avg, MUON_DTYPE_FP32,
                       exp_avg_sq, MUON_DTYPE_FP32, n, hp, step, stream);
}

size_t grad_norm_clip_workspace_size(int32_t n_bufs) {
  return n_bufs > 0 ? static_cast<size_t>(n_bufs) * muon::kReduceBlocks * sizeof(double) : 0;
}

int grad_norm_clip(const muon_grad_buffer_t* bufs, int32_t n_bufs, float max_norm, float eps,
                   void* workspace, size_t workspace_bytes, muon_clip_state_t* out,
                   hipStream_t stream) {
  if (out == nullptr) return fail(MUON_ERR_INVALID_ARG, "out is null");
  if (n_bufs < 0 || (n_bufs > 0 && bufs == nullptr))
    return fail(MUON_ERR_INVALID_ARG, "bad buffer list");
  if (!std::isfinite(max_norm) || !std::isfinite(eps) || eps < 0.0f)
    return fail(MUON_ERR_INVALID_ARG, "max_norm must be finite and eps finite and >= 0");
  for (int32_t b = 0; b < n_bufs; ++b) {
    if (bufs[b].n < 0) return fail(MUON_ERR_INVALID_ARG, "buffer " + std::to_string(b) + ": n < 0");
    if (!dtype_ok(bufs[b].dtype))
      return fail(MUON_ERR_BAD_DTYPE, "buffer " + std::to_string(b) + ": bad dtype");
    if (bufs[b].n > 0 && bufs[b].ptr == nullptr)
      return fail(MUON_ERR_INVALID_ARG, "buffer " + std::to_string(b) + " is null");
  }
  const size_t need = grad_norm_clip_workspace_size(n_bufs);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                   reinterpret_cast<uintptr_t>(workspace) % alignof(double) != 0))
    return fail(MUON_ERR_WORKSPACE_TOO_SMALL,
                "grad_norm_clip needs " + std::to_string(need) + " bytes, 8-byte aligned");
  double* partials = static_cast<double*>(workspace);
  for (int32_t b = 0; b < n_bufs; ++b) {
    const hipError_t e = muon::launch_sumsq(bufs[b].ptr, bufs[b].dtype, bufs[b].n,
                                            partials + static_cast<size_t>(b) * muon::kReduceBlocks,
                                            stream);
    if (e != hipSuccess) return hip_fail(e, "sum-of-squares kernel launch");
  }
  const hipError_t e = muon::launch_clip_finalize(partials, n_bufs * muon::kReduceBlocks,
                                                  max_norm, eps,
                                                  reinterpret_cast<muon::ClipState*>(out), stream);
  if (e != hipSuccess) return hip_fail(e, "clip kernel launch");
  return MUON_OK;
}

size_t state_stats_workspace_size(void) {
  return static_cast<size_t>(muon::kReduceBlocks) * muon::kStatsPartialBytes;
}

int state_stats(const float* x, int64_t n, void* workspace, size_t workspace_bytes,
                muon_state_stats_t* out, hipStream_t stream) {
  if (out == nullptr) return fail(MUON_ERR_INVALID_ARG, "out is null");
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && x == nullptr) return fail(MUON_ERR_INVALID_ARG, "x is null");
  if (reinterpret_cast<uintptr_t>(out) % alignof(double) != 0)
    return fail(MUON_ERR_INVALID_ARG, "out must be 8-byte aligned");
  const size_t need = state_stats_workspace_size();
  if (workspace == nullptr || workspace_bytes < need ||
      reinterpret_cast<uintptr_t>(workspace) % alignof(double) != 0)
    return fail(MUON_ERR_WORKSPACE_TOO_SMALL,
                "state_stats needs " + std::to_string(need) + " bytes, 8-byte aligned");
  const hipError_t e = muon::launch_state_stats(x, n, workspace, out, stream);
  if (e != hipSuccess) return hip_fail(e, "statistics kernel launch");
  return MUON_OK;
}

}  // extern "C"
