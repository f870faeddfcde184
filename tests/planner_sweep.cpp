// Seeded sweep of the host-side planners (muon_workspace_size,
// muon_plan_create_ex, muon_plan_get_info, muon_plan_table_bytes and the
// MuonClip planner) over valid and invalid descriptors: sides up to the
// longest accepted, offsets past 2^32 elements, waves under small caps,
// overlaps and out-of-range matrices.  Built by
// tests/test_planner_sanitized.py with the host code under AddressSanitizer
// and UndefinedBehaviorSanitizer; it makes no HIP call and needs no GPU.
//
// Prints "ok <valid plans> <rejected>" and exits 0, or exits 1 on a broken
// invariant.
#include <algorithm>
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "muon.h"

namespace {

struct Rng {  // splitmix64
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int64_t range(int64_t lo, int64_t hi) {  // inclusive
    return lo + static_cast<int64_t>(next() % static_cast<uint64_t>(hi - lo + 1));
  }
};

int g_fail = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #cond); \
      g_fail = 1;                                                        \
    }                                                                    \
  } while (0)

const int32_t kLongestBf16 = 16383 * 256;  // bf16 NS pads to 256: 16-bit tile coordinates
const int32_t kLongestFp32 = 65535 * 64;

int64_t plan_once(const std::vector<muon_matrix_t>& mats, int64_t flat, int32_t pd, int32_t gd,
                  int32_t nd, size_t cap, uint32_t flags, bool expect_ok) {
  size_t ws = 0;
  const int rc_ws =
      muon_workspace_size(mats.data(), static_cast<int32_t>(mats.size()), flat, pd, gd, nd, cap, &ws);
  muon_plan_t* plan = nullptr;
  size_t ws2 = 0;
  const int rc = muon_plan_create_ex(mats.data(), static_cast<int32_t>(mats.size()), flat, pd, gd,
                                     nd, cap, flags, &plan, &ws2);
  if (flags == 0) CHECK(rc == rc_ws);
  if (expect_ok) CHECK(rc == MUON_OK);
  if (rc != MUON_OK) {
    CHECK(plan == nullptr);
    CHECK(muon_last_error()[0] != '\0');
    return -1;
  }
  if (flags == 0) CHECK(ws == ws2);
  CHECK(cap == 0 || ws2 <= cap);
  muon_plan_info_t info;
  CHECK(muon_plan_get_info(plan, &info) == MUON_OK);
  CHECK(info.n_mats == static_cast<int32_t>(mats.size()));
  CHECK(info.workspace_bytes == ws2);
  CHECK(info.n_waves >= (mats.empty() ? 0 : 1));
  CHECK(info.small_mats + info.split_tile_mats <= info.n_mats);
  CHECK(info.fused_apply_mats <= info.n_mats);
  const size_t tb = muon_plan_table_bytes(plan);
  CHECK(mats.empty() ? tb == 0 : (tb > 0 && tb % 256 == 0));
  // a step refuses a plan that was never uploaded, before any HIP call
  muon_hparams_t hp;
  std::memset(&hp, 0, sizeof(hp));
  hp.lr = 0.02f;
  hp.momentum = 0.95f;
  hp.ns_a = 1.5f;
  hp.ns_b = -0.5f;
  hp.ns_steps = 5;
  hp.eps = 1e-7f;
  if (!mats.empty()) {
    void* fake = reinterpret_cast<void*>(uintptr_t{1} << 20);
    CHECK(muon_stage_momentum(plan, 0, fake, static_cast<float*>(fake), fake, ws2, &hp, nullptr) ==
          MUON_ERR_INVALID_ARG);
  }
  muon_plan_destroy(plan);
  return static_cast<int64_t>(ws2);
}

}  // namespace

int main() {
  Rng rng{20261202};
  int valid = 0, rejected = 0;
  const int32_t dts[2] = {MUON_DTYPE_FP32, MUON_DTYPE_BF16};

  // 1. random valid layouts: ragged sides, gaps, offsets past 2^32
  for (int t = 0; t < 400; ++t) {
    const int n = static_cast<int>(rng.range(0, 24));
    const int32_t nd = dts[rng.range(0, 1)];
    int64_t off = rng.range(0, 3) == 0 ? (int64_t{1} << 32) + rng.range(0, 1 << 20) : rng.range(0, 64);
    std::vector<muon_matrix_t> mats;
    for (int i = 0; i < n; ++i) {
      muon_matrix_t m;
      const int kind = static_cast<int>(rng.range(0, 9));
      if (kind == 0) {
        m.rows = 1;
        m.cols = static_cast<int32_t>(rng.range(1, 70000));
      } else if (kind == 1) {
        m.rows = static_cast<int32_t>(rng.range(1, 70000));
        m.cols = 1;
      } else {
        m.rows = static_cast<int32_t>(rng.range(1, 3000));
        m.cols = static_cast<int32_t>(rng.range(1, 3000));
      }
      m.offset = off;
      off += static_cast<int64_t>(m.rows) * m.cols + rng.range(0, 9);
      mats.push_back(m);
    }
    const int64_t flat = off + rng.range(0, 5);
    const uint32_t flags = static_cast<uint32_t>(rng.range(0, 3));
    // caps: none, or a few times the largest matrix's own need (waves)
    size_t cap = 0;
    if (!mats.empty() && rng.range(0, 1)) {
      size_t biggest = 0;
      for (const muon_matrix_t& m : mats) {
        size_t one = 0;
        CHECK(muon_workspace_size(&m, 1, flat, dts[1], dts[1], nd, 0, &one) == MUON_OK);
        if (one > biggest) biggest = one;
      }
      cap = biggest * static_cast<size_t>(rng.range(1, 4));
    }
    const int64_t ws = plan_once(mats, flat, dts[rng.range(0, 1)], dts[rng.range(0, 1)], nd, cap,
                                 flags, true);
    if (ws >= 0) ++valid;
  }

  // 2. the longest accepted sides (and one past them) for each NS dtype
  for (int32_t nd : dts) {
    const int32_t L = nd == MUON_DTYPE_BF16 ? kLongestBf16 : kLongestFp32;
    for (int shape = 0; shape < 2; ++shape) {
      muon_matrix_t m{(int64_t{1} << 33) + 7, shape ? L : 1, shape ? 1 : L};
      std::vector<muon_matrix_t> v{m};
      if (plan_once(v, m.offset + L, nd, nd, nd, 0, 0, true) >= 0) ++valid;
      m.rows = shape ? L + 1 : 1;
      m.cols = shape ? 1 : L + 1;
      v[0] = m;
      if (plan_once(v, m.offset + L + 1, nd, nd, nd, 0, 0, false) < 0) ++rejected;
      else CHECK(false);
    }
  }

  // 3. invalid descriptors are rejected
  for (int t = 0; t < 300; ++t) {
    std::vector<muon_matrix_t> mats;
    int64_t off = rng.range(0, 100);
    const int n = static_cast<int>(rng.range(1, 8));
    for (int i = 0; i < n; ++i) {
      muon_matrix_t m{off, static_cast<int32_t>(rng.range(1, 500)), static_cast<int32_t>(rng.range(1, 500))};
      off += static_cast<int64_t>(m.rows) * m.cols;
      mats.push_back(m);
    }
    int64_t flat = off;
    const int bad = static_cast<int>(rng.range(0, 5));
    const int i = static_cast<int>(rng.range(0, n - 1));
    if (bad == 0) mats[i].rows = -static_cast<int32_t>(rng.range(0, 5));
    if (bad == 1) mats[i].offset = -rng.range(1, 1000);
    if (bad == 2) flat = off - rng.range(1, 100);  // last matrix past the end
    if (bad == 3 && n > 1) mats[i].offset = mats[(i + 1) % n].offset + rng.range(0, 3);  // overlap
    if (bad == 4) mats[i].cols = 0;
    if (bad == 5) flat = -1;
    if (bad == 2) {
      // only the matrix that reaches flat_numel is out of range
      int64_t end = 0;
      for (const muon_matrix_t& m : mats) end = std::max<int64_t>(end, m.offset + int64_t{m.rows} * m.cols);
      if (end <= flat) continue;
    }
    if (bad == 3 && n == 1) continue;
    if (plan_once(mats, flat, dts[1], dts[1], dts[1], 0, 0, false) < 0) ++rejected;
    else CHECK(false);
  }
  // bad dtypes, flags, counts, null pointers, a cap below one matrix
  {
    std::vector<muon_matrix_t> one{{0, 300, 300}};
    muon_plan_t* p = nullptr;
    size_t ws = 0;
    CHECK(muon_plan_create_ex(one.data(), 1, 90000, 7, 1, 1, 0, 0, &p, &ws) == MUON_ERR_BAD_DTYPE);
    CHECK(muon_plan_create_ex(one.data(), 1, 90000, 1, 1, 1, 0, 8u, &p, &ws) == MUON_ERR_INVALID_ARG);
    CHECK(muon_plan_create_ex(one.data(), -1, 90000, 1, 1, 1, 0, 0, &p, &ws) == MUON_ERR_INVALID_ARG);
    CHECK(muon_plan_create_ex(nullptr, 1, 90000, 1, 1, 1, 0, 0, &p, &ws) == MUON_ERR_INVALID_ARG);
    CHECK(muon_plan_create_ex(one.data(), 1, 90000, 1, 1, 1, 0, 0, nullptr, &ws) == MUON_ERR_INVALID_ARG);
    CHECK(muon_plan_create_ex(one.data(), 1, 90000, 1, 1, 1, 1024, 0, &p, &ws) ==
          MUON_ERR_WORKSPACE_TOO_SMALL);
    CHECK(muon_workspace_size(one.data(), 1, 90000, 1, 1, 1, 0, nullptr) == MUON_ERR_INVALID_ARG);
    CHECK(muon_plan_table_bytes(nullptr) == 0);
    muon_plan_destroy(nullptr);
    rejected += 7;
  }

  // 4. MuonClip planner: strided and whole blocks, valid and overlapping
  for (int t = 0; t < 200; ++t) {
    std::vector<muon_clip_target_t> tg;
    const int n = static_cast<int>(rng.range(1, 12));
    int64_t off = rng.range(0, 1) ? (int64_t{1} << 32) : 0;
    const int groups = static_cast<int>(rng.range(0, 4));
    for (int i = 0; i < n; ++i) {
      muon_clip_target_t c;
      c.rows = static_cast<int32_t>(rng.range(1, 300));
      c.cols = static_cast<int32_t>(rng.range(1, 300));
      c.ld = c.cols + rng.range(0, 2) * rng.range(0, 50);
      c.offset = off;
      c.group = static_cast<int32_t>(rng.range(0, groups > 0 ? groups - 1 : 0));
      c.reserved = 0;
      off += (c.rows - 1) * c.ld + c.cols + rng.range(0, 5);
      tg.push_back(c);
    }
    const bool overlap = n > 1 && rng.range(0, 3) == 0;
    if (overlap) tg[1].offset = tg[0].offset;
    muon_clip_plan_t* cp = nullptr;
    size_t ws = 0;
    const int rc = muon_clip_plan_create(tg.data(), n, off, MUON_DTYPE_BF16, groups, &cp, &ws);
    if (overlap) {
      CHECK(rc == MUON_ERR_OVERLAP);
      ++rejected;
    } else {
      CHECK(rc == MUON_OK);
      if (rc == MUON_OK) {
        CHECK(muon_clip_plan_table_bytes(cp) > 0);
        ++valid;
      }
    }
    muon_clip_plan_destroy(cp);
  }

  if (g_fail) return 1;
  std::printf("ok %d %d\n", valid, rejected);
  return 0;
}
