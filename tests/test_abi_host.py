"""Host-only checks of the C ABI: the library loads, exports every symbol
include/muon.h declares, and rejects bad input before any HIP call."""

import ctypes
import os
import re

import pytest

import muon_newton_schulz_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "muon.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_binding_names():
    assert set(_declared_functions()) == set(M.EXPORTED)


def test_library_loads_and_exports_every_symbol():
    L = M.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings():
    assert M.muon_status_string(0) == "ok"
    for code in range(-7, 0):
        assert M.muon_status_string(code) not in ("ok", "unknown status")
    assert M.muon_status_string(-99) == "unknown status"


def _err(fn, *a, **k):
    with pytest.raises(M.MuonError) as e:
        fn(*a, **k)
    return e.value.status


def test_workspace_size_validation():
    ws = M.muon_workspace_size
    assert _err(ws, [(0, 0, 5)], 10, "bf16", "bf16", "bf16") == M.MUON_ERR_BAD_SHAPE
    assert _err(ws, [(0, 4, 4)], 15, "bf16", "bf16", "bf16") == M.MUON_ERR_BAD_SHAPE
    assert _err(ws, [(-1, 2, 2)], 15, "bf16", "bf16", "bf16") == M.MUON_ERR_BAD_SHAPE
    assert _err(ws, [(0, 4, 4), (15, 2, 2)], 100, "bf16", "bf16", "bf16") == M.MUON_ERR_OVERLAP
    assert _err(ws, [(20, 4, 4), (0, 5, 5)], 100, "bf16", "bf16", "bf16") == M.MUON_ERR_OVERLAP
    with pytest.raises(M.MuonError):
        ws([(0, 4, 4)], 16, "fp16", "bf16", "bf16")
    # a cap smaller than one matrix needs
    assert _err(ws, [(0, 300, 300)], 90000, "bf16", "bf16", "bf16", 1024) == \
        M.MUON_ERR_WORKSPACE_TOO_SMALL
    assert "matrix 0" in M.muon_last_error()


def test_workspace_size_layout():
    # bf16 NS pads to 256: a 300x100 (tall) matrix is oriented 100x300 ->
    # m_pad 256, n_pad 512; X ping-pong (2*256*512) and A, B (2*256*256), bf16.
    b = M.muon_workspace_size([(0, 300, 100)], 30000, "bf16", "bf16", "bf16")
    k1 = (512 // 64) * (256 // 64)
    # fp64 partials (k1*8 <= 256), norms, inverse norms, and the NS
    # kernels' round counters (8 groups x 256 bytes)
    fixed = 256 + 256 + 256 + 2048
    assert k1 * 8 <= 256
    assert b == fixed + 2 * (2 * 256 * 512 + 2 * 256 * 256)
    # fp32 NS pads to 64: 128x256 -> X ping-pong and A, B in fp32
    b = M.muon_workspace_size([(0, 128, 256)], 128 * 256, "fp32", "fp32", "fp32")
    k1 = 2 * 4
    assert b == 256 * 3 + 2048 + 4 * (2 * 128 * 256 + 2 * 128 * 128)
    # empty plan
    assert M.muon_workspace_size([], 0, "bf16", "bf16", "bf16") == 0


def test_waves_bound_the_workspace():
    mats = [(k * 512 * 512, 512, 512) for k in range(6)]
    one = M.muon_workspace_size(mats[:1], 512 * 512, "bf16", "bf16", "bf16")
    full = M.muon_workspace_size(mats, 6 * 512 * 512, "bf16", "bf16", "bf16")
    capped = M.muon_workspace_size(mats, 6 * 512 * 512, "bf16", "bf16", "bf16", 2 * one + 1024)
    assert capped <= 2 * one + 1024
    assert capped < full


def test_adamw_validation_before_any_hip_call():
    import torch
    p = torch.zeros(8, dtype=torch.bfloat16)
    g = torch.zeros(8, dtype=torch.bfloat16)
    m = torch.zeros(8)
    v = torch.zeros(8)
    hp = M.AdamWHParamsC(0.01, 0.9, 0.95, 1e-8, 0.1)
    assert _err(M.adamw_step, p, None, g, m, v, hp, 1, stream=0) == M.MUON_ERR_INVALID_ARG
    p32 = torch.zeros(8)
    assert _err(M.adamw_step, p32, None, p32, m, v, hp, 0, stream=0) == M.MUON_ERR_INVALID_ARG
    bad = M.AdamWHParamsC(0.01, 1.0, 0.95, 1e-8, 0.1)
    assert _err(M.adamw_step, p32, None, p32, m, v, bad, 1, stream=0) == M.MUON_ERR_INVALID_ARG
    assert _err(M.adamw_step, p32, None, p32, m, torch.zeros(7), hp, 1, stream=0) == \
        M.MUON_ERR_INVALID_ARG


def test_guard_entry_points_validate_before_any_hip_call():
    L = M.lib()
    P = ctypes.c_void_p
    fake = P(4096)  # never dereferenced: every case fails validation first
    bufs = (M.MuonGradBuffer * 2)(M.MuonGradBuffer(fake, 10, 1, 0), M.MuonGradBuffer(fake, 10, 7, 0))
    ws_need = M.grad_norm_clip_workspace_size(2)
    assert ws_need == 2 * 1024 * 8
    assert M.grad_norm_clip_workspace_size(0) == 0
    assert L.grad_norm_clip(bufs, 2, 1.0, 1e-6, fake, ws_need, fake, None) == M.MUON_ERR_BAD_DTYPE
    bufs[1] = M.MuonGradBuffer(None, 10, 0, 0)
    assert L.grad_norm_clip(bufs, 2, 1.0, 1e-6, fake, ws_need, fake, None) == M.MUON_ERR_INVALID_ARG
    bufs[1] = M.MuonGradBuffer(None, -1, 0, 0)
    assert L.grad_norm_clip(bufs, 2, 1.0, 1e-6, fake, ws_need, fake, None) == M.MUON_ERR_INVALID_ARG
    bufs[1] = M.MuonGradBuffer(None, 0, 0, 0)  # empty buffers may be null
    assert L.grad_norm_clip(bufs, 2, 1.0, 1e-6, fake, ws_need - 8, fake, None) == \
        M.MUON_ERR_WORKSPACE_TOO_SMALL
    assert L.grad_norm_clip(bufs, 2, 1.0, 1e-6, fake, ws_need, None, None) == M.MUON_ERR_INVALID_ARG
    assert L.grad_norm_clip(bufs, 2, float("nan"), 1e-6, fake, ws_need, fake, None) == \
        M.MUON_ERR_INVALID_ARG
    assert L.grad_norm_clip(bufs, 2, 1.0, -1.0, fake, ws_need, fake, None) == M.MUON_ERR_INVALID_ARG
    assert L.grad_norm_clip(None, 1, 1.0, 1e-6, fake, ws_need, fake, None) == M.MUON_ERR_INVALID_ARG
    s_need = M.state_stats_workspace_size()
    assert s_need == 1024 * 64
    assert L.state_stats(fake, 10, fake, s_need, None, None) == M.MUON_ERR_INVALID_ARG
    assert L.state_stats(fake, -1, fake, s_need, fake, None) == M.MUON_ERR_INVALID_ARG
    assert L.state_stats(None, 10, fake, s_need, fake, None) == M.MUON_ERR_INVALID_ARG
    assert L.state_stats(fake, 10, fake, s_need - 1, fake, None) == M.MUON_ERR_WORKSPACE_TOO_SMALL
    assert L.state_stats(fake, 10, P(4097), s_need, fake, None) == M.MUON_ERR_WORKSPACE_TOO_SMALL
    assert L.state_stats(fake, 10, fake, s_need, P(4100), None) == M.MUON_ERR_INVALID_ARG


def test_hparam_structs_carry_the_clip_pointer():
    # the binding's structs mirror include/muon.h: the clip pointer is last
    assert [f for f, _ in M.MuonHParamsC._fields_][-1] == "clip"
    assert [f for f, _ in M.AdamWHParamsC._fields_][-1] == "clip"
    assert ctypes.sizeof(M.MuonClipState) == 16
    assert ctypes.sizeof(M.MuonStateStats) == 56
    assert ctypes.sizeof(M.MuonGradBuffer) == 24
    h = M._hp(M.MuonHParamsC(0.02, 0.1, 0.95, 1, 1.5, -0.5, 0.0, 5, 1e-7, 0, 0.2))
    assert h.clip is None


def test_adamw_step_ex_validates_state_dtypes():
    L = M.lib()
    P = ctypes.c_void_p
    fake = P(4096)
    hp = M.AdamWHParamsC(0.01, 0.9, 0.95, 1e-8, 0.1)
    args = lambda mdt, vdt: (fake, 0, None, fake, 0, fake, mdt, fake, vdt, 8,  # noqa: E731
                             ctypes.byref(hp), 1, None)
    assert L.adamw_step_ex(*args(2, 0)) == M.MUON_ERR_BAD_DTYPE   # m cannot be fp16
    assert L.adamw_step_ex(*args(0, 3)) == M.MUON_ERR_BAD_DTYPE
    assert L.adamw_step_ex(*args(-1, 0)) == M.MUON_ERR_BAD_DTYPE
    h0 = M.AdamWHParamsC(0.01, 0.9, 0.95, 1e-8, 0.1)
    assert L.adamw_step_ex(fake, 0, None, fake, 0, fake, 1, fake, 2, 0, ctypes.byref(h0), 0,
                           None) == M.MUON_ERR_INVALID_ARG  # step 0


def _clip_plan_rc(targets, flat_numel=1000, dtype=1, n_groups=0):
    L = M.lib()
    arr = (M.MuonClipTarget * max(1, len(targets)))(*[M.MuonClipTarget(*t) for t in targets])
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)
    return L.muon_clip_plan_create(arr, len(targets), flat_numel, dtype, n_groups,
                                   ctypes.byref(h), ctypes.byref(ws))


def test_clip_plan_validates_before_any_hip_call():
    # (offset, ld, rows, cols, group, reserved)
    assert ctypes.sizeof(M.MuonClipTarget) == 32
    assert _clip_plan_rc([(0, 10, 10, 10, 0, 0)], dtype=2) == M.MUON_ERR_BAD_DTYPE
    assert _clip_plan_rc([(0, 10, 0, 10, 0, 0)]) == M.MUON_ERR_BAD_SHAPE          # rows 0
    assert _clip_plan_rc([(0, 5, 2, 10, 0, 0)]) == M.MUON_ERR_BAD_SHAPE           # ld < cols
    assert _clip_plan_rc([(-1, 10, 2, 10, 0, 0)]) == M.MUON_ERR_BAD_SHAPE         # offset < 0
    assert _clip_plan_rc([(991, 10, 1, 10, 0, 0)]) == M.MUON_ERR_BAD_SHAPE        # past the end
    assert _clip_plan_rc([(0, 100, 10, 10, 0, 0)], flat_numel=909) == M.MUON_ERR_BAD_SHAPE
    assert _clip_plan_rc([(0, 100, 10, 10, 0, 0)], flat_numel=910) != M.MUON_ERR_BAD_SHAPE
    assert _clip_plan_rc([(0, 1 << 16, 1 << 16, 1 << 16, 0, 0)],
                         flat_numel=1 << 40) == M.MUON_ERR_BAD_SHAPE             # > 2^31 elements
    assert _clip_plan_rc([(0, 10, 1, 10, 1, 0)], n_groups=1) == M.MUON_ERR_INVALID_ARG
    assert _clip_plan_rc([(0, 10, 1, 10, -1, 0)]) == M.MUON_ERR_INVALID_ARG
    # overlaps: contiguous blocks, and interleaved strided blocks
    assert _clip_plan_rc([(0, 10, 2, 10, 0, 0), (19, 10, 1, 10, 0, 0)]) == M.MUON_ERR_OVERLAP
    assert _clip_plan_rc([(0, 20, 5, 10, 0, 0), (9, 20, 5, 10, 0, 0)]) == M.MUON_ERR_OVERLAP
    # two column blocks of one matrix interleave without sharing elements:
    # validation passes and the call gets as far as the device (no GPU here)
    rc = _clip_plan_rc([(0, 20, 5, 10, 0, 0), (10, 20, 5, 10, 0, 0)])
    assert rc not in (M.MUON_ERR_OVERLAP, M.MUON_ERR_BAD_SHAPE, M.MUON_ERR_INVALID_ARG)
    L = M.lib()
    assert L.muon_clip_plan_create(None, 1, 10, 1, 0, ctypes.byref(ctypes.c_void_p()),
                                   None) == M.MUON_ERR_INVALID_ARG
    fake = ctypes.c_void_p(4096)
    assert L.muon_clip(None, fake, 0, 1.0, None, fake, 8, None, None, None) == \
        M.MUON_ERR_INVALID_ARG
    L.muon_clip_plan_destroy(None)  # a null plan is a no-op


def test_plan_flags_validate_before_any_hip_call():
    L = M.lib()
    mats = (M.MuonMatrix * 1)(M.MuonMatrix(0, 8, 8))
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)

    def rc(flags):
        return L.muon_plan_create_ex(mats, 1, 64, 1, 1, 1, 0, flags, ctypes.byref(h),
                                     ctypes.byref(ws))
    assert M.MUON_PLAN_TILED_ONLY == 1 and M.MUON_PLAN_WHOLE_TILES == 2
    assert M.MUON_PLAN_FREE_ROUNDS == 4
    assert rc(8) == M.MUON_ERR_INVALID_ARG
    assert rc(1 << 31) == M.MUON_ERR_INVALID_ARG
    # the known flags pass validation (creation is host-only)
    for f in range(8):
        assert rc(f) == M.MUON_OK
        L.muon_plan_destroy(h)


def test_longest_side_a_plan_accepts():
    # elementwise tile coordinates (64-element tiles of the side padded to
    # the GEMM tile) are packed in 16 bits: bf16 NS pads to 256, so the
    # longest side is 16383 * 256; fp32 NS pads to 64: 65535 * 64
    ws = M.muon_workspace_size
    for nsd, longest in (("bf16", 16383 * 256), ("fp32", 65535 * 64)):
        for shape in ((1, longest), (longest, 1)):
            assert ws([(0, *shape)], longest, nsd, nsd, nsd) > 0
        for shape in ((1, longest + 1), (longest + 1, 1)):
            assert _err(ws, [(0, *shape)], longest + 1, nsd, nsd, nsd) == M.MUON_ERR_BAD_SHAPE
            assert "too large" in M.muon_last_error()


def test_stage_ns_apply_validates_before_any_hip_call():
    L = M.lib()
    hp = M.MuonHParamsC()
    fake = ctypes.c_void_p(4096)
    assert L.muon_stage_ns_apply(None, 0, fake, fake, 1 << 20, ctypes.byref(hp), None) == \
        M.MUON_ERR_INVALID_ARG
    # plan info carries the count of matrices whose update the last NS phase applies
    names = [f[0] for f in M.MuonPlanInfo._fields_]
    assert names[-2:] == ["fused_apply_mats", "round_sync_phases"]


def test_plans_are_host_only_until_uploaded():
    # creation makes no HIP call (this container has no GPU) and keeps its
    # tables in host memory; every step refuses a plan not yet uploaded
    L = M.lib()
    mats = (M.MuonMatrix * 2)(M.MuonMatrix(0, 300, 520), M.MuonMatrix(156000, 520, 300))
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)
    assert L.muon_plan_create(mats, 2, 312000, 1, 1, 1, 0, ctypes.byref(h),
                              ctypes.byref(ws)) == M.MUON_OK
    assert h.value and ws.value > 0
    nb = L.muon_plan_table_bytes(h)
    assert nb > 0 and nb % 256 == 0
    info = M.MuonPlanInfo()
    assert L.muon_plan_get_info(h, ctypes.byref(info)) == M.MUON_OK and info.n_mats == 2
    fake = ctypes.c_void_p(1 << 20)
    hp = M.MuonHParamsC(0.02, 0.1, 0.95, 1, 1.5, -0.5, 0.0, 5, 1e-7, 0, 0.2)
    assert L.muon_step(h, fake, fake, fake, fake, ws.value, ctypes.byref(hp), None,
                       None) == M.MUON_ERR_INVALID_ARG
    assert "muon_plan_upload" in M.muon_last_error()
    assert L.muon_stage_ns_phase(h, 0, fake, ws.value, ctypes.byref(hp), 0, 1,
                                 None) == M.MUON_ERR_INVALID_ARG
    # upload argument checks come before any HIP call
    assert L.muon_plan_upload(h, None, nb, None) == M.MUON_ERR_INVALID_ARG
    assert L.muon_plan_upload(h, ctypes.c_void_p((1 << 20) + 8), nb, None) == \
        M.MUON_ERR_INVALID_ARG                                  # not 256-byte aligned
    assert L.muon_plan_upload(h, fake, nb - 1, None) == M.MUON_ERR_INVALID_ARG
    assert L.muon_plan_upload(None, fake, nb, None) == M.MUON_ERR_INVALID_ARG
    L.muon_plan_destroy(h)
    assert L.muon_plan_table_bytes(None) == 0
    # an empty plan has no tables
    e = ctypes.c_void_p(0)
    assert L.muon_plan_create(None, 0, 0, 1, 1, 1, 0, ctypes.byref(e), None) == M.MUON_OK
    assert L.muon_plan_table_bytes(e) == 0
    L.muon_plan_destroy(e)


def test_clip_plans_are_host_only_until_uploaded():
    L = M.lib()
    arr = (M.MuonClipTarget * 2)(M.MuonClipTarget(0, 10, 5, 10, 0, 0),
                                 M.MuonClipTarget(50, 10, 5, 10, 0, 0))
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)
    assert L.muon_clip_plan_create(arr, 2, 100, 1, 0, ctypes.byref(h), ctypes.byref(ws)) == \
        M.MUON_OK
    nb = L.muon_clip_plan_table_bytes(h)
    assert nb > 0
    fake = ctypes.c_void_p(1 << 20)
    assert L.muon_clip(h, fake, 0, 1.0, None, fake, 1 << 12, None, None, None) == \
        M.MUON_ERR_INVALID_ARG
    assert "muon_clip_plan_upload" in M.muon_last_error()
    assert L.muon_clip_plan_upload(h, None, nb, None) == M.MUON_ERR_INVALID_ARG
    assert L.muon_clip_plan_upload(h, fake, nb - 1, None) == M.MUON_ERR_INVALID_ARG
    L.muon_clip_plan_destroy(h)


def test_library_allocates_no_device_memory_and_never_synchronises():
    # the product library's sources (the stand-alone ceiling programs aside)
    # call no HIP allocator, no blocking copy and no synchronisation
    csrc = os.path.join(ROOT, "muon_newton_schulz_amd", "csrc")
    from muon_newton_schulz_amd.build import SOURCES
    banned = re.compile(r"\bhip(Malloc\w*|Free\w*|HostMalloc|HostAlloc|MallocAsync|Memcpy|"
                        r"Memset|DeviceSynchronize|StreamSynchronize|EventSynchronize)\s*\(")
    for f in SOURCES + ["muon_internal.h"]:
        text = re.sub(r"//[^\n]*", "", open(os.path.join(csrc, f)).read())
        assert not banned.search(text), (f, banned.search(text).group(0))


def test_round_barrier_choice():
    # Phases 1 and 2 hold each XCD's tile rounds together only where the
    # plan's cost model predicts almost no idle time.  2048-sided matrices
    # mix split diagonal tiles (10 of 16 MFMA blocks) into every round of
    # the triangle, so they run free; larger ones run their diagonal tiles
    # last, and their rounds are uniform.  Phase 3 never holds; neither does
    # a list of at most 4 rounds of 256 tiles (the hold comes every 4th
    # round), nor the fp32 engine.
    def phases(mats, nsd="bf16"):
        n = max(o + r * c for o, r, c in mats)
        plan = M.muon_plan_create(mats, n, nsd, nsd, nsd, upload=False)
        try:
            return plan.info().round_sync_phases
        finally:
            plan.close()
    sq = [(k * 2048 * 2048, 2048, 2048) for k in range(64)]
    assert phases(sq) == 0
    big = [(k * 4096 * 8192, 4096, 8192) for k in range(8)]
    assert phases(big) == 0b11
    assert phases(big[:7]) == 0         # 7 x 136 triangle tiles: 4 rounds
    assert phases(big, "fp32") == 0
