"""MI355X-native Muon (Newton-Schulz) and AdamW optimizer step.

Thin ctypes binding over ``libmuon.so`` (C ABI in ``include/muon.h``).  The
functions keep the C names; they only marshal arguments (tensor ->
device pointer, dtype -> code, current torch stream -> hipStream_t) and
turn status codes into ``MuonError``.  Every step of the optimizer runs in
the library's HIP kernels; there is no Python or CPU fallback: if the
library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmuon.so")

MUON_OK = 0
MUON_ERR_INVALID_ARG = -1
MUON_ERR_BAD_SHAPE = -2
MUON_ERR_OVERLAP = -3
MUON_ERR_WORKSPACE_TOO_SMALL = -4
MUON_ERR_BAD_DTYPE = -5
MUON_ERR_HIP = -6
MUON_ERR_UNSUPPORTED = -7

MUON_DTYPE_FP32 = 0
MUON_DTYPE_BF16 = 1
MUON_DTYPE_FP16 = 2

EXPORTED = [
    "muon_workspace_size", "muon_plan_create", "muon_plan_create_ex", "muon_plan_destroy",
    "muon_plan_get_info", "muon_plan_table_bytes", "muon_plan_upload",
    "muon_step", "muon_step_noalloc", "muon_stage_momentum", "muon_stage_ns_phase",
    "muon_stage_apply",
    "muon_stage_ns_apply",
    "muon_stage_export_x", "muon_stage_export_norms", "adamw_step", "adamw_step_ex",
    "muon_status_string",
    "muon_last_error", "grad_norm_clip_workspace_size", "grad_norm_clip",
    "state_stats_workspace_size", "state_stats",
    "muon_clip_plan_create", "muon_clip_plan_destroy", "muon_clip_plan_table_bytes",
    "muon_clip_plan_upload", "muon_clip",
]

MUON_CLIP_FROBENIUS = 0
MUON_CLIP_MAX_LOGIT = 1
# size of the library's static device workspace (muon_step_noalloc)
MUON_NOALLOC_WORKSPACE_BYTES = 256 << 20


class MuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class MuonMatrix(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class MuonHParamsC(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("momentum", ctypes.c_float), ("nesterov", ctypes.c_int32),
                ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
                ("ns_steps", ctypes.c_int32), ("eps", ctypes.c_float),
                ("scale_mode", ctypes.c_int32), ("rms_target", ctypes.c_float),
                ("clip", ctypes.c_void_p)]


class AdamWHParamsC(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("clip", ctypes.c_void_p)]


class MuonClipState(ctypes.Structure):
    """Host view of muon_clip_state_t (the device copy lives in a 16-byte tensor)."""
    _fields_ = [("norm", ctypes.c_float), ("scale", ctypes.c_float), ("skip", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class MuonGradBuffer(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("n", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class MuonStateStats(ctypes.Structure):
    """Host view of muon_state_stats_t."""
    _fields_ = [("mean", ctypes.c_double), ("var", ctypes.c_double), ("min", ctypes.c_double),
                ("max", ctypes.c_double), ("absmax", ctypes.c_double),
                ("count", ctypes.c_int64), ("nonfinite", ctypes.c_int64)]


class MuonClipTarget(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("ld", ctypes.c_int64), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("group", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class MuonPlanInfo(ctypes.Structure):
    _fields_ = [("n_mats", ctypes.c_int32), ("n_waves", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("ns_dtype", ctypes.c_int32),
                ("k1_tiles", ctypes.c_int64), ("syrk_tiles", ctypes.c_int64),
                ("bx_tiles", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
                ("ns_flops_per_iter_alg", ctypes.c_double), ("small_mats", ctypes.c_int32),
                ("split_tile_mats", ctypes.c_int32), ("fused_apply_mats", ctypes.c_int32),
                ("round_sync_phases", ctypes.c_int32)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libmuon.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m muon_newton_schulz_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    mats_p = ctypes.POINTER(MuonMatrix)
    L.muon_workspace_size.argtypes = [mats_p, I32, I64, I32, I32, I32, SZ, ctypes.POINTER(SZ)]
    L.muon_plan_create.argtypes = [mats_p, I32, I64, I32, I32, I32, SZ, ctypes.POINTER(P),
                                   ctypes.POINTER(SZ)]
    L.muon_plan_create_ex.argtypes = [mats_p, I32, I64, I32, I32, I32, SZ, ctypes.c_uint32,
                                      ctypes.POINTER(P), ctypes.POINTER(SZ)]
    L.muon_plan_destroy.argtypes = [P]
    L.muon_plan_destroy.restype = None
    L.muon_plan_get_info.argtypes = [P, ctypes.POINTER(MuonPlanInfo)]
    L.muon_plan_table_bytes.argtypes = [P]
    L.muon_plan_table_bytes.restype = SZ
    L.muon_plan_upload.argtypes = [P, P, SZ, P]
    hp_p = ctypes.POINTER(MuonHParamsC)
    L.muon_step.argtypes = [P, P, P, P, P, SZ, hp_p, P, P]
    L.muon_step_noalloc.argtypes = [P, P, P, P, hp_p, P, P]
    L.muon_stage_momentum.argtypes = [P, I32, P, P, P, SZ, hp_p, P]
    L.muon_stage_ns_phase.argtypes = [P, I32, P, SZ, hp_p, I32, I32, P]
    L.muon_stage_apply.argtypes = [P, I32, P, P, SZ, hp_p, P, P]
    L.muon_stage_ns_apply.argtypes = [P, I32, P, P, SZ, hp_p, P]
    L.muon_stage_export_x.argtypes = [P, I32, P, SZ, I32, P, P]
    L.muon_stage_export_norms.argtypes = [P, I32, P, SZ, P, P]
    L.adamw_step.argtypes = [P, I32, P, P, I32, P, P, I64, ctypes.POINTER(AdamWHParamsC), I64, P]
    L.adamw_step_ex.argtypes = [P, I32, P, P, I32, P, I32, P, I32, I64,
                                ctypes.POINTER(AdamWHParamsC), I64, P]
    L.grad_norm_clip_workspace_size.argtypes = [I32]
    L.grad_norm_clip_workspace_size.restype = SZ
    L.grad_norm_clip.argtypes = [ctypes.POINTER(MuonGradBuffer), I32, ctypes.c_float,
                                 ctypes.c_float, P, SZ, P, P]
    L.state_stats_workspace_size.argtypes = []
    L.state_stats_workspace_size.restype = SZ
    L.state_stats.argtypes = [P, I64, P, SZ, P, P]
    L.muon_clip_plan_create.argtypes = [ctypes.POINTER(MuonClipTarget), I32, I64, I32, I32,
                                        ctypes.POINTER(P), ctypes.POINTER(SZ)]
    L.muon_clip_plan_destroy.argtypes = [P]
    L.muon_clip_plan_destroy.restype = None
    L.muon_clip_plan_table_bytes.argtypes = [P]
    L.muon_clip_plan_table_bytes.restype = SZ
    L.muon_clip_plan_upload.argtypes = [P, P, SZ, P]
    L.muon_clip.argtypes = [P, P, I32, ctypes.c_float, P, P, SZ, P, P, P]
    L.muon_status_string.argtypes = [I32]
    L.muon_status_string.restype = ctypes.c_char_p
    L.muon_last_error.argtypes = []
    L.muon_last_error.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name not in ("muon_plan_destroy", "muon_clip_plan_destroy", "muon_status_string",
                        "muon_last_error", "muon_plan_table_bytes", "muon_clip_plan_table_bytes",
                        "grad_norm_clip_workspace_size", "state_stats_workspace_size"):
            getattr(L, name).restype = ctypes.c_int
    _lib_handle = L
    return L


def _check(rc: int) -> None:
    if rc != MUON_OK:
        msg = lib().muon_last_error().decode(errors="replace")
        raise MuonError(rc, msg or muon_status_string(rc))


def muon_status_string(status: int) -> str:
    return lib().muon_status_string(status).decode()


def muon_last_error() -> str:
    return lib().muon_last_error().decode(errors="replace")


# ---------------------------------------------------------------- marshalling

def dtype_code(dt) -> int:
    import torch
    table = {"fp32": MUON_DTYPE_FP32, "bf16": MUON_DTYPE_BF16, "fp16": MUON_DTYPE_FP16,
             torch.float32: MUON_DTYPE_FP32, torch.bfloat16: MUON_DTYPE_BF16,
             torch.float16: MUON_DTYPE_FP16}
    if dt not in table:
        raise MuonError(MUON_ERR_BAD_DTYPE, f"unsupported dtype {dt}")
    return table[dt]


def _mats_array(mats: Sequence[Tuple[int, int, int]]):
    arr = (MuonMatrix * max(1, len(mats)))()
    for k, (o, r, c) in enumerate(mats):
        arr[k] = MuonMatrix(int(o), int(r), int(c))
    return arr


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _buf(t, name: str, min_numel: int = 0, dtypes=None, optional: bool = False):
    """Checks a tensor before its address crosses the C ABI, which cannot
    see sizes: a GPU tensor, contiguous, with at least ``min_numel``
    elements of an allowed dtype.  Returns it."""
    if t is None:
        if optional:
            return None
        raise MuonError(MUON_ERR_INVALID_ARG, f"{name} is None")
    if not getattr(t, "is_cuda", False):
        raise MuonError(MUON_ERR_INVALID_ARG, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise MuonError(MUON_ERR_INVALID_ARG, f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise MuonError(MUON_ERR_INVALID_ARG,
                        f"{name} has {t.numel()} elements, needs at least {min_numel}")
    if dtypes is not None and dtype_code(t.dtype) not in dtypes:
        raise MuonError(MUON_ERR_BAD_DTYPE, f"{name} has dtype {t.dtype}")
    return t


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _hp(hp, clip=None) -> MuonHParamsC:
    if isinstance(hp, MuonHParamsC):
        h = MuonHParamsC.from_buffer_copy(hp)
    else:
        h = MuonHParamsC(float(hp.lr), float(hp.weight_decay), float(hp.momentum),
                         int(bool(hp.nesterov)), float(hp.ns_a), float(hp.ns_b),
                         float(hp.ns_c), int(hp.ns_steps), float(hp.eps), int(hp.scale_mode),
                         float(hp.rms_target))
    if clip is not None:
        h.clip = _ptr(clip)
    return h


def _ahp(hp, clip=None) -> AdamWHParamsC:
    if isinstance(hp, AdamWHParamsC):
        h = AdamWHParamsC.from_buffer_copy(hp)
    else:
        h = AdamWHParamsC(float(hp.lr), float(hp.beta1), float(hp.beta2), float(hp.eps),
                          float(hp.weight_decay))
    if clip is not None:
        h.clip = _ptr(clip)
    return h


# ---------------------------------------------------------------- plan

class MuonPlan:
    """Owns a muon_plan_t (destroyed with the object) and, once uploaded, the
    device tensor holding its tables."""

    def __init__(self, handle: int, workspace_bytes: int, n_mats: int, flat_numel: int = 0,
                 param_dtype: int = MUON_DTYPE_BF16, grad_dtype: int = MUON_DTYPE_BF16):
        self.handle = handle
        self.workspace_bytes = workspace_bytes
        self.n_mats = n_mats
        self.flat_numel = flat_numel
        self.param_dtype = param_dtype
        self.grad_dtype = grad_dtype
        self.tables = None

    @property
    def table_bytes(self) -> int:
        return muon_plan_table_bytes(self)

    def upload(self, device=None, stream=None) -> None:
        """Allocate the table buffer on ``device`` (torch's current device if
        None) and copy the tables into it on ``stream`` (current stream)."""
        import torch
        dev = torch.device("cuda") if device is None else torch.device(device)
        tables = torch.empty(max(1, self.table_bytes), dtype=torch.uint8, device=dev)
        with torch.cuda.device(tables.device):
            muon_plan_upload(self, tables, stream)
        self.tables = tables

    def info(self) -> MuonPlanInfo:
        return muon_plan_get_info(self)

    def alloc_workspace(self, device="cuda"):
        import torch
        return torch.empty(max(1, self.workspace_bytes), dtype=torch.uint8, device=device)

    def close(self):
        if self.handle:
            lib().muon_plan_destroy(ctypes.c_void_p(self.handle))
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def muon_workspace_size(mats, flat_numel: int, param_dtype, grad_dtype, ns_dtype,
                        workspace_cap: int = 0) -> int:
    arr = _mats_array(mats)
    out = ctypes.c_size_t(0)
    _check(lib().muon_workspace_size(arr, len(mats), int(flat_numel), dtype_code(param_dtype),
                                     dtype_code(grad_dtype), dtype_code(ns_dtype),
                                     int(workspace_cap), ctypes.byref(out)))
    return out.value


MUON_PLAN_TILED_ONLY = 1
MUON_PLAN_WHOLE_TILES = 2
MUON_PLAN_FREE_ROUNDS = 4


def muon_plan_create(mats, flat_numel: int, param_dtype, grad_dtype, ns_dtype="bf16",
                     workspace_cap: int = 0, tiled_only: bool = False,
                     whole_tiles: bool = False, free_rounds: bool = False,
                     upload: bool = True) -> MuonPlan:
    """tiled_only: every matrix on the tiled NS path (no fused small-matrix
    kernel); whole_tiles: every NS tile computed whole (no split diagonal
    or edge tiles); free_rounds: the NS kernels never hold an XCD's tile
    rounds together.  Results are bitwise the same either way.
    upload: copy the tables to a new device tensor on torch's current device
    and stream (MuonPlan.upload); without it the plan stays host-only."""
    arr = _mats_array(mats)
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)
    _check(lib().muon_plan_create_ex(arr, len(mats), int(flat_numel), dtype_code(param_dtype),
                                     dtype_code(grad_dtype), dtype_code(ns_dtype),
                                     int(workspace_cap),
                                     (MUON_PLAN_TILED_ONLY if tiled_only else 0)
                                     | (MUON_PLAN_WHOLE_TILES if whole_tiles else 0)
                                     | (MUON_PLAN_FREE_ROUNDS if free_rounds else 0),
                                     ctypes.byref(h), ctypes.byref(ws)))
    plan = MuonPlan(h.value, ws.value, len(mats), int(flat_numel), dtype_code(param_dtype),
                    dtype_code(grad_dtype))
    if upload:
        plan.upload()
    return plan


def muon_plan_destroy(plan: MuonPlan) -> None:
    plan.close()


def muon_plan_table_bytes(plan: MuonPlan) -> int:
    return int(lib().muon_plan_table_bytes(ctypes.c_void_p(plan.handle)))


def muon_plan_upload(plan: MuonPlan, tables, stream=None) -> None:
    """tables: a uint8 GPU tensor of at least muon_plan_table_bytes bytes,
    kept alive by the caller while the plan is used (MuonPlan.upload keeps
    it on the plan)."""
    _buf(tables, "tables", muon_plan_table_bytes(plan))
    _check(lib().muon_plan_upload(ctypes.c_void_p(plan.handle), _ptr(tables), _nbytes(tables),
                                  _stream(stream)))


def muon_plan_get_info(plan: MuonPlan) -> MuonPlanInfo:
    info = MuonPlanInfo()
    _check(lib().muon_plan_get_info(ctypes.c_void_p(plan.handle), ctypes.byref(info)))
    return info


F32 = (MUON_DTYPE_FP32,)


def _flat_args(plan: MuonPlan, params=None, grads=None, momentum=None, out_update=None):
    n = plan.flat_numel
    if params is not None:
        _buf(params, "params", n, (plan.param_dtype,))
    if grads is not None:
        _buf(grads, "grads", n, (plan.grad_dtype,))
    if momentum is not None:
        _buf(momentum, "momentum", n, F32)
    _buf(out_update, "out_update", n, F32, optional=True)


def muon_step(plan: MuonPlan, params, grads, momentum, workspace, hp, out_update=None,
              stream=None, clip=None) -> None:
    """clip: optional device clip state from grad_norm_clip (scale and guard)."""
    _flat_args(plan, _buf(params, "params"), _buf(grads, "grads"), _buf(momentum, "momentum"),
               out_update)
    _buf(workspace, "workspace")
    h = _hp(hp, clip)
    _check(lib().muon_step(ctypes.c_void_p(plan.handle), _ptr(params), _ptr(grads),
                           _ptr(momentum), _ptr(workspace), _nbytes(workspace), ctypes.byref(h),
                           _ptr(out_update), _stream(stream)))


def muon_step_noalloc(plan: MuonPlan, params, grads, momentum, hp, out_update=None,
                      stream=None, clip=None) -> None:
    """muon_step on the library's static device workspace (no workspace
    argument, nothing allocated); the plan's workspace_bytes must be at most
    MUON_NOALLOC_WORKSPACE_BYTES (create it with that workspace_cap)."""
    _flat_args(plan, _buf(params, "params"), _buf(grads, "grads"), _buf(momentum, "momentum"),
               out_update)
    h = _hp(hp, clip)
    _check(lib().muon_step_noalloc(ctypes.c_void_p(plan.handle), _ptr(params), _ptr(grads),
                                   _ptr(momentum), ctypes.byref(h), _ptr(out_update),
                                   _stream(stream)))


def muon_stage_momentum(plan: MuonPlan, wave: int, grads, momentum, workspace, hp,
                        stream=None, clip=None) -> None:
    _flat_args(plan, grads=_buf(grads, "grads"), momentum=_buf(momentum, "momentum"))
    _buf(workspace, "workspace")
    h = _hp(hp, clip)
    _check(lib().muon_stage_momentum(ctypes.c_void_p(plan.handle), wave, _ptr(grads),
                                     _ptr(momentum), _ptr(workspace), _nbytes(workspace),
                                     ctypes.byref(h), _stream(stream)))


def muon_stage_ns_phase(plan: MuonPlan, wave: int, workspace, hp, iter: int, phase: int,
                        stream=None) -> None:
    _buf(workspace, "workspace")
    h = _hp(hp)
    _check(lib().muon_stage_ns_phase(ctypes.c_void_p(plan.handle), wave, _ptr(workspace),
                                     _nbytes(workspace), ctypes.byref(h), iter, phase,
                                     _stream(stream)))


def muon_stage_apply(plan: MuonPlan, wave: int, params, workspace, hp, out_update=None,
                     stream=None, clip=None) -> None:
    _flat_args(plan, params=_buf(params, "params"), out_update=out_update)
    _buf(workspace, "workspace")
    h = _hp(hp, clip)
    _check(lib().muon_stage_apply(ctypes.c_void_p(plan.handle), wave, _ptr(params),
                                  _ptr(workspace), _nbytes(workspace), ctypes.byref(h),
                                  _ptr(out_update), _stream(stream)))


def muon_stage_ns_apply(plan: MuonPlan, wave: int, params, workspace, hp, stream=None,
                        clip=None) -> None:
    """Phase 3 of the last NS iteration with the update applied: bitwise
    muon_stage_ns_phase(..., ns_steps - 1, 3) then muon_stage_apply(...)."""
    _flat_args(plan, params=_buf(params, "params"))
    _buf(workspace, "workspace")
    h = _hp(hp, clip)
    _check(lib().muon_stage_ns_apply(ctypes.c_void_p(plan.handle), wave, _ptr(params),
                                     _ptr(workspace), _nbytes(workspace), ctypes.byref(h),
                                     _stream(stream)))


def muon_stage_export_x(plan: MuonPlan, wave: int, workspace, iter_done: int, out,
                        stream=None) -> None:
    """out: fp32, flat_numel elements (the wave's matrices at their offsets)."""
    _buf(workspace, "workspace")
    _buf(out, "out", plan.flat_numel, F32)
    _check(lib().muon_stage_export_x(ctypes.c_void_p(plan.handle), wave, _ptr(workspace),
                                     _nbytes(workspace), iter_done, _ptr(out), _stream(stream)))


def muon_stage_export_norms(plan: MuonPlan, wave: int, workspace, out, stream=None) -> None:
    """out: fp32, at least as many elements as the wave has matrices."""
    _buf(workspace, "workspace")
    _buf(out, "out", 1 if plan.n_mats else 0, F32)
    _check(lib().muon_stage_export_norms(ctypes.c_void_p(plan.handle), wave, _ptr(workspace),
                                         _nbytes(workspace), _ptr(out), _stream(stream)))


def adamw_step(params, master, grads, exp_avg, exp_avg_sq, hp, step: int, stream=None,
               clip=None) -> None:
    """params/grads may be bf16 or fp32 tensors; master (fp32) may be None;
    exp_avg may be fp32 or bf16 and exp_avg_sq fp32, bf16 or fp16 (the
    compressed states of adamw_step_ex); clip: optional device clip state
    from grad_norm_clip."""
    n = _buf(params, "params").numel()
    for name, t in (("grads", grads), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq),
                    ("master", master)):
        _buf(t, name, optional=name == "master")
        if t is not None and t.numel() != n:
            raise MuonError(MUON_ERR_INVALID_ARG, f"{name} has {t.numel()} elements, expected {n}")
    h = _ahp(hp, clip)
    _check(lib().adamw_step_ex(_ptr(params), dtype_code(params.dtype), _ptr(master), _ptr(grads),
                               dtype_code(grads.dtype), _ptr(exp_avg), dtype_code(exp_avg.dtype),
                               _ptr(exp_avg_sq), dtype_code(exp_avg_sq.dtype), n,
                               ctypes.byref(h), int(step), _stream(stream)))


# ------------------------------------------ clipping, step guard, statistics

def grad_norm_clip_workspace_size(n_bufs: int) -> int:
    return int(lib().grad_norm_clip_workspace_size(int(n_bufs)))


def grad_norm_clip(grads: Sequence, max_norm: float, eps: float = 1e-6, out=None,
                   workspace=None, stream=None):
    """Global gradient norm over the given tensors, clip scale and skip flag,
    written to ``out`` (a 16-byte device tensor, allocated if None) and
    returned; pass it as ``clip=`` to the steps of the same iteration."""
    import torch
    bufs = (MuonGradBuffer * max(1, len(grads)))()
    dev = None
    for k, g in enumerate(grads):
        _buf(g, f"grads[{k}]")
        dev = g.device
    dev = dev if dev is not None else torch.device("cuda")
    if out is None:
        out = torch.zeros(16, dtype=torch.uint8, device=dev)
    if _nbytes(_buf(out, "out")) < ctypes.sizeof(MuonClipState):
        raise MuonError(MUON_ERR_INVALID_ARG, "out: 16 bytes of device memory")
    need = grad_norm_clip_workspace_size(len(grads))
    if workspace is None:
        workspace = torch.empty(max(8, need), dtype=torch.uint8, device=dev)
    _buf(workspace, "workspace")
    for k, g in enumerate(grads):
        bufs[k] = MuonGradBuffer(_ptr(g), int(g.numel()), dtype_code(g.dtype), 0)
    _check(lib().grad_norm_clip(bufs, len(grads), float(max_norm), float(eps),
                                _ptr(workspace), _nbytes(workspace), _ptr(out),
                                _stream(stream)))
    return out


def read_clip_state(out) -> dict:
    """Copy a device clip state to the host (synchronises)."""
    c = MuonClipState.from_buffer_copy(bytes(out.cpu().numpy().tobytes()))
    return {"norm": c.norm, "scale": c.scale, "skip": bool(c.skip)}


def state_stats_workspace_size() -> int:
    return int(lib().state_stats_workspace_size())


def state_stats(x, out=None, workspace=None, stream=None):
    """Statistics of a fp32 state tensor into ``out`` (a 56-byte device
    tensor, allocated if None), returned."""
    import torch
    _buf(x, "x", dtypes=F32)
    if out is None:
        out = torch.zeros(ctypes.sizeof(MuonStateStats), dtype=torch.uint8, device=x.device)
    if _nbytes(_buf(out, "out")) < ctypes.sizeof(MuonStateStats):
        raise MuonError(MUON_ERR_INVALID_ARG, "out: 56 bytes of device memory")
    if workspace is None:
        workspace = torch.empty(state_stats_workspace_size(), dtype=torch.uint8, device=x.device)
    _check(lib().state_stats(_ptr(x), int(x.numel()), _ptr(_buf(workspace, "workspace")),
                             _nbytes(workspace), _ptr(out), _stream(stream)))
    return out


def read_state_stats(out) -> dict:
    """Copy device statistics to the host (synchronises)."""
    s = MuonStateStats.from_buffer_copy(bytes(out.cpu().numpy().tobytes()))
    return {k: getattr(s, k) for k, _ in MuonStateStats._fields_}


# ---------------------------------------------------------------- MuonClip

class MuonClipPlan:
    """Owns a muon_clip_plan_t (destroyed with the object) and, once uploaded,
    the device tensor holding its tables."""

    def __init__(self, handle: int, workspace_bytes: int, n_targets: int, n_groups: int,
                 flat_numel: int, param_dtype: int):
        self.handle = handle
        self.workspace_bytes = workspace_bytes
        self.n_targets = n_targets
        self.n_groups = n_groups
        self.flat_numel = flat_numel
        self.param_dtype = param_dtype
        self.tables = None

    def upload(self, device=None, stream=None) -> None:
        import torch
        dev = torch.device("cuda") if device is None else torch.device(device)
        nb = int(lib().muon_clip_plan_table_bytes(ctypes.c_void_p(self.handle)))
        tables = torch.empty(max(1, nb), dtype=torch.uint8, device=dev)
        with torch.cuda.device(tables.device):
            _check(lib().muon_clip_plan_upload(ctypes.c_void_p(self.handle), _ptr(tables),
                                               _nbytes(tables), _stream(stream)))
        self.tables = tables

    def alloc_workspace(self, device="cuda"):
        import torch
        return torch.empty(max(8, self.workspace_bytes), dtype=torch.uint8, device=device)

    def close(self):
        if self.handle:
            lib().muon_clip_plan_destroy(ctypes.c_void_p(self.handle))
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def muon_clip_plan_create(targets, flat_numel: int, param_dtype, n_groups: int = 0,
                          upload: bool = True) -> MuonClipPlan:
    """targets: (offset, rows, cols[, ld[, group]]) per block (ld defaults
    to cols, group to 0).  upload: copy the tables to a new device tensor on
    torch's current device and stream."""
    arr = (MuonClipTarget * max(1, len(targets)))()
    for i, t in enumerate(targets):
        off, rows, cols = int(t[0]), int(t[1]), int(t[2])
        ld = int(t[3]) if len(t) > 3 else cols
        group = int(t[4]) if len(t) > 4 else 0
        arr[i] = MuonClipTarget(off, ld, rows, cols, group, 0)
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)
    pd = dtype_code(param_dtype)
    _check(lib().muon_clip_plan_create(arr, len(targets), int(flat_numel), pd, int(n_groups),
                                       ctypes.byref(h), ctypes.byref(ws)))
    plan = MuonClipPlan(h.value, ws.value, len(targets), int(n_groups), int(flat_numel), pd)
    if upload:
        plan.upload()
    return plan


def muon_clip(plan: MuonClipPlan, params, mode, tau: float, max_logits=None, workspace=None,
              norms_out=None, scales_out=None, stream=None) -> None:
    """MuonClip in place on ``params`` (the flat buffer the plan describes).
    mode: "frobenius" / MUON_CLIP_FROBENIUS or "max_logit" / MUON_CLIP_MAX_LOGIT."""
    m = {"frobenius": MUON_CLIP_FROBENIUS, "max_logit": MUON_CLIP_MAX_LOGIT}.get(mode, mode)
    _buf(params, "params", plan.flat_numel, (plan.param_dtype,))
    if m == MUON_CLIP_MAX_LOGIT:
        _buf(max_logits, "max_logits", plan.n_groups, F32)
    _buf(norms_out, "norms_out", plan.n_targets, F32, optional=True)
    _buf(scales_out, "scales_out", plan.n_targets, F32, optional=True)
    if workspace is None and m == MUON_CLIP_FROBENIUS:
        workspace = plan.alloc_workspace(params.device)
    _buf(workspace, "workspace", optional=True)
    _check(lib().muon_clip(ctypes.c_void_p(plan.handle), _ptr(params), int(m), float(tau),
                           _ptr(max_logits), _ptr(workspace),
                           _nbytes(workspace) if workspace is not None else 0,
                           _ptr(norms_out), _ptr(scales_out), _stream(stream)))
