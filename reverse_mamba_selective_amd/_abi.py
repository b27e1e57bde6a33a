"""ctypes view of include/r2l_scan.h (argument marshalling only).

Loading fails loudly when libr2l_scan.so has not been built: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# R2L_LIB_PATH: another build of the library (the host-sanitized one of build.py --sanitize)
LIB_PATH = os.environ.get("R2L_LIB_PATH") or os.path.join(HERE, "libr2l_scan.so")

R2L_OK = 0
R2L_ERR_INVALID_ARG = -1
R2L_ERR_UNSUPPORTED = -2
R2L_ERR_ALIAS = -3
R2L_ERR_MISALIGNED = -4
R2L_ERR_WORKSPACE = -5
R2L_ERR_HIP = -6

R2L_DTYPE_F32 = 0
R2L_DTYPE_BF16 = 1

R2L_OP_SCAN = 0
R2L_OP_PREFIX = 1
R2L_OP_COMMIT = 2
R2L_OP_BIDIR = 3
R2L_OP_SAVE = 4
R2L_OP_PREFIX_SAVE = 5

ABI_VERSION = 8
NOALLOC_SCRATCH_BYTES = 64 << 20   # r2l_scan_noalloc's scratch array per device

EXPORTS = ("r2l_scan", "prefix_scan_state", "block_commit_state", "r2l_scan_noalloc",
           "r2l_workspace_size",
           "r2l_status_string", "r2l_last_error", "r2l_abi_version", "r2l_check_access",
           "r2l_describe_plan", "r2l_scan_backward", "r2l_backward_workspace_size",
           "r2l_check_access_backward", "prefix_scan_backward", "bidir_scan",
           "r2l_check_access_bidir", "r2l_sidecar_forward", "r2l_sidecar_workspace_size",
           "r2l_check_access_sidecar", "r2l_sidecar_tune", "r2l_gemm_context_create",
           "r2l_gemm_context_destroy", "r2l_scan_save", "r2l_checkpoint_size",
           "r2l_scan_backward_saved", "r2l_check_access_save", "r2l_check_access_backward_saved",
           "prefix_scan_save", "prefix_scan_backward_saved")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class ScanArgs(ctypes.Structure):
    """Mirror of ``r2l_scan_args`` (same field order, natural alignment)."""
    _fields_ = [
        ("batch", _i64), ("seqlen", _i64), ("cu_seqlens", _vp), ("total_tokens", _i64),
        ("max_seqlen", _i64), ("dim", _i64), ("dstate", _i32), ("dtype", _i32),
        ("x", _vp), ("x_stride", _i64), ("x_batch_stride", _i64),
        ("dt", _vp), ("dt_stride", _i64), ("dt_batch_stride", _i64),
        ("Bm", _vp), ("Bm_stride", _i64), ("Bm_batch_stride", _i64),
        ("Cm", _vp), ("Cm_stride", _i64), ("Cm_batch_stride", _i64),
        ("A", _vp), ("Dskip", _vp), ("delta_softplus", _i32),
        ("chunk_tokens", _i32), ("state_split", _i32),
        ("h_in", _vp), ("h_out", _vp),
        ("res", _vp), ("res_stride", _i64), ("res_batch_stride", _i64), ("s", ctypes.c_float),
        ("out", _vp), ("out_stride", _i64), ("out_batch_stride", _i64),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
    ]


class GradArgs(ctypes.Structure):
    """Mirror of ``r2l_grad_args``."""
    _fields_ = [
        ("dout", _vp), ("dout_stride", _i64), ("dout_batch_stride", _i64),
        ("dh_out", _vp),
        ("dx", _vp), ("dx_stride", _i64), ("dx_batch_stride", _i64),
        ("ddt", _vp), ("ddt_stride", _i64), ("ddt_batch_stride", _i64),
        ("dBm", _vp), ("dCm", _vp), ("dA", _vp), ("dDskip", _vp), ("dh_in", _vp), ("ds", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
    ]


class DirArgs(ctypes.Structure):
    """Mirror of ``r2l_dir_args`` (the reverse direction of bidir_scan)."""
    _fields_ = [
        ("dt", _vp), ("dt_stride", _i64), ("dt_batch_stride", _i64),
        ("Bm", _vp), ("Bm_stride", _i64), ("Bm_batch_stride", _i64),
        ("Cm", _vp), ("Cm_stride", _i64), ("Cm_batch_stride", _i64),
        ("A", _vp), ("Dskip", _vp),
    ]


class SidecarArgs(ctypes.Structure):
    """Mirror of ``r2l_sidecar_args``."""
    _fields_ = [
        ("batch", _i64), ("seqlen", _i64), ("cu_seqlens", _vp), ("total_tokens", _i64),
        ("max_seqlen", _i64), ("d_model", _i64), ("d_inner", _i64), ("dstate", _i32),
        ("dt_rank", _i32), ("d_conv", _i32), ("dtype", _i32),
        ("hidden", _vp), ("hidden_stride", _i64), ("W_in", _vp), ("conv_w", _vp), ("conv_b", _vp),
        ("W_x", _vp), ("W_dt", _vp), ("dt_bias", _vp), ("A", _vp), ("Dskip", _vp), ("W_out", _vp),
        ("s", ctypes.c_float), ("out", _vp), ("out_stride", _i64),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t), ("gemm", _vp),
    ]


class AccessReport(ctypes.Structure):
    """Mirror of ``r2l_access_report`` (include/r2l_scan_debug.h)."""
    _fields_ = [("launches", _i64), ("accesses", _i64), ("vector_staging", _i64),
                ("message", ctypes.c_char * 512)]


class PlanInfo(ctypes.Structure):
    """Mirror of ``r2l_plan_info`` (include/r2l_scan_debug.h)."""
    _fields_ = [("lanes_per_channel", _i32), ("chunked", _i32), ("chunk_tokens", _i64),
                ("chunks", _i64), ("workspace_bytes", _i64), ("launches", _i32)]


class R2LError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%d): %s" % (func, status_string(status), status, detail))


_lib = None


def load(path: str = LIB_PATH):
    """Load the library once; raises if it is missing or from another ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            "libr2l_scan.so is not built at %s; run `python -m reverse_mamba_selective_amd.build` "
            "(hipcc for gfx950). There is no fallback implementation." % path)
    lib = ctypes.CDLL(path)
    ptr = ctypes.POINTER(ScanArgs)
    for name in ("r2l_scan", "prefix_scan_state", "block_commit_state", "r2l_scan_noalloc"):
        f = getattr(lib, name)
        f.restype = _i32
        f.argtypes = [ptr, _vp]
    lib.r2l_workspace_size.restype = _i32
    lib.r2l_workspace_size.argtypes = [_i32, ptr, ctypes.POINTER(ctypes.c_size_t)]
    lib.r2l_status_string.restype = ctypes.c_char_p
    lib.r2l_status_string.argtypes = [_i32]
    lib.r2l_last_error.restype = ctypes.c_char_p
    lib.r2l_last_error.argtypes = []
    lib.r2l_abi_version.restype = _i32
    lib.r2l_abi_version.argtypes = []
    lib.r2l_describe_plan.restype = _i32
    lib.r2l_describe_plan.argtypes = [_i32, ptr, ctypes.POINTER(PlanInfo)]
    lib.r2l_check_access.restype = _i32
    lib.r2l_check_access.argtypes = [_i32, ptr, ctypes.POINTER(_i32), ctypes.POINTER(AccessReport)]
    gptr = ctypes.POINTER(GradArgs)
    for fn in (lib.r2l_scan_backward, lib.prefix_scan_backward):
        fn.restype = _i32
        fn.argtypes = [ptr, gptr, _vp]
    lib.r2l_backward_workspace_size.restype = _i32
    lib.r2l_backward_workspace_size.argtypes = [ptr, gptr, ctypes.POINTER(ctypes.c_size_t)]
    lib.r2l_check_access_backward.restype = _i32
    lib.r2l_check_access_backward.argtypes = [_i32, ptr, gptr, ctypes.POINTER(_i32),
                                              ctypes.POINTER(AccessReport)]
    fptr, szt = ctypes.POINTER(ctypes.c_float), ctypes.c_size_t
    for fn in (lib.r2l_scan_save, lib.prefix_scan_save):
        fn.restype = _i32
        fn.argtypes = [ptr, fptr, szt, _vp]
    lib.r2l_checkpoint_size.restype = _i32
    lib.r2l_checkpoint_size.argtypes = [ptr, ctypes.POINTER(szt)]
    for fn in (lib.r2l_scan_backward_saved, lib.prefix_scan_backward_saved):
        fn.restype = _i32
        fn.argtypes = [ptr, gptr, fptr, szt, _vp]
    lib.r2l_check_access_save.restype = _i32
    lib.r2l_check_access_save.argtypes = [_i32, ptr, fptr, szt, ctypes.POINTER(_i32),
                                          ctypes.POINTER(AccessReport)]
    lib.r2l_check_access_backward_saved.restype = _i32
    lib.r2l_check_access_backward_saved.argtypes = [_i32, ptr, gptr, fptr, szt,
                                                    ctypes.POINTER(_i32),
                                                    ctypes.POINTER(AccessReport)]
    dptr = ctypes.POINTER(DirArgs)
    lib.bidir_scan.restype = _i32
    lib.bidir_scan.argtypes = [ptr, dptr, _vp]
    lib.r2l_check_access_bidir.restype = _i32
    lib.r2l_check_access_bidir.argtypes = [ptr, dptr, ctypes.POINTER(_i32),
                                           ctypes.POINTER(AccessReport)]
    sptr = ctypes.POINTER(SidecarArgs)
    for fn in (lib.r2l_sidecar_forward, lib.r2l_sidecar_tune):
        fn.restype = _i32
        fn.argtypes = [sptr, _vp]
    lib.r2l_gemm_context_create.restype = _i32
    lib.r2l_gemm_context_create.argtypes = [ctypes.POINTER(_vp)]
    lib.r2l_gemm_context_destroy.restype = _i32
    lib.r2l_gemm_context_destroy.argtypes = [_vp]
    lib.r2l_sidecar_workspace_size.restype = _i32
    lib.r2l_sidecar_workspace_size.argtypes = [sptr, ctypes.POINTER(ctypes.c_size_t)]
    lib.r2l_check_access_sidecar.restype = _i32
    lib.r2l_check_access_sidecar.argtypes = [sptr, ctypes.POINTER(_i32), ctypes.POINTER(AccessReport)]
    if lib.r2l_abi_version() != ABI_VERSION:
        raise ImportError("libr2l_scan.so ABI %d, binding expects %d"
                          % (lib.r2l_abi_version(), ABI_VERSION))
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().r2l_status_string(status).decode()


def last_error() -> str:
    return load().r2l_last_error().decode()


def call(func: str, args: ScanArgs, stream: int | None) -> None:
    lib = load()
    st = getattr(lib, func)(ctypes.byref(args), _vp(stream or 0))
    if st != R2L_OK:
        raise R2LError(st, func, last_error())


def workspace_size(op: int, args: ScanArgs) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    st = lib.r2l_workspace_size(op, ctypes.byref(args), ctypes.byref(n))
    if st != R2L_OK:
        raise R2LError(st, "r2l_workspace_size", last_error())
    return int(n.value)


def check_access(op: int, args: ScanArgs, cu_seqlens_host=None):
    """Host replay of every access the call would make (no device touched).

    Returns (status, report); status 0 means every access is in bounds.
    ``cu_seqlens_host``: sequence of batch+1 ints for the ragged layout.
    """
    lib = load()
    rep = AccessReport()
    cu = None
    if cu_seqlens_host is not None:
        arr = (_i32 * len(cu_seqlens_host))(*[int(v) for v in cu_seqlens_host])
        cu = ctypes.cast(arr, ctypes.POINTER(_i32))
    st = lib.r2l_check_access(op, ctypes.byref(args), cu, ctypes.byref(rep))
    return st, rep


def backward_workspace_size(args: ScanArgs, grad: GradArgs) -> int:
    n = ctypes.c_size_t(0)
    st = load().r2l_backward_workspace_size(ctypes.byref(args), ctypes.byref(grad), ctypes.byref(n))
    if st != R2L_OK:
        raise R2LError(st, "r2l_backward_workspace_size", last_error())
    return int(n.value)


def call_backward(args: ScanArgs, grad: GradArgs, stream: int | None, reverse: bool = True) -> None:
    func = "r2l_scan_backward" if reverse else "prefix_scan_backward"
    st = getattr(load(), func)(ctypes.byref(args), ctypes.byref(grad), _vp(stream or 0))
    if st != R2L_OK:
        raise R2LError(st, func, last_error())


def check_access_backward(args: ScanArgs, grad: GradArgs, cu_seqlens_host=None, reverse=True):
    """Host replay of every access r2l_scan_backward (or, reverse=False,
    prefix_scan_backward) would make; (status, report)."""
    lib = load()
    rep = AccessReport()
    cu = None
    if cu_seqlens_host is not None:
        arr = (_i32 * len(cu_seqlens_host))(*[int(v) for v in cu_seqlens_host])
        cu = ctypes.cast(arr, ctypes.POINTER(_i32))
    st = lib.r2l_check_access_backward(1 if reverse else 0, ctypes.byref(args), ctypes.byref(grad),
                                       cu, ctypes.byref(rep))
    return st, rep


def _fptr(addr):
    return ctypes.cast(_vp(addr or 0), ctypes.POINTER(ctypes.c_float))


def _cu_ptr(cu_seqlens_host):
    if cu_seqlens_host is None:
        return None, None
    arr = (_i32 * len(cu_seqlens_host))(*[int(v) for v in cu_seqlens_host])
    return arr, ctypes.cast(arr, ctypes.POINTER(_i32))


def checkpoint_size(args: ScanArgs) -> int:
    n = ctypes.c_size_t(0)
    st = load().r2l_checkpoint_size(ctypes.byref(args), ctypes.byref(n))
    if st != R2L_OK:
        raise R2LError(st, "r2l_checkpoint_size", last_error())
    return int(n.value)


def call_save(args: ScanArgs, ckpt: int, ckpt_bytes: int, stream: int | None,
              reverse: bool = True) -> None:
    func = "r2l_scan_save" if reverse else "prefix_scan_save"
    st = getattr(load(), func)(ctypes.byref(args), _fptr(ckpt), ckpt_bytes, _vp(stream or 0))
    if st != R2L_OK:
        raise R2LError(st, func, last_error())


def call_backward_saved(args: ScanArgs, grad: GradArgs, ckpt: int, ckpt_bytes: int,
                        stream: int | None, reverse: bool = True) -> None:
    func = "r2l_scan_backward_saved" if reverse else "prefix_scan_backward_saved"
    st = getattr(load(), func)(ctypes.byref(args), ctypes.byref(grad), _fptr(ckpt), ckpt_bytes,
                               _vp(stream or 0))
    if st != R2L_OK:
        raise R2LError(st, func, last_error())


def check_access_save(args: ScanArgs, ckpt: int, ckpt_bytes: int, cu_seqlens_host=None,
                      reverse: bool = True):
    """Host replay of r2l_scan_save (prefix_scan_save); (status, report)."""
    rep = AccessReport()
    keep, cu = _cu_ptr(cu_seqlens_host)
    st = load().r2l_check_access_save(1 if reverse else 0, ctypes.byref(args), _fptr(ckpt),
                                      ckpt_bytes, cu, ctypes.byref(rep))
    return st, rep


def check_access_backward_saved(args: ScanArgs, grad: GradArgs, ckpt: int, ckpt_bytes: int,
                                cu_seqlens_host=None, reverse: bool = True):
    """Host replay of r2l_scan_backward_saved (prefix_scan_backward_saved);
    (status, report)."""
    rep = AccessReport()
    keep, cu = _cu_ptr(cu_seqlens_host)
    st = load().r2l_check_access_backward_saved(1 if reverse else 0, ctypes.byref(args),
                                                ctypes.byref(grad), _fptr(ckpt), ckpt_bytes, cu,
                                                ctypes.byref(rep))
    return st, rep


def _dir_ref(rev):
    return None if rev is None else ctypes.byref(rev)


def call_bidir(args: ScanArgs, rev: DirArgs | None, stream: int | None) -> None:
    st = load().bidir_scan(ctypes.byref(args), _dir_ref(rev), _vp(stream or 0))
    if st != R2L_OK:
        raise R2LError(st, "bidir_scan", last_error())


def check_access_bidir(args: ScanArgs, rev: DirArgs | None, cu_seqlens_host=None):
    """Host replay of every access bidir_scan would make; (status, report)."""
    lib = load()
    rep = AccessReport()
    cu = None
    if cu_seqlens_host is not None:
        arr = (_i32 * len(cu_seqlens_host))(*[int(v) for v in cu_seqlens_host])
        cu = ctypes.cast(arr, ctypes.POINTER(_i32))
    st = lib.r2l_check_access_bidir(ctypes.byref(args), _dir_ref(rev), cu, ctypes.byref(rep))
    return st, rep


def sidecar_workspace_size(args: SidecarArgs) -> int:
    n = ctypes.c_size_t(0)
    st = load().r2l_sidecar_workspace_size(ctypes.byref(args), ctypes.byref(n))
    if st != R2L_OK:
        raise R2LError(st, "r2l_sidecar_workspace_size", last_error())
    return int(n.value)


def call_sidecar(args: SidecarArgs, stream: int | None, tune: bool = False) -> None:
    func = "r2l_sidecar_tune" if tune else "r2l_sidecar_forward"
    st = getattr(load(), func)(ctypes.byref(args), _vp(stream or 0))
    if st != R2L_OK:
        raise R2LError(st, func, last_error())


def check_access_sidecar(args: SidecarArgs, cu_seqlens_host=None):
    """Host replay of r2l_sidecar_forward's accesses; (status, report)."""
    lib = load()
    rep = AccessReport()
    cu = None
    if cu_seqlens_host is not None:
        arr = (_i32 * len(cu_seqlens_host))(*[int(v) for v in cu_seqlens_host])
        cu = ctypes.cast(arr, ctypes.POINTER(_i32))
    st = lib.r2l_check_access_sidecar(ctypes.byref(args), cu, ctypes.byref(rep))
    return st, rep


def describe_plan(op: int, args: ScanArgs) -> dict:
    """The plan the library picks for this call (see r2l_describe_plan)."""
    info = PlanInfo()
    st = load().r2l_describe_plan(op, ctypes.byref(args), ctypes.byref(info))
    if st != R2L_OK:
        raise R2LError(st, "r2l_describe_plan", last_error())
    return {f: getattr(info, f) for f, _ in PlanInfo._fields_}


def gemm_context_create() -> int:
    """r2l_gemm_context_create on the current device; returns the handle."""
    h = _vp(0)
    st = load().r2l_gemm_context_create(ctypes.byref(h))
    if st != R2L_OK:
        raise R2LError(st, "r2l_gemm_context_create", last_error())
    return h.value


def gemm_context_destroy(handle: int) -> None:
    st = load().r2l_gemm_context_destroy(_vp(handle))
    if st != R2L_OK:
        raise R2LError(st, "r2l_gemm_context_destroy", last_error())
