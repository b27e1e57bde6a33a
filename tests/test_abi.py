"""The C ABI on the CPU: the library loads, exports what the header declares,
the ctypes struct matches the C layout, and every argument check returns its
documented status before anything reaches the HIP runtime (no GPU needed).
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from reverse_mamba_selective_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "r2l_scan.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_functions():
    names = set()
    for h in HEADERS:
        names |= set(re.findall(r"^R2L_API\s+(?:r2l_status|const char \*|int32_t)\s*\**\s*(\w+)\s*\(",
                                open(h).read(), re.M))
    return sorted(names)


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(_abi.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    lib = _abi.load()
    for f in declared_functions():
        assert hasattr(lib, f)


def test_abi_version_and_status_strings():
    lib = _abi.load()
    assert lib.r2l_abi_version() == _abi.ABI_VERSION
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert _abi.status_string(code) and _abi.status_string(code) != "unknown status"
    assert _abi.status_string(-99) == "unknown status"


@pytest.mark.parametrize("cls,cname", [(_abi.ScanArgs, "r2l_scan_args"),
                                        (_abi.GradArgs, "r2l_grad_args"),
                                        (_abi.DirArgs, "r2l_dir_args"),
                                        (_abi.SidecarArgs, "r2l_sidecar_args"),
                                        (_abi.AccessReport, "r2l_access_report"),
                                        (_abi.PlanInfo, "r2l_plan_info")])
def test_struct_layout_matches_c(cls, cname):
    fields = [f[0] for f in cls._fields_]
    prog = ["#include <stddef.h>", "#include <stdio.h>", '#include "r2l_scan_debug.h"',
            "int main(void){", 'printf("%%zu\\n", sizeof(%s));' % cname]
    prog += ['printf("%%zu\\n", offsetof(%s, %s));' % (cname, f) for f in fields]
    prog += ["return 0;}"]
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "layout.c")
        open(src, "w").write("\n".join(prog))
        exe = os.path.join(d, "layout")
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        vals = [int(v) for v in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(cls)
    for f, off in zip(fields, vals[1:]):
        assert getattr(cls, f).offset == off, f


# ---- argument checks (fake device addresses: nothing is ever launched) ------

BASE = 0x7F0000000000  # plausible, 4 KiB aligned, never dereferenced on the host


def good_args(**over):
    """A valid-looking dense bf16 call; tests break exactly one thing."""
    D, N, B, L = 256, 16, 2, 8
    a = _abi.ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate, a.dtype = B, L, D, N, _abi.R2L_DTYPE_BF16
    a.delta_softplus = 1
    nxt = [BASE]

    def region(nbytes):
        p = nxt[0]
        nxt[0] += (nbytes + 4095) // 4096 * 4096 + 4096
        return p

    rows = B * L
    a.x, a.x_stride = region(rows * D * 2), D
    a.dt, a.dt_stride = region(rows * D * 2), D
    a.Bm, a.Bm_stride = region(rows * N * 2), N
    a.Cm, a.Cm_stride = region(rows * N * 2), N
    a.A = region(D * N * 4)
    a.Dskip = region(D * 4)
    a.out, a.out_stride = region(rows * D * 2), D
    a.chunk_tokens = -1
    for k, v in over.items():
        setattr(a, k, v)
    return a


def status(func, a):
    lib = _abi.load()
    return getattr(lib, func)(ctypes.byref(a), None)


def test_null_args_pointer():
    assert _abi.load().r2l_scan(None, None) == _abi.R2L_ERR_INVALID_ARG


@pytest.mark.parametrize("field,value,code", [
    ("batch", -1, _abi.R2L_ERR_INVALID_ARG),
    ("dim", 0, _abi.R2L_ERR_INVALID_ARG),
    ("seqlen", -3, _abi.R2L_ERR_INVALID_ARG),
    ("dstate", 8, _abi.R2L_ERR_UNSUPPORTED),
    ("dstate", 0, _abi.R2L_ERR_UNSUPPORTED),
    ("dtype", 7, _abi.R2L_ERR_UNSUPPORTED),
    ("delta_softplus", 2, _abi.R2L_ERR_INVALID_ARG),
    ("state_split", 3, _abi.R2L_ERR_INVALID_ARG),
    ("x", None, _abi.R2L_ERR_INVALID_ARG),
    ("dt", None, _abi.R2L_ERR_INVALID_ARG),
    ("Bm", None, _abi.R2L_ERR_INVALID_ARG),
    ("Cm", None, _abi.R2L_ERR_INVALID_ARG),
    ("A", None, _abi.R2L_ERR_INVALID_ARG),
    ("out", None, _abi.R2L_ERR_INVALID_ARG),
    ("x_stride", 100, _abi.R2L_ERR_INVALID_ARG),
    ("Bm_stride", 15, _abi.R2L_ERR_INVALID_ARG),
    ("x", BASE + 1, _abi.R2L_ERR_MISALIGNED),
    ("A", BASE + 8 * 4096 * 40 + 4, _abi.R2L_ERR_MISALIGNED),
    ("h_in", BASE + 0x1000000 + 8, _abi.R2L_ERR_MISALIGNED),
    ("Dskip", BASE + 0x1000000 + 2, _abi.R2L_ERR_MISALIGNED),
])
def test_scan_argument_checks(field, value, code):
    a = good_args(**{field: value})
    assert status("r2l_scan", a) == code
    assert _abi.last_error() != ""


def test_alias_rules():
    a = good_args()
    # out exactly x (in-place hook) and exactly res are allowed by the checks;
    # they are not launched here. Partial overlaps are refused.
    a.out = a.x + 2
    assert status("r2l_scan", a) == _abi.R2L_ERR_ALIAS
    a = good_args()
    a.out = a.dt
    assert status("r2l_scan", a) == _abi.R2L_ERR_ALIAS
    a = good_args()
    a.res, a.res_stride = a.out + 64, a.out_stride
    assert status("r2l_scan", a) == _abi.R2L_ERR_ALIAS
    a = good_args()
    a.out, a.out_stride = a.x, a.x_stride + 2  # same base, other stride: not an exact alias
    a.x_stride = 256
    assert status("r2l_scan", a) == _abi.R2L_ERR_ALIAS
    a = good_args(h_out=BASE + 0x2000000)
    a.h_in = a.h_out + 64
    assert status("r2l_scan", a) == _abi.R2L_ERR_ALIAS
    a = good_args(h_out=BASE + 0x2000000)
    a.h_out = a.A
    assert status("r2l_scan", a) == _abi.R2L_ERR_ALIAS


def test_prefix_needs_an_output_and_commit_needs_the_state():
    a = good_args(out=None, Cm=None)
    assert status("prefix_scan_state", a) == _abi.R2L_ERR_INVALID_ARG
    assert "h_out or out" in _abi.last_error()
    a = good_args(out=None, Cm=None)
    assert status("block_commit_state", a) == _abi.R2L_ERR_INVALID_ARG
    a = good_args(out=None, Cm=None, h_out=BASE + 0x2000000, h_in=BASE + 0x3000000)
    assert status("block_commit_state", a) == _abi.R2L_ERR_INVALID_ARG


def test_ragged_shape_checks():
    a = good_args(cu_seqlens=BASE + 0x4000000, total_tokens=-1, max_seqlen=4)
    assert status("r2l_scan", a) == _abi.R2L_ERR_INVALID_ARG
    a = good_args(cu_seqlens=BASE + 0x4000000, total_tokens=16, max_seqlen=17)
    assert status("r2l_scan", a) == _abi.R2L_ERR_INVALID_ARG
    a = good_args(cu_seqlens=BASE + 0x4000002, total_tokens=16, max_seqlen=8)
    assert status("r2l_scan", a) == _abi.R2L_ERR_MISALIGNED


def test_workspace_rules():
    # a long state-only prefix is chunked and needs workspace
    a = good_args(out=None, Cm=None, h_out=BASE + 0x2000000, chunk_tokens=0, batch=1,
                  seqlen=100000)
    need = _abi.workspace_size(_abi.R2L_OP_PREFIX, a)
    assert need > 0
    assert status("prefix_scan_state", a) == _abi.R2L_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = BASE + 0x5000000 + 128, need
    assert status("prefix_scan_state", a) == _abi.R2L_ERR_MISALIGNED
    a.workspace, a.workspace_bytes = BASE + 0x5000000, need - 1
    assert status("prefix_scan_state", a) == _abi.R2L_ERR_WORKSPACE
    # forcing no chunking needs none; the serving shapes need none
    a.chunk_tokens = -1
    assert _abi.workspace_size(_abi.R2L_OP_PREFIX, a) == 0
    serve = good_args(batch=64, seqlen=32, dim=2048, chunk_tokens=0)
    assert _abi.workspace_size(_abi.R2L_OP_SCAN, serve) == 0
    # a forced chunk length gives Q, S and the per-chunk entry states
    f = good_args(batch=2, seqlen=100, dim=64, chunk_tokens=32)
    q = 2 * 4 * 64 * 16 * 4
    s = 2 * 4 * 64 * 4
    assert _abi.workspace_size(_abi.R2L_OP_SCAN, f) == q + ((s + 255) // 256 * 256) + q
    assert _abi.workspace_size(_abi.R2L_OP_COMMIT, good_args(batch=2, seqlen=100, dim=64,
                                                             chunk_tokens=32, out=None)) \
        == q + ((s + 255) // 256 * 256)


def test_bad_workspace_query():
    lib = _abi.load()
    n = ctypes.c_size_t(0)
    assert lib.r2l_workspace_size(9, ctypes.byref(good_args()), ctypes.byref(n)) \
        == _abi.R2L_ERR_INVALID_ARG
    assert lib.r2l_workspace_size(0, ctypes.byref(good_args()), None) == _abi.R2L_ERR_INVALID_ARG


def test_noalloc_checks_and_scratch_limit():
    """r2l_scan_noalloc: the header's scratch size is the binding's; the same
    argument checks as r2l_scan; a plan needing more scratch than the array
    holds is refused with R2L_ERR_WORKSPACE before anything is launched."""
    m = re.search(r"#define R2L_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == _abi.NOALLOC_SCRATCH_BYTES
    for field, value, code in [("x", None, _abi.R2L_ERR_INVALID_ARG),
                               ("dstate", 8, _abi.R2L_ERR_UNSUPPORTED),
                               ("x", BASE + 1, _abi.R2L_ERR_MISALIGNED),
                               ("Bm_stride", 15, _abi.R2L_ERR_INVALID_ARG)]:
        assert status("r2l_scan_noalloc", good_args(**{field: value})) == code
    a = good_args(batch=1, seqlen=300000, dim=512, chunk_tokens=256)
    a.x, a.dt, a.Bm, a.Cm, a.A, a.Dskip, a.out = (BASE + (i << 32) for i in range(1, 8))
    a.x_stride = a.dt_stride = a.out_stride = 512
    need = _abi.workspace_size(_abi.R2L_OP_SCAN, a)
    assert need > _abi.NOALLOC_SCRATCH_BYTES
    assert status("r2l_scan_noalloc", a) == _abi.R2L_ERR_WORKSPACE
    assert "scratch" in _abi.last_error()


def test_gemm_context_create_destroy_and_misuse():
    """The sidecar's GEMM context is the caller's: create / destroy through the
    ABI, and every misuse refused with a status (no device needed)."""
    import torch
    from test_access_bounds import make_sidecar
    lib = _abi.load()
    assert lib.r2l_gemm_context_create(None) == _abi.R2L_ERR_INVALID_ARG
    assert lib.r2l_gemm_context_destroy(None) == _abi.R2L_ERR_INVALID_ARG
    # a host buffer that is not a context (zeros): refused, not freed
    junk = (ctypes.c_uint8 * 256)()
    assert lib.r2l_gemm_context_destroy(ctypes.addressof(junk)) == _abi.R2L_ERR_INVALID_ARG
    h = ctypes.c_void_p(0)
    st = lib.r2l_gemm_context_create(ctypes.byref(h))
    if torch.cuda.is_available():
        assert st == _abi.R2L_OK and h.value
        assert lib.r2l_gemm_context_destroy(h) == _abi.R2L_OK
    else:
        assert st == _abi.R2L_ERR_HIP and not h.value, (st, _abi.last_error())
    # a sidecar call that runs needs a live context: NULL and junk are refused
    # by the argument checks, before anything reaches HIP
    a, _ = make_sidecar(batch=2, seqlen=16)
    a.gemm = None
    assert lib.r2l_sidecar_forward(ctypes.byref(a), None) == _abi.R2L_ERR_INVALID_ARG
    assert lib.r2l_sidecar_tune(ctypes.byref(a), None) == _abi.R2L_ERR_INVALID_ARG
    a.gemm = ctypes.addressof(junk)
    assert lib.r2l_sidecar_forward(ctypes.byref(a), None) == _abi.R2L_ERR_INVALID_ARG
    assert "not a live GEMM context" in _abi.last_error()
