"""Python binding of liblcma.so: half-precision GEMM (classic MFMA and LCMA / Strassen) on MI355X.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  Names follow the C ABI in ``include/lcma.h``; tensors are torch
device tensors (PyTorch provides device memory and streams, nothing else).

The library must have been built (``python complexity_half_precision_amd/build.py``
or ``__graft_entry__.build()``); importing fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# LCMA_LIBRARY may name another build of the same library (the host
# sanitizer build the CPU tests run against); the default is the in-tree one.
LIB_PATH = os.environ.get("LCMA_LIBRARY") or os.path.join(_HERE, "liblcma.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python {os.path.join(_HERE, 'build.py')}` "
        "(there is no fallback implementation)")

# torch first: its wheel carries its own HIP runtime, and the library must bind
# to that one.  Loaded before torch, the library would pull in the system HIP
# runtime as a second copy in the process, which then finds no device and
# cannot use torch's allocations.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------- constants (lcma.h)
F16, BF16 = 0, 1
ALGO_AUTO, ALGO_CLASSIC, ALGO_L1, ALGO_L2 = 0, 1, 2, 3
SPLIT_AUTO, SPLIT_NONE, SPLIT_ALL = 0, 1, 2
COMBINE_AUTO, COMBINE_PREPASS, COMBINE_AT_LOAD, COMBINE_UNFUSED, COMBINE_L2_ON_CHIP = 0, 1, 2, 3, 4
OK, E_INVALID, E_UNSUPPORTED, E_BAD_DESCRIPTOR, E_WORKSPACE, E_HIP, E_NOMEM = range(7)
ALGO_NAMES = {ALGO_CLASSIC: "classic", ALGO_L1: "l1", ALGO_L2: "l2"}
_ALGO = {"auto": ALGO_AUTO, "classic": ALGO_CLASSIC, "l1": ALGO_L1, "l2": ALGO_L2}
_SPLIT = {"auto": SPLIT_AUTO, "none": SPLIT_NONE, "all": SPLIT_ALL}
ORDER_AUTO, ORDER_PLAIN = 0, 1
_ORDER = {"auto": ORDER_AUTO, "plain": ORDER_PLAIN}
_COMBINE = {"auto": COMBINE_AUTO, "prepass": COMBINE_PREPASS, "at_load": COMBINE_AT_LOAD, "unfused": COMBINE_UNFUSED,
            "l2_on_chip": COMBINE_L2_ON_CHIP}

_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t


class lcma_desc(ctypes.Structure):
    _fields_ = [("ms", _i32), ("ks", _i32), ("ns", _i32), ("rank", _i32),
                ("U", ctypes.POINTER(ctypes.c_int8)), ("V", ctypes.POINTER(ctypes.c_int8)),
                ("W", ctypes.POINTER(ctypes.c_int8))]


class lcma_options(ctypes.Structure):
    _fields_ = [("split", _i32), ("combine", _i32), ("bf16_ops_f16", _i32), ("num_cus", _i32),
                ("peak_tflops", ctypes.c_double), ("hbm_gbps", ctypes.c_double),
                ("classic_eff", ctypes.c_double), ("fused_eff", ctypes.c_double), ("order", _i32),
                ("accuracy_optin", _i32)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_lib_status_str = _sig("lcma_status_str", ctypes.c_char_p, [_i32])
_lib_desc_builtin = _sig("lcma_desc_builtin", _i32, [_i32, ctypes.POINTER(lcma_desc)])
_lib_desc_winograd = _sig("lcma_desc_winograd", _i32, [ctypes.POINTER(lcma_desc)])
_lib_desc_validate = _sig("lcma_desc_validate", _i32, [ctypes.POINTER(lcma_desc)])
_lib_plan_ex = _sig("lcma_plan_ex", _i32, [_i64, _i64, _i64, _i32, ctypes.POINTER(lcma_desc), _i32,
                                           ctypes.POINTER(lcma_options), ctypes.POINTER(_vp)])
_lib_plan_info = _sig("lcma_plan_info", _i32, [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_sz),
                                               ctypes.POINTER(ctypes.c_double)])
_lib_plan_estimate = _sig("lcma_plan_estimate", _i32, [_vp, _i32, ctypes.POINTER(ctypes.c_double)])
_lib_gemm = _sig("lcma_gemm", _i32, [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp])
_lib_measure_mfma = _sig("lcma_measure_mfma", _i32, [_vp, _i32, _i32, _i32, _vp])
_lib_measure_copy = _sig("lcma_measure_copy", _i32, [_vp, _vp, _sz, _vp])
_lib_measure_read = _sig("lcma_measure_read", _i32, [_vp, _sz, _vp, _vp])
_lib_gemm_noalloc = _sig("lcma_gemm_noalloc", _i32, [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp])
_lib_prepass = _sig("lcma_prepass", _i32, [_vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp])
_lib_fused = _sig("lcma_fused", _i32, [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp])
_lib_plan_operand = _sig("lcma_plan_operand", _i32, [_vp, _i32, _i32, ctypes.POINTER(_i64),
                                                     ctypes.POINTER(_i64), ctypes.POINTER(_i32)])
_lib_plan_schedule = _sig("lcma_plan_schedule", _i32, [_vp, ctypes.POINTER(_i32), _i64,
                                                       ctypes.POINTER(_i64), ctypes.POINTER(_i32)])
_lib_plan_runs = _sig("lcma_plan_runs", _i32, [_vp, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                               ctypes.POINTER(ctypes.c_int8)])
_lib_classic = _sig("gemm_classic", _i32, [_i64, _i64, _i64, _i32, _vp, _i64, _vp, _i64, _vp, _i64, _vp])
_lib_plan_destroy = _sig("lcma_plan_destroy", None, [_vp])

EXPORTED = ["lcma_status_str", "lcma_desc_builtin", "lcma_desc_winograd", "lcma_desc_validate", "lcma_plan", "lcma_plan_ex",
            "lcma_plan_info", "lcma_plan_estimate", "lcma_gemm", "lcma_prepass", "lcma_fused",
            "lcma_plan_operand", "lcma_plan_schedule", "lcma_plan_runs", "gemm_classic", "lcma_plan_destroy", "lcma_gemm_noalloc",
            "lcma_measure_mfma", "lcma_measure_copy", "lcma_measure_read"]
SCRATCH_BYTES = 64 << 20   # LCMA_SCRATCH_BYTES


class LcmaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {lcma_status_str(status)} (status {status})")


def _check(status: int, what: str):
    if status != OK:
        raise LcmaError(status, what)


def lcma_status_str(status: int) -> str:
    return _lib_status_str(status).decode()


# ---------------------------------------------------------------- marshalling helpers

def _dt(dtype) -> int:
    if dtype in (F16, BF16):
        return dtype
    name = str(dtype).replace("torch.", "")
    if name in ("f16", "float16", "half"):
        return F16
    if name in ("bf16", "bfloat16"):
        return BF16
    raise ValueError(f"unsupported dtype {dtype!r}")


def _ptr(x):
    """Device address of a tensor (or an int address / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _ld(t, default):
    if t is None or isinstance(t, int):
        return default
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("operands must be 2-D with unit column stride (row-major)")
    return t.stride(0)


_TORCH_DT = {F16: torch.float16, BF16: torch.bfloat16}


def _device_of_stream(stream, *tensors):
    """Device the call runs on (the stream's, else the current one), after
    checking that every tensor argument is a device tensor at all."""
    for what, t in tensors:
        if isinstance(t, torch.Tensor) and not t.is_cuda:
            raise ValueError(f"{what} must be a device tensor (got {t.device})")
    return torch.cuda.current_device() if stream is None or isinstance(stream, int) else stream.device.index


def _check_matrix(t, rows, cols, ld, dtype, what, device):
    """Checks a tensor argument against the extent the library will address:
    rows x cols elements at leading dimension ld from its data pointer, on the
    plan's device and of the plan's storage type.  Raw integer addresses (and
    None) pass unchecked: the C ABI cannot see buffer sizes, this layer can."""
    if t is None or isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor or a device address, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor (got {t.device})")
    if t.device.index != device:
        raise ValueError(f"{what} is on {t.device}, the call runs on cuda:{device}")
    if dtype is not None and t.dtype != _TORCH_DT[dtype]:
        raise ValueError(f"{what} has dtype {t.dtype}, the plan's storage type is {_TORCH_DT[dtype]}")
    if rows <= 0 or cols <= 0:
        return
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{what} must be 2-D with unit column stride (row-major)")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{what} has shape {tuple(t.shape)}, the call addresses {rows} x {cols}")
    if ld < cols:
        raise ValueError(f"{what}: leading dimension {ld} < {cols} columns")
    need = t.storage_offset() + (rows - 1) * ld + cols
    have = t.untyped_storage().nbytes() // t.element_size()
    if need > have:
        raise ValueError(f"{what}: {rows} rows at leading dimension {ld} need {need} elements of storage, "
                         f"the tensor's storage holds {have}")


def _check_workspace(ws, nbytes, device):
    if ws is None or isinstance(ws, int):
        return
    if not ws.is_cuda or ws.device.index != device:
        raise ValueError(f"workspace must be a device tensor on cuda:{device} (got {ws.device})")
    have = ws.untyped_storage().nbytes() - ws.storage_offset() * ws.element_size()
    if not ws.is_contiguous() or have < nbytes:
        raise ValueError(f"workspace: a contiguous buffer of at least {nbytes} bytes is needed")


def _check_call(plan, A, lda, B, ldb, C, ldc, stream, need_c=True, workspace=None):
    dev = _device_of_stream(stream, ("A", A), ("B", B), ("C", C if need_c else None), ("workspace", workspace))
    _check_matrix(A, plan.M, plan.K, lda, plan.dtype, "A", dev)
    _check_matrix(B, plan.K, plan.N, ldb, plan.dtype, "B", dev)
    if need_c:
        _check_matrix(C, plan.M, plan.N, ldc, plan.dtype, "C", dev)
    return dev


def _current_stream():
    # torch's raw handle of the current stream (one C call; building a
    # torch.cuda.Stream object costs ~3 us per library call)
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _stream(stream):
    if stream is None:
        return _current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Desc:
    """Owns int8 tables and exposes them as an ``lcma_desc``."""

    def __init__(self, ms, ks, ns, U, V, W):
        import numpy as np
        self.U = np.ascontiguousarray(np.asarray(U, dtype=np.int8).ravel())
        self.V = np.ascontiguousarray(np.asarray(V, dtype=np.int8).ravel())
        self.W = np.ascontiguousarray(np.asarray(W, dtype=np.int8).ravel())
        rank = self.U.size // (ms * ks)
        p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int8))
        self.c = lcma_desc(ms, ks, ns, rank, p(self.U), p(self.V), p(self.W))


def _desc_tables(d):
    import numpy as np
    tab = lambda ptr, n: np.ctypeslib.as_array(ptr, shape=(n,)).copy()
    return (d.ms, d.ks, d.ns, d.rank, tab(d.U, d.rank * d.ms * d.ks).reshape(d.rank, -1),
            tab(d.V, d.rank * d.ks * d.ns).reshape(d.rank, -1), tab(d.W, d.rank * d.ms * d.ns).reshape(d.rank, -1))


def lcma_desc_builtin(levels: int):
    """The built-in Strassen scheme as (ms, ks, ns, rank, U, V, W) numpy int8 tables."""
    d = lcma_desc()
    _check(_lib_desc_builtin(levels, ctypes.byref(d)), "lcma_desc_builtin")
    return _desc_tables(d)


def lcma_desc_winograd():
    """Winograd's variant (rank 7) as (ms, ks, ns, rank, U, V, W) numpy int8 tables."""
    d = lcma_desc()
    _check(_lib_desc_winograd(ctypes.byref(d)), "lcma_desc_winograd")
    return _desc_tables(d)


def winograd_desc() -> "Desc":
    """Winograd's variant as a description for lcma_plan_ex(desc=...)."""
    ms, ks, ns, _, U, V, W = lcma_desc_winograd()
    return Desc(ms, ks, ns, U, V, W)


def lcma_desc_validate(desc: Desc) -> int:
    """Status of the C validator (OK or E_BAD_DESCRIPTOR)."""
    return _lib_desc_validate(ctypes.byref(desc.c))


class Plan:
    """An ``lcma_plan_t``; destroyed with the object."""

    def __init__(self, handle, M, N, K, dtype):
        self.handle = handle
        self.M, self.N, self.K, self.dtype = M, N, K, dtype

    def __del__(self, _destroy=_lib_plan_destroy):
        # the library function is bound at definition time: module globals may
        # already be cleared when a plan dies at interpreter exit
        h, self.handle = getattr(self, "handle", None), None
        if h:
            _destroy(h)

    @property
    def info(self):
        return lcma_plan_info(self)


def lcma_plan_ex(M, N, K, dtype, desc: Desc | None = None, force="auto", split="auto", combine="auto",
                 bf16_ops_f16=0, num_cus=0, peak_tflops=0.0, hbm_gbps=0.0, classic_eff=0.0,
                 fused_eff=0.0, order="auto", accuracy_optin=0) -> Plan:
    opts = lcma_options(_SPLIT[split] if isinstance(split, str) else split,
                        _COMBINE[combine] if isinstance(combine, str) else combine,
                        bf16_ops_f16, num_cus, peak_tflops, hbm_gbps, classic_eff, fused_eff,
                        _ORDER[order] if isinstance(order, str) else order, int(accuracy_optin))
    h = _vp()
    st = _lib_plan_ex(M, N, K, _dt(dtype), ctypes.byref(desc.c) if desc is not None else None,
                      _ALGO[force] if isinstance(force, str) else force, ctypes.byref(opts), ctypes.byref(h))
    _check(st, "lcma_plan_ex")
    return Plan(h.value, M, N, K, _dt(dtype))


def lcma_plan(M, N, K, dtype, desc: Desc | None = None, force="auto") -> Plan:
    return lcma_plan_ex(M, N, K, dtype, desc, force)


def lcma_plan_info(plan: Plan):
    """(algorithm name, workspace bytes, estimated seconds)."""
    a, ws, est = _i32(), _sz(), ctypes.c_double()
    _check(_lib_plan_info(plan.handle, ctypes.byref(a), ctypes.byref(ws), ctypes.byref(est)), "lcma_plan_info")
    return ALGO_NAMES[a.value], ws.value, est.value


def lcma_plan_estimate(plan: Plan, algo) -> float:
    e = ctypes.c_double()
    _check(_lib_plan_estimate(plan.handle, _ALGO[algo] if isinstance(algo, str) else algo, ctypes.byref(e)),
           "lcma_plan_estimate")
    return e.value


def lcma_plan_operand(plan: Plan, side: int, r: int):
    """(byte offset in the workspace or -1, leading dimension, dtype code) of a combined operand."""
    off, ld, dt = _i64(), _i64(), _i32()
    _check(_lib_plan_operand(plan.handle, side, r, ctypes.byref(off), ctypes.byref(ld), ctypes.byref(dt)),
           "lcma_plan_operand")
    return off.value, ld.value, dt.value


def lcma_plan_schedule(plan: Plan):
    """(items as a list of (worker, group, pos0, pos1, slot), product order)."""
    n = _i64()
    _check(_lib_plan_schedule(plan.handle, None, 0, ctypes.byref(n), None), "lcma_plan_schedule")
    buf = (_i32 * (5 * max(n.value, 1)))()
    order = (_i32 * 49)()
    _check(_lib_plan_schedule(plan.handle, buf, n.value, ctypes.byref(n), order), "lcma_plan_schedule")
    items = [tuple(buf[5 * i:5 * i + 5]) for i in range(n.value)]
    return items, list(order)


def lcma_plan_runs(plan: Plan, nblocks: int):
    """Run schedule of a persistent unfused plan: a list of (product, carry,
    folds into each of the `nblocks` output blocks), one entry per run."""
    out = []
    prod, carry = _i32(), _i32()
    fold = (ctypes.c_int8 * nblocks)()
    for j in range(64):           # runs 0..rank-1; the first index past them is rejected
        st = _lib_plan_runs(plan.handle, j, ctypes.byref(prod), ctypes.byref(carry), fold)
        if st != 0:
            if j == 0:
                _check(st, "lcma_plan_runs")
            break
        out.append((prod.value, carry.value, list(fold)))
    return out


def lcma_gemm(plan: Plan, A, B, C, workspace=None, workspace_bytes=None, stream=None, lda=None, ldb=None,
              ldc=None) -> None:
    ws_bytes = workspace_bytes if workspace_bytes is not None else (
        0 if workspace is None or isinstance(workspace, int) else workspace.numel() * workspace.element_size())
    lda, ldb, ldc = lda or _ld(A, plan.K), ldb or _ld(B, plan.N), ldc or _ld(C, plan.N)
    dev = _check_call(plan, A, lda, B, ldb, C, ldc, stream, workspace=workspace)
    _check_workspace(workspace, ws_bytes, dev)
    _check(_lib_gemm(plan.handle, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(workspace), ws_bytes,
                     _stream(stream)), "lcma_gemm")


def lcma_gemm_prepared(plan: Plan, A, B, C, workspace=None, workspace_bytes=None, stream=None, lda=None, ldb=None,
                       ldc=None):
    """Checks the arguments of one lcma_gemm call once and returns a function
    that enqueues exactly that call (same buffers, leading dimensions,
    workspace and stream, the current one at preparation when `stream` is
    None) with no per-call checks: for loops that repeat a call on fixed
    buffers, where the checks would take as long as a short kernel.  The
    returned function holds references to the tensors."""
    ws_bytes = workspace_bytes if workspace_bytes is not None else (
        0 if workspace is None or isinstance(workspace, int) else workspace.numel() * workspace.element_size())
    lda, ldb, ldc = lda or _ld(A, plan.K), ldb or _ld(B, plan.N), ldc or _ld(C, plan.N)
    dev = _check_call(plan, A, lda, B, ldb, C, ldc, stream, workspace=workspace)
    _check_workspace(workspace, ws_bytes, dev)
    args = (plan.handle, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(workspace), ws_bytes, _stream(stream))
    held = (plan, A, B, C, workspace)

    def call() -> None:
        _check(_lib_gemm(*args), "lcma_gemm")
    call.held = held
    return call


def lcma_gemm_noalloc(plan: Plan, A, B, C, stream=None, lda=None, ldb=None, ldc=None) -> None:
    """lcma_gemm with the workspace taken from the library's static device scratch
    array (no allocation; plans with a workspace above SCRATCH_BYTES are refused)."""
    lda, ldb, ldc = lda or _ld(A, plan.K), ldb or _ld(B, plan.N), ldc or _ld(C, plan.N)
    _check_call(plan, A, lda, B, ldb, C, ldc, stream)
    _check(_lib_gemm_noalloc(plan.handle, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _stream(stream)),
           "lcma_gemm_noalloc")


def lcma_measure_mfma(out, workgroups: int, iters: int, dtype="bf16", stream=None) -> float:
    """Enqueues the MFMA reference loop; returns the flops it performs."""
    if out.numel() < workgroups * 512 or out.dtype != torch.float32 or not out.is_cuda:
        raise ValueError("out: a float32 device tensor of workgroups * 512 elements is needed")
    _check(_lib_measure_mfma(_ptr(out), workgroups, iters, _dt(dtype), _stream(stream)), "lcma_measure_mfma")
    return float(workgroups) * 8 * iters * 16 * 16384


def lcma_measure_copy(src, dst, stream=None) -> None:
    """Enqueues the HBM stream reference: dst = src (same byte size)."""
    n = src.numel() * src.element_size()
    if not (src.is_cuda and dst.is_cuda) or dst.numel() * dst.element_size() < n:
        raise ValueError("src, dst: device tensors, dst at least as large as src")
    _check(_lib_measure_copy(_ptr(src), _ptr(dst), n, _stream(stream)), "lcma_measure_copy")


def lcma_measure_read(src, out, stream=None) -> None:
    """Enqueues the read-only HBM stream reference over src; out is a device
    tensor of at least 4 bytes that the kernel may write (value unspecified)."""
    n = src.numel() * src.element_size()
    if not (src.is_cuda and out.is_cuda) or out.numel() * out.element_size() < 4:
        raise ValueError("src, out: device tensors, out at least 4 bytes")
    _check(_lib_measure_read(_ptr(src), n, _ptr(out), _stream(stream)), "lcma_measure_read")


def _ws_bytes(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def lcma_prepass(plan: Plan, A, B, workspace, stream=None, lda=None, ldb=None) -> None:
    ws_bytes = _ws_bytes(workspace)
    lda, ldb = lda or _ld(A, plan.K), ldb or _ld(B, plan.N)
    dev = _check_call(plan, A, lda, B, ldb, None, 0, stream, need_c=False, workspace=workspace)
    _check_workspace(workspace, ws_bytes, dev)
    _check(_lib_prepass(plan.handle, _ptr(A), lda, _ptr(B), ldb, _ptr(workspace), ws_bytes, _stream(stream)),
           "lcma_prepass")


def lcma_fused(plan: Plan, A, B, C, workspace, stream=None, lda=None, ldb=None, ldc=None) -> None:
    ws_bytes = _ws_bytes(workspace)
    lda, ldb, ldc = lda or _ld(A, plan.K), ldb or _ld(B, plan.N), ldc or _ld(C, plan.N)
    dev = _check_call(plan, A, lda, B, ldb, C, ldc, stream, workspace=workspace)
    _check_workspace(workspace, ws_bytes, dev)
    _check(_lib_fused(plan.handle, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(workspace), ws_bytes,
                      _stream(stream)), "lcma_fused")


def gemm_classic(A, B, C, stream=None, M=None, N=None, K=None, dtype=None, lda=None, ldb=None, ldc=None) -> None:
    M = M if M is not None else A.shape[0]
    K = K if K is not None else A.shape[1]
    N = N if N is not None else B.shape[1]
    dt = _dt(dtype if dtype is not None else A.dtype)
    lda, ldb, ldc = lda or _ld(A, K), ldb or _ld(B, N), ldc or _ld(C, N)
    dev = _device_of_stream(stream, ("A", A), ("B", B), ("C", C))
    _check_matrix(A, M, K, lda, dt, "A", dev)
    _check_matrix(B, K, N, ldb, dt, "B", dev)
    _check_matrix(C, M, N, ldc, dt, "C", dev)
    _check(_lib_classic(M, N, K, dt, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _stream(stream)), "gemm_classic")


def workspace_for(plan: Plan, device="cuda"):
    """A device buffer of the plan's workspace size (uint8; None when no workspace is needed)."""
    import torch
    _, ws, _ = lcma_plan_info(plan)
    return torch.empty(ws, dtype=torch.uint8, device=device) if ws > 0 else None


def gemm(A, B, algo="auto", out=None, stream=None, **plan_kw):
    """C = A @ B through a plan (allocates C and the workspace with torch)."""
    import torch
    M, K = A.shape
    N = B.shape[1]
    plan = lcma_plan_ex(M, N, K, A.dtype, force=algo, **plan_kw)
    C = out if out is not None else torch.empty((M, N), dtype=A.dtype, device=A.device)
    ws = workspace_for(plan, A.device)
    lcma_gemm(plan, A, B, C, ws, stream=stream)
    return C
