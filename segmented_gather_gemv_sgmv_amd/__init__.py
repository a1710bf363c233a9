"""SGMV for MI355X: multi-LoRA shrink/expand as hand-written HIP kernels.

Thin Python binding over the C ABI of ``libsgmv.so`` (declared in
``include/sgmv.h``).  The functions here only check and marshal torch
tensors (dtype, device, shape, contiguity), pick up torch's current HIP
stream and pass raw device pointers; every arithmetic step runs in the HIP
kernels.  There is no fallback: if the library has not been built, calls
raise.

    lora_apply(y, x, A_stack, B_stack, seg_indptr, adapter_ids, scale)
        y[i] += scale * (x[i] @ A_stack[a]) @ B_stack[a]   for row i of a segment naming a
    sgmv_shrink(v, x, A_stack, seg_indptr, adapter_ids)
        v[i] = x[i] @ A_stack[a]   (v float32)
    sgmv_expand(y, v, B_stack, seg_indptr, adapter_ids, scale)
        y[i] += scale * v[i] @ B_stack[a]

The math is the LoRA correction y = xW + xAB computed per request as
v_i = x_i A_i then v_i B_i over back-to-back stacked adapter matrices
(Punica walkthrough, omica.com.cn/news/959180, sections 2.1-2.2).
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
# SGMV_LIBRARY names another build of the same library (e.g. the host-side
# AddressSanitizer build that the CPU tests load); by default the in-tree one.
LIBRARY = os.environ.get("SGMV_LIBRARY") or os.path.join(_HERE, "libsgmv.so")

SGMV_F32, SGMV_F16, SGMV_BF16 = 0, 1, 2
SGMV_MAX_RANK = 128
STATUS = {
    0: "SGMV_OK", 1: "SGMV_ERR_NULL_PTR", 2: "SGMV_ERR_BAD_SHAPE", 3: "SGMV_ERR_BAD_DTYPE",
    4: "SGMV_ERR_UNSUPPORTED", 5: "SGMV_ERR_WORKSPACE", 6: "SGMV_ERR_HIP",
    7: "SGMV_ERR_BAD_SEGMENTS", 8: "SGMV_ERR_SCRATCH",
}
SGMV_NOALLOC_SCRATCH_BYTES = 16 << 20
SGMV_MAX_PROBLEMS = 8


class LoraProblem(ctypes.Structure):
    """sgmv_lora_problem of sgmv.h: one add-on of a lora_apply_multi call."""
    _fields_ = [("y", ctypes.c_void_p), ("x", ctypes.c_void_p), ("A_stack", ctypes.c_void_p),
                ("B_stack", ctypes.c_void_p), ("H1", ctypes.c_int32), ("H2", ctypes.c_int32),
                ("scale", ctypes.c_float)]


# (name, restype, argtypes) of every symbol the header declares.
_i32, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
ABI = [
    ("sgmv_abi_version", ctypes.c_int, []),
    ("sgmv_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("sgmv_last_hip_error", ctypes.c_char_p, []),
    ("sgmv_shrink_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32]),
    ("sgmv_shrink", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                   _vp, _sz, _vp]),
    ("sgmv_expand", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32,
                                   _i32, _vp]),
    ("lora_apply_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    ("lora_apply", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                  _i32, _f32, _i32, _vp, _sz, _vp]),
    ("lora_apply_noalloc", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                          _i32, _i32, _f32, _i32, _vp]),
    ("sgmv_set_fused_wait", ctypes.c_int, [ctypes.c_double]),
    ("sgmv_validate_segments", ctypes.c_int, [_vp, _vp, _i32, _i32, _i32]),
    ("sgmv_build_segments", ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    ("sgmv_group_rows", ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    ("sgmv_load_adapter", ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _i32,
                                         _i32, _vp]),
    ("lora_apply_multi_workspace_bytes", _sz, [_vp, _i32, _i32, _i32, _i32, _i32]),
    ("lora_apply_multi", ctypes.c_int, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp,
                                        _sz, _vp]),
    ("lora_linear_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    ("lora_linear", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                   _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
]


class SGMVError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS.get(code, code)}")
        self.code = code


_lib_handle = None
_lib_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded ``libsgmv.so`` with argument types set (raises if not built).

    torch is imported first on purpose: torch ships its own HIP runtime
    (soname libamdhip64.so.7), and the library must bind to that same
    runtime so that torch's streams and allocations are valid in its calls.
    Loaded the other way round, the process would hold two HIP runtimes."""
    global _lib_handle
    with _lib_lock:
        if _lib_handle is None:
            import torch  # noqa: F401  (see above)
            if not os.path.exists(LIBRARY):
                raise RuntimeError(
                    f"{LIBRARY} is missing: build it with "
                    "`python -m segmented_gather_gemv_sgmv_amd.build` (there is no fallback)")
            handle = ctypes.CDLL(LIBRARY)
            for name, restype, argtypes in ABI:
                fn = getattr(handle, name)
                fn.restype = restype
                fn.argtypes = argtypes
            _lib_handle = handle
    return _lib_handle


def _check(code: int, what: str):
    if code != 0:
        if code == 6:  # SGMV_ERR_HIP: add the HIP runtime's own message
            what = f"{what} ({lib().sgmv_last_hip_error().decode()})"
        raise SGMVError(code, what)


# -- torch marshalling -----------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(dtype) -> int:
    torch = _torch()
    codes = {torch.float32: SGMV_F32, torch.float16: SGMV_F16, torch.bfloat16: SGMV_BF16}
    if dtype not in codes:
        raise TypeError(f"unsupported dtype {dtype}; expected float32, float16 or bfloat16")
    return codes[dtype]


def _stream_ptr(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def _need(t, name, device, dtype=None, ndim=None):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def _segments(seg_indptr, adapter_ids, device):
    torch = _torch()
    _need(seg_indptr, "seg_indptr", device, torch.int32, 1)
    _need(adapter_ids, "adapter_ids", device, torch.int32, 1)
    if seg_indptr.numel() != adapter_ids.numel() + 1:
        raise ValueError("seg_indptr must have exactly one more entry than adapter_ids")
    return adapter_ids.numel()


class _WorkspaceCache:
    """One growable, zero-initialised device buffer per (device, stream).

    Calls on one stream run in order, so they can share its buffer; the
    library leaves the buffer's counter region zero after every call, as it
    requires on entry.  Not used while a stream is capturing a graph: a
    captured call would keep the buffer's address in the graph, and the
    cache may later replace that buffer or hand it to eager calls on a
    stream the graph does not order against.  Graph captures must pass an
    explicit workspace (see ``need_workspace``)."""

    def __init__(self):
        self._bufs = {}
        self._lock = threading.Lock()

    def get(self, device, stream: int, nbytes: int, what: str):
        torch = _torch()
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(
                f"{what}: no workspace given while a HIP graph is being captured; pass "
                f"workspace= a zeroed uint8 device tensor of at least {nbytes} bytes, owned by "
                "the caller for as long as the graph may be replayed")
        key = (device, stream)
        with self._lock:
            buf = self._bufs.get(key)
            if buf is None or buf.numel() < nbytes:
                buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
                self._bufs[key] = buf
            return buf


_workspaces = _WorkspaceCache()


def shrink_workspace_bytes(num_rows, num_segments, H1, r, dtype) -> int:
    return int(lib().sgmv_shrink_workspace_bytes(num_rows, num_segments, H1, r, dtype_code(dtype)))


def lora_apply_workspace_bytes(num_rows, num_segments, H1, H2, r, dtype) -> int:
    return int(lib().lora_apply_workspace_bytes(num_rows, num_segments, H1, H2, r,
                                                dtype_code(dtype)))


def sgmv_shrink(v, x, A_stack, seg_indptr, adapter_ids, workspace=None):
    """v[i, :] = x[i, :] @ A_stack[a] (float32 v, overwritten for covered rows)."""
    torch = _torch()
    dev = x.device
    _need(x, "x", dev, None, 2)
    _need(A_stack, "A_stack", dev, x.dtype, 3)
    _need(v, "v", dev, torch.float32, 2)
    S = _segments(seg_indptr, adapter_ids, dev)
    R, H1 = x.shape
    N, H1a, r = A_stack.shape
    if H1a != H1 or tuple(v.shape) != (R, r):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, A_stack {tuple(A_stack.shape)}, "
                         f"v {tuple(v.shape)}")
    dt = dtype_code(x.dtype)
    stream = _stream_ptr(dev)
    need = shrink_workspace_bytes(R, S, H1, r, x.dtype)
    if workspace is None and need > 0:
        workspace = _workspaces.get(dev, stream, need, "sgmv_shrink")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sgmv_shrink(v.data_ptr(), x.data_ptr(), A_stack.data_ptr(), seg_indptr.data_ptr(),
                             adapter_ids.data_ptr(), S, R, N, H1, r, dt, ws_ptr, ws_bytes, stream),
           "sgmv_shrink")
    return v


def sgmv_expand(y, v, B_stack, seg_indptr, adapter_ids, scale=1.0):
    """y[i, :] += scale * v[i, :] @ B_stack[a], rounded once to y's dtype."""
    torch = _torch()
    dev = y.device
    _need(y, "y", dev, None, 2)
    _need(B_stack, "B_stack", dev, y.dtype, 3)
    _need(v, "v", dev, torch.float32, 2)
    S = _segments(seg_indptr, adapter_ids, dev)
    R, H2 = y.shape
    N, r, H2b = B_stack.shape
    if H2b != H2 or tuple(v.shape) != (R, r):
        raise ValueError(f"shape mismatch: y {tuple(y.shape)}, B_stack {tuple(B_stack.shape)}, "
                         f"v {tuple(v.shape)}")
    _check(lib().sgmv_expand(y.data_ptr(), v.data_ptr(), B_stack.data_ptr(), seg_indptr.data_ptr(),
                             adapter_ids.data_ptr(), S, R, N, r, H2, float(scale),
                             dtype_code(y.dtype), _stream_ptr(dev)),
           "sgmv_expand")
    return y


def lora_apply(y, x, A_stack, B_stack, seg_indptr, adapter_ids, scale=1.0, workspace=None):
    """y[i, :] += scale * (x[i, :] @ A_stack[a]) @ B_stack[a], fp32 accumulation.

    ``workspace`` (optional): a uint8 device tensor of at least
    ``lora_apply_workspace_bytes(...)`` bytes that was zero when first used
    (e.g. ``torch.zeros``); by default a per-stream cached buffer is used."""
    dev = x.device
    _need(x, "x", dev, None, 2)
    _need(y, "y", dev, x.dtype, 2)
    _need(A_stack, "A_stack", dev, x.dtype, 3)
    _need(B_stack, "B_stack", dev, x.dtype, 3)
    S = _segments(seg_indptr, adapter_ids, dev)
    R, H1 = x.shape
    N, H1a, r = A_stack.shape
    Nb, rb, H2 = B_stack.shape
    if H1a != H1 or Nb != N or rb != r or tuple(y.shape) != (R, H2):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, y {tuple(y.shape)}, "
                         f"A_stack {tuple(A_stack.shape)}, B_stack {tuple(B_stack.shape)}")
    dt = dtype_code(x.dtype)
    stream = _stream_ptr(dev)
    need = lora_apply_workspace_bytes(R, S, H1, H2, r, x.dtype)
    if workspace is None:
        workspace = _workspaces.get(dev, stream, need, "lora_apply")
    _check(lib().lora_apply(y.data_ptr(), x.data_ptr(), A_stack.data_ptr(), B_stack.data_ptr(),
                            seg_indptr.data_ptr(), adapter_ids.data_ptr(), S, R, N, H1, H2, r,
                            float(scale), dt, workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), stream),
           "lora_apply")
    return y


def lora_apply_noalloc(y, x, A_stack, B_stack, seg_indptr, adapter_ids, scale=1.0):
    """lora_apply without a workspace argument: the library's static per-GPU
    scratch (SGMV_NOALLOC_SCRATCH_BYTES) serves every call, and nothing is
    allocated, so the call may be captured in a graph as it stands.  Calls
    that may overlap on one GPU race on that scratch."""
    dev = x.device
    _need(x, "x", dev, None, 2)
    _need(y, "y", dev, x.dtype, 2)
    _need(A_stack, "A_stack", dev, x.dtype, 3)
    _need(B_stack, "B_stack", dev, x.dtype, 3)
    S = _segments(seg_indptr, adapter_ids, dev)
    R, H1 = x.shape
    N, H1a, r = A_stack.shape
    Nb, rb, H2 = B_stack.shape
    if H1a != H1 or Nb != N or rb != r or tuple(y.shape) != (R, H2):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, y {tuple(y.shape)}, "
                         f"A_stack {tuple(A_stack.shape)}, B_stack {tuple(B_stack.shape)}")
    _check(lib().lora_apply_noalloc(y.data_ptr(), x.data_ptr(), A_stack.data_ptr(),
                                    B_stack.data_ptr(), seg_indptr.data_ptr(),
                                    adapter_ids.data_ptr(), S, R, N, H1, H2, r, float(scale),
                                    dtype_code(x.dtype), _stream_ptr(dev)),
           "lora_apply_noalloc")
    return y


def lora_linear_workspace_bytes(num_rows, num_segments, H1, H2, r, dtype) -> int:
    return int(lib().lora_linear_workspace_bytes(num_rows, num_segments, H1, H2, r,
                                                 dtype_code(dtype)))


def lora_linear(x, W, A_stack, B_stack, seg_indptr, adapter_ids, scale=1.0, bias=None,
                out=None, workspace=None):
    """Adapted linear layer, base product fused in: returns
    y = x @ W.T (+ bias) + scale * (x @ A_stack[a]) @ B_stack[a] per row of
    each segment (base product only on other rows), float32 sums, rounded
    once.  W is [H2, H1] (torch's linear weight layout), bias [H2] or None.
    ``out`` (optional) receives y; ``workspace`` as for lora_apply."""
    torch = _torch()
    dev = x.device
    _need(x, "x", dev, None, 2)
    _need(W, "W", dev, x.dtype, 2)
    _need(A_stack, "A_stack", dev, x.dtype, 3)
    _need(B_stack, "B_stack", dev, x.dtype, 3)
    S = _segments(seg_indptr, adapter_ids, dev)
    R, H1 = x.shape
    H2, H1w = W.shape
    N, H1a, r = A_stack.shape
    if H1w != H1 or H1a != H1 or tuple(B_stack.shape) != (N, r, H2):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, W {tuple(W.shape)}, "
                         f"A_stack {tuple(A_stack.shape)}, B_stack {tuple(B_stack.shape)}")
    if bias is not None:
        _need(bias, "bias", dev, x.dtype, 1)
        if bias.shape[0] != H2:
            raise ValueError(f"bias must be [{H2}], got {tuple(bias.shape)}")
    if out is None:
        out = torch.empty((R, H2), dtype=x.dtype, device=dev)
    else:
        _need(out, "out", dev, x.dtype, 2)
        if tuple(out.shape) != (R, H2):
            raise ValueError(f"out must be {(R, H2)}, got {tuple(out.shape)}")
    dt = dtype_code(x.dtype)
    stream = _stream_ptr(dev)
    need = lora_linear_workspace_bytes(R, S, H1, H2, r, x.dtype)
    if workspace is None:
        workspace = _workspaces.get(dev, stream, need, "lora_linear")
    _check(lib().lora_linear(out.data_ptr(), x.data_ptr(), W.data_ptr(),
                             None if bias is None else bias.data_ptr(), A_stack.data_ptr(),
                             B_stack.data_ptr(), seg_indptr.data_ptr(), adapter_ids.data_ptr(),
                             S, R, N, H1, H2, r, float(scale), dt, workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), stream),
           "lora_linear")
    return out


def lora_apply_multi_workspace_bytes(shapes, num_rows, num_segments, r, dtype) -> int:
    """Workspace bytes of a lora_apply_multi call whose problems have the
    given (H1, H2) shapes."""
    arr = (LoraProblem * len(shapes))(*[LoraProblem(None, None, None, None, int(h1), int(h2), 1.0)
                                        for h1, h2 in shapes])
    return int(lib().lora_apply_multi_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p),
                                                      len(shapes), num_rows, num_segments, r,
                                                      dtype_code(dtype)))


def lora_apply_multi(problems, seg_indptr, adapter_ids, workspace=None):
    """Several add-ons over one batch in one call: ``problems`` is a list of
    ``(y, x, A_stack, B_stack, scale)`` (each y updated in place, as by
    ``lora_apply``); all share the segment table, rows, adapter count, rank
    and dtype.  Returns the list of y tensors."""
    torch = _torch()
    problems = list(problems)
    if not 1 <= len(problems) <= SGMV_MAX_PROBLEMS:
        raise ValueError(f"between 1 and {SGMV_MAX_PROBLEMS} problems, got {len(problems)}")
    y0, x0, A0, _, _ = problems[0]
    dev = x0.device
    R = x0.shape[0]
    N, _, r = A0.shape
    dt = dtype_code(x0.dtype)
    S = _segments(seg_indptr, adapter_ids, dev)
    arr = (LoraProblem * len(problems))()
    for k, (y, x, A_stack, B_stack, scale) in enumerate(problems):
        _need(x, "x", dev, x0.dtype, 2)
        _need(y, "y", dev, x0.dtype, 2)
        _need(A_stack, "A_stack", dev, x0.dtype, 3)
        _need(B_stack, "B_stack", dev, x0.dtype, 3)
        H1, H2 = x.shape[1], y.shape[1]
        if (x.shape[0] != R or y.shape[0] != R or tuple(A_stack.shape) != (N, H1, r)
                or tuple(B_stack.shape) != (N, r, H2)):
            raise ValueError(f"problem {k}: shapes disagree (x {tuple(x.shape)}, y {tuple(y.shape)}, "
                             f"A {tuple(A_stack.shape)}, B {tuple(B_stack.shape)})")
        arr[k] = LoraProblem(y.data_ptr(), x.data_ptr(), A_stack.data_ptr(), B_stack.data_ptr(),
                             H1, H2, float(scale))
    stream = _stream_ptr(dev)
    parr = ctypes.cast(arr, ctypes.c_void_p)
    need = int(lib().lora_apply_multi_workspace_bytes(parr, len(problems), R, S, r, dt))
    if need == 0:
        raise SGMVError(4, "lora_apply_multi_workspace_bytes")
    if workspace is None:
        workspace = _workspaces.get(dev, stream, need, "lora_apply_multi")
    _check(lib().lora_apply_multi(parr, len(problems), seg_indptr.data_ptr(),
                                  adapter_ids.data_ptr(), S, R, N, r, dt, workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), stream),
           "lora_apply_multi")
    return [pr[0] for pr in problems]


def load_adapter(A_stack, B_stack, slot: int, A, B):
    """Copy adapters from host tensors into the device stacks, on the current
    stream: A [H1, r] and B [r, H2] for one adapter into slot ``slot``, or
    A [count, H1, r] and B [count, r, H2] into slots [slot, slot + count).
    Pin the host tensors for an asynchronous copy."""
    dev = A_stack.device
    _need(A_stack, "A_stack", dev, None, 3)
    _need(B_stack, "B_stack", dev, A_stack.dtype, 3)
    N, H1, r = A_stack.shape
    H2 = B_stack.shape[2]
    if A.device.type != "cpu" or B.device.type != "cpu":
        raise ValueError("A and B must be host tensors")
    count = 1 if A.dim() == 2 else A.shape[0]
    if tuple(A.shape[-2:]) != (H1, r) or tuple(B.shape[-2:]) != (r, H2) or \
            A.dim() not in (2, 3) or B.dim() != A.dim() or (A.dim() == 3 and B.shape[0] != count):
        raise ValueError(f"A must be [count,] {(H1, r)} and B [count,] {(r, H2)}")
    if A.dtype != A_stack.dtype or B.dtype != A_stack.dtype:
        raise TypeError("A and B must have the stacks' dtype")
    if not A.is_contiguous() or not B.is_contiguous():
        raise ValueError("A and B must be contiguous")
    _check(lib().sgmv_load_adapter(A_stack.data_ptr(), B_stack.data_ptr(), int(slot), count, N,
                                   A.data_ptr(), B.data_ptr(), H1, H2, r,
                                   dtype_code(A_stack.dtype), _stream_ptr(dev)),
           "sgmv_load_adapter")


def set_fused_wait(seconds: float) -> None:
    """Patience of the single-kernel lora_apply's expand workgroups (see sgmv.h)."""
    _check(lib().sgmv_set_fused_wait(float(seconds)), "sgmv_set_fused_wait")


def validate_segments(seg_indptr, adapter_ids, num_rows, num_adapters) -> int:
    """Check a host (CPU) copy of a segment table; returns the status code."""
    import numpy as np
    seg = np.ascontiguousarray(np.asarray(seg_indptr), dtype=np.int32)
    ids = np.ascontiguousarray(np.asarray(adapter_ids), dtype=np.int32)
    if seg.ndim != 1 or ids.ndim != 1 or seg.shape[0] != ids.shape[0] + 1:
        raise ValueError("seg_indptr must have exactly one more entry than adapter_ids")
    return int(lib().sgmv_validate_segments(seg.ctypes.data, ids.ctypes.data if ids.size else None,
                                            ids.shape[0], num_rows, num_adapters))


def _outputs(out, sizes, dev, names):
    """Caller-provided int32 output tensors (checked) or new ones."""
    torch = _torch()
    if out is None:
        return [torch.empty(n, dtype=torch.int32, device=dev) for n in sizes]
    if len(out) != len(sizes):
        raise ValueError(f"out must hold {len(sizes)} tensors: {', '.join(names)}")
    for t, n, name in zip(out, sizes, names):
        _need(t, name, dev, torch.int32, 1)
        if t.numel() != n:
            raise ValueError(f"{name} must have {n} entries, got {t.numel()}")
    return list(out)


def build_segments(row_ids, num_adapters: int, out=None):
    """Segment table from per-row adapter ids (int32 device tensor), one
    segment per maximal run of equal ids.  Returns ``(seg_indptr,
    adapter_ids, num_segments)``: tables of ``num_rows + 1`` / ``num_rows``
    entries whose tail describes empty segments (so they can go straight to
    ``lora_apply``) and a one-element device tensor with the real count.
    ``out`` may supply those three tensors."""
    torch = _torch()
    dev = row_ids.device
    _need(row_ids, "row_ids", dev, torch.int32, 1)
    R = row_ids.numel()
    seg, ids, count = _outputs(out, (R + 1, R, 1), dev,
                               ("seg_indptr", "adapter_ids", "num_segments"))
    _check(lib().sgmv_build_segments(row_ids.data_ptr() if R else None, R, int(num_adapters),
                                     seg.data_ptr(), ids.data_ptr() if R else None,
                                     count.data_ptr(), _stream_ptr(dev)),
           "sgmv_build_segments")
    return seg, ids, count


def group_rows(row_ids, num_adapters: int, out=None):
    """Stable grouping of rows by adapter (int32 device tensor of per-row
    ids).  Returns ``(perm, seg_indptr, adapter_ids, num_segments)``: row j
    of the grouped batch is row ``perm[j]``; the table describes the grouped
    batch with one segment per adapter present, padded with empty segments
    to min(num_rows, num_adapters) entries.  ``out`` may supply those four
    tensors."""
    torch = _torch()
    dev = row_ids.device
    _need(row_ids, "row_ids", dev, torch.int32, 1)
    R = row_ids.numel()
    M = min(R, max(int(num_adapters), 0))
    perm, seg, ids, count = _outputs(out, (R, M + 1, M, 1), dev,
                                     ("perm", "seg_indptr", "adapter_ids", "num_segments"))
    _check(lib().sgmv_group_rows(row_ids.data_ptr() if R else None, R, int(num_adapters),
                                 perm.data_ptr() if R else None, seg.data_ptr(),
                                 ids.data_ptr() if M else None, count.data_ptr(),
                                 _stream_ptr(dev)),
           "sgmv_group_rows")
    return perm, seg, ids, count


__all__ = [
    "lora_linear", "lora_linear_workspace_bytes",
    "build_segments", "group_rows", "lora_apply_multi", "lora_apply_multi_workspace_bytes",
    "load_adapter",
    "LoraProblem",
    "lora_apply", "lora_apply_noalloc", "sgmv_shrink", "sgmv_expand", "lora_apply_workspace_bytes",
    "shrink_workspace_bytes", "validate_segments", "set_fused_wait", "lib", "SGMVError", "ABI", "LIBRARY",
]
