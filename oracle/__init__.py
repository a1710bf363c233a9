"""CPU oracle for the SGMV LoRA add-on -- TEST INFRASTRUCTURE ONLY.

A plain fp64 C implementation (``sgmv_oracle.c``) of the multi-LoRA correction
y_i += s * (x_i A_a) B_a over contiguous row segments, loaded through ctypes.
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the HIP product library never does and
shares no code, header or helper with it.

What it follows: the LoRA forward y = xW + xAB with A [H1, r] and B [r, H2]
(Punica walkthrough, omica.com.cn/news/959180, section 2.1) and its two-step
batched evaluation v_i = x_i A_i, then v_i B_i, over back-to-back stacked
adapter matrices (same page, section 2.2).  The C file's header lists the
readings taken where the pages are silent.

Inputs are float32 numpy arrays holding values already rounded to the working
dtype (exact in float32); all arithmetic is double precision.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sgmv_oracle.c")
LIBRARY = os.path.join(_HERE, "libsgmv_oracle.so")

# Plain optimisation only: no fast-math and no FMA contraction, so the
# compiled code keeps the sums exactly in the order the C source writes them.
CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", "-fno-fast-math"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc and return the path of the shared library."""
    tmp = output + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, source], check=True)
    os.replace(tmp, output)
    return output


_P = ctypes.POINTER
_i32 = ctypes.c_int32


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        dp, fp, ip = _P(ctypes.c_double), _P(ctypes.c_float), _P(_i32)
        lib.sgmv_oracle_shrink.argtypes = [dp, fp, fp, ip, ip, _i32, _i32, _i32, _i32, _i32]
        lib.sgmv_oracle_expand.argtypes = [dp, dp, fp, ip, ip, _i32, _i32, _i32, _i32, _i32,
                                           ctypes.c_double]
        lib.sgmv_oracle_lora_apply.argtypes = [dp, dp, fp, fp, fp, fp, ip, ip, _i32, _i32, _i32,
                                               _i32, _i32, _i32, ctypes.c_double]
        lib.sgmv_oracle_lora_linear.argtypes = [dp, fp, fp, fp, fp, fp, ip, ip, _i32, _i32, _i32,
                                                _i32, _i32, _i32, ctypes.c_double]
        for f in (lib.sgmv_oracle_shrink, lib.sgmv_oracle_expand, lib.sgmv_oracle_lora_apply,
                  lib.sgmv_oracle_lora_linear):
            f.restype = ctypes.c_int
        self.lib = lib

    # -- marshalling helpers (no arithmetic) ---------------------------------
    @staticmethod
    def _f32(a):
        return np.ascontiguousarray(a, dtype=np.float32)

    @staticmethod
    def _i32a(a):
        return np.ascontiguousarray(a, dtype=np.int32)

    @staticmethod
    def _ptr(a, ctype):
        return a.ctypes.data_as(_P(ctype))

    def _segs(self, seg_indptr, adapter_ids):
        seg = self._i32a(seg_indptr)
        ids = self._i32a(adapter_ids)
        if seg.ndim != 1 or ids.ndim != 1 or seg.shape[0] != ids.shape[0] + 1:
            raise ValueError("seg_indptr must have one more entry than adapter_ids")
        return seg, ids

    # -- the three operations -------------------------------------------------
    def shrink(self, x, A_stack, seg_indptr, adapter_ids, v_init=None):
        """v[i] = x[i] @ A_stack[a] for covered rows; other rows keep v_init."""
        x, A = self._f32(x), self._f32(A_stack)
        seg, ids = self._segs(seg_indptr, adapter_ids)
        R, H1 = x.shape
        N, H1a, r = A.shape
        if H1a != H1:
            raise ValueError("x and A_stack disagree on H1")
        v = (np.zeros((R, r)) if v_init is None
             else np.array(v_init, dtype=np.float64, copy=True, order="C"))
        rc = self.lib.sgmv_oracle_shrink(self._ptr(v, ctypes.c_double), self._ptr(x, ctypes.c_float),
                                         self._ptr(A, ctypes.c_float), self._ptr(seg, _i32),
                                         self._ptr(ids, _i32), ids.shape[0], R, N, H1, r)
        if rc:
            raise ValueError("oracle rejected the segment table or shapes")
        return v

    def expand(self, y0, v, B_stack, seg_indptr, adapter_ids, scale):
        """y = y0 with y[i] += scale * v[i] @ B_stack[a] for covered rows."""
        y = np.array(y0, dtype=np.float64, copy=True, order="C")
        v = np.ascontiguousarray(v, dtype=np.float64)
        B = self._f32(B_stack)
        seg, ids = self._segs(seg_indptr, adapter_ids)
        R, H2 = y.shape
        N, r, H2b = B.shape
        if H2b != H2 or v.shape != (R, r):
            raise ValueError("shape mismatch between y, v and B_stack")
        rc = self.lib.sgmv_oracle_expand(self._ptr(y, ctypes.c_double), self._ptr(v, ctypes.c_double),
                                         self._ptr(B, ctypes.c_float), self._ptr(seg, _i32),
                                         self._ptr(ids, _i32), ids.shape[0], R, N, r, H2,
                                         float(scale))
        if rc:
            raise ValueError("oracle rejected the segment table or shapes")
        return y

    def lora_apply(self, y0, x, A_stack, B_stack, seg_indptr, adapter_ids, scale):
        """Return (y, v): y = y0 + scale * (x A) B per segment, v = x A (0 outside)."""
        y0, x = self._f32(y0), self._f32(x)
        A, B = self._f32(A_stack), self._f32(B_stack)
        seg, ids = self._segs(seg_indptr, adapter_ids)
        R, H1 = x.shape
        N, H1a, r = A.shape
        Nb, rb, H2 = B.shape
        if H1a != H1 or Nb != N or rb != r or y0.shape != (R, H2):
            raise ValueError("shape mismatch between x, y0 and the stacks")
        y = np.empty((R, H2))
        v = np.empty((R, r))
        rc = self.lib.sgmv_oracle_lora_apply(
            self._ptr(y, ctypes.c_double), self._ptr(v, ctypes.c_double),
            self._ptr(y0, ctypes.c_float), self._ptr(x, ctypes.c_float),
            self._ptr(A, ctypes.c_float), self._ptr(B, ctypes.c_float),
            self._ptr(seg, _i32), self._ptr(ids, _i32), ids.shape[0], R, N, H1, H2, r,
            float(scale))
        if rc:
            raise ValueError("oracle rejected the segment table or shapes")
        return y, v

    def lora_linear(self, x, W, bias, A_stack, B_stack, seg_indptr, adapter_ids, scale):
        """y = x @ W^T (+ bias) for every row, plus scale * (x A) B on the rows
        of each segment.  W is [H2, H1]; bias is [H2] or None."""
        x, W = self._f32(x), self._f32(W)
        A, B = self._f32(A_stack), self._f32(B_stack)
        seg, ids = self._segs(seg_indptr, adapter_ids)
        R, H1 = x.shape
        H2, H1w = W.shape
        N, H1a, r = A.shape
        if H1w != H1 or H1a != H1 or B.shape != (N, r, H2):
            raise ValueError("shape mismatch between x, W and the stacks")
        bp = None
        if bias is not None:
            bias = self._f32(bias)
            if bias.shape != (H2,):
                raise ValueError("bias must be [H2]")
            bp = self._ptr(bias, ctypes.c_float)
        y = np.empty((R, H2))
        rc = self.lib.sgmv_oracle_lora_linear(
            self._ptr(y, ctypes.c_double), self._ptr(x, ctypes.c_float),
            self._ptr(W, ctypes.c_float), bp, self._ptr(A, ctypes.c_float),
            self._ptr(B, ctypes.c_float), self._ptr(seg, _i32), self._ptr(ids, _i32),
            ids.shape[0], R, N, H1, H2, r, float(scale))
        if rc:
            raise ValueError("oracle rejected the segment table or shapes")
        return y


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default


def shrink(*args, **kwargs):
    return get().shrink(*args, **kwargs)


def expand(*args, **kwargs):
    return get().expand(*args, **kwargs)


def lora_apply(*args, **kwargs):
    return get().lora_apply(*args, **kwargs)


def lora_linear(*args, **kwargs):
    return get().lora_linear(*args, **kwargs)
