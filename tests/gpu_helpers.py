"""Shared helpers for the GPU parity tests: move a workload to the device,
run the HIP library, and compare with the oracle under the stated bounds.

Tolerances (elementwise, against the oracle's double-precision result):
  fp16 / bf16 inputs, fp32 accumulation:  |gpu - ref| <= 1e-2 + 1e-2 * |ref|
  fp32 inputs:                            |gpu - ref| <= 1e-5 + 1e-5 * |ref|
"""
from __future__ import annotations

import numpy as np

TOL = {"f16": 1e-2, "bf16": 1e-2, "f32": 1e-5}


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def to_device(w, device="cuda:0"):
    """Device copies of a workload's arrays (exact: values are dtype-rounded)."""
    import torch
    dt = torch_dtype(w.dtype)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(dt)
    return dict(
        x=t(w.x), A=t(w.A), B=t(w.B), y0=t(w.y0),
        seg=torch.from_numpy(w.seg_indptr.astype(np.int32)).to(device),
        ids=torch.from_numpy(w.adapter_ids.astype(np.int32)).to(device),
    )


def gpu_lora_apply(w, d=None, device="cuda:0"):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    d = to_device(w, device) if d is None else d
    y = d["y0"].clone()
    sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale)
    torch.cuda.synchronize()
    return y.double().cpu().numpy()


def gpu_shrink(w, d=None, device="cuda:0", fill=0.0):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    d = to_device(w, device) if d is None else d
    v = torch.full((w.num_rows, w.r), fill, dtype=torch.float32, device=device)
    sg.sgmv_shrink(v, d["x"], d["A"], d["seg"], d["ids"])
    torch.cuda.synchronize()
    return v.double().cpu().numpy()


def gpu_expand(w, v, d=None, device="cuda:0"):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    d = to_device(w, device) if d is None else d
    y = d["y0"].clone()
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device)
    sg.sgmv_expand(y, vt, d["B"], d["seg"], d["ids"], w.scale)
    torch.cuda.synchronize()
    return y.double().cpu().numpy()


def assert_close(got, ref, dtype, what=""):
    tol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = tol + tol * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance; worst at {i}: "
            f"got {got[i]!r}, ref {ref[i]!r}, err {err[i]:.3e} > {bound[i]:.3e}")
    return float((err / bound).max()) if err.size else 0.0
