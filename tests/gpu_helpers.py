"""Shared helpers for the GPU parity tests: move a workload to the device,
run the HIP library, and compare with the oracle under the stated bounds.

Tolerances (elementwise, against the oracle's double-precision result):
  fp16 / bf16 inputs, fp32 accumulation:  |gpu - ref| <= 1e-2 + 1e-2 * |ref|
  fp32 inputs:                            |gpu - ref| <= 1e-5 * m
where m is the magnitude of the terms summed into that element: the same
oracle evaluated on the absolute values of every input (and of the scale),
m = |y0| + |s| sum_k (sum_h |x_h| |A_hk|) |B_kj| for y and
m = sum_h |x_h| |A_hk| for v.  m >= |ref|, and m = |ref| when no terms
cancel, so this is the stated "1e-5 relative" bound, taken relative to the
size of the sum rather than of its (possibly cancelled) value.
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


COUNTER_BYTES = 65536 * 4  # the workspace's counter region (include/sgmv.h)


def gpu_lora_apply(w, d=None, device="cuda:0"):
    """lora_apply on a fresh zeroed workspace.  Afterwards the tile counters
    must be back at zero and the sticky flag (last int of the counter region:
    an expand workgroup gave up waiting for its shrink workgroups) must still
    be clear: at the default patience the hand-off never falls back."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    d = to_device(w, device) if d is None else d
    y = d["y0"].clone()
    need = sg.lora_apply_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.H2, w.r,
                                         torch_dtype(w.dtype))
    ws = torch.zeros(max(need, COUNTER_BYTES), dtype=torch.uint8, device=device)
    sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale, workspace=ws)
    torch.cuda.synchronize()
    counters = ws[:COUNTER_BYTES].view(torch.int32)
    assert int(counters[-1].item()) == 0, "a fused expand workgroup fell back (sticky flag set)"
    assert int(counters[:-1].abs().sum().item()) == 0, "tile counters not returned to zero"
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


def magnitude(w, seg=None, ids=None):
    """(m_y, m_v): the oracle's lora_apply on the absolute values of y0, x,
    A, B and the scale, i.e. the magnitude of the terms of each element of
    y and of v."""
    import oracle
    seg = w.seg_indptr if seg is None else seg
    ids = w.adapter_ids if ids is None else ids
    return oracle.lora_apply(np.abs(w.y0), np.abs(w.x), np.abs(w.A), np.abs(w.B), seg, ids,
                             abs(w.scale))


def magnitude_expand(w, v):
    """Magnitude of the terms of y when expand is fed v."""
    import oracle
    return oracle.expand(np.abs(w.y0), np.abs(np.asarray(v, np.float64)).astype(np.float32),
                         np.abs(w.B), w.seg_indptr, w.adapter_ids, abs(w.scale))


def assert_close(got, ref, dtype, what="", mag=None):
    """Elementwise check under the bound of `dtype` (see the module notes);
    fp32 needs `mag`, the magnitude of each element's terms."""
    tol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == "f32":
        if mag is None:
            raise TypeError(f"{what}: a float32 comparison needs the terms' magnitude (mag=)")
        mag = np.asarray(mag, dtype=np.float64)
        assert mag.shape == ref.shape, (mag.shape, ref.shape)
        bound = tol * mag
    else:
        bound = tol + tol * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance; worst at {i}: "
            f"got {got[i]!r}, ref {ref[i]!r}, err {err[i]:.3e} > {bound[i]:.3e}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), 0.0)
    return float(ratio.max()) if err.size else 0.0
