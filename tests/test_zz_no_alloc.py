"""lora_apply_noalloc (no workspace argument: the library's static per-GPU
scratch) against lora_apply with a caller-owned workspace, through the C
ABI: two calls in a row, the second smaller, each bit for bit equal to
lora_apply and within the parity bound of the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import assert_close, to_device, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU (run with -m 'not gpu' on CPU)"
    import segmented_gather_gemv_sgmv_amd as sg
    sg.lib()


def _args(w, d, y):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    return (y.data_ptr(), d["x"].data_ptr(), d["A"].data_ptr(), d["B"].data_ptr(),
            d["seg"].data_ptr(), d["ids"].data_ptr(), w.num_segments, w.num_rows,
            w.num_adapters, w.H1, w.H2, w.r, ctypes.c_float(w.scale),
            sg.dtype_code(torch_dtype(w.dtype)))


def _with_workspace(w, d):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    lib = sg.lib()
    y = d["y0"].clone()
    dt = sg.dtype_code(torch_dtype(w.dtype))
    need = lib.lora_apply_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.H2, w.r, dt)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.lora_apply(*_args(w, d, y), ws.data_ptr(), need, st)
    assert rc == 0, sg.STATUS.get(rc, rc)
    torch.cuda.synchronize()
    return y


def _noalloc(w, d):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    lib = sg.lib()
    y = d["y0"].clone()
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.lora_apply_noalloc(*_args(w, d, y), st)
    assert rc == 0, sg.STATUS.get(rc, rc)
    torch.cuda.synchronize()
    return y


CALL_PAIRS = {
    # decode vector kernel, then a smaller decode call
    "decode_then_smaller": (lambda: wl.llama7b_decode(0),
                            lambda: wl.small_random(81, "f16", 4096, 4096, 16, 64, 20, 20)),
    # row-heavy MFMA path (two launches), then a smaller row-heavy call
    "prefill_then_smaller": (lambda: wl.prefill(0),
                             lambda: wl.small_random(82, "bf16", 2048, 1024, 64, 6, 700, 5)),
    # a mixed batch, then a tiny float32 call
    "mixed_then_tiny": (lambda: wl.mixed_batch(0), lambda: wl.tiny(0)),
}


@pytest.mark.parametrize("case", list(CALL_PAIRS))
def test_noalloc_equals_lora_apply(case):
    for make in CALL_PAIRS[case]:
        w = make()
        print(f"noalloc {case}: {w.name}", flush=True)
        d = to_device(w)
        ref = _with_workspace(w, d)
        got = _noalloc(w, d)
        assert torch_equal(got, ref), f"{w.name}: lora_apply_noalloc differs from lora_apply"
        if w.num_rows * w.H2 <= 1 << 22:
            y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids,
                                         w.scale)
            mag = None
            if w.dtype == "f32":
                from gpu_helpers import magnitude
                mag = magnitude(w)[0]
            assert_close(got.double().cpu().numpy(), y_ref, w.dtype, w.name, mag)


def torch_equal(a, b):
    import torch
    return bool(torch.equal(a, b))


def test_noalloc_in_a_graph_replays():
    """Captured as it stands (nothing to allocate): every replay, with eager
    noalloc calls of another shape in between, equals the eager result."""
    import torch
    w = wl.skewed_decode(0)
    d = to_device(w)
    ref = _with_workspace(w, d)
    other = wl.small_random(83, "f16", 1024, 2048, 16, 8, 48, 12)
    do = to_device(other)
    ref_other = _with_workspace(other, do)
    import segmented_gather_gemv_sgmv_amd as sg
    y = d["y0"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sg.lora_apply_noalloc(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sg.lora_apply_noalloc(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale)
    for rep in range(3):
        y.copy_(d["y0"])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"
        yo = do["y0"].clone()
        sg.lora_apply_noalloc(yo, do["x"], do["A"], do["B"], do["seg"], do["ids"], other.scale)
        torch.cuda.synchronize()
        assert torch.equal(yo, ref_other), f"eager call after replay {rep}"
