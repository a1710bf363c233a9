"""lora_apply_multi: several add-ons over one batch in one call, against the
oracle per problem, and against one lora_apply per problem where it takes
that route."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import assert_close, magnitude, to_device

pytestmark = pytest.mark.gpu


def _problems(seed, dtype, shapes, r, N, R, S, allow_empty=True):
    """Workloads sharing one segment table (that of the first)."""
    ws = [wl.small_random(seed + k, dtype, H1, H2, r, N, R, S, allow_empty=allow_empty)
          for k, (H1, H2) in enumerate(shapes)]
    for w in ws[1:]:
        w.seg_indptr, w.adapter_ids = ws[0].seg_indptr, ws[0].adapter_ids
    return ws


def _run(ws, workspace=None):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    ds = [to_device(w) for w in ws]
    ys = [d["y0"].clone() for d in ds]
    sg.lora_apply_multi([(y, d["x"], d["A"], d["B"], w.scale) for y, d, w in zip(ys, ds, ws)],
                        ds[0]["seg"], ds[0]["ids"], workspace=workspace)
    torch.cuda.synchronize()
    return [y.double().cpu().numpy() for y in ys]


CASES = {
    # decode: one launch (q, k, v, o-like shapes)
    "decode_qkvo_f16": ("f16", [(1024, 1024), (1024, 512), (1024, 512), (1024, 1024)], 16, 64,
                        64, 64),
    "decode_mixed_bf16_r64": ("bf16", [(640, 1728), (1728, 640)], 64, 40, 96, 60),
    "decode_f32_r8_8probs": ("f32", [(256, 192)] * 8, 8, 6, 50, 30),
    # row-heavy: one lora_apply per problem (MFMA tiles)
    "prefill_two_f16": ("f16", [(1024, 1024), (1024, 2048)], 16, 4, 600, 4),
}


@pytest.mark.parametrize("case", list(CASES))
def test_multi_matches_oracle(case):
    dtype, shapes, r, N, R, S = CASES[case]
    ws = _problems(len(case), dtype, shapes, r, N, R, S)
    got = _run(ws)
    for k, (w, y) in enumerate(zip(ws, got)):
        y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
        assert_close(y, y_ref, dtype, f"{case} problem {k}", magnitude(w)[0])


def test_multi_row_heavy_equals_separate_calls():
    """Row-heavy calls run one lora_apply per problem: bit for bit the same."""
    from gpu_helpers import gpu_lora_apply
    dtype, shapes, r, N, R, S = CASES["prefill_two_f16"]
    ws = _problems(3, dtype, shapes, r, N, R, S)
    got = _run(ws)
    for w, y in zip(ws, got):
        assert np.array_equal(y, gpu_lora_apply(w))


def test_multi_self_contained_path_is_bit_identical():
    """Zero patience: every expand item recomputes its partials; the output
    is bit-identical, the sticky flag is set and the counters end at zero."""
    import ctypes
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    dtype, shapes, r, N, R, S = CASES["decode_qkvo_f16"]
    ws = _problems(5, dtype, shapes, r, N, R, S)
    probe = [sg.LoraProblem(None, None, None, None, H1, H2, 1.0) for H1, H2 in shapes]
    arr = (sg.LoraProblem * len(probe))(*probe)
    need = sg.lib().lora_apply_multi_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p),
                                                     len(probe), R, S, r, 1)
    ws_buf = torch.zeros(need, dtype=torch.uint8, device="cuda")
    normal = _run(ws, ws_buf)
    counters = ws_buf[:262144].view(torch.int32)
    assert int(counters.abs().sum()) == 0
    try:
        sg.set_fused_wait(0.0)
        alone = _run(ws, ws_buf)
    finally:
        sg.set_fused_wait(0.02)
    assert all(np.array_equal(a, b) for a, b in zip(normal, alone))
    assert int(counters[-1]) == 1
    assert int(counters[:-1].abs().sum()) == 0


def test_multi_argument_errors():
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    dtype, shapes, r, N, R, S = CASES["decode_qkvo_f16"]
    ws = _problems(9, dtype, shapes[:2], r, N, R, S)
    ds = [to_device(w) for w in ws]
    with pytest.raises(ValueError):
        sg.lora_apply_multi([], ds[0]["seg"], ds[0]["ids"])
    with pytest.raises(ValueError):  # x rows disagree
        sg.lora_apply_multi([(ds[0]["y0"], ds[0]["x"][:10], ds[0]["A"], ds[0]["B"], 1.0)],
                            ds[0]["seg"], ds[0]["ids"])
