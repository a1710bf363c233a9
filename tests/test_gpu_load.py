"""On-demand adapter loading (sgmv_load_adapter): host adapters copied into
stack slots arrive bit for bit, and lora_apply over them matches the oracle."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import assert_close, magnitude, to_device, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,r", [("f16", 16), ("bf16", 64), ("f32", 8)])
def test_load_then_apply(dtype, r):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(61, dtype, 512, 768, r, 6, 40, 8, allow_empty=False)
    td = torch_dtype(dtype)
    d = to_device(w)
    A_dev = torch.zeros_like(d["A"])
    B_dev = torch.zeros_like(d["B"])
    # load the slots in a scrambled order from pinned host copies
    for slot in [3, 0, 5, 1, 4, 2]:
        hA = torch.empty(w.H1, r, dtype=td, pin_memory=True)
        hB = torch.empty(r, w.H2, dtype=td, pin_memory=True)
        hA.copy_(torch.from_numpy(w.A[slot]).to(td))
        hB.copy_(torch.from_numpy(w.B[slot]).to(td))
        sg.load_adapter(A_dev, B_dev, slot, hA, hB)
        torch.cuda.synchronize()  # the host buffers go out of scope next
    assert torch.equal(A_dev, d["A"]) and torch.equal(B_dev, d["B"])
    # several consecutive slots in one call
    A2 = torch.zeros_like(d["A"])
    B2 = torch.zeros_like(d["B"])
    hA = torch.empty(tuple(d["A"].shape), dtype=td, pin_memory=True)
    hB = torch.empty(tuple(d["B"].shape), dtype=td, pin_memory=True)
    hA.copy_(torch.from_numpy(w.A).to(td))
    hB.copy_(torch.from_numpy(w.B).to(td))
    sg.load_adapter(A2, B2, 1, hA[1:5], hB[1:5])
    torch.cuda.synchronize()
    assert torch.equal(A2[1:5], d["A"][1:5]) and torch.equal(B2[1:5], d["B"][1:5])
    assert int(A2[0].abs().sum()) == 0 and int(A2[5].abs().sum()) == 0
    y = d["y0"].clone()
    sg.lora_apply(y, d["x"], A_dev, B_dev, d["seg"], d["ids"], w.scale)
    torch.cuda.synchronize()
    y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    assert_close(y.double().cpu().numpy(), y_ref, dtype, f"loaded {dtype}", magnitude(w)[0])


def test_load_adapter_shape_errors():
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    A_dev = torch.zeros(4, 64, 8, dtype=torch.float16, device="cuda")
    B_dev = torch.zeros(4, 8, 32, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        sg.load_adapter(A_dev, B_dev, 0, torch.zeros(64, 4, dtype=torch.float16),
                        torch.zeros(8, 32, dtype=torch.float16))
    with pytest.raises(sg.SGMVError):
        sg.load_adapter(A_dev, B_dev, 4, torch.zeros(64, 8, dtype=torch.float16),
                        torch.zeros(8, 32, dtype=torch.float16))
