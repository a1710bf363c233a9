"""Device segment builders (sgmv_build_segments, sgmv_group_rows) against
the oracle, bit for bit, and lora_apply driven by their tables against the
oracle applied to the grouped batch."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import assert_close, to_device
from oracle import segments as og

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "segments_hand_worked.json")


def _cases():
    g = json.load(open(GOLDEN))
    rng = np.random.default_rng(11)
    out = [("golden", g["row_ids"], g["num_adapters"]), ("empty", [], 3), ("one", [2], 3),
           ("one_invalid", [9], 3)]
    for R, N in [(1023, 5), (1024, 64), (1025, 64), (2049, 7), (3000, 600), (5000, 4096)]:
        out.append((f"random_{R}_{N}", rng.integers(-3, N + 3, size=R).tolist(), N))
        out.append((f"sorted_{R}_{N}", np.sort(rng.integers(0, N, size=R)).tolist(), N))
    out.append(("all_same_2000", [5] * 2000, 8))
    out.append(("all_distinct_1500", list(range(1500)), 1500))
    return out


CASES = _cases()


def _dev(ids):
    import torch
    return torch.tensor(np.asarray(ids, dtype=np.int32), dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("case", [c[0] for c in CASES])
def test_build_segments_matches_oracle(case):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    _, row_ids, N = next(c for c in CASES if c[0] == case)
    seg, ids, count = sg.build_segments(_dev(row_ids), N)
    torch.cuda.synchronize()
    e_seg, e_ids, e_count = og.build_segments(row_ids, N)
    assert seg.cpu().tolist() == e_seg
    assert ids.cpu().tolist() == e_ids
    assert int(count.item()) == e_count


@pytest.mark.parametrize("case", [c[0] for c in CASES])
def test_group_rows_matches_oracle(case):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    _, row_ids, N = next(c for c in CASES if c[0] == case)
    perm, seg, ids, count = sg.group_rows(_dev(row_ids), N)
    torch.cuda.synchronize()
    e_perm, e_seg, e_ids, e_count = og.group_rows(row_ids, N)
    assert perm.cpu().tolist() == e_perm
    assert seg.cpu().tolist() == e_seg
    assert ids.cpu().tolist() == e_ids
    assert int(count.item()) == e_count


def test_group_rows_rejects_too_many_adapters():
    import segmented_gather_gemv_sgmv_amd as sg
    with pytest.raises(sg.SGMVError) as e:
        sg.group_rows(_dev([0, 1]), 4097)
    assert e.value.code == 4


def _reference(w, row_ids, absolute=False):
    """The oracle on the batch grouped by the (pinned) oracle grouping, with
    the rows put back in place; rows without an adapter keep y0.  With
    ``absolute``, the oracle on the inputs' absolute values (the magnitude
    of each element's terms)."""
    f = np.abs if absolute else (lambda a: a)
    perm, seg, aid, count = og.group_rows(row_ids, w.num_adapters)
    perm = np.asarray(perm)
    y_g, _ = oracle.lora_apply(f(w.y0[perm]), f(w.x[perm]), f(w.A), f(w.B),
                               np.asarray(seg[:count + 1], dtype=np.int32),
                               np.asarray(aid[:count], dtype=np.int32), f(w.scale))
    y = np.empty_like(y_g)
    y[perm] = y_g
    return y


@pytest.mark.parametrize("dtype,H1,H2,r,N,R", [("f16", 512, 768, 16, 6, 300),
                                               ("bf16", 1024, 512, 64, 9, 700),
                                               ("f32", 256, 384, 8, 5, 130)])
def test_lora_apply_from_per_row_ids(dtype, H1, H2, r, N, R):
    """Per-row adapter ids -> device table -> lora_apply, both ways: the run
    table over the batch as it is, and the grouped table over the batch
    reordered by perm; rows whose id is not an adapter stay untouched."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(51 + R, dtype, H1, H2, r, N, R, 1)
    rng = np.random.default_rng(R)
    row_ids = rng.integers(-1, N + 1, size=R)
    row_ids[: R // 3] = np.sort(row_ids[: R // 3])  # some long runs too
    y_ref = _reference(w, row_ids.tolist())
    mag = _reference(w, row_ids.tolist(), absolute=True)
    d = to_device(w)
    rid = _dev(row_ids)

    seg, ids, _ = sg.build_segments(rid, N)
    y = d["y0"].clone()
    sg.lora_apply(y, d["x"], d["A"], d["B"], seg, ids, w.scale)
    torch.cuda.synchronize()
    assert_close(y.double().cpu().numpy(), y_ref, dtype, "run table", mag)

    perm, seg, ids, _ = sg.group_rows(rid, N)
    p = perm.long()
    yg = d["y0"].index_select(0, p).contiguous()
    sg.lora_apply(yg, d["x"].index_select(0, p).contiguous(), d["A"], d["B"], seg, ids, w.scale)
    y = torch.empty_like(yg)
    y[p] = yg
    torch.cuda.synchronize()
    assert_close(y.double().cpu().numpy(), y_ref, dtype, "grouped table", mag)
    invalid = (row_ids < 0) | (row_ids >= N)
    assert np.array_equal(y.double().cpu().numpy()[invalid], w.y0[invalid].astype(np.float64))


@pytest.mark.parametrize("group", [False, True, "auto"], ids=["runs", "grouped", "auto"])
def test_lora_linear_module(group):
    """LoRALinear = torch's dense linear for the base product plus the SGMV
    add-on for per-row adapters: its output equals the oracle's add-on
    applied to that same base output."""
    import torch
    from segmented_gather_gemv_sgmv_amd.lora_linear import LoRALinear
    R, H1, H2, r, N = 96, 512, 384, 16, 5
    w = wl.small_random(77, "f16", H1, H2, r, N, R, 1)
    rng = np.random.default_rng(5)
    weight = torch.tensor(rng.normal(0, 0.05, size=(H2, H1)), dtype=torch.float16, device="cuda")
    bias = torch.tensor(rng.normal(0, 1, size=H2), dtype=torch.float16, device="cuda")
    row_ids = rng.integers(-1, N, size=R)
    d = to_device(w)
    layer = LoRALinear(weight, d["A"], d["B"], scale=w.scale, bias=bias, group=group)
    y = layer(d["x"], _dev(row_ids))
    base = torch.nn.functional.linear(d["x"], weight, bias)
    torch.cuda.synchronize()
    wb = wl.Workload(w.name, w.dtype, H1, H2, r, N, w.seg_indptr, w.adapter_ids, w.scale, w.x,
                     w.A, w.B, base.float().cpu().numpy())
    y_ref = _reference(wb, row_ids.tolist())
    assert_close(y.double().cpu().numpy(), y_ref, "f16", "LoRALinear")
