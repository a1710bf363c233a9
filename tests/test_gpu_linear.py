"""GPU parity of lora_linear (the adapted linear layer with the base product
fused in) against the fp64 CPU oracle.

y = x W^T + bias + scale * (x A_a) B_a per row of each segment, base product
only elsewhere; tolerances as for the add-on (tests/gpu_helpers.py).  The
cases reach the three tile shapes of the matrix-core kernels (64 x 64 tiles
whose K range is split over workgroups, 128 x 128 tiles, and 256 x 256 tiles
for many rows), ragged row, column and K tails, and the element-wise kernel (float32, misaligned pointers,
sizes not a multiple of 8).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import COUNTER_BYTES, assert_close, to_device, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import segmented_gather_gemv_sgmv_amd as sg
    sg.lib()  # fails loudly if the HIP library is missing


def _dev(a, dtype, device="cuda:0"):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(torch_dtype(dtype))


def _gpu_linear(w, W, b, d=None, seg=None, ids=None, expect_flag=0):
    """lora_linear on a fresh zeroed workspace.  Afterwards every counter
    (the split-K tile counters and the folded shrink's) must be back at zero
    and the sticky flag (a folded workgroup gave up waiting for the others'
    shares of v) must read `expect_flag`."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    d = to_device(w) if d is None else d
    seg = d["seg"] if seg is None else seg
    ids = d["ids"] if ids is None else ids
    need = sg.lora_linear_workspace_bytes(w.num_rows, int(seg.numel()) - 1, w.H1, w.H2, w.r,
                                          torch_dtype(w.dtype))
    ws = torch.zeros(max(need, COUNTER_BYTES), dtype=torch.uint8, device="cuda:0")
    y = sg.lora_linear(d["x"], _dev(W, w.dtype), d["A"], d["B"], seg, ids, w.scale,
                       bias=_dev(b, w.dtype), workspace=ws)
    torch.cuda.synchronize()
    counters = ws[:COUNTER_BYTES].view(torch.int32)
    assert int(counters[-1].item()) == expect_flag, "sticky flag"
    assert int(counters[:-1].abs().sum().item()) == 0, "counters not returned to zero"
    return y.double().cpu().numpy()


def _oracle(w, W, b, seg=None, ids=None, absolute=False):
    """The oracle's adapted layer; with ``absolute``, on the inputs' absolute
    values (the magnitude of each element's terms, for the float32 bound)."""
    seg = w.seg_indptr if seg is None else seg
    ids = w.adapter_ids if ids is None else ids
    f = np.abs if absolute else (lambda a: a)
    return oracle.lora_linear(f(w.x), f(W), None if b is None else f(b), f(w.A), f(w.B), seg,
                              ids, f(w.scale))


# (seed, dtype, H1, H2, r, N, R, S, uncovered tail, bias)
CASES = [
    (1, "f16", 256, 256, 16, 8, 64, 64, 0, True),     # decode: 64 x 64 tiles, split K
    (2, "bf16", 512, 328, 16, 6, 37, 9, 5, True),     # ragged rows and columns
    (3, "f16", 328, 200, 32, 5, 50, 7, 0, False),     # K tail inside a chunk, no bias
    (4, "f16", 264, 520, 64, 4, 200, 6, 11, True),    # 128 x 128 tiles, ragged tails
    (5, "bf16", 1024, 384, 128, 3, 130, 3, 0, True),  # square tiles, r = 128
    (6, "f16", 640, 136, 8, 9, 300, 40, 3, True),     # many segments per tile
    (7, "f16", 96, 64, 5, 4, 20, 5, 2, True),         # odd rank
    (8, "f32", 72, 40, 8, 4, 19, 4, 3, True),         # float32: element-wise kernel
    (9, "f16", 100, 60, 4, 3, 10, 3, 0, True),        # H1 % 8 != 0: element-wise kernel
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_random_shapes(case):
    seed, dtype, H1, H2, r, N, R, S, tail, bias = case
    w = wl.small_random(seed, dtype, H1, H2, r, N, R, S, uncovered_tail=tail)
    W, b = wl.base_layer(seed, dtype, H1, H2, bias=bias)
    print(f"lora_linear {case}", flush=True)
    assert_close(_gpu_linear(w, W, b), _oracle(w, W, b), dtype, str(case),
                 _oracle(w, W, b, absolute=True))


@pytest.mark.parametrize("dtype,R,H1,H2,r", [("f16", 64, 256, 128, 16), ("bf16", 150, 192, 264, 8),
                                             ("f16", 33, 128, 72, 64)])
def test_integer_inputs_match_bit_for_bit(dtype, R, H1, H2, r):
    w = wl.integer_exact(11, dtype, H1, H2, r, 5, R, 6, density=0.2, scale=2.0)
    W, b = wl.base_layer(11, dtype, H1, H2, integer=True, density=0.2)
    ref = _oracle(w, W, b)
    limit = 2048 if dtype == "f16" else 256
    assert np.abs(ref).max() <= limit, "inputs leave the exactly representable range"
    got = _gpu_linear(w, W, b)
    assert np.array_equal(got, ref)


def test_without_segments_is_the_base_layer():
    import torch
    w = wl.small_random(12, "f16", 256, 192, 16, 4, 80, 4)
    W, b = wl.base_layer(12, "f16", 256, 192)
    d = to_device(w)
    empty_seg = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    empty_ids = torch.zeros(0, dtype=torch.int32, device="cuda:0")
    got = _gpu_linear(w, W, b, d, empty_seg, empty_ids)
    ref = _oracle(w, W, b, np.zeros(1, np.int32), np.zeros(0, np.int32))
    assert_close(got, ref, "f16", "no segments")


@pytest.mark.parametrize("rows", [40, 150], ids=["skinny_tiles", "square_tiles"])
def test_c_abi_no_segments_null_tables(rows):
    """num_segments == 0 with NULL seg_indptr, adapter_ids and stacks, as the
    header allows, through the matrix-core tiles (fp16, sizes multiples of 8,
    aligned pointers): the kernel must read no table and return the base
    layer."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    H1, H2 = 256, 192
    w = wl.small_random(21, "f16", H1, H2, 16, 2, rows, 2)
    W, b = wl.base_layer(21, "f16", H1, H2)
    x = _dev(w.x, "f16")
    Wd = _dev(W, "f16")
    bd = _dev(b, "f16")
    y = torch.full((rows, H2), 7.0, dtype=torch.float16, device="cuda:0")
    lib = sg.lib()
    need = int(lib.lora_linear_workspace_bytes(rows, 0, H1, H2, 16, sg.SGMV_F16))
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda:0")
    rc = lib.lora_linear(y.data_ptr(), x.data_ptr(), Wd.data_ptr(), bd.data_ptr(), None, None,
                         None, None, 0, rows, 0, H1, H2, 16, 2.0, sg.SGMV_F16, ws.data_ptr(),
                         ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, sg.STATUS.get(rc, rc)
    torch.cuda.synchronize()
    ref = _oracle(w, W, b, np.zeros(1, np.int32), np.zeros(0, np.int32))
    assert_close(y.double().cpu().numpy(), ref, "f16", "S=0, NULL tables")


def test_invalid_adapter_rows_get_the_base_product():
    import torch
    w = wl.small_random(13, "f16", 128, 128, 16, 4, 40, 4, allow_empty=False)
    W, b = wl.base_layer(13, "f16", 128, 128)
    ids = w.adapter_ids.copy()
    ids[1], ids[3] = -1, 4  # -1 and N = 4 name no adapter
    got = _gpu_linear(w, W, b, ids=torch.from_numpy(ids).to("cuda:0"))
    ref = _oracle(w, W, b)  # the valid table: right for segments 0 and 2
    ref_base = _oracle(w, W, b, np.zeros(1, np.int32), np.zeros(0, np.int32))
    for s in range(4):
        lo, hi = int(w.seg_indptr[s]), int(w.seg_indptr[s + 1])
        want = ref[lo:hi] if s in (0, 2) else ref_base[lo:hi]
        assert_close(got[lo:hi], want, "f16", f"segment {s}")


def test_misaligned_pointers_take_general_path():
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(14, "f16", 64, 48, 8, 3, 12, 3)
    W, b = wl.base_layer(14, "f16", 64, 48)
    d = to_device(w)
    big = torch.zeros(12 * 64 + 1, dtype=torch.float16, device="cuda:0")
    xo = big[1:].view(12, 64)
    xo.copy_(d["x"])
    y = sg.lora_linear(xo, _dev(W, "f16"), d["A"], d["B"], d["seg"], d["ids"], w.scale,
                       bias=_dev(b, "f16"))
    torch.cuda.synchronize()
    assert_close(y.double().cpu().numpy(), _oracle(w, W, b), "f16", "misaligned x")


def test_decode_full_size_against_oracle():
    """The decode layer at its real size: 64 one-row segments, H = 4096, r = 16."""
    w = wl.llama7b_decode(0)
    W, b = wl.base_layer(0, w.dtype, w.H1, w.H2, bias=False)
    print("lora_linear decode 64 x 4096 x 4096", flush=True)
    assert_close(_gpu_linear(w, W, b), _oracle(w, W, b), w.dtype, "decode")


def test_prefill_full_size_sampled_rows():
    """Prefill at its real size (4096 rows, 16 segments); the oracle checks
    every fourth segment's first and last rows and 40 rows spread over the
    batch, each as a one-row problem with its segment's adapter."""
    w = wl.prefill(0)
    W, b = wl.base_layer(0, w.dtype, w.H1, w.H2)
    print("lora_linear prefill 4096 x 4096 x 4096", flush=True)
    got = _gpu_linear(w, W, b)
    seg, ids = w.seg_indptr, w.adapter_ids
    rows = set(np.linspace(0, w.num_rows - 1, 40).astype(int).tolist())
    for s in range(0, len(ids), 4):
        rows |= {int(seg[s]), int(seg[s + 1]) - 1}
    for i in sorted(rows):
        s = int(np.searchsorted(seg, i, side="right") - 1)
        ref = oracle.lora_linear(w.x[i:i + 1], W, b, w.A, w.B, np.array([0, 1], np.int32),
                                 ids[s:s + 1], w.scale)
        assert_close(got[i:i + 1], ref, w.dtype, f"row {i}")


@pytest.mark.parametrize("dtype,R,H1,H2,r", [("f16", 64, 256, 256, 16), ("bf16", 37, 512, 328, 16),
                                             ("f16", 20, 1024, 200, 32), ("bf16", 9, 2048, 64, 64)])
def test_folded_shrink_fallback_is_bit_identical(dtype, R, H1, H2, r):
    """Decode shapes fold the shrink into the tile launch: each workgroup
    publishes a share of v and waits for the others' before its correction.
    With no patience every workgroup recomputes its v itself; the result
    must be the same bits, the sticky flag set and the counters back at
    zero."""
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(31, dtype, H1, H2, r, 6, R, max(1, R // 2))
    W, b = wl.base_layer(31, dtype, H1, H2)
    d = to_device(w)
    normal = _gpu_linear(w, W, b, d)
    try:
        sg.set_fused_wait(0.0)
        alone = _gpu_linear(w, W, b, d, expect_flag=1)
    finally:
        sg.set_fused_wait(0.02)
    assert np.array_equal(normal, alone)
    assert_close(normal, _oracle(w, W, b), dtype, "folded", _oracle(w, W, b, absolute=True))


def test_prefill_tiling_every_row():
    """Every row of the prefill batch (4096 rows, the same 16 segments and
    adapters, 128 x 128 tiles) against the oracle, at H1 = 1024 and H2 = 512
    so that the oracle finishes in seconds: the row tiling, the segment
    boundaries inside tiles and the ragged last tile are those of the
    full-size layer, only the K and column extents are shorter."""
    full = wl.prefill(0)
    lengths = np.diff(full.seg_indptr)
    w = wl.make_workload("prefill_tiling_4096x1024x512", "f16", 1024, 512, 16, 16, lengths,
                         full.adapter_ids, 2.0, rng=np.random.default_rng(7))
    W, b = wl.base_layer(7, w.dtype, w.H1, w.H2)
    print("lora_linear prefill tiling 4096 x 1024 -> 512", flush=True)
    assert_close(_gpu_linear(w, W, b), _oracle(w, W, b), w.dtype, "prefill tiling",
                 _oracle(w, W, b, absolute=True))


# 256 x 256 tiles (linear_wide_kernel): at least 128 tiles and segments of
# 32 or more rows on average.  H1 a multiple of 128 takes the direct-load
# stages (cases 42, 43, 44, 47), other H1 the register-staged chunks.  (seed, dtype, H1, H2, r, N, R, S, uncovered
# tail, bias)
WIDE_CASES = [
    (41, "f16", 264, 4088, 16, 8, 2000, 12, 7, True),   # ragged rows, columns, K chunk
    (42, "bf16", 256, 4096, 16, 6, 2048, 16, 0, True),  # bf16
    (43, "f16", 128, 2048, 40, 5, 4096, 24, 0, False),  # rank passes 16 + 16 + 8, no bias
    (44, "bf16", 128, 4096, 128, 3, 2100, 4, 30, True),  # r = 128, uncovered tail rows
    (46, "f16", 64, 2048, 16, 8, 16640, 520, 0, True),   # table past LDS (520 segments)
    (47, "bf16", 256, 4040, 32, 6, 2000, 10, 5, True),   # direct-load stages, ragged rows and columns
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_wide_tiles_every_element(case):
    """Every element of the 256 x 256 tile path against the oracle, and a
    second call bit for bit equal to the first."""
    seed, dtype, H1, H2, r, N, R, S, tail, bias = case
    w = wl.small_random(seed, dtype, H1, H2, r, N, R, S, uncovered_tail=tail)
    W, b = wl.base_layer(seed, dtype, H1, H2, bias=bias)
    d = to_device(w)
    print(f"lora_linear wide tiles {case}", flush=True)
    got = _gpu_linear(w, W, b, d)
    assert_close(got, _oracle(w, W, b), dtype, str(case), _oracle(w, W, b, absolute=True))
    assert np.array_equal(_gpu_linear(w, W, b, d), got)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_wide_tiles_integer_inputs_bit_for_bit(dtype):
    """Exact integers through the 256 x 256 tiles: the correction's bf16
    terms of v (and, for fp16, of the weights) add up exactly, so y must
    equal the oracle's value bit for bit."""
    w = wl.integer_exact(11, dtype, 64, 4096, 16, 5, 2048, 6, density=0.2, scale=2.0)
    W, b = wl.base_layer(11, dtype, 64, 4096, integer=True, density=0.2)
    ref = _oracle(w, W, b)
    limit = 2048 if dtype == "f16" else 256
    assert np.abs(ref).max() <= limit, "inputs leave the exactly representable range"
    assert np.array_equal(_gpu_linear(w, W, b), ref)


def test_wide_tiles_invalid_adapters_and_null_tables():
    """Segments naming no adapter get the base product; with no segments and
    NULL tables the wide tiles return the base layer."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(45, "f16", 128, 4096, 16, 4, 2048, 6, allow_empty=False)
    W, b = wl.base_layer(45, "f16", 128, 4096)
    ids = w.adapter_ids.copy()
    ids[1], ids[4] = -1, 4
    got = _gpu_linear(w, W, b, ids=torch.from_numpy(ids).to("cuda:0"))
    ref = _oracle(w, W, b)
    ref_base = _oracle(w, W, b, np.zeros(1, np.int32), np.zeros(0, np.int32))
    for s in range(6):
        lo, hi = int(w.seg_indptr[s]), int(w.seg_indptr[s + 1])
        want = ref_base[lo:hi] if s in (1, 4) else ref[lo:hi]
        assert_close(got[lo:hi], want, "f16", f"segment {s}")
    rows, H1, H2 = w.num_rows, w.H1, w.H2
    x, Wd, bd = _dev(w.x, "f16"), _dev(W, "f16"), _dev(b, "f16")
    y = torch.full((rows, H2), 7.0, dtype=torch.float16, device="cuda:0")
    lib = sg.lib()
    need = int(lib.lora_linear_workspace_bytes(rows, 0, H1, H2, 16, sg.SGMV_F16))
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda:0")
    rc = lib.lora_linear(y.data_ptr(), x.data_ptr(), Wd.data_ptr(), bd.data_ptr(), None, None,
                         None, None, 0, rows, 0, H1, H2, 16, 2.0, sg.SGMV_F16, ws.data_ptr(),
                         ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, sg.STATUS.get(rc, rc)
    torch.cuda.synchronize()
    assert_close(y.double().cpu().numpy(), ref_base, "f16", "S=0, NULL tables")


def test_repeated_calls_are_bitwise_identical():
    w = wl.small_random(15, "f16", 1024, 512, 16, 16, 64, 64)
    W, b = wl.base_layer(15, "f16", 1024, 512)
    d = to_device(w)
    first = _gpu_linear(w, W, b, d)
    for _ in range(3):
        assert np.array_equal(_gpu_linear(w, W, b, d), first)


# (rows, H1, H2, segments): decode tiles with the shrink folded in, and the
# 256 x 256 tiles after the mixed shrink launch.
@pytest.mark.parametrize("R,H1,H2,S", [(48, 512, 256, 12), (2048, 128, 4096, 8)],
                         ids=["decode_tiles", "wide_tiles"])
def test_graph_replay_matches_eager(R, H1, H2, S):
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(16, "bf16", H1, H2, 16, 8, R, S)
    W, b = wl.base_layer(16, "bf16", H1, H2)
    d = to_device(w)
    Wd, bd = _dev(W, "bf16"), _dev(b, "bf16")
    need = sg.lora_linear_workspace_bytes(R, S, H1, H2, 16, torch.bfloat16)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    out = torch.empty((R, H2), dtype=torch.bfloat16, device="cuda:0")
    sg.lora_linear(d["x"], Wd, d["A"], d["B"], d["seg"], d["ids"], w.scale, bias=bd, out=out,
                   workspace=ws)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sg.lora_linear(d["x"], Wd, d["A"], d["B"], d["seg"], d["ids"], w.scale, bias=bd,
                           out=out, workspace=ws)
    torch.cuda.synchronize()
    for _ in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    assert_close(eager.double().cpu().numpy(), _oracle(w, W, b), "bf16", "graph")
