"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Covers the five reference workloads at full size (every output element),
random shapes that span several tiles and ragged tails for every dtype and a
range of ranks (vectorised and general kernels), exact integer inputs that
must match bit for bit, edge cases of the segment table, misaligned
pointers, determinism and HIP graph replay.
"""
import zlib

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import (assert_close, gpu_expand, gpu_lora_apply, gpu_shrink, magnitude,
                         magnitude_expand, to_device, torch_dtype, COUNTER_BYTES)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU (run with -m 'not gpu' on CPU)"
    import segmented_gather_gemv_sgmv_amd as sg
    sg.lib()  # fail loudly if the HIP library is missing
    yield


_cache = {}


def _config(key):
    if key not in _cache:
        i, ctl = key
        w = wl.config(i, control=ctl)
        y, v = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
        my, mv = magnitude(w) if w.dtype == "f32" else (None, None)
        _cache.clear()  # keep at most one full-size workload in memory
        _cache[key] = (w, y, v, my, mv)
    return _cache[key]


CONFIG_KEYS = [(0, False), (1, False), (2, False), (2, True), (3, False), (4, False)]
CONFIG_IDS = ["tiny", "llama7b_decode", "skewed_zipf", "skewed_control", "prefill", "mlp_up"]


@pytest.mark.parametrize("key", CONFIG_KEYS, ids=CONFIG_IDS)
def test_config_all_entry_points(key):
    w, y_ref, v_ref, my, mv = _config(key)
    d = to_device(w)
    assert_close(gpu_lora_apply(w, d), y_ref, w.dtype, f"lora_apply {w.name}", my)
    assert_close(gpu_shrink(w, d), v_ref, w.dtype, f"sgmv_shrink {w.name}", mv)
    # expand alone, fed the oracle's v rounded to float32
    y_e = oracle.expand(w.y0, v_ref.astype(np.float32), w.B, w.seg_indptr, w.adapter_ids, w.scale)
    me = magnitude_expand(w, v_ref) if w.dtype == "f32" else None
    assert_close(gpu_expand(w, v_ref, d), y_e, w.dtype, f"sgmv_expand {w.name}", me)


def test_mixed_batch_all_entry_points():
    """A serving batch of two 512-row prefill segments and 128 one-row decode
    segments on 130 distinct adapters, every output element of every entry
    point against the oracle."""
    w = wl.mixed_batch(0)
    y_ref, v_ref = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    d = to_device(w)
    print(f"mixed batch {w.name}", flush=True)
    assert_close(gpu_lora_apply(w, d), y_ref, w.dtype, "lora_apply mixed")
    assert_close(gpu_shrink(w, d), v_ref, w.dtype, "sgmv_shrink mixed")
    y_e = oracle.expand(w.y0, v_ref.astype(np.float32), w.B, w.seg_indptr, w.adapter_ids, w.scale)
    assert_close(gpu_expand(w, v_ref, d), y_e, w.dtype, "sgmv_expand mixed")


RANDOM_CASES = [
    # dtype, H1, H2, r, adapters, rows, segments
    ("f32", 256, 256, 8, 4, 16, 4),
    ("f32", 1000, 776, 4, 7, 53, 9),
    ("f32", 513, 300, 16, 5, 37, 6),
    ("f32", 2048, 1024, 64, 3, 19, 3),
    ("f32", 300, 260, 128, 2, 9, 2),
    ("f16", 4096, 4096, 16, 9, 70, 11),
    ("f16", 1536, 2560, 8, 6, 100, 5),
    ("f16", 1000, 1000, 32, 4, 45, 7),
    ("f16", 640, 1032, 64, 5, 33, 4),
    ("f16", 520, 904, 128, 3, 21, 3),
    ("bf16", 5120, 1384, 64, 8, 40, 12),
    ("bf16", 2048, 2048, 16, 10, 77, 20),
    ("bf16", 777, 999, 8, 4, 29, 5),
    # general kernel: ranks without a vector kernel, ragged H2
    ("f16", 300, 250, 1, 3, 17, 4),
    ("f16", 513, 257, 3, 4, 23, 5),
    ("bf16", 1024, 700, 12, 5, 31, 6),
    ("f32", 400, 333, 5, 3, 14, 3),
    ("f16", 256, 384, 4, 3, 12, 3),
    ("bf16", 384, 128, 100, 2, 9, 2),
]


@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: "-".join(map(str, c)))
def test_random_shapes(case):
    dtype, H1, H2, r, N, R, S = case
    w = wl.small_random(zlib.crc32(repr(case).encode()), dtype, H1, H2, r, N, R, S, allow_empty=True,
                        uncovered_tail=R // 7)
    y_ref, v_ref = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    my, mv = magnitude(w)
    d = to_device(w)
    assert_close(gpu_lora_apply(w, d), y_ref, dtype, "lora_apply", my)
    cov = int(w.seg_indptr[-1])
    v = gpu_shrink(w, d, fill=-3.5)
    assert_close(v[:cov], v_ref[:cov], dtype, "sgmv_shrink", mv[:cov])
    assert np.all(v[cov:] == -3.5), "shrink wrote rows outside every segment"


@pytest.mark.parametrize("dtype,r", [("f32", 8), ("f32", 5), ("f16", 16), ("f16", 64),
                                     ("f16", 3), ("bf16", 16), ("bf16", 64), ("bf16", 12)])
def test_integer_inputs_match_bit_for_bit(dtype, r):
    # {-1,0,1} inputs: every partial sum is a small integer, exact in float32
    w = wl.integer_exact(11 + r, dtype, 1536, 1040, r, 6, 67, 9, density=0.08, scale=2.0)
    y_ref, v_ref = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    assert np.abs(y_ref).max() < 256  # exact in every output dtype
    d = to_device(w)
    assert np.array_equal(gpu_lora_apply(w, d), y_ref)
    cov = int(w.seg_indptr[-1])
    assert np.array_equal(gpu_shrink(w, d)[:cov], v_ref[:cov])
    y_e = oracle.expand(w.y0, v_ref.astype(np.float32), w.B, w.seg_indptr, w.adapter_ids, w.scale)
    assert np.array_equal(gpu_expand(w, v_ref, d), y_e)


@pytest.mark.parametrize("dtype,r,H1,R,S", [("f16", 16, 2048, 600, 3), ("bf16", 64, 1024, 520, 4),
                                            ("f16", 128, 2048, 2400, 4)])
def test_integer_inputs_row_heavy_bit_for_bit(dtype, r, H1, R, S):
    """Row-heavy integer cases: every entry point runs on the MFMA tiles (the
    last one splits H1 into grouped chunk ranges) and must match exactly."""
    w = wl.integer_exact(7 * r + R, dtype, H1, 1024, r, 5, R, S, density=0.05, scale=2.0)
    y_ref, v_ref = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    assert np.abs(y_ref).max() < 256 and np.abs(v_ref).max() < 2048
    d = to_device(w)
    assert np.array_equal(gpu_lora_apply(w, d), y_ref)
    cov = int(w.seg_indptr[-1])
    assert np.array_equal(gpu_shrink(w, d)[:cov], v_ref[:cov])
    y_e = oracle.expand(w.y0, v_ref.astype(np.float32), w.B, w.seg_indptr, w.adapter_ids, w.scale)
    assert np.array_equal(gpu_expand(w, v_ref, d), y_e)


def test_long_segments_and_many_segments():
    # one long segment (many row tiles) plus > 256 short ones (multi-pass tile scan)
    rng = np.random.default_rng(5)
    lengths = [300] + list(rng.integers(0, 3, size=700)) + [41]
    ids = rng.integers(0, 40, size=len(lengths))
    w = wl.make_workload("long_and_many", "f16", 512, 768, 16, 40, lengths, ids, 1.25, seed=6)
    y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    assert_close(gpu_lora_apply(w), y_ref, "f16", "long and many segments")


def test_empty_and_degenerate_tables():
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(3, "f16", 256, 512, 16, 4, 20, 5)
    d = to_device(w)
    # no segments, and segments that are all empty: y unchanged
    for seg, ids in [(np.array([0], np.int32), np.array([], np.int32)),
                     (np.array([0, 0, 0, 0], np.int32), np.array([1, 2, 3], np.int32))]:
        y = d["y0"].clone()
        sg.lora_apply(y, d["x"], d["A"], d["B"], torch.from_numpy(seg).cuda(),
                      torch.from_numpy(ids).cuda(), 2.0)
        torch.cuda.synchronize()
        assert torch.equal(y, d["y0"])
    # zero rows
    e = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    ey = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    sg.lora_apply(ey, e, d["A"], d["B"], torch.zeros(1, dtype=torch.int32, device="cuda"),
                  torch.zeros(0, dtype=torch.int32, device="cuda"), 1.0)
    # a segment starting at the last row, and a single-row batch
    for seg, R in [([19, 20], 20), ([0, 1], 1)]:
        ws = wl.make_workload("edge", "f16", 256, 512, 16, 4, [0] * 0 + [seg[1] - seg[0]], [2],
                              0.5, seed=4, num_rows=R)
        ws.seg_indptr = np.array(seg, np.int32)
        y_ref, _ = oracle.lora_apply(ws.y0, ws.x, ws.A, ws.B, ws.seg_indptr, ws.adapter_ids,
                                     ws.scale)
        assert_close(gpu_lora_apply(ws), y_ref, "f16", f"edge {seg}")


def test_zero_B_or_scale_leaves_y_bitwise():
    w = wl.small_random(8, "bf16", 1024, 1024, 16, 5, 40, 6)
    d = to_device(w)
    d["B"].zero_()
    assert np.array_equal(gpu_lora_apply(w, d), w.y0.astype(np.float64))
    d = to_device(w)
    w.scale = 0.0
    assert np.array_equal(gpu_lora_apply(w, d), w.y0.astype(np.float64))


def test_invalid_adapter_ids_are_skipped():
    """Segments naming an adapter outside the stack are skipped by the kernels'
    guards: their rows stay as they were, the other segments are computed."""
    w = wl.small_random(9, "f16", 512, 512, 16, 4, 24, 4, allow_empty=False)
    good = w.adapter_ids.copy()
    bad = good.copy()
    bad[1] = 4        # == num_adapters
    bad[3] = -7
    d = to_device(w)
    import torch
    d["ids"] = torch.from_numpy(bad).cuda()
    y = gpu_lora_apply(w, d)
    y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, good, w.scale)
    for s in range(4):
        rows = slice(int(w.seg_indptr[s]), int(w.seg_indptr[s + 1]))
        if s in (1, 3):
            assert np.array_equal(y[rows], w.y0[rows].astype(np.float64))
        else:
            assert_close(y[rows], y_ref[rows], "f16", f"segment {s}")


@pytest.mark.parametrize("kind", ["one_row_each", "empty_and_two_rows", "bad_adapter",
                                  "offset_start"])
def test_decode_guess_holds_or_falls_back(kind):
    """With as many rows as segments, lora_apply's single-launch shrink items
    guess that segment i is row i alone and stream their A chunk before the
    segment scan; the guess is checked before anything is published.  Tables
    of that size where it holds and where it does not (an empty segment next
    to a two-row one, an adapter id out of range, a table that starts past
    row 0) must all match the oracle, with the counters back at zero and no
    fallback of the hand-off."""
    import torch
    S, N, H = 48, 7, 1024
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    lengths = np.ones(S, np.int64)
    if kind == "empty_and_two_rows":
        lengths[5], lengths[6] = 0, 2
    ids = rng.integers(0, N, size=S).astype(np.int32)
    w = wl.make_workload(f"guess_{kind}", "f16", H, H, 16, N, lengths, ids, 1.5, rng=rng)
    if kind == "offset_start":
        # row 0 uncovered, segments 0 .. S - 2 one row each, the last empty
        w.seg_indptr = np.minimum(np.arange(1, S + 2, dtype=np.int32), S)
    assert w.num_rows == w.num_segments == S
    good = w.adapter_ids.copy()
    d = to_device(w)
    if kind == "bad_adapter":
        bad = good.copy()
        bad[S // 2] = N
        d["ids"] = torch.from_numpy(bad).cuda()
        good = bad
    y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr,
                                 np.where((good >= 0) & (good < N), good, 0), w.scale)
    if kind == "bad_adapter":  # the row of the bad segment keeps its y
        y_ref[S // 2] = w.y0[S // 2]
    my, _ = magnitude(w)
    assert_close(gpu_lora_apply(w, d), y_ref, "f16", kind, my)


@pytest.mark.parametrize("kind,dtype,r,R", [
    ("all_rows", "f16", 16, 128), ("all_rows", "f32", 8, 14), ("all_rows", "bf16", 64, 40),
    ("short_end", "f16", 16, 128), ("late_start", "f16", 16, 100), ("bad_adapter", "f16", 16, 64)])
def test_single_segment_guess_holds_or_falls_back(kind, dtype, r, R):
    """With one segment, lora_apply's single-launch shrink items guess that
    it covers every row (tiles of its class) and stream their A chunk before
    the segment scan; the guess is checked before anything is published.
    Segments that do cover every row, that stop short of the last rows, that
    start past row 0, or that name an adapter out of range must all match
    the oracle, with the counters back at zero and no fallback."""
    import torch
    N, H = 5, 512
    rng = np.random.default_rng(zlib.crc32(f"{kind}{dtype}{r}{R}".encode()))
    w = wl.make_workload(f"one_{kind}", dtype, H, H, r, N, [R], [3], 1.25, rng=rng)
    if kind == "short_end":
        w.seg_indptr = np.array([0, R - 3], np.int32)
    elif kind == "late_start":
        w.seg_indptr = np.array([2, R], np.int32)
    d = to_device(w)
    ids = w.adapter_ids.copy()
    if kind == "bad_adapter":
        d["ids"] = torch.tensor([N], dtype=torch.int32, device="cuda")
    y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, ids, w.scale)
    if kind == "bad_adapter":
        y_ref = w.y0.astype(np.float64)
    my, _ = magnitude(w)
    assert_close(gpu_lora_apply(w, d), y_ref, dtype, kind, my)


@pytest.mark.parametrize("shape", ["rows_eq_segments", "one_segment"])
@pytest.mark.parametrize("dtype,r,H", [("f32", 4, 512), ("f32", 16, 768), ("bf16", 8, 1024),
                                       ("bf16", 16, 1024), ("f16", 32, 512), ("bf16", 64, 1024),
                                       ("f16", 128, 512)])
def test_guessed_tables_across_dtypes_and_ranks(shape, dtype, r, H):
    """Both guessed table shapes (one row per segment; one segment over every
    row) on every class a dtype and rank can put them in: one-row vector
    tiles, 4-row vector tiles (float32, rank 8), MFMA tiles (fp16 and bf16
    from rank 16, one partial tile at 13 rows)."""
    N = 6
    rng = np.random.default_rng(zlib.crc32(f"{shape}{dtype}{r}{H}".encode()))
    if shape == "rows_eq_segments":
        R = 40
        lengths, ids = np.ones(R, np.int64), rng.integers(0, N, size=R).astype(np.int32)
    else:
        R = 37 if r < 64 else 13  # a ragged last tile; at r >= 64 a single partial one
        lengths, ids = [R], [int(rng.integers(0, N))]
    w = wl.make_workload(f"guess_{shape}", dtype, H, H, r, N, lengths, ids, 0.75, rng=rng)
    y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    my, _ = magnitude(w)
    assert_close(gpu_lora_apply(w), y_ref, dtype, f"{shape} {dtype} r{r}", my)


def test_misaligned_pointers_take_general_path():
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(10, "f16", 1024, 1024, 16, 4, 30, 5)
    y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    d = to_device(w)

    def shifted(t):  # same values, data pointer off by one element
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        view = buf[1:].view(t.shape)
        view.copy_(t)
        return view

    y = shifted(d["y0"])
    sg.lora_apply(y, shifted(d["x"]), shifted(d["A"]), shifted(d["B"]), d["seg"], d["ids"],
                  w.scale)
    torch.cuda.synchronize()
    assert_close(y.double().cpu().numpy(), y_ref, "f16", "misaligned")


def test_repeated_calls_are_bitwise_identical():
    import torch
    w = wl.config(1)
    d = to_device(w)
    outs = [gpu_lora_apply(w, d) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("which", ["skewed", "decode_guess", "one_segment_guess"])
def test_graph_replay_matches_eager(which):
    """lora_apply captured in a HIP graph: every replay, with eager work and
    synchronisations in between, equals the eager result (a scanned table
    and both guessed ones)."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = {"skewed": lambda: wl.config(2), "decode_guess": lambda: wl.config(1),
         "one_segment_guess": lambda: wl.config(2, control=True)}[which]()
    d = to_device(w)
    y_eager = torch.from_numpy(gpu_lora_apply(w, d))
    ws = torch.zeros(sg.lora_apply_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.H2, w.r,
                                                   torch_dtype(w.dtype)),
                     dtype=torch.uint8, device="cuda")
    y = d["y0"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale, workspace=ws)
    for rep in range(4):
        y.copy_(d["y0"])
        junk = torch.randn(1 << 16, device="cuda").sum()  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.double().cpu(), y_eager), f"replay {rep}"
        del junk


def test_two_launch_graph_replay_with_changing_table():
    """A call that takes two launches, captured in a HIP graph and replayed
    while the segment table's contents change between replays (its size
    fixed): each replay's expand launch takes exactly the items its own
    shrink launch listed, never the longer list an earlier replay left."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    R, H1, H2, r, N = 2000, 512, 4096, 128, 6  # rank 128: B passes through LDS in slices
    tables = {
        "full": [300, 180, 250, 170, 200, 160, 140, 120, 130, 110, 120, 120],
        "small": [1, 0, 3, 17, 0, 1, 40, 2, 0, 9, 1, 5],
        "mid": [600, 0, 1, 1, 7, 300, 0, 15, 16, 2, 400, 3],
    }
    S = len(tables["full"])
    ids = [3, 0, 5, 1, 4, 2, 5, 0, 1, 3, 2, 4]
    ws_of = {k: wl.make_workload(k, "f16", H1, H2, r, N, v, ids, 1.25, seed=78, num_rows=R)
             for k, v in tables.items()}
    w = ws_of["full"]
    need = sg.lora_apply_workspace_bytes(R, S, H1, H2, r, torch.float16)
    # the item table after the partials: this shape takes two launches
    assert (need - COUNTER_BYTES) % (R * r * 4) != 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    d = to_device(w)
    y = d["y0"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale, workspace=ws)
    for name in ["full", "small", "full", "mid", "small", "mid"]:
        wk = ws_of[name]
        d["seg"].copy_(torch.from_numpy(wk.seg_indptr.astype(np.int32)))
        y.copy_(d["y0"])
        g.replay()
        torch.cuda.synchronize()
        y_ref, _ = oracle.lora_apply(wk.y0, wk.x, wk.A, wk.B, wk.seg_indptr, wk.adapter_ids,
                                     wk.scale)
        assert_close(y.double().cpu().numpy(), y_ref, "f16", f"replay on {name}")
        assert int(ws[:COUNTER_BYTES].view(torch.int32).abs().sum()) == 0


def test_capture_without_workspace_is_refused():
    """A capture that relies on the binding's cached workspace is refused
    (the graph would keep a buffer the cache may replace or share); a graph
    captured with its own workspace keeps replaying correctly after a larger
    eager call has grown the cache."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(71, "f16", 1024, 1024, 16, 8, 40, 10)
    d = to_device(w)
    y_ref = gpu_lora_apply(w, d)
    y = d["y0"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale)  # warm the cache
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="workspace"):
        with torch.cuda.graph(g):
            sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale)
    torch.cuda.synchronize()
    ws = torch.zeros(sg.lora_apply_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.H2, w.r,
                                                   torch.float16),
                     dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale, workspace=ws)
    big = wl.small_random(72, "f16", 4096, 4096, 16, 8, 600, 40)
    big_ref = oracle.lora_apply(big.y0, big.x, big.A, big.B, big.seg_indptr, big.adapter_ids,
                                big.scale)[0]
    db = to_device(big)
    for rep in range(3):
        y.copy_(d["y0"])
        g.replay()
        yb = db["y0"].clone()
        sg.lora_apply(yb, db["x"], db["A"], db["B"], db["seg"], db["ids"], big.scale)  # cache grows
        torch.cuda.synchronize()
        assert np.array_equal(y.double().cpu().numpy(), y_ref), f"replay {rep}"
        assert_close(yb.double().cpu().numpy(), big_ref, "f16", f"eager {rep}")


SELF_CONTAINED_CASES = {
    # MFMA row tiles, one long segment
    "skewed_control": lambda: wl.config(2, control=True),
    # one-row (GEMV) tiles only: the decode batch
    "decode": lambda: wl.config(1),
    # both classes in one launch: MFMA tiles and one-row tiles
    "mixed_small": lambda: wl.mixed_batch(3, long_rows=(40, 23, 2), short=60, H=2048, r=32,
                                          dtype="bf16", num_adapters=80),
    # float32: four-row vector tiles for the long segments, one-row tiles
    # (H1 = 2048: an adapter's A above the size whose tiles skip the hand-off)
    "f32_vector_tiles": lambda: wl.make_workload("f32_mix", "f32", 2048, 768, 8, 12,
                                                 [1, 9, 1, 1, 4, 2, 1, 7], list(range(8)),
                                                 1.5, seed=4),
}


@pytest.mark.parametrize("dtype,H1,H2,r,lengths", [
    ("f32", 256, 256, 8, [4, 4, 4, 4]),                       # the tiny config's shape
    ("f16", 1024, 1000, 16, [1, 5, 0, 16, 2, 1, 9]),          # MFMA and one-row tiles
    ("bf16", 512, 512, 32, [3, 1, 17, 1]),                    # 256-column expand items:
    ("bf16", 256, 504, 64, [2, 1, 1, 30]),                    # two per tile, the second ragged
    ("f16", 1000, 512, 8, [1, 3, 1, 6, 2]),                   # four-row vector tiles
])
def test_small_adapters_skip_the_handoff(dtype, H1, H2, r, lengths):
    """When an adapter's A is small (<= 32 KB) and a tile has at most two
    column chunks, the single launch has no shrink items: each expand item
    computes its tile's v itself.  Parity with the oracle, and the counters
    and the sticky flag are never touched, at the default patience and at
    zero patience alike."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    N = 5
    ids = [(3 * k + 1) % N for k in range(len(lengths))]
    w = wl.make_workload(f"small_{dtype}_{r}", dtype, H1, H2, r, N, lengths, ids, 1.25,
                         seed=H1 + r)
    y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    my, _ = magnitude(w)
    y = gpu_lora_apply(w)
    assert_close(y, y_ref, dtype, w.name, my)
    try:
        sg.set_fused_wait(0.0)
        y0 = gpu_lora_apply(w)  # asserts the flag stays clear: nothing waited
    finally:
        sg.set_fused_wait(0.02)
    assert np.array_equal(y, y0)


@pytest.mark.parametrize("case", list(SELF_CONTAINED_CASES))
def test_fused_self_contained_path_is_bit_identical(case):
    """With zero patience every expand workgroup of the single-kernel
    hand-off recomputes its rows' partial sums itself; the output must be
    bit-identical to the normal hand-off path, and the sticky flag is set."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = SELF_CONTAINED_CASES[case]()
    d = to_device(w)
    ws = torch.zeros(sg.lora_apply_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.H2, w.r,
                                                   torch_dtype(w.dtype)),
                     dtype=torch.uint8, device="cuda")

    def run():
        y = d["y0"].clone()
        sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale, workspace=ws)
        torch.cuda.synchronize()
        return y

    normal = run()
    counters = ws[:262144].view(torch.int32)
    assert int(counters[-1]) == 0 and int(counters[:-1].abs().sum()) == 0
    try:
        sg.set_fused_wait(0.0)
        alone = run()
    finally:
        sg.set_fused_wait(0.02)
    assert torch.equal(normal, alone)
    assert int(counters[-1]) == 1, "the self-contained path did not run"
    assert int(counters[:-1].abs().sum()) == 0, "counters not returned to zero"


def test_workspace_reused_across_shapes():
    """One workspace serves calls of different shapes in any order (the
    counters sit at a fixed offset and are left at zero)."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    shapes = [(0, "f16", 4096, 4096, 16, 64, 64, 64), (1, "bf16", 1024, 3072, 64, 9, 200, 40),
              (2, "f16", 2048, 1024, 8, 5, 30, 3), (3, "f32", 512, 768, 16, 7, 300, 90)]
    work = [wl.small_random(sd, dt, H1, H2, r, N, R, S) for sd, dt, H1, H2, r, N, R, S in shapes]
    need = max(max(sg.lora_apply_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.H2, w.r,
                                                 torch_dtype(w.dtype)),
                   sg.shrink_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.r,
                                             torch_dtype(w.dtype))) for w in work)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for w in work + work[::-1] + work:
        d = to_device(w)
        y = d["y0"].clone()
        sg.lora_apply(y, d["x"], d["A"], d["B"], d["seg"], d["ids"], w.scale, workspace=ws)
        torch.cuda.synchronize()
        y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
        my, mv = magnitude(w)
        assert_close(y.double().cpu().numpy(), y_ref, w.dtype, w.name, my)
        assert int(ws[:262144].view(torch.int32).abs().sum()) == 0
        # sgmv_shrink on the same workspace (its tile counters sit there too)
        v = torch.zeros(w.num_rows, w.r, dtype=torch.float32, device="cuda")
        sg.sgmv_shrink(v, d["x"], d["A"], d["seg"], d["ids"], workspace=ws)
        torch.cuda.synchronize()
        v_ref = oracle.shrink(w.x, w.A, w.seg_indptr, w.adapter_ids)
        covered = np.zeros(w.num_rows, bool)
        for k in range(w.num_segments):
            covered[w.seg_indptr[k]:w.seg_indptr[k + 1]] = True
        assert_close(v.double().cpu().numpy()[covered], v_ref[covered], w.dtype, w.name + " shrink",
                     mv[covered])
        assert int(ws[:262144].view(torch.int32).abs().sum()) == 0


def test_shrink_in_kernel_reduction_is_deterministic():
    """Decode-shaped sgmv_shrink splits H1 over several workgroups per row
    and the last of them sums the chunks in order: repeated calls give the
    same bits, rows outside every segment keep their contents, and the tile
    counters are left at zero."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(11, "f16", 4096, 1024, 16, 40, 48, 40, uncovered_tail=8)
    d = to_device(w)
    need = sg.shrink_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.r, torch.float16)
    assert need > 262144, "the shape must split H1 (partials after the counters)"
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        v = torch.full((w.num_rows, w.r), 7.0, dtype=torch.float32, device="cuda")
        sg.sgmv_shrink(v, d["x"], d["A"], d["seg"], d["ids"], workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:262144].view(torch.int32).abs().sum()) == 0
        outs.append(v.clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    got = outs[0].double().cpu().numpy()
    v_ref = oracle.shrink(w.x, w.A, w.seg_indptr, w.adapter_ids)
    R = w.num_rows
    end = int(w.seg_indptr[-1])
    assert end <= R - 8
    assert np.all(got[end:] == 7.0)
    covered = np.zeros(R, bool)
    for k in range(w.num_segments):
        covered[w.seg_indptr[k]:w.seg_indptr[k + 1]] = True
    assert_close(got[covered], v_ref[covered], w.dtype, "decode shrink")


@pytest.mark.parametrize("seed,dtype,H1,H2,r,N,R,S,tail", [
    (41, "bf16", 1024, 3072, 64, 7, 3000, 5, 0),
    (42, "f16", 512, 3000, 128, 4, 2000, 3, 37),  # ragged last column chunk
    # more than two rounds of one-chunk workgroups: each shrink workgroup
    # sums several LDS-sized chunks (ragged last range)
    (43, "f16", 2048, 1024, 128, 6, 2400, 4, 19),
    (44, "bf16", 4096, 1024, 64, 9, 2048, 8, 0),
])
def test_two_launch_mfma_path(seed, dtype, H1, H2, r, N, R, S, tail):
    """Row-heavy calls too large for one resident round of single-kernel
    items run as a shrink launch and an expand launch; ragged segments
    (some empty) and rows outside every segment included."""
    import segmented_gather_gemv_sgmv_amd as sg
    w = wl.small_random(seed, dtype, H1, H2, r, N, R, S, uncovered_tail=tail)
    need = sg.lora_apply_workspace_bytes(R, S, H1, H2, r, torch_dtype(dtype))
    assert (need - COUNTER_BYTES) % (R * r * 4) != 0, "the expand item table: two launches"
    y_ref, _ = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    y = gpu_lora_apply(w)
    assert_close(y, y_ref, dtype, w.name)
    if tail:
        assert np.array_equal(y[R - tail:], w.y0[R - tail:].astype(y.dtype))


@pytest.mark.parametrize("S,R,lengths_kind", [(1500, 1500, "ones"), (1300, 700, "sparse"),
                                              (40, 160, "mixed")])
def test_tile_mappings(S, R, lengths_kind):
    """Decode-shaped batches through the single-kernel lora_apply: the direct
    tile mapping (more than 1024 segments), the compact mapping with many
    empty segments, and tiles of four rows."""
    rng = np.random.default_rng(S + R)
    if lengths_kind == "ones":
        lengths = [1] * S
    elif lengths_kind == "sparse":
        lengths = [0] * S
        for i in rng.choice(S, size=R, replace=True):
            lengths[i] += 1
    else:
        lengths = list(rng.integers(0, 9, size=S))
        lengths[-1] += R - sum(lengths)
    ids = rng.integers(0, 24, size=S)
    w = wl.make_workload("decode_map", "f16", 1024, 1536, 16, 24, lengths, ids, 0.75,
                         seed=S, num_rows=R)
    assert w.seg_indptr[-1] <= R
    y_ref, v_ref = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    assert_close(gpu_lora_apply(w), y_ref, "f16", f"decode mapping {lengths_kind}")
    # sgmv_shrink over the same table: thousands of one-row tiles take no
    # H1 split ("ones", "sparse"); the mixed case splits H1 and the tiles'
    # last workgroups reduce it in-kernel.
    cov = np.zeros(R, bool)
    for k in range(S):
        cov[w.seg_indptr[k]:w.seg_indptr[k + 1]] = True
    v = gpu_shrink(w, fill=-2.0)
    assert_close(v[cov], v_ref[cov], "f16", f"decode mapping shrink {lengths_kind}")
    assert np.all(v[~cov] == -2.0)
