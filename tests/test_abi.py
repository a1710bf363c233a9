"""CPU checks of the C ABI boundary: the library loads, exports every symbol
the header declares, and rejects bad arguments before enqueueing anything.
No call here launches a kernel (there is no GPU on this side)."""
import ctypes
import os
import re

import numpy as np
import pytest

import segmented_gather_gemv_sgmv_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgmv.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sg.LIBRARY):
        from segmented_gather_gemv_sgmv_amd import build
        build.build()
    return sg.lib()


def test_header_symbols_exported(lib):
    names = _header_functions()
    assert {"lora_apply", "sgmv_shrink", "sgmv_expand"} <= names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sgmv.h but not exported"
    assert names == {n for n, _, _ in sg.ABI}, "binding table and header disagree"


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+SGMV_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.sgmv_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for code in range(0, 9):
        s = lib.sgmv_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.sgmv_status_string(0) == b"ok"
    assert lib.sgmv_status_string(99) == b"unknown status"


FAKE = 0x1000  # a non-null, 16-byte-aligned value; never dereferenced on these paths


def _apply(lib, **kw):
    a = dict(y=FAKE, x=FAKE, A=FAKE, B=FAKE, seg=FAKE, ids=FAKE, S=4, R=16, N=4, H1=256, H2=256,
             r=8, scale=1.0, dtype=0, ws=FAKE, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.lora_apply(a["y"], a["x"], a["A"], a["B"], a["seg"], a["ids"], a["S"], a["R"],
                          a["N"], a["H1"], a["H2"], a["r"], a["scale"], a["dtype"], a["ws"],
                          a["ws_bytes"], a["stream"])


def test_lora_apply_rejects_bad_arguments(lib):
    assert _apply(lib, dtype=7) == 3
    assert _apply(lib, r=0) == 2
    assert _apply(lib, r=129) == 2
    assert _apply(lib, H1=0) == 2
    assert _apply(lib, H2=-1) == 2
    assert _apply(lib, R=-1) == 2
    assert _apply(lib, S=-2) == 2
    assert _apply(lib, N=-1) == 2
    for p in ("y", "x", "A", "B", "seg", "ids"):
        assert _apply(lib, **{p: None}) == 1, p
    need = lib.lora_apply_workspace_bytes(16, 4, 256, 256, 8, 0)
    assert need > 0
    assert _apply(lib, ws=None, ws_bytes=need) == 5
    assert _apply(lib, ws_bytes=need - 1) == 5


def test_empty_batches_are_noops(lib):
    # nothing is enqueued, so NULL pointers are fine
    none = dict(y=None, x=None, A=None, B=None, seg=None, ids=None, ws=None)
    assert _apply(lib, R=0, **none) == 0
    assert _apply(lib, S=0, **none) == 0
    assert lib.sgmv_shrink(None, None, None, None, None, 0, 5, 1, 64, 8, 1, None, 0, None) == 0
    assert lib.sgmv_expand(None, None, None, None, None, 3, 0, 1, 8, 64, 1.0, 1, None) == 0


def test_shrink_expand_reject_bad_arguments(lib):
    assert lib.sgmv_shrink(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 4, 256, 8, 5, None, 0, None) == 3
    assert lib.sgmv_shrink(FAKE, None, FAKE, FAKE, FAKE, 4, 16, 4, 256, 8, 1, None, 0, None) == 1
    assert lib.sgmv_shrink(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 4, 0, 8, 1, None, 0, None) == 2
    need = lib.sgmv_shrink_workspace_bytes(64, 64, 4096, 16, 1)
    assert need > 0  # the H1 reduction is split for this shape
    assert lib.sgmv_shrink(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 4096, 16, 1, None, need,
                           None) == 5
    assert lib.sgmv_expand(FAKE, FAKE, None, FAKE, FAKE, 4, 16, 4, 8, 256, 1.0, 1, None) == 1
    assert lib.sgmv_expand(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 4, 200, 256, 1.0, 1, None) == 2


def test_workspace_sizes(lib):
    for R, S, H1, H2, r, dt in [(64, 64, 4096, 4096, 16, 1), (4096, 16, 4096, 4096, 16, 1),
                                (256, 110, 5120, 13824, 64, 2), (16, 4, 256, 256, 8, 0),
                                (7, 3, 100, 90, 5, 1)]:
        n = lib.lora_apply_workspace_bytes(R, S, H1, H2, r, dt)
        counters = 256 * 1024  # fixed counter region at the front
        # then float32 partials, whole [num_rows][r] chunks (and, for calls
        # that take two launches, the expand launch's item table after them)
        assert n >= counters + R * r * 4
        assert n == lib.lora_apply_workspace_bytes(R, S, H1, H2, r, dt)
        m = lib.sgmv_shrink_workspace_bytes(R, S, H1, r, dt)
        assert m == 0 or counters < m <= n
    assert lib.lora_apply_workspace_bytes(16, 4, 256, 256, 0, 0) == 0


def test_validate_segments():
    ok = sg.validate_segments([0, 2, 2, 5], [1, 0, 3], num_rows=6, num_adapters=4)
    assert ok == 0
    assert sg.validate_segments([0], [], num_rows=0, num_adapters=0) == 0
    assert sg.validate_segments([0, 3, 2], [0, 0], 6, 4) == 7       # decreasing
    assert sg.validate_segments([0, 3, 7], [0, 0], 6, 4) == 7       # past num_rows
    assert sg.validate_segments([-1, 3], [0], 6, 4) == 7            # negative start
    assert sg.validate_segments([0, 3], [4], 6, 4) == 7             # id out of range
    assert sg.validate_segments([0, 3], [-1], 6, 4) == 7
    with pytest.raises(ValueError):
        sg.validate_segments([0, 3], [0, 1], 6, 4)


def test_binding_raises_without_library(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(sg, "LIBRARY", str(tmp_path / "missing.so"))
    monkeypatch.setattr(sg, "_lib_handle", None)
    with pytest.raises(RuntimeError, match="missing"):
        sg.lib()


def test_set_fused_wait_validates(lib):
    assert lib.sgmv_set_fused_wait(-1.0) == 2
    assert lib.sgmv_set_fused_wait(11.0) == 2
    assert lib.sgmv_set_fused_wait(float("nan")) == 2
    assert lib.sgmv_set_fused_wait(0.0) == 0
    assert lib.sgmv_set_fused_wait(0.02) == 0


def test_last_hip_error_is_readable(lib):
    assert isinstance(lib.sgmv_last_hip_error(), bytes)


def test_lora_apply_multi_host_checks(lib):
    """Argument errors of lora_apply_multi come back before anything is
    enqueued; the descriptor layout matches the header's."""
    import ctypes
    import segmented_gather_gemv_sgmv_amd as sg
    assert ctypes.sizeof(sg.LoraProblem) == 48
    arr = (sg.LoraProblem * 2)()
    p = ctypes.cast(arr, ctypes.c_void_p)
    assert lib.lora_apply_multi(None, 1, None, None, 1, 1, 1, 16, 1, None, 0, None) == 1
    assert lib.lora_apply_multi(p, 0, None, None, 1, 1, 1, 16, 1, None, 0, None) == 2
    assert lib.lora_apply_multi(p, 9, None, None, 1, 1, 1, 16, 1, None, 0, None) == 2
    for k in range(2):  # H1 = H2 = 0
        arr[k] = sg.LoraProblem(None, None, None, None, 0, 0, 1.0)
    assert lib.lora_apply_multi(p, 2, None, None, 1, 1, 1, 16, 1, None, 0, None) == 2
    for k in range(2):
        arr[k] = sg.LoraProblem(None, None, None, None, 4096, 4096, 1.0)
    assert lib.lora_apply_multi(p, 2, None, None, 64, 64, 64, 16, 1, None, 0, None) == 1
    one = lib.lora_apply_workspace_bytes(64, 64, 4096, 4096, 16, 1)
    assert lib.lora_apply_multi_workspace_bytes(p, 2, 64, 64, 16, 1) >= one
    assert lib.lora_apply_multi_workspace_bytes(p, 0, 64, 64, 16, 1) == 0


def test_load_adapter_host_checks(lib):
    """Argument errors of sgmv_load_adapter come back before any copy."""
    dummy = 0x1000  # never dereferenced: every call below fails a host check
    L = lib.sgmv_load_adapter
    assert L(dummy, dummy, 0, 1, 4, dummy, dummy, 64, 64, 8, 9, None) == 3
    assert L(dummy, dummy, 4, 1, 4, dummy, dummy, 64, 64, 8, 1, None) == 2
    assert L(dummy, dummy, 2, 3, 4, dummy, dummy, 64, 64, 8, 1, None) == 2
    assert L(dummy, dummy, 0, 0, 4, dummy, dummy, 64, 64, 8, 1, None) == 2
    assert L(dummy, dummy, -1, 1, 4, dummy, dummy, 64, 64, 8, 1, None) == 2
    assert L(dummy, dummy, 0, 1, 4, dummy, dummy, 64, 64, 0, 1, None) == 2
    assert L(None, dummy, 0, 1, 4, dummy, dummy, 64, 64, 8, 1, None) == 1
    assert L(dummy, dummy, 0, 1, 4, dummy, None, 64, 64, 8, 1, None) == 1


def _linear(lib, **kw):
    a = dict(y=FAKE, x=FAKE, W=FAKE, bias=None, A=FAKE, B=FAKE, seg=FAKE, ids=FAKE, S=4, R=16,
             N=4, H1=256, H2=256, r=8, scale=1.0, dtype=1, ws=FAKE, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return lib.lora_linear(a["y"], a["x"], a["W"], a["bias"], a["A"], a["B"], a["seg"], a["ids"],
                           a["S"], a["R"], a["N"], a["H1"], a["H2"], a["r"], a["scale"],
                           a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


def test_lora_linear_host_checks(lib):
    assert _linear(lib, dtype=9) == 3
    assert _linear(lib, r=0) == 2
    assert _linear(lib, H1=0) == 2
    assert _linear(lib, H2=0) == 2
    assert _linear(lib, R=-1) == 2
    for p in ("y", "x", "W", "A", "B", "seg", "ids"):
        assert _linear(lib, **{p: None}) == 1, p
    # without segments the stacks and the table are not needed ...
    need0 = lib.lora_linear_workspace_bytes(16, 0, 256, 256, 8, 1)
    assert _linear(lib, S=0, A=None, B=None, seg=None, ids=None, ws=None, ws_bytes=need0) == 5
    # ... and an empty batch enqueues nothing at all
    assert _linear(lib, R=0, y=None, x=None, W=None, ws=None, ws_bytes=0) == 0
    need = lib.lora_linear_workspace_bytes(16, 4, 256, 256, 8, 1)
    assert need > 256 * 1024
    assert _linear(lib, ws=None, ws_bytes=need) == 5
    assert _linear(lib, ws_bytes=need - 1) == 5


def test_lora_linear_workspace_sizes(lib):
    counters = 256 * 1024
    for R, S, H1, H2, r, dt in [(64, 64, 4096, 4096, 16, 1), (4096, 16, 4096, 4096, 16, 1),
                                (256, 110, 5120, 13824, 64, 2), (16, 4, 256, 256, 8, 0),
                                (7, 3, 100, 90, 5, 1), (5, 0, 64, 64, 4, 2)]:
        n = lib.lora_linear_workspace_bytes(R, S, H1, H2, r, dt)
        assert n >= counters + R * r * 4
        assert n == lib.lora_linear_workspace_bytes(R, S, H1, H2, r, dt)
    # decode shapes split K over workgroups and keep float32 partial tiles
    assert (lib.lora_linear_workspace_bytes(64, 64, 4096, 4096, 16, 1)
            > lib.lora_apply_workspace_bytes(64, 64, 4096, 4096, 16, 1))
    assert lib.lora_linear_workspace_bytes(16, 4, 256, 256, 0, 1) == 0


def _noalloc(lib, **kw):
    a = dict(y=FAKE, x=FAKE, A=FAKE, B=FAKE, seg=FAKE, ids=FAKE, S=4, R=16, N=4, H1=256, H2=256,
             r=8, scale=1.0, dtype=0, stream=None)
    a.update(kw)
    return lib.lora_apply_noalloc(a["y"], a["x"], a["A"], a["B"], a["seg"], a["ids"], a["S"],
                                  a["R"], a["N"], a["H1"], a["H2"], a["r"], a["scale"],
                                  a["dtype"], a["stream"])


def test_noalloc_rejects_bad_arguments_and_oversized_calls(lib):
    """The allocation-free entry point returns lora_apply's errors, and
    SGMV_ERR_SCRATCH for a call whose workspace would exceed the static
    scratch, all before it touches the device."""
    assert _noalloc(lib, dtype=7) == 3
    assert _noalloc(lib, r=0) == 2
    assert _noalloc(lib, H2=0) == 2
    for p in ("y", "x", "A", "B", "seg", "ids"):
        assert _noalloc(lib, **{p: None}) == 1, p
    assert _noalloc(lib, R=0) == 0 and _noalloc(lib, S=0) == 0  # no-ops
    m = re.search(r"#define\s+SGMV_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)",
                  open(HEADER).read())
    limit = int(m.group(1)) << int(m.group(2))
    assert limit == sg.SGMV_NOALLOC_SCRATCH_BYTES
    # a prefill-sized call at a large rank needs more than the scratch holds
    R, S, H, r = 65536, 16, 8192, 128
    need = lib.lora_apply_workspace_bytes(R, S, H, H, r, 1)
    assert need > limit
    assert _noalloc(lib, R=R, S=S, H1=H, H2=H, r=r, dtype=1) == 8
    assert b"lora_apply_noalloc" in lib.sgmv_status_string(8)
