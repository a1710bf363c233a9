"""A seeded sweep of random shapes through every entry point, against the
fp64 oracle (bounds of gpu_helpers).  The shapes are drawn so that each
kernel choice comes up several times: decode batches (rows <= segments),
row-heavy ones (rows >= 4 x segments: MFMA tiles for fp16/bf16 and ranks
16..128), mixed ones, vector and general ranks, H that is not a multiple of
8 (general kernels), empty segments, rows outside every segment, and H1
splits long enough to be reduced in-kernel.  Sizes keep the oracle within a
fraction of a second per case."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import (assert_close, gpu_expand, gpu_lora_apply, gpu_shrink, magnitude,
                         magnitude_expand, to_device)

pytestmark = pytest.mark.gpu

RANKS = [1, 3, 4, 8, 12, 16, 24, 32, 64, 100, 128]
H_CHOICES = [64, 100, 200, 256, 520, 1004, 1024, 1536, 2048, 2056, 4096]


def _draw(case):
    rng = np.random.default_rng(1000 + case)
    dtype = ["f16", "bf16", "f32"][case % 3]
    kind = ["decode", "rowheavy", "mixed"][(case // 3) % 3]
    # row-heavy cases mostly take the MFMA ranks, so that the tiles come up
    r = int(rng.choice([16, 32, 64, 128] if kind == "rowheavy" and rng.random() < 0.75
                       else RANKS))
    H1 = int(rng.choice(H_CHOICES))
    H2 = int(rng.choice(H_CHOICES))
    if kind == "decode":
        S = int(rng.integers(8, 160))
        R = int(rng.integers(1, S + 1))
    elif kind == "rowheavy":
        S = int(rng.integers(1, 12))
        R = int(rng.integers(4 * S, 4 * S + 700))
    else:
        S = int(rng.integers(4, 60))
        R = int(rng.integers(S, 4 * S))
    # keep the oracle quick: about 2e7 multiply-adds at most
    while R > 1 and R * r * (H1 + H2) > 20_000_000:
        R = max(1, R // 2)
        S = max(1, min(S, R))
    N = int(rng.integers(1, 24))
    tail = int(rng.integers(0, 3)) if R > 2 else 0
    return wl.small_random(2000 + case, dtype, H1, H2, r, N, R, S, allow_empty=True,
                           uncovered_tail=tail)


@pytest.mark.parametrize("case", range(48))
def test_random_shape_all_entry_points(case):
    w = _draw(case)
    d = to_device(w)
    y_ref, v_ref = oracle.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    my, mv = magnitude(w)
    assert_close(gpu_lora_apply(w, d), y_ref, w.dtype, f"lora_apply {w.name}", my)
    covered = np.zeros(w.num_rows, bool)
    for k in range(w.num_segments):
        covered[w.seg_indptr[k]:w.seg_indptr[k + 1]] = True
    v = gpu_shrink(w, d, fill=-1.25)
    assert_close(v[covered], v_ref[covered], w.dtype, f"sgmv_shrink {w.name}", mv[covered])
    assert np.all(v[~covered] == -1.25), "shrink wrote rows outside every segment"
    y_e = oracle.expand(w.y0, v_ref.astype(np.float32), w.B, w.seg_indptr, w.adapter_ids, w.scale)
    y = gpu_expand(w, v_ref, d)
    assert_close(y, y_e, w.dtype, f"sgmv_expand {w.name}", magnitude_expand(w, v_ref))
    assert np.array_equal(y[~covered], w.y0[~covered].astype(np.float64)), \
        "expand changed rows outside every segment"
