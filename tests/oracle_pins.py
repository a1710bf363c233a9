"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes an oracle object (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with something other than itself:
a hand-worked example, a library matmul, pure-Python brute force, exact
integer arithmetic, or an invariant of the definition.  ``test_oracle.py``
runs them on the real oracle; ``test_oracle_mutants.py`` runs them on copies
of the oracle with planted mistakes and checks that every mistake is caught.

The method: y_i += s * (x_i A_a) B_a per contiguous row segment, with all
adapters' A [H1, r] and B [r, H2] stacked back to back (Punica walkthrough,
omica.com.cn/news/959180, sections 2.1-2.2).
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rel_close(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.abs(a - b)
    bound = tol * (1.0 + np.abs(b))
    assert np.all(err <= bound), f"max err {err.max():.3e}, worst ratio {(err / bound).max():.3g}"


def _small(seed=0, dtype="f32", H1=24, H2=20, r=4, N=5, R=11, S=4, **kw):
    return wl.small_random(seed, dtype, H1, H2, r, N, R, S, **kw)


def _run(orc, w, **over):
    args = dict(y0=w.y0, x=w.x, A_stack=w.A, B_stack=w.B, seg_indptr=w.seg_indptr,
                adapter_ids=w.adapter_ids, scale=w.scale)
    args.update(over)
    return orc.lora_apply(**args)


# -- worked example ------------------------------------------------------------

def pin_hand_worked_example(orc):
    """Numbers worked by hand from the definition (tests/golden)."""
    with open(os.path.join(GOLDEN, "hand_worked_example.json")) as f:
        g = json.load(f)
    y, v = orc.lora_apply(np.array(g["y0"], np.float32), np.array(g["x"], np.float32),
                          np.array(g["A_stack"], np.float32), np.array(g["B_stack"], np.float32),
                          g["seg_indptr"], g["adapter_ids"], g["scale"])
    assert np.array_equal(y, np.array(g["y_expected"], np.float64)), y
    assert np.array_equal(v, np.array(g["v_expected"], np.float64)), v
    vs = orc.shrink(np.array(g["x"], np.float32), np.array(g["A_stack"], np.float32),
                    g["seg_indptr"], g["adapter_ids"])
    assert np.array_equal(vs, np.array(g["v_expected"], np.float64)), vs


# -- library routines ----------------------------------------------------------

def pin_single_segment_is_matmul(orc):
    """One segment over every row reduces to y0 + s * (x @ A_a) @ B_a."""
    w = _small(seed=1, H1=37, H2=29, r=6, N=3, R=9, S=1)
    for a in range(3):
        ids = np.array([a], np.int32)
        seg = np.array([0, w.num_rows], np.int32)
        y, v = _run(orc, w, seg_indptr=seg, adapter_ids=ids)
        X, A, B = (t.astype(np.float64) for t in (w.x, w.A[a], w.B[a]))
        v_ref = X @ A
        _rel_close(v, v_ref, 1e-12)
        _rel_close(y, w.y0.astype(np.float64) + w.scale * (v_ref @ B), 1e-12)


def pin_gather_bmm_identity(orc):
    """Per-row adapter gather plus batched products (numpy einsum) agree."""
    w = _small(seed=2, H1=40, H2=33, r=5, N=6, R=23, S=7)
    per_row = np.full(w.num_rows, -1)
    for s in range(w.num_segments):
        per_row[w.seg_indptr[s]:w.seg_indptr[s + 1]] = w.adapter_ids[s]
    cov = per_row >= 0
    X = w.x.astype(np.float64)[cov]
    Ag = w.A.astype(np.float64)[per_row[cov]]
    Bg = w.B.astype(np.float64)[per_row[cov]]
    v_ref = np.einsum("ih,ihk->ik", X, Ag)
    d_ref = np.einsum("ik,ikj->ij", v_ref, Bg)
    y, v = _run(orc, w)
    y_ref = w.y0.astype(np.float64).copy()
    y_ref[cov] += w.scale * d_ref
    _rel_close(y, y_ref, 1e-12)
    _rel_close(v[cov], v_ref, 1e-12)


# -- brute force -------------------------------------------------------------------

def pin_brute_force_tiny(orc):
    """Pure-Python sum over (h, k) pairs in the other association, x (A B)."""
    w = _small(seed=3, H1=5, H2=4, r=3, N=3, R=6, S=3, allow_empty=False)
    y, _ = _run(orc, w)
    y_ref = w.y0.astype(np.float64).copy()
    for s in range(w.num_segments):
        a = int(w.adapter_ids[s])
        for i in range(int(w.seg_indptr[s]), int(w.seg_indptr[s + 1])):
            for j in range(w.H2):
                tot = 0.0
                for h, k in itertools.product(range(w.H1), range(w.r)):
                    tot += float(w.x[i, h]) * float(w.A[a, h, k]) * float(w.B[a, k, j])
                y_ref[i, j] += w.scale * tot
    _rel_close(y, y_ref, 1e-12)


# -- exact integer arithmetic ----------------------------------------------------

def pin_integer_exact(orc):
    """{-1,0,1} inputs: the exact answer comes from int64 matmuls, bit for bit."""
    w = wl.integer_exact(4, "f32", 64, 48, 8, 5, 30, 6, density=0.3, scale=2.0)
    y, v = _run(orc, w)
    y_ref = w.y0.astype(np.int64).copy()
    v_ref = np.zeros((w.num_rows, w.r), np.int64)
    for s in range(w.num_segments):
        a = int(w.adapter_ids[s])
        lo, hi = int(w.seg_indptr[s]), int(w.seg_indptr[s + 1])
        v_ref[lo:hi] = w.x[lo:hi].astype(np.int64) @ w.A[a].astype(np.int64)
        y_ref[lo:hi] += 2 * (v_ref[lo:hi] @ w.B[a].astype(np.int64))
    assert np.array_equal(y, y_ref.astype(np.float64))
    assert np.array_equal(v, v_ref.astype(np.float64))


# -- invariants of the definition -----------------------------------------------

def pin_zero_weights_or_scale_leave_y(orc):
    """B = 0, A = 0 or s = 0 leave y equal to y0 exactly."""
    w = _small(seed=5)
    y0 = w.y0.astype(np.float64)
    for over in (dict(B_stack=np.zeros_like(w.B)), dict(A_stack=np.zeros_like(w.A)),
                 dict(scale=0.0)):
        y, _ = _run(orc, w, **over)
        assert np.array_equal(y, y0), over.keys()
    y, _ = _run(orc, w)
    assert not np.array_equal(y, y0)


def pin_linear_in_scale_and_x(orc):
    """The correction is linear in s and in x."""
    w = _small(seed=6)
    y0 = w.y0.astype(np.float64)
    d1 = _run(orc, w)[0] - y0
    d2 = _run(orc, w, scale=2 * w.scale)[0] - y0
    _rel_close(d2, 2 * d1, 1e-12)
    d3 = _run(orc, w, scale=-0.75 * w.scale)[0] - y0
    _rel_close(d3, -0.75 * d1, 1e-12)
    rng = np.random.default_rng(7)
    # multiples of 2**-8 in [-4, 4]: their sum is exact in float32
    x1 = (rng.integers(-1024, 1025, size=w.x.shape) / 256.0).astype(np.float32)
    x2 = (rng.integers(-1024, 1025, size=w.x.shape) / 256.0).astype(np.float32)
    e1 = _run(orc, w, x=x1)[0] - y0
    e2 = _run(orc, w, x=x2)[0] - y0
    e12 = _run(orc, w, x=(x1 + x2))[0] - y0
    _rel_close(e12, e1 + e2, 1e-12)
    e3 = _run(orc, w, x=(3 * x1))[0] - y0
    _rel_close(e3, 3 * e1, 1e-12)


def pin_segment_permutation(orc):
    """Reordering segments with their ids (and the rows) reorders output rows."""
    w = _small(seed=8, R=17, S=5, allow_empty=False)
    y, v = _run(orc, w)
    perm = np.array([3, 0, 4, 2, 1])
    lens = np.diff(w.seg_indptr)
    rows = np.concatenate([np.arange(w.seg_indptr[s], w.seg_indptr[s + 1]) for s in perm])
    seg_p = wl.indptr_from_lengths(lens[perm])
    yp, vp = _run(orc, w, x=w.x[rows], y0=w.y0[rows], seg_indptr=seg_p,
                  adapter_ids=w.adapter_ids[perm])
    assert np.array_equal(yp, y[rows])
    assert np.array_equal(vp, v[rows])


def pin_adapter_relabel(orc):
    """Reordering the adapter stack together with the ids changes nothing."""
    w = _small(seed=9, N=6, S=5)
    y, _ = _run(orc, w)
    perm = np.array([2, 5, 0, 1, 4, 3])          # new slot j holds old adapter perm[j]
    inv = np.argsort(perm)
    yp, _ = _run(orc, w, A_stack=w.A[perm], B_stack=w.B[perm],
                 adapter_ids=inv[w.adapter_ids].astype(np.int32))
    assert np.array_equal(yp, y)


def pin_rows_outside_segments_untouched(orc):
    """Rows after the last segment keep y0 and get v = 0; empty segments are no-ops."""
    w = _small(seed=10, R=15, S=4, uncovered_tail=4)
    y, v = _run(orc, w)
    tail = slice(int(w.seg_indptr[-1]), w.num_rows)
    assert np.array_equal(y[tail], w.y0[tail].astype(np.float64))
    assert np.all(v[tail] == 0)
    # put an empty segment, naming another adapter, in front of every segment
    seg = [int(t) for t in w.seg_indptr]
    ids = [int(t) for t in w.adapter_ids]
    seg2, ids2 = [seg[0]], []
    for s in range(len(ids)):
        seg2 += [seg[s], seg[s + 1]]
        ids2 += [(ids[s] + 1) % w.num_adapters, ids[s]]
    ye, _ = _run(orc, w, seg_indptr=np.array(seg2, np.int32),
                 adapter_ids=np.array(ids2, np.int32))
    assert np.array_equal(ye, y)


def pin_split_merge_same_adapter(orc):
    """Cutting a segment in two pieces with the same adapter changes nothing."""
    w = _small(seed=11, R=12, S=1)
    y, _ = _run(orc, w)
    a = w.adapter_ids[0]
    for cut in (1, 5, 11):
        ys, _ = _run(orc, w, seg_indptr=np.array([0, cut, 12], np.int32),
                     adapter_ids=np.array([a, a], np.int32))
        assert np.array_equal(ys, y)


def pin_shrink_expand_compose(orc):
    """lora_apply equals expand(shrink(x)); shrink leaves uncovered rows as given."""
    w = _small(seed=12, R=14, S=4, uncovered_tail=3)
    y, v = _run(orc, w)
    v_init = np.full((w.num_rows, w.r), 7.25)
    vs = orc.shrink(w.x, w.A, w.seg_indptr, w.adapter_ids, v_init=v_init)
    cov = slice(0, int(w.seg_indptr[-1]))
    assert np.array_equal(vs[cov], v[cov])
    assert np.all(vs[int(w.seg_indptr[-1]):] == 7.25)
    ye = orc.expand(w.y0, v, w.B, w.seg_indptr, w.adapter_ids, w.scale)
    assert np.array_equal(ye, y)


def pin_rejects_malformed_tables(orc):
    w = _small(seed=13, R=8, S=2, allow_empty=False)
    bad = [
        (np.array([0, 5, 3], np.int32), w.adapter_ids),            # decreasing
        (np.array([0, 4, 9], np.int32), w.adapter_ids),            # past the last row
        (w.seg_indptr, np.array([0, w.num_adapters], np.int32)),   # id out of range
        (w.seg_indptr, np.array([-1, 0], np.int32)),               # negative id
    ]
    for seg, ids in bad:
        try:
            _run(orc, w, seg_indptr=seg, adapter_ids=ids)
        except ValueError:
            continue
        raise AssertionError(f"malformed table accepted: {seg} {ids}")


# -- the adapted linear layer (base product folded in) --------------------------

def _linear_case(seed, H1=24, H2=20, r=4, N=5, R=11, S=4, bias=True):
    w = _small(seed=seed, H1=H1, H2=H2, r=r, N=N, R=R, S=S)
    W, b = wl.base_layer(seed, "f32", H1, H2, bias=bias)
    return w, W, b


def pin_linear_single_segment_is_matmul(orc):
    """One segment over every row: y = x W^T + b + s (x A_a) B_a, numpy fp64."""
    w, W, b = _linear_case(21, H1=40, H2=28, r=6, R=9)
    seg, ids = np.array([0, 9], np.int32), np.array([3], np.int32)
    y = orc.lora_linear(w.x, W, b, w.A, w.B, seg, ids, w.scale)
    x = w.x.astype(np.float64)
    ref = (x @ W.T.astype(np.float64) + b.astype(np.float64)
           + w.scale * ((x @ w.A[3].astype(np.float64)) @ w.B[3].astype(np.float64)))
    _rel_close(y, ref, 1e-12)


def pin_linear_integer_exact(orc):
    """{-1,0,1} x, W, A, B and integer bias over several segments (one empty,
    one adapter named twice, uncovered rows at both ends): int64 arithmetic
    gives the exact answer, bit for bit."""
    w = wl.integer_exact(6, "f32", 72, 40, 8, 6, 26, 3, density=0.3, scale=2.0)
    W, b = wl.base_layer(6, "f32", 72, 40, integer=True, density=0.3)
    seg = np.array([2, 9, 9, 15, 23], np.int32)
    ids = np.array([4, 1, 4, 0], np.int32)
    y = orc.lora_linear(w.x, W, b, w.A, w.B, seg, ids, 2.0)
    xi = w.x.astype(np.int64)
    ref = xi @ W.astype(np.int64).T + b.astype(np.int64)
    for s in range(4):
        lo, hi, a = int(seg[s]), int(seg[s + 1]), int(ids[s])
        ref[lo:hi] += 2 * ((xi[lo:hi] @ w.A[a].astype(np.int64)) @ w.B[a].astype(np.int64))
    assert np.array_equal(y, ref.astype(np.float64))


def pin_linear_bias_and_uncovered_rows(orc):
    """No bias equals a zero bias; rows outside every segment get exactly the
    base product (numpy fp64), and the bias shifts every row by b."""
    w, W, b = _linear_case(22, R=13, S=3)
    seg = np.array([3, 5, 8, 10], np.int32)
    ids = np.array([1, 4, 2], np.int32)
    y_nb = orc.lora_linear(w.x, W, None, w.A, w.B, seg, ids, w.scale)
    y_zb = orc.lora_linear(w.x, W, np.zeros_like(b), w.A, w.B, seg, ids, w.scale)
    assert np.array_equal(y_nb, y_zb)
    y_b = orc.lora_linear(w.x, W, b, w.A, w.B, seg, ids, w.scale)
    _rel_close(y_b - y_nb, np.broadcast_to(b.astype(np.float64), y_b.shape), 1e-12)
    base = w.x.astype(np.float64) @ W.T.astype(np.float64)
    out = [0, 1, 2, 10, 11, 12]
    _rel_close(y_nb[out], base[out], 1e-12)
    assert not np.allclose(y_nb[3:10], base[3:10])


ALL_PINS = [
    pin_hand_worked_example,
    pin_single_segment_is_matmul,
    pin_gather_bmm_identity,
    pin_brute_force_tiny,
    pin_integer_exact,
    pin_zero_weights_or_scale_leave_y,
    pin_linear_in_scale_and_x,
    pin_segment_permutation,
    pin_adapter_relabel,
    pin_rows_outside_segments_untouched,
    pin_split_merge_same_adapter,
    pin_shrink_expand_compose,
    pin_rejects_malformed_tables,
    pin_linear_single_segment_is_matmul,
    pin_linear_integer_exact,
    pin_linear_bias_and_uncovered_rows,
]
