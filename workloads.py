"""Seeded synthetic inputs for SGMV, shared by the tests and the benchmark.

This module only draws numbers and builds segment tables; it holds none of
the method's arithmetic, and both the CPU oracle and the HIP library receive
exactly the arrays it returns.

Shapes follow the Llama-7B/13B projection sizes the workloads are quoted on;
no model weights or datasets are involved.  Every generator uses
``numpy.random.default_rng(seed)`` and draws in a fixed order: the segment
structure first, then x, A_stack, B_stack and y0.  Distributions:
x ~ N(0, 1), A ~ U(-1/sqrt(H1), 1/sqrt(H1)), B ~ N(0, std 1/sqrt(r)),
y0 ~ N(0, 1).  Draws are float32 and are then rounded to the working dtype
with round-to-nearest-even; the float32 arrays handed out hold those rounded
values exactly, so the oracle (which reads them as float) and the GPU (which
reads the dtype copy) see identical inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp32/fp16/bf16 (nearest-even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        # Finite inputs only (the generators draw finite values), so adding
        # the rounding bias cannot carry out of 32 bits.
        bits = a.view(np.uint32)
        out = bits + np.uint32(0x7FFF)
        out += (bits >> np.uint32(16)) & np.uint32(1)
        out &= np.uint32(0xFFFF0000)
        return out.view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class Workload:
    """One SGMV problem: inputs plus the segment table.

    x [R, H1], A [N, H1, r], B [N, r, H2], y0 [R, H2] are float32 arrays that
    hold dtype-rounded values; seg_indptr [S+1] and adapter_ids [S] are int32.
    """

    name: str
    dtype: str
    H1: int
    H2: int
    r: int
    num_adapters: int
    seg_indptr: np.ndarray
    adapter_ids: np.ndarray
    scale: float
    x: np.ndarray
    A: np.ndarray
    B: np.ndarray
    y0: np.ndarray
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def num_rows(self) -> int:
        return int(self.x.shape[0])

    @property
    def num_segments(self) -> int:
        return int(self.adapter_ids.shape[0])

    @property
    def seg_lengths(self) -> np.ndarray:
        return np.diff(self.seg_indptr)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def indptr_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(lengths)
    return out


def largest_remainder(weights, total: int) -> np.ndarray:
    """Integer lengths proportional to ``weights`` that sum to ``total``.

    Floors the exact shares, then hands the leftover units to the largest
    fractional parts (ties to the earlier index).
    """
    w = np.asarray(weights, dtype=np.float64)
    exact = w * (total / w.sum())
    base = np.floor(exact).astype(np.int64)
    left = int(total - base.sum())
    order = np.argsort(-(exact - base), kind="stable")
    base[order[:left]] += 1
    return base


def zipf_lengths(total: int, count: int, s: float) -> np.ndarray:
    """Segment lengths following Zipf(s) over ``count`` ranks, summing to total."""
    k = np.arange(1, count + 1, dtype=np.float64)
    return largest_remainder(k ** (-s), total)


def _draw_tensors(rng, R, H1, H2, r, N, dtype):
    x = rng.standard_normal((R, H1), dtype=np.float32)
    bound = np.float32(1.0 / np.sqrt(H1))
    A = (rng.random((N, H1, r), dtype=np.float32) * (2 * bound) - bound).astype(np.float32)
    B = rng.standard_normal((N, r, H2), dtype=np.float32) * np.float32(1.0 / np.sqrt(r))
    y0 = rng.standard_normal((R, H2), dtype=np.float32)
    return (round_to_dtype(x, dtype), round_to_dtype(A, dtype),
            round_to_dtype(B, dtype), round_to_dtype(y0, dtype))


def make_workload(name, dtype, H1, H2, r, num_adapters, lengths, adapter_ids, scale,
                  seed=0, rng=None, num_rows=None, note="") -> Workload:
    """Draw x, A, B, y0 for a given segment structure (structure first, then tensors)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    seg = indptr_from_lengths(lengths)
    R = int(seg[-1]) if num_rows is None else int(num_rows)
    x, A, B, y0 = _draw_tensors(rng, R, H1, H2, r, num_adapters, dtype)
    return Workload(name, dtype, H1, H2, r, num_adapters, seg,
                    np.asarray(adapter_ids, dtype=np.int32), float(scale), x, A, B, y0, note)


# -- the five reference workloads ---------------------------------------------

def tiny(seed=0) -> Workload:
    """256 -> 256, r=8, 4 adapters, 16 rows in 4 segments of 4 rows, fp32, s=1."""
    return make_workload("tiny_sgmv_256x256_r8", "f32", 256, 256, 8, 4, [4, 4, 4, 4],
                         [0, 1, 2, 3], 1.0, seed=seed)


def llama7b_decode(seed=0) -> Workload:
    """Llama-2-7B decode: 4096 -> 4096, r=16, 64 adapters, 64 one-row segments
    (adapter i for row i), fp16, s = alpha/r = 2."""
    return make_workload("llama7b_decode_4096_r16_64x1", "f16", 4096, 4096, 16, 64,
                         [1] * 64, list(range(64)), 2.0, seed=seed)


def skewed_decode(seed=0, control=False) -> Workload:
    """Skewed multi-tenant decode: 4096 -> 4096, r=16, 256 stacked adapters, 128
    rows in 32 segments with Zipf(1.1) lengths over 32 adapters chosen at
    random; ``control=True`` puts all 128 rows in one segment (the first chosen
    adapter).  fp16, s=2."""
    rng = np.random.default_rng(seed)
    chosen = rng.choice(256, size=32, replace=False).astype(np.int32)
    lengths = zipf_lengths(128, 32, 1.1)
    if control:
        name, lengths, ids = "skewed_decode_control_1x128", [128], [int(chosen[0])]
    else:
        name, ids = "skewed_decode_zipf_4096_r16_32seg", chosen
    w = make_workload(name, "f16", 4096, 4096, 16, 256, lengths, ids, 2.0, rng=rng)
    w.extra["chosen_adapters"] = chosen.tolist()
    return w


def prefill(seed=0) -> Workload:
    """Prefill: 4096 -> 4096, r=16, 16 adapters, 4096 rows in 16 segments whose
    lengths are U(64, 512) draws rescaled to sum to 4096, fp16, s=2."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(64.0, 512.0, size=16)
    lengths = largest_remainder(u, 4096)
    return make_workload("prefill_4096_r16_16seg", "f16", 4096, 4096, 16, 16, lengths,
                         list(range(16)), 2.0, rng=rng)


def mlp_up_decode(seed=0) -> Workload:
    """Llama-13B up-projection shape: 5120 -> 13824, r=64, 512 stacked adapters,
    256 decode rows each assigned uniformly to one of 128 adapters drawn from
    the 512, rows sorted by adapter so equal ids form segments, bf16, s=0.5."""
    rng = np.random.default_rng(seed)
    chosen = rng.choice(512, size=128, replace=False).astype(np.int32)
    per_row = rng.choice(chosen, size=256)
    per_row = np.sort(per_row, kind="stable")
    ids, lengths = np.unique(per_row, return_counts=True)
    return make_workload("llama13b_up_5120x13824_r64_decode", "bf16", 5120, 13824, 64, 512,
                         lengths, ids, 0.5, rng=rng)


def mixed_batch(seed=0, long_rows=(512, 512), short=128, H=4096, r=16, dtype="f16",
                num_adapters=256) -> Workload:
    """A serving batch that mixes prefill and decode requests: segments of
    ``long_rows`` rows (prefill prompts) and ``short`` one-row segments
    (decode steps), each segment on its own adapter, the adapters drawn
    without replacement from a stack of ``num_adapters``, the segment order
    shuffled.  4096 -> 4096, r=16, fp16, s=2 by default (two 512-row
    segments plus 128 one-row segments: 1152 rows over 130 adapters)."""
    rng = np.random.default_rng(seed)
    lengths = np.array(list(long_rows) + [1] * short, dtype=np.int64)
    order = rng.permutation(len(lengths))
    lengths = lengths[order]
    ids = rng.choice(num_adapters, size=len(lengths), replace=False).astype(np.int32)
    name = f"mixed_{H}_r{r}_{'+'.join(map(str, long_rows))}+{short}x1"
    return make_workload(name, dtype, H, H, r, num_adapters, lengths, ids, 32.0 / r, rng=rng)


def decode_batch(rows: int, distinct: bool = True, seed=0, H=4096, r=16, dtype="f16",
                 num_adapters=256) -> Workload:
    """A decode batch of ``rows`` rows at the Llama-2-7B projection shape:
    every row its own one-row segment on its own adapter (``distinct``,
    adapters 0..rows-1), or all rows one segment on adapter 0 -- the two
    ends of the pages' comparison of distinct and identical models in a
    batch.  fp16, s = 2."""
    if distinct:
        lengths, ids = [1] * rows, list(range(rows))
    else:
        lengths, ids = [rows], [0]
    name = f"decode_{'distinct' if distinct else 'same'}_{H}_r{r}_{rows}rows"
    return make_workload(name, dtype, H, H, r, num_adapters, lengths, ids, 32.0 / r, seed=seed)


CONFIGS = {
    0: tiny,
    1: llama7b_decode,
    2: skewed_decode,
    3: prefill,
    4: mlp_up_decode,
}


def config(i: int, seed: int = 0, control: bool = False) -> Workload:
    if i == 2:
        return skewed_decode(seed, control=control)
    return CONFIGS[i](seed)


# -- small and special inputs for tests ----------------------------------------

def random_segments(rng, num_rows, num_segments, num_adapters, allow_empty=True,
                    uncovered_tail=0):
    """A random valid segment table over the first num_rows - uncovered_tail rows."""
    covered = num_rows - uncovered_tail
    if num_segments == 0:
        return np.zeros(1, dtype=np.int32), np.zeros(0, dtype=np.int32)
    if allow_empty:
        cuts = np.sort(rng.integers(0, covered + 1, size=num_segments - 1))
    else:
        cuts = np.sort(rng.choice(np.arange(1, covered), size=num_segments - 1, replace=False))
    seg = np.concatenate([[0], cuts, [covered]]).astype(np.int32)
    ids = rng.integers(0, num_adapters, size=num_segments).astype(np.int32)
    return seg, ids


def small_random(seed, dtype, H1, H2, r, num_adapters, num_rows, num_segments,
                 allow_empty=True, uncovered_tail=0, scale=1.5) -> Workload:
    rng = np.random.default_rng(seed)
    seg, ids = random_segments(rng, num_rows, num_segments, num_adapters, allow_empty,
                               uncovered_tail)
    x, A, B, y0 = _draw_tensors(rng, num_rows, H1, H2, r, num_adapters, dtype)
    return Workload(f"random_{dtype}_{H1}x{H2}_r{r}_R{num_rows}_S{num_segments}", dtype,
                    H1, H2, r, num_adapters, seg, ids, float(scale), x, A, B, y0)


def integer_exact(seed, dtype, H1, H2, r, num_adapters, num_rows, num_segments,
                  density=0.05, scale=2.0) -> Workload:
    """Sparse {-1, 0, 1} x, A, B and small-integer y0.

    Every partial sum of the add-on is then a small integer, exact in float32
    and in any summation order, so any correct implementation that
    accumulates in float32 or wider returns the exact value.
    """
    rng = np.random.default_rng(seed)
    seg, ids = random_segments(rng, num_rows, num_segments, num_adapters, True, 0)

    def tern(shape):
        mag = rng.random(shape) < density
        sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
        return (mag * sign).astype(np.float32)

    x = tern((num_rows, H1))
    A = tern((num_adapters, H1, r))
    B = tern((num_adapters, r, H2))
    y0 = rng.integers(-8, 9, size=(num_rows, H2)).astype(np.float32)
    return Workload(f"intexact_{dtype}_{H1}x{H2}_r{r}", dtype, H1, H2, r, num_adapters,
                    seg, ids, float(scale), x, A, B, y0)


# -- base layer of an adapted linear layer --------------------------------------

def base_layer(seed, dtype, H1, H2, bias=True, integer=False, density=0.05):
    """Weight W [H2, H1] (one row per output feature) and bias [H2] or None.

    From their own generator, numpy.random.default_rng(seed + 1000003), so
    that adding a base layer changes none of a workload's other draws.
    Floating: W and bias ~ U(-1/sqrt(H1), 1/sqrt(H1)), the usual initial
    range of a linear layer, rounded to the dtype.  integer=True: W sparse
    {-1, 0, 1} with the given density and bias small integers, so that with
    the integer_exact add-on every partial sum is a small integer.
    """
    rng = np.random.default_rng(seed + 1000003)
    if integer:
        mag = rng.random((H2, H1)) < density
        sign = np.where(rng.random((H2, H1)) < 0.5, -1.0, 1.0)
        W = (mag * sign).astype(np.float32)
        b = rng.integers(-8, 9, size=H2).astype(np.float32) if bias else None
        return W, b
    bound = np.float32(1.0 / np.sqrt(H1))
    W = rng.random((H2, H1), dtype=np.float32) * (2 * bound) - bound
    b = (rng.random(H2, dtype=np.float32) * (2 * bound) - bound) if bias else None
    return round_to_dtype(W, dtype), (None if b is None else round_to_dtype(b, dtype))
