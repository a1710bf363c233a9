"""Pins of the segment-table oracle (oracle/segments.py) against a
hand-worked example, a library routine (numpy's stable argsort) and the
invariants that define the two tables; planted mistakes must fail them."""
import json
import os

import numpy as np
import pytest

from oracle import segments as og

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "segments_hand_worked.json")


def _cases():
    rng = np.random.default_rng(7)
    out = [([], 4), ([2], 4), ([-3], 4), ([1, 1, 1, 1], 2), ([0, 1, 0, 1, 0], 2)]
    for R, N in [(17, 3), (100, 8), (1500, 40), (3000, 600)]:
        ids = rng.integers(-2, N + 2, size=R)
        out.append((ids.tolist(), N))
        out.append((np.sort(rng.integers(0, N, size=R)).tolist(), N))
    return out


CASES = _cases()


def check_runs(row_ids, N, seg, aid, count):
    R = len(row_ids)
    norm = [a if 0 <= a < N else -1 for a in row_ids]
    assert len(seg) == R + 1 and len(aid) == R and 0 <= count <= R
    assert seg[0] == 0 and all(seg[k] <= seg[k + 1] for k in range(R))
    assert all(seg[k] == R for k in range(count, R + 1))
    assert all(aid[k] == -1 for k in range(count, R))
    # expanding the segments gives back the normalised ids, row by row
    rebuilt = []
    for k in range(count):
        assert seg[k] < seg[k + 1], "real segments are non-empty"
        rebuilt += [aid[k]] * (seg[k + 1] - seg[k])
    assert rebuilt == norm
    # maximal runs: neighbours differ
    assert all(aid[k] != aid[k + 1] for k in range(count - 1))


def check_grouped(row_ids, N, perm, seg, aid, count):
    R = len(row_ids)
    norm = [a if 0 <= a < N else -1 for a in row_ids]
    assert sorted(perm) == list(range(R)), "perm is a permutation"
    grouped = sum(1 for a in norm if a >= 0)
    M = min(R, N)
    assert len(seg) == M + 1 and len(aid) == M
    assert all(seg[k] == grouped for k in range(count, M + 1))
    assert all(aid[k] == -1 for k in range(count, M))
    assert [aid[k] for k in range(count)] == sorted(set(a for a in norm if a >= 0))
    assert seg[0] == 0
    for k in range(count):
        rows = perm[seg[k]:seg[k + 1]]
        assert rows and all(norm[i] == aid[k] for i in rows)
        assert rows == sorted(rows), "stable within an adapter"
    tail = perm[grouped:]
    assert all(norm[i] == -1 for i in tail) and tail == sorted(tail)


def test_hand_worked_example():
    g = json.load(open(GOLDEN))
    seg, aid, count = og.build_segments(g["row_ids"], g["num_adapters"])
    assert (seg, aid, count) == (g["runs"]["seg_indptr"], g["runs"]["adapter_ids"],
                                 g["runs"]["count"])
    perm, seg, aid, count = og.group_rows(g["row_ids"], g["num_adapters"])
    assert (perm, seg, aid, count) == (g["grouped"]["perm"], g["grouped"]["seg_indptr"],
                                       g["grouped"]["adapter_ids"], g["grouped"]["count"])


@pytest.mark.parametrize("case", range(len(CASES)))
def test_run_table_invariants(case):
    row_ids, N = CASES[case]
    check_runs(row_ids, N, *og.build_segments(row_ids, N))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_grouping_invariants_and_stable_sort(case):
    row_ids, N = CASES[case]
    perm, seg, aid, count = og.group_rows(row_ids, N)
    check_grouped(row_ids, N, perm, seg, aid, count)
    # library routine: a stable argsort by adapter, rows without one last
    keys = np.array([a if 0 <= a < N else N for a in row_ids], dtype=np.int64)
    assert perm == np.argsort(keys, kind="stable").tolist()


def _mutant_runs_split_every_row(row_ids, N):
    seg, aid, count = og.build_segments(row_ids, N)
    R = len(row_ids)
    norm = [a if 0 <= a < N else -1 for a in row_ids]
    return list(range(R)) + [R], norm, R


def _mutant_runs_raw_ids(row_ids, N):
    return og.build_segments(row_ids, 1 << 30)  # out-of-range ids kept as adapters


def _mutant_group_unstable(row_ids, N):
    perm, seg, aid, count = og.group_rows(row_ids, N)
    for k in range(count):
        perm[seg[k]:seg[k + 1]] = perm[seg[k]:seg[k + 1]][::-1]
    return perm, seg, aid, count


def _mutant_group_tail_first(row_ids, N):
    perm, seg, aid, count = og.group_rows(row_ids, N)
    grouped = seg[count]
    return perm[grouped:] + perm[:grouped], seg, aid, count


def _mutant_group_bad_padding(row_ids, N):
    perm, seg, aid, count = og.group_rows(row_ids, N)
    return perm, seg[:count + 1] + [len(row_ids)] * (len(seg) - count - 1), aid, count


@pytest.mark.parametrize("mutant", [_mutant_runs_split_every_row, _mutant_runs_raw_ids])
def test_run_pins_catch_mutants(mutant):
    failed = False
    for row_ids, N in CASES + [(json.load(open(GOLDEN))["row_ids"], 5)]:
        try:
            check_runs(row_ids, N, *mutant(row_ids, N))
        except AssertionError:
            failed = True
    assert failed, "a planted mistake passed every pin"


@pytest.mark.parametrize("mutant", [_mutant_group_unstable, _mutant_group_tail_first,
                                    _mutant_group_bad_padding])
def test_grouping_pins_catch_mutants(mutant):
    failed = False
    for row_ids, N in CASES + [(json.load(open(GOLDEN))["row_ids"], 5)]:
        try:
            check_grouped(row_ids, N, *mutant(row_ids, N))
        except AssertionError:
            failed = True
    assert failed, "a planted mistake passed every pin"
