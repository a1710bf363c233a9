"""CPU oracle for segment tables built from per-row adapter ids -- TEST
INFRASTRUCTURE ONLY (imported by tests/, never by the HIP product library,
with which it shares no code).

A serving batch is tagged per row with the adapter each request uses (the
per-sample LoRA indices of Punica walkthrough, omica.com.cn/news/959180,
section 3.2), while SGMV consumes the batch as contiguous segments, each
naming one adapter (Punica review, nubint.ai, "Proposed method").  Two plain
definitions, written as loops over the rows:

* ``build_segments``: one segment per maximal run of equal ids in row order.
* ``group_rows``: the rows grouped by adapter in increasing id order, each
  group in increasing row order, then the rows without an adapter; one
  segment per adapter present.

Reading taken (the pages do not say): an id outside [0, num_adapters) means
"no adapter"; such a row belongs to no segment of the grouped table and to
segments with adapter id -1 in the run table.  The tables are padded with
empty segments to ``num_rows`` (runs) or ``min(num_rows, num_adapters)``
(grouping) entries, the form the device builders write.
"""
from __future__ import annotations


def _norm(a: int, num_adapters: int) -> int:
    return a if 0 <= a < num_adapters else -1


def build_segments(row_ids, num_adapters: int):
    """Run-length segments.  Returns (seg_indptr [R+1], adapter_ids [R],
    count) as Python lists and an int."""
    ids = [_norm(int(a), num_adapters) for a in row_ids]
    R = len(ids)
    seg, aid = [], []
    for i in range(R):
        if i == 0 or ids[i] != ids[i - 1]:
            seg.append(i)
            aid.append(ids[i])
    count = len(aid)
    seg += [R] * (R + 1 - count)
    aid += [-1] * (R - count)
    return seg, aid, count


def group_rows(row_ids, num_adapters: int):
    """Stable grouping.  Returns (perm [R], seg_indptr [M+1],
    adapter_ids [M], count) with M = min(R, num_adapters)."""
    ids = [_norm(int(a), num_adapters) for a in row_ids]
    R = len(ids)
    rows_of = {}
    for i in range(R):
        rows_of.setdefault(ids[i], []).append(i)
    perm, seg, aid = [], [], []
    for a in sorted(k for k in rows_of if k >= 0):
        seg.append(len(perm))
        aid.append(a)
        perm.extend(rows_of[a])
    grouped = len(perm)
    perm.extend(rows_of.get(-1, []))
    count = len(aid)
    M = min(R, num_adapters)  # at most one segment per adapter
    seg += [grouped] * (M + 1 - count)
    aid += [-1] * (M - count)
    return perm, seg, aid, count
