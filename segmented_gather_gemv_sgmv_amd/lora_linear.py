"""A linear layer with per-row LoRA adapters, served by SGMV.

    y = x W^T (+ b) + scale * (x A_a) B_a,   a = row_ids[i] for row i

which is the adapted layer y = xW + xAB of Punica walkthrough
(omica.com.cn/news/959180, section 2.1) evaluated for a batch whose rows
each carry their own adapter index (same page, section 3.2).  The base
product is an ordinary dense GEMM (torch's `linear`); the LoRA add-on goes
through the library: the per-row ids become a segment table on the device
(`build_segments`, or `group_rows` when rows of one adapter are scattered
through the batch and should share their weight reads), then `lora_apply`
adds the correction in place.  Rows whose id is not an adapter get the base
output only.  Nothing is read back to the host.

Which table: the run table has one entry per row (runs of equal ids, padded
with empty segments, since their number is known only on the device), the
grouped table one entry per adapter present (padded to min(rows,
adapters)).  The library sizes its grid from the table's length, so a long
padded table over few real segments makes it launch many workgroups that
find no work; ``group="auto"`` (the default) therefore groups when the batch
has more rows than there are adapters, where rows necessarily share
adapters, and keeps the cheaper run table otherwise (decode batches).
"""
from __future__ import annotations

import torch

from . import build_segments, group_rows, lora_apply


class LoRALinear(torch.nn.Module):
    """Base weight [H2, H1] (torch's linear layout), optional bias [H2], and
    the adapter stacks A_stack [N, H1, r], B_stack [N, r, H2] (all one dtype,
    on one GPU).  ``group=True`` reorders the rows by adapter before the
    add-on (one segment per adapter) and back after it; ``group=False``
    keeps the batch order with one segment per run of equal ids;
    ``group="auto"`` groups when the batch has more rows than adapters."""

    def __init__(self, weight, A_stack, B_stack, scale: float = 1.0, bias=None,
                 group="auto"):
        super().__init__()
        if A_stack.dim() != 3 or B_stack.dim() != 3:
            raise ValueError("A_stack and B_stack must be [N, H1, r] and [N, r, H2]")
        N, H1, r = A_stack.shape
        if weight.shape[1] != H1 or B_stack.shape != (N, r, weight.shape[0]):
            raise ValueError("weight, A_stack and B_stack disagree on H1, H2, r or N")
        self.weight = torch.nn.Parameter(weight, requires_grad=False)
        self.bias = None if bias is None else torch.nn.Parameter(bias, requires_grad=False)
        self.register_buffer("A_stack", A_stack.contiguous())
        self.register_buffer("B_stack", B_stack.contiguous())
        self.scale = float(scale)
        if group not in (True, False, "auto"):
            raise ValueError("group must be True, False or 'auto'")
        self.group = group

    @property
    def num_adapters(self) -> int:
        return self.A_stack.shape[0]

    def forward(self, x, row_ids, workspace=None):
        """x [R, H1]; row_ids [R] int32 on the same device.  ``workspace`` is
        passed to lora_apply (required when the call is captured in a
        graph)."""
        x = x.contiguous()
        y = torch.nn.functional.linear(x, self.weight, self.bias).contiguous()
        group = self.group
        if group == "auto":
            group = x.shape[0] > self.num_adapters
        if not group:
            seg, ids, _ = build_segments(row_ids, self.num_adapters)
            return lora_apply(y, x, self.A_stack, self.B_stack, seg, ids, self.scale,
                              workspace=workspace)
        perm, seg, ids, _ = group_rows(row_ids, self.num_adapters)
        p = perm.long()
        yg = y.index_select(0, p)
        lora_apply(yg, x.index_select(0, p), self.A_stack, self.B_stack, seg, ids, self.scale,
                   workspace=workspace)
        y[p] = yg
        return y
