"""The dual-stream schedule of one MoE layer: the LoRA side on an auxiliary stream.

The prhub summary of vLLM PR #42290 (implementation steps 2 and 3; executive
summary) runs each of the layer's two projections as a fork and a join: the
LoRA delta (add_inputs = 0 into a zero-filled buffer) on an auxiliary stream
beside the base GEMM on the main one, then the delta added onto the base
output.  It uses four events -- fork and join of w13, fork and join of w2 --
so that no event is recorded again while a wait on it may still be pending.
vLLM PR #29257 (Purpose) likewise runs the base MoE align and the LoRA align
on two streams; here that is the w13 fork, where the LoRA align goes first on
the auxiliary stream.

This module only orders work: every step runs in the library's kernels (or
in whatever the caller's base callables launch).  Both streams keep the
default priority.  The schedule is graph-capturable: captured under
torch.cuda.graph, the fork and join become graph edges.
"""
from __future__ import annotations

import torch

from . import moe_lora_accumulate

W13, W2 = 0, 1


class LoraStreams:
    """One auxiliary stream and four events (fork / join of w13, fork / join of w2)."""

    def __init__(self, device=None):
        self.aux = torch.cuda.Stream(device=device)
        self.events = [torch.cuda.Event() for _ in range(4)]

    def fork_join(self, stage: int, base_fn, lora_fn, y=None, delta=None, lora_first=False):
        """Run lora_fn on the auxiliary stream beside base_fn on the current one.

        stage: W13 or W2 (selects the event pair).  lora_fn and base_fn are
        callables that enqueue work on the stream current when they are called.
        lora_fn may read what the current stream produced before this call;
        base_fn runs after the fork is recorded.  When y and delta are given,
        the join adds delta onto y (moe_lora_accumulate) on the current stream
        once both sides are done.  lora_first: enqueue the LoRA side before
        the base side (the base side goes first by default; the order changes
        no result, only which kernels reach the compute units first)."""
        if stage not in (W13, W2):
            raise ValueError("stage is W13 or W2")
        fork, join = self.events[2 * stage], self.events[2 * stage + 1]
        main = torch.cuda.current_stream()
        fork.record(main)
        self.aux.wait_event(fork)
        # Base side first by default.  Inside a captured graph, enqueuing the
        # LoRA side first made a layer's w2 fork cost about as much as the base
        # GEMM again (20b-like decode layer: 520 us, against 420 serial and 409
        # base first).  Launched eagerly, the order made no difference (455 us
        # either way in the same run).
        if not lora_first:
            base_fn()
        with torch.cuda.stream(self.aux):
            lora_fn()
            join.record(self.aux)
        if lora_first:
            base_fn()
        main.wait_event(join)
        if y is not None:
            moe_lora_accumulate(y, delta)
