"""Speculative decoding that stays on the device: each step drafts a tree
with the EAGLE-3 draft head, runs the target model's pass over it, accepts
the longest matching root path, commits the accepted rows' K/V to every
target layer, and extends the draft's context with those rows (course lesson
"EAGLE-3 speculative decoding: the tree-verifier method", "Verify-accept
semantics"; news write-up of the EAGLE-3 paper, draft stage: the draft reads
the target's low / mid / high features of every committed token together
with the embedding of the token after it).

One step is a fixed sequence of kernel launches on one stream with no host
read in between, so it can be captured once in a HIP graph and replayed:
every quantity that varies per step (sequence lengths, the next root, the
accepted rows) lives in device buffers that the kernels read and write.

Order within a step: draft.grow (positions from the shared lengths, root
from the previous step) -> target.run (positions, attention prefixes) ->
eagle3_spec_advance (old lengths to `start`, lengths += accept_len + 1,
accepted rows and their next tokens, next root, emitted tokens) ->
target.commit(start) -> draft.extend (K/V of the new context rows at start..,
the full draft layer at the end node -> a_root for the next tree).
"""
from __future__ import annotations

import torch

from . import binding as B_


class SpecLoop:
    def __init__(self, target, draft, cap: int):
        """target: TargetModel whose features are (low, mid, high); draft:
        DraftHead built with prefix_len=target.plen and extend_rows >= the
        draft tree's depth + 1; cap: emitted tokens kept per sequence."""
        if draft.plen is not target.plen:
            raise ValueError("the draft and the target must share one prefix_len tensor")
        if len(target.features) != 3:
            raise ValueError("the target must keep three feature layers (low, mid, high)")
        if draft.R < draft.steps + 1:
            raise ValueError("extend_rows must cover the deepest accepted path (draft steps + 1)")
        if draft.N + 1 != target.T or draft.B != target.B:
            raise ValueError("the draft tree and the target pass differ in size")
        self.t, self.d = target, draft
        B, R, dv = draft.B, draft.R, draft.dev
        i32 = dict(dtype=torch.int32, device=dv)
        self.start = torch.empty(B, **i32)
        self.path_rows = torch.empty(B, R, **i32)
        self.tok_ahead = torch.empty(B, R, **i32)
        self.last_rows = torch.empty(B, **i32)
        self.out_seq = torch.full((B, cap), -1, **i32)
        self.out_len = torch.zeros(B, **i32)

    def step(self):
        t, d = self.t, self.d
        d.grow()
        t.run(d.parent, d.tokens)
        B_.eagle3_spec_advance(t.accept_len, t.path, t.out_tokens, t.plen, self.start, self.path_rows,
                               self.tok_ahead, self.last_rows, d.root, self.out_seq, self.out_len)
        t.commit(self.start)
        lo, mid, hi = (t.feat[i] for i in t.features)
        d.extend(lo, mid, hi, self.path_rows, self.tok_ahead, self.start, self.last_rows)

    def graph(self):
        """Capture one step in a HIP graph (call after at least one eager step,
        so every workspace is sized); each replay runs the next step."""
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        return g
