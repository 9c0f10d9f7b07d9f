"""Replay of another run's draft-tree selections through the oracle's
arithmetic (test infrastructure).

The oracle's draft_tree asks a chooser for every selection it makes (a
node's children, each step's frontier, the final tree). `Replay` answers
with the recorded selections of another run (the GPU's), so the oracle
evaluates its own arithmetic along exactly those branches, and notes per
sequence how far each recorded selection falls below the best alternative in
the oracle's numbers ("margin": 0 when the two agree; inf when a recorded
child is not among the oracle's top `wide` logits of its row)."""
import numpy as np


class Replay:
    def __init__(self, C, follow, wide=16):
        self.C, self.f, self.wide = C, follow, wide
        self.B = np.asarray(follow["selected"]).shape[0]
        self.margin = {k: np.zeros(self.B) for k in ("lm", "frontier", "final")}

    def _note(self, kind, per_seq):
        self.margin[kind] = np.maximum(self.margin[kind], per_seq)

    def children(self, step, idx, val):
        C = self.C
        ids = np.asarray(self.f["ids"][step - 1]).reshape(-1, C).astype(np.int32)
        v = np.full(ids.shape, -np.inf)
        for r in range(ids.shape[0]):
            for j in range(C):
                hit = np.flatnonzero(idx[r] == ids[r, j])
                if len(hit):
                    v[r, j] = val[r, hit[0]]
        # the weakest recorded child against the C-th best logit of its row
        worst = np.maximum(val[:, C - 1] - v.min(axis=1), 0.0)
        self._note("lm", worst.reshape(self.B, -1).max(axis=1))
        return ids, v

    def _gap(self, score, chosen):
        lo = np.where(chosen, score, np.inf).min(axis=1)
        hi = np.where(chosen, -np.inf, score).max(axis=1)
        return np.where((~chosen).any(axis=1), np.maximum(hi - lo, 0.0), 0.0)

    def frontier(self, step, cand, start):
        order = np.asarray(self.f["frontier"][step - 1]).astype(np.int64)
        chosen = np.zeros(cand.shape, bool)
        np.put_along_axis(chosen, order, True, 1)
        self._note("frontier", self._gap(cand, chosen))
        return order

    def final(self, pool_score, N):
        sel = np.asarray(self.f["selected"]).astype(np.int64)
        chosen = np.zeros(pool_score.shape, bool)
        np.put_along_axis(chosen, sel, True, 1)
        self._note("final", self._gap(pool_score, chosen))
        return sel


def replay(orc, shape, W, l, m, h, ctx_tok, follow, vocab=None):
    """oracle.draft_tree along `follow`'s selections (with the trimmed draft
    vocabulary `vocab`, if any); the result carries the margins under
    "margin"."""
    ch = Replay(shape.topk, follow)
    r = orc.draft_tree(shape, W, l, m, h, ctx_tok, chooser=ch, vocab=vocab)
    r["margin"] = ch.margin
    return r
