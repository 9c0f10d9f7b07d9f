"""Lossless pin on a tiny random-weight decoder (CPU only).

The course lesson states that greedy tree verification emits exactly what
the target would emit decoding one token at a time. Plain greedy decoding is
the reference here: speculative output must be token-identical to it, for
every seed and tree shape, and the acceptance lengths must follow the planted
match probability (all matches: the full depth; none: one token per step).
"""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("seed", range(5))
def test_speculative_equals_greedy(orc, seed):
    greedy, _ = orc.toy_greedy(seed=seed)
    spec, steps = orc.toy_speculative(seed=seed)
    assert len(greedy) == synth.TOY.new_tokens
    assert np.array_equal(spec, greedy)
    assert 1 + sum(s["accept_len"] + 1 for s in steps) >= synth.TOY.new_tokens   # prefill emits one


@pytest.mark.parametrize("tree", ["chain4", "lesson", "chain1"])
def test_speculative_equals_greedy_other_trees(orc, tree):
    parent = {"chain4": synth.chain_tree(4), "lesson": synth.lesson_tree_7(), "chain1": synth.chain_tree(1)}[tree]
    greedy, _ = orc.toy_greedy(seed=1, n_new=40)
    spec, _ = orc.toy_speculative(seed=1, n_new=40, parent=parent)
    assert np.array_equal(spec, greedy)


def test_all_match_accepts_full_depth_and_none_gives_one(orc):
    greedy, _ = orc.toy_greedy(seed=2, n_new=30)
    spec, steps = orc.toy_speculative(seed=2, n_new=30, p_match=1.0)
    assert np.array_equal(spec, greedy)
    assert all(s["accept_len"] == 4 for s in steps)
    spec0, steps0 = orc.toy_speculative(seed=2, n_new=12, p_match=0.0)
    assert np.array_equal(spec0, greedy[:12])
    # a random id matches only by chance (1/4096 per edge)
    assert sum(s["accept_len"] for s in steps0) <= 1
