"""Pins for the oracle's tree mask and greedy acceptance (CPU only).

What fixes the answers here, independently of oracle.c:
* the course lesson's worked chain cases (5 guesses: 4 right -> 5 tokens,
  1 right -> 2, none right -> 1) and its 7-node example tree with 4 paths
  (tests/golden/lesson_cases.json);
* the fully matching / fully mismatching trees (accept the full depth /
  emit exactly one token);
* an independent acceptance formula, written here with a reachability matrix
  and bit tests instead of path enumeration, checked exhaustively on all 2^15
  match patterns of the 15-draft binary tree and on thousands of random trees;
* the closed-form expected acceptance length under independent per-edge
  matches, checked statistically, and under ranked sibling matches (siblings
  as alternatives) on chains, random top-k trees and the best-first trees of
  a calibrated drafter;
* the best-first tree (synth.ranked_tree) against brute-force enumeration of
  every rank path of a small tree, and its expected acceptance length against
  a chain of the same size.
"""
import itertools
import json
import os

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "lesson_cases.json")


def reach(parent):
    """anc[n, t] = t is n or an ancestor of n, by transitive closure of the
    child->parent relation (boolean matrix squaring), not by walking."""
    T = len(parent)
    A = np.eye(T, dtype=bool)
    for n in range(1, T):
        A[n, parent[n]] = True
    for _ in range(int(np.ceil(np.log2(max(T, 2)))) + 1):
        A = (A.astype(np.int64) @ A.astype(np.int64)) > 0
    return A


def accept_by_reachability(parent, tokens, idx):
    """Node n accepted iff every node on its ancestor chain other than the
    root matches the target's argmax at that node's parent."""
    T = len(parent)
    anc = reach(parent)
    ok = np.ones(T, dtype=bool)
    ok[1:] = tokens[1:] == idx[parent[1:]]
    accepted = np.array([bool(np.all(ok[anc[n]])) for n in range(T)])
    depth = anc.sum(axis=1) - 1
    a = int(depth[accepted].max())
    end = int(np.flatnonzero(accepted & (depth == a)).min())
    chain = np.flatnonzero(anc[end])          # ancestors ascending = root first
    out = list(tokens[chain[1:]]) + [idx[end]]
    return a, end, chain, out


def test_tree_mask_matches_reachability(orc):
    rng = np.random.default_rng(7)
    for T in (1, 2, 16, 61, 64, 65, 128):
        parent = synth.random_tree(rng, T)
        mask, depth = orc.tree_mask(parent)
        anc = reach(parent)
        bits = np.zeros((T, T), dtype=bool)
        for n in range(T):
            for t in range(T):
                bits[n, t] = (int(mask[0, n, t // 64]) >> (t % 64)) & 1
        assert np.array_equal(bits, anc)
        assert np.array_equal(depth[0], anc.sum(axis=1) - 1)


def test_tree_check_rejects_bad_trees(orc):
    assert orc.tree_check(np.array([-1, 0, 1]))
    assert not orc.tree_check(np.array([0, 0, 1]))        # root must have parent -1
    assert not orc.tree_check(np.array([-1, 2, 0]))       # parent after child
    assert not orc.tree_check(np.array([-1, 1]))          # self loop
    with pytest.raises(ValueError):
        orc.tree_mask(np.array([-1, 0, 3, 1]))


def test_lesson_chain_cases(orc):
    g = json.load(open(GOLD))
    rng = np.random.default_rng(1)
    for case in g["chain_cases"]:
        n = case["drafts"]
        parent = synth.chain_tree(n)
        idx = rng.integers(0, 1000, size=n + 1).astype(np.int32)
        tok = (idx[parent.clip(0)] + 1).astype(np.int32)    # every draft wrong ...
        for i in range(1, case["first_correct"] + 1):       # ... except the first few
            tok[i] = idx[i - 1]
        alen, path, out, end = orc.accept(tok, parent, idx)
        emitted = out[0][out[0] >= 0]
        assert len(emitted) == case["tokens_out"]
        assert alen[0] == case["first_correct"]
        assert list(emitted[:-1]) == list(tok[1:1 + case["first_correct"]])
        assert emitted[-1] == idx[case["first_correct"]]


def test_lesson_tree_paths(orc):
    g = json.load(open(GOLD))["lesson_tree"]
    parent = np.array(g["parent"], np.int32)
    assert np.array_equal(parent, synth.lesson_tree_7())
    has_child = np.zeros(len(parent), bool)
    has_child[parent[1:]] = True
    leaves = np.flatnonzero(~has_child)
    assert list(leaves) == g["leaves"] and len(leaves) == g["paths"]
    # a miss at d2a must not stop d2b's branch: accept along root-d1-d2b-d3c
    idx = np.arange(100, 108, dtype=np.int32)
    tok = np.full(8, 999, np.int32)
    tok[1] = idx[0]; tok[3] = idx[1]; tok[6] = idx[3]
    alen, path, out, end = orc.accept(tok, parent, idx)
    assert alen[0] == 3 and end[0] == 6
    assert list(path[0, :4]) == [0, 1, 3, 6]
    assert list(out[0, :4]) == [tok[1], tok[3], tok[6], idx[6]]


@pytest.mark.parametrize("depth,n", [(7, 60), (8, 60), (3, 10)])
def test_full_match_and_full_mismatch(orc, depth, n):
    rng = np.random.default_rng(depth * 100 + n)
    for _ in range(20):
        parent = synth.topk_tree(rng, n, depth, 10)
        T = n + 1
        idx = rng.integers(0, 128256, size=T).astype(np.int32)
        tok = idx[np.maximum(parent, 0)].astype(np.int32)
        tok[0] = 5
        alen, path, out, end = orc.accept(tok, parent, idx)
        assert alen[0] == depth                      # full depth accepted
        assert np.sum(out[0] >= 0) == depth + 1      # tau = depth + 1
        bad = (idx[np.maximum(parent, 0)] + 1).astype(np.int32)
        alen, path, out, end = orc.accept(bad, parent, idx)
        assert alen[0] == 0 and end[0] == 0
        assert list(out[0][out[0] >= 0]) == [idx[0]]  # exactly one token


def test_exhaustive_binary_tree(orc):
    parent = synth.binary_tree_15()
    T = 16
    idx = (np.arange(T) * 7 + 3).astype(np.int32)
    pats = np.array(list(itertools.product([False, True], repeat=15)))
    B = pats.shape[0]
    tok = np.tile((idx[np.maximum(parent, 0)] + 1000).astype(np.int32), (B, 1))
    match = idx[parent[1:]]
    tok[:, 1:] = np.where(pats, match[None, :], tok[:, 1:])
    alen, path, out, end = orc.accept(tok, np.tile(parent, (B, 1)), np.tile(idx, (B, 1)))
    for b in range(0, B, 1):
        a, e, chain, o = accept_by_reachability(parent, tok[b], idx)
        assert alen[b] == a and end[b] == e, b
        assert list(path[b, :a + 1]) == list(chain) and list(out[b, :a + 1]) == o


@pytest.mark.parametrize("T", [2, 5, 17, 33, 64, 100])
def test_random_trees_against_reachability(orc, T):
    rng = np.random.default_rng(T)
    B = 1500 if T <= 64 else 300
    parents = np.stack([synth.random_tree(rng, T, max_children=int(rng.integers(1, 6))) for _ in range(B)])
    idx = rng.integers(0, 50, size=(B, T)).astype(np.int32)
    p = rng.uniform(0.3, 1.0, size=B)
    tok = rng.integers(0, 50, size=(B, T)).astype(np.int32)
    for b in range(B):
        m = rng.random(T) < p[b]
        tok[b, m] = idx[b, np.maximum(parents[b], 0)][m]
    alen, path, out, end = orc.accept(tok, parents, idx)
    for b in range(B):
        a, e, chain, o = accept_by_reachability(parents[b], tok[b], idx[b])
        assert (alen[b], end[b]) == (a, e)
        assert list(out[b, :a + 1]) == o and np.all(out[b, a + 1:] == -1)


def closed_form_tau(parent, p, V):
    """E[tau] = 1 + sum_d P(some root path accepts >= d drafts), with
    P_n(d) = 1 - prod_{c child of n} (1 - p' P_c(d-1)), P_n(0) = 1 and
    p' = p + (1-p)/V (a random id matches by chance)."""
    T = len(parent)
    pp = p + (1 - p) / V
    kids = [[] for _ in range(T)]
    for n in range(1, T):
        kids[parent[n]].append(n)
    dmax = T
    f = np.ones((T, dmax + 1))
    for d in range(1, dmax + 1):
        for n in range(T):
            f[n, d] = 1 - np.prod([1 - pp * f[c, d - 1] for c in kids[n]]) if kids[n] else 0.0
    return 1 + f[0, 1:].sum()


def test_expected_tau_closed_form_chain():
    # a chain of gamma drafts: E[tau] = sum_{i=0}^{gamma} p^i (V -> infinity)
    for gamma in (1, 4, 7):
        got = closed_form_tau(synth.chain_tree(gamma), 0.88, 10**12)
        assert abs(got - sum(0.88 ** i for i in range(gamma + 1))) < 1e-9
    assert abs(closed_form_tau(synth.binary_tree_15(), 0.88, 4096) - 4.476) < 5e-4


@pytest.mark.parametrize("tree,p,V", [("binary", 0.88, 4096), ("topk", 0.88, 128256), ("topk", 0.6, 128256)])
def test_mean_tau_matches_closed_form(orc, tree, p, V):
    rng = np.random.default_rng(11)
    parent = synth.binary_tree_15() if tree == "binary" else synth.topk_tree(rng, 60, 7, 10)
    T = len(parent)
    B = 20000
    idx = rng.integers(0, V, size=(B, T)).astype(np.int32)
    u = rng.random((B, T))
    rid = rng.integers(0, V, size=(B, T)).astype(np.int32)
    tok = synth.plant_tokens(np.tile(parent, (B, 1)), idx, np.full(B, p), u, rid)
    alen, _, _, _ = orc.accept(tok, np.tile(parent, (B, 1)), idx)
    tau = alen + 1.0
    want = closed_form_tau(parent, p, V)
    se = tau.std() / np.sqrt(B)
    assert abs(tau.mean() - want) < 4 * se, (tau.mean(), want, se)


def closed_form_tau_ranked(parent, p, V):
    """E[tau] with siblings as alternatives (synth.plant_tokens_ranked): rank
    j of a node's children carries the target's token with probability
    q_j = p (1 - p)^(j - 1), exclusively; any other child matches by chance
    with probability 1/V. With P_n(d) = P(a path from n accepts >= d drafts):
    P_n(d) = sum_j q_j P_cj(d-1) + r_n(d), where r_n(d) (no ranked match) is
    (1 - sum_j q_j) times the chance-match term of the independent formula,
    and the chance term is dropped to first order when V is large."""
    T = len(parent)
    kids = [[] for _ in range(T)]
    for n in range(1, T):
        kids[parent[n]].append(n)
    f = np.ones((T, T + 1))
    for d in range(1, T + 1):
        for n in range(T):
            if not kids[n]:
                f[n, d] = 0.0
                continue
            q = [p * (1 - p) ** j for j in range(len(kids[n]))]
            ranked = sum(qj * f[c, d - 1] for qj, c in zip(q, kids[n]))
            none = 1 - sum(q)
            chance = 1 - np.prod([1 - f[c, d - 1] / V for c in kids[n]])
            f[n, d] = ranked + none * chance
    return 1 + f[0, 1:].sum()


def test_ranked_planting_is_the_independent_one_on_a_chain():
    rng = np.random.default_rng(5)
    parent = np.tile(synth.chain_tree(40), (3, 1))
    idx = rng.integers(0, 1000, size=parent.shape).astype(np.int32)
    u = rng.random(parent.shape)
    rid = rng.integers(0, 1000, size=parent.shape).astype(np.int32)
    p = np.array([0.6, 0.8, 0.95])
    assert np.array_equal(synth.plant_tokens_ranked(parent, idx, p, u, rid), synth.plant_tokens(parent, idx, p, u, rid))


def test_ranked_planting_plants_at_most_one_sibling():
    rng = np.random.default_rng(6)
    parent = np.stack([synth.topk_tree(rng, 60, 7, 10) for _ in range(50)])
    V = 10 ** 6
    idx = rng.integers(0, V, size=parent.shape).astype(np.int32)
    u = rng.random(parent.shape)
    rid = rng.integers(0, V, size=parent.shape).astype(np.int32)
    tok = synth.plant_tokens_ranked(parent, idx, np.full(50, 0.9), u, rid)
    for b in range(50):
        for n in range(len(parent[b])):
            kids = np.nonzero(parent[b] == n)[0]
            hits = [c for c in kids if tok[b, c] == idx[b, n] and tok[b, c] != rid[b, c]]
            assert len(hits) <= 1
            if hits:  # the planted child is the first one whose uniform passes
                first = next(c for c in kids if u[b, c] < 0.9)
                assert hits[0] == first


@pytest.mark.parametrize("kind,p", [("chain", 0.7), ("topk", 0.7), ("topk", 0.9), ("ranked", 0.7), ("ranked", 0.9)])
def test_mean_tau_ranked_matches_closed_form(orc, kind, p):
    rng = np.random.default_rng(12)
    parent = {"chain": lambda: synth.chain_tree(40), "topk": lambda: synth.topk_tree(rng, 40, 7, 10),
              "ranked": lambda: synth.ranked_tree(p, 40, 8, 10)}[kind]()
    T, B, V = len(parent), 20000, 128256
    idx = rng.integers(0, V, size=(B, T)).astype(np.int32)
    u = rng.random((B, T))
    rid = rng.integers(0, V, size=(B, T)).astype(np.int32)
    tok = synth.plant_tokens_ranked(np.tile(parent, (B, 1)), idx, np.full(B, p), u, rid)
    alen, _, _, _ = orc.accept(tok, np.tile(parent, (B, 1)), idx)
    tau = alen + 1.0
    want = closed_form_tau_ranked(parent, p, V)
    se = tau.std() / np.sqrt(B)
    assert abs(tau.mean() - want) < 4 * se, (tau.mean(), want, se)
    if kind == "chain":
        assert abs(want - closed_form_tau(parent, p, V)) < 1e-9


def _rank_paths(parent):
    """Each node's path as the tuple of its ranks (1-based position among its
    siblings in index order), root = ()."""
    out = [()]
    for n in range(1, len(parent)):
        sib = [c for c in range(1, len(parent)) if parent[c] == parent[n]]
        out.append(out[parent[n]] + (sib.index(n) + 1,))
    return out


@pytest.mark.parametrize("p,N", [(0.7, 12), (0.55, 20), (0.9, 9)])
def test_ranked_tree_is_the_top_n_by_path_probability(p, N):
    depth, branch = 3, 3
    parent = synth.ranked_tree(p, N, depth, branch)
    assert len(parent) == N + 1 and parent[0] == -1 and all(0 <= parent[n] < n for n in range(1, N + 1))
    paths = _rank_paths(parent)
    assert len(set(paths)) == N + 1 and all(len(t) <= depth and max(t, default=1) <= branch for t in paths)
    prob = lambda t: float(np.prod([p * (1 - p) ** (j - 1) for j in t]))  # noqa: E731
    every = [t for d in range(1, depth + 1) for t in itertools.product(range(1, branch + 1), repeat=d)]
    best = sorted((prob(t) for t in every), reverse=True)[:N]
    got = sorted((prob(t) for t in paths[1:]), reverse=True)
    assert np.allclose(got, best, rtol=0, atol=1e-15)
    # closed under parents and siblings of lower rank (both at least as likely)
    have = set(paths)
    for t in paths[1:]:
        assert t[:-1] in have and (t[-1] == 1 or t[:-1] + (t[-1] - 1,) in have)


@pytest.mark.parametrize("p", [0.6, 0.8, 0.95])
def test_ranked_tree_beats_a_chain_of_the_same_size(p):
    """Without a depth limit the chain is one of the candidate trees, so the
    best-first tree's expected acceptance is at least the chain's; with the
    8-step limit it still beats a chain of 8."""
    V = 128256
    for N in (20, 40):
        free = closed_form_tau_ranked(synth.ranked_tree(p, N, N, 10), p, V)
        assert free >= closed_form_tau_ranked(synth.chain_tree(N), p, V) - 1e-12
    assert closed_form_tau_ranked(synth.ranked_tree(p, 40, 8, 10), p, V) > \
        closed_form_tau_ranked(synth.chain_tree(8), p, V)
