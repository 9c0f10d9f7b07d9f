"""Pins for the oracle's EAGLE-3 draft head and tree growth (CPU only).

* The fusion FCs are plain matrix products over the concatenation (numpy fp64
  matmul on an explicit concatenation); W_in . [a; e] = W_a . a + W_e . e.
* Step-mode pairing and positions ([news] draft stage, steps 2-3): the input
  row of every frontier node is rebuilt by hand from the explicit
  concatenation [output of its tree parent; embedding of its own token], with
  the parent found through the candidate pool's own parent links, and its
  key row by a hand-written RMSNorm, projection and complex-rotation RoPE at
  position context + depth - 1.
* Tree selection: the rerank equals a brute-force full sort of the pool
  (numpy lexsort); closure under parents; a peaked draft degenerates to a chain
  of full depth; the drafted tree has n_drafts nodes, parents before children,
  at most top-k children per node and depth at most the number of steps.
* Replay of recorded choices (tests/draft_replay.py, used to check another
  run's choices): replaying its own choices reproduces its own tree with zero
  margins; swapping one taken child for the next one down costs exactly that
  logit gap.
* Trimmed draft vocabulary (VocabTrim / FR-Spec reading): the root's children
  equal a brute-force top-k of fp64 logits (numpy matmul of a hand-written
  RMSNorm) with every dropped id set to -inf, their logp is taken against the
  log-sum-exp of the kept ids alone, every drafted token is a kept id, and
  keeping every id reproduces the untrimmed draft exactly.
"""
import dataclasses

import numpy as np
import pytest

import synth
from tests.draft_replay import replay


def f64(a):
    return (synth.bf16_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def test_draft_fuse_is_a_matmul_on_the_concatenation(orc):
    rng = np.random.default_rng(0)
    M, k, V = 9, 64, 50
    l, m, h, a = (synth.normal_bf16(rng, (M, k)) for _ in range(4))
    E = synth.normal_bf16(rng, (V, k), 0.1)
    Wf, Wi = synth.normal_bf16(rng, (k, 3 * k), 0.1), synth.normal_bf16(rng, (k, 2 * k), 0.1)
    tok = rng.integers(0, V, size=M).astype(np.int32)
    x, g = orc.draft_fuse(tok, E, Wf, Wi, l=l, m=m, h=h, want_g=True)
    gref = np.concatenate([f64(l), f64(m), f64(h)], 1) @ f64(Wf).T
    np.testing.assert_allclose(f64(g), gref, rtol=2 ** -8, atol=1e-30)
    xref = np.concatenate([f64(g), f64(E)[tok]], 1) @ f64(Wi).T
    np.testing.assert_allclose(f64(x), xref, rtol=2 ** -8, atol=1e-30)
    xs = orc.draft_fuse(tok, E, Wf, Wi, a_prev=a)
    split = f64(a) @ f64(Wi)[:, :k].T + f64(E)[tok] @ f64(Wi)[:, k:].T      # W_in [a; e] = W_a a + W_e e
    np.testing.assert_allclose(f64(xs), split, rtol=2 ** -8, atol=1e-30)


def test_rerank_equals_full_sort_and_is_closed(orc):
    rng = np.random.default_rng(1)
    B, C, steps, N = 20, 10, 8, 60
    pool_s, pool_t, pool_p = [], [], []
    fr_score = np.zeros((B, 1), np.float32)
    fr_pool = np.full((B, 1), -1, np.int32)
    n = 0
    for step in range(1, steps + 1):
        F = fr_score.shape[1]
        logp = -np.abs(rng.standard_normal((B, F, C))).astype(np.float32) * 3
        ids = rng.integers(0, 1000, size=(B, F, C)).astype(np.int32)
        cand, cpar, npool, nscore, ntok, nslot = orc.tree_expand(fr_score, fr_pool, ids, logp, n, C)
        pool_s.append(cand); pool_t.append(ids.reshape(B, -1)); pool_p.append(cpar)
        n += F * C
        fr_score, fr_pool = nscore, npool
    S, Tk, Pp = (np.concatenate(x, 1) for x in (pool_s, pool_t, pool_p))
    parent, tokens, near = orc.tree_rerank(S, Tk, Pp, np.arange(B), N)
    for b in range(B):
        brute = np.lexsort((np.arange(S.shape[1]), -S[b].astype(np.float64)))[:N]   # score desc, creation asc
        chosen = np.sort(brute)
        assert list(tokens[b, 1:]) == list(Tk[b, chosen])
        assert orc.tree_check(parent[b])                                  # parents before children
        sel = set(chosen.tolist())
        assert all(Pp[b, c] < 0 or int(Pp[b, c]) in sel for c in chosen)  # closed under parents
        kids = np.bincount(parent[b, 1:], minlength=N + 1)
        assert kids.max() <= C
        _, depth = orc.tree_mask(parent[b])
        assert depth.max() <= steps


def test_peaked_draft_is_a_full_depth_chain(orc):
    """One child per node carries logp 0 and the rest -50: the selected tree
    contains the full-depth chain of those children."""
    B, C, steps, N = 1, 10, 8, 60
    fr_score = np.zeros((B, 1), np.float32); fr_pool = np.full((B, 1), -1, np.int32)
    pool = []
    n = 0
    for step in range(steps):
        F = fr_score.shape[1]
        logp = np.full((B, F, C), -50.0, np.float32)
        logp[:, :, 3] = 0.0
        ids = (np.arange(F * C).reshape(1, F, C) + 1000 * step).astype(np.int32)
        cand, cpar, npool, nscore, ntok, _ = orc.tree_expand(fr_score, fr_pool, ids, logp, n, C)
        pool.append((cand, ids.reshape(B, -1), cpar))
        n += F * C
        fr_score, fr_pool = nscore, npool
    S, Tk, Pp = (np.concatenate([p[i] for p in pool], 1) for i in range(3))
    parent, tokens, _ = orc.tree_rerank(S, Tk, Pp, [7], N)
    _, depth = orc.tree_mask(parent[0])
    assert depth.max() == steps
    zero = np.flatnonzero(S[0] == 0.0)
    assert len(zero) == steps and set(Tk[0, zero]).issubset(set(tokens[0]))


def test_draft_tree_invariants(orc):
    s = synth.DRAFT_SMALL
    W = synth.draft_weights(s)
    l, m, h, tok = synth.draft_inputs(s, 0)
    r = orc.draft_tree(s, W, l, m, h, tok)
    N = s.n_drafts
    for b in range(s.B):
        par, tk = r["parent"][b], r["tokens"][b]
        assert orc.tree_check(par) and len(par) == N + 1 and tk[0] == tok[b, -1]
        _, depth = orc.tree_mask(par)
        assert 1 <= depth.max() <= s.steps
        for n in range(N + 1):                   # siblings carry distinct tokens (distinct top-k ids)
            kids = np.flatnonzero(par == n)
            assert len(set(tk[kids])) == len(kids) and len(kids) <= s.topk
    # scores never grow along a path (the premise of the near-tie flag rule)
    ps, pp = r["pool_score"], r["pool_parent"]
    for b in range(s.B):
        has = pp[b] >= 0
        assert (ps[b][has] <= ps[b][pp[b][has]]).all()
    # row-independence: one sequence alone gives the same tree
    l1, m1, h1, t1 = synth.draft_inputs(s, 0, batch=slice(3, 4))
    r1 = orc.draft_tree(s, W, l1, m1, h1, t1)
    assert np.array_equal(r1["parent"][0], r["parent"][3]) and np.array_equal(r1["tokens"][0], r["tokens"][3])


def _bf16(x):
    return synth.f32_to_bf16(np.asarray(x, np.float64).astype(np.float32))


def _hand_rope(x, pos, theta):
    """Rotate-half RoPE written as a complex rotation of the pairs
    (j, j + D/2) by pos * theta^(-2j/D), in fp64."""
    D = x.shape[-1]
    j = np.arange(D // 2)
    ang = pos * theta ** (-2.0 * j / D)
    z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], -1)


@pytest.mark.parametrize("seed", [0, 1])
def test_draft_step_rows_pair_parent_output_with_own_token(orc, seed):
    """Every frontier node's input row is W_in [a_parent; E[token]] with the
    parent taken from the pool's parent links (step 2: the root, whose output
    is a_root), and its key row sits at position ctx + depth - 1 (depth =
    step - 1). Two sequences, three growth steps, rebuilt by hand."""
    s = dataclasses.replace(synth.DRAFT_SMALL, B=2, steps=3, n_drafts=30)
    W = synth.draft_weights(s)
    l, m, h, tok = synth.draft_inputs(s, seed)
    l, m, h, tok = l[:2], m[:2], h[:2], tok[:2]
    r = orc.draft_tree(s, W, l, m, h, tok)
    C, k, qd, kvd = s.topk, s.k, s.Hq * s.D, s.Hkv * s.D
    E, Wi = f64(W["embed"]), f64(W["w_in"])
    Wk = f64(W["wqkv"])[qd:qd + kvd]
    starts = [0] + [C + (st - 2) * C * C for st in range(2, s.steps + 1)]     # pool offset of each step
    # frontier pool indices per step, from the recorded choices
    fr_pool = [starts[st - 1] + np.asarray(r["choices"]["frontier"][st - 1]) for st in range(1, s.steps)]
    assert len(r["rows"]) == s.steps - 1
    n_checked = 0
    for rr in r["rows"]:
        st = rr["step"]
        assert (rr["pos"] == s.ctx + (st - 1) - 1).all()            # depth st - 1 -> ctx + depth - 1
        for b in range(s.B):
            for i in range(C):
                node = fr_pool[st - 2][b, i]                         # this frontier node's pool index
                assert rr["tokens"][b, i] == r["pool_token"][b, node]
                par = r["pool_parent"][b, node]
                if st == 2:
                    assert par == -1
                    a_par = f64(r["a_root"][b])
                else:
                    slot = np.flatnonzero(fr_pool[st - 3][b] == par)
                    assert len(slot) == 1                            # the parent is in the previous frontier
                    a_par = f64(r["a_steps"][st - 3][b * C + slot[0]])
                x_hand = np.concatenate([a_par, E[r["pool_token"][b, node]]]) @ Wi.T
                got = f64(rr["x"][b, i])
                ulp = 2.0 ** -7 * np.abs(x_hand)
                assert np.all(np.abs(got - x_hand) <= ulp + 1e-30), (st, b, i)
                # key row: RMSNorm -> K projection -> RoPE at ctx + depth - 1
                xr = f64(rr["x"][b, i])
                hn = f64(_bf16(xr / np.sqrt(np.mean(xr * xr) + s.eps)))
                kl = f64(_bf16(hn @ Wk.T)).reshape(s.Hkv, s.D)
                k_hand = _hand_rope(kl, s.ctx + st - 2, s.theta)
                kg = f64(r["tree_k"][b, (st - 2) * C + i])
                assert np.all(np.abs(kg - k_hand) <= 2.0 ** -7 * np.abs(k_hand) + 1e-6), (st, b, i)
                n_checked += 1
    assert n_checked == (s.steps - 1) * s.B * C


def test_replay_margins(orc):
    s = synth.DRAFT_SMALL
    W = synth.draft_weights(s)
    l, m, h, tok = synth.draft_inputs(s, 1)
    r = orc.draft_tree(s, W, l, m, h, tok)
    f = replay(orc, s, W, l, m, h, tok, r["choices"])
    assert np.array_equal(f["parent"], r["parent"]) and np.array_equal(f["tokens"], r["tokens"])
    assert np.array_equal(f["pool_score"], r["pool_score"])
    assert all((v == 0).all() for v in f["margin"].values())
    # swap, at the last step, the 10th child of sequence 0's first frontier node for the 11th
    idx, val, _, _ = orc.lmhead(orc.rmsnorm(r["a_steps"][-1][:1], eps=s.eps), W["lm_head"], topk=s.topk + 1)
    ids = [a.copy() for a in r["choices"]["ids"]]
    ids[-1][0, 0, s.topk - 1] = idx[0, s.topk]
    g = replay(orc, s, W, l, m, h, tok, dict(r["choices"], ids=ids))
    assert g["margin"]["lm"][0] == val[0, s.topk - 1] - val[0, s.topk] > 0
    assert (g["margin"]["lm"][1:] == 0).all()
    # a final selection that drops the best entry for a worse one
    sel = r["choices"]["selected"].copy()
    ps = r["pool_score"][2]
    best = int(np.argmax(ps))
    out = int(np.flatnonzero(~np.isin(np.arange(len(ps)), sel[2]))[0])
    sel[2][sel[2] == best] = out
    sel[2].sort()
    h2 = replay(orc, s, W, l, m, h, tok, dict(r["choices"], selected=sel))
    assert h2["margin"]["final"][2] >= ps[best] - ps[out] > 0 and h2["margin"]["final"][0] == 0


def test_bf16_draft_logits_move_with_last_bit_noise(orc):
    """With bf16 storage at every layer boundary, flipping the last bit of 1%
    of one input tensor moves the oracle's own draft logits along fixed
    choices by several 1e-2: other correct bf16 arithmetic lands anywhere in
    that band, so GPU draft trees are compared by replaying their choices, not
    bit for bit. Last-bit noise in fp32 storage moves them by less than 1e-4."""
    s = synth.DRAFT_SMALL
    W = synth.draft_weights(s)
    l, m, h, tok = synth.draft_inputs(s, 0)
    r = orc.draft_tree(s, W, l, m, h, tok)
    noisy = l.copy()
    noisy[np.random.default_rng(5).random(l.shape) < 0.01] ^= np.uint16(1)
    f = replay(orc, s, W, noisy, m, h, tok, r["choices"])
    moved = max(np.abs(a - b).max() for a, b in zip(f["lm_val"], replay(orc, s, W, l, m, h, tok,
                                                                         r["choices"])["lm_val"]))
    assert moved > 0.03
    cv = lambda a: synth.bf16_to_f32(a)  # noqa: E731
    W32 = {k: cv(v) for k, v in W.items()}
    r32 = orc.draft_tree(s, W32, cv(l), cv(m), cv(h), tok)
    n32 = cv(l).copy()
    n32.view(np.uint32)[np.random.default_rng(5).random(l.shape) < 0.01] ^= np.uint32(1)
    f32 = replay(orc, s, W32, n32, cv(m), cv(h), tok, r32["choices"])
    g32 = replay(orc, s, W32, cv(l), cv(m), cv(h), tok, r32["choices"])
    assert max(np.abs(a - b).max() for a, b in zip(f32["lm_val"], g32["lm_val"])) < 1e-4


def test_trimmed_vocab_root_children_are_the_restricted_top_k(orc):
    s = synth.DRAFT_SMALL_TRIM
    vocab = synth.draft_vocab(s)
    assert len(vocab) == s.vocab_keep and (np.diff(vocab) > 0).all()
    W = synth.draft_weights(s)
    l, m, h, tok = synth.draft_inputs(s, 0)
    r = orc.draft_tree(s, W, l, m, h, tok, vocab=vocab)
    C = s.topk
    a = f64(r["a_root"])
    hn = f64(_bf16(a / np.sqrt(np.mean(a * a, axis=1, keepdims=True) + s.eps)))
    logits = hn @ f64(W["lm_head"]).T                                    # [B, V] fp64
    dropped = np.ones(s.V, bool)
    dropped[vocab] = False
    masked = np.where(dropped[None, :], -np.inf, logits)
    ids1 = np.asarray(r["choices"]["ids"][0]).reshape(s.B, C)
    for b in range(s.B):
        order = np.lexsort((np.arange(s.V), -masked[b]))[:C]
        assert np.array_equal(ids1[b], order), b
        kept = logits[b, vocab]
        lse = kept.max() + np.log(np.exp(kept - kept.max()).sum())
        want = (logits[b, order] - lse).astype(np.float32)
        # step-1 pool entries are the root's children, score = logp
        assert np.allclose(r["pool_score"][b, :C], want, rtol=0, atol=1e-5)
        # the full-vocabulary lse is larger: dropping rows raises every logp
        full = logits[b].max() + np.log(np.exp(logits[b] - logits[b].max()).sum())
        assert full > lse
    # every drafted token is a kept id (the root is the context's own token)
    assert np.isin(r["tokens"][:, 1:], vocab).all()
    assert np.isin(r["pool_token"], vocab).all()


def test_trimmed_vocab_keeping_every_id_is_the_full_draft(orc):
    s = dataclasses.replace(synth.DRAFT_SMALL, B=2, steps=4, n_drafts=30)
    W = synth.draft_weights(s)
    l, m, h, tok = (a[:2] for a in synth.draft_inputs(s, 1))
    r = orc.draft_tree(s, W, l, m, h, tok)
    t = orc.draft_tree(s, W, l, m, h, tok, vocab=np.arange(s.V, dtype=np.int32))
    for key in ("parent", "tokens", "pool_score", "pool_token", "pool_parent"):
        assert np.array_equal(r[key], t[key]), key
    with pytest.raises(ValueError):
        orc.draft_tree(s, W, l, m, h, tok, vocab=np.array([5, 3] + list(range(10, 30)), np.int32))


def test_trimmed_vocab_replay_of_own_choices(orc):
    s = dataclasses.replace(synth.DRAFT_SMALL_TRIM, B=2, steps=4, n_drafts=30)
    vocab = synth.draft_vocab(s)
    W = synth.draft_weights(s)
    l, m, h, tok = (a[:2] for a in synth.draft_inputs(s, 2))
    r = orc.draft_tree(s, W, l, m, h, tok, vocab=vocab)
    f = replay(orc, s, W, l, m, h, tok, r["choices"], vocab=vocab)
    assert np.array_equal(f["parent"], r["parent"]) and np.array_equal(f["tokens"], r["tokens"])
    assert all((v == 0).all() for v in f["margin"].values())


def test_draft_context_in_pieces_equals_the_whole_ingest(orc):
    """The draft's context rows taken in two pieces (the second on top of the
    first's cached rows) give the whole ingest's K/V rows and output: the
    piecewise form the decoding loop uses after each acceptance."""
    s = dataclasses.replace(synth.DRAFT_SMALL, B=2, ctx=40)
    cv = lambda a: synth.bf16_to_f32(a) if a.dtype == np.uint16 else a  # noqa: E731
    W = {k: cv(v) for k, v in synth.draft_weights(s).items()}
    l, m, h, tok = (cv(a)[:2, :40] if a.dtype == np.uint16 else a[:2, :40] for a in synth.draft_inputs(s, 3))
    r = orc.draft_tree(s, W, l, m, h, tok)
    B = 2
    k1, v1, _ = orc.draft_context(s, W, l[:, :23], m[:, :23], h[:, :23], tok[:, :23], np.zeros(B, np.int32))
    k2, v2, a = orc.draft_context(s, W, l[:, 23:], m[:, 23:], h[:, 23:], tok[:, 23:], np.full(B, 23, np.int32),
                                  prev_k=k1, prev_v=v1)
    kk, vv = np.concatenate([k1, k2], 1), np.concatenate([v1, v2], 1)
    assert np.abs(kk - r["k_ctx"]).max() <= 1e-6 * np.abs(r["k_ctx"]).max()
    assert np.abs(vv - r["v_ctx"]).max() <= 1e-6 * np.abs(r["v_ctx"]).max()
    assert np.abs(a - r["a_root"]).max() <= 1e-5 * np.abs(r["a_root"]).max()
    # an earlier row as `last`: only the rows up to it are visible to it
    _, _, a_mid = orc.draft_context(s, W, l[:, 23:], m[:, 23:], h[:, 23:], tok[:, 23:], np.full(B, 23, np.int32),
                                    prev_k=k1, prev_v=v1, last=np.array([5, 9]))
    for b, j in ((0, 5), (1, 9)):
        n = 23 + j + 1
        _, _, a_ref = orc.draft_context(s, W, l[b:b + 1, :n], m[b:b + 1, :n], h[b:b + 1, :n], tok[b:b + 1, :n],
                                        np.zeros(1, np.int32))
        assert np.abs(a_mid[b] - a_ref[0]).max() <= 1e-5 * np.abs(a_ref).max()
