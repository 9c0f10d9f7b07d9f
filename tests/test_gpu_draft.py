"""GPU parity of the EAGLE-3 draft head and the tree growth kernels against the
oracle (news write-up of the EAGLE-3 paper, draft stage; Spec-Bench blog post,
section 4.2 for top-k 10 / 60 drafts).

* tree_expand / tree_rerank kernels: bit-exact on the same fp32 inputs
  (including exact score ties, which rank by creation index).
* fp32 draft head at a small shape: the drafted tree identical to the
  oracle's (as the set of root-to-node token paths) for every sequence
  without a near-tie (1e-3) that can reach the final tree.
* bf16 draft head (small shape, 3 seeds; full size, sequence 0): bf16
  storage at every layer boundary moves the logits by up to ~1e-2, while
  random weights leave neighbouring top logits only a few 1e-2 apart, so
  several trees are correct. The GPU's choices are replayed through the
  oracle's arithmetic (tests/draft_replay.py): context K/V, hidden states,
  logits and pool scores along them meet the bf16 tolerance (normwise 2e-2);
  no choice falls below the best alternative in the oracle's numbers by more
  than twice that tolerance (2 x 2e-2 x the largest |logit| or |score|: a
  selection that is best for some values within the tolerance of the
  oracle's); the tree equals the renumbered selection exactly.
* Trimmed draft vocabulary (half of the rows kept; small shape and full
  size): the vocab_map kernel exactly (ids out of range give -1 and the
  range status), and the trimmed draft head by the same replay, through the
  oracle's trimmed head; every drafted token a kept id.
"""
import numpy as np
import pytest
import torch

import synth
from tests._gpu import dev, host, normwise_rel
from tests.draft_replay import replay

pytestmark = pytest.mark.gpu


def _expand_case(rng, B, F, C, NF, pool_len, tie=False):
    fr_score = (-np.abs(rng.standard_normal((B, F))) * 2).astype(np.float32)
    val = (rng.standard_normal((B, F, C)) * 3).astype(np.float32)
    lse = (np.abs(rng.standard_normal((B, F))) * 2 + 5).astype(np.float32)
    if tie:
        val[:, :, 1] = val[:, :, 0]                       # equal siblings: creation order decides
        fr_score[:, 1:] = fr_score[:, :1]
        val[:, 1:] = val[:, :1]
    ids = rng.integers(0, 5000, size=(B, F, C)).astype(np.int32)
    fr_pool = rng.integers(0, max(pool_len, 1), size=(B, F)).astype(np.int32)
    return fr_score, fr_pool, ids, val, lse


@pytest.mark.parametrize("tie", [False, True])
def test_tree_expand_matches_oracle(orc, tie):
    import tree_draft_verification_amd as e3
    rng = np.random.default_rng(11 + tie)
    B, F, C, NF, pool_len, cap = 5, 10, 10, 10, 110, 400
    fr_score, fr_pool, ids, val, lse = _expand_case(rng, B, F, C, NF, pool_len, tie)
    # the oracle's logp: fp32(value - lse), the same subtraction the kernel makes
    logp = (val - lse[:, :, None]).astype(np.float32)
    cand, cpar, npool, nscore, ntok, nslot = orc.tree_expand(fr_score, fr_pool, ids, logp, pool_len, NF)
    fr_mask = rng.integers(0, 2 ** 62, size=(B, F, 2)).astype(np.uint64)
    row_base = 20
    d = {n: dev(a) for n, a in dict(fr_score=fr_score, fr_pool=fr_pool, fr_mask=fr_mask, ids=ids, val=val,
                                      lse=lse).items()}
    ps = torch.full((B, cap), -7.0, device="cuda")
    pt = torch.full((B, cap), -7, dtype=torch.int32, device="cuda")
    pp = torch.full((B, cap), -7, dtype=torch.int32, device="cuda")
    o = {n: torch.empty(B, NF, dtype=t, device="cuda") for n, t in
         dict(pool=torch.int32, score=torch.float32, token=torch.int32, arow=torch.int32).items()}
    o["mask"] = torch.empty(B, NF, 2, dtype=torch.int64, device="cuda")
    e3.eagle3_tree_expand(d["fr_score"], d["fr_pool"], d["fr_mask"], 3, 17, d["ids"], d["val"], d["lse"], pool_len,
                          row_base, ps, pt, pp, o["pool"], o["score"], o["token"], o["mask"], o["arow"])
    torch.cuda.synchronize()
    sl = slice(pool_len, pool_len + F * C)
    assert np.array_equal(host(ps)[:, sl].view(np.uint32), cand.view(np.uint32))
    assert np.array_equal(host(pt)[:, sl], ids.reshape(B, -1))
    assert np.array_equal(host(pp)[:, sl], cpar)
    assert (host(ps)[:, :pool_len] == -7.0).all() and (host(ps)[:, sl.stop:] == -7.0).all()   # nothing else written
    assert np.array_equal(host(o["pool"]), npool)
    assert np.array_equal(host(o["score"]).view(np.uint32), nscore.view(np.uint32))
    assert np.array_equal(host(o["token"]), ntok)
    assert np.array_equal(host(o["arow"]), np.arange(B)[:, None] * 17 + 3 + nslot)
    want = fr_mask[np.arange(B)[:, None], nslot].copy()
    for b in range(B):
        for r in range(NF):
            bit = row_base + r
            want[b, r, bit // 64] |= np.uint64(1) << np.uint64(bit % 64)
    assert np.array_equal(host(o["mask"]).view(np.uint64), want)


@pytest.mark.parametrize("P,N,tie", [(710, 60, False), (710, 60, True), (61, 60, False), (5, 5, False)])
def test_tree_rerank_matches_oracle(orc, P, N, tie):
    import tree_draft_verification_amd as e3
    rng = np.random.default_rng(P + N + tie)
    B, cap = 7, P + 3
    score = (-np.abs(rng.standard_normal((B, P))) * 4).astype(np.float32)
    if tie:
        score[:, 50:120] = score[:, 10:11]                  # a block of equal scores across the boundary
    # parents: an earlier entry with a score not below the child's (closure), or -1
    parent = np.full((B, P), -1, np.int32)
    for b in range(B):
        for i in range(10, P):
            cands = np.flatnonzero(score[b, :i] >= score[b, i])
            if len(cands):
                parent[b, i] = rng.choice(cands)
    token = rng.integers(0, 9999, size=(B, P)).astype(np.int32)
    root = rng.integers(0, 9999, size=B).astype(np.int32)
    ref_par, ref_tok, _ = orc.tree_rerank(score, token, parent, root, N)
    pad = lambda a, v: np.concatenate([a, np.full((B, cap - P), v, a.dtype)], 1)  # noqa: E731
    ds, dt, dp, dr = dev(pad(score, 0.0)), dev(pad(token, 0)), dev(pad(parent, -1)), dev(root)
    par = torch.full((B, N + 1), -9, dtype=torch.int32, device="cuda")
    tok = torch.full((B, N + 1), -9, dtype=torch.int32, device="cuda")
    e3.eagle3_tree_rerank(ds, dt, dp, P, dr, par, tok)
    torch.cuda.synchronize()
    assert np.array_equal(host(par), ref_par)
    assert np.array_equal(host(tok), ref_tok)


def _paths(parent, tokens):
    out = set()
    for n in range(len(parent)):
        p, seq = n, []
        while p > 0:
            seq.append(int(tokens[p]))
            p = int(parent[p])
        out.add(tuple(reversed(seq)))
    return out


def _valid(parent):
    return parent[0] == -1 and all(0 <= parent[n] < n for n in range(1, len(parent)))


def _f32(W, *arrays):
    cv = lambda a: synth.bf16_to_f32(a) if a.dtype == np.uint16 else a  # noqa: E731
    return {k: cv(v) for k, v in W.items()}, [cv(a) for a in arrays]


def _gpu_draft(shape, W, l, m, h, tok, vocab=None):
    import tree_draft_verification_amd as e3
    wd = {k: dev(v) for k, v in W.items()}
    head = e3.DraftHead(wd, l.shape[0], shape.ctx, shape.Hq, shape.Hkv, shape.D, shape.steps, shape.topk,
                        shape.n_drafts, shape.theta, shape.eps, vocab=None if vocab is None else dev(vocab))
    dl, dm, dh, dt = dev(l), dev(m), dev(h), dev(tok)
    record = []
    head.run(dl, dm, dh, dt, record=record)
    torch.cuda.synchronize()
    rec = [{k: (host(v) if isinstance(v, torch.Tensor) else v) for k, v in r.items()} for r in record]
    return head, rec


def _check_choices(orc, s, W, l, m, h, tok, head, rec, seqs, tol=2e-2, vocab=None):
    """The GPU's choices, replayed through the oracle's arithmetic: every
    number the GPU produced along them within `tol` (normwise), and no choice
    worse than the best alternative in the oracle's numbers by more than
    2 x tol x the largest |logit| (children) or |pool score| (frontiers, the
    final tree). The tree structure must then equal the renumbering of the
    GPU's selection exactly."""
    seqs = np.asarray(seqs)
    C, N = s.topk, s.n_drafts
    P = s.pool_len
    gscore = host(head.pool_score)[seqs, :P]
    selected = np.stack([np.lexsort((np.arange(P), -gscore[i].astype(np.float64)))[:N] for i in range(len(seqs))])
    follow = dict(ids=[r["ids"][seqs] for r in rec],
                  frontier=[r["next_pool"][seqs] - (r["pool_len"] if i else 0) for i, r in enumerate(rec)],
                  selected=selected)
    f = replay(orc, s, W, l, m, h, tok, follow, vocab=vocab)
    assert np.array_equal(host(head.parent)[seqs], f["parent"]), "tree structure differs"
    assert np.array_equal(host(head.tokens)[seqs], f["tokens"])
    assert normwise_rel(host(head.a_root)[seqs], f["a_root"])[0] <= tol
    d_logit, max_logit = 0.0, 0.0
    for i, r in enumerate(rec):
        ref = f["lm_val"][i]
        assert np.isfinite(ref).all(), f"step {i + 1}: a taken child is not among the oracle's top 16"
        rel, err = normwise_rel(r["val"][seqs], ref)
        assert rel <= tol, f"step {i + 1}: logits off by {rel}"
        d_logit = max(d_logit, err)
        max_logit = max(max_logit, float(np.abs(ref).max()))
        if i:
            assert normwise_rel(r["a"].reshape(-1, C, s.k)[seqs], f["a_steps"][i - 1].reshape(-1, C, s.k))[0] <= tol
    rel_s, d_score = normwise_rel(gscore, f["pool_score"])
    assert rel_s <= tol, f"pool scores off by {rel_s}"
    max_score = float(np.abs(f["pool_score"]).max())
    mg = f["margin"]
    assert (mg["lm"] <= 2 * tol * max_logit).all(), (mg["lm"], max_logit)
    assert (mg["frontier"] <= 2 * tol * max_score).all(), (mg["frontier"], max_score)
    assert (mg["final"] <= 2 * tol * max_score).all(), (mg["final"], max_score)
    return dict(d_logit=d_logit, d_score=d_score, max_margin={k: float(v.max()) for k, v in mg.items()},
                n_off=int(sum((v > 0).sum() for v in mg.values())))


def test_draft_head_small_f32_matches_oracle(orc):
    """fp32 storage keeps both sides within ~1e-6, so every selection away
    from a 1e-3 near-tie must agree exactly."""
    s = synth.DRAFT_SMALL
    W, (l, m, h) = _f32(synth.draft_weights(s), *synth.draft_inputs(s, 0)[:3])
    tok = synth.draft_inputs(s, 0)[3]
    ref = orc.draft_tree(s, W, l, m, h, tok)
    head, rec = _gpu_draft(s, W, l, m, h, tok)
    par, tk = host(head.parent), host(head.tokens)
    clean = 0
    for b in range(s.B):
        assert _valid(par[b])
        if not ref["flagged"][b]:
            clean += 1
            assert _paths(par[b], tk[b]) == _paths(ref["parent"][b], ref["tokens"][b]), f"sequence {b}"
    assert clean >= s.B // 2
    info = _check_choices(orc, s, W, l, m, h, tok, head, rec, range(s.B), tol=1e-5)
    print(f"fp32: {clean}/{s.B} unflagged trees identical; {info}")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_draft_head_small_matches_oracle(orc, seed):
    s = synth.DRAFT_SMALL
    W = synth.draft_weights(s)
    l, m, h, tok = synth.draft_inputs(s, seed)
    head, rec = _gpu_draft(s, W, l, m, h, tok)
    ref = orc.draft_tree(s, W, l, m, h, tok)
    # context K/V in the draft cache (rows of sequence b are blocks b*nb.. in order)
    kc = host(head.k_cache).reshape(s.B, head.nb, s.Hkv, 16, s.D).transpose(0, 1, 3, 2, 4)
    kc = kc.reshape(s.B, head.nb * 16, s.Hkv, s.D)[:, :s.ctx]
    assert normwise_rel(kc, ref["k_ctx"])[0] <= 2e-2
    vc = host(head.v_cache).reshape(s.B, head.nb, s.Hkv, s.D, 16).transpose(0, 1, 4, 2, 3)
    vc = vc.reshape(s.B, head.nb * 16, s.Hkv, s.D)[:, :s.ctx]
    assert normwise_rel(vc, ref["v_ctx"])[0] <= 2e-2
    par = host(head.parent)
    assert all(_valid(p) for p in par)
    info = _check_choices(orc, s, W, l, m, h, tok, head, rec, range(s.B))
    same = sum(_paths(par[b], host(head.tokens)[b]) == _paths(ref["parent"][b], ref["tokens"][b])
               for b in range(s.B))
    print(f"seed {seed}: {same}/{s.B} trees identical to the oracle's own; {info}")


@pytest.fixture(scope="module")
def full_size_draft():
    """The full-size draft head (64 sequences, k 4096, context 1024, vocab
    128256), run once on the GPU for the tests below."""
    s = synth.DRAFT_B64
    W = synth.draft_weights(s)
    l, m, h, tok = synth.draft_inputs(s, 0)
    head, rec = _gpu_draft(s, W, l, m, h, tok)
    del l, m, h
    out = dict(s=s, W=W, tok=tok, parent=host(head.parent), tokens=host(head.tokens), head=head, rec=rec)
    yield out
    del out["head"]
    torch.cuda.empty_cache()


@pytest.mark.slow
@pytest.mark.timeout(400)
def test_draft_head_full_size_sequence0(orc, full_size_draft):
    f = full_size_draft
    s, W = f["s"], f["W"]
    assert all(_valid(p) for p in f["parent"])
    l0, m0, h0, t0 = synth.draft_inputs(s, 0, batch=slice(0, 1))
    info = _check_choices(orc, s, W, l0, m0, h0, t0, f["head"], f["rec"], [0])
    print(f"full size, sequence 0: {info}")


@pytest.mark.slow
@pytest.mark.timeout(400)
def test_verify_on_drafted_trees(orc, full_size_draft):
    """The verify step on the trees the draft head just built (8B shapes, 64
    sequences, prefix 1024, the target's head = the head the draft used; the
    draft and target are independent random models, so acceptance is rare).
    Sequence 0 against the oracle: attention within the bf16 tolerance, the
    accepted path and emitted tokens exact unless flagged."""
    import dataclasses
    import oracle as orc_mod
    import tree_draft_verification_amd as e3
    f = full_size_draft
    shape = synth.VerifyShape("draft-b64-verify", 6, B=64, Hq=32, Hkv=8, D=128, V=128256, n_drafts=60, depth=8)
    inp = dataclasses.replace(synth.verify_inputs(shape, 0), parent=f["parent"])
    Wl = f["W"]["lm_head"]
    kc, vc, bt, pl, w = (dev(x) for x in (inp.kv.k_cache, inp.kv.v_cache, inp.kv.block_table, inp.kv.prefix_len, Wl))
    step = e3.VerifyStep(shape.B, shape.T, shape.Hq, shape.Hkv, shape.D, shape.V, kc, vc, bt, pl, w)
    par, q, kt, vt, tk = dev(inp.parent), dev(inp.q), dev(inp.k_tree), dev(inp.v_tree), dev(f["tokens"])
    step.run(par, q, kt, vt, tk)
    torch.cuda.synchronize()
    acc_len = host(step.accept_len)
    assert ((acc_len >= 0) & (acc_len <= 8)).all()
    one = dataclasses.replace(synth.verify_inputs(shape, 0, batch=slice(0, 1)), parent=f["parent"][:1])
    ref = orc_mod.verify_step(one, Wl, tokens=f["tokens"][:1])
    rel = normwise_rel(host(step.attn).reshape(shape.B, -1)[:1], ref["attn"].reshape(1, -1))[0]
    assert rel <= 2e-2
    idx = host(step.idx).reshape(shape.B, shape.T)[0]
    clean = ref["gap"][0] >= 1e-3
    assert np.array_equal(idx[clean], ref["idx"][0][clean])
    if not ref["flagged"][0]:
        for name in ("accept_len", "path", "out_tokens"):
            assert np.array_equal(host(getattr(step, name))[:1], ref[name]), name
    print(f"verify on drafted trees: accept_len mean {acc_len.mean():.3f} (sequence 0: {acc_len[0]}, "
          f"flagged {bool(ref['flagged'][0])}), attention rel err {rel:.2e}")


def test_vocab_map_kernel():
    import tree_draft_verification_amd as e3
    rng = np.random.default_rng(3)
    vmap = np.sort(rng.choice(50000, 3000, replace=False)).astype(np.int32)
    for n in (1, 1023, 1024, 6400):
        ids = rng.integers(0, 3000, size=n).astype(np.int32)
        d_ids, d_map = dev(ids), dev(vmap)
        out = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        st = torch.full((1,), 99, dtype=torch.int32, device="cuda")
        e3.eagle3_vocab_map(d_ids, d_map, out=out, status=st)
        e3.eagle3_vocab_map(d_ids, d_map)                          # in place
        torch.cuda.synchronize()
        assert np.array_equal(host(out), vmap[ids]) and np.array_equal(host(d_ids), vmap[ids])
        assert int(host(st)[0]) == 0
    # out-of-range ids: -1 there, the rest mapped, the range status set
    ids = np.array([0, 2999, 3000, -1, 17, 1 << 30], np.int32)
    out = torch.empty(len(ids), dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    e3.eagle3_vocab_map(dev(ids), dev(vmap), out=out, status=st)
    torch.cuda.synchronize()
    assert host(out).tolist() == [vmap[0], vmap[2999], -1, -1, vmap[17], -1]
    assert int(host(st)[0]) == -4                                   # EAGLE3_ERR_RANGE
    # nothing to map: the status still reads OK
    e3.eagle3_vocab_map(torch.empty(0, dtype=torch.int32, device="cuda"), dev(vmap), status=st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0


@pytest.mark.parametrize("seed", [0, 1])
def test_draft_head_small_trimmed_vocab_matches_oracle(orc, seed):
    s = synth.DRAFT_SMALL_TRIM
    vocab = synth.draft_vocab(s)
    W = synth.draft_weights(s)
    l, m, h, tok = synth.draft_inputs(s, seed)
    head, rec = _gpu_draft(s, W, l, m, h, tok, vocab)
    tk = host(head.tokens)
    assert np.isin(tk[:, 1:], vocab).all() and np.isin(host(head.pool_token)[:, :s.pool_len], vocab).all()
    info = _check_choices(orc, s, W, l, m, h, tok, head, rec, range(s.B), vocab=vocab)
    ref = orc.draft_tree(s, W, l, m, h, tok, vocab=vocab)
    same = sum(_paths(host(head.parent)[b], tk[b]) == _paths(ref["parent"][b], ref["tokens"][b])
               for b in range(s.B))
    print(f"trimmed vocab ({s.vocab_keep} of {s.V}), seed {seed}: {same}/{s.B} trees identical to the "
          f"oracle's own; {info}")


@pytest.mark.slow
@pytest.mark.timeout(400)
def test_draft_head_full_size_trimmed_vocab_sequence0(orc):
    """The full-size draft head with half of the 128256 vocabulary rows
    kept; sequence 0 replayed through the oracle's trimmed head."""
    s = synth.DRAFT_B64_TRIM
    vocab = synth.draft_vocab(s)
    W = synth.draft_weights(s)
    l, m, h, tok = synth.draft_inputs(s, 0)
    head, rec = _gpu_draft(s, W, l, m, h, tok, vocab)
    del l, m, h
    assert all(_valid(p) for p in host(head.parent))
    assert np.isin(host(head.tokens)[:, 1:], vocab).all()
    l0, m0, h0, t0 = synth.draft_inputs(s, 0, batch=slice(0, 1))
    info = _check_choices(orc, s, W, l0, m0, h0, t0, head, rec, [0], vocab=vocab)
    print(f"full size, trimmed vocab, sequence 0: {info}")
    del head
    torch.cuda.empty_cache()
