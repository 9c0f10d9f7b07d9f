"""GPU checks of the device-resident speculative decoding loop (SpecLoop:
draft tree -> target pass -> acceptance -> commit -> draft context extension,
one fixed launch sequence per step).

* eagle3_spec_advance against a plain restatement of its bookkeeping.
* fp32 storage (small target and draft over a 16-token vocabulary, so
  multi-token acceptances occur): the emitted tokens of every sequence equal
  the oracle's own greedy continuation of the target, token by token, up to
  the first oracle near-tie (top-2 gap below 1e-3); the sequence lengths
  grow by exactly the emitted count.
* the draft's context extension of every step (fp32 and bf16) replayed
  through the oracle's draft_context on the same inputs (the target's
  feature rows of the accepted path, the tokens after them, the cache rows
  before the step): the new cache rows and the draft output a_root within
  1e-5 (fp32) / 2e-2 (bf16) normwise.
* bf16 storage: the same against the bf16 oracle up to its first gap below
  2e-2 (bf16 rounding moves these logits by a few 1e-3); a loop replayed
  from a captured HIP graph reproduces the eager loop bit for bit (emitted
  tokens, lengths, caches, the draft's a_root).
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests._gpu import dev, host, normwise_rel

pytestmark = pytest.mark.gpu


def test_spec_advance_bookkeeping():
    import tree_draft_verification_amd as e3
    rng = np.random.default_rng(1)
    B, T, R, cap = 7, 61, 9, 20
    a = rng.integers(0, R, size=B).astype(np.int32)
    a[0], a[1] = 0, R - 1
    path = np.full((B, T), -1, np.int32)
    out_t = np.full((B, T), -1, np.int32)
    for b in range(B):
        path[b, :a[b] + 1] = np.concatenate([[0], np.sort(rng.choice(np.arange(1, T), a[b], replace=False))])
        out_t[b, :a[b] + 1] = rng.integers(0, 1000, size=a[b] + 1)
    plen = rng.integers(10, 500, size=B).astype(np.int32)
    out_len = rng.integers(0, 15, size=B).astype(np.int32)
    out_seq = np.full((B, cap), -7, np.int32)
    d = dict(plen=dev(plen), start=dev(np.zeros(B, np.int32)), rows=dev(np.zeros((B, R), np.int32)),
             tok=dev(np.zeros((B, R), np.int32)), last=dev(np.zeros(B, np.int32)), root=dev(np.zeros(B, np.int32)),
             seq=dev(out_seq), n=dev(out_len))
    e3.eagle3_spec_advance(dev(a), dev(path), dev(out_t), d["plen"], d["start"], d["rows"], d["tok"], d["last"],
                           d["root"], d["seq"], d["n"])
    torch.cuda.synchronize()
    assert np.array_equal(host(d["start"]), plen)
    assert np.array_equal(host(d["plen"]), plen + a + 1)
    assert np.array_equal(host(d["last"]), np.arange(B) * R + a)
    for b in range(B):
        j = np.arange(R)
        want_rows = np.where(j <= a[b], b * T + path[b, np.minimum(j, a[b])], -1)
        assert np.array_equal(host(d["rows"])[b], want_rows)
        assert np.array_equal(host(d["tok"])[b], np.where(j <= a[b], out_t[b, np.minimum(j, a[b])], 0))
        assert host(d["root"])[b] == out_t[b, a[b]]
        seq = out_seq[b].copy()
        for jj in range(a[b] + 1):
            if out_len[b] + jj < cap:
                seq[out_len[b] + jj] = out_t[b, jj]
        assert np.array_equal(host(d["seq"])[b], seq)
    assert np.array_equal(host(d["n"]), out_len + a + 1)


def _build(seed, S, f32):
    import tree_draft_verification_amd as e3
    ts, ds = synth.LOOP_TARGET_SMALL, synth.LOOP_DRAFT_SMALL
    R = ds.steps + 1
    Wt = synth.target_weights(ts)
    Wd = synth.draft_weights(ds)
    Wd["embed"], Wd["lm_head"] = Wt["embed"], Wt["lm_head"]
    tin = synth.target_inputs(ts, seed, reserve=S * R + 16, dtype="f32" if f32 else "bf16")
    l, m, h, ctx_tok = synth.draft_inputs(ds, seed)
    if f32:
        cv = synth.bf16_to_f32
        Wt = {k: cv(v) for k, v in Wt.items()}
        Wd = {k: cv(v) for k, v in Wd.items()}
        l, m, h = cv(l), cv(m), cv(h)
    target = e3.TargetModel({k: dev(v) for k, v in Wt.items()}, ts.layers, ts.B, ts.T, ts.Hq, ts.Hkv, ts.D,
                            [dev(c) for c in tin.k_cache], [dev(c) for c in tin.v_cache], dev(tin.block_table),
                            dev(tin.prefix_len), ts.theta, ts.eps, features=ts.features)
    draft = e3.DraftHead({k: dev(v) for k, v in Wd.items()}, ds.B, ds.ctx, ds.Hq, ds.Hkv, ds.D, ds.steps, ds.topk,
                         ds.n_drafts, ds.theta, ds.eps, prefix_len=target.plen, reserve=S * R + 16, extend_rows=R)
    draft.ingest(dev(l), dev(m), dev(h), dev(ctx_tok))
    loop = e3.SpecLoop(target, draft, cap=S * R)
    loop.host_draft_weights = Wd
    return loop, tin, Wt, ctx_tok


def _check_greedy(orc, loop, tin, Wt, ctx_tok, tie):
    """Emitted tokens against the oracle's greedy continuation, each sequence
    up to (not including) its first choice with a top-2 gap below `tie`."""
    n_out, seq = host(loop.out_len), host(loop.out_seq)
    want, gaps = orc.target_greedy(tin, Wt, ctx_tok[:, -1], int(n_out.max()))
    checked = 0
    for b in range(len(n_out)):
        near = np.flatnonzero(gaps[b, :n_out[b]] < tie)
        upto = int(near[0]) if len(near) else int(n_out[b])
        assert np.array_equal(seq[b, :upto], want[b, :upto]), (b, seq[b, :n_out[b]], want[b, :n_out[b]])
        checked += upto
    return checked


@pytest.mark.parametrize("seed", [0, 1])
def test_loop_f32_emits_the_targets_greedy_tokens(orc, seed):
    S = 6
    loop, tin, Wt, ctx_tok = _build(seed, S, f32=True)
    acc = []
    for _ in range(S):
        loop.step()
        torch.cuda.synchronize()
        acc.append(host(loop.t.accept_len).copy())
    acc = np.stack(acc)
    n_out = host(loop.out_len)
    assert np.array_equal(n_out, (acc + 1).sum(0))
    assert np.array_equal(host(loop.t.plen), tin.prefix_len + n_out)
    checked = _check_greedy(orc, loop, tin, Wt, ctx_tok, 1e-3)
    assert acc.max() >= 1, "no step accepted a draft: the multi-row paths went untested"
    print(f"seed {seed}: accept_len per step {acc.T.tolist()}, {checked} emitted tokens equal the greedy ones")


def test_loop_bf16_graph_replay_equals_eager_and_greedy(orc):
    S = 5
    eager, tin, Wt, ctx_tok = _build(2, S, f32=False)
    for _ in range(S):
        eager.step()
    torch.cuda.synchronize()
    rep, _, _, _ = _build(2, S, f32=False)
    rep.step()                                   # sizes every workspace, then capture
    torch.cuda.synchronize()
    g = rep.graph()
    for _ in range(S - 1):
        g.replay()
        torch.cuda.synchronize()                 # host work between replays
    for name in ("out_len", "out_seq"):
        assert np.array_equal(host(getattr(rep, name)), host(getattr(eager, name))), name
    assert np.array_equal(host(rep.t.plen), host(eager.t.plen))
    assert np.array_equal(host(rep.d.a_root), host(eager.d.a_root))
    for i in range(tin.shape.layers):
        assert np.array_equal(host(rep.t.k_caches[i]), host(eager.t.k_caches[i]))
        assert np.array_equal(host(rep.t.v_caches[i]), host(eager.t.v_caches[i]))
    assert np.array_equal(host(rep.d.k_cache), host(eager.d.k_cache))
    checked = _check_greedy(orc, eager, tin, Wt, ctx_tok, 2e-2)
    print(f"bf16: {host(eager.out_len).tolist()} tokens emitted in {S} steps, {checked} checked against greedy")


def _draft_rows(cache, B, nb):
    """Paged draft cache with its identity table -> rows [B, nb * 16, Hkv, D]."""
    if cache.ndim == 4 and cache.shape[2] == 16:                      # K: [blocks, Hkv, 16, D]
        x = cache.reshape(B, nb, cache.shape[1], 16, cache.shape[3]).transpose(0, 1, 3, 2, 4)
    else:                                                              # V: [blocks, Hkv, D, 16]
        x = cache.reshape(B, nb, cache.shape[1], cache.shape[2], 16).transpose(0, 1, 4, 2, 3)
    return x.reshape(B, nb * 16, x.shape[-2], x.shape[-1])


@pytest.mark.parametrize("f32", [True, False])
def test_loop_draft_extension_matches_oracle(orc, f32):
    S = 3
    loop, tin, Wt, ctx_tok = _build(3, S, f32)
    ts, ds = synth.LOOP_TARGET_SMALL, synth.LOOP_DRAFT_SMALL
    d, t = loop.d, loop.t
    tol = 1e-5 if f32 else 2e-2
    B, T, R = ds.B, ts.T, d.R
    worst = 0.0
    for step in range(S):
        kc0, vc0 = host(d.k_cache), host(d.v_cache)
        loop.step()
        torch.cuda.synchronize()
        a, path, out, start = host(t.accept_len), host(t.path), host(t.out_tokens), host(loop.start)
        feats = [host(t.feat[i]) for i in ts.features]
        rows = np.stack([b * T + np.where(np.arange(R) <= a[b], path[b, :R], path[b, 0]) for b in range(B)])
        l, m, h = (f[rows] for f in feats)
        tok = np.where(np.arange(R)[None, :] <= a[:, None], out[:, :R], 0).astype(np.int32)
        pk, pv = _draft_rows(kc0, B, d.nb), _draft_rows(vc0, B, d.nb)
        kn, vn, a_last = orc.draft_context(ds, loop.host_draft_weights, l, m, h, tok, start, pk, pv, last=a)
        k1, v1 = _draft_rows(host(d.k_cache), B, d.nb), _draft_rows(host(d.v_cache), B, d.nb)
        for b in range(B):
            sl = slice(int(start[b]), int(start[b]) + int(a[b]) + 1)
            for got, want in ((k1[b, sl], kn[b, :a[b] + 1]), (v1[b, sl], vn[b, :a[b] + 1])):
                rel = normwise_rel(got, want)[0]
                worst = max(worst, rel)
                assert rel <= tol, (step, b, rel)
            # the rows before the step are untouched
            assert np.array_equal(k1[b, :start[b]], pk[b, :start[b]])
        rel = normwise_rel(host(d.a_root), a_last)[0]
        worst = max(worst, rel)
        assert rel <= tol, (step, rel)
    print(f"{'fp32' if f32 else 'bf16'}: draft extension over {S} steps within {worst:.2e}")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_loop_8b_full_size(orc):
    """The 8B loop (64 sequences, 1024-token contexts, 32-layer target, the
    EAGLE-3 draft head), three steps from a captured graph: lengths and
    emitted counts consistent, and for sequences 0 and 1 the emitted tokens
    equal the bf16 oracle's greedy continuation up to its first top-2 gap
    below 5e-2 (32 layers of bf16 storage move these logits by up to a few
    1e-2; each layer alone is bounded by the layer replay test), and the last
    step's draft extension replayed through the oracle within 2e-2."""
    import tree_draft_verification_amd as e3
    ts, ds = synth.LOOP_TARGET_8B, synth.DRAFT_B64
    S, R = 3, ds.steps + 1
    Wt = synth.target_weights(ts)
    Wd = synth.draft_weights(ds)
    Wd["embed"], Wd["lm_head"] = Wt["embed"], Wt["lm_head"]
    tin = synth.target_inputs(ts, 0, reserve=S * R + 16)
    l, m, h, ctx_tok = synth.draft_inputs(ds, 0)
    print("8B loop: inputs drawn", flush=True)
    wt = {k: dev(v) for k, v in Wt.items()}
    wd = {k: (wt[k] if k in ("embed", "lm_head") else dev(v)) for k, v in Wd.items()}
    target = e3.TargetModel(wt, ts.layers, ts.B, ts.T, ts.Hq, ts.Hkv, ts.D, [dev(c) for c in tin.k_cache],
                            [dev(c) for c in tin.v_cache], dev(tin.block_table), dev(tin.prefix_len), ts.theta, ts.eps,
                            features=ts.features)
    draft = e3.DraftHead(wd, ds.B, ds.ctx, ds.Hq, ds.Hkv, ds.D, ds.steps, ds.topk, ds.n_drafts, ds.theta, ds.eps,
                         prefix_len=target.plen, reserve=S * R + 16, extend_rows=R)
    draft.ingest(dev(l), dev(m), dev(h), dev(ctx_tok))
    del l, m, h
    loop = e3.SpecLoop(target, draft, cap=S * R)
    loop.step()
    torch.cuda.synchronize()
    g = loop.graph()
    kc0, vc0 = host(draft.k_cache), host(draft.v_cache)
    for _ in range(S - 1):
        if _ == S - 2:
            torch.cuda.synchronize()
            kc0, vc0 = host(draft.k_cache), host(draft.v_cache)
        g.replay()
    torch.cuda.synchronize()
    print("8B loop: GPU steps done", flush=True)
    n_out = host(loop.out_len)
    assert np.array_equal(host(target.plen), tin.prefix_len + n_out)
    assert (n_out >= S).all() and (n_out <= S * R).all()
    # the last step's draft extension, sequences 0 and 1
    a, path, out, start = host(target.accept_len), host(target.path), host(target.out_tokens), host(loop.start)
    feats = [host(target.feat[i]) for i in ts.features]
    sel = [0, 1]
    rows = np.stack([b * ts.T + np.where(np.arange(R) <= a[b], path[b, :R], path[b, 0]) for b in sel])
    lf, mf, hf = (f[rows] for f in feats)
    tok = np.where(np.arange(R)[None, :] <= a[sel, None], out[sel, :R], 0).astype(np.int32)
    pk, pv = _draft_rows(kc0, ds.B, draft.nb)[sel], _draft_rows(vc0, ds.B, draft.nb)[sel]
    one = dataclasses.replace(ds, B=2)
    kn, vn, a_last = orc.draft_context(one, Wd, lf, mf, hf, tok, start[sel], pk, pv, last=a[sel])
    k1 = _draft_rows(host(draft.k_cache), ds.B, draft.nb)
    for i, b in enumerate(sel):
        s0 = int(start[b])
        assert normwise_rel(k1[b, s0:s0 + a[b] + 1], kn[i, :a[b] + 1])[0] <= 2e-2
    assert normwise_rel(host(draft.a_root)[sel], a_last)[0] <= 2e-2
    print("8B loop: draft extension replayed", flush=True)
    # lossless: sequences 0 and 1 against the oracle's greedy continuation
    two = dataclasses.replace(tin, shape=dataclasses.replace(ts, B=2), prefix_len=tin.prefix_len[:2],
                              block_table=tin.block_table[:2])
    want, gaps = orc.target_greedy(two, Wt, ctx_tok[:2, -1], int(n_out[:2].max()))
    seq = host(loop.out_seq)
    checked = 0
    for b in range(2):
        near = np.flatnonzero(gaps[b, :n_out[b]] < 5e-2)
        upto = int(near[0]) if len(near) else int(n_out[b])
        assert np.array_equal(seq[b, :upto], want[b, :upto]), (b, seq[b, :n_out[b]], want[b, :n_out[b]])
        checked += upto
    print(f"8B loop: emitted {n_out[:4].tolist()}..., {checked} tokens of sequences 0-1 equal the greedy ones",
          flush=True)
