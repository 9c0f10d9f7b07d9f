"""Pins for the oracle's target decoder pass over draft trees (CPU only).

What fixes the answers, independently of the oracle's own composition:
* one layer for a single node, written out in numpy fp64 from the textbook
  definitions (RMSNorm, the three projections, RoPE as a complex rotation,
  softmax attention over the paged prefix and the node itself with query
  head h reading KV head h // (Hq / Hkv), output projection + residual,
  SiLU(gate) * up, down projection + residual);
* with every output projection zeroed the layers are the identity on the
  residual stream, so the argmax is a brute-force numpy argmax of
  RMSNorm(E[token]) against the LM head;
* a chain through the tree pass equals feeding its tokens one at a time and
  appending each one's K/V to the cache (causal decoding);
* every node of a random tree sees only its root path: its output equals the
  last node's output of the chain made of that path;
* the greedy continuation fed back as one chain reproduces itself.
"""
import dataclasses

import numpy as np
import pytest

import synth

S = dataclasses.replace(synth.TARGET_SMALL, B=2, n_drafts=14, depth=5, prefix=(40, 90))


def f32_inputs(shape, seed=0):
    inp = synth.target_inputs(shape, seed, dtype="f32")
    W = {k: synth.bf16_to_f32(v) for k, v in synth.target_weights(shape).items()}
    return inp, W


def _rows_of(kv, b, layer_cache_k, layer_cache_v, L):
    """Logical prefix rows [L, Hkv, D] of sequence b from the paged cache."""
    bs = kv.block_size
    ks, vs = [], []
    for t in range(L):
        blk = kv.block_table[b, t // bs]
        ks.append(layer_cache_k[blk, :, t % bs, :])
        vs.append(layer_cache_v[blk, :, :, t % bs])
    return np.asarray(ks, np.float64), np.asarray(vs, np.float64)


def _rms(x, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _rope(x, pos, theta):
    D = x.shape[-1]
    j = np.arange(D // 2)
    z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * pos * theta ** (-2.0 * j / D))
    return np.concatenate([z.real, z.imag], -1)


def test_one_layer_single_node_by_hand(orc):
    s = dataclasses.replace(S, n_drafts=0, depth=0, layers=1)
    inp, W = f32_inputs(s, 1)
    r = orc.target_forward(inp, W)
    qd, kvd, G = s.Hq * s.D, s.Hkv * s.D, s.Hq // s.Hkv
    wqkv = W["l0.wqkv"].astype(np.float64)
    for b in range(s.B):
        P = int(inp.prefix_len[b])
        x = W["embed"][inp.tokens[b, 0]].astype(np.float64)
        h = _rms(x, s.eps)
        q = _rope((h @ wqkv[:qd].T).reshape(s.Hq, s.D), P, s.theta)
        k = _rope((h @ wqkv[qd:qd + kvd].T).reshape(s.Hkv, s.D), P, s.theta)
        v = (h @ wqkv[qd + kvd:].T).reshape(s.Hkv, s.D)
        Kp, Vp = _rows_of(inp.kv(0), b, inp.k_cache[0], inp.v_cache[0], P)
        attn = np.empty((s.Hq, s.D))
        for hh in range(s.Hq):
            g = hh // G
            keys = np.concatenate([Kp[:, g], k[g][None]])
            vals = np.concatenate([Vp[:, g], v[g][None]])
            sc = keys @ q[hh] / np.sqrt(s.D)
            w = np.exp(sc - sc.max())
            attn[hh] = (w / w.sum()) @ vals
        x1 = x + attn.reshape(-1) @ W["l0.wo"].astype(np.float64).T
        gu = _rms(x1, s.eps) @ W["l0.wgu"].astype(np.float64).T
        gate, up = gu[:s.F], gu[s.F:]
        x2 = x1 + (gate / (1 + np.exp(-gate)) * up) @ W["l0.wd"].astype(np.float64).T
        got = r["x"][1][b, 0].astype(np.float64)
        assert np.abs(got - x2).max() <= 1e-5 * np.abs(x2).max(), b
        krow = r["rows"][0][0][b, 0].astype(np.float64)
        assert np.abs(krow - k).max() <= 1e-5 * np.abs(k).max()


def test_zero_output_projections_leave_the_embedding(orc):
    inp, W = f32_inputs(S, 2)
    for i in range(S.layers):
        W[f"l{i}.wo"] = np.zeros_like(W[f"l{i}.wo"])
        W[f"l{i}.wd"] = np.zeros_like(W[f"l{i}.wd"])
    r = orc.target_forward(inp, W)
    E, Wl = W["embed"].astype(np.float64), W["lm_head"].astype(np.float64)
    for b in range(S.B):
        assert np.array_equal(r["x"][-1][b], W["embed"][inp.tokens[b]])
        logits = _rms(E[inp.tokens[b]], S.eps) @ Wl.T
        order = np.argsort(-logits, axis=1, kind="stable")
        srt = np.take_along_axis(logits, order, 1)
        clear = (srt[:, 0] - srt[:, 1]) > 1e-6
        assert np.array_equal(r["idx"][b][clear], order[clear, 0])


def _chain_inputs(inp, b, toks, plen, k_cache, v_cache, table):
    """Inputs of one sequence whose tree is a chain over `toks`."""
    s = dataclasses.replace(inp.shape, B=1, n_drafts=len(toks) - 1)
    return synth.TargetInputs(s, inp.seed, synth.chain_tree(len(toks) - 1)[None], np.asarray(toks, np.int32)[None],
                              np.array([plen], np.int32), table, k_cache, v_cache)


def test_chain_equals_token_by_token_decoding(orc):
    s = dataclasses.replace(S, B=1, n_drafts=11, depth=11)
    inp, W = f32_inputs(s, 3)
    inp = dataclasses.replace(inp, parent=synth.chain_tree(s.n_drafts)[None])
    whole = orc.target_forward(inp, W)
    P0 = int(inp.prefix_len[0])
    T = s.T
    # grow the cache by hand: enough fresh blocks after the prefix's
    bs = 16
    nb0 = (P0 + bs - 1) // bs
    need = (P0 + T + bs - 1) // bs
    kc = [np.concatenate([c, np.full((need - nb0,) + c.shape[1:], np.nan, c.dtype)]) for c in inp.k_cache]
    vc = [np.concatenate([c, np.full((need - nb0,) + c.shape[1:], np.nan, c.dtype)]) for c in inp.v_cache]
    nblk0 = inp.k_cache[0].shape[0]
    table = np.concatenate([inp.block_table[0, :nb0], nblk0 + np.arange(need - nb0)]).astype(np.int32)[None]
    for t in range(T):
        one = _chain_inputs(inp, 0, [inp.tokens[0, t]], P0 + t, kc, vc, table)
        r = orc.target_forward(one, W)
        want = whole["x"][-1][0, t].astype(np.float64)
        got = r["x"][-1][0, 0].astype(np.float64)
        assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max(), t
        assert r["idx"][0, 0] == whole["idx"][0, t] or whole["gap"][0, t] < 1e-5
        pos = P0 + t
        for layer, (kr, vr) in enumerate(r["rows"]):
            kc[layer][table[0, pos // bs], :, pos % bs, :] = kr[0, 0]
            vc[layer][table[0, pos // bs], :, :, pos % bs] = vr[0, 0]


def test_every_node_sees_only_its_root_path(orc):
    inp, W = f32_inputs(S, 4)
    r = orc.target_forward(inp, W)
    for b in range(S.B):
        par = inp.parent[b]
        for n in (1, 5, len(par) - 1, len(par) // 2):
            path = [n]
            while par[path[-1]] > 0:
                path.append(int(par[path[-1]]))
            path = [0] + path[::-1]
            one = _chain_inputs(inp, b, inp.tokens[b, path], int(inp.prefix_len[b]), inp.k_cache, inp.v_cache,
                                inp.block_table[b:b + 1])
            c = orc.target_forward(one, W)
            want = r["x"][-1][b, n].astype(np.float64)
            got = c["x"][-1][0, -1].astype(np.float64)
            assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max(), (b, n)


def test_greedy_continuation_is_the_chain_pass_of_its_own_tokens(orc):
    """Feeding the greedy tokens back as one chain through the tree pass gives
    the same argmax at every node (and each next token is that argmax)."""
    s = dataclasses.replace(S, B=2)
    _, W = f32_inputs(s, 5)
    inp = synth.target_inputs(s, 5, dtype="f32", reserve=32)
    root = inp.tokens[:, 0]
    n = 9
    toks, gaps = orc.target_greedy(inp, W, root, n)
    for b in range(s.B):
        chain = np.concatenate([[root[b]], toks[b, :-1]]).astype(np.int32)
        one = _chain_inputs(inp, b, chain, int(inp.prefix_len[b]), inp.k_cache, inp.v_cache,
                            inp.block_table[b:b + 1])
        r = orc.target_forward(one, W)
        clear = gaps[b] >= 1e-5
        assert np.array_equal(r["idx"][0][clear], toks[b][clear])
    # the caches of the inputs are left alone
    again, _ = orc.target_greedy(inp, W, root, n)
    assert np.array_equal(again, toks)
