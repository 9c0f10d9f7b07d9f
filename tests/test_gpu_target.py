"""GPU parity of the target model's pass over draft trees (TargetModel: the
decoder layers at M = B * T rows, RoPE at cached length + depth, tree
attention over each layer's paged prefix, LM head, acceptance, commit)
against the oracle's target_forward / target_layer.

* node positions: bit-exact.
* small shape, fp32 storage: every layer's output within 1e-5 (normwise),
  the tree K/V rows likewise, argmax equal wherever the oracle's top-2 gap is
  at least 1e-3, accepted paths exact for unflagged sequences.
* small shape, bf16 storage: each layer replayed through the oracle on the
  GPU's own input of that layer (so rounding differences do not compound)
  within the bf16 tolerance (2e-2 normwise); the oracle's LM head on the
  GPU's final hidden state gives the GPU's argmax wherever its gap is at
  least 1e-3; acceptance on the GPU's argmax equals the oracle's accept rule
  on it exactly; the whole forward within 2e-2 of the oracle's own.
* commit: the accepted path's K/V rows land in every layer's cache at the
  positions after the prefix, bit for bit.
* full 8B shape (32 layers, 64 sequences): one root path of sequence 0
  replayed layer by layer, and the LM head on the final hidden state.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests._gpu import dev, host, normwise_rel

pytestmark = pytest.mark.gpu


def _model(inp, W, features=()):
    import tree_draft_verification_amd as e3
    s = inp.shape
    wd = {k: dev(v) for k, v in W.items()}
    kc = [dev(c) for c in inp.k_cache]
    vc = [dev(c) for c in inp.v_cache]
    m = e3.TargetModel(wd, s.layers, s.B, s.T, s.Hq, s.Hkv, s.D, kc, vc, dev(inp.block_table), dev(inp.prefix_len),
                       s.theta, s.eps, features=features)
    return m


def _f32(inp, W):
    cv = synth.bf16_to_f32
    inp = dataclasses.replace(inp, k_cache=[cv(c) for c in inp.k_cache], v_cache=[cv(c) for c in inp.v_cache])
    return inp, {k: cv(v) for k, v in W.items()}


def test_node_positions():
    import tree_draft_verification_amd as e3
    rng = np.random.default_rng(0)
    for B, T in ((1, 1), (5, 61), (64, 128)):
        plen = rng.integers(0, 5000, size=B).astype(np.int32)
        depth = rng.integers(0, 9, size=(B, T)).astype(np.int32)
        pos = torch.full((B, T), -1, dtype=torch.int32, device="cuda")
        e3.eagle3_node_positions(dev(plen), dev(depth), pos)
        torch.cuda.synchronize()
        assert np.array_equal(host(pos), plen[:, None] + depth)


def test_target_small_f32_matches_oracle(orc):
    s = synth.TARGET_SMALL
    inp, W = _f32(synth.target_inputs(s, 0), synth.target_weights(s))
    ref = orc.target_forward(inp, W)
    m = _model(inp, W)
    rec = []
    m.run(dev(inp.parent), dev(inp.tokens), record=rec)
    torch.cuda.synchronize()
    assert np.array_equal(host(m.pos), ref["pos"])
    for i, x in enumerate(rec):
        rel = normwise_rel(host(x), ref["x"][i])[0]
        assert rel <= 1e-5, (i, rel)
    for i in range(s.layers):
        assert normwise_rel(host(m.k_rows[i]), ref["rows"][i][0])[0] <= 1e-5
        assert normwise_rel(host(m.v_rows[i]), ref["rows"][i][1])[0] <= 1e-5
    idx = host(m.idx).reshape(s.B, s.T)
    clean = ref["gap"] >= 1e-3
    assert np.array_equal(idx[clean], ref["idx"][clean])
    for b in range(s.B):
        if not ref["flagged"][b]:
            assert host(m.accept_len)[b] == ref["accept_len"][b]
            assert np.array_equal(host(m.path)[b], ref["path"][b])


@pytest.mark.parametrize("seed", [0, 1])
def test_target_small_bf16_layer_replay(orc, seed):
    s = synth.TARGET_SMALL
    inp, W = synth.target_inputs(s, seed), synth.target_weights(s)
    m = _model(inp, W)
    rec = []
    tok = dev(inp.tokens)
    m.run(dev(inp.parent), tok, record=rec)
    torch.cuda.synchronize()
    xs = [host(x) for x in rec]
    mask, depth = orc.tree_mask(inp.parent)
    pos = (inp.prefix_len[:, None] + depth).astype(np.int32)
    assert np.array_equal(xs[0], W["embed"][inp.tokens])            # the embedding gather is a copy
    worst = 0.0
    for i in range(s.layers):
        want, kr, vr = orc.target_layer(s, W, i, xs[i], pos, mask, inp.kv(i))
        rel = normwise_rel(xs[i + 1], want)[0]
        worst = max(worst, rel)
        assert rel <= 2e-2, (i, rel)
        assert normwise_rel(host(m.k_rows[i]), kr)[0] <= 2e-2
        assert normwise_rel(host(m.v_rows[i]), vr)[0] <= 2e-2
    hf = orc.rmsnorm(xs[-1].reshape(-1, s.k), eps=s.eps)
    idx2, _, gap, _ = orc.lmhead(hf, W["lm_head"], topk=2)
    idx = host(m.idx).reshape(-1)
    clean = gap >= 1e-3
    assert np.array_equal(idx[clean], idx2[clean, 0])
    alen, path, out, _ = orc.accept(inp.tokens, inp.parent, idx.reshape(s.B, s.T))
    assert np.array_equal(host(m.accept_len), alen) and np.array_equal(host(m.path), path)
    assert np.array_equal(host(m.out_tokens), out)
    # the free-running forward stays within the bf16 tolerance of the oracle's
    ref = orc.target_forward(inp, W)
    assert normwise_rel(xs[-1], ref["x"][-1])[0] <= 2e-2
    print(f"seed {seed}: worst layer replay {worst:.2e}")


def test_target_commit_appends_the_accepted_rows(orc):
    s = synth.TARGET_SMALL
    inp, W = synth.target_inputs(s, 2, reserve=16), synth.target_weights(s)
    # every node carries the oracle's argmax at its parent, planted depth by
    # depth (a node's argmax depends on its ancestors' tokens), so the whole
    # deepest path is accepted
    _, depth = orc.tree_mask(inp.parent)
    tok = inp.tokens.copy()
    for d in range(1, int(depth.max()) + 1):
        idx = orc.target_forward(dataclasses.replace(inp, tokens=tok), W)["idx"]
        for b in range(s.B):
            for n in np.flatnonzero(depth[b] == d):
                tok[b, n] = idx[b, inp.parent[b, n]]
    m = _model(inp, W)
    m.run(dev(inp.parent), dev(tok))
    torch.cuda.synchronize()
    m.commit()
    torch.cuda.synchronize()
    path, alen = host(m.path), host(m.accept_len)
    assert alen.max() >= 3
    bs = 16
    for i in range(s.layers):
        kc, vc = host(m.k_caches[i]), host(m.v_caches[i])
        kr, vr = host(m.k_rows[i]), host(m.v_rows[i])
        for b in range(s.B):
            P = int(inp.prefix_len[b])
            for j in range(alen[b] + 1):
                p = P + j
                blk = inp.block_table[b, p // bs]
                assert np.array_equal(kc[blk, :, p % bs, :], kr[b, path[b, j]])
                assert np.array_equal(vc[blk, :, :, p % bs], vr[b, path[b, j]])
            # the prefix itself is untouched
            for t in (0, P - 1):
                blk = inp.block_table[b, t // bs]
                assert np.array_equal(kc[blk, :, t % bs], inp.k_cache[i][blk, :, t % bs])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_target_8b_full_size_root_path_replay(orc):
    """The 8B target over 64 trees of 61 nodes (32 layers): for the deepest
    root path of sequence 0, each layer replayed through the oracle on the
    GPU's input rows of that path (its rows attend only to each other and the
    prefix, so the path alone is a complete input), and the oracle's LM head
    on the GPU's final hidden rows of the path."""
    s = synth.TARGET_8B
    inp, W = synth.target_inputs(s, 0), synth.target_weights(s)
    print("8B target: inputs drawn", flush=True)
    m = _model(inp, W)
    rec = []
    m.run(dev(inp.parent), dev(inp.tokens), record=rec)
    torch.cuda.synchronize()
    print("8B target: GPU pass done", flush=True)
    par = inp.parent[0]
    _, depth = orc.tree_mask(par)
    n = int(np.argmax(depth[0]))
    path = [n]
    while par[path[-1]] > 0:
        path.append(int(par[path[-1]]))
    path = np.array([0] + path[::-1])
    chain = synth.chain_tree(len(path) - 1)[None]
    mask, cdepth = orc.tree_mask(chain)
    pos = (inp.prefix_len[0] + cdepth).astype(np.int32)
    worst = 0.0
    for i in range(s.layers):
        x_in = host(rec[i][0])[path][None]
        want, _, _ = orc.target_layer(s, W, i, x_in, pos, mask, inp.kv(i, slice(0, 1)))
        rel = normwise_rel(host(rec[i + 1][0])[path][None], want)[0]
        worst = max(worst, rel)
        assert rel <= 2e-2, (i, rel)
        if i % 8 == 7:
            print(f"8B target: layers 0..{i} replayed, worst {worst:.2e}", flush=True)
    hf = orc.rmsnorm(host(rec[-1][0])[path], eps=s.eps)
    idx2, _, gap, _ = orc.lmhead(hf, W["lm_head"], topk=2)
    idx = host(m.idx).reshape(s.B, s.T)[0, path]
    clean = gap >= 1e-3
    assert np.array_equal(idx[clean], idx2[clean, 0])
    al = host(m.accept_len)
    assert ((al >= 0) & (al <= s.depth)).all()
    print(f"8B target, sequence 0 path of {len(path)} nodes: worst layer replay {worst:.2e}; "
          f"accept_len mean {al.mean():.3f}")
