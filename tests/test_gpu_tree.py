"""GPU parity of the ancestor mask and greedy acceptance against the oracle:
bit-exact (integer work)."""
import itertools

import numpy as np
import pytest
import torch

import synth
from _gpu import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import tree_draft_verification_amd as t
    return t


@pytest.mark.parametrize("T", [1, 2, 16, 61, 64, 65, 100, 128])
def test_tree_mask_bit_exact(orc, lib, T):
    rng = np.random.default_rng(T)
    B = 7
    parent = np.stack([synth.random_tree(rng, T, max_children=int(rng.integers(1, 11))) for _ in range(B)])
    W = (T + 63) // 64
    ref_mask, ref_depth = orc.tree_mask(parent, W)
    for Wc in sorted({W, 2}):
        mask = torch.empty((B, T, Wc), dtype=torch.int64, device="cuda")
        depth = torch.empty((B, T), dtype=torch.int32, device="cuda")
        status = torch.full((B,), 99, dtype=torch.int32, device="cuda")
        lib.eagle3_tree_mask(dev(parent), Wc, mask, depth, status)
        torch.cuda.synchronize()
        got = host(mask).view(np.uint64)
        want, _ = orc.tree_mask(parent, Wc)
        assert np.array_equal(got, want)
        assert np.array_equal(host(depth), ref_depth)
        assert np.all(host(status) == 0)


def test_tree_mask_flags_bad_trees(lib):
    parent = np.array([[-1, 0, 1, 2], [0, 0, 1, 2], [-1, 0, 3, 1], [-1, 1, 0, 0]], np.int32)
    mask = torch.empty((4, 4, 1), dtype=torch.int64, device="cuda")
    status = torch.full((4,), 99, dtype=torch.int32, device="cuda")
    lib.eagle3_tree_mask(dev(parent), 1, mask, None, status)
    torch.cuda.synchronize()
    assert list(host(status)) == [0, -3, -3, -3]


def run_accept(lib, tok, parent, idx, use_mask, orc):
    B, T = parent.shape
    W = (T + 63) // 64
    al = torch.empty((B,), dtype=torch.int32, device="cuda")
    path = torch.empty((B, T), dtype=torch.int32, device="cuda")
    out = torch.empty((B, T), dtype=torch.int32, device="cuda")
    if use_mask:
        m, _ = orc.tree_mask(parent, W)
        lib.eagle3_accept_path(dev(tok), dev(idx), al, path, out, mask=dev(m))
    else:
        lib.eagle3_accept_path(dev(tok), dev(idx), al, path, out, parent=dev(parent))
    torch.cuda.synchronize()
    return host(al), host(path), host(out)


@pytest.mark.parametrize("use_mask", [False, True])
def test_accept_exhaustive_binary_tree(orc, lib, use_mask):
    parent = synth.binary_tree_15()
    T = 16
    idx = (np.arange(T) * 7 + 3).astype(np.int32)
    pats = np.array(list(itertools.product([False, True], repeat=15)))
    B = pats.shape[0]
    tok = np.tile((idx[np.maximum(parent, 0)] + 1000).astype(np.int32), (B, 1))
    tok[:, 1:] = np.where(pats, idx[parent[1:]][None, :], tok[:, 1:])
    P = np.tile(parent, (B, 1)); I = np.tile(idx, (B, 1))
    want = orc.accept(tok, P, I)
    got = run_accept(lib, tok, P, I, use_mask, orc)
    for g, w in zip(got, want[:3]):
        assert np.array_equal(g, w)


@pytest.mark.parametrize("T", [1, 2, 33, 61, 64, 65, 128])
@pytest.mark.parametrize("use_mask", [False, True])
def test_accept_random_trees(orc, lib, T, use_mask):
    rng = np.random.default_rng(T * 3 + use_mask)
    B = 600
    parent = np.stack([synth.random_tree(rng, T, max_children=int(rng.integers(1, 6))) for _ in range(B)])
    idx = rng.integers(0, 20, size=(B, T)).astype(np.int32)
    u = rng.random((B, T))
    rid = rng.integers(0, 20, size=(B, T)).astype(np.int32)
    tok = synth.plant_tokens(parent, idx, rng.uniform(0.3, 1.0, size=B), u, rid)
    want = orc.accept(tok, parent, idx)
    got = run_accept(lib, tok, parent, idx, use_mask, orc)
    for g, w in zip(got, want[:3]):
        assert np.array_equal(g, w)


def test_accept_lesson_cases(orc, lib):
    # chain of 5 drafts: first 4 right -> 5 tokens; first 1 -> 2; none -> 1
    parent = np.tile(synth.chain_tree(5), (3, 1))
    idx = np.tile(np.arange(10, 16, dtype=np.int32), (3, 1))
    tok = idx[:, np.maximum(parent[0], 0)] + 100
    tok[0, 1:5] = idx[0, 0:4]
    tok[1, 1] = idx[1, 0]
    al, path, out = run_accept(lib, tok.astype(np.int32), parent, idx, False, orc)
    assert list(al) == [4, 1, 0]
    assert [int((o >= 0).sum()) for o in out] == [5, 2, 1]


def test_accept_validate_mode_flags_bad_ids(orc, lib):
    """Validate mode (status non-NULL): one bad id planted per sequence. A
    token outside [0, V) and a target id below 0 give EAGLE3_ERR_RANGE, a
    parent[] out of topological order EAGLE3_ERR_TREE; clean sequences get
    EAGLE3_OK and their outputs still equal the oracle's."""
    rng = np.random.default_rng(5)
    B, T, V = 5, 61, 3001
    parent = np.stack([synth.random_tree(rng, T, max_children=10) for _ in range(B)])
    idx = rng.integers(0, V, size=(B, T)).astype(np.int32)
    tok = synth.plant_tokens(parent, idx, np.full(B, 0.9), rng.random((B, T)), rng.integers(0, V, size=(B, T)))
    tok = tok.astype(np.int32)
    want = orc.accept(tok, parent, idx)
    tok[1, 17] = V                       # token past the vocabulary
    idx[2, 40] = -1                      # negative target id
    parent[3, 30] = 45                   # a parent after its child
    al = torch.empty((B,), dtype=torch.int32, device="cuda")
    path = torch.empty((B, T), dtype=torch.int32, device="cuda")
    out = torch.empty((B, T), dtype=torch.int32, device="cuda")
    status = torch.full((B,), 99, dtype=torch.int32, device="cuda")
    lib.eagle3_accept_path(dev(tok), dev(idx), al, path, out, parent=dev(parent), V=V, status=status)
    torch.cuda.synchronize()
    assert list(host(status)) == [0, -4, -4, -3, 0]
    for b in (0, 4):
        assert host(al)[b] == want[0][b] and np.array_equal(host(path)[b], want[1][b])
    # the same call in mask mode: the range checks still apply, the tree check needs parent[]
    m, _ = orc.tree_mask(np.where(np.arange(B)[:, None] == 3, np.stack([synth.chain_tree(T - 1)] * B), parent), 1)
    status.fill_(99)
    lib.eagle3_accept_path(dev(tok), dev(idx), al, path, out, mask=dev(m), V=V, status=status)
    torch.cuda.synchronize()
    assert list(host(status)) == [0, -4, -4, 0, 0]
