"""CPU oracle for the EAGLE-3 draft-tree verify step and draft head.

TEST INFRASTRUCTURE: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg import this package. It never imports the GPU
package, and the GPU package never imports it.

The arithmetic lives in ``oracle.c`` (fp64, fixed order, row-independent);
this module marshals numpy arrays through ctypes and composes the steps the
pages describe:

* ``verify_step``: tree mask -> tree attention -> RMSNorm -> LM-head argmax
  -> greedy acceptance (course lesson "EAGLE-3 speculative decoding: the
  tree-verifier method", sections "Verify-accept semantics" and "Tree draft
  vs chain draft").
* ``ToyDecoder``: a tiny random-weight Llama-style decoder used to show the
  lossless property (the lesson: the result is identical to the target's own
  autoregressive output).
* ``draft_*``: the EAGLE-3 draft head (news write-up of the EAGLE-3 paper,
  draft-stage paragraphs) and EAGLE-2 style tree growth.

Parity status per function is listed in the module docstring of each test
file that pins it; functions with no independent pin say "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
F32, BF16 = 0, 1
ERR_TREE = -3

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I = ctypes.c_int
D = ctypes.c_double


def _declare(L):
    L.orc_round_bf16.argtypes = [D]
    L.orc_round_bf16.restype = ctypes.c_uint16
    L.orc_tree_check.argtypes = [P, I]
    L.orc_tree_check.restype = I
    L.orc_tree_mask.argtypes = [P, I, I, I, P, P]
    L.orc_tree_mask.restype = I
    L.orc_tree_attn.argtypes = [I, I, I, I, I, I, I, D, P, P, P, P, P, I, P, I, P, P, I, P, P]
    L.orc_tree_attn.restype = None
    L.orc_rmsnorm.argtypes = [I, P, P, I, I, D, P]
    L.orc_rmsnorm.restype = None
    L.orc_lmhead.argtypes = [I, P, P, I, I, I, I, P, P, P, P]
    L.orc_lmhead.restype = None
    L.orc_accept.argtypes = [P, P, P, I, I, P, P, P, P]
    L.orc_accept.restype = I
    L.orc_gemm.argtypes = [I, P, P, P, I, I, I, P]
    L.orc_gemm.restype = None
    L.orc_swiglu.argtypes = [I, P, P, I, I, I, P]
    L.orc_swiglu.restype = None
    L.orc_rope.argtypes = [I, P, P, I, I, I, D]
    L.orc_rope.restype = None
    L.orc_embed.argtypes = [I, P, P, I, I, P]
    L.orc_embed.restype = None
    L.orc_draft_fuse.argtypes = [I, P, P, P, P, P, P, P, P, I, I, P, P]
    L.orc_draft_fuse.restype = None
    L.orc_select_topk.argtypes = [P, P, I, I, I, P]
    L.orc_select_topk.restype = None


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt(a):
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle takes float32 or bf16 bit patterns (uint16), got {a.dtype}")


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


# ------------------------------------------------------------------ primitives

def round_bf16(x: float) -> int:
    return int(lib().orc_round_bf16(float(x)))


def tree_check(parent) -> bool:
    parent = _c(parent, np.int32)
    return lib().orc_tree_check(_p(parent), parent.shape[-1]) == 0


def tree_mask(parent, W: int | None = None):
    parent = _c(np.atleast_2d(parent), np.int32)
    B, T = parent.shape
    W = W or (T + 63) // 64
    mask = np.zeros((B, T, W), dtype=np.uint64)
    depth = np.zeros((B, T), dtype=np.int32)
    if lib().orc_tree_mask(_p(parent), B, T, W, _p(mask), _p(depth)) != 0:
        raise ValueError("parent[] is not a tree in topological order with the root first")
    return mask, depth


def tree_attn(q, k_tree, v_tree, kv: synth.PagedKV, mask, scale=None, want_lse=True):
    """q [B,Tq,Hq,D]; k_tree/v_tree [B,Tk,Hkv,D]; mask uint64 [B,Tq,W]."""
    q, k_tree, v_tree = _c(q), _c(k_tree), _c(v_tree)
    dt = _dt(q)
    B, Tq, Hq, Dh = q.shape
    Tk, Hkv = k_tree.shape[1], k_tree.shape[2]
    mask = _c(mask, np.uint64)
    W = mask.shape[-1]
    scale = float(1.0 / np.sqrt(Dh)) if scale is None else float(scale)
    out = np.empty(q.shape, dtype=q.dtype)
    lse = np.empty((B, Tq, Hq), dtype=np.float32) if want_lse else None
    kc, vc = _c(kv.k_cache), _c(kv.v_cache)
    bt, pl = _c(kv.block_table, np.int32), _c(kv.prefix_len, np.int32)
    lib().orc_tree_attn(dt, B, Tq, Tk, Hq, Hkv, Dh, scale, _p(q), _p(k_tree), _p(v_tree),
                        _p(kc), _p(vc), kv.block_size, _p(bt), bt.shape[1], _p(pl),
                        _p(mask), W, _p(out), _p(lse))
    return out, lse


def rmsnorm(x, gamma=None, eps=1e-5):
    x = _c(x)
    M, K = x.reshape(-1, x.shape[-1]).shape
    y = np.empty_like(x)
    g = None if gamma is None else _c(gamma, x.dtype)
    lib().orc_rmsnorm(_dt(x), _p(x), _p(g), M, K, float(eps), _p(y))
    return y


def lmhead(h, w, topk=2):
    """Full-vocab fp64 logits -> (idx [M,topk], val [M,topk], gap [M], lse [M])."""
    h, w = _c(h), _c(w)
    assert h.dtype == w.dtype
    K = h.shape[-1]
    M = h.size // K
    N = w.shape[0]
    idx = np.empty((M, topk), dtype=np.int32)
    val = np.empty((M, topk), dtype=np.float64)
    gap = np.empty(M, dtype=np.float64)
    lse = np.empty(M, dtype=np.float64)
    lib().orc_lmhead(_dt(h), _p(h), _p(w), M, N, K, topk, _p(idx), _p(val), _p(gap), _p(lse))
    return idx, val, gap, lse


def accept(tokens, parent, target_idx):
    tokens = _c(np.atleast_2d(tokens), np.int32)
    parent = _c(np.atleast_2d(parent), np.int32)
    target_idx = _c(np.atleast_2d(target_idx), np.int32)
    B, T = parent.shape
    alen = np.empty(B, dtype=np.int32)
    path = np.empty((B, T), dtype=np.int32)
    out = np.empty((B, T), dtype=np.int32)
    end = np.empty(B, dtype=np.int32)
    if lib().orc_accept(_p(tokens), _p(parent), _p(target_idx), B, T, _p(alen), _p(path), _p(out), _p(end)) != 0:
        raise ValueError("bad tree")
    return alen, path, out, end


def gemm(A, Bm, R=None):
    A, Bm = _c(A), _c(Bm)
    M, K = A.shape
    N = Bm.shape[0]
    C = np.empty((M, N), dtype=A.dtype)
    Rr = None if R is None else _c(R, A.dtype)
    lib().orc_gemm(_dt(A), _p(A), _p(Bm), _p(Rr), M, N, K, _p(C))
    return C


def swiglu(X, Wgu):
    X, Wgu = _c(X), _c(Wgu)
    M, K = X.shape
    F = Wgu.shape[0] // 2
    Y = np.empty((M, F), dtype=X.dtype)
    lib().orc_swiglu(_dt(X), _p(X), _p(Wgu), M, F, K, _p(Y))
    return Y


def rope(x, pos, theta):
    """x [M, H, D] (copied), pos [M]."""
    x = np.array(x, copy=True, order="C")
    M, H, Dh = x.shape
    pos = _c(pos, np.int32)
    lib().orc_rope(_dt(x), _p(x), _p(pos), M, H, Dh, float(theta))
    return x


def embed(E, ids):
    E = _c(E)
    ids = _c(ids, np.int32)
    out = np.empty((ids.shape[0], E.shape[1]), dtype=E.dtype)
    lib().orc_embed(_dt(E), _p(E), _p(ids), ids.shape[0], E.shape[1], _p(out))
    return out


def draft_fuse(tok, E, Wf, Wi, l=None, m=None, h=None, a_prev=None, want_g=False):
    E, Wf, Wi = _c(E), _c(Wf), _c(Wi)
    tok = _c(tok, np.int32)
    M, k = tok.shape[0], E.shape[1]
    x = np.empty((M, k), dtype=E.dtype)
    g = np.empty((M, k), dtype=E.dtype) if want_g else None
    args = [None if a is None else _c(a) for a in (l, m, h, a_prev)]
    lib().orc_draft_fuse(_dt(E), *[_p(a) for a in args], _p(tok), _p(E), _p(Wf), _p(Wi), M, k, _p(g), _p(x))
    return (x, g) if want_g else x


def select_topk(score, order_id, k):
    score = _c(np.atleast_2d(score), np.float32)
    order_id = _c(np.atleast_2d(order_id), np.int32)
    B, n = score.shape
    sel = np.empty((B, k), dtype=np.int32)
    lib().orc_select_topk(_p(score), _p(order_id), B, n, k, _p(sel))
    return sel


# ------------------------------------------------------------------ verify step

GAP_FLAG = 1e-3


def verify_forward(inp: synth.VerifyInputs, W_lm, eps=1e-5):
    """Attention -> RMSNorm -> LM head for every node (tokens not needed:
    the synthetic q/k/v of the verify workloads do not depend on tokens)."""
    B, T = inp.parent.shape
    mask, depth = tree_mask(inp.parent)
    attn, lse = tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    K = inp.q.shape[2] * inp.q.shape[3]
    h = rmsnorm(attn.reshape(B * T, K), eps=eps)
    idx, val, gap, _ = lmhead(h, W_lm, topk=2)
    return dict(mask=mask, depth=depth, attn=attn, attn_lse=lse, hidden=h,
                idx=idx[:, 0].reshape(B, T).copy(), top2=idx.reshape(B, T, 2), val=val.reshape(B, T, 2),
                gap=gap.reshape(B, T))


def accepted_nodes(parent, tokens, idx):
    """Boolean [B,T]: node accepted = root, or its parent accepted and its token
    equals the target's argmax at the parent."""
    parent = np.atleast_2d(parent)
    B, T = parent.shape
    acc = np.zeros((B, T), dtype=bool)
    acc[:, 0] = True
    for b in range(B):
        for n in range(1, T):
            p = parent[b, n]
            acc[b, n] = acc[b, p] and tokens[b, n] == idx[b, p]
    return acc


def flags(parent, tokens, idx, gap, thresh=GAP_FLAG):
    """A sequence is flagged when some accepted node has a top-2 gap below
    ``thresh``: its argmax decides its children and the correction token, and
    a difference of rounding order may legitimately flip it."""
    acc = accepted_nodes(parent, tokens, idx)
    return np.any(acc & (np.asarray(gap) < thresh), axis=1)


def verify_step(inp: synth.VerifyInputs, W_lm, tokens=None):
    fw = verify_forward(inp, W_lm)
    if tokens is None:
        tokens = synth.plant_tokens(inp.parent, fw["idx"], inp.p_seq, inp.plant_u, inp.plant_id)
    alen, path, out, end = accept(tokens, inp.parent, fw["idx"])
    fw.update(tokens=tokens, accept_len=alen, path=path, out_tokens=out, end=end,
              flagged=flags(inp.parent, tokens, fw["idx"], fw["gap"]))
    return fw


# ------------------------------------------------------------------ toy decoder

class ToyDecoder:
    """fp32 random-weight Llama-style decoder with a paged KV cache.

    reading: pre-norm RMSNorm (gamma = 1) -> fused QKV -> rotate-half RoPE
    at position P + depth(node) -> tree attention over the cached prefix plus
    the node's ancestors -> output projection + residual -> RMSNorm -> SwiGLU
    MLP + residual; final RMSNorm -> LM head -> argmax.
    """

    def __init__(self, shape: synth.ToyShape = synth.TOY, seed: int = 0, max_pos: int = 512):
        self.s = shape
        self.w = synth.toy_weights(shape, seed)
        self.bs = 16
        nblk = (max_pos + self.bs - 1) // self.bs
        H, Dh = shape.H, shape.D
        self.k_cache = [np.zeros((nblk, H, self.bs, Dh), np.float32) for _ in range(shape.layers)]
        self.v_cache = [np.zeros((nblk, H, Dh, self.bs), np.float32) for _ in range(shape.layers)]
        self.table = np.arange(nblk, dtype=np.int32)[None, :]
        self.P = 0

    def kv(self, layer):
        return synth.PagedKV(self.k_cache[layer], self.v_cache[layer], self.table,
                             np.array([self.P], np.int32), self.bs)

    def forward(self, tokens, parent):
        """Tree forward at positions P + depth; returns (idx, gap, kv_rows)."""
        s = self.s
        T = len(tokens)
        mask, depth = tree_mask(parent)
        pos = (self.P + depth[0]).astype(np.int32)
        x = embed(self.w["embed"], np.asarray(tokens, np.int32))
        HD = s.H * s.D
        rows = []
        for i in range(s.layers):
            h = rmsnorm(x, eps=s.eps)
            qkv = gemm(h, self.w[f"l{i}.wqkv"])
            q = rope(qkv[:, :HD].reshape(T, s.H, s.D), pos, s.theta)
            k = rope(qkv[:, HD:2 * HD].reshape(T, s.H, s.D), pos, s.theta)
            v = np.ascontiguousarray(qkv[:, 2 * HD:].reshape(T, s.H, s.D))
            a, _ = tree_attn(q[None], k[None], v[None], self.kv(i), mask, want_lse=False)
            x = gemm(a[0].reshape(T, HD), self.w[f"l{i}.wo"], R=x)
            h2 = rmsnorm(x, eps=s.eps)
            f = swiglu(h2, self.w[f"l{i}.wgu"])
            x = gemm(f, self.w[f"l{i}.wd"], R=x)
            rows.append((k, v))
        hf = rmsnorm(x, eps=s.eps)
        idx, _, gap, _ = lmhead(hf, self.w["lm_head"], topk=2)
        return idx[:, 0].copy(), gap, rows

    def commit(self, rows, nodes):
        """Append the K/V rows of `nodes` (in order) at positions P, P+1, ..."""
        for i, (k, v) in enumerate(rows):
            for j, n in enumerate(nodes):
                p = self.P + j
                blk, slot = self.table[0, p // self.bs], p % self.bs
                self.k_cache[i][blk, :, slot, :] = k[n]
                self.v_cache[i][blk, :, :, slot] = v[n]
        self.P += len(nodes)

    def prefill(self, prompt):
        T = len(prompt)
        idx, gap, rows = self.forward(prompt, synth.chain_tree(T - 1))
        self.commit(rows, list(range(T)))
        return int(idx[-1]), float(gap[-1])


def toy_greedy(shape=synth.TOY, seed=0, n_new=None):
    n_new = n_new or shape.new_tokens
    m = ToyDecoder(shape, seed)
    first, g0 = m.prefill(synth.toy_prompt(shape, seed))
    out, gaps = [first], [g0]
    while len(out) < n_new:
        idx, gap, rows = m.forward([out[-1]], np.array([-1], np.int32))
        m.commit(rows, [0])
        out.append(int(idx[0])); gaps.append(float(gap[0]))
    return np.asarray(out, np.int32), np.asarray(gaps)


def toy_speculative(shape=synth.TOY, seed=0, n_new=None, parent=None, p_match=None):
    """Speculative decoding with a fixed tree and planted drafts.

    Drafts are planted depth by depth: a node's token is the target's argmax
    at its parent (taken from an oracle tree forward in which every shallower
    node already holds its final token) with probability p, else a uniform
    random id. Returns (tokens, steps) where steps records every verify step."""
    n_new = n_new or shape.new_tokens
    p_match = shape.p_match if p_match is None else p_match
    parent = synth.binary_tree_15() if parent is None else np.asarray(parent, np.int32)
    T = parent.shape[0]
    _, depth = tree_mask(parent)
    depth = depth[0]
    rs = synth.toy_plant_stream(shape, seed)
    m = ToyDecoder(shape, seed)
    first, _ = m.prefill(synth.toy_prompt(shape, seed))
    out = [first]
    steps = []
    while len(out) < n_new:
        u = rs.random(T)
        rid = rs.integers(0, shape.V, size=T).astype(np.int32)
        tok = rid.copy()
        tok[0] = out[-1]
        for d in range(1, int(depth.max()) + 1):
            idx, _, _ = m.forward(tok, parent)
            for n in range(1, T):
                if depth[n] == d and u[n] < p_match:
                    tok[n] = idx[parent[n]]
        idx, gap, rows = m.forward(tok, parent)
        alen, path, otok, end = accept(tok, parent, idx)
        a = int(alen[0])
        steps.append(dict(P=m.P, tokens=tok.copy(), idx=idx.copy(), gap=gap.copy(), accept_len=a,
                          path=path[0, :a + 1].copy(), out_tokens=otok[0, :a + 1].copy(),
                          flagged=bool(flags(parent[None], tok[None], idx[None], gap[None])[0])))
        m.commit(rows, list(path[0, :a + 1]))
        out.extend(int(t) for t in otok[0, :a + 1])
    return np.asarray(out[:n_new], np.int32), steps
