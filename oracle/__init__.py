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
import dataclasses
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
    L.orc_silu_mul.argtypes = [I, P, I, I, P]
    L.orc_silu_mul.restype = None
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


def silu_mul(GU):
    GU = _c(GU)
    M, F = GU.shape[0], GU.shape[1] // 2
    Y = np.empty((M, F), dtype=GU.dtype)
    lib().orc_silu_mul(_dt(GU), _p(GU), M, F, _p(Y))
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
        tokens = synth.plant_for(inp, fw["idx"])
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
    MLP (gate/up product stored, then gated) + residual; final RMSNorm -> LM
    head -> argmax.
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
            f = silu_mul(gemm(h2, self.w[f"l{i}.wgu"]))
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


# ------------------------------------------------------------------ target model

def target_layer(shape, W, i, x, pos, mask, kv):
    """Decoder layer i of the target over the tree rows of B sequences.

    Course lesson "EAGLE-3 speculative decoding: the tree-verifier method":
    the target runs once over the whole tree, each token attending to the
    cached context and its own ancestors. reading: a Llama decoder layer
    (pre-norm RMSNorm with gamma = 1, GQA projections, rotate-half RoPE at
    position prefix length + depth, tree attention over the layer's paged
    prefix plus the ancestor-masked tree rows, output projection + residual,
    RMSNorm, SwiGLU MLP + residual), every intermediate stored in x's type.
    x [B, T, k]; pos [B, T]; mask [B, T, W]. Returns (x_out, k_rows, v_rows)
    with the rows' K (after RoPE) and V [B, T, Hkv, D] for the cache."""
    s = shape
    B, T, k = x.shape
    qd, kvd = s.Hq * s.D, s.Hkv * s.D
    wqkv = W[f"l{i}.wqkv"]
    xr = x.reshape(B * T, k)
    h = rmsnorm(xr, eps=s.eps)
    p = pos.reshape(-1)
    q = rope(gemm(h, wqkv[:qd]).reshape(B * T, s.Hq, s.D), p, s.theta)
    kr = rope(gemm(h, wqkv[qd:qd + kvd]).reshape(B * T, s.Hkv, s.D), p, s.theta)
    vr = gemm(h, wqkv[qd + kvd:]).reshape(B * T, s.Hkv, s.D)
    q4, k4, v4 = q.reshape(B, T, s.Hq, s.D), kr.reshape(B, T, s.Hkv, s.D), vr.reshape(B, T, s.Hkv, s.D)
    attn, _ = tree_attn(q4, k4, v4, kv, mask, want_lse=False)
    xr = gemm(attn.reshape(B * T, qd), W[f"l{i}.wo"], R=xr)
    f = silu_mul(gemm(rmsnorm(xr, eps=s.eps), W[f"l{i}.wgu"]))
    xr = gemm(f, W[f"l{i}.wd"], R=xr)
    return xr.reshape(B, T, k), k4, v4


def target_forward(inp: synth.TargetInputs, W, batch=None, layers=None):
    """The target's pass over the draft trees: embedding of every node's
    token, the decoder layers, final RMSNorm, LM head (top-2) and the greedy
    acceptance of the nodes' tokens. ``batch`` selects sequences; ``layers``
    runs only the first n layers. Returns the per-layer inputs "x" (x[0] is
    the embedding, x[n] the last layer's output), the tree K/V rows per layer,
    argmax / gap per node and the accepted path."""
    s = inp.shape
    sel = np.arange(s.B) if batch is None else np.arange(s.B)[batch]
    parent, tokens = inp.parent[sel], inp.tokens[sel]
    B, T = parent.shape
    n_layers = s.layers if layers is None else layers
    mask, depth = tree_mask(parent)
    pos = (inp.prefix_len[sel][:, None] + depth).astype(np.int32)
    x = embed(W["embed"], tokens.reshape(-1)).reshape(B, T, s.k)
    xs, rows = [x], []
    for i in range(n_layers):
        x, kr, vr = target_layer(s, W, i, x, pos, mask, inp.kv(i, sel))
        xs.append(x)
        rows.append((kr, vr))
    hf = rmsnorm(x.reshape(B * T, s.k), eps=s.eps)
    idx, val, gap, _ = lmhead(hf, W["lm_head"], topk=2)
    idx1 = idx[:, 0].reshape(B, T).copy()
    alen, path, out, end = accept(tokens, parent, idx1)
    return dict(x=xs, rows=rows, mask=mask, depth=depth, pos=pos, hidden=hf, idx=idx1, gap=gap.reshape(B, T),
                accept_len=alen, path=path, out_tokens=out, end=end,
                flagged=flags(parent, tokens, idx1, gap.reshape(B, T)))


def target_greedy(inp: synth.TargetInputs, W, root, n: int):
    """The target's own greedy continuation, one token at a time (course
    lesson, "Verify-accept semantics": speculative decoding must emit exactly
    these tokens). For every sequence: feed `root` at position prefix_len,
    take the argmax, append that node's K/V to the cache of every layer (in
    the reserved blocks after the prefix), feed the argmax next, n times.
    Returns tokens [B, n] and the top-2 gap of each choice [B, n]; the caches
    of `inp` are not modified."""
    s = inp.shape
    B = s.B
    kc = [c.copy() for c in inp.k_cache]
    vc = [c.copy() for c in inp.v_cache]
    bs = 16
    toks = np.zeros((B, n), np.int32)
    gaps = np.zeros((B, n))
    for b in range(B):
        P = int(inp.prefix_len[b])
        cur = int(root[b])
        for t in range(n):
            if (P + t) // bs >= inp.block_table.shape[1]:
                raise ValueError("the block table has no room for the continuation")
            one = synth.TargetInputs(dataclasses.replace(s, B=1, n_drafts=0, depth=0), inp.seed,
                                     np.array([[-1]], np.int32), np.array([[cur]], np.int32),
                                     np.array([P + t], np.int32), inp.block_table[b:b + 1], kc, vc)
            r = target_forward(one, W)
            for layer, (kr, vr) in enumerate(r["rows"]):
                blk, slot = inp.block_table[b, (P + t) // bs], (P + t) % bs
                kc[layer][blk, :, slot, :] = kr[0, 0]
                vc[layer][blk, :, :, slot] = vr[0, 0]
            cur = int(r["idx"][0, 0])
            toks[b, t] = cur
            gaps[b, t] = r["gap"][0, 0]
    return toks, gaps


# ------------------------------------------------------------------ draft head

def _page(rows_k, rows_v, bs=16):
    """Contiguous per-sequence K/V rows [B, L, Hkv, D] -> PagedKV (identity tables)."""
    B, L, Hkv, Dh = rows_k.shape
    nb = (L + bs - 1) // bs
    kc = np.zeros((B * nb, Hkv, bs, Dh), rows_k.dtype)
    vc = np.zeros((B * nb, Hkv, Dh, bs), rows_v.dtype)
    for b in range(B):
        for j in range(nb):
            n = min(bs, L - j * bs)
            kc[b * nb + j, :, :n, :] = rows_k[b, j * bs:j * bs + n].transpose(1, 0, 2)
            vc[b * nb + j, :, :, :n] = rows_v[b, j * bs:j * bs + n].transpose(1, 2, 0)
    table = (np.arange(B)[:, None] * nb + np.arange(nb)[None, :]).astype(np.int32)
    return synth.PagedKV(kc, vc, table, np.full(B, L, np.int32), bs)


def _draft_layer_tail(s, W, x, attn):
    """Output projection + residual, RMSNorm, SwiGLU MLP + residual of the
    draft's decoder layer (reading R15: a Llama layer)."""
    x = gemm(attn, W["wo"], R=x)
    f = silu_mul(gemm(rmsnorm(x, eps=s.eps), W["wgu"]))
    return gemm(f, W["wd"], R=x)


def draft_context(shape, W, l, m, h, tok_ahead, start, prev_k=None, prev_v=None, last=None):
    """Context rows entering the draft (news write-up of the EAGLE-3 paper,
    draft stage: row t fuses the target's low / mid / high features of token
    t with the embedding of token t + 1, its K/V at position t join the
    draft's cache, and the whole layer runs at the newest row to give the
    output the next tree grows from).

    l, m, h [B, n, k]; tok_ahead [B, n]; start [B]: position of row 0;
    prev_k, prev_v [B, >= start, Hkv, D]: the rows already cached (rows
    0..start[b]-1 of sequence b are used); last [B]: the row that runs the
    whole layer (default n - 1); it attends to the cached rows and new rows
    0..last. Returns the new rows' K (after RoPE) and V [B, n, Hkv, D] and the
    layer output at row last [B, k]."""
    s = shape
    B, n, k = l.shape
    qd, kvd = s.Hq * s.D, s.Hkv * s.D
    wq, wk, wv = W["wqkv"][:qd], W["wqkv"][qd:qd + kvd], W["wqkv"][qd + kvd:]
    start = np.asarray(start, np.int32)
    last = np.full(B, n - 1, np.int64) if last is None else np.asarray(last, np.int64)
    x = draft_fuse(np.asarray(tok_ahead, np.int32).reshape(-1), W["embed"], W["w_fuse"], W["w_in"],
                   l=l.reshape(-1, k), m=m.reshape(-1, k), h=h.reshape(-1, k))
    hn = rmsnorm(x, eps=s.eps)
    pos = (start[:, None] + np.arange(n, dtype=np.int32)[None, :]).reshape(-1)
    kr = rope(gemm(hn, wk).reshape(B * n, s.Hkv, s.D), pos, s.theta).reshape(B, n, s.Hkv, s.D)
    vr = gemm(hn, wv).reshape(B, n, s.Hkv, s.D)
    out = np.empty((B, k), x.dtype)
    for b in range(B):
        L0, j = int(start[b]), int(last[b])
        old_k = prev_k[b, :L0] if L0 else np.zeros((0, s.Hkv, s.D), kr.dtype)
        old_v = prev_v[b, :L0] if L0 else np.zeros((0, s.Hkv, s.D), vr.dtype)
        cache = _page(np.concatenate([old_k, kr[b, :j + 1]])[None], np.concatenate([old_v, vr[b, :j + 1]])[None])
        row = b * n + j
        q = rope(gemm(hn[row:row + 1], wq).reshape(1, s.Hq, s.D), np.array([L0 + j], np.int32), s.theta)
        empty = np.zeros((1, 0, s.Hkv, s.D), x.dtype)
        attn, _ = tree_attn(q[:, None], empty, empty, cache, np.zeros((1, 1, 1), np.uint64), want_lse=False)
        out[b] = _draft_layer_tail(s, W, x[row:row + 1], attn.reshape(1, qd))[0]
    return kr, vr, out


class OwnChoice:
    """The selections of draft_tree itself: a node's children are its top-k
    logits by (value desc, id asc); the next frontier and the final tree are
    the top candidates by (score desc, creation asc).

    draft_tree asks a chooser for every selection it makes, so a caller can
    evaluate this arithmetic along other selections (the tests replay another
    run's choices that way); `wide` is how many of each row's top logits the
    chooser is shown."""

    def __init__(self, C):
        self.C = C
        self.wide = C + 1

    def children(self, step, idx, val):
        """-> ids [M, C], their logits [M, C]."""
        return idx[:, :self.C], val[:, :self.C]

    def frontier(self, step, cand, start):
        """-> the next frontier as indices into this step's candidates [B, C]."""
        creation = np.tile(np.arange(start, start + cand.shape[1], dtype=np.int32), (cand.shape[0], 1))
        return select_topk(cand, creation, self.C)

    def final(self, pool_score, N):
        """-> pool indices of the final tree [B, N] (any order)."""
        P = pool_score.shape[1]
        return select_topk(pool_score, np.tile(np.arange(P, dtype=np.int32), (pool_score.shape[0], 1)), N)


def draft_tree(shape, W, l, m, h, ctx_tok, gap=GAP_FLAG, chooser=None, vocab=None):
    """EAGLE-3 draft head and EAGLE-2 style tree growth, for B sequences.

    News write-up of the EAGLE-3 paper, draft stage: context row t fuses the
    target's low/mid/high features (g_t = W_fuse [l_t; m_t; h_t]) with the
    embedding of the token one step ahead (x_t = W_in [g_t; E[tok_{t+1}]]);
    every row's K/V enters the draft cache (RoPE at position t); the full
    single layer runs at the last context row, giving a_root. From step 2 on,
    the target's feature of a drafted token is unavailable and the draft's own
    output of the parent stands in: x_n = W_in [a_parent; E[tok_n]].
    readings: the layer is a Llama decoder layer; a node at depth d sits at
    position ctx + d - 1 and attends to the draft cache plus the draft rows of
    its ancestors and itself; logp = fp32(logit - lse) of RMSNorm(a) through
    the target's LM head; score(child) = fp32(score(parent) + logp); each step
    keeps the top-k candidates as the next frontier and every candidate in the
    pool; the final tree is the top n_drafts of the pool by (score desc,
    creation asc), renumbered in creation order under the root.

    chooser: who makes the selections (default OwnChoice). Returns parent,
    tokens [B, n+1]; "flagged" per sequence (own choices only): some selection
    boundary within `gap` that can reach the final tree (a top-k boundary of a
    node's children or a frontier boundary whose score at stake lies within
    `gap` of the n-th pool score, or the final rerank boundary); "choices"
    (the selections made); "rows": per growth step s >= 2 the frontier's
    tokens, the row of each frontier node's parent in the previous step's
    outputs (a_root for step 2), the position and the fused inputs x.

    vocab: a trimmed draft vocabulary (Spec-Bench blog post, sections 1, 3.2
    and 5.1: VocabTrim / FR-Spec / SpecVocab shrink the draft's search space
    by 40-60%): the kept token ids, strictly ascending. reading: the draft LM
    head keeps only those rows of the LM-head weight, its top-k, lse and logp
    range over the kept rows alone, and each chosen row maps back to its full
    vocabulary id before it enters the tree (and the next step's embedding).
    Ascending ids make the lowest kept row on a tie the lowest full id."""
    s = shape
    B, ctx, k = l.shape
    qd, kvd, C = s.Hq * s.D, s.Hkv * s.D, s.topk
    wq, wk, wv = W["wqkv"][:qd], W["wqkv"][qd:qd + kvd], W["wqkv"][qd + kvd:]
    own = chooser is None
    ch = OwnChoice(C) if own else chooser
    near = np.zeros(B, bool)
    lm_vals, a_steps, rows = [], [], []
    choices = {"ids": [], "frontier": []}

    def layer_tail(x, attn):
        return _draft_layer_tail(s, W, x, attn)

    if vocab is not None:
        vocab = np.asarray(vocab, np.int64)
        if vocab.ndim != 1 or len(vocab) <= C or (np.diff(vocab) <= 0).any() or vocab[0] < 0 \
                or vocab[-1] >= W["lm_head"].shape[0]:
            raise ValueError("vocab must be strictly ascending ids of the LM head's rows, more than topk of them")
        w_head = W["lm_head"][vocab]
    else:
        w_head = W["lm_head"]

    def head(a, step):
        idx, val, _, lse = lmhead(rmsnorm(a, eps=s.eps), w_head, topk=ch.wide)
        if vocab is not None:
            idx = vocab[idx]
        ids, v = ch.children(step, idx, val)
        ids = np.asarray(ids).reshape(-1, C).astype(np.int32)
        v = np.asarray(v).reshape(-1, C)
        lm_vals.append(v.reshape(B, -1, C))
        logp = (v - lse[:, None]).astype(np.float32)
        choices["ids"].append(ids.reshape(B, -1, C))
        return ids, logp, val[:, C - 1] - val[:, C]

    def take(cand, step, start):
        order = np.asarray(ch.frontier(step, cand, start)).astype(np.int64)
        choices["frontier"].append(order)
        return order

    # context rows -> draft cache
    x = draft_fuse(ctx_tok.reshape(-1), W["embed"], W["w_fuse"], W["w_in"],
                   l=l.reshape(-1, k), m=m.reshape(-1, k), h=h.reshape(-1, k))
    hn = rmsnorm(x, eps=s.eps)
    pos = np.tile(np.arange(ctx, dtype=np.int32), B)
    kr = rope(gemm(hn, wk).reshape(B * ctx, s.Hkv, s.D), pos, s.theta)
    vr = gemm(hn, wv).reshape(B * ctx, s.Hkv, s.D)
    cache = _page(kr.reshape(B, ctx, s.Hkv, s.D), vr.reshape(B, ctx, s.Hkv, s.D))
    # the last context row runs the whole layer: a_root
    last = np.arange(B) * ctx + ctx - 1
    qr = rope(gemm(hn[last], wq).reshape(B, s.Hq, s.D), np.full(B, ctx - 1, np.int32), s.theta)
    empty = np.zeros((B, 0, s.Hkv, s.D), x.dtype)
    attn, _ = tree_attn(qr[:, None], empty, empty, cache, np.zeros((B, 1, 1), np.uint64), want_lse=False)
    a_prev = layer_tail(x[last], attn.reshape(B, qd))                      # [B, k]
    a_root = a_prev
    # step 1: the root's top-k children are the first frontier
    ids, logp, lm_gap = head(a_prev, 1)
    # near-ties seen along the way: (gap [B, n], score at stake [B, n])
    ties = [(lm_gap[:, None], logp[:, C - 1:C].astype(np.float32))]
    pool_score = [logp.astype(np.float32)]                                 # [B, C] per step
    pool_tok = [ids.reshape(B, C)]
    pool_par = [np.full((B, C), -1, np.int32)]
    order = take(pool_score[0], 1, 0)
    fr_pool = order.astype(np.int32)                                       # pool index of each frontier slot
    fr_score = np.take_along_axis(pool_score[0], order, 1)
    fr_tok = np.take_along_axis(pool_tok[0], order, 1)
    fr_arow = np.zeros((B, C), np.int64)                                   # parent's row in a_prev (the root)
    fr_rows = [[[] for _ in range(C)] for _ in range(B)]                   # ancestors' draft rows
    tk = np.zeros((B, (s.steps - 1) * C, s.Hkv, s.D), x.dtype)
    tv = np.zeros_like(tk)
    n_pool = C
    for step in range(2, s.steps + 1):
        base = (step - 2) * C
        per_seq = a_prev.shape[0] // B
        a_par = a_prev[(np.arange(B)[:, None] * per_seq + fr_arow).reshape(-1)]
        xs = draft_fuse(fr_tok.reshape(-1), W["embed"], W["w_fuse"], W["w_in"], a_prev=a_par)
        hs = rmsnorm(xs, eps=s.eps)
        # the frontier of step s holds nodes of depth s - 1: position ctx + depth - 1
        ps = np.full(B * C, ctx + step - 2, np.int32)
        rows.append(dict(step=step, tokens=fr_tok.copy(), parent_row=fr_arow.copy(), pos=ps.reshape(B, C).copy(),
                         x=xs.reshape(B, C, k).copy()))
        q = rope(gemm(hs, wq).reshape(B * C, s.Hq, s.D), ps, s.theta)
        tk[:, base:base + C] = rope(gemm(hs, wk).reshape(B * C, s.Hkv, s.D), ps, s.theta).reshape(B, C, s.Hkv, s.D)
        tv[:, base:base + C] = gemm(hs, wv).reshape(B, C, s.Hkv, s.D)
        mask = np.zeros((B, C, 2), np.uint64)
        for b in range(B):
            for i in range(C):
                fr_rows[b][i] = fr_rows[b][i] + [base + i]
                for r in fr_rows[b][i]:
                    mask[b, i, r // 64] |= np.uint64(1) << np.uint64(r % 64)
        attn, _ = tree_attn(q.reshape(B, C, s.Hq, s.D), tk, tv, cache, mask, want_lse=False)
        a_prev = layer_tail(xs, attn.reshape(B * C, qd))                   # [B*C, k]
        a_steps.append(a_prev)
        ids, logp, lm_gap = head(a_prev, step)
        cand = (fr_score[:, :, None] + logp.reshape(B, C, C)).astype(np.float32).reshape(B, C * C)
        ties.append((lm_gap.reshape(B, C), cand.reshape(B, C, C)[:, :, C - 1]))
        pool_score.append(cand)
        pool_tok.append(ids.reshape(B, C * C))
        pool_par.append(np.repeat(fr_pool, C, axis=1))
        if own:
            creation = np.tile(np.arange(n_pool, n_pool + C * C, dtype=np.int32), (B, 1))
            srt = np.take_along_axis(cand, select_topk(cand, creation, C + 1), 1)
            ties.append(((srt[:, C - 1] - srt[:, C])[:, None], srt[:, C - 1:C]))
        order = take(cand, step, n_pool)
        new_rows = [[list(fr_rows[b][o // C]) for o in order[b]] for b in range(B)]
        fr_arow = (order // C).astype(np.int64)                           # parent = frontier slot o // C
        fr_pool = (n_pool + order).astype(np.int32)
        fr_score = np.take_along_axis(cand, order, 1)
        fr_tok = np.take_along_axis(ids.reshape(B, C * C), order, 1)
        fr_rows = new_rows
        n_pool += C * C
    ps_all = np.concatenate(pool_score, 1)
    tok_all = np.concatenate(pool_tok, 1)
    par_all = np.concatenate(pool_par, 1)
    N = s.n_drafts
    sel = np.sort(np.asarray(ch.final(ps_all, N)).astype(np.int64), axis=1)
    choices["selected"] = sel
    if own:
        _, _, nb_ = tree_rerank(ps_all, tok_all, par_all, ctx_tok[:, -1], N, gap)
        near |= nb_
        # A near-tie (the k-th / (k+1)-th child of one node, or the last / first
        # candidate outside a frontier) may resolve the other way on another
        # machine. Scores never grow along a path, so it can change the final
        # tree only if the score at stake is within `gap` of the N-th pool score.
        theta = np.take_along_axis(ps_all, sel, 1).min(axis=1, keepdims=True)
        for g, sc in ties:
            near |= ((g < gap) & (sc >= theta - gap)).any(axis=1)
    parent = np.full((B, N + 1), -1, np.int32)
    tokens = np.zeros((B, N + 1), np.int32)
    for b in range(B):
        new = {int(c): i + 1 for i, c in enumerate(sel[b])}
        tokens[b, 0] = ctx_tok[b, -1]
        for c in sel[b]:
            pp = int(par_all[b, c])
            parent[b, new[int(c)]] = 0 if pp < 0 else new.get(pp, -2)   # -2: parent not in the tree
            tokens[b, new[int(c)]] = tok_all[b, c]
    return dict(parent=parent, tokens=tokens, flagged=near, pool_score=ps_all, pool_token=tok_all,
                pool_parent=par_all, x_ctx=x.reshape(B, ctx, k), k_ctx=kr.reshape(B, ctx, s.Hkv, s.D),
                v_ctx=vr.reshape(B, ctx, s.Hkv, s.D), a_root=a_root, a_steps=a_steps, lm_val=lm_vals,
                choices=choices, rows=rows, tree_k=tk, tree_v=tv)


def tree_rerank(pool_score, pool_token, pool_parent, root_token, N, gap=GAP_FLAG):
    """Pool -> top N by (score desc, creation asc) -> creation order under the
    root (node 0 = root_token): parent, tokens [B, N+1]; `near` flags a gap
    below `gap` at the N-th / (N+1)-th boundary."""
    pool_score = np.atleast_2d(pool_score).astype(np.float32)
    B, P = pool_score.shape
    k = min(N + 1, P)
    order = select_topk(pool_score, np.tile(np.arange(P, dtype=np.int32), (B, 1)), k)
    srt = np.take_along_axis(pool_score, order, 1)
    near = (srt[:, N - 1] - srt[:, N]) < gap if P > N else np.zeros(B, bool)
    parent = np.full((B, N + 1), -1, np.int32)
    tokens = np.zeros((B, N + 1), np.int32)
    for b in range(B):
        chosen = np.sort(order[b, :N])                                     # creation order
        new = {int(c): i + 1 for i, c in enumerate(chosen)}
        tokens[b, 0] = root_token[b]
        for c in chosen:
            pp = int(pool_parent[b, c])
            parent[b, new[int(c)]] = 0 if pp < 0 else new[pp]
            tokens[b, new[int(c)]] = pool_token[b, c]
    return parent, tokens, near


def tree_expand(fr_score, fr_pool, child_ids, child_logp, pool_len, NF):
    """One growth step: F frontier nodes x C children (logp per child) ->
    candidates with score fp32(score(parent) + logp) (creation order slot
    major), and the next frontier: the top NF by (score desc, creation asc).
    Returns cand_score [B, F*C], cand_parent [B, F*C] (pool index of the
    parent), next_pool / next_score / next_token / next_slot [B, NF]."""
    fr_score = np.asarray(fr_score, np.float32)
    B, F, C = child_ids.shape
    cand = (fr_score[:, :, None] + np.asarray(child_logp, np.float32)).astype(np.float32).reshape(B, F * C)
    cpar = np.repeat(np.asarray(fr_pool, np.int32), C, axis=1)
    creation = np.tile(np.arange(pool_len, pool_len + F * C, dtype=np.int32), (B, 1))
    order = select_topk(cand, creation, NF)
    return (cand, cpar, (pool_len + order).astype(np.int32), np.take_along_axis(cand, order, 1),
            np.take_along_axis(child_ids.reshape(B, F * C), order, 1), (order // C).astype(np.int32))
