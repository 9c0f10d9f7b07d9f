"""EAGLE-3 draft head and EAGLE-2 style tree growth on the GPU, composed from
libeagle3 calls (news write-up of "EAGLE-3: Scaling up Inference Acceleration
of Large Language Models via Training-Time Test", draft-stage paragraphs; tree
parameters from the Spec-Bench blog post, section 4.2: top-k 10, 60 drafts).

Context ingest: every context row t fuses the target's low/mid/high features
with the embedding of the token one step ahead (g = W_fuse [l; m; h],
x = W_in [g; E[tok]]); RMSNorm(x) gives the row's K/V (RoPE at position t),
which go to a paged draft cache. The whole decoder layer runs only at the last
context row; its output a_root seeds the tree.

Growth: step 1 takes the top-k of the draft distribution at the root. Each
later step runs the layer once for every frontier node n, on
x = W_in [a_parent(n); E[tok_n]] at position ctx + depth(n) - 1, attending
to the draft cache plus the draft rows of n's ancestors and n itself (the
tree-attention kernel with a two-word mask); the top-k children of each node
get score = fp32(score(n) + logp), every candidate joins the pool, and the
top-k candidates form the next frontier. The final tree is the top n_drafts
of the pool, renumbered in creation order under the root.
readings: Llama decoder layer (pre-norm, GQA, SwiGLU); logp from the target's
LM head applied to RMSNorm(a); ties rank by creation index.

Trimmed draft vocabulary (Spec-Bench blog post, sections 1, 3.2 and 5.1:
VocabTrim / FR-Spec / SpecVocab): with `vocab` (kept ids, strictly
ascending), the draft LM head holds only those rows (gathered once), its
top-k, lse and logp range over them, and eagle3_vocab_map turns the chosen
rows back into full-vocabulary ids before the tree and the next step's
embedding see them.

This module owns buffers and launch order only; every step is a kernel.
"""
from __future__ import annotations

import torch

from . import binding as B_


class DraftHead:
    def __init__(self, weights: dict, B: int, ctx: int, Hq: int, Hkv: int, D: int, steps: int = 8, topk: int = 10,
                 n_drafts: int = 60, theta: float = 500000.0, eps: float = 1e-5, device="cuda", vocab=None,
                 prefix_len=None, reserve: int = 0, extend_rows: int = 0):
        """prefix_len: an int32 [B] device tensor to use as the draft cache's
        length (shared with a target model that advances it; it must read
        ctx for every sequence when ingest runs), else one of its own;
        reserve: cache room for that many rows after the context;
        extend_rows: rows per sequence that extend() takes (0: no extend)."""
        self.dev = torch.device(device)
        self.w = {k: v.to(self.dev).contiguous() for k, v in weights.items()}
        E = self.w["embed"]
        self.V, self.k = E.shape
        self.B, self.ctx, self.Hq, self.Hkv, self.D = B, ctx, Hq, Hkv, D
        self.steps, self.C, self.N = steps, topk, n_drafts
        self.theta, self.eps = theta, eps
        self.qd, self.kvd = Hq * D, Hkv * D
        self.dtype = E.dtype
        if self.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("draft weights must be bf16 or fp32")
        self.F = self.w["wd"].shape[1]
        self.wgu_paired = None
        if self.dtype == torch.bfloat16 and self.F % 128 == 0:
            self.wgu_paired = torch.empty_like(self.w["wgu"])
            B_.eagle3_copy_rows(self.w["wgu"], self.wgu_paired, 2 * self.F,
                                src_rows=B_.pair_gate_up_rows(self.F, self.dev))
        self.Tk = (steps - 1) * topk                      # tree keys: one row per frontier node per step
        self.W = (self.Tk + 63) // 64
        self.pool_cap = topk + (steps - 1) * topk * topk
        if self.Tk + topk > 64 * 2:
            raise ValueError("the draft tree needs more than two mask words")
        if n_drafts > self.pool_cap:
            raise ValueError("n_drafts exceeds the candidate pool")
        wqkv = self.w["wqkv"]
        self.wq, self.wk, self.wv = wqkv[:self.qd], wqkv[self.qd:self.qd + self.kvd], wqkv[self.qd + self.kvd:]
        bf, i32, dv = self.dtype, torch.int32, self.dev
        C, M = topk, B * topk
        # paged draft cache: identity block table, one run of blocks per sequence
        self.nb = (ctx + reserve + 15) // 16
        self.k_cache = torch.zeros(B * self.nb, Hkv, 16, D, dtype=bf, device=dv)
        self.v_cache = torch.zeros(B * self.nb, Hkv, D, 16, dtype=bf, device=dv)
        self.table = (torch.arange(B, device=dv)[:, None] * self.nb + torch.arange(self.nb, device=dv)).to(i32)
        self.plen = prefix_len if prefix_len is not None else torch.full((B,), ctx, dtype=i32, device=dv)
        # frontier positions of growth step s: cache length + s - 2 (depth s - 1)
        self.step_depth = torch.arange(steps - 1, dtype=i32, device=dv)[:, None, None].expand(steps - 1, B, C) \
            .contiguous()
        self.fr_pos = torch.empty(B, C, dtype=i32, device=dv)
        self.root = torch.zeros(B, dtype=i32, device=dv)    # node 0 of the next tree
        self.zero_start = torch.zeros(B, dtype=i32, device=dv)
        self.last = (torch.arange(B, device=dv) * ctx + ctx - 1).to(i32)
        self.ctx_pos = torch.arange(ctx, device=dv).repeat(B).to(i32)
        self.zero_pos = torch.zeros(M, dtype=i32, device=dv)
        # tree keys [B, Tk, Hkv, D]; unwritten rows stay zero and are masked out
        self.tk = torch.zeros(B, self.Tk, Hkv, D, dtype=bf, device=dv)
        self.tv = torch.zeros_like(self.tk)
        self.key_rows = [(torch.arange(B, device=dv)[:, None] * self.Tk + s * C + torch.arange(C, device=dv)).reshape(-1)
                         .to(i32) for s in range(steps - 1)]
        e = lambda *s: torch.empty(*s, dtype=bf, device=dv)  # noqa: E731
        self.x1, self.a_root = e(B, self.k), e(B, self.k)
        self.xs, self.hs, self.x2, self.h2, self.hn = (e(M, self.k) for _ in range(5))
        self.a = [e(M, self.k), e(M, self.k)]
        self.a_par = e(M, self.k)
        self.q, self.attn = e(M, self.qd), e(M, self.qd)
        self.kt, self.vt = e(M, self.kvd), e(M, self.kvd)
        self.gu, self.f = e(M, 2 * self.F), e(M, self.F)
        self.ids = torch.empty(M, C, dtype=i32, device=dv)
        self.val = torch.empty(M, C, dtype=torch.float32, device=dv)
        self.lse = torch.empty(M, dtype=torch.float32, device=dv)
        self.lm_w, self.vmap = self.w["lm_head"], None
        if vocab is not None:
            vh = torch.as_tensor(vocab).to("cpu", torch.int64).reshape(-1)
            if len(vh) <= C or not bool((vh[1:] > vh[:-1]).all()) or vh[0] < 0 or vh[-1] >= self.lm_w.shape[0]:
                raise ValueError("vocab must be strictly ascending LM-head row ids, more than topk of them")
            self.vmap = vh.to(dv, i32)
            self.lm_w = torch.empty(len(vh), self.k, dtype=bf, device=dv)
            B_.eagle3_copy_rows(self.w["lm_head"], self.lm_w, len(vh), src_rows=self.vmap)
        self.lm_ws = torch.empty(B_.eagle3_lmhead_workspace(M, self.lm_w.shape[0], self.k, C, B_._dtype(E)),
                                 dtype=torch.uint8, device=dv)
        f32 = torch.float32
        self.pool_score = torch.empty(B, self.pool_cap, dtype=f32, device=dv)
        self.pool_token = torch.empty(B, self.pool_cap, dtype=i32, device=dv)
        self.pool_parent = torch.empty(B, self.pool_cap, dtype=i32, device=dv)
        self.root_score = torch.zeros(B, 1, dtype=f32, device=dv)
        self.root_pool = torch.full((B, 1), -1, dtype=i32, device=dv)
        self.root_mask = torch.zeros(B, 1, 2, dtype=torch.int64, device=dv)
        self.fr = [dict(score=torch.empty(B, C, dtype=f32, device=dv), pool=torch.empty(B, C, dtype=i32, device=dv),
                        token=torch.empty(B, C, dtype=i32, device=dv),
                        mask=torch.empty(B, C, 2, dtype=torch.int64, device=dv),
                        arow=torch.empty(B, C, dtype=i32, device=dv)) for _ in range(2)]
        self.parent = torch.empty(B, n_drafts + 1, dtype=i32, device=dv)
        self.tokens = torch.empty(B, n_drafts + 1, dtype=i32, device=dv)
        self._ctx_bufs = None
        self._ws = None
        self._gws = None   # GEMM workspace: K splits or tile counters (shared: one stream)
        # the fusion's workspace (g, then the FCs' K splits or tile counters)
        self._fws = torch.empty(max(B_.PERSIST_WS_BYTES,
                                    B_.eagle3_draft_fuse_workspace(max(M, B * extend_rows), self.k, B_._dtype(E))),
                                dtype=torch.uint8, device=dv)
        self.R = extend_rows
        if extend_rows:
            Re = B * extend_rows
            z = lambda *s: torch.zeros(*s, dtype=bf, device=dv)  # noqa: E731
            self.ext = dict(l=z(Re, self.k), m=z(Re, self.k), h=z(Re, self.k), g=z(Re, self.k), x=z(Re, self.k),
                            hn=z(Re, self.k), k=z(Re, self.kvd), v=z(Re, self.kvd),
                            pos=torch.empty(Re, dtype=i32, device=dv),
                            depth=torch.arange(extend_rows, dtype=i32, device=dv).repeat(B, 1),
                            last_pos=torch.empty(B, dtype=i32, device=dv),
                            minus1=torch.full((B, 1), -1, dtype=i32, device=dv))
        # optional (start, end) event pairs, one taken per LM-head call, in call order
        self.events = []

    # ----------------------------------------------------------- context
    def _ctx_buffers(self):
        if self._ctx_bufs is None:
            R, bf, dv = self.B * self.ctx, self.dtype, self.dev
            self._ctx_bufs = dict(g=torch.empty(R, self.k, dtype=bf, device=dv),
                                  x=torch.empty(R, self.k, dtype=bf, device=dv),
                                  hn=torch.empty(R, self.k, dtype=bf, device=dv),
                                  k=torch.empty(R, self.kvd, dtype=bf, device=dv),
                                  v=torch.empty(R, self.kvd, dtype=bf, device=dv))
        return self._ctx_bufs

    def ingest(self, l, m, h, ctx_tok):
        """l, m, h [B, ctx, k] bf16 and ctx_tok [B, ctx] int32 (device): fills
        the draft cache and a_root."""
        B, ctx, k = self.B, self.ctx, self.k
        R = B * ctx
        cb = self._ctx_buffers()
        w = self.w
        self.ctx_tok = ctx_tok
        self.root.copy_(ctx_tok[:, -1])
        B_.eagle3_draft_fuse(ctx_tok.reshape(R), w["embed"], w["w_in"], cb["x"], w_fuse=w["w_fuse"],
                             l=l.reshape(R, k), m=m.reshape(R, k), h=h.reshape(R, k), g_out=cb["g"], ws=self._fws)
        B_.eagle3_rmsnorm(cb["x"], cb["hn"], eps=self.eps)
        self._gemm([cb["hn"]], self.wk, cb["k"])
        self._gemm([cb["hn"]], self.wv, cb["v"])
        B_.eagle3_rope(cb["k"], R, self.Hkv, self.D, self.kvd, self.ctx_pos, 0, self.theta)
        kr = cb["k"].view(B, ctx, self.Hkv, self.D)
        vr = cb["v"].view(B, ctx, self.Hkv, self.D)
        B_.eagle3_commit_kv(kr, vr, None, self.zero_start, self.k_cache, self.v_cache, self.table, max_n=ctx)
        # the full layer at the last context row of every sequence
        B_.eagle3_copy_rows(cb["x"], self.x1, B, src_rows=self.last)
        h1 = self.hs[:B]
        B_.eagle3_rmsnorm(self.x1, h1, eps=self.eps)
        q = self.q[:B]
        self._gemm([h1], self.wq, q)
        B_.eagle3_rope(q, B, self.Hq, self.D, self.qd, self.zero_pos, ctx - 1, self.theta)
        none = self.tk[:, :0]
        attn = self.attn[:B]
        a = B_.tree_attn_args(q.view(B, 1, self.Hq, self.D), none, none, self.k_cache, self.v_cache, self.table,
                              self.plen, attn.view(B, 1, self.Hq, self.D), mask=self.root_mask)
        B_.eagle3_tree_attn(a, self._attn_ws(a))
        self._layer_tail(self.x1, attn, self.a_root, B)

    def _gemm(self, a, b, c, residual=None):
        need = B_.eagle3_gemm_workspace(a, b, c, residual=residual)
        ws = None
        if need:
            if self._gws is None or self._gws.numel() < need:
                self._gws = torch.empty(need, dtype=torch.uint8, device=self.dev)
            ws = self._gws
        B_.eagle3_gemm(a, b, c, residual=residual, ws=ws)

    def _attn_ws(self, a):
        need = max(256, B_.eagle3_tree_attn_workspace(a))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.dev)
        return self._ws

    def _layer_tail(self, x, attn, out, M):
        w = self.w
        x2, h2, gu, f = self.x2[:M], self.h2[:M], self.gu[:M], self.f[:M]
        self._gemm([attn], w["wo"], x2, residual=x)
        B_.eagle3_rmsnorm(x2, h2, eps=self.eps)
        # the fused projection + gating where the separate projection would
        # not split K (few rows keep the split, which fills the chip); a split
        # workspace (at least 2 M N 4 bytes, N = 2F >= 256) exceeds the tile
        # counters' bytes of a persistent call
        if self.wgu_paired is not None and B_.eagle3_gemm_workspace([h2], w["wgu"], gu) <= B_.PERSIST_WS_BYTES:
            B_.eagle3_gemm_swiglu([h2], self.wgu_paired, f)
        else:
            self._gemm([h2], w["wgu"], gu)
            B_.eagle3_silu_mul(gu, f)
        self._gemm([f], w["wd"], out, residual=x2)

    def _head(self, a, M):
        hn = self.hn[:M]
        B_.eagle3_rmsnorm(a, hn, eps=self.eps)
        ev = self.events.pop(0) if self.events else None
        if ev:
            ev[0].record()
        B_.eagle3_lmhead_argmax(hn, self.lm_w, self.C, self.ids[:M], self.val[:M], None, self.lse[:M],
                                self.lm_ws)
        if ev:
            ev[1].record()
        if self.vmap is not None:
            B_.eagle3_vocab_map(self.ids[:M], self.vmap)

    # ----------------------------------------------------------- growth
    def grow(self, record=None):
        """Steps 1..steps, then the rerank: self.parent, self.tokens [B, N+1].
        With a list as `record`, each step appends device copies of its child
        ids / logits / lse [B, F, C] and the next frontier's pool indices."""
        B, C, D = self.B, self.C, self.D
        M = B * C
        # step 1: the root's children
        self._head(self.a_root, B)
        nx = self.fr[0]
        B_.eagle3_tree_expand(self.root_score, self.root_pool, self.root_mask, 0, 1, self.ids[:B].view(B, 1, C),
                              self.val[:B].view(B, 1, C), self.lse[:B], 0, 0, self.pool_score, self.pool_token,
                              self.pool_parent, nx["pool"], nx["score"], nx["token"], nx["mask"], nx["arow"])
        if record is not None:
            record.append(dict(ids=self.ids[:B].view(B, 1, C).clone(), val=self.val[:B].view(B, 1, C).clone(),
                               lse=self.lse[:B].view(B, 1).clone(), next_pool=nx["pool"].clone(), pool_len=0))
        a_src = self.a_root
        pool_len = C
        for s in range(2, self.steps + 1):
            fr, nx = self.fr[s % 2], self.fr[(s + 1) % 2]
            a_out = self.a[s % 2]
            B_.eagle3_copy_rows(a_src, self.a_par, M, src_rows=fr["arow"].view(-1))
            B_.eagle3_draft_fuse(fr["token"].view(-1), self.w["embed"], self.w["w_in"], self.xs, a_prev=self.a_par,
                                 ws=self._fws)
            B_.eagle3_rmsnorm(self.xs, self.hs, eps=self.eps)
            self._gemm([self.hs], self.wq, self.q)
            self._gemm([self.hs], self.wk, self.kt)
            self._gemm([self.hs], self.wv, self.vt)
            B_.eagle3_node_positions(self.plen, self.step_depth[s - 2], self.fr_pos)
            pos = self.fr_pos.view(-1)
            B_.eagle3_rope(self.q, M, self.Hq, D, self.qd, pos, 0, self.theta)
            B_.eagle3_rope(self.kt, M, self.Hkv, D, self.kvd, pos, 0, self.theta)
            rows = self.key_rows[s - 2]
            tk2, tv2 = self.tk.view(B * self.Tk, self.kvd), self.tv.view(B * self.Tk, self.kvd)
            B_.eagle3_copy_rows(self.kt, tk2, M, dst_rows=rows)
            B_.eagle3_copy_rows(self.vt, tv2, M, dst_rows=rows)
            a = B_.tree_attn_args(self.q.view(B, C, self.Hq, D), self.tk, self.tv, self.k_cache, self.v_cache,
                                  self.table, self.plen, self.attn.view(B, C, self.Hq, D), mask=fr["mask"])
            B_.eagle3_tree_attn(a, self._attn_ws(a))
            self._layer_tail(self.xs, self.attn, a_out, M)
            self._head(a_out, M)
            B_.eagle3_tree_expand(fr["score"], fr["pool"], fr["mask"], 0, C, self.ids.view(B, C, C),
                                  self.val.view(B, C, C), self.lse, pool_len, (s - 1) * C, self.pool_score,
                                  self.pool_token, self.pool_parent, nx["pool"], nx["score"], nx["token"],
                                  nx["mask"], nx["arow"])
            if record is not None:
                record.append(dict(ids=self.ids.view(B, C, C).clone(), val=self.val.view(B, C, C).clone(),
                                   lse=self.lse.view(B, C).clone(), next_pool=nx["pool"].clone(),
                                   pool_len=pool_len, a=a_out.clone()))
            pool_len += C * C
            a_src = a_out
        self.pool_len = pool_len
        B_.eagle3_tree_rerank(self.pool_score, self.pool_token, self.pool_parent, pool_len, self.root, self.parent,
                              self.tokens)
        return self.parent, self.tokens

    # ----------------------------------------------------------- extend
    def extend(self, l, m, h, path_rows, tok_ahead, start, last_rows):
        """New context rows after an acceptance (arguments as written by
        eagle3_spec_advance): for every sequence, R = extend_rows rows whose
        features are rows path_rows of the target's l, m, h [rows, k] and
        whose next tokens are tok_ahead; their K/V go to the cache at
        positions start.. (rows past the accepted ones land after the new
        length, where nothing reads them until the next extend overwrites
        them), and the full layer at row last_rows (the end node, at position
        prefix_len - 1 with prefix_len already advanced) gives a_root."""
        B, R, k = self.B, self.R, self.k
        Re = B * R
        e, w = self.ext, self.w
        for src, dst in ((l, e["l"]), (m, e["m"]), (h, e["h"])):
            B_.eagle3_copy_rows(src, dst, Re, src_rows=path_rows.view(-1))
        B_.eagle3_draft_fuse(tok_ahead.view(-1), w["embed"], w["w_in"], e["x"], w_fuse=w["w_fuse"], l=e["l"],
                             m=e["m"], h=e["h"], g_out=e["g"], ws=self._fws)
        B_.eagle3_rmsnorm(e["x"], e["hn"], eps=self.eps)
        self._gemm([e["hn"]], self.wk, e["k"])
        self._gemm([e["hn"]], self.wv, e["v"])
        B_.eagle3_node_positions(start, e["depth"], e["pos"].view(B, R))
        B_.eagle3_rope(e["k"], Re, self.Hkv, self.D, self.kvd, e["pos"], 0, self.theta)
        B_.eagle3_commit_kv(e["k"].view(B, R, self.Hkv, self.D), e["v"].view(B, R, self.Hkv, self.D), None, start,
                            self.k_cache, self.v_cache, self.table, max_n=R)
        B_.eagle3_copy_rows(e["x"], self.x1, B, src_rows=last_rows)
        h1, q, attn = self.hs[:B], self.q[:B], self.attn[:B]
        B_.eagle3_rmsnorm(self.x1, h1, eps=self.eps)
        self._gemm([h1], self.wq, q)
        B_.eagle3_node_positions(self.plen, e["minus1"], e["last_pos"].view(B, 1))
        B_.eagle3_rope(q, B, self.Hq, self.D, self.qd, e["last_pos"], 0, self.theta)
        none = self.tk[:, :0]
        a = B_.tree_attn_args(q.view(B, 1, self.Hq, self.D), none, none, self.k_cache, self.v_cache, self.table,
                              self.plen, attn.view(B, 1, self.Hq, self.D), mask=self.root_mask)
        B_.eagle3_tree_attn(a, self._attn_ws(a))
        self._layer_tail(self.x1, attn, self.a_root, B)

    def run(self, l, m, h, ctx_tok, record=None):
        self.ingest(l, m, h, ctx_tok)
        return self.grow(record)
