"""The target model's own pass over a batch of draft trees on the GPU: token
embedding, Llama decoder layers, final RMSNorm, LM-head argmax and greedy
acceptance, composed from libeagle3 calls (course lesson "EAGLE-3
speculative decoding: the tree-verifier method": the target runs once over
the whole tree with each token attending to the cached context and its
ancestors, then the accept rule).

Per layer, over M = B * T tree rows: RMSNorm -> Q and (one GEMM) K, V projections -> RoPE
at the sequence's cached length + the node's depth -> tree attention over
that layer's paged prefix plus the ancestor-masked tree rows -> output
projection + residual -> RMSNorm -> gate/up projection -> SiLU(gate) * up ->
down projection + residual (in bf16 the gate/up projection and the gating
are one call, eagle3_gemm_swiglu, on the weight in paired layout). The tree rows' K/V of every layer stay in
device buffers, so the accepted path can be appended to each layer's cache
(eagle3_commit_kv) after acceptance. readings: pre-norm layer with gamma = 1,
GQA (query head h reads KV head h / (Hq / Hkv)), rotate-half RoPE.

This module owns buffers and launch order only; every step is a kernel.
"""
from __future__ import annotations

import torch

from . import binding as B_


class TargetModel:
    def __init__(self, weights: dict, layers: int, B: int, T: int, Hq: int, Hkv: int, D: int,
                 k_caches, v_caches, block_table, prefix_len, theta: float = 500000.0, eps: float = 1e-5,
                 features=(), device="cuda"):
        self.dev = torch.device(device)
        self.w = weights
        E = weights["embed"]
        self.V, self.k = E.shape
        self.dtype = E.dtype
        if self.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("target weights must be bf16 or fp32")
        self.layers, self.B, self.T, self.Hq, self.Hkv, self.D = layers, B, T, Hq, Hkv, D
        self.theta, self.eps = theta, eps
        self.qd, self.kvd = Hq * D, Hkv * D
        self.F = weights["l0.wd"].shape[1]
        self.W = (T + 63) // 64
        if len(k_caches) != layers or len(v_caches) != layers:
            raise ValueError("one K and one V cache per layer")
        self.k_caches, self.v_caches, self.table, self.plen = k_caches, v_caches, block_table, prefix_len
        self.features = tuple(features)
        self.proj = []
        for i in range(layers):
            wqkv = weights[f"l{i}.wqkv"]
            # (Q rows, the adjacent K and V rows as one weight)
            self.proj.append((wqkv[:self.qd], wqkv[self.qd:]))
        # bf16: the gate/up weights in the paired layout of the fused
        # projection + gating call (one extra copy of those weights)
        self.fused_mlp = self.dtype == torch.bfloat16 and self.F % 128 == 0
        self.wgu_paired = []
        if self.fused_mlp:
            tab = B_.pair_gate_up_rows(self.F, self.dev)
            for i in range(layers):
                w = weights[f"l{i}.wgu"]
                wp = torch.empty_like(w)
                B_.eagle3_copy_rows(w, wp, 2 * self.F, src_rows=tab)
                self.wgu_paired.append(wp)
        M, dt, dv = B * T, self.dtype, self.dev
        i32 = dict(dtype=torch.int32, device=dv)
        e = lambda *s: torch.empty(*s, dtype=dt, device=dv)  # noqa: E731
        self.mask = torch.empty(B, T, self.W, dtype=torch.int64, device=dv)
        self.depth = torch.empty(B, T, **i32)
        self.pos = torch.empty(B, T, **i32)
        self.status = torch.empty(B, **i32)
        self.x, self.h = e(M, self.k), e(M, self.k)
        self.q, self.attn = e(M, self.qd), e(M, self.qd)
        self.gu, self.f = e(M, 2 * self.F), e(M, self.F)
        # K and V projections as one GEMM ([M, 2 kvd], each row K then V),
        # then each half gathered into its row buffer
        self.kv = e(M, 2 * self.kvd)
        self.k_src = torch.arange(0, 2 * M, 2, **i32)
        self.v_src = torch.arange(1, 2 * M, 2, **i32)
        # tree rows' K (after RoPE) and V of every layer, kept for the commit
        self.k_rows = [e(B, T, Hkv, D) for _ in range(layers)]
        self.v_rows = [e(B, T, Hkv, D) for _ in range(layers)]
        self.feat = {i: e(M, self.k) for i in self.features}
        self.hidden = e(M, self.k)
        self.idx = torch.empty(M, 1, **i32)
        self.val = torch.empty(M, 1, dtype=torch.float32, device=dv)
        self.gap = torch.empty(M, dtype=torch.float32, device=dv)
        self.accept_len = torch.empty(B, **i32)
        self.path = torch.empty(B, T, **i32)
        self.out_tokens = torch.empty(B, T, **i32)
        dtc = B_._dtype(E)
        self.lm_ws = torch.empty(max(256, B_.eagle3_lmhead_workspace(M, self.V, self.k, 1, dtc)),
                                 dtype=torch.uint8, device=dv)
        # K-split workspace of the projections when they have few output tiles,
        # also the tile counters of the persistent gate/up call
        need = max(B_.eagle3_gemm_workspace([self.h], self.proj[0][1], self.kv),
                   B_.eagle3_gemm_workspace([self.h], self.proj[0][0], self.q), B_.PERSIST_WS_BYTES)
        self.gemm_ws = torch.empty(need, dtype=torch.uint8, device=dv)
        self._attn_ws = None
        # optional: a list of (start, end) HIP event pairs per layer for the
        # gate/up GEMM and the attention, recorded in call order
        self.events = None

    def _ev(self, name, i, j):
        if self.events is not None:
            self.events[name][i][j].record()

    def _attn(self, i):
        B, T = self.B, self.T
        a = B_.tree_attn_args(self.q.view(B, T, self.Hq, self.D), self.k_rows[i], self.v_rows[i], self.k_caches[i],
                              self.v_caches[i], self.table, self.plen, self.attn.view(B, T, self.Hq, self.D),
                              mask=self.mask)
        need = B_.eagle3_tree_attn_workspace(a)
        if self._attn_ws is None or self._attn_ws.numel() < need:
            self._attn_ws = torch.empty(max(256, need), dtype=torch.uint8, device=self.dev)
        B_.eagle3_tree_attn(a, self._attn_ws)

    def forward(self, parent, tokens, record=None, layers=None):
        """Tree masks, positions, embedding, the decoder layers, final
        RMSNorm and LM-head argmax / top-2 gap over every node. parent,
        tokens: int32 [B, T] on the device. With a list as `record`, the
        input of every layer and the last layer's output are appended (device
        copies, [B, T, k]); `layers` runs only the first n layers."""
        B, T, M, D = self.B, self.T, self.B * self.T, self.D
        n_layers = self.layers if layers is None else layers
        B_.eagle3_tree_mask(parent, self.W, self.mask, self.depth, self.status)
        B_.eagle3_node_positions(self.plen, self.depth, self.pos)
        pos = self.pos.view(-1)
        B_.eagle3_embed(self.w["embed"], tokens.view(-1), self.x)
        ws = self.gemm_ws
        for i in range(n_layers):
            if record is not None:
                record.append(self.x.view(B, T, self.k).clone())
            wq, wkv = self.proj[i]
            kr, vr = self.k_rows[i].view(M, self.kvd), self.v_rows[i].view(M, self.kvd)
            B_.eagle3_rmsnorm(self.x, self.h, eps=self.eps)
            B_.eagle3_gemm([self.h], wq, self.q, ws=ws)
            B_.eagle3_gemm([self.h], wkv, self.kv, ws=ws)
            kv2 = self.kv.view(2 * M, self.kvd)
            B_.eagle3_copy_rows(kv2, kr, M, src_rows=self.k_src)
            B_.eagle3_copy_rows(kv2, vr, M, src_rows=self.v_src)
            B_.eagle3_rope(self.q, M, self.Hq, D, self.qd, pos, 0, self.theta)
            B_.eagle3_rope(kr, M, self.Hkv, D, self.kvd, pos, 0, self.theta)
            self._ev("attn", i, 0)
            self._attn(i)
            self._ev("attn", i, 1)
            B_.eagle3_gemm([self.attn], self.w[f"l{i}.wo"], self.x, residual=self.x, ws=ws)
            B_.eagle3_rmsnorm(self.x, self.h, eps=self.eps)
            self._ev("gu", i, 0)
            if self.fused_mlp:
                B_.eagle3_gemm_swiglu([self.h], self.wgu_paired[i], self.f, ws=ws)
            else:
                B_.eagle3_gemm([self.h], self.w[f"l{i}.wgu"], self.gu, ws=ws)
            self._ev("gu", i, 1)
            if not self.fused_mlp:
                B_.eagle3_silu_mul(self.gu, self.f)
            B_.eagle3_gemm([self.f], self.w[f"l{i}.wd"], self.x, residual=self.x, ws=ws)
            if i in self.feat:
                B_.eagle3_copy_rows(self.x, self.feat[i], M)
        if record is not None:
            record.append(self.x.view(B, T, self.k).clone())
        B_.eagle3_rmsnorm(self.x, self.hidden, eps=self.eps)
        B_.eagle3_lmhead_argmax(self.hidden, self.w["lm_head"], 1, self.idx, self.val, self.gap, None, self.lm_ws)

    def accept(self, tokens):
        B_.eagle3_accept_path(tokens, self.idx.view(self.B, self.T), self.accept_len, self.path, self.out_tokens,
                              mask=self.mask)

    def run(self, parent, tokens, record=None):
        self.forward(parent, tokens, record)
        self.accept(tokens)

    def commit(self, start=None):
        """Append the accepted path's K/V rows of every layer to that layer's
        cache at positions start.. (default: prefix_len, which the caller
        then advances)."""
        st = self.plen if start is None else start
        for i in range(self.layers):
            B_.eagle3_commit_kv(self.k_rows[i], self.v_rows[i], self.path, st, self.k_caches[i],
                                self.v_caches[i], self.table)
