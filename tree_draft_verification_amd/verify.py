"""One tree-verify step on one stream: ancestor masks -> tree attention ->
RMSNorm -> LM-head argmax -> greedy acceptance.

This module only owns device buffers and enqueues the C-ABI calls in order
(course lesson "EAGLE-3 speculative decoding: the tree-verifier method":
one target pass over the whole tree, then the accept rule). For the verify
workloads the tree-attention output of a node, reshaped to [Hq * D], is the
hidden state that feeds the LM head (reading: Hq * D equals the hidden size).
"""
from __future__ import annotations

import torch

from . import binding as B_


class VerifyStep:
    def __init__(self, B, T, Hq, Hkv, D, V, k_cache, v_cache, block_table, prefix_len, w_lm,
                 dtype=torch.bfloat16, split_keys=0, eps=1e-5, device="cuda"):
        self.B, self.T, self.Hq, self.Hkv, self.D, self.V = B, T, Hq, Hkv, D, V
        self.K = Hq * D
        self.W = (T + 63) // 64
        self.eps = eps
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.mask = torch.empty((B, T, self.W), dtype=torch.int64, device=dev)  # uint64 bits
        self.depth = torch.empty((B, T), **i32)
        self.status = torch.empty((B,), **i32)
        self.attn = torch.empty((B, T, Hq, D), dtype=dtype, device=dev)
        self.hidden = torch.empty((B * T, self.K), dtype=dtype, device=dev)
        self.idx = torch.empty((B * T, 1), **i32)
        self.val = torch.empty((B * T, 1), dtype=torch.float32, device=dev)
        self.gap = torch.empty((B * T,), dtype=torch.float32, device=dev)
        self.accept_len = torch.empty((B,), **i32)
        self.path = torch.empty((B, T), **i32)
        self.out_tokens = torch.empty((B, T), **i32)
        self.k_cache, self.v_cache, self.block_table, self.prefix_len, self.w_lm = (
            k_cache, v_cache, block_table, prefix_len, w_lm)
        self.split_keys = split_keys
        dt = B_.BF16 if dtype == torch.bfloat16 else B_.F32
        self.lm_ws = torch.empty(max(256, B_.eagle3_lmhead_workspace(B * T, V, self.K, 1, dt)),
                                 dtype=torch.uint8, device=dev)
        self._attn_ws = None

    def _args(self, q, k_tree, v_tree):
        a = B_.tree_attn_args(q, k_tree, v_tree, self.k_cache, self.v_cache, self.block_table, self.prefix_len,
                              self.attn, mask=self.mask, split_keys=self.split_keys, norm_out=self.hidden,
                              norm_eps=self.eps)
        need = B_.eagle3_tree_attn_workspace(a)
        if self._attn_ws is None or self._attn_ws.numel() < need:
            self._attn_ws = torch.empty(max(256, need), dtype=torch.uint8, device=q.device)
        return a

    def forward(self, parent, q, k_tree, v_tree, stream=None, events=None):
        """Enqueue a0-a3 (mask, attention with the RMSNorm of its output rows,
        LM-head argmax). ``events``:
        optional {"attn": (start, end), "lmhead": (start, end)} HIP events
        recorded around those calls on the same stream."""
        ev = events or {}
        B_.eagle3_tree_mask(parent, self.W, self.mask, self.depth, self.status, stream=stream)
        a = self._args(q, k_tree, v_tree)
        self._record(ev, "attn", 0, stream)
        B_.eagle3_tree_attn(a, self._attn_ws, stream=stream)
        self._record(ev, "attn", 1, stream)
        self._record(ev, "lmhead", 0, stream)
        B_.eagle3_lmhead_argmax(self.hidden, self.w_lm, 1, self.idx, self.val, self.gap, None, self.lm_ws,
                                stream=stream)
        self._record(ev, "lmhead", 1, stream)

    @staticmethod
    def _record(ev, name, i, stream):
        if name in ev:
            ev[name][i].record(stream if stream is not None else torch.cuda.current_stream())

    def accept(self, tokens, stream=None):
        """Enqueue a4 (greedy acceptance) on the argmax of forward()."""
        B_.eagle3_accept_path(tokens, self.idx.view(self.B, self.T), self.accept_len, self.path, self.out_tokens,
                              mask=self.mask, stream=stream)

    def run(self, parent, q, k_tree, v_tree, tokens, stream=None, events=None):
        self.forward(parent, q, k_tree, v_tree, stream, events)
        self.accept(tokens, stream)

    def graph(self, parent, q, k_tree, v_tree, tokens):
        """Capture one whole step (mask, attention, norm, LM head, accept) in a
        HIP graph; replaying it re-runs the step on the same buffers. The graph
        holds no memset nodes (every kernel writes its outputs in full)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run(parent, q, k_tree, v_tree, tokens)   # sizes the workspaces outside the capture
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run(parent, q, k_tree, v_tree, tokens)
        return g

