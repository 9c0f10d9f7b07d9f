"""A small fp32 Llama-style decoder run entirely through libeagle3 calls, used
to show the lossless property of tree verification on the GPU (course lesson
"EAGLE-3 speculative decoding: the tree-verifier method", section
"Verify-accept semantics": accepting the drafts that equal the target's argmax
and appending the target's token reproduces the target's own autoregressive
output).

Every layer op (embedding, RMSNorm, the QKV/O/MLP GEMMs, RoPE at position
P + depth, tree attention over the paged cache, SiLU gating, LM-head argmax,
acceptance, KV commit) is a kernel of the library; this module owns the
buffers and the host loop (one device-to-host read per verify step).
reading: pre-norm layer, gamma = 1, rotate-half RoPE, untied embedding/head.
"""
from __future__ import annotations

import torch

from . import binding as B_


class ToyDecoderGPU:
    def __init__(self, weights: dict, layers: int, H: int, D: int, F: int, theta: float, eps: float,
                 max_pos: int = 512, device="cuda"):
        self.w = {k: v.to(device=device, dtype=torch.float32).contiguous() for k, v in weights.items()}
        self.layers, self.H, self.D, self.F, self.theta, self.eps = layers, H, D, F, theta, eps
        self.HD = H * D
        self.K = self.w["embed"].shape[1]
        self.V = self.w["embed"].shape[0]
        self.dev = torch.device(device)
        nblk = (max_pos + 15) // 16
        self.k_cache = [torch.zeros(nblk, H, 16, D, device=self.dev) for _ in range(layers)]
        self.v_cache = [torch.zeros(nblk, H, D, 16, device=self.dev) for _ in range(layers)]
        self.table = torch.arange(nblk, dtype=torch.int32, device=self.dev)[None]
        self.P = 0
        self.plen = torch.zeros(1, dtype=torch.int32, device=self.dev)
        self.gemm_w = {}
        for i in range(layers):
            wqkv = self.w[f"l{i}.wqkv"]
            self.gemm_w[i] = (wqkv[:self.HD], wqkv[self.HD:2 * self.HD], wqkv[2 * self.HD:])

    def _f32(self, *shape):
        return torch.empty(*shape, dtype=torch.float32, device=self.dev)

    def forward(self, tokens: torch.Tensor, parent: torch.Tensor):
        """Tree forward at positions P + depth. tokens, parent: int32 [T] on the
        device. Returns (argmax [T], top-2 gap [T], per-layer (k, v) rows, mask)."""
        T = tokens.shape[0]
        W = (T + 63) // 64
        i32 = dict(dtype=torch.int32, device=self.dev)
        mask = torch.empty(1, T, W, dtype=torch.int64, device=self.dev)
        depth = torch.empty(1, T, **i32)
        B_.eagle3_tree_mask(parent[None], W, mask, depth)
        x = self._f32(T, self.K)
        B_.eagle3_embed(self.w["embed"], tokens, x)
        rows = []
        for i in range(self.layers):
            h = self._f32(T, self.K)
            B_.eagle3_rmsnorm(x, h, eps=self.eps)
            wq, wk, wv = self.gemm_w[i]
            q, k, v = self._f32(T, self.HD), self._f32(T, self.HD), self._f32(T, self.HD)
            B_.eagle3_gemm([h], wq, q)
            B_.eagle3_gemm([h], wk, k)
            B_.eagle3_gemm([h], wv, v)
            B_.eagle3_rope(q, T, self.H, self.D, self.HD, depth, self.P, self.theta)
            B_.eagle3_rope(k, T, self.H, self.D, self.HD, depth, self.P, self.theta)
            attn = self._f32(T, self.HD)
            q4, k4, v4 = q.view(1, T, self.H, self.D), k.view(1, T, self.H, self.D), v.view(1, T, self.H, self.D)
            a = B_.tree_attn_args(q4, k4, v4, self.k_cache[i], self.v_cache[i], self.table, self.plen,
                                  attn.view(1, T, self.H, self.D), mask=mask)
            B_.eagle3_tree_attn(a, None, 0)
            B_.eagle3_gemm([attn], self.w[f"l{i}.wo"], x, residual=x)
            h2 = self._f32(T, self.K)
            B_.eagle3_rmsnorm(x, h2, eps=self.eps)
            gu = self._f32(T, 2 * self.F)
            B_.eagle3_gemm([h2], self.w[f"l{i}.wgu"], gu)
            f = self._f32(T, self.F)
            B_.eagle3_silu_mul(gu, f)
            B_.eagle3_gemm([f], self.w[f"l{i}.wd"], x, residual=x)
            rows.append((k4, v4))
        hf = self._f32(T, self.K)
        B_.eagle3_rmsnorm(x, hf, eps=self.eps)
        idx = torch.empty(T, 2, **i32)
        val = self._f32(T, 2)
        gap = self._f32(T)
        ws = torch.empty(B_.eagle3_lmhead_workspace(T, self.V, self.K, 2, B_.F32), dtype=torch.uint8, device=self.dev)
        B_.eagle3_lmhead_argmax(hf, self.w["lm_head"], 2, idx, val, gap, None, ws)
        return idx[:, 0].contiguous(), gap, rows, mask

    def commit(self, rows, path: torch.Tensor, n: int):
        """Append the K/V rows listed by path [1, T] (-1 terminated) at P.."""
        for i, (k4, v4) in enumerate(rows):
            B_.eagle3_commit_kv(k4, v4, path, self.plen, self.k_cache[i], self.v_cache[i], self.table)
        self.P += n
        self.plen.fill_(self.P)

    def prefill(self, prompt: torch.Tensor):
        T = prompt.shape[0]
        parent = torch.arange(-1, T - 1, dtype=torch.int32, device=self.dev)
        idx, gap, rows, _ = self.forward(prompt, parent)
        path = torch.arange(T, dtype=torch.int32, device=self.dev)[None]
        self.commit(rows, path, T)
        return int(idx[-1]), float(gap[-1])

    def greedy_step(self, token: int):
        tok = torch.tensor([token], dtype=torch.int32, device=self.dev)
        par = torch.tensor([-1], dtype=torch.int32, device=self.dev)
        idx, gap, rows, _ = self.forward(tok, par)
        self.commit(rows, torch.zeros(1, 1, dtype=torch.int32, device=self.dev), 1)
        return int(idx[0]), float(gap[0])

    def verify_step(self, tokens: torch.Tensor, parent: torch.Tensor):
        """One speculative step on a planted tree: forward, accept, commit the
        accepted path. Returns (accept_len, emitted tokens, argmax, gap) on the host."""
        T = tokens.shape[0]
        idx, gap, rows, mask = self.forward(tokens, parent)
        i32 = dict(dtype=torch.int32, device=self.dev)
        al, path, out = torch.empty(1, **i32), torch.empty(1, T, **i32), torch.empty(1, T, **i32)
        B_.eagle3_accept_path(tokens[None], idx[None], al, path, out, mask=mask)
        a = int(al[0])
        self.commit(rows, path, a + 1)
        return a, out[0, :a + 1].cpu().numpy(), idx.cpu().numpy(), gap.cpu().numpy()
