"""ctypes binding of libeagle3.so: one Python function per C entry point,
same names, argument marshalling only (torch tensors -> device pointers,
the current torch stream -> hipStream_t). Every computation runs in the HIP
kernels; when the library is missing this module raises at import.
Structures built here (TreeAttnArgs) hold raw device pointers: the caller
keeps the tensors alive until the enqueued work has finished.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libeagle3.so")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_TREE, ERR_RANGE, ERR_HIP, ERR_WORKSPACE = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python tree_draft_verification_amd/build.py` "
                      "(there is no fallback path)")
_lib = ctypes.CDLL(LIB_PATH)

P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class TreeAttnArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", I), ("B", I), ("Tq", I), ("Tk", I), ("Hq", I), ("Hkv", I), ("D", I), ("W", I),
        ("scale", F),
        ("q", P), ("k_tree", P), ("v_tree", P), ("k_cache", P), ("v_cache", P),
        ("num_blocks", I), ("block_size", I),
        ("block_table", P), ("max_blocks", I), ("prefix_len", P),
        ("mask", P), ("parent", P), ("out", P), ("lse", P),
        ("split_keys", I),
        ("norm_out", P), ("norm_eps", F),
        ("status", P),
    ]


class GemmArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", I), ("M", I), ("N", I), ("nseg", I),
        ("a", P * 3), ("a_rows", P * 3), ("a_nrows", I * 3), ("k", I * 3),
        ("b", P), ("residual", P), ("c", P), ("ldc", I), ("ws", P), ("ws_bytes", SZ),
    ]


def _sig(name, res, *args):
    fn = getattr(_lib, name)
    fn.restype = res
    fn.argtypes = list(args)
    return fn


_status_string = _sig("eagle3_status_string", ctypes.c_char_p, I)
_abi_version = _sig("eagle3_abi_version", I)
_tree_mask = _sig("eagle3_tree_mask", I, P, I, I, I, P, P, P, P)
_tree_attn_ws = _sig("eagle3_tree_attn_workspace", SZ, ctypes.POINTER(TreeAttnArgs))
_tree_attn = _sig("eagle3_tree_attn", I, ctypes.POINTER(TreeAttnArgs), P, SZ, P)
_rmsnorm = _sig("eagle3_rmsnorm", I, P, P, I, I, F, I, P, P)
_lmhead_ws = _sig("eagle3_lmhead_workspace", SZ, I, I, I, I, I)
_lmhead = _sig("eagle3_lmhead_argmax", I, P, P, I, I, I, I, I, P, P, P, P, P, SZ, P)
_lmhead_noalloc = _sig("eagle3_lmhead_argmax_noalloc", I, P, P, I, I, I, I, I, P, P, P, P, P)
_accept = _sig("eagle3_accept_path", I, P, P, P, I, P, I, I, P, P, P, I, P, P)
_gemm = _sig("eagle3_gemm", I, ctypes.POINTER(GemmArgs), P)
_gemm_swiglu = _sig("eagle3_gemm_swiglu", I, ctypes.POINTER(GemmArgs), P)
_gemm_ws = _sig("eagle3_gemm_workspace", SZ, ctypes.POINTER(GemmArgs))
_silu_mul = _sig("eagle3_silu_mul", I, P, I, I, I, P, P)
_rope = _sig("eagle3_rope", I, P, I, I, I, I, P, I, F, I, P)
_embed = _sig("eagle3_embed", I, P, P, I, I, I, I, P, P)
_commit_kv = _sig("eagle3_commit_kv", I, P, P, I, P, I, I, I, I, I, P, P, P, I, I, P, P)
_copy_rows = _sig("eagle3_copy_rows", I, P, P, I, P, P, I, I, SZ, P)
_vocab_map = _sig("eagle3_vocab_map", I, P, I, P, I, P, P, P)
_node_pos = _sig("eagle3_node_positions", I, P, P, I, I, P, P)
_spec_adv = _sig("eagle3_spec_advance", I, P, P, P, I, I, I, P, P, P, P, P, P, P, P, I, P)
_draft_fuse_ws = _sig("eagle3_draft_fuse_workspace", SZ, I, I, I)
_draft_fuse = _sig("eagle3_draft_fuse", I, P, P, P, P, P, P, P, P, I, I, I, I, P, P, P, SZ, P)
_tree_expand = _sig("eagle3_tree_expand", I, P, P, P, I, I, P, P, P, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P)
_tree_rerank = _sig("eagle3_tree_rerank", I, P, P, P, I, I, I, I, P, P, P, P)


class Eagle3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {eagle3_status_string(status)} ({status})")
        self.status = status


def _check(rc: int, where: str):
    if rc != OK:
        raise Eagle3Error(rc, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def eagle3_status_string(status: int) -> str:
    return _status_string(status).decode()


def eagle3_abi_version() -> int:
    return _abi_version()


def eagle3_tree_mask(parent, W, mask, depth=None, status=None, stream=None):
    B, T = parent.shape
    _check(_tree_mask(_ptr(parent), B, T, W, _ptr(mask), _ptr(depth), _ptr(status), _stream(stream)),
           "eagle3_tree_mask")


def tree_attn_args(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, out, mask=None, parent=None,
                   lse=None, scale=None, split_keys=0, norm_out=None, norm_eps=1e-5, status=None) -> TreeAttnArgs:
    B, Tq, Hq, D = q.shape
    Tk, Hkv = k_tree.shape[1], k_tree.shape[2]
    W = mask.shape[-1] if mask is not None else (Tq + 63) // 64
    a = TreeAttnArgs()
    a.dtype = _dtype(q)
    a.B, a.Tq, a.Tk, a.Hq, a.Hkv, a.D, a.W = B, Tq, Tk, Hq, Hkv, D, W
    a.scale = float(scale if scale is not None else D ** -0.5)
    a.q, a.k_tree, a.v_tree = _ptr(q), _ptr(k_tree), _ptr(v_tree)
    a.k_cache, a.v_cache = _ptr(k_cache), _ptr(v_cache)
    a.num_blocks, a.block_size = k_cache.shape[0], k_cache.shape[2]
    a.block_table, a.max_blocks, a.prefix_len = _ptr(block_table), block_table.shape[1], _ptr(prefix_len)
    a.mask, a.parent, a.out, a.lse = _ptr(mask), _ptr(parent), _ptr(out), _ptr(lse)
    a.split_keys = int(split_keys)
    a.norm_out, a.norm_eps = _ptr(norm_out), float(norm_eps)
    a.status = _ptr(status)
    return a


def eagle3_tree_attn_workspace(args: TreeAttnArgs) -> int:
    return int(_tree_attn_ws(ctypes.byref(args)))


def eagle3_tree_attn(args: TreeAttnArgs, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(_tree_attn(ctypes.byref(args), _ptr(ws), ws_bytes, _stream(stream)), "eagle3_tree_attn")


def eagle3_rmsnorm(x, y, gamma=None, eps=1e-5, stream=None):
    K = x.shape[-1]
    M = x.numel() // K
    _check(_rmsnorm(_ptr(x), _ptr(gamma), M, K, float(eps), _dtype(x), _ptr(y), _stream(stream)), "eagle3_rmsnorm")


def eagle3_lmhead_workspace(M, N, K, topk, dtype) -> int:
    return int(_lmhead_ws(M, N, K, topk, dtype))


def eagle3_lmhead_argmax(hidden, w, topk, idx, val=None, gap=None, lse=None, ws=None, stream=None):
    K = hidden.shape[-1]
    M = hidden.numel() // K
    N = w.shape[0]
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lmhead(_ptr(hidden), _ptr(w), M, N, K, topk, _dtype(hidden), _ptr(idx), _ptr(val), _ptr(gap), _ptr(lse),
                   _ptr(ws), ws_bytes, _stream(stream)), "eagle3_lmhead_argmax")


def eagle3_lmhead_argmax_noalloc(hidden, w, topk, idx, val=None, gap=None, lse=None, stream=None):
    K = hidden.shape[-1]
    M = hidden.numel() // K
    N = w.shape[0]
    _check(_lmhead_noalloc(_ptr(hidden), _ptr(w), M, N, K, topk, _dtype(hidden), _ptr(idx), _ptr(val), _ptr(gap),
                           _ptr(lse), _stream(stream)), "eagle3_lmhead_argmax_noalloc")


def eagle3_accept_path(tokens, target_idx, accept_len, path, out_tokens, parent=None, mask=None, V=0, status=None,
                       stream=None):
    B, T = tokens.shape
    W = mask.shape[-1] if mask is not None else (T + 63) // 64
    _check(_accept(_ptr(tokens), _ptr(parent), _ptr(mask), W, _ptr(target_idx), B, T, _ptr(accept_len), _ptr(path),
                   _ptr(out_tokens), int(V), _ptr(status), _stream(stream)), "eagle3_accept_path")


def _gemm_args(a, b, c, residual, a_rows, ldc, M, ws):
    a = list(a)
    g = GemmArgs()
    g.dtype = _dtype(b)
    g.M = int(M if M is not None else c.shape[0])
    g.N = int(b.shape[0])
    g.nseg = len(a)
    rows = list(a_rows) if a_rows is not None else [None] * len(a)
    for i, t in enumerate(a):
        g.a[i] = _ptr(t)
        g.k[i] = int(t.shape[-1])
        g.a_rows[i] = _ptr(rows[i])
        g.a_nrows[i] = int(t.shape[0]) if rows[i] is not None else 0
    g.b, g.residual, g.c, g.ldc = _ptr(b), _ptr(residual), _ptr(c), int(ldc)
    g.ws = _ptr(ws)
    g.ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    return g


def eagle3_gemm_workspace(a, b, c, M=None, residual=None, a_rows=None) -> int:
    """Bytes of workspace eagle3_gemm would use for this call: to split K, or
    PERSIST_WS_BYTES for the tile counters of its persistent form."""
    return int(_gemm_ws(ctypes.byref(_gemm_args(a, b, c, residual, a_rows, 0, M, None))))


def eagle3_gemm(a, b, c, residual=None, a_rows=None, a_nrows=None, ldc=0, M=None, stream=None, ws=None):
    """C = [a_0 | a_1 | ...] . b^T (+ residual); a: list of [rows, k_s] tensors
    (a_rows[s]: optional int32 row gather of segment s; ws: optional workspace
    that lets a call with few output tiles split K, or a large one run
    persistent work-groups: eagle3_gemm_workspace gives the bytes)."""
    g = _gemm_args(a, b, c, residual, a_rows, ldc, M, ws)
    _check(_gemm(ctypes.byref(g), _stream(stream)), "eagle3_gemm")


PERSIST_WS_BYTES = 1024  # EAGLE3_PERSIST_WS_BYTES


def eagle3_gemm_swiglu(a, b, y, a_rows=None, ldc=0, M=None, stream=None, ws=None):
    """y = silu(A . Wg^T) * (A . Wu^T) with b the gate/up weight in paired
    layout (see pair_gate_up_rows); y [M, N / 2]. ws (optional, at least
    PERSIST_WS_BYTES): room for the tile counters of the persistent path."""
    g = _gemm_args(a, b, y, None, a_rows, ldc, M if M is not None else y.shape[0], ws)
    _check(_gemm_swiglu(ctypes.byref(g), _stream(stream)), "eagle3_gemm_swiglu")


def pair_gate_up_rows(F, device):
    """int32 row table that eagle3_copy_rows uses to turn [Wg; Wu] ([2F, K],
    gate rows first) into the paired layout of eagle3_gemm_swiglu: row r of
    the result is gate row 128 (r / 256) + r % 256 for r % 256 < 128, else up
    row 128 (r / 256) + r % 256 - 128."""
    if F % 128:
        raise ValueError("the paired gate/up layout needs F % 128 == 0")
    r = torch.arange(2 * F)
    j, q = r // 256, r % 256
    src = torch.where(q < 128, 128 * j + q, F + 128 * j + q - 128)
    return src.to(device=device, dtype=torch.int32)


def eagle3_silu_mul(gu, y, stream=None):
    M, F = y.shape[0], y.shape[-1]
    _check(_silu_mul(_ptr(gu), M, F, _dtype(gu), _ptr(y), _stream(stream)), "eagle3_silu_mul")


def eagle3_rope(x, M, H, D, ld, pos, pos_offset, theta, stream=None):
    _check(_rope(_ptr(x), M, H, D, ld, _ptr(pos), int(pos_offset), float(theta), _dtype(x), _stream(stream)),
           "eagle3_rope")


def eagle3_embed(E, ids, out, stream=None):
    M, K, V = ids.shape[0], E.shape[1], E.shape[0]
    _check(_embed(_ptr(E), _ptr(ids), M, K, V, _dtype(E), _ptr(out), _stream(stream)), "eagle3_embed")


def eagle3_copy_rows(src, dst, n, src_rows=None, dst_rows=None, stream=None):
    """dst[dst_rows[i]] = src[src_rows[i]] for i < n (rows = first dimension)."""
    rb = src[0].numel() * src.element_size()
    if dst[0].numel() * dst.element_size() != rb:
        raise ValueError("row sizes differ")
    _check(_copy_rows(_ptr(src), _ptr(src_rows), src.shape[0], _ptr(dst), _ptr(dst_rows), dst.shape[0], int(n), rb,
                      _stream(stream)), "eagle3_copy_rows")


def eagle3_node_positions(prefix_len, depth, pos, stream=None):
    """pos[b, t] = prefix_len[b] + depth[b, t]; depth, pos [B, T] int32."""
    B, T = depth.shape
    _check(_node_pos(_ptr(prefix_len), _ptr(depth), B, T, _ptr(pos), _stream(stream)), "eagle3_node_positions")


def eagle3_spec_advance(accept_len, path, out_tokens, prefix_len, start, path_rows, tok_ahead, last_rows, root,
                        out_seq=None, out_len=None, stream=None):
    """Bookkeeping after acceptance: path_rows, tok_ahead [B, R]; the rest [B]."""
    B, T = path.shape
    R = path_rows.shape[-1]
    cap = out_seq.shape[-1] if out_seq is not None else 0
    _check(_spec_adv(_ptr(accept_len), _ptr(path), _ptr(out_tokens), B, T, R, _ptr(prefix_len), _ptr(start),
                     _ptr(path_rows), _ptr(tok_ahead), _ptr(last_rows), _ptr(root), _ptr(out_seq), _ptr(out_len), cap,
                     _stream(stream)), "eagle3_spec_advance")


def eagle3_vocab_map(ids, vmap, out=None, status=None, stream=None):
    """out[i] = vmap[ids[i]] over every element of ids (out defaults to ids:
    in place); -1 for an id outside [0, len(vmap))."""
    out = ids if out is None else out
    if out.numel() != ids.numel():
        raise ValueError("ids and out differ in size")
    _check(_vocab_map(_ptr(ids), ids.numel(), _ptr(vmap), vmap.numel(), _ptr(out), _ptr(status), _stream(stream)),
           "eagle3_vocab_map")


def eagle3_commit_kv(k_rows, v_rows, src, start, k_cache, v_cache, block_table, max_n=None, stream=None):
    """k_rows/v_rows [B, rows, Hkv, D]; src [B, max_n] int32 (-1 ends a list),
    or None for rows 0..max_n-1."""
    B, rows, Hkv, D = k_rows.shape
    max_n = src.shape[1] if src is not None else int(max_n if max_n is not None else rows)
    _check(_commit_kv(_ptr(k_rows), _ptr(v_rows), rows, _ptr(src), max_n, B, Hkv, D, _dtype(k_rows),
                      _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1], k_cache.shape[0],
                      _ptr(start), _stream(stream)), "eagle3_commit_kv")


def eagle3_draft_fuse_workspace(M, k, dtype) -> int:
    return int(_draft_fuse_ws(M, k, dtype))


def eagle3_draft_fuse(tok, E, w_in, x_out, w_fuse=None, l=None, m=None, h=None, a_prev=None, g_out=None, ws=None,
                      stream=None):
    M, k, V = tok.shape[0], E.shape[1], E.shape[0]
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_draft_fuse(_ptr(l), _ptr(m), _ptr(h), _ptr(a_prev), _ptr(tok), _ptr(E), _ptr(w_fuse), _ptr(w_in), M, k,
                       V, _dtype(E), _ptr(g_out), _ptr(x_out), _ptr(ws), ws_bytes, _stream(stream)),
           "eagle3_draft_fuse")


def eagle3_tree_expand(fr_score, fr_pool, fr_mask, fr_arow_base, arow_stride, child_ids, child_val, child_lse,
                       pool_len, row_base, pool_score, pool_token, pool_parent, next_pool, next_score, next_token,
                       next_mask, next_arow, stream=None):
    B, F, C = child_ids.shape
    NF = next_pool.shape[1]
    _check(_tree_expand(_ptr(fr_score), _ptr(fr_pool), _ptr(fr_mask), int(fr_arow_base), int(arow_stride),
                        _ptr(child_ids), _ptr(child_val), _ptr(child_lse), B, F, C, NF, int(pool_len),
                        pool_score.shape[1], int(row_base), _ptr(pool_score), _ptr(pool_token), _ptr(pool_parent),
                        _ptr(next_pool), _ptr(next_score), _ptr(next_token), _ptr(next_mask), _ptr(next_arow),
                        _stream(stream)), "eagle3_tree_expand")


def eagle3_tree_rerank(pool_score, pool_token, pool_parent, pool_len, root_token, parent, tokens, stream=None):
    B, cap = pool_score.shape
    N = parent.shape[1] - 1
    _check(_tree_rerank(_ptr(pool_score), _ptr(pool_token), _ptr(pool_parent), B, int(pool_len), cap, N,
                        _ptr(root_token), _ptr(parent), _ptr(tokens), _stream(stream)), "eagle3_tree_rerank")


def exported_symbols():
    """Names this binding resolved from the library (for load checks)."""
    return sorted(n for n in dir(_lib) if n.startswith("eagle3_"))
