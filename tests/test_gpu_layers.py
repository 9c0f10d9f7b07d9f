"""GPU parity of the dense layers (GEMM with segmented / gathered A, SiLU
gating, the fused gate/up projection + gating, RoPE, embedding gather, KV
commit) and of the EAGLE-3 draft fusion,
against the oracle on the same inputs. bf16 normwise <= 2e-2, fp32 <= 1e-5;
copies bit-exact."""
import numpy as np
import pytest
import torch

import synth
from _gpu import as_f64, dev, host, normwise_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import tree_draft_verification_amd as t
    return t


def _bf16_ulp(x16):
    """one unit in the last place of each bf16 value (bit patterns)"""
    e = (x16.astype(np.int32) >> 7) & 0xFF
    return np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)


# (4000, 4100, ...) fills the chip with 256-row tiles and leaves ragged M and N tails;
# with a workspace, (640, 4096, ...) splits K in 3 across segment boundaries and
# (64, 1000, ...) in 8 with a ragged N tile
@pytest.mark.parametrize("M,N,k,split", [(1, 128, [64], False), (200, 300, [128, 64, 192], False),
                                         (640, 256, [256, 128], False), (4000, 4100, [128, 64, 64], False),
                                         (640, 4096, [1024, 512, 512], True), (64, 1000, [4096, 4096], True)])
def test_gemm_bf16_segments_and_gather(orc, lib, M, N, k, split):
    rng = np.random.default_rng(M + N)
    segs = [synth.normal_bf16(rng, (M if s != 1 else 50, ks)) for s, ks in enumerate(k)]
    rows = [None] * len(k)
    if len(k) > 1:
        rows[1] = rng.integers(0, 50, size=M).astype(np.int32)     # gathered segment (an embedding table)
    B = synth.normal_bf16(rng, (N, sum(k)), 0.05)
    R = synth.normal_bf16(rng, (M, N))
    A = np.concatenate([s if r is None else s[r] for s, r in zip(segs, rows)], axis=1)
    ref = orc.gemm(A, B, R)
    sd = [dev(s) for s in segs]
    rd = [None if r is None else dev(r) for r in rows]
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Bd, Rd = dev(B), dev(R)
    ws = None
    if split:
        need = lib.eagle3_gemm_workspace(sd, Bd, c)
        assert need > 0
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    lib.eagle3_gemm(sd, Bd, c, residual=Rd, a_rows=rd, ws=ws)
    torch.cuda.synchronize()
    got = host(c)
    rel, mx = normwise_rel(got, ref)
    assert rel <= 2e-2, (rel, mx)
    # fp32 accumulation vs fp64: the stored bf16 values agree, or differ by one
    # unit where the exact value sits next to a rounding boundary
    d = np.abs(as_f64(got) - as_f64(ref))
    ulp = np.maximum(_bf16_ulp(ref), _bf16_ulp(got))
    # plus the fp32 accumulation error, which scales with the summands
    # (where the result cancels, one unit of the result is smaller than that)
    S = np.abs(as_f64(A)) @ np.abs(as_f64(B)).T + np.abs(as_f64(R))
    bad = d > ulp * 1.0001 + 4e-6 * S
    assert not bad.any(), (int(bad.sum()), d[bad][:5], as_f64(ref)[bad][:5], np.argwhere(bad)[:5])
    assert (got == ref).mean() >= 0.98, (got == ref).mean()


def test_gemm_split_k_in_place_residual(orc, lib):
    """Split-K path with the residual aliasing the output (x += A . B^T), as
    the draft layer's O and down projections do; the split result stays within
    the unsplit path's bound of it."""
    rng = np.random.default_rng(9)
    M, N, K = 640, 4096, 4096
    A, B, X = synth.normal_bf16(rng, (M, K)), synth.normal_bf16(rng, (N, K), 0.02), synth.normal_bf16(rng, (M, N))
    ref = orc.gemm(A, B, X)
    Ad, Bd = dev(A), dev(B)
    x = dev(X)
    x0 = dev(X)
    need = lib.eagle3_gemm_workspace([Ad], Bd, x)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    lib.eagle3_gemm([Ad], Bd, x, residual=x, ws=ws)
    lib.eagle3_gemm([Ad], Bd, x0, residual=x0)
    torch.cuda.synchronize()
    got, unsplit = host(x), host(x0)
    rel, mx = normwise_rel(got, ref)
    assert rel <= 2e-2, (rel, mx)
    d = np.abs(as_f64(got) - as_f64(ref))
    S = np.abs(as_f64(A)) @ np.abs(as_f64(B)).T + np.abs(as_f64(X))
    bad = d > np.maximum(_bf16_ulp(ref), _bf16_ulp(got)) * 1.0001 + 4e-6 * S
    assert not bad.any(), int(bad.sum())
    assert (got == unsplit).mean() >= 0.98


# Persistent 256-row tiles (a workspace of at least PERSIST_WS_BYTES, one A
# segment, at least four tiles per CU or one; 256 CUs): (8000, 8200, ...) has
# 1056 tiles with a ragged N tile and a last row tile whose upper half lies
# past M; (16384, 4096, ...) exactly 1024; (3904, 4096, ...) 256, one per
# work-group, with a last row tile of 64 rows; K from the 4-chunk minimum up.
@pytest.mark.parametrize("M,N,k,res", [(8000, 8200, [256], "separate"), (16384, 4096, [128], None),
                                       (8000, 8200, [192], "in_place"), (3904, 4096, [512], "separate")])
def test_gemm_persistent_matches_plain_and_oracle(orc, lib, M, N, k, res):
    rng = np.random.default_rng(7 * M + N + len(k))
    segs = [synth.normal_bf16(rng, (M, ks)) for ks in k]
    B = synth.normal_bf16(rng, (N, sum(k)), 0.05)
    R = synth.normal_bf16(rng, (M, N)) if res else None
    A = np.concatenate(segs, axis=1)
    ref = orc.gemm(A, B, R)
    sd = [dev(s) for s in segs]
    Bd = dev(B)
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    assert lib.eagle3_gemm_workspace(sd, Bd, c) == lib.PERSIST_WS_BYTES
    ws = torch.full((lib.PERSIST_WS_BYTES,), 0xA5, dtype=torch.uint8, device="cuda")
    plain = torch.empty_like(c)
    if res == "in_place":
        c.copy_(dev(R))
        plain.copy_(dev(R))
        lib.eagle3_gemm(sd, Bd, c, residual=c, ws=ws)
        lib.eagle3_gemm(sd, Bd, plain, residual=plain)
    else:
        Rd = dev(R) if res else None
        lib.eagle3_gemm(sd, Bd, c, residual=Rd, ws=ws)
        lib.eagle3_gemm(sd, Bd, plain, residual=Rd)
    torch.cuda.synchronize()
    got = host(c)
    assert np.array_equal(got, host(plain))            # the per-tile kernel's arithmetic
    rel, mx = normwise_rel(got, ref)
    assert rel <= 2e-2, (rel, mx)
    d = np.abs(as_f64(got) - as_f64(ref))
    S = np.abs(as_f64(A)) @ np.abs(as_f64(B)).T + (np.abs(as_f64(R)) if res else 0.0)
    bad = d > np.maximum(_bf16_ulp(ref), _bf16_ulp(got)) * 1.0001 + 4e-6 * S
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5])
    # the same workspace again for the first 7950 rows (still persistent, a
    # last tile of 14 rows; every counter zeroed anew) on a zeroed output:
    # rows past them stay untouched
    if M == 8000 and res != "in_place":
        M2 = 7950
        c2 = torch.zeros_like(c)
        assert lib.eagle3_gemm_workspace([s[:M2] for s in sd], Bd, c2, M=M2) == lib.PERSIST_WS_BYTES
        lib.eagle3_gemm([s[:M2] for s in sd], Bd, c2, residual=dev(R)[:M2] if res else None, M=M2, ws=ws)
        torch.cuda.synchronize()
        g2 = host(c2)
        assert np.array_equal(g2[:M2], got[:M2])
        assert not g2[M2:].view(np.uint16).any()


def test_gemm_persistent_taken_only_where_it_applies(lib):
    """Workspace query: the tile counters for one plain A segment with at
    least four 256 x 256 tiles per CU or one; 0 with a row gather, several
    segments or two tiles per CU (per-tile kernels)."""
    assert torch.cuda.get_device_properties(0).multi_processor_count == 256
    M, N, k = 8000, 8192, 256
    bf = dict(dtype=torch.bfloat16, device="cuda")
    a = [torch.empty(M, k, **bf), torch.empty(50, k, **bf)]
    rows = [None, torch.zeros(M, dtype=torch.int32, device="cuda")]
    b = torch.empty(N, 2 * k, **bf)
    c = torch.empty(M, N, **bf)
    assert lib.eagle3_gemm_workspace(a[:1], b[:, :k].contiguous(), c) == lib.PERSIST_WS_BYTES
    assert lib.eagle3_gemm_workspace(a, b, c, a_rows=rows) == 0
    assert lib.eagle3_gemm_workspace([a[0], a[0]], b, c) == 0
    assert lib.eagle3_gemm_workspace(a[:1], torch.empty(4096, k, **bf), c[:3904, :4096], M=3904) == \
        lib.PERSIST_WS_BYTES
    assert lib.eagle3_gemm_workspace(a[:1], torch.empty(4096, k, **bf), c[:, :4096]) == 0   # 512 tiles


def test_gemm_f32_and_in_place_residual(orc, lib):
    rng = np.random.default_rng(3)
    M, N, K = 37, 90, 70
    A, B, X = synth.normal_f32(rng, (M, K)), synth.normal_f32(rng, (N, K), 0.1), synth.normal_f32(rng, (M, N))
    ref = orc.gemm(A, B, X)
    x = dev(X)
    Ad, Bd = dev(A), dev(B)
    lib.eagle3_gemm([Ad], Bd, x, residual=x)
    torch.cuda.synchronize()
    rel, _ = normwise_rel(host(x), ref)
    assert rel <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_silu_mul(orc, lib, dtype):
    rng = np.random.default_rng(4)
    GU = synth.normal_f32(rng, (33, 2 * 100), 2.0)
    if dtype == "bf16":
        GU = synth.f32_to_bf16(GU)
    ref = orc.silu_mul(GU)
    gu = dev(GU)
    y = torch.empty(33, 100, dtype=gu.dtype, device="cuda")
    lib.eagle3_silu_mul(gu, y)
    torch.cuda.synchronize()
    rel, _ = normwise_rel(host(y), ref)
    assert rel <= (2e-2 if dtype == "bf16" else 1e-5)


# (1000, 32768, [128]) with a workspace: 4 x 256 tiles of 256 x 256, so the
# persistent path runs (one work-group per CU, several tiles each; the last
# row tile holds 232 rows); (300, 16384, [256]): one tile per work-group, the
# upper half of the last row tile past M
@pytest.mark.parametrize("M,F,k,ws", [(1, 128, [64], False), (200, 256, [128, 64, 192], False),
                                      (1000, 384, [256], False), (640, 512, [4096], False),
                                      (1000, 32768, [128], True), (1000, 32768, [128], False),
                                      (300, 16384, [256], True)])
def test_gemm_swiglu_fused(orc, lib, M, F, k, ws):
    """The fused gate/up projection + gating against the oracle's
    silu_mul(gemm(A, [Wg; Wu])), and bit for bit against the two separate
    calls on the GPU (the weight turned into the paired layout by
    eagle3_copy_rows)."""
    rng = np.random.default_rng(M + F)
    segs = [synth.normal_bf16(rng, (M if s != 1 else 50, ks)) for s, ks in enumerate(k)]
    rows = [None] * len(k)
    if len(k) > 1:
        rows[1] = rng.integers(0, 50, size=M).astype(np.int32)
    Wgu = synth.normal_bf16(rng, (2 * F, sum(k)), 0.05)
    A = np.concatenate([s if r is None else s[r] for s, r in zip(segs, rows)], axis=1)
    ref = orc.silu_mul(orc.gemm(A, Wgu))
    sd = [dev(s) for s in segs]
    rd = [None if r is None else dev(r) for r in rows]
    w = dev(Wgu)
    wp = torch.empty_like(w)
    lib.eagle3_copy_rows(w, wp, 2 * F, src_rows=lib.pair_gate_up_rows(F, "cuda"))
    y = torch.full((M, F), 3.0, dtype=torch.bfloat16, device="cuda")
    wsb = torch.full((lib.PERSIST_WS_BYTES,), 0xAB, dtype=torch.uint8, device="cuda") if ws else None
    lib.eagle3_gemm_swiglu(sd, wp, y, a_rows=rd, ws=wsb)
    gu = torch.empty(M, 2 * F, dtype=torch.bfloat16, device="cuda")
    lib.eagle3_gemm(sd, w, gu, a_rows=rd)
    y2 = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
    lib.eagle3_silu_mul(gu, y2)
    torch.cuda.synchronize()
    assert normwise_rel(host(y), ref)[0] <= 2e-2
    assert np.array_equal(host(y), host(y2))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_with_offset_and_stride(orc, lib, dtype):
    rng = np.random.default_rng(5)
    M, H, D, theta, off = 9, 4, 64, 500000.0, 1000
    X = synth.normal_f32(rng, (M, 3 * H * D))          # rows of a fused QKV output
    if dtype == "bf16":
        X = synth.f32_to_bf16(X)
    depth = rng.integers(0, 8, size=M).astype(np.int32)
    ref = orc.rope(X[:, H * D:2 * H * D].reshape(M, H, D), depth + off, theta)   # the k part
    x = dev(X)
    dd = dev(depth)
    lib.eagle3_rope(x[:, H * D:], M, H, D, 3 * H * D, dd, off, theta)
    torch.cuda.synchronize()
    got = host(x)
    rel, _ = normwise_rel(got[:, H * D:2 * H * D].reshape(M, H, D), ref)
    assert rel <= (2e-2 if dtype == "bf16" else 1e-5)
    assert np.array_equal(got[:, :H * D], X[:, :H * D]) and np.array_equal(got[:, 2 * H * D:], X[:, 2 * H * D:])


def test_embed_and_commit_are_exact_copies(orc, lib):
    rng = np.random.default_rng(6)
    E = synth.normal_bf16(rng, (500, 128))
    ids = rng.integers(0, 500, size=40).astype(np.int32)
    Ed, idd = dev(E), dev(ids)
    out = torch.empty(40, 128, dtype=torch.bfloat16, device="cuda")
    lib.eagle3_embed(Ed, idd, out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), orc.embed(E, ids))
    # commit rows 0, 3, 5 (then -1) of sequence 0 and rows 1 of sequence 1 into a paged cache
    B, T, Hkv, D = 2, 8, 2, 64
    kr, vr = synth.normal_bf16(rng, (B, T, Hkv, D)), synth.normal_bf16(rng, (B, T, Hkv, D))
    kv = synth.paged_kv(60, 0, [20, 5], Hkv, D, max_blocks=4)
    src = np.array([[0, 3, 5, -1, 2, 2, 2, 2], [1, -1, 0, 0, 0, 0, 0, 0]], np.int32)
    kc, vc, bt = dev(kv.k_cache), dev(kv.v_cache), dev(kv.block_table)
    lib.eagle3_commit_kv(dev(kr), dev(vr), dev(src), dev(kv.prefix_len), kc, vc, bt)
    torch.cuda.synchronize()
    K2, V2 = host(kc), host(vc)
    for b, rows in ((0, [0, 3, 5]), (1, [1])):
        for j, r in enumerate(rows):
            pos = int(kv.prefix_len[b]) + j
            blk, slot = kv.block_table[b, pos // 16], pos % 16
            assert np.array_equal(K2[blk, :, slot, :], kr[b, r])
            assert np.array_equal(V2[blk, :, :, slot], vr[b, r])
    untouched = np.ones(K2.shape[0], bool)
    for b, n in ((0, 3), (1, 1)):
        for j in range(n):
            untouched[kv.block_table[b, (int(kv.prefix_len[b]) + j) // 16]] = False
    assert np.array_equal(K2[untouched].view(np.uint16), kv.k_cache[untouched])


@pytest.mark.parametrize("mode", ["context", "step"])
def test_draft_fuse(orc, lib, mode):
    rng = np.random.default_rng(7)
    M, k, V = 70, 256, 1000
    l, m, h, a = (synth.normal_bf16(rng, (M, k)) for _ in range(4))
    E = synth.normal_bf16(rng, (V, k), 0.02)
    Wf = synth.normal_bf16(rng, (k, 3 * k), 0.02)
    Wi = synth.normal_bf16(rng, (k, 2 * k), 0.02)
    tok = rng.integers(0, V, size=M).astype(np.int32)
    x = torch.empty(M, k, dtype=torch.bfloat16, device="cuda")
    Ed, Wfd, Wid, td = dev(E), dev(Wf), dev(Wi), dev(tok)
    if mode == "context":
        ref, gref = orc.draft_fuse(tok, E, Wf, Wi, l=l, m=m, h=h, want_g=True)
        g = torch.empty(M, k, dtype=torch.bfloat16, device="cuda")
        ld, md, hd = dev(l), dev(m), dev(h)
        lib.eagle3_draft_fuse(td, Ed, Wid, x, w_fuse=Wfd, l=ld, m=md, h=hd, g_out=g)
        torch.cuda.synchronize()
        rel, _ = normwise_rel(host(g), gref)
        assert rel <= 2e-2
    else:
        ref = orc.draft_fuse(tok, E, Wf, Wi, a_prev=a)
        ad = dev(a)
        lib.eagle3_draft_fuse(td, Ed, Wid, x, a_prev=ad)
        torch.cuda.synchronize()
    rel, mx = normwise_rel(host(x), ref)
    assert rel <= 2e-2, (rel, mx)
