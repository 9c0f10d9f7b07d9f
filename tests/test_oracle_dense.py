"""Pins for the oracle's LM head (argmax / top-k / gap / lse), RMSNorm, bf16
rounding and dense layers (CPU only).

References: torch float64 on the CPU (matmul, argmax, logsumexp, rms_norm,
silu, complex rotation for RoPE), closed forms, exact ties built into the
data, and bf16 conversions done by torch.
"""
import numpy as np
import pytest
import torch

import synth


def f64(a):
    return (synth.bf16_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


# ------------------------------------------------------------- bf16 rounding

def test_round_bf16_special_values(orc):
    assert orc.round_bf16(1.0) == 0x3F80
    assert orc.round_bf16(1.0 + 2.0 ** -8) == 0x3F80                 # tie -> even
    assert orc.round_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82             # tie -> even (up)
    assert orc.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81    # no double rounding
    assert orc.round_bf16(-2.5) == 0xC020
    assert orc.round_bf16(0.0) == 0 and orc.round_bf16(-0.0) == 0x8000
    assert orc.round_bf16(3.0e38 * 10) == 0x7F80                      # overflow -> inf


def test_round_bf16_matches_torch_on_fp32_values(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(2000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(2000) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.round_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)
    assert np.array_equal(synth.f32_to_bf16(x), ref)   # the generators' rounding too


# ------------------------------------------------------------- LM head

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lmhead_against_torch(orc, dtype):
    rng = np.random.default_rng(1)
    M, N, K = 37, 3001, 96
    h = synth.normal_f32(rng, (M, K))
    w = synth.normal_f32(rng, (N, K), 0.05)
    if dtype == "bf16":
        h, w = synth.f32_to_bf16(h), synth.f32_to_bf16(w)
    idx, val, gap, lse = orc.lmhead(h, w, topk=5)
    logits = torch.from_numpy(f64(h)) @ torch.from_numpy(f64(w)).T
    np.testing.assert_allclose(val[:, 0], logits.max(dim=1).values.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=1).numpy(), rtol=1e-13)
    am = logits.argmax(dim=1).numpy()
    assert np.array_equal(idx[:, 0], am)
    L = logits.numpy()
    for m in range(M):
        order = np.lexsort((np.arange(N), -L[m]))[:5]     # value desc, id asc
        assert list(idx[m]) == list(order)
        srt = np.sort(L[m])[::-1]
        assert abs(gap[m] - (srt[0] - srt[1])) < 1e-12


def test_lmhead_exact_ties_pick_lowest_index(orc):
    rng = np.random.default_rng(2)
    M, N, K = 8, 64, 32
    h = synth.f32_to_bf16(synth.normal_f32(rng, (M, K)))
    w = synth.f32_to_bf16(synth.normal_f32(rng, (N, K)))
    w[50] = w[7]; w[63] = w[7]; w[33] = w[20]        # exact duplicate rows
    idx, val, gap, _ = orc.lmhead(h, w, topk=4)
    logits = f64(h) @ f64(w).T
    for m in range(M):
        top = idx[m, 0]
        assert logits[m, top] == logits[m].max()
        assert top == np.flatnonzero(logits[m] == logits[m].max()).min()
        if top in (7, 20):
            assert gap[m] == 0.0
            twin = 50 if top == 7 else 33
            assert idx[m, 1] == twin


def test_lmhead_one_hot_reads_a_column(orc):
    rng = np.random.default_rng(3)
    N, K = 500, 40
    w = synth.normal_f32(rng, (N, K))
    h = np.eye(K, dtype=np.float32)[:10] * 1.0
    idx, val, _, _ = orc.lmhead(h, w, topk=1)
    for k in range(10):
        assert idx[k, 0] == int(np.argmax(w[:, k]))
        assert val[k, 0] == float(w[:, k].max())


# ------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rmsnorm_against_torch(orc, dtype):
    rng = np.random.default_rng(4)
    x = synth.normal_f32(rng, (33, 4096), 0.1)
    g = (1 + synth.normal_f32(rng, (4096,), 0.1)).astype(np.float32)
    if dtype == "bf16":
        x, g = synth.f32_to_bf16(x), synth.f32_to_bf16(g)
    y = orc.rmsnorm(x, g, eps=1e-5)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(f64(x)), (4096,), torch.from_numpy(f64(g)), eps=1e-5).numpy()
    tol = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    np.testing.assert_allclose(f64(y), ref, rtol=tol, atol=1e-30)


def test_rmsnorm_constant_row_closed_form(orc):
    c = 0.37
    x = np.full((2, 256), c, np.float32)
    y = orc.rmsnorm(x, eps=1e-5)
    np.testing.assert_allclose(y, np.float32(c / np.sqrt(np.float64(np.float32(c)) ** 2 + 1e-5)), rtol=1e-6)


# ------------------------------------------------------------- dense layers

def test_gemm_and_residual_against_torch(orc):
    rng = np.random.default_rng(5)
    A = synth.normal_f32(rng, (17, 70)); Bm = synth.normal_f32(rng, (23, 70)); R = synth.normal_f32(rng, (17, 23))
    C = orc.gemm(A, Bm, R)
    ref = (torch.from_numpy(A.astype(np.float64)) @ torch.from_numpy(Bm.astype(np.float64)).T).numpy() + R
    np.testing.assert_allclose(C, ref.astype(np.float32), rtol=1e-6, atol=1e-6)
    Ab, Bb = synth.f32_to_bf16(A), synth.f32_to_bf16(Bm)
    Cb = orc.gemm(Ab, Bb)
    ref = f64(Ab) @ f64(Bb).T
    np.testing.assert_allclose(f64(Cb), ref, rtol=2.0 ** -8, atol=1e-30)


def test_swiglu_against_torch(orc):
    rng = np.random.default_rng(6)
    X = synth.normal_f32(rng, (9, 64)); W = synth.normal_f32(rng, (2 * 40, 64), 0.2)
    Y = orc.swiglu(X, W)
    g = torch.from_numpy(X.astype(np.float64)) @ torch.from_numpy(W[:40].astype(np.float64)).T
    u = torch.from_numpy(X.astype(np.float64)) @ torch.from_numpy(W[40:].astype(np.float64)).T
    np.testing.assert_allclose(Y, (torch.nn.functional.silu(g) * u).numpy().astype(np.float32), rtol=1e-6, atol=1e-7)


def test_rope_is_a_complex_rotation(orc):
    rng = np.random.default_rng(7)
    M, H, D, theta = 6, 3, 64, 500000.0
    x = synth.normal_f32(rng, (M, H, D))
    pos = np.array([0, 1, 7, 128, 200, 4095], np.int32)
    y = orc.rope(x, pos, theta)
    z = x[..., :D // 2].astype(np.float64) + 1j * x[..., D // 2:].astype(np.float64)
    freq = theta ** (-np.arange(D // 2) * 2.0 / D)
    z = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    ref = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(y, ref.astype(np.float32), rtol=1e-6, atol=1e-6)
    assert np.array_equal(y[0], x[0])                  # position 0 is the identity


def test_embed_copies_rows(orc):
    rng = np.random.default_rng(8)
    E = synth.f32_to_bf16(synth.normal_f32(rng, (100, 16)))
    ids = np.array([5, 0, 99, 5], np.int32)
    assert np.array_equal(orc.embed(E, ids), E[ids])


def test_silu_mul_against_torch(orc):
    rng = np.random.default_rng(9)
    GU = synth.normal_f32(rng, (7, 2 * 33), 2.0)
    Y = orc.silu_mul(GU)
    t = torch.from_numpy(GU.astype(np.float64))
    ref = (torch.nn.functional.silu(t[:, :33]) * t[:, 33:]).numpy()
    np.testing.assert_allclose(Y, ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    # agrees with the fused form up to the storage rounding of the gate/up product
    X = synth.normal_f32(rng, (5, 40)); W = synth.normal_f32(rng, (2 * 12, 40), 0.3)
    np.testing.assert_allclose(orc.silu_mul(orc.gemm(X, W)), orc.swiglu(X, W), rtol=1e-5, atol=1e-6)
