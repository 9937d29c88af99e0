"""Pins for the oracle's per-step operations: grouped RMSNorm, the
dequantizing matvec, split-half RoPE, GQA attention, SiLU and argmax.

Each is checked against library routines (torch / numpy), closed forms and
invariants that a dropped term, a wrong sign or index, or a transposed
operand would break.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(99)


# ---------------------------------------------------------------- RMSNorm ---

def test_grouped_rmsnorm_g1_is_torch_rms_norm():
    h = RNG.standard_normal(96)
    g = RNG.uniform(0.5, 1.5, 96).astype(np.float32)
    got = oracle.rmsnorm_grouped(h, g, 1, 1e-6)
    ref = F.rms_norm(torch.from_numpy(h), (96,), weight=torch.from_numpy(g).double(), eps=1e-6)
    assert np.allclose(got, ref.numpy(), rtol=1e-13, atol=0)


def test_grouped_rmsnorm_groups_are_independent():
    h = RNG.standard_normal(64)
    g = np.ones(64, np.float32)
    y = oracle.rmsnorm_grouped(h, g, 2, 0.0)
    for j in range(2):
        seg = y[j * 32:(j + 1) * 32]
        assert abs(np.sqrt(np.mean(seg ** 2)) - 1.0) < 1e-13
    # scaling one group leaves the output unchanged (eps = 0)
    h2 = h.copy()
    h2[32:] *= 7.5
    assert np.allclose(oracle.rmsnorm_grouped(h2, g, 2, 0.0), y, rtol=1e-13, atol=1e-15)
    # each group equals torch rms_norm over that group alone
    for j in range(2):
        ref = F.rms_norm(torch.from_numpy(h[j * 32:(j + 1) * 32]), (32,), eps=1e-6).numpy()
        assert np.allclose(oracle.rmsnorm_grouped(h, g, 2, 1e-6)[j * 32:(j + 1) * 32], ref,
                           rtol=1e-13)


def test_grouped_rmsnorm_gain_is_elementwise_over_full_hidden():
    h = RNG.standard_normal(16)
    g = np.arange(1, 17, dtype=np.float32)
    y1 = oracle.rmsnorm_grouped(h, np.ones(16, np.float32), 2, 1e-6)
    y2 = oracle.rmsnorm_grouped(h, g, 2, 1e-6)
    assert np.allclose(y2, y1 * g, rtol=1e-14)


# ---------------------------------------------------------------- matvec ----

def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("wdt", ["f32", "bf16", "fp8", "mxfp4"])
def test_matvec_equals_numpy_matmul_on_library_decoded_weights(wdt):
    N, K = 37, 96
    w32 = torch.randn(N, K, generator=torch.Generator().manual_seed(3)) * 0.02
    x = RNG.standard_normal(K)
    if wdt == "f32":
        m = oracle.Mat("f32", w32.numpy())
        dense = w32.double().numpy()
    else:
        bits = _bits(w32.to(torch.bfloat16))
        m = oracle.Mat.from_draw(wdt, bits)
        if wdt == "bf16":
            dense = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
        elif wdt == "fp8":
            v = torch.from_numpy(m.w).view(torch.float8_e4m3fn).double().numpy()
            dense = v * m.s.astype(np.float64)[:, None]
        else:
            table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
            nib = np.stack([m.w & 15, m.w >> 4], -1).reshape(N, K)
            sc = torch.from_numpy(m.s).view(torch.float8_e8m0fnu).double().numpy()
            dense = table[nib] * np.repeat(sc, 32, axis=1)
    got = m.matvec(x)
    assert np.allclose(got, dense @ x, rtol=1e-12, atol=1e-15)
    # a transposed operand would not even have the right length
    assert got.shape == (N,)


def test_matvec_q4s_equals_numpy_matmul_on_decoded_weights():
    N, K = 37, 192
    w32 = torch.randn(N, K, generator=torch.Generator().manual_seed(4)) * 0.02
    bits = _bits(w32.to(torch.bfloat16))
    m = oracle.Mat.from_draw("q4s", bits)
    assert m.w.shape == (N, K // 2) and m.s.shape == (N, K // 64)
    nib = np.stack([m.w & 15, m.w >> 4], -1).reshape(N, K).astype(np.int64)
    dense = np.where(nib >= 8, nib - 16, nib) * np.repeat(m.s.astype(np.float64), 64, axis=1)
    x = RNG.standard_normal(K)
    got = m.matvec(x)
    assert np.allclose(got, dense @ x, rtol=1e-12, atol=1e-15)


def test_matvec_dequant_is_close_to_bf16_weights():
    # quantization error stays inside the formats' half-step bounds
    N, K = 64, 256
    w = (torch.randn(N, K, generator=torch.Generator().manual_seed(5)) * 0.02).to(torch.bfloat16)
    bits = _bits(w)
    wd = w.double().numpy()
    x = np.zeros(K)
    for k in (0, 17, 200):
        x[:] = 0
        x[k] = 1.0
        y8 = oracle.Mat.from_draw("fp8", bits).matvec(x)
        y4 = oracle.Mat.from_draw("mxfp4", bits).matvec(x)
        amax_row = np.abs(wd).max(axis=1)
        # top binade [256, 448] has step 32 code units: half a step is 16 * s
        assert np.all(np.abs(y8 - wd[:, k]) <= amax_row / 448 * 16 + 1e-12)
        blk = np.abs(wd[:, (k // 32) * 32:(k // 32 + 1) * 32]).max(axis=1)
        # step 2 * 2^e at the top, 2^e <= amax / 4, saturation from [7, 8) to 6
        assert np.all(np.abs(y4 - wd[:, k]) <= blk * 0.5 + 1e-12)
        yq = oracle.Mat.from_draw("q4s", bits).matvec(x)
        b64 = np.abs(wd[:, (k // 64) * 64:(k // 64 + 1) * 64]).max(axis=1)
        assert np.all(np.abs(yq - wd[:, k]) <= b64 / 7 * 0.5 * (1 + 1e-6) + 1e-12)


# ------------------------------------------------------------------- RoPE ---

def test_rope_position_zero_is_identity():
    u = RNG.standard_normal(4 * 16)
    assert np.array_equal(oracle.rope(u, 4, 16, 0, 1e4), u)


def test_rope_hd2_is_plane_rotation_by_pos_radians():
    u = np.array([0.3, -1.2])
    p = 5
    c, s = math.cos(p), math.sin(p)
    want = np.array([0.3 * c + 1.2 * s, 0.3 * s - 1.2 * c])
    assert np.allclose(oracle.rope(u, 1, 2, p, 1e4), want, rtol=1e-15, atol=1e-15)


def test_rope_split_half_pairs_and_complex_rotation():
    hd, nh, pos, theta = 16, 3, 37, 1e4
    u = RNG.standard_normal(nh * hd)
    got = oracle.rope(u, nh, hd, pos, theta).reshape(nh, hd)
    v = u.reshape(nh, hd)
    half = hd // 2
    ang = pos * theta ** (-2.0 * np.arange(half) / hd)
    z = (v[:, :half] + 1j * v[:, half:]) * np.exp(1j * ang)
    assert np.allclose(got[:, :half], z.real, rtol=1e-13, atol=1e-14)
    assert np.allclose(got[:, half:], z.imag, rtol=1e-13, atol=1e-14)
    # each (i, i + hd/2) pair keeps its norm
    assert np.allclose(got[:, :half] ** 2 + got[:, half:] ** 2,
                       v[:, :half] ** 2 + v[:, half:] ** 2, rtol=1e-13)


def test_rope_scores_depend_only_on_relative_position():
    hd = 128
    q = RNG.standard_normal(hd)
    k = RNG.standard_normal(hd)
    def score(m, n):
        return oracle.rope(q, 1, hd, m, 1e4) @ oracle.rope(k, 1, hd, n, 1e4)
    assert abs(score(10, 3) - score(1010, 1003)) < 1e-10
    assert abs(score(7, 7) - q @ k) < 1e-12
    assert abs(score(10, 3) - score(3, 10)) > 1e-6          # not symmetric in m, n


# -------------------------------------------------------------- attention ---

def _cache_with(kvdt, n_kv, cap, hd, k, v):
    c = oracle.KVCache(kvdt, n_kv, cap, hd)
    for p in range(k.shape[1]):
        c.store(k[:, p].ravel(), v[:, p].ravel(), p)
    return c


@pytest.mark.parametrize("kvdt", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("n_qh,n_kv", [(8, 2), (4, 4), (32, 8)])
def test_attention_matches_torch_sdpa(kvdt, n_qh, n_kv):
    hd, cap, L = 16, 40, 29
    k = RNG.standard_normal((n_kv, L, hd))
    v = RNG.standard_normal((n_kv, L, hd))
    c = _cache_with(kvdt, n_kv, cap, hd, k, v)
    q = RNG.standard_normal(n_qh * hd)
    got, probs = oracle.attention(q, c, n_qh, L, want_probs=True)
    K = torch.from_numpy(c.dequant("k", L))[None]
    V = torch.from_numpy(c.dequant("v", L))[None]
    Q = torch.from_numpy(q.reshape(1, n_qh, 1, hd))
    ref = F.scaled_dot_product_attention(Q, K, V, enable_gqa=True)
    assert np.allclose(got, ref.numpy().ravel(), rtol=1e-12, atol=1e-13)
    assert np.allclose(probs.sum(axis=1), 1.0, atol=1e-14)


def test_attention_special_cases():
    hd, n_kv, n_qh, cap = 16, 2, 8, 8
    k = RNG.standard_normal((n_kv, 5, hd))
    v = RNG.standard_normal((n_kv, 5, hd))
    c = _cache_with("f32", n_kv, cap, hd, k, v)
    # one position: output is that value row, for every head of the group
    q = RNG.standard_normal(n_qh * hd)
    o1 = oracle.attention(q, c, n_qh, 1).reshape(n_qh, hd)
    vd = c.dequant("v", 5)
    for h in range(n_qh):
        assert np.allclose(o1[h], vd[h // 4, 0], rtol=1e-15)
    # zero query: uniform weights -> mean of the value rows
    o0 = oracle.attention(np.zeros(n_qh * hd), c, n_qh, 5).reshape(n_qh, hd)
    for h in range(n_qh):
        assert np.allclose(o0[h], vd[h // 4].mean(axis=0), rtol=1e-13)


def test_gqa_equals_mha_on_repeated_kv():
    hd, n_kv, rep, L = 16, 2, 4, 11
    k = RNG.standard_normal((n_kv, L, hd))
    v = RNG.standard_normal((n_kv, L, hd))
    q = RNG.standard_normal(n_kv * rep * hd)
    gqa = oracle.attention(q, _cache_with("f32", n_kv, 16, hd, k, v), n_kv * rep, L)
    kr = np.repeat(k, rep, axis=0)                              # contiguous groups
    vr = np.repeat(v, rep, axis=0)
    mha = oracle.attention(q, _cache_with("f32", n_kv * rep, 16, hd, kr, vr), n_kv * rep, L)
    assert np.allclose(gqa, mha, rtol=1e-14)


def test_attention_scale_shift_invariance():
    # adding a constant to every score (via a component shared by all keys)
    # leaves the softmax unchanged: checks the max-subtraction is harmless
    hd, L = 16, 9
    k = RNG.standard_normal((1, L, hd))
    v = RNG.standard_normal((1, L, hd))
    q = RNG.standard_normal(hd) * 30.0                           # large scores
    out = oracle.attention(q, _cache_with("f32", 1, L, hd, k, v), 1, L)
    s = (k[0].astype(np.float32).astype(np.float64) @ q) / 4.0
    a = np.exp(s - s.max())
    a /= a.sum()
    assert np.allclose(out, a @ v[0].astype(np.float32).astype(np.float64), rtol=1e-12)


# ------------------------------------------------------------ silu, argmax ---

def test_silu_matches_torch():
    for z in (-30.0, -2.5, -1e-3, 0.0, 0.7, 4.0, 40.0):
        assert abs(oracle.silu(z) - F.silu(torch.tensor(z, dtype=torch.float64)).item()) < 1e-15


def test_argmax_first_maximum_wins():
    v = np.array([1.0, 3.0, 2.0, 3.0, 3.0])
    assert oracle.argmax(v) == 1
    v = RNG.standard_normal(1000)
    assert oracle.argmax(v) == int(np.argmax(v))
