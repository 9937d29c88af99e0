"""Pins for the oracle's storage codecs (bf16, fp8 E4M3FN, E2M1, E8M0, Q4S int4, int8 KV).

Each codec is checked against something other than its own formula: torch's
independent dtype decoders, the published OCP E2M1 table, brute-force nearest
search over the code table, hand-computed values, and the byte counts the
k3_run.c page prints for its MXFP4 experts.
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------------- bf16 ---

def test_bf16_value_matches_torch_all_patterns():
    bits = np.arange(0, 1 << 16, 257, dtype=np.uint16)        # 256 spread patterns
    mine = oracle.bf16_value(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(mine[fin], ref[fin])


def test_bf16_round_matches_torch_rne():
    x = RNG.standard_normal(4000).astype(np.float32) * np.float32(0.05)
    # exact ties: bf16 value + half an ulp (low half = 0x8000)
    b = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    ties = ((b.astype(np.uint32) << 16) | 0x8000).view(np.float32)[:200]
    allx = np.concatenate([x, ties, np.float32([0.0, -0.0, 1.0, -3.5])])
    mine = oracle.bf16_round(allx)
    ref = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


# -------------------------------------------------------------------- fp8 ---

def test_fp8_value_matches_torch_all_256_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.fp8_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    fin = ~np.isnan(ref)
    assert np.array_equal(mine[fin], ref[fin])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def _fp8_finite_table():
    c = np.arange(256, dtype=np.uint8)
    v = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    ok = ~np.isnan(v)
    return c[ok], v[ok]


def _brute_nearest(x, codes, vals):
    """Nearest representable value; ties go to the code with an even last
    mantissa bit; beyond the largest magnitude saturate.  Sign from x."""
    out = []
    mags = vals[(vals >= 0) & ~((vals == 0) & (codes != 0))]
    mcodes = codes[(vals >= 0) & ~((vals == 0) & (codes != 0))]
    for t in x:
        a = abs(float(t))
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            best = [i for i in best if (mcodes[i] & 1) == 0]
        out.append(float(np.copysign(mags[best[0]], t)))
    return np.array(out)


def test_fp8_encode_brute_force_nearest_even():
    codes, vals = _fp8_finite_table()
    pos = np.sort(np.unique(vals[vals >= 0]))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)           # every tie
    rnd = (RNG.standard_normal(3000) * 60).astype(np.float32)
    rnd = rnd[np.abs(rnd) < 448]
    x = np.concatenate([mids, -mids, rnd, np.float32([0.0, 448.0, -448.0, 2.0 ** -10])])
    enc = oracle.fp8_encode(x)
    got = oracle.fp8_value(enc)
    want = _brute_nearest(x, codes, vals)
    assert np.array_equal(np.abs(got), np.abs(want))
    # and torch's own fp32 -> e4m3fn cast agrees inside the finite range
    tor = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.abs(got), np.abs(tor))


def test_fp8_encode_saturates():
    for v in (448.0, 460.0, 464.0, 479.0, 500.0, 1e6):
        assert oracle.fp8_value(oracle.fp8_encode(np.float32([v])))[0] == 448.0
        assert oracle.fp8_value(oracle.fp8_encode(np.float32([-v])))[0] == -448.0


def test_fp8_encode_decode_roundtrip_every_code():
    codes, vals = _fp8_finite_table()
    enc = oracle.fp8_encode(vals.astype(np.float32))
    nz = vals != 0
    assert np.array_equal(enc[nz], codes[nz])


# ------------------------------------------------------------- E2M1 / E8M0 ---

def test_e2m1_values_are_the_ocp_table():
    # OCP Microscaling v1.0, FP4 E2M1 element table
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oracle.e2m1_value(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == table
    assert list(-got[8:]) == table
    assert math.copysign(1.0, got[8]) == -1.0


def test_e2m1_encode_ties_and_saturation():
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             5.01: 6.0, 6.0: 6.0, 7.0: 6.0, 100.0: 6.0, 0.2: 0.0, 0.26: 0.5, 0.5: 0.5}
    for x, want in cases.items():
        for sgn in (1.0, -1.0):
            got = oracle.e2m1_value(oracle.e2m1_encode(np.float32([sgn * x])))[0]
            assert got == sgn * want, (sgn * x, got)


def test_e2m1_encode_brute_force_random():
    codes = np.arange(16, dtype=np.uint8)
    vals = oracle.e2m1_value(codes)
    x = (RNG.uniform(-7, 7, 4000)).astype(np.float32)
    got = oracle.e2m1_value(oracle.e2m1_encode(x))
    want = _brute_nearest(x, codes, vals)
    assert np.array_equal(got, want)


def test_e8m0_matches_torch():
    b = np.arange(255, dtype=np.uint8)
    mine = oracle.e8m0_value(b)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(mine, ref)
    assert np.isnan(oracle.e8m0_value(np.uint8([255]))[0])


# ------------------------------------------------------------- quantizers ---

def _bf16_draw(n, k, std=0.02, seed=7):
    t = torch.Generator().manual_seed(seed)
    w = (torch.randn(n, k, generator=t) * std).to(torch.bfloat16)
    return w.view(torch.int16).numpy().view(np.uint16), w.double().numpy()


def test_quant_fp8_rows_properties():
    bits, w = _bf16_draw(64, 96)
    bits[3] = 0                         # an all-zero row
    w[3] = 0.0
    codes, s = oracle.quant_fp8_rows(bits)
    assert s[3] == 0.0 and not codes[3].any()
    dq = oracle.fp8_value(codes)
    for n in range(64):
        if n == 3:
            continue
        amax = np.abs(w[n]).max()
        # the row maximum maps to the top finite code
        assert abs(dq[n][np.argmax(np.abs(w[n]))]) == 448.0
        # every element is the nearest E4M3 value to w/s (brute force)
        t = (w[n].astype(np.float32) / s[n]).astype(np.float32)
        cds, vals = _fp8_finite_table()
        want = _brute_nearest(np.clip(t, -448, 448), cds, vals)
        assert np.array_equal(np.abs(dq[n]), np.abs(want))
        # the scale is amax/448 to fp32 precision
        assert abs(float(s[n]) * 448.0 - amax) <= amax * 2 ** -23


def test_quant_mxfp4_properties():
    bits, w = _bf16_draw(16, 128)
    bits[2, 32:64] = 0                  # an all-zero block
    w[2, 32:64] = 0.0
    q, e = oracle.quant_mxfp4(bits)
    assert q.shape == (16, 64) and e.shape == (16, 4)
    assert e[2, 1] == 0 and not q[2, 16:32].any()
    lo, hi = q & 15, q >> 4
    nib = np.stack([lo, hi], -1).reshape(16, 128)
    vals = oracle.e2m1_value(nib)
    for n in range(16):
        for b in range(4):
            blk = w[n, b * 32:(b + 1) * 32]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            m, ex = math.frexp(amax)                        # amax = m * 2^ex, m in [0.5, 1)
            assert int(e[n, b]) - 127 == (ex - 1) - 2       # floor(log2 amax) - emax(E2M1)
            scaled = blk / 2.0 ** (int(e[n, b]) - 127)
            got = vals[n, b * 32:(b + 1) * 32]
            want = _brute_nearest(scaled.astype(np.float32), np.arange(16, dtype=np.uint8),
                                  oracle.e2m1_value(np.arange(16, dtype=np.uint8)))
            assert np.array_equal(got, want)
            assert np.abs(got).max() in (4.0, 6.0)


def test_mxfp4_expert_bytes_match_k3_page():
    """k3_run.c prints ~25.8 GB of routed experts read per token and a
    1.45 TB expert pool; with 92 MoE layers (93 layers, first dense) and
    3 matrices of 3072 x 3584 per expert at 4 bits + one E8M0 byte per 32,
    the packing must give exactly 17,547,264 bytes per expert."""
    inter, latent = 3072, 3584
    q13 = np.zeros((2 * inter, latent // 2), np.uint8)
    e13 = np.zeros((2 * inter, latent // 32), np.uint8)
    q2 = np.zeros((latent, inter // 2), np.uint8)
    e2 = np.zeros((latent, inter // 32), np.uint8)
    per_expert = q13.nbytes + e13.nbytes + q2.nbytes + e2.nbytes
    assert per_expert == 17_547_264
    assert round(92 * 16 * per_expert / 1e9, 1) == 25.8
    assert round(92 * 896 * per_expert / 1e12, 2) == 1.45
    # embed + lm_head, 2 x 163840 x 7168 bf16 = the page's 4.70 GB
    assert round(2 * 163840 * 7168 * 2 / 1e9, 2) == 4.70


# -------------------------------------------------------------------- Q4S ---

def test_q4s_values_are_twos_complement_nibbles():
    assert list(oracle.q4s_value(np.arange(16, dtype=np.uint8))) == \
        [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def _q4s_nibbles(q):
    n, half = q.shape
    return np.stack([q & 15, q >> 4], -1).reshape(n, 2 * half)      # even k = low nibble


def test_quant_q4s_hand_values():
    # block max 7/16 makes s = a/7 = 1/16 exactly; codes are then w * 16 with
    # ties to even (0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 3.5 -> 4)
    w = torch.zeros(2, 128, dtype=torch.bfloat16)
    vals = [0.03125, 0.09375, 0.15625, -0.15625, 0.21875, 0.4375, -0.4375, 0.0625, -0.03125]
    w[0, :len(vals)] = torch.tensor(vals)
    w[0, 64] = 1.75                       # second block: a = 1.75, s = 0.25
    w[0, 65] = -0.375                     # -1.5 steps -> -2
    q, sc = oracle.quant_q4s(w.view(torch.int16).numpy().view(np.uint16))
    assert q.shape == (2, 64) and sc.shape == (2, 2)
    assert sc[0, 0] == 0.0625 and sc[0, 1] == 0.25
    assert sc[1, 0] == 0.0 and sc[1, 1] == 0.0 and not q[1].any()     # all-zero blocks
    codes = oracle.q4s_value(_q4s_nibbles(q))
    assert list(codes[0, :len(vals)]) == [0, 2, 2, -2, 4, 7, -7, 1, 0]
    assert list(codes[0, 64:66]) == [7, -2]
    assert not codes[0, len(vals):64].any() and not codes[0, 66:].any()
    assert q[0, 0] == (0 | (2 << 4)) and q[0, 1] == (2 | (0xE << 4))  # -2 is nibble 0xE, high


def test_quant_q4s_properties():
    bits, w = _bf16_draw(16, 256)
    bits[5, 64:128] = 0
    w[5, 64:128] = 0.0
    q, sc = oracle.quant_q4s(bits)
    nib = _q4s_nibbles(q)
    assert not (nib == 8).any()                                      # -8 is never produced
    codes = oracle.q4s_value(nib)
    assert sc[5, 1] == 0.0 and not codes[5, 64:128].any()
    levels = np.arange(-7, 8, dtype=np.float64)
    for n in range(16):
        for b in range(4):
            blk = w[n, b * 64:(b + 1) * 64]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            s = float(sc[n, b])
            assert s == float(np.float32(np.float32(amax) / np.float32(7)))
            t = (blk.astype(np.float32) / np.float32(s)).astype(np.float64)
            for i, tv in enumerate(t):                               # brute-force nearest level
                d = np.abs(levels - tv)
                best = levels[d == d.min()]
                want = best[0] if len(best) == 1 else best[np.argmin(np.abs(best) % 2)]
                assert codes[n, b * 64 + i] == want, (n, b, i, tv)
            assert np.abs(codes[n, b * 64:(b + 1) * 64]).max() == 7
            assert np.all(np.abs(codes[n, b * 64:(b + 1) * 64] * s - blk) <= s * 0.5 * (1 + 1e-6))


# ----------------------------------------------------------------- int8 KV ---

def test_int8_kv_codec_hand_values():
    # a = 127/64 makes s = a/127 = 1/64 exactly; then codes are x * 64
    x = np.zeros(128, np.float32)
    x[:7] = [1.984375, -1.984375, 0.984375, 0.9921875, 0.0078125, 0.0234375, -0.0078125]
    codes, s = oracle.kv_quant_int8(x)
    assert s == 0.015625
    assert list(codes[:7]) == [127, -127, 63, 64, 0, 2, 0]      # 63.5 -> 64, 0.5 -> 0, 1.5 -> 2
    assert not codes[7:].any()
    assert oracle.int8_dequant(63, s) == 0.984375


def test_int8_kv_codec_zero_block_and_range():
    codes, s = oracle.kv_quant_int8(np.zeros(128, np.float32))
    assert s == 0.0 and not codes.any()
    x = RNG.standard_normal(128).astype(np.float32)
    codes, s = oracle.kv_quant_int8(x)
    assert codes.min() >= -127 and codes.max() <= 127
    assert abs(codes[np.argmax(np.abs(x))]) == 127
    # dequantized error within half a step
    dq = np.array([oracle.int8_dequant(c, s) for c in codes])
    assert np.abs(dq - x).max() <= s * 0.5 * (1 + 1e-6)
