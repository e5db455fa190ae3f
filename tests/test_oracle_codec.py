"""Pins of the oracle's number formats (CPU only).

Each codec is checked against its closed-form definition, a brute-force
nearest-value search, and torch's CPU casts -- three routes that share no
code with ``oracle/codec.py``.
"""
import numpy as np
import pytest
import torch

from oracle.codec import (bf16_decode, bf16_encode, bf16_round, dequant_blocks,
                          e4m3_decode, e4m3_encode, e4m3_quantize_rows)


# ------------------------------------------------------------------ bf16 --

def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    mine = bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_bf16_encode_matches_torch_on_random_and_halfway_values(np_rng):
    v = np_rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact halfway points between neighbouring bf16 values: ties to even
    base = np.arange(0x3F80, 0x4080, dtype=np.uint32) << 16
    half = (base | 0x8000).view(np.float32)
    v = np.concatenate([v, half, -half, np.float32([1e-39, -3e-40, 3.3e38])])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_encode(v), ref)


def test_bf16_round_from_fp64_is_nearest(np_rng):
    """Direct fp64 -> bf16 rounding, checked by bracketing neighbours."""
    v = np_rng.standard_normal(20_000) * 10.0 ** np_rng.integers(-6, 6, 20_000)
    r = bf16_round(v)
    # neighbours on the bf16 grid around r
    bits = bf16_encode(r).astype(np.int32)
    up = bf16_decode((bits + 1).astype(np.uint16))
    dn = bf16_decode((bits - 1).astype(np.uint16))
    err = np.abs(v - r)
    assert np.all(err <= np.abs(v - up))
    assert np.all(err <= np.abs(v - dn))


# ------------------------------------------------------------------ e4m3 --

def _formula_decode(c):
    s = -1.0 if c & 0x80 else 1.0
    e, mt = (c >> 3) & 0xF, c & 7
    if e == 15 and mt == 7:
        return float("nan")
    if e == 0:
        return s * 2.0 ** -6 * mt / 8.0
    return s * 2.0 ** (e - 7) * (1 + mt / 8.0)


def test_e4m3_decode_all_codes_formula_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3_decode(codes)
    formula = np.array([_formula_decode(int(c)) for c in codes])
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    for other in (formula, ref):
        nan = np.isnan(other)
        assert np.array_equal(np.isnan(mine), nan)
        assert np.array_equal(mine[~nan], other[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])


def _brute_encode(v):
    """Nearest finite e4m3 code; ties -> even mantissa; saturate at 448."""
    codes = np.array([c for c in range(128) if not np.isnan(_formula_decode(c))])
    vals = np.array([_formula_decode(c) for c in codes])
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(v):
        a = min(abs(float(x)), 448.0)
        d = np.abs(vals - a)
        cand = codes[d == d.min()]
        c = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
        out[i] = c | (0x80 if np.signbit(x) else 0)
    return out


def test_e4m3_encode_brute_force_on_bf16_range():
    # every bf16 value with |v| in [2**-12, 512): covers subnormals,
    # every binade, ties, and saturation
    bits = np.arange(1 << 16, dtype=np.uint16)
    v = bf16_decode(bits)
    sel = np.isfinite(v) & (np.abs(v) < 512) & ((np.abs(v) >= 2.0 ** -12) | (v == 0))
    v = v[sel].astype(np.float32)
    assert np.array_equal(e4m3_encode(v), _brute_encode(v))


def test_e4m3_encode_matches_torch_cast(np_rng):
    v = (np_rng.standard_normal(300_000) * 60).astype(np.float32)
    v = np.concatenate([v, np.float32([0.0, -0.0, 448.0, 463.9, 464.0, 470.0,
                                       2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9 * 1.5])])
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(v), ref)


# ------------------------------------------------------- block quantiser --

def test_block_quantiser_invariants(np_rng):
    v = (np_rng.standard_normal((64, 512)) * np.exp(np_rng.standard_normal((64, 1)))).astype(np.float32)
    v[3, 128:256] = 0.0                      # an all-zero block
    codes, s = e4m3_quantize_rows(v, 128)
    assert codes.shape == v.shape and s.shape == (64, 4)
    assert np.all(np.isfinite(s)) and np.all(s > 0)
    assert s[3, 1] == 1.0 and np.all(codes[3, 128:256] == 0)
    dq = dequant_blocks(codes, s, 128)
    # every non-zero block maps its largest magnitude to +-448
    g = np.abs(e4m3_decode(codes)).reshape(64, 4, 128).max(axis=2)
    nz = np.abs(v).reshape(64, 4, 128).max(axis=2) > 0
    assert np.all(g[nz] == 448.0)
    # |v - dq| <= half an e4m3 ulp of v/s, times s
    q = np.abs(v.astype(np.float64) / np.repeat(s, 128, axis=1))
    _, ex = np.frexp(q)
    ulp = np.ldexp(1.0, np.maximum(ex - 4, -9))
    assert np.all(np.abs(v - dq) <= 0.5 * ulp * np.repeat(s, 128, axis=1) * (1 + 1e-6))


def test_block_scale_is_correctly_rounded_fp32_division(np_rng):
    v = (np_rng.standard_normal((16, 128)) * 3).astype(np.float32)
    _, s = e4m3_quantize_rows(v, 128)
    amax = np.abs(v).max(axis=1).astype(np.float64)
    exact = amax / 448.0
    # the fp32 scale is the nearest fp32 to amax/448
    f = s[:, 0].astype(np.float64)
    nxt = np.nextafter(s[:, 0], np.float32(np.inf)).astype(np.float64)
    prv = np.nextafter(s[:, 0], np.float32(0)).astype(np.float64)
    assert np.all(np.abs(f - exact) <= np.abs(nxt - exact))
    assert np.all(np.abs(f - exact) <= np.abs(prv - exact))


@pytest.mark.parametrize("shape", [(256, 384), (128, 128)])
def test_weight_block_dequant_layout(shape, np_rng):
    """dequant_blocks pairs each 128x128 block with its own scale."""
    R, C = shape
    codes = np_rng.integers(0, 0x7E, size=shape, dtype=np.uint8)
    s = np_rng.uniform(0.5, 2, size=(R // 128, C // 128)).astype(np.float32)
    dq = dequant_blocks(codes, s, 128)
    for bi in range(R // 128):
        for bj in range(C // 128):
            blk = dq[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            ref = e4m3_decode(codes[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]) * float(s[bi, bj])
            assert np.array_equal(blk, ref)


# ---------------------------------------------------------------- MXFP4 --
# OCP Microscaling Formats (MX) v1.0: FP4 E2M1 element magnitudes, in code
# order 0..7, as the format's definition tabulates them.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_codes_match_the_format_table():
    from oracle.codec import e2m1_decode
    v = e2m1_decode(np.arange(16))
    assert list(v[:8]) == E2M1_MAGNITUDES
    assert list(-v[8:]) == E2M1_MAGNITUDES          # bit 3 is the sign
    assert np.signbit(v[8])                         # code 8 is -0


def test_e8m0_is_a_power_of_two_with_bias_127():
    from oracle.codec import e8m0_decode
    e = np.arange(255)
    assert np.array_equal(e8m0_decode(e), np.ldexp(1.0, e - 127))
    assert e8m0_decode(np.array([127]))[0] == 1.0 and np.isnan(e8m0_decode(np.array([255]))[0])


def test_mxfp4_decode_packing_and_block_scales():
    """Element 2i in the low nibble of byte i; one scale per 32 elements."""
    from oracle.codec import mxfp4_decode
    codes = np.arange(64).reshape(1, 64) % 16
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.array([[127 + 3, 127 - 2]], np.uint8)
    v = mxfp4_decode(packed, scales)
    mags = np.array(E2M1_MAGNITUDES + [-m for m in E2M1_MAGNITUDES])
    want = mags[codes[0]] * np.where(np.arange(64) < 32, 8.0, 0.25)
    assert np.array_equal(v[0], want)


def test_synth_mxfp4_storage_is_nearest_with_saturation():
    """The stored codes are the nearest e2m1 value of v / 2**X (brute-force
    search over the 8 magnitudes; exact ties excluded), with X =
    floor(log2(amax)) - 2 per 32 elements."""
    import torch
    import synth
    from oracle.codec import mxfp4_decode
    g = torch.Generator().manual_seed(3)
    w = torch.randn((8, 256), generator=g) * 0.02
    w[0, :32] = 0.0                                 # an all-zero block
    packed, sc = synth._mx_fp4(w)
    v = mxfp4_decode(packed.numpy(), sc.numpy())
    wn = w.double().numpy()
    for r in range(8):
        for b in range(8):
            blk = wn[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                assert np.all(v[r, 32 * b:32 * b + 32] == 0)
                continue
            X = np.floor(np.log2(amax)) - 2
            assert sc.numpy()[r, b] == X + 127
            q = np.abs(blk) / 2.0 ** X
            d = np.abs(q[:, None] - np.array(E2M1_MAGNITUDES)[None, :])
            near = np.array(E2M1_MAGNITUDES)[np.argmin(d, axis=1)]
            got = np.abs(v[r, 32 * b:32 * b + 32]) / 2.0 ** X
            assert np.array_equal(got, near)
            assert np.all(np.sign(v[r, 32 * b:32 * b + 32]) * np.sign(blk) >= 0)


def test_mxfp8_decode_applies_one_scale_per_32_elements():
    from oracle.codec import e4m3_decode, mxfp8_decode
    codes = (np.arange(64, dtype=np.uint8) * 3).reshape(1, 64)
    codes[codes & 0x7F == 0x7F] = 0                  # no NaN codes
    scales = np.array([[127 - 4, 127 + 5]], np.uint8)
    v = mxfp8_decode(codes, scales)
    want = e4m3_decode(codes[0]) * np.where(np.arange(64) < 32, 2.0 ** -4, 2.0 ** 5)
    assert np.array_equal(v[0], want)


def test_synth_mxfp8_storage_is_nearest_e4m3_of_the_quotient():
    """Brute force over all finite e4m3 magnitudes: the stored code is a
    nearest one to v / 2**X (X = floor(log2(amax)) - 8, the quotient of the
    block maximum lands in [256, 512) and saturates at 448)."""
    import torch
    import synth
    from oracle.codec import e4m3_decode, mxfp8_decode
    g = torch.Generator().manual_seed(4)
    w = torch.randn((6, 128), generator=g) * 0.02
    codes, sc = synth._mx_fp8(w)
    v = mxfp8_decode(codes.numpy(), sc.numpy())
    grid = np.unique(np.abs(e4m3_decode(np.arange(256, dtype=np.uint8))))
    grid = grid[np.isfinite(grid)]
    wn = w.double().numpy()
    for r in range(6):
        for b in range(4):
            blk = wn[r, 32 * b:32 * b + 32]
            X = np.floor(np.log2(np.abs(blk).max())) - 8
            assert sc.numpy()[r, b] == X + 127
            q = np.minimum(np.abs(blk.astype(np.float32) / np.float32(2.0 ** X)), 448.0)
            got = np.abs(v[r, 32 * b:32 * b + 32]) / 2.0 ** X
            dist = np.abs(q[:, None] - grid[None, :])
            assert np.all(np.abs(q - got) <= dist.min(axis=1) + 1e-12)
