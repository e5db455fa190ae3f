"""Number formats of the oracle: bf16 and OCP e4m3fn, plus the fp8 block rule.

Test infrastructure only (see ``oracle/__init__.py``).

Definitions written from the formats themselves:

* bf16: the upper 16 bits of an IEEE binary32 -- 1 sign, 8 exponent
  (bias 127), 7 stored mantissa bits; rounding is to nearest, ties to even.
* e4m3fn (OCP 8-bit floating point, "E4M3"): 1 sign, 4 exponent (bias 7),
  3 mantissa bits; exponent field 0 is subnormal (value ``2**-6 * M/8``);
  ``S.1111.111`` is NaN; there is no infinity; the largest finite value is
  ``1.75 * 2**8 = 448``.  Encoding rounds to nearest, ties to even, keeps
  subnormals and saturates to +-448.
* Block rule for the fp8 layer (weights per 128x128 block, activations per
  row per 128 columns): ``s = fp32(amax / 448)``; ``code = e4m3(fp32(v / s))``;
  ``s = 1`` and all codes 0 when amax is 0.  Scales are plain fp32.
* MXFP4 (OCP Microscaling formats, FP4 E2M1 elements with an E8M0 scale
  shared by 32 consecutive elements): an element is 1 sign, 2 exponent
  (bias 1) and 1 mantissa bit; exponent field 0 is subnormal (``0.5 * M``);
  the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  An E8M0 scale byte ``e`` is
  the power of two ``2**(e - 127)`` (255 is NaN).  Element j of a row is
  stored in byte j // 2, the even element in the low nibble.
* MXFP8 (OCP Microscaling, FP8 E4M3 elements with an E8M0 scale shared by
  32 consecutive elements): one e4m3fn byte per element, scaled by
  ``2**(e - 127)``.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# ----------------------------------------------------------------- bf16 --

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even).

    Works directly from the float64 value (no intermediate fp32 rounding).
    Returns float64 holding exactly representable bf16 values; overflow
    gives +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    fin = np.isfinite(v) & (v != 0)
    mant, ex = np.frexp(v[fin])           # v = mant * 2**ex, 0.5 <= |mant| < 1
    # 8 significant bits for normals; fixed quantum 2**-133 below 2**-126.
    q_exp = np.maximum(ex - 8, -133)
    quantum = np.ldexp(1.0, q_exp)
    r = np.rint(v[fin] / quantum) * quantum   # np.rint: ties to even
    bf_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > bf_max, np.sign(r) * np.inf, r)
    out[fin] = r
    out[~fin] = v[~fin]
    return out


def bf16_encode(v: np.ndarray) -> np.ndarray:
    """float64/float32 values -> uint16 bf16 patterns (nearest, ties to even)."""
    r = bf16_round(v).astype(np.float32)     # exact: bf16 values fit fp32
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- e4m3fn --

def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes -> exact float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mt = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(mt / 8.0, -6),
                   np.ldexp(1.0 + mt / 8.0, e - 7))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return s * val


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32/float64 values -> uint8 e4m3fn codes.

    Nearest representable value, ties to even mantissa, subnormals kept,
    magnitudes beyond 448 saturate to 448.  The sign of zero is kept.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v)
    a = np.abs(v)
    codes = np.zeros(v.shape, dtype=np.int64)
    nz = a > 0
    mant, ex = np.frexp(a[nz])             # a = mant * 2**ex
    # 4 significant bits for normals (>= 2**-6); fixed quantum 2**-9 below.
    quantum = np.ldexp(1.0, np.maximum(ex - 4, -9))
    r = np.rint(a[nz] / quantum) * quantum
    r = np.minimum(r, E4M3_MAX)
    # r is now exactly representable; split it into exponent / mantissa.
    rc = np.zeros(r.shape, dtype=np.int64)
    pos = r > 0
    m2, e2 = np.frexp(r[pos])               # r = m2 * 2**e2, m2 in [0.5, 1)
    unb = e2 - 1                            # r = 1.f * 2**unb
    normal = unb >= -6
    field_e = np.where(normal, unb + 7, 0)
    mfield = np.where(normal,
                      np.rint((m2 * 2.0 - 1.0) * 8.0),
                      np.rint(r[pos] / 2.0 ** -9))
    rc[pos] = (field_e << 3) | mfield.astype(np.int64)
    codes[nz] = rc
    codes = codes | np.where(sign, 0x80, 0)
    return codes.astype(np.uint8)


def e4m3_quantize_rows(v32: np.ndarray, block: int = 128):
    """Per-row, per-``block``-column fp8 quantisation of an fp32 matrix.

    ``v32`` is a float32 ``[n, K]`` array with ``K % block == 0``.  Returns
    ``(codes uint8 [n, K], scales float32 [n, K/block])`` following the block
    rule in the module docstring; every division is a correctly rounded fp32
    division (numpy float32 arithmetic).
    """
    v32 = np.asarray(v32, dtype=np.float32)
    n, K = v32.shape
    assert K % block == 0
    g = v32.reshape(n, K // block, block)
    amax = np.abs(g).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0))
    scale = scale.astype(np.float32)
    q = (g / scale[:, :, None]).astype(np.float32)
    codes = e4m3_encode(q).reshape(n, K)
    return codes, scale


def dequant_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """Exact float64 values of a block-scaled e4m3 matrix.

    ``codes [R, C]`` with ``scales [R/block_r, C/block]`` where the row block
    is ``R // scales.shape[0]`` (128 for weights, 1 for activation rows).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    R, C = codes.shape
    sr, sc = scales.shape
    br, bc = R // sr, C // sc
    table = e4m3_decode(np.arange(256, dtype=np.uint8))   # value of every code
    vals = table[codes].reshape(sr, br, sc, bc)
    return (vals * np.asarray(scales, np.float64)[:, None, :, None]).reshape(R, C)


# ---------------------------------------------------------------- MXFP4 --

def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit e2m1 codes (values 0..15) -> exact float64 values."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    e = (c >> 1) & 0x3
    mt = (c & 1).astype(np.float64)
    val = np.where(e == 0, 0.5 * mt, np.ldexp(1.0 + mt / 2.0, e - 1))
    return np.where(c & 0x8, -val, val)


def e8m0_decode(e: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> float64 powers of two (NaN for 255)."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))


def mxfp4_decode(packed: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """Packed MXFP4 matrix -> exact float64 values.

    ``packed [rows, cols/2]`` uint8 (element 2i in the low nibble of byte i,
    element 2i+1 in the high nibble); ``scales [rows, cols/block]`` E8M0
    bytes, one per ``block`` consecutive elements of a row.
    """
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[0], -1)
    return e2m1_decode(codes) * np.repeat(e8m0_decode(scales), block, axis=1)


def mxfp8_decode(codes: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """MXFP8 matrix -> exact float64 values: ``codes [rows, cols]`` e4m3fn
    bytes, ``scales [rows, cols/block]`` E8M0 bytes."""
    return e4m3_decode(codes) * np.repeat(e8m0_decode(scales), block, axis=1)
