"""Storage-format rounding and quantizers used by the oracle (TEST INFRASTRUCTURE ONLY).

Every routine here is written from the public definition of the storage format,
element by element, with exact float64 arithmetic wherever the format allows:

* bf16: the upper 16 bits of an IEEE binary32, rounded to nearest, ties to even.
* fp8 e4m3 (OCP 8-bit float, "FN" flavour): 1 sign, 4 exponent bits (bias 7),
  3 mantissa bits, subnormals, no infinities, largest finite 448, code 0x7F/0xFF
  is NaN.  Conversions round to nearest-even and saturate to +-448.
* fp4 e2m1 (OCP MX v1.0 element type): 1 sign, 2 exponent bits (bias 1), 1 mantissa
  bit; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; round to nearest-even, saturate at 6.
* MXFP4 block (OCP MX v1.0): 32 contiguous elements share one e8m0 scale 2^X with
  X = floor(log2(amax)) - 2 (2 = largest exponent of e2m1), clamped to [-127, 127].

Where the pages fix the use: [V4-CN] §2.3.4 (RoPE dims kept in BF16, the other KV
dims in FP8) and §3.4 (the indexer's QK path cached, loaded and multiplied in
MXFP4 with 1x32 scaling tiles).  The per-entry FP8 scale s = amax/448 (computed in
fp32) is the reading taken here; the pages do not give the scale recipe.

Decisions (a quantized code) are taken in the precision the format and the
reading fix: the scale and x/s are single fp32 operations, exactly as a device
quantizer computes them from fp32 inputs.

Parity: pinned in tests/test_oracle_quant.py against brute-force nearest-code
search over the full code tables and, where defined for the same inputs, torch's
own bf16 / float8_e4m3fn casts.
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- bf16


def bf16_bits(x) -> np.ndarray:
    """Round float64/float32 values to bf16 and return the 16-bit patterns (uint16).

    float64 inputs are first rounded to float32 (nearest-even), as a device that
    computes in fp32 and stores bf16 does.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    # nearest-even on the 16 dropped bits
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    rounded = np.where(nan, (u >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Value of x after storage as bf16 (float64 result)."""
    return bf16_decode(bf16_bits(x))


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------- fp8 e4m3

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """fp8 e4m3 codes (uint8) -> float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def _rne(v):
    """Round to nearest integer, ties to even (float64, exact for |v| < 2^52)."""
    return np.rint(v)


def e4m3_encode(x) -> np.ndarray:
    """float32-valued inputs -> e4m3 codes, nearest-even, saturating at +-448."""
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    nan = np.isnan(v)
    a_safe = np.where(nan, 0.0, a)
    # binade exponent: a in [2^e, 2^(e+1)); below the normal range the quantum is fixed
    _, ex = np.frexp(np.where(a_safe > 0, a_safe, 1.0))
    e = np.maximum(ex - 1, -6)
    quantum = np.exp2(e - 3.0)
    mag = _rne(a_safe / quantum) * quantum
    mag = np.minimum(mag, E4M3_MAX)
    # encode the (representable) magnitude
    _, ex2 = np.frexp(np.where(mag > 0, mag, 1.0))
    e2 = ex2 - 1
    normal = mag >= 2.0 ** -6
    exp_field = np.where(normal, e2 + 7, 0)
    mant = np.where(normal, mag / np.exp2(e2 - 3.0) - 8.0, mag / 2.0 ** -9)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    # the sign bit follows the input's sign, also when the magnitude rounds to 0
    code = np.where(np.signbit(v), code | 0x80, code)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


# ------------------------------------------------------------------- fp4 e2m1

E2M1_MAX = 6.0
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """4-bit e2m1 codes (0..15) -> float64 values."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return sign * mag


def e2m1_encode(x) -> np.ndarray:
    """Values (already divided by the block scale) -> 4-bit codes, nearest-even, saturating."""
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    quantum = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    mag = np.minimum(_rne(a / quantum) * quantum, E2M1_MAX)
    # magnitude -> code via the value table (exact match)
    idx = np.searchsorted(E2M1_VALUES, mag)
    code = idx.astype(np.int64)
    code = np.where(np.signbit(v), code | 0x8, code)
    return code.astype(np.uint8)


def mxfp4_quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantize rows of fp32 values [..., n] (n % 32 == 0) to MXFP4.

    Returns (packed, scales): packed uint8 [..., n/2] with element 2j in the low
    nibble and 2j+1 in the high nibble; scales uint8 e8m0 [..., n/32] (code = X+127).
    """
    v = np.asarray(x, dtype=np.float32).astype(np.float64)
    n = v.shape[-1]
    assert n % 32 == 0, "MXFP4 needs the row length to be a multiple of 32"
    blocks = v.reshape(v.shape[:-1] + (n // 32, 32))
    amax = np.max(np.abs(blocks), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, (ex - 1) - 2, -127)
    X = np.clip(X, -127, 127)
    scaled = blocks / np.exp2(X.astype(np.float64))[..., None]
    codes = e2m1_encode(scaled).reshape(v.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


def mxfp4_dequantize(packed, scales) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    lo = e2m1_decode(p & 0xF)
    hi = e2m1_decode(p >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * 2,))
    X = np.asarray(scales, dtype=np.int64) - 127
    n = vals.shape[-1]
    blocks = vals.reshape(vals.shape[:-1] + (n // 32, 32))
    return (blocks * np.exp2(X.astype(np.float64))[..., None]).reshape(vals.shape)


# ------------------------------------------------------- FP8-mixed KV entries


def fp8mix_quantize(x, rope_dims: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Quantize KV entries [..., D] (fp32 values) to the mixed layout of [V4-CN] §2.3.4.

    The first D-R ("non-RoPE") dims become e4m3 codes with one fp32 scale per
    entry, s = amax/448 (s = 1 for an all-zero entry); the last R (RoPE) dims are
    kept as bf16.  Returns (codes uint8 [..., D-R], rope_bits uint16 [..., R],
    scale float32 [...]).
    """
    v = np.asarray(x, dtype=np.float32)
    D = v.shape[-1]
    nope = v[..., : D - rope_dims]
    rope = v[..., D - rope_dims:]
    amax = np.max(np.abs(nope), axis=-1)
    # single fp32 division, as the format's scale is stored and applied in fp32
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    scaled = (nope / s[..., None]).astype(np.float32)
    codes = e4m3_encode(scaled)
    return codes, bf16_bits(rope), s


def fp8mix_dequantize(codes, rope_bits, scale) -> np.ndarray:
    nope = e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]
    return np.concatenate([nope, bf16_decode(rope_bits)], axis=-1)
