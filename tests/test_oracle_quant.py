"""Pins of oracle/quant.py (storage rounding and quantizers) against things other than itself.

* bf16 / e4m3 against torch's own casts (library routines) on the same values;
* e4m3 / e2m1 encoders against brute-force nearest-code search over the whole code
  table, ties to the even code, saturation at the largest finite value;
* MXFP4 block scale against its defining property (largest element lands in [4, 8)).
"""

import numpy as np
import pytest
import torch

from oracle import quant as Q


def _edge_values():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(4000) * 3,
        rng.standard_normal(1000) * 1e-3,
        rng.standard_normal(1000) * 300,
        np.array([0.0, -0.0, 1.0, -1.0, 448.0, 449.0, 464.0, 480.0, 1e6, -1e6,
                  2.0 ** -6, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875]),
    ])
    return v.astype(np.float32)


def test_bf16_matches_torch_cast():
    v = _edge_values()
    mine = Q.bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    # exact decode of the stored value
    back = Q.bf16_decode(mine)
    assert np.array_equal(back, torch.from_numpy(v).to(torch.bfloat16).float().numpy().astype(np.float64))


def test_bf16_ties_to_even():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1+2^-7: goes to the even 1.0
    assert Q.round_bf16(np.float32(1 + 2 ** -8)) == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert Q.round_bf16(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = Q.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.nanmax(mine) == 448.0


def _brute_nearest(v, table_vals, table_codes):
    """Nearest table value; ties -> even code; the sign follows v."""
    out = []
    for x in v:
        a = abs(float(x))
        d = np.abs(table_vals - a)
        best = d.min()
        cands = table_codes[d == best]
        even = [c for c in cands if c % 2 == 0]
        c = int(even[0] if even else cands[0])
        out.append(c)
    return np.array(out)


def test_e4m3_encode_brute_force():
    v = _edge_values()
    pos_codes = np.arange(0x7F, dtype=np.uint8)   # 0x00..0x7E: all finite non-negative
    vals = Q.e4m3_decode(pos_codes)
    brute = _brute_nearest(np.minimum(np.abs(v), 448.0), vals, pos_codes.astype(np.int64))
    brute = np.where(np.signbit(v), brute | 0x80, brute)
    assert np.array_equal(Q.e4m3_encode(v), brute.astype(np.uint8))


def test_e4m3_encode_matches_torch_in_range():
    v = _edge_values()
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(Q.e4m3_encode(v), ref)


def test_e4m3_saturates():
    c = Q.e4m3_encode(np.array([1e9, -1e9, 500.0], dtype=np.float32))
    assert list(Q.e4m3_decode(c)) == [448.0, -448.0, 448.0]


def test_e2m1_table_and_brute_force():
    assert list(Q.e2m1_decode(np.arange(8))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(Q.e2m1_decode(np.arange(8, 16))) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-8, 8, 5000),
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -5.0, 100.0])])
    brute = _brute_nearest(np.minimum(np.abs(v), 6.0), Q.E2M1_VALUES, np.arange(8))
    brute = np.where(np.signbit(v), brute | 0x8, brute)
    assert np.array_equal(Q.e2m1_encode(v), brute.astype(np.uint8))


def test_mxfp4_block_scale_property_and_nearest():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((7, 128)) * np.exp2(rng.integers(-10, 10, (7, 1)))).astype(np.float32)
    x[3, 32:64] = 0.0                                  # an all-zero block
    packed, sc = Q.mxfp4_quantize(x)
    assert packed.shape == (7, 64) and sc.shape == (7, 4)
    X = sc.astype(np.int64) - 127
    blocks = x.astype(np.float64).reshape(7, 4, 32)
    amax = np.abs(blocks).max(-1)
    nz = amax > 0
    ratio = amax[nz] / np.exp2(X[nz])
    assert np.all((ratio >= 4.0) & (ratio < 8.0))
    assert X[3, 1] == -127
    deq = Q.mxfp4_dequantize(packed, sc).reshape(7, 4, 32)
    # every element is the nearest point of scale * {+-e2m1 grid} (saturating)
    grid = np.concatenate([-Q.E2M1_VALUES[::-1], Q.E2M1_VALUES])
    for b in range(7):
        for j in range(4):
            s = np.exp2(X[b, j])
            pts = grid * s
            for e in range(32):
                xv = blocks[b, j, e]
                best = np.abs(pts - xv).min()
                assert abs(deq[b, j, e] - xv) == best


def test_mxfp4_nibble_order():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 4.0      # amax 4 -> X = 0, element code for 4.0 = 6
    x[0, 1] = -1.0     # code 0x8 | 2 = 0xA
    packed, sc = Q.mxfp4_quantize(x)
    assert sc[0, 0] == 127
    assert packed[0, 0] == (0x6 | (0xA << 4))


def test_fp8mix_roundtrip_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 512)).astype(np.float32)
    codes, rope_bits, s = Q.fp8mix_quantize(x, 64)
    assert codes.shape == (50, 448) and rope_bits.shape == (50, 64) and s.shape == (50,)
    deq = Q.fp8mix_dequantize(codes, rope_bits, s)
    # the largest non-RoPE element of every entry maps to +-448 exactly (up to fp32 rounding of s)
    amax = np.abs(x[:, :448]).max(1)
    assert np.allclose(np.abs(Q.e4m3_decode(codes)).max(1), 448.0)
    # e4m3 has 3 mantissa bits: relative error <= 2^-4 for normal values
    nope = x[:, :448].astype(np.float64)
    big = np.abs(nope) >= (2.0 ** -6) * s[:, None] * 1.0001
    rel = np.abs(deq[:, :448] - nope)[big] / np.abs(nope)[big]
    assert rel.max() <= 2.0 ** -4 * 1.0001
    assert np.all(np.abs(deq[:, :448] - nope) <= amax[:, None] / 448 * 2.0 ** -7 + 1e-30 + np.abs(nope) * 2.0 ** -4)
    # RoPE dims are plain bf16
    assert np.array_equal(deq[:, 448:], Q.round_bf16(x[:, 448:]))
    # an all-zero entry keeps scale 1
    z = np.zeros((1, 512), dtype=np.float32)
    _, _, s0 = Q.fp8mix_quantize(z, 64)
    assert s0[0] == 1.0


@pytest.mark.parametrize("n", [0, 1])
def test_zero_sign(n):
    # -0.0 keeps its sign bit in both formats
    assert Q.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert Q.e2m1_encode(np.array([-0.0]))[0] == 0x8
