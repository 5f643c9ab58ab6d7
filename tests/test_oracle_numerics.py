"""Pins of the oracle's number formats (bf16, E4M3, E8M0 / MX blocks).

Each check compares the oracle with something other than itself: values the
pages print, closed forms, or torch's own dtype casts (library routines that
the oracle does not call).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_float_storage_example(orc):
    """The page's FP32 storage example (4.8125, bias 2^(n-1)-1) and its bf16 / E4M3 consequences."""
    g = json.load(open(os.path.join(GOLD, "float_storage_example.json")))
    v = g["value"]
    bits = int(g["derived"]["bf16_bits"], 16)
    assert orc.f64_to_bf16(np.array([v]))[0] == bits
    # decode by the page's field rule: (-1)^s * 1.mantissa * 2^(exp - 127)
    exp_field = (bits >> 7) & 0xFF
    mant = bits & 0x7F
    assert exp_field - 127 == g["true_exponent"]
    assert 1 + mant / 128 == g["mantissa_value"]
    assert orc.bf16_to_f64(np.array([bits], np.uint16))[0] == v
    code = int(g["derived"]["e4m3_code"], 16)
    assert (code >> 3) & 0xF == g["true_exponent"] + (2 ** (4 - 1) - 1)
    assert orc.f64_to_e4m3(np.array([v]))[0] == code
    assert orc.e4m3_to_f64(np.array([code], np.uint8))[0] == g["derived"]["e4m3_value"]


def test_bf16_round_matches_torch_cast(orc):
    rng = np.random.default_rng(0)
    vals = [rng.standard_normal(20000).astype(np.float32),
            (rng.standard_normal(5000) * 1e30).astype(np.float32),
            (rng.standard_normal(5000) * 1e-38).astype(np.float32),     # fp32 subnormal range
            np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38, 3.4e38, np.inf, -np.inf], np.float32)]
    # exact ties between two bf16 values: mantissa bit 15 set, lower bits clear
    tie_bits = (rng.integers(0, 2**16, 5000).astype(np.uint32) << 16) | 0x8000
    tie_bits &= ~np.uint32(0x7F800000) | np.uint32(0x3F800000)        # keep exponents finite
    vals.append(tie_bits.view(np.float32))
    x = np.concatenate(vals)
    got = orc.f64_to_bf16(x.astype(np.float64))
    want = _torch_bf16_bits(x)
    np.testing.assert_array_equal(got, want)


def test_bf16_round_from_double_closed_forms(orc):
    one = 1.0
    step = 2.0 ** -7
    cases = {
        one + step / 2: 0x3F80,                       # tie -> even (1.0)
        one + step / 2 + 2.0 ** -40: 0x3F81,          # just above the tie
        one + 1.5 * step: 0x3F82,                     # tie between 0x3F81 and 0x3F82 -> even
        -(one + step / 2 - 2.0 ** -40): 0xBF80,
        2.0 ** -133: 0x0001,                          # smallest bf16 subnormal
        2.0 ** -134: 0x0000,                          # half of it: tie -> even (zero)
        2.0 ** -134 + 2.0 ** -160: 0x0001,
        (2 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,          # rounds up past the largest finite value
        (2 - 2.0 ** -7) * 2.0 ** 127: 0x7F7F,
    }
    for v, bits in cases.items():
        assert orc.f64_to_bf16(np.array([v]))[0] == bits, (v, hex(bits))


def test_e4m3_decode_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_to_f64(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_after_clamp(orc):
    """torch's float8_e4m3fn cast rounds to nearest even but does not saturate,
    so the reference clamps to +-448 first (the oracle's reading)."""
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(4000) * 100, rng.standard_normal(2000) * 1e-2,
                        rng.uniform(-600, 600, 2000), rng.standard_normal(500) * 1e-3,
                        np.array([0.0, -0.0, 448.0, -448.0, 464.0, 479.9, 480.0, 1e6, -1e6, 2.0 ** -10,
                                  3 * 2.0 ** -11, 2.0 ** -9 * 0.5, 2.0 ** -9 * 1.5])]).astype(np.float32)
    xc = np.clip(x, -448, 448)
    want = torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.f64_to_e4m3(x.astype(np.float64))
    # torch may drop the sign of a negative value that rounds to zero; compare magnitudes there
    zero = (want & 0x7F) == 0
    np.testing.assert_array_equal(got[~zero], want[~zero])
    assert np.all((got[zero] & 0x7F) == 0)
    assert np.all((got[zero] >> 7) == np.signbit(x[zero]).astype(np.uint8))


def _block_reference(v: np.ndarray):
    """Closed form of one MX block from the rule: scale byte = floor(log2 amax) + 119."""
    amax = float(np.max(np.abs(v)))
    if amax == 0.0:
        return 0, None
    m, ex = math.frexp(amax)
    e = min(127, max(-127, ex - 1 - 8))
    return e + 127, e


def test_mx_block_closed_forms(orc):
    rng = np.random.default_rng(2)
    R, C = 64, 256
    x32 = (rng.standard_normal((R, C)) * np.exp(rng.uniform(-20, 20, (R, 1)))).astype(np.float32)
    x32[3, :32] = 0.0                             # an all-zero block
    x32[5, 32:64] = -0.0
    x32[7, :32] = 2.0 ** rng.integers(-20, 20, 32) * np.sign(rng.standard_normal(32))   # powers of two
    xb = _torch_bf16_bits(x32)
    q, s = orc.mxfp8_quantize(xb, axis=0)
    xv = orc.bf16_to_f64(xb)
    for r in range(R):
        for b in range(C // 32):
            blk = xv[r, b * 32:(b + 1) * 32]
            byte, e = _block_reference(blk)
            assert s[r, b] == byte, (r, b)
            codes = q[r, b * 32:(b + 1) * 32]
            if e is None:
                assert np.all((codes & 0x7F) == 0)
                continue
            scaled = np.clip(blk * 2.0 ** (-e), -448, 448).astype(np.float32)
            want = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            nz = (want & 0x7F) != 0
            np.testing.assert_array_equal(codes[nz], want[nz])
            # the block maximum lands in [256, 448]
            mags = np.abs(orc.e4m3_to_f64(codes))
            assert 256 <= mags.max() <= 448
    # powers of two round-trip exactly when they are within the block's 2^-9..448 window
    blk = xv[7, :32]
    byte = s[7, 0]
    deq = orc.e4m3_to_f64(q[7, :32]) * 2.0 ** (int(byte) - 127)
    keep = np.abs(blk) >= 2.0 ** (int(byte) - 127 - 9)
    np.testing.assert_array_equal(deq[keep], blk[keep])


def test_mx_axis1_group_restart(orc):
    """Group-aware blocks along rows restart at every group offset and scale rows are packed."""
    rng = np.random.default_rng(3)
    sizes = np.array([0, 5, 32, 33, 0, 70], np.int32)
    M, C = int(sizes.sum()), 64
    x32 = rng.standard_normal((M, C)).astype(np.float32) * 3
    xb = _torch_bf16_bits(x32)
    q, s = orc.mxfp8_quantize(xb, axis=1, group_sizes=sizes)
    assert s.shape == (1 + 1 + 2 + 3, C)
    xv = orc.bf16_to_f64(xb)
    o, P = 0, 0
    for n in sizes:
        for b in range((n + 31) // 32):
            r0, r1 = o + 32 * b, o + min(n, 32 * (b + 1))
            for c in range(C):
                byte, e = _block_reference(xv[r0:r1, c])
                assert s[P + b, c] == byte
                scaled = np.clip(xv[r0:r1, c] * 2.0 ** (-e), -448, 448).astype(np.float32)
                want = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                nz = (want & 0x7F) != 0
                np.testing.assert_array_equal(q[r0:r1, c][nz], want[nz])
        o += n
        P += (n + 31) // 32


# --------------------------------------------------------------------------- NaN and infinities
# E4M3FN has no infinity and one NaN per sign (0x7F / 0xFF); E8M0 reserves
# 0xFF for NaN; E2M1 has neither (OCP MX v1.0 element and scale formats).
# Reading of the MX block rule for a block holding a NaN or an infinity: its
# amax has no finite exponent, so the block scale is the E8M0 NaN, which makes
# every element of the block NaN; each code is then the element format's
# encoding of NaN with the value's sign (E2M1: its largest code, as a
# saturation).

_NONFINITE_BF16 = {"nan": 0x7FC0, "-nan": 0xFFC0, "inf": 0x7F80, "-inf": 0xFF80}


def test_e4m3_encode_nonfinite_matches_torch(orc):
    vals = np.array([np.nan, -np.nan, np.inf, -np.inf], np.float64)
    vals[1] = np.copysign(np.nan, -1.0)
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.f64_to_e4m3(vals)
    assert got.tolist() == ref.tolist() == [0x7F, 0xFF, 0x7F, 0xFF]


def test_e8m0_decode(orc):
    s = orc.e8m0_to_f64(np.arange(256, dtype=np.uint8))
    assert np.isnan(s[255]) and not np.isnan(s[:255]).any()
    np.testing.assert_array_equal(s[:255], 2.0 ** (np.arange(255) - 127.0))


def _row_with(blocks):
    """bf16 bits [1, 32*len(blocks)]: block b holds normal draws, with the
    listed non-finite patterns planted at the listed positions."""
    rng = np.random.default_rng(5)
    x = orc_bits(rng.standard_normal(32 * len(blocks)).astype(np.float32))
    for b, plant in enumerate(blocks):
        for pos, name in plant:
            x[32 * b + pos] = _NONFINITE_BF16[name]
    return x[None, :]


def orc_bits(a32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_mx_block_nonfinite(orc):
    x = _row_with([[(3, "nan")], [(0, "-inf")], [], [(31, "inf"), (7, "-nan")]])
    q, s = orc.mxfp8_quantize(x, 0)
    assert s[0, 0] == 0xFF and s[0, 1] == 0xFF and s[0, 3] == 0xFF and s[0, 2] != 0xFF
    sign = (x[0] >> 15).astype(np.uint8)
    for b in (0, 1, 3):
        np.testing.assert_array_equal(q[0, 32 * b:32 * b + 32], 0x7F | (sign[32 * b:32 * b + 32] << 7))
    # the finite block is quantised as on its own
    q2, s2 = orc.mxfp8_quantize(np.ascontiguousarray(x[:, 64:96]), 0)
    assert s2[0, 0] == s[0, 2] and np.array_equal(q2[0], q[0, 64:96])
    # decoded: every element of a NaN-scale block is NaN, the finite block is finite
    v = orc.e4m3_to_f64(q[0]) * np.repeat(orc.e8m0_to_f64(s[0]), 32)
    assert np.isnan(v[:64]).all() and np.isnan(v[96:]).all() and np.isfinite(v[64:96]).all()


def test_mx_block_nonfinite_grouped_columns(orc):
    rng = np.random.default_rng(9)
    x = orc_bits(rng.standard_normal((70, 16)).astype(np.float32))
    x[40, 5] = _NONFINITE_BF16["-inf"]       # group 1 (rows 30..69), its block 0 (rows 30..61)
    q, s = orc.mxfp8_quantize(x, 1, np.array([30, 40], np.int32))
    # blocks: group 0 -> scale row 0; group 1 -> rows 1 (30..61), 2 (62..69)
    assert s[1, 5] == 0xFF and (s[[0, 2], 5] != 0xFF).all() and (np.delete(s[1], 5) != 0xFF).all()
    sign = (x[30:62, 5] >> 15).astype(np.uint8)
    np.testing.assert_array_equal(q[30:62, 5], 0x7F | (sign << 7))


def test_e2m1_nonfinite(orc):
    v = np.array([np.nan, np.copysign(np.nan, -1.0), np.inf, -np.inf, 1e300, -7.0])
    assert orc.f64_to_e2m1(v).tolist() == [7, 15, 7, 15, 7, 15]
    x = np.ascontiguousarray(np.tile(_row_with([[], [(2, "-nan")], [], []]), (2, 1)))
    q, s = orc.mxfp4_quantize(x)
    assert (s[:, 1] == 0xFF).all() and (s[:, [0, 2, 3]] != 0xFF).all()
    sign = (x[:, 32:64] >> 15).astype(np.uint8)
    np.testing.assert_array_equal(q[:, 32:64], 7 | (sign << 3))
