"""Pins for the oracle's MXFP4 decoding (CPU only).

The e2m1 table is checked against the format's bit-field definition, the E8M0
scale decode against torch's float8_e8m0fnu dtype (an independent library
decoder), and the nibble order against hand-packed bytes.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import f64_to_bf16_bits


def _e2m1_from_bits(code: int) -> float:
    # 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
    # subnormal: value = m/2; otherwise 2^(e-1) * (1 + m/2).
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def test_e2m1_table_matches_bit_fields():
    for c in range(16):
        got = oracle.decode_e2m1(np.array([c], dtype=np.uint8))[0]
        want = _e2m1_from_bits(c)
        assert got == want and np.signbit(got) == np.signbit(want), (c, got, want)


def test_e2m1_values_are_the_eight_magnitudes():
    mags = sorted(set(abs(float(v)) for v in oracle.E2M1_VALUES))
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e8m0_matches_torch_exhaustive():
    s = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.decode_e8m0(s)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[120] == 2.0 ** -7 and got[124] == 2.0 ** -3


def test_dequant_exhaustive_codes_times_scales():
    # every code x every finite scale byte, as a [256, 32] block matrix
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)            # 32 codes
    q = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)       # 16 bytes
    q = np.broadcast_to(q, (255, 16))
    s = np.arange(255, dtype=np.uint8)[:, None]
    W = oracle.dequant_mxfp4(q, s)
    for si in (0, 1, 100, 120, 124, 127, 200, 254):
        for kk in range(32):
            want = _e2m1_from_bits(int(codes[kk])) * 2.0 ** (si - 127)
            assert W[si, kk] == want


def test_nibble_order_low_first():
    # byte 0x71: low nibble 1 (0.5), high nibble 7 (6.0)
    q = np.array([[0x71, 0xA2]], dtype=np.uint8)
    assert list(oracle.unpack_codes(q)[0]) == [1, 7, 2, 10]
    W = oracle.dequant_mxfp4(np.tile(q, (1, 8)), np.array([[127]], dtype=np.uint8))
    assert list(W[0, :4]) == [0.5, 6.0, 1.0, -1.0]


def test_scale_applies_per_32_block():
    q = np.full((1, 32), 0x22, dtype=np.uint8)                   # 64 ones
    s = np.array([[127, 130]], dtype=np.uint8)
    W = oracle.dequant_mxfp4(q, s)
    assert np.all(W[0, :32] == 1.0) and np.all(W[0, 32:] == 8.0)


def test_generated_weights_exact_in_bf16():
    # each decoded weight at scale bytes 120..124 is exactly a bf16 value,
    # so a GPU dequantising to bf16 loses nothing
    vals = np.array([v * 2.0 ** (s - 127) for v in oracle.E2M1_VALUES for s in range(120, 125)])
    back = oracle.bf16_to_f64(f64_to_bf16_bits(vals))
    np.testing.assert_array_equal(back, vals)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_to_f64(bits)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


@pytest.mark.parametrize("shape", [(3, 64), (2, 5, 96)])
def test_dequant_shape_and_mismatch(shape):
    q = np.zeros(shape[:-1] + (shape[-1] // 2,), dtype=np.uint8)
    s = np.full(shape[:-1] + (shape[-1] // 32,), 127, dtype=np.uint8)
    assert oracle.dequant_mxfp4(q, s).shape == shape
    with pytest.raises(ValueError):
        oracle.dequant_mxfp4(q, s[..., :-1])


# ----------------------------------------------------------- weight layout --

def _blocked_by_loops(q):
    # the definition written out byte by byte: byte i of MX block b of row r
    # goes to offset b*256 + (r % 16)*16 + i of its 16-row group
    R, KH = q.shape
    out = np.zeros(R * KH, dtype=np.uint8)
    for r in range(R):
        base = (r // 16) * 16 * KH
        for b in range(KH // 16):
            for i in range(16):
                out[base + b * 256 + (r % 16) * 16 + i] = q[r, b * 16 + i]
    return out.reshape(R, KH)


def test_blocked_layout_matches_definition_and_inverts():
    rng = np.random.default_rng(11)
    q = rng.integers(0, 256, size=(48, 80), dtype=np.uint8)  # 3 row groups, 5 blocks
    qb = oracle.blocked_from_canonical(q)
    np.testing.assert_array_equal(qb, _blocked_by_loops(q))
    np.testing.assert_array_equal(oracle.canonical_from_blocked(qb), q)
    # leading dimensions (experts) are independent
    q3 = rng.integers(0, 256, size=(2, 32, 48), dtype=np.uint8)
    qb3 = oracle.blocked_from_canonical(q3)
    for e in range(2):
        np.testing.assert_array_equal(qb3[e], _blocked_by_loops(q3[e]))
    # a wave's 64 lanes (16 rows x 4 blocks) read one contiguous kilobyte
    flat = qb.reshape(-1)
    lanes = [flat[b * 256 + r * 16: b * 256 + r * 16 + 16] for b in range(4) for r in range(16)]
    np.testing.assert_array_equal(np.concatenate(lanes), flat[:1024])
    assert all(np.array_equal(lanes[b * 16 + r], q[r, b * 16:(b + 1) * 16])
               for b in range(4) for r in range(16))
    with pytest.raises(ValueError):
        oracle.blocked_from_canonical(q[:40])
