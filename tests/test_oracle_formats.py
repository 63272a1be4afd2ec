"""Pins for the oracle's element decoders and dequantiser.

Each decoder is checked over its whole domain against something other than the
oracle: the hand-written E2M1 table (OCP MX FP4), torch's own float8_e8m0fnu and
float8_e4m3fn conversions (library routines for the same OCP formats), and
hand-worked bytes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from golden_io import e2m1_table, e4m3_cases, mx_bytes, nvfp4_cases


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e2m1_all_codes_match_table():
    table = e2m1_table()
    assert len(table) == 16
    for code, v in table.items():
        assert _same(oracle.e2m1(code), v), code
        # only the low nibble is the code
        assert _same(oracle.e2m1(code | 0xF0), v)


def test_e8m0_all_bytes_match_torch_and_ldexp():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64)
    for b in range(256):
        got = oracle.e8m0(b)
        if b == 255:
            assert math.isnan(got) and math.isnan(float(ref[b]))
            continue
        assert got == math.ldexp(1.0, b - 127)
        assert got == float(ref[b])


def test_e4m3_all_bytes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for b in range(256):
        assert _same(oracle.e4m3(b), float(ref[b])), hex(b)


def test_e4m3_hand_worked():
    for b, v in e4m3_cases():
        assert _same(oracle.e4m3(b), v), hex(b)


def test_mx_hand_worked_bytes():
    for byte, scale, v0, v1 in mx_bytes():
        # one 32-element block whose first byte is the worked byte
        q = np.zeros((1, 16), dtype=np.uint8)
        q[0, 0] = byte
        s = np.array([[scale]], dtype=np.uint8)
        out = oracle.dequant(q, s, 1, 32, oracle.MXFP4)
        assert _same(out[0, 0], v0) and _same(out[0, 1], v1), (hex(byte), hex(scale))


def test_nvfp4_hand_worked():
    for code, sbyte, ts, v in nvfp4_cases():
        q = np.zeros((1, 8), dtype=np.uint8)
        q[0, 0] = code
        s = np.array([[sbyte]], dtype=np.uint8)
        out = oracle.dequant(q, s, 1, 16, oracle.NVFP4, ts)
        assert _same(out[0, 0], v)


def test_exhaustive_mx_code_scale_grid():
    """All 16 codes x 256 scale bytes against table * 2^(b-127)."""
    table = e2m1_table()
    q = np.zeros((256, 16), dtype=np.uint8)
    for c in range(16):
        # elements 2c' hold codes: put code c at element c (byte c//2, nibble c%2)
        q[:, c // 2] |= (c << (4 * (c % 2)))
    s = np.arange(256, dtype=np.uint8).reshape(256, 1)
    out = oracle.dequant(q, s, 256, 32, oracle.MXFP4)
    for b in range(256):
        for c in range(16):
            want = math.nan if b == 255 else table[c] * math.ldexp(1.0, b - 127)
            assert _same(out[b, c], want), (b, c)


def test_block_of_ones_dot():
    """32 codes 0x2 (=1.0) at scale 0x7F dotted with ones is 32."""
    q = np.full((1, 16), 0x22, dtype=np.uint8)
    s = np.array([[0x7F]], dtype=np.uint8)
    w = oracle.dequant(q, s, 1, 32, oracle.MXFP4)
    assert float(w.sum()) == 32.0


def test_nibble_order_low_first():
    q = np.zeros((1, 16), dtype=np.uint8)
    q[0, 3] = 0x71          # element 6 = code 1 (0.5), element 7 = code 7 (6.0)
    s = np.array([[0x7F]], dtype=np.uint8)
    w = oracle.dequant(q, s, 1, 32, oracle.MXFP4)[0]
    assert w[6] == 0.5 and w[7] == 6.0
    assert np.count_nonzero(w) == 2


def test_block_axis_is_along_row():
    """Scale j of row r covers elements [32j, 32j+32) of that row only."""
    rows, K = 3, 96
    q = np.full((rows, K // 2), 0x22, dtype=np.uint8)
    s = np.full((rows, K // 32), 0x7F, dtype=np.uint8)
    s[1, 2] = 0x81            # x4 on row 1, last block
    w = oracle.dequant(q, s, rows, K, oracle.MXFP4)
    assert np.all(w[0] == 1.0) and np.all(w[2] == 1.0)
    assert np.all(w[1, :64] == 1.0) and np.all(w[1, 64:] == 4.0)


def _indep_dequant_mx(q, s, K):
    """Independent decoder: golden E2M1 table and torch's E8M0 conversion."""
    table = np.array([e2m1_table()[c] for c in range(16)])
    lo = q & 0xF
    hi = q >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(q.shape[0], K)
    sc = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return table[codes] * np.repeat(sc, 32, axis=1)


def _indep_dequant_nv(q, s, ts, K):
    table = np.array([e2m1_table()[c] for c in range(16)])
    codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], K)
    sc = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return table[codes] * np.repeat(sc, 16, axis=1) * ts


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("shape", [(16, 64), (40, 256)])
def test_random_bytes_against_independent_decoder(seed, shape):
    """MXFP4 dequant over 8 seeds x 2 shapes (the windlass README test sizes) and NVFP4."""
    rows, K = shape
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    s = rng.integers(100, 150, size=(rows, K // 32), dtype=np.uint8)
    got = oracle.dequant(q, s, rows, K, oracle.MXFP4)
    np.testing.assert_array_equal(got, _indep_dequant_mx(q, s, K))
    s16 = rng.integers(0, 0x7F, size=(rows, K // 16), dtype=np.uint8)
    ts = float(np.float32(rng.uniform(0.01, 2.0)))
    got = oracle.dequant(q, s16, rows, K, oracle.NVFP4, ts)
    np.testing.assert_array_equal(got, _indep_dequant_nv(q, s16, ts, K))


def test_blob_stride_pins_page_sizes():
    """Blob sizes reproduce the pages' byte counts.

    GLM-5.2 MXFP4 expert stride 20.05 MB (windlass README, fetch analysis: 336 x 20.05 MB)
    = 3 * 6144 * 2048 * (1/2 + 1/32); GLM-5.3 MXFP4 d=4096, f=2048 gives 13,369,344 B;
    43 * 288 of those at NVFP4-like 1/16 scale density give the 163.3 GiB of experts of
    "A hot expert cache ...", section "Try it".
    """
    assert oracle.blob_stride(6144, 2048, oracle.MXFP4) == 20_054_016
    assert oracle.blob_stride(4096, 2048, oracle.MXFP4) == 13_369_344
    assert oracle.blob_stride(256, 128, oracle.MXFP4) == 52_224
    assert oracle.blob_stride(6144, 2048, oracle.NVFP4) == 21_233_920
    gib = 43 * 288 * 3 * 4096 * 2048 * (0.5 + 1 / 16) / 2**30
    assert abs(gib - 163.3) < 0.05
