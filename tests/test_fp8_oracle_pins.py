"""Pins of the fp8 weight oracle against what fixes it from outside: the OCP E4M3
format's own closed forms, torch's float8_e4m3fn conversions (a library routine), and
the quantiser's invariants (every block reaches the largest code; each weight is
within half a step of the e4m3 grid at its scale)."""
import numpy as np
import pytest
import torch

from oracle import fp8_oracle as F

pytestmark = pytest.mark.filterwarnings("ignore")


def test_decode_closed_forms():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x80: -0.0}
    for c, v in cases.items():
        got = F.e4m3_decode(np.array([c]))[0]
        assert got == v and np.signbit(got) == np.signbit(v), hex(c)
    assert np.isnan(F.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    pos = F.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)           # codes 0x00..0x7E ascend strictly


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes.numpy())
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.isnan(ref).sum() == 2


def test_encode_ties_to_even_and_saturates():
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (17.0, 0x58), (2.0 ** -10, 0x00),
             (1.5 * 2.0 ** -10, 0x01), (464.0, 0x7E), (500.0, 0x7E), (-500.0, 0xFE),
             (-3.3, 0xC5), (0.0, 0x00), (-0.0, 0x80), (300.0, 0x79)]
    for v, c in cases:
        assert int(F.e4m3_encode(np.array([v]))[0]) == c, v


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    # exact midpoints between neighbouring grid values as well
    g = F.e4m3_decode(np.arange(0x7F))
    mids = ((g[1:] + g[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x), ref)


def test_quantizer_invariants():
    rng = np.random.default_rng(1)
    E, K, N = 3, 300, 200                       # partial blocks on both edges
    w = (rng.standard_normal((E, K, N)) * 0.02).astype(np.float32)
    w[1, 128:256, 0:128] = 0.0                  # an all-zero block
    w[2, 0:128, 128:] = 0.0
    w[2, 5, 130] = -3.0                         # a block with one nonzero value
    q, s = F.quantize(w)
    assert q.shape == w.shape and q.dtype == np.uint8 and s.shape == (E, 3, 2)
    vals = F.e4m3_decode(q)
    for e in range(E):
        for i in range(3):
            for j in range(2):
                blk = w[e, i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
                vb = vals[e, i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
                amax = np.abs(blk).max()
                if amax == 0:
                    assert s[e, i, j] == 1.0 and np.all(vb == 0)
                else:
                    assert s[e, i, j] == np.float32(amax) / np.float32(448)
                    assert np.abs(vb).max() == 448.0      # the largest weight maps to 448
    assert int(q[2, 5, 130]) == 0xFE                  # -3.0 / (3/448) = -448
    # every weight is within half an e4m3 step (at its magnitude) of code * scale
    deq = F.dequantize(q, s)
    full = np.repeat(np.repeat(s.astype(np.float64), 128, 1), 128, 2)[:, :K, :N]
    r = np.abs(w.astype(np.float64) / full)
    step = np.where(r < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(r, 2.0 ** -6))) - 3))
    assert np.all(np.abs(deq - w) <= 0.5 * step * full * (1 + 1e-6) + 1e-30)


def test_quantizer_catches_a_planted_scale_error():
    """The invariants above fail if the scale used amax / 240 (another fp8 maximum)."""
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((1, 128, 128))).astype(np.float32)
    q, s = F.quantize(w)
    bad_s = np.float32(np.abs(w).max()) / np.float32(240)
    assert s[0, 0, 0] != bad_s
    assert np.abs(F.e4m3_decode(q)).max() == 448.0
