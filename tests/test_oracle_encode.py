"""Pins of the oracle's f32 -> E4M3 encode (round to nearest even, sign-preserving zero,
saturating) against the decode round trip, exact midpoints, and torch's float8_e4m3fn cast."""
import numpy as np
import torch


def torch_enc(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_round_trip_every_code(orc):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = orc.e4m3_value(codes).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(vals), codes.astype(np.uint8))


def test_midpoints_round_to_even(orc):
    pos = orc.e4m3_value(np.arange(0x7F))
    for c in range(0x7E):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)
        assert float(mid) == (pos[c] + pos[c + 1]) / 2          # exact in f32
        even = c if c % 2 == 0 else c + 1
        below, above = np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))
        got = orc.e4m3_encode(np.array([mid, below, above, -mid], dtype=np.float32))
        assert list(got) == [even, c, c + 1, 0x80 | even], c


def test_special_values(orc):
    x = np.array([0.0, -0.0, -1e-40, 1e-40, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -11,
                  448.0, -448.0, 1000.0, -1e30, 464.0], dtype=np.float32)
    assert list(orc.e4m3_encode(x)) == [0x00, 0x80, 0x80, 0x00, 0x00, 0x80, 0x01,
                                        0x7E, 0xFE, 0x7E, 0xFE, 0x7E]


def test_strided_sweep_vs_torch(orc):
    # every 37th f32 bit pattern from 0 up to 448.0, both signs (~30.8M values)
    top = np.frombuffer(np.float32(448.0).tobytes(), dtype=np.uint32)[0]
    bits = np.arange(0, top + 1, 37, dtype=np.uint32)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    x = bits.view(np.float32)
    ours = orc.e4m3_encode(x)
    ref = torch_enc(x)
    bad = np.flatnonzero(ours != ref)
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r} ours={ours[bad[0]]:#x} torch={ref[bad[0]]:#x}"


def test_subnormal_region_vs_torch(orc):
    # every 7th f32 in [2^-12, 2^-5] (the E4M3 subnormals, the zero/2^-9 tie region and the first
    # normal binades) and every 997th f32 below 2^-12, both signs
    b = lambda v: int(np.frombuffer(np.float32(v).tobytes(), dtype=np.uint32)[0])
    bits = np.concatenate([np.arange(0, b(2.0 ** -12), 997, dtype=np.uint32),
                           np.arange(b(2.0 ** -12), b(2.0 ** -5) + 1, 7, dtype=np.uint32)])
    x = bits.view(np.float32)
    assert np.array_equal(orc.e4m3_encode(x), torch_enc(x))
    assert np.array_equal(orc.e4m3_encode(-x), torch_enc(-x))
