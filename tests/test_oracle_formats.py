"""Pins of the oracle's number formats against library routines and brute force.

e4m3fn and bfloat16 are fixed by their published definitions (OCP 8-bit
floating point E4M3; bfloat16 = the top half of an IEEE binary32).  torch's
own CPU conversions serve as the library routine; a nearest-value search over
all codes serves as brute force.
"""
import numpy as np
import torch

import oracle


def _torch_e4m3_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_table_matches_library_decode():
    ours = oracle.e4m3_table()
    ref = _torch_e4m3_values()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.isnan(ours).sum() == 2            # S.1111.111 only


def test_e4m3_known_codes():
    t = oracle.e4m3_table()
    assert t[0x7E] == 448.0                     # largest finite
    assert t[0x38] == 1.0
    assert t[0x08] == 2.0 ** -6                 # smallest normal
    assert t[0x01] == 2.0 ** -9                 # smallest subnormal
    assert t[0xB8] == -1.0


def _brute_encode(v):
    """Nearest finite e4m3 value by exhaustive search; ties go to the even code."""
    t = oracle.e4m3_table()
    pos = t[:127]
    out = []
    for x in v:
        a = abs(x)
        dist = np.abs(pos - a)
        best = np.flatnonzero(dist == dist.min())
        code = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
        if np.signbit(x):
            code |= 0x80
        out.append(code)
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_brute_force():
    t = oracle.e4m3_table()[:127]
    mids = (t[1:] + t[:-1]) / 2
    eps = np.abs(mids) * 2.0 ** -20 + 2.0 ** -30
    rng = np.random.default_rng(0)
    v = np.concatenate([
        t, mids, mids + eps, mids - eps,
        rng.uniform(-500, 500, 4000), rng.uniform(-0.05, 0.05, 2000),
        np.array([448.0, 449.0, 463.9, 464.0, 465.0, 1e6, -1e6, 0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -11]),
    ])
    v = np.concatenate([v, -v])
    v = v.astype(np.float32).astype(np.float64)  # the oracle only ever encodes float32 values
    assert np.array_equal(oracle.e4m3_encode(v), _brute_encode(v))


def test_e4m3_encode_matches_library_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(200_000) * 60, rng.uniform(-448, 448, 200_000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), ref)


def test_e4m3_saturates_and_nan():
    c = oracle.e4m3_encode(np.array([500.0, -500.0, np.inf, np.nan]))
    assert list(c[:3]) == [0x7E, 0xFE, 0x7E]
    assert c[3] == 0x7F


def test_bf16_round_matches_library_on_float32():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    ours = oracle.bf16_round(f.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_round_midpoints():
    # every bf16 number and the midpoints around it (exactly representable in float32)
    hi = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (hi << 16).view(np.float32)
    mids = ((hi << 16) | 0x8000).view(np.float32)
    for arr in (vals, mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))):
        arr = np.concatenate([arr, -arr])
        ref = torch.from_numpy(arr.copy()).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(oracle.bf16_round(arr.astype(np.float64)), ref)


def test_bf16_round_float64_ties_not_rounded_twice():
    # 1 + 2^-8 is a bf16 tie (rounds to even: 1); 1 + 2^-8 + 2^-40 is above it (rounds up)
    # a float32 detour would round the second one to the tie and then to 1
    v = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8])
    assert list(oracle.bf16_round(v)) == [1.0, 1 + 2.0 ** -7, 1 + 4 * 2.0 ** -8]


def test_bf16_bits_roundtrip():
    rng = np.random.default_rng(3)
    v = oracle.bf16_round(rng.standard_normal(1000))
    assert np.array_equal(oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(v)), v)
