"""Pins of the oracle's number-format codecs (CPU only).

The oracle's bf16 and e4m3fn codecs are written from the format definitions.
They are pinned here against (a) hand-worked tables from those definitions
(tests/golden/), and (b) independent library routines: torch's CPU casts to
bfloat16 and float8_e4m3fn, swept over every bf16 value, every rounding tie
and the values one fp32 ulp either side of each tie.
"""
import struct

import numpy as np
import pytest
import torch

import oracle


def f32_from_bits(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


def bits_f32(a):
    return np.ascontiguousarray(a, np.uint32).view(np.float32)


# --------------------------------------------------------------------------
# golden tables
# --------------------------------------------------------------------------

def test_e4m3fn_golden_decode(golden):
    rows = [r for r in golden("e4m3fn_ocp.txt") if r[0] == "decode"]
    assert len(rows) >= 10
    for _, pat, val in rows:
        got = oracle.e4m3fn_to_f32(int(pat, 16))
        if val == "nan":
            assert np.isnan(got), pat
        else:
            want = float(val)
            assert got == want and np.signbit(got) == np.signbit(want), (pat, got)


def test_e4m3fn_golden_encode(golden):
    rows = [r for r in golden("e4m3fn_ocp.txt") if r[0] == "encode"]
    assert len(rows) >= 10
    for _, inp, pat in rows:
        v = f32_from_bits(int(inp, 16))
        assert oracle.e4m3fn_rne(v) == int(pat, 16), (inp, hex(oracle.e4m3fn_rne(v)))


def test_bf16_golden(golden):
    rows = golden("bf16_rne.txt")
    assert len(rows) >= 10
    for inp, pat in rows:
        v = f32_from_bits(int(inp, 16))
        assert oracle.bf16_rne(v) == int(pat, 16), (inp, hex(oracle.bf16_rne(v)))


# --------------------------------------------------------------------------
# bf16 against torch's cast
# --------------------------------------------------------------------------

def _all_bf16_finite():
    b = np.arange(1 << 16, dtype=np.uint32)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF].astype(np.uint16)


def test_bf16_decode_all_patterns():
    b = _all_bf16_finite()
    got = oracle.bf16_to_f32_array(b)
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _bf16_ties_and_neighbours():
    """Every bf16 value, every midpoint between bf16 neighbours and one fp32
    ulp either side of each midpoint, both signs (as fp32 bit patterns)."""
    b = np.arange(0, 0x7F80, dtype=np.uint32)          # +0 .. largest finite
    exact = b << 16
    mid = exact + 0x8000                                # ties (incl. overflow tie)
    pats = np.concatenate([exact, mid, mid - 1, mid + 1])
    pats = pats[((pats >> 23) & 0xFF) != 0xFF]          # drop inf/nan patterns
    return np.concatenate([pats, pats | 0x80000000]).astype(np.uint32)


def test_bf16_rne_matches_torch_on_ties():
    v = bits_f32(_bf16_ties_and_neighbours())
    got = oracle.bf16_rne_array(v)
    want = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(v.view(np.uint32)[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_bf16_rne_matches_torch_random():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]
    v = bits_f32(u)
    got = oracle.bf16_rne_array(v)
    want = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# e4m3fn against torch's cast
# --------------------------------------------------------------------------

def test_e4m3fn_decode_all_patterns():
    b = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3fn_to_f32_array(b)
    want = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2                               # 0x7F and 0xFF only
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def _torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3fn_rne_all_bf16_in_range():
    """Every bf16 value with |v| <= 448 (includes every e4m3fn tie)."""
    b = _all_bf16_finite()
    v = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    v = v[np.abs(v) <= 448.0]
    assert v.size > 30000
    assert np.array_equal(oracle.e4m3fn_rne_array(v), _torch_e4m3(v))


def test_e4m3fn_rne_ties_and_neighbours():
    pos = oracle.e4m3fn_to_f32_array(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2.0                   # exact in fp32
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)
    u = m32.view(np.uint32)
    cand = np.concatenate([u, u - 1, u + 1, pos.astype(np.float32).view(np.uint32)])
    v = cand.view(np.float32)
    v = np.concatenate([v, -v])
    v = v[np.abs(v) <= 448.0]
    assert np.array_equal(oracle.e4m3fn_rne_array(v), _torch_e4m3(v))


def test_e4m3fn_rne_strided_sweep():
    """A strided sweep of every fp32 pattern in [0, 448] (both signs)."""
    top = 0x43E00000                                    # 448.0
    u = np.arange(0, top + 1, 4099, dtype=np.uint32)
    u = np.concatenate([u, np.array([top], np.uint32)])
    v = u.view(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.e4m3fn_rne_array(v), _torch_e4m3(v))


def test_e4m3fn_rne_error_bound():
    """|dec(enc(v)) - v| <= half a step of the e4m3fn grid at v."""
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(200_000) * rng.choice([1e-3, 1.0, 50.0], 200_000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    d = oracle.e4m3fn_to_f32_array(oracle.e4m3fn_rne_array(v)).astype(np.float64)
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = 2.0 ** (e - 3)
    assert np.all(np.abs(d - v) <= step / 2 + 0.0)


@pytest.mark.parametrize("v", [0.0, -0.0])
def test_e4m3fn_signed_zero(v):
    assert oracle.e4m3fn_rne(v) == (0x80 if np.signbit(v) else 0x00)
