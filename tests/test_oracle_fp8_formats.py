"""Pins of the oracle's fp8 scale variants: power-of-two (UE8M0) scales,
column-major TMA-aligned layout, packed exponent bytes, and fp8 rows on the
low-latency path (CPU only).

UE8M0 scales are pinned by a hand-worked table (tests/golden/ue8m0_scales.txt),
by their defining inequalities (power of two, 448 p >= amax, minimal) and by
torch's own fp8 cast of the exact quotient x / p.  The layouts are pinned as
numpy index permutations of the row-major result; the low-latency rows by
the normal-mode rows at the same slots.
"""
import struct

import numpy as np
import pytest
import torch

import oracle
from combine_dispatch_layout_amd import workloads as W

UE, CM, PK = oracle.SCALE_UE8M0, oracle.SCALE_COLMAJOR, oracle.SCALE_PACKED


def f32_from_hex(h):
    return struct.unpack("<f", struct.pack("<I", int(h, 16)))[0]


def test_ue8m0_golden(golden):
    rows = golden("ue8m0_scales.txt")
    assert len(rows) >= 6
    for amax_hex, p, byte in rows:
        a = f32_from_hex(amax_hex)
        grp = np.zeros(128, np.uint16)
        grp[5] = int(amax_hex, 16) >> 16                      # bf16 pattern of amax
        assert oracle.bf16_to_f32(int(grp[5])) == a
        q, pv, e = oracle.quant_group_fp8_ue8m0(grp)
        assert pv == np.float32(float(p)) and e + 127 == int(byte), (amax_hex, pv, e)


def rand_groups(seed, n, scale):
    g = torch.Generator().manual_seed(seed)
    return W.bf16_bits((torch.randn(n, 128, generator=g) * scale).to(torch.bfloat16))


@pytest.mark.parametrize("scale", [1e-38, 1e-6, 1.0, 300.0, 1e30])
def test_ue8m0_definition_and_torch_cast(scale):
    xb = rand_groups(int(np.log2(scale) + 200), 64, scale)
    for grp in xb:
        q, p, e = oracle.quant_group_fp8_ue8m0(grp)
        x = oracle.bf16_to_f32_array(grp).astype(np.float64)
        a = np.abs(x).max()
        assert p == 2.0 ** e and e >= -127
        assert 448.0 * p >= a
        assert e == -127 or 224.0 * p < a                      # minimal
        want = torch.from_numpy((x / p).astype(np.float32)).to(torch.float8_e4m3fn)
        assert np.array_equal(q, want.view(torch.uint8).numpy())


def test_ue8m0_zero_group():
    z = np.zeros(128, np.uint16)
    z[1::2] = 0x8000
    q, p, e = oracle.quant_group_fp8_ue8m0(z)
    assert e == -127
    assert np.array_equal(q, np.where(z == 0x8000, 0x80, 0).astype(np.uint8))


def setup_rows(T=37, H=512, L=6, k=3, seed=3):
    w = W.Workload("fmt", T=T, H=H, E=L, L=L, k=k, seed_base=seed)
    x = W.bf16_bits(W.make_hidden(w))
    ids = W.make_topk_ids(w).numpy()
    _, seg, d, _ = oracle.layout(ids, 0, L)
    return x, ids, d, int(seg[-1]), H // 128


@pytest.mark.parametrize("flags", [CM, UE | CM, UE | PK, UE | CM | PK])
def test_scale_layouts_are_permutations(flags):
    x, ids, d, R, G = setup_rows()
    rpm = 13                                                  # several matrices, ragged
    base_flags = flags & UE
    Q0, S0 = oracle.dispatch_fp8_fmt(x, d, 3, R, base_flags)
    s_rm = S0.view(np.float32).reshape(R, G)
    Q, S = oracle.dispatch_fp8_fmt(x, d, 3, R, flags, rows_per_mat=rpm, fill=0xEE)
    assert np.array_equal(Q, Q0)                              # payload is layout independent
    nmat = -(-R // rpm)
    ld = -(-rpm // 4) * 4
    if flags & PK:
        words = -(-G // 4)
        exp_bytes = (np.log2(s_rm).astype(np.int64) + 127).astype(np.uint8)
        assert np.all(2.0 ** (exp_bytes.astype(np.int64) - 127) == s_rm)
        padded = np.full((R, words * 4), 0xEE, np.uint8)
        padded[:, :G] = exp_bytes
        if flags & CM:
            got = S.reshape(nmat, words, ld, 4)
            for row in range(R):
                mat, r = divmod(row, rpm)
                assert np.array_equal(got[mat, :, r, :].reshape(-1)[:G], exp_bytes[row])
        else:
            assert np.array_equal(S.reshape(R, words * 4)[:, :G], exp_bytes)
    else:
        got = S.view(np.float32).reshape(nmat, G, ld)
        want = np.full((nmat * rpm, G), np.nan, np.float32)
        want[:R] = s_rm
        want = want.reshape(nmat, rpm, G).transpose(0, 2, 1)
        assert np.array_equal(got[:, :, :rpm].view(np.uint32)[~np.isnan(want)],
                              want.view(np.uint32)[~np.isnan(want)])
        assert np.all(S.reshape(nmat, G, ld, 4)[:, :, rpm:, :] == 0xEE)   # alignment padding


@pytest.mark.parametrize("flags", [0, UE, CM, UE | CM | PK])
def test_ll_fp8_rows_match_normal_rows(flags):
    x, ids, d, R, G = setup_rows(T=50, L=5, k=2)
    cap = 12                                                  # some experts overflow
    Q, S, mm, ll, ovf = oracle.dispatch_ll_fp8(x, ids, 0, 5, cap, flags, fill=0xEE)
    _, mm0, ll0, ovf0 = oracle.dispatch_ll(x, ids, 0, 5, cap)
    assert np.array_equal(mm, mm0) and np.array_equal(ll, ll0) and ovf == ovf0 == 1
    Qn, Sn = oracle.dispatch_fp8_fmt(x, ll, 2, 5 * cap, flags, rows_per_mat=cap, fill=0xEE)
    assert np.array_equal(Q.reshape(5 * cap, -1), Qn) and np.array_equal(S, Sn)


# --------------------------------------------------------------------------
# per-tensor fp8 cast (the w8a8 permuted buffer)
# --------------------------------------------------------------------------

def test_tensor_cast_golden(golden):
    rows = golden("fp8_tensor_cast.txt")
    assert len(rows) >= 15
    for xb, s, q in rows:
        got = oracle.cast_fp8_tensor(np.array([int(xb, 16)], np.uint16), float(s))
        assert int(got[0]) == int(q, 16), (xb, s)


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]                                    # no inf / NaN


@pytest.mark.parametrize("s", [1.0, 2.0, 0.25, 0.37, 3.0, 1e-3, 2.0 ** -10, 1e4, 0.0123])
def test_tensor_cast_matches_torch_on_every_bf16(s):
    """Every finite bf16 value against torch's CPU float32 division, clamp and
    float8_e4m3fn cast (round to nearest even, sign kept on zero)."""
    b = _all_finite_bf16()
    x = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float()
    want = (x / torch.tensor(s, dtype=torch.float32)).clamp(-448.0, 448.0) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.cast_fp8_tensor(b, s), want)


def test_tensor_dispatch_rows():
    """Every destination row of a token carries the token's cast row; other
    rows keep the fill."""
    w = W.WORKLOADS["tiny"]
    x, ids, _ = W.make_inputs(w)
    xb = W.bf16_bits(x)
    _, seg, d, _ = oracle.layout(ids.numpy(), 0, w.L)
    R = int(seg[-1])
    Q = oracle.dispatch_fp8_tensor(xb, d, w.k, R + 2, scale=0.5, fill=0xEE)
    q = oracle.cast_fp8_tensor(xb, 0.5)
    for i in range(w.T * w.k):
        if d[i] >= 0:
            assert np.array_equal(Q[d[i]], q[i // w.k])
    assert np.all(Q[R:] == 0xEE)


def test_nonfinite_golden(golden):
    """The oracle's reading of NaN and infinity in the three fp8
    quantisations (amax skips NaN, an infinite amax gives an infinite or
    capped scale, a NaN quotient is the NaN code with x's sign), against a
    hand-worked table."""
    rows = golden("fp8_nonfinite.txt")
    assert len(rows) == 7
    for mode, xs, scale, codes in rows:
        x = np.array([int(v, 16) for v in xs.split(",")], np.uint16)
        want = np.array([int(v, 16) for v in codes.split(",")], np.uint8)
        if mode == "group":
            q, s = oracle.quant_group_fp8(x)
            assert np.float32(s).view(np.uint32) == int(scale, 16), (xs, np.float32(s).view(np.uint32))
        elif mode == "ue8m0":
            q, p, e = oracle.quant_group_fp8_ue8m0(x)
            assert e == int(scale), (xs, e)
            assert p == 2.0 ** int(scale)
        else:
            q = oracle.cast_fp8_tensor(x, float(mode.split(":")[1]))
        assert np.array_equal(q, want), (mode, xs, [hex(v) for v in q])


def test_nonfinite_elements_leave_finite_groups_alone():
    """A NaN or infinity changes only its own group: the other groups of the
    row quantise exactly as they do without it (the definition is per group)."""
    g = torch.Generator().manual_seed(7)
    x = W.bf16_bits(torch.randn(4 * 128, generator=g).to(torch.bfloat16))
    base_q, base_s = [], []
    for g in range(4):
        q, s = oracle.quant_group_fp8(x[g * 128:(g + 1) * 128])
        base_q.append(q)
        base_s.append(s)
    for bad in (0x7FC0, 0xFF80, 0x7F80):
        y = x.copy()
        y[128 + 5] = bad
        for g in (0, 2, 3):
            q, s = oracle.quant_group_fp8(y[g * 128:(g + 1) * 128])
            assert np.array_equal(q, base_q[g]) and s == base_s[g]
