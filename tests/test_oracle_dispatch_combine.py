"""Pins of the oracle's dispatch (normal, low latency, fp8) and combine.

Dispatch is pinned by row identities (numpy gathers), by the relation between
the low-latency and normal layouts and by a hand-worked low-latency example.
The fp8 quantisation is pinned by its invariants (every nonzero group reaches
448, the error bound of e4m3fn rounding, sign and zero handling) and by a
torch formulation of the group quantisation on top of torch's own fp8 cast.
The combine is pinned by a hand-worked table, by the fp64 value of the same
sum (within one bf16 ulp), and by the exact round trips of the method
(unit weights give n_t * x; softmax weights over all-local slots give x).
"""
import numpy as np
import pytest
import torch

import oracle
from combine_dispatch_layout_amd import workloads as W


def small(name, **kw):
    return W.WORKLOADS[name].scaled(**kw)


# --------------------------------------------------------------------------
# normal and low-latency dispatch
# --------------------------------------------------------------------------

@pytest.mark.parametrize("w", [small("tiny"), small("dsv3_prefill", T=96, H=136),
                               small("zipf_prefill", T=80, H=64)],
                         ids=lambda w: w.name)
def test_dispatch_rows_are_source_rows(w):
    x = W.bf16_bits(W.make_hidden(w))
    ids = W.make_topk_ids(w).numpy()
    counts, seg, src2dst, reorder = oracle.layout(ids, w.expert_begin, w.L)
    R = int(seg[-1])
    P = oracle.dispatch(x, src2dst, w.k, R + 3, fill=0xFFFF)
    t_of_slot = np.arange(w.T * w.k) // w.k
    valid = src2dst >= 0
    assert np.array_equal(P[src2dst[valid]], x[t_of_slot[valid]])
    assert np.all(P[R:] == 0xFFFF)                       # nothing beyond R written


def test_dispatch_ll_golden(golden):
    g = {row[0]: row[1:] for row in golden("layout_worked.txt")}
    T, k, b, L, cap = (int(g[n][0]) for n in ("T", "k", "expert_begin", "L", "cap"))
    ids = np.array([int(v) for v in g["topk_ids"]], np.int32).reshape(T, k)
    x = (np.arange(T * 4, dtype=np.uint16) + 0x3F00).reshape(T, 4)
    B, mm, ll, ovf = oracle.dispatch_ll(x, ids, b, L, cap, fill=0xAAAA)
    assert ll.tolist() == [int(v) for v in g["ll_src2dst"]]
    assert mm.tolist() == [int(v) for v in g["masked_m"]]
    assert ovf == int(g["ll_overflow"][0])
    Bf = B.reshape(L * cap, 4)
    for i, r in enumerate(ll):
        if r >= 0:
            assert np.array_equal(Bf[r], x[i // k])


@pytest.mark.parametrize("cap_scale", [8, 1])
def test_dispatch_ll_matches_normal_layout(cap_scale):
    w = small("ll_decode", T=40, H=72)
    cap = w.T * cap_scale if cap_scale > 1 else 3          # 3 forces overflow
    x = W.bf16_bits(W.make_hidden(w))
    ids = W.make_topk_ids(w).numpy()
    counts, seg, src2dst, _ = oracle.layout(ids, w.expert_begin, w.L)
    B, mm, ll, ovf = oracle.dispatch_ll(x, ids, w.expert_begin, w.L, cap)
    assert np.array_equal(mm, np.minimum(counts, cap))
    assert ovf == int(np.any(counts > cap))
    P = oracle.dispatch(x, src2dst, w.k, int(seg[-1]))
    loc = ids.reshape(-1) - w.expert_begin
    Bf = B.reshape(w.L * cap, w.H)
    for i in range(w.T * w.k):
        if src2dst[i] < 0:
            assert ll[i] == -1
            continue
        e = loc[i]
        slot = src2dst[i] - seg[e]
        if slot >= cap:
            assert ll[i] == -1
        else:
            assert ll[i] == e * cap + slot
            assert np.array_equal(Bf[ll[i]], P[src2dst[i]])


# --------------------------------------------------------------------------
# fp8 group quantisation
# --------------------------------------------------------------------------

def torch_group_quant(xb, group=128):
    """Group quantisation expressed with torch ops and torch's own fp8 cast."""
    x = W.bits_to_bf16(xb).float().reshape(-1, group)
    a = x.abs().amax(dim=1, keepdim=True)
    s = a / 448.0
    v = torch.where(a > 0, (x / s).clamp(-448.0, 448.0), x)
    q = v.to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(-1).numpy(), s.reshape(-1).numpy()


def _rows(seed, rows, H, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return W.bf16_bits((torch.randn(rows, H, generator=g) * scale).to(torch.bfloat16))


@pytest.mark.parametrize("scale", [1.0, 1e-3, 300.0, 1e-38])
def test_quant_matches_torch_formulation(scale):
    x = _rows(5, 16, 1024, scale)
    counts, seg, src2dst, _ = oracle.layout(np.arange(16, dtype=np.int32)[:, None], 0, 16)
    Q, S = oracle.dispatch_fp8(x, src2dst, 1, 16)
    q, s = torch_group_quant(x)
    assert np.array_equal(Q.reshape(-1), q)
    assert np.array_equal(S.reshape(-1).view(np.uint32), s.view(np.uint32))


def test_quant_invariants():
    x = _rows(9, 64, 7168)
    G = 7168 // 128
    ids = np.arange(64, dtype=np.int32)[:, None]
    _, _, src2dst, _ = oracle.layout(ids, 0, 64)
    Q, S = oracle.dispatch_fp8(x, src2dst, 1, 64)
    xf = oracle.bf16_to_f32_array(x).reshape(64, G, 128).astype(np.float64)
    dq = oracle.e4m3fn_to_f32_array(Q).reshape(64, G, 128).astype(np.float64)
    s = S.reshape(64, G, 1).astype(np.float64)
    # scale is amax / 448 rounded to fp32
    a = np.abs(xf).max(axis=2, keepdims=True)
    assert np.allclose(s, a / 448.0, rtol=2 ** -23, atol=0)
    # every nonzero group has an element at +-448
    qg = Q.reshape(64, G, 128)
    assert np.all(np.any((qg == 0x7E) | (qg == 0xFE), axis=2))
    # dequantised values are within e4m3fn rounding of x (relative 2^-4 in the
    # normal range, 2^-10 * s in the subnormal range, plus fp32 division slack)
    err = np.abs(dq * s - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)
    # signs are kept
    assert np.all((np.signbit(dq) == np.signbit(xf)) | (xf == 0))


def test_quant_zero_group_and_exact_scale_one():
    z = np.zeros(128, np.uint16)
    z[::2] = 0x8000                                      # -0.0 in half the lanes
    q, s = oracle.quant_group_fp8(z)
    assert s == 0.0
    assert np.array_equal(q, np.where(z == 0x8000, 0x80, 0x00).astype(np.uint8))
    # a group whose amax is 448 has s == 1 and q == e4m3(x) element-wise
    x = _rows(2, 1, 128, 100.0).reshape(-1).copy()
    x[17] = 0x43E0                                        # bf16 448.0
    q, s = oracle.quant_group_fp8(x)
    assert s == 1.0
    assert np.array_equal(q, oracle.e4m3fn_rne_array(oracle.bf16_to_f32_array(x)))


def test_dispatch_fp8_rows_identical_per_token():
    w = small("fp8_dispatch", T=48, H=256)
    x = W.bf16_bits(W.make_hidden(w))
    ids = W.make_topk_ids(w).numpy()
    _, seg, src2dst, _ = oracle.layout(ids, w.expert_begin, w.L)
    R = int(seg[-1])
    Q, S = oracle.dispatch_fp8(x, src2dst, w.k, R)
    for t in range(w.T):
        rows = [d for d in src2dst[t * w.k:(t + 1) * w.k] if d >= 0]
        if not rows:
            continue
        q1, s1 = oracle.dispatch_fp8(x[t:t + 1], np.array([0], np.int32), 1, 1)
        for d in rows:
            assert np.array_equal(Q[d], q1[0]) and np.array_equal(S[d], s1[0])


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

def test_combine_golden(golden):
    g = golden("combine_worked.txt")
    head = {r[0]: r[1:] for r in g if r[0] in ("H", "k", "Y")}
    H, k = int(head["H"][0]), int(head["k"][0])
    Y = np.array([int(v, 16) for v in head["Y"]], np.uint16).reshape(-1, H)
    rows = [r for r in g if r[0] == "row"]
    T = len(rows)
    map_ = np.array([[int(r[2]), int(r[3])] for r in rows], np.int32).reshape(-1)
    w = np.array([[float(r[4]), float(r[5])] for r in rows], np.float32)
    want = np.array([[int(r[6], 16), int(r[7], 16)] for r in rows], np.uint16)
    got = oracle.combine(Y, map_, w, T, k)
    assert np.array_equal(got, want), (got, want)


def bf16_ulp(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("w", [small("tiny"), small("dsv3_prefill", T=64, H=512),
                               small("zipf_prefill", T=64, H=256)],
                         ids=lambda w: w.name)
def test_combine_within_one_ulp_of_fp64(w):
    ids = W.make_topk_ids(w).numpy()
    wt = W.make_topk_weights(w).numpy()
    _, seg, src2dst, _ = oracle.layout(ids, w.expert_begin, w.L)
    R = int(seg[-1])
    g = torch.Generator().manual_seed(77)
    Y = W.bf16_bits(torch.randn(R, w.H, generator=g).to(torch.bfloat16))
    out = oracle.bf16_to_f32_array(oracle.combine(Y, src2dst, wt, w.T, w.k)).reshape(w.T, w.H)
    ref = oracle.combine_f64(Y, src2dst, wt, w.T, w.k)
    assert np.all(np.abs(out - ref) <= bf16_ulp(ref))
    # a real rounding error bound: half an ulp plus the fp32 chain's error
    y = oracle.bf16_to_f32_array(Y).reshape(R, w.H).astype(np.float64)
    mag = np.zeros_like(ref)
    for t in range(w.T):
        for j in range(w.k):
            d = src2dst[t * w.k + j]
            if d >= 0:
                mag[t] += abs(wt[t, j]) * np.abs(y[d])
    assert np.all(np.abs(out - ref) <= bf16_ulp(ref) / 2 + w.k * 2.0 ** -24 * mag)


def test_combine_unit_weights_is_count_times_x():
    """Unit weights: out = bf16(n_t * x_t), exact for n_t in {1, 2, 4, 8}."""
    w = small("zipf_prefill", T=64, H=128)
    x = W.make_hidden(w)
    xb = W.bf16_bits(x)
    ids = W.make_topk_ids(w).numpy()
    for n in (1, 2, 4, 8):
        sub = ids[:, :n].copy()
        _, seg, src2dst, _ = oracle.layout(sub, 0, w.L)
        P = oracle.dispatch(xb, src2dst, n, int(seg[-1]))
        out = oracle.combine(P, src2dst, np.ones((w.T, n), np.float32), w.T, n)
        want = W.bf16_bits((x.float() * n).to(torch.bfloat16))
        assert np.array_equal(out, want)


@pytest.mark.parametrize("name", ["tiny", "zipf_prefill"])
def test_combine_softmax_roundtrip_is_identity(name):
    """All experts local + softmax weights: combine(dispatch(x)) == x."""
    w = W.WORKLOADS[name]
    if w.T * w.H > 1 << 22:
        w = w.scaled(T=512, H=1024)
    x, ids, wt = W.make_inputs(w)
    xb = W.bf16_bits(x)
    _, seg, src2dst, _ = oracle.layout(ids.numpy(), 0, w.L)
    P = oracle.dispatch(xb, src2dst, w.k, int(seg[-1]))
    out = oracle.combine(P, src2dst, wt.numpy(), w.T, w.k)
    assert np.array_equal(out, xb)


def test_combine_ll_equals_normal_bitwise():
    w = small("ll_decode", T=64, H=256)
    x, ids, wt = W.make_inputs(w)
    xb = W.bf16_bits(x)
    _, seg, src2dst, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    P = oracle.dispatch(xb, src2dst, w.k, int(seg[-1]))
    B, mm, ll, ovf = oracle.dispatch_ll(xb, ids.numpy(), w.expert_begin, w.L, w.T * w.k)
    assert ovf == 0
    a = oracle.combine(P, src2dst, wt.numpy(), w.T, w.k)
    b = oracle.combine(B.reshape(-1, w.H), ll, wt.numpy(), w.T, w.k)
    assert np.array_equal(a, b)


def test_combine_empty():
    out = oracle.combine(np.zeros((0, 16), np.uint16), np.zeros(0, np.int32),
                         np.zeros((0, 8), np.float32), 0, 8)
    assert out.shape == (0, 16)
    out = oracle.combine(np.zeros((0, 16), np.uint16), np.full(6, -1, np.int32),
                         np.ones((3, 2), np.float32), 3, 2)
    assert np.all(out == 0)


def test_all_core_timing_build_matches_the_oracle():
    """The OpenMP build the benchmark times on every host core computes what
    the single-threaded oracle does, bit for bit (so its timing measures the
    same work): dispatch rows and combine outputs at several thread counts,
    with invalid slots, a token without a valid slot and a ragged T."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=301, H=640)
    x, ids, wts = W.make_inputs(w)
    ids[7, :] = -1                                  # a token with no valid slot
    xb = W.bf16_bits(x)
    _, seg, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(seg[-1])
    P = oracle.dispatch(xb, d, w.k, R)
    want = oracle.combine(P, d, wts.numpy(), w.T, w.k)
    for threads in (1, 3, 8):
        assert np.array_equal(oracle.omp_dispatch(xb, d, w.k, R, threads), P)
        assert np.array_equal(oracle.omp_combine(P, d, wts.numpy(), w.T, w.k, threads), want)
