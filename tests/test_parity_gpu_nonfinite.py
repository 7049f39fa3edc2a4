"""GPU parity of the fp8 quantisations on rows holding NaN and infinity.

The pages say nothing of non-finite hidden states; the oracle states the
reading (a group's amax skips NaN, an infinite amax gives an infinite fp32
scale or a power-of-two scale capped at 2^127, a NaN quotient becomes the
e4m3fn NaN code with the sign of x, the per-tensor cast saturates +-inf).
Here the kernels must match that reading bit for bit on every fp8 path:
the unfused and fused normal dispatches in every scale format, the
low-latency dispatches, and the per-tensor cast.  Groups
without a non-finite value in the same rows and waves must be unaffected.
"""
import numpy as np
import pytest
import torch

import combine_dispatch_layout_amd as cdl
import oracle
from combine_dispatch_layout_amd import workloads as W
from gpu_util import DEV, announce, status_word, u8

pytestmark = pytest.mark.gpu

UE, CM, PK = cdl.FP8_SCALE_UE8M0, cdl.FP8_SCALE_COLMAJOR, cdl.FP8_SCALE_PACKED
FORMATS = [0, UE, CM, UE | CM, UE | PK, UE | CM | PK]

# bf16 patterns planted into the rows: quiet and signalling-looking NaNs of
# both signs, both infinities
NAN_P, NAN_N, NAN_S, INF_P, INF_N = 0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80


def planted_rows(w, seed=5):
    """Hidden states of the workload with non-finite values planted in some
    groups of 128 (one NaN; an infinity; both infinities and a NaN; a group
    of only NaNs and zeros; an infinity among subnormals) of every third
    token, and one whole token of NaNs."""
    x, ids, wts = W.make_inputs(w)
    xb = W.bf16_bits(x).copy()
    G = w.H // 128
    rng = np.random.default_rng(seed)
    for t in range(0, w.T, 3):
        g = int(rng.integers(G))
        kind = t % 5
        base = g * 128
        if kind == 0:
            xb[t, base + int(rng.integers(128))] = (NAN_P, NAN_N, NAN_S)[t % 3]
        elif kind == 1:
            xb[t, base + int(rng.integers(128))] = INF_P if t % 2 else INF_N
        elif kind == 2:
            xb[t, base + 3] = INF_P
            xb[t, base + 70] = INF_N
            xb[t, base + 100] = NAN_N
        elif kind == 3:
            xb[t, base:base + 128] = 0
            xb[t, base + 1:base + 128:2] = NAN_N
            xb[t, base + 64] = 0x8000
        else:
            xb[t, base:base + 128] = 0x0001                    # subnormal bf16
            xb[t, base + 17] = INF_P
    xb[1, :] = NAN_P
    return W.bits_to_bf16(xb), xb, ids, wts


def filled(nbytes, fill=0xEE):
    return torch.full((max(nbytes, 1),), fill, dtype=torch.uint8, device=DEV)


def raw(t):
    return t.detach().contiguous().cpu().view(torch.uint8).numpy().reshape(-1)


@pytest.mark.parametrize("flags", FORMATS)
@pytest.mark.parametrize("T", [300, 4096])
def test_fp8_nonfinite_normal_paths(flags, T):
    """Unfused scatter, fused permute with the binding's workspace and with
    one of only the layout's size: every byte and scale as the oracle gives
    them."""
    w = W.WORKLOADS["fp8_dispatch"].scaled(T=T, H=1152 if T < 1000 else 7168)
    announce("fp8 non-finite normal T=%d flags=%d" % (T, flags))
    x, xb, ids, _ = planted_rows(w)
    _, s_, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    cap = int(s_[-1]) + 3
    Q, S = oracle.dispatch_fp8_fmt(xb, d, w.k, cap, flags, rows_per_mat=cap, fill=0xEE)
    assert np.any((Q & 0x7F) == 0x7F)                                   # NaN codes occur
    nbytes = cdl.fp8_scale_bytes(cap, w.H, flags, cap)
    xd, idd = x.to(DEV), ids.to(DEV)
    st = status_word()
    lay = cdl.dispatch_layout(idd, w.expert_begin, w.L)
    outs = []
    q = torch.zeros(cap, w.H, dtype=torch.uint8, device=DEV)
    sb = filled(nbytes)
    cdl.dispatch_fp8(xd, lay, out_q=q, out_scales=sb, status=st, scale_flags=flags)
    outs.append((q, sb))
    q = torch.zeros(cap, w.H, dtype=torch.uint8, device=DEV)
    sb = filled(nbytes)
    cdl.permute_fp8(xd, idd, w.expert_begin, w.L, out_q=q, out_scales=sb, status=st,
                    scale_flags=flags)
    outs.append((q, sb))
    q = torch.zeros(cap, w.H, dtype=torch.uint8, device=DEV)
    sb = filled(nbytes)
    ws = torch.empty(cdl.layout_workspace_size(w.T, w.k, w.L), dtype=torch.uint8, device=DEV)
    cdl.permute_fp8(xd, idd, w.expert_begin, w.L, out_q=q, out_scales=sb, status=st,
                    scale_flags=flags, workspace=ws)
    outs.append((q, sb))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i, (q, sb) in enumerate(outs):
        assert np.array_equal(u8(q), Q), "payload, call %d" % i
        assert np.array_equal(raw(sb), S), "scales, call %d" % i


@pytest.mark.parametrize("flags", [0, UE | CM | PK])
def test_fp8_nonfinite_low_latency(flags):
    """The low-latency fp8 dispatch, from a layout and in one call (rows of a
    small batch split over several waves)."""
    w = W.WORKLOADS["ll_decode"]
    announce("fp8 non-finite low latency flags=%d" % flags)
    x, xb, ids, _ = planted_rows(w, seed=9)
    cap = w.cap
    Q, S, mm, ll, ovf = oracle.dispatch_ll_fp8(xb, ids.numpy(), w.expert_begin, w.L, cap, flags,
                                               fill=0xEE)
    assert not ovf
    xd, idd = x.to(DEV), ids.to(DEV)
    lay = cdl.dispatch_layout(idd, w.expert_begin, w.L)
    q = torch.zeros(w.L, cap, w.H, dtype=torch.uint8, device=DEV)
    sb = filled(S.size)
    q, sb, gmm, gll = cdl.dispatch_ll_fp8(xd, lay, cap, scale_flags=flags, out_q=q, out_scales=sb)
    q2 = torch.zeros(w.L, cap, w.H, dtype=torch.uint8, device=DEV)
    sb2 = filled(S.size)
    _, q2, sb2, gmm2, gll2 = cdl.permute_ll_fp8(xd, idd, w.expert_begin, w.L, cap,
                                                scale_flags=flags, out_q=q2, out_scales=sb2)
    torch.cuda.synchronize()
    for qq, ss, m_, l_ in ((q, sb, gmm, gll), (q2, sb2, gmm2, gll2)):
        assert np.array_equal(m_.cpu().numpy(), mm) and np.array_equal(l_.cpu().numpy(), ll)
        assert np.array_equal(u8(qq).reshape(-1), Q.reshape(-1))
        assert np.array_equal(raw(ss), S)


@pytest.mark.parametrize("scale", [None, 0.5, 0.37])
def test_fp8_tensor_cast_nonfinite(scale):
    """Per-tensor cast: +-inf saturate, NaNs keep their sign, finite
    elements of the same chunks unchanged (the power-of-two scales take the
    multiply path, 0.37 the division)."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=700, H=1024)
    announce("fp8 tensor non-finite scale=%s" % scale)
    x, xb, ids, _ = planted_rows(w, seed=13)
    _, s_, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s_[-1])
    want = oracle.dispatch_fp8_tensor(xb, d, w.k, R + 2, 1.0 if scale is None else scale,
                                      fill=0xA5)
    assert np.any(want[:R] == 0x7F) and np.any(want[:R] == 0xFF)
    q = torch.full((R + 2, w.H), 0xA5, dtype=torch.uint8, device=DEV)
    sd = None if scale is None else torch.tensor([scale], dtype=torch.float32, device=DEV)
    st = status_word()
    cdl.permute_fp8_tensor(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, scale=sd, out_q=q[:R],
                           status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(u8(q), want)
