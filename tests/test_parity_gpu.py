"""GPU parity of the HIP path against the CPU oracle (MI355X only).

Every test calls the C ABI through the Python binding and compares with the
oracle on the same seeded inputs:
  * layout (counts, seg_indptr, src2dst, reorder_topk_ids): bit-exact;
  * normal / low-latency dispatch rows, masked_m, ll_src2dst: bit-exact;
  * fp8 payload bytes and fp32 scales: bit-exact;
  * combine: within one bf16 ulp (max |gpu - oracle| / |oracle| <= 7.9e-3,
    with an absolute allowance of 2^-22 * sum|w*y| where cancellation makes
    |oracle| tiny); the kernels follow the oracle's fp32 fma order, so the
    results are also expected to be bit-exact and that is asserted too.
Sizes span several layout tiles (1024 slots) with a ragged tail; the full
workload sizes are checked as well (in the launch configuration the
benchmark uses).
"""
import zlib

import numpy as np
import pytest
import torch

import combine_dispatch_layout_amd as cdl
import oracle
from combine_dispatch_layout_amd import workloads as W
from gpu_util import DEV, announce, bf16_filled, bits16, npy, status_word, u8

UE_, CM_, PK_ = cdl.FP8_SCALE_UE8M0, cdl.FP8_SCALE_COLMAJOR, cdl.FP8_SCALE_PACKED

pytestmark = pytest.mark.gpu

REL_TOL = 7.9e-3


def combine_close(got_bits, want_bits, mag):
    g = oracle.bf16_to_f32_array(got_bits).astype(np.float64)
    w = oracle.bf16_to_f32_array(want_bits).astype(np.float64)
    err = np.abs(g - w)
    ok = err <= np.maximum(REL_TOL * np.abs(w), 2.0 ** -22 * mag.reshape(-1))
    return bool(ok.all()), float((err / np.maximum(np.abs(w), 1e-30)).max(initial=0.0))


def magnitude(Ybits, map_, wts, T, k):
    """sum_j |w_j * y_j| per output element, in fp64 (for the cancellation
    allowance)."""
    H = Ybits.shape[-1]
    y = oracle.bf16_to_f32_array(Ybits).reshape(-1, H).astype(np.float64)
    mag = np.zeros((T, H))
    for j in range(k):
        r = map_.reshape(T, k)[:, j]
        ok = r >= 0
        mag[ok] += np.abs(wts[ok, j:j + 1].astype(np.float64)) * np.abs(y[r[ok]])
    return mag


def run_normal(w, x, ids, wts, canary_rows=4):
    """GPU: layout, dispatch into a canaried buffer, combine of the rows."""
    xd, idd, wd = x.to(DEV), ids.to(DEV), wts.to(DEV)
    lay = cdl.dispatch_layout(idd, w.expert_begin, w.L)
    R = lay.num_rows()
    buf = bf16_filled(R + canary_rows, w.H, 0x7F7F)
    st = status_word()
    cdl.dispatch(xd, lay, out=buf[:R], status=st)
    outbuf = bf16_filled(w.T + canary_rows, w.H, 0x7F7F)
    cdl.combine(buf[:R], lay.src2dst, wd, out=outbuf[:w.T], status=st)
    torch.cuda.synchronize()
    return lay, R, buf, outbuf, int(st.item())


def check_layout(lay, ids, b, L):
    c, s, d, r = oracle.layout(ids.numpy(), b, L)
    assert np.array_equal(npy(lay.counts), c)
    assert np.array_equal(npy(lay.seg_indptr), s)
    assert np.array_equal(npy(lay.src2dst), d)
    assert np.array_equal(npy(lay.reorder_topk_ids), r)
    return c, s, d, r


PARITY = [
    W.WORKLOADS["tiny"],
    W.WORKLOADS["dsv3_prefill"].scaled(T=1000),                 # 8 tiles, ragged
    W.WORKLOADS["zipf_prefill"].scaled(T=2000, H=1024),         # 16 tiles, skewed
    W.WORKLOADS["zipf_prefill"].scaled(T=300, H=4096),
    W.WORKLOADS["dsv3_prefill"].scaled(T=777, expert_begin=64, H=2048),  # rank 2 of 8
]


@pytest.mark.parametrize("w", PARITY, ids=lambda w: "%s_T%d_H%d_b%d" % (w.name, w.T, w.H, w.expert_begin))
def test_normal_path_parity(w):
    announce("normal %s T=%d H=%d b=%d" % (w.name, w.T, w.H, w.expert_begin))
    x, ids, wts = W.make_inputs(w)
    lay, R, buf, outbuf, st = run_normal(w, x, ids, wts)
    assert st == 0
    c, s, d, r = check_layout(lay, ids, w.expert_begin, w.L)
    xb = W.bf16_bits(x)
    P = oracle.dispatch(xb, d, w.k, R)
    got = bits16(buf)
    assert np.array_equal(got[:R], P)
    assert np.all(got[R:] == 0x7F7F)                          # canary rows untouched
    want = oracle.combine(P, d, wts.numpy(), w.T, w.k)
    out = bits16(outbuf)
    assert np.all(out[w.T:] == 0x7F7F)
    ok, worst = combine_close(out[:w.T], want, magnitude(P, d, wts.numpy(), w.T, w.k))
    assert ok, worst
    assert np.array_equal(out[:w.T], want)                   # same fp32 fma order


@pytest.mark.parametrize("w", [W.WORKLOADS["fp8_dispatch"].scaled(T=1000),
                               W.WORKLOADS["fp8_dispatch"].scaled(T=130, H=384, expert_begin=32)],
                         ids=lambda w: "T%d_H%d" % (w.T, w.H))
def test_fp8_dispatch_parity(w):
    announce("fp8 T=%d H=%d" % (w.T, w.H))
    x, ids, wts = W.make_inputs(w)
    lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L)
    R = lay.num_rows()
    G = w.H // 128
    q = torch.full((R + 2, w.H), 0xA5, dtype=torch.uint8, device=DEV)
    sc = torch.full((R + 2, G), -7.0, dtype=torch.float32, device=DEV)
    st = status_word()
    cdl.dispatch_fp8(x.to(DEV), lay, out_q=q[:R], out_scales=sc[:R], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    _, _, d, _ = check_layout(lay, ids, w.expert_begin, w.L)
    Q, S = oracle.dispatch_fp8(W.bf16_bits(x), d, w.k, R)
    gq, gs = u8(q), npy(sc)
    assert np.array_equal(gq[:R], Q)
    assert np.array_equal(gs[:R].view(np.uint32), S.view(np.uint32))
    assert np.all(gq[R:] == 0xA5) and np.all(gs[R:] == -7.0)


@pytest.mark.parametrize("k", [1, 3, 12, 48, 64])
def test_scatter_blocks_parity(k):
    """The scatters from a layout take their tokens from per-block lists of
    the tokens with a destination: blocks of min(128, 1024 / k) tokens (a
    multiple of 4; 128, 128, 84, 20 and 16 here), three full blocks and a
    ragged one.  bf16 and fp8 rows bit-exact, canary rows untouched."""
    tb = min(128, 1024 // k // 4 * 4)
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=3 * tb + 5, H=256, k=k)
    announce("scatter blocks k=%d T=%d" % (k, w.T))
    x, ids, _ = W.make_inputs(w)
    lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L)
    R = lay.num_rows()
    _, _, d, _ = check_layout(lay, ids, w.expert_begin, w.L)
    xd = x.to(DEV)
    buf = bf16_filled(R + 2, w.H, 0x7F7F)
    q = torch.full((R + 2, w.H), 0xA5, dtype=torch.uint8, device=DEV)
    sc = torch.full((R + 2, w.H // 128), -7.0, dtype=torch.float32, device=DEV)
    st = status_word()
    cdl.dispatch(xd, lay, out=buf[:R], status=st)
    cdl.dispatch_fp8(xd, lay, out_q=q[:R], out_scales=sc[:R], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = bits16(buf)
    assert np.array_equal(got[:R], oracle.dispatch(W.bf16_bits(x), d, k, R))
    assert np.all(got[R:] == 0x7F7F)
    Q, S = oracle.dispatch_fp8(W.bf16_bits(x), d, k, R)
    gq, gs = u8(q), npy(sc)
    assert np.array_equal(gq[:R], Q) and np.array_equal(gs[:R].view(np.uint32), S.view(np.uint32))
    assert np.all(gq[R:] == 0xA5) and np.all(gs[R:] == -7.0)


def test_fp8_every_bf16_value_with_unit_scale():
    """Groups whose amax is 448 have s = 1, so the GPU's e4m3 conversion sees
    every bf16 value in [-448, 448] unchanged: all ties, subnormals, signs."""
    announce("fp8 exhaustive bf16 through s=1 groups")
    b = np.arange(1 << 16, dtype=np.uint32)
    v = oracle.bf16_to_f32_array(b.astype(np.uint16))
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    vals = b[keep].astype(np.uint16)
    per = 127
    ngroups = -(-vals.size // per)
    pad = np.zeros(ngroups * per, np.uint16)
    pad[:vals.size] = vals
    rows = np.concatenate([pad.reshape(ngroups, per), np.full((ngroups, 1), 0x43E0, np.uint16)], 1)
    H = 128 * 8
    T = -(-ngroups // 8)
    xb = np.zeros((T * 8, 128), np.uint16)
    xb[:ngroups] = rows
    xb = xb.reshape(T, H)
    ids = torch.arange(T, dtype=torch.int32).reshape(T, 1)
    lay = cdl.dispatch_layout(ids.to(DEV), 0, T)
    q, s = cdl.dispatch_fp8(W.bits_to_bf16(xb).to(DEV), lay)
    torch.cuda.synchronize()
    _, _, d, _ = oracle.layout(ids.numpy(), 0, T)
    Q, S = oracle.dispatch_fp8(xb, d, 1, T)
    assert np.array_equal(u8(q), Q)
    assert np.array_equal(npy(s).view(np.uint32), S.view(np.uint32))
    assert np.all(S.reshape(-1)[:ngroups] == 1.0)


@pytest.mark.parametrize("E", [-120, -3, 0, 5, 100])
def test_fp8_ue8m0_every_bf16_value(E):
    """UE8M0 scales over every bf16 value: each group holds 127 values of
    [-448, 448] scaled by 2^E (rounded to bf16) and the anchor 448 * 2^E, so
    the group's power-of-two scale is 2^E and the conversion sees every
    quotient the unit-scale test sees (fewer where 2^E * v underflows bf16),
    at five exponents.  Codes and scales bit-exact."""
    announce("fp8 UE8M0 exhaustive bf16, scale 2^%d" % E)
    UE = cdl.FP8_SCALE_UE8M0
    b = np.arange(1 << 16, dtype=np.uint32)
    v = oracle.bf16_to_f32_array(b.astype(np.uint16))
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    scaled = (torch.from_numpy(v[keep].astype(np.float32)) * (2.0 ** E)).to(torch.bfloat16)
    vals = W.bf16_bits(scaled)
    anchor = W.bf16_bits((torch.tensor([448.0]) * (2.0 ** E)).to(torch.bfloat16))[0]
    per = 127
    ngroups = -(-vals.size // per)
    pad = np.zeros(ngroups * per, np.uint16)
    pad[:vals.size] = vals
    rows = np.concatenate([pad.reshape(ngroups, per), np.full((ngroups, 1), anchor, np.uint16)], 1)
    H = 128 * 8
    T = -(-ngroups // 8)
    xb = np.zeros((T * 8, 128), np.uint16)
    xb[:ngroups] = rows
    xb = xb.reshape(T, H)
    ids = torch.arange(T, dtype=torch.int32).reshape(T, 1)
    lay = cdl.dispatch_layout(ids.to(DEV), 0, T)
    q, s = cdl.dispatch_fp8(W.bits_to_bf16(xb).to(DEV), lay, scale_flags=UE)
    torch.cuda.synchronize()
    _, _, d, _ = oracle.layout(ids.numpy(), 0, T)
    Q, S = oracle.dispatch_fp8_fmt(xb, d, 1, T, UE, rows_per_mat=T)
    assert np.array_equal(u8(q), Q)
    assert np.array_equal(s.detach().contiguous().cpu().view(torch.uint8).numpy().reshape(-1), S.reshape(-1))
    sv = s.detach().cpu().numpy().reshape(-1)[:ngroups]
    assert np.all(sv == np.float32(2.0 ** E))


@pytest.mark.parametrize("cap_mode", ["full", "tight"])
def test_low_latency_parity(cap_mode):
    w = W.WORKLOADS["ll_decode"]
    if cap_mode == "tight":
        w = w.scaled(T=96, H=512, cap=3)                       # forces overflow
    announce("ll %s T=%d H=%d cap=%d" % (cap_mode, w.T, w.H, w.cap))
    x, ids, wts = W.make_inputs(w)
    xd, idd, wd = x.to(DEV), ids.to(DEV), wts.to(DEV)
    lay = cdl.dispatch_layout(idd, w.expert_begin, w.L)
    st = status_word()
    B = bf16_filled(w.L * w.cap, w.H, 0x7F7F).view(w.L, w.cap, w.H)
    B, mm, llmap = cdl.dispatch_ll(xd, lay, w.cap, out=B, status=st)
    out = cdl.combine(B, llmap, wd, status=st)
    torch.cuda.synchronize()
    xb = W.bf16_bits(x)
    OB, omm, oll, ovf = oracle.dispatch_ll(xb, ids.numpy(), w.expert_begin, w.L, w.cap,
                                           fill=0x7F7F)
    assert np.array_equal(npy(mm), omm)
    assert np.array_equal(npy(llmap), oll)
    assert (int(st.item()) & cdl.CDL_STATUS_LL_OVERFLOW) == (cdl.CDL_STATUS_LL_OVERFLOW if ovf else 0)
    assert (int(st.item()) & ~cdl.CDL_STATUS_LL_OVERFLOW) == 0
    # compare the written rows and the first padding rows of every expert
    gB = B.view(w.L * w.cap, w.H)
    for e in range(w.L):
        n = min(int(omm[e]) + 2, w.cap)
        rows = np.arange(e * w.cap, e * w.cap + n)
        assert np.array_equal(bits16(gB[torch.from_numpy(rows).to(DEV)]),
                              OB.reshape(-1, w.H)[rows])
    want = oracle.combine(OB.reshape(-1, w.H), oll, wts.numpy(), w.T, w.k)
    assert np.array_equal(bits16(out), want)


@pytest.mark.parametrize("case", ["full", "tight", "ragged_b32", "T0"])
def test_permute_ll_parity(case):
    """cdl_permute_ll (layout + padded scatter in one call) against the
    oracle's layout and low-latency dispatch."""
    w = W.WORKLOADS["ll_decode"]
    if case == "tight":
        w = w.scaled(T=96, H=512, cap=3)                       # forces overflow
    elif case == "ragged_b32":
        w = w.scaled(T=777, H=256, cap=300, expert_begin=32)   # several workgroups per token batch
    elif case == "T0":
        w = w.scaled(T=0, H=256)
    announce("permute_ll %s T=%d H=%d cap=%d" % (case, w.T, w.H, w.cap))
    ids = W.make_topk_ids(w)
    x = W.make_hidden(w) if w.T else torch.zeros(0, w.H, dtype=torch.bfloat16)
    st = status_word()
    B = bf16_filled(w.L * w.cap, w.H, 0x7F7F).view(w.L, w.cap, w.H)
    lay, B, mm, llmap = cdl.permute_ll(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, w.cap, out=B,
                                       status=st)
    torch.cuda.synchronize()
    check_layout(lay, ids, w.expert_begin, w.L)
    OB, omm, oll, ovf = oracle.dispatch_ll(W.bf16_bits(x), ids.numpy(), w.expert_begin, w.L, w.cap,
                                           fill=0x7F7F)
    assert np.array_equal(npy(mm), omm)
    assert np.array_equal(npy(llmap), oll)
    assert int(st.item()) == (cdl.CDL_STATUS_LL_OVERFLOW if ovf else 0)
    assert np.array_equal(bits16(B.view(w.L * w.cap, w.H)), OB.reshape(-1, w.H))


def test_graph_replay_low_latency_step():
    """cdl_permute_ll + cdl_combine captured in a HIP graph (no memset nodes:
    the library issues none): every replay, with eager work and
    synchronisations between replays, gives the eager result bit for bit."""
    w = W.WORKLOADS["ll_decode"]
    announce("graph replay ll step")
    x, ids, wts = W.make_inputs(w)
    xd, idd, wd = x.to(DEV), ids.to(DEV), wts.to(DEV)
    lay, B, mm, llm = cdl.permute_ll(xd, idd, w.expert_begin, w.L, w.cap)
    ref = cdl.combine(B, llm, wd)
    torch.cuda.synchronize()
    ref_bits, ref_mm, ref_llm = bits16(ref), npy(mm), npy(llm)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # warm-up on the capture stream
        _, B_w, _, llm_w = cdl.permute_ll(xd, idd, w.expert_begin, w.L, w.cap)
        cdl.combine(B_w, llm_w, wd)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay_g, B_g, mm_g, llm_g = cdl.permute_ll(xd, idd, w.expert_begin, w.L, w.cap)
        out_g = cdl.combine(B_g, llm_g, wd)
    for rep in range(4):
        out_g.fill_(1.0)                               # eager work between replays
        mm_g.fill_(-7)
        llm_g.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits16(out_g), ref_bits), rep
        assert np.array_equal(npy(mm_g), ref_mm), rep
        assert np.array_equal(npy(llm_g), ref_llm), rep
        check_layout(lay_g, ids, w.expert_begin, w.L)


@pytest.mark.parametrize("flags,cap,T,own_ws", [(0, 1024, 128, True), (UE_ | CM_ | PK_, 1024, 128, True),
                                                (UE_ | CM_ | PK_, 1024, 128, False),
                                                (UE_ | CM_, 5, 100, True), (UE_ | CM_, 5, 100, False),
                                                (CM_, 256, 2500, True), (0, 256, 2500, True)])
def test_permute_ll_fp8_parity(flags, cap, T, own_ws):
    """One-call LL fp8 dispatch; T = 2500 takes the count kernel and 4 tokens
    per permute workgroup (the fp8 plan).  The binding's own workspace, or
    (own_ws = False) one of the layout's size passed in."""
    w = W.WORKLOADS["ll_decode"]
    if T != w.T:
        w = w.scaled(T=T, H=512)
    announce("permute_ll fp8 flags=%d cap=%d" % (flags, cap))
    x, ids, wts = W.make_inputs(w)
    Q, S, mm, ll, ovf = oracle.dispatch_ll_fp8(W.bf16_bits(x), ids.numpy(), w.expert_begin, w.L,
                                               cap, flags, fill=0xEE)
    q = torch.zeros(w.L, cap, w.H, dtype=torch.uint8, device=DEV)
    sb = torch.full((max(S.size, 1),), 0xEE, dtype=torch.uint8, device=DEV)
    st = status_word()
    ws = None if own_ws else torch.empty(cdl.layout_workspace_size(w.T, w.k, w.L),
                                         dtype=torch.uint8, device=DEV)
    lay, q, sb, gmm, gll = cdl.permute_ll_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, cap,
                                              scale_flags=flags, out_q=q, out_scales=sb, status=st,
                                              workspace=ws)
    torch.cuda.synchronize()
    check_layout(lay, ids, w.expert_begin, w.L)
    assert np.array_equal(npy(gmm), mm) and np.array_equal(npy(gll), ll)
    assert (int(st.item()) != 0) == bool(ovf)
    assert np.array_equal(u8(q).reshape(-1), Q.reshape(-1))
    assert np.array_equal(sb.cpu().numpy().reshape(-1)[:S.size], S)


@pytest.mark.parametrize("T,k", [(1, 8), (64, 8), (128, 8), (129, 8), (600, 2), (512, 8), (513, 8),
                                 (1024, 4), (1025, 4), (2048, 2), (2049, 2)])
def test_layout_self_count_threshold(T, k):
    """Batches just below and above the size (T*k = 4096) up to which every
    layout workgroup counts all slots itself, and the sizes where its tokens
    per workgroup change, give the oracle's layout and rows."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=T, k=k, H=64)
    announce("self-count threshold T=%d k=%d" % (T, k))
    x, ids, wts = W.make_inputs(w)
    lay = cdl.dispatch_layout(ids.to(DEV), 0, w.L)
    lay2, rows = cdl.permute(x.to(DEV), ids.to(DEV), 0, w.L)
    torch.cuda.synchronize()
    _, s_, d, _ = check_layout(lay, ids, 0, w.L)
    check_layout(lay2, ids, 0, w.L)
    R = int(s_[-1])
    assert np.array_equal(bits16(rows[:R]), oracle.dispatch(W.bf16_bits(x), d, k, R))


def test_full_size_dsv3_prefill():
    """The benchmark's workload at full size: everything compared."""
    w = W.WORKLOADS["dsv3_prefill"]
    announce("full dsv3_prefill")
    x, ids, wts = W.make_inputs(w)
    lay, R, buf, outbuf, st = run_normal(w, x, ids, wts, canary_rows=2)
    assert st == 0
    _, _, d, _ = check_layout(lay, ids, w.expert_begin, w.L)
    xb = W.bf16_bits(x)
    P = oracle.dispatch(xb, d, w.k, R)
    assert np.array_equal(bits16(buf[:R]), P)
    want = oracle.combine(P, d, wts.numpy(), w.T, w.k)
    assert np.array_equal(bits16(outbuf[:w.T]), want)


def test_full_size_zipf_prefill_sampled():
    """T=16384, H=4096, E=L=128, Zipf experts: exact layout, sampled rows and
    sampled combined tokens (the oracle computes them one by one), and the
    all-local softmax round trip combine(dispatch(x)) == x everywhere."""
    w = W.WORKLOADS["zipf_prefill"]
    announce("full zipf_prefill")
    x, ids, wts = W.make_inputs(w)
    lay, R, buf, outbuf, st = run_normal(w, x, ids, wts, canary_rows=2)
    assert st == 0 and R == w.T * w.k
    _, _, d, _ = check_layout(lay, ids, w.expert_begin, w.L)
    xb = W.bf16_bits(x)
    rng = np.random.default_rng(1)
    slots = rng.choice(w.T * w.k, 4096, replace=False)
    rows = d[slots]
    got = bits16(buf[torch.from_numpy(rows.astype(np.int64)).to(DEV)])
    assert np.array_equal(got, xb[slots // w.k])
    toks = np.sort(rng.choice(w.T, 512, replace=False))
    sub_map = d.reshape(w.T, w.k)[toks]
    sub_rows = np.unique(sub_map[sub_map >= 0])
    remap = {int(r): i for i, r in enumerate(sub_rows)}
    # the oracle's row r is x[token of r]; build the sampled rows directly
    src_tok = np.empty(R, np.int64)
    src_tok[d] = np.arange(w.T * w.k) // w.k
    sub_y = xb[src_tok[sub_rows]]
    m2 = np.array([remap[int(r)] if r >= 0 else -1 for r in sub_map.reshape(-1)], np.int32)
    want = oracle.combine(sub_y, m2, wts.numpy()[toks], toks.size, w.k)
    out = bits16(outbuf[:w.T])
    assert np.array_equal(out[toks], want)
    assert np.array_equal(out, xb)                            # softmax round trip


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def test_empty_batch():
    announce("T=0")
    ids = torch.zeros(0, 8, dtype=torch.int32, device=DEV)
    lay = cdl.dispatch_layout(ids, 0, 32)
    torch.cuda.synchronize()
    assert npy(lay.counts).tolist() == [0] * 32
    assert npy(lay.seg_indptr).tolist() == [0] * 33
    x = torch.zeros(0, 256, dtype=torch.bfloat16, device=DEV)
    P = cdl.dispatch(x, lay)
    assert P.shape == (0, 256)
    out = cdl.combine(P, lay.src2dst, torch.zeros(0, 8, device=DEV))
    assert out.shape == (0, 256)
    B, mm, ll = cdl.dispatch_ll(x, lay, 4)
    torch.cuda.synchronize()
    assert npy(mm).tolist() == [0] * 32 and ll.numel() == 0


@pytest.mark.parametrize("case", ["T1_k1", "all_invalid", "one_hot_expert", "duplicates",
                                  "odd_H", "H8", "max_L", "max_k"])
def test_edge_cases(case):
    announce("edge " + case)
    g = torch.Generator().manual_seed(zlib.crc32(case.encode()))
    b, L, E = 0, 16, 64
    T, k, H = 300, 4, 256
    if case == "T1_k1":
        T, k = 1, 1
        ids = torch.tensor([[3]], dtype=torch.int32)
    elif case == "all_invalid":
        ids = torch.randint(L, E, (T, k), generator=g, dtype=torch.int32)
        ids[::7] = -1
    elif case == "one_hot_expert":
        ids = torch.full((T, k), -1, dtype=torch.int32)
        ids[:, 0] = 5
    elif case == "duplicates":
        ids = torch.randint(-1, L + 2, (T, k), generator=g, dtype=torch.int32)
        ids[:, 1] = ids[:, 0]
    elif case == "odd_H":
        H = 100
        ids = torch.randint(-1, E + 1, (T, k), generator=g, dtype=torch.int32)
    elif case == "H8":
        H = 8
        ids = torch.randint(0, L, (T, k), generator=g, dtype=torch.int32)
    elif case == "max_L":
        T, k, L, E, H = 700, 8, 2048, 2048, 64
        ids = torch.multinomial(torch.ones(T, E), k, generator=g).to(torch.int32)
    elif case == "max_k":
        T, k, L, E, H = 200, 64, 128, 128, 128
        ids = torch.multinomial(torch.ones(T, E), k, generator=g).to(torch.int32)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    wts = torch.randn(T, k, generator=g).softmax(-1)
    w = W.Workload(case, T=T, H=H, E=E, L=L, k=k, expert_begin=b)
    lay, R, buf, outbuf, st = run_normal(w, x, ids, wts)
    assert st == 0
    _, _, d, _ = check_layout(lay, ids, b, L)
    P = oracle.dispatch(W.bf16_bits(x), d, k, R)
    got = bits16(buf)
    assert np.array_equal(got[:R], P) and np.all(got[R:] == 0x7F7F)
    want = oracle.combine(P, d, wts.numpy(), T, k)
    out = bits16(outbuf)
    assert np.array_equal(out[:T], want) and np.all(out[T:] == 0x7F7F)


def test_rows_overflow_flag_and_no_out_of_bounds_write():
    announce("dispatch cap_rows < R")
    w = W.WORKLOADS["tiny"]
    x, ids, wts = W.make_inputs(w)
    lay = cdl.dispatch_layout(ids.to(DEV), 0, w.L)
    R = lay.num_rows()
    cap = R // 2
    buf = bf16_filled(R, w.H, 0x7F7F)
    st = status_word()
    cdl.dispatch(x.to(DEV), lay, out=buf[:cap], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == cdl.CDL_STATUS_ROWS_OVERFLOW
    _, _, d, _ = oracle.layout(ids.numpy(), 0, w.L)
    P = oracle.dispatch(W.bf16_bits(x), d, w.k, R)
    got = bits16(buf)
    assert np.array_equal(got[:cap], P[:cap]) and np.all(got[cap:] == 0x7F7F)


def test_combine_map_range_flag():
    announce("combine map beyond y_rows")
    y = torch.randn(4, 64).to(torch.bfloat16).to(DEV)
    m = torch.tensor([0, 9, 3, -1], dtype=torch.int32, device=DEV)
    wts = torch.ones(2, 2, device=DEV)
    st = status_word()
    out = cdl.combine(y, m, wts, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == cdl.CDL_STATUS_MAP_RANGE
    assert np.array_equal(bits16(out[0]), bits16(y[0]))
    assert np.array_equal(bits16(out[1]), bits16(y[3]))


@pytest.mark.parametrize("H", [7168, 200])
def test_combine_timed_matches_combine(H):
    """cdl_combine_timed: the same bits as cdl_combine (vector and element
    paths), and its launch events hold the kernel's duration."""
    import ctypes
    announce("combine timed H=%d" % H)
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=900, H=H)
    x, ids, wts = W.make_inputs(w)
    _, s_, d, _ = oracle.layout(ids.numpy(), 0, w.L)
    R = int(s_[-1])
    y = torch.randn(R, H, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    m = torch.from_numpy(d).to(DEV)
    wd = wts.to(DEV)
    ref = cdl.combine(y, m, wd)
    out = torch.empty(w.T, H, dtype=torch.bfloat16, device=DEV)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    rc = cdl.library().cdl_combine_timed(
        P(y.data_ptr()), R, H, P(m.data_ptr()), P(wd.data_ptr()), w.T, w.k, P(out.data_ptr()),
        None, P(e0.cuda_event), P(e1.cuda_event), P(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(bits16(out), bits16(ref))
    want = oracle.combine(W.bf16_bits(y.cpu()), d, wts.numpy(), w.T, w.k)
    assert np.array_equal(bits16(out), want)
    assert e0.elapsed_time(e1) > 0


def test_combine_extreme_values():
    """Combine on rows of bf16 subnormals, values near the bf16 maximum (sums
    that overflow to infinity), exact cancellations and negative or large
    weights: bit-exact against the oracle (fp32 fma chain, subnormals kept,
    one bf16 rounding)."""
    announce("combine extreme values")
    g = torch.Generator().manual_seed(31)
    T, k, H, R = 256, 4, 512, 600
    pats = []
    sub = torch.randint(1, 0x80, (R // 4, H), generator=g, dtype=torch.int32)          # +subnormals
    pats.append(sub | (torch.randint(0, 2, sub.shape, generator=g, dtype=torch.int32) << 15))
    big = torch.randint(0x7F00, 0x7F7F, (R // 4, H), generator=g, dtype=torch.int32)   # near max
    pats.append(big | (torch.randint(0, 2, big.shape, generator=g, dtype=torch.int32) << 15))
    nrm = W.bf16_bits(torch.randn(R // 4, H, generator=g).to(torch.bfloat16)).astype(np.int32)
    pats.append(torch.from_numpy(nrm))
    pats.append(torch.from_numpy(nrm) ^ 0x8000)                                         # negations
    ybits = torch.cat(pats).to(torch.int32).numpy().astype(np.uint16)
    y = W.bits_to_bf16(ybits)
    m = torch.randint(-1, R, (T, k), generator=g, dtype=torch.int32)
    # rows [R/2, 3R/4) hold normal values and rows [3R/4, R) their negations:
    # every third token adds a row and its negation with equal weights (exact 0)
    pick = torch.randint(0, R // 4, (T,), generator=g, dtype=torch.int32)
    m[::3, 0] = 2 * (R // 4) + pick[::3]
    m[::3, 1] = 3 * (R // 4) + pick[::3]
    m[::3, 2:] = -1
    w = torch.randn(T, k, generator=g) * 4.0
    w[::5] = 1.0
    w[1::7, 0] = -1.0
    w[::3, :2] = 1.0
    out = cdl.combine(y.to(DEV), m.reshape(-1).to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    want = oracle.combine(ybits, m.reshape(-1).numpy(), w.numpy(), T, k)
    got = bits16(out)
    assert np.array_equal(got, want)
    assert np.any((got & 0x7FFF) == 0x7F80)                                            # infinities reached
    assert np.any(((got & 0x7F80) == 0) & ((got & 0x7F) != 0))                          # subnormal results
    assert np.all(got[::3] == 0)                                                        # cancellations give +0


def test_fp8_rejects_ragged_groups():
    ids = torch.zeros(2, 1, dtype=torch.int32, device=DEV)
    lay = cdl.dispatch_layout(ids, 0, 1)
    with pytest.raises(cdl.CdlError):
        cdl.dispatch_fp8(torch.zeros(2, 200, dtype=torch.bfloat16, device=DEV), lay, rows=2)


def test_deterministic_repeats():
    announce("determinism zipf T=4000")
    w = W.WORKLOADS["zipf_prefill"].scaled(T=4000, H=512)
    x, ids, wts = W.make_inputs(w)
    a = run_normal(w, x, ids, wts)
    b = run_normal(w, x, ids, wts)
    assert np.array_equal(npy(a[0].src2dst), npy(b[0].src2dst))
    assert np.array_equal(bits16(a[2]), bits16(b[2]))
    assert np.array_equal(bits16(a[3]), bits16(b[3]))


# --------------------------------------------------------------------------
# fused permute (layout + scatter in one call)
# --------------------------------------------------------------------------

PERMUTE = PARITY + [W.WORKLOADS["dsv3_prefill"], W.WORKLOADS["ll_decode"].scaled(mode="normal"),
                    W.WORKLOADS["zipf_prefill"].scaled(T=5000, H=256),
                    # last workgroup only partly filled, expert 0 local: its
                    # past-the-end waves must neither load nor store a row
                    W.WORKLOADS["dsv3_prefill"].scaled(T=1001, H=512)]


@pytest.mark.parametrize("w", PERMUTE, ids=lambda w: "%s_T%d_H%d_b%d" % (w.name, w.T, w.H, w.expert_begin))
def test_permute_parity(w):
    announce("permute %s T=%d H=%d b=%d" % (w.name, w.T, w.H, w.expert_begin))
    x, ids, wts = W.make_inputs(w)
    c, s, d, r = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s[-1])
    cap = R + 1                                  # one spare row, then canaries
    buf = bf16_filled(cap + 3, w.H, 0x7F7F)
    st = status_word()
    lay, _ = cdl.permute(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out=buf[:cap], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    check_layout(lay, ids, w.expert_begin, w.L)
    P = oracle.dispatch(W.bf16_bits(x), d, w.k, R)
    got = bits16(buf)
    assert np.array_equal(got[:R], P)
    assert np.all(got[R:] == 0x7F7F)


def test_full_size_zipf_prefill_permute_sampled():
    """The Zipf workload at full size through the fused permute and the
    combine, as timed: exact layout, sampled rows, and the all-local softmax
    round trip combine(permute(x)) == x for every token."""
    w = W.WORKLOADS["zipf_prefill"]
    announce("full zipf_prefill permute")
    x, ids, wts = W.make_inputs(w)
    st = status_word()
    lay, rows = cdl.permute(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, status=st)
    out = cdl.combine(rows, lay.src2dst, wts.to(DEV), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    _, s_, d, _ = check_layout(lay, ids, w.expert_begin, w.L)
    assert int(s_[-1]) == w.T * w.k
    xb = W.bf16_bits(x)
    slots = np.random.default_rng(2).choice(w.T * w.k, 4096, replace=False)
    got = bits16(rows[torch.from_numpy(d[slots].astype(np.int64)).to(DEV)])
    assert np.array_equal(got, xb[slots // w.k])
    assert np.array_equal(bits16(out), xb)


@pytest.mark.parametrize("fp8", [False, True])
def test_permute_many_superblocks(fp8):
    """2^19 tokens of top-8 over 32 of 256 experts: hundreds of superblocks,
    so every permute workgroup reads its superblock counts and recounts its
    superblock's earlier slots in several rounds; layout, rows (and for bf16
    the combine) against the oracle."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=1 << 19, H=128 if fp8 else 64)
    announce("permute many superblocks T=%d fp8=%d" % (w.T, fp8))
    x, ids, wts = W.make_inputs(w)
    c, s_, d, r = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s_[-1])
    st = status_word()
    xb = W.bf16_bits(x)
    if fp8:
        lay, q, sc = cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, rows=R,
                                     status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        check_layout(lay, ids, w.expert_begin, w.L)
        Q, S = oracle.dispatch_fp8(xb, d, w.k, R)
        assert np.array_equal(u8(q), Q)
        assert np.array_equal(npy(sc).view(np.uint32), S.view(np.uint32))
        return
    lay, rows = cdl.permute(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, rows=R, status=st)
    out = cdl.combine(rows, lay.src2dst, wts.to(DEV), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    check_layout(lay, ids, w.expert_begin, w.L)
    P = oracle.dispatch(xb, d, w.k, R)
    assert np.array_equal(bits16(rows), P)
    assert np.array_equal(bits16(out), oracle.combine(P, d, wts.numpy(), w.T, w.k))


@pytest.mark.parametrize("dtype", [torch.float8_e4m3fn, torch.uint8, torch.float16])
def test_dispatch_rows_of_other_dtypes(dtype):
    """Rows already quantised per tensor (the pages keep the permuted buffer
    in fp8 then) or of any 1- or 2-byte type are dispatched bit for bit, by
    the fused permute and by the scatter from a layout."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=1000, H=512)
    announce("rows of dtype %s" % dtype)
    x, ids, wts = W.make_inputs(w)
    g = torch.Generator().manual_seed(77)
    raw = torch.randint(0, 256, (w.T, w.H), generator=g, dtype=torch.uint8)
    xd = raw.view(dtype) if dtype != torch.float16 else W.make_hidden(w).to(torch.float16)
    words = xd.view(torch.int16).numpy().view(np.uint16)       # the rows as 16-bit words
    _, s_, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s_[-1])
    want = oracle.dispatch(words, d, w.k, R)
    st = status_word()
    lay, rows = cdl.permute(xd.to(DEV), ids.to(DEV), w.expert_begin, w.L, rows=R, status=st)
    rows2 = cdl.dispatch(xd.to(DEV), lay, rows=R, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert rows.dtype == dtype and rows2.dtype == dtype and rows.shape == (R, w.H)
    for r in (rows, rows2):
        got = r.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("scale", [None, 0.5, 0.37, 3.0])
@pytest.mark.parametrize("w", [W.WORKLOADS["dsv3_prefill"].scaled(T=1000, H=512),
                               # an odd number of 16-byte chunks (the one-chunk
                               # path), and a last block of one pair per row
                               W.WORKLOADS["dsv3_prefill"].scaled(T=1000, H=520),
                               W.WORKLOADS["dsv3_prefill"].scaled(T=1000, H=1040),
                               W.WORKLOADS["tiny"],
                               W.WORKLOADS["ll_decode"].scaled(mode="normal", T=100, H=1024),
                               W.WORKLOADS["dsv3_prefill"]],
                         ids=lambda w: "%s_T%d_H%d" % (w.name, w.T, w.H))
def test_permute_fp8_tensor_parity(w, scale):
    """Per-tensor fp8 cast on the permute (the w8a8 buffer): no scale (1),
    a power of two, and two scales that need the division; hidden states
    scaled by 300 s so that some quotients saturate at +-448.  Rows
    bit-exact, canary rows untouched."""
    announce("permute fp8 tensor %s T=%d scale=%s" % (w.name, w.T, scale))
    x, ids, wts = W.make_inputs(w)
    x = (x.float() * (300.0 * (1.0 if scale is None else scale))).to(torch.bfloat16)
    xb = W.bf16_bits(x)
    _, s_, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s_[-1])
    want = oracle.dispatch_fp8_tensor(xb, d, w.k, R + 2, 1.0 if scale is None else scale,
                                      fill=0xA5)
    assert np.any(want[:R] == 0x7E) and np.any(want[:R] == 0xFE)        # saturated
    q = torch.full((R + 2, w.H), 0xA5, dtype=torch.uint8, device=DEV)
    sd = None if scale is None else torch.tensor([scale], dtype=torch.float32, device=DEV)
    st = status_word()
    lay, _ = cdl.permute_fp8_tensor(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, scale=sd,
                                    out_q=q[:R], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    check_layout(lay, ids, w.expert_begin, w.L)
    assert np.array_equal(u8(q), want)


def test_permute_fp8_tensor_rows_overflow():
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=300, H=256)
    announce("permute fp8 tensor cap < R")
    x, ids, _ = W.make_inputs(w)
    _, s_, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s_[-1])
    cap = R - 7
    want = oracle.dispatch_fp8_tensor(W.bf16_bits(x), d, w.k, R, fill=0xA5)
    q = torch.full((R, w.H), 0xA5, dtype=torch.uint8, device=DEV)
    st = status_word()
    cdl.permute_fp8_tensor(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q[:cap], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == cdl.CDL_STATUS_ROWS_OVERFLOW
    got = u8(q)
    assert np.array_equal(got[:cap], want[:cap]) and np.all(got[cap:] == 0xA5)


def test_permute_default_capacity_and_repeat():
    """rows defaults to T*k (no host sync); two calls give identical bits."""
    w = W.WORKLOADS["zipf_prefill"].scaled(T=3000, H=512)
    announce("permute default cap T=%d" % w.T)
    x, ids, wts = W.make_inputs(w)
    lay1, out1 = cdl.permute(x.to(DEV), ids.to(DEV), 0, w.L)
    lay2, out2 = cdl.permute(x.to(DEV), ids.to(DEV), 0, w.L)
    torch.cuda.synchronize()
    assert out1.shape[0] == w.T * w.k
    R = lay1.num_rows()
    assert torch.equal(lay1.src2dst, lay2.src2dst)
    assert torch.equal(out1[:R].view(torch.int16), out2[:R].view(torch.int16))
    _, s, d, _ = check_layout(lay1, ids, 0, w.L)
    assert np.array_equal(bits16(out1[:R]), oracle.dispatch(W.bf16_bits(x), d, w.k, R))


def test_layout_workspace_reuse_across_shapes():
    """One workspace, never initialised, serves a sequence of layouts and
    permutes of different shapes (including T = 0 and T = 1); every call
    matches the oracle."""
    shapes = [W.WORKLOADS["dsv3_prefill"], W.WORKLOADS["tiny"],
              W.WORKLOADS["zipf_prefill"].scaled(T=5000, H=256),
              W.WORKLOADS["dsv3_prefill"].scaled(T=0), W.WORKLOADS["ll_decode"],
              W.WORKLOADS["dsv3_prefill"].scaled(T=1), W.WORKLOADS["dsv3_prefill"]]
    big = max(cdl.layout_workspace_size(w.T, w.k, w.L) for w in shapes)
    ws = torch.full((big,), 0xA5, dtype=torch.uint8, device=DEV)
    st = status_word()
    for n, w in enumerate(shapes):
        announce("workspace reuse %d: %s T=%d" % (n, w.name, w.T))
        ids = W.make_topk_ids(w)
        lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L, workspace=ws)
        x = W.make_hidden(w) if w.T else torch.zeros(0, w.H, dtype=torch.bfloat16)
        lay2, rows = cdl.permute(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, workspace=ws,
                                 status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        _, s_, d, _ = check_layout(lay, ids, w.expert_begin, w.L)
        check_layout(lay2, ids, w.expert_begin, w.L)
        R = int(s_[-1])
        if w.T:
            assert np.array_equal(bits16(rows[:R]), oracle.dispatch(W.bf16_bits(x), d, w.k, R))


def test_permute_rows_overflow_flag():
    w = W.WORKLOADS["tiny"]
    announce("permute cap < R")
    x, ids, wts = W.make_inputs(w)
    _, s, d, _ = oracle.layout(ids.numpy(), 0, w.L)
    R = int(s[-1])
    cap = R - 5
    buf = bf16_filled(R, w.H, 0x7F7F)
    st = status_word()
    lay, _ = cdl.permute(x.to(DEV), ids.to(DEV), 0, w.L, out=buf[:cap], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == cdl.CDL_STATUS_ROWS_OVERFLOW
    P = oracle.dispatch(W.bf16_bits(x), d, w.k, R)
    got = bits16(buf)
    assert np.array_equal(got[:cap], P[:cap]) and np.all(got[cap:] == 0x7F7F)


@pytest.mark.parametrize("b", [0, -100, 2**31 - 40, -2**31])
def test_permute_int32_extreme_ids(b):
    """Ids at the ends of int32 and expert ranges next to them: same layout
    and rows as the oracle (the local expert is computed without wrap-around)."""
    announce("permute extreme ids b=%d" % b)
    g = np.random.default_rng(b & 0xFFFF)
    ext = [-2**31, -2**31 + 1, -101, -100, -69, -1, 0, 1, 31, 32, 2**31 - 41, 2**31 - 40,
           2**31 - 9, 2**31 - 8, 2**31 - 1]
    T, k, L, H = 300, 4, 32, 64
    ids = g.choice(ext + [min(b + i, 2**31 - 1) for i in range(0, 32, 3)], size=(T, k))
    ids = torch.from_numpy(np.clip(ids, -2**31, 2**31 - 1).astype(np.int32))
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    lay, rows = cdl.permute(x.to(DEV), ids.to(DEV), b, L)
    torch.cuda.synchronize()
    _, s_, d, _ = check_layout(lay, ids, b, L)
    R = int(s_[-1])
    assert np.array_equal(bits16(rows[:R]), oracle.dispatch(W.bf16_bits(x), d, k, R))


@pytest.mark.parametrize("case", ["T0", "T1", "all_invalid", "max_k", "max_L", "H8"])
def test_permute_edge_cases(case):
    announce("permute edge " + case)
    g = torch.Generator().manual_seed(zlib.crc32(case.encode()))
    T, k, L, E, H, b = 200, 4, 16, 64, 64, 0
    if case == "T0":
        T = 0
    elif case == "T1":
        T, k = 1, 3
    elif case == "max_k":
        T, k, L, E = 150, 64, 128, 128
    elif case == "max_L":
        T, k, L, E = 900, 8, 2048, 2048
    elif case == "H8":
        H = 8
    if case in ("max_k", "max_L"):
        ids = torch.multinomial(torch.ones(max(T, 1), E), k, generator=g).to(torch.int32)[:T]
    else:
        ids = torch.randint(-1, E + 1, (T, k), generator=g, dtype=torch.int32)
    if case == "all_invalid":
        ids = torch.randint(L, E, (T, k), generator=g, dtype=torch.int32)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    c, s, d, r = oracle.layout(ids.numpy(), b, L)
    R = int(s[-1])
    buf = bf16_filled(R + 2, H, 0x7F7F)
    lay, _ = cdl.permute(x.to(DEV), ids.to(DEV), b, L, out=buf[:R])
    torch.cuda.synchronize()
    check_layout(lay, ids, b, L)
    got = bits16(buf)
    assert np.array_equal(got[:R], oracle.dispatch(W.bf16_bits(x), d, k, R))
    assert np.all(got[R:] == 0x7F7F)
    # the same case through the per-tensor fp8 permute (rows cast, canaries kept)
    q = torch.full((R + 2, H), 0xA5, dtype=torch.uint8, device=DEV)
    lay2, _ = cdl.permute_fp8_tensor(x.to(DEV), ids.to(DEV), b, L, out_q=q[:R])
    torch.cuda.synchronize()
    check_layout(lay2, ids, b, L)
    assert np.array_equal(u8(q), oracle.dispatch_fp8_tensor(W.bf16_bits(x), d, k, R + 2, fill=0xA5))


@pytest.mark.parametrize("w", [W.WORKLOADS["fp8_dispatch"],
                               W.WORKLOADS["fp8_dispatch"].scaled(T=333, H=1152, expert_begin=96),
                               W.WORKLOADS["fp8_dispatch"].scaled(T=2501, H=1024, expert_begin=32)],
                         ids=lambda w: "T%d_H%d" % (w.T, w.H))
def test_permute_fp8_parity(w):
    announce("permute fp8 T=%d H=%d" % (w.T, w.H))
    x, ids, wts = W.make_inputs(w)
    _, s, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s[-1])
    G = w.H // 128
    q = torch.full((R + 2, w.H), 0xA5, dtype=torch.uint8, device=DEV)
    sc = torch.full((R + 2, G), -7.0, dtype=torch.float32, device=DEV)
    st = status_word()
    lay, _, _ = cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q[:R],
                                out_scales=sc[:R], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    check_layout(lay, ids, w.expert_begin, w.L)
    Q, S = oracle.dispatch_fp8(W.bf16_bits(x), d, w.k, R)
    gq, gs = u8(q), npy(sc)
    assert np.array_equal(gq[:R], Q)
    assert np.array_equal(gs[:R].view(np.uint32), S.view(np.uint32))
    assert np.all(gq[R:] == 0xA5) and np.all(gs[R:] == -7.0)


@pytest.mark.parametrize("L", [1, 63, 64, 65, 128])
@pytest.mark.parametrize("T", [100, 1500])
@pytest.mark.parametrize("A", [1, 16])
def test_layout_expert_scan_paths(L, T, A):
    """Small batches with up to 64 local experts scan them inside one wave
    (DPP), other batches across the workgroup: the layout (counts, padded
    seg_indptr, src2dst, reorder) at both sides of 64, for a batch that counts
    itself (T = 100, k = 8) and one that uses the count kernel (T = 1500),
    with and without padding."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=T, L=L, H=64, expert_begin=0, E=max(L, 256))
    announce("expert scan L=%d T=%d A=%d" % (L, T, A))
    x, ids, wts = W.make_inputs(w)
    c, s_, d, r = oracle.layout_aligned(ids.numpy(), 0, L, A)
    lay = cdl.dispatch_layout(ids.to(DEV), 0, L, alignment=A)
    lay2, _ = cdl.permute(x.to(DEV), ids.to(DEV), 0, L, alignment=A)
    torch.cuda.synchronize()
    for g in (lay, lay2):
        assert np.array_equal(npy(g.counts), c) and np.array_equal(npy(g.seg_indptr), s_)
        assert np.array_equal(npy(g.src2dst), d)
        assert np.array_equal(npy(g.reorder_topk_ids), r)


@pytest.mark.parametrize("T,L,fp8", [(1, 32, False), (5, 8, False), (100, 8, False), (512, 32, False),
                                    (513, 32, False), (100, 8, True), (512, 32, True), (513, 32, True)])
def test_permute_small_batches_all_rows(T, L, fp8):
    """Batches of up to 512 tokens that count themselves (T*k <= 4096) load
    every token's row whether or not it has a local slot.  With few local
    experts most tokens have none: their rows must not be stored anywhere
    (canary rows past R stay untouched), and the rows of the others match the
    oracle; 513 tokens take the path that checks each token first."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=T, L=L, H=1024, expert_begin=256 - L)
    announce("permute small batch T=%d L=%d fp8=%d" % (T, L, fp8))
    x, ids, wts = W.make_inputs(w)
    _, s, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s[-1])
    st = status_word()
    if fp8:
        q = torch.full((R + 2, w.H), 0xA5, dtype=torch.uint8, device=DEV)
        sc = torch.full((R + 2, w.H // 128), -7.0, dtype=torch.float32, device=DEV)
        lay, _, _ = cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q[:R],
                                    out_scales=sc[:R], status=st)
        torch.cuda.synchronize()
        Q, S = oracle.dispatch_fp8(W.bf16_bits(x), d, w.k, R)
        gq, gs = u8(q), npy(sc)
        assert np.array_equal(gq[:R], Q)
        assert np.array_equal(gs[:R].view(np.uint32), S.view(np.uint32))
        assert np.all(gq[R:] == 0xA5) and np.all(gs[R:] == -7.0)
    else:
        buf = bf16_filled(R + 3, w.H, 0x7F7F)
        lay, _ = cdl.permute(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out=buf[:R], status=st)
        torch.cuda.synchronize()
        got = bits16(buf)
        assert np.array_equal(got[:R], oracle.dispatch(W.bf16_bits(x), d, w.k, R))
        assert np.all(got[R:] == 0x7F7F)
    assert int(st.item()) == 0
    check_layout(lay, ids, w.expert_begin, w.L)


@pytest.mark.parametrize("H", [128, 1152, 7168, 8320])
@pytest.mark.parametrize("T", [1, 64])
def test_permute_fp8_small_batch_rows_over_waves(T, H):
    """Small self-counted fp8 batches split each row over 7 waves of 2
    chunks per lane: one group (only wave 0 has chunks), ragged packing
    (9 groups), one full 7168-wide pass, and two passes (65 groups).  Normal
    permute (fp32 scales, canary rows) and low-latency permute (packed
    column-major UE8M0 scales) against the oracle."""
    w = W.WORKLOADS["ll_decode"].scaled(T=T, H=H)
    announce("fp8 small batch over waves T=%d H=%d" % (T, H))
    x, ids, wts = W.make_inputs(w)
    xb = W.bf16_bits(x)
    _, s_, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s_[-1])
    st = status_word()
    q = torch.full((R + 2, H), 0xA5, dtype=torch.uint8, device=DEV)
    sc = torch.full((R + 2, H // 128), -7.0, dtype=torch.float32, device=DEV)
    lay, _, _ = cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q[:R],
                                out_scales=sc[:R], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    check_layout(lay, ids, w.expert_begin, w.L)
    Q, S = oracle.dispatch_fp8(xb, d, w.k, R)
    gq, gs = u8(q), npy(sc)
    assert np.array_equal(gq[:R], Q) and np.array_equal(gs[:R].view(np.uint32), S.view(np.uint32))
    assert np.all(gq[R:] == 0xA5) and np.all(gs[R:] == -7.0)
    flags = UE_ | CM_ | PK_
    cap = 64
    Q2, S2, mm, ll, ovf = oracle.dispatch_ll_fp8(xb, ids.numpy(), w.expert_begin, w.L, cap, flags,
                                                 fill=0xEE)
    q2 = torch.zeros(w.L, cap, H, dtype=torch.uint8, device=DEV)
    sb = torch.full((max(S2.size, 1),), 0xEE, dtype=torch.uint8, device=DEV)
    lay2, q2, sb, gmm, gll = cdl.permute_ll_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, cap,
                                                scale_flags=flags, out_q=q2, out_scales=sb,
                                                status=st)
    torch.cuda.synchronize()
    assert not ovf and int(st.item()) == 0
    assert np.array_equal(npy(gmm), mm) and np.array_equal(npy(gll), ll)
    assert np.array_equal(u8(q2).reshape(-1), Q2.reshape(-1))
    assert np.array_equal(sb.cpu().numpy().reshape(-1)[:S2.size], S2)


@pytest.mark.parametrize("T,k,H", [(1, 8, 7168), (512, 8, 7168), (513, 8, 7168), (200, 9, 512),
                                   (100, 8, 9000), (64, 8, 8), (40, 1, 200), (3, 8, 8192)])
def test_combine_small_batch_kernel(T, k, H):
    """Batches of up to 512 tokens with k <= 8 use the combine kernel that
    loads all of a token's slots at once (one chunk per thread, a second pass
    past 1024 chunks); 513 tokens and k = 9 take the other one.  Both give
    the oracle's bits and write nothing past the T output rows."""
    announce("combine small batch T=%d k=%d H=%d" % (T, k, H))
    g = torch.Generator().manual_seed(T * 131 + k * 7 + H)
    R = max(1, (T * k) // 2)
    y = torch.randn(R, H, generator=g).to(torch.bfloat16)
    m = torch.randint(-R // 2, R, (T * k,), generator=g, dtype=torch.int32)
    m[m < 0] = -1
    wts = torch.randn(T, k, generator=g).softmax(-1)
    outbuf = bf16_filled(T + 2, H, 0x7F7F)
    st = status_word()
    cdl.combine(y.to(DEV), m.to(DEV), wts.to(DEV), out=outbuf[:T], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = bits16(outbuf)
    want = oracle.combine(W.bf16_bits(y), m.numpy(), wts.numpy(), T, k)
    assert np.array_equal(got[:T], want)
    assert np.all(got[T:] == 0x7F7F)


@pytest.mark.parametrize("T,k,H", [(600, 8, 264), (700, 8, 4096), (600, 8, 7168), (520, 64, 512),
                                   (530, 3, 20480), (600, 1, 8), (515, 8, 7176)])
def test_combine_pipelined_kernel(T, k, H):
    """Batches past 512 tokens (or k > 8) take the combine that keeps the
    rows of two valid slots in flight, two chunks per lane, on a workgroup
    sized to the row: one ragged wave (H = 264: 33 chunks), rows that need
    several passes (H = 20480: 2560 chunks over 1024 lanes), tokens with many
    valid slots (k = 64, about half of them valid) so the two buffers are
    refilled many times, and a row whose length is not a whole number of
    waves.  Bits as the oracle's; rows past T untouched."""
    announce("combine pipelined T=%d k=%d H=%d" % (T, k, H))
    g = torch.Generator().manual_seed(T * 17 + k * 5 + H)
    R = max(1, (T * k) // 2)
    y = torch.randn(R, H, generator=g).to(torch.bfloat16)
    m = torch.randint(-R // 2, R, (T * k,), generator=g, dtype=torch.int32)
    m[m < 0] = -1
    m[:k] = torch.arange(k, dtype=torch.int32) % R          # one token with every slot valid
    wts = torch.randn(T, k, generator=g).softmax(-1)
    outbuf = bf16_filled(T + 2, H, 0x7F7F)
    st = status_word()
    cdl.combine(y.to(DEV), m.to(DEV), wts.to(DEV), out=outbuf[:T], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = bits16(outbuf)
    want = oracle.combine(W.bf16_bits(y), m.numpy(), wts.numpy(), T, k)
    assert np.array_equal(got[:T], want)
    assert np.all(got[T:] == 0x7F7F)


def test_permute_rejects_unsupported_shapes():
    ids = torch.zeros(2, 1, dtype=torch.int32, device=DEV)
    with pytest.raises(cdl.CdlError):
        cdl.permute(torch.zeros(2, 100, dtype=torch.bfloat16, device=DEV), ids, 0, 1)
    with pytest.raises(cdl.CdlError):
        cdl.permute_fp8(torch.zeros(2, 200, dtype=torch.bfloat16, device=DEV), ids, 0, 1)


def test_fp8_group_magnitudes():
    """Groups at every binary magnitude from bf16 subnormals to the largest
    bf16 values: both sides of the fast-quotient threshold (amax 2^-96), groups
    made of subnormals, signed zeros, and all-zero groups."""
    announce("fp8 group magnitudes")
    g = torch.Generator().manual_seed(4242)
    exps = list(range(-133, 128))
    G = len(exps) * 2
    base = torch.randn(G, 128, generator=g)
    scale = torch.tensor([2.0 ** e for e in exps for _ in range(2)], dtype=torch.float64)
    # finite inputs only (NaN / Inf are outside the contract): clip at the
    # largest bf16 magnitude below the overflow threshold
    vals = (base.double() * scale[:, None]).clamp(-3.3e38, 3.3e38).float().to(torch.bfloat16)
    assert torch.isfinite(vals.float()).all()
    xb = W.bf16_bits(vals).copy()
    xb[1, :] = 0x0000                      # an all-zero group
    xb[3, ::3] = 0x8000                    # signed zeros inside a group
    rows = -(-G // 8)
    xfull = np.zeros((rows * 8, 128), np.uint16)
    xfull[:G] = xb
    xfull = xfull.reshape(rows, 1024)
    ids = torch.arange(rows, dtype=torch.int32).reshape(rows, 1)
    lay = cdl.dispatch_layout(ids.to(DEV), 0, rows)
    q, s = cdl.dispatch_fp8(W.bits_to_bf16(xfull).to(DEV), lay)
    lay2, q2, s2 = cdl.permute_fp8(W.bits_to_bf16(xfull).to(DEV), ids.to(DEV), 0, rows, rows=rows)
    torch.cuda.synchronize()
    _, _, d, _ = oracle.layout(ids.numpy(), 0, rows)
    Q, S = oracle.dispatch_fp8(xfull, d, 1, rows)
    assert np.array_equal(u8(q), Q) and np.array_equal(u8(q2), Q)
    assert np.array_equal(npy(s).view(np.uint32), S.view(np.uint32))
    assert np.array_equal(npy(s2).view(np.uint32), S.view(np.uint32))


# --------------------------------------------------------------------------
# expert alignment
# --------------------------------------------------------------------------

ALIGNED = [W.WORKLOADS["tiny"], W.WORKLOADS["dsv3_prefill"].scaled(T=1000, H=512),
           W.WORKLOADS["zipf_prefill"].scaled(T=2000, H=256)]


@pytest.mark.parametrize("A", [2, 16, 128])
@pytest.mark.parametrize("w", ALIGNED, ids=lambda w: "%s_T%d" % (w.name, w.T))
def test_permute_aligned_parity(w, A):
    announce("aligned %s T=%d A=%d" % (w.name, w.T, A))
    x, ids, wts = W.make_inputs(w)
    c, s, d, r = oracle.layout_aligned(ids.numpy(), w.expert_begin, w.L, A)
    R = int(s[-1])
    # layout alone
    lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L, alignment=A)
    torch.cuda.synchronize()
    assert np.array_equal(npy(lay.counts), c) and np.array_equal(npy(lay.seg_indptr), s)
    assert np.array_equal(npy(lay.src2dst), d)
    assert np.array_equal(npy(lay.reorder_topk_ids), r)
    # fused permute into a canaried buffer: real rows bit-exact, padding untouched
    buf = bf16_filled(R + 2, w.H, 0x7F7F)
    st = status_word()
    lay2, _ = cdl.permute(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out=buf[:R], status=st,
                          alignment=A)
    out = cdl.combine(buf[:R], lay2.src2dst, wts.to(DEV), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(npy(lay2.src2dst), d)
    assert np.array_equal(npy(lay2.reorder_topk_ids), r)
    P = oracle.dispatch(W.bf16_bits(x), d, w.k, R, fill=0x7F7F)
    assert np.array_equal(bits16(buf[:R]), P)                 # padding rows keep 0x7F7F
    assert np.all(bits16(buf[R:]) == 0x7F7F)
    # the combine reads only real rows: same result as the unaligned path
    c0, s0, d0, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    want = oracle.combine(oracle.dispatch(W.bf16_bits(x), d0, w.k, int(s0[-1])), d0,
                          wts.numpy(), w.T, w.k)
    assert np.array_equal(bits16(out), want)


def test_full_size_dsv3_aligned_and_deepgemm_fp8():
    """The bench's NEXT-row configurations at full size (4096 tokens,
    H = 7168, 32 of 256 experts, top-8, segments padded to 128 rows, output
    sized to the padded row count): the bf16 permute (padding rows untouched)
    and the fp8 permute in the DeepGEMM format (packed column-major UE8M0
    scales), bit for bit against the oracle."""
    w = W.WORKLOADS["dsv3_prefill"]
    A = 128
    announce("full dsv3_prefill aligned 128 + DeepGEMM fp8")
    x, ids, wts = W.make_inputs(w)
    xb = W.bf16_bits(x)
    c, s_, d, r = oracle.layout_aligned(ids.numpy(), w.expert_begin, w.L, A)
    Rp = int(s_[-1])
    buf = bf16_filled(Rp + 2, w.H, 0x7F7F)
    st = status_word()
    lay, _ = cdl.permute(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out=buf[:Rp], status=st,
                         alignment=A)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(npy(lay.seg_indptr), s_) and np.array_equal(npy(lay.src2dst), d)
    assert np.array_equal(npy(lay.reorder_topk_ids), r)
    assert np.array_equal(bits16(buf[:Rp]), oracle.dispatch(xb, d, w.k, Rp, fill=0x7F7F))
    assert np.all(bits16(buf[Rp:]) == 0x7F7F)
    flags = UE_ | CM_ | PK_
    Q, S = oracle.dispatch_fp8_fmt(xb, d, w.k, Rp, flags, rows_per_mat=Rp, fill=0xEE)
    q = torch.zeros(Rp, w.H, dtype=torch.uint8, device=DEV)
    sb = filled_scales(cdl.fp8_scale_bytes(Rp, w.H, flags, Rp))
    cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q, out_scales=sb,
                    status=st, scale_flags=flags, alignment=A)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    real = d[d >= 0]
    assert np.array_equal(u8(q)[real], Q[real])
    assert np.array_equal(raw_bytes(sb), S)


def test_permute_fp8_aligned_parity():
    w = W.WORKLOADS["fp8_dispatch"].scaled(T=600, H=1024)
    A = 128
    announce("aligned fp8 T=%d" % w.T)
    x, ids, wts = W.make_inputs(w)
    c, s, d, r = oracle.layout_aligned(ids.numpy(), w.expert_begin, w.L, A)
    R = int(s[-1])
    q = torch.full((R, w.H), 0xA5, dtype=torch.uint8, device=DEV)
    sc = torch.full((R, w.H // 128), -7.0, dtype=torch.float32, device=DEV)
    lay, _, _ = cdl.permute_fp8(x.to(DEV), ids.to(DEV), 0, w.L, out_q=q, out_scales=sc, alignment=A)
    torch.cuda.synchronize()
    assert np.array_equal(npy(lay.src2dst), d)
    Q, S = oracle.dispatch_fp8(W.bf16_bits(x), d, w.k, R)
    real = np.zeros(R, bool)
    real[d[d >= 0]] = True
    assert np.array_equal(u8(q)[real], Q[real])
    assert np.array_equal(npy(sc)[real].view(np.uint32), S[real].view(np.uint32))
    assert np.all(u8(q)[~real] == 0xA5) and np.all(npy(sc)[~real] == -7.0)


def test_layout_aligned_reorder_capacity_flag():
    """A reorder_topk_ids capacity below the padded row count: entries past
    it are not written and the status bit is set."""
    import ctypes
    w = W.WORKLOADS["tiny"]
    announce("aligned reorder capacity")
    ids = W.make_topk_ids(w)
    A = 64
    c, s, d, r = oracle.layout_aligned(ids.numpy(), 0, w.L, A)
    R = int(s[-1])
    cap = R - 100
    idd = ids.to(DEV)
    counts = torch.empty(w.L, dtype=torch.int32, device=DEV)
    seg = torch.empty(w.L + 1, dtype=torch.int64, device=DEV)
    s2d = torch.empty(w.T * w.k, dtype=torch.int32, device=DEV)
    reorder = torch.full((R,), 12345, dtype=torch.int32, device=DEV)
    ws = torch.empty(cdl.layout_workspace_size(w.T, w.k, w.L), dtype=torch.uint8, device=DEV)
    st = status_word()
    P = ctypes.c_void_p
    rc = cdl.library().cdl_dispatch_layout_aligned(
        P(idd.data_ptr()), w.T, w.k, 0, w.L, A, P(counts.data_ptr()), P(seg.data_ptr()),
        P(s2d.data_ptr()), P(reorder.data_ptr()), cap, P(st.data_ptr()), P(ws.data_ptr()),
        ws.numel(), P(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    assert int(st.item()) == cdl.CDL_STATUS_REORDER_OVERFLOW
    assert np.array_equal(npy(s2d), d) and np.array_equal(npy(seg), s)
    got = npy(reorder)
    assert np.array_equal(got[:cap], r[:cap]) and np.all(got[cap:] == 12345)


# --------------------------------------------------------------------------
# rank layout
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name,R,rpn", [("dsv3_prefill", 8, 8), ("dsv3_prefill", 32, 8),
                                        ("ll_decode", 8, 1), ("zipf_prefill", 16, 4),
                                        ("tiny", 1, 1), ("dsv3_prefill", 64, 16),
                                        ("dsv3_prefill", 128, 8), ("dsv3_prefill", 4, 2)])
def test_rank_layout_parity(name, R, rpn):
    """Up to 64 ranks take the bit-mask kernel (8-byte flag stores when R is a
    multiple of 8, byte stores otherwise), more ranks the general one."""
    w = W.WORKLOADS[name]
    announce("rank layout %s R=%d rpn=%d" % (name, R, rpn))
    ids = W.make_topk_ids(w).clone()
    ids[::5, 0] = -1                                  # unrouted slots
    ids[1::7, -1] = w.E                               # FlashInfer-style invalid id
    rl = cdl.rank_layout(ids.to(DEV), w.E, R, rpn)
    torch.cuda.synchronize()
    pr, pn, pe, ir = oracle.rank_layout(ids.numpy(), w.E, R, rpn)
    assert np.array_equal(npy(rl.num_tokens_per_rank), pr)
    assert np.array_equal(npy(rl.num_tokens_per_rdma_rank), pn)
    assert np.array_equal(npy(rl.num_tokens_per_expert), pe)
    assert np.array_equal(npy(rl.is_token_in_rank), ir)


def test_rank_layout_edge_cases():
    announce("rank layout edges")
    rl = cdl.rank_layout(torch.zeros(0, 8, dtype=torch.int32, device=DEV), 64, 8, 2)
    torch.cuda.synchronize()
    assert npy(rl.num_tokens_per_rank).tolist() == [0] * 8
    assert npy(rl.num_tokens_per_expert).tolist() == [0] * 64
    g = torch.Generator().manual_seed(9)
    T, k, E, R = 1000, 64, 128, 64                    # k = 64, duplicate ranks per token
    ids = torch.randint(-2, E + 3, (T, k), generator=g, dtype=torch.int32)
    rl = cdl.rank_layout(ids.to(DEV), E, R, 8)
    torch.cuda.synchronize()
    pr, pn, pe, ir = oracle.rank_layout(ids.numpy(), E, R, 8)
    assert np.array_equal(npy(rl.num_tokens_per_rank), pr)
    assert np.array_equal(npy(rl.num_tokens_per_rdma_rank), pn)
    assert np.array_equal(npy(rl.num_tokens_per_expert), pe)
    assert np.array_equal(npy(rl.is_token_in_rank), ir)
    with pytest.raises(cdl.CdlError):
        cdl.rank_layout(ids.to(DEV), 100, 8, 1)


# --------------------------------------------------------------------------
# fp8 scale formats and fp8 on the low-latency path
# --------------------------------------------------------------------------

UE, CM, PK = cdl.FP8_SCALE_UE8M0, cdl.FP8_SCALE_COLMAJOR, cdl.FP8_SCALE_PACKED
FORMATS = [0, UE, CM, UE | CM, UE | PK, UE | CM | PK]


def raw_bytes(t):
    return t.detach().contiguous().cpu().view(torch.uint8).numpy().reshape(-1)


def filled_scales(nbytes, fill=0xEE):
    return torch.full((max(nbytes, 1),), fill, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("flags", FORMATS)
def test_fp8_scale_formats_parity(flags):
    w = W.WORKLOADS["fp8_dispatch"].scaled(T=517, H=640)          # 5 groups: ragged packing
    announce("fp8 format %d" % flags)
    x, ids, wts = W.make_inputs(w)
    c, s, d, r = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s[-1])
    cap = R + 3                                                     # ld = roundup(cap, 4)
    Q, S = oracle.dispatch_fp8_fmt(W.bf16_bits(x), d, w.k, cap, flags, rows_per_mat=cap,
                                   fill=0xEE)
    nbytes = cdl.fp8_scale_bytes(cap, w.H, flags, cap)
    assert nbytes == S.size
    # unfused scatter from a layout
    lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L)
    q = torch.zeros(cap, w.H, dtype=torch.uint8, device=DEV)
    sb = filled_scales(nbytes)
    st = status_word()
    cdl.dispatch_fp8(x.to(DEV), lay, out_q=q, out_scales=sb, status=st, scale_flags=flags)
    # fused permute (T = 517 counts itself: one kernel) with the binding's
    # workspace ...
    q2 = torch.zeros(cap, w.H, dtype=torch.uint8, device=DEV)
    sb2 = filled_scales(nbytes)
    cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q2, out_scales=sb2,
                    status=st, scale_flags=flags)
    # ... and with one of only the layout's size
    q3 = torch.zeros(cap, w.H, dtype=torch.uint8, device=DEV)
    sb3 = filled_scales(nbytes)
    ws = torch.empty(cdl.layout_workspace_size(w.T, w.k, w.L), dtype=torch.uint8, device=DEV)
    cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q3, out_scales=sb3,
                    status=st, scale_flags=flags, workspace=ws)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(u8(q), Q) and np.array_equal(u8(q2), Q) and np.array_equal(u8(q3), Q)
    assert np.array_equal(raw_bytes(sb), S) and np.array_equal(raw_bytes(sb2), S)
    assert np.array_equal(raw_bytes(sb3), S)


@pytest.mark.parametrize("H", [1152, 7296])
@pytest.mark.parametrize("flags", [CM, UE | CM | PK])
@pytest.mark.parametrize("A", [1, 128])
def test_permute_fp8_colmajor_large(flags, A, H):
    """Column-major scales at the fp8 dispatch shape (4096 tokens, count
    kernel), with segments padded to 128 rows or not: the split permute
    (H = 1152, 9 groups: ragged packing) and the one-kernel permute of rows
    of two passes (H = 7296, 57 groups).  Every real row's scales land in its
    column; padding rows, rows past R and the TMA padding of each column keep
    the fill."""
    w = W.WORKLOADS["fp8_dispatch"].scaled(H=H)
    announce("fp8 colmajor flags=%d A=%d H=%d" % (flags, A, H))
    x, ids, wts = W.make_inputs(w)
    _, s_, d, _ = oracle.layout_aligned(ids.numpy(), w.expert_begin, w.L, A)
    cap = int(s_[-1]) + 5
    Q, S = oracle.dispatch_fp8_fmt(W.bf16_bits(x), d, w.k, cap, flags, rows_per_mat=cap, fill=0xEE)
    q = torch.zeros(cap, w.H, dtype=torch.uint8, device=DEV)
    sb = filled_scales(cdl.fp8_scale_bytes(cap, w.H, flags, cap))
    st = status_word()
    cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q, out_scales=sb,
                    status=st, scale_flags=flags, alignment=A)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    gq = u8(q)
    assert np.array_equal(gq[d[d >= 0]], Q[d[d >= 0]])
    assert np.array_equal(raw_bytes(sb), S)


def test_fp8_ue8m0_group_magnitudes():
    """Power-of-two scales over every binary magnitude, zero groups and
    subnormal groups, in the packed column-major format."""
    announce("fp8 ue8m0 magnitudes")
    g = torch.Generator().manual_seed(77)
    exps = list(range(-133, 125))
    vals = (torch.randn(len(exps), 128, generator=g).double()
            * torch.tensor([2.0 ** e for e in exps], dtype=torch.float64)[:, None])
    vals = vals.clamp(-3.3e38, 3.3e38).float().to(torch.bfloat16)
    xb = W.bf16_bits(vals).copy()
    xb[0, :] = 0
    xb[2, ::2] = 0x8000
    G8 = 8
    rows = -(-xb.shape[0] // G8)
    xfull = np.zeros((rows * G8, 128), np.uint16)
    xfull[:xb.shape[0]] = xb
    xfull = xfull.reshape(rows, 128 * G8)
    ids = torch.arange(rows, dtype=torch.int32).reshape(rows, 1)
    _, _, d, _ = oracle.layout(ids.numpy(), 0, rows)
    for flags in (UE, UE | CM | PK):
        Q, S = oracle.dispatch_fp8_fmt(xfull, d, 1, rows, flags, rows_per_mat=rows, fill=0xEE)
        lay = cdl.dispatch_layout(ids.to(DEV), 0, rows)
        q = torch.zeros(rows, 128 * G8, dtype=torch.uint8, device=DEV)
        sb = filled_scales(S.size)
        cdl.dispatch_fp8(W.bits_to_bf16(xfull).to(DEV), lay, out_q=q, out_scales=sb,
                         scale_flags=flags)
        torch.cuda.synchronize()
        assert np.array_equal(u8(q), Q)
        assert np.array_equal(raw_bytes(sb), S)


@pytest.mark.parametrize("flags,cap", [(0, 1024), (UE, 1024), (CM, 1024), (UE | CM | PK, 1024),
                                       (UE | CM, 5)])
def test_ll_fp8_parity(flags, cap):
    w = W.WORKLOADS["ll_decode"]
    if cap < 100:
        w = w.scaled(T=100, H=512)
    announce("ll fp8 flags=%d cap=%d" % (flags, cap))
    x, ids, wts = W.make_inputs(w)
    Q, S, mm, ll, ovf = oracle.dispatch_ll_fp8(W.bf16_bits(x), ids.numpy(), w.expert_begin, w.L,
                                               cap, flags, fill=0xEE)
    lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L)
    q = torch.zeros(w.L, cap, w.H, dtype=torch.uint8, device=DEV)
    sb = filled_scales(S.size)
    st = status_word()
    q, sb, gmm, gll = cdl.dispatch_ll_fp8(x.to(DEV), lay, cap, scale_flags=flags, out_q=q,
                                          out_scales=sb, status=st)
    torch.cuda.synchronize()
    assert np.array_equal(npy(gmm), mm) and np.array_equal(npy(gll), ll)
    assert (int(st.item()) != 0) == bool(ovf)
    assert np.array_equal(u8(q).reshape(-1), Q.reshape(-1))
    assert np.array_equal(raw_bytes(sb), S)


def test_calls_on_a_side_stream():
    """Every call enqueues on torch's current stream: the permute, the
    combine and the low-latency dispatch issued on a side stream (inputs
    copied there, nothing synchronised in between) give the oracle's
    results once that stream is synchronised."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=700, H=1024)
    announce("side stream T=%d" % w.T)
    x, ids, wts = W.make_inputs(w)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        xd, idd, wd = x.to(DEV, non_blocking=False), ids.to(DEV), wts.to(DEV)
        lay, rows = cdl.permute(xd, idd, w.expert_begin, w.L)
        out = cdl.combine(rows, lay.src2dst, wd)
        lay2, buf, mm, llmap = cdl.permute_ll(xd, idd, w.expert_begin, w.L, 64)
        out2 = cdl.combine(buf, llmap, wd)
    side.synchronize()
    _, s_, d, _ = check_layout(lay, ids, w.expert_begin, w.L)
    R = int(s_[-1])
    P = oracle.dispatch(W.bf16_bits(x), d, w.k, R)
    assert np.array_equal(bits16(rows[:R]), P)
    want = oracle.combine(P, d, wts.numpy(), w.T, w.k)
    assert np.array_equal(bits16(out), want)
    assert np.array_equal(bits16(out2), want)                # LL combine = normal combine


@pytest.mark.parametrize("A", [16, 128])
def test_permute_fp8_tensor_aligned(A):
    """Per-tensor fp8 permute with expert segments padded to A rows: the
    padded layout, real rows bit-exact, padding rows and rows past the
    padded count untouched."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=900, H=256)
    announce("permute fp8 tensor aligned A=%d" % A)
    x, ids, _ = W.make_inputs(w)
    c, s_, d, r = oracle.layout_aligned(ids.numpy(), w.expert_begin, w.L, A)
    Rp = int(s_[-1])
    want = oracle.dispatch_fp8_tensor(W.bf16_bits(x), d, w.k, Rp + 3, fill=0xA5)
    q = torch.full((Rp + 3, w.H), 0xA5, dtype=torch.uint8, device=DEV)
    st = status_word()
    lay, _ = cdl.permute_fp8_tensor(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q[:Rp],
                                    status=st, alignment=A)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(npy(lay.seg_indptr), s_) and np.array_equal(npy(lay.src2dst), d)
    assert np.array_equal(npy(lay.reorder_topk_ids), r)
    assert np.array_equal(u8(q), want)


def test_fp8_quotient_just_above_448():
    """Groups whose scale fl(amax / 448) rounds down, so that the quotient of
    x = +-amax is 448 + 2^-15 (2464 of the bf16 amax values do this): the
    kernels convert the quotient without a clamp, and the conversion must
    still give the code of 448 (0x7E / 0xFE), as the oracle's clamp does.
    The split permute (3000 tokens), the one-kernel permute of a small batch
    (64 tokens) and the scatter from a layout."""
    ab = np.arange(1, 0x7F80, dtype=np.uint32)
    a = (ab << 16).view(np.float32)
    s = (a / np.float32(448)).astype(np.float32)
    q = (a / s).astype(np.float32)
    pick = ab[(q > 448) & (a >= np.float32(2.0 ** -96))]
    assert len(pick) == 2464 and q[(a >= np.float32(2.0 ** -96))].max() == np.float32(448 + 2.0 ** -15)
    T, H = 3000, 1024
    G = H // 128
    rng = np.random.default_rng(11)
    amax = pick[rng.integers(len(pick), size=(T, G))]
    # magnitudes below amax (bf16 patterns of positive values are ordered),
    # random signs, and +-amax at two places of every group
    mag = (rng.random((T, G, 128)) * amax[..., None]).astype(np.uint32)
    xb = (mag | (rng.integers(2, size=mag.shape, dtype=np.uint32) << 15)).astype(np.uint16)
    xb[:, :, 5] = amax
    xb[:, :, 77] = amax | 0x8000
    xb = xb.reshape(T, H)
    ids = torch.zeros(T, 1, dtype=torch.int32)
    x = W.bits_to_bf16(xb).to(DEV)
    announce("fp8 quotient 448 + 2^-15")
    _, _, d, _ = oracle.layout(ids.numpy(), 0, 1)
    Q, S = oracle.dispatch_fp8(xb, d, 1, T)
    assert np.all(Q.reshape(T, G, 128)[:, :, 5] == 0x7E) and np.all(Q.reshape(T, G, 128)[:, :, 77] == 0xFE)
    st = status_word()
    lay, q1, s1 = cdl.permute_fp8(x, ids.to(DEV), 0, 1, rows=T, status=st)
    q2, s2 = cdl.dispatch_fp8(x, lay, status=st)
    lay3, q3, s3 = cdl.permute_fp8(x[:64].contiguous(), ids[:64].to(DEV), 0, 1, rows=64, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for qq, ss in ((q1, s1), (q2, s2)):
        assert np.array_equal(u8(qq), Q)
        assert np.array_equal(npy(ss).view(np.uint32), S.view(np.uint32))
    assert np.array_equal(u8(q3), Q[:64])
    assert np.array_equal(npy(s3).view(np.uint32), S.view(np.uint32)[:64])


@pytest.mark.parametrize("path", ["dispatch", "permute"])
@pytest.mark.parametrize("H", [1024, 7168, 8320])
@pytest.mark.parametrize("flags", [0, UE | PK])
def test_fp8_rows_overflow_flag(path, H, flags):
    """fp8 rows into a buffer of cap_rows < R rows (the scatter from a given
    layout, and the permute; 1000 tokens of top-8 take the count kernel, so
    rows of one pass go through the held-row kernels and H = 8320 through
    the two-pass ones): CDL_STATUS_ROWS_OVERFLOW, the first cap_rows rows and
    their row-major scales as the oracle's, nothing written past them."""
    w = W.WORKLOADS["fp8_dispatch"].scaled(T=1000, H=H)
    announce("fp8 %s cap < R H=%d flags=%d" % (path, H, flags))
    x, ids, _ = W.make_inputs(w)
    _, s, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s[-1])
    cap = R - 7
    Q, S = oracle.dispatch_fp8_fmt(W.bf16_bits(x), d, w.k, R, flags, fill=0xEE)
    nb = cdl.fp8_scale_bytes(cap, H, flags, cap)
    q = torch.full((R, H), 0xA5, dtype=torch.uint8, device=DEV)
    sb = torch.full((nb + 64,), 0xEE, dtype=torch.uint8, device=DEV)
    st = status_word()
    if path == "dispatch":
        lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L)
        cdl.dispatch_fp8(x.to(DEV), lay, out_q=q[:cap], out_scales=sb[:nb], status=st,
                         scale_flags=flags)
    else:
        cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q[:cap],
                        out_scales=sb[:nb], status=st, scale_flags=flags)
    torch.cuda.synchronize()
    assert int(st.item()) == cdl.CDL_STATUS_ROWS_OVERFLOW
    gq, gs = u8(q), raw_bytes(sb)
    assert np.array_equal(gq[:cap], Q[:cap]) and np.all(gq[cap:] == 0xA5)
    assert np.array_equal(gs[:nb], S[:nb]) and np.all(gs[nb:] == 0xEE)


@pytest.mark.parametrize("path,T,H", [("dispatch", 1000, 1024), ("dispatch", 300, 8320),
                                      ("permute", 1000, 1024), ("permute", 100, 1024),
                                      ("tensor", 1000, 1024), ("ll", 128, 1024),
                                      ("ll_onecall", 128, 1024)])
def test_fp8_outputs_at_minimum_alignment(path, T, H):
    """The fp8 calls accept e4m3fn rows at 8-byte and scales at 4-byte
    alignment: outputs placed 8 (rows) and 4 (scales) bytes past a 256-byte
    boundary give the oracle's bytes, and the bytes around them keep their
    canaries."""
    w = W.WORKLOADS["fp8_dispatch"].scaled(T=T, H=H)
    announce("fp8 minimum alignment %s T=%d H=%d" % (path, T, H))
    x, ids, _ = W.make_inputs(w)
    xb = W.bf16_bits(x)
    _, s, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s[-1])
    st = status_word()
    if path in ("ll", "ll_onecall"):
        cap = 64
        flags = UE | CM | PK
        Q, S, _, _, _ = oracle.dispatch_ll_fp8(xb, ids.numpy(), w.expert_begin, w.L, cap, flags,
                                               fill=0xEE)
        nq, ns = w.L * cap * H, S.size
        qbuf = torch.full((nq + 16,), 0xA5, dtype=torch.uint8, device=DEV)
        qbuf[8:8 + nq] = 0                     # rows past masked_m keep the oracle's zeros
        sbuf = torch.full((ns + 8,), 0xEE, dtype=torch.uint8, device=DEV)
        q = qbuf[8:8 + nq].view(w.L, cap, H)
        sc = sbuf[4:4 + ns]
        if path == "ll":
            lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L)
            cdl.dispatch_ll_fp8(x.to(DEV), lay, cap, scale_flags=flags, out_q=q, out_scales=sc,
                                status=st)
        else:
            cdl.permute_ll_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, cap, scale_flags=flags,
                               out_q=q, out_scales=sc, status=st)
        Qw, Sw = Q.reshape(-1), S
    else:
        rows = R + 3
        if path == "tensor":
            Qw = oracle.dispatch_fp8_tensor(xb, d, w.k, rows, fill=0xA5).reshape(-1)
            Sw = None
        else:
            Q, S = oracle.dispatch_fp8(xb, d, w.k, rows)
            Qw, Sw = Q.reshape(-1), S.reshape(-1).view(np.uint8)
        nq = rows * H
        qbuf = torch.full((nq + 16,), 0xA5, dtype=torch.uint8, device=DEV)
        q = qbuf[8:8 + nq].view(rows, H)
        if Sw is not None:
            ns = Sw.size
            sbuf = torch.full((ns + 8,), 0xEE, dtype=torch.uint8, device=DEV)
            sc = sbuf[4:4 + ns]
        if path == "dispatch":
            lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L)
            cdl.dispatch_fp8(x.to(DEV), lay, out_q=q, out_scales=sc, status=st)
        elif path == "permute":
            cdl.permute_fp8(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q, out_scales=sc,
                            status=st)
        else:
            cdl.permute_fp8_tensor(x.to(DEV), ids.to(DEV), w.expert_begin, w.L, out_q=q, status=st)
    torch.cuda.synchronize()
    gq = u8(qbuf)
    if path not in ("ll", "ll_onecall"):
        assert int(st.item()) == 0
        # rows past R are not written: the oracle's zeros there stand for the canary
        gq_rows = gq[8:8 + nq].reshape(-1, H)
        want = Qw.reshape(-1, H).copy()
        if path != "tensor":
            want[R:] = 0xA5
        assert np.array_equal(gq_rows, want)
    else:
        assert np.array_equal(gq[8:8 + nq], Qw)
    assert np.all(gq[:8] == 0xA5) and np.all(gq[8 + nq:] == 0xA5)
    if Sw is not None:
        gs = raw_bytes(sbuf)
        if path in ("ll", "ll_onecall"):
            assert np.array_equal(gs[4:4 + ns], Sw)
        else:
            ws_ = Sw.reshape(rows, -1).copy()
            ws_[R:] = 0xEE
            assert np.array_equal(gs[4:4 + ns], ws_.reshape(-1))
        assert np.all(gs[:4] == 0xEE) and np.all(gs[4 + ns:] == 0xEE)


@pytest.mark.parametrize("off", [16, 2])
def test_bf16_rows_at_16_and_2_byte_alignment(off):
    """bf16 rows and outputs placed off bytes past a 256-byte boundary: at 16
    the vector kernels run, at 2 the dispatch and the combine take their
    element-wise kernels and the permute (which needs 16-byte rows) refuses
    the call; results are the oracle's, canaries around the outputs kept."""
    w = W.WORKLOADS["dsv3_prefill"].scaled(T=700, H=512)
    announce("bf16 alignment off=%d" % off)
    x, ids, wts = W.make_inputs(w)
    xb = W.bf16_bits(x)
    _, s, d, _ = oracle.layout(ids.numpy(), w.expert_begin, w.L)
    R = int(s[-1])
    e = off // 2                                   # offset in bf16 elements

    def placed(rows, fill):
        buf = bf16_filled(1, rows * w.H + e + 8, fill).view(-1)
        return buf, buf[e:e + rows * w.H].view(rows, w.H)

    xbuf, xo = placed(w.T, 0)
    xo.copy_(x.to(DEV))
    lay = cdl.dispatch_layout(ids.to(DEV), w.expert_begin, w.L)
    pbuf, P = placed(R, 0x7F7F)
    st = status_word()
    cdl.dispatch(xo, lay, out=P, status=st)
    obuf, out = placed(w.T, 0x7F7F)
    cdl.combine(P, lay.src2dst, wts.to(DEV), out=out, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    Pw = oracle.dispatch(xb, d, w.k, R)
    gp, go = bits16(pbuf), bits16(obuf)
    assert np.array_equal(gp[e:e + R * w.H].reshape(R, w.H), Pw)
    assert np.all(gp[:e] == 0x7F7F) and np.all(gp[e + R * w.H:] == 0x7F7F)
    assert np.array_equal(go[e:e + w.T * w.H].reshape(w.T, w.H),
                          oracle.combine(Pw, d, wts.numpy(), w.T, w.k))
    assert np.all(go[:e] == 0x7F7F) and np.all(go[e + w.T * w.H:] == 0x7F7F)
    qbuf, Q = placed(R, 0x7F7F)
    if off % 16 == 0:
        cdl.permute(xo, ids.to(DEV), w.expert_begin, w.L, out=Q, status=st)
        torch.cuda.synchronize()
        assert np.array_equal(bits16(qbuf)[e:e + R * w.H].reshape(R, w.H), Pw)
    else:
        with pytest.raises(cdl.CdlError):
            cdl.permute(xo, ids.to(DEV), w.expert_begin, w.L, out=Q, status=st)


def test_low_latency_capacity_zero():
    """cap = 0: every valid slot overflows.  masked_m is all zero,
    ll_src2dst all -1, the overflow bit is set, no row is written, and the
    combine over the empty buffer gives +0 for every token (bf16 and fp8
    rows, one call and separate calls)."""
    w = W.WORKLOADS["ll_decode"].scaled(H=512)
    announce("LL cap 0")
    x, ids, wts = W.make_inputs(w)
    xd, idd = x.to(DEV), ids.to(DEV)
    lay = cdl.dispatch_layout(idd, w.expert_begin, w.L)
    runs = []
    st = status_word()
    B, mm, ll = cdl.dispatch_ll(xd, lay, 0, status=st)
    runs.append((st, mm, ll, B))
    st = status_word()
    _, B, mm, ll = cdl.permute_ll(xd, idd, w.expert_begin, w.L, 0, status=st)
    runs.append((st, mm, ll, B))
    st = status_word()
    q, sc, mm, ll = cdl.dispatch_ll_fp8(xd, lay, 0, scale_flags=UE | CM | PK, status=st)
    runs.append((st, mm, ll, None))
    st = status_word()
    _, q, sc, mm, ll = cdl.permute_ll_fp8(xd, idd, w.expert_begin, w.L, 0, scale_flags=UE | CM | PK,
                                          status=st)
    runs.append((st, mm, ll, None))
    torch.cuda.synchronize()
    for st, mm, ll, B in runs:
        assert int(st.item()) == cdl.CDL_STATUS_LL_OVERFLOW
        assert np.all(npy(mm) == 0) and np.all(npy(ll) == -1)
        if B is not None:
            assert B.numel() == 0
            out = cdl.combine(B, ll, wts.to(DEV))
            torch.cuda.synchronize()
            assert np.all(bits16(out) == 0)
