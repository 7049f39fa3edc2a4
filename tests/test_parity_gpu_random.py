"""GPU parity over a seeded sweep of random configurations (MI355X only).

The hand-picked cases in test_parity_gpu.py pin each kernel path; this sweep
crosses the sizes and options that select those paths (tokens, top-k, local
experts and their offset, hidden size, alignment, fp8 scale format, per-tensor
scale, low-latency capacity) so that combinations nobody wrote down are run
too.  Every case goes through the fused and unfused normal paths, the combine,
both fp8 formats, the low-latency calls and the rank layout, each compared
with the oracle bit for bit.  Routing ids are drawn with duplicates, unrouted slots (-1), the
FlashInfer invalid id (E) and experts of other ranks; hidden rows are spread
over binades (and some rows are zero) so that fp8 scales of many exponents
occur.  Sizes are bounded so that the oracle finishes each case in about a
second; eight larger cases (1500-4500 tokens, rows up to H = 7168) take the
count kernel and the launch configurations of the benchmark shapes.
"""
import numpy as np
import pytest
import torch

import combine_dispatch_layout_amd as cdl
import oracle
from combine_dispatch_layout_amd import workloads as W
from gpu_util import DEV, announce, bf16_filled, bits16, npy, status_word, u8

pytestmark = pytest.mark.gpu

UE, CM, PK = cdl.FP8_SCALE_UE8M0, cdl.FP8_SCALE_COLMAJOR, cdl.FP8_SCALE_PACKED
FORMATS = [0, UE, CM, UE | CM, UE | PK, UE | CM | PK]
MAX_ELEMS = 1 << 24          # bound on dispatched elements per buffer (rows * H)


def _configs(n, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([0, 1, 2, 3, rng.integers(4, 65), rng.integers(65, 600),
                            rng.integers(600, 3000), rng.integers(3000, 6001)]))
        k = int(rng.choice([1, 2, 3, 4, 6, 8, 8, 9, 13, 16, 32, 64]))
        T = min(T, (1 << 17) // k)
        E = int(rng.choice([8, 16, 64, 128, 256, 512, 2048]))
        L = int(min(E, rng.choice([1, 2, 7, 8, 32, 33, 64, 128, 300, 2048])))
        b = int(rng.integers(0, E - L + 1)) if rng.random() < 0.8 else int(rng.integers(-50, 50))
        A = int(rng.choice([1, 1, 1, 2, 16, 128]))
        rows = max(T * k + L * (A - 1), 1)
        Hmax = max(128, min(8320, MAX_ELEMS // rows // 128 * 128))
        H128 = int(rng.integers(1, Hmax // 128 + 1)) * 128          # fp8 rows
        H8 = int(max(8, H128 - 8 * rng.integers(0, 16)))              # bf16 / per-tensor rows
        Hany = int(max(1, H8 - rng.integers(0, 8)))                   # unfused bf16 rows
        flags = int(rng.choice(FORMATS))
        scale = [None, 0.5, 0.37, 3.0, 2.0 ** -6][int(rng.integers(0, 5))]
        skew = float(rng.choice([0.0, 0.0, 1.2]))
        out.append(dict(i=i, T=T, k=k, E=E, L=L, b=b, A=A, H128=H128, H8=H8, Hany=Hany,
                        flags=flags, scale=scale, skew=skew, seed=int(rng.integers(1 << 30))))
    return out


def _large_configs(n, seed=7168):
    """Batches with the count kernel and rows up to one full pass (H <= 7168):
    the launch configurations of the benchmark shapes, with random routing
    parameters.  One local expert in 4 to 16 keeps R, and the oracle's work,
    near T * k / 8."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1500, 4501))
        k = int(rng.choice([4, 6, 8]))
        E = 256
        L = int(rng.choice([16, 32, 64]))
        b = int(rng.integers(0, E - L + 1))
        A = int(rng.choice([1, 1, 128]))
        H128 = int(rng.choice([4096, 6144, 7168]))
        H8 = int(H128 - 16 * rng.integers(0, 4))
        Hany = int(H8 - rng.integers(0, 8))
        flags = int(rng.choice(FORMATS))
        scale = [None, 0.5, 0.37, 3.0, 2.0 ** -6][int(rng.integers(0, 5))]
        skew = float(rng.choice([0.0, 1.2]))
        out.append(dict(i=1000 + i, T=T, k=k, E=E, L=L, b=b, A=A, H128=H128, H8=H8, Hany=Hany,
                        flags=flags, scale=scale, skew=skew, seed=int(rng.integers(1 << 30))))
    return out


CONFIGS = _configs(96) + _large_configs(8)


def _name(c):
    return "T%d_k%d_E%d_L%d_b%d_A%d_H%d" % (c["T"], c["k"], c["E"], c["L"], c["b"], c["A"],
                                           c["H128"])


def _inputs(c, H):
    g = torch.Generator().manual_seed(c["seed"])
    T, k, E = c["T"], c["k"], c["E"]
    if c["skew"]:
        p = torch.arange(1, E + 3, dtype=torch.float64).pow(-c["skew"])
        ids = torch.multinomial(p.expand(max(T, 1), E + 2).float(), k, replacement=True,
                                generator=g)[:T].to(torch.int32) - 1        # -1 .. E
    else:
        ids = torch.randint(-1, E + 1, (T, k), generator=g, dtype=torch.int32)
    if T and k > 1:
        ids[::11, 1] = ids[::11, 0]                                        # duplicates
    mag = torch.pow(2.0, torch.randint(-24, 24, (T, 1), generator=g).float())
    x = (torch.randn(T, H, generator=g) * mag).to(torch.bfloat16)
    if T:
        x[::13] = 0
    wts = torch.randn(T, k, generator=g)
    return x, ids, wts


def _check_layout(lay, c, ids):
    cnt, s, d, r = oracle.layout_aligned(ids.numpy(), c["b"], c["L"], c["A"])
    assert np.array_equal(npy(lay.counts), cnt)
    assert np.array_equal(npy(lay.seg_indptr), s)
    assert np.array_equal(npy(lay.src2dst), d)
    assert np.array_equal(npy(lay.reorder_topk_ids), r)
    return s, d


@pytest.mark.parametrize("c", CONFIGS, ids=_name)
def test_random_normal_path(c):
    """permute (fused) and dispatch_layout + dispatch (unfused), then the
    combine of the dispatched rows."""
    T, k, L, b, A = c["T"], c["k"], c["L"], c["b"], c["A"]
    H = c["H8"]
    announce("random normal %s H=%d" % (_name(c), H))
    x, ids, wts = _inputs(c, H)
    _, s, d, _ = oracle.layout_aligned(ids.numpy(), b, L, A)
    R = int(s[-1])
    want = oracle.dispatch(W.bf16_bits(x), d, k, R + 2, fill=0x7F7F)
    buf = bf16_filled(R + 2, H, 0x7F7F)
    st = status_word()
    lay, _ = cdl.permute(x.to(DEV), ids.to(DEV), b, L, out=buf[:R], status=st, alignment=A)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    _check_layout(lay, c, ids)
    assert np.array_equal(bits16(buf), want)
    out = bf16_filled(T + 1, H, 0x7F7F)
    cdl.combine(buf[:R], lay.src2dst, wts.to(DEV), out=out[:T], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = bits16(out)
    assert np.array_equal(got[:T], oracle.combine(want[:R], d, wts.numpy(), T, k))
    assert np.all(got[T:] == 0x7F7F)
    # unfused, with a hidden size that need not be a multiple of 8
    Ha = c["Hany"]
    xa = x[:, :Ha].contiguous()
    lay2 = cdl.dispatch_layout(ids.to(DEV), b, L, alignment=A)
    buf2 = bf16_filled(R + 2, Ha, 0x7F7F)
    cdl.dispatch(xa.to(DEV), lay2, out=buf2[:R], status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    _check_layout(lay2, c, ids)
    assert np.array_equal(bits16(buf2), oracle.dispatch(W.bf16_bits(xa), d, k, R + 2, fill=0x7F7F))


@pytest.mark.parametrize("c", CONFIGS, ids=_name)
def test_random_fp8_paths(c):
    """permute_fp8 and dispatch_fp8 in the case's scale format, and the
    per-tensor fp8 permute with the case's scale."""
    T, k, L, b, A, flags = c["T"], c["k"], c["L"], c["b"], c["A"], c["flags"]
    H = c["H128"]
    announce("random fp8 %s flags=%d scale=%s" % (_name(c), flags, c["scale"]))
    x, ids, _ = _inputs(c, H)
    xb = W.bf16_bits(x)
    _, s, d, _ = oracle.layout_aligned(ids.numpy(), b, L, A)
    R = int(s[-1])
    cap = R + 3
    Q, S = oracle.dispatch_fp8_fmt(xb, d, k, cap, flags, rows_per_mat=cap, fill=0xEE)
    nbytes = cdl.fp8_scale_bytes(cap, H, flags, cap)
    assert nbytes == S.size or (nbytes == 0 and S.size == 1)
    st = status_word()
    q = torch.zeros(cap, H, dtype=torch.uint8, device=DEV)
    sb = torch.full((max(nbytes, 1),), 0xEE, dtype=torch.uint8, device=DEV)
    lay, _, _ = cdl.permute_fp8(x.to(DEV), ids.to(DEV), b, L, out_q=q, out_scales=sb, status=st,
                                alignment=A, scale_flags=flags)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    _check_layout(lay, c, ids)
    assert np.array_equal(u8(q), Q)
    assert np.array_equal(sb.cpu().numpy()[:nbytes], S[:nbytes])
    # unfused, from the layout just made
    q2 = torch.zeros(cap, H, dtype=torch.uint8, device=DEV)
    sb2 = torch.full((max(nbytes, 1),), 0xEE, dtype=torch.uint8, device=DEV)
    cdl.dispatch_fp8(x.to(DEV), lay, out_q=q2, out_scales=sb2, status=st, scale_flags=flags)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(u8(q2), Q)
    assert np.array_equal(sb2.cpu().numpy()[:nbytes], S[:nbytes])
    # per-tensor cast, H a multiple of 8
    H8 = c["H8"]
    x8 = x[:, :H8].contiguous()
    sc = c["scale"]
    want = oracle.dispatch_fp8_tensor(W.bf16_bits(x8), d, k, R + 2, 1.0 if sc is None else sc,
                                      fill=0xA5)
    q3 = torch.full((R + 2, H8), 0xA5, dtype=torch.uint8, device=DEV)
    sd = None if sc is None else torch.tensor([sc], dtype=torch.float32, device=DEV)
    lay3, _ = cdl.permute_fp8_tensor(x8.to(DEV), ids.to(DEV), b, L, scale=sd, out_q=q3[:R],
                                     status=st, alignment=A)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    _check_layout(lay3, c, ids)
    assert np.array_equal(u8(q3), want)


def _ll_cap(c):
    T, k, L = c["T"], c["k"], c["L"]
    rng = np.random.default_rng(c["seed"])
    fair = max(1, -(-T * k // max(L, 1)))
    cap = int(rng.choice([1, 3, fair, 2 * fair, T * k + 1]))
    return max(1, min(cap, MAX_ELEMS // (L * c["H128"]) or 1))


@pytest.mark.parametrize("c", CONFIGS, ids=_name)
def test_random_low_latency(c):
    """permute_ll + the LL combine, and permute_ll_fp8 in the case's scale
    format, with a capacity that may overflow."""
    T, k, L, b, flags = c["T"], c["k"], c["L"], c["b"], c["flags"]
    H = c["H128"]
    cap = _ll_cap(c)
    announce("random ll %s cap=%d flags=%d" % (_name(c), cap, flags))
    x, ids, wts = _inputs(c, H)
    xb = W.bf16_bits(x)
    OB, omm, oll, ovf = oracle.dispatch_ll(xb, ids.numpy(), b, L, cap, fill=0x7F7F)
    st = status_word()
    B = bf16_filled(L * cap, H, 0x7F7F).view(L, cap, H)
    lay, B, mm, llmap = cdl.permute_ll(x.to(DEV), ids.to(DEV), b, L, cap, out=B, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == (cdl.CDL_STATUS_LL_OVERFLOW if ovf else 0)
    _check_layout(lay, dict(c, A=1), ids)
    assert np.array_equal(npy(mm), omm) and np.array_equal(npy(llmap), oll)
    assert np.array_equal(bits16(B.view(L * cap, H)), OB.reshape(-1, H))
    out = cdl.combine(B, llmap, wts.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bits16(out), oracle.combine(OB.reshape(-1, H), oll, wts.numpy(), T, k))
    # fp8 rows
    Q, S, mm2, ll2, ovf2 = oracle.dispatch_ll_fp8(xb, ids.numpy(), b, L, cap, flags, fill=0xEE)
    q = torch.zeros(L, cap, H, dtype=torch.uint8, device=DEV)
    sb = torch.full((max(S.size, 1),), 0xEE, dtype=torch.uint8, device=DEV)
    st2 = status_word()
    lay2, q, sb, gmm, gll = cdl.permute_ll_fp8(x.to(DEV), ids.to(DEV), b, L, cap, scale_flags=flags,
                                               out_q=q, out_scales=sb, status=st2)
    torch.cuda.synchronize()
    assert (int(st2.item()) != 0) == bool(ovf2)
    assert np.array_equal(npy(gmm), mm2) and np.array_equal(npy(gll), ll2)
    assert np.array_equal(u8(q).reshape(-1), Q.reshape(-1))
    assert np.array_equal(sb.cpu().numpy().reshape(-1)[:S.size], S)


@pytest.mark.parametrize("c", CONFIGS, ids=_name)
def test_random_rank_layout(c):
    """rank_layout over the case's global ids with a rank count that divides
    E (one workgroup for small batches of top-8 or less over up to 64 ranks,
    per-workgroup partials and their reduction otherwise)."""
    T, k, E = c["T"], c["k"], c["E"]
    rng = np.random.default_rng(c["seed"] + 1)
    R = int(rng.choice([r for r in (1, 2, 4, 8, 16, 32, 64, 128, 256, 1024) if E % r == 0]))
    rpn = int(rng.choice([n for n in (1, 2, 4, 8, 16) if R % n == 0]))
    announce("random rank layout %s R=%d rpn=%d" % (_name(c), R, rpn))
    _, ids, _ = _inputs(c, 8)
    rl = cdl.rank_layout(ids.to(DEV), E, R, rpn)
    torch.cuda.synchronize()
    pr, pn, pe, ir = oracle.rank_layout(ids.numpy(), E, R, rpn)
    assert np.array_equal(npy(rl.num_tokens_per_rank), pr)
    assert np.array_equal(npy(rl.num_tokens_per_rdma_rank), pn)
    assert np.array_equal(npy(rl.num_tokens_per_expert), pe)
    assert np.array_equal(npy(rl.is_token_in_rank), ir)
