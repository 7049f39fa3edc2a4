"""cdl_permute_noalloc (the permute with its scratch in a static device array)
against cdl_permute (scratch in a caller workspace), through the C ABI.

Two calls in a row, the second with a smaller input, so that the second
finds the first call's contents in the shared scratch; every output must be
bit-identical to cdl_permute's, and to the oracle's.  Inputs whose scratch
would exceed the static buffer are refused before any work.
"""
import ctypes

import numpy as np
import pytest
import torch

import combine_dispatch_layout_amd as cdl
import oracle
from combine_dispatch_layout_amd import workloads as W
from gpu_util import DEV, announce, bits16, npy, status_word

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p


def _run(noalloc, x, ids, b, L, cap):
    """One permute through the C ABI; returns its outputs as host arrays."""
    lib = cdl.library()
    T, k = ids.shape
    H = x.shape[1]
    counts = torch.full((L,), -7, dtype=torch.int32, device=DEV)
    seg = torch.full((L + 1,), -7, dtype=torch.int64, device=DEV)
    s2d = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    reo = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    out = torch.zeros(cap, H, dtype=torch.bfloat16, device=DEV)
    st = status_word()
    stream = P(torch.cuda.current_stream().cuda_stream)
    common = (P(x.data_ptr()), T, H, k, P(ids.data_ptr()), b, L, 1, P(counts.data_ptr()),
              P(seg.data_ptr()), P(s2d.data_ptr()), P(reo.data_ptr()), T * k, P(out.data_ptr()),
              cap, P(st.data_ptr()))
    if noalloc:
        rc = lib.cdl_permute_noalloc(*common, stream)
    else:
        wsb = cdl.layout_workspace_size(T, k, L)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        rc = lib.cdl_permute(*common, P(ws.data_ptr()), wsb, stream)
    assert rc == 0, cdl.status_string(rc)
    torch.cuda.synchronize()
    return npy(counts), npy(seg), npy(s2d), npy(reo), bits16(out), int(st.item())


@pytest.mark.parametrize("first,second", [("dsv3_prefill", "tiny"),
                                          ("zipf_prefill", "dsv3_prefill")])
def test_noalloc_permute_matches_workspace_permute(first, second):
    for i, name in enumerate((first, second)):
        w = W.WORKLOADS[name]
        if name == "zipf_prefill":
            w = w.scaled(T=6000, H=256)             # many superblocks, ragged tail
        if i == 1 and name == "dsv3_prefill":
            w = w.scaled(T=2500, H=512)             # smaller than the first call
        announce("noalloc permute call %d: %s T=%d H=%d" % (i, w.name, w.T, w.H))
        x, ids, _ = W.make_inputs(w)
        xd, idd = x.to(DEV), ids.to(DEV)
        c, s_, d, r = oracle.layout(ids.numpy(), w.expert_begin, w.L)
        R = int(s_[-1])
        cap = R + 2
        got = _run(True, xd, idd, w.expert_begin, w.L, cap)
        ref = _run(False, xd, idd, w.expert_begin, w.L, cap)
        for g, e in zip(got, ref):
            assert np.array_equal(g, e)
        assert got[5] == 0
        assert np.array_equal(got[0], c) and np.array_equal(got[1], s_)
        assert np.array_equal(got[2], d) and np.array_equal(got[3][:R], r)
        assert np.array_equal(got[4][:R], oracle.dispatch(W.bf16_bits(x), d, w.k, R))


def test_noalloc_permute_refuses_scratch_beyond_its_buffer():
    lib = cdl.library()
    # the largest layout workspaces: many tokens over the most local experts
    T, k, L = (1 << 22), 64, 2048
    need = lib.cdl_dispatch_layout_workspace_size(T, k, L)
    assert need > cdl.NOALLOC_SCRATCH_BYTES
    rc = lib.cdl_permute_noalloc(P(0x1000), T, 128, k, P(0x1000), 0, L, 1, P(0x1000), P(0x1000),
                                 P(0x1000), P(0x1000), T * k, P(0x1000), 1, None, None)
    assert rc == cdl.CDL_ERR_SCRATCH
    assert "scratch" in cdl.status_string(rc)
