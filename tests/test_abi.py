"""The C ABI on the CPU: the library loads, exports every entry point that
include/cdl.h declares, and rejects bad arguments before any HIP call (so
these tests run without a GPU)."""
import ctypes
import os
import re

import pytest

import combine_dispatch_layout_amd as cdl
import oracle
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "cdl.h")

OK, ENULL, ESIZE, EUNSUP, EWS, EBIG = 0, -1, -2, -3, -4, -5
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
NULL = None


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cdl_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = cdl.library()
    names = declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding():
    src = open(HEADER).read()
    for name, val in [("CDL_STATUS_ROWS_OVERFLOW", cdl.CDL_STATUS_ROWS_OVERFLOW),
                      ("CDL_STATUS_LL_OVERFLOW", cdl.CDL_STATUS_LL_OVERFLOW),
                      ("CDL_STATUS_MAP_RANGE", cdl.CDL_STATUS_MAP_RANGE),
                      ("CDL_FP8_GROUP", cdl.FP8_GROUP)]:
        m = re.search(r"#define\s+%s\s+\(?(-?\d+)\)?" % name, src)
        assert m and int(m.group(1)) == val, name


def test_status_strings():
    for code in (OK, ENULL, ESIZE, EUNSUP, EWS, EBIG, -6):
        s = cdl.status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in cdl.status_string(-99)


def test_permute_fp8_workspace_size():
    """Every format needs only the layout's workspace (column-major scales
    are written in place)."""
    lib = cdl.library()
    base = lib.cdl_dispatch_layout_workspace_size(4096, 8, 32)
    f = lib.cdl_permute_fp8_workspace_size
    CM, PK, UE = cdl.FP8_SCALE_COLMAJOR, cdl.FP8_SCALE_PACKED, cdl.FP8_SCALE_UE8M0
    for flags in (0, UE, CM, UE | CM, UE | PK, UE | CM | PK):
        assert f(4096, 8, 32, 7168, flags, 4200) == base
    assert f(4096, 8, 32, 640, UE | CM | PK, 100) == base
    assert f(4096, 8, 32, 7168, PK, 4200) == 0                         # packed needs UE8M0
    assert f(4096, 8, 32, 7000, CM, 4200) == 0                        # H not a multiple of 128
    assert f(4096, 8, 32, 7168, PK, 4200) == 0                        # packing needs UE8M0
    assert f(4096, 8, 32, 7168, CM, -1) == 0


def test_workspace_size():
    lib = cdl.library()
    assert lib.cdl_dispatch_layout_workspace_size(4096, 8, 32) >= 32 * 32 * 4
    assert lib.cdl_dispatch_layout_workspace_size(0, 8, 32) > 0
    assert lib.cdl_dispatch_layout_workspace_size(-1, 8, 32) == 0
    assert lib.cdl_dispatch_layout_workspace_size(10, 0, 32) == 0
    assert lib.cdl_dispatch_layout_workspace_size(10, 8, 0) == 0
    assert lib.cdl_dispatch_layout_workspace_size(10, 8, 2049) == 0
    assert lib.cdl_dispatch_layout_workspace_size(1 << 28, 8, 32) == 0


def test_expected_m_matches_oracle(golden):
    for T, n, k, E, want in golden("expected_m.txt"):
        assert cdl.ll_expected_m(int(T), int(n), int(k), int(E)) == int(want)
        assert oracle.expected_m(int(T), int(n), int(k), int(E)) == int(want)
    assert cdl.ll_expected_m(5, 1, 1, 0) == -1


def layout_call(T=16, k=2, L=4, ids=FAKE, counts=FAKE, seg=FAKE, s2d=FAKE, reorder=FAKE,
                ws=FAKE, ws_bytes=1 << 20):
    return cdl.library().cdl_dispatch_layout(ids, T, k, 0, L, counts, seg, s2d, reorder, ws,
                                             ws_bytes, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), ESIZE), (dict(k=0), ESIZE), (dict(k=65), ESIZE), (dict(L=0), ESIZE),
    (dict(L=2049), ESIZE), (dict(T=1 << 28, k=8), EBIG), (dict(counts=NULL), ENULL),
    (dict(seg=NULL), ENULL), (dict(ids=NULL), ENULL), (dict(s2d=NULL), ENULL),
    (dict(reorder=NULL), ENULL), (dict(ws=NULL), ENULL), (dict(ws_bytes=16), EWS),
])
def test_layout_rejects(kw, code):
    assert layout_call(**kw) == code


def test_dispatch_layout_aligned_rejects():
    f = cdl.library().cdl_dispatch_layout_aligned
    # ids, T, k, b, L, A, counts, seg, s2d, reorder, rcap, status, ws, wsb, stream
    base = [FAKE, 16, 2, 0, 4, 8, FAKE, FAKE, FAKE, FAKE, 64, NULL, FAKE, 1 << 20, NULL]
    names = ["ids", "T", "k", "b", "L", "A", "counts", "seg", "s2d", "reorder", "rcap", "status",
             "ws", "wsb", "stream"]

    def call(**over):
        a = list(base)
        for n, v in over.items():
            a[names.index(n)] = v
        return f(*a)

    assert call(A=0) == ESIZE
    assert call(A=4096) == ESIZE
    assert call(rcap=-5) == ESIZE
    assert call(counts=NULL) == ENULL
    assert call(reorder=NULL) == ENULL
    assert call(wsb=4) == EWS


def test_dispatch_rejects():
    lib = cdl.library()
    # x, T, H, k, src2dst, out, cap_rows, status, stream
    assert lib.cdl_dispatch(FAKE, 4, 0, 2, FAKE, FAKE, 8, NULL, NULL) == ESIZE
    assert lib.cdl_dispatch(FAKE, 4, 8, 0, FAKE, FAKE, 8, NULL, NULL) == ESIZE
    assert lib.cdl_dispatch(FAKE, 4, 8, 2, FAKE, FAKE, -1, NULL, NULL) == ESIZE
    assert lib.cdl_dispatch(NULL, 4, 8, 2, FAKE, FAKE, 8, NULL, NULL) == ENULL
    assert lib.cdl_dispatch(FAKE, 4, 8, 2, NULL, FAKE, 8, NULL, NULL) == ENULL
    assert lib.cdl_dispatch(FAKE, 4, 8, 2, FAKE, NULL, 8, NULL, NULL) == ENULL
    assert lib.cdl_dispatch(FAKE, 4, 8, 2, FAKE, FAKE, 1 << 31, NULL, NULL) == EBIG
    assert lib.cdl_dispatch(NULL, 0, 8, 2, NULL, NULL, 0, NULL, NULL) == OK  # empty: no launch


def test_dispatch_fp8_rejects():
    lib = cdl.library()
    f = lib.cdl_dispatch_fp8
    assert f(FAKE, 4, 200, 2, FAKE, FAKE, FAKE, 8, NULL, NULL) == EUNSUP
    assert f(FAKE, 4, 256, 2, FAKE, NULL, FAKE, 8, NULL, NULL) == ENULL
    assert f(FAKE, 4, 256, 2, FAKE, FAKE, NULL, 8, NULL, NULL) == ENULL
    assert f(ctypes.c_void_p(0x1008), 4, 256, 2, FAKE, FAKE, FAKE, 8, NULL, NULL) == EUNSUP
    assert f(NULL, 0, 256, 2, NULL, NULL, NULL, 0, NULL, NULL) == OK


def test_dispatch_ll_rejects():
    lib = cdl.library()
    f = lib.cdl_dispatch_ll
    args = [FAKE, 4, 256, 2, FAKE, 0, 8, FAKE, FAKE, FAKE, 16, FAKE, FAKE, FAKE, NULL, NULL]

    def call(**over):
        a = list(args)
        names = ["x", "T", "H", "k", "ids", "b", "L", "s2d", "seg", "counts", "cap", "out",
                 "mm", "ll", "status", "stream"]
        for n, v in over.items():
            a[names.index(n)] = v
        return f(*a)

    assert call(H=100) == EUNSUP
    assert call(L=0) == ESIZE
    assert call(cap=-1) == ESIZE
    assert call(cap=1 << 28, L=16) == EBIG
    assert call(mm=NULL) == ENULL
    assert call(ll=NULL) == ENULL
    assert call(out=NULL) == ENULL
    assert call(x=ctypes.c_void_p(0x1002)) == EUNSUP


def test_permute_ll_rejects():
    lib = cdl.library()
    f = lib.cdl_permute_ll
    names = ["x", "T", "H", "k", "ids", "b", "L", "counts", "seg", "s2d", "reorder", "rcap", "cap",
             "out", "mm", "ll", "status", "ws", "wsb", "stream"]
    args = [FAKE, 4, 256, 2, FAKE, 0, 8, FAKE, FAKE, FAKE, NULL, 0, 16, FAKE, FAKE, FAKE, NULL,
            FAKE, 1 << 20, NULL]

    def call(fn=f, extra=None, **over):
        a = list(args)
        for n, v in over.items():
            a[names.index(n)] = v
        if extra is not None:
            a = a[:14] + extra + a[14:]
        return fn(*a)

    assert call(H=100) == EUNSUP
    assert call(L=0) == ESIZE
    assert call(cap=-1) == ESIZE
    assert call(cap=1 << 28, L=16) == EBIG
    assert call(mm=NULL) == ENULL
    assert call(ll=NULL) == ENULL
    assert call(out=NULL) == ENULL
    assert call(counts=NULL) == ENULL
    assert call(ws=NULL) == ENULL
    assert call(wsb=8) == EWS
    assert call(rcap=5) == ENULL                       # capacity without a buffer
    assert call(x=ctypes.c_void_p(0x1002)) == EUNSUP
    assert call(out=ctypes.c_void_p(0x1008)) == EUNSUP
    g = lib.cdl_permute_ll_fp8
    # the same arguments with out_scales and scale_flags after out_q
    assert call(g, [FAKE, 0], H=200) == EUNSUP
    assert call(g, [FAKE, 4]) == EUNSUP                # packed needs UE8M0
    assert call(g, [NULL, 0]) == ENULL
    assert call(g, [FAKE, 0], mm=NULL) == ENULL


def test_hidden_size_limit():
    """Rows are addressed with 32-bit byte offsets: H above CDL_MAX_HIDDEN is
    rejected by every row call before any launch."""
    lib = cdl.library()
    big = (1 << 24) + 128
    # x, T, H, k, s2d, out, cap_rows, status, stream
    assert lib.cdl_dispatch(FAKE, 4, big, 2, FAKE, FAKE, 8, NULL, NULL) == EBIG
    assert lib.cdl_dispatch_fp8(FAKE, 4, big, 2, FAKE, FAKE, FAKE, 8, NULL, NULL) == EBIG
    # y, y_rows, H, map, w, T, k, out, status, stream
    assert lib.cdl_combine(FAKE, 8, big, FAKE, FAKE, 4, 2, FAKE, NULL, NULL) == EBIG
    # x, T, H, k, ids, b, L, s2d, seg, counts, cap, out, mm, ll, status, stream
    assert lib.cdl_dispatch_ll(FAKE, 4, big, 2, FAKE, 0, 8, FAKE, FAKE, FAKE, 16, FAKE, FAKE, FAKE,
                               NULL, NULL) == EBIG
    # x, T, H, k, ids, b, L, A, counts, seg, s2d, reorder, rcap, out, cap_rows, status, ws, wsb, stream
    assert lib.cdl_permute(FAKE, 4, big, 2, FAKE, 0, 8, 1, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 8, NULL,
                           FAKE, 1 << 20, NULL) == EBIG


def test_combine_rejects():
    lib = cdl.library()
    f = lib.cdl_combine
    # y, y_rows, H, map, w, T, k, out, status, stream
    assert f(FAKE, 8, 0, FAKE, FAKE, 4, 2, FAKE, NULL, NULL) == ESIZE
    assert f(FAKE, -1, 8, FAKE, FAKE, 4, 2, FAKE, NULL, NULL) == ESIZE
    assert f(FAKE, 8, 8, NULL, FAKE, 4, 2, FAKE, NULL, NULL) == ENULL
    assert f(FAKE, 8, 8, FAKE, NULL, 4, 2, FAKE, NULL, NULL) == ENULL
    assert f(FAKE, 8, 8, FAKE, FAKE, 4, 2, NULL, NULL, NULL) == ENULL
    assert f(NULL, 8, 8, FAKE, FAKE, 4, 2, FAKE, NULL, NULL) == ENULL
    assert f(FAKE, 8, 8, FAKE, FAKE, 4, 99, FAKE, NULL, NULL) == ESIZE
    assert f(NULL, 0, 8, NULL, NULL, 0, 2, NULL, NULL, NULL) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        cdl.dispatch_layout(torch.zeros(4, 2, dtype=torch.int32), 0, 4)


def test_permute_rejects():
    lib = cdl.library()
    names = ["x", "T", "H", "k", "ids", "b", "L", "A", "counts", "seg", "s2d", "reorder", "rcap",
             "out", "cap", "status", "ws", "wsb", "stream"]
    base = [FAKE, 4, 256, 2, FAKE, 0, 8, 1, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 16, NULL, FAKE,
            1 << 20, NULL]

    def call(**over):
        a = list(base)
        for n, v in over.items():
            a[names.index(n)] = v
        return lib.cdl_permute(*a)

    assert call(k=0) == ESIZE
    assert call(L=0) == ESIZE
    assert call(H=0) == ESIZE
    assert call(cap=-1) == ESIZE
    assert call(H=100) == EUNSUP
    assert call(x=ctypes.c_void_p(0x1004)) == EUNSUP
    assert call(out=NULL) == ENULL
    assert call(x=NULL) == ENULL
    assert call(ws=NULL) == ENULL
    assert call(wsb=8) == EWS
    assert call(cap=1 << 31) == EBIG
    assert call(A=0) == ESIZE
    assert call(A=1025) == ESIZE
    assert call(rcap=-1) == ESIZE
    assert call(reorder=NULL) == ENULL
    assert call(reorder=NULL, rcap=0) != ENULL      # no reorder output requested
    assert call(T=(1 << 28) - 1, k=8, A=1024, L=2048) == EBIG   # padded rows reach 2^31


def test_permute_fp8_rejects():
    lib = cdl.library()
    names = ["x", "T", "H", "k", "ids", "b", "L", "A", "counts", "seg", "s2d", "reorder", "rcap",
             "q", "s", "sf", "cap", "status", "ws", "wsb", "stream"]
    base = [FAKE, 4, 256, 2, FAKE, 0, 8, 1, FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 0, 16, NULL,
            FAKE, 1 << 20, NULL]

    def call(**over):
        a = list(base)
        for n, v in over.items():
            a[names.index(n)] = v
        return lib.cdl_permute_fp8(*a)

    assert call(H=200) == EUNSUP
    assert call(q=NULL) == ENULL
    assert call(s=NULL) == ENULL
    assert call(q=ctypes.c_void_p(0x1004)) == EUNSUP
    assert call(counts=NULL) == ENULL
    assert call(sf=4) == EUNSUP                      # packed needs UE8M0
    assert call(sf=8) == EUNSUP                      # unknown flag


def test_fp8_scale_bytes():
    f = cdl.library().cdl_fp8_scale_bytes
    assert f(10, 256, 0, 10) == 10 * 2 * 4
    assert f(10, 256, 2, 10) == 2 * 12 * 4          # [G][ld], ld = 12
    assert f(10, 640, 5, 10) == 10 * 2 * 4          # 5 groups -> 2 words per row
    assert f(10, 640, 7, 3) == 4 * 2 * 4 * 4        # 4 matrices of [2 words][ld 4]
    assert f(10, 200, 0, 10) == 0                   # H % 128
    assert f(10, 256, 4, 10) == 0                   # packed without UE8M0


def test_dispatch_fp8_ex_and_ll_fp8_reject():
    lib = cdl.library()
    f = lib.cdl_dispatch_fp8_ex
    # x, T, H, k, s2d, q, s, sf, cap, status, stream
    assert f(FAKE, 4, 256, 2, FAKE, FAKE, FAKE, 6, 8, NULL, NULL) == EUNSUP
    assert f(FAKE, 4, 200, 2, FAKE, FAKE, FAKE, 0, 8, NULL, NULL) == EUNSUP
    assert f(FAKE, 4, 256, 2, FAKE, NULL, FAKE, 0, 8, NULL, NULL) == ENULL
    g = lib.cdl_dispatch_ll_fp8
    # x, T, H, k, ids, b, L, s2d, seg, counts, cap, q, s, sf, mm, ll, status, stream
    args = [FAKE, 4, 256, 2, FAKE, 0, 8, FAKE, FAKE, FAKE, 16, FAKE, FAKE, 0, FAKE, FAKE, NULL, NULL]
    a = list(args); a[13] = 4
    assert g(*a) == EUNSUP
    a = list(args); a[12] = NULL
    assert g(*a) == ENULL
    a = list(args); a[2] = 200
    assert g(*a) == EUNSUP


def test_rank_layout_rejects():
    lib = cdl.library()
    assert lib.cdl_rank_layout_workspace_size(16, 2, 256, 8, 4) > 0
    assert lib.cdl_rank_layout_workspace_size(16, 2, 250, 8, 4) == 0        # E % R
    assert lib.cdl_rank_layout_workspace_size(16, 2, 256, 8, 3) == 0        # R % rpn
    assert lib.cdl_rank_layout_workspace_size(16, 2, 9000, 8, 1) == 0       # E too large
    f = lib.cdl_rank_layout
    # ids, T, k, E, R, rpn, per_rank, per_node, per_expert, in_rank, ws, wsb, stream
    assert f(FAKE, 16, 2, 250, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, NULL) == EUNSUP
    assert f(FAKE, 16, 2, 256, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, NULL) == ESIZE
    assert f(FAKE, 16, 2, 256, 8, 1, NULL, FAKE, FAKE, FAKE, FAKE, 1 << 20, NULL) == ENULL
    assert f(FAKE, 16, 2, 256, 8, 1, FAKE, FAKE, NULL, FAKE, FAKE, 1 << 20, NULL) == ENULL
    assert f(FAKE, 16, 2, 256, 8, 1, FAKE, FAKE, FAKE, NULL, FAKE, 1 << 20, NULL) == ENULL
    assert f(FAKE, 16, 2, 256, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 8, NULL) == EWS


def test_permute_fp8_tensor_rejects():
    lib = cdl.library()
    P = ctypes.c_void_p
    cnt, seg, s2d, reo, q = FAKE, FAKE, FAKE, FAKE, FAKE
    ws_b = lib.cdl_dispatch_layout_workspace_size(64, 2, 8)

    def call(x=FAKE, T=64, H=256, k=2, ids=FAKE, L=8, A=1, out=FAKE, scale=None, cap=128,
             ws=FAKE, wsb=ws_b):
        return lib.cdl_permute_fp8_tensor(x, T, H, k, ids, 0, L, A, cnt, seg, s2d, reo, 128, out,
                                          scale, cap, None, ws, wsb, None)
    assert call(x=NULL) == ENULL
    assert call(out=NULL) == ENULL
    assert call(H=12) == EUNSUP                               # H % 8
    assert call(x=P(0x1008)) == EUNSUP                        # x not 16-byte aligned
    assert call(out=P(0x1004)) == EUNSUP                      # out_q not 8-byte aligned
    assert call(scale=P(0x1002)) == EUNSUP                    # scale not 4-byte aligned
    assert call(cap=-1) == ESIZE
    assert call(H=(1 << 24) + 8) == EBIG
    assert call(wsb=16) == EWS


def test_header_is_plain_c_and_links(tmp_path):
    """include/cdl.h compiles as C99 with no HIP or torch header, and a C
    program links against libcdl.so and calls its pure host functions."""
    import subprocess
    src = tmp_path / "use_cdl.c"
    src.write_text(
        '#include <stdio.h>\n#include "cdl.h"\n'
        "int main(void) {\n"
        "    if (cdl_ll_expected_m(128, 8, 8, 256) != 33) return 1;\n"
        "    if (cdl_dispatch_layout_workspace_size(4096, 8, 32) == 0) return 2;\n"
        "    if (cdl_status_string(CDL_OK) == 0) return 3;\n"
        "    if (cdl_dispatch_layout(0, -1, 8, 0, 32, 0, 0, 0, 0, 0, 0, 0) != CDL_ERR_BAD_SIZE) return 4;\n"
        '    printf("ok\\n");\n    return 0;\n}\n')
    exe = tmp_path / "use_cdl"
    lib_dir = os.path.dirname(cdl.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", lib_dir, "-lcdl",
                    "-Wl,-rpath," + lib_dir], check=True, capture_output=True, timeout=120)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


class _NoLaunch:
    """The real library for its host-only size queries; any other entry point
    (one that would enqueue work) fails the test if reached."""

    HOST_ONLY = {"cdl_dispatch_layout_workspace_size", "cdl_permute_fp8_workspace_size",
                 "cdl_fp8_scale_bytes", "cdl_status_string"}

    def __init__(self, lib):
        self._lib = lib
        self.launched = []

    def __getattr__(self, name):
        if name in self.HOST_ONLY:
            return getattr(self._lib, name)
        self.launched.append(name)
        raise AssertionError("%s reached before the argument checks refused the call" % name)


@pytest.fixture
def no_launch(monkeypatch):
    """The binding on CPU tensors with the GPU-tensor check lifted, so that
    the shape checks behind it can be exercised without a GPU."""
    import combine_dispatch_layout_amd.api as api
    stub = _NoLaunch(api.library())
    monkeypatch.setattr(api, "library", lambda: stub)
    monkeypatch.setattr(api, "_need_gpu", lambda t, name: None)
    return stub


def test_fp8_calls_refuse_a_narrow_out_q_before_any_launch(no_launch):
    """The fp8 kernels write H bytes per destination row at row * H: an out_q
    narrower than H is refused by the binding, before any kernel is queued."""
    import torch
    T, k, L, H = 8, 2, 4, 256
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    ids = torch.zeros(T, k, dtype=torch.int32)
    narrow = torch.empty(T * k, H - 128, dtype=torch.uint8)
    flat = torch.empty(T * k * H, dtype=torch.uint8)
    for bad in (narrow, flat):
        with pytest.raises(ValueError, match="out_q"):
            cdl.permute_fp8(x, ids, 0, L, out_q=bad)
        with pytest.raises(ValueError, match="out_q"):
            cdl.permute_fp8_tensor(x, ids, 0, L, out_q=bad)
        lay = cdl.Layout(T, k, 0, L, ids, torch.empty(L, dtype=torch.int32),
                         torch.empty(L + 1, dtype=torch.int64),
                         torch.empty(T * k, dtype=torch.int32),
                         torch.empty(T * k, dtype=torch.int32))
        with pytest.raises(ValueError, match="out_q"):
            cdl.dispatch_fp8(x, lay, out_q=bad)
    assert no_launch.launched == []


def test_permute_noalloc_refuses_before_any_hip_call():
    """cdl_permute_noalloc checks its sizes, and that the layout's scratch
    fits its static buffer, on the host before any HIP call (so this runs
    without a GPU)."""
    lib = cdl.library()
    f = lib.cdl_permute_noalloc
    T, k, L = 1 << 22, 64, 2048
    assert lib.cdl_dispatch_layout_workspace_size(T, k, L) > cdl.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, T, 128, k, FAKE, 0, L, 1, FAKE, FAKE, FAKE, FAKE, T * k, FAKE, 1, NULL,
             NULL) == cdl.CDL_ERR_SCRATCH
    assert f(FAKE, 8, 128, 0, FAKE, 0, 4, 1, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 1, NULL,
             NULL) == ESIZE
    assert f(FAKE, 8, 128, 2, FAKE, 0, 0, 1, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 1, NULL,
             NULL) == ESIZE
    assert "scratch" in cdl.status_string(cdl.CDL_ERR_SCRATCH)
    assert lib.cdl_dispatch_layout_workspace_size(4096, 8, 32) <= cdl.NOALLOC_SCRATCH_BYTES
