"""Python binding of libcdl (argument marshalling only).

Every step of the hot path runs in the HIP kernels of ``libcdl.so``; this
module checks tensor devices, dtypes and shapes, allocates outputs with torch
(device memory only) and passes raw pointers and the current HIP stream to
the C ABI declared in ``include/cdl.h``.  There is no CPU fallback: if the
library is not built, or a tensor is not on a GPU, the call raises.

The calls mirror the dispatcher pages' flow ([0.4.4 diff]
_DeepEPDispatcherImplNormal: preprocess -> permute -> post-reorder combine;
[deepep.py] _DeepEPDispatcherImplLowLatency: low-latency dispatch returning
masked_m, and combine with the top-k weights):

    lay = dispatch_layout(topk_ids, expert_begin, num_local_experts)
    rows = dispatch(x, lay)                      # [R, H] bf16, expert-major
    lay, rows = permute(x, topk_ids, expert_begin, num_local_experts)  # both
    q, scales = dispatch_fp8(x, lay)             # [R, H] e4m3fn + [R, H/128] f32
    buf, masked_m, ll_map = dispatch_ll(x, lay, cap)   # [L, cap, H]
    out = combine(expert_out, lay.src2dst, topk_weights)  # [T, H] bf16
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcdl.so")

CDL_OK = 0
CDL_STATUS_ROWS_OVERFLOW = 1
CDL_STATUS_LL_OVERFLOW = 2
CDL_STATUS_MAP_RANGE = 4
CDL_STATUS_REORDER_OVERFLOW = 8
CDL_ERR_SCRATCH = -7
NOALLOC_SCRATCH_BYTES = 1 << 20
FP8_GROUP = 128
FP8_SCALE_UE8M0 = 1
FP8_SCALE_COLMAJOR = 2
FP8_SCALE_PACKED = 4

_lib = None


class CdlError(RuntimeError):
    """A libcdl call returned a negative status code."""

    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s: %s (code %d)" % (what, status_string(code), code))


def library():
    """Load libcdl.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libcdl.so is not built at %s; run __graft_entry__.build() or "
                "python -m combine_dispatch_layout_amd.build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.cdl_dispatch_layout_workspace_size.argtypes = [i64, i32, i32]
        L.cdl_dispatch_layout_workspace_size.restype = sz
        L.cdl_dispatch_layout.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.cdl_dispatch_layout.restype = ctypes.c_int
        L.cdl_dispatch_layout_aligned.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp,
                                                  i64, vp, vp, sz, vp]
        L.cdl_dispatch_layout_aligned.restype = ctypes.c_int
        L.cdl_permute.argtypes = [vp, i64, i64, i32, vp, i32, i32, i32, vp, vp, vp, vp, i64, vp,
                                  i64, vp, vp, sz, vp]
        L.cdl_permute.restype = ctypes.c_int
        L.cdl_permute_noalloc.argtypes = [vp, i64, i64, i32, vp, i32, i32, i32, vp, vp, vp, vp,
                                          i64, vp, i64, vp, vp]
        L.cdl_permute_noalloc.restype = ctypes.c_int
        L.cdl_permute_fp8.argtypes = [vp, i64, i64, i32, vp, i32, i32, i32, vp, vp, vp, vp, i64,
                                      vp, vp, i32, i64, vp, vp, sz, vp]
        L.cdl_fp8_scale_bytes.argtypes = [i64, i64, i32, i64]
        L.cdl_fp8_scale_bytes.restype = sz
        L.cdl_dispatch_fp8_ex.argtypes = [vp, i64, i64, i32, vp, vp, vp, i32, i64, vp, vp]
        L.cdl_dispatch_fp8_ex.restype = ctypes.c_int
        L.cdl_dispatch_ll_fp8.argtypes = [vp, i64, i64, i32, vp, i32, i32, vp, vp, vp, i64, vp, vp,
                                          i32, vp, vp, vp, vp]
        L.cdl_dispatch_ll_fp8.restype = ctypes.c_int
        L.cdl_permute_fp8.restype = ctypes.c_int
        L.cdl_rank_layout_workspace_size.argtypes = [i64, i32, i32, i32, i32]
        L.cdl_rank_layout_workspace_size.restype = sz
        L.cdl_permute_fp8_tensor.argtypes = [vp, i64, i64, i32, vp, i32, i32, i32, vp, vp, vp,
                                             vp, i64, vp, vp, i64, vp, vp, sz, vp]
        L.cdl_permute_fp8_tensor.restype = ctypes.c_int
        L.cdl_permute_fp8_workspace_size.argtypes = [i64, i32, i32, i64, i32, i64]
        L.cdl_permute_fp8_workspace_size.restype = sz
        L.cdl_rank_layout.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.cdl_rank_layout.restype = ctypes.c_int
        L.cdl_dispatch.argtypes = [vp, i64, i64, i32, vp, vp, i64, vp, vp]
        L.cdl_dispatch.restype = ctypes.c_int
        L.cdl_dispatch_fp8.argtypes = [vp, i64, i64, i32, vp, vp, vp, i64, vp, vp]
        L.cdl_dispatch_fp8.restype = ctypes.c_int
        L.cdl_dispatch_ll.argtypes = [vp, i64, i64, i32, vp, i32, i32, vp, vp, vp, i64, vp, vp,
                                      vp, vp, vp]
        L.cdl_permute_ll.argtypes = [vp, i64, i64, i32, vp, i32, i32, vp, vp, vp, vp, i64, i64, vp,
                                     vp, vp, vp, vp, sz, vp]
        L.cdl_permute_ll.restype = ctypes.c_int
        L.cdl_permute_ll_fp8.argtypes = [vp, i64, i64, i32, vp, i32, i32, vp, vp, vp, vp, i64, i64,
                                         vp, vp, i32, vp, vp, vp, vp, sz, vp]
        L.cdl_permute_ll_fp8.restype = ctypes.c_int
        L.cdl_dispatch_ll.restype = ctypes.c_int
        L.cdl_combine.argtypes = [vp, i64, i64, vp, vp, i64, i32, vp, vp, vp]
        L.cdl_combine.restype = ctypes.c_int
        L.cdl_combine_timed.argtypes = [vp, i64, i64, vp, vp, i64, i32, vp, vp, vp, vp, vp]
        L.cdl_combine_timed.restype = ctypes.c_int
        L.cdl_ll_expected_m.argtypes = [i64, i32, i32, i32]
        L.cdl_ll_expected_m.restype = i64
        L.cdl_status_string.argtypes = [ctypes.c_int]
        L.cdl_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return library().cdl_status_string(int(code)).decode()


def _check(rc: int, what: str) -> None:
    if rc != CDL_OK:
        raise CdlError(rc, what)


# Every entry point has its argtypes declared (library()), so pointers pass as
# plain ints: no ctypes object per argument.
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


# torch's raw current-stream query: the stream handle without building a
# torch.cuda.Stream object (a few microseconds per call otherwise)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _need_gpu(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (libcdl has no CPU path)" % name)


def _need(t: torch.Tensor, name: str, dtype, shape=None) -> None:
    _need_gpu(t, name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _same_device(dev: torch.device, **tensors) -> None:
    """Every given tensor (None skipped) lives on `dev`: the kernels of one
    call run on one device and take every pointer as that device's memory."""
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError("%s is on %s, the call's inputs on %s" % (name, t.device, dev))


def _need_q_rows(t: torch.Tensor, H: int) -> None:
    """out_q of the normal-mode fp8 calls: [rows, H] bytes.  The kernels
    write H bytes per destination row at row * H, up to rows rows, so a
    narrower buffer would be written past its end."""
    _need(t, "out_q", torch.uint8)
    if t.dim() != 2 or t.shape[1] != H:
        raise ValueError("out_q must be [rows, H] with H = %d, got %s" % (H, tuple(t.shape)))


_ROW_DTYPES_2 = (torch.bfloat16, torch.float16, torch.int16)
_ROW_DTYPES_1 = (torch.uint8, torch.int8, torch.float8_e4m3fn, torch.float8_e5m2)


def _rows16(t: torch.Tensor, name: str) -> torch.Tensor:
    """[n, H] rows of 1- or 2-byte elements viewed as 16-bit words.  The
    scatter moves bits, so any such dtype is dispatched exactly: bf16 hidden
    states, or rows already quantised to fp8 per tensor, whose permuted
    buffer stays fp8."""
    _need_gpu(t, name)
    if t.dim() != 2:
        raise ValueError("%s must be [rows, H]" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.dtype in _ROW_DTYPES_2:
        return t.view(torch.int16)
    if t.dtype in _ROW_DTYPES_1:
        if t.shape[1] % 2:
            raise ValueError("%s: rows of 1-byte elements need an even width" % name)
        return t.view(torch.int16)
    raise TypeError("%s must have 1- or 2-byte elements (bf16, fp16, fp8, int8), got %s"
                    % (name, t.dtype))


@dataclasses.dataclass
class Layout:
    """Caller-owned routing layout: the explicit form of the pages' dispatch
    ``handle``.  Device tensors; nothing here is synchronised."""
    T: int
    k: int
    expert_begin: int
    num_local_experts: int
    topk_ids: torch.Tensor          # [T, k] int32 (global ids)
    counts: torch.Tensor            # [L] int32 (true counts)
    seg_indptr: torch.Tensor        # [L+1] int64 (segments padded to `alignment`)
    src2dst: torch.Tensor           # [T*k] int32
    reorder_buf: torch.Tensor       # [T*k + L*(alignment-1)] int32 (first R entries valid)
    alignment: int = 1

    def num_rows(self) -> int:
        """R, the number of dispatched rows (synchronises with the device)."""
        return int(self.seg_indptr[self.num_local_experts].item())

    @property
    def reorder_topk_ids(self) -> torch.Tensor:
        """Local expert of every dispatched row (synchronises for R)."""
        return self.reorder_buf[: self.num_rows()]


def layout_workspace_size(T: int, k: int, L: int) -> int:
    n = library().cdl_dispatch_layout_workspace_size(T, k, L)
    if n == 0:
        raise CdlError(-2, "cdl_dispatch_layout_workspace_size")
    return int(n)


def dispatch_layout(topk_ids: torch.Tensor, expert_begin: int, num_local_experts: int,
                    workspace: Optional[torch.Tensor] = None, alignment: int = 1) -> Layout:
    """Per-expert counts, seg_indptr, src2dst and reorder_topk_ids of the
    rank's slots (global ids outside [expert_begin, expert_begin+L) are
    invalid).  With alignment > 1 every expert segment is padded to a
    multiple of `alignment` rows (padding rows have reorder id -1).  int64
    ids are narrowed to int32 here."""
    lay, ws = _new_layout(topk_ids, expert_begin, num_local_experts, workspace, alignment)
    rc = library().cdl_dispatch_layout_aligned(
        _ptr(lay.topk_ids), lay.T, lay.k, lay.expert_begin, lay.num_local_experts,
        lay.alignment, _ptr(lay.counts), _ptr(lay.seg_indptr), _ptr(lay.src2dst),
        _ptr(lay.reorder_buf), lay.reorder_buf.numel(), None, _ptr(ws),
        ws.numel() * ws.element_size(), _stream(lay.topk_ids.device))
    _check(rc, "cdl_dispatch_layout_aligned")
    return lay


def _new_layout(topk_ids: torch.Tensor, expert_begin: int, num_local_experts: int,
                workspace: Optional[torch.Tensor], alignment: int = 1):
    _need_gpu(topk_ids, "topk_ids")
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, k]")
    if topk_ids.dtype != torch.int32:
        topk_ids = topk_ids.to(torch.int32)
    topk_ids = topk_ids.contiguous()
    T, k = topk_ids.shape
    L = int(num_local_experts)
    dev = topk_ids.device
    ws_bytes = layout_workspace_size(T, k, L)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError("workspace too small: need %d bytes" % ws_bytes)
    A = int(alignment)
    if A < 1:
        raise ValueError("alignment must be >= 1")
    lay = Layout(T, k, int(expert_begin), L, topk_ids,
                 torch.empty(L, dtype=torch.int32, device=dev),
                 torch.empty(L + 1, dtype=torch.int64, device=dev),
                 torch.empty(T * k, dtype=torch.int32, device=dev),
                 torch.empty(max(T * k + L * (A - 1), 1), dtype=torch.int32, device=dev), A)
    return lay, workspace


def permute(x: torch.Tensor, topk_ids: torch.Tensor, expert_begin: int, num_local_experts: int,
            out: Optional[torch.Tensor] = None, rows: Optional[int] = None,
            status: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None,
            alignment: int = 1) -> Tuple[Layout, torch.Tensor]:
    """Layout + normal-mode scatter in one call (two kernels, one for T*k <= 4096).  `out` holds
    `rows` rows (default T*k + L*(alignment-1), an upper bound on R); the
    first R rows receive the dispatched rows (padding rows are not written).
    Returns (layout, out).  x holds bf16 rows, or any 1- or 2-byte element
    type (rows are copied bit for bit; `out` has x's dtype)."""
    xw = _rows16(x, "x")
    lay, ws = _new_layout(topk_ids, expert_begin, num_local_experts, workspace, alignment)
    T, k, L = lay.T, lay.k, lay.num_local_experts
    if x.shape[0] != T:
        raise ValueError("x must be [T, H] with T = %d" % T)
    if out is None:
        out = torch.empty(lay.reorder_buf.numel() if rows is None else int(rows), x.shape[1],
                          dtype=x.dtype, device=x.device)
    if out.dtype != x.dtype or out.dim() != 2 or out.shape[1] != x.shape[1]:
        raise ValueError("out must be [rows, H] of x's dtype")
    ow = _rows16(out, "out")
    H = xw.shape[1]
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(x.device, topk_ids=lay.topk_ids, out=out, status=status, workspace=ws)
    rc = library().cdl_permute(_ptr(xw), T, H, k, _ptr(lay.topk_ids), lay.expert_begin, L,
                               lay.alignment, _ptr(lay.counts), _ptr(lay.seg_indptr),
                               _ptr(lay.src2dst), _ptr(lay.reorder_buf), lay.reorder_buf.numel(),
                               _ptr(ow), ow.shape[0], _ptr(status), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(x.device))
    _check(rc, "cdl_permute")
    return lay, out


def permute_fp8(x: torch.Tensor, topk_ids: torch.Tensor, expert_begin: int,
                num_local_experts: int, rows: Optional[int] = None,
                out_q: Optional[torch.Tensor] = None, out_scales: Optional[torch.Tensor] = None,
                status: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                alignment: int = 1, scale_flags: int = 0):
    """Layout + fp8 (e4m3fn, groups of 128) scatter in one call.  Returns
    (layout, q [rows, H] uint8, scales [rows, H/128] fp32)."""
    _need(x, "x", torch.bfloat16)
    lay, ws = _new_layout(topk_ids, expert_begin, num_local_experts, workspace, alignment)
    T, k, L = lay.T, lay.k, lay.num_local_experts
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T = %d" % T)
    H = x.shape[1]
    if H % FP8_GROUP:
        raise CdlError(-3, "permute_fp8 (H must be a multiple of 128)")
    n = lay.reorder_buf.numel() if rows is None else int(rows)
    if out_q is None:
        out_q = torch.empty(n, H, dtype=torch.uint8, device=x.device)
    if out_scales is None:
        out_scales = new_scale_tensor(out_q.shape[0], H, scale_flags, x.device)
    _need_q_rows(out_q, H)
    _check_scale_buffer(out_scales, out_q.shape[0], H, scale_flags, out_q.shape[0])
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(x.device, topk_ids=lay.topk_ids, out_q=out_q, out_scales=out_scales,
                 status=status, workspace=ws)
    rc = library().cdl_permute_fp8(_ptr(x), T, H, k, _ptr(lay.topk_ids), lay.expert_begin, L,
                                   lay.alignment, _ptr(lay.counts), _ptr(lay.seg_indptr),
                                   _ptr(lay.src2dst), _ptr(lay.reorder_buf),
                                   lay.reorder_buf.numel(), _ptr(out_q), _ptr(out_scales),
                                   int(scale_flags), out_q.shape[0], _ptr(status), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(x.device))
    _check(rc, "cdl_permute_fp8")
    return lay, out_q, out_scales


def permute_fp8_tensor(x: torch.Tensor, topk_ids: torch.Tensor, expert_begin: int,
                       num_local_experts: int, scale: Optional[torch.Tensor] = None,
                       rows: Optional[int] = None, out_q: Optional[torch.Tensor] = None,
                       status: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, alignment: int = 1):
    """Layout + scatter with every row cast to fp8 per tensor:
    e4m3fn(clamp(x / scale, +-448)), scale a device fp32 scalar or None for 1
    (the w8a8 per-tensor permuted buffer).  Returns (layout, q [rows, H] uint8
    holding e4m3fn bytes)."""
    _need(x, "x", torch.bfloat16)
    lay, ws = _new_layout(topk_ids, expert_begin, num_local_experts, workspace, alignment)
    T, k, L = lay.T, lay.k, lay.num_local_experts
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T = %d" % T)
    H = x.shape[1]
    n = lay.reorder_buf.numel() if rows is None else int(rows)
    if out_q is None:
        out_q = torch.empty(n, H, dtype=torch.uint8, device=x.device)
    _need_q_rows(out_q, H)
    if scale is not None:
        _need(scale, "scale", torch.float32)
        if scale.numel() != 1:
            raise ValueError("scale must hold one value")
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(x.device, topk_ids=lay.topk_ids, out_q=out_q, scale=scale, status=status,
                 workspace=ws)
    rc = library().cdl_permute_fp8_tensor(_ptr(x), T, H, k, _ptr(lay.topk_ids), lay.expert_begin,
                                          L, lay.alignment, _ptr(lay.counts),
                                          _ptr(lay.seg_indptr), _ptr(lay.src2dst),
                                          _ptr(lay.reorder_buf), lay.reorder_buf.numel(),
                                          _ptr(out_q), _ptr(scale), out_q.shape[0],
                                          _ptr(status), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(x.device))
    _check(rc, "cdl_permute_fp8_tensor")
    return lay, out_q


@dataclasses.dataclass
class RankLayout:
    """Where a token batch goes before the exchange (device tensors)."""
    num_tokens_per_rank: torch.Tensor       # [R] int32
    num_tokens_per_rdma_rank: torch.Tensor  # [R / ranks_per_node] int32
    num_tokens_per_expert: torch.Tensor     # [E] int32 (global experts)
    is_token_in_rank: torch.Tensor          # [T, R] bool


def rank_layout(topk_ids: torch.Tensor, num_experts: int, num_ranks: int,
                ranks_per_node: int = 1) -> RankLayout:
    """Per-rank / per-node token counts, per-expert slot counts and the
    token-in-rank table of global top-k ids (ids outside [0, E) are
    unrouted)."""
    _need_gpu(topk_ids, "topk_ids")
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, k]")
    ids = topk_ids.to(torch.int32).contiguous()
    T, k = ids.shape
    E, R, rpn = int(num_experts), int(num_ranks), int(ranks_per_node)
    wsb = library().cdl_rank_layout_workspace_size(T, k, E, R, rpn)
    if wsb == 0:
        raise CdlError(-3, "cdl_rank_layout_workspace_size (sizes)")
    dev = ids.device
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    out = RankLayout(torch.empty(R, dtype=torch.int32, device=dev),
                     torch.empty(R // rpn, dtype=torch.int32, device=dev),
                     torch.empty(E, dtype=torch.int32, device=dev),
                     torch.empty(T, R, dtype=torch.bool, device=dev))
    rc = library().cdl_rank_layout(_ptr(ids), T, k, E, R, rpn, _ptr(out.num_tokens_per_rank),
                                   _ptr(out.num_tokens_per_rdma_rank),
                                   _ptr(out.num_tokens_per_expert), _ptr(out.is_token_in_rank),
                                   _ptr(ws), wsb, _stream(dev))
    _check(rc, "cdl_rank_layout")
    return out


def permute_fp8_workspace_size(T: int, k: int, L: int, H: int, scale_flags: int,
                               rows: int) -> int:
    """Workspace bytes for permute_fp8 (rows = output rows) and
    permute_ll_fp8 (rows = L * cap) in a scale format: the layout workspace
    size for every valid format."""
    n = library().cdl_permute_fp8_workspace_size(T, k, L, H, scale_flags, rows)
    if n == 0:
        raise CdlError(-3, "cdl_permute_fp8_workspace_size")
    return int(n)


def fp8_scale_bytes(rows: int, H: int, scale_flags: int = 0, rows_per_mat: int = 0) -> int:
    n = library().cdl_fp8_scale_bytes(rows, H, scale_flags, rows_per_mat or max(rows, 1))
    if n == 0 and rows > 0:
        raise CdlError(-3, "cdl_fp8_scale_bytes (format)")
    return int(n)


def new_scale_tensor(rows: int, H: int, scale_flags: int, device, rows_per_mat: int = 0):
    """A scale buffer of the right size, typed and shaped for its format:
    fp32 [rows, G] (row-major), fp32 [mats, G, ld] (column-major), int32
    [rows, ceil(G/4)] or [mats, ceil(G/4), ld] (packed exponent bytes)."""
    G = H // FP8_GROUP
    rpm = rows_per_mat or max(rows, 1)
    packed = bool(scale_flags & FP8_SCALE_PACKED)
    dtype = torch.int32 if packed else torch.float32
    words = -(-G // 4) if packed else G
    if scale_flags & FP8_SCALE_COLMAJOR:
        mats = -(-rows // rpm) if rows else 0
        ld = -(-rpm // 4) * 4
        t = torch.empty(mats, words, ld, dtype=dtype, device=device)
    else:
        t = torch.empty(rows, words, dtype=dtype, device=device)
    assert t.numel() * 4 == fp8_scale_bytes(rows, H, scale_flags, rpm)
    return t


def dispatch(x: torch.Tensor, layout: Layout, out: Optional[torch.Tensor] = None,
             rows: Optional[int] = None, status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Normal-mode scatter: out[src2dst[t*k+j]] = x[t].  Allocates [R, H]
    (reading R from the device) unless `out` or `rows` is given.  x holds bf16
    rows, or any 1- or 2-byte element type (e.g. fp8 rows quantised per
    tensor): rows are copied bit for bit and `out` has x's dtype."""
    T, k = layout.T, layout.k
    xw = _rows16(x, "x")
    if x.shape[0] != T:
        raise ValueError("x must be [T, H] with T = %d" % T)
    if out is None:
        n = layout.num_rows() if rows is None else int(rows)
        out = torch.empty(n, x.shape[1], dtype=x.dtype, device=x.device)
    if out.dtype != x.dtype or out.dim() != 2 or out.shape[1] != x.shape[1]:
        raise ValueError("out must be [rows, H] of x's dtype")
    ow = _rows16(out, "out")
    H = xw.shape[1]
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(x.device, src2dst=layout.src2dst, out=out, status=status)
    rc = library().cdl_dispatch(_ptr(xw), T, H, k, _ptr(layout.src2dst), _ptr(ow), ow.shape[0],
                                _ptr(status), _stream(x.device))
    _check(rc, "cdl_dispatch")
    return out


def dispatch_fp8(x: torch.Tensor, layout: Layout, out_q: Optional[torch.Tensor] = None,
                 out_scales: Optional[torch.Tensor] = None, rows: Optional[int] = None,
                 status: Optional[torch.Tensor] = None,
                 scale_flags: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Normal-mode scatter with per-token groups of 128 quantised to
    e4m3fn.  Returns (q [rows, H] uint8 holding e4m3fn bytes, scales in the
    `scale_flags` format -- fp32 [rows, H/128] by default);
    ``q.view(torch.float8_e4m3fn)`` reinterprets."""
    T, k = layout.T, layout.k
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T = %d" % T)
    H = x.shape[1]
    if H % FP8_GROUP:
        raise CdlError(-3, "dispatch_fp8 (H must be a multiple of 128)")
    if out_q is None:
        n = layout.num_rows() if rows is None else int(rows)
        out_q = torch.empty(n, H, dtype=torch.uint8, device=x.device)
    if out_scales is None:
        out_scales = new_scale_tensor(out_q.shape[0], H, scale_flags, x.device)
    _need_q_rows(out_q, H)
    _check_scale_buffer(out_scales, out_q.shape[0], H, scale_flags, out_q.shape[0])
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(x.device, src2dst=layout.src2dst, out_q=out_q, out_scales=out_scales,
                 status=status)
    rc = library().cdl_dispatch_fp8_ex(_ptr(x), T, H, k, _ptr(layout.src2dst), _ptr(out_q),
                                       _ptr(out_scales), int(scale_flags), out_q.shape[0],
                                       _ptr(status), _stream(x.device))
    _check(rc, "cdl_dispatch_fp8_ex")
    return out_q, out_scales


def _check_scale_buffer(t: torch.Tensor, rows: int, H: int, scale_flags: int, rpm: int) -> None:
    _need_gpu(t, "out_scales")
    if not t.is_contiguous():
        raise ValueError("out_scales must be contiguous")
    need = fp8_scale_bytes(rows, H, scale_flags, rpm)
    if t.numel() * t.element_size() < need:
        raise ValueError("out_scales holds %d bytes, the format needs %d"
                         % (t.numel() * t.element_size(), need))


def dispatch_ll(x: torch.Tensor, layout: Layout, cap: int, out: Optional[torch.Tensor] = None,
                status: Optional[torch.Tensor] = None):
    """Low-latency dispatch into a padded [L, cap, H] buffer.  Returns (out,
    masked_m [L] int32, ll_src2dst [T*k] int32).  Rows at or beyond
    masked_m[e] are left as they were (never cleared)."""
    T, k, L = layout.T, layout.k, layout.num_local_experts
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T = %d" % T)
    H = x.shape[1]
    if out is None:
        out = torch.empty(L, cap, H, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (L, cap, H))
    masked_m = torch.empty(L, dtype=torch.int32, device=x.device)
    ll_map = torch.empty(T * k, dtype=torch.int32, device=x.device)
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(x.device, topk_ids=layout.topk_ids, out=out, status=status)
    rc = library().cdl_dispatch_ll(_ptr(x), T, H, k, _ptr(layout.topk_ids), layout.expert_begin,
                                   L, _ptr(layout.src2dst), _ptr(layout.seg_indptr),
                                   _ptr(layout.counts), int(cap), _ptr(out), _ptr(masked_m),
                                   _ptr(ll_map), _ptr(status), _stream(x.device))
    _check(rc, "cdl_dispatch_ll")
    return out, masked_m, ll_map


def dispatch_ll_fp8(x: torch.Tensor, layout: Layout, cap: int, scale_flags: int = 0,
                    out_q: Optional[torch.Tensor] = None,
                    out_scales: Optional[torch.Tensor] = None,
                    status: Optional[torch.Tensor] = None):
    """Low-latency dispatch with fp8 rows.  Returns (q [L, cap, H] uint8,
    scales (every expert's cap rows are one matrix of the format), masked_m,
    ll_src2dst)."""
    T, k, L = layout.T, layout.k, layout.num_local_experts
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T = %d" % T)
    H = x.shape[1]
    if H % FP8_GROUP:
        raise CdlError(-3, "dispatch_ll_fp8 (H must be a multiple of 128)")
    if out_q is None:
        out_q = torch.empty(L, cap, H, dtype=torch.uint8, device=x.device)
    _need(out_q, "out_q", torch.uint8, (L, cap, H))
    if out_scales is None:
        out_scales = new_scale_tensor(L * cap, H, scale_flags, x.device, rows_per_mat=cap)
        if not scale_flags & FP8_SCALE_COLMAJOR:
            out_scales = out_scales.view(L, cap, -1)
    _check_scale_buffer(out_scales, L * cap, H, scale_flags, cap)
    masked_m = torch.empty(L, dtype=torch.int32, device=x.device)
    ll_map = torch.empty(T * k, dtype=torch.int32, device=x.device)
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(x.device, topk_ids=layout.topk_ids, out_q=out_q, out_scales=out_scales,
                 status=status)
    rc = library().cdl_dispatch_ll_fp8(_ptr(x), T, H, k, _ptr(layout.topk_ids),
                                       layout.expert_begin, L, _ptr(layout.src2dst),
                                       _ptr(layout.seg_indptr), _ptr(layout.counts), int(cap),
                                       _ptr(out_q), _ptr(out_scales), int(scale_flags),
                                       _ptr(masked_m), _ptr(ll_map), _ptr(status),
                                       _stream(x.device))
    _check(rc, "cdl_dispatch_ll_fp8")
    return out_q, out_scales, masked_m, ll_map


def permute_ll(x: torch.Tensor, topk_ids: torch.Tensor, expert_begin: int,
               num_local_experts: int, cap: int, out: Optional[torch.Tensor] = None,
               status: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """The low-latency dispatch in one call: layout + padded [L, cap, H]
    scatter.  Returns (layout, out, masked_m, ll_src2dst)."""
    _need(x, "x", torch.bfloat16)
    lay, ws = _new_layout(topk_ids, expert_begin, num_local_experts, workspace, 1)
    T, k, L = lay.T, lay.k, lay.num_local_experts
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T = %d" % T)
    H = x.shape[1]
    if out is None:
        out = torch.empty(L, cap, H, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (L, cap, H))
    masked_m = torch.empty(L, dtype=torch.int32, device=x.device)
    ll_map = torch.empty(T * k, dtype=torch.int32, device=x.device)
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(x.device, topk_ids=lay.topk_ids, out=out, status=status, workspace=ws)
    rc = library().cdl_permute_ll(_ptr(x), T, H, k, _ptr(lay.topk_ids), lay.expert_begin, L,
                                  _ptr(lay.counts), _ptr(lay.seg_indptr), _ptr(lay.src2dst),
                                  _ptr(lay.reorder_buf), lay.reorder_buf.numel(), int(cap),
                                  _ptr(out), _ptr(masked_m), _ptr(ll_map), _ptr(status), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(x.device))
    _check(rc, "cdl_permute_ll")
    return lay, out, masked_m, ll_map


def permute_ll_fp8(x: torch.Tensor, topk_ids: torch.Tensor, expert_begin: int,
                   num_local_experts: int, cap: int, scale_flags: int = 0,
                   out_q: Optional[torch.Tensor] = None,
                   out_scales: Optional[torch.Tensor] = None,
                   status: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None):
    """permute_ll with fp8 rows.  Returns (layout, q [L, cap, H] uint8,
    scales, masked_m, ll_src2dst)."""
    _need(x, "x", torch.bfloat16)
    lay, ws = _new_layout(topk_ids, expert_begin, num_local_experts, workspace, 1)
    T, k, L = lay.T, lay.k, lay.num_local_experts
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H] with T = %d" % T)
    H = x.shape[1]
    if H % FP8_GROUP:
        raise CdlError(-3, "permute_ll_fp8 (H must be a multiple of 128)")
    if out_q is None:
        out_q = torch.empty(L, cap, H, dtype=torch.uint8, device=x.device)
    _need(out_q, "out_q", torch.uint8, (L, cap, H))
    if out_scales is None:
        out_scales = new_scale_tensor(L * cap, H, scale_flags, x.device, rows_per_mat=cap)
        if not scale_flags & FP8_SCALE_COLMAJOR:
            out_scales = out_scales.view(L, cap, -1)
    _check_scale_buffer(out_scales, L * cap, H, scale_flags, cap)
    masked_m = torch.empty(L, dtype=torch.int32, device=x.device)
    ll_map = torch.empty(T * k, dtype=torch.int32, device=x.device)
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(x.device, topk_ids=lay.topk_ids, out_q=out_q, out_scales=out_scales,
                 status=status, workspace=ws)
    rc = library().cdl_permute_ll_fp8(_ptr(x), T, H, k, _ptr(lay.topk_ids), lay.expert_begin, L,
                                      _ptr(lay.counts), _ptr(lay.seg_indptr), _ptr(lay.src2dst),
                                      _ptr(lay.reorder_buf), lay.reorder_buf.numel(), int(cap),
                                      _ptr(out_q), _ptr(out_scales), int(scale_flags),
                                      _ptr(masked_m), _ptr(ll_map), _ptr(status), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(x.device))
    _check(rc, "cdl_permute_ll_fp8")
    return lay, out_q, out_scales, masked_m, ll_map


def combine(y: torch.Tensor, map_: torch.Tensor, topk_weights: torch.Tensor,
            out: Optional[torch.Tensor] = None,
            status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = bf16(sum over valid j of w[t,j] * y[map[t*k+j]]) with fp32
    accumulation.  `y` is [rows, H] or the low-latency [L, cap, H] buffer;
    `map_` is src2dst or ll_src2dst."""
    _need_gpu(y, "y")
    if y.dtype != torch.bfloat16 or not y.is_contiguous():
        raise TypeError("y must be a contiguous bfloat16 tensor")
    H = y.shape[-1]
    y_rows = y.numel() // H if H else 0
    _need(topk_weights, "topk_weights", torch.float32)
    if topk_weights.dim() != 2:
        raise ValueError("topk_weights must be [T, k]")
    T, k = topk_weights.shape
    _need(map_, "map", torch.int32, (T * k,))
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=y.device)
    _need(out, "out", torch.bfloat16, (T, H))
    if status is not None:
        _need(status, "status", torch.int32)
    _same_device(y.device, map=map_, topk_weights=topk_weights, out=out, status=status)
    rc = library().cdl_combine(_ptr(y), y_rows, H, _ptr(map_), _ptr(topk_weights), T, k,
                               _ptr(out), _ptr(status), _stream(y.device))
    _check(rc, "cdl_combine")
    return out


def ll_expected_m(T: int, num_ranks: int, k: int, num_experts: int) -> int:
    return int(library().cdl_ll_expected_m(T, num_ranks, k, num_experts))
