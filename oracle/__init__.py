"""CPU oracle for the MoE dispatch/combine hot path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``cdl_oracle.c`` (plain C,
single-threaded, built with gcc) through ctypes and works on numpy arrays;
it imports nothing from the HIP library's package and shares no code with it.

Every function follows the passage cited in ``cdl_oracle.c``.  All functions
here are pinned by ``tests/test_oracle_*.py`` (brute force on tiny inputs,
library routines, closed forms, format-definition tables and invariants); none
is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cdl_oracle.c")
# CDL_ORACLE_LIB names another build of cdl_oracle.c to load instead (the
# sanitizer test runs the pins against an ASan/UBSan build that way)
_LIB = os.environ.get("CDL_ORACLE_LIB") or os.path.join(_HERE, "libcdl_oracle.so")

GCC_FLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


_SRC_OMP = os.path.join(_HERE, "cdl_oracle_omp.c")
_LIB_OMP = os.path.join(_HERE, "libcdl_oracle_omp.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libcdl_oracle.so``, and its
    all-core timing build (the same loops over tokens with OpenMP, for the
    benchmark's CPU baseline only) into ``oracle/libcdl_oracle_omp.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    if force or not os.path.exists(_LIB_OMP):
        tmp = _LIB_OMP + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-fopenmp", "-o", tmp, _SRC, _SRC_OMP, "-lm"])
        os.replace(tmp, _LIB_OMP)
    return _LIB


_lib = None

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def lib():
    """Load the oracle library, building it first if nothing is built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_e4m3fn_to_f32.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3fn_to_f32.restype = ctypes.c_float
        L.oracle_e4m3fn_rne.argtypes = [ctypes.c_float]
        L.oracle_e4m3fn_rne.restype = ctypes.c_uint8
        L.oracle_layout.argtypes = [_i32p, _i64, _i32, _i32, _i32, _i32p, _i64p,
                                    _i32p, _i32p]
        L.oracle_layout.restype = _i64
        L.oracle_layout_aligned.argtypes = [_i32p, _i64, _i32, _i32, _i32, _i32, _i32p,
                                            _i64p, _i32p, _i32p]
        L.oracle_layout_aligned.restype = _i64
        L.oracle_rank_layout.argtypes = [_i32p, _i64, _i32, _i32, _i32, _i32, _i32p, _i32p,
                                         _i32p, _u8p]
        L.oracle_rank_layout.restype = _i32
        L.oracle_quant_group_fp8_ue8m0.argtypes = [_u16p, _i64, _u8p,
                                                   ctypes.POINTER(ctypes.c_float),
                                                   ctypes.POINTER(ctypes.c_int32)]
        L.oracle_quant_group_fp8_ue8m0.restype = None
        L.oracle_dispatch_fp8_fmt.argtypes = [_u16p, _i64, _i64, _i32, _i32p, _i64, _i32, _i64,
                                              _u8p, _u8p]
        L.oracle_dispatch_fp8_fmt.restype = _i32
        L.oracle_dispatch_ll_fp8.argtypes = [_u16p, _i64, _i64, _i32, _i32p, _i32, _i32, _i64,
                                             _i64, _i32, _u8p, _u8p, _i32p, _i32p]
        L.oracle_dispatch_ll_fp8.restype = _i32
        L.oracle_dispatch.argtypes = [_u16p, _i64, _i64, _i32, _i32p, _u16p]
        L.oracle_dispatch.restype = None
        L.oracle_dispatch_ll.argtypes = [_u16p, _i64, _i64, _i32, _i32p, _i32,
                                         _i32, _i64, _u16p, _i32p, _i32p]
        L.oracle_dispatch_ll.restype = _i32
        L.oracle_cast_fp8_tensor.argtypes = [_u16p, _i64, ctypes.c_float, _u8p]
        L.oracle_cast_fp8_tensor.restype = None
        L.oracle_quant_group_fp8.argtypes = [_u16p, _i64, _u8p,
                                             ctypes.POINTER(ctypes.c_float)]
        L.oracle_quant_group_fp8.restype = None
        L.oracle_dispatch_fp8.argtypes = [_u16p, _i64, _i64, _i32, _i32p, _i64,
                                          _u8p, _f32p]
        L.oracle_dispatch_fp8.restype = _i32
        L.oracle_combine.argtypes = [_u16p, _i64, _i64, _i32p, _f32p, _i64, _i32,
                                     _u16p]
        L.oracle_combine.restype = _i64
        L.oracle_combine_f64.argtypes = [_u16p, _i64, _i64, _i32p, _f32p, _i64,
                                         _i32, _f64p]
        L.oracle_combine_f64.restype = None
        L.oracle_expected_m.argtypes = [_i64, _i32, _i32, _i32]
        L.oracle_expected_m.restype = _i64
        L.oracle_bf16_rne_n.argtypes = [_f32p, _i64, _u16p]
        L.oracle_bf16_rne_n.restype = None
        L.oracle_bf16_to_f32_n.argtypes = [_u16p, _i64, _f32p]
        L.oracle_bf16_to_f32_n.restype = None
        L.oracle_e4m3fn_rne_n.argtypes = [_f32p, _i64, _u8p]
        L.oracle_e4m3fn_rne_n.restype = None
        L.oracle_e4m3fn_to_f32_n.argtypes = [_u8p, _i64, _f32p]
        L.oracle_e4m3fn_to_f32_n.restype = None
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# scalar codecs (format definitions)
# --------------------------------------------------------------------------

def bf16_to_f32(b: int) -> float:
    return lib().oracle_bf16_to_f32(int(b))


def bf16_rne(v: float) -> int:
    return int(lib().oracle_bf16_rne(float(v)))


def e4m3fn_to_f32(b: int) -> float:
    return lib().oracle_e4m3fn_to_f32(int(b))


def e4m3fn_rne(v: float) -> int:
    return int(lib().oracle_e4m3fn_rne(float(v)))


def bf16_rne_array(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32).reshape(-1)
    out = np.zeros(v.size, np.uint16)
    lib().oracle_bf16_rne_n(v, v.size, out)
    return out


def bf16_to_f32_array(b: np.ndarray) -> np.ndarray:
    b = _c(b, np.uint16).reshape(-1)
    out = np.zeros(b.size, np.float32)
    lib().oracle_bf16_to_f32_n(b, b.size, out)
    return out


def e4m3fn_rne_array(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32).reshape(-1)
    out = np.zeros(v.size, np.uint8)
    lib().oracle_e4m3fn_rne_n(v, v.size, out)
    return out


def e4m3fn_to_f32_array(b: np.ndarray) -> np.ndarray:
    b = _c(b, np.uint8).reshape(-1)
    out = np.zeros(b.size, np.float32)
    lib().oracle_e4m3fn_to_f32_n(b, b.size, out)
    return out


# --------------------------------------------------------------------------
# hot-path steps
# --------------------------------------------------------------------------

def layout(topk_ids: np.ndarray, expert_begin: int, L: int):
    """Stable counting-sort layout. Returns counts[L] i32, seg_indptr[L+1] i64,
    src2dst[T*k] i32, reorder_topk_ids[R] i32."""
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    counts = np.zeros(L, np.int32)
    seg = np.zeros(L + 1, np.int64)
    src2dst = np.zeros(T * k, np.int32)
    reorder = np.zeros(max(T * k, 1), np.int32)
    R = lib().oracle_layout(ids.reshape(-1), T, k, expert_begin, L, counts, seg,
                            src2dst, reorder)
    if R < 0:
        raise MemoryError("oracle_layout failed")
    return counts, seg, src2dst, reorder[:R].copy()


def layout_aligned(topk_ids: np.ndarray, expert_begin: int, L: int, alignment: int):
    """Layout with segments padded to multiples of `alignment`; padding rows
    have reorder id -1.  Returns counts, seg_indptr, src2dst, reorder[R_pad]."""
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    counts = np.zeros(L, np.int32)
    seg = np.zeros(L + 1, np.int64)
    src2dst = np.zeros(T * k, np.int32)
    cap = T * k + L * max(alignment - 1, 0)
    reorder = np.zeros(max(cap, 1), np.int32)
    R = lib().oracle_layout_aligned(ids.reshape(-1), T, k, expert_begin, L, alignment,
                                    counts, seg, src2dst, reorder)
    if R < 0:
        raise ValueError("oracle_layout_aligned failed")
    return counts, seg, src2dst, reorder[:R].copy()


def rank_layout(topk_ids: np.ndarray, E: int, num_ranks: int, ranks_per_node: int = 1):
    """(num_tokens_per_rank [R], num_tokens_per_rdma_rank [R/rpn],
    num_tokens_per_expert [E], is_token_in_rank [T, R] bool)."""
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    R = num_ranks
    per_rank = np.zeros(R, np.int32)
    per_node = np.zeros(max(R // max(ranks_per_node, 1), 1), np.int32)
    per_expert = np.zeros(max(E, 1), np.int32)
    in_rank = np.zeros(max(T * R, 1), np.uint8)
    rc = lib().oracle_rank_layout(ids.reshape(-1), T, k, E, R, ranks_per_node, per_rank,
                                  per_node, per_expert, in_rank)
    if rc != 0:
        raise ValueError("bad rank-layout sizes")
    return (per_rank, per_node[:R // ranks_per_node], per_expert[:E],
            in_rank[:T * R].reshape(T, R).astype(bool))


def dispatch(x_bits: np.ndarray, src2dst: np.ndarray, k: int, rows: int,
             fill: int = 0) -> np.ndarray:
    """Normal-mode scatter of bf16 rows (uint16 patterns) into [rows, H]."""
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    P = np.full((rows, H), fill, np.uint16)
    lib().oracle_dispatch(x.reshape(-1), T, H, k, _c(src2dst, np.int32),
                          P.reshape(-1))
    return P


def dispatch_ll(x_bits: np.ndarray, topk_ids: np.ndarray, expert_begin: int,
                L: int, cap: int, fill: int = 0):
    """Low-latency scatter into [L, cap, H]. Returns (B, masked_m, ll_src2dst,
    overflow)."""
    x = _c(x_bits, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, H = x.shape
    k = ids.shape[1]
    B = np.full((L, cap, H), fill, np.uint16)
    masked_m = np.zeros(L, np.int32)
    ll = np.zeros(T * k, np.int32)
    ovf = lib().oracle_dispatch_ll(x.reshape(-1), T, H, k, ids.reshape(-1),
                                   expert_begin, L, cap, B.reshape(-1), masked_m,
                                   ll)
    if ovf < 0:
        raise MemoryError("oracle_dispatch_ll failed")
    return B, masked_m, ll, int(ovf)


def quant_group_fp8(x_bits: np.ndarray) -> Tuple[np.ndarray, float]:
    x = _c(x_bits, np.uint16).reshape(-1)
    q = np.zeros(x.size, np.uint8)
    s = ctypes.c_float(0.0)
    lib().oracle_quant_group_fp8(x, x.size, q, ctypes.byref(s))
    return q, s.value


def cast_fp8_tensor(x_bits: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Per-tensor fp8 cast: e4m3fn_rne(clamp(fl(x / scale), +-448)) of
    every bf16 value, same shape, uint8."""
    x = _c(x_bits, np.uint16)
    q = np.zeros(x.shape, np.uint8)
    lib().oracle_cast_fp8_tensor(x.reshape(-1), x.size, float(scale), q.reshape(-1))
    return q


def dispatch_fp8_tensor(x_bits: np.ndarray, src2dst: np.ndarray, k: int, rows: int,
                        scale: float = 1.0, fill: int = 0) -> np.ndarray:
    """Normal dispatch of per-tensor fp8 rows: Q [rows, H] u8 with
    Q[src2dst[i]] = cast_fp8_tensor(x[i // k], scale); other rows hold
    `fill`."""
    q = cast_fp8_tensor(x_bits, scale)
    T, H = q.shape
    Q = np.full((rows, H), fill, np.uint8)
    d = np.asarray(src2dst).reshape(-1)
    for i in np.nonzero(d >= 0)[0]:
        Q[d[i]] = q[i // k]
    return Q


def dispatch_fp8(x_bits: np.ndarray, src2dst: np.ndarray, k: int, rows: int,
                 group: int = 128):
    """fp8 normal dispatch: Q [rows, H] u8 and S [rows, H/group] f32."""
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    if H % group:
        raise ValueError("group must divide H")
    Q = np.zeros((rows, H), np.uint8)
    S = np.zeros((rows, H // group), np.float32)
    rc = lib().oracle_dispatch_fp8(x.reshape(-1), T, H, k, _c(src2dst, np.int32),
                                   group, Q.reshape(-1), S.reshape(-1))
    if rc != 0:
        raise RuntimeError("oracle_dispatch_fp8 failed: %d" % rc)
    return Q, S


SCALE_UE8M0, SCALE_COLMAJOR, SCALE_PACKED = 1, 2, 4


def scale_buffer_bytes(rows: int, G: int, flags: int, rows_per_mat: int) -> int:
    """Size in bytes of a scale buffer for `rows` destination rows."""
    words = (G + 3) // 4 if flags & SCALE_PACKED else G
    if flags & SCALE_COLMAJOR:
        nmat = -(-rows // rows_per_mat) if rows else 0
        ld = -(-rows_per_mat // 4) * 4
        return nmat * words * ld * 4
    return rows * words * 4


def quant_group_fp8_ue8m0(x_bits: np.ndarray):
    x = _c(x_bits, np.uint16).reshape(-1)
    q = np.zeros(x.size, np.uint8)
    p = ctypes.c_float(0.0)
    e = ctypes.c_int32(0)
    lib().oracle_quant_group_fp8_ue8m0(x, x.size, q, ctypes.byref(p), ctypes.byref(e))
    return q, p.value, e.value


def dispatch_fp8_fmt(x_bits: np.ndarray, src2dst: np.ndarray, k: int, rows: int, flags: int,
                     rows_per_mat: int = 0, group: int = 128, fill: int = 0):
    """fp8 dispatch with a scale format; returns (Q [rows, H] u8, S raw bytes
    of scale_buffer_bytes(...), filled with `fill` where not written)."""
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    rpm = rows_per_mat or max(rows, 1)
    Q = np.zeros((rows, H), np.uint8)
    S = np.full(max(scale_buffer_bytes(rows, H // group, flags, rpm), 1), fill, np.uint8)
    rc = lib().oracle_dispatch_fp8_fmt(x.reshape(-1), T, H, k, _c(src2dst, np.int32), group,
                                       flags, rpm, Q.reshape(-1), S)
    if rc != 0:
        raise ValueError("oracle_dispatch_fp8_fmt failed: %d" % rc)
    return Q, S


def dispatch_ll_fp8(x_bits: np.ndarray, topk_ids: np.ndarray, expert_begin: int, L: int,
                    cap: int, flags: int, group: int = 128, fill: int = 0):
    """Returns (Q [L, cap, H] u8, S bytes, masked_m, ll_src2dst, overflow)."""
    x = _c(x_bits, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, H = x.shape
    k = ids.shape[1]
    Q = np.zeros((L, cap, H), np.uint8)
    S = np.full(max(scale_buffer_bytes(L * cap, H // group, flags, cap), 1), fill, np.uint8)
    mm = np.zeros(L, np.int32)
    ll = np.zeros(T * k, np.int32)
    ovf = lib().oracle_dispatch_ll_fp8(x.reshape(-1), T, H, k, ids.reshape(-1), expert_begin, L,
                                       cap, group, flags, Q.reshape(-1), S, mm, ll)
    if ovf < 0:
        raise ValueError("oracle_dispatch_ll_fp8 failed")
    return Q, S, mm, ll, int(ovf)


def combine(y_bits: np.ndarray, map_: np.ndarray, weights: np.ndarray,
            T: int, k: int) -> np.ndarray:
    """Weighted gather-combine; returns bf16 patterns [T, H]."""
    y = _c(y_bits, np.uint16)
    H = y.shape[-1]
    y2 = y.reshape(-1, H) if y.size else np.zeros((0, H), np.uint16)
    out = np.zeros((T, H), np.uint16)
    bad = lib().oracle_combine(y2.reshape(-1), y2.shape[0], H, _c(map_, np.int32),
                               _c(weights, np.float32).reshape(-1), T, k,
                               out.reshape(-1))
    if bad < 0:
        raise MemoryError("oracle_combine failed")
    if bad:
        raise ValueError("map holds %d entries beyond y_rows" % bad)
    return out


def combine_f64(y_bits: np.ndarray, map_: np.ndarray, weights: np.ndarray,
                T: int, k: int) -> np.ndarray:
    y = _c(y_bits, np.uint16)
    H = y.shape[-1]
    y2 = y.reshape(-1, H) if y.size else np.zeros((0, H), np.uint16)
    out = np.zeros((T, H), np.float64)
    lib().oracle_combine_f64(y2.reshape(-1), y2.shape[0], H, _c(map_, np.int32),
                             _c(weights, np.float32).reshape(-1), T, k,
                             out.reshape(-1))
    return out


def expected_m(T: int, num_ranks: int, k: int, E: int) -> int:
    return int(lib().oracle_expected_m(T, num_ranks, k, E))


# ---------------------------------------------------------------------------
# all-core timing build (benchmark CPU baseline only; never used for parity)
# ---------------------------------------------------------------------------

_lib_omp = None


def lib_omp():
    """The OpenMP timing build of the dispatch and combine loops."""
    global _lib_omp
    if _lib_omp is None:
        if not os.path.exists(_LIB_OMP):
            build(force=True)
        L = ctypes.CDLL(_LIB_OMP)
        L.oracle_omp_dispatch.argtypes = [_u16p, _i64, _i64, _i32, _i32p, _u16p, _i32]
        L.oracle_omp_dispatch.restype = None
        L.oracle_omp_combine.argtypes = [_u16p, _i64, _i64, _i32p, _f32p, _i64, _i32, _u16p,
                                         _i32]
        L.oracle_omp_combine.restype = _i64
        _lib_omp = L
    return _lib_omp


def omp_dispatch(x_bits: np.ndarray, src2dst: np.ndarray, k: int, rows: int,
                 threads: int) -> np.ndarray:
    """dispatch() on `threads` host threads (timing build; same rows)."""
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    P = np.zeros((rows, H), np.uint16)
    lib_omp().oracle_omp_dispatch(x.reshape(-1), T, H, k, _c(src2dst, np.int32), P.reshape(-1),
                                  int(threads))
    return P


def omp_combine(y_bits: np.ndarray, map_: np.ndarray, weights: np.ndarray, T: int, k: int,
                threads: int) -> np.ndarray:
    """combine() on `threads` host threads (timing build; same bits)."""
    y = _c(y_bits, np.uint16)
    H = y.shape[-1]
    y2 = y.reshape(-1, H) if y.size else np.zeros((0, H), np.uint16)
    out = np.zeros((T, H), np.uint16)
    bad = lib_omp().oracle_omp_combine(y2.reshape(-1), y2.shape[0], H, _c(map_, np.int32),
                                       _c(weights, np.float32).reshape(-1), T, k,
                                       out.reshape(-1), int(threads))
    if bad < 0:
        raise MemoryError("oracle_omp_combine failed")
    if bad:
        raise ValueError("map holds %d entries beyond y_rows" % bad)
    return out
