"""CPU oracle for MoE token layout / dispatch / combine (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The HIP product path never
imports this package, and this package imports nothing from it.

The arithmetic lives in ``ep_oracle.c`` (plain C, single-threaded loops, fp64
for the combine sum); this module only builds/loads it and marshals numpy
arrays.  Each function states the passage of the pages it follows; the pages
are cited by title:

  [SYM] "DeepEP Symmetric Memory 全面架构分析"
  [V2]  "DeepEP V2 ElasticBuffer 架构深度分析"
  [V1]  "第 3 章 V1：Buffer 初始化与通信域建立"

Every function here is pinned by tests that do not reuse its code (brute
force on tiny inputs, numpy routines, invariants, the pages' closed form for
the expected number of ranks per token, torch's bf16 conversion, and exact
special cases of the combine); there are no unpinned functions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")

OK = 0
CAPACITY = -3
BAD_EXPERT = -4


def build(force: bool = True) -> str:
    """Compile ``ep_oracle.c`` with gcc into ``libep_oracle.so`` (in-tree)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def open_library(path: str):
    """Load an oracle build and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.oracle_layout.restype = ctypes.c_int
    lib.oracle_layout.argtypes = [i32, i32, i32, i32, i32, i32, i64] + [vp] * 8
    lib.oracle_dispatch.restype = None
    lib.oracle_dispatch.argtypes = [i32, i32, i32, i64] + [vp] * 6
    lib.oracle_combine.restype = None
    lib.oracle_combine.argtypes = [i32, i32, i32, i64] + [vp] * 4
    lib.oracle_float_to_e4m3.restype = None
    lib.oracle_float_to_e4m3.argtypes = [i64, vp, vp]
    lib.oracle_e4m3_to_float.restype = None
    lib.oracle_e4m3_to_float.argtypes = [i64, vp, vp]
    lib.oracle_quantize_fp8.restype = None
    lib.oracle_quantize_fp8.argtypes = [i32, i32, vp, vp, vp]
    lib.oracle_dispatch_fp8.restype = None
    lib.oracle_dispatch_fp8.argtypes = [i32, i32, i32, i64] + [vp] * 6 + [i64, i64, vp, vp]
    lib.oracle_group_layout.restype = ctypes.c_int
    lib.oracle_group_layout.argtypes = [i32, i32, i32, i64, vp, vp]
    lib.oracle_dispatch_hier.restype = None
    lib.oracle_dispatch_hier.argtypes = [i32, i32, i32, i32, i32, i64, i64] + [vp] * 8
    lib.oracle_combine_hier.restype = None
    lib.oracle_combine_hier.argtypes = [i32, i32, i32, i32, i32, i64, i64] + [vp] * 6
    lib.oracle_combine_topk_weights.restype = None
    lib.oracle_combine_topk_weights.argtypes = [i32, i32, i64, vp, vp, vp]
    lib.oracle_double_to_bf16.restype = None
    lib.oracle_double_to_bf16.argtypes = [i64, vp, vp]
    lib.oracle_bf16_to_double.restype = None
    lib.oracle_bf16_to_double.argtypes = [i64, vp, vp]
    return lib


_lib = None
_override = None  # set by use_library() to route calls to another build


def _load():
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = open_library(_LIB)
    return _lib


class use_library:
    """Context manager: route this module's calls to another oracle build.

    The tests use it to check that the pins reject builds with a planted
    mistake.
    """

    def __init__(self, lib):
        self.lib = lib

    def __enter__(self):
        global _override
        self._prev, _override = _override, self.lib
        return self.lib

    def __exit__(self, *exc):
        global _override
        _override = self._prev
        return False


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


@dataclass
class Layout:
    status: int
    expert_count: np.ndarray      # [E] int32
    expert_offset: np.ndarray     # [E] int32
    rank_row_count: np.ndarray    # [R] int32
    rank_token_count: np.ndarray  # [R] int32
    group_token_count: np.ndarray  # [G] int32
    is_token_in_rank: np.ndarray  # [T,R] uint8
    token_slot: np.ndarray        # [T,K] int32


def layout(topk_idx: np.ndarray, E: int, R: int, S: int, G: int = 1, A: int = 1) -> Layout:
    """Routing layout ([SYM] §6.1 and §7.3; [V1] §3.2 for groups).

    Counts per expert, rank and group, the token-to-rank map, the aligned
    within-slice expert offsets and the destination slot of every
    (token, top-k) entry in stable token order.
    """
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    assert E % R == 0 and R % G == 0 and A >= 1 and S >= 0
    out = Layout(
        status=0,
        expert_count=np.empty(E, np.int32),
        expert_offset=np.empty(E, np.int32),
        rank_row_count=np.empty(R, np.int32),
        rank_token_count=np.empty(R, np.int32),
        group_token_count=np.empty(G, np.int32),
        is_token_in_rank=np.empty((T, R), np.uint8),
        token_slot=np.empty((T, K), np.int32),
    )
    out.status = _load().oracle_layout(
        T, K, E, R, G, A, S, _p(idx), _p(out.expert_count), _p(out.expert_offset),
        _p(out.rank_row_count), _p(out.rank_token_count), _p(out.group_token_count),
        _p(out.is_token_in_rank), _p(out.token_slot))
    return out


def dispatch(x: np.ndarray, token_slot: np.ndarray, num_rows: int,
             topk_weights: np.ndarray | None = None, recv_x: np.ndarray | None = None,
             with_src: bool = True, with_weight: bool = True):
    """Dispatch scatter ([SYM] §6.1, §9.2; [V2] TokenLayout block).

    Returns ``(recv_x[num_rows,H] uint16, recv_src_token[num_rows] int32,
    recv_weight[num_rows] fp32)``.  Rows no slot references keep the
    contents of ``recv_x`` as given (zeros by default), -1 in the source map
    and NaN in the weight map; they are unspecified on the GPU and are never
    compared.
    """
    x = _c(x, np.uint16)
    slot = _c(token_slot, np.int32)
    T, H = x.shape
    K = slot.shape[1] if slot.ndim == 2 else 0
    assert slot.shape == (T, K)
    if recv_x is None:
        recv_x = np.zeros((num_rows, H), np.uint16)
    src = np.full(num_rows, -1, np.int32) if with_src else None
    rw = np.full(num_rows, np.nan, np.float32) if with_weight else None
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    _load().oracle_dispatch(T, H, K, num_rows, _p(x), _p(w), _p(slot), _p(recv_x),
                            _p(src), _p(rw))
    return recv_x, src, rw


def combine(y: np.ndarray, token_slot: np.ndarray, topk_weights: np.ndarray | None = None) -> np.ndarray:
    """Weighted top-k gather-reduce back to token order ([SYM] §9.2).

    ``out[t,h] = bf16_rne(sum_j w[t,j] * y[slot[t,j],h])``, summed in double
    over ascending j, skipping slots outside ``[0, rows(y))``.
    """
    y = _c(y, np.uint16)
    slot = _c(token_slot, np.int32)
    T, K = slot.shape
    H = y.shape[1]
    out = np.empty((T, H), np.uint16)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    _load().oracle_combine(T, H, K, y.shape[0], _p(y), _p(slot), _p(w), _p(out))
    return out


def group_layout(is_token_in_rank: np.ndarray, G: int, SG: int, with_status: bool = False):
    """Group slots of the hierarchical path: a stable compaction, per group,
    of the tokens with an entry in the group ([V2] hybrid dispatch; [V1]
    §3.2 groups of ranks).  ``[T,G]`` int32, -1 where absent or past SG.
    With ``with_status`` returns (slots, status): CAPACITY if some group
    has more than SG tokens, else OK."""
    m = _c(is_token_in_rank, np.uint8)
    T, R = m.shape
    out = np.empty((T, G), np.int32)
    status = _load().oracle_group_layout(T, R, G, SG, _p(m), _p(out))
    return (out, status) if with_status else out


def dispatch_hier(x, group_slot, token_slot, R, S, SG, recv_x=None, topk_weights=None,
                  with_meta=False):
    """Two-level dispatch: rows to the group buffer once per group, then
    from the group rows to every expert row.  Returns (group_buf, recv_x),
    and with ``with_meta`` also (recv_src_token, recv_weight) [R*S], where a
    row whose group row was dropped gets -1 and 0 (rows no slot names stay
    -1 and 0 as well)."""
    x = _c(x, np.uint16)
    gsl = _c(group_slot, np.int32)
    slot = _c(token_slot, np.int32)
    T, H = x.shape
    G = gsl.shape[1]
    K = slot.shape[1]
    gbuf = np.zeros((G * SG, H), np.uint16)
    if recv_x is None:
        recv_x = np.zeros((R * S, H), np.uint16)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    src = np.full(R * S, -1, np.int32)
    rw = np.zeros(R * S, np.float32)
    _load().oracle_dispatch_hier(T, H, K, R, G, S, SG, _p(x), _p(w), _p(gsl), _p(slot), _p(gbuf),
                                 _p(recv_x), _p(src), _p(rw))
    return (gbuf, recv_x, src, rw) if with_meta else (gbuf, recv_x)


def combine_hier(y, token_slot, topk_weights, group_slot, R, S, SG):
    """Two-level combine: per-(token, group) partials rounded to bf16, then
    their sum per token.  Returns (group_buf, out)."""
    y = _c(y, np.uint16)
    slot = _c(token_slot, np.int32)
    gsl = _c(group_slot, np.int32)
    T, K = slot.shape
    G = gsl.shape[1]
    H = y.shape[1]
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    gbuf = np.zeros((G * SG, H), np.uint16)
    out = np.empty((T, H), np.uint16)
    _load().oracle_combine_hier(T, H, K, R, G, S, SG, _p(y), _p(slot), _p(w), _p(gsl),
                                _p(gbuf), _p(out))
    return gbuf, out


def combine_topk_weights(recv_weight: np.ndarray, token_slot: np.ndarray) -> np.ndarray:
    """Per-row weights gathered back into token order ([SYM] §9.2,
    combined_topk_weights); 0 where the slot is outside ``[0, rows)``."""
    rw = _c(recv_weight, np.float32)
    slot = _c(token_slot, np.int32)
    T, K = slot.shape
    out = np.empty((T, K), np.float32)
    _load().oracle_combine_topk_weights(T, K, rw.shape[0], _p(rw), _p(slot), _p(out))
    return out


def float_to_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code (ties to even, saturating at 448) of fp32 values."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_float_to_e4m3(v.size, _p(v), _p(out))
    return out


def e4m3_to_float(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    out = np.empty(q.shape, np.float32)
    _load().oracle_e4m3_to_float(q.size, _p(q), _p(out))
    return out


def quantize_fp8(x: np.ndarray):
    """Per-token, per-128-channel e4m3 quantisation of bf16 rows: returns
    ``(codes [T,H] uint8, scales [T,H/128] fp32)`` with sf = amax/448 and
    codes = e4m3(x * (448/amax)) in fp32 (the reading of the FP8 dispatch
    arguments of [SYM] §6.1; the pages give no rule)."""
    x = _c(x, np.uint16)
    T, H = x.shape
    assert H % 128 == 0
    q = np.empty((T, H), np.uint8)
    sf = np.empty((T, H // 128), np.float32)
    _load().oracle_quantize_fp8(T, H, _p(x), _p(q), _p(sf))
    return q, sf


def dispatch_fp8(q: np.ndarray, sf: np.ndarray, token_slot: np.ndarray, num_rows: int,
                 topk_weights: np.ndarray | None = None, column_major_sf: bool = False,
                 sf_alignment: int = 4):
    """FP8 dispatch ([SYM] §6.1 sf arguments, [V2] TMA-aligned column-major
    scale layout).  Returns ``(recv_q [rows,H], recv_sf (flat), strides,
    recv_src_token, recv_weight)``; the scale of (row, block b) is
    ``recv_sf[row*strides[0] + b*strides[1]]``."""
    q = _c(q, np.uint8)
    sf = _c(sf, np.float32)
    slot = _c(token_slot, np.int32)
    T, H = q.shape
    K = slot.shape[1]
    nb = H // 128
    if column_major_sf:
        strides = (1, -(-num_rows // sf_alignment) * sf_alignment)
        size = strides[1] * nb
    else:
        strides = (nb, 1)
        size = num_rows * nb
    recv_q = np.zeros((num_rows, H), np.uint8)
    recv_sf = np.full(size, np.nan, np.float32)
    src = np.full(num_rows, -1, np.int32)
    rw = np.full(num_rows, np.nan, np.float32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    _load().oracle_dispatch_fp8(T, H, K, num_rows, _p(q), _p(sf), _p(w), _p(slot), _p(recv_q),
                                _p(recv_sf), strides[0], strides[1], _p(src), _p(rw))
    return recv_q, recv_sf, strides, src, rw


def double_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round doubles to bf16 bit patterns, nearest-even (used by combine)."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_double_to_bf16(v.size, _p(v), _p(out))
    return out


def bf16_to_double(b: np.ndarray) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    _load().oracle_bf16_to_double(b.size, _p(b), _p(out))
    return out


def default_rank_stride(T: int, K: int, E: int, R: int, A: int = 1) -> int:
    """Worst-case rows one source rank can put in one destination slice.

    Each token sends at most min(K, L) rows to a rank and alignment pads each
    of the L segments by at most A-1 rows, so T*min(K, L) + L*(A-1) rows never
    overflow; this mirrors sizing the symmetric buffer from
    num_max_tokens_per_rank ([SYM] §9.1, §9.5).
    """
    L = E // R
    return max(1, T * min(K, L) + L * (A - 1))
