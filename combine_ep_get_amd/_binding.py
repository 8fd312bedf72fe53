"""ctypes binding of libepget (include/ep_get.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module turns
tensors into raw device pointers, fills the ``ep_problem`` struct, passes the
current HIP stream and raises on error codes.  Loading fails loudly if the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libepget.so")

EP_OK = 0
EP_ERR_INVALID_ARG = -1
EP_ERR_HIP = -2
EP_ERR_CAPACITY = -3
EP_ERR_BAD_EXPERT = -4
EP_ERR_SCRATCH_LIMIT = -5
EP_NOALLOC_SCRATCH_BYTES = 8 << 20

EP_MAX_RANKS = 1024
EP_MAX_EXPERTS = 2048
EP_MAX_EXPERTS_PER_RANK = 256
EP_MAX_TOPK = 32
EP_MAX_HIDDEN = 1 << 24

# Every function the C header declares, checked by the test-suite.
EXPORTS = ("ep_workspace_bytes", "ep_rank_stride_hint", "ep_get_layout", "ep_dispatch",
           "ep_layout_dispatch", "ep_combine", "ep_quantize_fp8", "ep_dispatch_fp8",
           "ep_layout_dispatch_fp8", "ep_get_group_layout", "ep_dispatch_hier", "ep_combine_hier",
           "ep_combine_topk_weights", "ep_read_status", "ep_error_string",
           "ep_layout_dispatch_noalloc")


class EpError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {error_string(code)} ({code})")


class Problem(ctypes.Structure):
    """``ep_problem``: T, H, E, K, R, G, A and the rank slice stride S."""
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_topk", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("expert_alignment", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("rank_stride_rows", ctypes.c_int64),
    ]

    @classmethod
    def make(cls, T, H, E, K, R, G=1, A=1, S=0):
        return cls(T, H, E, K, R, G, A, 0, S)

    @property
    def num_rows(self) -> int:
        return self.num_ranks * self.rank_stride_rows


_lib = None


def load():
    """Load libepget.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "or python -m combine_ep_get_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.ep_workspace_bytes.restype = sz
        lib.ep_workspace_bytes.argtypes = [P]
        lib.ep_rank_stride_hint.restype = ctypes.c_int64
        lib.ep_rank_stride_hint.argtypes = [P]
        lib.ep_get_layout.restype = ctypes.c_int
        lib.ep_get_layout.argtypes = [P] + [vp] * 10 + [sz, vp]
        lib.ep_dispatch.restype = ctypes.c_int
        lib.ep_dispatch.argtypes = [P] + [vp] * 6 + [vp]
        lib.ep_layout_dispatch.restype = ctypes.c_int
        lib.ep_layout_dispatch.argtypes = [P] + [vp] * 10 + [sz] + [vp] * 5 + [vp]
        lib.ep_layout_dispatch_noalloc.restype = ctypes.c_int
        lib.ep_layout_dispatch_noalloc.argtypes = [P] + [vp] * 10 + [vp] * 5 + [vp]
        lib.ep_combine.restype = ctypes.c_int
        lib.ep_combine.argtypes = [P] + [vp] * 4 + [vp]
        lib.ep_quantize_fp8.restype = ctypes.c_int
        lib.ep_quantize_fp8.argtypes = [P] + [vp] * 3 + [vp]
        lib.ep_dispatch_fp8.restype = ctypes.c_int
        lib.ep_dispatch_fp8.argtypes = [P] + [vp] * 6 + [ctypes.c_int64, ctypes.c_int64] + [vp] * 2 + [vp]
        i64 = ctypes.c_int64
        lib.ep_layout_dispatch_fp8.restype = ctypes.c_int
        lib.ep_layout_dispatch_fp8.argtypes = [P] + [vp] * 10 + [sz] + [vp] * 5 + [i64, i64] + [vp] * 2 + [vp]
        lib.ep_get_group_layout.restype = ctypes.c_int
        lib.ep_get_group_layout.argtypes = [P, vp, i64, vp, vp, vp]
        lib.ep_dispatch_hier.restype = ctypes.c_int
        lib.ep_dispatch_hier.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp]
        lib.ep_combine_hier.restype = ctypes.c_int
        lib.ep_combine_hier.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp]
        lib.ep_combine_topk_weights.restype = ctypes.c_int
        lib.ep_combine_topk_weights.argtypes = [P] + [vp] * 3 + [vp]
        lib.ep_read_status.restype = ctypes.c_int
        lib.ep_read_status.argtypes = [vp, vp]
        lib.ep_error_string.restype = ctypes.c_char_p
        lib.ep_error_string.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


# Element types the C calls read, by the C type of the argument.
def _dtypes():
    import torch
    return {
        "int32": (torch.int32,),
        "int64": (torch.int64,),
        "float": (torch.float32,),
        "uint8": (torch.uint8, torch.bool),
        "bf16": (torch.bfloat16, torch.int16, torch.uint16),
        "e4m3": (torch.float8_e4m3fn, torch.uint8, torch.int8),
        "bytes": None,
    }


def _arg(t, what: str, ctype: str, count: int):
    """Pointer for argument `what` of C element type `ctype`, which the call
    reads or writes over `count` elements.  None gives NULL; an int is taken
    as a raw device address, unchecked.  A tensor must be dense, of that
    element type, hold at least `count` elements (bytes for "bytes") and be
    on the GPU: the kernels would read past a short array, and a host
    address in a kernel is a GPU memory fault."""
    if t is None or isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError(f"{what}: libepget takes contiguous arrays; call .contiguous() first")
    allowed = _dtypes()[ctype]
    if allowed is not None and t.dtype not in allowed:
        raise ValueError(f"{what}: dtype {t.dtype}, expected one of {allowed}")
    have = t.numel() * t.element_size() if allowed is None else t.numel()
    if have < count:
        raise ValueError(f"{what}: {have} {'bytes' if allowed is None else 'elements'}, "
                         f"the call uses {count}")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: a {t.device.type} tensor; the library takes device memory")
    return t.data_ptr()


def _sizes(problem):
    """T, H, K, E, R, G and the receive rows R * S of a problem."""
    return (problem.num_tokens, problem.hidden, problem.num_topk, problem.num_experts,
            problem.num_ranks, problem.num_groups, problem.num_ranks * problem.rank_stride_rows)


def _layout_ptrs(problem, topk_idx, expert_count, expert_offset, rank_row_count, rank_token_count,
                 group_token_count, is_token_in_rank, token_slot, cumulative_expert_recv,
                 workspace, workspace_bytes):
    T, _, K, E, R, G, _ = _sizes(problem)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    return (_arg(topk_idx, "topk_idx", "int32", T * K), _arg(expert_count, "expert_count", "int32", E),
            _arg(expert_offset, "expert_offset", "int32", E),
            _arg(rank_row_count, "rank_row_count", "int32", R),
            _arg(rank_token_count, "rank_token_count", "int32", R),
            _arg(group_token_count, "group_token_count", "int32", G),
            _arg(is_token_in_rank, "is_token_in_rank", "uint8", T * R),
            _arg(token_slot, "token_slot", "int32", T * K),
            _arg(cumulative_expert_recv, "cumulative_expert_recv", "int64", E),
            _arg(workspace, "workspace", "bytes", workspace_bytes), workspace_bytes)


def _fp8_rows_ptrs(problem, x_fp8, x_sf, recv_x_fp8, recv_sf, sf_token_stride, sf_hidden_stride):
    T, H, _, _, _, _, rows = _sizes(problem)
    nsf = H // 128
    sf_span = (rows - 1) * sf_token_stride + (nsf - 1) * sf_hidden_stride + 1 if rows and nsf else 0
    return (_arg(x_fp8, "x_fp8", "e4m3", T * H), _arg(x_sf, "x_sf", "float", T * nsf),
            _arg(recv_x_fp8, "recv_x_fp8", "e4m3", rows * H), _arg(recv_sf, "recv_sf", "float", sf_span))


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def error_string(code: int) -> str:
    return load().ep_error_string(code).decode()


def _check(rc: int, where: str) -> int:
    if rc != EP_OK:
        raise EpError(rc, where)
    return rc


class BoundCall:
    """One entry point with its arguments marshalled once.  Calling it issues
    the same C call again (same pointers, sizes and stream), so a loop that
    repeats a step pays only for the call itself.  The tensors must stay
    alive and in place while it is used.  The problem is copied when the
    call is bound: the tensors were checked against its sizes then, so later
    changes to the caller's struct are not seen (bind again instead)."""

    def __init__(self, name: str, problem: Problem, args: tuple):
        self.name = name
        self._fn = getattr(load(), name)
        self.problem = Problem.from_buffer_copy(problem)
        self._args = (ctypes.byref(self.problem), *args)

    def __call__(self) -> int:
        return _check(self._fn(*self._args), self.name)


def _run(name: str, problem: Problem, args: tuple, bind: bool):
    """Calls the entry point on `problem` and args now, or with bind=True
    returns it as a BoundCall."""
    if bind:
        return BoundCall(name, problem, args)
    return _check(getattr(load(), name)(ctypes.byref(problem), *args), name)


def ep_workspace_bytes(problem: Problem) -> int:
    return load().ep_workspace_bytes(ctypes.byref(problem))


def ep_rank_stride_hint(problem: Problem) -> int:
    return load().ep_rank_stride_hint(ctypes.byref(problem))


def ep_get_layout(problem, topk_idx, expert_count, expert_offset, rank_row_count,
                  rank_token_count, group_token_count, is_token_in_rank, token_slot,
                  cumulative_expert_recv, workspace, workspace_bytes=None, stream=None, bind=False):
    lay = _layout_ptrs(problem, topk_idx, expert_count, expert_offset, rank_row_count,
                       rank_token_count, group_token_count, is_token_in_rank, token_slot,
                       cumulative_expert_recv, workspace, workspace_bytes)
    return _run("ep_get_layout", problem, (*lay, _stream(stream)), bind)


def _dispatch_ptrs(problem, x, topk_weights, recv_x, recv_src_token, recv_weight):
    T, H, K, _, _, _, rows = _sizes(problem)
    return (_arg(x, "x", "bf16", T * H), _arg(topk_weights, "topk_weights", "float", T * K),
            _arg(recv_x, "recv_x", "bf16", rows * H), _arg(recv_src_token, "recv_src_token", "int32", rows),
            _arg(recv_weight, "recv_weight", "float", rows))


def ep_dispatch(problem, x, topk_weights, token_slot, recv_x, recv_src_token=None,
                recv_weight=None, stream=None, bind=False):
    T, _, K, _, _, _, _ = _sizes(problem)
    px, pw, prx, psrc, prw = _dispatch_ptrs(problem, x, topk_weights, recv_x, recv_src_token, recv_weight)
    return _run("ep_dispatch", problem, (px, pw, _arg(token_slot, "token_slot", "int32", T * K),
        prx, psrc, prw, _stream(stream)), bind)


def ep_layout_dispatch(problem, topk_idx, expert_count, expert_offset, rank_row_count,
                       rank_token_count, group_token_count, is_token_in_rank, token_slot,
                       cumulative_expert_recv, workspace, workspace_bytes, x, topk_weights, recv_x,
                       recv_src_token=None, recv_weight=None, stream=None, bind=False):
    """ep_get_layout followed by ep_dispatch (one kernel for decode-sized batches)."""
    lay = _layout_ptrs(problem, topk_idx, expert_count, expert_offset, rank_row_count,
                       rank_token_count, group_token_count, is_token_in_rank, token_slot,
                       cumulative_expert_recv, workspace, workspace_bytes)
    rows = _dispatch_ptrs(problem, x, topk_weights, recv_x, recv_src_token, recv_weight)
    return _run("ep_layout_dispatch", problem, (*lay, *rows, _stream(stream)), bind)


def ep_layout_dispatch_noalloc(problem, topk_idx, expert_count, expert_offset, rank_row_count,
                               rank_token_count, group_token_count, is_token_in_rank, token_slot,
                               cumulative_expert_recv, status, x, topk_weights, recv_x,
                               recv_src_token=None, recv_weight=None, stream=None, bind=False):
    """ep_layout_dispatch with the layout scratch in the library's static
    device buffer (no workspace argument); the status word goes to `status`
    (one int32 on the device, read with ep_read_status)."""
    T, _, K, E, R, G, _ = _sizes(problem)
    lay = (_arg(topk_idx, "topk_idx", "int32", T * K), _arg(expert_count, "expert_count", "int32", E),
           _arg(expert_offset, "expert_offset", "int32", E),
           _arg(rank_row_count, "rank_row_count", "int32", R),
           _arg(rank_token_count, "rank_token_count", "int32", R),
           _arg(group_token_count, "group_token_count", "int32", G),
           _arg(is_token_in_rank, "is_token_in_rank", "uint8", T * R),
           _arg(token_slot, "token_slot", "int32", T * K),
           _arg(cumulative_expert_recv, "cumulative_expert_recv", "int64", E),
           _arg(status, "status", "int32", 1))
    rows = _dispatch_ptrs(problem, x, topk_weights, recv_x, recv_src_token, recv_weight)
    return _run("ep_layout_dispatch_noalloc", problem, (*lay, *rows, _stream(stream)), bind)


def ep_combine(problem, y, token_slot, topk_weights, out, stream=None, bind=False):
    T, H, K, _, _, _, rows = _sizes(problem)
    return _run("ep_combine", problem, (_arg(y, "y", "bf16", rows * H),
        _arg(token_slot, "token_slot", "int32", T * K),
        _arg(topk_weights, "topk_weights", "float", T * K),
        _arg(out, "out", "bf16", T * H), _stream(stream)), bind)


def ep_quantize_fp8(problem, x, x_fp8, x_sf, stream=None, bind=False):
    T, H, _, _, _, _, _ = _sizes(problem)
    return _run("ep_quantize_fp8", problem, (_arg(x, "x", "bf16", T * H),
        _arg(x_fp8, "x_fp8", "e4m3", T * H),
        _arg(x_sf, "x_sf", "float", T * (H // 128)), _stream(stream)), bind)


def ep_dispatch_fp8(problem, x_fp8, x_sf, topk_weights, token_slot, recv_x_fp8, recv_sf,
                    sf_token_stride, sf_hidden_stride, recv_src_token=None, recv_weight=None,
                    stream=None, bind=False):
    T, _, K, _, _, _, rows = _sizes(problem)
    px, psf, prx, prsf = _fp8_rows_ptrs(problem, x_fp8, x_sf, recv_x_fp8, recv_sf, sf_token_stride,
                                        sf_hidden_stride)
    return _run("ep_dispatch_fp8", problem, (px, psf,
        _arg(topk_weights, "topk_weights", "float", T * K),
        _arg(token_slot, "token_slot", "int32", T * K), prx, prsf,
        sf_token_stride, sf_hidden_stride,
        _arg(recv_src_token, "recv_src_token", "int32", rows),
        _arg(recv_weight, "recv_weight", "float", rows), _stream(stream)), bind)


def ep_layout_dispatch_fp8(problem, topk_idx, expert_count, expert_offset, rank_row_count,
                           rank_token_count, group_token_count, is_token_in_rank, token_slot,
                           cumulative_expert_recv, workspace, workspace_bytes, x_fp8, x_sf,
                           topk_weights, recv_x_fp8, recv_sf, sf_token_stride, sf_hidden_stride,
                           recv_src_token=None, recv_weight=None, stream=None, bind=False):
    """ep_get_layout followed by ep_dispatch_fp8 (one kernel for decode-sized batches)."""
    T, _, K, _, _, _, rows = _sizes(problem)
    lay = _layout_ptrs(problem, topk_idx, expert_count, expert_offset, rank_row_count,
                       rank_token_count, group_token_count, is_token_in_rank, token_slot,
                       cumulative_expert_recv, workspace, workspace_bytes)
    px, psf, prx, prsf = _fp8_rows_ptrs(problem, x_fp8, x_sf, recv_x_fp8, recv_sf, sf_token_stride,
                                        sf_hidden_stride)
    return _run("ep_layout_dispatch_fp8", problem, (*lay, px, psf,
        _arg(topk_weights, "topk_weights", "float", T * K), prx, prsf,
        sf_token_stride, sf_hidden_stride,
        _arg(recv_src_token, "recv_src_token", "int32", rows),
        _arg(recv_weight, "recv_weight", "float", rows),
        _stream(stream)), bind)


def ep_get_group_layout(problem, is_token_in_rank, group_stride_rows, group_slot, status=None,
                        stream=None, bind=False):
    """Group slots of the two-level path; `status` (one int32 on the device,
    e.g. the layout's workspace) is lowered to EP_ERR_CAPACITY when a group
    overflows SG rows."""
    T, _, _, _, R, G, _ = _sizes(problem)
    return _run("ep_get_group_layout", problem, (
        _arg(is_token_in_rank, "is_token_in_rank", "uint8", T * R),
        group_stride_rows, _arg(group_slot, "group_slot", "int32", T * G),
        _arg(status, "status", "bytes", 4), _stream(stream)), bind)


def ep_dispatch_hier(problem, x, topk_weights, token_slot, group_slot, group_stride_rows,
                     group_buf, recv_x, recv_src_token=None, recv_weight=None, stream=None, bind=False):
    T, H, K, _, _, G, _ = _sizes(problem)
    px, pw, prx, psrc, prw = _dispatch_ptrs(problem, x, topk_weights, recv_x, recv_src_token, recv_weight)
    return _run("ep_dispatch_hier", problem, (px, pw,
        _arg(token_slot, "token_slot", "int32", T * K),
        _arg(group_slot, "group_slot", "int32", T * G), group_stride_rows,
        _arg(group_buf, "group_buf", "bf16", G * group_stride_rows * H),
        prx, psrc, prw, _stream(stream)), bind)


def ep_combine_hier(problem, y, token_slot, topk_weights, group_slot, group_stride_rows,
                    group_buf, out, stream=None, bind=False):
    T, H, K, _, _, G, rows = _sizes(problem)
    return _run("ep_combine_hier", problem, (_arg(y, "y", "bf16", rows * H),
        _arg(token_slot, "token_slot", "int32", T * K),
        _arg(topk_weights, "topk_weights", "float", T * K),
        _arg(group_slot, "group_slot", "int32", T * G), group_stride_rows,
        _arg(group_buf, "group_buf", "bf16", G * group_stride_rows * H),
        _arg(out, "out", "bf16", T * H), _stream(stream)), bind)


def ep_combine_topk_weights(problem, recv_weight, token_slot, combined_topk_weights,
                            stream=None, bind=False):
    T, _, K, _, _, _, rows = _sizes(problem)
    return _run("ep_combine_topk_weights", problem, (
        _arg(recv_weight, "recv_weight", "float", rows),
        _arg(token_slot, "token_slot", "int32", T * K),
        _arg(combined_topk_weights, "combined_topk_weights", "float",
        T * K), _stream(stream)), bind)


def ep_read_status(workspace, stream=None) -> int:
    """Synchronises the stream and returns the layout's device status code."""
    return load().ep_read_status(_arg(workspace, "workspace", "bytes", 4), _stream(stream))
