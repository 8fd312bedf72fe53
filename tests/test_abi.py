"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the header declares, and rejects invalid problems before it
enqueues anything."""
import ctypes
import os
import re

import pytest

import combine_ep_get_amd as ep

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "ep_get.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", text))


def test_header_and_binding_agree():
    assert declared_functions() == set(ep.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ep.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_error_strings():
    assert ep.error_string(ep.EP_OK) == "ok"
    assert "capacity" in ep.error_string(ep.EP_ERR_CAPACITY)
    assert "expert" in ep.error_string(ep.EP_ERR_BAD_EXPERT)


def P(**kw):
    base = dict(T=4096, H=7168, E=256, K=8, R=8, G=1, A=1, S=32768)
    base.update(kw)
    return ep.Problem.make(**base)


def test_stride_hint_and_workspace():
    assert ep.ep_rank_stride_hint(P()) == 4096 * 8
    assert ep.ep_rank_stride_hint(P(E=16, R=4, K=4, T=128)) == 128 * 4
    assert ep.ep_rank_stride_hint(P(E=64, R=16, K=8, T=100)) == 100 * 4   # min(K, L) = 4
    assert ep.ep_rank_stride_hint(P(A=8)) == 4096 * 8 + 32 * 7
    assert ep.ep_workspace_bytes(P()) > 0
    assert ep.ep_workspace_bytes(P(T=0)) > 0
    # the largest batch: T*K + E*A = INT32_MAX - 65536 at most
    assert ep.ep_workspace_bytes(P(T=(2**31 - 1 - 2**16 - 256) // 8, S=1)) > 0
    assert ep.ep_workspace_bytes(P(T=(2**31 - 1 - 2**16 - 256) // 8 + 1, S=1)) == 0


@pytest.mark.parametrize("bad", [
    dict(E=255), dict(E=4096, R=8), dict(R=2048, E=2048), dict(E=1024, R=2),   # limits
    dict(K=0), dict(K=33), dict(H=7), dict(H=0), dict(H=(1 << 24) + 8), dict(T=-1), dict(G=3), dict(G=0),
    dict(A=0), dict(S=0), dict(S=2**31 // 8 + 1),
    dict(T=(2**31 - 1 - 2**16 - 256) // 8 + 1, S=1),      # T*K + E*A one tile short of int32
    # one chunk of 128 tokens past a 2^30-entry count table (pitch 4160)
    dict(T=258111 * 128 + 1, E=2048, R=1024, G=1024, S=1),
])
def test_invalid_problems_rejected_before_launch(bad):
    p = P(**bad)
    lib = ep.load()
    fake = 1 << 20   # never dereferenced: validation fails first
    rc = lib.ep_get_layout(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake,
                           fake, fake, 1 << 30, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_combine(ctypes.byref(p), fake, fake, fake, fake, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_combine_topk_weights(ctypes.byref(p), fake, fake, fake, None) == ep.EP_ERR_INVALID_ARG


def test_count_table_limit():
    """The largest chunk table the layout addresses with 32-bit offsets:
    258111 chunks of 128 tokens x 4160 columns is under 2^30 entries, one
    more chunk is not."""
    big = dict(E=2048, R=1024, G=1024, S=1)
    assert ep.ep_workspace_bytes(P(T=258111 * 128, **big)) > 0
    assert ep.ep_workspace_bytes(P(T=258111 * 128 + 1, **big)) == 0
    # one token per layout chunk at K = 32; the table grows with T
    assert ep.ep_workspace_bytes(P(T=258111 * 32, K=32, **big)) > 0
    assert ep.ep_workspace_bytes(P(T=258111 * 32 + 1, K=32, **big)) == 0


def test_noalloc_scratch_limit_refused_on_host():
    """ep_layout_dispatch_noalloc refuses a problem whose layout workspace
    exceeds the static scratch before any device call (so this runs without
    a GPU): large16k fits, a batch sixteen times larger at E = 2048 does not."""
    lib = ep.load()
    fake = 1 << 20   # never dereferenced
    ok = P(T=16384, R=16, G=2)
    assert ep.ep_workspace_bytes(ok) <= ep.EP_NOALLOC_SCRATCH_BYTES
    big = P(T=16384 * 16, E=2048, R=1024, G=1024, S=1)
    assert ep.ep_workspace_bytes(big) > ep.EP_NOALLOC_SCRATCH_BYTES
    rc = lib.ep_layout_dispatch_noalloc(ctypes.byref(big), *([fake] * 15), None)
    assert rc == ep.EP_ERR_SCRATCH_LIMIT
    assert "scratch" in ep.error_string(rc)
    # invalid problems are still invalid arguments
    rc = lib.ep_layout_dispatch_noalloc(ctypes.byref(P(K=0)), *([fake] * 15), None)
    assert rc == ep.EP_ERR_INVALID_ARG


def test_reserved_field_must_be_zero():
    p = P()
    p.reserved = 1
    assert ep.ep_workspace_bytes(p) == 0


def test_bad_pointers_rejected():
    p = P()
    lib = ep.load()
    a = 1 << 20
    # misaligned x
    assert lib.ep_dispatch(ctypes.byref(p), a + 2, a, a, a, a, a, None) == ep.EP_ERR_INVALID_ARG
    # NULL output
    assert lib.ep_combine(ctypes.byref(p), a, a, a, None, None) == ep.EP_ERR_INVALID_ARG
    # workspace too small or misaligned
    need = ep.ep_workspace_bytes(p)
    args = [a] * 8
    assert lib.ep_get_layout(ctypes.byref(p), *args, None, a, need - 1, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_get_layout(ctypes.byref(p), *args, None, a + 16, need, None) == ep.EP_ERR_INVALID_ARG
    # cumulative counter must be 8-byte aligned
    assert lib.ep_get_layout(ctypes.byref(p), *args, a + 4, a, need, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_read_status(None, None) == ep.EP_ERR_INVALID_ARG


def test_fp8_argument_checks():
    lib = ep.load()
    a = 1 << 20
    p = P(H=7168 + 8)   # not a multiple of 128
    assert lib.ep_quantize_fp8(ctypes.byref(p), a, a, a, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch_fp8(ctypes.byref(p), a, a, a, a, a, a, 56, 1, a, a, None) == ep.EP_ERR_INVALID_ARG
    p = P()
    # non-positive scale strides
    assert lib.ep_dispatch_fp8(ctypes.byref(p), a, a, a, a, a, a, 0, 1, a, a, None) == ep.EP_ERR_INVALID_ARG
    # misaligned fp8 rows
    assert lib.ep_dispatch_fp8(ctypes.byref(p), a + 8, a, a, a, a, a, 56, 1, a, a, None) == ep.EP_ERR_INVALID_ARG


def test_layout_dispatch_argument_checks():
    """The fused call checks the arguments of both calls it stands for."""
    p = P()
    lib = ep.load()
    a = 1 << 20
    need = ep.ep_workspace_bytes(p)
    lay = [a] * 8
    # small workspace (a layout argument)
    assert lib.ep_layout_dispatch(ctypes.byref(p), *lay, None, a, need - 1,
                                  a, a, a, a, a, None) == ep.EP_ERR_INVALID_ARG
    # misaligned x and NULL recv_x (dispatch arguments)
    assert lib.ep_layout_dispatch(ctypes.byref(p), *lay, None, a, need,
                                  a + 2, a, a, a, a, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_layout_dispatch(ctypes.byref(p), *lay, None, a, need,
                                  a, a, None, a, a, None) == ep.EP_ERR_INVALID_ARG


def test_binding_refuses_strided_views():
    """A transposed or sliced view would be read as if it were dense."""
    import torch
    p = P()
    view = torch.zeros((8, 16), dtype=torch.int16).t()
    with pytest.raises(ValueError, match="contiguous"):
        ep.ep_combine(p, view, 1 << 20, None, 1 << 20, stream=0)


def test_binding_checks_types_sizes_and_device():
    """The binding refuses, before any call, arrays of the wrong element type,
    arrays shorter than the problem needs and host tensors (a kernel would
    read past the first and fault on the others)."""
    import torch
    T, H, K, E, R = 4, 64, 2, 8, 2
    p = ep.Problem.make(T, H, E, K, R, 1, 1, 8)
    rows = R * 8
    a = 1 << 20
    slot = torch.zeros((T, K), dtype=torch.int32)
    with pytest.raises(ValueError, match="token_slot: dtype"):
        ep.ep_combine(p, a, slot.long(), None, a, stream=0)
    with pytest.raises(ValueError, match="topk_weights: dtype"):
        ep.ep_combine(p, a, a, torch.zeros((T, K), dtype=torch.float64), a, stream=0)
    with pytest.raises(ValueError, match="y: 1023 elements, the call uses 1024"):
        ep.ep_combine(p, torch.zeros(rows * H - 1, dtype=torch.int16), a, None, a, stream=0)
    with pytest.raises(ValueError, match="out: dtype"):
        ep.ep_combine(p, a, a, None, torch.zeros((T, H), dtype=torch.float32), stream=0)
    with pytest.raises(ValueError, match="token_slot: a cpu tensor"):
        ep.ep_combine(p, a, slot, None, a, stream=0)
    with pytest.raises(ValueError, match="recv_src_token: 15 elements"):
        ep.ep_dispatch(p, a, None, a, a, torch.zeros(rows - 1, dtype=torch.int32), stream=0)
    with pytest.raises(ValueError, match="workspace: 100 bytes, the call uses 4096"):
        ep.ep_get_layout(p, a, a, a, a, a, None, a, a, None, torch.zeros(100, dtype=torch.uint8), 4096,
                         stream=0)
    with pytest.raises(ValueError, match="recv_sf: 10 elements"):
        ep.ep_dispatch_fp8(ep.Problem.make(T, 128, E, K, R, 1, 1, 8), a, a, None, a, a,
                           torch.zeros(10, dtype=torch.float32), 1, 1, stream=0)


def test_layout_dispatch_fp8_argument_checks():
    lib = ep.load()
    a = 1 << 20
    need = ep.ep_workspace_bytes(P())
    lay = [a] * 8
    p = P(H=7168 + 8)   # not a multiple of 128
    assert lib.ep_layout_dispatch_fp8(ctypes.byref(p), *lay, None, a, need, a, a, a, a, a, 56, 1,
                                      a, a, None) == ep.EP_ERR_INVALID_ARG
    p = P()
    assert lib.ep_layout_dispatch_fp8(ctypes.byref(p), *lay, None, a, need, a, a, a, a, a, 0, 1,
                                      a, a, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_layout_dispatch_fp8(ctypes.byref(p), *lay, None, a, need, a + 8, a, a, a, a, 56, 1,
                                      a, a, None) == ep.EP_ERR_INVALID_ARG
