"""The benchmark's own configuration against the CPU oracle: each workload
through the one-call layout and dispatch at the default (worst-case) slice
stride, then the combine reading the dispatched buffer, exactly as bench.py
runs a step.

The receive buffer at that stride is large (30 GB at 16384 tokens), so the
dispatched rows are compared on the device (the rows the slots name against
the rows of x they came from), and the combine against the oracle run on a
compact copy of the valid rows: slot s of the oracle's layout becomes row
rank(s) of the compact buffer, where rank(s) orders the valid slots."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-3, 1e-2


@pytest.fixture(scope="module")
def ep():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import combine_ep_get_amd as ep
    ep.load()
    return ep


@pytest.mark.parametrize("name", ["tiny", "decode128", "prefill4k", "zipf8k", "large16k"])
def test_one_call_step_at_default_stride(ep, name):
    print(f"[parity-bench-config] {name}", flush=True)
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    dev = torch.device("cuda:0")
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, wl.A, 1)
    S = ep.ep_rank_stride_hint(p)
    p.rank_stride_rows = S
    assert S == oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R, wl.A)
    rows = wl.R * S

    d_idx = torch.from_numpy(inp.topk_idx).to(dev)
    d_w = torch.from_numpy(inp.topk_weights).to(dev)
    d_x = torch.from_numpy(inp.x.view(np.int16)).to(dev)
    bufs = ep.alloc_layout(p, dev)
    recv = torch.empty((rows, wl.H), dtype=torch.int16, device=dev)
    recv_src = torch.empty(rows, dtype=torch.int32, device=dev)
    recv_w = torch.empty(rows, dtype=torch.float32, device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.int16, device=dev)
    ep.ep_layout_dispatch(p, d_idx, *bufs.args(), None, d_x, d_w, recv, recv_src, recv_w)
    ep.ep_combine(p, recv, bufs.token_slot, d_w, out)
    assert ep.ep_read_status(bufs.workspace) == ep.EP_OK
    torch.cuda.synchronize()

    ref = oracle.layout(inp.topk_idx, wl.E, wl.R, S, wl.G, wl.A)
    assert ref.status == oracle.OK
    for f in ("expert_count", "expert_offset", "rank_row_count", "rank_token_count", "group_token_count",
              "is_token_in_rank", "token_slot"):
        assert np.array_equal(getattr(bufs, f).cpu().numpy(), getattr(ref, f)), f

    # rows, source indices and weights at every valid slot, on the device
    slot = ref.token_slot.ravel()
    valid = slot >= 0
    t_of = np.repeat(np.arange(wl.T), wl.K)[valid]
    d_slots = torch.from_numpy(slot[valid].astype(np.int64)).to(dev)
    d_t = torch.from_numpy(t_of.astype(np.int64)).to(dev)
    assert torch.equal(recv.index_select(0, d_slots), d_x.index_select(0, d_t))
    assert torch.equal(recv_src.index_select(0, d_slots), d_t.to(torch.int32))
    w_valid = torch.from_numpy(inp.topk_weights.ravel()[valid]).to(dev)
    assert torch.equal(recv_w.index_select(0, d_slots).view(torch.int32), w_valid.view(torch.int32))

    # combine: the oracle over a compact copy of the valid rows
    order = np.sort(slot[valid])
    compact = np.full(slot.shape, -1, np.int64)
    compact[valid] = np.searchsorted(order, slot[valid])
    compact = compact.reshape(wl.T, wl.K).astype(np.int32)
    y_compact, _, _ = oracle.dispatch(inp.x, compact, len(order))
    want = oracle.bf16_to_double(oracle.combine(y_compact, compact, inp.topk_weights))
    got = oracle.bf16_to_double(out.cpu().numpy().view(np.uint16))
    bad = ~(np.abs(got - want) <= ATOL + RTOL * np.abs(want))
    assert not bad.any(), f"{bad.sum()} combine elements out of tolerance, first at {np.argwhere(bad)[:3]}"
