"""The hot path captured in a HIP graph replays correctly.

The hot calls enqueue kernels only (no memsets, copies or host syncs), so
a serving loop can capture layout + dispatch + combine (or the one-call
layout-and-dispatch + combine), the FP8 quantise + dispatch, or the
two-level path once and replay it.
Each replay is checked against the eager result, with the program's own
eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,fused", [("decode128", False), ("prefill4k", False), ("decode128", True),
                                        ("prefill4k", True)])
def test_graph_replay_matches_eager(name, fused):
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import combine_ep_get_amd as ep
    ep.load()
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, wl.A, 1)
    S = ep.ep_rank_stride_hint(p)
    p.rank_stride_rows = S
    rows = wl.R * S
    dev = torch.device("cuda:0")
    d_idx = torch.from_numpy(inp.topk_idx).to(dev)
    d_w = torch.from_numpy(inp.topk_weights).to(dev)
    d_x = torch.from_numpy(inp.x.view(np.int16)).to(dev)
    bufs = ep.alloc_layout(p, dev, cumulative=True)
    recv = torch.zeros((rows, wl.H), dtype=torch.int16, device=dev)
    out = torch.empty_like(d_x)

    def step():
        if fused:
            ep.ep_layout_dispatch(p, d_idx, *bufs.args(), None, d_x, d_w, recv, None, None)
        else:
            ep.ep_get_layout(p, d_idx, *bufs.args())
            ep.ep_dispatch(p, d_x, d_w, bufs.token_slot, recv, None, None)
        ep.ep_combine(p, recv, bufs.token_slot, d_w, out)

    # eager reference (also warms up)
    step()
    torch.cuda.synchronize()
    ref_slot = bufs.token_slot.clone()
    ref_out = out.clone()
    ref_counts = bufs.expert_count.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, wl.G, wl.A)
    np.testing.assert_array_equal(ref_slot.cpu().numpy(), lay.token_slot)
    cum0 = bufs.cumulative_expert_recv.clone()
    for i in range(4):
        # eager work between replays: scribble over the outputs
        bufs.token_slot.fill_(-7)
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs.token_slot, ref_slot), f"replay {i}"
        assert torch.equal(out, ref_out), f"replay {i}"
        assert torch.equal(bufs.expert_count, ref_counts), f"replay {i}"
        # each replay adds this layout's counts once more
        want = cum0 + (i + 1) * ref_counts.to(torch.int64)
        assert torch.equal(bufs.cumulative_expert_recv, want), f"replay {i}"
    assert ep.ep_read_status(bufs.workspace) == ep.EP_OK


def _capture(step):
    """Warm up on a side stream, then capture step() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["decode128", "prefill4k"])
def test_graph_replay_fp8_and_two_level(name):
    """Quantise + one-call FP8 layout-and-dispatch, and the two-level path
    (layout, group slots, group dispatch and expand, partial and group
    combine), each captured once and replayed against its eager result."""
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import combine_ep_get_amd as ep
    ep.load()
    print(f"[graph] fp8 and two-level {name}", flush=True)
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    G = 2
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, G, wl.A, 1)
    S = ep.ep_rank_stride_hint(p)
    p.rank_stride_rows = S
    rows = wl.R * S
    dev = torch.device("cuda:0")
    d_idx = torch.from_numpy(inp.topk_idx).to(dev)
    d_w = torch.from_numpy(inp.topk_weights).to(dev)
    d_x = torch.from_numpy(inp.x.view(np.int16)).to(dev)
    bufs = ep.alloc_layout(p, dev)
    nsf = wl.H // 128
    d_q = torch.empty((wl.T, wl.H), dtype=torch.uint8, device=dev)
    d_sf = torch.empty((wl.T, nsf), dtype=torch.float32, device=dev)
    recv_q = torch.zeros((rows, wl.H), dtype=torch.uint8, device=dev)
    recv_sf = torch.zeros(rows * nsf, dtype=torch.float32, device=dev)
    SG = wl.T
    gslot = torch.empty((wl.T, G), dtype=torch.int32, device=dev)
    gbuf = torch.zeros((G * SG, wl.H), dtype=torch.int16, device=dev)
    recv = torch.zeros((rows, wl.H), dtype=torch.int16, device=dev)
    out = torch.empty_like(d_x)

    def fp8_step():
        ep.ep_quantize_fp8(p, d_x, d_q, d_sf)
        ep.ep_layout_dispatch_fp8(p, d_idx, *bufs.args(), None, d_q, d_sf, d_w, recv_q, recv_sf, nsf, 1,
                                  None, None)

    def hier_step():
        ep.ep_get_layout(p, d_idx, *bufs.args())
        ep.ep_get_group_layout(p, bufs.is_token_in_rank, SG, gslot)
        ep.ep_dispatch_hier(p, d_x, d_w, bufs.token_slot, gslot, SG, gbuf, recv)
        ep.ep_combine_hier(p, recv, bufs.token_slot, d_w, gslot, SG, gbuf, out)

    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, G, wl.A)
    valid = lay.token_slot[lay.token_slot >= 0]
    sf_rows = (valid[:, None] * nsf + np.arange(nsf)[None, :]).ravel()

    fp8_step()
    torch.cuda.synchronize()
    ref_q = recv_q.cpu().numpy()[valid]
    ref_sf = recv_sf.cpu().numpy()[sf_rows]
    g = _capture(fp8_step)
    for i in range(3):
        recv_q.zero_()
        recv_sf.zero_()
        d_q.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(recv_q.cpu().numpy()[valid], ref_q, err_msg=f"fp8 replay {i}")
        np.testing.assert_array_equal(recv_sf.cpu().numpy()[sf_rows], ref_sf, err_msg=f"fp8 replay {i}")
    del g

    hier_step()
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref_gslot = gslot.clone()
    ref_recv = recv.cpu().numpy()[valid]
    np.testing.assert_array_equal(ref_gslot.cpu().numpy(), oracle.group_layout(lay.is_token_in_rank, G, SG))
    g = _capture(hier_step)
    for i in range(3):
        out.fill_(0)
        gslot.fill_(-7)
        recv.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gslot, ref_gslot), f"two-level replay {i}"
        assert torch.equal(out, ref_out), f"two-level replay {i}"
        np.testing.assert_array_equal(recv.cpu().numpy()[valid], ref_recv, err_msg=f"two-level replay {i}")
    assert ep.ep_read_status(bufs.workspace) == ep.EP_OK
