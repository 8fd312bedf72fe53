"""The hot path captured in a HIP graph replays correctly.

The hot calls enqueue kernels only (no memsets, copies or host syncs), so
a serving loop can capture layout + dispatch + combine (or the one-call
layout-and-dispatch + combine) once and replay it.
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
