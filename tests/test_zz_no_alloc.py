"""ep_layout_dispatch_noalloc (layout scratch in the library's static device
buffer) against ep_layout_dispatch (the caller's workspace), through the C
ABI: every layout output, the status word, the received rows and their
source indices and weights, bit for bit.

The calls run back to back with shrinking batches, so that each later call
finds the scratch holding an earlier, larger call's tables: 16384 tokens in
two groups (count pass plus one kernel, two rounds of per-chunk sums),
12000 tokens of the same routing at expert alignment 2 (94 chunks: the
separate count, scan, assign and dispatch kernels), a 128-token decode batch
(one kernel) and the 128-token correctness batch with out-of-range ids (the
status reports them).
"""
import dataclasses

import numpy as np
import pytest
import torch

import ep_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import combine_ep_get_amd as ep
    ep.load()
    return ep


def _case(name, A=1, bad_ids=False, T=None):
    wl = ep_inputs.WORKLOADS[name]
    if T is not None:
        wl = dataclasses.replace(wl, name=f"{name}[:{T}]", T=T)
    inp = ep_inputs.make_inputs(wl)
    idx = inp.topk_idx.copy()
    if bad_ids:
        idx[::7, 0] = wl.E + 3
    counts = np.bincount(idx[(idx >= 0) & (idx < wl.E)], minlength=wl.E)
    per_rank = ((counts + A - 1) // A * A).reshape(wl.R, -1).sum(1)
    S = int(per_rank.max())
    return wl, inp, idx, S, A


def _run_both(ep, wl, inp, idx, S, A):
    dev = torch.device("cuda:0")
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, A, S)
    assert ep.ep_workspace_bytes(p) <= ep.EP_NOALLOC_SCRATCH_BYTES
    d_idx = torch.from_numpy(idx).to(dev)
    d_x = torch.from_numpy(inp.x.view(np.int16)).to(dev)
    d_w = torch.from_numpy(inp.topk_weights).to(dev)
    rows = wl.R * S
    outs = []
    for noalloc in (False, True):
        bufs = ep.alloc_layout(p, dev, cumulative=True)
        recv = torch.zeros((rows, wl.H), dtype=torch.int16, device=dev)
        src = torch.full((rows,), -7, dtype=torch.int32, device=dev)
        rw = torch.zeros(rows, dtype=torch.float32, device=dev)
        lay = bufs.args()[:-1]   # without the workspace
        if noalloc:
            status = torch.full((1,), 12345, dtype=torch.int32, device=dev)
            ep.ep_layout_dispatch_noalloc(p, d_idx, *lay, status, d_x, d_w, recv, src, rw)
            code = ep.ep_read_status(status)
        else:
            ep.ep_layout_dispatch(p, d_idx, *lay, bufs.workspace, None, d_x, d_w, recv, src, rw)
            code = ep.ep_read_status(bufs.workspace)
        torch.cuda.synchronize()
        outs.append((bufs, recv, src, rw, code))
    return outs


@pytest.mark.parametrize("order", ["shrinking"])
def test_noalloc_matches_workspace_call(ep, order):
    cases = [_case("large16k"), _case("large16k", A=2, T=12000), _case("decode128"),
             _case("tiny", bad_ids=True)]
    for wl, inp, idx, S, A in cases:
        print(f"[no-alloc] {wl.name} T={wl.T} A={A} S={S}", flush=True)
        (b0, r0, s0, w0, c0), (b1, r1, s1, w1, c1) = _run_both(ep, wl, inp, idx, S, A)
        assert c0 == c1, (wl.name, c0, c1)
        if wl.name == "tiny":
            assert c1 == ep.EP_ERR_BAD_EXPERT
        else:
            assert c1 == ep.EP_OK
        for name in ("expert_count", "expert_offset", "rank_row_count", "rank_token_count",
                     "group_token_count", "is_token_in_rank", "token_slot", "cumulative_expert_recv"):
            assert torch.equal(getattr(b0, name), getattr(b1, name)), (wl.name, name)
        assert torch.equal(r0, r1), (wl.name, "recv_x")
        assert torch.equal(s0, s1), (wl.name, "recv_src_token")
        assert torch.equal(w0.view(torch.int32), w1.view(torch.int32)), (wl.name, "recv_weight")
        del b0, b1, r0, r1
        torch.cuda.empty_cache()


def test_noalloc_refuses_oversized_problem(ep):
    p = ep.Problem.make(16384 * 16, 7168, 2048, 8, 1024, 1024, 1, 1)
    fake = 1 << 20   # never dereferenced: the size check comes first
    with pytest.raises(ep.EpError) as e:
        ep.ep_layout_dispatch_noalloc(p, *([fake] * 15))
    assert e.value.code == ep.EP_ERR_SCRATCH_LIMIT
