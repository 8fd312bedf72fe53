"""Two-level (hierarchical) path: HIP vs the CPU oracle.

Group slots, group rows and received rows bit for bit; the per-(token,
group) partial rows bit for bit (both sides fold in fp32 with FMA and round
to bf16); the final combine within the usual tolerance."""
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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()

def assert_same(got, want, what=""):
    """Bitwise equality; the fast check first, numpy's report on failure."""
    got, want = np.asarray(got), np.asarray(want)
    if got.shape != want.shape or not np.array_equal(got, want):
        np.testing.assert_array_equal(got, want, err_msg=what)



def u16(t):
    return t.cpu().numpy().view(np.uint16)


def run(ep, idx, w, x, E, R, G, S, SG, y=None):
    T, K = idx.shape
    H = x.shape[1]
    p = ep.Problem.make(T, H, E, K, R, G, 1, S)
    bufs = ep.alloc_layout(p)
    ep.ep_get_layout(p, dev(idx), *bufs.args())
    ref = oracle.layout(idx, E, R, S, G)
    gslot = torch.empty((T, G), dtype=torch.int32, device="cuda")
    # the group overflow status goes to the layout's status word
    ep.ep_get_group_layout(p, bufs.is_token_in_rank, SG, gslot, bufs.workspace)
    status = ep.ep_read_status(bufs.workspace)
    ref_gs, ref_gstatus = oracle.group_layout(ref.is_token_in_rank, G, SG, with_status=True)
    assert_same(bufs.token_slot.cpu().numpy(), ref.token_slot)
    assert_same(gslot.cpu().numpy(), ref_gs)
    assert status == min(ref.status, ref_gstatus), (status, ref.status, ref_gstatus)
    # dispatch
    gbuf = torch.zeros((G * SG, H), dtype=torch.int16, device="cuda")
    recv = torch.zeros((R * S, H), dtype=torch.int16, device="cuda")
    src = torch.full((R * S,), -1, dtype=torch.int32, device="cuda")
    rw = torch.zeros(R * S, dtype=torch.float32, device="cuda")
    d_w = dev(w)
    ep.ep_dispatch_hier(p, dev(x.view(np.int16)), d_w, bufs.token_slot, gslot, SG, gbuf, recv, src, rw)
    torch.cuda.synchronize()
    ref_gbuf, ref_rx, ref_src, ref_rw = oracle.dispatch_hier(x, ref_gs, ref.token_slot, R, S, SG,
                                                             topk_weights=w, with_meta=True)
    valid_g = ref_gs[ref_gs >= 0]
    assert_same(u16(gbuf)[valid_g], ref_gbuf[valid_g])
    s = ref.token_slot[ref.token_slot >= 0]
    # rows of entries whose group row was dropped are not written
    kept = s[ref_src[s] >= 0]
    assert_same(u16(recv)[kept], ref_rx[kept])
    assert_same(src.cpu().numpy()[s], ref_src[s])
    assert_same(rw.cpu().numpy()[s].view(np.int32), ref_rw[s].view(np.int32))
    if ref_gstatus == oracle.OK:
        t_of = np.repeat(np.arange(T), K).reshape(T, K)[ref.token_slot >= 0]
        assert_same(ref_src[s], t_of)
    # combine
    if y is None:
        y = ep_inputs.permuted_rows(ref_rx, seed=13)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    gbuf.zero_()
    ep.ep_combine_hier(p, dev(y.view(np.int16)), bufs.token_slot, d_w, gslot, SG, gbuf, out)
    torch.cuda.synchronize()
    ref_pbuf, ref_out = oracle.combine_hier(y, ref.token_slot, w, ref_gs, R, S, SG)
    assert_same(u16(gbuf)[valid_g], ref_pbuf[valid_g])
    g_ = oracle.bf16_to_double(u16(out))
    r_ = oracle.bf16_to_double(ref_out)
    assert np.all(np.abs(g_ - r_) <= ATOL + RTOL * np.abs(r_))


@pytest.mark.parametrize("name,G", [("large16k", 2), ("prefill4k", 4), ("zipf8k", 8), ("tiny", 2), ("decode128", 2)])
def test_hier_workloads(ep, name, G):
    print(f"[parity-hier] {name} G={G}", flush=True)
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    counts = np.bincount(inp.topk_idx.ravel(), minlength=wl.E)
    S = int(counts.reshape(wl.R, -1).sum(1).max())
    y = ep_inputs.expert_outputs(wl.R * S, wl.H, seed=8) if wl.T * wl.H < 2e6 else None
    run(ep, inp.topk_idx, inp.topk_weights, inp.x, wl.E, wl.R, G, S, wl.T, y=y)


def test_hier_small_group_capacity_and_empty_entries(ep):
    rng = np.random.default_rng(17)
    T, K, E, R, G, H = 2500, 6, 96, 12, 3, 136
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    w = rng.standard_normal((T, K)).astype(np.float32)
    x = ep_inputs.bf16_normal(rng, (T, H))
    counts = np.bincount(idx[idx >= 0], minlength=E)
    S = int(counts.reshape(R, -1).sum(1).max())
    ref = oracle.layout(idx, E, R, S, G)
    SG = int(ref.group_token_count.min()) - 10   # the later tokens of each group are dropped
    run(ep, idx, w, x, E, R, G, S, SG)
    # a bad id on top: the layout's bad-id status is kept, not replaced by the
    # group overflow
    idx[5, 2] = E + 1
    run(ep, idx, w, x, E, R, G, S, SG)


@pytest.mark.parametrize("K,G", [(1, 2), (3, 4), (4, 2), (8, 8), (9, 2), (12, 4)])
def test_hier_topk_widths(ep, K, G):
    """Partial combine with the K rows gathered once (K <= 8: one or two
    groups' folds from registers) and, past 8, gathered group by group."""
    print(f"[parity-hier] K={K} G={G}", flush=True)
    rng = np.random.default_rng(100 + K * G)
    T, E, R, H = 700, 64, 8, 264
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = -1
    w = rng.standard_normal((T, K)).astype(np.float32)
    x = ep_inputs.bf16_normal(rng, (T, H))
    counts = np.bincount(idx[idx >= 0], minlength=E)
    S = int(counts.reshape(R, -1).sum(1).max())
    run(ep, idx, w, x, E, R, G, S, T)


@pytest.mark.parametrize("E,R,G,K", [
    (256, 16, 16, 8),    # the fewest groups that take the ballot walk
    (256, 32, 16, 12),   # and top-k past 8 (the partial combine gathers per group)
    (256, 128, 64, 8),   # one wave's worth of groups
    (260, 130, 65, 8),   # one group past it: a second ballot round with one lane
    (1920, 192, 96, 8),  # two ranks per group
    (2048, 1024, 128, 8),  # eight ranks per group, the largest R
    (1024, 1024, 1024, 8),  # one rank per group
])
def test_hier_many_groups(ep, E, R, G, K):
    """More than eight groups: every two-level stage finds the token's group
    rows with a ballot over 64 groups at a time (past 64, in several rounds)."""
    print(f"[parity-hier] E={E} R={R} G={G} K={K}", flush=True)
    rng = np.random.default_rng(E + R + G + K)
    T, H = 300, 64
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    x = ep_inputs.bf16_normal(rng, (T, H))
    counts = np.bincount(idx.ravel(), minlength=E)
    S = max(1, int(counts.reshape(R, -1).sum(1).max()))
    run(ep, idx, w, x, E, R, G, S, T)


@pytest.mark.parametrize("T,R,G,density,offset", [
    (40000, 8, 2, 0.3, 0),     # three passes of 16384 tokens, ragged tail; words of 4 ranks
    (16384, 16, 2, 0.05, 0),   # one full pass; two words per group
    (16385, 12, 4, 0.2, 0),    # one token past a pass; three rank bytes per group
    (33000, 8, 8, 0.1, 0),     # one rank per group
    (20000, 8, 1, 0.02, 0),    # a single group of all ranks
    (5000, 8, 2, 0.3, 1),      # map not 4-byte aligned: bytes even though 4 ranks per group
    (1024, 8, 2, 0.5, 0),      # the largest batch for 64-thread workgroups, one full pass
    (4097, 8, 4, 0.3, 0),      # one token past the 256-thread workgroups' pass
    (3000, 1024, 128, 0.005, 0),  # more groups than a wave has lanes
    (1, 4, 1, 1.0, 0),
])
def test_group_layout_maps(ep, T, R, G, density, offset):
    """ep_get_group_layout on synthetic maps, apart from ep_get_layout: any
    nonzero byte marks the rank, rows with no rank anywhere occur, and the
    per-group capacity drops the later tokens of the fuller groups."""
    print(f"[parity-hier] group layout T={T} R={R} G={G} offset={offset}", flush=True)
    rng = np.random.default_rng(T + 7 * R + G)
    m = np.where(rng.random((T, R)) < density, rng.integers(1, 256, (T, R)), 0).astype(np.uint8)
    p = ep.Problem.make(T, 8, R * min(8, 2048 // R), 1, R, G, 1, 1)   # E <= 2048
    for SG in (T, max(1, int(density * T * (R // G) * 0.5))):
        flat = torch.zeros(T * R + offset, dtype=torch.uint8, device="cuda")
        flat[offset:] = dev(m.ravel())
        gslot = torch.empty((T, G), dtype=torch.int32, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        ep.ep_get_group_layout(p, flat[offset:].view(T, R), SG, gslot, status)
        torch.cuda.synchronize()
        want, want_status = oracle.group_layout(m, G, SG, with_status=True)
        assert_same(gslot.cpu().numpy(), want, f"SG={SG}")
        assert int(status.item()) == want_status, f"SG={SG}"
