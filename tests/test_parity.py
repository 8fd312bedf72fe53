"""HIP path vs the CPU oracle, element by element, through the C ABI.

Layout outputs, slots and dispatched rows must match bit for bit; the bf16
combine output must satisfy |gpu - oracle| <= 1e-3 + 1e-2*|oracle| on every
element (the oracle sums in fp64, the kernel in fp32 with FMA).
"""
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



def bf16_dev(a_u16):
    return dev(a_u16.view(np.int16))


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def gpu_layout(ep, idx, E, R, S, G=1, A=1, H=8):
    T, K = idx.shape
    p = ep.Problem.make(T, H, E, K, R, G, A, S)
    bufs = ep.alloc_layout(p)
    d_idx = dev(idx) if T else torch.empty((0, K), dtype=torch.int32, device="cuda")
    ep.ep_get_layout(p, d_idx, *bufs.args())
    status = ep.ep_read_status(bufs.workspace)
    return p, bufs, status


def assert_layout_matches(ep, bufs, status, ref):
    code = {oracle.OK: ep.EP_OK, oracle.CAPACITY: ep.EP_ERR_CAPACITY,
            oracle.BAD_EXPERT: ep.EP_ERR_BAD_EXPERT}[ref.status]
    assert status == code
    for name in ("expert_count", "expert_offset", "rank_row_count", "rank_token_count",
                 "group_token_count", "is_token_in_rank", "token_slot"):
        assert_same(getattr(bufs, name).cpu().numpy(), getattr(ref, name),
                                      name)


def combine_close(got_u16, ref_u16):
    g = oracle.bf16_to_double(got_u16)
    r = oracle.bf16_to_double(ref_u16)
    bad = ~(np.abs(g - r) <= ATOL + RTOL * np.abs(r))
    assert not bad.any(), f"{bad.sum()} combine elements out of tolerance, first at {np.argwhere(bad)[:3]}"


def tight_stride(ref_counts, E, R, A=1):
    L = E // R
    aligned = -(-ref_counts // A) * A
    return int(max(1, aligned.reshape(R, L).sum(1).max()))


def run_full(ep, idx, w, x, E, R, G, A, S, y=None, check_src=True):
    """Layout + dispatch + combine on both sides; returns nothing, asserts."""
    T, K = idx.shape
    H = x.shape[1]
    ref = oracle.layout(idx, E, R, S, G, A)
    p, bufs, status = gpu_layout(ep, idx, E, R, S, G, A, H)
    assert_layout_matches(ep, bufs, status, ref)
    rows = R * S
    # dispatch
    d_x, d_w = bf16_dev(x), dev(w)
    recv = torch.empty((rows, H), dtype=torch.int16, device="cuda")
    src = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    rw = torch.full((rows,), -7.0, dtype=torch.float32, device="cuda")
    ep.ep_dispatch(p, d_x, d_w, bufs.token_slot, recv, src, rw)
    torch.cuda.synchronize()
    ref_rx, ref_src, ref_rw = oracle.dispatch(x, ref.token_slot, rows, w)
    s = ref.token_slot.ravel()
    s = s[s >= 0]
    got_rx = host_u16(recv)
    assert_same(got_rx[s], ref_rx[s])
    if check_src:
        assert_same(src.cpu().numpy()[s], ref_src[s])
        assert_same(rw.cpu().numpy()[s], ref_rw[s])
    # combine on expert outputs in the receive layout
    if y is None:
        y = ep_inputs.permuted_rows(ref_rx, seed=11)
    d_y = bf16_dev(y)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ep.ep_combine(p, d_y, bufs.token_slot, d_w, out)
    out_unit = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ep.ep_combine(p, d_y, bufs.token_slot, None, out_unit)
    torch.cuda.synchronize()
    combine_close(host_u16(out), oracle.combine(y, ref.token_slot, w))
    combine_close(host_u16(out_unit), oracle.combine(y, ref.token_slot, None))
    return ref, bufs, got_rx


# --------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["tiny", "decode128", "prefill4k", "zipf8k", "large16k"])
def test_workload_parity(ep, name):
    print(f"[parity] workload={name}", flush=True)
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    counts = np.bincount(inp.topk_idx.ravel(), minlength=wl.E)
    S = tight_stride(counts, wl.E, wl.R)
    y = None
    if name in ("tiny", "decode128"):
        y = ep_inputs.expert_outputs(wl.R * S, wl.H, seed=3)
    run_full(ep, inp.topk_idx, inp.topk_weights, inp.x, wl.E, wl.R, wl.G, wl.A, S, y=y)


@pytest.mark.parametrize("name", ["tiny", "decode128", "prefill4k", "zipf8k", "large16k"])
def test_workload_layout_at_default_stride(ep, name):
    """Layout at the worst-case slice stride the benchmark uses."""
    inp = ep_inputs.make_inputs(name, with_x=False)
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    ref = oracle.layout(inp.topk_idx, wl.E, wl.R, S, wl.G)
    p, bufs, status = gpu_layout(ep, inp.topk_idx, wl.E, wl.R, S, wl.G)
    assert ep.ep_rank_stride_hint(p) == S
    assert_layout_matches(ep, bufs, status, ref)


def test_unit_weight_combine_of_dispatch_is_x_times_k(ep):
    inp = ep_inputs.make_inputs("prefill4k")
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, 1, S)
    bufs = ep.alloc_layout(p)
    ep.ep_get_layout(p, dev(inp.topk_idx), *bufs.args())
    recv = torch.empty((wl.R * S, wl.H), dtype=torch.int16, device="cuda")
    d_x = bf16_dev(inp.x)
    ep.ep_dispatch(p, d_x, None, bufs.token_slot, recv)
    out = torch.empty_like(d_x)
    ep.ep_combine(p, recv, bufs.token_slot, None, out)
    torch.cuda.synchronize()
    # K is a power of two, so every partial sum is exact and out == K*x as
    # values.  Sums start from +0, so an all -0 column gives +0: compare
    # values (-0 == +0), not bit patterns.
    xk = (d_x.view(torch.bfloat16).float() * wl.K).to(torch.bfloat16)
    assert torch.equal(out.view(torch.bfloat16).float(), xk.float())


# --------------------------------------------------------------- edge cases

def _route_uniform(rng, T, E, K):
    return np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, K), np.int32)


def _case(ep, idx, E, R, G=1, A=1, S=None, H=64, seed=0):
    rng = np.random.default_rng(seed)
    T, K = idx.shape
    if S is None:
        counts = np.bincount(idx[(idx >= 0) & (idx < E)].ravel(), minlength=E)
        S = tight_stride(counts, E, R, A) + 5
    w = rng.standard_normal((T, K)).astype(np.float32)
    x = ep_inputs.bf16_normal(rng, (T, H))
    return run_full(ep, idx, w, x, E, R, G, A, S)


def test_single_token(ep):
    _case(ep, np.array([[5, 1, 9, 14]], np.int32), E=16, R=4, H=256)


def test_topk_equals_local_experts(ep):
    rng = np.random.default_rng(1)
    E, R = 32, 8
    idx = _route_uniform(rng, 300, E, E // R)
    _case(ep, idx, E, R, H=128)


def test_all_tokens_to_the_same_experts(ep):
    T, K = 3000, 8  # several chunks, every entry on experts 0..7 (rank 0)
    idx = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    ref, bufs, _ = _case(ep, idx, E=64, R=8, H=64)
    assert (bufs.rank_row_count.cpu().numpy()[1:] == 0).all()


def test_one_rank_empty(ep):
    rng = np.random.default_rng(2)
    E, R, T, K = 64, 8, 2500, 6
    idx = np.stack([rng.choice(np.arange(8, 64), K, replace=False) for _ in range(T)]).astype(np.int32)
    ref, bufs, _ = _case(ep, idx, E, R, H=64)
    assert bufs.rank_token_count.cpu().numpy()[0] == 0


@pytest.mark.parametrize("A", [2, 4, 128])
def test_expert_alignment(ep, A):
    rng = np.random.default_rng(A)
    idx = _route_uniform(rng, 1500, 64, 8)
    _case(ep, idx, 64, 8, A=A, H=64)


def test_empty_entries_and_duplicates(ep):
    rng = np.random.default_rng(4)
    idx = rng.integers(0, 48, size=(2100, 5)).astype(np.int32)   # duplicates allowed
    idx[rng.random(idx.shape) < 0.2] = -1
    _case(ep, idx, 48, 6, G=3, H=72)


def test_capacity_exact_and_one_short(ep):
    rng = np.random.default_rng(5)
    E, R, A = 64, 8, 4
    idx = _route_uniform(rng, 1200, E, 8)
    counts = np.bincount(idx.ravel(), minlength=E)
    S = tight_stride(counts, E, R, A)
    ref, _, _ = _case(ep, idx, E, R, A=A, S=S, H=64)
    assert ref.status == oracle.OK
    ref, _, _ = _case(ep, idx, E, R, A=A, S=S - 1, H=64)
    assert ref.status == oracle.CAPACITY


def test_bad_expert_id(ep):
    rng = np.random.default_rng(6)
    idx = _route_uniform(rng, 1100, 32, 4)
    idx[17, 2] = 32
    idx[900, 0] = -5
    ref, _, _ = _case(ep, idx, 32, 4, H=64)
    assert ref.status == oracle.BAD_EXPERT


def test_empty_batch(ep):
    idx = np.zeros((0, 4), np.int32)
    p, bufs, status = gpu_layout(ep, idx, 16, 4, 8, H=64)
    assert status == ep.EP_OK
    ref = oracle.layout(idx, 16, 4, 8)
    assert_layout_matches(ep, bufs, status, ref)
    # dispatch/combine of nothing is a no-op
    ep.ep_dispatch(p, None, None, None, None)
    ep.ep_combine(p, None, None, None, None)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(ep, seed):
    rng = np.random.default_rng(100 + seed)
    R = int(rng.choice([1, 2, 4, 8, 16]))
    L = int(rng.choice([1, 3, 8, 32]))
    E = R * L
    K = int(rng.integers(1, min(E, 12) + 1))
    T = int(rng.choice([1, 7, 129, 1000, 3333, 7001]))
    G = int(rng.choice([g for g in (1, 2, 4) if R % g == 0]))
    A = int(rng.choice([1, 1, 2, 8]))
    H = 8 * int(rng.integers(1, 200))
    idx = _route_uniform(rng, T, E, K)
    print(f"[parity] random seed={seed} T={T} H={H} E={E} K={K} R={R} G={G} A={A}", flush=True)
    _case(ep, idx, E, R, G=G, A=A, H=H, seed=seed)


@pytest.mark.parametrize("T,H,E,K,R", [
    (300, 16384, 64, 6, 8),       # 32 KB rows: several workgroups per row in both kernels
    (17, 65536, 16, 4, 4),        # 128 KB rows
    (131072, 32, 256, 8, 16),     # 1024 layout chunks: eight rounds of the scan pass
    (5000, 8, 32, 5, 4),          # one 16-byte vector per row
    (2100, 8200, 64, 4, 8),       # 1025 vectors: a last column run of one vector
])
def test_wide_rows_and_long_batches(ep, T, H, E, K, R):
    rng = np.random.default_rng(T + H)
    idx = _route_uniform(rng, T, E, K)
    print(f"[parity] T={T} H={H} E={E} K={K} R={R}", flush=True)
    _case(ep, idx, E, R, H=H, seed=T)


def test_largest_hidden_size(ep):
    """Rows of EP_MAX_HIDDEN channels (32 MiB): thousands of column pieces
    per token in every row kernel."""
    idx = np.array([[0, 3], [2, 1], [3, 0]], np.int32)
    print(f"[parity] H={ep.EP_MAX_HIDDEN}", flush=True)
    _case(ep, idx, E=4, R=2, H=ep.EP_MAX_HIDDEN, seed=5)


def test_large_expert_count_and_rank_count(ep):
    rng = np.random.default_rng(8)
    E, R, K, T = 2048, 1024, 32, 1500
    idx = _route_uniform(rng, T, E, K)
    _case(ep, idx, E, R, H=16)
    E, R = 2048, 8   # 256 local experts per rank
    _case(ep, _route_uniform(rng, T, E, K), E, R, H=16)


@pytest.mark.parametrize("T,E,R,G,K", [
    (100, 130, 65, 5, 6),      # one chunk; rows of 65 bytes: unaligned row starts
    (2500, 200, 100, 4, 6),    # count + table sums (15 chunks)
    (9000, 2048, 1024, 8, 3),  # count + scan (27 chunks of 341 tokens, 8 experts per thread)
    (300, 2048, 1024, 1024, 8),  # three chunks: the one call runs as a single kernel
    (512, 1024, 128, 8, 8),      # four chunks: the one call runs the count pass and one kernel
])
def test_many_ranks_map_and_unique_counts(ep, T, E, R, G, K):
    """More than 64 ranks: the chunk's map rows are cleared, then each entry
    sets its rank's byte; unique tokens per rank and group count a token's
    first entry on each.  Empty entries and two entries of one token on the
    same rank occur."""
    print(f"[parity] many ranks T={T} E={E} R={R} G={G} K={K}", flush=True)
    rng = np.random.default_rng(T + R)
    idx = _route_uniform(rng, T, E, K)
    L = E // R
    same_rank = rng.random(T) < 0.3           # second entry on the first entry's rank
    idx[same_rank, 1] = (idx[same_rank, 0] // L) * L + (idx[same_rank, 0] + 1) % L
    dup = idx[same_rank, 1] == idx[same_rank, 0]
    idx[np.flatnonzero(same_rank)[dup], 1] = -1
    idx[rng.random(idx.shape) < 0.05] = -1
    H = 64
    counts = np.bincount(idx[idx >= 0].ravel(), minlength=E)
    S = tight_stride(counts, E, R) + 5
    w = rng.standard_normal((T, K)).astype(np.float32)
    x = ep_inputs.bf16_normal(rng, (T, H))
    ref, _, _ = run_full(ep, idx, w, x, E, R, G, 1, S)
    # the one-call layout and dispatch leaves the same layout and rows
    p = ep.Problem.make(T, H, E, K, R, G, 1, S)
    bufs = ep.alloc_layout(p)
    recv = torch.empty((R * S, H), dtype=torch.int16, device="cuda")
    ep.ep_layout_dispatch(p, dev(idx), *bufs.args(), None, bf16_dev(x), dev(w), recv, None, None)
    assert_layout_matches(ep, bufs, ep.ep_read_status(bufs.workspace), ref)
    sl = ref.token_slot[ref.token_slot >= 0]
    assert_same(host_u16(recv)[sl], oracle.dispatch(x, ref.token_slot, R * S, w)[0][sl])


@pytest.mark.parametrize("T,H,K", [(20001, 8, 4), (5000, 64, 8), (17000, 504, 6), (40000, 8, 1), (20000, 16, 2),
                                   (3001, 8, 3), (900, 512, 4)])
def test_narrow_rows(ep, T, H, K):
    """Rows under 1 KB take one thread per (entry, vector) in dispatch and per
    (token, vector) in combine once the batch fills the chip that way:
    one-vector rows with a ragged last workgroup, 8 and 63 vectors; a small
    batch of one-vector rows that stays on the per-token kernels; and 64
    vectors, the first width that always does."""
    print(f"[parity] narrow rows T={T} H={H} K={K}", flush=True)
    rng = np.random.default_rng(T + H)
    idx = _route_uniform(rng, T, 64, K)
    idx[rng.random(idx.shape) < 0.05] = -1
    _case(ep, idx, 64, 8, H=H, seed=T)


def test_cumulative_expert_counts_and_cached_layout(ep):
    """Cumulative per-expert receive counts across calls, and dispatch/combine
    reusing one layout (cached mode) for new activations."""
    inp = ep_inputs.make_inputs("prefill4k")
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, 1, S)
    bufs = ep.alloc_layout(p, cumulative=True)
    ref = oracle.layout(inp.topk_idx, wl.E, wl.R, S)
    idx2 = ep_inputs.make_inputs("prefill4k", seed=5, with_x=False).topk_idx
    ref2 = oracle.layout(idx2, wl.E, wl.R, S)
    ep.ep_get_layout(p, dev(inp.topk_idx), *bufs.args())
    ep.ep_get_layout(p, dev(idx2), *bufs.args())
    ep.ep_get_layout(p, dev(inp.topk_idx), *bufs.args())
    want = 2 * ref.expert_count.astype(np.int64) + ref2.expert_count
    assert_same(bufs.cumulative_expert_recv.cpu().numpy(), want)
    # cached mode: the last layout serves two dispatch/combine rounds
    rows = wl.R * S
    recv = torch.empty((rows, wl.H), dtype=torch.int16, device="cuda")
    rw = torch.empty(rows, dtype=torch.float32, device="cuda")
    comb_w = torch.empty((wl.T, wl.K), dtype=torch.float32, device="cuda")
    s = ref.token_slot.ravel()
    for seed in (21, 22):
        x = ep_inputs.bf16_normal(np.random.default_rng(seed), (wl.T, wl.H))
        ep.ep_dispatch(p, bf16_dev(x), dev(inp.topk_weights), bufs.token_slot, recv, None, rw)
        ep.ep_combine_topk_weights(p, rw, bufs.token_slot, comb_w)
        torch.cuda.synchronize()
        ref_rx, _, _ = oracle.dispatch(x, ref.token_slot, rows, inp.topk_weights)
        assert_same(host_u16(recv)[s], ref_rx[s])
        assert_same(comb_w.cpu().numpy(), inp.topk_weights)


def test_combined_topk_weights_with_invalid_slots(ep):
    rng = np.random.default_rng(9)
    idx = rng.integers(0, 32, size=(1500, 4)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    E, R = 32, 4
    counts = np.bincount(idx[idx >= 0].ravel(), minlength=E)
    S = tight_stride(counts, E, R) - 3          # overflow: some slots become -1
    ref = oracle.layout(idx, E, R, S)
    assert ref.status == oracle.CAPACITY
    p, bufs, status = gpu_layout(ep, idx, E, R, S, H=64)
    assert_layout_matches(ep, bufs, status, ref)
    recv_w = rng.standard_normal(R * S).astype(np.float32)
    out = torch.empty((1500, 4), dtype=torch.float32, device="cuda")
    ep.ep_combine_topk_weights(p, dev(recv_w), bufs.token_slot, out)
    torch.cuda.synchronize()
    assert_same(out.cpu().numpy(), oracle.combine_topk_weights(recv_w, ref.token_slot))


@pytest.mark.parametrize("T,K,E,R,bad,short", [
    (21000, 8, 256, 16, True, False),    # 165 chunks: count + scan + assign
    (21000, 8, 256, 16, False, True),
    (1024, 8, 2048, 8, True, True),      # 8 chunks, 2048 experts: count + summing assign
    (3000, 3, 12, 3, False, True),       # K not dividing the chunk
])
def test_device_errors_in_every_layout_mode(ep, T, K, E, R, bad, short):
    rng = np.random.default_rng(T + K + E)
    idx = _route_uniform(rng, T, E, K)
    if bad:
        idx[rng.integers(0, T, 5), rng.integers(0, K, 5)] = E + 3
        idx[7, 0] = -9
    counts = np.bincount(idx[(idx >= 0) & (idx < E)].ravel(), minlength=E)
    S = tight_stride(counts, E, R) - (7 if short else 0)
    ref = oracle.layout(idx, E, R, S)
    assert ref.status == (oracle.BAD_EXPERT if bad else oracle.CAPACITY)
    p, bufs, status = gpu_layout(ep, idx, E, R, S, H=64)
    assert_layout_matches(ep, bufs, status, ref)


@pytest.mark.parametrize("name", ["tiny", "decode128", "zipf8k", "large16k"])
def test_repeatable(ep, name):
    """Ten runs of the layout (every mode) and of the one-call layout and
    dispatch with the combine after it give bitwise identical slots, rows and
    outputs: no atomic decides an order anywhere."""
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    outs = []
    for _ in range(10):
        _, bufs, _ = gpu_layout(ep, inp.topk_idx, wl.E, wl.R, S)
        outs.append(bufs.token_slot.cpu().numpy())
    assert all((o == outs[0]).all() for o in outs)
    counts = np.bincount(inp.topk_idx.ravel(), minlength=wl.E)
    S = tight_stride(counts, wl.E, wl.R)
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, wl.A, S)
    bufs = ep.alloc_layout(p)
    recv = torch.zeros((wl.R * S, wl.H), dtype=torch.int16, device="cuda")
    out = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
    d_idx, d_x, d_w = dev(inp.topk_idx), bf16_dev(inp.x), dev(inp.topk_weights)
    first = None
    for _ in range(10):
        ep.ep_layout_dispatch(p, d_idx, *bufs.args(), None, d_x, d_w, recv)
        ep.ep_combine(p, recv, bufs.token_slot, d_w, out)
        got = (bufs.token_slot.clone(), recv.clone(), out.clone())
        if first is None:
            first = got
        else:
            assert all(torch.equal(a, b) for a, b in zip(first, got))
    assert ep.ep_read_status(bufs.workspace) == ep.EP_OK


def test_bound_calls_repeat_the_direct_calls(ep):
    """Calls marshalled once (bind=True) give the direct calls' results, and
    repeating them repeats the work."""
    inp = ep_inputs.make_inputs("decode128")
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, wl.A, S)
    rows = wl.R * S
    d_idx, d_x, d_w = dev(inp.topk_idx), bf16_dev(inp.x), dev(inp.topk_weights)
    a, b = ep.alloc_layout(p, cumulative=True), ep.alloc_layout(p, cumulative=True)
    ra = torch.zeros((rows, wl.H), dtype=torch.int16, device="cuda")
    rb = torch.zeros_like(ra)
    oa = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
    ob = torch.empty_like(oa)
    calls = [ep.ep_get_layout(p, d_idx, *a.args(), bind=True),
             ep.ep_dispatch(p, d_x, d_w, a.token_slot, ra, bind=True),
             ep.ep_combine(p, ra, a.token_slot, d_w, oa, bind=True)]
    for _ in range(2):
        for f in calls:
            f()
        ep.ep_get_layout(p, d_idx, *b.args())
        ep.ep_dispatch(p, d_x, d_w, b.token_slot, rb)
        ep.ep_combine(p, rb, b.token_slot, d_w, ob)
    torch.cuda.synchronize()
    assert torch.equal(a.token_slot, b.token_slot)
    assert torch.equal(ra, rb)
    assert torch.equal(oa, ob)
    # the cumulative counter saw both bound layouts
    assert torch.equal(a.cumulative_expert_recv, 2 * a.expert_count.to(torch.int64))
    assert torch.equal(a.cumulative_expert_recv, b.cumulative_expert_recv)
