"""ep_layout_dispatch (layout and dispatch in one call) vs the CPU oracle.

Decode-sized batches (one layout chunk) run as a single kernel in which each
dispatching workgroup derives its token's slots itself; batches of up to 128
chunks (with expert_alignment 1) run the count pass and then one kernel that
does the same from the per-chunk counts; other batches run the separate
kernels.  All must give the layout outputs, slots and dispatched rows of the
oracle bit for bit, and must write no receive row that no slot names.
"""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from test_parity import assert_layout_matches, assert_same, bf16_dev, dev, host_u16, tight_stride

pytestmark = pytest.mark.gpu

SENTINEL = -21555  # int16 pattern of receive rows before dispatch


@pytest.fixture(scope="module")
def ep():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import combine_ep_get_amd as ep
    ep.load()
    return ep


def run_fused(ep, idx, w, x, E, R, G=1, A=1, S=None, cumulative=False, weights=True):
    T, K = idx.shape
    H = x.shape[1]
    if S is None:
        S = max(1, oracle.default_rank_stride(T, K, E, R, A))
    print(f"[fused] T={T} K={K} E={E} R={R} G={G} A={A} S={S} H={H}", flush=True)
    ref = oracle.layout(idx, E, R, S, G, A)
    p = ep.Problem.make(T, H, E, K, R, G, A, S)
    bufs = ep.alloc_layout(p, cumulative=cumulative)
    rows = R * S
    recv = torch.full((rows, H), SENTINEL, dtype=torch.int16, device="cuda")
    src = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    rw = torch.full((rows,), -7.0, dtype=torch.float32, device="cuda")
    d_idx = dev(idx) if T else torch.empty((0, K), dtype=torch.int32, device="cuda")
    d_x = bf16_dev(x) if T else torch.empty((0, H), dtype=torch.int16, device="cuda")
    d_w = dev(w) if (weights and T) else None
    ep.ep_layout_dispatch(p, d_idx, *bufs.args(), None, d_x, d_w, recv, src, rw)
    status = ep.ep_read_status(bufs.workspace)
    assert_layout_matches(ep, bufs, status, ref)
    if cumulative:
        assert_same(bufs.cumulative_expert_recv.cpu().numpy(), ref.expert_count.astype(np.int64))
    ref_rx, ref_src, ref_rw = oracle.dispatch(x, ref.token_slot, rows, w if weights else None)
    s = ref.token_slot.ravel()
    s = s[s >= 0]
    got = host_u16(recv)
    assert_same(got[s], ref_rx[s], "recv_x")
    assert_same(src.cpu().numpy()[s], ref_src[s], "recv_src_token")
    assert_same(rw.cpu().numpy()[s], ref_rw[s], "recv_weight")
    untouched = np.ones(rows, bool)
    untouched[s] = False
    assert (got[untouched] == np.uint16(SENTINEL & 0xFFFF)).all(), "a row no slot names was written"
    assert (src.cpu().numpy()[untouched] == -7).all()
    return ref, bufs


@pytest.mark.parametrize("name", ["tiny", "decode128", "prefill4k", "zipf8k", "large16k"])
def test_workloads(ep, name):
    """Every workload through the call the benchmark times: one chunk
    (tiny, decode128), 32 and 64 chunks with the per-chunk sums loaded late
    and early (prefill4k, zipf8k), 128 chunks in two rounds (large16k).  The
    default stride too where its receive buffer stays small."""
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    counts = np.bincount(inp.topk_idx.ravel(), minlength=wl.E)
    strides = [tight_stride(counts, wl.E, wl.R)]
    if name in ("tiny", "decode128", "prefill4k"):
        strides.append(None)
    for S in strides:
        run_fused(ep, inp.topk_idx, inp.topk_weights, inp.x, wl.E, wl.R, wl.G, wl.A, S)


@pytest.mark.parametrize("seed", range(16))
def test_random_small_cases(ep, seed):
    """-1 entries, duplicate experts, groups, alignment, odd K and H."""
    rng = np.random.default_rng(1000 + seed)
    idx, E, R, G, K = ep_inputs.random_small_case(rng, max_T=96, max_E=64, max_K=8,
                                                  allow_duplicates=seed % 2 == 1)
    T = idx.shape[0]
    A = int(rng.choice([1, 1, 2, 4]))
    H = int(rng.choice([8, 64, 264, 1032]))
    x = ep_inputs.bf16_normal(rng, (T, H))
    w = rng.standard_normal((T, K)).astype(np.float32)
    run_fused(ep, idx, w, x, E, R, G, A, cumulative=seed % 3 == 0, weights=seed % 4 != 0)


@pytest.mark.parametrize("T,K", [(1, 1), (1, 32), (32, 32), (128, 8), (129, 8), (170, 6), (171, 6),
                                 (341, 3), (1024, 1), (1025, 1)])
def test_chunk_boundary(ep, T, K):
    """Batches exactly at, and one token past, a single layout chunk."""
    rng = np.random.default_rng(T * 100 + K)
    E, R = 64, 8
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    x = ep_inputs.bf16_normal(rng, (T, 128))
    w = rng.random((T, K)).astype(np.float32)
    run_fused(ep, idx, w, x, E, R)


def test_many_experts_and_ranks(ep):
    """E = 2048 over R = 1024 ranks (two experts each, more ranks than a wave)."""
    rng = np.random.default_rng(7)
    T, K, E, R = 96, 8, 2048, 1024
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    x = ep_inputs.bf16_normal(rng, (T, 64))
    w = rng.random((T, K)).astype(np.float32)
    run_fused(ep, idx, w, x, E, R, G=4)


def test_skewed_routing_and_capacity(ep):
    """Every token on the same experts; a slice one row short overflows."""
    T, K, E, R = 100, 4, 32, 4
    idx = np.tile(np.array([0, 1, 2, 9], np.int32), (T, 1))
    rng = np.random.default_rng(3)
    x = ep_inputs.bf16_normal(rng, (T, 256))
    w = rng.random((T, K)).astype(np.float32)
    ref, _ = run_fused(ep, idx, w, x, E, R, S=3 * T)
    assert ref.status == oracle.OK
    ref, _ = run_fused(ep, idx, w, x, E, R, S=3 * T - 1)
    assert ref.status == oracle.CAPACITY


def test_bad_expert_id(ep):
    rng = np.random.default_rng(4)
    T, K, E, R = 50, 4, 16, 4
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    idx[7, 2] = E + 3
    idx[9, 0] = -5
    idx[11, 1] = -1
    x = ep_inputs.bf16_normal(rng, (T, 64))
    w = rng.random((T, K)).astype(np.float32)
    ref, _ = run_fused(ep, idx, w, x, E, R)
    assert ref.status == oracle.BAD_EXPERT


def test_empty_batch(ep):
    x = np.zeros((0, 64), np.uint16)
    run_fused(ep, np.zeros((0, 4), np.int32), np.zeros((0, 4), np.float32), x, 16, 4)


def test_matches_separate_calls_repeatedly(ep):
    """Two calls in a row, the second smaller, against ep_get_layout + ep_dispatch."""
    for name, T in (("decode128", 128), ("decode128", 40)):
        inp = ep_inputs.make_inputs(name)
        wl = inp.wl
        idx, w, x = inp.topk_idx[:T], inp.topk_weights[:T], inp.x[:T]
        S = oracle.default_rank_stride(T, wl.K, wl.E, wl.R)
        p = ep.Problem.make(T, wl.H, wl.E, wl.K, wl.R, wl.G, wl.A, S)
        a, b = ep.alloc_layout(p), ep.alloc_layout(p)
        rows = wl.R * S
        ra = torch.zeros((rows, wl.H), dtype=torch.int16, device="cuda")
        rb = torch.zeros_like(ra)
        d_idx, d_x, d_w = dev(idx), bf16_dev(x), dev(w)
        ep.ep_layout_dispatch(p, d_idx, *a.args(), None, d_x, d_w, ra)
        ep.ep_get_layout(p, d_idx, *b.args())
        ep.ep_dispatch(p, d_x, d_w, b.token_slot, rb)
        torch.cuda.synchronize()
        for name_ in ("expert_count", "expert_offset", "rank_row_count", "rank_token_count",
                      "is_token_in_rank", "token_slot"):
            assert torch.equal(getattr(a, name_), getattr(b, name_)), name_
        assert torch.equal(ra, rb)


@pytest.mark.parametrize("seed", range(12))
def test_multi_chunk_random_cases(ep, seed):
    """Two to 128 chunks: -1 entries, duplicates, bad ids, groups, R above a wave."""
    rng = np.random.default_rng(2000 + seed)
    R = int(rng.choice([2, 8, 96, 128]))
    L = int(rng.choice([1, 2, 5, 16]))
    E = min(R * L, 2048)
    L = E // R
    K = int(rng.integers(1, min(E, 9) + 1))
    chunk_tokens = 1024 // K
    T = int(rng.integers(chunk_tokens + 1, min(128 * chunk_tokens, 17000) + 1))
    G = int(rng.choice([g for g in (1, 2, 4) if R % g == 0]))
    if seed % 2:
        idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    else:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    idx[rng.random((T, K)) < 0.1] = -1
    if seed % 3 == 0:
        idx[rng.integers(0, T, 3), rng.integers(0, K, 3)] = E + 5
    H = int(rng.choice([8, 64, 520]))
    x = ep_inputs.bf16_normal(rng, (T, H))
    w = rng.standard_normal((T, K)).astype(np.float32)
    S = None   # the default (worst-case) stride, unless that buffer passes 256 MB
    if R * oracle.default_rank_stride(T, K, E, R) * H * 2 > 256 << 20:
        S = tight_stride(np.bincount(idx[(idx >= 0) & (idx < E)], minlength=E), E, R)
    run_fused(ep, idx, w, x, E, R, G, S=S, cumulative=seed % 4 == 0)


@pytest.mark.parametrize("T,K,A,short", [(700, 8, 1, True), (700, 8, 4, False), (64 * 128, 8, 1, False),
                                         (65 * 128, 8, 1, False), (128 * 128, 8, 1, True),
                                         (129 * 128, 8, 1, False), (3000, 3, 1, True)])
def test_multi_chunk_paths_and_capacity(ep, T, K, A, short):
    """The two-launch path at its limits (64 and 65 chunks: one and two rounds
    of per-chunk sums; 128 chunks; a slice one row short), and the batches
    that take the separate kernels (A > 1, 129 chunks)."""
    rng = np.random.default_rng(T + K + A)
    E, R = 64, 8
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    S = None
    if short:
        counts = np.bincount(idx.ravel(), minlength=E)
        S = tight_stride(counts, E, R, A) - 1
    x = ep_inputs.bf16_normal(rng, (T, 64))
    w = rng.random((T, K)).astype(np.float32)
    ref, _ = run_fused(ep, idx, w, x, E, R, A=A, S=S)
    assert ref.status == (oracle.CAPACITY if short else oracle.OK)


@pytest.mark.parametrize("T,K,H", [(2100, 4, 8200), (2100, 4, 7168), (1100, 8, 2056), (300, 8, 1032),
                                   (5000, 1, 8)])
def test_multi_chunk_row_widths(ep, T, K, H):
    """The two-launch path on rows of 1 to 1025 16-byte vectors (one vector
    per thread up to several per thread, whole rows and rows split into
    column runs)."""
    rng = np.random.default_rng(T * K + H)
    E, R = 64, 8
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    counts = np.bincount(idx.ravel(), minlength=E)
    x = ep_inputs.bf16_normal(rng, (T, H))
    w = rng.random((T, K)).astype(np.float32)
    run_fused(ep, idx, w, x, E, R, S=tight_stride(counts, E, R))


def test_largest_hidden_size(ep):
    """The one-chunk kernel on rows of EP_MAX_HIDDEN channels (32 MiB)."""
    rng = np.random.default_rng(6)
    idx = np.array([[0, 3], [2, 1], [3, 0]], np.int32)
    x = ep_inputs.bf16_normal(rng, (3, ep.EP_MAX_HIDDEN))
    w = rng.random((3, 2)).astype(np.float32)
    run_fused(ep, idx, w, x, 4, 2)


@pytest.mark.parametrize("T,K,E,R,G", [(3000, 32, 2048, 8, 2), (1500, 32, 64, 64, 4), (2000, 17, 512, 128, 4)])
def test_multi_chunk_wide_top_k(ep, T, K, E, R, G):
    """Top-k up to 32 across many chunks: several rounds of positions per wave,
    256 experts per rank, one expert per rank, R above a wave."""
    rng = np.random.default_rng(T + K + E)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    counts = np.bincount(idx.ravel(), minlength=E)
    x = ep_inputs.bf16_normal(rng, (T, 64))
    w = rng.random((T, K)).astype(np.float32)
    run_fused(ep, idx, w, x, E, R, G, S=tight_stride(counts, E, R), cumulative=True)


@pytest.mark.parametrize("seed", range(10))
def test_few_chunk_single_kernel(ep, seed):
    """Batches of two to four chunks run as a single kernel (the layout
    workgroups take the batch chunk by chunk): alignment, slices one row
    short, bad and empty ids, duplicates, groups, R above a wave."""
    rng = np.random.default_rng(3000 + seed)
    R = int(rng.choice([2, 8, 96, 128]))
    L = int(rng.choice([1, 2, 4]))
    E = R * L
    K = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1024 // K + 1, 4096 // K + 1))
    G = int(rng.choice([g for g in (1, 2, 4) if R % g == 0]))
    A = int(rng.choice([1, 1, 2, 3]))
    if seed % 2:
        idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    else:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    idx[rng.random((T, K)) < 0.05] = -1
    if seed % 3 == 0:
        idx[rng.integers(0, T, 2), rng.integers(0, K, 2)] = E + 1
    S = None
    if seed % 4 == 1:
        ok = (idx >= 0) & (idx < E)
        S = tight_stride(np.bincount(idx[ok], minlength=E), E, R, A) - 1
    x = ep_inputs.bf16_normal(rng, (T, 64))
    w = rng.standard_normal((T, K)).astype(np.float32)
    ref, _ = run_fused(ep, idx, w, x, E, R, G, A, S=S, cumulative=seed % 3 == 1)
    if S is not None and ref.status != oracle.BAD_EXPERT:
        assert ref.status == oracle.CAPACITY
