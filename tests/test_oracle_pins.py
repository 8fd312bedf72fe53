"""Pins for the CPU oracle: checks against things other than the oracle itself.

- a hand-worked example (tests/golden/layout_handworked.json);
- brute force on tiny inputs, straight from the definition of each output
  (position of an entry = number of earlier entries naming the same expert),
  which is a different algorithm from the oracle's counting sort;
- numpy routines: bincount for the expert histogram, a stable argsort for the
  slot order, fancy indexing and an fp64 einsum for dispatch and combine;
- invariants: counts sum to T*K, slots are injective and fill each segment,
  source indices rise inside each segment, unit-weight combine of dispatched
  rows gives x*K exactly, one-hot weights give x back;
- the pages' closed form for the expected number of distinct ranks a token
  touches under uniform routing ("DeepEP V2 ElasticBuffer 架构深度分析",
  get_theoretical_num_sms block, get_expected_topk);
- torch's float32 -> bfloat16 conversion and a nearest-value search over all
  bf16 values for the rounding step.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import ep_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_handworked.json")
STATUS = {"ok": oracle.OK, "capacity": oracle.CAPACITY, "bad_expert": oracle.BAD_EXPERT}


# ---------------------------------------------------------------- brute force

def brute_layout(idx, E, R, G, A, S):
    """Every output from its definition, with plain loops (tiny inputs only)."""
    T, K = idx.shape
    L = E // R
    valid = lambda e: 0 <= e < E
    flat = [(t, j, int(idx[t, j])) for t in range(T) for j in range(K)]
    count = [sum(1 for (_, _, e) in flat if e == x) for x in range(E)]
    align = lambda v: -(-v // A) * A
    offset = [sum(align(count[(x // L) * L + l]) for l in range(x % L)) for x in range(E)]
    rank_rows = [sum(count[r * L + l] for l in range(L)) for r in range(R)]
    in_rank = np.array([[int(any(valid(int(idx[t, j])) and int(idx[t, j]) // L == r
                                 for j in range(K))) for r in range(R)] for t in range(T)],
                       dtype=np.uint8).reshape(T, R)
    rank_tok = [int(in_rank[:, r].sum()) for r in range(R)]
    per_g = R // G
    group_tok = [sum(1 for t in range(T) if in_rank[t, g * per_g:(g + 1) * per_g].any())
                 for g in range(G)]
    slot = np.full((T, K), -1, np.int64)
    for n, (t, j, e) in enumerate(flat):
        if not valid(e):
            continue
        pos = sum(1 for (_, _, e2) in flat[:n] if e2 == e)
        off = offset[e] + pos
        slot[t, j] = (e // L) * S + off if off < S else -1
    bad = any(e != -1 and not valid(e) for (_, _, e) in flat)
    over = any(offset[r * L + L - 1] + align(count[r * L + L - 1]) > S for r in range(R))
    status = oracle.BAD_EXPERT if bad else (oracle.CAPACITY if over else oracle.OK)
    return dict(status=status, expert_count=count, expert_offset=offset,
                rank_row_count=rank_rows, rank_token_count=rank_tok,
                group_token_count=group_tok, is_token_in_rank=in_rank, token_slot=slot)


def assert_layout_equal(lay, ref):
    assert lay.status == ref["status"]
    for name in ("expert_count", "expert_offset", "rank_row_count", "rank_token_count",
                 "group_token_count"):
        np.testing.assert_array_equal(getattr(lay, name), np.asarray(ref[name]), err_msg=name)
    np.testing.assert_array_equal(lay.is_token_in_rank, np.asarray(ref["is_token_in_rank"]))
    np.testing.assert_array_equal(lay.token_slot, np.asarray(ref["token_slot"]))


# ---------------------------------------------------------------- golden

def test_golden_handworked_layout():
    g = json.load(open(GOLDEN))
    idx = np.array(g["topk_idx"], np.int32)
    for case in g["cases"]:
        lay = oracle.layout(idx, g["E"], g["R"], case["S"], g["G"], case["A"])
        ref = dict(case)
        ref["status"] = STATUS[case["status"]]
        assert_layout_equal(lay, ref)


def test_golden_handworked_combine():
    g = json.load(open(GOLDEN))
    idx = np.array(g["topk_idx"], np.int32)
    lay = oracle.layout(idx, g["E"], g["R"], 8, 1, 1)
    s = np.arange(16, dtype=np.float32)
    y = torch.from_numpy(np.stack([s, s / 2], 1)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = oracle.combine(y, lay.token_slot, np.array(g["combine"]["weights"], np.float32))
    np.testing.assert_array_equal(oracle.bf16_to_double(out), np.array(g["combine"]["out"]))


def test_golden_rounding_ties():
    g = json.load(open(GOLDEN))["rounding"]
    got = oracle.double_to_bf16(np.array(g["sums"], np.float64))
    np.testing.assert_array_equal(got, np.array(g["bf16_bits"], np.uint16))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(60))
def test_layout_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    idx, E, R, G, K = ep_inputs.random_small_case(
        rng, max_T=24, max_E=12, max_K=5, allow_empty=seed % 2 == 0,
        allow_duplicates=seed % 3 == 0)
    T = idx.shape[0]
    A = int(rng.choice([1, 1, 2, 3, 4]))
    Sfull = oracle.default_rank_stride(T, K, E, R, A)
    S = int(rng.choice([Sfull, max(1, Sfull // 2), max(1, Sfull // 4), Sfull + 3]))
    if seed % 10 == 7 and T:
        idx[rng.integers(0, T), rng.integers(0, K)] = E + int(rng.integers(0, 3))  # bad id
    lay = oracle.layout(idx, E, R, S, G, A)
    assert_layout_equal(lay, brute_layout(idx, E, R, G, A, S))


def test_negative_bad_id_flags_error():
    idx = np.array([[0, -2], [1, 0]], np.int32)
    lay = oracle.layout(idx, 2, 1, 4)
    assert lay.status == oracle.BAD_EXPERT
    assert lay.token_slot[0, 1] == -1 and lay.expert_count.tolist() == [2, 1]


def test_empty_batch():
    idx = np.zeros((0, 4), np.int32)
    lay = oracle.layout(idx, 16, 4, 1)
    assert lay.status == oracle.OK
    assert lay.expert_count.sum() == 0 and lay.token_slot.shape == (0, 4)
    assert (lay.rank_token_count == 0).all()


# ---------------------------------------------------------------- numpy routines + invariants

def _check_workload_layout(idx, E, R, G, S, A=1):
    T, K = idx.shape
    L = E // R
    lay = oracle.layout(idx, E, R, S, G, A)
    assert lay.status == oracle.OK
    # numpy histogram
    np.testing.assert_array_equal(lay.expert_count, np.bincount(idx.ravel(), minlength=E))
    assert lay.expert_count.sum() == T * K
    assert lay.rank_row_count.sum() == T * K
    # slot order: a stable argsort of the flattened expert ids lists the
    # entries of each expert in exactly the order the slots number them
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    slots = lay.token_slot.ravel()
    se = flat[order]
    starts = np.searchsorted(se, np.arange(E))
    pos = np.arange(len(order)) - starts[se]
    align = lambda v: -(-v // A) * A
    seg = align(lay.expert_count).reshape(R, L)
    off = (np.cumsum(seg, axis=1) - seg).ravel()
    expect = (se // L) * S + off[se] + pos
    np.testing.assert_array_equal(slots[order], expect)
    # injective, and the image is exactly the union of the segment ranges
    assert len(np.unique(slots)) == len(slots)
    img = np.concatenate([(e // L) * S + off[e] + np.arange(lay.expert_count[e]) for e in range(E)])
    np.testing.assert_array_equal(np.sort(slots), np.sort(img))
    # token-to-rank map
    rs = lay.is_token_in_rank.sum(1)
    assert (rs >= 1).all() and (rs <= min(K, R)).all()
    np.testing.assert_array_equal(lay.rank_token_count, lay.is_token_in_rank.sum(0))
    assert (lay.rank_token_count <= lay.rank_row_count).all()
    ranks = idx // L
    for r in range(R):
        np.testing.assert_array_equal(lay.is_token_in_rank[:, r], (ranks == r).any(1))
    per_g = R // G
    for g in range(G):
        assert lay.group_token_count[g] == lay.is_token_in_rank[:, g * per_g:(g + 1) * per_g].any(1).sum()
    return lay


@pytest.mark.parametrize("name", ["tiny", "prefill4k", "decode128", "zipf8k", "large16k"])
def test_workload_layout_invariants(name):
    wl = ep_inputs.WORKLOADS[name]
    inp = ep_inputs.make_inputs(wl, with_x=False)
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    _check_workload_layout(inp.topk_idx, wl.E, wl.R, wl.G, S)


def test_layout_invariants_with_alignment():
    wl = ep_inputs.WORKLOADS["zipf8k"]
    inp = ep_inputs.make_inputs(wl, with_x=False)
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R, 8)
    _check_workload_layout(inp.topk_idx, wl.E, wl.R, 1, S, A=8)


# ---------------------------------------------------------------- closed form from the pages

def expected_ranks_per_token(E, R, K):
    """G*(1 - C(E - E/G, K)/C(E, K)) with the R ranks as the G groups."""
    return R * (1 - math.comb(E - E // R, K) / math.comb(E, K))


@pytest.mark.parametrize("E,R,K,routing,T", [
    (16, 4, 4, "uniform", 20000),
    (256, 8, 8, "gauss_topk", 20000),
    (256, 16, 8, "gauss_topk", 20000),
])
def test_ranks_per_token_matches_closed_form(E, R, K, routing, T):
    rng = np.random.default_rng(1234)
    idx, _ = ep_inputs.route(T, E, K, routing, rng)
    lay = oracle.layout(idx, E, R, oracle.default_rank_stride(T, K, E, R))
    rs = lay.is_token_in_rank.sum(1).astype(np.float64)
    mu = expected_ranks_per_token(E, R, K)
    assert abs(rs.mean() - mu) <= 5 * rs.std() / math.sqrt(T) + 1e-12, (rs.mean(), mu)


def test_closed_form_values_at_the_workloads():
    assert round(expected_ranks_per_token(16, 4, 4), 3) == 2.912
    assert round(expected_ranks_per_token(256, 8, 8), 3) == 5.295
    assert round(expected_ranks_per_token(256, 16, 8), 3) == 6.523


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("name", ["tiny", "decode128"])
def test_dispatch_rows_are_copies(name):
    wl = ep_inputs.WORKLOADS[name]
    inp = ep_inputs.make_inputs(wl)
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, wl.G)
    rows = wl.R * S
    rx, src, rw = oracle.dispatch(inp.x, lay.token_slot, rows, inp.topk_weights)
    t_of = np.repeat(np.arange(wl.T), wl.K)
    s = lay.token_slot.ravel()
    np.testing.assert_array_equal(rx[s], inp.x[t_of])            # bytewise
    np.testing.assert_array_equal(src[s], t_of)
    np.testing.assert_array_equal(rw[s], inp.topk_weights.ravel())
    untouched = np.setdiff1d(np.arange(rows), s)
    assert (src[untouched] == -1).all() and (rx[untouched] == 0).all()
    # source token indices rise inside each segment
    L = wl.E // wl.R
    for e in range(wl.E):
        base = (e // L) * S + lay.expert_offset[e]
        seg = src[base:base + lay.expert_count[e]]
        assert (np.diff(seg) > 0).all()


def test_dispatch_without_weights_or_maps():
    inp = ep_inputs.make_inputs("tiny")
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S)
    rx, src, rw = oracle.dispatch(inp.x, lay.token_slot, wl.R * S, None, with_src=False)
    assert src is None
    np.testing.assert_array_equal(rw[lay.token_slot.ravel()], 1.0)


def test_combined_topk_weights_round_trip():
    """Weights carried by the dispatched rows come back in token order."""
    inp = ep_inputs.make_inputs("tiny")
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S)
    _, _, rw = oracle.dispatch(inp.x, lay.token_slot, wl.R * S, inp.topk_weights)
    np.testing.assert_array_equal(oracle.combine_topk_weights(rw, lay.token_slot), inp.topk_weights)
    slot = lay.token_slot.copy()
    slot[0, 1] = -1
    slot[1, 0] = wl.R * S     # outside the buffer
    got = oracle.combine_topk_weights(rw, slot)
    assert got[0, 1] == 0.0 and got[1, 0] == 0.0


# ---------------------------------------------------------------- combine

def _dispatched(name):
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, wl.G)
    rx, _, _ = oracle.dispatch(inp.x, lay.token_slot, wl.R * S)
    return inp, lay, rx


@pytest.mark.parametrize("name", ["tiny", "decode128"])
def test_unit_weight_combine_is_x_times_k(name):
    inp, lay, rx = _dispatched(name)
    out = oracle.combine(rx, lay.token_slot, None)
    # K is a power of two: K*x is exact in bf16 (no overflow at these values).
    # The sum starts from +0, so a column of -0 inputs gives +0: compare values.
    xk = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).float() * inp.wl.K
    np.testing.assert_array_equal(oracle.bf16_to_double(out), xk.double().numpy())
    ones = np.ones_like(inp.topk_weights)
    np.testing.assert_array_equal(oracle.combine(rx, lay.token_slot, ones), out)


def test_one_hot_combine_returns_x():
    inp, lay, rx = _dispatched("tiny")
    w = np.zeros_like(inp.topk_weights)
    w[:, 0] = 1.0
    np.testing.assert_array_equal(oracle.combine(rx, lay.token_slot, w), inp.x)
    w = np.zeros_like(inp.topk_weights)
    w[:, -1] = 1.0
    np.testing.assert_array_equal(oracle.combine(rx, lay.token_slot, w), inp.x)


def test_renormalised_weights_return_x():
    inp, lay, rx = _dispatched("tiny")
    out = oracle.bf16_to_double(oracle.combine(rx, lay.token_slot, inp.topk_weights))
    x = oracle.bf16_to_double(inp.x)
    assert np.all(np.abs(out - x) <= 1e-3 + 1e-2 * np.abs(x))


@pytest.mark.parametrize("name", ["tiny", "decode128"])
def test_weighted_combine_matches_numpy_gather(name):
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S)
    y = ep_inputs.expert_outputs(wl.R * S, wl.H, seed=7)
    out = oracle.combine(y, lay.token_slot, inp.topk_weights)
    yf = torch.from_numpy(y.view(np.int16)).view(torch.bfloat16).double().numpy()
    ref = np.einsum("tk,tkh->th", inp.topk_weights.astype(np.float64), yf[lay.token_slot])
    ref_bf16 = torch.from_numpy(ref).float().to(torch.bfloat16).double().numpy()
    got = oracle.bf16_to_double(out)
    # within the combine tolerance, and equal to torch's rounding of the fp64
    # sum for all but double-rounding ties
    assert np.all(np.abs(got - ref) <= 1e-3 + 1e-2 * np.abs(ref))
    assert (got == ref_bf16).mean() > 0.9999


def test_combine_skips_empty_slots():
    y = np.zeros((4, 8), np.uint16)
    y[2] = 0x3F80  # 1.0
    slot = np.array([[2, -1], [-1, -1], [2, 9]], np.int32)
    out = oracle.bf16_to_double(oracle.combine(y, slot, np.array([[2, 5], [1, 1], [1, 7]], np.float32)))
    np.testing.assert_array_equal(out[:, 0], [2.0, 0.0, 1.0])


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_matches_torch_on_floats():
    rng = np.random.default_rng(5)
    with np.errstate(over="ignore"):
        big = (rng.standard_normal(50000) * 3e38).astype(np.float32)     # near overflow
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(50000) * 1e-39).astype(np.float32),   # subnormals
        big,
        rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.3961776e38], np.float32),
    ])
    f = f[np.isfinite(f) | np.isinf(f)]
    f = f[~np.isnan(f)]
    ours = oracle.double_to_bf16(f.astype(np.float64))
    theirs = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)


def test_bf16_rounding_is_nearest_even_for_doubles():
    # every finite non-negative bf16 value, ascending
    pos = np.arange(0, 0x7F80, dtype=np.uint16)
    vals = torch.from_numpy(pos.view(np.int16)).view(torch.bfloat16).double().numpy()
    rng = np.random.default_rng(9)
    d = np.abs(np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                               (vals[1:200] + vals[:199]) / 2]))  # exact midpoints
    got = oracle.double_to_bf16(d)
    i = np.clip(np.searchsorted(vals, d), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    pick_hi = (d - lo > hi - d) | ((d - lo == hi - d) & (pos[i] % 2 == 0))
    want = np.where(pick_hi, pos[i], pos[i - 1])
    np.testing.assert_array_equal(got, want)
