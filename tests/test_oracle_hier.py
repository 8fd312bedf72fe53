"""Pins for the oracle's hierarchical (two-level) path.

- group slots against a numpy restatement (cumulative sum of the per-group
  token flags) and against the layout's group_token_count;
- two-level dispatch must leave exactly the rows the flat dispatch leaves;
- one-hot weights through the two-level combine return x exactly;
- weighted two-level combine stays within the bound set by rounding each
  group partial to bf16, against the flat fp64 combine;
- a hand-worked fixture (tests/golden/combine_hier_handworked.json) fixes
  the bits of the partials and of the output: the fp32 fold, its top-k
  order, the bf16 rounding of each partial and the exact sum over groups.
"""
import json
import os

import numpy as np
import pytest
import torch

import ep_inputs
import oracle


def _setup(name, seed=None, with_x=True):
    inp = ep_inputs.make_inputs(name, seed=seed, with_x=with_x)
    wl = inp.wl
    counts = np.bincount(inp.topk_idx.ravel(), minlength=wl.E)
    S = int(counts.reshape(wl.R, -1).sum(1).max())
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, wl.G)
    return inp, wl, S, lay


def restated_group_slots(is_token_in_rank, G, SG):
    T, R = is_token_in_rank.shape
    rpg = R // G
    out = np.full((T, G), -1, np.int64)
    for g in range(G):
        flags = is_token_in_rank[:, g * rpg:(g + 1) * rpg].any(1)
        pos = np.cumsum(flags) - 1
        ok = flags & (pos < SG)
        out[ok, g] = g * SG + pos[ok]
    return out


@pytest.mark.parametrize("name,G", [("large16k", 2), ("prefill4k", 2), ("prefill4k", 4), ("zipf8k", 8), ("tiny", 1)])
def test_group_slots(name, G):
    inp, wl, S, lay = _setup(name, with_x=False)
    T = wl.T
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, G)
    gs = oracle.group_layout(lay.is_token_in_rank, G, T)
    np.testing.assert_array_equal(gs, restated_group_slots(lay.is_token_in_rank, G, T))
    np.testing.assert_array_equal((gs >= 0).sum(0), lay.group_token_count)
    assert oracle.group_layout(lay.is_token_in_rank, G, T, with_status=True)[1] == oracle.OK
    # capacity: a smaller group slice drops the later tokens and reports it;
    # exactly the fullest group's count does not
    SG = int(lay.group_token_count.min()) - 1
    gs2, st = oracle.group_layout(lay.is_token_in_rank, G, SG, with_status=True)
    np.testing.assert_array_equal(gs2, restated_group_slots(lay.is_token_in_rank, G, SG))
    assert st == oracle.CAPACITY
    full = int(lay.group_token_count.max())
    assert oracle.group_layout(lay.is_token_in_rank, G, full, with_status=True)[1] == oracle.OK
    assert oracle.group_layout(lay.is_token_in_rank, G, full - 1, with_status=True)[1] == oracle.CAPACITY


@pytest.mark.parametrize("name", ["tiny", "prefill4k"])
def test_two_level_dispatch_equals_flat(name):
    inp, wl, S, lay = _setup(name)
    G = max(wl.G, 2) if wl.R % 2 == 0 else 1
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, G)
    gs = oracle.group_layout(lay.is_token_in_rank, G, wl.T)
    gbuf, rx = oracle.dispatch_hier(inp.x, gs, lay.token_slot, wl.R, S, wl.T)
    flat, _, _ = oracle.dispatch(inp.x, lay.token_slot, wl.R * S)
    assert np.array_equal(rx, flat)
    # every group row holds its token's row
    t_idx, g_idx = np.nonzero(gs >= 0)
    assert np.array_equal(gbuf[gs[t_idx, g_idx]], inp.x[t_idx])


def test_two_level_dispatch_marks_dropped_entries():
    """With a group capacity below the fullest group, every entry keeps its
    flat row and metadata exactly when its token kept a row in the entry's
    group; the others get source -1, weight 0 and no row."""
    inp, wl, S, lay = _setup("prefill4k")
    G = 4
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, G)
    SG = int(lay.group_token_count.min()) - 50
    gs = oracle.group_layout(lay.is_token_in_rank, G, SG)
    _, rx, src, rw = oracle.dispatch_hier(inp.x, gs, lay.token_slot, wl.R, S, SG,
                                          topk_weights=inp.topk_weights, with_meta=True)
    flat, fsrc, frw = oracle.dispatch(inp.x, lay.token_slot, wl.R * S, inp.topk_weights)
    T, K = lay.token_slot.shape
    t_of = np.repeat(np.arange(T), K).reshape(T, K)
    slot = lay.token_slot
    grp = (slot // S) // (wl.R // G)
    kept = gs[t_of, grp] >= 0
    assert 0 < (~kept).sum() < kept.sum()
    s_kept, s_drop = slot[kept], slot[~kept]
    assert np.array_equal(rx[s_kept], flat[s_kept])
    assert np.array_equal(src[s_kept], fsrc[s_kept]) and np.array_equal(rw[s_kept], frw[s_kept])
    assert np.all(src[s_drop] == -1) and np.all(rw[s_drop] == 0)
    assert not np.any(rx[s_drop])


def test_two_level_combine_one_hot_returns_x():
    inp, wl, S, lay = _setup("tiny")
    G = 2
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, G)
    gs = oracle.group_layout(lay.is_token_in_rank, G, wl.T)
    _, rx = oracle.dispatch_hier(inp.x, gs, lay.token_slot, wl.R, S, wl.T)
    w = np.zeros_like(inp.topk_weights)
    w[:, 0] = 1.0
    _, out = oracle.combine_hier(rx, lay.token_slot, w, gs, wl.R, S, wl.T)
    np.testing.assert_array_equal(oracle.bf16_to_double(out), oracle.bf16_to_double(inp.x))


@pytest.mark.parametrize("name,G", [("tiny", 1), ("tiny", 2), ("decode128", 2), ("decode128", 8)])
def test_two_level_combine_within_partial_rounding_bound(name, G):
    inp, wl, S, lay = _setup(name)
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, G)
    gs = oracle.group_layout(lay.is_token_in_rank, G, wl.T)
    y = ep_inputs.expert_outputs(wl.R * S, wl.H, seed=4)
    gbuf, out = oracle.combine_hier(y, lay.token_slot, inp.topk_weights, gs, wl.R, S, wl.T)
    flat = oracle.bf16_to_double(oracle.combine(y, lay.token_slot, inp.topk_weights))
    got = oracle.bf16_to_double(out)
    part = np.zeros_like(flat)
    for g in range(G):
        ok = gs[:, g] >= 0
        part[ok] += np.abs(oracle.bf16_to_double(gbuf[gs[ok, g]]))
    # rounding a value to bf16 moves it by at most half an ulp, 2^-8 of its
    # magnitude: once per partial, once for each of the two final results
    # (fp32 folding error is far smaller)
    bound = 2.0 ** -8 * (part + np.abs(flat) + np.abs(got)) + 1e-30
    assert np.all(np.abs(got - flat) <= bound)
    # with one group the output is the token's single group row: a bf16
    # value rounded again to bf16 is unchanged
    if G == 1:
        t = np.nonzero(gs[:, 0] >= 0)[0]
        np.testing.assert_array_equal(out[t], gbuf[gs[t, 0]])


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "combine_hier_handworked.json")


def _golden_case(c):
    """Arrays of one hand-worked case: y filled with y_other except the
    named rows."""
    R, S, H = c["R"], c["S"], c["H"]
    y = np.full((R * S, H), int(c["y_other"], 16), np.uint16)
    for row, vals in c["y"].items():
        y[int(row)] = [int(v, 16) for v in vals]
    slot = np.array(c["token_slot"], np.int32)
    gsl = np.array(c["group_slot"], np.int32)
    w = np.array([[float.fromhex(v) for v in r] for r in c["weights"]], np.float32)
    return y, slot, gsl, w


@pytest.mark.parametrize("case", [c["name"] for c in json.load(open(GOLDEN))["cases"]])
def test_golden_handworked_two_level_combine(case):
    c = next(c for c in json.load(open(GOLDEN))["cases"] if c["name"] == case)
    y, slot, gsl, w = _golden_case(c)
    gbuf, out = oracle.combine_hier(y, slot, w, gsl, c["R"], c["S"], c["SG"])
    for row, vals in c["group_rows"].items():
        assert [int(v) for v in gbuf[int(row)]] == [int(v, 16) for v in vals], (case, "group row", row)
    assert out.tolist() == [[int(v, 16) for v in r] for r in c["out"]], (case, "out")
