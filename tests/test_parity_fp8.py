"""FP8 quantisation and FP8 dispatch: HIP path vs the CPU oracle, bit for
bit (codes, scales, rows, scale placement in both layouts)."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle

pytestmark = pytest.mark.gpu


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



def gpu_quantize(ep, x_u16):
    T, H = x_u16.shape
    p = ep.Problem.make(T, H, 8, 1, 1, 1, 1, 1)
    q = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    sf = torch.empty((T, H // 128), dtype=torch.float32, device="cuda")
    ep.ep_quantize_fp8(p, dev(x_u16.view(np.int16)), q, sf)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "decode128", "prefill4k", "zipf8k"])
def test_quantize_parity(ep, name):
    inp = ep_inputs.make_inputs(name)
    q, sf = gpu_quantize(ep, inp.x)
    rq, rsf = oracle.quantize_fp8(inp.x)
    assert_same(sf, rsf)
    assert_same(q, rq)


def test_quantize_ties_subnormals_and_zero_blocks(ep):
    # block 0: amax 448 makes the scale exactly 1, so the values below land
    # on e4m3 rounding midpoints and in the subnormal range unchanged
    mags = oracle.e4m3_to_float(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([[448.0], mids[:63], -mids[63:126], [0.001, -0.0005]])[:128]
    row = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    x = np.zeros((3, 512), np.int16)
    x[0, :128] = row
    rng = np.random.default_rng(0)
    x[1] = ep_inputs.bf16_normal(rng, (512,)).view(np.int16) * 0  # all-zero row
    x[2] = ep_inputs.bf16_normal(rng, (512,)).view(np.int16)
    x = x.view(np.uint16)
    q, sf = gpu_quantize(ep, x)
    rq, rsf = oracle.quantize_fp8(x)
    assert_same(sf, rsf)
    assert_same(q, rq)


def test_quantize_every_bf16_value_at_unit_scale(ep):
    # every bf16 value with |v| <= 448, 127 to a block behind a leading 448
    # (which makes the block's scale exactly 1): the conversion is checked on
    # each input the format can hold
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    vals = vals[keep]
    nblk = -(-vals.size // 127)
    body = np.zeros(nblk * 127, np.float32)
    body[:vals.size] = vals
    blocks = np.zeros((nblk, 128), np.float32)
    blocks[:, 0] = 448.0
    blocks[:, 1:] = body.reshape(nblk, 127)
    nb_row = 16
    rows = -(-nblk // nb_row)
    x = np.zeros((rows * nb_row, 128), np.float32)
    x[:nblk] = blocks
    x = x.reshape(rows, nb_row * 128)
    x_u16 = (x.view(np.uint32) >> 16).astype(np.uint16)
    q, sf = gpu_quantize(ep, x_u16)
    rq, rsf = oracle.quantize_fp8(x_u16)
    assert_same(sf, rsf)
    assert_same(q, rq)


def test_quantize_nan_and_inf_inputs(ep):
    # not finite inputs: a NaN is skipped by the block maximum and encodes as
    # 0x7F; an infinity makes the scale infinite and every code of its block
    # zero except its own, which is NaN times zero
    rng = np.random.default_rng(5)
    x = ep_inputs.bf16_normal(rng, (4, 512)).view(np.uint16).copy()
    x[0, 3] = 0x7FC0          # NaN
    x[1, 130] = 0x7F80        # +inf
    x[2, 300] = 0xFF80        # -inf
    x[3, 511] = 0xFFC1        # NaN with payload and sign
    q, sf = gpu_quantize(ep, x)
    rq, rsf = oracle.quantize_fp8(x)
    assert_same(sf, rsf)
    assert_same(q, rq)


@pytest.mark.parametrize("name,column_major", [("tiny", False), ("decode128", True),
                                               ("prefill4k", False), ("prefill4k", True),
                                               ("zipf8k", True)])
def test_dispatch_fp8_parity(ep, name, column_major):
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    counts = np.bincount(inp.topk_idx.ravel(), minlength=wl.E)
    S = int((counts.reshape(wl.R, -1).sum(1)).max())
    rows = wl.R * S
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, wl.G)
    q, sf = oracle.quantize_fp8(inp.x)
    rq, rsf, (ts, hs), rsrc, rw = oracle.dispatch_fp8(q, sf, lay.token_slot, rows, inp.topk_weights,
                                                     column_major_sf=column_major)
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, 1, S)
    bufs = ep.alloc_layout(p)
    ep.ep_get_layout(p, dev(inp.topk_idx), *bufs.args())
    g_q = torch.empty((rows, wl.H), dtype=torch.uint8, device="cuda")
    g_sf = torch.full((rsf.size,), float("nan"), dtype=torch.float32, device="cuda")
    g_src = torch.empty(rows, dtype=torch.int32, device="cuda")
    g_w = torch.empty(rows, dtype=torch.float32, device="cuda")
    ep.ep_dispatch_fp8(p, dev(q), dev(sf), dev(inp.topk_weights), bufs.token_slot, g_q, g_sf, ts, hs,
                       g_src, g_w)
    torch.cuda.synchronize()
    assert_same(bufs.token_slot.cpu().numpy(), lay.token_slot)
    s = lay.token_slot.ravel()
    assert_same(g_q.cpu().numpy()[s], rq[s])
    nb = wl.H // 128
    got_sf = g_sf.cpu().numpy()
    idx = (s[:, None] * ts + np.arange(nb)[None, :] * hs).ravel()
    assert_same(got_sf[idx], rsf[idx])
    assert_same(g_src.cpu().numpy()[s], rsrc[s])
    assert_same(g_w.cpu().numpy()[s], rw[s])


@pytest.mark.parametrize("H,column_major", [(256, False), (256, True), (896, True)])
def test_dispatch_fp8_narrow_rows(ep, H, column_major):
    """FP8 rows under 1 KB with enough entries to take the packed dispatch (one
    thread per (entry, 16-byte vector), the scales placed by the first H/128
    vectors' threads), in both scale layouts; 896-byte rows are the widest."""
    print(f"[parity-fp8] narrow rows H={H} column_major={column_major}", flush=True)
    rng = np.random.default_rng(H + column_major)
    T, E, R, K = 3000, 64, 8, 6
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = -1
    w = rng.standard_normal((T, K)).astype(np.float32)
    x = ep_inputs.bf16_normal(rng, (T, H))
    counts = np.bincount(idx[idx >= 0].ravel(), minlength=E)
    S = int((counts.reshape(R, -1).sum(1)).max())
    rows = R * S
    lay = oracle.layout(idx, E, R, S, 1)
    q, sf = oracle.quantize_fp8(x)
    rq, rsf, (ts, hs), rsrc, rw = oracle.dispatch_fp8(q, sf, lay.token_slot, rows, w,
                                                     column_major_sf=column_major)
    p = ep.Problem.make(T, H, E, K, R, 1, 1, S)
    bufs = ep.alloc_layout(p)
    ep.ep_get_layout(p, dev(idx), *bufs.args())
    g_q = torch.empty((rows, H), dtype=torch.uint8, device="cuda")
    g_sf = torch.full((rsf.size,), float("nan"), dtype=torch.float32, device="cuda")
    g_src = torch.empty(rows, dtype=torch.int32, device="cuda")
    g_w = torch.empty(rows, dtype=torch.float32, device="cuda")
    ep.ep_dispatch_fp8(p, dev(q), dev(sf), dev(w), bufs.token_slot, g_q, g_sf, ts, hs, g_src, g_w)
    torch.cuda.synchronize()
    s = lay.token_slot.ravel()
    s = s[s >= 0]
    assert_same(g_q.cpu().numpy()[s], rq[s])
    nb = H // 128
    idx_sf = (s[:, None] * ts + np.arange(nb)[None, :] * hs).ravel()
    assert_same(g_sf.cpu().numpy()[idx_sf], rsf[idx_sf])
    assert_same(g_src.cpu().numpy()[s], rsrc[s])
    assert_same(g_w.cpu().numpy()[s], rw[s])


@pytest.mark.parametrize("name,column_major", [("tiny", False), ("decode128", True), ("decode128", False),
                                               ("prefill4k", True)])
def test_layout_dispatch_fp8_parity(ep, name, column_major):
    """The one-call FP8 layout and dispatch: one kernel for the one-chunk
    batches, the count pass and one kernel for prefill4k (32 chunks)."""
    inp = ep_inputs.make_inputs(name)
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    rows = wl.R * S
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, wl.G)
    q, sf = oracle.quantize_fp8(inp.x)
    rq, rsf, (ts, hs), rsrc, rw = oracle.dispatch_fp8(q, sf, lay.token_slot, rows, inp.topk_weights,
                                                     column_major_sf=column_major)
    p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, 1, S)
    bufs = ep.alloc_layout(p)
    g_q = torch.empty((rows, wl.H), dtype=torch.uint8, device="cuda")
    g_sf = torch.full((rsf.size,), float("nan"), dtype=torch.float32, device="cuda")
    g_src = torch.empty(rows, dtype=torch.int32, device="cuda")
    g_w = torch.empty(rows, dtype=torch.float32, device="cuda")
    ep.ep_layout_dispatch_fp8(p, dev(inp.topk_idx), *bufs.args(), None, dev(q), dev(sf),
                              dev(inp.topk_weights), g_q, g_sf, ts, hs, g_src, g_w)
    assert ep.ep_read_status(bufs.workspace) == ep.EP_OK
    for field in ("expert_count", "expert_offset", "rank_row_count", "rank_token_count",
                  "is_token_in_rank", "token_slot"):
        assert_same(getattr(bufs, field).cpu().numpy(), getattr(lay, field), field)
    s = lay.token_slot.ravel()
    assert_same(g_q.cpu().numpy()[s], rq[s])
    nb = wl.H // 128
    idx = (s[:, None] * ts + np.arange(nb)[None, :] * hs).ravel()
    assert_same(g_sf.cpu().numpy()[idx], rsf[idx])
    assert_same(g_src.cpu().numpy()[s], rsrc[s])
    assert_same(g_w.cpu().numpy()[s], rw[s])


def test_fp8_rejects_hidden_not_multiple_of_128(ep):
    p = ep.Problem.make(16, 200, 8, 2, 2, 1, 1, 64)
    with pytest.raises(ep.EpError):
        ep.ep_quantize_fp8(p, 1 << 20, 1 << 20, 1 << 20)


@pytest.mark.parametrize("T,K,column_major", [(300, 8, False), (500, 8, True), (2000, 3, False)])
def test_layout_dispatch_fp8_few_chunks(ep, T, K, column_major):
    """The one-call FP8 path on two to six chunks: the single kernel up to
    four chunks, the count pass and one kernel beyond."""
    rng = np.random.default_rng(T + K)
    E, R, H = 64, 8, 1024
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    x = ep_inputs.bf16_normal(rng, (T, H))
    w = rng.random((T, K)).astype(np.float32)
    S = oracle.default_rank_stride(T, K, E, R)
    rows = R * S
    lay = oracle.layout(idx, E, R, S, 1)
    q, sf = oracle.quantize_fp8(x)
    rq, rsf, (ts, hs), rsrc, rw = oracle.dispatch_fp8(q, sf, lay.token_slot, rows, w,
                                                     column_major_sf=column_major)
    p = ep.Problem.make(T, H, E, K, R, 1, 1, S)
    bufs = ep.alloc_layout(p)
    g_q = torch.empty((rows, H), dtype=torch.uint8, device="cuda")
    g_sf = torch.full((rsf.size,), float("nan"), dtype=torch.float32, device="cuda")
    g_src = torch.empty(rows, dtype=torch.int32, device="cuda")
    g_w = torch.empty(rows, dtype=torch.float32, device="cuda")
    ep.ep_layout_dispatch_fp8(p, dev(idx), *bufs.args(), None, dev(q), dev(sf), dev(w), g_q, g_sf, ts, hs,
                              g_src, g_w)
    assert ep.ep_read_status(bufs.workspace) == ep.EP_OK
    assert_same(bufs.token_slot.cpu().numpy(), lay.token_slot, "token_slot")
    assert_same(bufs.is_token_in_rank.cpu().numpy(), lay.is_token_in_rank, "is_token_in_rank")
    s = lay.token_slot.ravel()
    assert_same(g_q.cpu().numpy()[s], rq[s])
    nb = H // 128
    sel = (s[:, None] * ts + np.arange(nb)[None, :] * hs).ravel()
    assert_same(g_sf.cpu().numpy()[sel], rsf[sel])
    assert_same(g_src.cpu().numpy()[s], rsrc[s])
    assert_same(g_w.cpu().numpy()[s], rw[s])


def _padded_case(kind):
    """Routing for the padded-scale-row cases: (idx, w, x, E, R, S)."""
    rng = np.random.default_rng(len(kind))
    if kind == "last_row":
        # two ranks of two experts, one entry on each rank per token: both
        # slices fill to exactly S = T rows, so row R*S-1 is written
        T, E, R, H = 300, 4, 2, 1024
        idx = np.stack([rng.integers(0, 2, T), rng.integers(2, 4, T)], axis=1).astype(np.int32)
        S = T
    else:
        T, K, H = {"two_call": (600, 8, 7168), "single_kernel": (128, 8, 7168),
                   "chunks": (2000, 8, 7168), "narrow": (3000, 6, 512)}[kind]
        E, R = 64, 8
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
        idx[rng.random(idx.shape) < 0.03] = -1
        counts = np.bincount(idx[idx >= 0].ravel(), minlength=E)
        S = int(counts.reshape(R, -1).sum(1).max()) + 5
    w = rng.standard_normal(idx.shape).astype(np.float32)
    x = ep_inputs.bf16_normal(rng, (idx.shape[0], H))
    return idx, w, x, E, R, S


@pytest.mark.parametrize("kind", ["two_call", "single_kernel", "chunks", "narrow", "last_row"])
def test_dispatch_fp8_scale_rows_padded_to_lines(ep, kind):
    """Token-major scale rows padded to whole 128-byte lines (token stride
    H/128 rounded up to 32 floats): the scales bit for bit at the packed
    layout's values, the padding of every written row 0 except on the last
    row of the buffer, and nothing written outside the written rows or past
    the buffer's required size."""
    print(f"[parity-fp8] padded scale rows {kind}", flush=True)
    idx, w, x, E, R, S = _padded_case(kind)
    T, K = idx.shape
    H = x.shape[1]
    nb = H // 128
    pad = -(-nb // 32) * 32
    assert pad > nb
    rows = R * S
    lay = oracle.layout(idx, E, R, S, 1)
    q, sf = oracle.quantize_fp8(x)
    rq, rsf, (ts, hs), rsrc, rw = oracle.dispatch_fp8(q, sf, lay.token_slot, rows, w)
    assert (ts, hs) == (nb, 1)
    p = ep.Problem.make(T, H, E, K, R, 1, 1, S)
    bufs = ep.alloc_layout(p)
    need = (rows - 1) * pad + nb   # the size the interface requires
    g_q = torch.empty((rows, H), dtype=torch.uint8, device="cuda")
    g_sf = torch.full((rows * pad + 64,), float("nan"), dtype=torch.float32, device="cuda")
    g_src = torch.empty(rows, dtype=torch.int32, device="cuda")
    g_w = torch.empty(rows, dtype=torch.float32, device="cuda")
    if kind in ("two_call", "narrow"):   # 512-byte rows take the narrow-row dispatch
        ep.ep_get_layout(p, dev(idx), *bufs.args())
        ep.ep_dispatch_fp8(p, dev(q), dev(sf), dev(w), bufs.token_slot, g_q, g_sf, pad, 1, g_src, g_w)
    else:
        ep.ep_layout_dispatch_fp8(p, dev(idx), *bufs.args(), None, dev(q), dev(sf), dev(w), g_q, g_sf,
                                  pad, 1, g_src, g_w)
    assert ep.ep_read_status(bufs.workspace) == ep.EP_OK
    assert_same(bufs.token_slot.cpu().numpy(), lay.token_slot, "token_slot")
    s = lay.token_slot.ravel()
    s = np.sort(s[s >= 0])
    assert_same(g_q.cpu().numpy()[s], rq[s])
    assert_same(g_src.cpu().numpy()[s], rsrc[s])
    assert_same(g_w.cpu().numpy()[s], rw[s])
    got = g_sf.cpu().numpy()
    grid = got[:rows * pad].reshape(rows, pad)
    assert_same(grid[s, :nb], rsf.reshape(rows, nb)[s])
    inner = s[s != rows - 1]
    assert np.all(grid[inner, nb:].view(np.uint32) == 0), "padding of written rows"
    unwritten = np.setdiff1d(np.arange(rows), s)
    assert np.all(np.isnan(grid[unwritten])), "rows no slot names"
    assert np.all(np.isnan(got[need:])), "past the required size"
    if kind == "last_row":
        assert s[-1] == rows - 1
        assert np.all(np.isnan(grid[rows - 1, nb:]))
