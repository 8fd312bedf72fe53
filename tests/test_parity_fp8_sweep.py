"""A seeded sweep of random problems through the FP8 dispatch against the CPU
oracle: quantised codes, received rows, scales at their strides, source
indices and weights bit for bit; the padding of line-padded scale rows 0
except on the buffer's last row.  The draws span all three scale layouts
(token-major, token-major padded to 128-byte lines, column-major), the
two-call and the one-call forms, hidden sizes of 128 to 7168 and batches of
1 to 6000 tokens."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from test_parity_fp8 import dev, ep  # noqa: F401  (ep is a fixture)

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(50000 + seed)
    R = int(rng.choice([1, 2, 4, 8, 16, 64]))
    L = int(rng.choice([1, 2, 4, 16, 32]))
    L = max(1, min(L, 2048 // R))
    E = R * L
    K = int(rng.integers(1, min(E, 12) + 1))
    T = int(np.exp(rng.uniform(0, np.log(6000))))
    H = 128 * int(rng.choice([1, 2, 3, 7, 16, 56]))
    while T * K * H > 20_000_000 and T > 1:
        T //= 2
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32) if T * E <= 4_000_000 else \
        np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, K)) < 0.05] = -1
    w = rng.standard_normal((T, K)).astype(np.float32)
    x = ep_inputs.bf16_normal(rng, (T, H))
    layout = ["token", "padded", "column"][int(rng.integers(0, 3))]
    one_call = bool(rng.integers(0, 2))
    return idx, w, x, E, R, layout, one_call


@pytest.mark.parametrize("seed", range(40))
def test_random_fp8_problem(ep, seed):
    idx, w, x, E, R, layout, one_call = draw(seed)
    T, K = idx.shape
    H = x.shape[1]
    nb = H // 128
    print(f"[fp8-sweep] seed={seed} T={T} K={K} E={E} R={R} H={H} {layout} one_call={one_call}", flush=True)
    counts = np.bincount(idx[idx >= 0], minlength=E)
    S = int(max(1, counts.reshape(R, -1).sum(1).max()))
    rows = R * S
    lay = oracle.layout(idx, E, R, S, 1)
    q, sf = oracle.quantize_fp8(x)
    rq, rsf, (ts, hs), rsrc, rw = oracle.dispatch_fp8(q, sf, lay.token_slot, rows, w,
                                                     column_major_sf=layout == "column")
    if layout == "padded":
        gts, ghs = -(-nb // 32) * 32, 1
        size = rows * gts
    else:
        gts, ghs = ts, hs
        size = rsf.size
    p = ep.Problem.make(T, H, E, K, R, 1, 1, S)
    bufs = ep.alloc_layout(p)
    g_q = torch.empty((rows, H), dtype=torch.uint8, device="cuda")
    g_sf = torch.full((size,), float("nan"), dtype=torch.float32, device="cuda")
    g_src = torch.empty(rows, dtype=torch.int32, device="cuda")
    g_w = torch.empty(rows, dtype=torch.float32, device="cuda")
    # the quantiser on the GPU: its codes and scales must be the oracle's
    d_q = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    d_sf = torch.empty((T, nb), dtype=torch.float32, device="cuda")
    ep.ep_quantize_fp8(p, dev(x.view(np.int16)), d_q, d_sf)
    torch.cuda.synchronize()
    assert np.array_equal(d_q.cpu().numpy(), q)
    assert np.array_equal(d_sf.cpu().numpy().view(np.uint32), sf.view(np.uint32))
    if one_call:
        ep.ep_layout_dispatch_fp8(p, dev(idx), *bufs.args(), None, d_q, d_sf, dev(w), g_q, g_sf, gts, ghs,
                                  g_src, g_w)
    else:
        ep.ep_get_layout(p, dev(idx), *bufs.args())
        ep.ep_dispatch_fp8(p, d_q, d_sf, dev(w), bufs.token_slot, g_q, g_sf, gts, ghs, g_src, g_w)
    assert ep.ep_read_status(bufs.workspace) == ep.EP_OK
    assert np.array_equal(bufs.token_slot.cpu().numpy(), lay.token_slot)
    s = lay.token_slot.ravel()
    s = np.sort(s[s >= 0])
    assert np.array_equal(g_q.cpu().numpy()[s], rq[s])
    assert np.array_equal(g_src.cpu().numpy()[s], rsrc[s])
    assert np.array_equal(g_w.cpu().numpy()[s].view(np.uint32), rw[s].view(np.uint32))
    got = g_sf.cpu().numpy()
    want = rsf[(s[:, None] * ts + np.arange(nb)[None, :] * hs).ravel()]
    have = got[(s[:, None] * gts + np.arange(nb)[None, :] * ghs).ravel()]
    assert np.array_equal(have.view(np.uint32), want.view(np.uint32))
    if layout == "padded":
        inner = s[s != rows - 1]
        pad = got[:rows * gts].reshape(rows, gts)[inner, nb:]
        assert np.all(pad.view(np.uint32) == 0)
