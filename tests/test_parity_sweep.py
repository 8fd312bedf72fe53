"""A seeded sweep of random problems through the one-call layout and
dispatch against the CPU oracle: every layout output, slot, received row,
source index and weight bit for bit, rows no slot names left untouched; then
the combine of expert outputs in that layout, weighted and with unit
weights, within the combine tolerance.

The draws span the interface: R from 1 to 256 ranks, 1 to 64 experts per
rank, top-k 1 to 32, batches from one token to 20000 (one chunk, two to four,
up to 128 and beyond, so every layout form runs), groups, alignment 1, 2 and
4, empty entries, duplicate experts, bad ids, and slices sized to overflow."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from test_parity import bf16_dev, combine_close, dev, host_u16, tight_stride
from test_parity_fused import ep, run_fused  # noqa: F401  (ep is a fixture)

pytestmark = pytest.mark.gpu


def draw(seed, big):
    rng = np.random.default_rng(90000 + seed)
    R = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 96, 128, 256]))
    L = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    L = max(1, min(L, 2048 // R, 256))
    E = R * L
    K = int(rng.integers(1, min(E, 32) + 1))
    T = int(rng.integers(1500, 20001)) if big else int(np.exp(rng.uniform(0, np.log(20000))))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if R % g == 0]))
    A = int(rng.choice([1, 1, 1, 2, 4]))
    H = int(rng.choice([8, 16, 64, 256, 520, 1024, 2056]))
    while T * K * H > 30_000_000 and T > 1:
        T //= 2
    if rng.integers(0, 4) == 0:
        idx = rng.integers(0, E, size=(T, K)).astype(np.int32)  # duplicates allowed
    elif T * E <= 4_000_000:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    else:
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, K)) < 0.08] = -1
    if rng.random() < 0.15:
        idx[rng.integers(0, T, 2), rng.integers(0, K, 2)] = E + 3
    x = ep_inputs.bf16_normal(rng, (T, H))
    w = rng.standard_normal((T, K)).astype(np.float32)
    counts = np.bincount(idx[(idx >= 0) & (idx < E)], minlength=E)
    S = oracle.default_rank_stride(T, K, E, R, A)
    if R * S * H * 2 > (256 << 20):   # keep the receive buffer small
        aligned = (counts + A - 1) // A * A
        S = tight_stride(counts, E, R) if A == 1 else int(aligned.reshape(R, L).sum(1).max()) + 1
    if rng.random() < 0.1:
        S = max(1, S - int(rng.integers(1, 4)))  # may overflow: the status is compared too
    return idx, w, x, E, R, G, A, S


@pytest.mark.parametrize("seed,big", [(s, False) for s in range(60)] + [(1000 + s, True) for s in range(30)])
def test_random_problem(ep, seed, big):
    idx, w, x, E, R, G, A, S = draw(seed, big)
    ref, bufs = run_fused(ep, idx, w, x, E, R, G, A=A, S=S, cumulative=seed % 5 == 0)
    T, K = idx.shape
    H = x.shape[1]
    if T == 0:
        return
    rows = R * S
    ref_rx, _, _ = oracle.dispatch(x, ref.token_slot, rows, w)
    y = ep_inputs.permuted_rows(ref_rx, seed=seed)
    p = ep.Problem.make(T, H, E, K, R, G, A, S)
    d_y = bf16_dev(y)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    out_unit = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ep.ep_combine(p, d_y, bufs.token_slot, dev(w), out)
    ep.ep_combine(p, d_y, bufs.token_slot, None, out_unit)
    torch.cuda.synchronize()
    combine_close(host_u16(out), oracle.combine(y, ref.token_slot, w))
    combine_close(host_u16(out_unit), oracle.combine(y, ref.token_slot, None))
