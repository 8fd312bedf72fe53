"""A seeded sweep of random problems through the two-level path against the
CPU oracle: group slots, group rows, received rows, their metadata and the
bf16 partials bit for bit, the combine within tolerance.  The draws span 2 to
1024 groups (the few-group and the ballot-walk forms), 1 to 64 ranks per
group, top-k 1 to 16, batches of 1 to 12000 tokens, empty entries, and group
slices sized to overflow."""
import numpy as np
import pytest

import ep_inputs
from test_parity_hier import ep, run  # noqa: F401  (ep is a fixture)

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(70000 + seed)
    G = int(rng.choice([2, 3, 4, 8, 16, 64, 256, 1024]))
    rpg = int(rng.choice([1, 2, 4, 8]))
    while G * rpg > 1024:
        rpg //= 2
    R = G * rpg
    L = int(rng.choice([1, 2, 4, 8]))
    L = max(1, min(L, 2048 // R))
    E = R * L
    K = int(rng.integers(1, min(E, 16) + 1))
    T = int(np.exp(rng.uniform(0, np.log(12000))))
    H = int(rng.choice([8, 64, 256, 1032]))
    while T * K * H > 8_000_000 and T > 1:
        T //= 2
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32) if T * E <= 4_000_000 else \
        np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, K)) < 0.05] = -1
    w = rng.standard_normal((T, K)).astype(np.float32)
    x = ep_inputs.bf16_normal(rng, (T, H))
    counts = np.bincount(idx[idx >= 0], minlength=E)
    S = int(max(1, counts.reshape(R, L).sum(1).max()))
    SG = T if rng.random() < 0.85 else max(1, int(T * rng.uniform(0.3, 0.9)))  # may overflow a group
    return idx, w, x, E, R, G, S, SG


@pytest.mark.parametrize("seed", range(40))
def test_random_two_level_problem(ep, seed):
    idx, w, x, E, R, G, S, SG = draw(seed)
    print(f"[hier-sweep] seed={seed} T={idx.shape[0]} K={idx.shape[1]} E={E} R={R} G={G} S={S} SG={SG} "
          f"H={x.shape[1]}", flush=True)
    run(ep, idx, w, x, E, R, G, S, SG)
