"""Seeded synthetic inputs for MoE token dispatch / combine.

This module only draws random numbers and shapes them into the router output
and activations that the dispatch/combine path consumes.  It holds none of the
method's arithmetic (no counts, offsets, slots, copies or reductions), so both
the CPU oracle's tests and the HIP path's tests/bench can use it without
sharing any of the computation under test.

Workloads (named by what they are):

- ``tiny``:      T=128,   H=256,  E=16,  k=4, R=4,  uniform distinct experts
- ``prefill4k``: T=4096,  H=7168, E=256, k=8, R=8,  top-8 of N(0,1) logits
- ``decode128``: T=128,   H=7168, E=256, k=8, R=8,  top-8 of N(0,1) logits
- ``zipf8k``:    T=8192,  H=4096, E=128, k=8, R=8,  Zipf(1.2) expert popularity
- ``large16k``:  T=16384, H=7168, E=256, k=8, R=16 (2 groups of 8)

The decode shape is the one the usage example of "DeepEP Symmetric Memory
architecture analysis" (section 9.2) constructs its buffer for: 128 tokens per
rank, hidden 7168, top-8 of 256 experts.

Draws use numpy's PCG64 ``default_rng(seed)``.  Activations are fp32 N(0,1)
rounded to bf16 (round-to-nearest-even, done by torch's dtype conversion) and
returned as raw uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens on this (source) rank
    H: int          # hidden size, bf16 elements per row
    E: int          # experts (global)
    K: int          # top-k
    R: int          # destination ranks, simulated as slices of one buffer
    G: int = 1      # scale-out groups (R % G == 0)
    routing: str = "gauss_topk"   # "uniform", "gauss_topk" or "zipf"
    zipf_s: float = 0.0
    seed: int = 0
    A: int = 1      # expert_alignment


WORKLOADS = {
    "tiny": Workload("tiny", T=128, H=256, E=16, K=4, R=4, routing="uniform"),
    "prefill4k": Workload("prefill4k", T=4096, H=7168, E=256, K=8, R=8),
    "decode128": Workload("decode128", T=128, H=7168, E=256, K=8, R=8),
    "zipf8k": Workload("zipf8k", T=8192, H=4096, E=128, K=8, R=8,
                       routing="zipf", zipf_s=1.2),
    "large16k": Workload("large16k", T=16384, H=7168, E=256, K=8, R=16, G=2),
}


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    """Router weights: softmax over the chosen logits (fp64 then fp32)."""
    z = z.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return (ez / ez.sum(axis=1, keepdims=True)).astype(np.float32)


def route(T: int, E: int, K: int, routing: str, rng: np.random.Generator,
          zipf_s: float = 0.0):
    """Draw top-k expert ids ``[T,K]`` int32 and weights ``[T,K]`` fp32.

    ``uniform``: each token picks K distinct experts uniformly at random, in
    random order; weights are a softmax of K fresh N(0,1) logits.

    ``gauss_topk``: router logits ``[T,E] ~ N(0,1)``; ids are the K largest in
    descending order; the softmax over all E renormalised over the chosen K
    equals the softmax of the K chosen logits, which is what is returned.

    ``zipf``: expert e has popularity proportional to ``(e+1)^-s``; each
    token draws K distinct experts by successive sampling without replacement
    (implemented as Gumbel-top-K on log-popularity, which has the same law);
    weights are a softmax of K fresh N(0,1) logits.
    """
    if routing == "uniform":
        keys = rng.random((T, E))
        idx = np.argsort(keys, axis=1, kind="stable")[:, :K]
        w = _softmax_rows(rng.standard_normal((T, K)))
    elif routing == "gauss_topk":
        logits = rng.standard_normal((T, E)).astype(np.float32)
        # descending order; stable sort on -logits breaks (measure-zero) ties
        # toward the lower expert id
        idx = np.argsort(-logits, axis=1, kind="stable")[:, :K]
        w = _softmax_rows(np.take_along_axis(logits, idx, axis=1))
    elif routing == "zipf":
        logp = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        g = rng.gumbel(size=(T, E))
        idx = np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :K]
        w = _softmax_rows(rng.standard_normal((T, K)))
    else:
        raise ValueError(f"unknown routing {routing!r}")
    return np.ascontiguousarray(idx, dtype=np.int32), np.ascontiguousarray(w, dtype=np.float32)


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) fp32 rounded to bf16 (RNE), as uint16 bit patterns."""
    import torch

    f = rng.standard_normal(shape, dtype=np.float32)
    b = torch.from_numpy(f).to(torch.bfloat16)
    return b.view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class Inputs:
    wl: Workload
    topk_idx: np.ndarray      # [T,K] int32
    topk_weights: np.ndarray  # [T,K] fp32
    x: np.ndarray             # [T,H] uint16 (bf16 bits)
    extra: dict = field(default_factory=dict)


def make_inputs(wl: Workload | str, *, with_x: bool = True, seed: int | None = None) -> Inputs:
    """Router output and token activations for one workload, fully seeded.

    The stream is: routing draws first, then x.  ``seed`` overrides the
    workload's seed.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    idx, w = route(wl.T, wl.E, wl.K, wl.routing, rng, wl.zipf_s)
    x = bf16_normal(rng, (wl.T, wl.H)) if with_x else np.zeros((0, wl.H), np.uint16)
    return Inputs(wl, idx, w, x)


def expert_outputs(rows: int, H: int, seed: int) -> np.ndarray:
    """Stand-in for expert outputs: ``[rows,H]`` bf16 N(0,1) bits (uint16)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xE0]))
    return bf16_normal(rng, (rows, H))


def permuted_rows(rows: np.ndarray, seed: int) -> np.ndarray:
    """A seeded row permutation of ``rows`` (stand-in expert outputs that mix
    different tokens' activations without drawing new normals)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x9E]))
    return rows[rng.permutation(rows.shape[0])]


def random_small_case(rng: np.random.Generator, *, max_T=64, max_E=16, max_K=6,
                      allow_empty=True, allow_duplicates=False):
    """A random tiny routing problem for brute-force checks.

    Returns ``(idx[T,K] int32, E, R, G, K)``; R divides E and G divides R.
    ``allow_empty`` puts some -1 (empty slot) entries in; ``allow_duplicates``
    lets a token name the same expert twice.
    """
    E = int(rng.integers(1, max_E + 1))
    divs = [r for r in range(1, E + 1) if E % r == 0]
    R = int(rng.choice(divs))
    gdivs = [g for g in range(1, R + 1) if R % g == 0]
    G = int(rng.choice(gdivs))
    K = int(rng.integers(1, min(max_K, E) + 1))
    T = int(rng.integers(0, max_T + 1))
    if allow_duplicates:
        idx = rng.integers(0, E, size=(T, K))
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]) if T else np.zeros((0, K), int)
    idx = idx.astype(np.int32)
    if allow_empty and T:
        mask = rng.random((T, K)) < 0.15
        idx[mask] = -1
    return np.ascontiguousarray(idx), E, R, G, K
