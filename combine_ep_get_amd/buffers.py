"""Allocation of the layout outputs and workspace with torch (plumbing)."""
from __future__ import annotations

from dataclasses import dataclass

import torch

from ._binding import Problem, ep_workspace_bytes


@dataclass
class LayoutBuffers:
    expert_count: torch.Tensor       # [E] int32
    expert_offset: torch.Tensor      # [E] int32
    rank_row_count: torch.Tensor     # [R] int32
    rank_token_count: torch.Tensor   # [R] int32
    group_token_count: torch.Tensor  # [G] int32
    is_token_in_rank: torch.Tensor   # [T,R] uint8
    token_slot: torch.Tensor         # [T,K] int32
    workspace: torch.Tensor          # uint8, 256-byte aligned (torch allocations are)
    cumulative_expert_recv: torch.Tensor | None = None  # [E] int64, or None

    def args(self):
        """Positional output arguments of ep_get_layout, in order."""
        return (self.expert_count, self.expert_offset, self.rank_row_count,
                self.rank_token_count, self.group_token_count, self.is_token_in_rank,
                self.token_slot, self.cumulative_expert_recv, self.workspace)


def alloc_layout(problem: Problem, device="cuda", cumulative: bool = False) -> LayoutBuffers:
    """Output buffers for ep_get_layout; `cumulative` adds a zeroed int64 [E]
    per-expert receive counter."""
    nbytes = ep_workspace_bytes(problem)
    if nbytes == 0:
        raise ValueError("invalid ep_problem")
    T, K, E = problem.num_tokens, problem.num_topk, problem.num_experts
    R, G = problem.num_ranks, problem.num_groups
    i32 = dict(dtype=torch.int32, device=device)
    return LayoutBuffers(
        expert_count=torch.empty(E, **i32),
        expert_offset=torch.empty(E, **i32),
        rank_row_count=torch.empty(R, **i32),
        rank_token_count=torch.empty(R, **i32),
        group_token_count=torch.empty(G, **i32),
        is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=device),
        token_slot=torch.empty((T, K), **i32),
        workspace=torch.empty(nbytes, dtype=torch.uint8, device=device),
        cumulative_expert_recv=torch.zeros(E, dtype=torch.int64, device=device) if cumulative else None,
    )
