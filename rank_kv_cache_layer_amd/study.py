"""Chained versus reference-based correction along an agent workflow (KVCMAS Sec. 3.2, Eq. 4
vs Eq. 6, the measure of Fig. 3(b)), run with the library's own factorisation and apply calls.

Given exact caches of one side of a segment, C_ref (context-free reference) and C_0 .. C_{n-1}
of the agents in execution order:
  * chained (Eq. 6): the first agent's cache is exact (dense prefill); agent k's is the
    materialised cache of agent k-1 plus the rank-r factorisation of the observed correction
    C_k - C_{k-1}, applied with weight 1 (kvc_anchor_refresh_svd, kvc_apply_lowrank_delta);
  * non-chained (Eq. 4): every agent's cache is C_ref plus the rank-r factorisation of
    C_k - C_ref, the first agent included.
Returns each agent's error ||C_hat_k - C_k||_F / ||C_k||_F for both (no alignment: positions
are equal, the study isolates the choice of reference)."""
from __future__ import annotations

from typing import Dict, List

import torch

from . import kvc


def _factor(delta: torch.Tensor, rank: int, oversample: int, power_iters: int, seed: int):
    a, b, _ = kvc.anchor_refresh_svd(delta.contiguous(), rank, out_dtype=torch.float32, oversample=oversample,
                                     power_iters=power_iters, seed=seed)
    return a, b


def _apply(src: torch.Tensor, a: torch.Tensor, b: torch.Tensor, rank: int) -> torch.Tensor:
    L, S, D = src.shape
    hd = 128 if D % 128 == 0 else D
    shp = kvc.shape_of(L, S, D // hd, hd)
    bb = b[:, None].contiguous()
    pool = kvc.PoolTensors([S], rank, rank, a, bb, a, bb, a, bb, a, bb)
    w = torch.ones((L, S, 1), dtype=torch.float32, device=src.device)
    out_k, out_v = torch.empty_like(src), torch.empty_like(src)
    kvc.apply_lowrank_delta(src, src, out_k, out_v, shp, 0, 0, pool, w, w, S)
    return out_v   # values: no rotation at all (the key output equals it at zero positions)


def chain_vs_reference(ref: torch.Tensor, agents: List[torch.Tensor], rank: int, oversample: int = 16,
                       power_iters: int = 2, seed: int = 0) -> Dict[str, List[float]]:
    rel = lambda x, y: float(torch.linalg.vector_norm((x - y).double()) / torch.linalg.vector_norm(y.double()))
    chained, nonchained = [0.0], []
    cur = agents[0].clone()
    for k in range(1, len(agents)):
        a, b = _factor(agents[k] - agents[k - 1], rank, oversample, power_iters, seed + k)
        cur = _apply(cur, a, b, rank)
        chained.append(rel(cur, agents[k]))
    for k in range(len(agents)):
        a, b = _factor(agents[k] - ref, rank, oversample, power_iters, seed + 100 + k)
        nonchained.append(rel(_apply(ref, a, b, rank), agents[k]))
    torch.cuda.synchronize()
    return {"chained": chained, "non_chained": nonchained}
