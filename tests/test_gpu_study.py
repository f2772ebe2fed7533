"""Chained versus reference-based correction (KVCMAS Sec. 3.2, Eq. 4 vs Eq. 6; the measure of
Fig. 3(b)) run with the library's factorisation and apply, against the same study computed by
the fp64 oracle's exact truncated SVD on the same synthetic caches; and the claim the pages
make for it: with an exact first agent, the chained error stays below the reference-based one,
which grows along the workflow."""
import numpy as np
import pytest
import torch

from oracle import kvc_oracle as O
from rank_kv_cache_layer_amd import study
from rank_kv_cache_layer_amd import workload as W

pytestmark = pytest.mark.gpu


def _oracle_study(ref, agents, rank):
    rel = lambda x, y: float(np.linalg.norm(x - y) / np.linalg.norm(y))
    trunc = lambda d: np.stack([(lambda A, B, s: A @ B)(*O.truncated_svd(d[l], rank)) for l in range(d.shape[0])])
    chained, cur = [0.0], agents[0].copy()
    for k in range(1, len(agents)):
        cur = cur + trunc(agents[k] - agents[k - 1])
        chained.append(rel(cur, agents[k]))
    nonchained = [rel(ref + trunc(a - ref), a) for a in agents]
    return chained, nonchained


def test_chained_vs_reference_matches_oracle_and_the_claim():
    print("[study] chained vs non-chained, 2 layers x 256 x 256, rank 32, 4 agents", flush=True)
    ref, agents = W.chain_study_caches(n_layers=2, seq_len=256, d=256, device="cuda:0")
    got = study.chain_vs_reference(ref, agents, rank=32, oversample=16, power_iters=3)
    want_c, want_n = _oracle_study(ref.double().cpu().numpy(), [a.double().cpu().numpy() for a in agents], 32)
    for g, w in zip(got["chained"] + got["non_chained"], want_c + want_n):
        assert abs(g - w) <= 0.05 * w + 2e-4, (got, want_c, want_n)
    c, n = got["chained"], got["non_chained"]
    assert c[0] == 0.0
    assert all(c[k] < n[k] for k in range(1, 4)), (c, n)
    assert n[1] < n[2] < n[3], n
    assert max(c) < 0.01 and n[3] > 5 * max(c), (c, n)
