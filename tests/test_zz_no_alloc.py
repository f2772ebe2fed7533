"""kvc_correct_hop_noalloc (library-owned per-GPU scratch, no workspace) against kvc_correct_hop on
the same inputs: identical outputs, gate rows and weights, on two calls in a row (the second
smaller, reusing the scratch the first left behind)."""
import numpy as np
import pytest
import torch

from rank_kv_cache_layer_amd import kvc
from rank_kv_cache_layer_amd import workload as W

from hop_helpers import DEV, make, params, shape

pytestmark = pytest.mark.gpu


def _both(spec):
    data = make(spec)
    k, v = data.k_src.to(DEV), data.v_src.to(DEV)
    pool = kvc.pool_from(data, DEV)
    prm = params(spec)
    res = []
    for noalloc in (False, True):
        ko, vo = torch.empty_like(k), torch.empty_like(v)
        out = kvc.alloc_match(spec.n_layers, spec.seq_len, spec.n_anchors, DEV)
        if noalloc:
            kvc.correct_hop_noalloc(k, v, ko, vo, shape(spec), spec.p_src, spec.p_tgt, pool, prm, out)
        else:
            kvc.correct_hop(k, v, ko, vo, shape(spec), spec.p_src, spec.p_tgt, pool, prm, out=out)
        torch.cuda.synchronize()
        res.append((ko, vo, out))
    (k1, v1, o1), (k2, v2, o2) = res
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(o1.flags, o2.flags) and o1.s_cov == o2.s_cov
    assert np.array_equal(o1.dist.cpu().numpy(), o2.dist.cpu().numpy(), equal_nan=True)
    assert np.array_equal(o1.stat.cpu().numpy(), o2.stat.cpu().numpy(), equal_nan=True)
    assert torch.equal(o1.w_k, o2.w_k) and torch.equal(o1.w_v, o2.w_v)


@pytest.mark.parametrize("mode", [W.SCORE_PAGES, W.SCORE_COS_R])
def test_noalloc_matches_correct_hop_two_calls(mode):
    tau = 0.3 if mode == W.SCORE_PAGES else 0.5
    big = W.llama8b_hop(n_layers=4, seq_len=1000, mode=mode, tau=tau)
    small = W.llama8b_hop(n_layers=2, seq_len=300, n_kv_heads=2, n_anchors=6, mode=mode, tau=tau,
                          anchor_len=[300, 250, 300, 180, 300, 290], gate_len=180)
    print(f"[noalloc] mode={mode} call 1: L={big.n_layers} S={big.seq_len} N={big.n_anchors}", flush=True)
    _both(big)
    print(f"[noalloc] mode={mode} call 2: L={small.n_layers} S={small.seq_len} N={small.n_anchors}", flush=True)
    _both(small)


def test_noalloc_sliced_ranks_two_calls():
    # base and delta ranks 128, then 64: the scoring in 64-rank steps and the apply in rank
    # slices, through the library-owned scratch, equal to the workspace entry point
    big = W.llama8b_hop(n_layers=2, seq_len=600, n_kv_heads=4, n_anchors=6, rank_base=128, rank_delta=128,
                        anchor_len=[600, 520, 600, 410, 600, 580], gate_len=300)
    small = W.llama8b_hop(n_layers=2, seq_len=333, n_kv_heads=2, n_anchors=5, rank_base=64, rank_delta=64)
    print(f"[noalloc] rank 128 call 1: L={big.n_layers} S={big.seq_len} N={big.n_anchors}", flush=True)
    _both(big)
    print(f"[noalloc] rank 64 call 2: L={small.n_layers} S={small.seq_len} N={small.n_anchors}", flush=True)
    _both(small)
