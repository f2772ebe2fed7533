"""Seeded random sweeps against the fp64 oracle on identical inputs.  Single hops: head_dim 64 or
128, two to eight heads, ragged token counts over several tiles, 2 to 24 anchors of full or ragged
lengths, base ranks 16 to 128, delta ranks 8 to 128, an optional gate prefix, random positions,
both scoring modes, and an unrelated layer when there are two; each case runs the library's
default path for its shape through the C ABI (KVCMAS Sec. 3.3 Eq. 7-8, App. A.3).  Batches: two
to six independent hops of one shape with ragged pools and mixed ranks in one batched call."""
import numpy as np
import pytest
import torch

from oracle import kvc_oracle as O
from rank_kv_cache_layer_amd import kvc
from rank_kv_cache_layer_amd import workload as W

from hop_helpers import DEV, assert_outputs_close, assert_weights_close, make, params, run_gpu, shape

pytestmark = pytest.mark.gpu


def _specs(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hd = int(rng.choice([64, 128]))
        nh = int(rng.choice([2, 4])) if hd == 128 else int(rng.choice([4, 8]))
        S = int(rng.integers(60, 700))
        N = int(rng.integers(2, 25))
        rb = int(rng.choice([16, 32, 64, 128]))
        rd = int(rng.choice([8, 16, 32, 64, 128]))
        L = int(rng.integers(1, 3))
        mode = int(rng.choice([W.SCORE_PAGES, W.SCORE_COS_R]))
        lens = [int(x) for x in rng.integers(max(1, S // 3), S + 1, size=N)] if rng.random() < 0.5 else None
        gate = int(rng.integers(1, S + 1)) if rng.random() < 0.4 else 0
        if lens is not None and gate > 0:
            gate = min(gate, max(lens))
        p_src = int(rng.integers(0, 2000))
        shift = int(rng.integers(0, 600))
        out.append(W.llama8b_hop(n_layers=L, seq_len=S, n_kv_heads=nh, head_dim=hd, n_anchors=N, rank_base=rb,
                                 rank_delta=rd, anchor_len=lens, gate_len=gate, mode=mode, p_src=p_src,
                                 p_tgt=p_src + shift, seed=int(rng.integers(0, 10 ** 6)),
                                 unrelated_layers=[1] if L > 1 else None))
    return out


SPECS = _specs()


@pytest.mark.parametrize("i", range(len(SPECS)))
def test_random_hop_matches_oracle(i):
    sp = SPECS[i]
    label = (f"sweep {i}: L={sp.n_layers} S={sp.seq_len} {sp.n_kv_heads}x{sp.head_dim} N={sp.n_anchors} "
             f"r={sp.rank_base}/{sp.rank_delta} mode={sp.mode} gate={sp.gate_len} "
             f"lens={'ragged' if sp.anchor_len else 'full'} seed={sp.seed}")
    print(f"[sweep] {label}", flush=True)
    data = make(sp)
    ref = O.correct_hop(data)
    gpu = run_gpu(data)
    assert gpu["s_cov"] == ref["s_cov"], label
    assert_outputs_close(gpu, ref, sp.dtype, label)
    assert_weights_close(gpu, ref, sp.dtype, label, sp.mode, sp.temp_weight)
    # decisions: bit-exact wherever the oracle's statistic is not within 0.05 of tau (rows without
    # a statistic are decided by the anchor sets alone)
    st = ref["stat"]
    decided = np.isnan(st) | (np.abs(st - sp.tau) >= 0.05)
    assert np.array_equal(gpu["flags"][decided], ref["flags"][decided]), \
        f"{label}: flags {gpu['flags']} vs oracle {ref['flags']}"


def _batches(n=8, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        nh, S, L = int(rng.choice([2, 4])), int(rng.integers(100, 600)), int(rng.integers(1, 3))
        mode = int(rng.choice([W.SCORE_PAGES, W.SCORE_COS_R]))
        specs = []
        for _h in range(int(rng.integers(2, 7))):
            N = int(rng.integers(2, 21))
            lens = [int(x) for x in rng.integers(max(1, S // 3), S + 1, size=N)] if rng.random() < 0.5 else None
            p_src = int(rng.integers(0, 1500))
            specs.append(W.llama8b_hop(n_layers=L, seq_len=S, n_kv_heads=nh, head_dim=128, n_anchors=N,
                                       rank_base=int(rng.choice([16, 32, 64])),
                                       rank_delta=int(rng.choice([16, 32, 64, 128])), anchor_len=lens, mode=mode,
                                       p_src=p_src, p_tgt=p_src + int(rng.integers(0, 500)),
                                       seed=int(rng.integers(0, 10 ** 6))))
        out.append(specs)
    return out


BATCHES = _batches()


@pytest.mark.parametrize("i", range(len(BATCHES)))
def test_random_independent_hops_batched(i):
    # App. B.1 "Workflow Structures": independent segments (ragged pools, mixed base and delta
    # ranks, one shape) corrected in one batched call equal one hop per call bit for bit, and the
    # oracle hop by hop
    specs = BATCHES[i]
    print(f"[sweep] batch {i}: {len(specs)} hops L={specs[0].n_layers} S={specs[0].seq_len} "
          f"mode={specs[0].mode} N={[s.n_anchors for s in specs]} "
          f"r={[(s.rank_base, s.rank_delta) for s in specs]}", flush=True)
    datas = [make(sp) for sp in specs]
    runs = []
    for one in (False, True):
        hl = []
        for sp, d in zip(specs, datas):
            k, v = d.k_src.to(DEV), d.v_src.to(DEV)
            hl.append(kvc.Hop(k, v, torch.empty_like(k), torch.empty_like(v), sp.p_src, sp.p_tgt, -1,
                              kvc.pool_from(d, DEV), kvc.alloc_match(sp.n_layers, sp.seq_len, sp.n_anchors, DEV)))
        kvc.correct_hops_batched(hl, shape(specs[0]), params(specs[0]), one_at_a_time=one)
        torch.cuda.synchronize()
        runs.append(hl)
    for j, (sp, d) in enumerate(zip(specs, datas)):
        a, b = runs[0][j], runs[1][j]
        assert torch.equal(a.k_out, b.k_out) and torch.equal(a.v_out, b.v_out), f"batch {i} hop {j}"
        assert torch.equal(a.out.flags, b.out.flags), f"batch {i} hop {j} flags"
        ref = O.correct_hop(d)
        gpu = dict(k_out=a.k_out.double().cpu().numpy(), v_out=a.v_out.double().cpu().numpy())
        assert_outputs_close(gpu, ref, sp.dtype, f"batch {i} hop {j}")
