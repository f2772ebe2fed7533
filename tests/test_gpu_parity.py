"""GPU parity of the HIP path (called through the C ABI) against the fp64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import kvc_oracle as O
from rank_kv_cache_layer_amd import kvc
from rank_kv_cache_layer_amd import workload as W

from hop_helpers import (DEV, assert_gate_equal, assert_outputs_close, assert_weights_close, make, params,
                         run_gpu, shape)

pytestmark = pytest.mark.gpu


def _check_hop(spec, options=0, label=""):
    print(f"[parity] {label or spec.name} dtype={spec.dtype} L={spec.n_layers} S={spec.seq_len} "
          f"D={spec.d_model} N={spec.n_anchors} r={spec.rank_base}/{spec.rank_delta} mode={spec.mode} "
          f"opt={options}", flush=True)
    data = make(spec)
    ref = O.correct_hop(data)
    gpu = run_gpu(data, options=options)
    assert gpu["s_cov"] == ref["s_cov"]
    assert_outputs_close(gpu, ref, spec.dtype, label)
    assert_gate_equal(gpu, ref, spec.n_anchors, label, tau=spec.tau)
    assert_weights_close(gpu, ref, spec.dtype, label, spec.mode, spec.temp_weight)
    return data, ref, gpu


# ------------------------------------------------------------------------- align
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("hd", [64, 128, 96, 6])
def test_align_rope_matches_oracle(dt, hd):
    print(f"[parity] align dtype={dt} head_dim={hd}", flush=True)
    g = torch.Generator().manual_seed(hd)
    L, S, H = 3, 77, 4
    x = torch.randn((L, S, H * hd), generator=g).to(dt)
    out = torch.empty_like(x, device=DEV)
    kvc.align_rope(x.to(DEV), out, kvc.shape_of(L, S, H, hd), 512, 812)
    ref = O.round_to(O.rope(x.double().numpy(), 300, hd), "f32" if dt == torch.float32 else "bf16")
    got = out.double().cpu().numpy()
    tol = 1e-5 if dt == torch.float32 else 2.0 ** -7
    assert np.max(np.abs(got - ref)) <= tol * np.max(np.abs(ref))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_align_zero_shift_bit_exact_and_in_place(dt):
    x = torch.randn((2, 64, 256)).to(dt).to(DEV)
    y = torch.empty_like(x)
    kvc.align_rope(x, y, kvc.shape_of(2, 64, 2, 128), 100, 100)
    assert torch.equal(x, y)
    z = x.clone()
    kvc.align_rope(z, z, kvc.shape_of(2, 64, 2, 128), 0, 37)
    kvc.align_rope(z, z, kvc.shape_of(2, 64, 2, 128), 37, 0)
    tol = 1e-5 if dt == torch.float32 else 2 * 2.0 ** -7
    assert (z.float() - x.float()).abs().max().item() <= tol * x.float().abs().max().item()


def test_align_dtype_conversion():
    x = torch.randn((1, 32, 128))
    y = torch.empty((1, 32, 128), dtype=torch.bfloat16, device=DEV)
    kvc.align_rope(x.to(DEV), y, kvc.shape_of(1, 32, 1, 128), 5, 5)
    assert torch.equal(y.cpu(), x.to(torch.bfloat16))


# ------------------------------------------------------------------- whole hop
def test_tiny_fp32_hop():
    _, ref, gpu = _check_hop(W.tiny(), label="tiny")
    assert list(gpu["flags"]) == [0, 0, O.FLAG_ENTROPY]


def test_tiny_fp32_cosine_mode():
    _, ref, gpu = _check_hop(W.tiny(mode=W.SCORE_COS_R), label="tiny-cos")
    assert list(gpu["flags"]) == [0, 0, O.FLAG_COS_BELOW]


@pytest.mark.parametrize("mode", [W.SCORE_PAGES, W.SCORE_COS_R])
@pytest.mark.parametrize("options", [0, 1, 2])   # two-pass MFMA, generic VALU, single-pass fused MFMA
def test_llama_shape_reduced_bf16(mode, options):
    # 8B shape per layer, fewer layers and a ragged token count (several tiles + tail)
    sp = W.llama8b_hop(n_layers=3, seq_len=1000, mode=mode, tau=0.3 if mode == W.SCORE_PAGES else 0.5)
    _check_hop(sp, options=options, label=f"llama-reduced-{mode}-{options}")


def test_unrelated_layers_flagged_bf16():
    sp = W.llama8b_long(n_layers=3, seq_len=520, unrelated_layers=[2])
    _, ref, gpu = _check_hop(sp, label="long-reduced")
    assert list(gpu["flags"]) == [0, 0, 0, O.FLAG_ENTROPY]


@pytest.mark.parametrize("mode", [W.SCORE_PAGES, W.SCORE_COS_R])
@pytest.mark.parametrize("rank", [16, 64, 128])
def test_ranks_bf16(rank, mode):
    # second mode: rank 16 on the generic scores, ranks 64 / 128 on the GEMM in column groups of 32;
    # ranks 64 / 128: the delta goes through the two-pass apply in rank slices of 32 (first mode:
    # scores and weights from the fused kernel)
    sp = W.llama8b_hop(n_layers=2, seq_len=300, n_anchors=6, rank_base=rank, rank_delta=rank,
                       n_kv_heads=4, mode=mode, tau=0.3 if mode == W.SCORE_PAGES else 0.5)
    _check_hop(sp, label=f"rank{rank}-{mode}")


@pytest.mark.parametrize("mode", [W.SCORE_PAGES, W.SCORE_COS_R])
def test_rank_sliced_delta_ragged_bf16(mode):
    # a rank-128 delta in four slices of 32 behind rank-32 scores, anchors of unequal length, a
    # ragged tail tile: every anchor covers the segment's first 180 rows (gate prefix), the
    # longest covers 333 = S, so the correction set is anchors 0 and 3
    sp = W.llama8b_hop(n_layers=2, seq_len=333, n_anchors=5, rank_base=32, rank_delta=128, n_kv_heads=2,
                       anchor_len=[333, 250, 180, 333, 201], gate_len=180, mode=mode,
                       tau=0.3 if mode == W.SCORE_PAGES else 0.5)
    _check_hop(sp, label=f"rank-delta-128-ragged-{mode}")


@pytest.mark.parametrize("mode", [W.SCORE_PAGES, W.SCORE_COS_R])
@pytest.mark.parametrize("rank", [64, 128, 256])
def test_rank_sliced_partial_coverage(rank, mode):
    # App. A.3 "Variable Segment Lengths" at the sliced delta ranks: the longest anchor (250 rows)
    # is shorter than the segment (333), so S_cov = 250 ends inside the second 128-token tile, rows
    # 250.. keep R(s) K / V exactly, and the correction set is the anchors of length 250 (0, 1, 3);
    # a slice's A rows past an anchor's length read as zeros.  Gate prefix 180 (all five anchors)
    rb = 32 if rank == 256 else rank
    sp = W.llama8b_hop(n_layers=2, seq_len=333, n_anchors=5, rank_base=rb, rank_delta=rank, n_kv_heads=2,
                       anchor_len=[250, 250, 180, 250, 201], gate_len=180, mode=mode,
                       tau=0.3 if mode == W.SCORE_PAGES else 0.5)
    data, ref, gpu = _check_hop(sp, label=f"rank{rank}-partial-{mode}")
    assert ref["s_cov"] == 250
    # rows past coverage keep the source: values bit for bit, keys re-aligned (within the bound above)
    assert np.array_equal(gpu["v_out"][:, 250:], O._np(data.v_src)[:, 250:])


@pytest.mark.parametrize("mode", [W.SCORE_PAGES, W.SCORE_COS_R])
@pytest.mark.parametrize("rank", [32, 128])
def test_no_live_anchor_writes_zero_weights(rank, mode):
    # an arena whose slots are all empty: no anchor scores, corrects or gates; the hop is flagged
    # (fewer than two compatible anchors), the output is the re-aligned source and every token
    # weight the caller asked for is written as 0 (the buffers start as NaN here)
    sp = W.llama8b_hop(n_layers=2, seq_len=200, n_anchors=4, rank_base=rank, rank_delta=rank, n_kv_heads=2,
                       mode=mode, tau=0.3 if mode == W.SCORE_PAGES else 0.5)
    data = make(sp)
    k, v = data.k_src.to(DEV), data.v_src.to(DEV)
    pool = kvc.pool_from(data, DEV)
    pool.live = [0] * sp.n_anchors
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    out = kvc.alloc_match(sp.n_layers, sp.seq_len, sp.n_anchors, DEV)
    out.w_k.fill_(float("nan"))
    out.w_v.fill_(float("nan"))
    kvc.correct_hop(k, v, ko, vo, shape(sp), sp.p_src, sp.p_tgt, pool, params(sp), out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.w_k).item() == 0 and torch.count_nonzero(out.w_v).item() == 0
    assert out.s_cov == 0
    assert np.all(out.flags.cpu().numpy() & O.FLAG_FEW_ANCHORS)
    exp_k = O.round_to(O.rope(O._np(data.k_src), sp.shift, sp.head_dim), "bf16")
    assert np.max(np.abs(ko.double().cpu().numpy() - exp_k)) <= 2.0 ** -7 * np.max(np.abs(exp_k))
    assert torch.equal(vo, v)


def test_rank256_delta_two_pass_bf16():
    # rank-256 deltas: eight slices per anchor through the two-pass apply, rank-16 two-pass scores
    sp = W.llama8b_hop(n_layers=2, seq_len=260, n_anchors=3, rank_base=16, rank_delta=256, n_kv_heads=2)
    _check_hop(sp, label="rank-delta-256")


def test_apply_rank128_given_weights_matches_correct_hop():
    # the explicit apply at rank 128 (slices) with the weights the match returned reproduces the
    # corrected hop bit for bit (same kernels, same operands)
    sp = W.llama8b_hop(n_layers=2, seq_len=260, n_kv_heads=2, n_anchors=4, rank_base=128, rank_delta=128)
    print(f"[parity] apply-r128 L=2 S=260 D={sp.d_model}", flush=True)
    data = make(sp)
    full = run_gpu(data)
    k, v = data.k_src.to(DEV), data.v_src.to(DEV)
    pool = kvc.pool_from(data, DEV)
    m = kvc.match_anchors(k, v, shape(sp), sp.p_src, pool, params(sp))
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    kvc.apply_lowrank_delta(k, v, ko, vo, shape(sp), sp.p_src, sp.p_tgt, pool, m.w_k, m.w_v, m.s_cov)
    torch.cuda.synchronize()
    assert torch.equal(ko, full["raw_k"]) and torch.equal(vo, full["raw_v"])


def test_rank8_delta_two_pass_bf16():
    # rank-8 corrections on the two-pass apply (padded to the MFMA's 16 on chip)
    sp = W.llama8b_hop(n_layers=2, seq_len=300, n_anchors=6, rank_base=16, rank_delta=8, n_kv_heads=2)
    _check_hop(sp, label="rank-delta-8")


def test_preconstructed_rank8_delta_weight_one():
    # App. A.2: a recurring relation's correction, profiled once at rank 8, reused with weight 1
    # and re-alignment and no matching: K_out = R(s) K + R(p_tgt) A B, V_out = V + A B
    sp = W.llama8b_hop(n_layers=2, seq_len=520, n_kv_heads=2, n_anchors=1, rank_base=16, rank_delta=8)
    print(f"[parity] pf-delta L=2 S=520 D={sp.d_model} r=8", flush=True)
    data = make(sp)
    k, v = data.k_src.to(DEV), data.v_src.to(DEV)
    pool = kvc.pool_from(data, DEV)
    w = torch.ones((2, 520, 1), dtype=torch.float32, device=DEV)
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    kvc.apply_lowrank_delta(k, v, ko, vo, shape(sp), sp.p_src, sp.p_tgt, pool, w, w, 520)
    torch.cuda.synchronize()
    for l in range(2):
        A, B = O.layer_factors(data, l, "k", "delta", [0])
        Av, Bv = O.layer_factors(data, l, "v", "delta", [0])
        exp_k = O.rope(O._np(data.k_src[l]), sp.shift, 128) + O.rope(A[0] @ B[0], sp.p_tgt, 128)
        exp_v = O._np(data.v_src[l]) + Av[0] @ Bv[0]
        gk, gv = ko[l].double().cpu().numpy(), vo[l].double().cpu().numpy()
        assert np.max(np.abs(gk - exp_k)) <= 2.0 ** -7 * np.max(np.abs(exp_k))
        assert np.max(np.abs(gv - exp_v)) <= 2.0 ** -7 * np.max(np.abs(exp_v))


def test_head_dim_64_bf16():
    sp = W.llama8b_hop(n_layers=2, seq_len=200, n_kv_heads=4, head_dim=64, n_anchors=5)
    _check_hop(sp, label="hd64")


# second scoring mode on its two MFMA kernels (option 0: one GEMM per layer-side over 128-token
# work-groups, column groups of 32 in passes of 20; option 2: the per-anchor-group kernel):
# head_dim 64, ragged anchors with a gate prefix, more than one pass, a ragged token tail; ranks
# 64 and 128 (two and four column groups per anchor, summed across waves before the cosine)
COS_CASES = {
    "hd64": dict(n_layers=2, seq_len=200, n_kv_heads=4, head_dim=64, n_anchors=5),
    # one head: two and four 32-channel chunks, so the epilogue's A rows ride on the first chunks'
    # trailing transfers
    "one_head_hd64": dict(n_layers=2, seq_len=230, n_kv_heads=1, head_dim=64, n_anchors=6,
                          anchor_len=[230, 180, 230, 230, 99, 230]),
    "one_head_hd128": dict(n_layers=2, seq_len=150, n_kv_heads=1, head_dim=128, n_anchors=21),
    "ragged": dict(n_layers=2, seq_len=400, n_kv_heads=2, n_anchors=5,
                   anchor_len=[330, 400, 250, 400, 390], gate_len=250),
    "two_passes": dict(n_layers=2, seq_len=330, n_kv_heads=2, n_anchors=23),
    "r64_ragged_two_passes": dict(n_layers=2, seq_len=333, n_kv_heads=2, n_anchors=12, rank_base=64,
                                  rank_delta=64, gate_len=200,
                                  anchor_len=[333, 300, 250, 333, 201, 333, 333, 290, 333, 260, 333, 333]),
    "r128_hd64": dict(n_layers=2, seq_len=260, n_kv_heads=4, head_dim=64, n_anchors=7, rank_base=128,
                      rank_delta=128, anchor_len=[260, 200, 260, 260, 150, 260, 230]),
    # the longest anchor shorter than the segment: S_cov < S at the sliced ranks
    "r64_partial": dict(n_layers=2, seq_len=333, n_kv_heads=2, n_anchors=6, rank_base=64, rank_delta=64,
                        gate_len=200, anchor_len=[300, 300, 250, 300, 201, 290]),
    "r128_partial": dict(n_layers=2, seq_len=260, n_kv_heads=2, n_anchors=5, rank_base=128, rank_delta=128,
                         gate_len=150, anchor_len=[230, 200, 230, 150, 230]),
}


@pytest.mark.parametrize("case", sorted(COS_CASES))
@pytest.mark.parametrize("options", [0, 2])
def test_cosine_mode_mfma_kernels(case, options):
    sp = W.llama8b_hop(mode=W.SCORE_COS_R, tau=0.5, **COS_CASES[case])
    _check_hop(sp, options=options, label=f"cos-{case}-{options}")


@pytest.mark.parametrize("mode", [W.SCORE_PAGES, W.SCORE_COS_R])
def test_wide_rows_bf16(mode):
    # D = 2048: eight channel tiles per token tile, 64 contraction chunks in the second mode, and
    # the per-column operand packing (rows too wide to stage in LDS)
    sp = W.llama8b_hop(n_layers=1, seq_len=200, n_kv_heads=16, n_anchors=3, mode=mode,
                       tau=0.3 if mode == W.SCORE_PAGES else 0.5)
    _check_hop(sp, label=f"wide-{mode}")


def test_odd_shape_bf16_generic_path():
    sp = W.llama8b_hop(n_layers=2, seq_len=70, n_kv_heads=3, head_dim=32, n_anchors=3, rank_base=8,
                       rank_delta=8, true_delta_rank=4)
    _check_hop(sp, label="odd")


def test_partial_coverage_and_gate_prefix():
    sp = W.llama8b_hop(n_layers=2, seq_len=400, n_kv_heads=2, n_anchors=5,
                       anchor_len=[330, 400, 250, 400, 390], gate_len=250)
    data, ref, gpu = _check_hop(sp, label="ragged")
    assert ref["s_cov"] == 400


def test_partial_coverage_short_pool():
    sp = W.llama8b_hop(n_layers=2, seq_len=400, n_kv_heads=2, n_anchors=4,
                       anchor_len=[300, 310, 290, 200], gate_len=128)
    data, ref, gpu = _check_hop(sp, label="short")
    assert ref["s_cov"] == 310
    # rows beyond the coverage keep the re-aligned source: values bit-exact, keys to the
    # rotation's rounding (fp32 on the GPU, fp64 in the oracle)
    k_al = O.round_to(O.rope(O._np(data.k_src), sp.shift, sp.head_dim), "bf16")
    assert np.max(np.abs(gpu["k_out"][:, 310:] - k_al[:, 310:])) <= 2.0 ** -8 * np.max(np.abs(k_al))
    assert np.array_equal(gpu["v_out"][:, 310:], O._np(data.v_src)[:, 310:])
    # ... and are exactly what the library's own re-alignment call writes
    al = torch.empty_like(gpu["raw_k"])
    kvc.align_rope(data.k_src.to(DEV), al, shape(sp), sp.p_src, sp.p_tgt)
    torch.cuda.synchronize()
    assert torch.equal(al[:, 310:], gpu["raw_k"][:, 310:])


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_zero_shift_zero_delta_bit_exact(dtype):
    sp = W.llama8b_hop(n_layers=2, seq_len=200, n_kv_heads=2, n_anchors=3, dtype=dtype, p_src=0, p_tgt=0)
    data = make(sp)
    for n in ("deltaA_k", "deltaA_v", "deltaB_k", "deltaB_v"):
        getattr(data, n).zero_()
    gpu = run_gpu(data)
    assert np.array_equal(gpu["k_out"], O._np(data.k_src))
    assert np.array_equal(gpu["v_out"], O._np(data.v_src))


def test_capacity_one_bypass_and_empty_pool():
    sp = W.llama8b_hop(n_layers=2, seq_len=128, n_kv_heads=2, n_anchors=1, capacity=1)
    data, ref, gpu = _check_hop(sp, label="cap1")
    assert np.all(gpu["flags"] == 0)
    sp0 = W.llama8b_hop(n_layers=2, seq_len=128, n_kv_heads=2, n_anchors=0)
    data0 = make(sp0)
    gpu0 = run_gpu(data0)
    assert np.all(gpu0["flags"] == O.FLAG_FEW_ANCHORS)
    k_al = O.round_to(O.rope(O._np(data0.k_src), sp0.shift, sp0.head_dim), "bf16")
    assert np.max(np.abs(gpu0["k_out"] - k_al)) <= 2.0 ** -7 * np.max(np.abs(k_al))
    assert np.array_equal(gpu0["v_out"], O._np(data0.v_src))


def test_identical_anchors_flag_entropy_one():
    sp = W.llama8b_hop(n_layers=2, seq_len=128, n_kv_heads=2, n_anchors=4)
    data = make(sp)
    for n in ("baseA_k", "baseA_v"):
        t = getattr(data, n)
        t[:, 128:] = t[:, :128].repeat(1, 3, 1)
    for n in ("baseB_k", "baseB_v"):
        t = getattr(data, n)
        t[:, 1:] = t[:, :1]
    gpu = run_gpu(data)
    assert np.all(gpu["flags"] == O.FLAG_ENTROPY)
    assert np.allclose(gpu["stat"], 1.0, atol=1e-12)


def test_repeated_runs_bit_identical():
    sp = W.llama8b_hop(n_layers=2, seq_len=300, n_kv_heads=4, n_anchors=8)
    data = make(sp)
    a = run_gpu(data)
    b = run_gpu(data)
    for key in ("k_out", "v_out", "dist", "stat", "flags", "w_k", "w_v"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_match_then_apply_equals_correct_hop():
    sp = W.llama8b_hop(n_layers=2, seq_len=260, n_kv_heads=4, n_anchors=6)
    data = make(sp)
    full = run_gpu(data)
    k, v = data.k_src.to(DEV), data.v_src.to(DEV)
    pool = kvc.pool_from(data, DEV)
    m = kvc.match_anchors(k, v, shape(sp), sp.p_src, pool, params(sp))
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    kvc.apply_lowrank_delta(k, v, ko, vo, shape(sp), sp.p_src, sp.p_tgt, pool, m.w_k, m.w_v, m.s_cov)
    torch.cuda.synchronize()
    assert torch.equal(ko, full["raw_k"]) and torch.equal(vo, full["raw_v"])
    assert np.array_equal(m.flags.cpu().numpy(), full["flags"])


def test_apply_explicit_one_hot_weights():
    # one-hot weights on anchor 2: K_out = R(s) K + R(p_tgt) A_2 B_2, V_out = V + A_2 B_2
    sp = W.llama8b_hop(n_layers=2, seq_len=192, n_kv_heads=2, n_anchors=4)
    data = make(sp)
    k, v = data.k_src.to(DEV), data.v_src.to(DEV)
    pool = kvc.pool_from(data, DEV)
    w = torch.zeros((2, 192, 4), dtype=torch.float32, device=DEV)
    w[..., 2] = 1.0
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    kvc.apply_lowrank_delta(k, v, ko, vo, shape(sp), sp.p_src, sp.p_tgt, pool, w, w, 192)
    torch.cuda.synchronize()
    for l in range(2):
        A, B = O.layer_factors(data, l, "k", "delta", [2])
        Av, Bv = O.layer_factors(data, l, "v", "delta", [2])
        exp_k = O.rope(O._np(data.k_src[l]), sp.shift, 128) + O.rope(A[0] @ B[0], sp.p_tgt, 128)
        exp_v = O._np(data.v_src[l]) + Av[0] @ Bv[0]
        gk, gv = ko[l].double().cpu().numpy(), vo[l].double().cpu().numpy()
        assert np.max(np.abs(gk - exp_k)) <= 2.0 ** -7 * np.max(np.abs(exp_k))
        assert np.max(np.abs(gv - exp_v)) <= 2.0 ** -7 * np.max(np.abs(exp_v))


def _run_chain(reqs, one_at_a_time=False):
    """All requests' hops through one kvc_correct_hops_batched call (each chain level batched
    unless one_at_a_time); returns the per-request hop data and the library's hop records."""
    datas, hl = [], []
    for hops in reqs:
        ds = [make(h) for h in hops]
        base = len(hl)
        k0, v0 = ds[0].k_src.to(DEV), ds[0].v_src.to(DEV)
        for i, (h, d) in enumerate(zip(hops, ds)):
            hl.append(kvc.Hop(k0 if i == 0 else None, v0 if i == 0 else None, torch.empty_like(k0),
                              torch.empty_like(v0), h.p_src, h.p_tgt, base + i - 1 if i else -1,
                              kvc.pool_from(d, DEV), kvc.alloc_match(h.n_layers, h.seq_len, h.n_anchors, DEV)))
        datas.append(ds)
    kvc.correct_hops_batched(hl, shape(reqs[0][0]), params(reqs[0][0]), one_at_a_time=one_at_a_time)
    torch.cuda.synchronize()
    return datas, hl


def _check_chain_identical_inputs(reqs, datas, hl, label):
    """Each hop against the oracle on the same inputs: hop h's source is the GPU's materialised
    (bf16) output of hop h - 1 (KVCMAS Sec. 3.2 Eq. 6; App. A.3 "Cache Materialization"), so every
    hop is held to the bf16 bound 2^-7 max|x| and bit-exact flags.  The drift of a chain the oracle
    runs on its own outputs is printed as a diagnostic only."""
    base = 0
    for q, (hops, ds) in enumerate(zip(reqs, datas)):
        src_k, src_v = ds[0].k_src, ds[0].v_src
        own_k, own_v = src_k, src_v
        for i, (h, d) in enumerate(zip(hops, ds)):
            gh = hl[base + i]
            ref = O.correct_hop(dataclasses.replace(d, k_src=src_k, v_src=src_v))
            gpu = dict(k_out=gh.k_out.double().cpu().numpy(), v_out=gh.v_out.double().cpu().numpy())
            assert_outputs_close(gpu, ref, h.dtype, f"{label} request {q} hop {i}")
            pred = i > 0 and hl[base + i - 1].out.flags[0].item() != 0
            flags = gh.out.flags.cpu().numpy()
            assert np.array_equal(flags, ref["flags"] | (kvc.FLAG_PRED_FLAGGED if pred else 0)), (label, q, i, flags)
            assert np.all(ref["flags"] == 0), "chain workload: every hop should match its anchor 0"
            own = O.correct_hop(dataclasses.replace(d, k_src=own_k, v_src=own_v))
            drift = max(np.max(np.abs(own[s] - gpu[s])) / np.max(np.abs(own[s])) for s in ("k_out", "v_out"))
            print(f"[parity] {label} request {q} hop {i}: N={h.n_anchors} r={h.rank_base}; oracle-only chain "
                  f"drift {drift:.2e} of max|x| (diagnostic)", flush=True)
            # the next hop's source: the GPU's bf16 output (the oracle's own, for the diagnostic)
            src_k, src_v = gh.k_out.cpu(), gh.v_out.cpu()
            own_k = torch.from_numpy(own["k_out"]).to(torch.bfloat16)
            own_v = torch.from_numpy(own["v_out"]).to(torch.bfloat16)
        base += len(hops)


@pytest.mark.parametrize("mode", [W.SCORE_PAGES, W.SCORE_COS_R])
@pytest.mark.parametrize("rank", [0, 128])
def test_batched_chain_matches_oracle_hop_by_hop(mode, rank):
    # rank 0: the chain specification's ranks (16 / 32); 128: every pool at rank 128 (first mode:
    # the sliced apply behind fused scores, so those hops run one call at a time; second mode: four
    # column groups per anchor and up to four passes)
    reqs = W.chain_specs(n_requests=2, n_hops=3, seq_len=256, n_layers=2, n_kv_heads=2)
    reqs = [[dataclasses.replace(h, rank_base=rank or h.rank_base, rank_delta=rank or h.rank_delta,
                                 mode=mode, tau=0.3 if mode == W.SCORE_PAGES else 0.5) for h in hops]
            for hops in reqs]
    print(f"[parity] chain mode={mode} ranks={[h.rank_base for hops in reqs for h in hops]}", flush=True)
    datas, hl = _run_chain(reqs)
    _check_chain_identical_inputs(reqs, datas, hl, f"chain-{mode}-{rank}")


@pytest.mark.parametrize("seed", [4, 9, 13])
def test_batched_chain_8b_heads_levels_batched(seed):
    # the chain specification at the 8B head layout (8 x 128, D = 1024), 4 layers, 1024 tokens,
    # 3 requests x 3 hops, pools of 10-20 anchors at ranks 16 / 32: each level runs as one grid per
    # kernel; the outputs, weights and gate rows equal those of one call per hop bit for bit (the
    # same tile code), and every hop matches the oracle on the GPU's own chained inputs
    reqs = W.chain_specs(n_requests=3, n_hops=3, seq_len=1024, n_layers=4, n_kv_heads=8, seed=seed)
    print(f"[parity] chain 8x128 seed {seed}: N={[h.n_anchors for hops in reqs for h in hops]} "
          f"r={[h.rank_base for hops in reqs for h in hops]}", flush=True)
    if seed == 4:
        assert {h.rank_base for hops in reqs for h in hops} == {16, 32}
    datas, hl = _run_chain(reqs)
    _, hl1 = _run_chain(reqs, one_at_a_time=True)
    for a, b in zip(hl, hl1):
        assert torch.equal(a.k_out, b.k_out) and torch.equal(a.v_out, b.v_out)
        assert torch.equal(a.out.flags, b.out.flags)
        assert torch.equal(a.out.dist.nan_to_num(-1.0), b.out.dist.nan_to_num(-1.0))
        assert torch.equal(a.out.w_k, b.out.w_k) and torch.equal(a.out.w_v, b.out.w_v)
    _check_chain_identical_inputs(reqs, datas, hl, f"chain-8x128-seed{seed}")


def test_fan_in_ragged_pools_in_one_batched_call():
    # App. B.1 "Workflow Structures": at fan-in each incoming segment keeps its own source cache
    # and is corrected separately; App. A.3 "Variable Segment Lengths": ragged anchors, gate set
    # (length >= k) and correction set (covering the longest covered prefix) differ
    S = 256
    segs = [dict(anchor_len=[S, S, S, S], p_src=40, p_tgt=700, seed=21),
            dict(anchor_len=[S, 180, S, 90, S], p_src=900, p_tgt=956, seed=22),
            dict(anchor_len=[200, 160, 200], p_src=3, p_tgt=1212, seed=23)]
    specs = [W.llama8b_hop(n_layers=2, seq_len=S, n_kv_heads=2, n_anchors=len(g["anchor_len"]), **g) for g in segs]
    datas = [make(sp) for sp in specs]
    print(f"[parity] fan-in: {len(specs)} segments, pools {[g['anchor_len'] for g in segs]}", flush=True)
    hl = []
    for sp, d in zip(specs, datas):
        k, v = d.k_src.to(DEV), d.v_src.to(DEV)
        hl.append(kvc.Hop(k, v, torch.empty_like(k), torch.empty_like(v), sp.p_src, sp.p_tgt, -1,
                          kvc.pool_from(d, DEV), kvc.alloc_match(sp.n_layers, S, sp.n_anchors, DEV)))
    kvc.correct_hops_batched(hl, shape(specs[0]), params(specs[0]))
    torch.cuda.synchronize()
    for i, (sp, d, h) in enumerate(zip(specs, datas, hl)):
        ref = O.correct_hop(d)
        gpu = dict(k_out=h.k_out.double().cpu().numpy(), v_out=h.v_out.double().cpu().numpy())
        assert_outputs_close(gpu, ref, sp.dtype, f"fan-in segment {i}")
        assert np.array_equal(h.out.flags.cpu().numpy(), ref["flags"]), i
    # the third segment: no anchor covers it, so its tail keeps the re-aligned source and the
    # gate (no anchor of length >= k) falls back
    assert O.correct_hop(datas[2])["s_cov"] == 200
    assert hl[2].out.flags[0].item() & O.FLAG_FEW_ANCHORS

