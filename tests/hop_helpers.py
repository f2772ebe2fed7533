"""Shared helpers of the GPU parity tests: run one hop through the C ABI and compare it with
the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

from oracle import kvc_oracle as O
from rank_kv_cache_layer_amd import kvc
from rank_kv_cache_layer_amd import workload as W

DEV = "cuda:0"
TOL_F32 = 1e-5            # max|gpu - oracle| <= TOL * max|oracle|, fp32 outputs
TOL_BF16 = 2.0 ** -7      # bf16 outputs with fp32 accumulation
W_ATOL = {W.F32: 1e-5, W.BF16: 2e-3}


def w_atol(dtype, mode=W.SCORE_PAGES, temp_weight=1.0):
    """Token-weight tolerance.  Second scoring mode in bf16: the weights are softmax(c / T_w) of
    cosines whose key-side MFMA operand is a rotated (canonical-frame) quantity rounded once to
    bf16, so |dc| reaches about 2^-8 (unit roundoff 2^-9 of a relative error on either factor of
    the cosine's first-order perturbation); the softmax moves no weight by more than half the
    largest logit change, so |dw| <= 2^-8 / (2 T_w) = 2^-9 / T_w (0.0195 at T_w = 0.1)."""
    if dtype == W.BF16 and mode == W.SCORE_COS_R:
        return max(W_ATOL[dtype], 2.0 ** -9 / temp_weight)
    return W_ATOL[dtype]


def place(head_dim):
    return lambda x, p: O.rope(x, p, head_dim)


def make(spec):
    return W.make_hop(spec, place_keys=place(spec.head_dim))


def params(spec, options=0):
    return kvc.params_of(spec.tau, spec.temp_gate, spec.temp_weight, spec.gate_len, spec.mode, options)


def shape(spec):
    return kvc.shape_of(spec.n_layers, spec.seq_len, spec.n_kv_heads, spec.head_dim)


def run_gpu(data, options=0, want_weights=True):
    sp = data.spec
    k = data.k_src.to(DEV)
    v = data.v_src.to(DEV)
    ko = torch.empty_like(k)
    vo = torch.empty_like(v)
    pool = kvc.pool_from(data, DEV)
    res = kvc.correct_hop(k, v, ko, vo, shape(sp), sp.p_src, sp.p_tgt, pool, params(sp, options),
                          theta=sp.theta, want_weights=want_weights)
    torch.cuda.synchronize()
    return dict(k_out=ko.double().cpu().numpy(), v_out=vo.double().cpu().numpy(),
                dist=res.dist.cpu().numpy(), stat=res.stat.cpu().numpy(), flags=res.flags.cpu().numpy(),
                w_k=None if res.w_k is None else res.w_k.double().cpu().numpy(),
                w_v=None if res.w_v is None else res.w_v.double().cpu().numpy(), s_cov=res.s_cov,
                raw_k=ko, raw_v=vo)


def assert_outputs_close(gpu, ref, dtype, label=""):
    tol = TOL_F32 if dtype == W.F32 else TOL_BF16
    for side in ("k_out", "v_out"):
        x = ref[side]
        err = np.max(np.abs(gpu[side] - x))
        bound = tol * np.max(np.abs(x))
        assert err <= bound, f"{label} {side}: max err {err:.3e} > {bound:.3e}"


def assert_gate_equal(gpu, ref, n_anchors, label="", check_margin=True, tau=None):
    assert np.array_equal(gpu["flags"], ref["flags"]), f"{label} flags gpu {gpu['flags']} oracle {ref['flags']}"
    if check_margin and tau is not None:
        st = ref["stat"][~np.isnan(ref["stat"])]
        assert np.all(np.abs(st - tau) >= 0.05) or st.size == 0, f"{label}: oracle statistic within 0.05 of tau"
    n = max(n_anchors, 1)
    dg, dr = gpu["dist"][:, :n_anchors], ref["dist"][:, :n_anchors]
    assert np.array_equal(np.isnan(dg), np.isnan(dr)), f"{label}: gate-set mismatch"
    m = ~np.isnan(dr)
    if m.any():
        assert np.allclose(dg[m], dr[m], rtol=1e-4, atol=1e-6), f"{label}: dist max err {np.max(np.abs(dg[m]-dr[m]))}"
    sg, sr = gpu["stat"], ref["stat"]
    assert np.array_equal(np.isnan(sg), np.isnan(sr))
    ms = ~np.isnan(sr)
    if ms.any():
        assert np.max(np.abs(sg[ms] - sr[ms])) < 2e-3, f"{label}: stat gpu {sg} oracle {sr}"
    del n


def assert_weights_close(gpu, ref, dtype, label="", mode=W.SCORE_PAGES, temp_weight=1.0):
    tol = w_atol(dtype, mode, temp_weight)
    for side in ("w_k", "w_v"):
        g, r = gpu[side], ref[side]
        n = r.shape[-1]
        err = np.max(np.abs(g[..., :n] - r))
        assert err <= tol, f"{label} {side}: max err {err:.3e} > {tol:.3e}"
