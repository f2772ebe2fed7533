"""Pins of the oracle's whole-hop correction: special cases that must be bit-exact,
the Eq. 12 round trip, the Eq. 6 chained/non-chained equivalence, partial coverage,
and a brute-force loop implementation on a tiny hop."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from oracle import kvc_oracle as O
from rank_kv_cache_layer_amd import workload as W


def place(head_dim):
    return lambda x, p: O.rope(x, p, head_dim)


def _zero_deltas(d):
    for n in ("deltaA_k", "deltaA_v", "deltaB_k", "deltaB_v"):
        getattr(d, n).zero_()


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
@pytest.mark.parametrize("p_src", [0, 11])
def test_zero_shift_zero_delta_reproduces_source_bit_exact(dtype, p_src):
    sp = W.tiny(dtype=dtype, p_src=p_src, p_tgt=p_src)
    d = W.make_hop(sp, place_keys=place(64))
    _zero_deltas(d)
    r = O.correct_hop(d)
    assert np.array_equal(r["k_out"], O._np(d.k_src))
    assert np.array_equal(r["v_out"], O._np(d.v_src))


def test_values_untouched_by_shift_when_delta_zero():
    d = W.make_hop(W.tiny(p_tgt=5000), place_keys=place(64))
    _zero_deltas(d)
    r = O.correct_hop(d)
    assert np.array_equal(r["v_out"], O._np(d.v_src))
    k_al = O.round_to(O.rope(O._np(d.k_src), 5000 - 11, 64), "f32")
    assert np.array_equal(r["k_out"], k_al)


def test_partial_coverage_rows_keep_aligned_source():
    sp = W.tiny(anchor_len=[200, 180, 256 - 100, 120], gate_len=100)
    d = W.make_hop(sp, place_keys=place(64))
    r = O.correct_hop(d, round_out=False)
    assert r["s_cov"] == 200
    sets = O.anchor_sets(d.anchor_len, 256, 100)
    assert sets["gate"] == [0, 1, 2, 3] and sets["corr"] == [0]
    k_al = O.rope(O._np(d.k_src), sp.shift, 64)
    assert np.array_equal(r["k_out"][:, 200:], k_al[:, 200:])
    assert np.array_equal(r["v_out"][:, 200:], O._np(d.v_src)[:, 200:])
    assert not np.allclose(r["k_out"][:, :200], k_al[:, :200])
    assert np.all(r["w_k"][:, 200:] == 0)
    assert np.all(r["w_k"][:, :200, 1:] == 0)      # anchors 1..3 do not cover S_cov


def test_one_hot_weights_give_align_plus_delta():
    # capacity-one pool: w = 1 on the sole anchor -> C_j = Align(C_i) + delta exactly
    sp = W.tiny(n_anchors=1, capacity=1, p_src=7, p_tgt=40)
    d = W.make_hop(sp, place_keys=place(64))
    r = O.correct_hop(d, round_out=False)
    assert np.all(r["flags"] == 0)
    for l in range(2):
        dk = O._np(d.deltaA_k[l]) @ O._np(d.deltaB_k[l, 0])
        dv = O._np(d.deltaA_v[l]) @ O._np(d.deltaB_v[l, 0])
        exp_k = O.rope(O._np(d.k_src[l]), 33, 64) + O.rope(dk, 40, 64)
        assert np.max(np.abs(r["k_out"][l] - exp_k)) < 1e-12
        assert np.max(np.abs(r["v_out"][l] - (O._np(d.v_src[l]) + dv))) < 1e-12


def test_eq12_round_trip_recovers_target():
    # Delta = C_j - Align(C_i) of rank <= r: factorise it, apply it, get C_j back
    rng = np.random.default_rng(0)
    S, D, hd, r = 96, 128, 64, 8
    p_i, p_j = 13, 70
    c_i_k, c_i_v = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    dk_can = rng.standard_normal((S, r)) @ rng.standard_normal((r, D))
    dv = rng.standard_normal((S, r)) @ rng.standard_normal((r, D))
    c_j_k = O.rope(c_i_k, p_j - p_i, hd) + O.rope(dk_can, p_j, hd)
    c_j_v = c_i_v + dv
    obs_k = O.observed_delta(c_j_k, c_i_k, p_i, p_j, hd, True)
    obs_v = O.observed_delta(c_j_v, c_i_v, p_i, p_j, hd, False)
    A_k, B_k, _ = O.truncated_svd(obs_k, r)
    A_v, B_v, _ = O.truncated_svd(obs_v, r)
    w = np.ones((S, 1))
    k_out, v_out = O.apply_delta(c_i_k, c_i_v, w, w, [A_k], B_k[None], [A_v], B_v[None], p_i, p_j, hd, S)
    assert np.max(np.abs(k_out - c_j_k)) < 1e-11
    assert np.max(np.abs(v_out - c_j_v)) < 1e-11


def test_eq6_chained_equals_non_chained_with_exact_deltas():
    # Delta_{j<-i} = Delta_{j<-ref} - Delta_{i<-ref}: both routes land on C_j
    rng = np.random.default_rng(1)
    S, D = 64, 128
    c_ref = rng.standard_normal((S, D))
    d_i = rng.standard_normal((S, D)) * 0.1
    d_j = rng.standard_normal((S, D)) * 0.1
    c_i = c_ref + d_i
    one = np.ones((S, 1))
    eye = [np.eye(S)]
    _, non_chained = O.apply_delta(c_ref, c_ref, one, one, eye, [d_j], eye, [d_j], 0, 0, 64, S)
    _, chained = O.apply_delta(c_i, c_i, one, one, eye, [d_j - d_i], eye, [d_j - d_i], 0, 0, 64, S)
    assert np.max(np.abs(chained - non_chained)) < 1e-13


# ------------------------------------------------------------------ brute force
def _bf_rope_row(x, dp, hd, theta=10000.0):
    out = list(x)
    h = hd // 2
    for head in range(len(x) // hd):
        for c in range(h):
            phi = dp * theta ** (-2.0 * c / hd)
            a, b = x[head * hd + c], x[head * hd + c + h]
            out[head * hd + c] = a * math.cos(phi) - b * math.sin(phi)
            out[head * hd + c + h] = a * math.sin(phi) + b * math.cos(phi)
    return out


def _bf_hop(d):
    sp = d.spec
    S, D, N, hd = sp.seq_len, sp.d_model, sp.n_anchors, sp.head_dim
    rC = sp.rank_base
    res = dict(k_out=[], v_out=[], w_k=[], w_v=[], q=[])
    for l in range(sp.n_layers):
        for side in "kv":
            src = getattr(d, f"{side}_src")[l].double().tolist()
            A = getattr(d, f"baseA_{side}")[l].double().tolist()
            B = getattr(d, f"baseB_{side}")[l].double().tolist()
            Ad = getattr(d, f"deltaA_{side}")[l].double().tolist()
            Bd = getattr(d, f"deltaB_{side}")[l].double().tolist()
            outs, ws = [], []
            q = [0.0] * N
            for t in range(S):
                z = src[t]
                zc = _bf_rope_row(z, -sp.p_src, hd) if side == "k" else z
                m = []
                for a in range(N):
                    tot = 0.0
                    for dd in range(D):
                        rec = sum(A[a * S + t][k] * B[a][k][dd] for k in range(rC))
                        tot += abs(zc[dd] - rec)
                        if side == "v":
                            q[a] += (z[dd] - rec) ** 2
                    m.append(tot / D)
                e = [math.exp(-(mi - min(m)) / sp.temp_weight) for mi in m]
                w = [x / sum(e) for x in e]
                ws.append(w)
                delta = [sum(w[a] * sum(Ad[a * S + t][k] * Bd[a][k][dd] for k in range(sp.rank_delta))
                             for a in range(N)) for dd in range(D)]
                if side == "k":
                    base = _bf_rope_row(z, sp.shift, hd)
                    rd = _bf_rope_row(delta, sp.p_tgt, hd)
                    outs.append([base[i] + rd[i] for i in range(D)])
                else:
                    outs.append([z[i] + delta[i] for i in range(D)])
            res[f"{side}_out"].append(outs)
            res[f"w_{side}"].append(ws)
            if side == "v":
                res["q"].append(q)
    return res


def test_brute_force_matches_vectorised_oracle():
    sp = W.tiny(seq_len=24, n_kv_heads=1, head_dim=32, n_anchors=3, rank_base=4, rank_delta=4,
                p_src=3, p_tgt=9)
    d = W.make_hop(sp, place_keys=place(32))
    bf = _bf_hop(d)
    r = O.correct_hop(d, round_out=False)
    assert np.max(np.abs(np.array(bf["k_out"]) - r["k_out"])) < 1e-12
    assert np.max(np.abs(np.array(bf["v_out"]) - r["v_out"])) < 1e-12
    assert np.max(np.abs(np.array(bf["w_k"]) - r["w_k"])) < 1e-12
    assert np.max(np.abs(np.array(bf["w_v"]) - r["w_v"])) < 1e-12
    q = np.array(bf["q"])
    assert np.allclose(q, np.array(r["q"]), rtol=1e-12, atol=0)
    # gate from brute-force sums
    tot = q.sum(axis=0)
    dd = [math.sqrt(x) for x in tot]
    e = [math.exp(-(x - min(dd))) for x in dd]
    g = [x / sum(e) for x in e]
    h = -sum(x * math.log2(x) for x in g if x > 0) / math.log2(len(g))
    assert r["stat"][0] == pytest.approx(h, rel=1e-10, abs=1e-14)
    assert np.allclose(r["dist"][0], dd, rtol=1e-12)


def test_brute_force_cosine_mode():
    sp = W.tiny(seq_len=16, n_kv_heads=1, head_dim=32, n_anchors=3, rank_base=4, rank_delta=4,
                mode=W.SCORE_COS_R)
    d = W.make_hop(sp, place_keys=place(32))
    r = O.correct_hop(d, round_out=False)
    S = sp.seq_len
    for l in range(sp.n_layers):
        v = d.v_src[l].double().tolist()
        A = d.baseA_v[l].double().tolist()
        B = d.baseB_v[l].double().tolist()
        pa = [0.0] * 3
        pp = [0.0] * 3
        aa = [0.0] * 3
        for a in range(3):
            for t in range(S):
                p = [sum(v[t][dd] * B[a][k][dd] for dd in range(32)) for k in range(4)]
                arow = A[a * S + t]
                num = sum(p[k] * arow[k] for k in range(4))
                npn = math.sqrt(sum(x * x for x in p))
                nan = math.sqrt(sum(x * x for x in arow))
                c = num / (npn * nan)
                pa[a] += num
                pp[a] += npn ** 2
                aa[a] += nan ** 2
                wrow = r["w_v"][l, t]
                assert c == pytest.approx(O.cos_scores(np.array([v[t]]), [np.array([arow])],
                                                       [np.array(B[a])])[0, 0], rel=1e-12)
        cs = r["cos_sums"][l]
        assert np.allclose(cs[0], pa, rtol=1e-12) and np.allclose(cs[1], pp, rtol=1e-12)
        assert np.allclose(cs[2], aa, rtol=1e-12)
        segcos = [pa[a] / math.sqrt(pp[a] * aa[a]) for a in range(3)]
        assert np.allclose(r["dist"][1 + l], segcos, rtol=1e-12)


def test_cosine_is_one_for_exact_low_rank_match():
    rng = np.random.default_rng(7)
    b = np.linalg.qr(rng.standard_normal((128, 8)))[0].T
    a = rng.standard_normal((20, 8))
    c = O.cos_scores(a @ b, [a], [b])
    assert np.allclose(c, 1.0, atol=1e-13)


def test_tiny_workload_decisions_with_margin():
    d = W.make_hop(W.tiny(), place_keys=place(64))
    r = O.correct_hop(d)
    assert list(r["flags"]) == [0, 0, O.FLAG_ENTROPY]
    assert np.all(np.abs(r["stat"] - 0.3) >= 0.05)


def test_bf16_rounding_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(100000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, 3.0e-39, -1.5e-39]      # ties and subnormals
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), ref)


def test_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert O.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert O.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
