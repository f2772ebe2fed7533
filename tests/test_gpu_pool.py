"""Anchor-pool updates on the GPU through the C ABI (KVCMAS App. A.3 "Cache Materialization and
Pool Updates", Eq. 12, Eq. 7): the observed correction against the fp64 oracle; an insert
into a caller-owned arena (exact reconstruction of exactly low-rank sources and corrections,
nothing outside the slot written, the Eq. 12 round trip through a correction with the new
anchor); and a gate-driven sequence (fallback, fallback, then the repeated source accepted
through the inserted anchor) whose pool decisions match the oracle policy."""
import numpy as np
import pytest
import torch

from oracle import kvc_oracle as O
from oracle import kvc_pool as P
from rank_kv_cache_layer_amd import kvc

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gen(seed):
    return torch.Generator().manual_seed(seed)


def _lowrank(L, S, D, r, g, scale=1.0):
    return (torch.randn((L, S, r), generator=g, dtype=torch.float64)
            @ torch.randn((L, r, D), generator=g, dtype=torch.float64)) * (scale / np.sqrt(r))


def _round(x, dtype):
    return x.to(dtype).double() if dtype == torch.bfloat16 else x.float().double()


@pytest.mark.parametrize("dtype,L,S,H,hd", [(torch.float32, 2, 64, 2, 64), (torch.bfloat16, 2, 128, 2, 128),
                                            (torch.float32, 1, 40, 3, 24)])
def test_observed_delta_matches_oracle(dtype, L, S, H, hd):
    print(f"[pool] observed delta {dtype} L={L} S={S} H={H} hd={hd}", flush=True)
    D, p_src, p_tgt = H * hd, 37, 101
    g = _gen(S + hd)
    ks, vs, kt, vt = (_round(torch.randn((L, S, D), generator=g, dtype=torch.float64), dtype) for _ in range(4))
    dev = [x.to(dtype).to(DEV).contiguous() for x in (ks, vs, kt, vt)]
    outs = [torch.full((L, S, D), float("nan"), device=DEV) for _ in range(4)]
    kvc.observed_delta(*dev, kvc.shape_of(L, S, H, hd), p_src, p_tgt, *outs)
    torch.cuda.synchronize()
    fr = O.inv_freq(hd)
    want = [O.rope(ks.numpy(), -p_src, hd, fr), vs.numpy(),
            O.observed_delta(kt.numpy(), ks.numpy(), p_src, p_tgt, hd, True),
            O.observed_delta(vt.numpy(), vs.numpy(), p_src, p_tgt, hd, False)]
    for name, got, w in zip(("k_base", "v_base", "k_delta", "v_delta"), outs, want):
        err = np.max(np.abs(got.double().cpu().numpy() - w))
        assert err <= 2e-6 * np.max(np.abs(w)), (name, err)
    # NULL outputs are skipped: only v_delta requested
    only = torch.full((L, S, D), 3.0, device=DEV)
    kvc.observed_delta(None, dev[1], None, dev[3], kvc.shape_of(L, S, H, hd), p_src, p_tgt, v_delta=only)
    torch.cuda.synchronize()
    assert np.max(np.abs(only.double().cpu().numpy() - want[3])) <= 2e-6 * np.max(np.abs(want[3]))


def _arena(L, V, R, D, rC, rD, dtype, fill=7.0):
    t = lambda *s: torch.full(s, fill, dtype=dtype, device=DEV)
    return kvc.PoolTensors(anchor_len=[0] * V, rank_base=rC, rank_delta=rD,
                           baseA_k=t(L, V * R, rC), baseB_k=t(L, V, rC, D), baseA_v=t(L, V * R, rC),
                           baseB_v=t(L, V, rC, D), deltaA_k=t(L, V * R, rD), deltaB_k=t(L, V, rD, D),
                           deltaA_v=t(L, V * R, rD), deltaB_v=t(L, V, rD, D), slot_rows=R, live=[0] * V)


def _pair(L, S, H, hd, r, p_src, p_tgt, seed, dtype):
    """Source with exactly rank-r canonical K and V, target by Eq. 12 with exactly rank-r
    corrections (keys canonical): C_j = Align(C_i) + R(p_tgt) Delta_K, V + Delta_V."""
    D = H * hd
    g = _gen(seed)
    kcan, v = _lowrank(L, S, D, r, g), _lowrank(L, S, D, r, g)
    dk, dv = _lowrank(L, S, D, r, g, 0.3), _lowrank(L, S, D, r, g, 0.3)
    fr = O.inv_freq(hd)
    ks = O.rope(kcan.numpy(), p_src, hd, fr)
    kt = O.rope(ks, p_tgt - p_src, hd, fr) + O.rope(dk.numpy(), p_tgt, hd, fr)
    vt = v.numpy() + dv.numpy()
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(DEV)
    return dict(k_src=dev(ks), v_src=dev(v.numpy()), k_tgt=dev(kt), v_tgt=dev(vt), kcan=kcan.numpy(), v=v.numpy(),
                dk=dk.numpy(), dv=dv.numpy(), kt=kt, vt=vt)


def test_insert_reconstructs_writes_only_its_slot_and_round_trips():
    L, S, H, hd, r, V, R = 2, 256, 2, 64, 8, 3, 320
    D, p_src, p_tgt, slot = H * hd, 29, 411, 1
    print(f"[pool] insert L={L} S={S} D={D} r={r} V={V} slot_rows={R}", flush=True)
    x = _pair(L, S, H, hd, r, p_src, p_tgt, 5, torch.float32)
    arena = _arena(L, V, R, D, r, r, torch.float32)
    shp = kvc.shape_of(L, S, H, hd)
    kvc.pool_insert(x["k_src"], x["v_src"], x["k_tgt"], x["v_tgt"], shp, p_src, p_tgt, arena, slot, oversample=8,
                    power_iters=2, seed=3)
    torch.cuda.synchronize()
    rows = slice(slot * R, slot * R + S)
    for Aname, Bname, want in (("baseA_k", "baseB_k", x["kcan"]), ("baseA_v", "baseB_v", x["v"]),
                               ("deltaA_k", "deltaB_k", x["dk"]), ("deltaA_v", "deltaB_v", x["dv"])):
        A = getattr(arena, Aname).double().cpu().numpy()
        B = getattr(arena, Bname).double().cpu().numpy()
        rec = np.einsum("lsr,lrd->lsd", A[:, rows], B[:, slot])
        rel = np.max(np.abs(rec - want)) / np.max(np.abs(want))
        print(f"[pool] {Aname} reconstruction {rel:.2e} of max|x|", flush=True)
        assert rel <= 1e-5, Aname
        # nothing outside the slot's rows / entry was written
        assert np.all(np.delete(A, np.r_[rows], axis=1) == 7.0), Aname
        assert np.all(np.delete(B, slot, axis=1) == 7.0), Bname
    # Eq. 12 round trip: correcting the same source with the new anchor gives the target
    lens, live = [0] * V, [0] * V
    lens[slot], live[slot] = S, 1
    arena.anchor_len, arena.live = lens, live
    ko, vo = torch.empty_like(x["k_src"]), torch.empty_like(x["v_src"])
    prm = kvc.params_of(0.3, 1.0, 0.1, 0, kvc.SCORE_PAGES)
    res = kvc.correct_hop(x["k_src"], x["v_src"], ko, vo, shp, p_src, p_tgt, arena, prm)
    torch.cuda.synchronize()
    for got, want in ((ko, x["kt"]), (vo, x["vt"])):
        rel = np.max(np.abs(got.double().cpu().numpy() - want)) / np.max(np.abs(want))
        print(f"[pool] round trip {rel:.2e} of max|x|", flush=True)
        assert rel <= 1e-5, rel
    assert int(res.flags[0].item()) & O.FLAG_FEW_ANCHORS   # one compatible anchor: dense fallback flagged


def test_gate_driven_sequence_matches_the_oracle_policy():
    # bf16, shapes of the two-pass kernels (D = 256, rank 16)
    L, S, H, hd, r, V = 2, 512, 2, 128, 16, 4
    D = H * hd
    print(f"[pool] sequence L={L} S={S} D={D} r={r} V={V}", flush=True)
    shp = kvc.shape_of(L, S, H, hd)
    arena = _arena(L, V, S, D, r, r, torch.bfloat16, fill=0.0)
    state, ref = kvc.PoolState(V), P.PoolPolicy(V)
    prm = kvc.params_of(0.3, 1.0, 0.1, 0, kvc.SCORE_PAGES)
    x1 = _pair(L, S, H, hd, r, 64, 300, 11, torch.bfloat16)
    x2 = _pair(L, S, H, hd, r, 64, 300, 12, torch.bfloat16)
    consumer = 2
    flags_seen = []
    for step, x in enumerate((x1, x2, x1, x1)):
        lens, live = state.view(consumer)
        arena.anchor_len, arena.live = lens, live
        ko, vo = torch.empty_like(x["k_src"]), torch.empty_like(x["v_src"])
        res = kvc.correct_hop(x["k_src"], x["v_src"], ko, vo, shp, 64, 300, arena, prm)
        torch.cuda.synchronize()
        flag = int(res.flags[0].item())
        flags_seen.append(flag)
        got = state.record_hop(consumer, S, flag != 0)
        assert got == ref.record_hop(consumer, S, flag != 0), step
        if flag != 0:
            kvc.pool_insert(x["k_src"], x["v_src"], x["k_tgt"], x["v_tgt"], shp, 64, 300, arena, got[0],
                            oversample=16, power_iters=2, seed=step)
            torch.cuda.synchronize()
        else:
            # accepted through the inserted anchor of the same source: the target, to bf16
            for o, want in ((ko, x["kt"]), (vo, x["vt"])):
                err = np.max(np.abs(o.double().cpu().numpy() - want))
                assert err <= 2.0 ** -6 * np.max(np.abs(want)), (step, err)
    # empty pool and one anchor: dense fallback (fewer than two compatible anchors); then the
    # repeated source matches its own anchor distinctly and is accepted, twice
    assert [f != 0 for f in flags_seen] == [True, True, False, False], flags_seen
    assert [a.uses if a else None for a in ref.slots] == [2, 2, None, None]
    assert list(state.c.uses[:V]) == [2, 2, 0, 0]
