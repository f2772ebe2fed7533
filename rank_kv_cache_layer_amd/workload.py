"""Seeded synthetic hop inputs for the per-hop KV-cache correction.

This module only draws random data and assembles it into the layouts the library
takes.  It holds none of the correction's arithmetic: no positional rotation, no
scores, no gate, no weights, no delta application, no rounding rule of its own
(dtype casts go through torch).  Both the fp64 oracle and the HIP path consume
exactly the tensors built here.

Shapes follow the workloads of "KVCMAS: Efficient KV cache Correction for Shared
Context in Multi-Agent Systems" (Sec. 3.1 memory example and Sec. 4.1 setup:
Llama-3.1-8B, 32 layers, 8 KV heads x 128, bf16, r = 32, pools of 10-20 anchors).

Construction of one (layer, side) slab, canonical positional frame:
  * source      Z = E * scale + A_s B_s
        E ~ N(0,1) [S x D], scale[d] ~ U(0.5, 2) per (layer, side) (unit for tiny),
        (A_s, B_s) a rank-r component with orthonormal rows in B_s.
  * base of anchor a:  (A_a, B_a), same distribution as (A_s, B_s).
        In a "matched" layer anchor 0 holds exactly (A_s, B_s); in an "unrelated"
        layer the source's component is a fresh draw that no anchor holds.
  * delta of anchor a: a rank-24 matrix U W (W orthonormal rows) whose rms is a
        fixed fraction of the source rms, padded/truncated to the delta rank.
        For the tiny workload both delta factors are plain Gaussians of std
        r^(-1/4) (unit-variance product).
Keys are drawn in the canonical frame.  Placing them at an absolute start
position p_src is a positional rotation, which this module does not implement:
callers pass a `place_keys(x, p)` callable (tests pass the oracle's), and
workloads without one keep p_src = 0, where canonical and stored frames agree.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import mmap
import multiprocessing
import os
from typing import Callable, List, Optional

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"
SCORE_PAGES = 0
SCORE_COS_R = 1

_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}

# stream tags for the seeded generators
_T_SCALE, _T_E, _T_SRCLR, _T_BASE, _T_DELTA, _T_MISC, _T_NOISE = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass
class HopSpec:
    name: str
    n_layers: int
    seq_len: int
    n_kv_heads: int
    head_dim: int
    n_anchors: int
    rank_base: int
    rank_delta: int
    dtype: str = BF16
    capacity: int = 0            # 0 -> same as n_anchors
    anchor_len: Optional[List[int]] = None   # None -> every anchor has seq_len rows
    p_src: int = 0
    p_tgt: int = 0
    theta: float = 10000.0
    tau: float = 0.3
    temp_gate: float = 1.0
    temp_weight: float = 0.1
    gate_len: int = 0            # 0 -> seq_len
    mode: int = SCORE_PAGES
    unrelated_layers: Optional[List[int]] = None   # layers whose source no anchor holds
    scaled: bool = True          # per-channel U(0.5, 2) scale
    true_delta_rank: int = 24    # 0 -> plain Gaussian delta factors (tiny workload)
    delta_rms_ratio: float = 0.1
    noise_ratio: float = 0.01    # exact target: rank-24 correction + this fraction of its rms as noise
    seed: int = 0
    source_seed: int = -1        # seed of the source slab (-1 -> seed); a chain shares A0's

    @property
    def d_model(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def shift(self) -> int:
        return self.p_tgt - self.p_src

    def lens(self) -> List[int]:
        if self.anchor_len is None:
            return [self.seq_len] * self.n_anchors
        assert len(self.anchor_len) == self.n_anchors
        return list(self.anchor_len)

    def cap(self) -> int:
        return self.capacity if self.capacity else self.n_anchors


@dataclasses.dataclass
class HopData:
    spec: HopSpec
    k_src: torch.Tensor          # [N_l, S, D]
    v_src: torch.Tensor
    baseA_k: torch.Tensor        # [N_l, sum(len), r_C]
    baseB_k: torch.Tensor        # [N_l, N, r_C, D]
    baseA_v: torch.Tensor
    baseB_v: torch.Tensor
    deltaA_k: torch.Tensor       # [N_l, sum(len), r_D]
    deltaB_k: torch.Tensor       # [N_l, N, r_D, D]
    deltaA_v: torch.Tensor
    deltaB_v: torch.Tensor
    anchor_len: List[int]
    anchor_offset: List[int]

    def tensors(self):
        return dict(k_src=self.k_src, v_src=self.v_src,
                    baseA_k=self.baseA_k, baseB_k=self.baseB_k,
                    baseA_v=self.baseA_v, baseB_v=self.baseB_v,
                    deltaA_k=self.deltaA_k, deltaB_k=self.deltaB_k,
                    deltaA_v=self.deltaA_v, deltaB_v=self.deltaB_v)


def _rng(*tags) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(t) for t in tags])))


def _orthonormal_rows(rng: np.random.Generator, r: int, d: int) -> np.ndarray:
    g = rng.standard_normal((d, r))
    q, rr = np.linalg.qr(g)
    q = q * np.sign(np.where(np.diag(rr) == 0, 1.0, np.diag(rr)))[None, :]
    return q.T.copy()                                   # [r, d]


def _workers() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n, int(os.environ.get("OMP_NUM_THREADS", n))))


def _lowrank(rng, s, r, d, sigma):
    a = rng.standard_normal((s, r)) * sigma
    b = _orthonormal_rows(rng, r, d)
    return a, b


def _delta_factors(spec: HopSpec, rng, s, r, d, rms_src):
    if spec.true_delta_rank == 0:
        std = float(r) ** -0.25
        return rng.standard_normal((s, r)) * std, rng.standard_normal((r, d)) * std
    k = spec.true_delta_rank
    sig_u = spec.delta_rms_ratio * rms_src * np.sqrt(d / k)
    u = rng.standard_normal((s, k)) * sig_u
    w = _orthonormal_rows(rng, max(k, r), d)
    if r <= k:
        return u[:, :r].copy(), w[:r].copy()
    a = np.zeros((s, r))
    a[:, :k] = u
    return a, w[:r].copy()


def _slab(spec: HopSpec, layer: int, side: int, place_keys, with_source: bool = True):
    """One (layer, side): returns source [S, D] (None without it) and per-anchor base/delta
    factors (fp64).  The factors are the same with or without the source."""
    S, D, N = spec.seq_len, spec.d_model, spec.n_anchors
    rC, rD = spec.rank_base, spec.rank_delta
    seed = spec.seed
    sseed = spec.seed if spec.source_seed < 0 else spec.source_seed
    lens = spec.lens()
    if spec.scaled:
        scale = _rng(sseed, layer, side, _T_SCALE).uniform(0.5, 2.0, size=D)
    else:
        scale = np.ones(D)
    rms_scale = float(np.sqrt(np.mean(scale ** 2)))
    sigma_b = np.sqrt(2.0) * rms_scale
    # the source's rank-r component; a matched layer's anchor 0 holds exactly these factors
    a_s, b_s = _lowrank(_rng(sseed, layer, side, _T_SRCLR), S, rC, D, sigma_b)
    unrelated = spec.unrelated_layers is not None and layer in spec.unrelated_layers
    base = []
    for a in range(N):
        if a == 0 and not unrelated:
            base.append((a_s[: lens[0]].copy(), b_s.copy()))
        else:
            base.append(_lowrank(_rng(seed, layer, side, _T_BASE, a), lens[a], rC, D, sigma_b))
    # the source's expected rms (E has variance scale^2 per channel; B_s has orthonormal rows, so
    # the low-rank part's mean square is ||A_s||^2 / (S D)): the deltas are sized from it, so they
    # do not depend on whether the source itself is drawn
    rms_src = float(np.sqrt(np.mean(scale ** 2) + np.sum(a_s ** 2) / (S * D)))
    z = None
    if with_source:
        e = _rng(sseed, layer, side, _T_E).standard_normal((S, D)) * scale[None, :]
        z = e + a_s @ b_s
    delta = []
    for a in range(N):
        rng = _rng(seed, layer, side, _T_DELTA, a)
        delta.append(_delta_factors(spec, rng, lens[a], rD, D, rms_src))
    if z is None:
        return z, base, delta
    if side == 0 and spec.p_src != 0:
        if place_keys is None:
            raise ValueError("p_src != 0 needs a place_keys callable for the key source")
        z = place_keys(z, spec.p_src)
    return z, base, delta


def target_noise(spec: HopSpec, layer: int, side: int, rows=None) -> np.ndarray:
    """The full-rank part of a matched layer's exact target correction: the relation's correction
    is the rank-24 matrix anchor 0 stores (Delta_true) plus Gaussian noise of rms
    noise_ratio x rms(Delta_true), which no rank-r anchor holds.  Rows `rows` (default all) of the
    [S, D] noise, fp64.  Only measurements use it (the normalised error against the exact target);
    the hop's inputs do not contain it."""
    S, D = spec.seq_len, spec.d_model
    sseed = spec.seed if spec.source_seed < 0 else spec.source_seed
    scale = _rng(sseed, layer, side, _T_SCALE).uniform(0.5, 2.0, size=D) if spec.scaled else np.ones(D)
    sigma_b = np.sqrt(2.0) * float(np.sqrt(np.mean(scale ** 2)))
    a_s, _ = _lowrank(_rng(sseed, layer, side, _T_SRCLR), S, spec.rank_base, D, sigma_b)
    rms_src = float(np.sqrt(np.mean(scale ** 2) + np.sum(a_s ** 2) / (S * D)))
    std = spec.noise_ratio * spec.delta_rms_ratio * rms_src
    z = _rng(spec.seed, layer, side, _T_NOISE).standard_normal((S, D)) * std
    return z if rows is None else z[np.asarray(rows)]


def _shared_empty(shape, dt: torch.dtype) -> torch.Tensor:
    """Tensor in an anonymous shared mapping: writes by forked workers are seen by the parent."""
    n = int(np.prod(shape))
    es = torch.empty((), dtype=dt).element_size()
    buf = mmap.mmap(-1, max(n * es, 1))
    raw = np.frombuffer(buf, dtype=np.uint8, count=n * es)
    return torch.from_numpy(raw).view(dt).view(shape)


_JOB = {}


def _one_blas_thread() -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    torch.set_num_threads(1)


def _fill(layer_side) -> None:
    spec, place_keys, out, offs, lens, ws = (_JOB[k] for k in ("spec", "place", "out", "offs", "lens", "ws"))
    layer, side = layer_side
    tag = "kv"[side]
    z, base, delta = _slab(spec, layer, side, place_keys, ws)
    if ws:
        out[f"{tag}_src"][layer].copy_(torch.from_numpy(z.astype(np.float32)))
    for a in range(spec.n_anchors):
        o, n = offs[a], lens[a]
        out[f"baseA_{tag}"][layer, o:o + n].copy_(torch.from_numpy(base[a][0].astype(np.float32)))
        out[f"baseB_{tag}"][layer, a].copy_(torch.from_numpy(base[a][1].astype(np.float32)))
        out[f"deltaA_{tag}"][layer, o:o + n].copy_(torch.from_numpy(delta[a][0].astype(np.float32)))
        out[f"deltaB_{tag}"][layer, a].copy_(torch.from_numpy(delta[a][1].astype(np.float32)))


def make_hop(spec: HopSpec, place_keys: Optional[Callable] = None, workers: Optional[int] = None,
             with_source: bool = True) -> HopData:
    """Build one hop's inputs; bit-identical for a given spec regardless of worker count.

    Large hops are filled by forked worker processes (each (layer, side) slab has its own
    seeded stream); that path is taken only while no GPU context exists in this process.
    with_source=False leaves k_src / v_src as zeros (a chained hop whose source is the previous
    hop's output); the anchor factors are the same either way."""
    S, D, N, L = spec.seq_len, spec.d_model, spec.n_anchors, spec.n_layers
    rC, rD = spec.rank_base, spec.rank_delta
    lens = spec.lens()
    offs = list(np.cumsum([0] + lens[:-1])) if N else []
    tot = int(sum(lens))
    dt = _TORCH_DT[spec.dtype]
    nw = workers or _workers()
    big = L * S * D >= (1 << 25)
    use_procs = nw > 1 and big and not torch.cuda.is_initialized()
    alloc = _shared_empty if use_procs else (lambda shp, d: torch.empty(shp, dtype=d))
    out = {}
    for side, tag in ((0, "k"), (1, "v")):
        out[f"{tag}_src"] = alloc((L, S, D), dt) if with_source else torch.zeros((L, S, D), dtype=dt)
        out[f"baseA_{tag}"] = alloc((L, tot, rC), dt)
        out[f"baseB_{tag}"] = alloc((L, N, rC, D), dt)
        out[f"deltaA_{tag}"] = alloc((L, tot, rD), dt)
        out[f"deltaB_{tag}"] = alloc((L, N, rD, D), dt)
    _JOB.update(spec=spec, place=place_keys, out=out, offs=offs, lens=lens, ws=with_source)
    jobs = [(l, s) for l in range(L) for s in (0, 1)]
    try:
        if nw == 1 or len(jobs) == 1:
            for j in jobs:
                _fill(j)
        elif use_procs:
            ctx = multiprocessing.get_context("fork")
            with _cf.ProcessPoolExecutor(min(nw, len(jobs)), mp_context=ctx, initializer=_one_blas_thread) as ex:
                list(ex.map(_fill, jobs))
        else:
            with _cf.ThreadPoolExecutor(nw) as ex:
                list(ex.map(_fill, jobs))
    finally:
        _JOB.clear()
    return HopData(spec=spec, anchor_len=lens, anchor_offset=[int(o) for o in offs], **out)


# ----------------------------------------------------------------------------------------
# Named workloads.  Sizes are those of the five hop configurations; `seq_len`,
# `n_layers` and friends can be overridden to get a smaller instance of the same recipe.

def tiny(**kw) -> HopSpec:
    """2 layers, 2 KV heads x 64, S = 256, fp32, 4 anchors of rank 8, shift 37."""
    base = dict(name="tiny", n_layers=2, seq_len=256, n_kv_heads=2, head_dim=64,
                n_anchors=4, rank_base=8, rank_delta=8, dtype=F32, p_src=11, p_tgt=48,
                tau=0.3, temp_weight=0.1, unrelated_layers=[1], scaled=False,
                true_delta_rank=0, seed=1)
    base.update(kw)
    return HopSpec(**base)


def llama8b_hop(**kw) -> HopSpec:
    """Llama-3.1-8B-shaped hop: 32 layers, 8 x 128, S = 4096, 20 anchors of rank 32."""
    rng = _rng(2, _T_MISC)
    p_src = int(rng.integers(0, 1025))
    s = int(rng.integers(16, 513))
    base = dict(name="llama8b_4k", n_layers=32, seq_len=4096, n_kv_heads=8, head_dim=128,
                n_anchors=20, rank_base=32, rank_delta=32, dtype=BF16, p_src=p_src,
                p_tgt=p_src + s, tau=0.3, temp_weight=0.1, seed=2)
    base.update(kw)
    return HopSpec(**base)


def llama8b_long(**kw) -> HopSpec:
    """32K shared segment, 20 anchors at r = 32, shift 300; layers 2, 5, 8, ... unrelated."""
    n_layers = kw.get("n_layers", 32)
    base = dict(name="llama8b_32k", n_layers=32, seq_len=32768, n_kv_heads=8, head_dim=128,
                n_anchors=20, rank_base=32, rank_delta=32, dtype=BF16, p_src=0, p_tgt=300,
                tau=0.3, temp_weight=0.1,
                unrelated_layers=[l for l in range(n_layers) if l % 3 == 2], seed=3)
    base.update(kw)
    return HopSpec(**base)


def llama8b_rank128(**kw) -> HopSpec:
    """4K segment corrected with 10 anchors at rank 128."""
    base = dict(name="llama8b_r128", n_layers=32, seq_len=4096, n_kv_heads=8, head_dim=128,
                n_anchors=10, rank_base=128, rank_delta=128, dtype=BF16, p_src=0, p_tgt=200,
                tau=0.3, temp_weight=0.1, seed=5)
    base.update(kw)
    return HopSpec(**base)


def chain_specs(n_requests: int = 8, n_hops: int = 3, seq_len: int = 8192, n_layers: int = 32,
                n_kv_heads: int = 8, head_dim: int = 128, seed: int = 4, **kw):
    """Concurrent batch of chains A0 -> A1 -> ... : per hop N ~ U{10..20}, shift ~ U{0..1024};
    per request r in {16, 32} (the base rank of an anchor describes the first agent's source,
    whose rank-r component every hop's matched anchor holds); the first source sits at
    p0 ~ U{0..1024}."""
    rng = _rng(seed, _T_MISC)
    reqs = []
    r0 = int(kw.pop("rank", 0))
    for q in range(n_requests):
        p = int(rng.integers(0, 1025))
        hops = []
        # every hop's matched anchor is built from the first agent's source (same source seed)
        src_seed = seed * 1000 + q * 10
        r = r0 or int(rng.choice([16, 32]))
        for h in range(n_hops):
            n = int(rng.integers(10, 21))
            s = int(rng.integers(0, 1025))
            spec = HopSpec(name=f"chain_q{q}_h{h}", n_layers=n_layers, seq_len=seq_len,
                           n_kv_heads=n_kv_heads, head_dim=head_dim, n_anchors=n,
                           rank_base=r, rank_delta=r, dtype=BF16, p_src=p, p_tgt=p + s,
                           tau=0.3, temp_weight=0.1, seed=src_seed + h, source_seed=src_seed)
            spec = dataclasses.replace(spec, **kw)
            hops.append(spec)
            p = p + s
        reqs.append(hops)
    return reqs


def decaying_matrices(n_mats: int, rows: int, cols: int, seed: int = 5, power: float = 1.5,
                      dtype=torch.float32, reflections: int = 0) -> torch.Tensor:
    """Z = U diag(i^-power) W^T with U, W orthonormal, one per matrix.

    reflections = 0: U, W from QR of Gaussians (Haar).  reflections = h > 0: U and W are each a
    product of h random Householder reflections, applied to the diagonal matrix as rank-one
    updates (the singular values are the same; far cheaper at 4096 x 1024)."""
    out = torch.empty((n_mats, rows, cols), dtype=dtype)
    k = min(rows, cols)
    sig = np.arange(1, k + 1, dtype=np.float64) ** (-power)

    def job(m):
        rng = _rng(seed, m, _T_MISC)
        if reflections > 0:
            z = np.zeros((rows, cols))
            z[np.arange(k), np.arange(k)] = sig
            for _ in range(reflections):
                u = rng.standard_normal(rows)
                u /= np.linalg.norm(u)
                z -= 2.0 * np.outer(u, u @ z)
                w = rng.standard_normal(cols)
                w /= np.linalg.norm(w)
                z -= 2.0 * np.outer(z @ w, w)
            out[m].copy_(torch.from_numpy(z.astype(np.float32)))
            return
        u, _ = np.linalg.qr(rng.standard_normal((rows, k)))
        w, _ = np.linalg.qr(rng.standard_normal((cols, k)))
        out[m].copy_(torch.from_numpy(((u * sig[None, :]) @ w.T).astype(np.float32)))

    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(n_mats)))
    return out


def singular_values(n: int, power: float = 1.5) -> np.ndarray:
    return np.arange(1, n + 1, dtype=np.float64) ** (-power)


def chain_study_caches(n_layers: int = 2, seq_len: int = 256, d: int = 256, n_agents: int = 4,
                       hop_rank: int = 24, hop_rms: float = 0.1, noise: float = 0.01, seed: int = 6,
                       device: str = "cpu"):
    """Exact caches of one side of a segment along A0 -> A1 -> ... (synthetic stand-in for the
    caches of Fig. 3(b)): a context-free reference C_ref, and C_k = C_ref + sum_{m <= k} E_m where
    each agent adds its own deviation E_m (rank hop_rank, rms hop_rms x rms(C_ref), plus a full
    rank component of rms noise x rms(E_m)).  Returns (C_ref, [C_0 .. C_{n-1}]) as fp32 tensors
    [n_layers][seq_len][d] on `device`."""
    rng = _rng(seed, _T_MISC, 77)
    ref = rng.standard_normal((n_layers, seq_len, d))
    caches, acc = [], ref.copy()
    for _ in range(n_agents):
        u = rng.standard_normal((n_layers, seq_len, hop_rank))
        w = np.stack([_orthonormal_rows(rng, hop_rank, d) for _ in range(n_layers)])
        e = np.einsum("lsr,lrd->lsd", u, w) * (hop_rms * np.sqrt(d / hop_rank))
        e += rng.standard_normal(e.shape) * noise * hop_rms
        acc = acc + e
        caches.append(acc.copy())
    t = lambda x: torch.from_numpy(x).float().to(device)
    return t(ref), [t(c) for c in caches]
