"""Plain fp64 CPU oracle of the per-hop KV-cache correction of KVCMAS.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module; only the tests, the smoke check and the CPU-baseline leg of the benchmark
do.  It shares no code with the HIP library.

Source: "KVCMAS: Efficient KV cache Correction for Shared Context in Multi-Agent
Systems" (arXiv 2609.34060).  Every function names the passage it follows:
  * Sec. 2.2 (alignment before reuse), App. A.2 and App. A.3 "Correction Weighting
    and Positional Alignment": keys are re-aligned with a deterministic positional
    rotation; values are not rotated.  Rotate-half RoPE, w_c = theta^(-2c/d_h).
  * Sec. 3.3 Eq. 7: anchor states stored as Z ~ A_Z B_Z (A = U_r Sigma_r, B = R_r^T).
  * Sec. 3.3 Eq. 8: delta estimate = sum_v w_v A_{Delta,v} B_{Delta,v}, sum w = 1.
  * App. A.3 Eq. 9-11: reliability gate on reconstructed value states over the
    prefix k, softmax(-d / T) with T = 1, normalised entropy, accept iff <= tau;
    fewer than two compatible anchors -> dense prefill.
  * App. A.3 "Correction Weighting": token-wise weights from the mean absolute
    distance, separately for keys and values, softmax over anchors.
  * App. A.3 "Variable Segment Lengths": gate set = anchors with length >= k;
    correction uses anchors covering the segment, else the longest covered prefix,
    the remaining rows keep the re-aligned source.
  * App. A.3 Eq. 12 and "Cache Materialization": target = Align(source) + delta.
  * App. C.3: a pool of capacity one bypasses the gate and uses its sole anchor.
  * Second scoring mode (not on the pages): cosine similarity between the source
    projected on an anchor's r-dim basis and the anchor's own coordinates, softmax
    with temperature; the hop is flagged when the best segment cosine is below tau.

Readings where the pages are silent are listed in the repository's design notes;
the ones that shape this code: canonical frame = segment-relative positions (token
t at position t), so every rotation is a per-hop constant; stored anchor keys and
key deltas are canonical; the key output is R(s) K_src + R(p_tgt) delta_K with
s = p_tgt - p_src (identical to R(p_tgt)(K_can + delta) in exact arithmetic, but
the written form keeps zero-shift, zero-delta bit-exact).

Parity pins for each function live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

PAGES = 0
COS_R = 1

FLAG_ENTROPY = 1       # normalised entropy above tau (Eq. 11)
FLAG_FEW_ANCHORS = 2   # fewer than two compatible anchors (App. A.3 "Reliability Gate")
FLAG_COS_BELOW = 4     # best segment cosine below tau (second scoring mode)


# --------------------------------------------------------------------------- RoPE
def inv_freq(head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """Rotary frequencies w_c = theta^(-2c/d_h), c = 0 .. d_h/2-1 (fp64)."""
    c = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * c / head_dim)


def rope(x: np.ndarray, dp: int, head_dim: int, freqs: Optional[np.ndarray] = None,
         theta: float = 10000.0) -> np.ndarray:
    """Rotate every head of x[..., D] by dp positions (rotate-half pairing).

    Pair (c, c + d_h/2) of each head turns by angle dp * w_c:
        x_c'       = x_c cos(phi) - x_{c+h} sin(phi)
        x_{c+h}'   = x_c sin(phi) + x_{c+h} cos(phi)
    dp = 0 returns x unchanged (R(0) is the identity by definition).
    Sec. 2.2 / App. A.2 / App. A.3: the deterministic key re-alignment.
    """
    x = np.asarray(x, dtype=np.float64)
    if dp == 0:
        return x.copy()
    if freqs is None:
        freqs = inv_freq(head_dim, theta)
    h = head_dim // 2
    phi = float(dp) * freqs
    cs, sn = np.cos(phi), np.sin(phi)
    shp = x.shape
    xh = x.reshape(shp[:-1] + (shp[-1] // head_dim, head_dim))
    a, b = xh[..., :h], xh[..., h:]
    out = np.empty_like(xh)
    out[..., :h] = a * cs - b * sn
    out[..., h:] = a * sn + b * cs
    return out.reshape(shp)


# ------------------------------------------------------------------- anchor sets
def anchor_sets(anchor_len: Sequence[int], seq_len: int, gate_len: int = 0) -> Dict:
    """App. A.3 "Variable Segment Lengths".

    gate set A_k   = anchors whose stored length is >= k (k = gate_len, 0 -> S)
    coverage S_cov = min(S, longest stored length)
    correction set = anchors whose length is >= S_cov
    """
    k = seq_len if gate_len == 0 else gate_len
    lens = list(anchor_len)
    gate = [a for a, n in enumerate(lens) if n >= k]
    s_cov = min(seq_len, max(lens)) if lens else 0
    corr = [a for a, n in enumerate(lens) if n >= s_cov] if lens else []
    return dict(k=k, gate=gate, s_cov=s_cov, corr=corr)


# ------------------------------------------------------------------ token scores
def pages_scores(z_can: np.ndarray, A: List[np.ndarray], B: List[np.ndarray]) -> np.ndarray:
    """Mean absolute distance between the (canonical) source rows and each anchor's
    reconstructed base, m[t, a] = (1/D) sum_d |Z[t, d] - (A_a B_a)[t, d]|.
    App. A.3 "Correction Weighting and Positional Alignment"; base from Eq. 7.
    z_can: [T, D]; A[a]: [T, r]; B[a]: [r, D]  ->  [T, len(A)]
    """
    T, D = z_can.shape
    out = np.empty((T, len(A)))
    for j, (a, b) in enumerate(zip(A, B)):
        out[:, j] = np.abs(z_can - a @ b).sum(axis=1) / D
    return out


def cos_scores(z_can: np.ndarray, A: List[np.ndarray], B: List[np.ndarray]) -> np.ndarray:
    """Second scoring mode: c[t, a] = cos(P_a[t], A_a[t]) with P_a = Z B_a^T, the source
    row expressed in anchor a's r-dim basis; 0 when either norm is 0."""
    T = z_can.shape[0]
    out = np.empty((T, len(A)))
    for j, (a, b) in enumerate(zip(A, B)):
        p = z_can @ b.T
        num = (p * a).sum(axis=1)
        den = np.sqrt((p * p).sum(axis=1)) * np.sqrt((a * a).sum(axis=1))
        out[:, j] = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    return out


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=axis, keepdims=True)


def token_weights(scores: np.ndarray, temp: float, mode: int) -> np.ndarray:
    """Eq. 8 weights, token-wise (App. A.3): softmax over anchors of -m/T (distances)
    or of c/T (cosines).  Rows sum to one."""
    if scores.shape[1] == 0:
        return scores.copy()
    z = -scores / temp if mode == PAGES else scores / temp
    return softmax(z, axis=1)


# --------------------------------------------------------------------------- gate
def gate_sums_pages(v: np.ndarray, A: List[np.ndarray], B: List[np.ndarray], k: int) -> np.ndarray:
    """Eq. 9 inner term for one layer: q_a = ||V[:k] - (A_a B_a)[:k]||_F^2."""
    return np.array([((v[:k] - a[:k] @ b) ** 2).sum() for a, b in zip(A, B)])


def gate_sums_cos(v: np.ndarray, A: List[np.ndarray], B: List[np.ndarray], k: int):
    """Second mode, one layer, prefix k: sum_t <P,A>, sum_t |P|^2, sum_t |A|^2."""
    pa, pp, aa = [], [], []
    for a, b in zip(A, B):
        p = v[:k] @ b.T
        pa.append((p * a[:k]).sum())
        pp.append((p * p).sum())
        aa.append((a[:k] * a[:k]).sum())
    return np.array(pa), np.array(pp), np.array(aa)


def normalized_entropy(g: np.ndarray) -> float:
    """Eq. 11: -sum g log2 g / log2 n, with 0 log 0 = 0."""
    n = g.size
    nz = g[g > 0]
    return float(-(nz * np.log2(nz)).sum() / math.log2(n))


def gate_decide_pages(q: np.ndarray, tau: float, temp: float, capacity: int, n_anchors: int):
    """Eq. 9-11 for one gate row.  q: [|A_k|] summed squared distances.
    Returns (d [|A_k|], H or nan, flag bits)."""
    d = np.sqrt(q)
    if n_anchors == 0:
        return d, float("nan"), FLAG_FEW_ANCHORS
    if d.size >= 2:
        g = softmax(-d / temp)
        h = normalized_entropy(g)
    else:
        h = float("nan")
    if capacity == 1:
        return d, h, 0          # App. C.3: capacity-one pool bypasses the gate
    if d.size < 2:
        return d, h, FLAG_FEW_ANCHORS
    return d, h, (FLAG_ENTROPY if h > tau else 0)


def gate_decide_cos(pa: np.ndarray, pp: np.ndarray, aa: np.ndarray, tau: float, capacity: int,
                    n_anchors: int):
    """Second mode: segment cosine per anchor; flagged when the best is below tau."""
    den = np.sqrt(pp * aa)
    c = np.where(den > 0, pa / np.where(den > 0, den, 1.0), 0.0)
    best = float(c.max()) if c.size else float("nan")
    if n_anchors == 0 or c.size == 0:
        return c, best, (0 if (capacity == 1 and n_anchors > 0) else FLAG_FEW_ANCHORS)
    if capacity == 1:
        return c, best, 0
    return c, best, (FLAG_COS_BELOW if best < tau else 0)


# -------------------------------------------------------------------- delta apply
def delta_hat(w: np.ndarray, A: List[np.ndarray], B: List[np.ndarray]) -> np.ndarray:
    """Eq. 8, token-wise: delta[t] = sum_a w[t, a] (A_a[t, :] B_a)."""
    out = None
    for j, (a, b) in enumerate(zip(A, B)):
        term = (w[:, j:j + 1] * a) @ b
        out = term if out is None else out + term
    return out


# ----------------------------------------------------------------------- rounding
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (8 significant bits), ties to even."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])                         # |x| = m 2^e, m in [0.5, 1)
    e = np.maximum(e, -125)                        # below 2^-126: fixed subnormal spacing
    ulp = np.ldexp(1.0, e - 8)
    out[nz] = np.rint(x[nz] / ulp) * ulp
    out[~nz] = x[~nz]
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------- one hop
def _np(t) -> np.ndarray:
    """torch tensor or array -> fp64 numpy (exact upcast)."""
    if hasattr(t, "detach"):
        return t.detach().to("cpu").double().numpy()
    return np.asarray(t, dtype=np.float64)


def layer_factors(data, layer: int, side: str, kind: str, anchors: Sequence[int]):
    """Anchor factors of one layer/side from the packed pool layout."""
    A_all = getattr(data, f"{kind}A_{side}")[layer]
    B_all = getattr(data, f"{kind}B_{side}")[layer]
    A, B = [], []
    for a in anchors:
        o, n = data.anchor_offset[a], data.anchor_len[a]
        A.append(_np(A_all[o:o + n]))
        B.append(_np(B_all[a]))
    return A, B


def correct_layer(data, layer: int, rows: Optional[np.ndarray] = None, want_gate: bool = True):
    """All per-layer quantities of one hop (App. A.3 procedure, one layer).

    rows: token indices whose scores/weights/outputs are wanted (default: all S).
    Returns dict with k_out, v_out (unrounded fp64, for `rows`), w_k, w_v ([rows, N]),
    and the gate sums over the prefix k (always over all k rows).
    """
    sp = data.spec
    S, D, N = sp.seq_len, sp.d_model, sp.n_anchors
    sets = anchor_sets(data.anchor_len, S, sp.gate_len)
    k, gate, s_cov, corr = sets["k"], sets["gate"], sets["s_cov"], sets["corr"]
    fr = inv_freq(sp.head_dim, sp.theta)
    if rows is None:
        rows = np.arange(S)
    rows = np.asarray(rows)
    res = {}
    for side in ("k", "v"):
        z = _np(getattr(data, f"{side}_src")[layer][rows])
        z_can = rope(z, -sp.p_src, sp.head_dim, fr) if side == "k" else z
        base = z if side == "v" else rope(z, sp.shift, sp.head_dim, fr)
        w_full = np.zeros((rows.size, N))
        delta = np.zeros((rows.size, D))
        cov_rows = rows < s_cov
        if corr and cov_rows.any():
            A_b, B_b = layer_factors(data, layer, side, "base", corr)
            A_d, B_d = layer_factors(data, layer, side, "delta", corr)
            r_idx = rows[cov_rows]
            A_b = [a[r_idx] for a in A_b]
            A_d = [a[r_idx] for a in A_d]
            zc = z_can[cov_rows]
            if sp.cap() == 1 and len(corr) == 1:
                w = np.ones((zc.shape[0], 1))
            elif sp.mode == PAGES:
                w = token_weights(pages_scores(zc, A_b, B_b), sp.temp_weight, PAGES)
            else:
                w = token_weights(cos_scores(zc, A_b, B_b), sp.temp_weight, COS_R)
            w_full[np.ix_(cov_rows, corr)] = w
            delta[cov_rows] = delta_hat(w, A_d, B_d)
        if side == "k":
            out = base + rope(delta, sp.p_tgt, sp.head_dim, fr)
        else:
            out = base + delta
        res[f"{side}_out"] = out
        res[f"w_{side}"] = w_full
    if want_gate:
        v = _np(data.v_src[layer][:k])
        A_g, B_g = layer_factors(data, layer, "v", "base", gate)
        A_g = [a[:k] for a in A_g]
        if sp.mode == PAGES:
            res["q"] = gate_sums_pages(v, A_g, B_g, k)
        else:
            res["cos_sums"] = gate_sums_cos(v, A_g, B_g, k)
    res["sets"] = sets
    return res


def gate_all(data, per_layer: List[Dict]):
    """Hop row (Eq. 9 sums over layers) and per-layer rows of the gate.

    Returns dist [1+N_l, N] (nan outside the gate set), stat [1+N_l] (normalised
    entropy, or best cosine in the second mode) and flags [1+N_l] (row 0 = hop).
    """
    sp = data.spec
    N = sp.n_anchors
    L = len(per_layer)
    sets = per_layer[0]["sets"] if per_layer else anchor_sets(data.anchor_len, sp.seq_len, sp.gate_len)
    gate = sets["gate"]
    dist = np.full((1 + L, N), np.nan)
    stat = np.full(1 + L, np.nan)
    flags = np.zeros(1 + L, dtype=np.int32)
    cap = sp.cap()
    if sp.mode == PAGES:
        rows = [np.sum([r["q"] for r in per_layer], axis=0) if gate else np.zeros(0)]
        rows += [r["q"] for r in per_layer]
        for i, q in enumerate(rows):
            d, h, f = gate_decide_pages(np.asarray(q, dtype=np.float64), sp.tau, sp.temp_gate, cap, N)
            dist[i, gate] = d
            stat[i] = h
            flags[i] = f
    else:
        tot = [np.sum([r["cos_sums"][j] for r in per_layer], axis=0) if gate else np.zeros(0)
               for j in range(3)]
        rows = [tot] + [list(r["cos_sums"]) for r in per_layer]
        for i, (pa, pp, aa) in enumerate(rows):
            c, best, f = gate_decide_cos(np.asarray(pa), np.asarray(pp), np.asarray(aa), sp.tau, cap, N)
            dist[i, gate] = c
            stat[i] = best
            flags[i] = f
    return dist, stat, flags


def correct_hop(data, layers: Optional[Sequence[int]] = None, rows=None, round_out: bool = True):
    """Full per-hop correction: re-align, score, gate, weight, apply (Sec. 3.3, App. A.3).

    The output is always produced; flags only tell the caller to prefill densely
    instead (the decision is taken by the caller, Sec. 3.3).  Output rounded to the
    hop's storage dtype (bf16 round-to-nearest-even) unless round_out is False.
    """
    sp = data.spec
    layers = list(range(sp.n_layers)) if layers is None else list(layers)
    per = [correct_layer(data, l, rows=rows) for l in layers]
    k_out = np.stack([p["k_out"] for p in per])
    v_out = np.stack([p["v_out"] for p in per])
    if round_out:
        k_out, v_out = round_to(k_out, sp.dtype), round_to(v_out, sp.dtype)
    dist, stat, flags = gate_all(data, per)
    return dict(k_out=k_out, v_out=v_out, w_k=np.stack([p["w_k"] for p in per]),
                w_v=np.stack([p["w_v"] for p in per]), dist=dist, stat=stat, flags=flags,
                s_cov=per[0]["sets"]["s_cov"] if per else 0,
                q=[p.get("q") for p in per], cos_sums=[p.get("cos_sums") for p in per])


def align_keys(k: np.ndarray, p_from: int, p_to: int, head_dim: int, theta: float = 10000.0):
    """Standalone re-alignment of keys from start position p_from to p_to (Sec. 2.2)."""
    return rope(k, p_to - p_from, head_dim, inv_freq(head_dim, theta))


def apply_delta(k_src, v_src, w_k, w_v, A_k, B_k, A_v, B_v, p_src, p_tgt, head_dim, s_cov,
                theta: float = 10000.0):
    """Explicit-weight apply for one layer (Eq. 8 and Eq. 12 form):
    K_out = R(s) K + R(p_tgt) sum_a w_k A_k,a B_k,a ;  V_out = V + sum_a w_v A_v,a B_v,a,
    with the delta restricted to rows < s_cov."""
    fr = inv_freq(head_dim, theta)
    k_src, v_src = np.asarray(k_src, np.float64), np.asarray(v_src, np.float64)
    dk = np.zeros_like(k_src)
    dv = np.zeros_like(v_src)
    if s_cov > 0 and len(A_k):
        dk[:s_cov] = delta_hat(w_k[:s_cov], [a[:s_cov] for a in A_k], B_k)
        dv[:s_cov] = delta_hat(w_v[:s_cov], [a[:s_cov] for a in A_v], B_v)
    k_out = rope(k_src, p_tgt - p_src, head_dim, fr) + rope(dk, p_tgt, head_dim, fr)
    return k_out, v_src + dv


# -------------------------------------------------------------- factor refresh
def truncated_svd(z: np.ndarray, rank: int):
    """Eq. 7: Z ~ U_r Sigma_r R_r^T = A B with A = U_r Sigma_r, B = R_r^T (fp64 SVD).
    Sign convention: each component is flipped so that the largest-magnitude entry of
    its left singular vector is positive.  Returns A [m, r], B [r, n], sigma [r]."""
    u, s, vt = np.linalg.svd(np.asarray(z, dtype=np.float64), full_matrices=False)
    u, s, vt = u[:, :rank], s[:rank], vt[:rank]
    idx = np.argmax(np.abs(u), axis=0)
    sgn = np.sign(u[idx, np.arange(u.shape[1])])
    sgn[sgn == 0] = 1.0
    u, vt = u * sgn[None, :], vt * sgn[:, None]
    return u * s[None, :], vt, s


def observed_delta(c_target: np.ndarray, c_source: np.ndarray, p_src: int, p_tgt: int,
                   head_dim: int, is_key: bool, theta: float = 10000.0):
    """Eq. 12: Delta = C_j - Align(C_i); stored keys are returned in the canonical
    frame, i.e. rotated back by -p_tgt."""
    fr = inv_freq(head_dim, theta)
    if not is_key:
        return np.asarray(c_target, np.float64) - np.asarray(c_source, np.float64)
    d = np.asarray(c_target, np.float64) - rope(c_source, p_tgt - p_src, head_dim, fr)
    return rope(d, -p_tgt, head_dim, fr)


# ------------------------------------------------------------------ measurements
def effective_rank(sigma: np.ndarray, frac: float = 0.9, squared: bool = True) -> int:
    """Fig. 2 / Fig. 7: minimum rank retaining `frac` of the singular-value energy
    (energy = sum sigma^2 when squared, else sum sigma)."""
    e = np.asarray(sigma, np.float64) ** (2 if squared else 1)
    c = np.cumsum(e) / e.sum()
    return int(np.searchsorted(c, frac - 1e-15) + 1)


def normalized_error(x_hat: np.ndarray, x: np.ndarray) -> float:
    """Fig. 3 / App. A.1: ||x_hat - x||_F / ||x||_F."""
    x = np.asarray(x, np.float64)
    return float(np.linalg.norm(np.asarray(x_hat, np.float64) - x) / np.linalg.norm(x))


def pool_state_bytes(n_layers: int, seq_len: int, d: int, n_anchors: int, n_consumers: int,
                     bytes_per: int = 2, rank: Optional[int] = None, sides: int = 2) -> int:
    """Sec. 3.1 / Eq. 8 memory accounting of an anchor pool: each anchor holds one base
    and one delta per consuming agent, for keys and values in every layer.  Full form:
    O(V N L D); low-rank form O(V N r (L + D))."""
    states = 1 + n_consumers
    per = seq_len * d if rank is None else rank * (seq_len + d)
    return states * sides * n_layers * per * bytes_per * n_anchors
