"""ctypes binding of libkvc (include/kvc.h).  Argument marshalling only: every step of the
correction runs in the library's HIP kernels.  torch tensors supply device memory and the
current HIP stream; a missing library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvc.so")

KVC_F32, KVC_BF16 = 0, 1
SCORE_PAGES, SCORE_COS_R = 0, 1
CALL_MATCH, CALL_APPLY, CALL_CORRECT = 1, 2, 3
FLAG_ENTROPY, FLAG_FEW_ANCHORS, FLAG_COS_BELOW, FLAG_PRED_FLAGGED = 1, 2, 4, 8
MAX_ANCHORS = 64

STATUS = {0: "KVC_OK", 1: "KVC_E_NULL", 2: "KVC_E_SHAPE", 3: "KVC_E_DTYPE", 4: "KVC_E_ALIGN",
          5: "KVC_E_ALIAS", 6: "KVC_E_WORKSPACE", 7: "KVC_E_HIP", 8: "KVC_E_PARAM",
          9: "KVC_E_UNSUPPORTED"}

EXPORTS = ["kvc_abi_version", "kvc_status_str", "kvc_last_error", "kvc_workspace_size",
           "kvc_align_rope", "kvc_match_anchors", "kvc_apply_lowrank_delta", "kvc_correct_hop",
           "kvc_correct_hop_noalloc",
           "kvc_correct_hops_batched", "kvc_hops_batched_workspace_size", "kvc_svd_workspace_size", "kvc_anchor_refresh_svd",
           "kvc_peak_copy", "kvc_peak_mfma_bf16", "kvc_peak_lds_read", "kvc_peak_valu",
           "kvc_observed_delta", "kvc_pool_state_init", "kvc_pool_record_hop", "kvc_pool_view",
           "kvc_pool_insert_workspace_size", "kvc_pool_insert"]
POOL_EVICT_WINDOW = 5


class KvcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Shape(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("seq_len", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32)]


class Rope(C.Structure):
    _fields_ = [("theta", C.c_double), ("inv_freq", C.POINTER(C.c_double))]


class Pool(C.Structure):
    _fields_ = [("n_anchors", C.c_int32), ("rank_base", C.c_int32), ("rank_delta", C.c_int32),
                ("capacity", C.c_int32), ("anchor_len", C.POINTER(C.c_int32)), ("dtype", C.c_int32),
                ("baseA_k", C.c_void_p), ("baseB_k", C.c_void_p), ("baseA_v", C.c_void_p),
                ("baseB_v", C.c_void_p), ("deltaA_k", C.c_void_p), ("deltaB_k", C.c_void_p),
                ("deltaA_v", C.c_void_p), ("deltaB_v", C.c_void_p), ("slot_rows", C.c_int32),
                ("pad_", C.c_int32), ("live", C.POINTER(C.c_uint8))]


class PoolStateC(C.Structure):
    _fields_ = [("capacity", C.c_int32), ("n_held", C.c_int32), ("clock", C.c_int64),
                ("stamp", C.c_int64 * MAX_ANCHORS), ("uses", C.c_int64 * MAX_ANCHORS),
                ("len", C.c_int32 * MAX_ANCHORS), ("consumer", C.c_int32 * MAX_ANCHORS)]


TRACE_MAX = 64
KERNEL_NAMES = {1: "pack_base", 3: "score_cos_mfma", 4: "score_generic", 5: "gate_finalize", 6: "softmax",
                7: "pack_delta", 8: "fused_hop", 9: "apply_generic", 10: "split_score", 11: "split_apply",
                12: "split_weights", 13: "score_cos_gemm", 14: "pack_cos"}


class Trace(C.Structure):
    _fields_ = [("capacity", C.c_int32), ("count", C.c_int32), ("kernel_id", C.c_int32 * TRACE_MAX),
                ("start", C.c_void_p * TRACE_MAX), ("stop", C.c_void_p * TRACE_MAX)]


class Params(C.Structure):
    _fields_ = [("tau", C.c_double), ("temp_gate", C.c_double), ("temp_weight", C.c_double),
                ("gate_len", C.c_int32), ("mode", C.c_int32), ("options", C.c_int32), ("pad_", C.c_int32),
                ("trace", C.POINTER(Trace))]


class MatchOut(C.Structure):
    _fields_ = [("dist", C.c_void_p), ("stat", C.c_void_p), ("flags", C.c_void_p),
                ("w_k", C.c_void_p), ("w_v", C.c_void_p), ("s_cov", C.POINTER(C.c_int32))]


class HopDesc(C.Structure):
    _fields_ = [("k_src", C.c_void_p), ("v_src", C.c_void_p), ("k_out", C.c_void_p),
                ("v_out", C.c_void_p), ("p_src", C.c_int64), ("p_tgt", C.c_int64),
                ("chain_prev", C.c_int32), ("pad_", C.c_int32), ("pool", Pool), ("out", MatchOut)]


_lib = None


def lib(path: Optional[str] = None):
    """Load libkvc.so (built in-tree by rank_kv_cache_layer_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libkvc.so not found at {p}: build it with `python -m rank_kv_cache_layer_amd.build`")
    L = C.CDLL(p)
    L.kvc_abi_version.restype = C.c_int32
    L.kvc_status_str.restype = C.c_char_p
    L.kvc_status_str.argtypes = [C.c_int]
    L.kvc_last_error.restype = C.c_char_p
    L.kvc_workspace_size.restype = C.c_size_t
    L.kvc_workspace_size.argtypes = [C.c_int32, Shape, C.POINTER(Pool), C.POINTER(Params)]
    L.kvc_align_rope.restype = C.c_int
    L.kvc_align_rope.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, Shape, C.c_int64, C.c_int64,
                                 C.POINTER(Rope), C.c_void_p]
    L.kvc_match_anchors.restype = C.c_int
    L.kvc_match_anchors.argtypes = [C.c_void_p, C.c_void_p, C.c_int, Shape, C.c_int64, C.POINTER(Rope),
                                    C.POINTER(Pool), C.POINTER(Params), C.POINTER(MatchOut), C.c_void_p,
                                    C.c_size_t, C.c_void_p]
    L.kvc_apply_lowrank_delta.restype = C.c_int
    L.kvc_apply_lowrank_delta.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, Shape,
                                          C.c_int64, C.c_int64, C.POINTER(Rope), C.POINTER(Pool), C.c_void_p,
                                          C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]
    L.kvc_correct_hop.restype = C.c_int
    L.kvc_correct_hop.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, Shape, C.c_int64,
                                  C.c_int64, C.POINTER(Rope), C.POINTER(Pool), C.POINTER(Params),
                                  C.POINTER(MatchOut), C.c_void_p, C.c_size_t, C.c_void_p]
    L.kvc_correct_hop_noalloc.restype = C.c_int
    L.kvc_correct_hop_noalloc.argtypes = [C.c_void_p] * 4 + [C.c_int, Shape, C.c_int64, C.c_int64, C.POINTER(Rope),
                                                           C.POINTER(Pool), C.POINTER(Params), C.POINTER(MatchOut),
                                                           C.c_void_p]
    L.kvc_hops_batched_workspace_size.restype = C.c_size_t
    L.kvc_hops_batched_workspace_size.argtypes = [C.POINTER(HopDesc), C.c_int32, C.c_int, Shape, C.POINTER(Params)]
    L.kvc_correct_hops_batched.restype = C.c_int
    L.kvc_correct_hops_batched.argtypes = [C.POINTER(HopDesc), C.c_int32, C.c_int, Shape, C.POINTER(Rope),
                                           C.POINTER(Params), C.c_void_p, C.c_size_t, C.c_void_p]
    L.kvc_svd_workspace_size.restype = C.c_size_t
    L.kvc_svd_workspace_size.argtypes = [C.c_int32] * 5
    L.kvc_anchor_refresh_svd.restype = C.c_int
    L.kvc_anchor_refresh_svd.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                         C.c_void_p, C.c_int, C.c_void_p, C.c_int32, C.c_int32, C.c_uint64,
                                         C.c_void_p, C.c_size_t, C.c_void_p]
    L.kvc_observed_delta.restype = C.c_int
    L.kvc_observed_delta.argtypes = [C.c_void_p] * 4 + [C.c_int, Shape, C.c_int64, C.c_int64, C.POINTER(Rope)] + \
        [C.c_void_p] * 5
    L.kvc_pool_state_init.restype = C.c_int
    L.kvc_pool_state_init.argtypes = [C.POINTER(PoolStateC), C.c_int32]
    L.kvc_pool_record_hop.restype = C.c_int
    L.kvc_pool_record_hop.argtypes = [C.POINTER(PoolStateC), C.c_int32, C.c_int32, C.c_int32,
                                      C.POINTER(C.c_int32), C.POINTER(C.c_int32)]
    L.kvc_pool_view.restype = C.c_int32
    L.kvc_pool_view.argtypes = [C.POINTER(PoolStateC), C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_uint8)]
    L.kvc_pool_insert_workspace_size.restype = C.c_size_t
    L.kvc_pool_insert_workspace_size.argtypes = [Shape, C.POINTER(Pool), C.c_int32]
    L.kvc_pool_insert.restype = C.c_int
    L.kvc_pool_insert.argtypes = [C.c_void_p] * 4 + [Shape, C.c_int64, C.c_int64, C.POINTER(Rope), C.POINTER(Pool),
                                                     C.c_int32, C.c_int32, C.c_int32, C.c_uint64, C.c_void_p,
                                                     C.c_size_t, C.c_void_p]
    L.kvc_peak_copy.restype = C.c_int
    L.kvc_peak_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    for f in (L.kvc_peak_mfma_bf16, L.kvc_peak_lds_read, L.kvc_peak_valu):
        f.restype = C.c_int
        f.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise KvcError(status, lib().kvc_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KVC_F32
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def shape_of(n_layers, seq_len, n_kv_heads, head_dim) -> Shape:
    return Shape(n_layers, seq_len, n_kv_heads, head_dim)


def rope_of(theta: float = 10000.0, inv_freq: Optional[Sequence[float]] = None):
    if inv_freq is None:
        return Rope(theta, None), None
    arr = (C.c_double * len(inv_freq))(*inv_freq)
    return Rope(theta, C.cast(arr, C.POINTER(C.c_double))), arr


@dataclass
class PoolTensors:
    """Device tensors of one anchor pool in the library's packed layout."""
    anchor_len: Sequence[int]
    rank_base: int
    rank_delta: int
    baseA_k: torch.Tensor
    baseB_k: torch.Tensor
    baseA_v: torch.Tensor
    baseB_v: torch.Tensor
    deltaA_k: torch.Tensor
    deltaB_k: torch.Tensor
    deltaA_v: torch.Tensor
    deltaB_v: torch.Tensor
    capacity: int = 0
    slot_rows: int = 0                      # > 0: fixed-capacity arena slots
    live: Optional[Sequence[int]] = None    # per-anchor mask, None = all live

    def c(self):
        n = len(self.anchor_len)
        lens = (C.c_int32 * max(n, 1))(*self.anchor_len)
        live = None
        if self.live is not None:
            live = (C.c_uint8 * max(n, 1))(*[1 if x else 0 for x in self.live])
        p = Pool(n, self.rank_base, self.rank_delta, self.capacity, C.cast(lens, C.POINTER(C.c_int32)),
                 _dt(self.baseA_k), _ptr(self.baseA_k), _ptr(self.baseB_k), _ptr(self.baseA_v),
                 _ptr(self.baseB_v), _ptr(self.deltaA_k), _ptr(self.deltaB_k), _ptr(self.deltaA_v),
                 _ptr(self.deltaB_v), self.slot_rows, 0,
                 C.cast(live, C.POINTER(C.c_uint8)) if live is not None else None)
        return p, (lens, live)


def params_of(tau=0.3, temp_gate=1.0, temp_weight=0.1, gate_len=0, mode=SCORE_PAGES, options=0,
              trace: Optional["KernelTrace"] = None) -> Params:
    return Params(tau, temp_gate, temp_weight, gate_len, mode, options, 0,
                  C.pointer(trace.c) if trace is not None else None)


class KernelTrace:
    """Caller-owned hipEvent pairs the library records around each kernel it launches."""

    def __init__(self, capacity: int = TRACE_MAX):
        # by SONAME, so the HIP runtime torch already loaded is reused (one runtime per process)
        self._hip = C.CDLL("libamdhip64.so.7")
        maps = open("/proc/self/maps").read()
        copies = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
        if len(copies) != 1:
            raise RuntimeError(f"more than one HIP runtime loaded: {sorted(copies)}")
        self.c = Trace()
        self.c.capacity = capacity
        for i in range(capacity):
            for arr in (self.c.start, self.c.stop):
                ev = C.c_void_p()
                if self._hip.hipEventCreate(C.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = ev.value

    def reset(self):
        self.c.count = 0

    def results(self):
        """[(kernel name, milliseconds)] of the traced launches; call after a stream sync."""
        out = []
        for i in range(self.c.count):
            ms = C.c_float()
            if self._hip.hipEventElapsedTime(C.byref(ms), C.c_void_p(self.c.start[i]), C.c_void_p(self.c.stop[i])):
                raise RuntimeError("hipEventElapsedTime failed")
            out.append((KERNEL_NAMES.get(self.c.kernel_id[i], str(self.c.kernel_id[i])), ms.value))
        return out

    def close(self):
        for i in range(self.c.capacity):
            for arr in (self.c.start, self.c.stop):
                if arr[i]:
                    self._hip.hipEventDestroy(C.c_void_p(arr[i]))
                    arr[i] = None


@dataclass
class MatchResult:
    dist: torch.Tensor     # float64 [1+N_l, N]
    stat: torch.Tensor     # float64 [1+N_l]
    flags: torch.Tensor    # int32 [1+N_l]
    w_k: Optional[torch.Tensor]
    w_v: Optional[torch.Tensor]
    s_cov: int


def alloc_match(n_layers, seq_len, n_anchors, device, want_weights=True) -> MatchResult:
    n = max(n_anchors, 1)
    return MatchResult(
        dist=torch.empty((1 + n_layers, n), dtype=torch.float64, device=device),
        stat=torch.empty((1 + n_layers,), dtype=torch.float64, device=device),
        flags=torch.empty((1 + n_layers,), dtype=torch.int32, device=device),
        w_k=torch.empty((n_layers, seq_len, n), dtype=torch.float32, device=device) if want_weights else None,
        w_v=torch.empty((n_layers, seq_len, n), dtype=torch.float32, device=device) if want_weights else None,
        s_cov=0)


def _mo(m: MatchResult):
    sc = C.c_int32(0)
    return MatchOut(_ptr(m.dist), _ptr(m.stat), _ptr(m.flags), _ptr(m.w_k), _ptr(m.w_v), C.pointer(sc)), sc


def workspace_size(call, shape: Shape, pool: PoolTensors, params: Optional[Params] = None) -> int:
    p, _keep = pool.c()
    return int(lib().kvc_workspace_size(call, shape, C.byref(p), C.byref(params) if params is not None else None))


def _ws(nbytes: int, device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return None
    if ws is not None:
        return ws
    return torch.empty((nbytes,), dtype=torch.uint8, device=device)


def align_rope(k_in: torch.Tensor, k_out: torch.Tensor, shape: Shape, pos_from: int, pos_to: int,
               theta: float = 10000.0, inv_freq=None, stream=None):
    rope, _keep = rope_of(theta, inv_freq)
    _check(lib().kvc_align_rope(_ptr(k_in), _ptr(k_out), _dt(k_in), _dt(k_out), shape, pos_from, pos_to,
                                C.byref(rope), _stream(stream)))


def match_anchors(k_src, v_src, shape: Shape, p_src: int, pool: PoolTensors, params: Params,
                  out: Optional[MatchResult] = None, theta=10000.0, workspace=None, stream=None) -> MatchResult:
    L = lib()
    p, _keep = pool.c()
    if out is None:
        out = alloc_match(shape.n_layers, shape.seq_len, len(pool.anchor_len), k_src.device)
    need = L.kvc_workspace_size(CALL_MATCH, shape, C.byref(p), C.byref(params))
    ws = _ws(need, k_src.device, workspace)
    mo, sc = _mo(out)
    rope, _k2 = rope_of(theta)
    _check(L.kvc_match_anchors(_ptr(k_src), _ptr(v_src), _dt(k_src), shape, p_src, C.byref(rope), C.byref(p),
                               C.byref(params), C.byref(mo), _ptr(ws), ws.numel() if ws is not None else 0,
                               _stream(stream)))
    out.s_cov = sc.value
    return out


def apply_lowrank_delta(k_src, v_src, k_out, v_out, shape: Shape, p_src: int, p_tgt: int, pool: PoolTensors,
                        w_k, w_v, s_cov: int, theta=10000.0, workspace=None, stream=None):
    L = lib()
    p, _keep = pool.c()
    need = L.kvc_workspace_size(CALL_APPLY, shape, C.byref(p), None)
    ws = _ws(need, k_src.device, workspace)
    rope, _k2 = rope_of(theta)
    _check(L.kvc_apply_lowrank_delta(_ptr(k_src), _ptr(v_src), _ptr(k_out), _ptr(v_out), _dt(k_src), shape,
                                     p_src, p_tgt, C.byref(rope), C.byref(p), _ptr(w_k), _ptr(w_v), s_cov,
                                     _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def correct_hop(k_src, v_src, k_out, v_out, shape: Shape, p_src: int, p_tgt: int, pool: PoolTensors,
                params: Params, out: Optional[MatchResult] = None, theta=10000.0, workspace=None,
                stream=None, want_weights=False) -> MatchResult:
    L = lib()
    p, _keep = pool.c()
    if out is None:
        out = alloc_match(shape.n_layers, shape.seq_len, len(pool.anchor_len), k_src.device, want_weights)
    need = L.kvc_workspace_size(CALL_CORRECT, shape, C.byref(p), C.byref(params))
    ws = _ws(need, k_src.device, workspace)
    mo, sc = _mo(out)
    rope, _k2 = rope_of(theta)
    _check(L.kvc_correct_hop(_ptr(k_src), _ptr(v_src), _ptr(k_out), _ptr(v_out), _dt(k_src), shape, p_src, p_tgt,
                             C.byref(rope), C.byref(p), C.byref(params), C.byref(mo), _ptr(ws),
                             ws.numel() if ws is not None else 0, _stream(stream)))
    out.s_cov = sc.value
    return out


NOALLOC_SCRATCH_BYTES = 384 << 20


def correct_hop_noalloc(k_src, v_src, k_out, v_out, shape: Shape, p_src: int, p_tgt: int, pool: PoolTensors,
                        params: Params, out: MatchResult, theta=10000.0, stream=None) -> MatchResult:
    """kvc_correct_hop_noalloc: the whole hop with the library's own per-GPU scratch (no workspace,
    no device allocation); `out` must be preallocated (alloc_match)."""
    L = lib()
    p, _keep = pool.c()
    mo, sc = _mo(out)
    rope, _k2 = rope_of(theta)
    _check(L.kvc_correct_hop_noalloc(_ptr(k_src), _ptr(v_src), _ptr(k_out), _ptr(v_out), _dt(k_src), shape, p_src,
                                     p_tgt, C.byref(rope), C.byref(p), C.byref(params), C.byref(mo),
                                     _stream(stream)))
    out.s_cov = sc.value
    return out


def correct_hop_workspace(shape: Shape, pool: PoolTensors, params: Params) -> int:
    p, _keep = pool.c()
    return int(lib().kvc_workspace_size(CALL_CORRECT, shape, C.byref(p), C.byref(params)))


@dataclass
class Hop:
    k_src: Optional[torch.Tensor]
    v_src: Optional[torch.Tensor]
    k_out: torch.Tensor
    v_out: torch.Tensor
    p_src: int
    p_tgt: int
    chain_prev: int
    pool: PoolTensors
    out: MatchResult


def hops_batched_workspace(hops: Sequence[Hop], shape: Shape, params: Params) -> int:
    """Workspace bytes kvc_correct_hops_batched needs to run each chain level as one batch."""
    n = len(hops)
    arr = (HopDesc * max(n, 1))()
    keep = []
    for i, h in enumerate(hops):
        p, lens = h.pool.c()
        keep.append(lens)
        arr[i] = HopDesc(_ptr(h.k_src), _ptr(h.v_src), _ptr(h.k_out), _ptr(h.v_out), h.p_src, h.p_tgt,
                         h.chain_prev, 0, p, MatchOut())
    return int(lib().kvc_hops_batched_workspace_size(arr, n, _dt(hops[0].k_out), shape, C.byref(params)))


def correct_hops_batched(hops: Sequence[Hop], shape: Shape, params: Params, theta=10000.0, workspace=None,
                         stream=None, one_at_a_time: bool = False):
    L = lib()
    n = len(hops)
    arr = (HopDesc * max(n, 1))()
    keep = []
    for i, h in enumerate(hops):
        p, lens = h.pool.c()
        keep.append(lens)
        mo = MatchOut(_ptr(h.out.dist), _ptr(h.out.stat), _ptr(h.out.flags), _ptr(h.out.w_k), _ptr(h.out.w_v),
                      None)
        arr[i] = HopDesc(_ptr(h.k_src), _ptr(h.v_src), _ptr(h.k_out), _ptr(h.v_out), h.p_src, h.p_tgt,
                         h.chain_prev, 0, p, mo)
    dt = _dt(hops[0].k_out)
    if one_at_a_time:   # the largest one-hop workspace: the library then runs the hops one by one
        need = max(int(L.kvc_workspace_size(CALL_CORRECT, shape, C.byref(arr[i].pool), C.byref(params)))
                   for i in range(n))
    else:
        need = int(L.kvc_hops_batched_workspace_size(arr, n, dt, shape, C.byref(params)))
    dev = hops[0].k_out.device
    ws = _ws(need, dev, workspace)
    rope, _k2 = rope_of(theta)
    # one hop at a time: announce only the one-hop size, so the library does not batch the levels
    nbytes = (min(ws.numel(), need) if one_at_a_time else ws.numel()) if ws is not None else 0
    _check(L.kvc_correct_hops_batched(arr, n, dt, shape, C.byref(rope), C.byref(params), _ptr(ws), nbytes,
                                      _stream(stream)))


def svd_workspace_size(n_mats, rows, cols, rank, oversample) -> int:
    return int(lib().kvc_svd_workspace_size(n_mats, rows, cols, rank, oversample))


def anchor_refresh_svd(z: torch.Tensor, rank: int, out_dtype=torch.float32, oversample: int = 16,
                       power_iters: int = 2, seed: int = 0, workspace=None, stream=None, a_out=None, b_out=None,
                       sigma_out=None):
    """z: float32 [n_mats, rows, cols] -> (A [n, rows, rank], B [n, rank, cols], sigma [n, rank]);
    a_out / b_out / sigma_out: optional preallocated results (their dtype then sets out_dtype)."""
    L = lib()
    n, m, k = z.shape
    if a_out is not None:
        out_dtype = a_out.dtype
    a = a_out if a_out is not None else torch.empty((n, m, rank), dtype=out_dtype, device=z.device)
    b = b_out if b_out is not None else torch.empty((n, rank, k), dtype=out_dtype, device=z.device)
    s = sigma_out if sigma_out is not None else torch.empty((n, rank), dtype=torch.float32, device=z.device)
    assert a.shape == (n, m, rank) and b.shape == (n, rank, k) and a.dtype == b.dtype and s.shape == (n, rank)
    need = L.kvc_svd_workspace_size(n, m, k, rank, oversample)
    ws = _ws(need, z.device, workspace)
    _check(L.kvc_anchor_refresh_svd(_ptr(z), n, m, k, rank, _ptr(a), _ptr(b), _dt(a), _ptr(s), oversample,
                                    power_iters, seed, _ptr(ws), ws.numel() if ws is not None else 0,
                                    _stream(stream)))
    return a, b, s


def peak_copy(dst: torch.Tensor, src: torch.Tensor, stream=None):
    """Measurement: dst <- src with the library's streaming copy kernel (same byte size)."""
    nb = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nb
    _check(lib().kvc_peak_copy(_ptr(dst), _ptr(src), nb, _stream(stream)))


def peak_loop(kind: str, sink: torch.Tensor, n_blocks: int, iters: int, stream=None):
    """Measurement loops: kind in {"mfma", "lds", "valu"}; sink holds n_blocks * 256 words."""
    assert sink.numel() >= n_blocks * 256 and sink.element_size() == 4
    f = {"mfma": lib().kvc_peak_mfma_bf16, "lds": lib().kvc_peak_lds_read, "valu": lib().kvc_peak_valu}[kind]
    _check(f(_ptr(sink), n_blocks, iters, _stream(stream)))


def pool_from(data, device) -> PoolTensors:
    """Device copy of a workload pool (rank_kv_cache_layer_amd.workload.HopData)."""
    t = lambda x: x.to(device, non_blocking=True).contiguous()
    sp = data.spec
    return PoolTensors(anchor_len=list(data.anchor_len), rank_base=sp.rank_base, rank_delta=sp.rank_delta,
                       baseA_k=t(data.baseA_k), baseB_k=t(data.baseB_k), baseA_v=t(data.baseA_v),
                       baseB_v=t(data.baseB_v), deltaA_k=t(data.deltaA_k), deltaB_k=t(data.deltaB_k),
                       deltaA_v=t(data.deltaA_v), deltaB_v=t(data.deltaB_v), capacity=sp.capacity)


# ------------------------------------------------------------------ pool updates (App. A.3)
def observed_delta(k_src, v_src, k_tgt, v_tgt, shape: Shape, p_src: int, p_tgt: int, k_base=None, v_base=None,
                   k_delta=None, v_delta=None, theta=10000.0, stream=None):
    """Eq. 12 in fp32 (kvc_observed_delta): canonical source and observed correction per side."""
    rope, _keep = rope_of(theta)
    t = next(x for x in (k_src, v_src, k_tgt, v_tgt) if x is not None)
    _check(lib().kvc_observed_delta(_ptr(k_src), _ptr(v_src), _ptr(k_tgt), _ptr(v_tgt), _dt(t), shape, p_src, p_tgt,
                                    C.byref(rope), _ptr(k_base), _ptr(v_base), _ptr(k_delta), _ptr(v_delta),
                                    _stream(stream)))


class PoolState:
    """Host bookkeeping of one slot's pool (kvc_pool_state): insert on fallback, LFU eviction."""

    def __init__(self, capacity: int):
        self.c = PoolStateC()
        _check(lib().kvc_pool_state_init(C.byref(self.c), capacity))

    def record_hop(self, consumer: int, seg_len: int, flagged: bool):
        slot, ev = C.c_int32(), C.c_int32()
        _check(lib().kvc_pool_record_hop(C.byref(self.c), consumer, seg_len, 1 if flagged else 0, C.byref(slot),
                                         C.byref(ev)))
        return slot.value, ev.value

    def view(self, consumer: int):
        n = self.c.capacity
        lens = (C.c_int32 * MAX_ANCHORS)()
        live = (C.c_uint8 * MAX_ANCHORS)()
        k = lib().kvc_pool_view(C.byref(self.c), consumer, lens, live)
        if k < 0:
            raise KvcError(8, "pool view: bad arguments")
        return list(lens[:n]), [int(x) for x in live[:n]]


def pool_insert_workspace(shape: Shape, arena: PoolTensors, oversample: int) -> int:
    p, _keep = arena.c()
    return int(lib().kvc_pool_insert_workspace_size(shape, C.byref(p), oversample))


def pool_insert(k_src, v_src, k_tgt, v_tgt, shape: Shape, p_src: int, p_tgt: int, arena: PoolTensors, slot: int,
                oversample: int = 16, power_iters: int = 2, seed: int = 0, theta=10000.0, workspace=None,
                stream=None):
    """Fills arena slot `slot` from a dense fallback (kvc_pool_insert)."""
    rope, _k1 = rope_of(theta)
    p, _k2 = arena.c()
    need = int(lib().kvc_pool_insert_workspace_size(shape, C.byref(p), oversample))
    ws = _ws(need, k_src.device, workspace)
    _check(lib().kvc_pool_insert(_ptr(k_src), _ptr(v_src), _ptr(k_tgt), _ptr(v_tgt), shape, p_src, p_tgt,
                                 C.byref(rope), C.byref(p), slot, oversample, power_iters, seed, _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream)))
