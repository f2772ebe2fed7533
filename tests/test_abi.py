"""CPU checks of the C ABI: the library loads without a GPU, exports every symbol the header
declares, and rejects invalid requests on the host before any launch."""
import ctypes as C
import os
import re

import pytest

from rank_kv_cache_layer_amd import kvc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    inc = os.path.join(ROOT, "include")
    txt = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    f = header_functions()
    for name in ("kvc_align_rope", "kvc_match_anchors", "kvc_apply_lowrank_delta", "kvc_anchor_refresh_svd",
                 "kvc_correct_hop", "kvc_correct_hops_batched", "kvc_workspace_size"):
        assert name in f


def test_library_exports_every_declared_symbol():
    L = kvc.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    assert sorted(header_functions()) == sorted(kvc.EXPORTS)
    assert L.kvc_abi_version() == 3


def test_trace_kernel_ids_named_by_the_binding():
    # every kernel id the header defines for the optional trace has a name in the binding, and
    # the binding names no id the header lacks
    txt = open(os.path.join(ROOT, "include", "kvc.h")).read()
    ids = {int(v) for v in re.findall(r"#define KVC_K_[A-Z0-9_]+\s+(\d+)", txt)}
    assert ids and ids == set(kvc.KERNEL_NAMES)
    assert len(set(kvc.KERNEL_NAMES.values())) == len(kvc.KERNEL_NAMES)


def test_status_strings():
    L = kvc.lib()
    for s in range(10):
        assert L.kvc_status_str(s)
    assert L.kvc_status_str(5) == b"output aliases input"


FAKE = 0x10000000  # never dereferenced: every call below fails validation first
SH = kvc.shape_of(2, 64, 2, 64)


def _rope():
    r, _ = kvc.rope_of(10000.0)
    return r


def _pool(n=2, r=8, dtype=kvc.KVC_BF16, lens=None, base=FAKE):
    lens = lens or [64] * n
    arr = (C.c_int32 * max(n, 1))(*lens)
    p = kvc.Pool(n, r, r, 0, C.cast(arr, C.POINTER(C.c_int32)), dtype, *([base] * 8))
    return p, arr


def _out():
    return kvc.MatchOut(FAKE, FAKE, FAKE, None, None, None)


def _err():
    return kvc.lib().kvc_last_error().decode()


def _align(**kw):
    a = dict(k_in=FAKE, k_out=FAKE + 1 << 20, in_t=kvc.KVC_BF16, out_t=kvc.KVC_BF16, shape=SH, p0=0, p1=5)
    a.update(kw)
    r = _rope()
    return kvc.lib().kvc_align_rope(a["k_in"], a["k_out"], a["in_t"], a["out_t"], a["shape"], a["p0"], a["p1"],
                                    C.byref(r), None)


def test_align_validation():
    assert _align(k_in=None) == 1
    assert _align(k_in=FAKE + 2) == 4
    assert _align(shape=kvc.shape_of(0, 64, 2, 64)) == 2
    assert _align(shape=kvc.shape_of(1, 64, 2, 63)) == 2
    assert _align(shape=kvc.shape_of(1, 64, 2, 512)) == 2
    assert _align(in_t=7) == 3
    assert _align(k_out=FAKE + 64) == 5                      # partial overlap
    assert _align(k_out=FAKE, out_t=kvc.KVC_F32) == 5        # in place needs equal dtypes
    assert "overlap" in _err() or "in-place" in _err()
    r = kvc.Rope(-1.0, None)
    assert kvc.lib().kvc_align_rope(FAKE, FAKE + (1 << 20), 1, 1, SH, 0, 3, C.byref(r), None) == 8
    assert kvc.lib().kvc_align_rope(FAKE, FAKE + (1 << 20), 1, 1, SH, 0, 3, None, None) == 1


def _correct(pool=None, prm=None, out="x", ws=None, wsb=0, **kw):
    L = kvc.lib()
    p, arr = pool if pool is not None else _pool()
    prm = prm or kvc.params_of()
    o = _out() if out == "x" else out
    a = dict(k=FAKE, v=FAKE + (1 << 24), ko=FAKE + (2 << 24), vo=FAKE + (3 << 24), dt=kvc.KVC_BF16, sh=SH)
    a.update(kw)
    return L.kvc_correct_hop(a["k"], a["v"], a["ko"], a["vo"], a["dt"], a["sh"], 0, 5, C.byref(_rope()),
                             C.byref(p), C.byref(prm), C.byref(o) if o is not None else None, ws, wsb, None)


def test_correct_hop_validation_codes():
    assert _correct(k=None) == 1
    assert _correct(out=None) == 1
    assert _correct(out=kvc.MatchOut(None, FAKE, FAKE, None, None, None)) == 1
    assert _correct(ko=FAKE + 8) == 4
    assert _correct(ko=FAKE) == 5                                  # output aliases the source
    assert _correct(vo=FAKE + (2 << 24)) == 5                      # k_out overlaps v_out
    assert _correct(dt=kvc.KVC_F32) == 3                           # pool dtype differs
    assert _correct(sh=kvc.shape_of(1, 0, 1, 64)) == 2
    assert _correct(prm=kvc.params_of(temp_gate=0.0)) == 8
    assert _correct(prm=kvc.params_of(temp_weight=-1.0)) == 8
    assert _correct(prm=kvc.params_of(gate_len=65)) == 8
    assert _correct(prm=kvc.params_of(mode=3)) == 8
    assert _correct(prm=kvc.params_of(options=4)) == 8
    assert _correct(prm=kvc.params_of(tau=float("nan"))) == 8
    assert _correct(pool=_pool(n=65)) == 2
    assert _correct(pool=_pool(n=2, lens=[64, 0])) == 2
    assert _correct(pool=_pool(base=FAKE + 4)) == 4
    p, arr = _pool()
    p.capacity = 1
    assert _correct(pool=(p, arr)) == 8                            # capacity below n_anchors
    assert _correct() == 6                                         # no workspace
    assert "workspace" in _err()


def test_workspace_size_query():
    L = kvc.lib()
    p, arr = _pool()
    prm = kvc.params_of()
    n = L.kvc_workspace_size(kvc.CALL_CORRECT, kvc.shape_of(32, 4096, 8, 128), C.byref(p), C.byref(prm))
    assert n > 2 * 32 * 4096 * 2 * 4
    assert L.kvc_workspace_size(99, SH, C.byref(p), C.byref(prm)) == 0
    assert L.kvc_workspace_size(kvc.CALL_MATCH, kvc.shape_of(0, 1, 1, 2), C.byref(p), C.byref(prm)) == 0


def test_apply_and_match_validation():
    L = kvc.lib()
    p, arr = _pool()
    r = _rope()
    assert L.kvc_apply_lowrank_delta(FAKE, FAKE + (1 << 24), FAKE, FAKE + (3 << 24), 1, SH, 0, 5, C.byref(r),
                                     C.byref(p), FAKE, FAKE, 64, None, 0, None) == 5
    assert L.kvc_apply_lowrank_delta(FAKE, FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24), 1, SH, 0, 5,
                                     C.byref(r), C.byref(p), None, FAKE, 64, None, 0, None) == 1
    assert L.kvc_apply_lowrank_delta(FAKE, FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24), 1, SH, 0, 5,
                                     C.byref(r), C.byref(p), FAKE, FAKE, 65, None, 0, None) == 8
    o = _out()
    prm = kvc.params_of()
    assert L.kvc_match_anchors(None, FAKE, 1, SH, 0, C.byref(r), C.byref(p), C.byref(prm), C.byref(o), None, 0,
                               None) == 1
    o2 = kvc.MatchOut(FAKE, FAKE, FAKE, FAKE + 4, None, None)
    assert L.kvc_match_anchors(FAKE, FAKE, 1, SH, 0, C.byref(r), C.byref(p), C.byref(prm), C.byref(o2), None, 0,
                               None) == 4


def test_batched_validation_before_launch():
    L = kvc.lib()
    p, arr = _pool()
    hop = kvc.HopDesc(FAKE, FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24), 0, 5, 0, 0, p, _out())
    hops = (kvc.HopDesc * 1)(hop)
    prm = kvc.params_of()
    assert L.kvc_correct_hops_batched(hops, 1, 1, SH, C.byref(_rope()), C.byref(prm), None, 0, None) == 8
    assert "chain_prev" in _err()
    assert L.kvc_correct_hops_batched(None, 1, 1, SH, C.byref(_rope()), C.byref(prm), None, 0, None) == 1
    assert L.kvc_correct_hops_batched(hops, 0, 1, SH, C.byref(_rope()), C.byref(prm), None, 0, None) == 0


def test_svd_validation():
    L = kvc.lib()
    assert L.kvc_anchor_refresh_svd(None, 1, 64, 64, 8, FAKE, FAKE, 0, FAKE, 4, 2, 0, FAKE, 1 << 30, None) == 1
    assert L.kvc_anchor_refresh_svd(FAKE, 1, 64, 64, 80, FAKE + (1 << 24), FAKE + (2 << 24), 0, FAKE + (3 << 24),
                                    4, 2, 0, FAKE + (4 << 24), 1 << 30, None) == 2
    assert L.kvc_anchor_refresh_svd(FAKE, 1, 64, 64, 8, FAKE + (1 << 24), FAKE + (2 << 24), 0, FAKE + (3 << 24),
                                    4, 99, 0, FAKE + (4 << 24), 1 << 30, None) == 8


def test_noalloc_rejects_requests_beyond_its_scratch():
    # the 32768-token 8B-shaped hop needs ~968 MiB of scratch, beyond the no-alloc entry point's
    # fixed 384 MiB: refused on the host before any device work (the pointers are never used)
    L = kvc.lib()
    n = 20
    lens = (C.c_int32 * n)(*([32768] * n))
    p = kvc.Pool(n, 32, 32, 0, C.cast(lens, C.POINTER(C.c_int32)), 1, *([FAKE] * 8), 0, 0, None)
    prm = kvc.params_of()
    mo = kvc.MatchOut(FAKE, FAKE, FAKE, None, None, None)
    sh = kvc.shape_of(32, 32768, 8, 128)
    assert L.kvc_workspace_size(3, sh, C.byref(p), C.byref(prm)) > kvc.NOALLOC_SCRATCH_BYTES
    st = L.kvc_correct_hop_noalloc(FAKE, FAKE + (1 << 36), FAKE + (2 << 36), FAKE + (3 << 36), 1, sh, 0, 300,
                                   C.byref(_rope()), C.byref(p), C.byref(prm), C.byref(mo), None)
    assert st == 6   # KVC_E_WORKSPACE
    assert b"maximum" in L.kvc_last_error()
