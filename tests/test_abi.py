"""The C ABI of libdpnorm without a GPU: every declared symbol is exported,
and every host-side check returns its documented status before anything is
enqueued (all calls here fail validation, so no device work is started)."""
import ctypes as C
import os
import re

import pytest

from sample_grad_norms_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")

# aligned fake device addresses: validation only compares and aligns them
A_ADDR, G_ADDR, P_ADDR, N_ADDR, WS_ADDR = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def declared_functions():
    names = set()
    for fn in os.listdir(HEADER_DIR):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(HEADER_DIR, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        names.update(re.findall(r"\b(dpnorm_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature"


def test_version_and_status_strings(lib):
    assert lib.dpnorm_version() >= 100
    for st in range(8):
        assert lib.dpnorm_status_string(st).startswith(b"DPNORM_")
    assert b"unknown" in lib.dpnorm_status_string(99)


@pytest.mark.parametrize("k,ms,mt", [(3, 1, 1), (4, 2, 0), (32, 11, 10), (96, 32, 32), (30, 10, 10)])
def test_hutchpp_split(lib, k, ms, mt):
    a, b = C.c_int64(0), C.c_int64(0)
    st = lib.dpnorm_hutchpp_split(k, C.byref(a), C.byref(b))
    if mt < 1:
        assert st == _lib.ERR_SIZE
    else:
        assert st == _lib.OK and (a.value, b.value) == (ms, mt)


@pytest.mark.parametrize("k", [2, 1, 0, 97])
def test_hutchpp_split_rejects(lib, k):
    a, b = C.c_int64(0), C.c_int64(0)
    assert lib.dpnorm_hutchpp_split(k, C.byref(a), C.byref(b)) == _lib.ERR_SIZE


def ws_query(lib, dt=_lib.BF16, B=2, T=100, d=64, p=32, k=8):
    nb = C.c_size_t(0)
    st = lib.dpnorm_hutch_workspace(dt, B, T, d, p, k, C.byref(nb))
    return st, nb.value


def test_workspace_query(lib):
    st, nb = ws_query(lib)
    assert st == _lib.OK and nb > 0 and nb % 256 == 0
    # linear in the batch for the per-sample buffers
    st2, nb2 = ws_query(lib, B=4)
    assert st2 == _lib.OK and nb2 > nb
    assert ws_query(lib, dt=7)[0] == _lib.ERR_DTYPE
    assert ws_query(lib, d=12)[0] == _lib.ERR_SIZE        # bf16 widths are multiples of 8
    assert ws_query(lib, dt=_lib.F32, d=12)[0] == _lib.OK  # fp32 widths multiples of 4
    assert ws_query(lib, k=0)[0] == _lib.ERR_SIZE
    assert ws_query(lib, k=65)[0] == _lib.ERR_SIZE
    assert ws_query(lib, B=0)[0] == _lib.ERR_SIZE
    assert ws_query(lib, T=0)[0] == _lib.ERR_SIZE
    assert lib.dpnorm_hutch_workspace(_lib.BF16, 2, 100, 64, 32, 8, None) == _lib.ERR_NULL


def test_grouped_workspace_covers_layers(lib):
    arr = (_lib.Layer * 3)(_lib.Layer(None, None, None, 64, 32), _lib.Layer(None, None, None, 128, 64),
                           _lib.Layer(None, None, None, 64, 512))
    nb = C.c_size_t(0)
    assert lib.dpnorm_hutch_grouped_workspace(arr, 3, _lib.BF16, 2, 100, 8, C.byref(nb)) == _lib.OK
    single = sum(ws_query(lib, d=y.d, p=y.p)[1] for y in arr)
    assert nb.value > 0 and nb.value <= single + 3 * 4096
    assert lib.dpnorm_hutch_grouped_workspace(arr, 0, _lib.BF16, 2, 100, 8, C.byref(nb)) == _lib.ERR_SIZE
    assert lib.dpnorm_hutch_grouped_workspace(None, 1, _lib.BF16, 2, 100, 8, C.byref(nb)) == _lib.ERR_NULL


def shared_input_layers(n_layers, dm=128, kv=64, hid=256):
    """Fake descriptors of a transformer stack in which q, k, v share one
    input and gate, up share another (distinct aligned fake addresses)."""
    shapes = [(dm, dm), (dm, kv), (dm, kv), (dm, dm), (dm, hid), (dm, hid), (hid, dm)]
    input_of = (0, 0, 0, 3, 4, 4, 6)
    arr = (_lib.Layer * (7 * n_layers))()
    for layer in range(n_layers):
        for j, (d, p) in enumerate(shapes):
            a = 0x10000000 + (7 * layer + input_of[j]) * 0x100000
            g = 0x80000000 + (7 * layer + j) * 0x100000
            arr[7 * layer + j] = _lib.Layer(a, g, g + 0x80000, d, p)
    return arr


def test_grouped_workspace_shared_inputs(lib):
    # 16 layers, B = 10, T = 1024: unshared, 1120 stage-2 items need no T
    # split; shared, 640 items split T in two and need the partial tiles
    arr = shared_input_layers(16)
    plain = (_lib.Layer * len(arr))(*[_lib.Layer(None, None, None, y.d, y.p) for y in arr])
    shared_b, plain_b = C.c_size_t(0), C.c_size_t(0)
    assert lib.dpnorm_hutch_grouped_workspace(arr, len(arr), _lib.BF16, 10, 1024, 32, C.byref(shared_b)) == _lib.OK
    assert lib.dpnorm_hutch_grouped_workspace(plain, len(arr), _lib.BF16, 10, 1024, 32, C.byref(plain_b)) == _lib.OK
    assert shared_b.value > plain_b.value > 0
    # one byte below both plans: rejected before anything is enqueued
    n = C.c_void_p(N_ADDR)
    st = lib.dpnorm_hutch_grouped(arr, len(arr), _lib.BF16, 10, 1024, 32, n, 0, None, 1.0, WS_ADDR,
                                  plain_b.value - 1, None)
    assert st == _lib.ERR_WORKSPACE


def hutch(lib, A=A_ADDR, G=G_ADDR, P=P_ADDR, dt=_lib.BF16, B=2, T=100, d=64, p=32, k=8, n=N_ADDR, acc=0,
          ws=WS_ADDR, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = ws_query(lib, dt, B, T, d, p, k)[1] - 1   # one byte short: never launches
    return lib.dpnorm_hutch(A, G, P, dt, B, T, d, p, k, n, acc, ws, ws_bytes, None)


def test_hutch_rejects_before_launch(lib):
    assert hutch(lib) == _lib.ERR_WORKSPACE
    assert hutch(lib, A=None) == _lib.ERR_NULL
    assert hutch(lib, G=None) == _lib.ERR_NULL
    assert hutch(lib, P=None) == _lib.ERR_NULL
    assert hutch(lib, n=None) == _lib.ERR_NULL
    assert hutch(lib, ws=None) == _lib.ERR_NULL
    assert hutch(lib, dt=5) == _lib.ERR_DTYPE
    assert hutch(lib, B=0) == _lib.ERR_SIZE
    assert hutch(lib, T=-1) == _lib.ERR_SIZE
    assert hutch(lib, d=20) == _lib.ERR_SIZE
    assert hutch(lib, k=100) == _lib.ERR_SIZE
    assert hutch(lib, A=A_ADDR + 8) == _lib.ERR_ALIGN
    assert hutch(lib, G=G_ADDR + 4) == _lib.ERR_ALIGN
    assert hutch(lib, P=P_ADDR + 1) == _lib.ERR_ALIGN
    assert hutch(lib, n=N_ADDR + 2) == _lib.ERR_ALIGN
    assert hutch(lib, acc=2) == _lib.ERR_VALUE
    big = ws_query(lib)[1]
    assert hutch(lib, ws=WS_ADDR + 128, ws_bytes=big) == _lib.ERR_ALIGN
    # outputs overlapping an input or the workspace
    assert hutch(lib, n=A_ADDR + 64, ws_bytes=big) == _lib.ERR_VALUE
    assert hutch(lib, n=P_ADDR, ws_bytes=big) == _lib.ERR_VALUE
    assert hutch(lib, n=WS_ADDR + 256, ws_bytes=big) == _lib.ERR_VALUE
    # B * T * max(d, p) too large for the byte sizes
    assert hutch(lib, B=1 << 20, T=1 << 20, d=1 << 24) == _lib.ERR_SIZE


def test_grouped_clip_checks(lib):
    arr = (_lib.Layer * 1)(_lib.Layer(A_ADDR, G_ADDR, P_ADDR, 64, 32))
    nb = C.c_size_t(0)
    assert lib.dpnorm_hutch_grouped_workspace(arr, 1, _lib.BF16, 2, 100, 8, C.byref(nb)) == _lib.OK
    args = (arr, 1, _lib.BF16, 2, 100, 8, N_ADDR, 0)
    for Cv in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.dpnorm_hutch_grouped(*args, N_ADDR + 64, Cv, WS_ADDR, nb.value, None) == _lib.ERR_VALUE
    # c overlapping n without being equal to it
    assert lib.dpnorm_hutch_grouped(*args, N_ADDR + 4, 1.0, WS_ADDR, nb.value, None) == _lib.ERR_VALUE
    # trace too short
    evs = (C.c_void_p * 2)(1, 2)
    kinds = (C.c_int32 * 2)()
    tr = _lib.Trace(C.cast(evs, C.POINTER(C.c_void_p)), C.cast(kinds, C.POINTER(C.c_int32)), 2, 0)
    assert lib.dpnorm_hutch_grouped_traced(*args, None, 1.0, WS_ADDR, nb.value, None, C.byref(tr)) == _lib.ERR_SIZE
    assert lib.dpnorm_hutch_grouped_traced(*args, None, 1.0, WS_ADDR, nb.value, None, None) == _lib.ERR_NULL


def test_clip_factor_checks(lib):
    assert lib.dpnorm_clip_factors(None, 4, 1.0, N_ADDR, None) == _lib.ERR_NULL
    assert lib.dpnorm_clip_factors(N_ADDR, 0, 1.0, N_ADDR, None) == _lib.ERR_SIZE
    assert lib.dpnorm_clip_factors(N_ADDR, 4, 0.0, N_ADDR, None) == _lib.ERR_VALUE
    assert lib.dpnorm_clip_factors(N_ADDR, 4, float("nan"), N_ADDR, None) == _lib.ERR_VALUE
    assert lib.dpnorm_clip_factors(N_ADDR, 4, 1.0, N_ADDR + 4, None) == _lib.ERR_VALUE
    assert lib.dpnorm_clip_factors(N_ADDR + 2, 4, 1.0, N_ADDR + 64, None) == _lib.ERR_ALIGN


def test_hutch_sign_checks(lib):
    def call(S=P_ADDR, k=8, A=A_ADDR, ws_bytes=None, acc=0):
        if ws_bytes is None:
            ws_bytes = ws_query(lib, _lib.BF16, 2, 100, 64, 32, k)[1] - 1   # one byte short: never launches
        return lib.dpnorm_hutch_sign(A, G_ADDR, S, _lib.BF16, 2, 100, 64, 32, k, N_ADDR, acc, WS_ADDR, ws_bytes, None)
    assert call() == _lib.ERR_WORKSPACE
    assert call(S=None) == _lib.ERR_NULL
    assert call(S=P_ADDR + 2) == _lib.ERR_ALIGN        # words need 4-byte alignment
    assert call(S=P_ADDR + 4) == _lib.ERR_WORKSPACE    # 4-byte aligned is enough
    assert call(k=0, ws_bytes=1 << 30) == _lib.ERR_SIZE
    assert call(k=65, ws_bytes=1 << 30) == _lib.ERR_SIZE
    assert call(acc=2, ws_bytes=1 << 30) == _lib.ERR_VALUE
    arr = (_lib.Layer * 1)(_lib.Layer(A_ADDR, G_ADDR, None, 64, 32))
    st = lib.dpnorm_hutch_sign_grouped(arr, 1, _lib.BF16, 2, 100, 8, N_ADDR, 0, None, 1.0, WS_ADDR, 1 << 30, None)
    assert st == _lib.ERR_NULL


def test_read_probe_checks(lib):
    assert lib.dpnorm_read_probe(None, 16384, None) == _lib.ERR_NULL
    for bad in (0, -16384, 16383, 16384 + 8):
        assert lib.dpnorm_read_probe(A_ADDR, bad, None) == _lib.ERR_SIZE
    assert lib.dpnorm_read_probe(A_ADDR + 8, 16384, None) == _lib.ERR_ALIGN


def test_event_helpers_reject_null(lib):
    assert lib.dpnorm_event_create(None) == _lib.ERR_NULL
    assert lib.dpnorm_event_destroy(None) == _lib.ERR_NULL
    assert lib.dpnorm_event_record(None, None) == _lib.ERR_NULL
    assert lib.dpnorm_event_synchronize(None) == _lib.ERR_NULL
    ms = C.c_float(0)
    assert lib.dpnorm_event_elapsed_ms(None, None, C.byref(ms)) == _lib.ERR_NULL


def test_hutchpp_checks(lib):
    nb = C.c_size_t(0)
    assert lib.dpnorm_hutchpp_workspace(_lib.BF16, 2, 100, 64, 32, 32, C.byref(nb)) == _lib.OK and nb.value > 0
    for k in (2, 97):
        assert lib.dpnorm_hutchpp_workspace(_lib.BF16, 2, 100, 64, 32, k, C.byref(nb)) == _lib.ERR_SIZE
    lib.dpnorm_hutchpp_workspace(_lib.BF16, 2, 100, 64, 32, 32, C.byref(nb))
    S_ADDR = 0x600000
    args = [A_ADDR, G_ADDR, S_ADDR, P_ADDR, _lib.BF16, 2, 100, 64, 32, 32, N_ADDR, 0, None, None, None, None]
    assert lib.dpnorm_hutchpp(*args, WS_ADDR, nb.value - 1, None) == _lib.ERR_WORKSPACE
    bad = list(args); bad[2] = None
    assert lib.dpnorm_hutchpp(*bad, WS_ADDR, nb.value, None) == _lib.ERR_NULL
    bad = list(args); bad[12] = N_ADDR      # head aliases n
    assert lib.dpnorm_hutchpp(*bad, WS_ADDR, nb.value, None) == _lib.ERR_VALUE
    bad = list(args); bad[4] = 9
    assert lib.dpnorm_hutchpp(*bad, WS_ADDR, nb.value, None) == _lib.ERR_DTYPE
    bad = list(args); bad[11] = 3
    assert lib.dpnorm_hutchpp(*bad, WS_ADDR, nb.value, None) == _lib.ERR_VALUE
    # resid is [B][m_s] floats (2 x 11 at k = 32): one that reaches n overlaps it
    bad = list(args); bad[15] = N_ADDR - 4 * 2 * 11 + 4
    assert lib.dpnorm_hutchpp(*bad, WS_ADDR, nb.value, None) == _lib.ERR_VALUE
    bad = list(args); bad[15] = N_ADDR + 2
    assert lib.dpnorm_hutchpp(*bad, WS_ADDR, nb.value, None) == _lib.ERR_ALIGN


def test_exact_checks(lib):
    nb = C.c_size_t(0)
    for route in (_lib.EXACT_AUTO, _lib.EXACT_EXPLICIT, _lib.EXACT_GRAM):
        assert lib.dpnorm_exact_workspace(_lib.BF16, 2, 100, 64, 32, route, C.byref(nb)) == _lib.OK
        assert nb.value > 0
    assert lib.dpnorm_exact_workspace(_lib.BF16, 2, 100, 64, 32, 5, C.byref(nb)) == _lib.ERR_DTYPE
    assert lib.dpnorm_exact_workspace(_lib.BF16, 2, 100, 60, 32, 0, C.byref(nb)) == _lib.ERR_SIZE
    lib.dpnorm_exact_workspace(_lib.BF16, 2, 100, 64, 32, 0, C.byref(nb))
    args = (A_ADDR, G_ADDR, _lib.BF16, 2, 100, 64, 32, _lib.EXACT_AUTO, N_ADDR, 0)
    assert lib.dpnorm_exact(*args, WS_ADDR, nb.value - 1, None) == _lib.ERR_WORKSPACE
    assert lib.dpnorm_exact(None, G_ADDR, _lib.BF16, 2, 100, 64, 32, 0, N_ADDR, 0, WS_ADDR, nb.value,
                            None) == _lib.ERR_NULL
    assert lib.dpnorm_exact(A_ADDR, G_ADDR, _lib.BF16, 2, 100, 64, 32, 0, A_ADDR, 0, WS_ADDR, nb.value,
                            None) == _lib.ERR_VALUE


def test_noalloc_rejects_plans_beyond_the_static_scratch(lib):
    """dpnorm_hutch_grouped_noalloc checks its plan against the static scratch
    before it touches the device: the 112-projection Llama-shaped stack at
    B=4, T=4096 needs far more than 64 MiB and is rejected, and so are
    invalid sizes."""
    shapes = [(2048, 2048), (2048, 512), (2048, 512), (2048, 2048), (2048, 8192), (2048, 8192), (8192, 2048)] * 16
    arr = (_lib.Layer * len(shapes))()
    for j, (d, p) in enumerate(shapes):
        arr[j] = _lib.Layer(A_ADDR + (j << 32), G_ADDR + (j << 32), P_ADDR + (j << 32), d, p)
    nb = C.c_size_t(0)
    assert lib.dpnorm_hutch_grouped_workspace(arr, len(shapes), _lib.BF16, 4, 4096, 32, C.byref(nb)) == _lib.OK
    assert nb.value > _lib.STATIC_SCRATCH_BYTES
    assert lib.dpnorm_hutch_grouped_noalloc(arr, len(shapes), _lib.BF16, 4, 4096, 32, N_ADDR, 0, None, 1.0,
                                            None) == _lib.ERR_WORKSPACE
    assert lib.dpnorm_hutch_grouped_noalloc(arr, 1, _lib.BF16, 4, 4096, 65, N_ADDR, 0, None, 1.0,
                                            None) == _lib.ERR_SIZE
    assert lib.dpnorm_hutch_grouped_noalloc(None, 1, _lib.BF16, 4, 4096, 32, N_ADDR, 0, None, 1.0,
                                            None) == _lib.ERR_NULL
