"""CPU tests of the C ABI: the library loads, exports every declared symbol,
sizes workspaces, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from post_weight_quantization_26_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(build_lib.LIB_PATH):
        build_lib.build()
    from post_weight_quantization_26_amd import _lib
    _lib.lib()
    return _lib


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("awq_act_stats", "awq_search_scale", "awq_search_clip", "awq_quantize_pack",
              "awq_workspace_bytes", "awq_last_error", "awq_scale_table"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    lib = ctypes.CDLL(build_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in L.SIGNATURES, f"binding lacks {name}"


def test_workspace_sizes(L):
    lib = L.lib()
    ws = lib.awq_workspace_bytes
    # search: s table + E batch + per-tile partials + row sums + curve
    full = ws(L.AWQ_OP_SEARCH_SCALE, 65536, 4096, 4096, 20, L.AWQ_BF16)
    e_bytes = 20 * 4096 * 4096 * 2
    part = 256 * 20 * 4096 * 4
    assert full >= e_bytes + part and full < e_bytes + part + (2 << 20)
    one = lib.awq_workspace_bytes_batch(L.AWQ_OP_SEARCH_SCALE, 65536, 4096, 4096, 20, 1, L.AWQ_BF16)
    assert one < full / 10
    assert lib.awq_workspace_bytes_batch(L.AWQ_OP_SEARCH_SCALE, 65536, 4096, 4096, 20, 20,
                                         L.AWQ_BF16) == full
    assert lib.awq_workspace_bytes_batch(L.AWQ_OP_SEARCH_SCALE, 65536, 4096, 4096, 20, 21,
                                         L.AWQ_BF16) == 0
    assert lib.awq_workspace_bytes_batch(L.AWQ_OP_PACK, 1, 64, 128, 1, 1, L.AWQ_BF16) == 0
    # the minimum a search accepts is batch 1: one byte less is rejected
    FAKEW = ctypes.c_void_p(0x10000)
    mse = (ctypes.c_double * 20)()
    a_best = ctypes.c_float()
    st = lib.awq_search_scale(FAKEW, FAKEW, L.AWQ_BF16, 65536, 4096, 4096, FAKEW,
                              L.float_array([0.5] * 20), 20, L.QConfig(4, 128, 1), FAKEW,
                              ctypes.byref(a_best), mse, None, FAKEW, one - 1, None)
    assert st == L.AWQ_E_WORKSPACE
    assert ws(L.AWQ_OP_PACK, 1, 4096, 4096, 1, L.AWQ_BF16) > 0
    assert ws(L.AWQ_OP_STATS, 65536, 1, 4096, 1, L.AWQ_BF16) >= 4096 * 8
    for bad in ((13, 1, 1, 1, 1, 1), (1, 0, 1, 1, 1, 1), (1, 1, 1, 1, 0, 1), (1, 1, 1, 1, 65, 1),
                (1, 1, 1, 1, 1, 7)):
        assert ws(*bad) == 0
    # split candidates: the candidate buffer doubles; float32 layers do not split
    for plain, split in ((L.AWQ_OP_SEARCH_SCALE, L.AWQ_OP_SEARCH_SCALE_SPLIT_E),
                         (L.AWQ_OP_SEARCH_CLIP, L.AWQ_OP_SEARCH_CLIP_SPLIT_E)):
        for dt in (L.AWQ_BF16, L.AWQ_F16):
            a, b = ws(plain, 65536, 4096, 4096, 20, dt), ws(split, 65536, 4096, 4096, 20, dt)
            assert b - a == 20 * 4096 * 4096 * 2
            a1 = lib.awq_workspace_bytes_batch(plain, 65536, 4096, 4096, 20, 1, dt)
            b1 = lib.awq_workspace_bytes_batch(split, 65536, 4096, 4096, 20, 1, dt)
            assert b1 - a1 == 4096 * 4096 * 2
        assert ws(split, 256, 512, 512, 20, L.AWQ_F32) == ws(plain, 256, 512, 512, 20, L.AWQ_F32)
    # a split search is refused a workspace sized for the plain one
    st = lib.awq_search_scale(FAKEW, FAKEW, L.AWQ_BF16, 65536, 4096, 4096, FAKEW,
                              L.float_array([0.5] * 20), 20, L.QConfig(4, 128, 1, 1), FAKEW,
                              ctypes.byref(a_best), mse, None, FAKEW, one, None)
    assert st == L.AWQ_E_WORKSPACE
    # fused searches: K/2 bytes per candidate row instead of 2K; 16-bit layers only
    for plain, fused in ((L.AWQ_OP_SEARCH_SCALE, L.AWQ_OP_SEARCH_SCALE_FUSED),
                         (L.AWQ_OP_SEARCH_CLIP, L.AWQ_OP_SEARCH_CLIP_FUSED)):
        for dt in (L.AWQ_BF16, L.AWQ_F16):
            a, b = ws(plain, 65536, 4096, 4096, 20, dt), ws(fused, 65536, 4096, 4096, 20, dt)
            assert a - b == 20 * 4096 * (4096 * 2 - 4096 // 2)
            a1 = lib.awq_workspace_bytes_batch(plain, 65536, 4096, 4096, 20, 1, dt)
            b1 = lib.awq_workspace_bytes_batch(fused, 65536, 4096, 4096, 20, 1, dt)
            assert a1 - b1 == 4096 * (4096 * 2 - 4096 // 2)
        assert ws(fused, 256, 512, 512, 20, L.AWQ_F32) == 0
        assert lib.awq_workspace_bytes_batch(fused, 256, 512, 512, 20, 2, L.AWQ_F32) == 0
    # a fused search takes its own (smaller) size; the unfused search does not
    fz = L.QConfig(4, 128, 1, L.AWQ_SEARCH_FUSED)
    f1 = lib.awq_workspace_bytes_batch(L.AWQ_OP_SEARCH_SCALE_FUSED, 65536, 4096, 4096, 20, 1,
                                       L.AWQ_BF16)
    st = lib.awq_search_scale(FAKEW, FAKEW, L.AWQ_BF16, 65536, 4096, 4096, FAKEW,
                              L.float_array([0.5] * 20), 20, fz, FAKEW,
                              ctypes.byref(a_best), mse, None, FAKEW, f1 - 1, None)
    assert st == L.AWQ_E_WORKSPACE
    st = lib.awq_search_scale(FAKEW, FAKEW, L.AWQ_BF16, 65536, 4096, 4096, FAKEW,
                              L.float_array([0.5] * 20), 20, L.QConfig(4, 128, 1), FAKEW,
                              ctypes.byref(a_best), mse, None, FAKEW, f1, None)
    assert st == L.AWQ_E_WORKSPACE


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p(0x10002)        # misaligned


def _search(L, op, **kw):
    a = dict(X=FAKE, W=FAKE, dtype=L.AWQ_BF16, T=256, N=256, K=256, vec=FAKE,
             grid=[0.25, 0.5, 1.0], qc=L.QConfig(4, 128, 1), out=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    lib = L.lib()
    grid = L.float_array(a["grid"])
    n = kw.get("n", len(a["grid"]))
    if op == "scale":
        a_best = ctypes.c_float()
        mse = (ctypes.c_double * 64)()
        return lib.awq_search_scale(a["X"], a["W"], a["dtype"], a["T"], a["N"], a["K"], a["vec"],
                                    grid, n, a["qc"], a["out"], ctypes.byref(a_best), mse, None,
                                    a["ws"], a["ws_bytes"], None)
    mc = ctypes.c_double()
    return lib.awq_search_clip(a["X"], a["W"], a["dtype"], a["T"], a["N"], a["K"], a["vec"], grid,
                               n, a["qc"], a["out"], ctypes.byref(mc), None, a["ws"],
                               a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), -1), (dict(W=None), -1), (dict(vec=None), -1), (dict(out=None), -1),
    (dict(T=0), -1), (dict(N=-3), -1), (dict(K=200), -1), (dict(K=0), -1),
    (dict(dtype=7), -1),
    (dict(qc=None), -2),
    (dict(grid=[0.5, 1.5]), -1), (dict(grid=[-0.1]), -1), (dict(grid=[float("nan")]), -1),
    (dict(grid=[0.5] * 65), -1), (dict(grid=[]), -1),
    (dict(X=MIS), -1), (dict(W=MIS), -1),
    (dict(ws=None), -3), (dict(ws_bytes=1000), -3), (dict(ws=MIS), -3),
    (dict(flags=3), -1), (dict(flags=4), -1), (dict(flags=-1), -1),
])
@pytest.mark.parametrize("op", ["scale", "clip"])
def test_search_rejects(L, kw, status, op):
    if kw.get("qc", 0) is None:
        kw = dict(kw, qc=L.QConfig(4, 16, 1))          # unsupported group size
    if "flags" in kw:
        kw = dict(qc=L.QConfig(4, 128, 1, kw["flags"]))
    assert _search(L, op, **kw) == status
    assert L.last_error()


def test_gram_searches_reject_split(L):
    lib = L.lib()
    a_best = ctypes.c_float()
    mse = (ctypes.c_double * 4)()
    st = lib.awq_search_scale_gram(FAKE, FAKE, L.AWQ_BF16, 256, 256, 256, FAKE,
                                   L.float_array([0.5]), 1, L.QConfig(4, 128, 1, 1), FAKE,
                                   ctypes.byref(a_best), mse, None, FAKE, 1 << 40, None)
    assert st == L.AWQ_E_UNSUPPORTED and "direct" in L.last_error()
    # a float32 layer accepts the flag (its candidates are float32 already)
    assert _search(L, "scale", dtype=L.AWQ_F32, qc=L.QConfig(4, 128, 1, 1), ws_bytes=10) == -3


@pytest.mark.parametrize("op", ["scale", "clip"])
def test_fused_search_limits(L, op):
    fused = L.QConfig(4, 128, 1, L.AWQ_SEARCH_FUSED)
    # a bf16 layer with N a multiple of 256 passes every check before the workspace one
    assert _search(L, op, qc=fused, ws_bytes=10) == L.AWQ_E_WORKSPACE
    assert _search(L, op, qc=L.QConfig(4, 64, 0, L.AWQ_SEARCH_FUSED), dtype=L.AWQ_F16, N=512,
                   ws_bytes=10) == L.AWQ_E_WORKSPACE
    # N not a multiple of 256, float32 layers
    assert _search(L, op, qc=fused, N=384) == L.AWQ_E_UNSUPPORTED
    assert "multiple of 256" in L.last_error()
    assert _search(L, op, qc=fused, dtype=L.AWQ_F32) == L.AWQ_E_UNSUPPORTED
    # the parameter table fits the fused workspace's candidate region at every group size
    for fused in (L.AWQ_OP_SEARCH_SCALE_FUSED, L.AWQ_OP_SEARCH_CLIP_FUSED):
        one = L.lib().awq_workspace_bytes_batch(fused, 4096, 4096, 4096, 20, 1, L.AWQ_BF16)
        assert one > 4096 * (4096 // 32) * 16


def test_fused_search_rejected_elsewhere(L):
    lib = L.lib()
    a_best = ctypes.c_float()
    mse = (ctypes.c_double * 4)()
    fused = L.QConfig(4, 128, 1, L.AWQ_SEARCH_FUSED)
    st = lib.awq_search_scale_gram(FAKE, FAKE, L.AWQ_BF16, 256, 256, 256, FAKE,
                                   L.float_array([0.5]), 1, fused, FAKE, ctypes.byref(a_best),
                                   mse, None, FAKE, 1 << 40, None)
    assert st == L.AWQ_E_UNSUPPORTED and "direct" in L.last_error()
    W = (ctypes.c_void_p * 2)(FAKE, FAKE)
    N = (ctypes.c_int64 * 2)(256, 256)
    st = lib.awq_search_scale_group(FAKE, W, N, 2, L.AWQ_BF16, 256, 256, FAKE,
                                    L.float_array([0.5]), 1, fused, FAKE, ctypes.byref(a_best),
                                    mse, None, FAKE, 1 << 40, None)
    assert st == L.AWQ_E_UNSUPPORTED and "single-layer" in L.last_error()


@pytest.mark.parametrize("qc,status", [((5, 128, 1), -2), ((2, 128, 1), -2), ((4, 16, 1), -2),
                                       ((4, 256, 1), -2), ((3, 48, 1), -2), ((4, 128, 2), -1)])
def test_search_rejects_qconfig(L, qc, status):
    assert _search(L, "scale", qc=L.QConfig(*qc)) == status


def test_clip_grid_excludes_zero(L):
    assert _search(L, "clip", grid=[0.0, 1.0]) == -1
    assert "out of range" in L.last_error()


def test_stats_rejects(L):
    lib = L.lib()
    f = lib.awq_act_stats
    assert f(None, 1, 16, 64, FAKE, FAKE, 1 << 30, None) == -1
    assert f(FAKE, 1, 0, 64, FAKE, FAKE, 1 << 30, None) == -1
    assert f(FAKE, 1, 16, 60, FAKE, FAKE, 1 << 30, None) == -1     # K not a multiple of 8
    assert f(FAKE, 0, 16, 62, FAKE, FAKE, 1 << 30, None) == -1     # f32: multiple of 4
    assert f(MIS, 1, 16, 64, FAKE, FAKE, 1 << 30, None) == -1
    assert f(FAKE, 1, 16, 64, FAKE, FAKE, 8, None) == -3
    assert f(FAKE, 9, 16, 64, FAKE, FAKE, 1 << 30, None) == -1


def test_stats_batches_rejects(L):
    lib = L.lib()
    acc, fin = lib.awq_act_stats_accumulate, lib.awq_act_stats_finalize
    MIS8 = ctypes.c_void_p(0x10004)       # 4-byte but not 8-byte aligned
    assert acc(FAKE, 1, 16, 64, None, FAKE, 1 << 30, None) == -1
    assert acc(FAKE, 1, 16, 64, MIS8, FAKE, 1 << 30, None) == -1
    assert "8-byte" in L.last_error()
    assert acc(FAKE, 1, 0, 64, FAKE, FAKE, 1 << 30, None) == -1
    assert acc(FAKE, 1, 16, 60, FAKE, FAKE, 1 << 30, None) == -1
    assert acc(MIS, 1, 16, 64, FAKE, FAKE, 1 << 30, None) == -1
    assert acc(FAKE, 1, 16, 64, FAKE, FAKE, 8, None) == -3
    assert fin(None, 16, 64, FAKE, None) == -1
    assert fin(FAKE, 0, 64, FAKE, None) == -1
    assert fin(FAKE, 16, 0, FAKE, None) == -1
    assert fin(MIS8, 16, 64, FAKE, None) == -1
    assert fin(FAKE, 16, 64, MIS, None) == -1
    assert "act_stats_finalize" in L.last_error()


def test_scale_table_rejects(L):
    lib = L.lib()
    assert lib.awq_scale_table(FAKE, 16, L.float_array([0.5, 2.0]), 2, FAKE, None) == -1
    assert lib.awq_scale_table(FAKE, 0, L.float_array([0.5]), 1, FAKE, None) == -1
    assert lib.awq_scale_table(None, 16, L.float_array([0.5]), 1, FAKE, None) == -1


def test_pack_rejects(L):
    lib = L.lib()
    f = lib.awq_quantize_pack
    qc = L.QConfig(4, 128, 1)
    args = lambda **k: [k.get("W", FAKE), k.get("dt", 1), k.get("N", 64), k.get("K", 256),
                        FAKE, None, k.get("qc", qc), FAKE, FAKE, FAKE, k.get("ws", FAKE),
                        k.get("wsb", 4096), None]
    assert f(*args(N=12)) == -1                     # N % 8
    assert f(*args(K=200)) == -1                    # K % 128
    assert f(*args(K=192, qc=L.QConfig(4, 64, 1))) == -1     # K % 128 for every group size
    assert f(*args(N=48, qc=L.QConfig(3, 128, 1))) == -1     # 3-bit rows fill words: N % 32
    assert "multiple of 32" in L.last_error()
    assert f(*args(qc=L.QConfig(2, 128, 1))) == -2
    assert f(*args(qc=L.QConfig(4, 16, 1))) == -2
    assert f(*args(W=None)) == -1
    assert f(*args(W=MIS)) == -1
    assert f(*args(wsb=0)) == -3
    assert f(*args(dt=5)) == -1


def test_profile_read_rejects_bad_kind(L):
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert L.lib().awq_profile_read(99, ctypes.byref(ms), ctypes.byref(n)) == -1


def test_binding_fails_loudly_without_library(monkeypatch, L):
    from post_weight_quantization_26_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libawq_mi355x.so")
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_autoawq_defaults():
    import json
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "quant_config_autoawq.json")))
    src = open(os.path.join(ROOT, "post_weight_quantization_26_amd", "api.py")).read()
    assert f"DEFAULT_BITS = {gold['w_bit']}" in src
    assert f"DEFAULT_GROUP = {gold['q_group_size']}" in src
    assert f"DEFAULT_ZERO_POINT = {gold['zero_point']}" in src


def _group(L, Ws=(FAKE, FAKE), Ns=(256, 128), n_layers=None, ws_bytes=1 << 40, K=256, T=256):
    lib = L.lib()
    n = len(Ws) if n_layers is None else n_layers
    wp = (ctypes.c_void_p * max(len(Ws), 1))(*[w.value if w is not None else None for w in Ws])
    nv = (ctypes.c_int64 * max(len(Ns), 1))(*Ns)
    a_best = ctypes.c_float()
    mse = (ctypes.c_double * 3)()
    return lib.awq_search_scale_group(FAKE, wp, nv, n, L.AWQ_BF16, T, K, FAKE,
                                      L.float_array([0.0, 0.5, 1.0]), 3, L.QConfig(4, 128, 1),
                                      FAKE, ctypes.byref(a_best), mse, None, FAKE, ws_bytes, None)


def test_group_search_rejects(L):
    assert _group(L, n_layers=0) == -1
    assert _group(L, Ws=(FAKE,) * 17, Ns=(128,) * 17) == -1
    assert _group(L, Ws=(FAKE, None)) == -1
    assert _group(L, Ws=(FAKE, MIS)) == -1
    assert _group(L, Ns=(256, 0)) == -1
    assert _group(L, K=200) == -1
    # the workspace is sized for the summed output channels
    lib = L.lib()
    one = lib.awq_workspace_bytes_batch(L.AWQ_OP_SEARCH_SCALE, 256, 256, 256, 3, 1, L.AWQ_BF16)
    both = lib.awq_workspace_bytes_batch(L.AWQ_OP_SEARCH_SCALE, 256, 384, 256, 3, 1, L.AWQ_BF16)
    assert both > one
    assert _group(L, ws_bytes=one) == -3
    assert "workspace" in L.last_error()
    assert _group(L, Ns=(256, (1 << 31) + 1)) == -1
    assert "N[1]" in L.last_error()
    assert _group(L, Ns=(256, (1 << 31) - 1)) == -1
    assert "in total" in L.last_error()


def test_fold_rejects(L):
    lib = L.lib()
    fn, fl = lib.awq_fold_norm, lib.awq_fold_linear
    ODD = ctypes.c_void_p(0x10001)
    assert fn(None, None, L.AWQ_BF16, 64, FAKE, None) == -1
    assert fn(FAKE, None, L.AWQ_BF16, 0, FAKE, None) == -1
    assert fn(FAKE, None, 7, 64, FAKE, None) == -1
    assert fn(FAKE, None, L.AWQ_BF16, 64, None, None) == -1
    assert fn(ODD, None, L.AWQ_BF16, 64, FAKE, None) == -1
    assert fn(MIS, None, L.AWQ_F32, 64, FAKE, None) == -1
    assert fn(FAKE, MIS, L.AWQ_F32, 64, FAKE, None) == -1
    assert fl(None, None, L.AWQ_BF16, 64, 64, FAKE, None) == -1
    assert fl(FAKE, None, L.AWQ_BF16, 64, 12, FAKE, None) == -1     # row of 24 bytes
    assert fl(FAKE, None, L.AWQ_F32, 64, 6, FAKE, None) == -1       # row of 24 bytes
    assert fl(MIS, None, L.AWQ_BF16, 64, 64, FAKE, None) == -1
    assert fl(FAKE, ODD, L.AWQ_BF16, 64, 64, FAKE, None) == -1
    assert fl(FAKE, None, L.AWQ_BF16, 0, 64, FAKE, None) == -1
    assert fl(FAKE, None, L.AWQ_BF16, 64, 64, None, None) == -1
    assert "fold_linear" in L.last_error()


def test_profile_kinds_match_header(L):
    src = open(HEADER).read()
    for name, kind in L.KERNEL_KINDS.items():
        assert re.search(rf"AWQ_K_{name.upper()}\s*=\s*{kind}\b", src) or \
            (name == "scale" and re.search(rf"AWQ_K_SCALE\s*=\s*{kind}\b", src)), name
    count = int(re.search(r"AWQ_K_COUNT\s*=\s*(\d+)", src).group(1))
    assert count == len(L.KERNEL_KINDS)


def test_w3a16_workspace_and_rejects(L):
    lib = L.lib()
    wsb = lib.awq_w3a16_workspace_bytes
    # decode (T <= 16): float32 partials per k chunk, token row and output row
    one = wsb(1, 4096, 4096, L.AWQ_BF16)
    assert one > 0 and one % (4096 * 4) == 0 and one <= 32 * 4096 * 4
    assert wsb(16, 4096, 4096, L.AWQ_F16) == 16 * one
    # prefill: the dequantised [N, K] operand rows
    assert wsb(17, 4096, 4096, L.AWQ_BF16) == 4096 * 4096 * 2
    assert wsb(4096, 4096, 4096, L.AWQ_F16) == 4096 * 4096 * 2
    assert wsb(1, 4104, 4096, L.AWQ_BF16) == 0                     # N not a multiple of 32
    assert wsb(1, 4096, 4096, L.AWQ_F32) == 0
    f = lib.awq_w3a16_matmul
    big = 1 << 40
    call = lambda **k: f(k.get("X", FAKE), k.get("dt", L.AWQ_BF16), k.get("T", 4),
                         k.get("N", 256), k.get("K", 256), FAKE, FAKE, FAKE, k.get("g", 128),
                         k.get("Y", FAKE), FAKE, k.get("wsb", big), None)
    assert call(X=None) == -1
    assert call(dt=L.AWQ_F32) == -2
    assert call(N=264) == -1
    assert "multiple of 32" in L.last_error()
    assert call(K=200) == -1
    assert call(g=16) == -2
    assert call(wsb=16) == -3
    assert "w3a16_matmul" in L.last_error()


def test_w4a16_workspace_and_rejects(L):
    lib = L.lib()
    wsb = lib.awq_w4a16_workspace_bytes
    # GEMM path (T > 16): the dequantised [N, K] operand rows (a smaller
    # workspace selects the on-the-fly GEMM, below)
    assert wsb(4096, 4096, 4096, L.AWQ_BF16) == 4096 * 4096 * 2
    # GEMV path: float32 partials per k chunk, token row and output channel
    one = wsb(1, 4096, 4096, L.AWQ_BF16)
    assert one > 0 and one % (4096 * 4) == 0 and one <= 32 * 4096 * 4
    assert wsb(16, 4096, 4096, L.AWQ_F16) == 16 * one
    for bad in ((0, 8, 128, 1), (1, 12, 128, 1), (1, 8, 200, 1), (1, 8, 128, 0), (1, 8, 128, 9)):
        assert wsb(*bad) == 0
    f = lib.awq_w4a16_matmul

    def call(**k):
        a = dict(X=FAKE, dt=L.AWQ_BF16, T=4, N=64, K=256, qw=FAKE, qz=FAKE, sc=FAKE, g=128,
                 Y=FAKE, ws=FAKE, wsb=1 << 30)
        a.update(k)
        return f(a["X"], a["dt"], a["T"], a["N"], a["K"], a["qw"], a["qz"], a["sc"], a["g"],
                 a["Y"], a["ws"], a["wsb"], None)

    assert call(X=None) == -1
    assert call(Y=None) == -1
    assert call(dt=L.AWQ_F32) == -2
    assert call(dt=9) == -1
    assert call(T=0) == -1
    assert call(N=12) == -1
    assert call(K=200) == -1
    assert call(g=16) == -2
    assert call(X=MIS) == -1
    assert call(sc=ctypes.c_void_p(0x10008)) == -1        # scales need 16-byte alignment
    assert call(Y=ctypes.c_void_p(0x10001)) == -1
    assert call(wsb=16) == -3
    assert call(ws=MIS) == -3
    assert "w4a16_matmul" in L.last_error()
    # prefill with too small a workspace is only for layers the on-the-fly
    # GEMM can address (K·N/2 < 2^31 bytes)
    assert call(T=4096, N=65536, K=65536, ws=None, wsb=0) == -3
    assert call(T=4096, N=65536, K=65536, wsb=16) == -3


def test_prepared_gram_sizes_and_rejects(L):
    lib = L.lib()
    ws = lib.awq_workspace_bytes
    T, K = 65536, 4096
    gbytes = lib.awq_gram_bytes(K)
    assert gbytes == K * (2 * K + 256) * 2            # upper tiles' hi/lo rows, padded
    assert lib.awq_gram_bytes(200) == 0 and lib.awq_gram_bytes(0) == 0
    build = ws(L.AWQ_OP_GRAM_BUILD, T, 1, K, 1, L.AWQ_BF16)
    gp = 15 * 136 * 256 * 256 * 4                     # 15 token slices x 136 upper tiles
    assert build == gp                                # X is read in place: no X^T
    assert ws(L.AWQ_OP_GRAM_BUILD, T, 1, K, 1, L.AWQ_F32) == 0
    for with_g, op in ((L.AWQ_OP_SEARCH_SCALE_GRAM_G, L.AWQ_OP_SEARCH_SCALE_GRAM),
                       (L.AWQ_OP_SEARCH_CLIP_GRAM_G, L.AWQ_OP_SEARCH_CLIP_GRAM)):
        # a prepared G: no partial tiles or G in the search's workspace
        assert ws(with_g, T, 4096, K, 20, L.AWQ_BF16) == \
            ws(op, T, 4096, K, 20, L.AWQ_BF16) - build - gbytes
        assert lib.awq_workspace_bytes_batch(with_g, T, 4096, K, 20, 1, L.AWQ_BF16) > 0
    f = lib.awq_gram_build
    big = 1 << 40
    assert f(FAKE, L.AWQ_BF16, T, K, None, big, FAKE, big, None) == -1
    assert f(FAKE, L.AWQ_F32, T, K, FAKE, big, FAKE, big, None) == -2
    assert f(FAKE, L.AWQ_BF16, T, 200, FAKE, big, FAKE, big, None) == -1
    assert f(FAKE, L.AWQ_BF16, 1 << 31, K, FAKE, big, FAKE, big, None) == -1   # past 2^31 - 1
    assert f(MIS, L.AWQ_BF16, T, K, FAKE, big, FAKE, big, None) == -1
    assert f(FAKE, L.AWQ_BF16, T, K, FAKE, gbytes - 1, FAKE, big, None) == -3
    assert f(FAKE, L.AWQ_BF16, T, K, FAKE, gbytes, FAKE, build - 1, None) == -3
    assert "gram_build" in L.last_error()
    a_best = ctypes.c_float()
    mse = (ctypes.c_double * 3)()
    g = L.float_array([0.0, 0.5, 1.0])
    qc = L.QConfig(4, 128, 1)
    sg = lib.awq_search_scale_gram_g
    assert sg(None, FAKE, L.AWQ_BF16, 256, 256, 256, FAKE, g, 3, qc, FAKE, ctypes.byref(a_best),
              mse, None, FAKE, big, None) == -1
    assert sg(FAKE, FAKE, L.AWQ_F32, 256, 256, 256, FAKE, g, 3, qc, FAKE, ctypes.byref(a_best),
              mse, None, FAKE, big, None) == -2
    assert "search_scale_gram_g" in L.last_error()
    mc = ctypes.c_double()
    cg = lib.awq_search_clip_gram_g
    r = L.float_array([0.5, 1.0])
    assert cg(FAKE, FAKE, L.AWQ_BF16, 256, 256, 200, FAKE, r, 2, qc, FAKE, ctypes.byref(mc), None,
              FAKE, big, None) == -1
    assert cg(FAKE, FAKE, L.AWQ_BF16, 256, 256, 256, FAKE, r, 2, qc, FAKE, ctypes.byref(mc), None,
              FAKE, 16, None) == -3
    gg = lib.awq_search_scale_group_gram_g
    wp = (ctypes.c_void_p * 2)(FAKE.value, FAKE.value)
    nv = (ctypes.c_int64 * 2)(256, 128)
    assert gg(FAKE, wp, nv, 2, L.AWQ_F16, 256, 256, FAKE, g, 3, qc, FAKE, ctypes.byref(a_best),
              mse, None, FAKE, big, None) == -2


def test_gram_workspace_and_rejects(L):
    lib = L.lib()
    ws = lib.awq_workspace_bytes
    direct = ws(L.AWQ_OP_SEARCH_SCALE, 65536, 4096, 4096, 20, L.AWQ_BF16)
    gram = ws(L.AWQ_OP_SEARCH_SCALE_GRAM, 65536, 4096, 4096, 20, L.AWQ_BF16)
    gs = 4096 * 8192 * 2
    # the build's float32 partial tiles: 15 token slices (136 upper tiles x 15
    # slices = 2040 units, 8 rounds of 256 CUs: the fewest rounds per slice
    # length for S <= 16) of 136 tiles of 256x256
    gp = 15 * 136 * 256 * 256 * 4
    # partials shrink to K/256 row tiles; the G build's partial tiles and the
    # G halves are added (X is read in place)
    assert gram > direct - 256 * 20 * 4096 * 4 + gp + gs - (1 << 20)
    assert gram < direct + gp + gs
    assert ws(L.AWQ_OP_SEARCH_SCALE_GRAM, 65536, 4096, 4096, 20, L.AWQ_F32) == 0
    assert ws(L.AWQ_OP_SEARCH_CLIP_GRAM, 700, 300, 384, 5, L.AWQ_BF16) > 384 * 768 * 2 + 384 * 768 * 2
    assert lib.awq_workspace_bytes_batch(L.AWQ_OP_SEARCH_CLIP_GRAM, 700, 300, 384, 5, 1,
                                         L.AWQ_BF16) > 0
    a_best = ctypes.c_float()
    mse = (ctypes.c_double * 3)()
    g = L.float_array([0.0, 0.5, 1.0])
    qc = L.QConfig(4, 128, 1)
    f = lib.awq_search_scale_gram
    assert f(FAKE, FAKE, L.AWQ_F32, 256, 256, 256, FAKE, g, 3, qc, FAKE, ctypes.byref(a_best), mse,
             None, FAKE, 1 << 40, None) == -2
    # fp16 layers go through the direct searches; the Gram path is bf16 only
    assert f(FAKE, FAKE, L.AWQ_F16, 256, 256, 256, FAKE, g, 3, qc, FAKE, ctypes.byref(a_best), mse,
             None, FAKE, 1 << 40, None) == -2
    assert f(FAKE, FAKE, L.AWQ_BF16, 1 << 31, 256, 256, FAKE, g, 3, qc, FAKE,
             ctypes.byref(a_best), mse, None, FAKE, 1 << 40, None) == -1
    assert f(FAKE, FAKE, L.AWQ_BF16, 256, 256, 200, FAKE, g, 3, qc, FAKE, ctypes.byref(a_best),
             mse, None, FAKE, 1 << 40, None) == -1
    need1 = lib.awq_workspace_bytes_batch(L.AWQ_OP_SEARCH_SCALE_GRAM, 256, 256, 256, 3, 1,
                                          L.AWQ_BF16)
    assert f(FAKE, FAKE, L.AWQ_BF16, 256, 256, 256, FAKE, g, 3, qc, FAKE, ctypes.byref(a_best),
             mse, None, FAKE, need1 - 1, None) == -3
    assert "search_scale_gram" in L.last_error()
    mc = ctypes.c_double()
    assert lib.awq_search_clip_gram(FAKE, FAKE, L.AWQ_BF16, 256, 256, 256, FAKE,
                                    L.float_array([0.0, 1.0]), 2, qc, FAKE, ctypes.byref(mc),
                                    None, FAKE, 1 << 40, None) == -1      # ratio 0 is invalid


def test_stats_noalloc_rejects(L):
    """The allocation-free stats entry point checks its arguments on the host,
    and refuses sizes whose float64 partials exceed its static 2^20-double
    scratch (before any device work)."""
    lib = L.lib()
    f = lib.awq_act_stats_noalloc
    assert f(None, L.AWQ_BF16, 64, 4096, FAKE, None) == L.AWQ_E_INVALID
    assert f(FAKE, L.AWQ_BF16, 64, 4096, None, None) == L.AWQ_E_INVALID
    assert f(MIS, L.AWQ_BF16, 64, 4096, FAKE, None) == L.AWQ_E_INVALID
    assert f(FAKE, L.AWQ_BF16, 64, 4100, FAKE, None) == L.AWQ_E_INVALID      # K % 8
    assert f(FAKE, 9, 64, 4096, FAKE, None) == L.AWQ_E_INVALID
    assert f(FAKE, L.AWQ_BF16, 0, 4096, FAKE, None) == L.AWQ_E_INVALID
    # 64 tokens make one chunk: K = 2^20 partials fit exactly, 2^20 + 8 do not
    assert f(FAKE, L.AWQ_BF16, 64, (1 << 20) + 8, FAKE, None) == L.AWQ_E_UNSUPPORTED
    assert "static scratch" in L.last_error()
    ws = lib.awq_workspace_bytes
    assert ws(L.AWQ_OP_STATS, 64, 1, 1 << 20, 1, L.AWQ_BF16) == 8 << 20
    # the benchmark layer's partials fit (64K tokens x 4096 channels, bf16 and f32)
    for dt in (L.AWQ_BF16, L.AWQ_F16, L.AWQ_F32):
        assert ws(L.AWQ_OP_STATS, 65536, 1, 4096, 1, dt) <= 8 << 20
        assert ws(L.AWQ_OP_STATS, 65536, 1, 11008, 1, dt) <= 8 << 20


def test_32bit_offset_edges(L):
    """Sizes at the edges of the kernels' 32-bit tile offsets and grids: the
    largest accepted size gets past the shape checks (it then fails only on
    the deliberately small workspace, AWQ_E_WORKSPACE), the next one is
    refused (AWQ_E_UNSUPPORTED). The search GEMM's 256-row tiles need
    512·K < 2^31 (split: 512·2K); the Gram search's 512·(2K + 256) (the
    Gram build reads X one 64-token k-tile at a time and takes any token
    count); the consumer GEMM's 512·K;
    element-wise launches N·K <= 2^34; the candidate GEMM's grid < 2^32
    work-items."""
    lib = L.lib()
    a_best = ctypes.c_float()
    mse = (ctypes.c_double * 4)()
    g = L.float_array([0.5])
    WS, UN = L.AWQ_E_WORKSPACE, L.AWQ_E_UNSUPPORTED

    def scale(fn, T, N, K, dt=L.AWQ_BF16, flags=0, X=FAKE):
        return fn(X, FAKE, dt, T, N, K, FAKE, g, 1, L.QConfig(4, 128, 1, flags), FAKE,
                  ctypes.byref(a_best), mse, None, FAKE, 1000, None)

    k22 = 1 << 22
    assert scale(lib.awq_search_scale, 256, 256, k22 - 128) == WS
    assert scale(lib.awq_search_scale, 256, 256, k22) == UN
    assert "32-bit tile offsets" in L.last_error()
    assert scale(lib.awq_search_scale, 256, 256, k22 // 2 - 128, flags=1) == WS
    assert scale(lib.awq_search_scale, 256, 256, k22 // 2, flags=1) == UN
    assert scale(lib.awq_search_scale, 256, 256, k22, dt=L.AWQ_F32) == WS     # 64-bit indices
    mc = ctypes.c_double()
    clip = lambda K: lib.awq_search_clip(FAKE, FAKE, L.AWQ_F16, 256, 256, K, FAKE, g, 1,
                                         L.QConfig(4, 128, 1), FAKE, ctypes.byref(mc), None, FAKE,
                                         1000, None)
    assert clip(k22 - 128) == WS and clip(k22) == UN
    # Gram: 2K + 256 per G row; any token count up to the shape limit 2^31 - 1
    t_max = (1 << 31) - 1
    assert scale(lib.awq_search_scale_gram, t_max, 256, 256) == WS
    assert scale(lib.awq_search_scale_gram_g, 256, 256, k22 // 2 - 256) == WS
    assert scale(lib.awq_search_scale_gram_g, 256, 256, k22 // 2 - 128) == UN
    big = 1 << 40
    gb = lib.awq_gram_build
    assert gb(FAKE, L.AWQ_BF16, t_max, 256, FAKE, 0, FAKE, big, None) == WS
    assert gb(FAKE, L.AWQ_BF16, 256, k22 // 2 - 128, FAKE, 0, FAKE, big, None) == UN
    assert lib.awq_workspace_bytes(L.AWQ_OP_GRAM_BUILD, t_max, 1, 256, 1, L.AWQ_BF16) > 0
    # the candidate GEMM's grid: 2^31 - 1 tokens x 2^20 rows is past 2^32 work-items
    assert scale(lib.awq_search_scale, (1 << 31) - 1, 1 << 20, 128) == UN
    assert "grid" in L.last_error()
    # element-wise launches: N·K <= 2^34
    assert scale(lib.awq_search_scale, 256, 1 << 20, 1 << 14) == WS
    assert scale(lib.awq_search_scale, 256, (1 << 20) + 8, 1 << 14) == UN
    pk = lambda N, K: lib.awq_quantize_pack(FAKE, L.AWQ_BF16, N, K, FAKE, None,
                                            L.QConfig(4, 128, 1), FAKE, FAKE, FAKE, FAKE, 0, None)
    assert pk(1 << 20, 1 << 14) == WS and pk((1 << 20) + 8, 1 << 14) == UN
    assert pk(8, k22 - 128) == WS and pk(8, k22) == UN
    # a workgroup's 128 qweight rows of N/8 words: 64·N < 2^31
    assert pk((1 << 25) - 8, 128) == WS and pk(1 << 25, 128) == UN
    # the consumer: 512·K < 2^31 on every path (T = 1 needs its workspace)
    wm = lambda K, fn=lib.awq_w4a16_matmul: fn(FAKE, L.AWQ_BF16, 1, 32, K, FAKE, FAKE, FAKE, 128,
                                               FAKE, FAKE, 0, None)
    assert wm(k22 - 128) == WS and wm(k22) == UN
    assert wm(k22 - 128, lib.awq_w3a16_matmul) == WS and wm(k22, lib.awq_w3a16_matmul) == UN
