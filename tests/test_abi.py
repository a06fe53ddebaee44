"""C ABI checks that need no GPU: the library loads, exports every function
include/fa.h declares, and rejects invalid arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from io_aware_transformer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libfa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_functions():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_header_status_codes_match_binding():
    text = open(HEADER).read()
    for name, code in re.findall(r"(FA_(?:OK|ERR_[A-Z]+))\s*=\s*(-?\d+)", text):
        assert _lib.STATUS[int(code)] == name


def test_status_strings_and_version():
    lib = _lib.load()
    for code, name in _lib.STATUS.items():
        assert lib.fa_status_str(code).decode() == name
    assert lib.fa_status_str(12345).decode() == "FA_ERR_UNKNOWN"
    assert lib.fa_version() == 130
    assert lib.fa_last_hip_error() == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first
MIS = 0x10008   # 8-byte aligned only


def fwd(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125, causal=1,
             dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_fwd(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["Hq"], a["Hkv"], a["N"],
                              a["d"], a["scale"], a["causal"], a["dtype"], None)


def bwd(ws_bytes=1 << 20, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, LSE=FAKE, dQ=FAKE, dK=FAKE, dV=FAKE, ws=0x100000,
             B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125, causal=1, dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_bwd(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"],
                              a["ws"], ws_bytes, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"],
                              a["causal"], a["dtype"], None)


E = _lib.STATUS_CODE


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), "FA_ERR_NULL"),
    (dict(V=None), "FA_ERR_NULL"),
    (dict(O=None), "FA_ERR_NULL"),
    (dict(B=-1), "FA_ERR_SHAPE"),
    (dict(N=-5), "FA_ERR_SHAPE"),
    (dict(N=(1 << 22) + 1), "FA_ERR_SHAPE"),
    (dict(Hq=0), "FA_ERR_SHAPE"),
    (dict(Hkv=0), "FA_ERR_SHAPE"),
    (dict(Hq=3, Hkv=2), "FA_ERR_SHAPE"),
    (dict(Hq=2, Hkv=4), "FA_ERR_SHAPE"),
    (dict(d=96), "FA_ERR_HEADDIM"),
    (dict(d=0), "FA_ERR_HEADDIM"),
    (dict(dtype=7), "FA_ERR_DTYPE"),
    (dict(Q=MIS), "FA_ERR_ALIGN"),
    (dict(LSE=MIS), "FA_ERR_ALIGN"),
    (dict(causal=2), "FA_ERR_ARG"),
    (dict(scale=float("nan")), "FA_ERR_ARG"),
    (dict(scale=float("inf")), "FA_ERR_ARG"),
    (dict(scale=3.0e38), "FA_ERR_ARG"),  # finite, but scale * log2(e) overflows float
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == E[code]


def test_fwd_empty_is_noop():
    # nothing to compute: no pointer is touched, no kernel launched
    assert fwd(Q=None, K=None, V=None, O=None, LSE=None, N=0) == 0
    assert fwd(Q=None, K=None, V=None, O=None, LSE=None, B=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dO=None), "FA_ERR_NULL"),
    (dict(LSE=None), "FA_ERR_NULL"),
    (dict(dK=None), "FA_ERR_NULL"),
    (dict(d=256), "FA_ERR_UNSUPPORTED"),
    (dict(d=48), "FA_ERR_HEADDIM"),
    (dict(dV=MIS), "FA_ERR_ALIGN"),
    (dict(ws=0x100010), "FA_ERR_ALIGN"),
    (dict(ws=None), "FA_ERR_WORKSPACE"),
    (dict(Hq=4, Hkv=3), "FA_ERR_SHAPE"),
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == E[code]


def test_bwd_workspace_too_small():
    need = _lib.load().fa_bwd_workspace_size(1, 2, 1, 16, 64, _lib.FA_BF16)
    assert need >= 2 * 16 * 4 and need % 256 == 0
    assert bwd(ws_bytes=need - 1) == E["FA_ERR_WORKSPACE"]


def test_workspace_size_formula():
    lib = _lib.load()
    # D term: float32 per (batch, query head, row), rounded up to 256 bytes
    assert lib.fa_bwd_workspace_size(4, 16, 16, 4096, 64, _lib.FA_BF16) == 4 * 16 * 4096 * 4
    assert lib.fa_bwd_workspace_size(1, 1, 1, 3, 64, _lib.FA_BF16) == 256
    assert lib.fa_bwd_workspace_size(0, 1, 1, 3, 64, _lib.FA_BF16) == 0
    assert lib.fa_bwd_workspace_size(1, 3, 2, 3, 64, _lib.FA_BF16) == 0  # invalid shape


def test_workspace_size_grouped_split():
    """Grouped heads add float partial dK / dV per query-head slice when the
    dK/dV grid (128 keys per workgroup) is under two workgroups per compute
    unit; 256 compute units stand in for a host without a device."""
    lib = _lib.load()
    d_term = lambda B, Hq, N: (B * Hq * N * 4 + 255) // 256 * 256
    part = lambda S, B, Hkv, N, d: (S * B * Hkv * N * d * 4 + 255) // 256 * 256
    # B1 Hq16 Hkv1 N8192: 64 workgroups, doubled to 512 at S = 8
    assert lib.fa_bwd_workspace_size(1, 16, 1, 8192, 128, _lib.FA_BF16) == d_term(1, 16, 8192) + 2 * part(8, 1, 1, 8192, 128)
    # B2 Hq32 Hkv8 N2048: 256 workgroups, S = 2
    assert lib.fa_bwd_workspace_size(2, 32, 8, 2048, 64, _lib.FA_BF16) == d_term(2, 32, 2048) + 2 * part(2, 2, 8, 2048, 64)
    # already 512 workgroups: no split
    assert lib.fa_bwd_workspace_size(8, 16, 4, 2048, 128, _lib.FA_BF16) == d_term(8, 16, 2048)
    # S divides the group: G = 3 cannot split
    assert lib.fa_bwd_workspace_size(1, 3, 1, 1000, 64, _lib.FA_BF16) == d_term(1, 3, 1000)
    # float32 has no split
    assert lib.fa_bwd_workspace_size(1, 16, 1, 8192, 128, _lib.FA_FP32) == d_term(1, 16, 8192)


def test_bwd_empty_is_noop():
    assert bwd(Q=None, K=None, V=None, O=None, dO=None, LSE=None, dQ=None, dK=None, dV=None, ws=None, N=0) == 0


def split(ws_bytes=1 << 24, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, ws=0x100000, B=2, Hq=8, Hkv=2, Nq=1, Nk=1000, d=128,
             scale=0.09, causal=1, splits=0, dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_fwd_split(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                    a["Nk"], a["d"], a["scale"], a["causal"], a["splits"], a["ws"], ws_bytes,
                                    a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), "FA_ERR_NULL"),
    (dict(O=None), "FA_ERR_NULL"),
    (dict(Nk=0), "FA_ERR_SHAPE"),
    (dict(Nq=-1), "FA_ERR_SHAPE"),
    (dict(Nk=(1 << 22) + 1), "FA_ERR_SHAPE"),
    (dict(Hq=6, Hkv=4), "FA_ERR_SHAPE"),
    (dict(d=80), "FA_ERR_HEADDIM"),
    (dict(d=256), "FA_ERR_UNSUPPORTED"),
    (dict(dtype=_lib.FA_FP32), "FA_ERR_UNSUPPORTED"),
    (dict(dtype=3), "FA_ERR_DTYPE"),
    (dict(splits=-1), "FA_ERR_ARG"),
    (dict(splits=4097), "FA_ERR_ARG"),
    (dict(causal=5), "FA_ERR_ARG"),
    (dict(K=MIS), "FA_ERR_ALIGN"),
    (dict(ws=0x100040), "FA_ERR_ALIGN"),
    (dict(ws=None), "FA_ERR_WORKSPACE"),
])
def test_split_rejects(kw, code):
    assert split(**kw) == E[code]


def test_split_workspace_and_parts():
    lib = _lib.load()
    # explicit splits: parts x rows x (d + 1) floats, each array rounded to 256 bytes
    rows = 2 * 8 * 3
    want = (7 * rows * 128 * 4 + 255) // 256 * 256 + (7 * rows * 4 + 255) // 256 * 256
    assert lib.fa_fwd_split_parts(2, 8, 2, 3, 1000, 128, 7) == 7
    assert lib.fa_fwd_split_workspace_size(2, 8, 2, 3, 1000, 128, 7, _lib.FA_BF16) == want
    # default: one workgroup per compute unit (3 waves at d = 128, 4 at d = 64),
    # at least 4 tiles of 32 keys per part
    assert lib.fa_fwd_split_parts(4, 32, 8, 1, 16384, 128, 0) == 24
    assert lib.fa_fwd_split_parts(4, 32, 8, 1, 16384, 64, 0) == 32
    assert lib.fa_fwd_split_parts(1, 1, 1, 1, 100, 64, 0) == 1
    assert lib.fa_fwd_split_parts(0, 8, 2, 1, 100, 64, 0) == 0
    assert lib.fa_fwd_split_workspace_size(2, 8, 2, 0, 1000, 128, 3, _lib.FA_BF16) == 0
    need = lib.fa_fwd_split_workspace_size(2, 8, 2, 1, 1000, 128, 0, _lib.FA_BF16)
    assert split(ws_bytes=need - 1) == E["FA_ERR_WORKSPACE"]


def test_split_empty_is_noop():
    assert split(Q=None, K=None, V=None, O=None, LSE=None, ws=None, Nq=0) == 0
    assert split(Q=None, K=None, V=None, O=None, LSE=None, ws=None, B=0) == 0


def merge(**kw):
    a = dict(Op=FAKE, Lp=FAKE, parts=3, rows=10, d=128, O=FAKE, LSE=FAKE, dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_lse_merge(a["Op"], a["Lp"], a["parts"], a["rows"], a["d"], a["O"], a["LSE"], a["dtype"],
                                    None)


@pytest.mark.parametrize("kw,code", [
    (dict(Op=None), "FA_ERR_NULL"),
    (dict(O=None), "FA_ERR_NULL"),
    (dict(parts=0), "FA_ERR_ARG"),
    (dict(rows=-1), "FA_ERR_SHAPE"),
    (dict(d=32), "FA_ERR_HEADDIM"),
    (dict(dtype=9), "FA_ERR_DTYPE"),
    (dict(Lp=MIS), "FA_ERR_ALIGN"),
])
def test_merge_rejects(kw, code):
    assert merge(**kw) == E[code]


def test_merge_empty_is_noop():
    assert merge(Op=None, Lp=None, O=None, LSE=None, rows=0) == 0


def fwdw(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125, wl=4, wr=0,
             dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_fwd_window(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["Hq"], a["Hkv"], a["N"],
                                     a["d"], a["scale"], a["wl"], a["wr"], a["dtype"], None)


def bwdw(ws_bytes=1 << 20, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, LSE=FAKE, dQ=FAKE, dK=FAKE, dV=FAKE, ws=0x100000,
             B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125, wl=4, wr=0, dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_bwd_window(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"],
                                     a["ws"], ws_bytes, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"],
                                     a["wl"], a["wr"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(wl=-2), "FA_ERR_ARG"),
    (dict(wr=-3), "FA_ERR_ARG"),
    (dict(Q=None), "FA_ERR_NULL"),
    (dict(d=40), "FA_ERR_HEADDIM"),
    (dict(Hq=3, Hkv=2), "FA_ERR_SHAPE"),
    (dict(O=MIS), "FA_ERR_ALIGN"),
    (dict(scale=float("nan")), "FA_ERR_ARG"),
])
def test_fwd_window_rejects(kw, code):
    assert fwdw(**kw) == E[code]


@pytest.mark.parametrize("kw,code", [
    (dict(wl=-5), "FA_ERR_ARG"),
    (dict(dV=None), "FA_ERR_NULL"),
    (dict(d=256), "FA_ERR_UNSUPPORTED"),
    (dict(ws=None), "FA_ERR_WORKSPACE"),
])
def test_bwd_window_rejects(kw, code):
    assert bwdw(**kw) == E[code]


def test_window_empty_is_noop():
    assert fwdw(Q=None, K=None, V=None, O=None, LSE=None, N=0) == 0
    assert bwdw(Q=None, K=None, V=None, O=None, dO=None, LSE=None, dQ=None, dK=None, dV=None, ws=None, B=0) == 0


def fwdv(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, cu=FAKE, batch=2, total=40, mx=30, Hq=2, Hkv=1, d=64,
             scale=0.125, causal=1, dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_fwd_varlen(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["cu"], a["batch"], a["total"],
                                     a["mx"], a["Hq"], a["Hkv"], a["d"], a["scale"], a["causal"], a["dtype"], None)


def bwdv(ws_bytes=1 << 20, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, LSE=FAKE, dQ=FAKE, dK=FAKE, dV=FAKE, ws=0x100000, cu=FAKE,
             batch=2, total=40, mx=30, Hq=2, Hkv=1, d=64, scale=0.125, causal=1, dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_bwd_varlen(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"],
                                     a["ws"], ws_bytes, a["cu"], a["batch"], a["total"], a["mx"], a["Hq"], a["Hkv"],
                                     a["d"], a["scale"], a["causal"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), "FA_ERR_NULL"),
    (dict(Q=None), "FA_ERR_NULL"),
    (dict(cu=FAKE + 2), "FA_ERR_ALIGN"),
    (dict(O=MIS), "FA_ERR_ALIGN"),
    (dict(total=-1), "FA_ERR_SHAPE"),
    (dict(batch=-1), "FA_ERR_SHAPE"),
    (dict(mx=-1), "FA_ERR_SHAPE"),
    (dict(mx=(1 << 22) + 1), "FA_ERR_SHAPE"),
    (dict(Hq=3, Hkv=2), "FA_ERR_SHAPE"),
    (dict(d=96), "FA_ERR_HEADDIM"),
    (dict(dtype=5), "FA_ERR_DTYPE"),
    (dict(causal=2), "FA_ERR_ARG"),
    (dict(scale=float("inf")), "FA_ERR_ARG"),
])
def test_fwd_varlen_rejects(kw, code):
    assert fwdv(**kw) == E[code]


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), "FA_ERR_NULL"),
    (dict(dK=None), "FA_ERR_NULL"),
    (dict(d=256), "FA_ERR_UNSUPPORTED"),
    (dict(ws=None), "FA_ERR_WORKSPACE"),
    (dict(total=-3), "FA_ERR_SHAPE"),
    (dict(dtype=_lib.FA_FP32), "FA_ERR_UNSUPPORTED"),
])
def test_bwd_varlen_rejects(kw, code):
    assert bwdv(**kw) == E[code]


def test_bwd_varlen_workspace_too_small():
    need = _lib.load().fa_bwd_varlen_workspace_size(40, 2, 1, 64, _lib.FA_BF16)
    assert need == (2 * 40 * 4 + 255) // 256 * 256
    assert bwdv(ws_bytes=need - 1) == E["FA_ERR_WORKSPACE"]
    assert bwdv(ws=0x100010) == E["FA_ERR_ALIGN"]


def test_varlen_workspace_size():
    f = _lib.load().fa_bwd_varlen_workspace_size
    assert f(16384, 16, 16, 128, _lib.FA_BF16) == 16 * 16384 * 4
    assert f(0, 16, 16, 128, _lib.FA_BF16) == 0
    assert f(100, 16, 3, 128, _lib.FA_BF16) == 0  # invalid heads
    assert f(100, 16, 16, 48, _lib.FA_BF16) == 0  # invalid d


def test_varlen_empty_is_noop():
    none = dict(Q=None, K=None, V=None, O=None, LSE=None, cu=None)
    assert fwdv(batch=0, **none) == 0
    assert fwdv(total=0, **none) == 0
    assert fwdv(mx=0, **none) == 0
    gnone = dict(none, dO=None, dQ=None, dK=None, dV=None, ws=None)
    assert bwdv(batch=0, **gnone) == 0
    assert bwdv(total=0, **gnone) == 0


def bwdn(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, LSE=FAKE, dQ=FAKE, dK=FAKE, dV=FAKE,
             B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125, causal=1, dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_bwd_noalloc(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"],
                                      a["dV"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"],
                                      a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), "FA_ERR_NULL"),
    (dict(dV=None), "FA_ERR_NULL"),
    (dict(Hq=3, Hkv=2), "FA_ERR_SHAPE"),
    (dict(d=96), "FA_ERR_HEADDIM"),
    (dict(d=256), "FA_ERR_UNSUPPORTED"),
    (dict(causal=2), "FA_ERR_ARG"),
    (dict(scale=float("inf")), "FA_ERR_ARG"),
    (dict(dtype=7), "FA_ERR_DTYPE"),
    # the fixed buffer holds FA_NOALLOC_MAX_ROWS rows of D_i
    (dict(B=1, Hq=16, Hkv=16, N=_lib.FA_NOALLOC_MAX_ROWS // 16 + 1), "FA_ERR_WORKSPACE"),
    (dict(B=2, Hq=1, Hkv=1, N=_lib.FA_NOALLOC_MAX_ROWS // 2 + 1), "FA_ERR_WORKSPACE"),
])
def test_bwd_noalloc_rejects(kw, code):
    assert bwdn(**kw) == E[code]


def test_bwd_noalloc_empty_is_noop():
    assert bwdn(B=0, Q=None) == E["FA_OK"]
    assert bwdn(N=0, Q=None) == E["FA_OK"]


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_MAX_ROWS \(1 << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == _lib.FA_NOALLOC_MAX_ROWS


def fwdd(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125, causal=1,
             p=0.1, seed=1, off=0, dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_fwd_dropout(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["Hq"], a["Hkv"], a["N"],
                                      a["d"], a["scale"], a["causal"], a["p"], a["seed"], a["off"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(p=-0.01), "FA_ERR_ARG"),
    (dict(p=float("nan")), "FA_ERR_ARG"),
    (dict(p=0.999), "FA_ERR_ARG"),      # rounds to 256 / 256
    (dict(d=256), "FA_ERR_UNSUPPORTED"),
    (dict(dtype=_lib.FA_FP32), "FA_ERR_UNSUPPORTED"),
    (dict(Q=None), "FA_ERR_NULL"),
    (dict(Hq=3, Hkv=2), "FA_ERR_SHAPE"),
])
def test_fwd_dropout_rejects(kw, code):
    assert fwdd(**kw) == E[code]


def test_dropout_largest_probability_accepted():
    # 255.4 / 256 rounds to t8 = 255: valid (validation reaches the pointers)
    assert fwdd(p=255.4 / 256, Q=None) == E["FA_ERR_NULL"]
    assert fwdd(B=0, Q=None) == E["FA_OK"]


def fwds(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, mask=FAKE, B=1, Hq=2, Hkv=1, N=300, d=64, scale=0.125,
             causal=1, dtype=_lib.FA_BF16)
    a.update(kw)
    return _lib.load().fa_fwd_blocksparse(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["mask"], a["B"], a["Hq"],
                                          a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), "FA_ERR_NULL"),
    (dict(d=256), "FA_ERR_UNSUPPORTED"),
    (dict(dtype=_lib.FA_FP32), "FA_ERR_UNSUPPORTED"),
    (dict(N=_lib.FA_SPARSE_MAX_N + 1), "FA_ERR_UNSUPPORTED"),
    (dict(causal=3), "FA_ERR_ARG"),
])
def test_fwd_blocksparse_rejects(kw, code):
    assert fwds(**kw) == E[code]
