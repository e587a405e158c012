"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call.  No call here reaches
a kernel launch."""
import ctypes
import re

import pytest

import structured_sparse_state_amd as pk
from structured_sparse_state_amd import build_lib


@pytest.fixture(scope="module")
def lib():
    return pk.library()


def test_exports_every_declared_function(lib):
    names = pk.header_functions()
    assert set(names) == {"pdssm_scan_fwd", "pdssm_scan_workspace_bytes", "pdssm_select",
                          "pdssm_compose", "pdssm_strerror", "pdssm_scan_fwd_save",
                          "pdssm_scan_bwd", "pdssm_scan_bwd_workspace_bytes", "pdssm_dict_hardmax",
                          "pdssm_decode_step", "pdssm_router_select", "pdssm_scan_fwd_noalloc",
                          "pdssm_router_pack_weights"}
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("name", sorted(build_lib.VARIANTS))
def test_test_builds_export_the_same_functions(name):
    """The test builds (other chunking, reversed ticket order) load through
    the binding's variant switch and export every declared function."""
    with pk.variant(name) as v:
        assert pk.library() is v
        for n in pk.header_functions():
            assert hasattr(v, n), n
        assert pk.pdssm_scan_workspace_bytes(1, 1, 100, 8, 4, 0) > 0
    assert pk.library() is not v


def test_header_constants_match_binding():
    text = open(pk.HEADER).read()
    defs = dict(re.findall(r"#define\s+(PDSSM_[A-Z0-9_]+)\s+(-?0x[0-9A-Fa-f]+u?|-?\d+)", text))
    assert defs
    for name, val in defs.items():
        v = int(val.rstrip("u"), 0)
        assert getattr(pk, name) == v, name


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, 42):
        assert pk.pdssm_strerror(code)


FAKE = 1 << 20          # an aligned, never-dereferenced address


def _scan(**kw):
    args = dict(sel=FAKE, dict_idx=FAKE, diag=FAKE, b=FAKE, c=FAKE, y=FAKE, x_final=None,
                B=2, H=3, L=100, N=16, K=8, flags=pk.PDSSM_LOGITS_BF16, x0=None, ws=FAKE,
                ws_bytes=1 << 40)
    args.update(kw)
    return pk.pdssm_scan_fwd(args["sel"], args["dict_idx"], args["diag"], args["b"], args["c"],
                             args["y"], args["x_final"], args["B"], args["H"], args["L"], args["N"],
                             args["K"], args["flags"], args["x0"], args["ws"], args["ws_bytes"], 0)


def test_scan_argument_errors(lib):
    for name in ("sel", "dict_idx", "diag", "b", "c", "y", "ws"):
        assert _scan(**{name: None}) == pk.PDSSM_ERR_NULL, name
    for bad in (dict(B=-1), dict(H=-1), dict(L=-1), dict(N=0), dict(N=65), dict(K=0),
                dict(K=32768), dict(B=1 << 40, H=1 << 20), dict(B=1 << 40, H=1 << 20, L=0)):
        assert _scan(**bad) == pk.PDSSM_ERR_DIM, bad
    assert _scan(flags=0x40) == pk.PDSSM_ERR_FLAGS
    for name in ("sel", "dict_idx", "diag", "b", "c", "y", "ws", "x0", "x_final"):
        assert _scan(**{name: FAKE + 4}) == pk.PDSSM_ERR_ALIGN, name
    need = pk.pdssm_scan_workspace_bytes(2, 3, 100, 16, 8, pk.PDSSM_LOGITS_BF16)
    assert _scan(ws_bytes=need - 1) == pk.PDSSM_ERR_WORKSPACE


def test_empty_shapes_need_no_buffers(lib):
    """No sequences, or sequences of no steps, are valid calls with nothing to
    compute: every buffer is empty, so any pointer (NULL included) is taken
    and nothing is launched.  (With no steps and an x_final buffer the call
    writes x_final = x0; that case runs on the GPU.)"""
    none = dict(sel=None, dict_idx=None, diag=None, b=None, c=None, y=None, ws=None, ws_bytes=0)
    for shape in (dict(B=0), dict(H=0), dict(B=0, H=0, L=0), dict(L=0)):
        assert _scan(**none, **shape) == pk.PDSSM_OK, shape
    assert _scan(**none, L=0, x_final=FAKE + 4) == pk.PDSSM_ERR_ALIGN
    assert _scan(**none, L=0, x_final=FAKE, x0=FAKE + 4) == pk.PDSSM_ERR_ALIGN
    s = pk.pdssm_scan_fwd_save
    for B, H, L in ((0, 3, 100), (2, 0, 100), (2, 3, 0)):
        assert s(None, None, None, None, None, None, None, None, None, B, H, L, 16, 8, 0, None, None,
                 0, 0) == pk.PDSSM_OK
        assert _bwd(sel=None, dict_idx=None, diag=None, b=None, c=None, xch=None, gy=None, gb=None,
                    gc=None, gd=None, ws=None, ws_bytes=0, B=B, H=H, L=L) == pk.PDSSM_OK
        assert pk.pdssm_select(None, None, B, H, L, 4, 0, 0) == pk.PDSSM_OK
        assert pk.pdssm_scan_workspace_bytes(B, H, L, 16, 8, 0) > 0
        assert pk.pdssm_scan_bwd_workspace_bytes(B, H, L, 16, 8, 0) > 0
    for B, H in ((0, 3), (2, 0)):
        assert pk.pdssm_compose(None, None, None, None, None, B, H, 8, 4, 2, 0, None, 0,
                                0) == pk.PDSSM_OK
        assert _dec(sel=None, dict_idx=None, diag=None, b=None, c=None, y=None, x=None, B=B,
                    H=H) == pk.PDSSM_OK
    assert pk.pdssm_compose(FAKE, FAKE, FAKE, None, FAKE, 1, 1, 0, 4, 2, 0, None, 0,
                            0) == pk.PDSSM_ERR_NULL
    assert pk.pdssm_compose(FAKE, FAKE, FAKE, FAKE + 4, FAKE, 1, 1, 0, 4, 2, 0, None, 0,
                            0) == pk.PDSSM_ERR_ALIGN
    assert _bwd(L=0, gx0=FAKE + 4) == pk.PDSSM_ERR_ALIGN
    assert pk.pdssm_dict_hardmax(None, None, 0, 4, 8, pk.PDSSM_LOGITS_F32, 0) == pk.PDSSM_OK
    for B, L, H in ((0, 100, 3), (2, 0, 3), (2, 100, 0)):
        assert pk.pdssm_router_select(None, None, None, B, L, H, 64, 256, 0, 0) == pk.PDSSM_OK
    # the size and flag checks still apply to empty calls
    assert _scan(**none, B=0, N=65) == pk.PDSSM_ERR_DIM
    assert _scan(**none, B=0, flags=0x40) == pk.PDSSM_ERR_FLAGS
    assert pk.pdssm_router_select(None, None, None, 0, 100, 3, 64, 48, 0, 0) == pk.PDSSM_ERR_DIM


def test_select_and_compose_argument_errors(lib):
    assert pk.pdssm_select(None, FAKE, 1, 1, 1, 4, 0, 0) == pk.PDSSM_ERR_NULL
    assert pk.pdssm_select(FAKE, FAKE, 1, 1, -1, 4, 0, 0) == pk.PDSSM_ERR_DIM
    assert pk.pdssm_select(FAKE, FAKE, 1, 1, 1, 4, pk.PDSSM_COMPLEX, 0) == pk.PDSSM_ERR_FLAGS
    assert pk.pdssm_select(FAKE + 2, FAKE, 1, 1, 1, 4, 0, 0) == pk.PDSSM_ERR_ALIGN
    c = pk.pdssm_compose
    assert c(FAKE, FAKE, FAKE, None, FAKE, 1, 1, 8, 4, 2, 0, FAKE, 1 << 30, 0) == pk.PDSSM_ERR_NULL
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 70, 2, 0, FAKE, 1 << 30, 0) == pk.PDSSM_ERR_DIM
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 4, 2, pk.PDSSM_Y_BF16, FAKE, 1 << 30,
             0) == pk.PDSSM_ERR_FLAGS
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 4, 2, 0, FAKE, 16, 0) == pk.PDSSM_ERR_WORKSPACE


def test_workspace_is_linear_in_length_not_quadratic_in_state(lib):
    """O(L N) memory (Methodology, "1. Novel Selection Mechanism": the
    selected matrices are never dense, so memory drops from O(L N^2) to
    O(L N)): the workspace grows linearly in L and B*H, at most linearly in
    N, and is a small fraction of the inputs."""
    f = pk.PDSSM_LOGITS_BF16 | pk.PDSSM_COMPLEX | pk.PDSSM_BC_BF16 | pk.PDSSM_Y_BF16
    ws = lambda B, H, L, N: pk.pdssm_scan_workspace_bytes(B, H, L, N, 64, f)
    base = ws(8, 32, 4096, 64)
    assert 0 < base
    assert ws(8, 32, 8192, 64) - 256 <= 2 * (base - 256) + 1
    assert ws(16, 32, 4096, 64) - 256 <= 2 * (base - 256) + 1
    assert ws(8, 32, 4096, 32) <= base
    inputs = 8 * 32 * 4096 * (64 * 8 + 64 * 4 * 2 + 64 * 2)
    assert base < 0.03 * inputs
    assert pk.pdssm_scan_workspace_bytes(-1, 1, 1, 1, 1, 0) == 0
    assert pk.pdssm_scan_workspace_bytes(1, 1, 1, 1, 1, 0x40) == 0


def _bwd(**kw):
    args = dict(sel=FAKE, dict_idx=FAKE, diag=FAKE, b=FAKE, c=FAKE, xch=FAKE, gy=FAKE, gxf=None,
                gb=FAKE, gc=FAKE, gd=FAKE, gx0=None, B=2, H=3, L=100, N=16, K=8,
                flags=pk.PDSSM_LOGITS_BF16, ws=FAKE, ws_bytes=1 << 40)
    args.update(kw)
    a = args
    return pk.pdssm_scan_bwd(a["sel"], a["dict_idx"], a["diag"], a["b"], a["c"], a["xch"], a["gy"],
                             a["gxf"], a["gb"], a["gc"], a["gd"], a["gx0"], a["B"], a["H"], a["L"],
                             a["N"], a["K"], a["flags"], a["ws"], a["ws_bytes"], 0)


def test_bwd_and_save_argument_errors(lib):
    for name in ("sel", "dict_idx", "diag", "b", "c", "xch", "gy", "gb", "gc", "gd", "ws"):
        assert _bwd(**{name: None}) == pk.PDSSM_ERR_NULL, name
    for bad in (dict(B=-1), dict(L=-1), dict(N=65), dict(K=0)):
        assert _bwd(**bad) == pk.PDSSM_ERR_DIM, bad
    assert _bwd(flags=0x40) == pk.PDSSM_ERR_FLAGS
    for name in ("sel", "diag", "xch", "gy", "gxf", "gb", "gd", "gx0", "ws"):
        assert _bwd(**{name: FAKE + 4}) == pk.PDSSM_ERR_ALIGN, name
    need = pk.pdssm_scan_bwd_workspace_bytes(2, 3, 100, 16, 8, pk.PDSSM_LOGITS_BF16)
    assert need > 0
    assert _bwd(ws_bytes=need - 1) == pk.PDSSM_ERR_WORKSPACE
    assert pk.pdssm_scan_bwd_workspace_bytes(-1, 1, 1, 1, 1, 0) == 0
    s = pk.pdssm_scan_fwd_save
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 2, 3, 100, 16, 8, 0, None, FAKE,
             1 << 40, 0) == pk.PDSSM_ERR_NULL
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 8, None, 2, 3, 100, 16, 8, 0, None,
             FAKE, 1 << 40, 0) == pk.PDSSM_ERR_ALIGN
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE + 2, 2, 3, 100, 16, 8, 0, None,
             FAKE, 1 << 40, 0) == pk.PDSSM_ERR_ALIGN


def test_bwd_workspace_is_linear(lib):
    f = pk.PDSSM_LOGITS_BF16 | pk.PDSSM_COMPLEX | pk.PDSSM_BC_BF16 | pk.PDSSM_Y_BF16
    ws = lambda B, H, L: pk.pdssm_scan_bwd_workspace_bytes(B, H, L, 64, 64, f)
    base = ws(8, 32, 4096)
    assert ws(8, 32, 8192) <= 2 * base
    assert ws(16, 32, 4096) <= 2 * base


def test_dict_hardmax_argument_errors(lib):
    h = pk.pdssm_dict_hardmax
    f = pk.PDSSM_LOGITS_F32
    assert h(None, FAKE, 2, 4, 8, f, 0) == pk.PDSSM_ERR_NULL
    assert h(FAKE, None, 2, 4, 8, f, 0) == pk.PDSSM_ERR_NULL
    for H, K, N in ((-1, 4, 8), (2, 0, 8), (2, 4, 0), (2, 4, 65), (2, 32768, 8)):
        assert h(FAKE, FAKE, H, K, N, f, 0) == pk.PDSSM_ERR_DIM, (H, K, N)
    for bad in (pk.PDSSM_SEL_I32, pk.PDSSM_SEL_I16, f | pk.PDSSM_COMPLEX):
        assert h(FAKE, FAKE, 2, 4, 8, bad, 0) == pk.PDSSM_ERR_FLAGS, bad
    assert h(FAKE + 4, FAKE, 2, 4, 8, f, 0) == pk.PDSSM_ERR_ALIGN
    assert h(FAKE, FAKE + 4, 2, 4, 8, pk.PDSSM_LOGITS_BF16, 0) == pk.PDSSM_ERR_ALIGN


def _dec(**kw):
    args = dict(sel=FAKE, dict_idx=FAKE, diag=FAKE, b=FAKE, c=FAKE, y=FAKE, x=FAKE, B=2, H=3, N=16,
                K=8, flags=pk.PDSSM_LOGITS_BF16)
    args.update(kw)
    return pk.pdssm_decode_step(args["sel"], args["dict_idx"], args["diag"], args["b"], args["c"],
                                args["y"], args["x"], args["B"], args["H"], args["N"], args["K"],
                                args["flags"], 0)


def test_decode_argument_errors(lib):
    for name in ("sel", "dict_idx", "diag", "b", "c", "y", "x"):
        assert _dec(**{name: None}) == pk.PDSSM_ERR_NULL, name
    for bad in (dict(B=-1), dict(H=-1), dict(N=0), dict(N=65), dict(K=0), dict(K=40000)):
        assert _dec(**bad) == pk.PDSSM_ERR_DIM, bad
    assert _dec(flags=0x40) == pk.PDSSM_ERR_FLAGS
    for name in ("sel", "dict_idx", "diag", "b", "c", "y", "x"):
        assert _dec(**{name: FAKE + 4}) == pk.PDSSM_ERR_ALIGN, name


def test_router_argument_errors(lib):
    r = pk.pdssm_router_select
    assert r(None, FAKE, FAKE, 2, 100, 3, 64, 256, 0, 0) == pk.PDSSM_ERR_NULL
    assert r(FAKE, FAKE, None, 2, 100, 3, 64, 256, 0, 0) == pk.PDSSM_ERR_NULL
    for B, L, H, K, D in ((-1, 100, 3, 64, 256), (2, -1, 3, 64, 256), (2, 100, -1, 64, 256),
                          (2, 100, 3, 0, 256), (2, 100, 3, 129, 256), (2, 100, 3, 64, 0),
                          (2, 100, 3, 64, 48), (2, 100, 3, 64, 16)):
        assert r(FAKE, FAKE, FAKE, B, L, H, K, D, 0, 0) == pk.PDSSM_ERR_DIM, (B, L, H, K, D)
    for flags in (2, 4, 0x80000000, pk.PDSSM_ROUTER_W_PACKED | 2):
        assert r(FAKE, FAKE, FAKE, 2, 100, 3, 64, 256, flags, 0) == pk.PDSSM_ERR_FLAGS, flags
    packed = pk.PDSSM_ROUTER_W_PACKED
    assert r(None, FAKE, FAKE, 2, 100, 3, 64, 256, packed, 0) == pk.PDSSM_ERR_NULL
    assert r(FAKE, FAKE + 2, FAKE, 2, 100, 3, 64, 256, packed, 0) == pk.PDSSM_ERR_ALIGN
    # packed weights are addressed by 32-bit offsets: H*P*D*2 bytes below 4 GB
    assert r(FAKE, FAKE, FAKE, 2, 100, 1024, 128, 16384, packed, 0) == pk.PDSSM_ERR_DIM
    assert r(FAKE + 2, FAKE, FAKE, 2, 100, 3, 64, 256, 0, 0) == pk.PDSSM_ERR_ALIGN
    assert r(FAKE, FAKE, FAKE + 2, 2, 100, 3, 64, 256, 0, 0) == pk.PDSSM_ERR_ALIGN


def test_router_pack_argument_errors(lib):
    p = pk.pdssm_router_pack_weights
    assert p(None, None, 0, 64, 256, 0) == pk.PDSSM_OK   # no heads: nothing read or written
    assert p(None, FAKE, 3, 64, 256, 0) == pk.PDSSM_ERR_NULL
    assert p(FAKE, None, 3, 64, 256, 0) == pk.PDSSM_ERR_NULL
    for H, K, D in ((-1, 64, 256), (3, 0, 256), (3, 129, 256), (3, 64, 0), (3, 64, 48),
                    (1024, 128, 16384)):
        assert p(FAKE, FAKE, H, K, D, 0) == pk.PDSSM_ERR_DIM, (H, K, D)
    assert p(FAKE + 2, FAKE, 3, 64, 256, 0) == pk.PDSSM_ERR_ALIGN
    assert p(FAKE, FAKE + 2, 3, 64, 256, 0) == pk.PDSSM_ERR_ALIGN


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """The allocation-free forward checks its fixed scratch on the host, before
    any HIP call: the very-long workload needs more than it holds."""
    flags = pk.PDSSM_LOGITS_BF16 | pk.PDSSM_COMPLEX | pk.PDSSM_BC_BF16 | pk.PDSSM_Y_BF16
    need = pk.pdssm_scan_workspace_bytes(2, 64, 131072, 64, 128, flags)
    assert need > 64 << 20
    rc = pk.pdssm_scan_fwd_noalloc(16, 16, 16, 16, 16, 16, 16, 2, 64, 131072, 64, 128, flags, None, 0)
    assert rc == pk.PDSSM_ERR_SCRATCH
    assert "scratch" in pk.pdssm_strerror(rc)
    assert pk.pdssm_scan_fwd_noalloc(16, 16, 16, 16, 16, 16, 16, 1, 1, 8, 65, 4, 0, None, 0) == pk.PDSSM_ERR_DIM
    assert pk.pdssm_scan_fwd_noalloc(16, 16, 16, 16, 16, 16, 16, 1, 1, 8, 8, 4, 0x100, None, 0) == pk.PDSSM_ERR_FLAGS
