"""Empty shapes on the GPU, through the C ABI, against the fp64 oracle.

With no steps the state is the initial one and the product of no step
operators is the identity: x_final = x0 (zero without x0), compose gives
pi[j] = j with d[j] = 1, and the gradient of x_final passes to x0 unchanged.
All three are copies or constants, so they must match the oracle exactly.
With no sequences (or no tokens, heads or matrices) a call succeeds and
writes nothing.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_state_amd as pk
from structured_sparse_state_amd import inputs as gen
from tests.gpu_common import x_to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _tail(inp):
    return (inp.N, 2) if inp.complex else (inp.N,)


@pytest.mark.parametrize("name", ["small", "long", "lm"])
def test_scan_of_no_steps(orc, name):
    for with_x0 in (True, False):
        say(f"[case] {name} L=0 x0={with_x0}")
        inp = gen.make_inputs(name, B=2, H=3, L=0, with_x0=with_x0, seed=91)
        g = inp.to(DEV)
        xf = torch.full((2, 3) + _tail(inp), float("nan"), device=DEV)
        y, xf = pk.scan(g, x_final=xf)
        torch.cuda.synchronize()
        _, xf_ref = orc.scan_inputs(inp)
        assert y.numel() == 0
        assert np.array_equal(x_to_np(xf, inp.complex), xf_ref)

        y, xf, xch, sel = pk.scan_save(g, want_sel=True)
        torch.cuda.synchronize()
        assert y.numel() == 0 and xch.numel() == 0 and sel.numel() == 0
        assert np.array_equal(x_to_np(xf, inp.complex), xf_ref)


@pytest.mark.parametrize("name", ["small", "lm"])
def test_compose_of_no_steps(orc, name):
    say(f"[case] compose {name} L=0")
    inp = gen.make_inputs(name, B=2, H=3, L=0, seed=92)
    pi, d = pk.compose(inp.to(DEV))
    torch.cuda.synchronize()
    pi_ref, d_ref = orc.compose_inputs(inp)
    assert np.array_equal(pi.cpu().numpy(), pi_ref)
    assert np.array_equal(x_to_np(d, inp.complex), d_ref)


@pytest.mark.parametrize("name", ["small", "lm"])
def test_backward_of_no_steps(orc, name):
    for with_gxf in (True, False):
        say(f"[case] backward {name} L=0 gx_final={with_gxf}")
        inp = gen.make_inputs(name, B=2, H=3, L=0, with_x0=True, seed=93)
        g = inp.to(DEV)
        gxf = torch.randn((2, 3) + _tail(inp), generator=torch.Generator().manual_seed(5)) \
            if with_gxf else None
        xch = torch.empty((2, 3, 0) + _tail(inp), device=DEV)
        gy = torch.empty((2, 3, 0), device=DEV, dtype=torch.bfloat16 if inp.y_bf16 else torch.float32)
        gb, gc, gd, gx0 = pk.scan_bwd(g, xch, gy, None if gxf is None else gxf.to(DEV))
        torch.cuda.synchronize()
        gxf_np = None if gxf is None else x_to_np(gxf, inp.complex)
        *_, gx0_ref = orc.scan_bwd(inp.sel_or_logits, inp.sel_mode, inp.dict_idx, inp.diag, inp.b,
                                   inp.c, np.zeros((2, 3, 0)), complex=inp.complex,
                                   bc_bf16=inp.bc_bf16, x0=inp.x0, gxf=gxf_np)
        assert gb.numel() == gc.numel() == gd.numel() == 0
        assert np.array_equal(x_to_np(gx0, inp.complex), gx0_ref)


def test_no_sequences_write_nothing():
    say("[case] B=0 / H=0 scans, selection, compose, backward")
    for B, H in ((0, 3), (2, 0)):
        inp = gen.make_inputs("lm", B=B, H=H, L=100, with_x0=True, seed=94).to(DEV)
        y, xf = pk.scan(inp)
        assert y.numel() == 0 and xf.numel() == 0
        y, xf, xch = pk.scan_save(inp)
        assert xch.numel() == 0
        pi, d = pk.compose(inp)
        assert pi.numel() == 0
        gb, gc, gd, gx0 = pk.scan_bwd(inp, xch, torch.empty((B, H, 100), device=DEV,
                                                            dtype=torch.bfloat16))
        assert gb.numel() == 0 and gx0.numel() == 0
        assert pk.select(inp.sel_or_logits, inp.sel_mode, inp.K).numel() == 0
    torch.cuda.synchronize()


def test_empty_router_hardmax_decode():
    say("[case] router / hardmax / decode with nothing to do")
    u = torch.zeros((2, 0, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((3, 8, 64), dtype=torch.bfloat16, device=DEV)
    assert pk.router_select(u, w).numel() == 0
    u = torch.zeros((2, 5, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((0, 8, 64), dtype=torch.bfloat16, device=DEV)
    assert pk.router_select(u, w).numel() == 0
    m = torch.zeros((0, 4, 8, 8), device=DEV)
    assert pk.dict_hardmax(m).numel() == 0
    x = torch.zeros((0, 3, 8), device=DEV)
    z = torch.zeros((0, 3, 8), device=DEV)
    y = pk.decode_step(torch.zeros((0, 3), dtype=torch.int32, device=DEV),
                       torch.zeros((3, 4, 8), dtype=torch.int32, device=DEV), z, z, z, x,
                       sel_mode="sel_i32", complex=False, bc_bf16=False, y_bf16=False)
    torch.cuda.synchronize()
    assert y.numel() == 0
