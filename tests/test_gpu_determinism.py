"""Bitwise reproducibility under PDSSM_DETERMINISTIC.

Without the flag a tile's carry may be composed from several earlier tiles'
records, whichever are ready first, so repeated calls agree only to fp32
rounding (the header allows any summation order).  With the flag every tile
takes its carry from the tile just before it, so the same operations run in
the same order: repeated calls, the allocation-free entry point and the
backward give identical bits.  The results still match the fp64 oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_state_amd as pk
from structured_sparse_state_amd import inputs as gen
from tests.gpu_common import seq_rel_err, tol_of, x_to_np, y_to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("name,B,H,L", [("lm", None, None, None), ("verylong", None, None, None),
                                        ("long", None, None, None), ("lm", 1, 4, 262144),
                                        ("long", 2, 1, 600000)])
def test_forward_bitwise_repeatable(name, B, H, L):
    """Full-size workloads (where the plain chain is also the default) and
    few long sequences (where the default composes from aggregate records)."""
    g = gen.make_inputs(name, B=B, H=H, L=L, device=DEV)
    say(f"[case] deterministic forward, {name} B={g.B} H={g.H} L={g.L}")
    ws = pk.workspace_for(g)
    runs = []
    for _ in range(3):
        y, xf = pk.scan(g, workspace=ws, deterministic=True)
        runs.append((y, xf))
    torch.cuda.synchronize()
    for y, xf in runs[1:]:
        assert same(y, runs[0][0]) and same(xf, runs[0][1])
    # the default mode agrees to rounding
    y0, xf0 = pk.scan(g, workspace=ws)
    torch.cuda.synchronize()
    lim = 2.0 ** -7 if y0.dtype == torch.bfloat16 else 1e-5
    assert seq_rel_err(y_to_np(y0), y_to_np(runs[0][0])) <= lim
    if name == "lm" and B is None:
        # the allocation-free entry point runs the same arithmetic
        y2, xf2 = pk.scan_noalloc(g, deterministic=True)
        torch.cuda.synchronize()
        assert same(y2, runs[0][0]) and same(xf2, runs[0][1])
    del g, runs
    torch.cuda.empty_cache()


def test_forward_deterministic_matches_oracle():
    orc = oracle.get()
    for name, kw in (("lm", dict(B=2, H=3, L=4096, with_x0=True)), ("long", dict(B=1, H=2, L=18000)),
                     ("small", dict(B=2, H=3, L=2048))):
        inp = gen.make_inputs(name, **kw)
        say(f"[case] deterministic vs oracle: {name} {kw}")
        y, xf = pk.scan(inp.to(DEV), deterministic=True)
        torch.cuda.synchronize()
        y_ref, xf_ref = orc.scan_inputs(inp, nthreads=8)
        tol = tol_of(inp)
        assert seq_rel_err(y_to_np(y), y_ref) <= tol
        assert seq_rel_err(x_to_np(xf, inp.complex), xf_ref) <= tol


@pytest.mark.parametrize("B,H,L", [(None, None, None), (1, 2, 100000)])
def test_backward_bitwise_repeatable(B, H, L):
    g = gen.make_inputs("lm", B=B, H=H, L=L, device=DEV)
    say(f"[case] deterministic forward-save and backward, lm B={g.B} H={g.H} L={g.L}")
    gy, gxf = gen.make_grads(g, seed=9)
    outs = []
    for _ in range(2):
        y, xf, xch, sel = pk.scan_save(g, want_sel=True, deterministic=True)
        grads = pk.scan_bwd(g, xch, gy, gxf, sel=sel, deterministic=True)
        outs.append((y, xf, xch, sel) + tuple(grads))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert same(a, b)
    # gradients fed with the scores (the backward's own selection) are the same bits
    grads2 = pk.scan_bwd(g, outs[0][2], gy, gxf, deterministic=True)
    torch.cuda.synchronize()
    for a, b in zip(outs[0][4:], grads2):
        assert same(a, b)
    del g, outs, grads2
    torch.cuda.empty_cache()


def test_backward_deterministic_matches_oracle():
    orc = oracle.get()
    inp = gen.make_inputs("lm", B=1, H=2, L=1500, with_x0=True, seed=31)
    g = inp.to(DEV)
    gy, gxf = gen.make_grads(g, seed=4)
    _, _, xch, sel = pk.scan_save(g, want_sel=True, deterministic=True)
    grads = pk.scan_bwd(g, xch, gy, gxf, sel=sel, deterministic=True)
    torch.cuda.synchronize()
    ref = orc.scan_bwd(inp.sel_or_logits, inp.sel_mode, inp.dict_idx, inp.diag, inp.b, inp.c, gy.cpu(),
                       complex=True, bc_bf16=True, x0=inp.x0, gxf=x_to_np(gxf, True), nthreads=8)
    for name, got, r in zip(("gb", "gc", "gd", "gx0"), grads, ref):
        a = got.float().cpu().numpy().astype(np.float64)
        a = a[..., 0] + 1j * a[..., 1]
        e = max(seq_rel_err(a[0, h].reshape(1, -1), r[0, h].reshape(1, -1)) for h in range(2))
        say(f"  {name} error {e:.2e}")
        assert e <= tol_of(inp), (name, e)
