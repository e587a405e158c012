"""The decode step captured in a HIP graph: a chain of T steps launched as
one graph, replayed several times with eager work in between, every replay
checked against the same chain run eagerly.

The decode kernel allocates nothing and records no memset, so a caller can
capture a whole decoding window (the state stays in the caller's buffer and
each step's inputs are fixed addresses).  Collisions in the step's scatter
are summed with LDS atomics in any order, so floating results are compared to
rounding; automaton states are exact integers and must match bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import structured_sparse_state_amd as pk
from structured_sparse_state_amd import inputs as gen
from tests.gpu_common import seq_rel_err, y_to_np, x_to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _steps(g, T):
    out = []
    for t in range(T):
        if g.sel_mode.startswith("sel"):
            sel = g.sel_or_logits[:, :, t].contiguous()
        else:
            sel = g.sel_or_logits[:, :, t, :].contiguous()
        out.append((sel, g.diag[:, :, t].contiguous(), g.b[:, :, t].contiguous(), g.c[:, :, t].contiguous()))
    return out


def _run(g, steps, x, ys):
    for t, (sel, d, b, c) in enumerate(steps):
        pk.decode_step(sel, g.dict_idx, d, b, c, x, sel_mode=g.sel_mode, complex=g.complex,
                       bc_bf16=g.bc_bf16, y_bf16=g.y_bf16, y=ys[t])


@pytest.mark.parametrize("case", ["lm", "parity"])
def test_decode_graph_replays_match_eager(case):
    T = 32
    if case == "lm":
        inp = gen.make_inputs("lm", B=2, H=4, L=T, with_x0=True)
    else:
        inp = gen.make_fsa_inputs("parity", B=2, H=3, L=T, N=8, m=2, sel_mode=gen.SEL_I32)
    say(f"[case] decode graph {case}: B={inp.B} H={inp.H} T={T} N={inp.N} K={inp.K}")
    g = inp.to(DEV)
    steps = _steps(g, T)
    shape = (g.B, g.H, g.N, 2) if g.complex else (g.B, g.H, g.N)
    x0 = g.x0 if g.x0 is not None else torch.zeros(shape, device=DEV, dtype=torch.float32)
    ydt = torch.bfloat16 if g.y_bf16 else torch.float32

    # the chain run eagerly
    x_ref = x0.clone()
    ys_ref = [torch.empty((g.B, g.H), device=DEV, dtype=ydt) for _ in range(T)]
    _run(g, steps, x_ref, ys_ref)
    torch.cuda.synchronize()
    y_ref = torch.stack(ys_ref, dim=-1)

    # the same chain captured once
    x = x0.clone()
    ys = [torch.empty((g.B, g.H), device=DEV, dtype=ydt) for _ in range(T)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(g, steps, x, ys)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        _run(g, steps, x, ys)

    for rep in range(3):
        x.copy_(x0)                  # eager: the window's initial state
        for yt in ys:
            yt.fill_(float("nan"))   # stale outputs must be rewritten
        graph.replay()
        torch.cuda.synchronize()
        y = torch.stack(ys, dim=-1)
        if case == "parity":
            assert torch.equal(y, y_ref) and torch.equal(x, x_ref), rep
        else:
            ey = seq_rel_err(y_to_np(y), y_to_np(y_ref))
            ex = seq_rel_err(x_to_np(x, True), x_to_np(x_ref, True))
            say(f"  replay {rep}: y difference {ey:.2e}, state difference {ex:.2e}")
            assert ey <= 2.0 ** -7 and ex <= 1e-5, (rep, ey, ex)
        # eager work on the same stream between replays
        _ = (x_ref * 2.0).sum().item()
