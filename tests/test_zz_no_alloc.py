"""The allocation-free forward scan (pdssm_scan_fwd_noalloc) against the
workspace entry point (pdssm_scan_fwd) and the fp64 oracle, on two calls in a
row through the C ABI, the second with a smaller input: its scratch keeps
the first call's records, which the second must not mistake for its own."""
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


def test_noalloc_matches_workspace_entry_point():
    orc = oracle.get()
    cases = [gen.make_inputs("lm", B=2, H=4, L=4096, with_x0=True, seed=811),
             gen.make_inputs("long", B=1, H=2, L=1500, seed=812)]
    for n, inp in enumerate(cases):
        say(f"[case] noalloc call {n}: B={inp.B} H={inp.H} L={inp.L} N={inp.N} K={inp.K}")
        g = inp.to(DEV)
        y_ws, xf_ws = pk.scan(g)
        y_na = torch.empty_like(y_ws)
        xf_na = torch.empty_like(xf_ws)
        torch.cuda.synchronize()
        rc = pk.pdssm_scan_fwd_noalloc(g.sel_or_logits, g.dict_idx, g.diag, g.b, g.c, y_na, xf_na,
                                       g.B, g.H, g.L, g.N, g.K, pk.flags_of(g), g.x0)
        assert rc == pk.PDSSM_OK, pk.pdssm_strerror(rc)
        torch.cuda.synchronize()
        tol = tol_of(inp)
        # the two entry points agree to rounding (tile carries compose in a
        # timing-dependent order) ...
        lim = 2.0 ** -7 if y_ws.dtype == torch.bfloat16 else 1e-5
        assert seq_rel_err(y_to_np(y_na), y_to_np(y_ws)) <= lim
        assert seq_rel_err(x_to_np(xf_na, inp.complex), x_to_np(xf_ws, inp.complex)) <= 1e-5
        # ... and both match the oracle
        y_ref, xf_ref = orc.scan_inputs(inp, nthreads=8)
        ey = seq_rel_err(y_to_np(y_na), y_ref)
        ex = seq_rel_err(x_to_np(xf_na, inp.complex), xf_ref)
        say(f"  y err {ey:.2e}, x_final err {ex:.2e}")
        assert ey <= tol and ex <= tol


def test_noalloc_automaton_exact():
    """An automaton run (D = I, one-hot states) is exact: bit-identical
    outputs from both entry points, twice in a row with a smaller second call."""
    orc = oracle.get()
    for n, L in enumerate((6000, 900)):
        inp = gen.make_fsa_inputs("cycle", B=2, H=3, L=L, N=32, m=11, sel_mode=gen.LOGITS_BF16,
                                  complex=True, seed=70 + n, start_state=3)
        say(f"[case] noalloc automaton call {n}: L={L}")
        g = inp.to(DEV)
        y_na, xf_na = pk.scan_noalloc(g)
        torch.cuda.synchronize()
        y_ref, xf_ref = orc.scan_inputs(inp)
        assert np.array_equal(y_to_np(y_na), y_ref)
        assert np.array_equal(x_to_np(xf_na, True), xf_ref)
