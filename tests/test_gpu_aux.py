"""GPU parity of the dictionary pre-compute and of the single-step decode.

pdssm_dict_hardmax must equal the oracle's column-wise hardmax bit for bit
(ties, -0/+0 and NaN included).  pdssm_decode_step, chained over T calls
through its in-place state, must give the fp64 oracle's scan over the same T
steps (y at every step and the final state) within the per-sequence
tolerance, and exact integers on automata.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_state_amd as pk
from structured_sparse_state_amd import inputs as gen
from tests import oracle_pins
from tests.gpu_common import seq_rel_err, tol_of, x_to_np, y_to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


HARDMAX_CASES = [
    # H, K, N, bf16, ties, specials
    (1, 1, 1, False, True, True),
    (2, 3, 8, False, True, True),
    (1, 5, 16, True, True, True),
    (3, 5, 33, True, True, False),
    (2, 7, 63, False, False, True),
    (32, 64, 64, False, False, False),   # LM-layer dictionary
    (32, 64, 64, True, True, True),
    (64, 128, 64, True, False, False),   # very-long-workload dictionary
]


@pytest.mark.parametrize("H,K,N,bf16,ties,specials", HARDMAX_CASES)
def test_dict_hardmax(orc, H, K, N, bf16, ties, specials):
    say(f"[case] hardmax H={H} K={K} N={N} bf16={bf16} ties={ties} specials={specials}")
    m = oracle_pins.hardmax_matrices(H, K, N, bf16=bf16, seed=1000 + H + K + N, ties=ties,
                                     specials=specials)
    ref = orc.dict_hardmax(m)
    got = pk.dict_hardmax(m.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


def test_dict_hardmax_many_matrices(orc):
    """More matrices than the kernel's 2^20 workgroups: each workgroup takes
    several (2M matrices of 8 x 8, ties and -0/+0/NaN entries)."""
    H, K, N = 2048, 1024, 8
    say(f"[case] hardmax many matrices H={H} K={K} N={N}")
    m = oracle_pins.hardmax_matrices(H, K, N, bf16=False, seed=4242, ties=True, specials=True)
    ref = orc.dict_hardmax(m)
    got = pk.dict_hardmax(m.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


def test_dict_hardmax_drives_scan(orc):
    """Maps from the GPU hardmax run the scan like the oracle's maps."""
    inp = gen.make_inputs("tiny", B=2, H=3, L=200, N=16, K=6, seed=77)
    m = gen.make_dense_dict(3, 6, 16, seed=78)
    inp.dict_idx = torch.from_numpy(orc.dict_hardmax(m))
    g = inp.to(DEV)
    g.dict_idx = pk.dict_hardmax(m.to(DEV))
    y, _ = pk.scan(g)
    torch.cuda.synchronize()
    y_ref, _ = orc.scan_inputs(inp)
    assert seq_rel_err(y_to_np(y), y_ref) <= tol_of(inp)


def step_slice(inp, t):
    """Step t of a batch as decode inputs (contiguous)."""
    if inp.sel_mode.startswith("sel"):
        sel = inp.sel_or_logits[:, :, t].contiguous()
    else:
        sel = inp.sel_or_logits[:, :, t, :].contiguous()
    return sel, inp.diag[:, :, t].contiguous(), inp.b[:, :, t].contiguous(), inp.c[:, :, t].contiguous()


def run_decode(inp):
    """T decode calls on the GPU; returns (y [B,H,T], final state)."""
    g = inp.to(DEV)
    shape = (g.B, g.H, g.N, 2) if g.complex else (g.B, g.H, g.N)
    x = g.x0.clone() if g.x0 is not None else torch.zeros(shape, device=DEV, dtype=torch.float32)
    ys = []
    for t in range(g.L):
        sel, d, b, c = step_slice(g, t)
        ys.append(pk.decode_step(sel, g.dict_idx, d, b, c, x, sel_mode=g.sel_mode, complex=g.complex,
                                 bc_bf16=g.bc_bf16, y_bf16=g.y_bf16))
    torch.cuda.synchronize()
    return torch.stack(ys, dim=-1), x


DECODE_CASES = [
    ("tiny", dict(B=2, H=2, L=40)),
    ("small", dict(B=2, H=3, L=40)),
    ("long", dict(B=1, H=3, L=40, with_x0=True)),
    ("lm", dict(B=2, H=4, L=40, with_x0=True)),
    ("verylong", dict(B=1, H=3, L=30)),
]


@pytest.mark.parametrize("name,kw", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_chain_matches_oracle(orc, name, kw):
    inp = gen.make_inputs(name, **kw)
    say(f"[case] decode {name}: B={inp.B} H={inp.H} T={inp.L} N={inp.N} K={inp.K} mode={inp.sel_mode}")
    y, x = run_decode(inp)
    y_ref, x_ref = orc.scan_inputs(inp)
    tol = tol_of(inp)
    ey = seq_rel_err(y_to_np(y), y_ref)
    xr = x_ref if inp.complex else np.real(x_ref)
    ex = seq_rel_err(x_to_np(x, inp.complex), xr)
    say(f"  y error {ey:.2e}, state error {ex:.2e}")
    assert ey <= tol and ex <= tol


@pytest.mark.parametrize("kind,count", [("parity", False), ("cycle", False), ("reset", True)])
def test_decode_automata_exact(orc, kind, count):
    inp = gen.make_fsa_inputs(kind, B=2, H=2, L=60, N=8, m=5, count_state=count,
                              sel_mode=gen.LOGITS_F32 if kind == "cycle" else gen.SEL_I32)
    say(f"[case] decode automaton {kind}")
    y, x = run_decode(inp)
    y_ref, x_ref = orc.scan_inputs(inp)
    assert np.array_equal(y_to_np(y), y_ref)
    assert np.array_equal(x_to_np(x, False), np.real(x_ref))


def test_decode_matches_gpu_scan():
    """The decode chain and one scan call over the same steps agree."""
    inp = gen.make_inputs("lm", B=2, H=3, L=48, with_x0=True).to(DEV)
    y_dec, x_dec = run_decode(inp)
    y_scan, x_scan = pk.scan(inp)
    torch.cuda.synchronize()
    assert seq_rel_err(y_to_np(y_dec), y_to_np(y_scan)) <= tol_of(inp)
    assert seq_rel_err(x_to_np(x_dec, True), x_to_np(x_scan, True)) <= 1e-4
