"""The library's test builds against the oracle and against the library.

* ``w5`` (PDSSM_SCAN_W=5): five chunk waves per scan workgroup, so other
  tile boundaries (80 steps at N = 64 instead of 112) and the general
  wave/chunk order.  The results must not depend on the chunking: the same
  parity cases pass with the same tolerances (LM scaled, long and very long
  at full length, automata bit-exact, ragged shapes), and the forward's
  saved selections are bit-identical to the library's.
* ``remap`` (PDSSM_TEST_TICKET_REMAP): the sequences of every tile row are
  handed out in reverse order, and per-head ticket streams are served by the
  workgroups in reverse, in the forward and the backward.  Parity cases pass
  as before, and under PDSSM_DETERMINISTIC the results are bit-identical to
  the library's, at the LM and very-long workloads' full sizes: the order in
  which tiles are dispatched changes no result.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_state_amd as pk
from structured_sparse_state_amd import inputs as gen
from tests import test_gpu_backward as bwd
from tests import test_gpu_parity as par
from tests.gpu_common import seq_rel_err, y_to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


# ---------------------------------------------------------------------------
# Chunk-size invariance: the parity cases under five chunk waves per tile.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,B,H,L", [("lm", 1, 3, 4096), ("long", 1, 2, 18000),
                                        ("verylong", 1, 1, 131072), ("small", 2, 3, 2048)])
def test_w5_workload_scaled(orc, name, B, H, L):
    with pk.variant("w5"):
        par.test_workload_scaled(orc, name, B, H, L)


@pytest.mark.parametrize("name,samples", [("long", 3), ("verylong", 2), ("lm", 3)])
def test_w5_workload_full_size_sampled(orc, name, samples):
    with pk.variant("w5"):
        par.test_workload_full_size_sampled(orc, name, samples)


@pytest.mark.parametrize("kind,m,count,mode,cplx,N,L", par.FSA)
def test_w5_automata_bit_exact(orc, kind, m, count, mode, cplx, N, L):
    with pk.variant("w5"):
        par.test_automata_bit_exact(orc, kind, m, count, mode, cplx, N, L)


@pytest.mark.parametrize("N,L,K,mode,cplx,bcbf,ybf", [
    (1, 1, 1, gen.SEL_I32, False, False, False),
    (5, 33, 7, gen.SEL_I16, True, True, False),
    (17, 300, 9, gen.LOGITS_BF16, False, False, True),
    (47, 2000, 33, gen.SEL_I32, True, False, False),
    (64, 5000, 128, gen.LOGITS_BF16, True, True, True),
    (64, 300, 32767, gen.SEL_I16, True, True, True),
])
def test_w5_shapes(orc, N, L, K, mode, cplx, bcbf, ybf):
    with pk.variant("w5"):
        par.test_shapes(orc, N, L, K, mode, cplx, bcbf, ybf)


@pytest.mark.parametrize("N,mode", [(8, gen.SEL_I32), (16, gen.LOGITS_BF16)])
def test_w5_many_tiles_per_workgroup(orc, N, mode):
    with pk.variant("w5"):
        par.test_many_tiles_per_workgroup(orc, N, mode)


def test_w5_saved_carries_and_backward(orc):
    """The forward's saved carries under five chunk waves feed the backward
    to the oracle's gradients; its saved selections equal the library's."""
    inp = gen.make_inputs("lm", B=1, H=2, L=1000, with_x0=True, seed=13)
    with pk.variant("w5"):
        bwd.check_save(orc, inp, "w5 lm")
        bwd.check_bwd(orc, inp, "w5 lm", saved_sel=True)
        g = inp.to(DEV)
        _, _, xch5, sel5 = pk.scan_save(g, want_sel=True)
    _, _, xch7, sel7 = pk.scan_save(g, want_sel=True)
    torch.cuda.synchronize()
    assert same(sel5, sel7)
    a, b = xch5.double().cpu().numpy(), xch7.double().cpu().numpy()
    assert seq_rel_err(a.reshape(2, -1), b.reshape(2, -1)) <= 1e-5


# ---------------------------------------------------------------------------
# Dispatch-order invariance: tickets handed out in reverse sequence order.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,B,H,L", [("lm", 2, 3, 4096), ("long", 2, 2, 18000), ("small", 4, 3, 2048)])
def test_remap_workload_scaled(orc, name, B, H, L):
    with pk.variant("remap"):
        par.test_workload_scaled(orc, name, B, H, L)


@pytest.mark.parametrize("name,samples", [("lm", 3), ("verylong", 2)])
def test_remap_workload_full_size_sampled(orc, name, samples):
    with pk.variant("remap"):
        par.test_workload_full_size_sampled(orc, name, samples)


@pytest.mark.parametrize("name,B,H,L", [("lm", 2, 3, 4096), ("long", 2, 2, 4000)])
def test_remap_bwd_scaled(orc, name, B, H, L):
    with pk.variant("remap"):
        bwd.check_bwd(orc, gen.make_inputs(name, B=B, H=H, L=L, with_x0=True), f"remap {name}",
                      saved_sel=True)


@pytest.mark.parametrize("kind,m,count,mode,cplx,N,L", par.FSA[:4])
def test_remap_automata_bit_exact(orc, kind, m, count, mode, cplx, N, L):
    with pk.variant("remap"):
        par.test_automata_bit_exact(orc, kind, m, count, mode, cplx, N, L)


@pytest.mark.parametrize("name", ["lm", "verylong"])
def test_remap_deterministic_bitwise(name):
    """Under PDSSM_DETERMINISTIC the reversed dispatch gives the library's
    bits: y and x_final of the forward, the saved carries and selections,
    and the backward's gradients."""
    cfg = gen.CONFIGS[name]
    say(f"[case] remap vs library, deterministic, {name} full size B={cfg['B']} H={cfg['H']} L={cfg['L']}")
    g = gen.make_inputs(name, device=DEV)
    y1, xf1 = pk.scan(g, deterministic=True)
    with pk.variant("remap"):
        y2, xf2 = pk.scan(g, deterministic=True)
    torch.cuda.synchronize()
    assert same(y1, y2) and same(xf1, xf2)
    del y1, xf1, y2, xf2
    if name == "lm":
        gy, gxf = gen.make_grads(g, seed=2)
        outs = []
        for v in (None, "remap"):
            if v is None:
                _, _, xch, sel = pk.scan_save(g, want_sel=True, deterministic=True)
                gr = pk.scan_bwd(g, xch, gy, gxf, sel=sel, deterministic=True)
            else:
                with pk.variant(v):
                    _, _, xch, sel = pk.scan_save(g, want_sel=True, deterministic=True)
                    gr = pk.scan_bwd(g, xch, gy, gxf, sel=sel, deterministic=True)
            outs.append((xch, sel) + tuple(gr))
        torch.cuda.synchronize()
        for a, b in zip(*outs):
            assert same(a, b)
    else:
        # default mode: within rounding of the library
        y1, _ = pk.scan(g)
        with pk.variant("remap"):
            y2, _ = pk.scan(g)
        torch.cuda.synchronize()
        assert seq_rel_err(y_to_np(y1[:, :4]), y_to_np(y2[:, :4])) <= 2.0 ** -7
    del g
    torch.cuda.empty_cache()
