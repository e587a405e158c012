"""The scan kernels' own hard selection on adversarial router scores.

The selection rule (include/pdssm.h; the Flash PD-SSM summary, Methodology
1, picks the entry with the largest score, and the tie rules are this
build's reading): the lowest index among equal maxima, -0 equal to +0, a NaN
above every number with the first NaN winning, scores compared exactly as
stored.  The scores here hold exact ties (small integers, in fp32 and bf16),
-0/+0 pairs at the maximum, one or several NaNs, +inf and -inf, and whole
rows of -inf (inputs.make_adversarial_scores).

Each case runs them through the paths the forward and backward scans use:
the cooperative selection of the forward scan kernel (one chunk per wave at
N = 64, four chunks per wave at N = 16), its general per-slice selection
(K = 200, and K = 3000 whose entry table does not fit in LDS), and the
backward's own selection from the scores.  The forward's saved int16
selections must equal the oracle's bit for bit; y, x_final and the
gradients must be within the parity tolerance of the fp64 oracle fed with
the same scores.
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


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def grad_to_np(t: torch.Tensor, cplx: bool) -> np.ndarray:
    a = t.float().cpu().numpy().astype(np.float64)
    return a[..., 0] + 1j * a[..., 1] if cplx else a


def per_seq_err(got: np.ndarray, ref: np.ndarray) -> float:
    B, H = ref.shape[:2]
    return max(seq_rel_err(got[bi, hi].reshape(1, -1), ref[bi, hi].reshape(1, -1))
               for bi in range(B) for hi in range(H))


CASES = [
    # N, K, mode, complex, bc_bf16, y_bf16, L
    (64, 64, gen.LOGITS_BF16, True, True, True, 700),      # cooperative, one chunk per wave
    (64, 40, gen.LOGITS_BF16, True, True, True, 300),      # one chunk per wave, short and empty slices
    (64, 8, gen.LOGITS_BF16, False, True, False, 300),     # one lane holds every score
    (64, 32, gen.LOGITS_F32, False, False, False, 300),    # one chunk per wave, fp32 slices
    (64, 20, gen.LOGITS_F32, True, False, False, 300),     # fp32, short and empty slices
    (16, 16, gen.LOGITS_F32, False, False, False, 900),    # cooperative, four chunks per wave
    (64, 200, gen.LOGITS_BF16, True, True, True, 500),     # per-slice selection
    (32, 3000, gen.LOGITS_F32, False, False, False, 300),  # per-slice, entry table beyond LDS
]


@pytest.mark.parametrize("N,K,mode,cplx,bcbf,ybf,L", CASES)
def test_adversarial_scores(orc, N, K, mode, cplx, bcbf, ybf, L):
    bf = mode == gen.LOGITS_BF16
    inp = gen.make_inputs("tiny", B=2, H=2, L=L, N=N, K=K, sel_mode=mode, complex=cplx,
                          bc_bf16=bcbf, y_bf16=ybf, dmin=0.8, dmax=1.0, with_x0=True,
                          seed=900 + N + K)
    inp.sel_or_logits = gen.make_adversarial_scores(2, 2, L, K, bf16=bf, seed=901 + K)
    say(f"[case] adversarial scores N={N} K={K} mode={mode} L={L}")
    g = inp.to(DEV)

    # Forward: the saved selections bit for bit, y and x_final to tolerance.
    y, xf, xch, sel = pk.scan_save(g, want_sel=True)
    y2, xf2 = pk.scan(g)
    torch.cuda.synchronize()
    ref_sel = orc.select(inp.sel_or_logits, mode, K)
    got_sel = sel.cpu().numpy().astype(np.int64)
    bad = np.argwhere(got_sel != ref_sel.astype(np.int64))
    assert bad.size == 0, f"{bad.shape[0]} selections differ, first at {tuple(bad[0])}"
    y_ref, xf_ref = orc.scan_inputs(inp, nthreads=8)
    tol = tol_of(inp)
    for yy, xx in ((y, xf), (y2, xf2)):
        ey = seq_rel_err(y_to_np(yy), y_ref)
        ex = seq_rel_err(x_to_np(xx, cplx), xf_ref)
        say(f"  y err {ey:.2e}, x_final err {ex:.2e}")
        assert ey <= tol and ex <= tol, (ey, ex)

    # Backward fed with the scores: its own selection picks the same entries.
    gy, gxf = gen.make_grads(g, seed=K)
    grads = pk.scan_bwd(g, xch, gy, gxf)
    torch.cuda.synchronize()
    ref = orc.scan_bwd(inp.sel_or_logits, mode, inp.dict_idx, inp.diag, inp.b, inp.c, gy.cpu(),
                       complex=cplx, bc_bf16=bcbf, x0=inp.x0, gxf=x_to_np(gxf, cplx), nthreads=8)
    for name, got, r in zip(("gb", "gc", "gd", "gx0"), grads, ref):
        e = per_seq_err(grad_to_np(got, cplx), r)
        say(f"  {name} error {e:.2e}")
        assert e <= tol, (name, e)
