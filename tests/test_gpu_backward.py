"""GPU parity of the backward scan and of the forward's saved chunk carries.

pdssm_scan_fwd_save must give the same y as pdssm_scan_fwd, the states
x_{16c-1} of the fp64 oracle and (bit-exact) the oracle's selections;
pdssm_scan_bwd must give the oracle's gradients, fed with either the scores or
the saved selections,
(gb, gc, gd, gx0) within the per-sequence relative tolerance (1e-4 with fp32
I/O, 2e-2 with bf16 b/c/y).  The oracle's gradients are themselves pinned to
torch autograd and finite differences (tests/oracle_pins.py).
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
    """seq_rel_err with the rms taken over each whole (b,h) sequence."""
    B, H = ref.shape[:2]
    return max(seq_rel_err(got[bi, hi].reshape(1, -1), ref[bi, hi].reshape(1, -1))
               for bi in range(B) for hi in range(H))


def check_save(orc, inp, label):
    say(f"[case] save {label}: B={inp.B} H={inp.H} L={inp.L} N={inp.N} cplx={inp.complex}")
    g = inp.to(DEV)
    y1, _ = pk.scan(g)
    y2, xf2, xch, sel = pk.scan_save(g, want_sel=True)
    torch.cuda.synchronize()
    # the same scan; the tiles' carries may compose in another order (the
    # look-back depends on timing), so y agrees to rounding
    lim = 2.0 ** -7 if y1.dtype == torch.bfloat16 else 1e-5
    assert seq_rel_err(y_to_np(y1), y_to_np(y2)) <= lim, f"{label}: y differs with the carries kept"
    ref_sel = orc.select(inp.sel_or_logits, inp.sel_mode, inp.K)
    assert np.array_equal(sel.cpu().numpy().astype(np.int64), ref_sel.astype(np.int64)), \
        f"{label}: saved selections differ from the oracle's"
    nch = xch.shape[2]
    tol = tol_of(inp)
    for c in range(nch):
        if c == 0:
            ref = np.zeros((inp.B, inp.H, inp.N), np.complex128) if inp.x0 is None else \
                x_to_np(inp.x0, inp.complex)
        else:
            L1 = 16 * c
            part = gen.ScanInputs(**{**inp.__dict__})
            part.L = L1
            part.sel_or_logits = inp.sel_or_logits[:, :, :L1].contiguous()
            part.diag = inp.diag[:, :, :L1].contiguous()
            part.b = inp.b[:, :, :L1].contiguous()
            part.c = inp.c[:, :, :L1].contiguous()
            _, ref = orc.scan_inputs(part)
        got = x_to_np(xch[:, :, c], inp.complex)
        if not inp.complex:
            ref = np.real(ref)
        e = seq_rel_err(got, ref)
        assert e <= tol, f"{label}: chunk {c} carry error {e:.3e}"


def check_bwd(orc, inp, label, with_gxf=True, seed=0, saved_sel=False):
    say(f"[case] bwd {label}: B={inp.B} H={inp.H} L={inp.L} N={inp.N} K={inp.K} mode={inp.sel_mode} "
        f"cplx={inp.complex} bf16={inp.bc_bf16}/{inp.y_bf16} x0={inp.x0 is not None} gxf={with_gxf} "
        f"saved_sel={saved_sel}")
    g = inp.to(DEV)
    gy, gxf = gen.make_grads(g, seed=seed, with_gx_final=with_gxf)
    _, _, xch, sel = pk.scan_save(g, want_sel=True)
    gb, gc, gd, gx0 = pk.scan_bwd(g, xch, gy, gxf, sel=sel if saved_sel else None)
    torch.cuda.synchronize()
    gxf_ref = None if gxf is None else x_to_np(gxf, inp.complex)
    ref = orc.scan_bwd(inp.sel_or_logits, inp.sel_mode, inp.dict_idx, inp.diag, inp.b, inp.c,
                       gy.cpu(), complex=inp.complex, bc_bf16=inp.bc_bf16, x0=inp.x0, gxf=gxf_ref,
                       nthreads=8)
    tol = tol_of(inp)
    for name, got, r in zip(("gb", "gc", "gd", "gx0"), (gb, gc, gd, gx0), ref):
        gn = grad_to_np(got, inp.complex)
        assert np.all(np.isfinite(gn)), f"{label}: {name} not finite"
        e = per_seq_err(gn, r)
        say(f"  {name} error {e:.2e}")
        assert e <= tol, f"{label}: {name} error {e:.3e} > {tol}"


SAVE_CASES = [
    ("tiny", dict(B=1, H=2, L=100)),
    ("lm", dict(B=1, H=2, L=300, with_x0=True)),
    ("long", dict(B=1, H=1, L=250)),
]


@pytest.mark.parametrize("name,kw", SAVE_CASES, ids=[c[0] for c in SAVE_CASES])
def test_fwd_save(orc, name, kw):
    check_save(orc, gen.make_inputs(name, **kw), name)


BWD_SHAPES = [
    # N, L, K, sel_mode, complex, bc_bf16, y_bf16
    (1, 1, 1, gen.SEL_I32, False, False, False),
    (3, 31, 5, gen.LOGITS_BF16, False, True, True),
    (5, 33, 7, gen.SEL_I16, True, True, False),
    (8, 129, 4, gen.LOGITS_F32, False, False, False),
    (16, 513, 16, gen.SEL_I32, True, False, False),
    # N in 17..32: two chunks per wave; L not a multiple of 16 leaves a
    # partial last chunk, and waves with one idle and one active lane group.
    (20, 129, 12, gen.LOGITS_BF16, True, True, True),
    (32, 149, 9, gen.SEL_I32, False, False, False),
    (24, 405, 40, gen.LOGITS_F32, True, False, False),
    (33, 129, 12, gen.LOGITS_BF16, True, True, True),
    (47, 2000, 33, gen.SEL_I32, True, False, False),
    (64, 17, 64, gen.LOGITS_BF16, True, True, True),
    (64, 1000, 128, gen.LOGITS_BF16, True, True, True),
    (64, 300, 3000, gen.SEL_I32, True, False, False),
]


@pytest.mark.parametrize("N,L,K,mode,cplx,bcbf,ybf", BWD_SHAPES)
def test_bwd_shapes(orc, N, L, K, mode, cplx, bcbf, ybf):
    for with_x0, with_gxf, saved in ((False, False, False), (True, True, False), (True, False, True)):
        inp = gen.make_inputs("tiny", B=2, H=2, L=L, N=N, K=K, sel_mode=mode, complex=cplx,
                              bc_bf16=bcbf, y_bf16=ybf, dmin=0.8, dmax=1.0, with_x0=with_x0,
                              seed=3000 + N * 7 + L)
        check_bwd(orc, inp, f"shape N={N} L={L} K={K}", with_gxf=with_gxf, seed=N + L,
                  saved_sel=saved)


@pytest.mark.parametrize("name,B,H,L", [("lm", 1, 3, 4096), ("long", 1, 2, 4000), ("small", 2, 2, 2048)])
def test_bwd_workloads_scaled(orc, name, B, H, L):
    check_bwd(orc, gen.make_inputs(name, B=B, H=H, L=L, with_x0=True), f"{name} scaled",
              saved_sel=(name == "lm"))


def test_bwd_lm_full_size_sampled(orc):
    """The LM workload at full size; sampled sequences against the oracle."""
    say("[case] bwd lm full size")
    g = gen.make_inputs("lm", device=DEV)
    gy, gxf = gen.make_grads(g, seed=5)
    _, _, xch, sel = pk.scan_save(g, want_sel=True)
    gb, gc, gd, gx0 = pk.scan_bwd(g, xch, gy, gxf, sel=sel)
    torch.cuda.synchronize()
    # the same call fed with the scores agrees to rounding: the chunk carries
    # compose in an order that depends on timing, so fp32 values may differ in
    # their last bits from call to call, and a bf16 output (gb, gc) by one
    # bf16 rounding step
    for name, a, b in zip(("gb", "gc", "gd", "gx0"), (gb, gc, gd, gx0), pk.scan_bwd(g, xch, gy, gxf)):
        lim = 2.0 ** -7 if a.dtype == torch.bfloat16 else 1e-4
        for (bi, hi) in ((0, 0), (5, 30)):
            e = per_seq_err(grad_to_np(a[bi:bi + 1, hi:hi + 1], True), grad_to_np(b[bi:bi + 1, hi:hi + 1], True))
            assert e <= lim, (name, bi, hi, e)
    tol = tol_of(g)
    for (bi, hi) in ((0, 0), (3, 17), (g.B - 1, g.H - 1)):
        one = g.sequence(bi, hi).to("cpu")
        gxf1 = x_to_np(gxf[bi:bi + 1, hi:hi + 1], g.complex)
        ref = orc.scan_bwd(one.sel_or_logits, one.sel_mode, one.dict_idx, one.diag, one.b, one.c,
                           gy[bi:bi + 1, hi:hi + 1].cpu(), complex=True, bc_bf16=one.bc_bf16,
                           x0=one.x0, gxf=gxf1)
        for name, got, r in zip(("gb", "gc", "gd", "gx0"), (gb, gc, gd, gx0), ref):
            e = per_seq_err(grad_to_np(got[bi:bi + 1, hi:hi + 1], True), r)
            say(f"  seq ({bi},{hi}) {name} error {e:.2e}")
            assert e <= tol, (bi, hi, name, e)
    del g, gb, gc, gd, gx0, xch
    torch.cuda.empty_cache()


def test_bwd_linear_in_upstream(orc):
    """Gradients are linear in (gy, gx_final): g(a + 2b) = g(a) + 2 g(b)."""
    inp = gen.make_inputs("tiny", B=1, H=2, L=200, N=16, K=8, complex=True, sel_mode=gen.SEL_I32,
                          with_x0=True, seed=42).to(DEV)
    _, _, xch = pk.scan_save(inp)
    gy1, gx1 = gen.make_grads(inp, seed=1)
    gy2, gx2 = gen.make_grads(inp, seed=2)
    r1 = pk.scan_bwd(inp, xch, gy1, gx1)
    r2 = pk.scan_bwd(inp, xch, gy2, gx2)
    r3 = pk.scan_bwd(inp, xch, gy1 + 2 * gy2, gx1 + 2 * gx2)
    torch.cuda.synchronize()
    for a, b, c in zip(r1, r2, r3):
        ref = (a + 2 * b).double()
        err = ((c.double() - ref).abs().max() / ref.abs().max()).item()
        assert err < 1e-5, err


def test_bwd_rows_beyond_2gib(orc):
    """One sequence whose rows span more than 2 GiB, with padding lanes
    (N = 33 in 64 lanes, complex fp32 rows, 8.3M steps): the padding lanes'
    accesses must stay dropped however long the sequence.  The last steps'
    gradients against the oracle: its forward over the prefix gives the state
    before them, its backward over them the gradients."""
    N, L, M = 33, 8_300_000, 1024
    say(f"[case] bwd rows beyond 2 GiB: N={N} L={L}")
    g = gen.make_inputs("long", B=1, H=1, L=L, N=N, seed=77, device=DEV)
    gy, gxf = gen.make_grads(g, seed=3)
    _, _, xch = pk.scan_save(g)
    gb, gc, gd, gx0 = pk.scan_bwd(g, xch, gy, gxf)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(gb).all()) and bool(torch.isfinite(gd).all())
    host = g.to("cpu")
    cut = L - M
    _, x_cut = orc.scan(host.sel_or_logits[:, :, :cut], host.sel_mode, host.dict_idx, host.diag[:, :, :cut],
                        host.b[:, :, :cut], host.c[:, :, :cut], complex=True, bc_bf16=False, nthreads=8)
    say("  oracle prefix forward done")
    x0 = np.stack([x_cut.real, x_cut.imag], axis=-1).astype(np.float32)
    ref = orc.scan_bwd(host.sel_or_logits[:, :, cut:], host.sel_mode, host.dict_idx, host.diag[:, :, cut:],
                       host.b[:, :, cut:], host.c[:, :, cut:], gy[:, :, cut:].cpu(), complex=True,
                       bc_bf16=False, x0=x0, gxf=x_to_np(gxf, True))
    tol = tol_of(g)
    for name, got, r in zip(("gb", "gc", "gd"), (gb, gc, gd), ref[:3]):
        e = per_seq_err(grad_to_np(got[:, :, cut:], True), r)
        say(f"  tail {name} error {e:.2e}")
        assert e <= tol, (name, e)
    del g, host, gb, gc, gd, gx0, xch
    torch.cuda.empty_cache()
