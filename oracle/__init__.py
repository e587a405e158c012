"""fp64 CPU oracle for the Flash PD-SSM forward scan -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library under
``structured_sparse_state_amd`` never does; the two share no code.

The arithmetic lives in ``pdssm_oracle.c`` (plain C, double precision,
sequential in time; see its header for what each function computes and which
passage of the Flash PD-SSM pages it follows).  This module compiles it with
gcc, loads it with ctypes and marshals numpy arrays.

Every function here is pinned by ``tests/test_oracle.py`` to things other than
itself: dense N x N matrix products, brute-force automaton simulation, closed
forms, invariants and a hand-worked example (``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "pdssm_oracle.c")
LIBRARY = os.path.join(HERE, "_pdssm_oracle.so")

SEL_KIND = {"sel_i32": 0, "sel_i16": 1, "logits_f32": 2, "logits_bf16": 3}
ERRORS = {-1: "selection index out of range", -2: "map entry out of range", -3: "bad argument"}

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-std=c11"]


def build(source: str = SOURCE, out: str = LIBRARY, extra=()) -> str:
    """Compile the oracle (gcc) into a shared library; returns its path."""
    cmd = ["gcc", *GCC_FLAGS, *extra, "-o", out, source, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """ctypes handle on one compiled oracle library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(out=path)
        lib = ctypes.CDLL(path)
        P, I64, I32, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        lib.pdssm_oracle_select.argtypes = [P, I, I64, I64, I64, I32, P]
        lib.pdssm_oracle_select.restype = I
        lib.pdssm_oracle_scan.argtypes = [P, I, P, P, P, P, P, I, I, I64, I64, I64, I32, I32, P, P, I]
        lib.pdssm_oracle_scan.restype = I
        lib.pdssm_oracle_compose.argtypes = [P, I, P, P, I, I64, I64, I64, I32, I32, P, P]
        lib.pdssm_oracle_compose.restype = I
        lib.pdssm_oracle_scan_bwd.argtypes = [P, I, P, P, P, P, P, P, P, I, I, I64, I64, I64, I32, I32,
                                              P, P, P, P, I]
        lib.pdssm_oracle_scan_bwd.restype = I
        lib.pdssm_oracle_dict_hardmax.argtypes = [P, I, I64, I32, I32, P]
        lib.pdssm_oracle_dict_hardmax.restype = I
        lib.pdssm_oracle_router_select.argtypes = [P, P, I64, I64, I64, I32, I32, P, P, I]
        lib.pdssm_oracle_router_select.restype = I
        self.lib = lib
        self.path = path

    @staticmethod
    def _check(rc: int):
        if rc != 0:
            raise ValueError(f"oracle: {ERRORS.get(rc, rc)}")

    @staticmethod
    def _arr(a, dtype=None):
        """Contiguous numpy view; bf16 torch tensors arrive as raw uint16 bits."""
        if a is None:
            return None
        if hasattr(a, "detach"):  # a torch tensor
            import torch
            t = a.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                t = t.view(torch.int16)
                return np.ascontiguousarray(t.numpy().view(np.uint16))
            a = t.numpy()
        a = np.ascontiguousarray(a)
        if dtype is not None and a.dtype != dtype:
            raise TypeError(f"expected {dtype}, got {a.dtype}")
        return a

    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    def select(self, sel_or_logits, sel_mode: str, K: int) -> np.ndarray:
        src = self._arr(sel_or_logits)
        shape = src.shape if sel_mode.startswith("sel") else src.shape[:-1]
        B, H, L = shape
        out = np.empty((B, H, L), dtype=np.int32)
        self._check(self.lib.pdssm_oracle_select(self._ptr(src), SEL_KIND[sel_mode], B, H, L, K,
                                                 self._ptr(out)))
        return out

    def dict_hardmax(self, m) -> np.ndarray:
        """dict_idx int32 [H,K,N] from dense matrices m [H,K,N,N] (fp32, or a
        bf16 torch tensor): the column-wise hardmax of every matrix."""
        src = self._arr(m)
        H, K, N, N2 = src.shape
        assert N == N2
        is_bf16 = src.dtype == np.uint16
        if not is_bf16 and src.dtype != np.float32:
            raise TypeError(f"expected fp32 or bf16, got {src.dtype}")
        out = np.empty((H, K, N), dtype=np.int32)
        self._check(self.lib.pdssm_oracle_dict_hardmax(self._ptr(src), int(is_bf16), H, K, N,
                                                        self._ptr(out)))
        return out

    def router_select(self, u, w, *, want_logits: bool = False, nthreads: int = 1):
        """sel int32 [B,H,L] (and the float64 scores [B,H,L,K] when asked)
        from bf16 inputs u [B,L,D] and router weights w [H,K,D]."""
        uu = self._arr(u)
        ww = self._arr(w)
        if uu.dtype != np.uint16 or ww.dtype != np.uint16:
            raise TypeError("u and w must be bf16")
        B, L, D = uu.shape
        H, K, D2 = ww.shape
        assert D == D2
        sel = np.empty((B, H, L), dtype=np.int32)
        lg = np.empty((B, H, L, K), dtype=np.float64) if want_logits else None
        self._check(self.lib.pdssm_oracle_router_select(self._ptr(uu), self._ptr(ww), B, L, H, K, D,
                                                         self._ptr(sel), self._ptr(lg), int(nthreads)))
        return (sel, lg) if want_logits else sel

    def scan(self, sel_or_logits, sel_mode: str, dict_idx, diag, b, c, *, complex: bool,
             bc_bf16: bool, x0=None, nthreads: int = 1):
        """Returns (y [B,H,L] float64, x_final [B,H,N] float64 or complex128)."""
        src = self._arr(sel_or_logits)
        dct = self._arr(dict_idx, np.int32)
        dg = self._arr(diag, np.float32)
        bb = self._arr(b)
        cc = self._arr(c)
        xx = self._arr(x0, np.float32)
        H, K, N = dct.shape
        B, H2, L = dg.shape[:3]
        assert H2 == H
        y = np.empty((B, H, L), dtype=np.float64)
        xf = np.empty((B, H, N, 2) if complex else (B, H, N), dtype=np.float64)
        self._check(self.lib.pdssm_oracle_scan(
            self._ptr(src), SEL_KIND[sel_mode], self._ptr(dct), self._ptr(dg), self._ptr(bb),
            self._ptr(cc), self._ptr(xx), int(complex), int(bc_bf16), B, H, L, N, K,
            self._ptr(y), self._ptr(xf), int(nthreads)))
        if complex:
            xf = xf[..., 0] + 1j * xf[..., 1]
        return y, xf

    def scan_bwd(self, sel_or_logits, sel_mode: str, dict_idx, diag, b, c, gy, *, complex: bool,
                 bc_bf16: bool, x0=None, gxf=None, nthreads: int = 1):
        """Gradients of sum_t gy_t y_t (+ the x_final term with gradient gxf).

        gy is [B,H,L] (any float dtype, read as float64); gxf is [B,H,N]
        float64 or complex128, or None.  Returns (gb, gc, gd) [B,H,L,N] and
        gx0 [B,H,N], float64 or complex128 (grad = dL/dRe + i dL/dIm).
        """
        src = self._arr(sel_or_logits)
        dct = self._arr(dict_idx, np.int32)
        dg = self._arr(diag, np.float32)
        bb = self._arr(b)
        cc = self._arr(c)
        xx = self._arr(x0, np.float32)
        g = self._arr(gy).astype(np.float64) if not hasattr(gy, "detach") else \
            np.ascontiguousarray(gy.detach().cpu().double().numpy())
        H, K, N = dct.shape
        B, _, L = dg.shape[:3]
        gf = None
        if gxf is not None:
            gf = np.asarray(gxf)
            if complex:
                gf = np.stack([gf.real, gf.imag], axis=-1) if np.iscomplexobj(gf) else gf
            gf = np.ascontiguousarray(gf, dtype=np.float64)
        shp = (B, H, L, N, 2) if complex else (B, H, L, N)
        gb = np.empty(shp, np.float64)
        gc = np.empty(shp, np.float64)
        gd = np.empty(shp, np.float64)
        gx0 = np.empty((B, H, N, 2) if complex else (B, H, N), np.float64)
        self._check(self.lib.pdssm_oracle_scan_bwd(
            self._ptr(src), SEL_KIND[sel_mode], self._ptr(dct), self._ptr(dg), self._ptr(bb),
            self._ptr(cc), self._ptr(xx), self._ptr(g), self._ptr(gf), int(complex), int(bc_bf16),
            B, H, L, N, K, self._ptr(gb), self._ptr(gc), self._ptr(gd), self._ptr(gx0), int(nthreads)))
        if complex:
            gb, gc, gd, gx0 = (a[..., 0] + 1j * a[..., 1] for a in (gb, gc, gd, gx0))
        return gb, gc, gd, gx0

    def compose(self, sel_or_logits, sel_mode: str, dict_idx, diag, *, complex: bool):
        """Total operator A_{L-1}...A_0 per sequence: (pi int32 [B,H,N], d [B,H,N])."""
        src = self._arr(sel_or_logits)
        dct = self._arr(dict_idx, np.int32)
        dg = self._arr(diag, np.float32)
        H, K, N = dct.shape
        B, _, L = dg.shape[:3]
        pi = np.empty((B, H, N), dtype=np.int32)
        d = np.empty((B, H, N, 2) if complex else (B, H, N), dtype=np.float64)
        self._check(self.lib.pdssm_oracle_compose(
            self._ptr(src), SEL_KIND[sel_mode], self._ptr(dct), self._ptr(dg), int(complex),
            B, H, L, N, K, self._ptr(pi), self._ptr(d)))
        if complex:
            d = d[..., 0] + 1j * d[..., 1]
        return pi, d

    def scan_inputs(self, inp, nthreads: int = 1, x0: Optional[object] = "from_inputs"):
        """Scan a ``ScanInputs`` batch (from structured_sparse_state_amd.inputs)."""
        x0v = inp.x0 if isinstance(x0, str) else x0
        return self.scan(inp.sel_or_logits, inp.sel_mode, inp.dict_idx, inp.diag, inp.b, inp.c,
                         complex=inp.complex, bc_bf16=inp.bc_bf16, x0=x0v, nthreads=nthreads)

    def compose_inputs(self, inp):
        return self.compose(inp.sel_or_logits, inp.sel_mode, inp.dict_idx, inp.diag,
                            complex=inp.complex)


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from this directory's source (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle(LIBRARY)
    return _default
