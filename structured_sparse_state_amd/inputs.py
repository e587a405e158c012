"""Seeded synthetic inputs for the PD recurrence scan.

This module only draws data: it holds none of the recurrence's arithmetic, so
both the HIP path and the fp64 oracle can be fed from it without sharing any
computation.  Every tensor is produced by ``torch`` random generators seeded
from a config id, on the device the caller asks for (CPU for oracle-sized
cases, the GPU for full-size workloads).  bf16 tensors come from one
round-to-nearest-even rounding of fp32 draws (``Tensor.to(torch.bfloat16)``).

Layouts (all contiguous, row-major):

* ``sel``      int32 / int16   ``[B, H, L]``        selected dictionary entry
* ``logits``   fp32 / bf16     ``[B, H, L, K]``     router scores (argmax picks)
* ``dict_idx`` int32           ``[H, K, N]``        column j of entry k has its
  single non-zero in row ``dict_idx[h, k, j]``
* ``diag``     fp32            ``[B, H, L, N]`` (real) or ``[B, H, L, N, 2]``
  (complex, interleaved re/im)
* ``b``, ``c`` fp32 / bf16     same shape as ``diag``
* ``x0``       fp32            ``[B, H, N]`` or ``[B, H, N, 2]`` (optional)

The workloads mirror the shapes the Flash PD-SSM pages describe (Technical
Summary, "Experimental Results": time series longer than 17,000 steps,
language-model layers, synthetic state tracking); no dataset is used.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

SEL_I32 = "sel_i32"
SEL_I16 = "sel_i16"
LOGITS_F32 = "logits_f32"
LOGITS_BF16 = "logits_bf16"
SEL_MODES = (SEL_I32, SEL_I16, LOGITS_F32, LOGITS_BF16)


@dataclasses.dataclass
class ScanInputs:
    """One batch of scan inputs plus the storage modes they use."""

    sel_mode: str
    sel_or_logits: torch.Tensor
    dict_idx: torch.Tensor
    diag: torch.Tensor
    b: torch.Tensor
    c: torch.Tensor
    complex: bool
    bc_bf16: bool
    y_bf16: bool
    x0: Optional[torch.Tensor] = None
    B: int = 0
    H: int = 0
    L: int = 0
    N: int = 0
    K: int = 0

    def to(self, device) -> "ScanInputs":
        out = dataclasses.replace(self)
        for f in ("sel_or_logits", "dict_idx", "diag", "b", "c", "x0"):
            v = getattr(self, f)
            if v is not None:
                setattr(out, f, v.to(device).contiguous())
        return out

    def input_bytes(self) -> int:
        n = 0
        for f in ("sel_or_logits", "dict_idx", "diag", "b", "c", "x0"):
            v = getattr(self, f)
            if v is not None:
                n += v.numel() * v.element_size()
        return n

    def sequence(self, bi: int, hi: int) -> "ScanInputs":
        """The single (b, h) sequence as a B=H=1 batch (views copied)."""
        out = dataclasses.replace(self, B=1, H=1)
        out.sel_or_logits = self.sel_or_logits[bi:bi + 1, hi:hi + 1].contiguous()
        out.dict_idx = self.dict_idx[hi:hi + 1].contiguous()
        out.diag = self.diag[bi:bi + 1, hi:hi + 1].contiguous()
        out.b = self.b[bi:bi + 1, hi:hi + 1].contiguous()
        out.c = self.c[bi:bi + 1, hi:hi + 1].contiguous()
        if self.x0 is not None:
            out.x0 = self.x0[bi:bi + 1, hi:hi + 1].contiguous()
        return out


# Config presets: (B, H, L, N, K) and the value distributions of each workload.
CONFIGS = {
    # Tiny: index selection, real fp32 everything.
    "tiny": dict(B=1, H=1, L=256, N=8, K=4, sel_mode=SEL_I32, dict_kind="map",
                 complex=False, dmin=0.5, dmax=1.0, bc_bf16=False, y_bf16=False, seed=1),
    # Small: fp32 router logits, real fp32.
    "small": dict(B=8, H=16, L=2048, N=16, K=16, sel_mode=LOGITS_F32, dict_kind="map",
                  complex=False, dmin=0.8, dmax=1.0, bc_bf16=False, y_bf16=False, seed=2),
    # Long time-series shape: permutation dictionaries, complex64 everything.
    "long": dict(B=4, H=32, L=18000, N=32, K=32, sel_mode=SEL_I32, dict_kind="perm",
                 complex=True, dmin=0.9, dmax=0.999, bc_bf16=False, y_bf16=False, seed=3),
    # LM-layer shape: bf16 logits, complex64 diag, bf16 b/c/y.
    "lm": dict(B=8, H=32, L=4096, N=64, K=64, sel_mode=LOGITS_BF16, dict_kind="map",
               complex=True, dmin=0.95, dmax=0.999, bc_bf16=True, y_bf16=True, seed=4),
    # Very long: int16 selection, complex64 diag, bf16 b/c/y.
    "verylong": dict(B=2, H=64, L=131072, N=64, K=128, sel_mode=SEL_I16, dict_kind="map",
                     complex=True, dmin=0.99, dmax=0.9999, bc_bf16=True, y_bf16=True, seed=5),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_dict(H: int, K: int, N: int, kind: str, g: torch.Generator, device) -> torch.Tensor:
    """Dictionary index maps [H, K, N]: iid targets ("map") or permutations ("perm")."""
    if kind == "map":
        return torch.randint(0, N, (H, K, N), generator=g, device=device, dtype=torch.int32)
    if kind == "perm":
        keys = torch.rand((H, K, N), generator=g, device=device)
        return torch.argsort(keys, dim=-1).to(torch.int32)
    raise ValueError(kind)


def make_inputs(name: str = "lm", *, device="cpu", seed: Optional[int] = None,
                B: Optional[int] = None, H: Optional[int] = None, L: Optional[int] = None,
                with_x0: bool = False, **overrides) -> ScanInputs:
    """Seeded inputs for a named workload, optionally with smaller B/H/L.

    The value distributions follow the named workload whatever the sizes, so
    a scaled-down case has the same statistics as the full one.
    """
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    B = cfg["B"] if B is None else B
    H = cfg["H"] if H is None else H
    L = cfg["L"] if L is None else L
    N, K = cfg["N"], cfg["K"]
    seed = cfg["seed"] if seed is None else seed
    g = _gen(device, seed)
    cplx = cfg["complex"]

    dict_idx = make_dict(H, K, N, cfg["dict_kind"], g, device)

    mode = cfg["sel_mode"]
    if mode in (SEL_I32, SEL_I16):
        dt = torch.int32 if mode == SEL_I32 else torch.int16
        sel = torch.randint(0, K, (B, H, L), generator=g, device=device, dtype=torch.int32).to(dt)
    else:
        sel = torch.randn((B, H, L, K), generator=g, device=device, dtype=torch.float32)
        if mode == LOGITS_BF16:
            sel = sel.to(torch.bfloat16)

    mag = cfg["dmin"] + (cfg["dmax"] - cfg["dmin"]) * torch.rand(
        (B, H, L, N), generator=g, device=device, dtype=torch.float32)
    if cplx:
        phase = (2.0 * math.pi) * torch.rand((B, H, L, N), generator=g, device=device,
                                             dtype=torch.float32)
        diag = torch.stack((mag * torch.cos(phase), mag * torch.sin(phase)), dim=-1)
        shape = (B, H, L, N, 2)
        # bf16 configs draw N(0,1) per component; fp32 complex draws N(0, 1/2).
        std = 1.0 if cfg["bc_bf16"] else math.sqrt(0.5)
    else:
        sign = torch.where(torch.rand((B, H, L, N), generator=g, device=device) < 0.5, -1.0, 1.0)
        diag = mag * sign
        shape = (B, H, L, N)
        std = 1.0
    b = std * torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    c = std * torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if cfg["bc_bf16"]:
        b = b.to(torch.bfloat16)
        c = c.to(torch.bfloat16)

    x0 = None
    if with_x0:
        xs = (B, H, N, 2) if cplx else (B, H, N)
        x0 = torch.randn(xs, generator=g, device=device, dtype=torch.float32)

    return ScanInputs(sel_mode=mode, sel_or_logits=sel.contiguous(), dict_idx=dict_idx.contiguous(),
                      diag=diag.contiguous(), b=b.contiguous(), c=c.contiguous(), complex=cplx,
                      bc_bf16=cfg["bc_bf16"], y_bf16=cfg["y_bf16"], x0=x0,
                      B=B, H=H, L=L, N=N, K=K)


# ---------------------------------------------------------------------------
# Finite-state-automaton inputs.  Each dictionary entry k is the transition
# function q -> delta(q, k) of an automaton written as an index map; D = I and
# b = 0, so the state stays a one-hot (or count) vector.  Which automata: the
# state-tracking families the Flash PD-SSM pages test (Technical Summary,
# "Synthetic State-Tracking": parity, modular counting, cycle navigation) plus
# a non-injective reset automaton.
# ---------------------------------------------------------------------------

def fsa_dictionary(kind: str, N: int, m: int) -> list:
    """Transition maps (lists of length N) of automaton family `kind` on m states.

    States m..N-1 (padding) map to themselves.
    """
    ident = list(range(N))

    def on_cycle(f):
        t = list(ident)
        for q in range(m):
            t[q] = f(q)
        return t

    if kind == "parity":          # {identity, swap of states 0 and 1}
        swap = list(ident)
        swap[0], swap[1] = 1, 0
        return [ident, swap]
    if kind == "modcount":        # {identity, +1 mod m}
        return [ident, on_cycle(lambda q: (q + 1) % m)]
    if kind == "cycle":           # {+1, -1, stay} on an m-cycle
        return [on_cycle(lambda q: (q + 1) % m), on_cycle(lambda q: (q - 1) % m), ident]
    if kind == "reset":           # non-injective: reset to 0, +1 mod m, merge 1 into 0
        merge = list(ident)
        merge[1] = 0
        return [on_cycle(lambda q: 0), on_cycle(lambda q: (q + 1) % m), merge]
    raise ValueError(kind)


def make_fsa_inputs(kind: str, *, B: int = 1, H: int = 1, L: int = 256, N: int = 8, m: int = 5,
                    seed: int = 11, device="cpu", start_state: int = 0, count_state: bool = False,
                    sel_mode: str = SEL_I32, complex: bool = False) -> ScanInputs:
    """Automaton inputs: D = I, b = 0, x0 = e_{start} (or all ones on the m states).

    The readout vector is c_i = base**i on the m automaton states (0 on
    padding), with base 2 for a one-hot state and m + 1 for a count state, so
    y_t is an exact integer that encodes the whole state vector at step t.
    """
    g = _gen(device, seed)
    maps = fsa_dictionary(kind, N, m)
    K = len(maps)
    dict_idx = torch.tensor(maps, dtype=torch.int32, device=device).unsqueeze(0).repeat(H, 1, 1)
    sel32 = torch.randint(0, K, (B, H, L), generator=g, device=device, dtype=torch.int32)
    if sel_mode == SEL_I32:
        sel = sel32
    elif sel_mode == SEL_I16:
        sel = sel32.to(torch.int16)
    else:
        # Logits whose unique maximum sits at the drawn index.
        lg = torch.randn((B, H, L, K), generator=g, device=device, dtype=torch.float32)
        lg.scatter_(-1, sel32.long().unsqueeze(-1), 8.0)
        sel = lg.to(torch.bfloat16) if sel_mode == LOGITS_BF16 else lg
    shape = (B, H, L, N, 2) if complex else (B, H, L, N)
    diag = torch.zeros(shape, dtype=torch.float32, device=device)
    if complex:
        diag[..., 0] = 1.0
    else:
        diag.fill_(1.0)
    b = torch.zeros(shape, dtype=torch.float32, device=device)
    c = torch.zeros(shape, dtype=torch.float32, device=device)
    base = float(m + 1) if count_state else 2.0
    enc = torch.tensor([base ** i for i in range(m)], dtype=torch.float32, device=device)
    if complex:
        c[..., :m, 0] = enc
    else:
        c[..., :m] = enc
    xs = (B, H, N, 2) if complex else (B, H, N)
    x0 = torch.zeros(xs, dtype=torch.float32, device=device)
    if count_state:
        if complex:
            x0[:, :, :m, 0] = 1.0
        else:
            x0[:, :, :m] = 1.0
    else:
        if complex:
            x0[:, :, start_state, 0] = 1.0
        else:
            x0[:, :, start_state] = 1.0
    return ScanInputs(sel_mode=sel_mode, sel_or_logits=sel.contiguous(), dict_idx=dict_idx.contiguous(),
                      diag=diag, b=b, c=c, complex=complex, bc_bf16=False, y_bf16=False, x0=x0,
                      B=B, H=H, L=L, N=N, K=K)


def make_dense_dict(H: int, K: int, N: int, *, bf16: bool = False, seed: int = 21, device="cpu",
                    ties: bool = False) -> torch.Tensor:
    """Dense dictionary matrices [H,K,N,N] (row i, column j) whose column-wise
    hardmax gives the index maps: N(0,1) draws, or, with ``ties``, a few
    distinct values so that equal maxima in a column are common.  bf16 from
    one RNE rounding of the fp32 draws."""
    g = _gen(device, seed)
    if ties:
        m = torch.randint(-3, 4, (H, K, N, N), generator=g, device=device).to(torch.float32) * 0.5
    else:
        m = torch.randn((H, K, N, N), generator=g, device=device, dtype=torch.float32)
    return m.to(torch.bfloat16) if bf16 else m


def make_router_inputs(B: int, L: int, H: int, K: int, D: int, *, seed: int = 31, device="cpu",
                       integers: bool = False):
    """Step inputs u bf16 [B,L,D] ~ N(0,1) and router weights w bf16 [H,K,D]
    ~ N(0, 1/D) (so every score is of order one), each from one RNE
    rounding of fp32 draws; with ``integers``, small integers instead, so
    that every fp32 sum of products is exact and equal scores are common."""
    g = _gen(device, seed)
    if integers:
        u = torch.randint(-3, 4, (B, L, D), generator=g, device=device).to(torch.bfloat16)
        w = torch.randint(-2, 3, (H, K, D), generator=g, device=device).to(torch.bfloat16)
        return u, w
    u = torch.randn((B, L, D), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn((H, K, D), generator=g, device=device, dtype=torch.float32) / math.sqrt(D)).to(
        torch.bfloat16)
    return u, w


def make_grads(inp: ScanInputs, *, seed: int = 0, with_gx_final: bool = True, device=None):
    """Seeded upstream gradients for the backward scan of ``inp``: gy in the
    storage of y ([B,H,L], N(0,1), bf16 rounded once when y is bf16) and
    gx_final fp32 [B,H,N(,2)] N(0,1), or None."""
    device = device or inp.diag.device
    g = _gen(device, 7919 + seed)
    gy = torch.randn((inp.B, inp.H, inp.L), generator=g, device=device, dtype=torch.float32)
    if inp.y_bf16:
        gy = gy.to(torch.bfloat16)
    gxf = None
    if with_gx_final:
        tail = (inp.N, 2) if inp.complex else (inp.N,)
        gxf = torch.randn((inp.B, inp.H) + tail, generator=g, device=device, dtype=torch.float32)
    return gy, gxf


def make_adversarial_scores(B: int, H: int, L: int, K: int, *, bf16: bool, seed: int = 71,
                            device="cpu") -> torch.Tensor:
    """Router scores [B, H, L, K] that exercise every rule of the hard
    selection, in fp32 or bf16 (every value is exact in both):

    * small integers in [-3, 3], so most rows hold exact ties at their maximum;
    * rows whose maximum is a -0 / +0 pair (every other score negative);
    * rows with one NaN, and rows with two or three NaNs;
    * rows with +inf at one or two places and -inf elsewhere in the row;
    * rows that are -inf throughout.

    Each step draws its row kind and the positions it uses from the seeded
    generator; nothing here depends on how the selection is computed."""
    g = _gen(device, seed)
    v = torch.randint(-3, 4, (B, H, L, K), generator=g, device=device).to(torch.float32)
    kind = torch.randint(0, 10, (B, H, L, 1), generator=g, device=device)
    pos = torch.randint(0, K, (B, H, L, 3), generator=g, device=device)
    cols = torch.arange(K, device=device).view(1, 1, 1, K)
    at = [cols == pos[..., i:i + 1] for i in range(3)]
    nan, inf = float("nan"), float("inf")
    # kind 3: all negative except a -0 (first drawn place) and a +0 (second)
    neg = -(v.abs() + 1.0)
    zero_row = torch.where(at[1], torch.zeros_like(v), neg)
    zero_row = torch.where(at[0], torch.full_like(v, -0.0), zero_row)
    v = torch.where(kind == 3, zero_row, v)
    # kind 4: one NaN; kind 5: up to three NaNs
    v = torch.where((kind == 4) & at[0], torch.full_like(v, nan), v)
    several = (kind == 5) & (at[0] | at[1] | at[2])
    v = torch.where(several, torch.full_like(v, nan), v)
    # kind 6: +inf at up to two places, -inf at a third (unless it is one of them)
    v = torch.where((kind == 6) & at[2], torch.full_like(v, -inf), v)
    v = torch.where((kind == 6) & (at[0] | at[1]), torch.full_like(v, inf), v)
    # kind 7: -inf throughout
    v = torch.where(kind == 7, torch.full_like(v, -inf), v)
    return v.to(torch.bfloat16) if bf16 else v
