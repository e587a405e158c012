"""Flash PD-SSM recurrence scan for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libpdssm.so`` (hand-written HIP
kernels, declared in ``include/pdssm.h``).  This module is a thin ctypes
binding with the same function names: it only turns torch tensors into
device pointers and the current HIP stream into a ``hipStream_t``.  Every
step runs in the library's kernels; there is no fallback, and a missing
library raises.

Higher-level helpers allocate outputs (and workspaces) with torch and call
the C entry points: ``scan`` and ``scan_save`` (forward), ``scan_bwd``
(gradients), ``router_select`` (router scores and their argmax) with
``router_pack_weights`` (the weights in the faster kernel's layout),
``dict_hardmax`` (index maps from dense matrices), ``decode_step`` (one
recurrent step), ``select`` and ``compose`` (test exports).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re
from typing import NamedTuple, Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libpdssm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pdssm.h")

# Flag and status values of include/pdssm.h (tests check they agree).
PDSSM_SEL_I32 = 0x0
PDSSM_SEL_I16 = 0x1
PDSSM_LOGITS_F32 = 0x2
PDSSM_LOGITS_BF16 = 0x3
PDSSM_SEL_MASK = 0x3
PDSSM_COMPLEX = 0x4
PDSSM_BC_BF16 = 0x8
PDSSM_Y_BF16 = 0x10
PDSSM_DETERMINISTIC = 0x20
PDSSM_FLAGS_ALL = 0x3F
PDSSM_ROUTER_W_PACKED = 0x1

PDSSM_OK = 0
PDSSM_ERR_NULL = -1
PDSSM_ERR_DIM = -2
PDSSM_ERR_FLAGS = -3
PDSSM_ERR_ALIGN = -4
PDSSM_ERR_WORKSPACE = -5
PDSSM_ERR_HIP = -6
PDSSM_ERR_SCRATCH = -7

SEL_FLAG = {"sel_i32": PDSSM_SEL_I32, "sel_i16": PDSSM_SEL_I16,
            "logits_f32": PDSSM_LOGITS_F32, "logits_bf16": PDSSM_LOGITS_BF16}

_LIB = None


class PdssmError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"pdssm status {status}: {text}")
        self.status = status


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    P, I64, I32, U32, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                            ctypes.c_size_t)
    lib.pdssm_scan_fwd.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I32, I32, U32, P, P, SZ, P]
    lib.pdssm_scan_fwd.restype = ctypes.c_int
    lib.pdssm_scan_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I32, I32, U32, P, P]
    lib.pdssm_scan_fwd_noalloc.restype = ctypes.c_int
    lib.pdssm_scan_workspace_bytes.argtypes = [I64, I64, I64, I32, I32, U32]
    lib.pdssm_scan_workspace_bytes.restype = SZ
    lib.pdssm_select.argtypes = [P, P, I64, I64, I64, I32, U32, P]
    lib.pdssm_select.restype = ctypes.c_int
    lib.pdssm_compose.argtypes = [P, P, P, P, P, I64, I64, I64, I32, I32, U32, P, SZ, P]
    lib.pdssm_compose.restype = ctypes.c_int
    lib.pdssm_scan_fwd_save.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I32, I32, U32, P,
                                        P, SZ, P]
    lib.pdssm_scan_fwd_save.restype = ctypes.c_int
    lib.pdssm_scan_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I32, I32, U32,
                                   P, SZ, P]
    lib.pdssm_scan_bwd.restype = ctypes.c_int
    lib.pdssm_scan_bwd_workspace_bytes.argtypes = [I64, I64, I64, I32, I32, U32]
    lib.pdssm_scan_bwd_workspace_bytes.restype = SZ
    lib.pdssm_strerror.argtypes = [ctypes.c_int]
    lib.pdssm_strerror.restype = ctypes.c_char_p
    lib.pdssm_dict_hardmax.argtypes = [P, P, I64, I32, I32, U32, P]
    lib.pdssm_dict_hardmax.restype = ctypes.c_int
    lib.pdssm_decode_step.argtypes = [P, P, P, P, P, P, P, I64, I64, I32, I32, U32, P]
    lib.pdssm_decode_step.restype = ctypes.c_int
    lib.pdssm_router_select.argtypes = [P, P, P, I64, I64, I64, I32, I32, U32, P]
    lib.pdssm_router_select.restype = ctypes.c_int
    lib.pdssm_router_pack_weights.argtypes = [P, P, I64, I32, I32, P]
    lib.pdssm_router_pack_weights.restype = ctypes.c_int
    return lib


def library() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        _LIB = _load(LIBRARY)
    return _LIB


_VARIANTS = {}


@contextlib.contextmanager
def variant(name: str):
    """Route every call in the block through the test build ``name`` of the
    library (``libpdssm_<name>.so``, see build_lib.VARIANTS)."""
    global _LIB
    if name not in _VARIANTS:
        _VARIANTS[name] = _load(os.path.join(HERE, f"libpdssm_{name}.so"))
    saved = library()
    _LIB = _VARIANTS[name]
    try:
        yield _LIB
    finally:
        _LIB = saved


def header_functions() -> list:
    """Names of the functions include/pdssm.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(pdssm_[a-z_]+)\s*\(", text)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# The C entry points, same names and argument order.  Tensors (or raw
# addresses) in, status code out.
# ---------------------------------------------------------------------------

def pdssm_scan_fwd(sel_or_logits, dict_idx, diag, b, c, y, x_final, B, H, L, N, K, flags, x0,
                   workspace, workspace_bytes, stream=None) -> int:
    return library().pdssm_scan_fwd(_ptr(sel_or_logits), _ptr(dict_idx), _ptr(diag), _ptr(b),
                                    _ptr(c), _ptr(y), _ptr(x_final), B, H, L, N, K, flags,
                                    _ptr(x0), _ptr(workspace), workspace_bytes, _stream(stream))


def pdssm_scan_fwd_noalloc(sel_or_logits, dict_idx, diag, b, c, y, x_final, B, H, L, N, K, flags,
                           x0, stream=None) -> int:
    return library().pdssm_scan_fwd_noalloc(_ptr(sel_or_logits), _ptr(dict_idx), _ptr(diag), _ptr(b),
                                            _ptr(c), _ptr(y), _ptr(x_final), B, H, L, N, K, flags,
                                            _ptr(x0), _stream(stream))


def pdssm_scan_workspace_bytes(B, H, L, N, K, flags) -> int:
    return library().pdssm_scan_workspace_bytes(B, H, L, N, K, flags)


def pdssm_scan_fwd_save(sel_or_logits, dict_idx, diag, b, c, y, x_final, x_chunks, sel_out, B, H,
                        L, N, K, flags, x0, workspace, workspace_bytes, stream=None) -> int:
    return library().pdssm_scan_fwd_save(_ptr(sel_or_logits), _ptr(dict_idx), _ptr(diag), _ptr(b),
                                         _ptr(c), _ptr(y), _ptr(x_final), _ptr(x_chunks),
                                         _ptr(sel_out), B, H, L, N, K, flags, _ptr(x0),
                                         _ptr(workspace), workspace_bytes, _stream(stream))


def pdssm_scan_bwd(sel_or_logits, dict_idx, diag, b, c, x_chunks, gy, gx_final, gb, gc, gd, gx0, B,
                   H, L, N, K, flags, workspace, workspace_bytes, stream=None) -> int:
    return library().pdssm_scan_bwd(_ptr(sel_or_logits), _ptr(dict_idx), _ptr(diag), _ptr(b),
                                    _ptr(c), _ptr(x_chunks), _ptr(gy), _ptr(gx_final), _ptr(gb),
                                    _ptr(gc), _ptr(gd), _ptr(gx0), B, H, L, N, K, flags,
                                    _ptr(workspace), workspace_bytes, _stream(stream))


def pdssm_scan_bwd_workspace_bytes(B, H, L, N, K, flags) -> int:
    return library().pdssm_scan_bwd_workspace_bytes(B, H, L, N, K, flags)


def pdssm_select(sel_or_logits, sel_out, B, H, L, K, flags, stream=None) -> int:
    return library().pdssm_select(_ptr(sel_or_logits), _ptr(sel_out), B, H, L, K, flags,
                                  _stream(stream))


def pdssm_compose(sel_or_logits, dict_idx, diag, pi_out, d_out, B, H, L, N, K, flags, workspace,
                  workspace_bytes, stream=None) -> int:
    return library().pdssm_compose(_ptr(sel_or_logits), _ptr(dict_idx), _ptr(diag), _ptr(pi_out),
                                   _ptr(d_out), B, H, L, N, K, flags, _ptr(workspace),
                                   workspace_bytes, _stream(stream))


def pdssm_dict_hardmax(m, dict_idx, H, K, N, flags, stream=None) -> int:
    return library().pdssm_dict_hardmax(_ptr(m), _ptr(dict_idx), H, K, N, flags, _stream(stream))


def pdssm_decode_step(sel_or_logits, dict_idx, diag, b, c, y, x, B, H, N, K, flags,
                      stream=None) -> int:
    return library().pdssm_decode_step(_ptr(sel_or_logits), _ptr(dict_idx), _ptr(diag), _ptr(b),
                                       _ptr(c), _ptr(y), _ptr(x), B, H, N, K, flags,
                                       _stream(stream))


def pdssm_router_select(u, w, sel_out, B, L, H, K, D, flags, stream=None) -> int:
    return library().pdssm_router_select(_ptr(u), _ptr(w), _ptr(sel_out), B, L, H, K, D, flags,
                                         _stream(stream))


def pdssm_router_pack_weights(w, w_packed, H, K, D, stream=None) -> int:
    return library().pdssm_router_pack_weights(_ptr(w), _ptr(w_packed), H, K, D, _stream(stream))


def pdssm_strerror(status: int) -> str:
    return library().pdssm_strerror(status).decode()


def check(status: int) -> None:
    if status != PDSSM_OK:
        raise PdssmError(status, pdssm_strerror(status))


# ---------------------------------------------------------------------------
# Convenience layer over ScanInputs-like objects (fields: sel_mode,
# sel_or_logits, dict_idx, diag, b, c, x0, complex, bc_bf16, y_bf16, B, H,
# L, N, K), all tensors on the GPU.
# ---------------------------------------------------------------------------

def flags_of(inp, deterministic: bool = False) -> int:
    f = SEL_FLAG[inp.sel_mode]
    if deterministic:
        f |= PDSSM_DETERMINISTIC
    if inp.complex:
        f |= PDSSM_COMPLEX
    if inp.bc_bf16:
        f |= PDSSM_BC_BF16
    if inp.y_bf16:
        f |= PDSSM_Y_BF16
    return f


def workspace_for(inp, device=None) -> torch.Tensor:
    n = pdssm_scan_workspace_bytes(inp.B, inp.H, inp.L, inp.N, inp.K, flags_of(inp))
    if n == 0:
        raise PdssmError(PDSSM_ERR_DIM, "invalid sizes")
    return torch.empty(n, dtype=torch.uint8, device=device or inp.diag.device)


def scan(inp, *, workspace: Optional[torch.Tensor] = None, want_x_final: bool = True,
         y: Optional[torch.Tensor] = None, x_final: Optional[torch.Tensor] = None, stream=None,
         x0="from_inputs", deterministic: bool = False):
    """Run pdssm_scan_fwd on a batch; returns (y, x_final or None).
    ``deterministic`` sets PDSSM_DETERMINISTIC (bitwise reproducible)."""
    dev = inp.diag.device
    if y is None:
        y = torch.empty((inp.B, inp.H, inp.L), device=dev,
                        dtype=torch.bfloat16 if inp.y_bf16 else torch.float32)
    if want_x_final and x_final is None:
        shape = (inp.B, inp.H, inp.N, 2) if inp.complex else (inp.B, inp.H, inp.N)
        x_final = torch.empty(shape, device=dev, dtype=torch.float32)
    if workspace is None:
        workspace = workspace_for(inp)
    x0t = inp.x0 if isinstance(x0, str) else x0
    check(pdssm_scan_fwd(inp.sel_or_logits, inp.dict_idx, inp.diag, inp.b, inp.c, y,
                         x_final if want_x_final else None, inp.B, inp.H, inp.L, inp.N, inp.K,
                         flags_of(inp, deterministic), x0t, workspace, workspace.numel(), stream))
    return y, (x_final if want_x_final else None)


def scan_noalloc(inp, *, y: Optional[torch.Tensor] = None, x_final: Optional[torch.Tensor] = None,
                 stream=None, deterministic: bool = False):
    """pdssm_scan_fwd_noalloc on a batch (the library's own device scratch in
    place of a workspace); returns (y, x_final).  Output tensors passed in are
    written in place, so the call itself allocates nothing."""
    dev = inp.diag.device
    if y is None:
        y = torch.empty((inp.B, inp.H, inp.L), device=dev,
                        dtype=torch.bfloat16 if inp.y_bf16 else torch.float32)
    if x_final is None:
        shape = (inp.B, inp.H, inp.N, 2) if inp.complex else (inp.B, inp.H, inp.N)
        x_final = torch.empty(shape, device=dev, dtype=torch.float32)
    check(pdssm_scan_fwd_noalloc(inp.sel_or_logits, inp.dict_idx, inp.diag, inp.b, inp.c, y, x_final,
                                 inp.B, inp.H, inp.L, inp.N, inp.K, flags_of(inp, deterministic), inp.x0,
                                 stream))
    return y, x_final


CARRY_STRIDE = 16   # steps per saved chunk carry (include/pdssm.h)


def scan_save(inp, *, workspace: Optional[torch.Tensor] = None, stream=None, want_sel: bool = False,
              deterministic: bool = False):
    """pdssm_scan_fwd_save on a batch: (y, x_final, x_chunks), plus the int16
    selections [B,H,L] when want_sel."""
    dev = inp.diag.device
    y = torch.empty((inp.B, inp.H, inp.L), device=dev,
                    dtype=torch.bfloat16 if inp.y_bf16 else torch.float32)
    tail = (inp.N, 2) if inp.complex else (inp.N,)
    x_final = torch.empty((inp.B, inp.H) + tail, device=dev, dtype=torch.float32)
    nch = (inp.L + CARRY_STRIDE - 1) // CARRY_STRIDE
    x_chunks = torch.empty((inp.B, inp.H, nch) + tail, device=dev, dtype=torch.float32)
    if workspace is None:
        workspace = workspace_for(inp)
    sel = torch.empty((inp.B, inp.H, inp.L), device=dev, dtype=torch.int16) if want_sel else None
    check(pdssm_scan_fwd_save(inp.sel_or_logits, inp.dict_idx, inp.diag, inp.b, inp.c, y, x_final,
                              x_chunks, sel, inp.B, inp.H, inp.L, inp.N, inp.K,
                              flags_of(inp, deterministic), inp.x0,
                              workspace, workspace.numel(), stream))
    if want_sel:
        return y, x_final, x_chunks, sel
    return y, x_final, x_chunks


def bwd_workspace_for(inp, device=None) -> torch.Tensor:
    n = pdssm_scan_bwd_workspace_bytes(inp.B, inp.H, inp.L, inp.N, inp.K, flags_of(inp))
    if n == 0:
        raise PdssmError(PDSSM_ERR_DIM, "invalid sizes")
    return torch.empty(n, dtype=torch.uint8, device=device or inp.diag.device)


def scan_bwd(inp, x_chunks, gy, gx_final=None, *, want_gx0: bool = True,
             workspace: Optional[torch.Tensor] = None, stream=None, out=None, sel=None,
             deterministic: bool = False):
    """pdssm_scan_bwd on a batch: (gb, gc, gd, gx0 or None), in the storage
    of b, c, diag and x0.  ``sel``: the forward's saved int16 selections
    (scan_save(want_sel=True)), used in place of the inputs' scores.  ``out``
    may hold a previous call's result tuple to write into instead of
    allocating."""
    dev = inp.diag.device
    if out is not None:
        gb, gc, gd, gx0 = out
    else:
        gb = torch.empty_like(inp.b)
        gc = torch.empty_like(inp.c)
        gd = torch.empty_like(inp.diag)
        tail = (inp.N, 2) if inp.complex else (inp.N,)
        gx0 = torch.empty((inp.B, inp.H) + tail, device=dev, dtype=torch.float32) if want_gx0 else None
    if workspace is None:
        workspace = bwd_workspace_for(inp)
    flags = flags_of(inp, deterministic)
    if sel is not None:
        flags = (flags & ~PDSSM_SEL_MASK) | PDSSM_SEL_I16
    check(pdssm_scan_bwd(inp.sel_or_logits if sel is None else sel, inp.dict_idx, inp.diag, inp.b,
                         inp.c, x_chunks, gy, gx_final, gb, gc, gd, gx0, inp.B, inp.H, inp.L, inp.N,
                         inp.K, flags,
                         workspace, workspace.numel(), stream))
    return gb, gc, gd, gx0


def select(sel_or_logits, sel_mode: str, K: int, stream=None) -> torch.Tensor:
    shape = sel_or_logits.shape if sel_mode.startswith("sel") else sel_or_logits.shape[:-1]
    B, H, L = shape
    out = torch.empty((B, H, L), dtype=torch.int32, device=sel_or_logits.device)
    check(pdssm_select(sel_or_logits, out, B, H, L, K, SEL_FLAG[sel_mode], stream))
    return out


def compose(inp, workspace: Optional[torch.Tensor] = None, stream=None):
    """Total operator of every sequence: (pi int32 [B,H,N], d fp32 [B,H,N(,2)])."""
    dev = inp.diag.device
    flags = SEL_FLAG[inp.sel_mode] | (PDSSM_COMPLEX if inp.complex else 0)
    pi = torch.empty((inp.B, inp.H, inp.N), dtype=torch.int32, device=dev)
    d = torch.empty((inp.B, inp.H, inp.N, 2) if inp.complex else (inp.B, inp.H, inp.N),
                    dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = workspace_for(inp)
    check(pdssm_compose(inp.sel_or_logits, inp.dict_idx, inp.diag, pi, d, inp.B, inp.H, inp.L,
                        inp.N, inp.K, flags, workspace, workspace.numel(), stream))
    return pi, d


def dict_hardmax(m: torch.Tensor, stream=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dict_idx int32 [H,K,N] from dense matrices m [H,K,N,N] (fp32 or bf16):
    the column-wise hardmax of every matrix."""
    H, K, N, N2 = m.shape
    if N != N2:
        raise ValueError("m must be [H,K,N,N]")
    flags = PDSSM_LOGITS_BF16 if m.dtype == torch.bfloat16 else PDSSM_LOGITS_F32
    if out is None:
        out = torch.empty((H, K, N), dtype=torch.int32, device=m.device)
    check(pdssm_dict_hardmax(m, out, H, K, N, flags, stream))
    return out


def decode_step(sel_or_logits, dict_idx, diag, b, c, x, *, sel_mode: str, complex: bool,
                bc_bf16: bool, y_bf16: bool, y: Optional[torch.Tensor] = None, stream=None):
    """One recurrent step for every (b, h): updates the state x [B,H,N(,2)]
    in place and returns y [B,H]."""
    B, H = diag.shape[:2]
    K, N = dict_idx.shape[1], dict_idx.shape[2]
    flags = SEL_FLAG[sel_mode] | (PDSSM_COMPLEX if complex else 0) | \
        (PDSSM_BC_BF16 if bc_bf16 else 0) | (PDSSM_Y_BF16 if y_bf16 else 0)
    if y is None:
        y = torch.empty((B, H), device=diag.device,
                        dtype=torch.bfloat16 if y_bf16 else torch.float32)
    check(pdssm_decode_step(sel_or_logits, dict_idx, diag, b, c, y, x, B, H, N, K, flags, stream))
    return y


class PackedRouterWeights(NamedTuple):
    """Router weights in the packed layout (bf16 [H, D/8, P, 8]) with the
    dictionary size K they were packed for."""
    data: torch.Tensor
    K: int


def router_pack_weights(w: torch.Tensor, *, stream=None) -> PackedRouterWeights:
    """The packed layout of router weights w [H,K,D] bf16 (pack once per
    weight update; router_select then runs its faster kernel)."""
    H, K, D = w.shape
    if w.dtype != torch.bfloat16:
        raise ValueError("w [H,K,D] must be bf16")
    P = 64 if K <= 64 else 128
    out = torch.empty((H, D // 8, P, 8), dtype=torch.bfloat16, device=w.device)
    check(pdssm_router_pack_weights(w, out, H, K, D, stream))
    return PackedRouterWeights(out, K)


def router_select(u: torch.Tensor, w, *, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """sel int16 [B,H,L] from bf16 step inputs u [B,L,D] and router weights
    w (bf16 [H,K,D], or PackedRouterWeights from router_pack_weights): the
    argmax of each head's K scores, computed on the matrix cores without
    writing the scores."""
    B, L, D = u.shape
    if isinstance(w, PackedRouterWeights):
        H, D8, P, _ = w.data.shape
        K, D2, wt, flags = w.K, D8 * 8, w.data, PDSSM_ROUTER_W_PACKED
    else:
        H, K, D2 = w.shape
        wt, flags = w, 0
    if D != D2 or u.dtype != torch.bfloat16 or wt.dtype != torch.bfloat16:
        raise ValueError("u [B,L,D] and the weights must be bf16 with the same D")
    if out is None:
        out = torch.empty((B, H, L), dtype=torch.int16, device=u.device)
    check(pdssm_router_select(u, wt, out, B, L, H, K, D, flags, stream))
    return out
