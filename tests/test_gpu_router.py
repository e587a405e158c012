"""GPU parity of the fused router product + argmax (pdssm_router_select).

The oracle computes every score in fp64 (exact products of the bf16 inputs)
and takes the first maximum.  The kernel sums in fp32, so where two scores
lie within their rounding error of each other either index is correct: the
test demands, for every (b,h,t), that the kernel's choice k satisfies
    s_max - s_k <= E_k + E_kmax,   E_j = D * 2^-24 * sum_d |u_d w_jd|
(the first-order bound on an fp32 sum of D exact products), and that it
equals the oracle's index whenever the two are not that close.  With
small-integer inputs every fp32 sum is exact, and the kernel must return the
oracle's index everywhere, ties included.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_state_amd as pk
from structured_sparse_state_amd import inputs as gen
from tests.gpu_common import seq_rel_err, y_to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


# Both weight layouts: [H,K,D] as given, and the packed layout of
# router_pack_weights (another kernel, the same contract).
LAYOUTS = ["plain", "packed"]


def weights_for(w, layout):
    return w if layout == "plain" else pk.router_pack_weights(w)


def check_choice(u, w, got, ref, lg):
    """got/ref int [B,H,L], lg fp64 scores [B,H,L,K] for the same tokens."""
    uf = u.double().abs().numpy()
    wf = w.double().abs().numpy()
    D = uf.shape[-1]
    bound = np.einsum("bld,hkd->bhlk", uf, wf) * D * 2.0 ** -24 * 1.001
    smax = lg.max(axis=-1)
    take = np.take_along_axis
    s_got = take(lg, got[..., None].astype(np.int64), -1)[..., 0]
    e_got = take(bound, got[..., None].astype(np.int64), -1)[..., 0]
    e_ref = take(bound, ref[..., None].astype(np.int64), -1)[..., 0]
    assert np.all((got >= 0) & (got < lg.shape[-1]))
    ok = (got == ref) | (smax - s_got <= e_got + e_ref)
    assert ok.all(), f"{(~ok).sum()} choices outside the rounding bound"
    return int((got != ref).sum())


ROUTER_SHAPES = [
    # B, L, H, K, D
    (1, 1, 1, 1, 32),
    (2, 100, 3, 5, 64),
    (1, 300, 2, 64, 256),
    (2, 257, 5, 33, 96),
    (1, 511, 4, 64, 2048),
    (3, 90, 1, 17, 160),
    # heads padded to 128 score columns (64 < K <= 128)
    (2, 300, 3, 100, 256),
    (1, 257, 2, 128, 512),
    (1, 513, 5, 65, 96),
    # feature counts that leave a partial last group of 128 features (8
    # steps), wrap the two-group token ring many times, or take 32-feature
    # stages
    (1, 260, 3, 64, 224),
    (1, 130, 2, 40, 4064),
    (2, 70, 2, 128, 4096),
    (1, 300, 9, 16, 1056),
]


@pytest.mark.parametrize("B,L,H,K,D", ROUTER_SHAPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_router_matches_oracle(orc, layout, B, L, H, K, D):
    say(f"[case] router {layout} B={B} L={L} H={H} K={K} D={D}")
    u, w = gen.make_router_inputs(B, L, H, K, D, seed=B * 1000 + L + K)
    ref, lg = orc.router_select(u, w, want_logits=True, nthreads=8)
    got = pk.router_select(u.to(DEV), weights_for(w.to(DEV), layout))
    torch.cuda.synchronize()
    n = check_choice(u, w, got.cpu().numpy(), ref, lg)
    say(f"  {n} near-tie choices differ from the oracle's of {ref.size}")


@pytest.mark.parametrize("B,L,H,K,D", [(1, 300, 3, 64, 64), (2, 129, 2, 7, 512), (1, 256, 2, 64, 2048),
                                       (1, 300, 3, 128, 64), (2, 129, 3, 97, 512)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_router_exact_integers(orc, layout, B, L, H, K, D):
    """Exact sums: the kernel's index equals the oracle's everywhere (the
    first maximum on ties)."""
    say(f"[case] router exact {layout} B={B} L={L} H={H} K={K} D={D}")
    u, w = gen.make_router_inputs(B, L, H, K, D, seed=7 + D, integers=True)
    ref = orc.router_select(u, w, nthreads=8)
    got = pk.router_select(u.to(DEV), weights_for(w.to(DEV), layout))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("B,L,H,K,D", [(1, 300, 3, 64, 64), (2, 129, 3, 40, 96), (1, 200, 2, 100, 128),
                                       (1, 256, 2, 128, 64)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_router_special_scores(orc, layout, B, L, H, K, D):
    """Scores that are +-inf, NaN or all zero reach the argmax's rule (NaN
    above every number and the first NaN winning, -0 equal to +0, the first
    maximum on ties): small-integer inputs, with some tokens holding an inf
    (inf * 0 gives NaN), a NaN, both infinities, or nothing but zeros.  Every
    finite sum is exact and inf/NaN arithmetic does not depend on the order
    of the sum, so the index must equal the oracle's everywhere."""
    say(f"[case] router special scores {layout} B={B} L={L} H={H} K={K} D={D}")
    u, w = gen.make_router_inputs(B, L, H, K, D, seed=11 + K + D, integers=True)
    u = u.float()
    g = torch.Generator().manual_seed(5 + K)
    d0 = torch.randint(0, D, (B, L), generator=g)
    d1 = (d0 + 1 + torch.randint(0, D - 1, (B, L), generator=g)) % D
    kind = torch.arange(L).view(1, L).expand(B, L) % 7
    rows = torch.arange(B).view(B, 1).expand(B, L)
    cols = torch.arange(L).view(1, L).expand(B, L)
    for k, val in ((1, float("inf")), (2, float("nan")), (4, float("-inf"))):
        m = kind == k
        u[rows[m], cols[m], d0[m]] = val
    m = kind == 4
    u[rows[m], cols[m], d1[m]] = float("inf")
    u[kind == 3] = 0.0
    u = u.to(torch.bfloat16)
    ref = orc.router_select(u, w, nthreads=8)
    got = pk.router_select(u.to(DEV), weights_for(w.to(DEV), layout))
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{bad.shape[0]} choices differ, first at {tuple(bad[0])}"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_router_lm_full_size_sampled(orc, layout):
    """The LM-layer router at full size (B=8 L=4096 H=32 K=64, D=2048): sampled
    tokens against the oracle, including the first and last of several
    256-token tiles."""
    B, L, H, K, D = 8, 4096, 32, 64, 2048
    say(f"[case] router lm full size {layout} B={B} L={L} H={H} K={K} D={D}")
    u, w = gen.make_router_inputs(B, L, H, K, D, seed=4, device=DEV)
    got = pk.router_select(u, weights_for(w, layout))
    torch.cuda.synchronize()
    ts = sorted({0, 1, 255, 256, 257, 511, 1000, 2047, 2048, 3071, 4094, 4095})
    for bi in (0, 5, B - 1):
        us = u[bi:bi + 1, ts].cpu().contiguous()
        ref, lg = orc.router_select(us, w.cpu(), want_logits=True, nthreads=8)
        check_choice(us, w.cpu(), got[bi:bi + 1][:, :, ts].cpu().numpy(), ref, lg)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_router_feeds_scan(orc, layout):
    """Router selections drive the scan exactly like the oracle's."""
    inp = gen.make_inputs("lm", B=1, H=4, L=300, seed=91)
    u, w = gen.make_router_inputs(1, 300, 4, 64, 128, seed=92, integers=True)
    inp.sel_or_logits = torch.from_numpy(orc.router_select(u, w)).to(torch.int16)
    inp.sel_mode = gen.SEL_I16
    g = inp.to(DEV)
    g.sel_or_logits = pk.router_select(u.to(DEV), weights_for(w.to(DEV), layout))
    assert torch.equal(g.sel_or_logits.cpu(), inp.sel_or_logits)
    y, _ = pk.scan(g)
    y_ref, _ = pk.scan(inp.to(DEV))
    torch.cuda.synchronize()
    # the same selections give the same scan, to rounding (the tiles'
    # carries may compose in another order from call to call)
    assert seq_rel_err(y_to_np(y), y_to_np(y_ref)) <= 2.0 ** -7


@pytest.mark.parametrize("H,K,D", [(1, 1, 32), (3, 64, 96), (2, 40, 256), (2, 65, 64), (3, 128, 160)])
def test_router_pack_layout(H, K, D):
    """The packed layout holds w[h][k][d] at [h][d/8][k][d%8] and zeros in the
    padding columns K <= k < P, bit for bit (a pure rearrangement)."""
    say(f"[case] router pack H={H} K={K} D={D}")
    _, w = gen.make_router_inputs(1, 1, H, K, D, seed=H + K + D)
    P = 64 if K <= 64 else 128
    got = pk.router_pack_weights(w.to(DEV))
    torch.cuda.synchronize()
    assert got.K == K and tuple(got.data.shape) == (H, D // 8, P, 8)
    want = torch.zeros(H, D // 8, P, 8, dtype=torch.bfloat16)
    want[:, :, :K, :] = w.view(H, K, D // 8, 8).permute(0, 2, 1, 3)
    assert torch.equal(got.data.cpu().view(torch.int16), want.view(torch.int16))
