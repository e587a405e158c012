"""The seeded input generator: determinism, shapes, value ranges (CPU only)."""
import math

import numpy as np
import torch

from structured_sparse_state_amd import inputs as gen


def test_deterministic_and_shapes():
    for name in ("tiny", "small", "long", "lm", "verylong"):
        a = gen.make_inputs(name, B=1, H=2, L=33)
        b = gen.make_inputs(name, B=1, H=2, L=33)
        for f in ("sel_or_logits", "dict_idx", "diag", "b", "c"):
            assert torch.equal(getattr(a, f), getattr(b, f)), (name, f)
        cfg = gen.CONFIGS[name]
        N, K = cfg["N"], cfg["K"]
        assert a.dict_idx.shape == (2, K, N) and a.dict_idx.dtype == torch.int32
        assert int(a.dict_idx.min()) >= 0 and int(a.dict_idx.max()) < N
        tail = (N, 2) if cfg["complex"] else (N,)
        assert a.diag.shape == (1, 2, 33) + tail
        assert a.b.shape == a.diag.shape and a.c.shape == a.diag.shape
        mag = a.diag.abs() if not cfg["complex"] else torch.sqrt(a.diag[..., 0].double() ** 2 +
                                                                  a.diag[..., 1].double() ** 2)
        assert float(mag.min()) >= cfg["dmin"] - 1e-6 and float(mag.max()) <= cfg["dmax"] + 1e-6
        if cfg["sel_mode"] in (gen.SEL_I32, gen.SEL_I16):
            assert int(a.sel_or_logits.min()) >= 0 and int(a.sel_or_logits.max()) < K
        else:
            assert a.sel_or_logits.shape == (1, 2, 33, K)


def test_permutation_dictionaries():
    a = gen.make_inputs("long", B=1, H=3, L=4)
    srt = torch.sort(a.dict_idx, dim=-1).values
    assert torch.equal(srt, torch.arange(32, dtype=torch.int32).expand_as(srt))


def test_bf16_is_round_to_nearest_even():
    # bf16 inputs are one RNE rounding of the fp32 draw: check against a
    # bit-level RNE written out here.
    x = torch.randn(10000, generator=torch.Generator().manual_seed(3))
    bits = x.view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    lsb = (bits >> 16) & 1
    rne = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = x.to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(got, rne)


def test_fsa_dictionaries():
    for kind, m in (("parity", 2), ("modcount", 5), ("cycle", 6), ("reset", 4)):
        maps = gen.fsa_dictionary(kind, 8, m)
        for f in maps:
            assert all(0 <= v < 8 for v in f)
            assert all(f[q] == q for q in range(m, 8))      # padding states fixed
    inp = gen.make_fsa_inputs("parity", L=10)
    assert float(inp.c[0, 0, 0, 1]) == 2.0 and float(inp.c[0, 0, 0, 0]) == 1.0
    assert math.isclose(float(inp.diag.sum()), 10 * 8)


def test_router_and_dictionary_generators():
    u1, w1 = gen.make_router_inputs(2, 5, 3, 4, 32, seed=9)
    u2, w2 = gen.make_router_inputs(2, 5, 3, 4, 32, seed=9)
    assert torch.equal(u1, u2) and torch.equal(w1, w2)
    assert u1.shape == (2, 5, 32) and w1.shape == (3, 4, 32)
    assert u1.dtype == torch.bfloat16 and w1.dtype == torch.bfloat16
    ui, wi = gen.make_router_inputs(1, 7, 2, 3, 16, integers=True)
    assert torch.equal(ui.float(), ui.float().round()) and float(ui.float().abs().max()) <= 3
    assert torch.equal(wi.float(), wi.float().round()) and float(wi.float().abs().max()) <= 2
    m = gen.make_dense_dict(2, 3, 8, seed=5)
    assert m.shape == (2, 3, 8, 8) and m.dtype == torch.float32
    assert torch.equal(m, gen.make_dense_dict(2, 3, 8, seed=5))
    assert gen.make_dense_dict(1, 2, 4, bf16=True).dtype == torch.bfloat16


def test_upstream_gradients():
    inp = gen.make_inputs("lm", B=1, H=2, L=20)
    gy, gxf = gen.make_grads(inp, seed=2)
    assert gy.shape == (1, 2, 20) and gy.dtype == torch.bfloat16
    assert gxf.shape == (1, 2, 64, 2) and gxf.dtype == torch.float32
    gy2, _ = gen.make_grads(inp, seed=2)
    assert torch.equal(gy, gy2)
    assert gen.make_grads(inp, seed=2, with_gx_final=False)[1] is None


def test_adversarial_scores_cover_every_rule():
    """The adversarial router scores hold ties, -0/+0 maxima, NaNs, +inf and
    all -inf rows, and every value is exact in bf16."""
    v = gen.make_adversarial_scores(2, 2, 500, 16, bf16=False, seed=3)
    assert v.shape == (2, 2, 500, 16) and v.dtype == torch.float32
    a = v.numpy()
    assert np.isnan(a).any(-1).sum() > 20
    assert (np.isnan(a).sum(-1) >= 2).sum() > 5          # several NaNs in one row
    assert np.isposinf(a).any(-1).sum() > 20
    assert np.isneginf(a).all(-1).sum() > 20             # whole rows of -inf
    negzero = (a == 0) & np.signbit(a)
    assert negzero.any(-1).sum() > 20
    finite = np.where(np.isfinite(a), a, 0)
    assert np.array_equal(finite, np.round(finite))      # small integers: exact ties
    vb = gen.make_adversarial_scores(2, 2, 500, 16, bf16=True, seed=3)
    assert vb.dtype == torch.bfloat16
    back = vb.float().numpy()
    same = (back == a) | (np.isnan(back) & np.isnan(a))
    num = ~np.isnan(a)
    assert same.all() and np.array_equal(np.signbit(back[num]), np.signbit(a[num]))
