"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of ``oracle/pdssm_oracle.c`` with one plausible error
(a transposed operand, a wrong sign, a dropped term, a wrong index or
tie-break), compiled with gcc into a temporary directory and run through the
same pins as the real oracle.  This shows the pins would catch such a mistake
in the oracle itself.  CPU only.
"""
import os

import pytest

import oracle
from tests import oracle_pins as pins

MUTANTS = {
    # D P instead of P D: d indexed by the destination row.
    "diag_by_destination": ("const double dr = diag[(row + j) * ncomp];",
                            "const double dr = diag[(row + i) * ncomp];"),
    # Gather instead of scatter: x'[pi[j]] += d[j] * x[pi[j]].
    "gather_not_scatter": ("const double xr = x[2 * j], xi = x[2 * j + 1];",
                           "const double xr = x[2 * i], xi = x[2 * i + 1];"),
    # Conjugated readout.
    "conjugate_readout": ("acc += cr * x[2 * i] - ci * x[2 * i + 1];",
                          "acc += cr * x[2 * i] + ci * x[2 * i + 1];"),
    # Sign error in the complex product.
    "complex_mul_sign": ("xn[2 * i] += dr * xr - di * xi;", "xn[2 * i] += dr * xr + di * xi;"),
    # b dropped.
    "drop_b": ("xn[2 * i] += load_value(b, (row + i) * ncomp, bc_bf16);",
               "xn[2 * i] += 0.0 * load_value(b, (row + i) * ncomp, bc_bf16);"),
    # Last maximum wins instead of the first.
    "last_max_wins": ("return v > best_v;", "return v >= best_v;"),
    # NaN not treated as the maximum.
    "nan_not_max": ("if (isnan(v))\n        return 1;", "if (isnan(v))\n        return 0;"),
    # Router weights read transposed ([H,D,K] instead of [H,K,D]).
    "router_w_transposed": ("const uint16_t *wr = w + (h * K + k) * (int64_t)D;",
                            "const uint16_t *wr = w + h * K * (int64_t)D + k;"),
    # Router scores missing the last input feature.
    "router_drop_last": ("for (int32_t d = 0; d < D; ++d)\n                    acc +=",
                         "for (int32_t d = 0; d < D - 1; ++d)\n                    acc +="),
    # Dictionary hardmax taken along rows instead of down each column.
    "hardmax_row_wise": ("double v = load_value(m, base + (int64_t)r * N + col, is_bf16);",
                         "double v = load_value(m, base + (int64_t)col * N + r, is_bf16);"),
    # Dictionary hardmax whose first candidate is taken from the wrong row.
    "hardmax_first_row": ("double best_v = load_value(m, base + col, is_bf16);",
                          "double best_v = load_value(m, base + (int64_t)col * N, is_bf16);"),
    # Initial state ignored.
    "ignore_x0": ("if (x0) {\n            for", "if (0) {\n            for"),
    # Readout of the state before the update (y_t from x_{t-1}).
    "readout_before_update": ("double *tmp = x;\n            x = xn;\n            xn = tmp;\n",
                              ""),
    # Composition: factor taken at the original source instead of the path.
    "compose_wrong_index": ("const int64_t e = (step * N + p) * ncomp;",
                            "const int64_t e = (step * N + j) * ncomp;"),
    # Composition in the wrong order: the path is advanced before the step's
    # factor is read, so d is taken at the destination.
    "compose_order": ("                p = dict_idx[(h * K + k) * N + p];\n", ""),
    # bf16 decoded as the low half.
    "bf16_low_half": ("uint32_t w = (uint32_t)bits << 16;", "uint32_t w = (uint32_t)bits << 15;"),
    # Backward: the readout's adjoint without conjugating c.
    "bwd_c_not_conjugated": ("lam[2 * i + 1] += -g * ci;", "lam[2 * i + 1] += g * ci;"),
    # Backward: the adjoint step as a scatter-style index (lambda read at j).
    "bwd_gather_at_source": ("const double lr = lam[2 * pi[j]], li = lam[2 * pi[j] + 1];",
                             "const double lr = lam[2 * j], li = lam[2 * j + 1];"),
    # Backward: d not conjugated in the adjoint step.
    "bwd_d_not_conjugated": ("lnew[2 * j + 1] = dr * li - di * lr;", "lnew[2 * j + 1] = dr * li + di * lr;"),
    # Backward: gd from x_t instead of x_{t-1}.
    "bwd_gd_wrong_state": ("const double *xp = xs + (size_t)t * N * 2;         /* x_{t-1} */",
                           "const double *xp = xs + (size_t)(t + 1) * N * 2;         /* x_{t-1} */"),
    # Backward: gc without the conjugate of x.
    "bwd_gc_sign": ("gc_out[e + 1] = -g * xt[2 * i + 1];", "gc_out[e + 1] = g * xt[2 * i + 1];"),
    # Backward: the x_final gradient dropped.
    "bwd_drop_gxf": ("        if (gxf) {\n", "        if (0) {\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    if name == "readout_before_update":
        # Move the state swap after the readout loop.
        src = src.replace(old, new)
        anchor = "            y_out[step] = acc;\n"
        assert src.count(anchor) == 1
        src = src.replace(anchor, anchor + old)
    elif name == "compose_order":
        src = src.replace(old, new)
        anchor = "                const int64_t e = (step * N + p) * ncomp;\n"
        assert src.count(anchor) == 1
        src = src.replace(anchor, old + anchor)
    else:
        src = src.replace(old, new)
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.build(source=path, out=os.path.join(tmp_path, "mutant.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
