"""The software exp2 of the kernels' compile-time variant GCA_SOFT_EXP
(csrc/exp2_poly, coefficients from csrc/fit_exp2.py): the committed header
holds the minimax fit, and its fp32 evaluation stays within 2^-10 relative
error of exp2 (numpy) over the arguments the softmax produces."""
import importlib.util
import os
import re

import numpy as np

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "geometric_context_attention_amd", "csrc")


def _fit():
    spec = importlib.util.spec_from_file_location("fit_exp2", os.path.join(CSRC, "fit_exp2.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _header_coeffs():
    text = open(os.path.join(CSRC, "gca_exp2_poly.h")).read()
    deg = int(re.search(r"GCA_EXP2_POLY_DEGREE (\d+)", text).group(1))
    return [float.fromhex(re.search(rf"GCA_EXP2_C{i} (\S+)f", text).group(1)) for i in range(deg + 1)]


def test_header_holds_the_minimax_fit():
    fit = _fit()
    c, E = fit.remez(3)
    assert E < 8e-5
    assert np.allclose(_header_coeffs(), np.float32(c), rtol=0, atol=1e-7)


def test_equioscillation():
    """A minimax relative fit of degree d touches its error bound with
    alternating signs at d + 2 points (Chebyshev's theorem)."""
    fit = _fit()
    c, E = fit.remez(3)
    f = np.linspace(0.0, 1.0, 400001)
    err = (np.polyval(c[::-1], f) - 2.0 ** f) / 2.0 ** f
    assert abs(np.max(np.abs(err)) - E) < 1e-3 * E
    peaks = f[np.abs(err) > 0.999 * E]
    signs = np.sign(err[np.abs(err) > 0.999 * E])
    groups = np.split(signs, np.nonzero(np.diff(peaks) > 1e-3)[0] + 1)
    assert len(groups) >= 5
    assert all(g[0] != h[0] for g, h in zip(groups, groups[1:]))


def test_fp32_evaluation_against_numpy_exp2():
    fit = _fit()
    c = np.array(_header_coeffs())
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-126.0, 16.0, 500_000), rng.uniform(-1.0, 1.0, 500_000),
                        np.arange(-126, 17, dtype=np.float64)]).astype(np.float32).astype(np.float64)
    got = fit.exp2_soft(x, c)
    rel = np.abs(got / np.exp2(x) - 1.0)
    assert rel.max() <= 2.0 ** -10
    assert rel.max() < 8e-5
    # exact powers of two stay exact up to the polynomial's value at 0
    n = np.arange(-100, 16, dtype=np.float64)
    assert np.allclose(fit.exp2_soft(n, c) / np.exp2(n), np.float32(c[0]), rtol=0, atol=1e-12)
