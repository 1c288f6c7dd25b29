"""Pins of the oracle's step after the read-out (CPU only).

"Paper Review: RWKV-7 Goose", The approach: the receptance also attends to the
current token without storing it in the state; the output is normalised per
head and gated.  The reading (current-token term s v with s = r . (u * k), a
per-head normalisation with affine and epsilon, an elementwise gate, three
orders) is pinned by a hand-worked fixture, closed forms of special cases and
invariants that a dropped term, a wrong variance divisor, a misplaced epsilon
or a swapped operand would break.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _toks(B=2, T=5, H=3, N=8, seed=0):
    sh = (B, T, H, N)
    return [_rand(sh, seed + i) for i in range(5)]   # y, r, k, v, g


def _heads(H=3, N=8, seed=50):
    return [_rand((H, N), seed + i) for i in range(3)]   # u, gamma, beta


def test_golden_fixture():
    with open(os.path.join(GOLDEN, "epilogue_n2.json")) as f:
        g = json.load(f)
    N = g["N"]
    tok = {x: np.array(g[x]).reshape(1, 1, 1, N) for x in ("y", "r", "k", "v", "g")}
    head = {x: np.array(g[x]).reshape(1, N) for x in ("u", "gamma", "beta")}
    for case in g["cases"]:
        out = oracle.epilogue(tok["y"], tok["r"], tok["k"], tok["v"], tok["g"], head["u"],
                              head["gamma"], head["beta"], eps=case["eps"], mode=case["mode"])
        np.testing.assert_allclose(out.ravel(), case["expected"], rtol=0, atol=g["tolerance_abs"])


def test_no_term_no_norm_no_gate_is_identity():
    """u = 0 (or absent), mode 0 and g = 1 leave y exactly as it is."""
    y, r, k, v, _ = _toks()
    np.testing.assert_array_equal(oracle.epilogue(y, r, k, v, mode=0), y)
    np.testing.assert_array_equal(
        oracle.epilogue(y, r, k, v, np.ones_like(y), np.zeros((3, 8)), mode=0), y)


@pytest.mark.parametrize("mode", [1, 2])
def test_normalised_head_has_zero_mean_unit_variance(mode):
    """Without affine, term (mode 1) and gate, and with eps = 0, every head of
    every token comes out with mean 0 and mean square deviation 1; in mode 2
    this holds with the term too, since it is added before normalising."""
    y, r, k, v, _ = _toks(N=16)
    u = _rand((3, 16), 9) if mode == 2 else None
    out = oracle.epilogue(y, r, k, v, u=u, eps=0.0, mode=mode)
    np.testing.assert_allclose(out.mean(axis=-1), 0.0, atol=1e-13)
    np.testing.assert_allclose((out ** 2).mean(axis=-1), 1.0, rtol=1e-13)


def test_two_channels_closed_form():
    """N = 2: (y - mean) is +-d with d = (y0 - y1)/2 and the variance is d^2,
    so the normalised head is +-d / sqrt(d^2 + eps): +-1 when eps = 0 (a sample
    variance, divisor N - 1, would give +-1/sqrt(2))."""
    y = _rand((1, 7, 2, 2), 3)
    zero = np.zeros_like(y)
    d = (y[..., 0] - y[..., 1]) / 2
    for eps in (0.0, 0.25, 4.0):
        out = oracle.epilogue(y, zero, zero, zero, eps=eps, mode=1)
        ref = d / np.sqrt(d * d + eps)
        np.testing.assert_allclose(out[..., 0], ref, rtol=1e-14)
        np.testing.assert_allclose(out[..., 1], -ref, rtol=1e-14)


def test_current_token_term_on_one_hot_receptance():
    """r = e_j: the term is u[h][j] k[j] v, added to y unchanged in mode 0."""
    B, T, H, N = 1, 3, 2, 8
    y, _, k, v, _ = _toks(B, T, H, N)
    u = _rand((H, N), 7)
    for j in (0, 5):
        r = np.zeros((B, T, H, N))
        r[..., j] = 1.0
        out = oracle.epilogue(y, r, k, v, u=u, mode=0)
        coef = u[None, None, :, j] * k[..., j]
        np.testing.assert_allclose(out - y, coef[..., None] * v, rtol=1e-13, atol=1e-15)


def test_term_coefficient_is_bilinear_in_r_and_k():
    """s = r . (u * k): swapping the roles of r and k leaves it unchanged, and
    scaling r by c and k by d scales it by c d (mode 0, g = 1, v = 1)."""
    y, r, k, _, _ = _toks()
    one = np.ones_like(y)
    u = _rand((3, 8), 11)
    base = oracle.epilogue(y, r, k, one, u=u, mode=0) - y
    np.testing.assert_allclose(oracle.epilogue(y, k, r, one, u=u, mode=0) - y, base, rtol=1e-12)
    np.testing.assert_allclose(oracle.epilogue(y, 2 * r, -3 * k, one, u=u, mode=0) - y, -6 * base,
                               rtol=1e-12, atol=1e-14)
    # one coefficient per token and head: the same in every channel
    np.testing.assert_allclose(base, base[..., :1] * one, rtol=1e-13)


@pytest.mark.parametrize("mode", [0, 1])
def test_linear_in_v(mode):
    """With y fixed (modes 0 and 1), the result is affine in v:
    out(v1 + c v2) = out(v1) + c (out(v2) - out(0))."""
    y, r, k, v1, g = _toks()
    v2 = _rand(y.shape, 20)
    u, gamma, beta = _heads()
    f = lambda v: oracle.epilogue(y, r, k, v, g, u, gamma, beta, mode=mode)
    zero = np.zeros_like(y)
    np.testing.assert_allclose(f(v1 + 2.5 * v2), f(v1) + 2.5 * (f(v2) - f(zero)), rtol=1e-12,
                               atol=1e-12)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_gate_scales_elementwise(mode):
    """out(g) = g * out(g = 1), channel by channel."""
    y, r, k, v, g = _toks()
    u, gamma, beta = _heads()
    ungated = oracle.epilogue(y, r, k, v, None, u, gamma, beta, mode=mode)
    np.testing.assert_allclose(oracle.epilogue(y, r, k, v, g, u, gamma, beta, mode=mode),
                               g * ungated, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("mode", [1, 2])
def test_affine_applies_after_normalising(mode):
    """Without term and gate, out(gamma, beta) = gamma * out(1, 0) + beta, per head."""
    y, r, k, v, _ = _toks()
    _, gamma, beta = _heads()
    plain = oracle.epilogue(y, r, k, v, mode=mode)
    np.testing.assert_allclose(oracle.epilogue(y, r, k, v, gamma=gamma, beta=beta, mode=mode),
                               gamma * plain + beta, rtol=1e-13, atol=1e-14)


def test_normalisation_ignores_scale_and_shift_of_y():
    """eps = 0: norm(c y + d) = norm(y) for c > 0 and a shift d common to the
    head's channels, and norm(-y) = -norm(y)."""
    y, r, k, v, _ = _toks()
    d = _rand(y.shape[:-1] + (1,), 30)
    base = oracle.epilogue(y, r, k, v, eps=0.0, mode=1)
    np.testing.assert_allclose(oracle.epilogue(3.5 * y + d, r, k, v, eps=0.0, mode=1), base,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.epilogue(-y, r, k, v, eps=0.0, mode=1), -base, rtol=1e-13,
                               atol=1e-13)


def test_heads_and_tokens_are_independent():
    """Each (token, head) sees only its own N channels and its head's u, gamma,
    beta: permuting tokens permutes the result, and a single head computed on
    its own matches the same head inside the batch."""
    y, r, k, v, g = _toks(B=2, T=6, H=3, N=8)
    u, gamma, beta = _heads()
    full = oracle.epilogue(y, r, k, v, g, u, gamma, beta, mode=1)
    perm = np.random.default_rng(1).permutation(6)
    np.testing.assert_array_equal(
        oracle.epilogue(y[:, perm], r[:, perm], k[:, perm], v[:, perm], g[:, perm], u, gamma, beta,
                        mode=1), full[:, perm])
    h = 2
    one = oracle.epilogue(*(x[:, :, h:h + 1] for x in (y, r, k, v, g)), u[h:h + 1],
                          gamma[h:h + 1], beta[h:h + 1], mode=1)
    np.testing.assert_array_equal(one[:, :, 0], full[:, :, h])


def test_constant_head_normalises_to_beta():
    """A head whose channels are all equal has zero deviation: with eps > 0 the
    normalised part is exactly beta (mode 1, no term, no gate)."""
    y = np.repeat(_rand((1, 4, 3, 1), 5), 8, axis=-1)
    zero = np.zeros_like(y)
    _, gamma, beta = _heads()
    out = oracle.epilogue(y, zero, zero, zero, gamma=gamma, beta=beta, eps=1e-5, mode=1)
    np.testing.assert_allclose(out, np.broadcast_to(beta, out.shape), rtol=0, atol=1e-12)
