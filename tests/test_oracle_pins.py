"""Pins of the fp64 oracle to facts other than itself (CPU only).

Each test ties the oracle to something the RWKV-7 pages or plain mathematics
fix: closed forms of special cases, exact rational arithmetic, brute-force
matrix products, invariants, hand-worked fixtures and finite differences.
None of these compares the oracle with a retyped copy of its own loop.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from rwkv_wkv7_delta_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng


def _rand(shape, seed):
    return rng0(seed).standard_normal(shape)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# Closed forms of special cases ("Paper Review", Background on the delta rule)
# ---------------------------------------------------------------------------

def test_linear_attention_closed_form():
    """a = b = 0, w = 1: the state only accumulates (linear attention), so
    y_t = s0 r_t + sum_{s<=t} v_s (k_s . r_t) and S_T = s0 + sum_s v_s k_s^T."""
    B, T, H, N = 2, 9, 3, 7
    r, k, v = (_rand((B, T, H, N), s) for s in (1, 2, 3))
    s0 = _rand((B, H, N, N), 4)
    z = np.zeros((B, T, H, N))
    y, sT = oracle.forward(r, np.ones_like(r), k, v, z, z, s0)
    kr = np.einsum("bshj,bthj->bhst", k, r)          # k_s . r_t
    mask = np.tril(np.ones((T, T))).T                 # s <= t
    ref = np.einsum("bhst,st,bshi->bthi", kr, mask, v) + np.einsum("bhij,bthj->bthi", s0, r)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sT, s0 + np.einsum("bshi,bshj->bhij", v, k), rtol=0, atol=1e-12)


def test_decay_only_closed_form():
    """a = b = 0 (the RWKV-6-style vector decay, no removal):
    y_t[i] = sum_j s0[i,j] G_t[j] r_t[j] + sum_{s<=t} v_s[i] sum_j k_s[j] r_t[j] prod_{u=s+1..t} w_u[j]."""
    B, T, H, N = 1, 8, 2, 6
    r, k, v = (_rand((B, T, H, N), s) for s in (5, 6, 7))
    w = rng0(8).uniform(0.3, 1.0, (B, T, H, N))
    s0 = _rand((B, H, N, N), 9)
    z = np.zeros_like(r)
    y, sT = oracle.forward(r, w, k, v, z, z, s0)
    ref = np.zeros_like(y)
    for bb in range(B):
        for hh in range(H):
            for t in range(T):
                G = np.prod(w[bb, : t + 1, hh], axis=0)
                acc = s0[bb, hh] @ (G * r[bb, t, hh])
                for s in range(t + 1):
                    P = np.prod(w[bb, s + 1: t + 1, hh], axis=0)
                    acc = acc + v[bb, s, hh] * np.dot(k[bb, s, hh] * P, r[bb, t, hh])
                ref[bb, t, hh] = acc
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


def test_value_replacement_exact():
    """w = 1, alpha = 1, unit kappa, k = kappa: after the write S_t kappa_t = v_t
    (relaxed value replacement, Abstract; separate removal/replacement keys,
    Architecture).  Reading with r_t = kappa_t therefore returns v_t."""
    B, T, H, N = 2, 12, 2, 8
    kap = _unit(_rand((B, T, H, N), 10))
    v = _rand((B, T, H, N), 11)
    s0 = _rand((B, H, N, N), 12)
    y, _ = oracle.forward(kap, np.ones_like(kap), kap, v, -kap, kap, s0)
    np.testing.assert_allclose(y, v, rtol=0, atol=1e-13)


def test_value_replacement_general_key():
    """Same transition with an arbitrary write key k: S_t kappa_t = (k_t . kappa_t) v_t."""
    B, T, H, N = 1, 10, 3, 8
    kap = _unit(_rand((B, T, H, N), 13))
    k = _rand((B, T, H, N), 14)
    v = _rand((B, T, H, N), 15)
    y, _ = oracle.forward(kap, np.ones_like(kap), k, v, -kap, kap, _rand((B, H, N, N), 16))
    np.testing.assert_allclose(y, np.sum(k * kap, -1, keepdims=True) * v, rtol=0, atol=1e-12)


def test_deltanet_sgd_step():
    """DeltaNet's delta rule is one SGD step on 0.5 ||S kappa - v||^2 (Background):
    with w = 1, a = -kappa, b = k = beta kappa the recurrence must equal
    S <- S - beta (S kappa - v) kappa^T, computed here from the loss gradient."""
    B, T, H, N = 1, 15, 2, 6
    kap = _unit(_rand((B, T, H, N), 17))
    beta = rng0(18).uniform(0.1, 0.9, (B, T, H, 1))
    v = _rand((B, T, H, N), 19)
    r = _rand((B, T, H, N), 20)
    s0 = _rand((B, H, N, N), 21)
    y, sT = oracle.forward(r, np.ones_like(r), beta * kap, v, -kap, beta * kap, s0)
    for hh in range(H):
        S = s0[0, hh].copy()
        for t in range(T):
            kt, vt, bt = kap[0, t, hh], v[0, t, hh], beta[0, t, hh, 0]
            grad = np.outer(S @ kt - vt, kt)          # d/dS of 0.5||S k - v||^2
            S = S - bt * grad
            np.testing.assert_allclose(y[0, t, hh], S @ r[0, t, hh], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sT[0, hh], S, rtol=0, atol=1e-12)


def test_householder_swap_random_state():
    """alpha = 2, kappa = (e_i - e_j)/sqrt(2), w = 1, v = 0: diag(w) + a b^T is the
    Householder reflection exchanging key channels i and j (the 'copy'
    transition, Architecture; Householder-like transition, The approach)."""
    N = 9
    s0 = _rand((1, 1, N, N), 22)
    for (i, j) in [(0, 8), (3, 4), (7, 2)]:
        kap = np.zeros(N)
        kap[i], kap[j] = 2 ** -0.5, -(2 ** -0.5)
        sh = (1, 1, 1, N)
        a = (-kap).reshape(sh)
        b = (2 * kap).reshape(sh)
        zero = np.zeros(sh)
        _, sT = oracle.forward(zero, np.ones(sh), zero, zero, a, b, s0)
        ref = s0[0, 0].copy()
        ref[:, [i, j]] = ref[:, [j, i]]
        np.testing.assert_allclose(sT[0, 0], ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("name", ["value_replacement_n2.json", "householder_swap_n4.json"])
def test_golden_fixture(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    N = g["N"]
    sh = (1, 1, 1, N)
    args = [np.array(g[x], dtype=np.float64).reshape(sh) for x in ("r", "w", "k", "v", "a", "b")]
    s0 = np.array(g["s0"], dtype=np.float64).reshape(1, 1, N, N)
    y, sT = oracle.forward(*args, s0)
    np.testing.assert_allclose(sT[0, 0], np.array(g["expected_sT"]), rtol=0, atol=g["tolerance_abs"])
    np.testing.assert_allclose(y[0, 0, 0], np.array(g["expected_y"]), rtol=0, atol=g["tolerance_abs"])


# ---------------------------------------------------------------------------
# Exact rational arithmetic and brute-force products
# ---------------------------------------------------------------------------

def _dyadic(rng, shape, values):
    return rng.choice(np.array(values, dtype=np.float64), size=shape)


def test_dyadic_inputs_bit_exact_against_fractions():
    """Entries in {0, +-1/2, +-1}, w in {1/2, 3/4, 1}: every intermediate is a
    short dyadic rational, so fp64 must reproduce the exact rational result
    computed with fractions.Fraction from S <- S (diag(w) + a b^T) + v k^T."""
    rng = rng0(23)
    B, T, H, N = 1, 8, 3, 4
    vals = [0.0, 0.5, -0.5, 1.0, -1.0]
    r, k, v, a, b = (_dyadic(rng, (B, T, H, N), vals) for _ in range(5))
    w = _dyadic(rng, (B, T, H, N), [0.5, 0.75, 1.0])
    s0 = _dyadic(rng, (B, H, N, N), vals)
    y, sT = oracle.forward(r, w, k, v, a, b, s0)
    F = Fraction
    for hh in range(H):
        S = [[F(s0[0, hh, i, j]) for j in range(N)] for i in range(N)]
        for t in range(T):
            M = [[(F(w[0, t, hh, i]) if i == j else F(0)) + F(a[0, t, hh, i]) * F(b[0, t, hh, j])
                  for j in range(N)] for i in range(N)]
            S = [[sum(S[i][m] * M[m][j] for m in range(N)) + F(v[0, t, hh, i]) * F(k[0, t, hh, j])
                  for j in range(N)] for i in range(N)]
            yt = [sum(S[i][j] * F(r[0, t, hh, j]) for j in range(N)) for i in range(N)]
            for i in range(N):
                assert F(float(yt[i])) == yt[i], "exact value not representable; pick other data"
                assert y[0, t, hh, i] == float(yt[i])
        for i in range(N):
            for j in range(N):
                assert sT[0, hh, i, j] == float(S[i][j])


def _transitions(w, a, b):
    """M_t = diag(w_t) + a_t b_t^T for one head, as a [T, N, N] array."""
    return np.einsum("tj,jk->tjk", w, np.eye(w.shape[-1])) + np.einsum("tj,tk->tjk", a, b)


def test_matrix_product_form():
    """S_T = S_0 M_1...M_T + sum_s v_s k_s^T M_{s+1}...M_T and y_t = S_t r_t."""
    inp = synth.generate(1, 7, 2, 5, dtype="fp32", seed=24, random_s0=True)
    y, sT = oracle.forward(*inp.tensors(), inp.s0)
    for hh in range(2):
        r, w, k, v, a, b = (x[0, :, hh].astype(np.float64) for x in inp.tensors())
        M = _transitions(w, a, b)
        T = r.shape[0]
        for t in range(T):
            St = inp.s0[0, hh].astype(np.float64)
            for u in range(t + 1):
                St = St @ M[u]
            for s in range(t + 1):
                P = np.outer(v[s], k[s])
                for u in range(s + 1, t + 1):
                    P = P @ M[u]
                St = St + P
            np.testing.assert_allclose(y[0, t, hh], St @ r[t], rtol=0, atol=1e-13)
        np.testing.assert_allclose(sT[0, hh], St, rtol=0, atol=1e-13)


def test_identity_start_gives_transition_product():
    """S0 = I, v = 0 => S_T = M_1 M_2 ... M_T."""
    inp = synth.generate(1, 6, 1, 6, dtype="fp32", seed=25)
    r, w, k, v, a, b = (x.astype(np.float64) for x in inp.tensors())
    _, sT = oracle.forward(r, w, k, np.zeros_like(v), a, b, np.eye(6)[None, None])
    P = np.eye(6)
    for Mt in _transitions(w[0, :, 0], a[0, :, 0], b[0, :, 0]):
        P = P @ Mt
    np.testing.assert_allclose(sT[0, 0], P, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_linear_in_initial_state_and_value():
    inp = synth.generate(2, 11, 2, 8, dtype="fp32", seed=26, random_s0=True)
    r, w, k, v, a, b = inp.tensors()
    s0 = inp.s0
    v2, s02 = _rand(v.shape, 27), _rand(s0.shape, 28)
    al, be = 0.7, -1.3
    y1, S1 = oracle.forward(r, w, k, v, a, b, s0)
    y2, S2 = oracle.forward(r, w, k, v2, a, b, s02)
    y3, S3 = oracle.forward(r, w, k, al * v.astype(np.float64) + be * v2, a, b,
                            al * s0.astype(np.float64) + be * s02)
    np.testing.assert_allclose(y3, al * y1 + be * y2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S3, al * S1 + be * S2, rtol=0, atol=1e-12)


def test_linear_in_receptance():
    inp = synth.generate(1, 9, 2, 8, dtype="fp32", seed=29, random_s0=True)
    r, w, k, v, a, b = inp.tensors()
    r2 = _rand(r.shape, 30)
    y1, _ = oracle.forward(r, w, k, v, a, b, inp.s0)
    y2, _ = oracle.forward(r2, w, k, v, a, b, inp.s0)
    y3, _ = oracle.forward(2.0 * r.astype(np.float64) - 0.5 * r2, w, k, v, a, b, inp.s0)
    np.testing.assert_allclose(y3, 2.0 * y1 - 0.5 * y2, rtol=0, atol=1e-12)


def test_value_row_permutation_equivariance():
    """Rows of S (value channels) evolve independently: permuting the value
    channels of v and the rows of s0 permutes y and the rows of S_T."""
    inp = synth.generate(1, 10, 2, 8, dtype="fp32", seed=31, random_s0=True)
    r, w, k, v, a, b = inp.tensors()
    perm = rng0(32).permutation(8)
    y, sT = oracle.forward(r, w, k, v, a, b, inp.s0)
    yp, sTp = oracle.forward(r, w, k, v[..., perm], a, b, inp.s0[:, :, perm, :])
    np.testing.assert_array_equal(yp, y[..., perm])
    np.testing.assert_array_equal(sTp, sT[:, :, perm, :])


def test_heads_and_batches_independent():
    inp = synth.generate(2, 7, 3, 6, dtype="fp32", seed=33, random_s0=True)
    y, sT = oracle.forward(*inp.tensors(), inp.s0)
    pairs = [(1, 2), (0, 1)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    ys, sTs = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    for p, (bb, hh) in enumerate(pairs):
        np.testing.assert_array_equal(ys[p, :, 0], y[bb, :, hh])
        np.testing.assert_array_equal(sTs[p, 0], sT[bb, hh])


def test_decode_steps_equal_forward():
    """Constant memory per token (Abstract): T decode steps on a resident state
    reproduce the sequence forward."""
    inp = synth.generate(2, 13, 3, 8, dtype="bf16", seed=34, random_s0=True)
    y, sT = oracle.forward(*inp.tensors(), inp.s0)
    state = inp.s0.astype(np.float64)
    for t in range(13):
        yt, state = oracle.decode_step(*(x[:, t] for x in inp.tensors()), state)
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(state, sT)


def test_continuation_equals_full_sequence():
    inp = synth.generate(1, 20, 2, 8, dtype="fp32", seed=35, random_s0=True)
    y, sT = oracle.forward(*inp.tensors(), inp.s0)
    y1, s1 = oracle.forward(*(x[:, :7] for x in inp.tensors()), inp.s0)
    y2, s2 = oracle.forward(*(x[:, 7:] for x in inp.tensors()), s1)
    np.testing.assert_array_equal(np.concatenate([y1, y2], 1), y)
    np.testing.assert_array_equal(s2, sT)


@pytest.mark.parametrize("L", [1, 3, 16, 64])
def test_chunked_equals_sequential(L):
    """The parallel-in-time chunk form (training stays parallelisable, Abstract)
    is an exact rearrangement: fp64 agreement to rounding, incl. ragged tails."""
    inp = synth.generate(2, 70, 2, 16, dtype="bf16", seed=36, random_s0=True)
    y, sT = oracle.forward(*inp.tensors(), inp.s0)
    yc, sTc = oracle.forward(*inp.tensors(), inp.s0, chunk_len=L)
    assert np.abs(yc - y).max() <= 1e-13 * np.abs(y).max()
    assert np.abs(sTc - sT).max() <= 1e-13 * np.abs(sT).max()


# ---------------------------------------------------------------------------
# Stability ("eigenvalues in a stable range", The approach)
# ---------------------------------------------------------------------------

def test_transition_eigenvalues_in_stable_range():
    """Under the synthetic distribution (alpha in (0,1), unit kappa, w in (0,1])
    M_t = diag(w) - kappa (kappa*alpha)^T is similar to a symmetric matrix, so its
    eigenvalues are real and lie in [min w - sum alpha kappa^2, max w] c [-1, 1].
    M_t is read off the oracle as S_1 with S_0 = I and v = 0."""
    N = 16
    inp = synth.generate(1, 40, 1, N, dtype="fp32", seed=37)
    r, w, k, v, a, b = (x.astype(np.float64) for x in inp.tensors())
    for t in range(40):
        sl = (slice(None), slice(t, t + 1))
        _, M = oracle.forward(r[sl], w[sl], k[sl], np.zeros_like(v[sl]), a[sl], b[sl],
                              np.eye(N)[None, None])
        ev = np.linalg.eigvals(M[0, 0])
        assert np.abs(ev.imag).max() < 1e-10
        wt, at, bt = w[0, t, 0], a[0, t, 0], b[0, t, 0]
        lo = wt.min() + np.dot(at, bt)      # = min w - sum alpha kappa^2
        assert ev.real.min() >= lo - 1e-12 and ev.real.max() <= wt.max() + 1e-12
        assert -1 <= lo and wt.max() <= 1


def test_state_norm_nonincreasing_without_writes_scalar_rate():
    """With a uniform in-context rate alpha in [0,1] per token, w in (0,1] and no
    writes (v = 0), ||M_t||_2 <= 1, so ||S_t||_F never grows."""
    B, T, H, N = 1, 60, 2, 8
    kap = _unit(_rand((B, T, H, N), 38))
    al = rng0(39).uniform(0, 1, (B, T, H, 1))
    w = rng0(40).uniform(0.5, 1, (B, T, H, N))
    state = _rand((B, H, N, N), 41)
    zero = np.zeros((B, H, N))
    prev = np.linalg.norm(state, axis=(-2, -1))
    for t in range(T):
        _, state = oracle.decode_step(zero, w[:, t], zero, zero, -kap[:, t], (al * kap)[:, t], state)
        cur = np.linalg.norm(state, axis=(-2, -1))
        assert np.all(cur <= prev * (1 + 1e-12))
        prev = cur


def test_state_stays_bounded_long_run():
    """Long run under the synthetic distribution with writes: finite and O(1)."""
    inp = synth.generate(1, 3000, 2, 64, dtype="bf16", seed=42)
    _, sT = oracle.forward(*inp.tensors())
    nrm = np.linalg.norm(sT, axis=(-2, -1))
    assert np.all(np.isfinite(sT)) and nrm.max() < 1e3


# ---------------------------------------------------------------------------
# Gradients
# ---------------------------------------------------------------------------

def _loss(ins, s0, dy, dsT):
    y, sT = oracle.forward(*ins, s0)
    return float((y * dy).sum() + (sT * dsT).sum())


def test_backward_finite_differences_exhaustive():
    """Central differences (h = 1e-6) of L = <dy, y> + <dsT, S_T> for every input
    element on a tiny problem."""
    inp = synth.generate(1, 6, 1, 5, dtype="fp32", seed=43, random_s0=True, backward=True)
    ins = [x.astype(np.float64) for x in inp.tensors()]
    s0 = inp.s0.astype(np.float64)
    dy = inp.dy.astype(np.float64)
    dsT = _rand(s0.shape, 44)
    grads = oracle.backward(*ins, s0, dy, dsT)
    h = 1e-6
    for q, arr in enumerate(ins + [s0]):
        g = grads[q]
        scale = np.abs(g).max()
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(ins, s0, dy, dsT)
            arr[idx] = old - h
            lm = _loss(ins, s0, dy, dsT)
            arr[idx] = old
            assert abs((lp - lm) / (2 * h) - g[idx]) <= 1e-7 * scale, (q, idx)


def test_backward_directional_derivatives_config_shape():
    """Random-direction JVPs at N = 64 (the workload head size), T = 32."""
    inp = synth.generate(2, 32, 2, 64, dtype="bf16", seed=45, random_s0=True, backward=True)
    ins = [x.astype(np.float64) for x in inp.tensors()]
    s0 = inp.s0.astype(np.float64)
    dy = inp.dy.astype(np.float64)
    dsT = 0.1 * _rand(s0.shape, 46)
    grads = oracle.backward(*ins, s0, dy, dsT)
    h = 1e-5
    for q in range(7):
        d = _rand(grads[q].shape, 100 + q)
        plus = [x.copy() for x in ins] + [s0.copy()]
        minus = [x.copy() for x in ins] + [s0.copy()]
        plus[q] += h * d
        minus[q] -= h * d
        fd = (_loss(plus[:6], plus[6], dy, dsT) - _loss(minus[:6], minus[6], dy, dsT)) / (2 * h)
        an = float((grads[q] * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (q, fd, an)


def test_backward_linear_attention_closed_form():
    """a = b = 0, w = 1: dv_s = sum_{t>=s} (k_s . r_t) dy_t,
    dk_s = sum_{t>=s} (v_s . dy_t) r_t + dsT^T v_s, dr_t = s0^T dy_t + sum_{s<=t} (v_s . dy_t) k_s."""
    B, T, H, N = 1, 8, 2, 5
    r, k, v, dy = (_rand((B, T, H, N), s) for s in (47, 48, 49, 50))
    s0 = _rand((B, H, N, N), 51)
    dsT = _rand((B, H, N, N), 52)
    z = np.zeros_like(r)
    dr, dw, dk, dv, da, db, ds0 = oracle.backward(r, np.ones_like(r), k, v, z, z, s0, dy, dsT)
    up = np.triu(np.ones((T, T)))        # [s, t]: t >= s
    kr = np.einsum("bshj,bthj->bhst", k, r)
    vdy = np.einsum("bshi,bthi->bhst", v, dy)
    np.testing.assert_allclose(dv, np.einsum("bhst,st,bthi->bshi", kr, up, dy)
                               + np.einsum("bhij,bshj->bshi", dsT, k), atol=1e-12)
    np.testing.assert_allclose(dk, np.einsum("bhst,st,bthj->bshj", vdy, up, r)
                               + np.einsum("bhij,bshi->bshj", dsT, v), atol=1e-12)
    np.testing.assert_allclose(dr, np.einsum("bhst,st,bshj->bthj", vdy, up, k)
                               + np.einsum("bhij,bthi->bthj", s0, dy), atol=1e-12)
    np.testing.assert_allclose(ds0, dsT + np.einsum("bthi,bthj->bhij", dy, r), atol=1e-12)


def test_backward_decay_only_closed_form():
    """a = b = 0 with decay: every gradient of L = sum_t <dy_t, y_t> + <dsT, S_T>
    written out from y_t = s0 (G_t * r_t) + sum_{s<=t} v_s <k_s * P(s,t), r_t>
    and S_T = s0 diag(G_T) + sum_s v_s (k_s * P(s,T))^T, where P(s,t) = the
    product of w_u over s < u <= t and G_t = the product over u <= t.  dw_u
    collects, divided by w_u, every term whose product contains w_u."""
    B, T, H, N = 1, 7, 2, 5
    r, k, v, dy = (_rand((B, T, H, N), s) for s in (55, 56, 57, 58))
    w = rng0(59).uniform(0.3, 1.0, (B, T, H, N))
    s0 = _rand((B, H, N, N), 60)
    dsT = _rand((B, H, N, N), 61)
    z = np.zeros_like(r)
    dr, dw, dk, dv, da, db, ds0 = oracle.backward(r, w, k, v, z, z, s0, dy, dsT)
    for hh in range(H):
        R, W, K, V, DY = (x[0, :, hh] for x in (r, w, k, v, dy))
        S0, DS = s0[0, hh], dsT[0, hh]

        def P(s, t):                          # prod of w_u, s < u <= t
            return np.prod(W[s + 1: t + 1], axis=0)

        def G(t):                             # prod of w_u, u <= t
            return np.prod(W[: t + 1], axis=0)

        ref_dv = np.zeros((T, N)); ref_dk = np.zeros((T, N)); ref_dr = np.zeros((T, N))
        ref_dw = np.zeros((T, N)); ref_ds0 = DS * G(T - 1)[None, :]
        for t in range(T):
            ref_dr[t] = (DY[t] @ S0) * G(t)
            ref_ds0 += np.outer(DY[t], G(t) * R[t])
            for s in range(t + 1):
                vd = V[s] @ DY[t]
                ref_dv[s] += DY[t] * np.dot(K[s] * P(s, t), R[t])
                ref_dk[s] += vd * R[t] * P(s, t)
                ref_dr[t] += vd * K[s] * P(s, t)
        for s in range(T):
            ref_dv[s] += DS @ (K[s] * P(s, T - 1))
            ref_dk[s] += (V[s] @ DS) * P(s, T - 1)
        for u in range(T):
            acc = np.zeros(N)
            for t in range(u, T):
                acc += (DY[t] @ S0) * G(t) * R[t]
                for s in range(u):
                    acc += (V[s] @ DY[t]) * K[s] * R[t] * P(s, t)
            for s in range(u):
                acc += (V[s] @ DS) * K[s] * P(s, T - 1)
            acc += np.einsum("ij,ij->j", DS, S0) * G(T - 1)
            ref_dw[u] = acc / W[u]
        for got, ref in ((dv, ref_dv), (dk, ref_dk), (dr, ref_dr), (dw, ref_dw)):
            np.testing.assert_allclose(got[0, :, hh], ref, rtol=0, atol=1e-11)
        np.testing.assert_allclose(ds0[0, hh], ref_ds0, rtol=0, atol=1e-11)


@pytest.mark.parametrize("L", [1, 5, 16, 64])
def test_chunked_backward_equals_sequential(L):
    inp = synth.generate(2, 70, 2, 16, dtype="bf16", seed=53, random_s0=True, backward=True)
    dsT = 0.1 * _rand(inp.s0.shape, 54)
    g = oracle.backward(*inp.tensors(), inp.s0, inp.dy, dsT)
    gc = oracle.backward(*inp.tensors(), inp.s0, inp.dy, dsT, chunk_len=L)
    for p, q in zip(gc, g):
        assert np.abs(p - q).max() <= 1e-12 * np.abs(q).max()


def test_generator_recipe():
    """The synthetic inputs follow the stated distribution and rounding."""
    inp = synth.generate(2, 33, 3, 64, dtype="bf16", seed=0, random_s0=True, backward=True)
    for x in inp.tensors() + (inp.dy,):
        assert x.dtype == np.float32
        assert np.array_equal(synth.round_to_bf16(x), x)
    assert inp.w.min() > 0.54 and inp.w.max() <= 1.0
    kap = -inp.a.astype(np.float64)
    assert np.allclose(np.linalg.norm(kap, axis=-1), 1.0, atol=1e-2)
    alpha = inp.b / np.where(kap == 0, 1, kap)
    assert np.nanmin(alpha[np.abs(kap) > 0.05]) > -0.01
    again = synth.generate(2, 33, 3, 64, dtype="bf16", seed=0, random_s0=True, backward=True)
    assert np.array_equal(again.r, inp.r) and np.array_equal(again.dy, inp.dy)
