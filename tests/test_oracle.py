"""Pins for the fp64 oracle: it is checked against what the definition and the
mathematics fix, never against itself or the HIP library.

Definition: GDPA page ("Generalized Dot-Product Attention (GDPA): kernel
optimisation for real recommendation-system training loads"), "Key summary" and
"Section details" (two products with an activation between them, no softmax
correction).  Taylor series: the same page's code figure of the ALU-only GELU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy import integrate

from oracle import gdpa_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(lq, lk, H=2, d=8, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    lq, lk = np.asarray(lq), np.asarray(lk)
    q_off = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    kv_off = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = rng.standard_normal((q_off[-1], H, d)) * scale
    k = rng.standard_normal((kv_off[-1], H, d)) * scale
    v = rng.standard_normal((kv_off[-1], H, d))
    do = rng.standard_normal((q_off[-1], H, d))
    return q, k, v, do, q_off, kv_off


# ---------------------------------------------------------------------------
# activations
# ---------------------------------------------------------------------------

def test_taylor_coefficients_match_page_and_closed_form():
    g = json.load(open(os.path.join(GOLDEN, "taylor_gelu_coefficients.json")))
    c1, c2, c4, c6 = R.TAYLOR6
    tol = 0.5 * 10.0 ** (-g["printed_digits"])
    assert abs(c1 - g["c1"]) <= tol
    assert abs(c2 - g["c2"]) <= tol
    assert abs(c4 - g["c4"]) <= tol
    assert abs(c6 - g["c6"]) <= tol


def test_taylor_series_is_erf_gelu_maclaurin():
    # The next term of x Phi(x)'s Maclaurin series is -x^8 / (336 sqrt(2 pi)); a
    # series of the tanh form would leave an x^4 residual instead.
    x = np.array([0.05, 0.1, 0.15, 0.2, 0.25])
    resid = (R.act_fwd(x, "gelu_taylor6") - R.act_fwd(x, "gelu")) / x ** 8
    expect = 1.0 / (336.0 * math.sqrt(2.0 * math.pi))
    np.testing.assert_allclose(resid, expect, rtol=2e-2)


def test_gelu_is_x_times_normal_cdf_by_quadrature():
    for x in (-3.0, -1.2, -0.3, 0.0, 0.4, 1.0, 2.5):
        half, _ = integrate.quad(lambda t: math.exp(-0.5 * t * t) / math.sqrt(2 * math.pi),
                                 0.0, x, epsabs=1e-14, epsrel=1e-13)
        assert abs(R.act_fwd(np.array(x), "gelu") - x * (0.5 + half)) < 1e-12


def test_activation_special_values_and_symmetry():
    x = np.linspace(-6, 6, 1001)
    assert R.act_fwd(np.array(0.0), "gelu") == 0.0
    assert R.act_fwd(np.array(0.0), "silu") == 0.0
    np.testing.assert_allclose(R.act_fwd(x, "gelu") - R.act_fwd(-x, "gelu"), x, atol=1e-14)
    np.testing.assert_allclose(R.act_fwd(x, "silu") - R.act_fwd(-x, "silu"), x, atol=1e-14)
    # Phi(1) from standard normal tables
    assert abs(R.act_fwd(np.array(1.0), "gelu") - 0.8413447460685429) < 1e-15
    # sigmoid(1) = e / (1 + e)
    assert abs(R.act_fwd(np.array(1.0), "silu") - math.e / (1 + math.e)) < 1e-15
    np.testing.assert_array_equal(R.act_fwd(x, "identity"), x)
    np.testing.assert_array_equal(R.act_fwd(x, "one"), np.ones_like(x))


@pytest.mark.parametrize("act", ["gelu", "silu", "gelu_taylor6", "identity", "one"])
def test_activation_derivative_matches_finite_differences(act):
    x = np.linspace(-5, 5, 2001)
    h = 1e-5
    fd = (R.act_fwd(x + h, act) - R.act_fwd(x - h, act)) / (2 * h)
    np.testing.assert_allclose(R.act_grad(x, act), fd, atol=1e-8, rtol=1e-8)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["gelu", "silu", "gelu_taylor6", "identity", "one"])
@pytest.mark.parametrize("window", [0, 1, 3])
def test_forward_equals_scalar_loops(act, window):
    lq = [5, 0, 7, 1, 4]
    lk = lq if window else [6, 3, 0, 2, 9]
    q, k, v, _, qo, ko = rand_case(lq, lk, H=2, d=4, seed=1)
    ref = R.gdpa_fwd_scalar(q, k, v, qo, ko, act, window)
    got = R.gdpa_fwd(q, k, v, qo, ko, act, window)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_windowed_forward_crossing_row_groups_equals_scalar():
    lq = [600, 530]
    q, k, v, _, qo, ko = rand_case(lq, lq, H=1, d=2, seed=2)
    ref = R.gdpa_fwd_scalar(q, k, v, qo, ko, "gelu", 5)
    got = R.gdpa_fwd(q, k, v, qo, ko, "gelu", 5)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _padded_dense_torch(q, k, v, qo, ko, act, window):
    """Pad every sample to the batch maxima and run one batched torch fp64
    computation with a dense validity mask."""
    B = len(qo) - 1
    H, d = q.shape[1], q.shape[2]
    lq, lk = np.diff(qo), np.diff(ko)
    mq, mk = int(lq.max()), int(lk.max())
    Qp = torch.zeros(B, H, mq, d, dtype=torch.float64)
    Kp = torch.zeros(B, H, mk, d, dtype=torch.float64)
    Vp = torch.zeros(B, H, mk, d, dtype=torch.float64)
    M = torch.zeros(B, 1, mq, mk, dtype=torch.float64)
    for b in range(B):
        Qp[b, :, :lq[b]] = torch.from_numpy(q[qo[b]:qo[b + 1]]).permute(1, 0, 2)
        Kp[b, :, :lk[b]] = torch.from_numpy(k[ko[b]:ko[b + 1]]).permute(1, 0, 2)
        Vp[b, :, :lk[b]] = torch.from_numpy(v[ko[b]:ko[b + 1]]).permute(1, 0, 2)
        i = torch.arange(mq)[:, None]
        j = torch.arange(mk)[None, :]
        m = (i < lq[b]) & (j < lk[b])
        if window:
            m &= (i - j).abs() < window
        M[b, 0] = m.double()
    S = torch.matmul(Qp, Kp.transpose(-1, -2).contiguous()) / d ** 0.5
    P = {"gelu": torch.nn.functional.gelu, "silu": torch.nn.functional.silu}[act](S) * M
    Op = torch.matmul(P, Vp)
    out = np.zeros_like(q)
    for b in range(B):
        out[qo[b]:qo[b + 1]] = Op[b, :, :lq[b]].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("act", ["gelu", "silu"])
@pytest.mark.parametrize("window", [0, 4])
def test_jagged_equals_padded_dense_library(act, window):
    lq = [17, 3, 0, 40, 9, 1]
    lk = lq if window else [5, 33, 8, 0, 12, 1]
    q, k, v, _, qo, ko = rand_case(lq, lk, H=3, d=16, seed=3)
    np.testing.assert_allclose(R.gdpa_fwd(q, k, v, qo, ko, act, window),
                               _padded_dense_torch(q, k, v, qo, ko, act, window),
                               rtol=1e-12, atol=1e-12)


def test_sample_permutation_invariance():
    lq = [7, 12, 0, 3, 20]
    lk = [9, 2, 4, 0, 15]
    q, k, v, do, qo, ko = rand_case(lq, lk, H=2, d=8, seed=4)
    o = R.gdpa_fwd(q, k, v, qo, ko, "gelu")
    dq, dk, dv = R.gdpa_bwd(q, k, v, do, qo, ko, "gelu")
    perm = [3, 0, 4, 2, 1]
    qs = [slice(qo[b], qo[b + 1]) for b in perm]
    ks = [slice(ko[b], ko[b + 1]) for b in perm]
    cat = lambda a, sl: np.concatenate([a[s] for s in sl])
    qo2 = np.concatenate([[0], np.cumsum([lq[b] for b in perm])])
    ko2 = np.concatenate([[0], np.cumsum([lk[b] for b in perm])])
    o2 = R.gdpa_fwd(cat(q, qs), cat(k, ks), cat(v, ks), qo2, ko2, "gelu")
    np.testing.assert_allclose(o2, cat(o, qs), rtol=0, atol=0)
    g2 = R.gdpa_bwd(cat(q, qs), cat(k, ks), cat(v, ks), cat(do, qs), qo2, ko2, "gelu")
    np.testing.assert_allclose(g2[0], cat(dq, qs), rtol=0, atol=0)
    np.testing.assert_allclose(g2[1], cat(dk, ks), rtol=0, atol=0)
    np.testing.assert_allclose(g2[2], cat(dv, ks), rtol=0, atol=0)


def test_empty_samples():
    lq = [0, 4, 3, 0]
    lk = [5, 0, 2, 0]
    q, k, v, do, qo, ko = rand_case(lq, lk, H=2, d=4, seed=5)
    o = R.gdpa_fwd(q, k, v, qo, ko, "gelu")
    assert o.shape == (7, 2, 4)
    assert np.all(o[0:4] == 0)          # sample 1 has no keys
    assert np.any(o[4:7] != 0)
    dq, dk, dv = R.gdpa_bwd(q, k, v, do, qo, ko, "gelu")
    assert np.all(dk[0:5] == 0) and np.all(dv[0:5] == 0)   # sample 0 has no queries
    assert np.all(dq[0:4] == 0)
    # an all-empty batch gives empty outputs
    z = np.zeros((0, 2, 4))
    assert R.gdpa_fwd(z, z, z, [0, 0, 0], [0, 0, 0], "silu").shape == (0, 2, 4)


def test_identity_activation_is_associative():
    lq = [6, 11, 1]
    lk = [9, 4, 13]
    q, k, v, _, qo, ko = rand_case(lq, lk, H=2, d=8, seed=6)
    o = R.gdpa_fwd(q, k, v, qo, ko, "identity")
    for b in range(3):
        for h in range(2):
            Q = q[qo[b]:qo[b + 1], h]
            K = k[ko[b]:ko[b + 1], h]
            V = v[ko[b]:ko[b + 1], h]
            np.testing.assert_allclose(o[qo[b]:qo[b + 1], h], Q @ (K.T @ V) / math.sqrt(8),
                                       rtol=1e-12, atol=1e-12)


def test_wide_window_equals_no_window():
    lq = [9, 14, 3]
    q, k, v, do, qo, ko = rand_case(lq, lq, H=2, d=4, seed=7)
    np.testing.assert_array_equal(R.gdpa_fwd(q, k, v, qo, ko, "silu", 14),
                                  R.gdpa_fwd(q, k, v, qo, ko, "silu", 0))


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _loss(q, k, v, do, qo, ko, act, window):
    return float(np.sum(R.gdpa_fwd(q, k, v, qo, ko, act, window) * do))


@pytest.mark.parametrize("act", ["gelu", "silu", "gelu_taylor6", "identity"])
@pytest.mark.parametrize("window", [0, 2])
def test_backward_matches_central_finite_differences(act, window):
    lq = [3, 0, 4]
    lk = lq if window else [4, 2, 3]
    q, k, v, do, qo, ko = rand_case(lq, lk, H=1, d=3, seed=8)
    g = R.gdpa_bwd(q, k, v, do, qo, ko, act, window)
    h = 1e-6
    for which, x, gx in ((0, q, g[0]), (1, k, g[1]), (2, v, g[2])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            lp = _loss(*args, do, qo, ko, act, window)
            args[which][idx] -= 2 * h
            lm = _loss(*args, do, qo, ko, act, window)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(gx, fd, atol=1e-7, rtol=1e-6)


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_backward_matches_torch_autograd_dense(act):
    lq = [8, 5, 13]
    lk = [11, 7, 2]
    q, k, v, do, qo, ko = rand_case(lq, lk, H=2, d=8, seed=9)
    dq, dk, dv = R.gdpa_bwd(q, k, v, do, qo, ko, act)
    f = {"gelu": torch.nn.functional.gelu, "silu": torch.nn.functional.silu}[act]
    for b in range(3):
        Q = torch.tensor(q[qo[b]:qo[b + 1]], requires_grad=True)
        K = torch.tensor(k[ko[b]:ko[b + 1]], requires_grad=True)
        V = torch.tensor(v[ko[b]:ko[b + 1]], requires_grad=True)
        dO = torch.tensor(do[qo[b]:qo[b + 1]])
        S = torch.einsum("ihe,jhe->hij", Q, K) / 8 ** 0.5
        O = torch.einsum("hij,jhe->ihe", f(S), V)
        (O * dO).sum().backward()
        np.testing.assert_allclose(dq[qo[b]:qo[b + 1]], Q.grad.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dk[ko[b]:ko[b + 1]], K.grad.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dv[ko[b]:ko[b + 1]], V.grad.numpy(), rtol=1e-11, atol=1e-12)


# Windowed samples longer than one group of query rows (the oracle evaluates
# them in groups of 512 queries with the keys their windows reach, and adds the
# groups' dK and dV contributions): checked against torch fp64 autograd on the
# whole per-sample score matrix with a banded validity mask (no groups).
ROW_GROUP_LENGTHS = [600, 1100, 0, 513, 7]


def _banded_autograd(q, k, v, do, qo, ko, window, f=None):
    """Per-sample (dQ, dK, dV) of sum(O * dO) through torch autograd, fp64, on the
    dense scores of each sample with the mask |i - j| < window; f is the
    activation, or None for softmax attention (scaled_dot_product_attention)."""
    d = q.shape[2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(qo) - 1):
        qs, qe, ks, ke = qo[b], qo[b + 1], ko[b], ko[b + 1]
        if qe == qs or ke == ks:
            continue
        t = lambda x: torch.tensor(x.transpose(1, 0, 2), requires_grad=True)   # [H, L, d]
        Q, K, V = t(q[qs:qe]), t(k[ks:ke]), t(v[ks:ke])
        i = torch.arange(qe - qs)[:, None]
        j = torch.arange(ke - ks)[None, :]
        m = (i - j).abs() < window
        if f is None:
            O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=m[None])
        else:
            S = torch.matmul(Q, K.transpose(-1, -2).contiguous()) / d ** 0.5
            O = torch.matmul(f(S) * m.double(), V)
        (O * torch.tensor(do[qs:qe].transpose(1, 0, 2))).sum().backward()
        dq[qs:qe] = Q.grad.numpy().transpose(1, 0, 2)
        dk[ks:ke] = K.grad.numpy().transpose(1, 0, 2)
        dv[ks:ke] = V.grad.numpy().transpose(1, 0, 2)
    return dq, dk, dv


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_windowed_backward_crossing_row_groups_equals_torch_autograd(act):
    q, k, v, do, qo, ko = rand_case(ROW_GROUP_LENGTHS, ROW_GROUP_LENGTHS, H=2, d=2, seed=21)
    got = R.gdpa_bwd(q, k, v, do, qo, ko, act, 5)
    f = {"gelu": torch.nn.functional.gelu, "silu": torch.nn.functional.silu}[act]
    want = _banded_autograd(q, k, v, do, qo, ko, 5, f)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-11, atol=1e-12)


def test_jfa_windowed_backward_crossing_row_groups_equals_torch_autograd():
    q, k, v, do, qo, ko = rand_case(ROW_GROUP_LENGTHS, ROW_GROUP_LENGTHS, H=2, d=2, seed=22)
    got = R.jfa_bwd(q, k, v, do, qo, ko, 5)
    want = _banded_autograd(q, k, v, do, qo, ko, 5, None)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-12)


def test_useful_pairs_counts_the_valid_set():
    for lq, lk, w in (([5, 0, 7], [3, 4, 7], 0), ([9, 1, 300], [9, 1, 300], 4)):
        brute = 0
        for a, c in zip(lq, lk):
            brute += int(R.valid_mask(np.arange(a), np.arange(c), a, c, w).sum())
        assert R.useful_pairs(lq, lk, w) == brute


# ---------------------------------------------------------------------------
# the pins catch planted mistakes (mutations applied to copies, on the CPU)
# ---------------------------------------------------------------------------

def test_pins_catch_a_wrong_gelu_derivative(monkeypatch):
    good = R.act_grad

    def bad(x, act):   # drops the x phi(x) term of GELU'
        if act == "gelu":
            return 0.5 * (1.0 + R.erf(np.asarray(x) * R._INV_SQRT2))
        return good(x, act)

    monkeypatch.setattr(R, "act_grad", bad)
    with pytest.raises(AssertionError):
        test_backward_matches_central_finite_differences("gelu", 0)


def test_pins_catch_an_inclusive_window(monkeypatch):
    good = R.valid_mask

    def bad(i, j, lq, lk, window):   # |i - j| <= w instead of < w
        return good(i, j, lq, lk, window + 1 if window else 0)

    monkeypatch.setattr(R, "valid_mask", bad)
    with pytest.raises(AssertionError):
        test_forward_equals_scalar_loops("gelu", 3)


def _mutated(fn, old, new):
    """A copy of oracle function `fn` with the source text `old` replaced by `new`,
    compiled in a copy of the oracle module's namespace."""
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) == 1, old
    ns = dict(vars(R))
    exec(compile(src.replace(old, new), R.__file__, "exec"), ns)
    return ns[fn.__name__]


@pytest.mark.parametrize("target", ["dk[ks + j0:ks + j1] +=", "dv[ks + j0:ks + j1] +="])
def test_pins_catch_row_group_gradients_overwritten(monkeypatch, target):
    """A windowed backward that stores each group's dK or dV contribution instead of
    adding it (key rows near a group boundary receive two groups' terms) fails the
    row-group pin, for GDPA and for JFA.  (Query rows belong to one group each.)"""
    bad = target.replace("+=", "=")
    monkeypatch.setattr(R, "gdpa_bwd", _mutated(R.gdpa_bwd, target, bad))
    with pytest.raises(AssertionError):
        test_windowed_backward_crossing_row_groups_equals_torch_autograd("gelu")
    monkeypatch.setattr(R, "jfa_bwd", _mutated(R.jfa_bwd, target, bad))
    with pytest.raises(AssertionError):
        test_jfa_windowed_backward_crossing_row_groups_equals_torch_autograd()


def test_pins_catch_a_missing_scale(monkeypatch):
    monkeypatch.setattr(R.math, "sqrt", lambda x: 1.0 if x in (4, 16) else math.pow(x, 0.5))
    with pytest.raises(AssertionError):
        test_jagged_equals_padded_dense_library("gelu", 0)


# ---------------------------------------------------------------------------
# pFFN as GDPA (shared weight rows for every query row)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_pffn_equals_per_sample_gdpa_with_replicated_weights(act):
    """Reading of the unified-modules diagram: every query row of every sample uses
    the same weight rows.  The one-sample form must equal jagged GDPA in which each
    sample gets its own copy of the weights, and the weight gradients must be the
    sums of the per-sample key/value gradients."""
    rng = np.random.default_rng(7)
    lq, M, H, d = [5, 0, 17, 9], 6, 2, 8
    tq = sum(lq)
    q = rng.standard_normal((tq, H, d))
    wk = rng.standard_normal((M, H, d))
    wv = rng.standard_normal((M, H, d))
    do = rng.standard_normal((tq, H, d))
    B = len(lq)
    q_off = np.concatenate([[0], np.cumsum(lq)])
    kv_off = np.arange(B + 1) * M
    kr, vr = np.concatenate([wk] * B), np.concatenate([wv] * B)
    o = R.pffn_fwd(q, wk, wv, act)
    np.testing.assert_allclose(o, R.gdpa_fwd(q, kr, vr, q_off, kv_off, act), rtol=1e-12, atol=1e-12)
    dq, dwk, dwv = R.pffn_bwd(q, wk, wv, do, act)
    gq, gk, gv = R.gdpa_bwd(q, kr, vr, do, q_off, kv_off, act)
    np.testing.assert_allclose(dq, gq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dwk, gk.reshape(B, M, H, d).sum(0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dwv, gv.reshape(B, M, H, d).sum(0), rtol=1e-12, atol=1e-12)


def test_pffn_identity_is_two_matrix_products():
    """With act = identity, pFFN is (Q W_K^T / sqrt(d)) W_V per head: two plain
    matrix products by a library routine (numpy matmul), and its weight gradient
    dW_V = P^T dO."""
    rng = np.random.default_rng(8)
    tq, M, H, d = 23, 7, 3, 16
    q, wk, wv, do = (rng.standard_normal(s) for s in ((tq, H, d), (M, H, d), (M, H, d), (tq, H, d)))
    o = R.pffn_fwd(q, wk, wv, "identity")
    _, _, dwv = R.pffn_bwd(q, wk, wv, do, "identity")
    for h in range(H):
        p = q[:, h] @ wk[:, h].T / np.sqrt(d)
        np.testing.assert_allclose(o[:, h], p @ wv[:, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dwv[:, h], p.T @ do[:, h], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# JFA: softmax attention on the jagged pairs
# ---------------------------------------------------------------------------

JFA_CASES = [
    ([5, 0, 17, 9, 33], [3, 4, 21, 0, 40], 0),
    ([12, 1, 30], [12, 1, 30], 4),
]


@pytest.mark.parametrize("lq,lk,window", JFA_CASES)
def test_jfa_equals_torch_sdpa_per_sample(lq, lk, window):
    """The oracle's jagged softmax attention equals the library routine
    (torch scaled_dot_product_attention, fp64, dense per sample with a boolean
    mask of the valid pairs); rows without keys give O = 0 and LSE = -inf; LSE is
    scipy's logsumexp of the masked scores."""
    import torch
    from scipy.special import logsumexp
    rng = np.random.default_rng(11)
    H, d = 2, 8
    q_off = np.concatenate([[0], np.cumsum(lq)])
    kv_off = np.concatenate([[0], np.cumsum(lk)])
    q, do = rng.standard_normal((q_off[-1], H, d)), rng.standard_normal((q_off[-1], H, d))
    k, v = rng.standard_normal((kv_off[-1], H, d)), rng.standard_normal((kv_off[-1], H, d))
    o, lse = R.jfa_fwd(q, k, v, q_off, kv_off, window)
    for b in range(len(lq)):
        qs, qe, ks, ke = q_off[b], q_off[b + 1], kv_off[b], kv_off[b + 1]
        if lq[b] == 0:
            continue
        if lk[b] == 0:
            assert np.all(o[qs:qe] == 0) and np.all(np.isneginf(lse[:, qs:qe]))
            continue
        m = R.valid_mask(np.arange(lq[b]), np.arange(lk[b]), lq[b], lk[b], window)
        t = lambda x: torch.tensor(x.transpose(1, 0, 2))
        ref = torch.nn.functional.scaled_dot_product_attention(t(q[qs:qe]), t(k[ks:ke]), t(v[ks:ke]),
                                                               attn_mask=torch.tensor(m)[None])
        np.testing.assert_allclose(o[qs:qe], ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)
        s = np.einsum("ihe,jhe->hij", q[qs:qe], k[ks:ke]) / np.sqrt(d)
        np.testing.assert_allclose(lse[:, qs:qe], logsumexp(np.where(m, s, -np.inf), axis=2), rtol=1e-12)


@pytest.mark.parametrize("lq,lk,window", JFA_CASES)
def test_jfa_backward_equals_torch_autograd(lq, lk, window):
    """Gradients of sum(O * dO) against torch autograd through fp64
    scaled_dot_product_attention, sample by sample."""
    import torch
    rng = np.random.default_rng(12)
    H, d = 2, 8
    q_off = np.concatenate([[0], np.cumsum(lq)])
    kv_off = np.concatenate([[0], np.cumsum(lk)])
    q, do = rng.standard_normal((q_off[-1], H, d)), rng.standard_normal((q_off[-1], H, d))
    k, v = rng.standard_normal((kv_off[-1], H, d)), rng.standard_normal((kv_off[-1], H, d))
    dq, dk, dv = R.jfa_bwd(q, k, v, do, q_off, kv_off, window)
    for b in range(len(lq)):
        qs, qe, ks, ke = q_off[b], q_off[b + 1], kv_off[b], kv_off[b + 1]
        if lq[b] == 0 or lk[b] == 0:
            assert np.all(dq[qs:qe] == 0) and np.all(dk[ks:ke] == 0) and np.all(dv[ks:ke] == 0)
            continue
        m = R.valid_mask(np.arange(lq[b]), np.arange(lk[b]), lq[b], lk[b], window)
        t = lambda x: torch.tensor(x.transpose(1, 0, 2), requires_grad=True)
        tq, tk, tv = t(q[qs:qe]), t(k[ks:ke]), t(v[ks:ke])
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(m)[None])
        (ref * torch.tensor(do[qs:qe].transpose(1, 0, 2))).sum().backward()
        for got, want in ((dq[qs:qe], tq.grad), (dk[ks:ke], tk.grad), (dv[ks:ke], tv.grad)):
            np.testing.assert_allclose(got, want.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# RMSNorm prologue (reading: per (token, head) RMSNorm over d, no gain, eps 1e-6,
# on the tensors named, right before GDPA; GDPA page, chart of tanh GELU against
# the 6th-order series)
# ---------------------------------------------------------------------------

def raw_case(lq, lk, H=2, d=8, seed=0):
    """Raw (unnormalised) inputs whose rows differ in scale by up to ~30x."""
    q, k, v, do, qo, ko = rand_case(lq, lk, H=H, d=d, seed=seed)
    rng = np.random.default_rng(seed + 100)
    q, k, v = (x * np.exp(rng.normal(0.0, 1.0, x.shape[:2] + (1,))) for x in (q, k, v))
    return q, k, v, do, qo, ko


def test_rms_norm_equals_torch_rms_norm():
    x = raw_case([7], [5], H=3, d=16, seed=1)[0]
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (16,), eps=1e-6).numpy()
    np.testing.assert_allclose(R.rms_norm(x), ref, rtol=1e-13, atol=1e-14)


def test_rms_norm_bwd_matches_central_finite_differences():
    x = raw_case([3], [2], H=2, d=6, seed=2)[0]
    dy = np.random.default_rng(3).standard_normal(x.shape)
    g = R.rms_norm_bwd(x, dy)
    fd = np.zeros_like(x)
    h = 1e-6
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = ((R.rms_norm(xp) * dy).sum() - (R.rms_norm(xm) * dy).sum()) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("norm", ["qkv", "kv", "qk", ""])
@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_norm_gdpa_equals_torch_autograd(norm, act):
    """Forward and raw-input gradients against torch's rms_norm and autograd (fp64)."""
    lq, lk = [6, 0, 9, 4], [5, 3, 7, 0]
    q, k, v, do, qo, ko = raw_case(lq, lk, H=2, d=8, seed=4)
    o = R.norm_gdpa_fwd(q, k, v, qo, ko, act, 0, norm)
    dq, dk, dv = R.norm_gdpa_bwd(q, k, v, do, qo, ko, act, 0, norm)
    f = {"gelu": torch.nn.functional.gelu, "silu": torch.nn.functional.silu}[act]
    nrm = lambda t, c: torch.nn.functional.rms_norm(t, (8,), eps=1e-6) if c in norm else t
    for b in range(len(lq)):
        Q = torch.tensor(q[qo[b]:qo[b + 1]], requires_grad=True)
        K = torch.tensor(k[ko[b]:ko[b + 1]], requires_grad=True)
        V = torch.tensor(v[ko[b]:ko[b + 1]], requires_grad=True)
        S = torch.einsum("ihe,jhe->hij", nrm(Q, "q"), nrm(K, "k")) / 8 ** 0.5
        O = torch.einsum("hij,jhe->ihe", f(S), nrm(V, "v"))
        (O * torch.tensor(do[qo[b]:qo[b + 1]])).sum().backward()
        np.testing.assert_allclose(o[qo[b]:qo[b + 1]], O.detach().numpy(), rtol=1e-11, atol=1e-12)
        for got, t in ((dq[qo[b]:qo[b + 1]], Q), (dk[ko[b]:ko[b + 1]], K), (dv[ko[b]:ko[b + 1]], V)):
            ref = t.grad.numpy() if t.grad is not None else np.zeros(t.shape)
            np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_norm_gdpa_is_scale_invariant_and_gradients_orthogonal():
    """Rescaling a normalised input's rows leaves O unchanged, and its raw gradient is
    orthogonal to the row (both exactly so as eps -> 0; here to eps's order)."""
    lq, lk = [9, 4], [6, 11]
    q, k, v, do, qo, ko = raw_case(lq, lk, H=2, d=8, seed=5)
    o = R.norm_gdpa_fwd(q, k, v, qo, ko, "gelu", 0, "qkv")
    c = np.exp(np.random.default_rng(6).normal(0.0, 1.0, q.shape[:2] + (1,)))
    # eps shifts r by a relative eps / (2 mean(x^2)) at most, on either side
    ms = min(np.mean(q * q, -1).min(), np.mean((q * c) ** 2, -1).min())
    tol = 10 * R.RMS_EPS / ms * np.abs(o).max()
    assert np.abs(R.norm_gdpa_fwd(q * c, k, v, qo, ko, "gelu", 0, "qkv") - o).max() <= tol
    for x, g in zip((q, k, v), R.norm_gdpa_bwd(q, k, v, do, qo, ko, "gelu", 0, "qkv")):
        dots = np.abs((x * g).sum(-1))
        assert dots.max() <= 1e-4 * (np.abs(x) * np.abs(g)).sum(-1).max()


def test_norm_gdpa_without_norm_is_gdpa():
    q, k, v, do, qo, ko = raw_case([5, 3], [4, 6], H=2, d=8, seed=7)
    np.testing.assert_array_equal(R.norm_gdpa_fwd(q, k, v, qo, ko, "silu", 0, ""),
                                  R.gdpa_fwd(q, k, v, qo, ko, "silu", 0))


def test_pins_catch_a_norm_gradient_without_the_projection(monkeypatch):
    """A plausible mistake, dx = r dx^ (dropping the term through r), fails the autograd pin."""
    monkeypatch.setattr(R, "rms_norm_bwd", lambda x, dy, eps=1e-6: dy / np.sqrt(
        np.mean(np.asarray(x) ** 2, axis=-1, keepdims=True) + eps))
    with pytest.raises(AssertionError):
        test_norm_gdpa_equals_torch_autograd("qkv", "gelu")
