"""fp64 CPU oracle for jagged Generalized Dot-Product Attention (GDPA).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and imports nothing from it.

Sources (cited by page title and section; no page text is reproduced):
  GDPA page  - aitrends.kr/articles/26275, "Generalized Dot-Product Attention
               (GDPA): kernel optimisation for real recommendation-system
               training loads" (Korean: 범용 내적 어텐션(GDPA)).
               * "Key summary": softmax replaced by a general activation such as
                 GELU or SiLU.
               * "Section details", diagram "Self-attention, PMA and pFFN unified
                 as GDPA": every variant is two matrix products with an
                 activation between them.
               * "Section details", paragraph on removing the softmax correction
                 step: no running max, no row sum, no rescale.
               * "Section details", code figure "ALU-only 6th-order Taylor
                 GELU": the series c1 x + c2 x^2 + c4 x^4 + c6 x^6.
  GEM page   - techlist.io/tags/distributed-training, "GEM training: how Meta
               doubled the efficiency of an LLM-scale ads foundation model",
               section "why high GPU utilisation is hard": variable lengths, the
               three attention shapes, the short local window.

Definition computed here, per sample b and head h, over the valid set
V_b = {(i, j): 0 <= i < Lq_b, 0 <= j < Lk_b, window == 0 or |i - j| < window}:

    S_ij = sum_e Q_ie K_je / sqrt(d)          (1/sqrt(d) scale: reading, see below)
    P_ij = act(S_ij)
    O_i  = sum_{j: (i,j) in V_b} P_ij V_j      (no normalisation)

and for the loss l = sum(O * dO):

    dP_ij = sum_e dO_ie V_je,   dS_ij = dP_ij act'(S_ij)
    dV_j = sum_i P_ij dO_i,     dQ_i = sum_j dS_ij K_j / sqrt(d),
    dK_j = sum_i dS_ij Q_i / sqrt(d)

(each sum only over valid pairs).

Readings where the pages are silent (listed with the others in the design notes):
  * scale 1/sqrt(d) on S before the activation;
  * GELU is the exact erf form x * Phi(x) (the pages' series is that function's
    Maclaurin series);
  * no causal mask; ``window`` w > 0 keeps |i - j| < w on per-sample indices and
    requires Lq_b == Lk_b;
  * rows with no valid partner (Lk_b == 0, or Lq_b == 0 for dK/dV) are zero.

Rows are independent in the definition, so windowed samples are evaluated in
groups of query rows with the keys their windows reach; nothing else is blocked
or reordered.  Parity pins: tests/test_oracle.py.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf, expit

# ---------------------------------------------------------------------------
# activations and their derivatives
# ---------------------------------------------------------------------------

_INV_SQRT2 = 1.0 / math.sqrt(2.0)
_INV_SQRT2PI = 1.0 / math.sqrt(2.0 * math.pi)

# GDPA page, "Section details", code figure of the ALU-only Taylor GELU: the
# coefficients of x, x^2, x^4, x^6.  Written here in closed form; the printed
# decimals are pinned against these in tests/golden/taylor_gelu_coefficients.json.
TAYLOR6 = (0.5, _INV_SQRT2PI, -_INV_SQRT2PI / 6.0, _INV_SQRT2PI / 40.0)

ACTIVATIONS = ("gelu", "silu", "gelu_taylor6", "identity", "one")


def act_fwd(x: np.ndarray, act: str) -> np.ndarray:
    """act(x) in fp64.  gelu: x * Phi(x) = x/2 (1 + erf(x / sqrt 2)); silu: x * sigmoid(x);
    gelu_taylor6: the GDPA page's series; identity: x; one: 1 (count probe)."""
    x = np.asarray(x, dtype=np.float64)
    if act == "gelu":
        return 0.5 * x * (1.0 + erf(x * _INV_SQRT2))
    if act == "silu":
        return x * expit(x)
    if act == "gelu_taylor6":
        c1, c2, c4, c6 = TAYLOR6
        x2 = x * x
        return c1 * x + c2 * x2 + c4 * x2 * x2 + c6 * x2 * x2 * x2
    if act == "identity":
        return x.copy()
    if act == "one":
        return np.ones_like(x)
    raise ValueError(f"unknown activation {act!r}")


def act_grad(x: np.ndarray, act: str) -> np.ndarray:
    """d act / dx in fp64.  gelu: Phi(x) + x phi(x); silu: s (1 + x (1 - s)), s = sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    if act == "gelu":
        return 0.5 * (1.0 + erf(x * _INV_SQRT2)) + x * _INV_SQRT2PI * np.exp(-0.5 * x * x)
    if act == "silu":
        s = expit(x)
        return s * (1.0 + x * (1.0 - s))
    if act == "gelu_taylor6":
        c1, c2, c4, c6 = TAYLOR6
        x2 = x * x
        return c1 + 2.0 * c2 * x + 4.0 * c4 * x2 * x + 6.0 * c6 * x2 * x2 * x
    if act == "identity":
        return np.ones_like(x)
    if act == "one":
        return np.zeros_like(x)
    raise ValueError(f"unknown activation {act!r}")


# ---------------------------------------------------------------------------
# helpers (input checking and the valid set)
# ---------------------------------------------------------------------------

def _check(q, k, v, q_off, kv_off, window):
    q_off = np.asarray(q_off, dtype=np.int64)
    kv_off = np.asarray(kv_off, dtype=np.int64)
    if q_off.ndim != 1 or kv_off.shape != q_off.shape or q_off[0] != 0 or kv_off[0] != 0:
        raise ValueError("offsets must be [B+1] and start at 0")
    if np.any(np.diff(q_off) < 0) or np.any(np.diff(kv_off) < 0):
        raise ValueError("offsets must be non-decreasing")
    if q.shape[0] != q_off[-1] or k.shape[0] != kv_off[-1] or v.shape != k.shape:
        raise ValueError("tensor rows do not match the offsets")
    if window < 0:
        raise ValueError("window must be >= 0")
    if window > 0 and np.any(np.diff(q_off) != np.diff(kv_off)):
        raise ValueError("a window needs Lq == Lk for every sample")
    return q_off, kv_off


def valid_mask(i: np.ndarray, j: np.ndarray, lq: int, lk: int, window: int) -> np.ndarray:
    """Boolean [len(i), len(j)]: (i, j) is a valid pair of a sample of lengths (lq, lk)."""
    i = np.asarray(i)[:, None]
    j = np.asarray(j)[None, :]
    m = (i >= 0) & (i < lq) & (j >= 0) & (j < lk)
    if window > 0:
        m &= np.abs(i - j) < window
    return m


def _row_groups(lq: int, lk: int, window: int, group: int = 512):
    """(query range, key range) pairs covering a sample.  Without a window the
    single group is the whole sample; with one, each group of query rows takes
    the keys its windows reach."""
    if window == 0:
        yield 0, lq, 0, lk
        return
    for i0 in range(0, lq, group):
        i1 = min(lq, i0 + group)
        yield i0, i1, max(0, i0 - window + 1), min(lk, i1 + window - 1)


# ---------------------------------------------------------------------------
# forward and backward
# ---------------------------------------------------------------------------

def gdpa_fwd(q, k, v, q_off, kv_off, act: str, window: int = 0) -> np.ndarray:
    """O [Tq, H, d] (fp64) for jagged inputs q [Tq, H, d], k/v [Tk, H, d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_off, kv_off = _check(q, k, v, q_off, kv_off, window)
    d = q.shape[2]
    scale = 1.0 / math.sqrt(d)
    o = np.zeros_like(q)
    for b in range(len(q_off) - 1):
        qs, lq = int(q_off[b]), int(q_off[b + 1] - q_off[b])
        ks, lk = int(kv_off[b]), int(kv_off[b + 1] - kv_off[b])
        if lq == 0 or lk == 0:
            continue
        for i0, i1, j0, j1 in _row_groups(lq, lk, window):
            qh = q[qs + i0:qs + i1].transpose(1, 0, 2)          # [H, n, d]
            kh = k[ks + j0:ks + j1].transpose(1, 0, 2)          # [H, m, d]
            vh = v[ks + j0:ks + j1].transpose(1, 0, 2)
            s = np.matmul(qh, kh.transpose(0, 2, 1)) * scale    # [H, n, m]
            p = act_fwd(s, act) * valid_mask(np.arange(i0, i1), np.arange(j0, j1), lq, lk, window)
            o[qs + i0:qs + i1] = np.matmul(p, vh).transpose(1, 0, 2)
    return o


def gdpa_bwd(q, k, v, do, q_off, kv_off, act: str, window: int = 0):
    """(dQ, dK, dV) in fp64 for the loss sum(O * dO)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    q_off, kv_off = _check(q, k, v, q_off, kv_off, window)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    d = q.shape[2]
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(q_off) - 1):
        qs, lq = int(q_off[b]), int(q_off[b + 1] - q_off[b])
        ks, lk = int(kv_off[b]), int(kv_off[b + 1] - kv_off[b])
        if lq == 0 or lk == 0:
            continue
        for i0, i1, j0, j1 in _row_groups(lq, lk, window):
            qh = q[qs + i0:qs + i1].transpose(1, 0, 2)
            kh = k[ks + j0:ks + j1].transpose(1, 0, 2)
            vh = v[ks + j0:ks + j1].transpose(1, 0, 2)
            doh = do[qs + i0:qs + i1].transpose(1, 0, 2)
            m = valid_mask(np.arange(i0, i1), np.arange(j0, j1), lq, lk, window)
            s = np.matmul(qh, kh.transpose(0, 2, 1)) * scale
            p = act_fwd(s, act) * m
            dp = np.matmul(doh, vh.transpose(0, 2, 1))
            ds = dp * act_grad(s, act) * m
            dq[qs + i0:qs + i1] += (np.matmul(ds, kh) * scale).transpose(1, 0, 2)
            dk[ks + j0:ks + j1] += (np.matmul(ds.transpose(0, 2, 1), qh) * scale).transpose(1, 0, 2)
            dv[ks + j0:ks + j1] += np.matmul(p.transpose(0, 2, 1), doh).transpose(1, 0, 2)
    return dq, dk, dv


def gdpa_fwd_scalar(q, k, v, q_off, kv_off, act: str, window: int = 0) -> np.ndarray:
    """The definition as plain Python loops over (b, h, i, j, e).  Tiny inputs only."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_off, kv_off = _check(q, k, v, q_off, kv_off, window)
    T, H, d = q.shape
    o = np.zeros_like(q)
    for b in range(len(q_off) - 1):
        lq, lk = int(q_off[b + 1] - q_off[b]), int(kv_off[b + 1] - kv_off[b])
        for h in range(H):
            for i in range(lq):
                acc = [0.0] * d
                for j in range(lk):
                    if window > 0 and abs(i - j) >= window:
                        continue
                    s = 0.0
                    for e in range(d):
                        s += float(q[q_off[b] + i, h, e]) * float(k[kv_off[b] + j, h, e])
                    p = float(act_fwd(np.array(s / math.sqrt(d)), act))
                    for e in range(d):
                        acc[e] += p * float(v[kv_off[b] + j, h, e])
                o[q_off[b] + i, h, :] = acc
    return o


def useful_pairs(lq, lk, window: int = 0) -> int:
    """|V| summed over samples: the number of valid (query, key) pairs."""
    total = 0
    for a, c in zip(np.asarray(lq, dtype=np.int64), np.asarray(lk, dtype=np.int64)):
        a, c = int(a), int(c)
        if window == 0:
            total += a * c
        else:
            for i in range(a):
                total += min(c, i + window) - max(0, i - window + 1)
    return total


# ---------------------------------------------------------------------------
# pFFN as GDPA
# ---------------------------------------------------------------------------
# GDPA page, "Section details", diagram "Self-attention, PMA and pFFN unified as
# GDPA": pFFN is the third module with the two-products-and-an-activation shape.
# The page defines nothing more; the reading used here: per head, learned weight
# matrices W_K, W_V [M, H, d] play the keys and values of every query row of the
# batch, so O_i = sum_j act(Q_i . W_K,j / sqrt(d)) W_V,j over all M weight rows,
# and the weight gradients dW_K, dW_V are sums over every query row.  Samples do
# not interact, so this is GDPA on one sample holding all Tq query rows.

def pffn_fwd(q, wk, wv, act: str) -> np.ndarray:
    """O [Tq, H, d] (fp64) of pFFN with shared weights wk, wv [M, H, d]."""
    tq, m = q.shape[0], wk.shape[0]
    return gdpa_fwd(q, wk, wv, np.array([0, tq]), np.array([0, m]), act, 0)


def pffn_bwd(q, wk, wv, do, act: str):
    """(dQ, dW_K, dW_V) in fp64 for the loss sum(O * dO)."""
    tq, m = q.shape[0], wk.shape[0]
    return gdpa_bwd(q, wk, wv, do, np.array([0, tq]), np.array([0, m]), act, 0)


# ---------------------------------------------------------------------------
# RMSNorm prologue: GDPA on normalised Q, K (and V)
# ---------------------------------------------------------------------------
# GDPA page, "Section details", the chart comparing tanh GELU with the 6th-order
# series: in the models, RMSNorm keeps the activation's inputs in range.  The pages
# say no more; the reading used here is the norm applied right before the
# attention, per (token, head) over the d features, with no gain and eps = 1e-6:
#     x^ = x r,   r = 1 / sqrt(mean_c x_c^2 + eps),
# on the tensors named in `norm` (a subset of "qkv"), and GDPA on the normalised
# tensors.  The gradient of the raw input follows from the chain rule through the
# norm: dx = r (dx^ - x^ mean_c(dx^_c x^_c)).

RMS_EPS = 1e-6


def rms_norm(x, eps: float = RMS_EPS) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rms_norm_bwd(x, dy, eps: float = RMS_EPS) -> np.ndarray:
    """Gradient of sum(rms_norm(x) * dy) with respect to x."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def _normed(q, k, v, norm: str):
    if set(norm) - set("qkv"):
        raise ValueError(f"norm must be a subset of 'qkv', got {norm!r}")
    return (rms_norm(q) if "q" in norm else np.asarray(q, np.float64),
            rms_norm(k) if "k" in norm else np.asarray(k, np.float64),
            rms_norm(v) if "v" in norm else np.asarray(v, np.float64))


def norm_gdpa_fwd(q, k, v, q_off, kv_off, act: str, window: int = 0, norm: str = "qkv") -> np.ndarray:
    """O of GDPA on the RMS-normalised tensors named in `norm`."""
    qn, kn, vn = _normed(q, k, v, norm)
    return gdpa_fwd(qn, kn, vn, q_off, kv_off, act, window)


def norm_gdpa_bwd(q, k, v, do, q_off, kv_off, act: str, window: int = 0, norm: str = "qkv"):
    """(dQ, dK, dV) with respect to the raw tensors for the loss sum(O * dO)."""
    qn, kn, vn = _normed(q, k, v, norm)
    dqn, dkn, dvn = gdpa_bwd(qn, kn, vn, do, q_off, kv_off, act, window)
    return (rms_norm_bwd(q, dqn) if "q" in norm else dqn,
            rms_norm_bwd(k, dkn) if "k" in norm else dkn,
            rms_norm_bwd(v, dvn) if "v" in norm else dvn)


# ---------------------------------------------------------------------------
# JFA: softmax attention on the same jagged pairs
# ---------------------------------------------------------------------------
# GEM page, section "why high GPU utilisation is hard" (jagged attention kernels)
# and GDPA page, "Section details" (GDPA drops the softmax's row max, row sum and
# correction; JFA is the variant that keeps them).  Per sample b, head h, over the
# same valid set V_b: P_ij = exp(S_ij) / sum_{j' : (i, j') in V_b} exp(S_ij'), O = P V.
# A row with no valid key has O = 0 and log-sum-exp -inf.  Backward for
# l = sum(O * dO): dP = dO V^T, D_i = sum_e dO_ie O_ie, dS = P (dP - D), then dV, dQ,
# dK as for GDPA.

def jfa_fwd(q, k, v, q_off, kv_off, window: int = 0):
    """(O [Tq, H, d], LSE [H, Tq]) in fp64; LSE_i = log sum_j exp(S_ij) over the valid keys."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_off, kv_off = _check(q, k, v, q_off, kv_off, window)
    d, H = q.shape[2], q.shape[1]
    scale = 1.0 / math.sqrt(d)
    o = np.zeros_like(q)
    lse = np.full((H, q.shape[0]), -np.inf)
    for b in range(len(q_off) - 1):
        qs, lq = int(q_off[b]), int(q_off[b + 1] - q_off[b])
        ks, lk = int(kv_off[b]), int(kv_off[b + 1] - kv_off[b])
        if lq == 0 or lk == 0:
            continue
        for i0, i1, j0, j1 in _row_groups(lq, lk, window):
            qh = q[qs + i0:qs + i1].transpose(1, 0, 2)
            kh = k[ks + j0:ks + j1].transpose(1, 0, 2)
            vh = v[ks + j0:ks + j1].transpose(1, 0, 2)
            m = valid_mask(np.arange(i0, i1), np.arange(j0, j1), lq, lk, window)
            s = np.where(m, np.matmul(qh, kh.transpose(0, 2, 1)) * scale, -np.inf)
            mx = s.max(axis=2, keepdims=True)
            e = np.exp(s - mx)                                  # exp(-inf) = 0 off the valid set
            tot = e.sum(axis=2, keepdims=True)
            o[qs + i0:qs + i1] = np.matmul(e / tot, vh).transpose(1, 0, 2)
            lse[:, qs + i0:qs + i1] = (mx + np.log(tot))[:, :, 0]
    return o, lse


def jfa_bwd(q, k, v, do, q_off, kv_off, window: int = 0):
    """(dQ, dK, dV) in fp64 for the loss sum(O * dO) of jfa_fwd."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    q_off, kv_off = _check(q, k, v, q_off, kv_off, window)
    o, lse = jfa_fwd(q, k, v, q_off, kv_off, window)
    d = q.shape[2]
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(q_off) - 1):
        qs, lq = int(q_off[b]), int(q_off[b + 1] - q_off[b])
        ks, lk = int(kv_off[b]), int(kv_off[b + 1] - kv_off[b])
        if lq == 0 or lk == 0:
            continue
        for i0, i1, j0, j1 in _row_groups(lq, lk, window):
            qh = q[qs + i0:qs + i1].transpose(1, 0, 2)
            kh = k[ks + j0:ks + j1].transpose(1, 0, 2)
            vh = v[ks + j0:ks + j1].transpose(1, 0, 2)
            doh = do[qs + i0:qs + i1].transpose(1, 0, 2)
            oh = o[qs + i0:qs + i1].transpose(1, 0, 2)
            m = valid_mask(np.arange(i0, i1), np.arange(j0, j1), lq, lk, window)
            s = np.matmul(qh, kh.transpose(0, 2, 1)) * scale
            p = np.where(m, np.exp(s - lse[:, qs + i0:qs + i1, None]), 0.0)
            dp = np.matmul(doh, vh.transpose(0, 2, 1))
            dd = (doh * oh).sum(axis=2, keepdims=True)          # D_i
            ds = p * (dp - dd)
            dq[qs + i0:qs + i1] += (np.matmul(ds, kh) * scale).transpose(1, 0, 2)
            dk[ks + j0:ks + j1] += (np.matmul(ds.transpose(0, 2, 1), qh) * scale).transpose(1, 0, 2)
            dv[ks + j0:ks + j1] += np.matmul(p.transpose(0, 2, 1), doh).transpose(1, 0, 2)
    return dq, dk, dv
