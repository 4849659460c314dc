"""Seeded synthetic jagged inputs for GDPA: the five workloads and edge-case builders.

This module is shared by the HIP path's tests/bench and by the CPU oracle's tests.
It holds input generation only (sequence lengths, random draws, the per-row RMS
normalisation of the inputs, rounding to the storage dtype) and none of the
attention arithmetic.

Workloads follow the shapes named on the GEM page (techlist.io, "GEM training:
how Meta doubled the efficiency of an LLM-scale ads foundation model",
section "why high GPU utilisation is hard for recommendation models": variable
sequence lengths; windowed self-attention over long histories; user-ad
cross-attention with long Q and short K/V; PMA with short Q and long K/V).
Production data is not available; these seeded draws stand in for it.

Recipe (all seeds explicit):
  * lengths: ``numpy.random.default_rng(seed)``, drawn first.
      - uniform{lo..hi}:   rng.integers(lo, hi + 1, size=B)
      - lognormal(med, mx): clip(rint(exp(N(ln med, sigma^2))), 1, mx),
        sigma = ln(mx / med) / 3 so that mx sits at +3 sigma.
  * values: ``torch.Generator(device).manual_seed(seed + 1)``; draw order
    Q, K, V, dO, each i.i.d. N(0, 1) in fp32.  PMA seed rows: 32 x H x d draws of
    N(0, 0.02^2), shared by every sample.
  * RMS normalisation of an input (per token and head, over d, no gain):
    x / sqrt(mean(x^2) + 1e-6), in fp32, before rounding.
  * raw inputs for the fused-norm path (rms = ""): with row_spread s > 0, each
    (token, head) row of Q, K and V is multiplied by exp(s N(0, 1)), drawn after dO
    in the order Q, K, V, so that rows differ in scale as un-normalised activations do.
  * rounding: fp32 -> storage dtype (bf16 round-to-nearest-even); the oracle is
    fed the rounded values widened to fp64.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

WORKLOADS = {
    1: dict(name="tiny_self_gelu_f32", B=4, H=2, d=32, act="gelu", window=0, dtype="f32",
            lq=("uniform", 1, 64), lk="same", rms="qkv", directions=("fwd",)),
    2: dict(name="jagged_self_silu_bf16", B=1024, H=4, d=128, act="silu", window=0, dtype="bf16",
            lq=("lognormal", 64, 512), lk="same", rms="qkv", directions=("fwd", "bwd")),
    3: dict(name="cross_user_ad_gelu_bf16", B=2048, H=8, d=64, act="gelu", window=0, dtype="bf16",
            lq=("lognormal", 256, 1024), lk=("fixed", 32), rms="qkv", directions=("fwd", "bwd")),
    4: dict(name="pma_gelu_bf16", B=512, H=4, d=128, act="gelu", window=0, dtype="bf16",
            lq=("fixed", 32), lk=("lognormal", 1024, 4096), rms="kv", pma_seeds=True,
            directions=("fwd", "bwd")),
    5: dict(name="windowed_self_gelu_bf16", B=128, H=4, d=128, act="gelu", window=128, dtype="bf16",
            lq=("uniform", 512, 8192), lk="same", rms="qkv", directions=("fwd", "bwd")),
}


def _draw_lengths(rng: np.random.Generator, spec, B: int) -> np.ndarray:
    kind = spec[0]
    if kind == "uniform":
        return rng.integers(spec[1], spec[2] + 1, size=B).astype(np.int64)
    if kind == "lognormal":
        med, mx = spec[1], spec[2]
        sigma = math.log(mx / med) / 3.0
        x = np.exp(rng.normal(math.log(med), sigma, size=B))
        return np.clip(np.rint(x), 1, mx).astype(np.int64)
    if kind == "fixed":
        return np.full(B, spec[1], dtype=np.int64)
    raise ValueError(f"unknown length spec {spec!r}")


def workload_lengths(cfg: int, seed: int = 0, B: Optional[int] = None):
    """(lq, lk) int64 arrays for workload ``cfg``; ``B`` overrides the batch size."""
    w = WORKLOADS[cfg]
    B = w["B"] if B is None else B
    rng = np.random.default_rng(seed)
    lq = _draw_lengths(rng, w["lq"], B)
    lk = lq.copy() if w["lk"] == "same" else _draw_lengths(rng, w["lk"], B)
    return lq, lk


def offsets(lengths: Sequence[int]) -> np.ndarray:
    """int32 [B+1] exclusive prefix sum; sample b owns rows off[b]..off[b+1]-1."""
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    if off[-1] > np.iinfo(np.int32).max:
        raise ValueError("total rows exceed int32")
    return off.astype(np.int32)


# ---------------------------------------------------------------------------
# value generation
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class JaggedInputs:
    """One batch of jagged GDPA inputs.  Tensors are [T, H, d] in the storage dtype."""
    cfg: Optional[int]
    H: int
    d: int
    act: str
    window: int
    dtype: str                    # "bf16" or "f32"
    lq: np.ndarray                # int64 [B]
    lk: np.ndarray                # int64 [B]
    q_off: np.ndarray             # int32 [B+1]
    kv_off: np.ndarray            # int32 [B+1]
    q: "object"                   # torch.Tensor
    k: "object"
    v: "object"
    do: "object"

    @property
    def B(self) -> int:
        return len(self.lq)

    def f64(self, name: str) -> np.ndarray:
        """A tensor's stored (rounded) values widened to fp64, on the host."""
        import torch
        t = getattr(self, name)
        return t.detach().to("cpu", torch.float64).numpy()


def _rms_normalise(x, eps: float = 1e-6):
    import torch
    return x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + eps)


def make_from_lengths(lq, lk, H: int, d: int, *, act: str = "gelu", window: int = 0,
                      dtype: str = "bf16", seed: int = 0, device: str = "cpu",
                      rms: str = "qkv", pma_seeds: bool = False, cfg: Optional[int] = None,
                      q_scale: float = 1.0, row_spread: float = 0.0) -> JaggedInputs:
    """Draw Q, K, V, dO for the given per-sample lengths (see the module recipe)."""
    import torch
    lq = np.asarray(lq, dtype=np.int64)
    lk = np.asarray(lk, dtype=np.int64)
    if len(lq) != len(lk):
        raise ValueError("lq and lk must have the same batch size")
    q_off, kv_off = offsets(lq), offsets(lk)
    Tq, Tk = int(q_off[-1]), int(kv_off[-1])
    g = torch.Generator(device=device)
    g.manual_seed(seed + 1)
    f32 = torch.float32
    if pma_seeds:
        if len(lq) and not np.all(lq == lq[0]):
            raise ValueError("PMA seeds need the same Lq for every sample")
        nseed = int(lq[0]) if len(lq) else 0
        seeds = torch.randn((nseed, H, d), generator=g, device=device, dtype=f32) * 0.02
        q = seeds.repeat(len(lq), 1, 1)
    else:
        q = torch.randn((Tq, H, d), generator=g, device=device, dtype=f32)
    k = torch.randn((Tk, H, d), generator=g, device=device, dtype=f32)
    v = torch.randn((Tk, H, d), generator=g, device=device, dtype=f32)
    do = torch.randn((Tq, H, d), generator=g, device=device, dtype=f32)
    if row_spread > 0.0:
        q, k, v = (x * torch.exp(row_spread * torch.randn(x.shape[:2] + (1,), generator=g, device=device,
                                                          dtype=f32)) for x in (q, k, v))
    if "q" in rms and not pma_seeds:
        q = _rms_normalise(q)
    if "k" in rms:
        k = _rms_normalise(k)
    if "v" in rms:
        v = _rms_normalise(v)
    if q_scale != 1.0:
        q = q * q_scale
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    q, k, v, do = (t.to(tdt).contiguous() for t in (q, k, v, do))
    return JaggedInputs(cfg=cfg, H=H, d=d, act=act, window=window, dtype=dtype, lq=lq, lk=lk,
                        q_off=q_off, kv_off=kv_off, q=q, k=k, v=v, do=do)


def make_workload(cfg: int, seed: int = 0, device: str = "cpu", B: Optional[int] = None,
                  act: Optional[str] = None, raw: bool = False) -> JaggedInputs:
    """Inputs of workload ``cfg`` (1..5); ``B`` shrinks the batch for fast tests.
    raw: no RMS normalisation, rows spread in scale (row_spread 1), for the fused-norm path."""
    w = WORKLOADS[cfg]
    lq, lk = workload_lengths(cfg, seed, B)
    return make_from_lengths(lq, lk, w["H"], w["d"], act=act or w["act"], window=w["window"],
                             dtype=w["dtype"], seed=seed, device=device, rms="" if raw else w["rms"],
                             pma_seeds=w.get("pma_seeds", False), cfg=cfg, row_spread=1.0 if raw else 0.0)


# pFFN as GDPA (the third module of the GDPA page's unified-modules diagram; read as
# shared weight rows W_K, W_V [M, H, d] for every query row of the batch): the query
# rows of the jagged self-attention batch (workload 2's lengths, Tq = 79,265 at seed
# 0) against M = 512 weight rows per head, H = 4, d = 128, SiLU.  The weights are
# drawn like keys and values (N(0, 1), RMS-normalised); they stand in for trained
# weights, which are not available.
PFFN = dict(name="pffn_silu_bf16", queries_of=2, M=512, H=4, d=128, act="silu", dtype="bf16", rms="qkv")


def make_pffn(seed: int = 0, device: str = "cpu", Tq: Optional[int] = None, M: Optional[int] = None,
              act: Optional[str] = None) -> JaggedInputs:
    """pFFN inputs as one sample: q [Tq, H, d], k = W_K and v = W_V [M, H, d], dO."""
    w = PFFN
    if Tq is None:
        lq, _ = workload_lengths(w["queries_of"], seed)
        Tq = int(np.sum(lq))
    return make_from_lengths([Tq], [w["M"] if M is None else M], w["H"], w["d"], act=act or w["act"],
                             window=0, dtype=w["dtype"], seed=seed, device=device, rms=w["rms"])


def pad_waste(lengths, multiple: Optional[int] = None) -> float:
    """Fraction of token slots that are padding when samples are padded to the
    batch max (``multiple=None``) or up to a multiple of ``multiple``."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if multiple is None:
        padded = len(lengths) * int(lengths.max())
    else:
        padded = int((-(-lengths // multiple) * multiple).sum())
    return 1.0 - float(lengths.sum()) / padded if padded else 0.0
