"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Tolerances (stated with the task's definition of the path):
  * fp32 path: max |err| <= 1e-4 * max |ref|
  * bf16 in / fp32 accumulate: relative L2 <= 1e-2 and max |err| <= 2e-2 * max |ref|,
    for O and separately for each of dQ, dK, dV.
  * the polynomial GELU against the exact-erf oracle: the bf16 bounds plus the
    fits' bounds propagated through the products (eps * sum_j |V_j| per element
    for O and eps * sum_i |dO_i| for dV; eps' * sum_j |dO_i|.|V_j| |K_j| / sqrt d
    for dQ and its mirror for dK).
Offset indexing is checked bit-exactly with count probes (act = one, fp32 outputs).
"""
import math

import numpy as np
import pytest
import torch

import recsys_attention_jagged_amd as G
from gdpa_workloads import WORKLOADS, make_from_lengths, make_pffn, make_workload, offsets
from oracle import gdpa_ref as R
from oracle import plan_ref as PR
from fp8_bounds import check_fp8, dequant_mx, quant_e4m3, quant_mx

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def dev_offsets(inp):
    return (torch.tensor(inp.q_off, dtype=torch.int32, device=DEV),
            torch.tensor(inp.kv_off, dtype=torch.int32, device=DEV))


def check_close(got, ref, what, f32=False, extra=None, floor=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    mx = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = np.abs(got - ref)
    if extra is not None:
        err = np.maximum(err - extra, 0.0)
    if f32:
        assert float(err.max(initial=0.0)) <= 1e-4 * mx + 1e-30, f"{what}: max err {err.max():.3e} vs max|ref| {mx:.3e}"
        return
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(err)) / nrm if nrm > 0 else float(np.linalg.norm(err))
    assert rel <= 1e-2, f"{what}: rel L2 {rel:.3e}"
    assert float(err.max(initial=0.0)) <= 2e-2 * mx + floor + 1e-30, \
        f"{what}: max err {err.max():.3e} vs 2e-2*{mx:.3e} + {floor:.1e}"


def run_fwd(inp, act=None, dtype=None, **opts):
    act = act or inp.act
    dtype = dtype or inp.dtype
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, dtype, **opts) as plan:
        o = plan.fwd(inp.q, inp.k, inp.v, qo, ko, act)
        torch.cuda.synchronize()
    return o.float().cpu().numpy()


def run_bwd(inp, act=None, dtype=None, **opts):
    act = act or inp.act
    dtype = dtype or inp.dtype
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, dtype, **opts) as plan:
        dq, dk, dv = plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, act)
        torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy() for t in (dq, dk, dv))


def oracle_fwd(inp, act=None):
    return R.gdpa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, act or inp.act,
                      inp.window)


def oracle_bwd(inp, act=None):
    return R.gdpa_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"), inp.q_off, inp.kv_off,
                      act or inp.act, inp.window)


# ---------------------------------------------------------------------------
# workloads at reduced batch (several tiles and ragged tails each)
# ---------------------------------------------------------------------------

SMALL_B = {2: 48, 3: 24, 4: 12, 5: 3}


def test_cfg1_fp32_forward():
    say("cfg1 fp32 forward, full size")
    inp = make_workload(1, device=DEV)
    check_close(run_fwd(inp), oracle_fwd(inp), "cfg1 O", f32=True)


def test_fp32_backward():
    say("fp32 backward on cfg1 shapes")
    inp = make_workload(1, device=DEV)
    g = run_bwd(inp)
    r = oracle_bwd(inp)
    for name, a, b in zip(("dQ", "dK", "dV"), g, r):
        check_close(a, b, f"fp32 {name}", f32=True)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("act,window", [("gelu", 0), ("silu", 0), ("gelu_taylor6", 0), ("identity", 0),
                                        ("gelu", 5), ("silu", 17)])
def test_fp32_path(d, act, window):
    """The fp32 path at every head dimension, the activations and windows, on ragged lengths
    with empty samples on either side, forward and backward, to the fp32 bound."""
    say(f"fp32 path d={d} act={act} window={window}")
    lq = [0, 1, 31, 33, 70, 5, 0]
    lk = lq if window else [4, 0, 40, 33, 9, 64, 0]
    inp = make_from_lengths(lq, lk, 2, d, act=act, window=window, dtype="f32", seed=61, device=DEV)
    check_close(run_fwd(inp), oracle_fwd(inp), f"fp32 O d={d} {act} w={window}", f32=True)
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp), oracle_bwd(inp)):
        check_close(a, b, f"fp32 {name} d={d} {act} w={window}", f32=True)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_workload_forward_small(cfg):
    say(f"cfg{cfg} forward, B={SMALL_B[cfg]}")
    inp = make_workload(cfg, device=DEV, B=SMALL_B[cfg])
    check_close(run_fwd(inp), oracle_fwd(inp), f"cfg{cfg} O")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_workload_backward_small(cfg):
    say(f"cfg{cfg} backward, B={SMALL_B[cfg]}")
    inp = make_workload(cfg, device=DEV, B=SMALL_B[cfg])
    g = run_bwd(inp)
    r = oracle_bwd(inp)
    for name, a, b in zip(("dQ", "dK", "dV"), g, r):
        check_close(a, b, f"cfg{cfg} {name}")


# ---------------------------------------------------------------------------
# every item layout, head dimension and activation
# ---------------------------------------------------------------------------

RAGGED = [0, 1, 5, 31, 32, 33, 64, 65, 100, 127, 128, 129, 200, 300]


FWD_LAYOUTS = [(32, 1, 1), (32, 1, 2), (64, 1, 1), (64, 1, 2), (128, 1, 1), (128, 1, 2), (128, 2, 1)]


@pytest.mark.parametrize("d,team,nb", FWD_LAYOUTS)
def test_layouts_forward(d, team, nb):
    say(f"forward layout d={d} team={team} blocks={nb}")
    rng = np.random.default_rng(d + 3 * team + nb)
    lq = rng.permutation(RAGGED)
    lk = rng.permutation(RAGGED)
    inp = make_from_lengths(lq, lk, 2, d, act="gelu", seed=3, device=DEV)
    check_close(run_fwd(inp, team=(team, 0, 0), blocks=(nb, 0, 0)), oracle_fwd(inp), f"O d={d} t={team} nb={nb}")


# (d, dQ team, dQ blocks, dK/dV team)
BWD_LAYOUTS = [(32, 1, 1, 1), (32, 1, 2, 1), (64, 1, 1, 1), (64, 1, 2, 1), (128, 1, 1, 1), (128, 1, 2, 1),
               (128, 2, 1, 2)]


@pytest.mark.parametrize("d,tq,nb,tk", BWD_LAYOUTS)
def test_layouts_backward(d, tq, nb, tk):
    say(f"backward layout d={d} dq team={tq} blocks={nb} dkdv team={tk}")
    rng = np.random.default_rng(10 * d + 3 * tq + nb + tk)
    lq = rng.permutation(RAGGED)
    lk = rng.permutation(RAGGED)
    inp = make_from_lengths(lq, lk, 2, d, act="silu", seed=4, device=DEV)
    g = run_bwd(inp, team=(0, tk, tq), blocks=(0, 1, nb))
    r = oracle_bwd(inp)
    for name, a, b in zip(("dQ", "dK", "dV"), g, r):
        check_close(a, b, f"{name} d={d} tq={tq} nb={nb} tk={tk}")


# The d = 128 dK/dV kernel's 16-row waves in two-wave (32-row items) and four-wave
# (64-row items) teams: windows that cut a wave's rows out of some q tiles, items cut
# into chunks (few bins), samples shorter than a team's rows, fp32 outputs.
@pytest.mark.parametrize("tk", [1, 2])
@pytest.mark.parametrize("window,bins", [(0, (0, 0, 0)), (5, (0, 0, 0)), (128, (0, 0, 0)), (0, (16, 16, 16)),
                                         (40, (8, 8, 8))])
def test_dkdv_16row_teams(tk, window, bins):
    say(f"dK/dV 16-row waves: team={tk} window={window} bins={bins}")
    L = [1, 15, 16, 17, 33, 47, 64, 65, 0, 300, 129, 700]
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=window, seed=80 + tk + window, device=DEV)
    r = oracle_bwd(inp)
    for dtype in ("bf16", "bf16_f32out"):
        g = run_bwd(inp, dtype=dtype, team=(0, tk, 0), bins=bins, unfused=True)
        for name, a, b in zip(("dQ", "dK", "dV"), g, r):
            check_close(a, b, f"{name} team={tk} window={window} bins={bins} {dtype}")


# d = 128 two-kernel backward with stored dS: the dK/dV kernel stores each 32 x 32 dS
# block, the dQ kernel multiplies the stored blocks by K
@pytest.mark.parametrize("window,bins", [(0, (0, 0, 0)), (9, (0, 0, 0)), (128, (0, 0, 0)), (0, (16, 16, 16)),
                                         (40, (8, 8, 8))])
@pytest.mark.parametrize("dtype", ["bf16", "bf16_f32out"])
@pytest.mark.parametrize("team", [1, 2])   # 32- or 64-row dK/dV items
def test_stored_ds_backward(window, bins, dtype, team):
    say(f"stored dS backward window={window} bins={bins} {dtype} dK/dV team={team}")
    L = [1, 15, 16, 17, 33, 47, 64, 65, 0, 300, 129, 700]
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=window, seed=90 + window, device=DEV)
    qo, ko = dev_offsets(inp)
    r = oracle_bwd(inp)
    with G.Plan(inp.q_off, inp.kv_off, 2, 128, window, dtype, bins=bins, unfused=True,
                team=(0, team, 0)) as plan:
        assert plan.stats()["ds_bytes"] > 0
        whole = [t.float().cpu().numpy() for t in plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, "gelu")]
        odt = torch.float32 if dtype == "bf16_f32out" else torch.bfloat16
        dq = torch.full(inp.q.shape, float("nan"), dtype=odt, device=DEV)
        dk = torch.full(inp.k.shape, float("nan"), dtype=odt, device=DEV)
        dv = torch.full(inp.v.shape, float("nan"), dtype=odt, device=DEV)
        args = (plan.handle, inp.q, inp.k, inp.v, inp.do, qo, ko, plan.B, 2, 128, "gelu", window)
        G.gdpa_bwd_dkdv(*args, dk, dv)
        G.gdpa_bwd_dq(*args, dq)
        torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), whole, r):
        check_close(a, b, f"{name} stored dS window={window} bins={bins} {dtype} team={team}")
    for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), whole):
        assert np.array_equal(a.float().cpu().numpy(), b), f"{name}: split calls differ from gdpa_bwd"
    # without a dS buffer, dQ alone recomputes dS
    with G.Plan(inp.q_off, inp.kv_off, 2, 128, window, dtype, bins=bins, unfused=True, store_ds=False) as plan:
        assert plan.stats()["ds_bytes"] == 0
        dq2 = torch.empty(inp.q.shape, dtype=torch.float32 if dtype == "bf16_f32out" else torch.bfloat16, device=DEV)
        G.gdpa_bwd_dq(plan.handle, inp.q, inp.k, inp.v, inp.do, qo, ko, plan.B, 2, 128, "gelu", window, dq2)
        torch.cuda.synchronize()
    check_close(dq2.float().cpu().numpy(), r[0], f"dQ alone window={window} {dtype}")


@pytest.mark.parametrize("bins", [(1, 1, 1), (3, 5, 6), (13, 9, 7)])
def test_few_bins_long_walks(bins):
    say(f"few bins {bins}: long per-wave walks across many items")
    rng = np.random.default_rng(sum(bins))
    lq = rng.permutation(RAGGED)
    lk = rng.permutation(RAGGED)
    inp = make_from_lengths(lq, lk, 3, 64, act="silu", seed=12, device=DEV)
    check_close(run_fwd(inp, bins=bins), oracle_fwd(inp), f"O bins={bins}")
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp, bins=bins), oracle_bwd(inp)):
        check_close(a, b, f"{name} bins={bins}")


# one-pass backward shapes: every Lk <= 32 (KV-stationary) or every Lq <= 32 (Q-stationary)
FUSED_CASES = [
    ([300, 5, 0, 77, 1, 64, 129], [32, 1, 0, 17, 32, 31, 2], 0),
    ([32, 1, 0, 17, 32, 31, 2], [300, 5, 0, 77, 1, 64, 129], 0),
    ([32, 1, 20, 0, 31], [32, 1, 20, 0, 31], 5),
]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("case", range(len(FUSED_CASES)))
@pytest.mark.parametrize("unfused", [False, True])
def test_one_pass_backward(d, case, unfused):
    lq, lk, window = FUSED_CASES[case]
    say(f"one-pass backward d={d} case={case} unfused={unfused}")
    inp = make_from_lengths(lq, lk, 3, d, act="gelu", window=window, seed=13 + case, device=DEV)
    with G.Plan(inp.q_off, inp.kv_off, 3, d, window, "bf16", unfused=unfused) as plan:
        assert plan.stats()["bwd_fused"] == (0 if unfused else (1 if case != 1 else 2))
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp, unfused=unfused), oracle_bwd(inp)):
        check_close(a, b, f"{name} d={d} case={case} unfused={unfused}")
    # fp32 outputs through the same kernels
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp, dtype="bf16_f32out", unfused=unfused), oracle_bwd(inp)):
        check_close(a, b, f"{name} f32out d={d} case={case}")


# items longer than a mean bin cut into chunks (fp32 partial slots + reduction
# kernel); few bins make the long samples' items exceed the mean bin cost
CHUNK_CASES = [
    # (lq, lk, bins, the list whose items must be cut, gdpa_bwd's kernels)
    ([32, 1, 20, 32, 5, 0], [3000, 5, 700, 1, 0, 0], (16, 16, 16), "dq", 2),   # one Q-stationary pass
    ([300, 5, 70, 129, 1], [1500, 7, 64, 1000, 33], (16, 16, 32), "fwd", 0),   # two kernels
    ([3000, 5, 700, 1, 0, 0], [32, 1, 20, 32, 5, 0], (16, 16, 16), "dkdv", 1),  # one KV-stationary pass
    ([4000, 7, 300], [64, 900, 33], (32, 32, 32), "dkdv", 0),                  # two kernels, every list cut
]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("case", range(len(CHUNK_CASES)))
@pytest.mark.parametrize("deal", ["zigzag", "greedy"])
def test_cut_items(d, case, deal):
    lq, lk, bins, cut, fused = CHUNK_CASES[case]
    say(f"cut items d={d} case={case} deal={deal}")
    inp = make_from_lengths(lq, lk, 2, d, act="gelu", seed=31 + case, device=DEV)
    opts = dict(bins=bins, deal=deal)
    with G.Plan(inp.q_off, inp.kv_off, 2, d, 0, "bf16", **opts) as plan:
        st = plan.stats()
    layout = PR.auto_layout(lq, lk, 0, d)
    want = [PR.plan_list(k, lq, lk, 2, 0, bins[i], *layout[k], mode=deal)["n_parts"]
            for i, k in enumerate(("fwd", "dkdv", "dq"))]
    assert list(st["n_parts"]) == want and want[("fwd", "dkdv", "dq").index(cut)] > 0
    assert st["bwd_fused"] == fused
    ro = oracle_fwd(inp)
    rg = oracle_bwd(inp)
    check_close(run_fwd(inp, **opts), ro, f"O cut d={d} case={case}")
    check_close(run_fwd(inp, dtype="bf16_f32out", **opts), ro, f"O f32out cut d={d} case={case}")
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp, **opts), rg):
        check_close(a, b, f"{name} cut d={d} case={case}")
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp, dtype="bf16_f32out", **opts), rg):
        check_close(a, b, f"{name} f32out cut d={d} case={case}")
    # the two-kernel path over the same cut lists
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp, unfused=True, **opts), rg):
        check_close(a, b, f"{name} cut unfused d={d} case={case}")


# ---------------------------------------------------------------------------
# fp8 (e4m3fn) Q and K in the forward
# ---------------------------------------------------------------------------

def run_fp8_fwd(inp, act=None, dtype="bf16", **opts):
    act = act or inp.act
    qo, ko = dev_offsets(inp)
    q8, sq = quant_e4m3(inp.q)
    k8, sk = quant_e4m3(inp.k)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, dtype, **opts) as plan:
        o = torch.empty(inp.q.shape, dtype=torch.float32 if dtype == "bf16_f32out" else torch.bfloat16, device=DEV)
        G.gdpa_fp8_fwd(plan.handle, q8.view(torch.uint8).to(DEV), k8.view(torch.uint8).to(DEV), inp.v, qo, ko,
                       plan.B, inp.H, inp.d, act, inp.window, sq, sk, o)
        torch.cuda.synchronize()
        n_parts = plan.stats()["n_parts"]
    # the oracle on the values the bytes stand for
    ref = R.gdpa_fwd(q8.double().numpy() * sq, k8.double().numpy() * sk, inp.f64("v"), inp.q_off, inp.kv_off, act,
                     inp.window)
    return o.float().cpu().numpy(), ref, n_parts


@pytest.mark.parametrize("d,team,nb", FWD_LAYOUTS)
def test_fp8_forward_layouts(d, team, nb):
    say(f"fp8 forward d={d} team={team} blocks={nb}")
    inp = make_from_lengths(JFA_LQ, JFA_LK, 2, d, act="silu", seed=71, device=DEV)
    o, ref, _ = run_fp8_fwd(inp, team=(team, 0, 0), blocks=(nb, 0, 0))
    check_close(o, ref, f"fp8 O d={d}")
    o32, ref, _ = run_fp8_fwd(inp, dtype="bf16_f32out", team=(team, 0, 0), blocks=(nb, 0, 0))
    check_close(o32, ref, f"fp8 O f32out d={d}")


@pytest.mark.parametrize("act", ["gelu", "identity"])
@pytest.mark.parametrize("window", [0, 17])
def test_fp8_forward_acts_windows(act, window):
    say(f"fp8 forward act={act} window={window}")
    L = [1, 31, 32, 33, 127, 300, 0, 65]
    inp = make_from_lengths(L, L, 2, 128, act=act, window=window, seed=72, device=DEV)
    o, ref, _ = run_fp8_fwd(inp)
    check_close(o, ref, f"fp8 O act={act} window={window}")


def test_fp8_forward_cut_items():
    inp = make_from_lengths([32, 1], [3000, 5], 2, 64, act="gelu", seed=73, device=DEV)
    o, ref, n_parts = run_fp8_fwd(inp, bins=(16, 16, 16))
    assert n_parts[0] > 0
    check_close(o, ref, "fp8 O cut")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fp8_forward_against_bf16_inputs(cfg):
    """What quantising costs a caller: the fp8 forward on e4m3 Q, K (per-tensor
    scales) against the oracle on the bf16 inputs, within the stated fp8 bounds."""
    say(f"cfg{cfg} fp8 forward vs the bf16-input oracle, B={SMALL_B[cfg]}")
    inp = make_workload(cfg, device=DEV, B=SMALL_B[cfg])
    o, ref_q, _ = run_fp8_fwd(inp)
    check_close(o, ref_q, f"cfg{cfg} fp8 O vs the quantised values")
    check_fp8(o, oracle_fwd(inp), f"cfg{cfg} fp8 O vs the bf16 inputs")


# block-scaled fp8 (MXFP8) Q and K in the forward
def run_mx_fwd(inp, act=None, dtype="bf16", **opts):
    act = act or inp.act
    qo, ko = dev_offsets(inp)
    q8, qs = quant_mx(inp.q)
    k8, ks = quant_mx(inp.k)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, dtype, **opts) as plan:
        o = torch.empty(inp.q.shape, dtype=torch.float32 if dtype == "bf16_f32out" else torch.bfloat16, device=DEV)
        G.gdpa_mx_fwd(plan.handle, q8.view(torch.uint8).to(DEV), qs.to(DEV), k8.view(torch.uint8).to(DEV),
                      ks.to(DEV), inp.v, qo, ko, plan.B, inp.H, inp.d, act, inp.window, o)
        torch.cuda.synchronize()
        n_parts = plan.stats()["n_parts"]
    # the oracle on the values the bytes and their block scales stand for
    ref = R.gdpa_fwd(dequant_mx(q8, qs), dequant_mx(k8, ks), inp.f64("v"), inp.q_off, inp.kv_off, act, inp.window)
    return o.float().cpu().numpy(), ref, n_parts


@pytest.mark.parametrize("d,team,nb", [l for l in FWD_LAYOUTS if l[0] >= 64])
def test_mx_forward_layouts(d, team, nb):
    say(f"MX forward d={d} team={team} blocks={nb}")
    inp = make_from_lengths(JFA_LQ, JFA_LK, 2, d, act="silu", seed=75, device=DEV)
    o, ref, _ = run_mx_fwd(inp, team=(team, 0, 0), blocks=(nb, 0, 0))
    check_close(o, ref, f"MX O d={d}")
    o32, ref, _ = run_mx_fwd(inp, dtype="bf16_f32out", team=(team, 0, 0), blocks=(nb, 0, 0))
    check_close(o32, ref, f"MX O f32out d={d}")


@pytest.mark.parametrize("act", ["gelu", "identity"])
@pytest.mark.parametrize("window", [0, 17])
def test_mx_forward_acts_windows(act, window):
    say(f"MX forward act={act} window={window}")
    L = [1, 31, 32, 33, 127, 300, 0, 65]
    inp = make_from_lengths(L, L, 2, 128, act=act, window=window, seed=76, device=DEV)
    # rows of very different scales: the block scales follow them
    g = torch.Generator(device=DEV).manual_seed(9)
    inp.q.mul_(torch.exp(torch.randn((inp.q.shape[0], 2, 1), generator=g, device=DEV) * 2).to(inp.q.dtype))
    o, ref, _ = run_mx_fwd(inp)
    check_close(o, ref, f"MX O act={act} window={window}")


@pytest.mark.parametrize("d", [64, 128])
def test_mx_forward_block_scales(d):
    """Scale blocks of one row whose magnitudes differ by 2^8 or more (q: block
    factors 2^-6, 2^4, 2^-2, 2^6; k: 2^3, 2^-5, 2^5, 2^-1): a scale applied to the
    wrong 32 columns moves O far outside the tolerance."""
    say(f"MX forward, block scales far apart, d={d}")
    L = [33, 1, 70, 31, 128]
    inp = make_from_lengths(L, L[::-1], 2, d, act="gelu", seed=79, device=DEV)
    nb = d // 32
    fq = torch.tensor([2.0 ** e for e in (-6, 4, -2, 6)[:nb]], device=DEV).repeat_interleave(32)
    fk = torch.tensor([2.0 ** e for e in (3, -5, 5, -1)[:nb]], device=DEV).repeat_interleave(32)
    inp.q.mul_(fq.to(inp.q.dtype))
    inp.k.mul_(fk.to(inp.k.dtype))
    _, qs = quant_mx(inp.q)
    _, ks = quant_mx(inp.k)
    # in every row, the two scale blocks of each 64-column MFMA block are >= 6 octaves apart
    assert int((qs[..., 0::2].int() - qs[..., 1::2].int()).abs().min()) >= 6
    assert int((ks[..., 0::2].int() - ks[..., 1::2].int()).abs().min()) >= 4
    o, ref, _ = run_mx_fwd(inp)
    check_close(o, ref, f"MX O block scales d={d}")


def test_mx_forward_cut_items():
    inp = make_from_lengths([32, 1], [3000, 5], 2, 64, act="gelu", seed=77, device=DEV)
    o, ref, n_parts = run_mx_fwd(inp, bins=(16, 16, 16))
    assert n_parts[0] > 0
    check_close(o, ref, "MX O cut")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_mx_forward_against_bf16_inputs(cfg):
    """The MX forward against the oracle on the quantised values (the kernel's arithmetic)
    and on the bf16 inputs (within the stated fp8 bounds)."""
    say(f"cfg{cfg} MX forward, B={SMALL_B[cfg]}")
    inp = make_workload(cfg, device=DEV, B=SMALL_B[cfg])
    o, ref_q, _ = run_mx_fwd(inp)
    check_close(o, ref_q, f"cfg{cfg} MX O vs the quantised values")
    check_fp8(o, oracle_fwd(inp), f"cfg{cfg} MX O vs the bf16 inputs")


def test_mx_forward_rejects():
    for d, dtype, act in ((32, "bf16", "gelu"), (64, "f32", "gelu"), (64, "bf16", "one")):
        inp = make_from_lengths([40, 3], [50, 7], 2, d, act="gelu", seed=78, device=DEV)
        qo, ko = dev_offsets(inp)
        b8 = torch.zeros(inp.q.shape, dtype=torch.uint8, device=DEV)
        k8 = torch.zeros(inp.k.shape, dtype=torch.uint8, device=DEV)
        sc = torch.full((2, 60, max(d // 32, 1)), 127, dtype=torch.uint8, device=DEV)
        with G.Plan(inp.q_off, inp.kv_off, 2, d, 0, dtype) as plan:
            with pytest.raises(G.GdpaError) as e:
                G.gdpa_mx_fwd(plan.handle, b8, sc, k8, sc, inp.v, qo, ko, 2, 2, d, act, 0, torch.empty_like(inp.q))
            assert G.STATUS[e.value.status] == "GDPA_ERR_UNSUPPORTED", (d, dtype, act)


# ---------------------------------------------------------------------------
# fp8 (e4m3fn) Q, K and dO in the backward (V bf16)
# ---------------------------------------------------------------------------

def run_fp8_bwd(inp, act=None, dtype="bf16", **opts):
    """gdpa_fp8_bwd on per-tensor e4m3 Q, K, dO; the oracle on the values the bytes stand for."""
    act = act or inp.act
    qo, ko = dev_offsets(inp)
    q8, sq = quant_e4m3(inp.q)
    k8, sk = quant_e4m3(inp.k)
    o8, so = quant_e4m3(inp.do)
    odt = torch.float32 if dtype == "bf16_f32out" else torch.bfloat16
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, dtype, **opts) as plan:
        dq = torch.empty(inp.q.shape, dtype=odt, device=DEV)
        dk = torch.empty(inp.k.shape, dtype=odt, device=DEV)
        dv = torch.empty(inp.v.shape, dtype=odt, device=DEV)
        G.gdpa_fp8_bwd(plan.handle, q8.view(torch.uint8).to(DEV), k8.view(torch.uint8).to(DEV), inp.v,
                       o8.view(torch.uint8).to(DEV), qo, ko, plan.B, inp.H, inp.d, act, inp.window, sq, sk, so,
                       dq, dk, dv)
        torch.cuda.synchronize()
        st = plan.stats()
    ref = R.gdpa_bwd(q8.double().numpy() * sq, k8.double().numpy() * sk, inp.f64("v"), o8.double().numpy() * so,
                     inp.q_off, inp.kv_off, act, inp.window)
    return tuple(t.float().cpu().numpy() for t in (dq, dk, dv)), ref, st


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("case", range(len(FUSED_CASES)))
def test_fp8_backward_one_pass(d, case):
    """Both one-pass shapes (KV- and Q-stationary), windows, empty and one-row samples,
    bf16 and fp32 outputs."""
    lq, lk, window = FUSED_CASES[case]
    say(f"fp8 backward d={d} case={case}")
    inp = make_from_lengths(lq, lk, 3, d, act="gelu", window=window, seed=81 + case, device=DEV)
    for dtype in ("bf16", "bf16_f32out"):
        got, ref, st = run_fp8_bwd(inp, dtype=dtype)
        assert st["bwd_fused"] == (1 if case != 1 else 2)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            check_close(a, b, f"fp8 {name} d={d} case={case} {dtype}")


@pytest.mark.parametrize("window", [0, 17])
@pytest.mark.parametrize("bins", [(0, 0, 0), (64, 64, 64)])   # 64: the 700-row sample's items are cut
@pytest.mark.parametrize("dtype", ["bf16", "bf16_f32out"])
@pytest.mark.parametrize("team", [1, 2])
def test_fp8_backward_stored_ds(window, bins, dtype, team):
    """d = 128 plans whose backward is the 16-row dK/dV kernel storing dS and dQ from
    the stored blocks: ragged lengths across tile edges, windows, cut items (few
    bins), fp32 outputs, 32- and 64-row dK/dV items."""
    say(f"fp8 backward stored dS window={window} bins={bins} {dtype} team={team}")
    L = [1, 15, 16, 17, 33, 47, 64, 65, 0, 300, 129, 700]
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=window, seed=93 + window, device=DEV)
    got, ref, st = run_fp8_bwd(inp, dtype=dtype, bins=bins, team=(0, team, 0))
    assert st["bwd_fused"] == 0 and st["ds_bytes"] > 0
    if bins[0]:
        assert sum(st["n_parts"]) > 0
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        check_close(a, b, f"fp8 {name} stored dS window={window} bins={bins} {dtype} team={team}")


@pytest.mark.parametrize("act", ["silu", "identity", "gelu_taylor6"])
def test_fp8_backward_acts(act):
    say(f"fp8 backward act={act}")
    for case in (0, 1):
        lq, lk, _ = FUSED_CASES[case]
        inp = make_from_lengths(lq, lk, 2, 64, act=act, seed=85 + case, device=DEV)
        got, ref, _ = run_fp8_bwd(inp)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            check_close(a, b, f"fp8 {name} act={act} case={case}")


@pytest.mark.parametrize("case", [0, 2])
def test_fp8_backward_cut_items(case):
    """Items longer than a mean bin, cut into chunks whose fp32 partials the reduction
    scales by the gradients' fp8 factors."""
    lq, lk, bins, _, fused = CHUNK_CASES[case]
    say(f"fp8 backward cut items case={case}")
    inp = make_from_lengths(lq, lk, 2, 64, act="gelu", seed=87 + case, device=DEV)
    got, ref, st = run_fp8_bwd(inp, bins=bins)
    assert st["bwd_fused"] == fused and sum(st["n_parts"]) > 0
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        check_close(a, b, f"fp8 {name} cut case={case}")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fp8_backward_against_bf16_inputs(cfg):
    """The fp8 backward against the oracle on the quantised values (the kernels'
    arithmetic) and on the bf16 inputs (within the stated fp8 bounds), on the four
    bf16 workloads (one-pass or stored-dS backward)."""
    say(f"cfg{cfg} fp8 backward, B={SMALL_B[cfg]}")
    inp = make_workload(cfg, device=DEV, B=SMALL_B[cfg])
    got, ref_q, st = run_fp8_bwd(inp)
    assert st["bwd_fused"] in (1, 2) or st["ds_bytes"] > 0
    for name, a, b, c in zip(("dQ", "dK", "dV"), got, ref_q, oracle_bwd(inp)):
        check_close(a, b, f"cfg{cfg} fp8 {name} vs the quantised values")
        check_fp8(a, c, f"cfg{cfg} fp8 {name} vs the bf16 inputs")


def test_fp8_backward_rejects():
    lq, lk = [40, 3], [50, 7]   # neither side within one tile: two-kernel backward
    inp = make_from_lengths(lq, lk, 2, 64, act="gelu", seed=89, device=DEV)
    qo, ko = dev_offsets(inp)
    q8 = torch.zeros(inp.q.shape, dtype=torch.uint8, device=DEV)
    k8 = torch.zeros(inp.k.shape, dtype=torch.uint8, device=DEV)
    o8 = torch.zeros(inp.q.shape, dtype=torch.uint8, device=DEV)
    g = [torch.empty_like(t) for t in (inp.q, inp.k, inp.v)]
    with G.Plan(inp.q_off, inp.kv_off, 2, 64, 0, "bf16") as plan:
        assert plan.stats()["bwd_fused"] == 0
        with pytest.raises(G.GdpaError) as e:
            G.gdpa_fp8_bwd(plan.handle, q8, k8, inp.v, o8, qo, ko, 2, 2, 64, "gelu", 0, 1.0, 1.0, 1.0, *g)
        assert G.STATUS[e.value.status] == "GDPA_ERR_UNSUPPORTED"
    one = make_from_lengths([40, 3], [32, 7], 2, 64, act="gelu", seed=89, device=DEV)
    qo, ko = dev_offsets(one)
    k8 = torch.zeros(one.k.shape, dtype=torch.uint8, device=DEV)
    g = [torch.empty_like(t) for t in (one.q, one.k, one.v)]
    with G.Plan(one.q_off, one.kv_off, 2, 64, 0, "bf16") as plan:
        assert plan.stats()["bwd_fused"] == 1
        for act, scales, status in (("one", (1.0, 1.0, 1.0), "GDPA_ERR_UNSUPPORTED"),
                                    ("gelu", (0.0, 1.0, 1.0), "GDPA_ERR_INVALID_ARG"),
                                    ("gelu", (1.0, float("inf"), 1.0), "GDPA_ERR_INVALID_ARG"),
                                    ("gelu", (1.0, 1.0, -1.0), "GDPA_ERR_INVALID_ARG")):
            with pytest.raises(G.GdpaError) as e:
                G.gdpa_fp8_bwd(plan.handle, q8, k8, one.v, o8, qo, ko, 2, 2, 64, act, 0, *scales, *g)
            assert G.STATUS[e.value.status] == status
    with G.Plan(one.q_off, one.kv_off, 2, 64, 0, "f32") as plan:
        with pytest.raises(G.GdpaError) as e:
            G.gdpa_fp8_bwd(plan.handle, q8, k8, one.v, o8, qo, ko, 2, 2, 64, "gelu", 0, 1.0, 1.0, 1.0, *g)
        assert G.STATUS[e.value.status] == "GDPA_ERR_UNSUPPORTED"


def test_fp8_forward_rejects():
    inp = make_from_lengths([40, 3], [50, 7], 2, 64, act="gelu", seed=74, device=DEV)
    qo, ko = dev_offsets(inp)
    b8 = torch.zeros(inp.q.shape, dtype=torch.uint8, device=DEV)
    k8 = torch.zeros(inp.k.shape, dtype=torch.uint8, device=DEV)
    o = torch.empty_like(inp.q)
    for dtype, act, sq, status in (("f32", "gelu", 1.0, "GDPA_ERR_UNSUPPORTED"), ("bf16", "one", 1.0,
                                   "GDPA_ERR_UNSUPPORTED"), ("bf16", "gelu", 0.0, "GDPA_ERR_INVALID_ARG"),
                                   ("bf16", "gelu", float("nan"), "GDPA_ERR_INVALID_ARG")):
        with G.Plan(inp.q_off, inp.kv_off, 2, 64, 0, dtype) as plan:
            with pytest.raises(G.GdpaError) as e:
                G.gdpa_fp8_fwd(plan.handle, b8, k8, inp.v, qo, ko, 2, 2, 64, act, 0, sq, 1.0, o)
            assert G.STATUS[e.value.status] == status, (dtype, act, sq)


# ---------------------------------------------------------------------------
# RMSNorm prologue: GDPA on normalised Q, K, V from the raw tensors
# ---------------------------------------------------------------------------

def run_norm(inp, norm, act=None, **opts):
    """gdpa_norm_fwd then gdpa_norm_bwd on one plan: (O, dQ, dK, dV, rstd) as numpy."""
    act = act or inp.act
    qo, ko = dev_offsets(inp)
    Tq, Tk = inp.q.shape[0], inp.k.shape[0]
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16", **opts) as plan:
        rstd = torch.full((inp.H * (Tq + 2 * Tk),), float("nan"), device=DEV)
        o = torch.empty_like(inp.q)
        dq, dk, dv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)
        args = (plan.handle, inp.q, inp.k, inp.v)
        G.gdpa_norm_rstd(*args, inp.H, inp.d, norm, rstd)
        G.gdpa_norm_fwd(*args, qo, ko, plan.B, inp.H, inp.d, act, inp.window, norm, rstd, o)
        G.gdpa_norm_bwd(*args, inp.do, qo, ko, plan.B, inp.H, inp.d, act, inp.window, norm, rstd, dq, dk, dv)
        torch.cuda.synchronize()
        n_parts = plan.stats()["n_parts"]
    return tuple(t.float().cpu().numpy() for t in (o, dq, dk, dv, rstd)) + (n_parts,)


def check_norm(got, inp, norm, act, what):
    o, dq, dk, dv, rstd = got[:5]
    args = (inp.f64("q"), inp.f64("k"), inp.f64("v"))
    check_close(o, R.norm_gdpa_fwd(*args, inp.q_off, inp.kv_off, act, inp.window, norm), f"norm O {what}")
    ref = R.norm_gdpa_bwd(*args, inp.f64("do"), inp.q_off, inp.kv_off, act, inp.window, norm)
    for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        check_close(a, b, f"norm {name} {what}")
    # the pre-pass: 1/rms per (head, row), [H, Tq] then [H, Tk, 2]; 1 where not normalised
    H, Tq, Tk = inp.H, inp.q.shape[0], inp.k.shape[0]
    inv = lambda x, on: (1.0 / np.sqrt(np.mean(x * x, -1) + R.RMS_EPS)).T if on else np.ones((H, x.shape[0]))
    want = np.concatenate([inv(args[0], "q" in norm).ravel(),
                           np.stack([inv(args[1], "k" in norm), inv(args[2], "v" in norm)], -1).ravel()])
    np.testing.assert_allclose(rstd, want, rtol=2e-6, err_msg=f"rstd {what}")


NORM_LAYOUTS = [(32, 1, 1, 1, 1), (32, 1, 2, 1, 2), (64, 1, 1, 1, 1), (64, 1, 2, 1, 2),
                (128, 1, 1, 1, 1), (128, 1, 2, 1, 2), (128, 2, 1, 2, 1)]


@pytest.mark.parametrize("d,tf,nb,tb,nbq", NORM_LAYOUTS)
def test_norm_prologue_layouts(d, tf, nb, tb, nbq):
    """Every forward layout, and the dQ / dK-dV layouts, with Q, K, V normalised."""
    say(f"norm prologue d={d} fwd {tf}x{nb} dq {tb}x{nbq} dkdv {tb}x1")
    inp = make_from_lengths(JFA_LQ, JFA_LK, 2, d, act="silu", rms="", row_spread=1.0, seed=61, device=DEV)
    got = run_norm(inp, "qkv", team=(tf, tb, tb if nbq == 1 else 1), blocks=(nb, 1, nbq))
    check_norm(got, inp, "qkv", "silu", f"d={d}")


@pytest.mark.parametrize("norm", ["q", "kv", "qk", ""])
@pytest.mark.parametrize("act", ["gelu", "identity"])
def test_norm_prologue_subsets(norm, act):
    say(f"norm prologue norm={norm!r} act={act}")
    inp = make_from_lengths(JFA_LQ, JFA_LK, 2, 64, act=act, rms="", row_spread=1.0, seed=62, device=DEV)
    check_norm(run_norm(inp, norm), inp, norm, act, f"norm={norm!r} act={act}")


@pytest.mark.parametrize("window", [1, 17, 128])
def test_norm_prologue_windows(window):
    say(f"norm prologue window={window}")
    L = [1, 31, 32, 33, 127, 300, 0, 65]
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=window, rms="", row_spread=1.0, seed=63, device=DEV)
    check_norm(run_norm(inp, "qkv"), inp, "qkv", "gelu", f"window={window}")


def test_norm_backward_parts_match_whole():
    """gdpa_norm_bwd_dkdv then gdpa_norm_bwd_dq give gdpa_norm_bwd's outputs bit for bit."""
    inp = make_from_lengths(JFA_LQ, JFA_LK, 2, 128, act="gelu", rms="", row_spread=1.0, seed=65, device=DEV)
    whole = run_norm(inp, "qkv")
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, 0, "bf16") as plan:
        rstd = torch.tensor(whole[4], device=DEV)
        dq, dk, dv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)
        args = (plan.handle, inp.q, inp.k, inp.v, inp.do, qo, ko, plan.B, inp.H, inp.d, "gelu", 0, "qkv", rstd)
        G.gdpa_norm_bwd_dkdv(*args, dk, dv)
        G.gdpa_norm_bwd_dq(*args, dq)
        torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), whole[1:4]):
        assert np.array_equal(a.float().cpu().numpy(), b), name


def test_norm_prologue_rejects():
    inp = make_from_lengths([40, 3], [50, 7], 2, 64, act="gelu", rms="", seed=66, device=DEV)
    qo, ko = dev_offsets(inp)
    rstd = torch.empty(2 * (43 + 2 * 57), device=DEV)
    o = torch.empty_like(inp.q)
    cases = (("f32", "gelu", 7, rstd, "GDPA_ERR_UNSUPPORTED"), ("bf16", "one", 7, rstd, "GDPA_ERR_UNSUPPORTED"),
             ("bf16", "gelu", 8, rstd, "GDPA_ERR_INVALID_ARG"), ("bf16", "gelu", 7, None, "GDPA_ERR_INVALID_ARG"))
    for dtype, act, norm, buf, status in cases:
        with G.Plan(inp.q_off, inp.kv_off, 2, 64, 0, dtype) as plan:
            with pytest.raises(G.GdpaError) as e:
                G.gdpa_norm_fwd(plan.handle, inp.q, inp.k, inp.v, qo, ko, 2, 2, 64, act, 0, norm, buf, o)
            assert G.STATUS[e.value.status] == status, (dtype, act, norm)


def test_norm_prologue_cut_items():
    """Chunks take the norm's gradient separately: it is linear in the normalised
    row's gradient, so the partial sums still add up."""
    say("norm prologue with cut items")
    inp = make_from_lengths([32, 3000, 1], [3000, 40, 5], 2, 64, act="silu", rms="", row_spread=1.0, seed=64,
                            device=DEV)
    got = run_norm(inp, "qkv", bins=(16, 16, 16))
    assert got[5][0] > 0 and got[5][1] > 0 and got[5][2] > 0, got[5]
    check_norm(got, inp, "qkv", "silu", "cut")


# ---------------------------------------------------------------------------
# JFA: jagged softmax attention through the same kernels
# ---------------------------------------------------------------------------

def run_jfa_fwd(inp, dtype="bf16", **opts):
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, dtype, **opts) as plan:
        o = torch.empty(inp.q.shape, dtype=torch.float32 if dtype == "bf16_f32out" else torch.bfloat16, device=DEV)
        lse = torch.empty((inp.H, inp.q.shape[0]), dtype=torch.float32, device=DEV)
        G.gdpa_jfa_fwd(plan.handle, inp.q, inp.k, inp.v, qo, ko, plan.B, inp.H, inp.d, inp.window, o, lse)
        torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check_lse(got, ref, what):
    """Row log-sum-exp: -inf exactly where the oracle has no valid key, else within 1e-3."""
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf rows differ"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(got[fin])), f"{what}: non-finite LSE"
    err = float(np.max(np.abs(got[fin] - ref[fin]), initial=0.0))
    assert err <= 1e-3, f"{what}: max LSE error {err:.2e}"


JFA_LQ = [5, 0, 70, 1, 33, 200, 31, 96, 7]
JFA_LK = [64, 3, 0, 2, 129, 31, 300, 96, 1]


@pytest.mark.parametrize("d,team,nb", FWD_LAYOUTS)
def test_jfa_forward_layouts(d, team, nb):
    say(f"JFA forward d={d} team={team} blocks={nb}")
    inp = make_from_lengths(JFA_LQ, JFA_LK, 2, d, act="gelu", seed=51, device=DEV)
    o, lse = run_jfa_fwd(inp, team=(team, 0, 0), blocks=(nb, 0, 0))
    ro, rl = R.jfa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, 0)
    check_close(o, ro, f"JFA O d={d}")
    check_lse(lse, rl, f"JFA LSE d={d}")
    o32, lse32 = run_jfa_fwd(inp, dtype="bf16_f32out", team=(team, 0, 0), blocks=(nb, 0, 0))
    check_close(o32, ro, f"JFA O f32out d={d}")


@pytest.mark.parametrize("window", [1, 2, 17, 128])
def test_jfa_forward_windows(window):
    say(f"JFA forward window={window}")
    L = [1, 31, 32, 33, 127, 300, 0, 65]
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=window, seed=52, device=DEV)
    o, lse = run_jfa_fwd(inp)
    ro, rl = R.jfa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, window)
    check_close(o, ro, f"JFA O window={window}")
    check_lse(lse, rl, f"JFA LSE window={window}")


JFA_CUT_CASES = [   # (lq, lk, d, window, team, nb): long rows of kv tiles cut into chunks
    ([32, 1], [3000, 5], 64, 0, 1, 1),
    ([32, 40, 3, 64], [2500, 700, 0, 1800], 128, 0, 2, 1),
    ([96, 17], [2000, 33], 32, 0, 1, 2),
    ([300, 5], [300, 5], 128, 100, 1, 1),
]


@pytest.mark.parametrize("case", range(len(JFA_CUT_CASES)))
def test_jfa_forward_cut_items(case):
    """A cut item's chunks keep unnormalised rows with their max and sum; the combine
    rescales them to the common max (also the LSE of those rows)."""
    lq, lk, d, window, team, nb = JFA_CUT_CASES[case]
    say(f"JFA forward cut items case={case}")
    inp = make_from_lengths(lq, lk, 2, d, act="gelu", window=window, seed=53 + case, device=DEV)
    opts = dict(bins=(16, 16, 16), team=(team, 0, 0), blocks=(nb, 0, 0))
    with G.Plan(inp.q_off, inp.kv_off, 2, d, window, "bf16", **opts) as plan:
        assert plan.stats()["n_parts"][0] > 0
    ro, rl = R.jfa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, window)
    o, lse = run_jfa_fwd(inp, **opts)
    check_close(o, ro, f"JFA O cut case={case}")
    check_lse(lse, rl, f"JFA LSE cut case={case}")
    o32, lse32 = run_jfa_fwd(inp, dtype="bf16_f32out", **opts)
    check_close(o32, ro, f"JFA O f32out cut case={case}")
    check_lse(lse32, rl, f"JFA LSE f32out cut case={case}")
    ow, lw = run_jfa_fwd(inp, split=False, team=(team, 0, 0), blocks=(nb, 0, 0))
    check_close(ow, ro, f"JFA O whole items case={case}")


def run_jfa_bwd(inp, dtype="bf16", **opts):
    """JFA forward on a whole-item plan, then the JFA backward on a plan with `opts`:
    (dQ, dK, dV, O, LSE, stat) as numpy."""
    qo, ko = dev_offsets(inp)
    Tq = inp.q.shape[0]
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16") as pf:
        o = torch.empty_like(inp.q)
        lse = torch.empty((inp.H, Tq), dtype=torch.float32, device=DEV)
        G.gdpa_jfa_fwd(pf.handle, inp.q, inp.k, inp.v, qo, ko, pf.B, inp.H, inp.d, inp.window, o, lse)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, dtype, **opts) as plan:
        odt = torch.float32 if dtype == "bf16_f32out" else torch.bfloat16
        dq = torch.empty(inp.q.shape, dtype=odt, device=DEV)
        dk = torch.empty(inp.k.shape, dtype=odt, device=DEV)
        dv = torch.empty(inp.v.shape, dtype=odt, device=DEV)
        stat = torch.empty((inp.H, Tq, 2), dtype=torch.float32, device=DEV)
        G.gdpa_jfa_bwd(plan.handle, inp.q, inp.k, inp.v, o, lse, inp.do, qo, ko, plan.B, inp.H, inp.d,
                       inp.window, stat, dq, dk, dv)
        torch.cuda.synchronize()
        n_parts = plan.stats()["n_parts"]
    out = tuple(t.float().cpu().numpy() for t in (dq, dk, dv, o, lse, stat))
    return out + (n_parts,)


def check_jfa_grads(got, inp, what, floor=(0.0, 0.0, 0.0)):
    ref = R.jfa_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"), inp.q_off, inp.kv_off, inp.window)
    for name, a, b, f in zip(("dQ", "dK", "dV"), got[:3], ref, floor):
        check_close(a, b, f"JFA {name} {what}", floor=f)


def check_jfa_stat(got, inp, what):
    """The pre-pass: (LSE log2 e, sum dO * O) per (head, row) from the forward's own O, LSE."""
    o, lse, stat = got[3], got[4], got[5]
    do = inp.f64("do")
    dref = np.einsum("thc,thc->ht", do, o.astype(np.float64))
    fin = np.isfinite(lse)
    assert np.array_equal(stat[..., 0][~fin], lse[~fin]), f"{what}: -inf rows"
    assert np.allclose(stat[..., 0][fin], lse[fin] * np.float32(1.4426950408889634), rtol=1e-6, atol=1e-6), what
    scale = float(np.max(np.abs(dref), initial=0.0)) + 1e-30
    assert float(np.max(np.abs(stat[..., 1] - dref), initial=0.0)) <= 1e-5 * scale, f"{what}: D"


JFA_BWD_LAYOUTS = [(32, 1), (32, 2), (64, 1), (64, 2), (128, 1), (128, 2)]


@pytest.mark.parametrize("d,nb", JFA_BWD_LAYOUTS)
def test_jfa_backward_layouts(d, nb):
    say(f"JFA backward d={d} dq blocks={nb}")
    inp = make_from_lengths(JFA_LQ, JFA_LK, 2, d, act="gelu", seed=54, device=DEV)
    got = run_jfa_bwd(inp, team=(0, 1, 1), blocks=(0, 1, nb))
    check_jfa_stat(got, inp, f"d={d}")
    check_jfa_grads(got, inp, f"d={d} nb={nb}")


@pytest.mark.parametrize("window", [1, 2, 17, 128])
def test_jfa_backward_windows(window):
    say(f"JFA backward window={window}")
    L = [1, 31, 32, 33, 127, 300, 0, 65]
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=window, seed=55, device=DEV)
    floor = (0.0, 0.0, 0.0)
    if window == 1:
        # every row attends to its own key only: P = 1, dS = dO.v - dO.o = 0 exactly, so
        # dQ = dK = 0 and the bound is the fp32 rounding of that cancellation (two
        # d-term dot products, each within d 2^-24 max|dO| max|V|), times |K| or |Q| / sqrt(d)
        mag = lambda n: float(np.max(np.abs(inp.f64(n))))
        e = 2 * inp.d * 2.0 ** -24 * mag("do") * mag("v") / math.sqrt(inp.d)
        floor = (e * mag("k"), e * mag("q"), 0.0)
    check_jfa_grads(run_jfa_bwd(inp), inp, f"window={window}", floor)


def test_jfa_backward_cut_items():
    """Long rows of tiles cut into chunks in both gradient lists: the chunk partials
    are linear in the steps once LSE and D are fixed."""
    say("JFA backward with cut items")
    inp = make_from_lengths([32, 3000, 1], [3000, 40, 5], 2, 64, act="gelu", seed=56, device=DEV)
    got = run_jfa_bwd(inp, bins=(16, 16, 16))
    assert got[6][1] > 0 and got[6][2] > 0, got[6]
    check_jfa_grads(got, inp, "cut")


def test_jfa_backward_parts_match_whole():
    """gdpa_jfa_bwd_dq then gdpa_jfa_bwd_dkdv give gdpa_jfa_bwd's outputs bit for bit; with
    stat from the pre-pass (gdpa_jfa_bwd_stat) dK/dV may run first, to rounding."""
    say("JFA backward in parts")
    inp = make_from_lengths(JFA_LQ, JFA_LK, 2, 128, act="gelu", seed=58, device=DEV)
    whole = run_jfa_bwd(inp)
    qo, ko = dev_offsets(inp)
    o = torch.tensor(whole[3], dtype=torch.bfloat16, device=DEV)
    lse = torch.tensor(whole[4], device=DEV)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, 0, "bf16") as plan:
        args = (plan.handle, inp.q, inp.k, inp.v)
        stat = torch.full((inp.H, inp.q.shape[0], 2), float("nan"), device=DEV)
        dq, dk, dv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)
        G.gdpa_jfa_bwd_dq(*args, o, lse, inp.do, qo, ko, plan.B, inp.H, inp.d, 0, stat, dq)
        G.gdpa_jfa_bwd_dkdv(*args, inp.do, qo, ko, plan.B, inp.H, inp.d, 0, stat, dk, dv)
        # the pre-pass route: stat first, dK/dV before dQ
        stat2 = torch.full_like(stat, float("nan"))
        dk2, dv2 = torch.empty_like(inp.k), torch.empty_like(inp.v)
        G.gdpa_jfa_bwd_stat(plan.handle, o, lse, inp.do, inp.H, inp.d, stat2)
        G.gdpa_jfa_bwd_dkdv(*args, inp.do, qo, ko, plan.B, inp.H, inp.d, 0, stat2, dk2, dv2)
        torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV", "stat"), (dq, dk, dv, stat), (whole[0], whole[1], whole[2], whole[5])):
        assert np.array_equal(a.float().cpu().numpy(), b, equal_nan=True), name
    s1, s2 = stat.cpu().numpy(), stat2.cpu().numpy()
    assert np.array_equal(s1[..., 0], s2[..., 0])   # the same LSE log2(e) product
    np.testing.assert_allclose(s2[..., 1], s1[..., 1], rtol=1e-5, atol=1e-5 * np.abs(s1[..., 1]).max())
    ref = R.jfa_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"), inp.q_off, inp.kv_off, 0)
    check_close(dk2.float().cpu().numpy(), ref[1], "JFA dK after the pre-pass")
    check_close(dv2.float().cpu().numpy(), ref[2], "JFA dV after the pre-pass")


# every Lk <= 32 (and Lk > 0 where Lq > 0): gdpa_jfa_bwd runs one KV-stationary pass;
# every Lq <= 32 instead: the two kernels
JFA_ONE_PASS = [
    # (lq, lk, window, bwd_fused)
    ([5, 0, 70, 1, 33, 200, 31, 96, 7], [32, 3, 5, 2, 29, 31, 1, 32, 17], 0, 1),
    ([1, 31, 32, 17, 5, 0], [1, 31, 32, 17, 5, 0], 4, 1),
    ([1, 31, 32, 17, 5], [1, 31, 32, 17, 5], 17, 1),
    ([1, 31, 32, 17, 5], [1, 31, 32, 17, 5], 1, 1),
    ([32, 32, 7], [300, 1000, 65], 0, 2),
]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("case", range(len(JFA_ONE_PASS)))
def test_jfa_backward_one_pass(d, case):
    """The one-pass JFA backward (D = sum_j P dP in the KV-stationary pass); against the
    oracle, and the two-kernel path on the same inputs; it reads neither O nor stat.
    A plan whose one-pass backward would be Q-stationary runs the two kernels."""
    lq, lk, window, fused = JFA_ONE_PASS[case]
    say(f"JFA one-pass backward d={d} case={case}")
    inp = make_from_lengths(lq, lk, 2, d, act="gelu", window=window, seed=60 + case, device=DEV)
    with G.Plan(inp.q_off, inp.kv_off, 2, d, window, "bf16") as plan:
        assert plan.stats()["bwd_fused"] == fused
    floor = (0.0, 0.0, 0.0)
    if window == 1:   # dQ = dK = 0 exactly; the fp32 rounding of dO.v - D bounds them
        mag = lambda n: float(np.max(np.abs(inp.f64(n))))
        e = 2 * inp.d * 2.0 ** -24 * mag("do") * mag("v") / math.sqrt(inp.d)
        floor = (e * mag("k"), e * mag("q"), 0.0)
    one = run_jfa_bwd(inp)
    check_jfa_grads(one, inp, f"one pass d={d} case={case}", floor)
    two = run_jfa_bwd(inp, unfused=True)
    check_jfa_grads(two, inp, f"two kernels d={d} case={case}", floor)
    # cut items (few bins): dK, dV from chunk partials
    cut = run_jfa_bwd(inp, bins=(2, 2, 2))
    check_jfa_grads(cut, inp, f"one pass, cut items d={d} case={case}", floor)
    if fused != 1:
        return
    # neither O nor stat is needed
    qo, ko = dev_offsets(inp)
    lse = torch.tensor(one[4], device=DEV)
    o = None
    with G.Plan(inp.q_off, inp.kv_off, 2, d, window, "bf16") as plan:
        dq, dk, dv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)
        G.gdpa_jfa_bwd(plan.handle, inp.q, inp.k, inp.v, o, lse, inp.do, qo, ko, plan.B, 2, d, window, None,
                       dq, dk, dv)
        torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), one[:3]):
        assert np.array_equal(a.float().cpu().numpy(), b), f"{name}: without O and stat"


def test_jfa_backward_rejects():
    inp = make_from_lengths([40, 3], [50, 7], 2, 128, act="gelu", seed=57, device=DEV)
    qo, ko = dev_offsets(inp)
    z = torch.zeros((2, 43, 2), dtype=torch.float32, device=DEV)
    for dtype, opts in (("bf16", dict(team=(0, 2, 1))), ("bf16", dict(team=(0, 1, 2))), ("f32", {})):
        with G.Plan(inp.q_off, inp.kv_off, 2, 128, 0, dtype, **opts) as plan:
            with pytest.raises(G.GdpaError) as e:
                G.gdpa_jfa_bwd(plan.handle, inp.q, inp.k, inp.v, inp.q, z, inp.do, qo, ko, 2, 2, 128, 0, z,
                               torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v))
            assert G.STATUS[e.value.status] == "GDPA_ERR_UNSUPPORTED"


def test_jfa_backward_rejects_fp32_output_plans():
    """On a GDPA_BF16_F32OUT plan the JFA forward writes fp32 O, which the backward
    (reading O as bf16) would misread: every JFA backward entry point refuses such a
    plan before launching anything, after the forward on the same plan ran."""
    say("JFA backward on an fp32-output plan")
    inp = make_from_lengths([40, 3], [50, 7], 2, 128, act="gelu", seed=59, device=DEV)
    qo, ko = dev_offsets(inp)
    Tq = inp.q.shape[0]
    with G.Plan(inp.q_off, inp.kv_off, 2, 128, 0, "bf16_f32out") as plan:
        o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
        lse = torch.empty((2, Tq), dtype=torch.float32, device=DEV)
        G.gdpa_jfa_fwd(plan.handle, inp.q, inp.k, inp.v, qo, ko, plan.B, 2, 128, 0, o, lse)
        torch.cuda.synchronize()
        ro, _ = R.jfa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, 0)
        check_close(o.cpu().numpy(), ro, "JFA O on the fp32-output plan")
        stat = torch.empty((2, Tq, 2), dtype=torch.float32, device=DEV)
        g = [torch.empty(t.shape, dtype=torch.float32, device=DEV) for t in (inp.q, inp.k, inp.v)]
        calls = (
            lambda: G.gdpa_jfa_bwd(plan.handle, inp.q, inp.k, inp.v, o, lse, inp.do, qo, ko, plan.B, 2, 128, 0, stat,
                                   *g),
            lambda: G.gdpa_jfa_bwd_dq(plan.handle, inp.q, inp.k, inp.v, o, lse, inp.do, qo, ko, plan.B, 2, 128, 0,
                                      stat, g[0]),
            lambda: G.gdpa_jfa_bwd_dkdv(plan.handle, inp.q, inp.k, inp.v, inp.do, qo, ko, plan.B, 2, 128, 0, stat,
                                        g[1], g[2]),
            lambda: G.gdpa_jfa_bwd_stat(plan.handle, o, lse, inp.do, 2, 128, stat),
        )
        for call in calls:
            with pytest.raises(G.GdpaError) as e:
                call()
            assert G.STATUS[e.value.status] == "GDPA_ERR_UNSUPPORTED"


# ---------------------------------------------------------------------------
# pFFN as GDPA: every query row against the same M weight rows
# ---------------------------------------------------------------------------

def run_pffn(inp, act, **opts):
    Tq, M = int(inp.q_off[-1]), int(inp.kv_off[-1])
    h = G.gdpa_pffn_plan_create(Tq, M, inp.H, inp.d, "bf16", **opts)
    try:
        st = G.gdpa_plan_stats(h)
        o = torch.empty_like(inp.q)
        dq, dwk, dwv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)
        G.gdpa_pffn_fwd(h, inp.q, inp.k, inp.v, act, o)
        G.gdpa_pffn_bwd(h, inp.q, inp.k, inp.v, inp.do, act, dq, dwk, dwv)
        torch.cuda.synchronize()
    finally:
        G.gdpa_plan_destroy(h)
    return st, [t.float().cpu().numpy() for t in (o, dq, dwk, dwv)]


@pytest.mark.parametrize("Tq,M,d,bins", [(300, 96, 64, 16), (1000, 200, 128, 32), (77, 32, 32, 8),
                                         (2500, 65, 128, 0), (0, 64, 64, 8), (50, 0, 128, 8)])
@pytest.mark.parametrize("act", ["silu", "gelu"])
def test_pffn(Tq, M, d, bins, act):
    say(f"pFFN Tq={Tq} M={M} d={d} bins={bins} act={act}")
    inp = make_from_lengths([Tq], [M], 2, d, act=act, seed=41, device=DEV)
    st, (o, dq, dwk, dwv) = run_pffn(inp, act, bins=(bins,) * 3)
    if Tq and M and bins:
        assert st["n_parts"][1] > 0   # the weight gradients are reduced over chunks
    q, wk, wv, do = (inp.f64(n) for n in ("q", "k", "v", "do"))
    check_close(o, R.pffn_fwd(q, wk, wv, act), f"pFFN O d={d}")
    for name, a, b in zip(("dQ", "dW_K", "dW_V"), (dq, dwk, dwv), R.pffn_bwd(q, wk, wv, do, act)):
        check_close(a, b, f"pFFN {name} d={d}")


def test_full_size_pffn():
    """The benchmark's pFFN batch (the jagged self-attention batch's 79,265 query rows against
    M = 512 shared weight rows, H = 4, d = 128, SiLU) in its launch configuration: O and dQ
    on sampled query rows (each depends only on its own row), and the weight gradients, sums
    over every query row, in full."""
    say("pFFN full size: 79,265 query rows x 512 weight rows, sampled O / dQ rows, full dW_K, dW_V")
    inp = make_pffn(device=DEV)
    st, (o, dq, dwk, dwv) = run_pffn(inp, inp.act)
    assert st["n_parts"][1] > 0   # the weight gradients are reduced over chunks
    q, wk, wv, do = (inp.f64(n) for n in ("q", "k", "v", "do"))
    idx = np.sort(np.random.default_rng(5).choice(q.shape[0], 2000, replace=False))
    for t, name in ((o, "O"), (dq, "dQ"), (dwk, "dW_K"), (dwv, "dW_V")):
        assert np.all(np.isfinite(t)), f"pFFN {name}: non-finite values"
    check_close(o[idx], R.pffn_fwd(q[idx], wk, wv, inp.act), "pFFN O sampled rows")
    check_close(dq[idx], R.pffn_bwd(q[idx], wk, wv, do[idx], inp.act)[0], "pFFN dQ sampled rows")
    _, dwk_ref, dwv_ref = R.pffn_bwd(q, wk, wv, do, inp.act)
    check_close(dwk, dwk_ref, "pFFN dW_K full")
    check_close(dwv, dwv_ref, "pFFN dW_V full")


def test_pffn_rejects_a_jagged_plan():
    inp = make_from_lengths([5, 7], [3, 4], 2, 64, act="silu", seed=1, device=DEV)
    with G.Plan(inp.q_off, inp.kv_off, 2, 64, 0, "bf16") as plan:
        with pytest.raises(G.GdpaError) as e:
            G.gdpa_pffn_fwd(plan.handle, inp.q, inp.k, inp.v, "silu", torch.empty_like(inp.q))
        assert G.STATUS[e.value.status] == "GDPA_ERR_PLAN_MISMATCH"


@pytest.mark.parametrize("act", ["gelu", "silu", "gelu_taylor6", "identity"])
def test_one_pass_backward_activations(act):
    say(f"one-pass backward activation {act}")
    for lq, lk in (([130, 7, 64], [32, 9, 30]), ([32, 9, 30], [130, 7, 64])):
        inp = make_from_lengths(lq, lk, 2, 64, act=act, seed=17, device=DEV)
        for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp), oracle_bwd(inp)):
            check_close(a, b, f"{name} {act}")


@pytest.mark.parametrize("act", ["gelu", "silu", "gelu_taylor6", "identity"])
def test_activations_forward_backward(act):
    say(f"activation {act}")
    inp = make_from_lengths([40, 130, 7, 260], [77, 20, 300, 129], 2, 64, act=act, seed=5, device=DEV)
    check_close(run_fwd(inp), oracle_fwd(inp), f"O {act}")
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp), oracle_bwd(inp)):
        check_close(a, b, f"{name} {act}")


# (team, blocks) for the forward / dK/dV / dQ lists
WIN_LAYOUTS = [((1, 1, 1), (1, 1, 1)), ((1, 1, 1), (2, 1, 2)), ((2, 2, 2), (1, 1, 1)), ((1, 2, 1), (2, 1, 2))]


@pytest.mark.parametrize("window", [1, 2, 17, 128, 1000])
@pytest.mark.parametrize("lay", range(len(WIN_LAYOUTS)))
def test_windows(window, lay):
    team, blocks = WIN_LAYOUTS[lay]
    say(f"window {window} team {team} blocks {blocks}")
    L = [1, 33, 128, 129, 700, 0, 300]
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=window, seed=6, device=DEV)
    check_close(run_fwd(inp, team=team, blocks=blocks), oracle_fwd(inp), f"O w={window}")
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp, team=team, blocks=blocks), oracle_bwd(inp)):
        check_close(a, b, f"{name} w={window}")


def _random_case(seed):
    """A seeded random configuration: batch size, head count, head dimension, activation,
    window and per-sample lengths drawn from a mix that stresses tile edges (0, 1, 31, 32, 33,
    63, 64, 65), short and long samples, and self- or cross-shaped batches."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 9))
    H = int(rng.choice([1, 2, 3]))
    d = int(rng.choice([32, 64, 128]))
    act = str(rng.choice(["gelu", "silu", "gelu_taylor6", "identity"]))
    edge = np.array([0, 1, 31, 32, 33, 63, 64, 65])
    def draw(n):
        pick = rng.random(n)
        return np.where(pick < 0.4, rng.choice(edge, n), np.where(pick < 0.8, rng.integers(1, 200, n),
                                                                  rng.integers(200, 700, n)))
    lq = draw(B)
    window = int(rng.choice([0, 0, 0, 0, 0, 0, 1, 7, 40, 128]))
    shape = rng.random()
    if window or shape < 0.3:       # self-attention
        lk = lq.copy()
    elif shape < 0.55:              # every key side in one tile (the KV-stationary one-pass backward)
        lk = rng.integers(1, 33, B)
    elif shape < 0.8:               # every query side in one tile (the Q-stationary one-pass backward)
        lk, lq = lq, rng.integers(1, 33, B)
    else:
        lk = draw(B)
    return [int(x) for x in lq], [int(x) for x in lk], H, d, act, window


@pytest.mark.parametrize("seed", range(24))
def test_random_configurations(seed):
    lq, lk, H, d, act, window = _random_case(seed)
    say(f"random case {seed}: lq={lq} lk={lk} H={H} d={d} act={act} window={window}")
    inp = make_from_lengths(lq, lk, H, d, act=act, window=window, seed=seed, device=DEV)
    ro, rg = oracle_fwd(inp), oracle_bwd(inp)
    check_close(run_fwd(inp), ro, f"O random {seed}")
    check_close(run_fwd(inp, dtype="bf16_f32out"), ro, f"O f32out random {seed}")
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp), rg):
        check_close(a, b, f"{name} random {seed}")
    for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp, unfused=True), rg):
        check_close(a, b, f"{name} unfused random {seed}")


@pytest.mark.parametrize("H,d", [(12, 64), (16, 32), (16, 128)])
def test_many_heads(H, d):
    """Head counts beyond the workloads' (the [T, H, d] head stride in every descriptor and
    store): forward and backward, self and cross shapes, against the oracle."""
    say(f"H={H} d={d}")
    for lq, lk, window in (([70, 0, 33, 129], [70, 0, 33, 129], 0), ([70, 1, 33, 5], [9, 40, 0, 64], 0),
                           ([70, 3, 33, 129], [70, 3, 33, 129], 17)):
        inp = make_from_lengths(lq, lk, H, d, act="gelu", window=window, seed=H + d, device=DEV)
        check_close(run_fwd(inp), oracle_fwd(inp), f"O H={H} d={d} lq={lq}")
        for name, a, b in zip(("dQ", "dK", "dV"), run_bwd(inp), oracle_bwd(inp)):
            check_close(a, b, f"{name} H={H} d={d} lq={lq}")


def test_side_stream_and_graph_capture():
    """Launches on a stream other than the default, and captured into a HIP graph (the launch
    path records no memset, allocation or copy): a side stream and every replay of the graph,
    with eager work and synchronisations between replays, reproduce the default stream's
    outputs bit for bit.  The plan cuts forward items, so the chunk reduction is captured too."""
    say("side stream and graph capture")
    lq, lk = [300, 5, 70, 129, 1], [1500, 7, 64, 1000, 33]
    inp = make_from_lengths(lq, lk, 2, 64, act="gelu", seed=71, device=DEV)
    qo, ko = dev_offsets(inp)
    B, H, d, win, act = len(lq), 2, 64, 0, "gelu"
    with G.Plan(inp.q_off, inp.kv_off, H, d, win, "bf16", bins=(16, 16, 32)) as plan:
        assert plan.stats()["n_parts"][0] > 0
        h = plan.handle

        def run(o, dq, dk, dv, stream):
            G.gdpa_fwd(h, inp.q, inp.k, inp.v, qo, ko, B, H, d, act, win, o, stream)
            G.gdpa_bwd(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, act, win, dq, dk, dv, stream)

        def outputs():
            return (torch.empty_like(inp.q), torch.empty_like(inp.q), torch.empty_like(inp.k),
                    torch.empty_like(inp.v))

        ref = outputs()
        run(*ref, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        check_close(ref[0].float().cpu().numpy(), oracle_fwd(inp), "O default stream")

        side = torch.cuda.Stream()
        got = outputs()
        with torch.cuda.stream(side):
            run(*got, side.cuda_stream)
        side.synchronize()
        for a, b, name in zip(got, ref, ("O", "dQ", "dK", "dV")):
            assert torch.equal(a, b), f"{name}: side stream differs"

        cap = outputs()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run(*cap, torch.cuda.current_stream().cuda_stream)
        for rep in range(3):
            for t in cap:
                t.fill_(float("nan"))   # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for a, b, name in zip(cap, ref, ("O", "dQ", "dK", "dV")):
                assert torch.equal(a, b), f"{name}: graph replay {rep} differs"


def test_empty_and_degenerate():
    say("empty samples, Lk=0, Lq=0, empty batch")
    lq = [0, 5, 0, 40, 3]
    lk = [7, 0, 0, 90, 1]
    inp = make_from_lengths(lq, lk, 3, 64, act="gelu", seed=7, device=DEV)
    o = run_fwd(inp)
    check_close(o, oracle_fwd(inp), "O degenerate")
    assert np.all(o[0:5] == 0.0)                         # sample 1 has no keys
    dq, dk, dv = run_bwd(inp)
    rq, rk, rv = oracle_bwd(inp)
    assert np.all(dk[0:7] == 0.0) and np.all(dv[0:7] == 0.0)   # sample 0 has no queries
    assert np.all(dq[0:5] == 0.0)
    for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), (rq, rk, rv)):
        check_close(a, b, f"{name} degenerate")
    # a batch with no rows at all
    z = make_from_lengths([0, 0], [0, 0], 2, 64, seed=1, device=DEV)
    assert run_fwd(z).shape == (0, 2, 64)


def test_outputs_fully_written():
    say("every output row is written (buffers pre-filled with NaN)")
    inp = make_from_lengths([0, 3, 70, 1], [5, 0, 33, 2], 2, 64, act="silu", seed=8, device=DEV)
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, 2, 64, 0, "bf16") as plan:
        o = torch.full_like(inp.q, float("nan"))
        dq = torch.full_like(inp.q, float("nan"))
        dk = torch.full_like(inp.k, float("nan"))
        dv = torch.full_like(inp.v, float("nan"))
        plan.fwd(inp.q, inp.k, inp.v, qo, ko, "silu", o=o)
        plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, "silu", dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t.float()).all()


# ---------------------------------------------------------------------------
# bit-exact offset indexing: count and bit probes
# ---------------------------------------------------------------------------

def _probe_expect(lq, lk, window, bit=None):
    """Per query row: number of valid keys (bit=None) or of valid keys whose local
    index has bit `bit` set.  Brute force over the valid set."""
    out = []
    for a, c in zip(lq, lk):
        m = R.valid_mask(np.arange(a), np.arange(c), a, c, window)
        if bit is not None:
            m = m & (((np.arange(c) >> bit) & 1) == 1)[None, :]
        out.append(m.sum(axis=1))
    return np.concatenate(out) if out else np.zeros(0)


@pytest.mark.parametrize("window", [0, 128])
@pytest.mark.parametrize("d,team,nb", [(32, 1, 1), (32, 1, 2), (128, 1, 2), (128, 2, 1)])
def test_index_probe_bit_exact(window, d, team, nb):
    say(f"count/bit probe window={window} d={d} team={team} blocks={nb}")
    L = [1, 31, 32, 33, 127, 128, 129, 600, 0, 1100] if window else None
    lq = L or [3, 31, 32, 33, 0, 128, 129, 257, 40, 1]
    lk = L or [129, 1, 64, 0, 5, 300, 33, 257, 511, 2]
    inp = make_from_lengths(lq, lk, 2, d, act="one", window=window, seed=9, device=DEV)
    # V[j, h, e] = bit e of the key's local index j (e < 16); V[j, h, 16:] = 1
    vals = []
    for c in lk:
        j = np.arange(c)[:, None]
        bits = ((j >> np.arange(16)[None, :]) & 1).astype(np.float32)
        vals.append(np.concatenate([bits, np.ones((c, d - 16), np.float32)], axis=1))
    V = np.concatenate(vals) if vals else np.zeros((0, d), np.float32)
    inp.v = torch.tensor(np.repeat(V[:, None, :], 2, axis=1), dtype=torch.bfloat16, device=DEV)
    o = run_fwd(inp, act="one", dtype="bf16_f32out", team=(team, 0, 0), blocks=(nb, 0, 0))
    cnt = _probe_expect(lq, lk, window)
    for h in range(2):
        np.testing.assert_array_equal(o[:, h, 16], cnt)
        for e in range(16):
            np.testing.assert_array_equal(o[:, h, e], _probe_expect(lq, lk, window, bit=e))


# ---------------------------------------------------------------------------
# the polynomial GELU against the exact-erf oracle
# ---------------------------------------------------------------------------

def poly_bounds(inp):
    """Per-element bounds of what the polynomial's fit errors can move O, dQ, dK, dV
    (eps on the value, eps' on the derivative), through the products:
      |dO_i|  <= eps  sum_j |V_j|                      (O = sum_j P_ij V_j)
      |ddV_j| <= eps  sum_i |dO_i|                     (dV = sum_i P_ij dO_i)
      |ddQ_i| <= eps' sum_j (|dO_i|.|V_j|) |K_j| / sqrt d   (dS = dP act', |dP_ij| <= |dO_i|.|V_j|)
      |ddK_j| <= eps' sum_i (|dO_i|.|V_j|) |Q_i| / sqrt d
    each sum over the valid pairs: the oracle on absolute values with act = one
    (P = 1) or identity (dS = dP) computes exactly these sums."""
    return _poly_bounds(*(inp.f64(n) for n in ("q", "k", "v", "do")), inp.q_off, inp.kv_off, inp.window)


def _poly_bounds(q, k, v, do, q_off, kv_off, window):
    ef, eg = G.gdpa_gelu_poly_bound(), G.gdpa_gelu_poly_grad_bound()
    aq, ak, av, ado = (np.abs(t) for t in (q, k, v, do))
    bo = R.gdpa_fwd(aq, ak, av, q_off, kv_off, "one", window) * ef
    bdv = R.gdpa_bwd(aq, ak, av, ado, q_off, kv_off, "one", window)[2] * ef
    bdq, bdk, _ = R.gdpa_bwd(aq, ak, av, ado, q_off, kv_off, "identity", window)
    return bo, (bdq * eg, bdk * eg, bdv)


def test_gelu_poly_within_stated_bound():
    say("poly GELU vs exact-erf oracle, windowed shapes, fwd + two-kernel bwd")
    L = [700, 1300, 129]
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=128, seed=11, device=DEV)
    bo, bgrad = poly_bounds(inp)
    check_close(run_fwd(inp, act="gelu_poly"), oracle_fwd(inp, "gelu"), "O poly", extra=bo)
    for name, a, b, e in zip(("dQ", "dK", "dV"), run_bwd(inp, act="gelu_poly"), oracle_bwd(inp, "gelu"), bgrad):
        check_close(a, b, f"{name} poly", extra=e)
    # taylor6 is the pages' series; against its own definition it must meet the bf16 bound
    check_close(run_fwd(inp, act="gelu_taylor6"), oracle_fwd(inp, "gelu_taylor6"), "O taylor6")


@pytest.mark.parametrize("d", [32, 64, 128])
def test_gelu_poly_one_pass_and_layouts(d):
    say(f"poly GELU vs exact-erf oracle, one-pass backward kernels and the forward, d={d}")
    for lq, lk in (([130, 7, 64], [32, 9, 30]), ([32, 9, 30], [130, 7, 64]), ([90, 3, 250], [60, 41, 250])):
        inp = make_from_lengths(lq, lk, 2, d, act="gelu", seed=19, device=DEV)
        bo, bgrad = poly_bounds(inp)
        check_close(run_fwd(inp, act="gelu_poly"), oracle_fwd(inp, "gelu"), f"O poly d={d}", extra=bo)
        for name, a, b, e in zip(("dQ", "dK", "dV"), run_bwd(inp, act="gelu_poly"), oracle_bwd(inp, "gelu"),
                                 bgrad):
            check_close(a, b, f"{name} poly d={d} lq={lq}", extra=e)


# ---------------------------------------------------------------------------
# full sizes, in the launch configuration the benchmark times: sampled rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled(cfg):
    w = WORKLOADS[cfg]
    say(f"cfg{cfg} full size (B={w['B']}), fwd + bwd, sampled samples")
    inp = make_workload(cfg, device=DEV)
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16") as plan:
        o = plan.fwd(inp.q, inp.k, inp.v, qo, ko, inp.act)
        dq, dk, dv = plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, inp.act)
        torch.cuda.synchronize()
    rng = np.random.default_rng(cfg)
    B = len(inp.lq)
    picks = sorted(set(rng.choice(B, size=min(4, B), replace=False).tolist()
                       + [int(np.argmax(inp.lq)), int(np.argmax(inp.lk))]))
    for b in picks:
        qs, qe = int(inp.q_off[b]), int(inp.q_off[b + 1])
        ks, ke = int(inp.kv_off[b]), int(inp.kv_off[b + 1])
        f = lambda t, a, e: t[a:e].to("cpu", torch.float64).numpy()
        one_q = np.array([0, qe - qs])
        one_k = np.array([0, ke - ks])
        q64, k64, v64, do64 = f(inp.q, qs, qe), f(inp.k, ks, ke), f(inp.v, ks, ke), f(inp.do, qs, qe)
        ro = R.gdpa_fwd(q64, k64, v64, one_q, one_k, inp.act, inp.window)
        rq, rk, rv = R.gdpa_bwd(q64, k64, v64, do64, one_q, one_k, inp.act, inp.window)
        check_close(f(o, qs, qe), ro, f"cfg{cfg} O sample {b}")
        check_close(f(dq, qs, qe), rq, f"cfg{cfg} dQ sample {b}")
        check_close(f(dk, ks, ke), rk, f"cfg{cfg} dK sample {b}")
        check_close(f(dv, ks, ke), rv, f"cfg{cfg} dV sample {b}")
    # properties at any size: finite everywhere, zero rows where no partner exists
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t.float()).all()


def test_full_size_poly_windowed():
    """The windowed batch at full size with the polynomial GELU, in the benchmark's launch
    configuration (bench.py --config 5 --act gelu_poly): sampled samples against the
    exact-erf oracle within the bf16 bounds plus the fit's bounds carried through the
    products."""
    say("windowed batch full size (B=128), polynomial GELU vs exact erf, sampled samples")
    inp = make_workload(5, device=DEV)
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16") as plan:
        o = plan.fwd(inp.q, inp.k, inp.v, qo, ko, "gelu_poly")
        dq, dk, dv = plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, "gelu_poly")
        torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    rng = np.random.default_rng(55)
    picks = sorted(set(rng.choice(len(inp.lq), size=3, replace=False).tolist() + [int(np.argmax(inp.lq))]))
    f = lambda t, a, e: t[a:e].to("cpu", torch.float64).numpy()
    for b in picks:
        qs, qe = int(inp.q_off[b]), int(inp.q_off[b + 1])
        one = np.array([0, qe - qs])
        q64, k64, v64, do64 = f(inp.q, qs, qe), f(inp.k, qs, qe), f(inp.v, qs, qe), f(inp.do, qs, qe)
        bo, bgrad = _poly_bounds(q64, k64, v64, do64, one, one, inp.window)
        check_close(f(o, qs, qe), R.gdpa_fwd(q64, k64, v64, one, one, "gelu", inp.window), f"poly O sample {b}",
                    extra=bo)
        refs = R.gdpa_bwd(q64, k64, v64, do64, one, one, "gelu", inp.window)
        for name, got, ref, e in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs, bgrad):
            check_close(f(got, qs, qe), ref, f"poly {name} sample {b}", extra=e)


def test_determinism_with_cut_items():
    say("bitwise determinism run to run, with chunks and their reduction")
    inp = make_from_lengths(*CHUNK_CASES[3][:2], 2, 128, act="gelu", seed=5, device=DEV)
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, 2, 128, 0, "bf16", bins=(32, 32, 32)) as plan:
        assert min(plan.stats()["n_parts"]) > 0
        a = plan.fwd(inp.q, inp.k, inp.v, qo, ko, "gelu")
        b = plan.fwd(inp.q, inp.k, inp.v, qo, ko, "gelu")
        g1 = plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, "gelu")
        g2 = plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, "gelu")
        torch.cuda.synchronize()
    assert torch.equal(a, b)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def test_determinism():
    say("bitwise determinism run to run")
    inp = make_workload(2, device=DEV, B=64)
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, 0, "bf16") as plan:
        a = plan.fwd(inp.q, inp.k, inp.v, qo, ko, "silu")
        b = plan.fwd(inp.q, inp.k, inp.v, qo, ko, "silu")
        g1 = plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, "silu")
        g2 = plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, "silu")
        torch.cuda.synchronize()
    assert torch.equal(a, b)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def _picks(inp, seed):
    rng = np.random.default_rng(seed)
    B = len(inp.lq)
    return sorted(set(rng.choice(B, size=min(4, B), replace=False).tolist()
                      + [int(np.argmax(inp.lq)), int(np.argmax(inp.lk))]))


def _slices(inp, b):
    return (int(inp.q_off[b]), int(inp.q_off[b + 1])), (int(inp.kv_off[b]), int(inp.kv_off[b + 1]))


_f64 = lambda t, a, e: t[a:e].to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled_jfa(cfg):
    """JFA forward and backward at full size in the benchmark's launch configuration;
    sampled samples against the oracle one by one."""
    say(f"cfg{cfg} full size JFA fwd + bwd, sampled samples")
    inp = make_workload(cfg, device=DEV)
    qo, ko = dev_offsets(inp)
    Tq = inp.q.shape[0]
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16") as plan:
        o = torch.empty_like(inp.q)
        lse = torch.empty((inp.H, Tq), dtype=torch.float32, device=DEV)
        stat = torch.empty((inp.H, Tq, 2), dtype=torch.float32, device=DEV)
        dq, dk, dv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)
        G.gdpa_jfa_fwd(plan.handle, inp.q, inp.k, inp.v, qo, ko, plan.B, inp.H, inp.d, inp.window, o, lse)
        G.gdpa_jfa_bwd(plan.handle, inp.q, inp.k, inp.v, o, lse, inp.do, qo, ko, plan.B, inp.H, inp.d, inp.window,
                       stat, dq, dk, dv)
        torch.cuda.synchronize()
    for b in _picks(inp, cfg):
        (qs, qe), (ks, ke) = _slices(inp, b)
        one_q, one_k = np.array([0, qe - qs]), np.array([0, ke - ks])
        args = (_f64(inp.q, qs, qe), _f64(inp.k, ks, ke), _f64(inp.v, ks, ke))
        ro, rl = R.jfa_fwd(*args, one_q, one_k, inp.window)
        rq, rk, rv = R.jfa_bwd(*args, _f64(inp.do, qs, qe), one_q, one_k, inp.window)
        check_close(_f64(o, qs, qe), ro, f"cfg{cfg} JFA O sample {b}")
        check_lse(lse[:, qs:qe].cpu().numpy(), rl, f"cfg{cfg} JFA LSE sample {b}")
        check_close(_f64(dq, qs, qe), rq, f"cfg{cfg} JFA dQ sample {b}")
        check_close(_f64(dk, ks, ke), rk, f"cfg{cfg} JFA dK sample {b}")
        check_close(_f64(dv, ks, ke), rv, f"cfg{cfg} JFA dV sample {b}")
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t.float()).all()


@pytest.mark.parametrize("cfg", [2, 4])
def test_full_size_sampled_norm(cfg):
    """The RMSNorm prologue at full size on raw inputs, in the benchmark's launch configuration."""
    say(f"cfg{cfg} full size norm prologue fwd + bwd, sampled samples")
    w = WORKLOADS[cfg]
    inp = make_workload(cfg, device=DEV, raw=True)
    norm = w["rms"]
    qo, ko = dev_offsets(inp)
    Tq, Tk = inp.q.shape[0], inp.k.shape[0]
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16") as plan:
        rstd = torch.empty((inp.H * (Tq + 2 * Tk),), dtype=torch.float32, device=DEV)
        o = torch.empty_like(inp.q)
        dq, dk, dv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)
        a = (plan.handle, inp.q, inp.k, inp.v)
        G.gdpa_norm_rstd(*a, inp.H, inp.d, norm, rstd)
        G.gdpa_norm_fwd(*a, qo, ko, plan.B, inp.H, inp.d, inp.act, inp.window, norm, rstd, o)
        G.gdpa_norm_bwd(*a, inp.do, qo, ko, plan.B, inp.H, inp.d, inp.act, inp.window, norm, rstd, dq, dk, dv)
        torch.cuda.synchronize()
    for b in _picks(inp, cfg):
        (qs, qe), (ks, ke) = _slices(inp, b)
        one_q, one_k = np.array([0, qe - qs]), np.array([0, ke - ks])
        args = (_f64(inp.q, qs, qe), _f64(inp.k, ks, ke), _f64(inp.v, ks, ke))
        ro = R.norm_gdpa_fwd(*args, one_q, one_k, inp.act, inp.window, norm)
        rq, rk, rv = R.norm_gdpa_bwd(*args, _f64(inp.do, qs, qe), one_q, one_k, inp.act, inp.window, norm)
        check_close(_f64(o, qs, qe), ro, f"cfg{cfg} norm O sample {b}")
        check_close(_f64(dq, qs, qe), rq, f"cfg{cfg} norm dQ sample {b}")
        check_close(_f64(dk, ks, ke), rk, f"cfg{cfg} norm dK sample {b}")
        check_close(_f64(dv, ks, ke), rv, f"cfg{cfg} norm dV sample {b}")
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t.float()).all()


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled_fp8(cfg):
    """The fp8 forward at full size (one scale per tensor over the whole batch)."""
    say(f"cfg{cfg} full size fp8 forward, sampled samples")
    inp = make_workload(cfg, device=DEV)
    qo, ko = dev_offsets(inp)
    q8, sq = quant_e4m3(inp.q)
    k8, sk = quant_e4m3(inp.k)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16") as plan:
        o = torch.empty_like(inp.q)
        G.gdpa_fp8_fwd(plan.handle, q8.view(torch.uint8).to(DEV), k8.view(torch.uint8).to(DEV), inp.v, qo, ko,
                       plan.B, inp.H, inp.d, inp.act, inp.window, sq, sk, o)
        torch.cuda.synchronize()
    for b in _picks(inp, cfg):
        (qs, qe), (ks, ke) = _slices(inp, b)
        ro = R.gdpa_fwd(q8[qs:qe].double().numpy() * sq, k8[ks:ke].double().numpy() * sk, _f64(inp.v, ks, ke),
                        np.array([0, qe - qs]), np.array([0, ke - ks]), inp.act, inp.window)
        check_close(_f64(o, qs, qe), ro, f"cfg{cfg} fp8 O sample {b}")
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled_fp8_backward(cfg):
    """The fp8 backward at full size in the benchmark's launch configuration (one factor per
    tensor over the whole batch; one pass or the stored-dS kernels): sampled samples against
    the oracle on the values the bytes stand for."""
    say(f"cfg{cfg} full size fp8 backward, sampled samples")
    inp = make_workload(cfg, device=DEV)
    qo, ko = dev_offsets(inp)
    q8, sq = quant_e4m3(inp.q)
    k8, sk = quant_e4m3(inp.k)
    o8, so = quant_e4m3(inp.do)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16") as plan:
        dq, dk, dv = (torch.empty_like(t) for t in (inp.q, inp.k, inp.v))
        G.gdpa_fp8_bwd(plan.handle, q8.view(torch.uint8).to(DEV), k8.view(torch.uint8).to(DEV), inp.v,
                       o8.view(torch.uint8).to(DEV), qo, ko, plan.B, inp.H, inp.d, inp.act, inp.window, sq, sk, so,
                       dq, dk, dv)
        torch.cuda.synchronize()
    for b in _picks(inp, cfg):
        (qs, qe), (ks, ke) = _slices(inp, b)
        ref = R.gdpa_bwd(q8[qs:qe].double().numpy() * sq, k8[ks:ke].double().numpy() * sk, _f64(inp.v, ks, ke),
                         o8[qs:qe].double().numpy() * so, np.array([0, qe - qs]), np.array([0, ke - ks]), inp.act,
                         inp.window)
        for name, got, r in zip(("dQ", "dK", "dV"), (_f64(dq, qs, qe), _f64(dk, ks, ke), _f64(dv, ks, ke)), ref):
            check_close(got, r, f"cfg{cfg} fp8 {name} sample {b}")
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled_mx(cfg):
    """The MXFP8 forward at full size: sampled samples against the oracle on the values the
    bytes and their block scales stand for."""
    say(f"cfg{cfg} full size MX forward, sampled samples")
    inp = make_workload(cfg, device=DEV)
    qo, ko = dev_offsets(inp)
    q8, qsc = quant_mx(inp.q)
    k8, ksc = quant_mx(inp.k)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16") as plan:
        o = torch.empty_like(inp.q)
        G.gdpa_mx_fwd(plan.handle, q8.view(torch.uint8).to(DEV), qsc.to(DEV), k8.view(torch.uint8).to(DEV),
                      ksc.to(DEV), inp.v, qo, ko, plan.B, inp.H, inp.d, inp.act, inp.window, o)
        torch.cuda.synchronize()
    for b in _picks(inp, cfg):
        (qs, qe), (ks, ke) = _slices(inp, b)
        ro = R.gdpa_fwd(dequant_mx(q8[qs:qe], qsc[:, qs:qe]), dequant_mx(k8[ks:ke], ksc[:, ks:ke]),
                        _f64(inp.v, ks, ke), np.array([0, qe - qs]), np.array([0, ke - ks]), inp.act, inp.window)
        check_close(_f64(o, qs, qe), ro, f"cfg{cfg} MX O sample {b}")
    assert torch.isfinite(o.float()).all()
