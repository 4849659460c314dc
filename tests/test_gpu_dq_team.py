"""dQ from the stored dS blocks in two-wave teams (plan option dq_team) against the
one-wave kernel.

The team kernel computes each 32-row q tile with the same products in the same
order as the one-wave kernel (the tile's K tiles in increasing order, steps outside
its band skipped), so wherever no item is cut into chunks its dQ equals the
one-wave kernel's bit for bit: windows, sample lengths that leave a team's second
tile empty or partial, an empty sample and a one-row sample, fp32 outputs and the fp8
backward.  With cut items the two lists cut at different places; there dQ is checked
against the oracle.  dK and dV do not depend on the option."""
import numpy as np
import pytest
import torch

import recsys_attention_jagged_amd as G
from fp8_bounds import check_fp8, quant_e4m3
from gdpa_workloads import make_from_lengths
from oracle import gdpa_ref as R

pytestmark = pytest.mark.gpu

DEV = "cuda"
L = [1, 15, 16, 17, 33, 47, 64, 65, 0, 300, 129, 700, 96, 97]


def say(*a):
    print(*a, flush=True)


def dev_offsets(inp):
    return (torch.tensor(inp.q_off, dtype=torch.int32, device=DEV),
            torch.tensor(inp.kv_off, dtype=torch.int32, device=DEV))


def bwd(inp, dtype, dq_team, bins=(0, 0, 0), fp8=None, split=False):
    """(dQ, dK, dV) and the plan's stats; by default no item is cut (split=False)"""
    qo, ko = dev_offsets(inp)
    odt = torch.float32 if dtype == "bf16_f32out" else torch.bfloat16
    with G.Plan(inp.q_off, inp.kv_off, inp.H, 128, inp.window, dtype, bins=bins, unfused=True, split=split,
                dq_team=dq_team) as plan:
        st = plan.stats()
        dq = torch.full(inp.q.shape, float("nan"), dtype=odt, device=DEV)
        dk = torch.full(inp.k.shape, float("nan"), dtype=odt, device=DEV)
        dv = torch.full(inp.v.shape, float("nan"), dtype=odt, device=DEV)
        if fp8 is None:
            G.gdpa_bwd(plan.handle, inp.q, inp.k, inp.v, inp.do, qo, ko, plan.B, inp.H, 128, inp.act,
                       inp.window, dq, dk, dv)
        else:
            (q8, sq), (k8, sk), (o8, so) = fp8
            G.gdpa_fp8_bwd(plan.handle, q8.view(torch.uint8).to(DEV), k8.view(torch.uint8).to(DEV), inp.v,
                           o8.view(torch.uint8).to(DEV), qo, ko, plan.B, inp.H, 128, inp.act, inp.window,
                           sq, sk, so, dq, dk, dv)
        torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (dq, dk, dv)], st


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


@pytest.mark.parametrize("window", [0, 9, 40, 128])
@pytest.mark.parametrize("dtype", ["bf16", "bf16_f32out"])
def test_dq_team_equals_one_wave(window, dtype):
    say(f"dQ team vs one wave: window={window} {dtype}")
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=window, seed=700 + window, device=DEV)
    team, st_t = bwd(inp, dtype, "auto")
    one, st_o = bwd(inp, dtype, "one_wave")
    assert st_t["dq_team"] == 2 and st_t["dq_team_items"] > 0 and st_t["dq_team_parts"] == 0, st_t
    assert st_o["dq_team"] == 1 and st_o["n_parts"][2] == 0, st_o
    for name, a, b in zip(("dQ", "dK", "dV"), team, one):
        assert np.all(np.isfinite(a)), f"{name}: non-finite values (rows left unwritten?)"
        assert np.array_equal(a, b), f"{name}: the team kernel differs from the one-wave kernel"
    ref = R.gdpa_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"), inp.q_off, inp.kv_off, "gelu",
                     window)
    assert rel_l2(team[0], ref[0]) <= 1e-2


@pytest.mark.parametrize("window", [0, 17])
def test_dq_team_fp8_equals_one_wave(window):
    say(f"dQ team vs one wave, fp8 backward: window={window}")
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=window, seed=720 + window, device=DEV)
    fp8 = (quant_e4m3(inp.q), quant_e4m3(inp.k), quant_e4m3(inp.do))
    team, st = bwd(inp, "bf16", "auto", fp8=fp8)
    one, _ = bwd(inp, "bf16", "one_wave", fp8=fp8)
    assert st["dq_team"] == 2
    for name, a, b in zip(("dQ", "dK", "dV"), team, one):
        assert np.array_equal(a, b), f"fp8 {name}: the team kernel differs from the one-wave kernel"
    (q8, sq), (k8, sk), (o8, so) = fp8
    ref = R.gdpa_bwd(q8.double().numpy() * sq, k8.double().numpy() * sk, inp.f64("v"), o8.double().numpy() * so,
                     inp.q_off, inp.kv_off, "gelu", window)
    check_fp8(team[0], ref[0], "fp8 dQ (team)")


@pytest.mark.parametrize("bins", [(64, 64, 64), (40, 40, 40)])
@pytest.mark.parametrize("dtype", ["bf16", "bf16_f32out"])
def test_dq_team_cut_items(bins, dtype):
    """Few bins: the team list's long items are cut into chunks whose 64-row partials
    the reduction adds; dQ against the oracle."""
    say(f"dQ team with cut items: bins={bins} {dtype}")
    inp = make_from_lengths(L, L, 2, 128, act="gelu", window=0, seed=740 + bins[0], device=DEV)
    team, st = bwd(inp, dtype, "auto", bins=bins, split=True)
    assert st["dq_team"] == 2 and st["dq_team_parts"] > 0 and st["dq_team_bins"] == bins[2], st
    ref = R.gdpa_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"), inp.q_off, inp.kv_off, "gelu", 0)
    for name, a, b in zip(("dQ", "dK", "dV"), team, ref):
        err = np.abs(a - b).max() / np.abs(b).max()
        assert rel_l2(a, b) <= 1e-2 and err <= 2e-2, f"{name}: rel {rel_l2(a, b):.3e} max {err:.3e}"
