"""Dispatch-round time factors in the greedy deal (the plan option `slot_time`).

The factors only move items between bins: each item computes the same arithmetic in
the same order wherever it runs, and cut items' chunks are summed in their fixed slot
order, so a plan dealt with the factors must give the outputs of one dealt by plain
cost bit for bit.  The cases cover the kernel layouts the factors apply to (the d = 128
two-wave forward and 16-row dK/dV kernels at four workgroups per CU, the d = 64 forward
with two blocks per wave at eight, dQ from stored dS in two-wave teams at three) and
check that the deal did change."""
import numpy as np
import pytest
import torch

import recsys_attention_jagged_amd as G
from gdpa_workloads import make_from_lengths
from oracle import gdpa_ref as R

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def dev_offsets(inp):
    return (torch.tensor(inp.q_off, dtype=torch.int32, device=DEV),
            torch.tensor(inp.kv_off, dtype=torch.int32, device=DEV))


def lengths(n, lo, hi, seed):
    return np.random.default_rng(seed).integers(lo, hi, size=n).tolist()


# (lq, lk, d, window, plan options, lists expected to take the factors)
CASES = [
    # windowed self-attention, d = 128: two-wave forward, 16-row dK/dV
    (lengths(24, 900, 2600, 1), None, 128, 64, {}, [1, 1, 0]),
    # jagged self-attention, d = 128, with a zero-length and a one-row sample
    ([0, 1] + lengths(14, 200, 1500, 2), None, 128, 0, {}, [1, 1, 0]),
    # cross-attention at d = 64, forward in one-wave teams of two blocks per wave
    (lengths(40, 1, 33, 3), lengths(40, 500, 4000, 4), 64, 0, {"team": (1, 0, 0), "blocks": (2, 0, 0)},
     None),
]


def run_all(plan, inp, qo, ko):
    o = plan.fwd(inp.q, inp.k, inp.v, qo, ko, inp.act)
    g = plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, inp.act)
    return (o,) + tuple(g)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_slot_time_bit_exact(case):
    lq, lk, d, window, opts, expect = CASES[case]
    lk = lq if lk is None else lk
    say(f"slot-time case={case} d={d} window={window} B={len(lq)}")
    inp = make_from_lengths(lq, lk, 2, d, act="gelu", window=window, seed=500 + case, device=DEV)
    qo, ko = dev_offsets(inp)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    with G.Plan(inp.q_off, inp.kv_off, 2, d, window, "bf16", slot_time="off", **opts) as po, \
            G.Plan(inp.q_off, inp.kv_off, 2, d, window, "bf16", **opts) as pw:
        so, sw = po.stats(), pw.stats()
        assert so["slot_weighted"] == [0, 0, 0]
        if expect is not None:
            assert sw["slot_weighted"] == expect, sw
        elif sw["bins"][0] == 8 * cus:
            # the d = 64 forward at eight workgroups per CU
            assert sw["slot_weighted"][0] == 1, sw
        else:
            pytest.skip(f"the d = 64 forward runs {sw['bins'][0]} workgroups here, not 8 per CU")
        if d == 128 and sw["dq_team"] == 2 and sw["dq_team_bins"] == 3 * cus:
            # dQ from stored dS in two-wave teams at three per CU
            assert sw["dq_team_slot_weighted"] == 1 and so["dq_team_slot_weighted"] == 0, sw
        weighted = list(sw["slot_weighted"]) + [sw["dq_team_slot_weighted"]]
        for lst in range(4):
            if weighted[lst]:
                assert not np.array_equal(po.export(lst), pw.export(lst)), f"list {lst}: the deal did not change"
        ref = run_all(po, inp, qo, ko)
        got = run_all(pw, inp, qo, ko)
    torch.cuda.synchronize()
    names = ("O", "dQ", "dK", "dV")
    for name, a, b in zip(names, got, ref):
        assert torch.equal(a, b), f"{name}: the weighted deal differs from the plain one (case {case})"
    if case == 0:
        o_ref = R.gdpa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, "gelu", window)
        err = got[0].float().cpu().numpy().astype(np.float64) - o_ref
        assert np.linalg.norm(err) <= 1e-2 * np.linalg.norm(o_ref)
