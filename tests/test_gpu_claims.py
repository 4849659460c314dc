"""Items claimed at run time (the plan option `claim`) against the planner's bins.

Wherever an item runs, it computes the same arithmetic in the same order, so a plan
whose workgroups claim items from a counter must give the outputs of a plan that walks
the planner's bins bit for bit: on every kernel that walks a list in one-wave teams
(forward, the one-pass backward in both shapes, the two-kernel backward at d <= 64,
JFA, the RMSNorm prologue, the fp8 entry points), with cut items, on repeated launches
of one plan (the counters set themselves back to zero at the end of a launch) and
through replays of a captured HIP graph.  The oracle checks the first launch."""
import numpy as np
import pytest
import torch

import recsys_attention_jagged_amd as G
from fp8_bounds import quant_e4m3
from gdpa_workloads import make_from_lengths, make_workload
from oracle import gdpa_ref as R

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def dev_offsets(inp):
    return (torch.tensor(inp.q_off, dtype=torch.int32, device=DEV),
            torch.tensor(inp.kv_off, dtype=torch.int32, device=DEV))


def rel_l2(got, ref):
    got = got.float().cpu().numpy().astype(np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


# (lq, lk, d, window, bins): KV-stationary one pass, Q-stationary one pass, two-kernel
# backward at d = 64 and d = 32 with a window, and few bins (cut items)
CASES = [
    ([300, 5, 0, 77, 1, 64, 129, 900], [32, 1, 0, 17, 32, 31, 2, 32], 64, 0, (0, 0, 0)),
    ([32, 1, 0, 17, 32, 31, 2, 32], [300, 5, 0, 77, 1, 64, 129, 2000], 128, 0, (0, 0, 0)),
    ([300, 5, 0, 77, 1, 64, 129, 700], [300, 5, 0, 77, 1, 64, 129, 700], 64, 17, (0, 0, 0)),
    ([33, 1, 0, 400, 64, 65], [33, 1, 0, 400, 64, 65], 32, 0, (0, 0, 0)),
    ([32, 1, 20, 32, 5, 0], [3000, 5, 700, 1, 0, 0], 64, 0, (16, 16, 16)),
    ([3000, 5, 700, 1, 0, 0], [32, 1, 20, 32, 5, 0], 128, 0, (16, 16, 16)),
]


def run_all(plan, inp, qo, ko):
    """forward and backward of the plan (as gdpa_fwd / gdpa_bwd run them)"""
    o = plan.fwd(inp.q, inp.k, inp.v, qo, ko, inp.act)
    g = plan.bwd(inp.q, inp.k, inp.v, inp.do, qo, ko, inp.act)
    return (o,) + tuple(g)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_claimed_equals_bins(case):
    lq, lk, d, window, bins = CASES[case]
    say(f"claimed items case={case} d={d}")
    inp = make_from_lengths(lq, lk, 2, d, act="gelu", window=window, seed=300 + case, device=DEV)
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, 2, d, window, "bf16", bins=bins, claim="bins") as pb:
        assert pb.stats()["claimed"] == [0, 0, 0]
        ref = run_all(pb, inp, qo, ko)
    with G.Plan(inp.q_off, inp.kv_off, 2, d, window, "bf16", bins=bins, claim="always") as pc:
        st = pc.stats()
        assert sum(st["claimed"]) > 0, st
        runs = [run_all(pc, inp, qo, ko) for _ in range(3)]
    torch.cuda.synchronize()
    names = ("O", "dQ", "dK", "dV")
    for r, got in enumerate(runs):
        for name, a, b in zip(names, got, ref):
            assert torch.equal(a, b), f"{name}: claimed launch {r} differs from the bins (case {case})"
    o_ref = R.gdpa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, "gelu", window)
    g_ref = R.gdpa_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"), inp.q_off, inp.kv_off, "gelu",
                       window)
    for name, a, b in zip(names, runs[0], (o_ref,) + tuple(g_ref)):
        assert rel_l2(a, b) <= 1e-2, name


@pytest.mark.parametrize("case", [0, 1, 4])
def test_claimed_other_entry_points(case):
    """JFA, the RMSNorm prologue and the fp8 entry points walk the same claimed lists."""
    lq, lk, d, window, bins = CASES[case]
    say(f"claimed items, other entry points, case={case}")
    inp = make_from_lengths(lq, lk, 2, d, act="gelu", window=window, seed=310 + case, device=DEV)
    qo, ko = dev_offsets(inp)
    Tq, Tk = inp.q.shape[0], inp.k.shape[0]
    q8, sq = quant_e4m3(inp.q)
    k8, sk = quant_e4m3(inp.k)
    o8, so = quant_e4m3(inp.do)
    q8, k8, o8 = (t.view(torch.uint8).to(DEV) for t in (q8, k8, o8))

    def run(claim):
        with G.Plan(inp.q_off, inp.kv_off, 2, d, window, "bf16", bins=bins, claim=claim) as p:
            h, B = p.handle, p.B
            out = []
            for _ in range(2):
                o = torch.empty_like(inp.q)
                lse = torch.empty((2, Tq), dtype=torch.float32, device=DEV)
                stat = torch.empty((2, Tq, 2), dtype=torch.float32, device=DEV)
                g = [torch.empty_like(t) for t in (inp.q, inp.k, inp.v)]
                G.gdpa_jfa_fwd(h, inp.q, inp.k, inp.v, qo, ko, B, 2, d, window, o, lse)
                G.gdpa_jfa_bwd(h, inp.q, inp.k, inp.v, o, lse, inp.do, qo, ko, B, 2, d, window, stat, *g)
                rstd = torch.empty(2 * (Tq + 2 * Tk), dtype=torch.float32, device=DEV)
                on = torch.empty_like(inp.q)
                gn = [torch.empty_like(t) for t in (inp.q, inp.k, inp.v)]
                G.gdpa_norm_rstd(h, inp.q, inp.k, inp.v, 2, d, "qkv", rstd)
                G.gdpa_norm_fwd(h, inp.q, inp.k, inp.v, qo, ko, B, 2, d, "gelu", window, "qkv", rstd, on)
                G.gdpa_norm_bwd(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, 2, d, "gelu", window, "qkv", rstd, *gn)
                of = torch.empty_like(inp.q)
                gf = [torch.empty_like(t) for t in (inp.q, inp.k, inp.v)]
                G.gdpa_fp8_fwd(h, q8, k8, inp.v, qo, ko, B, 2, d, "gelu", window, sq, sk, of)
                G.gdpa_fp8_bwd(h, q8, k8, inp.v, o8, qo, ko, B, 2, d, "gelu", window, sq, sk, so, *gf)
                out.append([o, lse, *g, on, *gn, of, *gf])
            torch.cuda.synchronize()
            return out

    ref = run("bins")[0]
    for r, got in enumerate(run("always")):
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"output {i}: claimed launch {r} differs from the bins (case {case})"


def test_claimed_graph_replays():
    """Replays of a captured forward + backward on a plan that claims items, with eager
    work and synchronisations between them, equal the eager launches bit for bit."""
    lq, lk, d, window, bins = CASES[4]
    say("claimed items, graph replays")
    inp = make_from_lengths(lq, lk, 2, d, act="gelu", seed=320, device=DEV)
    qo, ko = dev_offsets(inp)
    B, H = len(lq), 2
    with G.Plan(inp.q_off, inp.kv_off, H, d, window, "bf16", bins=bins, claim="always") as plan:
        assert sum(plan.stats()["claimed"]) > 0
        h = plan.handle

        def run(o, dq, dk, dv, stream):
            G.gdpa_fwd(h, inp.q, inp.k, inp.v, qo, ko, B, H, d, "gelu", window, o, stream)
            G.gdpa_bwd(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, "gelu", window, dq, dk, dv, stream)

        def outputs():
            return (torch.empty_like(inp.q), torch.empty_like(inp.q), torch.empty_like(inp.k),
                    torch.empty_like(inp.v))

        ref = outputs()
        run(*ref, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        cap = outputs()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run(*cap, torch.cuda.current_stream().cuda_stream)
        for rep in range(3):
            for t in cap:
                t.zero_()
            graph.replay()
            torch.cuda.synchronize()
            for a, b, name in zip(cap, ref, ("O", "dQ", "dK", "dV")):
                assert torch.equal(a, b), f"{name}: graph replay {rep} differs"
            eager = outputs()
            run(*eager, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            for a, b, name in zip(eager, ref, ("O", "dQ", "dK", "dV")):
                assert torch.equal(a, b), f"{name}: eager launch after replay {rep} differs"


@pytest.mark.parametrize("cfg", [3, 4])
def test_claimed_workloads(cfg):
    """Reduced batches of the cross-attention and PMA workloads with every one-wave list
    claimed: the outputs equal the bins' bit for bit."""
    inp = make_workload(cfg, device=DEV, B={3: 96, 4: 48}[cfg])
    say(f"cfg{cfg} claimed, B={len(inp.lq)}")
    qo, ko = dev_offsets(inp)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16", claim="always") as pa:
        assert sum(pa.stats()["claimed"]) > 0
        got = run_all(pa, inp, qo, ko)
    with G.Plan(inp.q_off, inp.kv_off, inp.H, inp.d, inp.window, "bf16", claim="bins") as pb:
        ref = run_all(pb, inp, qo, ko)
    torch.cuda.synchronize()
    for name, a, b in zip(("O", "dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"cfg{cfg} {name}: claimed differs from the bins"
