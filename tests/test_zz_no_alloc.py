"""gdpa_fwd_noalloc (the forward for callers that cannot allocate device memory)
against gdpa_fwd through the C ABI: two calls in a row on host-only plans, the
second on a smaller batch, each equal to gdpa_fwd on a device plan of the same
layout and within the bf16 tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import recsys_attention_jagged_amd as G
from gdpa_workloads import make_from_lengths
from oracle import gdpa_ref as R

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _check_bf16(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(err)) / max(float(np.linalg.norm(ref)), 1e-30)
    assert np.all(np.isfinite(got)), what
    assert rel <= 1e-2, f"{what}: rel L2 {rel:.3e}"
    assert float(err.max(initial=0.0)) <= 2e-2 * float(np.abs(ref).max(initial=0.0)) + 1e-30, what


CASES = [   # (lq, lk, d, window, act, bins): the first has cut items (chunk slots in the scratch)
    ([32, 3000, 1, 0, 200], [3000, 40, 5, 7, 200], 128, 0, "gelu", (16, 16, 16)),
    ([70, 1, 33, 5], [70, 1, 33, 5], 64, 9, "silu", (8, 8, 8)),
]


@pytest.mark.parametrize("dtype", ["bf16", "bf16_f32out"])
def test_noalloc_forward_matches_gdpa_fwd_twice(dtype):
    print(f"no-alloc forward, {dtype}", flush=True)
    outs = []
    for lq, lk, d, window, act, bins in CASES:
        inp = make_from_lengths(lq, lk, 2, d, act=act, window=window, seed=71, device=DEV)
        qo = torch.tensor(inp.q_off, dtype=torch.int32, device=DEV)
        ko = torch.tensor(inp.kv_off, dtype=torch.int32, device=DEV)
        odt = torch.float32 if dtype == "bf16_f32out" else torch.bfloat16
        B = len(lq)
        host = G.gdpa_plan_create(inp.q_off, inp.kv_off, B, 2, d, window, dtype, host_only=True, bins=bins)
        dev = G.gdpa_plan_create(inp.q_off, inp.kv_off, B, 2, d, window, dtype, bins=bins)
        try:
            # the host-only plan's layout and chunks equal the device plan's
            for kind in ("fwd",):
                assert np.array_equal(G.gdpa_plan_export(host, kind), G.gdpa_plan_export(dev, kind))
            assert G.gdpa_plan_stats(host)["n_parts"][0] == G.gdpa_plan_stats(dev)["n_parts"][0]
            a = torch.full(inp.q.shape, float("nan"), dtype=odt, device=DEV)
            b = torch.full(inp.q.shape, float("nan"), dtype=odt, device=DEV)
            G.gdpa_fwd_noalloc(host, inp.q, inp.k, inp.v, qo, ko, B, 2, d, act, window, a)
            G.gdpa_fwd(dev, inp.q, inp.k, inp.v, qo, ko, B, 2, d, act, window, b)
            torch.cuda.synchronize()
            outs.append(G.gdpa_plan_stats(host)["n_parts"][0])
        finally:
            G.gdpa_plan_destroy(host)
            G.gdpa_plan_destroy(dev)
        ga, gb = a.float().cpu().numpy(), b.float().cpu().numpy()
        assert np.array_equal(ga, gb), f"no-alloc forward differs from gdpa_fwd ({dtype}, d={d})"
        ref = R.gdpa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, act, window)
        _check_bf16(ga, ref, f"no-alloc O ({dtype}, d={d})")
    assert outs[0] > 0   # the first batch had chunks, so the slots in the scratch were used


def test_noalloc_rejects():
    inp = make_from_lengths([40, 3], [50, 7], 2, 128, act="gelu", seed=72, device=DEV)
    qo = torch.tensor(inp.q_off, dtype=torch.int32, device=DEV)
    ko = torch.tensor(inp.kv_off, dtype=torch.int32, device=DEV)
    o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    f32 = G.gdpa_plan_create(inp.q_off, inp.kv_off, 2, 2, 128, 0, "f32", host_only=True)
    try:
        with pytest.raises(G.GdpaError) as e:
            G.gdpa_fwd_noalloc(f32, inp.q.float(), inp.k.float(), inp.v.float(), qo, ko, 2, 2, 128, "gelu", 0, o)
        assert G.STATUS[e.value.status] == "GDPA_ERR_UNSUPPORTED"
        with pytest.raises(G.GdpaError) as e:
            G.gdpa_fwd_noalloc(f32, inp.q, inp.k, inp.v, qo, ko, 2, 2, 64, "gelu", 0, o)
        assert G.STATUS[e.value.status] == "GDPA_ERR_PLAN_MISMATCH"
    finally:
        G.gdpa_plan_destroy(f32)
