"""The stated fp8 bounds hold the quantisation's own error with room for the
kernels' bf16 rounding: the oracle on e4m3-quantised Q, K (and dO) against the
oracle on the bf16 inputs, on each bf16 workload (seeded, reduced batch)."""
import numpy as np
import pytest

from fp8_bounds import FP8_MAX, FP8_REL_L2, KERNEL_MAX, KERNEL_REL_L2, fp8_errors, quant_e4m3
from gdpa_workloads import make_workload
from oracle import gdpa_ref as R

BATCH = {2: 8, 3: 6, 4: 3, 5: 1}


def _dequant(x):
    b, s = quant_e4m3(x)
    return b.double().numpy() * s


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_quantisation_error_leaves_room_for_the_kernels(cfg):
    inp = make_workload(cfg, B=BATCH[cfg])
    q8, k8, do8 = _dequant(inp.q), _dequant(inp.k), _dequant(inp.do)
    outs = [("O", R.gdpa_fwd(q8, k8, inp.f64("v"), inp.q_off, inp.kv_off, inp.act, inp.window),
             R.gdpa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, inp.act, inp.window))]
    got = R.gdpa_bwd(q8, k8, inp.f64("v"), do8, inp.q_off, inp.kv_off, inp.act, inp.window)
    ref = R.gdpa_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"), inp.q_off, inp.kv_off, inp.act,
                     inp.window)
    outs += list(zip(("dQ", "dK", "dV"), got, ref))
    for name, a, b in outs:
        rel, mx = fp8_errors(a, b)
        assert rel <= FP8_REL_L2 - KERNEL_REL_L2 and mx <= FP8_MAX - KERNEL_MAX, (cfg, name, rel, mx)
        # the quantisation did happen (an identity cast would pass anything)
        assert rel >= 0.01, (cfg, name, rel)


def test_quant_e4m3_round_trip():
    """448 and the scale's inverse are exact; values are rounded to 3 mantissa bits."""
    import torch
    x = torch.tensor([[448.0, -448.0, 1.0, 0.0, 1.0625, 3.3]])
    b, s = quant_e4m3(x)
    assert s == 1.0
    got = b.float().numpy()[0]
    np.testing.assert_array_equal(got[:5], [448.0, -448.0, 1.0, 0.0, 1.0])   # 1.0625 rounds to even
    assert got[5] == 3.25
