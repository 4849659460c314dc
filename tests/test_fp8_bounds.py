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


def test_quant_mx_blocks():
    """Per 32-column block: scale 2^(floor(log2 amax) - 8), the largest element in
    [256, 448] after scaling; every element within half an e4m3 ulp (2^-4 relative,
    or 2^-10 of the block scale below the normal range) of its value, except those
    past 448 times the scale, which saturate to it."""
    import torch
    from fp8_bounds import dequant_mx, quant_mx
    g = torch.Generator().manual_seed(3)
    x = torch.randn((7, 3, 64), generator=g) * torch.exp(torch.randn((7, 3, 1), generator=g) * 3)
    x[2, 1, :32] = 0.0          # an all-zero block
    x[4, 0, 5] = 1.0e4          # one large element in a block
    q, s = quant_mx(x)
    assert q.shape == x.shape and s.shape == (3, 7, 2) and s.dtype == torch.uint8
    assert int(s[1, 2, 0]) == 0 and float(q[2, 1, :32].float().abs().max()) == 0.0
    xd = dequant_mx(q, s)
    xb = x.double().numpy().reshape(7, 3, 2, 32)
    amax = np.abs(xb).max(-1)
    e = s.numpy().astype(np.int64).transpose(1, 0, 2) - 127
    nz = amax > 0
    assert np.array_equal(e[nz], np.floor(np.log2(amax[nz])).astype(np.int64) - 8)
    qb = np.abs(q.float().numpy().reshape(7, 3, 2, 32)).max(-1)
    assert np.all((qb[nz] >= 256) & (qb[nz] <= 448))
    sc = np.exp2(e.astype(np.float64))[..., None]
    xd = xd.reshape(7, 3, 2, 32)
    sat = np.abs(xb) > 448 * sc
    assert np.array_equal(xd[sat], np.sign(xb[sat]) * 448 * np.broadcast_to(sc, xb.shape)[sat])
    err = np.abs(xd - xb)[~sat]
    tol = np.maximum(np.abs(xb) * 2.0 ** -4, sc * 2.0 ** -10)[~sat]
    assert np.all(err <= tol)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_mx_quantisation_error_within_the_fp8_bounds(cfg):
    """Block scales track each block's range, so the forward's error against the bf16
    inputs stays under the per-tensor bounds (with the same room for the kernels)."""
    from fp8_bounds import dequant_mx, quant_mx
    inp = make_workload(cfg, B=BATCH[cfg])
    q8, k8 = dequant_mx(*quant_mx(inp.q)), dequant_mx(*quant_mx(inp.k))
    got = R.gdpa_fwd(q8, k8, inp.f64("v"), inp.q_off, inp.kv_off, inp.act, inp.window)
    ref = R.gdpa_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_off, inp.kv_off, inp.act, inp.window)
    rel, mx = fp8_errors(got, ref)
    assert rel <= FP8_REL_L2 - KERNEL_REL_L2 and mx <= FP8_MAX - KERNEL_MAX, (cfg, rel, mx)
    assert rel >= 0.005, (cfg, rel)
