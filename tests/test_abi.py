"""CPU tests of the C ABI: the library loads and exports every declared symbol,
host-only plans match the reference planner bit for bit, and argument errors are
reported before anything touches a device.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import recsys_attention_jagged_amd as G
from gdpa_workloads import WORKLOADS, offsets, workload_lengths
from oracle import plan_ref as PR

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gdpa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdpa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = G.load_library()
    names = declared_functions()
    assert "gdpa_fwd" in names and "gdpa_bwd" in names and "gdpa_plan_create" in names
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings_and_poly_bound():
    for code, name in G.STATUS.items():
        assert G.gdpa_status_string(code) == name
    assert 0 < G.gdpa_gelu_poly_bound() < 2e-4
    assert 0 < G.gdpa_gelu_poly_grad_bound() < 2 ** -10


def _poly_header():
    text = open(os.path.join(ROOT, "recsys_attention_jagged_amd", "csrc", "gelu_poly.h")).read()
    num = r"([-+0-9.eE]+)f?"
    radius = float(re.search(r"#define GDPA_GELU_POLY_R " + num, text).group(1))
    tables = {}
    for name in ("kGeluPolyCoef", "kGeluPolyGradCoef"):
        body = re.search(name + r"\[[^]]*\] = \{(.*?)\};", text, flags=re.S).group(1)
        tables[name] = np.array([float(t.strip().rstrip("f")) for t in body.split(",") if t.strip()])
    return radius, tables["kGeluPolyCoef"], tables["kGeluPolyGradCoef"]


def test_gelu_poly_tables_meet_the_library_bounds():
    """The polynomial GELU's coefficient tables, evaluated here in the device's fp32
    Horner order, against the oracle's exact GELU and GELU' on a dense grid that runs
    past the clamp: the errors stay within the bounds the library reports."""
    from oracle import gdpa_ref as R
    radius, a, b = _poly_header()
    x = np.linspace(-2 * radius, 2 * radius, 400_001).astype(np.float32)
    u = x * x
    p = np.zeros_like(u)
    for c in a[::-1]:
        p = (p * u + np.float32(c)).astype(np.float32)
    q = np.zeros_like(u)
    for c in b[::-1]:
        q = (q * u + np.float32(c)).astype(np.float32)
    inside = np.abs(x) <= np.float32(radius)
    f = np.where(inside, np.float32(0.5) * x + p, np.maximum(x, np.float32(0))).astype(np.float64)
    g = np.where(inside, x * q + np.float32(0.5), (x > 0).astype(np.float32)).astype(np.float64)
    xd = x.astype(np.float64)
    ef = np.abs(f - R.act_fwd(xd, "gelu")).max()
    eg = np.abs(g - R.act_grad(xd, "gelu")).max()
    assert ef <= G.gdpa_gelu_poly_bound() * (1 + 1e-6), ef
    assert eg <= G.gdpa_gelu_poly_grad_bound() * (1 + 1e-6), eg
    # and the bounds are tight: the grid comes within a few percent of them
    assert ef >= 0.9 * G.gdpa_gelu_poly_bound() and eg >= 0.9 * G.gdpa_gelu_poly_grad_bound()


def _tail_header():
    text = open(os.path.join(ROOT, "recsys_attention_jagged_amd", "csrc", "gelu_tail.h")).read()
    bound = float(re.search(r"#define GDPA_GELU_TAIL_BOUND ([-+0-9.eE]+)", text).group(1))
    body = re.search(r"kGeluTailCoef\[[^]]*\] = \{(.*?)\};", text, flags=re.S).group(1)
    coef = [float(t.strip().rstrip("f")) for t in body.split(",") if t.strip()]
    return bound, np.array(coef, dtype=np.float32)


def test_gelu_tail_table_meets_its_bound():
    """The forward's exact GELU, max(x, 0) - |x| 2^p(|x|) with the fitted tail p of
    gelu_tail.h, evaluated here in the device's fp32 order (Horner by FMA, exp2 and
    the final FMA rounded to fp32), against the oracle's x Phi(x) on a dense grid
    and far past the fit range (no clamp): the error stays within the header's bound
    (which also carries one ulp of the hardware exp2), and the chain falls to -inf
    far out, where 2^p is 0."""
    from oracle import gdpa_ref as R
    bound, c = _tail_header()
    assert len(c) == 6 and c[-1] < 0

    def fma32(a, b, d):
        with np.errstate(over="ignore"):
            return (a.astype(np.float64) * b.astype(np.float64) + d.astype(np.float64)).astype(np.float32)

    x = np.concatenate([np.linspace(-12, 12, 1_200_001), np.logspace(1, 30, 3001),
                        -np.logspace(1, 30, 3001)]).astype(np.float32)
    z = np.abs(x)
    p = np.full_like(z, c[-1])
    for ck in c[-2::-1]:
        p = fma32(p, z, np.full_like(z, ck))
    t = np.exp2(p.astype(np.float64)).astype(np.float32)
    f = fma32(-z, t, np.maximum(x, np.float32(0)))
    err = np.abs(f.astype(np.float64) - R.act_fwd(x.astype(np.float64), "gelu"))
    assert err.max() <= bound, err.max()
    assert np.all(np.isfinite(f)) and np.all(p[np.abs(x) > 1e10] == -np.inf)


def _host_plan(lq, lk, H, d, window, P=1024, team=(0, 0, 0), blocks=(0, 0, 0), deal="greedy", split=True):
    qo, ko = offsets(lq), offsets(lk)
    return G.gdpa_plan_create(qo, ko, len(lq), H, d, window, "bf16", host_only=True,
                              bins=(P, P, P), team=team, blocks=blocks, deal=deal, split=split)


def _ref_exports(lq, lk, H, window, P, d, layout=None, deal="greedy", split=True):
    layout = layout or PR.auto_layout(list(lq), list(lk), window, d)
    return {kind: PR.export(PR.plan_list(kind, list(lq), list(lk), H, window, P, *layout[kind], mode=deal,
                                         split=split))
            for kind in PR.LISTS}


@pytest.mark.parametrize("cfg,deal", [(1, "greedy"), (2, "greedy"), (3, "greedy"), (4, "greedy"), (5, "greedy"),
                                      (2, "zigzag"), (4, "zigzag")])
def test_plan_bit_exact_vs_reference_on_workloads(cfg, deal):
    w = WORKLOADS[cfg]
    lq, lk = workload_lengths(cfg)
    lq, lk = [int(x) for x in lq], [int(x) for x in lk]
    plan = _host_plan(lq, lk, w["H"], w["d"], w["window"], deal=deal)
    try:
        ref = _ref_exports(lq, lk, w["H"], w["window"], 1024, w["d"], deal=deal)
        for kind in PR.LISTS:
            got = G.gdpa_plan_export(plan, kind)
            np.testing.assert_array_equal(got, np.asarray(ref[kind], dtype=np.int32), err_msg=kind)
        st = G.gdpa_plan_stats(plan)
        assert st["Tq"] == sum(lq) and st["Tk"] == sum(lk)
        for i, kind in enumerate(("fwd", "dkdv", "dq")):
            assert st["n_parts"][i] == max([-1] + [r[5] for r in np.asarray(ref[kind][6 + 1024 + 1:]).reshape(-1, 6)]) + 1
    finally:
        G.gdpa_plan_destroy(plan)


EDGE = [
    ([0, 0, 0], [0, 0, 0], 0),
    ([1], [1], 0),
    ([5, 0, 70, 1, 33, 200], [64, 3, 0, 2, 129, 31], 0),
    ([70, 1, 33, 200, 0, 513], [70, 1, 33, 200, 0, 513], 9),
    ([31, 32, 33, 63, 64, 65, 127, 128, 129], [129, 128, 127, 65, 64, 63, 33, 32, 31], 0),
]


@pytest.mark.parametrize("lq,lk,window", EDGE)
@pytest.mark.parametrize("d,team,blocks", [(64, (1, 1, 1), (1, 1, 1)), (64, (1, 1, 1), (2, 1, 2)),
                                           (128, (2, 2, 2), (1, 1, 1)), (128, (1, 2, 1), (2, 1, 2)),
                                           (128, (0, 0, 0), (0, 0, 0)), (32, (0, 0, 0), (0, 0, 0))])
@pytest.mark.parametrize("P,deal,split", [(1, "greedy", True), (7, "greedy", True), (1024, "greedy", True),
                                          (16, "round_robin", True), (5, "zigzag", True), (3, "greedy", False)])
def test_plan_bit_exact_vs_reference_edge_cases(lq, lk, window, d, team, blocks, P, deal, split):
    plan = _host_plan(lq, lk, 3, d, window, P=P, team=team, blocks=blocks, deal=deal, split=split)
    try:
        auto = PR.auto_layout(list(lq), list(lk), window, d)
        layout = {kind: (team[i] or auto[kind][0], blocks[i] or auto[kind][1])
                  for i, kind in enumerate(("fwd", "dkdv", "dq"))}
        ref = _ref_exports(lq, lk, 3, window, P, d, layout, deal=deal, split=split)
        for kind in PR.LISTS:
            np.testing.assert_array_equal(G.gdpa_plan_export(plan, kind), np.asarray(ref[kind], np.int32))
    finally:
        G.gdpa_plan_destroy(plan)


def test_plan_stats_valid_pairs_and_balance():
    lq, lk = workload_lengths(5, B=16)
    plan = _host_plan(lq, lk, 4, 128, 128)
    try:
        st = G.gdpa_plan_stats(plan)
        from oracle.gdpa_ref import useful_pairs
        assert st["valid_pairs"] == useful_pairs(lq, lk, 128)
        assert all(b == 1024 for b in st["bins"])
    finally:
        G.gdpa_plan_destroy(plan)


def test_plan_picks_one_pass_backward():
    """gdpa_bwd's kernel choice: one KV-stationary pass when every Lk <= 32, one
    Q-stationary pass when every Lq <= 32, else two kernels (never with unfused)."""
    def mode(lq, lk, window=0, **kw):
        p = G.gdpa_plan_create(offsets(lq), offsets(lk), len(lq), 2, 64, window, "bf16", host_only=True, **kw)
        try:
            return G.gdpa_plan_stats(p)["bwd_fused"]
        finally:
            G.gdpa_plan_destroy(p)
    assert mode([300, 5, 0], [32, 1, 0]) == 1
    assert mode([300, 5, 7], [32, 1, 0]) == 0          # queries without keys: dQ rows would have no item
    assert mode([32, 1, 0], [900, 5, 0]) == 2
    assert mode([32, 0, 1], [900, 5, 3]) == 0          # keys without queries
    assert mode([32, 33], [900, 5]) == 0
    assert mode([20, 32], [20, 32], window=4) == 1
    assert mode([300, 5], [32, 1], unfused=True) == 0
    assert mode([300, 5], [32, 1], blocks=(0, 0, 0), team=(0, 0, 0)) == 1
    lq, lk = workload_lengths(3)
    assert mode(list(lq), list(lk)) == 1
    lq, lk = workload_lengths(4)
    assert mode(list(lq), list(lk)) == 2
    lq, lk = workload_lengths(2)
    assert mode(list(lq), list(lk)) == 0


def test_plan_claims_long_item_lists():
    """Items claimed at run time: by default, the lists whose kernel walks them in
    one-wave teams and whose items average 64 steps or more (none of the four bf16
    workloads; PMA-like batches of 8192 keys per sample); never the d = 128 16-row
    dK/dV list or dQ from stored dS; every one-wave list with claim = always; none
    with claim = bins or on an fp32 plan."""
    def claimed(lq, lk, d=64, window=0, dtype="bf16", H=2, **kw):
        p = G.gdpa_plan_create(offsets(lq), offsets(lk), len(lq), H, d, window, dtype, host_only=True, **kw)
        try:
            st = G.gdpa_plan_stats(p)
            return st["claimed"], st["n_items"], st["n_steps"]
        finally:
            G.gdpa_plan_destroy(p)
    want = {2: [0, 0, 0], 3: [0, 0, 0], 4: [0, 0, 0], 5: [0, 0, 0]}
    for cfg in (2, 3, 4, 5):
        w = WORKLOADS[cfg]
        lq, lk = workload_lengths(cfg)
        c, n_items, n_steps = claimed(list(lq), list(lk), d=w["d"], window=w["window"], H=w["H"])
        assert c == want[cfg], (cfg, c)
        for l in range(3):   # the rule: 64 steps or more per item (every item here has steps)
            assert bool(c[l]) == (n_steps[l] >= 64 * n_items[l]) or (cfg in (2, 5) and l > 0), (cfg, l)
    c, n_items, n_steps = claimed([32] * 512, [8192] * 512, d=128, H=4)
    assert c == [1, 0, 1] and n_steps[2] >= 64 * n_items[2], (c, n_items, n_steps)
    lq, lk = [300, 5, 0, 77], [300, 5, 0, 77]
    assert claimed(lq, lk, claim="always")[0] == [1, 1, 1]
    assert claimed(lq, lk, d=128, claim="always")[0][1:] == [0, 0]   # 16-row dK/dV; dQ from stored dS
    assert claimed(lq, lk, claim="bins")[0] == [0, 0, 0]
    assert claimed(lq, lk, dtype="f32", claim="always")[0] == [0, 0, 0]


def test_plan_slot_time_factors():
    """The greedy deal's dispatch-round factors: taken by the d = 128 forward (two-wave
    teams) and dK/dV lists of the jagged and windowed self-attention workloads at four
    workgroups per CU (a host-only plan's bins), by no list of the cross-attention and
    PMA workloads here (their d = 64 forward runs eight per CU on the device, their
    backward is the one-pass kernel), never with explicit bins or slot_time = off.  The
    deal follows the factors: bins of the first dispatch round get about f_last / f_first
    times the streaming steps of those of the last."""
    def plan(lq, lk, d, window, H, **kw):
        return G.gdpa_plan_create(offsets(lq), offsets(lk), len(lq), H, d, window, "bf16", host_only=True, **kw)

    def steps_by_round(p, lst):
        e = np.asarray(G.gdpa_plan_export(p, lst))
        P, n = int(e[0]), int(e[1])
        ptr = e[6:6 + P + 1]
        it = e[6 + P + 1:].reshape(n, 6)
        steps = np.maximum(it[:, 4] - it[:, 3] + 1, 0)
        per_bin = np.add.reduceat(np.append(steps, 0), ptr[:-1])[:P] * (np.diff(ptr) > 0)
        rnd = (np.arange(P) % (P // 8)) // 32   # host-only plans: 256 CUs, 32 per XCD
        return [float(per_bin[rnd == j].mean()) for j in range(4)]

    want = {2: [1, 1, 0], 3: [0, 0, 0], 4: [0, 0, 0], 5: [1, 1, 0]}
    for cfg in (2, 3, 4, 5):
        w = WORKLOADS[cfg]
        lq, lk = workload_lengths(cfg)
        args = (list(lq), list(lk), w["d"], w["window"], w["H"])
        for kw, exp in (({}, want[cfg]), ({"slot_time": "off"}, [0, 0, 0]), ({"bins": (1024, 1024, 1024)}, [0, 0, 0])):
            p = plan(*args, **kw)
            try:
                st = G.gdpa_plan_stats(p)
                assert st["slot_weighted"] == exp, (cfg, kw, st["slot_weighted"])
                if cfg == 5:
                    for lst, f_first, f_last in ((0, 0.92, 1.07), (1, 0.88, 1.07)):
                        r = steps_by_round(p, lst)
                        ratio = r[0] / r[3]
                        target = f_last / f_first if exp[lst] else 1.0
                        assert abs(ratio / target - 1) < 0.03, (kw, lst, r, target)
            finally:
                G.gdpa_plan_destroy(p)


def test_plan_dq_team_list():
    """dQ from stored dS in two-wave teams: a d = 128 two-kernel plan carries list 3, the
    dQ list dealt again as 64-row items (team 2, one block), exported like the others and
    equal to the planner reference's dQ list of that layout; dq_team = one_wave keeps the
    one-wave kernel over the dQ list (no list 3); plans without stored dS (d = 64, a
    one-pass backward) have none, and exporting list 3 from them is an error."""
    lq = [1, 15, 16, 17, 33, 47, 64, 65, 0, 300, 129, 700, 96, 97]
    P = 64

    def plan(d, **kw):
        return G.gdpa_plan_create(offsets(lq), offsets(lq), len(lq), 2, d, 0, "bf16", host_only=True,
                                  bins=(P, P, P), **kw)

    p = plan(128)
    try:
        st = G.gdpa_plan_stats(p)
        assert st["ds_bytes"] > 0 and st["dq_team"] == 2 and st["dq_team_bins"] == P
        ex = list(G.gdpa_plan_export(p, "dq_team"))
        assert ex[2:6] == [64, 32, 2, 1] and ex[1] == st["dq_team_items"]
        assert ex == PR.export(PR.plan_list("dq", lq, lq, 2, 0, P, 2, 1))
    finally:
        G.gdpa_plan_destroy(p)
    p = plan(128, dq_team="one_wave")
    try:
        st = G.gdpa_plan_stats(p)
        assert st["ds_bytes"] > 0 and st["dq_team"] == 1 and st["dq_team_items"] == 0
        with pytest.raises(G.GdpaError):
            G.gdpa_plan_export(p, 3)
    finally:
        G.gdpa_plan_destroy(p)
    p = plan(64)
    try:
        st = G.gdpa_plan_stats(p)
        assert st["ds_bytes"] == 0 and st["dq_team"] == 0
        with pytest.raises(G.GdpaError):
            G.gdpa_plan_export(p, 3)
    finally:
        G.gdpa_plan_destroy(p)


# ---------------------------------------------------------------------------
# error paths (forced from the host)
# ---------------------------------------------------------------------------

def _status_of(fn, *args, **kw):
    with pytest.raises(G.GdpaError) as e:
        fn(*args, **kw)
    return e.value.status


def test_create_rejects_bad_arguments():
    qo = offsets([3, 4])
    bad = lambda **kw: _status_of(G.gdpa_plan_create, kw.pop("qo", qo), kw.pop("ko", qo), kw.pop("B", 2),
                                  kw.pop("H", 2), kw.pop("d", 64), kw.pop("window", 0),
                                  kw.pop("dtype", "bf16"), host_only=True, **kw)
    assert bad(d=48) == 3                      # UNSUPPORTED
    assert bad(d=256) == 3
    assert bad(H=0) == 1                       # INVALID_ARG
    assert bad(window=-1) == 1
    assert bad(dtype=7) == 1
    assert bad(blocks=(3, 0, 0)) == 1
    assert bad(blocks=(0, 2, 0)) == 1          # dK/dV: one kv block per wave
    assert bad(blocks=(0, 0, -1)) == 1
    assert bad(team=(3, 0, 0)) == 1
    assert bad(team=(2, 0, 0)) == 1            # two-wave teams only at d = 128
    assert bad(claim=3) == 1
    assert bad(claim=-1) == 1
    assert bad(slot_time=2) == 1
    assert bad(slot_time=-1) == 1
    assert bad(dq_team=2) == 1
    assert bad(dq_team=-1) == 1
    assert bad(d=128, team=(0, 0, 2), blocks=(0, 0, 2)) == 1   # two-wave teams: one block per wave
    assert bad(d=128, team=(2, 0, 0), blocks=(2, 0, 0)) == 1
    assert bad(qo=np.array([1, 3, 7], np.int32)) == 2           # BAD_OFFSETS: not starting at 0
    assert bad(qo=np.array([0, 5, 3], np.int32)) == 2           # decreasing
    assert bad(ko=offsets([3, 5]), window=4) == 2               # window with Lq != Lk
    lib = G.load_library()
    out = ctypes.c_void_p()
    assert lib.gdpa_plan_create(None, None, 1, 1, 64, 0, 1, None, None, ctypes.byref(out)) == 1
    assert lib.gdpa_plan_create(qo.ctypes.data, qo.ctypes.data, 2, 1, 64, 0, 1, None, None, None) == 1
    assert "NULL" in G.gdpa_last_error()


def test_calls_reject_host_only_and_mismatched_plans():
    qo = offsets([3, 4])
    plan = G.gdpa_plan_create(qo, qo, 2, 2, 64, 0, "bf16", host_only=True)
    try:
        fake = 1 << 20   # never dereferenced: validation fails first
        assert _status_of(G.gdpa_fwd, plan, fake, fake, fake, fake, fake, 2, 2, 64, "gelu", 0, fake, 0) == 4
        assert _status_of(G.gdpa_bwd, plan, fake, fake, fake, fake, fake, fake, 2, 2, 64, "gelu", 0,
                          fake, fake, fake, 0) == 4
        assert _status_of(G.gdpa_fwd, None, fake, fake, fake, fake, fake, 2, 2, 64, "gelu", 0, fake, 0) == 1
        assert _status_of(G.gdpa_plan_export, plan, 5) == 1
    finally:
        G.gdpa_plan_destroy(plan)
    G.gdpa_plan_destroy(None)


def test_oversized_sample_is_unsupported():
    qo = np.array([0, 1 << 22], np.int32)     # 4M rows x 8 heads x 128 x 2 B > 2 GiB per slice
    assert _status_of(G.gdpa_plan_create, qo, qo, 1, 8, 128, 0, "bf16", host_only=True) == 3


def test_export_capacity_check():
    qo = offsets([300])
    plan = G.gdpa_plan_create(qo, qo, 1, 1, 64, 0, "bf16", host_only=True)
    try:
        lib = G.load_library()
        n = ctypes.c_size_t(0)
        assert lib.gdpa_plan_export(plan, 0, None, ctypes.byref(n)) == 0 and n.value > 0
        small = np.zeros(2, np.int32)
        m = ctypes.c_size_t(2)
        assert lib.gdpa_plan_export(plan, 0, small.ctypes.data, ctypes.byref(m)) == 1
        assert m.value == n.value
    finally:
        G.gdpa_plan_destroy(plan)


def test_pffn_host_plan_is_one_sample():
    """A pFFN plan is the plan of one sample holding every query row and the M
    weight rows, bit for bit; only its own calls accept it."""
    Tq, M = 1000, 300
    h = G.gdpa_pffn_plan_create(Tq, M, 2, 64, "bf16", host_only=True, bins=(16, 16, 16))
    try:
        ref = _ref_exports([Tq], [M], 2, 0, 16, 64)
        for kind in PR.LISTS:
            np.testing.assert_array_equal(G.gdpa_plan_export(h, kind), np.asarray(ref[kind], np.int32))
        st = G.gdpa_plan_stats(h)
        assert st["Tq"] == Tq and st["Tk"] == M and st["valid_pairs"] == Tq * M
        assert G.STATUS[_status_of(G.gdpa_pffn_fwd, h, None, None, None, "silu", None, 0)] == "GDPA_ERR_PLAN_MISMATCH"
    finally:
        G.gdpa_plan_destroy(h)
    assert G.STATUS[_status_of(G.gdpa_pffn_plan_create, -1, 3, 2, 64, "bf16", host_only=True)] == "GDPA_ERR_INVALID_ARG"


def test_noalloc_forward_rejects_a_plan_beyond_its_scratch_before_any_device_call():
    """gdpa_fwd_noalloc checks the plan's forward list against its fixed 32 MiB scratch
    on the host: 20 samples x 60000 heads make 1.2 M forward items (57.6 MB of records),
    refused with INVALID_ARG before anything touches a device (none is present here)."""
    lq = [64] * 20
    qo = offsets(lq)
    plan = G.gdpa_plan_create(qo, qo, 20, 60000, 128, 0, "bf16", host_only=True)
    try:
        assert G.gdpa_plan_stats(plan)["n_items"][0] == 20 * 60000
        fake = 1 << 20   # never dereferenced
        st = G.load_library().gdpa_fwd_noalloc(plan, fake, fake, fake, fake, fake, 20, 60000, 128, 0, 0, fake, 0)
        assert G.STATUS[st] == "GDPA_ERR_INVALID_ARG"
        assert "bytes of scratch" in G.gdpa_last_error()
    finally:
        G.gdpa_plan_destroy(plan)
