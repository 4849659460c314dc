"""The host tile planner built with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, CPU only) and run on the five workloads and edge sets: no sanitizer finding,
and every work list equal to the one the library's own build exports.

Source of the planner's rules: GDPA page ("Generalized Dot-Product Attention
(GDPA): kernel optimisation for real recommendation-system training loads"),
"Section details", jagged-input paragraph and zigzag tile-scheduling diagram."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import recsys_attention_jagged_amd as G
from gdpa_workloads import WORKLOADS, offsets, workload_lengths

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "recsys_attention_jagged_amd", "csrc")
DEAL = {"greedy": 0, "zigzag": 1, "round_robin": 2}


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan_sanitize") / "plan_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", CSRC, os.path.join(ROOT, "tests", "native", "plan_sanitize.cpp"),
           os.path.join(CSRC, "plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _run(exe, lq, lk, H, d, window, P=1024, deal="greedy", split=True, team=(0, 0, 0), blocks=(0, 0, 0)):
    head = [len(lq), H, window, d, P, DEAL[deal], int(split), *team, *blocks]
    text = " ".join(map(str, head)) + "\n" + " ".join(map(str, lq)) + "\n" + " ".join(map(str, lk)) + "\n"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], input=text, capture_output=True, text=True, env=env, timeout=300)
    assert p.returncode == 0, p.stderr[-4000:]
    assert "runtime error" not in p.stderr and "Sanitizer" not in p.stderr, p.stderr[-4000:]
    lines = p.stdout.strip().splitlines()
    assert len(lines) == 3
    return [np.array(l.split()[2:], dtype=np.int64) for l in lines]


def _library(lq, lk, H, d, window, P=1024, deal="greedy", split=True, team=(0, 0, 0), blocks=(0, 0, 0)):
    plan = G.gdpa_plan_create(offsets(lq), offsets(lk), len(lq), H, d, window, "bf16", host_only=True,
                              bins=(P, P, P), team=team, blocks=blocks, deal=deal, split=split)
    try:
        return [G.gdpa_plan_export(plan, kind).astype(np.int64) for kind in ("fwd", "dkdv", "dq")]
    finally:
        G.gdpa_plan_destroy(plan)


@pytest.mark.parametrize("cfg", sorted(WORKLOADS))
def test_sanitized_planner_on_workloads(sanitized, cfg):
    w = WORKLOADS[cfg]
    lq, lk = (x.tolist() for x in workload_lengths(cfg))
    for deal in ("greedy", "zigzag"):
        got = _run(sanitized, lq, lk, w["H"], w["d"], w["window"], deal=deal)
        want = _library(lq, lk, w["H"], w["d"], w["window"], deal=deal)
        for g, x in zip(got, want):
            np.testing.assert_array_equal(g, x)


EDGE = [
    ([0, 0, 0], [0, 0, 0], 0, 1),
    ([1], [1], 0, 7),
    ([5, 0, 70, 1, 33, 200], [64, 3, 0, 2, 129, 31], 0, 3),
    ([70, 1, 33, 200, 0, 513], [70, 1, 33, 200, 0, 513], 9, 16),
    ([32] * 6, [1, 4000, 31, 32, 33, 0], 0, 2),
    ([31, 32, 33, 63, 64, 65, 127, 128, 129], [129, 128, 127, 65, 64, 63, 33, 32, 31], 0, 1024),
]


@pytest.mark.parametrize("lq,lk,window,P", EDGE)
@pytest.mark.parametrize("d,team,blocks", [(128, (0, 0, 0), (0, 0, 0)), (128, (2, 2, 1), (1, 1, 1)),
                                           (64, (1, 1, 1), (2, 1, 2))])
@pytest.mark.parametrize("split", [True, False])
def test_sanitized_planner_on_edge_sets(sanitized, lq, lk, window, P, d, team, blocks, split):
    for deal in ("greedy", "zigzag", "round_robin"):
        got = _run(sanitized, lq, lk, 3, d, window, P, deal, split, team, blocks)
        want = _library(lq, lk, 3, d, window, P, deal, split, team, blocks)
        for g, x in zip(got, want):
            np.testing.assert_array_equal(g, x)
