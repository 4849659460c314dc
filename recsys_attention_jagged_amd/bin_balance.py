"""Per-bin load balance of the GDPA kernels, measured with the clock-probe library.

The GDPA page (aitrends.kr/articles/26275, "Section details", the figure of tile
scheduling) compares the per-SM load of round-robin and sorted zigzag scheduling of
jagged tiles (max:min 12:1 against 5:4).  Here every bin is one persistent
workgroup; the clock-probe build stamps the real-time clock (100 MHz) at the start
and the end of each bin's walk, so the busy time of every bin is measured directly.

    python -m recsys_attention_jagged_amd.build --bin-clock      # on the build host
    python -m recsys_attention_jagged_amd.bin_balance [--config 2] [--deals greedy zigzag round_robin]

Prints one JSON line per (deal, kernel): busy time per bin with items (max, mean,
min), max:min and max:mean, the kernel's span (last end - first start), the mean
busy time of the bins in each dispatch round on their CU (a launch of k workgroups
per CU places them in k rounds of one per CU), and the planner's own max:min bin
cost for the list.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--config", default="2", choices=["2", "3", "4", "5"])
    ap.add_argument("--deals", nargs="+", default=["greedy", "zigzag", "round_robin"])
    ap.add_argument("--reps", type=int, default=3, help="launches per kernel; the median one is reported")
    ap.add_argument("--claim", default="bins", choices=["bins", "auto", "always"],
                    help="how workgroups get items (the plan option): with claims, a 'bin' is one workgroup")
    ap.add_argument("--slot-time", default="auto", choices=["auto", "off"],
                    help="the plan's dispatch-slot time factors for the greedy deal (the plan option)")
    ap.add_argument("--dump", default=None, metavar="FILE.npz",
                    help="also save every bin's stamps with its list's exported items")
    args = ap.parse_args(argv)

    import numpy as np
    import torch

    import recsys_attention_jagged_amd as G
    from recsys_attention_jagged_amd.build import LIB_BIN_CLOCK
    from gdpa_workloads import WORKLOADS, make_workload

    if not os.path.exists(LIB_BIN_CLOCK):
        print(f"{LIB_BIN_CLOCK} is not built: python -m recsys_attention_jagged_amd.build --bin-clock",
              file=sys.stderr)
        return 2
    G.LIB_PATH = LIB_BIN_CLOCK          # every call below goes to the clock-probe library
    lib = G.load_library()
    lib.gdpa_debug_bin_clock.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdpa_debug_bin_clock.restype = ctypes.c_int

    cfg = int(args.config)
    inp = make_workload(cfg, device="cuda")
    qo = torch.tensor(inp.q_off, dtype=torch.int32, device="cuda")
    ko = torch.tensor(inp.kv_off, dtype=torch.int32, device="cuda")
    B, H, d, win, act = len(inp.lq), inp.H, inp.d, inp.window, inp.act
    o = torch.empty_like(inp.q)
    dq, dk, dv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)

    def stamps(plan):
        n = ctypes.c_size_t(1 << 16)
        buf = (ctypes.c_ulonglong * n.value)()
        st = lib.gdpa_debug_bin_clock(ctypes.c_void_p(plan.handle), buf, ctypes.byref(n))
        if st != 0:
            raise RuntimeError(G.gdpa_last_error())
        return np.frombuffer(buf, dtype=np.uint64)[:n.value].reshape(-1, 2).astype(np.int64)

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    dump = {}
    for deal in args.deals:
        plan = G.Plan(inp.q_off, inp.kv_off, H, d, win, "bf16", deal=deal, claim=args.claim, slot_time=args.slot_time)
        st = plan.stats()
        h = plan.handle
        kernels = [("fwd", 0, lambda: G.gdpa_fwd(h, inp.q, inp.k, inp.v, qo, ko, B, H, d, act, win, o))]
        if st["bwd_fused"]:
            lst = 1 if st["bwd_fused"] == 1 else 2
            kernels.append(("bwd", lst, lambda: G.gdpa_bwd(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, act,
                                                           win, dq, dk, dv)))
        else:
            kernels.append(("dkdv", 1, lambda: G.gdpa_bwd_dkdv(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d,
                                                               act, win, dk, dv)))
            # dQ from stored dS in two-wave teams walks the plan's list 3
            kernels.append(("dq", 3 if st["dq_team"] == 2 else 2,
                            lambda: G.gdpa_bwd_dq(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, act, win, dq)))
        for name, lst, call in kernels:
            runs = []
            for _ in range(args.reps + 1):      # the first launch warms up
                torch.cuda.synchronize()
                stamps(plan)                    # clear what an earlier launch left
                call()
                torch.cuda.synchronize()
                s = stamps(plan)
                stamps_last = s.copy()
                P = st["dq_team_bins"] if lst == 3 else st["bins"][lst]
                has = s[:P, 1] > 0              # bins with items
                busy_all = (s[:P, 1] - s[:P, 0]) * 10 / 1e3   # us
                busy = busy_all[has]
                span = (s[:P][has, 1].max() - s[:P][has, 0].min()) * 10 / 1e3
                # dispatch round of each bin on its CU: bin p runs on the workgroup at position
                # p % (P / 8) of its XCD's dispatch order, and each round places one per CU
                by_slot = []
                if P % cus == 0 and cus % 8 == 0:
                    slot = (np.arange(P) % (P // 8)) // (cus // 8)
                    by_slot = [round(float(busy_all[(slot == j) & has].mean()), 1)
                               for j in range(P // cus) if np.any((slot == j) & has)]
                runs.append((span, busy, by_slot))
            span, busy, by_slot = sorted(runs[1:], key=lambda r: r[0])[len(runs[1:]) // 2]
            if args.dump:
                dump[f"{deal}_{name}_stamps"] = stamps_last
                dump[f"{deal}_{name}_export"] = np.asarray(G.gdpa_plan_export(h, lst))
            print(json.dumps({
                "workload": WORKLOADS[cfg]["name"], "deal": deal, "claimed": st["claimed"][lst] if lst < 3 else 0,
                "slot_weighted": st["slot_weighted"][lst] if lst < 3 else st["dq_team_slot_weighted"], "kernel": name,
                "bins": int(busy.size),
                "busy_us": {"max": round(float(busy.max()), 1), "mean": round(float(busy.mean()), 1),
                            "min": round(float(busy.min()), 1)},
                "max_over_min": round(float(busy.max() / busy.min()), 3),
                "max_over_mean": round(float(busy.max() / busy.mean()), 3),
                "span_us": round(float(span), 1),
                "busy_by_slot_us": by_slot,
                "planned_cost_max_over_min": (round(st["bin_cost_max"][lst] / max(st["bin_cost_min"][lst], 1), 3)
                                              if lst < 3 else None),
            }), flush=True)
        plan.close()
    if args.dump:
        np.savez(args.dump, **dump)
    return 0


if __name__ == "__main__":
    sys.exit(main())
