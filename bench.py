"""Benchmark of the weight-informed activation-sparse linear on one MI355X.

Headline workload: the Llama-2-7B-shaped FFN down projection, W 4096 x 11008
bf16 (std 0.02), x = SiLU(g) * u with g, u ~ N(0, 1) rounded to bf16, one
token per step (batch-1 decode), WINA top-K at 50 % sparsity (K = 5504, the
headline) and 65 % sparsity (K = 3853). A step is one full forward, one fused
launch: a gate workgroup (scores, top-K select) and the product workgroups
(predicate, compaction, gather-GEMV).

Weights rotate through 12 handle-owned copies (1.08 GB) so the 256 MB
Infinity Cache never serves them; tokens rotate through 256 seeded tokens held
in HBM. Before a leg is timed every ring copy runs once untimed (each copy's
speculation starts from its own previous threshold, whatever --warmup is).
Steps are captured into HIP graphs and replayed; the timed region is bracketed
by torch.cuda.synchronize() and, inside it, by HIP events on the replay stream:
tokens/s and ms per step come from the events (the wall clock of the bracket
is reported beside them). The same-kernel dense forward is timed the same way,
so speedup_vs_dense compares like with like; a kernel-to-kernel speed-up
(average launch durations from HIP events around 600 back-to-back launches)
is reported beside it.

Printed: one JSON line with tokens/s, ms per step, the fused kernel's
achieved HBM bandwidth on algorithmic bytes against the 8 TB/s peak, the
same-kernel dense baseline, the practical gather ceiling (a read-only kernel
streaming the same kept columns), hipBLASLt's dense GEMV for context, and the
CPU oracle timed on the host at one thread and at all threads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-GEMV tokens/s & achieved HBM GB/s at 50%/65% sparsity, bf16"
PEAK_GBS = 8000.0
RING = 12
NTOK = 256
KERNEL_LAUNCHES = 600  # back-to-back launches per kernel-duration measurement


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle budget (split between the one-thread and all-thread runs)")
    ap.add_argument("--only", choices=["sparse50", "sparse65", "fixed50", "dense", "ceiling", "all", "r8_k512",
                                       "r16_k256"],
                    default="all",
                    help="restrict the measured legs (short profiler runs of one leg)")
    ap.add_argument("--counters-run", action="store_true",
                    help="short eager run for memory-counter passes: 12 + 48 headline forwards "
                         "(K=5504), then three plain 256 MiB device copies; prints one line")
    ap.add_argument("--timeline", action="store_true",
                    help="per-workgroup timelines of the fused forward from the timeline build of the library "
                         "(Llama-2-7B down at K=5504 and K=3853, Phi-4 gate and down with the statistical gate); "
                         "prints one line of phase times")
    ap.add_argument("--workload", default="llama7b_down",
                    choices=["llama7b_down", "llama3_block", "phi4_ffn_stat", "qwen_ffn_b16", "llama2_ffn_chain",
                             "llama2_ds_decode"],
                    help="llama7b_down is the headline; the others measure the remaining layer shapes")
    return ap.parse_args(argv)


def algorithmic_bytes(m, n, K, B=1):
    """Bytes one forward must move: the kept columns (K*m bf16), x and c for
    every input (n*(2+4)), and y (m fp32)."""
    return K * m * 2 + B * n * 2 + n * 4 + B * m * 4


FUSED_SOURCES = ["fused.hip", "gate_body.h", "product_body.h", "device_common.h"]
DS_SOURCES = ["double_sparse.hip", "gate_body.h", "device_common.h"]


def sources_sha256(names):
    """sha256 over the named kernel sources, in order (identifies the build the
    memory counters were taken from)."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "free_activation_sparse_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile(kernel, sources, K):
    """HBM bytes per launch of `kernel` from the committed memory-counter
    summary, or None when its sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_memory_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source sha256: ([0-9a-f]{64})", text)
    if not m or m.group(1) != sources_sha256(sources):
        return None
    t = re.search(r"bytes per launch \(K=%d\): (\d+)" % K, text)
    return int(t.group(1)) if t else None


# ---------------------------------------------------------------------------
# Timing helpers (f(i, stream) enqueues step i on the given HIP stream)
# ---------------------------------------------------------------------------
def _capture(torch, f, count, first=0):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream()
        for i in range(first, first + count):
            f(i, s.cuda_stream)
    return g


def prime(torch, f, count):
    """Untimed eager calls 0 .. count-1 (every ring copy and token slot once)."""
    s = torch.cuda.current_stream().cuda_stream
    for i in range(count):
        f(i, s)
    torch.cuda.synchronize()


def timed_steps(torch, f, steps, warmup, G=120):
    """Warm up, then time exactly `steps` calls of f replayed from HIP graphs
    of up to G calls. Returns (seconds between HIP events recorded on the
    replay stream around the timed replays, wall seconds of the
    synchronize-bracketed region)."""
    cache = {}

    def graph_of(count):
        if count not in cache:
            cache[count] = _capture(torch, f, count)
        return cache[count]
    full, tail = divmod(steps, G)
    wfull, wtail = divmod(warmup, G)
    plan_warm = [G] * wfull + ([wtail] if wtail else [])
    plan_timed = [G] * full + ([tail] if tail else [])
    for cnt in set(plan_warm + plan_timed):
        graph_of(cnt)
    for cnt in plan_warm:
        cache[cnt].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for cnt in plan_timed:
        cache[cnt].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) * 1e-3, wall


def graph_us(torch, f, count=KERNEL_LAUNCHES):
    """Average microseconds per call of f, from HIP events on the replay
    stream around one replay of a graph of `count` back-to-back calls (after
    one untimed replay of the same graph)."""
    g = _capture(torch, f, count)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / count


def _r(v, nd=4):
    return round(v, nd) if isinstance(v, float) else v


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the sparse linear is measured on one GPU; split by output rows, each GPU would run the same "
              "kernels on its own rows with no exchange before the product)",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "llama2_ffn_chain":
        return run_ffn_chain(args)
    if args.workload == "llama2_ds_decode":
        return run_ds_decode(args)
    if args.workload != "llama7b_down":
        return run_workload(args)
    if args.counters_run:
        return counters_run()
    if args.timeline:
        return run_timeline()
    return run_headline(args)


def run_headline(args):
    import numpy as np
    import torch

    import free_activation_sparse_amd as fas
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m, n = 4096, 11008
    Wh = wl.weight(2, 0)
    Wd = torch.from_numpy(Wh.view(np.int16)).to(dev).view(torch.bfloat16)
    X = torch.from_numpy(wl.tokens(2, 0, 0, NTOK).view(np.int16)).to(dev).view(torch.bfloat16).contiguous()
    Ks = {"sparse50": wl.k_from_sparsity(n, 0.5), "sparse65": wl.k_from_sparsity(n, 0.65)}
    Y = torch.empty((RING, m), dtype=torch.float32, device=dev)

    def make_ring(**gate):
        return [fas.SparseLinear(Wd, c=None, **gate) for _ in range(RING)]

    def layer_step(ring, dense=False):
        """f(i, stream): forward of token i % 256 through ring copy i % 12."""
        def f(i, s):
            h, x, y = ring[i % RING], X[i % NTOK], Y[i % RING]
            if dense:
                fas.sparse_linear_forward_dense(h.handle, x.data_ptr(), 1, y.data_ptr(), fas.SL_F32, s)
            else:
                fas.sparse_linear_forward(h.handle, x.data_ptr(), 1, y.data_ptr(), fas.SL_F32, 0, 0, 0, s)
        return f

    def stage_step(ring, bit):
        def f(i, s):
            k = i % RING
            fas.sparse_linear_forward_stages(ring[k].handle, X[k].data_ptr(), 1, Y[k].data_ptr(), fas.SL_F32,
                                             0, 0, 0, bit, s)
        return f

    def sync_all(ring):
        for h in ring:
            h.sync_status()  # raises if a fused hand-off timed out in any timed call

    # Fixed (calibrated) threshold leg: tau = the median score over the 256
    # tokens (scores from the library's norms; plain numpy on the host, outside
    # any timed region), so that about half of each token's inputs are kept
    fixed_tau, fixed_kept = None, None
    want = {"all": ("sparse50", "sparse65", "fixed50", "dense", "ceiling")}.get(args.only, (args.only,))
    if "fixed50" in want:
        probe = fas.SparseLinear(Wd, c=None, gate="topk", K=1)
        c_host = probe.norms().cpu().numpy().astype(np.float64)
        probe.close()
        xs = (wl.tokens(2, 0, 0, NTOK).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        sc = (np.abs(xs) * c_host[None, :]).astype(np.float32)
        fixed_tau = float(np.median(sc))
        fixed_kept = float((sc > np.float32(fixed_tau)).sum(axis=1).mean())

    results = {}
    for leg in ("sparse50", "sparse65", "fixed50"):
        if leg not in want:
            continue
        if leg == "fixed50":
            K = fixed_kept  # mean kept count over the tokens (algorithmic bytes)
            ring = make_ring(gate="fixed", tau=fixed_tau)
        else:
            K = Ks[leg]
            ring = make_ring(gate="topk", K=K)
        step = layer_step(ring)
        prime(torch, step, 2 * RING)
        ev, wall = timed_steps(torch, step, args.steps, args.warmup)
        fused_us = graph_us(torch, step)
        sync_all(ring)
        # the two-launch form (gate kernel, then product kernel), and each of
        # its kernels alone (ring copy i keeps the selection of token i, so the
        # product-only launches move exactly the bytes of a full forward)
        for h in ring:
            h.set_fused(False)
        two_us = graph_us(torch, step)
        prime(torch, step, RING)
        gate_us = None
        if leg != "fixed50":  # a fixed threshold without outputs launches no gate kernel
            gate_us = graph_us(torch, stage_step(ring, fas.SL_STAGE_GATE))
        prod_us = graph_us(torch, stage_step(ring, fas.SL_STAGE_PRODUCT))
        for h in ring:
            h.set_fused(True)
        ab = algorithmic_bytes(m, n, K)
        results[leg] = {
            "K": K, "sparsity": 1 - K / n,
            **({"tau": fixed_tau, "gate": "fixed threshold (median score of the 256 tokens)"} if leg == "fixed50" else {}),
            "tokens_per_s": args.steps / ev, "us_per_step": ev / args.steps * 1e6,
            "wall_us_per_step": wall / args.steps * 1e6,
            "fused_kernel_us": fused_us, "algorithmic_bytes": ab,
            "fused_achieved_GBps": ab / (fused_us * 1e-6) / 1e9,
            "step_achieved_GBps": ab / (ev / args.steps) / 1e9,
            "two_launch_us_per_step": two_us,
            "gate_kernel_us": gate_us, "product_kernel_us": prod_us,
            "product_achieved_GBps": ab / (prod_us * 1e-6) / 1e9,
        }
        for h in ring:
            h.close()
        del ring

    dense = None
    if "dense" in want:
        ring = make_ring(gate="topk", K=Ks["sparse50"])
        step = layer_step(ring, dense=True)
        prime(torch, step, RING)
        ev_a, wall_a = timed_steps(torch, step, args.steps, args.warmup)
        k_a = graph_us(torch, step)
        # the ordered split reduction needs no clearing of y (no fill kernel
        # before the product): the speed-ups are taken against the faster form
        for h in ring:
            h.set_deterministic(True)
        ev_o, wall_o = timed_steps(torch, step, args.steps, args.warmup)
        k_o = graph_us(torch, step)
        for h in ring:
            h.set_deterministic(False)
        ab = algorithmic_bytes(m, n, n)
        dense = {"us_per_step_atomic": ev_a / args.steps * 1e6, "us_per_step_ordered": ev_o / args.steps * 1e6,
                 "launch_us_atomic": k_a, "launch_us_ordered": k_o,
                 "best_us_per_step": min(ev_a, ev_o) / args.steps * 1e6, "best_launch_us": min(k_a, k_o),
                 "algorithmic_bytes": ab, "achieved_GBps": ab / (min(k_a, k_o) * 1e-6) / 1e9}
        for h in ring:
            h.close()
        del ring
        # hipBLASLt / rocBLAS dense GEMV on the row-major weights, for context
        Wr = [Wd.clone() for _ in range(RING)]
        Yb = torch.empty((RING, m), dtype=torch.bfloat16, device=dev)

        def mv(i):
            torch.matmul(Wr[i % RING], X[i % NTOK], out=Yb[i % RING])
        for i in range(2 * RING):
            mv(i)
        # hipBLASLt calls are not captured in a graph here: time them eagerly
        # between two events, with the GPU first asleep so the host runs ahead
        count = 1200
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(100_000_000)
        e0.record()
        for i in range(count):
            mv(i)
        e1.record()
        torch.cuda.synchronize()
        dense["torch_matmul_us_per_step"] = e0.elapsed_time(e1) * 1e3 / count
        del Wr

    ceiling = {}
    if "ceiling" in want:
        # the practical ceiling: a read-only kernel streaming each token's own
        # kept columns (the masks come from the library's forward, untimed)
        sink = torch.zeros(1, dtype=torch.float32, device=dev)
        for leg, K in Ks.items():
            ring = make_ring(gate="topk", K=K)
            mk = torch.empty((RING, n), dtype=torch.uint8, device=dev)
            s0 = torch.cuda.current_stream().cuda_stream
            for r in range(RING):
                fas.sparse_linear_forward(ring[r].handle, X[r].data_ptr(), 1, Y[r].data_ptr(), fas.SL_F32,
                                          mk[r].data_ptr(), 0, 0, s0)
            torch.cuda.synchronize()
            idx = [torch.nonzero(mk[r]).flatten().to(torch.int32).contiguous() for r in range(RING)]
            counts = [int(t.numel()) for t in idx]
            assert all(c == K for c in counts), counts

            def gath(i, s, ring=ring, idx=idx):
                r = i % RING
                fas.sparse_linear_gather_ceiling(ring[r].handle, idx[r].data_ptr(), idx[r].numel(), sink.data_ptr(), s)
            us = graph_us(torch, gath)
            kept_bytes = K * m * 2
            ceiling[leg] = {"K": K, "launch_us": us, "kept_weight_bytes": kept_bytes,
                            "achieved_GBps": kept_bytes / (us * 1e-6) / 1e9,
                            "frac_of_peak": kept_bytes / (us * 1e-6) / 1e9 / PEAK_GBS}
            for h in ring:
                h.close()
            del ring

    cpu = None
    if not args.no_cpu and "sparse50" in results:
        cpu = cpu_baseline(wl, Wh, Ks["sparse50"], args.cpu_seconds)

    head = results.get("sparse50") or results.get("sparse65") or results.get("fixed50")
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"] if head else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_step"] * 1e-3 if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama2_7b_down_proj_4096x11008_bf16_topk_50pct",
                   "m": m, "n": n, "K": Ks["sparse50"], "batch": 1, "tokens": NTOK,
                   "weight_ring_copies": RING, "weight_ring_bytes": RING * m * n * 2,
                   "launch": "graph", "timing": "HIP events around the timed graph replays"},
    }
    if head:
        out["wall_ms_per_step"] = head["wall_us_per_step"] * 1e-3
        K0 = head["K"]
        out["roofline"] = {
            "bound": "hbm",
            "achieved": round(head["fused_achieved_GBps"], 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["fused_achieved_GBps"] / PEAK_GBS, 4),
            "traffic": traffic_from_profile("fused_kernel", FUSED_SOURCES, K0) if isinstance(K0, int) else None,
            "kernel": "fused_kernel (gate workgroup + gather-GEMV workgroups)",
            "kernel_us": round(head["fused_kernel_us"], 3),
            "algorithmic_bytes": head["algorithmic_bytes"],
        }
    out["cpu_baseline"] = cpu
    out["legs"] = {k: {kk: _r(vv) for kk, vv in v.items()} for k, v in results.items()}
    if dense:
        out["dense_same_kernel"] = {k: _r(v) for k, v in dense.items()}
        for k, v in results.items():
            bar = 0.8 / (1 - v["sparsity"])
            out["legs"][k]["speedup_vs_dense"] = round(dense["best_us_per_step"] / v["us_per_step"], 4)
            out["legs"][k]["kernel_speedup_vs_dense"] = round(dense["best_launch_us"] / v["fused_kernel_us"], 4)
            out["legs"][k]["speedup_bar"] = round(bar, 4)
    if ceiling:
        out["gather_ceiling"] = {k: {kk: _r(vv) for kk, vv in v.items()} for k, v in ceiling.items()}
        for k, v in ceiling.items():
            if k in results:
                out["legs"][k]["fused_vs_ceiling"] = round(v["launch_us"] / results[k]["fused_kernel_us"], 4)
    out["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(out))


# ---------------------------------------------------------------------------
# Other layer shapes: a step is one forward of every linear of the workload for
# a batch of B tokens (ring copies of the weights so that >= 1 GiB rotates).
# ---------------------------------------------------------------------------
def workload_legs(name):
    """[(leg name, B, [(cfg, linear, gate kwargs), ...], groups or None)]"""
    import workloads as wl
    if name == "llama3_block":
        ps = wl.component_sparsities(3)
        lins = [(3, li, dict(gate="topk", K=wl.k_from_sparsity(l.n, round(ps[li], 6))))
                for li, l in enumerate(wl.CONFIGS[3].linears)]
        # "grouped": the linears that share an input in one launch each
        # (q, k, v | o | gate, up | down: 4 launches instead of 7)
        names = [l.name for l in wl.CONFIGS[3].linears]
        groups = [[names.index(a) for a in g] for g in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))]
        return [("grouped", 1, lins, groups), ("block", 1, lins, None)]
    if name == "phi4_ffn_stat":
        lins = [(4, li, dict(gate="stat", s_keep=0.10)) for li in range(3)]
        # "B1_grouped": gate and up in one launch (gate's token for both), then down;
        # "B<b>_grouped": gate and up's gates for the batch in one launch, then
        # each linear's union product, then down
        legs = [("B1_grouped", 1, lins, [[0, 1], [2]]), ("B1", 1, lins, None)]
        for b in (2, 4, 8):
            legs += [(f"B{b}_grouped", b, lins, [[0, 1], [2]]), (f"B{b}", b, lins, None)]
        return legs
    if name == "qwen_ffn_b16":
        legs = []
        for p in (0.65, 0.90):
            lins = [(5, li, dict(gate="topk", K=wl.k_from_sparsity(wl.CONFIGS[5].linears[li].n, p)))
                    for li in range(3)]
            # gate and up share x: their 2 x 16 gates in one launch ("_grouped")
            legs.append((f"p{int(p * 100)}_grouped", 16, lins, [[0, 1], [2]]))
            legs.append((f"p{int(p * 100)}", 16, lins, None))
        return legs
    raise ValueError(name)


def run_workload(args):
    import numpy as np
    import torch

    import free_activation_sparse_amd as fas
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    legs = workload_legs(args.workload)
    NT = 48  # token batches rotated through
    host_w = {}

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    results = {}
    for leg, B, lins, groups in legs:
        total = sum(wl.CONFIGS[cfg].linears[li].m * wl.CONFIGS[cfg].linears[li].n * 2 for cfg, li, _ in lins)
        R = max(2, -(-(1 << 30) // total))
        rings, Xs, Ys, dims = [], [], [], []
        for cfg, li, gk in lins:
            lin = wl.CONFIGS[cfg].linears[li]
            if (cfg, li) not in host_w:
                host_w[(cfg, li)] = wl.weight(cfg, li)
            Wd = dev_bf16(host_w[(cfg, li)])
            rings.append([fas.SparseLinear(Wd, c=None, max_batch=B, **gk) for _ in range(R)])
            del Wd
            toks = np.stack([wl.tokens(cfg, li, t * B, B) for t in range(NT)])
            Xs.append(dev_bf16(toks).reshape(NT, B, lin.n).contiguous())
            Ys.append(torch.empty((R, B, lin.m), dtype=torch.float32, device=dev))
            dims.append((lin.name, lin.m, lin.n))
        # launch units: groups of linears sharing x (one launch each), or one
        # linear per unit
        units = groups if groups is not None else [[L] for L in range(len(lins))]

        def unit_step(u, dense=False):
            def f(i, s):
                if len(u) > 1 and not dense:
                    # a group's linears share x (the tokens of its first linear)
                    fas.sparse_linear_forward_group_batch([rings[L][i % R].handle for L in u],
                                                          Xs[u[0]][i % NT].data_ptr(), B,
                                                          [Ys[L][i % R].data_ptr() for L in u], fas.SL_F32, s)
                    return
                for L in u:
                    h = rings[L][i % R]
                    x = Xs[u[0] if groups is not None else L][i % NT].data_ptr()
                    if dense:
                        fas.sparse_linear_forward_dense(h.handle, x, B, Ys[L][i % R].data_ptr(), fas.SL_F32, s)
                    else:
                        fas.sparse_linear_forward(h.handle, x, B, Ys[L][i % R].data_ptr(), fas.SL_F32, 0, 0, 0, s)
            return f

        def step_of(dense):
            fs = [unit_step(u, dense) for u in units]

            def f(i, s):
                for g in fs:
                    g(i, s)
            return f

        step = step_of(False)
        prime(torch, step, 2 * R)
        ev, wall = timed_steps(torch, step, args.steps, args.warmup, G=60)
        unit_us = [graph_us(torch, unit_step(u), count=240) for u in units]
        for ring in rings:
            for h in ring:
                h.sync_status()
        dstep = step_of(True)
        prime(torch, dstep, R)
        dsteps = max(20, args.steps // 4)
        dev_s, _ = timed_steps(torch, dstep, dsteps, min(args.warmup, dsteps), G=60)
        dense_unit_us = [graph_us(torch, unit_step(u, True), count=120) for u in units]
        # untimed side pass: kept (B = 1) or union (B > 1) column counts per
        # linear, from the library's masks (one token batch per ring copy)
        kept = []
        for L, (name, m, n) in enumerate(dims):
            mk = torch.empty((B, n), dtype=torch.uint8, device=dev)
            tot = 0
            x_of = (lambda t: Xs[[u for u in units if L in u][0][0]][t]) if groups is not None else (lambda t: Xs[L][t])
            for t in range(NT):
                fas.sparse_linear_forward(rings[L][0].handle, x_of(t).data_ptr(), B, Ys[L][0].data_ptr(),
                                          fas.SL_F32, mk.data_ptr(), 0, 0, torch.cuda.current_stream().cuda_stream)
                tot += int(mk.bool().any(dim=0).sum().item())
            kept.append(tot / NT)
        lin_rows, unit_rows = [], []
        tot_bytes, touched_w = 0, 0
        lin_bytes = []
        for L, (name, m, n) in enumerate(dims):
            ab = kept[L] * m * 2 + B * n * 2 + n * 4 + B * m * 4
            lin_bytes.append(ab)
            tot_bytes += ab
            touched_w += kept[L] * m * 2
            lin_rows.append({"linear": name, "m": m, "n": n, "columns_read": round(kept[L], 1),
                             "column_density": round(kept[L] / n, 4)})
        for ui, u in enumerate(units):
            ub = sum(lin_bytes[L] for L in u)
            unit_rows.append({"linears": [dims[L][0] for L in u], "launch_us": round(unit_us[ui], 3),
                              "dense_launch_us": round(dense_unit_us[ui], 3),
                              "algorithmic_bytes": round(ub),
                              "achieved_GBps": round(ub / (unit_us[ui] * 1e-6) / 1e9, 1)})
        us_step = ev / args.steps * 1e6
        dense_us_step = dev_s / dsteps * 1e6
        density = touched_w / total
        kernel = ("fused_group_kernel" if groups is not None else "fused_kernel") if B == 1 else \
            ("gate_group_kernel + union_kernel (per linear)" if groups is not None else
             "gate_kernel + union_kernel (per linear)")
        res = {"B": B, "tokens_per_s": B * args.steps / ev, "us_per_step": us_step,
               "wall_us_per_step": wall / args.steps * 1e6,
               "launch_us_sum": sum(unit_us), "algorithmic_bytes": tot_bytes,
               "achieved_GBps": tot_bytes / (sum(unit_us) * 1e-6) / 1e9, "kernel": kernel,
               "dense_same_kernel_us_per_step": dense_us_step,
               "speedup_vs_dense": dense_us_step / us_step,
               "kernel_speedup_vs_dense": sum(dense_unit_us) / sum(unit_us),
               "dense_weight_bytes": total, "touched_weight_bytes": round(touched_w),
               "touched_density": density, "ring_copies": R, "linears": lin_rows, "launches": unit_rows}
        if B == 1:
            res["speedup_bar"] = 0.8 / density  # 0.8 x dense / touched bytes
        else:
            # iid tokens keep 1 - (1 - f)^B of the columns between them: the
            # union bound caps any speed-up at dense / touched bytes
            res["union_bound"] = 1.0 / density
            res["speedup_vs_union_bound"] = (dense_us_step / us_step) / (1.0 / density)
        results[leg] = res
        for ring in rings:
            for h in ring:
                h.close()
        del rings, Xs, Ys
        torch.cuda.empty_cache()

    first = legs[0][0]
    head = results[first]
    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["us_per_step"] * 1e-3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": {"workload": args.workload, "headline_leg": first, "launch": "graph",
                                        "timing": "HIP events around the timed graph replays"},
        "roofline": {"bound": "hbm", "achieved": round(head["achieved_GBps"], 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(head["achieved_GBps"] / PEAK_GBS, 4), "traffic": None,
                     "kernel": head["kernel"] + " (summed algorithmic bytes / summed launch durations of one step)"},
        "cpu_baseline": None if args.no_cpu else workload_cpu_baseline(legs[0], host_w, min(args.cpu_seconds, 10.0)),
        "legs": {k: {kk: _r(vv) for kk, vv in v.items()} for k, v in results.items()},
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out))


def run_ffn_chain(args):
    """Sparse FFN chain of one token on Llama-2-7B FFN shapes (gate/up
    11008 x 4096, down 4096 x 11008, bf16 std 0.02, seeded synthetic weights;
    hidden state x ~ N(0,1)), WINA top-K at 50 % on each projection: the
    grouped gate/up launch, the SiLU(g) u epilogue and the down projection's
    fused forward, all on the device (sparse_linear_forward_ffn)."""
    import numpy as np
    import torch

    import free_activation_sparse_amd as fas
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    n, m = 4096, 11008
    Ks = (2048, 2048, 5504)
    shapes = ((m, n), (m, n), (n, m))
    host = [wl.random_matrix(300 + i, a, b, "bf16") for i, (a, b) in enumerate(shapes)]
    R = max(2, -(-(1 << 30) // sum(a * b * 2 for a, b in shapes)))
    rings = []
    for W, K in zip(host, Ks):
        Wd = torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).to(dev).view(torch.bfloat16)
        rings.append([fas.SparseLinear(Wd, c=None, gate="topk", K=K) for _ in range(R)])
        del Wd
    NT = 64
    X = torch.from_numpy(wl.random_tokens(310, NT, n, "bf16", "normal").view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty((R, n), dtype=torch.float32, device=dev)
    nb = fas.sparse_linear_ffn_workspace_bytes(rings[1][0].handle)
    WS = torch.empty((R, (nb + 255) // 256 * 256), dtype=torch.uint8, device=dev)

    def step(i, s):
        r = i % R
        fas.sparse_linear_forward_ffn(rings[0][r].handle, rings[1][r].handle, rings[2][r].handle,
                                      X[i % NT].data_ptr(), Y[r].data_ptr(), fas.SL_F32, WS[r].data_ptr(),
                                      WS.shape[1], s)
    prime(torch, step, 2 * R)
    ev, wall = timed_steps(torch, step, args.steps, args.warmup, G=60)
    for ring in rings:
        for h in ring:
            h.sync_status()
    kept_bytes = sum(K * a * 2 for K, (a, b) in zip(Ks, shapes))
    dense_bytes = sum(a * b * 2 for a, b in shapes)
    us = ev / args.steps * 1e6
    out = {"metric": "sparse FFN chain tokens/s (Llama-2-7B FFN shapes, top-K 50 % per projection)",
           "value": args.steps / ev, "unit": "tokens/s", "ms_per_step": us * 1e-3,
           "wall_ms_per_step": wall / args.steps * 1e3,
           "config": {"workload": "llama2_7b_ffn_chain_gate_up_11008x4096_down_4096x11008_bf16_topk_50pct",
                      "K": Ks, "weight_ring_copies": R, "timing": "HIP events around the timed graph replays"},
           "kept_weight_bytes": kept_bytes, "dense_weight_bytes": dense_bytes,
           "kept_GBps": kept_bytes / (us * 1e-6) / 1e9, "launches_per_token": 3,
           "data": "synthetic", "device": torch.cuda.get_device_name(0),
           "cpu_baseline": None if args.no_cpu else ffn_cpu_baseline(
               host, Ks, wl.random_tokens(310, 8, n, "bf16", "normal"), min(args.cpu_seconds, 10.0))}
    print(json.dumps(out))
    for ring in rings:
        for h in ring:
            h.close()


def ds_algorithmic_bytes(B, H, n, d, r, k):
    """Bytes one Double Sparsity decode launch must move when every sequence
    holds n tokens: label rows of all n tokens (r bf16 each), the key and value
    rows of the min(k, n) kept tokens (d bf16 each), q (d bf16), the channel
    list (r int32), out (d fp32), and the lengths (int32). A dense step
    (k >= n) reads no label rows."""
    kept = min(k, n)
    label = n * r * 2 if k < n else 0
    return B * H * (label + kept * d * 2 * 2 + d * 2 + d * 4) + H * r * 4 + B * 4


def run_ds_decode(args):
    """Double Sparsity decode attention for one Llama-2-7B attention layer:
    16 sequences of 8192 cached tokens, 32 heads of 128 channels, bf16 caches
    with 8 seeded outlier channels per head (synthetic; see
    workloads/decode_attention.py). Legs: 1/16 of the channels and 1/16 of the
    tokens (r = 8, k = 512, the pages' headline sparsity), the SGLang example's
    r = 16, k = 256, and the same kernel attending to every token (dense).
    Caches rotate through copies so that a step never finds the previous
    step's rows in the 256 MB Infinity Cache; steps are replayed from HIP
    graphs."""
    import numpy as np
    import torch

    import free_activation_sparse_amd as fas
    from workloads import decode_attention as wda

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = wda.CASES["llama2_7b_b16_s8192_r8_k512"]
    inp = wda.make_inputs(base)
    B, H, S, d = inp.key.shape
    order = wda.channel_order(base)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    R = 3
    Q = bf(inp.q)
    Ks, Vs = [bf(inp.key)], [bf(inp.value)]
    for _ in range(R - 1):
        Ks.append(Ks[0].clone())
        Vs.append(Vs[0].clone())
    del inp
    sl = torch.full((B,), S, dtype=torch.int32, device=dev)
    last = sl - 1
    out = torch.empty((R, B, H, d), dtype=torch.float32, device=dev)
    legs = {}
    plan = (("r8_k512", 8, 512), ("r16_k256", 16, 256), ("dense", 8, S))
    if args.only in ("r8_k512", "r16_k256"):   # short profiler runs: one leg
        plan = tuple(p for p in plan if p[0] == args.only)
    for name, r, k in plan:
        if args.counters_run:
            ch = torch.from_numpy(np.ascontiguousarray(order[:, :r])).to(dev)
            Ls = [torch.empty((B, H, S, r), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            for i in range(R):
                fas.label_cache_update(Ks[i], Ls[i], ch)
            for i in range(12):
                j = i % R
                fas.ds_decode_attention(Q.data_ptr(), Ks[j].data_ptr(), Vs[j].data_ptr(), Ls[j].data_ptr(),
                                        ch.data_ptr(), sl.data_ptr(), B, H, S, d, r, k, d ** -0.5,
                                        out[j].data_ptr(), 0, 0)
            torch.cuda.synchronize()
            a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
            b = torch.empty_like(a)
            for _ in range(3):
                b.copy_(a)
            torch.cuda.synchronize()
            print(json.dumps({"counters_run": "done", "decodes": 12, "r": r, "k": k, "copy_bytes": 256 << 20}))
            return
        ch = torch.from_numpy(np.ascontiguousarray(order[:, :r])).to(dev)
        Ls = []
        if k < S:
            for i in range(R):
                L = torch.empty((B, H, S, r), dtype=torch.bfloat16, device=dev)
                fas.label_cache_update(Ks[i], L, ch)
                Ls.append(L)
        scale = d ** -0.5

        def step(i, s, r=r, k=k, ch=ch, Ls=Ls):
            j = i % R
            fas.ds_decode_attention(Q.data_ptr(), Ks[j].data_ptr(), Vs[j].data_ptr(),
                                    Ls[j].data_ptr() if Ls else 0, ch.data_ptr(), sl.data_ptr(), B, H, S, d, r, k,
                                    scale, out[j].data_ptr(), 0, s)
        steps = args.steps if k < S else max(20, args.steps // 10)
        ev, wall = timed_steps(torch, step, steps, min(args.warmup, steps), G=60)
        kus = graph_us(torch, step, count=120 if k < S else 30)
        nbytes = ds_algorithmic_bytes(B, H, S, d, r, k)
        legs[name] = {"r": r, "k": k, "us_per_step": ev / steps * 1e6, "wall_us_per_step": wall / steps * 1e6,
                      "kernel_us": kus, "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (kus * 1e-6) / 1e9,
                      "sequences_per_s": B * steps / ev}
        if Ls:
            # decode append: the newest token of every sequence (position seq_len - 1)
            upd = lambda i, s, L=Ls[0], ch=ch, r=r: fas.ds_label_cache_update(
                Ks[0].data_ptr(), L.data_ptr(), ch.data_ptr(), last.data_ptr(), B, H, S, d, r, 1, s)
            legs[name]["label_append_us"] = graph_us(torch, upd, count=120)
            pre = lambda i, s, L=Ls[0], ch=ch, r=r: fas.ds_label_cache_update(
                Ks[0].data_ptr(), L.data_ptr(), ch.data_ptr(), 0, B, H, S, d, r, S, s)
            legs[name]["label_prefill_us"] = graph_us(torch, pre, count=20)
        del Ls
    head = legs.get("r8_k512") or next(iter(legs.values()))
    for name in ("r8_k512", "r16_k256"):
        if name in legs and "dense" in legs:
            legs[name]["speedup_vs_dense"] = legs["dense"]["us_per_step"] / legs[name]["us_per_step"]
            legs[name]["kernel_speedup_vs_dense"] = legs["dense"]["kernel_us"] / legs[name]["kernel_us"]
    res = {"metric": "Double Sparsity decode attention sequences/s (one layer) & achieved HBM GB/s",
           "value": head["sequences_per_s"], "unit": "sequences/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["us_per_step"] * 1e-3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "llama2_7b_ds_decode_b16_h32_d128_s8192_r8_k512", "batch": B, "heads": H,
                      "head_dim": d, "seq_len": S, "label_channels": 8, "heavy_tokens": 512,
                      "cache_ring_copies": R, "launch": "graph",
                      "timing": "HIP events around the timed graph replays"},
           "roofline": {"bound": "hbm", "achieved": round(head["achieved_GBps"], 1), "peak": PEAK_GBS,
                        "unit": "GB/s", "frac": round(head["achieved_GBps"] / PEAK_GBS, 4),
                        "traffic": traffic_from_profile("ds_decode_kernel", DS_SOURCES, head["k"]),
                        "kernel": "ds_decode_kernel", "kernel_us": round(head["kernel_us"], 2),
                        "algorithmic_bytes": head["algorithmic_bytes"]},
           "legs": legs, "device": torch.cuda.get_device_name(0)}
    res["cpu_baseline"] = None if args.no_cpu else ds_cpu_baseline(base, min(args.cpu_seconds, 10.0))
    print(json.dumps(res))


# Slots of the fused forward's timestamps (sparse_linear_set_timeline).
TL_GATE = {"keys": 3, "window_counted": 18, "window_pivot": 19, "first_barrier": 7, "histogram": 8, "pivot_bin": 9, "candidates": 10, "ranked": 11,
           "stat_keys": 14, "extremes_and_plain_sums": 15, "first_threshold_checked": 16, "totals_in_lds": 17,
           "totals_summed": 12, "threshold_computed": 13, "threshold": 5, "selected": 6,
           "published": 1, "acks_in": 2}
TL_PROD = {"compacted": 1, "early_poll_back": 2, "pair_polled": 3, "end": 22}


def timeline_summary(launches):
    """Per-phase times (us since the launch's first workgroup started) from
    [launch][workgroup][32] timestamp arrays (workgroup 0 = the gate): the
    gate's phases as medians over launches, the product workgroups' as
    medians over launches of their p10 / median / p90 / max."""
    import numpy as np

    gate = {k: [] for k in TL_GATE}
    prod = {k: {"p10": [], "median": [], "p90": [], "max": []} for k in list(TL_PROD) + ["wave_end_max"]}
    hits, nwg = [], []
    for a in launches:
        a = a.astype(np.int64)
        a = a[a[:, 0] != 0]  # workgroups that record (the gate first; clearing workgroups record nothing)
        n = a.shape[0]
        base = a[:, 0].min()
        us = lambda v: (v - base) * 0.01  # s_memrealtime: 100 MHz
        for k, slot in TL_GATE.items():
            if a[0, slot] != 0:
                gate[k].append(us(a[0, slot]))
        p = a[1:]
        cols = {k: p[:, slot] for k, slot in TL_PROD.items()}
        cols["wave_end_max"] = p[:, 4:20].max(axis=1)
        for k, v in cols.items():
            v = v[v != 0]
            if v.size:
                t = us(v)
                for q, f in (("p10", 10), ("median", 50), ("p90", 90)):
                    prod[k][q].append(float(np.percentile(t, f)))
                prod[k]["max"].append(float(t.max()))
        seen = p[:, 2] != 0
        if seen.any():
            hits.append(float((p[seen, 20] != 0).mean()))
        nwg.append(n)
    med = lambda xs: round(float(np.median(xs)), 2) if xs else None
    return {"workgroups": int(np.median(nwg)),
            "gate_us": {k: med(v) for k, v in gate.items() if v},
            "product_us": {k: {q: med(x) for q, x in v.items()} for k, v in prod.items() if v["median"]},
            "early_poll_saw_pair": med(hits)}


def run_timeline():
    """Timelines of the fused forward (timeline build of the library): 16
    launches per case after the ring is primed, each with the timestamp
    buffer installed alone; plus the same build's graph-replay launch time
    without the buffer (the timestamps' own cost shows against the regular
    library's time)."""
    import numpy as np
    import torch

    import free_activation_sparse_amd as fas
    from free_activation_sparse_amd import build as fbuild
    import workloads as wl

    fas.LIB_PATH = fbuild.LIB_TIMELINE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    buf = torch.zeros(1024 * 32, dtype=torch.int64, device=dev)
    cases = [("llama7b_down_topk50", 2, 0, dict(gate="topk", K=wl.k_from_sparsity(11008, 0.5))),
             ("llama7b_down_topk65", 2, 0, dict(gate="topk", K=wl.k_from_sparsity(11008, 0.65))),
             ("phi4_gate_stat10", 4, 0, dict(gate="stat", s_keep=0.10)),
             ("phi4_down_stat10", 4, 2, dict(gate="stat", s_keep=0.10))]
    out = {"timeline": "fused_kernel", "clock": "s_memrealtime (100 MHz)", "cases": {}}
    weights = {}
    for name, cfg, li, gk in cases:
        lin = wl.CONFIGS[cfg].linears[li]
        m, n = lin.m, lin.n
        if (cfg, li) not in weights:
            weights[(cfg, li)] = torch.from_numpy(np.ascontiguousarray(wl.weight(cfg, li)).view(np.int16)).to(dev) \
                .view(torch.bfloat16)
        R = max(2, -(-(1 << 30) // (m * n * 2)))
        ring = [fas.SparseLinear(weights[(cfg, li)], c=None, **gk) for _ in range(R)]
        X = torch.from_numpy(wl.tokens(cfg, li, 0, 64).view(np.int16)).to(dev).view(torch.bfloat16).contiguous()
        Y = torch.zeros((R, m), dtype=torch.float32, device=dev)

        def f(i, s):
            fas.sparse_linear_forward(ring[i % R].handle, X[i % 64].data_ptr(), 1, Y[i % R].data_ptr(), fas.SL_F32,
                                      0, 0, 0, s)
        prime(torch, f, 2 * R)
        launch_us = graph_us(torch, f, count=240)
        s = torch.cuda.current_stream().cuda_stream
        launches = []
        for i in range(2 * R, 2 * R + 16):
            buf.zero_()
            torch.cuda.synchronize()
            fas.sparse_linear_set_timeline(buf.data_ptr())
            f(i, s)
            torch.cuda.synchronize()
            fas.sparse_linear_set_timeline(0)
            launches.append(buf.view(1024, 32).cpu().numpy().copy())
        for h in ring:
            h.sync_status()
            h.close()
        res = timeline_summary(launches)
        res.update({"m": m, "n": n, "gate": gk, "launch_us_graph": round(launch_us, 3)})
        out["cases"][name] = res
        print(f"[timeline] {name}: launch {launch_us:.2f} us, published at {res['gate_us'].get('published')} us",
              file=sys.stderr, flush=True)
        del ring, X, Y
        torch.cuda.empty_cache()
    out["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(out))


def counters_run():
    """Few dispatches, for rocprofv3 --pmc passes (each dispatch is profiled
    on its own): 60 eager headline forwards over the 12-copy ring, then a plain
    256 MiB device-to-device copy three times, whose counters calibrate the
    byte scale."""
    import numpy as np
    import torch

    import free_activation_sparse_amd as fas
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m, n, K = 4096, 11008, wl.k_from_sparsity(11008, 0.5)
    Wd = torch.from_numpy(wl.weight(2, 0).view(np.int16)).to(dev).view(torch.bfloat16)
    X = torch.from_numpy(wl.tokens(2, 0, 0, NTOK).view(np.int16)).to(dev).view(torch.bfloat16).contiguous()
    ring = [fas.SparseLinear(Wd, c=None, gate="topk", K=K) for _ in range(RING)]
    Y = torch.empty((RING, m), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    for i in range(60):
        fas.sparse_linear_forward(ring[i % RING].handle, X[i % NTOK].data_ptr(), 1, Y[i % RING].data_ptr(),
                                  fas.SL_F32, 0, 0, 0, s)
    torch.cuda.synchronize()
    a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    for h in ring:
        h.sync_status()
    print(json.dumps({"counters_run": "done", "forwards": 60, "K": K, "copy_bytes": 256 << 20}))


# ---------------------------------------------------------------------------
# CPU baselines: the oracle as it stands, timed on the host
# ---------------------------------------------------------------------------
def host_cpu_model():
    """The host CPU's model name (from /proc/cpuinfo) and the CPUs visible."""
    name = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": name, "cpus_visible": os.cpu_count()}


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return 1


def _timed_oracle(run_one, seconds, max_units):
    """Calls run_one(i) until `seconds` pass or max_units are done; returns
    (units, elapsed seconds)."""
    done = 0
    t0 = time.perf_counter()
    while True:
        run_one(done)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= max_units:
            return done, el


def _two_thread_settings(run_one, seconds, max_units, unit, describe):
    """The oracle at one BLAS/OpenMP thread and at the library's default
    thread count (all cores); the all-thread run is the reported value."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover - threadpoolctl is installed here
        threadpool_limits = None
    half = seconds / 2
    single = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1, e1 = _timed_oracle(run_one, half, max_units)
        single = {"value": round(d1 / e1, 4), "unit": unit, "cores": 1,
                  "sample": f"{d1} {describe}, {e1:.1f} s"}
    dn, en = _timed_oracle(run_one, half, max_units)
    out = {"value": round(dn / en, 4), "unit": unit, "cores": _oracle_threads(), "kind": "oracle",
           "sample": f"{dn} {describe}, {en:.1f} s", "single_thread": single, "host": host_cpu_model()}
    if single is not None and single["value"] > 0:
        ratio = out["value"] / single["value"]
        out["all_threads_over_one"] = round(ratio, 3)
        if ratio < 1.25:
            out["note"] = ("cores is the thread count the oracle was allowed; its rate equals the one-thread "
                           "rate, so the per-unit work runs effectively on one thread")
    return out


def cpu_baseline(wl, Wh, K, seconds):
    """The oracle as it stands, per token, on the host (scores, lexsort top-K,
    gathered fp64 product), bounded by `seconds`."""
    import oracle
    c = oracle.column_norms(Wh)  # init-time, not timed (the library precomputes c too)
    return _two_thread_settings(lambda i: oracle.forward(Wh, c, wl.token(2, 0, i % NTOK), "topk", K=K),
                                seconds, NTOK, "tokens/s",
                                f"tokens of the 4096x11008 bf16 layer at K={K} (fp64 numpy oracle: scores, "
                                "lexsort top-K, gathered product)")


def workload_cpu_baseline(leg, host_w, seconds):
    """The sparse-linear oracle on the host for a workload's first leg: tokens
    one at a time through every linear of the leg (the union of a batch is an
    execution detail, so the oracle's work per token is the same), bounded by
    `seconds` (column norms precomputed)."""
    import oracle
    import workloads as wl
    name, B, lins = leg[:3]
    cs = {(cfg, li): oracle.column_norms(host_w[(cfg, li)]) for cfg, li, _ in lins}

    def one(i):
        for cfg, li, gk in lins:
            x = wl.token(cfg, li, i)
            oracle.forward(host_w[(cfg, li)], cs[(cfg, li)], x, gk["gate"], K=gk.get("K"), s_keep=gk.get("s_keep"))
    return _two_thread_settings(one, seconds, 64, "tokens/s",
                                f"tokens through the {len(lins)} linears of leg {name} (fp64 numpy oracle per "
                                "linear: scores, select, gathered product)")


def ffn_cpu_baseline(host, Ks, tokens, seconds):
    """The FFN-chain oracle (oracle.ffn_chain: gate and up forwards, h =
    bf16(SiLU(g) u) rounded once, down forward) on the host, per token,
    bounded by `seconds` (column norms precomputed, as the library does at
    init)."""
    import oracle
    cs = [oracle.column_norms(W) for W in host]
    kw = [dict(mode="topk", K=K) for K in Ks]
    return _two_thread_settings(
        lambda i: oracle.ffn_chain(host[0], cs[0], kw[0], host[1], cs[1], kw[1], host[2], cs[2], kw[2],
                                   tokens[i % len(tokens)]),
        seconds, 64, "tokens/s",
        f"tokens through gate/up 11008x4096 and down 4096x11008 at K={Ks} (fp64 numpy oracle.ffn_chain)")


def ds_cpu_baseline(case, seconds):
    """The Double Sparsity oracle on the host, one (sequence, head) pair at a
    time (label cache, fp32 label scores, lexsort top-k, fp64 attention),
    bounded by `seconds`; reported per sequence (32 heads)."""
    from oracle import double_sparse as ods
    from workloads import decode_attention as wda
    inp = wda.make_inputs(case, batch=1)
    S, k = case.max_seq, case.k

    def one(done):
        h = done % case.heads
        lab = ods.label_cache(inp.key[:, h:h + 1], inp.channels[h:h + 1])[0, 0]
        s = ods.approx_scores(inp.q[0, h], lab, inp.channels[h], S)
        idx = ods.heavy_tokens(s, k)
        ods.sparse_attention(inp.q[0, h], inp.key[0, h], inp.value[0, h], idx, case.head_dim ** -0.5)
    res = _two_thread_settings(one, seconds, case.batch * case.heads, "pairs/s",
                               f"(sequence, head) pairs at r={case.r}, k={k} (numpy oracle: label cache, fp32 label "
                               "scores, lexsort top-k, fp64 attention)")
    # reported per sequence: pairs/s / heads
    for d in (res, res.get("single_thread")):
        if d:
            d["value"] = round(d["value"] / case.heads, 4)
            d["unit"] = "sequences/s"
    res["sample"] += f"; sequences/s = pairs/s / {case.heads} heads"
    return res


if __name__ == "__main__":
    main()
