"""Benchmark of the weight-informed activation-sparse linear on one MI355X.

Workload: the Llama-2-7B-shaped FFN down projection, W 4096 x 11008 bf16
(std 0.02), x = SiLU(g) * u with g, u ~ N(0, 1) rounded to bf16, one token per
step (batch-1 decode), WINA top-K at 50 % sparsity (K = 5504, the headline) and
65 % sparsity (K = 3853). A step is one full forward, one fused launch: a gate
workgroup (scores, top-K select) and the product workgroups (predicate,
compaction, gather-GEMV). The two-launch form (gate kernel, then product
kernel) is timed beside it.

Weights rotate through 12 handle-owned copies (1.08 GB) so the 256 MB
Infinity Cache never serves them; tokens rotate through 256 seeded tokens held
in HBM. Steps are captured into HIP graphs and replayed, so the host's per-call
overhead does not throttle the GPU; the timed region is bracketed by
torch.cuda.synchronize().

Printed: one JSON line with tokens/s, ms per step, the fused kernel's
achieved HBM bandwidth on algorithmic bytes against the 8 TB/s peak (its
duration from HIP events on its stream around back-to-back launches), the
same-kernel dense baseline, hipBLASLt's dense GEMV for context, and the CPU
oracle timed on the host.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["sparse50", "sparse65", "fixed50", "dense", "all", "r8_k512", "r16_k256"],
                    default="all",
                    help="restrict the measured legs (short profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for memory counters)")
    ap.add_argument("--counters-run", action="store_true",
                    help="short eager run for memory-counter passes: 12 + 48 headline forwards "
                         "(K=5504), then three plain 256 MiB device copies; prints one line")
    ap.add_argument("--workload", default="llama7b_down",
                    choices=["llama7b_down", "llama3_block", "phi4_ffn_stat", "qwen_ffn_b16", "llama2_ffn_chain",
                             "llama2_ds_decode"],
                    help="llama7b_down is the headline; the others measure the remaining layer shapes")
    return ap.parse_args()


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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the sparse linear is measured on one GPU; split by output rows, each GPU would run the same "
              "kernels on its own rows with no exchange before the product)",
              file=sys.stderr)
        sys.exit(2)

    if args.workload == "llama2_ffn_chain":
        run_ffn_chain(args)
        return
    if args.workload == "llama2_ds_decode":
        run_ds_decode(args)
        return
    if args.workload != "llama7b_down":
        run_workload(args)
        return
    if args.counters_run:
        counters_run()
        return

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

    def make_ring(K):
        return [fas.SparseLinear(Wd, c=None, gate="topk", K=K) for _ in range(RING)]

    # Fixed (calibrated) threshold leg: tau = the median score over the 256
    # tokens (c from the library; plain numpy on the host, outside any timed
    # region), so that about half of each token's inputs are kept
    fixed_tau, fixed_kept = None, None
    if args.only in ("all", "fixed50"):
        probe = fas.SparseLinear(Wd, c=None, gate="topk", K=1)
        c_host = probe.norms().cpu().numpy().astype(np.float64)
        probe.close()
        xs = (wl.tokens(2, 0, 0, NTOK).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        sc = (np.abs(xs) * c_host[None, :]).astype(np.float32)
        fixed_tau = float(np.median(sc))
        fixed_kept = float((sc > np.float32(fixed_tau)).sum(axis=1).mean())

    def layer_step(ring, dense):
        """f(i, stream): forward of token i % 256 through ring copy i % 12."""
        def f(i, s):
            h, x, y = ring[i % RING], X[i % NTOK], Y[i % RING]
            if dense:
                fas.sparse_linear_forward_dense(h.handle, x.data_ptr(), 1, y.data_ptr(), fas.SL_F32,
                                                s.cuda_stream)
            else:
                fas.sparse_linear_forward(h.handle, x.data_ptr(), 1, y.data_ptr(), fas.SL_F32, 0, 0, 0,
                                          s.cuda_stream)
        return f

    def run_steps(f, steps, warmup):
        """Warm up, then time exactly `steps` calls of f; returns seconds. In
        graph mode the calls are captured in chunks of 120 and replayed."""
        if args.mode == "eager":
            s = torch.cuda.current_stream()
            for i in range(warmup):
                f(i, s)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                f(i, s)
            torch.cuda.synchronize()
            return time.perf_counter() - t0
        G = RING * 10
        cache = {}

        def graph_of(count):
            if count not in cache:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    s = torch.cuda.current_stream()
                    for i in range(count):
                        f(i, s)
                cache[count] = g
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
        t0 = time.perf_counter()
        for cnt in plan_timed:
            cache[cnt].replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def time_graph(fn, count=600):
        """Average microseconds per call of fn(i, stream), from HIP events on the
        replay stream around one replay of a graph holding `count` calls
        back to back."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s = torch.cuda.current_stream()
            for i in range(count):
                fn(i, s)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / count

    def kernel_times(ring, dense):
        """(gate us, product us, fused us, two-launch us). The fused launch and
        the two-launch forward are timed whole; the gate and product kernels of
        the two-launch form are also launched alone, back to back (ring copy i
        keeps the selection of token i, so the product-only launches move
        exactly the bytes of a full forward)."""
        if dense:
            return 0.0, time_graph(layer_step(ring, True)), None, None
        fused_us = time_graph(layer_step(ring, False))
        for h in ring:
            h.set_fused(False)
        two_us = time_graph(layer_step(ring, False))
        s0 = torch.cuda.current_stream()
        for i in range(RING):
            fas.sparse_linear_forward(ring[i].handle, X[i].data_ptr(), 1, Y[i].data_ptr(), fas.SL_F32,
                                      0, 0, 0, s0.cuda_stream)

        def stage(bit):
            def f(i, s):
                k = i % RING
                fas.sparse_linear_forward_stages(ring[k].handle, X[k].data_ptr(), 1, Y[k].data_ptr(),
                                                 fas.SL_F32, 0, 0, 0, bit, s.cuda_stream)
            return f
        gate_us = time_graph(stage(fas.SL_STAGE_GATE))
        prod_us = time_graph(stage(fas.SL_STAGE_PRODUCT))
        for h in ring:
            h.set_fused(True)
        return gate_us, prod_us, fused_us, two_us

    results = {}
    legs = ["sparse50", "sparse65", "fixed50"] if args.only == "all" else ([args.only] if args.only != "dense" else [])
    for leg in legs:
        if leg == "fixed50":
            K = fixed_kept  # mean kept count over the tokens (algorithmic bytes)
            ring = [fas.SparseLinear(Wd, c=None, gate="fixed", tau=fixed_tau) for _ in range(RING)]
        else:
            K = Ks[leg]
            ring = make_ring(K)
        secs = run_steps(layer_step(ring, False), args.steps, args.warmup)
        gate_us, prod_us, fused_us, two_us = kernel_times(ring, False)
        for h in ring:
            h.sync_status()
        ab = algorithmic_bytes(m, n, K)
        results[leg] = {
            "K": K, "sparsity": 1 - K / n,
            **({"tau": fixed_tau, "gate": "fixed threshold (median score of the 256 tokens)"} if leg == "fixed50" else {}),
            "tokens_per_s": args.steps / secs, "ms_per_step": secs / args.steps * 1e3,
            "fused_kernel_us": fused_us, "algorithmic_bytes": ab,
            "fused_achieved_GBps": ab / (fused_us * 1e-6) / 1e9,
            "step_achieved_GBps": ab / (secs / args.steps) / 1e9,
            "two_launch_us_per_step": two_us,
            "gate_kernel_us": gate_us, "product_kernel_us": prod_us,
            "product_achieved_GBps": ab / (prod_us * 1e-6) / 1e9,
        }
        for h in ring:
            h.close()
        del ring

    dense = None
    if args.only in ("all", "dense"):
        ring = make_ring(Ks["sparse50"])
        secs = run_steps(layer_step(ring, True), args.steps, args.warmup)
        _, prod_us, _, _ = kernel_times(ring, True)
        # the ordered split reduction needs no clearing of y (no fill kernel
        # before the product): the speedup is taken against the faster form
        for h in ring:
            h.set_deterministic(True)
        ordered_us = time_graph(layer_step(ring, True))
        for h in ring:
            h.set_deterministic(False)
        ab = algorithmic_bytes(m, n, n)
        best_us = min(secs / args.steps * 1e6, ordered_us)
        dense = {"tokens_per_s": args.steps / secs, "ms_per_step": secs / args.steps * 1e3,
                 "product_kernel_us": prod_us, "achieved_GBps": ab / (prod_us * 1e-6) / 1e9,
                 "ordered_reduction_us_per_step": ordered_us, "best_us_per_step": best_us}
        for h in ring:
            h.close()
        del ring
        # hipBLASLt / rocBLAS dense GEMV on the row-major weights, for context
        Wr = [Wd.clone() for _ in range(RING)]
        Yb = torch.empty((RING, m), dtype=torch.bfloat16, device=dev)

        def mv(i):
            torch.matmul(Wr[i % RING], X[i % NTOK], out=Yb[i % RING])
        for i in range(args.warmup):
            mv(i)
        # hipBLASLt calls cannot be captured in a graph: time them eagerly between
        # two events, with the GPU first asleep so the host runs ahead
        count = 1200
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(100_000_000)
        e0.record()
        for i in range(count):
            mv(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / count
        dense["torch_matmul_us_per_step"] = us
        dense["torch_matmul_tokens_per_s"] = 1e6 / us
        del Wr

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu and "sparse50" in results:
        cpu = cpu_baseline(wl, Wh, Ks["sparse50"], args.cpu_seconds)

    head = results.get("sparse50") or results.get("sparse65")
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"] if head else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"] if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama2_7b_down_proj_4096x11008_bf16_topk_50pct",
                   "m": m, "n": n, "K": Ks["sparse50"], "batch": 1, "tokens": NTOK,
                   "weight_ring_copies": RING, "weight_ring_bytes": RING * m * n * 2,
                   "launch": args.mode},
    }
    if head:
        out["roofline"] = {
            "bound": "hbm",
            "achieved": round(head["fused_achieved_GBps"], 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["fused_achieved_GBps"] / PEAK_GBS, 4),
            "traffic": traffic_from_profile("fused_kernel", FUSED_SOURCES, Ks["sparse50"]),
            "kernel": "fused_kernel (gate workgroup + gather-GEMV workgroups)",
            "kernel_us": round(head["fused_kernel_us"], 3),
            "algorithmic_bytes": head["algorithmic_bytes"],
        }
    out["cpu_baseline"] = cpu
    out["legs"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in results.items()}
    if dense:
        out["dense_same_kernel"] = {k: round(v, 4) for k, v in dense.items()}
        for k, v in results.items():
            bar = 0.8 / (1 - v["sparsity"])
            out["legs"][k]["speedup_vs_dense"] = round(v["tokens_per_s"] * dense["best_us_per_step"] * 1e-6, 4)
            out["legs"][k]["speedup_bar"] = round(bar, 4)
    out["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(out))


# ---------------------------------------------------------------------------
# Other layer shapes: a step is one forward of every linear of the workload for
# a batch of B tokens (ring copies of the weights so that >= 1 GiB rotates).
# ---------------------------------------------------------------------------
def workload_legs(name):
    """[(leg name, B, [(cfg, linear, gate kwargs), ...])]"""
    import workloads as wl
    if name == "llama3_block":
        ps = wl.component_sparsities(3)
        lins = [(3, li, dict(gate="topk", K=wl.k_from_sparsity(l.n, round(ps[li], 6))))
                for li, l in enumerate(wl.CONFIGS[3].linears)]
        # "grouped": the linears that share an input in one launch each
        # (q, k, v | o | gate, up | down: 4 launches instead of 7)
        names = [l.name for l in wl.CONFIGS[3].linears]
        groups = [[names.index(a) for a in g] for g in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))]
        return [("block", 1, lins), ("grouped", 1, lins, groups)]
    if name == "phi4_ffn_stat":
        lins = [(4, li, dict(gate="stat", s_keep=0.10)) for li in range(3)]
        # "B1_grouped": gate and up in one launch (gate's token for both), then down
        return [(f"B{b}", b, lins) for b in (1, 2, 4, 8)] + [("B1_grouped", 1, lins, [[0, 1], [2]])]
    if name == "qwen_ffn_b16":
        legs = []
        for p in (0.65, 0.90):
            lins = [(5, li, dict(gate="topk", K=wl.k_from_sparsity(wl.CONFIGS[5].linears[li].n, p)))
                    for li in range(3)]
            legs.append((f"p{int(p * 100)}", 16, lins))
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
    for spec in legs:
        leg, B, lins = spec[:3]
        groups = spec[3] if len(spec) > 3 else None
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

        def step(i, s, stages=3):
            if groups is not None:
                # one token: a group's linears share x (the token of its first linear)
                for g in groups:
                    fas.sparse_linear_forward_group([rings[L][i % R].handle for L in g], Xs[g[0]][i % NT].data_ptr(),
                                                    [Ys[L][i % R].data_ptr() for L in g], fas.SL_F32, s.cuda_stream)
                return
            for L in range(len(lins)):
                h = rings[L][i % R]
                fas.sparse_linear_forward_stages(h.handle, Xs[L][i % NT].data_ptr(), B, Ys[L][i % R].data_ptr(),
                                                 fas.SL_F32, 0, 0, 0, stages, s.cuda_stream)

        secs = _replay_timed(torch, step, args.steps, args.warmup)
        # untimed side pass: kept (B = 1) or union (B > 1) column counts per linear
        kept = []
        for L, (name, m, n) in enumerate(dims):
            mk = torch.empty((B, n), dtype=torch.uint8, device=dev)
            tot = 0
            for t in range(NT):
                fas.sparse_linear_forward(rings[L][0].handle, Xs[L][t].data_ptr(), B, Ys[L][0].data_ptr(),
                                          fas.SL_F32, mk.data_ptr(), 0, 0, torch.cuda.current_stream().cuda_stream)
                tot += int(mk.bool().any(dim=0).sum().item())
            kept.append(tot / NT)
        # per-linear kernel times: ring copy r keeps the selection of token batch r
        prod_us, gate_us = [], []
        for L in range(len(lins)):
            s0 = torch.cuda.current_stream()
            for r in range(R):
                fas.sparse_linear_forward(rings[L][r].handle, Xs[L][r].data_ptr(), B, Ys[L][r].data_ptr(),
                                          fas.SL_F32, 0, 0, 0, s0.cuda_stream)

            def one(bit, L=L):
                def f(i, s):
                    r = i % R
                    fas.sparse_linear_forward_stages(rings[L][r].handle, Xs[L][r].data_ptr(), B,
                                                     Ys[L][r].data_ptr(), fas.SL_F32, 0, 0, 0, bit, s.cuda_stream)
                return f
            gate_us.append(_graph_us(torch, one(fas.SL_STAGE_GATE)))
            prod_us.append(_graph_us(torch, one(fas.SL_STAGE_PRODUCT)))
        lin_rows = []
        tot_bytes = 0
        for L, (name, m, n) in enumerate(dims):
            ab = kept[L] * m * 2 + B * n * 2 + n * 4 + B * m * 4
            tot_bytes += ab
            lin_rows.append({"linear": name, "m": m, "n": n, "columns_read": round(kept[L], 1),
                             "gate_us": round(gate_us[L], 3), "product_us": round(prod_us[L], 3),
                             "product_GBps": round(ab / (prod_us[L] * 1e-6) / 1e9, 1)})
        results[leg] = {"B": B, "tokens_per_s": B * args.steps / secs, "ms_per_step": secs / args.steps * 1e3,
                        "product_us_sum": sum(prod_us), "product_bytes_sum": tot_bytes,
                        "product_GBps": tot_bytes / (sum(prod_us) * 1e-6) / 1e9,
                        "dense_weight_bytes": total, "ring_copies": R, "linears": lin_rows}
        for ring in rings:
            for h in ring:
                h.close()
        del rings, Xs, Ys
        torch.cuda.empty_cache()

    first = legs[0][0]
    head = results[first]
    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": {"workload": args.workload, "headline_leg": first, "launch": "graph"},
        "roofline": {"bound": "hbm", "achieved": round(head["product_GBps"], 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(head["product_GBps"] / PEAK_GBS, 4), "traffic": None,
                     "kernel": "product kernels of one step (summed bytes / summed durations)"},
        "cpu_baseline": None if args.no_cpu else workload_cpu_baseline(legs[0], host_w, min(args.cpu_seconds, 10.0)),
        "legs": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                 for k, v in results.items()},
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
                                      WS.shape[1], s.cuda_stream)
    secs = _replay_timed(torch, step, args.steps, args.warmup)
    for ring in rings:
        for h in ring:
            h.sync_status()
    kept_bytes = sum(K * a * 2 for K, (a, b) in zip(Ks, shapes))
    dense_bytes = sum(a * b * 2 for a, b in shapes)
    us = secs / args.steps * 1e6
    out = {"metric": "sparse FFN chain tokens/s (Llama-2-7B FFN shapes, top-K 50 % per projection)",
           "value": args.steps / secs, "unit": "tokens/s", "ms_per_step": us * 1e-3,
           "config": {"workload": "llama2_7b_ffn_chain_gate_up_11008x4096_down_4096x11008_bf16_topk_50pct",
                      "K": Ks, "weight_ring_copies": R},
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
                                    scale, out[j].data_ptr(), 0, s.cuda_stream)
        steps = args.steps if k < S else max(20, args.steps // 10)
        secs = _replay_timed(torch, step, steps, min(args.warmup, steps))
        kus = _graph_us(torch, step, count=120 if k < S else 30)
        nbytes = ds_algorithmic_bytes(B, H, S, d, r, k)
        legs[name] = {"r": r, "k": k, "us_per_step": secs / steps * 1e6, "kernel_us": kus,
                      "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (kus * 1e-6) / 1e9,
                      "sequences_per_s": B * steps / secs}
        if Ls:
            # decode append: the newest token of every sequence (position seq_len - 1)
            upd = lambda i, s, L=Ls[0], ch=ch, r=r: fas.ds_label_cache_update(
                Ks[0].data_ptr(), L.data_ptr(), ch.data_ptr(), last.data_ptr(), B, H, S, d, r, 1, s.cuda_stream)
            legs[name]["label_append_us"] = _graph_us(torch, upd, count=120)
            pre = lambda i, s, L=Ls[0], ch=ch, r=r: fas.ds_label_cache_update(
                Ks[0].data_ptr(), L.data_ptr(), ch.data_ptr(), 0, B, H, S, d, r, S, s.cuda_stream)
            legs[name]["label_prefill_us"] = _graph_us(torch, pre, count=20)
        del Ls
    head = legs.get("r8_k512") or next(iter(legs.values()))
    for name in ("r8_k512", "r16_k256"):
        if name in legs and "dense" in legs:
            legs[name]["speedup_vs_dense"] = legs["dense"]["kernel_us"] / legs[name]["kernel_us"]
    res = {"metric": "Double Sparsity decode attention sequences/s (one layer) & achieved HBM GB/s",
           "value": head["sequences_per_s"], "unit": "sequences/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["us_per_step"] * 1e-3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "llama2_7b_ds_decode_b16_h32_d128_s8192_r8_k512", "batch": B, "heads": H,
                      "head_dim": d, "seq_len": S, "label_channels": 8, "heavy_tokens": 512,
                      "cache_ring_copies": R, "launch": "graph"},
           "roofline": {"bound": "hbm", "achieved": round(head["achieved_GBps"], 1), "peak": PEAK_GBS,
                        "unit": "GB/s", "frac": round(head["achieved_GBps"] / PEAK_GBS, 4),
                        "traffic": traffic_from_profile("ds_decode_kernel", DS_SOURCES, head["k"]),
                        "kernel": "ds_decode_kernel", "kernel_us": round(head["kernel_us"], 2),
                        "algorithmic_bytes": head["algorithmic_bytes"]},
           "legs": legs, "device": torch.cuda.get_device_name(0)}
    res["cpu_baseline"] = None if args.no_cpu else ds_cpu_baseline(base, min(args.cpu_seconds, 10.0))
    print(json.dumps(res))


def _replay_timed(torch, f, steps, warmup, G=60):
    """Warm up, then time exactly `steps` calls of f(i, stream) replayed from
    HIP graphs of G calls; returns seconds."""
    cache = {}

    def graph_of(count):
        if count not in cache:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                s = torch.cuda.current_stream()
                for i in range(count):
                    f(i, s)
            cache[count] = g
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
    t0 = time.perf_counter()
    for cnt in plan_timed:
        cache[cnt].replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def _graph_us(torch, fn, count=240):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream()
        for i in range(count):
            fn(i, s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / count


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


def cpu_baseline(wl, Wh, K, seconds):
    """The oracle as it stands, per token, on the host: bounded by `seconds`."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    c = oracle.column_norms(Wh)  # init-time, not timed (the library precomputes c too)
    done = 0
    t0 = time.perf_counter()
    while True:
        x = wl.token(2, 0, done)
        oracle.forward(Wh, c, x, "topk", K=K)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= 256:
            break
    return {"value": round(done / el, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} tokens of the 4096x11008 bf16 layer at K={K} (fp64 numpy oracle: scores, "
                      f"lexsort top-K, gathered product), {el:.1f} s on {os.cpu_count()} host CPUs visible"}


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return 1


def workload_cpu_baseline(leg, host_w, seconds):
    """The sparse-linear oracle on the host for a workload's first leg: tokens
    one at a time through every linear of the leg (the union of a batch is an
    execution detail, so the oracle's work per token is the same), bounded by
    `seconds` (column norms precomputed)."""
    import oracle
    import workloads as wl
    name, B, lins = leg[:3]
    cs = {(cfg, li): oracle.column_norms(host_w[(cfg, li)]) for cfg, li, _ in lins}
    done = 0
    t0 = time.perf_counter()
    while True:
        for cfg, li, gk in lins:
            x = wl.token(cfg, li, done)
            mode = gk["gate"]
            oracle.forward(host_w[(cfg, li)], cs[(cfg, li)], x, mode, K=gk.get("K"), s_keep=gk.get("s_keep"))
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= 64:
            break
    return {"value": round(done / el, 4), "unit": "tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"{done} tokens through the {len(lins)} linears of leg {name} (fp64 numpy oracle per "
                      f"linear: scores, select, gathered product), {el:.1f} s on {os.cpu_count()} host CPUs visible"}


def ffn_cpu_baseline(host, Ks, tokens, seconds):
    """The sparse-linear oracle through the FFN chain on the host, per token:
    gate and up forwards, h = bf16(SiLU(g) u), down forward; bounded by
    `seconds` (column norms precomputed, as the library does at init)."""
    import numpy as np
    import oracle
    import workloads as wl
    cs = [oracle.column_norms(W) for W in host]
    done = 0
    t0 = time.perf_counter()
    while True:
        x = tokens[done % len(tokens)]
        g = oracle.forward(host[0], cs[0], x, "topk", K=Ks[0])["y"]
        u = oracle.forward(host[1], cs[1], x, "topk", K=Ks[1])["y"]
        h = wl.f32_to_bf16_bits((g / (1.0 + np.exp(-g)) * u).astype(np.float32))
        oracle.forward(host[2], cs[2], h, "topk", K=Ks[2])
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= 64:
            break
    return {"value": round(done / el, 4), "unit": "tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"{done} tokens through gate/up 11008x4096 and down 4096x11008 at K={Ks} (fp64 numpy "
                      f"oracle per projection, numpy SiLU(g) u), {el:.1f} s on {os.cpu_count()} host CPUs visible"}


def ds_cpu_baseline(case, seconds):
    """The Double Sparsity oracle on the host, one (sequence, head) pair at a
    time (label cache, fp32 label scores, lexsort top-k, fp64 attention),
    bounded by `seconds`; reported per sequence (32 heads)."""
    import numpy as np
    from oracle import double_sparse as ods
    from workloads import decode_attention as wda
    inp = wda.make_inputs(case, batch=1)
    S, k = case.max_seq, case.k
    done = 0
    t0 = time.perf_counter()
    while True:
        h = done % case.heads
        lab = ods.label_cache(inp.key[:, h:h + 1], inp.channels[h:h + 1])[0, 0]
        s = ods.approx_scores(inp.q[0, h], lab, inp.channels[h], S)
        idx = ods.heavy_tokens(s, k)
        ods.sparse_attention(inp.q[0, h], inp.key[0, h], inp.value[0, h], idx, case.head_dim ** -0.5)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= case.batch * case.heads:
            break
    return {"value": round(done / case.heads / el, 4), "unit": "sequences/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": f"{done} (sequence, head) pairs (the heads of one {S}-token sequence, repeated: as many "
                      f"pairs as one batch-{case.batch} step) at r={case.r}, k={k} (numpy oracle: label cache, "
                      f"fp32 label scores, lexsort top-k, fp64 attention), {el:.1f} s on {os.cpu_count()} host "
                      f"CPUs visible; sequences/s = pairs/s / {case.heads} heads"}


if __name__ == "__main__":
    main()
