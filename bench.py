#!/usr/bin/env python3
"""Benchmark of speculative-decoding verification on one MI355X.

One step = one full verification of one batch (every row streamed, acceptance
test, first-reject scan, correction / bonus draw, emission). The default
workload is the draft-target configuration the headline metric is quoted on:
B=32 sequences, k=4 draft tokens, V=128256, bf16 logits, stochastic at T=0.7.

Inputs are generated on the host from fixed seeds, copied to HBM, and
replicated into enough rotating copies (together more than 3x the 256 MB
Infinity Cache) that every step reads its logits from HBM, not from cache.
Before timing, the GPU result of one step is checked against the CPU oracle;
the benchmark refuses to report a number if parity fails.

Prints ONE JSON line (rank 0, N=1). Fields beyond the required ones:
logit_GBps / hbm_frac (algorithmic bytes of a whole step over its time),
kernel_us (live HIP-event duration of one step: the linear kernel's one launch,
or a tree step's two launches), parity.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec + logit GB/s (% HBM peak), V=128256 k=4"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published
INFINITY_CACHE_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="c2_linear",
                    choices=["c1_tiny", "c2_linear", "c3_mtp", "c4_medusa_sparse", "c5_medusa_full",
                             *STEP_CONFIGS])
    ap.add_argument("--mode", default=None,
                    help="greedy | stochastic | typical (trees) (default: the config's own)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="rotating input copies (0 = auto)")
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead of a HIP graph")
    ap.add_argument("--commit", action="store_true",
                    help="linear configs: verify and commit in one launch (spec_verify_linear_commit)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device copies of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--source-hash", action="store_true",
                    help="print the hash of the kernel sources that measured traffic is keyed on")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """sha256 over what defines the verification kernels: their sources and the
    header with comments and runs of whitespace taken out (edits to those do not
    change the kernels), and the compiler flags, in a fixed order."""
    import hashlib
    import re
    from acceptance_row_softmax_amd import _build
    h = hashlib.sha256()
    for rel in ("acceptance_row_softmax_amd/csrc/specverify.hip", "acceptance_row_softmax_amd/csrc/sv_device.hpp",
                "acceptance_row_softmax_amd/csrc/sv_rows.hpp", "acceptance_row_softmax_amd/csrc/sv_host.hpp",
                "include/specverify.h"):
        with open(os.path.join(ROOT, rel), "r", encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(rel.encode() + b"\0" + text.encode() + b"\0")
    h.update(" ".join(_build.HIPCC_FLAGS).encode())
    return h.hexdigest()


def measured_traffic(workload_key: str):
    """HBM bytes per launch from the committed counter summaries under profiles/
    (lines "bench-traffic: {json}"), if one was taken on this workload with the
    current kernel sources; else None."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    src = kernel_source_hash()
    for name in sorted(os.listdir(pdir)):
        if not name.endswith((".md", ".txt")):
            continue
        with open(os.path.join(pdir, name), encoding="utf-8") as f:
            for ln in f:
                if not ln.startswith("bench-traffic: "):
                    continue
                rec = json.loads(ln[len("bench-traffic: "):])
                if rec.get("workload") == workload_key and rec.get("source_sha256") == src:
                    return rec
    return None


def copy_probe(mib: int):
    """Ten plain device-to-device copies of `mib` MiB: each reads and writes exactly
    that many bytes, which scales the HBM byte counters of a counter run."""
    import torch
    n = mib << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 10}), flush=True)


# The steps around verification, each timed on its own (one JSON line each):
#  sample_c2_step  one draft position of the draft-target workload sampled on the
#                  device: 32 rows of V = 128256 bf16 at T = 0.7
#  sample_c3       the first token of the MTP workload sampled from the carried
#                  logits: 256 rows of V = 129280 bf16 at T = 1
#  commit_c3       commit of the MTP workload's verification: B = 256, k = 1
#  tree_mask_c5    attention mask of the Cartesian K = 4, top-8 tree (4681 nodes)
STEP_CONFIGS = ("sample_c2_step", "sample_c3", "commit_c3", "tree_mask_c5")


def _graph_time(torch, calls, copies, steps, warmup):
    """Warm up, then time exactly `steps` calls: a graph over the `copies` calls
    replayed as often as it fits, then one over the first (steps mod copies) of
    them; returns (K, wall ms per call, event ms per call)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        calls(i % copies)
    torch.cuda.synchronize()
    K = max(1, steps)
    reps, rem = divmod(K, copies)
    graphs = []
    for n in ((copies,) if reps else ()) + ((rem,) if rem else ()):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                calls(i)
        g.replay()
        graphs.append(g)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(reps):
        graphs[0].replay()
    if rem:
        graphs[-1].replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return K, (t1 - t0) * 1e3 / K, ev0.elapsed_time(ev1) / K


def bench_steps(args):
    import numpy as np
    import torch

    import acceptance_row_softmax_amd as sv
    import gen
    import oracle

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = args.config
    cpu = None
    if cfg.startswith("sample"):
        if cfg == "sample_c2_step":
            w = gen.c2_linear(args.seed)
            x, T = np.ascontiguousarray(w.draft[:, 0, :]), 0.7
        else:
            w = gen.c3_mtp(args.seed, "stochastic")
            x, T = np.ascontiguousarray(w.target[:, 0, :]), 1.0
        mode = args.mode or "stochastic"
        rows, V = x.shape
        u = gen.uniforms(gen.key(98, args.seed, 1), rows).astype(np.float32)
        esz = 4 if w.dtype == gen.DT_F32 else 2
        alg = rows * V * esz
        tdt = {gen.DT_F32: torch.float32, gen.DT_BF16: torch.bfloat16, gen.DT_F16: torch.float16}[w.dtype]
        base = torch.from_numpy(x.view(np.int16) if esz == 2 else x).to(dev).view(tdt)
        copies = max(1, math.ceil(3 * INFINITY_CACHE_BYTES / alg) + 1)
        xs = [base] + [base.clone() for _ in range(copies - 1)]
        du = torch.from_numpy(u).to(dev)
        ws = torch.zeros(sv.lib().spec_sample_workspace(rows, V, sv.sv_dtype(base)), dtype=torch.uint8, device=dev)
        first = sv.sample(xs[0], du, mode=mode, temperature=T, workspace=ws)
        torch.cuda.synchronize()
        o = oracle.sample(mode, T, x, u, V, w.dtype)
        differ = first["tokens"].cpu().numpy() != o["tokens"]
        parity = {"checked": int(rows), "exceptions": int(differ.sum()),
                  "near_tie_sequences": int((o["near_tie"] != 0).sum()), "ok": bool(not (differ & (o["near_tie"] == 0)).any())}
        K, ms, ev_ms = _graph_time(torch, lambda i: sv.sample(xs[i], du, mode=mode, temperature=T, workspace=ws),
                                   copies, args.steps, args.warmup)
        t0 = time.perf_counter()
        n_rep = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            oracle.sample(mode, T, x, u, V, w.dtype)
            n_rep += 1
        el = time.perf_counter() - t0
        cpu = {"value": n_rep * rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"the full batch ({rows} rows) x {n_rep}, {el:.1f}s, single-threaded oracle"}
        metric, unit, value = "sampled rows/sec + logit GB/s (% HBM peak)", "rows/s", rows / (ms * 1e-3)
        kernel, dtype = "sample_kernel", gen.DTYPE_NAMES[w.dtype]
        workload = f"{cfg}: {rows} rows of V={V} {dtype} logits, {mode}" + (f" T={T}" if mode == "stochastic" else "")
    elif cfg == "commit_c3":
        B, k, cap = 256, 1, 1 << 16
        rng = np.random.default_rng(args.seed)
        acc = rng.integers(0, k + 1, size=B).astype(np.int32)
        out = rng.integers(0, 129280, size=(B, k + 1)).astype(np.int32)
        drafts = out[:, :k].copy()
        ln = rng.integers(100, 3000, size=B).astype(np.int32)
        hist = np.zeros((B, cap), np.int32)
        d = {n_: torch.from_numpy(a).to(dev) for n_, a in (("acc", acc), ("out", out), ("x", drafts))}
        dl, dh = torch.from_numpy(ln).to(dev), torch.from_numpy(hist).to(dev)
        first = sv.commit_linear(d["acc"], d["out"], d["x"], dl, dh)
        torch.cuda.synchronize()
        o_ln, o_hist, o = oracle.commit_linear(acc, out, drafts, ln, hist)
        ok = (np.array_equal(dl.cpu().numpy(), o_ln) and np.array_equal(dh.cpu().numpy(), o_hist)
              and np.array_equal(first["shifted"].cpu().numpy(), o["shifted"]))
        parity = {"checked": B, "exceptions": 0 if ok else B, "near_tie_sequences": 0, "ok": bool(ok)}
        sh = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
        nx = torch.empty(B, dtype=torch.int32, device=dev)
        ef = torch.empty(B, dtype=torch.int32, device=dev)
        L = sv.lib()

        def call(i):
            # the current stream at call time: the capture stream inside graph capture
            st = L.spec_commit_linear(B, k, d["acc"].data_ptr(), d["out"].data_ptr(), d["x"].data_ptr(),
                                      dl.data_ptr(), dh.data_ptr(), cap, sh.data_ptr(), nx.data_ptr(),
                                      ef.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert st == 0
        steps = min(args.steps, 8000)     # lengths grow by at most 2 per call: stay within capacity
        K, ms, ev_ms = _graph_time(torch, call, 8, steps, args.warmup)
        alg = B * (4 + (k + 1) * 4 + k * 4 + 4) + B * (4 + (k + 1) * 4 * 2 + 4 + 4)
        metric, unit, value = "committed sequences/sec", "sequences/s", B / (ms * 1e-3)
        kernel, dtype, workload = "commit_kernel", "int32", f"{cfg}: B={B} sequences, k={k}, history capacity {cap}"
    else:   # tree_mask_c5
        parent, _ = gen.cartesian_tree([8, 8, 8, 8])
        n = len(parent)
        W = (n + 31) // 32
        dp = torch.from_numpy(parent).to(dev)
        first = sv.tree_mask(dp)
        torch.cuda.synchronize()
        m = first["mask"].cpu().numpy()[0].view(np.uint32)
        bits = ((m[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(n, -1)[:, :n]
        ok = np.array_equal(bits.astype(np.uint8), oracle.tree_mask(parent))
        parity = {"checked": n, "exceptions": 0 if ok else n, "near_tie_sequences": 0, "ok": bool(ok)}
        mask = torch.empty((1, n, W), dtype=torch.int32, device=dev)
        L = sv.lib()

        def call(i):
            assert L.spec_tree_mask(1, n, dp.data_ptr(), 0, mask.data_ptr(), None,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
        K, ms, ev_ms = _graph_time(torch, call, 8, args.steps, args.warmup)
        alg = n * W * 4 + n * 4
        metric, unit, value = "mask rows/sec + mask GB/s", "rows/s", n / (ms * 1e-3)
        kernel, dtype, workload = "tree_mask_kernel", "u32", f"{cfg}: Cartesian K=4 top-8 tree, {n} nodes, {W} words per row"
    if not parity["ok"]:
        print(f"[bench] PARITY FAILED: {parity}", file=sys.stderr, flush=True)
        sys.exit(1)
    gbps = alg / (ev_ms * 1e-3) / 1e9
    line = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype, "data": "synthetic (seeded generator; no dataset)",
            "config": {"workload": workload, "graph": True},
            "roofline": {"bound": "hbm", "kernel": kernel, "achieved": gbps, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                         "launch_us": ev_ms * 1e3, "algorithmic_bytes": alg},
            "cpu_baseline": cpu, "parity": parity}
    print(json.dumps(line), flush=True)


# Typical acceptance (trees, --mode typical): the rule's constants are the
# caller's; these are the example setting the benchmark uses.
TYPICAL_EPS, TYPICAL_DELTA = 0.09, 0.3


def make_workload(cfg, mode, seed):
    import dataclasses
    import gen
    defaults = {"c1_tiny": "stochastic", "c2_linear": "stochastic", "c3_mtp": "stochastic",
                "c4_medusa_sparse": "greedy", "c5_medusa_full": "greedy"}
    mode = mode or defaults[cfg]
    if mode == "typical":
        # the stochastic workload's inputs (logits, candidates, uniforms), judged by typical acceptance
        return dataclasses.replace(gen.CONFIGS[cfg](seed, "stochastic"), mode="typical")
    return gen.CONFIGS[cfg](seed, mode)


def describe(w):
    import gen
    dt = gen.DTYPE_NAMES[w.dtype]
    if hasattr(w, "k"):
        return (f"{w.name}: linear draft verification, B={w.B} k={w.k} V={w.V} {dt} logits, "
                f"{w.mode}" + (f" T={w.temperature}" if w.mode == "stochastic" else ""))
    extra = ""
    if w.mode == "stochastic":
        extra = f" T={w.temperature}"
    elif w.mode == "typical":
        extra = f" acceptance T={w.temperature} eps={TYPICAL_EPS} delta={TYPICAL_DELTA}"
    return (f"{w.name}: candidate-tree verification, B={w.B} trees of {w.n_nodes} nodes, V={w.V} "
            f"{dt} logits, {w.mode}" + extra)


def positions(w):
    return w.B * w.k if hasattr(w, "k") else w.B * (w.n_nodes - 1)


def main():
    args = parse()
    if args.source_hash:
        print(kernel_source_hash())
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this verification engine runs on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported. Batches shard by sequence with no "
              "communication, so N GPUs run N independent copies of this benchmark.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import acceptance_row_softmax_amd as sv
    import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.config in STEP_CONFIGS:
        bench_steps(args)
        return
    t_gen = time.time()
    w = make_workload(args.config, args.mode, args.seed)
    linear = hasattr(w, "k")
    stoch = w.mode in ("stochastic", "typical")
    alg_bytes = w.algorithmic_bytes()
    print(f"[bench] {describe(w)}; algorithmic bytes/step {alg_bytes} "
          f"(generated in {time.time() - t_gen:.1f}s)", file=sys.stderr, flush=True)

    def dev_logits(a):
        a = np.ascontiguousarray(a)
        if w.dtype == gen.DT_F32:
            return torch.from_numpy(a).to(dev)
        t = torch.from_numpy(a.view(np.int16)).to(dev)
        return t.view(torch.bfloat16 if w.dtype == gen.DT_BF16 else torch.float16)

    copies = args.copies or max(1, math.ceil(3 * INFINITY_CACHE_BYTES / alg_bytes) + 1)
    if linear:
        base = {"t": dev_logits(w.target),
                "d": dev_logits(w.draft) if (stoch and w.k > 0) else None,
                "x": torch.from_numpy(w.draft_tokens.astype(np.int32)).to(dev) if w.k > 0 else None,
                "u": torch.from_numpy(w.uniforms.astype(np.float32)).to(dev)}
    else:
        base = {"lg": dev_logits(w.logits),
                "par": torch.from_numpy(np.asarray(w.parent, np.int32)).to(dev),
                "cand": torch.from_numpy(w.cand.astype(np.int32)).to(dev),
                "u": torch.from_numpy(w.uniforms.astype(np.float32)).to(dev)}
    sets = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()}
                     for _ in range(copies - 1)]
    outs = []

    commit = None
    if linear and args.commit:
        # the sequences' lengths and histories, committed in place by every call
        # (capacity for every call of the run: warmup, parity, graph, timed steps and
        # the per-launch event pairs; lengths grow by at most k + 1 per call)
        cap = (args.steps + args.warmup + 2 * copies + 410) * (w.k + 1)
        commit = {"seq_len": torch.zeros(w.B, dtype=torch.int32, device=dev),
                  "history": torch.zeros((w.B, cap), dtype=torch.int32, device=dev)}

    def call(i):
        s = sets[i]
        if linear:
            kw = commit or {}
            if len(outs) <= i:
                outs.append(sv.verify_linear(s["t"], s["d"], s["x"], s["u"], mode=w.mode,
                                             temperature=w.temperature, **kw))
                return outs[i]
            return sv.verify_linear(s["t"], s["d"], s["x"], s["u"], mode=w.mode,
                                    temperature=w.temperature, out=outs[i], **kw)
        if w.mode == "typical":
            return sv.verify_tree(s["par"], s["cand"], s["lg"], s["u"], w.max_depth, mode="typical",
                                  temperature=w.temperature, epsilon=TYPICAL_EPS, delta=TYPICAL_DELTA)
        r = sv.verify_tree(s["par"], s["cand"], s["lg"], s["u"], w.max_depth, mode=w.mode,
                           temperature=w.temperature)
        return r

    # ---------------------------------------------------------------- parity gate
    import oracle
    first = call(0)
    torch.cuda.synchronize()
    if linear:
        o = oracle.verify_linear(w.mode, w.temperature, w.target, w.draft if stoch else None,
                                 w.draft_tokens, w.uniforms, w.V, w.dtype)
        g_acc = first["accept_len"].cpu().numpy()
        g_out = first["out_tokens"].cpu().numpy()
        differ = (g_acc != o["accept_len"]) | np.any(g_out != o["out_tokens"], axis=1)
    else:
        sample = list(range(w.B))          # every tree of the batch
        if w.mode == "typical":
            o = oracle.verify_tree_typical(w.temperature, TYPICAL_EPS, TYPICAL_DELTA, w.parent, w.cand[sample],
                                           w.logits[sample], w.uniforms[sample], w.V, w.dtype, w.max_depth)
        else:
            o = oracle.verify_tree(w.mode, w.temperature, w.parent, w.cand[sample], w.logits[sample],
                                   w.uniforms[sample], w.V, w.dtype, w.max_depth)
        g_acc = first["accept_len"].cpu().numpy()[sample]
        g_out = first["out_tokens"].cpu().numpy()[sample]
        differ = (g_acc != o["accept_len"]) | np.any(g_out != o["out_tokens"], axis=1)
    # a near tie in a draw that decides the accepted length excuses any difference,
    # one in the final draw only a different final token
    L_o = np.maximum(o["accept_len"], 0)
    final_col = np.arange(g_out.shape[1])[None, :] == L_o[:, None]
    diff_path = (g_acc != o["accept_len"]) | np.any((g_out != o["out_tokens"]) & ~final_col, axis=1)
    if "path_nodes" in o:
        diff_path |= np.any(first["path_nodes"].cpu().numpy()[sample] != o["path_nodes"], axis=1)
    bad = (diff_path & ((o["near_tie"] & oracle.NT_DECISION) == 0)) | (differ & (o["near_tie"] == 0))
    parity = {"checked": int(len(differ)), "exceptions": int(differ.sum()),
              "near_tie_sequences": int((o["near_tie"] != 0).sum()), "ok": bool(not bad.any())}
    if not parity["ok"]:
        print(f"[bench] PARITY FAILED: {parity}", file=sys.stderr, flush=True)
        sys.exit(1)
    print(f"[bench] parity vs oracle ok: {parity}", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- warmup
    for i in range(args.warmup):
        call(i % copies)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    # exactly --steps launches: a graph over all the input copies, replayed as often
    # as it fits, then one over the first (steps mod copies) of them
    K = max(1, args.steps)
    stream = torch.cuda.current_stream()
    if not args.no_graph:
        reps, rem = divmod(K, copies)
        graphs = []
        for n in ((copies,) if reps else ()) + ((rem,) if rem else ()):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    call(i)
            g.replay()
            graphs.append(g)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(reps):
            graphs[0].replay()
        if rem:
            graphs[-1].replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gpu_ms = ev0.elapsed_time(ev1)
        # graph replays must reproduce the eager result
        if linear:
            eager = call(0)
            torch.cuda.synchronize()
            assert torch.equal(eager["out_tokens"], outs[0]["out_tokens"])
    else:
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(K):
            call(i % copies)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gpu_ms = ev0.elapsed_time(ev1)
    wall_ms = (t1 - t0) * 1e3
    ms_per_step = wall_ms / K

    # ---------------------------------------------------------------- kernel duration (HIP events)
    # A linear step is one kernel launch, so the launch duration is the timed
    # region's event time over its K launches (launch gaps included: an upper
    # bound). A tree step is two launches (streaming, then the path search); the
    # figure covers both.
    # Second figure: one event pair per launch, with the GPU held by a spin kernel
    # while the host enqueues, so that host launch gaps stay out of the pairs.
    nprof = min(K, 400)
    cal0, cal1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cal0.record(stream)
    torch.cuda._sleep(1_000_000)
    cal1.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(cal0.elapsed_time(cal1), 1e-3)
    hold = int(cycles_per_ms * max(20.0, nprof * 0.1))   # >= 0.1 ms of host time per step
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nprof)]
    torch.cuda._sleep(hold)
    for n in range(nprof):
        evs[n][0].record(stream)
        call(n % copies)
        evs[n][1].record(stream)
    torch.cuda.synchronize()
    pair_us = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in evs]))
    dom_us = gpu_ms * 1e3 / K
    dominant = "linear_kernel" if linear else "tree_stream_kernel+tree_walk_kernel"

    # ---------------------------------------------------------------- the same bytes, only read
    # The same input copies read by spec_read_probe (the streaming waves' load
    # pattern, no arithmetic, one word written per chunk), K launches timed the same
    # way: what reading these bytes costs by itself on this GPU.
    pr_bufs = [((s["t"], s["d"]) if linear else (s["lg"], None)) for s in sets]
    sink = torch.empty(sv.read_probe_words(*pr_bufs[0]), dtype=torch.int32, device=dev)
    probe = lambda i: sv.read_probe(*pr_bufs[i], sink=sink)
    if not args.no_graph:
        _, _, pr_ms = _graph_time(torch, probe, copies, K, args.warmup)
    else:
        for i in range(args.warmup):
            probe(i % copies)
        pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        pe0.record(stream)
        for i in range(K):
            probe(i % copies)
        pe1.record(stream)
        torch.cuda.synchronize()
        pr_ms = pe0.elapsed_time(pe1) / K
    plain_us = pr_ms * 1e3

    npos = positions(w)
    value = npos / (ms_per_step * 1e-3)
    step_gbps = alg_bytes / (ms_per_step * 1e-3) / 1e9
    dom_gbps = alg_bytes / (dom_us * 1e-6) / 1e9
    traffic = measured_traffic(f"{args.config}/{w.mode}/seed{args.seed}")

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        n_rep, t_c0 = 0, time.perf_counter()
        while True:
            if linear:
                oracle.verify_linear(w.mode, w.temperature, w.target, w.draft if stoch else None,
                                     w.draft_tokens, w.uniforms, w.V, w.dtype)
                per = w.B * w.k
                what = f"the full batch ({w.B} sequences)"
            elif w.mode == "typical":
                oracle.verify_tree_typical(w.temperature, TYPICAL_EPS, TYPICAL_DELTA, w.parent, w.cand[:1],
                                           w.logits[:1], w.uniforms[:1], w.V, w.dtype, w.max_depth)
                per = w.n_nodes - 1
                what = "one tree of the batch"
            else:
                oracle.verify_tree(w.mode, w.temperature, w.parent, w.cand[:1], w.logits[:1],
                                   w.uniforms[:1], w.V, w.dtype, w.max_depth)
                per = w.n_nodes - 1
                what = "one tree of the batch"
            n_rep += 1
            el = time.perf_counter() - t_c0
            if el > args.cpu_seconds:
                break
        cpu = {"value": n_rep * per / el, "unit": "positions/s", "cores": 1, "kind": "oracle",
               "sample": f"{what} x {n_rep} repetitions, {el:.1f}s, single-threaded double-precision "
                         f"oracle on {platform.processor() or platform.machine()} "
                         f"({os.cpu_count()} host cores visible)"}

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {gen.DT_F32: "f32", gen.DT_BF16: "bf16", gen.DT_F16: "f16"}[w.dtype],
        "data": "synthetic (seeded generator; no dataset)",
        "config": {"workload": describe(w) + (" + commit in the same launch" if commit else ""),
                   "global_batch": w.B,
                   "positions_per_step": npos, "algorithmic_bytes_per_step": alg_bytes,
                   "input_copies": copies, "graph": not args.no_graph},
        "logit_GBps": step_gbps,
        "hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "kernel_us": pair_us,
        "gpu_ms_timed_region": gpu_ms,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": dom_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dom_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "traffic_detail": traffic, "launch_us": dom_us,
                     "algorithmic_bytes": alg_bytes,
                     "plain_read_us": plain_us, "plain_read_GBps": alg_bytes / (plain_us * 1e-6) / 1e9,
                     "frac_of_plain_read": plain_us / dom_us},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
