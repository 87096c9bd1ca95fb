"""Benchmark of the gate-first sparse FFN forward pass on one MI355X.

Workload (the decode shape): D = 2560, H = 7168, bf16 weights with fp32
accumulation, R-S+ gate, sparsity 0.9, batch 1, a stream of 1024 sequential
tokens. One step = the 1024 tokens, each a separate sffn_forward_sparse call
with T = 1, captured once into a HIP graph and replayed. Token t reads weight
replica t % R (R = 16 byte-identical copies, 1.76 GB in all) so that the
weights come from HBM and not from the 256 MB on-package cache.

Prints one JSON line: tokens/s of the sparse path (`value`), touched-byte HBM
GB/s, the dense comparator and LoPA on the same kind of stream, the roofline
of the dominant kernel (the longest per-token launch) from its own measured launch
durations, and the fp64 CPU oracle timed on a bounded sample of the same
stream as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CALIB_BYTES = 256 << 20   # the calibration copy reads and writes this many bytes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("activation_sparse_gated_amd/csrc/sffn_kernels.hip",
                "activation_sparse_gated_amd/csrc/sffn_api.hip"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_graph_durations(name: str):
    """Mean duration (us) per kernel over the timed graph replays, from the committed
    rocprofv3 kernel trace of the bench command, if it was taken on the current kernel
    sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("graph_replay_mean_us")


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _rocpd_rows(db_dir, query):
    import glob
    import sqlite3
    rows = []
    for db in sorted(glob.glob(os.path.join(db_dir, "**", "*.db"), recursive=True)):
        con = sqlite3.connect(db)
        rows += con.execute(query).fetchall()
        con.close()
    return rows


# bench.py launches this one-byte fill right before the warmup of the timed graph
# replays and right after them, so a kernel trace can be cut to the timed region
MARKER_KERNEL = "FillFunctor<unsigned char>"


def summarize_trace(db_dir: str, out: str, command: str) -> None:
    """Kernel-trace summary (count, mean/min/max duration) of a rocprofv3 run as markdown,
    for the whole run and, when bench.py's markers are present, for the dispatches of the
    timed graph replays alone; the graph-replay means also go to a JSON file beside it
    (with the kernel source hash) for bench.py's roofline."""
    rows = _rocpd_rows(db_dir, "select name, start, end from kernels order by start")
    short = [r[0].split("(")[0].replace("void ", "") for r in rows]
    marks = [i for i, n in enumerate(short) if MARKER_KERNEL in n]

    def table(idx):
        acc = {}
        for i in idx:
            d = (rows[i][2] - rows[i][1]) / 1e3
            a = acc.setdefault(short[i], [])
            a.append(d)
        out_rows = sorted(acc.items(), key=lambda kv: -sum(kv[1]))
        lines = ["| kernel | launches | mean us | min us | max us | total ms |", "|---|---|---|---|---|---|"]
        for name, ds in out_rows:
            lines.append(f"| `{name}` | {len(ds)} | {sum(ds) / len(ds):.3f} | {min(ds):.3f} | "
                         f"{max(ds):.3f} | {sum(ds) / 1e3:.3f} |")
        return lines, {name: sum(ds) / len(ds) for name, ds in out_rows}

    lines = [f"# rocprofv3 kernel trace: {os.path.basename(out)}", "", "Command (from the repo root):",
             "", "```", command, "```", ""]
    graph = None
    if len(marks) >= 2:
        idx = [i for i in range(marks[0] + 1, marks[1]) if MARKER_KERNEL not in short[i]]
        t, graph = table(idx)
        span_us = (rows[marks[1]][1] - rows[marks[0]][2]) / 1e3
        lines += ["## Timed graph replays (warmup and timed steps, between the markers)", "",
                  f"{len(idx)} dispatches over {span_us:,.1f} us.", ""] + t + [""]
    t, _ = table(range(len(rows)))
    lines += ["## Whole run (graph replays, eager passes, set-up)", ""] + t
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    if graph is not None:
        with open(os.path.splitext(out)[0] + ".json", "w") as f:
            json.dump({"source_hash": kernel_source_hash(), "command": command,
                       "graph_replay_mean_us": {k: round(v, 4) for k, v in graph.items()}}, f,
                      indent=2)


def summarize_pmc(fetch_dir: str, write_dir: str, kernel: str, out: str, command: str,
                  workload: str = "decode") -> None:
    """HBM bytes per launch of `kernel` from FETCH_SIZE and WRITE_SIZE runs, each scaled by
    what the same counter reads for the calibration copy of CALIB_BYTES in the same run."""
    q = ("select kernel_name, counter_name, avg(value), count(*) from counters_collection "
         "group by kernel_name, counter_name")
    res = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        vals = {name: (v, c) for name, cn, v, c in _rocpd_rows(d, q) if cn == counter}
        # the calibration is the one scalar multiply of a float tensor (torch.mul(t, 1.0))
        calib = [v for name, (v, c) in vals.items()
                 if "AUnaryFunctor<float, float, float" in name and "MulFunctor" in name]
        kern = [v for name, (v, c) in vals.items() if kernel + "<" in name or kernel + "(" in name]
        if not calib or not kern:
            raise SystemExit(f"{counter}: calibration copy or {kernel} not found in {d}")
        scale = CALIB_BYTES / (max(calib) * 1024.0)
        res[counter] = {"kib_per_dispatch": kern[0], "calib_kib": max(calib), "scale": scale,
                        "bytes_per_launch": kern[0] * 1024.0 * scale}
    d = {"kernel": kernel, "workload": workload, "source_hash": kernel_source_hash(),
         "command": command, "calibration_copy_bytes": CALIB_BYTES,
         "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"],
         "hbm_bytes_per_launch": round(res["FETCH_SIZE"]["bytes_per_launch"]
                                       + res["WRITE_SIZE"]["bytes_per_launch"], 0)}
    with open(out, "w") as f:
        json.dump(d, f, indent=2)



def summarize_counters(db_dir: str, out: str, command: str) -> None:
    """Per-kernel averages of every counter in a rocprofv3 --pmc run, as markdown."""
    q = ("select kernel_name, counter_name, avg(value), count(*) from counters_collection "
         "group by kernel_name, counter_name order by kernel_name, counter_name")
    rows = _rocpd_rows(db_dir, q)
    lines = [f"# rocprofv3 counters: {os.path.basename(out)}", "", "Command (from the repo root):",
             "", "```", command, "```", "", "| kernel | counter | mean per dispatch | dispatches |",
             "|---|---|---|---|"]
    for name, cn, v, c in rows:
        short = name.split("(")[0].replace("void ", "")
        if "AUnaryFunctor<float, float, float" in name and "MulFunctor" in name:
            # the run's plain copy of known size, for scaling byte counters
            lines.append(f"| calibration copy ({CALIB_BYTES:,} B read, {CALIB_BYTES:,} B written) "
                         f"| {cn} | {v:,.1f} | {c} |")
            continue
        if not short.startswith("sffn::"):
            continue
        lines.append(f"| `{short}` | {cn} | {v:,.1f} | {c} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _calibration_copy(torch):
    """A plain copy of known size (one scalar multiply of CALIB_BYTES of floats), for
    scaling the HBM byte counters of a profile of this run."""
    calib = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    calib_out = torch.empty_like(calib)
    torch.mul(calib, 1.0, out=calib_out)
    torch.cuda.synchronize()
    del calib, calib_out


def _graph_time(torch, fn, steps, warmup):
    """Capture fn once into a HIP graph; ms per replay."""
    g = torch.cuda.CUDAGraph()
    fn()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _quant_batches(torch, sffn, h, fwd_sparse, fwd_dense, reps, x, y, n, args, sizes=(16, 64)):
    """Per-token-list, union (and, with fwd_dense, dense) calls of T tokens through a
    quantised forward; the weight tuple of each call is reps[c % len(reps)], x and y hold
    n tokens."""
    out = {}
    nk = sffn.sffn_kernel_kinds()
    for TB in sizes:
        rq = {}
        for name, fwd in (("per_token", fwd_sparse), ("union", fwd_sparse), ("dense", fwd_dense)):
            if fwd is None:
                continue

            def fn(TB=TB, fwd=fwd, name=name):
                for c in range(n // TB):
                    a_ = (h.ptr, x[TB * c:TB * c + TB]) + reps[c % len(reps)] + (y[TB * c:TB * c + TB], TB)
                    if name == "union":
                        fwd(*a_, sffn.SFFN_MODE_UNION)
                    elif name == "per_token":
                        fwd(*a_, sffn.SFFN_MODE_PER_TOKEN)
                    else:
                        fwd(*a_)
            ms = _graph_time(torch, fn, max(2, args.steps // 2), 1)
            rq[name + "_tokens_per_s"] = round(TB * (n // TB) / (ms * 1e-3), 1)
            if name == "union":
                sffn.sffn_timing_enable(h.ptr, True)
                fn()
                torch.cuda.synchronize()
                sffn.sffn_timing_enable(h.ptr, False)
                kb = {}
                for kd in range(nk):
                    ms_k, launches = sffn.sffn_timing_read(h.ptr, kd, reset=(kd == nk - 1))
                    if launches:
                        kb[sffn.sffn_kernel_name(kd)] = round(ms_k * 1e3 / launches, 3)
                rq["union_kernel_us"] = kb
        if "dense_tokens_per_s" in rq:
            rq["union_vs_dense"] = round(rq["union_tokens_per_s"] / rq["dense_tokens_per_s"], 3)
        out[f"T{TB}"] = rq
    return out


def bench_lopa_batched(torch, sffn, gen, to_dev, act, args):
    """LoPA token batches (D=2560, H'=9787, r=400, s=0.9; 8 weight replicas, 32 calls
    per replay): per-token lists and the union of live sets, T = 4, 16, 64."""
    D, Hp, r, R = 2560, 9787, 400, 8
    w = gen.lopa_weights(D, Hp, r, 0.9, cfg=3, dtype="bf16")
    W = {k: to_dev(w[k]) for k in ("V", "U", "W3", "W2T")}
    reps = [{k: (W[k] if i == 0 else W[k].clone()) for k in W} for i in range(R)]
    xb = to_dev(gen.tokens(D, 64 * 32, cfg=3, dtype="bf16"))
    h = sffn.Handle(D, Hp, r, 64, act, sffn.SFFN_BF16)
    y = torch.zeros(64 * 32, D, dtype=torch.float32, device="cuda")
    out = {}
    for T in (4, 16, 64):
        res = {}
        for name, mode in (("per_token", sffn.SFFN_MODE_PER_TOKEN), ("union", sffn.SFFN_MODE_UNION)):
            def fn():
                for c in range(32):
                    rp = reps[c % R]
                    sffn.sffn_forward_lopa(h.ptr, xb[c * T:(c + 1) * T], rp["V"], rp["U"], rp["W3"],
                                           rp["W2T"], y[c * T:(c + 1) * T], T, mode)
            ms = _graph_time(torch, fn, max(2, args.steps // 4), 1) / 32
            res[name + "_tokens_per_s"] = round(T / (ms * 1e-3), 1)
        res["union_vs_per_token"] = round(res["union_tokens_per_s"] / res["per_token_tokens_per_s"], 3)
        out[f"T{T}"] = res
        log(f"lopa batched T={T}: " + ", ".join(f"{k} {v:,}" for k, v in res.items()))
    h.close()
    del reps, W
    torch.cuda.empty_cache()
    return out


def bench_batched(torch, sffn, gen, to_dev, x1, reps, D, H, act, args):
    """Token batches of T = 1, 4, 16, 64 at s = 0.9 (i.i.d. tokens, independent live sets):
    per-token lists, union of live sets, and the dense comparator. 64 calls per replay."""
    R = len(reps)
    out = {}
    xb = to_dev(gen.tokens(D, 64 * 64, cfg=4, dtype="bf16"))
    sizes = [int(v) for v in args.batched_sizes.split(",") if v]
    modes = [v for v in args.batched_modes.split(",") if v]
    for T in sizes:
        h = sffn.Handle(D, H, 0, T, act, sffn.SFFN_BF16)
        y = torch.zeros(64 * T, D, dtype=torch.float32, device="cuda")
        calls = 64
        res = {}
        for name, mode in (("per_token", sffn.SFFN_MODE_PER_TOKEN), ("union", sffn.SFFN_MODE_UNION),
                           ("dense", None)):
            if name not in modes:
                continue

            def fn():
                for c in range(calls):
                    rp = reps[c % R]
                    xs, ys = xb[c * T:(c + 1) * T], y[c * T:(c + 1) * T]
                    if mode is None:
                        sffn.sffn_forward_dense(h.ptr, xs, rp["W1"], rp["W3"], rp["W2T"], ys, T)
                    else:
                        sffn.sffn_forward_sparse(h.ptr, xs, rp["W1"], rp["W3"], rp["W2T"], ys, T,
                                                 mode)
            ms = _graph_time(torch, fn, max(2, args.steps // 4), 1)
            res[name + "_tokens_per_s"] = round(calls * T / (ms * 1e-3), 1)
        if "union_tokens_per_s" in res and "dense_tokens_per_s" in res:
            res["union_vs_dense"] = round(res["union_tokens_per_s"] / res["dense_tokens_per_s"], 3)
        out[f"T{T}"] = res
        log(f"batched T={T}: " + ", ".join(f"{k} {v:,}" for k, v in res.items()))
        h.close()
    return out


def bench_prefill(torch, sffn, gen, to_dev, reps, D, H, act, args):
    """Large batches (prefill) of T tokens in one call, D=2560, H=7168, s=0.9: the union
    path and the dense comparator as MFMA GEMMs (above 1024 tokens the down pass is one
    hipBLASLt GEMM over every unit), their per-kernel durations, and the same FFN as three
    hipBLASLt bf16 matmuls through torch for comparison."""
    import torch.nn.functional as F
    sizes = [int(v) for v in args.prefill_sizes.split(",") if v]
    R = len(reps)
    tmax = max(sizes)
    h = sffn.Handle(D, H, 0, tmax, act, sffn.SFFN_BF16)
    xb = to_dev(gen.tokens(D, tmax, cfg=5, dtype="bf16"))
    y = torch.zeros(tmax, D, dtype=torch.float32, device="cuda")
    peak = 2500.0  # TFLOP/s, dense bf16 MFMA
    out = {}
    for T in sizes:
        calls = max(2, 4096 // T)
        res = {"calls_per_replay": calls}
        flops = 6.0 * H * D * T  # gate, up and down over every unit (the union is ~all units)
        for name, dense in (("union", False), ("dense", True)):
            def fn():
                for c in range(calls):
                    rp = reps[c % R]
                    if dense:
                        sffn.sffn_forward_dense(h.ptr, xb[:T], rp["W1"], rp["W3"], rp["W2T"], y[:T], T)
                    else:
                        sffn.sffn_forward_sparse(h.ptr, xb[:T], rp["W1"], rp["W3"], rp["W2T"], y[:T],
                                                 T, sffn.SFFN_MODE_UNION)
            ms = _graph_time(torch, fn, max(2, args.steps // 4), 1) / calls
            res[name + "_tokens_per_s"] = round(T / (ms * 1e-3), 1)
            res[name + "_TFLOPs"] = round(flops / (ms * 1e-3) / 1e12, 1)
        # per-kernel durations of the union path (events at kernel begin and end)
        sffn.sffn_timing_enable(h.ptr, True)
        for c in range(4):
            rp = reps[c % R]
            sffn.sffn_forward_sparse(h.ptr, xb[:T], rp["W1"], rp["W3"], rp["W2T"], y[:T], T,
                                     sffn.SFFN_MODE_UNION)
        torch.cuda.synchronize()
        sffn.sffn_timing_enable(h.ptr, False)
        kt = {}
        nk = sffn.sffn_kernel_kinds()
        for kd in range(nk):
            ms_k, launches = sffn.sffn_timing_read(h.ptr, kd, reset=(kd == nk - 1))
            if launches:
                kt[sffn.sffn_kernel_name(kd)] = round(ms_k * 1e3 / launches, 2)
        res["kernel_us"] = kt
        if "k_gate_up_gemm" in kt:
            res["gate_up_TFLOPs"] = round(4.0 * H * D * T / (kt["k_gate_up_gemm"] * 1e-6) / 1e12, 1)
        down = kt.get("k_down_gemm") or kt.get("down_gemm_hipblaslt")
        if down:
            res["down_TFLOPs"] = round(2.0 * H * D * T / (down * 1e-6) / 1e12, 1)
        res["frac_of_mfma_peak"] = round(res["union_TFLOPs"] / peak, 4)
        # the same FFN as torch bf16 matmuls (hipBLASLt), eager, same weights
        xt = xb[:T].view(torch.bfloat16)
        # every replica, as the library calls rotate through them (two would stay in the
        # memory-side cache at small T)
        wt = [{k: rp[k].view(torch.bfloat16) for k in ("W1", "W3", "W2T")} for rp in reps]

        def torch_ffn(wd):
            z = F.linear(xt, wd["W1"])
            u = F.linear(xt, wd["W3"])
            a = (torch.where(z >= 0, F.silu(z), torch.zeros_like(z)) if act == sffn.SFFN_ACT_RSPLUS
                 else torch.relu(z)) * u
            return torch.matmul(a, wd["W2T"])
        for i in range(3):
            torch_ffn(wt[i % R])
        torch.cuda.synchronize()
        n_t = max(4, calls)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n_t):
            torch_ffn(wt[i % R])
        e1.record()
        torch.cuda.synchronize()
        ms_t = e0.elapsed_time(e1) / n_t
        res["torch_bf16_tokens_per_s"] = round(T / (ms_t * 1e-3), 1)
        res["torch_bf16_TFLOPs"] = round(flops / (ms_t * 1e-3) / 1e12, 1)
        res["union_vs_dense"] = round(res["union_tokens_per_s"] / res["dense_tokens_per_s"], 3)
        res["union_vs_torch"] = round(res["union_tokens_per_s"] / res["torch_bf16_tokens_per_s"], 3)
        out[f"T{T}"] = res
        log(f"prefill T={T}: " + ", ".join(f"{k} {v:,}" for k, v in res.items() if not isinstance(v, dict))
            + f", kernels (us) {kt}")
    h.close()
    return out


def bench_moe(torch, sffn, gen, to_dev, act, args):
    """A synthetic top-2 mixture of 8 sparse experts of the decode shape (D=2560, H=7168,
    s=0.9; 880 MB of expert weights), 64 tokens per call, 16 routings per replay."""
    D, H, E, K, T, calls = 2560, 7168, 8, 2, 64, 16
    ex = [gen.standard_weights(D, H, 0.9, cfg=6, replica=e, dtype="bf16") for e in range(E)]
    W = [{k: to_dev(w[k]) for k in ("W1", "W3", "W2T")} for w in ex]
    del ex
    xs = to_dev(gen.tokens(D, T * calls, cfg=6, dtype="bf16"))
    routes = [gen.moe_routing(T, E, K, cfg=6, layer=c) for c in range(calls)]
    h = sffn.Handle(D, H, 0, T, act, sffn.SFFN_BF16)
    y = torch.zeros(T * calls, D, dtype=torch.float32, device="cuda")
    # union of live sets of each (call, expert): bytes each expert's weights contribute
    cnt = torch.zeros(T, dtype=torch.int32, device="cuda")
    idx = torch.zeros(T, H, dtype=torch.int32, device="cuda")
    ybuf = torch.zeros(T, D, dtype=torch.float32, device="cuda")
    byts = 0
    for c, (route, _) in enumerate(routes):
        for e in range(E):
            toks = np.flatnonzero((route == e).any(axis=1))
            if toks.size == 0:
                continue
            xe = xs[c * T:(c + 1) * T][torch.from_numpy(toks).cuda()].contiguous()
            sffn.sffn_forward_sparse(h.ptr, xe, W[e]["W1"], W[e]["W3"], W[e]["W2T"], ybuf, int(toks.size),
                                     sffn.SFFN_MODE_UNION, cnt, idx)
            torch.cuda.synchronize()
            cc = cnt.cpu().numpy()
            ii = idx.cpu().numpy()
            u = len(set(np.concatenate([ii[t, :cc[t]] for t in range(toks.size)]).tolist()))
            byts += 2 * (H * D + 2 * u * D)
    out = {}
    for name, dense in (("sparse", False), ("dense", True)):
        def fn():
            for c, (route, gate) in enumerate(routes):
                sffn.sffn_forward_moe(h.ptr, xs[c * T:(c + 1) * T], [w["W1"] for w in W],
                                      [w["W3"] for w in W], [w["W2T"] for w in W], route, gate,
                                      y[c * T:(c + 1) * T], T, dense=dense)
        ms = _graph_time(torch, fn, max(2, args.steps // 4), 1)
        out[name + "_tokens_per_s"] = round(calls * T / (ms * 1e-3), 1)
        if not dense:
            out["sparse_touched_GBps"] = round(byts / (ms * 1e-3) / 1e9, 1)
    out["sparse_vs_dense"] = round(out["sparse_tokens_per_s"] / out["dense_tokens_per_s"], 3)
    log("moe: " + ", ".join(f"{k} {v:,}" for k, v in out.items()))
    h.close()
    return out


def _device_layer(torch, D, H, sparsity, gen, layer, seed_base):
    """One FFN layer of the stack workload drawn on the device: W1, W3, W2T ~ N(0, 1/D)
    from a generator seeded per layer, W1[:, 0] = -Phi^-1(s) (the recipe of the
    inputs module, drawn by torch so that 32 layers of the wide shape take seconds)."""
    g = torch.Generator(device="cuda")
    out = {}
    for i, k in enumerate(("W1", "W3", "W2T")):
        g.manual_seed(seed_base + 1000 * layer + i)
        w = torch.randn(H, D, generator=g, device="cuda", dtype=torch.float32) / np.sqrt(D)
        if k == "W1":
            w[:, 0] = float(gen.gate_offset(sparsity))
        out[k] = w.to(torch.bfloat16).view(torch.int16)
        del w
    return out


def bench_stacks(torch, sffn, gen, to_dev, act, args):
    """32-layer stacks at s = 0.895, batch-1 decode of 256 tokens through all layers.
    Each layer has its own independently drawn weights (2.4 GB and 9.7 GB per stack);
    every (token, layer) pair gets its own input (layers are not chained), so each
    layer sees the workload's sparsity. Per-layer sparsity is measured outside the
    timed region."""
    out = {}
    for (D, H) in ((2048, 6144), (4096, 12288)):
        s = 0.895
        layers = [_device_layer(torch, D, H, s, gen, l, 2026 * 7919 + D) for l in range(32)]
        ntok = 256
        xs = to_dev(gen.tokens(D, ntok * 32, cfg=5, dtype="bf16"))
        h = sffn.Handle(D, H, 0, 1, act, sffn.SFFN_BF16)
        y = torch.zeros(ntok * 32, D, dtype=torch.float32, device="cuda")
        cnt = torch.zeros(ntok * 32, dtype=torch.int32, device="cuda")
        idx = torch.zeros(1, H, dtype=torch.int32, device="cuda")
        # live counts of the first 8 tokens through every layer (outside the timed region)
        for t in range(8):
            for l in range(32):
                i = t * 32 + l
                L = layers[l]
                sffn.sffn_forward_sparse(h.ptr, xs[i], L["W1"], L["W3"], L["W2T"], y[i], 1,
                                         sffn.SFFN_MODE_PER_TOKEN, cnt[i:i + 1], idx[0])
        torch.cuda.synchronize()
        kl = cnt[:8 * 32].view(8, 32).cpu().numpy().astype(np.float64)
        layer_sparsity = 1.0 - kl.mean(axis=0) / H
        res = {}
        for name, dense in (("sparse", False), ("dense", True)):
            def fn():
                for t in range(ntok):
                    for l in range(32):
                        i = t * 32 + l
                        L = layers[l]
                        if dense:
                            sffn.sffn_forward_dense(h.ptr, xs[i], L["W1"], L["W3"], L["W2T"], y[i], 1)
                        else:
                            sffn.sffn_forward_sparse(h.ptr, xs[i], L["W1"], L["W3"], L["W2T"], y[i], 1)
            ms = _graph_time(torch, fn, 2, 1)
            res[name + "_stack_tokens_per_s"] = round(ntok / (ms * 1e-3), 1)
            res[name + "_layer_tokens_per_s"] = round(ntok * 32 / (ms * 1e-3), 1)
        res["sparse_vs_dense"] = round(res["sparse_stack_tokens_per_s"] / res["dense_stack_tokens_per_s"], 3)
        res["layers"] = "32 independent draws, inputs not chained"
        res["layer_sparsity_min"] = round(float(layer_sparsity.min()), 4)
        res["layer_sparsity_mean"] = round(float(layer_sparsity.mean()), 4)
        res["layer_sparsity_max"] = round(float(layer_sparsity.max()), 4)
        out[f"D{D}_H{H}"] = res
        log(f"stack D={D} H={H}: " + ", ".join(f"{k} {v:,}" if not isinstance(v, str) else f"{k} {v}"
                                               for k, v in res.items()))
        h.close()
        del layers
        torch.cuda.empty_cache()
    return out


def _device_lopa_layer(torch, D, Hp, r, sparsity, gen, replica, seed_base):
    """One LoPA layer drawn on the device with the recipe of the inputs module:
    V ~ N(0, 1/D) with V[0] = e_0, U ~ N(0, 1/r) with U[:, 0] = c, W3 ~ N(0, 1/D),
    W2T ~ N(0, 1/H')."""
    g = torch.Generator(device="cuda")
    out = {}
    for i, (k, shape, std) in enumerate((("V", (r, D), D), ("U", (Hp, r), r), ("W3", (Hp, D), D),
                                         ("W2T", (Hp, D), Hp))):
        g.manual_seed(seed_base + 1000 * replica + i)
        w = torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32) / np.sqrt(std)
        if k == "V":
            w[0].zero_()
            w[0, 0] = 1.0
        if k == "U":
            w[:, 0] = float(gen.gate_offset(sparsity))
        out[k] = w.to(torch.bfloat16).view(torch.int16)
        del w
    return out


def bench_wide_lopa(torch, sffn, gen, act, args):
    """Standard gating against LoPA at one parameter count on the wide shape: D = 4096,
    H = 12288 against r = 640, H' = 16799, s = 0.9, batch-1 decode of 256 tokens over
    4 independently drawn replicas of each layer (and the dense comparator)."""
    D, H, r, s, R, n = 4096, 12288, 640, 0.9, 4, 256
    Hp = 16799
    std = [_device_layer(torch, D, H, s, gen, q, 4096 * 31 + q) for q in range(R)]
    lop = [_device_lopa_layer(torch, D, Hp, r, s, gen, q, 4096 * 37) for q in range(R)]
    xs = torch.from_numpy(gen.tokens(D, n, cfg=7, dtype="bf16").view(np.int16)).cuda()
    y = torch.zeros(n, D, dtype=torch.float32, device="cuda")
    cnt = torch.zeros(n, dtype=torch.int32, device="cuda")
    hs = sffn.Handle(D, H, 0, 1, act, sffn.SFFN_BF16)
    hl = sffn.Handle(D, Hp, r, 1, act, sffn.SFFN_BF16)
    idx = torch.zeros(Hp, dtype=torch.int32, device="cuda")
    out = {"shape": f"D={D}, H={H} against r={r}, H'={Hp}", "sparsity_target": s}
    for t in range(n):
        L = std[t % R]
        sffn.sffn_forward_sparse(hs.ptr, xs[t], L["W1"], L["W3"], L["W2T"], y[t], 1,
                                 sffn.SFFN_MODE_PER_TOKEN, cnt[t:t + 1], idx[:H])
    torch.cuda.synchronize()
    out["standard_measured_sparsity"] = round(float(1 - cnt.double().mean().item() / H), 4)
    for t in range(n):
        L = lop[t % R]
        sffn.sffn_forward_lopa(hl.ptr, xs[t], L["V"], L["U"], L["W3"], L["W2T"], y[t], 1,
                               sffn.SFFN_MODE_PER_TOKEN, cnt[t:t + 1], idx)
    torch.cuda.synchronize()
    out["lopa_measured_sparsity"] = round(float(1 - cnt.double().mean().item() / Hp), 4)

    def f_std():
        for t in range(n):
            L = std[t % R]
            sffn.sffn_forward_sparse(hs.ptr, xs[t], L["W1"], L["W3"], L["W2T"], y[t], 1)

    def f_dense():
        for t in range(n):
            L = std[t % R]
            sffn.sffn_forward_dense(hs.ptr, xs[t], L["W1"], L["W3"], L["W2T"], y[t], 1)

    def f_lopa():
        for t in range(n):
            L = lop[t % R]
            sffn.sffn_forward_lopa(hl.ptr, xs[t], L["V"], L["U"], L["W3"], L["W2T"], y[t], 1,
                                   sffn.SFFN_MODE_PER_TOKEN)

    for name, fn in (("standard", f_std), ("dense", f_dense), ("lopa", f_lopa)):
        ms = _graph_time(torch, fn, max(2, args.steps // 4), 1)
        out[name + "_tokens_per_s"] = round(n / (ms * 1e-3), 1)
    out["lopa_vs_standard"] = round(out["lopa_tokens_per_s"] / out["standard_tokens_per_s"], 3)
    out["standard_vs_dense"] = round(out["standard_tokens_per_s"] / out["dense_tokens_per_s"], 3)
    out["lopa_vs_dense"] = round(out["lopa_tokens_per_s"] / out["dense_tokens_per_s"], 3)
    log("wide lopa: " + ", ".join(f"{k} {v}" for k, v in out.items()))
    hs.close()
    hl.close()
    del std, lop
    torch.cuda.empty_cache()
    return out


def main() -> int:
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        summarize_trace(sys.argv[2], sys.argv[3], sys.argv[4])
        return 0
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4])
        return 0
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        summarize_pmc(*sys.argv[2:7], *(sys.argv[7:8] or ["decode"]))
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=1024)
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--sparsity", type=float, default=0.9)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU oracle baseline sample")
    ap.add_argument("--no-extras", action="store_true", help="skip the dense and LoPA streams")
    ap.add_argument("--only-lopa", action="store_true",
                    help="of the extra lines run only the LoPA streams (for counter collection)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-batched", action="store_true",
                    help="run only the batched-decode lines (for counter collection)")
    ap.add_argument("--batched-sizes", default="1,4,16,64", help="token batch sizes T")
    ap.add_argument("--batched-modes", default="per_token,union,dense",
                    help="batched lines to run: per_token, union, dense")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the large-batch (prefill) lines")
    ap.add_argument("--prefill-sizes", default="256,1024,2048", help="large batch sizes T")
    args = ap.parse_args()

    if args.gpus != 1:
        log(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
            "(the library's FFN path runs on one GPU and has no cross-GPU step).")
        return 2

    import torch

    from activation_sparse_gated_amd import inputs as gen
    from activation_sparse_gated_amd import sffn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    sffn.load()
    D, H, n, R, s = 2560, 7168, args.tokens, args.replicas, args.sparsity
    act = sffn.SFFN_ACT_RSPLUS

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    x_np = gen.tokens(D, n, cfg=2, dtype="bf16")
    w_np = gen.standard_weights(D, H, s, cfg=2, dtype="bf16")
    log(f"generated decode inputs in {time.time() - t0:.1f}s")

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    x = to_dev(x_np)
    W = {k: to_dev(w_np[k]) for k in ("W1", "W3", "W2T")}
    reps = [{k: (W[k] if r == 0 else W[k].clone()) for k in W} for r in range(R)]
    y = torch.zeros(n, D, dtype=torch.float32, device="cuda")
    cnt = torch.zeros(n, dtype=torch.int32, device="cuda")
    idx = torch.zeros(n, H, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    if args.only_batched:
        _calibration_copy(torch)
        res = bench_batched(torch, sffn, gen, to_dev, x, reps, D, H, act, args)
        print(json.dumps({"batched": res}), flush=True)
        return 0
    if args.only_prefill:
        res = bench_prefill(torch, sffn, gen, to_dev, reps, D, H, act, args)
        print(json.dumps({"prefill": res}), flush=True)
        return 0

    hs = sffn.Handle(D, H, 0, 1, act, sffn.SFFN_BF16)

    # live counts of every token (outside the timed region)
    for t in range(n):
        rp = reps[t % R]
        sffn.sffn_forward_sparse(hs.ptr, x[t], rp["W1"], rp["W3"], rp["W2T"], y[t], 1,
                                 sffn.SFFN_MODE_PER_TOKEN, cnt[t:t + 1], idx[t])
    torch.cuda.synchronize()
    k = cnt.cpu().numpy().astype(np.int64)
    meas_sparsity = 1.0 - k.mean() / H

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            fn()  # one eager pass on the capture stream before capturing
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time_graph(g, steps, warmup):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps  # ms per step

    def sparse_stream():
        for t in range(n):
            rp = reps[t % R]
            sffn.sffn_forward_sparse(hs.ptr, x[t], rp["W1"], rp["W3"], rp["W2T"], y[t], 1,
                                     sffn.SFFN_MODE_PER_TOKEN)

    g_sparse = capture(sparse_stream)
    marker = torch.empty(1, dtype=torch.uint8, device="cuda")
    marker.fill_(1)   # trace marker: the timed graph replays start
    ms_step = time_graph(g_sparse, args.steps, args.warmup)
    marker.fill_(2)   # trace marker: they end
    torch.cuda.synchronize()
    tok_s = n / (ms_step * 1e-3)
    bytes_tok = 2 * (H * D + 2 * k * D) + 6 * D          # weights read + x in + y out
    touched_gbps = bytes_tok.sum() / (ms_step * 1e-3) / 1e9
    log(f"sparse: {ms_step:.3f} ms/step, {tok_s:,.0f} tokens/s, {touched_gbps:,.0f} GB/s touched")

    # per-kernel durations, measured with HIP events at each kernel's own begin and end on
    # the stream it runs on; every 8th call of four passes over the token stream is timed,
    # so the calls between keep the GPU as busy as in the graph replay
    sffn.sffn_timing_enable(hs.ptr, 8)
    sffn.sffn_timing_read(hs.ptr, 0, reset=True)
    for _ in range(4):
        sparse_stream()
    torch.cuda.synchronize()
    sffn.sffn_timing_enable(hs.ptr, 0)
    kt = {}
    for kd in range(sffn.sffn_kernel_kinds()):
        ms, launches = sffn.sffn_timing_read(hs.ptr, kd)
        if launches:
            kt[sffn.sffn_kernel_name(kd)] = ms * 1e3 / launches   # us per launch
    sffn.sffn_timing_read(hs.ptr, 0, reset=True)
    dom = max(kt, key=kt.get)
    kmean = float(k.mean())
    # algorithmic bytes per launch of each batch-1 kernel (bf16 weights, fp32 unit products)
    algo_bytes = {
        "k_gate_up_t1": 2 * (H * D + kmean * D) + 2 * D + 4 * H,     # W1, live W3 rows, x, a out
        "k_down_t1": 2 * kmean * D + 4 * H + 4 * D,                  # live W2T rows, a in, y out
    }
    gate_bytes = algo_bytes.get(dom, float("nan"))
    # durations of the same kernels inside the timed graph replays, from the committed kernel
    # trace of this command when it was taken on the current sources (eager launches run
    # slower: the host cannot keep the GPU busy between them)
    gdur = read_graph_durations("decode_headline_kernel_trace") or {}

    def graph_us(kind):
        for name, us in gdur.items():
            if name.startswith(f"sffn::{kind}<") or name == f"sffn::{kind}":
                return us
        return None

    kt_graph = {kk: graph_us(kk) for kk in kt}
    if all(v is not None for v in kt_graph.values()):
        dom_us, dur_src = kt_graph[dom], ("rocprofv3 kernel trace of this command, timed graph "
                                          "replays (profiles/decode_headline_kernel_trace.json)")
    else:
        kt_graph = None
        dom_us, dur_src = kt[dom], "HIP events at the kernel's begin and end, eager pass"
    achieved = gate_bytes / (dom_us * 1e-6) / 1e9
    log("kernels (us/launch): " + ", ".join(f"{n_} {v:.2f}" for n_, v in kt.items()))
    log(f"dominant {dom}: {gate_bytes / 1e6:.2f} MB algorithmic per launch, {achieved:,.0f} GB/s")

    _calibration_copy(torch)

    extras = {}
    if not args.no_extras and not args.only_lopa:
        def dense_stream():
            for t in range(n):
                rp = reps[t % R]
                sffn.sffn_forward_dense(hs.ptr, x[t], rp["W1"], rp["W3"], rp["W2T"], y[t], 1)

        g_dense = capture(dense_stream)
        ms_dense = time_graph(g_dense, args.steps, args.warmup)
        sffn.sffn_timing_enable(hs.ptr, True)
        sffn.sffn_timing_read(hs.ptr, 0, reset=True)
        dense_stream()
        torch.cuda.synchronize()
        sffn.sffn_timing_enable(hs.ptr, False)
        kt_dense = {}
        for kd in range(sffn.sffn_kernel_kinds()):
            ms_, l_ = sffn.sffn_timing_read(hs.ptr, kd)
            if l_:
                kt_dense[sffn.sffn_kernel_name(kd)] = round(ms_ * 1e3 / l_, 3)
        sffn.sffn_timing_read(hs.ptr, 0, reset=True)
        dense_tok_s = n / (ms_dense * 1e-3)
        dense_gbps = n * (2 * 3 * H * D + 6 * D) / (ms_dense * 1e-3) / 1e9
        log(f"dense: {ms_dense:.3f} ms/step, {dense_tok_s:,.0f} tokens/s, {dense_gbps:,.0f} GB/s")
        extras.update({"dense_kernel_us": kt_dense,
                       "dense_tokens_per_s": round(dense_tok_s, 1),
                       "dense_GBps": round(dense_gbps, 1),
                       "speedup_vs_dense": round(tok_s / dense_tok_s, 3)})
        del g_dense

        # the workload's other sparsities: the same draws with W1's bias column set for s
        other = {}
        for s_o in (0.69, 0.76, 0.896):
            bits = gen.to_bf16_bits(np.array([gen.gate_offset(s_o)], np.float64)).view(np.int16)[0]
            W1o = W["W1"].clone()
            W1o[:, 0] = int(bits)
            W1r = [W1o if rr == 0 else W1o.clone() for rr in range(R)]
            for t in range(n):
                rp = reps[t % R]
                sffn.sffn_forward_sparse(hs.ptr, x[t], W1r[t % R], rp["W3"], rp["W2T"], y[t], 1,
                                         sffn.SFFN_MODE_PER_TOKEN, cnt[t:t + 1], idx[t])
            torch.cuda.synchronize()
            ko = cnt.cpu().numpy().astype(np.int64)

            def other_stream():
                for t in range(n):
                    rp = reps[t % R]
                    sffn.sffn_forward_sparse(hs.ptr, x[t], W1r[t % R], rp["W3"], rp["W2T"], y[t], 1,
                                             sffn.SFFN_MODE_PER_TOKEN)
            g_o = capture(other_stream)
            ms_o = time_graph(g_o, max(2, args.steps // 2), 1)
            del g_o, W1r, W1o
            tok_o = n / (ms_o * 1e-3)
            gbps_o = (2 * (H * D + 2 * ko * D) + 6 * D).sum() / (ms_o * 1e-3) / 1e9
            other[f"s{s_o}"] = {"tokens_per_s": round(tok_o, 1), "touched_GBps": round(float(gbps_o), 1),
                                "touched_frac_of_peak": round(float(gbps_o) / 8000.0, 4),
                                "measured_sparsity": round(float(1 - ko.mean() / H), 4),
                                "k_mean": round(float(ko.mean()), 1),
                                "speedup_vs_dense": round(tok_o / dense_tok_s, 3)}
            log(f"sparsity {s_o}: {tok_o:,.0f} tokens/s, {gbps_o:,.0f} GB/s touched, "
                f"measured {other[f's{s_o}']['measured_sparsity']}, {tok_o / dense_tok_s:.2f}x dense")
        extras["other_sparsities"] = other

    if not args.no_extras or args.only_lopa:
        # LoPA at constant parameter count: D = 2560, H' = 9787, r = 400
        Hp, r = 9787, 400
        wl = gen.lopa_weights(D, Hp, r, s, cfg=3, dtype="bf16")
        xl = to_dev(gen.tokens(D, n, cfg=3, dtype="bf16"))
        WL = {kk: to_dev(wl[kk]) for kk in ("V", "U", "W3", "W2T")}
        repl = [{kk: (WL[kk] if rr == 0 else WL[kk].clone()) for kk in WL} for rr in range(R)]
        hl = sffn.Handle(D, Hp, r, 1, act, sffn.SFFN_BF16)
        cl = torch.zeros(n, dtype=torch.int32, device="cuda")
        il = torch.zeros(n, Hp, dtype=torch.int32, device="cuda")
        for t in range(n):
            rp = repl[t % R]
            sffn.sffn_forward_lopa(hl.ptr, xl[t], rp["V"], rp["U"], rp["W3"], rp["W2T"], y[t], 1,
                                   sffn.SFFN_MODE_PER_TOKEN, cl[t:t + 1], il[t])
        torch.cuda.synchronize()
        kl = cl.cpu().numpy().astype(np.int64)

        def lopa_stream():
            for t in range(n):
                rp = repl[t % R]
                sffn.sffn_forward_lopa(hl.ptr, xl[t], rp["V"], rp["U"], rp["W3"], rp["W2T"], y[t], 1,
                                       sffn.SFFN_MODE_PER_TOKEN)

        g_lopa = capture(lopa_stream)
        ms_lopa = time_graph(g_lopa, args.steps, args.warmup)
        sffn.sffn_timing_enable(hl.ptr, 8)
        sffn.sffn_timing_read(hl.ptr, 0, reset=True)
        for _ in range(4):
            lopa_stream()
        torch.cuda.synchronize()
        sffn.sffn_timing_enable(hl.ptr, 0)
        lopa_kt = {}
        for kd in range(sffn.sffn_kernel_kinds()):
            ms_, l_ = sffn.sffn_timing_read(hl.ptr, kd)
            if l_:
                lopa_kt[sffn.sffn_kernel_name(kd)] = round(ms_ * 1e3 / l_, 3)
        sffn.sffn_timing_read(hl.ptr, 0, reset=True)
        lopa_tok_s = n / (ms_lopa * 1e-3)
        lopa_gbps = (2 * (r * (D + Hp) + 2 * kl * D) + 6 * D).sum() / (ms_lopa * 1e-3) / 1e9
        log(f"lopa: {ms_lopa:.3f} ms/step, {lopa_tok_s:,.0f} tokens/s, {lopa_gbps:,.0f} GB/s touched")
        extras.update({"lopa_tokens_per_s": round(lopa_tok_s, 1),
                       "lopa_touched_GBps": round(lopa_gbps, 1),
                       "lopa_measured_sparsity": round(float(1 - kl.mean() / Hp), 4),
                       "lopa_kernel_us": lopa_kt,
                       "lopa_speedup_vs_dense": (round(lopa_tok_s / extras["dense_tokens_per_s"], 3)
                                                 if "dense_tokens_per_s" in extras else None)})
        del g_lopa
        hl.close()

        # full LoPA gate on the same weights: tiled-identity G, RMSNorm of V x, double activation
        fl = sffn.SFFN_FLAG_G_TILED | sffn.SFFN_FLAG_RMSNORM | sffn.SFFN_FLAG_DOUBLE_ACT
        hf = sffn.Handle(D, Hp, r, 1, act, sffn.SFFN_BF16, fl)
        for t in range(n):
            rp = repl[t % R]
            sffn.sffn_forward_lopa(hf.ptr, xl[t], rp["V"], rp["U"], rp["W3"], rp["W2T"], y[t], 1,
                                   sffn.SFFN_MODE_PER_TOKEN, cl[t:t + 1], il[t])
        torch.cuda.synchronize()
        kf = cl.cpu().numpy().astype(np.int64)
        # W2T rows the double activation keeps: live units with W3_i . x > 0 (a byte count only,
        # in fp32 with torch, outside the timed region)
        valid = torch.arange(Hp, device="cuda")[None, :] < cl[:, None]
        rows = torch.arange(n, device="cuda")[:, None].expand(n, Hp)[valid]
        live_mask = torch.zeros(n, Hp, dtype=torch.bool, device="cuda")
        live_mask[rows, il[valid].long()] = True
        u3 = xl.view(torch.bfloat16).float() @ WL["W3"].view(torch.bfloat16).float().T
        k2f = ((u3 > 0) & live_mask).sum(1).cpu().numpy().astype(np.int64)
        del u3, live_mask, rows, valid

        def lopa_full_stream():
            for t in range(n):
                rp = repl[t % R]
                sffn.sffn_forward_lopa(hf.ptr, xl[t], rp["V"], rp["U"], rp["W3"], rp["W2T"], y[t],
                                       1, sffn.SFFN_MODE_PER_TOKEN)

        g_full = capture(lopa_full_stream)
        ms_full = time_graph(g_full, args.steps, args.warmup)
        full_tok_s = n / (ms_full * 1e-3)
        full_gbps = (2 * (r * (D + Hp) + kf * D + k2f * D) + 6 * D).sum() / (ms_full * 1e-3) / 1e9
        log(f"lopa full gate: {ms_full:.3f} ms/step, {full_tok_s:,.0f} tokens/s, "
            f"{full_gbps:,.0f} GB/s touched, k {kf.mean():.0f}, W2 rows {k2f.mean():.0f}")
        extras["lopa_full_gate"] = {
            "flags": "G_TILED|RMSNORM|DOUBLE_ACT", "tokens_per_s": round(full_tok_s, 1),
            "touched_GBps": round(float(full_gbps), 1),
            "measured_sparsity": round(float(1 - kf.mean() / Hp), 4),
            "w2_rows_mean": round(float(k2f.mean()), 1),
            "speedup_vs_dense": (round(full_tok_s / extras["dense_tokens_per_s"], 3)
                                 if "dense_tokens_per_s" in extras else None)}
        del g_full
        hf.close()

    # ---------------------------------------------------------------- weight-only int8 decode
    if not args.no_extras and not args.only_lopa:
        # the decode workload's fp64 draws quantized per row to int8 (same streams and offset)
        wq = gen.standard_weights_int8(D, H, s, cfg=2)
        WQ = {kk: torch.from_numpy(np.ascontiguousarray(wq[kk])).cuda()
              for kk in ("W1", "W3", "W2T", "W1_scale", "W3_scale", "W2T_scale")}
        repq = [{kk: (WQ[kk] if rr == 0 else WQ[kk].clone()) for kk in WQ} for rr in range(R)]
        hq = sffn.Handle(D, H, 0, 1, act, sffn.SFFN_I8)
        for t in range(n):
            rp = repq[t % R]
            sffn.sffn_forward_sparse_i8(hq.ptr, x[t], rp["W1"], rp["W1_scale"], rp["W3"],
                                        rp["W3_scale"], rp["W2T"], rp["W2T_scale"], y[t], 1,
                                        sffn.SFFN_MODE_PER_TOKEN, cnt[t:t + 1], idx[t])
        torch.cuda.synchronize()
        kq = cnt.cpu().numpy().astype(np.int64)

        def q8_stream(dense):
            def fn():
                for t in range(n):
                    rp = repq[t % R]
                    if dense:
                        sffn.sffn_forward_dense_i8(hq.ptr, x[t], rp["W1"], rp["W1_scale"], rp["W3"],
                                                   rp["W3_scale"], rp["W2T"], rp["W2T_scale"],
                                                   y[t], 1)
                    else:
                        sffn.sffn_forward_sparse_i8(hq.ptr, x[t], rp["W1"], rp["W1_scale"],
                                                    rp["W3"], rp["W3_scale"], rp["W2T"],
                                                    rp["W2T_scale"], y[t], 1,
                                                    sffn.SFFN_MODE_PER_TOKEN)
            return fn

        res_q = {}
        for name, dense in (("sparse", False), ("dense", True)):
            g_q = capture(q8_stream(dense))
            ms_q = time_graph(g_q, args.steps, args.warmup)
            del g_q
            kk_ = H if dense else kq
            # int8 weight bytes, the fp32 scales of the rows read, x in and y out
            bytes_q = (H * D + 2 * kk_ * D) + 4 * (H + 2 * kk_) + 6 * D
            if dense:
                bytes_q = np.full(n, 3 * H * D + 12 * H + 6 * D)
            res_q[name + "_tokens_per_s"] = round(n / (ms_q * 1e-3), 1)
            res_q[name + "_touched_GBps"] = round(float(np.sum(bytes_q)) / (ms_q * 1e-3) / 1e9, 1)
        # per-kernel durations of the int8 sparse stream
        sffn.sffn_timing_enable(hq.ptr, True)
        q8_stream(False)()
        torch.cuda.synchronize()
        sffn.sffn_timing_enable(hq.ptr, False)
        ktq = {}
        nk = sffn.sffn_kernel_kinds()
        for kd in range(nk):
            ms, launches = sffn.sffn_timing_read(hq.ptr, kd, reset=(kd == nk - 1))
            if launches:
                ktq[sffn.sffn_kernel_name(kd)] = round(ms * 1e3 / launches, 3)
        res_q["kernel_us"] = ktq
        res_q["measured_sparsity"] = round(float(1 - kq.mean() / H), 4)
        res_q["sparse_vs_dense_int8"] = round(res_q["sparse_tokens_per_s"] / res_q["dense_tokens_per_s"], 3)
        res_q["sparse_vs_dense_bf16"] = round(res_q["sparse_tokens_per_s"] / extras["dense_tokens_per_s"], 3)
        # batches of 4 tokens: per-token lists, the union of live sets, the dense comparator
        hq4 = sffn.Handle(D, H, 0, 4, act, sffn.SFFN_I8)
        b4 = {}
        for name, mode, dense in (("per_token", sffn.SFFN_MODE_PER_TOKEN, False),
                                  ("union", sffn.SFFN_MODE_UNION, False), ("dense", 0, True)):
            def fn4():
                for c in range(n // 4):
                    rp = repq[c % R]
                    args_q = (hq4.ptr, x[4 * c:4 * c + 4], rp["W1"], rp["W1_scale"], rp["W3"],
                              rp["W3_scale"], rp["W2T"], rp["W2T_scale"], y[4 * c:4 * c + 4], 4)
                    if dense:
                        sffn.sffn_forward_dense_i8(*args_q)
                    else:
                        sffn.sffn_forward_sparse_i8(*args_q, mode)
            g4 = capture(fn4)
            ms4 = time_graph(g4, args.steps, args.warmup)
            del g4
            b4[name + "_tokens_per_s"] = round(n / (ms4 * 1e-3), 1)
        b4["union_vs_dense"] = round(b4["union_tokens_per_s"] / b4["dense_tokens_per_s"], 3)
        res_q["batch4"] = b4
        hq4.close()
        # union and dense batches of 16 and 64 tokens (one MFMA pass over the codes per call)
        hq64 = sffn.Handle(D, H, 0, 64, act, sffn.SFFN_I8)
        res_q["batched"] = _quant_batches(
            torch, sffn, hq64, sffn.sffn_forward_sparse_i8, sffn.sffn_forward_dense_i8,
            [tuple(rp[k] for k in ("W1", "W1_scale", "W3", "W3_scale", "W2T", "W2T_scale"))
             for rp in repq], x, y, n, args)
        hq64.close()
        extras["int8"] = res_q
        log("int8: " + ", ".join(f"{kk} {v:,}" for kk, v in res_q.items() if not isinstance(v, dict))
            + f", kernels (us/launch) {ktq}, batch of 4 {b4}")
        hq.close()
        del repq, WQ

        # weight-only int4 with one scale per 128 columns: the decode workload's draws
        w4 = gen.standard_weights_int4(D, H, s, cfg=2)
        W4 = {kk: torch.from_numpy(np.ascontiguousarray(w4[kk])).cuda()
              for kk in ("W1", "W3", "W2T", "W1_scale", "W3_scale", "W2T_scale")}
        rep4 = [{kk: (W4[kk] if rr == 0 else W4[kk].clone()) for kk in W4} for rr in range(R)]
        h4 = sffn.Handle(D, H, 0, 1, act, sffn.SFFN_I4)

        def q4_call(t, dense=False, live=False):
            rp = rep4[t % R]
            if dense:
                sffn.sffn_forward_dense_i4(h4.ptr, x[t], rp["W1"], rp["W1_scale"], rp["W3"],
                                           rp["W3_scale"], rp["W2T"], rp["W2T_scale"], y[t], 1)
            else:
                sffn.sffn_forward_sparse_i4(h4.ptr, x[t], rp["W1"], rp["W1_scale"], rp["W3"],
                                            rp["W3_scale"], rp["W2T"], rp["W2T_scale"], y[t], 1,
                                            sffn.SFFN_MODE_PER_TOKEN, cnt[t:t + 1] if live else None,
                                            idx[t] if live else None)
        for t in range(n):
            q4_call(t, live=True)
        torch.cuda.synchronize()
        k4 = cnt.cpu().numpy().astype(np.int64)
        res4 = {}
        G4 = D // 128
        for name, dense in (("sparse", False), ("dense", True)):
            def fn4(dense=dense):
                for t in range(n):
                    q4_call(t, dense=dense)
            g4 = capture(fn4)
            ms4 = time_graph(g4, args.steps, args.warmup)
            del g4
            rows = np.full(n, H) if dense else k4
            # packed int4 rows (D/2 bytes), their group scales, x in and y out
            b4 = (H * D // 2 + 2 * rows * D // 2) + 4 * G4 * (H + 2 * rows) + 6 * D
            res4[name + "_tokens_per_s"] = round(n / (ms4 * 1e-3), 1)
            res4[name + "_touched_GBps"] = round(float(np.sum(b4)) / (ms4 * 1e-3) / 1e9, 1)
        sffn.sffn_timing_enable(h4.ptr, True)
        for t in range(n):
            q4_call(t)
        torch.cuda.synchronize()
        sffn.sffn_timing_enable(h4.ptr, False)
        kt4 = {}
        for kd in range(nk):
            ms_k, launches = sffn.sffn_timing_read(h4.ptr, kd, reset=(kd == nk - 1))
            if launches:
                kt4[sffn.sffn_kernel_name(kd)] = round(ms_k * 1e3 / launches, 3)
        res4["kernel_us"] = kt4
        res4["measured_sparsity"] = round(float(1 - k4.mean() / H), 4)
        res4["sparse_vs_dense_int4"] = round(res4["sparse_tokens_per_s"] / res4["dense_tokens_per_s"], 3)
        res4["sparse_vs_dense_bf16"] = round(res4["sparse_tokens_per_s"] / extras["dense_tokens_per_s"], 3)
        # batches of 4 tokens: per-token lists, the union of live sets, the dense comparator
        h44 = sffn.Handle(D, H, 0, 4, act, sffn.SFFN_I4)
        b44 = {}
        for name, mode, dense in (("per_token", sffn.SFFN_MODE_PER_TOKEN, False),
                                  ("union", sffn.SFFN_MODE_UNION, False), ("dense", 0, True)):
            def fn44():
                for c in range(n // 4):
                    rp = rep4[c % R]
                    args_4 = (h44.ptr, x[4 * c:4 * c + 4], rp["W1"], rp["W1_scale"], rp["W3"],
                              rp["W3_scale"], rp["W2T"], rp["W2T_scale"], y[4 * c:4 * c + 4], 4)
                    if dense:
                        sffn.sffn_forward_dense_i4(*args_4)
                    else:
                        sffn.sffn_forward_sparse_i4(*args_4, mode)
            g44 = capture(fn44)
            ms44 = time_graph(g44, args.steps, args.warmup)
            del g44
            b44[name + "_tokens_per_s"] = round(n / (ms44 * 1e-3), 1)
        b44["union_vs_dense"] = round(b44["union_tokens_per_s"] / b44["dense_tokens_per_s"], 3)
        res4["batch4"] = b44
        h44.close()
        h464 = sffn.Handle(D, H, 0, 64, act, sffn.SFFN_I4)
        res4["batched"] = _quant_batches(
            torch, sffn, h464, sffn.sffn_forward_sparse_i4, sffn.sffn_forward_dense_i4,
            [tuple(rp[k] for k in ("W1", "W1_scale", "W3", "W3_scale", "W2T", "W2T_scale"))
             for rp in rep4], x, y, n, args)
        h464.close()
        extras["int4_group128"] = res4
        log("int4: " + ", ".join(f"{kk} {v:,}" for kk, v in res4.items() if not isinstance(v, dict))
            + f", kernels (us/launch) {kt4}, batch of 4 {b44}")
        h4.close()
        del rep4, W4

        # quantised LoPA: the LoPA workload's fp64 draws with V, U, W3, W2T in int8 rows, and
        # with V, U in int8 rows and W3, W2T in int4 (one scale per 128 columns)
        names = ("V", "U", "W3", "W2T", "V_scale", "U_scale", "W3_scale", "W2T_scale")
        for bits in (8, 4):
            wlq = (gen.lopa_weights_int8 if bits == 8 else gen.lopa_weights_int4)(D, Hp, r, s, cfg=3)
            WLQ = {kk: torch.from_numpy(np.ascontiguousarray(wlq[kk])).cuda() for kk in names}
            replq = [{kk: (WLQ[kk] if rr == 0 else WLQ[kk].clone()) for kk in WLQ} for rr in range(R)]
            hlq = sffn.Handle(D, Hp, r, 1, act, sffn.SFFN_I8 if bits == 8 else sffn.SFFN_I4)
            fwd = sffn.sffn_forward_lopa_i8 if bits == 8 else sffn.sffn_forward_lopa_i4

            def lq_call(t, live=False):
                rp = replq[t % R]
                fwd(hlq.ptr, xl[t], rp["V"], rp["V_scale"], rp["U"], rp["U_scale"], rp["W3"],
                    rp["W3_scale"], rp["W2T"], rp["W2T_scale"], y[t], 1, sffn.SFFN_MODE_PER_TOKEN,
                    cl[t:t + 1] if live else None, il[t] if live else None)
            for t in range(n):
                lq_call(t, live=True)
            torch.cuda.synchronize()
            klq = cl.cpu().numpy().astype(np.int64)

            def lq_stream():
                for t in range(n):
                    lq_call(t)
            g_lq = capture(lq_stream)
            ms_lq = time_graph(g_lq, args.steps, args.warmup)
            del g_lq
            lq_tok_s = n / (ms_lq * 1e-3)
            # int8 V and U rows and their row scales; the live W3 and W2T rows (int8 with a
            # row scale, or int4 with a scale per 128 columns); x in and y out
            if bits == 8:
                lq_bytes = (r * (D + Hp) + 2 * klq * D) + 4 * (r + Hp + 2 * klq) + 6 * D
            else:
                lq_bytes = (r * (D + Hp) + klq * D) + 4 * (r + Hp) + 2 * klq * 4 * (D // 128) + 6 * D
            sffn.sffn_timing_enable(hlq.ptr, True)
            lq_stream()
            torch.cuda.synchronize()
            sffn.sffn_timing_enable(hlq.ptr, False)
            ktl = {}
            for kd in range(nk):
                ms_k, launches = sffn.sffn_timing_read(hlq.ptr, kd, reset=(kd == nk - 1))
                if launches:
                    ktl[sffn.sffn_kernel_name(kd)] = round(ms_k * 1e3 / launches, 3)
            extras["lopa_int8" if bits == 8 else "lopa_int4_up_down"] = {
                "tokens_per_s": round(lq_tok_s, 1),
                "touched_GBps": round(float(np.sum(lq_bytes)) / (ms_lq * 1e-3) / 1e9, 1),
                "touched_MB_per_token": round(float(np.mean(lq_bytes)) / 1e6, 3),
                "measured_sparsity": round(float(1 - klq.mean() / Hp), 4),
                "speedup_vs_lopa_bf16": round(lq_tok_s / extras["lopa_tokens_per_s"], 3),
                "speedup_vs_dense_bf16": round(lq_tok_s / extras["dense_tokens_per_s"], 3),
                "kernel_us": ktl}
            # batches of 4 tokens: token by token, and the union of the four live sets
            hlq4 = sffn.Handle(D, Hp, r, 4, act, sffn.SFFN_I8 if bits == 8 else sffn.SFFN_I4)
            bq4 = {}
            for name, mode in (("per_token", sffn.SFFN_MODE_PER_TOKEN),
                               ("union", sffn.SFFN_MODE_UNION)):
                def fnq4():
                    for c in range(n // 4):
                        rp = replq[c % R]
                        fwd(hlq4.ptr, xl[4 * c:4 * c + 4], rp["V"], rp["V_scale"], rp["U"],
                            rp["U_scale"], rp["W3"], rp["W3_scale"], rp["W2T"], rp["W2T_scale"],
                            y[4 * c:4 * c + 4], 4, mode)
                gq4 = capture(fnq4)
                msq4 = time_graph(gq4, args.steps, args.warmup)
                del gq4
                bq4[name + "_tokens_per_s"] = round(4 * (n // 4) / (msq4 * 1e-3), 1)
                if mode == sffn.SFFN_MODE_UNION:
                    sffn.sffn_timing_enable(hlq4.ptr, True)
                    fnq4()
                    torch.cuda.synchronize()
                    sffn.sffn_timing_enable(hlq4.ptr, False)
                    ktq4 = {}
                    for kd in range(nk):
                        ms_k, launches = sffn.sffn_timing_read(hlq4.ptr, kd, reset=(kd == nk - 1))
                        if launches:
                            ktq4[sffn.sffn_kernel_name(kd)] = round(ms_k * 1e3 / launches, 3)
                    bq4["union_kernel_us"] = ktq4
            bq4["union_vs_per_token"] = round(bq4["union_tokens_per_s"] / bq4["per_token_tokens_per_s"], 3)
            extras["lopa_int8" if bits == 8 else "lopa_int4_up_down"]["batch4"] = bq4
            hlq4.close()
            hlq64 = sffn.Handle(D, Hp, r, 64, act, sffn.SFFN_I8 if bits == 8 else sffn.SFFN_I4)
            extras["lopa_int8" if bits == 8 else "lopa_int4_up_down"]["batched_union"] = _quant_batches(
                torch, sffn, hlq64, fwd, None,
                [tuple(rp[k] for k in ("V", "V_scale", "U", "U_scale", "W3", "W3_scale", "W2T",
                                       "W2T_scale")) for rp in replq], xl, y, n, args)
            hlq64.close()
            log(f"lopa int{bits}: {ms_lq:.3f} ms/step, {lq_tok_s:,.0f} tokens/s, "
                f"kernels (us/launch) {ktl}, batch of 4 {bq4}")
            hlq.close()
            del replq, WLQ

    # ---------------------------------------------------------------- batched decode and stacks
    if not args.no_extras and not args.only_lopa:
        extras["batched"] = bench_batched(torch, sffn, gen, to_dev, x, reps, D, H, act, args)
        extras["lopa_batched"] = bench_lopa_batched(torch, sffn, gen, to_dev, act, args)
        extras["lopa_wide"] = bench_wide_lopa(torch, sffn, gen, act, args)
        extras["stacks"] = bench_stacks(torch, sffn, gen, to_dev, act, args)
        extras["moe_top2_8x"] = bench_moe(torch, sffn, gen, to_dev, act, args)
        extras["prefill"] = bench_prefill(torch, sffn, gen, to_dev, reps, D, H, act, args)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        from oracle import reference as ref
        threads = ref.num_threads()
        done, t0 = 0, time.time()
        while time.time() - t0 < args.cpu_seconds and done < 64 * n:
            ref.ffn_standard(x_np[done % n], w_np["W1"], w_np["W3"], w_np["W2T"],
                             act=ref.ACT_RSPLUS)
            done += 1
        dt = time.time() - t0
        # the same oracle on one thread, over a shorter sample
        ref.set_threads(1)
        done1, t1 = 0, time.time()
        while time.time() - t1 < args.cpu_seconds / 4:
            ref.ffn_standard(x_np[done1 % n], w_np["W1"], w_np["W3"], w_np["W2T"],
                             act=ref.ACT_RSPLUS)
            done1 += 1
        dt1 = time.time() - t1
        ref.set_threads(threads)
        cpu_model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        cpu_model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        cpu = {"value": round(done / dt, 2), "unit": "tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{done} tokens of the {n}-token decode stream (cycled from token 0) "
                         f"through the fp64 sparse oracle: {dt:.1f} s, OpenMP over {threads} "
                         f"threads",
               "one_thread_value": round(done1 / dt1, 2),
               "one_thread_sample": f"{done1} tokens on 1 thread: {dt1:.1f} s",
               "cpu_model": cpu_model, "os_cpu_count": os.cpu_count()}
        log(f"cpu oracle: {cpu['value']} tokens/s on {threads} threads ({done} tokens), "
            f"{cpu['one_thread_value']} tokens/s on 1 thread; {cpu_model}")
        if not args.no_extras:
            # the 32-layer stacks: the first 8 stack tokens through all 32 layers,
            # extrapolated (the oracle's time does not depend on the weight values, so one
            # drawn layer stands for each of the 32)
            stk = {}
            for (Ds, Hs) in ((2048, 6144), (4096, 12288)):
                ws = gen.standard_weights(Ds, Hs, 0.895, cfg=5, dtype="bf16")
                xs_np = gen.tokens(Ds, 8 * 32, cfg=5, dtype="bf16")
                t2 = time.time()
                ref.ffn_standard(xs_np, ws["W1"], ws["W3"], ws["W2T"], act=ref.ACT_RSPLUS)
                dts = time.time() - t2
                stk[f"D{Ds}_H{Hs}"] = {
                    "stack_tokens_per_s": round(8 / dts, 3),
                    "layer_tokens_per_s": round(8 * 32 / dts, 1),
                    "sample": f"extrapolated: 8 stack tokens x 32 layers through the fp64 sparse "
                              f"oracle on {threads} threads, {dts:.2f} s"}
                del ws
            cpu["stacks_extrapolated"] = stk
            log("cpu oracle stacks (extrapolated from 8 tokens): " + ", ".join(
                f"{k} {v['stack_tokens_per_s']} stack tokens/s" for k, v in stk.items()))
            # LoPA (D = 2560, H' = 9787, r = 400): the LoPA workload's tokens through the fp64
            # LoPA oracle for about a quarter of the decode sample's time
            wlo = gen.lopa_weights(D, 9787, 400, s, cfg=3, dtype="bf16")
            xlo = gen.tokens(D, 256, cfg=3, dtype="bf16")
            donel, t3 = 0, time.time()
            while time.time() - t3 < args.cpu_seconds / 4:
                ref.ffn_lopa(xlo[donel % 256], wlo["V"], wlo["U"], wlo["W3"], wlo["W2T"],
                             act=ref.ACT_RSPLUS)
                donel += 1
            dtl = time.time() - t3
            cpu["lopa"] = {"tokens_per_s": round(donel / dtl, 2),
                           "sample": f"{donel} LoPA tokens through the fp64 LoPA oracle on "
                                     f"{threads} threads: {dtl:.1f} s"}
            log(f"cpu oracle lopa: {cpu['lopa']['tokens_per_s']} tokens/s")
            del wlo

    traffic = read_traffic(dom, "decode")
    out = {
        "metric": "sparse-FFN tokens/s + touched-bytes HBM GB/s vs dense, D=2560 H=7168 90% sparsity",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode: D=2560 H=7168, bf16 weights, fp32 accumulate, R-S+ gate, "
                               f"sparsity {s}, batch 1, {n} sequential tokens per step, "
                               f"{R} rotating weight replicas",
                   "D": D, "H": H, "sparsity": s, "batch": 1, "tokens_per_step": n,
                   "replicas": R, "parallelism": "single GPU"},
        "touched_GBps": round(float(touched_gbps), 1),
        "touched_frac_of_peak": round(float(touched_gbps) / HBM_PEAK_GBPS, 4),
        "measured_sparsity": round(float(meas_sparsity), 4),
        "k_mean": round(float(k.mean()), 1),
        "k_std": round(float(k.std()), 1),
        "us_per_token": round(ms_step * 1e3 / n, 3),
        "kernel_us": {kk: round(v, 3) for kk, v in kt.items()},
        "kernels_per_token": len(kt),
        "kernel_us_graph_replay": ({kk: round(v, 3) for kk, v in kt_graph.items()}
                                   if kt_graph else None),
        # time per token that no kernel of the token covers (graph-replay durations when known)
        "per_token_gap_us": round(ms_step * 1e3 / n - sum((kt_graph or kt).values()), 3),
        **extras,
        "roofline": {"bound": "hbm", "achieved": round(float(achieved), 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(float(achieved) / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": dom,
                     "bytes_per_launch": round(float(gate_bytes), 0),
                     "avg_launch_us": round(dom_us, 3),
                     "duration_source": dur_src},
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
    }
    hs.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
