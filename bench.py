#!/usr/bin/env python3
"""Attention-forward benchmark on one MI355X.

One step = one call of the library's forward on one batch of synthetic input
(all steps of the hot path run inside that call). The headline workload is
causal bf16 attention, B=2, H=16, S=4096, D=128; ``value`` is its whole-job
throughput in TFLOP/s with inputs resident in HBM, over exactly --steps
timed calls after --warmup untimed ones.

FLOP convention: 4 * D per (query, key) pair the row attends to (Q.K^T and
P.V, 2 flops per multiply-add each); a causal head of length S has
S(S+1)/2 pairs. Top-k sparse MLA counts 2 * (Dqk + Dv) flops per pair and
reports GB/s of algorithmic bytes (every gathered 1152-byte key row counted
each time it is gathered, plus Q, O, indices and LSE once).

Printed: ONE JSON line on stdout (progress goes to stderr), carrying
``roofline`` for the timed kernel (its own average launch time from HIP
events on the launch stream vs. the dense bf16 MFMA peak) and
``cpu_baseline`` (the fp64 CPU oracle timed on a bounded sample of the same
workload on this host's cores).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def causal_pairs(Sq, Skv):
    i = np.arange(Sq, dtype=np.int64)
    return int(np.clip(i + (Skv - Sq) + 1, 0, Skv).sum())


def dense_flops(w):
    B, Hq, Sq, D = w["q"].shape
    Skv = w["k"].shape[2]
    pairs = causal_pairs(Sq, Skv) if w["causal"] else Sq * Skv
    return 4.0 * D * pairs * B * Hq


def blocksparse_flops(w):
    B, Hq, Sq, D = w["q"].shape
    lists = w["block_idx"].numpy()
    seq = w["seqlens"].numpy()
    blk = w["block"]
    pairs = 0
    for b in range(B):
        L = int(seq[b])
        for qb in range(lists.shape[0]):
            rows = max(0, min(L, (qb + 1) * blk) - qb * blk)
            keys = sum(max(0, min(L, (x + 1) * blk) - x * blk) for x in lists[qb] if x >= 0)
            pairs += rows * keys
    return 4.0 * D * pairs * Hq


def topk_work(w, idx):
    T, Hq, Dqk = w["q"].shape
    Dv = w["dv"]
    valid = int((idx >= 0).sum())
    flops = 2.0 * (Dqk + Dv) * valid * Hq
    es = w["q"].element_size()
    nbytes = valid * Dqk * es + T * Hq * Dqk * es + T * Hq * Dv * es + idx.numel() * 4 + T * Hq * 4
    return flops, nbytes


def make_call(w, order="idx_a", rescale_threshold=0.0):
    """Uploads a workload and returns a zero-argument launcher of one forward
    (dense and block-sparse with the given running-max rescale threshold;
    0 = the exact running max)."""
    import flashattention_online_softmax_amd as fa
    dev = "cuda"
    if w["kind"] == "dense" and w.get("split"):
        q, k, v = (w[n].to(dev) for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        B, Hq, Sq, D = q.shape
        n = fa.load().fa_fwd_splitkv_workspace_elems(B, Hq, Sq, k.shape[2], D, 0)
        ws = torch.empty(max(n, 1), dtype=torch.float32, device=dev)
        return lambda: fa.fa_fwd_splitkv(q, k, v, scale=w["scale"], causal=w["causal"], workspace=ws, out=o, lse=lse,
                                         rescale_threshold=rescale_threshold)
    if w["kind"] == "dense":
        q, k, v = (w[n].to(dev) for n in ("q", "k", "v"))
        mask = w["mask"].to(dev) if w.get("mask") is not None else None
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        return lambda: fa.fa_fwd(q, k, v, scale=w["scale"], causal=w["causal"], mask=mask, out=o, lse=lse,
                                 rescale_threshold=rescale_threshold)
    if w["kind"] == "varlen":
        q, k, v, cq, ck = (w[n].to(dev) for n in ("q", "k", "v", "cu_q", "cu_k"))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        return lambda: fa.fa_fwd_varlen(q, k, v, cq, ck, w["max_q"], scale=w["scale"], causal=w["causal"], out=o,
                                        lse=lse, rescale_threshold=rescale_threshold)
    if w["kind"] == "blocksparse":
        q, k, v = (w[n].to(dev) for n in ("q", "k", "v"))
        bi, seq = w["block_idx"].to(dev), w["seqlens"].to(dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        return lambda: fa.fa_fwd_blocksparse(q, k, v, bi, scale=w["scale"], seqlens=seq, out=o, lse=lse,
                                             rescale_threshold=rescale_threshold)
    q, kv, idx = w["q"].to(dev), w["kv"].to(dev), w[order].to(dev)
    vv = kv[:, :w["dv"]]
    o = torch.empty((q.shape[0], q.shape[1], w["dv"]), dtype=q.dtype, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    return lambda: fa.fa_fwd_topk_gather(q, kv, vv, idx, scale=w["scale"], out=o, lse=lse)


def varlen_flops(w):
    Hq, D = w["q"].shape[1], w["q"].shape[2]
    lq, lk = np.diff(w["cu_q"].numpy()), np.diff(w["cu_k"].numpy())
    pairs = sum(causal_pairs(int(a), int(b)) if w["causal"] else int(a) * int(b) for a, b in zip(lq, lk))
    return 4.0 * D * pairs * Hq


def workload_flops(w):
    if w["kind"] == "dense":
        return dense_flops(w)
    if w["kind"] == "varlen":
        return varlen_flops(w)
    if w["kind"] == "blocksparse":
        return blocksparse_flops(w)
    return topk_work(w, w["idx_a"])[0]


def make_bwd_call(w, path="auto"):
    """Launcher of one backward (fa_bwd) of a dense workload: dO seeded and
    synthetic, O and LSE from one forward with the exact running max. path:
    "ds" (dQ from the stored dS, its workspace allocated once here), "rc" (dQ
    recomputing S and dP) or "auto" (the binding's choice for these sizes).
    Returns (launcher, the path taken)."""
    import flashattention_online_softmax_amd as fa
    import synth
    q, k, v = (w[n].to("cuda") for n in ("q", "k", "v"))
    dout = synth.cast(synth.normal(synth.rng(1080), tuple(q.shape)), q.dtype).to("cuda")
    o, lse = fa.fa_fwd(q, k, v, scale=w["scale"], causal=w["causal"], rescale_threshold=0.0)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    B, H, S = q.shape[:3]
    ws = fa._ds_work(q, B, H, k.shape[1], S, k.shape[2], {"auto": "auto", "ds": True, "rc": None}[path], w["causal"])
    call = lambda: fa.fa_bwd(q, k, v, o, lse, dout, scale=w["scale"], causal=w["causal"], dq=dq, dk=dk, dv=dv,
                             delta=delta, ds_workspace=ws)
    return call, ("ds" if ws is not None else "rc")


def time_calls(call, steps, warmup, warm_seconds=1.0):
    """Returns (wall ms per step over exactly `steps` calls bracketed by device
    synchronisations, mean kernel ms from per-launch HIP events on the launch
    stream). The untimed warm-up is `warmup` calls, continued until the GPU has
    run for `warm_seconds` (its clock ramps up under load for a while)."""
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < warm_seconds:
        call()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    kern = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    return wall, kern


# The sources of the forward kernels' code object (the kernels the traffic
# records cover): a change to any of them voids the records.
FORWARD_SOURCES = ("fa_fwd16.hip", "fa_topk16.hip", "fa_asm.h", "fa_copy.h", "fa_device.h", "fa_internal.h",
                   "fa_tiles.h")


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "flashattention_online_softmax_amd", "csrc")
    for f in FORWARD_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "flashattention_online_softmax_amd", "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, launches_per_step=1):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_digest") != source_digest():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, target_s, threads, seed=99):
    """The fp64 oracle on a bounded random sample of query rows of a dense
    workload; returns TFLOP/s (algorithmic flops of the sampled rows / time)."""
    import oracle
    B, Hq, Sq, D = w["q"].shape
    Skv = w["k"].shape[2]
    g = np.random.default_rng(seed)
    kk = w["k"].to(torch.float64).numpy()
    vv = w["v"].to(torch.float64).numpy()

    def run(rows):
        t0 = time.perf_counter()
        oracle.attn_dense(w["q"], kk, vv, scale=float(np.float32(w["scale"])), causal=w["causal"],
                          mask=w.get("mask"), rows=rows, nthreads=threads)
        return time.perf_counter() - t0

    def flops(rows):
        i = rows % Sq
        # masked keys of a boolean mask are counted too (the method computes them)
        keys = np.clip(i + (Skv - Sq) + 1, 0, Skv) if w["causal"] else np.full(rows.shape, Skv)
        return 4.0 * D * float(keys.sum())

    probe = np.sort(g.choice(B * Hq * Sq, size=min(B * Hq * Sq, 64 * threads), replace=False))
    t = run(probe)
    # All rows when the whole workload fits in the time budget, else a sample.
    n = int(min(B * Hq * Sq, max(len(probe), len(probe) * target_s / max(t, 1e-3))))
    rows = np.sort(g.choice(B * Hq * Sq, size=n, replace=False))
    t = run(rows)
    return {"value": flops(rows) / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d random query rows of %d (%.1f s, fp64, %d threads)" % (n, B * Hq * Sq, t, threads),
            "seconds": t}


def cpu_oracle_topk(w, target_s, threads):
    """The fp64 oracle on a bounded sample of tokens of the top-k workload
    (all heads of each sampled token); GB/s of algorithmic bytes and TFLOP/s."""
    import oracle
    T, Hq, Dqk = w["q"].shape
    g = np.random.default_rng(98)
    kv64 = w["kv"].to(torch.float64).numpy()
    v64 = np.ascontiguousarray(kv64[:, :w["dv"]])
    idx = w["idx_a"]

    def run(toks):
        rows = (toks[:, None] * Hq + np.arange(Hq)[None, :]).reshape(-1)
        t0 = time.perf_counter()
        oracle.attn_topk(w["q"], kv64, v64, idx, scale=float(np.float32(w["scale"])), rows=rows, nthreads=threads)
        return time.perf_counter() - t0

    probe = np.sort(g.choice(T, size=min(T, 4), replace=False))
    t = run(probe)
    n = int(min(T, max(len(probe), len(probe) * target_s / max(t, 1e-3))))
    toks = np.sort(g.choice(T, size=n, replace=False))
    t = run(toks)
    sub = idx[torch.from_numpy(toks)]
    valid = int((sub >= 0).sum())
    es = w["q"].element_size()
    nbytes = valid * Dqk * es + n * Hq * (Dqk + w["dv"]) * es + sub.numel() * 4 + n * Hq * 4
    flops = 2.0 * (Dqk + w["dv"]) * valid * Hq
    return {"gbs": nbytes / t / 1e9, "tflops": flops / t / 1e12, "cores": threads,
            "sample": "%d random tokens of %d, all %d heads (%.1f s)" % (n, T, Hq, t)}


def cpu_oracle_blocksparse(w, target_s, threads):
    """The fp64 oracle on a bounded sample of query rows of the block-sparse
    workload; TFLOP/s over the sampled rows' key counts."""
    import oracle
    B, Hq, Sq, D = w["q"].shape
    g = np.random.default_rng(97)
    lists = w["block_idx"].numpy()
    seq = w["seqlens"].numpy()
    blk = w["block"]

    def run(rows):
        t0 = time.perf_counter()
        oracle.attn_blocksparse(w["q"], w["k"], w["v"], w["block_idx"], scale=float(np.float32(w["scale"])),
                                seqlens=w["seqlens"], rows=rows, nthreads=threads)
        return time.perf_counter() - t0

    def flops(rows):
        tot = 0
        for r in rows:
            i, b = int(r % Sq), int(r // (Hq * Sq))
            L = int(seq[b])
            if i >= L:
                continue
            tot += sum(max(0, min(L, (x + 1) * blk) - x * blk) for x in lists[i // blk] if x >= 0)
        return 4.0 * D * tot

    probe = np.sort(g.choice(B * Hq * Sq, size=64 * threads, replace=False))
    t = run(probe)
    n = int(min(B * Hq * Sq, max(len(probe), len(probe) * target_s / max(t, 1e-3))))
    rows = np.sort(g.choice(B * Hq * Sq, size=n, replace=False))
    t = run(rows)
    return {"tflops": flops(rows) / t / 1e12, "cores": threads,
            "sample": "%d random query rows of %d (%.1f s)" % (n, B * Hq * Sq, t)}


def time_secondary(name, w, steps, rescale_threshold=0.0):
    """Kernel time and throughput of one forward workload (secondary figure)."""
    fl = workload_flops(w)
    c = make_call(w, rescale_threshold=rescale_threshold)
    _, km = time_calls(c, steps, 2, 0.3)
    del c
    torch.cuda.empty_cache()
    return {"tflops": round(fl / (km * 1e-3) / 1e12, 2), "kernel_ms": round(km, 4),
            "frac_mfma_peak": round(fl / (km * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "rescale_threshold_log2": rescale_threshold, "traffic": measured_traffic(name)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="causal_bf16_s4096")
    ap.add_argument("--no-secondary", action="store_true", help="skip every secondary figure")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", default=None,
                    help="time only this workload (any kind) for --steps calls and print its figure; "
                         "for profiling one kernel")
    ap.add_argument("--threshold", type=float, default=0.0, help="rescale threshold of --only (log2 units)")
    ap.add_argument("--backward", action="store_true", help="with --only (a dense workload): time the backward")
    ap.add_argument("--recompute", action="store_true",
                    help="with --backward: the dQ path that recomputes S and dP (default: the binding's choice)")
    ap.add_argument("--stored-ds", action="store_true",
                    help="with --backward: the dQ path that reads the dS the dK/dV kernel stores")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the benchmark, run --steps plain device copies of this many "
                         "bytes (the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build runs the forward on a single "
              "MI355X (--gpus 1); multi-GPU runs are not part of it.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        wall, kern = time_calls(lambda: dst.copy_(src), args.steps, args.warmup)
        print(json.dumps({"copy_bytes": args.copy_bytes, "kernel_ms": kern,
                          "gbs_read_plus_write": 2 * args.copy_bytes / (kern * 1e-3) / 1e9}))
        return

    import synth
    import flashattention_online_softmax_amd as fa
    fa.load()  # raises if the HIP library is not built

    if args.only:
        log("only %s (threshold %g%s)" % (args.only, args.threshold, ", backward" if args.backward else ""))
        w = synth.workload(args.only)
        fl = workload_flops(w)
        if args.backward:
            fl *= 2.5  # five products over the pairs against the forward's two
            c, taken = make_bwd_call(w, "rc" if args.recompute else "ds" if args.stored_ds else "auto")
        else:
            c = make_call(w, rescale_threshold=args.threshold)
        wall, km = time_calls(c, args.steps, args.warmup, 0.3)
        tag = "_bwd" if args.backward else ""
        out = {"workload": args.only + tag, "kernel_ms": round(km, 4),
               "tflops": round(fl / (km * 1e-3) / 1e12, 2), "rescale_threshold_log2": args.threshold}
        if w["kind"] == "topk":
            out["gbs"] = round(topk_work(w, w["idx_a"])[1] / (km * 1e-3) / 1e9, 1)
        if args.backward:
            out["dq_path"] = {"ds": "stored dS", "rc": "S and dP recomputed"}[taken]
        print(json.dumps(out), flush=True)
        return

    log("generating %s" % args.workload)
    w = synth.workload(args.workload)
    if w["kind"] != "dense":
        raise SystemExit("headline workload must be a dense one")
    flops = dense_flops(w)
    # The contract path: the exact running max (rescale threshold 0).
    call = make_call(w, rescale_threshold=0.0)
    log("timing %d steps after %d warmup" % (args.steps, args.warmup))
    wall_ms, kern_ms = time_calls(call, args.steps, args.warmup)
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    B, H, S, D = w["q"].shape
    traffic = measured_traffic(args.workload)
    result = {
        "metric": "attention fwd TFLOP/s (bf16, causal, D=128) + % of MFMA peak; GB/s for top-k sparse",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), cast to bf16)",
        "config": {"workload": args.workload, "B": B, "H": H, "S": S, "D": D,
                   "causal": bool(w["causal"]), "flops_per_step": flops,
                   "rescale_threshold_log2": 0.0},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel_ms": round(kern_ms, 4)},
    }
    torch.cuda.synchronize()
    nsec = max(5, args.steps // 2)

    if not args.no_secondary:
        sec = {}
        # The lazy rescale (threshold 8) on the same inputs: this machine's
        # cost of the exact running max.
        log("secondary %s lazy rescale" % args.workload)
        c8 = make_call(w, rescale_threshold=8.0)
        _, km8 = time_calls(c8, nsec, 2, 0.3)
        del c8
        sec[args.workload + "_lazy8"] = {"tflops": round(flops / (km8 * 1e-3) / 1e12, 2), "kernel_ms": round(km8, 4),
                                         "frac_mfma_peak": round(flops / (km8 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                         "exact_max_cost": round(kern_ms / km8 - 1.0, 4)}
        for name in ("causal_bf16_s8192", "gqa_mask_f16_s8192", "blocksparse_f16_s8192", "splitkv_bf16_q512_k65536",
                     "varlen_bf16_b16"):
            log("secondary %s" % name)
            w2 = synth.workload(name)
            sec[name] = time_secondary(name, w2, nsec, 0.0)
            if name == "splitkv_bf16_q512_k65536":
                B2, H2, S2, _ = w2["q"].shape
                sec[name]["key_ranges"] = fa.splitkv_splits(B2, H2, S2, w2["k"].shape[2])
            if name == "causal_bf16_s8192":
                lz = time_secondary(name, w2, nsec, 8.0)
                lz.pop("traffic")
                sec[name + "_lazy8"] = lz
                lz["exact_max_cost"] = round(sec[name]["kernel_ms"] / lz["kernel_ms"] - 1.0, 4)
            del w2
        log("secondary topk_mla_bf16_t4096")
        w5 = synth.workload("topk_mla_bf16_t4096")
        topk_traffic = measured_traffic("topk_mla_bf16_t4096")
        for order in ("idx_a", "idx_b"):
            fl, nb = topk_work(w5, w5[order])
            c5 = make_call(w5, order)
            _, km = time_calls(c5, max(5, args.steps // 10), 2, 0.3)
            sec["topk_mla_bf16_t4096_" + ("self_first" if order == "idx_a" else "self_last")] = {
                "gbs": round(nb / (km * 1e-3) / 1e9, 1), "tflops": round(fl / (km * 1e-3) / 1e12, 2),
                "kernel_ms": round(km, 4), "frac_hbm_peak": round(nb / (km * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "algorithmic_bytes": nb, "traffic": topk_traffic}
            del c5
        torch.cuda.empty_cache()
        # The backward of the headline workload (dQ, dK, dV from dO), counted
        # as five products over the causal pairs: 2.5 times the forward's flop.
        log("secondary %s backward" % args.workload)
        names = {"ds": "stored dS", "rc": "S and dP recomputed"}
        cb, taken = make_bwd_call(w, "auto")
        _, kmb = time_calls(cb, max(5, args.steps // 10), 2, 0.3)
        del cb
        torch.cuda.empty_cache()
        other = "rc" if taken == "ds" else "ds"
        cb, _ = make_bwd_call(w, other)
        _, kmo = time_calls(cb, max(5, args.steps // 10), 2, 0.3)
        del cb
        torch.cuda.empty_cache()
        flb = 2.5 * flops
        for key, km_, pth in (("_bwd", kmb, taken), ("_bwd_other_path", kmo, other)):
            sec[args.workload + key] = {"tflops": round(flb / (km_ * 1e-3) / 1e12, 2), "kernel_ms": round(km_, 4),
                                        "frac_mfma_peak": round(flb / (km_ * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                        "dq_path": names[pth]}
        result["secondary"] = sec
        result["page_figures"] = {
            "exact_max_fwd_cost_gb200": "+~4% (sparse-MLA training forward, T=S=16384, W=2048, H=128; NVIDIA GB200)",
            "bf16_output_floor_rel_l2": "1.66e-3 at T=S=4096, W=2048, H=128 (numerical, fp64 reference)"}

    del call
    if not args.no_cpu_baseline:
        # The machine's CPU share for one GPU is 16 threads; more would oversubscribe it.
        threads = min(16, os.cpu_count() or 1)
        log("cpu baseline (oracle, %d threads, ~%.0f s)" % (threads, args.cpu_seconds))
        cb = cpu_baseline(w, args.cpu_seconds, threads)
        cb.pop("seconds")
        cb["value"] = round(cb["value"], 6)
        cb["cpu_model"] = cpu_model()
        cb["threads_note"] = "capped at 16, the host CPU share of one GPU (os.cpu_count() = %d)" % (os.cpu_count() or 0)
        if not args.no_secondary:
            # The oracle per configuration, each on a bounded sample (~3 s).
            per = {}
            for name in ("dense_f32_s128", "causal_bf16_s8192", "gqa_mask_f16_s8192"):
                log("cpu oracle %s" % name)
                w2 = synth.workload(name)
                r = cpu_baseline(w2, 3.0, threads, seed=96)
                per[name] = {"tflops": round(r["value"], 6), "sample": r["sample"]}
                del w2
            log("cpu oracle blocksparse_f16_s8192")
            r = cpu_oracle_blocksparse(synth.workload("blocksparse_f16_s8192"), 3.0, threads)
            per["blocksparse_f16_s8192"] = {"tflops": round(r["tflops"], 6), "sample": r["sample"]}
            log("cpu oracle topk_mla_bf16_t4096")
            r = cpu_oracle_topk(synth.workload("topk_mla_bf16_t4096"), 3.0, threads)
            per["topk_mla_bf16_t4096"] = {"gbs": round(r["gbs"], 3), "tflops": round(r["tflops"], 6),
                                          "sample": r["sample"]}
            cb["per_config"] = per
        result["cpu_baseline"] = cb

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
