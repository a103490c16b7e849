#!/usr/bin/env python3
"""Benchmark: chunked fused linear cross-entropy, forward + backward, one MI355X.

One step is one ``flce_fwd_bwd`` call over the whole workload (every chunk:
forward tile GEMM + log-sum-exp epilogue, combine, in-place dlogits, dX GEMM,
dW GEMM, final loss, and the call's stream synchronisation), with inputs
already resident in HBM.  The default workload is the Llama-3-8B LM head
(N = 8192 tokens = 8 x 1024, H = 4096, V = 128256, bf16 inputs, fp32
accumulation and fp32 dW, 5% of labels ignored, chunks of 1024 tokens).

FLOPs are counted as 6 N H V per step (three GEMMs of 2 N H V each).

Printed: one JSON line on stdout.  ``roofline`` describes the kernel class
with the largest total time, from HIP events recorded around each launch on
the launch stream during the timed steps.  Its ``traffic`` is the HBM bytes
per launch of that kernel measured by rocprofv3 counters (FETCH_SIZE and
WRITE_SIZE, each scaled by what the counter reads for a plain copy of known
size), taken from the summary under profiles/ for this workload; it is null
when no summary covers the kernel or the kernel source has changed since the
counters were taken (the summary records the source's SHA-256).
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

METRIC = "FLCE fwd+bwd tokens/s and TFLOP/s (% bf16 MFMA peak), Llama-3-8B head"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(name, chunks, H, V):
    """Algorithmic work of one kernel class summed over a step's launches.

    Returns (bound, amount, unit): flops for the GEMM tiles whose roofline is
    MFMA, bytes for the rest (each array read or written once)."""
    if name in ("fwd_tile", "dx_gemm"):
        return "mfma", sum(2.0 * c * H * V for c in chunks), "flop"
    if name == "dw_gemm":
        # 2 c H V flops against the fp32 dW read-modify-write (a store only on
        # the first chunk) plus G and X: below the MFMA ridge, so bytes bound it
        b = sum((4.0 if i == 0 else 8.0) * V * H + 2.0 * c * V + 2.0 * c * H
                for i, c in enumerate(chunks))
        return "hbm", b, "byte"
    if name == "dlogits":                      # bf16 logits read, G written in place
        return "hbm", sum(4.0 * c * V for c in chunks), "byte"
    if name == "pack_x":                       # bf16 X chunk read, written packed and packed transposed
        return "hbm", sum(6.0 * c * H for c in chunks), "byte"
    if name == "pair_rows":                    # X rows gathered, dX rows scattered (bf16)
        return "hbm", sum(8.0 * c * H for c in chunks), "byte"
    return "hbm", None, "byte"


def counter_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from profiles/traffic_<workload>.txt,
    or None if absent or if the kernel source changed since it was measured."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = os.path.join(ROOT, fields.get("source", ""))
    if not os.path.isfile(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != fields.get("source_sha256"):
            return None
    v = fields.get(f"{kernel}.traffic_bytes_per_launch")
    return float(v) if v else None


def host_info():
    """Threads the host BLAS uses, the process's CPU affinity count and the
    BLAS library, for the oracle baselines."""
    info = {"cores": os.cpu_count() or 1, "affinity_cores": None, "blas": None}
    try:
        info["affinity_cores"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):    # pragma: no cover - informational only
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["cores"] = max(int(i.get("num_threads", 1)) for i in blas)
            info["blas"] = blas[0].get("internal_api")
    except Exception:       # pragma: no cover - informational only
        pass
    return info


def cpu_baseline(inp, n_tok):
    import oracle
    X = inp.X_f64()[:n_tok]
    W = inp.W_f64()
    y = inp.labels[:n_tok]
    t0 = time.perf_counter()
    oracle.flce(X, W, y)
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "kind": "oracle", **host_info(),
            "seconds": round(dt, 3),
            "sample": f"first {n_tok} tokens of the {inp.wl.name} workload (H={inp.wl.H}, "
                      f"V={inp.wl.V}), fp64 loss + dX + dW on the host"}


KERNELS_FROM = "an untimed pass of the same steps, events around every launch"
ROOFLINE_FROM = "the timed steps, events around the dominant kernel's launches only"
CE_N, CE_V = 8192, 128256     # the Llama-3-8B head's logits: 8 x 1024 tokens x vocabulary


def kernel_summary(prof, steps, chunks, H, V, workload):
    """Per-kernel-class times of the timed steps and the roofline of the
    class with the largest share of the step."""
    kernels = {}
    for name, (tot, n) in prof.items():
        if n == 0:
            continue
        steps_n = n / steps
        avg = tot / n
        bound, amount, unit = kernel_work(name, chunks, H, V)
        k = {"avg_ms": round(avg, 5), "launches_per_step": steps_n,
             "ms_per_step": round(tot / steps, 4)}
        if amount is not None:
            per_launch = amount / steps_n
            if unit == "flop":
                k["tflops"] = round(per_launch / (avg * 1e-3) / 1e12, 2)
            else:
                k["gbps"] = round(per_launch / (avg * 1e-3) / 1e9, 1)
        kernels[name] = k
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    return kernels, roofline(dom, prof[dom], steps, chunks, H, V, workload)


def roofline(dom, tot_n, steps, chunks, H, V, workload):
    """The roofline line of kernel class `dom` from its summed event time and
    launch count (tot_n) over `steps` steps."""
    tot, n = tot_n
    avg = tot / n
    bound, amount, unit = kernel_work(dom, chunks, H, V)
    per_launch = amount / (n / steps) if amount is not None else None
    if per_launch is not None and unit == "flop":
        ach = round(per_launch / (avg * 1e-3) / 1e12, 2)
        return {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": counter_traffic(dom, workload), "avg_ms": round(avg, 5)}
    ach = round(per_launch / (avg * 1e-3) / 1e9, 1) if per_launch is not None else None
    return {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4) if ach else None,
            "traffic": counter_traffic(dom, workload), "avg_ms": round(avg, 5)}


def timed_steps(step, steps, chunks, H, V, workload):
    """Per-kernel times from an untimed pass of `steps` steps with events
    around every launch, then `steps` timed steps with events around the
    dominant kernel class's launches only (its live duration for the
    roofline; about 50 event pairs per step would cost the stream a
    fraction of a millisecond).  Each step ends in the call's own
    synchronisation (the loss comes back to the host), so the host clock
    also times every step on its own.  Returns (ms per timed step, the
    median step in ms, the kernels table, the roofline, the last step's
    result)."""
    import torch
    import linear_cross_entropy_04_amd as fl
    fl.flce_profile_select(None)
    fl.flce_profile_enable(True)
    fl.flce_profile_read()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kernels, _ = kernel_summary(fl.flce_profile_read(), steps, chunks, H, V, workload)
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    fl.flce_profile_select([dom])
    fl.flce_profile_read()
    torch.cuda.synchronize()
    each = []
    t0 = time.perf_counter()
    for _ in range(steps):
        t1 = time.perf_counter()
        res = step()
        each.append(time.perf_counter() - t1)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    prof = fl.flce_profile_read()
    fl.flce_profile_enable(False)
    fl.flce_profile_select(None)
    median = 1e3 * sorted(each)[len(each) // 2]
    return ms, median, kernels, roofline(dom, prof[dom], steps, chunks, H, V, workload), res


def copy_reference(mib, dev):
    """One plain device copy of `mib` MiB: a transfer of known size that the
    hardware byte counters of the same run can be scaled by."""
    import torch
    src = torch.empty(mib << 18, dtype=torch.float32, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def bench_ce(args):
    """Cross-entropy on given bf16 logits [8192, 128256], in place: one step
    is one flce_ce_fwd_bwd (label pass, row kernel, final loss, sync).  The
    call overwrites the logits with their gradient, so after the first step
    the rows hold gradient values; the work per step does not depend on
    them.  Roofline: HBM, 3 N V 2 bytes (the row read twice, written once)."""
    import numpy as np
    import torch
    import datagen
    import linear_cross_entropy_04_amd as fl
    import oracle

    dev = torch.device("cuda:0")
    t0 = time.time()
    Zraw, y_np = datagen.make_logits(CE_N, CE_V, "bf16", seed=20270)
    log(f"logits {CE_N} x {CE_V} bf16 drawn in {time.time() - t0:.1f}s")
    L = torch.from_numpy(Zraw.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.from_numpy(y_np).to(dev)
    ws = torch.empty(fl.flce_ce_workspace_bytes(CE_N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_reference_mib:
        copy_reference(args.copy_reference_mib, dev)
    loss0 = fl.flce_ce_fwd_bwd(L, y, -100, ws, stream=stream)      # on the drawn logits
    for _ in range(max(args.warmup - 1, 0)):
        fl.flce_ce_fwd_bwd(L, y, -100, ws, stream=stream)
    torch.cuda.synchronize()
    fl.flce_profile_select(["ce_rows"])        # events around the row kernel only
    fl.flce_profile_enable(True)
    fl.flce_profile_read()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        fl.flce_ce_fwd_bwd(L, y, -100, ws, stream=stream)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t1) / args.steps
    prof = fl.flce_profile_read()
    fl.flce_profile_enable(False)
    fl.flce_profile_select(None)
    tot, n = prof["ce_rows"]
    k_ms = tot / n
    traffic = 3.0 * CE_N * CE_V * 2
    gbps = traffic / (k_ms * 1e-3) / 1e9
    out = {
        "metric": "cross-entropy on given logits fwd+bwd tokens/s, Llama-3-8B head logits",
        "value": round(CE_N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; logits ~ N(0, 1.28^2), uniform labels, 5% ignored)",
        "config": {"workload": "llama3-8b-head-logits", "N": CE_N, "V": CE_V},
        "loss": loss0,
        "kernels": {"ce_rows": {"avg_ms": round(k_ms, 5), "gbps": round(gbps, 1)}},
        "roofline": {"kernel": "ce_rows", "bound": "hbm", "achieved": round(gbps, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBS, 4),
                     "traffic": counter_traffic("ce_rows", "llama3-8b-head-logits")},
    }
    if not args.no_cpu_baseline:
        n_tok = 1024
        Z64 = datagen.bf16_bits_to_f32(Zraw[:n_tok]).astype(np.float64)
        t2 = time.perf_counter()
        oracle.cross_entropy(Z64, y_np[:n_tok])
        dt = time.perf_counter() - t2
        out["cpu_baseline"] = {"value": n_tok / dt, "unit": "tokens/s",
                               "kind": "oracle", **host_info(),
                               "seconds": round(dt, 3),
                               "sample": f"first {n_tok} rows of the logits, fp64 loss + gradient"}
    else:
        out["cpu_baseline"] = None
    log(f"ce: {ms:.3f} ms/step, kernel {k_ms:.3f} ms at {gbps:.0f} GB/s, loss={loss0:.6f}")
    print(json.dumps(out), flush=True)


ORPO_PAIRS, ORPO_T = 8, 512   # 8 pairs of 512-token sequences: 8192 rows on the Llama-3-8B head


PAIR_PARAMS = {"orpo": dict(beta=0.1, gamma=0.0, alpha=1.0),
               "simpo": dict(beta=2.0, gamma=1.0, alpha=0.0),
               "cpo": dict(beta=0.1, gamma=0.0, alpha=1.0),
               "dpo": dict(beta=0.1, gamma=0.0, alpha=0.0)}


def bench_orpo(args):
    """A pairwise preference loss (--op orpo, simpo, cpo or dpo) on the
    Llama-3-8B head: 8 preference pairs of 512-token sequences (8192 rows,
    H = 4096, V = 128256, bf16), one pair (1024 rows) per chunk; one step is
    one flce_pair_fwd_bwd (DPO with fixed reference log-probabilities).
    FLOPs 6 N H V as for the fused loss (the same three GEMMs over every
    row)."""
    import numpy as np
    import torch
    import datagen
    import linear_cross_entropy_04_amd as fl

    dev = torch.device("cuda:0")
    B, T, H, V = ORPO_PAIRS, ORPO_T, 4096, 128256
    chunk_pairs = 1
    t0 = time.time()
    inp = datagen.make_pairs(B, T, H, V, "bf16", seed=20280)
    log(f"preference batch {B} pairs x {T} tokens drawn in {time.time() - t0:.1f}s")
    N = 2 * B * T
    X = torch.from_numpy(inp.X.view(np.int16)).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(inp.W.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.from_numpy(inp.labels).to(dev)
    dX = torch.empty_like(X)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    nbytes = fl.flce_orpo_workspace_bytes(B, T, H, V, fl.FLCE_BF16, chunk_pairs)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_reference_mib:
        copy_reference(args.copy_reference_mib, dev)

    kind = args.op
    pp = PAIR_PARAMS[kind]
    ref = [None, None]
    if kind == "dpo":     # a reference head's sequence log-probabilities (not timed)
        Wref = (W.float() * 1.01).to(torch.bfloat16)
        ref = list(fl.sequence_logps(Wref, X, y.view(2 * B, T), chunk_pairs=chunk_pairs))

    def step():
        return fl.flce_pair_fwd_bwd(kind, X, W, y, B, -100, pp["beta"], pp["gamma"], pp["alpha"],
                                    chunk_pairs, dX, dW, ws, ref[0], ref[1], stream=stream)

    for _ in range(args.warmup):
        loss, nll = step()
    torch.cuda.synchronize()
    chunks = [2 * chunk_pairs * T] * (B // chunk_pairs)
    ms, med, kernels, roof, (loss, nll) = timed_steps(step, args.steps, chunks, H, V,
                                                      f"llama3-8b-head-{kind}")
    tflops = 6.0 * N * H * V / (ms * 1e-3) / 1e12
    out = {
        "metric": f"{kind.upper()} fused-linear preference loss fwd+bwd tokens/s, Llama-3-8B head",
        "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(med, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; X ~ N(0,1), W ~ N(0,0.02^2); per pair a shared prompt of "
                "T/8..T/2 unscored tokens, per sequence 0..T/4 unscored padding tokens, "
                "uniform response labels)",
        "config": {"workload": f"llama3-8b-head-{kind}", "pairs": B, "T": T, "N": N, "H": H,
                   "V": V, "chunk_pairs": chunk_pairs, **pp, "workspace_bytes": nbytes},
        "tflops": round(tflops, 2), "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "loss": loss, "nll": nll, "kernels": kernels, "kernels_from": KERNELS_FROM,
        "roofline": roof, "roofline_from": ROOFLINE_FROM,
    }
    if not args.no_cpu_baseline:
        import oracle
        n_pairs = 4                                  # the first four pairs: 4096 rows
        rows = np.concatenate([np.arange(0, n_pairs * T), np.arange(B * T, (B + n_pairs) * T)])
        X64, W64 = inp.X_f64()[rows], inp.W_f64()
        rr = None
        if kind == "dpo":
            rr = [r.double().cpu().numpy()[:n_pairs] for r in ref]
        t2 = time.perf_counter()
        oracle.preference(kind, X64, W64, inp.labels[rows], n_pairs, -100,
                          ref_chosen=rr[0] if rr else None, ref_rejected=rr[1] if rr else None,
                          **pp)
        dt = time.perf_counter() - t2
        out["cpu_baseline"] = {"value": rows.size / dt, "unit": "tokens/s",
                               "kind": "oracle", **host_info(),
                               "seconds": round(dt, 3),
                               "sample": f"the first {n_pairs} pairs ({rows.size} rows), fp64 "
                                         "loss + dX + dW on the host"}
    else:
        out["cpu_baseline"] = None
    log(f"{kind}: {ms:.3f} ms/step  {tflops:.1f} TFLOP/s  loss={loss:.6f} nll={nll:.6f}")
    for name, k in kernels.items():
        log(f"  {name:12s} {k}")
    print(json.dumps(out), flush=True)


KTO_SEQS, KTO_T = 16, 512     # 16 unpaired 512-token sequences: 8192 rows on the Llama-3-8B head


def bench_kto(args):
    """KTO on the Llama-3-8B head: 16 unpaired sequences of 512 tokens (8192
    rows, H = 4096, V = 128256, bf16), two sequences (1024 rows) per chunk,
    fixed reference log-probabilities; one step is one flce_kto_fwd_bwd.
    FLOPs 6 N H V."""
    import numpy as np
    import torch
    import datagen
    import linear_cross_entropy_04_amd as fl

    dev = torch.device("cuda:0")
    S, T, H, V = KTO_SEQS, KTO_T, 4096, 128256
    chunk_seqs = 2
    pp = dict(beta=0.1, z0=0.0, lambda_d=1.0, lambda_u=1.0)
    t0 = time.time()
    inp, des_np, R_np = datagen.make_unpaired(S, T, H, V, "bf16", seed=20290)
    log(f"unpaired batch {S} x {T} tokens drawn in {time.time() - t0:.1f}s")
    N = S * T
    X = torch.from_numpy(inp.X.view(np.int16)).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(inp.W.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.from_numpy(inp.labels).to(dev)
    des = torch.from_numpy(des_np).to(dev)
    R = torch.from_numpy(R_np).to(dev)
    dX = torch.empty_like(X)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    nbytes = fl.flce_kto_workspace_bytes(S, T, H, V, fl.FLCE_BF16, chunk_seqs)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_reference_mib:
        copy_reference(args.copy_reference_mib, dev)

    def step():
        return fl.flce_kto_fwd_bwd(X, W, y, S, -100, des, R, pp["beta"], pp["z0"],
                                   pp["lambda_d"], pp["lambda_u"], chunk_seqs, dX, dW, ws,
                                   stream=stream)

    for _ in range(args.warmup):
        loss = step()
    torch.cuda.synchronize()
    chunks = [chunk_seqs * T] * (S // chunk_seqs)
    ms, med, kernels, roof, loss = timed_steps(step, args.steps, chunks, H, V, "llama3-8b-head-kto")
    tflops = 6.0 * N * H * V / (ms * 1e-3) / 1e12
    out = {
        "metric": "KTO fused-linear preference loss fwd+bwd tokens/s, Llama-3-8B head",
        "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(med, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; X ~ N(0,1), W ~ N(0,0.02^2); per sequence T/8..T/2 prompt "
                "and 0..T/4 padding tokens unscored, uniform response labels, half desirable, "
                "reference sums around the head's expected log-probability)",
        "config": {"workload": "llama3-8b-head-kto", "sequences": S, "T": T, "N": N, "H": H,
                   "V": V, "chunk_seqs": chunk_seqs, **pp, "workspace_bytes": nbytes},
        "tflops": round(tflops, 2), "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "loss": loss, "kernels": kernels, "kernels_from": KERNELS_FROM,
        "roofline": roof, "roofline_from": ROOFLINE_FROM,
    }
    if not args.no_cpu_baseline:
        import oracle
        n_s = 8                                      # the first 8 sequences: 4096 rows
        rows = np.arange(n_s * T)
        t2 = time.perf_counter()
        oracle.kto(inp.X_f64()[rows], inp.W_f64(), inp.labels[rows], n_s,
                   des_np[:n_s].astype(bool), R_np[:n_s].astype(np.float64), -100, **pp)
        dt = time.perf_counter() - t2
        out["cpu_baseline"] = {"value": rows.size / dt, "unit": "tokens/s",
                               "kind": "oracle", **host_info(),
                               "seconds": round(dt, 3),
                               "sample": f"the first {n_s} sequences ({rows.size} rows), fp64 "
                                         "loss + dX + dW on the host"}
    else:
        out["cpu_baseline"] = None
    log(f"kto: {ms:.3f} ms/step  {tflops:.1f} TFLOP/s  loss={loss:.6f}")
    for name, k in kernels.items():
        log(f"  {name:12s} {k}")
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=1, help="workload id (datagen.WORKLOADS)")
    ap.add_argument("--chunk", type=int, default=None, help="chunk tokens (default: the workload's)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", choices=("flce", "ce", "orpo", "simpo", "cpo", "dpo", "kto"),
                    default="flce",
                    help="flce: the fused linear cross-entropy step (default); ce: cross-entropy "
                         "on given logits of the Llama-3-8B head's size; orpo, simpo, cpo, dpo: "
                         "a fused-linear preference loss on 8 pairs of 512-token sequences on "
                         "the same head; kto: the unpaired one on 16 such sequences")
    ap.add_argument("--share", choices=("dp8", "tp8"), default=None,
                    help="measure one GPU's share of the workload sharded over 8 GPUs: dp8 = "
                         "its N/8 tokens with the whole head, tp8 = all tokens against its V/8 "
                         "vocabulary rows (labels reduced modulo V/8, so the call is a valid "
                         "loss on the shard; the work is the shard's)")
    ap.add_argument("--no-fwd-only", action="store_true",
                    help="skip timing the forward-only call (keeps profiler traces to the "
                         "fwd+bwd steps)")
    ap.add_argument("--copy-reference-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the multi-GPU "
              "sharding of this path is a design only)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("bench.py needs --steps >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    if args.op == "ce":
        bench_ce(args)
        return
    if args.op in PAIR_PARAMS:
        bench_orpo(args)
        return
    if args.op == "kto":
        bench_kto(args)
        return

    import numpy as np
    import torch
    import datagen
    import linear_cross_entropy_04_amd as fl

    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = datagen.make(args.workload)
    if args.share:
        inp = datagen.share_of(inp, args.share)
    wl = inp.wl
    log(f"workload {wl.name}: N={wl.N} H={wl.H} V={wl.V} drawn in {time.time() - t0:.1f}s")
    N, H, V = wl.N, wl.H, wl.V
    chunk = wl.chunk_tokens if args.chunk is None else args.chunk
    dt = fl.FLCE_BF16 if wl.dtype == "bf16" else fl.FLCE_F32
    st, C, peak_scratch = fl.flce_plan(N, H, V, dt, chunk_tokens=chunk)
    if st != fl.FLCE_OK:
        raise fl.FLCEError(st, "flce_plan")

    if wl.dtype == "bf16":
        X = torch.from_numpy(inp.X.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(inp.W.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        X = torch.from_numpy(inp.X).to(dev)
        W = torch.from_numpy(inp.W).to(dev)
    y = torch.from_numpy(inp.labels).to(dev)
    dX = torch.empty_like(X)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    ws = fl.workspace(N, H, V, dt, chunk, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_reference_mib:
        copy_reference(args.copy_reference_mib, dev)

    def step():
        return fl.flce_fwd_bwd(X, W, y, -100, chunk, dX, dW, ws, stream=stream)

    for _ in range(args.warmup):
        loss = step()
    torch.cuda.synchronize()
    chunks = [min(C, N - c0) for c0 in range(0, N, C)]
    ms, med, kernels, roof, loss = timed_steps(step, args.steps, chunks, H, V, wl.name)

    # the same steps without events, to show what the event records cost
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed_noev = time.perf_counter() - t1

    # the forward-only call (loss, no gradients) on the same workload
    fwd_ms = None
    if not args.no_fwd_only:
        for _ in range(2):
            fl.flce_fwd(X, W, y, -100, chunk, ws, stream=stream)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            fl.flce_fwd(X, W, y, -100, chunk, ws, stream=stream)
        torch.cuda.synchronize()
        fwd_ms = 1e3 * (time.perf_counter() - t2) / args.steps

    flops = 6.0 * N * H * V
    tflops = flops / (ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(N / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(med, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; X ~ N(0,1), W ~ N(0,0.02^2), uniform labels, 5% ignored)",
        "config": {"workload": wl.name, "N": N, "H": H, "V": V, "chunk_tokens": C,
                   "share_of_8_gpus": args.share,
                   "ignored_tokens": int((inp.labels == -100).sum()),
                   "peak_scratch_bytes": peak_scratch,
                   "nxv_logits_bytes": N * V * (2 if wl.dtype == "bf16" else 4)},
        "tflops": round(tflops, 2),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "ms_per_step_without_events": round(1e3 * elapsed_noev / args.steps, 4),
        "fwd_only_ms_per_step": round(fwd_ms, 4) if fwd_ms is not None else None,
        "loss": loss,
        "kernels": kernels,
        "kernels_from": KERNELS_FROM,
        "roofline": roof,
        "roofline_from": ROOFLINE_FROM,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_sample_tokens} tokens ...")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens)
    else:
        out["cpu_baseline"] = None
    log(f"{ms:.3f} ms/step  {tflops:.1f} TFLOP/s  ({out['pct_bf16_peak']:.1f}% of bf16 peak)  "
        f"loss={loss:.6f}")
    for name, k in kernels.items():
        log(f"  {name:12s} {k}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
