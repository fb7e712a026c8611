#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

A step is one spec_verify_sample (or spec_verify_greedy) call over one batch
of synthetic logits resident in HBM: the whole hot path (streaming pass,
per-row select or merge, accept / residual / extra-token draw, outputs).
The timed loop rotates over enough copies of the inputs (>= 512 MB by
default) that they cannot stay in the 256 MB last-level cache, so it
measures HBM reads.

Prints one JSON line:
  value         verified positions per second (sum_b (K_b + 1) per step);
                with --mode draft, draft tokens sampled per second (sum_b K_b)
  roofline      the streaming kernel: algorithmic bytes per launch (every
                logit once) / its average duration from HIP events recorded
                around each launch in a profiled pass of the same loop,
                against the 8 TB/s HBM peak
  cpu_baseline  the fp64 CPU oracle on the same workload, on this host
"""
import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "verified positions/sec + achieved HBM GB/s (% of peak), B×(K+1)×V logits"
METRIC_DRAFT = "draft tokens sampled/sec + achieved HBM GB/s (% of peak), B×K×V draft logits"
METRIC_LIK = "positions scored/sec (speculative likelihood: both parts, beta, NLL) + achieved HBM GB/s, 2×B×K×V logits"
STREAM_KERNEL = {"sample_topk": "topk_cand_kernel", "sample": "row_stats_kernel", "greedy": "row_stats_kernel",
                 "draft_topk": "topk_cand_kernel", "draft": "row_stats_kernel",
                 "argmax_topk": "topk_cand_kernel", "argmax": "row_stats_kernel",
                 "likelihood_topk": "topk_cand_kernel", "likelihood": "row_stats_kernel",
                 # full rows with top-p: statistics and cut in one kernel per row
                 "sample_topp": "nucleus_row_kernel", "draft_topp": "nucleus_row_kernel",
                 "argmax_topp": "nucleus_row_kernel", "likelihood_topp": "nucleus_row_kernel"}


def stream_kind(mode: str, top_k: bool, top_p: bool) -> str:
    """Key of STREAM_KERNEL: the kernel that reads every logit row once."""
    if mode == "greedy":
        return "greedy"
    return mode + ("_topk" if top_k else "_topp" if top_p else "")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_sha() -> str:
    """Hash of the HIP sources; a stored counter reading is used only if it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rejection_sampling_verify_07_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, mode: str):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{workload}/{mode}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_sha():
        return None
    return rec.get("bytes_per_launch")


def record_traffic(workload: str, mode: str, fetch_csv: str, write_csv: str, copy_mb: float) -> dict:
    """Per-launch HBM bytes of the streaming kernel from two rocprofv3 --pmc runs.

    fetch_csv / write_csv are the counter_collection.csv files of runs with
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of this same bench command
    with --copy-calibration-mb copy_mb.  Each counter is scaled by what it
    reads for that plain device copy of known size (the last five copy
    dispatches: copy_mb MB read and written each), and the result is stored
    in profiles/traffic.json under the current kernel-source hash.
    """
    import csv

    topk = re.search(r"_top\d", workload) is not None
    topp = re.search(r"_topp", workload) is not None
    kind_kernel = STREAM_KERNEL[stream_kind(mode, topk, topp)]

    def per_dispatch(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            vals[key] = (r["Kernel_Name"], vals.get(key, ("", 0.0))[1] + float(r["Counter_Value"]))
        return [vals[k] for k in sorted(vals)]

    out = {}
    known = copy_mb * 1e6
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = per_dispatch(path, counter)
        copies = [v for n, v in rows if "copy" in n.lower()][-5:]
        stream = sorted(v for n, v in rows if kind_kernel in n)
        if len(copies) < 5 or not stream:
            raise SystemExit(f"record-traffic: found {len(copies)} copy and {len(stream)} {kind_kernel} dispatches")
        copy_kib = sorted(copies)[2]
        factor = known / (copy_kib * 1024.0)
        out[counter] = {"stream_kib_median": stream[len(stream) // 2], "copy_kib": copy_kib, "factor": factor,
                        "bytes": stream[len(stream) // 2] * 1024.0 * factor, "dispatches": len(stream)}
    rec = {"source_sha": kernel_source_sha(), "kernel": kind_kernel,
           "bytes_per_launch": round(out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]),
           "fetch_bytes": round(out["FETCH_SIZE"]["bytes"]), "write_bytes": round(out["WRITE_SIZE"]["bytes"]),
           "calibration": {"copy_mb": copy_mb, "fetch_factor": round(out["FETCH_SIZE"]["factor"], 4),
                           "write_factor": round(out["WRITE_SIZE"]["factor"], 4)},
           "raw_kib": {"fetch": out["FETCH_SIZE"]["stream_kib_median"], "write": out["WRITE_SIZE"]["stream_kib_median"],
                       "copy_fetch": out["FETCH_SIZE"]["copy_kib"], "copy_write": out["WRITE_SIZE"]["copy_kib"]}}
    try:
        with open(TRAFFIC_FILE) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec[f"{workload}/{mode}"] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
    return rec


EPS_BOUNDARY = 1e-6  # a draw whose uniform lies this close to its threshold or CDF edge is a boundary draw


def draws_vs_oracle(w, mode, gpu, ref):
    """Outcome of the measured call against the oracle on the same inputs.

    For the sampling calls: the realized acceptance rate (accepted guesses /
    guesses) and beta at the first rejection (1 - the residual mass), and the
    oracle's boundary draws -- accept draws (|u - min(1, p/q)| < 1e-6 at an
    evaluated position), final draws (u within 1e-6 of the chosen token's CDF
    interval edge), top-p cuts within 1e-6 of top_p -- with the number of
    sequences whose accepted count or tokens differ from the oracle's outside
    them.  Greedy and draft-side sampling: compared entries and mismatches.
    """
    import numpy as np

    if mode == "greedy":
        bad = int(np.sum(gpu["num_accepted"] != ref["num_accepted"]) + np.sum(gpu["tokens"] != ref["tokens"]))
        return {"compared_sequences": int(w.batch), "mismatches": bad}
    if mode == "draft":
        ids_g, ids_o = gpu["ids"], ref["ids"]
        boundary = (ref["dist"] < EPS_BOUNDARY) | (ref["p_margin"] < EPS_BOUNDARY)
        return {"compared_rows": int(ids_o.size), "boundary_final": int(boundary.sum()),
                "mismatches": int(np.sum((ids_g != ids_o) & ~boundary))}
    if mode == "likelihood":
        return None
    cu, lens = w.cu_draft, w.draft_lens
    nacc = gpu["num_accepted"].astype(np.int64)
    rej = nacc < lens
    out = {"acceptance_rate": round(float(nacc.sum() / max(int(lens.sum()), 1)), 4),
           "beta_at_rejection_mean": round(float(np.mean(1.0 - gpu["residual_mass"][rej])), 4) if rej.any() else None,
           "rejecting_sequences": int(rej.sum()), "compared_sequences": int(w.batch)}
    b_acc = b_fin = b_topp = mism = 0
    for b in range(w.batch):
        K, t0, d0 = int(lens[b]), int(cu[b]) + b, int(cu[b])
        n_o = int(ref["num_accepted"][b])
        if ref.get("p_margin") is not None and ref["p_margin"][b] < EPS_BOUNDARY:
            b_topp += 1
            continue
        if any(ref["d_acc"][d0 + k] < EPS_BOUNDARY for k in range(min(n_o + 1, K))):
            b_acc += 1
            continue
        if mode == "sample" and ref["d_fin"][b] < EPS_BOUNDARY:
            b_fin += 1
            mism += int(gpu["num_accepted"][b] != n_o)
            continue
        if mode == "argmax" and ref["gap"][b] < 1e-4:
            b_fin += 1
            mism += int(gpu["num_accepted"][b] != n_o)
            continue
        same = gpu["num_accepted"][b] == n_o and np.array_equal(gpu["tokens"][t0:t0 + K + 1],
                                                                ref["tokens"][t0:t0 + K + 1])
        mism += int(not same)
    out.update({"boundary_accept": b_acc, "boundary_final": b_fin, "boundary_topp": b_topp,
                "mismatches_outside_boundary": mism})
    return out


def cpu_baseline(w, mode, seconds):
    import oracle

    units = w.rows_draft if mode in ("draft", "likelihood") else w.positions()
    unit = "draft tokens/s" if mode == "draft" else "positions/s"
    visible = len(os.sched_getaffinity(0))
    # the host's CPU share of one GPU is 16 cores on the machines this runs on:
    # the oracle's thread pool is sized to that share, not to every visible core
    threads = max(1, min(16, visible))
    ref = oracle.verify_workload(w, mode, threads=threads)  # also warms (page in, build)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.verify_workload(w, mode, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # the same oracle on one host core (at least one full batch, about half the time above)
    t1 = time.perf_counter()
    reps1 = 0
    while True:
        oracle.verify_workload(w, mode, threads=1)
        reps1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= seconds / 2:
            break
    return ref, {
        "value": reps * units / el,
        "unit": unit,
        "cores": threads,
        "cores_visible": visible,
        "kind": "oracle",
        "sample": f"the full batch of the same workload ({w.batch} sequences, {units} {unit[:-2]}), "
                  f"{reps} repetitions in {el:.1f} s, sequences split over {threads} host threads "
                  f"(the CPU share of one GPU; {visible} cores visible to the process)",
        "single_core": {"value": reps1 * units / el1, "cores": 1,
                        "sample": f"the same batch, {reps1} repetitions in {el1:.1f} s on one thread"},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=5, help="workload 1..5 (default 5: V=151936, top-k 50)")
    ap.add_argument("--mode", choices=["sample", "greedy", "argmax", "draft", "likelihood"], default="sample",
                    help="sample / greedy / argmax: spec_verify_*; draft: spec_draft_sample over the draft rows")
    ap.add_argument("--dtype", choices=["bf16", "f16"], default=None,
                    help="store a 16-bit workload's logits in this type instead (same values before rounding)")
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="nucleus filter after temperature and top-k (1 = off), for every call but greedy")
    ap.add_argument("--rotate-mb", type=float, default=512.0, help="total size of the rotated input copies")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile-pass", action="store_true")
    ap.add_argument("--batches", type=int, default=5,
                    help="after the K timed steps, this many further batches of >= --batch-ms each (spread)")
    ap.add_argument("--batch-ms", type=float, default=200.0)
    ap.add_argument("--copy-calibration-mb", type=float, default=0.0,
                    help="also run a plain device copy of this size (for counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store the streaming kernel's HBM bytes from two rocprofv3 --pmc runs (no GPU needed)")
    args = ap.parse_args()

    if args.record_traffic:
        import workloads as W

        name = W.WORKLOADS[args.config]["name"]
        if args.dtype is not None:
            name = name.replace(W.WORKLOADS[args.config]["dtype"], args.dtype)
        if args.top_p < 1.0:
            name = f"{name}_topp{args.top_p:g}"  # as the timed run names it
        rec = record_traffic(name, args.mode, args.record_traffic[0], args.record_traffic[1],
                             args.copy_calibration_mb or 256.0)
        print(json.dumps(rec))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; the verify step shards by sequence with no exchange "
              "across GPUs, so a single-GPU figure is the measured one and no multi-GPU figure is produced", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rejection_sampling_verify_07_amd as sv
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.dtype is not None and W.WORKLOADS[args.config]["dtype"] != args.dtype:
        if W.WORKLOADS[args.config]["dtype"] == "f32":
            print("--dtype applies to the 16-bit workloads (3, 4, 5)", file=sys.stderr)
            sys.exit(2)
        spec = dict(W.WORKLOADS[args.config], dtype=args.dtype)
        spec["name"] = spec["name"].replace(W.WORKLOADS[args.config]["dtype"], args.dtype)
        w = W.make_workload(spec, args.config)
    else:
        w = W.make_config(args.config)
    if args.top_p < 1.0:
        import dataclasses

        w = dataclasses.replace(w, top_p=args.top_p, name=f"{w.name}_topp{args.top_p:g}")
    mode = args.mode
    if mode not in ("draft", "argmax", "likelihood") and mode not in w.modes:
        print(f"config {args.config} is not measured in {mode} mode", file=sys.stderr)
        sys.exit(2)
    kind = stream_kind(mode, w.top_k > 0, w.top_p < 1.0)
    bytes_step = w.algorithmic_bytes(mode)
    copies = max(1, int(np.ceil(args.rotate_mb * 1e6 / bytes_step)))

    def to_dev(a):
        if w.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        t16 = torch.bfloat16 if w.dtype == "bf16" else torch.float16
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(t16)

    tgt0, drf0 = to_dev(w.likelihood_rows()[0] if mode == "likelihood" else w.target), to_dev(w.draft)
    ids = torch.from_numpy(w.draft_ids).to(dev)
    cu = torch.from_numpy(w.cu_draft).to(dev) if w.ragged else None
    kmax = w.k_max if cu is not None else None
    plans = []
    ws = None
    for i in range(copies):
        tgt = tgt0 if (i == 0 or mode == "draft") else tgt0.clone()
        drf = drf0 if (i == 0 or mode == "greedy") else drf0.clone()
        if mode == "likelihood":
            p = sv.LikelihoodPlan(tgt, drf, ids, cu_draft=cu, batch=None if cu is not None else w.batch,
                                  temperature=w.temperature, top_k=w.top_k, max_draft=kmax, workspace=ws,
                                  top_p=w.top_p)
        elif mode == "draft":
            p = sv.DraftPlan(drf, cu_draft=cu, batch=None if cu is not None else w.batch, temperature=w.temperature,
                             top_k=w.top_k, seed=w.seed, offset=w.offset, max_draft=kmax, workspace=ws,
                             top_p=w.top_p)
        elif mode == "greedy":
            p = sv.GreedyPlan(tgt, ids, cu_draft=cu, max_draft=kmax, workspace=ws)
        else:
            p = sv.SamplePlan(tgt, drf, ids, cu_draft=cu, temperature=w.temperature, top_k=w.top_k, seed=w.seed,
                              offset=w.offset, max_draft=kmax, workspace=ws, argmax=mode == "argmax",
                              top_p=w.top_p)
        ws = p.workspace
        plans.append(p)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        plans[i % copies]()
    torch.cuda.synchronize()

    # ---- timed region
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(K):
        plans[i % copies]()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / K
    positions = w.rows_draft if mode in ("draft", "likelihood") else w.positions()  # units per step
    value = positions / (ms_step * 1e-3)

    # ---- spread: further batches of at least --batch-ms each (the value above is the K-step region)
    spread = None
    if args.batches > 0:
        n_b = max(K, int(np.ceil(args.batch_ms / max(ms_step, 1e-6))))
        per = []
        for _ in range(args.batches):
            torch.cuda.synchronize()
            e0.record()
            for i in range(n_b):
                plans[i % copies]()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / n_b * 1e3)
        spread = {"batches": args.batches, "steps_per_batch": n_b, "median_us": round(float(np.median(per)), 3),
                  "min_us": round(min(per), 3), "max_us": round(max(per), 3)}

    # ---- profiled pass: HIP events around each streaming-kernel launch
    roof = None
    if not args.no_profile_pass:
        ev = sv.HipEvents(K)
        pairs = [ev.pair(i) for i in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            plans[i % copies].profiled(pairs[i])
        torch.cuda.synchronize()
        dur = np.array(ev.elapsed_ms()) * 1e-3
        ev.close()
        avg = float(dur.mean())
        achieved = bytes_step / avg / 1e9
        traffic = stored_traffic(w.name, mode)
        roof = {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": STREAM_KERNEL[kind], "bytes_per_launch": bytes_step,
            "avg_us": round(avg * 1e6, 3), "median_us": round(float(np.median(dur)) * 1e6, 3),
        }
        # practical roof: a plain read of the same bytes with the same loads and
        # tiles, over as many rotated buffers, timed the same way
        nbytes = bytes_step // 16 * 16
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
        reads = [sv.StreamReadPlan(b) for b in bufs]
        evr = sv.HipEvents(K)
        pairs_r = [evr.pair(i) for i in range(K)]
        for i in range(min(K, 20)):
            reads[i % copies].profiled(pairs_r[i])
        torch.cuda.synchronize()
        for i in range(K):
            reads[i % copies].profiled(pairs_r[i])
        torch.cuda.synchronize()
        dr = np.array(evr.elapsed_ms()) * 1e-3
        evr.close()
        del bufs, reads
        practical = nbytes / float(dr.mean()) / 1e9
        roof.update({"practical_roof": round(practical, 1), "frac_of_practical": round(achieved / practical, 4),
                     "practical_roof_kernel": "spec_profile_stream_read: plain read, 6 nontemporal 16-byte loads "
                                              "per thread, 256 threads, one tile per workgroup",
                     "practical_avg_us": round(float(dr.mean()) * 1e6, 3)})

    if args.copy_calibration_mb > 0:
        n = int(args.copy_calibration_mb * 1e6) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    draws = None
    if not args.no_cpu_baseline:
        ref, cpu = cpu_baseline(w, mode, args.cpu_seconds)
        p0 = plans[0]
        p0()
        torch.cuda.synchronize()
        if mode == "draft":
            gpu = {"ids": p0.out.cpu().numpy()}
        elif mode == "likelihood":
            gpu = None
        else:
            gpu = {k: v.cpu().numpy() for k, v in p0.out.items()}
        draws = draws_vs_oracle(w, mode, gpu, ref) if gpu is not None else None

    line = {
        "metric": {"draft": METRIC_DRAFT, "likelihood": METRIC_LIK}.get(mode, METRIC),
        "value": round(value, 1),
        "unit": "draft tokens/s" if mode == "draft" else "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "mode": mode, "batch": w.batch, "positions_per_step": w.positions(),
            "draft_tokens_per_step": w.rows_draft, "vocab": w.vocab, "input_dtype": w.dtype,
            "temperature": w.temperature, "top_k": w.top_k, "top_p": w.top_p, "bytes_per_step": bytes_step,
            "rotated_copies": copies, "hbm_gbs_whole_step": round(bytes_step / (ms_step * 1e-3) / 1e9, 1),
            "wall_s": round(wall, 4),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "timing_spread": spread,
        "draws": draws,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
