#!/usr/bin/env python3
"""Decode throughput of River-LLM token-level early exit on one MI355X.

Workload (default): Llama-3.1-8B-shaped decoder with random fp16 weights and its int4
(group 128) river copy, batch 1, a 2048-token random prompt prefilled at full depth, then
--steps decode tokens with forced exit layers drawn uniformly from {8..20} (mean 14).
A step is one decode token through all 32 layers (backbone up to the exit layer, river
after it) and the LM head; the timed region runs --steps steps with inputs resident in HBM.

The decode runs as one persistent cooperative kernel (8 steps per launch; with
RIVER_PERSIST=0 the per-op kernels replayed from a captured graph). Also measured in the
same run:
  * per-launch HIP-event timing of that kernel over the same S steps -> the roofline object;
  * per-launch timing of every per-op decode kernel (the graph path, one pass per kernel) ->
    a per-kernel breakdown of that path;
  * the full-depth fp16 decode (backbone only, no exit test) over the same positions;
  * the CPU oracle on a bounded sample (one backbone layer, one river layer and the LM head,
    scaled to a token by the realized mean exit layer).

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="llama3.1-8b-shape")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-full", action="store_true", help="skip the full-depth fp16 decode")
    ap.add_argument("--no-breakdown", action="store_true", help="skip per-kernel timing passes")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--pmc-summary", nargs=5, metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_FETCH_CSV",
                                                        "CALIB_WRITE_CSV", "BENCH_LOG"),
                    help="host only: write the HBM-traffic summary of k_persist from rocprofv3 "
                         "counter CSVs (FETCH_SIZE / WRITE_SIZE runs of this script, then the same "
                         "two counters on --calib-copy) and the bench output of the FETCH_SIZE run")
    ap.add_argument("--tau-sweep", type=int, default=0, metavar="N",
                    help="instead of the forced-schedule run: decode in tau mode at N values of tau "
                         "(quantiles of the similarities of a no-exit run) and report tokens/s "
                         "against the realised exit layers (batch 1)")
    args = ap.parse_args()
    if args.pmc_summary:
        write_pmc_summary(*args.pmc_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calib_copy:
        calib_copy(torch)
        return

    from token_level_early_amd import bytes_model as bm
    from token_level_early_amd import configs, river, synth

    cfgd = configs.ALL[args.config]
    c = configs.model_cfg(cfgd)
    B, P, S, W = cfgd["batch"], cfgd["prompt"], args.steps, args.warmup
    L = c["L"]
    dev = "cuda"
    t0 = time.time()
    w = synth.weights(c, seed=args.seed, device=dev)
    torch.cuda.synchronize()
    log(f"weights generated in {time.time() - t0:.1f}s")
    Tmax = P + W + S
    rv = river.River(c, w, max_seq=Tmax, max_prefill=P, batch=B)
    rv_chunk = int(os.environ.get("RIVER_PERSIST_CHUNK", "8"))
    torch.cuda.synchronize()
    log(f"river built in {time.time() - t0:.1f}s")
    toks = synth.prompt(c, B, P, seed=args.seed, device=dev)
    if args.tau_sweep:
        tau_sweep(args, c, cfgd, rv, toks, S, W, P, L, torch, bm, log)
        rv.close()
        return
    sched_np = synth.schedule(cfgd, W + S, B, seed=args.seed)
    sched = torch.from_numpy(sched_np).to(dev)

    def prefill_and_warm(backbone=False):
        pre = rv.prefill(toks, prefill_exit=L)
        if backbone:
            out = rv.decode_backbone_steps(pre["tokens"], W)
        else:
            out = rv.decode_steps(pre["tokens"], sched=sched[:W].contiguous())
        torch.cuda.synchronize()
        return out[-1].clone()

    tp = time.time()
    tok = prefill_and_warm()
    log(f"prefill {P} + warmup {W} in {time.time() - tp:.2f}s")

    # ---- timed region: S early-exit decode steps (graph replay)
    ex = torch.empty(S, B, dtype=torch.int32, device=dev)
    tok_out = torch.empty(S, B, dtype=torch.int32, device=dev)
    st_sched = sched[W:].contiguous()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    rv.decode_steps(tok, sched=st_sched, tok_out=tok_out, exit_layer=ex)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    exits_sb = ex.cpu().numpy()  # [S][B]
    assert np.array_equal(exits_sb, sched_np[W:]), "realized exit layers differ from the schedule"
    exits = exits_sb.mean(axis=1)
    positions = [P + W + s for s in range(S)]
    step_bytes = [bm.batch_step_bytes(c, [int(e) for e in exits_sb[s]], [positions[s]] * B) for s in range(S)]
    bytes_total = sum(step_bytes)
    tok_s = S * B / (ms / 1e3)
    step_gbs = bytes_total / (ms / 1e3) / 1e9
    log(f"early exit: {S} steps in {ms:.2f} ms -> {tok_s:.1f} tok/s, {step_gbs:.0f} GB/s "
        f"({100 * step_gbs / HBM_PEAK_GBS:.1f}% of HBM peak), mean exit {exits.mean():.2f}")

    # ---- dominant kernel: per-launch HIP events around the persistent decode kernel
    roof_pass = None
    tok = prefill_and_warm()
    n_launch = -(-S // rv_chunk)
    durs = []
    if rv.decode_path() == "persistent":
        rv.timer_arm("persist", n_launch)
        rv.decode_steps(tok, sched=st_sched, tok_out=tok_out, exit_layer=ex)
        durs = rv.timer_read(n_launch)
    if len(durs) == n_launch:
        launch_bytes = []
        for i in range(n_launch):
            lo, hi = i * rv_chunk, min(S, (i + 1) * rv_chunk)
            launch_bytes.append(sum(step_bytes[lo:hi]))
        avg_us = 1e3 * float(np.mean(durs))
        gbs = float(np.mean(launch_bytes)) / (avg_us * 1e-6) / 1e9
        # spread over the launches: tokens/s of each launch (its steps x rows / its duration)
        lt = [(min(S, (i + 1) * rv_chunk) - i * rv_chunk) * B / (durs[i] / 1e3) for i in range(n_launch)]
        roof_pass = {"launches": n_launch, "steps_per_launch": rv_chunk, "avg_us": round(avg_us, 2),
                     "bytes_per_launch": int(np.mean(launch_bytes)), "GB/s": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "tokens_per_s_p10_p50_p90": [round(float(np.percentile(lt, q)), 1) for q in (10, 50, 90)]}
        log(f"persistent kernel: {roof_pass}")

    # ---- per-kernel timing passes of the per-op kernels (direct launches, HIP events)
    kernels = {}
    if not args.no_breakdown:
        for op in ("gu", "down", "qkv", "o", "attn", "lm"):
            tok = prefill_and_warm()
            per_step = 1 if op == "lm" else L
            rv.timer_arm(op, S * per_step)
            rv.decode_steps(tok, sched=st_sched, tok_out=tok_out, exit_layer=ex)
            durs = np.array(rv.timer_read(S * per_step))
            tot_b = 0
            for s in range(S):
                es = [int(e) for e in exits_sb[s]]
                for l in range(1, per_step + 1):
                    tot_b += bm.batch_op_bytes(c, op, es, l, [positions[s]] * B)
            n = len(durs)
            avg_us = 1e3 * durs.mean()
            gbs = (tot_b / n) / (avg_us * 1e-6) / 1e9
            kernels[op] = {"launches": n, "avg_us": round(avg_us, 3),
                           "bytes_per_launch": int(tot_b / n), "GB/s": round(gbs, 1),
                           "frac": round(gbs / HBM_PEAK_GBS, 4),
                           "share_of_step": round(durs.sum() / ms, 4)}
            log(f"  {op:5s} avg {avg_us:8.2f} us  {gbs:7.0f} GB/s  share {durs.sum() / ms:.3f}")

    # ---- full-depth fp16 decode over the same positions
    full = None
    if not args.no_full:
        tok = prefill_and_warm(backbone=True)
        torch.cuda.synchronize()
        ev0.record()
        rv.decode_backbone_steps(tok, S, tok_out=tok_out)
        ev1.record()
        torch.cuda.synchronize()
        fms = ev0.elapsed_time(ev1)
        fbytes = sum(bm.batch_step_bytes(c, [L] * B, [p] * B) for p in positions)
        full = {"tokens_per_s": round(S * B / (fms / 1e3), 2), "ms_per_step": round(fms / S, 4),
                "GB/s": round(fbytes / (fms / 1e3) / 1e9, 1),
                "frac": round(fbytes / (fms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "speedup_of_early_exit": round(fms / ms, 4)}
        log(f"full depth: {full}")

    # ---- all-river decode (forced exit 0: every block on the int4 copy) over the same positions:
    # the all-quantised comparator, the speed the early exit approaches as exits move earlier
    allr = None
    if not args.no_full:
        tok = prefill_and_warm()
        zero = torch.zeros_like(st_sched)
        torch.cuda.synchronize()
        ev0.record()
        rv.decode_steps(tok, sched=zero, tok_out=tok_out)
        ev1.record()
        torch.cuda.synchronize()
        zms = ev0.elapsed_time(ev1)
        zbytes = sum(bm.batch_step_bytes(c, [0] * B, [p] * B) for p in positions)
        allr = {"tokens_per_s": round(S * B / (zms / 1e3), 2), "ms_per_step": round(zms / S, 4),
                "GB/s": round(zbytes / (zms / 1e3) / 1e9, 1),
                "frac": round(zbytes / (zms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "speedup_over_full_depth": round(fms / zms, 4) if full else None}
        log(f"all river: {allr}")

    # ---- achievable ceiling on this part: a plain device copy and a plain read of 1 GiB
    ceiling = hbm_ceiling(torch)
    log(f"measured HBM ceiling: {ceiling}")

    # ---- CPU oracle on a bounded sample
    cpu = None
    if not args.no_cpu and B == 1:
        cpu = cpu_baseline(c, w, rv, exits, positions, log)
        log(f"cpu oracle: {cpu}")
    rv.close()

    roof = None
    if roof_pass:
        roof = {"kernel": f"k_persist (early-exit decode, {rv_chunk} steps per launch)",
                "bound": "hbm", "achieved": roof_pass["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": roof_pass["frac"], "traffic": None,
                "avg_launch_us": roof_pass["avg_us"], "bytes_per_launch": roof_pass["bytes_per_launch"],
                "launches": roof_pass["launches"], "steps_per_launch": rv_chunk,
                "tokens_per_s_p10_p50_p90": roof_pass["tokens_per_s_p10_p50_p90"]}
    elif "gu" in kernels:  # per-op path: its largest kernel
        g = kernels["gu"]
        roof = {"kernel": "gate|up projection (per-op path)" if B == 1 else "k_b_gemm gate|up (batched MFMA)",
                "bound": "hbm", "achieved": g["GB/s"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": g["frac"], "traffic": None,
                "avg_launch_us": g["avg_us"], "bytes_per_launch": g["bytes_per_launch"]}
    if roof is not None:
        tr = pmc_traffic(roof, args.config)
        if tr is not None:
            roof["traffic"] = tr["bytes_per_launch"]
            roof["traffic_detail"] = tr

    out = {
        "metric": ("decode tokens/s at 8B shape (bs=1,ctx 2048) at fixed exit schedule; % HBM roofline"
                   if args.config == "llama3.1-8b-shape" else
                   f"decode tokens/s (all rows) at {args.config}, fixed exit schedule; % HBM roofline"),
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": W,
        "ms_per_step": round(ms / S, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "dtype_detail": "fp16 activations and KV cache, fp16 / int4 (fp16 group scales) weights, fp32 accumulation",
        "data": "synthetic (seeded random weights, prompt and exit schedule)",
        "config": {"workload": f"{args.config} decode, batch {B}, prompt {P}, forced exit "
                               f"e~{cfgd['sched'][0]}{{{cfgd['sched'][1]}..{cfgd['sched'][2]}}} "
                               f"(realized mean {exits.mean():.2f})",
                   "batch": B, "prompt": P, "decode_steps": S, "positions": [P + W, P + W + S - 1]},
        "hbm_roofline_pct": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "step": {"bytes_per_step": int(bytes_total / S), "achieved_GB/s": round(step_gbs, 1),
                 "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "hbm_measured_ceiling": ceiling,
        "kernels_per_op_path": kernels,
        "full_depth_fp16": full,
        "all_river_int4": allr,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


PMC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "k_persist_llama8b_decode_pmc.json")
KERNEL_SOURCES = ("persist.hip", "attn.hpp", "gemv.hpp", "common.hpp", "params.hpp", "api.cpp")


def kernel_source_hash():
    """Hash of the sources that define the persistent decode kernel and its launch."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "token_level_early_amd", "csrc")
    for n in KERNEL_SOURCES:
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def tau_sweep(args, c, cfgd, rv, toks, S, W, P, L, torch, bm, log):
    """Speed against exit rate in tau mode (the pages' trade-off between exit rate and speed,
    here on synthetic inputs, so without an accuracy axis). A run with tau = 2 (cos <= 1: never
    exits) records s(l) of every tested layer; the sweep's tau values are quantiles of those;
    each tau then decodes the same S positions after the same prefill and warm-up."""
    if rv.B != 1:
        raise SystemExit("--tau-sweep measures batch 1")
    dev = "cuda"
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(tau, sim=None):
        pre = rv.prefill(toks, prefill_exit=L)
        out = rv.decode_steps(pre["tokens"], S=W, tau=tau)
        torch.cuda.synchronize()
        ex = torch.empty(S, 1, dtype=torch.int32, device=dev)
        ev0.record()
        rv.decode_steps(out[-1].clone(), S=S, tau=tau, exit_layer=ex, sim=sim)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1), ex.cpu().numpy()[:, 0]

    sim = torch.empty(S, 1, L, dtype=torch.float32, device=dev)
    run(2.0, sim)
    sv = sim.cpu().numpy()[:, 0, :]
    sv = sv[~np.isnan(sv)]
    qs = np.linspace(0.05, 0.95, args.tau_sweep)
    taus = [float(np.float32(np.quantile(sv, q))) for q in qs]
    positions = [P + W + s for s in range(S)]
    points = []
    for q, tau in zip(qs, taus):
        ms, ex = run(tau)
        nbytes = sum(bm.batch_step_bytes(c, [int(e)], [p]) for e, p in zip(ex, positions))
        gbs = nbytes / (ms / 1e3) / 1e9
        pt = {"tau": round(tau, 6), "similarity_quantile": round(float(q), 3),
              "tokens_per_s": round(S / (ms / 1e3), 2), "mean_exit_layer": round(float(ex.mean()), 3),
              "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
        points.append(pt)
        log(f"tau sweep: {pt}")
    print(json.dumps({"metric": f"decode tokens/s against exit rate, tau mode, {args.config}",
                      "unit": "tokens/s", "n_gpus": 1, "steps": S, "warmup": W,
                      "higher_is_better": True, "data": "synthetic (seeded random weights and prompt)",
                      "config": {"workload": f"{cfgd['name']} decode, batch 1, prompt {P}, tau mode",
                                 "similarities": "s(l) of a no-exit run, layers >= entry"},
                      "tau_sweep": points}))


def pmc_traffic(roof, config):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by the plain-copy calibration), or None when those
    counters were taken on other kernel sources, another kernel or another workload."""
    try:
        with open(PMC_FILE) as f:
            pm = json.load(f)
    except (OSError, ValueError):
        return None
    if pm.get("source_hash") != kernel_source_hash() or not roof["kernel"].startswith(pm.get("kernel", "?")):
        return None
    if pm.get("workload", "").split(" ")[0] != config:  # counted on another workload
        return None
    return {"bytes_per_launch": pm["hbm_bytes_per_launch"], "fetch_bytes": pm["fetch_bytes_per_launch"],
            "write_bytes": pm["write_bytes_per_launch"],
            "ratio_to_algorithmic": round(pm["hbm_bytes_per_launch"] / pm["algorithmic_bytes_per_launch_same_launches"], 4),
            "launches": pm["workload"],
            "calibration": pm["calibration"], "source": os.path.relpath(PMC_FILE, os.path.dirname(PMC_FILE) + "/..")}


def _pmc_rows(path, name_prefix, counter):
    """Per-dispatch values (KiB) of `counter` for kernels whose name starts with name_prefix,
    in dispatch order, from a rocprofv3 counter-collection CSV."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and r["Kernel_Name"].lstrip("void ").startswith(name_prefix):
                rows.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return [v for _, v in sorted(rows)]


def write_pmc_summary(f_csv, w_csv, cf_csv, cw_csv, bench_log):
    """profiles/k_persist_llama8b_decode_pmc.json from the four counter runs: FETCH_SIZE and
    WRITE_SIZE of the last `roofline.launches` k_persist dispatches (the roofline pass), each
    scaled by what the same counter reads per byte of a plain 512 MiB device copy."""
    line = [l for l in open(bench_log) if l.startswith("{") and '"metric"' in l][-1]
    out = json.loads(line)
    roof = out["roofline"]
    n = int(roof["launches"])
    fetch = _pmc_rows(f_csv, "k_persist", "FETCH_SIZE")[-n:]
    write = _pmc_rows(w_csv, "k_persist", "WRITE_SIZE")[-n:]
    cf = _pmc_rows(cf_csv, "__amd_rocclr_copyBuffer", "FETCH_SIZE")
    cw = _pmc_rows(cw_csv, "__amd_rocclr_copyBuffer", "WRITE_SIZE")
    if len(fetch) != n or len(write) != n or not cf or not cw:
        raise SystemExit(f"pmc summary: expected {n} k_persist dispatches and copy dispatches in the CSVs")
    copy_bytes = 512 << 20
    kf, kw = sum(cf) / len(cf), sum(cw) / len(cw)
    fs, ws = copy_bytes / (kf * 1024), copy_bytes / (kw * 1024)
    fb = sum(fetch) / n * 1024 * fs
    wb = sum(write) / n * 1024 * ws
    summary = {
        "kernel": "k_persist",
        "workload": (f"{out['config']['workload']}, {roof['steps_per_launch']} steps per launch "
                     f"(roofline-pass launches of bench.py --no-cpu --no-full --no-breakdown --steps {out['steps']})"),
        "source_hash": kernel_source_hash(),
        "fetch_bytes_per_launch": int(fb),
        "write_bytes_per_launch": int(wb),
        "hbm_bytes_per_launch": int(fb + wb),
        "algorithmic_bytes_per_launch_same_launches": int(roof["bytes_per_launch"]),
        "calibration": {"copy_bytes": copy_bytes, "fetch_size_kib_per_copy": kf, "write_size_kib_per_copy": kw,
                        "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
                        "copy_kernel": "__amd_rocclr_copyBuffer (torch copy_ of 512 MiB)"},
        "raw_kib_per_dispatch": {"FETCH_SIZE": fetch, "WRITE_SIZE": write},
    }
    with open(PMC_FILE, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    print(json.dumps({k: summary[k] for k in ("hbm_bytes_per_launch", "algorithmic_bytes_per_launch_same_launches")}))


def hbm_ceiling(torch):
    """Bandwidth that plain library kernels reach on this part, for context beside the 8 TB/s
    vendor peak: torch copy_ of 1 GiB (reads and writes 1 GiB each) and a float32 sum over
    1 GiB of fp16 (reads it once); best of 5 after one untimed call, HIP events."""
    n = 512 << 20  # fp16 elements = 1 GiB
    x = torch.ones(n, dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    t_copy = best(lambda: y.copy_(x))
    t_read = best(lambda: x.sum(dtype=torch.float32))
    nbytes = 2 * n
    del x, y
    return {"copy_GB/s": round(2 * nbytes / (t_copy / 1e3) / 1e9, 1),
            "read_GB/s": round(nbytes / (t_read / 1e3) / 1e9, 1),
            "how": "torch copy_ of 1 GiB (2 GiB moved) and float32 sum over 1 GiB fp16, best of 5"}


def calib_copy(torch):
    """A plain device copy of known size, three times, for scaling the FETCH_SIZE / WRITE_SIZE
    counters: each copy reads and writes exactly 512 MiB."""
    n = 256 << 20  # fp16 elements = 512 MiB
    x = torch.ones(n, dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": 2 * n, "copies": 3}), flush=True)


def cpu_baseline(c, w, rv, exits, positions, log):
    """Times the CPU oracle (fp64 NumPy) on one backbone layer, one river layer and the LM head
    at the bench's context length, and scales to ms per decode token with the realized mean
    exit layer: t_tok = e*t_backbone + (L-e)*t_river + t_head."""
    import torch

    from oracle import river_oracle as O
    from token_level_early_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    L = c["L"]
    lay = [0, 1]
    host = synth.to_numpy({"embed": w["embed"], "lm_head": w["lm_head"], "final_norm": w["final_norm"],
                           "layers": [w["layers"][i] if i in lay else None for i in range(L)]})
    orc = O.RiverOracle(c, host, layers=lay)
    kv = rv.kv_view()
    pos = positions[0]
    Kc = [kv[l, 0, 0, :, : pos + 1].cpu().numpy().copy() for l in lay]
    Vc = [kv[l, 1, 0, :, : pos + 1].cpu().numpy().copy() for l in lay]
    h = rv.hidden()[0, 0].cpu().numpy()

    def timed(fn, reps):
        fn()  # first call pays one-time conversions
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t) / reps

    reps = 3
    t_bb = timed(lambda: O.block_decode(c, orc.bb[0], orc.norms(0), h, pos, Kc[0], Vc[0]), reps)
    t_rv = timed(lambda: O.block_decode(c, orc.rv[1], orc.norms(1), h, pos, Kc[1], Vc[1]), reps)
    t_hd = timed(lambda: orc.head_logits(h), reps)
    e = float(np.mean(exits))
    ms_tok = 1e3 * (e * t_bb + (L - e) * t_rv + t_hd)
    return {"value": round(1e3 / ms_tok, 4), "unit": "tokens/s", "ms_per_token": round(ms_tok, 2),
            "cores": threads, "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"fp64 NumPy oracle: backbone block (layer 1), river block (layer 2) and LM "
                      f"head at position {pos}, {reps} reps each after one untimed call; token "
                      f"time = e*t_bb + (L-e)*t_river + t_head with realized mean e={e:.2f}"}


if __name__ == "__main__":
    main()
