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
  * the CPU oracle (the tests' fp64 reference) decoding two whole tokens of the timed run from
    the GPU's state (a bounded sample; see cpu_baseline).
A pass whose device status reports an error, or whose tokens differ between the timed and the
roofline pass, ends the run with an error instead of a number.

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
    ap.add_argument("--cpu-tokens", type=int, default=2,
                    help="decode tokens the CPU oracle times (consecutive steps of the timed run)")
    ap.add_argument("--no-full", action="store_true", help="skip the full-depth fp16 decode")
    ap.add_argument("--no-breakdown", action="store_true", help="skip per-kernel timing passes")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--pmc-summary", nargs=5, metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_FETCH_CSV",
                                                        "CALIB_WRITE_CSV", "BENCH_LOG"),
                    help="host only: write the HBM-traffic summary of k_persist from rocprofv3 "
                         "counter CSVs (FETCH_SIZE / WRITE_SIZE runs of this script, then the same "
                         "two counters on --calib-copy) and the bench output of the FETCH_SIZE run")
    ap.add_argument("--trace-summary", nargs=3, metavar=("RESULTS_DB", "BENCH_LOG", "OUT_MD"),
                    help="host only: write a markdown summary of a rocprofv3 --kernel-trace --stats "
                         "run of this script (its rocpd database and its log) with the persistent "
                         "kernel's algorithmic bytes per launch and achieved bandwidth")
    ap.add_argument("--pmc-table", nargs=4, metavar=("CSV", "OUT_MD", "TITLE", "COMMAND"),
                    help="host only: per-kernel means of every counter in a rocprofv3 --pmc CSV")
    ap.add_argument("--phase-trace", metavar="OUT_MD",
                    help="instead of the timed run: decode one 8-step launch on the library built "
                         "with RIVER_PHASE_TRACE and write the per-phase timing of the persistent "
                         "kernel (batch 1) to OUT_MD")
    ap.add_argument("--tau-sweep", type=int, default=0, metavar="N",
                    help="instead of the forced-schedule run: decode in tau mode at N values of tau "
                         "(quantiles of the similarities of a no-exit run) and report tokens/s "
                         "against the realised exit layers (batch 1)")
    args = ap.parse_args()
    if args.pmc_summary:
        write_pmc_summary(*args.pmc_summary)
        return
    if args.trace_summary:
        write_trace_summary(*args.trace_summary)
        return
    if args.pmc_table:
        write_pmc_table(*args.pmc_table)
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
    if args.phase_trace:
        phase_trace(args, c, cfgd, w, torch, bm, river, synth, log)
        return
    rv = river.River(c, w, max_seq=Tmax, max_prefill=P, batch=B)
    rv_chunk = int(os.environ.get("RIVER_PERSIST_CHUNK", "8"))
    torch.cuda.synchronize()
    log(f"river built in {time.time() - t0:.1f}s")
    toks = synth.prompt(c, B, P, seed=args.seed, device=dev)
    if args.tau_sweep:
        tau_sweep(args, c, cfgd, rv, toks, S, W, P, L, torch, bm, log)
        rv.close()
        return
    tau = None
    if cfgd.get("sched") is None:
        # tau-mode workload: tau calibrated on these inputs (bisection on the fraction of decode
        # tokens that exit by layer `exit_by`), then every step decides its own exit
        tau = calibrate_tau(rv, c, cfgd, toks, torch, log)
        sched_np, sched, st_sched = None, None, None
    else:
        sched_np = synth.schedule(cfgd, W + S, B, seed=args.seed)
        sched = torch.from_numpy(sched_np).to(dev)
        st_sched = sched[W:].contiguous()

    def decode(tok, n, sch, **kw):
        if tau is None:
            return rv.decode_steps(tok, sched=sch, **kw)
        return rv.decode_steps(tok, S=n, tau=tau, **kw)

    def prefill_and_warm(backbone=False):
        pre = rv.prefill(toks, prefill_exit=L)
        if backbone:
            out = rv.decode_backbone_steps(pre["tokens"], W)
        else:
            out = decode(pre["tokens"], W, None if sched is None else sched[:W].contiguous())
        torch.cuda.synchronize()
        check_status(rv, "prefill and warm-up")
        return out[-1].clone()

    tp = time.time()
    tok = prefill_and_warm()
    tok_first = tok.clone()
    log(f"prefill {P} + warmup {W} in {time.time() - tp:.2f}s")

    # ---- timed region: S early-exit decode steps
    ex = torch.empty(S, B, dtype=torch.int32, device=dev)
    tok_out = torch.empty(S, B, dtype=torch.int32, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    decode(tok, S, st_sched, tok_out=tok_out, exit_layer=ex)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    check_status(rv, "timed early-exit run")
    exits_sb = ex.cpu().numpy()  # [S][B]
    toks_timed = tok_out.cpu().numpy().copy()
    if sched_np is not None and not np.array_equal(exits_sb, sched_np[W:]):
        fail("realized exit layers differ from the schedule")
    cpu_input = None
    if not args.no_cpu and B == 1:  # the GPU's state the CPU oracle continues from
        cpu_input = cpu_sample_inputs(rv, exits_sb, toks_timed, int(tok_first[0]), P + W, args.cpu_tokens)
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
        decode(tok, S, st_sched, tok_out=tok_out, exit_layer=ex)
        durs = rv.timer_read(n_launch)
        check_status(rv, "roofline pass")
        if not (np.array_equal(tok_out.cpu().numpy(), toks_timed) and np.array_equal(ex.cpu().numpy(), exits_sb)):
            fail("the roofline pass produced other tokens or exit layers than the timed pass")
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
            decode(tok, S, st_sched, tok_out=tok_out, exit_layer=ex)
            durs = np.array(rv.timer_read(S * per_step))
            check_status(rv, f"per-op timing pass {op}")
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
        check_status(rv, "full-depth run")
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
        zero = torch.zeros(S, B, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        ev0.record()
        rv.decode_steps(tok, sched=zero, tok_out=tok_out)
        ev1.record()
        torch.cuda.synchronize()
        zms = ev0.elapsed_time(ev1)
        check_status(rv, "all-river run")
        zbytes = sum(bm.batch_step_bytes(c, [0] * B, [p] * B) for p in positions)
        allr = {"tokens_per_s": round(S * B / (zms / 1e3), 2), "ms_per_step": round(zms / S, 4),
                "GB/s": round(zbytes / (zms / 1e3) / 1e9, 1),
                "frac": round(zbytes / (zms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "speedup_over_full_depth": round(fms / zms, 4) if full else None}
        log(f"all river: {allr}")

    # ---- prompt prefill at full depth (the step before decode): whole-prompt time and the
    # arithmetic rate of its linear maps and causal attention
    pf = prefill_rate(rv, toks, c, B, P, torch)
    log(f"prefill: {pf}")

    # ---- achievable ceiling on this part: a plain device copy and a plain read of 1 GiB
    ceiling = hbm_ceiling(torch)
    log(f"measured HBM ceiling: {ceiling}")

    # ---- CPU oracle on a bounded sample
    rv.close()
    cpu = None
    if cpu_input is not None:
        cpu = cpu_baseline(c, w, cpu_input, log)
        log(f"cpu oracle: {cpu}")

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
        "config": {"workload": f"{args.config} decode, batch {B}, prompt {P}, " + (
                       f"forced exit e~{cfgd['sched'][0]}{{{cfgd['sched'][1]}..{cfgd['sched'][2]}}}"
                       if tau is None else f"tau mode, tau={tau:.6f} calibrated so that about "
                       f"{int(100 * cfgd['exit_frac'])}% of tokens exit by layer {cfgd['exit_by']}")
                   + f" (realized mean exit {exits.mean():.2f})",
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
        "prefill_full_depth": pf,
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
        check_status(rv, f"tau sweep, tau={tau}")
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


def prefill_rate(rv, toks, c, B, P, torch, reps=2):
    """Full-depth prefill of the bench prompt, best of `reps` after one untimed call (HIP
    events on the current stream). FLOPs: 2 per weight per prompt row for the linear maps of
    every block, 2*2*H*D per (query, visible key) pair for causal attention (QK^T and PV), the
    LM head on the last position of each row."""
    L, d, H, D, Hkv, F, V = c["L"], c["d"], c["H"], c["D"], c["Hkv"], c["F"], c["V"]
    P_l = (H + 2 * Hkv) * D * d + d * H * D + 3 * F * d
    lin = 2.0 * B * P * P_l * L + 2.0 * B * V * d
    att = 2.0 * 2 * H * D * B * (P * (P + 1) / 2) * L
    rv.prefill(toks, prefill_exit=L)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rv.prefill(toks, prefill_exit=L)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    check_status(rv, "prefill timing")
    return {"ms": round(best, 2), "tokens_per_s": round(B * P / (best / 1e3), 1),
            "TFLOP/s": round((lin + att) / (best / 1e3) / 1e12, 1),
            "frac_of_fp16_mfma_peak": round((lin + att) / (best / 1e3) / 2.5e15, 4),
            "linear_TFLOP": round(lin / 1e12, 2), "attention_TFLOP": round(att / 1e12, 2),
            "how": f"full-depth prefill of {B} x {P} tokens, best of {reps} after one untimed call"}


def phase_trace(args, c, cfgd, w, torch, bm, river, synth, log):
    """Per-phase timing of the persistent kernel from the phase-trace library: one 8-step launch
    of the bench workload (after its prefill and two warm launches), timestamps of every
    workgroup at every phase boundary. Per phase: crit = growth of the last workgroup's finish
    time over the previous phase's (the phase's share of the step), wait+stage = mean over
    workgroups from finishing the previous phase to having the input staged, stream = mean from
    staged to done; blocks split by route (backbone up to the exit layer, river after)."""
    import numpy as np
    B, P = cfgd["batch"], cfgd["prompt"]
    if B != 1:
        fail("--phase-trace measures the batch-1 persistent kernel")
    L, S, W = c["L"], 8, 16
    rv = river.River(c, w, max_seq=P + W + S + 8, max_prefill=P, batch=1, lib_path=river.LIB_PHASETRACE_PATH)
    if rv.decode_path() != "persistent":
        fail("the phase trace needs the persistent decode path")
    toks = synth.prompt(c, 1, P, seed=args.seed, device="cuda")
    sched_np = synth.schedule(cfgd, W + S, 1, seed=args.seed)
    sched = torch.from_numpy(sched_np).to("cuda")
    pre = rv.prefill(toks, prefill_exit=L)
    out = rv.decode_steps(pre["tokens"], sched=sched[:W].contiguous())  # two warm launches
    tok = out[-1].clone()
    out = rv.decode_steps(tok, sched=sched[W:].contiguous())
    torch.cuda.synchronize()
    check_status(rv, "phase-trace launch")
    t = rv.phase_trace().astype(np.float64) * 0.01  # 100 MHz ticks -> us
    rv.close()
    exits = [int(e) for e in sched_np[W:, 0]]
    positions = [P + W + s for s in range(S)]
    EV = {"start": 0, "qkv_st": 1, "qkv": 2, "att": 3, "o_st": 4, "o": 5, "gu_st": 6, "gu": 7, "dn_st": 8, "dn": 9}
    phases = [("qkv", "start", "qkv_st", "qkv"), ("attn", "qkv", None, "att"), ("o", "att", "o_st", "o"),
              ("gu", "o", "gu_st", "gu"), ("down", "gu", "dn_st", "dn")]
    rows = {"backbone": {}, "river": {}}
    layer_tot = {"backbone": [], "river": []}
    head = {"lm": [], "barrier": []}
    step_us = []
    for s in range(S):
        prev_end = None
        if s > 0:
            prev_end = t[s - 1, L, EV["att"]].max()
        for l in range(1, L + 1):
            T = t[s, l - 1]
            kind = "backbone" if l <= exits[s] else "river"
            start_max = prev_end if prev_end is not None else T[EV["start"]].max()
            prev = start_max
            for name, a0, st, a1 in phases:
                end = T[EV[a1]].max()
                r = rows[kind].setdefault(name, {"crit": [], "wait": [], "stream": [], "bytes": []})
                r["crit"].append(end - prev)
                if st is not None:
                    r["wait"].append(float(np.mean(T[EV[st]] - T[EV[a0]])))
                    r["stream"].append(float(np.mean(T[EV[a1]] - T[EV[st]])))
                r["bytes"].append(bm.batch_op_bytes(c, name, [exits[s]], l, [positions[s]]))
                prev = end
            layer_tot[kind].append(T[EV["dn"]].max() - start_max)
            prev_end = T[EV["dn"]].max()
        H = t[s, L]
        head["lm"].append(H[EV["qkv"]].max() - prev_end)
        head["barrier"].append(H[EV["att"]].max() - H[EV["qkv"]].max())
        if s > 0:
            step_us.append(H[EV["att"]].max() - t[s - 1, L, EV["att"]].max())
    lines = ["# k_persist per-phase timing (phase-trace build), " + cfgd["name"] + ", batch 1", "",
             "Command: `python bench.py --config " + cfgd["name"] + " --phase-trace " + args.phase_trace + "`",
             "(library `token_level_early_amd/libriver_phasetrace.so`: the same sources built with "
             "`-DRIVER_PHASE_TRACE`; thread 0 of each of the 256 workgroups stores the 100 MHz realtime "
             "counter at every phase boundary).", "",
             f"Workload: {P}-token prompt, one persistent launch of {S} steps at positions "
             f"{positions[0]}..{positions[-1]}, forced exit layers {exits} (blocks up to the exit layer run "
             "the fp16 backbone, the rest the int4 river).", "",
             "Per phase, means over the blocks of that route and the 8 steps: **crit** = growth of the last "
             "workgroup's finish time over the previous phase's (the phase's share of the step); "
             "**wait+stage** = mean over workgroups from finishing the previous phase to having this "
             "phase's input staged in LDS; **stream** = mean from staged to done; **bytes** = algorithmic "
             "bytes of the phase; **GB/s** = bytes / crit.", ""]
    for kind in ("backbone", "river"):
        n = len(layer_tot[kind])
        if not n:
            continue
        lines += [f"## {kind} blocks ({n} block-steps): {np.mean(layer_tot[kind]):.1f} us per block", "",
                  "| phase | crit us | wait+stage us | stream us | bytes MB | GB/s |", "|---|---|---|---|---|---|"]
        for name, *_ in phases:
            r = rows[kind][name]
            crit = float(np.mean(r["crit"]))
            wt = f"{np.mean(r['wait']):.2f}" if r["wait"] else "-"
            stv = f"{np.mean(r['stream']):.2f}" if r["stream"] else "-"
            byt = float(np.mean(r["bytes"]))
            lines.append(f"| {name} | {crit:.2f} | {wt} | {stv} | {byt / 1e6:.2f} | {byt / (crit * 1e-6) / 1e9:.0f} |")
        lines.append("")
    lm_b = bm.batch_op_bytes(c, "lm", exits[:1], L + 1, positions[:1])
    lines += ["## LM head and step", "",
              f"LM head (final norm, {c['V']} rows): crit {np.mean(head['lm']):.1f} us "
              f"({lm_b / (np.mean(head['lm']) * 1e-6) / 1e9:.0f} GB/s); grid barrier after it "
              f"{np.mean(head['barrier']):.2f} us.", "",
              f"Step time (barrier to barrier, steps 1..{S - 1}): {np.mean(step_us):.1f} us "
              f"({1e6 / np.mean(step_us):.1f} tokens/s in this launch).", ""]
    with open(args.phase_trace, "w") as f:
        f.write("\n".join(lines))
    log("\n".join(lines))


def write_pmc_table(csv_path, out_md, title, command):
    """Markdown table of a rocprofv3 --pmc CSV: per kernel, the dispatch count and the mean of
    every collected counter (derived counters such as MfmaUtil included as rocprofv3 computed
    them)."""
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            k = r["Kernel_Name"]
            if k.startswith("void at::") or k.startswith("at::"):
                continue
            d = per.setdefault(k, {})
            d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for d in per.values() for c in d})
    md = [f"# {title}", "", "Command (run from /tmp with `TMPDIR=/tmp`, `R` = repository root, `OUT` = an output directory):", "", "```",
          command, "```", "", "| kernel | dispatches | " + " | ".join(f"mean {c}" for c in names) + " |",
          "|---|---:|" + "---:|" * len(names)]
    for k, d in sorted(per.items(), key=lambda kv: -len(next(iter(kv[1].values())))):
        n = len(next(iter(d.values())))
        md.append(f"| `{k[:100]}` | {n} | " + " | ".join(
            f"{sum(d[c]) / len(d[c]):.4g}" if c in d else "-" for c in names) + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")
    print(out_md)


def write_trace_summary(db, bench_log, out_md):
    """Markdown summary of a kernel-trace run: the rocpd database's top_kernels view (torch's
    own kernels, which only generate the synthetic inputs, left out) and, for the persistent
    decode kernel, the bench's algorithmic bytes per launch against the traced average duration."""
    import re
    import sqlite3
    rows = sqlite3.connect(db).execute(
        "select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
    lines = [l for l in open(bench_log) if l.startswith("{") and '"metric"' in l]
    out = json.loads(lines[-1]) if lines else None
    cmd = [l for l in open(bench_log) if "[rocprofv3] '" in l]
    md = ["# rocprofv3 kernel trace", ""]
    if cmd:
        md += ["Traced command (run from /tmp with `TMPDIR=/tmp`, `R` = repository root, `OUT` = an output directory):", "",
               "```", "rocprofv3 --kernel-trace --stats -d $OUT -o kt -- "
               + re.sub(r"\S*/bench\.py", "$R/bench.py", cmd[0].split("'")[1]), "```", ""]
    if out:
        md += [f"Workload: {out['config']['workload']}; {out['steps']} timed steps after {out['warmup']} warm-up steps.", ""]
    md += ["| kernel | calls | total us | avg us | % of GPU time |", "|---|---:|---:|---:|---:|"]
    persist = None
    for name, calls, tot, avg, pct in rows:
        if name.startswith("void at::") or name.startswith("at::"):
            continue
        md.append(f"| `{name[:110]}` | {calls} | {tot:.1f} | {avg:.2f} | {pct:.2f} |")
        if name.startswith("void k_persist") and persist is None:
            persist = (name, calls, avg)
    if out and out.get("roofline") and persist:
        # the roofline pass: of the early-exit kernel's dispatches (its warm-up launches, the timed
        # pass, the roofline pass and, when run, the all-river pass, in that order), the window of
        # `launches` consecutive ones whose mean is closest to the live HIP-event average
        r = out["roofline"]
        n = int(r["launches"])
        seq = [d / 1e3 for (d,) in sqlite3.connect(db).execute(
            "select duration from kernels where name = ? order by start", (persist[0],))]
        best = min(range(len(seq) - n + 1), key=lambda i: abs(sum(seq[i:i + n]) / n - r["avg_launch_us"]))
        avg = sum(seq[best:best + n]) / n
        gbs = r["bytes_per_launch"] / (avg * 1e-6) / 1e9
        md += ["", f"Persistent decode kernel, roofline pass ({n} launches of {r['steps_per_launch']} steps: "
               f"dispatches {best + 1}..{best + n} of the {len(seq)} of `{persist[0].split('(')[0]}`, the window of {n} "
               f"consecutive ones closest to the live average): {r['bytes_per_launch'] / 1e9:.2f} GB algorithmic per launch "
               f"(bytes model at the realised exit layers and positions: {out['config']['workload'].split('(')[-1].rstrip(')')}); "
               f"traced average {avg:.1f} us per launch against {r['avg_launch_us']:.1f} us timed live with HIP "
               f"events; {gbs:.0f} GB/s = {gbs / HBM_PEAK_GBS:.3f} of 8 TB/s from the traced durations."]
    if out and out.get("prefill_full_depth"):
        pf = out["prefill_full_depth"]
        md += ["", f"Full-depth prefill in the same run: {pf['ms']} ms, {pf['TFLOP/s']} TFLOP/s "
               f"({pf['frac_of_fp16_mfma_peak']:.3f} of the 2.5 PF fp16 MFMA peak)."]
    st = [l.strip() for l in open(bench_log) if l.startswith("rocprofv3 exit status")]
    if st:
        coop = "launches" if persist else "does not launch"
        md += ["", f"{st[-1]} (the program {coop} cooperative kernels; the database was complete and "
               "the program's last line printed before rocprofv3 ended)."]
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")
    print(out_md)


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


def fail(msg):
    """Ends the run with a non-zero status: a number measured on a failed run is not reported."""
    log(f"bench failed: {msg}")
    print(json.dumps({"error": msg}), flush=True)
    sys.exit(3)


def check_status(rv, what):
    """The device error word after a pass (a persistent launch that gave up a bounded wait ends
    early and would otherwise time as a faster, wrong run)."""
    rc = rv.device_status()
    if rc != 0:
        fail(f"{what}: device status {rc} ({rv.lib.river_last_error().decode()})")


def calibrate_tau(rv, c, cfgd, toks, torch, log, iters=8, steps=48):
    """tau for a tau-mode workload: bisection on [0, 1] until about `exit_frac` of `steps` decode
    tokens (after a full-depth prefill) exit by layer `exit_by`; tau is an fp32 value."""
    L = c["L"]
    lo, hi = 0.0, 1.0
    for _ in range(iters):
        mid = float(np.float32((lo + hi) / 2))
        pre = rv.prefill(toks, prefill_exit=L)
        ex = torch.empty(steps, rv.B, dtype=torch.int32, device="cuda")
        rv.decode_steps(pre["tokens"], S=steps, tau=mid, exit_layer=ex)
        torch.cuda.synchronize()
        check_status(rv, "tau calibration")
        frac = float((ex.cpu().numpy() <= cfgd["exit_by"]).mean())
        if frac > cfgd["exit_frac"]:
            lo = mid
        else:
            hi = mid
    tau = float(np.float32((lo + hi) / 2))
    log(f"calibrated tau = {tau:.6f} ({iters} bisection steps over {steps} decode tokens)")
    return tau


def cpu_sample_inputs(rv, exits_sb, toks_timed, tok_first, pos0, ntok):
    """Picks `ntok` consecutive steps of the timed run for the CPU oracle -- the run of steps
    whose exit layers span the fewest layers (so the oracle materialises the fewest blocks),
    later steps first among equals -- and copies the GPU state the oracle continues from: the
    input tokens and the shared cache (all layers, positions before the first sampled step)."""
    S = exits_sb.shape[0]
    ntok = max(1, min(ntok, S))
    ex = exits_sb[:, 0].astype(int)
    best = None
    for s in range(S - ntok + 1):
        e = ex[s:s + ntok]
        key = (int(e.max() - e.min()), -int(e.max()), s)
        if best is None or key < best[0]:
            best = (key, s)
    s0 = best[1]
    toks_in = [tok_first if s == 0 else int(toks_timed[s - 1, 0]) for s in range(s0, s0 + ntok)]
    pos = pos0 + s0
    kv = rv.kv_view()[:, :, 0, :, :pos].cpu().numpy()  # [L][2][Hkv][pos][D]
    return {"s0": s0, "pos": pos, "exits": [int(x) for x in ex[s0:s0 + ntok]], "toks_in": toks_in,
            "gpu_toks": [int(toks_timed[s, 0]) for s in range(s0, s0 + ntok)], "kv": kv}


def cpu_baseline(c, w, inp, log):
    """Times the CPU oracle (fp64 NumPy, tests' reference implementation, as it stands) on whole
    decode tokens: consecutive steps of the timed GPU run, each at its own position with the
    GPU's input token, forced exit layer and shared cache (prompt and earlier decode slots).
    The oracle's set-up (fp64 copies of the blocks those tokens run, the river quantisation of
    the river blocks) is not timed. When the host lacks the memory for those copies, one
    backbone block, one river block and the LM head are timed instead and scaled to a token."""
    import torch  # noqa: F401  (weights live on the GPU; copied to host per layer)

    from oracle import river_oracle as O
    from token_level_early_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    L, d, V = c["L"], c["d"], c["V"]
    exits, pos, ntok = inp["exits"], inp["pos"], len(inp["exits"])
    bb = list(range(max(exits)))               # 0-based blocks some sampled token runs on the backbone
    rvl = list(range(min(exits), L))           # ... and on the river
    P_l = sum(int(np.prod(t.shape)) for k, t in w["layers"][0].items() if k not in ("attn_norm", "mlp_norm"))
    need = 8 * P_l * (len(bb) + len(rvl)) + 8 * V * d + 2 * P_l * len(set(bb) | set(rvl)) + 2 * inp["kv"].nbytes
    try:
        import psutil
        avail = psutil.virtual_memory().available
    except Exception:
        avail = 0
    if need > 0.8 * avail:
        log(f"cpu oracle: {need / 1e9:.1f} GB needed for whole tokens, {avail / 1e9:.1f} GB available: "
            "timing one block of each kind instead")
        return cpu_block_sample(c, w, inp, threads, log)
    t0 = time.time()
    used = sorted(set(bb) | set(rvl))
    host = synth.to_numpy({"embed": w["embed"], "lm_head": w["lm_head"], "final_norm": w["final_norm"],
                           "layers": [w["layers"][i] if i in used else None for i in range(L)]})
    orc = O.RiverOracle(c, host, layers=bb, river_layers=rvl)
    for lw in host["layers"]:  # the fp64 copies are built; drop the fp16 matrices
        if lw is not None:
            for m in list(lw):
                if m not in ("attn_norm", "mlp_norm"):
                    lw[m] = None
    kvo = orc.new_kv(1, pos + ntok)
    kvo.K[:, 0, :, :pos] = inp["kv"][:, 0]
    kvo.V[:, 0, :, :pos] = inp["kv"][:, 1]
    kvo.pos[0] = pos
    orc.head_logits(np.zeros(d, np.float16))  # builds the fp64 head once (set-up, not timed)
    log(f"cpu oracle set-up {time.time() - t0:.1f}s ({len(bb)} backbone + {len(rvl)} river blocks)")
    t = time.perf_counter()
    agree = 0
    for j in range(ntok):
        o = orc.decode_step(kvo, [inp["toks_in"][j]], forced_exit=[exits[j]], keep_hidden=False)
        agree += int(o["tokens"][0]) == inp["gpu_toks"][j]
    dt = time.perf_counter() - t
    return {"value": round(ntok / dt, 4), "unit": "tokens/s", "ms_per_token": round(1e3 * dt / ntok, 2),
            "cores": threads, "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"fp64 NumPy oracle decoding {ntok} whole tokens: steps {inp['s0']}..{inp['s0'] + ntok - 1} "
                      f"of the timed run (positions {pos}..{pos + ntok - 1}, exit layers {exits}), each with "
                      f"the GPU's input token and shared cache; set-up (fp64 blocks, river quantisation) "
                      f"untimed; greedy tokens equal to the GPU's: {agree}/{ntok}"}


def cpu_block_sample(c, w, inp, threads, log):
    """Fallback: one backbone block, one river block and the LM head at the sampled position,
    scaled to a token by the sampled exit layers: t_tok = e*t_bb + (L-e)*t_river + t_head."""
    from oracle import river_oracle as O
    from token_level_early_amd import synth
    L = c["L"]
    lay = [0, 1]
    host = synth.to_numpy({"embed": w["embed"], "lm_head": w["lm_head"], "final_norm": w["final_norm"],
                           "layers": [w["layers"][i] if i in lay else None for i in range(L)]})
    orc = O.RiverOracle(c, host, layers=lay)
    pos = inp["pos"]
    Kc = [inp["kv"][l, 0].copy() for l in lay]
    Vc = [inp["kv"][l, 1].copy() for l in lay]
    h = host["embed"][inp["toks_in"][0]].copy()

    def timed(fn, reps):
        fn()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t) / reps

    def blk(i, W):
        K = np.concatenate([Kc[i], np.zeros_like(Kc[i][:, :1])], axis=1)
        V = np.concatenate([Vc[i], np.zeros_like(Vc[i][:, :1])], axis=1)
        return O.block_decode(c, W, orc.norms(i), h, pos, K, V)

    t_bb = timed(lambda: blk(0, orc.bb[0]), 3)
    t_rv = timed(lambda: blk(1, orc.rv[1]), 3)
    t_hd = timed(lambda: orc.head_logits(h), 3)
    e = float(np.mean(inp["exits"]))
    ms_tok = 1e3 * (e * t_bb + (L - e) * t_rv + t_hd)
    return {"value": round(1e3 / ms_tok, 4), "unit": "tokens/s", "ms_per_token": round(ms_tok, 2),
            "cores": threads, "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"fp64 NumPy oracle: backbone block (layer 1), river block (layer 2) and LM head "
                      f"at position {pos}, 3 reps each after one untimed call; token time = "
                      f"e*t_bb + (L-e)*t_river + t_head with e={e:.2f} (host memory too small for whole tokens)"}


if __name__ == "__main__":
    main()
