"""Throughput of the deterministic attention backward on one MI355X.

Workload: causal attention backward, B=1, H=32, S=8192, D=128, bf16 inputs
drawn from N(0,1) (seeded), O and LSE from the library's forward. One step is
one attn_bwd_deterministic call (preprocess D = rowsum(dO*O), main kernel,
dQ convert) with all inputs resident in HBM. Counted FLOPs per step follow the
usual attention-backward convention, 10*B*H*S^2*D, halved for causal.

Prints one JSON line. Progress goes to stderr.
"""
import argparse
import ctypes
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

CONFIGS = {
    # name: (B, H, S, D, causal, seed)
    "causal_b1_h32_s8192_d128": (1, 32, 8192, 128, True, 104),
    "full_b2_h32_s4096_d128": (2, 32, 4096, 128, False, 103),
    "causal_b4_h16_s2048_d64": (4, 16, 2048, 64, True, 102),
    "full_b1_h16_s16384_d128": (1, 16, 16384, 128, False, 105),
    "causal_b1_h16_s16384_d128": (1, 16, 16384, 128, True, 105),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles, so the library can record them around its main kernel."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


_C_TOKEN = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'', re.S)


def strip_c_comments(text):
    """C/C++ source without its comments (string and character literals kept)."""
    return _C_TOKEN.sub(lambda m: "" if m.group(0).startswith("/") else m.group(0), text)


def code_lines(text):
    """The code of a C/C++ source: comments removed, then blank lines and
    trailing blanks dropped, so a comment edit leaves it unchanged."""
    return "\n".join(line.rstrip() for line in strip_c_comments(text).splitlines() if line.strip())


def kernel_source_hash():
    """sha256 over the code of the HIP library sources (comments and blank lines
    never reach the binary): identifies the kernel build a profile was taken on."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "deterministic_attention_backward_fa_amd", "csrc")
    files = sorted(f for ext in ("*.h", "*.hip", "*.cpp") for f in glob.glob(os.path.join(csrc, ext)))
    files.append(os.path.join(ROOT, "include", "detattn.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(code_lines(open(f).read()).encode())
    return h.hexdigest()


def profiled_traffic(config_name):
    """HBM bytes per main-kernel launch from the committed rocprofv3 PMC summary of this
    workload, or None when there is none or the kernel sources changed since it was taken."""
    import re

    path = os.path.join(ROOT, "profiles", f"bwd_main_{config_name}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", open(path).read(), flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec


def counted_flops(B, H, S, D, causal):
    f = 10.0 * B * H * S * S * D
    return f / 2 if causal else f


def tiles_executed(plan, B, H, causal):
    n_q, n_kv, r = plan["n_q"], plan["n_kv"], plan["block_kv"] // plan["block_q"]
    per_head = sum((n_q - j * r) if causal else n_q for j in range(n_kv))
    return B * H * per_head


def warm_up(da, torch, tensors, shape, causal, sched, calls, **opts):
    """`calls` untimed calls of one schedule (own workspace and outputs)."""
    q, k, v, o, do, lse = tensors
    B, H, S, D = shape
    ws = da.alloc_workspace(B, H, S, D)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    for _ in range(calls):
        da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws, out=out, **opts)
    torch.cuda.synchronize()


def time_schedule(da, torch, ev, tensors, shape, causal, sched, steps, warmup, cold=False, **opts):
    """Warm (default): `steps` back-to-back calls between two events. Cold: before
    each call 512 MiB of scratch is overwritten, so no input or workspace byte
    is left in L2 or the Infinity Cache; each call is timed on its own (the
    overwrite is outside the timed events)."""
    q, k, v, o, do, lse = tensors
    B, H, S, D = shape
    ws = da.alloc_workspace(B, H, S, D)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    for _ in range(warmup):
        da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws, out=out, **opts)
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]
    begins = [ev.create() for _ in range(steps)]
    ends = [ev.create() for _ in range(steps)]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=q.device) if cold else None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    per_call = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)] \
        if cold else []
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        if cold:
            flush.fill_(s & 255)
            per_call[s][0].record()
        da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws, out=out,
                                  main_begin_event=begins[s], main_end_event=ends[s], **opts)
        if cold:
            per_call[s][1].record()
    t1.record()
    torch.cuda.synchronize()
    total_ms = sum(a.elapsed_time(b) for a, b in per_call) if cold else t0.elapsed_time(t1)
    del flush
    main_ms = [ev.elapsed_ms(b, e) for b, e in zip(begins, ends)]
    for e in begins + ends:
        ev.destroy(e)
    # bit equality of every timed call's outputs can only be seen at the end of
    # the timed loop (one set of output buffers); up to 10 further calls, untimed,
    # are each compared with the first warm-up result
    same = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(ref, out))
    for _ in range(min(steps, 10)):
        da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws, out=out, **opts)
        same = same and all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(ref, out))
    status = da.detattn_device_status(ws)
    srt = sorted(main_ms)
    return {"ms_per_step": total_ms / steps, "main_ms": sum(main_ms) / steps,
            "main_ms_median": srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2]),
            "main_ms_min": srt[0], "status": status, "repeat_bitwise": bool(same)}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg_shape, causal, seed, budget_s=15.0, max_heads=64):
    """The fp64 oracle (unchanged) on whole heads of the same workload until ~budget_s of CPU time."""
    import torch

    from deterministic_attention_backward_fa_amd.synth import make_qkvdo
    from oracle import ref

    B, H, S, D = cfg_shape
    q, k, v, do = make_qkvdo(B, H, S, D, seed)
    scale = 1.0 / math.sqrt(D)
    heads, elapsed = 0, 0.0
    while heads < min(max_heads, B * H) and elapsed < budget_s:
        b, h = divmod(heads, H)
        sl = [t[b:b + 1, h:h + 1] for t in (q, k, v, do)]
        t0 = time.perf_counter()
        ref.attn_bwd(*sl, scale, causal)
        elapsed += time.perf_counter() - t0
        heads += 1
        log(f"[cpu_baseline] oracle head {heads}: {elapsed:.1f} s cumulative")
    flops = counted_flops(1, heads, S, D, causal)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": ref.max_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"fp64 oracle backward (forward statistics recomputed) on {heads} of {B * H} heads "
                      f"(S={S}, D={D}, {'causal' if causal else 'full'}), {elapsed:.1f} s wall",
            "seconds": elapsed}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="causal_b1_h32_s8192_d128", choices=sorted(CONFIGS))
    ap.add_argument("--shape", default=None,
                    help="another workload instead of --config: B,H,S,D,full|causal (inputs seeded with 200)")
    ap.add_argument("--schedule", default=None, help="headline schedule (default: shift / symmetric_shift)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true", help="skip the other schedules")
    ap.add_argument("--dq-mode", default="default", choices=["default", "rmw", "atomic", "xcd_local"],
                    help="ordered dQ accumulation mechanism for the deterministic schedules")
    ap.add_argument("--block-q", type=int, default=0, help="Q tile rows (0 = library default)")
    ap.add_argument("--block-kv", type=int, default=0, help="KV tile rows (0 = library default)")
    ap.add_argument("--dispatch", default="default", choices=["default", "ticket", "ring"],
                    help="serial_ascending / descending_q / atomic_nondet: ticket counter or static rings")
    ap.add_argument("--ring-size", type=int, default=0,
                    help="workgroups per ring of the shift schedules (0 = library default)")
    ap.add_argument("--pair-columns", action="store_true",
                    help="symmetric shift with both columns of a pair item resident in registers (D = 64, 64x64 tiles)")
    ap.add_argument("--cold", action="store_true",
                    help="overwrite 512 MiB between timed calls (no input left in L2 or the Infinity Cache); "
                         "each call timed on its own")
    ap.add_argument("--cooperative-launch", action="store_true",
                    help="ring dispatch through HIP's cooperative launch instead of a plain launch")
    ap.add_argument("--trace", action="store_true", help="log the headline schedule's per-tile phase breakdown")
    ap.add_argument("--trace-gantt", action="store_true",
                    help="with --trace: also print a text timeline of the traced workgroups")
    ap.add_argument("--no-companion", action="store_true",
                    help="skip the full-mask companion workload of the default run")
    ap.add_argument("--xcd-study", action="store_true",
                    help="only measure the device-scope flag hand-off between workgroup pairs on one XCD and across XCDs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 3 x 1 GiB")
        return

    import deterministic_attention_backward_fa_amd as da
    from deterministic_attention_backward_fa_amd.synth import make_qkvdo

    if args.xcd_study:
        # workgroups w and w' share an XCD when w = w' (mod 8) under round-robin dispatch
        pairs = [(0, 8), (3, 11), (5, 13), (0, 1), (0, 4), (2, 7), (1, 6)]
        res = []
        for a, b in pairs:
            r = da.detattn_xcd_handoff(a, b, 8192)
            r.update(wg_a=a, wg_b=b, same_xcd=r["xcd_a"] == r["xcd_b"])
            res.append(r)
            log(f"[bench] hand-off wg {a} (XCD {r['xcd_a']}) <-> wg {b} (XCD {r['xcd_b']}): {r['ns']:.0f} ns, "
                f"{r['cycles']:.0f} cycles per round trip")
        same = [r["ns"] for r in res if r["same_xcd"] and not r["timed_out"]]
        cross = [r["ns"] for r in res if not r["same_xcd"] and not r["timed_out"]]
        print(json.dumps({"xcd_handoff": res, "round_trip_ns_same_xcd": sum(same) / len(same) if same else None,
                          "round_trip_ns_cross_xcd": sum(cross) / len(cross) if cross else None}), flush=True)
        return

    if args.shape:
        f = args.shape.split(",")
        if len(f) != 5 or f[4] not in ("full", "causal"):
            ap.error("--shape takes B,H,S,D,full|causal")
        B, H, S, D, causal, seed = int(f[0]), int(f[1]), int(f[2]), int(f[3]), f[4] == "causal", 200
        args.config = f"{f[4]}_b{B}_h{H}_s{S}_d{D}"
    else:
        B, H, S, D, causal, seed = CONFIGS[args.config]
    headline = args.schedule or ("symmetric_shift" if causal else "shift")
    log(f"[bench] {args.config}: generating inputs (seed {seed})")
    q, k, v, do = (t.cuda() for t in make_qkvdo(B, H, S, D, seed))
    o, lse = da.detattn_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    tensors = (q, k, v, o, do, lse)
    ev = HipEvents()
    scheds = [headline]
    if not args.only_headline:
        scheds += [s for s in (["serial_ascending", "descending_q"] +
                               (["symmetric_shift"] if causal else ["shift"]) + ["atomic_nondet"]) if s != headline]
    flops = counted_flops(B, H, S, D, causal)
    tile_opts = {k: v for k, v in (("block_q", args.block_q), ("block_kv", args.block_kv)) if v}
    results = {}
    def sched_opts(sched):
        opts = {"dq_mode": args.dq_mode} if (args.dq_mode != "default" and sched != "atomic_nondet") else {}
        opts.update(tile_opts)
        if args.ring_size and sched in ("shift", "symmetric_shift"):
            opts["ring_size"] = args.ring_size
        if args.dispatch != "default" and sched in ("serial_ascending", "descending_q", "atomic_nondet"):
            opts["dispatch"] = args.dispatch
        if args.pair_columns and sched == "symmetric_shift":
            opts["pair_columns"] = True
        if args.cooperative_launch:
            opts["cooperative_launch"] = True
        return opts

    # Every schedule runs its warm-up calls before any schedule is timed: the
    # schedule timed first otherwise measured 2-4% slower than the same
    # schedule timed after the others (the device was still warming up).
    for sched in scheds:
        warm_up(da, torch, tensors, (B, H, S, D), causal, sched, args.warmup, **sched_opts(sched))
    for sched in scheds:
        log(f"[bench] timing {sched}: warmup {args.warmup}, steps {args.steps}")
        opts = sched_opts(sched)
        r = time_schedule(da, torch, ev, tensors, (B, H, S, D), causal, sched, args.steps, args.warmup,
                          cold=args.cold, **opts)
        r["tflops"] = flops / (r["ms_per_step"] * 1e-3) / 1e12
        results[sched] = r
        log(f"[bench] {sched}: {r['ms_per_step']:.3f} ms/step, main {r['main_ms']:.3f} ms, "
            f"{r['tflops']:.1f} TFLOP/s, status {r['status']}, repeat bitwise {r['repeat_bitwise']}")
    head = results[headline]
    plan_opts = sched_opts(headline)
    plan = da.detattn_bwd_plan(B, H, S, D, causal, headline, **plan_opts)
    tiles = tiles_executed(plan, B, H, causal)
    algo_flops = 10.0 * plan["block_q"] * plan["block_kv"] * D * tiles
    achieved = algo_flops / (head["main_ms"] * 1e-3) / 1e12
    atomic = results.get("atomic_nondet")
    traffic = profiled_traffic(args.config) if not plan_opts and not args.cold else None  # taken warm, default plan
    line = {
        "metric": "deterministic attn-bwd TFLOP/s (bf16, full+causal) and ratio vs atomic nondet",
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{'causal' if causal else 'full'} attention backward B={B} H={H} S={S} D={D}",
                   "schedule": headline, "block_q": plan["block_q"], "block_kv": plan["block_kv"],
                   "grid": plan["grid"], "ring": plan["ring"], "parallelism": "single GPU",
                   "caches": "cold (512 MiB overwritten before each call)" if args.cold else "warm"},
        "ratio_vs_atomic": round(head["tflops"] / atomic["tflops"], 4) if atomic else None,
        "ratio_vs_atomic_note": ("the atomic reference is bound by device-scope fp32 atomic adds (about 1.35 TB/s "
                                 "of dQ partials), so this ratio says little about the cost of ordering; "
                                 "roofline.frac is the binding target"),
        "schedules": {s: {"tflops": round(r["tflops"], 2), "ms_per_step": round(r["ms_per_step"], 4),
                          "main_ms": round(r["main_ms"], 4), "main_ms_median": round(r["main_ms_median"], 4),
                          "main_ms_min": round(r["main_ms_min"], 4), "repeat_bitwise": r["repeat_bitwise"],
                          "ratio_vs_atomic": round(r["tflops"] / atomic["tflops"], 4) if atomic else None}
                      for s, r in results.items()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                     "traffic_detail": traffic,
                     "kernel": "bwd_main_kernel", "algorithmic_flops_per_launch": algo_flops,
                     "avg_launch_ms": round(head["main_ms"], 4),
                     "median_launch_ms": round(head["main_ms_median"], 4),
                     "min_launch_ms": round(head["main_ms_min"], 4)},
    }
    if args.trace:
        from deterministic_attention_backward_fa_amd import trace as dtrace

        recs, _ = dtrace.collect(da, tensors, causal, headline, **sched_opts(headline))
        summ = dtrace.summarize(recs)
        log(f"[bench] trace {headline}: tile period median {summ['tile_period_median']:.0f} ticks, "
            f"{summ['early_turn_fraction'] * 100:.0f}% of tiles find their turn at the dS^T barrier "
            f"({summ['workgroups']} WGs)")
        for name, share in summ["share"].items():
            log(f"[bench]   {share * 100:5.1f}%  {summ['ticks'][name]:8.0f}  {name}")
        log("[bench] traced span: " + ", ".join(f"{k} {v * 100:.1f}%" for k, v in summ["span_share"].items()))
        line["trace_share"] = {k: round(v, 4) for k, v in summ["share"].items()}
        line["trace_span_share"] = {k: round(v, 4) for k, v in summ["span_share"].items()}
        if args.trace_gantt:
            log(f"[bench] timeline of {headline} ('#' tile compute, 'w' waiting for the dQ turn, "
                f"'e' column switch, 's' start-up (registration, first K/V), ' ' idle; one row per workgroup):")
            log(dtrace.gantt(recs))
    # The metric covers both masks: the default run also times the full-mask
    # workload (every schedule) and reports it beside the causal headline.
    default_run = (not args.shape and args.config == "causal_b1_h32_s8192_d128" and not args.only_headline
                   and not tile_opts and not args.ring_size and args.dispatch == "default"
                   and args.dq_mode == "default" and not args.schedule and not args.pair_columns
                   and not args.cooperative_launch and not args.cold)
    if default_run and not args.no_companion:
        cB, cH, cS, cD, ccausal, cseed = CONFIGS["full_b2_h32_s4096_d128"]
        log(f"[bench] companion full_b2_h32_s4096_d128: generating inputs (seed {cseed})")
        cq, ck, cv, cdo = (t.cuda() for t in make_qkvdo(cB, cH, cS, cD, cseed))
        co, clse = da.detattn_fwd(cq, ck, cv, causal=ccausal)
        torch.cuda.synchronize()
        cflops = counted_flops(cB, cH, cS, cD, ccausal)
        cres = {}
        for sched in ("shift", "serial_ascending", "descending_q", "atomic_nondet"):
            warm_up(da, torch, (cq, ck, cv, co, cdo, clse), (cB, cH, cS, cD), ccausal, sched, args.warmup)
        for sched in ("shift", "serial_ascending", "descending_q", "atomic_nondet"):
            r = time_schedule(da, torch, ev, (cq, ck, cv, co, cdo, clse), (cB, cH, cS, cD), ccausal, sched, args.steps,
                              args.warmup)
            r["tflops"] = cflops / (r["ms_per_step"] * 1e-3) / 1e12
            cres[sched] = r
            log(f"[bench] companion {sched}: {r['ms_per_step']:.3f} ms/step, {r['tflops']:.1f} TFLOP/s, "
                f"status {r['status']}, repeat bitwise {r['repeat_bitwise']}")
        ca = cres["atomic_nondet"]["tflops"]
        line["full_mask"] = {
            "workload": f"full attention backward B={cB} H={cH} S={cS} D={cD}", "schedule": "shift",
            "value": round(cres["shift"]["tflops"], 2), "unit": "TFLOP/s",
            "ratio_vs_atomic": round(cres["shift"]["tflops"] / ca, 4),
            "schedules": {k_: {"tflops": round(r["tflops"], 2), "ms_per_step": round(r["ms_per_step"], 4),
                               "repeat_bitwise": r["repeat_bitwise"], "ratio_vs_atomic": round(r["tflops"] / ca, 4)}
                          for k_, r in cres.items()}}
        del cq, ck, cv, cdo, co, clse
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: fp64 oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline((B, H, S, D), causal, seed)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
