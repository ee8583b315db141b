#!/usr/bin/env python3
"""Benchmark of the MTGR HSTU layer on one MI355X.

One step = the whole hot path over one batch: jagged segments, input Group
LayerNorm, UQKV projection + SiLU, masked SiLU attention, GroupNorm(AV) * U,
output projection + residual, and the backward of all of it (dQ, dK, dV,
dU, dGLN and every weight gradient).  Workload: a token-balanced bf16 batch
of exactly 65,536 tokens of long-tail users (history lognormal(6, 1) clipped
to [32, 3000], 0-64 real-time tokens, 20 candidates), d_model 1024, 8 heads
of 128, seeded synthetic data with random-init weights.

Prints one JSON line.  ``value`` is the attention throughput (forward +
backward algorithmic flops, 12 d P for P mask-visible pairs, over the summed
duration of the attention kernels measured with HIP events on their stream
inside the timed steps); ``users_per_sec`` is whole-step throughput.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU-oracle baseline sample (0 disables it)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--serving", action="store_true",
                    help="time the 22-layer fp16 one-request serving forward per candidate count instead "
                         "(eager layer calls, one stack call, graph replay)")
    ap.add_argument("--requests", type=int, default=200, help="timed requests per K and mode (--serving)")
    ap.add_argument("--head", action="store_true",
                    help="time the candidate head with its loss and backward on the 65,536-token batch")
    ap.add_argument("--forward-batches", action="store_true",
                    help="users/s of the forward-only workloads: one bf16 d_model 512 layer over 32 users, and the "
                         "22-layer fp16 d_model 1024 stack over 64 users (one graph)")
    ap.add_argument("--stochastic-length", type=int, default=0, metavar="S_KEEP",
                    help="time Stochastic Length sampling (histories cut to S_KEEP tokens) of a long-tail user "
                         "pool and the layer step on the 65,536-token batch cut from it, against the batch "
                         "without sampling")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after the timed steps, copy MIB MiB device-to-device 3 times (a plain copy kernel "
                         "of known size, the calibration for HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="offline: summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --copy-probe N' into profiles/traffic.json and a markdown table")
    ap.add_argument("--counter-summary", nargs="+", metavar="PMC_DIR",
                    help="offline: per-kernel table of rocprofv3 --pmc runs (SQ_* and GRBM_GUI_ACTIVE counters of "
                         "'bench.py --steps 3 --warmup 1 --cpu-seconds 0') with MFMA-busy and vector-ALU fractions")
    ap.add_argument("--stats-summary", metavar="STATS_CSV",
                    help="offline: turn a rocprofv3 --stats kernel_stats.csv into a markdown table on stdout")
    ap.add_argument("--probe-mib", type=int, default=256, help="copy size used by --pmc-summary")
    return ap.parse_args()


def profile_summary(lib):
    n = 64
    names = (ctypes.c_char_p * n)()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    lib.mtgr_profile_summary.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
    k = lib.mtgr_profile_summary(n, names, ms, cnt)
    if k < 0:
        raise RuntimeError(f"mtgr_profile_summary failed: {k}")
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(k, n))}


def kernel_work(T, d, P, ds_bytes):
    """Algorithmic work of one launch of each kernel step: (bound, amount)
    with flops for MFMA-bound steps and HBM bytes for streaming ones."""
    e = 2  # bf16 bytes
    return {
        "attn_fwd": ("mfma", 4 * d * P),
        "attn_bwd_dkdv": ("mfma", 6 * d * P),   # dV, dA = dO V^T, dK
        # dQ = dS K from stored dS: streams dS, reads K and the SiLU' factor of Q, writes dQ
        "attn_bwd_dq": ("hbm", ds_bytes + 3 * T * d * e),
        "gemm_uqkv_silu": ("mfma", 8 * T * d * d),
        "gemm_out_resid": ("mfma", 2 * T * d * d),
        "gemm_dy": ("mfma", 2 * T * d * d),
        "gemm_dW_o": ("mfma", 2 * T * d * d),
        "gemm_dxhat": ("mfma", 8 * T * d * d),
        "gemm_dW_uqkv": ("mfma", 8 * T * d * d),
        "gln1_fwd": ("hbm", T * (2 * e * d + 9)),
        "gln2_gate_fwd": ("hbm", T * (3 * e * d + 9)),
        "gln2_gate_bwd": ("hbm", T * (6 * e * d + 9)),
        "gln1_bwd": ("hbm", T * (4 * e * d + 9)),
    }


# HIP kernel name fragments -> kernel step names used in the JSON line
KERNEL_STEPS = [
    ("attn_bwd_dkdv_mfma", "attn_bwd_dkdv"),
    ("attn_bwd_dq_stream", "attn_bwd_dq"),
    ("attn_fwd_mfma", "attn_fwd"),
]


def _pmc_rows(d):
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _per_dispatch(rows, counter):
    """{kernel name: [value per dispatch]} for one counter (summed over the
    dimensions rocprofv3 reports it in)."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in acc.items():
        out.setdefault(name, []).append(v)
    return out


def code_hash(text):
    """SHA-256 of C++ source with comments and whitespace removed: an edit to
    a comment leaves it unchanged, an edit to the code does not."""
    import hashlib
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def attn_source_hash():
    """Hash of the attention kernels' code: counters taken on other code are stale."""
    path = os.path.join(ROOT, "generative_recommendation_ranking_grouplayernorm_amd", "csrc", "attn.hip")
    return code_hash(open(path).read())


def pmc_summary(fetch_dir, write_dir, probe_mib):
    """Per-launch HBM traffic of the attention kernels from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the ratio of the bytes a
    plain device copy of probe_mib MiB moves to what the same counter reads
    for it."""
    fetch = _per_dispatch(_pmc_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_pmc_rows(write_dir), "WRITE_SIZE")
    nbytes = probe_mib * 1024 * 1024

    def copy_kib(tab):
        # the probe's dispatches: copy-kernel launches that move at least half the probe size
        # (the same kernel also serves the small copies of the timed steps)
        cands = {k: [x for x in v if x * 1024 > 0.5 * nbytes] for k, v in tab.items() if "copy" in k.lower()}
        cands = {k: v for k, v in cands.items() if v}
        if not cands:
            raise SystemExit("copy probe kernel not found in the counter runs")
        k = max(cands, key=lambda n: len(cands[n]))
        vals = sorted(cands[k])
        return k, vals[len(vals) // 2]

    ck, cf = copy_kib(fetch)
    _, cw = copy_kib(write)
    f_scale = nbytes / (cf * 1024)
    w_scale = nbytes / (cw * 1024)
    res = {"_calibration": {"copy_kernel": ck, "copy_bytes": nbytes, "fetch_kib": cf, "write_kib": cw,
                            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
           "_source_sha256": attn_source_hash()}
    lines = ["| kernel step | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |",
             "|---|---|---|---|---|"]
    for frag, step in KERNEL_STEPS:
        fk = [k for k in fetch if frag in k]
        wk = [k for k in write if frag in k]
        if not fk or not wk:
            continue
        fv = [v for k in fk for v in fetch[k]]
        wv = [v for k in wk for v in write[k]]
        f_avg, w_avg = sum(fv) / len(fv), sum(wv) / len(wv)
        tot = f_avg * 1024 * f_scale + w_avg * 1024 * w_scale
        res[step] = round(tot)
        lines.append(f"| {step} | {len(fv)} | {f_avg:.0f} | {w_avg:.0f} | {tot / 1e9:.3f} GB |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(res, f, indent=1)
    print("\n".join(lines))
    print(f"\ncalibration: {ck} moving {nbytes} B reads FETCH_SIZE {cf:.0f} KiB (scale {f_scale:.4f}), "
          f"WRITE_SIZE {cw:.0f} KiB (scale {w_scale:.4f})")


def counter_summary(dirs):
    """Per-kernel averages of SQ_* / GRBM_GUI_ACTIVE counters from rocprofv3
    --pmc runs, with derived fractions.  On this part the SQ and GRBM
    counters cover half of the chip (4 of the 8 XCDs): SQ_INSTS_MFMA of the
    UQKV projection reads exactly half of its known instruction count
    (8 T d^2 / 32768), so instruction counts are doubled and GRBM_GUI_ACTIVE
    (summed over the 4 counted XCDs) divided by 4 gives the clock cycles of
    the dispatch.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (512 counted SIMDs
    x cycles); the vector-ALU issue estimate counts 4 cycles per plain and 8
    per transcendental wave instruction (measured issue costs of one wave)."""
    import collections
    import csv
    import glob
    import re

    rows = []
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += list(csv.DictReader(open(f)))
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = collections.defaultdict(dict)
    for r in rows:
        # one template instance serves several products: tell them apart by grid size
        k = (r["Kernel_Name"], int(r["Grid_Size"]))
        acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[k][(r["Dispatch_Id"], r["Process_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])

    def short(k):
        name, grid = k
        m = re.search(r"mtgr(?:\d+|::)(\w+?)(?:I|<)", name)
        base = m.group(1) if m else name[:40]
        e = re.search(r"(true|false), (\d), mtgr::GemmCfg", name) or re.search(r"Lb(\d)ELi(\d)ENS_7GemmCfg", name)
        if e:
            base += f" epi {e.group(2)}"
        return f"{base}, grid {grid}"

    print("| kernel | dispatches | avg us | clock GHz | MFMA instr | executed TFLOP/s | MFMA busy | VALU instr "
          "(trans) | VALU issue est. | LDS instr | LDS bank-conflict cycles | wait / wave cycles |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for k in sorted(acc, key=lambda k: -sum(dur[k].values()) / len(dur[k])):
        n = len(dur[k])
        a = {c: v / n for c, v in acc[k].items()}
        ns = sum(dur[k].values()) / n
        cyc = a.get("GRBM_GUI_ACTIVE", 0) / 4
        if cyc <= 0 or ns <= 0:
            continue
        mfma = 2 * a.get("SQ_INSTS_MFMA", 0)
        valu = 2 * a.get("SQ_INSTS_VALU", 0)
        trans = 2 * a.get("SQ_INSTS_VALU_TRANS_F32", 0)
        busy = a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (512 * cyc)
        valu_est = ((valu - trans) * 4 + trans * 8) / (1024 * cyc)
        wait = a.get("SQ_WAIT_ANY", 0) / a["SQ_WAVE_CYCLES"] if a.get("SQ_WAVE_CYCLES") else float("nan")
        print(f"| `{short(k)}` | {n // 2} | {ns / 1e3:.1f} | {cyc / ns:.2f} | {mfma:.3g} | "
              f"{mfma * 32768 / (ns * 1e-9) / 1e12:.0f} | {busy:.3f} | {valu:.3g} ({trans:.2g}) | {valu_est:.3f} | "
              f"{2 * a.get('SQ_INSTS_LDS', 0):.3g} | {2 * a.get('SQ_LDS_BANK_CONFLICT', 0):.3g} | {wait:.3f} |")


def stats_summary(path):
    import csv

    rows = list(csv.DictReader(open(path)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    print("| kernel | calls | total us | avg us | % |")
    print("|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        name = name if len(name) <= 110 else name[:107] + "..."
        print(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
              f"{float(r['AverageNs']) / 1e3:.1f} | {100 * float(r['TotalDurationNs']) / tot:.1f} |")


def cpu_baseline(batch, params, x, R, budget_s):
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole users in batch order until the time budget is spent."""
    import numpy as np

    from generative_recommendation_ranking_grouplayernorm_amd import flops as fl
    from oracle import mtgr_oracle as orc

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    p = params[0]
    scale = 1.0 / batch.max_len
    attn_t = layer_t = 0.0
    attn_f = 0
    users = 0
    toks = 0
    for b in range(batch.B):
        off, g, ts, xs, rows = orc.select_users(batch.offsets, batch.group_ids, batch.timestamps, x, [b])
        d = x.shape[1]
        rng = np.random.default_rng(b)
        q, k, v, do = (rng.normal(0, 0.35, size=(len(rows), d)) for _ in range(4))
        t0 = time.perf_counter()
        orc.hstu_attention(q, k, v, off, g, ts, p.H, 1.0, scale)
        orc.hstu_attention_bwd(q, k, v, do, off, g, ts, p.H, 1.0, scale)
        t1 = time.perf_counter()
        out, sv = orc.layer_fwd(p, xs, off, g, ts, 1.0, scale)
        orc.layer_bwd(p, xs, sv, R[rows], off, g, ts, 1.0, scale)
        t2 = time.perf_counter()
        attn_t += t1 - t0
        layer_t += t2 - t1
        fwd, bwd = fl.attention_flops(off, g, ts, d)
        attn_f += fwd + bwd
        users += 1
        toks += len(rows)
        if attn_t + layer_t >= budget_s:
            break
    return {
        "value": attn_f / attn_t / 1e12,
        "unit": "TFLOP/s",
        "cores": int(min(threads, cores)),
        "cores_available": int(cores),
        "blas_threads": int(threads),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": f"first {users} users ({toks} tokens) of the same 65,536-token batch, fp64 NumPy: "
                  f"attention fwd+bwd timed alone ({attn_t:.2f} s), then the whole layer fwd+bwd "
                  f"({layer_t:.2f} s)",
        "users_per_sec": users / layer_t,
    }


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.probe_mib)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU path is a "
              f"design note, not part of this build.", file=sys.stderr)
        sys.exit(2)
    if args.serving:
        serving_bench(args)
        return
    if args.stochastic_length > 0:
        sl_bench(args)
        return
    if args.head:
        head_bench(args)
        return
    if args.forward_batches:
        forward_batches_bench(args)
        return
    import numpy as np
    import torch

    import generative_recommendation_ranking_grouplayernorm_amd.binding as mb
    from generative_recommendation_ranking_grouplayernorm_amd import flops as fl
    from mtgr_inputs import CONFIGS, config_inputs

    cfg_id = 4
    cfg = CONFIGS[cfg_id]
    dev = torch.device("cuda:0")
    lib = mb.load_library()
    batch, params, x = config_inputs(cfg_id, seed=args.seed)
    p = params[0]
    d, H, G = cfg["d"], cfg["H"], 4
    T, B = batch.T, batch.B
    dt = torch.bfloat16
    rng = np.random.default_rng([args.seed, cfg_id, 3])
    R = rng.normal(0, 1, size=(T, d)).astype(np.float32)
    scale = 1.0 / batch.max_len

    def to(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(dev)

    dev_p = {k: to(getattr(p, k)) for k in ("W_uqkv", "gamma1", "beta1", "gamma2", "beta2", "W_o")}
    xd, Rd = to(x), to(R)
    off = torch.from_numpy(batch.offsets).to(dev)
    g = torch.from_numpy(batch.group_ids).to(dev)
    ts = torch.from_numpy(batch.timestamps).to(dev)
    prm = mb.make_params(dev_p, H)
    saved = mb.alloc_saved(T, d, dt, dev)
    sv = mb.make_saved(saved)
    x_out = torch.empty(T, d, dtype=dt, device=dev)
    dx = torch.empty(T, d, dtype=dt, device=dev)
    grads = mb.alloc_grads(d, G, False, dev)
    ws_f = mb.workspace(mb.OP_LAYER_FWD, B, T, d, H, dt, dev)
    # a row-length bound sizes the backward for stored score gradients
    ws_b = mb.workspace(mb.OP_LAYER_BWD, B, T, d, H, dt, dev, max_len=batch.max_len)
    stream = torch.cuda.current_stream()

    def step():
        mb.mtgr_hstu_layer_fwd(prm, xd, x_out, sv, off, g, ts, scale, ws_f, stream)
        mb.mtgr_hstu_layer_bwd(prm, xd, sv, Rd, dx, grads, off, g, ts, scale, ws_b, max_len=batch.max_len,
                               stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps), timing {args.steps} steps", file=sys.stderr, flush=True)
    lib.mtgr_profile_enable(1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_total = ev[0].elapsed_time(ev[-1])
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    prof = profile_summary(lib)
    lib.mtgr_profile_enable(0)
    ms_step = ms_total / args.steps
    if args.copy_probe > 0:
        n = args.copy_probe * 1024 * 1024 // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: 3 x {args.copy_probe} MiB device-to-device", file=sys.stderr, flush=True)
        del src, dst

    P = fl.visible_pairs(batch.offsets, batch.group_ids, batch.timestamps)
    attn_flops = 12 * d * P
    attn_ms = sum(prof.get(k, (0.0, 0))[0]
                  for k in ("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dq_rest")) / args.steps
    value = attn_flops / (attn_ms / 1e3) / 1e12
    layer_flops = 12 * d * P + fl.layer_gemm_flops(T, d, backward=True)

    work = kernel_work(T, d, P, fl.ds_stream_bytes(batch.offsets, batch.group_ids, H))
    kernels = {}
    for name, (tot, n) in prof.items():
        avg = tot / max(n, 1)
        ent = {"avg_ms": round(avg, 5), "launches": n, "ms_per_step": round(tot / args.steps, 5)}
        if name in work:
            bound, amount = work[name]
            if bound == "mfma":
                ach = amount / (avg / 1e3) / 1e12
                ent.update(bound="mfma", achieved=round(ach, 2), unit="TFLOP/s", frac=round(ach / BF16_PEAK_TFLOPS, 4))
            else:
                ach = amount / (avg / 1e3) / 1e9
                ent.update(bound="hbm", achieved=round(ach, 1), unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4))
        kernels[name] = ent
    dom = max((k for k in kernels if "bound" in kernels[k]), key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        try:
            tj = json.load(open(tpath))
            # counters describe the kernels they were taken on
            traffic = tj.get(dom) if tj.get("_source_sha256") == attn_source_hash() else None
        except Exception:
            traffic = None
    roofline = {"kernel": dom, "bound": dk["bound"], "achieved": dk["achieved"],
                "peak": BF16_PEAK_TFLOPS if dk["bound"] == "mfma" else HBM_PEAK_GBS,
                "unit": dk["unit"], "frac": dk["frac"], "traffic": traffic}

    gln = gln_rotated(mb, T, d, G, dt, dev, stream)

    cpu = None
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(batch, params, x, R, args.cpu_seconds)

    out = {
        "metric": "fused jagged HSTU attn TFLOP/s (fwd+bwd, bf16, d=1024) + users/sec on 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": {"min": round(step_ms[0], 4), "median": round(step_ms[len(step_ms) // 2], 4),
                    "p90": round(step_ms[min(len(step_ms) - 1, (9 * len(step_ms)) // 10)], 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded long-tail jagged users, random-init weights)",
        "config": {"workload": "MTGR HSTU layer fwd+bwd, token-balanced batch", "tokens": T, "users": B,
                   "d_model": d, "heads": H, "head_dim": d // H, "max_len": batch.max_len,
                   "visible_pairs": P, "parallelism": "single GPU"},
        "users_per_sec": round(B / (ms_step / 1e3), 1),
        "attn_ms_per_step": round(attn_ms, 4),
        "attn_frac_of_bf16_peak": round(value / BF16_PEAK_TFLOPS, 4),
        "layer_tflops": round(layer_flops / (ms_step / 1e3) / 1e12, 2),
        "roofline": roofline,
        "kernels": kernels,
        "gln_hbm_rotated": gln,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def gln_rotated(mb, T, d, G, dt, dev, stream, sets=4, reps=3):
    """Group LayerNorm forward and backward through the C ABI on the layer's
    [T, d] shape, each launch on the next of ``sets`` distinct buffer sets
    (together larger than the 256 MB last-level cache, so every launch reads
    from HBM), HIP events around each launch on the stream it runs on.
    Bytes per launch: forward x in, y out, mean/rstd out (+ group id);
    backward dy and x in, dx out, mean/rstd and group id in (the per-group
    gamma/beta sums are a few KB)."""
    import torch

    e = 2
    gen = torch.Generator(device=dev).manual_seed(0)
    g = torch.randint(0, G, (T,), generator=gen, device=dev, dtype=torch.int64).sort().values.to(torch.uint8)
    gam = torch.ones(G, d, dtype=dt, device=dev)
    bet = torch.zeros(G, d, dtype=dt, device=dev)
    bufs = []
    for _ in range(sets):
        x = torch.randn(T, d, generator=gen, device=dev).to(dt)
        bufs.append(dict(x=x, y=torch.empty_like(x), dy=torch.randn(T, d, generator=gen, device=dev).to(dt),
                         dx=torch.empty_like(x), mean=torch.empty(T, device=dev), rstd=torch.empty(T, device=dev)))
    dg = torch.empty(G, d, device=dev)
    db = torch.empty(G, d, device=dev)
    ws = mb.workspace(mb.OP_GLN_BWD, 0, T, d, 1, dt, dev)
    times = {"fwd": [], "bwd": []}
    for r in range(reps + 1):
        for b in bufs:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(stream)
            mb.mtgr_group_layernorm(b["x"], b["y"], gam, bet, g, 1e-5, b["mean"], b["rstd"], stream=stream)
            ev[1].record(stream)
            mb.mtgr_group_layernorm_bwd(b["dy"], b["x"], b["mean"], b["rstd"], gam, g, b["dx"], dg, db, ws,
                                        stream=stream)
            ev[2].record(stream)
            torch.cuda.synchronize()
            if r > 0:  # the first round warms up
                times["fwd"].append(ev[0].elapsed_time(ev[1]))
                times["bwd"].append(ev[1].elapsed_time(ev[2]))
    nbytes = {"fwd": T * (2 * e * d + 8 + 1), "bwd": T * (3 * e * d + 8 + 1)}
    out = {"buffer_sets": sets, "set_bytes": int(sets and 4 * T * d * e + 8 * T), "launches": reps * sets}
    for k in ("fwd", "bwd"):
        ms = sorted(times[k])[len(times[k]) // 2]
        gbs = nbytes[k] / (ms / 1e3) / 1e9
        out[k] = {"median_ms": round(ms, 5), "bytes": nbytes[k], "GB/s": round(gbs, 1),
                  "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def serving_bench(args):
    """One request (one user, 1000 history tokens, 32 real-time tokens, K
    candidates) through 22 fp16 layers of d_model 1024, per K in the sweep.
    Three ways to issue it: 22 single-layer calls from Python, one stack
    call, one graph launch; and the graph of the whole request (layers and
    the candidate head's logits, 1024 -> 512 -> 2 tasks).  Latency = host clock from the first call to the
    end of a stream synchronisation, one request at a time; throughput =
    requests issued back to back on one stream, then one synchronisation.
    GPU time = the summed kernel durations of one request (HIP events around
    every kernel step, a separate pass)."""
    import numpy as np
    import torch

    import generative_recommendation_ranking_grouplayernorm_amd.binding as mb
    from generative_recommendation_ranking_grouplayernorm_amd import flops as fl
    from mtgr_inputs import CONFIGS, config_inputs

    cfg_id = 5
    cfg = CONFIGS[cfg_id]
    dev = torch.device("cuda:0")
    lib = mb.load_library()
    dt = torch.float16
    d, H, L = cfg["d"], cfg["H"], cfg["layers"]
    _, params, _ = config_inputs(cfg_id, seed=args.seed)

    def to(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(dev)

    keep = [{k: to(getattr(p, k)) for k in ("W_uqkv", "gamma1", "beta1", "gamma2", "beta2", "W_o")}
            for p in params]
    lps = [mb.make_params(t, H) for t in keep]
    from mtgr_inputs import make_head_params

    hp = make_head_params(d, 512, 2, np.random.default_rng([args.seed, 5, 77]), True)
    hdev = {k: to(getattr(hp, k)) for k in ("W1", "b1", "W2", "b2")}
    hprm = mb.make_head_params(hdev)
    stream = torch.cuda.current_stream()
    n = max(args.requests, 10)
    results = {}
    for K in cfg["K_sweep"]:
        batch, _, x = config_inputs(cfg_id, seed=args.seed, K=K)
        T = batch.T
        scale = 1.0 / batch.max_len
        xd = to(x)
        y = torch.empty_like(xd)
        off = torch.from_numpy(batch.offsets).to(dev)
        g = torch.from_numpy(batch.group_ids).to(dev)
        ts = torch.from_numpy(batch.timestamps).to(dev)
        ws_l = mb.workspace(mb.OP_LAYER_FWD, 1, T, d, H, dt, dev)
        ws_s = mb.workspace(mb.OP_STACK_FWD, 1, T, d, H, dt, dev)
        h2 = torch.empty_like(xd)
        graph = mb.mtgr_stack_graph_create(lps, xd, y, off, g, ts, scale, ws_s)
        logits = torch.empty(K, 2, device=dev)
        ws_h = mb.head_workspace(1, K, d, 512, 2, dt, dev)
        ws_s2 = mb.workspace(mb.OP_STACK_FWD, 1, T, d, H, dt, dev)
        y2 = torch.empty_like(xd)
        graph_h = mb.mtgr_serving_graph_create(lps, hprm, xd, y2, logits, K, off, g, ts, scale, ws_s2, ws_h)

        def layers():
            src, dst = xd, (y if L % 2 == 1 else h2)
            for i, lp in enumerate(lps):
                mb.mtgr_hstu_layer_fwd(lp, src, dst, None, off, g, ts, scale, ws_l, stream)
                src, dst = dst, (h2 if dst is y else y)

        def stack():
            mb.mtgr_hstu_stack_fwd(lps, xd, y, off, g, ts, scale, ws_s, stream)

        def replay():
            graph.launch(stream)

        def replay_head():
            graph_h.launch(stream)

        modes = {"layer_calls": layers, "stack_call": stack, "graph": replay, "graph_with_head": replay_head}
        res = {}
        for name, fn in modes.items():
            for _ in range(max(args.warmup, 3)):
                fn()
            torch.cuda.synchronize()
            lat = []
            for _ in range(n):
                t0 = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                lat.append((time.perf_counter() - t0) * 1e3)
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            thr = n / (time.perf_counter() - t0)
            lat = np.array(lat)
            res[name] = {"p50_ms": round(float(np.percentile(lat, 50)), 4),
                         "p99_ms": round(float(np.percentile(lat, 99)), 4),
                         "mean_ms": round(float(lat.mean()), 4),
                         "requests_per_sec": round(thr, 1)}
        # kernel time of one request, measured on the eager stack call
        lib.mtgr_profile_enable(1)
        for _ in range(5):
            stack()
        torch.cuda.synchronize()
        prof = profile_summary(lib)
        lib.mtgr_profile_enable(0)
        res["gpu_ms_per_request"] = round(sum(v[0] for v in prof.values()) / 5, 4)
        res["kernels_ms_per_request"] = {k: round(v[0] / 5, 4) for k, v in sorted(prof.items())}
        P = fl.visible_pairs(batch.offsets, batch.group_ids, batch.timestamps)
        res["tokens"] = T
        res["fwd_gflop"] = round(L * (4 * d * P + fl.layer_gemm_flops(T, d, backward=False)) / 1e9, 2)
        graph.close()
        graph_h.close()
        results[K] = res
        print(f"[bench] K={K}: " + ", ".join(f"{m} p50 {res[m]['p50_ms']} ms" for m in modes),
              file=sys.stderr, flush=True)
    g20 = results[min(results)]
    out = {
        "metric": "serving request latency, 22-layer fp16 forward, one request",
        "value": g20["graph"]["p50_ms"],
        "unit": "ms (P50, K=20, graph replay)",
        "n_gpus": 1,
        "requests": n,
        "higher_is_better": False,
        "dtype": "f16",
        "data": "synthetic (seeded request, random-init weights)",
        "config": {"workload": "MTGR serving forward, 1 user x (8 profile + 1000 history + 32 real-time + K "
                               "candidates), 22 layers, d_model 1024, 8 heads of 128",
                   "K_sweep": list(results)},
        "per_K": results,
    }
    print(json.dumps(out))


def sl_bench(args):
    """Stochastic Length: a pool of long-tail users (four times the budget)
    has each history cut to a random window of S_KEEP tokens and the longest
    prefix within 65,536 tokens becomes the training batch.  Reports the
    sampling kernels' time (HIP events, median of repeated calls) and
    bandwidth, and the layer forward + backward on that batch against the
    token-balanced batch of the same budget without sampling."""
    import numpy as np
    import torch

    import generative_recommendation_ranking_grouplayernorm_amd.binding as mb
    from generative_recommendation_ranking_grouplayernorm_amd import flops as fl
    from mtgr_inputs import CONFIGS, config_inputs, make_uniform_draws, make_user_pool

    cfg_id, budget, s_keep = 4, 65536, args.stochastic_length
    cfg = CONFIGS[cfg_id]
    dev = torch.device("cuda:0")
    lib = mb.load_library()
    dt = torch.bfloat16
    d, H = cfg["d"], cfg["H"]
    pool = make_user_pool(cfg_id, 4 * budget, seed=args.seed)
    u = torch.from_numpy(make_uniform_draws(pool.B, seed=args.seed)).to(dev)
    gen = torch.Generator(device="cpu").manual_seed(args.seed)
    x = torch.randn(pool.T, d, generator=gen).to(dt).to(dev)
    off = torch.from_numpy(pool.offsets).to(dev)
    g = torch.from_numpy(pool.group_ids).to(dev)
    ts = torch.from_numpy(pool.timestamps).to(dev)
    off_o = torch.empty(pool.B + 1, dtype=torch.int32, device=dev)
    g_o = torch.empty(pool.T, dtype=torch.uint8, device=dev)
    ts_o = torch.empty(pool.T, dtype=torch.int64, device=dev)
    x_o = torch.empty_like(x)
    fit = torch.empty(2, dtype=torch.int64, device=dev)
    ws = mb.workspace(mb.OP_STOCHASTIC_LENGTH, pool.B, pool.T, d, H, dt, dev)
    stream = torch.cuda.current_stream()

    def sample():
        mb.mtgr_stochastic_length(off, g, ts, x, u, s_keep, budget, off_o, g_o, ts_o, x_o, fit, ws, stream)

    for _ in range(3):
        sample()
    torch.cuda.synchronize()
    times = []
    for _ in range(max(args.steps, 10)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sample()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    sl_ms = float(np.median(times))
    Bf, Tf = (int(v) for v in fit.cpu())
    T_all = int(off_o[-1].item())
    # algorithmic bytes: every row of the cut batch read and written
    # (features, group id, timestamp), plus offsets and draws
    sl_bytes = Tf * (2 * d * 2 + 2 * 1 + 2 * 8) + pool.B * (4 + 4 + 4)
    sl_gbs = sl_bytes / (sl_ms / 1e3) / 1e9

    def layer_step_ms(offsets_t, g_t, ts_t, xin, B, T, max_len, params):
        p = params[0]
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(dev)
        dev_p = {k: to(getattr(p, k)) for k in ("W_uqkv", "gamma1", "beta1", "gamma2", "beta2", "W_o")}
        prm = mb.make_params(dev_p, H)
        saved = mb.alloc_saved(T, d, dt, dev)
        sv = mb.make_saved(saved)
        y = torch.empty(T, d, dtype=dt, device=dev)
        dx = torch.empty_like(y)
        R = torch.randn(T, d, generator=gen).to(dt).to(dev)
        grads = mb.alloc_grads(d, 4, False, dev)
        ws_f = mb.workspace(mb.OP_LAYER_FWD, B, T, d, H, dt, dev)
        ws_b = mb.workspace(mb.OP_LAYER_BWD, B, T, d, H, dt, dev, max_len=max_len)
        scale = 1.0 / max_len

        def step():
            mb.mtgr_hstu_layer_fwd(prm, xin, y, sv, offsets_t, g_t, ts_t, scale, ws_f, stream)
            mb.mtgr_hstu_layer_bwd(prm, xin, sv, R, dx, grads, offsets_t, g_t, ts_t, scale, ws_b, max_len=max_len,
                                   stream=stream)

        for _ in range(max(args.warmup, 2)):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    _, params, _ = config_inputs(cfg_id, seed=args.seed)
    off_h = off_o[:Bf + 1].cpu().numpy()
    max_len_sl = int(np.max(np.diff(off_h)))
    ms_sl = layer_step_ms(off_o[:Bf + 1].clone(), g_o[:Tf], ts_o[:Tf], x_o[:Tf], Bf, Tf, max_len_sl, params)
    P_sl = fl.visible_pairs(off_h, g_o[:Tf].cpu().numpy(), ts_o[:Tf].cpu().numpy())
    base, _, xb = config_inputs(cfg_id, seed=args.seed)
    xbd = torch.from_numpy(np.ascontiguousarray(xb, dtype=np.float32)).to(dt).to(dev)
    ms_base = layer_step_ms(torch.from_numpy(base.offsets).to(dev), torch.from_numpy(base.group_ids).to(dev),
                            torch.from_numpy(base.timestamps).to(dev), xbd, base.B, base.T, int(base.max_len),
                            params)
    P_base = fl.visible_pairs(base.offsets, base.group_ids, base.timestamps)
    ups_sl = Bf / (ms_sl / 1e3)
    ups_base = base.B / (ms_base / 1e3)
    out = {
        "metric": "users/sec of the layer fwd+bwd at a 65,536-token budget with Stochastic Length sampling",
        "value": round(ups_sl, 1),
        "unit": "users/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded long-tail user pool, random-init weights)",
        "config": {"workload": "Stochastic Length on a long-tail user pool, then MTGR HSTU layer fwd+bwd",
                   "s_keep": s_keep, "token_budget": budget, "pool_users": pool.B, "pool_tokens": pool.T,
                   "d_model": d, "heads": H},
        "sampled": {"users": Bf, "tokens": Tf, "max_len": max_len_sl, "visible_pairs": P_sl,
                    "ms_per_step": round(ms_sl, 4), "users_per_sec": round(ups_sl, 1)},
        "unsampled": {"users": base.B, "tokens": base.T, "max_len": int(base.max_len), "visible_pairs": P_base,
                      "ms_per_step": round(ms_base, 4), "users_per_sec": round(ups_base, 1)},
        "users_per_sec_ratio": round(ups_sl / ups_base, 3),
        "sampling": {"ms": round(sl_ms, 4), "kept_tokens_of_pool": T_all, "bytes": sl_bytes,
                     "roofline": {"bound": "hbm", "achieved": round(sl_gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(sl_gbs / HBM_PEAK_GBS, 4)}},
    }
    print(json.dumps(out))


def head_bench(args):
    """Candidate head (Linear 1024 -> 512, SiLU, Linear 512 -> 2 tasks) with
    its binary cross-entropy loss and backward on the last-layer output of
    the 65,536-token bf16 batch (2,220 candidates).  Per kernel step: HIP
    events on the stream (library instrumentation) over the timed calls."""
    import numpy as np
    import torch

    import generative_recommendation_ranking_grouplayernorm_amd.binding as mb
    from mtgr_inputs import config_inputs, make_head_params, make_labels

    dev = torch.device("cuda:0")
    lib = mb.load_library()
    dt = torch.bfloat16
    batch, _, x = config_inputs(4, seed=args.seed)
    d, h, nt = 1024, 512, 2
    rng = np.random.default_rng([args.seed, 4, 9])
    hp = make_head_params(d, h, nt, rng, True)
    n_cand = int(np.sum(batch.group_ids == 3))
    y = torch.from_numpy(make_labels(n_cand, rng)).to(dev)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(dev)
    dev_p = {"W1": to(hp.W1), "b1": to(hp.b1), "W2": to(hp.W2), "b2": to(hp.b2)}
    prm = mb.make_head_params(dev_p)
    xd = to(x)
    off = torch.from_numpy(batch.offsets).to(dev)
    g = torch.from_numpy(batch.group_ids).to(dev)
    ws = mb.head_workspace(batch.B, n_cand, d, h, nt, dt, dev)
    loss = torch.empty(1, device=dev)
    logits = torch.empty(n_cand, nt, device=dev)
    dx = torch.empty(batch.T, d, dtype=dt, device=dev)
    grads = {"W1": torch.empty(h, d, device=dev), "b1": torch.empty(h, device=dev),
             "W2": torch.empty(nt, h, device=dev), "b2": torch.empty(nt, device=dev)}
    stream = torch.cuda.current_stream()

    def call():
        mb.mtgr_candidate_head_loss(prm, xd, off, g, n_cand, y, loss, logits, dx, grads, ws, stream)

    for _ in range(max(args.warmup, 3)):
        call()
    torch.cuda.synchronize()
    lib.mtgr_profile_enable(1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    prof = profile_summary(lib)
    lib.mtgr_profile_enable(0)
    for _ in range(3):
        call()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e2.record(stream)
    for _ in range(args.steps):
        call()
    e3.record(stream)
    torch.cuda.synchronize()
    ms = e2.elapsed_time(e3) / args.steps
    T = batch.T
    work = {  # algorithmic work per call
        "head_hidden": ("mfma", 2 * n_cand * d * h),
        "head_dW1": ("mfma", 2 * n_cand * d * h),
        "head_dX": ("mfma", 2 * n_cand * d * h),
        "head_expand": ("hbm", T * d * 2 + n_cand * d * 2),
        "head_gather": ("hbm", 2 * n_cand * d * 2),
    }
    kernels = {}
    for name, (tot, n) in prof.items():
        avg = tot / max(n, 1)
        ent = {"avg_ms": round(avg, 5), "ms_per_call": round(tot / args.steps, 5)}
        if name in work:
            bound, amount = work[name]
            if bound == "mfma":
                ach = amount / (avg / 1e3) / 1e12
                ent.update(bound="mfma", achieved=round(ach, 2), unit="TFLOP/s", frac=round(ach / BF16_PEAK_TFLOPS, 4))
            else:
                ach = amount / (avg / 1e3) / 1e9
                ent.update(bound="hbm", achieved=round(ach, 1), unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4))
        kernels[name] = ent
    out = {
        "metric": "candidate head + loss + backward time per training batch",
        "value": round(ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": False,
        "dtype": "bf16",
        "data": "synthetic (seeded 65,536-token batch, random-init head, Bernoulli labels)",
        "config": {"workload": "candidate head (d 1024 -> 512 -> 2 tasks) with BCE loss and backward",
                   "tokens": T, "users": batch.B, "candidates": n_cand, "d_model": d, "hidden": h, "tasks": nt},
        "loss": float(loss.item()),
        "kernels": kernels,
    }
    print(json.dumps(out))


def forward_batches_bench(args):
    """Forward-only throughput of two batch workloads: a bf16 layer of
    d_model 512 (4 heads of 128) over 32 long-tail users, users/s =
    B / t_layer_fwd; and 22 fp16 layers of d_model 1024 (8 heads of 128) over
    64 users, users/s = B / t_22-layer fwd, with the forward GFLOP per user
    (context: the pages print 137.87 GFLOPs per sample for their 22-layer,
    d_model 1024 model, counted their own way).  HIP events around timed
    repeats after warm-up; inputs resident in HBM."""
    import numpy as np
    import torch

    import generative_recommendation_ranking_grouplayernorm_amd.binding as mb
    from generative_recommendation_ranking_grouplayernorm_amd import flops as fl
    from mtgr_inputs import CONFIGS, config_inputs

    dev = torch.device("cuda:0")
    mb.load_library()
    stream = torch.cuda.current_stream()
    out = {"metric": "users/sec of forward-only batch workloads", "n_gpus": 1, "data": "synthetic",
           "higher_is_better": True, "workloads": {}}
    for cfg_id, dt in ((2, torch.bfloat16), (3, torch.float16)):
        cfg = CONFIGS[cfg_id]
        batch, params, x = config_inputs(cfg_id, seed=args.seed)
        d, H, L = cfg["d"], cfg["H"], cfg["layers"]
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(dev)
        keep = [{k: to(getattr(p, k)) for k in ("W_uqkv", "gamma1", "beta1", "gamma2", "beta2", "W_o")}
                for p in params]
        lps = [mb.make_params(t, H) for t in keep]
        xd = to(x)
        y = torch.empty_like(xd)
        off = torch.from_numpy(batch.offsets).to(dev)
        g = torch.from_numpy(batch.group_ids).to(dev)
        ts = torch.from_numpy(batch.timestamps).to(dev)
        scale = 1.0 / batch.max_len
        ws = mb.workspace(mb.OP_STACK_FWD, batch.B, batch.T, d, H, dt, dev)
        graph = mb.mtgr_stack_graph_create(lps, xd, y, off, g, ts, scale, ws)
        for _ in range(max(args.warmup, 3)):
            graph.launch(stream)
        torch.cuda.synchronize()
        reps = max(args.steps, 5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            graph.launch(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        graph.close()
        P = fl.visible_pairs(batch.offsets, batch.group_ids, batch.timestamps)
        gflop = L * (4 * d * P + fl.layer_gemm_flops(batch.T, d, backward=False)) / 1e9
        out["workloads"][cfg["name"]] = {
            "dtype": "bf16" if dt == torch.bfloat16 else "f16", "layers": L, "users": batch.B, "tokens": batch.T,
            "d_model": d, "heads": H, "ms_per_batch": round(ms, 4), "users_per_sec": round(batch.B / (ms / 1e3), 1),
            "fwd_gflop_per_user": round(gflop / batch.B, 2), "tflops": round(gflop / ms, 1)}
        print(f"[bench] {cfg['name']}: {ms:.3f} ms, {batch.B / (ms / 1e3):.0f} users/s", file=sys.stderr, flush=True)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
