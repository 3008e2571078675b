#!/usr/bin/env python3
"""Benchmark of one speculative cycle on one MI355X: DSpark Markov-head draft
(gamma sequential positions for a batch of requests) followed by lossless
verification of the drafted block.

A step is one whole cycle on one batch of seeded synthetic inputs already
resident in HBM:

* --path qfree (default): spec_draft_sample_markov without draft logits, then
  spec_verify_markov, which rebuilds only the draft row a residual draw needs;
* --path materialized: the draft writes its fp32 logits [B, gamma, V] and
  spec_verify reads them back.

W2 is packed once (spec_pack_w2) before timing, as at weight load.  value =
B * gamma * steps / time ("verified+drafted tokens/s": every drafted token is
also verified in the same step).  Prints ONE JSON line on stdout; progress
goes to stderr.

Roofline: every kernel of a step is timed in a second timed region with
hipEvents that the library records on the launch stream; the dominant
kernel's algorithmic bytes per launch divided by its average duration give
`achieved`.  `traffic` comes from committed rocprofv3 counter summaries of
that kernel when they were taken on the current kernel source.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified+drafted tokens/s at B=128,gamma=16,V=152k; % of HBM roofline"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_bytes(wl):
    """Algorithmic bytes per launch of each streaming kernel (every input read
    once, every output written once; W2 counted once per draft call)."""
    B, g, V, r = wl["B"], wl["gamma"], wl["V"], wl["r"]
    lb = 2 if wl["logit_dtype"] == "bf16" else 4
    wb = 2 if wl["w_dtype"] == "bf16" else 4
    return {
        # U_k read, q_k written, W2 / gamma, the B gathered W1 rows
        "draft_tile": B * V * (lb + 4) + r * V * wb / g + B * r * wb,
        # U_k read; per (row, 32-token segment) its max and 4 group sums, per
        # (row, share) one 16-byte summary (256 shares) written
        "draft_tile_qfree": B * V * lb + B * ((V + 31) // 32) * (4 + 4 * 4) + B * 256 * 16
                            + r * V * wb / g + B * r * wb,
        # the whole draft in one launch: per position U_k, the W1 rows and the
        # same summaries; W2 once
        "draft_persist": g * (B * V * lb + B * ((V + 31) // 32) * (4 + 4 * 4) + B * 256 * 16
                              + B * r * wb) + r * V * wb,
        "verify_rows_p": B * (g + 1) * V * lb,
        "verify_rows_q": B * g * V * 4,
    }


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "draft_persist": ["draft_sampling_lossless_head_amd/csrc/draft_persist.hip",
                      "draft_sampling_lossless_head_amd/csrc/stream_finalize.hpp",
                      "draft_sampling_lossless_head_amd/csrc/device_common.hpp",
                      "draft_sampling_lossless_head_amd/csrc/launch.hpp"],
    "draft_tile_qfree": ["draft_sampling_lossless_head_amd/csrc/draft_kernels.hip",
                         "draft_sampling_lossless_head_amd/csrc/device_common.hpp",
                         "draft_sampling_lossless_head_amd/csrc/launch.hpp"],
    "draft_tile": ["draft_sampling_lossless_head_amd/csrc/draft_kernels.hip",
                   "draft_sampling_lossless_head_amd/csrc/device_common.hpp"],
    "verify_rows_p": ["draft_sampling_lossless_head_amd/csrc/verify_kernels.hip",
                      "draft_sampling_lossless_head_amd/csrc/device_common.hpp"],
    "verify_rows_q": ["draft_sampling_lossless_head_amd/csrc/verify_kernels.hip",
                      "draft_sampling_lossless_head_amd/csrc/device_common.hpp"],
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from profiles/<kernel>__<workload>.traffic.json,
    or None when missing or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return t.get("traffic_bytes_per_launch")


def bias_flops(wl):
    """Algorithmic flops of the Markov bias contraction E . W2 per launch of
    each kernel that performs it (2 B r V per draft position)."""
    B, g, V, r = wl["B"], wl["gamma"], wl["V"], wl["r"]
    return {"draft_persist": 2.0 * B * r * V * g, "draft_tile_qfree": 2.0 * B * r * V,
            "draft_tile": 2.0 * B * r * V}


def measured_mfma(kernel, workload):
    """Matrix-core busy fraction from profiles/<kernel>__<workload>.mfma.json,
    or None when missing or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return t.get("mfma_busy_frac")


def mfma_from_sq(sq_csv, kernel_substr, label, workload):
    """Matrix-core busy fraction of one kernel from a rocprofv3 --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES (cycles, summed over SIMDs) and SQ_WAVE_CYCLES
    (quad-cycles, summed over waves): busy / (4 x wave cycles), i.e. the share
    of the kernel's wave-occupied SIMD cycles in which the matrix core works
    (one wave per SIMD in the persistent draft).  Writes
    profiles/<label>__<workload>.mfma.json tagged with the kernel's source hash."""
    import csv

    vals = {}
    with open(sq_csv) as f:
        for r in csv.DictReader(f):
            if kernel_substr in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if "SQ_VALU_MFMA_BUSY_CYCLES" not in vals or "SQ_WAVE_CYCLES" not in vals:
        raise SystemExit(f"no SQ_VALU_MFMA_BUSY_CYCLES / SQ_WAVE_CYCLES for {kernel_substr!r}")
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    rec = dict(kernel=label, kernel_match=kernel_substr, workload=workload,
               counters_per_dispatch=avg, dispatches=len(vals["SQ_WAVE_CYCLES"]),
               mfma_busy_frac=avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (4.0 * avg["SQ_WAVE_CYCLES"]),
               source_sha=source_sha(KERNEL_SOURCES[label]))
    path = os.path.join(ROOT, "profiles", f"{label}__{workload}.mfma.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def traffic_from_pmc(fetch_csv, write_csv, kernel_substr, label, workload, probe_bytes):
    """HBM bytes per launch of one kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE in KiB per dispatch), each scaled so that the
    largest device copy in the same run (the --copy-probe-mib copy) reads and
    writes exactly probe_bytes.  Writes profiles/<label>__<workload>.traffic.json
    tagged with the hash of the kernel's sources."""
    import csv

    def rows(path, counter):
        with open(path) as f:
            return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]

    out = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        rr = rows(path, counter)
        probe = max(float(r["Counter_Value"]) for r in rr if "copyBuffer" in r["Kernel_Name"])
        scale = probe_bytes / (probe * 1024.0)
        vals = [float(r["Counter_Value"]) for r in rr if kernel_substr in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"no dispatch of {kernel_substr!r} in {path}")
        out[counter] = dict(kib_per_dispatch=sum(vals) / len(vals), dispatches=len(vals),
                            probe_kib=probe, scale=scale,
                            bytes_per_launch=sum(vals) / len(vals) * 1024.0 * scale)
    rec = dict(kernel=label, kernel_match=kernel_substr, workload=workload,
               read_bytes_per_launch=out["FETCH_SIZE"]["bytes_per_launch"],
               write_bytes_per_launch=out["WRITE_SIZE"]["bytes_per_launch"],
               traffic_bytes_per_launch=out["FETCH_SIZE"]["bytes_per_launch"]
               + out["WRITE_SIZE"]["bytes_per_launch"],
               counters=out, probe_bytes=probe_bytes,
               source_sha=source_sha(KERNEL_SOURCES[label]))
    path = os.path.join(ROOT, "profiles", f"{label}__{workload}.traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(wl, seed, nsample, threads):
    """The fp64 oracle (as it stands) on the first nsample requests: draft then
    verify of each request, requests spread over `threads` host threads."""
    import concurrent.futures

    import numpy as np

    import oracle
    import workloads

    B, g = wl["B"], wl["gamma"]
    lb, wbt = wl["logit_dtype"], wl["w_dtype"]
    W1 = workloads.as_f64(wl["W1"], wbt)
    W2 = workloads.as_f64(wl["W2"], wbt)
    ud = oracle.draft_uniforms(seed, 0, nsample, g)
    uv = oracle.verify_uniforms(seed, 0, nsample, g)
    U = [workloads.as_f64(wl["U"][b], lb) for b in range(nsample)]
    P = [workloads.as_f64(wl["P"][b], lb) for b in range(nsample)]
    T = wl["T"]

    def one(b):
        d = oracle.draft_markov(U[b], W1, W2, int(wl["x0"][b]), T, ud[b])
        v = oracle.verify(P[b], d["q_logits"], d["tokens"], T, uv[b, :g], uv[b, g])
        return v["n"]

    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        ns = list(ex.map(one, range(nsample)))
    dt = time.perf_counter() - t0
    return dict(value=nsample * g / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"first {nsample} of {B} requests of the same workload (draft + verify, "
                       f"fp64, {threads} threads), {dt:.2f} s wall",
                mean_tau=float(np.mean(ns)) + 1.0)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="markov-152k-b128")
    ap.add_argument("--path", choices=("qfree", "materialized"), default="qfree",
                    help="q-free cycle (no draft-logit tensor) or materialized draft logits")
    ap.add_argument("--engine", choices=("persistent", "persistent_coop", "per_position"),
                    default="persistent",
                    help="q-free draft: one persistent launch (plain, or cooperative), or two "
                         "launches per position")
    ap.add_argument("--sigma", type=float, default=None, help="override target/draft noise")
    ap.add_argument("--cpu-sample", type=int, default=64, help="requests timed on the oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="only the timed region (no per-kernel timing passes, no CPU baseline)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter CSVs into the traffic "
                         "record of --traffic-kernel")
    ap.add_argument("--mfma-from", metavar="SQ_CSV",
                    help="no GPU run: turn a rocprofv3 --pmc run with SQ_VALU_MFMA_BUSY_CYCLES and "
                         "SQ_WAVE_CYCLES into the matrix-core record of --traffic-kernel")
    ap.add_argument("--traffic-kernel", default="draft_tile_stream<16, false>")
    ap.add_argument("--traffic-label", default="draft_tile_qfree")
    args = ap.parse_args()
    if args.mfma_from:
        mfma_from_sq(args.mfma_from, args.traffic_kernel, args.traffic_label, args.workload)
        return
    if args.traffic_from:
        traffic_from_pmc(args.traffic_from[0], args.traffic_from[1], args.traffic_kernel,
                         args.traffic_label, args.workload, (args.copy_probe_mib or 1024) << 20)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the method's requests are "
              "independent, so several GPUs would each run this same step on their own share of "
              "the batch with no exchange; this benchmark does not launch several GPUs.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_sampling_lossless_head_amd as sd
    import workloads

    cfg = dict(workloads.CONFIGS[args.workload])
    if args.sigma is not None:
        cfg["sigma"] = args.sigma
    t0 = time.time()
    wl = workloads.make_markov(cfg)
    log(f"generated {args.workload} in {time.time() - t0:.1f}s")
    B, g, V, r, T = wl["B"], wl["gamma"], wl["V"], wl["r"], wl["T"]
    lb, wbt = wl["logit_dtype"], wl["w_dtype"]
    dev = torch.device("cuda:0")

    def to_dev(x, dt=None):
        t = torch.from_numpy(np.ascontiguousarray(x))
        if dt == "bf16":
            t = t.view(torch.bfloat16)
        return t.to(dev)

    U, P = to_dev(wl["U"], lb), to_dev(wl["P"], lb)
    W1, W2, x0 = to_dev(wl["W1"], wbt), to_dev(wl["W2"], wbt), to_dev(wl["x0"])
    qfree = args.path == "qfree"
    sd.spec_draft_set_persistent({"per_position": 0, "persistent": 1, "persistent_coop": 2}[args.engine])
    W2T = sd.spec_pack_w2(W2)          # once per model load
    d_out = dict(tokens=torch.empty((B, g), dtype=torch.int32, device=dev),
                 q_logZ=torch.empty((B, g), dtype=torch.float32, device=dev),
                 q_tok_prob=torch.empty((B, g), dtype=torch.float32, device=dev))
    if not qfree:
        d_out["q_logits"] = torch.empty((B, g, V), dtype=torch.float32, device=dev)
    v_out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                 out_tokens=torch.empty((B, g + 1), dtype=torch.int32, device=dev))
    ws_d = torch.empty(sd.workspace_bytes("markov", B=B, gamma=g, V=V, r=r), dtype=torch.uint8,
                       device=dev)
    if qfree:
        nws_v = sd.workspace_bytes("verify_markov", B=B, gamma_max=g, V=V, r=r)
    else:
        nws_v = sd.workspace_bytes("verify", B=B, gamma_max=g, V=V)
    ws_v = torch.empty(nws_v, dtype=torch.uint8, device=dev)
    seed = 0

    def step(i):
        sd.spec_draft_sample_markov(U, x0, W1, None, T, W2T=W2T, seed=seed, offset=i,
                                    out=d_out, workspace=ws_d)
        if qfree:
            sd.spec_verify_markov(P, U, x0, W1, None, d_out["tokens"], d_out["q_logZ"],
                                  d_out["q_tok_prob"], T, W2T=W2T, seed=seed, offset=i,
                                  out=v_out, workspace=ws_v)
        else:
            sd.spec_verify(P, d_out["q_logits"], d_out["tokens"], T, seed=seed, offset=i,
                           out=v_out, workspace=ws_v)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = B * g * args.steps / elapsed
    tau = float(v_out["accepted"].float().mean().item()) + 1.0
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value / 1e6:.3f} M tok/s, "
        f"mean tau {tau:.3f}")

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.quick:
        print(json.dumps({"metric": METRIC, "value": round(value, 1), "unit": "tokens/s",
                          "ms_per_step": round(ms_per_step, 4), "steps": args.steps,
                          "quick": True}), flush=True)
        return

    # Second timed region: the same steps with every kernel bracketed by events.
    sd.spec_profile_enable("*")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    prof_ms_per_step = (time.perf_counter() - t1) * 1e3 / args.steps
    sd.spec_profile_enable(None)
    kernels = {}
    names = ["w2_pack", "draft_persist", "draft_tile", "draft_tile_qfree", "draft_finalize", "verify_rows_p",
             "verify_rows_q", "verify_decide", "verify_residual_rows", "verify_resid", "verify_final_partials",
             "verify_final_draw"]
    for name in names:
        sd.spec_profile_enable(name)
        for i in range(args.steps):
            step(args.warmup + i)
        n, ms = sd.spec_profile_read()
        sd.spec_profile_enable(None)
        if n:
            kernels[name] = dict(launches_per_step=n / args.steps, avg_us=ms * 1e3 / n,
                                 us_per_step=ms * 1e3 / args.steps)
    nbytes = kernel_bytes(wl)
    for name, kb in nbytes.items():
        if name in kernels:
            kernels[name]["alg_bytes_per_launch"] = kb
            kernels[name]["achieved_GBs"] = kb / (kernels[name]["avg_us"] * 1e-6) / 1e9
    dom = max((k for k in kernels if k in nbytes), key=lambda k: kernels[k]["us_per_step"])
    ach = kernels[dom]["achieved_GBs"]
    roofline = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4),
                    traffic=measured_traffic(dom, args.workload), kernel=dom,
                    alg_bytes_per_launch=nbytes[dom],
                    avg_launch_us=round(kernels[dom]["avg_us"], 2))
    result_extra = {}
    fl = bias_flops(wl)
    mk = max((k for k in kernels if k in fl), key=lambda k: kernels[k]["us_per_step"], default=None)
    mfma = None
    if mk is not None:
        tf = fl[mk] / (kernels[mk]["avg_us"] * 1e-6) / 1e12
        mfma = dict(kernel=mk, dtype="bf16", flops_per_launch=fl[mk], achieved=round(tf, 1),
                    peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s", frac=round(tf / MFMA_PEAK_TFLOPS, 4),
                    busy_frac_counter=measured_mfma(mk, args.workload))
    log("kernels: " + json.dumps({k: {a: round(b, 2) for a, b in v.items()}
                                  for k, v in kernels.items()}))

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Zipf+Gaussian logits, random-init weights)",
        "config": {"workload": args.workload, "B": B, "gamma": g, "V": V, "r": r,
                   "logits": lb, "weights": wbt, "accumulate": "fp32", "T": T,
                   "sigma": float(wl["sigma"][0]), "head": "markov",
                   "verify": "fixed-length", "path": args.path,
                   "engine": args.engine if qfree else "per_position"},
        "roofline": roofline,
        "mfma": mfma,
        "breakdown": {
            "drafted_per_s": None, "verified_per_s": None,
            "mean_tau": round(tau, 4),
            "emitted_per_s": round(tau * B * args.steps / elapsed, 1),
            "profiled_ms_per_step": round(prof_ms_per_step, 4),
            "kernels": {k: {a: round(b, 3) for a, b in v.items()} for k, v in kernels.items()},
        },
    }
    # The per-position acceptance rate alpha_k = sum min(p_k, q_k) (not part of
    # the cycle): target rows against the draft's base rows U_k, the same
    # number of timed launches.  Algorithmic bytes: every used P and U row read
    # once; the kernel reads them twice (normalisers, then the sums).
    if wl["logit_dtype"] == "bf16":
        sd.spec_profile_enable("acceptance_rate")
        aout = dict(alpha=torch.empty((B, g), dtype=torch.float32, device=dev),
                    tv=torch.empty((B, g), dtype=torch.float32, device=dev))
        for i in range(args.steps):
            sd.spec_acceptance_rate(P, U, T, out=aout)
        n, ms = sd.spec_profile_read()
        sd.spec_profile_enable(None)
        if n:
            ab = B * g * V * 4
            us = ms * 1e3 / n
            result_extra["acceptance_rate"] = dict(
                avg_us=round(us, 2), alg_bytes_per_launch=ab, achieved_GBs=round(ab / us / 1e3, 1),
                read_bytes_per_launch=2 * ab, read_GBs=round(2 * ab / us / 1e3, 1),
                mean_alpha=round(float(aout["alpha"].mean().item()), 4))
    # DSpark's confidence head over the drafted tokens (hidden states h_k of a
    # 4096-wide backbone, bf16) and the prefix scheduler on its output (an
    # engine whose step time is flat up to 4 B tokens, then grows linearly).
    # Not part of the timed cycle.  Algorithmic bytes of the head: every h row,
    # the embedding row of each previous token, c and the token read, w once.
    if wbt == "bf16" and lb == "bf16":
        dh = 4096
        cw = workloads.make_confidence(B, g, 8, r, dh, 1234)
        h_d, w_d = to_dev(cw["h"], "bf16"), to_dev(cw["w"])
        sps_d = to_dev(workloads.make_schedule(B, g, 1234)["sps"])
        c_d = torch.empty((B, g), dtype=torch.float32, device=dev)
        s_out = dict(lens=torch.empty(B, dtype=torch.int32, device=dev),
                     B=torch.empty(1, dtype=torch.int32, device=dev),
                     tau=torch.empty(1, dtype=torch.float64, device=dev))
        sd.spec_confidence_head(h_d, x0, d_out["tokens"], W1, w_d, out=c_d)
        for name in ("confidence_head", "prefix_schedule"):
            # Three cycles ahead of the launches keep the device queue ahead of
            # the host, so the event brackets time the kernels, not the host.
            for i in range(3):
                step(args.warmup + i)
            sd.spec_profile_enable(name)
            for i in range(args.steps):
                if name == "confidence_head":
                    sd.spec_confidence_head(h_d, x0, d_out["tokens"], W1, w_d, out=c_d)
                else:
                    sd.spec_prefix_schedule(c_d, sps_d, out=s_out)
            n, ms = sd.spec_profile_read()
            sd.spec_profile_enable(None)
            if not n:
                continue
            us = ms * 1e3 / n
            if name == "confidence_head":
                cb = B * g * (dh * 2 + r * 2 + 4 + 4) + (dh + r) * 4
                result_extra[name] = dict(avg_us=round(us, 2), alg_bytes_per_launch=cb,
                                          achieved_GBs=round(cb / us / 1e3, 1),
                                          mean_c=round(float(c_d.mean().item()), 4), d=dh)
            else:
                result_extra[name] = dict(avg_us=round(us, 2), candidates=B * g,
                                          chosen_batch=int(s_out["B"].item()),
                                          tau=round(float(s_out["tau"].item()), 3),
                                          mean_len=round(float(s_out["lens"].float().mean().item()), 3))
        # DSpark's whole step: draft gamma positions, score them with the
        # confidence head, schedule the lengths, verify only the scheduled
        # prefixes (ragged lengths).  Emitted = sum of (accepted + 1).
        if qfree:
            v2 = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                      out_tokens=torch.empty((B, g + 1), dtype=torch.int32, device=dev))

            def dstep(i):
                sd.spec_draft_sample_markov(U, x0, W1, None, T, W2T=W2T, seed=seed, offset=i,
                                            out=d_out, workspace=ws_d)
                sd.spec_confidence_head(h_d, x0, d_out["tokens"], W1, w_d, out=c_d)
                sd.spec_prefix_schedule(c_d, sps_d, out=s_out)
                sd.spec_verify_markov(P, U, x0, W1, None, d_out["tokens"], d_out["q_logZ"],
                                      d_out["q_tok_prob"], T, W2T=W2T, lens=s_out["lens"],
                                      seed=seed, offset=i, out=v2, workspace=ws_v)

            emitted = torch.zeros((), dtype=torch.int64, device=dev)
            lens_sum = torch.zeros((), dtype=torch.int64, device=dev)
            for i in range(3):   # warm-up, including torch's first (lazily loaded) sums
                dstep(i)
                emitted += v2["accepted"].sum() + B
                lens_sum += s_out["lens"].sum()
            torch.cuda.synchronize()
            emitted.zero_()
            lens_sum.zero_()
            torch.cuda.synchronize()
            t0d = time.perf_counter()
            for i in range(args.steps):
                dstep(args.warmup + i)
                emitted += v2["accepted"].sum() + B
                lens_sum += s_out["lens"].sum()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0d) / args.steps
            result_extra["dspark_cycle"] = dict(
                ms_per_step=round(dt * 1e3, 4), drafted=B * g,
                mean_len=round(float(lens_sum.item()) / (B * args.steps), 3),
                emitted_per_step=round(float(emitted.item()) / args.steps, 2),
                emitted_per_s=round(float(emitted.item()) / args.steps / dt, 1),
                sps_table="synthetic: flat to 4B tokens, then 1/B")
    # Tree drafts: the top 64 of 1024 candidate nodes per request by survival
    # probability, for every request of the batch (not part of the cycle).
    tw = workloads.make_trees(B, 1024, 1234)
    par_d, tc_d = to_dev(tw["parent"]), to_dev(tw["c"])
    t_out = dict(sel=torch.empty((B, 64), dtype=torch.int32, device=dev),
                 score=torch.empty(B, dtype=torch.float64, device=dev))
    for i in range(3):
        step(args.warmup + i)
    sd.spec_profile_enable("tree_select")
    for i in range(args.steps):
        sd.spec_tree_select(par_d, tc_d, 64, out=t_out)
    n, ms = sd.spec_profile_read()
    sd.spec_profile_enable(None)
    if n:
        result_extra["tree_select"] = dict(avg_us=round(ms * 1e3 / n, 2), trees=B, nodes=1024,
                                           budget=64,
                                           mean_score=round(float(t_out["score"].mean().item()), 3))
    tdraft = sum(kernels[k]["us_per_step"] for k in kernels if k.startswith("draft")
                 or k == "w2_pack")
    tver = sum(kernels[k]["us_per_step"] for k in kernels if k.startswith("verify"))
    result["breakdown"].update(result_extra)
    if tdraft > 0:
        result["breakdown"]["drafted_per_s"] = round(B * g / (tdraft * 1e-6), 1)
    if tver > 0:
        result["breakdown"]["verified_per_s"] = round(B * g / (tver * 1e-6), 1)

    if not args.no_cpu_baseline:
        threads = min(args.cpu_sample, len(os.sched_getaffinity(0)), 16)
        log(f"oracle baseline on {args.cpu_sample} requests, {threads} threads ...")
        result["cpu_baseline"] = cpu_baseline(wl, seed, min(args.cpu_sample, B), threads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
