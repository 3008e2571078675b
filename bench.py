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

Besides the headline workload the line carries, under "configs", one entry
per other configuration of the benchmark matrix (smaller batches, high
acceptance, the 32000-token vocabulary at T = 1 and T = 0, the RNN head,
ragged scheduled lengths), each with its own step time and roofline.

Roofline: every kernel of a step is timed in a further pass with hipEvents
that the library records on the launch stream; the dominant kernel's
algorithmic bytes per launch (every input of the method read once and every
output written once; the kernel's own scratch is not counted) divided by its
average duration give `achieved`.  `traffic` comes from committed rocprofv3
counter summaries of that kernel when they were taken on the current kernel
source; the excess over the algorithmic bytes is the kernel's overhead.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified+drafted tokens/s at B=128,gamma=16,V=152k; % of HBM roofline"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
MALL_FLUSH_BYTES = 512 << 20   # twice the 256 MB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic bytes and flops
# ---------------------------------------------------------------------------

def _nbytes(dt):
    return 2 if dt == "bf16" else 4


def kernel_bytes(wl, n_resid=None):
    """Algorithmic bytes per launch of each streaming kernel: every input of
    the method read once and every output written once, W2 counted once per
    call.  The kernels' own scratch (softmax summaries, token words) is not
    counted.  n_resid: requests whose final draw is a residual draw (the
    rest draw a bonus token); all of them when None."""
    B, g, V, r = wl["B"], wl["gamma"], wl["V"], wl["r"]
    lb, wb = _nbytes(wl["logit_dtype"]), _nbytes(wl["w_dtype"])
    lens = wl.get("lens")
    L = B * g if lens is None else int(sum(int(x) for x in lens))
    n_resid = B if n_resid is None else n_resid
    draft_out = B * g * (4 + 4 + 4)           # tokens, log Z, q(x)
    return {
        # per position: U_k read, q_k written, W2 / gamma, the B gathered W1 rows
        "draft_tile": B * V * (lb + 4) + r * V * wb / g + B * r * wb,
        # per position: U_k read, W2 / gamma, the W1 rows; outputs in the finalize
        "draft_tile_qfree": B * V * lb + r * V * wb / g + B * r * wb,
        # the whole draft in one launch: U, W2 once, the W1 rows, anchors, outputs
        "draft_persist": B * g * V * lb + r * V * wb + B * g * r * wb + B * 4 + draft_out,
        # target rows (the bonus row included)
        "verify_rows_p": (L + B) * V * lb,
        "verify_rows_q": L * V * 4,
        # the final draw of the q-free path: the target row and base row of every
        # residual draw, the target row of every bonus draw, W2 once, W1 rows
        "verify_resid": n_resid * V * 2 * lb + (B - n_resid) * V * lb + r * V * wb
                        + n_resid * r * wb,
    }


def cycle_bytes(wl, path, n_resid=None):
    """Algorithmic bytes of one whole cycle (draft + verify) of a path."""
    kb = kernel_bytes(wl, n_resid)
    B, g, V, r = wl["B"], wl["gamma"], wl["V"], wl["r"]
    lb, wb = _nbytes(wl["logit_dtype"]), _nbytes(wl["w_dtype"])
    # the RNN head also reads the hidden states and its three gate matrices
    head = (B * g * wl["d"] * 2 + 3 * r * (2 * r + wl["d"]) * wb) if wl.get("head") == "rnn" else 0
    if path == "qfree":
        return kb["draft_persist"] + head + kb["verify_rows_p"] + kb["verify_resid"]
    q = B * g * V * 4
    return (B * g * V * lb + q + r * V * wb + B * g * r * wb) + head + kb["verify_rows_p"] + q


def bias_flops(wl):
    """Algorithmic flops of the Markov bias contraction E . W2 per launch of
    each kernel that performs it (2 B r V per draft position)."""
    B, g, V, r = wl["B"], wl["gamma"], wl["V"], wl["r"]
    return {"draft_persist": 2.0 * B * r * V * g, "draft_tile_qfree": 2.0 * B * r * V,
            "draft_tile": 2.0 * B * r * V}


# ---------------------------------------------------------------------------
# Committed counter records (profiles/), gated on the kernel's source
# ---------------------------------------------------------------------------

def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_CS = "draft_sampling_lossless_head_amd/csrc/"
KERNEL_SOURCES = {
    "draft_persist": [_CS + "draft_persist.hip", _CS + "stream_finalize.hpp",
                      _CS + "device_common.hpp", _CS + "launch.hpp"],
    "draft_tile_qfree": [_CS + "draft_kernels.hip", _CS + "device_common.hpp",
                         _CS + "launch.hpp"],
    "draft_tile": [_CS + "draft_kernels.hip", _CS + "device_common.hpp"],
    "verify_rows_p": [_CS + "verify_kernels.hip", _CS + "device_common.hpp"],
    "verify_rows_q": [_CS + "verify_kernels.hip", _CS + "device_common.hpp"],
    "verify_resid": [_CS + "residual_kernels.hip", _CS + "device_common.hpp",
                     _CS + "launch.hpp"],
}


def _record(kernel, workload, kind):
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.{kind}.json")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return t


def measured_traffic(kernel, workload):
    """HBM bytes per launch from profiles/<kernel>__<workload>.traffic.json,
    or None when missing or taken on a different kernel source."""
    t = _record(kernel, workload, "traffic")
    return None if t is None else t.get("traffic_bytes_per_launch")


def measured_mfma(kernel, workload):
    """Matrix-core busy fraction from profiles/<kernel>__<workload>.mfma.json,
    or None when missing or taken on a different kernel source."""
    t = _record(kernel, workload, "mfma")
    return None if t is None else t.get("mfma_busy_frac")


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


# ---------------------------------------------------------------------------
# One workload on the device
# ---------------------------------------------------------------------------

class Cycle:
    """Device copies of one workload and the step that runs its cycle: the
    Markov head q-free (persistent or per-position engine) or materialised,
    the RNN head q-free (spec_verify_rnn) or materialised; ragged lengths
    verify only the first L_b positions of each request from packed target
    rows."""

    def __init__(self, sd, torch, wl, path, seed=0):
        import numpy as np

        import workloads

        self.sd, self.torch, self.wl, self.path, self.seed = sd, torch, wl, path, seed
        dev = torch.device("cuda:0")
        B, g, V, r = wl["B"], wl["gamma"], wl["V"], wl["r"]
        lb, wbt = wl["logit_dtype"], wl["w_dtype"]

        def to_dev(x, dt=None):
            t = torch.from_numpy(np.ascontiguousarray(x))
            if dt == "bf16":
                t = t.view(torch.bfloat16)
            return t.to(dev)

        self.to_dev = to_dev
        self.U, self.P = to_dev(wl["U"], lb), to_dev(wl["P"], lb)
        self.W1, self.x0 = to_dev(wl["W1"], wbt), to_dev(wl["x0"])
        self.W2dev = to_dev(wl["W2"], wbt)
        self.W2T = sd.spec_pack_w2(self.W2dev) if wbt == "bf16" else None   # once per model load
        self.W2 = None if self.W2T is not None else self.W2dev   # the Markov calls use W2T
        self.rnn = wl["head"] == "rnn"
        if self.rnn:
            self.H = to_dev(wl["H"], wl["h_dtype"])
            self.Wg, self.Wc, self.Wo = (to_dev(wl[k], wbt) for k in ("Wg", "Wc", "Wo"))
        lens = wl.get("lens")
        self.lens = None if lens is None else to_dev(lens)
        self.p_off = None if lens is None else to_dev(workloads.packed_offsets(lens + 1))
        self.qfree = path == "qfree"
        self.T = wl["T"]
        self.d_out = dict(tokens=torch.empty((B, g), dtype=torch.int32, device=dev),
                          q_logZ=torch.empty((B, g), dtype=torch.float32, device=dev),
                          q_tok_prob=torch.empty((B, g), dtype=torch.float32, device=dev))
        if not self.qfree:
            self.d_out["q_logits"] = torch.empty((B, g, V), dtype=torch.float32, device=dev)
        self.v_out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                          out_tokens=torch.empty((B, g + 1), dtype=torch.int32, device=dev))
        kind = "rnn" if self.rnn else "markov"
        dims = dict(B=B, gamma=g, V=V, r=r, d=wl.get("d", 0))
        self.ws_d = torch.empty(sd.workspace_bytes(kind, **dims), dtype=torch.uint8, device=dev)
        if self.qfree:
            nws_v = sd.workspace_bytes("verify_markov", B=B, gamma_max=g, V=V, r=r)
        else:
            nws_v = sd.workspace_bytes("verify", B=B, gamma_max=g, V=V)
        self.ws_v = torch.empty(nws_v, dtype=torch.uint8, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)

    def draft(self, i):
        sd = self.sd
        if self.rnn:
            sd.spec_draft_sample_rnn(self.U, self.x0, self.H, self.W1, self.W2dev, self.Wg, self.Wc,
                                     self.Wo, self.T, W2T=self.W2T, q_free=self.qfree,
                                     seed=self.seed, offset=i, out=self.d_out,
                                     workspace=self.ws_d)
        else:
            sd.spec_draft_sample_markov(self.U, self.x0, self.W1, self.W2, self.T, W2T=self.W2T,
                                        seed=self.seed, offset=i, out=self.d_out,
                                        workspace=self.ws_d)

    def verify(self, i, lens=None, out=None):
        sd, d = self.sd, self.d_out
        lens = self.lens if lens is None else lens
        out = self.v_out if out is None else out
        if self.qfree and self.rnn:
            sd.spec_verify_rnn(self.P, self.U, d["cond"], self.W2, d["tokens"], d["q_logZ"],
                               d["q_tok_prob"], self.T, W2T=self.W2T, lens=lens,
                               p_row_off=self.p_off, seed=self.seed, offset=i, out=out,
                               workspace=self.ws_v, diagnostics=False)
        elif self.qfree:
            sd.spec_verify_markov(self.P, self.U, self.x0, self.W1, self.W2, d["tokens"],
                                  d["q_logZ"], d["q_tok_prob"], self.T, W2T=self.W2T, lens=lens,
                                  p_row_off=self.p_off, seed=self.seed, offset=i, out=out,
                                  workspace=self.ws_v, diagnostics=False)
        else:
            sd.spec_verify(self.P, d["q_logits"], d["tokens"], self.T, lens=lens,
                           p_row_off=self.p_off, seed=self.seed, offset=i, out=out,
                           workspace=self.ws_v, diagnostics=False)

    def step(self, i):
        self.draft(i)
        self.verify(i)

    def wall(self, warmup, steps, offset0=0):
        """W untimed steps, then K steps between two synchronisations."""
        torch = self.torch
        for i in range(warmup):
            self.step(offset0 + i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(offset0 + warmup + i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def per_step_ms(self, steps, offset0, flush=None):
        """Duration of each step from hipEvents on the launch stream; with
        `flush` (a device buffer larger than the Infinity Cache) every step is
        preceded by a write of that buffer, outside the timed events."""
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            if flush is not None:
                flush.fill_(i & 0xFF)
            ev[i][0].record()
            self.step(offset0 + i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def kernel_times(self, steps, offset0, names):
        """Average launch duration of each named kernel (library hipEvents on
        the launch stream), one pass of `steps` cycles per kernel."""
        sd = self.sd
        res = {}
        for name in names:
            sd.spec_profile_enable(name)
            for i in range(steps):
                self.step(offset0 + i)
            n, ms = sd.spec_profile_read()
            sd.spec_profile_enable(None)
            if n:
                res[name] = dict(launches_per_step=n / steps, avg_us=ms * 1e3 / n,
                                 us_per_step=ms * 1e3 / steps)
        return res


KERNEL_NAMES = ["w2_pack", "draft_persist", "draft_tile", "draft_tile_qfree", "draft_finalize",
                "rnn_hidden_proj", "rnn_gates", "verify_rows_p", "verify_rows_q",
                "verify_decide", "verify_residual_rows", "verify_resid", "verify_final_partials",
                "verify_final_draw"]


def _stats(ms):
    return dict(median=round(statistics.median(ms), 4), min=round(min(ms), 4),
                mean=round(sum(ms) / len(ms), 4))


def roofline_of(cyc, kernels, workload_name):
    """Roofline object of the dominant streaming kernel of a timed cycle."""
    wl = cyc.wl
    acc = cyc.v_out["accepted"].cpu()
    L = cyc.lens.cpu() if cyc.lens is not None else None
    n_resid = int(((acc < (L if L is not None else wl["gamma"])) & (acc >= 0)).sum().item())
    nbytes = kernel_bytes(wl, n_resid)
    for name, kb in nbytes.items():
        if name in kernels:
            kernels[name]["alg_bytes_per_launch"] = round(kb)
            kernels[name]["achieved_GBs"] = round(kb / (kernels[name]["avg_us"] * 1e-6) / 1e9, 1)
    dom = max((k for k in kernels if k in nbytes), key=lambda k: kernels[k]["us_per_step"])
    ach = kernels[dom]["achieved_GBs"]
    traffic = measured_traffic(dom, workload_name)
    rf = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
              frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic, kernel=dom,
              alg_bytes_per_launch=round(nbytes[dom]),
              avg_launch_us=round(kernels[dom]["avg_us"], 2))
    if traffic is not None:
        rf["traffic_over_alg"] = round(traffic / nbytes[dom], 3)
        rf["overhead_bytes_per_launch"] = round(traffic - nbytes[dom])
    return rf, n_resid


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, and a sampled check of one GPU step
# ---------------------------------------------------------------------------

def cpu_baseline(wl, seed, offset, nsample, threads, gpu=None, min_seconds=10.0, max_steps=40):
    """The fp64 oracle (as it stands) on the first nsample requests: draft then
    verify of each request, requests spread over `threads` host threads, step
    after step (the uniforms of steps offset, offset + 1, ...) until about
    min_seconds of wall time (at most max_steps).  gpu: host copies of the GPU
    step at `offset`; the oracle's first step is compared with it request by
    request (draws within 1e-6 of a CDF boundary are counted, not failed)."""
    import concurrent.futures

    import numpy as np

    import oracle
    import workloads
    from oracle import compare

    B, g = wl["B"], wl["gamma"]
    lb, wbt = wl["logit_dtype"], wl["w_dtype"]
    W1 = workloads.as_f64(wl["W1"], wbt)
    W2 = workloads.as_f64(wl["W2"], wbt)
    U = [workloads.as_f64(wl["U"][b], lb) for b in range(nsample)]
    P = [workloads.as_f64(wl["P"][b], lb) for b in range(nsample)]
    T = wl["T"]

    def step(off):
        ud = oracle.draft_uniforms(seed, off, nsample, g)
        uv = oracle.verify_uniforms(seed, off, nsample, g)

        def one(b):
            d = oracle.draft_markov(U[b], W1, W2, int(wl["x0"][b]), T, ud[b])
            v = oracle.verify(P[b], d["q_logits"], d["tokens"], T, uv[b, :g], uv[b, g])
            return d, v

        with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
            return list(ex.map(one, range(nsample))), ud, uv

    t0 = time.perf_counter()
    res, ud, uv = step(offset)          # the step compared with the GPU's
    steps = 1
    while time.perf_counter() - t0 < min_seconds and steps < max_steps:
        step(offset + steps)
        steps += 1
    dt = time.perf_counter() - t0
    out = dict(value=steps * nsample * g / dt, unit="tokens/s", cores=threads, kind="oracle",
               sample=f"first {nsample} of {B} requests of the same workload, {steps} steps "
                      f"(uniforms of steps {offset}..{offset + steps - 1}; draft + verify, fp64, "
                      f"{threads} threads), {dt:.2f} s wall",
               mean_tau=float(np.mean([v["n"] for _, v in res])) + 1.0)
    if gpu is not None:
        td, tv = compare.Tally(), compare.Tally()
        mismatches = []
        for b in range(nsample):
            d, _ = res[b]
            try:
                same = compare.compare_draft_request(d, U[b], {k: x[b] for k, x in gpu["d"].items()},
                                                     T, ud[b], f"draft b={b}", td,
                                                     check_logits=False)
                if same:
                    gv = {k: x[b] for k, x in gpu["v"].items()}
                    gv["q_logZ"] = gpu["d"]["q_logZ"][b]
                    compare.compare_verify_request(P[b], d["q_logits"], d["tokens"], T,
                                                   uv[b, :g], uv[b, g], gv, f"verify b={b}", tv)
            except AssertionError as e:
                mismatches.append(str(e)[:200])
        out["check"] = dict(step_offset=offset, requests=nsample,
                            draft=td.as_dict(), verify=tv.as_dict(),
                            boundary_draws=td.boundary + tv.boundary,
                            fallbacks=tv.fallbacks, mismatches=len(mismatches),
                            first_mismatch=mismatches[0] if mismatches else None)
    return out


# ---------------------------------------------------------------------------
# The benchmark matrix beyond the headline workload
# ---------------------------------------------------------------------------

SWEEP = [
    # name, base config, overrides, path
    ("markov-152k-b32", "markov-152k-b128", dict(B=32), "qfree"),
    ("markov-152k-b64", "markov-152k-b128", dict(B=64), "qfree"),
    ("markov-152k-b128-sigma0.3", "markov-152k-b128", dict(sigma=0.3), "qfree"),
    ("markov-32k-b32", "markov-32k-b32", dict(), "qfree"),
    ("markov-32k-b32-greedy", "markov-32k-b32", dict(T=0.0), "qfree"),
    ("rnn-32k-b64", "rnn-32k-b64", dict(), "qfree"),
    ("rnn-32k-b64-materialized", "rnn-32k-b64", dict(), "materialized"),
    ("ragged-128k-b256", "ragged-128k-b256", dict(), "qfree"),
]


def make_workload(base, over):
    import workloads

    cfg = dict(workloads.CONFIGS[base])
    for k in ("sigma", "T"):
        if k in over:
            cfg[k] = over[k]
    maker = workloads.make_rnn if cfg["head"] == "rnn" else workloads.make_markov
    return maker(cfg, B=over.get("B"))


def sweep_line(sd, torch, name, base, over, path, warmup, steps):
    t0 = time.time()
    wl = make_workload(base, over)
    gen_s = time.time() - t0
    cyc = Cycle(sd, torch, wl, path)
    B, g = wl["B"], wl["gamma"]
    elapsed = cyc.wall(warmup, steps)
    ms = cyc.per_step_ms(steps, warmup + steps)
    kernels = cyc.kernel_times(steps, warmup, KERNEL_NAMES)
    rf, n_resid = roofline_of(cyc, kernels, name)
    acc = cyc.v_out["accepted"].float()
    lens = wl.get("lens")
    verified = B * g if lens is None else int(sum(int(x) for x in lens))
    cb = cycle_bytes(wl, cyc.path, n_resid)
    line = dict(workload=name, B=B, gamma=g, V=wl["V"], r=wl["r"], head=wl["head"],
                logits=wl["logit_dtype"], T=wl["T"], path=cyc.path,
                sigma=float(wl["sigma"][0]) if lens is None else "U(0.2,1.5) per request",
                ms_per_step=round(elapsed * 1e3 / steps, 4), step_ms=_stats(ms),
                drafted_per_s=round(B * g * steps / elapsed, 1),
                verified_per_s=round(verified * steps / elapsed, 1),
                mean_tau=round(float(acc.mean().item()) + 1.0, 4),
                roofline=rf,
                cycle=dict(alg_bytes=round(cb), achieved_GBs=round(cb / (elapsed / steps) / 1e9, 1),
                           frac=round(cb / (elapsed / steps) / 1e9 / HBM_PEAK_GBS, 4)),
                kernels={k: {a: round(b, 3) for a, b in v.items()} for k, v in kernels.items()},
                generated_s=round(gen_s, 1))
    log(f"  {name}: {line['ms_per_step']} ms/step, {line['drafted_per_s'] / 1e6:.3f} M tok/s, "
        f"{rf['kernel']} {rf['avg_launch_us']} us ({rf['frac']:.3f} of HBM peak)")
    del cyc
    torch.cuda.empty_cache()
    return line


# ---------------------------------------------------------------------------
# Pieces of DSpark's step around the cycle (not part of the timed cycle)
# ---------------------------------------------------------------------------

def around_the_cycle(sd, torch, cyc, warmup, steps):
    import workloads

    wl, dev = cyc.wl, torch.device("cuda:0")
    B, g, V, r, T = wl["B"], wl["gamma"], wl["V"], wl["r"], wl["T"]
    U, P, x0, W1, d_out = cyc.U, cyc.P, cyc.x0, cyc.W1, cyc.d_out
    out = {}
    # acceptance rate alpha_k = sum min(p_k, q_k), target rows against the
    # draft's base rows U_k; the kernel reads every P and U row twice
    sd.spec_profile_enable("acceptance_rate")
    aout = dict(alpha=torch.empty((B, g), dtype=torch.float32, device=dev),
                tv=torch.empty((B, g), dtype=torch.float32, device=dev))
    for i in range(steps):
        sd.spec_acceptance_rate(P, U, T, out=aout)
    n, ms = sd.spec_profile_read()
    sd.spec_profile_enable(None)
    if n:
        ab = B * g * V * 4
        us = ms * 1e3 / n
        out["acceptance_rate"] = dict(
            avg_us=round(us, 2), alg_bytes_per_launch=ab, achieved_GBs=round(ab / us / 1e3, 1),
            read_bytes_per_launch=2 * ab, read_GBs=round(2 * ab / us / 1e3, 1),
            mean_alpha=round(float(aout["alpha"].mean().item()), 4))
    # DSpark's confidence head over the drafted tokens (hidden states h_k of a
    # 4096-wide backbone, bf16) and the prefix scheduler on its output (an
    # engine whose step time is flat up to 4 B tokens, then grows linearly)
    dh = 4096
    cw = workloads.make_confidence(B, g, 8, r, dh, 1234)
    h_d, w_d = cyc.to_dev(cw["h"], "bf16"), cyc.to_dev(cw["w"])
    sps_d = cyc.to_dev(workloads.make_schedule(B, g, 1234)["sps"])
    c_d = torch.empty((B, g), dtype=torch.float32, device=dev)
    s_out = dict(lens=torch.empty(B, dtype=torch.int32, device=dev),
                 B=torch.empty(1, dtype=torch.int32, device=dev),
                 tau=torch.empty(1, dtype=torch.float64, device=dev))
    sd.spec_confidence_head(h_d, x0, d_out["tokens"], W1, w_d, out=c_d)
    for name in ("confidence_head", "prefix_schedule"):
        # three cycles ahead of the launches keep the device queue ahead of the
        # host, so the event brackets time the kernels, not the host
        for i in range(3):
            cyc.step(warmup + i)
        sd.spec_profile_enable(name)
        for i in range(steps):
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
            out[name] = dict(avg_us=round(us, 2), alg_bytes_per_launch=cb,
                             achieved_GBs=round(cb / us / 1e3, 1),
                             mean_c=round(float(c_d.mean().item()), 4), d=dh)
        else:
            out[name] = dict(avg_us=round(us, 2), candidates=B * g,
                             chosen_batch=int(s_out["B"].item()),
                             tau=round(float(s_out["tau"].item()), 3),
                             mean_len=round(float(s_out["lens"].float().mean().item()), 3))
    # DSpark's whole step: draft, confidence head, schedule, verification of the
    # scheduled prefixes only (ragged lengths).  Emitted = sum of (accepted + 1).
    v2 = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
              out_tokens=torch.empty((B, g + 1), dtype=torch.int32, device=dev))

    def dstep(i):
        cyc.draft(i)
        sd.spec_confidence_head(h_d, x0, d_out["tokens"], W1, w_d, out=c_d)
        sd.spec_prefix_schedule(c_d, sps_d, out=s_out)
        cyc.verify(i, lens=s_out["lens"], out=v2)

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
    for i in range(steps):
        dstep(warmup + i)
        emitted += v2["accepted"].sum() + B
        lens_sum += s_out["lens"].sum()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0d) / steps
    out["dspark_cycle"] = dict(
        ms_per_step=round(dt * 1e3, 4), drafted=B * g,
        mean_len=round(float(lens_sum.item()) / (B * steps), 3),
        emitted_per_step=round(float(emitted.item()) / steps, 2),
        emitted_per_s=round(float(emitted.item()) / steps / dt, 1),
        sps_table="synthetic: flat to 4B tokens, then 1/B")
    # tree drafts: the top 64 of 1024 candidate nodes per request by survival
    tw = workloads.make_trees(B, 1024, 1234)
    par_d, tc_d = cyc.to_dev(tw["parent"]), cyc.to_dev(tw["c"])
    t_out = dict(sel=torch.empty((B, 64), dtype=torch.int32, device=dev),
                 score=torch.empty(B, dtype=torch.float64, device=dev))
    for i in range(3):
        cyc.step(warmup + i)
    sd.spec_profile_enable("tree_select")
    for i in range(steps):
        sd.spec_tree_select(par_d, tc_d, 64, out=t_out)
    n, ms = sd.spec_profile_read()
    sd.spec_profile_enable(None)
    if n:
        out["tree_select"] = dict(avg_us=round(ms * 1e3 / n, 2), trees=B, nodes=1024, budget=64,
                                  mean_score=round(float(t_out["score"].mean().item()), 3))
    # tree verification: 32 requests, 16-node trees over 4 levels, the
    # workload's vocabulary (bf16 rows); the children of a node hold the
    # highest tokens of its draft row, first child the argmax
    import numpy as np
    BT, MT = 32, 16
    tvw = workloads.make_tree_verify(BT, MT, V, seed=1234, dtype="bf16", sigma=1.0, levels=4)
    Qf = workloads.bf16_bits_to_f32(tvw["Q"])
    tok = np.empty((BT, MT), dtype=np.int32)
    for b in range(BT):
        seen = {}
        for v in range(MT):
            pa = int(tvw["parent"][b, v])
            k = seen.get(pa, 0)
            seen[pa] = k + 1
            row = Qf[b, pa + 1]
            tok[b, v] = int(np.argpartition(-row, k)[k]) if k else int(np.argmax(row))
    Pt, Qt = cyc.to_dev(tvw["P"], "bf16"), cyc.to_dev(tvw["Q"], "bf16")
    part, tokt = cyc.to_dev(tvw["parent"]), cyc.to_dev(tok)
    tv_out = sd.spec_verify_tree(Pt, Qt, part, tokt, T, seed=5)
    for i in range(3):
        cyc.step(warmup + i)
    sd.spec_profile_enable("verify_tree")
    for i in range(steps):
        sd.spec_verify_tree(Pt, Qt, part, tokt, T, seed=5, offset=i, out=tv_out)
    n, ms = sd.spec_profile_read()
    sd.spec_profile_enable(None)
    if n:
        out["verify_tree"] = dict(avg_us=round(ms * 1e3 / n, 2), trees=BT, nodes=MT, V=V,
                                  mean_accepted=round(float(tv_out["accepted"].float().mean().item()), 3))
    del Pt, Qt
    return out


def gemm_only(torch, steps, warmup):
    """GEMM-only measurement of the draft's bias contraction, for comparison
    with the fused draft: one position's product [M, r] x [r, V] (M = 128
    requests, r = 256, V = 151936; bf16 inputs and output, fp32 accumulation)
    by the library GEMM (torch.mm, i.e. hipBLASLt), with the weight warm: the
    same W2 every call, so its 78 MB stay in the Infinity Cache.  Two weight
    layouts (W2 [r, V] row-major, and W2^T [V, r] as a linear layer's weight)
    and, for scale, M = 2048 (all 16 positions' rows at once, which the
    sequential draft cannot do).  Each call is timed with hipEvents on the
    stream it runs on.  Prints one JSON line."""
    K, N = 256, 151936
    g = torch.Generator(device="cuda").manual_seed(5)
    W = (0.02 * torch.randn(K, N, device="cuda", generator=g)).to(torch.bfloat16)
    WT = W.t().contiguous()
    res = {}
    for M in (128, 2048):
        A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        out = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        for lay, rhs in (("W2[r,V]", W), ("W2T[V,r]", WT.t())):
            for _ in range(warmup):
                torch.mm(A, rhs, out=out)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for a, b in ev:
                a.record()
                torch.mm(A, rhs, out=out)
                b.record()
            torch.cuda.synchronize()
            us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
            avg = sum(us) / len(us)
            flops = 2.0 * M * K * N
            out_bytes = M * N * 2
            res[f"M{M} {lay}"] = dict(
                avg_us=round(avg, 2), median_us=round(us[len(us) // 2], 2), min_us=round(us[0], 2),
                tflops=round(flops / (avg * 1e-6) / 1e12, 1),
                mfma_frac=round(flops / (avg * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                mfma_floor_us=round(flops / (MFMA_PEAK_TFLOPS * 1e12) * 1e6, 2),
                out_write_floor_us=round(out_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2))
            log(f"gemm-only M={M} {lay}: {avg:.2f} us avg, {res[f'M{M} {lay}']['tflops']} TFLOP/s")
        del A, out
    print(json.dumps({"metric": "bias contraction GEMM-only (library GEMM, W2 warm)",
                      "unit": "TFLOP/s", "dtype": "bf16", "peak": MFMA_PEAK_TFLOPS,
                      "shape": {"K": K, "N": N}, "steps": steps, "warmup": warmup,
                      "variants": res}), flush=True)


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
    ap.add_argument("--cpu-sample", type=int, default=128,
                    help="requests per oracle step (steps repeat for about 10 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="only the headline workload (no per-configuration lines)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the kernels around the cycle (alpha, head, scheduler, trees)")
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
    ap.add_argument("--gemm-only", action="store_true",
                    help="only the GEMM-only measurement of the bias contraction (library GEMM, "
                         "W2 warm); prints its own JSON line")
    ap.add_argument("--traffic-kernel", default="draft_persist<16, 5, 4, false, false>")
    ap.add_argument("--traffic-label", default="draft_persist")
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

    import torch

    if args.gemm_only:
        gemm_only(torch, args.steps, min(args.warmup, 20))
        return

    import draft_sampling_lossless_head_amd as sd

    over = {} if args.sigma is None else dict(sigma=args.sigma)
    base = args.workload
    t0 = time.time()
    wl = make_workload(base, over)
    log(f"generated {args.workload} in {time.time() - t0:.1f}s")
    B, g, V, r, T = wl["B"], wl["gamma"], wl["V"], wl["r"], wl["T"]
    sd.spec_draft_set_persistent({"per_position": 0, "persistent": 1,
                                  "persistent_coop": 2}[args.engine])
    cyc = Cycle(sd, torch, wl, args.path)
    qfree = cyc.qfree

    elapsed = cyc.wall(args.warmup, args.steps)
    ms_per_step = elapsed * 1e3 / args.steps
    value = B * g * args.steps / elapsed
    tau = float(cyc.v_out["accepted"].float().mean().item()) + 1.0
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value / 1e6:.3f} M tok/s, "
        f"mean tau {tau:.3f}")

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.quick:
        print(json.dumps({"metric": METRIC, "value": round(value, 1), "unit": "tokens/s",
                          "ms_per_step": round(ms_per_step, 4), "steps": args.steps,
                          "quick": True}), flush=True)
        return

    # Per-step durations (hipEvents on the launch stream): Infinity Cache warm
    # (W2 and the small buffers stay resident between steps), then flushed by a
    # 512 MB write before every step.
    off = args.warmup + args.steps
    warm_ms = cyc.per_step_ms(args.steps, off)
    flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    cold_ms = cyc.per_step_ms(args.steps, off, flush=flush)
    del flush
    # Every kernel of the step, timed on its own pass.
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if qfree:   # completion word of the last draft (1: the persistent waits gave up)
        sd.spec_draft_status(cyc.ws_d, B, g, V, r, out=status)
    kernels = cyc.kernel_times(args.steps, args.warmup, KERNEL_NAMES)
    roofline, n_resid = roofline_of(cyc, kernels, args.workload)
    cb = cycle_bytes(wl, cyc.path, n_resid)
    roofline["cycle"] = dict(alg_bytes=round(cb),
                             achieved_GBs=round(cb / (ms_per_step * 1e-3) / 1e9, 1),
                             frac=round(cb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             note="whole-cycle algorithmic bytes / ms_per_step")
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
    # One more step at offset 0, kept for the oracle check of the CPU baseline.
    cyc.step(0)
    gpu_out = dict(d={k: v.cpu().numpy() for k, v in cyc.d_out.items()
                      if k not in ("q_logits", "cond")},
                   v={k: v.cpu().numpy() for k, v in cyc.v_out.items()})

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Zipf+Gaussian logits, random-init weights)",
        "config": {"workload": args.workload, "B": B, "gamma": g, "V": V, "r": r,
                   "logits": wl["logit_dtype"], "weights": wl["w_dtype"], "accumulate": "fp32",
                   "T": T, "sigma": float(wl["sigma"][0]), "head": wl["head"],
                   "verify": "fixed-length", "path": cyc.path,
                   "engine": args.engine if qfree else "per_position"},
        "roofline": roofline,
        "mfma": mfma,
        "step_ms": {"mall_warm": _stats(warm_ms), "mall_flushed": _stats(cold_ms),
                    "flush_bytes": MALL_FLUSH_BYTES},
        "breakdown": {
            "mean_tau": round(tau, 4),
            "emitted_per_s": round(tau * B * args.steps / elapsed, 1),
            "draft_status": int(status.item()),
            "kernels": {k: {a: round(b, 3) for a, b in v.items()} for k, v in kernels.items()},
        },
    }
    tdraft = sum(kernels[k]["us_per_step"] for k in kernels
                 if k.startswith("draft") or k.startswith("rnn"))
    tver = sum(kernels[k]["us_per_step"] for k in kernels if k.startswith("verify"))
    if tdraft > 0:
        result["breakdown"]["drafted_per_s"] = round(B * g / (tdraft * 1e-6), 1)
    if tver > 0:
        result["breakdown"]["verified_per_s"] = round(B * g / (tver * 1e-6), 1)
    if not args.no_extras and wl["w_dtype"] == "bf16" and wl["logit_dtype"] == "bf16":
        result["breakdown"].update(around_the_cycle(sd, torch, cyc, args.warmup, args.steps))
    del cyc
    torch.cuda.empty_cache()

    if not args.no_sweep and args.workload == "markov-152k-b128" and args.sigma is None:
        log("benchmark matrix ...")
        sweep_warmup = min(args.warmup, 10)
        result["configs"] = [sweep_line(sd, torch, name, b, o, p, sweep_warmup, args.steps)
                             for name, b, o, p in SWEEP]

    if not args.no_cpu_baseline and wl["head"] == "markov":
        threads = min(args.cpu_sample, len(os.sched_getaffinity(0)), 16)
        log(f"oracle baseline on {args.cpu_sample} requests, {threads} threads ...")
        result["cpu_baseline"] = cpu_baseline(wl, 0, 0, min(args.cpu_sample, B), threads,
                                              gpu_out)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
