"""Benchmark of the KDA hot path on one MI355X.

One step = one kda_chunk_fwd call over the headline workload (bf16, B=4,
H=16, T=4096, dk=dv=128, chunk 64, nonzero initial state), inputs already
resident in HBM.  value = tokens per second (B*T tokens per step).

The same JSON line carries the other workloads of the path, each timed with
HIP events on the launch stream over its own loop of K launches:
  long_context  chunk forward, bf16 B1 H32 T65536 (slow forgetting)
  varlen        chunk forward, 64 packed sequences of 128..8192 tokens, H16
  decode        100 consecutive in-place decode steps, N256 H32 d128
  backward      gradients of the headline forward
  gdn2          Gated DeltaNet-2 chunk forward at the headline's shapes, and its
                decode step at the decode workload's shapes
For the headline and the decode step it also reports the time of single
launches that each follow a 1 GiB read (the 256 MB last-level cache then
holds none of the launch's inputs): the HBM-cold figure beside the
back-to-back one.

The headline is timed last, after the other legs, the chunk-kernel legs (long
context, varlen) just before it: the shader clock climbs for some 25 ms of
chunk-kernel work (and the memory-bound decode steps leave it lower), so the
headline's K timed steps after its W warm-up steps run at the clock a busy GPU
holds for this kernel whatever W is.

Before the legs it measures what this GPU reaches on the roofline's two
resources with its own kernels (libkda_peaks.so): a streaming copy, a
read-only stream and a loop of bf16 matrix-core products ("achievable"); the
headline also reports its rates as fractions of those.

Each workload reports a roofline: algorithmic bytes (every input read once,
every output written once) and, for the chunk forward, algorithmic matrix
flops, divided by the measured launch time, against the published MI355X
peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16).  "traffic" and the executed
matrix-core figures come from committed rocprofv3 counter runs
(profiles/counters.json) and are reported only while the kernel source is
unchanged since those runs.

With --gate head (one decay per token and head: Gated DeltaNet) or --gate
none (no forget gate: DeltaNet) the headline and decode workloads run
through the *_gated entry points; with --fused the inputs are stored raw
(gate logits in bf16, beta logits, q and k not normalised) and the *_fused
entry points prepare them in the kernel.  --only runs a single workload
(for profiling).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--gate channel|head|none] [--fused] [--only NAME] [--no-flush]
                       [--calib-copy] [--prep-baseline] [--no-peaks] [--no-graph]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix throughput, published (no sparsity)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "gated_delta_rule_38_amd", "csrc")
CHUNK = 64
# the sources each timed kernel is compiled from (its counters go stale when any changes)
KERNEL_SOURCES = {
    "chunk_fwd_bf16_kernel": ["chunk_fwd_bf16.hip", "chunk_walk.h", "chunk_common.h", "kda_device.h"],
    # the two-segment path of long dense sequences: its three chunk-kernel
    # launches, the final states and the output correction, and its plan
    "chunk_split_path": ["chunk_split.hip", "chunk_fwd_bf16.hip", "chunk_walk.h", "chunk_common.h",
                         "kda_device.h", "kda_sizes.cpp"],
    "recurrent_step_kernel": ["recurrent_step.hip", "kda_device.h"],
    "bwd_chunk_kernel": ["bwd_chunk.hip", "chunk_fwd.hip", "chunk_walk.h", "chunk_common.h",
                         "kda_device.h"],
    "gdn2_chunk_kernel": ["gdn2_chunk.hip", "chunk_walk.h", "chunk_common.h", "kda_device.h"],
    "gdn2_step_kernel": ["gdn2_step.hip", "kda_device.h"],
}
WORKLOADS = ["headline", "long_context", "varlen", "decode", "backward", "gdn2"]


def _code_only(text):
    """C++ source with comments and blank space removed: edits to comments do
    not change the compiled kernel, so they do not retire measured counters."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel):
    """Hash of the sources of a kernel; "name[...]" names an instantiation or a
    workload of the same sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel.split("[")[0]]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_counters(kernel):
    """The committed counter record of a kernel (HBM bytes, matrix-core
    figures per launch), or {} when absent or taken on other sources."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return {}
    if rec.get("source_sha256_16") != source_hash(kernel):
        return {}
    return rec


# alpha values per token and head for each forget gate
GATE_WIDTH = {"channel": lambda dk: dk, "head": lambda dk: 1, "none": lambda dk: 0}
GATE_NAME = {"channel": "KDA", "head": "Gated DeltaNet", "none": "DeltaNet"}


def chunk_bytes(tokens, H, dk, dv, nstates, es=2, gate="channel", ges=4, initial=True):
    """Algorithmic HBM bytes of one chunk-wise forward over `tokens` packed
    tokens: every input read once, every output written once (ges: bytes per
    gate element, 4 for float32 alpha, es for logits in the storage dtype;
    initial: whether an initial state is read)."""
    tok = tokens * H
    aw = GATE_WIDTH[gate](dk)
    return (tok * (2 * dk * es + dv * es + aw * ges + 4 + dv * es)  # q, k, v, alpha, beta, o
            + (2 if initial else 1) * nstates * H * dk * dv * 4)     # initial + final state


def chunk_flops(tokens, H, dk, dv, C=CHUNK):
    """Algorithmic matrix flops of one chunk-wise forward, triangle-aware, per
    token and head: 6 dk dv (three state-sized products: Kr S, Qr S and the
    state update) + C (3 dk + 2 dv) (the Gram, the intra-chunk attention, the
    solve and M U, each over half a chunk on average) + 2 C^2 / 3 (the
    triangular inverse)."""
    return tokens * H * (6 * dk * dv + C * (3 * dk + 2 * dv) + 2 * C * C / 3)


def gdn2_chunk_bytes(tokens, H, dk, dv, nstates, es=2, initial=True):
    """Algorithmic HBM bytes of one Gated DeltaNet-2 chunk-wise forward: q, k, v
    and o in the storage dtype, alpha, erase and write float32 per key channel,
    the states float32."""
    return (tokens * H * (2 * dk * es + dv * es + 3 * dk * 4 + dv * es)
            + (2 if initial else 1) * nstates * H * dk * dv * 4)


def gdn2_chunk_flops(tokens, H, dk, dv, C=CHUNK):
    """Algorithmic matrix flops of one Gated DeltaNet-2 chunk-wise forward per
    token and head: 8 dk dv (Kr S, Qr S, and the state update over the two
    rows each token writes) + C (4 dk + 4 dv) (four Gram products, L_c V, the
    solve and the two-row intra-chunk product, each over half a chunk on
    average) + 2 C^2 / 3 (the triangular inverse)."""
    return tokens * H * (8 * dk * dv + C * (4 * dk + 4 * dv) + 2 * C * C / 3)


def gdn2_step_bytes(N, H, dk, dv, es=2):
    """Algorithmic HBM bytes of one Gated DeltaNet-2 decode step."""
    return N * H * (2 * dk * dv * 4 + (2 * dk + dv) * es + 3 * dk * 4 + dv * es)


def decode_bytes(N, H, dk, dv, es=2, gate="channel", ges=4):
    """Algorithmic HBM bytes of one decode step."""
    aw = GATE_WIDTH[gate](dk)
    return N * H * (2 * dk * dv * 4 + (2 * dk + dv) * es + aw * ges + 4 + dv * es)


def backward_bytes(tokens, H, dk, dv, nstates, es=2):
    """Algorithmic HBM bytes of one backward call: q, k, v, alpha, beta, dout,
    S0 and dS_T read once; dq, dk, dv, dalpha, dbeta (float32) and dS0 written
    once."""
    return (tokens * H * (2 * dk * es + dv * es + dk * 4 + 4 + dv * es
                          + 4 * (2 * dk + dv + dk) + 4) + 3 * nstates * H * dk * dv * 4)


def backward_flops(tokens, H, dk, dv, C=CHUNK):
    """Algorithmic matrix flops of one chunk-form backward call, triangle-aware,
    per token and head: the forward that stores the chunk-start states
    (chunk_flops) and the reverse sweep, 14 dk dv (seven state-sized products:
    Kr SP, Kc dW, dO SP^T, dX SP^T, U dW^T, Qr^T dO, Kr^T dX) + C (6 dk + 5 dv)
    (A and M again, dM Kc, dA Kc, dA^T Kr, dM^T Qr over the key channels;
    M^T dO, T'^T dU, T' Y, dY U^T, dO U^T over the value columns, each over
    half a chunk on average) + 2 C^2 / 3 (the triangular inverse again)."""
    return (chunk_flops(tokens, H, dk, dv, C)
            + tokens * H * (14 * dk * dv + C * (6 * dk + 5 * dv) + 2 * C * C / 3))


def roofline(bytes_alg, ms, kernel, flops_alg=None):
    """The roofline object for one kernel: algorithmic bytes (and flops) per
    launch over the measured launch time against the published peaks."""
    gbs = bytes_alg / (ms / 1e3) / 1e9
    rec = measured_counters(kernel)
    r = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": gbs / HBM_PEAK_GBS, "traffic": rec.get("bytes_per_launch"),
         "kernel": kernel.split("[")[0], "algorithmic_bytes_per_launch": bytes_alg,
         "avg_launch_ms": ms}
    if flops_alg is not None:
        tfs = flops_alg / (ms / 1e3) / 1e12
        r["mfma"] = {"achieved": tfs, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": tfs / MFMA_BF16_PEAK_TFS, "algorithmic_flops_per_launch": flops_alg}
        if rec.get("mfma_flops_bf16_per_launch") is not None:
            r["mfma"]["executed_flops_per_launch"] = rec["mfma_flops_bf16_per_launch"]
            r["mfma"]["busy_frac"] = rec.get("mfma_busy_frac")
        # fraction of the binding roofline: the larger of the two floors over the time
        floor = max(flops_alg / (MFMA_BF16_PEAK_TFS * 1e12), bytes_alg / (HBM_PEAK_GBS * 1e9))
        r["binding_frac"] = floor / (ms / 1e3)
        if flops_alg / (MFMA_BF16_PEAK_TFS * 1e12) > bytes_alg / (HBM_PEAK_GBS * 1e9):
            r["bound"] = "mfma"
    return r


def achievable_peaks(torch, dev, stream):
    """What this GPU reaches on the two roofline resources, measured with the
    benchmark's own kernels (libkda_peaks.so): a streaming 1 GiB copy and a
    1 GiB read-only stream (HBM GB/s; the copy counts its reads and writes)
    and independent chains of bf16 16x16x32 matrix-core products on every
    SIMD (TFLOP/s).  Each is the best of 5 timed launches after 2 warm-ups."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_delta_rule_38_amd", "libkda_peaks.so"))
    vp, sz, i, u32, f = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32,
                         ctypes.c_float)
    lib.kda_peak_copy.argtypes = [vp, vp, sz, i, vp]
    lib.kda_peak_read.argtypes = [vp, sz, u32, vp, i, vp]
    lib.kda_peak_mfma.argtypes = [i, f, vp, i, vp]
    st = ctypes.c_void_p(stream.cuda_stream)
    blocks = 256 * 8
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def best(launch):
        for _ in range(2):
            launch()
        ts = []
        for _ in range(5):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return min(ts)

    def ok(rc):
        if rc != 0:
            raise RuntimeError("peak probe failed with hipError %d" % rc)
    t_copy = best(lambda: ok(lib.kda_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks,
                                               st)))
    t_read = best(lambda: ok(lib.kda_peak_read(src.data_ptr(), nbytes, 0x9E3779B9,
                                               sink.data_ptr(), blocks, st)))
    iters = 20000
    chains = lib.kda_peak_mfma_chains()
    t_mfma = best(lambda: ok(lib.kda_peak_mfma(iters, 12345.678, sink.data_ptr(), blocks, st)))
    flops = blocks * 4 * chains * iters * 2 * 16 * 16 * 32
    del src, dst, sink
    return {"hbm_copy_GBs": 2 * nbytes / t_copy / 1e9, "hbm_read_GBs": nbytes / t_read / 1e9,
            "mfma_bf16_TFs": flops / t_mfma / 1e12,
            "how": "libkda_peaks.so: 1 GiB streaming copy (reads + writes counted), 1 GiB "
                   "read-only stream, %d workgroups x 4 waves x %d chains of %d bf16 "
                   "16x16x32 MFMA; best of 5 launches" % (blocks, chains, iters)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The shader clock climbs for some 25 ms of this work (about 1.9 to 2.35 GHz,
    # read with s_memtime against s_memrealtime from a one-wave sampler on a second
    # stream); 200 warm-up steps (~36 ms) put the timed steps at the steady clock.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the decode steps replayed from a HIP graph")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the achievable HBM and matrix-core rates")
    ap.add_argument("--only", choices=WORKLOADS, default=None,
                    help="run one workload only (profiling runs)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the single launches timed after a cache flush")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--gate", choices=sorted(GATE_WIDTH), default="channel",
                    help="forget gate: per key channel (KDA, the default), per head (Gated "
                         "DeltaNet) or none (DeltaNet)")
    ap.add_argument("--fused", action="store_true",
                    help="raw inputs (bf16 gate logits, beta logits, q and k not normalised) "
                         "prepared in the kernel")
    ap.add_argument("--prep-baseline", action="store_true",
                    help="with --fused: also time the same preparation done by torch "
                         "elementwise kernels followed by the plain entry point")
    args = ap.parse_args()
    gate = args.gate
    fused = args.fused
    fl = dict(gate_logits=gate != "none", beta_logits=True, qk_l2norm=True)
    ges = 2 if fused else 4
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the workload shards by (batch, head) with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    plain = gate == "channel" and not fused
    run = {w: (args.only is None or args.only == w) for w in WORKLOADS}
    if args.skip_decode:
        run["decode"] = False
    if not plain:  # the variants cover the headline and the decode step
        run["long_context"] = run["varlen"] = run["backward"] = run["gdn2"] = False

    import torch
    import gated_delta_rule_38_amd as kda
    from workloads import CONFIGS, gen

    dev = torch.device("cuda:0")
    kda.load_library()
    stream = torch.cuda.current_stream(dev)  # the launch stream of every libkda call

    def timed(fn, steps, warmup):
        """Average ms per call over `steps` calls after `warmup` untimed ones,
        HIP events on the launch stream around the whole loop."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    flush_buf = [None]

    def flushed(fn, n):
        """Median and min ms of n single calls, each after a 1 GiB read (a sum
        over a buffer) that leaves none of the call's inputs in the caches and
        only clean lines behind (a write there would leave dirty lines whose
        write-back then competes with the call)."""
        if flush_buf[0] is None:
            flush_buf[0] = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        ts = []
        for _ in range(n):
            flush_buf[0].sum()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        return {"median_ms": ts[len(ts) // 2], "min_ms": ts[0], "launches": n}

    out = {}
    if not args.no_peaks:
        out["achievable"] = achievable_peaks(torch, dev, stream)
    cfg = CONFIGS[1]
    B, T, H, dk, dv = cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv
    d = None
    if run["headline"] or run["backward"] or not args.no_cpu_baseline:
        d = gen.chunk_inputs(cfg, device=dev, gate=gate, raw=fused)

    def headline_leg():
        """The headline leg: kda_chunk_fwd (or the variant chosen) on B4 H16 T4096."""
        if run["headline"]:
            o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
            fs = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)

            def step():
                if fused:
                    kda.kda_chunk_fwd_fused(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                            d["initial_state"], o=o, final_state=fs, gate_kind=gate,
                                            **fl)
                elif gate == "channel":
                    kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                      d["initial_state"], o=o, final_state=fs)
                else:
                    kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                            d["initial_state"], o=o, final_state=fs, gate=gate)

            t0 = time.perf_counter()
            ms = timed(step, args.steps, args.warmup)
            wall = time.perf_counter() - t0
            variant = ([] if gate == "channel" else ["gate=%s" % gate]) + (["fused"] if fused else [])
            kname = "chunk_fwd_bf16_kernel" + ("[%s]" % ",".join(variant) if variant else "")
            wl = {"channel": "kda_chunk_fwd", "head": "kda_chunk_fwd_gated (per-head alpha)",
                  "none": "kda_chunk_fwd_gated (no gate)"}[gate]
            if fused:
                wl = ("kda_chunk_fwd_fused (%s gate, bf16 gate logits, beta logits, q/k L2 norm "
                      "in-kernel)" % gate)
            out.update({
                "metric": "%s%s chunk-fwd tokens/s (B4 H16 T4096 d128) + decode GB/s vs roofline" % (
                    GATE_NAME[gate], " (fused input preparation)" if fused else ""),
                "value": B * T / (ms / 1e3),
                "unit": "tokens/s",
                "n_gpus": 1,
                "steps": args.steps,
                "warmup": args.warmup,
                "ms_per_step": ms,
                "higher_is_better": True,
                "scaling": "weak",
                "vs_baseline": None,
                "dtype": "bf16",
                "data": "synthetic",
                "config": {"workload": wl + " bf16 B4 H16 T4096 dk128 dv128 chunk64, "
                                       "initial state N(0,0.02)",
                           "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": CHUNK,
                           "parallelism": "single GPU"},
                "roofline": roofline(chunk_bytes(B * T, H, dk, dv, B, gate=gate, ges=ges), ms, kname,
                                     chunk_flops(B * T, H, dk, dv)),
                "timed_wall_s": wall,
                "timed_after": [w for w in ("decode", "gdn2", "backward", "long_context",
                                            "varlen") if run[w]],
            })
            if "achievable" in out:
                rf = out["roofline"]
                rf["frac_of_achievable_read"] = rf["achieved"] / out["achievable"]["hbm_read_GBs"]
                if "mfma" in rf:
                    rf["mfma"]["frac_of_achievable"] = (rf["mfma"]["achieved"] /
                                                        out["achievable"]["mfma_bf16_TFs"])
            if not args.no_flush:
                out["roofline"]["hbm_cold"] = flushed(step, 20)

            if fused and args.prep_baseline:
                def prep():
                    qn = torch.nn.functional.normalize(d["q"].float(), dim=-1, eps=1e-3).to(
                        d["q"].dtype)
                    kn = torch.nn.functional.normalize(d["k"].float(), dim=-1, eps=1e-3).to(
                        d["k"].dtype)
                    a = None if d["alpha"] is None else torch.sigmoid(d["alpha"].float())
                    return qn, kn, a, torch.sigmoid(d["beta"])

                def unfused():
                    qn, kn, a, b = prep()
                    kda.kda_chunk_fwd_gated(qn, kn, d["v"], a, b, d["initial_state"], o=o,
                                            final_state=fs, gate=gate)
                n = max(10, args.steps // 2)
                out["prep_baseline"] = {
                    "what": "torch elementwise preparation (normalise q and k, sigmoid of the "
                            "logits) then kda_chunk_fwd_gated, same inputs",
                    "prep_ms": timed(prep, n, n), "prep_plus_chunk_ms": timed(unfused, n, n),
                    "fused_ms": ms}
            del o, fs


    if run["decode"]:
        dc = CONFIGS[3]
        ddc = gen.decode_inputs(dc, device=dev, gate=gate, raw=fused)
        state = ddc["state"].clone()
        od = torch.empty((dc.B, dc.H, dc.dv), dtype=torch.bfloat16, device=dev)
        sargs = [[None if ddc[n] is None else ddc[n][t] for n in ("q", "k", "v", "alpha", "beta")]
                 for t in range(dc.steps)]

        def dstep(t, st):
            if fused:
                kda.kda_recurrent_step_fused(*sargs[t], st, o=od, gate_kind=gate, **fl)
            elif gate == "channel":
                kda.kda_recurrent_step(*sargs[t], st, o=od)
            else:
                kda.kda_recurrent_step_gated(*sargs[t], st, o=od, gate=gate)
        warm = state.clone()
        for t in range(3):
            dstep(t, warm)
        torch.cuda.synchronize()
        del warm
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for t in range(dc.steps):
            dstep(t, state)
        f1.record(stream)
        torch.cuda.synchronize()
        us = f0.elapsed_time(f1) * 1e3 / dc.steps
        dbytes = decode_bytes(dc.B, dc.H, dc.dk, dc.dv, gate=gate, ges=ges)
        kname = "recurrent_step_kernel" + ("" if plain else "[variant]")
        out["decode"] = {
            "workload": "%s bf16 N256 H32 dk128 dv128, fp32 state in place, "
                        "100 consecutive steps" % (
                            "kda_recurrent_step_fused (gate %s)" % gate if fused else
                            "kda_recurrent_step" if gate == "channel" else
                            "kda_recurrent_step_gated (gate %s)" % gate),
            "us_per_step": us, "tokens_per_s": dc.B / (us / 1e6),
            "roofline": roofline(dbytes, us / 1e3, kname),
        }
        if not args.no_graph:
            # the same 100 steps captured once in a HIP graph and replayed: checked against
            # the eager steps from the same start, then timed over 5 replays
            ge = ddc["state"].clone()
            for t in range(dc.steps):
                dstep(t, ge)
            torch.cuda.synchronize()
            oe = od.clone()
            gs = ddc["state"].clone()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for t in range(dc.steps):
                    dstep(t, gs)
            graph.replay()
            torch.cuda.synchronize()
            same = bool(torch.equal(gs, ge) and torch.equal(od, oe))
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            for _ in range(5):
                graph.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            gus = g0.elapsed_time(g1) * 1e3 / (5 * dc.steps)
            out["decode"]["graph"] = {
                "what": "the 100 steps captured in one HIP graph, 5 replays timed",
                "us_per_step": gus, "tokens_per_s": dc.B / (gus / 1e6),
                "achieved_GBs": decode_bytes(dc.B, dc.H, dc.dk, dc.dv, gate=gate, ges=ges) /
                (gus / 1e6) / 1e9, "replay_equals_eager": same}
            out["decode"]["graph"]["frac"] = out["decode"]["graph"]["achieved_GBs"] / HBM_PEAK_GBS
            del ge, gs, oe, graph
        if not args.no_flush:
            cnt = [0]

            def one():
                dstep(cnt[0] % dc.steps, state)
                cnt[0] += 1
            cold = flushed(one, 20)
            cold["achieved_GBs_median"] = dbytes / (cold["median_ms"] / 1e3) / 1e9
            cold["frac_median"] = cold["achieved_GBs_median"] / HBM_PEAK_GBS
            out["decode"]["roofline"]["hbm_cold"] = cold
        if "value" not in out:  # --only decode: the decode step is the line's workload
            out.update({"metric": "KDA decode step GB/s (N256 H32 d128) vs roofline",
                        "value": dbytes / (us / 1e6) / 1e9, "unit": "GB/s", "n_gpus": 1,
                        "steps": dc.steps, "warmup": 3, "ms_per_step": us / 1e3,
                        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                        "dtype": "f32", "data": "synthetic",
                        "config": {"workload": out["decode"]["workload"]},
                        "roofline": out["decode"]["roofline"]})
        del ddc, state, sargs

    if run["gdn2"]:
        g2 = gen.draw_gdn2(B, T, H, dk, dv, "bf16", alpha_mu=4.0, s0_std=0.02, seed=1, device=dev)
        og = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
        fg = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)

        def gstep():
            kda.kda_gdn2_chunk_fwd(g2["q"], g2["k"], g2["v"], g2["alpha"], g2["erase"],
                                   g2["write"], g2["initial_state"], o=og, final_state=fg)
        gms = timed(gstep, args.steps, args.warmup if args.only else max(5, args.warmup // 10))
        out["gdn2"] = {
            "workload": "kda_gdn2_chunk_fwd (Gated DeltaNet-2: per-channel forget, erase and "
                        "write gates) bf16 B4 H16 T4096 dk128 dv128 chunk64, initial state "
                        "N(0,0.02)",
            "ms_per_step": gms, "tokens_per_s": B * T / (gms / 1e3),
            "roofline": roofline(gdn2_chunk_bytes(B * T, H, dk, dv, B), gms, "gdn2_chunk_kernel",
                                 gdn2_chunk_flops(B * T, H, dk, dv))}
        if not args.no_flush:
            out["gdn2"]["roofline"]["hbm_cold"] = flushed(gstep, 10)
        del g2, og, fg
        dc = CONFIGS[3]
        g = torch.Generator(device=dev)
        g.manual_seed(3)
        gst = (0.05 * torch.randn((dc.B, dc.H, dc.dk, dc.dv), generator=g, device=dev,
                                  dtype=torch.float64)).float()
        steps_in = gen.draw_gdn2(dc.B, 8, dc.H, dc.dk, dc.dv, "bf16", alpha_mu=4.0, seed=5,
                                 device=dev)
        sin = [[steps_in[n][:, t].contiguous() for n in ("q", "k", "v", "alpha", "erase",
                                                          "write")] for t in range(8)]
        ogd = torch.empty((dc.B, dc.H, dc.dv), dtype=torch.bfloat16, device=dev)
        cnt = [0]

        def gdstep():
            kda.kda_gdn2_recurrent_step(*sin[cnt[0] % 8], gst, o=ogd)
            cnt[0] += 1
        gus = timed(gdstep, dc.steps, 3) * 1e3
        gb = gdn2_step_bytes(dc.B, dc.H, dc.dk, dc.dv)
        out["gdn2_decode"] = {
            "workload": "kda_gdn2_recurrent_step bf16 N256 H32 dk128 dv128, fp32 state in place, "
                        "100 consecutive steps (8 input sets in turn)",
            "us_per_step": gus, "tokens_per_s": dc.B / (gus / 1e6),
            "roofline": roofline(gb, gus / 1e3, "gdn2_step_kernel")}
        del gst, steps_in, sin, ogd

    if run["backward"]:
        gg = torch.Generator(device=dev)
        gg.manual_seed(11)
        dout = torch.randn((B, T, H, dv), generator=gg, device=dev).to(d["q"].dtype)
        dsT = torch.randn((B, H, dk, dv), generator=gg, device=dev)
        ws = torch.empty(max(1, kda.kda_backward_workspace_size(B, T, H, dk, dv, 0)),
                         dtype=torch.uint8, device=dev)

        def bstep():
            return kda.kda_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                    d["initial_state"], dout, dsT, workspace=ws)
        nb = max(2, args.steps // 20)
        bms = timed(bstep, nb, 2)
        out["backward"] = {
            "workload": "kda_backward bf16 B4 H16 T4096 dk128 dv128 (per-channel gate), "
                        "fp32 gradients",
            "ms_per_step": bms, "tokens_per_s": B * T / (bms / 1e3),
            "roofline": roofline(backward_bytes(B * T, H, dk, dv, B), bms, "bwd_chunk_kernel",
                                 backward_flops(B * T, H, dk, dv))}
        del dout, dsT, ws

    for name, ci in (("long_context", 2), ("varlen", 4)):
        if not run[name]:
            continue
        c = CONFIGS[ci]
        dd = gen.chunk_inputs(c, device=dev)
        toks = dd["q"].shape[0] * dd["q"].shape[1]
        nst = dd["cu_seqlens"].numel() - 1 if dd["cu_seqlens"] is not None else c.B
        ol = torch.empty_like(dd["v"])
        fl_ = torch.empty((nst, c.H, c.dk, c.dv), dtype=torch.float32, device=dev)
        wsb = kda.kda_chunk_fwd_workspace_size(1, toks, c.H, c.dk, c.dv,
                                               nst if dd["cu_seqlens"] is not None else 0)
        # dense shapes with few units and long sequences take the two-segment
        # path when the workspace holds its buffers
        split_b = 0 if dd["cu_seqlens"] is not None else kda.kda_chunk_fwd_split_workspace_size(
            c.B, c.T, c.H, c.dk, c.dv)
        ws = torch.empty(max(1, wsb, split_b), dtype=torch.uint8, device=dev)

        def lstep():
            kda.kda_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"],
                              dd["initial_state"], cu_seqlens=dd["cu_seqlens"],
                              cu_seqlens_host=dd["cu_seqlens_host"], o=ol, final_state=fl_,
                              workspace=ws)
        lms = timed(lstep, args.steps, args.warmup if args.only else max(5, args.warmup // 10))
        desc = ("kda_chunk_fwd bf16 B1 H32 T65536 dk128 dv128 chunk64, zero initial state, "
                "alpha = sigmoid(N(5,1))" if name == "long_context" else
                "kda_chunk_fwd bf16 varlen: 64 packed sequences, lengths U{128..8192} "
                "(%d tokens), H16 dk128 dv128, initial states N(0,0.02)" % toks)
        out[name] = {"workload": desc, "ms_per_step": lms, "tokens_per_s": toks / (lms / 1e3),
                     "path": "two time segments at once" if split_b else "single pass",
                     "roofline": roofline(chunk_bytes(toks, c.H, c.dk, c.dv, nst,
                                                      initial=dd["initial_state"] is not None),
                                          lms,
                                          ("chunk_split_path[%s]" if split_b else
                                           "chunk_fwd_bf16_kernel[%s]") % name,
                                          chunk_flops(toks, c.H, c.dk, c.dv))}
        if not args.no_flush:
            out[name]["roofline"]["hbm_cold"] = flushed(lstep, 5)
        del dd, ol, fl_, ws

    # The headline leg runs after the other legs, the chunk-kernel legs (long context,
    # varlen) last: they bring the shader clock to the chunk kernel's steady value (it climbs
    # for some 25 ms of chunk-kernel work, and memory-bound decode steps leave it lower), so
    # the headline's timed steps run at that clock whatever the warm-up count.  With --only headline the default
    # 200 warm-up steps do the same.
    headline_leg()

    for name in ("long_context", "varlen", "backward", "gdn2"):  # --only of one of these
        if "value" not in out and name in out:
            rec = out[name]
            out.update({"metric": "KDA %s tokens/s vs roofline" % name, "value":
                        rec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                        "steps": args.steps, "warmup": args.warmup,
                        "ms_per_step": rec["ms_per_step"], "higher_is_better": True,
                        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                        "data": "synthetic", "config": {"workload": rec["workload"]},
                        "roofline": rec["roofline"]})

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = src.numel() * 4

    if not args.no_cpu_baseline and d is not None:
        import oracle
        # one unit per (batch, head): [B*H, T, d] blocks of the stored inputs
        def units(x):
            x = x.cpu()
            return x.transpose(1, 2).reshape((B * H, T) + tuple(x.shape[3:])).contiguous()
        host = {n: units(d[n]) for n in ("q", "k", "v", "beta")}
        s0 = d["initial_state"].cpu().reshape(B * H, dk, dv)
        cores = min(len(os.sched_getaffinity(0)), B * H)
        c0 = time.perf_counter()
        a_units = None if d["alpha"] is None else units(d["alpha"])
        if fused:
            qh, kh, alpha, bh = oracle.prepare(host["q"], host["k"], a_units, host["beta"], gate,
                                               lead=(B * H, T), **fl)
        else:
            qh, kh, bh = host["q"], host["k"], host["beta"]
            alpha = oracle.channel_gate(a_units, gate, dk, (B * H, T))
        oracle.forward_units(qh, kh, host["v"], alpha, bh, s0, threads=cores)
        cw = time.perf_counter() - c0
        out["cpu_baseline"] = {"value": B * T / cw, "unit": "tokens/s", "cores": cores,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": "the whole B4 H16 T4096 workload (64 (batch, head) "
                                         "units x 4096 tokens), fp64 token loop incl. input "
                                         "widening; wall %.2f s" % cw}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
