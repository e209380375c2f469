"""Benchmark of the KDA hot path on one MI355X.

One step = one kda_chunk_fwd call over the headline workload (bf16, B=4,
H=16, T=4096, dk=dv=128, chunk 64, nonzero initial state), inputs already
resident in HBM.  value = tokens per second (B*T tokens per step).  The same
line also carries the decode workload (256 sequences x 32 heads, d=128, fp32
state in place, 100 consecutive steps) as GB/s against the HBM roofline.

With --gate head (one decay per token and head: Gated DeltaNet) or --gate
none (no forget gate: DeltaNet) the same workloads run through the *_gated
entry points with alpha drawn per head (or absent); the default is the
per-channel gate of KDA.  With --fused the inputs are stored raw (gate
logits in bf16, beta logits, q and k not normalised) and the *_fused entry
points prepare them in the kernel.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--calib-copy] [--skip-decode] [--gate channel|head|none] [--fused]
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "gated_delta_rule_38_amd", "csrc")
# the sources each timed kernel is compiled from (its counters go stale when any changes)
KERNEL_SOURCES = {
    "chunk_fwd_bf16_kernel": ["chunk_fwd_bf16.hip", "chunk_common.h", "kda_device.h"],
    "recurrent_step_kernel": ["recurrent_step.hip", "kda_device.h"],
    "backward_kernel": ["backward.hip", "kda_device.h"],
}


def _code_only(text):
    """C++ source with comments and blank space removed: edits to comments do
    not change the compiled kernel, so they do not retire measured counters."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel):
    """Hash of the sources of a kernel; "name[gate=...]" names an instantiation
    of the same sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel.split("[")[0]]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when absent or taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


# alpha values per token and head for each forget gate
GATE_WIDTH = {"channel": lambda dk: dk, "head": lambda dk: 1, "none": lambda dk: 0}
GATE_NAME = {"channel": "KDA", "head": "Gated DeltaNet", "none": "DeltaNet"}


def chunk_bytes(B, T, H, dk, dv, es=2, nstates=None, gate="channel", ges=4):
    """Algorithmic HBM bytes of one chunk-wise forward: every input read once,
    every output written once (ges: bytes per gate element, 4 for float32
    alpha, es for logits in the storage dtype)."""
    ns = B if nstates is None else nstates
    tok = B * T * H
    aw = GATE_WIDTH[gate](dk)
    return (tok * (2 * dk * es + dv * es + aw * ges + 4 + dv * es)  # q, k, v, alpha, beta, o
            + 2 * ns * H * dk * dv * 4)                              # initial + final state


def decode_bytes(N, H, dk, dv, es=2, gate="channel", ges=4):
    """Algorithmic HBM bytes of one decode step."""
    aw = GATE_WIDTH[gate](dk)
    return N * H * (2 * dk * dv * 4 + (2 * dk + dv) * es + aw * ges + 4 + dv * es)


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
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--gate", choices=sorted(GATE_WIDTH), default="channel",
                    help="forget gate: per key channel (KDA, the default), per head (Gated "
                         "DeltaNet) or none (DeltaNet)")
    ap.add_argument("--fused", action="store_true",
                    help="raw inputs (bf16 gate logits, beta logits, q and k not normalised) "
                         "prepared in the kernel")
    ap.add_argument("--backward", action="store_true",
                    help="also time kda_backward (gradients of the same forward, random dL/do "
                         "and dL/dS_T) on the chunk workload")
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
              "(the workload shards by (batch, head) with no exchange; see DESIGN.md). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_38_amd as kda
    from workloads import CONFIGS, gen

    dev = torch.device("cuda:0")
    kda.load_library()
    cfg = CONFIGS[1]
    d = gen.chunk_inputs(cfg, device=dev, gate=gate, raw=fused)
    B, T, H, dk, dv = cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)

    def step():
        if fused:
            kda.kda_chunk_fwd_fused(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                    d["initial_state"], o=o, final_state=fs, gate_kind=gate, **fl)
        elif gate == "channel":
            kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                              o=o, final_state=fs)
        else:
            kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                    d["initial_state"], o=o, final_state=fs, gate=gate)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)  # the launch stream of kda_chunk_fwd
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    tokens = B * T
    value = tokens * args.steps / (ms * args.steps / 1e3)
    alg = chunk_bytes(B, T, H, dk, dv, gate=gate, ges=ges)
    achieved = alg / (ms / 1e3) / 1e9
    variant = ([] if gate == "channel" else ["gate=%s" % gate]) + (["fused"] if fused else [])
    traffic = measured_traffic("chunk_fwd_bf16_kernel" +
                               ("[%s]" % ",".join(variant) if variant else ""))
    gname = GATE_NAME[gate]
    wl = {"channel": "kda_chunk_fwd", "head": "kda_chunk_fwd_gated (per-head alpha)",
          "none": "kda_chunk_fwd_gated (no gate)"}[gate]
    if fused:
        wl = ("kda_chunk_fwd_fused (%s gate, bf16 gate logits, beta logits, q/k L2 norm "
              "in-kernel)" % gate)

    out = {
        "metric": "%s%s chunk-fwd tokens/s (B4 H16 T4096 d128) + decode GB/s vs roofline" % (
            gname, " (fused input preparation)" if fused else ""),
        "value": value,
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
                   "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": 64,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "chunk_fwd_bf16_kernel", "algorithmic_bytes_per_launch": alg,
                     "avg_launch_ms": ms},
        "timed_wall_s": wall,
    }

    if fused and args.prep_baseline:
        def prep():
            qn = torch.nn.functional.normalize(d["q"].float(), dim=-1, eps=1e-3).to(d["q"].dtype)
            kn = torch.nn.functional.normalize(d["k"].float(), dim=-1, eps=1e-3).to(d["k"].dtype)
            a = None if d["alpha"] is None else torch.sigmoid(d["alpha"].float())
            return qn, kn, a, torch.sigmoid(d["beta"])

        def unfused():
            qn, kn, a, b = prep()
            kda.kda_chunk_fwd_gated(qn, kn, d["v"], a, b, d["initial_state"], o=o, final_state=fs,
                                    gate=gate)

        def time_fn(fn, n):
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            for _ in range(n):
                fn()
            g1.record(stream)
            torch.cuda.synchronize()
            return g0.elapsed_time(g1) / n
        n = max(10, args.steps // 2)
        out["prep_baseline"] = {
            "what": "torch elementwise preparation (normalise q and k, sigmoid of the logits) "
                    "then kda_chunk_fwd_gated, same inputs",
            "prep_ms": time_fn(prep, n), "prep_plus_chunk_ms": time_fn(unfused, n),
            "fused_ms": ms}

    if args.backward and gate == "channel" and not fused:
        gg = torch.Generator(device=dev)
        gg.manual_seed(11)
        dout = torch.randn((B, T, H, dv), generator=gg, device=dev).to(d["q"].dtype)
        dsT = torch.randn((B, H, dk, dv), generator=gg, device=dev)
        ws = torch.empty(kda.kda_backward_workspace_size(B, T, H, dk, dv, 0), dtype=torch.uint8,
                         device=dev)

        def bstep():
            return kda.kda_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                    d["initial_state"], dout, dsT, workspace=ws)
        nb = max(2, args.steps // 20)
        for _ in range(2):
            bstep()
        torch.cuda.synchronize()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(nb):
            bstep()
        b1.record(stream)
        torch.cuda.synchronize()
        bms = b0.elapsed_time(b1) / nb
        # inputs q, k, v, alpha, beta, dout, S0, dS_T read once; dq, dk, dv,
        # dalpha, dbeta (fp32) and dS_0 written once
        es = 2
        bbytes = (B * T * H * (2 * dk * es + dv * es + dk * 4 + 4 + dv * es
                               + 4 * (2 * dk + dv + dk) + 4) + 3 * B * H * dk * dv * 4)
        out["backward"] = {
            "workload": "kda_backward bf16 B4 H16 T4096 dk128 dv128 (per-channel gate), "
                        "fp32 gradients",
            "ms_per_step": bms, "tokens_per_s": B * T / (bms / 1e3),
            "roofline": {"bound": "hbm", "achieved": bbytes / (bms / 1e3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bbytes / (bms / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("backward_kernel"),
                         "kernel": "backward_kernel", "algorithmic_bytes_per_launch": bbytes}}

    if not args.skip_decode:
        dc = CONFIGS[3]
        dd = gen.decode_inputs(dc, device=dev, gate=gate, raw=fused)
        state = dd["state"].clone()
        od = torch.empty((dc.B, dc.H, dc.dv), dtype=torch.bfloat16, device=dev)
        sargs = [[None if dd[n] is None else dd[n][t] for n in ("q", "k", "v", "alpha", "beta")]
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
        gbs = dbytes / (us / 1e6) / 1e9
        out["decode"] = {
            "workload": "%s bf16 N256 H32 dk128 dv128, fp32 state in place, "
                        "100 consecutive steps" % (
                            "kda_recurrent_step_fused (gate %s)" % gate if fused else
                            "kda_recurrent_step" if gate == "channel" else
                            "kda_recurrent_step_gated (gate %s)" % gate),
            "us_per_step": us, "tokens_per_s": dc.B / (us / 1e6),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("recurrent_step_kernel")
                         if gate == "channel" and not fused else None,
                         "kernel": "recurrent_step_kernel",
                         "algorithmic_bytes_per_launch": dbytes},
        }

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = src.numel() * 4

    if not args.no_cpu_baseline:
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
        out["cpu_baseline"] = {"value": tokens / cw, "unit": "tokens/s", "cores": cores,
                               "kind": "oracle",
                               "sample": "the whole B4 H16 T4096 workload (64 (batch, head) "
                                         "units x 4096 tokens), fp64 token loop incl. input "
                                         "widening; wall %.2f s" % cw}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
