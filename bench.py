"""Throughput of libgdr on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long|prefill|varlen]
                    [--no-cpu-baseline] [--chunk-only]

One step is one pass of the whole hot path on synthetic, seeded inputs that
are resident in HBM before the timed region starts:
  * gdr_chunk_fwd on the chunk workload (default ``long``: B=1, T=32768,
    Nqk=16, Nv=32, D=128, bf16 q/k/v, fp32 gates and states, the largest
    single-GPU workload), and
  * gdr_recurrent_step on the decode workload (256 sequences x 1 token, same
    heads, fp32 states updated in place).
``value`` is the chunkwise forward's tokens/s from its GPU time in the timed
region: K whole steps through the untimed entry points, each chunk call
between two events on the launch stream.  The same K steps then run through
the timed entry points, whose events, recorded by the runtime at each
kernel's start and end, give every kernel's own duration (the figure
rocprofv3's kernel trace reports); those events add a few microseconds at
each kernel boundary, which is why the throughput is taken without them.  The rooflines
come from the kernel durations: ``roofline`` is the chunk path's dominant
kernel against the bf16 matrix-core peak, ``roofline_decode`` the decode step
against HBM bandwidth.  ``ms_per_step`` is the host wall clock of a whole step
of the timed region.

After the timed steps, outside the step: the prefill workload (T=4096) is
timed the same way beside the chunk workload (``chunk_fwd_prefill``); both
are also timed cold (``cold``), with a 512 MiB buffer written between calls
so that no input is left in the 256 MB Infinity Cache; the chunk workload
with 64-token chunks is timed warm (``chunk_fwd_chunk64``).  Unless
``--chunk-only``: the decode step with its state stored in bf16
(``decode_bf16_state``), ``gdr_recurrent_multi`` on 256 sequences x 4
tokens (``multi_token``), the decode step with its conv update and gates
fused in front (``decode_conv``), the gated RMSNorm on the chunk workload's
output rows (``gated_rmsnorm``) and fused behind the decode step
(``decode_gated``), and the conv/gate prologue of the chunked path on the
chunk workload (``conv_prefill``).  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
D = 128
L = 128


def alg_flops_chunk(lengths, Nqk, Nv, chunk=L):
    """Algorithmic FLOPs of the chunkwise forward with chunks of `chunk`
    tokens, split by the kernel that performs each term: intra (Grams once
    per query/key head, the triangular inverse, the U/W/P products on
    triangles) and inter (the three products with the state: W S^T, Q S^T,
    V_new^T K)."""
    intra = inter = 0.0
    for n in lengths:
        full, tail = divmod(int(n), chunk)
        for ell, cnt in ((chunk, full), (tail, 1 if tail else 0)):
            if cnt == 0:
                continue
            intra += cnt * (Nqk * 2 * D * ell * ell + Nv * (ell ** 3 / 3 + 3 * D * ell * (ell + 1)))
            inter += cnt * Nv * 6 * ell * D * D
    return intra, inter


def alg_bytes_decode(N, Nqk, Nv, es=2, state_es=4):
    state = N * Nv * D * D * state_es * 2
    qkv = N * (2 * Nqk + Nv) * D * es
    gb = N * Nv * 4 * 2
    out = N * Nv * D * es
    return state + qkv + gb + out


MULTI_TOKENS = 4


def alg_bytes_multi(N, tokens, Nqk, Nv, es=2):
    """One read and one write of every fp32 state, plus per token the decode
    step's bytes: q and k once per q/k head, v and out per value head, g and
    beta."""
    state = N * Nv * D * D * 4 * 2
    per_tok = (2 * Nqk * D + Nv * D + Nv * D) * es + Nv * 4 * 2
    return state + N * tokens * per_tok


def alg_bytes_decode_conv(N, Nqk, Nv, K=4, es=2):
    """The decode step's bytes with q, k, v replaced by the token's projected
    channels, plus each channel's conv window read and written and the conv
    kernels (read once); a, b per (sequence, head); A_log, dt_bias per head."""
    C = (2 * Nqk + Nv) * D
    state = N * Nv * D * D * 4 * 2
    return (state + N * C * es + 2 * N * C * K * es + C * K * es + N * Nv * D * es
            + N * Nv * 4 * 2 + Nv * 4 * 2)


def alg_bytes_conv_prefill(T, N, Nqk, Nv, K=4, es=2):
    """Projected channels read and q/k/v written once, a and b read and g and
    beta written, kernels read once, every cached window read and written."""
    C = (2 * Nqk + Nv) * D
    return 2 * T * C * es + 4 * T * Nv * 4 + C * K * es + 2 * N * C * K * es + 2 * Nv * 4


def alg_bytes_gated_rmsnorm(rows, es=2):
    """x and z read, y written once: three rows of D values per row."""
    return 3 * rows * D * es + D * es


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from profiles/traffic.json (two rocprofv3
    --pmc runs, FETCH_SIZE and WRITE_SIZE, scaled by what the same counters
    read for a plain 512 MiB copy), or None when the kernel's sources have
    changed since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(here, "profiles", "traffic.json")) as f:
            rec = json.load(f)["kernels"][kernel]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(here, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sha256"]:
            return None
        return int(rec["hbm_bytes"])
    except (OSError, KeyError, ValueError):
        return None


class ChunkLeg:
    """One chunk workload resident on the device, with its outputs and
    workspace, called through the timed entry point."""

    def __init__(self, gdr, inp, dev, scale, chunk=L):
        import torch
        self.gdr, self.inp, self.scale, self.chunk = gdr, inp, scale, chunk
        dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
        self.t = dict(q=torch.from_numpy(inp.q).to(dev, dt), k=torch.from_numpy(inp.k).to(dev, dt),
                      v=torch.from_numpy(inp.v).to(dev, dt), g=torch.from_numpy(inp.g).to(dev),
                      beta=torch.from_numpy(inp.beta).to(dev),
                      cu=torch.from_numpy(inp.cu_seqlens).to(dev),
                      s0=torch.from_numpy(inp.state_in).to(dev))
        self.out = torch.empty((inp.T, inp.Nv, D), dtype=dt, device=dev)
        self.sout = torch.empty_like(self.t["s0"])
        code = gdr.GDR_BF16 if inp.dtype == "bf16" else gdr.GDR_F32
        self.ws = torch.empty(gdr.workspace_size(inp.T, inp.N, inp.Nqk, inp.Nv, code),
                              dtype=torch.uint8, device=dev)

    def __call__(self, timings=None):
        t = self.t
        self.gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["s0"],
                           scale=self.scale, out=self.out, state_out=self.sout, workspace=self.ws,
                           chunk=self.chunk, timings=timings)

    def flops(self):
        return alg_flops_chunk(np.diff(self.inp.cu_seqlens).tolist(), self.inp.Nqk, self.inp.Nv,
                               self.chunk)

    def summarise(self, tims, steps, call_ms):
        """The call's GPU time from stream events around untimed calls
        (``call_ms``), and per-kernel figures from the timed calls' event
        records (``tims``: one list of (kernel, ms) per call)."""
        spans = [ms for tim in tims for n, ms in tim if n == "span"]
        per_kernel = {}
        for tim in tims:
            for n, ms in tim:
                if n != "span":
                    per_kernel.setdefault(n, []).append(ms)
        f_intra, f_inter = self.flops()
        span_s = float(np.mean(call_ms)) * 1e-3
        kst = {}
        for n, lst in per_kernel.items():
            per_call = len(lst) / steps
            avg = float(np.mean(lst))
            f = {"intra": f_intra, "inter": f_inter}.get(n)
            kst[n] = {"avg_ms": round(avg, 4), "launches_per_call": per_call,
                      "alg_tflops": round(f / (avg * per_call * 1e-3) / 1e12, 2) if f else None}
        f_tot = f_intra + f_inter
        return {"workload": self.inp.name, "tokens": self.inp.T, "sequences": self.inp.N,
                "gpu_ms": round(span_s * 1e3, 4), "tokens_per_s": round(self.inp.T / span_s, 1),
                "alg_gflop": round(f_tot / 1e9, 3),
                "alg_tflops": round(f_tot / span_s / 1e12, 2),
                "frac_bf16_mfma_peak": round(f_tot / span_s / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
                "kernel_sum_ms": round(sum(v["avg_ms"] * v["launches_per_call"] for v in kst.values()), 4),
                "span_with_kernel_events_ms": round(float(np.mean(spans)), 4),
                "kernels": kst}


def call_events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def time_chunk(leg, steps, warmup, flush=None):
    """After `warmup` untimed calls: `steps` untimed calls, each between two
    events on the launch stream (the call's GPU time), then `steps` calls
    through the timed entry point (each kernel's duration).  With `flush` (a
    512 MiB device buffer) the buffer is rewritten before every call, so the
    call starts with no input left in the Infinity Cache (cold)."""
    import torch
    for _ in range(warmup):
        leg()
    torch.cuda.synchronize()
    evs = call_events(steps)
    for a, b in evs:
        if flush is not None:
            flush.add_(1.0)
        a.record()
        leg()
        b.record()
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in evs]
    tims = []
    for _ in range(steps):
        if flush is not None:
            flush.add_(1.0)
        tim = []
        leg(tim)
        tims.append(tim)
    torch.cuda.synchronize()
    return leg.summarise(tims, steps, call_ms)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["prefill", "long", "varlen"], default="long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk-only", action="store_true",
                    help="time the step and the chunk figures only (for profiling runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB device to device once; "
                         "a profiler's byte counters on that plain copy calibrate the ones on the "
                         "kernels")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the gated delta rule shards over sequences and "
              "value heads with no exchange, and this build runs on a single MI355X; "
              "use --gpus 1", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import gated_deltanet_chunked_amd as gdr
    from gated_deltanet_chunked_amd.inputs import WORKLOAD_SEEDS, WORKLOADS, workload_inputs
    gdr.load()   # raises if libgdr.so is missing: there is no fallback
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scale = D ** -0.5

    pre = workload_inputs(args.workload)
    dec = workload_inputs("decode")
    leg = ChunkLeg(gdr, pre, dev, scale)
    T, N, Nqk, Nv = pre.T, pre.N, pre.Nqk, pre.Nv

    Dd = ChunkLeg(gdr, dec, dev, scale).t     # the decode step's inputs on the device
    dstate = Dd["s0"].clone()
    dout = torch.empty((dec.N, dec.Nv, D), dtype=Dd["q"].dtype, device=dev)

    def step(timings):
        leg(timings)
        gdr.recurrent_step(Dd["q"], Dd["k"], Dd["v"], Dd["g"], Dd["beta"], dstate,
                           state_out=dstate, out=dout, scale=scale, timings=timings)
    if args.copy_probe_mib > 0:
        # a plain device-to-device copy of known size whose source is cold:
        # 1 GiB written after the source pushes it out of the 256 MB
        # Infinity Cache, so a byte counter sees the whole copy
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device=dev)
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, flush
    for _ in range(args.warmup):
        step([])
    torch.cuda.synchronize()

    # the timed region: K whole steps through the untimed entry points, with
    # one event pair on the launch stream around each chunk call
    evs = call_events(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        leg()
        b.record()
        gdr.recurrent_step(Dd["q"], Dd["k"], Dd["v"], Dd["g"], Dd["beta"], dstate,
                           state_out=dstate, out=dout, scale=scale)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [a.elapsed_time(b) for a, b in evs]

    # the same K steps through the timed entry points: every kernel's duration
    # from events the runtime records at its start and end (they add about
    # 3 us at each kernel boundary, so the throughput above is taken without)
    chunk_tims, dec_ms = [], []
    for _ in range(args.steps):
        tim = []
        step(tim)
        dec_ms.extend(ms for n, ms in tim if n == "decode")
        chunk_tims.append([(n, ms) for n, ms in tim if n != "decode"])
    torch.cuda.synchronize()

    chunk = leg.summarise(chunk_tims, args.steps, call_ms)
    tok_s = chunk["tokens_per_s"]
    dec_s = float(np.mean(dec_ms)) * 1e-3
    dec_bytes = alg_bytes_decode(dec.N, dec.Nqk, dec.Nv)
    dec_gbps = dec_bytes / dec_s / 1e9
    roof_dec = dict(kernel="decode", bound="hbm", achieved=round(dec_gbps, 1), peak=HBM_PEAK_GBPS,
                    unit="GB/s", frac=round(dec_gbps / HBM_PEAK_GBPS, 4),
                    traffic=measured_traffic("decode"),
                    per_launch=f"{dec_bytes} algorithmic bytes")

    # the chunk path's dominant kernel: the most GPU time per call
    f_intra, f_inter = leg.flops()
    kst = chunk["kernels"]
    dom = max((k for k in kst if k in ("intra", "inter")),
              key=lambda k: kst[k]["avg_ms"] * kst[k]["launches_per_call"])
    per_launch_flops = {"intra": f_intra, "inter": f_inter}[dom] / kst[dom]["launches_per_call"]
    ach = per_launch_flops / (kst[dom]["avg_ms"] * 1e-3) / 1e12
    roof = dict(kernel=dom, bound="mfma", achieved=round(ach, 2), peak=MFMA_PEAK_TFLOPS["bf16"],
                unit="TFLOP/s", frac=round(ach / MFMA_PEAK_TFLOPS["bf16"], 4),
                traffic=measured_traffic(f"{dom}_{args.workload}"),
                per_launch=f"{per_launch_flops:.6g} algorithmic FLOP per launch, "
                           f"{kst[dom]['launches_per_call']:g} launches per call")

    res = {
        "metric": "chunk GDR fwd tokens/s + % MFMA peak; decode-step GB/s (% HBM peak)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; distributions of the Qwen3-Next gate initialisation)",
        "config": {"workload": WORKLOADS[args.workload] + " + " + WORKLOADS["decode"],
                   "tokens": T, "sequences": N, "Nqk": Nqk, "Nv": Nv, "D": D, "chunk": L,
                   "decode_sequences": dec.N},
        "chunk_fwd": chunk,
        "decode": {"gpu_ms": round(dec_s * 1e3, 4), "gbps": round(dec_gbps, 1),
                   "frac_hbm_peak": round(dec_gbps / HBM_PEAK_GBPS, 4),
                   "tokens_per_s": round(dec.N / dec_s, 1), "alg_bytes": dec_bytes},
        "roofline": roof,
        "roofline_decode": roof_dec,
    }

    # ---- beside the step: the prefill workload, and cold (Infinity Cache
    # flushed) figures of both chunk workloads
    flush = torch.zeros(1 << 27, dtype=torch.float32, device=dev)   # 512 MiB
    if args.workload != "prefill":
        leg1 = ChunkLeg(gdr, workload_inputs("prefill"), dev, scale)
        res["chunk_fwd_prefill"] = time_chunk(leg1, args.steps, args.warmup)
    else:
        leg1 = leg
    cold = {"what": "512 MiB buffer written before every call; same calls otherwise"}
    cold[args.workload] = time_chunk(leg, args.steps, 1, flush)
    if args.workload != "prefill":
        cold["prefill"] = time_chunk(leg1, args.steps, 1, flush)
    res["cold"] = cold
    del flush, leg1

    # the same workload with 64-token chunks (GDR_FLAG_CHUNK64): same inputs
    # and results up to rounding, twice the chunks
    leg64 = ChunkLeg(gdr, leg.inp, dev, scale, chunk=64)
    res["chunk_fwd_chunk64"] = time_chunk(leg64, args.steps, args.warmup)
    del leg64

    if not args.chunk_only:
        res.update(extras(gdr, dec, Dd, dout, pre, WORKLOAD_SEEDS[args.workload], args, dev, scale))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(pre, scale)
    print(json.dumps(res), flush=True)
    return 0


def extras(gdr, dec, Dd, dout, pre, seed, args, dev, scale):
    """The decode variants and the prefill prologue, measured after the timed
    steps and reported beside them (not part of the step)."""
    import torch
    res = {}
    T, N, Nqk, Nv = pre.T, pre.N, pre.Nqk, pre.Nv

    # decode with the state stored in bf16 (a bf16 state cache)
    bstate = Dd["s0"].to(torch.bfloat16)
    for _ in range(args.warmup):
        gdr.recurrent_step(Dd["q"], Dd["k"], Dd["v"], Dd["g"], Dd["beta"], bstate,
                           state_out=bstate, out=dout, scale=scale)
    btim = []
    for _ in range(args.steps):
        gdr.recurrent_step(Dd["q"], Dd["k"], Dd["v"], Dd["g"], Dd["beta"], bstate,
                           state_out=bstate, out=dout, scale=scale, timings=btim)
    torch.cuda.synchronize()
    bdec_s = float(np.mean([ms for _, ms in btim])) * 1e-3
    bdec_bytes = alg_bytes_decode(dec.N, dec.Nqk, dec.Nv, state_es=2)
    bdec_gbps = bdec_bytes / bdec_s / 1e9
    res["decode_bf16_state"] = {"gpu_ms": round(bdec_s * 1e3, 4), "gbps": round(bdec_gbps, 1),
                                "frac_hbm_peak": round(bdec_gbps / HBM_PEAK_GBPS, 4),
                                "tokens_per_s": round(dec.N / bdec_s, 1), "alg_bytes": bdec_bytes}
    del bstate

    # several tokens per sequence (gdr_recurrent_multi): 256 sequences x 4
    # tokens, the decode heads, fp32 states updated in place
    from gated_deltanet_chunked_amd.inputs import make_inputs
    mt = make_inputs([MULTI_TOKENS] * dec.N, dec.Nqk, dec.Nv, seed=4, state_std=0.01)
    M = ChunkLeg(gdr, mt, dev, scale).t
    mout = torch.empty((mt.T, mt.Nv, D), dtype=M["q"].dtype, device=dev)
    for _ in range(args.warmup):
        gdr.recurrent_multi(M["q"], M["k"], M["v"], M["g"], M["beta"], M["cu"], M["s0"],
                            scale=scale, out=mout, state_out=M["s0"])
    mtim = []
    for _ in range(args.steps):
        gdr.recurrent_multi(M["q"], M["k"], M["v"], M["g"], M["beta"], M["cu"], M["s0"],
                            scale=scale, out=mout, state_out=M["s0"], timings=mtim)
    torch.cuda.synchronize()
    multi_s = float(np.mean([ms for _, ms in mtim])) * 1e-3
    multi_bytes = alg_bytes_multi(mt.N, MULTI_TOKENS, mt.Nqk, mt.Nv)
    multi_gbps = multi_bytes / multi_s / 1e9
    res["multi_token"] = {"workload": f"{mt.N} sequences x {MULTI_TOKENS} tokens, Nqk={mt.Nqk} "
                                      f"Nv={mt.Nv} bf16, fp32 states in place",
                          "gpu_ms": round(multi_s * 1e3, 4), "gbps": round(multi_gbps, 1),
                          "frac_hbm_peak": round(multi_gbps / HBM_PEAK_GBPS, 4),
                          "tokens_per_s": round(mt.T / multi_s, 1), "alg_bytes": multi_bytes}
    del M, mout

    # decode with the conv update and gates fused in front
    # (gdr_recurrent_step_conv): 256 sequences, bf16 activations, fp32 states
    from gated_deltanet_chunked_amd.inputs import prologue_inputs
    pi = prologue_inputs(dec.N, dec.Nqk, dec.Nv, seed=4)
    cv = {k_: torch.from_numpy(getattr(pi, k_)).to(dev, torch.bfloat16)
          for k_ in ("mixed_qkv", "conv_state", "conv_w")}
    cf = {k_: torch.from_numpy(getattr(pi, k_)).to(dev) for k_ in ("a", "b", "A_log", "dt_bias",
                                                                   "state_in")}
    cs_a, cs_b = cv["conv_state"], torch.empty_like(cv["conv_state"])
    for _ in range(args.warmup):
        gdr.recurrent_step_conv(cv["mixed_qkv"], cs_a, cv["conv_w"], None, cf["a"], cf["b"],
                                cf["A_log"], cf["dt_bias"], cf["state_in"], conv_state_out=cs_b,
                                out=dout, scale=scale)
        cs_a, cs_b = cs_b, cs_a
    ctim = []
    for _ in range(args.steps):
        gdr.recurrent_step_conv(cv["mixed_qkv"], cs_a, cv["conv_w"], None, cf["a"], cf["b"],
                                cf["A_log"], cf["dt_bias"], cf["state_in"], conv_state_out=cs_b,
                                out=dout, scale=scale, timings=ctim)
        cs_a, cs_b = cs_b, cs_a
    torch.cuda.synchronize()
    conv_s = float(np.mean([ms for _, ms in ctim])) * 1e-3
    conv_bytes = alg_bytes_decode_conv(dec.N, dec.Nqk, dec.Nv)
    conv_gbps = conv_bytes / conv_s / 1e9
    res["decode_conv"] = {"workload": f"{dec.N} sequences x 1 token, Nqk={dec.Nqk} Nv={dec.Nv} "
                                      "bf16, conv update (kernel 4) and gates fused in front, "
                                      "fp32 states",
                          "gpu_ms": round(conv_s * 1e3, 4), "gbps": round(conv_gbps, 1),
                          "frac_hbm_peak": round(conv_gbps / HBM_PEAK_GBPS, 4),
                          "tokens_per_s": round(dec.N / conv_s, 1), "alg_bytes": conv_bytes}
    del cv, cf, cs_a, cs_b

    # the gated RMSNorm behind the rule: standalone on the chunk workload's
    # output rows (in place, as a caller applies it to gdr_chunk_fwd's out),
    # and fused into the decode step
    from gated_deltanet_chunked_amd.inputs import make_gate
    rows = T * Nv
    nx = torch.randn((T, Nv, D), device=dev, generator=torch.Generator(device=dev).manual_seed(seed))
    nx = nx.to(torch.bfloat16)
    z, w = make_gate((T, Nv, D), seed=seed)
    nz = torch.from_numpy(z).to(dev, torch.bfloat16)
    nw = torch.from_numpy(w).to(dev, torch.bfloat16)
    ny = torch.empty_like(nx)
    for _ in range(args.warmup):
        gdr.gated_rmsnorm(nx, nz, nw, out=ny)
    ntim = []
    for _ in range(args.steps):
        gdr.gated_rmsnorm(nx, nz, nw, out=ny, timings=ntim)
    torch.cuda.synchronize()
    norm_s = float(np.mean([ms for _, ms in ntim])) * 1e-3
    norm_bytes = alg_bytes_gated_rmsnorm(rows)
    norm_gbps = norm_bytes / norm_s / 1e9
    res["gated_rmsnorm"] = {"workload": f"{rows} rows of {D} bf16 (T={T} x Nv={Nv}), weight given",
                            "gpu_ms": round(norm_s * 1e3, 4), "gbps": round(norm_gbps, 1),
                            "frac_hbm_peak": round(norm_gbps / HBM_PEAK_GBPS, 4),
                            "alg_bytes": norm_bytes}
    del nx, nz, nw, ny
    dz, dw = make_gate((dec.N, dec.Nv, D), seed=4)
    dz = torch.from_numpy(dz).to(dev, torch.bfloat16)
    dw = torch.from_numpy(dw).to(dev, torch.bfloat16)
    gstate = Dd["s0"].clone()
    for _ in range(args.warmup):
        gdr.recurrent_step_gated(Dd["q"], Dd["k"], Dd["v"], Dd["g"], Dd["beta"], gstate, dz, dw,
                                 out=dout, scale=scale)
    gtim = []
    for _ in range(args.steps):
        gdr.recurrent_step_gated(Dd["q"], Dd["k"], Dd["v"], Dd["g"], Dd["beta"], gstate, dz, dw,
                                 out=dout, scale=scale, timings=gtim)
    torch.cuda.synchronize()
    gd_s = float(np.mean([ms for _, ms in gtim])) * 1e-3
    gd_bytes = alg_bytes_decode(dec.N, dec.Nqk, dec.Nv) + dec.N * dec.Nv * D * 2 + D * 2
    gd_gbps = gd_bytes / gd_s / 1e9
    res["decode_gated"] = {"workload": f"{dec.N} sequences x 1 token, Nqk={dec.Nqk} Nv={dec.Nv} "
                                       "bf16, gated RMSNorm fused behind, fp32 states",
                           "gpu_ms": round(gd_s * 1e3, 4), "gbps": round(gd_gbps, 1),
                           "frac_hbm_peak": round(gd_gbps / HBM_PEAK_GBPS, 4),
                           "tokens_per_s": round(dec.N / gd_s, 1), "alg_bytes": gd_bytes}
    del dz, dw, gstate

    # the conv/gate prologue of the chunked path (gdr_conv_prefill) on the
    # chunk workload's tokens: cached windows in, new windows out
    from gated_deltanet_chunked_amd.inputs import prefill_prologue_inputs
    pp = prefill_prologue_inputs(np.diff(pre.cu_seqlens).tolist(), Nqk, Nv, seed=seed)
    px = torch.from_numpy(pp.mixed_qkv).to(dev, torch.bfloat16)
    pcs = torch.from_numpy(pp.conv_state).to(dev, torch.bfloat16)
    pw = torch.from_numpy(pp.conv_w).to(dev, torch.bfloat16)
    pf = {k_: torch.from_numpy(getattr(pp, k_)).to(dev) for k_ in ("a", "b", "A_log", "dt_bias")}
    pcu = torch.from_numpy(pp.cu_seqlens).to(dev)
    pcs_out = torch.empty_like(pcs)
    for _ in range(args.warmup):
        gdr.conv_prefill(px, pcs, pw, None, pf["a"], pf["b"], pf["A_log"], pf["dt_bias"], pcu,
                         conv_state_out=pcs_out)
    ptim = []
    for _ in range(args.steps):
        gdr.conv_prefill(px, pcs, pw, None, pf["a"], pf["b"], pf["A_log"], pf["dt_bias"], pcu,
                         conv_state_out=pcs_out, timings=ptim)
    torch.cuda.synchronize()
    cp_s = float(np.mean([ms for _, ms in ptim])) * 1e-3
    cp_bytes = alg_bytes_conv_prefill(T, N, Nqk, Nv)
    cp_gbps = cp_bytes / cp_s / 1e9
    res["conv_prefill"] = {"workload": f"{T} tokens in {N} sequences, Nqk={Nqk} Nv={Nv} bf16, "
                                       "conv kernel 4, cached windows in and out",
                           "gpu_ms": round(cp_s * 1e3, 4), "gbps": round(cp_gbps, 1),
                           "frac_hbm_peak": round(cp_gbps / HBM_PEAK_GBPS, 4),
                           "tokens_per_s": round(T / cp_s, 1), "alg_bytes": cp_bytes}
    return res


def cpu_baseline(pre, scale):
    """The fp64 oracle on the host cores, on a bounded sample of the prefill
    workload: the first value heads of the first sequence, as many as fit in
    roughly ten seconds (the rule is independent per head)."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    nthr = oracle.threads(threads)
    G = pre.Nv // pre.Nqk
    T0, T1 = int(pre.cu_seqlens[0]), int(pre.cu_seqlens[1])

    def run(heads, nthreads=nthr, t1=T1):
        j0, j1 = heads[0] // G, heads[-1] // G + 1
        t = time.perf_counter()
        oracle.recurrent(pre.q[T0:t1, j0:j1], pre.k[T0:t1, j0:j1], pre.v[T0:t1, heads[0]:heads[-1] + 1],
                         pre.g[T0:t1, heads[0]:heads[-1] + 1], pre.beta[T0:t1, heads[0]:heads[-1] + 1],
                         None if pre.state_in is None else pre.state_in[:1, heads[0]:heads[-1] + 1],
                         np.array([0, t1 - T0], np.int32), scale, nthreads=nthreads)
        return time.perf_counter() - t

    heads = list(range(G))           # one query/key group first
    dt = run(heads)
    per_head = dt / len(heads)
    nh = int(min(pre.Nv, max(G, (10.0 / max(per_head, 1e-6)) // G * G)))
    if nh > len(heads):
        heads = list(range(nh))
        dt = run(heads)
    # tokens/s of the whole workload at this rate: every head of every token
    tok_s = (T1 - T0) * len(heads) / pre.Nv / dt
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    # one thread, on the first 4096 tokens of one query/key group (the T=4096
    # prefill workload's length)
    n1 = min(4096, T1 - T0)
    dt1 = run(list(range(G)), nthreads=1, t1=T0 + n1)
    single = {"value": round(n1 * G / pre.Nv / dt1, 1), "unit": "tokens/s", "cores": 1,
              "sample": f"first {n1} tokens, value heads 0..{G - 1} of {pre.Nv}, {dt1:.2f} s"}
    return {"value": round(tok_s, 1), "unit": "tokens/s", "cores": nthr, "kind": "oracle",
            "sample": f"first sequence ({T1 - T0} tokens), value heads 0..{len(heads) - 1} of "
                      f"{pre.Nv}, fp64 per-token recurrence, {dt:.1f} s on {cpu}",
            "single_thread": single}


if __name__ == "__main__":
    sys.exit(main())
