"""Throughput of libgdr on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill|long|varlen]
                    [--no-cpu-baseline]

One step is one pass of the whole hot path on synthetic, seeded inputs that
are resident in HBM before the timed region starts:
  * gdr_chunk_fwd on the prefill workload (default: B=1, T=4096, Nqk=16,
    Nv=32, D=128, bf16 q/k/v, fp32 gates and states), and
  * gdr_recurrent_step on the decode workload (256 sequences x 1 token, same
    heads, fp32 states updated in place).
``value`` is the chunkwise forward's tokens/s from its GPU time: the span from
its first kernel's start to its last kernel's end, taken from HIP events that
the runtime records at each kernel's start and end inside the timed region.
The same events give every kernel's own duration (the figure rocprofv3's
kernel trace reports), from which the decode step's GB/s and the rooflines
are computed.  ``ms_per_step`` is the host wall clock of a whole step.  After
the timed steps the decode step is also measured with its state stored in
bf16 (``gdr_recurrent_step_bf16_state``, half the state bytes), reported as
``decode_bf16_state``, ``gdr_recurrent_multi`` on 256 sequences x 4 tokens
as ``multi_token``, and the decode step with its conv update and gates fused
in front as ``decode_conv``, and the conv/gate prologue of the chunked path on
the prefill workload as ``conv_prefill``; none of them is part of the step.  One JSON line is printed.
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


def alg_flops_chunk(lengths, Nqk, Nv):
    """Algorithmic FLOPs of the chunkwise forward, split by the kernel that
    performs each term: intra (Grams once per query/key head, the triangular
    inverse, the U/W/P products on triangles) and inter (the three products
    with the state: W S^T, Q S^T, V_new^T K)."""
    intra = inter = 0.0
    for n in lengths:
        full, tail = divmod(int(n), L)
        for ell, cnt in ((L, full), (tail, 1 if tail else 0)):
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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["prefill", "long", "varlen"], default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    from gated_deltanet_chunked_amd.inputs import config_inputs, CONFIG_NAMES
    gdr.load()   # raises if libgdr.so is missing: there is no fallback
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scale = D ** -0.5

    cfg = {"prefill": 1, "varlen": 2, "long": 3}[args.workload]
    pre = config_inputs(cfg)
    dec = config_inputs(4)

    def to_dev(inp):
        dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
        return dict(q=torch.from_numpy(inp.q).to(dev, dt), k=torch.from_numpy(inp.k).to(dev, dt),
                    v=torch.from_numpy(inp.v).to(dev, dt), g=torch.from_numpy(inp.g).to(dev),
                    beta=torch.from_numpy(inp.beta).to(dev),
                    cu=torch.from_numpy(inp.cu_seqlens).to(dev),
                    s0=torch.from_numpy(inp.state_in).to(dev))

    P, Dd = to_dev(pre), to_dev(dec)
    T, N, Nqk, Nv = pre.T, pre.N, pre.Nqk, pre.Nv
    out = torch.empty((T, Nv, D), dtype=P["q"].dtype, device=dev)
    sout = torch.empty_like(P["s0"])
    ws = torch.empty(gdr.workspace_size(T, N, Nqk, Nv, gdr.GDR_BF16), dtype=torch.uint8, device=dev)
    dstate = Dd["s0"].clone()
    dout = torch.empty((dec.N, dec.Nv, D), dtype=Dd["q"].dtype, device=dev)

    def step(timings):
        gdr.chunk_fwd(P["q"], P["k"], P["v"], P["g"], P["beta"], P["cu"], P["s0"], scale=scale,
                      out=out, state_out=sout, workspace=ws, timings=timings)
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

    chunk_ms, dec_ms = [], []
    per_kernel = {}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        tim = []
        step(tim)
        for name, ms in tim:
            if name == "span":
                chunk_ms.append(ms)
            elif name == "decode":
                dec_ms.append(ms)
            else:
                per_kernel.setdefault(name, []).append(ms)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # ---- prefill figures
    lengths = np.diff(pre.cu_seqlens).tolist()
    f_intra, f_inter = alg_flops_chunk(lengths, Nqk, Nv)
    f_total = f_intra + f_inter
    chunk_s = float(np.mean(chunk_ms)) * 1e-3
    tok_s = T / chunk_s
    # average duration of one launch of each kernel, and launches per call
    kstats = {}
    for name, lst in per_kernel.items():
        kstats[name] = dict(avg_ms=float(np.mean(lst)), launches_per_call=len(lst) / args.steps)
    # ---- decode figures
    dec_s = float(np.mean(dec_ms)) * 1e-3
    dec_bytes = alg_bytes_decode(dec.N, dec.Nqk, dec.Nv)
    dec_gbps = dec_bytes / dec_s / 1e9

    # the dominant kernel: the one with the most GPU time per step
    per_step = {name: s["avg_ms"] * s["launches_per_call"] for name, s in kstats.items()}
    per_step["decode"] = dec_s * 1e3
    dom = max(per_step, key=per_step.get)
    if dom == "decode":
        roof = dict(kernel="decode", bound="hbm", achieved=round(dec_gbps, 1), peak=HBM_PEAK_GBPS,
                    unit="GB/s", frac=round(dec_gbps / HBM_PEAK_GBPS, 4),
                    traffic=measured_traffic("decode"),
                    per_launch=f"{dec_bytes} algorithmic bytes")
    else:
        f_dom = {"intra": f_intra, "inter": f_inter}.get(dom, 0.0)
        launches = per_kernel[dom]
        per_launch_flops = f_dom / kstats[dom]["launches_per_call"]
        ach = per_launch_flops / (kstats[dom]["avg_ms"] * 1e-3) / 1e12
        roof = dict(kernel=dom, bound="mfma", achieved=round(ach, 2), peak=MFMA_PEAK_TFLOPS["bf16"],
                    unit="TFLOP/s", frac=round(ach / MFMA_PEAK_TFLOPS["bf16"], 4),
                    traffic=measured_traffic(dom) if args.workload == "prefill" else None,
                    per_launch=f"{per_launch_flops:.4g} algorithmic FLOP")
        del launches

    # ---- decode with the state stored in bf16 (a bf16 state cache): measured
    # after the timed steps, on the same decode inputs, and reported beside them
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

    # ---- several tokens per sequence (gdr_recurrent_multi): 256 sequences x 4
    # tokens, the decode heads, fp32 states updated in place; measured after
    # the timed steps and reported beside them
    from gated_deltanet_chunked_amd.inputs import make_inputs
    mt = make_inputs([MULTI_TOKENS] * dec.N, dec.Nqk, dec.Nv, seed=4, state_std=0.01)
    M = to_dev(mt)
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

    # ---- decode with the conv update and gates fused in front
    # (gdr_recurrent_step_conv): the decode heads, 256 sequences, bf16
    # activations, fp32 states in place; measured after the timed steps
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

    # ---- the conv/gate prologue of the chunked path (gdr_conv_prefill) at the
    # prefill shape: cached windows in, new windows out; measured after the
    # timed steps
    from gated_deltanet_chunked_amd.inputs import prefill_prologue_inputs
    pp = prefill_prologue_inputs(np.diff(pre.cu_seqlens).tolist(), Nqk, Nv, seed=cfg)
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
        "config": {"workload": CONFIG_NAMES[cfg] + " + " + CONFIG_NAMES[4],
                   "tokens": T, "sequences": N, "Nqk": Nqk, "Nv": Nv, "D": D, "chunk": L,
                   "decode_sequences": dec.N},
        "chunk_fwd": {"gpu_ms": round(chunk_s * 1e3, 4), "tokens_per_s": round(tok_s, 1),
                      "alg_tflops": round(f_total / chunk_s / 1e12, 2),
                      "frac_bf16_mfma_peak": round(f_total / chunk_s / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
                      "alg_gflop": round(f_total / 1e9, 3),
                      "kernel_sum_ms": round(sum(v["avg_ms"] * v["launches_per_call"]
                                                 for v in kstats.values()), 4),
                      "kernels": {k: {"avg_ms": round(v["avg_ms"], 4),
                                      "launches_per_call": v["launches_per_call"],
                                      "alg_tflops": (round({"intra": f_intra, "inter": f_inter}[k]
                                                           / (v["avg_ms"] * v["launches_per_call"] * 1e-3)
                                                           / 1e12, 2)
                                                     if k in ("intra", "inter") else None)}
                                  for k, v in kstats.items()}},
        "decode": {"gpu_ms": round(dec_s * 1e3, 4), "gbps": round(dec_gbps, 1),
                   "frac_hbm_peak": round(dec_gbps / HBM_PEAK_GBPS, 4),
                   "tokens_per_s": round(dec.N / dec_s, 1), "alg_bytes": dec_bytes},
        "decode_bf16_state": {"gpu_ms": round(bdec_s * 1e3, 4), "gbps": round(bdec_gbps, 1),
                              "frac_hbm_peak": round(bdec_gbps / HBM_PEAK_GBPS, 4),
                              "tokens_per_s": round(dec.N / bdec_s, 1), "alg_bytes": bdec_bytes},
        "multi_token": {"workload": f"{mt.N} sequences x {MULTI_TOKENS} tokens, Nqk={mt.Nqk} "
                                    f"Nv={mt.Nv} bf16, fp32 states in place",
                        "gpu_ms": round(multi_s * 1e3, 4), "gbps": round(multi_gbps, 1),
                        "frac_hbm_peak": round(multi_gbps / HBM_PEAK_GBPS, 4),
                        "tokens_per_s": round(mt.T / multi_s, 1), "alg_bytes": multi_bytes},
        "decode_conv": {"workload": f"{dec.N} sequences x 1 token, Nqk={dec.Nqk} Nv={dec.Nv} bf16, "
                                    "conv update (kernel 4) and gates fused in front, fp32 states",
                        "gpu_ms": round(conv_s * 1e3, 4), "gbps": round(conv_gbps, 1),
                        "frac_hbm_peak": round(conv_gbps / HBM_PEAK_GBPS, 4),
                        "tokens_per_s": round(dec.N / conv_s, 1), "alg_bytes": conv_bytes},
        "conv_prefill": {"workload": f"{T} tokens in {N} sequences, Nqk={Nqk} Nv={Nv} bf16, "
                                     "conv kernel 4, cached windows in and out",
                         "gpu_ms": round(cp_s * 1e3, 4), "gbps": round(cp_gbps, 1),
                         "frac_hbm_peak": round(cp_gbps / HBM_PEAK_GBPS, 4),
                         "tokens_per_s": round(T / cp_s, 1), "alg_bytes": cp_bytes},
        "roofline": roof,
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(pre, scale)
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline(pre, scale):
    """The fp64 oracle on the host cores, on a bounded sample of the prefill
    workload: the first value heads of the first sequence, as many as fit in
    roughly ten seconds (the rule is independent per head)."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    nthr = oracle.threads(threads)
    G = pre.Nv // pre.Nqk
    T0, T1 = int(pre.cu_seqlens[0]), int(pre.cu_seqlens[1])

    def run(heads):
        j0, j1 = heads[0] // G, heads[-1] // G + 1
        t = time.perf_counter()
        oracle.recurrent(pre.q[T0:T1, j0:j1], pre.k[T0:T1, j0:j1], pre.v[T0:T1, heads[0]:heads[-1] + 1],
                         pre.g[T0:T1, heads[0]:heads[-1] + 1], pre.beta[T0:T1, heads[0]:heads[-1] + 1],
                         None if pre.state_in is None else pre.state_in[:1, heads[0]:heads[-1] + 1],
                         np.array([0, T1 - T0], np.int32), scale, nthreads=nthr)
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
    return {"value": round(tok_s, 1), "unit": "tokens/s", "cores": nthr, "kind": "oracle",
            "sample": f"first sequence ({T1 - T0} tokens), value heads 0..{len(heads) - 1} of "
                      f"{pre.Nv}, fp64 per-token recurrence, {dt:.1f} s on {cpu}"}


if __name__ == "__main__":
    sys.exit(main())
