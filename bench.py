"""Benchmark of the sparse MLA training backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

A step is one smla_bwd call (CSR build, delta, dQ, dKV-intermediate, gather,
d_sink) over the resident, seeded headline workload (T=4096, H=128, topk=512,
D=512, num_kv=5120: 128-row sliding window + up to 384 of 1024 pool rows).
O and lse are produced once by the library's own forward (smla_fwd).  The
workspace and outputs are preallocated, so nothing is allocated while timing.

Prints ONE JSON line: value = nominal TFLOPS (10*T*H*topk*512 flops per call,
padded slots counted), ms_per_step, the skewed and long workloads timed the
same way after it ("workloads"), the roofline of the dominant kernel
(timed live inside the timed calls with HIP events that the library records on
the calls' stream at its stage boundaries) and, on rank 0 at N=1, the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_FLOP_PER_CLK_PER_CU = 4096   # 4 SIMDs x one 16x16x32 bf16 MFMA (16,384 flop) per 16 clocks
D = 512


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline",
                    help="a seeded workload of sparse_mla_attention_smla_amd/inputs.py: headline (the "
                         "default and the metric's), skewed, long, mid, small, tiny, or headline_h16/"
                         "h32/h48/h64/h96 (the headline's tokens and indices at other head counts)")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--phased", choices=["on", "off"], default="off",
                    help="also time the bounded-workspace backward (1024-token phases); its "
                         "smaller dQ/intermediate launches would mix into a kernel trace")
    ap.add_argument("--cpu-sample-tokens", type=int, default=3072,
                    help="tokens of the oracle baseline sample (about 10 s of host work)")
    ap.add_argument("--stage-steps", type=int, default=10)
    ap.add_argument("--graph", choices=["on", "off"], default="on",
                    help="also time the call captured in a HIP graph and replayed (graph_replay)")
    ap.add_argument("--stage-events", choices=["on", "off"], default="on",
                    help="time delta/dQ/intermediate/gather with events recorded inside the "
                         "timed calls (off: plain calls, stages timed through their entry points)")
    ap.add_argument("--also", default="skewed,long",
                    help="comma-separated workloads timed after the main one with plain smla_bwd "
                         "calls (their own seeded inputs, O/lse from the library forward); '' for none")
    ap.add_argument("--also-steps", type=int, default=20)
    ap.add_argument("--pe", choices=["on", "off"], default="on",
                    help="also time the has_pe=True variant (smla_fwd_pe, smla_bwd_pe) on the same "
                         "workload with seeded positional parts q_pe [T,H,64], k_pe [num_kv,64]")
    ap.add_argument("--mode", choices=["full", "profile"], default="full",
                    help="profile: only the timed backward calls, then a plain device copy of "
                         "COPY_BYTES (the reference for scaling HBM byte counters); prints no JSON")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def _code_only(text: str) -> str:
    """C/C++ source without comments and with whitespace collapsed (the sources
    hold no string literal that contains a comment marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the HIP sources, comments and layout aside: a stored HBM-traffic
    figure is only valid for this code."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_mla_attention_smla_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(f.encode())
            h.update(_code_only(open(os.path.join(csrc, f)).read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current sources (else None)."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except ValueError:
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def device_info():
    """CU count and peak shader clock of device 0 (hipDeviceGetAttribute through
    the HIP runtime that torch loaded), and the bf16 MFMA peak they imply."""
    import ctypes

    import torch
    props = torch.cuda.get_device_properties(0)
    cus = int(props.multi_processor_count)
    clock_khz = None
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (value 5 in hip_runtime_api.h): peak clock in kHz
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0 and 5e5 < v.value < 5e6:
            clock_khz = int(v.value)
    except OSError:
        pass
    info = {"name": props.name, "arch": props.gcnArchName, "cus": cus,
            "peak_clock_ghz": None if clock_khz is None else clock_khz / 1e6,
            "mfma_bf16_flop_per_clk_per_cu": MFMA_BF16_FLOP_PER_CLK_PER_CU}
    if clock_khz is not None:
        info["derived_bf16_peak_tflops"] = round(cus * MFMA_BF16_FLOP_PER_CLK_PER_CU * clock_khz * 1e3 / 1e12, 1)
    info["peak_used_tflops"] = PEAK_BF16_TFLOPS
    info["peak_note"] = ("fractions divide by the published 2500 TFLOPS dense bf16 peak; "
                         "derived = CUs x 4096 flop/clk x peak clock")
    return info


def time_graph(w, step, reps):
    """ms per call when one smla_bwd call, captured in a HIP graph on a side stream,
    is replayed (same kernels, same buffers; the graph holds no allocation)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for _ in range(3):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(reps):
            g.replay()
        b.record(s)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del g
    return {"ms": round(ms, 4), "tflops": round(w.flops() / (ms * 1e-3) / 1e12, 1),
            "note": "the same call captured once in a HIP graph (with its own helper stream) and replayed; launch gaps only differ"}


def time_phased(B, w, q, kv, dO, O, lse, idx, sink, scale, ph_tokens, ws, dq, dkv, ds, reps):
    """ms per call of the bounded-workspace backward on the same inputs and outputs."""
    import torch
    T, H, N, K = w.T, w.H, w.num_kv, w.topk
    ph_ws = torch.empty(B.lib().smla_bwd_phased_workspace_bytes(T, H, N, K, ph_tokens, 0),
                        dtype=torch.uint8, device="cuda")

    def phased():
        B.smla_bwd_phased(q, kv, dO, O, lse, idx, sink, scale, phase_tokens=ph_tokens, workspace=ph_ws,
                          out=(dq, dkv, ds))
    phased()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        phased()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    return {"phase_tokens": ph_tokens, "ms": round(ms, 4),
            "tflops": round(w.flops() / (ms * 1e-3) / 1e12, 1),
            "workspace_gib": round(ph_ws.numel() / 2 ** 30, 3),
            "full_workspace_gib": round(ws.numel() / 2 ** 30, 3)}


def time_pe(B, w, q, kv, dO, idx, sink, reps, warmup):
    """The has_pe=True variant on the same workload: ms per smla_bwd_pe call and per
    smla_fwd_pe call (medians), with seeded positional parts (scale 1/sqrt(512 + 64))."""
    import numpy as np
    import torch

    from sparse_mla_attention_smla_amd import inputs
    T, H, N, K = w.T, w.H, w.num_kv, w.topk
    qpe_h, kpe_h = inputs.make_pe(w.name)

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    q_pe, k_pe = d16(qpe_h), d16(kpe_h)
    scale = 1.0 / math.sqrt(D + 64)
    O, lse = B.smla_fwd_pe(q, q_pe, kv, k_pe, idx, sink, scale)
    outs = (torch.empty_like(q), torch.empty_like(q_pe), torch.empty_like(kv), torch.empty_like(k_pe),
            torch.empty(H, dtype=torch.float32, device="cuda"))
    ws = torch.empty(B.bwd_pe_workspace_bytes(T, H, N, K), dtype=torch.uint8, device="cuda")

    def bwd():
        B.smla_bwd_pe(q, q_pe, kv, k_pe, dO, O, lse, idx, sink, scale, workspace=ws, out=outs)

    def fwd():
        B.smla_fwd_pe(q, q_pe, kv, k_pe, idx, sink, scale, out=(O, lse))

    res = {}
    for name, fn in (("bwd", bwd), ("fwd", fwd)):
        # as for the other workloads: warm-up calls (the clock settles over the
        # first few tens of calls after an idle spell), then each call timed alone
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        res[name] = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
    # nominal flops: the plain op's plus the positional products (S, dq_pe and the
    # positional intermediate in the backward; S in the forward), 64 wide
    bwd_flops = w.flops() + 6.0 * T * H * K * 64
    fwd_flops = 4.0 * T * H * K * D + 2.0 * T * H * K * 64
    del ws
    bms, fms = float(np.median(res["bwd"])), float(np.median(res["fwd"]))
    return {"bwd_ms": round(bms, 4), "bwd_ms_p10": round(float(np.percentile(res["bwd"], 10)), 4),
            "bwd_ms_p90": round(float(np.percentile(res["bwd"], 90)), 4),
            "bwd_tflops": round(bwd_flops / (bms * 1e-3) / 1e12, 1),
            "bwd_frac_of_bf16_peak": round(bwd_flops / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "fwd_ms": round(fms, 4), "fwd_tflops": round(fwd_flops / (fms * 1e-3) / 1e12, 1),
            "note": f"smla_bwd_pe / smla_fwd_pe with q_pe [T,H,64], k_pe [num_kv,64]; median of {reps} calls "
                    f"after {warmup} warm-up calls; nominal flops 10*T*H*topk*512 + 6*T*H*topk*64 (backward), "
                    "4*T*H*topk*512 + 2*T*H*topk*64 (forward)"}


def time_workload(B, name, steps, warmup):
    """ms per plain smla_bwd call (median, p10, p90 of `steps` calls after `warmup`)
    on another seeded workload, inputs resident, workspace and outputs preallocated."""
    import numpy as np
    import torch

    from sparse_mla_attention_smla_amd import inputs
    w = inputs.WORKLOADS[name]
    T, H, N, K = w.T, w.H, w.num_kv, w.topk
    print(f"[bench] generating {name}: T={T} H={H} num_kv={N} topk={K}", file=sys.stderr, flush=True)
    x = inputs.make(name, sink=True)

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    q, kv, dO = d16(x["q"]), d16(x["kv"]), d16(x["dO"])
    idx = torch.from_numpy(x["idx"]).cuda()
    sink = torch.from_numpy(x["sink"]).cuda()
    nnz = int((x["idx"] >= 0).sum())
    del x
    scale = 1.0 / math.sqrt(D)
    O, lse = B.smla_fwd(q, kv, idx, sink, scale)
    outs = (torch.empty_like(q), torch.empty_like(kv), torch.empty(H, dtype=torch.float32, device="cuda"))
    ws = torch.empty(B.bwd_workspace_bytes(T, H, N, K), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        B.smla_bwd(q, kv, dO, O, lse, idx, sink, scale, workspace=ws, out=outs)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        B.smla_bwd(q, kv, dO, O, lse, idx, sink, scale, workspace=ws, out=outs)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    med = float(np.median(per))
    print(f"[bench] {name}: {med:.3f} ms/call (median of {steps})", file=sys.stderr, flush=True)
    row = {"ms_median": round(med, 4), "ms_p10": round(float(np.percentile(per, 10)), 4),
           "ms_p90": round(float(np.percentile(per, 90)), 4),
           "tflops": round(w.flops() / (med * 1e-3) / 1e12, 2),
           "frac_of_bf16_peak": round(w.flops() / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "valid_slot_tflops": round(10.0 * nnz * H * D / (med * 1e-3) / 1e12, 2),
           "steps": steps, "warmup": warmup,
           "config": f"T={T} H={H} D={D} num_kv={N} topk={K}, {w.selection}, valid slots {nnz}"}
    del q, kv, dO, idx, sink, O, lse, outs, ws
    torch.cuda.empty_cache()
    return row


def cpu_baseline(w, n_tokens):
    """Time the fp64 oracle backward (as it stands) on an evenly spaced token sample."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import smla_oracle as orc
    from sparse_mla_attention_smla_amd import inputs

    x = inputs.make(w.name, sink=True)
    toks = np.linspace(0, w.T - 1, n_tokens).round().astype(int)
    scale = 1.0 / math.sqrt(D)
    kv64 = orc.bf16_to_f64(x["kv"])
    # O and lse of the sampled tokens from the oracle forward (not timed)
    O = np.zeros((w.T, w.H, D), dtype=np.uint16)
    lse = np.zeros((w.T, w.H), dtype=np.float32)
    for t in toks:
        o_t, l_t = orc.forward_token(orc.bf16_to_f64(x["q"][t]), kv64, x["idx"][t],
                                     x["sink"].astype(np.float64), scale)
        O[t], lse[t] = orc.emit_forward_outputs(o_t, l_t)
    # The whole oracle backward (delta, dq, P/dS, the per-slot intermediate, its
    # accumulation into dkv, d_sink) on the sampled tokens, timed in chunks of
    # 256 tokens so that the oracle's per-token outputs stay small.
    dt = 0.0
    for i in range(0, len(toks), 256):
        tt = toks[i:i + 256]
        q, dO, Os, ls, ix = x["q"][tt], x["dO"][tt], O[tt], lse[tt], x["idx"][tt]
        t0 = time.perf_counter()
        orc.backward(q, x["kv"], dO, Os, ls, ix, x["sink"], scale)
        dt += time.perf_counter() - t0
    flops = 10.0 * n_tokens * w.H * w.topk * D
    pools = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in pools] or [1])
    blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '?')} "
                             f"({i.get('threading_layer', '?')}, {i.get('num_threads', '?')} threads)"
                             for i in pools if i.get("user_api") == "blas"})) or "unknown"
    return {
        "value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
        "sample": f"fp64 NumPy oracle backward (delta, dq, P, dS, interm, dkv accumulation, d_sink) "
                  f"on {n_tokens} evenly spaced of {w.T} tokens of the {w.name} workload; "
                  f"{dt:.2f} s; extrapolated {dt * w.T / n_tokens * 1e3:.0f} ms per full call",
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
        "blas": blas,
    }


def _cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (unknown elsewhere)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path (how it would shard is described with the design); run with "
              "--gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_mla_attention_smla_amd import binding as B
    from sparse_mla_attention_smla_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev_info = device_info()
    w = inputs.WORKLOADS[args.workload]
    T, H, N, K = w.T, w.H, w.num_kv, w.topk
    scale = 1.0 / math.sqrt(D)
    print(f"[bench] generating {w.name}: T={T} H={H} num_kv={N} topk={K}", file=sys.stderr, flush=True)
    x = inputs.make(w.name, sink=True)

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    q, kv, dO = d16(x["q"]), d16(x["kv"]), d16(x["dO"])
    idx = torch.from_numpy(x["idx"]).cuda()
    sink = torch.from_numpy(x["sink"]).cuda()
    nnz = int((x["idx"] >= 0).sum())
    del x
    O, lse = B.smla_fwd(q, kv, idx, sink, scale)
    dq = torch.empty_like(q)
    dkv = torch.empty_like(kv)
    d_sink = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = B.bwd_workspace(T, H, N, K, q.device)
    torch.cuda.synchronize()

    def step(events=None):
        B.smla_bwd(q, kv, dO, O, lse, idx, sink, scale, workspace=ws, out=(dq, dkv, d_sink),
                   events=events)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps between synchronisations.  Each call also
    # records five events on its stream at its stage boundaries (smla_bwd_timed),
    # which time delta, dQ, the intermediate and the gather inside the real calls.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for evs in sev:
        for e in evs:
            e.record()      # creates the event
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        step(sev[i] if args.stage_events == "on" else None)
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    ms = float(ev[0].elapsed_time(ev[-1]) / args.steps)
    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"[bench] {ms:.3f} ms/call, {tflops:.1f} TFLOPS (wall {wall * 1e3 / args.steps:.3f} ms)",
          file=sys.stderr, flush=True)
    if args.mode == "profile":
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] profile mode: {args.steps} backward calls, then {args.steps} copies of "
              f"{COPY_BYTES} bytes", file=sys.stderr, flush=True)
        return

    # ---- per-stage timing: delta, dQ, the intermediate and the gather from the
    # events inside the timed calls; the CSR build and d_sink, which run hidden on
    # the library's helper stream there, from their entry points called alone
    # (same stream, same buffers)
    delta = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dsp = torch.empty((B.dsp_numel(T, H, K),), dtype=torch.bfloat16, device="cuda")
    interm = torch.empty((T * K, D), dtype=torch.bfloat16, device="cuda")
    row_ptr = torch.empty(N + 1, dtype=torch.int32, device="cuda")
    slots = torch.empty(T * K, dtype=torch.int32, device="cuda")
    dq2 = torch.empty_like(q)
    dkv2 = torch.empty_like(kv)
    ds2 = torch.empty(H, dtype=torch.float32, device="cuda")
    csr_ws = torch.empty(B.lib().smla_csr_workspace_bytes(T, K, N), dtype=torch.uint8, device="cuda")
    g_ws = torch.empty(B.lib().smla_gather_workspace_bytes(T, K, N), dtype=torch.uint8, device="cuda")
    s_ws = torch.empty(max(4, B.lib().smla_dsink_workspace_bytes(T, H)), dtype=torch.uint8, device="cuda")
    stages = {
        "csr": lambda: B.smla_build_csr(idx, N, out=(row_ptr, slots), workspace=csr_ws),
        "delta": lambda: B.smla_delta(O, dO, delta=delta),
        "dq": lambda: B.smla_dq(q, kv, dO, lse, delta, idx, scale, dsp=dsp, dq=dq2),
        "interm": lambda: B.smla_interm(q, dO, dsp, idx, N, interm=interm),
        "gather": lambda: B.smla_gather(interm, row_ptr, slots, T, K, N, dkv=dkv2, workspace=g_ws),
        "dsink": lambda: B.smla_dsink(lse, delta, sink, d_sink=ds2, workspace=s_ws),
    }
    stage_ms = {}
    in_step = ("delta", "dq", "interm", "gather")
    if args.stage_events == "on":
        for k, name in enumerate(in_step):
            stage_ms[name] = float(np.mean([e[k].elapsed_time(e[k + 1]) for e in sev]))
        stages = {k: v for k, v in stages.items() if k not in in_step}
    for name, fn in stages.items():
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.stage_steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        stage_ms[name] = a.elapsed_time(b) / args.stage_steps

    # algorithmic work per launch (nominal: all T*topk slots), see the design notes
    qb = T * H * D * 2
    algo = {
        "delta": ("hbm", 2 * qb + T * H * 4),
        "dq": ("mfma", 6.0 * T * H * K * D),
        "interm": ("hbm", 2 * qb + nnz * 2 * H * 2 + nnz * D * 2),
        "gather": ("hbm", nnz * D * 2 + nnz * 4 + N * D * 2),
    }
    stage_rows = {}
    for name, tms in stage_ms.items():
        row = {"ms": round(tms, 4)}
        if name in algo:
            bound, work = algo[name]
            if bound == "mfma":
                a_ = work / (tms * 1e-3) / 1e12
                row.update(bound="mfma", achieved_tflops=round(a_, 1), frac=round(a_ / PEAK_BF16_TFLOPS, 4))
            else:
                a_ = work / (tms * 1e-3) / 1e9
                row.update(bound="hbm", achieved_gbs=round(a_, 1), frac=round(a_ / PEAK_HBM_GBS, 4))
        stage_rows[name] = row
    dom = max(algo, key=lambda n: stage_ms[n])
    bound, work = algo[dom]
    tms = stage_ms[dom]
    if bound == "mfma":
        achieved, peak, unit = work / (tms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = work / (tms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"kernel": dom, "bound": bound, "achieved": round(achieved, 1), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4), "traffic": stored_traffic(dom),
                "algorithmic_per_launch": work, "ms_per_launch": round(tms, 4)}

    # the forward that produces O and lse (not part of the step; reported beside it)
    o2 = torch.empty_like(q)
    lse2 = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def fwd():
        B.smla_fwd(q, kv, idx, sink, scale, out=(o2, lse2))
    fwd()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.stage_steps):
        fwd()
    b.record()
    torch.cuda.synchronize()
    fwd_ms = a.elapsed_time(b) / args.stage_steps
    fwd_tf = 4.0 * T * H * K * D / (fwd_ms * 1e-3) / 1e12
    forward = {"ms": round(fwd_ms, 4), "bound": "mfma", "achieved_tflops": round(fwd_tf, 1),
               "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
               "note": "smla_fwd (O and lse) on the same inputs; nominal 4*T*H*topk*512 flops"}

    # the bounded-workspace backward (token phases of 1024) on the same inputs
    phased_row = None
    ph_tokens = 1024
    graph_row = time_graph(w, step, args.steps) if args.graph == "on" else None
    if args.phased == "on":
        phased_row = time_phased(B, w, q, kv, dO, O, lse, idx, sink, scale, ph_tokens, ws, dq2, dkv2,
                                 ds2, args.stage_steps)

    pe_row = None
    if args.pe == "on":
        print("[bench] has_pe variant", file=sys.stderr, flush=True)
        pe_row = time_pe(B, w, q, kv, dO, idx, sink, args.also_steps, 10)

    # the other full-size workloads (parity-test configs) timed beside the main one
    also_rows = {}
    for name in [a.strip() for a in args.also.split(",") if a.strip()]:
        if name != w.name:
            also_rows[name] = time_workload(B, name, args.also_steps, 5)

    cpu = None
    if args.cpu_baseline == "on":
        print(f"[bench] cpu baseline: oracle on {args.cpu_sample_tokens} tokens", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(w, args.cpu_sample_tokens)

    out = {
        "metric": "sparse-MLA bwd TFLOPS & ms/call at T=4096 H=128 topk=512 D=512 (1 GPU)",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_median": round(float(np.median(per)), 4),
        "ms_p10": round(float(np.percentile(per, 10)), 4),
        "ms_p90": round(float(np.percentile(per, 90)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "valid_slot_tflops": round(tflops * nnz / (T * K), 2),
        "valid_slot_frac_of_bf16_peak": round(tflops * nnz / (T * K) / PEAK_BF16_TFLOPS, 4),
        "device": dev_info,
        "dtype": "bf16",
        "data": "synthetic (seeded; O and lse from the library forward)",
        "config": {"workload": f"{w.name}: T={T} H={H} D={D} num_kv={N} topk={K}, "
                               "SWA(128) + up to 384 of the pool rows (stride 4), sink on",
                   "global_batch": T, "seq_len": T, "parallelism": "none (1 GPU)",
                   "valid_slots": nnz},
        "stages": stage_rows,
        "stages_timed": ("delta, dq, interm, gather: events inside the timed calls; csr, dsink: "
                         "entry points alone" if args.stage_events == "on" else "entry points alone"),
        "forward": forward,
        "phased": phased_row,
        "has_pe": pe_row,
        "workloads": also_rows or None,
        "graph_replay": graph_row,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "context": {"pages_own_backward_mi355x": {"ms": 3.238, "tflops": 424},
                    "ratio_to_pages": round(tflops / 424.0, 3),
                    "note": "the page's pool size and selection are unknown, so its workload is "
                            "not identical; hence vs_baseline is null"},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
