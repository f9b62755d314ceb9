#!/usr/bin/env python3
"""Benchmark of the GDN layer forward on one MI355X.

One step = one call of the whole layer (short conv + SiLU, L2 norm, chunked
gated delta rule, gated RMS norm, final state) over the Wan2.1-1.3B-shaped
workload at 480x832, 81 frames: B=1, T=32760 (21x30x52 latent tokens), H=12,
d=128, bf16 I/O with an fp32 state, seeded synthetic inputs already resident
in device memory.

Prints ONE JSON line on stdout.  Beside the headline tokens/s it reports:
  roofline     -- the dominant kernel (largest summed time per call) on the
                  layer's per-unit basis: 1288 B per token-head (q, k, v,
                  gate in and y out in bf16, plus fp32 log a and b) times the
                  token-heads one launch covers, over that kernel's average
                  launch duration (HIP events recorded on the launch stream
                  around each kernel, live in this run), against the MI355X
                  HBM peak of 8 TB/s; `traffic` is the kernel's measured HBM
                  bytes per launch (copy-calibrated FETCH_SIZE + WRITE_SIZE
                  from the committed rocprofv3 summary, null when that
                  summary was taken on other kernel sources);
  layer        -- the whole call against the same floor (1288 B per
                  token-head; a bidirectional call reads its inputs and
                  writes y once at best, so the same floor), and the measured
                  traffic of the whole call over those algorithmic bytes;
  cpu_baseline -- the fp64 oracle (the test yardstick) timed on this host's
                  cores on the same workload, and the parity of the last timed
                  GPU output against it.
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Algorithmic bytes per token-head of each kernel's own inputs and outputs
# (bf16 I/O, d = 128, chunk 64).  prep reads q, k, v (768 B) and log a, b
# (8 B) and writes the chunk record (5 matrices of 64 x 128 bf16 per 64 tokens
# = 1280 B); state reads the record's -W, (D K)^T and U~ (768 B) and writes
# the chunk-entry state (8 value blocks x 4 KB per 64 tokens = 512 B); out
# reads Q', O0 (512 B), the entry state (512 B) and the gate (256 B) and
# writes y (256 B).
def kernel_bytes_per_token_head(D: int, es: int) -> dict:
    """Algorithmic HBM bytes per token-head of each kernel's own contract
    (es = bytes per I/O element; states and gates are fp32):
      prep : q, k, v in (3 D es), log a and b in (8), the chunk record out
             (-W, Q', (D K)^T, U~, O0: 5 D es per token);
      state: -W, (D K)^T, U~ in (3 D es), the chunk-entry state out
             (D x D per 64 tokens: D^2 es / 64);
      out  : Q', O0 in (2 D es), chunk-entry state in (D^2 es / 64),
             gate in and y out (2 D es)."""
    return {
        "gdn_prep_kernel": 3 * D * es + 8 + 5 * D * es,
        "gdn_state_kernel": 3 * D * es + D * D * es // 64,
        "gdn_out_kernel": 2 * D * es + D * D * es // 64 + 2 * D * es,
    }


def layer_bytes_per_token_head(D: int, es: int) -> int:
    """The layer's own floor: q, k, v, gate in and y out, log a and b in."""
    return 5 * D * es + 8
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "linear_attention_token_fwd_amd", "csrc")


# the layer's kernels, and the launch plan (its ranges set the work per dispatch)
KERNEL_SOURCES = ("frag.hpp", "sync.hpp", "kernels.hpp", "gdn_api.hip")
MIXER_SOURCES = KERNEL_SOURCES + ("gemm.hpp", "gdn_proj.hip")    # + the projection GEMM


def csrc_hash(sources=KERNEL_SOURCES) -> str:
    """sha256 over the kernel sources and the launch plan, to tell whether a
    stored profile still describes the dispatches being run."""
    import hashlib
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def profiled_traffic(kernel: str, stem: str, sources=KERNEL_SOURCES):
    """HBM bytes per dispatch of `kernel` from the committed rocprofv3 summary
    profiles/<stem>.txt (FETCH_SIZE + WRITE_SIZE counters, copy-calibrated),
    or None if there is none or it was taken on different kernel sources."""
    path = os.path.join(HERE, "profiles", f"{stem}.txt")
    if not os.path.exists(path):
        return None
    src, val = None, None
    with open(path) as f:
        for line in f:
            if line.startswith("source_sha256:"):
                src = line.split(":", 1)[1].strip()
            if line.startswith(f"traffic_bytes[{kernel}]:"):
                val = float(line.split(":", 1)[1])
    return val if src == csrc_hash(sources) else None


class HipEvents:
    """Minimal hipEvent API through ctypes (events on a given stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs[i] = e
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def sync(self, e):
        self.hip.hipEventSynchronize(e)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, help="workload id (default 1: T=32760 H=12 d=128)")
    ap.add_argument("--batch", type=int, default=0,
                    help="batch rows B (default: the workload's own, 1); e.g. 2 for a classifier-free-guidance pair")
    ap.add_argument("--no-graph-cache", action="store_true",
                    help="turn the library's launch-graph cache off: every call launches its kernels directly")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: all available)")
    ap.add_argument("--mixer", action="store_true",
                    help="time the whole token mixer (in-projection with the gate parameterisation, the layer, "
                         "out-projection) at T=32760, C=1536, H=12, d=128 instead of the layer alone")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (gdn_bwd) on the workload instead of the forward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (read 1 GiB, write 1 GiB) three times, to "
                         "calibrate the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gdn_inputs
    import linear_attention_token_fwd_amd as gdn

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}), flush=True)
        return 0
    if args.no_graph_cache:
        gdn.gdn_set_graph_cache_limit(0)
    if args.bwd:
        return run_bwd(args)
    if args.mixer:
        return run_mixer(args)
    w = gdn_inputs.WORKLOADS[args.workload]
    log(f"workload {w.id}: {w.name}")
    t0 = time.time()
    inp = gdn_inputs.generate(w, B=args.batch or None)
    log(f"inputs generated in {time.time() - t0:.1f} s")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = gdn.to_device(inp, dtype=dt)
    B, T, H, D = inp["q"].shape
    out = torch.empty((B, T, H, D), dtype=dt, device="cuda")
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    S_T_rev = torch.empty_like(S_T) if w.bidirectional else None
    io = gdn.GDN_BF16 if w.dtype == "bf16" else gdn.GDN_F32
    ws_bytes = (gdn.gdn_fwd_bidir_workspace_bytes if w.bidirectional else gdn.gdn_fwd_workspace_bytes)(
        B, T, H, D, io)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    lib = gdn.load()
    p = gdn.make_params(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"],
                        d["conv_v"], d["norm_w"], d["S0"], out, S_T, workspace)
    stream = torch.cuda.Stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    rev_ptr = ctypes.c_void_p(S_T_rev.data_ptr() if S_T_rev is not None else None)

    def step():
        if w.bidirectional:
            st = lib.gdn_fwd_bidir(ctypes.byref(p), rev_ptr, sptr)
        else:
            st = lib.gdn_fwd(ctypes.byref(p), sptr)
        if st != gdn.GDN_OK:
            raise gdn.GdnError(st, "step")

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = B * T / (ms_per_step * 1e-3)
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step, {tokens_per_s:.4e} tokens/s")

    # ---- per-kernel durations from HIP events recorded on each launch's stream
    ev = HipEvents()
    bid = 1 if w.bidirectional else 0
    nl = lib.gdn_fwd_launch_count(ctypes.byref(p), bid)
    names = [lib.gdn_fwd_launch_name(ctypes.byref(p), bid, i).decode() for i in range(nl)]
    reps = min(args.steps, 20)
    evs = [ev.create(2 * nl) for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        st = lib.gdn_fwd_timed(ctypes.byref(p), rev_ptr, bid, evs[i], 2 * nl, sptr)
        if st != gdn.GDN_OK:
            raise gdn.GdnError(st, "gdn_fwd_timed")
    torch.cuda.synchronize()
    per_launch = {}   # kernel -> list of single-launch durations (ms)
    per_call = {}     # kernel -> list of summed durations per call (ms)
    for i in range(reps):
        tot = {}
        for j, nm in enumerate(names):
            ev.sync(evs[i][2 * j + 1])
            dms = ev.elapsed_ms(evs[i][2 * j], evs[i][2 * j + 1])
            per_launch.setdefault(nm, []).append(dms)
            tot[nm] = tot.get(nm, 0.0) + dms
        for nm, v in tot.items():
            per_call.setdefault(nm, []).append(v)
    launches_per_call = {nm: names.count(nm) for nm in set(names)}
    es = 2 if w.dtype == "bf16" else 4
    kernels = {}
    token_heads = B * T * H * (2 if w.bidirectional else 1)   # per direction scanned
    tag = f"T{T}_H{H}_d{D}_{w.dtype}" + ("_bidir" if w.bidirectional else "") + (f"_B{B}" if B > 1 else "")
    for nm in per_launch:
        per_launch_ms = float(np.mean(per_launch[nm]))
        call_ms = float(np.mean(per_call[nm]))
        own_bytes = kernel_bytes_per_token_head(D, es)[nm] * token_heads
        if nm == "gdn_out_kernel" and w.bidirectional:  # + fp32 accumulator write and read
            own_bytes += 2 * 4 * D * B * T * H
        kernels[nm] = {"launches_per_call": launches_per_call[nm], "avg_ms": per_launch_ms,
                       "ms_per_call": call_ms, "own_io_bytes_per_launch": own_bytes / launches_per_call[nm],
                       "own_io_GBps": own_bytes / (call_ms * 1e-3) / 1e9,
                       "traffic_per_launch": profiled_traffic(nm, f"gdn_kernels_{tag}")}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_call"])
    kd = kernels[dom]
    # the layer's per-unit figure times the token-heads one launch of the dominant kernel covers
    unit_bytes = layer_bytes_per_token_head(D, es)
    alg_per_launch = unit_bytes * token_heads / kd["launches_per_call"]
    achieved = alg_per_launch / (kd["avg_ms"] * 1e-3) / 1e9
    traffic = kd["traffic_per_launch"]
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic),
                "traffic_over_algorithmic": None if traffic is None else round(traffic / alg_per_launch, 3),
                "algorithmic_bytes_per_launch": round(alg_per_launch),
                "token_heads_per_launch": token_heads // kd["launches_per_call"],
                "avg_launch_ms": round(kd["avg_ms"], 5)}
    # the whole call: one read of the inputs and one write of y per token-head, either direction count
    layer_bytes = unit_bytes * B * T * H
    call_traffic = None
    if all(k["traffic_per_launch"] is not None for k in kernels.values()):
        call_traffic = sum(k["traffic_per_launch"] * k["launches_per_call"] for k in kernels.values())
    layer = {"algorithmic_bytes": layer_bytes, "floor_ms": layer_bytes / (HBM_PEAK_GBS * 1e9) * 1e3,
             "frac_of_hbm_roofline": round(layer_bytes / (HBM_PEAK_GBS * 1e9) * 1e3 / ms_per_step, 4),
             "traffic_per_call": None if call_traffic is None else round(call_traffic),
             "traffic_over_algorithmic": None if call_traffic is None else round(call_traffic / layer_bytes, 3)}
    for nm, k in kernels.items():
        log(f"  {nm}: {k['avg_ms']:.4f} ms/launch x{k['launches_per_call']} = {k['ms_per_call']:.4f} ms/call, "
            f"own I/O {k['own_io_GBps']:.0f} GB/s")

    # ---- CPU baseline: the fp64 oracle on this host, same workload
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        y_gpu = out.double().cpu().numpy()
        st_gpu = S_T.double().cpu().numpy()
        log("running the oracle on the host ...")
        t1 = time.perf_counter()
        if w.bidirectional:
            ry, rs, _, used = oracle.inputs_for(inp, threads=args.cpu_threads, bidir=True)
        else:
            ry, rs, used = oracle.inputs_for(inp, threads=args.cpu_threads)
        cpu_s = time.perf_counter() - t1
        cpu = {"value": round(B * T / cpu_s, 2), "unit": "tokens/s", "cores": int(used), "kind": "oracle",
               "sample": f"the whole workload ({B}x{T} tokens x {H} heads, fp64, one thread per head"
                         f"{' and direction' if w.bidirectional else ''}), {cpu_s:.2f} s wall",
               "host_cores_available": len(os.sched_getaffinity(0))}

        def rel(a, b):
            return float(np.linalg.norm(a - b) / np.linalg.norm(b))
        parity = {"y_rel_l2": rel(y_gpu, ry), "S_T_rel_l2": rel(st_gpu, rs)}
        log(f"oracle {cpu_s:.2f} s on {used} threads; parity {parity}")

    res = {
        "metric": "GDN layer fwd tokens/s at T=32760,H=12,d=128 bf16; % of MI355X roofline",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name + (f", run as a batch of B={B}" if B != w.B else ""),
                   "launches": "direct" if args.no_graph_cache or w.bidirectional else "cached graph",
                   "B": B, "T": T, "H": H,
                   "d": D, "chunk": 64,
                   "bidirectional": w.bidirectional},
        "roofline": roofline,
        "layer": layer,
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(res), flush=True)
    return 0


GEMM_KERNELS = {"in_proj": "gdn_gemm_kernel<in-projection>", "out_proj": "gdn_gemm_kernel<plain>"}


def run_mixer(args) -> int:
    """One step = one gdn_mixer_fwd call: in-projection (bf16 MFMA GEMM with
    the gate parameterisation in its epilogue), the layer, out-projection."""
    import numpy as np
    import torch

    import gdn_inputs
    import linear_attention_token_fwd_amd as gdn

    w = gdn_inputs.MIXER_WORKLOADS[1]
    log(f"mixer workload: {w.name}")
    inp = gdn_inputs.generate_mixer(w)
    B, T, H, D, C = w.B, w.T, w.H, w.D, w.C
    N = 4 * H * D + 2 * H

    def dev(a, dt=torch.float32):
        return None if a is None else torch.from_numpy(a).to("cuda").to(dt).contiguous()
    x, w_in, w_out = dev(inp["x"], torch.bfloat16), dev(inp["w_in"], torch.bfloat16), dev(inp["w_out"], torch.bfloat16)
    b_in, b_out, A_log = dev(inp["b_in"]), dev(inp["b_out"]), dev(inp["A_log"])
    conv = [dev(inp[k]) for k in ("conv_q", "conv_k", "conv_v")]
    norm_w = dev(inp["norm_w"])
    out = torch.empty((B, T, C), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    workspace = torch.empty(gdn.gdn_mixer_workspace_bytes(B, T, H, D, C), dtype=torch.uint8, device="cuda")
    lib = gdn.load()
    p = gdn.mixer_params(x, w_in, b_in, A_log, *conv, norm_w, None, w_out, b_out, out, S_T, workspace, H, D)
    stream = torch.cuda.Stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step():
        st = lib.gdn_mixer_fwd(ctypes.byref(p), sptr)
        if st != gdn.GDN_OK:
            raise gdn.GdnError(st, "gdn_mixer_fwd")

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    tokens_per_s = B * T / (ms_per_step * 1e-3)
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step, {tokens_per_s:.4e} tokens/s")

    # ---- per-kernel durations (HIP events on each launch's stream)
    ev = HipEvents()
    lp = gdn._sizes(B, T, H, D, gdn.GDN_BF16)
    nl = lib.gdn_fwd_launch_count(ctypes.byref(lp), 0)
    names = ["in_proj", "out_proj"] + [lib.gdn_fwd_launch_name(ctypes.byref(lp), 0, i).decode() for i in range(nl)]
    reps = min(args.steps, 20)
    nev = 4 + 2 * nl
    evs = [ev.create(nev) for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        st = lib.gdn_mixer_fwd_timed(ctypes.byref(p), evs[i], nev, sptr)
        if st != gdn.GDN_OK:
            raise gdn.GdnError(st, "gdn_mixer_fwd_timed")
    torch.cuda.synchronize()
    per_launch, per_call = {}, {}
    for i in range(reps):
        tot = {}
        for j, nm in enumerate(names):
            ev.sync(evs[i][2 * j + 1])
            dms = ev.elapsed_ms(evs[i][2 * j], evs[i][2 * j + 1])
            per_launch.setdefault(nm, []).append(dms)
            tot[nm] = tot.get(nm, 0.0) + dms
        for nm, v in tot.items():
            per_call.setdefault(nm, []).append(v)
    flops = {"in_proj": 2.0 * B * T * C * N, "out_proj": 2.0 * B * T * H * D * C}
    kb = kernel_bytes_per_token_head(D, 2)
    kernels = {}
    for nm in per_launch:
        n = names.count(nm)
        k = {"launches_per_call": n, "avg_ms": float(np.mean(per_launch[nm])),
             "ms_per_call": float(np.mean(per_call[nm]))}
        if nm in flops:
            k["kernel"] = GEMM_KERNELS[nm]
            k["flops_per_launch"] = flops[nm]
            k["TFLOPs"] = flops[nm] / (k["avg_ms"] * 1e-3) / 1e12
        else:
            k["bytes_per_launch"] = kb[nm] * B * T * H / n
            k["GBps"] = kb[nm] * B * T * H / (k["ms_per_call"] * 1e-3) / 1e9
        kernels[nm] = k
        log(f"  {nm}: {k['avg_ms']:.4f} ms/launch x{n} = {k['ms_per_call']:.4f} ms/call")
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_call"])
    kd = kernels[dom]
    if dom in flops:
        achieved = kd["flops_per_launch"] / (kd["avg_ms"] * 1e-3) / 1e12
        traffic = profiled_traffic(kd["kernel"], f"gdn_mixer_T{T}_C{C}_H{H}_d{D}_bf16", MIXER_SOURCES)
        roofline = {"kernel": kd["kernel"], "bound": "mfma", "achieved": round(achieved, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": None if traffic is None else round(traffic), "avg_launch_ms": round(kd["avg_ms"], 5)}
    else:
        achieved = kd["bytes_per_launch"] / (kd["avg_ms"] * 1e-3) / 1e9
        traffic = profiled_traffic(dom, f"gdn_mixer_T{T}_C{C}_H{H}_d{D}_bf16", MIXER_SOURCES)
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": None if traffic is None else round(traffic), "avg_launch_ms": round(kd["avg_ms"], 5)}

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        from oracle import proj as oproj
        got = out.double().cpu().numpy()
        got_s = S_T.double().cpu().numpy()
        log("running the oracle on the host ...")
        t1 = time.perf_counter()
        ref, ref_s, _ = oproj.mixer(inp["x"], inp["w_in"], inp["b_in"], inp["A_log"], inp["conv_q"],
                                    inp["conv_k"], inp["conv_v"], inp["norm_w"], inp["w_out"], inp["b_out"],
                                    H, D, threads=args.cpu_threads)
        cpu_s = time.perf_counter() - t1
        cores = min(H, len(os.sched_getaffinity(0))) if args.cpu_threads == 0 else args.cpu_threads
        cpu = {"value": round(B * T / cpu_s, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"the whole workload ({B}x{T} tokens, fp64 projections with numpy, the layer one "
                         f"thread per head), {cpu_s:.2f} s wall",
               "host_cores_available": len(os.sched_getaffinity(0))}
        parity = {"out_rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
                  "S_T_rel_l2": float(np.linalg.norm(got_s - ref_s) / np.linalg.norm(ref_s))}
        log(f"oracle {cpu_s:.2f} s; parity {parity}")

    res = {
        "metric": "GDN token mixer fwd tokens/s (in-projection, layer, out-projection) at T=32760,C=1536,"
                  "H=12,d=128 bf16",
        "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layer launches": "direct" if args.no_graph_cache else "cached graph",
                   "B": B, "T": T, "H": H, "d": D, "C": C, "chunk": 64},
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "cpu_baseline": cpu, "parity": parity,
    }
    print(json.dumps(res), flush=True)
    return 0


BWD_SOURCES = ("frag.hpp", "bwd.hpp", "gdn_bwd.hip")
MFMA_F32_PEAK_TFLOPS = 157.3


def bwd_flops_per_chunk_head(D: int) -> dict:
    """fp32 MFMA flops per (chunk, head) of the backward's kernels, as
    executed (the triangular 64 x 64 products in 10 of their 16 tiles):
      prep : K K^T (tri), P = Q K^T (tri), U~ = T V, W = T K, P W
      state: U = W S^T, S += U^T D K              (per chunk and head)
      out  : Q' S^T, P U~
      dstate: dS (D K)^T, X W, dO^T Q'
      grad : W S^T, K dS'^T, dO S, U dS', dW = dU S (64 D^2 each); P^T dO,
             T^T dW, T^T dU, F K, F^T K, G^T Q, G K (64 64 D each);
             dO U^T, dR_W W^T, dR_U U~^T (tri; E o K K^T comes from prep)."""
    t, tri = 64 * 64 * D, 64 * 64 * D * 10 / 16
    sq = 64 * D * D
    return {"bwd_prep_kernel": 2 * (2 * tri + 3 * t), "bwd_state_kernel": 2 * (2 * sq),
            "bwd_out_kernel": 2 * (sq + t), "bwd_dstate_kernel": 2 * (3 * sq),
            "bwd_grad_kernel": 2 * (5 * sq + 7 * t + 3 * tri)}


def run_bwd(args) -> int:
    """One step = one gdn_bwd call (the layer's gradients with respect to
    all inputs, the forward recomputed inside) on the workload."""
    import numpy as np
    import torch

    import gdn_inputs
    import linear_attention_token_fwd_amd as gdn

    w = gdn_inputs.WORKLOADS[args.workload]
    if w.bidirectional:
        log("the backward covers the single-direction layer; use another workload")
        return 2
    log(f"backward workload: {w.name}")
    inp = gdn_inputs.generate(w, B=args.batch or None)
    B, T, H, D = inp["q"].shape
    grads = gdn_inputs.generate_grads(w, seed=5000 + w.id, T=T, H=H, B=B)
    io = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = gdn.to_device(inp, dtype=io)
    dy = torch.from_numpy(grads["dy"]).to(io).cuda()
    dS = torch.from_numpy(grads["dS_T"]).cuda()
    out = {n: torch.empty((B, T, H, D), dtype=io, device="cuda") for n in ("q", "k", "v", "gate")}
    out.update({n: torch.empty((B, T, H), device="cuda") for n in ("log_a", "beta")})
    out.update({n: torch.empty((H * D, 4), device="cuda") for n in ("conv_q", "conv_k", "conv_v")})
    out["norm_w"] = torch.empty((H, D), device="cuda")
    out["S0"] = torch.empty((B, H, D, D), device="cuda")
    ws = torch.empty(gdn.gdn_bwd_workspace_bytes(B, T, H, D, gdn.GDN_BF16 if io == torch.bfloat16 else gdn.GDN_F32),
                     dtype=torch.uint8, device="cuda")
    lib = gdn.load()
    p = gdn.bwd_params(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"],
                       d["conv_v"], d["norm_w"], d["S0"], dy, dS, out, ws)
    stream = torch.cuda.Stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step():
        st = lib.gdn_bwd(ctypes.byref(p), sptr)
        if st != gdn.GDN_OK:
            raise gdn.GdnError(st, "gdn_bwd")

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    tokens_per_s = B * T / (ms_per_step * 1e-3)
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step, {tokens_per_s:.4e} tokens/s")

    # ---- per-kernel durations (HIP events on the launch stream)
    ev = HipEvents()
    names = gdn.gdn_bwd_launch_names()
    reps = min(args.steps, 10)
    nev = 2 * len(names)
    evs = [ev.create(nev) for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        st = lib.gdn_bwd_timed(ctypes.byref(p), evs[i], nev, sptr)
        if st != gdn.GDN_OK:
            raise gdn.GdnError(st, "gdn_bwd_timed")
    torch.cuda.synchronize()
    per = {nm: [] for nm in names}
    for i in range(reps):
        for j, nm in enumerate(names):
            ev.sync(evs[i][2 * j + 1])
            per[nm].append(ev.elapsed_ms(evs[i][2 * j], evs[i][2 * j + 1]))
    NC = (T + 63) // 64
    fl = bwd_flops_per_chunk_head(D)
    kernels = {}
    for nm in names:
        k = {"avg_ms": float(np.mean(per[nm]))}
        if nm in fl:
            k["flops_per_launch"] = fl[nm] * B * H * NC
            k["TFLOPs"] = k["flops_per_launch"] / (k["avg_ms"] * 1e-3) / 1e12
        kernels[nm] = k
        log(f"  {nm}: {k['avg_ms']:.4f} ms" + (f", {k['TFLOPs']:.1f} TFLOP/s" if "TFLOPs" in k else ""))
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    kd = kernels[dom]
    achieved = kd.get("TFLOPs", 0.0)
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F32_PEAK_TFLOPS, 4), "traffic": None,
                "avg_launch_ms": round(kd["avg_ms"], 5)}

    cpu = None
    if not args.no_cpu_baseline:
        # the autograd oracle on a bounded sample: the first 256 tokens of one head
        from oracle import bwd as obwd
        Ts = min(T, 6144)
        sample = {n: (None if inp[n] is None else
                      (inp[n][:1, :Ts, :1] if n in ("q", "k", "v", "gate", "log_a", "beta") else
                       inp[n][:D] if n.startswith("conv") else inp[n][:1] if n == "norm_w" else inp[n][:1, :1]))
                  for n in obwd.NAMES}
        threads = torch.get_num_threads()
        log("running the backward oracle on a sample ...")
        t1 = time.perf_counter()
        obwd.backward(sample, grads["dy"][:1, :Ts, :1], grads["dS_T"][:1, :1])
        cpu_s = time.perf_counter() - t1
        cpu = {"value": round(Ts / cpu_s / H, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"one head, first {Ts} tokens (torch fp64 autograd, token loop), {cpu_s:.2f} s wall; "
                         f"tokens/s of the {H}-head layer = sampled token-heads/s / {H}"}
        log(f"oracle sample {cpu_s:.2f} s")

    res = {
        "metric": f"GDN layer backward tokens/s at T={T},H={H},d={D} {w.dtype} I/O",
        "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name + " (backward: all gradients, forward recomputed)", "B": B, "T": T, "H": H,
                   "d": D, "io": w.dtype, "chunk": 64},
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
