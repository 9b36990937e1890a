#!/usr/bin/env python3
"""Benchmark of libgdn on one MI355X: the gated delta-rule scan hot path.

One step = one gdn_forward call (chunk preparation + state chain) over the
whole synthetic input of the workload, inputs already resident in HBM.
Default workload: the 480p bidirectional DiT linear block, B=2, H=16,
T=32760 (21 latent frames of 30x52 tokens), dk=dv=128, bf16 inputs, fp32
state and output, forward + reverse scans summed.

Prints ONE JSON line with tokens/s (B*T tokens per step), the algorithmic
TFLOP/s and fraction of the bf16 matrix-core peak, the per-kernel roofline of
the dominant kernel measured live with HIP events (algorithmic bytes = the
boundary tensors, each once; the workspace is reported apart), the error of
sampled (batch, head) chains against the double-precision oracle, and that
oracle timed on the host on a bounded sample of the same workload.

The streaming workload (stream480) is timed as its rollout: 21 in-place calls
of one latent frame each (1560 tokens, the state carried in place), eagerly
and as one captured HIP graph replayed; one step = one rollout.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload bidir480]
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

MI355X_HBM_GBS = 8000.0          # published HBM3E bandwidth
MI355X_BF16_TFLOPS = 2516.6      # dense bf16 matrix peak: 256 CU x 4096 flop/clk x 2.4 GHz
MI355X_FP32_TFLOPS = 157.3
REF_CHUNK = 64                   # chunk length the algorithmic flop count is quoted at


def flops_per_token_head_dir(dk: int, dv: int, C: int = REF_CHUNK) -> float:
    """Algorithmic flops of the chunked method per token, head and direction:
    W S^T, Q S^T, K^T Vnew (2 C dk dv per chunk each); K K^T strict, Q K^T,
    Tinv (beta gamma K) (C(C+-1) dk); Tinv (beta V) and P Vnew (C(C+1) dv);
    the triangular inverse (C^3/3), all divided by C."""
    return 6 * dk * dv + (3 * C + 1) * dk + 2 * (C + 1) * dv + C * C / 3.0


def path_bytes(w, xs: int) -> float:
    """Boundary tensors read once and written once (workspace excluded)."""
    th = w.B * w.T * w.H
    per_th = (2 * w.dk + w.dv) * xs + w.dirs * 8 + w.dv * 4
    states = w.dirs * w.B * w.H * w.dv * w.dk * 4 * (2 if w.state_std > 0 else 1)
    return th * per_th + states


def kernel_bytes(w, xs: int) -> dict:
    """Algorithmic bytes of each kernel, boundary tensors only, each once: the
    preparation pass reads q, k and the gates; the chain reads q, k, v and the
    states and writes out and the final states.  Workspace traffic (the
    prepared triangles and scales) is excluded and reported apart."""
    th = w.B * w.T * w.H
    states = w.dirs * w.B * w.H * w.dv * w.dk * 4 * (2 if w.state_std > 0 else 1)
    return {"prep": th * (2 * w.dk * xs + w.dirs * 8),
            "chain": th * ((2 * w.dk + w.dv) * xs + w.dv * 4) + states,
            "path": path_bytes(w, xs)}


def chain_kernel_name(dtype: str, chunk: int = 0) -> str:
    """bf16 operands run the column-owning chain, fp32 operands and 128-token
    chunks the two-role one."""
    return "column_chain_kernel" if dtype == "bf16" and chunk != 128 else "chain_kernel"


def prep_kernel_name(chunk: int = 0) -> str:
    """128-token chunks have a preparation kernel of their own."""
    return "chunk_prep_wide_kernel" if chunk == 128 else "chunk_prep_kernel"


def host_cores():
    """(threads to use, cores visible): the affinity mask, capped by the
    cgroup CPU quota and by OMP_NUM_THREADS when either is set (the host's
    own thread budget)."""
    visible = len(os.sched_getaffinity(0))
    avail = visible
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            avail = min(avail, max(1, int(quota) // int(period)))
    except (OSError, ValueError):
        pass
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        avail = min(avail, int(omp))
    return avail, visible


def sampled_parity(w, x, out, s_out, direction, erase=True, exclusive="none", threads=None, epilogue=None) -> dict:
    """max |gpu - oracle| / RMS(oracle) over two (batch, head) chains computed
    in full by the oracle (every token, both directions when bidirectional,
    and the final states; with `epilogue`, the oracle's readout epilogue on
    its output).  Chains are independent, so this is the oracle restricted
    to those chains."""
    import numpy as np

    import oracle

    heads = list(dict.fromkeys([(0, 0), (w.B - 1, w.H - 1)]))
    t0 = time.perf_counter()
    ro, rs = oracle.forward_heads(x, heads, direction, nthreads=threads, erase=erase, exclusive=exclusive)
    if epilogue is not None:
        gate = np.stack([epilogue["gate"][b, :, h] for b, h in heads])
        ro = oracle.readout_epilogue(ro, gate, epilogue["norm_weight"], 1e-6)
    dt = time.perf_counter() - t0

    def rel(got, ref):
        ref = np.asarray(ref, np.float64)
        rms = float(np.sqrt(np.mean(ref * ref)))
        return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / max(rms, 1e-30)

    o = out.cpu().numpy()
    so = s_out.cpu().numpy()
    eo = max(rel(o[b, :, h], ro[i]) for i, (b, h) in enumerate(heads))
    es = max(rel(so[:, b, h], rs[:, i]) for i, (b, h) in enumerate(heads))
    return {"heads": [list(h) for h in heads], "out_max_err_over_rms": eo, "state_max_err_over_rms": es,
            "tol": 2e-2 if w.dtype == "bf16" else 1e-4, "finite": bool(np.all(np.isfinite(o))),
            "oracle_seconds": round(dt, 2)}


KERNEL_SOURCES = {
    "chain_kernel": ["gdn_chain.hip", "gdn_common.h"],
    "column_chain_kernel": ["gdn_colchain.hip", "gdn_common.h"],
    "chunk_prep_kernel": ["gdn_prep.hip", "gdn_common.h"],
    "chunk_prep_wide_kernel": ["gdn_prep_wide.hip", "gdn_common.h"],
    "vda_frame_kernel": ["gdn_vda.hip", "gdn_common.h"],
    "vda_chain_bf16_kernel": ["gdn_vda.hip", "gdn_common.h"],
    "vda_readout_kernel": ["gdn_vda.hip", "gdn_common.h"],
}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the sources a kernel is built from (tells whether measured
    counters still describe the code being timed)."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "gated_delta_rule_scan_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>_traffic.md), or None when there is none or
    the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic-json:"):
            d = json.loads(line.split(":", 1)[1])
            if d.get("source_hash") == kernel_source_hash(kernel):
                return d["bytes_per_launch"]
    return None


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime (the library records them
    on the stream its kernels run on)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = h
        self.n = n

    def ptr(self, i: int) -> int:
        return ctypes.addressof(self.arr) + i * ctypes.sizeof(ctypes.c_void_p)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.arr[i])


def cpu_baseline(w, x, target_s: float, erase: bool = True, exclusive: str = "none") -> dict:
    """Time the double-precision oracle on the host on a bounded sample of the
    workload: every (batch, head) chain if that fits about `target_s` seconds,
    else the first tokens of every chain.  `erase` and `exclusive` select the
    same operator the GPU leg runs."""
    import oracle

    threads, visible = host_cores()
    cal_T = min(w.T, 1024)
    t0 = time.perf_counter()
    oracle.forward_heads({"q": x["q"][:, :cal_T], "k": x["k"][:, :cal_T], "v": x["v"][:, :cal_T],
                          "log_alpha": x["log_alpha"][:1, :, :cal_T], "beta": x["beta"][:1, :, :cal_T],
                          "state_in": None}, [(0, 0)], "fwd", nthreads=1)
    per_tok = (time.perf_counter() - t0) / cal_T           # one chain, one thread
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    n_chains = len(heads) * w.dirs
    waves = -(-n_chains // threads)
    est = waves * w.T * per_tok
    Ts = w.T if est <= target_s else max(1024, int(w.T * target_s / est))
    xs = {"q": x["q"][:, :Ts], "k": x["k"][:, :Ts], "v": x["v"][:, :Ts],
          "log_alpha": x["log_alpha"][:, :, :Ts], "beta": x["beta"][:, :, :Ts], "state_in": x["state_in"]}
    t0 = time.perf_counter()
    oracle.forward_heads(xs, heads, w.direction, nthreads=threads, erase=erase, exclusive=exclusive)
    dt = time.perf_counter() - t0
    thd = n_chains * Ts / dt                                # token-head-directions per second
    used = min(threads, n_chains)
    what = "the whole workload" if Ts == w.T else f"the first {Ts} of {w.T} tokens of every chain"
    return {"value": thd / (w.H * w.dirs), "unit": "tokens/s", "cores": used, "cores_available": threads,
            "cores_visible": visible, "kind": "oracle",
            "sample": f"{what}: {len(heads)} heads x {w.dirs} direction(s), {used} threads, {dt:.1f} s; "
                      f"tokens/s = token-head-directions/s / (H*dirs)",
            "seconds": round(dt, 2)}


VDA_KERNEL = {"vda_frame": "vda_frame_kernel", "vda_chain": "vda_chain_bf16_kernel", "vda_readout": "vda_readout_kernel"}
VDA_FRAME = {"stream480": 1560, "bidir480": 1560, "causal720": 3600, "bidir720": 3600, "causal720_slow": 3600}


def run_vda(args, w) -> int:
    """One gdn_vda_forward per step on the workload's shape, frames of one
    latent frame's tokens (30 x 52 at 480p, 45 x 80 at 720p)."""
    import numpy as np
    import torch

    import gated_delta_rule_scan_amd as gdn
    import synth
    from oracle import vda as vda_oracle

    frame = VDA_FRAME.get(args.workload, 64)
    x = synth.generate_frames(w, frame)
    xs = 2 if w.dtype == "bf16" else 4

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    d = {k: dev(v) for k, v in x.items()}
    epi = {}
    if args.vda_epilogue:
        e = synth.generate_epilogue(w)
        epi = dict(gate=dev(e["gate"]), norm_weight=dev(e["norm_weight"]), norm_eps=1e-6)
    out = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    s_out = torch.empty((w.dirs, w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
    ws = None

    def step(ev_ptr=None):
        nonlocal ws
        _, _ = gdn.vda_forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], w.direction, frame,
                               out=out, state_out=s_out, workspace=ws, timing_events=ev_ptr, write=args.vda_write,
                               lag=args.vda_lag, **epi)

    nb = gdn.gdn_vda_workspace_bytes(gdn.gdn_vda_problem_t(
        B=w.B, T=w.T, H=w.H, dk=w.dk, dv=w.dv, frame=frame,
        dtype=gdn.GDN_DTYPE_BF16 if w.dtype == "bf16" else gdn.GDN_DTYPE_F32), gdn.DIRECTIONS[w.direction])
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    # K calls with the library's four HIP events each for the per-kernel
    # durations, then the timed steps: the same K calls without per-call events
    ev = HipEvents(4 * K)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        step(ev.ptr(4 * i))
    e1.record()
    torch.cuda.synchronize()
    ms_step_events = e0.elapsed_time(e1) / K
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / K
    km = {n: sum(ev.elapsed_ms(4 * i + a, 4 * i + a + 1) for i in range(K)) / K
          for n, a in (("vda_frame", 0), ("vda_chain", 1), ("vda_readout", 2))}
    ev.close()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    B, T, H, dk, dv, dirs = w.B, w.T, w.H, w.dk, w.dv, w.dirs
    NF = (T + frame - 1) // frame
    nfr = dirs * B * H * NF
    tok_hd = B * T * H * dirs
    # algorithmic bytes and flops per launch of each kernel (every tensor once)
    kb = {"vda_frame": B * T * H * (dk + dv) * xs + dirs * B * T * H * 4 + nfr * (dk * dk + dv * dk) * 4,
          "vda_chain": nfr * (dk * dk + 2 * dv * dk) * 4 + 2 * dirs * B * H * dv * dk * 4,
          "vda_readout": B * T * H * dk * xs + nfr * dv * dk * 4 + B * T * H * dv * 4}
    kf = {"vda_frame": tok_hd * 2 * (dk * dk + dv * dk) + nfr * (2 * dk ** 3 + 2 * dv * dk * dk),
          "vda_chain": nfr * 2 * dv * dk * dk,
          "vda_readout": tok_hd * 2 * dk * dv}
    dom = max(km, key=km.get)
    peak_mfma = MI355X_BF16_TFLOPS if w.dtype == "bf16" else MI355X_FP32_TFLOPS
    res = {
        "metric": "frame-wise delta operator (VDA) tokens/s, 1 MI355X",
        "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "operator": ("frame-wise delta (Video Delta Attention)" if args.vda_write == "inverse"
                                                 else "additive frame writes, keys / sqrt(U)"),
                   "readout_lag": args.vda_lag, "epilogue": bool(args.vda_epilogue), "frame": frame,
                   "frames": NF, "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "direction": w.direction},
        "kernels_ms": km,
        "ms_per_step_with_kernel_events": ms_step_events,
        "tflops": sum(kf.values()) / (ms_step * 1e-3) / 1e12,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": kb[dom] / (km[dom] * 1e-3) / 1e9,
                     "peak": MI355X_HBM_GBS, "unit": "GB/s", "frac": kb[dom] / (km[dom] * 1e-3) / 1e9 / MI355X_HBM_GBS,
                     # counters were taken on the operator's default options only
                     "traffic": (measured_traffic(VDA_KERNEL[dom], args.workload)
                                 if (args.vda_write, args.vda_lag, args.vda_epilogue) == ("inverse", 0, False) else None),
                     "alg_bytes_per_launch": kb[dom], "avg_launch_ms": km[dom],
                     "mfma_tflops": kf[dom] / (km[dom] * 1e-3) / 1e12,
                     "mfma_frac": kf[dom] / (km[dom] * 1e-3) / 1e12 / peak_mfma},
    }
    if not args.no_cpu_baseline:
        # the oracle on one host thread (BLAS pinned to one thread) over whole
        # (batch, head) chains, both directions, until about --cpu-seconds
        from threadpoolctl import threadpool_limits
        t0 = time.perf_counter()
        n = 0
        with threadpool_limits(limits=1):
            for b, h in [(b_, h_) for b_ in range(B) for h_ in range(H)]:
                if n and time.perf_counter() - t0 > args.cpu_seconds:
                    break
                sel = {k: x[k][b:b + 1, :, h:h + 1] for k in ("q", "k", "v")}
                ekw = {}
                if args.vda_epilogue:
                    ekw = dict(gate=e["gate"][b:b + 1, :, h:h + 1], norm_weight=e["norm_weight"], norm_eps=1e-6)
                vda_oracle.forward(sel["q"], sel["k"], sel["v"], x["log_alpha"][:, b:b + 1, :, h:h + 1],
                                   x["beta"][:, b:b + 1, :, h:h + 1], None, w.direction, frame,
                                   write=args.vda_write, lag=args.vda_lag, **ekw)
                n += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": n * T / dt / H, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} of {B * H} (batch, head) chains over all {T} tokens, "
                                         f"{w.dirs} direction(s), numpy float64 on one thread, {dt:.1f} s; "
                                         f"tokens/s = chains x T / s / H",
                               "seconds": round(dt, 2)}
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bidir480")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--dv-tile", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle check of sampled chains")
    ap.add_argument("--serial", action="store_true", help="keep the preparation pass before the chain (no overlap)")
    ap.add_argument("--no-erase", action="store_true",
                    help="time the erase-free variant (gated linear attention, GDN_OPT_NO_ERASE) instead of the delta rule")
    ap.add_argument("--epilogue", action="store_true",
                    help="the readout epilogue (RMS norm over dv and sigmoid gate) after the scan")
    ap.add_argument("--exclusive", choices=["none", "fwd", "rev", "both"], default="none",
                    help="directions that read before the token's own write (GDN_OPT_EXCLUSIVE_*: disjoint regions)")
    ap.add_argument("--vda", action="store_true",
                    help="time the frame-wise delta operator (gdn_vda_forward) on the workload's frames instead")
    ap.add_argument("--vda-write", choices=("inverse", "additive"), default="inverse",
                    help="--vda: the operator's inverse write or the additive write (keys / sqrt(U))")
    ap.add_argument("--vda-lag", type=int, default=0, help="--vda: readout lag in frames (disjoint-region readout)")
    ap.add_argument("--vda-epilogue", action="store_true", help="--vda: fused RMS-norm and sigmoid-gate epilogue")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run one plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the scan shards over (batch, head, "
                                   "direction) chains with no communication; run with --gpus 1"}))
        return 2

    import numpy as np
    import torch

    import gated_delta_rule_scan_amd as gdn
    import synth

    w = synth.WORKLOADS[args.workload]
    if args.vda:
        return run_vda(args, w)
    if w.frame:
        return run_stream(args, w)
    xs = 2 if w.dtype == "bf16" else 4
    x = synth.generate(w)
    d = {k: _dev(v) for k, v in x.items()}
    epi = {}
    if args.epilogue:
        e = synth.generate_epilogue(w)
        epi = dict(gate=_dev(e["gate"]), norm_weight=_dev(e["norm_weight"]), norm_eps=1e-6)
    out = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    s_out = torch.empty((w.dirs, w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
    nws = gdn.workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.direction, args.chunk, args.dv_tile,
                              args.exclusive)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    C = args.chunk or 64

    def step(ev_ptr=None):
        gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], w.direction, chunk=args.chunk,
                    dv_tile=args.dv_tile, out=out, state_out=s_out, workspace=ws, timing_events=ev_ptr,
                    serial=args.serial, erase=not args.no_erase, exclusive=args.exclusive, **epi)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    # per-kernel durations: K calls, each with four HIP events recorded by the
    # library (prep start/end on the stream prep runs on, chain start/end on
    # the caller's stream)
    ev = HipEvents(4 * K)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(K):
        step(ev.ptr(4 * i))
    e1.record()
    torch.cuda.synchronize()
    ms_step_events = e0.elapsed_time(e1) / K
    # the timed steps: the same K calls as a user makes them (no per-call events)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(K):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(stop) / K
    prep_ms = sum(ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(K)) / K
    chain_ms = sum(ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(K)) / K
    # one call's span, prep start to chain end (the library's own events)
    spans = sorted(max(ev.elapsed_ms(4 * i, 4 * i + 3), ev.elapsed_ms(4 * i + 2, 4 * i + 3)) for i in range(K))
    # the chain started before the preparation pass ended: the two ran concurrently
    concurrent = all(ev.elapsed_ms(4 * i + 1, 4 * i + 2) < 0 for i in range(K))
    ev.close()

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    tokens = w.B * w.T
    th_dirs = w.B * w.T * w.H * w.dirs
    flops = th_dirs * flops_per_token_head_dir(w.dk, w.dv)
    tflops = flops / (ms_step * 1e-3) / 1e12
    kb = kernel_bytes(w, xs)
    kt = {"prep": prep_ms, "chain": chain_ms}
    dom = max(kt, key=kt.get)
    dom_name = chain_kernel_name(w.dtype, args.chunk) if dom == "chain" else prep_kernel_name(args.chunk)
    # the dominant kernel's roofline: the chain moves every boundary tensor but
    # the gates, so the path's boundary bytes are its algorithmic bytes
    dom_bytes = kb["path"] if dom == "chain" else kb["prep"]
    achieved = dom_bytes / (kt[dom] * 1e-3) / 1e9
    peak_mfma = MI355X_BF16_TFLOPS if w.dtype == "bf16" else MI355X_FP32_TFLOPS
    res = {
        "metric": "gated-delta scan tokens/s + TFLOP/s (% MFMA peak) at 480p latent, 1 MI355X",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "direction": w.direction, "chunk": C, "dv_tile": args.dv_tile or "auto",
                   "prep": "concurrent with the chain" if concurrent else "before the chain",
                   "operator": "erase-free (gated linear attention)" if args.no_erase else "gated delta rule",
                   "exclusive_readout": args.exclusive,
                   "readout_epilogue": bool(args.epilogue),
                   "inputs": "seeded synthetic video-latent-shaped (synth.WORKLOADS)"},
        "tflops": tflops,
        "mfma_frac": tflops / peak_mfma,
        "path_bytes": kb["path"],
        "path_hbm_gbs": kb["path"] / (ms_step * 1e-3) / 1e9,
        "path_hbm_frac": kb["path"] / (ms_step * 1e-3) / 1e9 / MI355X_HBM_GBS,
        "kernels_ms": {"chunk_prep": prep_ms, "state_chain": chain_ms},
        "call_ms_median": spans[K // 2], "call_ms_min": spans[0],
        "ms_per_step_with_kernel_events": ms_step_events,
        "roofline": {"kernel": dom_name, "bound": "hbm",
                     "achieved": achieved, "peak": MI355X_HBM_GBS, "unit": "GB/s", "frac": achieved / MI355X_HBM_GBS,
                     # the committed counters were taken with the default options
                     "traffic": (measured_traffic(dom_name, args.workload)
                                 if not args.no_erase and args.exclusive == "none" and not args.chunk
                                 and not args.dv_tile and not args.epilogue else None),
                     "alg_bytes_per_launch": dom_bytes,
                     "workspace_bytes_per_launch": nws,
                     "avg_launch_ms": kt[dom], "source_hash": kernel_source_hash(dom_name)},
        "wall_s_timed": wall,
    }
    if dom == "chain" and prep_ms > 0:
        # the path's other kernel, the same way: its boundary reads (q, k and
        # the gates, each once) per launch over its average launch time
        pname = prep_kernel_name(args.chunk)
        pa = kb["prep"] / (prep_ms * 1e-3) / 1e9
        res["prep_roofline"] = {
            "kernel": pname, "bound": "hbm", "achieved": pa, "peak": MI355X_HBM_GBS, "unit": "GB/s",
            "frac": pa / MI355X_HBM_GBS,
            "traffic": (measured_traffic(pname, args.workload)
                        if not args.no_erase and args.exclusive == "none" and not args.chunk
                        and not args.dv_tile and not args.epilogue else None),
            "alg_bytes_per_launch": kb["prep"], "avg_launch_ms": prep_ms, "beside_chain": bool(concurrent),
            "source_hash": kernel_source_hash(pname)}
    if not args.no_parity:
        res["parity"] = sampled_parity(w, x, out, s_out, w.direction, erase=not args.no_erase,
                                       exclusive=args.exclusive, threads=host_cores()[0],
                                       epilogue=e if args.epilogue else None)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds, erase=not args.no_erase, exclusive=args.exclusive)
        res["gpu_over_cpu"] = res["value"] / res["cpu_baseline"]["value"]
    print(json.dumps(res), flush=True)
    return 0


def _dev(a):
    import numpy as np
    import torch

    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_stream(args, w) -> int:
    """The streaming rollout: one call per latent frame (w.frame tokens), the
    state carried in place (state_in is state_out), as a causal video model
    generating frame by frame calls it.  Inputs are cut into per-frame device
    tensors beforehand; each step is the whole rollout, timed eagerly and as
    one captured HIP graph replayed (the library takes its serial order under
    capture).  Per-frame latency = rollout time / frames."""
    import torch

    import gated_delta_rule_scan_amd as gdn
    import synth

    xs = 2 if w.dtype == "bf16" else 4
    x = synth.generate(w)
    fr = w.frame
    bounds = [(f0, min(w.T, f0 + fr)) for f0 in range(0, w.T, fr)]
    NF = len(bounds)
    frames = []
    for f0, f1 in bounds:
        frames.append({k: _dev(x[k][:, f0:f1]) for k in ("q", "k", "v")} |
                      {k: _dev(x[k][:, :, f0:f1]) for k in ("log_alpha", "beta")})
    s0 = _dev(x["state_in"]) if x["state_in"] is not None else None
    state = torch.zeros((w.dirs, w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
    outs = [torch.empty((w.B, f1 - f0, w.H, w.dv), dtype=torch.float32, device="cuda") for f0, f1 in bounds]
    nws = gdn.workspace_bytes(w.B, fr, w.H, w.dk, w.dv, w.dtype, w.direction, args.chunk, args.dv_tile)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def reset():
        if s0 is not None:
            state.copy_(s0)
        else:
            state.zero_()

    def rollout(evs=None):
        for i, f in enumerate(frames):
            gdn.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], state, w.direction, out=outs[i],
                        state_out=state, workspace=ws, timing_events=None if evs is None else evs.ptr(4 * i),
                        serial=args.serial, chunk=args.chunk, dv_tile=args.dv_tile)

    for _ in range(max(1, args.warmup)):
        reset()
        rollout()
    torch.cuda.synchronize()
    K = args.steps
    # per-kernel durations over one rollout (library events per call)
    ev = HipEvents(4 * NF)
    reset()
    rollout(ev)
    torch.cuda.synchronize()
    prep_ms = sum(ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(NF)) / NF
    chain_ms = sum(ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(NF)) / NF
    ev.close()
    # eager: K rollouts, the state reset (a 1-kernel fill or copy) before each
    t_eager = 0.0
    for _ in range(K):
        reset()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        rollout()
        b.record()
        torch.cuda.synchronize()
        t_eager += a.elapsed_time(b)
    ms_eager = t_eager / K
    # the rollout captured once as a HIP graph, replayed K times
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rollout()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rollout()
    t_graph = 0.0
    for _ in range(K):
        reset()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        t_graph += a.elapsed_time(b)
    ms_graph = t_graph / K
    # the graph's last replay is a full rollout from the initial state
    out = torch.cat(outs, dim=1)
    tokens = w.B * w.T
    flops = tokens * w.H * w.dirs * flops_per_token_head_dir(w.dk, w.dv)
    kb = kernel_bytes(w, xs)
    # per frame: the boundary tensors of one call (the carried state read and written once)
    sb = w.dirs * w.B * w.H * w.dv * w.dk * 4
    fb = (kb["path"] - sb * (2 if w.state_std > 0 else 1)) / NF + 2 * sb
    kt = {"prep": prep_ms, "chain": chain_ms}
    dom = max(kt, key=kt.get)
    dom_name = chain_kernel_name(w.dtype, args.chunk) if dom == "chain" else prep_kernel_name(args.chunk)
    dom_bytes = fb if dom == "chain" else kb["prep"] / NF
    achieved = dom_bytes / (kt[dom] * 1e-3) / 1e9
    res = {
        "metric": "gated-delta scan tokens/s + TFLOP/s (% MFMA peak) at 480p latent, 1 MI355X",
        "value": tokens / (ms_eager * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_eager, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "frame": fr, "frames": NF, "dk": w.dk,
                   "dv": w.dv, "direction": w.direction, "chunk": args.chunk or 64, "calls_per_step": NF,
                   "state": "carried in place across the calls",
                   "inputs": "seeded synthetic video-latent-shaped (synth.WORKLOADS)"},
        "ms_per_frame_eager": ms_eager / NF,
        "ms_per_frame_graph": ms_graph / NF,
        "tokens_per_s_graph": tokens / (ms_graph * 1e-3),
        "tflops": flops / (ms_eager * 1e-3) / 1e12,
        "kernels_ms_per_frame": {"chunk_prep": prep_ms, "state_chain": chain_ms},
        "roofline": {"kernel": dom_name, "bound": "hbm", "achieved": achieved, "peak": MI355X_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / MI355X_HBM_GBS, "traffic": None,
                     "alg_bytes_per_launch": dom_bytes, "workspace_bytes_per_launch": nws,
                     "avg_launch_ms": kt[dom], "source_hash": kernel_source_hash(dom_name)},
    }
    if not args.no_parity:
        res["parity"] = sampled_parity(w, x, out, state, w.direction, threads=host_cores()[0])
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
        res["gpu_over_cpu"] = res["value"] / res["cpu_baseline"]["value"]
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
