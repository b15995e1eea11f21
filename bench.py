#!/usr/bin/env python3
"""Benchmark of the GDN layer hot path on one MI355X.

One step = one call of gdn_prefill_chunked over the prefill workload
(B=1, T=4096 tokens, 16 key / 48 value heads, d_k = d_v = 128, chunk 64,
bf16 inputs, fp32 recurrent state, fp32 y): conv + SiLU + L2 norm, the
chunk-local prep, the conv history roll and the state pass with the fused
sigmoid gate.  Inputs are synthetic (gdn_inputs, seed 2) and resident in HBM
before the timed region.  The same run also times single-token decode at
B=1 and B=64 (each step on a different state set, rotated so the states do
not stay in the 256 MB Infinity Cache) and the fp64 CPU oracle on the host.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s + decode steps/s (1 GPU), % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
ROTATE_BYTES = 512 << 20   # rotated state sets per decode timing

# HBM bytes per launch of the roofline kernels, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs scaled by the same counters on a 1 GiB device copy (the
# summaries under profiles/ give the commands and figures).  Each entry holds
# for the kernel source with the given SHA-256 only; after any change to that
# file the bench reports the traffic as null until the counters are taken again.
MEASURED_TRAFFIC = {
    "prefill_state": {"source": "gated_deltanet_layer_gdn_amd/csrc/prefill.hip",
        "sha256": "4278b816ea36e932c8d53f44403afc5035bc16db3a9146f2d24a512898987fe7",
        "read_bytes": 220512960, "write_bytes": 103845888},
    "decode_b64": {"source": "gated_deltanet_layer_gdn_amd/csrc/decode.hip",
        "sha256": "51950c41a5f5bf594acc405e8e0ba297df929a0dc536f20ede747bc9aa40e674",
        "read_bytes": 213097863, "write_bytes": 202900176},
    "decode_b1": {"source": "gated_deltanet_layer_gdn_amd/csrc/decode.hip",
        "sha256": "51950c41a5f5bf594acc405e8e0ba297df929a0dc536f20ede747bc9aa40e674",
        "read_bytes": 3376042, "write_bytes": 3170304},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(key):
    """Measured HBM bytes per launch (read + write), or None if the kernel
    source changed since the counters were taken."""
    import hashlib
    e = MEASURED_TRAFFIC.get(key)
    if not e or e["sha256"] is None:
        return None
    with open(os.path.join(ROOT, e["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != e["sha256"]:
            return None
    return e["read_bytes"] + e["write_bytes"]


def prefill_flops_per_token(H_k, H_v, d_k, d_v, C):
    """Algorithmic flops of the whole chunked prefill per token (triangular
    products at triangular size, K K^T and Q K^T once per key head)."""
    return (H_v * (C * C / 3 + (C - 1) * (d_k + d_v) + 6 * d_k * d_v + (C + 1) * d_v)
            + H_k * (2 * C * d_k))


def state_pass_flops_per_token(H_v, d_k, d_v, C):
    """Algorithmic flops of the state-pass kernel per token: K S^T, Q S^T and
    the rank-C state update (2 d_k d_v each) plus (I+A)^{-1} R and P U
    (triangular, C d_v each)."""
    return H_v * (6 * d_k * d_v + 2 * C * d_v)


def state_pass_bytes_per_token(H_v, d_v, in_bytes, out_bytes):
    """Algorithmic HBM bytes per token of the state-pass kernel: the v
    channels of x and z read once, g and beta read once, y written once (the
    state in and out is added per launch).  The chunk-local intermediates it
    also reads (q, k, (I+A)^{-1}, P, gate table) are this design's, not the
    method's, and are not counted."""
    return H_v * d_v * in_bytes + H_v * d_v * in_bytes + 2 * H_v * 4 + H_v * d_v * out_bytes


def prefill_bytes_per_token(C_ch, H_v, d_v, in_bytes, out_bytes):
    """Algorithmic HBM bytes per token of a fully fused prefill: x and z read
    once, g and beta read once, y written once."""
    return C_ch * in_bytes + H_v * d_v * in_bytes + 2 * H_v * 4 + H_v * d_v * out_bytes


def decode_kernel_bytes_per_seq(H_v, d_k, d_v, in_bytes, out_bytes):
    """Algorithmic bytes per sequence of the decode state-stream kernel: the
    fp32 state read and written once, z read, y written, g and beta read."""
    return 2 * H_v * d_v * d_k * 4 + H_v * d_v * (in_bytes + out_bytes) + 2 * H_v * 4


def decode_step_bytes_per_seq(C_ch, H_v, d_k, d_v, in_bytes, out_bytes):
    """Algorithmic bytes per sequence of a whole decode step (conv history in
    and out, x, z, g, beta, state in and out, y)."""
    return (decode_kernel_bytes_per_seq(H_v, d_k, d_v, in_bytes, out_bytes)
            + 2 * 3 * C_ch * in_bytes + C_ch * in_bytes)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=64)
    ap.add_argument("--decode-rounds", type=int, default=5,
                    help="graph replays per decode timing (each replays R rotated steps)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run --steps plain device copies of MIB MiB (for scaling the HBM "
                         "byte counters of rocprofv3 against a kernel of known traffic)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus "
              f"{args.gpus}", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_layer_gdn_amd as gdn
    from gated_deltanet_layer_gdn_amd import _lib
    from gdn_inputs import workload_inputs

    if not os.path.exists(_lib.SO_PATH):
        from gated_deltanet_layer_gdn_amd import build as _b
        _b.build()
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "copies": args.steps}), flush=True)
        return

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    # ------------------------------------------------------------ prefill
    wl, I = workload_inputs(2)
    G = wl.geom
    C = args.chunk
    d = gdn.Dims(B=G.B, H_k=G.H_k, H_v=G.H_v, d_k=G.d_k, d_v=G.d_v, W=G.W, in_dtype=gdn.BF16,
                 out_dtype=gdn.F32)
    D = {k: dev(v) for k, v in I.items()}
    y = torch.empty((G.B, G.T, G.H_v, G.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.prefill_workspace_bytes(d, G.T, C), dtype=torch.uint8, device="cuda")
    log(f"[bench] prefill workload: {wl.name}, chunk {C}, workspace {ws.numel() / 2**20:.1f} MiB")

    def prefill(kernel_ms=None):
        gdn.prefill_chunked(d, D["x"], D["z"], D["g"], D["beta"], D["w"], D["hist"], D["S"],
                            chunk=C, y=y, ws=ws, kernel_ms=kernel_ms)

    for _ in range(args.warmup):
        prefill()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        prefill()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    tok_s = G.B * G.T / (ms_step * 1e-3)
    log(f"[bench] prefill: {ms_step * 1e3:.1f} us/step, {tok_s:.4g} tokens/s")

    names = ["conv", "prep", "state"]
    per = {n: [] for n in names}
    for _ in range(args.steps):
        km = []
        prefill(kernel_ms=km)
        for n, v in zip(names, km):
            per[n].append(v)
    kern_ms = {n: float(np.mean(v)) for n, v in per.items()}
    log("[bench] prefill kernels (us): " + ", ".join(f"{n} {v * 1e3:.1f}" for n, v in kern_ms.items()))

    F_step = prefill_flops_per_token(G.H_k, G.H_v, G.d_k, G.d_v, C) * G.B * G.T
    B_step = prefill_bytes_per_token(G.C_ch, G.H_v, G.d_v, 2, 4) * G.B * G.T + 2 * (
        G.B * G.H_v * G.d_v * G.d_k * 4)
    t_s = ms_step * 1e-3
    step_frac = {
        "mfma": F_step / (t_s * PEAK_BF16_TFLOPS * 1e12),
        "hbm": B_step / (t_s * PEAK_HBM_GBS * 1e9),
    }
    step_frac["roofline"] = max(step_frac["mfma"], step_frac["hbm"])
    # Dominant kernel: the state pass.  Its binding roofline is the larger of
    # its MFMA time and its HBM time at the published peaks; with an
    # arithmetic intensity below the ridge (2500 TFLOP/s / 8 TB/s = 312.5
    # flop/B) that is HBM.
    F_state = state_pass_flops_per_token(G.H_v, G.d_k, G.d_v, C) * G.B * G.T
    B_state = state_pass_bytes_per_token(G.H_v, G.d_v, 2, 4) * G.B * G.T + 2 * (
        G.B * G.H_v * G.d_v * G.d_k * 4)
    t_state = kern_ms["state"] * 1e-3
    mfma_frac = F_state / (t_state * PEAK_BF16_TFLOPS * 1e12)
    hbm_frac = B_state / (t_state * PEAK_HBM_GBS * 1e9)
    if hbm_frac >= mfma_frac:
        achieved = B_state / t_state / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = F_state / t_state / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    roofline.update({"traffic": measured_traffic("prefill_state"),
                     "kernel": "state_kernel_ws (state pass + gate)",
                     "bytes_per_launch": B_state, "flops_per_launch": F_state,
                     "arithmetic_intensity": round(F_state / B_state, 1),
                     "mfma_frac": round(mfma_frac, 4), "hbm_frac": round(hbm_frac, 4),
                     "avg_launch_us": round(kern_ms["state"] * 1e3, 2)})

    # ------------------------------------------------------------ decode
    decode = {}
    copy_gbs = None
    if not args.no_decode:
        # Attainable streaming rate on this GPU: a 1 GiB device-to-device copy.
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * (1 << 30) / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9
        del src, dst
        log(f"[bench] device copy 1 GiB: {copy_gbs:.0f} GB/s (read + write)")
        for idx, key in ((1, "b1"), (3, "b64")):
            wl_d, Id = workload_inputs(idx)
            Gd = wl_d.geom
            dd = gdn.Dims(B=Gd.B, H_k=Gd.H_k, H_v=Gd.H_v, d_k=Gd.d_k, d_v=Gd.d_v, W=Gd.W,
                          in_dtype=gdn.BF16, out_dtype=gdn.F32)
            state_bytes = Id["S"].nbytes
            R = max(2, math.ceil(ROTATE_BYTES / state_bytes))
            Dd = {k: dev(v) for k, v in Id.items()}
            Ss = [Dd["S"].clone() for _ in range(R)]
            Hs = [Dd["hist"].clone() for _ in range(R)]
            yd = torch.empty((Gd.B, Gd.H_v, Gd.d_v), dtype=torch.float32, device="cuda")
            wsd = torch.empty(gdn.decode_workspace_bytes(dd), dtype=torch.uint8, device="cuda")
            x1 = Dd["x"].reshape(Gd.B, Gd.C_ch)
            z1 = Dd["z"].reshape(Gd.B, Gd.H_v, Gd.d_v)
            g1 = Dd["g"].reshape(Gd.B, Gd.H_v)
            b1 = Dd["beta"].reshape(Gd.B, Gd.H_v)

            def step(r, kernel_ms=None):
                gdn.decode_step(dd, x1, z1, g1, b1, Dd["w"], Hs[r], Ss[r], y=yd, ws=wsd,
                                kernel_ms=kernel_ms)

            for r in range(R):  # warm-up, and the graph's first capture is clean
                step(r)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for r in range(R):
                    step(r)
            graph.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.decode_rounds):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ms_dec = e0.elapsed_time(e1) / (args.decode_rounds * R)
            # eager (one Python call per step) for reference
            e0.record()
            for r in range(R):
                step(r)
            e1.record()
            torch.cuda.synchronize()
            ms_eager = e0.elapsed_time(e1) / R
            kms = {"conv": [], "state": []}
            for i in range(max(4 * R, 12)):
                km = []
                step(i % R, kernel_ms=km)
                kms["conv"].append(km[0])
                kms["state"].append(km[1])
            k_state = float(np.mean(kms["state"]))
            kb = decode_kernel_bytes_per_seq(Gd.H_v, Gd.d_k, Gd.d_v, 2, 4) * Gd.B
            sb = decode_step_bytes_per_seq(Gd.C_ch, Gd.H_v, Gd.d_k, Gd.d_v, 2, 4) * Gd.B
            ach = kb / (k_state * 1e-3) / 1e9
            decode[key] = {
                "workload": wl_d.name, "steps_per_s": round(1e3 / ms_dec, 1),
                "seq_steps_per_s": round(Gd.B * 1e3 / ms_dec, 1), "us_per_step": round(ms_dec * 1e3, 3),
                "us_per_step_eager": round(ms_eager * 1e3, 3), "rotated_state_sets": R,
                "step_hbm_frac": round(sb / (ms_dec * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
                "kernels_us": {"conv": round(float(np.mean(kms["conv"])) * 1e3, 3),
                               "state": round(k_state * 1e3, 3)},
                "roofline": {"bound": "hbm", "kernel": "decode_kernel (state stream + gate)",
                             "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(ach / PEAK_HBM_GBS, 4),
                             "traffic": measured_traffic("decode_" + key),
                             "bytes_per_launch": kb,
                             "attainable_copy_GBs": round(copy_gbs, 1),
                             "frac_of_copy": round(ach / copy_gbs, 4)},
            }
            log(f"[bench] decode {key}: {ms_dec * 1e3:.2f} us/step (graph), {ms_eager * 1e3:.2f} "
                f"eager; state kernel {k_state * 1e3:.2f} us = {ach:.0f} GB/s")
            del Ss, Hs, Dd

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nth = oracle.default_threads()
        passes = 3
        t = time.perf_counter()
        for _ in range(passes):
            oracle.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"], H_k=G.H_k,
                         H_v=G.H_v, d_k=G.d_k, d_v=G.d_v, eps=d.l2_eps, nthreads=nth)
        dt = time.perf_counter() - t
        cpu = {"value": round(passes * G.B * G.T / dt, 1), "unit": "tokens/s", "cores": nth,
               "kind": "oracle",
               "sample": f"the whole prefill workload (B=1, T={G.T}, all {G.H_v} value heads) "
                         f"through the fp64 oracle {passes} times, {dt:.2f} s wall on {nth} "
                         f"threads"}
        log(f"[bench] cpu oracle: {cpu['value']:.1f} tokens/s on {nth} threads ({passes} passes, {dt:.2f} s)")

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "precision": "bf16 MFMA on hi/lo split operands, fp32 accumulation, fp32 state and y",
        "data": "synthetic",
        "config": {"workload": f"GDN prefill B={G.B} T={G.T} H_k={G.H_k} H_v={G.H_v} "
                               f"d_k=d_v={G.d_k} chunk={C}, bf16 in, fp32 state, fp32 y",
                   "B": G.B, "T": G.T, "H_k": G.H_k, "H_v": G.H_v, "d_k": G.d_k, "d_v": G.d_v,
                   "chunk": C},
        "roofline": roofline,
        "step_fractions": {k: round(v, 4) for k, v in step_frac.items()},
        "prefill_kernels_us": {k: round(v * 1e3, 2) for k, v in kern_ms.items()},
        "decode": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
