#!/usr/bin/env python3
"""Benchmark of the GDN layer hot path on one MI355X.

Headline step: one call of gdn_prefill_chunked over the long-context prefill
workload (B=1, T=65536 tokens, 16 key / 48 value heads, d_k = d_v = 128,
chunk 64, bf16 inputs, fp32 recurrent state, fp32 y), starting from the zero
initial state: conv + SiLU + L2 norm, the chunk-local prep, the conv history
roll and the state pass with the fused sigmoid gate.  The step includes
putting the zero initial state back (a 3 MB device copy), so every timed call
does the same work.  Inputs are synthetic (gdn_inputs, seed 4) and resident
in HBM before the timed region.

The same run reports, each as its own leg: the same workload at chunk 128,
the T=4096 prefill workload, single-token decode at B=1 and B=64 (captured
HIP graphs, each step on a different state set, rotated so that the states
do not stay in the 256 MB Infinity Cache), cold-cache repetitions of every
prefill leg (a 512 MiB device write between repetitions), and the fp64 CPU
oracle on the host's cores.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s + decode steps/s (1 GPU), % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
ROTATE_BYTES = 512 << 20   # rotated state sets per decode timing
COLD_BYTES = 512 << 20     # device write between cold repetitions
CSRC = os.path.join(ROOT, "gated_deltanet_layer_gdn_amd", "csrc")

# HBM bytes per call from rocprofv3 FETCH_SIZE and WRITE_SIZE runs (one
# counter per run), scaled by what the same counters read on a 1 GiB device
# copy (reads x2, writes x1; the summaries under profiles/ give the commands
# and the raw figures).  Each leg's figures hold for the sources of its
# kernels, whose combined SHA-256 is recorded with them; after any change to
# those sources the bench reports the leg's traffic as null until the
# counters are taken again.
LEG_SOURCES = {
    "long64": ("conv.hip", "prep.hip", "prefill.hip", "gdn_device.h", "gdn_internal.h"),
    "long128": ("conv.hip", "prep.hip", "prefill.hip", "gdn_device.h", "gdn_internal.h"),
    "t4096": ("conv.hip", "prep.hip", "prefill.hip", "gdn_device.h", "gdn_internal.h"),
    "decode_b1": ("conv.hip", "decode.hip", "gdn_device.h", "gdn_internal.h"),
    "decode_b64": ("conv.hip", "decode.hip", "gdn_device.h", "gdn_internal.h"),
    "mtp_verify": ("conv.hip", "decode.hip", "gdn_device.h", "gdn_internal.h"),
    "varlen_prefill": ("conv.hip", "prep.hip", "prefill.hip", "gdn_device.h", "gdn_internal.h"),
    "gated_rmsnorm": ("epilogue.hip", "gdn_device.h", "gdn_internal.h"),
}
MEASURED_TRAFFIC = {
    # leg -> {"sha256": sources' hash, "read": bytes, "write": bytes}; from
    # profiles/gdn_hbm_bytes_prefill_t65536_t4096_decode.txt (sums over the leg's kernels)
    "long64": {"sha256": "3718e9a19065089207ea07a56925cd56e2a26b4c536360b82949931fbfb04df4",
               "read": 4321000000, "write": 3263090000},
    "long128": {"sha256": "3718e9a19065089207ea07a56925cd56e2a26b4c536360b82949931fbfb04df4",
               "read": 10215130000, "write": 7288780000},
    "t4096": {"sha256": "3718e9a19065089207ea07a56925cd56e2a26b4c536360b82949931fbfb04df4",
               "read": 325820000, "write": 214160000},
    "decode_b1": {"sha256": "053b9905f7aaf031ee90567d640dc9da83d1e07f35922dee8d64bb7616beeca2",
               "read": 3720000, "write": 3270000},
    "decode_b64": {"sha256": "053b9905f7aaf031ee90567d640dc9da83d1e07f35922dee8d64bb7616beeca2",
               "read": 218480000, "write": 209450000},
    # profiles/gdn_serving_mtp_verify_b64_varlen8_rmsnorm4096.txt (per step or call)
    "mtp_verify": {"sha256": "053b9905f7aaf031ee90567d640dc9da83d1e07f35922dee8d64bb7616beeca2",
                   "read": 244650000, "write": 628410000},
    "varlen_prefill": {"sha256": "3718e9a19065089207ea07a56925cd56e2a26b4c536360b82949931fbfb04df4",
                       "read": 829500000, "write": 568990000},
    "gated_rmsnorm": {"sha256": "7c3dcbf2cd36e667884d09c932cc5ba6cf264706e9f159d0b3bbe60f5c094e02",
                      "read": 151030000, "write": 50330000},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_sha256(names) -> str:
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(leg):
    """Measured HBM bytes per call of a leg (read + write over its kernels),
    or None if its sources changed since the counters were taken."""
    e = MEASURED_TRAFFIC.get(leg)
    if not e or e["sha256"] != sources_sha256(LEG_SOURCES[leg]):
        return None
    return int(e["read"] + e["write"])


def prefill_flops_per_token(H_k, H_v, d_k, d_v, C):
    """Algorithmic flops of the whole chunked prefill per token: per value head
    C^2/3 (the triangular inverse), (C-1)(d_k+d_v) (the triangular products of
    the WY factors), 6 d_k d_v (K S^T, Q S^T and the state update),
    (C+1) d_v (P U and the gate); per key head 2 C d_k (K K^T, Q K^T)."""
    return (H_v * (C * C / 3 + (C - 1) * (d_k + d_v) + 6 * d_k * d_v + (C + 1) * d_v)
            + H_k * (2 * C * d_k))


def prefill_bytes_per_token(C_ch, H_v, d_v, in_bytes, out_bytes):
    """Algorithmic HBM bytes per token of the whole prefill: x and z read
    once, g and beta read once, y written once (the state in and out is
    added per call)."""
    return C_ch * in_bytes + H_v * d_v * in_bytes + 2 * H_v * 4 + H_v * d_v * out_bytes


def state_pass_flops_per_token(H_v, d_k, d_v, C):
    """Algorithmic flops of the state-pass kernel alone per token: K S^T, Q S^T
    and the rank-C state update (2 d_k d_v each) plus (I+A)^{-1} R and P U
    (triangular, C d_v each)."""
    return H_v * (6 * d_k * d_v + 2 * C * d_v)


def state_pass_bytes_per_token(H_v, d_v, in_bytes, out_bytes):
    """Algorithmic HBM bytes per token of the state-pass kernel alone: the v
    channels of x and z, g and beta, y (the state in and out per call)."""
    return H_v * d_v * in_bytes + H_v * d_v * in_bytes + 2 * H_v * 4 + H_v * d_v * out_bytes


def decode_kernel_bytes_per_seq(H_v, d_k, d_v, in_bytes, out_bytes):
    """Algorithmic bytes per sequence of the decode state-stream kernel: the
    fp32 state read and written once, z read, y written, g and beta read."""
    return 2 * H_v * d_v * d_k * 4 + H_v * d_v * (in_bytes + out_bytes) + 2 * H_v * 4


def decode_step_bytes_per_seq(C_ch, H_v, d_k, d_v, in_bytes, out_bytes):
    """Algorithmic bytes per sequence of a whole decode step (conv history in
    and out, x, z, g, beta, state in and out, y)."""
    return (decode_kernel_bytes_per_seq(H_v, d_k, d_v, in_bytes, out_bytes)
            + 2 * 3 * C_ch * in_bytes + C_ch * in_bytes)


def serving_legs(args, gdn, torch, np):
    """The serving shapes and the output epilogue, each against the HBM
    roofline (all HBM-bound):
    * an MTP verify step (gdn_decode_multi): B = 64 sequences, T = 3 tokens,
      the state after every token stored to a slot of its own, graph-replayed
      over rotated slot groups so the state sets exceed the 256 MB Infinity
      Cache; algorithmic bytes per sequence: the fp32 state read once and
      written T times, the conv history likewise, T tokens of x, z, g, beta
      and y;
    * a packed variable-length prefill (gdn_prefill_varlen) of 8 sequences of
      mixed lengths (4096 .. 129 tokens, 10,422 in all) from zero states,
      chunk 64 (up to three sequences side by side): the prefill's algorithmic
      bytes per token plus each sequence's state in and out;
    * the zero-centred grouped RMS norm and gate (gdn_gated_rmsnorm) over the
      ungated readout of 4096 tokens: fp32 o and bf16 z read, bf16 y written.
    Inputs are seeded draws of the layer's laws (x, z ~ N(0, 1) bf16, g =
    -softplus(N(0, 1)), beta = sigmoid(N(0, 1)), conv weights ~ N(0, 0.5^2),
    states ~ N(0, 0.1^2))."""
    H_k, H_v, d = 16, 48, 128
    C_ch = 2 * H_k * d + H_v * d
    st_bytes = H_v * d * d * 4
    hist_bytes = 3 * C_ch * 2
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    nrm = lambda *shape: torch.randn(*shape, device="cuda", generator=gen)
    out = {}

    # MTP verify step
    B, T = 64, 3
    dm = gdn.Dims(B=B, H_k=H_k, H_v=H_v, d_k=d, d_v=d, in_dtype=gdn.BF16, out_dtype=gdn.F32)
    per_group = B * (1 + T)
    R = max(2, math.ceil(ROTATE_BYTES / (B * st_bytes)))
    n_slots = R * per_group
    rec_pool = 0.1 * nrm(n_slots, H_v, d, d)
    conv_pool = nrm(n_slots, 3, C_ch).bfloat16()
    x = nrm(B, T, C_ch).bfloat16()
    z = nrm(B, T, H_v, d).bfloat16()
    g = -torch.nn.functional.softplus(nrm(B, T, H_v))
    beta = torch.sigmoid(nrm(B, T, H_v))
    w = (0.5 * nrm(C_ch, 4)).bfloat16()
    y = torch.empty(B, T, H_v, d, device="cuda")
    ws = torch.empty(T * gdn.decode_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    ins = [torch.arange(r * per_group, r * per_group + B, dtype=torch.int32, device="cuda")
           for r in range(R)]
    outs = [torch.arange(r * per_group + B, (r + 1) * per_group, dtype=torch.int32,
                         device="cuda").reshape(B, T) for r in range(R)]

    def mstep(r):
        gdn.decode_multi(dm, x, z, g, beta, w, conv_pool, rec_pool, ins[r], outs[r], y=y, ws=ws)

    for r in range(R):
        mstep(r)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(R):
            mstep(r)
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.decode_rounds):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (args.decode_rounds * R)
    tok_bytes = C_ch * 2 + H_v * d * 2 + 2 * H_v * 4 + H_v * d * 4
    mb = B * ((1 + T) * (st_bytes + hist_bytes) + T * tok_bytes)
    out["mtp_verify"] = {
        "workload": f"gdn_decode_multi B={B} T={T}, the state after each token to its own slot, "
                    f"16/48 heads d=128, bf16 in, fp32 y; {R} slot groups rotated, one graph",
        "us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(mb / (ms * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(mb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("mtp_verify"),
                     "alg_bytes_per_step": int(mb)}}
    log(f"[bench] mtp verify B={B} T={T}: {ms * 1e3:.1f} us/step = "
        f"{mb / (ms * 1e-3) / 1e9:.0f} GB/s of algorithmic bytes")
    del rec_pool, conv_pool, graph

    # packed variable-length prefill
    lens = [4096, 2048, 1536, 1024, 777, 512, 300, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    Tt = int(cu[-1])
    dv = gdn.Dims(B=len(lens), H_k=H_k, H_v=H_v, d_k=d, d_v=d, in_dtype=gdn.BF16, out_dtype=gdn.F32)
    xv = nrm(Tt, C_ch).bfloat16()
    zv = nrm(Tt, H_v, d).bfloat16()
    gv = -torch.nn.functional.softplus(nrm(Tt, H_v))
    bv = torch.sigmoid(nrm(Tt, H_v))
    rec = torch.zeros(len(lens), H_v, d, d, device="cuda")
    hist = torch.zeros(len(lens), 3, C_ch, device="cuda").bfloat16()
    yv = torch.empty(Tt, H_v, d, device="cuda")
    wsv = torch.empty(gdn.prefill_varlen_workspace_bytes(dv, cu, 64), dtype=torch.uint8, device="cuda")
    slots = list(range(len(lens)))

    def vstep():
        rec.zero_()
        hist.zero_()
        gdn.prefill_varlen(dv, cu, xv, zv, gv, bv, w, hist, rec, slots, chunk=64, y=yv, ws=wsv)

    for _ in range(args.warmup):
        vstep()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        vstep()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    vb = prefill_bytes_per_token(C_ch, H_v, d, 2, 4) * Tt + len(lens) * 2 * st_bytes
    out["varlen_prefill"] = {
        "workload": f"gdn_prefill_varlen of {len(lens)} sequences {lens} ({Tt} tokens), chunk 64, "
                    f"zero initial states (reset inside the timed step), fp32 y",
        "us_per_call": round(ms * 1e3, 1), "tokens_per_s": round(Tt / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(vb / (ms * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(vb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("varlen_prefill"),
                     "alg_bytes_per_call": int(vb)}}
    log(f"[bench] varlen prefill {len(lens)} sequences, {Tt} tokens: {ms * 1e3:.1f} us = "
        f"{Tt / (ms * 1e-3) / 1e6:.2f} M tokens/s")
    del xv, zv, yv, wsv

    # grouped RMS norm + gate over the ungated readout
    Tn = 4096
    dn = gdn.Dims(B=1, H_k=H_k, H_v=H_v, d_k=d, d_v=d, in_dtype=gdn.BF16, out_dtype=gdn.BF16)
    o = nrm(1, Tn, H_v, d)
    zn = nrm(1, Tn, H_v, d).bfloat16()
    nw = 0.1 * nrm(d)
    yn = torch.empty(1, Tn, H_v, d, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        gdn.gated_rmsnorm(dn, o, zn, nw, y=yn)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        gdn.gated_rmsnorm(dn, o, zn, nw, y=yn)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nb = Tn * H_v * d * (4 + 2 + 2) + d * 4
    out["gated_rmsnorm"] = {
        "workload": f"gdn_gated_rmsnorm over {Tn} tokens x 48 heads x 128 (fp32 o, bf16 z and y)",
        "us_per_call": round(ms * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(nb / (ms * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("gated_rmsnorm"),
                     "alg_bytes_per_call": int(nb)}}
    log(f"[bench] gated rmsnorm {Tn} tokens: {ms * 1e3:.2f} us = {nb / (ms * 1e-3) / 1e9:.0f} GB/s")
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def fractions(F, Bytes, t_s):
    mf = F / (t_s * PEAK_BF16_TFLOPS * 1e12)
    hf = Bytes / (t_s * PEAK_HBM_GBS * 1e9)
    return {"mfma": round(mf, 4), "hbm": round(hf, 4), "roofline": round(max(mf, hf), 4)}


def attn_causal_flops(B, T, pos0, H_q, d):
    """Products of causal attention: 2 d flops per (query, visible key) pair
    for q k^T and as many for P v, per query head."""
    pairs = T * pos0 + T * (T + 1) / 2
    return 4.0 * d * H_q * B * pairs


def attn_bytes(B, T, pos0, H_q, H_kv, d, out_bytes):
    """Algorithmic HBM bytes of one attention call: q, k, v in (bf16), the new
    keys and values written to the cache, the whole visible cache read once,
    o out."""
    L = pos0 + T
    return B * (T * (H_q + 2 * H_kv) * d * 2 + T * 2 * H_kv * d * 2 + L * 2 * H_kv * d * 2
                + T * H_q * d * out_bytes)


def hybrid_leg(args, gdn, torch, np, dev, T):
    """The 3 GDN : 1 full-attention block over one T-token prefill (B=1,
    hidden 5120): three times (GDN input projections, then the GDN layer with
    its sigmoid gate, bf16 y) and once (RoPE + KV-cache write + causal GQA
    attention, 24 query / 2 KV heads of 256, bf16 o).  The attention layer's
    q/k/v/o projections, the GDN output projections and the MLPs are plain
    GEMMs outside this path and are not timed."""
    from gdn_inputs import make_attn_inputs, make_inputs, make_proj_inputs, Geometry
    hidden = 5120
    d = gdn.Dims(B=1, H_k=16, H_v=48, d_k=128, d_v=128, in_dtype=gdn.BF16, out_dtype=gdn.BF16)
    geom = Geometry(B=1, T=T, H_k=16, H_v=48, d_k=128, d_v=128)
    layers = []
    for li in range(3):
        P = make_proj_inputs(1, T, hidden, 16, 48, 128, seed=40 + li)
        I = make_inputs(geom, seed=50 + li)
        L = {"h": dev(P["h"]), "w": dev(P["w_in"]), "A": dev(P["A_log"]), "dtb": dev(P["dt_bias"]),
             "cw": dev(I["w"]), "hist": dev(I["hist"]), "S": dev(I["S"])}
        L["out"] = gdn.in_proj(d, L["h"], L["w"], L["A"], L["dtb"])
        L["y"] = torch.empty((1, T, 48, 128), dtype=torch.bfloat16, device="cuda")
        L["ws"] = torch.empty(gdn.prefill_workspace_bytes(d, T, 64), dtype=torch.uint8,
                              device="cuda")
        L["S0"], L["h0"] = L["S"].clone(), L["hist"].clone()
        layers.append(L)
    a = gdn.AttnDims(B=1, H_q=24, H_kv=2, d_h=256, rot_dim=64, rope_base=1e7,
                     out_dtype=gdn.BF16)
    A = {k: dev(v) for k, v in make_attn_inputs(1, T, 0, T, 24, 2, 256, seed=60).items()}
    o = torch.empty((1, T, 24, 256), dtype=torch.bfloat16, device="cuda")
    aws = torch.empty(gdn.attn_workspace_bytes(a, T, 0), dtype=torch.uint8, device="cuda")

    def gdn_layer(L):
        x, z, g, beta = L["out"]
        gdn.in_proj(d, L["h"], L["w"], L["A"], L["dtb"], x, z, g, beta)
        L["S"].copy_(L["S0"])
        L["hist"].copy_(L["h0"])
        gdn.prefill_chunked(d, x, z, g, beta, L["cw"], L["hist"], L["S"], chunk=64, y=L["y"],
                            ws=L["ws"])

    def attn_layer():
        gdn.attn_prefill(a, A["q"], A["k"], A["v"], A["k_cache"], A["v_cache"], pos0=0, o=o,
                         ws=aws)

    def block():
        for L in layers:
            gdn_layer(L)
        attn_layer()

    def timed(fn, reps):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = max(args.steps // 2, 3)
    ms_block = timed(block, reps)
    ms_gdn = timed(lambda: gdn_layer(layers[0]), reps)
    ms_attn = timed(attn_layer, reps)
    # torch's fused attention on the same shapes (KV heads expanded) for context
    qt = A["q"].transpose(1, 2).contiguous()
    kt = A["k"].transpose(1, 2).repeat_interleave(12, 1).contiguous()
    vt = A["v"].transpose(1, 2).repeat_interleave(12, 1).contiguous()
    sdpa = lambda: torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    try:
        ms_sdpa = timed(sdpa, reps)
    except RuntimeError:  # pragma: no cover
        ms_sdpa = None
    # Decode side: one token through the block's token mixing at context T (3
    # GDN decode steps and one attention step at position T over the cached
    # T positions), captured as one graph and replayed.  The projections of a
    # decode step are weight-streaming GEMVs outside this path and are not
    # in it.
    gd = Geometry(B=1, T=1, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=False)
    Id = make_inputs(gd, seed=70)
    dd = gdn.Dims(B=1, H_k=16, H_v=48, d_k=128, d_v=128, in_dtype=gdn.BF16, out_dtype=gdn.BF16)
    dls = []
    for li in range(3):
        Dd = {k: dev(v) for k, v in Id.items()}
        Dd["y"] = torch.empty((1, 48, 128), dtype=torch.bfloat16, device="cuda")
        Dd["ws"] = torch.empty(gdn.decode_workspace_bytes(dd), dtype=torch.uint8, device="cuda")
        dls.append(Dd)
    A1 = {k: dev(v) for k, v in make_attn_inputs(1, 1, T, T + 1, 24, 2, 256, seed=71).items()}
    o1 = torch.empty((1, 1, 24, 256), dtype=torch.bfloat16, device="cuda")
    aws1 = torch.empty(gdn.attn_workspace_bytes(a, 1, T), dtype=torch.uint8, device="cuda")

    def dec_attn():
        gdn.attn_prefill(a, A1["q"], A1["k"], A1["v"], A1["k_cache"], A1["v_cache"], pos0=T,
                         o=o1, ws=aws1)

    def dec_block():
        for Dd in dls:
            gdn.decode_step(dd, Dd["x"].reshape(1, -1), Dd["z"].reshape(1, 48, 128),
                            Dd["g"].reshape(1, 48), Dd["beta"].reshape(1, 48), Dd["w"],
                            Dd["hist"], Dd["S"], y=Dd["y"], ws=Dd["ws"])
        dec_attn()

    def graph_us(fn, reps=50):
        fn()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        gr.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    us_dec_block = graph_us(dec_block)
    us_dec_attn = graph_us(dec_attn)
    Fa = attn_causal_flops(1, T, 0, 24, 256)
    Ba = attn_bytes(1, T, 0, 24, 2, 256, 2)
    res = {
        "workload": f"hybrid block, 3 GDN layers (input projections hidden {hidden} + GDN prefill "
                    f"chunk 64, bf16 y) + 1 attention layer (RoPE rot 64 base 1e7, 24Q/2KV heads "
                    f"of 256, bf16 KV cache and o), B=1 T={T}",
        "tokens_per_s": round(T / (ms_block * 1e-3), 1),
        "us_per_block": round(ms_block * 1e3, 1),
        "us_per_gdn_layer": round(ms_gdn * 1e3, 1),
        "us_attention_layer": round(ms_attn * 1e3, 1),
        "attention": {
            "roofline": {"bound": "mfma", "achieved": round(Fa / ms_attn / 1e9, 1),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(Fa / ms_attn / 1e9 / PEAK_BF16_TFLOPS, 4),
                         "alg_flops_per_call": int(Fa), "alg_bytes_per_call": int(Ba)},
            "torch_sdpa_us": None if ms_sdpa is None else round(ms_sdpa * 1e3, 1),
        },
        "decode": {
            "workload": f"one token at context {T}: 3 GDN decode steps (B=1, bf16 y) + 1 "
                        f"attention step over {T} cached positions, one graph replayed",
            "us_per_token": round(us_dec_block, 2),
            "us_attention_step": round(us_dec_attn, 2),
            "attention_kv_bytes": int(2 * T * 2 * 256 * 2),
        },
    }
    log(f"[bench] hybrid block T={T}: {ms_block * 1e3:.0f} us ({T / ms_block * 1e-3:.2f} M tokens/s); "
        f"GDN layer {ms_gdn * 1e3:.0f} us, attention {ms_attn * 1e3:.0f} us = "
        f"{Fa / ms_attn / 1e9:.0f} TFLOP/s (torch sdpa {res['attention']['torch_sdpa_us']} us); "
        f"decode token {us_dec_block:.1f} us (attention step {us_dec_attn:.1f} us)")
    del layers, A, o, aws, qt, kt, vt, dls, A1
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=64, help="chunk size of the headline leg")
    ap.add_argument("--cold-reps", type=int, default=10)
    ap.add_argument("--decode-rounds", type=int, default=5,
                    help="graph replays per decode timing (each replays R rotated steps)")
    ap.add_argument("--legs", default="all",
                    help="comma list of: long64, long128, t4096, decode_b1, decode_b64, in_proj, "
                         "hybrid, serving, cpu (default all); the headline leg always runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run --steps plain device copies of MIB MiB (for scaling the HBM "
                         "byte counters of rocprofv3 against a kernel of known traffic)")
    ap.add_argument("--decode-graph-only", type=int, default=0, metavar="ROUNDS",
                    help="only replay the captured B=1 decode graph ROUNDS times (for a kernel "
                         "trace of the graph replay alone, without eager or timed launches)")
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

    if args.decode_graph_only:
        # The B=1 decode step as a captured graph of R steps on rotated state
        # sets, replayed; no other launch reaches the GPU after the capture.
        wl_d, Id = workload_inputs(1)
        Gd = wl_d.geom
        dd = gdn.Dims(B=1, H_k=Gd.H_k, H_v=Gd.H_v, d_k=Gd.d_k, d_v=Gd.d_v, in_dtype=gdn.BF16,
                      out_dtype=gdn.F32)
        R = max(2, math.ceil(ROTATE_BYTES / Id["S"].nbytes))
        Dd = {k: dev(v) for k, v in Id.items()}
        Ss = [Dd["S"].clone() for _ in range(R)]
        Hs = [Dd["hist"].clone() for _ in range(R)]
        yd = torch.empty((1, Gd.H_v, Gd.d_v), dtype=torch.float32, device="cuda")
        wsd = torch.empty(gdn.decode_workspace_bytes(dd), dtype=torch.uint8, device="cuda")
        args_d = (Dd["x"].reshape(1, Gd.C_ch), Dd["z"].reshape(1, Gd.H_v, Gd.d_v),
                  Dd["g"].reshape(1, Gd.H_v), Dd["beta"].reshape(1, Gd.H_v), Dd["w"])
        for r in range(R):
            gdn.decode_step(dd, *args_d, Hs[r], Ss[r], y=yd, ws=wsd)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for r in range(R):
                gdn.decode_step(dd, *args_d, Hs[r], Ss[r], y=yd, ws=wsd)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.decode_graph_only):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (args.decode_graph_only * R)
        print(json.dumps({"decode_graph_us_per_step": round(us, 3), "steps_per_graph": R,
                          "replays": args.decode_graph_only}), flush=True)
        return

    legs = set(args.legs.split(",")) if args.legs != "all" else {
        "long64", "long128", "t4096", "decode_b1", "decode_b64", "in_proj", "hybrid", "serving",
        "cpu"}
    if args.no_cpu_baseline:
        legs.discard("cpu")
    head_leg = "long64" if args.chunk == 64 else "long128"
    if args.chunk not in (64, 128):
        raise SystemExit("--chunk must be 64 or 128 (the long-context workload's chunk sizes)")
    legs.add(head_leg)

    cold_buf = torch.empty(COLD_BYTES // 4, dtype=torch.float32, device="cuda")

    def prefill_leg(wl, I, C, steps, warmup):
        """Warm back-to-back steps (the contract's K timed steps), per-kernel
        durations from the library's HIP events, and cold repetitions."""
        G = wl.geom
        d = gdn.Dims(B=G.B, H_k=G.H_k, H_v=G.H_v, d_k=G.d_k, d_v=G.d_v, W=G.W,
                     in_dtype=gdn.BF16, out_dtype=gdn.F32)
        D = {k: dev(v) for k, v in I.items()}
        S0, h0 = D["S"].clone(), D["hist"].clone()
        y = torch.empty((G.B, G.T, G.H_v, G.d_v), dtype=torch.float32, device="cuda")
        ws = torch.empty(gdn.prefill_workspace_bytes(d, G.T, C), dtype=torch.uint8, device="cuda")
        log(f"[bench] prefill {wl.name}, chunk {C}, workspace {ws.numel() / 2**20:.1f} MiB")

        def step(kernel_ms=None):
            D["S"].copy_(S0)
            D["hist"].copy_(h0)
            gdn.prefill_chunked(d, D["x"], D["z"], D["g"], D["beta"], D["w"], D["hist"], D["S"],
                                chunk=C, y=y, ws=ws, kernel_ms=kernel_ms)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        names = ["conv", "prep", "state"]
        per = {n: [] for n in names}
        for _ in range(max(steps, 5)):
            km = []
            step(kernel_ms=km)
            for n, v in zip(names, km):
                per[n].append(v)
        kern = {n: float(np.mean(v)) for n, v in per.items()}
        cold = []
        for r in range(args.cold_reps):
            D["S"].copy_(S0)
            D["hist"].copy_(h0)
            cold_buf.fill_(float(r))
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record()
            gdn.prefill_chunked(d, D["x"], D["z"], D["g"], D["beta"], D["w"], D["hist"], D["S"],
                                chunk=C, y=y, ws=ws)
            c1.record()
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1))
        ntok = G.B * G.T
        F = prefill_flops_per_token(G.H_k, G.H_v, G.d_k, G.d_v, C) * ntok
        state_bytes = G.B * G.H_v * G.d_v * G.d_k * 4
        Bytes = prefill_bytes_per_token(G.C_ch, G.H_v, G.d_v, 2, 4) * ntok + 2 * state_bytes
        t_kern = sum(kern.values()) * 1e-3
        ach = Bytes / t_kern / 1e9
        F_st = state_pass_flops_per_token(G.H_v, G.d_k, G.d_v, C) * ntok
        B_st = state_pass_bytes_per_token(G.H_v, G.d_v, 2, 4) * ntok + 2 * state_bytes
        t_st = kern["state"] * 1e-3
        res = {
            "workload": f"GDN prefill B={G.B} T={G.T} H_k={G.H_k} H_v={G.H_v} d_k=d_v={G.d_k} "
                        f"chunk={C}, bf16 in, fp32 state, fp32 y, zero initial state",
            "tokens_per_s": round(ntok / (ms * 1e-3), 1),
            "us_per_step": round(ms * 1e3, 2),
            "cold": {"reps": len(cold), "median_us": round(float(np.median(cold)) * 1e3, 2),
                     "min_us": round(float(np.min(cold)) * 1e3, 2),
                     "tokens_per_s_median": round(ntok / (float(np.median(cold)) * 1e-3), 1),
                     "protocol": f"{COLD_BYTES >> 20} MiB device write before each call"},
            "kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
            "step_fractions": fractions(F, Bytes, ms * 1e-3),
            "roofline": {
                "bound": "hbm" if Bytes * PEAK_BF16_TFLOPS * 1e12 > F * PEAK_HBM_GBS * 1e9
                else "mfma",
                "kernel": ("gdn_prefill_chunked: prep_kernel (with the q/k conv at this size) + state_kernel_ws"
                           if -(-G.T // C) * G.H_k * G.B > 4096 else
                           "gdn_prefill_chunked: conv_qk_kernel + prep_kernel + state_kernel_ws")
                          if C == 64 else
                          "gdn_prefill_chunked: conv_kernel + prep_kernel + state_kernel",
                "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": None,
                "alg_bytes_per_call": int(Bytes), "alg_flops_per_call": int(F),
                "arithmetic_intensity": round(F / Bytes, 1),
                "mfma_frac": round(F / t_kern / (PEAK_BF16_TFLOPS * 1e12), 4),
                "avg_call_us": round(t_kern * 1e6, 2),
            },
            "state_pass": {
                "kernel": "state_kernel_ws" if C == 64 else "state_kernel",
                "alg_bytes": int(B_st), "alg_flops": int(F_st),
                "hbm_frac": round(B_st / t_st / (PEAK_HBM_GBS * 1e9), 4),
                "mfma_frac": round(F_st / t_st / (PEAK_BF16_TFLOPS * 1e12), 4),
                "avg_launch_us": round(kern["state"] * 1e3, 2),
            },
        }
        log(f"[bench] prefill T={G.T} C={C}: {ms * 1e3:.1f} us/step warm, cold median "
            f"{res['cold']['median_us']:.1f} us; kernels (us) " +
            ", ".join(f"{n} {v * 1e3:.1f}" for n, v in kern.items()) +
            f"; whole-call {ach:.0f} GB/s = {ach / PEAK_HBM_GBS:.3f} of HBM peak")
        del D, y, ws, S0, h0
        torch.cuda.empty_cache()
        return res

    out_legs = {}
    wl4 = I4 = None
    if legs & {"long64", "long128", "cpu"}:
        t = time.perf_counter()
        wl4, I4 = workload_inputs(4)
        log(f"[bench] long-context inputs drawn in {time.perf_counter() - t:.1f} s")
    for leg, C in (("long64", 64), ("long128", 128)):
        if leg in legs:
            out_legs[leg] = prefill_leg(wl4, I4, C, args.steps, args.warmup)
    if "t4096" in legs:
        wl2, I2 = workload_inputs(2)
        out_legs["t4096"] = prefill_leg(wl2, I2, 64, args.steps, args.warmup)
        del I2
    for leg, res in out_legs.items():
        res["roofline"]["traffic"] = measured_traffic(leg)

    # ------------------------------------------------------------ decode
    decode = {}
    copy_gbs = None
    if legs & {"decode_b1", "decode_b64"}:
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
        if "decode_" + key not in legs:
            continue
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

        def dstep(r, kernel_ms=None):
            gdn.decode_step(dd, x1, z1, g1, b1, Dd["w"], Hs[r], Ss[r], y=yd, ws=wsd,
                            kernel_ms=kernel_ms)

        for r in range(R):  # warm-up, and the graph's first capture is clean
            dstep(r)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for r in range(R):
                dstep(r)
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
        e0.record()
        for r in range(R):
            dstep(r)
        e1.record()
        torch.cuda.synchronize()
        ms_eager = e0.elapsed_time(e1) / R
        kms = []
        for i in range(max(4 * R, 12)):
            km = []
            dstep(i % R, kernel_ms=km)
            kms.append(km)
        kmean = [float(np.mean([k[j] for k in kms])) for j in range(len(kms[0]))]
        k_state = kmean[-1]
        sb = decode_step_bytes_per_seq(Gd.C_ch, Gd.H_v, Gd.d_k, Gd.d_v, 2, 4) * Gd.B
        kb = decode_kernel_bytes_per_seq(Gd.H_v, Gd.d_k, Gd.d_v, 2, 4) * Gd.B
        ach = kb / (k_state * 1e-3) / 1e9
        decode[key] = {
            "workload": wl_d.name, "steps_per_s": round(1e3 / ms_dec, 1),
            "seq_steps_per_s": round(Gd.B * 1e3 / ms_dec, 1), "us_per_step": round(ms_dec * 1e3, 3),
            "us_per_step_eager": round(ms_eager * 1e3, 3), "rotated_state_sets": R,
            "step_hbm_frac": round(sb / (ms_dec * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
            "step_alg_bytes": int(sb),
            "kernels_us": {"conv_step": round(kmean[0] * 1e3, 3),
                           "state": round(kmean[1] * 1e3, 3)},
            "roofline": {"bound": "hbm", "kernel": "decode_kernel (state stream + gate)",
                         "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode_" + key),
                         "alg_bytes_per_launch": int(kb),
                         "attainable_copy_GBs": round(copy_gbs, 1),
                         "frac_of_copy": round(ach / copy_gbs, 4)},
        }
        log(f"[bench] decode {key}: {ms_dec * 1e3:.2f} us/step (graph), {ms_eager * 1e3:.2f} "
            f"eager; state kernel {k_state * 1e3:.2f} us = {ach:.0f} GB/s")
        del Ss, Hs, Dd

    # ------------------------------------------------------------ input projections
    proj = None
    if "in_proj" in legs:
        # The GDN input projections (one fused bf16 GEMM, hidden 5120 -> C_ch +
        # H_v d_v + 2 H_v = 16,480 outputs, with the decay/beta epilogue) over
        # the T=4096 prefill's tokens.  A torch bf16 matmul of the same shape
        # is timed beside it as the attainable-GEMM reference of this GPU.
        from gdn_inputs import make_proj_inputs
        Tp, hidden = 4096, 5120
        dp = gdn.Dims(B=1, H_k=16, H_v=48, d_k=128, d_v=128)
        P = make_proj_inputs(1, Tp, hidden, 16, 48, 128, seed=5)
        hP, wP = dev(P["h"]), dev(P["w_in"])
        AP, dP = dev(P["A_log"]), dev(P["dt_bias"])
        outs = gdn.in_proj(dp, hP, wP, AP, dP)
        for _ in range(args.warmup):
            gdn.in_proj(dp, hP, wP, AP, dP, *outs)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            gdn.in_proj(dp, hP, wP, AP, dP, *outs)
        e1.record()
        torch.cuda.synchronize()
        ms_p = e0.elapsed_time(e1) / args.steps
        Np = dp.C_ch + dp.H_v * dp.d_v + 2 * dp.H_v
        Fp = 2.0 * Tp * Np * hidden
        h2 = hP.reshape(Tp, hidden)
        for _ in range(3):
            r_ = h2 @ wP.t()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            r_ = h2 @ wP.t()
        e1.record()
        torch.cuda.synchronize()
        ms_t = e0.elapsed_time(e1) / args.steps
        del r_
        proj = {"workload": f"input projections, {Tp} tokens, hidden {hidden} -> {Np} outputs "
                            f"(x, z, beta, log decay), bf16 in/out, fp32 accumulation",
                "us_per_call": round(ms_p * 1e3, 1),
                "roofline": {"bound": "mfma", "achieved": round(Fp / ms_p / 1e9, 1),
                             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(Fp / ms_p / 1e9 / PEAK_BF16_TFLOPS, 4),
                             "alg_flops_per_call": int(Fp)},
                "attainable_gemm_TFLOPs": round(Fp / ms_t / 1e9, 1)}
        log(f"[bench] in_proj: {ms_p * 1e3:.1f} us = {Fp / ms_p / 1e9:.0f} TFLOP/s; torch matmul of "
            f"the same shape {Fp / ms_t / 1e9:.0f} TFLOP/s")
        del hP, wP, outs

    # ------------------------------------------------------------ serving shapes, epilogue
    serving = serving_legs(args, gdn, torch, np) if "serving" in legs else None

    # ------------------------------------------------------------ hybrid 3:1 block
    hybrid = None
    if "hybrid" in legs:
        # 2048 tokens: within the dense-attention budget of the pages' text
        # core; 4096: dense attention past it (an upper bound of its cost)
        hybrid = {f"T{T}": hybrid_leg(args, gdn, torch, np, dev, T) for T in (2048, 4096)}

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if "cpu" in legs:
        import oracle
        G4 = wl4.geom
        nth = oracle.default_threads()
        try:
            host_cpus = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            host_cpus = os.cpu_count()

        def run(T_s, heads, nthreads):
            sl = {k: np.ascontiguousarray(I4[k][:, :T_s]) for k in ("x", "z", "g", "beta")}
            t = time.perf_counter()
            oracle.layer(sl["x"], sl["z"], sl["g"], sl["beta"], I4["w"], I4["hist"], I4["S"],
                         H_k=G4.H_k, H_v=G4.H_v, d_k=G4.d_k, d_v=G4.d_v, eps=1e-6,
                         heads=heads, nthreads=nthreads)
            return time.perf_counter() - t

        # The whole long-context workload twice (about 10 s on 16 threads), and
        # a one-thread sample.
        T_mt = G4.T
        dts = [run(T_mt, None, nth) for _ in range(2)]
        dt = float(np.median(dts))
        T_1, h_1 = 4096, 8
        dt1 = run(T_1, [(0, h) for h in range(h_1)], 1)
        rate1 = T_1 * h_1 / G4.H_v / dt1
        cpu = {"value": round(T_mt / dt, 1), "unit": "tokens/s", "cores": nth, "kind": "oracle",
               "sample": f"the whole long-context workload ({T_mt} tokens, all {G4.H_v} value "
                         f"heads) through the fp64 oracle, twice: {dts[0]:.2f} and {dts[1]:.2f} s "
                         f"wall on {nth} threads",
               "cpu_model": cpu_model(), "host_cpus": host_cpus,
               "one_thread_tokens_per_s": round(rate1, 1),
               "one_thread_sample": f"{T_1} tokens x {h_1} of {G4.H_v} value heads on 1 thread "
                                    f"({dt1:.2f} s), scaled to whole-layer tokens"}
        log(f"[bench] cpu oracle: {cpu['value']:.1f} tokens/s on {nth} threads, "
            f"{rate1:.1f} on 1 thread ({cpu['cpu_model']})")

    H = out_legs[head_leg]
    G4 = wl4.geom
    out = {
        "metric": METRIC, "value": H["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(H["us_per_step"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "precision": "bf16 MFMA (fp32 accumulation) on split operands x = hi + lo: hi bf16, lo "
                     "bf16 or, for q, k and P on the d=128 chunk-64 path, scaled e4m3 bytes "
                     "(about 13 significant bits in all); (I+A)^-1 plain bf16; fp32 state, "
                     "fp32 y",
        "data": "synthetic",
        "config": {"workload": H["workload"], "B": G4.B, "T": G4.T, "H_k": G4.H_k,
                   "H_v": G4.H_v, "d_k": G4.d_k, "d_v": G4.d_v, "chunk": args.chunk},
        "roofline": H["roofline"],
        "step_fractions": H["step_fractions"],
        "prefill": out_legs,
        "decode": decode,
        "in_proj": proj,
        "serving": serving,
        "hybrid_block": hybrid,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
