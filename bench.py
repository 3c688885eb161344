"""Benchmark of the norm-quantize -> packed FP8 GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..5]

A step is one pass of the whole path over one batch: every producer site of
the workload (gated-residual AdaRMS or per-token-table LayerNorm, static FP8
out) followed by its packed sibling GEMM (dequant + bias + column split,
bf16 out). The default workload is the widest configuration: the
per-token-table adaLN FFN site over 2048 tokens at D = 16384 (chunks 3-5)
feeding the merged gate|up GEMM 2048 x 32768 x 16384, whose FP8 matrix-core
bound GEMM is the dominant kernel. ``--workload 2`` is the AdaRMS decoder
step (256 tokens, D = 2048; QKV 2048|256|256 from site 1, gate|up
8192|8192 from site 2), ``--workload 3`` the video-DiT QKV step and
``--workload 4`` the small-M latency band.

Timing. Inputs and packed weights are resident in HBM before the timed
region. Steps are captured into HIP graphs (the per-call host cost of the
Python binding is larger than a step's GPU time) and replayed; the timed
region is bracketed by device synchronisation. Each step reads a different
copy of the weights and activations, rotating through enough copies that the
working set is at least 512 MiB, so the 256 MiB Infinity Cache cannot serve
repeated weight streams (``--warm`` drops the rotation and labels the line:
the cache-served figure). Per-kernel durations come from HIP events around
graph replays of that kernel alone on the launch stream, over a rotation
extended until that table's smallest kernel moves at least 512 MiB of its
own buffers per replay (each added set with its own outputs), so no
per-kernel figure comes from the cache either.

Output: one JSON line on stdout (metric, value, roofline of the dominant
kernel, the CPU oracle's throughput on a bounded sample, per-kernel table).
The plain default run (workload 5) then measures workloads 3, 2, 4 and 1 the
same way and appends their steps, rooflines and per-kernel tables to that
line as ``other_workloads`` (``--no-other-workloads`` leaves them out);
``wall_s_total`` is the whole run's wall time.

``--ffn`` (workloads 2 and 5) appends the FFN tail that follows the gate/up
projection: the gate/up GEMM runs with the GEGLU quantiser as its epilogue
(FP8 codes out instead of the bf16 gate|up output) and the down projection
consumes those codes. The unfused pair (bf16 gate/up GEMM, standalone GEGLU
quantiser) is timed beside it for comparison but is not part of the step.

``--rope`` (workload 2) makes the QKV GEMM feed the attention head directly:
its epilogue splits q | k | v, rotates q and k by adjacent-pair RoPE (the q
and k weight rows pair-interleaved at bind) and writes q and the suffix
rows of the K/V caches; the unfused pair (bf16 QKV GEMM, standalone split +
RoPE + cache kernel) is timed beside it.

``--mxfp4`` (AdaRMS workloads 1, 2, 4) runs the MXFP4 band instead: the
producers emit OCP MX FP4 (dynamic per-32 block scales) and the norm-fed
GEMMs take MXFP4 weights packed at bind; metric and roofline are the same,
with the FP4 matrix-core peak. With ``--ffn`` (workload 2) the MXFP4
gate/up GEMM carries the GEGLU quantiser and the down projection stays in
static FP8; ``--fp4-full`` runs the down projection in MXFP4 as well (the
gate/up GEMM's epilogue quantises the GEGLU to MXFP4 for the MXFP4 down
GEMM; the unfused bf16 gate|up GEMM + GEGLU -> MXFP4 kernel is timed beside
it).
``--oproj`` quantises the attention output to MXFP4 for an MXFP4 O
projection, and ``--rope`` gives the MXFP4 QKV GEMM the split + RoPE +
KV-cache epilogue.

``--tp T`` (workloads 3 and 5) measures one GPU's share of a
tensor-parallel job over T GPUs: the producer over every row (its output is
replicated across the ranks) and the packed GEMM on rank 0's slice of every
sibling (N_i / T output columns, whole heads). The joint weight scale of a
real T-way job is the all-reduced maximum over the ranks, taken once at
bind; the slice here is packed with its own scale, which changes no
kernel's work.

``--oproj`` (workload 2) adds the O projection of a seeded attention output:
the static FP8 quantiser and the packed GEMM. With ``--rope --oproj --ffn``
a step is the whole decoder layer around the attention core.
"""

from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # dense FP8 MFMA (datasheet 5.0 PFLOP/s)
FP4_PEAK_TFLOPS = 10100.0      # dense FP4 MFMA (datasheet 10.1 PFLOP/s)
RIDGE = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
ROTATE_BYTES = 512 << 20
DEFAULT_WORKLOAD = 5
OTHER_WORKLOADS = (3, 2, 4, 1)   # appended to the default line, in this order
TABLE_MEM_BYTES = 16 << 30   # copies the per-kernel table may add
TABLE_MAX_SETS = 256
WARM_REPEATS = 16   # --warm: the one buffer set repeated this often per graph
METRIC = "packed FP8 GEMM TFLOP/s (%MFMA peak) + norm-quant GB/s (%HBM peak)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5])
    p.add_argument("--rows", type=int, default=None,
                   help="override the producer row count (e.g. the small-M sweep)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-other-workloads", action="store_true",
                   help="the default line (workload 5, plain) also measures workloads "
                        "3, 2, 4 and 1 and appends their steps and per-kernel tables as "
                        "`other_workloads`; this leaves them out")
    p.add_argument("--ffn", action="store_true",
                   help="workloads 2 and 5: fuse GEGLU + FP8 into the gate/up "
                        "GEMM and append the down projection")
    p.add_argument("--mxfp4", action="store_true",
                   help="AdaRMS workloads: MXFP4 producers and GEMMs (the FP4 band)")
    p.add_argument("--fp4-full", action="store_true",
                   help="with --mxfp4 --ffn: the down projection in MXFP4 too (GEGLU emits MXFP4)")
    p.add_argument("--oproj", action="store_true",
                   help="workload 2: quantise a seeded attention output and "
                        "run the O projection")
    p.add_argument("--rope", action="store_true",
                   help="workload 2: the QKV GEMM writes RoPE'd q and the KV "
                        "caches through its epilogue")
    p.add_argument("--tp", type=int, default=1,
                   help="workloads 3, 5: time one rank's share of a T-way column-parallel GEMM")
    p.add_argument("--warm", action="store_true",
                   help="one set of buffers, no rotation: repeats may be served from the "
                        "Infinity Cache (a labelled warm figure, not the rotated one)")
    p.add_argument("--kernel-reps", type=int, default=20)
    p.add_argument("--hbm-calibration", action="store_true",
                   help="time a plain device copy of known size (HBM ceiling, "
                        "and the reference for counter-derived traffic)")
    p.add_argument("--prewarm-s", type=float, default=2.0,
                   help="seconds of untimed replays before the warmup steps "
                        "(engine clocks ramp up from idle over ~1 s)")
    # counter passes (run under rocprofv3 --pmc) and their summary
    p.add_argument("--profile-kernel", default=None,
                   help="launch only this kernel of the step (norm1, gemm1, "
                        "norm2, gemm2) --launches times over the rotation sets")
    p.add_argument("--copy-kernel", action="store_true",
                   help="launch a plain device copy of COPY_BYTES --launches "
                        "times (the reference for counter scaling)")
    p.add_argument("--launches", type=int, default=20)
    p.add_argument("--summarize-pmc", nargs=4, default=None,
                   metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                   help="turn four rocprofv3 --pmc output folders (FETCH_SIZE and "
                        "WRITE_SIZE of --profile-kernel, then of --copy-kernel) into "
                        "profiles/traffic_w<workload>_<kernel>.json")
    return p.parse_args()


# ------------------------------------------------------------------ setup

def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


class Step:
    """Device buffers of one rotation set and the launches of one step."""


def build_sets(wid, rows, frt, torch, rope=False, mx=False, tp=1):
    import workloads as wl
    w = wl.WORKLOADS[wid]
    inp = wl.producer_inputs(wid, rows=rows)
    cal = wl.producer_inputs(wid, calib=True, rows=rows)
    D = w.D
    R = inp["rows"]
    dev = {}
    if w.form == "adarms":
        dev["res"] = bf16_dev(inp["residual"])
        dev["x"] = bf16_dev(inp["x"])
        dev["gate"] = bf16_dev(inp["gate"])
        dev["mod"] = bf16_dev(inp["mod"])
        if w.sites == 2:
            dev["x2"] = bf16_dev(inp["x2"])
            dev["mod2"] = bf16_dev(inp["mod2"])
    else:
        dev["x"] = bf16_dev(inp["x"])
        dev["temb"] = bf16_dev(inp["temb"].reshape(R, -1))
        dev["table"] = torch.from_numpy(inp["table"]).cuda()

    # ---- calibration on the GPU: amax of each site's producer output on
    # the calibration batch (the GEMM input), scale = amax / 448
    scales = []
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    if w.form == "adarms":
        cres = bf16_dev(cal["residual"])
        cx = bf16_dev(cal["x"])
        cg = bf16_dev(cal["gate"])
        cm = bf16_dev(cal["mod"])
        rout = torch.empty_like(cres)
        frt.frt_ada_norm_quant_fp8(cres, cm, None, x=cx, gate=cg, eps=wl.EPS,
                                   residual_out=rout, amax_out=amax)
        torch.cuda.synchronize()
        scales.append(np.float32(amax.item()) / np.float32(448.0))
        if w.sites == 2:
            amax.zero_()
            cm2 = bf16_dev(cal["mod2"])
            cx2 = bf16_dev(cal["x2"])
            frt.frt_ada_norm_quant_fp8(rout, cm2, None, x=cx2,
                                       gate=cm[0, 2 * D:3 * D], eps=wl.EPS,
                                       amax_out=amax)
            torch.cuda.synchronize()
            scales.append(np.float32(amax.item()) / np.float32(448.0))
    else:
        frt.frt_ptok_table_norm_quant_fp8(
            bf16_dev(cal["x"]), bf16_dev(cal["temb"].reshape(R, -1)),
            torch.from_numpy(cal["table"]).cuda(), None, cal["shift_idx"],
            cal["scale_idx"], eps=wl.EPS, amax_out=amax)
        torch.cuda.synchronize()
        scales.append(np.float32(amax.item()) / np.float32(448.0))
    act = [torch.tensor([float(s)], dtype=torch.float32, device="cuda") for s in scales]

    # ---- bind: pack every GEMM's siblings on the GPU (timed separately)
    packs = []
    pack_ms = []
    for site in range(len(w.gemms)):
        ww = wl.weights(wid, site)
        if tp > 1:
            ww = wl.tp_shard(ww, tp, 0, wl.TP_UNIT[wid])
        Ws = [bf16_dev(x) for x in ww["W"]]
        if rope and site == 0:
            # q and k rows pair-interleaved before packing (bind time)
            nh, kv, hd = wl.QKV_HEADS[wid]
            for i, heads in ((0, nh), (1, kv)):
                t = torch.empty_like(Ws[i])
                frt.frt_interleave_pairs_bf16(Ws[i], t, heads, hd)
                Ws[i] = t
        bs = [None if b is None else bf16_dev(b) for b in ww["b"]]
        N = sum(ww["splits"])
        bc = torch.empty(N, dtype=torch.bfloat16, device="cuda") if w.bias else None
        if mx:
            W8 = torch.empty(N, D // 2, dtype=torch.uint8, device="cuda")
            wsc = torch.empty(D // 256, N, 8, dtype=torch.uint8, device="cuda")
            pack = lambda: frt.frt_pack_weights_mxfp4(Ws, bs if w.bias else None, W8, wsc, bc)  # noqa: E731
        else:
            W8 = torch.empty(N, D, dtype=torch.uint8, device="cuda")
            wsc = torch.empty(1, dtype=torch.float32, device="cuda")
            pack = lambda: frt.frt_pack_weights_fp8(Ws, bs if w.bias else None, W8, wsc, bc)  # noqa: E731
        # the first call also loads the packer's kernels: time a second one
        pack()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pack()
        e1.record()
        torch.cuda.synchronize()
        pack_ms.append(e0.elapsed_time(e1))
        packs.append({"W8": W8, "ws": wsc, "bias": bc, "splits": list(ww["splits"])})
        del Ws, bs
    return w, dev, act, packs, pack_ms


def build_ffn(w, rows, act, packs, frt, torch, mx=False, full=False):
    """The FFN tail's bind: pack the down projection and calibrate the
    GEGLU output scale on the calibration batch (its producer codes through
    the bf16 gate/up GEMM and the standalone quantiser's amax; with `mx` the
    MXFP4 producers and gate/up GEMM)."""
    import workloads as wl
    H = wl.FFN_HIDDEN[w.cid]
    Wd = bf16_dev(wl.down_weights(w.cid))
    if full:        # MXFP4 down projection: dynamic block scales, no calibration
        Wd4 = torch.empty(w.D, H // 2, dtype=torch.uint8, device="cuda")
        Sd4 = torch.empty(H // 256, w.D, 8, dtype=torch.uint8, device="cuda")
        frt.frt_pack_weights_mxfp4([Wd], None, Wd4, Sd4)
        return {"H": H, "W8": Wd4, "ws": Sd4, "scale": None, "full": True}
    Wd8 = torch.empty(w.D, H, dtype=torch.uint8, device="cuda")
    wsd = torch.empty(1, dtype=torch.float32, device="cuda")
    frt.frt_pack_weights_fp8([Wd], None, Wd8, wsd)
    del Wd
    cal = wl.producer_inputs(w.cid, calib=True, rows=rows)
    x8 = torch.empty(rows, w.D, dtype=torch.uint8, device="cuda")
    H2 = 2 * H
    gu = torch.empty(rows, H2, dtype=torch.bfloat16, device="cuda")
    p = packs[-1]
    if mx:
        D = w.D
        x4 = torch.empty(rows, D // 2, dtype=torch.uint8, device="cuda")
        xs = torch.empty(D // 256, rows, 8, dtype=torch.uint8, device="cuda")
        rout = torch.empty(rows, D, dtype=torch.bfloat16, device="cuda")
        cm = bf16_dev(cal["mod"])
        frt.frt_ada_norm_quant_mxfp4(bf16_dev(cal["residual"]), cm, x4, xs, x=bf16_dev(cal["x"]),
                                     gate=bf16_dev(cal["gate"]), eps=wl.EPS, residual_out=rout)
        frt.frt_ada_norm_quant_mxfp4(rout, bf16_dev(cal["mod2"]), x4, xs, x=bf16_dev(cal["x2"]),
                                     gate=cm[0, 2 * D:3 * D], eps=wl.EPS)
        frt.frt_packed_gemm_mxfp4_split(x4, xs, p["W8"], p["ws"], [gu], [H2])
    elif w.form == "adarms":
        D = w.D
        rout = torch.empty(rows, D, dtype=torch.bfloat16, device="cuda")
        cm = bf16_dev(cal["mod"])
        frt.frt_ada_norm_quant_fp8(bf16_dev(cal["residual"]), cm, None, x=bf16_dev(cal["x"]),
                                   gate=bf16_dev(cal["gate"]), eps=wl.EPS, residual_out=rout)
        frt.frt_ada_norm_quant_fp8(rout, bf16_dev(cal["mod2"]), act[1], x=bf16_dev(cal["x2"]),
                                   gate=cm[0, 2 * D:3 * D], eps=wl.EPS, out_fp8=x8)
    else:
        frt.frt_ptok_table_norm_quant_fp8(
            bf16_dev(cal["x"]), bf16_dev(cal["temb"].reshape(rows, -1)),
            torch.from_numpy(cal["table"]).cuda(), act[0], cal["shift_idx"],
            cal["scale_idx"], eps=wl.EPS, out_fp8=x8)
    if not mx:
        frt.frt_packed_gemm_fp8_split(x8, p["W8"], act[-1], p["ws"], [gu], [H2])
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    frt.frt_geglu_quant_fp8(gu, H, None, amax_out=amax)
    torch.cuda.synchronize()
    s_h = np.float32(amax.item()) / np.float32(448.0)
    return {"H": H, "W8": Wd8, "ws": wsd, "full": False,
            "scale": torch.tensor([float(s_h)], dtype=torch.float32, device="cuda")}


def make_rotation(w, dev, packs, rows, torch, ffn=None, warm=False, n_sets=None, first=0):
    """Copies of activations and weights so one pass over the sets moves at
    least ROTATE_BYTES. Warm: one set, listed WARM_REPEATS times, so that a
    graph still holds many launches (the host's replay calls are slower than
    one short launch). `n_sets` forces the count; `first` > 0 returns only
    sets first .. n_sets - 1 (fresh copies, to extend an existing rotation)."""
    per = sum(t.numel() * t.element_size() for t in dev.values()
              if t.dim() > 1 and t.shape[0] == rows)
    per += sum(p["W8"].numel() for p in packs)
    if ffn is not None:
        per += ffn["W8"].numel()
    n = 1 if warm else max(1, math.ceil(ROTATE_BYTES / max(per, 1)))
    if n_sets is not None:
        n = n_sets
    sets = []
    for i in range(first, n):
        s = {"dev": {}, "packs": []}
        for k, t in dev.items():
            rotate = t.dim() > 1 and t.shape[0] == rows
            s["dev"][k] = t.clone() if (rotate and i > 0) else t
        for p in packs:
            q = dict(p)
            if i > 0:
                q["W8"] = p["W8"].clone()
                if p["ws"].numel() > 1:      # MXFP4 block scales rotate with their codes
                    q["ws"] = p["ws"].clone()
            s["packs"].append(q)
        if ffn is not None:
            s["ffn"] = dict(ffn)
            if i > 0:
                s["ffn"]["W8"] = ffn["W8"].clone()
                if ffn["ws"].numel() > 1:
                    s["ffn"]["ws"] = ffn["ws"].clone()
        sets.append(s)
    if warm:
        sets = sets * WARM_REPEATS
    return sets, per


def make_oproj(w, rows, frt, torch, mx=False):
    """O projection: packed W_o, the attention output and its calibrated
    static scale, the FP8 input and the bf16 output buffers (with `mx`: the
    MXFP4 pack of W_o and the MXFP4 input buffers)."""
    import workloads as wl
    inp, cal = wl.o_proj_inputs(w.cid), wl.o_proj_inputs(w.cid, calib=True)
    Wo = bf16_dev(inp["W_o"])
    if mx:
        Ko = Wo.shape[1]
        W4 = torch.empty(w.D, Ko // 2, dtype=torch.uint8, device="cuda")
        S4 = torch.empty(Ko // 256, w.D, 8, dtype=torch.uint8, device="cuda")
        frt.frt_pack_weights_mxfp4([Wo], None, W4, S4)
        att = bf16_dev(inp["att"])
        return {"W8": W4, "ws": S4, "att": att, "scale": None,
                "o4": (torch.empty(rows, Ko // 2, dtype=torch.uint8, device="cuda"),
                       torch.empty(Ko // 256, rows, 8, dtype=torch.uint8, device="cuda")),
                "out": torch.empty(rows, w.D, dtype=torch.bfloat16, device="cuda")}
    W8 = torch.empty(Wo.shape, dtype=torch.uint8, device="cuda")
    ws = torch.empty(1, dtype=torch.float32, device="cuda")
    frt.frt_pack_weights_fp8([Wo], None, W8, ws)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    frt.frt_quantize_fp8_static(bf16_dev(cal["att"]), None, amax_out=amax)
    torch.cuda.synchronize()
    s = np.float32(amax.item()) / np.float32(448.0)
    att = bf16_dev(inp["att"])
    return {"W8": W8, "ws": ws, "att": att,
            "scale": torch.tensor([float(s)], dtype=torch.float32, device="cuda"),
            "o8": torch.empty(att.shape, dtype=torch.uint8, device="cuda"),
            "out": torch.empty(rows, w.D, dtype=torch.bfloat16, device="cuda")}


def make_rope(w, rows, torch):
    """Rope table, q output and the K/V caches of the attention head."""
    import workloads as wl
    nh, kv, hd = wl.QKV_HEADS[w.cid]
    P = wl.ROPE_PREFIX[w.cid]
    T = P + rows
    return {"nh": nh, "kv": kv, "hd": hd, "P": P, "T": T,
            "table": bf16_dev(wl.rope_table(rows, hd, P)),
            "q": torch.empty(rows, nh, hd, dtype=torch.bfloat16, device="cuda"),
            "kc": torch.zeros(T, kv, hd, dtype=torch.bfloat16, device="cuda"),
            "vc": torch.zeros(T, kv, hd, dtype=torch.bfloat16, device="cuda"),
            "qkv": torch.empty(rows, (nh + 2 * kv) * hd, dtype=torch.bfloat16, device="cuda")}


def make_outputs(w, rows, packs, torch, ffn=None):
    D = w.D
    o = {"x8": [torch.empty(rows, D, dtype=torch.uint8, device="cuda")
                for _ in packs]}
    o["rout"] = torch.empty(rows, D, dtype=torch.bfloat16, device="cuda")
    o["rout2"] = torch.empty(rows, D, dtype=torch.bfloat16, device="cuda")
    o["gemm"] = [[torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
                  for n in p["splits"]] for p in packs]
    if ffn is not None:
        H = ffn["H"]
        o["hid8"] = torch.empty(rows, H, dtype=torch.uint8, device="cuda")
        o["dn"] = torch.empty(rows, D, dtype=torch.bfloat16, device="cuda")
        o["gu"] = torch.empty(rows, 2 * H, dtype=torch.bfloat16, device="cuda")
        o["hid8_unfused"] = torch.empty(rows, H, dtype=torch.uint8, device="cuda")
        if ffn["full"]:
            for k in ("hid4", "hid4_unfused"):
                o[k] = (torch.empty(rows, H // 2, dtype=torch.uint8, device="cuda"),
                        torch.empty(H // 256, rows, 8, dtype=torch.uint8, device="cuda"))
    return o


def step_launches_mx(w, s, outs, rows, frt, eps):
    """The MXFP4 band's step: the AdaRMS producers emit MXFP4, the packed
    GEMMs take MXFP4 operands. With the FFN tail the gate/up GEMM carries
    the GEGLU quantiser (FP8 codes) and the static-FP8 down projection
    follows."""
    d = s["dev"]
    D = w.D
    o4 = outs["x4"]
    L = [("norm1_mx", lambda: frt.frt_ada_norm_quant_mxfp4(
        d["res"], d["mod"], o4[0][0], o4[0][1], x=d["x"], gate=d["gate"], eps=eps,
        residual_out=outs["rout"]))]
    p0 = s["packs"][0]
    L.append(("gemm1_mx", lambda: frt.frt_packed_gemm_mxfp4_split(
        o4[0][0], o4[0][1], p0["W8"], p0["ws"], outs["gemm"][0], p0["splits"], bias_cat=p0["bias"])))
    if len(s["packs"]) > 1:
        p1 = s["packs"][1]
        L.append(("norm2_mx", lambda: frt.frt_ada_norm_quant_mxfp4(
            outs["rout"], d["mod2"], o4[1][0], o4[1][1], x=d["x2"],
            gate=d["mod"][0, 2 * D:3 * D], eps=eps, residual_out=outs["rout2"])))
        L.append(("gemm2_mx", lambda: frt.frt_packed_gemm_mxfp4_split(
            o4[1][0], o4[1][1], p1["W8"], p1["ws"], outs["gemm"][1], p1["splits"],
            bias_cat=p1["bias"])))
        f = s.get("ffn")
        if f is not None and f["full"]:
            h4 = outs["hid4"]
            L[-1] = ("gemm2_mx_geglu4", lambda: frt.frt_packed_gemm_mxfp4_geglu_mxfp4(
                o4[1][0], o4[1][1], p1["W8"], p1["ws"], h4[0], h4[1], bias_cat=p1["bias"]))
            L.append(("gemm_down_mx", lambda: frt.frt_packed_gemm_mxfp4_split(
                h4[0], h4[1], f["W8"], f["ws"], [outs["dn"]], [w.D])))
        elif f is not None:
            L[-1] = ("gemm2_mx_geglu", lambda: frt.frt_packed_gemm_mxfp4_geglu_quant(
                o4[1][0], o4[1][1], p1["W8"], p1["ws"], f["scale"], outs["hid8"],
                bias_cat=p1["bias"]))
            L.append(("gemm_down", lambda: frt.frt_packed_gemm_fp8_split(
                outs["hid8"], f["W8"], f["scale"], f["ws"], [outs["dn"]], [w.D])))
    r = s.get("rope")
    if r is not None:
        L[1] = ("gemm1_mx_rope", lambda: frt.frt_packed_gemm_mxfp4_qkv_rope(
            o4[0][0], o4[0][1], p0["W8"], p0["ws"], r["nh"], r["kv"], r["hd"], r["table"], r["P"],
            r["q"], r["kc"], r["vc"], bias_cat=p0["bias"]))
    o = s.get("oproj")
    if o is not None:
        L.insert(2, ("quant_o_mx", lambda: frt.frt_quantize_mxfp4(o["att"], o["o4"][0], o["o4"][1])))
        L.insert(3, ("gemm_o_mx", lambda: frt.frt_packed_gemm_mxfp4_split(
            o["o4"][0], o["o4"][1], o["W8"], o["ws"], [o["out"]], [w.D])))
    return L


def step_launches(w, s, act, outs, rows, frt, eps):
    """The step's launches for rotation set `s`: list of (kind, callable).
    With the FFN tail the last (gate/up) GEMM becomes the GEGLU-fused one
    and the down projection follows."""
    d = s["dev"]
    D = w.D
    L = []
    if w.form == "adarms":
        L.append(("norm1", lambda: frt.frt_ada_norm_quant_fp8(
            d["res"], d["mod"], act[0], x=d["x"], gate=d["gate"], eps=eps,
            residual_out=outs["rout"], out_fp8=outs["x8"][0])))
    else:
        L.append(("norm1", lambda: frt.frt_ptok_table_norm_quant_fp8(
            d["x"], d["temb"], d["table"], act[0], w.shift_idx, w.scale_idx,
            eps=eps, out_fp8=outs["x8"][0])))
    p0 = s["packs"][0]
    L.append(("gemm1", lambda: frt.frt_packed_gemm_fp8_split(
        outs["x8"][0], p0["W8"], act[0], p0["ws"], outs["gemm"][0],
        p0["splits"], bias_cat=p0["bias"])))
    if len(s["packs"]) > 1:
        p1 = s["packs"][1]
        L.append(("norm2", lambda: frt.frt_ada_norm_quant_fp8(
            outs["rout"], d["mod2"], act[1], x=d["x2"],
            gate=d["mod"][0, 2 * D:3 * D], eps=eps, residual_out=outs["rout2"],
            out_fp8=outs["x8"][1])))
        L.append(("gemm2", lambda: frt.frt_packed_gemm_fp8_split(
            outs["x8"][1], p1["W8"], act[1], p1["ws"], outs["gemm"][1],
            p1["splits"], bias_cat=p1["bias"])))
    o = s.get("oproj")
    if o is not None:
        L.insert(2, ("quant_o", lambda: frt.frt_quantize_fp8_static(
            o["att"], o["scale"], out_fp8=o["o8"])))
        L.insert(3, ("gemm_o", lambda: frt.frt_packed_gemm_fp8_split(
            o["o8"], o["W8"], o["scale"], o["ws"], [o["out"]], [w.D])))
    r = s.get("rope")
    if r is not None:
        L[1] = ("gemm1_rope", lambda: frt.frt_packed_gemm_fp8_qkv_rope(
            outs["x8"][0], p0["W8"], act[0], p0["ws"], r["nh"], r["kv"], r["hd"],
            r["table"], r["P"], r["q"], r["kc"], r["vc"], bias_cat=p0["bias"]))
    f = s.get("ffn")
    if f is not None:
        last, pl = L[-1][0], s["packs"][-1]
        L[-1] = (last + "_geglu", lambda: frt.frt_packed_gemm_fp8_geglu_quant(
            outs["x8"][-1], pl["W8"], act[-1], pl["ws"], f["scale"], outs["hid8"],
            bias_cat=pl["bias"]))
        L.append(("gemm_down", lambda: frt.frt_packed_gemm_fp8_split(
            outs["hid8"], f["W8"], f["scale"], f["ws"], [outs["dn"]], [w.D])))
    return L


def unfused_launches(w, s, act, outs, frt, mx=False):
    """The unfused forms of the fused launches (timed for comparison only):
    the bf16 gate|up GEMM (FP8 or, with `mx`, MXFP4) and the standalone
    GEGLU quantiser; the bf16 QKV GEMM and the standalone split + RoPE +
    cache kernel."""
    L = []
    f = s.get("ffn")
    if f is not None and f["full"]:
        pl = s["packs"][-1]
        H, h4 = f["H"], outs["hid4_unfused"]
        gx4, gxs = outs["x4"][-1]
        L.append(("gateup_bf16_mx", lambda: frt.frt_packed_gemm_mxfp4_split(
            gx4, gxs, pl["W8"], pl["ws"], [outs["gu"]], [2 * H], bias_cat=pl["bias"])))
        L.append(("geglu_mx", lambda: frt.frt_geglu_quant_mxfp4(outs["gu"], H, h4[0], h4[1])))
    elif f is not None:
        pl = s["packs"][-1]
        H = f["H"]
        if mx:
            x4, xs = outs["x4"][-1]
            L.append(("gateup_bf16_mx", lambda: frt.frt_packed_gemm_mxfp4_split(
                x4, xs, pl["W8"], pl["ws"], [outs["gu"]], [2 * H], bias_cat=pl["bias"])))
        else:
            L.append(("gateup_bf16", lambda: frt.frt_packed_gemm_fp8_split(
                outs["x8"][-1], pl["W8"], act[-1], pl["ws"], [outs["gu"]], [2 * H],
                bias_cat=pl["bias"])))
        L.append(("geglu", lambda: frt.frt_geglu_quant_fp8(
            outs["gu"], H, f["scale"], out_fp8=outs["hid8_unfused"])))
    r = s.get("rope")
    if r is not None:
        p0 = s["packs"][0]
        width = (r["nh"] + 2 * r["kv"]) * r["hd"]
        if mx:
            qx4, qxs = outs["x4"][0]
            L.append(("qkv_bf16_mx", lambda: frt.frt_packed_gemm_mxfp4_split(
                qx4, qxs, p0["W8"], p0["ws"], [r["qkv"]], [width], bias_cat=p0["bias"])))
        else:
            L.append(("qkv_bf16", lambda: frt.frt_packed_gemm_fp8_split(
                outs["x8"][0], p0["W8"], act[0], p0["ws"], [r["qkv"]], [width],
                bias_cat=p0["bias"])))
        L.append(("rope_split", lambda: frt.frt_qkv_split_rope_kvcache(
            r["qkv"], r["table"], r["nh"], r["kv"], r["hd"], r["P"], r["q"], r["kc"], r["vc"])))
    return L


def kernel_work(w, kind, rows, packs, ffn=None, rope=None, oproj=None):
    """Algorithmic bytes and FLOPs of one launch."""
    D = w.D
    if oproj is not None and kind in ("quant_o_mx", "gemm_o_mx"):
        Ko = oproj["att"].shape[1]
        if kind == "quant_o_mx":        # bf16 in, codes + scales out
            return rows * Ko * 2 + rows * (Ko // 2 + Ko // 32), 0.0
        return rows * (Ko // 2 + Ko // 32) + D * (Ko // 2 + Ko // 32) + rows * D * 2, 2.0 * rows * D * Ko
    if rope is not None and kind in ("gemm1_mx_rope", "qkv_bf16_mx"):
        N = (rope["nh"] + 2 * rope["kv"]) * rope["hd"]
        out = rows * N * 2 + (rows * rope["hd"] * 2 if kind == "gemm1_mx_rope" else 0)
        return rows * (D // 2 + D // 32) + N * (D // 2 + D // 32) + out, 2.0 * rows * N * D
    if ffn is not None and kind in ("geglu_mx", "gemm_down_mx"):
        H = ffn["H"]
        if kind == "geglu_mx":          # bf16 [M, 2H] in, codes + scales out
            return rows * 2 * H * 2 + rows * (H // 2 + H // 32), 0.0
        return rows * (H // 2 + H // 32) + D * (H // 2 + H // 32) + rows * D * 2, 2.0 * rows * D * H
    if ffn is not None and kind in ("gemm2_mx_geglu", "gemm2_mx_geglu4", "gateup_bf16_mx"):
        H = ffn["H"]
        bias = 2 * H * 2 if packs[-1]["bias"] is not None else 0
        out = {"gemm2_mx_geglu": rows * H, "gemm2_mx_geglu4": rows * (H // 2 + H // 32)}.get(
            kind, rows * 2 * H * 2)
        return (rows * (D // 2 + D // 32) + 2 * H * (D // 2 + D // 32) + out + bias,
                2.0 * rows * 2 * H * D)
    if kind.endswith("_mx"):
        if kind.startswith("norm"):     # res, x, rout bf16; codes D/2; scales D/32
            gate = rows * D * 2 if (w.cid == 4 and kind == "norm1_mx") else D * 2
            return rows * D * 2 * 3 + gate + 3 * D * 2 + rows * (D // 2 + D // 32), 0.0
        p = packs[0 if kind == "gemm1_mx" else 1]
        N = sum(p["splits"])
        b = rows * (D // 2 + D // 32) + N * (D // 2 + D // 32) + rows * N * 2 + \
            (N * 2 if p["bias"] is not None else 0)
        return b, 2.0 * rows * N * D
    if oproj is not None and kind in ("quant_o", "gemm_o"):
        Ko = oproj["att"].shape[1]
        if kind == "quant_o":           # bf16 in, codes out
            return rows * Ko * 3, 0.0
        return rows * Ko + D * Ko + rows * D * 2, 2.0 * rows * D * Ko
    if rope is not None and kind in ("gemm1_rope", "qkv_bf16", "rope_split"):
        N = (rope["nh"] + 2 * rope["kv"]) * rope["hd"]
        table = rows * rope["hd"] * 2
        if kind == "rope_split":        # bf16 qkv in, q + k/v rows out, table
            return rows * N * 2 * 2 + table, 0.0
        out = rows * N * 2 + (table if kind == "gemm1_rope" else 0)
        return rows * D + N * D + out, 2.0 * rows * N * D
    if ffn is not None:
        H = ffn["H"]
        p = packs[-1]
        bias = 2 * H * 2 if p["bias"] is not None else 0
        if kind.endswith("_geglu"):     # x8 + W8 [2H, D] + codes [M, H]
            return rows * D + 2 * H * D + rows * H + bias, 2.0 * rows * 2 * H * D
        if kind == "gemm_down":         # codes + W8 [D, H] + bf16 [M, D]
            return rows * H + D * H + rows * D * 2, 2.0 * rows * D * H
        if kind == "gateup_bf16":
            return rows * D + 2 * H * D + rows * 2 * H * 2 + bias, 2.0 * rows * 2 * H * D
        if kind == "geglu":             # bf16 [M, 2H] in, codes out
            return rows * 2 * H * 2 + rows * H, 0.0
    if kind.startswith("norm"):
        if w.form == "adarms":
            gate = rows * D * 2 if (w.cid == 4 and kind == "norm1") else D * 2
            if kind == "norm2":
                gate = D * 2
            b = rows * D * 2 * 3 + gate + 3 * D * 2 + rows * D   # res, x, rout; codes
        else:
            b = rows * D * 2 + rows * D * 4 + 2 * D * 4 + rows * D
        return b, 0.0
    p = packs[0 if kind == "gemm1" else 1]
    N = sum(p["splits"])
    b = rows * D + N * D + rows * N * 2 + (N * 2 if p["bias"] is not None else 0)
    return b, 2.0 * rows * N * D


# ------------------------------------------------------------------ timing

def tensor_bytes(v):
    """Bytes of the tensors in `v` (a tensor, or nested lists/tuples of them)."""
    if isinstance(v, (list, tuple)):
        return sum(tensor_bytes(x) for x in v)
    return v.numel() * v.element_size()


def capture(fn_list, torch):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fn_list:
            fn()
    return g


def prewarm(g, seconds, torch):
    """Replay `g` until `seconds` of wall time have passed (clock ramp)."""
    t_end = time.perf_counter() + seconds
    n = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()
        n += 8
    return n


def time_graph(g, reps, torch):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def cpu_baseline(w, rows, budget_s=20.0):
    """The oracle as it stands on the host cores: the same step (producers
    and exact GEMMs) on the same seeded inputs, repeated within a budget."""
    import workloads as wl
    from oracle import gemm, pack, producers
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 0) for i in threadpool_info()
                if i.get("user_api") == "blas"]
        cores = max(blas) if blas else len(os.sched_getaffinity(0))
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    # a row sample bounded so that one pass stays within a few seconds
    sample = rows if w.form == "adarms" and rows <= 256 else min(rows, 64)
    inp = wl.producer_inputs(w.cid, rows=sample) if w.cid != 4 else \
        wl.producer_inputs(w.cid, rows=min(sample, 64))
    sample = inp["rows"]
    # the GEMMs run on a sample of output rows of W when the whole packed
    # matrix is too large for the host pass (FLOPs are counted on the sample)
    packed = []
    n_cols = 0
    for site in range(len(w.gemms)):
        ww = wl.weights(w.cid, site)
        tot = sum(ww["splits"])
        frac = min(1.0, 8192.0 / tot) if tot * w.D > (1 << 26) else 1.0
        Ws = [x[:max(1, int(x.shape[0] * frac))] for x in ww["W"]]
        bs = [None if b is None else b[:max(1, int(b.shape[0] * frac))] for b in ww["b"]]
        packed.append(pack.pack_weights(Ws, bs))
        n_cols += sum(x.shape[0] for x in Ws)
    per_row_flops = 2.0 * n_cols * w.D
    s_a = np.float32(0.01)
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or not times:
        t0 = time.perf_counter()
        if w.form == "adarms":
            r = producers.ada_norm_quant_fp8(inp["residual"], inp["x"], inp["gate"],
                                             inp["mod"], s_a, wl.EPS)
            codes = [r["codes"]]
            if w.sites == 2:
                D = w.D
                r2 = producers.ada_norm_quant_fp8(r["residual_out"], inp["x2"],
                                                  inp["mod"][0, 2 * D:3 * D],
                                                  inp["mod2"], s_a, wl.EPS)
                codes.append(r2["codes"])
        else:
            r = producers.ptok_norm_quant_fp8(inp["x"], inp["temb"], inp["table"],
                                              s_a, w.shift_idx, w.scale_idx, wl.EPS)
            codes = [r["codes"]]
        for c, (w8, s_w, bias, splits) in zip(codes, packed):
            gemm.packed_gemm_split(c, w8, s_a, s_w, bias if w.bias else None, splits)
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 and time.perf_counter() > t_end - budget_s / 2:
            break
    t = float(np.median(times))
    flops = per_row_flops * sample
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"workload {w.cid} step on {sample} of {rows} rows and "
                      f"{n_cols} of {sum(sum(g) for g in w.gemms)} GEMM output "
                      f"columns (producers + exact fp64 GEMMs), median of "
                      f"{len(times)} runs, {t:.2f} s each"}


# ------------------------------------------------------- counter traffic

COPY_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")


# the sources a kernel kind is built from: its own file plus the shared
# headers and the ABI layer that fills its arguments
_SHARED_SOURCES = ("frt_api.hip", "frt_device.h", "frt_internal.h")


def _kernel_files(kind):
    csrc = os.path.join(ROOT, "norm_quantize_packed_amd", "csrc")
    every = sorted(n for n in os.listdir(csrc) if n.endswith((".hip", ".h", ".inc")))
    if kind is None:
        return csrc, every
    if kind.startswith("norm"):
        own = {"frt_norm.hip"}
    elif kind.startswith("gemm") or kind.startswith(("gateup", "qkv")):
        own = {"frt_gemm.hip", "frt_gemm_epilogue.inc"}
    else:
        return csrc, every
    return csrc, sorted(set(_SHARED_SOURCES) | own)


def kernel_sources_sha(kind=None):
    """sha256 over the HIP sources a kernel kind is built from (every source
    when `kind` is None): a counter record is used only while the kernel it
    measured is unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc, names = _kernel_files(kind)
    for name in names:
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def copy_kernel(torch, launches):
    """Plain device copies of COPY_BYTES, rotating over 4 buffer pairs
    (2 GiB) so the copies stream from and to HBM."""
    pairs = [(torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1),
              torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")) for _ in range(4)]
    torch.cuda.synchronize()
    for i in range(launches):
        src, dst = pairs[i % 4]
        dst.copy_(src)
    torch.cuda.synchronize()


def _pmc_rows(folder, counter, name_filter):
    """(kernel name, value) of `counter` per dispatch, in dispatch order, for
    kernels whose name passes `name_filter`, from a rocprofv3 --pmc
    --output-format csv folder."""
    import csv
    rows = []
    for dirpath, _, files in os.walk(folder):
        for f in files:
            if f.endswith("counter_collection.csv"):
                with open(os.path.join(dirpath, f)) as fh:
                    for r in csv.DictReader(fh):
                        if r["Counter_Name"] == counter and name_filter(r["Kernel_Name"]):
                            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return [(k, v) for _, k, v in sorted(rows)]


def _pmc_values(folder, counter, name_filter):
    """Per-dispatch values of `counter` (see _pmc_rows)."""
    return [v for _, v in _pmc_rows(folder, counter, name_filter)]


def _pmc_per_call(folder, counter, name_filter, n):
    """Values of `counter` per call over the last `n` calls of a kernel kind
    whose call may be several dispatches of different kernels (a GEMM plan
    of two launches): the dispatches of one call are the distinct kernel
    names among the last `n` rows, in a repeating order, and are summed."""
    rows = _pmc_rows(folder, counter, name_filter)
    d = len({k for k, _ in rows[-n:]}) if rows else 1
    rows = rows[-n * d:]
    if len(rows) < n * d:
        return []
    calls = [rows[i * d:(i + 1) * d] for i in range(n)]
    if any([k for k, _ in c] != [k for k, _ in calls[0]] for c in calls):
        raise SystemExit(f"{counter}: the profiled calls do not repeat one dispatch sequence")
    return [sum(v for _, v in c) for c in calls]


def summarize_pmc(a):
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = a.summarize_pmc
    kind = a.profile_kernel
    if kind is None:
        raise SystemExit("--summarize-pmc needs --profile-kernel (the kernel it covers)")
    is_gemm = kind.startswith("gemm")
    want = (lambda n: "gemm" in n and "frt::" in n) if is_gemm else \
        (lambda n: "norm_kernel" in n and "frt::" in n)
    is_copy = lambda n: "copyBuffer" in n  # noqa: E731
    # the profiled calls are the last --launches calls of their kind (set-up
    # launches of the same kernels come first); a call's dispatches are summed
    n = a.launches
    fk = _pmc_per_call(fetch_dir, "FETCH_SIZE", want, n)
    wk = _pmc_per_call(write_dir, "WRITE_SIZE", want, n)
    fc = _pmc_values(cfetch_dir, "FETCH_SIZE", is_copy)[-n:]
    wc = _pmc_values(cwrite_dir, "WRITE_SIZE", is_copy)[-n:]
    if not (fk and wk and fc and wc):
        raise SystemExit("missing counter rows: %d %d %d %d" % (len(fk), len(wk), len(fc), len(wc)))
    med = lambda v: float(np.median(v))  # noqa: E731
    # counters are KiB per dispatch; the copy moves COPY_BYTES each way
    f_scale = COPY_BYTES / (med(fc) * 1024.0)
    w_scale = COPY_BYTES / (med(wc) * 1024.0)
    fetch_b = med(fk) * 1024.0 * f_scale
    write_b = med(wk) * 1024.0 * w_scale
    rec = {"workload": a.workload, "kernel": kind, "calls": [len(fk), len(wk)],
           "fetch_kib_median": med(fk), "write_kib_median": med(wk),
           "copy_fetch_kib_median": med(fc), "copy_write_kib_median": med(wc),
           "copy_bytes_each_way": COPY_BYTES,
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "traffic_bytes": round(fetch_b + write_b),
           "sources_sha256": kernel_sources_sha(kind)}
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"traffic_w{a.workload}_{kind}.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def load_traffic(wid, kind):
    """Counter-derived HBM bytes per launch, or None when no record exists
    or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_w{wid}_{kind}.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_sha(kind):
        return None
    return int(rec["traffic_bytes"])


def hbm_calibration(torch, nbytes=1 << 30, reps=20):
    """Reference rates: a device-to-device copy of `nbytes` (read + write),
    a read-only reduction over `nbytes`, and the per-launch floor of an
    almost empty kernel replayed from a graph (every kernel pays it)."""
    def timed(fn, n):
        t_end = time.perf_counter() + 1.5
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    us = timed(lambda: dst.copy_(src), reps)
    gbs = 2 * nbytes / us / 1e3
    print(json.dumps({"hbm_calibration": "device copy", "bytes_read": nbytes,
                      "bytes_written": nbytes, "us_per_copy": round(us, 2),
                      "GB/s": round(gbs, 1),
                      "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4)}), flush=True)
    del dst
    f = src.view(torch.float32)
    us = timed(lambda: f.sum(), reps)
    gbs = nbytes / us / 1e3
    print(json.dumps({"hbm_calibration": "read-only reduction (sum)", "bytes_read": nbytes,
                      "us": round(us, 2), "GB/s": round(gbs, 1),
                      "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4)}), flush=True)
    del src, f
    tiny = torch.zeros(64, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(20):
            tiny.add_(1.0)
    us = timed(g.replay, 200) / 20
    print(json.dumps({"hbm_calibration": "launch floor (64-element add, graph replay)",
                      "us_per_launch": round(us, 3)}), flush=True)


def main():
    a = parse()
    if a.summarize_pmc:
        summarize_pmc(a)
        return
    if a.hbm_calibration:
        import torch
        hbm_calibration(torch)
        return
    if a.copy_kernel:
        import torch
        copy_kernel(torch, a.launches)
        return
    if a.gpus != 1:
        print(f"bench.py: the path runs on one GPU; --gpus {a.gpus} is not "
              "supported (its producers and GEMMs shard by rows or heads with "
              "no exchange on the forward path, so one GPU's shard is what is "
              "measured)", file=sys.stderr)
        sys.exit(2)
    import torch
    import norm_quantize_packed_amd as frt
    import workloads as wl

    t_start = time.perf_counter()
    torch.cuda.init()
    frt.load_library()
    res = measure(a, torch, frt, wl)
    if res is None:
        return
    # the default line also carries the other workloads' steps and per-kernel
    # tables (same steps and warm-up, no CPU baseline), measured after it
    plain = not (a.ffn or a.rope or a.oproj or a.mxfp4 or a.fp4_full or a.tp > 1
                 or a.rows is not None or a.warm)
    if a.workload == DEFAULT_WORKLOAD and plain and not a.no_other_workloads:
        res["other_workloads"] = []
        for wid in OTHER_WORKLOADS:
            t0 = time.perf_counter()
            b = argparse.Namespace(**vars(a))
            b.workload, b.no_cpu_baseline = wid, True
            r = measure(b, torch, frt, wl)
            gc.collect()
            torch.cuda.empty_cache()
            res["other_workloads"].append({
                "workload": r["config"]["workload"], "rows": r["config"]["rows"],
                "D": r["config"]["D"], "gemms": r["config"]["gemms"],
                "ms_per_step": r["ms_per_step"], "value": r["value"], "unit": r["unit"],
                "rotation_sets": r["config"]["rotation_sets"],
                "kernel_table_sets": r["config"]["kernel_table_sets"],
                "roofline": r["roofline"], "kernels": r["kernels"],
                "wall_s": round(time.perf_counter() - t0, 1)})
    res["wall_s_total"] = round(time.perf_counter() - t_start, 1)
    print(json.dumps(res), flush=True)


def measure(a, torch, frt, wl):
    """One workload's line (a dict), or None for a --profile-kernel run."""
    w0 = wl.WORKLOADS[a.workload]
    rows = a.rows if a.rows is not None else w0.rows
    if (a.rope or a.oproj) and a.workload not in wl.QKV_HEADS:
        raise SystemExit(f"--rope: the attention head is defined for workloads {sorted(wl.QKV_HEADS)}")
    if a.mxfp4 and wl.WORKLOADS[a.workload].form != "adarms":
        raise SystemExit("--mxfp4: the MXFP4 band covers the AdaRMS workloads' producer + packed "
                         "GEMM step (1, 2, 4), with --rope / --oproj / --ffn the rest of the layer (2)")
    if a.fp4_full and not (a.mxfp4 and a.ffn):
        raise SystemExit("--fp4-full: the MXFP4 band's FFN tail with an MXFP4 down projection "
                         "(needs --mxfp4 --ffn)")
    if a.tp < 1 or (a.tp > 1 and (a.workload not in wl.TP_UNIT or a.ffn or a.rope or a.oproj or a.mxfp4)):
        raise SystemExit(f"--tp: one rank's share of the packed GEMM, for workloads {sorted(wl.TP_UNIT)} "
                         "alone")
    w, dev, act, packs, pack_ms = build_sets(a.workload, rows, frt, torch, rope=a.rope, mx=a.mxfp4,
                                             tp=a.tp)
    ffn = None
    if a.ffn:
        if a.workload not in wl.FFN_HIDDEN:
            raise SystemExit("--ffn: the FFN tail follows the gate/up GEMM of "
                             f"workloads {sorted(wl.FFN_HIDDEN)}")
        ffn = build_ffn(w, rows, act, packs, frt, torch, mx=a.mxfp4, full=a.fp4_full)
    sets, per_set = make_rotation(w, dev, packs, rows, torch, ffn, warm=a.warm)
    rp = make_rope(w, rows, torch) if a.rope else None
    op = make_oproj(w, rows, frt, torch, mx=a.mxfp4) if a.oproj else None

    def attach(st, i):
        if rp is not None:
            st["rope"] = rp
        if op is not None:   # each rotation set streams its own W_o copy
            fresh = i > 0 and not a.warm
            st["oproj"] = dict(op, W8=op["W8"].clone() if fresh else op["W8"])
            if a.mxfp4 and fresh:
                st["oproj"]["ws"] = op["ws"].clone()

    def new_outputs():
        o = make_outputs(w, rows, packs, torch, ffn)
        if a.mxfp4:
            o["x4"] = [(torch.empty(rows, w.D // 2, dtype=torch.uint8, device="cuda"),
                        torch.empty(w.D // 256, rows, 8, dtype=torch.uint8, device="cuda"))
                       for _ in packs]
        return o

    def launches(s, o):
        return (step_launches_mx(w, s, o, rows, frt, wl.EPS) if a.mxfp4 else
                step_launches(w, s, act, o, rows, frt, wl.EPS))

    outs = new_outputs()
    for i, st in enumerate(sets):
        attach(st, i)
    nset = len(sets)

    steps_fns = [launches(s, outs) for s in sets]
    if a.profile_kernel:
        # one kernel kind, eagerly, over the rotation sets (after one full
        # step so every input it reads is defined)
        for _, fn in steps_fns[0]:
            fn()
        kinds = dict(steps_fns[0])
        if a.profile_kernel not in kinds:
            raise SystemExit(f"--profile-kernel: choose one of {sorted(kinds)}")
        torch.cuda.synchronize()
        for i in range(a.launches):
            dict(steps_fns[i % nset])[a.profile_kernel]()
        torch.cuda.synchronize()
        print(json.dumps({"profile_kernel": a.profile_kernel, "launches": a.launches,
                          "workload": w.name, "rotation_sets": nset}), flush=True)
        return None

    # eager reference of one step, then graph replays must reproduce it
    for _, fn in steps_fns[0]:
        fn()
    torch.cuda.synchronize()
    final = [outs["dn"]] if ffn is not None else outs["gemm"][-1]
    ref = [t.clone() for t in final]
    chunk = capture([fn for st in steps_fns for _, fn in st], torch)
    single = capture([fn for _, fn in steps_fns[0]], torch)
    for _ in range(3):
        chunk.replay()
        torch.cuda.synchronize()
        single.replay()
        torch.cuda.synchronize()
        for r, t in zip(ref, final):
            if not torch.equal(r, t):
                raise RuntimeError("graph replay differs from the eager step")

    # warmup + timed steps (exactly a.steps steps). Steps past the last whole
    # pass over the rotation sets run as one graph of exactly those steps
    # (the first `rem` sets): replayed one step at a time, a step shorter than
    # the host's replay call would time the host (16 x 512: 17.7 us a step
    # for 6.2 us of kernels)
    prefix = {}
    for k in (a.warmup, a.steps):
        rem = k % nset
        if rem and rem not in prefix:
            prefix[rem] = capture([fn for st in steps_fns[:rem] for _, fn in st], torch)

    def run_steps(k):
        full, rem = divmod(k, nset)
        for _ in range(full):
            chunk.replay()
        if rem:
            prefix[rem].replay()

    prewarm(chunk, a.prewarm_s, torch)
    run_steps(a.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    run_steps(a.steps)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / a.steps

    # per-kernel durations: graphs of one kernel kind over rotation sets.
    # The step's rotation counts every byte of a set, most of which a small
    # kernel of a large step never touches (workload 5's producer touches
    # 235 MB of a ~1.1 GB set), so the table extends the rotation until the
    # kernel with the fewest bytes moves ROTATE_BYTES over its launches
    # (within TABLE_MEM_BYTES of copies and TABLE_MAX_SETS), each added set
    # with its own outputs: no kernel's figure is served from the Infinity
    # Cache by a repeat of its own buffers.
    kinds = [k for k, _ in steps_fns[0]]
    has_extra = ffn is not None or rp is not None
    extra0 = unfused_launches(w, sets[0], act, outs, frt, mx=a.mxfp4) if has_extra else []
    all_kinds = kinds + [k for k, _ in extra0]
    work = {k: kernel_work(w, k, rows, packs, ffn, rp, op) for k in all_kinds}
    tab_sets, tab_fns, tab_outs = sets, steps_fns, [outs] * nset
    if not a.warm:
        out_bytes = tensor_bytes(list(outs.values()))
        least = min(b for b, _ in work.values())
        need = math.ceil(ROTATE_BYTES / max(least, 1))
        cap = max(nset, TABLE_MEM_BYTES // max(per_set + out_bytes, 1))
        n_tab = max(nset, min(need, cap, TABLE_MAX_SETS))
        if n_tab > nset:
            more = make_rotation(w, dev, packs, rows, torch, ffn, n_sets=n_tab, first=nset)[0]
            for i, st in enumerate(more):
                attach(st, nset + i)
            more_outs = [new_outputs() for _ in more]
            tab_sets = sets + more
            tab_outs = tab_outs + more_outs
            tab_fns = steps_fns + [launches(st, o) for st, o in zip(more, more_outs)]
    n_tab = len(tab_sets)
    timed = [[fn for _, fn in st] for st in tab_fns]
    if has_extra:
        extra = [unfused_launches(w, st, act, o, frt, mx=a.mxfp4) for st, o in zip(tab_sets, tab_outs)]
        timed = [t + [fn for _, fn in e] for t, e in zip(timed, extra)]
    for t in timed[nset:]:   # every added set's intermediate buffers defined once
        for fn in t:
            fn()
    torch.cuda.synchronize()
    table = []
    for ki, kind in enumerate(all_kinds):
        g = capture([timed[s][ki] for s in range(n_tab)], torch)
        prewarm(g, 0.3, torch)
        us = time_graph(g, a.kernel_reps, torch) * 1e3 / n_tab
        b, f = work[kind]
        row = {"kernel": kind, "us": round(us, 3), "bytes": int(b),
               "GB/s": round(b / us / 1e3, 1), "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
               "rotated_mib": round(n_tab * b / 2**20, 1)}
        if f:
            peak = FP4_PEAK_TFLOPS if "_mx" in kind else FP8_PEAK_TFLOPS
            row["TFLOP/s"] = round(f / us / 1e6, 2)
            row["mfma_frac"] = round(f / us / 1e6 / peak, 4)
            row["bound"] = "mfma" if f / b > peak * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
        else:
            row["bound"] = "hbm"
        if kind not in kinds:
            row["in_step"] = False      # the unfused comparison
        table.append(row)
        del g

    gemm_flops = sum(kernel_work(w, k, rows, packs, ffn, rp, op)[1] for k in kinds)
    norm_bytes = sum(kernel_work(w, k, rows, packs, ffn, rp, op)[0] for k in kinds if k.startswith("norm"))
    norm_us = sum(r["us"] for r in table if r["kernel"].startswith("norm"))
    dom = max((r for r in table if r["kernel"] in kinds), key=lambda r: r["us"])
    # (records cover the full workload shapes: not a --rows or --tp variant)
    traffic = (load_traffic(a.workload, dom["kernel"])
               if a.rows is None and a.tp == 1 and not a.warm else None)
    if dom["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dom["TFLOP/s"],
                "peak": FP4_PEAK_TFLOPS if "_mx" in dom["kernel"] else FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": dom["mfma_frac"], "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": dom["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": dom["hbm_frac"], "traffic": traffic}
    roof["kernel"] = dom["kernel"]
    roof["algorithmic_bytes"] = dom["bytes"]
    roof["traffic_unit"] = "bytes/launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)"

    value = gemm_flops / (ms * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4_e2m1" if a.mxfp4 else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name + ("+mxfp4" if a.mxfp4 else "")
                               + ("+qkv_rope_kvcache" if rp is not None else "")
                               + ("+o_proj" if op is not None else "")
                               + ("+ffn_geglu_down" if ffn is not None else "")
                               + ("+fp4_down" if a.fp4_full else "")
                               + (f"+tp{a.tp}_rank0" if a.tp > 1 else "")
                               + ("+warm" if a.warm else ""),
                   "rows": rows, "D": w.D,
                   "gemms": [list(p["splits"]) for p in packs], "bias": w.bias,
                   "rotation_sets": 1 if a.warm else nset,
                   "rotation_mib": round((1 if a.warm else nset) * per_set / 2**20, 1),
                   "kernel_table_sets": 1 if a.warm else n_tab,
                   "cache": "warm: one buffer set, repeats may hit the Infinity Cache" if a.warm
                            else "rotated: each pass moves >= 512 MiB of distinct buffers",
                   "step_gemm_gflop": round(gemm_flops / 1e9, 3)},
        "norm_gbps": round(norm_bytes / (norm_us * 1e3), 1) if norm_us else None,
        "norm_hbm_frac": round(norm_bytes / (norm_us * 1e3) / HBM_PEAK_GBS, 4) if norm_us else None,
        "roofline": roof,
        "kernels": table,
        "pack_ms": [round(x, 3) for x in pack_ms],
        "prewarm_s": a.prewarm_s,
        "wall_s_timed": round(wall, 4),
    }
    if ffn is not None:
        res["config"]["ffn"] = {"H": ffn["H"], "down": [w.D, ffn["H"]]}
    if rp is not None:
        res["config"]["rope"] = {k: rp[k] for k in ("nh", "kv", "hd", "P", "T")}
    if a.tp > 1:
        res["config"]["tp"] = {"ranks": a.tp, "rank": 0, "full_gemms": [list(g) for g in w.gemms]}
    if (not a.no_cpu_baseline and ffn is None and rp is None and op is None and not a.mxfp4
            and a.tp == 1 and not a.warm):
        res["cpu_baseline"] = cpu_baseline(w, rows)
    return res


if __name__ == "__main__":
    main()
