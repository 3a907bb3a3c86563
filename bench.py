#!/usr/bin/env python3
"""Throughput of the conv + KDA token mixer forward on one MI355X.

One step = kda_conv_forward (modality-aware short conv of q, k, v) followed by
kda_forward_chunks + kda_forward_scan (the two kernels of kda_forward) on one
stream, over one batch of the workload, inputs resident in HBM.  Prints one
JSON line.  The default workload is the 5-second 480x832 video stream
(512 text tokens + a 21x30x52 latent-patch grid, T = 33272, 16 heads of
dk = dv = 128, bf16 with fp32 accumulation).

Per-kernel durations come from HIP events recorded on the launch stream
between the three calls over the timed steps; the dominant kernel's roofline
uses the algorithmic bytes per launch of roofline_bytes().
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix-core peak, TFLOP/s

# HBM byte counters per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, in KiB), taken on
# the source files whose digest is stored beside them; a kernel whose sources changed since reports
# traffic null.  A plain 1 GiB device copy reads FETCH_SIZE = 524302 KiB and WRITE_SIZE = 1048576 KiB,
# hence the scale factors.
FETCH_SCALE = 1048576.0 / 524302.0
WRITE_SCALE = 1.0
KERNEL_SOURCES = {
    "conv": ("conv.hip", "common.h", "launch.h"),
    "chunks": ("kda.hip", "mfma.h", "common.h", "launch.h"),
    "scan": ("kda.hip", "mfma.h", "common.h", "launch.h"),
    "mla": ("mla.hip", "mfma.h", "common.h", "launch.h"),
    "kda_backward": ("kda_bwd.hip", "mfma.h", "common.h", "launch.h"),
}
# "kda_backward" is the sum over its three launches (records, ordered passes, gradients) per call.
MEASURED_TRAFFIC = {
    ("video_5s_480x832", "conv"): ("a9c80efba93f3ca5", 253456.1, 399264.0),
    ("video_5s_480x832", "chunks"): ("ce0c9745cfae1169", 270456.2, 586560.7),
    ("video_5s_480x832", "scan"): ("ce0c9745cfae1169", 293367.0, 133100.4),
    ("mla_video_5s_480x832", "mla"): ("fcf382f21189afaf", 1538698.3, 133088.0),
    ("video_5s_480x832", "kda_backward"): ("b0f36027eacb2097", 11119862.9, 10420261.1),
}
# Matrix-core operations per dispatch (rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
# SQ_INSTS_VALU_MFMA_MOPS_F32, each count is 512 flops), taken the same way.
MEASURED_MFMA_MOPS = {
    ("video_5s_480x832", "chunks"): ("ce0c9745cfae1169", 46858240.0, 2129920.0),
    ("video_5s_480x832", "scan"): ("ce0c9745cfae1169", 115015680.0, 0.0),
    ("mla_video_5s_480x832", "mla"): ("fcf382f21189afaf", 22151168000.0, 0.0),
    ("video_5s_480x832", "kda_backward"): ("b0f36027eacb2097", 0.0, 613416960.0),
}


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_sequence_modality_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """Counter-measured HBM bytes per launch, or None if not taken on the current sources."""
    rec = MEASURED_TRAFFIC.get((workload, kernel))
    if rec is None or rec[0] != source_digest(kernel):
        return None
    return int(round((rec[1] * FETCH_SCALE + rec[2] * WRITE_SCALE) * 1024))


def measured_mfma_flops(workload: str, kernel: str):
    """Counter-measured matrix-core flops per launch, or None if not taken on the current sources."""
    rec = MEASURED_MFMA_MOPS.get((workload, kernel))
    if rec is None or rec[0] != source_digest(kernel):
        return None
    return int(round((rec[1] + rec[2]) * 512))


def roofline_bytes(cfg) -> dict:
    """Algorithmic HBM bytes per launch of each kernel (what its interface must move).

    conv   : read q, k, v and write q', k', v'               6 d elements / token-head
             (+ the 3 x 31 taps per channel, once per launch)
    chunks : read q', k', v', alpha (3 dk + dv) and beta (1); write the chunk
             transform W, Qt, Kh (3 dk), Bq (64: a 64x64 block per 64 tokens)
             and Ut (dv), plus the fp32 chunk decay (dk per 64 tokens)
    scan   : read that transform back; write o (dv)
    """
    es = 4 if cfg.dtype == "f32" else 2
    th = cfg.B * cfg.T * cfg.H                      # token-heads per launch
    nch = (cfg.T + 63) // 64
    chunk_heads = cfg.B * cfg.H * nch
    conv = th * (3 * cfg.dk + 3 * cfg.dv) * es
    conv += 31 * cfg.H * (2 * cfg.dk + cfg.dv) * es
    ws = th * (3 * cfg.dk + 64 + cfg.dv) * es + chunk_heads * cfg.dk * 4
    chunks = th * ((3 * cfg.dk + cfg.dv) * es + es) + ws
    scan = ws + th * cfg.dv * es
    path_min = th * ((3 * cfg.dk + 3 * cfg.dv) * es + (3 * cfg.dk + cfg.dv + 1) * es + cfg.dv * es)
    return {"conv": conv, "chunks": chunks, "scan": scan, "path_min": path_min}


def mfma_flops(cfg) -> dict:
    """Matrix-core flops per launch as the kernels issue them (dense 16x16 tiles).

    chunks : per chunk-head, the 10 lower-triangle 16x16 tiles of A and Bq over
             dk (2 products each), W and Ut from the block-lower-triangular Tm
             (6 tile products per 16 columns), and the fp32 off-diagonal levels
             of Tm (16 tile products of 16x16x16)
    scan   : per chunk-head and 16 value columns, U = Ut - W S and
             S <- Gam S + Kh^T U (2 x 4 x dk/32 tile products) and the output
             (4 x dk/32 + 6 tile products); each tile product is 16x16x32
    The conv runs on the vector ALU (paired bf16 dot products), not on MFMA.
    """
    nch = (cfg.T + 63) // 64
    ch = cfg.B * cfg.H * nch
    t32 = 2 * 16 * 16 * 32                  # one 16x16x32 product
    nks = cfg.dk // 32
    chunks = ch * (10 * nks * 2 * t32 + (cfg.dk // 16 + cfg.dv // 16) * 6 * t32 + 16 * 2 * 16 * 16 * 16)
    scan = ch * (cfg.dv // 16) * ((2 * 4 * nks) + (4 * nks + 6)) * t32
    return {"chunks": chunks, "scan": scan}


def copy_bandwidth(torch, mib: int = 1024, reps: int = 5) -> float:
    """Measured device-to-device copy rate (read + write bytes / s) of a plain torch copy."""
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def cpu_baseline(cfg, frames: int) -> dict:
    """The fp64 oracle, as it stands, on a prefix of the same stream (text + first frames)."""
    import oracle
    from linear_attention_sequence_modality_amd.inputs import make_inputs

    gt, gh, gw = cfg.grid
    frames = gt if frames <= 0 else min(frames, gt)
    sample = cfg.with_(name=cfg.name + "_prefix", grid=(frames, gh, gw))
    inp = make_inputs(sample)
    t0 = time.perf_counter()
    oracle.conv_kda_forward(inp, sample.n_text, sample.grid)
    dt = time.perf_counter() - t0
    return {"value": sample.B * sample.T / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "fp64 C oracle (conv + sequential KDA recurrence, OpenMP over heads) on the "
                      "first %d of %d latent frames of the same stream: B=%d, T=%d (%d text + %dx%dx%d), "
                      "H=%d, dk=dv=%d; %.1f s wall" % (sample.grid[0], gt, sample.B, sample.T,
                                                      sample.n_text, *sample.grid, sample.H, sample.dk, dt)}


def mla_flops(cfg) -> float:
    """Matrix-core flops of one MLA attention launch: S = Q K^T over d_nope + d_dir and O = P V."""
    return 2.0 * cfg.B * cfg.H * cfg.T * cfg.T * (cfg.d_nope + cfg.d_dir + cfg.dv)


def mla_cpu_baseline(cfg, rows: int) -> dict:
    """The fp64 MLA oracle, as it stands, on ``rows`` query rows of every head of the same stream."""
    import numpy as np

    from oracle import mla as oracle_mla
    from linear_attention_sequence_modality_amd.inputs import make_mla_inputs

    inp = make_mla_inputs(cfg)
    sel = np.linspace(0, cfg.T - 1, rows).astype(int).tolist()
    t0 = time.perf_counter()
    oracle_mla.mla_attention(inp["q_nope"], inp["q_dir"], inp["k_nope"], inp["k_dir"], inp["v"], rows=sel)
    dt = time.perf_counter() - t0
    return {"value": cfg.B * rows / dt, "unit": "tokens/s", "cores": int(os.environ.get("OMP_NUM_THREADS", "0")) or
            os.cpu_count(), "kind": "oracle",
            "sample": "fp64 numpy oracle (scores, softmax, weighted values per head) on %d of the %d query "
                      "rows of each of the %d heads, against all %d keys; %.1f s wall; cores = the BLAS "
                      "threads numpy may use" % (rows, cfg.T, cfg.H, cfg.T, dt)}


def mla_main(args, torch) -> int:
    """One step = one mla_attention_forward launch over the whole stream."""
    from linear_attention_sequence_modality_amd import kda
    from linear_attention_sequence_modality_amd.inputs import MLA_WORKLOAD, make_mla_inputs

    cfg = MLA_WORKLOAD[args.mla_workload]
    torch.cuda.set_device(0)
    dev = {k: v.cuda() for k, v in make_mla_inputs(cfg).items()}
    x = [dev[k] for k in ("q_nope", "q_dir", "k_nope", "k_dir", "v")]
    o = torch.empty_like(dev["v"])
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        kda.mla_attention_forward(*x, o=o, stream=stream)
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in events:
        e[0].record(stream)
        kda.mla_attention_forward(*x, o=o, stream=stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    fl = mla_flops(cfg)
    tfs = fl / (ms * 1e-3) / 1e12
    result = {
        "metric": "MLA attention core forward tokens/s at 1 GPU; % of bf16-MFMA roofline",
        "value": round(cfg.B * cfg.T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "H": cfg.H, "d_nope": cfg.d_nope,
                   "d_dir": cfg.d_dir, "dv": cfg.dv, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "mla_attention", "achieved": round(tfs, 1),
                     "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                     "traffic": measured_traffic(cfg.name, "mla"), "flop_per_launch": fl,
                     "mfma_flop_counted": measured_mfma_flops(cfg.name, "mla"), "us": round(ms * 1e3, 1)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = mla_cpu_baseline(cfg, args.mla_cpu_rows)
    print(json.dumps(result), flush=True)
    return 0


MFMA_FP32_PEAK_TFS = 157.3    # MI355X dense fp32 matrix-core peak, TFLOP/s


def backward_flops(cfg) -> float:
    """fp32 multiply-add flops of one kda_backward launch sequence: the dense products per
    (batch, head, chunk) of the per-chunk transform (once, for the records the later
    kernels read), the two ordered passes and the gradient kernel."""
    C, dk, dv = 64, cfg.dk, cfg.dv
    mm = lambda m, n, k: 2.0 * m * n * k
    fwd = mm(C, C, dk) * 2 + mm(C, dk, C) + mm(C, dv, C)                 # A, Bq, W, Ut
    states = mm(C, dv, dk) + mm(dk, dv, C)
    reverse = mm(C, dv, C) + mm(C, dv, dk) + mm(dk, dv, C) * 2
    grads = (mm(C, dv, dk) + mm(C, dv, C) + mm(C, dv, dk) + mm(C, C, dv) + mm(C, dk, dv) + mm(C, dk, C)
             + mm(C, dk, dv) * 2 + mm(C, C, dv) + mm(C, C, dk) + mm(C, C, C) * 2 + mm(C, dv, C) + mm(C, dk, C)
             + mm(C, dk, C) + mm(C, dk, C) * 2)
    n_chunks = (cfg.T + C - 1) // C
    return cfg.B * cfg.H * n_chunks * (fwd + states + reverse + grads)


def backward_main(args, torch) -> int:
    """One step = kda_backward then kda_conv_backward over the whole stream."""
    import numpy as np

    from linear_attention_sequence_modality_amd import kda
    from linear_attention_sequence_modality_amd.inputs import WORKLOAD, make_inputs

    cfg = WORKLOAD[args.workload]
    torch.cuda.set_device(0)
    inp = {k: v.cuda() for k, v in make_inputs(cfg).items()}
    desc = kda.make_desc(cfg.n_text, cfg.grid, causal_t=cfg.causal_t)
    wt = (inp["w_text_q"], inp["w_text_k"], inp["w_text_v"])
    wv = (inp["w_vis_q"], inp["w_vis_k"], inp["w_vis_v"])
    qc, kc, vc = kda.kda_conv_forward(desc, inp["q"], inp["k"], inp["v"], wt, wv)
    g = np.random.default_rng(0)
    d_o = torch.from_numpy(g.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dv)).astype(np.float32)).to(
        cfg.torch_dtype).cuda()
    ws = torch.empty(kda.kda_backward_workspace_size(desc, cfg.B, cfg.H, cfg.dk, cfg.dv, cfg.torch_dtype),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        gk = kda.kda_backward(desc, qc, kc, vc, inp["alpha"], inp["beta"], d_o, workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        kda.kda_conv_backward(desc, inp["q"], inp["k"], inp["v"], wt, wv, gk["dq"], gk["dk"], gk["dv"],
                              stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in events:
        step(e)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kda_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    conv_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    fl = backward_flops(cfg)
    tfs = fl / (kda_ms * 1e-3) / 1e12
    es = 2 if cfg.dtype == "bf16" else 4
    conv_bytes = 3 * cfg.B * cfg.T * cfg.H * (2 * cfg.dk + cfg.dv) * es   # dy read twice, x read, dx written
    result = {
        "metric": "conv+KDA backward tokens/s at 1 GPU; % of fp32 matrix-core roofline",
        "value": round(cfg.B * cfg.T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "H": cfg.H, "dk": cfg.dk, "dv": cfg.dv,
                   "n_text": cfg.n_text, "grid": list(cfg.grid), "chunk": 64, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "kda_backward", "achieved": round(tfs, 2),
                     "peak": MFMA_FP32_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tfs / MFMA_FP32_PEAK_TFS, 4),
                     "traffic": measured_traffic(cfg.name, "kda_backward"), "flop_per_launch": fl,
                     "mfma_flop_counted": measured_mfma_flops(cfg.name, "kda_backward")},
        "kernels": {"kda_backward": {"us": round(kda_ms * 1e3, 1), "TFLOP/s": round(tfs, 2)},
                    "kda_conv_backward": {"us": round(conv_ms * 1e3, 1),
                                          "GB/s": round(conv_bytes / (conv_ms * 1e-3) / 1e9, 1),
                                          "frac_hbm": round(conv_bytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = backward_cpu_baseline(cfg, args.backward_cpu_tokens)
    print(json.dumps(result), flush=True)
    return 0


def backward_cpu_baseline(cfg, tokens: int) -> dict:
    """The fp64 adjoint oracle, as it stands, on the first ``tokens`` text-free tokens of every head."""
    import numpy as np

    from oracle import backward as ob
    from linear_attention_sequence_modality_amd.inputs import make_inputs

    sample = cfg.with_(name=cfg.name + "_prefix", n_text=min(cfg.n_text, tokens), grid=(0, 0, 0))
    inp = make_inputs(sample)
    g = np.random.default_rng(0)
    d_o = g.standard_normal((sample.B, sample.T, sample.H, sample.dv))
    t0 = time.perf_counter()
    ob.kda_recurrence_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], d_o)
    dt = time.perf_counter() - t0
    return {"value": sample.B * sample.T / dt, "unit": "tokens/s",
            "cores": int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count(), "kind": "oracle",
            "sample": "fp64 numpy token-level adjoint of the KDA recurrence (no conv) on %d tokens of each of "
                      "the %d heads (dk=%d, dv=%d); %.1f s wall; cores = the BLAS threads numpy may use" % (
                          sample.T, sample.H, sample.dk, sample.dv, dt)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="video_5s_480x832")
    ap.add_argument("--cpu-frames", type=int, default=0,
                    help="latent frames in the CPU-baseline sample (0 = the whole stream)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (three times) and "
                         "exit: the reference kernel for scaling HBM byte counters")
    ap.add_argument("--backward", action="store_true",
                    help="measure the backward (kda_backward + kda_conv_backward) instead")
    ap.add_argument("--backward-cpu-tokens", type=int, default=512,
                    help="tokens per head in the backward CPU-baseline sample")
    ap.add_argument("--mla", action="store_true",
                    help="measure the MLA attention core instead (one launch per step)")
    ap.add_argument("--mla-workload", default="mla_video_5s_480x832")
    ap.add_argument("--mla-cpu-rows", type=int, default=512,
                    help="query rows per head in the MLA CPU-baseline sample")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU path only: the conv + KDA mixer shards by head "
              "with no communication, and this benchmark runs on one GPU only "
              "(got --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.arange(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "copies": 3}), flush=True)
        return 0

    if args.mla:
        return mla_main(args, torch)
    if args.backward:
        return backward_main(args, torch)

    from linear_attention_sequence_modality_amd import kda
    from linear_attention_sequence_modality_amd.inputs import WORKLOAD, make_inputs

    cfg = WORKLOAD[args.workload]
    torch.cuda.set_device(0)
    inp = {k: v.cuda() for k, v in make_inputs(cfg).items()}
    desc = kda.make_desc(cfg.n_text, cfg.grid, causal_t=cfg.causal_t)
    dt = cfg.torch_dtype
    qc, kc, vc = (torch.empty_like(inp[s]) for s in ("q", "k", "v"))
    o = torch.empty_like(inp["v"])
    ws = torch.empty(kda.kda_forward_workspace_size(desc, cfg.B, cfg.H, cfg.dk, cfg.dv, dt),
                     dtype=torch.uint8, device="cuda")
    wt = (inp["w_text_q"], inp["w_text_k"], inp["w_text_v"])
    wv = (inp["w_vis_q"], inp["w_vis_k"], inp["w_vis_v"])
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        kda.kda_conv_forward(desc, inp["q"], inp["k"], inp["v"], wt, wv, qc, kc, vc, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        kda.kda_forward_chunks(desc, qc, kc, vc, inp["alpha"], inp["beta"], ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        kda.kda_forward_scan(desc, cfg.B, cfg.H, cfg.dk, cfg.dv, dt, ws, o, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nev = 4
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    step_ms = sorted(e[0].elapsed_time(e[-1]) for e in events)
    # cold steps: a 1 GiB fill before each one evicts L2 and the 256 MB Infinity Cache
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    n_cold = max(3, args.steps // 4)
    cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(n_cold)]
    for i in range(n_cold):
        scratch.fill_(i & 255)
        step(cold_ev[i])
    torch.cuda.synchronize()
    cold_ms = sorted(e[0].elapsed_time(e[-1]) for e in cold_ev)
    del scratch
    copy_gbs = copy_bandwidth(torch)

    names = ("conv", "chunks", "scan")
    ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in events) / args.steps for j, n in enumerate(names)}
    rb = roofline_bytes(cfg)
    fl = mfma_flops(cfg)
    kernels = {}
    for n in names:
        gbs = rb[n] / (ms[n] * 1e-3) / 1e9
        kernels[n] = {"us": round(ms[n] * 1e3, 2), "bytes": rb[n], "GB/s": round(gbs, 1),
                      "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                      "frac_measured_copy": round(gbs / copy_gbs, 4)}
        if n in fl:
            tf = fl[n] / (ms[n] * 1e-3) / 1e12
            kernels[n].update({"mfma_flop": fl[n], "mfma_flop_counted": measured_mfma_flops(cfg.name, n),
                               "TFLOP/s": round(tf, 1), "frac_mfma_bf16": round(tf / MFMA_BF16_PEAK_TFS, 4)})
    dom = max(names, key=lambda n: ms[n])
    ms_step = elapsed / args.steps * 1e3
    tokens = cfg.B * cfg.T
    value = tokens * args.steps / elapsed
    path_gbs = rb["path_min"] / (ms_step * 1e-3) / 1e9

    result = {
        "metric": "conv+KDA forward tokens/s at 1 GPU; % of HBM / bf16-MFMA roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "H": cfg.H, "dk": cfg.dk,
                   "dv": cfg.dv, "n_text": cfg.n_text, "grid": list(cfg.grid),
                   "chunk": 64, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["GB/s"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kernels[dom]["frac_hbm"],
                     "traffic": measured_traffic(cfg.name, dom)},
        "kernels": kernels,
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 4), "min": round(step_ms[0], 4),
                    "cold_median": round(cold_ms[len(cold_ms) // 2], 4), "cold_min": round(cold_ms[0], 4),
                    "cold_tokens_per_s": round(tokens / (cold_ms[len(cold_ms) // 2] * 1e-3), 1),
                    "cold": "each step after a 1 GiB fill that evicts L2 and the Infinity Cache"},
        "measured_copy_GB/s": round(copy_gbs, 1),
        "path": {"min_bytes": rb["path_min"], "GB/s_vs_path_min": round(path_gbs, 1),
                 "frac_of_path_roofline": round(path_gbs / HBM_PEAK_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_frames)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
