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
uses the algorithmic bytes per launch of roofline_bytes() (the measurement plan's
per-token-head figures).
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
    "chunks": ("kda.hip", "kda_ws.h", "mfma.h", "common.h", "launch.h"),
    "scan": ("kda_scan.hip", "kda_ws.h", "mfma.h", "common.h", "launch.h"),
    "mla": ("mla.hip", "mfma.h", "common.h", "launch.h"),
    "mla_latent": ("mla_proj.hip", "mfma.h", "common.h", "launch.h"),
    "kda_backward": ("kda_bwd.hip", "mfma.h", "common.h", "launch.h"),
}
# "kda_backward" is the sum over its three launches (records, ordered passes, gradients) per call,
# "scan" over the state pass's three (summaries, chain, replay), "mla_latent" over its two.
MEASURED_TRAFFIC = {
    ("video_5s_480x832", "conv"): ("1e1ee127d724456d", 213833.5, 399264.5),
    ("video_5s_480x832", "chunks"): ("cfa2c67a3dfbdee9", 270451.6, 586560.9),
    ("video_5s_480x832", "scan"): ("9026246c558a04e4", 517482.5, 180197.6),
    ("mla_video_5s_480x832", "mla"): ("9bcc320e76aca060", 1537386.9, 133088.0),
    ("mla_video_5s_480x832", "mla_latent"): ("e6aee03f454abe42", 235091.0, 303607.0),
    ("video_5s_480x832", "kda_backward"): ("c134e420cfa7abe2", 10597820.1, 10058142.1),
}
# Matrix-core operations per dispatch (rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
# SQ_INSTS_VALU_MFMA_MOPS_F32, each count is 512 flops), taken the same way.
MEASURED_MFMA_MOPS = {
    ("video_5s_480x832", "chunks"): ("cfa2c67a3dfbdee9", 46858240.0, 2129920.0),
    ("video_5s_480x832", "scan"): ("9026246c558a04e4", 244776960.0, 2097152.0),
    ("mla_video_5s_480x832", "mla"): ("9bcc320e76aca060", 22151168000.0, 0.0),
    ("mla_video_5s_480x832", "mla_latent"): ("e6aee03f454abe42", 425984000.0, 0.0),
    ("video_5s_480x832", "kda_backward"): ("c134e420cfa7abe2", 0.0, 575078400.0),
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
    """Algorithmic HBM bytes per launch of each kernel: the per-token-head figures of the
    measurement plan (at d = dk = dv = 128 in bf16: conv 1536, chunk transform 2306, state
    pass 1536, path minimum 2818) times the token-heads of one launch.

    conv     : read q, k, v and write q', k', v'                  (3 dk + 3 dv) elements
               (+ the 3 x 31 taps per channel, once per launch)
    chunks   : read q', k', v', alpha (3 dk + dv) and beta (1); write a chunk
               workspace of five vectors per token (three over dk: W, the output
               operator, Kh; two over dv: Ut and the intra-chunk output)
                                                                  (6 dk + 3 dv + 1)
    scan     : read that workspace back and write o               (3 dk + 3 dv)
    path_min : conv in and out, KDA in and out (no workspace)
    The workspace these kernels exchange is smaller than those five vectors: W, Qt and
    Kh over dk, Bq as 64 values and Ut over dv per token-head, plus the fp32 chunk decay
    per chunk.  What their interfaces move with it is in chunks_interface and
    scan_interface.  (The segmented state pass reads the W, Kh, Ut and decay of every
    chunk outside a stream's last segment a second time, for the segment summaries:
    traffic above these bytes, reported by the counters.)
    """
    es = 4 if cfg.dtype == "f32" else 2
    th = cfg.B * cfg.T * cfg.H                      # token-heads per launch
    dk, dv = cfg.dk, cfg.dv
    nch = (cfg.T + 63) // 64
    chunk_heads = cfg.B * cfg.H * nch
    conv = th * (3 * dk + 3 * dv) * es
    conv += 31 * cfg.H * (2 * dk + dv) * es
    chunks = th * (6 * dk + 3 * dv + 1) * es
    scan = th * (3 * dk + 3 * dv) * es
    ws = th * (3 * dk + 64 + dv) * es + chunk_heads * dk * 4
    chunks_if = th * ((3 * dk + dv) * es + es) + ws
    scan_if = ws + th * dv * es
    path_min = th * ((3 * dk + 3 * dv) * es + (3 * dk + dv + 1) * es + dv * es)
    return {"conv": conv, "chunks": chunks, "scan": scan, "path_min": path_min,
            "chunks_interface": chunks_if, "scan_interface": scan_if}


def seg_plan(cfg):
    """The state pass's cut of each stream's chunks into segments (as the library plans it):
    about 256 (segment, head) units over the chip, at most 32 segments per stream."""
    nch = (cfg.T + 63) // 64
    work = cfg.B * nch * cfg.H
    target = (work + 255) // 256 if work > 256 else 1
    p = min(32, max(1, (nch + target - 1) // target))
    length = (nch + p - 1) // p
    return (nch + length - 1) // length, length


def mfma_flops(cfg) -> dict:
    """Matrix-core flops per launch as the kernels issue them (dense 16x16 tiles).

    chunks : per chunk-head, the 10 lower-triangle 16x16 tiles of A and Bq over
             dk (2 products each), W and Ut from the block-lower-triangular Tm
             (6 tile products per 16 columns), and the fp32 off-diagonal levels
             of Tm (16 tile products of 16x16x16)
    scan   : the segmented state pass, bf16 products (each a 16x16x32 tile):
             segment summaries, per chunk-head of every segment but a stream's
             last, U = Ut - W S and S <- Gam S + Kh^T U for L (dv columns) and
             for Phi (dk columns); the replay, per chunk-head and 16 value
             columns, U and S as above (2 x 4 x dk/32) and the output
             (4 x dk/32 + 6)
    scan_f32 : the chain of segment start states on fp32 16x16x4 products: per
             (stream, head, 16 state columns) and step (rounded up to whole
             groups of four), (dk/16)^2 x 4 products
    The conv runs on the vector ALU (paired bf16 dot products), not on MFMA.
    """
    nch = (cfg.T + 63) // 64
    ch = cfg.B * cfg.H * nch
    t32 = 2 * 16 * 16 * 32                  # one 16x16x32 product
    nks = cfg.dk // 32
    chunks = ch * (10 * nks * 2 * t32 + (cfg.dk // 16 + cfg.dv // 16) * 6 * t32 + 16 * 2 * 16 * 16 * 16)
    replay = ch * (cfg.dv // 16) * ((2 * 4 * nks) + (4 * nks + 6)) * t32
    nseg, length = seg_plan(cfg)
    summed = cfg.B * cfg.H * (nseg - 1) * length if nseg > 1 else 0
    per_chunk = sum(4 * (w // 16) * nks + (cfg.dk // 16) * (w // 16) * 2 for w in (cfg.dv, cfg.dk))
    steps = ((nseg - 1 + 3) // 4) * 4 if nseg > 1 else 0
    chain = cfg.B * cfg.H * (cfg.dv // 16) * steps * (cfg.dk // 16) ** 2 * 4 * (2 * 16 * 16 * 4)
    return {"chunks": chunks, "scan": replay + summed * per_chunk * t32, "scan_f32": chain}


def gemm_tflops(torch, n: int = 8192, reps: int = 5) -> float:
    """Measured dense bf16 matrix-core rate of a plain library GEMM (torch.matmul, n^3, fp32
    accumulation inside the library), beside the vendor peak: the matrix-core calibration."""
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


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


def cpu_baseline(cfg, frames: int, single_tokens: int):
    """The fp64 oracle, as it stands, on a prefix of the same stream (text + first frames), on
    all the threads OpenMP gives it, and on one thread over a shorter prefix.  Returns (the
    oracle's outputs (q', k', v', o, S_T) when the prefix is the whole stream, else None; the
    baseline record)."""
    import oracle
    from linear_attention_sequence_modality_amd.inputs import make_inputs

    gt, gh, gw = cfg.grid
    frames = gt if frames <= 0 else min(frames, gt)
    sample = cfg.with_(name=cfg.name + "_prefix", grid=(frames, gh, gw))
    inp = make_inputs(sample)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    ref = oracle.conv_kda_forward(inp, sample.n_text, sample.grid, sample.causal_t)
    dt = time.perf_counter() - t0
    # one thread: the text tokens and as many whole latent frames as fit single_tokens
    f1 = min(frames, max(1, (single_tokens - cfg.n_text) // max(1, gh * gw))) if gt else 0
    one = cfg.with_(name=cfg.name + "_prefix1", grid=(f1, gh, gw) if gt else cfg.grid)
    outs = None
    if frames == gt:
        # the sample is the whole stream (same seed, same draws): keep the oracle's
        # outputs for the parity figures of the run
        outs = ref
    inp1 = make_inputs(one)
    oracle.set_num_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.conv_kda_forward(inp1, one.n_text, one.grid)
        dt1 = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(threads)
    return outs, {"value": sample.B * sample.T / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "nproc": os.cpu_count(),
            "single_thread": {"value": one.B * one.T / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": "B=%d, T=%d (%d text + %dx%dx%d), H=%d; %.1f s wall" % (
                                  one.B, one.T, one.n_text, *one.grid, one.H, dt1)},
            "sample": "fp64 C oracle (conv + sequential KDA recurrence, OpenMP over heads) on the "
                      "first %d of %d latent frames of the same stream: B=%d, T=%d (%d text + %dx%dx%d), "
                      "H=%d, dk=dv=%d; %.1f s wall on %d threads (host nproc %s)" % (
                          sample.grid[0], gt, sample.B, sample.T, sample.n_text, *sample.grid, sample.H,
                          sample.dk, dt, threads, os.cpu_count())}


def stage_parity(torch, kda, cfg, desc, inp, ws, ref) -> dict:
    """The run's outputs against the oracle's on the whole stream: the gate metric (max over
    (b, h) of max |x - ref| / max |ref|) and the element-wise figure, per stage."""
    import oracle

    dt = cfg.torch_dtype
    wt = (inp["w_text_q"], inp["w_text_k"], inp["w_text_v"])
    wv = (inp["w_vis_q"], inp["w_vis_k"], inp["w_vis_v"])
    qc, kc, vc = kda.kda_conv_forward(desc, inp["q"], inp["k"], inp["v"], wt, wv)
    sT = torch.empty(cfg.B, cfg.H, cfg.dk, cfg.dv, dtype=torch.float32, device="cuda")
    o = kda.kda_forward(desc, qc, kc, vc, inp["alpha"], inp["beta"], final_state=sT, workspace=ws)
    torch.cuda.synchronize()
    out = {}
    for name, got, want in zip(("q'", "k'", "v'", "o"), (qc, kc, vc, o), ref[:4]):
        g = got.double().cpu().numpy()
        out[name] = {"rel_err": float("%.3g" % oracle.rel_err(g, want)),
                     "elementwise": float("%.3g" % oracle.rel_err_elementwise(g, want))}
    g = sT.double().cpu().numpy()
    out["S_T"] = {"rel_err": float("%.3g" % oracle.rel_err_state(g, ref[4])),
                  "elementwise": float("%.3g" % oracle.rel_err_elementwise(g, ref[4], layout="state"))}
    out["gate"] = 2e-2 if dt == torch.bfloat16 else 1e-4
    return out


def mla_flops(cfg) -> float:
    """Matrix-core flops of one MLA attention launch: S = Q K^T over d_nope + d_dir and O = P V."""
    return 2.0 * cfg.B * cfg.H * cfg.T * cfg.T * (cfg.d_nope + cfg.d_dir + cfg.dv)


def mla_cpu_baseline(cfg, rows: int) -> dict:
    """The fp64 MLA oracle, as it stands, on the same layer: the latent projections of every
    token, then attention for ``rows`` query rows of every head."""
    import numpy as np

    from oracle import mla as oracle_mla
    from linear_attention_sequence_modality_amd.inputs import make_mla_latent_inputs

    inp = make_mla_latent_inputs(cfg)
    sel = np.linspace(0, cfg.T - 1, rows).astype(int).tolist()
    t0 = time.perf_counter()
    oracle_mla.mla_layer(inp["x"], inp["q_nope"], inp["q_dir"], inp["w_dkv"], inp["w_kr"], inp["w_uk"], inp["w_uv"],
                         rows=sel)
    dt = time.perf_counter() - t0
    return {"value": cfg.B * rows / dt, "unit": "tokens/s", "cores": int(os.environ.get("OMP_NUM_THREADS", "0")) or
            os.cpu_count(), "kind": "oracle",
            "sample": "fp64 numpy oracle: the latent projections of all %d tokens, then scores, softmax and "
                      "weighted values for %d of the query rows of each of the %d heads against all keys; "
                      "%.1f s wall; cores = the BLAS threads numpy may use" % (cfg.B * cfg.T, rows, cfg.H, dt)}


def mla_latent_flops(cfg) -> float:
    """Matrix-core flops of the latent projections: x W_dkv^T, x W_kr^T, c W_uk^T, c W_uv^T."""
    rows = cfg.B * cfg.T
    return 2.0 * rows * (cfg.model_width * (cfg.latent_width + cfg.d_dir)
                         + cfg.latent_width * cfg.H * (cfg.d_nope + cfg.dv))


def mla_main(args, torch) -> int:
    """One step = the MLA token mixer from hidden states: mla_latent_forward (two launches)
    then mla_attention_forward, each timed with HIP events on the launch stream."""
    from linear_attention_sequence_modality_amd import kda
    from linear_attention_sequence_modality_amd.inputs import MLA_WORKLOAD, make_mla_latent_inputs

    cfg = MLA_WORKLOAD[args.mla_workload]
    torch.cuda.set_device(0)
    dev = {k: v.cuda() for k, v in make_mla_latent_inputs(cfg).items()}
    w = [dev[k] for k in ("w_dkv", "w_kr", "w_uk", "w_uv")]
    lat = [torch.empty(cfg.B, cfg.T, cfg.latent_width, dtype=torch.bfloat16, device="cuda"),
           torch.empty(cfg.B, cfg.T, cfg.d_dir, dtype=torch.bfloat16, device="cuda"),
           torch.empty(cfg.B, cfg.T, cfg.H, cfg.d_nope, dtype=torch.bfloat16, device="cuda"),
           torch.empty(cfg.B, cfg.T, cfg.H, cfg.dv, dtype=torch.bfloat16, device="cuda")]
    o = torch.empty_like(lat[3])
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        kda.mla_latent_forward(dev["x"], *w, cfg.H, outputs=lat, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        kda.mla_attention_forward(dev["q_nope"], dev["q_dir"], lat[2], lat[1], lat[3], o=o, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in events:
        step(e)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_lat = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    ms_att = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    fl_att, fl_lat = mla_flops(cfg), mla_latent_flops(cfg)
    tfs_att = fl_att / (ms_att * 1e-3) / 1e12
    tfs_lat = fl_lat / (ms_lat * 1e-3) / 1e12
    result = {
        "metric": "MLA token mixer forward (latent projections + attention) tokens/s at 1 GPU; "
                  "% of bf16-MFMA roofline",
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
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "H": cfg.H, "d_model": cfg.model_width,
                   "d_c": cfg.latent_width, "d_nope": cfg.d_nope, "d_dir": cfg.d_dir, "dv": cfg.dv,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "mla_attention", "achieved": round(tfs_att, 1),
                     "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tfs_att / MFMA_BF16_PEAK_TFS, 4),
                     "traffic": measured_traffic(cfg.name, "mla"), "flop_per_launch": fl_att,
                     "mfma_flop_counted": measured_mfma_flops(cfg.name, "mla"), "us": round(ms_att * 1e3, 1)},
        "kernels": {"latent": {"us": round(ms_lat * 1e3, 1), "flop": fl_lat, "TFLOP/s": round(tfs_lat, 1),
                               "frac_mfma_bf16": round(tfs_lat / MFMA_BF16_PEAK_TFS, 4),
                               "traffic": measured_traffic(cfg.name, "mla_latent")},
                    "attention": {"us": round(ms_att * 1e3, 1), "flop": fl_att, "TFLOP/s": round(tfs_att, 1),
                                  "frac_mfma_bf16": round(tfs_att / MFMA_BF16_PEAK_TFS, 4)}},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = mla_cpu_baseline(cfg, args.mla_cpu_rows)
    print(json.dumps(result), flush=True)
    return 0


MFMA_FP32_PEAK_TFS = 157.3    # MI355X dense fp32 matrix-core peak, TFLOP/s


def backward_flops(cfg) -> float:
    """fp32 multiply-add flops of one kda_backward launch sequence: the dense products per
    (batch, head, chunk) of the per-chunk transform (once, for the records the later
    kernels read), the two ordered passes and the gradient kernel.  The decayed products
    inside a chunk (A and Bq in the transform, two row-side and two column-side products in
    the gradient kernel) cover the 10 block pairs on and below the diagonal of 16-row
    blocks, each 16 x 16 with the contraction over the channels (A, Bq) or over the 16 rows
    of a block (the others)."""
    C, dk, dv = 64, cfg.dk, cfg.dv
    mm = lambda m, n, k: 2.0 * m * n * k
    tri_form = 10 * mm(16, 16, dk)
    tri_apply = 10 * mm(16, dk, 16)
    fwd = tri_form * 2 + mm(C, dk, C) + mm(C, dv, C)                   # A, Bq, W, Ut
    states = mm(C, dv, dk) + mm(dk, dv, C)
    reverse = mm(C, dv, C) + mm(C, dv, dk) + mm(dk, dv, C) * 2
    grads = (mm(C, dv, dk)                      # U = Ut - W S
             + mm(C, dv, C) + mm(C, dv, dk)     # dU = Bq^T dO + Kh dS'
             + mm(C, C, dv)                     # dBq
             + mm(C, dk, dv) * 3                # dQt = dO S^T, dKh = U dS'^T, dW = -dU S^T
             + mm(C, C, dv) + mm(C, C, dk)      # dTm = dU V^T + dW Kt^T
             + mm(C, C, C) * 2                  # Tm^T dTm, dM
             + mm(C, dv, C) + mm(C, dk, C)      # dX, dY
             + tri_apply * 4)                   # R(dA, K), R(dBq, K), C(dA, K), C(dBq, Q)
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


def fused_path(torch, kda, cfg, desc, inp, steps, warmup, ms_step):
    """The same step through kda_conv_kda_forward (the conv formed inside the chunk
    transform; q', k', v' never written): its time per step beside the two-call path's,
    and the activation memory it does without."""
    wt = (inp["w_text_q"], inp["w_text_k"], inp["w_text_v"])
    wv = (inp["w_vis_q"], inp["w_vis_k"], inp["w_vis_v"])
    ws = torch.empty(kda.kda_conv_kda_forward_workspace_size(desc, cfg.B, cfg.H, cfg.dk, cfg.dv,
                                                             cfg.torch_dtype), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(inp["v"])
    stream = torch.cuda.current_stream()

    def call():
        kda.kda_conv_kda_forward(desc, inp["q"], inp["k"], inp["v"], wt, wv, inp["alpha"], inp["beta"], o=o,
                                 workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    es = 4 if cfg.dtype == "f32" else 2
    return {"call": "kda_conv_kda_forward", "ms_per_step": round(ms, 4),
            "tokens_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1),
            "time_vs_two_calls": round(ms / ms_step, 3),
            "activation_bytes_not_held": cfg.B * cfg.T * cfg.H * (2 * cfg.dk + cfg.dv) * es}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="video_5s_480x832")
    ap.add_argument("--cpu-frames", type=int, default=0,
                    help="latent frames in the CPU-baseline sample (0 = the whole stream)")
    ap.add_argument("--cpu-single-tokens", type=int, default=4096,
                    help="tokens per stream in the one-thread CPU-baseline sample")
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
    fused = fused_path(torch, kda, cfg, desc, inp, args.steps, args.warmup, ms_step=elapsed / args.steps * 1e3)
    copy_gbs = copy_bandwidth(torch)
    gemm_tfs = gemm_tflops(torch)

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
        if n + "_f32" in fl:
            kernels[n]["mfma_flop_f32"] = fl[n + "_f32"]
        if n + "_interface" in rb:
            kernels[n]["interface_bytes"] = rb[n + "_interface"]
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
        "measured_bf16_gemm_TFLOP/s": round(gemm_tfs, 1),
        "path": {"min_bytes": rb["path_min"], "GB/s_vs_path_min": round(path_gbs, 1),
                 "frac_of_path_roofline": round(path_gbs / HBM_PEAK_GBS, 4)},
        "fused_path": fused,
    }
    if not args.no_cpu_baseline:
        ref, result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_frames, args.cpu_single_tokens)
        if ref is not None:
            result["parity"] = stage_parity(torch, kda, cfg, desc, inp, ws, ref)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
