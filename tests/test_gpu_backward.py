"""KDA backward, HIP path vs the fp64 adjoint oracle (needs an MI355X).

Gates as for the forward: max relative error per (batch, head) over max |ref|
<= 1e-4 for fp32 streams, 2e-2 for bf16 streams, for the gradients of q, k,
v, alpha, beta and the initial state.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob
from linear_attention_sequence_modality_amd import kda
from linear_attention_sequence_modality_amd.inputs import StreamConfig, make_inputs

from gpu_common import TOL, check_backward, desc_of, edge_alpha, rel, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [
    StreamConfig("bwd_f32", B=2, H=2, dk=64, dv=64, n_text=11, grid=(2, 6, 9), dtype="f32", seed=81),
    StreamConfig("bwd_bf16", B=1, H=2, dk=128, dv=128, n_text=7, grid=(3, 5, 9), dtype="bf16", seed=82),
    StreamConfig("bwd_one_chunk", B=1, H=2, dk=64, dv=128, n_text=64, grid=(0, 0, 0), dtype="bf16", seed=83),
    StreamConfig("bwd_one_token", B=2, H=1, dk=128, dv=64, n_text=1, grid=(0, 0, 0), dtype="bf16", seed=84),
    StreamConfig("bwd_long", B=1, H=1, dk=128, dv=128, n_text=0, grid=(4, 12, 13), dtype="bf16", seed=85),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_backward_matches_the_adjoint_oracle(cfg):
    check_backward(cfg, make_inputs(cfg))


DECAY = [("bf16", 128), ("f32", 64), ("f32", 128)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d", DECAY, ids=["%s_d%d" % x for x in DECAY])
@pytest.mark.parametrize("kind", ["strong", "edge"])
def test_backward_under_strong_decay(kind, dtype, d):
    """Fast forgetting, where a chunk's decay leaves the fp32 range.

    strong: alpha = sigmoid(N(-1.5, 1)), about 0.2 per token, so a 64-token chunk
    decays by about 2^-150 per channel; edge: alpha = 2^-14 on runs of tokens
    (any 8 consecutive tokens decay by 2^-112, inside the 2^-120 the forward
    accepts), one run over whole chunks.  The decayed products inside a chunk
    must stay finite and match the fp64 adjoint of the recurrence.

    At the edge, d alpha of a token with alpha = 2^-14 is d log alpha / alpha, and
    the chunked form gets d log alpha as a reverse running sum of terms of order
    one that cancel down to order alpha: their fp32 rounding (about 2^-24 each,
    a few dozen of them) is divided by 2^-14, which bounds d alpha's relative
    error near 2^-24 * 8 * 2^14 = 8e-3 in fp32 streams.  So there d log alpha is
    gated at the standard tolerance and d alpha at 2e-2 (the bf16 gate, which
    the bf16 stream meets anyway)."""
    if dtype == "f32" and d == 128 and not kda.supports(torch.float32, 128, 128):
        pytest.skip("fp32 at dk = dv = 128 is refused by this build of the library")
    cfg = StreamConfig("bwd_decay_%s" % kind, B=1, H=2, dk=d, dv=d, n_text=21, grid=(3, 7, 9), dtype=dtype,
                       seed=87 if kind == "strong" else 88)
    if kind == "strong":
        host = make_inputs(cfg, alpha_mean=-1.5)
    else:
        host = make_inputs(cfg)
        host["alpha"] = torch.from_numpy(edge_alpha(cfg, host)).to(cfg.torch_dtype)
    check_backward(cfg, host, dalpha_tol=2e-2 if kind == "edge" else None)


@pytest.mark.timeout(120)
def test_backward_without_state_arguments_and_deterministic():
    """initial_state and d_final_state absent mean zero; two calls agree bit for bit."""
    cfg = CASES[1]
    host = make_inputs(cfg)
    g = np.random.default_rng(3)
    dO = torch.from_numpy(g.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dv)).astype(np.float32)).to(cfg.torch_dtype)
    dev = {k: v.cuda() for k, v in host.items()}
    args = (desc_of(cfg), dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dO.cuda())
    a = kda.kda_backward(*args)
    b = kda.kda_backward(*args)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dalpha", "dbeta", "d_initial_state"):
        assert torch.equal(a[name], b[name]), name
    ref = ob.kda_recurrence_backward(host["q"], host["k"], host["v"], host["alpha"], host["beta"], dO)
    e = rel(a["dk"].double().cpu().numpy(), ref["dk"])
    say("  no-state rel err dk %.2e" % e)
    assert e <= TOL[cfg.dtype]


CONV_CASES = [
    StreamConfig("cbwd_bf16", B=2, H=2, dk=128, dv=64, n_text=9, grid=(3, 5, 7), dtype="bf16", seed=91),
    StreamConfig("cbwd_causal_f32", B=1, H=2, dk=64, dv=64, n_text=5, grid=(4, 3, 6), dtype="f32", causal_t=1, seed=92),
    StreamConfig("cbwd_text", B=1, H=1, dk=64, dv=64, n_text=70, grid=(0, 0, 0), dtype="bf16", seed=93),
    # visual only, symmetric padding: the input gradient comes from the mirrored-tap conv alone
    StreamConfig("cbwd_vis_f32", B=2, H=1, dk=64, dv=128, n_text=0, grid=(5, 6, 9), dtype="f32", seed=94),
    # the video workload's width (2048 channels: 8 channel blocks) and enough token ranges that
    # each tap-gradient workgroup walks several of them
    StreamConfig("cbwd_wide_bf16", B=1, H=16, dk=128, dv=128, n_text=40, grid=(3, 20, 50), dtype="bf16", seed=95),
    # 64 channels per stream: half a 128-channel tap-gradient block; time-causal, two batches,
    # row and w counts off the 8 x 8 tile
    StreamConfig("cbwd_narrow_causal_bf16", B=2, H=1, dk=64, dv=64, n_text=3, grid=(4, 9, 10), dtype="bf16",
                 causal_t=1, seed=96),
    # one latent slice (an image): every tile is a single step of the march
    StreamConfig("cbwd_image_bf16", B=1, H=2, dk=128, dv=64, n_text=5, grid=(1, 17, 19), dtype="bf16", seed=97),
    # 20 batches x 16 channel blocks: more (batch, channel block) pairs than compute units, so
    # each visual tap-gradient block walks every tile of its pair
    StreamConfig("cbwd_many_pairs_bf16", B=20, H=16, dk=128, dv=128, n_text=3, grid=(2, 3, 9), dtype="bf16",
                 seed=98),
    # one visual token and nothing else: every tap but the centre falls outside the grid
    StreamConfig("cbwd_one_visual_bf16", B=2, H=1, dk=64, dv=64, n_text=0, grid=(1, 1, 1), dtype="bf16", seed=99),
    # a column of two latent slices, time-causal: only the a = 1, 2 taps meet the grid
    StreamConfig("cbwd_column_causal_f32", B=1, H=2, dk=128, dv=64, n_text=2, grid=(2, 1, 1), dtype="f32",
                 causal_t=1, seed=100),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cfg", CONV_CASES, ids=[c.name for c in CONV_CASES])
def test_conv_backward_matches_the_adjoint_oracle(cfg):
    say("case %s B=%d T=%d %s causal_t=%d" % (cfg.name, cfg.B, cfg.T, cfg.dtype, cfg.causal_t))
    host = make_inputs(cfg)
    g = np.random.default_rng(cfg.seed)
    dys = {s: torch.from_numpy(g.standard_normal(tuple(host[s].shape)).astype(np.float32)).to(cfg.torch_dtype)
           for s in ("q", "k", "v")}
    dev = {k: v.cuda() for k, v in host.items()}
    out = kda.kda_conv_backward(desc_of(cfg), dev["q"], dev["k"], dev["v"],
                                (dev["w_text_q"], dev["w_text_k"], dev["w_text_v"]),
                                (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"]),
                                dys["q"].cuda(), dys["k"].cuda(), dys["v"].cuda())
    torch.cuda.synchronize()
    for i, s in enumerate(("q", "k", "v")):
        B, T, H, d = host[s].shape
        dx, dwt, dwv = ob.short_conv_backward(host[s].reshape(B, T, H * d), host["w_text_" + s], host["w_vis_" + s],
                                              dys[s].reshape(B, T, H * d), cfg.n_text, cfg.grid, cfg.causal_t)
        e_x = rel(out["d" + s].double().cpu().numpy(), dx.reshape(B, T, H, d))
        e_t = float(np.abs(out["dw_text"][i].double().cpu().numpy() - dwt).max() / max(np.abs(dwt).max(), 1e-30))
        e_v = float(np.abs(out["dw_vis"][i].double().cpu().numpy() - dwv).max() / max(np.abs(dwv).max(), 1e-30))
        say("  %s: rel err dx %.2e dw_text %.2e dw_vis %.2e" % (s, e_x, e_t, e_v))
        tol = TOL[cfg.dtype]
        assert e_x <= tol and e_t <= tol and (cfg.n_vis == 0 or e_v <= tol)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,h", [("video_5s_480x832", 7), ("image_4096px", 2)])
def test_conv_backward_at_full_size_one_head(name, h):
    """kda_conv_backward over a whole workload stream (every channel, in the launch
    configuration of bench.py --backward): the input and tap gradients of one head's
    channels of q, k and v against the adjoint oracle run on those channels alone (the
    conv is depthwise).  The 4096x4096 image is a single latent slice, so its tap
    gradients sum every tap over 65 536 tokens and its mirrored-tap conv takes the
    single-slice path."""
    from linear_attention_sequence_modality_amd.inputs import WORKLOAD

    cfg = WORKLOAD[name]
    say("case %s conv backward head %d B=%d T=%d H=%d d=%d %s" % (name, h, cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dtype))
    host = make_inputs(cfg)
    g = np.random.default_rng(cfg.seed + 7)
    dys = {s: torch.from_numpy(g.standard_normal(tuple(host[s].shape)).astype(np.float32)).to(cfg.torch_dtype)
           for s in ("q", "k", "v")}
    dev = {k: v.cuda() for k, v in host.items()}
    out = kda.kda_conv_backward(desc_of(cfg), dev["q"], dev["k"], dev["v"],
                                (dev["w_text_q"], dev["w_text_k"], dev["w_text_v"]),
                                (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"]),
                                dys["q"].cuda(), dys["k"].cuda(), dys["v"].cuda())
    torch.cuda.synchronize()
    for i, s in enumerate(("q", "k", "v")):
        B, T, H, d = host[s].shape
        ch = slice(h * d, (h + 1) * d)
        dx, dwt, dwv = ob.short_conv_backward(host[s][:, :, h], host["w_text_" + s][ch], host["w_vis_" + s][ch],
                                              dys[s][:, :, h], cfg.n_text, cfg.grid, cfg.causal_t)
        e_x = rel(out["d" + s][:, :, h:h + 1].double().cpu().numpy(), dx[:, :, None, :])
        gwt = out["dw_text"][i][ch].double().cpu().numpy()
        gwv = out["dw_vis"][i][ch].double().cpu().numpy()
        e_t = float(np.abs(gwt - dwt).max() / max(np.abs(dwt).max(), 1e-30))
        e_v = float(np.abs(gwv - dwv).max() / max(np.abs(dwv).max(), 1e-30))
        say("  %s: rel err dx %.2e dw_text %.2e dw_vis %.2e" % (s, e_x, e_t, e_v))
        tol = TOL[cfg.dtype]
        assert np.isfinite(gwt).all() and np.isfinite(gwv).all()
        assert e_x <= tol and e_t <= tol and e_v <= tol


@pytest.mark.timeout(300)
def test_conv_and_kda_backward_chain_matches_the_oracle():
    """kda_backward then kda_conv_backward: the gradients of the conv inputs, the taps,
    alpha, beta and the initial state of the whole mixer."""
    cfg = StreamConfig("chain", B=1, H=2, dk=64, dv=64, n_text=6, grid=(2, 4, 5), dtype="f32", seed=95)
    say("case chain T=%d" % cfg.T)
    host = make_inputs(cfg)
    g = np.random.default_rng(5)
    dO = torch.from_numpy(g.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dv)).astype(np.float32))
    S0 = torch.from_numpy((g.standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)) * 0.3).astype(np.float32))
    dev = {k: v.cuda() for k, v in host.items()}
    d = desc_of(cfg)
    wt = (dev["w_text_q"], dev["w_text_k"], dev["w_text_v"])
    wv = (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"])
    qc, kc, vc = kda.kda_conv_forward(d, dev["q"], dev["k"], dev["v"], wt, wv)
    gk = kda.kda_backward(d, qc, kc, vc, dev["alpha"], dev["beta"], dO.cuda(), initial_state=S0.cuda())
    gc = kda.kda_conv_backward(d, dev["q"], dev["k"], dev["v"], wt, wv, gk["dq"], gk["dk"], gk["dv"])
    torch.cuda.synchronize()
    ref = ob.conv_kda_backward(host, cfg.n_text, cfg.grid, dO, 0, S0)
    errs = {"dq": rel(gc["dq"].double().cpu().numpy(), ref["dq"]),
            "dk": rel(gc["dk"].double().cpu().numpy(), ref["dk"]),
            "dv": rel(gc["dv"].double().cpu().numpy(), ref["dv"]),
            "dalpha": rel(gk["dalpha"].double().cpu().numpy(), ref["dalpha"]),
            "dbeta": rel(gk["dbeta"].double().cpu().numpy()[..., None], ref["dbeta"][..., None]),
            "dS0": oracle.rel_err_state(gk["d_initial_state"].double().cpu().numpy(), ref["dS0"])}
    for i, s in enumerate(("q", "k", "v")):
        for kind, idx in (("dw_text_", 0), ("dw_vis_", 1)):
            got = (gc["dw_text"] if idx == 0 else gc["dw_vis"])[i].double().cpu().numpy()
            want = ref[kind + s]
            errs[kind + s] = float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-30))
    say("  chain rel errors: " + ", ".join("%s %.1e" % kv for kv in errs.items()))
    for name, e in errs.items():
        assert e <= TOL["f32"], name


def test_backward_at_the_video_workload_is_exact_along_q_and_v():
    """At the full 5 s 480x832 stream (B=1, T=33272, H=16, d=128, bf16), in the launch
    configuration bench.py times: o is linear in q, and in v for fixed k, alpha and beta, so
    L = sum(dO * o) changes by exactly <dq, dq_step> (and <dv, dv_step>) along a step in q (v).
    Both gradients depend on every chunk of the ordered passes (dq on the states, dv on the
    state gradients).  Steps over the whole stream, steps confined to single chunks (q: the
    identity then holds per token and head), and a step along dv in one chunk; all within
    bf16 output rounding."""
    from linear_attention_sequence_modality_amd.inputs import WORKLOAD

    cfg = WORKLOAD["video_5s_480x832"]
    say("case video_5s_480x832 B=%d T=%d H=%d d=%d %s" % (cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dtype))
    inp = {k: v.cuda() for k, v in make_inputs(cfg).items()}
    desc = kda.make_desc(cfg.n_text, cfg.grid, causal_t=cfg.causal_t)
    g = torch.Generator(device="cpu").manual_seed(96)
    d_o = torch.randn(cfg.B, cfg.T, cfg.H, cfg.dv, generator=g).to(cfg.torch_dtype).cuda()
    q, k, v, al, be = inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"]
    grads = kda.kda_backward(desc, q, k, v, al, be, d_o)

    o_base = kda.kda_forward(desc, q, k, v, al, be)
    n_chunks = (cfg.T + 63) // 64

    def stepped(x, step):
        x2 = (x.float() + step.float()).to(x.dtype)
        return x2, x2.double() - x.double()             # the step the bf16 inputs really take

    # steps over the whole stream: dL = <dq, step> (<dv, step>)
    for name in ("q", "v"):
        x, dx = (q, grads["dq"]) if name == "q" else (v, grads["dv"])
        x2, st = stepped(x, (0.5 * torch.randn(x.shape, generator=g)).to(x.dtype).cuda())
        o2 = kda.kda_forward(desc, x2, k, v, al, be) if name == "q" else kda.kda_forward(desc, q, k, x2, al, be)
        lhs = (d_o.double() * (o2.double() - o_base.double())).sum().item()
        rhs = (dx.double() * st).sum().item()
        e = abs(lhs - rhs) / abs(rhs)
        say("  %s step on all chunks: dL %.6e, <d%s, step> %.6e, rel err %.2e" % (name, lhs, name, rhs, e))
        assert e <= TOL[cfg.dtype]
    # q steps confined to single chunks (first, middle, last): o_t moves by S_t^T step_t, so the
    # identity holds per token and head, <dO_t, o2_t - o_t> = <dq_t, step_t>, compared as vectors
    for chunk in (0, n_chunks // 2, n_chunks - 1):
        t0, t1 = 64 * chunk, min(cfg.T, 64 * chunk + 64)
        step = torch.zeros_like(q)
        step[:, t0:t1] = (0.5 * torch.randn(step[:, t0:t1].shape, generator=g)).to(q.dtype).cuda()
        x2, st = stepped(q, step)
        o2 = kda.kda_forward(desc, x2, k, v, al, be)
        lhs = (d_o[:, t0:t1].double() * (o2[:, t0:t1].double() - o_base[:, t0:t1].double())).sum(-1)
        rhs = (grads["dq"][:, t0:t1].double() * st[:, t0:t1]).sum(-1)
        e = ((lhs - rhs).norm() / rhs.norm()).item()
        say("  q step on chunk %d: per token-head rel err %.2e over %d pairs" % (chunk, e, rhs.numel()))
        assert e <= TOL[cfg.dtype]
    # v step confined to the middle chunk, along dv there: dL = <dv, step> > 0 without cancellation
    chunk = n_chunks // 2
    t0, t1 = 64 * chunk, 64 * chunk + 64
    dvc = grads["dv"][:, t0:t1].float()
    step = torch.zeros_like(v)
    step[:, t0:t1] = (0.5 * dvc / dvc.abs().max()).to(v.dtype)
    x2, st = stepped(v, step)
    o2 = kda.kda_forward(desc, q, k, x2, al, be)
    lhs = (d_o[:, t0:].double() * (o2[:, t0:].double() - o_base[:, t0:].double())).sum().item()
    rhs = (grads["dv"].double() * st).sum().item()
    e = abs(lhs - rhs) / abs(rhs)
    say("  v step along dv on chunk %d: dL %.6e, <dv, step> %.6e, rel err %.2e" % (chunk, lhs, rhs, e))
    assert e <= TOL[cfg.dtype]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,h", [("video_5s_480x832", 5), ("image_4096px", 11)])
def test_backward_at_full_size_one_head_against_the_oracle(name, h):
    """Every gradient (dq, dk, dv, dalpha, dbeta, dS0) of one sampled head of a full workload
    stream (the 5 s 480x832 video, T=33272, 520 chunks; the 4096x4096 image, T=66048, 1032
    chunks; H=16, d=128, bf16), with an initial state and a final-state gradient, in the
    launch configuration bench.py times, against the fp64 adjoint oracle run on that head
    alone (heads are independent)."""
    from linear_attention_sequence_modality_amd.inputs import WORKLOAD

    cfg = WORKLOAD[name]
    say("case %s backward head %d B=%d T=%d H=%d d=%d %s" % (name, h, cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dtype))
    host = make_inputs(cfg)
    g = np.random.default_rng(97)
    dO = torch.from_numpy(g.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dv)).astype(np.float32)).to(cfg.torch_dtype)
    S0 = torch.from_numpy((g.standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)) * 0.3).astype(np.float32))
    dST = torch.from_numpy(g.standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)).astype(np.float32))
    dev = {k: v.cuda() for k, v in host.items()}
    out = kda.kda_backward(desc_of(cfg), dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dO.cuda(),
                           initial_state=S0.cuda(), d_final_state=dST.cuda())
    torch.cuda.synchronize()
    sl = slice(h, h + 1)
    ref = ob.kda_recurrence_backward(host["q"][:, :, sl], host["k"][:, :, sl], host["v"][:, :, sl],
                                     host["alpha"][:, :, sl], host["beta"][:, :, sl], dO[:, :, sl],
                                     S0[:, sl], dST[:, sl])
    errs = {}
    for name in ("dq", "dk", "dv", "dalpha"):
        got = out[name][:, :, sl].double().cpu().numpy()
        assert np.isfinite(got).all()
        errs[name] = rel(got, ref[name])
    errs["dbeta"] = rel(out["dbeta"][:, :, sl].double().cpu().numpy()[..., None], ref["dbeta"][..., None])
    errs["dS0"] = oracle.rel_err_state(out["d_initial_state"][:, sl].double().cpu().numpy(), ref["dS0"])
    say("  rel errors: " + ", ".join("%s %.2e" % kv for kv in errs.items()))
    for name, e in errs.items():
        assert e <= TOL[cfg.dtype], "%s rel err %.3e" % (name, e)
