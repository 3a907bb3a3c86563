"""HIP path vs the fp64 oracle, element by element (needs an MI355X).

Gates (max relative error per (batch, head), over max |ref|): 1e-4 for fp32
streams, 2e-2 for bf16 streams.  Small streams are compared in full; the full
sized workloads are compared on every token of sampled heads (the conv is
depthwise and the scan is per head, so a head's outputs depend only on that
head's inputs and the oracle can compute them alone).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_modality_amd import kda
from linear_attention_sequence_modality_amd.inputs import WORKLOAD, StreamConfig, make_inputs

from gpu_common import (TOL, check_stream, desc_of, heads_slice, oracle_conv_heads, oracle_end_to_end_heads,
                        rel, run_path, say, to_dev)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# Every head of the 16 is compared on one of the three full-size workloads.
SAMPLED_HEADS = {"video_5s_480x832": (0, 3, 6, 9, 13), "image_4096px": (1, 4, 8, 11, 15),
                 "video_30s_480x832": (2, 5, 7, 10, 12, 14)}


def _check_stream(cfg, inp, heads=None, S0=None, want_state=False):
    return check_stream(cfg, inp, heads=heads, S0=S0, want_state=want_state)


def _check_kda_stage(cfg, inp, heads=None):
    """KDA alone on the generated (already normalised) q, k, v."""
    dev = to_dev(inp)
    o = kda.kda_forward(desc_of(cfg), dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"])
    torch.cuda.synchronize()
    heads = tuple(range(cfg.H)) if heads is None else heads
    ro, _ = oracle.kda_recurrence(heads_slice(inp["q"], heads), heads_slice(inp["k"], heads),
                                  heads_slice(inp["v"], heads), heads_slice(inp["alpha"], heads),
                                  heads_slice(inp["beta"][..., None], heads)[..., 0], want_state=False)
    e = rel(heads_slice(o, heads), ro)
    say("  kda stage %s rel err %.2e" % (cfg.name, e))
    assert e <= TOL[cfg.dtype]


# ---- the five stream workloads -------------------------------------------------

@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["tiny_fp32", "proxy_image_1024px"])
def test_workload_full(name):
    cfg = WORKLOAD[name]
    inp = make_inputs(cfg)
    _check_stream(cfg, inp)
    _check_kda_stage(cfg, inp)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(SAMPLED_HEADS))
def test_workload_sampled_heads(name):
    cfg = WORKLOAD[name]
    inp = make_inputs(cfg)
    _check_stream(cfg, inp, heads=SAMPLED_HEADS[name])
    _check_kda_stage(cfg, inp, heads=SAMPLED_HEADS[name][:1])


# ---- edge cases (small, compared in full) -----------------------------------------

def _small(name, **kw):
    base = dict(B=1, H=2, dk=128, dv=128, n_text=7, grid=(3, 5, 9), dtype="bf16", seed=77)
    base.update(kw)
    return StreamConfig(name, **base)


EDGE = [
    _small("tail_0", n_text=64, grid=(1, 8, 8)),              # T = 128: whole chunks
    _small("tail_1", n_text=1, grid=(1, 8, 8)),               # T = 65: one-token tail
    _small("tail_63", n_text=63, grid=(1, 8, 8)),             # T = 127
    _small("text_only", n_text=200, grid=(0, 0, 0)),
    _small("vision_only", n_text=0, grid=(2, 7, 11)),
    _small("single_token", n_text=1, grid=(0, 0, 0)),
    _small("single_visual_token", n_text=0, grid=(1, 1, 1)),
    _small("single_token_fp32", n_text=1, grid=(0, 0, 0), dk=64, dv=64, dtype="f32"),
    _small("image_grid_t1", n_text=3, grid=(1, 12, 20)),
    _small("batch3", B=3, n_text=5, grid=(2, 6, 7)),
    _small("causal_t", causal_t=1, grid=(4, 5, 6)),
    _small("dk64_dv128", dk=64, dv=128),
    _small("dk128_dv64", dk=128, dv=64),
    _small("bf16_64", dk=64, dv=64, H=3),
    _small("fp32_64", dk=64, dv=64, dtype="f32", grid=(2, 9, 13)),
    _small("fp32_causal", dk=64, dv=64, dtype="f32", causal_t=1, B=2),
    _small("fp32_128", dtype="f32", grid=(3, 9, 13)),
    _small("fp32_128_64", dk=128, dv=64, dtype="f32"),
    _small("fp32_64_128", dk=64, dv=128, dtype="f32", B=2),
    _small("narrow_w", grid=(3, 4, 1), n_text=2),             # grid_w = 1, ragged w-runs
    _small("wide_w", grid=(2, 2, 37), n_text=9),
    # single-slice grids take the conv's row-group march: several runs of 8 row
    # groups, a ragged last group, both paddings, both dtypes
    _small("image_tall", grid=(1, 70, 9), n_text=4),
    _small("image_causal", causal_t=1, grid=(1, 41, 23), n_text=2),
    _small("fp32_image", dk=64, dv=64, dtype="f32", grid=(1, 37, 19), n_text=5),
    _small("fp32_image_causal", dk=64, dv=64, dtype="f32", causal_t=1, grid=(1, 9, 9)),
]


@pytest.mark.timeout(120)
@pytest.mark.parametrize("cfg", EDGE, ids=[c.name for c in EDGE])
def test_edge_case(cfg):
    _check_stream(cfg, make_inputs(cfg))


@pytest.mark.timeout(120)
@pytest.mark.parametrize("name", ["single_token", "single_visual_token"])
def test_one_token_error_is_the_rounding_of_q_and_k(name):
    """A one-token bf16 stream with no initial state has o = beta (q'.k') v'.

    The dot product cancels: q'.k' is small next to sum |q'_i k'_i|, and the
    bf16 rounding of the stored q' and k' moves it by up to 2u times that sum
    (u = 2^-8). So against the fp64 oracle the error of o is the cancellation
    ratio kappa = sum |q'_i k'_i| / |q'.k'| times the rounding, and kappa, not
    the path, sets the error.

    Fed the oracle's own conv outputs rounded to bf16 (round to nearest even
    through fp32, as the path stores them), the oracle must agree with the path
    to the three roundings that are left: q'.k' and beta v' as operands of the
    product, and o itself. Each is at most u relative, so the gate is 3u, with no
    kappa in it."""
    cfg = next(c for c in EDGE if c.name == name)
    inp = make_inputs(cfg)
    qc, kc, vc, o, _ = run_path(cfg, to_dev(inp))
    heads = tuple(range(cfg.H))
    rq, rk, rv, ro, _ = oracle_end_to_end_heads(cfg, inp, heads)

    def bf16(x):
        return torch.from_numpy(x).float().bfloat16().double().numpy()

    beta = heads_slice(inp["beta"][..., None], heads)[..., 0]
    ro_r, _ = oracle.kda_recurrence(bf16(rq), bf16(rk), bf16(rv), heads_slice(inp["alpha"], heads), beta,
                                    want_state=False)
    oh = heads_slice(o, heads)
    u = 2.0 ** -8
    kappa = np.abs(rq * rk).sum(-1) / np.abs((rq * rk).sum(-1))          # [B, 1, H]
    e_full, e_round = rel(oh, ro), rel(oh, ro_r)
    say("  %s: kappa per head %s; o vs oracle %.2e (2 u kappa = %.2e), vs oracle on bf16 q', k', v' %.2e "
        "(gate 3u = %.2e)" % (name, np.array2string(kappa.ravel(), precision=1), e_full,
                              2 * u * kappa.max(), e_round, 3 * u))
    assert e_full <= TOL["bf16"]
    assert e_round <= 3 * u
    # the closed form the two oracles follow at T = 1
    closed = beta[..., None] * (rq * rk).sum(-1, keepdims=True) * rv
    assert np.allclose(ro, closed, rtol=1e-12, atol=1e-12 * np.abs(closed).max())


@pytest.mark.timeout(120)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_initial_and_final_state(dtype):
    cfg = _small("state_" + dtype, dk=64, dv=64, dtype=dtype, B=2, H=3, n_text=11, grid=(2, 6, 9))
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)) * 0.5
    _check_stream(cfg, make_inputs(cfg), S0=S0.astype(np.float32), want_state=True)


@pytest.mark.timeout(120)
def test_split_and_resume_matches_one_shot():
    """KDA over [0, T1) then [T1, T) with the carried state equals one pass."""
    cfg = _small("resume", dk=128, dv=128, H=2, n_text=0, grid=(1, 10, 19))   # T = 190
    inp = to_dev(make_inputs(cfg))
    T, T1 = cfg.T, 77
    d_all = kda.make_desc(T, (0, 0, 0))
    sT = torch.empty(cfg.B, cfg.H, cfg.dk, cfg.dv, device="cuda")
    o = kda.kda_forward(d_all, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], final_state=sT)
    part = {k: inp[k] for k in ("q", "k", "v", "alpha", "beta")}
    # clone: the library requires 16-byte aligned buffers, slices of beta are not
    first = {k: x[:, :T1].clone() for k, x in part.items()}
    second = {k: x[:, T1:].clone() for k, x in part.items()}
    s1 = torch.empty_like(sT)
    o1 = kda.kda_forward(kda.make_desc(T1, (0, 0, 0)), *[first[k] for k in ("q", "k", "v", "alpha", "beta")],
                         final_state=s1)
    s2 = torch.empty_like(sT)
    o2 = kda.kda_forward(kda.make_desc(T - T1, (0, 0, 0)), *[second[k] for k in ("q", "k", "v", "alpha", "beta")],
                         initial_state=s1, final_state=s2)
    torch.cuda.synchronize()
    oo = torch.cat([o1, o2], dim=1).double().cpu().numpy()
    e_o = rel(oo, o.double().cpu().numpy())
    e_s = oracle.rel_err_state(s2.double().cpu().numpy(), sT.double().cpu().numpy())
    say("  resume rel err o %.2e S %.2e" % (e_o, e_s))
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]


@pytest.mark.timeout(120)
@pytest.mark.parametrize("T,B", [(64 * 70 + 13, 1), (64 * 300 - 5, 2)])
def test_forward_equals_the_two_kernels(T, B):
    """kda_forward is kda_forward_chunks + kda_forward_scan: equal bit for bit,
    final state included, with an initial state that aliases the final one."""
    cfg = _small("pipe", B=B, n_text=T, grid=(0, 0, 0))
    say("case forward vs two kernels T=%d B=%d chunks=%d" % (T, B, (T + 63) // 64))
    inp = to_dev(make_inputs(cfg))
    d = desc_of(cfg)
    x = [inp[k] for k in ("q", "k", "v", "alpha", "beta")]
    g = torch.Generator().manual_seed(5)
    s0 = (torch.randn(cfg.B, cfg.H, cfg.dk, cfg.dv, generator=g) * 0.1).cuda()
    need = kda.kda_forward_workspace_size(d, cfg.B, cfg.H, cfg.dk, cfg.dv, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1 = torch.empty_like(inp["v"])
    s1 = torch.empty_like(s0)
    kda.kda_forward_chunks(d, *x, ws)
    kda.kda_forward_scan(d, cfg.B, cfg.H, cfg.dk, cfg.dv, torch.bfloat16, ws, o1, initial_state=s0,
                         final_state=s1)
    o2 = torch.full_like(inp["v"], float("nan"))
    s2 = s0.clone()                       # initial state, overwritten in place by the final state
    kda.kda_forward(d, *x, initial_state=s2, final_state=s2, o=o2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2)
    # and the two-kernel path itself against the oracle on one head
    host = make_inputs(cfg)
    ro, _ = oracle.kda_recurrence(*[heads_slice(host[k], (1,)) for k in ("q", "k", "v", "alpha")],
                                  heads_slice(host["beta"][..., None], (1,))[..., 0],
                                  S0=s0[:, 1:2].double().cpu().numpy(), want_state=False)
    e = rel(heads_slice(o2, (1,)), ro)
    say("  forward rel err o %.2e" % e)
    assert e <= TOL["bf16"]


@pytest.mark.timeout(120)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_time_causal_stream_in_segments_equals_one_pass(dtype):
    """A time-causal stream cut along t into segments (text in the first only):
    each segment's conv, given the inputs of the two latent slices before it
    (kda_conv_forward_stream), equals the same slices of the one-pass conv bit
    for bit, and KDA over the segments with the carried state matches the
    oracle of the whole stream."""
    kw = dict(dk=64, dv=64) if dtype == "f32" else {}
    cfg = _small("stream", B=2, n_text=5, grid=(8, 6, 9), causal_t=1, dtype=dtype, **kw)
    say("case stream in segments %s T=%d" % (dtype, cfg.T))
    host = make_inputs(cfg)
    dev = to_dev(host)
    wt = (dev["w_text_q"], dev["w_text_k"], dev["w_text_v"])
    wv = (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"])
    whole = kda.kda_conv_forward(desc_of(cfg), dev["q"], dev["k"], dev["v"], wt, wv)
    gt, gh, gw = cfg.grid
    sl = gh * gw
    cuts = [0, 3, 5, 8]                      # latent slices of each segment
    state = None
    outs = []
    for i in range(3):
        t0, t1 = cuts[i], cuts[i + 1]
        lo = 0 if i == 0 else cfg.n_text + t0 * sl
        hi = cfg.n_text + t1 * sl
        seg = {k: dev[k][:, lo:hi].contiguous() for k in ("q", "k", "v", "alpha", "beta")}
        if i == 0:
            d = kda.make_desc(cfg.n_text, (t1, gh, gw), causal_t=1)
            conv = kda.kda_conv_forward(d, seg["q"], seg["k"], seg["v"], wt, wv)
        else:
            d = kda.make_desc(0, (t1 - t0, gh, gw), causal_t=1)
            hlo = cfg.n_text + (t0 - 2) * sl
            hist = [dev[k][:, hlo:lo].contiguous() for k in ("q", "k", "v")]
            conv = kda.kda_conv_forward(d, seg["q"], seg["k"], seg["v"], wt, wv, history=hist)
        for c, w in zip(conv, whole):
            assert torch.equal(c, w[:, lo:hi])
        fin = torch.empty(cfg.B, cfg.H, cfg.dk, cfg.dv, device="cuda")
        outs.append(kda.kda_forward(d, *conv, seg["alpha"], seg["beta"], initial_state=state, final_state=fin))
        state = fin
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1)
    heads = tuple(range(cfg.H))
    _, _, _, ro, rs = oracle_end_to_end_heads(cfg, host, heads)
    e_o = rel(heads_slice(o, heads), ro)
    e_s = oracle.rel_err_state(state.double().cpu().numpy(), rs)
    say("  segments rel err o %.2e S %.2e" % (e_o, e_s))
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype]


def _varlen_run(cfgs, s0_scale=0.3):
    """Pack the streams' inputs (sharing the first stream's conv weights) and run the
    variable-length conv and KDA; also run each stream alone.  Returns what the checks need."""
    hosts = [make_inputs(c) for c in cfgs]
    for h in hosts[1:]:
        for w in ("w_text_q", "w_text_k", "w_text_v", "w_vis_q", "w_vis_k", "w_vis_v"):
            h[w] = hosts[0][w]
    devs = [to_dev(h) for h in hosts]
    d0 = devs[0]
    wt = (d0["w_text_q"], d0["w_text_k"], d0["w_text_v"])
    wv = (d0["w_vis_q"], d0["w_vis_k"], d0["w_vis_v"])
    descs = [desc_of(c) for c in cfgs]
    pack = {k: torch.cat([d[k][0] for d in devs], dim=0).contiguous() for k in ("q", "k", "v", "alpha", "beta")}
    c0 = cfgs[0]
    g = torch.Generator().manual_seed(11)
    s0 = (torch.randn(len(cfgs), c0.H, c0.dk, c0.dv, generator=g) * s0_scale).cuda()
    sT = torch.empty_like(s0)
    qc, kc, vc = kda.kda_conv_forward_varlen(descs, pack["q"], pack["k"], pack["v"], wt, wv)
    o = kda.kda_forward_varlen(descs, qc, kc, vc, pack["alpha"], pack["beta"], initial_state=s0, final_state=sT)
    alone = []
    for i, (c, d) in enumerate(zip(cfgs, devs)):
        cq, ck, cv = kda.kda_conv_forward(descs[i], d["q"], d["k"], d["v"], wt, wv)
        st = torch.empty(1, c.H, c.dk, c.dv, device="cuda")
        oi = kda.kda_forward(descs[i], cq, ck, cv, d["alpha"], d["beta"], initial_state=s0[i:i + 1].contiguous(),
                             final_state=st)
        alone.append((cq, ck, cv, oi, st))
    torch.cuda.synchronize()
    return hosts, s0, (qc, kc, vc, o, sT), alone


@pytest.mark.timeout(120)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_batch_equals_each_stream_alone(dtype):
    """A batch mixing a video, a text-only stream, a one-chunk image, a time-causal
    video and a one-token stream: each stream's conv outputs, o and final state equal
    those of the stream run alone, bit for bit, and match the oracle."""
    kw = dict(dk=64, dv=64) if dtype == "f32" else {}
    cfgs = [_small("vl_video", n_text=7, grid=(3, 5, 9), dtype=dtype, seed=1, **kw),
            _small("vl_text", n_text=200, grid=(0, 0, 0), dtype=dtype, seed=2, **kw),
            _small("vl_image", n_text=0, grid=(1, 8, 8), dtype=dtype, seed=3, **kw),
            _small("vl_causal", n_text=3, grid=(2, 6, 7), causal_t=1, dtype=dtype, seed=4, **kw),
            _small("vl_one", n_text=1, grid=(0, 0, 0), dtype=dtype, seed=5, **kw)]
    say("case varlen %s T=%s" % (dtype, [c.T for c in cfgs]))
    hosts, s0, packed, alone = _varlen_run(cfgs)
    qc, kc, vc, o, sT = packed
    tok = 0
    heads = tuple(range(cfgs[0].H))
    for i, (c, h, al) in enumerate(zip(cfgs, hosts, alone)):
        sl = slice(tok, tok + c.T)
        for x, y in zip((qc, kc, vc, o), al[:4]):
            assert torch.equal(x[sl], y[0]), (c.name, "packed != alone")
        assert torch.equal(sT[i:i + 1], al[4]), (c.name, "state")
        _, _, _, ro, rs = oracle_end_to_end_heads(c, h, heads, s0[i:i + 1].double().cpu().numpy())
        e_o = rel(heads_slice(o[sl][None], heads), ro)
        e_s = oracle.rel_err_state(sT[i:i + 1].double().cpu().numpy(), rs)
        say("  %s T=%d rel err o %.2e S %.2e" % (c.name, c.T, e_o, e_s))
        assert e_o <= TOL[dtype] and e_s <= TOL[dtype]
        tok += c.T


@pytest.mark.timeout(120)
def test_varlen_batch_of_the_most_streams():
    """KDA_MAX_SEQS text streams of ragged lengths (1 to 150 tokens): every stream's o
    and final state equal its own call."""
    rng = np.random.default_rng(9)
    lens = [int(x) for x in rng.integers(1, 151, size=kda.KDA_MAX_SEQS)]
    lens[0], lens[-1] = 64, 1
    cfgs = [_small("vl_%d" % i, n_text=n, grid=(0, 0, 0), H=1, seed=100 + i) for i, n in enumerate(lens)]
    say("case varlen %d streams, %d tokens" % (len(cfgs), sum(lens)))
    _, _, packed, alone = _varlen_run(cfgs)
    o, sT = packed[3], packed[4]
    tok = 0
    for i, (c, al) in enumerate(zip(cfgs, alone)):
        assert torch.equal(o[tok:tok + c.T], al[3][0]), c.name
        assert torch.equal(sT[i:i + 1], al[4]), c.name
        tok += c.T


@pytest.mark.timeout(120)
def test_graph_capture_replays_match_eager():
    """The measured step (conv, chunk kernel, state pass) allocates, synchronises and
    clears nothing inside the library, so it can be captured in a HIP graph: three
    replays, with eager work and synchronisations between them, each equal the eager
    result bit for bit."""
    cfg = _small("graph", B=1, n_text=40, grid=(4, 9, 13))
    say("case graph capture T=%d" % cfg.T)
    dev = to_dev(make_inputs(cfg))
    d = desc_of(cfg)
    wt = (dev["w_text_q"], dev["w_text_k"], dev["w_text_v"])
    wv = (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"])
    qc, kc, vc = (torch.empty_like(dev[s]) for s in ("q", "k", "v"))
    o = torch.empty_like(dev["v"])
    sT = torch.empty(cfg.B, cfg.H, cfg.dk, cfg.dv, device="cuda")
    ws = torch.empty(kda.kda_forward_workspace_size(d, cfg.B, cfg.H, cfg.dk, cfg.dv, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def step(stream=None):
        kda.kda_conv_forward(d, dev["q"], dev["k"], dev["v"], wt, wv, qc, kc, vc, stream=stream)
        kda.kda_forward(d, qc, kc, vc, dev["alpha"], dev["beta"], final_state=sT, o=o, workspace=ws,
                        stream=stream)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (qc, kc, vc, o, sT)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)            # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for rep in range(3):
        for x in (qc, kc, vc, o, sT):
            x.fill_(float("nan"))        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, r in zip((qc, kc, vc, o, sT), ref):
            assert torch.equal(x, r), "replay %d differs from eager" % rep


@pytest.mark.timeout(120)
def test_wrapper_allocations_on_a_side_stream():
    """The binding allocates o, the conv outputs and the workspace on the current stream;
    launched on a side stream that is not made current, the kernels must still own that
    memory until they are done.  Allocations on the current stream right after the call
    (which would reuse freed blocks) must not disturb the result."""
    cfg = WORKLOAD["proxy_image_1024px"].with_(name="side_stream", B=2)
    say("case side stream T=%d B=%d" % (cfg.T, cfg.B))
    dev = to_dev(make_inputs(cfg))
    d = desc_of(cfg)
    ref = kda.conv_kda_forward(d, dev)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    got = kda.conv_kda_forward(d, dev, stream=side)
    churn = []
    for _ in range(8):   # fill freed blocks on the current stream with NaN
        churn.append(torch.full((64 << 20,), float("nan"), device="cuda"))
    side.synchronize()
    torch.cuda.synchronize()
    del churn
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


# ---- hygiene -----------------------------------------------------------------------

@pytest.mark.timeout(120)
def test_deterministic_and_every_output_written():
    cfg = _small("hygiene", B=2, n_text=13, grid=(3, 7, 10))
    dev = to_dev(make_inputs(cfg))
    d = desc_of(cfg)
    runs = []
    for poison in (float("nan"), 12345.0):
        q2 = torch.full_like(dev["q"], poison)
        k2 = torch.full_like(dev["k"], poison)
        v2 = torch.full_like(dev["v"], poison)
        kda.kda_conv_forward(d, dev["q"], dev["k"], dev["v"],
                             (dev["w_text_q"], dev["w_text_k"], dev["w_text_v"]),
                             (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"]), q2, k2, v2)
        need = kda.kda_forward_workspace_size(d, cfg.B, cfg.H, cfg.dk, cfg.dv, torch.bfloat16)
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")    # NaN bit patterns
        o = torch.full_like(dev["v"], poison)
        kda.kda_forward(d, q2, k2, v2, dev["alpha"], dev["beta"], o=o, workspace=ws)
        torch.cuda.synchronize()
        for t in (q2, k2, v2, o):
            assert torch.isfinite(t.float()).all()
        runs.append([t.clone() for t in (q2, k2, v2, o)])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


@pytest.mark.timeout(300)
def test_conv_repeatable_with_the_chip_full():
    """The conv's tile pipeline at a size that keeps several blocks resident per CU
    for many t-steps (a multi-frame 30 x 52 grid, 16 heads of 128): two runs into
    poisoned outputs agree bit for bit, and sampled heads match the oracle."""
    cfg = WORKLOAD["video_5s_480x832"].with_(name="video_8f", grid=(8, 30, 52))
    inp = make_inputs(cfg)
    dev = to_dev(inp)
    d = desc_of(cfg)
    say("case %s T=%d H=%d" % (cfg.name, cfg.T, cfg.H))
    runs = []
    for poison in (float("nan"), -3.0):
        outs = [torch.full_like(dev[x], poison) for x in ("q", "k", "v")]
        kda.kda_conv_forward(d, dev["q"], dev["k"], dev["v"],
                             (dev["w_text_q"], dev["w_text_k"], dev["w_text_v"]),
                             (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"]), *outs)
        torch.cuda.synchronize()
        runs.append(outs)
    for a, b in zip(*runs):
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a, b)
    heads = (3, 14)
    for name, got in zip(("q", "k", "v"), runs[0]):
        e = rel(heads_slice(got, heads), oracle_conv_heads(cfg, inp, name, heads))
        say("  %s rel err %.2e" % (name, e))
        assert e <= TOL[cfg.dtype]


@pytest.mark.timeout(120)
def test_no_writes_outside_outputs():
    cfg = _small("guard", n_text=9, grid=(2, 5, 6), dk=64, dv=128)
    dev = to_dev(make_inputs(cfg))
    d = desc_of(cfg)
    pad = 4096
    canary = 77.0

    def guarded(like):
        buf = torch.full((like.numel() + 2 * pad,), canary, dtype=like.dtype, device="cuda")
        return buf, buf[pad:pad + like.numel()].view(like.shape)

    bufs = [guarded(dev[s]) for s in ("q", "k", "v")]
    kda.kda_conv_forward(d, dev["q"], dev["k"], dev["v"],
                         (dev["w_text_q"], dev["w_text_k"], dev["w_text_v"]),
                         (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"]), *[b[1] for b in bufs])
    ob, o = guarded(dev["v"])
    need = kda.kda_forward_workspace_size(d, cfg.B, cfg.H, cfg.dk, cfg.dv, torch.bfloat16)
    wsb = torch.full((need + 2 * pad,), 0x5A, dtype=torch.uint8, device="cuda")
    sb = torch.full((cfg.B * cfg.H * cfg.dk * cfg.dv + 2 * pad,), canary, device="cuda")
    sT = sb[pad:pad + cfg.B * cfg.H * cfg.dk * cfg.dv].view(cfg.B, cfg.H, cfg.dk, cfg.dv)
    kda.kda_forward(d, bufs[0][1], bufs[1][1], bufs[2][1], dev["alpha"], dev["beta"], final_state=sT,
                    o=o, workspace=wsb[pad:pad + need])
    torch.cuda.synchronize()
    for buf, _ in bufs + [(ob, None)]:
        assert torch.all(buf[:pad].float() == canary) and torch.all(buf[-pad:].float() == canary)
    assert torch.all(wsb[:pad] == 0x5A) and torch.all(wsb[-pad:] == 0x5A)
    assert torch.all(sb[:pad] == canary) and torch.all(sb[-pad:] == canary)
