"""MLA attention core, HIP path vs the fp64 oracle (needs an MI355X).

Gate: max relative error per (batch, head) over max |ref| <= 2e-2 (bf16 in and
out, fp32 accumulation).  Small streams are compared in full; the full-size
streams on sampled query rows of sampled heads (a query row depends on all keys
of its head only, so the oracle computes those rows alone).
"""
import numpy as np
import pytest
import torch

from oracle import mla as oracle_mla
from linear_attention_sequence_modality_amd import kda
from linear_attention_sequence_modality_amd.inputs import MLA_WORKLOAD, MlaConfig, make_mla_inputs, make_mla_latent_inputs

from gpu_common import TOL, rel, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

KEYS = ("q_nope", "q_dir", "k_nope", "k_dir", "v")


def _run(cfg, scale=None, rows=None, heads=None):
    say("case %s B=%d T=%d H=%d rows=%s heads=%s scale=%s" % (cfg.name, cfg.B, cfg.T, cfg.H,
                                                              None if rows is None else len(rows), heads, scale))
    host = make_mla_inputs(cfg)
    dev = {k: v.cuda() for k, v in host.items()}
    o = kda.mla_attention_forward(*[dev[k] for k in KEYS], scale=scale)
    torch.cuda.synchronize()
    ref = oracle_mla.mla_attention(*[host[k] for k in KEYS], scale=scale, rows=rows, heads=heads)
    got = o.double().cpu().numpy()
    if rows is not None:
        got = got[:, rows]
    if heads is not None:
        got = got[:, :, list(heads)]
    e = rel(got, ref)
    say("  rel err o %.2e" % e)
    assert e <= TOL["bf16"]
    return o


@pytest.mark.timeout(120)
@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 128, 129, 333, 700])
def test_small_streams(T):
    _run(MlaConfig("mla_T%d" % T, B=2, T=T, H=2, seed=30 + T))


@pytest.mark.timeout(120)
@pytest.mark.parametrize("scale", [0.02, 0.25, 1.0])
def test_flat_and_peaked_softmax(scale):
    """From nearly uniform weights to scores spread over tens of units (the online
    maximum then moves often and far)."""
    _run(MlaConfig("mla_scale", B=1, T=517, H=3, seed=41), scale=scale)


@pytest.mark.timeout(120)
def test_batches_do_not_mix():
    """Each batch's queries see only that batch's keys: a batch changed alone
    leaves the other batches' outputs bit for bit unchanged."""
    cfg = MlaConfig("mla_mix", B=3, T=200, H=2, seed=43)
    dev = {k: v.cuda() for k, v in make_mla_inputs(cfg).items()}
    o1 = kda.mla_attention_forward(*[dev[k] for k in KEYS])
    dev["k_dir"][1] += 1.0
    dev["v"][1] *= 2.0
    o2 = kda.mla_attention_forward(*[dev[k] for k in KEYS])
    torch.cuda.synchronize()
    assert torch.equal(o1[0], o2[0]) and torch.equal(o1[2], o2[2])
    assert not torch.equal(o1[1], o2[1])


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,heads", [("mla_image_1024px", (0, 3)), ("mla_video_5s_480x832", (2, 13))])
def test_full_size_sampled(name, heads):
    cfg = MLA_WORKLOAD[name]
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 1, 127, 128, cfg.T - 1] + [int(x) for x in rng.integers(0, cfg.T, 59)]))
    _run(cfg, rows=rows, heads=heads)


@pytest.mark.timeout(120)
def test_deterministic():
    cfg = MLA_WORKLOAD["mla_tiny"]
    dev = {k: v.cuda() for k, v in make_mla_inputs(cfg).items()}
    a = kda.mla_attention_forward(*[dev[k] for k in KEYS])
    b = kda.mla_attention_forward(*[dev[k] for k in KEYS])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.timeout(120)
def test_ragged_tail_reads_nothing_past_the_stream_and_writes_only_o():
    """Inputs sit in buffers padded with NaN right after their last token: a key
    tile that ran past the end and used what it read would turn o into NaN.  The
    output's guard bands must keep their canary."""
    cfg = MlaConfig("mla_guard", B=2, T=65, H=2, seed=47)
    host = make_mla_inputs(cfg)
    pad = 1 << 14

    def guarded(t, fill):
        buf = torch.full((t.numel() + 2 * pad,), fill, dtype=t.dtype, device="cuda")
        view = buf[pad:pad + t.numel()].view(t.shape)
        view.copy_(t.cuda())
        return buf, view

    ins = {k: guarded(host[k], float("nan")) for k in KEYS}
    ob, o = guarded(torch.zeros_like(host["v"]), 3.0)
    kda.mla_attention_forward(*[ins[k][1] for k in KEYS], o=o)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert torch.all(ob[:pad].float() == 3.0) and torch.all(ob[-pad:].float() == 3.0)
    ref = oracle_mla.mla_attention(*[host[k] for k in KEYS])
    e = rel(o.double().cpu().numpy(), ref)
    say("  guard rel err o %.2e" % e)
    assert e <= TOL["bf16"]


# ---- the latent path (mla_latent_forward) ----------------------------------------------

LATENT_W = ("w_dkv", "w_kr", "w_uk", "w_uv")


def _latent_check(cfg, host, got, rows=None):
    """got: (c, k_dir, k_nope, v) device tensors; compared with the fp64 oracle on token rows
    ``rows`` (default: all) under the gate metric, per head for k_nope and v."""
    x = host["x"] if rows is None else host["x"][:, rows]
    ref = oracle_mla.mla_latent(x, *[host[k] for k in LATENT_W], cfg.H)
    errs = []
    for name, g, r in zip(("c", "k_dir", "k_nope", "v"), got, ref):
        g = g.double().cpu().numpy()
        if rows is not None:
            g = g[:, rows]
        if g.ndim == 3:
            g, r = g[:, :, None], r[:, :, None]
        errs.append(rel(g, r))
        assert np.isfinite(g).all()
    say("  rel err c %.2e k_dir %.2e k_nope %.2e v %.2e" % tuple(errs))
    assert max(errs) <= TOL["bf16"]


@pytest.mark.timeout(120)
@pytest.mark.parametrize("name", ["mla_tiny", "mla_image_1024px"])
def test_latent_projections(name):
    cfg = MLA_WORKLOAD[name]
    say("case latent %s B=%d T=%d H=%d d_model=%d d_c=%d" % (cfg.name, cfg.B, cfg.T, cfg.H, cfg.model_width,
                                                            cfg.latent_width))
    host = make_mla_latent_inputs(cfg)
    dev = {k: v.cuda() for k, v in host.items()}
    got = kda.mla_latent_forward(dev["x"], *[dev[k] for k in LATENT_W], cfg.H)
    torch.cuda.synchronize()
    _latent_check(cfg, host, got)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("T", [1, 255, 256, 257, 511])
def test_latent_ragged_row_counts(T):
    """Row counts around the 256-row tile, at widths where the latent, K_direct, keys and
    values are one or a few 64-column tiles."""
    cfg = MlaConfig("latent_T%d" % T, B=1, T=T, H=1, seed=60 + T, d_model=96, d_c=64, d_nope=64, dv=64)
    say("case latent ragged T=%d" % T)
    host = make_mla_latent_inputs(cfg)
    dev = {k: v.cuda() for k, v in host.items()}
    got = kda.mla_latent_forward(dev["x"], *[dev[k] for k in LATENT_W], cfg.H)
    torch.cuda.synchronize()
    _latent_check(cfg, host, got)


@pytest.mark.timeout(300)
def test_latent_at_the_video_layer_size_sampled_rows():
    cfg = MLA_WORKLOAD["mla_video_5s_480x832"]
    say("case latent %s T=%d d_model=%d d_c=%d" % (cfg.name, cfg.T, cfg.model_width, cfg.latent_width))
    host = make_mla_latent_inputs(cfg)
    dev = {k: v.cuda() for k, v in host.items()}
    got = kda.mla_latent_forward(dev["x"], *[dev[k] for k in LATENT_W], cfg.H)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = sorted(set([0, 255, 256, cfg.T - 1] + [int(x) for x in rng.integers(0, cfg.T, 120)]))
    _latent_check(cfg, host, got, rows=rows)
    # and twice gives the same bits
    again = kda.mla_latent_forward(dev["x"], *[dev[k] for k in LATENT_W], cfg.H)
    torch.cuda.synchronize()
    for a, b in zip(got, again):
        assert torch.equal(a, b)


@pytest.mark.timeout(120)
def test_layer_from_hidden_states():
    """The whole MLA mixer from hidden states: latent projections then attention, against the
    oracle's layer (which decompresses from the unrounded latent)."""
    cfg = MLA_WORKLOAD["mla_tiny"]
    say("case mla layer %s" % cfg.name)
    host = make_mla_latent_inputs(cfg)
    dev = {k: v.cuda() for k, v in host.items()}
    o, _ = kda.mla_layer_forward(dev["x"], dev["q_nope"], dev["q_dir"], {k: dev[k] for k in LATENT_W})
    torch.cuda.synchronize()
    ref = oracle_mla.mla_layer(host["x"], host["q_nope"], host["q_dir"], *[host[k] for k in LATENT_W])
    e = rel(o.double().cpu().numpy(), ref)
    say("  rel err o %.2e" % e)
    assert e <= TOL["bf16"]


@pytest.mark.timeout(60)
def test_latent_refusals():
    """Host-side refusals, before any launch: fp32, a latent width off the 64-column tiling,
    a misaligned pointer."""
    cfg = MLA_WORKLOAD["mla_tiny"]
    host = make_mla_latent_inputs(cfg)
    dev = {k: v.cuda() for k, v in host.items()}
    with pytest.raises(kda.KdaError) as e:
        kda.mla_latent_forward(dev["x"].float(), *[dev[k].float() for k in LATENT_W], cfg.H)
    assert e.value.status == kda.KDA_ERR_UNSUPPORTED
    dm = cfg.model_width
    w_dkv = torch.zeros(96, dm, dtype=torch.bfloat16, device="cuda")
    w_uk = torch.zeros(cfg.H * cfg.d_nope, 96, dtype=torch.bfloat16, device="cuda")
    w_uv = torch.zeros(cfg.H * cfg.dv, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.mla_latent_forward(dev["x"], w_dkv, dev["w_kr"], w_uk, w_uv, cfg.H)
    assert e.value.status == kda.KDA_ERR_UNSUPPORTED
    buf = torch.empty(dev["x"].numel() + 8, dtype=torch.bfloat16, device="cuda")
    x_mis = buf[1:1 + dev["x"].numel()].view(dev["x"].shape)
    with pytest.raises(kda.KdaError) as e:
        kda.mla_latent_forward(x_mis, *[dev[k] for k in LATENT_W], cfg.H)
    assert e.value.status == kda.KDA_ERR_INVALID_ARG
