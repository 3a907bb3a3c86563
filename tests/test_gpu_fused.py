"""kda_conv_kda_forward (the conv inside the chunk transform) against the oracle and
against the two-call path kda_conv_forward + kda_forward (needs an MI355X).

The fused call forms q', k', v' inside the chunk transform instead of reading them,
so its o must match the oracle of conv then KDA at the dtype's tolerance (R13), and
the two-call path to the rounding of q', k', v' (the two sum the taps in different
orders, so a conv output can differ in its last bf16 bit).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_modality_amd import kda
from linear_attention_sequence_modality_amd.inputs import WORKLOAD, StreamConfig, make_inputs

from gpu_common import TOL, desc_of, heads_slice, oracle_end_to_end_heads, rel, rel_elem, say, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _fused(cfg, dev, S0=None, want_state=True, workspace=None):
    sT = torch.empty(cfg.B, cfg.H, cfg.dk, cfg.dv, device="cuda") if want_state else None
    s0 = None if S0 is None else torch.as_tensor(S0, dtype=torch.float32).cuda().contiguous()
    wt = (dev["w_text_q"], dev["w_text_k"], dev["w_text_v"])
    wv = (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"])
    o = kda.kda_conv_kda_forward(desc_of(cfg), dev["q"], dev["k"], dev["v"], wt, wv, dev["alpha"], dev["beta"],
                                 initial_state=s0, final_state=sT, workspace=workspace)
    torch.cuda.synchronize()
    return o, sT


def _two_call(cfg, dev, S0=None):
    sT = torch.empty(cfg.B, cfg.H, cfg.dk, cfg.dv, device="cuda")
    s0 = None if S0 is None else torch.as_tensor(S0, dtype=torch.float32).cuda().contiguous()
    _, _, _, o = kda.conv_kda_forward(desc_of(cfg), dev, initial_state=s0, final_state=sT)
    torch.cuda.synchronize()
    return o, sT


def _check(cfg, S0=None, heads=None):
    say("case %s B=%d T=%d H=%d dk=%d dv=%d %s causal_t=%d" % (cfg.name, cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv,
                                                              cfg.dtype, cfg.causal_t))
    inp = make_inputs(cfg)
    dev = to_dev(inp)
    o, sT = _fused(cfg, dev, S0)
    o2, sT2 = _two_call(cfg, dev, S0)
    heads = tuple(range(cfg.H)) if heads is None else heads
    _, _, _, ro, rs = oracle_end_to_end_heads(cfg, inp, heads, S0)
    oh = heads_slice(o, heads)
    e_o = rel(oh, ro)
    e_s = oracle.rel_err_state(sT[:, list(heads)].double().cpu().numpy(), rs)
    e_2 = rel(o.double().cpu().numpy(), o2.double().cpu().numpy())
    e_s2 = oracle.rel_err_state(sT.double().cpu().numpy(), sT2.double().cpu().numpy())
    say("  fused vs oracle: o %.2e, S_T %.2e [o elementwise %.2e]; fused vs two calls: o %.2e, S_T %.2e"
        % (e_o, e_s, rel_elem(oh, ro), e_2, e_s2))
    assert np.isfinite(oh).all()
    assert e_o <= TOL[cfg.dtype] and e_s <= TOL[cfg.dtype]
    assert e_2 <= TOL[cfg.dtype] and e_s2 <= TOL[cfg.dtype]
    return e_2


CASES = [
    StreamConfig("fused_f32", B=2, H=2, dk=64, dv=64, n_text=11, grid=(2, 6, 9), dtype="f32", seed=301),
    StreamConfig("fused_f32_128", B=1, H=2, dk=128, dv=128, n_text=21, grid=(3, 5, 7), dtype="f32", seed=302),
    StreamConfig("fused_f32_128_64", B=1, H=1, dk=128, dv=64, n_text=5, grid=(3, 4, 11), dtype="f32", seed=303),
    StreamConfig("fused_bf16", B=1, H=2, dk=128, dv=128, n_text=7, grid=(3, 5, 9), dtype="bf16", seed=304),
    StreamConfig("fused_bf16_64_128", B=2, H=3, dk=64, dv=128, n_text=40, grid=(4, 7, 6), dtype="bf16", seed=305),
    StreamConfig("fused_bf16_128_64", B=1, H=2, dk=128, dv=64, n_text=0, grid=(5, 9, 13), dtype="bf16", seed=306),
    StreamConfig("fused_text_only", B=2, H=2, dk=128, dv=128, n_text=150, grid=(0, 0, 0), dtype="bf16", seed=307),
    StreamConfig("fused_image", B=2, H=2, dk=128, dv=128, n_text=33, grid=(1, 17, 19), dtype="bf16", seed=308),
    StreamConfig("fused_causal", B=1, H=2, dk=128, dv=128, n_text=9, grid=(5, 6, 8), dtype="bf16", seed=309,
                 causal_t=1),
    StreamConfig("fused_causal_f32", B=1, H=2, dk=64, dv=64, n_text=3, grid=(4, 5, 5), dtype="f32", seed=310,
                 causal_t=1),
    StreamConfig("fused_one_token", B=2, H=1, dk=128, dv=128, n_text=1, grid=(0, 0, 0), dtype="bf16", seed=311),
    StreamConfig("fused_long", B=1, H=2, dk=128, dv=128, n_text=64, grid=(6, 20, 26), dtype="bf16", seed=312),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_fused_matches_the_oracle_and_the_two_calls(cfg):
    S0 = (np.random.default_rng(cfg.seed).standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)) * 0.4).astype(np.float32)
    _check(cfg, S0=S0)


@pytest.mark.timeout(600)
def test_fused_at_the_video_workload_sampled_heads():
    """The 5 s video stream (T = 33 272, 16 heads, bf16) with the launch configuration
    bench.py times for the fused path: o and S_T of two heads against the oracle, and
    the whole o against the two-call path."""
    _check(WORKLOAD["video_5s_480x832"], heads=(5, 12))


@pytest.mark.timeout(600)
def test_fused_at_the_image_workload_sampled_heads():
    """The 4096x4096 image stream (T = 66 048: one latent slice of 256 x 256, 16 heads,
    bf16), whose chunks each span a quarter of an image row: o and S_T of two heads
    against the oracle, and the whole o against the two-call path."""
    _check(WORKLOAD["image_4096px"], heads=(3, 10))


@pytest.mark.timeout(120)
def test_fused_refusals():
    cfg = CASES[3]
    dev = to_dev(make_inputs(cfg))
    d = desc_of(cfg)
    need = kda.kda_conv_kda_forward_workspace_size(d, cfg.B, cfg.H, cfg.dk, cfg.dv, cfg.torch_dtype)
    assert need > kda.kda_forward_workspace_size(d, cfg.B, cfg.H, cfg.dk, cfg.dv, cfg.torch_dtype)
    short = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        _fused(cfg, dev, workspace=short)
    assert e.value.status == kda.KDA_ERR_WORKSPACE
    # a tap array that overlaps the output
    o = torch.empty_like(dev["v"])
    wt = (dev["w_text_q"], dev["w_text_k"], o.view(-1)[: dev["w_text_v"].numel()].view_as(dev["w_text_v"]))
    wv = (dev["w_vis_q"], dev["w_vis_k"], dev["w_vis_v"])
    with pytest.raises(kda.KdaError) as e:
        kda.kda_conv_kda_forward(d, dev["q"], dev["k"], dev["v"], wt, wv, dev["alpha"], dev["beta"], o=o)
    assert e.value.status == kda.KDA_ERR_INVALID_ARG
