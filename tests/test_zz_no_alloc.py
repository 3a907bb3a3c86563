"""kda_forward_noalloc (the workspace in the library's own device array) against
kda_forward with a caller's workspace, through the C ABI, on two calls in a row
(the second smaller), in bf16 and fp32, with initial and final states.

The two entry points run the same kernels on the same inputs, so o and the
final state must agree bit for bit; the first call's stream is also checked
against the fp64 oracle within the dtype's gate.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_modality_amd import kda
from linear_attention_sequence_modality_amd.inputs import StreamConfig, make_inputs

from gpu_common import TOL, heads_slice, rel, say, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _run_both(cfg, seed_s0):
    host = make_inputs(cfg)
    dev = to_dev(host)
    d = kda.make_desc(cfg.n_text, cfg.grid, causal_t=cfg.causal_t)
    need = kda.kda_forward_workspace_size(d, cfg.B, cfg.H, cfg.dk, cfg.dv, cfg.torch_dtype)
    assert 0 < need <= kda.KDA_NOALLOC_SCRATCH_BYTES, need
    g = torch.Generator().manual_seed(seed_s0)
    s0 = (torch.randn(cfg.B, cfg.H, cfg.dk, cfg.dv, generator=g) * 0.3).cuda()
    x = [dev[n] for n in ("q", "k", "v", "alpha", "beta")]
    o_ref = torch.full_like(dev["v"], float("nan"))
    s_ref = torch.full_like(s0, float("nan"))
    kda.kda_forward(d, *x, initial_state=s0, final_state=s_ref, o=o_ref)
    o_na = torch.full_like(dev["v"], float("nan"))
    s_na = torch.full_like(s0, float("nan"))
    kda.kda_forward_noalloc(d, *x, initial_state=s0, final_state=s_na, o=o_na)
    torch.cuda.synchronize()
    return host, s0, (o_ref, s_ref), (o_na, s_na)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_noalloc_equals_forward_twice(dtype, d):
    big = StreamConfig("na_big", B=2, H=3, dk=d, dv=d, n_text=37, grid=(6, 11, 13), dtype=dtype, seed=41)
    small = StreamConfig("na_small", B=1, H=2, dk=d, dv=d, n_text=5, grid=(2, 3, 7), dtype=dtype, seed=42)
    for i, cfg in enumerate((big, small)):
        say("case noalloc %s call %d T=%d B=%d H=%d d=%d" % (dtype, i, cfg.T, cfg.B, cfg.H, d))
        host, s0, (o_ref, s_ref), (o_na, s_na) = _run_both(cfg, 7 + i)
        assert torch.isfinite(o_na.float()).all() and torch.isfinite(s_na).all()
        assert torch.equal(o_na, o_ref), "o differs from kda_forward"
        assert torch.equal(s_na, s_ref), "final state differs from kda_forward"
        heads = tuple(range(cfg.H))
        ro, rs = oracle.kda_recurrence(*[heads_slice(host[n], heads) for n in ("q", "k", "v", "alpha")],
                                       heads_slice(host["beta"][..., None], heads)[..., 0],
                                       S0=s0.double().cpu().numpy())
        e_o = rel(o_na.double().cpu().numpy(), ro)
        e_s = oracle.rel_err_state(s_na.double().cpu().numpy(), rs)
        say("  noalloc rel err o %.2e S %.2e" % (e_o, e_s))
        assert e_o <= TOL[dtype] and e_s <= TOL[dtype]


def test_noalloc_rejects_a_workspace_beyond_its_array():
    """A shape whose workspace exceeds the array fails on the host before anything runs."""
    cfg = StreamConfig("na_huge", B=1, H=16, dk=128, dv=128, n_text=8192, grid=(0, 0, 0), dtype="bf16")
    d = kda.make_desc(cfg.n_text, cfg.grid)
    need = kda.kda_forward_workspace_size(d, cfg.B, cfg.H, cfg.dk, cfg.dv, torch.bfloat16)
    assert need > kda.KDA_NOALLOC_SCRATCH_BYTES
    t = torch.empty(cfg.B, cfg.T, cfg.H, cfg.dk, dtype=torch.bfloat16, device="cuda")
    b = torch.empty(cfg.B, cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(t)
    with pytest.raises(kda.KdaError) as e:
        kda.kda_forward_noalloc(d, t, t.clone(), t.clone(), t.clone(), b, o=o)
    assert e.value.status == kda.KDA_ERR_WORKSPACE
