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

from gpu_common import TOL, desc_of, rel, say

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
    say("case %s B=%d T=%d H=%d dk=%d dv=%d %s" % (cfg.name, cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv, cfg.dtype))
    host = make_inputs(cfg)
    g = np.random.default_rng(cfg.seed)
    dO = torch.from_numpy(g.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dv)).astype(np.float32)).to(cfg.torch_dtype)
    S0 = torch.from_numpy((g.standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)) * 0.3).astype(np.float32))
    dST = torch.from_numpy(g.standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)).astype(np.float32))
    dev = {k: v.cuda() for k, v in host.items()}
    out = kda.kda_backward(desc_of(cfg), dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dO.cuda(),
                           initial_state=S0.cuda(), d_final_state=dST.cuda())
    torch.cuda.synchronize()
    ref = ob.kda_recurrence_backward(host["q"], host["k"], host["v"], host["alpha"], host["beta"], dO, S0, dST)
    errs = {}
    for name in ("dq", "dk", "dv", "dalpha"):
        errs[name] = rel(out[name].double().cpu().numpy(), ref[name])
    errs["dbeta"] = rel(out["dbeta"].double().cpu().numpy()[..., None], ref["dbeta"][..., None])
    errs["dS0"] = oracle.rel_err_state(out["d_initial_state"].double().cpu().numpy(), ref["dS0"])
    say("  rel errors: " + ", ".join("%s %.2e" % kv for kv in errs.items()))
    for name, e in errs.items():
        assert e <= TOL[cfg.dtype], "%s rel err %.3e" % (name, e)


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
