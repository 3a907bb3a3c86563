"""Shared helpers for the GPU parity tests (HIP path vs the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from oracle import backward as ob
from linear_attention_sequence_modality_amd import kda
from linear_attention_sequence_modality_amd.inputs import StreamConfig, make_inputs

# Max relative error (per (batch, head): max |x - ref| over max |ref|) allowed
# for each input dtype: fp32 in and out, or bf16 in and out with fp32 accumulation.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp: dict) -> dict:
    return {k: v.cuda() for k, v in inp.items()}


def desc_of(cfg: StreamConfig):
    return kda.make_desc(cfg.n_text, cfg.grid, causal_t=cfg.causal_t)


def run_path(cfg: StreamConfig, dev: dict, S0=None, want_state=False):
    """HIP conv then HIP KDA on the current stream; returns host fp64 numpy arrays."""
    d = desc_of(cfg)
    sT = None
    if want_state:
        sT = torch.empty(cfg.B, cfg.H, cfg.dk, cfg.dv, dtype=torch.float32, device="cuda")
    s0 = None if S0 is None else torch.as_tensor(S0, dtype=torch.float32).cuda().contiguous()
    qc, kc, vc, o = kda.conv_kda_forward(d, dev, initial_state=s0, final_state=sT)
    torch.cuda.synchronize()
    return qc, kc, vc, o, sT


def heads_slice(x: torch.Tensor, heads) -> np.ndarray:
    """[B, T, H, d] -> fp64 numpy [B, T, len(heads), d] of the chosen heads."""
    return x[:, :, list(heads)].double().cpu().numpy()


def weight_slice(w: torch.Tensor, heads, d: int) -> np.ndarray:
    """[H*d, taps] -> fp64 numpy [len(heads)*d, taps]."""
    return torch.cat([w[h * d:(h + 1) * d] for h in heads]).double().cpu().numpy()


def oracle_conv_heads(cfg, inp_cpu: dict, stream: str, heads) -> np.ndarray:
    d = cfg.dv if stream == "v" else cfg.dk
    x = heads_slice(inp_cpu[stream], heads)
    return oracle.short_conv_heads(x, weight_slice(inp_cpu["w_text_" + stream], heads, d),
                                   weight_slice(inp_cpu["w_vis_" + stream], heads, d),
                                   cfg.n_text, cfg.grid, cfg.causal_t)


def oracle_end_to_end_heads(cfg, inp_cpu: dict, heads, S0=None):
    qc = oracle_conv_heads(cfg, inp_cpu, "q", heads)
    kc = oracle_conv_heads(cfg, inp_cpu, "k", heads)
    vc = oracle_conv_heads(cfg, inp_cpu, "v", heads)
    s0 = None if S0 is None else np.asarray(S0)[:, list(heads)]
    o, st = oracle.kda_recurrence(qc, kc, vc, heads_slice(inp_cpu["alpha"], heads),
                                  heads_slice(inp_cpu["beta"][..., None], heads)[..., 0], s0)
    return qc, kc, vc, o, st


def rel(x: np.ndarray, ref: np.ndarray) -> float:
    return oracle.rel_err(x, ref)


def rel_elem(x: np.ndarray, ref: np.ndarray, layout: str = "tokens") -> float:
    """Element-wise relative error (floor 1e-6 of each (b, h)'s max |ref|): reported, not gated."""
    return oracle.rel_err_elementwise(x, ref, layout=layout)


def check_stream(cfg: StreamConfig, inp: dict, heads=None, S0=None, want_state=False):
    """Conv + KDA on the GPU against the oracle on the chosen heads (all by default).

    Gates the per-(b, h) max relative error of q', k', v', o (and S_T) at the
    dtype's tolerance; prints the element-wise error of o and S_T beside it.
    """
    say("case %s B=%d T=%d H=%d dk=%d dv=%d %s causal_t=%d heads=%s" % (
        cfg.name, cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv, cfg.dtype, cfg.causal_t, heads))
    dev = to_dev(inp)
    qc, kc, vc, o, sT = run_path(cfg, dev, S0=S0, want_state=want_state)
    heads = tuple(range(cfg.H)) if heads is None else heads
    rq, rk, rv, ro, rs = oracle_end_to_end_heads(cfg, inp, heads, S0)
    tol = TOL[cfg.dtype]
    oh = heads_slice(o, heads)
    errs = {"q'": rel(heads_slice(qc, heads), rq), "k'": rel(heads_slice(kc, heads), rk),
            "v'": rel(heads_slice(vc, heads), rv), "o": rel(oh, ro)}
    extra = {"o elementwise": rel_elem(oh, ro)}
    if want_state:
        sh = sT[:, list(heads)].double().cpu().numpy()
        errs["S_T"] = oracle.rel_err_state(sh, rs)
        extra["S_T elementwise"] = rel_elem(sh, rs, layout="state")
    say("  rel errors: " + ", ".join("%s %.2e" % kv for kv in errs.items()) +
        "  [" + ", ".join("%s %.2e" % kv for kv in extra.items()) + "]")
    assert np.isfinite(oh).all(), "non-finite o"
    for name, e in errs.items():
        assert e <= tol, "%s rel err %.3e > %.1e" % (name, e, tol)
    return errs


def edge_alpha(cfg: StreamConfig, inp: dict) -> np.ndarray:
    """alpha = 2^-14 (exact in bf16 and fp32) on runs of tokens of chosen channels: any 8
    consecutive tokens then decay by 2^-112, just inside the 2^-120 the chunk
    factorisation accepts.  Runs start at several offsets from the chunk and
    16-token sub-block boundaries and one covers whole chunks."""
    a = inp["alpha"].float().numpy().copy()
    T, dk = cfg.T, cfg.dk
    tiny = np.float32(2.0 ** -14)
    runs = [(0, 8, range(0, dk, 5)), (13, 9, range(1, dk, 3)), (56, 16, range(2, dk, 7)),
            (64 + 7, 8, range(0, dk)), (128, 128, range(3, dk, 4)), (T - 11, 11, range(0, dk, 2))]
    for t0, n, chans in runs:
        t0 = min(max(t0, 0), T - 1)
        a[:, t0:min(t0 + n, T), :, list(chans)] = tiny
    return a


def check_backward(cfg: StreamConfig, host: dict, dalpha_tol=None, S0_scale=0.3):
    """kda_backward on the GPU against the fp64 adjoint oracle: every gradient (q, k, v,
    alpha, beta, the initial state) gated per (batch, head) at the dtype's tolerance, with a
    seeded dO, initial state and final-state gradient.  dalpha_tol: gate d alpha there and
    d log alpha = alpha * d alpha at the standard tolerance (where alpha is tiny)."""
    say("case %s B=%d T=%d H=%d dk=%d dv=%d %s" % (cfg.name, cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv, cfg.dtype))
    g = np.random.default_rng(cfg.seed)
    dO = torch.from_numpy(g.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dv)).astype(np.float32)).to(cfg.torch_dtype)
    S0 = torch.from_numpy((g.standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)) * S0_scale).astype(np.float32))
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
    gates = {name: TOL[cfg.dtype] for name in errs}
    if dalpha_tol is not None:
        # d log alpha = alpha * d alpha at the standard gate; d alpha at its own
        a = host["alpha"].double().numpy()
        errs["alpha*dalpha"] = rel(a * out["dalpha"].double().cpu().numpy(), a * ref["dalpha"])
        gates["alpha*dalpha"] = TOL[cfg.dtype]
        gates["dalpha"] = dalpha_tol
    say("  rel errors: " + ", ".join("%s %.2e" % kv for kv in errs.items()))
    for name in ("dq", "dk", "dv", "dalpha", "dbeta"):
        assert torch.isfinite(out[name].float()).all(), "non-finite " + name
    for name, e in errs.items():
        assert e <= gates[name], "%s rel err %.3e > %.1e" % (name, e, gates[name])
