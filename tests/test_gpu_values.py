"""The method's own value edge cases through the HIP path, against the oracle.

The gated delta rule S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
(Chimera, method step (5); the KDA paragraph of the prerequisites: alpha is a
channel-wise forget gate in (0, 1], beta a scalar write strength) fixes what
these inputs must give:
  * strong forgetting (alpha near 0) and alpha at the smallest values the
    kernels accept (any 8 consecutive tokens of a channel decay by more than
    2^-120): the decay factorisation inside a chunk must not overflow;
  * alpha = 1: no decay, the delta rule alone;
  * beta = 0: nothing is written, the initial state only decays, o_t = S_0^T (prod alpha * q_t);
  * beta = 1, alpha = 1 and orthonormal keys: every write is exact, so a query
    equal to an earlier key reads back that key's value exactly.
Every case runs the conv and KDA (or KDA alone where the keys must stay
orthonormal) with an initial state and checks o and S_T against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_modality_amd import kda
from linear_attention_sequence_modality_amd.inputs import StreamConfig, make_inputs

from gpu_common import TOL, check_stream, edge_alpha, heads_slice, rel, rel_elem, say, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# (dtype, dk = dv): the bf16 stream at the workloads' head size, fp32 at both sizes
DTYPES = [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)]
IDS = ["%s_d%d" % d for d in DTYPES]


def _cfg(name, dtype, d, **kw):
    base = dict(B=2, H=2, dk=d, dv=d, n_text=21, grid=(4, 7, 9), dtype=dtype, seed=321)
    base.update(kw)
    return StreamConfig(name, **base)


def _s0(cfg, scale=0.5, seed=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)) * scale).astype(np.float32)


def _with(inp, cfg, **tensors):
    out = dict(inp)
    for name, val in tensors.items():
        out[name] = torch.as_tensor(val).to(cfg.torch_dtype)
    return out


def _skip_unsupported(dtype, d):
    if dtype == "f32" and d == 128 and not kda.supports(torch.float32, 128, 128):
        pytest.skip("fp32 at dk = dv = 128 is refused by this build of the library")


@pytest.mark.timeout(120)
@pytest.mark.parametrize("dtype,d", DTYPES, ids=IDS)
def test_strong_forgetting(dtype, d):
    """alpha = sigmoid(N(-3, 1)): about 0.05 per token and channel."""
    _skip_unsupported(dtype, d)
    cfg = _cfg("strong_decay", dtype, d)
    check_stream(cfg, make_inputs(cfg, alpha_mean=-3.0), S0=_s0(cfg), want_state=True)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("dtype,d", DTYPES, ids=IDS)
def test_alpha_at_the_factorisation_edge(dtype, d):
    _skip_unsupported(dtype, d)
    cfg = _cfg("alpha_edge", dtype, d, n_text=40, grid=(3, 8, 11))
    inp = make_inputs(cfg)
    check_stream(cfg, _with(inp, cfg, alpha=edge_alpha(cfg, inp)), S0=_s0(cfg), want_state=True)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("dtype,d", DTYPES, ids=IDS)
def test_alpha_one(dtype, d):
    """No decay at all: the plain delta rule, with an initial state."""
    _skip_unsupported(dtype, d)
    cfg = _cfg("alpha_one", dtype, d)
    inp = make_inputs(cfg)
    check_stream(cfg, _with(inp, cfg, alpha=np.ones(tuple(inp["alpha"].shape), np.float32)),
                 S0=_s0(cfg), want_state=True)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("dtype,d", DTYPES, ids=IDS)
def test_beta_zero_decays_the_initial_state(dtype, d):
    """beta = 0: o_t = S_0^T (prod_{u<=t} alpha_u * q_t) and S_T = Diag(prod alpha) S_0."""
    _skip_unsupported(dtype, d)
    cfg = _cfg("beta_zero", dtype, d)
    inp = make_inputs(cfg)
    inp = _with(inp, cfg, beta=np.zeros(tuple(inp["beta"].shape), np.float32))
    check_stream(cfg, inp, S0=_s0(cfg, scale=1.0), want_state=True)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("dtype,d", DTYPES, ids=IDS)
def test_exact_recall_with_orthonormal_keys(dtype, d):
    """alpha = 1, beta = 1, the keys of each (b, h) a permutation of the unit vectors
    (T = dk tokens, so two chunks at dk = 128): S_t = sum_{s<=t} k_s v_s^T, and the
    query q_t = k_{s(t)} with s(t) <= t reads back v_{s(t)} exactly.  Queries of
    odd tokens are a mix of two earlier keys, which reads back the same mix of
    values (exact in fp32 accumulation; one rounding to the output dtype)."""
    _skip_unsupported(dtype, d)
    B, H, T = 2, 3, d
    cfg = StreamConfig("recall", B=B, H=H, dk=d, dv=d, n_text=T, grid=(0, 0, 0), dtype=dtype, seed=5)
    rng = np.random.default_rng(17)
    eye = np.eye(d, dtype=np.float32)
    k = np.empty((B, T, H, d), np.float32)
    q = np.empty_like(k)
    src = np.empty((B, T, H), np.int64)
    for b in range(B):
        for h in range(H):
            perm = rng.permutation(d)
            k[b, :, h] = eye[perm[:T]]
            for t in range(T):
                s = int(rng.integers(0, t + 1))
                src[b, t, h] = s
                q[b, t, h] = k[b, s, h]
                if t % 2 == 1 and t > 0:
                    s2 = int(rng.integers(0, t + 1))
                    q[b, t, h] = 0.5 * k[b, s, h] + 0.25 * k[b, s2, h]
    v = rng.standard_normal((B, T, H, d)).astype(np.float32)
    host = {"q": q, "k": k, "v": v, "alpha": np.ones((B, T, H, d), np.float32),
            "beta": np.ones((B, T, H), np.float32)}
    host = {n: torch.from_numpy(x).to(cfg.torch_dtype) for n, x in host.items()}
    dev = to_dev(host)
    sT = torch.empty(B, H, d, d, device="cuda")
    o = kda.kda_forward(kda.make_desc(T, (0, 0, 0)), dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"],
                        final_state=sT)
    torch.cuda.synchronize()
    heads = tuple(range(H))
    ro, rs = oracle.kda_recurrence(*[heads_slice(host[n], heads) for n in ("q", "k", "v", "alpha")],
                                   heads_slice(host["beta"][..., None], heads)[..., 0])
    og = o.double().cpu().numpy()
    e_o, e_s = rel(og, ro), oracle.rel_err_state(sT.double().cpu().numpy(), rs)
    say("case recall %s d=%d: rel err o %.2e S %.2e [o elementwise %.2e]" % (
        dtype, d, e_o, e_s, rel_elem(og, ro)))
    # the oracle itself reads back the stored values: o_t = v_{s(t)} on even tokens
    vv = host["v"].double().numpy()
    even = np.arange(0, T, 2)
    for b in range(B):
        for h in range(H):
            want = vv[b, src[b, even, h], h]
            np.testing.assert_allclose(ro[b, even, h], want, rtol=0, atol=1e-12)
            # and the kernels return exactly the stored (already rounded) values
            np.testing.assert_array_equal(og[b, even, h], want)
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype]
