"""Conv + KDA forward and KDA backward on seeded random stream shapes against the
oracle (needs an MI355X).

Each case draws a layout (text length, (t, h, w) grid, batch, heads, head sizes,
dtype, time padding, an initial state or not) from a fixed seed, so the cases are
the same on every run; together they sweep the paths a fixed list might miss:
ragged chunks and tiles at every edge, single-slice grids (the conv's row-group
march) and multi-slice ones, one to many segments of the state pass, and both
dtypes at both head sizes.  Gates as for every stream test (R13).
"""
import numpy as np
import pytest
import torch

from linear_attention_sequence_modality_amd.inputs import StreamConfig, make_inputs

from gpu_common import check_backward, check_stream

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _case(i):
    r = np.random.default_rng(9000 + i)
    dtype = ["bf16", "f32"][int(r.integers(0, 2))]
    dk = int(r.choice([64, 128]))
    dv = int(r.choice([64, 128]))
    gt = int(r.choice([0, 1, 1, 2, 3, 5]))
    gh = int(r.integers(1, 40)) if gt else 0
    gw = int(r.integers(1, 40)) if gt else 0
    n_text = int(r.integers(0 if gt else 1, 300))
    B = int(r.integers(1, 4))
    H = int(r.integers(1, 4))
    causal = int(r.integers(0, 2)) if gt else 0
    return StreamConfig("rand%02d" % i, B=B, H=H, dk=dk, dv=dv, n_text=n_text, grid=(gt, gh, gw), dtype=dtype,
                        seed=9100 + i, causal_t=causal), bool(r.integers(0, 2))


def _long_case(i):
    """Longer streams, so that the state pass cuts each into several segments
    (the cut follows B * H * chunks / 256)."""
    r = np.random.default_rng(9500 + i)
    dtype = ["bf16", "f32"][int(r.integers(0, 2))]
    d = int(r.choice([64, 128]))
    gt, gh, gw = int(r.integers(2, 7)), int(r.integers(10, 41)), int(r.integers(10, 41))
    return StreamConfig("long%02d" % i, B=int(r.integers(1, 3)), H=int(r.integers(2, 5)), dk=d, dv=d,
                        n_text=int(r.integers(0, 600)), grid=(gt, gh, gw), dtype=dtype, seed=9600 + i,
                        causal_t=int(r.integers(0, 2))), True


CASES = [_case(i) for i in range(16)] + [_long_case(i) for i in range(4)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0].name for c in CASES])
def test_random_shape(i):
    cfg, with_state = CASES[i]
    S0 = None
    if with_state:
        S0 = (np.random.default_rng(cfg.seed).standard_normal((cfg.B, cfg.H, cfg.dk, cfg.dv)) * 0.4).astype(
            np.float32)
    check_stream(cfg, make_inputs(cfg), S0=S0, want_state=True)


def _bwd_case(i):
    r = np.random.default_rng(9700 + i)
    dtype = ["bf16", "f32"][int(r.integers(0, 2))]
    gt = int(r.choice([0, 1, 2, 3]))
    gh = int(r.integers(1, 20)) if gt else 0
    gw = int(r.integers(1, 24)) if gt else 0
    return StreamConfig("brand%02d" % i, B=int(r.integers(1, 3)), H=int(r.integers(1, 3)),
                        dk=int(r.choice([64, 128])), dv=int(r.choice([64, 128])),
                        n_text=int(r.integers(0 if gt else 1, 200)), grid=(gt, gh, gw), dtype=dtype,
                        seed=9800 + i), float(r.choice([3.0, 1.0, -1.5]))


BWD_CASES = [_bwd_case(i) for i in range(10)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("i", range(len(BWD_CASES)), ids=[c[0].name for c in BWD_CASES])
def test_random_shape_backward(i):
    """kda_backward on seeded random layouts (ragged chunk tails, one to a few chunks
    per stream, both dtypes, dk and dv drawn independently, alpha centred on
    sigmoid(3), sigmoid(1) or sigmoid(-1.5)) against the fp64 adjoint oracle."""
    cfg, alpha_mean = BWD_CASES[i]
    check_backward(cfg, make_inputs(cfg, alpha_mean=alpha_mean))
