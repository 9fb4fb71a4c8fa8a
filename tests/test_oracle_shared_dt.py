"""Pin of the reading used for a Δraw shared by the channels (one value per token).

Page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별", §1.2: Δ comes from a
one-output projection of the token, broadcast over the channels, plus each channel's own
parameter.  The forward is then the ordinary forward on the broadcast [B, D, L] array, and
the gradient with respect to the shared [B, L] value is the sum over channels of the
per-channel gradients.  Checked here against fp64 central finite differences of the oracle's
forward taken with respect to the shared value itself, for both oracle implementations.
"""
import numpy as np
import pytest

from gen import make_inputs
from oracle import ss_ref


def _bwd(impl, inp, dt_raw):
    args = (inp.x, dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip, inp.dy)
    if impl == "c":
        from oracle import cref
        return cref.bwd(*args, z=inp.z, h0=inp.h0, dh_final=inp.dh_final)
    return ss_ref.ss_bwd(*[np.asarray(a, np.float64) for a in args], z=inp.z, h0=inp.h0,
                         dh_final=inp.dh_final)


@pytest.mark.parametrize("impl", ["numpy", "c"])
def test_shared_dt_gradient_is_channel_sum(impl):
    Bn, L, D, N = 2, 6, 4, 3
    inp = make_inputs(Bn, L, D, N, seed=41, gate=True, with_h0=True, with_dy=True,
                      with_dh_final=True, a_perturb=True, dt_shared=True)
    assert inp.dt_tok.shape == (Bn, L)
    assert np.array_equal(inp.dt_raw, np.broadcast_to(inp.dt_tok[:, None, :], (Bn, D, L)))
    tok = inp.dt_tok.astype(np.float64)

    def loss(tok_v):
        dtr = np.broadcast_to(tok_v[:, None, :], (Bn, D, L))
        y, hf = ss_ref.ss_fwd(inp.x, dtr, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                              z=inp.z, h0=inp.h0)
        return float(np.sum(inp.dy * y) + np.sum(inp.dh_final * hf))

    eps = 1e-6
    fd = np.empty_like(tok)
    for i in np.ndindex(tok.shape):
        tp, tm = tok.copy(), tok.copy()
        tp[i] += eps
        tm[i] -= eps
        fd[i] = (loss(tp) - loss(tm)) / (2 * eps)
    g = _bwd(impl, inp, np.broadcast_to(tok[:, None, :], (Bn, D, L)))["ddt_raw"].sum(axis=1)
    err = np.max(np.abs(g - fd)) / np.max(np.abs(fd))
    assert err < 1e-6, err


def test_shared_dt_planted_mistake_fails():
    """Taking one channel's gradient instead of the sum over channels fails the pin."""
    Bn, L, D, N = 1, 5, 3, 2
    inp = make_inputs(Bn, L, D, N, seed=42, with_dy=True, dt_shared=True, a_perturb=True)
    g = _bwd("numpy", inp, inp.dt_raw)["ddt_raw"]
    assert np.max(np.abs(g[:, 0, :] - g.sum(axis=1))) > 1e-3 * np.max(np.abs(g.sum(axis=1)))
