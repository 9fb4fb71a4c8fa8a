"""GPU parity on the degenerate cases of the method, against the fp64 oracle.

- A = 0: no decay, the state integrates its inputs (Ā = 1); the exact hold's gain takes its
  limit δ and its A-derivative the limit δ²/2, where the closed forms divide by A = 0 (the
  kernels must take the series side and leak no infinity or NaN);
- A slightly positive: the state grows (exp(δA) > 1), still finite over the sequence;
- x = 0 with an initial state: pure decay, y_t = C_t·Ā^t·h0 (D·x drops out);
- z = 0: the gate closes, y = 0 exactly, and dz = dy·s/2;
- B = 0: nothing enters the state; D = 0: no skip term.
Every forward layout and plan, both discretisations, and the backward.  Tolerances as
everywhere: 1e-4 · max|ref| (float32 inputs) for outputs, 5e-4 · max|ref| for gradients.
"""
import numpy as np
import pytest

from gen import make_inputs
from oracle import cref
from tests.gpu_util import TOL_GRAD, assert_close, dev, note

pytestmark = pytest.mark.gpu

KINDS = ["A_zero", "A_positive", "A_some_zero", "x_zero", "z_zero", "B_zero", "D_zero"]


def _case(kind, seed):
    inp = make_inputs(2, 200, 70, 16, seed=seed, gate=True, with_h0=True, with_dy=True,
                      with_dh_final=True, a_perturb=True)
    if kind == "A_zero":
        inp.A[:] = 0.0
    elif kind == "A_positive":
        inp.A[:] = np.abs(inp.A) * np.float32(0.01)
    elif kind == "A_some_zero":
        inp.A[:, ::3] = 0.0
    elif kind == "x_zero":
        inp.x[:] = 0.0
    elif kind == "z_zero":
        inp.z[:] = 0.0
    elif kind == "B_zero":
        inp.Bm[:] = 0.0
    elif kind == "D_zero":
        inp.Dskip[:] = 0.0
    return inp


def _close(got, ref, tol, what):
    """Relative to the reference's largest value; an all-zero reference must be met exactly."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if np.max(np.abs(ref)) == 0.0:
        assert np.max(np.abs(got)) == 0.0, f"{what}: expected exact zeros"
        return
    assert_close(got, ref, tol, what)


@pytest.mark.parametrize("disc", [0, 1], ids=["euler", "zoh"])
@pytest.mark.parametrize("layout,plan", [(0, 0), (0, 2), (1, 0), (2, 0), (3, 2)],
                         ids=["auto", "auto-chunked", "quad", "lane", "oct-chunked"])
@pytest.mark.parametrize("kind", KINDS)
def test_degenerate_fwd(gpu, kind, layout, plan, disc):
    import torch
    inp = _case(kind, seed=3100 + KINDS.index(kind))
    note(f"degenerate fwd {kind} layout={layout} plan={plan} disc={disc}")
    t = dev(inp)
    y, hf = gpu.ss_fwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"],
                       z=t["z"], h0=t["h0"], return_final=True, layout=layout, plan=plan,
                       chunk=64 if plan == 2 else 0, disc=disc)
    torch.cuda.synchronize()
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z, h0=inp.h0, zoh=bool(disc))
    _close(y.cpu().numpy(), yr, 1e-4, "y")
    _close(hf.cpu().numpy(), hr, 1e-4, "h_final")
    if kind == "z_zero":
        assert float(y.abs().max()) == 0.0


@pytest.mark.parametrize("disc", [0, 1], ids=["euler", "zoh"])
@pytest.mark.parametrize("ckpt", [False, True], ids=["recompute", "ckpt"])
@pytest.mark.parametrize("kind", KINDS)
def test_degenerate_bwd(gpu, kind, ckpt, disc):
    import torch
    inp = _case(kind, seed=3200 + KINDS.index(kind))
    note(f"degenerate bwd {kind} ckpt={ckpt} disc={disc}")
    t = dev(inp)
    args = (t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"])
    hck = None
    if ckpt:
        _, hck = gpu.ss_fwd(*args, z=t["z"], h0=t["h0"], return_ckpt=True, disc=disc)
    g = gpu.ss_bwd(*args, t["dy"], z=t["z"], h0=t["h0"], dh_final=t["dh_final"], h_ckpt=hck,
                   disc=disc)
    torch.cuda.synchronize()
    ref = cref.bwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip, inp.dy,
                   z=inp.z, h0=inp.h0, dh_final=inp.dh_final, zoh=bool(disc))
    for k in ("dx", "ddt_raw", "dz", "ddt_bias", "dA", "dB", "dC", "dD", "dh0"):
        _close(g[k].cpu().numpy(), ref[k], TOL_GRAD, k)
