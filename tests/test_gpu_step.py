"""GPU parity of the single-token (decode) step ss_step against the fp64 oracle.

The step is the recurrence carried one token further: its definition is the forward at
L = 1 started from the given state, so the oracle is cref.fwd on one step with h0 = the
state; T consecutive steps must give the forward over T tokens (the resume identity).
Tolerances as the forward: 1e-4·max|ref| (float32 inputs), 2e-3·max|ref| (bfloat16).
"""
import numpy as np
import pytest

from gen import make_inputs
from oracle import cref
from tests.gpu_util import assert_close, note, tol_for

pytestmark = pytest.mark.gpu


def _dev(inp, t):
    """Device tensors of step t of a seeded sequence: x etc. [B, D], B/C [B, N]."""
    import torch
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    col = lambda a: torch.from_numpy(np.ascontiguousarray(a[..., t])).to(dt).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return dict(x=col(inp.x), dt_raw=col(inp.dt_raw), z=None if inp.z is None else col(inp.z),
                Bm=col(inp.Bm), Cm=col(inp.Cm), dt_bias=f32(inp.dt_bias), A=f32(inp.A),
                Dskip=f32(inp.Dskip))


CASES = [
    # B, D, N, dtype, gate
    (4, 96, 16, "bf16", True),
    (3, 70, 16, "f32", False),
    (2, 33, 32, "bf16", True),
    (5, 17, 8, "f32", True),
    (2, 40, 4, "bf16", False),
    (3, 9, 2, "f32", True),
    (1, 5, 1, "bf16", True),
    (64, 640, 16, "bf16", True),
]


@pytest.mark.parametrize("inplace", [True, False], ids=["inplace", "out"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}D{}N{}-{}-g{}".format(*c))
def test_step_matches_one_token_forward(gpu, case, inplace):
    import torch
    Bn, D, N, dt, gate = case
    inp = make_inputs(Bn, 1, D, N, dtype=dt, seed=500 + D + N, gate=gate, with_h0=True,
                      a_perturb=True)
    note(f"step {case} inplace={inplace}")
    t = _dev(inp, 0)
    h = torch.from_numpy(np.ascontiguousarray(inp.h0, np.float32)).cuda()
    h_out = None if inplace else torch.full_like(h, float("nan"))
    y = gpu.ss_step(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"], h,
                    z=t["z"] if gate else None, h_out=h_out)
    torch.cuda.synchronize()
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z if gate else None, h0=inp.h0)
    assert_close(y.cpu().numpy(), yr[..., 0], tol_for(inp), "y")
    hn = (h if inplace else h_out).cpu().numpy()
    assert_close(hn, hr, tol_for(inp), "state")
    if not inplace:
        assert np.array_equal(h.cpu().numpy(), inp.h0.astype(np.float32)), "h_in was modified"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_steps_equal_forward(gpu, dt):
    """T decode steps from h0 give the forward's y_t at every t and its final state."""
    import torch
    Bn, T, D, N = 2, 40, 48, 16
    inp = make_inputs(Bn, T, D, N, dtype=dt, seed=77, gate=True, with_h0=True, a_perturb=True)
    note(f"step sequence {dt}")
    h = torch.from_numpy(np.ascontiguousarray(inp.h0, np.float32)).cuda()
    ys = []
    for t in range(T):
        s = _dev(inp, t)
        ys.append(gpu.ss_step(s["x"], s["dt_raw"], s["dt_bias"], s["A"], s["Bm"], s["Cm"],
                              s["Dskip"], h, z=s["z"]).cpu().numpy())
    y = np.stack(ys, axis=-1)
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z, h0=inp.h0)
    assert_close(y, yr, tol_for(inp), "y over T steps")
    assert_close(h.cpu().numpy(), hr, tol_for(inp), "state after T steps")
