"""ss_fwd_noalloc: the forward with the library's static per-GPU scratch instead of a
workspace.  Its results must equal ss_fwd's (same plan, same kernels) on consecutive calls
that reuse the scratch, the second on a smaller input, and they must meet the oracle's
tolerance.  Runs through the C ABI (ctypes binding)."""
import numpy as np
import pytest

from gen import make_inputs
from oracle import cref
from tests.gpu_util import TOL_BF16, TOL_F32, assert_close, dev, note

pytestmark = pytest.mark.gpu

CASES = [
    # B, L, D, N, dtype, gate, h0, plan, chunk, layout: scratch-using plans, largest first
    (2, 2048, 256, 16, "bf16", True, True, 2, 0, 0),    # chunked, four lanes
    (1, 640, 96, 16, "f32", True, False, 2, 64, 2),     # chunked, one lane: B/C staging too
    (1, 104, 20, 16, "f32", False, True, 0, 0, 2),      # single pass, one lane: staging only
]


def _run_pair(gpu, case, stream=None):
    import torch
    Bn, L, D, N, dt, gate, h0, plan, chunk, layout = case
    inp = make_inputs(Bn, L, D, N, dtype=dt, seed=900 + L, gate=gate, with_h0=h0, a_perturb=True)
    t = dev(inp)
    z = t["z"] if gate else None
    h = t["h0"] if h0 else None
    args = (t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"])
    dims = gpu.make_dims(Bn, L, D, N, gpu.SS_BF16 if dt == "bf16" else gpu.SS_F32, plan, chunk,
                         layout)
    assert gpu.workspace_size(dims) > 0, "the case must use scratch"
    nck = (L + 15) // 16
    ref_y, ref_hf, ref_ck = gpu.ss_fwd(*args, z=z, h0=h, return_final=True, return_ckpt=True,
                                       plan=plan, chunk=chunk, layout=layout)
    y = torch.full_like(ref_y, float("nan"))
    hf = torch.full_like(ref_hf, float("nan"))
    ck = torch.full((Bn, D, nck, N), float("nan"), dtype=torch.float32, device=y.device)
    gpu.ss_fwd_noalloc(*args, y, z=z, h0=h, h_final=hf, h_ckpt=ck, plan=plan, chunk=chunk,
                       layout=layout, stream=stream)
    torch.cuda.synchronize()
    # the same kernels on the same plan: identical bits
    assert torch.equal(y, ref_y)
    assert torch.equal(hf, ref_hf)
    assert torch.equal(ck, ref_ck)
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z if gate else None, h0=inp.h0 if h0 else None)
    tol = TOL_BF16 if dt == "bf16" else TOL_F32
    assert_close(y.cpu().numpy(), yr, tol, "y")
    assert_close(hf.cpu().numpy(), hr, tol, "h_final")


def test_noalloc_matches_fwd_on_consecutive_calls(gpu):
    """Two calls in a row share the scratch; the second has a smaller input and runs on a
    side stream (the scratch then comes from that stream's device)."""
    import torch
    note(f"ss_fwd_noalloc {CASES[0]}")
    _run_pair(gpu, CASES[0])
    note(f"ss_fwd_noalloc {CASES[1]} on a side stream")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _run_pair(gpu, CASES[1], stream=side)
    torch.cuda.synchronize()
    note(f"ss_fwd_noalloc {CASES[2]}")
    _run_pair(gpu, CASES[2])


def test_noalloc_rejects_oversized_plan(gpu):
    """A plan whose workspace exceeds the static scratch is refused before anything runs."""
    import torch
    Bn, L, D, N = 1, 65536, 256, 16
    dims = gpu.make_dims(Bn, L, D, N, gpu.SS_BF16, gpu.SS_PLAN_CHUNKED, 32)
    assert gpu.workspace_size(dims) > (64 << 20)
    x = torch.zeros((Bn, D, L), dtype=torch.bfloat16, device="cuda")
    Bm = torch.zeros((Bn, N, L), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros((D, N), dtype=torch.float32, device="cuda")
    v = torch.zeros((D,), dtype=torch.float32, device="cuda")
    y = torch.empty((Bn, D, L), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu.SSError) as ei:
        gpu.ss_fwd_noalloc(x, x, v, p, Bm, Bm, v, y, plan=gpu.SS_PLAN_CHUNKED, chunk=32)
    assert ei.value.code == -8
