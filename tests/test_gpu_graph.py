"""The library's calls inside HIP graphs.

Every entry point only launches kernels on the caller's stream (no allocation, no memset, no
synchronisation), so a serving loop or a training step can be captured once and replayed.
Each graph here is replayed several times with eager work and synchronisations between the
replays, and every replay is checked against the eager result of the same calls; the eager
result is itself checked against the fp64 oracle.
"""
import numpy as np
import pytest

from gen import make_inputs
from oracle import cref
from tests.gpu_util import TOL_GRAD, assert_close, dev, note, tol_for

pytestmark = pytest.mark.gpu


def test_decode_loop_graph(gpu):
    """T decode steps (state in place) captured as one graph."""
    import torch
    Bn, T, D, N = 4, 8, 256, 16
    inp = make_inputs(Bn, T, D, N, dtype="bf16", seed=1200, gate=True, with_h0=True,
                      a_perturb=True)
    note("graph: decode loop")
    bf = torch.bfloat16
    # per-step inputs staged token-major: [T, B, D] and [T, B, N]
    tok = lambda a: torch.from_numpy(np.ascontiguousarray(np.moveaxis(a, 2, 0))).to(bf).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    xs, dts, zs, Bs, Cs = tok(inp.x), tok(inp.dt_raw), tok(inp.z), tok(inp.Bm), tok(inp.Cm)
    dtb, A, Dk, h0 = f32(inp.dt_bias), f32(inp.A), f32(inp.Dskip), f32(inp.h0)
    h = h0.clone()
    ys = torch.empty((T, Bn, D), dtype=torch.float32, device="cuda")

    def run(stream=None):
        for t in range(T):
            gpu.ss_step(xs[t], dts[t], dtb, A, Bs[t], Cs[t], Dk, h, z=zs[t], y=ys[t], stream=stream)

    run()
    torch.cuda.synchronize()
    y_eager, h_eager = ys.clone(), h.clone()
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip, z=inp.z,
                      h0=inp.h0)
    assert_close(np.moveaxis(y_eager.cpu().numpy(), 0, 2), yr, tol_for(inp), "eager y")
    assert_close(h_eager.cpu().numpy(), hr, tol_for(inp), "eager state")

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        h.copy_(h0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            run(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        h.copy_(h0)                                   # eager work between replays
        ys.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, y_eager), f"replay {rep}: y differs from the eager run"
        assert torch.equal(h, h_eager), f"replay {rep}: state differs from the eager run"


def test_training_step_graph(gpu):
    """Chunked forward with checkpoints and the backward on them, captured as one graph."""
    import selective_state_space_34_amd as ss
    import torch
    Bn, L, D, N = 2, 512, 128, 16
    inp = make_inputs(Bn, L, D, N, dtype="bf16", seed=1201, gate=True, with_h0=True,
                      with_dy=True, with_dh_final=True, a_perturb=True)
    note("graph: training step")
    t = dev(inp)
    args = (t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"])
    nck = (L + ss.CKPT_STEPS - 1) // ss.CKPT_STEPS
    y = torch.empty((Bn, D, L), dtype=torch.float32, device="cuda")
    hf = torch.empty((Bn, D, N), dtype=torch.float32, device="cuda")
    hck = torch.empty((Bn, D, nck, N), dtype=torch.float32, device="cuda")
    dims = ss.make_dims(Bn, L, D, N, ss.SS_BF16, ss.SS_PLAN_CHUNKED)
    wsf = torch.empty(max(ss.workspace_size(dims), 1), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(ss.workspace_size(dims, backward=True), dtype=torch.uint8, device="cuda")
    grads = ss.ss_bwd(*args[:7], t["dy"], z=t["z"], h0=t["h0"], dh_final=t["dh_final"])

    def step(stream=None):
        ss.ss_fwd(*args, z=t["z"], h0=t["h0"], y=y, h_final=hf, h_ckpt=hck, workspace=wsf,
                  plan=ss.SS_PLAN_CHUNKED, stream=stream)
        ss.ss_bwd(*args, t["dy"], z=t["z"], h0=t["h0"], dh_final=t["dh_final"], h_ckpt=hck,
                  workspace=wsb, out=grads, stream=stream)

    step()
    torch.cuda.synchronize()
    eager = {k: (None if v is None else v.clone()) for k, v in grads.items()}
    y_eager = y.clone()
    ref = cref.bwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip, inp.dy,
                   z=inp.z, h0=inp.h0, dh_final=inp.dh_final)
    for k, v in eager.items():
        assert_close(v.cpu().numpy(), ref[k], TOL_GRAD, f"eager {k}")

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        step(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for v in list(grads.values()) + [y]:          # eager work between replays
            if v is not None:
                v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep}: y differs"
        for k, v in grads.items():
            if v is not None:
                assert torch.equal(v, eager[k]), f"replay {rep}: {k} differs from the eager run"
