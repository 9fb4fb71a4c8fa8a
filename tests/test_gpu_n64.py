"""GPU parity at state size N = 64 against the fp64 oracle (which is written for any N).

At N = 64 the forward runs on eight lanes of eight states per channel (the automatic and
eight-lane layouts), in both memory orders, both discretisations, single-pass and chunked,
with checkpoints; the decode step on sixteen lanes of four states; the block forward around
such a scan.  The backward and the layouts whose per-lane state would not fit return
SS_ERR_UNSUPPORTED, checked here through the binding before any launch.  Tolerances as for
every other N: 1e-4 / 2e-3 · max|ref| (float32 / bfloat16 inputs), block 1e-4.
"""
import numpy as np
import pytest

from gen import make_block_inputs, make_inputs
from oracle import block_ref, cref
from tests.gpu_util import assert_close, dev, gpu_fwd, note, tol_for

pytestmark = pytest.mark.gpu

N = 64

CASES = [
    # B, L, D, dtype, gate, h0, plan, chunk, disc
    (2, 256, 64, "f32", True, True, 0, 0, 0),        # single pass
    (1, 2000, 70, "bf16", True, True, 0, 0, 0),      # chunked, D not a block multiple
    (2, 1024, 33, "f32", False, True, 2, 64, 0),
    (1, 8, 3, "bf16", True, False, 0, 0, 0),
    (2, 512, 48, "f32", True, True, 0, 0, 1),        # exact hold
    (1, 1536, 40, "bf16", True, True, 2, 96, 1),
    (2, 128, 2048, "bf16", True, True, 0, 0, 0),     # many channels, single pass
]


@pytest.mark.parametrize("layout", [0, 3], ids=["auto", "oct"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}L{}D{}-{}-g{}-h{}-p{}-c{}-z{}".format(*c))
def test_n64_fwd(gpu, case, layout):
    Bn, L, D, dt, gate, h0, plan, chunk, disc = case
    inp = make_inputs(Bn, L, D, N, dtype=dt, seed=2000 + L + D, gate=gate, with_h0=h0,
                      a_perturb=True)
    note(f"n64 fwd {case} layout={layout}")
    y, hf = gpu_fwd(gpu, inp, gate=gate, h0=h0, final=True, plan=plan, chunk=chunk,
                    layout=layout, disc=disc)
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z if gate else None, h0=inp.h0 if h0 else None, zoh=bool(disc))
    assert_close(y, yr, tol_for(inp), "y")
    assert_close(hf, hr, tol_for(inp), "h_final")


@pytest.mark.parametrize("case", [(1, 333, 40, "bf16", True), (2, 200, 96, "f32", False)],
                         ids=lambda c: "B{}L{}D{}-{}-g{}".format(*c))
def test_n64_fwd_token_major(gpu, case):
    import torch
    Bn, L, D, dt, gate = case
    inp = make_inputs(Bn, L, D, N, dtype=dt, seed=2100 + L, gate=gate, with_h0=True,
                      a_perturb=True)
    note(f"n64 fwd token-major {case}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tok = lambda a: torch.from_numpy(np.ascontiguousarray(np.swapaxes(a, 1, 2))).to(tdt).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    y, hf = gpu.ss_fwd(tok(inp.x), tok(inp.dt_raw), f32(inp.dt_bias), f32(inp.A), tok(inp.Bm),
                       tok(inp.Cm), f32(inp.Dskip), z=tok(inp.z) if gate else None,
                       h0=f32(inp.h0), return_final=True, order=1)
    torch.cuda.synchronize()
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z if gate else None, h0=inp.h0)
    assert_close(np.swapaxes(y.cpu().numpy(), 1, 2), yr, tol_for(inp), "y")
    assert_close(hf.cpu().numpy(), hr, tol_for(inp), "h_final")


def test_n64_checkpoints(gpu):
    """The state entering every 16th step, written by the chunked eight-lane forward."""
    import torch
    inp = make_inputs(1, 704, 40, N, dtype="bf16", seed=2200, gate=True, with_h0=True,
                      a_perturb=True)
    note("n64 checkpoints")
    t = dev(inp)
    _, ck = gpu.ss_fwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"],
                       z=t["z"], h0=t["h0"], return_ckpt=True, plan=2, chunk=96)
    torch.cuda.synchronize()
    ckn = ck.cpu().numpy()
    assert ckn.shape == (1, 40, 704 // 16, N)
    assert_close(ckn[:, :, 0], inp.h0, 0.0, "checkpoint 0")
    for i in (1, 5, 6, 43):
        cut = lambda a: np.ascontiguousarray(a[..., :16 * i])
        _, hi = cref.fwd(cut(inp.x), cut(inp.dt_raw), inp.dt_bias, inp.A, cut(inp.Bm),
                         cut(inp.Cm), inp.Dskip, z=cut(inp.z), h0=inp.h0)
        assert_close(ckn[:, :, i], hi, tol_for(inp), f"checkpoint {i}")


@pytest.mark.parametrize("case", [(4, 96, "bf16", True, 0), (3, 70, "f32", False, 1)],
                         ids=lambda c: "B{}D{}-{}-g{}-z{}".format(*c))
def test_n64_decode_step(gpu, case):
    import torch
    Bn, D, dt, gate, disc = case
    T = 12
    inp = make_inputs(Bn, T, D, N, dtype=dt, seed=2300 + D, gate=gate, with_h0=True,
                      a_perturb=True)
    note(f"n64 step {case}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    col = lambda a, t: torch.from_numpy(np.ascontiguousarray(a[..., t])).to(tdt).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    h = f32(inp.h0)
    ys = []
    for t in range(T):
        ys.append(gpu.ss_step(col(inp.x, t), col(inp.dt_raw, t), f32(inp.dt_bias), f32(inp.A),
                              col(inp.Bm, t), col(inp.Cm, t), f32(inp.Dskip), h,
                              z=col(inp.z, t) if gate else None, disc=disc).cpu().numpy())
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z if gate else None, h0=inp.h0, zoh=bool(disc))
    assert_close(np.stack(ys, axis=-1), yr, tol_for(inp), "y over T steps")
    assert_close(h.cpu().numpy(), hr, tol_for(inp), "state after T steps")


def test_n64_block(gpu):
    import torch
    inp = make_block_inputs(2, 96, 64, 128, N, dtype="bf16", seed=2400, with_h0=True)
    note("n64 block")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    y, hf, proj = gpu.ss_block_fwd(bf(inp.u), bf(inp.W_in), f32(inp.W_x), f32(inp.dt_bias),
                                   f32(inp.A), f32(inp.Dskip), h0=f32(inp.h0), return_final=True,
                                   return_proj=True)
    torch.cuda.synchronize()
    ref = block_ref.block_fwd(inp.u, inp.W_in, inp.W_x, inp.dt_bias, inp.A, inp.Dskip, h0=inp.h0)
    for k in ("x", "z", "dt", "B", "C"):
        assert_close(proj[k].cpu().numpy(), ref[k], 1e-4, k)
    assert_close(y.cpu().numpy(), ref["y"], 1e-4, "y")
    assert_close(hf.cpu().numpy(), ref["h_final"], 1e-4, "h_final")


def test_n64_unsupported(gpu):
    """Rejected before any launch: the backward, one lane or four lanes per channel, and
    channel-major rows with L % 8 != 0."""
    inp = make_inputs(1, 64, 8, N, seed=2500, gate=True, with_dy=True, a_perturb=True)
    t = dev(inp)
    args = (t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"])
    with pytest.raises(gpu.SSError) as e:
        gpu.ss_bwd(*args, t["dy"], z=t["z"])
    assert e.value.code == -7
    for layout in (1, 2):
        with pytest.raises(gpu.SSError) as e:
            gpu.ss_fwd(*args, z=t["z"], layout=layout)
        assert e.value.code == -7
    odd = make_inputs(1, 63, 8, N, seed=2501, a_perturb=True)
    to = dev(odd)
    with pytest.raises(gpu.SSError) as e:
        gpu.ss_fwd(to["x"], to["dt_raw"], to["dt_bias"], to["A"], to["Bm"], to["Cm"], to["Dskip"])
    assert e.value.code == -7
