"""GPU parity of the exact zero-order-hold backward (ss_bwd with disc = SS_DISC_ZOH) against
the fp64 oracle's ss_bwd(..., zoh=True), which finite differences of its separately pinned
exact-hold forward pin on the CPU.

Page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별", §2.1: the input term
is g·B x with the gain g = (exp(δA) - 1)/A, so the adjoint uses g in dB and dx, ∂g/∂δ = Ā in
dδ and ∂g/∂A in dA.  The kernels form g and ∂g/∂A as series below |δA| = 1/8 and by their
closed forms above; the step sizes below put δA on both sides of that switch and at both
limits.  Tolerance as the first-order backward: 5e-4·max|ref| per gradient tensor.
"""
import numpy as np
import pytest

from gen import make_inputs, workload, workload_inputs
from oracle import cref
from tests.gpu_util import TOL_GRAD, assert_close, dev, note

pytestmark = pytest.mark.gpu

ZOH = 1
GRADS = ("dx", "ddt_raw", "dz", "ddt_bias", "dA", "dB", "dC", "dD", "dh0")


def gpu_bwd_zoh(ss, inp, gate, h0, dhf, chunk=0, ckpt=False, layout=0, disc=ZOH):
    import torch
    t = dev(inp)
    z = t["z"] if gate else None
    h0t = t["h0"] if h0 else None
    hck = None
    if ckpt:
        _, hck = ss.ss_fwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"],
                           z=z, h0=h0t, return_ckpt=True, layout=layout, disc=disc)
    g = ss.ss_bwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dy"],
                  z=z, h0=h0t, dh_final=t["dh_final"] if dhf else None, h_ckpt=hck, chunk=chunk,
                  disc=disc)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in g.items()}


def oracle_bwd_zoh(inp, gate, h0, dhf, zoh=True):
    return cref.bwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip, inp.dy,
                    z=inp.z if gate else None, h0=inp.h0 if h0 else None,
                    dh_final=inp.dh_final if dhf else None, zoh=zoh)


def compare(got, ref, tol=TOL_GRAD):
    errs = {}
    for k in GRADS:
        if ref[k] is None:
            assert got[k] is None, k
            continue
        errs[k] = assert_close(got[k], ref[k], tol, k)
    return errs


CASES = [
    # B, L, D, N, dtype, gate, h0, dh_final, chunk
    (1, 64, 64, 16, "f32", True, True, True, 0),
    (2, 200, 70, 16, "bf16", True, True, True, 0),      # ragged last chunk and tile, D % 64 != 0
    (1, 1, 5, 16, "f32", True, True, True, 0),
    (2, 7, 3, 4, "f32", False, True, False, 16),
    (1, 333, 40, 8, "bf16", True, False, True, 32),     # L % 8 != 0: element loads
    (2, 256, 16, 32, "f32", True, True, True, 64),
    (1, 96, 24, 2, "f32", True, True, True, 16),        # N = 2: padded states (A = 0 lanes)
    (3, 130, 9, 1, "bf16", False, True, True, 48),      # N = 1, odd L
    (1, 300, 1024, 16, "bf16", True, True, True, 0),    # sequential carries
]


@pytest.mark.parametrize("ckpt", [False, True], ids=["recompute", "ckpt"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}L{}D{}N{}-{}-g{}-h{}-f{}-c{}".format(*c))
def test_zoh_bwd_small(gpu, case, ckpt):
    Bn, L, D, N, dt, gate, h0, dhf, chunk = case
    inp = make_inputs(Bn, L, D, N, dtype=dt, seed=1300 + L + N, gate=gate, with_h0=h0,
                      with_dy=True, with_dh_final=dhf, a_perturb=True)
    note(f"zoh bwd {case} ckpt={ckpt}")
    got = gpu_bwd_zoh(gpu, inp, gate, h0, dhf, chunk, ckpt=ckpt)
    compare(got, oracle_bwd_zoh(inp, gate, h0, dhf))


# dt_bias -60: δ ~ 1e-26 (series, ∂g/∂A underflows); -2: δ ~ 0.13, so |δA_n| spans the switch
# at 1/8; -9.5 and 3: ordinary small and large steps; 50: exp(δA) = 0, g = -1/A, ∂g/∂A = 1/A²
@pytest.mark.parametrize("bias", [-60.0, -2.0, -9.5, 3.0, 50.0])
@pytest.mark.parametrize("ckpt", [False, True], ids=["recompute", "ckpt"])
def test_zoh_bwd_step_sizes(gpu, bias, ckpt):
    inp = make_inputs(2, 256, 64, 16, seed=18, gate=True, with_h0=True, with_dy=True,
                      with_dh_final=True, a_perturb=True)
    inp.dt_bias[:] = bias
    note(f"zoh bwd dt_bias={bias} ckpt={ckpt}")
    got = gpu_bwd_zoh(gpu, inp, True, True, True, ckpt=ckpt)
    compare(got, oracle_bwd_zoh(inp, True, True, True))


def test_zoh_bwd_differs_from_first_order(gpu):
    """The disc flag reaches the adjoint kernels: at δ ~ 0.7 the two holds' gradients differ
    by far more than the tolerance, and each matches its own oracle."""
    inp = make_inputs(1, 128, 64, 16, seed=19, gate=True, with_h0=True, with_dy=True,
                      with_dh_final=True, a_perturb=True)
    inp.dt_bias[:] = 0.0
    note("zoh bwd vs euler")
    g0 = gpu_bwd_zoh(gpu, inp, True, True, True, disc=0)
    g1 = gpu_bwd_zoh(gpu, inp, True, True, True, disc=ZOH)
    compare(g0, oracle_bwd_zoh(inp, True, True, True, zoh=False))
    compare(g1, oracle_bwd_zoh(inp, True, True, True))
    for k in ("dx", "ddt_raw", "dA", "dB"):
        scale = float(np.max(np.abs(g1[k])))
        assert float(np.max(np.abs(g1[k] - g0[k]))) > 20 * TOL_GRAD * scale, k


@pytest.mark.parametrize("layout", [1, 2, 3], ids=["quad", "lane", "oct"])
def test_zoh_bwd_checkpoints_from_every_layout(gpu, layout):
    """Exact-hold checkpoints written by each forward layout drive the backward to the same
    gradients as the recomputing backward."""
    inp = make_inputs(2, 520, 72, 16, dtype="bf16", seed=20, gate=True, with_h0=True,
                      with_dy=True, with_dh_final=True, a_perturb=True)
    note(f"zoh bwd checkpoints from layout {layout}")
    ref = gpu_bwd_zoh(gpu, inp, True, True, True)
    got = gpu_bwd_zoh(gpu, inp, True, True, True, ckpt=True, layout=layout)
    for k in GRADS:
        assert_close(got[k], ref[k], 2e-5, f"{k} layout={layout}")


@pytest.mark.parametrize("variant", [(1, False), (1, True), (0, True)],
                         ids=["tok", "tok-shared", "shared"])
@pytest.mark.parametrize("ckpt", [False, True], ids=["recompute", "ckpt"])
def test_zoh_bwd_variants(gpu, variant, ckpt):
    """Token-major tensors and a Δraw shared by the channels, with the exact hold."""
    import torch
    order, shared = variant
    inp = make_inputs(2, 200, 70, 16, dtype="bf16", seed=21, gate=True, with_h0=True,
                      with_dy=True, with_dh_final=True, a_perturb=True, dt_shared=shared)
    note(f"zoh bwd variant order={order} shared={shared} ckpt={ckpt}")
    dt = torch.bfloat16
    lay = (lambda a: np.ascontiguousarray(np.swapaxes(a, 1, 2))) if order == 1 else np.ascontiguousarray
    t_in = lambda a: torch.from_numpy(lay(a)).to(dt).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    x, z, Bm, Cm = t_in(inp.x), t_in(inp.z), t_in(inp.Bm), t_in(inp.Cm)
    dtr = torch.from_numpy(np.ascontiguousarray(inp.dt_tok)).to(dt).cuda() if shared else t_in(inp.dt_raw)
    dy = torch.from_numpy(lay(inp.dy).astype(np.float32)).cuda()
    dtb, A, Dk, h0, dhf = map(f32, (inp.dt_bias, inp.A, inp.Dskip, inp.h0, inp.dh_final))
    hck = None
    if ckpt:
        _, hck = gpu.ss_fwd(x, dtr, dtb, A, Bm, Cm, Dk, z=z, h0=h0, return_ckpt=True,
                            order=order, disc=ZOH)
    g = gpu.ss_bwd(x, dtr, dtb, A, Bm, Cm, Dk, dy, z=z, h0=h0, dh_final=dhf, h_ckpt=hck,
                   order=order, disc=ZOH)
    torch.cuda.synchronize()
    ref = oracle_bwd_zoh(inp, True, True, True)
    if shared:
        ref["ddt_raw"] = ref["ddt_raw"].sum(axis=1)
    back = lambda a: lay(a.cpu().numpy()) if order == 1 else a.cpu().numpy()
    for k in GRADS:
        seq = k in ("dx", "dz", "dB", "dC") or (k == "ddt_raw" and not shared)
        got = back(g[k]) if seq else g[k].cpu().numpy()
        assert_close(got, ref[k], TOL_GRAD, k)


def test_zoh_c4_full_backward(gpu):
    """The full B=4 L=4096 D=2048 N=16 bf16 fwd+bwd workload with the exact hold, in the
    training launch (forward checkpoints, then the backward), every gradient element."""
    w = workload("c4")
    inp = workload_inputs(w)
    note("zoh c4 backward full")
    got = gpu_bwd_zoh(gpu, inp, True, False, False, ckpt=True)
    errs = compare(got, oracle_bwd_zoh(inp, True, False, False))
    print("zoh c4 gradient errors:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
