"""GPU parity of the backward (ss_bwd through the C ABI) against the fp64 oracle.

Every gradient is compared element by element: max|g_gpu - g_ref| <= 5e-4·max|g_ref|
per tensor.  The full S6 fwd+bwd workload (B=4 L=4096 D=2048 N=16, bf16 inputs, gate)
is compared in full against the C oracle's backward.
"""
import numpy as np
import pytest

from gen import make_inputs, workload, workload_inputs
from oracle import cref
from tests.gpu_util import TOL_GRAD, assert_close, dev, note

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt_raw", "dz", "ddt_bias", "dA", "dB", "dC", "dD", "dh0")


def gpu_bwd(ss, inp, gate, h0, dhf, chunk=0, ckpt=False, layout=0):
    """ss_bwd; with ckpt, on the checkpoints of an ss_fwd call (in the given layout)."""
    import torch
    t = dev(inp)
    hck = None
    if ckpt:
        _, hck = ss.ss_fwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"],
                           z=t["z"] if gate else None, h0=t["h0"] if h0 else None,
                           return_ckpt=True, layout=layout)
    g = ss.ss_bwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dy"],
                  z=t["z"] if gate else None, h0=t["h0"] if h0 else None,
                  dh_final=t["dh_final"] if dhf else None, h_ckpt=hck, chunk=chunk)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in g.items()}


def oracle_bwd(inp, gate, h0, dhf):
    return cref.bwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip, inp.dy,
                    z=inp.z if gate else None, h0=inp.h0 if h0 else None,
                    dh_final=inp.dh_final if dhf else None)


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
    (1, 96, 24, 2, "f32", True, True, True, 16),        # N = 2: two padded states per quad
    (3, 130, 9, 1, "bf16", False, True, True, 48),      # N = 1, odd L
    (2, 1024, 130, 16, "bf16", True, False, False, 0),
    (1, 300, 1024, 16, "bf16", True, True, True, 0),    # B*D*N >= 16384: sequential carries
]


@pytest.mark.parametrize("ckpt", [False, True], ids=["recompute", "ckpt"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}L{}D{}N{}-{}-g{}-h{}-f{}-c{}".format(*c))
def test_bwd_small(gpu, case, ckpt):
    Bn, L, D, N, dt, gate, h0, dhf, chunk = case
    inp = make_inputs(Bn, L, D, N, dtype=dt, seed=300 + L + N, gate=gate, with_h0=h0, with_dy=True,
                      with_dh_final=dhf, a_perturb=True)
    note(f"bwd {case} ckpt={ckpt}")
    got = gpu_bwd(gpu, inp, gate, h0, dhf, chunk, ckpt=ckpt)
    ref = oracle_bwd(inp, gate, h0, dhf)
    compare(got, ref)


def test_bwd_deterministic(gpu):
    inp = make_inputs(2, 512, 96, 16, dtype="bf16", seed=5, gate=True, with_h0=True, with_dy=True,
                      with_dh_final=True)
    note("bwd determinism")
    a = gpu_bwd(gpu, inp, True, True, True)
    b = gpu_bwd(gpu, inp, True, True, True)
    for k in GRADS:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


def test_bwd_chunk_sizes_agree(gpu):
    inp = make_inputs(1, 640, 64, 16, seed=6, gate=True, with_h0=True, with_dy=True, with_dh_final=True)
    note("bwd chunk sizes")
    ref = gpu_bwd(gpu, inp, True, True, True, chunk=64)
    for c in (16, 32, 48):
        got = gpu_bwd(gpu, inp, True, True, True, chunk=c)
        for k in GRADS:
            assert_close(got[k], ref[k], 2e-5, f"{k} chunk={c}")


@pytest.mark.parametrize("layout", [1, 2, 3], ids=["quad", "lane", "oct"])
def test_bwd_checkpoints_from_every_layout(gpu, layout):
    """Checkpoints written by each forward layout drive the backward to the same result."""
    inp = make_inputs(2, 520, 72, 16, dtype="bf16", seed=7, gate=True, with_h0=True, with_dy=True,
                      with_dh_final=True, a_perturb=True)
    note(f"bwd checkpoints from layout {layout}")
    ref = gpu_bwd(gpu, inp, True, True, True)
    got = gpu_bwd(gpu, inp, True, True, True, ckpt=True, layout=layout)
    for k in GRADS:
        assert_close(got[k], ref[k], 2e-5, f"{k} layout={layout}")


@pytest.mark.parametrize("ckpt", [False, True], ids=["recompute", "ckpt"])
def test_c4_full_backward(gpu, ckpt):
    """The full B=4 L=4096 D=2048 N=16 bf16 fwd+bwd workload, every gradient element."""
    w = workload("c4")
    inp = workload_inputs(w)
    note(f"c4 backward full ckpt={ckpt}")
    got = gpu_bwd(gpu, inp, True, False, False, ckpt=ckpt)
    ref = oracle_bwd(inp, True, False, False)
    errs = compare(got, ref)
    print("c4 gradient errors:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)


@pytest.mark.parametrize("ckpt", [False, True], ids=["recompute", "ckpt"])
@pytest.mark.parametrize("N", [8, 16, 32])
def test_bwd_s4d_detection_per_wave(gpu, N, ckpt):
    """A = -(n+1) except for one state of one channel: the wave holding that channel runs the
    general exponentials, the others the power path (one exponential and a chain of products
    per lane) in the aggregate and final passes; every gradient matches the oracle."""
    inp = make_inputs(2, 300, 200, N, dtype="f32", seed=40 + N, gate=True, with_h0=True,
                      with_dy=True, with_dh_final=True)
    inp.A[77, N // 2 - 1] *= 1.01
    note(f"bwd s4d detection N={N} ckpt={ckpt}")
    got = gpu_bwd(gpu, inp, True, True, True, ckpt=ckpt)
    ref = oracle_bwd(inp, True, True, True)
    compare(got, ref)


@pytest.mark.parametrize("ckpt", [False, True])
def test_bwd_power_mixed_steps(gpu, ckpt):
    """A = -(n+1) with per-channel dt_bias from Δ→0 to Δ→∞ in every wave: the reverse pairs'
    chain started from ds times the first state's factor, the final pass's power path and the
    partial-plane channel sums; every gradient matches the oracle."""
    inp = make_inputs(2, 640, 64, 16, dtype="f32", seed=93, gate=True, with_h0=True,
                      with_dy=True, with_dh_final=True)
    inp.dt_bias[:] = np.resize(np.array([-60.0, -9.5, -2.0, 0.5, 3.0, 50.0], np.float32),
                               inp.dt_bias.shape)
    note(f"bwd power path mixed step sizes ckpt={ckpt}")
    got = gpu_bwd(gpu, inp, True, True, True, ckpt=ckpt)
    ref = oracle_bwd(inp, True, True, True)
    compare(got, ref)
