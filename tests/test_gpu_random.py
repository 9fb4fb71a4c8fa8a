"""Seeded random sweep of the boundary's option space against the fp64 oracle.

Every case draws its sizes and options from a fixed seed (so the list is the same on every
run and each case names itself): B, L, D, N, input dtype, gate, h0, plan, chunk, layout,
memory order, shared Δraw and discretisation for the forward; the same plus checkpoints for
the backward; and decode steps.  Half the forward and backward cases (by a hash of the case's
name) keep A = -(n+1), the S4D-real A on which the kernels take their power path, the others
perturb it.  Sizes stay small enough for the oracle to run in
milliseconds, but L and D are drawn across tile, chunk and workgroup boundaries (ragged
tails, L % 8 != 0, D off every block multiple).  Tolerances as everywhere: 1e-4 / 2e-3 ·
max|ref| for outputs, 5e-4 · max|ref| for gradients.
"""
import zlib

import numpy as np
import pytest

from gen import make_inputs
from oracle import cref
from tests.gpu_util import TOL_GRAD, assert_close, note, tol_for

pytestmark = pytest.mark.gpu

NS = (1, 2, 4, 8, 16, 32, 64)


def _fwd_cases(n=160, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        N = int(rng.choice(NS))
        order = int(rng.integers(2))
        c = dict(B=int(rng.integers(1, 4)), L=int(rng.choice([1, 7, 8, 31, 64, 100, 257, 700, 1500, 2049, 4104])),
                 D=int(rng.choice([1, 3, 17, 64, 65, 130, 300, 1030])), N=N,
                 dt=str(rng.choice(["f32", "bf16"])), gate=bool(rng.integers(2)),
                 h0=bool(rng.integers(2)), plan=int(rng.integers(3)), layout=int(rng.integers(4)),
                 order=order, shared=bool(rng.integers(2)), disc=int(rng.integers(2)))
        c["chunk"] = int(rng.choice([0, 0, 32, 64, 96])) if c["plan"] == 2 else 0
        # N = 64 runs on eight lanes only (automatic or eight-lane layout, rows it can tile)
        if N == 64 and (c["layout"] in (1, 2) or (order == 0 and c["L"] % 8)):
            continue
        out.append(c)
    return out


def _bwd_cases(n=64, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append(dict(B=int(rng.integers(1, 4)), L=int(rng.choice([1, 15, 16, 40, 64, 100, 333, 1000])),
                        D=int(rng.choice([1, 5, 64, 70, 129, 260])), N=int(rng.choice(NS[:-1])),
                        dt=str(rng.choice(["f32", "bf16"])), gate=bool(rng.integers(2)),
                        h0=bool(rng.integers(2)), dhf=bool(rng.integers(2)),
                        chunk=int(rng.choice([0, 16, 32, 48, 64])), ckpt=bool(rng.integers(2)),
                        order=int(rng.integers(2)), shared=bool(rng.integers(2)),
                        disc=int(rng.integers(2))))
    return out


def _name(c):
    return "-".join(f"{k}{int(v) if isinstance(v, bool) else v}" for k, v in c.items())


def _perturb_a(c):
    """A perturbed (general exponentials) or exactly -(n+1) (the power path), half each."""
    return zlib.crc32(("A" + _name(c)).encode()) % 2 == 0


def _to_dev(inp, c):
    """Device tensors of a case in its memory order (Δraw [B, L] when shared)."""
    import torch
    tdt = torch.bfloat16 if c["dt"] == "bf16" else torch.float32
    lay = (lambda a: np.ascontiguousarray(np.swapaxes(a, 1, 2))) if c["order"] else np.ascontiguousarray
    t_in = lambda a: None if a is None else torch.from_numpy(lay(a)).to(tdt).cuda()
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    d = dict(x=t_in(inp.x), z=t_in(inp.z), Bm=t_in(inp.Bm), Cm=t_in(inp.Cm),
             dt_bias=f32(inp.dt_bias), A=f32(inp.A), Dskip=f32(inp.Dskip), h0=f32(inp.h0),
             dh_final=f32(inp.dh_final))
    d["dt_raw"] = (torch.from_numpy(np.ascontiguousarray(inp.dt_tok)).to(tdt).cuda()
                   if c["shared"] else t_in(inp.dt_raw))
    d["dy"] = None if inp.dy is None else torch.from_numpy(lay(inp.dy).astype(np.float32)).cuda()
    return d


def _back(t, c):
    a = t.cpu().numpy()
    return np.swapaxes(a, 1, 2) if c["order"] else a


@pytest.mark.parametrize("c", _fwd_cases(), ids=_name)
def test_random_fwd(gpu, c):
    import torch
    inp = make_inputs(c["B"], c["L"], c["D"], c["N"], dtype=c["dt"], seed=zlib.crc32(_name(c).encode()),
                      gate=c["gate"], with_h0=c["h0"], a_perturb=_perturb_a(c), dt_shared=c["shared"])
    note(f"random fwd {_name(c)} a_perturb={_perturb_a(c)}")
    t = _to_dev(inp, c)
    y, hf = gpu.ss_fwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"],
                       z=t["z"], h0=t["h0"], return_final=True, plan=c["plan"], chunk=c["chunk"],
                       layout=c["layout"], disc=c["disc"], order=c["order"])
    torch.cuda.synchronize()
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z, h0=inp.h0, zoh=bool(c["disc"]))
    assert_close(_back(y, c), yr, tol_for(inp), "y")
    assert_close(hf.cpu().numpy(), hr, tol_for(inp), "h_final")


@pytest.mark.parametrize("c", _bwd_cases(), ids=_name)
def test_random_bwd(gpu, c):
    import torch
    inp = make_inputs(c["B"], c["L"], c["D"], c["N"], dtype=c["dt"], seed=zlib.crc32(_name(c).encode()),
                      gate=c["gate"], with_h0=c["h0"], with_dy=True, with_dh_final=c["dhf"],
                      a_perturb=_perturb_a(c), dt_shared=c["shared"])
    note(f"random bwd {_name(c)} a_perturb={_perturb_a(c)}")
    t = _to_dev(inp, c)
    args = (t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"])
    hck = None
    if c["ckpt"]:
        _, hck = gpu.ss_fwd(*args, z=t["z"], h0=t["h0"], return_ckpt=True, disc=c["disc"],
                            order=c["order"])
    g = gpu.ss_bwd(*args, t["dy"], z=t["z"], h0=t["h0"], dh_final=t["dh_final"] if c["dhf"] else None,
                   h_ckpt=hck, chunk=c["chunk"], disc=c["disc"], order=c["order"])
    torch.cuda.synchronize()
    ref = cref.bwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip, inp.dy,
                   z=inp.z, h0=inp.h0, dh_final=inp.dh_final if c["dhf"] else None,
                   zoh=bool(c["disc"]))
    if c["shared"]:
        ref["ddt_raw"] = ref["ddt_raw"].sum(axis=1)
    for k in ("dx", "ddt_raw", "dz", "ddt_bias", "dA", "dB", "dC", "dD", "dh0"):
        if ref[k] is None:
            assert g[k] is None, k
            continue
        seq = k in ("dx", "dz", "dB", "dC") or (k == "ddt_raw" and not c["shared"])
        got = _back(g[k], c) if seq else g[k].cpu().numpy()
        assert_close(got, ref[k], TOL_GRAD, k)


@pytest.mark.parametrize("seed", range(16))
def test_random_step(gpu, seed):
    import torch
    rng = np.random.default_rng(7000 + seed)
    B, D, N = int(rng.integers(1, 6)), int(rng.choice([1, 3, 33, 70, 257])), int(rng.choice(NS))
    dt, gate = str(rng.choice(["f32", "bf16"])), bool(rng.integers(2))
    shared, disc = bool(rng.integers(2)), int(rng.integers(2))
    T = 5
    inp = make_inputs(B, T, D, N, dtype=dt, seed=7100 + seed, gate=gate, with_h0=True,
                      a_perturb=True, dt_shared=shared)
    note(f"random step seed={seed} B{B} D{D} N{N} {dt} g{gate} s{shared} z{disc}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    col = lambda a, t: torch.from_numpy(np.ascontiguousarray(a[..., t])).to(tdt).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    h = f32(inp.h0)
    ys = []
    for t in range(T):
        dr = col(inp.dt_tok, t) if shared else col(inp.dt_raw, t)
        ys.append(gpu.ss_step(col(inp.x, t), dr, f32(inp.dt_bias), f32(inp.A), col(inp.Bm, t),
                              col(inp.Cm, t), f32(inp.Dskip), h, z=col(inp.z, t) if gate else None,
                              disc=disc).cpu().numpy())
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z, h0=inp.h0, zoh=bool(disc))
    assert_close(np.stack(ys, axis=-1), yr, tol_for(inp), "y")
    assert_close(h.cpu().numpy(), hr, tol_for(inp), "state")
