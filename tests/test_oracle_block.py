"""Pins of the block oracle (oracle/block_ref.py): the selection projections and the gated
block around the scan.

[SEL] "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별", §1.2: B_t, C_t are
N-output linear maps of the token and Δ_t = softplus(Parameter + one-output linear map);
[SSM] "상태공간 모델(SSM)과 Mamba 아키텍처", §3: the input is projected two ways, one branch
through the scan, the other through the SiLU gate.  Checked against pure-Python loops on tiny
shapes, against a permutation special case that reduces the block to the scan oracle on
known inputs, and by planted mistakes that must each fail a pin.
"""
import numpy as np
import pytest

from gen import make_block_inputs
from oracle import block_ref, ss_ref


def _loops(u, W_in, W_x):
    """Projections by explicit loops: xz[b,t,o] = Σ_i u[b,t,i] W_in[o,i], etc."""
    Bn, L, Din = u.shape
    D2 = W_in.shape[0]
    D = D2 // 2
    P = W_x.shape[0]
    N = (P - 1) // 2
    xz = np.zeros((Bn, L, D2))
    for b in range(Bn):
        for t in range(L):
            for o in range(D2):
                s = 0.0
                for i in range(Din):
                    s += float(u[b, t, i]) * float(W_in[o, i])
                xz[b, t, o] = s
    x, z = xz[..., :D], xz[..., D:]
    p = np.zeros((Bn, L, P))
    for b in range(Bn):
        for t in range(L):
            for o in range(P):
                s = 0.0
                for d in range(D):
                    s += x[b, t, d] * float(W_x[o, d])
                p[b, t, o] = s
    return x, z, p[..., 0], p[..., 1:1 + N], p[..., 1 + N:]


def _scan_tokmajor(x, z, dt, Bm, Cm, inp):
    """The scan oracle on token-major intermediates, Δraw broadcast over channels."""
    Bn, L, D = x.shape
    cm = lambda a: np.swapaxes(a, 1, 2)
    y, hf = ss_ref.ss_fwd(cm(x), np.broadcast_to(dt[:, None, :], (Bn, D, L)), inp.dt_bias,
                          inp.A, cm(Bm), cm(Cm), inp.Dskip, z=cm(z), h0=inp.h0)
    return np.swapaxes(y, 1, 2), hf


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


def pin_loops(fwd, seed=1, Bn=2, L=5, Din=6, D=4, N=3):
    inp = make_block_inputs(Bn, L, Din, D, N, seed=seed, with_h0=True)
    out = fwd(inp.u, inp.W_in, inp.W_x, inp.dt_bias, inp.A, inp.Dskip, h0=inp.h0)
    x, z, dt, Bm, Cm = _loops(inp.u, inp.W_in, inp.W_x)
    y, hf = _scan_tokmajor(x, z, dt, Bm, Cm, inp)
    return max(rel(out["x"], x), rel(out["z"], z), rel(out["dt"], dt), rel(out["B"], Bm),
               rel(out["C"], Cm), rel(out["y"], y), rel(out["h_final"], hf))


def pin_permutation(fwd, seed=2, Bn=1, L=9, D=5, N=2):
    """D_in = D, W_in = [P; Q] with permutations P, Q (not symmetric): x = u Pᵀ, z = u Qᵀ,
    and W_x rows that pick single channels of x, so every intermediate is a known
    rearrangement of u and the output is the scan of those rearranged inputs."""
    inp = make_block_inputs(Bn, L, D, D, N, seed=seed, with_h0=True)
    rng = np.random.default_rng(seed)
    p, q = rng.permutation(D), np.roll(np.arange(D), 1)
    W_in = np.zeros((2 * D, D), np.float32)
    W_in[np.arange(D), p] = 1.0
    W_in[D + np.arange(D), q] = 1.0
    pick = rng.integers(0, D, size=1 + 2 * N)
    W_x = np.zeros((1 + 2 * N, D), np.float32)
    W_x[np.arange(1 + 2 * N), pick] = 1.0
    out = fwd(inp.u, W_in, W_x, inp.dt_bias, inp.A, inp.Dskip, h0=inp.h0)
    u = inp.u.astype(np.float64)
    x, z = u[..., p], u[..., q]
    dt, Bm, Cm = x[..., pick[0]], x[..., pick[1:1 + N]], x[..., pick[1 + N:]]
    y, hf = _scan_tokmajor(x, z, dt, Bm, Cm, inp)
    return max(rel(out["x"], x), rel(out["z"], z), rel(out["y"], y), rel(out["h_final"], hf))


PINS = {"loops": (pin_loops, 1e-12), "permutation": (pin_permutation, 1e-12)}


@pytest.mark.parametrize("pin", sorted(PINS))
def test_block_pin(pin):
    f, tol = PINS[pin]
    err = f(block_ref.block_fwd)
    assert err <= tol, f"{pin}: {err:.3e}"


def test_block_c_scan_matches_numpy():
    """impl="c" (float32 inputs to the C scan) agrees with the float64 numpy path."""
    inp = make_block_inputs(2, 40, 16, 24, 8, seed=3, with_h0=True)
    a = block_ref.block_fwd(inp.u, inp.W_in, inp.W_x, inp.dt_bias, inp.A, inp.Dskip, h0=inp.h0)
    b = block_ref.block_fwd(inp.u, inp.W_in, inp.W_x, inp.dt_bias, inp.A, inp.Dskip, h0=inp.h0,
                            impl="c")
    assert rel(b["y"], a["y"]) < 1e-6 and rel(b["h_final"], a["h_final"]) < 1e-6
    chans = np.array([0, 5, 47])
    c = block_ref.block_fwd(inp.u, inp.W_in, inp.W_x, inp.dt_bias, inp.A, inp.Dskip, h0=inp.h0,
                            impl="c", chans=chans)
    ycm = np.swapaxes(a["y"], 1, 2).reshape(-1, 40)
    assert rel(c["y"], ycm[chans]) < 1e-6


def _mutant(kind):
    def fwd(u, W_in, W_x, dt_bias, A, Dskip, h0=None):
        u64, Wi, Wx = (np.asarray(v, np.float64) for v in (u, W_in, W_x))
        D = Wi.shape[0] // 2
        N = (Wx.shape[0] - 1) // 2
        xz = u64 @ Wi.T
        x, z = (xz[..., D:], xz[..., :D]) if kind == "swap_xz" else (xz[..., :D], xz[..., D:])
        p = x @ Wx.T
        dt, Bm, Cm = p[..., 0], p[..., 1:1 + N], p[..., 1 + N:]
        if kind == "swap_bc":
            Bm, Cm = Cm, Bm
        if kind == "dt_last":
            dt = p[..., -1]
        if kind == "gate_from_x":
            z = x
        Bn, L, _ = x.shape
        cm = lambda a: np.swapaxes(a, 1, 2)
        y, hf = ss_ref.ss_fwd(cm(x), np.broadcast_to(dt[:, None, :], (Bn, D, L)), dt_bias, A,
                              cm(Bm), cm(Cm), Dskip, z=cm(z), h0=h0)
        return dict(x=x, z=z, dt=dt, B=Bm, C=Cm, y=np.swapaxes(y, 1, 2), h_final=hf)
    return fwd


@pytest.mark.parametrize("kind", ["swap_xz", "swap_bc", "dt_last", "gate_from_x"])
def test_block_pins_catch_planted_mistakes(kind):
    bad = _mutant(kind)
    assert any(f(bad) > tol for f, tol in PINS.values()), kind


def test_block_weights_transposed_is_caught():
    """A projection with W instead of Wᵀ (square case, D_in = 2D) fails the loop pin."""
    def fwd(u, W_in, W_x, dt_bias, A, Dskip, h0=None):
        out = block_ref.block_fwd(u, np.ascontiguousarray(W_in.T), W_x, dt_bias, A, Dskip, h0=h0)
        return out
    inp = make_block_inputs(1, 4, 8, 4, 2, seed=5, with_h0=True)
    out = fwd(inp.u, inp.W_in, inp.W_x, inp.dt_bias, inp.A, inp.Dskip, h0=inp.h0)
    x, *_ = _loops(inp.u, inp.W_in, inp.W_x)
    assert rel(out["x"], x) > 1e-3
