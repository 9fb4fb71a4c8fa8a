"""Pins of the oracle's exact zero-order-hold variant (zoh=True).

Page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별", §2.1: discretising
dh/dt = A h + B x with x held constant over a step of length δ gives
    Ā = exp(δA),   B̄ = (δA)^{-1}(exp(δA) - I)·δB = (exp(δA) - 1)/A · B   (A diagonal),
and §1.1 (with the note "상태공간 모델(SSM)과 Mamba 아키텍처", §2): with constant
parameters the recurrence is a convolution with K_k = C Ā^k B̄.  Each pin checks the oracle
against something it does not compute itself: np.convolve over the exact kernel, a
numerical integration of the ODE over every step (classical Runge-Kutta, many substeps),
the δ→0 limit (the first-order form) and the δ→∞ limit (the ODE's steady state -Bx/A).
Both oracle implementations (numpy, C) are checked, and planted mistakes must fail a pin.
"""
import numpy as np
import pytest

from gen import make_inputs
from oracle import ss_ref


def _c_fwd(*args, z=None, h0=None, zoh=False):
    from oracle import cref
    return cref.fwd(*args, z=z, h0=h0, zoh=zoh)


def _np_fwd(*args, z=None, h0=None, zoh=False):
    return ss_ref.ss_fwd(*args, z=z, h0=h0, zoh=zoh)


IMPLS = {"numpy": _np_fwd, "c": _c_fwd}


@pytest.fixture(params=sorted(IMPLS))
def fwd(request):
    return IMPLS[request.param]


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def pin_zoh_lti(fwd, seed=21, L=64, D=3, N=5, Bn=2):
    """Constant δ, B, C, no gate, h0 = 0: y = x * K + D x, K_k = Σ_n C_n Ā_n^k (Ā_n - 1)/A_n B_n."""
    inp = make_inputs(Bn, L, D, N, seed=seed, a_perturb=True)
    rng = np.random.default_rng(seed)
    dt_raw = np.repeat(rng.standard_normal((Bn, D, 1)), L, axis=2).astype(np.float32)
    B0 = rng.standard_normal((Bn, N, 1)).astype(np.float32)
    C0 = rng.standard_normal((Bn, N, 1)).astype(np.float32)
    Bm, Cm = np.repeat(B0, L, axis=2), np.repeat(C0, L, axis=2)
    y, _ = fwd(inp.x, dt_raw, inp.dt_bias, inp.A, Bm, Cm, inp.Dskip, zoh=True)
    worst = 0.0
    for b in range(Bn):
        for d in range(D):
            u = float(inp.dt_bias[d]) + float(dt_raw[b, d, 0])
            delta = np.logaddexp(0.0, u)                       # softplus, by the library
            a = inp.A[d].astype(np.float64)
            abar = np.exp(delta * a)
            bbar = (abar - 1.0) / a * B0[b, :, 0].astype(np.float64)
            K = (C0[b, :, 0][None, :] * abar[None, :] ** np.arange(L)[:, None] * bbar[None, :]).sum(1)
            xd = inp.x[b, d].astype(np.float64)
            ref = np.convolve(xd, K)[:L] + float(inp.Dskip[d]) * xd
            worst = max(worst, rel_err(y[b, d], ref))
    return worst


def pin_zoh_ode(fwd, seed=22, L=6, D=2, N=3, Bn=1, substeps=4000):
    """States match a Runge-Kutta integration of dh/dt = A h + B_t x_t over each step of
    length δ_t (x and B held constant within the step), started from h0."""
    inp = make_inputs(Bn, L, D, N, seed=seed, with_h0=True, a_perturb=True)
    worst = 0.0
    for Lp in range(1, L + 1):
        cut = lambda arr: np.ascontiguousarray(arr[..., :Lp])
        _, hf = fwd(cut(inp.x), cut(inp.dt_raw), inp.dt_bias, inp.A, cut(inp.Bm), cut(inp.Cm),
                    inp.Dskip, h0=inp.h0, zoh=True)
        for b in range(Bn):
            for d in range(D):
                h = inp.h0[b, d].astype(np.float64)
                a = inp.A[d].astype(np.float64)
                for t in range(Lp):
                    delta = np.logaddexp(0.0, float(inp.dt_bias[d]) + float(inp.dt_raw[b, d, t]))
                    f = inp.Bm[b, :, t].astype(np.float64) * float(inp.x[b, d, t])
                    k = delta / substeps
                    for _ in range(substeps):
                        k1 = a * h + f
                        k2 = a * (h + 0.5 * k * k1) + f
                        k3 = a * (h + 0.5 * k * k2) + f
                        k4 = a * (h + k * k3) + f
                        h = h + k / 6.0 * (k1 + 2 * k2 + 2 * k3 + k4)
                worst = max(worst, rel_err(hf[b, d], h))
    return worst


def pin_zoh_small_step(fwd, seed=23, L=32, D=4, N=6):
    """δ → 0 (dt_bias = -30): exact hold and first order agree to O(δ|A|)."""
    inp = make_inputs(1, L, D, N, seed=seed, with_h0=True, a_perturb=True)
    inp.dt_bias[:] = -30.0
    args = (inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip)
    y1, h1 = fwd(*args, h0=inp.h0, zoh=False)
    y2, h2 = fwd(*args, h0=inp.h0, zoh=True)
    return max(rel_err(y2, y1), rel_err(h2, h1))


def pin_zoh_large_step(fwd, seed=24, L=16, D=3, N=4):
    """δ → ∞ (dt_bias = +50, A <= -1): Ā = 0 and B̄x = -B x / A, the ODE's steady state."""
    inp = make_inputs(1, L, D, N, seed=seed, with_h0=True, a_perturb=True)
    inp.dt_bias[:] = 50.0
    _, hf = fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip, h0=inp.h0,
                zoh=True)
    ref = -(inp.Bm[0, :, -1][None, :].astype(np.float64) * inp.x[0, :, -1][:, None]) / inp.A
    return rel_err(hf[0], ref)


def pin_zoh_golden(fwd):
    """Hand-unrolled exact-hold cases (tests/golden/hand_unrolled_zoh.json): δ = ln 2 makes
    the gains 1/2 (A = -1) and 3/8 (A = -2), and ln 2 itself at A = 0."""
    import json
    import math
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_unrolled_zoh.json")) as f:
        cases = json.load(f)["cases"]
    ln2 = math.log(2.0)
    worst = 0.0
    for c in cases:
        L, N = c["L"], c["N"]
        x = np.array(c["x"], np.float32).reshape(1, 1, L)
        dtr = np.array(c["dt_raw"], np.float32).reshape(1, 1, L)
        dtb = np.array([c["dt_bias"]], np.float32)
        A = np.array(c["A"], np.float32).reshape(1, N)
        Bm = np.array(c["B"], np.float32).reshape(1, N, L)
        Cm = np.array(c["C"], np.float32).reshape(1, N, L)
        Dk = np.array([c["D"]], np.float32)
        h0 = None if c["h0"] is None else np.array(c["h0"], np.float32).reshape(1, 1, N)
        y, hf = fwd(x, dtr, dtb, A, Bm, Cm, Dk, h0=h0, zoh=True)
        y_exp = np.array([p + q * ln2 for p, q in c["y"]])
        h_exp = np.array([p + q * ln2 for p, q in c["h_final"]])
        worst = max(worst, rel_err(np.asarray(y).reshape(-1), y_exp),
                    rel_err(np.asarray(hf).reshape(-1), h_exp))
    return worst


PINS = {"zoh_lti": (pin_zoh_lti, 1e-12), "zoh_ode": (pin_zoh_ode, 1e-10),
        "zoh_small_step": (pin_zoh_small_step, 1e-10), "zoh_large_step": (pin_zoh_large_step, 1e-12),
        "zoh_golden": (pin_zoh_golden, 1e-12)}


@pytest.mark.parametrize("pin", sorted(PINS))
def test_zoh_pin(fwd, pin):
    f, tol = PINS[pin]
    err = f(fwd)
    assert err <= tol, f"{pin}: {err:.3e} > {tol:.1e}"


def test_zoh_numpy_equals_c():
    inp = make_inputs(2, 96, 5, 16, dtype="bf16", seed=25, gate=True, with_h0=True,
                      a_perturb=True)
    args = (inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip)
    y1, h1 = _np_fwd(*args, z=inp.z, h0=inp.h0, zoh=True)
    y2, h2 = _c_fwd(*args, z=inp.z, h0=inp.h0, zoh=True)
    assert rel_err(y2, y1) <= 1e-12 and rel_err(h2, h1) <= 1e-12


def test_zoh_differs_from_first_order():
    """At ordinary step sizes the two discretisations give different outputs."""
    inp = make_inputs(1, 64, 4, 8, seed=26, a_perturb=True)
    args = (inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip)
    y1, _ = _np_fwd(*args)
    y2, _ = _np_fwd(*args, zoh=True)
    assert rel_err(y2, y1) > 1e-4


# planted mistakes in a copy of the exact-hold oracle: each must fail some pin
def _mutant(kind):
    def fwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z=None, h0=None, zoh=True):
        x, dt_raw, dt_bias, A, Bm, Cm, Dskip = (np.asarray(v, np.float64) for v in
                                                (x, dt_raw, dt_bias, A, Bm, Cm, Dskip))
        Bn, D, L = x.shape
        N = A.shape[1]
        delta = ss_ref.softplus(dt_bias[None, :, None] + dt_raw)
        h = np.zeros((Bn, D, N)) if h0 is None else np.asarray(h0, np.float64).copy()
        y = np.empty((Bn, D, L))
        for t in range(L):
            dl = delta[:, :, t, None]
            abar = np.exp(dl * A[None])
            if not zoh:
                fb = dl
            elif kind == "exp_not_expm1":
                fb = np.exp(dl * A[None]) / A[None]
            elif kind == "no_divide_by_A":
                fb = np.expm1(dl * A[None])
            elif kind == "sign":
                fb = -np.expm1(dl * A[None]) / A[None]
            else:
                fb = np.expm1(dl * A[None]) / A[None]
            h = abar * h + fb * Bm[:, None, :, t] * x[:, :, t, None]
            y[:, :, t] = (Cm[:, None, :, t] * h).sum(-1) + Dskip[None] * x[:, :, t]
        return y, h
    return fwd


@pytest.mark.parametrize("kind", ["exp_not_expm1", "no_divide_by_A", "sign"])
def test_zoh_pins_catch_planted_mistakes(kind):
    bad = _mutant(kind)
    caught = []
    for name, (f, tol) in PINS.items():
        if name == "zoh_ode":
            continue  # slow; the other pins suffice for these mutants
        with np.errstate(divide="ignore", invalid="ignore"):
            err = f(bad)
        if not err <= tol:        # a NaN error (0/0 of a planted form) counts as caught
            caught.append(name)
    assert caught, f"no pin caught mutant {kind}"
