"""Pins of the oracle's exact zero-order-hold backward (ss_bwd(..., zoh=True)).

The exact hold of page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별", §2.1,
makes the input term f·B x with f = (e^{δA} - 1)/A, so the adjoint picks up ∂f/∂δ = Ā and
∂f/∂A.  The forward it differentiates is pinned on its own (tests/test_oracle_zoh.py: exact
convolution kernel, Runge-Kutta integration of the ODE, both step-size limits); here the
backward is pinned to that forward by fp64 central finite differences over every input,
once at ordinary step sizes (the closed form of ∂f/∂A) and once at small ones (its series
branch), by the adjoint identity, by the δ -> 0 limit where both holds agree, and numpy = C.
"""
import numpy as np
import pytest

from gen import make_inputs
from oracle import ss_ref

NAMES = ["x", "dt_raw", "dt_bias", "A", "Bm", "Cm", "Dskip", "z", "h0"]
GRAD = {"x": "dx", "dt_raw": "ddt_raw", "dt_bias": "ddt_bias", "A": "dA", "Bm": "dB",
        "Cm": "dC", "Dskip": "dD", "z": "dz", "h0": "dh0"}


def _case(seed, Bn=2, L=7, D=3, N=4, gate=True, h0=True, bias=None):
    inp = make_inputs(Bn, L, D, N, seed=seed, gate=gate, with_h0=h0, with_dy=True,
                      with_dh_final=True, a_perturb=True)
    args = {k: (None if getattr(inp, k) is None else getattr(inp, k).astype(np.float64))
            for k in NAMES}
    if bias is not None:
        args["dt_bias"][:] = bias
    return args, inp.dy.astype(np.float64), inp.dh_final.astype(np.float64)


def _loss(args, dy, dhf, zoh=True):
    y, hf = ss_ref.ss_fwd(args["x"], args["dt_raw"], args["dt_bias"], args["A"], args["Bm"],
                          args["Cm"], args["Dskip"], z=args["z"], h0=args["h0"], zoh=zoh)
    return float(np.sum(dy * y) + np.sum(dhf * hf))


def _bwd(args, dy, dhf, zoh=True, impl="numpy"):
    a = (args["x"], args["dt_raw"], args["dt_bias"], args["A"], args["Bm"], args["Cm"],
         args["Dskip"], dy)
    if impl == "c":
        from oracle import cref
        return cref.bwd(*a, z=args["z"], h0=args["h0"], dh_final=dhf, zoh=zoh)
    return ss_ref.ss_bwd(*a, z=args["z"], h0=args["h0"], dh_final=dhf, zoh=zoh)


def _fd_errors(args, dy, dhf, grads, eps=1e-6):
    """Relative error, per input, of the gradients against central differences of the loss."""
    errs = {}
    for name in NAMES:
        if args[name] is None:
            continue
        base = args[name]
        fd = np.empty_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = base[i]
            base[i] = old + eps
            lp = _loss(args, dy, dhf)
            base[i] = old - eps
            lm = _loss(args, dy, dhf)
            base[i] = old
            fd[i] = (lp - lm) / (2 * eps)
        g = grads[GRAD[name]]
        errs[name] = float(np.max(np.abs(g - fd)) / max(np.max(np.abs(fd)), 1e-12))
    return errs


def _step_products(args):
    delta = ss_ref.softplus(args["dt_bias"][None, :, None] + args["dt_raw"])
    return np.abs(delta[:, :, :, None] * args["A"][None, :, None, :])


@pytest.mark.parametrize("regime,bias,gate,h0", [
    ("large_step", 0.0, True, True),      # |δA| >= 1e-2 nearly everywhere: closed form of ∂f/∂A
    ("mixed", None, True, True),          # the workload's step sizes: both branches
    ("mixed_nogate", None, False, False),
    ("small_step", -7.0, True, True),     # |δA| < 1e-2 everywhere: series of ∂f/∂A
])
def test_zoh_finite_differences(regime, bias, gate, h0):
    args, dy, dhf = _case(seed=31, gate=gate, h0=h0, bias=bias)
    frac = float((_step_products(args) >= 1e-2).mean())
    expect = {"large_step": (0.9, 1.0), "mixed": (0.2, 0.8), "mixed_nogate": (0.2, 0.8),
              "small_step": (0.0, 0.0)}[regime]
    assert expect[0] <= frac <= expect[1], frac
    grads = _bwd(args, dy, dhf)
    errs = _fd_errors(args, dy, dhf, grads)
    bad = {k: v for k, v in errs.items() if v >= 1e-6}
    assert not bad, f"{regime}: {bad}"


def test_zoh_first_order_gradients_fail_the_exact_hold():
    """The pins tell the two holds apart: first-order gradients against differences of the
    exact-hold forward miss in dx, dΔraw, dA and dB (at δ near 0.7, where the holds differ
    by far more than the pins' tolerance)."""
    args, dy, dhf = _case(seed=32, bias=0.0)
    errs = _fd_errors(args, dy, dhf, _bwd(args, dy, dhf, zoh=False))
    for name in ("x", "dt_raw", "A", "Bm"):
        assert errs[name] > 1e-3, (name, errs[name])


def test_zoh_dot_product_identity():
    args, dy, dhf = _case(seed=33, L=9)
    grads = _bwd(args, dy, dhf)
    rng = np.random.default_rng(1)
    v = {k: rng.standard_normal(a.shape) for k, a in args.items() if a is not None}
    eps = 1e-5
    plus = {k: (a + eps * v[k] if a is not None else None) for k, a in args.items()}
    minus = {k: (a - eps * v[k] if a is not None else None) for k, a in args.items()}
    jv = (_loss(plus, dy, dhf) - _loss(minus, dy, dhf)) / (2 * eps)
    jtdy = sum(float(np.sum(grads[GRAD[k]] * v[k])) for k in v)
    assert abs(jv - jtdy) <= 1e-7 * max(abs(jv), 1.0)


def test_zoh_small_step_limit():
    """δ -> 0 (dt_bias = -30): the exact hold's gradients approach the first-order ones."""
    args, dy, dhf = _case(seed=34, bias=-30.0)
    g1 = _bwd(args, dy, dhf, zoh=False)
    g2 = _bwd(args, dy, dhf, zoh=True)
    for k, a in g1.items():
        if a is None:
            continue
        err = np.max(np.abs(g2[k] - a)) / max(np.max(np.abs(a)), 1e-300)
        assert err < 1e-10, (k, err)


def test_zoh_dfda_branches_meet():
    """The series and closed form of ∂f/∂A agree where the branch switches (|δA| = 1e-2)."""
    delta = np.array([0.5, 0.5, 2e-3, 2e-3])
    A = np.array([-0.02 * (1 - 1e-9), -0.02 * (1 + 1e-9), -5.0 * (1 - 1e-9), -5.0 * (1 + 1e-9)])
    _, dfa = ss_ref.bbar_factor_grads(delta, A, True)
    assert abs(dfa[0] - dfa[1]) <= 1e-9 * abs(dfa[0])
    assert abs(dfa[2] - dfa[3]) <= 1e-9 * abs(dfa[2])


@pytest.mark.parametrize("gate,h0", [(True, True), (False, False)])
def test_zoh_numpy_equals_c_backward(gate, h0):
    args, dy, dhf = _case(seed=35, Bn=3, L=33, D=5, N=16, gate=gate, h0=h0)
    args["dt_bias"][0] = -7.0                       # one channel on the series branch
    gn = _bwd(args, dy, dhf)
    gc = _bwd(args, dy, dhf, impl="c")
    for k, a in gn.items():
        if a is None:
            assert gc[k] is None
            continue
        err = np.max(np.abs(a - gc[k])) / max(np.max(np.abs(a)), 1e-300)
        assert err < 1e-12, f"{k}: {err:.2e}"
