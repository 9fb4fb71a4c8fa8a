"""Pins of the oracle's backward: fp64 central finite differences of the oracle's
own forward, the dot-product (adjoint) identity, and numpy = C.

The backward is the adjoint of the recurrence of the "3.2 선택적 스캔 알고리즘…"
page (§2.1 discretisation, §2.2 recurrence) with the readout and gate; its
recomputation scheme (§3.3) must reproduce exactly these gradients.
"""
import numpy as np
import pytest

from gen import make_inputs
from oracle import ss_ref

NAMES = ["x", "dt_raw", "dt_bias", "A", "Bm", "Cm", "Dskip", "z", "h0"]
GRAD = {"x": "dx", "dt_raw": "ddt_raw", "dt_bias": "ddt_bias", "A": "dA", "Bm": "dB",
        "Cm": "dC", "Dskip": "dD", "z": "dz", "h0": "dh0"}


def _case(seed=3, Bn=2, L=7, D=3, N=4, gate=True, h0=True):
    inp = make_inputs(Bn, L, D, N, seed=seed, gate=gate, with_h0=h0, with_dy=True,
                      with_dh_final=True, a_perturb=True)
    args = {k: (None if getattr(inp, k) is None else getattr(inp, k).astype(np.float64))
            for k in NAMES}
    return inp, args


def _loss(args, dy, dhf):
    y, hf = ss_ref.ss_fwd(args["x"], args["dt_raw"], args["dt_bias"], args["A"], args["Bm"],
                          args["Cm"], args["Dskip"], z=args["z"], h0=args["h0"])
    return float(np.sum(dy * y) + np.sum(dhf * hf))


def _bwd_numpy(args, dy, dhf):
    return ss_ref.ss_bwd(args["x"], args["dt_raw"], args["dt_bias"], args["A"], args["Bm"],
                         args["Cm"], args["Dskip"], dy, z=args["z"], h0=args["h0"], dh_final=dhf)


def _bwd_c(args, dy, dhf):
    from oracle import cref
    return cref.bwd(args["x"], args["dt_raw"], args["dt_bias"], args["A"], args["Bm"],
                    args["Cm"], args["Dskip"], dy, z=args["z"], h0=args["h0"], dh_final=dhf)


@pytest.mark.parametrize("gate,h0", [(True, True), (False, False)])
def test_finite_differences(gate, h0):
    inp, args = _case(gate=gate, h0=h0)
    dy = inp.dy.astype(np.float64)
    dhf = inp.dh_final.astype(np.float64)
    grads = _bwd_numpy(args, dy, dhf)
    eps = 1e-6
    for name in NAMES:
        if args[name] is None:
            assert grads[GRAD[name]] is None
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
        err = np.max(np.abs(g - fd)) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-6, f"d{name}: rel err {err:.2e}"


def test_dot_product_identity():
    """<dy, J v> = <J^T dy, v> for a random direction v over every input at once."""
    inp, args = _case(seed=5, L=9)
    dy = inp.dy.astype(np.float64)
    dhf = inp.dh_final.astype(np.float64)
    grads = _bwd_numpy(args, dy, dhf)
    rng = np.random.default_rng(0)
    v = {k: rng.standard_normal(a.shape) for k, a in args.items() if a is not None}
    eps = 1e-5
    plus = {k: (a + eps * v[k] if a is not None else None) for k, a in args.items()}
    minus = {k: (a - eps * v[k] if a is not None else None) for k, a in args.items()}
    jv = (_loss(plus, dy, dhf) - _loss(minus, dy, dhf)) / (2 * eps)
    jtdy = sum(float(np.sum(grads[GRAD[k]] * v[k])) for k in v)
    assert abs(jv - jtdy) <= 1e-7 * max(abs(jv), 1.0)


def test_numpy_equals_c_backward():
    from gen import round_bf16  # noqa: F401  (bf16-valued inputs exercise the same path)
    inp, args = _case(seed=7, Bn=3, L=33, D=5, N=16)
    dy = inp.dy.astype(np.float64)
    dhf = inp.dh_final.astype(np.float64)
    gn = _bwd_numpy(args, dy, dhf)
    gc = _bwd_c(args, dy, dhf)
    for k, a in gn.items():
        if a is None:
            assert gc[k] is None
            continue
        err = np.max(np.abs(a - gc[k])) / max(np.max(np.abs(a)), 1e-300)
        assert err < 1e-12, f"{k}: {err:.2e}"


def test_backward_recompute_from_chunks_equals_stored():
    """Recomputing states chunk by chunk from stored chunk-start states (the
    recomputation of §3.3) reproduces the stored-state gradients: the gradient
    depends only on the states, not on how they are obtained."""
    inp, args = _case(seed=9, Bn=1, L=24, D=2, N=3)
    dy = inp.dy.astype(np.float64)
    dhf = inp.dh_final.astype(np.float64)
    full = _bwd_numpy(args, dy, dhf)
    T = 8
    # split the sequence into chunks; backward of the chunk with the carried adjoint
    L = args["x"].shape[-1]
    sl = lambda a, s: None if a is None else np.ascontiguousarray(a[..., s])
    # chunk-start states from forward calls
    starts = [args["h0"]]
    for c0 in range(0, L - T, T):
        s = slice(c0, c0 + T)
        _, hf = ss_ref.ss_fwd(sl(args["x"], s), sl(args["dt_raw"], s), args["dt_bias"], args["A"],
                              sl(args["Bm"], s), sl(args["Cm"], s), args["Dskip"],
                              z=sl(args["z"], s), h0=starts[-1])
        starts.append(hf)
    g = dhf
    acc = {k: 0.0 for k in ("ddt_bias", "dA", "dD")}
    pieces = {k: [] for k in ("dx", "ddt_raw", "dz", "dB", "dC")}
    for ci in range(len(starts) - 1, -1, -1):
        s = slice(ci * T, (ci + 1) * T)
        r = ss_ref.ss_bwd(sl(args["x"], s), sl(args["dt_raw"], s), args["dt_bias"], args["A"],
                          sl(args["Bm"], s), sl(args["Cm"], s), args["Dskip"], sl(dy, s),
                          z=sl(args["z"], s), h0=starts[ci], dh_final=g)
        g = r["dh0"]
        for k in acc:
            acc[k] = acc[k] + r[k]
        for k in pieces:
            pieces[k].insert(0, r[k])
    np.testing.assert_allclose(g, full["dh0"], rtol=1e-12, atol=1e-14)
    for k in acc:
        np.testing.assert_allclose(acc[k], full[k], rtol=1e-12, atol=1e-14)
    for k in pieces:
        np.testing.assert_allclose(np.concatenate(pieces[k], -1), full[k], rtol=1e-12, atol=1e-14)
