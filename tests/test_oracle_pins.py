"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each pin checks the oracle (both the numpy and the C implementation) against a
value it does not compute itself: hand-worked golden numbers, the LTI
convolution identity computed with np.convolve, the Δ→0 / Δ→∞ limits, a
brute-force closed form, arbitrary bracketings of the associative operator,
split-call resume, linearity, and library routines for softplus / sigmoid / SiLU.
test_pins_catch_planted_mistakes plants plausible mistakes in a copy of the
oracle and checks that some pin fails for each.

Sources: "3.2 선택적 스캔(Selective Scan) 알고리즘…" page (§1.1 LTI equations and
convolution kernel, §1.2 selection, §2.1 ZOH, §2.2 associative operator,
§4.1 Δ limits); "상태공간 모델(SSM)과 Mamba 아키텍처" note (§2 recurrence and
convolution modes and their equivalence under LTI, §3 gate branch).
"""
import json
import math
import os
import random

import numpy as np
import pytest

from gen import make_inputs
from oracle import ss_ref

HERE = os.path.dirname(os.path.abspath(__file__))


def _c_fwd(*args, z=None, h0=None):
    from oracle import cref
    return cref.fwd(*args, z=z, h0=h0)


IMPLS = {"numpy": ss_ref.ss_fwd, "c": _c_fwd}


@pytest.fixture(params=sorted(IMPLS))
def fwd(request):
    return IMPLS[request.param]


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------------------------
# pin functions: each takes a forward implementation and returns a relative error
# ---------------------------------------------------------------------------------------------

def pin_golden(fwd):
    """Hand-unrolled cases (tests/golden/hand_unrolled.json)."""
    with open(os.path.join(HERE, "golden", "hand_unrolled.json")) as f:
        cases = json.load(f)["cases"]
    worst = 0.0
    ln2 = math.log(2.0)
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
        y, hf = fwd(x, dtr, dtb, A, Bm, Cm, Dk, h0=h0)
        y_exp = np.array([p + q * ln2 for p, q in c["y"]])
        h_exp = np.array([p + q * ln2 for p, q in c["h_final"]])
        worst = max(worst, rel_err(np.asarray(y).reshape(-1), y_exp),
                    rel_err(np.asarray(hf).reshape(-1), h_exp))
    return worst


def pin_lti_convolution(fwd, seed=11, L=64, D=3, N=5, Bn=2):
    """Constant Δ, B, C per channel: the scan is the causal convolution y = x * K + D x,
    K_k = Σ_n C_n Ā_n^k δ B_n, computed here with np.convolve and Ā^k by np.power."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bn, D, L)).astype(np.float32)
    dtb = np.log(np.expm1(rng.uniform(0.01, 0.5, D))).astype(np.float32)
    dtr = np.repeat(rng.standard_normal((Bn, D, 1)).astype(np.float32) * 0.3, L, axis=2)
    A = (-rng.uniform(0.2, 3.0, (D, N))).astype(np.float32)
    B0 = rng.standard_normal((Bn, N, 1)).astype(np.float32)
    C0 = rng.standard_normal((Bn, N, 1)).astype(np.float32)
    Bm = np.repeat(B0, L, axis=2)
    Cm = np.repeat(C0, L, axis=2)
    Dk = rng.standard_normal(D).astype(np.float32)
    y, _ = fwd(x, dtr, dtb, A, Bm, Cm, Dk)
    y = np.asarray(y).reshape(Bn, D, L)
    ref = np.empty((Bn, D, L))
    k = np.arange(L, dtype=np.float64)
    for b in range(Bn):
        for d in range(D):
            u = float(dtb[d]) + float(dtr[b, d, 0])
            delta = np.logaddexp(0.0, u)                      # library softplus
            abar = np.exp(delta * A[d].astype(np.float64))    # [N]
            K = np.zeros(L)
            for n in range(N):
                K += float(C0[b, n, 0]) * np.power(abar[n], k) * delta * float(B0[b, n, 0])
            ref[b, d] = np.convolve(x[b, d].astype(np.float64), K)[:L] + float(Dk[d]) * x[b, d].astype(np.float64)
    return rel_err(y, ref)


def pin_delta_to_zero(fwd, seed=12, L=32, D=4, N=6):
    """dt_bias = -60: δ ≈ e^-60, so Ā = 1 and B̄x ≈ 0 in fp64: h_t = h0 and
    y_t = C_t·h0 + D x_t (Δ→0 keeps the state, §4.1 of the selective-scan page)."""
    inp = make_inputs(1, L, D, N, seed=seed, with_h0=True)
    dtb = np.full(D, -60.0, np.float32)
    y, hf = fwd(inp.x, inp.dt_raw, dtb, inp.A, inp.Bm, inp.Cm, inp.Dskip, h0=inp.h0)
    h0 = inp.h0.astype(np.float64)
    ref = np.einsum("bnl,bdn->bdl", inp.Cm.astype(np.float64), h0) + \
        inp.Dskip.astype(np.float64)[None, :, None] * inp.x
    return max(rel_err(np.asarray(y).reshape(ref.shape), ref),
               rel_err(np.asarray(hf).reshape(h0.shape), h0))


def pin_delta_to_inf(fwd, seed=13, L=32, D=4, N=6):
    """dt_bias = +50 and A <= -1: Ā <= e^-48, so the state resets every step to
    h_t = δ_t B_t x_t (Δ→∞ focuses on the current input, §4.1)."""
    inp = make_inputs(1, L, D, N, seed=seed, with_h0=True)
    dtb = np.full(D, 50.0, np.float32)
    y, _ = fwd(inp.x, inp.dt_raw, dtb, inp.A, inp.Bm, inp.Cm, inp.Dskip, h0=inp.h0)
    u = 50.0 + inp.dt_raw.astype(np.float64)                  # softplus(u) = u + log1p(e^-u) ~ u
    delta = u + np.log1p(np.exp(-u))
    x = inp.x.astype(np.float64)
    CB = np.einsum("bnl,bnl->bl", inp.Cm.astype(np.float64), inp.Bm.astype(np.float64))
    ref = delta * x * CB[:, None, :] + inp.Dskip.astype(np.float64)[None, :, None] * x
    return rel_err(np.asarray(y).reshape(ref.shape), ref)


def pin_brute_force(fwd, seed=14, L=8, D=2, N=3, Bn=2):
    """Closed form with no recurrence: h_t = e^{A S_t} h0 + Σ_{s<=t} e^{A (S_t - S_s)} δ_s B_s x_s,
    S_t = Σ_{r<=t} δ_r (a product of exponentials is the exponential of the sum).
    Pure-Python loops over every term."""
    inp = make_inputs(Bn, L, D, N, seed=seed, gate=True, with_h0=True)
    y, hf = fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                z=inp.z, h0=inp.h0)
    y = np.asarray(y).reshape(Bn, D, L)
    ref = np.zeros((Bn, D, L))
    for b in range(Bn):
        for d in range(D):
            deltas = [math.log1p(math.exp(float(inp.dt_bias[d]) + float(inp.dt_raw[b, d, t])))
                      for t in range(L)]
            S = [sum(deltas[:t + 1]) for t in range(L)]
            for t in range(L):
                acc = 0.0
                for n in range(N):
                    a = float(inp.A[d, n])
                    h = math.exp(a * S[t]) * float(inp.h0[b, d, n])
                    for s in range(t + 1):
                        h += math.exp(a * (S[t] - S[s])) * deltas[s] * float(inp.Bm[b, n, s]) * \
                            float(inp.x[b, d, s])
                    acc += float(inp.Cm[b, n, t]) * h
                acc += float(inp.Dskip[d]) * float(inp.x[b, d, t])
                zt = float(inp.z[b, d, t])
                ref[b, d, t] = acc * zt / (1.0 + math.exp(-zt))
    return rel_err(y, ref)


def pin_resume(fwd, seed=15, L=48, L1=17, D=3, N=4):
    """fwd(x[0:L]) equals fwd(x[L1:L]) started from the final state of fwd(x[0:L1])."""
    inp = make_inputs(2, L, D, N, seed=seed, gate=True)
    a = (inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip)
    y, hf = fwd(*a, z=inp.z)
    s1 = lambda arr: np.ascontiguousarray(arr[..., :L1])
    s2 = lambda arr: np.ascontiguousarray(arr[..., L1:])
    y1, h1 = fwd(s1(inp.x), s1(inp.dt_raw), inp.dt_bias, inp.A, s1(inp.Bm), s1(inp.Cm),
                 inp.Dskip, z=s1(inp.z))
    y2, h2 = fwd(s2(inp.x), s2(inp.dt_raw), inp.dt_bias, inp.A, s2(inp.Bm), s2(inp.Cm),
                 inp.Dskip, z=s2(inp.z), h0=np.asarray(h1, np.float64).astype(np.float32))
    # h1 is fp64; the float32 hand-over rounds it, so compare at float32 resolution
    yy = np.concatenate([np.asarray(y1).reshape(2, D, L1), np.asarray(y2).reshape(2, D, L - L1)], -1)
    return max(rel_err(yy, np.asarray(y).reshape(2, D, L)),
               rel_err(np.asarray(h2).reshape(2, D, N), np.asarray(hf).reshape(2, D, N)))


def pin_linearity(fwd, seed=16, L=24, D=3, N=4):
    """With δ, B, C fixed and no gate the scan is linear in (x, h0) (a linear recurrence)."""
    i1 = make_inputs(1, L, D, N, seed=seed, with_h0=True)
    i2 = make_inputs(1, L, D, N, seed=seed + 100, with_h0=True)
    al, be = np.float32(0.75), np.float32(-1.5)
    common = (i1.dt_raw, i1.dt_bias, i1.A, i1.Bm, i1.Cm, i1.Dskip)
    y1, _ = fwd(i1.x, *common, h0=i1.h0)
    y2, _ = fwd(i2.x, *common, h0=i2.h0)
    y3, _ = fwd(al * i1.x + be * i2.x, *common, h0=al * i1.h0 + be * i2.h0)
    return rel_err(y3, float(al) * np.asarray(y1) + float(be) * np.asarray(y2))


def pin_associativity(seed=17, L=40, D=3, N=4):
    """Every bracketing of the affine-pair operator of §2.2 gives the sequential states."""
    inp = make_inputs(1, L, D, N, seed=seed, with_h0=True)
    x = inp.x.astype(np.float64)[0]
    delta = ss_ref.softplus(inp.dt_bias.astype(np.float64)[:, None] + inp.dt_raw[0])
    a = np.exp(delta[:, :, None] * inp.A.astype(np.float64)[:, None, :])      # [D,L,N]
    bx = delta[:, :, None] * inp.Bm[0].T.astype(np.float64)[None] * x[:, :, None]
    rng = random.Random(seed)

    def reduce(lo, hi):  # combined pair of steps lo..hi-1, random split points
        if hi - lo == 1:
            return a[:, lo], bx[:, lo]
        m = rng.randint(lo + 1, hi - 1)
        return ss_ref.combine(reduce(m, hi), reduce(lo, m))

    _, hf = ss_ref.ss_fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                          h0=inp.h0)
    worst = 0.0
    for _ in range(5):
        P, H = reduce(0, L)
        hf_tree = P * inp.h0[0].astype(np.float64) + H
        worst = max(worst, rel_err(hf_tree, hf[0]))
    return worst


PINS = {
    "golden": (pin_golden, 1e-12),
    "lti_convolution": (pin_lti_convolution, 1e-12),
    "delta_to_zero": (pin_delta_to_zero, 1e-14),
    "delta_to_inf": (pin_delta_to_inf, 1e-12),
    "brute_force": (pin_brute_force, 1e-12),
    "resume": (pin_resume, 1e-6),
    "linearity": (pin_linearity, 1e-6),
}


@pytest.mark.parametrize("pin", sorted(PINS))
def test_pin(fwd, pin):
    f, tol = PINS[pin]
    err = f(fwd)
    assert err <= tol, f"{pin}: {err:.3e} > {tol:.1e}"


def test_resume_exact_fp64_handover():
    """Resume with the exact fp64 state hand-over (numpy oracle accepts fp64 h0)."""
    inp = make_inputs(1, 30, 2, 3, seed=21)
    a = (inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip)
    y, hf = ss_ref.ss_fwd(*a)
    L1 = 11
    c = lambda arr, sl: np.ascontiguousarray(arr[..., sl])
    y1, h1 = ss_ref.ss_fwd(c(inp.x, slice(0, L1)), c(inp.dt_raw, slice(0, L1)), inp.dt_bias, inp.A,
                           c(inp.Bm, slice(0, L1)), c(inp.Cm, slice(0, L1)), inp.Dskip)
    y2, h2 = ss_ref.ss_fwd(c(inp.x, slice(L1, None)), c(inp.dt_raw, slice(L1, None)), inp.dt_bias,
                           inp.A, c(inp.Bm, slice(L1, None)), c(inp.Cm, slice(L1, None)),
                           inp.Dskip, h0=h1)
    assert rel_err(np.concatenate([y1, y2], -1), y) < 1e-14
    assert rel_err(h2, hf) < 1e-14


def test_associativity():
    assert pin_associativity() < 1e-13


def test_softplus_sigmoid_library():
    u = np.concatenate([np.linspace(-80, 80, 4001), [-1e-3, 0.0, 1e-3, 709.0, -745.0]])
    assert np.max(np.abs(ss_ref.softplus(u) - np.logaddexp(0.0, u)) /
                  np.maximum(np.logaddexp(0.0, u), 1e-300)) < 1e-14
    assert ss_ref.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-16)
    from scipy.special import expit
    zz = np.linspace(-700, 700, 7001)
    assert np.max(np.abs(ss_ref.sigmoid(zz) - expit(zz))) < 1e-15


def test_gate_is_silu(fwd):
    """The gate multiplies the ungated output by SiLU(z) (torch's silu as the library check)."""
    import torch
    inp = make_inputs(2, 20, 3, 4, seed=18, gate=True)
    a = inp.oracle_args()
    y0, _ = fwd(*a)
    y1, _ = fwd(*a, z=inp.z)
    silu = torch.nn.functional.silu(torch.from_numpy(inp.z.astype(np.float64))).numpy()
    assert rel_err(np.asarray(y1).reshape(silu.shape), np.asarray(y0).reshape(silu.shape) * silu) < 1e-13


def test_skip_only(fwd):
    """B = 0 and h0 = 0: the state stays zero and y = D x."""
    inp = make_inputs(1, 16, 5, 4, seed=19)
    Bz = np.zeros_like(inp.Bm)
    y, hf = fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, Bz, inp.Cm, inp.Dskip)
    assert np.all(np.asarray(hf) == 0.0)
    assert rel_err(np.asarray(y).reshape(inp.x.shape), inp.Dskip[None, :, None] * inp.x.astype(np.float64)) < 1e-15


def test_contractive_bound():
    """A < 0 gives Ā in (0,1], so |h_t| <= |h0| + Σ_s |δ_s B_s x_s| for every t."""
    inp = make_inputs(1, 64, 4, 6, seed=20, with_h0=True)
    x = inp.x.astype(np.float64)
    delta = ss_ref.softplus(inp.dt_bias[None, :, None].astype(np.float64) + inp.dt_raw)
    beta = np.abs(delta[:, :, None, :] * inp.Bm[:, None, :, :] * x[:, :, None, :])  # [B,D,N,L]
    bound = np.abs(inp.h0)[..., None] + np.cumsum(beta, axis=-1)
    for L in (1, 7, 64):
        sl = lambda arr: np.ascontiguousarray(arr[..., :L])
        _, hf = ss_ref.ss_fwd(sl(inp.x), sl(inp.dt_raw), inp.dt_bias, inp.A, sl(inp.Bm), sl(inp.Cm),
                              inp.Dskip, h0=inp.h0)
        assert np.all(np.abs(hf) <= bound[..., L - 1] * (1 + 1e-12))


def test_numpy_equals_c():
    """The two oracle implementations agree on a gated, h0, bf16-valued case."""
    from oracle import cref
    inp = make_inputs(2, 300, 7, 16, seed=22, gate=True, with_h0=True, dtype="bf16", a_perturb=True)
    a = inp.oracle_args()
    y_n, h_n = ss_ref.ss_fwd(*a, z=inp.z, h0=inp.h0)
    y_c, h_c = cref.fwd(*a, z=inp.z, h0=inp.h0)
    assert rel_err(y_c, y_n) < 1e-12 and rel_err(h_c, h_n) < 1e-12
    chans = np.array([13, 0, 6])
    y_s, h_s = cref.fwd(*a, z=inp.z, h0=inp.h0, chans=chans)
    assert np.array_equal(y_s, y_c.reshape(-1, 300)[chans])
    assert np.array_equal(h_s, h_c.reshape(-1, 16)[chans])


# ---------------------------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must fail at least one pin
# ---------------------------------------------------------------------------------------------

def _mutant(kind):
    sp, sg = ss_ref.softplus, ss_ref.sigmoid

    def fwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z=None, h0=None):
        f = lambda a: None if a is None else np.asarray(a, np.float64)
        x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0 = map(f, (x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0))
        Bn, D, L = x.shape
        N = A.shape[1]
        u = dt_bias[None, :, None] + dt_raw
        delta = np.exp(u) if kind == "exp_not_softplus" else sp(u)
        h = np.zeros((Bn, D, N)) if h0 is None else h0.copy()
        y = np.empty((Bn, D, L))
        for t in range(L):
            dl = delta[:, :, t, None]
            Asg = -A if kind == "sign_of_A" else A
            abar = np.exp(dl * Asg[None])
            tb = t - 1 if (kind == "B_index_off_by_one" and t > 0) else t
            bx = (1.0 if kind == "no_delta_in_Bbar" else dl) * Bm[:, None, :, tb] * x[:, :, t, None]
            if kind == "readout_before_update":
                s = (Cm[:, None, :, t] * h).sum(-1)
                h = abar * h + bx
            else:
                h = abar * h + bx
                s = (Cm[:, None, :, t] * h).sum(-1)
            if kind != "drop_D":
                s = s + Dskip[None, :] * x[:, :, t]
            if z is not None:
                zt = z[:, :, t]
                s = s * (sg(zt) if kind == "gate_sigmoid_only" else zt * sg(zt))
            y[:, :, t] = s
        return y, h
    return fwd


MUTANTS = ["exp_not_softplus", "sign_of_A", "B_index_off_by_one", "no_delta_in_Bbar",
           "readout_before_update", "drop_D", "gate_sigmoid_only"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind):
    f = _mutant(kind)
    failed = []
    for name, (pin, tol) in PINS.items():
        with np.errstate(all="ignore"):
            err = pin(f)
        if not (err <= tol):
            failed.append(name)
    assert failed, f"no pin caught mutant {kind}"
