"""Plain fp64 CPU oracle of the selective scan (S6): forward and backward.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the bench's CPU
baseline may import this module; the library's product path never does.

Sources (cited by page title and section):
  [SEL]  "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별"
         (booiljung.github.io): §1.1 LTI equations, §1.2 selection equations,
         §2.1 ZOH discretisation equations, §2.2 associative operator,
         §3.3 recomputation, §4.1 Δ as a gate.
  [SSM]  "상태공간 모델(SSM)과 Mamba 아키텍처" (study note): §2 recurrence and
         convolution modes, §3 S6 flowchart with the SiLU gate branch.
  [REV]  Review of "Mamba: Linear-Time Sequence Modeling with Selective State
         Spaces" (honbul.tistory.com): §2 definition of S6.

Where the pages leave a point open, the plainest reading the rest supports is taken
(marked R#):
  R1  B̄ = δ·B, the first-order form; the exact zero-order-hold (δA)⁻¹(e^{δA} − 1)·δB that
      [SEL §2.1] prints reduces to it as δA -> 0, and [SEL §4.1] reasons with it.
  R5  the readout adds D·x to Σ_n C h (D = 0 gives the pages' form).
  R6  the SiLU branch multiplies the readout: y = (C·h + D·x)·silu(z).
  R7  the state before the first step is h0 (or 0); h_final is the state after the last.
  With zoh=True the exact zero-order-hold form that [SEL §2.1] prints replaces R1:
      B̄x = (exp(δA) - 1) / A · B x    (δ B x where A = 0, its limit)
  the exact solution over one step of dh/dt = A h + B x with x held constant.

What it computes, per batch row b and channel d:
  u_t     = dt_bias[d] + dt_raw[b,d,t]                    [SEL §1.2], [REV §2]
  δ_t     = softplus(u_t) = log(1 + e^{u_t})              [SEL §1.2]
  Ā_{t,n} = exp(δ_t A[d,n])                               [SEL §2.1]; A diagonal, so elementwise
  B̄x      = δ_t B[b,n,t] x_t                              R1: first-order form of [SEL §2.1], as in [SEL §4.1]
  h_t     = Ā_t ⊙ h_{t-1} + B̄x,  h_{-1} = h0 or 0        [SEL §2.2], [SSM §2]; R7
  s_t     = Σ_n C[b,n,t] h_{t,n} + D[d] x_t               [SEL §1.1] readout; R5 adds D·x
  y_t     = s_t · z_t σ(z_t)  (gate on), else s_t         [SSM §3] SiLU gate branch; R6
  h_final = h_{L-1}

Evaluated sequentially in float64 on exactly the float32 (or bf16-exact) values
the GPU receives.  No blocking, fusion or reordering: one time step after the
other, vectorised only over independent (b, d) channels.

The backward is the exact adjoint of that recurrence (reverse sweep over t with
every h stored), the plain form the pages' recomputation scheme [SEL §3.3] has to
reproduce.
"""
import numpy as np


def softplus(u):
    """log(1 + e^u) in fp64, written as max(u,0) + log1p(e^{-|u|}) so neither branch overflows."""
    u = np.asarray(u, dtype=np.float64)
    return np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))


def sigmoid(z):
    """1/(1+e^{-z}) in fp64 without overflow for either sign of z."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def bbar_factor(dl, A, zoh):
    """The factor of B x in B̄x: δ (first order, R1) or (exp(δA) - 1)/A (exact zero-order
    hold, [SEL §2.1]), evaluated with expm1 so small δA loses nothing."""
    if not zoh:
        return dl * np.ones_like(A)
    num = np.expm1(dl * A)
    safe = np.where(A == 0.0, 1.0, A)
    return np.where(A == 0.0, dl * np.ones_like(A), num / safe)


def bbar_factor_grads(dl, A, zoh):
    """Partial derivatives (∂f/∂δ, ∂f/∂A) of the factor f of bbar_factor.

    First order, f = δ: (1, 0).  Exact hold, f = (e^{δA} - 1)/A:
      ∂f/∂δ = e^{δA} = Ā
      ∂f/∂A = (δĀ - f)/A = δ² Σ_{k>=0} (k+1)(δA)^k/(k+2)!   (term-by-term derivative of
              f = δ Σ_k (δA)^k/(k+1)!), the closed form where |δA| >= 1e-2 and the series,
              ten terms, below that, where the closed form would cancel.
    """
    ones = np.ones_like(dl * A)
    if not zoh:
        return ones, np.zeros_like(ones)
    u = dl * A
    abar = np.exp(u)
    small = np.abs(u) < 1e-2
    series = np.zeros_like(u)
    fact = 2.0                                                   # (k+2)!
    for k in range(10):
        series = series + (k + 1) * u ** k / fact
        fact *= k + 3
    safe = np.where(small, 1.0, A * ones)
    closed = (dl * abar - np.expm1(u) / safe) / safe
    return abar, np.where(small, dl * dl * series, closed)


def ss_fwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z=None, h0=None, zoh=False):
    """Forward scan.  Returns (y [B,D,L], h_final [B,D,N]) in float64.

    Shapes: x, dt_raw, z [B,D,L]; Bm, Cm [B,N,L]; A [D,N]; dt_bias, Dskip [D]; h0 [B,D,N].
    zoh: exact zero-order-hold B̄ instead of the first-order δ·B.
    """
    x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0 = map(
        _f64, (x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0))
    Bn, D, L = x.shape
    N = A.shape[1]
    delta = softplus(dt_bias[None, :, None] + dt_raw)            # [B,D,L]
    h = np.zeros((Bn, D, N)) if h0 is None else h0.copy()
    y = np.empty((Bn, D, L))
    for t in range(L):
        dl = delta[:, :, t, None]                                  # [B,D,1]
        abar = np.exp(dl * A[None, :, :])                          # [B,D,N]
        bx = bbar_factor(dl, A[None, :, :], zoh) * Bm[:, None, :, t] * x[:, :, t, None]
        h = abar * h + bx
        s = (Cm[:, None, :, t] * h).sum(axis=-1) + Dskip[None, :] * x[:, :, t]
        if z is not None:
            zt = z[:, :, t]
            s = s * zt * sigmoid(zt)
        y[:, :, t] = s
    return y, h


def ss_bwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, dy, z=None, h0=None, dh_final=None, zoh=False):
    """Gradients of sum(dy*y) + sum(dh_final*h_final) with respect to every input.

    Returns a dict of float64 arrays: dx, ddt_raw, dz (None without gate) [B,D,L];
    ddt_bias [D]; dA [D,N]; dB, dC [B,N,L]; dD [D]; dh0 [B,D,N] (None without h0).

    Adjoint of the recurrence, swept from t = L-1 down to 0 with g = ∂/∂h_t:
      ds_t  = dy_t z_t σ(z_t)                      (dy_t without gate)
      dz_t  = dy_t s_t σ(z_t) (1 + z_t (1 - σ(z_t)))
      g    += ds_t C_t                             (g was Ā_{t+1} ⊙ g_{t+1}, or dh_final)
      dC_t += ds_t h_t ;  dD += ds_t x_t ;  dB_t += g δ_t x_t
      dx_t  = ds_t D + Σ_n g δ_t B_t
      dδ_t  = Σ_n g (A Ā_t h_{t-1} + B_t x_t) ;  dA += g δ_t Ā_t h_{t-1}
      ddt_raw_t = dδ_t σ(u_t) ;  ddt_bias += ddt_raw_t
      g     = Ā_t ⊙ g                              (after t = 0 this is dh0)
    With zoh=True the input term is f B x with f = (Ā - 1)/A (bbar_factor) in place of δ B x:
      dB_t += g f x ;  dx_t = ds_t D + Σ_n g f B_t
      dδ_t  = Σ_n g (A Ā_t h_{t-1} + Ā_t B_t x_t)   (∂f/∂δ = Ā)
      dA   += g (δ_t Ā_t h_{t-1} + ∂f/∂A B_t x_t)
    """
    x, dt_raw, dt_bias, A, Bm, Cm, Dskip, dy, z, h0, dh_final = map(
        _f64, (x, dt_raw, dt_bias, A, Bm, Cm, Dskip, dy, z, h0, dh_final))
    Bn, D, L = x.shape
    N = A.shape[1]
    u = dt_bias[None, :, None] + dt_raw
    delta = softplus(u)
    sig_u = sigmoid(u)
    # forward, storing every state: hs[t+1] = h_t, hs[0] = h_{-1}
    hs = np.empty((L + 1, Bn, D, N))
    hs[0] = 0.0 if h0 is None else h0
    abar_all = np.empty((L, Bn, D, N))
    s_all = np.empty((Bn, D, L))
    for t in range(L):
        dl = delta[:, :, t, None]
        abar = np.exp(dl * A[None])
        abar_all[t] = abar
        fb = bbar_factor(dl, A[None], zoh)
        hs[t + 1] = abar * hs[t] + fb * Bm[:, None, :, t] * x[:, :, t, None]
        s_all[:, :, t] = (Cm[:, None, :, t] * hs[t + 1]).sum(-1) + Dskip[None, :] * x[:, :, t]

    dx = np.empty((Bn, D, L))
    ddt_raw = np.empty((Bn, D, L))
    dz = np.empty((Bn, D, L)) if z is not None else None
    dA = np.zeros((D, N))
    dB = np.zeros((Bn, N, L))
    dC = np.zeros((Bn, N, L))
    dD = np.zeros(D)
    g = np.zeros((Bn, D, N)) if dh_final is None else dh_final.copy()
    for t in range(L - 1, -1, -1):
        if z is not None:
            zt = z[:, :, t]
            sz = sigmoid(zt)
            ds = dy[:, :, t] * zt * sz
            dz[:, :, t] = dy[:, :, t] * s_all[:, :, t] * sz * (1.0 + zt * (1.0 - sz))
        else:
            ds = dy[:, :, t]
        xt = x[:, :, t]
        dl = delta[:, :, t]
        g = g + ds[:, :, None] * Cm[:, None, :, t]
        dC[:, :, t] += np.einsum("bd,bdn->bn", ds, hs[t + 1])
        dD += (ds * xt).sum(axis=0)
        fb = bbar_factor(dl[:, :, None], A[None], zoh)             # [B,D,N]
        dfd, dfa = bbar_factor_grads(dl[:, :, None], A[None], zoh)
        bx = Bm[:, None, :, t] * xt[:, :, None]                    # B_t x_t  [B,D,N]
        dB[:, :, t] += np.einsum("bdn,bdn->bn", g, fb * xt[:, :, None])
        dx[:, :, t] = ds * Dskip[None, :] + (g * fb * Bm[:, None, :, t]).sum(-1)
        abar = abar_all[t]
        hprev = hs[t]
        ddelta = (g * (A[None] * abar * hprev + dfd * bx)).sum(-1)
        dA += (g * (dl[:, :, None] * abar * hprev + dfa * bx)).sum(axis=0)
        ddt_raw[:, :, t] = ddelta * sig_u[:, :, t]
        g = abar * g
    ddt_bias = ddt_raw.sum(axis=(0, 2))
    return dict(dx=dx, ddt_raw=ddt_raw, dz=dz, ddt_bias=ddt_bias, dA=dA, dB=dB, dC=dC, dD=dD,
                dh0=(g if h0 is not None else None))


def combine(later, earlier):
    """The associative operator on affine pairs, [SEL §2.2]:
    (a_j, b_j) • (a_i, b_i) = (a_j a_i, a_j b_i + b_j), with (a_i, b_i) the earlier step."""
    aj, bj = later
    ai, bi = earlier
    return aj * ai, aj * bi + bj
