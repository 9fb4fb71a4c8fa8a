"""Plain fp64 CPU oracle of the selection projections and the gated block around the scan.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the bench's CPU baseline may
import this module; the library's product path never does.

Sources (cited by page title and section):
  [SEL]  "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별": §1.2 the
         selection equations (B_t and C_t are N-output linear maps of the token, Δ_t is the
         softplus of a parameter plus a one-output linear map of it).
  [SSM]  "상태공간 모델(SSM)과 Mamba 아키텍처" (study note): §3, the block projects its input
         two ways; one branch goes through the selective SSM, the other through the SiLU
         gate, and the two are multiplied.

Readings (where the pages leave a point open):
  R15  Weights are stored as (outputs, inputs), so a projection is p = v · Wᵀ.  The input
       projection W_in [2D, D_in] maps the block input u [B, L, D_in] to the scan input
       x = first D outputs and the gate input z = last D outputs.
  R16  The selection projection W_x [1 + 2N, D] acts on x: output 0 is Δraw (one value per
       token, shared by the channels, to which each channel adds its dt_bias: the
       "Parameter"), outputs 1..N are B_t, outputs N+1..2N are C_t.
  R17  Nothing else is in the block (the pages name no convolution and no output
       projection); y [B, L, D] is the gated scan output.
What it computes (each projection one library matrix product in float64, then the scan
oracle of oracle/ss_ref.py or oracle/cref.py on the channel-major views):
  [x | z]      = u · W_inᵀ
  [Δraw|B|C]   = x · W_xᵀ
  y            = S6(x, Δraw broadcast over channels, dt_bias, A, B, C, Dskip, gate z, h0)
"""
import numpy as np

from . import ss_ref


def in_projection(u, W_in):
    """u [B, L, D_in], W_in [2D, D_in] -> x, z [B, L, D] (float64)."""
    u = np.asarray(u, np.float64)
    W = np.asarray(W_in, np.float64)
    D = W.shape[0] // 2
    xz = u @ W.T
    return xz[..., :D], xz[..., D:]


def selection_projections(x, W_x):
    """x [B, L, D], W_x [1 + 2N, D] -> Δraw [B, L], B [B, L, N], C [B, L, N] (float64)."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W_x, np.float64)
    N = (W.shape[0] - 1) // 2
    p = x @ W.T
    return p[..., 0], p[..., 1:1 + N], p[..., 1 + N:]


def block_fwd(u, W_in, W_x, dt_bias, A, Dskip, h0=None, impl="numpy", chans=None):
    """The block's forward.  Returns dict x, z, dt, B, C (token-major, float64), y [B, L, D]
    and h_final [B, D, N]; with impl="c" the scan runs in the C oracle (chans: sampled
    channels b*D + d, then y is [len(chans), L] and h_final [len(chans), N])."""
    x, z = in_projection(u, W_in)
    dt, Bm, Cm = selection_projections(x, W_x)
    Bn, L, D = x.shape
    cm = lambda a: np.ascontiguousarray(np.swapaxes(a, 1, 2))   # [B, L, X] -> [B, X, L]
    dt_raw = np.broadcast_to(dt[:, None, :], (Bn, D, L))
    args = (cm(x), dt_raw, dt_bias, A, cm(Bm), cm(Cm), Dskip)
    if impl == "c":
        from . import cref
        y, hf = cref.fwd(*args, z=cm(z), h0=h0, chans=chans)
    else:
        assert chans is None
        y, hf = ss_ref.ss_fwd(*args, z=cm(z), h0=h0)
    if chans is None:
        y = np.swapaxes(y, 1, 2)
    return dict(x=x, z=z, dt=dt, B=Bm, C=Cm, y=y, h_final=hf)
