"""GPU parity of the boundary variants against the fp64 oracle: token-major sequence tensors
(SS_ORDER_BLD: x, dt_raw, z, y and their gradients [B, L, D]; B, C, dB, dC [B, L, N]) and a
Δraw shared by the channels (SS_DT_SHARED: one value per token, [B, L]).

Page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별", §3.1 writes the
input as (B, L, D); §1.2 makes Δ a one-output projection of the token broadcast over the
channels.  The oracle runs on the channel-major arrays (the shared Δraw as its broadcast
view); the GPU gets the same values in the variant's memory order, and its outputs are
brought back to channel-major before the comparison.  The gradient of a shared Δraw is the
sum over channels of the oracle's per-channel gradients (pinned on the CPU by finite
differences).  Tolerances as the default layout: 1e-4 / 2e-3 · max|ref| for outputs,
5e-4 · max|ref| for gradients.
"""
import numpy as np
import pytest

from gen import make_inputs
from oracle import cref
from tests.gpu_util import TOL_GRAD, assert_close, note, tol_for

pytestmark = pytest.mark.gpu


def _tok(a):
    """[B, X, L] -> token-major [B, L, X] (contiguous)."""
    return np.ascontiguousarray(np.swapaxes(a, 1, 2))


def _dev_inputs(inp, order, shared):
    import torch
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    lay = _tok if order == 1 else np.ascontiguousarray
    t_in = lambda a: None if a is None else torch.from_numpy(lay(a)).to(dt).cuda()
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    d = dict(x=t_in(inp.x), z=t_in(inp.z), Bm=t_in(inp.Bm), Cm=t_in(inp.Cm),
             dt_bias=f32(inp.dt_bias), A=f32(inp.A), Dskip=f32(inp.Dskip), h0=f32(inp.h0),
             dh_final=f32(inp.dh_final))
    if shared:
        d["dt_raw"] = torch.from_numpy(np.ascontiguousarray(inp.dt_tok)).to(dt).cuda()
    else:
        d["dt_raw"] = t_in(inp.dt_raw)
    d["dy"] = None if inp.dy is None else torch.from_numpy(lay(inp.dy).astype(np.float32)).cuda()
    return d


def _back(a, order):
    """GPU output in the variant's order -> channel-major numpy."""
    a = a.cpu().numpy()
    return _tok(a) if order == 1 else a


FWD_CASES = [
    # B, L, D, N, dtype, gate, h0, plan, chunk
    (2, 256, 64, 16, "f32", True, True, 0, 0),
    (1, 200, 70, 16, "bf16", True, True, 1, 0),      # L % 8 != 0, D not a block multiple
    (2, 1000, 33, 8, "f32", False, True, 2, 64),
    (1, 2056, 48, 32, "bf16", True, True, 2, 264),
    (3, 64, 17, 1, "f32", True, False, 1, 0),
    (1, 7, 3, 4, "bf16", True, True, 0, 0),
    (1, 64, 24576, 16, "bf16", True, True, 0, 0),    # mixed four/eight-lane launch
]


@pytest.mark.parametrize("layout", [0, 2, 3], ids=["auto", "lane", "oct"])
@pytest.mark.parametrize("variant", [(1, False), (1, True), (0, True)],
                         ids=["tok", "tok-shared", "shared"])
@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "B{}L{}D{}N{}-{}-g{}-h{}-p{}-c{}".format(*c))
def test_fwd_variants(gpu, case, variant, layout):
    import torch
    Bn, L, D, N, dt, gate, h0, plan, chunk = case
    order, shared = variant
    inp = make_inputs(Bn, L, D, N, dtype=dt, seed=700 + L, gate=gate, with_h0=h0, a_perturb=True,
                      dt_shared=shared)
    note(f"fwd variant order={order} shared={shared} {case} layout={layout}")
    t = _dev_inputs(inp, order, shared)
    # checkpoints need user chunks that are multiples of 16 (SS_ERR_UNSUPPORTED otherwise)
    want_ck = not (plan == 2 and chunk % 16)
    out = gpu.ss_fwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"],
                     z=t["z"] if gate else None, h0=t["h0"] if h0 else None,
                     return_final=True, return_ckpt=want_ck, plan=plan, chunk=chunk,
                     layout=layout, order=order)
    y, hf, ck = out if want_ck else (*out, None)
    torch.cuda.synchronize()
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z if gate else None, h0=inp.h0 if h0 else None)
    assert_close(_back(y, order), yr, tol_for(inp), "y")
    assert_close(hf.cpu().numpy(), hr, tol_for(inp), "h_final")
    if ck is None:
        return
    # checkpoints: state entering step 16 i equals the oracle's state after 16 i steps
    ckn = ck.cpu().numpy()
    for i in range(1, ckn.shape[2]):
        cut = lambda a: np.ascontiguousarray(a[..., :16 * i])
        _, hi = cref.fwd(cut(inp.x), cut(inp.dt_raw), inp.dt_bias, inp.A, cut(inp.Bm),
                         cut(inp.Cm), inp.Dskip, z=cut(inp.z) if gate else None,
                         h0=inp.h0 if h0 else None)
        assert_close(ckn[:, :, i], hi, tol_for(inp), f"checkpoint {i}")
        if i >= 3:
            break


BWD_CASES = [
    # B, L, D, N, dtype, gate, h0, dh_final
    (1, 64, 64, 16, "f32", True, True, True),
    (2, 200, 70, 16, "bf16", True, True, True),
    (1, 333, 40, 8, "bf16", True, False, True),
    (2, 96, 24, 2, "f32", False, True, False),
    (1, 300, 1024, 16, "bf16", True, True, True),
]
GRADS = ("dx", "ddt_raw", "dz", "ddt_bias", "dA", "dB", "dC", "dD", "dh0")


@pytest.mark.parametrize("ckpt", [False, True], ids=["recompute", "ckpt"])
@pytest.mark.parametrize("variant", [(1, False), (1, True), (0, True)],
                         ids=["tok", "tok-shared", "shared"])
@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}L{}D{}N{}-{}-g{}-h{}-f{}".format(*c))
def test_bwd_variants(gpu, case, variant, ckpt):
    import torch
    Bn, L, D, N, dt, gate, h0, dhf = case
    order, shared = variant
    inp = make_inputs(Bn, L, D, N, dtype=dt, seed=800 + L + N, gate=gate, with_h0=h0,
                      with_dy=True, with_dh_final=dhf, a_perturb=True, dt_shared=shared)
    note(f"bwd variant order={order} shared={shared} {case} ckpt={ckpt}")
    t = _dev_inputs(inp, order, shared)
    z = t["z"] if gate else None
    h0t = t["h0"] if h0 else None
    hck = None
    if ckpt:
        _, hck = gpu.ss_fwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"],
                            z=z, h0=h0t, return_ckpt=True, order=order)
    g = gpu.ss_bwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dy"],
                   z=z, h0=h0t, dh_final=t["dh_final"] if dhf else None, h_ckpt=hck, order=order)
    torch.cuda.synchronize()
    ref = cref.bwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip, inp.dy,
                   z=inp.z if gate else None, h0=inp.h0 if h0 else None,
                   dh_final=inp.dh_final if dhf else None)
    if shared:
        ref["ddt_raw"] = ref["ddt_raw"].sum(axis=1)
    for k in GRADS:
        if ref[k] is None:
            assert g[k] is None, k
            continue
        if k in ("dx", "dz", "dB", "dC") or (k == "ddt_raw" and not shared):
            got = _back(g[k], order)
        else:
            got = g[k].cpu().numpy()
        assert_close(got, ref[k], TOL_GRAD, k)


@pytest.mark.parametrize("case", [(4, 96, 16, "bf16", True), (3, 70, 16, "f32", False),
                                  (2, 33, 32, "bf16", True), (3, 9, 2, "f32", True)],
                         ids=lambda c: "B{}D{}N{}-{}-g{}".format(*c))
def test_step_shared_dt(gpu, case):
    """Decode steps with one Δraw per (row, token): T steps equal the forward over T tokens."""
    import torch
    Bn, D, N, dt, gate = case
    T = 12
    inp = make_inputs(Bn, T, D, N, dtype=dt, seed=900 + D + N, gate=gate, with_h0=True,
                      a_perturb=True, dt_shared=True)
    note(f"step shared dt {case}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    col = lambda a, s: torch.from_numpy(np.ascontiguousarray(a[..., s])).to(tdt).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    h = f32(inp.h0)
    ys = []
    for s in range(T):
        ys.append(gpu.ss_step(col(inp.x, s), col(inp.dt_tok, s), f32(inp.dt_bias), f32(inp.A),
                              col(inp.Bm, s), col(inp.Cm, s), f32(inp.Dskip), h,
                              z=col(inp.z, s) if gate else None).cpu().numpy())
    yr, hr = cref.fwd(inp.x, inp.dt_raw, inp.dt_bias, inp.A, inp.Bm, inp.Cm, inp.Dskip,
                      z=inp.z if gate else None, h0=inp.h0)
    assert_close(np.stack(ys, axis=-1), yr, tol_for(inp), "y over T steps")
    assert_close(h.cpu().numpy(), hr, tol_for(inp), "state after T steps")
