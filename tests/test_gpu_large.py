"""GPU parity at the largest sizes: tensors past 2^31 elements (buffers past 4 GB), where any
32-bit element offset would wrap.

The inputs are drawn on the GPU by gen.device (seeded, the benchmark recipe) and never
cross the bus whole; for sampled channels, always including the first and the last (whose
elements sit past the 2^31 mark), the exact values the kernels read are copied back and the
fp64 oracle runs on that channel alone over its whole sequence.  Outputs of a channel depend
only on that channel (and its batch row's B, C), so each comparison is exact in kind:
y and h_final (forward, decode step); dx, dΔraw, dz (backward); dA, dD and ddt_bias of a
channel, the oracle summed over its batch rows.  dB and dC are sums over every channel of a
row (here 1100 sequences of a million steps each, minutes of oracle time), so at this size
they are not compared; the same reduction kernels are checked element by element on the
B=4 L=4096 D=2048 workload.  Tolerances as everywhere: 2e-3·max|ref| (bf16 inputs) per
output row, 5e-4·max|ref| per gradient row.
"""
import numpy as np
import pytest

from oracle import cref
from tests.gpu_util import TOL_BF16, TOL_GRAD, assert_close, note

pytestmark = pytest.mark.gpu


def _samples(B, D, seed, k=4):
    rng = np.random.default_rng(seed)
    fixed = [(0, 0), (B - 1, D - 1), (B - 1, 0), (0, D - 1)]
    extra = [(int(rng.integers(B)), int(rng.integers(D))) for _ in range(k)]
    return list(dict.fromkeys(fixed + extra))


def _free():
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _oracle_fwd(h):
    return cref.fwd(h.x, h.dt_raw, h.dt_bias, h.A, h.Bm, h.Cm, h.Dskip, z=h.z, h0=h.h0)


@pytest.mark.parametrize("order", [0, 1], ids=["channel-major", "token-major"])
def test_fwd_past_2e31_elements(gpu, order):
    """Channel-major: the chunked group kernel (rows 64-bit, steps within a row 32-bit).
    Token-major with L·D >= 2^31: the group kernel's 32-bit offsets do not apply, the plan
    takes the one-lane kernel."""
    import torch
    from gen.device import make_device_inputs
    B, L, D, N = (2, 1_048_600, 1100, 16) if order == 0 else (1, 2_000_000, 1100, 16)
    assert B * L * D > 2 ** 31 and (order == 0 or L * D >= 2 ** 31)
    note(f"large fwd order={order} B={B} L={L} D={D} N={N}")
    c = make_device_inputs(B, L, D, N, dtype="bf16", seed=51 + order, gate=True, order=order)
    hosts = {s: c.channel(*s) for s in _samples(B, D, 7 + order)}
    y, hf = gpu.ss_fwd(c.x, c.dt_raw, c.dt_bias_t, c.A_t, c.Bm, c.Cm, c.Dskip_t, z=c.z,
                       return_final=True, order=order)
    torch.cuda.synchronize()
    for (b, d), h in hosts.items():
        yr, hr = _oracle_fwd(h)
        got = (y[b, d] if order == 0 else y[b, :, d]).cpu().numpy()
        assert_close(got, yr[0, 0], TOL_BF16, f"y[{b},{d}]")
        assert_close(hf[b, d].cpu().numpy(), hr[0, 0], TOL_BF16, f"h_final[{b},{d}]")
    del y, hf, c
    _free()


def test_bwd_past_2e31_elements(gpu):
    """The training launch (forward checkpoints, then the backward) on 2.3e9 elements."""
    import torch
    from gen.device import make_device_inputs
    B, L, D, N = 2, 1_048_576, 1100, 16
    note(f"large bwd B={B} L={L} D={D} N={N}")
    c = make_device_inputs(B, L, D, N, dtype="bf16", seed=53, gate=True, with_dy=True)
    ds = [0, D - 1, 517]
    hosts = {(b, d): c.channel(b, d) for d in ds for b in range(B)}
    y, ck = gpu.ss_fwd(c.x, c.dt_raw, c.dt_bias_t, c.A_t, c.Bm, c.Cm, c.Dskip_t, z=c.z,
                       return_ckpt=True)
    del y
    g = gpu.ss_bwd(c.x, c.dt_raw, c.dt_bias_t, c.A_t, c.Bm, c.Cm, c.Dskip_t, c.dy, z=c.z,
                   h_ckpt=ck)
    torch.cuda.synchronize()
    for d in ds:
        acc = {"dA": 0.0, "dD": 0.0, "ddt_bias": 0.0}
        for b in range(B):
            h = hosts[(b, d)]
            r = cref.bwd(h.x, h.dt_raw, h.dt_bias, h.A, h.Bm, h.Cm, h.Dskip, h.dy, z=h.z)
            for k in ("dx", "ddt_raw", "dz"):
                assert_close(g[k][b, d].cpu().numpy(), r[k][0, 0], TOL_GRAD, f"{k}[{b},{d}]")
            for k in acc:
                acc[k] = acc[k] + r[k]
        assert_close(g["dA"][d].cpu().numpy(), acc["dA"][0], TOL_GRAD, f"dA[{d}]")
        assert_close(g["dD"][d:d + 1].cpu().numpy(), acc["dD"], TOL_GRAD, f"dD[{d}]")
        assert_close(g["ddt_bias"][d:d + 1].cpu().numpy(), acc["ddt_bias"], TOL_GRAD,
                     f"ddt_bias[{d}]")
    del g, ck, c
    _free()


def test_step_state_past_2e31_elements(gpu):
    """A decode step whose state [B, D, N] holds 2.16e9 floats (8.6 GB), updated in place."""
    import torch
    from gen.device import make_device_inputs
    B, D, N = 4096, 33_000, 16
    assert B * D * N > 2 ** 31
    note(f"large step B={B} D={D} N={N}")
    c = make_device_inputs(B, 1, D, N, dtype="bf16", seed=55, gate=True, with_h0=True)
    hosts = {s: c.channel(*s) for s in _samples(B, D, 9)}
    col = lambda t: t[..., 0]
    h = c.h0
    y = gpu.ss_step(col(c.x), col(c.dt_raw), c.dt_bias_t, c.A_t, col(c.Bm), col(c.Cm), c.Dskip_t,
                    h, z=col(c.z))
    torch.cuda.synchronize()
    for (b, d), hh in hosts.items():
        yr, hr = _oracle_fwd(hh)
        assert_close(y[b, d:d + 1].cpu().numpy(), yr[0, 0], TOL_BF16, f"y[{b},{d}]")
        assert_close(h[b, d].cpu().numpy(), hr[0, 0], TOL_BF16, f"state[{b},{d}]")
    del y, h, c
    _free()
