"""GPU parity of the block forward (ss_block_fwd through the C ABI) against the fp64 block
oracle (oracle/block_ref.py).

Note "상태공간 모델(SSM)과 Mamba 아키텍처", §3 and page "3.2 선택적 스캔(Selective Scan)
알고리즘과 정보의 압축 및 선별", §1.2: [x | z] = u·W_inᵀ (bf16 operands, float32
accumulation on the matrix cores), [Δraw | B | C] = x·W_xᵀ (float32), then the gated scan.
Each bf16 product is exact in float32, so the projections differ from the fp64 oracle by
float32 accumulation only; every output is held to the float32 tolerance of the scan,
max|gpu - ref| <= 1e-4·max|ref| per tensor.  Small shapes compare every element (ragged in
every GEMM dimension); the block workload at full size compares sampled tokens of the
projections and sampled channels of y, the oracle computing everything itself in float64.
"""
import numpy as np
import pytest

from gen import make_block_inputs, workload, workload_inputs
from oracle import block_ref
from tests.gpu_util import assert_close, note

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _dev(inp):
    import torch
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return dict(u=bf(inp.u), W_in=bf(inp.W_in), W_x=f32(inp.W_x), dt_bias=f32(inp.dt_bias),
                A=f32(inp.A), Dskip=f32(inp.Dskip), h0=f32(inp.h0))


CASES = [
    # B, L, d_in, D, N, h0, layout
    (2, 64, 64, 128, 16, True, 0),
    (1, 100, 40, 36, 8, True, 0),      # M, 2D, d_in off every tile size; D % 16 != 0
    (3, 33, 16, 20, 4, False, 0),
    (1, 1, 8, 4, 1, True, 0),
    (1, 50, 24, 64, 32, True, 0),
    (2, 300, 72, 96, 16, True, 2),     # one lane per channel
    (1, 520, 256, 512, 16, True, 3),   # eight lanes per channel
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}L{}Din{}D{}N{}-h{}-lay{}".format(*c))
def test_block_small(gpu, case):
    import torch
    Bn, L, Din, D, N, h0, layout = case
    inp = make_block_inputs(Bn, L, Din, D, N, dtype="bf16", seed=1000 + L + D, with_h0=h0)
    note(f"block {case}")
    t = _dev(inp)
    y, hf, proj = gpu.ss_block_fwd(t["u"], t["W_in"], t["W_x"], t["dt_bias"], t["A"], t["Dskip"],
                                   h0=t["h0"], return_final=True, return_proj=True, layout=layout)
    torch.cuda.synchronize()
    ref = block_ref.block_fwd(inp.u, inp.W_in, inp.W_x, inp.dt_bias, inp.A, inp.Dskip, h0=inp.h0)
    for k in ("x", "z", "dt", "B", "C"):
        assert_close(proj[k].cpu().numpy(), ref[k], TOL, k)
    assert_close(y.cpu().numpy(), ref["y"], TOL, "y")
    assert_close(hf.cpu().numpy(), ref["h_final"], TOL, "h_final")


def test_block_full_size_sampled(gpu):
    """The block workload (u [8, 2048, 2560], W_in [10240, 2560], D = 5120, N = 16) in the
    launch the bench times: sampled tokens of every projection, sampled channels of y."""
    import torch
    w = workload("p2")
    inp = workload_inputs(w)
    note("block p2 full size")
    t = _dev(inp)
    y, proj = gpu.ss_block_fwd(t["u"], t["W_in"], t["W_x"], t["dt_bias"], t["A"], t["Dskip"],
                               return_proj=True)
    torch.cuda.synchronize()
    M = w.batch * w.seqlen
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 128, replace=False)]))
    u2 = inp.u.reshape(M, -1)[toks][:, None, :]             # sampled tokens as [T, 1, d_in]
    x_r, z_r = block_ref.in_projection(u2, inp.W_in)
    dt_r, B_r, C_r = block_ref.selection_projections(x_r, inp.W_x)
    got = {k: proj[k].cpu().numpy() for k in proj}
    assert_close(got["x"].reshape(M, -1)[toks], x_r[:, 0], TOL, "x (sampled tokens)")
    assert_close(got["z"].reshape(M, -1)[toks], z_r[:, 0], TOL, "z (sampled tokens)")
    assert_close(got["dt"].reshape(M)[toks], dt_r[:, 0], TOL, "dt (sampled tokens)")
    assert_close(got["B"].reshape(M, -1)[toks], B_r[:, 0], TOL, "B (sampled tokens)")
    assert_close(got["C"].reshape(M, -1)[toks], C_r[:, 0], TOL, "C (sampled tokens)")
    # y on sampled channels: the oracle's own projections of every token, then its scan
    C = w.batch * w.dim
    chans = np.unique(np.concatenate([[0, C - 1], rng.choice(C, 48, replace=False)]))
    ref = block_ref.block_fwd(inp.u, inp.W_in, inp.W_x, inp.dt_bias, inp.A, inp.Dskip,
                              impl="c", chans=chans)
    ycm = np.swapaxes(y.cpu().numpy(), 1, 2).reshape(C, w.seqlen)
    assert_close(ycm[chans], ref["y"], TOL, "y (sampled channels)")


# the last shape spans many tiles and is ragged in M, 2D and d_in
@pytest.mark.parametrize("shape", [(1, 100, 40, 36), (2, 256, 128, 128), (1, 517, 264, 200),
                                   (1, 4100, 264, 4100)],
                         ids=lambda s: "B{}L{}Din{}D{}".format(*s))
def test_in_proj(gpu, shape):
    """The block's first stage alone (ss_in_proj): every element of x and z."""
    import torch
    Bn, L, Din, D = shape
    inp = make_block_inputs(Bn, L, Din, D, 1, dtype="bf16", seed=1100 + L)
    note(f"in_proj {shape}")
    t = _dev(inp)
    x, z = gpu.ss_in_proj(t["u"], t["W_in"])
    torch.cuda.synchronize()
    x_r, z_r = block_ref.in_projection(inp.u, inp.W_in)
    assert_close(x.cpu().numpy(), x_r, TOL, "x")
    assert_close(z.cpu().numpy(), z_r, TOL, "z")
