"""Seeded input generator: reproducibility, per-tensor streams, bf16 rounding, recipe."""
import numpy as np
import pytest
import torch

from gen import WORKLOADS, bf16_bits, bits_to_f32, make_inputs, round_bf16


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  3.3895314e38, 1e-40], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(a), ref)


def test_bf16_ties_to_even_by_hand():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert bf16_bits(np.array([1.0 + 2 ** -8], np.float32))[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even (1 + 2^-6)
    assert bf16_bits(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 0x3F82
    assert bits_to_f32(np.array([0x3F80], np.uint16))[0] == 1.0


def test_seeded_and_independent_streams():
    a = make_inputs(2, 64, 8, 16, seed=4, gate=True)
    b = make_inputs(2, 64, 8, 16, seed=4, gate=False, with_h0=True)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.Bm, b.Bm) and np.array_equal(a.dt_raw, b.dt_raw)
    c = make_inputs(2, 64, 8, 16, seed=5, gate=True)
    assert not np.array_equal(a.x, c.x)


def test_recipe():
    inp = make_inputs(1, 4096, 512, 16, seed=2, a_perturb=False, dtype="bf16", gate=True)
    for t in (inp.x, inp.dt_raw, inp.z, inp.Bm, inp.Cm):
        assert t.dtype == np.float32
        assert np.array_equal(round_bf16(t), t)        # bf16-exact values
    assert np.array_equal(inp.A, -np.arange(1, 17, dtype=np.float32)[None].repeat(512, 0))
    dt = np.log1p(np.exp(inp.dt_bias.astype(np.float64)))
    assert dt.min() >= 1e-3 * (1 - 1e-6) and dt.max() <= 1e-1 * (1 + 1e-6)
    assert abs(np.std(inp.dt_raw) - 0.5) < 0.01 and abs(np.std(inp.x) - 1.0) < 0.01
    p = make_inputs(1, 8, 512, 16, seed=2, a_perturb=True)
    ratio = np.log(p.A / -np.arange(1, 17)[None])
    assert abs(np.std(ratio) - 0.1) < 0.01


def test_workloads_table():
    names = [w.name for w in WORKLOADS]
    assert names == ["c0", "c1", "c2", "c3", "c4", "d1", "p2"]
    c2 = WORKLOADS[2]
    assert (c2.batch, c2.seqlen, c2.dim, c2.dstate, c2.dtype, c2.gate) == (8, 2048, 5120, 16, "bf16", True)
    assert WORKLOADS[3].seqlen == 1048576 and WORKLOADS[4].backward
    d1 = WORKLOADS[5]
    assert d1.decode and d1.seqlen == 1 and (d1.batch, d1.dim, d1.dstate) == (256, 5120, 16)


@pytest.mark.parametrize("order", [0, 1])
def test_device_inputs_channel_rows(order):
    """gen.device (run here on the CPU device): a channel's host case holds exactly that
    channel's rows of the drawn tensors, and the per-channel parameters equal make_inputs'."""
    import torch
    from gen.device import make_device_inputs
    B, L, D, N = 2, 40, 5, 4
    c = make_device_inputs(B, L, D, N, dtype="bf16", seed=3, gate=True, order=order,
                           with_dy=True, with_h0=True, device="cpu")
    seq = (B, D, L) if order == 0 else (B, L, D)
    assert tuple(c.x.shape) == seq and c.x.dtype == torch.bfloat16
    assert tuple(c.Bm.shape) == ((B, N, L) if order == 0 else (B, L, N))
    ref = make_inputs(1, 1, D, N, seed=3, a_perturb=True)
    assert np.array_equal(c.dt_bias, ref.dt_bias) and np.array_equal(c.A, ref.A)
    assert np.array_equal(c.Dskip, ref.Dskip)
    h = c.channel(1, 3)
    xs = c.x.float().numpy()
    want = xs[1, 3, :] if order == 0 else xs[1, :, 3]
    assert np.array_equal(h.x[0, 0], want)
    bs = c.Bm.float().numpy()
    assert np.array_equal(h.Bm[0], bs[1] if order == 0 else bs[1].T)
    assert np.array_equal(h.h0[0, 0], c.h0[1, 3].numpy())
    assert h.A.shape == (1, N) and h.dt_bias.shape == (1,)
    # values are bf16-exact and the draws are seeded
    assert np.array_equal(round_bf16(h.x), h.x)
    c2 = make_device_inputs(B, L, D, N, dtype="bf16", seed=3, gate=True, order=order,
                            device="cpu")
    assert torch.equal(c2.x, c.x) and torch.equal(c2.Cm, c.Cm)
