"""Helpers of the GPU parity tests: move seeded inputs to the device, run the HIP
path through the C ABI, compare with the oracle at the stated tolerance."""
import sys

import numpy as np

# max|gpu - ref| <= TOL * max|ref| (per tensor)
TOL_F32 = 1e-4
TOL_BF16 = 2e-3
TOL_GRAD = 5e-4


def tol_for(inp):
    return TOL_BF16 if inp.dtype == "bf16" else TOL_F32


def note(msg):
    """Name the case on stdout before a GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(inp):
    """Device tensors of a seeded case (bf16 values are exact, so the cast is exact)."""
    import torch
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32

    def t_in(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()

    def t32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return dict(x=t_in(inp.x), dt_raw=t_in(inp.dt_raw), z=t_in(inp.z), Bm=t_in(inp.Bm),
                Cm=t_in(inp.Cm), dt_bias=t32(inp.dt_bias), A=t32(inp.A), Dskip=t32(inp.Dskip),
                h0=t32(inp.h0), dy=t32(inp.dy), dh_final=t32(inp.dh_final))


def gpu_fwd(ss, inp, *, gate=True, h0=True, final=True, plan=0, chunk=0, layout=0, disc=0):
    import torch
    t = dev(inp)
    out = ss.ss_fwd(t["x"], t["dt_raw"], t["dt_bias"], t["A"], t["Bm"], t["Cm"], t["Dskip"],
                    z=t["z"] if gate else None, h0=t["h0"] if h0 else None,
                    return_final=final, plan=plan, chunk=chunk, layout=layout, disc=disc)
    torch.cuda.synchronize()
    if final:
        return out[0].cpu().numpy(), out[1].cpu().numpy()
    return out.cpu().numpy(), None


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def assert_close(got, ref, tol, what):
    e = rel_err(got, ref)
    assert e <= tol, f"{what}: max|err|/max|ref| = {e:.3e} > {tol:.1e}"
    return e
