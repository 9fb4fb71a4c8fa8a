"""Python binding of the MI355X selective-scan (S6) library (include/ss.h).

Argument marshalling only: torch supplies device memory and the current stream,
every step of the scan runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback: if the compiled library is missing, ``load()`` raises.

    y = ss_fwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z=None, h0=None)
    y, h_final = ss_fwd(..., return_final=True)
    y, h_final, h_ckpt = ss_fwd(..., return_final=True, return_ckpt=True)
    grads = ss_bwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, dy, z=None, h0=None, dh_final=None,
                   h_ckpt=None)
    y_t = ss_step(x_t, dt_raw_t, dt_bias, A, B_t, C_t, Dskip, h, z_t=None)   # h updated in place

Layouts: x, dt_raw, z, y [B, D, L]; Bm, Cm [B, N, L]; A [D, N]; dt_bias, Dskip [D];
h0, h_final [B, D, N]; h_ckpt [B, D, ceil(L/16), N] (state entering every 16th step).  x, dt_raw, z, Bm, Cm are float32 or bfloat16 (all the same);
everything else is float32.
"""
import ctypes
import os

from ._build import LIB, build, stale, tree_id  # noqa: F401

SS_F32, SS_BF16 = 0, 1
SS_PLAN_AUTO, SS_PLAN_SINGLE, SS_PLAN_CHUNKED = 0, 1, 2
SS_LAYOUT_AUTO, SS_LAYOUT_QUAD, SS_LAYOUT_LANE, SS_LAYOUT_OCT = 0, 1, 2, 3
SS_DISC_EULER, SS_DISC_ZOH = 0, 1
SS_ORDER_BDL, SS_ORDER_BLD = 0, 1
SS_DT_FULL, SS_DT_SHARED = 0, 1

ERRORS = {0: "SS_OK", -1: "SS_ERR_NULL", -2: "SS_ERR_DIMS", -3: "SS_ERR_DTYPE", -4: "SS_ERR_ALIGN",
          -5: "SS_ERR_WORKSPACE", -6: "SS_ERR_HIP", -7: "SS_ERR_UNSUPPORTED", -8: "SS_ERR_SCRATCH"}

EXPORTS = ("ss_fwd", "ss_bwd", "ss_step", "ss_fwd_workspace_size", "ss_bwd_workspace_size",
           "ss_block_fwd", "ss_block_fwd_workspace_size", "ss_in_proj", "ss_strerror",
           "ss_last_hip_error", "ss_version", "ss_build_id", "ss_fwd_noalloc")


class ss_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("plan", ctypes.c_int32),
                ("chunk", ctypes.c_int64), ("layout", ctypes.c_int32), ("disc", ctypes.c_int32),
                ("order", ctypes.c_int32), ("dt_layout", ctypes.c_int32)]


class ss_block_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("d_in", ctypes.c_int64),
                ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("plan", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class SSError(RuntimeError):
    def __init__(self, code, lib=None):
        msg = ERRORS.get(code, str(code))
        if lib is not None:
            msg += ": " + lib.ss_strerror(code).decode()
            if code == -6:
                msg += f" (hipError {lib.ss_last_hip_error()})"
        super().__init__(msg)
        self.code = code


_lib = None


def load(path: str = LIB, expect: str = None):
    """Load libss.so (built in-tree by ``build()``).  Raises if it is missing, or if its build
    identity (ss_build_id) differs from ``expect`` (default: the digest of the sources in this
    tree, ``tree_id()``): a library built from other sources is never used."""
    global _lib
    if _lib is not None and expect is None and path == LIB:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} (run selective_state_space_34_amd.build())")
    lib = ctypes.CDLL(path)
    lib.ss_build_id.restype = ctypes.c_char_p
    got = lib.ss_build_id().decode()
    want = tree_id() if expect is None else expect
    if got != want:
        raise RuntimeError(f"{path} was built from other sources (library id {got[:16]}..., "
                           f"expected {want[:16]}...): rebuild it with build()")
    P = ctypes.c_void_p
    D = ctypes.POINTER(ss_dims)
    lib.ss_fwd.argtypes = [D] + [P] * 12 + [P, ctypes.c_size_t, P]
    lib.ss_fwd.restype = ctypes.c_int
    lib.ss_bwd.argtypes = [D] + [P] * 9 + [P, P, P] + [P] * 9 + [P, ctypes.c_size_t, P]
    lib.ss_bwd.restype = ctypes.c_int
    lib.ss_fwd_noalloc.argtypes = [D] + [P] * 12 + [P]
    lib.ss_fwd_noalloc.restype = ctypes.c_int
    lib.ss_step.argtypes = [D] + [P] * 12
    lib.ss_step.restype = ctypes.c_int
    for f in ("ss_fwd_workspace_size", "ss_bwd_workspace_size"):
        getattr(lib, f).argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
        getattr(lib, f).restype = ctypes.c_int
    BD = ctypes.POINTER(ss_block_dims)
    lib.ss_block_fwd.argtypes = [BD] + [P] * 14 + [P, ctypes.c_size_t, P]
    lib.ss_block_fwd.restype = ctypes.c_int
    lib.ss_block_fwd_workspace_size.argtypes = [BD, ctypes.POINTER(ctypes.c_size_t)]
    lib.ss_block_fwd_workspace_size.restype = ctypes.c_int
    lib.ss_in_proj.argtypes = [BD] + [P] * 5
    lib.ss_in_proj.restype = ctypes.c_int
    lib.ss_strerror.argtypes = [ctypes.c_int]
    lib.ss_strerror.restype = ctypes.c_char_p
    lib.ss_last_hip_error.restype = ctypes.c_int
    lib.ss_version.restype = ctypes.c_int
    if expect is None and path == LIB:
        _lib = lib
    return lib


def make_dims(batch, seqlen, dim, dstate, in_dtype=SS_F32, plan=SS_PLAN_AUTO, chunk=0,
              layout=SS_LAYOUT_AUTO, disc=SS_DISC_EULER, order=SS_ORDER_BDL, dt_layout=SS_DT_FULL):
    return ss_dims(batch, seqlen, dim, dstate, in_dtype, plan, chunk, layout, disc, order,
                   dt_layout)


def workspace_size(dims, backward=False) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    fn = lib.ss_bwd_workspace_size if backward else lib.ss_fwd_workspace_size
    rc = fn(ctypes.byref(dims), ctypes.byref(n))
    if rc != 0:
        raise SSError(rc, lib)
    return n.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _seq_shape(x, order):
    """(B, D, L) of a sequence tensor in the given order."""
    if x.dim() != 3:
        raise ValueError(f"x must be 3-D, got shape {tuple(x.shape)}")
    if order == SS_ORDER_BDL:
        return tuple(x.shape)
    if order == SS_ORDER_BLD:
        Bn, L, D = x.shape
        return Bn, D, L
    raise ValueError(f"order must be SS_ORDER_BDL or SS_ORDER_BLD, got {order}")


def _dims_of(x, A, dt_raw, plan, chunk, layout=SS_LAYOUT_AUTO, disc=SS_DISC_EULER,
             order=SS_ORDER_BDL):
    import torch
    Bn, D, L = _seq_shape(x, order)
    N = A.shape[1]
    if x.dtype == torch.float32:
        dt = SS_F32
    elif x.dtype == torch.bfloat16:
        dt = SS_BF16
    else:
        raise ValueError(f"x dtype must be float32 or bfloat16, got {x.dtype}")
    dtl = SS_DT_SHARED if dt_raw.dim() == 2 else SS_DT_FULL
    return make_dims(Bn, L, D, N, dt, plan, chunk, layout, disc, order, dtl)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _seq(Bn, D, L, order):
    return (Bn, D, L) if order == SS_ORDER_BDL else (Bn, L, D)


def _check_inputs(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0, order=SS_ORDER_BDL):
    """Shapes: x, z [B, D, L] ([B, L, D] token-major); dt_raw as x, or [B, L] (one value
    per token); Bm, Cm [B, N, L] ([B, L, N]); A [D, N]; dt_bias, Dskip [D]; h0 [B, D, N]."""
    import torch
    Bn, D, L = _seq_shape(x, order)
    N = A.shape[1]
    dev = x.device
    f32 = torch.float32
    _check(dt_raw, "dt_raw", (Bn, L) if dt_raw.dim() == 2 else _seq(Bn, D, L, order), x.dtype, dev)
    _check(z, "z", _seq(Bn, D, L, order), x.dtype, dev)
    _check(Bm, "Bm", _seq(Bn, N, L, order), x.dtype, dev)
    _check(Cm, "Cm", _seq(Bn, N, L, order), x.dtype, dev)
    _check(A, "A", (D, N), f32, dev)
    _check(dt_bias, "dt_bias", (D,), f32, dev)
    _check(Dskip, "Dskip", (D,), f32, dev)
    _check(h0, "h0", (Bn, D, N), f32, dev)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")


CKPT_STEPS = 16


def ss_fwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z=None, h0=None, *, return_final=False,
           return_ckpt=False, y=None, h_final=None, h_ckpt=None, workspace=None,
           plan=SS_PLAN_AUTO, chunk=0, layout=SS_LAYOUT_AUTO, disc=SS_DISC_EULER,
           order=SS_ORDER_BDL, stream=None):
    """Forward scan through the C ABI.  Returns y, (y, h_final) with return_final, and
    the checkpoints last with return_ckpt (or when h_ckpt is passed).  disc: SS_DISC_EULER
    (input term δ·B·x) or SS_DISC_ZOH (exact zero-order hold).  order: SS_ORDER_BDL or
    SS_ORDER_BLD (token-major x, z, y, Bm, Cm); a 2-D dt_raw [B, L] is one value per token."""
    import torch
    lib = load()
    _check_inputs(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0, order)
    dims = _dims_of(x, A, dt_raw, plan, chunk, layout, disc, order)
    Bn, D, L = _seq_shape(x, order)
    N = A.shape[1]
    if y is None:
        y = torch.empty(_seq(Bn, D, L, order), dtype=torch.float32, device=x.device)
    _check(y, "y", _seq(Bn, D, L, order), torch.float32, x.device)
    if return_final and h_final is None:
        h_final = torch.empty((Bn, D, N), dtype=torch.float32, device=x.device)
    _check(h_final, "h_final", (Bn, D, N), torch.float32, x.device)
    nck = (L + CKPT_STEPS - 1) // CKPT_STEPS
    if return_ckpt and h_ckpt is None:
        h_ckpt = torch.empty((Bn, D, nck, N), dtype=torch.float32, device=x.device)
    _check(h_ckpt, "h_ckpt", (Bn, D, nck, N), torch.float32, x.device)
    need = workspace_size(dims)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.ss_fwd(ctypes.byref(dims), _ptr(x), _ptr(dt_raw), _ptr(dt_bias), _ptr(A), _ptr(Bm),
                    _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_final), _ptr(h_ckpt),
                    _ptr(workspace), wbytes, _stream(stream))
    if rc != 0:
        raise SSError(rc, lib)
    out = (y,)
    if return_final or h_final is not None:
        out += (h_final,)
    if h_ckpt is not None:
        out += (h_ckpt,)
    return out if len(out) > 1 else y


def ss_fwd_noalloc(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, y, z=None, h0=None, *, h_final=None,
                   h_ckpt=None, plan=SS_PLAN_AUTO, chunk=0, layout=SS_LAYOUT_AUTO,
                   disc=SS_DISC_EULER, order=SS_ORDER_BDL, stream=None):
    """ss_fwd without a workspace: the library's static scratch (SS_NOALLOC_SCRATCH_MIB MiB per
    GPU) serves the chunked and one-lane plans, and nothing is allocated, here or in the
    library.  The caller passes every output (y, and h_final / h_ckpt if wanted).  Calls that
    overlap on one GPU share that scratch and race; calls ordered on one stream do not."""
    import torch
    lib = load()
    _check_inputs(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0, order)
    dims = _dims_of(x, A, dt_raw, plan, chunk, layout, disc, order)
    Bn, D, L = _seq_shape(x, order)
    N = A.shape[1]
    if y is None:
        raise ValueError("y is required")
    _check(y, "y", _seq(Bn, D, L, order), torch.float32, x.device)
    _check(h_final, "h_final", (Bn, D, N), torch.float32, x.device)
    nck = (L + CKPT_STEPS - 1) // CKPT_STEPS
    _check(h_ckpt, "h_ckpt", (Bn, D, nck, N), torch.float32, x.device)
    rc = lib.ss_fwd_noalloc(ctypes.byref(dims), _ptr(x), _ptr(dt_raw), _ptr(dt_bias), _ptr(A),
                            _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(h0), _ptr(y),
                            _ptr(h_final), _ptr(h_ckpt), _stream(stream))
    if rc != 0:
        raise SSError(rc, lib)
    return y


def ss_bwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, dy, z=None, h0=None, dh_final=None, *,
           h_ckpt=None, workspace=None, chunk=0, order=SS_ORDER_BDL, disc=SS_DISC_EULER,
           out=None, stream=None):
    """Backward through the C ABI.  Returns a dict dx, ddt_raw, ddt_bias, dA, dB, dC, dD,
    dz (None without gate), dh0 (None without h0); all float32, each shaped like its input
    (order as in ss_fwd).  h_ckpt: the checkpoints of an ss_fwd call on the same inputs
    (optional; made with the same disc).  disc: the discretisation the forward used."""
    import torch
    lib = load()
    _check_inputs(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0, order)
    dims = _dims_of(x, A, dt_raw, SS_PLAN_CHUNKED, chunk, disc=disc, order=order)
    Bn, D, L = _seq_shape(x, order)
    N = A.shape[1]
    dev = x.device
    f32 = torch.float32
    sq = _seq(Bn, D, L, order)
    _check(dy, "dy", sq, f32, dev)
    _check(dh_final, "dh_final", (Bn, D, N), f32, dev)
    _check(h_ckpt, "h_ckpt", (Bn, D, (L + CKPT_STEPS - 1) // CKPT_STEPS, N), f32, dev)
    shapes = dict(dx=sq, ddt_raw=tuple(dt_raw.shape), ddt_bias=(D,), dA=(D, N),
                  dB=_seq(Bn, N, L, order), dC=_seq(Bn, N, L, order), dD=(D,), dz=sq,
                  dh0=(Bn, D, N))
    g = {} if out is None else dict(out)
    for k, shp in shapes.items():
        if (k == "dz" and z is None) or (k == "dh0" and h0 is None):
            g[k] = None
            continue
        if g.get(k) is None:
            g[k] = torch.empty(shp, dtype=f32, device=dev)
        _check(g[k], k, shp, f32, dev)
    need = workspace_size(dims, backward=True)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.ss_bwd(ctypes.byref(dims), _ptr(x), _ptr(dt_raw), _ptr(dt_bias), _ptr(A), _ptr(Bm),
                    _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_final), _ptr(h_ckpt),
                    _ptr(g["dx"]), _ptr(g["ddt_raw"]), _ptr(g["ddt_bias"]), _ptr(g["dA"]),
                    _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]),
                    _ptr(workspace), wbytes, _stream(stream))
    if rc != 0:
        raise SSError(rc, lib)
    return g


def ss_step(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, h, z=None, *, h_out=None, y=None,
            disc=SS_DISC_EULER, stream=None):
    """One decode step through the C ABI: x, z [B, D]; dt_raw [B, D] or [B] (one value per
    token); Bm, Cm [B, N]; h [B, D, N]
    float32, the state before the token.  The state after it goes to h_out (default: h
    itself, updated in place).  Returns y [B, D] float32."""
    import torch
    lib = load()
    if x.dim() != 2:
        raise ValueError(f"x must be [B, D], got shape {tuple(x.shape)}")
    Bn, D = x.shape
    N = A.shape[1]
    dev = x.device
    f32 = torch.float32
    if x.dtype == torch.float32:
        dt = SS_F32
    elif x.dtype == torch.bfloat16:
        dt = SS_BF16
    else:
        raise ValueError(f"x dtype must be float32 or bfloat16, got {x.dtype}")
    _check(x, "x", (Bn, D), x.dtype, dev)
    _check(dt_raw, "dt_raw", (Bn,) if dt_raw.dim() == 1 else (Bn, D), x.dtype, dev)
    _check(z, "z", (Bn, D), x.dtype, dev)
    _check(Bm, "Bm", (Bn, N), x.dtype, dev)
    _check(Cm, "Cm", (Bn, N), x.dtype, dev)
    _check(A, "A", (D, N), f32, dev)
    _check(dt_bias, "dt_bias", (D,), f32, dev)
    _check(Dskip, "Dskip", (D,), f32, dev)
    _check(h, "h", (Bn, D, N), f32, dev)
    if h_out is None:
        h_out = h
    _check(h_out, "h_out", (Bn, D, N), f32, dev)
    if y is None:
        y = torch.empty((Bn, D), dtype=f32, device=dev)
    _check(y, "y", (Bn, D), f32, dev)
    dims = make_dims(Bn, 1, D, N, dt, disc=disc,
                     dt_layout=SS_DT_SHARED if dt_raw.dim() == 1 else SS_DT_FULL)
    rc = lib.ss_step(ctypes.byref(dims), _ptr(x), _ptr(dt_raw), _ptr(dt_bias), _ptr(A), _ptr(Bm),
                     _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(h), _ptr(h_out), _ptr(y), _stream(stream))
    if rc != 0:
        raise SSError(rc, lib)
    return y


def make_block_dims(batch, seqlen, d_in, dim, dstate, plan=SS_PLAN_AUTO, layout=SS_LAYOUT_AUTO):
    return ss_block_dims(batch, seqlen, d_in, dim, dstate, plan, layout)


def block_workspace_size(dims) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    rc = lib.ss_block_fwd_workspace_size(ctypes.byref(dims), ctypes.byref(n))
    if rc != 0:
        raise SSError(rc, lib)
    return n.value


def ss_block_fwd(u, W_in, W_x, dt_bias, A, Dskip, h0=None, *, return_final=False,
                 return_proj=False, y=None, workspace=None, plan=SS_PLAN_AUTO,
                 layout=SS_LAYOUT_AUTO, stream=None):
    """Projections and gated scan through the C ABI: u [B, L, d_in] bf16, W_in [2D, d_in]
    bf16, W_x [1 + 2N, D] float32, dt_bias, Dskip [D], A [D, N], h0 [B, D, N] float32.
    Returns y [B, L, D] float32; with return_final also h_final [B, D, N]; with return_proj
    also a dict of the projections x, z [B, L, D], dt [B, L], B, C [B, L, N] (float32)."""
    import torch
    lib = load()
    if u.dim() != 3:
        raise ValueError(f"u must be [B, L, d_in], got shape {tuple(u.shape)}")
    Bn, L, Din = u.shape
    D, N = A.shape
    dev = u.device
    f32, bf = torch.float32, torch.bfloat16
    _check(u, "u", (Bn, L, Din), bf, dev)
    _check(W_in, "W_in", (2 * D, Din), bf, dev)
    _check(W_x, "W_x", (1 + 2 * N, D), f32, dev)
    _check(dt_bias, "dt_bias", (D,), f32, dev)
    _check(A, "A", (D, N), f32, dev)
    _check(Dskip, "Dskip", (D,), f32, dev)
    _check(h0, "h0", (Bn, D, N), f32, dev)
    dims = make_block_dims(Bn, L, Din, D, N, plan, layout)
    if y is None:
        y = torch.empty((Bn, L, D), dtype=f32, device=dev)
    _check(y, "y", (Bn, L, D), f32, dev)
    hf = torch.empty((Bn, D, N), dtype=f32, device=dev) if return_final else None
    proj = None
    if return_proj:
        proj = dict(x=torch.empty((Bn, L, D), dtype=f32, device=dev),
                    z=torch.empty((Bn, L, D), dtype=f32, device=dev),
                    dt=torch.empty((Bn, L), dtype=f32, device=dev),
                    B=torch.empty((Bn, L, N), dtype=f32, device=dev),
                    C=torch.empty((Bn, L, N), dtype=f32, device=dev))
    need = block_workspace_size(dims)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    g = (lambda k: None) if proj is None else (lambda k: _ptr(proj[k]))
    rc = lib.ss_block_fwd(ctypes.byref(dims), _ptr(u), _ptr(W_in), _ptr(W_x), _ptr(dt_bias),
                          _ptr(A), _ptr(Dskip), _ptr(h0), _ptr(y), _ptr(hf), g("x"), g("z"),
                          g("dt"), g("B"), g("C"), _ptr(workspace), wbytes, _stream(stream))
    if rc != 0:
        raise SSError(rc, lib)
    out = (y,)
    if return_final:
        out += (hf,)
    if return_proj:
        out += (proj,)
    return out if len(out) > 1 else y


def ss_in_proj(u, W_in, *, x=None, z=None, stream=None):
    """[x | z] = u · W_inᵀ through the C ABI: u [B, L, d_in] bf16, W_in [2D, d_in] bf16;
    returns x, z [B, L, D] float32."""
    import torch
    lib = load()
    Bn, L, Din = u.shape
    D = W_in.shape[0] // 2
    dev = u.device
    _check(u, "u", (Bn, L, Din), torch.bfloat16, dev)
    _check(W_in, "W_in", (2 * D, Din), torch.bfloat16, dev)
    if x is None:
        x = torch.empty((Bn, L, D), dtype=torch.float32, device=dev)
    if z is None:
        z = torch.empty((Bn, L, D), dtype=torch.float32, device=dev)
    _check(x, "x", (Bn, L, D), torch.float32, dev)
    _check(z, "z", (Bn, L, D), torch.float32, dev)
    dims = make_block_dims(Bn, L, Din, D, 1)
    rc = lib.ss_in_proj(ctypes.byref(dims), _ptr(u), _ptr(W_in), _ptr(x), _ptr(z), _stream(stream))
    if rc != 0:
        raise SSError(rc, lib)
    return x, z
