"""Thin ctypes binding of libngv.so (the C ABI in include/ngv.h).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are PyTorch device tensors (fp32 volumes, fp64 scalars), used for
their memory and the current stream. Each function has the name of the C
entry point it calls and the same argument order, with sizes taken from the
tensors; a negative status raises NgvError.

The library must exist (built by ``non_gemm_voxel_amd.build``): there is no
fallback of any kind.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libngv.so")

NGV_OK, NGV_EINVAL, NGV_EWORKSPACE, NGV_EHIP, NGV_EUNSUPPORTED = 0, -1, -2, -3, -4


class NgvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"ngv error {code}: {msg}")
        self.code = code


class ngv_dims(ctypes.Structure):
    _fields_ = [("nx", ctypes.c_int64), ("ny", ctypes.c_int64), ("nz", ctypes.c_int64)]


class ngv_xform(ctypes.Structure):
    _fields_ = [("A", ctypes.c_float * 9), ("t", ctypes.c_float * 3), ("S", ctypes.c_float * 9),
                ("xmin", ctypes.c_float * 3), ("xmax", ctypes.c_float * 3)]


class ngv_slab(ctypes.Structure):
    _fields_ = [("z0", ctypes.c_int64), ("nz", ctypes.c_int64), ("zrange", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NgvError(NGV_EHIP, f"{LIB_PATH} is not built (run non_gemm_voxel_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    dp = ctypes.POINTER(ngv_dims)
    xp = ctypes.POINTER(ngv_xform)
    sp = ctypes.POINTER(ngv_slab)
    i, f, sz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.ngv_workspace_bytes.argtypes = [i, i]
    L.ngv_workspace_bytes.restype = sz
    L.ngv_status_str.argtypes = [i]
    L.ngv_status_str.restype = ctypes.c_char_p
    L.ngv_warp_fwd.argtypes = [_P, dp, sp, _P, dp, xp, _P, i, _P]
    L.ngv_warp_fwd_slab.argtypes = [_P, dp, sp, _P, dp, xp, _P, _P]
    L.ngv_warp_bwd.argtypes = [_P, dp, sp, _P, dp, xp, _P, _P, _P, _P, i, _P, sz, _P]
    L.ngv_mi_loss_fwd_bwd.argtypes = [_P, _P, dp, i, f, f, f, f, f, _P, _P, i, _P, sz, _P]
    L.ngv_lncc_loss_fwd_bwd.argtypes = [_P, _P, dp, i, f, f, _P, _P, i, _P, sz, _P]
    L.ngv_adam_step.argtypes = [_P, _P, _P, _P, dp, i, _P, f, f, f, f, f, _P, sz, _P]
    L.ngv_warp_bwd_adam.argtypes = [_P, dp, sp, _P, dp, xp, _P, _P, _P, _P, i, _P, f, f, f, f, _P, _P, i, _P, sz,
                                    _P]
    L.ngv_warp_zrange.argtypes = [_P, dp, dp, xp, _P, _P, sz, _P]
    L.ngv_warp_fwd_mi.argtypes = [_P, dp, sp, _P, dp, xp, _P, i, _P, i, f, f, f, f, f, _P, i, _P, sz, _P]
    L.ngv_mi_grad.argtypes = [_P, _P, dp, i, f, f, f, f, f, _P, i, _P, sz, _P]
    L.ngv_mse_loss_fwd_bwd.argtypes = [_P, _P, dp, f, _P, _P, i, _P, sz, _P]
    L.ngv_mi_loss_fwd_bwd_order.argtypes = [_P, _P, dp, i, i, f, f, f, f, f, _P, _P, i, _P, sz, _P]
    L.ngv_mi_loss_fwd_bwd_noalloc.argtypes = [_P, _P, dp, i, f, f, f, f, f, _P, _P, i, _P]
    L.ngv_warp_lncc_mi_bwd.argtypes = [_P, dp, _P, dp, xp, _P, i, f, f, _P, i, f, f, f, f, f, _P, _P, _P, i, _P, sz,
                                       _P]
    L.ngv_warp_bwd_adam_slab.argtypes = [_P, dp, sp, _P, dp, xp, _P, _P, _P, _P, i, _P, f, f, f, f, _P, _P, i, _P,
                                         sz, _P]
    L.ngv_warp_bwd_adam_slab_mi.argtypes = [_P, dp, sp, _P, dp, xp, _P, _P, _P, i, f, f, f, f, f, _P, _P, _P, i, _P,
                                            f, f, f, f, _P, _P, i, _P, sz, _P]
    L.ngv_warp_compose.argtypes = [_P, dp, _P, dp, xp, _P, _P]
    L.ngv_warp_bwd_adam_mi.argtypes = [_P, dp, _P, dp, xp, _P, _P, i, f, f, f, f, f, _P, _P, i, _P, f, f, f, f, _P,
                                       _P, i, _P, sz, _P]
    for name in ("ngv_warp_fwd", "ngv_warp_fwd_slab", "ngv_warp_bwd", "ngv_mi_loss_fwd_bwd",
                 "ngv_lncc_loss_fwd_bwd", "ngv_adam_step", "ngv_warp_bwd_adam", "ngv_warp_zrange", "ngv_warp_fwd_mi", "ngv_mi_grad", "ngv_mse_loss_fwd_bwd",
                 "ngv_warp_compose", "ngv_mi_loss_fwd_bwd_order", "ngv_warp_bwd_adam_slab", "ngv_warp_bwd_adam_mi",
                 "ngv_mi_loss_fwd_bwd_noalloc", "ngv_warp_lncc_mi_bwd", "ngv_warp_bwd_adam_slab_mi"):
        getattr(L, name).restype = i
    _lib = L
    return L


def _check(code):
    if code != NGV_OK:
        raise NgvError(code, lib().ngv_status_str(code).decode())


def _dims(shape):
    nz, ny, nx = shape[-3:]
    return ngv_dims(nx, ny, nz)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _vol(t, name, dtype=torch.float32):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise NgvError(NGV_EINVAL, f"{name} must be a contiguous {dtype} CUDA tensor")


def _stream(stream, device):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _slab(slab):
    """None, (z0, nz) or (z0, nz, zrange) with zrange a CUDA tensor of 2
    float64 from ngv_warp_zrange."""
    if slab is None:
        return None
    z0, nz = slab[0], slab[1]
    zr = slab[2] if len(slab) > 2 else None
    if zr is not None:
        _vol(zr, "zrange", torch.float64)
        if zr.numel() != 2:
            raise NgvError(NGV_EINVAL, "zrange must hold 2 float64")
    return ngv_slab(int(z0), int(nz), None if zr is None else zr.data_ptr())


def make_xform(A=None, t=None, S=None, xmin=(-1.0, -1.0, -1.0), xmax=(1.0, 1.0, 1.0)):
    x = ngv_xform()
    A = np.eye(3) if A is None else np.asarray(A)
    t = np.zeros(3) if t is None else np.asarray(t)
    S = np.eye(3) if S is None else np.asarray(S)
    x.A[:] = [float(v) for v in np.asarray(A, np.float32).reshape(9)]
    x.t[:] = [float(v) for v in np.asarray(t, np.float32).reshape(3)]
    x.S[:] = [float(v) for v in np.asarray(S, np.float32).reshape(9)]
    x.xmin[:] = [float(v) for v in np.asarray(xmin, np.float32).reshape(3)]
    x.xmax[:] = [float(v) for v in np.asarray(xmax, np.float32).reshape(3)]
    return x


def ngv_workspace_bytes(bins=32, win=9):
    return int(lib().ngv_workspace_bytes(bins, win))


_ws_cache = {}


def workspace(device, bins=32, win=9):
    """A cached workspace buffer for calls on `device` (O(1) in the volume size)."""
    need = ngv_workspace_bytes(bins, win)
    key = torch.device(device)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=key)
        _ws_cache[key] = ws
    return ws


def ngv_warp_fwd(M, u, xform, W, mdims=None, slab=None, accumulate=False, stream=None):
    """W (+)= M~(A x + t + S u(x)). M: (nz_slab, ny, nx) planes of a moving image
    of size mdims = (nz, ny, nx) (default: M's shape); slab = (z0, nz) or
    (z0, nz, zrange) with zrange from ngv_warp_zrange."""
    for t_, n in ((M, "M"), (u, "u"), (W, "W")):
        _vol(t_, n)
    md = _dims(mdims if mdims is not None else M.shape)
    sl = _slab(slab)
    _check(lib().ngv_warp_fwd(_ptr(M), ctypes.byref(md), ctypes.byref(sl) if sl else None, _ptr(u),
                              ctypes.byref(_dims(W.shape)), ctypes.byref(xform), _ptr(W), int(accumulate),
                              _stream(stream, W.device)))


def ngv_warp_fwd_slab(M, u, xform, W, slab, mdims=None, stream=None):
    """One call of a sequence over the slabs (z0, nz, zrange), in increasing z:
    the first slab that reaches a voxel writes its part of W, later ones add;
    the top slab's call zeroes the voxels no slab reaches."""
    for t_, n in ((M, "M"), (u, "u"), (W, "W")):
        _vol(t_, n)
    md = _dims(mdims if mdims is not None else M.shape)
    sl = _slab(slab)
    _check(lib().ngv_warp_fwd_slab(_ptr(M), ctypes.byref(md), ctypes.byref(sl) if sl else None, _ptr(u),
                                   ctypes.byref(_dims(W.shape)), ctypes.byref(xform), _ptr(W),
                                   _stream(stream, W.device)))


def ngv_warp_bwd(M, u, xform, gW, gu, gA9, gt3, mdims=None, slab=None, accumulate=False, ws=None, stream=None):
    for t_, n in ((M, "M"), (u, "u"), (gW, "gW"), (gu, "gu")):
        _vol(t_, n)
    _vol(gA9, "gA9", torch.float64)
    _vol(gt3, "gt3", torch.float64)
    md = _dims(mdims if mdims is not None else M.shape)
    sl = _slab(slab)
    ws = ws if ws is not None else workspace(gW.device)
    _check(lib().ngv_warp_bwd(_ptr(M), ctypes.byref(md), ctypes.byref(sl) if sl else None, _ptr(u),
                              ctypes.byref(_dims(gW.shape)), ctypes.byref(xform), _ptr(gW), _ptr(gu), _ptr(gA9),
                              _ptr(gt3), int(accumulate), _ptr(ws), ws.numel(), _stream(stream, gW.device)))


def ngv_mi_loss_fwd_bwd(F, W, loss, gW=None, bins=32, frange=(0.0, 1.0), wrange=(0.0, 1.0), weight=1.0,
                        accumulate=False, ws=None, stream=None):
    for t_, n in ((F, "F"), (W, "W"), (gW, "gW")):
        _vol(t_, n)
    _vol(loss, "loss", torch.float64)
    ws = ws if ws is not None else workspace(F.device, bins)
    _check(lib().ngv_mi_loss_fwd_bwd(_ptr(F), _ptr(W), ctypes.byref(_dims(F.shape)), bins, frange[0], frange[1],
                                     wrange[0], wrange[1], weight, _ptr(loss), _ptr(gW), int(accumulate), _ptr(ws),
                                     ws.numel(), _stream(stream, F.device)))


def ngv_mi_loss_fwd_bwd_noalloc(F, W, loss, gW=None, bins=32, frange=(0.0, 1.0), wrange=(0.0, 1.0), weight=1.0,
                                accumulate=False, stream=None):
    """ngv_mi_loss_fwd_bwd with the library's fixed per-GPU scratch instead of
    a workspace (no device allocation, here or in the library)."""
    for t_, n in ((F, "F"), (W, "W"), (gW, "gW")):
        _vol(t_, n)
    _vol(loss, "loss", torch.float64)
    _check(lib().ngv_mi_loss_fwd_bwd_noalloc(_ptr(F), _ptr(W), ctypes.byref(_dims(F.shape)), bins, frange[0],
                                             frange[1], wrange[0], wrange[1], weight, _ptr(loss), _ptr(gW),
                                             int(accumulate), _stream(stream, F.device)))


def ngv_mi_loss_fwd_bwd_order(F, W, loss, gW=None, bins=32, fixed_order=0, frange=(0.0, 1.0), wrange=(0.0, 1.0),
                              weight=1.0, accumulate=False, ws=None, stream=None):
    """MI with the fixed image's Parzen kernel of the given order (0: box, as in
    Mattes et al.'s original pair; 3: cubic B-spline, as ngv_mi_loss_fwd_bwd)."""
    for t_, n in ((F, "F"), (W, "W"), (gW, "gW")):
        _vol(t_, n)
    _vol(loss, "loss", torch.float64)
    ws = ws if ws is not None else workspace(F.device, bins)
    _check(lib().ngv_mi_loss_fwd_bwd_order(_ptr(F), _ptr(W), ctypes.byref(_dims(F.shape)), bins, int(fixed_order),
                                           frange[0], frange[1], wrange[0], wrange[1], weight, _ptr(loss), _ptr(gW),
                                           int(accumulate), _ptr(ws), ws.numel(), _stream(stream, F.device)))


def ngv_lncc_loss_fwd_bwd(F, W, loss, gW=None, win=9, eps=1e-5, weight=1.0, accumulate=False, ws=None,
                          stream=None):
    for t_, n in ((F, "F"), (W, "W"), (gW, "gW")):
        _vol(t_, n)
    _vol(loss, "loss", torch.float64)
    ws = ws if ws is not None else workspace(F.device, 32, win)
    _check(lib().ngv_lncc_loss_fwd_bwd(_ptr(F), _ptr(W), ctypes.byref(_dims(F.shape)), win, eps, weight,
                                       _ptr(loss), _ptr(gW), int(accumulate), _ptr(ws), ws.numel(),
                                       _stream(stream, F.device)))


def _step_dev(step_dev):
    if step_dev is not None:
        _vol(step_dev, "step_dev", torch.int32)
    return _ptr(step_dev)


def ngv_adam_step(u, gu, m1, m2, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, smooth_sigma=0.0, ws=None,
                  stream=None, step_dev=None):
    """step_dev: None, or a CUDA int32 tensor holding the step number (then
    `step` is ignored), for updates replayed from a captured graph."""
    for t_, n in ((u, "u"), (gu, "gu"), (m1, "m1"), (m2, "m2")):
        _vol(t_, n)
    ws = ws if ws is not None else workspace(u.device)
    _check(lib().ngv_adam_step(_ptr(u), _ptr(gu), _ptr(m1), _ptr(m2), ctypes.byref(_dims(u.shape)), int(step),
                               _step_dev(step_dev), lr, beta1, beta2, eps, smooth_sigma, _ptr(ws), ws.numel(),
                               _stream(stream, u.device)))


def ngv_warp_bwd_adam(M, u, xform, gW, m1, m2, step, lr, gA9, gt3, gu_partial=None, beta1=0.9, beta2=0.999,
                      eps=1e-8, mdims=None, slab=None, accumulate_affine=False, ws=None, stream=None, step_dev=None):
    """Sampler backward of this slab plus gu_partial, fed into the Adam step of
    u, m1, m2 in place (no smoothing); dA, dt (+)= this slab's sums."""
    for t_, n in ((M, "M"), (u, "u"), (gW, "gW"), (m1, "m1"), (m2, "m2"), (gu_partial, "gu_partial")):
        _vol(t_, n)
    _vol(gA9, "gA9", torch.float64)
    _vol(gt3, "gt3", torch.float64)
    md = _dims(mdims if mdims is not None else M.shape)
    sl = _slab(slab)
    ws = ws if ws is not None else workspace(gW.device)
    _check(lib().ngv_warp_bwd_adam(_ptr(M), ctypes.byref(md), ctypes.byref(sl) if sl else None, _ptr(u),
                                   ctypes.byref(_dims(gW.shape)), ctypes.byref(xform), _ptr(gW), _ptr(gu_partial),
                                   _ptr(m1), _ptr(m2), int(step), _step_dev(step_dev), lr, beta1, beta2, eps,
                                   _ptr(gA9), _ptr(gt3), int(accumulate_affine), _ptr(ws), ws.numel(),
                                   _stream(stream, gW.device)))


def ngv_warp_bwd_adam_mi(M, u, xform, F, gW, m1, m2, step, lr, gA9, gt3, bins=32, frange=(0.0, 1.0),
                         wrange=(0.0, 1.0), weight=1.0, beta1=0.9, beta2=0.999, eps=1e-8, mdims=None,
                         accumulate_affine=False, ws=None, stream=None, step_dev=None):
    """Sampler backward with the MI gradient formed in the same sweep (from F,
    the recomputed W and the table of the latest MI forward in ws) plus gW
    (None: no other term), fed into the Adam step of u, m1, m2 in place; whole
    moving image only; dA, dt (+)= the sums."""
    for t_, n in ((M, "M"), (u, "u"), (F, "F"), (gW, "gW"), (m1, "m1"), (m2, "m2")):
        _vol(t_, n)
    _vol(gA9, "gA9", torch.float64)
    _vol(gt3, "gt3", torch.float64)
    md = _dims(mdims if mdims is not None else M.shape)
    ws = ws if ws is not None else workspace(F.device, bins)
    _check(lib().ngv_warp_bwd_adam_mi(_ptr(M), ctypes.byref(md), _ptr(u), ctypes.byref(_dims(F.shape)),
                                      ctypes.byref(xform), _ptr(F), _ptr(gW), bins, frange[0], frange[1], wrange[0],
                                      wrange[1], weight, _ptr(m1), _ptr(m2), int(step), _step_dev(step_dev), lr, beta1,
                                      beta2, eps, _ptr(gA9), _ptr(gt3), int(accumulate_affine), _ptr(ws), ws.numel(),
                                      _stream(stream, F.device)))


def ngv_warp_bwd_adam_slab(M, u, xform, gW, gu, m1, m2, step, lr, gA9, gt3, slab, beta1=0.9, beta2=0.999,
                           eps=1e-8, mdims=None, accumulate_affine=False, ws=None, stream=None, step_dev=None):
    """One call of a sequence over the slabs (z0, nz, zrange), in increasing z:
    this slab's part of the sampler backward; voxels no later slab reaches get
    their Adam step on u, m1, m2; gu is scratch for the partial sums."""
    for t_, n in ((M, "M"), (u, "u"), (gW, "gW"), (gu, "gu"), (m1, "m1"), (m2, "m2")):
        _vol(t_, n)
    _vol(gA9, "gA9", torch.float64)
    _vol(gt3, "gt3", torch.float64)
    md = _dims(mdims if mdims is not None else M.shape)
    sl = _slab(slab)
    ws = ws if ws is not None else workspace(gW.device)
    _check(lib().ngv_warp_bwd_adam_slab(_ptr(M), ctypes.byref(md), ctypes.byref(sl) if sl else None, _ptr(u),
                                        ctypes.byref(_dims(gW.shape)), ctypes.byref(xform), _ptr(gW), _ptr(gu),
                                        _ptr(m1), _ptr(m2), int(step), _step_dev(step_dev), lr, beta1, beta2, eps,
                                        _ptr(gA9), _ptr(gt3), int(accumulate_affine), _ptr(ws), ws.numel(),
                                        _stream(stream, gW.device)))


def ngv_warp_bwd_adam_slab_mi(M, u, xform, gW, F, W, gu, m1, m2, step, lr, gA9, gt3, slab, bins=32,
                              frange=(0.0, 1.0), wrange=(0.0, 1.0), weight_mi=1.0, beta1=0.9, beta2=0.999, eps=1e-8,
                              mdims=None, accumulate_affine=False, ws=None, stream=None, step_dev=None):
    """ngv_warp_bwd_adam_slab with the MI gradient formed in the call from F,
    the stored W and the table of the latest MI forward in ws, added to gW's
    value (gW None: the MI term alone)."""
    for t_, n in ((M, "M"), (u, "u"), (gW, "gW"), (F, "F"), (W, "W"), (gu, "gu"), (m1, "m1"), (m2, "m2")):
        _vol(t_, n)
    _vol(gA9, "gA9", torch.float64)
    _vol(gt3, "gt3", torch.float64)
    md = _dims(mdims if mdims is not None else M.shape)
    sl = _slab(slab)
    ws = ws if ws is not None else workspace(F.device, bins)
    _check(lib().ngv_warp_bwd_adam_slab_mi(_ptr(M), ctypes.byref(md), ctypes.byref(sl) if sl else None, _ptr(u),
                                           ctypes.byref(_dims(F.shape)), ctypes.byref(xform), _ptr(gW), _ptr(F),
                                           _ptr(W), bins, frange[0], frange[1], wrange[0], wrange[1], weight_mi,
                                           _ptr(gu), _ptr(m1), _ptr(m2), int(step), _step_dev(step_dev), lr, beta1,
                                           beta2, eps, _ptr(gA9), _ptr(gt3), int(accumulate_affine), _ptr(ws),
                                           ws.numel(), _stream(stream, F.device)))


def ngv_warp_zrange(u, xform, zrange, mdims, ws=None, stream=None):
    """zrange[0], zrange[1] = min, max over the output grid of the z-component
    of S u in voxels of a moving grid of size mdims = (nz, ny, nx)."""
    _vol(u, "u")
    _vol(zrange, "zrange", torch.float64)
    ws = ws if ws is not None else workspace(u.device)
    _check(lib().ngv_warp_zrange(_ptr(u), ctypes.byref(_dims(u.shape)), ctypes.byref(_dims(mdims)),
                                 ctypes.byref(xform), _ptr(zrange), _ptr(ws), ws.numel(), _stream(stream, u.device)))


def ngv_warp_fwd_mi(M, u, xform, W, F, loss, bins=32, frange=(0.0, 1.0), wrange=(0.0, 1.0), weight=1.0,
                    mdims=None, slab=None, accumulate=False, accumulate_loss=False, ws=None, stream=None):
    """ngv_warp_fwd plus the MI forward over (F, final W) in the same sweep;
    the log-ratio table stays in ws for ngv_mi_grad. W = None: the samples
    feed the histogram only (the first sweep of a fused step)."""
    for t_, n in ((M, "M"), (u, "u"), (W, "W"), (F, "F")):
        _vol(t_, n)
    _vol(loss, "loss", torch.float64)
    md = _dims(mdims if mdims is not None else M.shape)
    sl = _slab(slab)
    ws = ws if ws is not None else workspace(F.device, bins)
    _check(lib().ngv_warp_fwd_mi(_ptr(M), ctypes.byref(md), ctypes.byref(sl) if sl else None, _ptr(u),
                                 ctypes.byref(_dims(F.shape)), ctypes.byref(xform), _ptr(W), int(accumulate), _ptr(F),
                                 bins, frange[0], frange[1], wrange[0], wrange[1], weight, _ptr(loss),
                                 int(accumulate_loss), _ptr(ws), ws.numel(), _stream(stream, F.device)))


def ngv_warp_lncc_mi_bwd(M, u, xform, F, loss, gu, gA9, gt3, win=9, eps=1e-5, weight=1.0, bins=None,
                         frange=(0.0, 1.0), wrange=(0.0, 1.0), weight_mi=1.0, mdims=None, accumulate_affine=False,
                         ws=None, stream=None):
    """The second sweep of a fused step: W sampled where needed (never read
    or stored), the LNCC gradient plus (bins given) the MI gradient from the
    table in ws, and the sampler backward: gu, gA9, gt3 and the LNCC loss."""
    for t_, n in ((M, "M"), (u, "u"), (F, "F"), (gu, "gu")):
        _vol(t_, n)
    for t_, n in ((loss, "loss"), (gA9, "gA9"), (gt3, "gt3")):
        _vol(t_, n, torch.float64)
    md = _dims(mdims if mdims is not None else M.shape)
    ws = ws if ws is not None else workspace(F.device, bins or 32, win)
    _check(lib().ngv_warp_lncc_mi_bwd(_ptr(M), ctypes.byref(md), _ptr(u), ctypes.byref(_dims(F.shape)),
                                      ctypes.byref(xform), _ptr(F), int(win), eps, weight, _ptr(loss), int(bins or 0),
                                      frange[0], frange[1], wrange[0], wrange[1], weight_mi, _ptr(gu), _ptr(gA9),
                                      _ptr(gt3), int(accumulate_affine), _ptr(ws), ws.numel(),
                                      _stream(stream, F.device)))


def ngv_mi_grad(F, W, gW, bins=32, frange=(0.0, 1.0), wrange=(0.0, 1.0), weight=1.0, accumulate=False, ws=None,
                stream=None):
    """gW (+)= d(MI loss)/dW from the table of the latest MI forward in ws."""
    for t_, n in ((F, "F"), (W, "W"), (gW, "gW")):
        _vol(t_, n)
    ws = ws if ws is not None else workspace(F.device, bins)
    _check(lib().ngv_mi_grad(_ptr(F), _ptr(W), ctypes.byref(_dims(F.shape)), bins, frange[0], frange[1], wrange[0],
                             wrange[1], weight, _ptr(gW), int(accumulate), _ptr(ws), ws.numel(),
                             _stream(stream, F.device)))


def ngv_mse_loss_fwd_bwd(F, W, loss, gW=None, weight=1.0, accumulate=False, ws=None, stream=None):
    """loss (+)= weight * mean((W - F)^2); gW (+)= its gradient (None: loss only)."""
    for t_, n in ((F, "F"), (W, "W"), (gW, "gW")):
        _vol(t_, n)
    _vol(loss, "loss", torch.float64)
    ws = ws if ws is not None else workspace(F.device)
    _check(lib().ngv_mse_loss_fwd_bwd(_ptr(F), _ptr(W), ctypes.byref(_dims(F.shape)), weight, _ptr(loss), _ptr(gW),
                                      int(accumulate), _ptr(ws), ws.numel(), _stream(stream, F.device)))


def ngv_warp_compose(uf, v, xform, w, stream=None):
    """w = v + uf~(A x + t + S v(x)) per component; uf (3, nz, ny, nx) on its own
    grid, v and w (3, ...) on the output grid; w may be v (in place)."""
    for t_, n in ((uf, "uf"), (v, "v"), (w, "w")):
        _vol(t_, n)
    for t_, n in ((uf, "uf"), (v, "v"), (w, "w")):
        if t_.dim() != 4 or t_.shape[0] != 3:
            raise NgvError(NGV_EINVAL, f"{n} must have shape (3, nz, ny, nx)")
    if tuple(v.shape) != tuple(w.shape):
        raise NgvError(NGV_EINVAL, "v and w must have the same shape")
    _check(lib().ngv_warp_compose(_ptr(uf), ctypes.byref(_dims(uf.shape)), _ptr(v), ctypes.byref(_dims(v.shape)),
                                  ctypes.byref(xform), _ptr(w), _stream(stream, w.device)))
