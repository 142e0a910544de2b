"""The C-ABI library on the host: it loads, exports every entry point that
include/ngv.h declares, and rejects bad arguments before touching a device
(no compute call is made here)."""
import ctypes
import os
import re

import pytest

from non_gemm_voxel_amd import ngv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ngv.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"NGV_API\s+[\w\s\*]+?\b(ngv_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    assert names == sorted(["ngv_workspace_bytes", "ngv_warp_fwd", "ngv_warp_fwd_slab", "ngv_warp_bwd", "ngv_mi_loss_fwd_bwd",
                            "ngv_lncc_loss_fwd_bwd", "ngv_adam_step", "ngv_status_str",
                            "ngv_warp_bwd_adam", "ngv_warp_zrange", "ngv_warp_fwd_mi", "ngv_mi_grad",
                            "ngv_mse_loss_fwd_bwd", "ngv_warp_compose", "ngv_mi_loss_fwd_bwd_order",
                            "ngv_warp_bwd_adam_slab", "ngv_warp_bwd_adam_mi", "ngv_mi_loss_fwd_bwd_noalloc",
                            "ngv_warp_lncc_mi_bwd", "ngv_warp_bwd_adam_slab_mi"])


def test_library_exports_every_declared_symbol():
    L = ngv.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_workspace_is_independent_of_volume_size():
    """The workspace size takes no volume size at all: the O(1) extra memory
    contract. Windows up to 11 share one small layout; windows 13..31 add
    per-block slices that grow with the window (and stay below 256 MB)."""
    L = ngv.lib()
    a = L.ngv_workspace_bytes(32, 5)
    assert a == L.ngv_workspace_bytes(32, 9) == L.ngv_workspace_bytes(32, 11) == L.ngv_workspace_bytes(32, 0) \
        == L.ngv_workspace_bytes(0, 9)
    assert a % 256 == 0 and a < 1 << 20
    assert L.ngv_workspace_bytes(128, 9) >= 128 * 128 * 12
    big = [L.ngv_workspace_bytes(32, w) for w in range(13, 33, 2)]
    assert all(b % 256 == 0 for b in big)
    assert big == sorted(big) and big[0] > L.ngv_workspace_bytes(256, 11) and big[-1] < 256 << 20
    assert L.ngv_workspace_bytes(256, 13) == L.ngv_workspace_bytes(0, 13) == big[0]


def test_status_strings():
    L = ngv.lib()
    for code in (0, -1, -2, -3, -4, -99):
        assert L.ngv_status_str(code)


def _fake(n=1):
    """Non-null addresses that are never dereferenced: every call below fails
    its argument checks first."""
    return ctypes.c_void_p(0x1000 * n)


def test_invalid_arguments_are_rejected_before_any_work():
    L = ngv.lib()
    d = ngv.ngv_dims(8, 8, 8)
    bad = ngv.ngv_dims(8, 0, 8)
    xf = ngv.make_xform()
    ws, wsb = _fake(), L.ngv_workspace_bytes(32, 9)
    B = ctypes.byref
    # sampler
    assert L.ngv_warp_fwd(None, B(d), None, _fake(), B(d), B(xf), _fake(), 0, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_fwd(_fake(), B(bad), None, _fake(), B(d), B(xf), _fake(), 0, None) == ngv.NGV_EINVAL
    slab = ngv.ngv_slab(5, 4)  # planes 5..8 of an 8-plane image
    assert L.ngv_warp_fwd(_fake(), B(d), B(slab), _fake(), B(d), B(xf), _fake(), 0, None) == ngv.NGV_EINVAL
    nan = ngv.make_xform()
    nan.A[0] = float("nan")
    assert L.ngv_warp_fwd(_fake(), B(d), None, _fake(), B(d), B(nan), _fake(), 0, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_fwd(_fake(), B(d), None, _fake(), B(d), B(xf), _fake(), 2, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd(_fake(), B(d), None, _fake(), B(d), B(xf), _fake(), _fake(), _fake(), _fake(), 0,
                          ws, 16, None) == ngv.NGV_EWORKSPACE
    assert L.ngv_warp_bwd(_fake(), B(d), None, _fake(), B(d), B(xf), _fake(), _fake(), _fake(), None, 0,
                          ws, wsb, None) == ngv.NGV_EINVAL
    # MI
    args = (_fake(), _fake(), B(d))
    assert L.ngv_mi_loss_fwd_bwd(*args, 4, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd(*args, 257, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws, wsb,
                                 None) == ngv.NGV_EINVAL
    # 256 bins are valid: the call gets as far as the workspace, sized here for 32
    assert L.ngv_mi_loss_fwd_bwd(*args, 256, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws, wsb,
                                 None) == ngv.NGV_EWORKSPACE
    assert L.ngv_mi_loss_fwd_bwd(*args, 32, 1.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws, wsb,
                                 None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd(*args, 32, 0.0, 1.0, 0.0, 1.0, 1.0, None, None, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd(ctypes.c_void_p(0x1004), _fake(), B(d), 32, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None,
                                 0, ws, wsb, None) == ngv.NGV_EINVAL  # F not 16-byte aligned
    assert L.ngv_mi_loss_fwd_bwd(*args, 32, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, None, wsb,
                                 None) == ngv.NGV_EWORKSPACE
    # LNCC
    assert L.ngv_lncc_loss_fwd_bwd(*args, 4, 1e-5, 1.0, _fake(), None, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_lncc_loss_fwd_bwd(*args, 1, 1e-5, 1.0, _fake(), None, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_lncc_loss_fwd_bwd(*args, 9, -1.0, 1.0, _fake(), None, 0, ws, wsb, None) == ngv.NGV_EINVAL
    for win in (13, 31):  # valid windows whose kernel needs the larger workspace
        assert L.ngv_lncc_loss_fwd_bwd(*args, win, 1e-5, 1.0, _fake(), None, 0, ws, wsb,
                                       None) == ngv.NGV_EWORKSPACE
    assert L.ngv_lncc_loss_fwd_bwd(*args, 33, 1e-5, 1.0, _fake(), None, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_lncc_loss_fwd_bwd(*args, 9, 1e-5, 1.0, _fake(), None, 0, _fake(), 100,
                                   None) == ngv.NGV_EWORKSPACE
    # Adam
    p4 = (_fake(), _fake(), _fake(), _fake(), B(d))
    assert L.ngv_adam_step(*p4, 0, None, 0.1, 0.9, 0.999, 1e-8, 0.0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_adam_step(*p4, 1, None, 0.1, 1.0, 0.999, 1e-8, 0.0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_adam_step(*p4, 1, None, 0.1, 0.9, 0.999, 1e-8, 2.0, ws, wsb, None) == ngv.NGV_EUNSUPPORTED
    # a device step counter must be 4-byte aligned (the host step is then ignored)
    assert L.ngv_adam_step(*p4, 0, ctypes.c_void_p(0x1002), 0.1, 0.9, 0.999, 1e-8, 0.0, ws, wsb,
                           None) == ngv.NGV_EINVAL
    # sampler backward fused with Adam
    wa = (_fake(), B(d), None, _fake(), B(d), B(xf), _fake(), None, _fake(), _fake())
    assert L.ngv_warp_bwd_adam(*wa, 0, None, 0.1, 0.9, 0.999, 1e-8, _fake(), _fake(), 0, ws, wsb,
                               None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam(*wa, 1, None, 0.1, 0.9, 1.0, 1e-8, _fake(), _fake(), 0, ws, wsb,
                               None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam(*wa, 1, None, 0.1, 0.9, 0.999, 1e-8, _fake(), _fake(), 0, ws, 16,
                               None) == ngv.NGV_EWORKSPACE
    # slab z-range bound
    assert L.ngv_warp_zrange(_fake(), B(d), B(d), B(xf), None, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_zrange(_fake(), B(d), B(d), B(xf), ctypes.c_void_p(0x1004), ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_zrange(_fake(), B(d), B(d), B(xf), _fake(), ws, 16, None) == ngv.NGV_EWORKSPACE
    mis = ngv.ngv_slab(0, 4, 0x1004)  # zrange not 8-byte aligned
    assert L.ngv_warp_fwd(_fake(), B(d), B(mis), _fake(), B(d), B(xf), _fake(), 0, None) == ngv.NGV_EINVAL
    # sampler sweep with the MI forward; MI gradient from the table
    sw = (_fake(), B(d), None, _fake(), B(d), B(xf), _fake(), 0, _fake())
    assert L.ngv_warp_fwd_mi(*sw, 4, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_fwd_mi(*sw, 32, 0.0, 1.0, 0.0, 1.0, 1.0, None, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_fwd_mi(*sw, 32, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), 2, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_fwd_mi(*sw, 32, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), 0, ws, 16, None) == ngv.NGV_EWORKSPACE
    assert L.ngv_mi_grad(_fake(), _fake(), B(d), 32, 0.0, 1.0, 0.0, 1.0, 1.0, None, 0, ws, wsb,
                         None) == ngv.NGV_EINVAL
    assert L.ngv_mi_grad(_fake(), _fake(), B(d), 32, 1.0, 0.0, 0.0, 1.0, 1.0, _fake(), 0, ws, wsb,
                         None) == ngv.NGV_EINVAL
    assert L.ngv_mi_grad(_fake(), _fake(), B(d), 32, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), 0, ws, 8,
                         None) == ngv.NGV_EWORKSPACE
    wa0 = (_fake(), B(d), None, _fake(), B(d), B(xf), _fake(), None, None, _fake())
    assert L.ngv_warp_bwd_adam(*wa0, 1, None, 0.1, 0.9, 0.999, 1e-8, _fake(), _fake(), 0, ws, wsb,
                               None) == ngv.NGV_EINVAL
    # slab sequence of the sampler forward: a slab with a z-range bound is required
    fs = (_fake(), B(d))
    fs_rest = (_fake(), B(d), B(xf), _fake(), None)
    assert L.ngv_warp_fwd_slab(*fs, None, *fs_rest) == ngv.NGV_EINVAL
    assert L.ngv_warp_fwd_slab(*fs, B(ngv.ngv_slab(0, 8)), *fs_rest) == ngv.NGV_EINVAL
    assert L.ngv_warp_fwd_slab(*fs, B(ngv.ngv_slab(0, 8, 0x1000)), _fake(), B(d), B(xf), None,
                               None) == ngv.NGV_EINVAL
    # slab sequence of the fused backward: a slab with a z-range bound is required
    sb = (_fake(), B(d))
    rest = (_fake(), B(d), B(xf), _fake(), _fake(), _fake(), _fake(), 1, None, 0.1, 0.9, 0.999, 1e-8, _fake(), _fake(),
            0, ws, wsb, None)
    assert L.ngv_warp_bwd_adam_slab(*sb, None, *rest) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam_slab(*sb, B(ngv.ngv_slab(0, 8)), *rest) == ngv.NGV_EINVAL
    rest_ws = rest[:-3] + (ws, 16, None)
    assert L.ngv_warp_bwd_adam_slab(*sb, B(ngv.ngv_slab(0, 8, 0x1000)), *rest_ws) == ngv.NGV_EWORKSPACE
    # sampler backward with the MI gradient and Adam: F required, MI and Adam
    # parameters checked, the workspace size
    mi0 = (_fake(), B(d), _fake(), B(d), B(xf))
    mi_rest = (_fake(), _fake(), 1, None, 0.1, 0.9, 0.999, 1e-8, _fake(), _fake(), 0)
    assert L.ngv_warp_bwd_adam_mi(*mi0, None, None, 32, 0.0, 1.0, 0.0, 1.0, 1.0, *mi_rest, ws, wsb,
                                  None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam_mi(*mi0, _fake(), None, 4, 0.0, 1.0, 0.0, 1.0, 1.0, *mi_rest, ws, wsb,
                                  None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam_mi(*mi0, _fake(), None, 32, 0.0, 1.0, 1.0, 1.0, 1.0, *mi_rest, ws, wsb,
                                  None) == ngv.NGV_EINVAL
    bad_step = mi_rest[:2] + (0,) + mi_rest[3:]
    assert L.ngv_warp_bwd_adam_mi(*mi0, _fake(), None, 32, 0.0, 1.0, 0.0, 1.0, 1.0, *bad_step, ws, wsb,
                                  None) == ngv.NGV_EINVAL
    bad_acc = mi_rest[:-1] + (2,)
    assert L.ngv_warp_bwd_adam_mi(*mi0, _fake(), None, 32, 0.0, 1.0, 0.0, 1.0, 1.0, *bad_acc, ws, wsb,
                                  None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam_mi(*mi0, _fake(), None, 32, 0.0, 1.0, 0.0, 1.0, 1.0, *mi_rest, ws, 16,
                                  None) == ngv.NGV_EWORKSPACE
    # the second sweep of the fused step: window, MI and affine arguments,
    # gu must not overlap u, the workspace size
    fz = (_fake(), B(d), _fake(2), B(d), B(xf), _fake(3))
    lr_ = (1e-5, 1.0, _fake(4))
    mi_ = (0.0, 1.0, 0.0, 1.0, 1.0)
    out = (_fake(5), _fake(6), _fake(7))
    assert L.ngv_warp_lncc_mi_bwd(*fz, 8, *lr_, 32, *mi_, *out, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_lncc_mi_bwd(*fz, 33, *lr_, 32, *mi_, *out, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_lncc_mi_bwd(*fz, 13, *lr_, 32, *mi_, *out, 0, ws, wsb, None) == ngv.NGV_EUNSUPPORTED
    assert L.ngv_warp_lncc_mi_bwd(*fz, 9, -1.0, 1.0, _fake(4), 32, *mi_, *out, 0, ws, wsb,
                                  None) == ngv.NGV_EINVAL
    assert L.ngv_warp_lncc_mi_bwd(*fz, 9, 1e-5, 1.0, None, 32, *mi_, *out, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_lncc_mi_bwd(*fz, 9, *lr_, 4, *mi_, *out, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_lncc_mi_bwd(*fz, 9, *lr_, 32, 1.0, 0.0, 0.0, 1.0, 1.0, *out, 0, ws, wsb,
                                  None) == ngv.NGV_EINVAL
    assert L.ngv_warp_lncc_mi_bwd(*fz, 9, *lr_, 32, *mi_, *out, 2, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_lncc_mi_bwd(*fz, 9, *lr_, 32, *mi_, _fake(2), _fake(6), _fake(7), 0, ws, wsb,
                                  None) == ngv.NGV_EINVAL  # gu is u
    assert L.ngv_warp_lncc_mi_bwd(*fz, 9, *lr_, 32, *mi_, ctypes.c_void_p(0x2000 - 4), _fake(6), _fake(7), 0, ws,
                                  wsb, None) == ngv.NGV_EINVAL  # gu overlaps u
    assert L.ngv_warp_lncc_mi_bwd(*fz, 9, *lr_, 32, *mi_, *out, 0, ws, 16, None) == ngv.NGV_EWORKSPACE
    # the backward slab sequence with the MI gradient: F and the stored W
    # required (gW may be null), a slab with a z-range bound, MI and Adam
    # parameters, the workspace size
    sm0 = (_fake(), B(d))
    sm1 = (_fake(2), B(d), B(xf), None)
    smi = (0.0, 1.0, 0.0, 1.0, 1.0, _fake(5), _fake(6), _fake(7), 1, None, 0.1, 0.9, 0.999, 1e-8, _fake(8), _fake(9), 0)
    zs = B(ngv.ngv_slab(0, 8, 0x1000))
    assert L.ngv_warp_bwd_adam_slab_mi(*sm0, zs, *sm1, _fake(3), None, 32, *smi, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam_slab_mi(*sm0, zs, *sm1, None, _fake(4), 32, *smi, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam_slab_mi(*sm0, B(ngv.ngv_slab(0, 8)), *sm1, _fake(3), _fake(4), 32, *smi, ws, wsb,
                                       None) == ngv.NGV_EINVAL  # no z-range bound
    assert L.ngv_warp_bwd_adam_slab_mi(*sm0, zs, *sm1, _fake(3), _fake(4), 4, *smi, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam_slab_mi(*sm0, zs, *sm1, _fake(3), _fake(4), 129, *smi, ws,
                                       L.ngv_workspace_bytes(256, 0), None) == ngv.NGV_EUNSUPPORTED
    bad_acc = smi[:-1] + (2,)
    assert L.ngv_warp_bwd_adam_slab_mi(*sm0, zs, *sm1, _fake(3), _fake(4), 32, *bad_acc, ws, wsb,
                                       None) == ngv.NGV_EINVAL
    assert L.ngv_warp_bwd_adam_slab_mi(*sm0, zs, *sm1, _fake(3), _fake(4), 32, *smi, ws, 16,
                                       None) == ngv.NGV_EWORKSPACE
    # MI with a choice of the fixed kernel
    assert L.ngv_mi_loss_fwd_bwd_order(*args, 32, 1, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws, wsb,
                                       None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd_order(*args, 4, 0, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws, wsb,
                                       None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd_order(*args, 32, 0, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws, 8,
                                       None) == ngv.NGV_EWORKSPACE
    # MSE
    assert L.ngv_mse_loss_fwd_bwd(*args, 1.0, None, None, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_mse_loss_fwd_bwd(*args, float("inf"), _fake(), None, 0, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_mse_loss_fwd_bwd(*args, 1.0, _fake(), None, 2, ws, wsb, None) == ngv.NGV_EINVAL
    assert L.ngv_mse_loss_fwd_bwd(*args, 1.0, _fake(), ctypes.c_void_p(0x1008), 0, ws, wsb,
                                  None) == ngv.NGV_EINVAL  # gW not 16-byte aligned
    assert L.ngv_mse_loss_fwd_bwd(*args, 1.0, _fake(), None, 0, ws, 16, None) == ngv.NGV_EWORKSPACE
    # warp composition: w overlapping the sampled field, bad grid, null pointers
    vol = 3 * 4 * 8 * 8 * 8
    assert L.ngv_warp_compose(_fake(), B(d), _fake(2), B(d), B(xf), ctypes.c_void_p(0x1000 + vol - 4),
                              None) == ngv.NGV_EINVAL
    assert L.ngv_warp_compose(_fake(), B(d), _fake(2), B(bad), B(xf), _fake(4), None) == ngv.NGV_EINVAL
    assert L.ngv_warp_compose(None, B(d), _fake(2), B(d), B(xf), _fake(4), None) == ngv.NGV_EINVAL
    assert L.ngv_warp_compose(_fake(), B(d), _fake(2), B(d), B(nan), _fake(4), None) == ngv.NGV_EINVAL


def test_size_limits():
    """Volumes whose voxel count overflows 64-bit indexing are invalid; the
    sampler calls (32-bit index arithmetic) stop at extents of 2^30 and
    moving-image planes of 2^31 voxels; the MI calls (32.32 fixed-point
    histogram in 64 bits) stop below 2^32 voxels; the calls that hold the MI
    histogram or table in LDS stop at 128 bins."""
    L = ngv.lib()
    B = ctypes.byref
    xf = ngv.make_xform()
    d = ngv.ngv_dims(8, 8, 8)
    huge = ngv.ngv_dims(1 << 31, 1 << 31, 1 << 31)
    assert L.ngv_warp_fwd(_fake(), B(d), None, _fake(), B(huge), B(xf), _fake(), 0, None) == ngv.NGV_EINVAL
    # the sampler's 32-bit index arithmetic: extents up to 2^30 in both grids,
    # moving-image planes below 2^31 voxels
    long_x = ngv.ngv_dims((1 << 30) + 1, 2, 2)
    at_lim = ngv.ngv_dims(1 << 30, 1, 1)
    wide = ngv.ngv_dims(1 << 16, 1 << 15, 2)  # a 2^31-voxel plane
    for md_, od_ in ((long_x, d), (d, long_x), (wide, d)):
        assert L.ngv_warp_fwd(_fake(), B(md_), None, _fake(), B(od_), B(xf), _fake(), 0, None) == \
            ngv.NGV_EUNSUPPORTED
        assert L.ngv_warp_zrange(_fake(), B(od_), B(md_), B(xf), _fake(), _fake(), L.ngv_workspace_bytes(256, 9),
                                 None) == ngv.NGV_EUNSUPPORTED
    assert L.ngv_warp_compose(_fake(), B(wide), _fake(), B(d), B(xf), _fake(1 << 40), None) == ngv.NGV_EUNSUPPORTED
    nan = ngv.make_xform(A=[[float("nan"), 0, 0], [0, 1, 0], [0, 0, 1]])
    assert L.ngv_warp_fwd(_fake(), B(wide), None, _fake(), B(d), B(nan), _fake(), 0, None) == ngv.NGV_EINVAL
    big = ngv.ngv_dims(2048, 2048, 1024)  # 2^32 voxels
    just = ngv.ngv_dims(2048, 2048, 1023)
    ws, wsb = _fake(), L.ngv_workspace_bytes(256, 9)
    assert L.ngv_workspace_bytes(256, 0) >= 256 * 256 * 12
    args = (_fake(), _fake(), B(big))
    assert L.ngv_mi_loss_fwd_bwd(*args, 32, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws, wsb,
                                 None) == ngv.NGV_EUNSUPPORTED
    assert L.ngv_mi_loss_fwd_bwd_order(*args, 32, 0, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws, wsb,
                                       None) == ngv.NGV_EUNSUPPORTED
    assert L.ngv_mi_grad(*args, 32, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), 0, ws, wsb, None) == ngv.NGV_EUNSUPPORTED
    # one plane less, 256 bins: past the size check, refused for a short workspace
    assert L.ngv_mi_loss_fwd_bwd(_fake(), _fake(), B(just), 256, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0, ws,
                                 L.ngv_workspace_bytes(32, 0), None) == ngv.NGV_EWORKSPACE
    sw = (_fake(), B(d), None, _fake(), B(big), B(xf), _fake(), 0, _fake())
    assert L.ngv_warp_fwd_mi(*sw, 32, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), 0, ws, wsb, None) == ngv.NGV_EUNSUPPORTED
    sw = (_fake(), B(d), None, _fake(), B(d), B(xf), _fake(), 0, _fake())
    assert L.ngv_warp_fwd_mi(*sw, 129, 0.0, 1.0, 0.0, 1.0, 1.0, _fake(), 0, ws, wsb, None) == ngv.NGV_EUNSUPPORTED
    mi_rest = (_fake(), _fake(), 1, None, 0.1, 0.9, 0.999, 1e-8, _fake(), _fake(), 0, ws, wsb, None)
    assert L.ngv_warp_bwd_adam_mi(_fake(), B(d), _fake(), B(big), B(xf), _fake(), None, 32, 0.0, 1.0, 0.0, 1.0,
                                  1.0, *mi_rest) == ngv.NGV_EUNSUPPORTED
    assert L.ngv_warp_bwd_adam_mi(_fake(), B(d), _fake(), B(d), B(xf), _fake(), None, 256, 0.0, 1.0, 0.0, 1.0,
                                  1.0, *mi_rest) == ngv.NGV_EUNSUPPORTED
    # the second sweep of the fused step reads the MI table from the
    # workspace (any bin count) but holds the MI size limit
    assert L.ngv_warp_lncc_mi_bwd(_fake(), B(d), _fake(2), B(big), B(xf), _fake(3), 9, 1e-5, 1.0, _fake(4), 32,
                                  0.0, 1.0, 0.0, 1.0, 1.0, _fake(1 << 40), _fake(6), _fake(7), 0, ws, wsb,
                                  None) == ngv.NGV_EUNSUPPORTED


def test_noalloc_mi_argument_checks():
    """The MI call without a workspace checks its arguments like the one with
    a workspace, and refuses more bins than its fixed scratch holds."""
    L = ngv.lib()
    B = ctypes.byref
    d = ngv.ngv_dims(8, 8, 8)
    args = (_fake(), _fake(), B(d))
    rng = (0.0, 1.0, 0.0, 1.0, 1.0)
    assert L.ngv_mi_loss_fwd_bwd_noalloc(*args, 129, *rng, _fake(), None, 0, None) == ngv.NGV_EUNSUPPORTED
    assert L.ngv_mi_loss_fwd_bwd_noalloc(*args, 257, *rng, _fake(), None, 0, None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd_noalloc(*args, 4, *rng, _fake(), None, 0, None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd_noalloc(None, _fake(), B(d), 32, *rng, _fake(), None, 0, None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd_noalloc(*args, 32, *rng, None, None, 0, None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd_noalloc(*args, 32, *rng, _fake(), None, 2, None) == ngv.NGV_EINVAL
    assert L.ngv_mi_loss_fwd_bwd_noalloc(*args, 32, 1.0, 1.0, 0.0, 1.0, 1.0, _fake(), None, 0,
                                         None) == ngv.NGV_EINVAL
    big = ngv.ngv_dims(2048, 2048, 1024)
    assert L.ngv_mi_loss_fwd_bwd_noalloc(_fake(), _fake(), B(big), 32, *rng, _fake(), None, 0,
                                         None) == ngv.NGV_EUNSUPPORTED


def test_binding_refuses_host_tensors():
    import torch
    F = torch.zeros((4, 4, 4))
    loss = torch.zeros(1, dtype=torch.float64)
    with pytest.raises(ngv.NgvError):
        ngv.ngv_lncc_loss_fwd_bwd(F, F, loss, win=3)


def test_header_is_c99_and_links(tmp_path):
    """A C99 program includes the header, links the library and makes the
    calls that need no device (sizes, status strings, argument checks)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = os.path.join(ROOT, "tests", "abi_c", "abi_check.c")
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(ngv.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}",
                        src, "-o", exe, f"-L{libdir}", "-l:libngv.so", f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "abi check ok" in r.stdout, r.stdout + r.stderr


def test_c_program_names_every_entry_point():
    """The C99 program takes the address of every function the header
    declares, so a declaration without a definition fails to link."""
    with open(os.path.join(ROOT, "include", "ngv.h")) as f:
        declared = set(re.findall(r"NGV_API\s+[\w\s\*]*?\b(ngv_\w+)\s*\(", f.read()))
    with open(os.path.join(ROOT, "tests", "abi_c", "abi_check.c")) as f:
        prog = f.read()
    assert declared and all(f"(entry_fn){n}" in prog for n in declared), sorted(
        n for n in declared if f"(entry_fn){n}" not in prog)


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With the library missing, the binding raises at the first call: there
    is no other path to fall back on."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from non_gemm_voxel_amd import ngv\n"
            "ngv.LIB_PATH = %r\n"
            "try:\n"
            "    ngv.lib()\n"
            "except ngv.NgvError as e:\n"
            "    print('raised', e)\n"
            "    raise SystemExit(0)\n"
            "raise SystemExit(1)\n") % (ROOT, str(tmp_path / "libngv.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "raised" in r.stdout, r.stdout + r.stderr
