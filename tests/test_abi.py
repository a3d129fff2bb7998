"""The C ABI loads, exports what include/fa.h declares, and rejects bad
arguments before touching the device (CPU only: no compute is launched)."""
import ctypes
import os
import re

import pytest

import io_aware_exact_20_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# Aligned, never dereferenced: every call below fails validation first.
FAKE = ctypes.c_void_p(0x10000)
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fa.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_dropout_mask",
            "fa_status_str", "fa_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_params_layout_matches_header():
    assert ctypes.sizeof(fa.Params) == 64
    assert fa.Params.seed.offset == 48 and fa.Params.out_f32.offset == 56


def _p(**kw):
    base = dict(B=1, H=2, N=16, d=64, dtype=fa.BF16, scale=0.125, causal=False,
                dropout_p=0.0, seed=0, out_f32=False)
    base.update(kw)
    return fa.make_params(**base)


def _fwd(lib, p, ptr=FAKE):
    return lib.fa_fwd(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, None)


BAD = [
    (dict(B=-1), fa.FA_EINVAL), (dict(H=-3), fa.FA_EINVAL), (dict(N=-1), fa.FA_EINVAL),
    (dict(N=2**31), fa.FA_EINVAL), (dict(d=80), fa.FA_EUNSUPPORTED),
    (dict(d=0), fa.FA_EUNSUPPORTED), (dict(d=512), fa.FA_EUNSUPPORTED),
    (dict(d=256, dtype=fa.F32), fa.FA_EUNSUPPORTED), (dict(dtype=7), fa.FA_EUNSUPPORTED),
    (dict(scale=0.0), fa.FA_EINVAL), (dict(scale=-1.0), fa.FA_EINVAL),
    (dict(scale=float("inf")), fa.FA_EINVAL), (dict(scale=float("nan")), fa.FA_EINVAL),
    (dict(dropout_p=1.0), fa.FA_EINVAL), (dict(dropout_p=-0.1), fa.FA_EINVAL),
    (dict(dropout_p=float("nan")), fa.FA_EINVAL),
]


@pytest.mark.parametrize("kw,status", BAD)
def test_invalid_params_rejected_before_launch(lib, kw, status):
    p = _p(**kw)
    assert _fwd(lib, p) == status
    assert lib.fa_last_error().decode()
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(p)) == ctypes.c_size_t(-1).value


def test_bad_flags_and_key_length(lib):
    p = _p()
    p.causal = 2
    assert _fwd(lib, p) == fa.FA_EINVAL
    p = _p()
    p.out_f32 = 5
    assert _fwd(lib, p) == fa.FA_EINVAL
    p = _p()
    p.Nk = -1
    assert _fwd(lib, p) == fa.FA_EINVAL
    # one head past 4 GiB (32-bit byte offsets)
    p = _p(N=2**24, d=128)
    assert _fwd(lib, p) == fa.FA_EUNSUPPORTED
    p = _p(N=16, d=128)
    p.Nk = 2**24
    assert _fwd(lib, p) == fa.FA_EUNSUPPORTED


def test_backward_workspace_follows_the_query_rows(lib):
    """The workspace holds per-query-row statistics: Nk does not change it."""
    p = _p(B=2, H=3, N=100, d=64)
    base = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    for nk in (1, 17, 5000):
        p.Nk = nk
        assert lib.fa_bwd_workspace_bytes(ctypes.byref(p)) == base


def test_split_forward_workspace_and_validation(lib):
    B, H, N, d = 2, 3, 5, 64
    p = _p(B=B, H=H, N=N, d=d)
    p.Nk = 1000
    sz = ctypes.c_size_t(-1).value
    assert lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), 0) == sz
    assert lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), 257) == sz
    # one chunk (all 1000 keys fit 1024 = 16 * 64): plain forward, no workspace
    assert lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), 1) == 0
    # 4 requested -> chunks of 256 keys, 4 used; O then LSE of every chunk
    rows = B * H * N
    o_bytes = (4 * rows * d * 4 + 255) // 256 * 256
    lse_bytes = 4 * ((rows * 4 + 255) // 256 * 256)
    assert lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), 4) == o_bytes + lse_bytes
    for bad in (0, 257, -3):
        assert lib.fa_fwd_splitkv(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, bad, FAKE,
                                  1 << 30, None) == fa.FA_EINVAL
    # workspace too small for the requested splits
    assert lib.fa_fwd_splitkv(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                              o_bytes, None) == fa.FA_EINVAL
    assert "workspace" in lib.fa_last_error().decode()


def test_null_and_misaligned_pointers(lib):
    p = _p()
    assert lib.fa_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == fa.FA_EINVAL
    assert lib.fa_fwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, None) == fa.FA_EINVAL
    assert "q is NULL" in lib.fa_last_error().decode()
    assert lib.fa_fwd(ctypes.byref(p), FAKE, FAKE, MISALIGNED, FAKE, FAKE, None) == fa.FA_EINVAL
    assert "v is not 16-byte aligned" in lib.fa_last_error().decode()


def test_empty_problem_is_ok_without_launch(lib):
    for kw in (dict(B=0), dict(H=0), dict(N=0)):
        p = _p(**kw)
        assert lib.fa_fwd(ctypes.byref(p), None, None, None, None, None, None) == fa.FA_OK
        assert lib.fa_bwd_workspace_bytes(ctypes.byref(p)) == 0
        assert lib.fa_bwd(ctypes.byref(p), *([None] * 10), 0, None) == fa.FA_OK


def test_workspace_size_and_too_small_workspace(lib):
    p = _p(B=2, H=3, N=100, d=128)
    rows = 2 * 3 * 100
    need = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    assert need == 2 * ((rows * 4 + 255) // 256 * 256)
    args = [FAKE] * 10
    assert lib.fa_bwd(ctypes.byref(p), *args, need - 1, None) == fa.FA_EINVAL
    assert "workspace" in lib.fa_last_error().decode()


def test_dropout_mask_validation(lib):
    p = _p(B=2, H=2, N=8, dropout_p=0.5)
    assert lib.fa_dropout_mask(ctypes.byref(p), 2, 0, FAKE, None) == fa.FA_EINVAL
    assert lib.fa_dropout_mask(ctypes.byref(p), 0, -1, FAKE, None) == fa.FA_EINVAL
    assert lib.fa_dropout_mask(ctypes.byref(p), 0, 0, None, None) == fa.FA_EINVAL
    p.dropout_p = 1.5
    assert lib.fa_dropout_mask(ctypes.byref(p), 0, 0, FAKE, None) == fa.FA_EINVAL


def test_status_strings(lib):
    for s in (fa.FA_OK, fa.FA_EINVAL, fa.FA_EUNSUPPORTED, fa.FA_EHIP):
        assert lib.fa_status_str(s).decode().startswith("FA_")


def test_backward_stages_validate(lib):
    p = _p(B=1, H=1, N=32, d=64)
    need = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    assert lib.fa_bwd_prepare(ctypes.byref(p), FAKE, FAKE, None, FAKE, need, None) == fa.FA_EINVAL
    assert lib.fa_bwd_prepare(ctypes.byref(p), FAKE, None, FAKE, FAKE, need, None) == fa.FA_EINVAL
    assert "lse" in lib.fa_last_error().decode()
    assert lib.fa_bwd_prepare(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, need - 4, None) == fa.FA_EINVAL
    assert lib.fa_bwd_dkdv(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           MISALIGNED, FAKE, need, None) == fa.FA_EINVAL
    assert "dv" in lib.fa_last_error().decode()
    assert lib.fa_bwd_dq(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need,
                         None) == fa.FA_EINVAL
    assert "dq is NULL" in lib.fa_last_error().decode()
    bad = _p(d=80)
    assert lib.fa_bwd_dq(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                         None) == fa.FA_EUNSUPPORTED
