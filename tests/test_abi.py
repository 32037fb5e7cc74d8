"""The C-ABI library loads, exports every declared symbol and rejects bad arguments (CPU only).

Every call here fails argument validation, which happens before any HIP call,
so nothing is launched and no device is needed.
"""
import re
import subprocess
from pathlib import Path

import pytest

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import _binding

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "fa.h"


@pytest.fixture(scope="module")
def lib():
    if not fa.library_path().exists():
        from exact_attention_forward_amd.build import build

        build()
    return fa.lib()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(_binding.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(fa.library_path())], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_[a-z_]+)\b", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_support_table_and_status_strings(lib):
    for hd in (8, 16, 32, 64, 128):
        assert fa.fa_is_supported(hd, fa.FA_F32) == 1
    for hd in (64, 128):
        assert fa.fa_is_supported(hd, fa.FA_BF16) == 1
        assert fa.fa_is_supported(hd, fa.FA_F16) == 1
    assert fa.fa_is_supported(32, fa.FA_F16) == 0
    for hd, dt in ((4, fa.FA_F32), (96, fa.FA_F32), (32, fa.FA_BF16), (256, fa.FA_BF16), (64, 7)):
        assert fa.fa_is_supported(hd, dt) == 0
    for st in (fa.FA_OK, fa.FA_ERR_ARG, fa.FA_ERR_ALIGN, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_ALIAS, fa.FA_ERR_LAUNCH, 9):
        assert isinstance(fa.fa_status_string(st), str) and fa.fa_status_string(st)


# Fake, never-dereferenced addresses: far apart, 16-byte aligned.
MB = 1 << 20
P = [0x10000000 + i * 256 * MB for i in range(12)]


def fwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, T=8, hd=64, scale=0.125, causal=1,
             dtype=fa.FA_F32, prec=0, stream=None)
    a.update(kw)
    return fa.fa_forward(*a.values())


def bwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], dO=P[5], dq=P[6], dk=P[7], dv=P[8], delta=P[9], B=1, H=2,
             T=8, hd=64, scale=0.125, causal=1, dtype=fa.FA_F32, prec=0, stream=None)
    a.update(kw)
    return fa.fa_backward(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_ARG),
    (dict(lse=None), fa.FA_ERR_ARG),
    (dict(B=0), fa.FA_ERR_ARG),
    (dict(H=-1), fa.FA_ERR_ARG),
    (dict(T=0), fa.FA_ERR_ARG),
    (dict(scale=0.0), fa.FA_ERR_ARG),
    (dict(scale=-0.5), fa.FA_ERR_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_ARG),
    (dict(causal=2), fa.FA_ERR_ARG),
    (dict(dtype=5), fa.FA_ERR_ARG),
    (dict(prec=9), fa.FA_ERR_ARG),
    (dict(B=1 << 20, H=1 << 11, T=1 << 11), fa.FA_ERR_ARG),
    (dict(H=1 << 19, T=32, dtype=fa.FA_BF16), fa.FA_ERR_ARG),  # H * hd = 2^25: row stride over the limit
    (dict(hd=96), fa.FA_ERR_UNSUPPORTED),
    (dict(hd=32, dtype=fa.FA_BF16), fa.FA_ERR_UNSUPPORTED),
    (dict(prec=fa.FA_PREC_BF16X2), fa.FA_ERR_UNSUPPORTED),
    (dict(k=P[1] + 8), fa.FA_ERR_ALIGN),
    (dict(o=P[3] + 4), fa.FA_ERR_ALIGN),
    (dict(o=P[0]), fa.FA_ERR_ALIAS),
    (dict(lse=P[3] + 16), fa.FA_ERR_ALIAS),
    (dict(o=P[2] + 1024), fa.FA_ERR_ALIAS),
])
def test_forward_validation(lib, kw, status):
    assert fwd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(delta=None), fa.FA_ERR_ARG),
    (dict(dO=None), fa.FA_ERR_ARG),
    (dict(T=-3), fa.FA_ERR_ARG),
    (dict(hd=48), fa.FA_ERR_UNSUPPORTED),
    (dict(dv=P[8] + 2), fa.FA_ERR_ALIGN),
    (dict(dq=P[5]), fa.FA_ERR_ALIAS),
    (dict(dk=P[6]), fa.FA_ERR_ALIAS),
    (dict(delta=P[4]), fa.FA_ERR_ALIAS),
    (dict(dv=P[0] + 64), fa.FA_ERR_ALIAS),
])
def test_backward_validation(lib, kw, status):
    assert bwd(**kw) == status


def test_stage_entry_points_validate(lib):
    assert fa.fa_backward_dq_delta(P[0], P[1], P[2], P[3], P[4], P[5], P[6], None, 1, 2, 8, 64, 0.1, 1, fa.FA_F32, 0,
                                   None) == fa.FA_ERR_ARG
    assert fa.fa_backward_dq_delta(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[3], 1, 2, 8, 64, 0.1, 1, fa.FA_F32, 0,
                                   None) == fa.FA_ERR_ALIAS
    assert fa.fa_backward_dq_delta(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], 1, 2, 8, 48, 0.1, 1, fa.FA_F32, 0,
                                   None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_backward_delta(P[3], P[5], None, 1, 2, 8, 64, fa.FA_F32, None) == fa.FA_ERR_ARG
    assert fa.fa_backward_delta(P[3], P[5], P[3], 1, 2, 8, 64, fa.FA_F32, None) == fa.FA_ERR_ALIAS
    assert fa.fa_backward_dq(P[0], P[1], P[2], P[4], P[5], P[9], P[6], 1, 2, 8, 24, 0.1, 1, fa.FA_F32, 0,
                             None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_backward_dq(P[0], P[1], P[2], P[4], P[5], P[9], P[0], 1, 2, 8, 64, 0.1, 1, fa.FA_F32, 0,
                             None) == fa.FA_ERR_ALIAS
    assert fa.fa_backward_dkv(P[0], P[1], P[2], P[4], P[5], P[9], P[7], P[7], 1, 2, 8, 64, 0.1, 1, fa.FA_F32, 0,
                              None) == fa.FA_ERR_ALIAS
    assert fa.fa_backward_dkv(P[0], P[1], P[2], P[4], P[5], P[9], P[7], P[8], 1, 2, 8, 64, 0.1, 0, fa.FA_BF16, 3,
                              None) == fa.FA_ERR_ARG


def test_unfused_and_control_entry_points_validate(lib):
    # float32 only
    assert fa.fa_forward_unfused(P[0], P[1], P[2], P[3], P[4], 1, 2, 8, 64, 0.1, 0, fa.FA_BF16, None) == \
        fa.FA_ERR_UNSUPPORTED
    assert fa.fa_forward_norescale(P[0], P[1], P[2], P[3], P[4], 1, 2, 8, 64, 0.1, 0, fa.FA_BF16, None) == \
        fa.FA_ERR_UNSUPPORTED
    # the score workspace is an output: it may not overlap an input or o
    assert fa.fa_forward_unfused(P[0], P[1], P[2], P[3], P[2], 1, 2, 8, 64, 0.1, 0, fa.FA_F32, None) == fa.FA_ERR_ALIAS
    assert fa.fa_forward_unfused(P[0], P[1], P[2], P[3], P[3] + 64, 1, 2, 8, 64, 0.1, 0, fa.FA_F32, None) == \
        fa.FA_ERR_ALIAS
    assert fa.fa_forward_unfused(P[0], P[1], P[2], P[3], None, 1, 2, 8, 64, 0.1, 0, fa.FA_F32, None) == fa.FA_ERR_ARG
    assert fa.fa_forward_unfused(P[0], P[1], P[2], P[3], P[4] + 4, 1, 2, 8, 64, 0.1, 0, fa.FA_F32, None) == \
        fa.FA_ERR_ALIGN
    assert fa.fa_forward_unfused(P[0], P[1], P[2], P[3], P[4], 1, 1 << 16, 8, 64, 0.1, 0, fa.FA_F32, None) == \
        fa.FA_ERR_ARG  # B * H above 65535
    assert fa.fa_forward_unfused(P[0], P[1], P[2], P[3], P[4], 1, 2, 8, 96, 0.1, 0, fa.FA_F32, None) == \
        fa.FA_ERR_UNSUPPORTED
    assert fa.fa_forward_norescale(P[0], P[1], P[2], P[3], P[4], 1, 2, 8, 64, -1.0, 0, fa.FA_F32, None) == \
        fa.FA_ERR_ARG
    assert fa.fa_forward_norescale(P[0], P[1], P[2], P[0], P[4], 1, 2, 8, 64, 0.1, 0, fa.FA_F32, None) == \
        fa.FA_ERR_ALIAS


def test_auto_splits_validates(lib):
    # argument checks run before the device is asked anything
    q = lambda **kw: fa.fa_forward_auto_splits(*{**dict(B=1, H=1, T=4096, hd=64, causal=1, dtype=fa.FA_BF16,
                                                        prec=0), **kw}.values())
    assert q(B=0) == fa.FA_ERR_ARG
    assert q(T=0) == fa.FA_ERR_ARG
    assert q(hd=48) == fa.FA_ERR_UNSUPPORTED
    assert q(prec=7) == fa.FA_ERR_ARG
    assert q(dtype=fa.FA_F32, prec=fa.FA_PREC_BF16) == fa.FA_ERR_UNSUPPORTED


def test_splitkv_validates(lib):
    args = lambda **kw: {**dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], ws=P[5], B=1, H=2, T=8, hd=64, scale=0.1,
                                causal=1, nsplit=4, dtype=fa.FA_F32, prec=0, stream=None), **kw}
    call = lambda **kw: fa.fa_forward_splitkv(*args(**kw).values())
    assert call(nsplit=0) == fa.FA_ERR_ARG
    assert call(nsplit=65) == fa.FA_ERR_ARG
    assert call(ws=None) == fa.FA_ERR_ARG
    assert call(ws=P[5] + 8) == fa.FA_ERR_ALIGN
    assert call(ws=P[0]) == fa.FA_ERR_ALIAS
    assert call(ws=P[3] + 1024) == fa.FA_ERR_ALIAS
    assert call(H=1 << 16) == fa.FA_ERR_ARG
    assert call(hd=96) == fa.FA_ERR_UNSUPPORTED
    assert call(dtype=fa.FA_BF16, hd=32) == fa.FA_ERR_UNSUPPORTED


def test_half_inputs_validate(lib):
    assert fwd(dtype=fa.FA_F16, hd=32) == fa.FA_ERR_UNSUPPORTED
    assert fwd(dtype=fa.FA_F16, prec=fa.FA_PREC_BF16) == fa.FA_ERR_UNSUPPORTED
    assert fwd(dtype=fa.FA_F16, prec=fa.FA_PREC_BF16X2) == fa.FA_ERR_UNSUPPORTED
    assert fwd(dtype=3) == fa.FA_ERR_ARG
    # half inputs are 2 bytes: o may start right after q's 2-byte extent
    n = 1 * 8 * 2 * 64
    assert fwd(dtype=fa.FA_F16, o=P[0] + 2 * n - 16) == fa.FA_ERR_ALIAS
    assert fa.fa_forward_nomax(P[0], P[1], P[2], P[3], P[4], 1, 2, 8, 64, 0.1, 0, fa.FA_BF16, None) == \
        fa.FA_ERR_UNSUPPORTED
    assert fa.fa_forward_nomax(P[0], P[1], P[2], P[3], None, 1, 2, 8, 64, 0.1, 0, fa.FA_F16, None) == fa.FA_ERR_ARG


def test_static_workspace_backward_validates(lib):
    def nows(**kw):
        a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], dO=P[5], dq=P[6], dk=P[7], dv=P[8], B=1, H=2, T=8,
                 hd=64, scale=0.125, causal=1, dtype=fa.FA_F32, prec=0, stream=None)
        a.update(kw)
        return fa.fa_backward_nows(*a.values())

    assert nows(dq=None) == fa.FA_ERR_ARG
    assert nows(scale=0.0) == fa.FA_ERR_ARG
    assert nows(hd=48) == fa.FA_ERR_UNSUPPORTED
    assert nows(dv=P[8] + 4) == fa.FA_ERR_ALIGN
    assert nows(dk=P[1]) == fa.FA_ERR_ALIAS
    # 2^22 + 1 rows of D do not fit the static workspace (8-wide float32 rows keep the fake buffers apart)
    assert nows(B=1, H=1, T=(1 << 22) + 1, hd=8) == fa.FA_ERR_TOO_LARGE
    assert fa.fa_status_string(fa.FA_ERR_TOO_LARGE) == "problem larger than the library's static workspace"
