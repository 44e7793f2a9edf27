"""The C-ABI library on the host: it loads, exports what include/fa.h
declares, validates arguments before any HIP call, and allocates nothing."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from exact_io_aware_07_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

A = 0x100000  # a 16-byte aligned stand-in address: never dereferenced on these paths


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_exported_entry_points():
    assert _declared() == sorted(fa.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    L = fa.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (fa_\w+)", out))
    assert set(_declared()) <= exported


def test_library_imports_no_device_allocator():
    out = subprocess.run(["nm", "-D", "--undefined-only", fa.LIB], capture_output=True, text=True).stdout
    for sym in ("hipMalloc", "hipMallocAsync", "hipMallocManaged", "hipExtMallocWithFlags",
                "hipFree", "hipFreeAsync", "hipHostMalloc", "hipMemcpy"):
        assert not re.search(rf"\b{sym}\b", out), sym


def test_strerror_covers_every_status():
    for st in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_WORKSPACE, fa.FA_ERR_HIP,
               fa.FA_ERR_TOO_LARGE):
        assert fa.fa_strerror(st).startswith("FA_")
    assert "unknown" in fa.fa_strerror(12345)


def _fwd(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=16, d=64, scale=0.125, causal=0, kv=None,
         it=fa.FA_BF16, ot=fa.FA_BF16):
    return fa.lib().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, kv, None, it, ot)


def _bwd(ws=A, ws_bytes=1 << 20, B=1, H=1, N=16, d=64, scale=0.125, causal=0, dtype=fa.FA_BF16,
         q=A, dq=A, ot=None):
    return fa.lib().fa_bwd(q, A, A, A, A, A, dq, A, A, B, H, N, d, scale, causal, None, ws,
                           ws_bytes, None, dtype, dtype if ot is None else ot)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=A + 8), fa.FA_ERR_INVALID_ARG),          # misaligned
    (dict(lse=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(kv=A + 1), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=-5), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(it=7), fa.FA_ERR_UNSUPPORTED),
    (dict(it=fa.FA_BF16, ot=fa.FA_F16), fa.FA_ERR_UNSUPPORTED),
    (dict(it=fa.FA_F32, ot=fa.FA_BF16), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 20, H=1 << 10, N=1 << 20), fa.FA_ERR_INVALID_ARG),  # grid too large
])
def test_forward_validation(kw, expect):
    assert _fwd(**kw) == expect


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_empty_forward_and_backward_are_ok_without_pointers(kw):
    assert _fwd(q=None, k=None, v=None, o=None, lse=None, **kw) == fa.FA_OK
    assert _bwd(ws=None, ws_bytes=0, q=None, dq=None, **kw) == fa.FA_OK


@pytest.mark.parametrize("kw,expect", [
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=16 * 4 - 1), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 4), fa.FA_ERR_WORKSPACE),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(dq=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(d=48), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_UNSUPPORTED),
    (dict(causal=-1), fa.FA_ERR_INVALID_ARG),
    (dict(ot=fa.FA_F16), fa.FA_ERR_UNSUPPORTED),                   # O neither bf16 nor fp32
    (dict(dtype=fa.FA_F32, ot=fa.FA_BF16), fa.FA_ERR_UNSUPPORTED),
    (dict(ot=fa.FA_F32, ws=None), fa.FA_ERR_WORKSPACE),            # fp32 O accepted, then checks go on
])
def test_backward_validation(kw, expect):
    assert _bwd(**kw) == expect


def test_workspace_size_is_one_float_per_row():
    assert fa.fa_bwd_workspace_bytes(8, 12, 1024, 64) == 8 * 12 * 1024 * 4
    assert fa.fa_bwd_workspace_bytes(-1, 1, 1, 64) == 0


def test_binding_rejects_host_tensors_instead_of_computing():
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError, match="device tensor"):
        fa.fa_fwd(x, x, x, x, lse, 0.125)


def test_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "exact_io_aware_07_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "attn_fwd64" not in text and "attn_bwd64" not in text, f


def test_stage_entry_points_validate_before_launch():
    L = fa.lib()
    bf = fa.FA_BF16
    assert L.fa_bwd_dsum(None, A, A, 1, 1, 16, 64, None, bf, bf) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_dsum(A, A, A + 2, 1, 1, 16, 64, None, bf, bf) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_dsum(A, A, A, 1, 1, 16, 80, None, bf, bf) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_bwd_dsum(A, A, A, 1, 1, 16, 64, None, bf, fa.FA_F16) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_bwd_dsum(None, None, None, 0, 1, 16, 64, None, bf, bf) == fa.FA_OK
    assert L.fa_bwd_dsum(None, None, None, 0, 1, 16, 64, None, bf, fa.FA_F32) == fa.FA_OK
    assert L.fa_bwd_dkdv(A, A, A, A, A, None, A, A, 1, 1, 16, 64, 0.125, 0, None, None,
                         fa.FA_BF16) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_dkdv(A, A, A, A, A, A, A, A, 1, 1, 16, 64, 0.125, 3, None, None,
                         fa.FA_BF16) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_dq(A, A, A, A, A, A, A, None, 1, 1, 16, 64, 0.125, 0, None, None,
                       bf, bf) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_dq(A, A, A, None, A, A, A, A, 1, 1, 16, 64, 0.125, 0, None, None,
                       bf, fa.FA_F32) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_dq(A, A, A, A, A, A, A + 2, A, 1, 1, 16, 64, 0.125, 0, None, None,
                       bf, bf) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_dq(A, A, A, A, A, A, A, A, 1, 1, 16, 64, 0.125, 0, None, None, 9, 9) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_bwd_dq(A, A, A, A, A, A, A, A, 1, 1, 16, 64, 0.125, 0, None, None, bf,
                       fa.FA_F16) == fa.FA_ERR_UNSUPPORTED


def test_sequence_longer_than_a_32_bit_head_is_unsupported():
    assert _fwd(N=4194304, d=128) == fa.FA_ERR_UNSUPPORTED
    assert _fwd(N=8388608, d=64) == fa.FA_ERR_UNSUPPORTED


def _part(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, Nq=16, Nk=16, d=64, scale=0.125, causal=0,
          qp=0, kp=0, kv=None, it=fa.FA_BF16):
    return fa.lib().fa_fwd_partial(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, qp, kp, kv,
                                   None, it)


@pytest.mark.parametrize("kw,expect", [
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(it=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=-1), fa.FA_ERR_INVALID_ARG),
    (dict(qp=1 << 29), fa.FA_ERR_INVALID_ARG),
    (dict(kp=-(1 << 29)), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=A + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lse=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=(1 << 31) // 256), fa.FA_ERR_UNSUPPORTED),
])
def test_partial_validation(kw, expect):
    assert _part(**kw) == expect


def test_empty_partial_is_ok_without_pointers():
    assert _part(q=None, k=None, v=None, o=None, lse=None, Nq=0) == fa.FA_OK


def _merge(oa=A, la=A, ob=A, lb=A, o=A, lse=A, rows=16, d=64, ot=fa.FA_F32):
    return fa.lib().fa_merge(oa, la, ob, lb, o, lse, rows, d, None, ot)


@pytest.mark.parametrize("kw,expect", [
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(ot=7), fa.FA_ERR_UNSUPPORTED),
    (dict(rows=-1), fa.FA_ERR_INVALID_ARG),
    (dict(ob=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=A + 4), fa.FA_ERR_INVALID_ARG),
    (dict(lb=A + 1), fa.FA_ERR_INVALID_ARG),
])
def test_merge_validation(kw, expect):
    assert _merge(**kw) == expect


def test_empty_merge_is_ok_without_pointers():
    assert _merge(oa=None, la=None, ob=None, lb=None, o=None, lse=None, rows=0) == fa.FA_OK


def _split(ws=A, ws_bytes=1 << 30, B=1, H=1, N=1000, d=64, splits=4, it=fa.FA_BF16,
           ot=fa.FA_BF16, o=A):
    return fa.lib().fa_fwd_split(A, A, A, o, A, B, H, N, d, 0.125, 0, None, splits, ws,
                                 ws_bytes, None, it, ot)


def test_split_workspace_counts_every_part():
    # N = 1000 in 4 parts: runs of ceil(1000 / 4) = 250 keys, rounded up to
    # 256, need 4 parts; each part keeps d + 1 fp32 per query row
    assert fa.fa_fwd_split_workspace_bytes(2, 3, 1000, 64, 4) == 4 * 2 * 3 * 1000 * 65 * 4
    # N = 100 in 4 parts: runs of 64 keys cover it in 2 parts
    assert fa.fa_fwd_split_workspace_bytes(1, 1, 100, 128, 4) == 2 * 100 * 129 * 4
    # one part (or N <= 64) runs the plain forward and needs none
    assert fa.fa_fwd_split_workspace_bytes(1, 1, 1000, 64, 1) == 0
    assert fa.fa_fwd_split_workspace_bytes(1, 1, 64, 64, 8) == 0
    assert fa.fa_fwd_split_workspace_bytes(1, 1, 1000, 64, 0) == 0
    assert fa.fa_fwd_split_workspace_bytes(1, 1, 1000, 64, 17) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(splits=0), fa.FA_ERR_INVALID_ARG),
    (dict(splits=17), fa.FA_ERR_INVALID_ARG),
    (dict(it=fa.FA_F32, ot=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(ot=fa.FA_F16), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 8), fa.FA_ERR_WORKSPACE),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
])
def test_split_validation(kw, expect):
    assert _split(**kw) == expect


def test_partial_without_keys_needs_no_key_pointers():
    # validation only: a null k / v is accepted when Nk == 0 and rejected otherwise
    assert _part(k=None, v=None, Nk=5) == fa.FA_ERR_INVALID_ARG
    assert _part(k=A + 8, Nk=5) == fa.FA_ERR_INVALID_ARG


def _fwd_gqa(q=A, k=A, v=A, o=A, lse=A, B=1, H=4, Hkv=2, N=16, d=64, scale=0.125, causal=0,
             kv=None, it=fa.FA_BF16, ot=fa.FA_BF16):
    return fa.lib().fa_fwd_gqa(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, kv, None, it, ot)


def _bwd_gqa(ws=A, ws_bytes=1 << 20, B=1, H=4, Hkv=2, N=16, d=64, scale=0.125, causal=0,
             dtype=fa.FA_BF16, dk=A):
    return fa.lib().fa_bwd_gqa(A, A, A, A, A, A, A, dk, A, B, H, Hkv, N, d, scale, causal, None,
                               ws, ws_bytes, None, dtype, dtype)


@pytest.mark.parametrize("kw,expect", [
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=-2), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),           # 4 query heads do not split into 3 groups
    (dict(H=4, Hkv=8), fa.FA_ERR_INVALID_ARG),      # more K/V heads than query heads
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=A + 4), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(it=fa.FA_F32, ot=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(it=fa.FA_BF16, ot=fa.FA_F16), fa.FA_ERR_UNSUPPORTED),
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
])
def test_gqa_forward_validation(kw, expect):
    assert _fwd_gqa(**kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),
    (dict(dk=None), fa.FA_ERR_INVALID_ARG),
    (dict(dk=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=4 * 4 * 16 - 1), fa.FA_ERR_WORKSPACE),  # below D for every query row
])
def test_gqa_backward_validation(kw, expect):
    assert _bwd_gqa(**kw) == expect


def test_gqa_empty_calls_are_ok_without_pointers():
    L = fa.lib()
    assert L.fa_fwd_gqa(None, None, None, None, None, 1, 4, 2, 0, 64, 0.125, 0, None, None,
                        fa.FA_BF16, fa.FA_BF16) == fa.FA_OK
    assert L.fa_bwd_gqa(None, None, None, None, None, None, None, None, None, 0, 4, 2, 16, 64,
                        0.125, 0, None, None, 0, None, fa.FA_BF16, fa.FA_BF16) == fa.FA_OK
    # the head counts are checked even when there is nothing to compute
    assert L.fa_fwd_gqa(None, None, None, None, None, 1, 4, 3, 0, 64, 0.125, 0, None, None,
                        fa.FA_BF16, fa.FA_BF16) == fa.FA_ERR_INVALID_ARG


def test_gqa_workspace_sizes():
    ws = fa.fa_bwd_gqa_workspace_bytes
    # enough K/V heads to fill the chip: D for every query row only
    assert ws(64, 32, 8, 4096, 128) == 64 * 32 * 4096 * 4
    # one K/V head (multi-query): the group is shared among workgroups, whose
    # fp32 partial dK and dV follow D (rounded up to 256 bytes)
    B, H, Hkv, N, d = 2, 32, 1, 4096, 128
    got = ws(B, H, Hkv, N, d)
    dsum = B * H * N * 4
    part = 2 * B * Hkv * N * d * 4
    assert got > dsum and (got - dsum) % part == 0
    shares = (got - dsum) // part
    assert shares > 1 and H // Hkv % shares == 0
    for bad in ((1, 4, 3, 16, 64), (1, 4, 0, 16, 64), (-1, 4, 2, 16, 64), (1, 4, 2, 16, 96)):
        assert ws(*bad) == 0


def _fwd_sp(q=A, mask=A, B=1, H=2, N=300, d=64, sb=0, sh=9, causal=0, it=fa.FA_BF16, ot=fa.FA_BF16):
    return fa.lib().fa_fwd_sparse(q, A, A, A, A, B, H, N, d, 0.125, causal, None, mask, sb, sh, None,
                                  it, ot)


def _bwd_sp(mask=A, ws=A, ws_bytes=1 << 20, B=1, H=2, N=300, d=64, sb=0, sh=9, dtype=fa.FA_BF16):
    return fa.lib().fa_bwd_sparse(A, A, A, A, A, A, A, A, A, B, H, N, d, 0.125, 0, None, mask, sb,
                                  sh, ws, ws_bytes, None, dtype, dtype)


@pytest.mark.parametrize("kw,expect", [
    (dict(mask=None), fa.FA_ERR_INVALID_ARG),
    (dict(sb=-1), fa.FA_ERR_INVALID_ARG),
    (dict(sh=-9), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(it=fa.FA_F32, ot=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(N=128 * 4096 + 1), fa.FA_ERR_UNSUPPORTED),  # a mask row longer than the LDS list
])
def test_sparse_forward_validation(kw, expect):
    assert _fwd_sp(**kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(mask=None), fa.FA_ERR_INVALID_ARG),
    (dict(sh=-1), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=2 * 300 * 4 - 1), fa.FA_ERR_WORKSPACE),
    (dict(N=128 * 4096 + 1), fa.FA_ERR_UNSUPPORTED),
])
def test_sparse_backward_validation(kw, expect):
    assert _bwd_sp(**kw) == expect


def test_sparse_empty_calls_need_no_pointers():
    L = fa.lib()
    assert L.fa_fwd_sparse(None, None, None, None, None, 0, 2, 300, 64, 0.125, 0, None, None, 0, 0,
                           None, fa.FA_BF16, fa.FA_BF16) == fa.FA_OK
    assert L.fa_bwd_sparse(None, None, None, None, None, None, None, None, None, 1, 2, 0, 64, 0.125,
                           0, None, None, 0, 0, None, 0, None, fa.FA_BF16, fa.FA_F32) == fa.FA_OK


def test_fp8_validation():
    L = fa.lib()
    q = lambda **kw: L.fa_fp8_quantize(*([A] * 11), kw.get("B", 1), 2, 300, kw.get("d", 64), None,
                                       kw.get("it", fa.FA_BF16))
    assert q(d=96) == fa.FA_ERR_UNSUPPORTED
    assert q(it=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert q(B=-1) == fa.FA_ERR_INVALID_ARG
    assert L.fa_fp8_quantize(*([A] * 3), None, None, *([A] * 6), 1, 2, 300, 64, None,
                             fa.FA_BF16) == fa.FA_ERR_INVALID_ARG  # q8 missing
    f = lambda **kw: L.fa_fwd_fp8(*([A] * 6), kw.get("rot", 1), A, A, 1, 2, 300, kw.get("d", 64),
                                  kw.get("scale", 0.125), 0, None, None, kw.get("ot", fa.FA_BF16))
    assert f(rot=2) == fa.FA_ERR_INVALID_ARG
    assert f(scale=0.0) == fa.FA_ERR_INVALID_ARG
    assert f(ot=9) == fa.FA_ERR_UNSUPPORTED
    assert f(d=32) == fa.FA_ERR_UNSUPPORTED
    w = lambda **kw: L.fa_fwd_fp8_incoherent(*([A] * 4), A, A, 1, 2, 300, 64, 0.125, 0, None,
                                             kw.get("ws", A), kw.get("wb", 1 << 30), None,
                                             kw.get("it", fa.FA_BF16), kw.get("ot", fa.FA_BF16))
    assert w(ws=None) == fa.FA_ERR_WORKSPACE
    assert w(wb=fa.fa_fwd_fp8_workspace_bytes(1, 2, 300, 64) - 1) == fa.FA_ERR_WORKSPACE
    assert w(it=fa.FA_BF16, ot=fa.FA_F16) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_fp8_workspace_bytes(1, 2, 300, 96) == 0


def test_fp8_workspace_holds_every_buffer():
    B, H, N, d = 2, 3, 300, 128
    np_ = 320
    need = 2 * B * H * N * d + B * H * d * np_ + 4 * (B * H * 3 + 2 * B * H * 5 + B * H)
    got = fa.fa_fwd_fp8_workspace_bytes(B, H, N, d)
    assert need <= got <= need + 7 * 256


def _plan_counts(mask, B, H, N, causal, columns):
    """Kept blocks per mask line, written out: a column (key block kb) counts
    query blocks from the diagonal on when causal; a row (query block qb)
    counts key blocks up to the diagonal."""
    nb = (N + 127) // 128
    m = mask.expand(B, H, nb, nb) if mask.dim() == 2 else mask
    out = {}
    for b in range(B):
        for h in range(H):
            for x in range(nb):
                if columns:
                    line = m[b, h, (x if causal else 0):, x]
                else:
                    line = m[b, h, x, :(x + 1 if causal else nb)]
                out[(b * H + h, x)] = int((line != 0).sum())
    return out


def _check_pieces(items, lines, counts):
    """Every line once, whole (first 0, slot -1) when it holds at most 8
    kept blocks, else in pieces of 8 with consecutive slots named by its
    cut line; the slots of the cut lines tile [0, total); the items of head
    bh at positions p with p % 8 == bh % 8 (the XCD of workgroup p) until
    that class runs out, longest first within each class."""
    seen = {}
    for bh, x, first, slot in items:
        seen.setdefault((bh, x), []).append((first, slot))
    assert set(seen) == set(counts)
    cut = {(c[0], c[1]): c for c in lines}
    sizes = []
    for key, n in counts.items():
        got = sorted(seen[key])
        if n <= 8:
            assert got == [(0, -1)] and key not in cut
            sizes.append(n)
            continue
        pieces = -(-n // 8)
        _, _, slot0, np_ = cut[key]
        assert np_ == pieces and got == [(8 * i, slot0 + i) for i in range(pieces)]
        sizes += [min(8, n - 8 * i) for i in range(pieces)]
    spans = sorted((c[2], c[3]) for c in lines)
    assert [s for s, _ in spans] == [sum(n for _, n in spans[:i]) for i in range(len(spans))]
    size_of = lambda it: min(8, counts[(it[0], it[1])] - it[2])
    assert sorted(size_of(it) for it in items) == sorted(sizes)
    for x in range(8):
        cls = [size_of(it) for it in items if it[0] % 8 == x]
        assert cls == sorted(cls, reverse=True)
        # a position of class x holds another class's item only after class x ran out
        foreign = [p for p, it in enumerate(items) if p % 8 == x and it[0] % 8 != x]
        if foreign:
            assert all(it[0] % 8 != x for it in items[foreign[0]:])
    return sum(n for _, n in spans)


@pytest.mark.parametrize("causal", [False, True])
def test_sparse_plan_cuts_long_lines_into_pieces_of_eight(causal):
    from exact_io_aware_07_amd import workloads as W
    B, H, N = 2, 3, 128 * 40
    mask = W.random_block_mask((B, H), N, 0.45, seed=7)
    mask[0, 1, :, 3] = 1                      # one full column
    mask[1, 2, :, 5] = 0                      # one empty column
    mask[1, 0, 30, :] = 1                     # one full row
    mask[0, 2, 4, :] = 0                      # one empty row
    plan = fa.fa_sparse_plan(mask, B, H, N, causal)
    c = plan["counts"].tolist()
    assert c[6:] == [0, 0] and len(plan["plan"]) >= 4 * (c[0] + c[1] + c[3] + c[4])
    cols = _check_pieces(plan["col_items"].tolist(), plan["cols"].tolist(),
                         _plan_counts(mask, B, H, N, causal, True))
    rows = _check_pieces(plan["row_items"].tolist(), plan["rows"].tolist(),
                         _plan_counts(mask, B, H, N, causal, False))
    assert (c[2], c[5]) == (cols, rows) and cols > 0 and rows > 0
    assert (c[1], c[4]) == (len(plan["cols"]), len(plan["rows"]))


def test_sparse_plan_of_a_short_mask_cuts_nothing():
    mask = torch.ones(8, 8, dtype=torch.uint8)
    plan = fa.fa_sparse_plan(mask, 2, 3, 1000, False)
    assert plan["counts"].tolist() == [48, 0, 0, 48, 0, 0, 0, 0]


def test_sparse_plan_validation_and_counts_only():
    L = fa.lib()
    counts = (ctypes.c_int * 8)()
    r = lambda *a: L.fa_sparse_plan(*a, counts)
    assert r(None, 0, 0, 1, 1, 300, 0, None, 0) == fa.FA_ERR_INVALID_ARG     # mask missing
    m = (ctypes.c_ubyte * 9)(*([1] * 9))
    assert r(m, 0, 0, 1, 1, 300, 2, None, 0) == fa.FA_ERR_INVALID_ARG        # causal 2
    assert r(m, -1, 0, 1, 1, 300, 0, None, 0) == fa.FA_ERR_INVALID_ARG
    assert L.fa_sparse_plan(m, 0, 0, 1, 1, 300, 0, None, 0, None) == fa.FA_ERR_INVALID_ARG
    assert r(m, 0, 0, 1, 1, 300, 0, None, 0) == fa.FA_OK
    assert list(counts) == [3, 0, 0, 3, 0, 0, 0, 0]
    buf = (ctypes.c_int * 24)()
    assert r(m, 0, 0, 1, 1, 300, 0, buf, 23) == fa.FA_ERR_INVALID_ARG        # 6 items, room for 5.75
    assert r(m, 0, 0, 1, 1, 300, 0, buf, 24) == fa.FA_OK
    assert list(buf) == [0, 0, 0, -1, 0, 1, 0, -1, 0, 2, 0, -1] * 2
    big = (ctypes.c_ubyte * (4097 * 4097))()
    assert r(big, 0, 0, 1, 1, 4097 * 128, 0, None, 0) == fa.FA_ERR_UNSUPPORTED


def test_sparse_planned_workspace_sizes():
    c = [3, 1, 5, 3, 1, 4, 0, 0]
    assert fa.fa_fwd_sparse_planned_workspace_bytes(1, 2, 300, 64, c) == 4 * 128 * 65 * 4
    assert fa.fa_fwd_sparse_planned_workspace_bytes(1, 2, 300, 64, [3, 0, 0, 3, 0, 0, 0, 0]) == 0
    dsum = 2 * 300 * 4
    up = lambda x: (x + 255) // 256 * 256
    assert fa.fa_bwd_sparse_planned_workspace_bytes(1, 2, 300, 128, c) == (
        up(dsum) + up(2 * 5 * 128 * 128 * 4) + 4 * 128 * 128 * 4)
    assert fa.fa_bwd_sparse_planned_workspace_bytes(1, 2, 300, 96, c) == 0


def test_sparse_planned_validation():
    L = fa.lib()
    C = lambda *v: (ctypes.c_int * 8)(*v)
    ok = C(6, 0, 0, 6, 0, 0, 0, 0)               # B=1 H=2 N=300: 6 lines of each kind
    fwd = lambda counts, ws=1 << 20, **kw: L.fa_fwd_sparse_planned(
        A, A, A, A, A, 1, 2, 300, 64, 0.125, 0, None, kw.get("mask", A), 0, 0, kw.get("plan", A),
        counts, A, ws, None, fa.FA_BF16, fa.FA_BF16)
    bwd = lambda counts, ws=1 << 20, **kw: L.fa_bwd_sparse_planned(
        *([A] * 9), 1, 2, 300, 64, 0.125, 0, None, kw.get("mask", A), 0, 0, kw.get("plan", A), counts,
        A, ws, None, fa.FA_BF16, fa.FA_BF16)
    for f in (fwd, bwd):
        assert f(C(5, 0, 0, 6, 0, 0, 0, 0)) == fa.FA_ERR_INVALID_ARG       # too few column items
        assert f(C(6, 0, 0, 5, 0, 0, 0, 0)) == fa.FA_ERR_INVALID_ARG       # too few row items
        assert f(C(7, 1, 0, 6, 0, 0, 0, 0)) == fa.FA_ERR_INVALID_ARG       # cut column without slots
        assert f(C(6, 0, 0, 7, 0, 2, 0, 0)) == fa.FA_ERR_INVALID_ARG       # slots without a cut row
        assert f(C(-1, 0, 0, 6, 0, 0, 0, 0)) == fa.FA_ERR_INVALID_ARG
        assert f(None) == fa.FA_ERR_INVALID_ARG
        assert f(ok, plan=None) == fa.FA_ERR_INVALID_ARG
        assert f(ok, plan=A + 2) == fa.FA_ERR_INVALID_ARG                 # misaligned plan
        assert f(ok, mask=None) == fa.FA_ERR_INVALID_ARG
    assert fwd(C(6, 0, 0, 7, 1, 2, 0, 0), ws=2 * 128 * 65 * 4 - 1) == fa.FA_ERR_WORKSPACE
    assert bwd(ok, ws=0) == fa.FA_ERR_WORKSPACE
    # empty problems need no pointers
    assert L.fa_fwd_sparse_planned(None, None, None, None, None, 0, 2, 300, 64, 0.125, 0, None, None, 0,
                                   0, None, C(0, 0, 0, 0, 0, 0, 0, 0), None, 0, None, fa.FA_BF16,
                                   fa.FA_BF16) == fa.FA_OK
    assert L.fa_bwd_sparse_planned(*([None] * 9), 1, 2, 0, 64, 0.125, 0, None, None, 0, 0, None,
                                   C(0, 0, 0, 0, 0, 0, 0, 0), None, 0, None, fa.FA_BF16,
                                   fa.FA_BF16) == fa.FA_OK


def test_autograd_wrapper_refuses_host_tensors_instead_of_computing():
    from exact_io_aware_07_amd import scaled_dot_product_attention
    q = torch.randn(1, 1, 16, 64, dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(ValueError, match="device tensor"):
        scaled_dot_product_attention(q, q, q)


def _bwd_noalloc(B=1, H=1, N=16, d=64, scale=0.125, causal=0, dtype=fa.FA_BF16, q=A, dq=A, lse=A):
    return fa.lib().fa_bwd_noalloc(q, A, A, A, A, lse, dq, A, A, B, H, N, d, scale, causal, None,
                                   None, dtype, dtype)


def test_noalloc_header_constant_matches_binding():
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_MAX_ROWS \(1 << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == fa.FA_NOALLOC_MAX_ROWS


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(dq=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(lse=A + 1), fa.FA_ERR_INVALID_ARG),
    (dict(d=48), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_UNSUPPORTED),
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    # one row past the built-in scratch: refused before any HIP call
    (dict(B=1, H=1, N=(1 << 22) + 1), fa.FA_ERR_TOO_LARGE),
    (dict(B=4, H=16, N=65537), fa.FA_ERR_TOO_LARGE),
])
def test_noalloc_backward_validation(kw, expect):
    assert _bwd_noalloc(**kw) == expect


def test_noalloc_backward_empty_is_ok_without_pointers():
    assert _bwd_noalloc(N=0, q=None, dq=None, lse=None) == fa.FA_OK
