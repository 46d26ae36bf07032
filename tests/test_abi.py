"""The C-ABI library loads, exports what include/flash_attn.h declares, and
rejects invalid calls with the documented status codes before any HIP call.

CPU only: no call here reaches a kernel launch (every case fails validation
or is an empty problem), so no GPU is needed.
"""
import ctypes
import os
import re

import pytest

from io_aware_exact_flash_amd import flash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")

FAKE = 0x10000        # 16-byte aligned, never dereferenced: validation fails first
FAKE_MISALIGNED = 0x10008


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flash_attn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("flash_attn_fwd", "flash_attn_bwd", "flash_attn_blocksparse_fwd",
                     "flash_attn_blocksparse_bwd", "flash_attn_bwd_workspace_size",
                     "flash_attn_fwd_splitkv", "flash_attn_fwd_splitkv_workspace_size",
                     "flash_attn_fwd_gqa", "flash_attn_bwd_gqa", "flash_attn_varlen_fwd",
                     "flash_attn_varlen_bwd", "flash_attn_varlen_bwd_workspace_size",
                     "flash_attn_fwd_dropout", "flash_attn_bwd_dropout", "flash_attn_varlen_fwd_dropout",
                     "flash_attn_varlen_bwd_dropout", "flash_attn_fwd_kvcache", "flash_attn_bwd_noalloc"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = flash.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in flash.SIGNATURES, f"binding lacks a signature for {name}"


def test_abi_version_and_status_strings():
    lib = flash.lib()
    assert lib.flash_attn_abi_version() == 1
    for code, name in enumerate(["FA_OK", "FA_ERR_INVALID_ARGUMENT", "FA_ERR_UNSUPPORTED",
                                 "FA_ERR_WORKSPACE_TOO_SMALL", "FA_ERR_HIP"]):
        assert flash.status_string(code) == name


def _fwd(**kw):
    a = dict(B=1, H=1, N=256, d=64, dt=flash.FA_BF16, q=FAKE, k=FAKE, v=FAKE, scale=0.125,
             causal=0, o=FAKE, lse=FAKE, stream=None)
    a.update(kw)
    return flash.lib().flash_attn_fwd(a["B"], a["H"], a["N"], a["d"], a["dt"], a["q"], a["k"], a["v"],
                                      a["scale"], a["causal"], a["o"], a["lse"], a["stream"])


def _bwd(ws_bytes=None, **kw):
    a = dict(B=1, H=2, N=256, d=128, dt=flash.FA_F16, scale=0.1, causal=1)
    a.update(kw)
    need = flash.lib().flash_attn_bwd_workspace_size(a["B"], a["H"], a["N"], a["d"], a["dt"])
    ptr = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE)
    ptr.update({k: v for k, v in kw.items() if k in ptr})
    return flash.lib().flash_attn_bwd(a["B"], a["H"], a["N"], a["d"], a["dt"], ptr["q"], ptr["k"],
                                      ptr["v"], ptr["o"], ptr["do"], ptr["lse"], a["scale"], a["causal"],
                                      ptr["dq"], ptr["dk"], ptr["dv"], ptr["ws"],
                                      need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), flash.FA_ERR_UNSUPPORTED),
    (dict(d=32), flash.FA_ERR_UNSUPPORTED),
    (dict(B=-1), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(N=-5), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(dt=7), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=-1.0), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(causal=2), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(q=None), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(lse=None), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(v=FAKE_MISALIGNED), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(B=1 << 20, H=1 << 10, N=1 << 12), flash.FA_ERR_UNSUPPORTED),
])
def test_forward_validation(kw, code):
    assert _fwd(**kw) == code
    assert flash.lib().flash_attn_last_error().decode().startswith("flash_attn_fwd:")


def test_forward_empty_problem_is_ok_without_launch():
    assert _fwd(B=0, q=None, k=None, v=None, o=None, lse=None) == flash.FA_OK
    assert _fwd(N=0, q=None, k=None, v=None, o=None, lse=None) == flash.FA_OK
    # validation of scalars still applies to empty problems
    assert _fwd(N=0, d=80) == flash.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(dt=flash.FA_F32), flash.FA_ERR_UNSUPPORTED),
    (dict(d=256), flash.FA_ERR_UNSUPPORTED),
    (dict(do=None), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(ws=None), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(dk=FAKE_MISALIGNED), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(causal=-1), flash.FA_ERR_INVALID_ARGUMENT),
])
def test_backward_validation(kw, code):
    assert _bwd(**kw) == code


def test_backward_workspace_too_small():
    lib = flash.lib()
    need = lib.flash_attn_bwd_workspace_size(1, 2, 256, 128, flash.FA_F16)
    # two float32 arrays of B*H*N rows, each rounded to 256 bytes plus 256 spare
    assert need == 2 * (2 * 256 * 4 + 256)
    assert _bwd(ws_bytes=need - 1) == flash.FA_ERR_WORKSPACE_TOO_SMALL
    assert lib.flash_attn_bwd_workspace_size(0, 2, 256, 128, flash.FA_F16) == 0
    assert lib.flash_attn_bwd_workspace_size(1, 1, 1000, 64, flash.FA_BF16) == 2 * (4096 + 256)


def test_blocksparse_validation():
    lib = flash.lib()
    args = (1, 1, 256, 64, flash.FA_F16, FAKE, FAKE, FAKE, 0.125, 0)
    assert lib.flash_attn_blocksparse_fwd(*args, None, 128, FAKE, FAKE, None) == flash.FA_ERR_INVALID_ARGUMENT
    assert lib.flash_attn_blocksparse_fwd(*args, FAKE, 64, FAKE, FAKE, None) == flash.FA_ERR_UNSUPPORTED
    bargs = (1, 1, 256, 64, flash.FA_F16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, 0)
    assert lib.flash_attn_blocksparse_bwd(*bargs, FAKE, 256, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                                          None) == flash.FA_ERR_UNSUPPORTED
    assert lib.flash_attn_blocksparse_bwd(*bargs, None, 128, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                                          None) == flash.FA_ERR_INVALID_ARGUMENT


def _split(ws_bytes=None, **kw):
    a = dict(B=1, H=2, N=300, d=128, dt=flash.FA_BF16, scale=0.1, causal=1, splits=3)
    a.update(kw)
    need = flash.lib().flash_attn_fwd_splitkv_workspace_size(a["B"], a["H"], a["N"], a["d"], a["dt"],
                                                             a["splits"])
    ptr = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=FAKE)
    ptr.update({k: v for k, v in kw.items() if k in ptr})
    return flash.lib().flash_attn_fwd_splitkv(a["B"], a["H"], a["N"], a["d"], a["dt"], ptr["q"], ptr["k"],
                                              ptr["v"], a["scale"], a["causal"], a["splits"], ptr["o"],
                                              ptr["lse"], ptr["ws"], need if ws_bytes is None else ws_bytes,
                                              None)


@pytest.mark.parametrize("kw,code", [
    (dict(splits=0, ws_bytes=1 << 20), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(splits=65, ws_bytes=1 << 30), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(dt=flash.FA_F32), flash.FA_ERR_UNSUPPORTED),
    (dict(d=80, ws_bytes=1 << 20), flash.FA_ERR_UNSUPPORTED),
    (dict(ws=None), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(o=FAKE_MISALIGNED), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), flash.FA_ERR_INVALID_ARGUMENT),
])
def test_splitkv_validation(kw, code):
    assert _split(**kw) == code
    assert flash.lib().flash_attn_last_error().decode().startswith("flash_attn_fwd_splitkv:")


def test_splitkv_workspace_size_and_too_small():
    lib = flash.lib()
    # 3 float32 partial outputs [B*H][N][d] (rounded to 256 bytes), then 3 partial LSE [B*H][N]
    po = 3 * 2 * 300 * 128 * 4
    assert lib.flash_attn_fwd_splitkv_workspace_size(1, 2, 300, 128, flash.FA_BF16, 3) == \
        ((po + 255) // 256) * 256 + 3 * 2 * 300 * 4
    assert lib.flash_attn_fwd_splitkv_workspace_size(1, 2, 0, 128, flash.FA_BF16, 3) == 0
    assert lib.flash_attn_fwd_splitkv_workspace_size(1, 2, 300, 128, flash.FA_BF16, 0) == 0
    need = lib.flash_attn_fwd_splitkv_workspace_size(1, 2, 300, 128, flash.FA_BF16, 3)
    assert _split(ws_bytes=need - 1) == flash.FA_ERR_WORKSPACE_TOO_SMALL
    # empty problems succeed without a launch
    assert _split(N=0, q=None, k=None, v=None, o=None, lse=None, ws=None, ws_bytes=0) == flash.FA_OK


def _gqa_fwd(H, Hkv, **kw):
    a = dict(B=1, N=256, d=64, dt=flash.FA_BF16, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE)
    a.update(kw)
    return flash.lib().flash_attn_fwd_gqa(a["B"], H, Hkv, a["N"], a["d"], a["dt"], a["q"], a["k"], a["v"],
                                          0.125, 1, a["o"], a["lse"], None)


def _gqa_bwd(H, Hkv, **kw):
    a = dict(B=1, N=256, d=128, dt=flash.FA_BF16)
    a.update(kw)
    need = flash.lib().flash_attn_bwd_gqa_workspace_size(a["B"], H, max(Hkv, 1), a["N"], a["d"], a["dt"])
    p = [FAKE] * 9
    if kw.get("null_dk"):
        p[7] = None
    return flash.lib().flash_attn_bwd_gqa(a["B"], H, Hkv, a["N"], a["d"], a["dt"], *p[:6], 0.125, 0,
                                          *p[6:], FAKE, need, None)


@pytest.mark.parametrize("H,Hkv", [(4, 3), (4, 0), (4, -1), (4, 8), (0, 1)])
def test_gqa_head_validation(H, Hkv):
    # Hkv must divide H (and be 0 exactly when H is): checked before any launch
    assert _gqa_fwd(H, Hkv) == flash.FA_ERR_INVALID_ARGUMENT
    assert flash.lib().flash_attn_last_error().decode().startswith("flash_attn_fwd_gqa:")
    assert _gqa_bwd(H, Hkv) == flash.FA_ERR_INVALID_ARGUMENT
    assert flash.lib().flash_attn_last_error().decode().startswith("flash_attn_bwd_gqa:")


def test_gqa_workspace_size():
    lib = flash.lib()
    base = lambda B, H, N: lib.flash_attn_bwd_workspace_size(B, H, N, 128, flash.FA_BF16)
    r256 = lambda b: (b + 255) // 256 * 256
    # one K/V head per query head, or enough (K/V head, 128-key block) units: no partials
    assert lib.flash_attn_bwd_gqa_workspace_size(2, 8, 8, 1000, 128, flash.FA_BF16) == base(2, 8, 1000)
    assert lib.flash_attn_bwd_gqa_workspace_size(8, 128, 64, 200, 128, flash.FA_BF16) == base(8, 128, 200)
    # 2 units, group of 4 heads: 4 ranges, float32 partial dK and dV [4][B*Hkv][N][d] each
    assert lib.flash_attn_bwd_gqa_workspace_size(1, 4, 1, 200, 128, flash.FA_BF16) == \
        base(1, 4, 200) + 2 * r256(4 * 1 * 200 * 128 * 4)
    # 256 units, group of 8: ceil(1024 / 256) = 4 ranges of two heads
    assert lib.flash_attn_bwd_gqa_workspace_size(8, 256, 32, 128, 64, flash.FA_BF16) == \
        lib.flash_attn_bwd_workspace_size(8, 256, 128, 64, flash.FA_BF16) + 2 * r256(4 * 256 * 128 * 64 * 4)
    for args in ((1, 4, 3, 200, 128), (1, 4, 0, 200, 128), (0, 4, 2, 200, 128), (1, 4, 2, 0, 128),
                 (1, 4, 2, 200, 96)):
        assert lib.flash_attn_bwd_gqa_workspace_size(*args, flash.FA_BF16) == 0


def test_gqa_other_checks_and_empty_problems():
    assert _gqa_fwd(4, 2, d=96) == flash.FA_ERR_UNSUPPORTED
    assert _gqa_bwd(4, 2, dt=flash.FA_F32) == flash.FA_ERR_UNSUPPORTED
    assert _gqa_bwd(4, 1, null_dk=True) == flash.FA_ERR_INVALID_ARGUMENT
    # the plain backward workspace is too small once partial sums are needed
    small = flash.lib().flash_attn_bwd_workspace_size(1, 4, 256, 128, flash.FA_BF16)
    assert flash.lib().flash_attn_bwd_gqa(1, 4, 1, 256, 128, flash.FA_BF16, *[FAKE] * 6, 0.125, 0,
                                          *[FAKE] * 4, small, None) == flash.FA_ERR_WORKSPACE_TOO_SMALL
    assert _gqa_fwd(4, 2, v=FAKE_MISALIGNED) == flash.FA_ERR_INVALID_ARGUMENT
    assert _gqa_fwd(0, 0, q=None, k=None, v=None, o=None, lse=None) == flash.FA_OK
    assert _gqa_fwd(4, 2, N=0, q=None, k=None, v=None, o=None, lse=None) == flash.FA_OK


def _vl_fwd(B=2, H=4, Hkv=2, total=500, max_seqlen=300, d=64, dt=flash.FA_BF16, cu=FAKE, **kw):
    p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE)
    p.update(kw)
    return flash.lib().flash_attn_varlen_fwd(B, H, Hkv, total, max_seqlen, d, dt, cu, p["q"], p["k"], p["v"],
                                             0.125, 1, p["o"], p["lse"], None)


def _vl_bwd(B=2, H=4, Hkv=2, total=500, max_seqlen=300, d=64, dt=flash.FA_BF16, cu=FAKE, ws_bytes=None):
    need = flash.lib().flash_attn_varlen_bwd_workspace_size(B, H, max(Hkv, 1), total, max_seqlen, d, dt)
    return flash.lib().flash_attn_varlen_bwd(B, H, Hkv, total, max_seqlen, d, dt, cu, *[FAKE] * 6, 0.125, 0,
                                             *[FAKE] * 4, need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(cu=FAKE + 2), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(total=-1), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(max_seqlen=-3), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(Hkv=3), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(H=1 << 16, Hkv=1 << 16, d=128), flash.FA_ERR_UNSUPPORTED),
    (dict(d=80), flash.FA_ERR_UNSUPPORTED),
])
def test_varlen_validation(kw, code):
    assert _vl_fwd(**kw) == code
    assert flash.lib().flash_attn_last_error().decode().startswith("flash_attn_varlen_fwd:")
    assert _vl_bwd(**kw) == code
    assert flash.lib().flash_attn_last_error().decode().startswith("flash_attn_varlen_bwd:")


def test_varlen_workspace_and_empty():
    lib = flash.lib()
    r256 = lambda b: (b + 255) // 256 * 256
    # per-row arrays of H*total rows (two, each + 256 spare bytes); 2 sequences x 1 K/V head x
    # ceil(300/128) = 6 units, group of 4: 4 ranges of float32 partials [4][B*Hkv][300][64]
    assert lib.flash_attn_varlen_bwd_workspace_size(2, 4, 1, 500, 300, 64, flash.FA_BF16) == \
        2 * (r256(4 * 500 * 4) + 256) + 2 * r256(4 * 2 * 300 * 64 * 4)
    assert lib.flash_attn_varlen_bwd_workspace_size(2, 4, 4, 500, 300, 64, flash.FA_BF16) == \
        2 * (r256(4 * 500 * 4) + 256)
    assert lib.flash_attn_varlen_bwd_workspace_size(2, 4, 4, 0, 300, 64, flash.FA_BF16) == 0
    assert _vl_bwd(Hkv=1, ws_bytes=2 * (r256(4 * 500 * 4) + 256)) == flash.FA_ERR_WORKSPACE_TOO_SMALL
    assert _vl_bwd(dt=flash.FA_F32) == flash.FA_ERR_UNSUPPORTED
    # empty batches launch nothing
    assert _vl_fwd(total=0, q=None, k=None, v=None, o=None, lse=None) == flash.FA_OK
    assert _vl_fwd(B=0, cu=None, total=0, max_seqlen=0, q=None, k=None, v=None, o=None, lse=None) == flash.FA_OK


@pytest.mark.parametrize("p,code", [(-0.1, flash.FA_ERR_INVALID_ARGUMENT), (1.0, flash.FA_ERR_INVALID_ARGUMENT),
                                    (0.999, flash.FA_ERR_INVALID_ARGUMENT), (float("nan"), flash.FA_ERR_INVALID_ARGUMENT)])
def test_dropout_validation(p, code):
    lib = flash.lib()
    assert lib.flash_attn_fwd_dropout(1, 2, 256, 64, flash.FA_BF16, FAKE, FAKE, FAKE, 0.125, 0, p, 1, 0, FAKE, FAKE,
                                      None) == code
    assert lib.flash_attn_last_error().decode().startswith("flash_attn_fwd_dropout:")
    need = lib.flash_attn_bwd_workspace_size(1, 2, 256, 64, flash.FA_BF16)
    assert lib.flash_attn_bwd_dropout(1, 2, 256, 64, flash.FA_BF16, *[FAKE] * 6, 0.125, 0, p, 1, 0, *[FAKE] * 3,
                                      FAKE, need, None) == code


def test_dropout_other_checks():
    lib = flash.lib()
    assert lib.flash_attn_fwd_dropout(1, 2, 256, 64, flash.FA_F32, FAKE, FAKE, FAKE, 0.125, 0, 0.1, 1, 0, FAKE,
                                      FAKE, None) == flash.FA_ERR_UNSUPPORTED
    assert lib.flash_attn_fwd_dropout(1, 2, 256, 96, flash.FA_BF16, FAKE, FAKE, FAKE, 0.125, 0, 0.1, 1, 0, FAKE,
                                      FAKE, None) == flash.FA_ERR_UNSUPPORTED
    assert lib.flash_attn_fwd_dropout(0, 2, 256, 64, flash.FA_BF16, None, None, None, 0.125, 0, 0.1, 1, 0, None,
                                      None, None) == flash.FA_OK


def test_splitkv_num_splits_heuristic():
    ns = flash.lib().flash_attn_fwd_splitkv_num_splits
    assert ns(1, 8, 8192, 128, 1) == 2      # 32 row blocks x 8 heads = 256 split-mode workgroups
    assert ns(4, 40, 8192, 128, 1) == 1     # the plain forward already has 2560 workgroups
    assert ns(1, 1, 512, 64, 0) == 2        # 16 key tiles: at most two ranges of eight
    assert ns(1, 1, 100, 64, 0) == 1
    assert ns(1, 1, 16384, 128, 1) == 8     # 64 row blocks: 8 ranges make 512 workgroups
    assert ns(0, 8, 8192, 128, 1) == 1


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        flash.fwd(q, q, q)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(flash, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(flash, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        flash.lib()


def _kv(**kw):
    a = dict(B=2, H=4, Hkv=2, Nq=1, Nk=100, d=128, dt=flash.FA_BF16, q=FAKE, k=FAKE, v=FAKE, lens=None,
             scale=0.1, causal=1, splits=1, o=FAKE, lse=FAKE, ws=None, wsb=0)
    a.update(kw)
    return flash.lib().flash_attn_fwd_kvcache(a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["dt"], a["q"],
                                              a["k"], a["v"], a["lens"], a["scale"], a["causal"], a["splits"],
                                              a["o"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), flash.FA_ERR_UNSUPPORTED),
    (dict(dt=flash.FA_F32), flash.FA_ERR_UNSUPPORTED),
    (dict(H=3), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(Nq=-1), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(splits=0), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(splits=65), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(causal=2), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(q=0), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(k=FAKE_MISALIGNED), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(lens=FAKE + 2), flash.FA_ERR_INVALID_ARGUMENT),
    (dict(splits=4), flash.FA_ERR_INVALID_ARGUMENT),          # workspace needed, none given
    (dict(splits=4, ws=FAKE, wsb=16), flash.FA_ERR_WORKSPACE_TOO_SMALL),
])
def test_kvcache_validation(kw, code):
    assert _kv(**kw) == code


def test_kvcache_workspace_size_and_splits():
    lib = flash.lib()
    assert lib.flash_attn_fwd_kvcache_workspace_size(2, 4, 2, 1, 100, 128, flash.FA_BF16, 1) == 0
    rows = 2 * 4 * 3
    got = lib.flash_attn_fwd_kvcache_workspace_size(2, 4, 2, 3, 100, 128, flash.FA_BF16, 5)
    assert got == ((5 * rows * 128 * 4 + 255) // 256) * 256 + 5 * rows * 4
    # long caches with few K/V heads are split, at most 64 ways; short ones are not
    assert lib.flash_attn_fwd_kvcache_num_splits(1, 8, 1, 1, 32768, 128) == 64
    assert lib.flash_attn_fwd_kvcache_num_splits(1, 8, 1, 1, 100, 128) == 1
    assert lib.flash_attn_fwd_kvcache_num_splits(64, 64, 64, 1, 4096, 128) == 1
    assert lib.flash_attn_fwd_kvcache_num_splits(0, 8, 1, 1, 100, 128) == 1


def test_kvcache_empty_problem_is_ok_without_launch():
    assert _kv(Nq=0, q=0, o=0, lse=0) == flash.FA_OK
    assert _kv(B=0, q=0, k=0, v=0, o=0, lse=0) == flash.FA_OK
