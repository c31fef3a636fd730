"""CPU-only checks of the C-ABI library: it loads without a GPU, exports every
function include/fp8w8a8.h declares, rejects bad arguments on the host before
touching the device, and implements the tile-table semantics (nearest M with
ties to the smaller key, null entries, missing or malformed files, the kill
switch)."""
import ctypes
import json
import os
import re
import subprocess
import sys

import pytest

from fp8_w8a8_quantized_token_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8w8a8.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(names) == set(_lib.SIGNATURES)


def test_version_and_padded_rows(lib):
    assert lib.fp8_version() >= 100
    for m, ra, want in [(0, 4, 0), (1, 4, 4), (5, 4, 8), (13, 4, 16), (31, 4, 32), (7, 1, 7)]:
        assert lib.fp8_padded_rows(m, ra) == want
    assert lib.fp8_padded_rows(-1, 4) == -1
    assert lib.fp8_padded_rows(3, 0) == -1


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def _err(lib):
    return lib.fp8_last_error().decode()


def test_quant_argument_errors(lib):
    q = lib.fp8_quant_per_token
    assert q(None, 4, 128, 128, FAKE, 128, FAKE, 1e-10, None) == _lib.FP8_ERR_INVALID
    assert "null" in _err(lib)
    assert q(FAKE, 4, 100, 100, FAKE, 100, FAKE, 1e-10, None) == _lib.FP8_ERR_INVALID
    assert "multiple of 16" in _err(lib)
    assert q(FAKE, 4, 128, 64, FAKE, 128, FAKE, 1e-10, None) == _lib.FP8_ERR_INVALID
    assert q(FAKE, -1, 128, 128, FAKE, 128, FAKE, 1e-10, None) == _lib.FP8_ERR_INVALID
    assert q(ctypes.c_void_p(0x10002), 4, 128, 128, FAKE, 128, FAKE, 1e-10, None) == _lib.FP8_ERR_INVALID
    assert q(FAKE, 4, 128, 128, FAKE, 128, FAKE, -1.0, None) == _lib.FP8_ERR_INVALID
    # M == 0 is a successful no-op even with null pointers
    assert q(None, 0, 128, 128, None, 128, None, 1e-10, None) == _lib.FP8_OK

    g = lib.fp8_quant_per_token_group
    assert g(FAKE, 4, 7168, 7168, 256, 4, FAKE, 7168, FAKE, 1e-10, None) == _lib.FP8_ERR_UNSUPPORTED
    assert "group_size" in _err(lib)
    assert g(FAKE, 4, 7168 + 64, 7232, 128, 4, FAKE, 7232, FAKE, 1e-10, None) == _lib.FP8_ERR_INVALID
    assert "divisible" in _err(lib)
    assert g(FAKE, 4, 7168, 7168, 128, 0, FAKE, 7168, FAKE, 1e-10, None) == _lib.FP8_ERR_INVALID
    assert g(None, 0, 7168, 7168, 128, 4, None, 7168, None, 1e-10, None) == _lib.FP8_OK


def test_quant_variant_argument_errors(lib):
    qe = lib.fp8_quant_per_token_ex
    silu, ue = _lib.QUANT_FUSE_SILU_MUL, _lib.QUANT_SCALE_UE8M0
    assert qe(FAKE, 4, 128, 128, FAKE, 128, FAKE, 1e-10, 4, None) == _lib.FP8_ERR_INVALID
    assert "flags" in _err(lib)
    # SiLU-and-mul reads 2K values per row
    assert qe(FAKE, 4, 128, 128, FAKE, 128, FAKE, 1e-10, silu, None) == _lib.FP8_ERR_INVALID
    assert "leading dimension" in _err(lib)
    assert qe(None, 4, 128, 256, FAKE, 128, FAKE, 1e-10, silu | ue, None) == _lib.FP8_ERR_INVALID
    assert qe(None, 0, 128, 256, None, 128, None, 1e-10, silu, None) == _lib.FP8_OK
    ge = lib.fp8_quant_per_token_group_ex
    assert ge(FAKE, 4, 7168, 7168, 128, 4, FAKE, 7168, FAKE, 1e-10, silu, None) == _lib.FP8_ERR_INVALID
    assert ge(FAKE, 4, 6144, 12288, 96, 4, FAKE, 6144, FAKE, 1e-10, silu, None) == _lib.FP8_ERR_UNSUPPORTED
    assert ge(FAKE, 4, 7168, 14336, 128, 4, FAKE, 7168, FAKE, 1e-10, 8, None) == _lib.FP8_ERR_INVALID
    assert ge(None, 0, 7168, 14336, 128, 4, None, 7168, None, 1e-10, silu | ue, None) == _lib.FP8_OK
    st = lib.fp8_quant_static
    assert st(FAKE, 4, 128, 128, None, FAKE, 128, None) == _lib.FP8_ERR_INVALID
    assert "null" in _err(lib)
    assert st(FAKE, 4, 120, 128, FAKE, FAKE, 128, None) == _lib.FP8_ERR_INVALID
    assert st(FAKE, 4, 128, 128, FAKE, ctypes.c_void_p(0x10008), 128, None) == _lib.FP8_ERR_INVALID
    assert st(None, 0, 128, 128, None, None, 128, None) == _lib.FP8_OK


def test_moe_argument_errors(lib):
    mq = lib.fp8_quant_per_token_group_masked
    assert mq(FAKE, 70000, 4, 256, 256, FAKE, 128, 4, FAKE, 256, FAKE, 1e-10, 0, None) == _lib.FP8_ERR_INVALID
    assert mq(FAKE, 8, 4, 256, 256, None, 128, 4, FAKE, 256, FAKE, 1e-10, 0, None) == _lib.FP8_ERR_INVALID
    assert "masked_m" in _err(lib)
    assert mq(FAKE, 8, 4, 256, 256, FAKE, 96, 4, FAKE, 256, FAKE, 1e-10, 0, None) == _lib.FP8_ERR_INVALID
    assert mq(FAKE, 8, 4, 256, 256, FAKE, 128, 4, FAKE, 256, FAKE, 1e-10, 1, None) == _lib.FP8_ERR_INVALID
    assert mq(None, 0, 4, 256, 256, None, 128, 4, None, 256, None, 1e-10, 0, None) == _lib.FP8_OK
    mm = lib.fp8_scaled_mm_blockwise_masked
    args = dict(a=FAKE, b=FAKE, sa=FAKE, ld=64, sb=FAKE, out=FAKE, mask=FAKE, E=8, M=64, N=512, K=1024)

    def call(cfg=None, **kw):
        a = dict(args, **kw)
        return mm(a["a"], a["b"], a["sa"], a["ld"], a["sb"], a["out"], a["mask"], a["E"], a["M"], a["N"],
                  a["K"], a["K"], a["K"], a["N"], 0, ctypes.byref(cfg) if cfg is not None else None, None)

    assert call(mask=None) == _lib.FP8_ERR_INVALID
    assert call(ld=62) == _lib.FP8_ERR_INVALID
    assert call(ld=66) == _lib.FP8_ERR_INVALID  # a multiple of 4 is required
    assert call(N=504) == _lib.FP8_ERR_UNSUPPORTED
    assert call(E=70000) == _lib.FP8_ERR_INVALID
    split2 = _lib.TileConfig(_lib.VARIANTS["t64x64deep"], 0, 0, 0, 2, 0)
    assert call(cfg=split2) == _lib.FP8_ERR_INVALID  # an explicit split is refused ...
    assert "split_k" in _err(lib)
    # ... while a table entry with a split runs unsplit under the default config
    # (exercised on the GPU at 7168x7168); here: that table entry does split
    cfg = _lib.TileConfig()
    assert lib.fp8_tile_config_lookup(_lib.KIND_BLOCKWISE, 7168, 7168, 64, ctypes.byref(cfg)) == 1
    assert cfg.split_k == 2
    tile = _lib.TileConfig(_lib.VARIANTS["t128x128"], 0, 0, 0, 1, 0)
    assert call(cfg=tile) == _lib.FP8_ERR_UNSUPPORTED
    assert call(E=0) == _lib.FP8_OK and call(M=0) == _lib.FP8_OK


def test_gemm_argument_errors(lib):
    cw = lib.fp8_scaled_mm_channelwise
    assert cw(None, FAKE, FAKE, FAKE, None, FAKE, 4, 256, 512, 512, 512, 256, None, 0, None) == _lib.FP8_ERR_INVALID
    assert cw(FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 256, 500, 512, 512, 256, None, 0, None) == _lib.FP8_ERR_INVALID
    assert cw(FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 256, 512, 256, 512, 256, None, 0, None) == _lib.FP8_ERR_INVALID
    assert cw(FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10002), FAKE, 4, 256, 512, 512, 512, 256, None, 0,
              None) == _lib.FP8_ERR_INVALID
    assert cw(None, None, None, None, None, None, 0, 256, 512, 512, 512, 256, None, 0, None) == _lib.FP8_OK
    bw = lib.fp8_scaled_mm_blockwise
    assert bw(FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, 4, 200, 512, 512, 512, 200, None, 0, None) == _lib.FP8_ERR_UNSUPPORTED
    assert bw(FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, 4, 256, 528, 528, 528, 256, None, 0, None) == _lib.FP8_ERR_UNSUPPORTED
    assert bw(FAKE, FAKE, FAKE, 2, FAKE, None, FAKE, 4, 256, 512, 512, 512, 256, None, 0, None) == _lib.FP8_ERR_INVALID
    assert "a_scale_ld" in _err(lib)


def test_linear_argument_errors(lib):
    cw = lib.fp8_linear_channelwise
    # x, b, b_scale, bias, out, M, N, K, ldx, ldb, ldc, eps, q, ldq, a_scale, ws, ws_bytes, cfg, stream
    ok = (FAKE, FAKE, FAKE, None, FAKE, 4, 256, 512, 512, 512, 256, 1e-10, FAKE, 512, FAKE, None, 0, None, None)
    assert cw(*((None,) + ok[1:])) == _lib.FP8_ERR_INVALID                      # null x
    assert cw(*(ok[:12] + (None,) + ok[13:])) == _lib.FP8_ERR_INVALID           # null q
    assert cw(*(ok[:7] + (500, 500, 512) + ok[10:])) == _lib.FP8_ERR_INVALID    # K % 16
    assert cw(*(ok[:13] + (256,) + ok[14:])) == _lib.FP8_ERR_INVALID            # ldq < K
    assert cw(*(ok[:11] + (-1.0,) + ok[12:])) == _lib.FP8_ERR_INVALID           # eps < 0
    assert cw(*((None,) * 5 + (0,) + ok[6:12] + (None, 512, None, None, 0, None, None))) == _lib.FP8_OK
    bw = lib.fp8_linear_blockwise
    # ..., ldc, row_alignment, eps, q, ...
    okb = (FAKE, FAKE, FAKE, None, FAKE, 4, 256, 512, 512, 512, 256, 4, 1e-10, FAKE, 512, FAKE, None, 0, None,
           None)
    assert bw(*(okb[:6] + (200,) + okb[7:10] + (200,) + okb[11:])) == _lib.FP8_ERR_UNSUPPORTED  # N % 128
    assert bw(*(okb[:7] + (528, 528, 528) + okb[10:14] + (528,) + okb[15:])) == _lib.FP8_ERR_UNSUPPORTED  # K % 128
    assert bw(*(okb[:11] + (0,) + okb[12:])) == _lib.FP8_ERR_INVALID                             # row_alignment


def test_linear_flag_errors(lib):
    cw, bw = lib.fp8_linear_channelwise_ex, lib.fp8_linear_blockwise_ex
    # as fp8_linear_channelwise, with flags before the stream
    ok = (FAKE, FAKE, FAKE, None, FAKE, 4, 256, 512, 512, 512, 256, 1e-10, FAKE, 512, FAKE, None, 0, None)
    assert cw(*(ok + (8, None))) == _lib.FP8_ERR_INVALID                          # unknown flag bit
    assert "flags" in _err(lib)
    # [gate | up] rows are 2K wide: ldx = K is too short under SiLU-and-mul
    assert cw(*(ok + (_lib.QUANT_FUSE_SILU_MUL, None))) == _lib.FP8_ERR_INVALID
    assert "leading dimension" in _err(lib)
    okb = (FAKE, FAKE, FAKE, None, FAKE, 4, 256, 512, 512, 512, 256, 4, 1e-10, FAKE, 512, FAKE, None, 0, None)
    assert bw(*(okb + (-1, None))) == _lib.FP8_ERR_INVALID
    assert bw(*(okb + (_lib.QUANT_FUSE_SILU_MUL | _lib.QUANT_SCALE_UE8M0, None))) == _lib.FP8_ERR_INVALID
    assert "leading dimension" in _err(lib)
    assert bw(*(okb[:6] + (200,) + okb[7:10] + (200,) + okb[11:] + (_lib.QUANT_SCALE_UE8M0, None))) == \
        _lib.FP8_ERR_UNSUPPORTED                                                  # N % 128
    for f in (0, 1, 2, 3):  # M == 0 launches nothing under any flag
        assert cw(*((None,) * 5 + (0,) + ok[6:12] + (None, 512, None, None, 0, None, f, None))) == _lib.FP8_OK
        assert bw(*((None,) * 5 + (0,) + okb[6:13] + (None, 512, None, None, 0, None, f, None))) == _lib.FP8_OK


def test_linear_launch_counts(lib):
    n = lib.fp8_linear_launches
    for kind in (_lib.KIND_CHANNELWISE, _lib.KIND_BLOCKWISE):
        assert n(kind, 0, 4096, 4096, None) == 0
        assert [n(kind, m, 4096, 4096, None) for m in (1, 2, 3, 4)] == [1, 1, 1, 1]
        assert [n(kind, m, 4096, 4096, None) for m in (5, 16, 32, 8192)] == [2, 2, 2, 2]
        cfg = _lib.TileConfig(_lib.VARIANTS["t64x64panel"], 0, 0, 0, 1, 0)
        assert n(kind, 4, 4096, 4096, ctypes.byref(cfg)) == 2
    assert n(7, 1, 4096, 4096, None) == _lib.FP8_ERR_INVALID


def test_linear_launch_counts_with_flags(lib):
    n = lib.fp8_linear_launches_ex
    silu, ue = _lib.QUANT_FUSE_SILU_MUL, _lib.QUANT_SCALE_UE8M0
    for kind in (_lib.KIND_CHANNELWISE, _lib.KIND_BLOCKWISE):
        assert [n(kind, m, 4096, 4096, None, ue) for m in (1, 2, 4, 5)] == [1, 1, 1, 2]
        assert n(kind, 0, 4096, 4096, None, silu) == 0
    # SiLU-and-mul stays in the single launch only for the fewest rows (on the
    # skinny kernel; the decode stream fuses every flag while its registers
    # hold the activation: M = 4 at K = 12288 does not fit)
    sk = ctypes.byref(_lib.TileConfig(_lib.VARIANTS["skinny"], 0, 0, 0, 1, 0))
    assert [n(_lib.KIND_CHANNELWISE, m, 4096, 12288, sk, silu) for m in (1, 2, 4)] == [1, 2, 2]
    assert [n(_lib.KIND_BLOCKWISE, m, 7168, 2048, sk, silu | ue) for m in (1, 2, 3, 4)] == [1, 1, 2, 2]
    assert [n(_lib.KIND_CHANNELWISE, m, 4096, 12288, None, f) for m in (1, 2, 4) for f in (0, silu)] == \
        [1, 1, 1, 1, 2, 2]
    assert n(_lib.KIND_CHANNELWISE, 1, 4096, 4096, None, 4) == _lib.FP8_ERR_INVALID
    assert n(_lib.KIND_CHANNELWISE, 1, 4096, 4096, None, 0) == lib.fp8_linear_launches(
        _lib.KIND_CHANNELWISE, 1, 4096, 4096, None)


def test_fused_linear_all_mode(lib, monkeypatch):
    n = lib.fp8_linear_launches_ex
    silu = _lib.QUANT_FUSE_SILU_MUL
    sk = ctypes.byref(_lib.TileConfig(_lib.VARIANTS["skinny"], 0, 0, 0, 1, 0))
    assert n(_lib.KIND_CHANNELWISE, 4, 4096, 12288, sk, silu) == 2
    monkeypatch.setenv("FP8W8A8_FUSED_LINEAR", "all")
    assert [n(_lib.KIND_CHANNELWISE, m, 4096, 12288, sk, silu) for m in (1, 2, 4)] == [1, 1, 1]
    assert n(_lib.KIND_BLOCKWISE, 4, 7168, 2048, sk, silu) == 1


def test_fused_linear_kill_switch(lib, monkeypatch):
    n = lib.fp8_linear_launches
    monkeypatch.setenv("FP8W8A8_FUSED_LINEAR", "0")
    assert n(_lib.KIND_CHANNELWISE, 1, 4096, 4096, None) == 2
    assert n(_lib.KIND_BLOCKWISE, 4, 4096, 4096, None) == 2
    monkeypatch.setenv("FP8W8A8_FUSED_LINEAR", "1")
    assert n(_lib.KIND_CHANNELWISE, 1, 4096, 4096, None) == 1
    monkeypatch.delenv("FP8W8A8_FUSED_LINEAR")
    assert n(_lib.KIND_BLOCKWISE, 4, 4096, 4096, None) == 1


def test_ue8m0_gemm_shares_blockwise_tiles(lib):
    # workspace queries take the UE8M0 kind and answer as for blockwise
    cfg = _lib.TileConfig(_lib.VARIANTS["t256x128panel"], 0, 0, 0, 2, 0)
    for m, n, k in ((300, 384, 1024), (64, 7168, 7168), (4096, 4096, 4096)):
        assert lib.fp8_scaled_mm_workspace_size(_lib.KIND_BLOCKWISE_UE8M0, m, n, k, ctypes.byref(cfg)) == \
            lib.fp8_scaled_mm_workspace_size(_lib.KIND_BLOCKWISE, m, n, k, ctypes.byref(cfg))
        assert lib.fp8_scaled_mm_workspace_size(_lib.KIND_BLOCKWISE_UE8M0, m, n, k, None) == \
            lib.fp8_scaled_mm_workspace_size(_lib.KIND_BLOCKWISE, m, n, k, None)
    assert lib.fp8_scaled_mm_workspace_size(3, 64, 256, 1024, None) == ctypes.c_size_t(-1).value
    # the same argument checks as the blockwise GEMM
    mm = lib.fp8_scaled_mm_blockwise_ue8m0
    assert mm(FAKE, FAKE, FAKE, 64, FAKE, None, FAKE, 64, 504, 1024, 1024, 1024, 504, None, 0, None) == \
        _lib.FP8_ERR_UNSUPPORTED
    assert mm(FAKE, FAKE, FAKE, 32, FAKE, None, FAKE, 64, 512, 1024, 1024, 1024, 512, None, 0, None) == \
        _lib.FP8_ERR_INVALID
    assert "a_scale_ld" in _err(lib)
    assert mm(None, None, None, 0, None, None, None, 0, 512, 1024, 1024, 1024, 512, None, 0, None) == _lib.FP8_OK


def test_workspace_errors(lib):
    cfg = _lib.TileConfig(_lib.VARIANTS["t64x64"], 0, 0, 0, 4, 0)
    # t64x64 runs 512-deep K stages: K = 2048 holds 4 stages, so 4 splits
    need = lib.fp8_scaled_mm_workspace_size(0, 64, 256, 2048, ctypes.byref(cfg))
    # fixed counter region (65536 ints) + 4 tiles x 4 splits x 64 x 64 fp32
    assert need == 65536 * 4 + 4 * 4 * 64 * 64 * 4
    # K = 1024 holds only 2 stages: the split count is capped at 2
    assert lib.fp8_scaled_mm_workspace_size(0, 64, 256, 1024, ctypes.byref(cfg)) == \
        65536 * 4 + 4 * 2 * 64 * 64 * 4
    r = lib.fp8_scaled_mm_channelwise_ex(FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 256, 2048, 2048,
                                         2048, 256, FAKE, need - 1, ctypes.byref(cfg), None)
    assert r == _lib.FP8_ERR_WORKSPACE
    skinny = _lib.TileConfig(_lib.VARIANTS["skinny"], 0, 0, 0, 1, 0)
    assert lib.fp8_scaled_mm_workspace_size(0, 16, 4096, 4096, ctypes.byref(skinny)) == 0
    bad = _lib.TileConfig(_lib.VARIANTS["skinny"], 0, 0, 0, 1, 0)
    r = lib.fp8_scaled_mm_channelwise_ex(FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 256, 1024, 1024,
                                         1024, 256, None, 0, ctypes.byref(bad), None)
    assert r == _lib.FP8_ERR_INVALID and "skinny" in _err(lib)
    dec = _lib.TileConfig(_lib.VARIANTS["decode"], 0, 0, 0, 1, 0)
    assert lib.fp8_scaled_mm_workspace_size(0, 16, 4096, 4096, ctypes.byref(dec)) == 0
    for m, k in ((65, 1024), (16, 1040)):   # M, K % 128
        bad = _lib.TileConfig(_lib.VARIANTS["decode"], 0, 0, 0, 1, 0)
        r = lib.fp8_scaled_mm_channelwise_ex(FAKE, FAKE, FAKE, FAKE, None, FAKE, m, 256, k, k,
                                             k, 256, None, 0, ctypes.byref(bad), None)
        assert r == _lib.FP8_ERR_INVALID and "decode" in _err(lib), (m, k)
    # split-K over each wave's block list: K = 12288 gives wave 0 twelve
    # blocks, so split_k 5 runs 4 splits of 3 (the last partial tile and
    # split of the 512 threads' 16-byte partials per 16-column tile)
    dec5 = _lib.TileConfig(_lib.VARIANTS["decode"], 0, 0, 0, 5, 0)
    assert lib.fp8_scaled_mm_workspace_size(0, 4, 4100, 12288, ctypes.byref(dec5)) == \
        65536 * 4 + 257 * 4 * 512 * 16
    # 33-64 rows: four 16-row activation tiles, four partials per thread
    assert lib.fp8_scaled_mm_workspace_size(0, 40, 4100, 12288, ctypes.byref(dec5)) == \
        65536 * 4 + 257 * 4 * 4 * 512 * 16
    dec2 = _lib.TileConfig(_lib.VARIANTS["decode"], 0, 0, 0, 2, 0)
    r = lib.fp8_scaled_mm_channelwise_ex(FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 256, 1024, 1024,
                                         1024, 256, None, 0, ctypes.byref(dec2), None)
    assert r == _lib.FP8_ERR_WORKSPACE
    unknown = _lib.TileConfig(99, 0, 0, 0, 1, 0)
    r = lib.fp8_scaled_mm_channelwise_ex(FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 256, 1024, 1024,
                                         1024, 256, None, 0, ctypes.byref(unknown), None)
    assert r == _lib.FP8_ERR_INVALID


def test_noalloc_argument_errors_and_scratch_limit(lib):
    """fp8_scaled_mm_noalloc validates on the host like the workspace GEMMs and
    refuses a split-K plan larger than its static scratch before any device
    work (so these calls run without a GPU)."""
    f = lib.fp8_scaled_mm_noalloc
    big = _lib.TileConfig(_lib.VARIANTS["t256x256panel"], 0, 0, 0, 8, 0)
    need = lib.fp8_scaled_mm_workspace_size(0, 4096, 4096, 4096, ctypes.byref(big))
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    r = f(0, FAKE, FAKE, FAKE, 0, FAKE, None, FAKE, 4096, 4096, 4096, 4096, 4096, 4096, ctypes.byref(big), None)
    assert r == _lib.FP8_ERR_WORKSPACE and "static scratch" in _err(lib)
    r = f(1, FAKE, FAKE, FAKE, 4096, FAKE, None, FAKE, 4096, 4096, 4096, 4096, 4096, 4096, ctypes.byref(big), None)
    assert r == _lib.FP8_ERR_WORKSPACE
    assert f(7, FAKE, FAKE, FAKE, 0, FAKE, None, FAKE, 4, 256, 256, 256, 256, 256, None, None) == _lib.FP8_ERR_INVALID
    assert f(0, None, FAKE, FAKE, 0, FAKE, None, FAKE, 4, 256, 256, 256, 256, 256, None, None) == _lib.FP8_ERR_INVALID
    # blockwise: N, K multiples of 128 and a_scale_ld >= M
    assert f(1, FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, 4, 200, 256, 256, 256, 200, None, None) == \
        _lib.FP8_ERR_UNSUPPORTED
    assert f(1, FAKE, FAKE, FAKE, 3, FAKE, None, FAKE, 4, 256, 256, 256, 256, 256, None, None) == \
        _lib.FP8_ERR_INVALID
    assert f(0, FAKE, FAKE, FAKE, 0, FAKE, None, FAKE, 0, 256, 256, 256, 256, 256, None, None) == _lib.FP8_OK


def test_probe_argument_errors(lib):
    """The measurement probes validate on the host (no device needed)."""
    assert lib.fp8_probe_stream_read(FAKE, 100, FAKE, 4, None) == _lib.FP8_ERR_INVALID  # not x16
    assert lib.fp8_probe_stream_read(None, 1024, FAKE, 4, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_strided_read(FAKE, 4096, 4096, 16, 48, FAKE, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_strided_read(FAKE, 4096, 4096, 3, 128, FAKE, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_l2_feed(FAKE, 1000, 4, 0, FAKE, 4, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_panel_feed(FAKE, 100, 4, 8, 0, FAKE, 4, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_panel_feed(FAKE, 4096, 4, 8, 4, FAKE, 4, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_panel_feed(FAKE, 1 << 24, 8, 8, 0, FAKE, 4, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_mfma(0, FAKE, 4, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_lds(4, 128, FAKE, 4, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_wave_read(FAKE, 1 << 20, 1024, 16, 0, FAKE, 4, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_wave_read(FAKE, 1000, 256, 8, 1, FAKE, 4, None) == _lib.FP8_ERR_INVALID
    odd = ctypes.c_void_p(0x10008)   # 8-byte aligned only
    assert lib.fp8_probe_mfma_dot(FAKE, FAKE, FAKE, FAKE, 1, 2, None) == _lib.FP8_ERR_INVALID   # form
    assert lib.fp8_probe_mfma_dot(FAKE, FAKE, FAKE, FAKE, 0, 0, None) == _lib.FP8_ERR_INVALID   # count
    assert lib.fp8_probe_mfma_dot(odd, FAKE, FAKE, FAKE, 1, 0, None) == _lib.FP8_ERR_INVALID
    assert lib.fp8_probe_mfma_dot(FAKE, None, FAKE, FAKE, 1, 1, None) == _lib.FP8_ERR_INVALID


# ---------------------------------------------------------------- tile table
def _lookup(lib, kind, n, k, m):
    c = _lib.TileConfig()
    r = lib.fp8_tile_config_lookup(kind, n, k, m, ctypes.byref(c))
    return r, c.as_dict()


def _write(dirpath, n, k, table, kind="channelwise"):
    p = os.path.join(dirpath, f"N={n},K={k},device_name=gfx950,dtype=fp8_w8a8_{kind}.json")
    with open(p, "w") as f:
        f.write(table if isinstance(table, str) else json.dumps(table))
    return p


@pytest.fixture
def table_dir(lib, tmp_path, monkeypatch):
    monkeypatch.delenv("FP8W8A8_TUNED_CONFIGS", raising=False)
    lib.fp8_tile_config_set_dir(str(tmp_path).encode())
    yield str(tmp_path)
    lib.fp8_tile_config_set_dir(None)


def test_table_nearest_m_and_ties(lib, table_dir):
    _write(table_dir, 4096, 4096, {
        "1": {"variant": "skinny", "split_k": 1},
        "64": {"variant": "t64x64", "split_k": 4},
        "128": {"variant": "t128x128", "split_k": 2},
        "512": None,
        "4096": {"variant": "t256x256", "split_k": 1},
    })
    r, c = _lookup(lib, 0, 4096, 4096, 1)
    assert r == 1 and c["variant"] == "skinny" and c["split_k"] == 1 and c["bm"] == 32
    assert _lookup(lib, 0, 4096, 4096, 40)[1]["variant"] == "t64x64"       # |40-64| < |40-1|
    assert _lookup(lib, 0, 4096, 4096, 96)[1]["variant"] == "t64x64"       # tie 64/128 -> smaller
    assert _lookup(lib, 0, 4096, 4096, 97)[1]["variant"] == "t128x128"
    r, c = _lookup(lib, 0, 4096, 4096, 600)                                # nearest is the null entry
    assert r == 0 and c == _default(lib, 0, 4096, 4096, 600)
    assert _lookup(lib, 0, 4096, 4096, 100000)[1]["variant"] == "t256x256"
    # the other kind and other shapes have no table
    assert _lookup(lib, 1, 4096, 4096, 64)[0] == 0
    assert _lookup(lib, 0, 4096, 12288, 64)[0] == 0


def _default(lib, kind, n, k, m):
    c = _lib.TileConfig()
    assert lib.fp8_tile_config_default(kind, n, k, m, ctypes.byref(c)) == 0
    return c.as_dict()


def test_table_kill_switch(lib, table_dir, monkeypatch):
    _write(table_dir, 4096, 4096, {"64": {"variant": "t128x128", "split_k": 2}})
    assert _lookup(lib, 0, 4096, 4096, 64)[0] == 1
    for off in ("0", "false", "OFF"):
        monkeypatch.setenv("FP8W8A8_TUNED_CONFIGS", off)
        assert _lookup(lib, 0, 4096, 4096, 64) == (0, _default(lib, 0, 4096, 4096, 64))
    monkeypatch.setenv("FP8W8A8_TUNED_CONFIGS", "1")
    assert _lookup(lib, 0, 4096, 4096, 64)[0] == 1


def test_table_malformed_and_missing(lib, table_dir):
    _write(table_dir, 1024, 1024, "{not json")
    _write(table_dir, 2048, 1024, {"64": {"variant": "no-such-kernel"}})
    _write(table_dir, 3072, 1024, {"sixty": {"variant": "t64x64"}})
    for n in (1024, 2048, 3072, 5120):
        assert _lookup(lib, 0, n, 1024, 64) == (0, _default(lib, 0, n, 1024, 64))


def test_table_blockwise_kind(lib, table_dir):
    _write(table_dir, 7168, 7168, {"16": {"variant": "skinny"}, "256": {"variant": "t64x64", "split_k": 3}},
           kind="blockwise")
    assert _lookup(lib, 1, 7168, 7168, 13)[1]["variant"] == "skinny"
    c = _lookup(lib, 1, 7168, 7168, 256)[1]
    assert (c["variant"], c["bm"], c["bn"], c["split_k"], c["waves"]) == ("t64x64", 64, 64, 3, 4)
    assert _lookup(lib, 0, 7168, 7168, 256)[0] == 0


def test_default_heuristic_shapes(lib):
    assert _default(lib, 0, 4096, 4096, 1)["variant"] == "skinny"
    assert _default(lib, 0, 4096, 4096, 32)["variant"] == "decode"   # 17-32 rows, one round
    assert _default(lib, 0, 4096, 4100, 32)["variant"] == "skinny"   # K % 128 != 0
    for m in (64, 512, 4096, 8192):
        c = _default(lib, 0, 4096, 4096, m)
        assert c["variant"] != "skinny" and c["split_k"] >= 1


def test_shipped_tables_parse(lib):
    """Every table shipped next to the library parses and names real kernels."""
    lib.fp8_tile_config_set_dir(None)
    cfg_dir = os.path.join(os.path.dirname(_lib.LIB_PATH), "configs")
    if not os.path.isdir(cfg_dir):
        pytest.skip("no shipped tables")
    for name in os.listdir(cfg_dir):
        m = re.match(r"N=(\d+),K=(\d+),device_name=gfx950,dtype=fp8_w8a8_(channelwise|blockwise)\.json",
                     name)
        assert m, name
        n, k, kind = int(m.group(1)), int(m.group(2)), m.group(3)
        table = json.load(open(os.path.join(cfg_dir, name)))
        for key, val in table.items():
            r, c = _lookup(lib, 0 if kind == "channelwise" else 1, n, k, int(key))
            if val is None:
                assert r == 0
            else:
                assert r == 1 and c["variant"] == val["variant"], (name, key)


def test_split_requests_above_k_stages_are_lowered(lib):
    # a split never gets an empty K range: split 4 over two 128-deep stages
    # sizes its workspace as split 2, three stages as split 3
    ws = lib.fp8_scaled_mm_workspace_size

    def size(variant, split, k, kind=_lib.KIND_CHANNELWISE, m=64, n=256):
        cfg = _lib.TileConfig(_lib.VARIANTS[variant], 0, 0, 0, split, 0)
        return ws(kind, m, n, k, ctypes.byref(cfg))

    for v in ("t64x32deep", "t64x64panel", "t32x32deep"):
        assert size(v, 4, 256) == size(v, 2, 256) > size(v, 1, 256)
        assert size(v, 4, 384) == size(v, 3, 384) > size(v, 2, 384)
        assert size(v, 4, 640, kind=_lib.KIND_BLOCKWISE) == size(v, 3, 640, kind=_lib.KIND_BLOCKWISE)


def test_split_k_partials_stay_within_32_bit_offsets(lib):
    # 9000 splits of a 256x256 tile keep 2.4 GB of partials per tile: refused
    # before anything is launched (the workspace given is ample)
    cfg = _lib.TileConfig(_lib.VARIANTS["t256x256panel"], 0, 0, 0, 9000, 0)
    k = 128 * 9000
    st = lib.fp8_scaled_mm_channelwise_ex(FAKE, FAKE, FAKE, FAKE, None, FAKE, 256, 256, k, k, k, 256, FAKE,
                                          1 << 62, ctypes.byref(cfg), None)
    assert st == _lib.FP8_ERR_UNSUPPORTED
    assert "partials" in _err(lib)


def test_missing_library_fails_loudly(tmp_path):
    # no CPU fallback: without the built library every entry point raises
    code = (
        "import sys\n"
        "from fp8_w8a8_quantized_token_amd import _lib, ops\n"
        f"_lib.LIB_PATH = {str(tmp_path / 'absent.so')!r}\n"
        "for call in (lambda: _lib.load(), lambda: ops.tile_config(0, 4096, 4096, 16),\n"
        "             lambda: ops.linear_launches(0, 1, 4096, 4096)):\n"
        "    try:\n"
        "        call()\n"
        "    except RuntimeError as e:\n"
        "        assert 'no fallback' in str(e), e\n"
        "    else:\n"
        "        sys.exit('no error raised')\n"
        "print('ok')\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stderr


def test_default_split_k_at_small_m(lib):
    # split-K in the default heuristic: 64x64 tiles at 32 < M <= 128 split when
    # few output tiles share a long K
    def d(kind, n, k, m):
        c = _default(lib, kind, n, k, m)
        return c["variant"], c["split_k"]
    cw, bw = _lib.KIND_CHANNELWISE, _lib.KIND_BLOCKWISE
    dv, pv = "t64x64deep", "t64x64panel"
    assert d(cw, 2048, 8192, 64) == (dv, 4)      # 32 tiles, 64 stages
    assert d(cw, 5120, 5120, 64) == (dv, 2)      # 80 tiles, 40 stages
    assert d(cw, 4096, 4096, 128) == (dv, 2)     # 128 tiles
    assert d(cw, 5120, 5120, 128) == (dv, 1)     # 160 tiles
    assert d(cw, 4096, 4096, 256) == (dv, 1)     # beyond M = 128
    assert d(bw, 1536, 7168, 96) == (pv, 4)
    assert d(bw, 4096, 2048, 64) == (pv, 1)      # 16 stages
    assert d(cw, 4096, 4096, 32)[0] == "decode"


def test_default_narrow_tile_on_uneven_skinny_rounds(lib):
    cw, bw = _lib.KIND_CHANNELWISE, _lib.KIND_BLOCKWISE

    def d(kind, n, k, m):
        c = _default(lib, kind, n, k, m)
        return c["variant"], c["split_k"]
    assert d(cw, 14336, 4096, 16) == ("t32x32deep", 1)   # 896 groups: 3.5 rounds
    assert d(cw, 14336, 4096, 8) == ("t32x32deep", 1)
    assert d(cw, 5120, 5120, 32) == ("t32x32deep", 2)    # 320 groups, 40 stages
    assert d(bw, 12288, 7168, 32) == ("t32x32deep", 2)   # N >= 12288
    assert d(cw, 4096, 4096, 32)[0] == "decode"          # one round: the decode stream
    assert d(cw, 8192, 4096, 32) == ("skinny", 1)        # two whole rounds


def test_default_decode_stream_at_decode_sizes(lib):
    cw, bw = _lib.KIND_CHANNELWISE, _lib.KIND_BLOCKWISE

    def d(kind, n, k, m):
        c = _default(lib, kind, n, k, m)
        return c["variant"], c["split_k"]
    dec = ("decode", 1)
    assert d(cw, 5120, 5120, 8) == dec                   # 320 groups: two workgroups per CU
    assert d(bw, 7168, 7168, 16) == dec
    assert d(cw, 14336, 4096, 4) == dec                  # past 3.5 rounds only at M <= 4
    assert d(cw, 24576, 4096, 1) == dec
    assert d(cw, 4096, 12288, 16) == dec                 # one round, 6 KB or deeper rows
    assert d(cw, 4096, 6144, 1) == dec
    assert d(cw, 4096, 4096, 16)[0] == "skinny"          # one round, shallow rows
    assert d(bw, 3072, 4096, 1)[0] == "skinny"
    assert d(cw, 4096, 5120, 1)[0] == "skinny"
    assert d(cw, 4096, 12304, 1)[0] == "skinny"          # K % 128 != 0
    assert d(cw, 4096, 12288, 17)[0] == "decode"         # 17-32 rows, one round
    assert d(cw, 6144, 4096, 17)[0] != "decode"          # 17-32 rows, more groups than CUs
    assert d(cw, 4096, 12288, 33)[0] != "decode"
