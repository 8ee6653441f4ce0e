"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, validates arguments before touching a device, and its host-side
planning and tile order behave as documented."""
import os
import re

import pytest

import dense_tiled_gemm_amd as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gemm_bt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(gemm_bt\w*)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = gb.load()
    names = declared_functions()
    assert set(names) == set(gb.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert gb.gemm_bt_version() >= 100
    for st in range(5):
        s = gb.status_string(st)
        assert s and s != "unknown status"
    assert gb.status_string(99) == "unknown status"


@pytest.mark.parametrize("args,want", [
    ((1, 1, 1, -1, 4, 4, gb.BF16, gb.F32), gb.ERR_INVALID_VALUE),
    ((1, 1, 1, 4, -1, 4, gb.BF16, gb.F32), gb.ERR_INVALID_VALUE),
    ((1, 1, 1, 4, 4, -1, gb.BF16, gb.F32), gb.ERR_INVALID_VALUE),
    ((1, 1, 1, 4, 4, 4, gb.F32, gb.F32), gb.ERR_UNSUPPORTED),   # fp32 inputs are not offered
    ((1, 1, 1, 4, 4, 4, gb.BF16, 7), gb.ERR_UNSUPPORTED),
    ((1, 1, 1, 4, 4, 1 << 31, gb.BF16, gb.F32), gb.ERR_UNSUPPORTED),
    ((1, 1, 1, 4, 1 << 23, 4, gb.BF16, gb.F32), gb.ERR_UNSUPPORTED),
    ((0, 0, 0, 0, 5, 5, gb.BF16, gb.F32), gb.OK),               # empty: nothing enqueued
    ((0, 0, 0, 5, 0, 5, gb.F16, gb.F16), gb.OK),
    ((16, 16, 0, 4, 4, 4, gb.BF16, gb.F32), gb.ERR_INVALID_VALUE),  # null C
    ((0, 16, 16, 4, 4, 4, gb.BF16, gb.F32), gb.ERR_INVALID_VALUE),  # null A
    ((17, 16, 16, 4, 4, 4, gb.BF16, gb.F32), gb.ERR_INVALID_VALUE),  # misaligned A
    ((16, 16, 18, 4, 4, 4, gb.BF16, gb.F32), gb.ERR_INVALID_VALUE),  # misaligned fp32 C
])
def test_argument_validation_before_any_device_call(args, want):
    A, B, C, M, N, K, i, o = args
    assert gb.gemm_bt(A, B, C, M, N, K, i, o, None) == want


@pytest.mark.parametrize("args,want", [
    ((16, 16, 16, -1, 4, 4, 4, 16, 16, 16), gb.ERR_INVALID_VALUE),       # negative batch
    ((16, 16, 16, 2, 4, 4, 4, -16, 16, 16), gb.ERR_INVALID_VALUE),       # negative stride
    ((16, 16, 16, 2, 4, 4, 4, 16, 16, 15), gb.ERR_INVALID_VALUE),        # items of C overlap
    ((16, 16, 16, 70000, 4, 4, 4, 16, 16, 16), gb.ERR_UNSUPPORTED),      # beyond the grid's y range
    ((0, 0, 0, 0, 4, 4, 4, 16, 16, 16), gb.OK),                          # no items: nothing enqueued
    ((0, 0, 0, 3, 0, 4, 4, 16, 16, 16), gb.OK),
    ((16, 0, 16, 2, 4, 4, 4, 16, 16, 16), gb.ERR_INVALID_VALUE),         # null B
])
def test_batched_argument_validation(args, want):
    A, B, C, Z, M, N, K, sa, sb, sc = args
    assert gb.gemm_bt_batched(A, B, C, Z, M, N, K, sa, sb, sc, gb.BF16, gb.F32, None) == want
    # the stride of C is checked only when there is more than one item
    assert gb.gemm_bt_batched(16, 16, 16, 1, 4, 4, 4, 0, 0, 0, gb.BF16, gb.F32, None) in (gb.ERR_NO_DEVICE, gb.OK)


def test_batched_plan():
    # the tile tier counts all items: 64 items of 512^2 fill 256 CUs with 256x256 tiles
    p = gb.gemm_bt_plan_batched(64, 512, 512, 512, gb.BF16, gb.BF16)
    assert (p.kernel, p.bm, p.grid, p.batch) == (4, 256, 4, 64)
    p = gb.gemm_bt_plan_batched(8, 512, 512, 512, gb.BF16, gb.BF16)   # 8 x 16 tiles of 128: half the CUs
    assert (p.bm, p.grid, p.batch) == (64, 64, 8)
    p = gb.gemm_bt_plan_batched(12, 512, 512, 512, gb.BF16, gb.BF16)  # 12 x 16 tiles of 128
    assert (p.bm, p.grid, p.batch) == (128, 16, 12)
    p = gb.gemm_bt_plan_batched(1, 512, 512, 512, gb.BF16, gb.BF16)
    assert (p.bm, p.batch) == (32, 1) and p.as_dict() == gb.gemm_bt_plan(512, 512, 512, gb.BF16, gb.BF16).as_dict()
    p = gb.gemm_bt_plan_batched(5, 16, 8192, 8192, gb.BF16, gb.BF16)  # streaming kernel per item
    assert (p.kernel, p.grid, p.batch) == (3, 1024, 5)
    assert gb.gemm_bt_plan_batched(0, 64, 64, 64, gb.BF16, gb.BF16).kernel == 0
    assert gb.gemm_bt_plan_batched(4, 64, 64, 0, gb.BF16, gb.BF16).kernel == 1
    with pytest.raises(gb.GemmBtError):
        gb.gemm_bt_plan_batched(65536, 64, 64, 64, gb.BF16, gb.BF16)
    # an item stride that breaks 16-byte alignment: unaligned DMA loads for 16-bit inputs, refused for 8-bit ones
    p = gb.gemm_bt_plan_batched(2, 64, 64, 64, gb.BF16, gb.F32, a_align=2)
    assert (p.kernel, p.vec) == (4, 1)  # 2-byte aligned rows: the DMA kernel, unaligned 16-byte loads
    with pytest.raises(gb.GemmBtError):
        gb.gemm_bt_plan_batched(2, 64, 64, 64, gb.FP8_E4M3, gb.F32, b_align=8)


def test_layout_plan_and_validation():
    KI, KO = gb.K_INNER, gb.K_OUTER
    # both K-inner is the gemm_bt plan
    assert gb.gemm_bt_plan_layout(4096, 4096, 4096, KI, KI, gb.BF16, gb.BF16).as_dict() == \
        gb.gemm_bt_plan(4096, 4096, 4096, gb.BF16, gb.BF16).as_dict()
    for la, lb, var in ((KO, KI, 0), (KI, KO, 1), (KO, KO, 2)):
        p = gb.gemm_bt_plan_layout(1000, 3000, 2048, la, lb, gb.BF16, gb.F32)
        assert (p.kernel, p.variant, p.bm, p.bn, p.tiles_m, p.tiles_n, p.grid) == (5, var, 128, 128, 8, 24, 192)
    assert gb.gemm_bt_plan_layout(200, 104, 301, KO, KO, gb.F16, gb.F16).kernel == 5  # any K when both are K-outer
    # 256 x 256 tiles from half the CUs up where 128 x 128 ones need more than one wave (144 and 136 tiles), not below
    assert gb.gemm_bt_plan_layout(3072, 3072, 3072, KI, KO, gb.BF16, gb.BF16).bm == 256
    assert gb.gemm_bt_plan_layout(2048, 4352, 4096, KO, KO, gb.BF16, gb.BF16).bm == 256
    assert gb.gemm_bt_plan_layout(2560, 2560, 4096, KI, KO, gb.BF16, gb.BF16).bm == 128
    assert gb.gemm_bt_plan_batched_layout(3, 2048, 2048, 4096, KI, KO, gb.BF16, gb.BF16).bm == 256
    for la, lb, var in ((KO, KI, 3), (KI, KO, 4), (KO, KO, 5)):  # 256 x 256 tiles when they fill every CU
        p = gb.gemm_bt_plan_layout(4096, 4096, 4096, la, lb, gb.BF16, gb.BF16)
        assert (p.kernel, p.variant, p.bm, p.threads, p.grid, p.lds_bytes) == (5, var, 256, 512, 256, 128 * 1024)
    assert gb.gemm_bt_plan_layout(8, 8, 0, KO, KO, gb.BF16, gb.F32).kernel == 1
    assert gb.gemm_bt_plan_layout(0, 8, 8, KO, KO, gb.BF16, gb.F32).kernel == 0
    refused = [(100, 64, 64, KO, KI, gb.BF16, gb.F32),    # K-outer A needs M % 8 == 0
               (64, 100, 64, KI, KO, gb.BF16, gb.F32),    # K-outer B needs N % 8 == 0
               (64, 64, 60, KO, KI, gb.BF16, gb.F32),     # a K-inner operand needs K % 8 == 0
               (64, 64, 64, KO, KI, gb.FP8_E4M3, gb.F32),  # 16-bit inputs only
               (64, 64, 64, KO, KI, gb.INT8, gb.INT32),
               (1 << 16, 64, 1 << 15, KO, KI, gb.BF16, gb.F32)]  # K-outer operand of 4 GiB
    for args in refused:
        with pytest.raises(gb.GemmBtError) as ei:
            gb.gemm_bt_plan_layout(*args)
        assert ei.value.status == gb.ERR_UNSUPPORTED, args
    with pytest.raises(gb.GemmBtError) as ei:
        gb.gemm_bt_plan_layout(64, 64, 64, 2, KI, gb.BF16, gb.F32)
    assert ei.value.status == gb.ERR_INVALID_VALUE
    with pytest.raises(gb.GemmBtError):
        gb.gemm_bt_plan_layout(64, 64, 64, KO, KI, gb.BF16, gb.F32, a_align=8)
    assert gb.gemm_bt_layout(16, 16, 16, 4, 4, 4, 3, 0, gb.BF16, gb.F32, None) == gb.ERR_INVALID_VALUE
    # batched layouts: the tier counts the tiles of all items; strides as for gemm_bt_batched
    p = gb.gemm_bt_plan_batched_layout(64, 512, 512, 512, KI, KO, gb.BF16, gb.BF16)
    assert (p.kernel, p.bm, p.grid, p.batch) == (5, 256, 4, 64)
    p = gb.gemm_bt_plan_batched_layout(8, 512, 512, 512, KO, KO, gb.BF16, gb.BF16)
    assert (p.kernel, p.bm, p.grid, p.batch) == (5, 128, 16, 8)
    assert gb.gemm_bt_plan_batched_layout(3, 64, 64, 64, KI, KI, gb.BF16, gb.F32).kernel == 4
    assert gb.gemm_bt_plan_batched_layout(0, 64, 64, 64, KO, KI, gb.BF16, gb.F32).kernel == 0
    with pytest.raises(gb.GemmBtError):
        gb.gemm_bt_plan_batched_layout(2, 64, 64, 64, KO, KI, gb.BF16, gb.F32, a_align=4)  # item stride breaks 16 B
    assert gb.gemm_bt_batched_layout(16, 16, 16, 2, 8, 8, 8, 64, 64, 63, KO, KO, gb.BF16, gb.F32, None) == \
        gb.ERR_INVALID_VALUE  # items of C overlap


def test_no_device_status_without_gpu():
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; this checks the no-device path only")
    # valid-looking arguments: the call must stop at the device query
    assert gb.gemm_bt(256, 256, 256, 4, 4, 4, gb.BF16, gb.F32, None) == gb.ERR_NO_DEVICE


def test_tier_band_above_one_wave():
    """256x256 tiles (DMA kernels) for exactly one wave of them on 256 CUs and above 1.375 waves (1.2 for rows that
    take the line ring, 17/16 for 8-bit inputs); 128x256 (or 128x128) tiles in between, where the nearly empty last
    wave costs more."""
    def bm(M, N, K=4096, ind=gb.BF16, outd=gb.BF16, batch=1):
        return gb.gemm_bt_plan_batched(batch, M, N, K, ind, outd).bm
    assert bm(4096, 4096) == 256                                  # 256 tiles: one wave
    # single products from just above one wave to 1.375 waves split their rows into two launches (the row split
    # test below); stacked items take 128x256 (or 128x128) tiles
    assert bm(2176, 4096, batch=2) == bm(2048, 4160, batch=2) == bm(2432, 4096, batch=2) == 128  # 288, 272, 304
    assert bm(2560, 4096, batch=2) == bm(2304, 4608, batch=2) == 128  # 320, 324 tiles (128x256 ones)
    assert bm(5120, 4608) == bm(5120, 5120) == 256                # 360, 400 tiles
    assert bm(2304, 4608, K=4104, batch=2) == 256                 # line-ring rows: above 1.2 waves
    assert bm(1536, 3072, 512, batch=4) == 128                    # 4 items x 72 tiles: 3 of them under 7/8
    # 8-bit inputs: a narrower band, up to 17/16 waves
    # (items of 68 and 72 tiles, 272 and 288 in all: single products and items that fill 7/8 of the CUs in one
    # wave split instead)
    assert bm(1024, 4352, ind=gb.FP8_E4M3, batch=4) == bm(1024, 4352, ind=gb.INT8, outd=gb.INT32, batch=4) == 128
    assert bm(1536, 3072, ind=gb.FP8_E4M3, batch=4) == bm(1536, 3072, ind=gb.INT8, outd=gb.INT32, batch=4) == 256
    assert bm(5120, 4096, ind=gb.FP8_E4M3) == 256


def test_row_split_plans():
    """A single product with just over one wave of 256x256 tiles (up to 1.375 waves) runs as two launches:
    R whole tile rows as one wave of 256x256 tiles (at least 7/8 of the CUs), then the remaining rows on their own
    plan (split along K through gemm_bt_ws when that plan splits).  The plan describes the first launch."""
    def plan(M, N, K=4096, ind=gb.BF16, outd=gb.BF16, batch=1):
        p = gb.gemm_bt_plan_batched(batch, M, N, K, ind, outd)
        return p.split_rows, p.bm, p.bn, p.grid
    assert plan(4352, 4096) == plan(4160, 4096) == plan(5120, 4096) == (4096, 256, 256, 256)  # 272, 272, 320 tiles
    assert plan(4608, 4608) == (3584, 256, 256, 252)        # 18 tile columns: 14 tile rows first
    assert plan(4100, 4100, K=136) == (3840, 256, 256, 255)  # line-ring rows and ragged edges alike
    assert plan(4096, 4096)[0] == plan(5120, 4608)[0] == 0   # one wave; 360 tiles (1.41 waves)
    # just past W whole waves: W waves first
    assert plan(8448, 4096) == plan(9728, 4096) == (8192, 256, 256, 512)  # 528, 608 tiles
    assert plan(12544, 4096) == (12288, 256, 256, 768)
    assert plan(8192, 4096)[0] == plan(9984, 4096)[0] == plan(6144, 4096)[0] == 0  # 2, 2.44, 1.5 waves
    assert plan(2176, 4096, batch=2)[0] == 0                # stacked items: one launch
    assert plan(4352, 4096, ind=gb.FP8_E4M3)[0] == plan(4352, 4096, ind=gb.INT8, outd=gb.INT32)[0] == 4096  # 8-bit
    assert plan(512, 40000)[0] == 0                          # 157 tiles per tile row: the first launch under 7/8
    # stacked items split by items: the first floor(CUs / tiles per item) of them as one wave
    def items(batch, M, N, K=4096):
        p = gb.gemm_bt_plan_batched(batch, M, N, K, gb.BF16, gb.BF16)
        return p.split_items, p.split_rows, p.bm, p.grid
    assert items(17, 256, 4096) == (16, 0, 256, 16) and items(9, 512, 4096) == (8, 0, 256, 32)
    assert items(68, 512, 512, 128) == (64, 0, 256, 4) and items(5, 1024, 4096, 2048) == (4, 0, 256, 64)
    assert items(4, 1536, 3072)[0] == 0                      # 72 tiles per item: 3 items fill under 7/8
    assert items(33, 256, 4096)[0] == 32 and items(33, 256, 2048, 64)[0] == 32  # 528 and 264 tiles
    assert items(16, 256, 4096)[0] == items(2, 2176, 4096)[0] == 0  # one wave; 144 tiles per item
    # the workspace is that of the second launch's split plan
    for M, rest in ((4608, 512), (4160, 64), (4352, 256)):
        p = gb.gemm_bt_plan_ws(M, 4096, 4096, gb.BF16, gb.BF16)
        r = gb.gemm_bt_plan_ws(rest, 4096, 4096, gb.BF16, gb.BF16)
        assert p.split_rows == 4096 and r.split_rows == 0
        assert p.workspace_bytes == r.workspace_bytes == gb.gemm_bt_workspace_size(M, 4096, 4096, gb.BF16, gb.BF16)
    assert gb.gemm_bt_plan_ws(4160, 4096, 4096, gb.BF16, gb.BF16).workspace_bytes > 0


def test_wide_tier_and_split_plans():
    """16-bit inputs (items stacked or not): 256x256 tiles where fewer of them than CUs stand against more than one
    wave of 128-row tiles of either width (for rows that take the line ring, once they fill 0.6 of the CUs); 128x256
    tiles where they make one wave and 128x128 ones would need two, and past one wave of 256x256 tiles once they make whole waves
    or more than 1.375 waves; the split plan (gemm_bt_ws) only where its tiles (32x64 for M <= 32, 64x64 for
    M <= 64, else 128x128) fill at most half the CUs and each piece keeps at least 32 K steps, one piece per
    workgroup."""
    def tile(M, N, K=4096, batch=1, ind=gb.BF16):
        p = gb.gemm_bt_plan_batched(batch, M, N, K, ind, gb.BF16)
        return p.bm, p.bn
    assert tile(2048, 4096) == (128, 256)                        # 256 tiles of 128x256: one wave
    assert tile(2176, 4096, batch=2) == tile(2304, 4096, batch=2) == (128, 256)  # 544, 576 (272, 288 of 256x256)
    # 256x256: 192, 160, 136, 144 (odd K), 160 (4-byte rows) tiles; 128-row tiles over one wave
    assert tile(3072, 4096) == tile(2560, 4096) == tile(2048, 4352) == tile(3000, 3000, K=3001) \
        == tile(5000, 2000, K=2002) == tile(3072, 3072, K=3072) == (256, 256)
    # line-ring rows: 160, 176, 192, 224 tiles of 256x256; under 0.6 of the CUs (144, 153) the ring's 128-row tiles
    assert tile(2560, 3900, K=3000) == tile(2600, 3900, K=3000) == tile(4000, 3000, K=5000) \
        == tile(2000, 7000, K=3000) == (256, 256)
    assert tile(3000, 3000, K=3000) == tile(2100, 4300, K=3000) == (128, 96)
    assert tile(2560, 2560) == tile(2816, 2816, K=2816) == tile(3072, 1536) == (128, 256)  # 200, 242, 144: one wave
    assert tile(2500, 2500, K=2496) == (128, 256)
    assert tile(2500, 2500, K=2504) == (128, 128)                # line-ring rows: no 128x256 twin
    assert tile(3072, 3072, K=3072, batch=2) == (128, 256)       # stacked items: 576 tiles of 128x256
    assert tile(1024, 1024, batch=9) == tile(2048, 2048, batch=3) == (256, 256)   # stacked: 144 and 192 tiles
    assert tile(2048, 2048) == (128, 128)                        # 128 tiles of 128x256: half the CUs
    assert tile(4096, 4096) == (256, 256)
    assert tile(512, 1024, K=128, batch=16) == (128, 256)        # items stacked: 256 tiles
    assert tile(512, 1024, K=72, batch=16) == (128, 128)         # 144-byte rows: the line ring's 128x128 tiles
    assert tile(2048, 4096, ind=gb.FP8_E4M3) != (128, 256)       # 16-bit inputs only
    # 8-bit inputs: 256x256 tiles from half the CUs up where 128x128 ones need more than one wave
    i8 = lambda M, N: gb.gemm_bt_plan(M, N, 4096, gb.INT8, gb.INT32).bm
    assert tile(3072, 3072, ind=gb.FP8_E4M3) == (256, 256) and i8(2048, 4352) == 256   # 144, 136 tiles
    assert tile(2560, 2560, ind=gb.FP8_E4M3) == (128, 128) and i8(2048, 2048) == 128   # 100, 64 tiles
    # 96x128 tiles for a single product when they make at most one wave and keep more CUs busy than 128x128
    assert tile(768, 4096) == tile(3000, 1000) == tile(1536, 2048) == (96, 128)  # 256 tiles each
    # or 128x96 tiles when those make more tiles within the wave (96x128: 264, 264, 264, 200 against 204)
    assert tile(1000, 3000) == tile(2048, 1536) == tile(1024, 3072) == tile(700, 3200) == (128, 96)
    assert tile(1500, 1500) == (96, 128)                                           # 192 either way: 96x128
    assert tile(1024, 4096) == (128, 128)                                          # 256 tiles of 128x128
    assert tile(768, 2048, batch=2) == (128, 128)                                  # single products only
    assert tile(768, 4096, batch=2) == (128, 256)          # stacked: one wave of 128x256, two of 128x128
    assert tile(768, 4096, ind=gb.FP8_E4M3) == (128, 128)                          # 16-bit inputs only
    # several waves of 128x128 tiles (line-ring rows, 256x256 tiles under 0.6 of the CUs): 128x96 (or 96x128)
    # tiles when 0.9 x their waves < the 128x128 waves
    assert tile(3072, 1536, K=3000) == tile(2048, 4352, K=3000) == (128, 96)   # 2 and 3 waves either way
    assert tile(1700, 3500, K=72) == (96, 128)             # 504 tiles (2 waves): 128x96 need 3
    assert tile(3072, 1536, K=3000, batch=2) != (128, 96)                        # single products only
    p = gb.gemm_bt_plan(768, 4096, 4096, gb.BF16, gb.BF16)
    assert (p.threads, p.stages, p.grid, p.lds_bytes) == (256, 4, 256, 4 * (96 + 128) * 64 * 2)
    p = gb.gemm_bt_plan(2048, 4096, 4096, gb.BF16, gb.BF16)
    assert (p.threads, p.stages, p.lds_bytes) == (512, 3, 3 * (128 + 256) * 64 * 2)
    for M, N, K, T, S in [(1024, 1024, 16384, 64, 4), (512, 1024, 32768, 32, 8), (300, 700, 30002, 18, 14),
                          (1024, 2048, 8192, 128, 2)]:
        p = gb.gemm_bt_plan_ws(M, N, K, gb.BF16, gb.F32)
        assert (p.bm, p.bn, p.split_tiles, p.grid) == (128, 128, T, T * S), (M, N, K)
        assert p.workspace_bytes == 16384 + T * S * 128 * 128 * 4
        assert gb.gemm_bt_workspace_size(M, N, K, gb.BF16, gb.F32) == p.workspace_bytes
        assert gb.gemm_bt_plan(M, N, K, gb.BF16, gb.F32).split_tiles == 0  # gemm_bt never splits
    for M, N, K in [(1000, 3000, 2050), (1024, 4096, 4096), (1024, 1024, 4096), (4096, 4096, 4096),
                    (16, 8192, 8192), (768, 768, 8192)]:
        assert gb.gemm_bt_plan_ws(M, N, K, gb.BF16, gb.F32).split_tiles == 0, (M, N, K)
        assert gb.gemm_bt_workspace_size(M, N, K, gb.BF16, gb.F32) == 0
    assert gb.gemm_bt_plan_ws(1024, 1024, 16384, gb.FP8_E4M3, gb.F32).split_tiles == 0  # 16-bit inputs only
    # M > 64: no 128x128 split when the plain grid already covers the CUs and M fills < 3/4 of the 128-row tiles
    assert gb.gemm_bt_plan_ws(65, 8192, 8192, gb.BF16, gb.BF16).split_tiles == 0    # 256 tiles of 64x64
    assert gb.gemm_bt_plan_ws(100, 4096, 16384, gb.BF16, gb.F32).split_tiles == 32  # rows 78 % full
    # thin products (M <= 64): 32x64 (M <= 32) or 64x64 tiles, split into as many pieces of >= 32 K steps as
    # fill the CUs, fewer when K is short
    for M, N, K, bm, T, S in [(64, 8192, 8192, 64, 128, 2), (33, 8192, 8192, 64, 128, 2), (32, 8192, 4096, 32, 128, 2),
                              (17, 8192, 8192, 32, 128, 2), (64, 4096, 16384, 64, 64, 4), (64, 3072, 8192, 64, 48, 4),
                              (17, 4096, 4096, 32, 64, 2), (40, 6000, 8195, 64, 94, 2), (64, 1024, 65536, 64, 16, 16)]:
        p = gb.gemm_bt_plan_ws(M, N, K, gb.BF16, gb.BF16)
        assert (p.bm, p.bn, p.bk, p.split_tiles, p.grid) == (bm, 64, 128, T, T * S), (M, N, K)  # 256-byte rows
        assert p.workspace_bytes == 16384 + T * S * bm * 64 * 4
        assert p.lds_bytes == 4 * (bm + 64) * 128 * 2
    for M, N, K in [(64, 8192, 2048), (64, 12288, 16384), (32, 12288, 8192), (16, 8192, 8192)]:
        assert gb.gemm_bt_plan_ws(M, N, K, gb.BF16, gb.BF16).split_tiles == 0, (M, N, K)  # K short, or >= 128 tiles
    # the tile height follows M across the thin range; every thin plan's workspace fits the no-allocation scratch
    # (16 KiB of counters + 16 MiB of partial tiles)
    for M in (17, 24, 32, 33, 48, 64):
        for ind, outd in ((gb.BF16, gb.BF16), (gb.F16, gb.F32), (gb.BF16, gb.F16)):
            p = gb.gemm_bt_plan_ws(M, 8192, 8192, ind, outd)
            assert (p.bm, p.bk, p.split_tiles, p.grid) == (32 if M <= 32 else 64, 128, 128, 256), (M, ind, outd)
            assert p.workspace_bytes <= 16384 + 16 * 2**20
    assert gb.gemm_bt_plan_ws(64, 8192, 8192, gb.FP8_E4M3, gb.F32).split_tiles == 0  # 16-bit inputs only
    assert gb.gemm_bt_plan_ws(64, 8192, 8192, gb.INT8, gb.INT32).split_tiles == 0


def test_line_ring_plans():
    """Rows 16-byte aligned but not 128-byte aligned (K % 8 == 0, K % 64 != 0 for 16-bit inputs) take the line-ring
    twins (variants 12..15) of the 128 x 128, 96 x 128, 128 x 96 and (above one tile per CU) 64 x 64 tiers,
    128 x 128 ring tiles where aligned rows
    would take 128 x 256 ones, and the ring's split form; everything else keeps its plain tier."""
    def plan(M, N, K, ind=gb.BF16, outd=gb.BF16, a_align=256, b_align=256, batch=1):
        p = gb.gemm_bt_plan_batched(batch, M, N, K, ind, outd, a_align, b_align)
        return p.variant, p.bm, p.bn, p.bk, p.stages
    assert plan(1024, 4096, 4104, gb.F16, gb.F16) == (12, 128, 128, 64, 4)
    assert plan(768, 4096, 4104) == (13, 96, 128, 64, 4)
    assert plan(1000, 3000, 2056, gb.BF16, gb.F32) == (14, 128, 96, 64, 4)
    assert plan(1000, 3000, 3000, gb.BF16, gb.F32)[0] == 14
    assert plan(512, 1024, 4104, batch=8)[0] == 12                      # batch items, each 16-byte aligned
    assert plan(1024, 4096, 4096, gb.F16, gb.F16)[0] == 1               # 128-byte aligned rows
    assert plan(1024, 4096, 4104, gb.F16, gb.F16, a_align=8)[0] == 1    # A only 8-byte aligned
    assert plan(1024, 4096, 4104, gb.F16, gb.F16, b_align=4)[0] == 1
    assert plan(1000, 3000, 2050, gb.BF16, gb.F32)[0] == 9              # 4-byte aligned rows
    assert plan(1000, 1000, 1000, gb.BF16, gb.F32)[0] == 2              # 64 x 64: one tile per CU, plain ring
    assert plan(1000, 1500, 3000)[0] == plan(700, 2000, 200)[0] == 15  # 64 x 64: more tiles than CUs, line ring
    assert plan(1000, 2000, 1024)[0] == 2                               # ... on aligned rows, plain
    assert plan(500, 500, 1000)[0] == 6                                 # 32 x 64 keeps its plain ring
    assert plan(4096, 4096, 4104)[0] == 0                               # 256 x 256 (five-slot ring)
    assert plan(2048, 4096, 4104)[0] == plan(2000, 4000, 1000)[0] == 12  # ring 128 x 128 instead of 128 x 256
    assert plan(3072, 4096, 1000)[0] == plan(3072, 4096, 4104)[0] == 0   # 192 tiles of 256 x 256: 0.75 of the CUs
    assert plan(2048, 4096, 4096)[0] == 7
    for K, v in ((16392, 12), (8200, 12), (16384, 1)):                  # the split form follows the rows too
        p = gb.gemm_bt_plan_ws(1024, 1024, K, gb.BF16, gb.BF16)
        assert (p.variant, p.bm, p.split_tiles, p.grid) == (v, 128, 64, 256), K
    assert plan(1024, 4096, 4112, gb.FP8_E4M3, gb.BF16)[0] == 4         # 16-bit inputs only


def test_layout_tier_band():
    """K-outer operands: 256x256 tiles at exactly one wave of them on 256 CUs and above 1.375 waves."""
    def bm(M, N, K=4096):
        return gb.gemm_bt_plan_layout(M, N, K, gb.K_INNER, gb.K_OUTER, gb.BF16, gb.BF16).bm
    assert bm(4096, 4096) == 256                                       # 256 tiles
    assert bm(4352, 4096) == bm(4864, 4096) == bm(5632, 4096) == 128   # 272, 304, 352 tiles
    assert bm(6144, 4096) == bm(8192, 8192) == 256                     # 384, 1024 tiles


def test_plan_choices():
    p = gb.gemm_bt_plan(4096, 4096, 4096, gb.BF16, gb.BF16)
    assert (p.kernel, p.bm, p.bn, p.vec, p.grid) == (4, 256, 256, 8, 256)
    # five-slot ring: one A or B tile (256 rows x 64 K) per slot, all of LDS
    assert (p.stages, p.lds_bytes) == (5, 5 * p.bm * p.bk * 2) and p.lds_bytes == 160 * 1024
    p = gb.gemm_bt_plan(2048, 1536, 4096, gb.BF16, gb.BF16)  # 128x128 tiles (192 > half the CUs): A+B stages
    assert p.bm == 128 and p.lds_bytes == p.stages * (p.bm + p.bn) * p.bk * 2 <= 160 * 1024
    p = gb.gemm_bt_plan(1024, 4096, 4096, gb.F16, gb.F16)
    assert (p.kernel, p.bm, p.bn, p.grid) == (4, 128, 128, 256)
    p = gb.gemm_bt_plan(1000, 3000, 2050, gb.BF16, gb.F32)  # 4-byte rows: DMA kernel + K tail
    assert (p.kernel, p.bm, p.bn, p.vec, p.tiles_m, p.tiles_n) == (4, 128, 96, 2, 8, 32)  # one wave of 128x96
    p = gb.gemm_bt_plan(1000, 3000, 2049, gb.BF16, gb.F32)
    assert (p.kernel, p.bm, p.vec) == (4, 128, 1)  # 2-byte aligned rows take the DMA kernel too
    p = gb.gemm_bt_plan(16, 8192, 8192, gb.BF16, gb.BF16)
    assert (p.kernel, p.bm, p.bn, p.ksplit, p.grid) == (3, 16, 8, 1, 1024)
    # several streaming workgroups fit on one CU
    assert 4 * p.lds_bytes <= 160 * 1024 and p.stages >= 3
    # rows that are not 16-byte aligned stream through the same kernel (unaligned DMA, K tail after the loop)
    for K, al in ((8190, 256), (8191, 256), (8192, 2)):
        q = gb.gemm_bt_plan(16, 8192, K, gb.BF16, gb.BF16, a_align=al)
        assert (q.kernel, q.variant, q.bn, q.grid) == (3, 1, 8, 1024) and q.vec < 8
    # 8-bit float inputs: the LDS-DMA kernel with 128-element K steps, also for M <= 16
    for code in (gb.FP8_E4M3, gb.FP8_E5M2):
        p = gb.gemm_bt_plan(4096, 4096, 4096, code, gb.BF16)
        assert (p.kernel, p.bm, p.bn, p.bk, p.vec, p.stages, p.lds_bytes) == (4, 256, 256, 128, 16, 5, 160 * 1024)
        assert gb.gemm_bt_plan(1024, 4096, 4096, code, gb.F16).bm == 128
        assert gb.gemm_bt_plan(16, 8192, 8192, code, gb.BF16).kernel == 4
        for args in ((64, 64, 40, code, gb.F32, 256, 256, 256), (64, 64, 48, code, gb.F32, 8, 256, 256),
                     (64, 64, 48, code, code, 256, 256, 256)):
            with pytest.raises(gb.GemmBtError):
                gb.gemm_bt_plan(*args)
    # 8-bit integer inputs: the same kernels and tiles, int32 out only, K <= 131071
    p = gb.gemm_bt_plan(4096, 4096, 4096, gb.INT8, gb.INT32)
    assert (p.kernel, p.bm, p.bn, p.bk, p.vec, p.stages, p.lds_bytes) == (4, 256, 256, 128, 16, 5, 160 * 1024)
    assert gb.gemm_bt_plan(1024, 4096, 4096, gb.INT8, gb.INT32).bm == 128
    assert gb.gemm_bt_plan(512, 512, 512, gb.INT8, gb.INT32).bm == 64
    assert gb.gemm_bt_plan(64, 64, 131056, gb.INT8, gb.INT32).kernel == 4
    assert gb.gemm_bt_plan(7, 9, 0, gb.INT8, gb.INT32).kernel == 1
    for args in ((64, 64, 48, gb.INT8, gb.F32), (64, 64, 48, gb.INT8, gb.BF16), (64, 64, 48, gb.BF16, gb.INT32),
                 (64, 64, 48, gb.FP8_E5M2, gb.INT32), (64, 64, 48, gb.INT32, gb.INT32), (64, 64, 48, gb.INT8, gb.INT8),
                 (64, 64, 40, gb.INT8, gb.INT32), (64, 64, 131072, gb.INT8, gb.INT32)):
        with pytest.raises(gb.GemmBtError):
            gb.gemm_bt_plan(*args)
    with pytest.raises(gb.GemmBtError):
        gb.gemm_bt_plan(64, 64, 48, gb.INT8, gb.INT32, a_align=8)
    p = gb.gemm_bt_plan(512, 512, 512, gb.BF16, gb.F32)  # 16 tiles of 128, 64 of 64: 32x64 tiles fill more CUs
    assert (p.kernel, p.bm, p.bn, p.grid) == (4, 32, 64, 128)
    p = gb.gemm_bt_plan(1024, 1024, 512, gb.BF16, gb.F32)  # 256 tiles of 64x64: all CUs
    assert (p.kernel, p.bm, p.bn, p.grid) == (4, 64, 64, 256)
    assert gb.gemm_bt_plan(512, 512, 512, gb.FP8_E4M3, gb.F32).bm == 64  # no 32x64 tier for 8-bit inputs
    assert gb.gemm_bt_plan(2048, 1536, 200, gb.BF16, gb.F32).bm == 128
    # at most half the CUs busy with 128x128 tiles: 64x64 (thin products)
    assert gb.gemm_bt_plan(1024, 2048, 4096, gb.BF16, gb.BF16).bm == 64   # 128 tiles of 128
    assert gb.gemm_bt_plan(128, 8192, 8192, gb.BF16, gb.BF16).bm == 64
    assert (gb.gemm_bt_plan(64, 8192, 8192, gb.BF16, gb.BF16).bm, gb.gemm_bt_plan(64, 8192, 8192, gb.BF16, gb.BF16).bn) == (32, 64)
    assert gb.gemm_bt_plan(1024, 1024, 200, gb.BF16, gb.F32).bm == 64
    assert gb.gemm_bt_plan(7, 9, 0, gb.BF16, gb.F32).kernel == 1   # K == 0: zero fill
    assert gb.gemm_bt_plan(0, 9, 5, gb.BF16, gb.F32).kernel == 0   # empty
    # alignment decides the load width
    assert gb.gemm_bt_plan(64, 64, 64, gb.BF16, gb.F32, a_align=4).vec == 2
    assert gb.gemm_bt_plan(64, 64, 63, gb.BF16, gb.F32).vec == 1
    assert gb.gemm_bt_plan(64, 64, 66, gb.BF16, gb.F32).vec == 2


@pytest.mark.parametrize("tiles_m,tiles_n,group_m", [(16, 16, 4), (8, 32, 4), (8, 24, 4), (4, 4, 4),
                                                     (3, 5, 4), (1, 256, 4), (7, 13, 2), (33, 1, 8)])
def test_tile_order_is_a_bijection(tiles_m, tiles_n, group_m):
    seen = set()
    for pid in range(tiles_m * tiles_n):
        tm, tn = gb.gemm_bt_tile_coord(pid, tiles_m, tiles_n, group_m)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
    assert len(seen) == tiles_m * tiles_n
    with pytest.raises(gb.GemmBtError):
        gb.gemm_bt_tile_coord(tiles_m * tiles_n, tiles_m, tiles_n, group_m)


def test_tile_order_keeps_each_die_on_a_compact_block():
    # 16 x 16 tiles (4096^2 with 256^2 tiles): workgroups pid = x (mod 8) run on
    # die x; each die should get a 4-row x 8-column block, so it reads 4 A
    # panels and 8 B panels instead of 1 x 32 or 32 x 1.
    for x in range(8):
        tiles = [gb.gemm_bt_tile_coord(pid, 16, 16, 4) for pid in range(x, 256, 8)]
        rows = {t[0] for t in tiles}
        cols = {t[1] for t in tiles}
        assert len(tiles) == 32 and len(rows) == 4 and len(cols) == 8
    # the first 8 workgroups (one per die, dispatched together) start 8 different blocks
    firsts = [gb.gemm_bt_tile_coord(pid, 16, 16, 4) for pid in range(8)]
    assert len(set(firsts)) == 8


def test_c_program_without_a_device():
    """The C++ program built against include/gemm_bt.h alone: on a machine without a GPU it must see the
    library's argument errors and GEMM_BT_ERR_NO_DEVICE."""
    import subprocess
    import torch

    exe = os.path.join(ROOT, "tests", "c_abi_check")
    if not os.path.exists(exe):
        pytest.skip("tests/c_abi_check is not built (run the build entry point)")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; the GPU tests run this program against the device")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("no-device ok"), (r.returncode, r.stdout, r.stderr)
