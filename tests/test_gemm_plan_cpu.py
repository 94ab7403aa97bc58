"""The scaled GEMM's dispatcher, on the host (no GPU): for every kernel and tile it can pick,
its grid covers the output, the 32-bit buffer ranges and offsets its kernels form stay
below 2^31, and shapes past the library's limits are refused before any pointer is used.

The plan comes from fp8_debug_gemm_plan, which runs the same host code as the GEMM entry
points.  The lower bounds checked for each kernel's offsets follow from which rows a
workgroup addresses (a tile addresses all of its rows, including those past the
operand's end, up to byte K - 1 of each), so a plan that under-reported them fails here."""

import ctypes
import itertools

import pytest

import fp8_quantized_gemm_amax_amd as fp8
from fp8_quantized_gemm_amax_amd.binding import lib

LIMIT32 = 2 ** 31 - 1
MAX_ELEMS = 2 ** 40
MODES = ["tensorwise", "blockwise", "blockwise_ue8m0", "rowwise"]
SLAB = {"tensorwise": False, "blockwise": True, "blockwise_ue8m0": True, "rowwise": False}

MS = [1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 511, 512,
      1000, 2048, 4095, 4096, 4097, 8192, 65536, 2 ** 20, 2 ** 26 + 3, LIMIT32]
NS = [1, 15, 16, 17, 100, 127, 128, 129, 255, 256, 257, 2048, 4096, 5632, 11008, 14336, 18432, 65536,
      2 ** 20 + 7, LIMIT32]
KS_ANY = [16, 112, 128, 144, 2048, 4096, 7168, 8192, 8208, 2 ** 23 - 128, 2 ** 23 - 16, 2 ** 23,
          2 ** 26 - 16, 2 ** 26, LIMIT32 - 15]
KS_SLAB = [k for k in KS_ANY if k % 128 == 0] + [2 ** 26 + 128]


def cdiv(a, b):
    return -(-a // b)


def scale_row_bytes(mode, K):
    if mode == "blockwise_ue8m0":
        return cdiv(K // 128, 4) * 4
    return 4 * (K // 128) if SLAB[mode] else 0


def shapes(mode):
    ks = KS_SLAB if SLAB[mode] else KS_ANY
    return itertools.product(MS, NS, ks)


def too_large(M, N, K):
    return M * K > MAX_ELEMS or N * K > MAX_ELEMS or M * N > MAX_ELEMS


def check_plan(mode, M, N, K, plan):
    assert 1 <= len(plan) <= 2
    # the launches write disjoint, adjacent column ranges that together are [0, N)
    assert plan[0]["n_begin"] == 0 and plan[-1]["n_end"] == N
    for a, b in zip(plan, plan[1:]):
        assert a["n_end"] == b["n_begin"] and a["n_begin"] < a["n_end"]
    SR = scale_row_bytes(mode, K)
    gemv = 1 <= M <= 16 and 32 * K <= LIMIT32
    dma = K % 128 == 0 and 256 * K <= LIMIT32
    for L in plan:
        n = L["n_end"] - L["n_begin"]
        assert 1 <= L["grid"] <= LIMIT32
        assert L["threads"] == 64 * L["waves"] + (64 if L["kernel"] == "skinny" else 0)
        assert 64 <= L["threads"] <= 1024
        assert 0 <= L["max_range"] <= L["max_offset"] <= LIMIT32 or L["kernel"] == "staged"
        k = L["kernel"]
        if k == "gemv_stream":
            assert gemv and mode == "blockwise" and M == 1 and K <= 8192
            assert L["variant"] == cdiv(K, 1024)
            waves = min(N, 256 * 24)
            assert L["grid"] == cdiv(waves, 4)
            assert L["max_offset"] >= N * K               # every weight row, read once
        elif k == "gemv_valu":
            assert gemv and M == 1 and not (mode == "blockwise" and K <= 8192 and N * K <= LIMIT32)
            assert L["grid"] * 4 >= N                       # one weight row per wave
            assert L["max_offset"] >= K
        elif k == "gemv_mfma":
            assert gemv and 2 <= M <= 16
            assert L["variant"] == (1 if M <= 4 else 2)
            rows = 16 * L["variant"]
            assert L["tile_n"] == rows and L["grid"] == cdiv(N, rows)
            assert L["max_offset"] >= max(rows, 16) * K     # weight block and A padded to 16 rows
            assert L["max_range"] >= min(rows, N) * K
        elif k == "staged":
            assert not gemv and not dma
            assert (L["tile_m"], L["tile_n"]) == ((16, 256) if M <= 16 else (128, 128))
            assert L["grid"] == cdiv(M, L["tile_m"]) * cdiv(N, L["tile_n"])
            assert L["max_range"] == 0 and L["max_offset"] == 0   # 64-bit pointers only
        elif k == "skinny":
            assert not gemv and dma and 17 <= M <= 128
            mb = L["variant"]
            assert mb == (2 if M <= 32 else 4 if M <= 64 else 8) and 16 * mb >= M
            cw = L["waves"]
            assert 2 <= cw <= 7 and L["tile_n"] == 16 * cw and L["grid"] == cdiv(N, 16 * cw)
            assert L["max_offset"] >= 16 * mb * K and L["max_offset"] >= 16 * K
            assert L["max_range"] >= M * K
            if SLAB[mode]:
                assert L["max_offset"] >= cdiv(16 * mb, 64) * 64 * SR
        elif k == "tile":
            assert not gemv and dma and M > 128
            bm, bn = L["tile_m"], L["tile_n"]
            assert L["grid"] == cdiv(M, bm) * cdiv(n, bn)
            assert L["max_offset"] >= max(bm, bn) * K and L["max_offset"] >= 64 * SR
            assert L["max_range"] >= min(bm, M) * K and L["max_range"] >= min(bn, n) * K
            if L["n_begin"] > 0:
                assert L["n_begin"] % 128 == 0              # weight blocks and scales are plain offsets
                assert L["grid"] <= 256                     # a tail launch is at most one round
                wide = cdiv(M, 256) * cdiv(n, 128)          # the tail in 256x128 tiles
                if plan[0]["tile_m"] == 128:                # after whole rounds of 128x128 tiles
                    assert mode != "blockwise" and (bm, bn, L["waves"], L["variant"]) == (128, 128, 8, 3)
                    r = plan[0]["grid"] % 512                # whole rounds, short by less than a column
                    assert 64 <= L["grid"] and (r == 0 or r > 512 - cdiv(M, 128))
                elif (bm, bn) == (128, 128):                # 256x128 tiles would fill at most half a round
                    assert 2 * wide <= 256 and (L["waves"], L["variant"]) == (8, 3)
                else:
                    assert (bm, bn) == (256, 128) and 2 * wide > 256
                    assert L["variant"] == (3 if wide >= 256 and K // 128 >= 48 else 2)
            if SLAB[mode]:
                assert 128 % (bn // (L["waves"] // (bm // 64))) == 0   # a wave's columns in one weight block
            if bn == 96:                                    # one round of them, where 128x128 is one round too
                assert not SLAB[mode] and cdiv(M, 128) * cdiv(N, 96) <= 256 and cdiv(M, 128) * cdiv(N, 128) <= 256
        else:
            raise AssertionError(k)


@pytest.mark.parametrize("mode", MODES)
def test_every_accepted_shape_has_a_plan_within_32_bit_addressing(mode):
    seen, tails = set(), set()
    for M, N, K in shapes(mode):
        if too_large(M, N, K):
            with pytest.raises(fp8.Fp8Error) as e:
                fp8.fp8_debug_gemm_plan(mode, M, N, K)
            assert e.value.status == "FP8_ERR_TOO_LARGE"
            continue
        plan = fp8.fp8_debug_gemm_plan(mode, M, N, K)
        check_plan(mode, M, N, K, plan)
        for L in plan:
            seen.add((L["kernel"], L["tile_m"] if L["kernel"] in ("tile", "staged") else 0,
                      L["tile_n"] if L["kernel"] in ("tile", "staged") else 0, L["variant"]))
            if L["n_begin"] > 0:
                tails.add((L["tile_m"], L["tile_n"], L["variant"]))
    # every kernel and tile the dispatcher has was reached by the sweep
    kinds = {s[0] for s in seen}
    expect = {"gemv_valu", "gemv_mfma", "staged", "skinny", "tile"} | ({"gemv_stream"} if mode == "blockwise" else set())
    assert kinds == expect
    tiles = {(s[1], s[2], s[3]) for s in seen if s[0] == "tile"}
    assert tiles == {(256, 256, 2), (256, 128, 2), (256, 128, 3), (128, 128, 2), (128, 128, 3)} | (
        set() if SLAB[mode] else {(128, 96, 3)})
    assert tails == {(128, 128, 3), (256, 128, 2), (256, 128, 3)}   # every kind of tail launch
    assert {(s[1], s[2]) for s in seen if s[0] == "staged"} == {(16, 256), (128, 128)}
    assert {s[3] for s in seen if s[0] == "skinny"} == {2, 4, 8}
    assert {s[3] for s in seen if s[0] == "gemv_mfma"} == {1, 2}


def test_large_tile_rounds_and_tail():
    """DeepSeek-V3 up-projection, 4096 tokens: 16 x 72 tiles of 256x256 are 4.5 rounds on 256
    CUs; 64 tile columns make 4 whole rounds and the last 8 columns (2048 outputs) run as
    256 tiles of 256x128, one round."""
    # (a whole round of tail tiles over 56 slabs: three stages)
    plan = fp8.fp8_debug_gemm_plan("blockwise", 4096, 18432, 7168)
    assert [(L["kernel"], L["tile_m"], L["tile_n"], L["variant"], L["grid"], L["n_begin"], L["n_end"], L["paired"])
            for L in plan] == [("tile", 256, 256, 2, 1024, 0, 16384, 0), ("tile", 256, 128, 3, 256, 16384, 18432, 0)]
    plan = fp8.fp8_debug_gemm_plan("blockwise_ue8m0", 4096, 18432, 7168)
    assert plan[0]["paired"] == 1 and plan[1]["paired"] == 0
    # Llama-3-8B MLP: 16 x 56 = 896 tiles, 3.5 rounds; 48 columns make 3 rounds, the last 8
    # columns 256 tiles of 256x128, one round, over 32 slabs: two stages
    plan = fp8.fp8_debug_gemm_plan("blockwise", 4096, 14336, 4096)
    assert [(L["grid"], L["variant"], L["n_begin"], L["n_end"]) for L in plan] == [(768, 2, 0, 12288), (256, 2, 12288, 14336)]
    # DeepSeek-V3, 2048 tokens: 8 x 72 tiles, 2.25 rounds; the last 8 columns would be 128
    # tiles of 256x128 (half a round), so they run as one round of 256 tiles of 128x128
    # (eight waves, three stages)
    plan = fp8.fp8_debug_gemm_plan("blockwise", 2048, 18432, 7168)
    assert [(L["tile_m"], L["tile_n"], L["waves"], L["grid"], L["variant"], L["n_begin"], L["n_end"]) for L in plan] == [
        (256, 256, 8, 512, 2, 0, 16384), (128, 128, 8, 256, 3, 16384, 18432)]
    # a small tail: one 256-column of 4096 x 4352 as 32 x 2 tiles of 128x128
    plan = fp8.fp8_debug_gemm_plan("tensorwise", 4096, 4352, 7168)
    assert [(L["tile_m"], L["tile_n"], L["grid"], L["n_begin"]) for L in plan] == [(256, 256, 256, 0), (128, 128, 64, 4096)]
    # a whole number of rounds: one launch
    plan = fp8.fp8_debug_gemm_plan("tensorwise", 4096, 4096, 4096)
    assert [(L["tile_m"], L["tile_n"], L["grid"]) for L in plan] == [(256, 256, 256)]
    # more than half a round left over: no split
    plan = fp8.fp8_debug_gemm_plan("tensorwise", 4096, 4096 + 256 * 12, 4096)
    assert len(plan) == 1 and plan[0]["grid"] == 16 * 28


def test_workload_kernels():
    """The kernels the named workloads run."""
    def kinds(mode, M, N, K):
        return [(L["kernel"], L["tile_m"], L["tile_n"]) for L in fp8.fp8_debug_gemm_plan(mode, M, N, K)]
    assert kinds("tensorwise", 16, 64, 128) == [("gemv_mfma", 16, 32)]
    assert kinds("tensorwise", 512, 5632, 2048) == [("tile", 128, 96)]
    assert kinds("rowwise", 512, 5632, 2048) == [("tile", 128, 96)]
    assert kinds("blockwise", 512, 5632, 2048) == [("tile", 128, 128)]
    assert kinds("tensorwise", 1, 11008, 4096) == [("gemv_valu", 1, 1)]
    assert kinds("tensorwise", 128, 11008, 4096) == [("skinny", 128, 48)]
    assert kinds("blockwise", 1, 18432, 7168) == [("gemv_stream", 1, 1)]
    assert kinds("blockwise_ue8m0", 1, 18432, 7168) == [("gemv_valu", 1, 1)]
    assert kinds("blockwise", 128, 18432, 7168) == [("skinny", 128, 80)]
    # a K tail, and a K too long for 32-bit offsets over 256 rows
    assert kinds("tensorwise", 4096, 4096, 4112)[0][0] == "staged"
    assert kinds("blockwise", 4096, 256, 2 ** 23)[0][0] == "staged"
    assert kinds("blockwise", 4096, 256, 2 ** 23 - 128)[0][0] == "tile"


def test_shape_errors_come_before_pointer_checks():
    """Too large or malformed shapes are refused before any pointer is looked at, so null
    pointers give the shape error (and nothing touches a device)."""
    L = lib()
    cases = [
        (L.fp8_gemm_scaled_tensorwise, 2 ** 31, 16, 16, "FP8_ERR_TOO_LARGE"),        # M above 2^31 - 1
        (L.fp8_gemm_scaled_tensorwise, 2 ** 25, 16, 2 ** 16, "FP8_ERR_TOO_LARGE"),   # M K = 2^41
        (L.fp8_gemm_scaled_tensorwise, 16, 2 ** 25, 2 ** 16, "FP8_ERR_TOO_LARGE"),   # N K = 2^41
        (L.fp8_gemm_scaled_rowwise, 2 ** 21, 2 ** 20, 16, "FP8_ERR_TOO_LARGE"),      # M N = 2^41
        (L.fp8_gemm_scaled_blockwise, 2 ** 21, 2 ** 20, 128, "FP8_ERR_TOO_LARGE"),
        (L.fp8_gemm_scaled_blockwise_ue8m0, 2 ** 21, 2 ** 20, 128, "FP8_ERR_TOO_LARGE"),
        (L.fp8_gemm_scaled_blockwise, 16, 16, 144, "FP8_ERR_BAD_SHAPE"),             # K % 128
        (L.fp8_gemm_scaled_tensorwise, 16, 16, 24, "FP8_ERR_BAD_SHAPE"),             # K % 16
    ]
    for fn, M, N, K, status in cases:
        code = fn(None, None, None, None, M, N, K, None, 0, None)
        assert fp8.binding.STATUS_NAMES[code] == status, (fn.__name__, M, N, K)
    # the largest accepted shapes still plan within 32-bit addressing
    for mode in MODES:
        for M, N, K in [(2 ** 20, 2 ** 20, 128), (LIMIT32, 512, 512), (16, 2 ** 24, 2 ** 16)]:
            check_plan(mode, M, N, K, fp8.fp8_debug_gemm_plan(mode, M, N, K))


def test_plan_query_errors():
    L = lib()
    plan = ctypes.create_string_buffer(256)
    assert fp8.binding.STATUS_NAMES[L.fp8_debug_gemm_plan(7, 16, 16, 128, plan)] == "FP8_ERR_BAD_SHAPE"
    assert fp8.binding.STATUS_NAMES[L.fp8_debug_gemm_plan(0, 16, 16, 128, None)] == "FP8_ERR_NULL_POINTER"
    assert fp8.binding.STATUS_NAMES[L.fp8_debug_gemm_plan(0, -1, 16, 128, plan)] == "FP8_ERR_BAD_SHAPE"
    assert fp8.fp8_debug_gemm_plan("tensorwise", 0, 16, 128) == []
    assert fp8.fp8_debug_gemm_plan("blockwise", 16, 0, 128) == []
