"""Host-side checks of the C ABI and the analytic models (no GPU needed).

The library is loaded but no kernel is launched: descriptor validation, plan
choice, the LDS sizing rule and the swizzle index map are pure host code.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import image_stencil_amd as isa
from image_stencil_amd import _abi, traffic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M):
            if m.group(1) not in ("if", "typedef", "defined"):
                names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_abi.LIB_PATH)
    declared = _declared_functions()
    assert {"conv2d_create", "conv2d_forward", "conv_chain_forward"} <= declared
    for name in declared:
        assert hasattr(lib, name), "symbol %s declared in include/ but not exported" % name
    # and the binding declares a signature for each
    assert declared == {s[0] for s in _abi.SIGNATURES}


def test_version():
    assert isa.is_version() == 1


def _status(desc):
    plan = ctypes.c_void_p()
    st = _abi.load().conv2d_create(ctypes.byref(desc), ctypes.byref(plan))
    if st == 0:
        _abi.load().conv2d_destroy(plan)
    return st


def test_create_validation():
    ok = isa.make_desc(1, 1, 64, 64, 1, 3, 3)
    assert _status(ok) == _abi.IS_OK
    bad = isa.make_desc(1, 1, 64, 64, 1, 4, 3)
    assert _status(bad) == _abi.IS_ERR_UNSUPPORTED          # even filter
    d = isa.make_desc(1, 1, 64, 64, 1, 3, 3)
    d.pad_h = 0
    assert _status(d) == _abi.IS_ERR_INVALID_ARG           # not same padding
    d = isa.make_desc(1, 1, 64, 64, 1, 3, 3)
    d.stride_w = 2
    assert _status(d) == _abi.IS_ERR_INVALID_ARG
    d = isa.make_desc(1, 0, 64, 64, 1, 3, 3)
    assert _status(d) == _abi.IS_ERR_INVALID_ARG           # no channels
    d = isa.make_desc(-1, 1, 64, 64, 1, 3, 3)
    assert _status(d) == _abi.IS_ERR_INVALID_ARG
    d = isa.make_desc(1, 4, 8, 8, 4, 3, 3)
    d.layout = _abi.IS_NHWC                                 # fp32 NHWC not offered
    assert _status(d) == _abi.IS_ERR_UNSUPPORTED
    d = isa.make_desc(1, 4, 8, 8, 4, 3, 3, dtype="f16")
    assert _status(d) == _abi.IS_OK
    d.out_dtype = _abi.IS_F32
    assert _status(d) == _abi.IS_ERR_UNSUPPORTED
    d = isa.make_desc(1, 1, 0, 0, 1, 3, 3)                  # empty image is valid
    assert _status(d) == _abi.IS_OK
    assert _abi.load().conv2d_create(None, None) == _abi.IS_ERR_INVALID_ARG


def test_forward_argument_errors_need_no_gpu():
    """Null and misaligned pointers are rejected before any launch."""
    p = isa.Plan(isa.make_desc(1, 1, 64, 64, 1, 3, 3))
    lib = _abi.load()
    assert lib.conv2d_forward(p.handle, None, 16, None, 4096 * 16, None) == _abi.IS_ERR_INVALID_ARG
    assert lib.conv2d_forward(p.handle, 0x1004, 0x2000, None, 0x100000, None) == _abi.IS_ERR_MISALIGNED
    # x and y overlapping
    assert lib.conv2d_forward(p.handle, 0x10000, 0x200, None, 0x10000 + 64, None) == _abi.IS_ERR_INVALID_ARG
    assert lib.conv2d_forward(None, 0x1000, 0x2000, None, 0x100000, None) == _abi.IS_ERR_INVALID_ARG


def test_plan_choice_and_counts():
    for R in (3, 5, 7):
        p = isa.Plan(isa.make_desc(1, 1, 8192, 8192, 1, R, R))
        info = p.info()
        assert info["kernel"] == "is_k1_single"
        assert info["flops"] == 2 * R * R * 8192 * 8192
        assert info["flops"] == traffic.conv_flops(1, 1, 8192, 8192, 1, R, R)
        assert info["bytes"] == traffic.conv_bytes(1, 1, 8192, 8192, 1, R, R)
        gx = info["grid"][0]
        assert gx == 32 * (8192 // info["tile"][1])
    # counts quoted for the workloads: 1.21/3.36/6.58 GFLOP and 536.9 MB for 8192^2
    assert round(traffic.conv_flops(1, 1, 8192, 8192, 1, 3, 3) / 1e9, 2) == 1.21
    assert round(traffic.conv_flops(1, 1, 8192, 8192, 1, 7, 7) / 1e9, 2) == 6.58
    assert round(traffic.conv_flops(1, 32, 720, 1280, 32, 3, 3) / 1e9, 2) == 16.99
    chain = [(1, 32, 5), (32, 32, 3), (32, 32, 3), (32, 4, 3)]
    assert round(traffic.chain_flops(1, 720, 1280, chain) / 1e9, 2) == 37.57
    assert round(traffic.conv_flops(8, 64, 256, 256, 64, 3, 3) / 1e9, 2) == 38.65
    # the 32 -> 32 3x3 fp32 layer runs on the fp32 matrix cores
    info = isa.Plan(isa.make_desc(1, 32, 720, 1280, 32, 3, 3, "f32", True)).info()
    assert info["kernel"] == "is_k5_mfma_f32"
    assert info["tile"] == (32, 13) and info["lds_bytes"] == 2 * 20 * 256 * 16
    # wide filters fall back to the one-thread-per-output kernel
    info = isa.Plan(isa.make_desc(1, 1, 64, 64, 1, 9, 9)).info()
    assert info["kernel"] == "is_k0_generic_nchw_f32"


def test_lds_tile_rule_matches_vulkan_table():
    """(tile_w + s - 1)(tile_h + r - 1) * channels * bytes reproduces the page's table."""
    for wx, wy, kb in _read_golden("vulkan_lds_tile_table.txt"):
        b = isa.is_lds_tile_bytes(int(wx), int(wy), 3, 3, 64, 2)
        assert b == float(kb) * 1024, (wx, wy, kb, b)
    assert isa.is_lds_tile_bytes(0, 8, 3, 3, 64, 2) == 0


def test_naive_traffic_model_matches_vulkan_table():
    rows = _read_golden("vulkan_naive_traffic_table.txt")
    total_in, total_reads = 0.0, 0.0
    for row in rows:
        if row[0] == "total":
            assert total_in == float(row[1]) and total_reads == float(row[2])
            continue
        _, cin, cin_p, cout, cout_p, kern, in_mb, reads_mb = row
        size, reads = traffic.naive_input_reads(720, 1280, int(cin_p), int(cout_p))
        # the page prints the input size rounded to MB (exact for layers 2-4)
        assert abs(size / traffic.MIB - float(in_mb)) < 0.5
        assert reads / traffic.MIB == pytest.approx(float(in_mb) * int(cout_p), abs=0.5 * int(cout_p))
        assert float(reads_mb) == float(in_mb) * int(cout_p)
        total_in += float(in_mb)
        total_reads += float(reads_mb)


def test_kepler_paper_formulas():
    # registers for n contiguous outputs of a KxK filter, K*(K+n-1): 3x3, n=2 -> 12
    assert traffic.special_case_registers(3, 2) == 12
    assert traffic.special_case_registers(5, 1) == 25
    # one thread owning W_T contiguous outputs reads (W_T+K-1)*K*C instead of W_T*K*K*C;
    # the ratio is (W_T+K-1)/(W_T*K)
    for wt, k, c in ((4, 3, 32), (8, 5, 16), (1, 3, 1)):
        a = traffic.shared_reads(wt, k, c, True)
        b = traffic.shared_reads(wt, k, c, False)
        assert a / b == pytest.approx((wt + k - 1) / (wt * k))


# ------------------------------------------------------------- LDS swizzle map
def _passes(words, banks=32):
    """Passes a warp access needs: the largest number of distinct words in one bank."""
    per_bank = {}
    for w in words:
        per_bank.setdefault(w % banks, set()).add(w)
    return max(len(v) for v in per_bank.values())


def test_swizzle_is_a_bijection_per_row():
    for nx, eb, cb in ((16, 4, 4), (32, 4, 4), (8, 4, 16), (64, 2, 16), (32, 2, 8), (128, 2, 16), (16, 8, 8)):
        for y in range(0, 70):
            cols = [isa.is_swizzle_col(y, x, nx, eb, cb) for x in range(nx)]
            assert sorted(cols) == list(range(nx)), (nx, eb, cb, y)
            # elements keep their offset inside a chunk
            per = cb // eb
            assert all(c % per == x % per for x, c in enumerate(cols))


def test_swizzle_spreads_columns_over_rows():
    """Property 3 of the page: for a fixed column, consecutive rows land in as many
    distinct swizzled columns as there are chunks in a row."""
    for nx, eb, cb in ((32, 4, 4), (16, 4, 4), (64, 2, 16)):
        chunks = nx * eb // cb
        per = cb // eb
        for x in range(nx):
            got = {isa.is_swizzle_col(y, x, nx, eb, cb) // per for y in range(chunks)}
            assert len(got) == chunks


def test_swizzle_rejects_bad_arguments():
    assert isa.is_swizzle_col(0, 0, 12, 4, 4) == -1      # nx not a power of two
    assert isa.is_swizzle_col(0, 0, 4, 4, 4) == -1       # row of 16 bytes < 32
    assert isa.is_swizzle_col(0, 16, 16, 4, 4) == -1     # x out of range
    assert isa.is_swizzle_col(0, 0, 16, 4, 2) == -1      # chunk smaller than element


def test_swizzle_worked_example():
    """The 32x16 and 32x32 float examples of the swizzling page (see the fixture)."""
    for rows, cols, eb, layout, access, passes in _read_golden("swizzle_32x16_example.txt"):
        rows, cols, eb, passes = int(rows), int(cols), int(eb), int(passes)

        def word(y, x):
            xs = isa.is_swizzle_col(y, x, cols, eb, eb) if layout == "swizzled" else x
            return y * cols + xs

        if access == "write":       # 32 consecutive values: rows 0.. of the array
            words = [word(t // cols, t % cols) for t in range(32)]
            got = _passes(words)
        else:                       # worst column over all columns
            got = max(_passes([word(y, x) for y in range(rows)]) for x in range(cols))
        assert got == passes, (rows, cols, layout, access, got, passes)


def test_separable_and_special_case_plans():
    """Separable filters: single channel fp32 only, square 3/5/7; counted work
    2 (R + S) per pixel. One channel with F filters and 1x1 layers go to the
    register-blocked kernel when F (or K) is even."""
    d = isa.make_desc(1, 1, 8192, 8192, 1, 7, 7, separable=True)
    info = isa.Plan(d).info()
    assert info["kernel"] == "is_k1_single_separable"
    assert info["flops"] == 2 * 14 * 8192 * 8192
    assert info["bytes"] == 4 * (2 * 8192 * 8192 + 14) + 4
    for bad in (isa.make_desc(1, 2, 64, 64, 1, 3, 3, separable=True),
                isa.make_desc(1, 1, 64, 64, 2, 3, 3, separable=True),
                isa.make_desc(1, 1, 64, 64, 1, 3, 5, separable=True),
                isa.make_desc(1, 1, 64, 64, 1, 9, 9, separable=True),
                isa.make_desc(1, 1, 64, 64, 1, 1, 1, separable=True),
                isa.make_desc(1, 1, 64, 64, 1, 3, 3, "f16", separable=True)):
        with pytest.raises(isa.ImgStencilError):
            isa.Plan(bad)
    weird = isa.make_desc(1, 1, 64, 64, 1, 3, 3)
    weird.separable = 2
    with pytest.raises(isa.ImgStencilError):
        isa.Plan(weird)
    # One channel with F filters: the multi-channel kernel, except two 5x5
    # filters on a large image, which take the single-channel kernel's
    # F-filter form with 64-row strips. Either way the other family is among
    # the tuning variants when it takes the shape.
    for (c, k, r) in ((1, 4, 3), (1, 8, 5), (1, 2, 1), (1, 6, 3), (1, 2, 5)):
        assert isa.Plan(isa.make_desc(1, c, 64, 128, k, r, r)).info()["kernel"] == "is_k2_multi", (c, k, r)
    for (k, r) in ((8, 3), (8, 1), (6, 3), (4, 5), (2, 1), (2, 3), (4, 1), (4, 3)):
        assert isa.Plan(isa.make_desc(1, 1, 4096, 4096, k, r, r)).info()["kernel"] == "is_k2_multi", (k, r)
    info = isa.Plan(isa.make_desc(1, 1, 4096, 4096, 2, 5, 5)).info()
    assert (info["kernel"], info["tile"], info["grid"]) == ("is_k1_single_fanout", (256, 64), (1024, 1, 1))
    vs = [(v["kernel"], v["param"]) for v in isa.conv2d_list_variants(isa.make_desc(1, 1, 4096, 4096, 8, 3, 3))]
    assert vs[0] == ("is_k2_multi", 8) and ("is_k1_single_fanout", 64) in vs
    vs = [(v["kernel"], v["param"]) for v in isa.conv2d_list_variants(isa.make_desc(1, 1, 4096, 4096, 2, 5, 5))]
    assert vs[0] == ("is_k1_single_fanout", 64) and ("is_k2_multi", 2) in vs
    assert "is_k1_single_fanout" not in [v["kernel"] for v in
                                         isa.conv2d_list_variants(isa.make_desc(1, 1, 4096, 4096, 4, 5, 5))]
    # 1x1 layers over several channels: the pointwise kernel when the planes
    # are whole 16-byte vectors (with the register-blocked kernel among the
    # tuning variants), else the multi-channel or fallback kernel
    for (c, k) in ((8, 16), (3, 4), (32, 32), (512, 8)):
        assert isa.Plan(isa.make_desc(1, c, 64, 128, k, 1, 1)).info()["kernel"] == "is_k8_pointwise", (c, k)
    vs = [(v["kernel"], v["param"]) for v in isa.conv2d_list_variants(isa.make_desc(1, 8, 64, 128, 16, 1, 1))]
    assert vs == [("is_k8_pointwise", 16), ("is_k8_pointwise", 8), ("is_k8_pointwise", 4),
                  ("is_k2_multi", 16), ("is_k2_multi", 8), ("is_k2_multi", 4)]
    # staged weights over 48 KB even at 4 channels per workgroup
    assert isa.Plan(isa.make_desc(1, 4000, 64, 128, 8, 1, 1)).info()["kernel"] == "is_k2_multi"
    assert isa.Plan(isa.make_desc(1, 8, 9, 30, 16, 1, 1)).info()["kernel"] == "is_k0_generic_nchw_f32"
    # one channel with 3 filters: no fan-out or register-blocked instance takes
    # it; the matrix-core form's 1-channel slabs do (16-byte or dword pixels)
    assert isa.Plan(isa.make_desc(1, 1, 64, 128, 3, 3, 3)).info()["kernel"] == "is_k2_multi_mfma"
    assert isa.Plan(isa.make_desc(1, 1, 64, 126, 3, 3, 3)).info()["kernel"] == "is_k2_multi_mfma"
    assert isa.Plan(isa.make_desc(1, 1, 64, 126, 3, 1, 1)).info()["kernel"] == "is_k0_generic_nchw_f32"


def test_tile_variants():
    """The tuning variants of a descriptor: the default plan first, then every
    other configuration that takes the shape; the fallback only when nothing
    else does. Each index creates a plan with that kernel and parameter."""
    def names(d):
        return [(v["kernel"], v["param"], v["is_default"]) for v in isa.conv2d_list_variants(d)]
    assert names(isa.make_desc(1, 1, 8192, 8192, 1, 3, 3)) == [
        ("is_k1_single", 64, True), ("is_k1_single", 4, False), ("is_k1_single", 8, False),
        ("is_k1_single", 16, False), ("is_k1_single", 32, False), ("is_k1_single", 128, False)]
    assert names(isa.make_desc(1, 32, 720, 1280, 32, 3, 3, "f32", True)) == [
        ("is_k5_mfma_f32", 0, True), ("is_k2_multi", 32, False), ("is_k2_multi", 16, False),
        ("is_k2_multi", 8, False), ("is_k2_multi", 4, False), ("is_k2_multi_mfma", 0, False)]
    # K a multiple of 4 over an even channel count from 4 on, 3x3 or 5x5: the
    # register-blocked kernel's products on the fp32 matrix cores (4 filters per
    # workgroup), its vector form among the variants; with 2 channels the vector
    # form is the plan and the matrix-core form a variant
    assert names(isa.make_desc(1, 32, 720, 1280, 4, 3, 3, "f32")) == [
        ("is_k2_multi_mfma", 0, True), ("is_k2_multi", 4, False)]
    assert names(isa.make_desc(2, 6, 40, 136, 4, 5, 5, "f32", True)) == [
        ("is_k2_multi_mfma", 0, True), ("is_k2_multi", 4, False), ("is_k2_multi", 2, False)]
    assert names(isa.make_desc(1, 8, 64, 128, 8, 3, 3, "f32")) == [
        ("is_k2_multi_mfma", 0, True), ("is_k2_multi", 8, False), ("is_k2_multi", 4, False)]
    assert names(isa.make_desc(1, 64, 64, 128, 32, 3, 3, "f32")) == [
        ("is_k2_multi_mfma", 0, True), ("is_k2_multi", 32, False), ("is_k2_multi", 16, False),
        ("is_k2_multi", 8, False), ("is_k2_multi", 4, False)]
    # 5x5 with 8 filters per group, which the vector form does not instantiate
    # over 4-channel slabs: the matrix-core form instead of the fallback
    assert names(isa.make_desc(1, 32, 64, 128, 8, 5, 5, "f32")) == [("is_k2_multi_mfma", 0, True)]
    assert names(isa.make_desc(1, 2, 64, 128, 8, 3, 3, "f32"))[0] == ("is_k2_multi", 8, True)
    assert ("is_k2_multi_mfma", 0, False) in names(isa.make_desc(1, 2, 64, 128, 8, 3, 3, "f32"))
    for (c, k, r, w) in ((3, 4, 3, 128), (2, 4, 3, 128), (8, 4, 9, 128), (8, 4, 1, 130)):
        assert isa.Plan(isa.make_desc(1, c, 64, w, k, r, r)).info()["kernel"] != "is_k2_multi_mfma", (c, k, r, w)
    # widths that are not whole 16-byte vectors: the matrix-core form's dword path
    for (c, k, r, w) in ((32, 4, 3, 130), (5, 3, 3, 126), (32, 32, 3, 30), (1, 32, 5, 70), (8, 8, 3, 13)):
        assert isa.Plan(isa.make_desc(1, c, 64, w, k, r, r)).info()["kernel"] == "is_k2_multi_mfma", (c, k, r, w)
    # any K: the last group of 4 filters masks the ones past K (an RGB output
    # layer 32 -> 3 took the one-thread-per-output fallback before); odd
    # channel counts that the vector form does not take (K = 3, 5x5 with 4
    # filters per group) get it over 1-channel slabs
    for (c, k, r) in ((32, 3, 3), (32, 1, 3), (6, 6, 3), (8, 7, 5), (4, 2, 3), (5, 3, 3), (3, 7, 5), (8, 8, 7),
                      (2, 16, 7), (3, 5, 7), (1, 4, 7)):
        info = isa.Plan(isa.make_desc(2, c, 40, 136, k, r, r)).info()
        assert info["kernel"] == "is_k2_multi_mfma" and info["grid"][0] == 2 * 3 * 3 * ((k + 3) // 4), (c, k, r, info)
    # odd channel counts, 3x3: the vector form with at most 16 filters per workgroup
    assert names(isa.make_desc(1, 3, 720, 1280, 32, 3, 3, "f32"))[0] == ("is_k2_multi", 16, True)
    assert ("is_k2_multi_mfma", 0, False) in names(isa.make_desc(1, 3, 720, 1280, 32, 3, 3, "f32"))
    assert names(isa.make_desc(1, 2, 720, 1280, 32, 3, 3, "f32"))[0] == ("is_k2_multi", 16, True)
    # 5x5 from 2 channels whatever the parity: the matrix-core form
    for c in (2, 3, 7):
        assert names(isa.make_desc(1, c, 720, 1280, 16, 5, 5, "f32"))[0] == ("is_k2_multi_mfma", 0, True), c
    assert "is_k2_multi_mfma" not in [n[0] for n in names(isa.make_desc(1, 1, 8192, 8192, 1, 3, 3))]
    assert isa.Plan(isa.make_desc(1, 5, 40, 136, 3, 3, 3)).info()["lds_bytes"] == 4 * 576 * 16
    assert isa.Plan(isa.make_desc(1, 8, 40, 136, 8, 7, 7)).info()["lds_bytes"] == 4 * 576 * 16   # 1-channel slabs
    # a plan that only the last resort takes is variant 0 and re-creates as itself
    assert names(isa.make_desc(1, 1, 64, 128, 4, 7, 7)) == [("is_k2_multi_mfma", 0, True)]
    assert isa.Plan(isa.make_desc(1, 1, 64, 128, 4, 7, 7), variant=0).info()["kernel"] == "is_k2_multi_mfma"
    assert isa.Plan(isa.make_desc(1, 32, 720, 1280, 4, 3, 3, "f32")).info()["lds_bytes"] == 53248
    assert names(isa.make_desc(8, 64, 256, 256, 64, 3, 3, "f16")) == [
        ("is_k4_mfma", 128, True), ("is_k4_mfma", 0, False), ("is_k4_mfma", 256, False)]
    assert names(isa.make_desc(1, 64, 72, 128, 32, 3, 3, "f16")) == [("is_k4_mfma", 128, True)]
    # fp16 MFMA units are 64 rows (32 for 16 outputs), or 60 (30) where that computes fewer rows (720)
    for (h, c, k, th) in ((256, 64, 64, 64), (720, 64, 64, 60), (720, 64, 32, 60), (720, 32, 16, 30),
                          (720, 32, 32, 60), (256, 32, 16, 32), (256, 32, 32, 64), (90, 32, 16, 30),
                          (1080, 64, 64, 60), (64, 64, 64, 64)):
        assert isa.Plan(isa.make_desc(1, c, h, 1280, k, 3, 3, "f16")).info()["tile"][1] == th, (h, c, k)
    # other swizzles keep 64-row units
    d720 = isa.make_desc(1, 64, 720, 1280, 64, 3, 3, "f16")
    assert [isa.Plan(d720, variant=i).info()["tile"][1] for i in range(3)] == [60, 64, 64]
    assert names(isa.make_desc(1, 1, 720, 1280, 64, 5, 5, "f16", True)) == [("is_k6_head_f16", 0, True)]
    # one channel to 16/32/64 fp32 outputs, 3x3 or 5x5: the fp32 MFMA first layer, the
    # register-blocked kernel's groups as variants; not for widths that are not whole vectors
    assert names(isa.make_desc(1, 1, 720, 1280, 32, 5, 5, "f32", True)) == [
        ("is_k9_head_f32", 0, True), ("is_k2_multi", 32, False), ("is_k2_multi", 16, False),
        ("is_k2_multi", 8, False), ("is_k2_multi", 4, False), ("is_k2_multi", 2, False)]
    assert isa.Plan(isa.make_desc(1, 1, 720, 1282, 32, 5, 5)).info()["kernel"] != "is_k9_head_f32"
    assert isa.Plan(isa.make_desc(1, 1, 720, 1280, 32, 7, 7)).info()["kernel"] != "is_k9_head_f32"
    assert isa.Plan(isa.make_desc(1, 1, 720, 1280, 8, 5, 5)).info()["kernel"] == "is_k2_multi"
    assert names(isa.make_desc(1, 3, 16, 30, 5, 3, 3)) == [("is_k2_multi_mfma", 0, True)]
    assert names(isa.make_desc(1, 3, 16, 30, 5, 1, 1)) == [("is_k0_generic_nchw_f32", 0, True)]
    sep = names(isa.make_desc(1, 1, 512, 512, 1, 7, 7, separable=True))
    assert {k for (k, _, _) in sep} == {"is_k1_single_separable"} and len(sep) == 6
    d = isa.make_desc(1, 1, 4096, 4096, 8, 3, 3)
    vs = isa.conv2d_list_variants(d)
    assert [(v["kernel"], v["param"]) for v in vs] == [("is_k2_multi", 8), ("is_k1_single_fanout", 4),
                                                       ("is_k1_single_fanout", 8), ("is_k1_single_fanout", 16),
                                                       ("is_k1_single_fanout", 32), ("is_k1_single_fanout", 64),
                                                       ("is_k1_single_fanout", 128), ("is_k2_multi", 4),
                                                       ("is_k2_multi", 2)]
    for i, v in enumerate(vs):
        p = isa.Plan(d, variant=i)
        info = p.info()
        assert info["kernel"] == v["kernel"]
        if v["kernel"] == "is_k2_multi":
            assert info["grid"][0] == 64 * 256 * (8 // v["param"])   # 64x16 tiles x channel groups
        else:
            assert info["grid"][0] == 16 * (4096 // v["param"])      # 256-column segments x strips
    with pytest.raises(isa.ImgStencilError):
        isa.Plan(d, variant=len(vs))
    with pytest.raises(isa.ImgStencilError):
        isa.Plan(d, variant=-1)
    # Tuning checks its arguments before touching the GPU.
    p = isa.Plan(d)
    n = ctypes.c_int()
    lib = isa.load()
    assert lib.conv2d_autotune(p.handle, 0x1000, 0x2000, None, 0x100000000, None, 0, None, 0,
                               ctypes.byref(n)) == _abi.IS_ERR_INVALID_ARG          # reps < 1
    assert lib.conv2d_autotune(p.handle, 0x1004, 0x2000, None, 0x100000000, None, 3, None, 0,
                               ctypes.byref(n)) == _abi.IS_ERR_MISALIGNED
    assert lib.conv2d_autotune(p.handle, None, 0x2000, None, 0x100000000, None, 3, None, 0,
                               ctypes.byref(n)) == _abi.IS_ERR_INVALID_ARG          # null x
    assert lib.conv2d_autotune(p.handle, 0x1000, 0x2000, None, 0x1000, None, 3, None, 0,
                               ctypes.byref(n)) == _abi.IS_ERR_INVALID_ARG          # x and y overlap
    assert lib.conv2d_autotune(None, 0x1000, 0x2000, None, 0x100000000, None, 3, None, 0,
                               ctypes.byref(n)) == _abi.IS_ERR_INVALID_ARG          # null plan


def _stencil(h, w, rs, mode=None, n=1):
    mode = isa.IS_CHAIN_AUTO if mode is None else mode
    return isa.make_chain_desc(n, h, w, [(1, 1, r, False) for r in rs], 1, mode)


def test_stencil_pipeline_grouping():
    """Chains of single-channel filters: the model fuses layers when the saved
    intermediate traffic outweighs the recomputed overlap; 7x7 layers and
    widths that are not a multiple of 4 are never fused; groups hold at most
    3 layers; the workspace holds one image per group boundary, at most two."""
    img = 4 * 8192 * 8192
    cases = [
        ((8192, 8192, [3, 3]), None, [2], "is_k7_fused_stencil", 0),
        ((8192, 8192, [3, 3]), isa.IS_CHAIN_UNFUSED, [1, 1], "layer_by_layer", img),
        ((8192, 8192, [3, 3]), isa.IS_CHAIN_FUSED, [2], "is_k7_fused_stencil", 0),
        ((8192, 8192, [5, 5, 5]), None, [3], "is_k7_fused_stencil", 0),
        ((8192, 8192, [3] * 7), None, [3, 3, 1], "fused_groups:3+3+1", 2 * img),
        ((8192, 8192, [7, 7]), None, [1, 1], "layer_by_layer", img),
        ((8192, 8192, [5, 3, 7, 3, 3]), None, [2, 1, 2], "fused_groups:2+1+2", 2 * img),
        ((8192, 8192, [7, 3]), None, [2], "is_k7_fused_stencil", 0),
        ((8192, 8192, [7, 5]), None, [1, 1], "layer_by_layer", img),
        ((8192, 8192, [7, 3, 7, 3]), None, [1, 3], "fused_groups:1+3", img),
        ((8192, 8190, [3, 3]), None, [1, 1], "layer_by_layer", 4 * 8192 * 8190),
        ((16, 16, [3, 3]), None, [2], "is_k7_fused_stencil", 0),
        ((8192, 8192, [3]), None, [1], "layer_by_layer", 0),
    ]
    for (h, w, rs), mode, groups, name, ws in cases:
        d = _stencil(h, w, rs, mode)
        assert isa.conv_chain_groups(d) == groups, (h, w, rs, mode)
        assert isa.conv_chain_kernel_name(d) == name, (h, w, rs, mode)
        assert isa.conv_chain_workspace_size(d) == ws, (h, w, rs, mode)
    for rs in ([3, 3, 3, 3], [7, 7], [7, 3, 7], [3]):
        with pytest.raises(isa.ImgStencilError):
            isa.conv_chain_groups(_stencil(64, 64, rs, isa.IS_CHAIN_FUSED))
    for rs in ([7, 3], [3, 7], [7, 5], [3, 3, 7]):
        assert isa.conv_chain_groups(_stencil(64, 64, rs, isa.IS_CHAIN_FUSED)) == [len(rs)]
    # the upscaling chain is not a stencil pipeline: layer by layer, or its own fused kernel
    spec = [(1, 32, 5, True), (32, 32, 3, True), (32, 32, 3, True), (32, 4, 3, False)]
    assert isa.conv_chain_groups(isa.make_chain_desc(1, 720, 1280, spec, 2, isa.IS_CHAIN_AUTO)) == [1, 1, 1, 1]
    assert isa.conv_chain_groups(isa.make_chain_desc(1, 720, 1280, spec, 2, isa.IS_CHAIN_FUSED)) == [4]


def test_chain_descriptor_checks():
    d = isa.make_chain_desc(1, 16, 16, [(1, 8, 5, True), (8, 4, 3, False)], depth_to_space=2)
    ws = isa.conv_chain_workspace_size(d)
    assert ws >= 2 * 4 * 8 * 16 * 16
    assert isa.conv_chain_kernel_name(d) in ("layer_by_layer", "is_k3_chain")
    bad = isa.make_chain_desc(1, 16, 16, [(1, 8, 5, True), (7, 4, 3, False)])
    with pytest.raises(isa.ImgStencilError):
        isa.conv_chain_workspace_size(bad)
    bad = isa.make_chain_desc(1, 16, 16, [(1, 8, 5, True), (8, 3, 3, False)], depth_to_space=2)
    with pytest.raises(isa.ImgStencilError):
        isa.conv_chain_workspace_size(bad)
    one = isa.make_chain_desc(1, 16, 16, [(1, 4, 3, False)], depth_to_space=1,
                              mode=isa.IS_CHAIN_UNFUSED)
    assert isa.conv_chain_workspace_size(one) == 0
    # the upscaling chain: AUTO asks for the layer-by-layer workspace, FUSED for none
    spec = [(1, 32, 5, True), (32, 32, 3, True), (32, 32, 3, True), (32, 4, 3, False)]
    auto = isa.make_chain_desc(1, 720, 1280, spec, 2, isa.IS_CHAIN_AUTO)
    assert isa.conv_chain_workspace_size(auto) == 2 * 4 * 32 * 720 * 1280
    assert isa.conv_chain_kernel_name(auto) == "layer_by_layer"
    fused = isa.make_chain_desc(1, 720, 1280, spec, 2, isa.IS_CHAIN_FUSED)
    assert isa.conv_chain_workspace_size(fused) == 0
    assert isa.conv_chain_kernel_name(fused) == "is_k3_chain"


def test_f16_chain_descriptor_checks():
    """The pages' net in fp16 storage: two ping-pong buffers of the widest
    layer (64 channels, 2 bytes), depth-to-space by 3 of the 9 channels, and
    layer by layer only."""
    spec = [(1, 64, 5, True), (64, 64, 3, True), (64, 32, 3, True), (32, 9, 3, False)]
    d = isa.make_chain_desc(1, 720, 1280, spec, 3, isa.IS_CHAIN_AUTO, "f16")
    assert isa.conv_chain_workspace_size(d) == 2 * 2 * 64 * 720 * 1280
    # AUTO: the first two layers in one launch; UNFUSED: one launch per layer
    assert isa.conv_chain_kernel_name(d) == "head_fused"
    assert isa.conv_chain_groups(d) == [2, 1, 1]
    du = isa.make_chain_desc(1, 720, 1280, spec, 3, isa.IS_CHAIN_UNFUSED, "f16")
    assert isa.conv_chain_kernel_name(du) == "layer_by_layer"
    assert isa.conv_chain_groups(du) == [1, 1, 1, 1]
    assert isa.conv_chain_workspace_size(du) == isa.conv_chain_workspace_size(d)
    # only a 1 -> 64 3x3 or 5x5 layer followed by 64 -> 64 3x3 is fused
    for first, second in (((1, 64, 3, True), (64, 64, 3, True)), ((1, 64, 5, False), (64, 64, 3, False))):
        assert isa.conv_chain_kernel_name(isa.make_chain_desc(1, 40, 64, [first, second], 1, isa.IS_CHAIN_AUTO,
                                                              "f16")) == "head_fused"
    for first, second in (((1, 32, 5, True), (32, 32, 3, True)), ((1, 64, 7, True), (64, 64, 3, True)),
                          ((1, 64, 5, True), (64, 32, 3, True))):
        assert isa.conv_chain_kernel_name(isa.make_chain_desc(1, 40, 64, [first, second], 1, isa.IS_CHAIN_AUTO,
                                                              "f16")) == "layer_by_layer"
    assert round(traffic.chain_flops(1, 720, 1280, [t[:3] for t in spec]) / 1e9, 2) == 109.65
    for mode in (isa.IS_CHAIN_FUSED,):
        with pytest.raises(isa.ImgStencilError):
            isa.conv_chain_workspace_size(isa.make_chain_desc(1, 720, 1280, spec, 3, mode, "f16"))
    with pytest.raises(isa.ImgStencilError):       # 9 channels do not make a 2x2 block
        isa.conv_chain_workspace_size(isa.make_chain_desc(1, 720, 1280, spec, 2, isa.IS_CHAIN_AUTO, "f16"))
    with pytest.raises(isa.ImgStencilError):       # factors 1 to 3 only
        isa.conv_chain_workspace_size(isa.make_chain_desc(1, 8, 8, [(1, 16, 3, False)], 4,
                                                          isa.IS_CHAIN_AUTO, "f16"))
    # a 32 -> 4 last layer before depth-to-space runs as 16 channels (4 of them
    # real) in the workspace; a 2 -> 4 one keeps its 4 channels
    def ws_f16(spec, f):
        return isa.conv_chain_workspace_size(isa.make_chain_desc(1, 10, 10, spec, f, isa.IS_CHAIN_AUTO, "f16"))
    assert ws_f16([(1, 32, 3, True), (32, 4, 3, False)], 2) == 2 * 6400
    assert ws_f16([(1, 2, 3, True), (2, 4, 3, False)], 2) == 2 * 1024
    # the first layer (one input channel) has its own fp16 kernel
    for k, r in ((64, 5), (32, 3), (16, 5)):
        info = isa.Plan(isa.make_desc(1, 1, 720, 1280, k, r, r, "f16", True)).info()
        assert info["kernel"] == "is_k6_head_f16"
        assert info["tile"] == (64, 32)
    assert isa.Plan(isa.make_desc(1, 1, 72, 128, 8, 3, 3, "f16", True)).info()["kernel"] != "is_k6_head_f16"


def test_persistent_grid_sizing():
    """Persistent kernels launch one workgroup per CU of the device, in a
    multiple of 8 (their units are dealt to 8 groups, one per XCD), fewer when
    the units need fewer."""
    g = isa.is_persistent_grid
    assert g(256, 256) == 256 and g(2240, 256) == 256      # 8x256x256 fp16 layer; 1280x720 fp32 layer
    assert g(100, 256) == 104 and g(3, 256) == 8 and g(1, 256) == 8
    assert g(1000, 80) == 80 and g(1000, 84) == 80 and g(1000, 32) == 32   # partitioned devices
    assert g(1000, 4) == 8 and g(9, 80) == 16
    assert g(0, 256) == 0 and g(5, 0) == 0
    for cus in (8, 32, 38, 80, 256, 304):
        for units in range(1, 400, 7):
            v = g(units, cus)
            assert v % 8 == 0 and 8 <= v <= max(8, cus // 8 * 8)
            assert v >= min(units, cus // 8 * 8) or v == 8
    # plans record the grid for 256 CUs
    p = isa.Plan(isa.make_desc(8, 64, 256, 256, 64, 3, 3, "f16"))
    assert p.info()["kernel"] == "is_k4_mfma" and p.info()["grid"][0] == 256
    p = isa.Plan(isa.make_desc(1, 64, 20, 40, 64, 3, 3, "f16"))
    assert p.info()["grid"][0] == g(p.info()["grid"][0], 256) == 8


def test_single_channel_kernel_keeps_32_bit_row_offsets():
    """The single-channel kernel's row offsets are 32-bit: its plans stop where
    4 (W + 256) reaches 2^31, and wider rows go to another kernel."""
    edge = (1 << 29) - 256
    assert isa.Plan(isa.make_desc(1, 1, 2, edge - 4, 1, 3, 3)).info()["kernel"] == "is_k1_single"
    for W in (edge, 1 << 29, 1 << 30):
        d = isa.make_desc(1, 1, 2, W, 1, 3, 3)
        assert isa.Plan(d).info()["kernel"] != "is_k1_single"
        assert all(not v["kernel"].startswith("is_k1_single") for v in isa.conv2d_list_variants(d))


def test_no_environment_variable_changes_a_plan():
    """Only IMGSTENCIL_LOG is read from the environment (logging); layouts and
    tiles come from the descriptor or a tuning variant."""
    srcs = [os.path.join(ROOT, "image_stencil_amd", "csrc", f)
            for f in os.listdir(os.path.join(ROOT, "image_stencil_amd", "csrc"))]
    names = set()
    for f in srcs:
        names |= set(re.findall(r'getenv\("([A-Z_0-9]+)"\)', open(f).read()))
    assert names <= {"IMGSTENCIL_LOG"}


def test_binding_rejects_mismatched_arguments():
    """conv2d / conv_chain check dtypes, channel counts, bias lengths and square
    chain filters before anything reaches the library (CPU tensors suffice:
    these checks come before the device check)."""
    import torch
    x = torch.zeros(1, 4, 8, 8)
    w = torch.zeros(4, 4, 3, 3)
    with pytest.raises(TypeError):
        isa.conv2d(x.double(), w.double())
    with pytest.raises(TypeError):
        isa.conv2d(x.bfloat16(), w.bfloat16())
    with pytest.raises(TypeError):
        isa.conv2d(x, w.half())
    with pytest.raises(ValueError):
        isa.conv2d(x[:, :3].contiguous(), w)               # 3 channels, weights for 4
    with pytest.raises(ValueError):
        isa.conv2d(x, w, torch.zeros(3))                   # bias for 3 of 4 outputs
    with pytest.raises(TypeError):
        isa.conv2d(x, w, torch.zeros(4, dtype=torch.float64))
    with pytest.raises(ValueError):
        isa.conv2d(x[0], w)                                # not 4-D
    with pytest.raises(TypeError, match="device tensor"):
        isa.conv2d(x, w)                                   # well formed: only the device check fails
    xc = torch.zeros(1, 1, 8, 8)
    l1 = (torch.zeros(8, 1, 5, 5), torch.zeros(8), True)
    l2 = (torch.zeros(4, 8, 3, 3), torch.zeros(4), False)
    with pytest.raises(ValueError):
        isa.conv_chain(torch.zeros(1, 2, 8, 8), [l1, l2])  # 2 input channels, layer 1 takes 1
    with pytest.raises(ValueError):
        isa.conv_chain(xc, [l1, (torch.zeros(4, 6, 3, 3), None, False)])   # 8 channels into a 6-channel layer
    with pytest.raises(ValueError):
        isa.conv_chain(xc, [(torch.zeros(8, 1, 5, 3), None, True)])       # not square
    with pytest.raises(ValueError):
        isa.conv_chain(xc, [(l1[0], torch.zeros(7), True), l2])          # short bias
    with pytest.raises(ValueError):
        isa.conv_chain(xc, [])
    with pytest.raises(TypeError):
        isa.conv_chain(xc.half(), [l1, l2])                 # fp16 input, fp32 weights
    with pytest.raises(TypeError, match="device tensor"):
        isa.conv_chain(xc, [l1, l2], depth_to_space=2)
    with pytest.raises(ValueError):
        isa.conv2d_separable(x, torch.zeros(3), torch.zeros(3))   # 4 channels


def test_offset_limits_of_every_kernel():
    """Each kernel's plan takes the largest image its 32-bit buffer offsets
    allow and gives the next larger width to another kernel (the GPU tests run
    the widths that are taken)."""
    def kernel(*desc):
        return isa.Plan(isa.make_desc(*desc)).info()["kernel"]
    cases = [  # (desc at the limit, desc one step wider, kernel)
        ((1, 32, 3840, 4068, 32, 3, 3, "f32", True), (1, 32, 3840, 4072, 32, 3, 3, "f32", True), "is_k5_mfma_f32"),
        ((1, 64, 5000, 6248, 64, 3, 3, "f16"), (1, 64, 5000, 6252, 64, 3, 3, "f16"), "is_k4_mfma"),
        ((1, 1, 3840, 4068, 32, 5, 5, "f32", True), (1, 1, 3840, 4072, 32, 5, 5, "f32", True), "is_k9_head_f32"),
        ((1, 32, 5000, 6248, 4, 3, 3, "f32", True), (1, 32, 5000, 6252, 4, 3, 3, "f32", True), "is_k2_multi_mfma"),
        ((1, 1, 5000, 6248, 64, 5, 5, "f16", True), (1, 1, 5000, 6252, 64, 5, 5, "f16", True), "is_k6_head_f16"),
    ]
    for at, past, name in cases:
        assert kernel(*at) == name, (at, kernel(*at))
        assert kernel(*past) != name, (past, kernel(*past))
    pipe = [(1, 1, 3, True), (1, 1, 3, True), (1, 1, 3, False)]
    assert isa.conv_chain_kernel_name(isa.make_chain_desc(1, 20000, 24996, pipe, 1, isa.IS_CHAIN_AUTO)) == \
        "is_k7_fused_stencil"
    assert isa.conv_chain_groups(isa.make_chain_desc(1, 20000, 25000, pipe, 1, isa.IS_CHAIN_AUTO)) == [1, 1, 1]
    up = [(1, 32, 5, True), (32, 32, 3, True), (32, 32, 3, True), (32, 4, 3, False)]
    assert isa.conv_chain_kernel_name(isa.make_chain_desc(1, 15000, 16664, up, 2, isa.IS_CHAIN_FUSED)) == "is_k3_chain"
    with pytest.raises(isa.ImgStencilError):
        isa.conv_chain_kernel_name(isa.make_chain_desc(1, 15000, 16668, up, 2, isa.IS_CHAIN_FUSED))
