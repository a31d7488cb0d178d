"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every symbol the header declares, the header compiles as C and C++, every
argument-validation status code is reachable, the kernels build without
register spills, and the product path does not touch the oracle."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")
PKG = os.path.join(ROOT, "moe_grouped_matmul_amd")


@pytest.fixture(scope="module")
def lib():
    from moe_grouped_matmul_amd import dg

    if not os.path.exists(dg.LIB_PATH):
        from moe_grouped_matmul_amd import build

        build.build()
    return dg.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("dg_fp8_gemm_nt", "dg_m_grouped_fp8_gemm_nt_contiguous", "dg_m_grouped_fp8_gemm_nt_masked",
              "dg_quant_1x128", "dg_quant_128x128"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dg_\w+)", out))
    assert set(_declared()) <= exported


@pytest.mark.parametrize("compiler,lang", [("gcc", "c"), ("g++", "c++")])
def test_header_compiles(compiler, lang, tmp_path):
    src = tmp_path / ("t." + ("c" if lang == "c" else "cpp"))
    src.write_text('#include "dg.h"\nint main(void){ return dg_get_m_alignment_for_contiguous_layout() == 128 ? 0 : 1; }\n')
    r = subprocess.run([compiler, "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.join(ROOT, "include"), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


# fake, never-dereferenced device addresses: every call below fails validation
# before any device work is attempted
P16 = 0x10000
P4 = 0x10004


def _err(lib):
    return lib.dg_get_last_error().decode()


def test_status_codes_from_host(lib):
    from moe_grouped_matmul_amd import dg

    s = ctypes.c_void_p(0)
    gemm = lib.dg_fp8_gemm_nt
    # shape errors
    assert gemm(P16, P16, P16, P16, P16, 64, 2112, 7000, None, 0, s) == dg.DG_ERR_SHAPE and "K" in _err(lib)
    assert gemm(P16, P16, P16, P16, P16, 64, 2110, 7168, None, 0, s) == dg.DG_ERR_SHAPE and "N" in _err(lib)
    assert gemm(P16, P16, P16, P16, P16, -1, 2112, 7168, None, 0, s) == dg.DG_ERR_SHAPE
    # zero rows: nothing to do
    assert gemm(None, None, None, None, None, 0, 2112, 7168, None, 0, s) == dg.DG_OK and _err(lib) == ""
    # null / alignment / workspace
    assert gemm(None, P16, P16, P16, P16, 64, 2112, 7168, None, 0, s) == dg.DG_ERR_INVALID_ARG
    assert gemm(P16 + 8, P16, P16, P16, P16, 64, 2112, 7168, None, 0, s) == dg.DG_ERR_ALIGN
    assert gemm(P16, P16 + 2, P16, P16, P16, 64, 2112, 7168, None, 0, s) == dg.DG_ERR_ALIGN
    assert gemm(P16, P16, P16, P16, P16, 64, 2112, 7168, P4, 64, s) == dg.DG_ERR_WORKSPACE
    assert gemm(P16, P16, P16, P16, P16, 64, 2112, 7168, P16, 6, s) == dg.DG_ERR_WORKSPACE
    contig = lib.dg_m_grouped_fp8_gemm_nt_contiguous
    assert contig(P16, P16, P16, P16, P16, P16, 256, 128, 256, 0, None, 0, s) == dg.DG_ERR_SHAPE
    assert contig(P16, P16, P16, P16, P16, None, 256, 128, 256, 2, None, 0, s) == dg.DG_ERR_INVALID_ARG
    assert contig(P16, P16, P16, P16, P16, P16 + 2, 256, 128, 256, 2, None, 0, s) == dg.DG_ERR_ALIGN
    # G beyond 1024 groups, and one expert's weights of 4 GiB or more
    assert contig(P16, P16, P16, P16, P16, P16, 256, 128, 256, 1025, None, 0, s) == dg.DG_ERR_SHAPE and "G" in _err(lib)
    assert contig(P16, P16, P16, P16, P16, P16, 256, 1 << 19, 8192, 2, None, 0, s) == dg.DG_ERR_SHAPE
    assert "4 GiB" in _err(lib)
    masked = lib.dg_m_grouped_fp8_gemm_nt_masked
    assert masked(P16, P16, P16, P16, P16, P16, 1025, 256, 128, 256, 0, None, 0, s) == dg.DG_ERR_SHAPE
    assert masked(P16, P16, P16, P16, P16, P16, 2, 256, 1 << 19, 8192, 0, None, 0, s) == dg.DG_ERR_SHAPE
    assert "4 GiB" in _err(lib)
    # one expert's rows past 32-bit offsets (max_m * K or max_m * N * 2 bytes)
    assert masked(P16, P16, P16, P16, P16, P16, 2, 1 << 20, 4096, 8192, 0, None, 0, s) == dg.DG_ERR_SHAPE
    assert masked(P16, P16, P16, P16, P16, P16, 0, 256, 128, 256, 0, None, 0, s) == dg.DG_ERR_SHAPE
    assert masked(P16, P16, P16, P16, P16, P16, 4, -1, 128, 256, 0, None, 0, s) == dg.DG_ERR_SHAPE
    assert masked(None, None, None, None, None, None, 4, 0, 128, 256, 0, None, 0, s) == dg.DG_OK
    assert masked(P16, P16, P16, P16, P16, None, 4, 8, 128, 256, 0, None, 0, s) == dg.DG_ERR_INVALID_ARG
    kg = lib.dg_k_grouped_fp8_gemm_nt_contiguous
    # (A, sfa, B, sfb, C, D, ks, G, M, N, K, ws, ws_bytes, stream)
    assert kg(P16, P16, P16, P16, None, P16, P16, 0, 256, 128, 256, None, 0, s) == dg.DG_ERR_SHAPE
    assert kg(P16, P16, P16, P16, None, P16, P16, 1025, 256, 128, 256, None, 0, s) == dg.DG_ERR_SHAPE
    assert kg(P16, P16, P16, P16, None, P16, P16, 2, 256, 128, 200, None, 0, s) == dg.DG_ERR_SHAPE
    assert kg(P16, P16, P16, P16, None, P16, P16, 2, -1, 128, 256, None, 0, s) == dg.DG_ERR_SHAPE
    assert kg(None, None, None, None, None, None, None, 2, 0, 128, 256, None, 0, s) == dg.DG_OK
    assert kg(P16, P16, P16, P16, None, P16, None, 2, 256, 128, 256, None, 0, s) == dg.DG_ERR_INVALID_ARG
    assert kg(P16, P16, P16, P16, P16 + 4, P16, P16, 2, 256, 128, 256, None, 0, s) == dg.DG_ERR_ALIGN
    assert kg(P16, P16, P16, P16, None, P16, P16 + 2, 2, 256, 128, 256, None, 0, s) == dg.DG_ERR_ALIGN
    assert kg(P16, P16, P16, P16, None, P16, P16, 2, 1 << 20, 4096, 4096, None, 0, s) == dg.DG_ERR_SHAPE
    # dense forms: weights of 4 GiB or more; rows too long for one tile of
    # 32-bit offsets; K split into row chunks otherwise (no status code)
    assert gemm(P16, P16, P16, P16, P16, 64, 1 << 19, 8192, None, 0, s) == dg.DG_ERR_SHAPE and "4 GiB" in _err(lib)
    assert lib.dg_fp8_gemm_nt_acc(P16, P16, P16, P16, None, P16, 64, 1 << 19, 8192, None, 0, s) == dg.DG_ERR_SHAPE
    assert lib.dg_fp8_gemm_nt_ue8m0(P16, P16, P16, P16, P16, 64, 1 << 19, 8192, None, 0, s) == dg.DG_ERR_SHAPE
    assert lib.dg_bf16_gemm_nt(P16, P16, P16, 64, 1 << 18, 8192, None, 0, s) == dg.DG_ERR_SHAPE
    assert gemm(P16, P16, P16, P16, P16, 64, 16, 1 << 24, None, 0, s) == dg.DG_ERR_SHAPE
    q1 = lib.dg_quant_1x128
    assert q1(P16, P16, P16, 1, 4, 100, s) == dg.DG_ERR_SHAPE
    assert q1(None, P16, P16, 1, 4, 128, s) == dg.DG_ERR_INVALID_ARG
    assert q1(P16, P16 + 4, P16, 1, 4, 128, s) == dg.DG_ERR_ALIGN
    assert q1(P16, P16, P16, 1, 0, 128, s) == dg.DG_OK
    # launch grid (ceil(M / 16) * (K / 128), G): each dimension's limit
    assert q1(P16, P16, P16, 65536, 4, 128, s) == dg.DG_ERR_SHAPE
    assert q1(P16, P16, P16, 1, 1 << 28, 1 << 14, s) == dg.DG_ERR_SHAPE
    assert q1(P16, P16, P16, 1, (1 << 31) - 15, 128, s) == dg.DG_ERR_SHAPE
    assert lib.dg_quant_1x128_ue8m0(P16, P16, P16, 65536, 4, 128, s) == dg.DG_ERR_SHAPE
    q2 = lib.dg_quant_128x128
    assert q2(P16, P16, P16, 1, 4, 130, s) == dg.DG_ERR_SHAPE
    assert q2(P16, P16, P16 + 1, 1, 4, 128, s) == dg.DG_ERR_ALIGN


def test_no_device_status_on_cpu_host(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device path only")
    from moe_grouped_matmul_amd import dg

    rc = lib.dg_fp8_gemm_nt(P16, P16, P16, P16, P16, 64, 2112, 7168, None, 0, ctypes.c_void_p(0))
    assert rc == dg.DG_ERR_DEVICE and _err(lib)
    assert lib.dg_get_num_cus() == 0


def test_utilities(lib):
    assert lib.dg_get_m_alignment_for_contiguous_layout() == 128
    assert lib.dg_version().decode().startswith("dg-mi355x")
    assert lib.dg_set_num_cus(64) == 0
    assert lib.dg_set_num_cus(0) == 0
    # dense small-M shapes ask for split-K scratch; large ones only when the
    # 256 x 128 tiles they run leave a partial last round on the (default 256)
    # CUs, whose tail tiles are then split along K: 4096x2112 -> 16 x 17 = 272
    # tiles, 16 tail tiles in 4 pieces of 256x128 fp32 partials after the
    # 4 KiB counter area; 256 x 256 tiles (4096x7168, 4096x4096) need none
    assert lib.dg_get_workspace_size(0, 64, 2112, 7168, 1) > 0
    assert lib.dg_set_num_cus(256) == 0  # the MI355X count, also when no device is visible
    assert lib.dg_get_workspace_size(0, 4096, 2112, 7168, 1) == 4096 + 16 * 4 * 256 * 128 * 4
    assert lib.dg_get_workspace_size(0, 4096, 7168, 16384, 1) == 0
    assert lib.dg_get_workspace_size(0, 4096, 4096, 7168, 1) == 0  # 256 x 256 tiles: whole rounds
    assert lib.dg_set_num_cus(0) == 0
    assert lib.dg_get_workspace_size(2, 256, 4096, 7168, 32) == 0


def test_kernels_have_no_register_spills(lib):
    report = os.path.join(PKG, "_build", "resource_usage.txt")
    if not os.path.exists(report):
        from moe_grouped_matmul_amd import build

        build.build()
    text = open(report).read()
    sizes = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
    assert sizes, "no resource-usage remarks recorded"
    assert all(s == 0 for s in sizes), text


def test_product_path_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", src, flags=re.M), f
                assert "import_module(\"oracle" not in src and "/oracle/" not in src, f


def test_dense_planner_choice(lib):
    # host logic only: 256 x 256 tiles when they fill whole rounds of the CUs
    # to >= 85%, else 256 x 128 tiles with a K-split tail; M <= 128 skinny
    from moe_grouped_matmul_amd import dg

    try:
        dg.dg_set_num_cus(256)
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 4096, 7168, 16384)      # 448 tiles: 0.875
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 4096, 4096, 7168)       # 256 tiles: 1.0
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 4096, 2112, 7168)  # 144 tiles: 0.56
        # one round of 256 x 256 tiles on >= 60% of the CUs: the fp8 forms take it, BF16 does not
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 2560, 4096, 2048)       # 160 tiles: 0.625
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT_UE8M0, 2560, 4096, 2048)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_BF16_GEMM_NT, 2560, 4096, 2048)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 8192, 2112, 7168)  # 288 tiles: 2 rounds
        # UE8M0 scales: the same 256 x 256 rule (no workspace needed there), else 256 x 128 tiles
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT_UE8M0, 4096, 7168, 16384)
        assert dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT_UE8M0, 4096, 7168, 16384) == 0
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT_UE8M0, 4096, 2112, 7168)
        assert dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT_UE8M0, 4096, 2112, 7168) > 0
        # K-grouped: 256 x 256 tiles of all groups where they fill whole rounds, else 256 x 128
        assert "kernel=wide tile=256x256 grid=256 tiles=3584" in dg.dg_describe_plan(dg.DG_OP_K_GROUPED, 4096, 7168,
                                                                                       33536, 8)
        assert "kernel=persistent tile=256x128" in dg.dg_describe_plan(dg.DG_OP_K_GROUPED, 300, 144, 1024, 3)
        # BF16: the same rule (K counted in bf16 elements, a multiple of 64)
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_BF16_GEMM_NT, 4096, 7168, 16384)
        assert dg.dg_get_workspace_size(dg.DG_OP_BF16_GEMM_NT, 4096, 7168, 16384) == 0
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_BF16_GEMM_NT, 300, 400, 576)
        assert dg.dg_describe_plan(dg.DG_OP_BF16_GEMM_NT, 300, 400, 100) == ""
        assert "kernel=skinny" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 128, 7168, 2048)
        # 64 < M <= 128: a 128 x 128 tile when it still fills the CUs through a K split
        assert "tile=128x128 tiles=56 splits=4" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 128, 7168, 16384)
        assert "tile=128x128 tiles=56 splits=4" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 100, 7168, 5120)
        assert "tile=64x64" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 128, 4096, 7168)
        assert "tile=64x64" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 64, 7168, 16384)
        assert "tail=16x4" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 4096, 2112, 7168)
        # weight loads streamed non-temporally where one workgroup reads each weight line
        assert "splits=5 weights=nt" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 64, 2112, 7168)
        assert "weights=default" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 128, 2112, 7168)   # two 64-row tiles
        assert "weights=default" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 128, 7168, 16384)  # one 128-row tile
        assert dg.dg_describe_plan(dg.DG_OP_MASKED, 128, 4096, 7168, 32) == \
            "kernel=persistent tile=128x256 grid=256 max_tiles=512 weights=nt"
        assert dg.dg_describe_plan(dg.DG_OP_MASKED, 256, 4096, 7168, 32).endswith("max_tiles=1024 weights=default")
        # 128 < M <= 256: 64 x 64 skinny tiles where the 256 x 128 tiles would
        # fill at most half the CUs and K <= 8192; otherwise the tile kernels
        assert "kernel=skinny tile=64x64 tiles=99 splits=2 weights=default" in \
            dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 160, 2112, 7168)
        assert "kernel=skinny tile=64x64 tiles=448 splits=1" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 256, 7168, 2048)
        assert "kernel=skinny tile=64x64 tiles=132" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT_UE8M0, 256, 2112, 7168)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 192, 7168, 16384)   # K > 8192
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 256, 24576, 1536)   # 192 tiles
        # 256 < M <= 512: 64x64, 64x128 or 128x128 tiles and a K split of at most
        # 4, the least estimated time from the bytes each CU pulls
        assert "kernel=skinny tile=64x64 tiles=231 splits=2" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 448, 2112, 7168)
        assert "kernel=skinny tile=64x128 tiles=119 splits=1" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 400, 2112, 1024)
        assert "kernel=skinny tile=128x128 tiles=224 splits=1" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 512, 7168, 2048)
        assert "kernel=skinny tile=128x128 tiles=128 splits=2" in \
            dg.dg_describe_plan(dg.DG_OP_GEMM_NT_UE8M0, 512, 4096, 7168)
        assert "kernel=skinny" not in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 512, 24576, 1536)   # 384 tiles
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 320, 7168, 16384)   # K > 8192
        assert dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT, 448, 2112, 7168) > 0
        # 512 < M <= 2048, K <= 8192: the skinny plan where its estimate beats
        # the 256 x 128 plan's by 15%
        assert "kernel=skinny tile=64x64 tiles=256 splits=1" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 1024, 1024, 4096)
        assert "kernel=skinny tile=128x128 tiles=72 splits=2" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 700, 1536, 5120)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 1536, 4096, 7168)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 1024, 2112, 7168)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 2100, 1024, 4096)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 700, 1536, 9216)   # K > 8192
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 2048, 7168, 2048)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_BF16_GEMM_NT, 1024, 1024, 4096)
        dg.dg_set_num_cus(100)  # the estimates hold for the whole chip only
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 1024, 1024, 4096)
        dg.dg_set_num_cus(256)
        # no default plan needs more split-K scratch than the allocation-free entry holds (40 MiB)
        worst = max(dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT, m, n, k)
                    for m in (1, 64, 100, 128, 129, 200, 256, 300, 384, 512, 520, 700, 1024, 1500, 2048, 2100, 4096)
                    for n in (16, 144, 1024, 2112, 4096, 7168, 24576, 32768) for k in (512, 1536, 2048, 4096, 7168, 16384))
        assert 0 < worst <= 40 << 20
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_BF16_GEMM_NT, 160, 2112, 7168)
        assert dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT, 160, 2112, 7168) > 0
        dg.dg_set_num_cus(4)
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 500, 496, 384)          # 4 tiles on 4 CUs
        assert dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 500, 496, 100) == ""                      # invalid K
        assert dg.dg_describe_plan(dg.DG_OP_MASKED, 500, 496, 100) == ""                      # invalid K
        dg.dg_set_num_cus(256)
        # contiguous: 256 x 256 tiles when they fill whole rounds, at any K
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_CONTIGUOUS, 36000, 4096, 7168, 8)
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_CONTIGUOUS, 25472, 7168, 2048, 8)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_CONTIGUOUS, 1152, 400, 2048, 3)  # 10 tiles on 3 CUs
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_CONTIGUOUS, 1024, 4096, 7168, 8)  # 64 tiles
    finally:
        dg.dg_set_num_cus(0)


def test_forced_config_parsing(lib, monkeypatch):
    # host logic only: DG_FORCE_CONFIG items the planner honours, and items it
    # ignores (a ring depth that is not compiled, a malformed item)
    from moe_grouped_matmul_amd import dg

    try:
        dg.dg_set_num_cus(256)
        default = dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 64, 7168, 2048)
        monkeypatch.setenv("DG_FORCE_CONFIG", "skinny=64x32x3x4")
        assert "kernel=skinny tile=64x128 tiles=56 splits=3" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 64, 7168, 2048)
        monkeypatch.setenv("DG_FORCE_CONFIG", "skinny=64x32x3x5")  # depth 5 is not compiled
        assert dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 64, 7168, 2048) == default
        monkeypatch.setenv("DG_FORCE_CONFIG", "skinny=64x32")  # malformed
        assert dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 64, 7168, 2048) == default
        monkeypatch.setenv("DG_FORCE_CONFIG", "skinny=64x16x4x8")  # honoured up to 2048 rows
        assert "kernel=skinny tile=64x64 tiles=176 splits=4" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 200, 2816, 1024)
        assert "kernel=skinny tile=64x64 tiles=352 splits=4" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 500, 2816, 1024)
        assert "kernel=skinny tile=64x64 tiles=704 splits=4" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 1000, 2816, 1024)
        assert "kernel=skinny" not in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 2049, 2816, 1024)
        monkeypatch.setenv("DG_FORCE_CONFIG", "kernel=persistent")
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 4096, 7168, 16384)
        assert "kernel=persistent" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 160, 2112, 7168)
        monkeypatch.setenv("DG_FORCE_CONFIG", "kernel=wide,chunk_rows=1000")
        plan = dg.dg_describe_plan(dg.DG_OP_GEMM_NT, 4096, 2112, 7168)
        assert "kernel=wide tile=256x256 grid=27 tiles=27" in plan and plan.endswith("chunks=6")  # 5 x 768 + 256 rows
    finally:
        dg.dg_set_num_cus(0)


def test_errors_are_thread_local(lib):
    # host logic only: concurrent calls failing for different reasons each read
    # back their own message (dg_get_last_error is per thread), and the
    # validation and plan description are safe to call from several threads
    import threading

    from moe_grouped_matmul_amd import dg

    s = ctypes.c_void_p(0)
    cases = [
        (lambda: lib.dg_fp8_gemm_nt(P16, P16, P16, P16, P16, 64, 2112, 7000, None, 0, s), dg.DG_ERR_SHAPE, "K"),
        (lambda: lib.dg_fp8_gemm_nt(P16, P16, P16, P16, P16, 64, 2110, 7168, None, 0, s), dg.DG_ERR_SHAPE, "N"),
        (lambda: lib.dg_m_grouped_fp8_gemm_nt_contiguous(P16, P16, P16, P16, P16, P16, 256, 128, 256, 1025, None, 0, s),
         dg.DG_ERR_SHAPE, "G"),
        (lambda: lib.dg_fp8_gemm_nt(P16 + 8, P16, P16, P16, P16, 64, 2112, 7168, None, 0, s), dg.DG_ERR_ALIGN,
         "align"),
    ]
    failures = []
    barrier = threading.Barrier(len(cases))

    def worker(call, code, word):
        barrier.wait()
        for _ in range(200):
            rc = call()
            msg = lib.dg_get_last_error().decode()
            plan = lib.dg_describe_plan(dg.DG_OP_GEMM_NT, 4096, 7168, 16384, 1)
            if rc != code or word not in msg or not plan:
                failures.append((rc, msg))
                return

    threads = [threading.Thread(target=worker, args=c) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not failures, failures[:3]
