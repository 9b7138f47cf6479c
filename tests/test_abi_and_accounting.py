"""CPU-only checks of the C ABI library and the accounting module.

No kernel is launched here: only symbol lookups, host-side argument checks (which
return before any HIP call) and static tables.
"""
import ctypes
import json
import os
import re

import pytest

import tiled_gemm_gemv_amd as mm
from tiled_gemm_gemv_amd import build as mm_build
from tiled_gemm_gemv_amd import roofline as rl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mm_build.LIB):
        mm_build.build()
    return mm.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("mm_gemm_f32", "mm_gemv_f32", "mm_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libmm.so does not export {name}"
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    assert mm.mm_status_string(mm.MM_OK) == "ok"
    assert "invalid" in mm.mm_status_string(mm.MM_ERR_INVALID_ARG)
    assert "device" in mm.mm_status_string(mm.MM_ERR_NO_DEVICE)
    assert "launch" in mm.mm_status_string(mm.MM_ERR_LAUNCH)
    assert mm.mm_status_string(12345) == "unknown status"


def test_config_table(lib):
    n = mm.mm_gemm_f32_num_configs()
    assert n >= 1
    names = [mm.mm_gemm_f32_config_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    assert mm.mm_gemm_f32_config_name(n) is None and mm.mm_gemm_f32_config_name(-1) is None
    for shape in [(1, 1, 1), (128, 128, 128), (1024, 1024, 1024), (1000, 1531, 777),
                  (8192, 14336, 4096)]:
        assert 0 <= mm.mm_gemm_f32_select(*shape) < n
    assert mm.mm_gemm_f32_select(8192, 14336, 4096) == 0


FAKE = 1 << 40   # never dereferenced: every call below fails the host-side checks


@pytest.mark.parametrize("args,why", [
    ((-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "negative size"),
    ((4, 4, 1 << 31, FAKE, 1 << 31, FAKE, 4, FAKE, 4), "size above"),
    ((4, 4, 8, FAKE, 7, FAKE, 4, FAKE, 4), "lda"),
    ((4, 5, 8, FAKE, 8, FAKE, 4, FAKE, 5), "ldb"),
    ((4, 5, 8, FAKE, 8, FAKE, 5, FAKE, 4), "ldc"),
    ((4, 5, 8, None, 8, FAKE, 5, FAKE, 5), "A is NULL"),
    ((4, 5, 8, FAKE, 8, None, 5, FAKE, 5), "B is NULL"),
    ((4, 5, 8, FAKE, 8, FAKE, 5, None, 5), "C is NULL"),
    ((4, 5, 0, FAKE, 0, FAKE, 5, FAKE, 5), "lda"),
    ((1 << 30, 4, 4, FAKE, 1 << 40, FAKE, 4, FAKE, 4), "overflow"),
])
def test_gemm_rejects_invalid_arguments(lib, args, why):
    st = lib.mm_gemm_f32(*args, None)
    assert st == mm.MM_ERR_INVALID_ARG
    assert why in mm.mm_last_error()
    with pytest.raises(mm.MMError):
        mm.mm_gemm_f32(*args, stream=1)


def test_gemm_config_index_checked(lib):
    n = mm.mm_gemm_f32_num_configs()
    assert lib.mm_gemm_f32_config(n, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, None) == \
        mm.MM_ERR_INVALID_ARG
    assert lib.mm_gemm_f32_config(-1, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, None) == \
        mm.MM_ERR_INVALID_ARG


def test_empty_outputs_enqueue_nothing(lib):
    # M == 0 or N == 0 returns before any HIP call, even with NULL pointers.
    assert lib.mm_gemm_f32(0, 5, 3, None, 3, FAKE, 5, None, 5, None) == mm.MM_OK
    assert lib.mm_gemm_f32(5, 0, 3, FAKE, 3, None, 1, None, 1, None) == mm.MM_OK
    assert lib.mm_gemv_f32(0, 7, None, FAKE, None, None) == mm.MM_OK


@pytest.mark.parametrize("args,why", [
    ((-2, 4, FAKE, FAKE, FAKE), "negative"),
    ((4, 1 << 31, FAKE, FAKE, FAKE), "size above"),
    ((4, 4, None, FAKE, FAKE), "A is NULL"),
    ((4, 4, FAKE, None, FAKE), "x is NULL"),
    ((4, 4, FAKE, FAKE, None), "y is NULL"),
])
def test_gemv_rejects_invalid_arguments(lib, args, why):
    assert lib.mm_gemv_f32(*args, None) == mm.MM_ERR_INVALID_ARG
    assert why in mm.mm_last_error()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(mm, "_lib", None)
    monkeypatch.setattr(mm, "_LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(OSError):
        mm.load()
    importlib.reload(mm)


# ------------------------------------------------------------------ accounting

def _golden():
    with open(os.path.join(ROOT, "tests", "golden", "page_counts.json")) as f:
        return json.load(f)


def test_accounting_matches_page_counts():
    g = _golden()
    assert rl.gemv_macs(4096, 4096) == g["fc_layer_macs"]["value"]
    assert rl.gemm_macs(1024, 1024, 1024) == g["square_gemm_macs"]["value"]
    assert rl.naive_element_reads(1024, 1024, 1024) == g["naive_reads_1024"]["value"]
    assert rl.tiled_element_reads(1024, 1024, 1024, 16) == g["tiled_reads_1024_t16"]["value"]
    assert rl.naive_element_reads(1024, 1024, 1024) // rl.tiled_element_reads(
        1024, 1024, 1024, 16) == 16
    assert rl.two_tile_bytes(32) == g["two_tiles_bytes_t32"]["value"]
    assert rl.naive_intensity() == g["arithmetic_intensity"]["naive"]
    assert rl.tiled_intensity(32) == g["arithmetic_intensity"]["tiled_t32"]
    for B, N in [(16, 1024), (32, 4096)]:
        assert rl.output_tile_reads_naive(B, N) == B * B * 2 * N
        assert rl.output_tile_reads_tiled(B, N) == 2 * N * B
        assert rl.output_tile_reads_naive(B, N) // rl.output_tile_reads_tiled(B, N) == B


def test_workload_accounting():
    assert rl.gemm_flops(8192, 14336, 4096) == 962_072_674_304
    assert rl.gemm_algorithmic_bytes(8192, 14336, 4096) == 838_860_800
    assert rl.gemv_algorithmic_bytes(4096, 4096) == 67_141_632
    assert rl.gemm_algorithmic_bytes(1000, 1531, 777) == 13_990_348
    assert rl.gemm_tile_model_bytes(8192, 14336, 4096, 256, 256) == 15_502_147_584
    assert abs(rl.gemm_bound_time(8192, 14336, 4096) - 6.116e-3) < 1e-5
    assert abs(rl.gemv_bound_time(4096, 4096) - 8.393e-6) < 1e-8
    assert abs(rl.MI355X_CUS * 256 * rl.MI355X_PEAK_SCLK_HZ - rl.MI355X_FP32_MFMA_PEAK) < 0.1e12
