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
    # the projection shape takes a tile of the direct-to-LDS pipeline
    assert "direct" in mm.mm_gemm_f32_config_name(mm.mm_gemm_f32_select(8192, 14336, 4096))


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


def test_gemv_t_workspace_sizes_and_checks(lib):
    ws = mm.mm_gemv_t_f32_workspace_bytes
    assert ws(4096, 4096) == 16 * 4096 * 4     # 16 strips of 256 columns, 16 row blocks
    assert ws(4096, 16384) == 4 * 16384 * 4    # 64 strips: 4 row blocks make ~256 workgroups
    assert ws(1000, 4096) == 3 * 4096 * 4      # at least 256 rows per block
    for M, N in [(511, 4096), (4096, 1001), (300, 8), (0, 5), (5, 0)]:
        assert ws(M, N) == 0, (M, N)           # served by the strips kernel
    assert ws(-1, 3) == -1 and ws(3, 1 << 31) == -1
    need = ws(4096, 4096)
    f = lib.mm_gemv_t_f32_ws
    for args, why in [((None, need), "workspace is NULL"), ((FAKE + 4, need), "16-byte"),
                      ((FAKE, need - 4), "smaller")]:
        assert f(4096, 4096, FAKE, FAKE, FAKE, *args, None) == mm.MM_ERR_INVALID_ARG
        assert why in mm.mm_last_error()
    for a, x, y, why in [(None, FAKE, FAKE, "A is NULL"), (FAKE, None, FAKE, "x is NULL"),
                         (FAKE, FAKE, None, "y is NULL"), (FAKE + 2, FAKE, FAKE, "aligned")]:
        assert f(4096, 4096, a, x, y, FAKE, need, None) == mm.MM_ERR_INVALID_ARG
        assert why in mm.mm_last_error()
    # no workspace needed: the checks of mm_gemv_t_f32, and nothing enqueued for N == 0
    assert f(300, 8, None, FAKE, FAKE, None, 0, None) == mm.MM_ERR_INVALID_ARG
    assert f(7, 0, None, FAKE, None, None, 0, None) == mm.MM_OK


def test_gemm_workspace_sizes_and_checks(lib):
    ws = mm.mm_gemm_f32_workspace_bytes
    assert ws(4096, 64, 4096) == 8 * 4096 * 64 * 4   # 64 tiles of 64 x 64: 8 K chunks
    assert ws(4096, 32, 4096) == 8 * 4096 * 32 * 4
    assert ws(16384, 48, 8192) == 2 * 16384 * 48 * 4  # 256 tiles: 2 chunks make ~512 workgroups
    assert ws(4096, 64, 2064) == 0                    # 2064 = 129 x 16: no whole 16-k chunks of 2064 / 2
    assert ws(4096, 64, 2080) == 2 * 4096 * 64 * 4    # 2080 = 2 x 65 x 16: 2 chunks
    assert ws(4096, 128, 4096) == 4 * 4096 * 128 * 4  # 128 tiles: 4 chunks
    assert ws(4096, 256, 4096) == 2 * 4096 * 256 * 4  # 256 tiles: 2 chunks
    # N % 4 != 0 above 32 columns: slices of N rounded up to 4, then B padded to that width
    assert ws(4096, 45, 4096) == (8 * 4096 * 48 + 4096 * 48) * 4
    assert ws(1000, 99, 2048) == (8 * 1000 * 100 + 2048 * 100) * 4
    assert ws(4096, 255, 4096) == (2 * 4096 * 256 + 4096 * 256) * 4
    for M, N, K in [(4096, 24, 4096), (4096, 25, 4096), (4096, 31, 4096), (4096, 260, 4096), (8192, 256, 4096),
                    (4096, 64, 1024), (0, 64, 4096), (64, 0, 4096), (64, 64, 0)]:
        assert ws(M, N, K) == 0, (M, N, K)            # served by mm_gemm_f32's kernels
    assert ws(-1, 3, 3) == -1 and ws(3, 3, 1 << 31) == -1
    need = ws(4096, 64, 4096)
    f = lib.mm_gemm_f32_ws
    base = (4096, 64, 4096, FAKE, 4096, FAKE, 64, FAKE, 64)
    for args, why in [((None, need), "workspace is NULL"), ((FAKE + 4, need), "16-byte"),
                      ((FAKE, need - 4), "smaller")]:
        assert f(*base, *args, None) == mm.MM_ERR_INVALID_ARG
        assert why in mm.mm_last_error()
    for i, why in [(3, "A is NULL"), (5, "B is NULL"), (7, "C is NULL")]:
        bad = list(base)
        bad[i] = None
        assert f(*bad, FAKE, need, None) == mm.MM_ERR_INVALID_ARG
        assert why in mm.mm_last_error()
    bad = list(base)
    bad[4] = 100  # lda < K
    assert f(*bad, FAKE, need, None) == mm.MM_ERR_INVALID_ARG and "lda" in mm.mm_last_error()
    # no workspace needed: the checks of mm_gemm_f32, and nothing enqueued for M == 0
    assert f(64, 8, 64, None, 64, FAKE, 8, FAKE, 8, None, 0, None) == mm.MM_ERR_INVALID_ARG
    assert f(0, 8, 64, None, 64, FAKE, 8, None, 8, None, 0, None) == mm.MM_OK


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


# ------------------------------------------------------------------ convolution

def _out_dim(i, f, st, p, d):
    return (i + 2 * p - d * (f - 1) - 1) // st + 1


def test_conv_out_dim(lib):
    for i, f, st, p, d in [(28, 3, 1, 1, 1), (56, 3, 2, 1, 1), (224, 7, 2, 3, 1), (64, 3, 1, 2, 2),
                           (5, 5, 1, 0, 1), (1, 1, 1, 0, 1), (7, 3, 3, 0, 2), (0, 1, 1, 1, 1),
                           (10, 4, 3, 5, 3)]:
        assert mm.mm_conv2d_out_dim(i, f, st, p, d) == _out_dim(i, f, st, p, d) >= 1
    # the dilated filter longer than the padded input, and arguments out of range
    for args in [(4, 5, 1, 0, 1), (4, 3, 1, 0, 2), (0, 1, 1, 0, 1), (0, 3, 1, 1, 1), (-1, 1, 1, 0, 1), (4, 0, 1, 0, 1),
                 (4, 1, 0, 0, 1), (4, 1, 1, -1, 1), (4, 1, 1, 0, 0), (1 << 29, 1, 1, 0, 1),
                 (8, 3, 1, 1 << 28, 1), (8, 1 << 29, 1, 0, 1)]:
        assert mm.mm_conv2d_out_dim(*args) == -1, args


def test_conv_config_table(lib):
    n = mm.mm_conv2d_f32_num_configs()
    assert n >= 1
    names = [mm.mm_conv2d_f32_config_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    # each name states the tile (BM x BN x BK), the wave tile and the waves: the wave tiles
    # divide the tile, and the waves are its wave grid (twice that where K is split over two
    # wave groups, "ks2")
    for name in names:
        m = re.match(r"(\d+)x(\d+)x(\d+) w(\d+)x(\d+) .*\((\d+) waves\)", name)
        assert m, name
        bm, bn, bk, wm, wn, waves = map(int, m.groups())
        assert bm % wm == 0 and bn % wn == 0 and bk % 16 == 0, name
        grid = (bm // wm) * (bn // wn)
        assert waves == (2 * grid if " ks2 " in name else grid), name
    assert mm.mm_conv2d_f32_config_name(n) is None
    for geo in [(1, 1, 1, 1, 1, 1, 1, 1, 1, 0, 0, 1, 1), (32, 3, 224, 224, 64, 7, 7, 2, 2, 3, 3, 1, 1),
                (32, 128, 28, 28, 128, 3, 3, 1, 1, 1, 1, 1, 1), (32, 256, 56, 56, 64, 1, 1, 1, 1, 0, 0, 1, 1),
                (2, 5, 13, 11, 7, 3, 3, 1, 1, 1, 1, 1, 1), (1, 1, 30000, 30000, 4096, 1, 1, 1, 1, 0, 0, 1, 1)]:
        assert 0 <= mm.mm_conv2d_f32_select(*geo) < n
    assert mm.mm_conv2d_f32_select(1, 1, 4, 4, 1, 5, 5, 1, 1, 0, 0, 1, 1) == -1   # does not fit
    assert mm.mm_conv2d_f32_select(-1, 1, 4, 4, 1, 1, 1, 1, 1, 0, 0, 1, 1) == -1


# N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw
GOOD = (2, 3, 8, 8, 4, 3, 3, 1, 1, 1, 1, 1, 1)


def _conv(lib, geo, x=FAKE, w=FAKE, y=FAKE, cfg=None):
    if cfg is None:
        return lib.mm_conv2d_f32(*geo, x, w, y, None)
    return lib.mm_conv2d_f32_config(cfg, *geo, x, w, y, None)


@pytest.mark.parametrize("change,why", [
    ({0: -1}, "negative size"), ({1: -1}, "negative size"), ({4: -3}, "negative size"),
    ({5: 0}, "filter size"), ({6: 0}, "filter size"),
    ({7: 0}, "stride"), ({8: -1}, "stride"),
    ({9: -1}, "padding"), ({10: -2}, "padding"),
    ({11: 0}, "dilation"), ({12: 0}, "dilation"),
    ({5: 9, 9: 0}, "does not fit"), ({6: 5, 10: 0, 12: 3}, "does not fit"),
    ({2: 1 << 29}, "2^29"), ({9: 1 << 28}, "2^29"), ({5: 3, 11: 1 << 28, 2: 1 << 28}, "2^29"),
    ({1: 1 << 16, 2: 256, 3: 64}, "C * H * W"),
    ({1: 1 << 25, 2: 1, 3: 1, 5: 9, 6: 9, 9: 4, 10: 4}, "C * R * S"),
    ({1: 1, 2: 30000, 3: 30000, 9: 2000, 10: 2000, 5: 1, 6: 1}, "padded plane"),
])
def test_conv_rejects_invalid_arguments(lib, change, why):
    geo = list(GOOD)
    for k, v in change.items():
        geo[k] = v
    assert _conv(lib, geo) == mm.MM_ERR_INVALID_ARG
    assert why in mm.mm_last_error(), mm.mm_last_error()


def test_conv_rejects_bad_pointers_and_config(lib):
    for kw, why in [({"x": None}, "x is NULL"), ({"w": None}, "w is NULL"),
                    ({"y": None}, "y is NULL"), ({"x": FAKE + 2}, "aligned")]:
        assert _conv(lib, GOOD, **kw) == mm.MM_ERR_INVALID_ARG
        assert why in mm.mm_last_error()
    n = mm.mm_conv2d_f32_num_configs()
    for cfg in (-1, n):
        assert _conv(lib, GOOD, cfg=cfg) == mm.MM_ERR_INVALID_ARG
    with pytest.raises(mm.MMError):
        mm.mm_conv2d_f32(*GOOD[:7], 0, 1, 1, 1, 1, 1, FAKE, FAKE, FAKE, stream=1)


def test_conv_without_outputs_enqueues_nothing(lib):
    # N == 0 or K == 0: no output element, so no HIP call, even with NULL pointers
    geo = list(GOOD)
    geo[0] = 0
    assert _conv(lib, geo, x=None, y=None) == mm.MM_OK
    geo = list(GOOD)
    geo[4] = 0
    assert _conv(lib, geo, w=None, y=None) == mm.MM_OK


def test_conv_accounting():
    P, Q = rl.conv_out_hw(224, 224, 7, 7, (2, 2), (3, 3))
    assert (P, Q) == (112, 112)
    assert rl.conv_flops(32, 3, 64, 7, 7, P, Q) == 2 * 64 * (32 * 112 * 112) * 147
    assert rl.conv_algorithmic_bytes(1, 2, 5, 5, 3, 3, 3, 3, 3) == 4 * (50 + 54 + 27)
    assert rl.im2col_matrix_bytes(1, 2, 3, 3, 3, 3) == 4 * 18 * 9
    # a 1x1 convolution of one image is the GEMM of its filters with its C x HW matrix
    assert rl.conv_flops(1, 256, 64, 1, 1, 56, 56) == rl.gemm_flops(64, 56 * 56, 256)


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="a GPU is present: the call would launch; the GPU suite checks its zeros")
def test_conv_empty_input_plane_returns_a_status(lib):
    # H = W = 0 with padding: P, Q >= 1 and every tap reads padding. The call must come
    # back with a status (here, without a GPU, the zero fill's launch error), not end the
    # process. It runs in a child process so that a crash fails this test alone.
    import subprocess
    import sys
    code = (
        "import ctypes, sys\n"
        f"lib = ctypes.CDLL({mm_build.LIB!r})\n"
        "f = lib.mm_conv2d_f32\n"
        "f.restype = ctypes.c_int\n"
        "f.argtypes = [ctypes.c_int64] * 13 + [ctypes.c_void_p] * 4\n"
        f"st = f(1, 1, 0, 0, 1, 1, 1, 1, 1, 1, 1, 1, 1, None, {FAKE}, {FAKE}, None)\n"
        "print(st)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"the call ended the process: rc {r.returncode}, {r.stderr[-500:]}"
    assert int(r.stdout.split()[-1]) in (mm.MM_OK, mm.MM_ERR_NO_DEVICE, mm.MM_ERR_LAUNCH)


def test_static_scratch_checks_before_any_launch(lib):
    f = lib.mm_gemm_f32_ws_static
    # a split that needs more than the static scratch (B padded to 256 columns)
    assert mm.mm_gemm_f32_workspace_bytes(4096, 255, 16384) > mm.MM_STATIC_SCRATCH_BYTES
    assert f(4096, 255, 16384, FAKE, 16384, FAKE, 255, FAKE, 255, None) == mm.MM_ERR_INVALID_ARG
    assert "static scratch" in mm.mm_last_error()
    # the argument checks of mm_gemm_f32, on split and unsplit shapes
    for i, why in [(3, "A is NULL"), (5, "B is NULL"), (7, "C is NULL")]:
        for shape in ((4096, 64, 4096), (300, 16, 4096)):
            args = [*shape, FAKE, shape[2], FAKE, shape[1], FAKE, shape[1]]
            args[i] = None
            assert f(*args, None) == mm.MM_ERR_INVALID_ARG
            assert why in mm.mm_last_error()
    assert f(4096, 64, 4096, FAKE, 100, FAKE, 64, FAKE, 64, None) == mm.MM_ERR_INVALID_ARG
    assert "lda" in mm.mm_last_error()
    # nothing to compute: no HIP call
    assert f(0, 64, 4096, None, 4096, FAKE, 64, None, 64, None) == mm.MM_OK
    # the header's size and the binding's agree; every split of N % 4 == 0 fits
    text = open(os.path.join(ROOT, "include", "mm.h")).read()
    m = re.search(r"#define MM_STATIC_SCRATCH_BYTES \((\d+) \* (\d+) \* (\d+)\)", text)
    assert m and int(m[1]) * int(m[2]) * int(m[3]) == mm.MM_STATIC_SCRATCH_BYTES
    for M, N, K in [(16320, 64, 2048), (4096, 256, 4096), (4096, 128, 8192), (255 * 64, 28, 2048)]:
        assert 0 < mm.mm_gemm_f32_workspace_bytes(M, N, K) <= mm.MM_STATIC_SCRATCH_BYTES
