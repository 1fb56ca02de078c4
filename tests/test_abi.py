"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/*.h, and rejects bad arguments (before any HIP call) with
QG_EINVAL and a message.  No kernel runs here."""
import ctypes
import glob
import os
import re

import pytest

from conftest import ROOT

qg = pytest.importorskip("gemm_qgemv_q4_amd")

P = ctypes.c_void_p


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text):
            name = m.group(1)
            if name.startswith(("qg", "qmm_", "qkv_")):
                names.add(name)
    return names


def test_header_declares_the_entry_points():
    names = declared_functions()
    for fn in ("qgemv_q4_0", "qgemv_q4_k", "qgemv_dual_q4_0", "qmm_affine_t", "qkv_split_f32",
               "qgemv_q4_k_multi", "qmm_affine_t_packed", "qmm_affine_t_qkv", "qg_last_error"):
        assert fn in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(qg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(qg.SIGNATURES)


def _err(status):
    assert status == qg.QG_EINVAL
    msg = qg.last_error()
    assert msg
    return msg


A = P(4096)  # fake, aligned, never dereferenced: validation fails first
B = P(8192)
C = P(16384)
D = P(32768)
E = P(65536)


@pytest.mark.parametrize("m,n,k", [(0, 1, 32), (1, 0, 32), (1, 1, 0), (-1, 4, 32)])
def test_q4_0_rejects_nonpositive_dims(m, n, k):
    assert "must all be > 0" in _err(qg.raw.qgemv_q4_0(A, B, C, m, n, k, None))


def test_q4_0_rejects_k_not_multiple_of_32():
    assert "QK4_0" in _err(qg.raw.qgemv_q4_0(A, B, C, 1, 1, 48, None))


def test_q4_0_rejects_null_and_misaligned():
    assert "null" in _err(qg.raw.qgemv_q4_0(None, B, C, 1, 1, 32, None))
    assert "null" in _err(qg.raw.qgemv_q4_0(A, None, C, 1, 1, 32, None))
    assert "aligned" in _err(qg.raw.qgemv_q4_0(P(4098), B, C, 1, 1, 32, None))
    assert "aligned" in _err(qg.raw.qgemv_q4_0(A, P(8194), C, 1, 1, 32, None))
    assert "alias" in _err(qg.raw.qgemv_q4_0(A, B, B, 1, 1, 32, None))


def test_q4_k_rejects_k_not_multiple_of_256():
    assert "256" in _err(qg.raw.qgemv_q4_k(A, B, C, 1, 4, 384, None))
    assert "must all be > 0" in _err(qg.raw.qgemv_q4_k(A, B, C, 1, 0, 256, None))


def test_dual_rejects_same_outputs_and_bad_weights():
    assert "different" in _err(qg.raw.qgemv_dual_q4_0(A, B, C, D, D, 1, 4, 32, None))
    assert "null" in _err(qg.raw.qgemv_dual_q4_0(A, None, C, D, E, 1, 4, 32, None))
    assert "QK4_0" in _err(qg.raw.qgemv_dual_q4_0(A, B, C, D, E, 1, 4, 40, None))


@pytest.mark.parametrize("gs", [0, 1, 3, 5, 48, 2048, -64])
def test_affine_rejects_bad_group_size(gs):
    assert "group_size" in _err(qg.raw.qmm_affine_t(A, B, C, D, E, 1, 1, 64, gs, None))


def test_affine_rejects_k_not_divisible_by_group_size():
    # the page's rejects_k_not_divisible_by_group_size case uses gs = 5; here K % gs
    assert "divisible" in _err(qg.raw.qmm_affine_t(A, B, C, D, E, 1, 1, 96, 64, None))
    assert "must all be > 0" in _err(qg.raw.qmm_affine_t(A, B, C, D, E, 0, 1, 64, 64, None))
    assert "null" in _err(qg.raw.qmm_affine_t(A, None, C, D, E, 1, 1, 64, 64, None))


def test_qkv_split_rejects_zero_and_overflow():
    assert "> 0" in _err(qg.raw.qkv_split_f32(A, B, C, D, 0, 4, 4, 4, None))
    assert "> 0" in _err(qg.raw.qkv_split_f32(A, B, C, D, 2, 4, 0, 4, None))
    big = 0xFFFFFFFF
    assert "overflows u32" in _err(qg.raw.qkv_split_f32(A, B, C, D, 1, big, 1, 1, None))
    assert "alias" in _err(qg.raw.qkv_split_f32(A, B, B, D, 1, 4, 4, 4, None))


def test_mfma_threshold_knob():
    old = qg.qg_get_mfma_min_m()
    try:
        qg.qg_set_mfma_min_m(7)
        assert qg.qg_get_mfma_min_m() == 7
        with pytest.raises(qg.QGError):
            qg.qg_set_mfma_min_m(0)
        assert qg.qg_get_mfma_min_m() == 7
    finally:
        qg.qg_set_mfma_min_m(old)


def test_kernel_mask_knob():
    old = qg.qg_get_kernel_mask()
    assert old == qg.QG_KERNEL_ALL
    try:
        qg.qg_set_kernel_mask(qg.QG_KERNEL_XR)
        assert qg.qg_get_kernel_mask() == qg.QG_KERNEL_XR
        with pytest.raises(qg.QGError, match="unknown bits"):
            qg.qg_set_kernel_mask(8)
        assert qg.qg_get_kernel_mask() == qg.QG_KERNEL_XR
        with qg.kernels(mask=0, mfma_min_m=5):
            assert (qg.qg_get_kernel_mask(), qg.qg_get_mfma_min_m()) == (0, 5)
        assert qg.qg_get_kernel_mask() == qg.QG_KERNEL_XR
    finally:
        qg.qg_set_kernel_mask(old)


def test_error_message_is_per_call():
    _err(qg.raw.qgemv_q4_0(A, B, C, 1, 1, 48, None))
    assert "QK4_0" in qg.last_error()
    _err(qg.raw.qgemv_q4_k(A, B, C, 1, 4, 384, None))
    assert "256" in qg.last_error()


def _multi(ws, ys, ns, ldys, parts, x, m, k):
    n_arr = (ctypes.c_int64 * max(1, len(ns)))(*ns)
    l_arr = (ctypes.c_int64 * max(1, len(ldys)))(*ldys)
    w_arr = (ctypes.c_void_p * max(1, len(ws)))(*ws)
    y_arr = (ctypes.c_void_p * max(1, len(ys)))(*ys)
    return qg.raw.qgemv_q4_k_multi(w_arr, y_arr, n_arr, l_arr, parts, x, m, k, None)


def test_multi_rejects_bad_part_lists():
    assert "parts" in _err(_multi([A], [C], [4], [4], 0, B, 1, 256))
    assert "parts" in _err(_multi([A] * 9, [C] * 9, [4] * 9, [4] * 9, 9, B, 1, 256))
    assert "ldy" in _err(_multi([A, D], [C, E], [4, 8], [4, 7], 2, B, 1, 256))
    assert "rows" in _err(_multi([A, D], [C, E], [4, 0], [4, 4], 2, B, 1, 256))
    assert "256" in _err(_multi([A], [C], [4], [4], 1, B, 1, 384))
    assert "null" in _err(_multi([A, None], [C, E], [4, 4], [4, 4], 2, B, 1, 256))
    assert "M and K" in _err(_multi([A], [C], [4], [4], 1, B, 0, 256))
    assert "null" in _err(qg.raw.qgemv_q4_k_multi(None, None, None, None, 1, B, 1, 256, None))


def test_packed_rejects_bad_shapes():
    assert "pack factor" in _err(qg.raw.qmm_affine_t_packed(A, B, C, D, E, 1, 1, 36, 4, None))
    assert "group_size" in _err(qg.raw.qmm_affine_t_packed(A, B, C, D, E, 1, 1, 64, 48, None))
    assert "divisible" in _err(qg.raw.qmm_affine_t_packed(A, B, C, D, E, 1, 1, 96, 64, None))
    assert "aligned" in _err(qg.raw.qmm_affine_t_packed(A, P(8194), C, D, E, 1, 1, 64, 32, None))
    assert "must all be > 0" in _err(qg.raw.qmm_affine_t_packed(A, B, C, D, E, 1, 0, 64, 32, None))


def test_qkv_fused_rejects_bad_spans_and_aliasing():
    F = P(1 << 17)
    G = P(1 << 18)
    assert "> 0" in _err(qg.raw.qmm_affine_t_qkv(A, B, C, D, E, F, G, 1, 64, 32, 0, 4, 4, None))
    assert "alias" in _err(qg.raw.qmm_affine_t_qkv(A, B, C, D, E, E, G, 1, 64, 32, 4, 4, 4, None))
    assert "group_size" in _err(qg.raw.qmm_affine_t_qkv(A, B, C, D, E, F, G, 1, 64, 3, 4, 4, 4, None))
    assert "null" in _err(qg.raw.qmm_affine_t_qkv(A, None, C, D, E, F, G, 1, 64, 32, 4, 4, 4, None))


def test_c_program_builds_and_runs_against_the_header(tmp_path):
    """The header compiles as C99 with -Wall -Wextra -Werror, a plain C program
    links against the library, and without a GPU its argument checks pass
    (with a GPU the same program also checks the bitwise equalities; the gpu
    test runs the copy built by the build step)."""
    import importlib.util
    import subprocess
    spec = importlib.util.spec_from_file_location("_qg_build_c", os.path.join(ROOT, "tests", "c", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    out = mod.build(str(tmp_path / "abi_check"))
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1")  # argument checks only, even on a GPU host
    res = subprocess.run([out], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi_check: ok" in res.stdout, res.stdout


def test_header_compiles_as_cpp(tmp_path):
    import shutil
    import subprocess
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    src = tmp_path / "h.cpp"
    src.write_text('#include "qgemv_q4.h"\nint main() { return qg_get_mfma_min_m() < 0; }\n')
    res = subprocess.run([cxx, "-std=c++11", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.join(ROOT, "include"), str(src)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
