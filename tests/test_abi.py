"""The C ABI library loads on the CPU, exports every function include/dg.h
declares, and rejects bad arguments on the host before touching a device."""

import ctypes
import os
import re

import pytest

import fp8_block_scaled_nt_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return dg.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
        assert name in dg._SIGNATURES, f"binding lacks {name}"


def test_host_only_functions(lib):
    assert lib.dg_get_m_alignment_for_contiguous_layout() == 128
    assert [lib.dg_get_sfa_ld(m) for m in (0, 1, 4, 5, 64, 2067)] == [0, 4, 4, 8, 64, 2068]
    assert lib.dg_status_string(0) == b"ok"
    assert lib.dg_status_string(3) == b"misaligned pointer"
    assert lib.dg_version().startswith(b"dg-gfx950")


P = ctypes.c_void_p
GOOD = P(0x10000)  # never dereferenced: every case below fails validation first
ODD = P(0x10004)


@pytest.mark.parametrize("args,status", [
    ((None, GOOD, GOOD, GOOD, GOOD, 64, 64, 128), 1),      # null a
    ((GOOD, GOOD, GOOD, GOOD, GOOD, -1, 64, 128), 1),      # negative m
    ((GOOD, GOOD, GOOD, GOOD, GOOD, 64, 0, 128), 1),       # n = 0
    ((GOOD, GOOD, GOOD, GOOD, GOOD, 64, 64, 100), 2),      # k not a multiple of 128
    ((GOOD, GOOD, GOOD, GOOD, GOOD, 64, 64, 0), 2),
    ((GOOD, ODD, GOOD, GOOD, GOOD, 64, 64, 128), 3),       # misaligned sfa
    ((GOOD, GOOD, GOOD, GOOD, GOOD, 0, 64, 128), 0),       # m = 0: no-op, no device needed
])
def test_dense_validation(lib, args, status):
    assert lib.dg_fp8_gemm_nt(*args, None) == status
    if status:
        assert len(lib.dg_last_error_message()) > 0


def test_grouped_validation(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, None, 128, 64, 128, 2, None) == 1
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 100, 64, 128, 2, None) == 2  # m not 128-aligned
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 128, 64, 128, 0, None) == 1  # no groups
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0, 64, 128, 2, None) == 0
    g = lib.dg_m_grouped_fp8_gemm_nt_masked
    assert g(GOOD, GOOD, GOOD, GOOD, GOOD, None, 4, 64, 64, 128, 0, None) == 1
    assert g(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 4, -1, 64, 128, 0, None) == 1
    assert g(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 4, 64, 64, 256 + 1, 0, None) == 2
    assert g(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0, 64, 64, 128, 0, None) == 0
    assert g(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 4, 0, 64, 128, 0, None) == 0


def test_k_grouped_validation(lib):
    f = lib.dg_k_grouped_fp8_gemm_nt
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, None, 2, 64, 64, 256, None) == 1      # null k_sizes
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, -1, 64, 64, 256, None) == 1     # negative group count
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 64, 64, 200, None) == 2      # k not whole slabs
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, P(0x10002), 2, 64, 64, 256, None) == 3  # k_sizes not 4-byte aligned
    assert f(GOOD, GOOD, GOOD, GOOD, ODD, GOOD, 2, 64, 64, 256, None) == 3       # misaligned d
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0, 64, 64, 256, None) == 0      # no groups: no-op
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 0, 64, 256, None) == 0       # m = 0: no-op


def test_swiglu_validation(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_masked_swiglu
    #       a     sfa   b     sfb   hq    hs    masked_m   g  max_m inter  k  expected_m
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, 4, 64, 256, 256, 0, None) == 1   # null hs
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 4, -1, 256, 256, 0, None) == 1   # negative max_m
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 4, 64, 192, 256, 0, None) == 2   # inter not whole blocks
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 4, 64, 0, 256, 0, None) == 2
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 4, 64, 256, 200, 0, None) == 2   # k not whole slabs
    assert f(GOOD, GOOD, GOOD, GOOD, ODD, GOOD, GOOD, 4, 64, 256, 256, 0, None) == 3    # misaligned hq
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, P(0x10002), 4, 64, 256, 256, 0, None) == 3
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0, 64, 256, 256, 0, None) == 0   # no groups: no-op
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 4, 0, 256, 256, 0, None) == 0    # max_m = 0: no-op


def test_contiguous_swiglu_validation(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous_swiglu
    #       a     sfa   b     sfb   hq    hs    m_indices   m  inter  k  groups
    assert f(GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD, 128, 256, 256, 4, None) == 1   # null hq
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, -128, 256, 256, 4, None) == 1  # negative m
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 128, 256, 256, 0, None) == 1   # no groups
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 100, 256, 256, 4, None) == 2   # m not 128-aligned
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 128, 192, 256, 4, None) == 2   # inter not whole blocks
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 128, 256, 200, 4, None) == 2   # k not whole slabs
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, ODD, GOOD, 128, 256, 256, 4, None) == 3    # misaligned hs
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, P(0x10002), 128, 256, 256, 4, None) == 3
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0, 256, 256, 4, None) == 0     # m = 0: no-op


def test_bf16_validation(lib):
    f = lib.dg_bf16_gemm_nt
    assert f(None, GOOD, GOOD, 64, 64, 128, None) == 1      # null a
    assert f(GOOD, GOOD, GOOD, -1, 64, 128, None) == 1      # negative m
    assert f(GOOD, GOOD, GOOD, 64, 64, 96, None) == 2       # k not a multiple of 64
    assert f(GOOD, GOOD, ODD, 64, 64, 128, None) == 3       # misaligned d
    assert f(GOOD, GOOD, GOOD, 0, 64, 128, None) == 0       # m = 0: no-op


def test_fp4_validation(lib):
    f = lib.dg_fp4_gemm_nt
    assert f(GOOD, GOOD, GOOD, None, GOOD, 64, 64, 256, None) == 1      # null sfb
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, -1, 64, 256, None) == 1      # negative m
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 64, 64, 128, None) == 2      # k not whole 128-byte rows
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 64, 64, 384, None) == 2
    assert f(GOOD, ODD, GOOD, GOOD, GOOD, 64, 64, 256, None) == 3       # misaligned sfa
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 0, 64, 256, None) == 0       # m = 0: no-op
    assert lib.dg_quantize_a_1x128_fp4(None, GOOD, GOOD, 4, 128, None) == 1
    assert lib.dg_quantize_a_1x128_fp4(GOOD, GOOD, GOOD, 4, 192, None) == 2
    assert lib.dg_quantize_b_128x128_fp4(GOOD, ODD, GOOD, 4, 128, None) == 3
    assert lib.dg_quantize_b_128x128_fp4(GOOD, GOOD, GOOD, 0, 128, None) == 0


def test_quant_validation(lib):
    assert lib.dg_quantize_a_1x128(None, GOOD, GOOD, 4, 128, None) == 1
    assert lib.dg_quantize_a_1x128(GOOD, GOOD, GOOD, 4, 130, None) == 2
    assert lib.dg_quantize_b_128x128(GOOD, ODD, GOOD, 4, 128, None) == 3
    assert lib.dg_quantize_b_128x128(GOOD, GOOD, GOOD, 0, 128, None) == 0


def test_workspace_size_validation(lib):
    out = ctypes.c_size_t(7)
    size = lambda *a: lib.dg_dense_workspace_size(*a, ctypes.byref(out))
    assert lib.dg_dense_workspace_size(0, 64, 64, 128, None) == 1       # null result pointer
    assert size(3, 64, 64, 128) == 1 and out.value == 0                 # unknown dtype
    assert size(0, 64, 64, 100) == 2                                    # fp8: k % 128
    assert size(1, 64, 64, 96) == 2                                     # bf16: k % 64
    assert size(2, 64, 64, 128) == 2                                    # fp4: k % 256
    assert size(0, -1, 64, 128) == 1 and size(0, 64, 0, 128) == 1
    out.value = 7
    assert size(0, 0, 64, 128) == 0 and out.value == 0                  # m = 0: no split, no device needed
    with pytest.raises(ValueError):
        dg.dense_workspace_size(64, 64, 128, dtype="fp16")


def test_no_device_is_reported_not_crashed(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    # valid-looking arguments reach the device query, which reports no device
    assert lib.dg_fp8_gemm_nt(GOOD, GOOD, GOOD, GOOD, GOOD, 64, 64, 128, None) == 4
    assert lib.dg_dense_workspace_size(0, 64, 2112, 7168, ctypes.byref(ctypes.c_size_t())) == 4


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dg, "_lib", None)
    monkeypatch.setattr(dg, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        dg.lib()
