"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, agrees with the oracle on the blob format, and rejects bad arguments
on the host before any HIP call is made."""
import ctypes
import os
import re

import pytest

import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmoe.h")


@pytest.fixture(scope="module")
def api():
    import int4_routed_expert_route_amd.api as api
    if not os.path.exists(api.LIB_PATH):
        pytest.skip("libmoe.so not built")
    api.lib()
    return api


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_expert_q4_gateup", "moe_expert_q4_down_combine", "moe_slot_stage"):
        assert n in names


def test_every_declared_symbol_is_exported(api):
    lib = ctypes.CDLL(api.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(api.exported_symbols()) == declared_functions()


def test_struct_layouts(api):
    assert ctypes.sizeof(api.moe_dims) == 16
    assert ctypes.sizeof(api.moe_stage_stats) == 24


@pytest.mark.parametrize("d,f", [(2816, 704), (128, 64), (256, 192)])
def test_blob_format_matches_oracle(api, d, f):
    dm = api.dims(d, f, 128, 8)
    sec = orc.blob_sections(d, f)
    assert api.moe_expert_blob_bytes(dm) == sec["total"]
    assert api.moe_expert_blob_offsets(dm) == [sec[n][0] for n in orc.SECTION_NAMES]


def test_bad_dims(api):
    assert api.moe_expert_blob_bytes(api.dims(100, 704, 128, 8)) == -1
    big = (1 << 64) - 1
    assert api.moe_workspace_size(0, 1, api.dims(2816, 704, 128, 0)) == big
    assert api.moe_workspace_size(0, 1, api.dims(2816, 704, 300, 8)) == big
    assert api.moe_workspace_size(2, 0, api.dims(2816, 704, 128, 8)) == big


def _p(v):
    return ctypes.c_void_p(v)


def test_validation_before_any_hip_call(api):
    """Fake, never-dereferenced pointers: every case fails a host check first."""
    lib = api.lib()
    dm = api.dims(2816, 704, 128, 8)
    A = 0x100000  # 256-byte aligned fake address
    ws = api.moe_workspace_size(api.MOE_CALL_ROUTE, 1, dm)
    # null input
    assert lib.moe_route(None, None, 1e-6, _p(A), None, 1, dm, _p(A), _p(A), _p(A), _p(A), ws, None) == api.MOE_ERR_ARG
    assert b"x is null" in lib.moe_last_error()
    # 4-byte aligned input
    assert lib.moe_route(_p(A + 4), None, 1e-6, _p(A), None, 1, dm, _p(A), _p(A), _p(A), _p(A), ws, None) == api.MOE_ERR_ALIGN
    # workspace too small
    assert lib.moe_route(_p(A), None, 1e-6, _p(A), None, 1, dm, _p(A), _p(A), _p(A), _p(A), ws - 1, None) == api.MOE_ERR_CAPACITY
    # bad T, bad dims, negative eps
    assert lib.moe_route(_p(A), None, 1e-6, _p(A), None, 0, dm, _p(A), _p(A), _p(A), _p(A), ws, None) == api.MOE_ERR_ARG
    assert lib.moe_route(_p(A), None, 1e-6, _p(A), None, 1, api.dims(2816, 700, 128, 8), _p(A), _p(A), _p(A), _p(A), ws, None) == api.MOE_ERR_ARG
    assert lib.moe_route(_p(A), None, -1.0, _p(A), None, 1, dm, _p(A), _p(A), _p(A), _p(A), ws, None) == api.MOE_ERR_ARG
    # the no-alloc router refuses sizes beyond its static scratch, before any HIP call
    nr = lib.moe_route_noalloc
    assert nr(_p(A), None, 1e-6, _p(A), None, 1 << 20, api.dims(2816, 704, 256, 8), _p(A), _p(A), _p(A),
              None) == api.MOE_ERR_CAPACITY
    assert b"16777216" in lib.moe_last_error()
    assert nr(None, None, 1e-6, _p(A), None, 1, dm, _p(A), _p(A), _p(A), None) == api.MOE_ERR_ARG
    assert nr(_p(A + 4), None, 1e-6, _p(A), None, 1, dm, _p(A), _p(A), _p(A), None) == api.MOE_ERR_ALIGN
    # permute limits
    assert lib.moe_permute(_p(A), 8193, dm, _p(A), _p(A), _p(A), _p(A), None, 0, None) == api.MOE_ERR_ARG
    # gate/up: slot stride, arena alignment, mask with grouping, offsets without sorted_pair
    stride = api.moe_expert_blob_bytes(dm)
    wsg = api.moe_workspace_size(api.MOE_CALL_GATEUP, 1, dm)
    g = lib.moe_expert_q4_gateup
    assert g(_p(A), _p(A), _p(A), 128, _p(A), stride + 16, None, None, None, 0, 1, dm, 0, _p(A), _p(A), wsg, None) == api.MOE_ERR_ARG
    assert g(_p(A), _p(A), _p(A), 128, _p(A + 16), stride, None, None, None, 0, 1, dm, 0, _p(A), _p(A), wsg, None) == api.MOE_ERR_ALIGN
    assert g(_p(A), _p(A), _p(A), 0, _p(A), stride, None, None, None, 0, 1, dm, 0, _p(A), _p(A), wsg, None) == api.MOE_ERR_ARG
    assert g(_p(A), _p(A), _p(A), 128, _p(A), stride, _p(A), _p(A), _p(A), 1, 1, dm, 0, _p(A), _p(A), wsg, None) == api.MOE_ERR_UNSUPPORTED
    assert g(_p(A), _p(A), _p(A), 128, _p(A), stride, _p(A), None, None, 1, 1, dm, 0, _p(A), _p(A), wsg, None) == api.MOE_ERR_ARG
    # bf16 operands are refused whatever the other arguments; the MFMA path needs the permutation
    assert g(_p(A), _p(A), _p(A), 128, _p(A), stride, _p(A), _p(A), None, 0, 1, dm, api.MOE_PREC_BF16_MFMA, _p(A),
             _p(A), 1 << 30, None) == api.MOE_ERR_UNSUPPORTED
    assert b"bf16" in lib.moe_last_error()
    assert api.moe_workspace_size(api.MOE_CALL_GATEUP, 4, dm, api.MOE_PREC_BF16_MFMA) == (1 << 64) - 1
    assert g(_p(A), _p(A), _p(A), 128, _p(A), stride, None, None, None, 0, 1, dm, 2, _p(A), _p(A), wsg, None) == api.MOE_ERR_UNSUPPORTED
    # the MFMA path keeps one LDS entry per K group of the down GEMM: f past
    # 128 groups of 64 is refused on the host for gate/up and down alike
    big = api.dims(2816, 8256, 128, 8)
    sbig = api.moe_expert_blob_bytes(big)
    for prec in (api.MOE_PREC_F16_MFMA, api.MOE_PREC_F16_MFMA_DIRECT):
        assert g(_p(A), _p(A), _p(A), 128, _p(A), sbig, _p(A), _p(A), None, 0, 1, big, prec, _p(A), _p(A),
                 1 << 30, None) == api.MOE_ERR_UNSUPPORTED
        assert b"8192" in lib.moe_last_error()
        assert lib.moe_expert_q4_down_combine(_p(A), _p(A), _p(A), _p(A), 128, _p(A), sbig, _p(A), _p(A), _p(A),
                                              None, 1, big, prec, _p(A), _p(A), 1 << 30, None) == api.MOE_ERR_UNSUPPORTED
    dc = lib.moe_expert_q4_down_combine
    wsd = api.moe_workspace_size(api.MOE_CALL_DOWN_COMBINE, 1, dm)
    assert dc(_p(A), _p(A), None, _p(A), 128, _p(A), stride, None, None, None, None, 1, dm, 0, _p(A), _p(A), wsd, None) == api.MOE_ERR_ARG
    assert dc(_p(A), _p(A), _p(A), _p(A), 128, _p(A), stride, None, None, None, _p(A + 8), 1, dm, 0, _p(A), _p(A), wsd, None) == api.MOE_ERR_ALIGN
    # the grouped down path needs per-pair outputs in its workspace
    assert api.moe_workspace_size(api.MOE_CALL_DOWN_COMBINE, 4, dm) == 4 * 8 * 2816 * 4
    assert dc(_p(A), _p(A), _p(A), _p(A), 128, _p(A), stride, _p(A), _p(A), _p(A), None, 4, dm, 0, _p(A), _p(A), 16, None) == api.MOE_ERR_CAPACITY
    # helpers
    assert lib.moe_shared_gemv_bf16(_p(A), _p(A), 1, 16, 12, _p(A), None) == api.MOE_ERR_ARG
    assert lib.moe_rms_rescale(_p(A), 1, 6, 1e-6, _p(A), None) == api.MOE_ERR_ARG


def test_cache_validation(api):
    lib = api.lib()
    A = 0x100000
    out = ctypes.c_void_p()
    blob = 3_345_408
    # slots fewer than k, more than experts, stride not a multiple of 256
    assert lib.moe_cache_create(2, 128, 4, 8, _p(A), blob, _p(A), blob, _p(A), ctypes.byref(out)) == api.MOE_ERR_ARG
    assert lib.moe_cache_create(2, 128, 129, 8, _p(A), blob, _p(A), blob, _p(A), ctypes.byref(out)) == api.MOE_ERR_ARG
    assert lib.moe_cache_create(2, 128, 64, 8, _p(A), blob, _p(A), blob + 1, _p(A), ctypes.byref(out)) == api.MOE_ERR_ARG
    assert lib.moe_cache_create(2, 128, 64, 8, None, blob, _p(A), blob, _p(A), ctypes.byref(out)) == api.MOE_ERR_ARG
    assert lib.moe_slot_stage(None, 0, 0, None, None, None, None, None, None) == api.MOE_ERR_ARG
    assert lib.moe_cache_wait(None, 0, None) == api.MOE_ERR_ARG
    assert lib.moe_status_string(api.MOE_ERR_ALIGN) == b"misaligned buffer"
