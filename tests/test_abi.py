"""Host-side checks of the C-ABI library that need no GPU: it loads, exports every
function include/ctg_moe.h declares, and rejects bad configurations before it
touches the device."""
import ctypes
import os

import pytest

from combine_top_gate_amd import binding
from conftest import gpu_available


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libctg_moe.so is not built (python -m combine_top_gate_amd.build)")
    return binding.load()


def test_exports_every_declared_function(lib):
    names = binding.header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    # and nothing declared is missing from the binding's prototypes
    for n in ("moe_dispatch", "moe_grouped_gemm", "moe_combine", "moe_layer"):
        assert n in names


def test_status_strings(lib):
    assert lib.moe_status_str(0) == b"MOE_OK"
    assert lib.moe_status_str(1) == b"MOE_ERR_INVALID_ARG"
    assert lib.moe_status_str(4) == b"MOE_ERR_DEVICE"


def _create(lib, cfg):
    ctx = ctypes.c_void_p()
    st = lib.moe_create(ctypes.byref(cfg), ctypes.byref(ctx))
    return st, ctx, lib.moe_last_error_message().decode()


@pytest.mark.parametrize("field,value,needle", [
    ("hidden", 100, "hidden"), ("hidden", 16384 + 128, "hidden"), ("inter", 0, "inter"),
    ("inter", 16384 + 128, "inter"), ("n_src", 0, "n_src"),
    ("n_src", 33, "n_src"), ("topk", 0, "topk"), ("n_experts", 300, "n_experts"),
    ("shared_inter", 64, "shared_inter"), ("max_tokens", -1, "max_tokens"),
    ("out", binding.MOE_F32, "dtype"), ("weight", binding.MOE_F32, "dtype"),
    ("sched", 7, "schedule"), ("dispatch_cus", 12, "dispatch_cus"), ("dispatch_cus", -8, "dispatch_cus"),
])
def test_invalid_configs_rejected_on_host(lib, field, value, needle):
    cfg = binding.make_config(8, 16, 7168, 2048, 32, 8)
    setattr(cfg, field, value)
    st, ctx, msg = _create(lib, cfg)
    assert st == binding.MOE_ERR_INVALID_ARG
    assert needle in msg
    assert not ctx.value


def test_topk_above_experts_rejected(lib):
    cfg = binding.make_config(2, 4, 256, 128, 4, 5)
    st, _, msg = _create(lib, cfg)
    assert st == binding.MOE_ERR_INVALID_ARG and "topk" in msg


def test_null_arguments(lib):
    assert lib.moe_create(None, None) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(None, 1, None, None, None, None) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_destroy(None) == binding.MOE_OK


@pytest.mark.skipif(gpu_available(), reason="checks the no-device error path")
def test_valid_config_without_device_is_hip_error(lib):
    cfg = binding.make_config(2, 4, 256, 128, 4, 2)
    st, ctx, msg = _create(lib, cfg)
    assert st == binding.MOE_ERR_HIP and not ctx.value


# Fake, never-dereferenced device addresses: every case below must be refused on
# the host before anything reaches the device.
_A16 = ctypes.c_void_p(0x10000)
_A4 = ctypes.c_void_p(0x10004)


@pytest.mark.parametrize("T,H,E,x,wr,lg,needle", [
    (-1, 256, 8, _A16, _A16, _A16, "T"),
    (4, 100, 8, _A16, _A16, _A16, "H"),
    (4, 0, 8, _A16, _A16, _A16, "H"),
    (4, 256, 0, _A16, _A16, _A16, "E"),
    (4, 256, 257, _A16, _A16, _A16, "E"),
    (4, 256, 8, None, _A16, _A16, "NULL"),
    (4, 256, 8, _A4, _A16, _A16, "aligned"),
    (4, 256, 8, _A16, _A16, ctypes.c_void_p(0x10002), "aligned"),
])
def test_router_logits_rejects_bad_arguments(lib, T, H, E, x, wr, lg, needle):
    assert lib.moe_router_logits(T, H, E, x, wr, lg, None) == binding.MOE_ERR_INVALID_ARG
    assert needle in lib.moe_last_error_message().decode()


@pytest.mark.parametrize("T,E,k,lg,ids,w,needle", [
    (-1, 8, 2, _A16, _A16, _A16, "T"),
    (4, 0, 1, _A16, _A16, _A16, "E"),
    (4, 300, 8, _A16, _A16, _A16, "E"),
    (4, 8, 0, _A16, _A16, _A16, "k"),
    (4, 8, 9, _A16, _A16, _A16, "k"),
    (4, 64, 17, _A16, _A16, _A16, "k"),
    (4, 8, 2, _A16, None, _A16, "NULL"),
    (4, 8, 2, _A16, _A16, ctypes.c_void_p(0x10001), "aligned"),
])
def test_topk_softmax_rejects_bad_arguments(lib, T, E, k, lg, ids, w, needle):
    assert lib.moe_topk_softmax(T, E, k, lg, ids, w, None) == binding.MOE_ERR_INVALID_ARG
    assert needle in lib.moe_last_error_message().decode()


def test_gate_calls_with_no_tokens_are_no_ops(lib):
    assert lib.moe_router_logits(0, 256, 8, None, None, None, None) == binding.MOE_OK
    assert lib.moe_topk_softmax(0, 8, 2, None, None, None, None) == binding.MOE_OK


def test_gate_workspace_sizes(lib):
    # 128 tokens x 256 experts: 16 tiles of 16 experts x 128 tokens, so K is split 16 ways
    assert lib.moe_gate_workspace_bytes(128, 7168, 256) == 16 * 128 * 256 * 4
    # 4096 tokens already give 512 tiles: no split
    assert lib.moe_gate_workspace_bytes(4096, 7168, 256) == 4096 * 256 * 4
    # a small batch is split 16 ways too
    assert lib.moe_gate_workspace_bytes(8, 7168, 256) == 16 * 8 * 256 * 4
    # from 256 tokens the router runs on 64 x 64 LDS tiles: 512 tokens give 32 tiles, so
    # K is split 8 ways (about 256 workgroups; 8 x 512 partial rows fit the 4096-row bound)
    assert lib.moe_gate_workspace_bytes(512, 7168, 256) == 8 * 512 * 256 * 4
    # 1024 tokens: 64 tiles want a 4-way split, which the 4096-row bound allows
    assert lib.moe_gate_workspace_bytes(1024, 7168, 256) == 4 * 1024 * 256 * 4
    # a short K cannot be split below 8 steps per slice
    assert lib.moe_gate_workspace_bytes(8, 256, 8) == 8 * 8 * 4
    assert lib.moe_gate_workspace_bytes(100, 2816, 256) == 11 * 100 * 256 * 4
    for bad in ((0, 256, 8), (4, 0, 8), (4, 256, 0), (-1, 256, 8)):
        assert lib.moe_gate_workspace_bytes(*bad) == 0


@pytest.mark.parametrize("T,H,E,k,ws,nbytes,needle", [
    (4, 100, 8, 2, _A16, 1 << 20, "H"),
    (4, 256, 300, 2, _A16, 1 << 20, "E"),
    (4, 256, 8, 9, _A16, 1 << 20, "k"),
    (4, 256, 8, 2, None, 1 << 20, "NULL"),
    (4, 256, 8, 2, _A4, 1 << 20, "aligned"),
    (4, 256, 8, 2, _A16, 4 * 8 * 4 - 4, "workspace"),
])
def test_fused_gate_rejects_bad_arguments(lib, T, H, E, k, ws, nbytes, needle):
    st = lib.moe_gate(T, H, E, k, _A16, _A16, ws, nbytes, None, _A16, _A16, None)
    assert st == binding.MOE_ERR_INVALID_ARG
    assert needle in lib.moe_last_error_message().decode()


def test_mfma_probe_rejects_bad_arguments(lib):
    assert lib.moe_mfma_fp8_probe(None, 4, 4, None) == -1
    assert lib.moe_mfma_fp8_probe(ctypes.c_void_p(0x10002), 4, 4, None) == -1
    assert lib.moe_mfma_fp8_probe(_A16, 0, 4, None) == -1
    assert lib.moe_mfma_fp8_probe(_A16, 4, 0, None) == -1


def test_mfma_dot_rejects_bad_arguments(lib):
    inv = binding.MOE_ERR_INVALID_ARG
    assert lib.moe_mfma_dot16x16(binding.MOE_BF16, _A16, _A16, _A16, None) == inv
    assert lib.moe_mfma_dot16x16(binding.MOE_FP8_E4M3, None, _A16, _A16, None) == inv
    assert lib.moe_mfma_dot16x16(binding.MOE_FP4_E2M1, _A16, None, _A16, None) == inv
    assert lib.moe_mfma_dot16x16(binding.MOE_FP8_E4M3, _A16, _A16, ctypes.c_void_p(0x10002), None) == inv


@pytest.mark.parametrize("T,H,E,k,needle", [
    (4097, 7168, 256, 8, "scratch"),   # 4097 x 256 fp32 partial sums exceed the 4 MiB array
    (-1, 256, 8, 2, "T"),
    (4, 100, 8, 2, "H"),
    (4, 256, 300, 2, "E"),
    (4, 256, 8, 9, "k"),
])
def test_noalloc_gate_rejects_bad_arguments(lib, T, H, E, k, needle):
    st = lib.moe_gate_noalloc(T, H, E, k, _A16, _A16, None, _A16, _A16, None)
    assert st == binding.MOE_ERR_INVALID_ARG
    assert needle in lib.moe_last_error_message().decode()


def test_noalloc_gate_null_and_empty(lib):
    assert lib.moe_gate_noalloc(0, 256, 8, 2, None, None, None, None, None, None) == binding.MOE_OK
    assert lib.moe_gate_noalloc(4, 256, 8, 2, None, _A16, None, _A16, _A16, None) == binding.MOE_ERR_INVALID_ARG
    # the largest shape it takes: 4096 tokens x 256 experts (no K split) fill the array exactly
    assert lib.moe_gate_workspace_bytes(4096, 7168, 256) == 4 << 20
