"""The C-ABI library loads on a machine without a GPU and exports what the header declares."""

import os
import re

import numpy as np
import pytest

from serving_attention_bsr_amd import lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "bsr_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsr_attn_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    so = lib.load()
    for name in declared_functions():
        assert hasattr(so, name), name


def test_abi_version():
    assert lib.bsr_attn_abi_version() == 4


def test_struct_sizes_match_header():
    # bsr_attn_config: 8 int32/float, max_batch, max_total_qo, int64, 9 int32, static_queues,
    # the ALiBi slope pointer
    assert lib.ctypes.sizeof(lib.bsr_attn_config) == 96
    assert lib.ctypes.sizeof(lib.bsr_plan_info) == 64


def test_host_only_handle_needs_workgroups():
    with pytest.raises(lib.BsrError) as e:
        lib.BsrAttention(8, 2, 64, 16, dtype="f32", device=-1)
    assert e.value.code == lib.BSR_ERR_INVALID_ARG


@pytest.mark.parametrize(
    "kw, code",
    [
        (dict(num_qo_heads=6, num_kv_heads=4), lib.BSR_ERR_INVALID_ARG),
        (dict(head_dim=96), lib.BSR_ERR_UNSUPPORTED),
        (dict(page_size=0), lib.BSR_ERR_INVALID_ARG),
        (dict(logits_soft_cap=-1.0), lib.BSR_ERR_INVALID_ARG),
        (dict(max_batch=0), lib.BSR_ERR_INVALID_ARG),
    ],
)
def test_create_rejects_bad_config(kw, code):
    args = dict(num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=16, dtype="f32", num_workgroups=4, device=-1)
    args.update(kw)
    with pytest.raises(lib.BsrError) as e:
        lib.BsrAttention(**args)
    assert e.value.code == code


def test_create_rejects_bad_cost_mfma():
    for bad in (-1, 16 * 256 + 1):
        with pytest.raises(lib.BsrError) as e:
            lib.BsrAttention(8, 2, 64, 16, num_workgroups=4, device=-1, max_batch=4, max_total_qo=4,
                             max_total_kv=64, cost_mfma=bad)
        assert e.value.code == lib.BSR_ERR_INVALID_ARG


def test_create_rejects_bad_slot2_speed():
    for bad in (-1, 65):
        with pytest.raises(lib.BsrError) as e:
            lib.BsrAttention(8, 2, 64, 16, num_workgroups=4, device=-1, max_batch=4, max_total_qo=4,
                             max_total_kv=64, slot2_speed=bad)
        assert e.value.code == lib.BSR_ERR_INVALID_ARG
    for ok in (0, 11, 16):
        lib.BsrAttention(8, 2, 64, 16, num_workgroups=4, device=-1, max_batch=4, max_total_qo=4, max_total_kv=64,
                         slot2_speed=ok).close()


def test_fp8_kv_handle_kernel_choice():
    """An FP8 K/V handle runs wide query rows on the MFMA tile body up to head dim
    128 (a decode row next to them makes the mixed kind); at head dim 256 every row
    runs on the decode body, long rows as 8-row tiles."""
    qo, kv, last = (np.array([0, 1, 41], dtype=np.int32), np.array([0, 4, 8], dtype=np.int32),
                    np.array([16, 16], dtype=np.int32))
    for d, kind, tile in ((64, lib.KERNEL_MIXED, 128), (128, lib.KERNEL_MIXED, 128), (256, lib.KERNEL_DECODE, 8)):
        h = lib.BsrAttention(8, 2, d, 16, dtype="bf16_kv_fp8", num_workgroups=8, device=-1, max_batch=4,
                             max_total_qo=64, max_total_kv=4096, causal=True)
        info = h.plan(qo, kv, last)
        assert info["kernel"] == kind and info["q_tile"] == tile, (d, info)
        h.close()
