"""ctypes binding of libbsr_attn.so (argument marshalling only).

The functions below carry the names of the C entry points declared in
include/bsr_attn.h and pass raw pointers through; every step of the attention
runs in the library's HIP kernels.  PyTorch provides device memory (workspace,
outputs) and the current stream.  If the library is missing the import fails:
there is no other implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BSR_ATTN_LIBRARY") or os.path.join(HERE, "libbsr_attn.so")

BSR_OK = 0
BSR_ERR_INVALID_ARG = 1
BSR_ERR_CAPACITY = 2
BSR_ERR_UNSUPPORTED = 3
BSR_ERR_HIP = 4
BSR_ERR_DEVICE = 5
BSR_DTYPE_F32 = 0
BSR_DTYPE_BF16 = 1
BSR_DTYPE_BF16_KV_FP8 = 2

KERNEL_DECODE = 1
KERNEL_MFMA = 2
KERNEL_MIXED = 3

EXPORTED = [
    "bsr_attn_abi_version",
    "bsr_attn_last_error",
    "bsr_attn_create",
    "bsr_attn_workspace_size",
    "bsr_attn_plan",
    "bsr_attn_plan_tree_mask",
    "bsr_attn_plan_composable",
    "bsr_attn_plan_get_info",
    "bsr_attn_run",
    "bsr_attn_run_static",
    "bsr_attn_check",
    "bsr_attn_merge_states",
    "bsr_attn_append_kv",
    "bsr_attn_plan_head_pages",
    "bsr_attn_page_summary",
    "bsr_attn_quest_select",
    "bsr_attn_destroy",
]


class BsrError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"bsr_attn error {code}: {msg}")
        self.code = code


class bsr_attn_config(ctypes.Structure):
    _fields_ = [
        ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("logits_soft_cap", ctypes.c_float),
        ("max_batch", ctypes.c_int32),
        ("max_total_qo", ctypes.c_int32),
        ("max_total_kv", ctypes.c_int64),
        ("num_workgroups", ctypes.c_int32),
        ("cost_alpha", ctypes.c_int32),
        ("cost_beta", ctypes.c_int32),
        ("min_kv_chunk", ctypes.c_int32),
        ("max_partial_rows", ctypes.c_int32),
        ("cost_item", ctypes.c_int32),
        ("cost_mfma", ctypes.c_int32),
        ("slot2_speed", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
        ("static_queues", ctypes.c_int32),
        ("alibi_slopes", ctypes.POINTER(ctypes.c_float)),
    ]


class bsr_format(ctypes.Structure):
    _fields_ = [
        ("num_block_rows", ctypes.c_int32),
        ("qo_indptr", ctypes.POINTER(ctypes.c_int32)),
        ("kv_indptr", ctypes.POINTER(ctypes.c_int32)),
        ("last_page_len", ctypes.POINTER(ctypes.c_int32)),
        ("kv_indices_offset", ctypes.c_int32),
    ]


class bsr_plan_info(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("num_workgroups", ctypes.c_int32),
        ("num_items", ctypes.c_int32),
        ("num_partial_items", ctypes.c_int32),
        ("num_partial_rows", ctypes.c_int32),
        ("num_merge_tasks", ctypes.c_int32),
        ("num_merge_sources", ctypes.c_int32),
        ("q_tile", ctypes.c_int32),
        ("kv_chunk", ctypes.c_int64),
        ("max_wg_cost", ctypes.c_int64),
        ("total_cost", ctypes.c_int64),
        ("blob_bytes", ctypes.c_int32),
        ("instance", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None
ABI_VERSION = 4  # BSR_ATTN_ABI_VERSION of the struct layouts above


def load():
    """Load libbsr_attn.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_i32, c_i64, vp = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    i32p = ctypes.POINTER(ctypes.c_int32)
    f32p = ctypes.c_void_p
    lib.bsr_attn_abi_version.restype = c_int
    lib.bsr_attn_last_error.restype = ctypes.c_char_p
    lib.bsr_attn_create.argtypes = [ctypes.POINTER(bsr_attn_config), c_int, ctypes.POINTER(vp)]
    lib.bsr_attn_workspace_size.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    lib.bsr_attn_plan.argtypes = [vp, i32p, i32p, i32p, c_i32, vp, vp, vp]
    lib.bsr_attn_plan_tree_mask.argtypes = [vp, i32p, i32p, i32p, c_i32, vp, vp, vp, vp]
    lib.bsr_attn_plan_composable.argtypes = [vp, c_i32, ctypes.POINTER(bsr_format), c_i32, vp, vp, vp]
    lib.bsr_attn_plan_get_info.argtypes = [vp, ctypes.POINTER(bsr_plan_info)]
    lib.bsr_attn_run.argtypes = [vp, vp, vp, vp, vp, vp, f32p, vp, vp]
    lib.bsr_attn_run_static.argtypes = [vp, vp, vp, vp, vp, vp, f32p, vp, vp]
    lib.bsr_attn_check.argtypes = [vp, vp, vp]
    lib.bsr_attn_merge_states.argtypes = [f32p, f32p, f32p, f32p, f32p, f32p, c_i64, c_i32, vp]
    lib.bsr_attn_append_kv.argtypes = [vp, vp, vp, vp, vp, vp, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, vp, vp,
                                       c_i64, vp]
    lib.bsr_attn_plan_head_pages.argtypes = [vp, i32p, i32p, i32p, c_i32, vp, vp, vp]
    lib.bsr_attn_page_summary.argtypes = [vp, vp, vp, vp, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_i64, vp, vp, vp]
    lib.bsr_attn_quest_select.argtypes = [vp, vp, vp, vp, vp, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32, c_i64,
                                          c_i32, vp, vp, vp, vp]
    lib.bsr_attn_destroy.argtypes = [vp]
    lib.bsr_attn_destroy.restype = None
    for name in EXPORTED:
        if name not in ("bsr_attn_last_error", "bsr_attn_destroy"):
            getattr(lib, name).restype = c_int
    if lib.bsr_attn_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.bsr_attn_abi_version()}, this binding expects "
                          f"{ABI_VERSION}; rebuild it with __graft_entry__.build()")
    _lib = lib
    return lib


def _check(rc):
    if rc != BSR_OK:
        raise BsrError(rc, load().bsr_attn_last_error().decode())


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _dptr(t):
    """Device (or host) address of a torch tensor, None stays None."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    if stream is None:
        return None
    return ctypes.c_void_p(stream.cuda_stream)


# --------------------------------------------------------------------------- #
# Entry points under their C names
# --------------------------------------------------------------------------- #

def bsr_attn_abi_version():
    return load().bsr_attn_abi_version()


def bsr_attn_create(cfg: bsr_attn_config, device: int):
    h = ctypes.c_void_p()
    _check(load().bsr_attn_create(ctypes.byref(cfg), device, ctypes.byref(h)))
    return h


def bsr_attn_workspace_size(h):
    dev, host = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().bsr_attn_workspace_size(h, ctypes.byref(dev), ctypes.byref(host)))
    return dev.value, host.value


def bsr_attn_plan(h, qo_indptr, kv_indptr, last_page_len, workspace, host_staging, stream):
    qo, kv, last = _i32(qo_indptr), _i32(kv_indptr), _i32(last_page_len)
    batch = len(qo) - 1
    _check(load().bsr_attn_plan(h, _ptr(qo), _ptr(kv), _ptr(last), batch, workspace, host_staging, stream))


def bsr_attn_plan_tree_mask(h, qo_indptr, kv_indptr, last_page_len, tree_mask_bits, workspace, host_staging,
                            stream):
    """tree_mask_bits: uint8 array, the packed bits described in the header."""
    qo, kv, last = _i32(qo_indptr), _i32(kv_indptr), _i32(last_page_len)
    bits = np.ascontiguousarray(np.asarray(tree_mask_bits, dtype=np.uint8))
    batch = len(qo) - 1
    _check(load().bsr_attn_plan_tree_mask(h, _ptr(qo), _ptr(kv), _ptr(last), batch, ctypes.c_void_p(bits.ctypes.data),
                                          workspace, host_staging, stream))


def pack_tree_masks(masks):
    """Pack per-request boolean [l_qo, l_qo] tree masks into the library's bit layout
    (request after request, row-major, least significant bit first)."""
    flat = [np.asarray(m, dtype=bool).reshape(-1) for m in masks]
    bits = np.concatenate(flat) if flat else np.zeros(0, dtype=bool)
    return np.packbits(bits, bitorder="little")


def bsr_attn_plan_composable(h, formats: Sequence[dict], total_qo, workspace, host_staging, stream):
    keep = []
    arr = (bsr_format * len(formats))()
    for i, f in enumerate(formats):
        qo, kv, last = _i32(f["qo_indptr"]), _i32(f["kv_indptr"]), _i32(f["last_page_len"])
        keep += [qo, kv, last]
        arr[i].num_block_rows = len(qo) - 1
        arr[i].qo_indptr = _ptr(qo)
        arr[i].kv_indptr = _ptr(kv)
        arr[i].last_page_len = _ptr(last)
        arr[i].kv_indices_offset = int(f["kv_indices_offset"])
    _check(load().bsr_attn_plan_composable(h, len(formats), arr, int(total_qo), workspace, host_staging, stream))


def bsr_attn_plan_get_info(h):
    info = bsr_plan_info()
    _check(load().bsr_attn_plan_get_info(h, ctypes.byref(info)))
    return info


def bsr_attn_run(h, q, k_pool, v_pool, kv_indices, o, lse, workspace, stream):
    _check(load().bsr_attn_run(h, q, k_pool, v_pool, kv_indices, o, lse, workspace, stream))


def bsr_attn_run_static(h, q, k_pool, v_pool, kv_indices, o, lse, host_staging, stream):
    _check(load().bsr_attn_run_static(h, q, k_pool, v_pool, kv_indices, o, lse, host_staging, stream))


def bsr_attn_check(h, workspace, stream):
    _check(load().bsr_attn_check(h, workspace, stream))


def bsr_attn_merge_states(o_a, lse_a, o_b, lse_b, o, lse, rows, head_dim, stream):
    _check(load().bsr_attn_merge_states(o_a, lse_a, o_b, lse_b, o, lse, rows, head_dim, stream))


def bsr_attn_append_kv(k_new, v_new, append_indptr, kv_indptr, kv_indices, last_page_len, batch, total_new,
                       num_kv_heads, head_dim, page_size, dtype, k_pool, v_pool, num_pages, stream):
    _check(load().bsr_attn_append_kv(k_new, v_new, append_indptr, kv_indptr, kv_indices, last_page_len, batch,
                                     total_new, num_kv_heads, head_dim, page_size, dtype, k_pool, v_pool, num_pages,
                                     stream))


def bsr_attn_plan_head_pages(h, qo_indptr, kv_indptr_heads, last_page_len, workspace, host_staging, stream):
    qo, kv, last = _i32(qo_indptr), _i32(kv_indptr_heads), _i32(last_page_len)
    batch = len(qo) - 1
    _check(load().bsr_attn_plan_head_pages(h, _ptr(qo), _ptr(kv), _ptr(last), batch, workspace, host_staging,
                                           stream))


def bsr_attn_page_summary(k_pool, kv_indptr, kv_indices, last_page_len, batch, num_entries, num_kv_heads, head_dim,
                          page_size, dtype, num_pages, k_min, k_max, stream):
    _check(load().bsr_attn_page_summary(k_pool, kv_indptr, kv_indices, last_page_len, batch, num_entries,
                                        num_kv_heads, head_dim, page_size, dtype, num_pages, k_min, k_max, stream))


def bsr_attn_quest_select(q, k_min, k_max, kv_indptr, kv_indices, batch, num_entries, max_pages, num_qo_heads,
                          num_kv_heads, head_dim, dtype, num_pages, page_budget, out_indptr, out_indices, scores,
                          stream):
    _check(load().bsr_attn_quest_select(q, k_min, k_max, kv_indptr, kv_indices, batch, num_entries, max_pages,
                                        num_qo_heads, num_kv_heads, head_dim, dtype, num_pages, page_budget,
                                        out_indptr, out_indices, scores, stream))


def bsr_attn_destroy(h):
    load().bsr_attn_destroy(h)


# --------------------------------------------------------------------------- #
# Convenience wrapper: owns the handle, the workspace and the staging buffer
# --------------------------------------------------------------------------- #

class BsrAttention:
    """One handle plus the caller-side buffers the C ABI asks for.

    device >= 0: workspace is a torch uint8 CUDA tensor, staging is pinned host
    memory.  device = -1: host-only (plans only, into a numpy staging buffer).
    """

    def __init__(
        self,
        num_qo_heads: int,
        num_kv_heads: int,
        head_dim: int,
        page_size: int,
        dtype: str = "bf16",
        causal: bool = False,
        sm_scale: float = 0.0,
        logits_soft_cap: float = 0.0,
        max_batch: int = 256,
        max_total_qo: int = 4096,
        max_total_kv: int = 1 << 22,
        num_workgroups: int = 0,
        device: int = 0,
        cost_alpha: int = 0,
        cost_beta: int = 0,
        min_kv_chunk: int = 0,
        max_partial_rows: int = 0,
        cost_item: int = 0,
        cost_mfma: int = 0,
        slot2_speed: int = 0,
        sliding_window: int = 0,
        alibi_slopes=None,
        static_queues: bool = False,
    ):
        cfg = bsr_attn_config()
        cfg.num_qo_heads = num_qo_heads
        cfg.num_kv_heads = num_kv_heads
        cfg.head_dim = head_dim
        cfg.page_size = page_size
        cfg.dtype = {"bf16": BSR_DTYPE_BF16, "f32": BSR_DTYPE_F32, "bf16_kv_fp8": BSR_DTYPE_BF16_KV_FP8}[dtype]
        cfg.causal = int(bool(causal))
        cfg.sm_scale = sm_scale
        cfg.logits_soft_cap = logits_soft_cap
        cfg.max_batch = max_batch
        cfg.max_total_qo = max_total_qo
        cfg.max_total_kv = max_total_kv
        cfg.num_workgroups = num_workgroups
        cfg.cost_alpha = cost_alpha
        cfg.cost_beta = cost_beta
        cfg.min_kv_chunk = min_kv_chunk
        cfg.max_partial_rows = max_partial_rows
        cfg.cost_item = cost_item
        cfg.cost_mfma = cost_mfma
        cfg.slot2_speed = slot2_speed
        cfg.sliding_window = sliding_window
        cfg.static_queues = int(static_queues)
        if alibi_slopes is not None:
            slopes = np.ascontiguousarray(np.asarray(alibi_slopes, dtype=np.float32))
            if slopes.shape != (num_qo_heads,):
                raise ValueError("alibi_slopes must hold one slope per query head")
            cfg.alibi_slopes = slopes.ctypes.data_as(ctypes.POINTER(ctypes.c_float))  # read by create only
        self.cfg = cfg
        self.dtype = dtype
        self.device = device
        self.handle = bsr_attn_create(cfg, device)
        cfg.alibi_slopes = None
        dev_bytes, host_bytes = bsr_attn_workspace_size(self.handle)
        self.workspace_bytes = dev_bytes
        if device >= 0:
            import torch

            self.workspace = torch.zeros(dev_bytes, dtype=torch.uint8, device=f"cuda:{device}")
            self.staging = torch.empty(host_bytes, dtype=torch.uint8, pin_memory=True)
            self._ws_ptr = _dptr(self.workspace)
            self._staging_ptr = _dptr(self.staging)
        else:
            self.workspace = None
            self.staging = np.zeros(host_bytes, dtype=np.uint8)
            self._ws_ptr = None
            self._staging_ptr = ctypes.c_void_p(self.staging.ctypes.data)

    def _stream(self):
        if self.device < 0:
            return None
        import torch

        return _stream_ptr(torch.cuda.current_stream(self.device))

    def plan(self, qo_indptr, kv_indptr, last_page_len, upload=True):
        """upload=False stages the plan without copying it into the workspace (for
        run_static, which uploads it into the library's static scratch)."""
        ws = self._ws_ptr if upload else None
        bsr_attn_plan(self.handle, qo_indptr, kv_indptr, last_page_len, ws, self._staging_ptr, self._stream())
        return self.info()

    def plan_tree_mask(self, qo_indptr, kv_indptr, last_page_len, masks, upload=True):
        """Plan with a tree mask per request (boolean [l_qo, l_qo] each)."""
        ws = self._ws_ptr if upload else None
        bsr_attn_plan_tree_mask(self.handle, qo_indptr, kv_indptr, last_page_len, pack_tree_masks(masks), ws,
                                self._staging_ptr, self._stream())
        return self.info()

    def plan_head_pages(self, qo_indptr, kv_indptr_heads, last_page_len, upload=True):
        """Plan with one page list per request and KV head (kv_indptr_heads: [B * H_kv + 1])."""
        ws = self._ws_ptr if upload else None
        bsr_attn_plan_head_pages(self.handle, qo_indptr, kv_indptr_heads, last_page_len, ws, self._staging_ptr,
                                 self._stream())
        return self.info()

    def plan_composable(self, formats, total_qo):
        bsr_attn_plan_composable(self.handle, formats, total_qo, self._ws_ptr, self._staging_ptr, self._stream())
        return self.info()

    def info(self):
        return bsr_attn_plan_get_info(self.handle).as_dict()

    def plan_bytes(self) -> np.ndarray:
        """Copy of the last plan as staged on the host."""
        n = self.info()["blob_bytes"]
        if self.device >= 0:
            return self.staging[:n].numpy().copy()
        return self.staging[:n].copy()

    def run(self, q, k_pool, v_pool, kv_indices, o=None, lse=None):
        import torch

        if o is None:
            o = torch.empty_like(q)
        if lse is None:
            lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
        bsr_attn_run(
            self.handle, _dptr(q), _dptr(k_pool), _dptr(v_pool), _dptr(kv_indices), _dptr(o), _dptr(lse),
            self._ws_ptr, self._stream(),
        )
        return o, lse

    def run_static(self, q, k_pool, v_pool, kv_indices, o=None, lse=None):
        """run() on the library's static scratch instead of this object's workspace."""
        import torch

        if o is None:
            o = torch.empty_like(q)
        if lse is None:
            lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
        bsr_attn_run_static(
            self.handle, _dptr(q), _dptr(k_pool), _dptr(v_pool), _dptr(kv_indices), _dptr(o), _dptr(lse),
            self._staging_ptr, self._stream(),
        )
        return o, lse

    def check(self, static=False):
        """static=True checks the runs of run_static (the static scratch)."""
        bsr_attn_check(self.handle, None if static else self._ws_ptr, self._stream())

    def close(self):
        if self.handle is not None:
            bsr_attn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def merge_states(o_a, lse_a, o_b, lse_b, o=None, lse=None):
    """⊕ of two fp32 state arrays on the GPU (o: [rows, D], lse: [rows])."""
    import torch

    rows, d = o_a.shape
    if o is None:
        o = torch.empty_like(o_a)
    if lse is None:
        lse = torch.empty_like(lse_a)
    bsr_attn_merge_states(
        _dptr(o_a), _dptr(lse_a), _dptr(o_b), _dptr(lse_b), _dptr(o), _dptr(lse), rows, d,
        _stream_ptr(torch.cuda.current_stream(o_a.device)),
    )
    return o, lse


def append_kv(k_new, v_new, append_indptr, kv_indptr, kv_indices, last_page_len, k_pool, v_pool):
    """Write new K/V rows ([total_new, H_kv, D]) into the paged pools ([num_pages, H_kv, P, D])
    in place; the index arrays are int32 tensors on the pools' device (see bsr_attn_append_kv)."""
    import torch

    for t in (k_new, v_new, k_pool, v_pool, append_indptr, kv_indptr, kv_indices, last_page_len):
        if not t.is_contiguous():
            raise ValueError("append_kv needs contiguous tensors")
    for t in (append_indptr, kv_indptr, kv_indices, last_page_len):
        if t.dtype != torch.int32:
            raise ValueError("index arrays must be int32")
    if k_new.dtype != k_pool.dtype or v_new.dtype != v_pool.dtype or k_pool.dtype != v_pool.dtype:
        raise ValueError("new rows and pools must share one dtype")
    if k_pool.dtype == torch.bfloat16:
        dtype = BSR_DTYPE_BF16
    elif k_pool.dtype == torch.float8_e4m3fn:
        dtype = BSR_DTYPE_BF16_KV_FP8
    elif k_pool.dtype == torch.float32:
        dtype = BSR_DTYPE_F32
    else:
        raise ValueError("dtype must be float32, bfloat16 or float8_e4m3fn")
    num_pages, h_kv, page_size, d = k_pool.shape
    total_new = k_new.shape[0]
    if tuple(k_new.shape) != (total_new, h_kv, d) or tuple(v_new.shape) != (total_new, h_kv, d):
        raise ValueError("k_new / v_new must be [total_new, H_kv, D] matching the pools")
    if tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("K and V pools differ in shape")
    batch = append_indptr.numel() - 1
    bsr_attn_append_kv(
        _dptr(k_new), _dptr(v_new), _dptr(append_indptr), _dptr(kv_indptr), _dptr(kv_indices), _dptr(last_page_len),
        batch, total_new, h_kv, d, page_size, dtype, _dptr(k_pool), _dptr(v_pool), num_pages,
        _stream_ptr(torch.cuda.current_stream(k_pool.device)),
    )


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return BSR_DTYPE_BF16
    if t.dtype == torch.float32:
        return BSR_DTYPE_F32
    raise ValueError("dtype must be float32 or bfloat16")


def quest_out_indptr(kv_indptr, num_kv_heads, page_budget):
    """Host CSR of the kept page lists: min(n_pages(r), budget) ids per (request, KV head)."""
    n = np.diff(np.asarray(kv_indptr, dtype=np.int64))
    kept = np.repeat(np.minimum(n, page_budget), num_kv_heads)
    return np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)


def page_summary(k_pool, kv_indptr, kv_indices, last_page_len, k_min=None, k_max=None):
    """Per-page key min/max ([num_pages, H_kv, D], the pool's dtype) of a page table's pages."""
    import torch

    num_pages, h_kv, page_size, d = k_pool.shape
    if k_min is None:
        k_min = torch.zeros((num_pages, h_kv, d), dtype=k_pool.dtype, device=k_pool.device)
    if k_max is None:
        k_max = torch.zeros((num_pages, h_kv, d), dtype=k_pool.dtype, device=k_pool.device)
    batch = kv_indptr.numel() - 1
    bsr_attn_page_summary(_dptr(k_pool), _dptr(kv_indptr), _dptr(kv_indices), _dptr(last_page_len), batch,
                          kv_indices.numel(), h_kv, d, page_size, _dtype_code(k_pool), num_pages, _dptr(k_min),
                          _dptr(k_max), _stream_ptr(torch.cuda.current_stream(k_pool.device)))
    return k_min, k_max


def quest_select(q, k_min, k_max, kv_indptr, kv_indices, page_budget, out_indptr, max_pages, out_indices=None,
                 scores=None):
    """Kept page ids per (request, KV head) into out_indices (CSR out_indptr, device int32)."""
    import torch

    batch, h_qo, d = q.shape
    num_pages, h_kv, _ = k_min.shape
    entries = kv_indices.numel()
    if out_indices is None:
        out_indices = torch.empty(max(int(out_indptr[-1].item()), 1), dtype=torch.int32, device=q.device)
    if scores is None:
        scores = torch.empty(max(h_kv * entries, 1), dtype=torch.float32, device=q.device)
    bsr_attn_quest_select(_dptr(q), _dptr(k_min), _dptr(k_max), _dptr(kv_indptr), _dptr(kv_indices), batch, entries,
                          max_pages, h_qo, h_kv, d, _dtype_code(q), num_pages, page_budget, _dptr(out_indptr),
                          _dptr(out_indices), _dptr(scores), _stream_ptr(torch.cuda.current_stream(q.device)))
    return out_indices
