"""ctypes binding of libfia.so (include/fia.h).

Argument marshalling only: torch provides device memory and the stream;
every step of the computation runs in the library's HIP kernels.  The library
is loaded on first use and a missing build raises ``FiaNotBuilt``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfia.so")

FIA_SUCCESS = 0
FIA_ERR_NULLPTR = 1
FIA_ERR_PARAM_INVALID = 2
FIA_ERR_UNSUPPORTED = 3
FIA_ERR_WORKSPACE = 4
FIA_ERR_HIP = 5
STATUS_NAMES = {0: "SUCCESS", 1: "ERR_NULLPTR", 2: "ERR_PARAM_INVALID", 3: "ERR_UNSUPPORTED",
                4: "ERR_WORKSPACE", 5: "ERR_HIP"}

DT_BF16, DT_FP16, DT_FP32, DT_FP8_E4M3FN, DT_INT32, DT_INT64, DT_UINT8, DT_INT8, DT_BOOL = range(9)
_TORCH_DT = {
    torch.bfloat16: DT_BF16, torch.float16: DT_FP16, torch.float32: DT_FP32,
    torch.float8_e4m3fn: DT_FP8_E4M3FN, torch.int32: DT_INT32, torch.int64: DT_INT64,
    torch.uint8: DT_UINT8, torch.int8: DT_INT8, torch.bool: DT_BOOL,
}

KIND_NAMES = {0: "fill", 1: "prefill", 2: "decode", 3: "sparse", 4: "fp32"}

EXPORTED = ["fia_get_workspace_size", "fia_sparse_get_workspace_size",
            "fia_sparse_flash_mla_get_workspace_size", "fia_run", "fia_run_no_alloc",
            "fia_executor_destroy", "fia_last_error", "fia_executor_kind",
            "fia_debug_gather_kv", "fia_debug_read_kv", "fia_debug_sparse_rows", "fia_peak_mfma_bf16",
            "fia_peak_hbm_read"]


class FiaNotBuilt(RuntimeError):
    pass


class FiaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class FiaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 5), ("stride", ctypes.c_int64 * 5)]


class FiaParams(ctypes.Structure):
    _fields_ = [
        ("input_layout", ctypes.c_char_p),
        ("num_heads", ctypes.c_int32),
        ("num_key_value_heads", ctypes.c_int32),
        ("scale_value", ctypes.c_double),
        ("sparse_mode", ctypes.c_int32),
        ("pre_tokens", ctypes.c_int64),
        ("next_tokens", ctypes.c_int64),
        ("pse_type", ctypes.c_int32),
        ("q_start_idx", ctypes.c_int64),
        ("kv_start_idx", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("inner_precise", ctypes.c_int32),
        ("softmax_lse_flag", ctypes.c_int32),
        ("actual_seq_lengths", ctypes.POINTER(ctypes.c_int64)),
        ("actual_seq_lengths_len", ctypes.c_int64),
        ("actual_seq_lengths_kv", ctypes.POINTER(ctypes.c_int64)),
        ("actual_seq_lengths_kv_len", ctypes.c_int64),
        ("kv_layout", ctypes.c_char_p),
        ("learnable_sink", ctypes.POINTER(FiaTensor)),
        ("key_antiquant_mode", ctypes.c_int32),
        ("value_antiquant_mode", ctypes.c_int32),
        ("key_antiquant_scale", ctypes.POINTER(FiaTensor)),
        ("value_antiquant_scale", ctypes.POINTER(FiaTensor)),
        ("key_antiquant_offset", ctypes.POINTER(FiaTensor)),
        ("value_antiquant_offset", ctypes.POINTER(FiaTensor)),
        ("actual_seq_lengths_kv_device", ctypes.POINTER(FiaTensor)),
        ("max_actual_seq_length_kv", ctypes.c_int64),
    ]


class FiaSparseParams(ctypes.Structure):
    _fields_ = [
        ("softmax_scale", ctypes.c_double),
        ("kv_quant_mode", ctypes.c_int32),
        ("tile_size", ctypes.c_int32),
        ("rope_head_dim", ctypes.c_int32),
        ("cmp_ratio", ctypes.c_int32),
        ("ori_mask_mode", ctypes.c_int32),
        ("cmp_mask_mode", ctypes.c_int32),
        ("ori_win_left", ctypes.c_int32),
        ("ori_win_right", ctypes.c_int32),
        ("layout_q", ctypes.c_char_p),
        ("layout_kv", ctypes.c_char_p),
        ("return_softmax_lse", ctypes.c_int32),
    ]


class FiaSfmlaParams(ctypes.Structure):
    _fields_ = [
        ("softmax_scale", ctypes.c_double),
        ("cmp_ratio", ctypes.c_int32),
        ("ori_mask_mode", ctypes.c_int32),
        ("cmp_mask_mode", ctypes.c_int32),
        ("ori_win_left", ctypes.c_int32),
        ("ori_win_right", ctypes.c_int32),
        ("layout_q", ctypes.c_char_p),
        ("layout_kv", ctypes.c_char_p),
        ("return_softmax_lse", ctypes.c_int32),
    ]


_LIB = None
_TP = ctypes.POINTER(FiaTensor)


def lib():
    """Load libfia.so (once).  Raises FiaNotBuilt when it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise FiaNotBuilt(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.fia_get_workspace_size.restype = ctypes.c_int
    L.fia_get_workspace_size.argtypes = [ctypes.POINTER(FiaParams), _TP, _TP, _TP, _TP, _TP, _TP,
                                         _TP, _TP, ctypes.POINTER(sz), ctypes.POINTER(vp)]
    L.fia_sparse_get_workspace_size.restype = ctypes.c_int
    L.fia_sparse_get_workspace_size.argtypes = [ctypes.POINTER(FiaSparseParams), _TP, _TP, _TP, _TP,
                                                _TP, _TP, _TP, _TP, _TP, ctypes.c_int64, _TP, _TP,
                                                _TP, ctypes.POINTER(sz), ctypes.POINTER(vp)]
    L.fia_sparse_flash_mla_get_workspace_size.restype = ctypes.c_int
    L.fia_sparse_flash_mla_get_workspace_size.argtypes = (
        [ctypes.POINTER(FiaSfmlaParams)] + [_TP] * 12 + [ctypes.c_int64] + [_TP] * 4 +
        [ctypes.POINTER(sz), ctypes.POINTER(vp)])
    L.fia_run.restype = ctypes.c_int
    L.fia_run.argtypes = [vp, sz, vp, vp]
    L.fia_run_no_alloc.restype = ctypes.c_int
    L.fia_run_no_alloc.argtypes = [vp, vp]
    L.fia_executor_destroy.restype = None
    L.fia_executor_destroy.argtypes = [vp]
    L.fia_last_error.restype = ctypes.c_char_p
    L.fia_last_error.argtypes = []
    L.fia_executor_kind.restype = ctypes.c_int32
    L.fia_executor_kind.argtypes = [vp]
    L.fia_debug_gather_kv.restype = ctypes.c_int
    L.fia_debug_gather_kv.argtypes = [vp, vp, sz, ctypes.c_int32, vp, vp]
    L.fia_debug_read_kv.restype = ctypes.c_int
    L.fia_debug_read_kv.argtypes = [vp, vp, sz, ctypes.c_int32, vp, ctypes.POINTER(ctypes.c_int64), vp]
    L.fia_debug_sparse_rows.restype = ctypes.c_int
    L.fia_debug_sparse_rows.argtypes = [vp, vp, sz, vp, vp, ctypes.POINTER(ctypes.c_int32), vp]
    L.fia_peak_mfma_bf16.restype = ctypes.c_int
    L.fia_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp]
    L.fia_peak_hbm_read.restype = ctypes.c_int
    L.fia_peak_hbm_read.argtypes = [vp, sz, ctypes.c_int32, vp, vp]
    _LIB = L
    return L


def _check(status: int):
    if status != FIA_SUCCESS:
        raise FiaError(status, lib().fia_last_error().decode(errors="replace"))


def describe(t: Optional[torch.Tensor]):
    """fia_tensor descriptor of a torch tensor (None -> NULL pointer)."""
    if t is None:
        return None
    if t.dtype not in _TORCH_DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > 5 or t.dim() < 1:
        raise ValueError("tensors must have 1..5 dims")
    d = FiaTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _TORCH_DT[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ptr(desc):
    return ctypes.pointer(desc) if desc is not None else None


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _int64_array(vals):
    if vals is None:
        return None, 0
    vals = [int(v) for v in vals]
    arr = (ctypes.c_int64 * max(1, len(vals)))(*vals)
    return arr, len(vals)


class _Plan:
    _exec = None

    def _alloc_workspace(self, device):
        self.workspace = torch.empty(max(1, self.workspace_size), dtype=torch.uint8, device=device)

    @property
    def kind(self) -> str:
        return KIND_NAMES.get(lib().fia_executor_kind(self._exec), "?")

    def run(self, stream=None):
        """Enqueue the planned attention on ``stream`` (default: current)."""
        _check(lib().fia_run(self.workspace.data_ptr(), self.workspace.numel(), self._exec,
                             _stream_handle(stream)))
        return self

    def run_no_alloc(self, stream=None):
        """Enqueue the planned attention without the plan's own workspace:
        fia_run_no_alloc, on the library's static device scratch."""
        _check(lib().fia_run_no_alloc(self._exec, _stream_handle(stream)))
        return self

    def close(self):
        if self._exec is not None and _LIB is not None:
            _LIB.fia_executor_destroy(self._exec)
        self._exec = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class AttentionPlan(_Plan):
    """Phase 1 of the dense / paged operator on torch tensors (see fia.h).

    Allocates ``attention_out`` / ``softmax_lse`` when not given, and the
    workspace.  ``run()`` enqueues phase 2; it may be called repeatedly.
    """

    def __init__(self, query, key, value, *, num_heads, num_key_value_heads=0,
                 scale_value, input_layout="BSND", sparse_mode=0, pre_tokens=2147483647,
                 next_tokens=2147483647, pse_type=0, pse_shift=None, q_start_idx=0,
                 kv_start_idx=0, atten_mask=None, block_table=None, block_size=0,
                 inner_precise=0, softmax_lse_flag=False, actual_seq_lengths=None,
                 actual_seq_lengths_kv=None, attention_out=None, softmax_lse=None,
                 kv_layout="PA_ND", learnable_sink=None, key_antiquant_mode=0,
                 value_antiquant_mode=0, key_antiquant_scale=None, value_antiquant_scale=None,
                 key_antiquant_offset=None, value_antiquant_offset=None,
                 actual_seq_lengths_kv_device=None, max_actual_seq_length_kv=0):
        L = lib()
        if attention_out is None:
            attention_out = torch.empty_like(query)
        if softmax_lse_flag and softmax_lse is None:
            if input_layout == "TND":
                shape = (query.shape[0], num_heads, 1)
            elif input_layout == "BNSD":
                shape = (query.shape[0], num_heads, query.shape[2], 1)
            else:
                shape = (query.shape[0], num_heads, query.shape[1], 1)
            softmax_lse = torch.empty(shape, dtype=torch.float32, device=query.device)
        self.query, self.key, self.value = query, key, value
        self.pse_shift, self.atten_mask, self.block_table = pse_shift, atten_mask, block_table
        self.out, self.lse = attention_out, softmax_lse
        self._lens = _int64_array(actual_seq_lengths)
        self._lens_kv = _int64_array(actual_seq_lengths_kv)
        p = FiaParams()
        p.input_layout = input_layout.encode()
        p.num_heads = num_heads
        p.num_key_value_heads = num_key_value_heads
        p.scale_value = scale_value
        p.sparse_mode = sparse_mode
        p.pre_tokens = pre_tokens
        p.next_tokens = next_tokens
        p.pse_type = pse_type
        p.q_start_idx = q_start_idx
        p.kv_start_idx = kv_start_idx
        p.block_size = block_size
        p.inner_precise = inner_precise
        p.softmax_lse_flag = 1 if softmax_lse_flag else 0
        p.kv_layout = kv_layout.encode()
        self.learnable_sink = learnable_sink
        self._sink_desc = describe(learnable_sink) if learnable_sink is not None else None
        if self._sink_desc is not None:
            p.learnable_sink = ctypes.pointer(self._sink_desc)
        p.key_antiquant_mode = key_antiquant_mode
        p.value_antiquant_mode = value_antiquant_mode
        self._aq = (key_antiquant_scale, value_antiquant_scale, key_antiquant_offset,
                    value_antiquant_offset)
        self._aq_descs = [describe(t) if t is not None else None for t in self._aq]
        for name, d in zip(("key_antiquant_scale", "value_antiquant_scale", "key_antiquant_offset",
                            "value_antiquant_offset"), self._aq_descs):
            if d is not None:
                setattr(p, name, ctypes.pointer(d))
        if self._lens[0] is not None:
            p.actual_seq_lengths = ctypes.cast(self._lens[0], ctypes.POINTER(ctypes.c_int64))
            p.actual_seq_lengths_len = self._lens[1]
        if self._lens_kv[0] is not None:
            p.actual_seq_lengths_kv = ctypes.cast(self._lens_kv[0], ctypes.POINTER(ctypes.c_int64))
            p.actual_seq_lengths_kv_len = self._lens_kv[1]
        # KV lengths on the device (int32 [B]): read by the partitioner kernel
        # at every run, so they may change between runs without a new plan.
        self.lengths_kv_device = actual_seq_lengths_kv_device
        self._dev_len_desc = (describe(actual_seq_lengths_kv_device)
                              if actual_seq_lengths_kv_device is not None else None)
        if self._dev_len_desc is not None:
            p.actual_seq_lengths_kv_device = ctypes.pointer(self._dev_len_desc)
        p.max_actual_seq_length_kv = int(max_actual_seq_length_kv)
        self._params = p
        self.batch = (len(actual_seq_lengths) if input_layout == "TND" else query.shape[0])
        descs = [describe(t) for t in (query, key, value, pse_shift, atten_mask, block_table,
                                       attention_out, softmax_lse if softmax_lse_flag else None)]
        self._descs = descs
        ws = ctypes.c_size_t(0)
        ex = ctypes.c_void_p(None)
        _check(L.fia_get_workspace_size(ctypes.byref(p), *[_ptr(d) for d in descs],
                                        ctypes.byref(ws), ctypes.byref(ex)))
        self._exec = ex
        self.workspace_size = ws.value
        self._alloc_workspace(query.device)

    def debug_gather(self, which: int, s2max: int, stream=None) -> torch.Tensor:
        """Rows 0..Lk-1 of key (0) / value (1) per batch, gathered by the
        library's row-address function into [B, s2max, KV_N, D]."""
        kvn = self._params.num_key_value_heads or self._params.num_heads
        D = self.query.shape[-1]
        dst = torch.zeros((self.batch, s2max, kvn, D), dtype=self.key.dtype, device=self.key.device)
        _check(lib().fia_debug_gather_kv(self._exec, self.workspace.data_ptr(),
                                         self.workspace.numel(), which, dst.data_ptr(),
                                         _stream_handle(stream)))
        return dst

    def read_kv(self, order, out=None, stream=None):
        """fia_debug_read_kv: read every visible key / value row once in the
        given order (0: per KV head, 1: whole token rows); returns the
        per-workgroup XOR words (a uint32 tensor on the device, viewed as
        int32)."""
        n = ctypes.c_int64(0)
        _check(lib().fia_debug_read_kv(self._exec, None, 0, order, None, ctypes.byref(n), None))
        if out is None or out.numel() < n.value:
            out = torch.empty(max(1, n.value), dtype=torch.int32, device=self.workspace.device)
        n = ctypes.c_int64(out.numel())
        _check(lib().fia_debug_read_kv(self._exec, self.workspace.data_ptr(), self.workspace.numel(),
                                       order, out.data_ptr(), ctypes.byref(n), _stream_handle(stream)))
        return out[: n.value]


def fused_infer_attention_score(query, key, value, **kw):
    """One-shot call: returns (attention_out, softmax_lse or None)."""
    plan = AttentionPlan(query, key, value, **kw)
    plan.run()
    return plan.out, plan.lse


class SparsePlan(_Plan):
    """Phase 1 of the shared-KV sparse decode on torch tensors (see fia.h)."""

    def __init__(self, q, ori_kv, cmp_kv, cmp_sparse_indices, ori_block_table, cmp_block_table,
                 seqused_kv, sinks, *, softmax_scale, max_seqused_kv, cmp_ratio=4,
                 ori_win_left=127, ori_win_right=0, ori_mask_mode=4, cmp_mask_mode=3,
                 kv_quant_mode=1, tile_size=64, rope_head_dim=64, layout_q="BSND",
                 layout_kv="PA_ND", return_softmax_lse=False, ori_sparse_indices=None,
                 cu_seqlens_q=None, attention_out=None):
        L = lib()
        if attention_out is None:
            attention_out = torch.empty_like(q)
        self.tensors = (q, ori_kv, cmp_kv, cmp_sparse_indices, ori_block_table, cmp_block_table,
                        seqused_kv, sinks, ori_sparse_indices, cu_seqlens_q)
        self.out = attention_out
        self.lse = None   # reserved on the page: not produced
        p = FiaSparseParams()
        p.softmax_scale = softmax_scale
        p.kv_quant_mode = kv_quant_mode
        p.tile_size = tile_size
        p.rope_head_dim = rope_head_dim
        p.cmp_ratio = cmp_ratio
        p.ori_mask_mode = ori_mask_mode
        p.cmp_mask_mode = cmp_mask_mode
        p.ori_win_left = ori_win_left
        p.ori_win_right = ori_win_right
        p.layout_q = layout_q.encode()
        p.layout_kv = layout_kv.encode()
        p.return_softmax_lse = 1 if return_softmax_lse else 0
        self._params = p
        d = [describe(t) for t in (q, ori_kv, cmp_kv, ori_sparse_indices, cmp_sparse_indices,
                                   ori_block_table, cmp_block_table, cu_seqlens_q, seqused_kv)]
        ds, dout = describe(sinks), describe(attention_out)
        self._descs = d + [ds, dout]
        ws = ctypes.c_size_t(0)
        ex = ctypes.c_void_p(None)
        _check(L.fia_sparse_get_workspace_size(ctypes.byref(p), *[_ptr(x) for x in d],
                                               int(max_seqused_kv), _ptr(ds), None, _ptr(dout),
                                               ctypes.byref(ws), ctypes.byref(ex)))
        self._exec = ex
        self.workspace_size = ws.value
        self._alloc_workspace(q.device)

    row_bytes = 640

    def debug_rows(self, stream=None):
        """(ids [B, S1, n_slots] int32, rows [B, S1, n_slots, row bytes] uint8)
        as the kernel gathers them; [T1, n_slots] and [T1, n_slots, row bytes]
        with TND (640 bytes per packed row, 1024 per fp16 / bf16 row)."""
        n = ctypes.c_int32(0)
        _check(lib().fia_debug_sparse_rows(self._exec, None, 0, None, None, ctypes.byref(n), None))
        lead = tuple(self.tensors[0].shape[:-2])
        dev = self.tensors[0].device
        ids = torch.empty(lead + (n.value,), dtype=torch.int32, device=dev)
        rows = torch.empty(lead + (n.value, self.row_bytes), dtype=torch.uint8, device=dev)
        _check(lib().fia_debug_sparse_rows(self._exec, self.workspace.data_ptr(),
                                           self.workspace.numel(), ids.data_ptr(),
                                           rows.data_ptr(), ctypes.byref(n),
                                           _stream_handle(stream)))
        return ids, rows


def kv_quant_sparse_attn_sharedkv(q, ori_kv, cmp_kv, cmp_sparse_indices, ori_block_table,
                                  cmp_block_table, seqused_kv, sinks, **kw):
    """One-shot call of the shared-KV sparse decode; returns attention_out."""
    plan = SparsePlan(q, ori_kv, cmp_kv, cmp_sparse_indices, ori_block_table, cmp_block_table,
                      seqused_kv, sinks, **kw)
    plan.run()
    return plan.out


class SparseFlashMlaPlan(SparsePlan):
    """Phase 1 of sparse_flash_mla (fp16 / bf16 rows) on torch tensors (see
    fia.h).  Allocates ``attention_out`` and, with ``return_softmax_lse``,
    ``softmax_lse`` ([B, 1, S1, N1] or [1, T1, N1]) when not given."""

    row_bytes = 1024

    def __init__(self, q, ori_kv, *, seqused_kv, softmax_scale, max_seqused_kv, cmp_kv=None,
                 cmp_sparse_indices=None, ori_block_table=None, cmp_block_table=None,
                 cu_seqlens_q=None, cu_seqlens_ori_kv=None, cu_seqlens_cmp_kv=None, sinks=None,
                 cmp_ratio=1, ori_mask_mode=4, cmp_mask_mode=None, ori_win_left=127,
                 ori_win_right=0, layout_q="BSND", layout_kv="PA_BBND",
                 return_softmax_lse=False, ori_sparse_indices=None, seqused_q=None,
                 attention_out=None, softmax_lse=None):
        L = lib()
        if attention_out is None:
            attention_out = torch.empty_like(q)
        if return_softmax_lse and softmax_lse is None:
            if layout_q == "TND":
                shape = (1, q.shape[0], q.shape[1])
            else:
                shape = (q.shape[0], 1, q.shape[1], q.shape[2])
            softmax_lse = torch.empty(shape, dtype=torch.float32, device=q.device)
        if cmp_mask_mode is None:
            cmp_mask_mode = 0 if cmp_kv is None else 3
        self.tensors = (q, ori_kv, cmp_kv, cmp_sparse_indices, ori_block_table, cmp_block_table,
                        cu_seqlens_q, cu_seqlens_ori_kv, cu_seqlens_cmp_kv, seqused_kv, sinks,
                        ori_sparse_indices, seqused_q)
        self.out, self.lse = attention_out, softmax_lse if return_softmax_lse else None
        p = FiaSfmlaParams()
        p.softmax_scale = softmax_scale
        p.cmp_ratio = cmp_ratio
        p.ori_mask_mode = ori_mask_mode
        p.cmp_mask_mode = cmp_mask_mode
        p.ori_win_left = ori_win_left
        p.ori_win_right = ori_win_right
        p.layout_q = layout_q.encode()
        p.layout_kv = layout_kv.encode()
        p.return_softmax_lse = 1 if return_softmax_lse else 0
        self._params = p
        d = [describe(t) for t in (q, ori_kv, cmp_kv, ori_sparse_indices, cmp_sparse_indices,
                                   ori_block_table, cmp_block_table, cu_seqlens_q,
                                   cu_seqlens_ori_kv, cu_seqlens_cmp_kv, seqused_q, seqused_kv)]
        tail = [describe(sinks), None, describe(attention_out),
                describe(softmax_lse) if return_softmax_lse else None]
        self._descs = d + tail
        ws = ctypes.c_size_t(0)
        ex = ctypes.c_void_p(None)
        _check(L.fia_sparse_flash_mla_get_workspace_size(
            ctypes.byref(p), *[_ptr(x) for x in d], int(max_seqused_kv), *[_ptr(x) for x in tail],
            ctypes.byref(ws), ctypes.byref(ex)))
        self._exec = ex
        self.workspace_size = ws.value
        self._alloc_workspace(q.device)


def sparse_flash_mla(q, ori_kv, **kw):
    """One-shot call of sparse_flash_mla; returns (attention_out, softmax_lse or None)."""
    plan = SparseFlashMlaPlan(q, ori_kv, **kw)
    plan.run()
    return plan.out, plan.lse
