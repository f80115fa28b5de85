"""Move seeded workloads (numpy, from ``workloads``) onto the GPU as torch
tensors and build library plans for them.  Marshalling only."""
from __future__ import annotations

import numpy as np
import torch

from . import fia
from .workloads import DenseCase, SfmlaCase, SparseCase


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> torch.bfloat16; other arrays as they are."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def kv_to_device(arr: np.ndarray, case: DenseCase, device) -> torch.Tensor:
    """Key / value rows: the query dtype, or fake-quantised int8 / e4m3fn codes."""
    if case.kv_quant is None:
        return to_device(arr, case.dtype, device)
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if case.kv_quant["kind"] == "fp8":
        t = t.view(torch.float8_e4m3fn)
    return t.to(device)


def antiquant_kwargs(case: DenseCase, device="cuda") -> dict:
    """AttentionPlan keyword arguments of a fake-quantised case."""
    aq = case.kv_quant
    if aq is None:
        return {}

    def tens(x):
        if x is None:
            return None
        return to_device(x, "bf16", device) if x.dtype == np.uint16 else torch.from_numpy(x).to(device)

    return dict(key_antiquant_mode=aq["kmode"], value_antiquant_mode=aq["vmode"],
                key_antiquant_scale=tens(aq["kscale"]), value_antiquant_scale=tens(aq["vscale"]),
                key_antiquant_offset=tens(aq["koff"]), value_antiquant_offset=tens(aq["voff"]))


def dense_tensors(case: DenseCase, device="cuda"):
    q = to_device(case.q, case.dtype, device)
    if case.paged:
        k = kv_to_device(case.k_pool, case, device)
        v = kv_to_device(case.v_pool, case, device)
        bt = torch.from_numpy(case.block_table).to(device)
    else:
        k = kv_to_device(case.k, case, device)
        v = kv_to_device(case.v, case, device)
        bt = None
    slopes = None if case.alibi_slopes is None else torch.from_numpy(case.alibi_slopes).to(device)
    return q, k, v, bt, slopes


def pse_tensor(case: DenseCase, device="cuda"):
    return None if case.pse_bias is None else to_device(case.pse_bias, case.dtype, device)


def mask_tensor(case: DenseCase, device="cuda"):
    return None if case.atten_mask is None else torch.from_numpy(case.atten_mask).to(device)


def dense_plan(case: DenseCase, device="cuda", tensors=None, **overrides) -> fia.AttentionPlan:
    q, k, v, bt, slopes = tensors if tensors is not None else dense_tensors(case, device)
    kw = dict(num_heads=case.num_heads, num_key_value_heads=case.num_kv_heads,
              scale_value=case.scale, input_layout=case.layout, sparse_mode=case.sparse_mode,
              pre_tokens=case.pre_tokens, next_tokens=case.next_tokens,
              pse_type=2 if slopes is not None else 0,
              pse_shift=slopes if slopes is not None else pse_tensor(case, device),
              q_start_idx=case.q_start_idx, kv_start_idx=case.kv_start_idx,
              block_table=bt, block_size=case.block_size if bt is not None else 0,
              softmax_lse_flag=case.lse, actual_seq_lengths=case.actual_seq_lengths,
              actual_seq_lengths_kv=case.actual_seq_lengths_kv, kv_layout=case.kv_layout,
              atten_mask=mask_tensor(case, device),
              learnable_sink=(None if case.learnable_sink is None
                              else to_device(case.learnable_sink, "bf16", device)),
              **antiquant_kwargs(case, device))
    kw.update(overrides)
    return fia.AttentionPlan(q, k, v, **kw)


def sparse_tensors(case: SparseCase, device="cuda"):
    return dict(
        q=to_device(case.q, "bf16", device),
        ori_kv=torch.from_numpy(case.ori_kv).to(device),
        cmp_kv=torch.from_numpy(case.cmp_kv).to(device),
        cmp_sparse_indices=(None if case.cmp_sparse_indices is None
                            else torch.from_numpy(case.cmp_sparse_indices).to(device)),
        ori_block_table=torch.from_numpy(case.ori_block_table).to(device),
        cmp_block_table=torch.from_numpy(case.cmp_block_table).to(device),
        seqused_kv=torch.tensor(case.seqused_kv, dtype=torch.int32, device=device),
        sinks=torch.from_numpy(case.sinks).to(device),
        cu_seqlens_q=(None if case.cu_seqlens_q is None
                      else torch.tensor(case.cu_seqlens_q, dtype=torch.int32, device=device)),
    )


def sparse_plan(case: SparseCase, device="cuda", tensors=None) -> fia.SparsePlan:
    t = tensors if tensors is not None else sparse_tensors(case, device)
    return fia.SparsePlan(t["q"], t["ori_kv"], t["cmp_kv"], t["cmp_sparse_indices"],
                          t["ori_block_table"], t["cmp_block_table"], t["seqused_kv"],
                          t["sinks"], softmax_scale=case.softmax_scale,
                          max_seqused_kv=max(case.seqused_kv), cmp_ratio=case.cmp_ratio,
                          ori_win_left=case.win_left, ori_win_right=case.win_right,
                          layout_q="BSND" if case.cu_seqlens_q is None else "TND",
                          cu_seqlens_q=t["cu_seqlens_q"])


def half_to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """fp16 / bf16 bit patterns (uint16) -> torch.float16 / torch.bfloat16."""
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(device)


def sfmla_tensors(case: SfmlaCase, device="cuda"):
    i32 = lambda x: None if x is None else torch.tensor(list(x), dtype=torch.int32, device=device)
    arr = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return dict(
        q=half_to_device(case.q, case.dtype, device),
        ori_kv=half_to_device(case.ori_kv, case.dtype, device),
        cmp_kv=None if case.cmp_kv is None else half_to_device(case.cmp_kv, case.dtype, device),
        cmp_sparse_indices=arr(case.cmp_sparse_indices),
        ori_block_table=arr(case.ori_block_table),
        cmp_block_table=arr(case.cmp_block_table),
        cu_seqlens_q=i32(case.cu_seqlens_q),
        cu_seqlens_ori_kv=i32(case.cu_seqlens_ori_kv),
        cu_seqlens_cmp_kv=i32(case.cu_seqlens_cmp_kv),
        seqused_kv=i32(case.seqused_kv),
        sinks=arr(case.sinks),
    )


def sfmla_plan(case: SfmlaCase, device="cuda", tensors=None) -> fia.SparseFlashMlaPlan:
    t = tensors if tensors is not None else sfmla_tensors(case, device)
    return fia.SparseFlashMlaPlan(
        t["q"], t["ori_kv"], seqused_kv=t["seqused_kv"], softmax_scale=case.softmax_scale,
        max_seqused_kv=max(case.seqused_kv), cmp_kv=t["cmp_kv"],
        cmp_sparse_indices=t["cmp_sparse_indices"], ori_block_table=t["ori_block_table"],
        cmp_block_table=t["cmp_block_table"], cu_seqlens_q=t["cu_seqlens_q"],
        cu_seqlens_ori_kv=t["cu_seqlens_ori_kv"], cu_seqlens_cmp_kv=t["cu_seqlens_cmp_kv"],
        sinks=t["sinks"], cmp_ratio=case.cmp_ratio, ori_win_left=case.win_left,
        ori_win_right=case.win_right, layout_q="BSND" if case.cu_seqlens_q is None else "TND",
        layout_kv=case.kv_layout, return_softmax_lse=case.return_lse)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 tensor -> uint16 bit patterns (numpy, on the host)."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
