"""fia_run_no_alloc, the entry point for callers that cannot allocate, against
fia_run on the same executors: bitwise-identical outputs and LSE, two calls in
a row with the second on a smaller input, for the kernel paths that use
scratch (split-KV decode, device-length decode, sparse) and one that does not
(prefill, whose work list also lives in the scratch).  Sizes past the scratch
are refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

from attention_online_softmax_flash_amd import fia
from attention_online_softmax_flash_amd import torch_io as TI
from attention_online_softmax_flash_amd import workloads as W
from oracle import fia_oracle as O
from parity import check_out, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _same_as_fia_run(plan):
    """Run through fia_run, then through fia_run_no_alloc into poisoned
    outputs; both results must be bit for bit the same."""
    plan.run()
    torch.cuda.synchronize()
    ref_o = plan.out.clone()
    ref_l = None if plan.lse is None else plan.lse.clone()
    plan.out.fill_(float("nan"))
    if plan.lse is not None:
        plan.lse.fill_(float("nan"))
    torch.cuda.synchronize()
    plan.run_no_alloc()
    torch.cuda.synchronize()
    assert torch.equal(plan.out, ref_o)
    if ref_l is not None:
        assert torch.equal(plan.lse, ref_l)
    return plan


def test_no_alloc_decode_then_smaller_decode():
    big = W.paged_decode_case("na1", 980, B=8, Q_N=32, KV_N=8, D=128,
                              kv_lens=[8192, 5000, 1, 4100, 7000, 300, 2048, 6666],
                              block_size=128, lse=True, poison_tail=True)
    small = W.paged_decode_case("na2", 981, B=2, Q_N=16, KV_N=4, D=64, kv_lens=[700, 33],
                                block_size=64, lse=True, poison_tail=True)
    for case in (big, small):
        plan = _same_as_fia_run(TI.dense_plan(case, DEV))
        assert plan.kind == "decode" and plan.workspace_size > 0
        check_out(to_f64(plan.out), O.fia_case(case)[0])


def test_no_alloc_sparse_then_smaller_sparse():
    big = W.c5_sparse_sharedkv()
    small = W.sfmla_case("na4", 983, B=2, N1=16, seqused_kv=[900, 130], K2=64, block_size1=32,
                         block_size2=16, window_only_ori=True)
    plan = _same_as_fia_run(TI.sparse_plan(big, DEV))
    assert plan.workspace_size > 0
    check_out(to_f64(plan.out), O.sparse_sharedkv(big))
    plan = _same_as_fia_run(TI.sfmla_plan(small, DEV))
    check_out(to_f64(plan.out), O.sparse_flash_mla(small)[0])


def test_no_alloc_prefill_and_device_length_decode():
    pre = W.dense_case("na5", 984, B=2, S1=300, S2=300, Q_N=8, KV_N=2, D=128, sparse_mode=3,
                       q_lens=[300, 129], kv_lens=[300, 129], lse=True, poison_pad=True)
    plan = _same_as_fia_run(TI.dense_plan(pre, DEV))
    assert plan.kind == "prefill"
    dec = W.paged_decode_case("na6", 985, B=3, Q_N=32, KV_N=8, D=128, kv_lens=[3000, 17, 1500],
                              block_size=128, lse=True, poison_tail=True)
    lens = torch.tensor(dec.actual_seq_lengths_kv, dtype=torch.int32, device=DEV)
    plan = _same_as_fia_run(TI.dense_plan(dec, DEV, actual_seq_lengths_kv=None,
                                          actual_seq_lengths_kv_device=lens,
                                          max_actual_seq_length_kv=3072))
    check_out(to_f64(plan.out), O.fia_case(dec)[0])


def test_no_alloc_refuses_a_workspace_past_the_scratch():
    """A decode plan whose split-KV partials need more than the 63 MiB
    workspace area is refused with FIA_ERR_UNSUPPORTED before any launch
    (phase 1 runs on descriptors whose addresses are never dereferenced)."""
    FAKE = 0x7F0000000000

    def T(shape, dt=fia.DT_BF16):
        d = fia.FiaTensor()
        d.data, d.dtype, d.ndim = FAKE, dt, len(shape)
        acc = 1
        for i in reversed(range(len(shape))):
            d.shape[i], d.stride[i] = shape[i], acc
            acc *= shape[i]
        return d

    B, S2 = 256, 16384
    q, kv = T((B, 1, 32, 128)), T((B, S2, 8, 128))
    p = fia.FiaParams()
    p.input_layout, p.num_heads, p.num_key_value_heads, p.scale_value = b"BSND", 32, 8, 0.088
    p.pre_tokens = p.next_tokens = 2147483647
    ws, ex = ctypes.c_size_t(0), ctypes.c_void_p(None)
    L = fia.lib()
    st = L.fia_get_workspace_size(ctypes.byref(p), ctypes.pointer(q), ctypes.pointer(kv),
                                  ctypes.pointer(kv), None, None, None, ctypes.pointer(q), None,
                                  ctypes.byref(ws), ctypes.byref(ex))
    assert st == 0 and ws.value > 63 * 2 ** 20
    try:
        st = L.fia_run_no_alloc(ex, None)
        assert st == fia.FIA_ERR_UNSUPPORTED
        assert "exceeds" in L.fia_last_error().decode()
    finally:
        L.fia_executor_destroy(ex)
