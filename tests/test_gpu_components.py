"""Full-size parity of the timed variants of the workloads: every component
the benchmark times, on the same seeded inputs and in the plan the benchmark
launches, against the oracle element by element.  (The five base workloads
are compared at full size in test_gpu_parity.py and test_gpu_sfmla.py.)"""
import pytest
import torch

from attention_online_softmax_flash_amd import torch_io as TI
from attention_online_softmax_flash_amd import workloads as W
from oracle import fia_oracle as O
from parity import check_out, to_f64
from test_gpu_parity import dense_parity, run_plan

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("make", [W.mask_prefill, W.bias_prefill, W.sink_prefill],
                         ids=["mask", "bias", "sink"])
def test_prefill_component_full(make):
    """Causal GQA prefill shapes (4 x 32 heads x up to 1631 rows) with an
    explicit mask, a [1, 32, 2048, 2048] bias or a learnable sink."""
    dense_parity(make(), "prefill")


@pytest.mark.parametrize("name", sorted(W.Q8_DECODES))
def test_fake_quant_decode_component_full(name):
    """The paged GQA decode (64 batches, KV lengths 1024-8192) over int8 /
    e4m3fn codes, PA_ND and BnNBsD pools."""
    dense_parity(W.q8_decode(name), "decode")


def test_device_length_decode_component_full():
    """The paged GQA decode with its KV lengths on the device, plan bound 8192."""
    case = W.c3_paged_decode(poison_tail=True)
    lens = torch.tensor(case.actual_seq_lengths_kv, dtype=torch.int32, device="cuda")
    dense_parity(case, "decode", actual_seq_lengths_kv=None, actual_seq_lengths_kv_device=lens,
                 max_actual_seq_length_kv=8192)


@pytest.mark.parametrize("make", [W.sparse_hca_decode, W.sparse_two_tokens, W.sparse_tnd_ragged],
                         ids=["hca", "s1_2", "tnd"])
def test_sparse_component_full(make):
    """Shared-KV sparse modes at B=16, N1=64, KV length 16384."""
    case = make()
    plan = run_plan(TI.sparse_plan(case, "cuda"))
    assert plan.kind == "sparse"
    check_out(to_f64(plan.out), O.sparse_sharedkv(case))
