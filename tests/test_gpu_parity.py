"""GPU parity: the HIP library (through the C ABI) against the float64 oracle
on identical seeded inputs, at the bar of the parity contract:
bf16 outputs |gpu - ref| <= 1e-2 + 1e-2 |ref|, LSE within 1e-3 absolute with
+inf matching exactly, gathers and sparse row selection bit-exact."""
import dataclasses

import numpy as np
import pytest
import torch

from attention_online_softmax_flash_amd import fia
from attention_online_softmax_flash_amd import torch_io as TI
from attention_online_softmax_flash_amd import workloads as W
from oracle import fia_oracle as O
from parity import check_lse, check_out, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_plan(plan):
    plan.run()
    torch.cuda.synchronize()
    return plan


def gpu_results(plan):
    out = to_f64(plan.out)
    lse = None if plan.lse is None else to_f64(plan.lse)[..., 0]
    return out, lse


def dense_parity(case, expect_kind=None, rows=None, heads=None, **over):
    plan = run_plan(TI.dense_plan(case, DEV, **over))
    if expect_kind:
        assert plan.kind == expect_kind
    out, lse = gpu_results(plan)
    ref_o, ref_l = O.fia_case(case, rows=rows, heads=heads)
    if rows is None and heads is None:
        check_out(out, ref_o)
        if lse is not None:
            check_lse(lse, ref_l)
    else:
        hs = list(range(case.num_heads)) if heads is None else list(heads)
        rs = list(range(case.q.shape[1])) if rows is None else list(rows)
        sel_o = np.ix_(range(out.shape[0]), rs, hs, range(out.shape[3]))
        check_out(out[sel_o], ref_o[sel_o])
        if lse is not None:
            sel_l = np.ix_(range(out.shape[0]), hs, rs)
            check_lse(lse[sel_l], ref_l[sel_l])
    return plan, out, lse


# ---------------------------------------------------------------------------
# The five workloads at full size.
# ---------------------------------------------------------------------------
def test_c1_tiny_dense_fp32():
    case = W.c1_tiny_dense()
    plan, out, lse = dense_parity(case, "fp32")
    ref_o, ref_l = O.fia_case(case)
    # stretch bound for the fp32 path
    check_out(out, ref_o, atol=1e-4, rtol=1e-4)
    check_lse(lse, ref_l, atol=1e-4)


def test_c2_causal_gqa_prefill_full_with_nan_padding():
    case = W.c2_causal_gqa(poison_pad=True, lse=True)
    plan, out, lse = dense_parity(case, "prefill")
    for b, L in enumerate(case.actual_seq_lengths):
        assert np.all(out[b, L:] == 0.0)
        assert np.all(np.isposinf(lse[b, :, L:]))


def test_c3_paged_decode_full_with_nan_tails():
    case = W.c3_paged_decode(poison_tail=True)
    dense_parity(case, "decode")


def test_c4_long_alibi_prefill_full():
    # Every head and every row of the long ALiBi prefill, output and LSE,
    # against the float64 oracle (about half a minute of host BLAS).
    case = W.c4_alibi_prefill(lse=True)
    dense_parity(case, "prefill")


def test_c5_sparse_sharedkv_full():
    case = W.c5_sparse_sharedkv()
    plan = run_plan(TI.sparse_plan(case, DEV))
    assert plan.kind == "sparse"
    check_out(to_f64(plan.out), O.sparse_sharedkv(case))


# ---------------------------------------------------------------------------
# Small sweeps: several tiles, ragged tails, every mask mode.
# ---------------------------------------------------------------------------
PREFILL_CASES = [
    # (B, S1, S2, Qn, KVn, D, mode, pre, nxt, q_lens, kv_lens, alibi)
    (2, 200, 200, 4, 4, 128, 0, None, None, None, None, False),
    (2, 200, 200, 8, 2, 128, 2, None, None, [200, 77], [200, 77], False),
    (2, 200, 300, 8, 2, 128, 3, None, None, [130, 1], [300, 129], False),
    (1, 257, 257, 4, 1, 128, 3, None, None, None, None, True),
    (2, 190, 190, 4, 4, 64, 3, None, None, [190, 65], [190, 65], True),
    (2, 160, 220, 4, 2, 128, 4, 40, 3, [160, 100], [220, 90], False),
    (1, 300, 100, 2, 2, 64, 3, None, None, None, None, False),
    (1, 150, 150, 4, 4, 128, 4, 0, 0, None, None, False),
    (3, 129, 129, 16, 2, 128, 2, None, None, [129, 0, 64], [129, 5, 64], False),
    (1, 64, 513, 8, 8, 64, 0, None, None, None, None, False),
    (2, 140, 140, 6, 3, 128, 4, 2147483647, 0, None, None, False),
]


@pytest.mark.parametrize("i", range(len(PREFILL_CASES)))
def test_prefill_sweep(i):
    B, S1, S2, Qn, KVn, D, mode, pre, nxt, ql, kl, alibi = PREFILL_CASES[i]
    kw = {}
    if pre is not None:
        kw.update(pre_tokens=pre, next_tokens=nxt)
    case = W.dense_case(f"pre{i}", 100 + i, B=B, S1=S1, S2=S2, Q_N=Qn, KV_N=KVn, D=D,
                        sparse_mode=mode, q_lens=ql, kv_lens=kl, alibi=alibi, lse=True,
                        poison_pad=True, **kw)
    dense_parity(case, "prefill")


def test_prefill_alibi_start_offsets():
    case = W.dense_case("alibi_off", 120, B=1, S1=140, S2=140, Q_N=4, KV_N=4, D=128,
                        sparse_mode=3, alibi=True, lse=True, q_start_idx=7, kv_start_idx=300)
    dense_parity(case, "prefill")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_alibi_scale_zero(D):
    # scale_value 0 with ALiBi: every score is its bias alone.
    case = W.dense_case(f"als0_{D}", 125 + D, B=2, S1=260, S2=260, Q_N=4, KV_N=2, D=D,
                        scale=0.0, sparse_mode=3, alibi=True, q_lens=[260, 70],
                        kv_lens=[260, 70], lse=True, poison_pad=True)
    dense_parity(case, "prefill")


@pytest.mark.parametrize("scale", [None, 0.0])
def test_prefill_alibi_with_mask(scale):
    # ALiBi together with an explicit mask tensor (both in the score
    # accumulators' initial value), a fully masked row included.
    case = W.dense_case("almask", 127, B=2, S1=200, S2=200, Q_N=4, KV_N=4, D=128, scale=scale,
                        alibi=True, q_lens=[200, 150], kv_lens=[200, 150], lse=True,
                        poison_pad=True)
    case = W.with_random_mask(case, 128, p_masked=0.2, dead_rows=(3,))
    dense_parity(case, "prefill")


@pytest.mark.parametrize("bs", [32, 128])
def test_prefill_alibi_paged(bs):
    # ALiBi over a paged cache: whole-tile pages (128) and per-row lookups (32).
    case = W.paged_decode_case("alpg", 129, B=2, Q_N=8, KV_N=2, D=128, kv_lens=[200, 131],
                               block_size=bs, S1=200, sparse_mode=3, lse=True, poison_tail=True,
                               extra_blocks=2)
    case.actual_seq_lengths = [200, 131]   # ALiBi: query and key lengths agree
    case.alibi_slopes = W.alibi_slopes(8)
    dense_parity(case, "prefill")


@pytest.mark.parametrize("layout", ["BNSD", "BSH"])
def test_prefill_other_layouts(layout):
    case = W.dense_case("lay", 130, B=2, S1=150, S2=150, Q_N=8, KV_N=2, D=128, sparse_mode=3,
                        lse=True)
    q, k, v, bt, slopes = TI.dense_tensors(case, DEV)
    if layout == "BNSD":
        tq, tk, tv = (x.permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    else:
        tq, tk, tv = (x.reshape(x.shape[0], x.shape[1], -1).contiguous() for x in (q, k, v))
    plan = run_plan(fia.AttentionPlan(tq, tk, tv, num_heads=8, num_key_value_heads=2,
                                      scale_value=case.scale, input_layout=layout,
                                      sparse_mode=3, softmax_lse_flag=True))
    out = plan.out.permute(0, 2, 1, 3) if layout == "BNSD" else plan.out.reshape(q.shape)
    ref_o, ref_l = O.fia_case(case)
    check_out(to_f64(out), ref_o)
    check_lse(to_f64(plan.lse)[..., 0], ref_l)


@pytest.mark.parametrize("D,layout", [(64, "BSND"), (128, "BSND"), (128, "BNSD"), (64, "BSH")])
def test_prefill_padded_tiles_are_written(D, layout):
    """Query tiles wholly past the actual length get no work item of their
    own; the live tiles' items write them.  Outputs start as NaN, so a row
    nobody writes fails; S1 = 1000 leaves a partial last tile and batch 1
    (length 130) has 2 live tiles for 6 padded ones."""
    case = W.dense_case("padtiles", 145, B=3, S1=1000, S2=900, Q_N=4, KV_N=2, D=D,
                        sparse_mode=3, q_lens=[0, 130, 999], kv_lens=[50, 900, 777], lse=True,
                        poison_pad=True)
    q, k, v, bt, slopes = TI.dense_tensors(case, DEV)
    if layout == "BNSD":
        q, k, v = (x.permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    elif layout == "BSH":
        q, k, v = (x.reshape(x.shape[0], x.shape[1], -1).contiguous() for x in (q, k, v))
    out = torch.full_like(q, float("nan"))
    lse = torch.full((3, 4, 1000, 1), float("nan"), dtype=torch.float32, device=DEV)
    plan = run_plan(fia.AttentionPlan(q, k, v, num_heads=4, num_key_value_heads=2,
                                      scale_value=case.scale, input_layout=layout,
                                      sparse_mode=3, softmax_lse_flag=True,
                                      actual_seq_lengths=[0, 130, 999],
                                      actual_seq_lengths_kv=[50, 900, 777],
                                      attention_out=out, softmax_lse=lse))
    assert plan.kind == "prefill"
    got = plan.out.permute(0, 2, 1, 3) if layout == "BNSD" else plan.out
    if layout == "BSH":
        got = got.reshape(3, 1000, 4, D)
    ref_o, ref_l = O.fia_case(case)
    check_out(to_f64(got), ref_o)
    check_lse(to_f64(plan.lse)[..., 0], ref_l)


def test_prefill_tnd():
    case = W.tnd_case("tnd", 140, q_lens=[100, 0, 257, 1], kv_lens=[100, 3, 300, 50],
                      Q_N=8, KV_N=4, D=128, sparse_mode=3, lse=True)
    dense_parity(case, "prefill")


def test_prefill_over_paged_kv():
    case = W.paged_decode_case("pp", 150, B=3, Q_N=8, KV_N=2, D=128, kv_lens=[300, 70, 513],
                               block_size=64, S1=70, sparse_mode=3, lse=True, poison_tail=True,
                               extra_blocks=3)
    case.actual_seq_lengths = [70, 70, 70]
    dense_parity(case, "prefill")


@pytest.mark.parametrize("bs", [64, 16])
def test_prefill_over_paged_kv_bnnbsd(bs):
    case = W.paged_decode_case("ppb", 151, B=3, Q_N=8, KV_N=2, D=128, kv_lens=[300, 70, 513],
                               block_size=bs, S1=70, sparse_mode=3, lse=True, poison_tail=True,
                               extra_blocks=3)
    case.actual_seq_lengths = [70, 70, 70]
    dense_parity(W.as_bnnbsd(case), "prefill")


MASK_PREFILL_CASES = [
    # (B, S1, S2, Qn, KVn, D, dims, per_batch, mode, q_lens, kv_lens)
    (2, 200, 300, 8, 2, 128, 3, True, 0, [200, 150], [300, 290]),
    (1, 130, 130, 4, 4, 128, 2, False, 1, None, None),
    (2, 70, 97, 8, 4, 64, 4, True, 0, [70, 33], [97, 60]),
]


@pytest.mark.parametrize("i", range(len(MASK_PREFILL_CASES)))
def test_prefill_explicit_mask(i):
    B, S1, S2, Qn, KVn, D, dims, pb, mode, ql, kl = MASK_PREFILL_CASES[i]
    case = W.dense_case(f"mp{i}", 700 + i, B=B, S1=S1, S2=S2, Q_N=Qn, KV_N=KVn, D=D,
                        q_lens=ql, kv_lens=kl, lse=True, poison_pad=True)
    case = W.with_random_mask(case, 710 + i, dims=dims, per_batch=pb, dead_rows=(5,), mode=mode)
    dense_parity(case, "prefill")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_explicit_mask_scale_zero(D):
    # scale_value 0 is legal: every visible key then gets the same weight.
    # Masked keys must still get weight 0 on tiles inside the visible range
    # (where -inf * 0 would be NaN), and a fully masked row gives 0 / +inf.
    case = W.dense_case(f"ms0_{D}", 760 + D, B=2, S1=200, S2=300, Q_N=4, KV_N=2, D=D,
                        scale=0.0, q_lens=[200, 131], kv_lens=[300, 250], lse=True,
                        poison_pad=True)
    case = W.with_random_mask(case, 770 + D, p_masked=0.2, dead_rows=(7,))
    plan, out, lse = dense_parity(case, "prefill")
    assert np.all(out[:, 7] == 0.0) and np.all(np.isposinf(lse[:, :, 7]))


def test_prefill_explicit_mask_paged():
    case = W.paged_decode_case("mpp", 720, B=2, Q_N=8, KV_N=2, D=128, kv_lens=[300, 129],
                               block_size=64, S1=40, lse=True, poison_tail=True, extra_blocks=2)
    case.actual_seq_lengths = [40, 40]
    dense_parity(W.with_random_mask(case, 721, dead_rows=(0,)), "prefill")


def test_decode_explicit_mask():
    case = W.paged_decode_case("mdp", 730, B=3, Q_N=32, KV_N=8, D=128, kv_lens=[1, 700, 1500],
                               block_size=128, lse=True, poison_tail=True, extra_blocks=2)
    dense_parity(W.with_random_mask(case, 731, p_masked=0.5), "decode")
    case = W.dense_case("mdd", 732, B=2, S1=1, S2=900, Q_N=8, KV_N=2, D=64, kv_lens=[900, 40],
                        lse=True, poison_pad=True)
    dense_parity(W.with_random_mask(case, 733, dims=2, per_batch=False, mode=1), "decode")


def test_fp32_explicit_mask():
    case = W.dense_case("mf", 740, B=2, S1=37, S2=50, Q_N=4, KV_N=2, D=64, dtype="fp32",
                        lse=True, poison_pad=True)
    plan, out, lse = dense_parity(W.with_random_mask(case, 741, dead_rows=(2,)), "fp32")


PSE_PREFILL_CASES = [
    # (B, S1, S2, Qn, KVn, D, mode, per_batch, one_row, q_lens, kv_lens, with_mask)
    (2, 200, 300, 8, 2, 128, 3, True, False, [200, 150], [300, 290], False),
    (1, 130, 130, 4, 4, 128, 0, False, True, None, None, False),
    (2, 70, 97, 8, 4, 64, 0, True, False, [70, 33], [97, 60], True),
    (1, 257, 257, 8, 1, 128, 2, False, False, None, None, False),
]


@pytest.mark.parametrize("i", range(len(PSE_PREFILL_CASES)))
def test_prefill_pse_bias(i):
    """pseType 0 bias tensor [B or 1, Q_N, Q_S or 1, KV_S'] in bf16."""
    B, S1, S2, Qn, KVn, D, mode, pb, one, ql, kl, wm = PSE_PREFILL_CASES[i]
    case = W.dense_case(f"pp{i}", 750 + i, B=B, S1=S1, S2=S2, Q_N=Qn, KV_N=KVn, D=D, sparse_mode=mode,
                        q_lens=ql, kv_lens=kl, lse=True, poison_pad=True)
    if wm:
        case = W.with_random_mask(case, 760 + i, dead_rows=(3,), mode=mode)
    dense_parity(W.with_random_bias(case, 770 + i, per_batch=pb, one_row=one), "prefill")


@pytest.mark.parametrize("bs", [64, 16])
def test_prefill_pse_bias_paged(bs):
    case = W.paged_decode_case("ppp", 780, B=2, Q_N=8, KV_N=2, D=128, kv_lens=[300, 129],
                               block_size=bs, S1=40, sparse_mode=3, lse=True, poison_tail=True,
                               extra_blocks=2)
    case.actual_seq_lengths = [40, 40]
    dense_parity(W.with_random_bias(case, 781), "prefill")


def test_decode_pse_bias():
    case = W.paged_decode_case("pdp", 790, B=3, Q_N=32, KV_N=8, D=128, kv_lens=[1, 700, 1500],
                               block_size=128, lse=True, poison_tail=True, extra_blocks=2)
    dense_parity(W.with_random_bias(case, 791, one_row=True), "decode")
    case = W.dense_case("pdd", 792, B=2, S1=1, S2=900, Q_N=8, KV_N=2, D=64, kv_lens=[900, 40],
                        lse=True, poison_pad=True)
    case = W.with_random_mask(case, 793, dims=2, per_batch=False, mode=1)
    dense_parity(W.with_random_bias(case, 794, per_batch=False, std=3.0), "decode")


def test_fp32_pse_bias():
    case = W.dense_case("pf", 795, B=2, S1=37, S2=50, Q_N=4, KV_N=2, D=64, dtype="fp32",
                        sparse_mode=3, lse=True, poison_pad=True)
    dense_parity(W.with_random_bias(case, 796), "fp32")


SINK_PREFILL_CASES = [
    # (B, S1, S2, Qn, KVn, D, mode, q_lens, kv_lens, with_mask, sink_mean)
    (2, 200, 300, 8, 2, 128, 3, [200, 150], [300, 290], False, 0.0),
    (2, 70, 97, 8, 4, 64, 0, [70, 33], [97, 60], True, 3.0),
    (3, 130, 130, 4, 4, 128, 2, None, [130, 0, 77], False, -1.0),
]


@pytest.mark.parametrize("i", range(len(SINK_PREFILL_CASES)))
def test_prefill_learnable_sink(i):
    B, S1, S2, Qn, KVn, D, mode, ql, kl, wm, mean = SINK_PREFILL_CASES[i]
    case = W.dense_case(f"sp{i}", 800 + i, B=B, S1=S1, S2=S2, Q_N=Qn, KV_N=KVn, D=D, sparse_mode=mode,
                        q_lens=ql, kv_lens=kl, lse=True, poison_pad=True)
    if wm:
        case = W.with_random_mask(case, 810 + i, dead_rows=(3,), mode=mode)
    dense_parity(W.with_random_sink(case, 820 + i, mean=mean), "prefill")


def test_decode_learnable_sink():
    # single-chunk rows, multi-chunk merges and a batch with no key
    case = W.paged_decode_case("sdp", 830, B=4, Q_N=32, KV_N=8, D=128, kv_lens=[1, 700, 5000, 0],
                               block_size=128, lse=True, poison_tail=True, extra_blocks=2)
    dense_parity(W.with_random_sink(case, 831), "decode")
    case = W.dense_case("sdd", 832, B=2, S1=1, S2=900, Q_N=8, KV_N=2, D=64, kv_lens=[900, 40],
                        lse=True, poison_pad=True)
    case = W.with_random_mask(case, 833, p_masked=0.995, dims=2, per_batch=False)
    dense_parity(W.with_random_sink(case, 834, mean=2.0), "decode")


FAKE_QUANT_CASES = [
    # (name, kind, kmode, vmode, offsets, per_tensor, builder)
    ("i8_chan_off_paged", "int8", 0, 0, True, False,
     lambda: W.paged_decode_case("fq0", 850, B=3, Q_N=32, KV_N=8, D=128, kv_lens=[1, 700, 5000],
                                 block_size=128, lse=True, poison_tail=True, extra_blocks=2)),
    ("i8_token_off_dense_d64", "int8", 1, 1, True, False,
     lambda: W.dense_case("fq1", 851, B=3, S1=1, S2=1030, Q_N=8, KV_N=2, D=64,
                          kv_lens=[1030, 33, 512], lse=True, poison_pad=True)),
    ("fp8_chan_bnnbsd", "fp8", 0, 0, False, False,
     lambda: W.as_bnnbsd(W.paged_decode_case("fq2", 852, B=2, Q_N=16, KV_N=4, D=128,
                                             kv_lens=[2049, 300], block_size=64, lse=True,
                                             poison_tail=True))),
    ("fp8_token_paged32", "fp8", 1, 1, False, False,
     lambda: W.paged_decode_case("fq3", 853, B=2, Q_N=8, KV_N=1, D=128, kv_lens=[77, 1500],
                                 block_size=32, lse=True, poison_tail=True, extra_blocks=1)),
    ("i8_mixed_off", "int8", 0, 1, True, False,
     lambda: W.paged_decode_case("fq4", 854, B=2, Q_N=64, KV_N=2, D=128, kv_lens=[900, 1800],
                                 block_size=128, lse=True, poison_tail=True)),
    ("i8_tensor", "int8", 0, 0, True, True,
     lambda: W.dense_case("fq5", 855, B=2, S1=1, S2=640, Q_N=4, KV_N=4, D=128, kv_lens=[640, 7],
                          lse=True, poison_pad=True)),
    # two KV heads per wave (adjacent heads, G <= 8): every column used (G = 8),
    # an odd group size with KV_N = 6, a dense BSND cache with mixed modes
    ("i8_token_pair_g8", "int8", 1, 1, True, False,
     lambda: W.paged_decode_case("fq6", 856, B=3, Q_N=64, KV_N=8, D=128, kv_lens=[1, 1500, 3000],
                                 block_size=64, lse=True, poison_tail=True, extra_blocks=1)),
    ("fp8_chan_pair_g3", "fp8", 0, 0, False, False,
     lambda: W.paged_decode_case("fq7", 857, B=2, Q_N=18, KV_N=6, D=128, kv_lens=[2100, 33],
                                 block_size=128, lse=True, poison_tail=True)),
    ("i8_mixed_pair_dense", "int8", 0, 1, True, False,
     lambda: W.dense_case("fq8", 858, B=2, S1=1, S2=1100, Q_N=16, KV_N=4, D=128,
                          kv_lens=[1100, 260], lse=True, poison_pad=True)),
]


@pytest.mark.parametrize("i", range(len(FAKE_QUANT_CASES)))
def test_decode_fake_quant_kv(i):
    """Fake-quantised int8 / e4m3fn key/value rows (scale * (code + offset))."""
    name, kind, km, vm, off, pt, build = FAKE_QUANT_CASES[i]
    case = W.with_kv_quant(build(), 860 + i, kind=kind, kmode=km, vmode=vm, offsets=off,
                           per_tensor=pt)
    dense_parity(case, "decode")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_decode_fake_quant_every_code_is_exact(kind):
    """Every code, one per batch entry with a single key: the output is the
    value code itself (exact in bf16) and the LSE is scale * key code (query
    e_0, scale 1 tables), so a wrong or flushed conversion of any code shows.
    e4m3fn NaN codes (0x7f, 0xff) are left out."""
    codes = np.arange(256)
    if kind == "fp8":
        codes = codes[(codes & 0x7F) != 0x7F]
    B, D = codes.size, 128
    case = W.dense_case("fqx", 880, B=B, S1=1, S2=4, Q_N=1, KV_N=1, D=D, kv_lens=[1] * B, lse=True,
                        scale=0.5)
    q = np.zeros_like(case.q)
    q[..., 0] = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    case = W.with_kv_quant(dataclasses.replace(case, q=q), 881, kind=kind, kmode=0, vmode=0)
    dt = np.int8 if kind == "int8" else np.uint8
    k = np.zeros(case.k.shape, dtype=dt)
    v = np.zeros(case.v.shape, dtype=dt)
    k[:, 0, 0, 0] = codes.astype(np.uint8).view(dt)
    v[:, 0, 0, :] = codes.astype(np.uint8).view(dt)[:, None]
    one = W.f32_to_bf16_bits(np.ones((1, D), np.float32))
    case = dataclasses.replace(case, k=k, v=v, kv_quant=dict(case.kv_quant, kscale=one, vscale=one))
    plan = run_plan(TI.dense_plan(case, DEV))
    out, lse = gpu_results(plan)
    want = O.decode_codes(codes.astype(np.uint8).view(dt), kind)
    np.testing.assert_array_equal(out[:, 0, 0, :], np.repeat(want[:, None], D, axis=1))
    np.testing.assert_allclose(lse[:, 0, 0], 0.5 * want, rtol=2e-6, atol=1e-9)


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_decode_fake_quant_every_code_two_heads_per_wave(kind):
    """The every-code check through the kernel that takes two adjacent KV
    heads per wave (dense BSND, KV_N = 2, G = 1): head 0 carries each code,
    head 1 the codes in reverse order, so both heads' key and value
    conversions and their output columns are checked bit-exactly."""
    codes = np.arange(256)
    if kind == "fp8":
        codes = codes[(codes & 0x7F) != 0x7F]
    rev = codes[::-1].copy()
    B, D = codes.size, 128
    case = W.dense_case("fqx2", 882, B=B, S1=1, S2=4, Q_N=2, KV_N=2, D=D, kv_lens=[1] * B, lse=True,
                        scale=0.5)
    q = np.zeros_like(case.q)
    q[..., 0] = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    case = W.with_kv_quant(dataclasses.replace(case, q=q), 883, kind=kind, kmode=0, vmode=0)
    dt = np.int8 if kind == "int8" else np.uint8
    k = np.zeros(case.k.shape, dtype=dt)
    v = np.zeros(case.v.shape, dtype=dt)
    for h, cs in ((0, codes), (1, rev)):
        k[:, 0, h, 0] = cs.astype(np.uint8).view(dt)
        v[:, 0, h, :] = cs.astype(np.uint8).view(dt)[:, None]
    one = W.f32_to_bf16_bits(np.ones((2, D), np.float32))
    case = dataclasses.replace(case, k=k, v=v, kv_quant=dict(case.kv_quant, kscale=one, vscale=one))
    plan = run_plan(TI.dense_plan(case, DEV))
    out, lse = gpu_results(plan)
    for h, cs in ((0, codes), (1, rev)):
        want = O.decode_codes(cs.astype(np.uint8).view(dt), kind)
        np.testing.assert_array_equal(out[:, 0, h, :], np.repeat(want[:, None], D, axis=1))
        np.testing.assert_allclose(lse[:, h, 0], 0.5 * want, rtol=2e-6, atol=1e-9)


def test_decode_fake_quant_tnd():
    case = W.tnd_case("fqt", 870, q_lens=[1, 1, 0, 1], kv_lens=[600, 5, 100, 1029], Q_N=8, KV_N=2,
                      D=128, lse=True)
    dense_parity(W.with_kv_quant(case, 871, kind="fp8", kmode=1, vmode=1), "decode")


BNNBSD_DECODE_CASES = [
    # (B, Qn, KVn, D, kv_lens, block_size)
    (3, 32, 8, 128, [1, 511, 1300], 128),
    (2, 8, 8, 128, [512, 513], 16),
    (2, 8, 8, 128, [1024, 1025], 16),     # one chunk / two chunks at the 1024-key boundary
    (2, 4, 2, 64, [999, 40], 32),
    (2, 16, 1, 128, [2048 + 7, 100], 64),
]


@pytest.mark.parametrize("i", range(len(BNNBSD_DECODE_CASES)))
def test_decode_bnnbsd(i):
    B, Qn, KVn, D, lens, bs = BNNBSD_DECODE_CASES[i]
    case = W.paged_decode_case(f"decb{i}", 260 + i, B=B, Q_N=Qn, KV_N=KVn, D=D, kv_lens=lens,
                               block_size=bs, lse=True, poison_tail=True, extra_blocks=2,
                               table_cols=(max(lens) + bs - 1) // bs + 1)
    dense_parity(W.as_bnnbsd(case), "decode")


DECODE_CASES = [
    # (B, Qn, KVn, D, kv_lens, block_size or None (dense), mode, pre, nxt)
    (3, 32, 8, 128, [1, 511, 1300], 128, 0, None, None),
    (2, 8, 8, 128, [512, 513], 16, 3, None, None),
    (2, 8, 8, 128, [1024, 1025], 16, 3, None, None),
    (2, 16, 1, 128, [2048 + 7, 100], 64, 0, None, None),
    (2, 32, 1, 128, [700, 3], 512, 0, None, None),
    (1, 64, 1, 128, [1500], 128, 0, None, None),
    (2, 4, 2, 64, [999, 40], 32, 0, None, None),
    (3, 8, 2, 128, [0, 600, 17], 128, 0, None, None),
    (2, 8, 2, 128, [900, 300], None, 0, None, None),
    (2, 8, 2, 128, [900, 300], 128, 2, None, None),
    (2, 8, 2, 128, [900, 300], 128, 4, 100, 0),
    (2, 8, 2, 128, [2000, 300], 128, 4, 1500, 5),
]


@pytest.mark.parametrize("i", range(len(DECODE_CASES)))
def test_decode_sweep(i):
    B, Qn, KVn, D, lens, bs, mode, pre, nxt = DECODE_CASES[i]
    if bs is None:
        S2 = max(lens)
        case = W.dense_case(f"dec{i}", 200 + i, B=B, S1=1, S2=S2, Q_N=Qn, KV_N=KVn, D=D,
                            sparse_mode=mode, kv_lens=lens, lse=True, poison_pad=True)
    else:
        case = W.paged_decode_case(f"dec{i}", 200 + i, B=B, Q_N=Qn, KV_N=KVn, D=D, kv_lens=lens,
                                   block_size=bs, lse=True, poison_tail=True, sparse_mode=mode,
                                   extra_blocks=2, table_cols=(max(lens) + bs - 1) // bs + 1)
    if pre is not None:
        case.pre_tokens, case.next_tokens = pre, nxt
    dense_parity(case, "decode")


def test_decode_tnd():
    case = W.tnd_case("dtnd", 240, q_lens=[1, 1, 0, 1], kv_lens=[600, 5, 100, 1029], Q_N=8,
                      KV_N=2, D=128, lse=True)
    dense_parity(case, "decode")


def test_decode_tnd_entry_without_query_writes_nothing():
    """A TND entry with no query token owns no output row; the row at its
    offset belongs to the next entry, here written directly by the split
    kernel (one chunk) before the merge runs, so a stray empty-row write by
    the merge would always show."""
    case = W.tnd_case("dtnd0", 241, q_lens=[1, 0, 1, 0], kv_lens=[600, 100, 300, 7], Q_N=8,
                      KV_N=2, D=128, lse=True)
    dense_parity(case, "decode")


FP32_CASES = [
    (2, 70, 70, 4, 2, 64, 3, None, None, [70, 33], [70, 33], True),
    (1, 40, 90, 2, 1, 128, 4, 10, 2, None, None, False),
    (2, 1, 300, 4, 4, 32, 0, None, None, None, [300, 0], False),
]


@pytest.mark.parametrize("i", range(len(FP32_CASES)))
def test_fp32_sweep(i):
    B, S1, S2, Qn, KVn, D, mode, pre, nxt, ql, kl, alibi = FP32_CASES[i]
    kw = {} if pre is None else dict(pre_tokens=pre, next_tokens=nxt)
    case = W.dense_case(f"f32_{i}", 300 + i, B=B, S1=S1, S2=S2, Q_N=Qn, KV_N=KVn, D=D,
                        dtype="fp32", sparse_mode=mode, q_lens=ql, kv_lens=kl, alibi=alibi,
                        lse=True, poison_pad=True, **kw)
    plan, out, lse = dense_parity(case, "fp32")
    ref_o, ref_l = O.fia_case(case)
    check_out(out, ref_o, atol=1e-4, rtol=1e-4)


def test_empty_kv_fills_zero_and_inf():
    case = W.dense_case("empty", 310, B=2, S1=5, S2=0, Q_N=4, KV_N=2, D=128, lse=True)
    plan = run_plan(TI.dense_plan(case, DEV))
    assert plan.kind == "fill"
    out, lse = gpu_results(plan)
    assert np.all(out == 0) and np.all(np.isposinf(lse))


# ---------------------------------------------------------------------------
# Shared-KV sparse decode sweep.
# ---------------------------------------------------------------------------
SPARSE_CASES = [
    # (B, N1, lens, K2, n_valid)
    (3, 64, [1, 5, 130], 512, None),
    (2, 128, [1000, 4096], 1024, None),
    (2, 64, [2000, 300], 512, 17),
]


@pytest.mark.parametrize("i", range(len(SPARSE_CASES)))
def test_sparse_sweep(i):
    B, N1, lens, K2, nv = SPARSE_CASES[i]
    case = W.sparse_case(f"sp{i}", 400 + i, B=B, N1=N1, seqused_kv=lens, K2=K2, n_valid=nv,
                         block_size1=64, block_size2=32, materialise_all_ori=False)
    plan = run_plan(TI.sparse_plan(case, DEV))
    check_out(to_f64(plan.out), O.sparse_sharedkv(case))


def test_sparse_non_power_of_two_scales():
    """Tile scales that are not powers of two (a random mix with powers of
    two, so both conversions run within one wave: the exact fp32 product for
    the former, the exponent-only hardware conversion for the latter)."""
    case = W.sparse_case("spnp2", 430, B=3, N1=64, seqused_kv=[2000, 300, 4100], K2=512,
                         block_size1=64, block_size2=32, materialise_all_ori=False)
    rng = np.random.default_rng(431)
    for pool in (case.ori_kv, case.cmp_kv):
        sc = np.ascontiguousarray(pool[..., 576:604]).view(np.float32)
        mult = rng.choice(np.array([1.0, 1.5, 0.75, 1.2345], np.float32), size=sc.shape)
        pool[..., 576:604] = (sc * mult).view(np.uint8)
    plan = run_plan(TI.sparse_plan(case, DEV))
    check_out(to_f64(plan.out), O.sparse_sharedkv(case))


def test_sparse_window_only():
    case = W.sparse_case("swa", 410, B=2, N1=64, seqused_kv=[300, 50], K2=512,
                         materialise_all_ori=False)
    t = TI.sparse_tensors(case, DEV)
    plan = run_plan(fia.SparsePlan(t["q"], t["ori_kv"], None, None, t["ori_block_table"], None,
                                   t["seqused_kv"], t["sinks"], softmax_scale=case.softmax_scale,
                                   max_seqused_kv=300, cmp_ratio=1))
    case.cmp_sparse_indices[...] = -1
    check_out(to_f64(plan.out), O.sparse_sharedkv(case))


def test_sparse_heavily_compressed():
    case = W.sparse_case("hca", 420, B=4, N1=64, seqused_kv=[100, 1000, 16384, 5000],
                         block_size1=64, block_size2=16, heavily_compressed=True,
                         materialise_all_ori=False)
    assert case.cmp_sparse_indices is None and case.cmp_ratio == 128
    plan = run_plan(TI.sparse_plan(case, DEV))
    check_out(to_f64(plan.out), O.sparse_sharedkv(case))


def test_sparse_heavily_compressed_rows_are_bit_exact():
    case = W.sparse_case("hcr", 421, B=2, N1=64, seqused_kv=[300, 2000], block_size1=32,
                         block_size2=16, heavily_compressed=True, materialise_all_ori=False)
    plan = TI.sparse_plan(case, DEV)
    ids, rows = plan.debug_rows()
    torch.cuda.synchronize()
    ids, rows = ids.cpu().numpy()[:, 0], rows.cpu().numpy()[:, 0]
    n_win = 128
    for b, L in enumerate(case.seqused_kv):
        win, comp = O.sparse_rows(L, 1, 0, None, cmp_ratio=128, win_left=127, win_right=0)
        assert [int(x) for x in ids[b, :n_win] if x >= 0] == win
        assert [int(x) & ((1 << 30) - 1) for x in ids[b, n_win:] if x >= 0] == comp
        for s in range(n_win, ids.shape[1]):
            x = int(ids[b, s])
            if x < 0:
                assert not rows[b, s].any()
            else:
                c = x & ((1 << 30) - 1)
                want = case.cmp_kv[case.cmp_block_table[b, c // 16], c % 16, 0]
                assert np.array_equal(rows[b, s], want)


SPARSE_MULTI_CASES = [
    # (B, S1, N1, seqused, K2, hca)
    (2, 4, 64, [300, 5000], 512, False),
    (3, 2, 128, [9, 700, 130], 1024, False),
    (2, 3, 64, [1000, 4000], 0, True),
]


@pytest.mark.parametrize("i", range(len(SPARSE_MULTI_CASES)))
def test_sparse_multi_token(i):
    """S1 > 1: token t at p = Lk - S1 + t, window band [p - 127, p], compressed
    rows right-down causal over the compressed sequence."""
    B, S1, N1, L, K2, hca = SPARSE_MULTI_CASES[i]
    case = W.sparse_case(f"smt{i}", 430 + i, B=B, N1=N1, seqused_kv=L, K2=K2 or 512, S1=S1,
                         block_size1=64, block_size2=32, heavily_compressed=hca,
                         materialise_all_ori=False)
    plan = run_plan(TI.sparse_plan(case, DEV))
    check_out(to_f64(plan.out), O.sparse_sharedkv(case))


def test_sparse_strided_query_and_output():
    """q and attention_out as strided views (heads outermost in memory, so the
    head stride is S1 * 512), N1 = 128 (two head blocks)."""
    case = W.sparse_case("sstr", 445, B=2, N1=128, seqused_kv=[900, 3000], K2=512, S1=3,
                         block_size1=64, block_size2=32, materialise_all_ori=False)
    t = TI.sparse_tensors(case, DEV)
    q = t["q"]
    t["q"] = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)   # [B, S1, N1, 512] view
    assert t["q"].stride(2) == 3 * 512
    out = torch.zeros(q.shape[0], q.shape[2], q.shape[1], q.shape[3], dtype=q.dtype, device=DEV)
    plan = fia.SparsePlan(t["q"], t["ori_kv"], t["cmp_kv"], t["cmp_sparse_indices"],
                          t["ori_block_table"], t["cmp_block_table"], t["seqused_kv"], t["sinks"],
                          softmax_scale=case.softmax_scale, max_seqused_kv=max(case.seqused_kv),
                          cmp_ratio=case.cmp_ratio, attention_out=out.permute(0, 2, 1, 3))
    run_plan(plan)
    check_out(to_f64(out.permute(0, 2, 1, 3)), O.sparse_sharedkv(case))


def test_sparse_multi_token_rows_are_bit_exact():
    case = W.sparse_case("smr", 440, B=2, N1=64, seqused_kv=[40, 3000], K2=512, S1=5,
                         block_size1=32, block_size2=16, materialise_all_ori=False)
    plan = TI.sparse_plan(case, DEV)
    ids, rows = plan.debug_rows()
    torch.cuda.synchronize()
    ids, rows = ids.cpu().numpy(), rows.cpu().numpy()
    n_win = 128
    for b, L in enumerate(case.seqused_kv):
        for t in range(5):
            win, comp = O.sparse_rows(L, 5, t, case.cmp_sparse_indices[b, t, 0], cmp_ratio=4,
                                      win_left=127, win_right=0)
            assert [int(x) for x in ids[b, t, :n_win] if x >= 0] == win, (b, t)
            assert [int(x) & ((1 << 30) - 1) for x in ids[b, t, n_win:] if x >= 0] == comp, (b, t)
            for s in range(ids.shape[2]):
                x = int(ids[b, t, s])
                if x < 0:
                    assert not rows[b, t, s].any()
                elif x >> 30:
                    c = x & ((1 << 30) - 1)
                    assert np.array_equal(rows[b, t, s], case.cmp_kv[case.cmp_block_table[b, c // 16], c % 16, 0])
                else:
                    assert np.array_equal(rows[b, t, s], case.ori_kv[case.ori_block_table[b, x // 32], x % 32, 0])


SPARSE_TND_CASES = [
    # (q_counts, N1, seqused, K2, hca)
    ([1, 3, 0, 2], 64, [300, 5000, 77, 1000], 512, False),
    ([2, 1], 128, [9, 4000], 1024, False),
    ([3, 1, 2], 64, [1000, 4000, 130], 0, True),
]


@pytest.mark.parametrize("i", range(len(SPARSE_TND_CASES)))
def test_sparse_tnd(i):
    """layout_q TND: entry b owns packed rows cu[b] .. cu[b + 1] - 1 of q
    [T1, N1, 512]; the row-to-entry map is read from cu_seqlens_q on the device."""
    counts, N1, L, K2, hca = SPARSE_TND_CASES[i]
    case = W.sparse_tnd_case(f"stnd{i}", 450 + i, q_counts=counts, B=len(counts), N1=N1,
                             seqused_kv=L, K2=K2 or 512, block_size1=64, block_size2=32,
                             heavily_compressed=hca, materialise_all_ori=False)
    plan = run_plan(TI.sparse_plan(case, DEV))
    assert tuple(plan.out.shape) == (sum(counts), N1, 512)
    check_out(to_f64(plan.out), O.sparse_sharedkv(case))


def test_sparse_tnd_rows_are_bit_exact():
    counts = [2, 0, 4, 1]
    case = W.sparse_tnd_case("stndr", 460, q_counts=counts, B=4, N1=64, seqused_kv=[40, 9, 3000, 700],
                             K2=512, block_size1=32, block_size2=16, materialise_all_ori=False)
    plan = TI.sparse_plan(case, DEV)
    ids, rows = plan.debug_rows()
    torch.cuda.synchronize()
    ids, rows = ids.cpu().numpy(), rows.cpu().numpy()
    assert ids.shape[0] == sum(counts)
    n_win = 128
    cu = case.cu_seqlens_q
    for b, L in enumerate(case.seqused_kv):
        for t in range(counts[b]):
            r = cu[b] + t
            win, comp = O.sparse_rows(L, counts[b], t, case.cmp_sparse_indices[r, 0], cmp_ratio=4,
                                      win_left=127, win_right=0)
            assert [int(x) for x in ids[r, :n_win] if x >= 0] == win, (b, t)
            assert [int(x) & ((1 << 30) - 1) for x in ids[r, n_win:] if x >= 0] == comp, (b, t)
            for s in range(ids.shape[1]):
                x = int(ids[r, s])
                if x < 0:
                    assert not rows[r, s].any()
                elif x >> 30:
                    c = x & ((1 << 30) - 1)
                    assert np.array_equal(rows[r, s], case.cmp_kv[case.cmp_block_table[b, c // 16], c % 16, 0])
                else:
                    assert np.array_equal(rows[r, s], case.ori_kv[case.ori_block_table[b, x // 32], x % 32, 0])


def test_sparse_tnd_rows_outside_every_entry_are_zero():
    """cu_seqlens_q ending before T1 (inconsistent counts): the rows past the
    last entry are written as 0, the others as usual."""
    case = W.sparse_tnd_case("stndz", 470, q_counts=[1, 2], B=2, N1=64, seqused_kv=[300, 80],
                             K2=512, block_size1=32, block_size2=16, materialise_all_ori=False)
    case.cu_seqlens_q = [0, 1, 2]
    plan = run_plan(TI.sparse_plan(case, DEV))
    got = to_f64(plan.out)
    assert np.all(got[2] == 0)
    check_out(got, O.sparse_sharedkv(case))


# ---------------------------------------------------------------------------
# Decode with KV lengths on the device (device-side partitioner).
# ---------------------------------------------------------------------------
def _dev_len_plan(case, lens_dev, bound, **kw):
    q, k, v, bt, _ = TI.dense_tensors(case, DEV)
    return fia.AttentionPlan(q, k, v, num_heads=case.num_heads,
                             num_key_value_heads=case.num_kv_heads, scale_value=case.scale,
                             sparse_mode=case.sparse_mode, pre_tokens=case.pre_tokens,
                             next_tokens=case.next_tokens, block_table=bt,
                             block_size=case.block_size if bt is not None else 0,
                             kv_layout=case.kv_layout, softmax_lse_flag=case.lse,
                             actual_seq_lengths_kv_device=lens_dev, max_actual_seq_length_kv=bound,
                             **TI.antiquant_kwargs(case, DEV), **kw)


DEV_LEN_CASES = [
    # (mode, pre, next, sink)
    (0, 2147483647, 2147483647, False),
    (3, 2147483647, 2147483647, True),
    (4, 700, 0, False),
]


@pytest.mark.parametrize("i", range(len(DEV_LEN_CASES)))
def test_decode_device_lengths_match_host_plan(i):
    """The partitioner kernel builds the plan the host builds for the same
    lengths: outputs and LSE equal the host-planned run bit for bit, and
    match the oracle.  The lengths then change on the device and the same
    executor runs again (no new plan), against a host plan of the new
    lengths; lengths past the bound are clamped to it."""
    mode, pre, nxt, sink = DEV_LEN_CASES[i]
    lens = [1, 700, 5000, 4097, 129, 2048]
    lens2 = [3000, 0, 1, 6000, 6001, 511]
    bound = 6000
    # the pool holds real rows for the longer of the two lengths of each entry
    alloc = [max(a, min(b, bound)) for a, b in zip(lens, lens2)]
    base = W.paged_decode_case(f"dl{i}", 480 + i, B=6, Q_N=32, KV_N=8, D=128, kv_lens=alloc,
                               block_size=128, sparse_mode=mode, lse=True)
    assert base.block_table.shape[1] * 128 >= bound
    case = dataclasses.replace(base, actual_seq_lengths_kv=lens, pre_tokens=pre, next_tokens=nxt)
    extra = {}
    if sink:
        case = W.with_random_sink(case, 481)
        extra["learnable_sink"] = TI.to_device(case.learnable_sink, "bf16", DEV)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=DEV)
    plan = run_plan(_dev_len_plan(case, lens_dev, bound, **extra))
    assert plan.kind == "decode"
    host = run_plan(TI.dense_plan(case, DEV))
    assert torch.equal(plan.out.view(torch.int16), host.out.view(torch.int16))
    assert torch.equal(plan.lse, host.lse)
    out, lse = gpu_results(plan)
    ref_o, ref_l = O.fia_case(case)
    check_out(out, ref_o)
    check_lse(lse, ref_l)
    # new lengths, same executor: shorter, longer, zero and one past the bound
    lens_dev.copy_(torch.tensor(lens2, dtype=torch.int32))
    run_plan(plan)
    case2 = dataclasses.replace(case, actual_seq_lengths_kv=[min(x, bound) for x in lens2])
    host2 = run_plan(TI.dense_plan(case2, DEV))
    assert torch.equal(plan.out.view(torch.int16), host2.out.view(torch.int16))
    assert torch.equal(plan.lse, host2.lse)
    out2, lse2 = gpu_results(plan)
    ref_o2, ref_l2 = O.fia_case(case2)
    check_out(out2, ref_o2)
    check_lse(lse2, ref_l2)


DEV_LEN_DENSE_CASES = [
    # (Q_N, KV_N, D, lse): dense BSND KV, group sizes 1 / 16 / 64, head dims 64 / 128
    (8, 8, 128, False),
    (32, 2, 64, True),
    (64, 1, 128, True),
]


@pytest.mark.parametrize("i", range(len(DEV_LEN_DENSE_CASES)))
def test_decode_device_lengths_dense_kv(i):
    """Device-resident lengths with a dense (non-paged) KV cache: equal to the
    host-planned run bit for bit and to the oracle; the bound is KV_S."""
    Qn, KVn, D, lse = DEV_LEN_DENSE_CASES[i]
    lens = [0, 1, 513, 1500, 2048]
    case = W.dense_case(f"dld{i}", 495 + i, B=5, S1=1, S2=2048, Q_N=Qn, KV_N=KVn, D=D,
                        kv_lens=lens, lse=lse)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q, k, v, _, _ = TI.dense_tensors(case, DEV)
    plan = run_plan(fia.AttentionPlan(q, k, v, num_heads=Qn, num_key_value_heads=KVn,
                                      scale_value=case.scale, softmax_lse_flag=lse,
                                      actual_seq_lengths_kv_device=lens_dev,
                                      max_actual_seq_length_kv=2048))
    host = run_plan(TI.dense_plan(case, DEV))
    assert torch.equal(plan.out.view(torch.int16), host.out.view(torch.int16))
    if lse:
        assert torch.equal(plan.lse, host.lse)
    out, lse_v = gpu_results(plan)
    ref_o, ref_l = O.fia_case(case)
    check_out(out, ref_o)
    if lse:
        check_lse(lse_v, ref_l)


DEV_LEN_QUANT_CASES = [
    # (kind, kmode, vmode, offsets, builder(kv_lens))
    ("int8", 1, 1, True,
     lambda kl: W.paged_decode_case("dlq0", 520, B=4, Q_N=32, KV_N=8, D=128, kv_lens=kl,
                                    block_size=128, lse=True)),
    ("fp8", 0, 0, False,
     lambda kl: W.as_bnnbsd(W.paged_decode_case("dlq1", 521, B=4, Q_N=16, KV_N=4, D=128,
                                                kv_lens=kl, block_size=64, lse=True))),
    ("int8", 0, 1, True,
     lambda kl: W.dense_case("dlq2", 522, B=4, S1=1, S2=3000, Q_N=8, KV_N=2, D=64, kv_lens=kl,
                             lse=True)),
]


@pytest.mark.parametrize("i", range(len(DEV_LEN_QUANT_CASES)))
def test_decode_fake_quant_device_lengths(i):
    """Fake-quantised key / value with device-resident lengths: equal to the
    host-planned run bit for bit and to the oracle, then again after the
    lengths change on the device (zero, one, the bound and one past it)."""
    kind, km, vm, off, build = DEV_LEN_QUANT_CASES[i]
    lens = [1, 700, 2999, 129]
    lens2 = [3000, 0, 1, 3001]
    bound = 3000
    alloc = [max(a, min(b, bound)) for a, b in zip(lens, lens2)]
    base = W.with_kv_quant(build(alloc), 530 + i, kind=kind, kmode=km, vmode=vm, offsets=off)
    case = dataclasses.replace(base, actual_seq_lengths_kv=lens)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=DEV)
    plan = run_plan(_dev_len_plan(case, lens_dev, bound))
    assert plan.kind == "decode"
    host = run_plan(TI.dense_plan(case, DEV))
    assert torch.equal(plan.out.view(torch.int16), host.out.view(torch.int16))
    assert torch.equal(plan.lse, host.lse)
    out, lse = gpu_results(plan)
    ref_o, ref_l = O.fia_case(case)
    check_out(out, ref_o)
    check_lse(lse, ref_l)
    lens_dev.copy_(torch.tensor(lens2, dtype=torch.int32))
    run_plan(plan)
    case2 = dataclasses.replace(base, actual_seq_lengths_kv=[min(x, bound) for x in lens2])
    host2 = run_plan(TI.dense_plan(case2, DEV))
    assert torch.equal(plan.out.view(torch.int16), host2.out.view(torch.int16))
    assert torch.equal(plan.lse, host2.lse)
    out2, lse2 = gpu_results(plan)
    ref_o2, ref_l2 = O.fia_case(case2)
    check_out(out2, ref_o2)
    check_lse(lse2, ref_l2)


DEV_LEN_PREFILL_CASES = [
    # (mask mode, paged block size (0: dense KV), D)
    (3, 128, 128),
    (0, 32, 128),
    (3, 0, 64),
]


@pytest.mark.parametrize("i", range(len(DEV_LEN_PREFILL_CASES)))
def test_prefill_device_lengths(i):
    """A 40-row prompt chunk against a cache whose lengths live on the
    device (items planned for the bound): equal to the host-planned run bit
    for bit and to the oracle, then again after the lengths change on the
    device (zero, one, the bound and one past it; with right-down causality
    rows with no visible key come out as 0 / +inf)."""
    mode, bs, D = DEV_LEN_PREFILL_CASES[i]
    lens = [40, 700, 2999, 129]
    lens2 = [3000, 0, 1, 3001]
    bound = 3000
    alloc = [max(a, min(b, bound)) for a, b in zip(lens, lens2)]
    if bs:
        base = W.paged_decode_case(f"dlp{i}", 540 + i, B=4, Q_N=8, KV_N=2, D=D, kv_lens=alloc,
                                   block_size=bs, S1=40, sparse_mode=mode, lse=True)
        assert base.block_table.shape[1] * bs >= bound
    else:
        base = W.dense_case(f"dlp{i}", 540 + i, B=4, S1=40, S2=bound, Q_N=8, KV_N=2, D=D,
                            kv_lens=alloc, sparse_mode=mode, lse=True)
    case = dataclasses.replace(base, actual_seq_lengths_kv=lens)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=DEV)
    plan = run_plan(_dev_len_plan(case, lens_dev, bound))
    assert plan.kind == "prefill"
    host = run_plan(TI.dense_plan(case, DEV))
    assert torch.equal(plan.out.view(torch.int16), host.out.view(torch.int16))
    assert torch.equal(plan.lse, host.lse)
    out, lse = gpu_results(plan)
    ref_o, ref_l = O.fia_case(case)
    check_out(out, ref_o)
    check_lse(lse, ref_l)
    lens_dev.copy_(torch.tensor(lens2, dtype=torch.int32))
    run_plan(plan)
    case2 = dataclasses.replace(base, actual_seq_lengths_kv=[min(x, bound) for x in lens2])
    host2 = run_plan(TI.dense_plan(case2, DEV))
    assert torch.equal(plan.out.view(torch.int16), host2.out.view(torch.int16))
    assert torch.equal(plan.lse, host2.lse)
    out2, lse2 = gpu_results(plan)
    ref_o2, ref_l2 = O.fia_case(case2)
    check_out(out2, ref_o2)
    check_lse(lse2, ref_l2)


def test_decode_device_lengths_graph_replay():
    """The decode with device-resident lengths captured once into a HIP graph
    (after one eager run) and replayed with new lengths written between the
    replays, with eager work in between: every replay equals the host-planned
    run of its lengths bit for bit."""
    lens_sets = [[700, 5000, 1, 2048], [6000, 0, 129, 3000], [1, 1, 4097, 5999]]
    bound = 6000
    alloc = [max(x) for x in zip(*lens_sets)]
    base = W.paged_decode_case("dlg", 490, B=4, Q_N=32, KV_N=8, D=128, kv_lens=alloc,
                               block_size=128, sparse_mode=3, lse=True)
    lens_dev = torch.tensor(lens_sets[0], dtype=torch.int32, device=DEV)
    plan = run_plan(_dev_len_plan(base, lens_dev, bound))   # eager run first
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            plan.run(stream)
    torch.cuda.synchronize()
    for rep in range(2):
        for lens in lens_sets:
            lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
            scratch = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
            graph.replay()
            torch.cuda.synchronize()
            host = run_plan(TI.dense_plan(dataclasses.replace(base, actual_seq_lengths_kv=lens), DEV))
            assert torch.equal(plan.out.view(torch.int16), host.out.view(torch.int16)), (rep, lens)
            assert torch.equal(plan.lse, host.lse), (rep, lens)
            del scratch


# ---------------------------------------------------------------------------
# Bit-exact gathers and row selection.
# ---------------------------------------------------------------------------
def test_paged_gather_is_bit_exact():
    case = W.paged_decode_case("g", 500, B=3, Q_N=8, KV_N=2, D=128, kv_lens=[1, 300, 1029],
                               block_size=16, poison_tail=True, extra_blocks=4)
    plan = TI.dense_plan(case, DEV)
    s2 = max(case.actual_seq_lengths_kv)
    for which, pool in ((0, case.k_pool), (1, case.v_pool)):
        got = plan.debug_gather(which, s2)
        torch.cuda.synchronize()
        got = got.cpu().view(torch.int16).numpy().view(np.uint16)
        for b, L in enumerate(case.actual_seq_lengths_kv):
            j = np.arange(L)
            want = pool[case.block_table[b, j // 16], j % 16]
            assert np.array_equal(got[b, :L], want), (which, b)


def test_paged_gather_of_fake_quant_codes_is_bit_exact():
    """One-byte key / value codes are gathered as bytes (the row of a code is
    D bytes long), through the same row-address function."""
    case = W.with_kv_quant(W.paged_decode_case("gq", 505, B=2, Q_N=8, KV_N=2, D=128,
                                               kv_lens=[77, 700], block_size=32, poison_tail=True),
                           506, kind="int8", kmode=1, vmode=1, offsets=True)
    plan = TI.dense_plan(case, DEV)
    s2 = max(case.actual_seq_lengths_kv)
    for which, pool in ((0, case.k_pool), (1, case.v_pool)):
        got = plan.debug_gather(which, s2)
        torch.cuda.synchronize()
        got = got.cpu().numpy().view(np.uint8)
        for b, L in enumerate(case.actual_seq_lengths_kv):
            want = O.gather_paged(pool, case.block_table[b], L, 32).view(np.uint8)
            assert np.array_equal(got[b, :L], want), (which, b)


def test_sparse_row_selection_is_bit_exact():
    case = W.sparse_case("sr", 510, B=3, N1=64, seqused_kv=[5, 300, 4000], K2=512, n_valid=100,
                         block_size1=32, block_size2=16, materialise_all_ori=False)
    case.cmp_sparse_indices[1, 0, 0, 3] = 10 ** 6      # out of range: must be skipped
    plan = TI.sparse_plan(case, DEV)
    ids, rows = plan.debug_rows()
    torch.cuda.synchronize()
    ids, rows = ids.cpu().numpy()[:, 0], rows.cpu().numpy()[:, 0]
    n_win = 128
    for b, L in enumerate(case.seqused_kv):
        win, comp = O.sparse_rows(L, 1, 0, case.cmp_sparse_indices[b, 0, 0], cmp_ratio=4,
                                  win_left=127, win_right=0)
        got_win = [int(x) for x in ids[b, :n_win] if x >= 0]
        assert got_win == win
        got_comp = [int(x) & ((1 << 30) - 1) for x in ids[b, n_win:] if x >= 0]
        assert got_comp == comp
        for s in range(ids.shape[1]):
            x = int(ids[b, s])
            if x < 0:
                assert not rows[b, s].any()
            elif x >> 30:
                c = x & ((1 << 30) - 1)
                want = case.cmp_kv[case.cmp_block_table[b, c // 16], c % 16, 0]
                assert np.array_equal(rows[b, s], want)
            else:
                want = case.ori_kv[case.ori_block_table[b, x // 32], x % 32, 0]
                assert np.array_equal(rows[b, s], want)


# ---------------------------------------------------------------------------
# Determinism and batch invariance.
# ---------------------------------------------------------------------------
def test_repeat_runs_are_bitwise_identical():
    case = W.paged_decode_case("det", 600, B=4, Q_N=32, KV_N=8, D=128,
                               kv_lens=[3000, 17, 1200, 4097], block_size=128)
    plan = run_plan(TI.dense_plan(case, DEV))
    first = plan.out.clone()
    first_lse = plan.lse.clone()
    for _ in range(3):
        run_plan(plan)
        assert torch.equal(plan.out, first) and torch.equal(plan.lse, first_lse)
    pc = W.dense_case("detp", 601, B=2, S1=300, S2=300, Q_N=8, KV_N=2, D=128, sparse_mode=3)
    pp = run_plan(TI.dense_plan(pc, DEV))
    f2 = pp.out.clone()
    run_plan(pp)
    assert torch.equal(pp.out, f2)
    sc = W.sparse_case("dets", 602, B=2, N1=64, seqused_kv=[5000, 700], K2=512,
                       materialise_all_ori=False)
    sp = run_plan(TI.sparse_plan(sc, DEV))
    f3 = sp.out.clone()
    run_plan(sp)
    assert torch.equal(sp.out, f3)


def test_decode_batch_invariance():
    lens = [4100, 90, 2500, 7000]
    case = W.dense_case("bi", 610, B=4, S1=1, S2=max(lens), Q_N=16, KV_N=4, D=128, kv_lens=lens,
                        lse=True)
    q, k, v, _, _ = TI.dense_tensors(case, DEV)
    full = run_plan(fia.AttentionPlan(q, k, v, num_heads=16, num_key_value_heads=4,
                                      scale_value=case.scale, softmax_lse_flag=True,
                                      actual_seq_lengths_kv=lens))
    for b in (0, 3):
        one = run_plan(fia.AttentionPlan(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(),
                                         v[b:b + 1].contiguous(), num_heads=16,
                                         num_key_value_heads=4, scale_value=case.scale,
                                         softmax_lse_flag=True, actual_seq_lengths_kv=[lens[b]]))
        assert torch.equal(one.out[0], full.out[b])
        assert torch.equal(one.lse[0], full.lse[b])
    # reversed batch order
    perm = [3, 2, 1, 0]
    rev = run_plan(fia.AttentionPlan(q[perm].contiguous(), k[perm].contiguous(),
                                     v[perm].contiguous(), num_heads=16, num_key_value_heads=4,
                                     scale_value=case.scale, softmax_lse_flag=True,
                                     actual_seq_lengths_kv=[lens[p] for p in perm]))
    for i, p in enumerate(perm):
        assert torch.equal(rev.out[i], full.out[p])


def test_prefill_batch_invariance():
    lens = [300, 129, 77]
    case = W.dense_case("pbi", 620, B=3, S1=300, S2=300, Q_N=8, KV_N=2, D=128, sparse_mode=3,
                        q_lens=lens, kv_lens=lens)
    q, k, v, _, _ = TI.dense_tensors(case, DEV)
    kw = dict(num_heads=8, num_key_value_heads=2, scale_value=case.scale, sparse_mode=3)
    full = run_plan(fia.AttentionPlan(q, k, v, actual_seq_lengths=lens, actual_seq_lengths_kv=lens, **kw))
    one = run_plan(fia.AttentionPlan(q[1:2].contiguous(), k[1:2].contiguous(), v[1:2].contiguous(),
                                     actual_seq_lengths=[lens[1]], actual_seq_lengths_kv=[lens[1]], **kw))
    assert torch.equal(one.out[0], full.out[1])


def test_sparse_batch_invariance():
    case = W.sparse_case("sbi", 630, B=3, N1=64, seqused_kv=[3000, 600, 5000], K2=512,
                         materialise_all_ori=False)
    t = TI.sparse_tensors(case, DEV)
    full = run_plan(TI.sparse_plan(case, DEV, tensors=t))
    sub = {k: (v[1:2].contiguous() if v is not None and k not in ("ori_kv", "cmp_kv", "sinks") else v)
           for k, v in t.items()}
    one = run_plan(fia.SparsePlan(sub["q"], sub["ori_kv"], sub["cmp_kv"],
                                  sub["cmp_sparse_indices"], sub["ori_block_table"],
                                  sub["cmp_block_table"], sub["seqused_kv"], sub["sinks"],
                                  softmax_scale=case.softmax_scale, max_seqused_kv=600))
    assert torch.equal(one.out[0], full.out[1])


@pytest.mark.parametrize("kind", ["bf16", "int8", "bf16_bnnbsd"])
def test_decode_read_probe_reads_exactly_the_visible_rows(kind):
    """fia_debug_read_kv (the access-pattern read ceiling the benchmark
    reports) reads every visible key and value row once and nothing else:
    the XOR of the words it read, in either order, equals the XOR of the
    visible rows gathered on the host (tail slots past each length hold NaN)."""
    case = W.paged_decode_case("rdp", 470, B=3, Q_N=32, KV_N=8, D=128, kv_lens=[1, 1500, 3000],
                               block_size=128, lse=True, poison_tail=True)
    if kind == "int8":
        case = W.with_kv_quant(case, 471, kind="int8", kmode=1, vmode=1, offsets=True)
    if kind.endswith("bnnbsd"):
        case = W.as_bnnbsd(case)
    want = np.uint32(0)
    for pool in (case.k_pool, case.v_pool):
        for b, L in enumerate(case.actual_seq_lengths_kv):
            rows = O.gather_paged(pool, case.block_table[b], L, case.block_size, case.kv_layout)
            want ^= np.bitwise_xor.reduce(np.ascontiguousarray(rows).view(np.uint32), axis=None)
    plan = TI.dense_plan(case, DEV)
    orders = [0] if kind.endswith("bnnbsd") else [0, 1]
    for order in orders:
        words = plan.read_kv(order)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(words.cpu().numpy().view(np.uint32), axis=None)
        assert got == want, (order, hex(int(got)), hex(int(want)))
