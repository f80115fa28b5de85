"""GPU parity of the sparse operators' second row format and of the shared
sparse kernel's fp8 conversion: sparse_flash_mla over fp16 / bf16 rows
(SWA / CSA / HCA; PA_BBND, BSND and TND KV; BSND and TND queries; optional
sink and LSE) against the float64 oracle, with bit-exact row selection, and
every e4m3fn code in every byte position of a packed row."""
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


def sfmla_parity(case):
    plan = run_plan(TI.sfmla_plan(case, DEV))
    assert plan.kind == "sparse"
    ref_o, ref_l = O.sparse_flash_mla(case)
    check_out(to_f64(plan.out), ref_o)
    if case.return_lse:
        check_lse(to_f64(plan.lse), ref_l)
    return plan


def test_sfmla_decode_bf16_full():
    """The shared-KV sparse decode shape with bf16 rows: B=16, N1=64, KV length
    16384, top-512 of the ratio-4 compressed rows, PA_BBND block 128, sinks,
    LSE; every ori row outside a query's window is NaN."""
    sfmla_parity(W.sfmla_decode_bf16())


SFMLA_CASES = [
    # (mode, dtype, kv_layout, B, N1, lens, K2, bs1, bs2, S1, sinks, lse)
    ("CSA", "bf16", "PA_BBND", 3, 64, [900, 300, 5000], 512, 128, 128, 1, True, True),
    ("CSA", "fp16", "PA_BBND", 2, 128, [2000, 777], 1024, 64, 16, 1, False, True),
    ("CSA", "bf16", "PA_BBND", 2, 8, [700, 90], 100, 1, 3, 1, True, True),
    ("CSA", "fp16", "PA_BBND", 3, 2, [37, 4000, 129], 1, 7, 1024, 1, True, False),
    ("HCA", "bf16", "PA_BBND", 2, 32, [20000, 3000], 0, 128, 16, 2, True, True),
    ("HCA", "fp16", "PA_BBND", 3, 64, [129, 1000, 9000], 0, 64, 5, 1, False, True),
    ("SWA", "fp16", "PA_BBND", 3, 16, [200, 50, 1], 0, 32, 16, 1, False, True),
    ("SWA", "bf16", "PA_BBND", 2, 128, [300, 127], 0, 16, 16, 3, True, True),
    ("CSA", "bf16", "BSND", 2, 64, [1500, 300], 512, 0, 0, 3, True, True),
    ("HCA", "fp16", "BSND", 2, 1, [3000, 900], 0, 0, 0, 1, True, True),
    ("SWA", "bf16", "BSND", 2, 4, [60, 500], 0, 0, 0, 2, False, True),
]


@pytest.mark.parametrize("i", range(len(SFMLA_CASES)))
def test_sfmla_sweep(i):
    mode, dt, lay, B, N1, lens, K2, bs1, bs2, S1, sinks, lse = SFMLA_CASES[i]
    case = W.sfmla_case(f"fm{i}", 900 + i, B=B, N1=N1, seqused_kv=lens, mode=mode, K2=max(K2, 1),
                        dtype=dt, kv_layout=lay, block_size1=max(bs1, 1), block_size2=max(bs2, 1),
                        S1=S1, sinks=sinks, lse=lse, window_only_ori=True)
    sfmla_parity(case)


SFMLA_TND_CASES = [
    # (counts, mode, dtype, kv_layout, N1, lens, K2)
    ([2, 0, 3, 1], "CSA", "bf16", "TND", 64, [300, 50, 2000, 9], 512),
    ([1, 4], "HCA", "fp16", "TND", 16, [900, 3000], 0),
    ([3, 1, 0], "SWA", "bf16", "TND", 8, [200, 40, 100], 0),
    ([2, 2], "CSA", "fp16", "PA_BBND", 128, [700, 1500], 1024),
]


@pytest.mark.parametrize("i", range(len(SFMLA_TND_CASES)))
def test_sfmla_tnd(i):
    counts, mode, dt, lay, N1, lens, K2 = SFMLA_TND_CASES[i]
    case = W.sfmla_tnd_case(f"ft{i}", 930 + i, q_counts=counts, B=len(counts), N1=N1,
                            seqused_kv=lens, mode=mode, K2=max(K2, 1), dtype=dt, kv_layout=lay,
                            block_size1=32, block_size2=16, window_only_ori=True)
    sfmla_parity(case)


def test_sfmla_tnd_rows_outside_every_entry():
    """cu_seqlens_q ending before T1: rows past the last entry are 0 / +inf."""
    case = W.sfmla_tnd_case("ftz", 940, q_counts=[1, 3], B=2, N1=8, seqused_kv=[300, 80], K2=64,
                            block_size1=32, block_size2=16)
    case.cu_seqlens_q = [0, 1, 2]
    plan = sfmla_parity(case)
    out = to_f64(plan.out)
    assert np.all(out[2:] == 0) and np.all(np.isposinf(to_f64(plan.lse)[0, 2:]))


def test_sfmla_empty_entries():
    """An entry with KV length 0 has no row: 0 and +inf, or 0 and the sink."""
    for sinks in (False, True):
        case = W.sfmla_case("fe", 941 + sinks, B=3, N1=16, seqused_kv=[0, 600, 0], K2=64,
                            block_size1=32, block_size2=16, sinks=sinks)
        plan = sfmla_parity(case)
        out, lse = to_f64(plan.out), to_f64(plan.lse)
        assert np.all(out[0] == 0) and np.all(out[2] == 0)
        if sinks:
            # (sink * log2 e) * ln 2 in fp32: the sink itself up to rounding
            np.testing.assert_allclose(lse[0, 0, 0], case.sinks.astype(np.float64), rtol=0, atol=1e-6)
        else:
            assert np.all(np.isposinf(lse[0])) and np.all(np.isposinf(lse[2]))


@pytest.mark.parametrize("lay", ["PA_BBND", "BSND"])
def test_sfmla_rows_are_bit_exact(lay):
    """The row list of every slot and its raw 1024 bytes against a CPU gather
    (window band, valid visible indices in index order, unused slots zero);
    block sizes 3 and 5 in the paged layout."""
    case = W.sfmla_case("fr", 950, B=3, N1=8, seqused_kv=[5, 300, 4000], K2=200, n_valid=120,
                        kv_layout=lay, block_size1=3, block_size2=5, S1=2)
    case.cmp_sparse_indices[1, 1, 0, 3] = 10 ** 6      # out of range: skipped
    case.cmp_sparse_indices[2, 0, 0, 7] = -5           # negative: skipped
    plan = TI.sfmla_plan(case, DEV)
    ids, rows = plan.debug_rows()
    torch.cuda.synchronize()
    ids, rows = ids.cpu().numpy(), rows.cpu().numpy()
    n_win = 128

    def row_bytes(which, b, r):
        kv = case.ori_kv if which == 0 else case.cmp_kv
        if lay == "PA_BBND":
            bt = case.ori_block_table if which == 0 else case.cmp_block_table
            bs = kv.shape[1]
            return kv[bt[b, r // bs], r % bs, 0].view(np.uint8)
        return kv[b, r, 0].view(np.uint8)

    for b, L in enumerate(case.seqused_kv):
        for t in range(2):
            win, comp = O.sparse_rows(L, 2, t, case.cmp_sparse_indices[b, t, 0], cmp_ratio=4,
                                      win_left=127, win_right=0)
            got = ids[b, t]
            assert [int(x) for x in got[:n_win] if x >= 0] == win
            assert [int(x) & ((1 << 30) - 1) for x in got[n_win:] if x >= 0] == comp
            for s in range(got.shape[0]):
                x = int(got[s])
                if x < 0:
                    assert not rows[b, t, s].any()
                else:
                    want = row_bytes(x >> 30, b, x & ((1 << 30) - 1))
                    assert np.array_equal(rows[b, t, s], want)


def test_sfmla_repeat_and_batch_invariance():
    case = W.sfmla_case("fbi", 960, B=3, N1=64, seqused_kv=[3000, 600, 5000], K2=512,
                        window_only_ori=True)
    t = TI.sfmla_tensors(case, DEV)
    full = run_plan(TI.sfmla_plan(case, DEV, tensors=t))
    first = full.out.clone()
    full.run()
    torch.cuda.synchronize()
    assert torch.equal(first, full.out)
    one_case = dataclasses.replace(case, q=case.q[1:2], cmp_sparse_indices=case.cmp_sparse_indices[1:2],
                                   ori_block_table=case.ori_block_table[1:2],
                                   cmp_block_table=case.cmp_block_table[1:2],
                                   seqused_kv=case.seqused_kv[1:2])
    one = run_plan(TI.sfmla_plan(one_case, DEV))
    assert torch.equal(one.out[0], full.out[1])
    assert torch.equal(one.lse[0], full.lse[1])


# ---------------------------------------------------------------------------
# The packed-row fp8 conversion of the sparse kernel: every code everywhere.
# ---------------------------------------------------------------------------
def _one_row_entries(rows):
    """A shared-KV case in the window-only mode where batch entry b has KV
    length 1 (its only row is rows[b]), q = 0 and sinks = -inf: every score
    is 0 and the single row gets weight 1, so the output is the row itself."""
    B = rows.shape[0]
    case = W.sparse_case("e4", 970, B=B, N1=64, seqused_kv=[1] * B, K2=512, block_size1=16,
                         block_size2=16)
    pool = np.zeros((B, 16, 1, 640), np.uint8)
    pool[:, 0, 0] = rows
    table = np.arange(B, dtype=np.int32)[:, None]
    # For the oracle the window-only mode is the compressed-sparse mode with
    # every index entry unused.
    return dataclasses.replace(case, q=np.zeros_like(case.q), ori_kv=pool, ori_block_table=table,
                               cmp_kv=np.zeros((1, 16, 1, 640), np.uint8),
                               cmp_sparse_indices=np.full((B, 1, 1, 512), -1, np.int32),
                               cmp_block_table=np.zeros((B, 1), np.int32),
                               sinks=np.full(64, -np.inf, np.float32))


def test_sparse_fp8_every_code_in_every_position():
    """Row b holds code (b + d) mod 256 at nope position d (every code at
    every one of the 448 byte positions over 256 entries, NaN codes 0x7F /
    0xFF replaced by 0x00), tile scales 2^-3 .. 2^3 and a bf16 rope ramp;
    the output must equal the exactly decoded row, bit for bit."""
    B = 256
    rows = np.zeros((B, 640), np.uint8)
    d = np.arange(448)
    for b in range(B):
        codes = ((b + d) % 256).astype(np.uint8)
        codes[(codes == 0x7F) | (codes == 0xFF)] = 0
        rows[b, 128:576] = codes
        rope = W.f32_to_bf16_bits(np.linspace(-3, 3, 64, dtype=np.float32) * (b + 1) / 7)
        rows[b, :128] = rope.view(np.uint8)
        rows[b, 576:604] = np.array([2.0 ** e for e in range(-3, 4)], np.float32).view(np.uint8)
    case = _one_row_entries(rows)
    t = TI.sparse_tensors(case, DEV)
    plan = run_plan(fia.SparsePlan(t["q"], t["ori_kv"], None, None, t["ori_block_table"], None,
                                   t["seqused_kv"], t["sinks"], softmax_scale=case.softmax_scale,
                                   max_seqused_kv=1, cmp_ratio=1))
    got = to_f64(plan.out)[:, 0]                         # [B, 64 heads, 512]
    want = np.stack([O.decode_packed_row(r) for r in rows])
    assert np.all(np.isfinite(want))
    for h in (0, 63):
        assert np.array_equal(got[:, h], want), np.argwhere(got[:, h] != want)[:5]
    # every e4m3fn value was seen, subnormals (exponent field 0) included
    seen = set(np.unique(rows[:, 128:576]).tolist())
    assert seen == set(range(256)) - {0x7F, 0xFF}


def test_sparse_fp8_nan_codes_poison_their_row():
    """A NaN code (0x7F or 0xFF) makes its row's output NaN, as in the oracle."""
    rows = np.zeros((2, 640), np.uint8)
    rows[:, 576:604] = np.ones(7, np.float32).view(np.uint8)
    rows[0, 128 + 5] = 0x7F
    rows[1, 128 + 300] = 0xFF
    case = _one_row_entries(rows)
    t = TI.sparse_tensors(case, DEV)
    plan = run_plan(fia.SparsePlan(t["q"], t["ori_kv"], None, None, t["ori_block_table"], None,
                                   t["seqused_kv"], t["sinks"], softmax_scale=case.softmax_scale,
                                   max_seqused_kv=1, cmp_ratio=1))
    got = to_f64(plan.out)
    assert np.isnan(O.sparse_sharedkv(case)).all()
    assert np.isnan(got).all()
