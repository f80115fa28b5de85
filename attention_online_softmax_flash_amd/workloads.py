"""Seeded synthetic inputs for fused inference attention.

This module draws random numbers and lays them out in memory; it holds none
of the attention arithmetic.  Both the CPU oracle (through the tests) and the
HIP library (through the binding, tests and benchmark) consume the arrays it
returns, so every comparison runs on identical bytes.

Storage conventions of the returned numpy arrays:
  * bf16 tensors are ``uint16`` bit patterns (numpy has no bfloat16);
  * fp32 tensors are ``float32``;
  * packed shared-KV rows are ``uint8`` with 640 bytes per row;
  * integer tensors (block tables, indices) are ``int32``.

Random streams are numpy PCG64 seeded per case.  Shapes and distributions
follow the workloads of the fused-inference-attention pages: BSND / TND /
PA_ND layouts, ragged per-batch lengths, paged KV cache with a randomly
permuted physical block order, and the shared-KV sparse decode rows
(aclnnFusedInferAttentionScoreV2 "Page attention scenario";
KvQuantSparseAttnSharedkv parameter table and constraints).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# Byte layout of one packed shared-KV row (KvQuantSparseAttnSharedkv,
# constraints: rope, nope and the per-tile scales concatenated, padded to 640).
ROW_BYTES = 640
ROPE_DIM = 64
NOPE_DIM = 448
TILE = 64
N_TILES = NOPE_DIM // TILE          # 7 scales
ROPE_OFF = 0                        # 64 bf16 = 128 bytes
NOPE_OFF = 128                      # 448 e4m3fn bytes
SCALE_OFF = 576                     # 7 fp32 = 28 bytes, then zero pad to 640
SPARSE_D = ROPE_DIM + NOPE_DIM      # 512: the logical row is [rope | nope]


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + r) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = (u[nan] >> np.uint32(16)).astype(np.uint16) | np.uint16(0x0040)
    return out


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's round to nearest even);
    return bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_f16_bits(rng.standard_normal(shape, dtype=np.float32))


# 0xFFFF is a NaN both as bfloat16 and as binary16: poison for rows that must
# never be read.
HALF_NAN_BITS = np.uint16(0xFFFF)


@dataclasses.dataclass
class DenseCase:
    """Inputs of one dense / paged attention call (query layout BSND or TND).

    q: [B, S1, Q_N, D] (BSND) or [T, Q_N, D] (TND).
    k, v: [B, S2, KV_N, D] (BSND), [T_kv, KV_N, D] (TND), or None when paged.
    k_pool, v_pool: [n_blocks, block_size, KV_N, D] (PA_ND) when paged, or
    [n_blocks, KV_N, block_size, D] when kv_layout is "BnNBsD".
    """
    name: str
    dtype: str                      # "bf16" | "fp32"
    layout: str                     # "BSND" | "TND"
    q: np.ndarray
    k: Optional[np.ndarray]
    v: Optional[np.ndarray]
    num_heads: int
    num_kv_heads: int
    scale: float
    sparse_mode: int = 0
    pre_tokens: int = 2147483647
    next_tokens: int = 2147483647
    alibi_slopes: Optional[np.ndarray] = None   # float32 [Q_N] (pseType 2)
    q_start_idx: int = 0
    kv_start_idx: int = 0
    actual_seq_lengths: Optional[list] = None
    actual_seq_lengths_kv: Optional[list] = None
    block_table: Optional[np.ndarray] = None    # int32 [B, max_blocks]
    block_size: int = 0
    k_pool: Optional[np.ndarray] = None
    v_pool: Optional[np.ndarray] = None
    kv_layout: str = "PA_ND"
    atten_mask: Optional[np.ndarray] = None     # uint8 / bool, modes 0 / 1; != 0 masks out
    pse_bias: Optional[np.ndarray] = None       # [B or 1, Q_N, Q_S or 1, KV_S'] (pseType 0), q's dtype
    learnable_sink: Optional[np.ndarray] = None  # bf16 bits [Q_N]
    # Fake-quantised key / value: k / v (or the pools) hold int8 or e4m3fn
    # (uint8) codes; dict(kind, kmode, vmode, kscale, vscale, koff, voff).
    kv_quant: Optional[dict] = None
    lse: bool = False
    seed: int = 0

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def batch(self) -> int:
        if self.layout == "TND":
            return len(self.actual_seq_lengths)
        return self.q.shape[0]


def with_random_mask(case: DenseCase, seed: int, *, p_masked=0.3, dims=3, per_batch=True,
                     dead_rows=(), mode=0) -> DenseCase:
    """The case with an explicit uint8 mask (1 = masked out), shape
    [B or 1, Q_S, KV_S'] (dims 3), [B or 1, 1, Q_S, KV_S'] (dims 4) or
    [Q_S, KV_S'] (dims 2), KV_S' = KV_S rounded up to a multiple of 4 (the
    padding columns are 1).  ``dead_rows`` are fully masked."""
    rng = rng_for(seed)
    B, S1 = case.q.shape[0], case.q.shape[1]
    S2 = case.block_size * case.block_table.shape[1] if case.paged else case.k.shape[1]
    S2p = -(-S2 // 4) * 4
    nb = B if (per_batch and dims != 2) else 1
    m = (rng.random((nb, S1, S2p)) < p_masked).astype(np.uint8)
    m[:, :, S2:] = 1
    for r in dead_rows:
        m[:, r, :] = 1
    if dims == 2:
        m = m[0]
    elif dims == 4:
        m = m[:, None]
    return dataclasses.replace(case, name=case.name + "_mask", atten_mask=m, sparse_mode=mode)


def with_random_bias(case: DenseCase, seed: int, *, per_batch=True, one_row=False,
                     std=1.0) -> DenseCase:
    """The case with a pseType 0 bias tensor of normal values (mean 0, ``std``)
    in the query's dtype, shape [B or 1, Q_N, Q_S or 1, KV_S'], KV_S' = KV_S
    rounded up to a multiple of 4 (the padding columns lie past every key)."""
    rng = rng_for(seed)
    B, S1 = case.q.shape[0], case.q.shape[1]
    S2 = case.block_size * case.block_table.shape[1] if case.paged else case.k.shape[1]
    S2p = -(-S2 // 4) * 4
    shape = (B if per_batch else 1, case.num_heads, 1 if one_row else S1, S2p)
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    bits = f32_to_bf16_bits(x) if case.dtype == "bf16" else x
    return dataclasses.replace(case, name=case.name + "_pse", pse_bias=bits)


def with_random_sink(case: DenseCase, seed: int, *, mean=0.0, std=2.0) -> DenseCase:
    """The case with a learnable sink: one bf16 logit per query head, normal
    values (``mean``, ``std``)."""
    rng = rng_for(seed)
    x = (mean + std * rng.standard_normal(case.num_heads)).astype(np.float32)
    return dataclasses.replace(case, name=case.name + "_sink", learnable_sink=f32_to_bf16_bits(x))


def with_kv_quant(case: DenseCase, seed: int, *, kind="int8", kmode=0, vmode=0, offsets=False,
                  per_tensor=False) -> DenseCase:
    """The case with its key / value replaced by fake-quantised codes of the
    same shape: int8 codes round(30 N(0,1)) clipped to [-128, 127], or e4m3fn
    codes of 8 N(0,1); rows that were NaN-poisoned get code 127 (int8) or
    0x7f (e4m3fn NaN).  Scales U(0.5, 1.5) / 32: per channel [KV_N, D] in
    bf16 bits (fp32 when the key is per channel and the value per token), one
    value (``per_tensor``), or per token fp32 [B, S2'] (S2' = S2 rounded up to
    a multiple of 4).  ``offsets`` (int8 only): N(0, 3) in the scale's
    layout and dtype."""
    import torch  # e4m3fn encoding of the fp8 codes uses torch's CPU cast
    rng = rng_for(seed)
    B = case.batch
    KVn, D = case.num_kv_heads, case.q.shape[-1]
    if case.layout == "TND":
        cum = [0] + [int(x) for x in case.actual_seq_lengths_kv]
        S2 = max(cum[i + 1] - cum[i] for i in range(B))
    else:
        S2 = case.block_size * case.block_table.shape[1] if case.paged else case.k.shape[1]
    S2p = max(4, -(-S2 // 4) * 4)

    def codes(orig):
        shape = orig.shape
        if kind == "int8":
            c = np.clip(np.rint(rng.standard_normal(shape) * 30.0), -128, 127).astype(np.int8)
        else:
            x = torch.from_numpy((rng.standard_normal(shape) * 8.0).astype(np.float32))
            c = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        if orig.dtype == np.uint16:
            bad = (orig & np.uint16(0x7FFF)) > np.uint16(0x7F80)
            c[bad] = 127 if kind == "int8" else 0x7F
        return c

    def table(mode, f32_chan):
        if mode == 1:
            sc = (rng.uniform(0.5, 1.5, (B, S2p)) / 32.0).astype(np.float32)
            off = rng.normal(0.0, 3.0, (B, S2p)).astype(np.float32) if offsets else None
            return sc, off
        shape = (1,) if per_tensor else (KVn, D)
        sc = (rng.uniform(0.5, 1.5, shape) / 32.0).astype(np.float32)
        off = rng.normal(0.0, 3.0, shape).astype(np.float32) if offsets else None
        if not f32_chan:
            sc = f32_to_bf16_bits(sc)
            off = None if off is None else f32_to_bf16_bits(off)
        return sc, off

    mixed = kmode == 0 and vmode == 1
    kscale, koff = table(kmode, mixed)
    vscale, voff = table(vmode, False)
    q = dict(kind=kind, kmode=kmode, vmode=vmode, kscale=kscale, vscale=vscale, koff=koff, voff=voff)
    if case.paged:
        return dataclasses.replace(case, name=case.name + "_" + kind, k_pool=codes(case.k_pool),
                                   v_pool=codes(case.v_pool), kv_quant=q)
    return dataclasses.replace(case, name=case.name + "_" + kind, k=codes(case.k), v=codes(case.v),
                               kv_quant=q)


def as_bnnbsd(case: DenseCase) -> DenseCase:
    """The same paged case with its pools stored BnNBsD [n_blocks, KV_N,
    block_size, D] (the values of every (block, slot, head) row unchanged)."""
    assert case.paged and case.kv_layout == "PA_ND"
    return dataclasses.replace(
        case, name=case.name + "_bnnbsd", kv_layout="BnNBsD",
        k_pool=np.ascontiguousarray(case.k_pool.transpose(0, 2, 1, 3)),
        v_pool=np.ascontiguousarray(case.v_pool.transpose(0, 2, 1, 3)))


def _draw(rng, shape, dtype):
    if dtype == "bf16":
        return normal_bf16(rng, shape)
    if dtype == "fp32":
        return rng.standard_normal(shape, dtype=np.float32)
    raise ValueError(dtype)


def _poison(arr, dtype):
    if dtype == "bf16":
        arr[...] = BF16_NAN
    else:
        arr[...] = np.float32(np.nan)


def dense_case(name, seed, *, B, S1, S2, Q_N, KV_N, D, dtype="bf16",
               scale=None, sparse_mode=0, pre_tokens=2147483647,
               next_tokens=2147483647, q_lens=None, kv_lens=None,
               alibi=False, q_start_idx=0, kv_start_idx=0, lse=False,
               poison_pad=False) -> DenseCase:
    """BSND query and key/value with optional ragged lengths.

    Rows past a batch's actual length are filled with N(0,1) values, or with
    NaN when ``poison_pad`` is set (they must never influence any output).
    """
    rng = rng_for(seed)
    q = _draw(rng, (B, S1, Q_N, D), dtype)
    k = _draw(rng, (B, S2, KV_N, D), dtype)
    v = _draw(rng, (B, S2, KV_N, D), dtype)
    if poison_pad:
        for b in range(B):
            if q_lens is not None:
                _poison(q[b, q_lens[b]:], dtype)
            if kv_lens is not None:
                _poison(k[b, kv_lens[b]:], dtype)
                _poison(v[b, kv_lens[b]:], dtype)
    slopes = alibi_slopes(Q_N) if alibi else None
    return DenseCase(
        name=name, dtype=dtype, layout="BSND", q=q, k=k, v=v,
        num_heads=Q_N, num_kv_heads=KV_N,
        scale=(1.0 / math.sqrt(D)) if scale is None else scale,
        sparse_mode=sparse_mode, pre_tokens=pre_tokens, next_tokens=next_tokens,
        alibi_slopes=slopes, q_start_idx=q_start_idx, kv_start_idx=kv_start_idx,
        actual_seq_lengths=None if q_lens is None else [int(x) for x in q_lens],
        actual_seq_lengths_kv=None if kv_lens is None else [int(x) for x in kv_lens],
        lse=lse, seed=seed)


def alibi_slopes(n_heads: int) -> np.ndarray:
    """Per-head slopes 2^(-8(h+1)/n) for h = 0..n-1 (the long-prefill workload)."""
    h = np.arange(n_heads, dtype=np.float64)
    return np.exp2(-8.0 * (h + 1.0) / n_heads).astype(np.float32)


def paginate(rng, k_rows_per_batch, v_rows_per_batch, *, block_size, dtype,
             poison_tail=False, extra_blocks=0):
    """Scatter per-batch K/V rows [L_b, KV_N, D] into PA_ND pools.

    Physical blocks are a random permutation of 0..n_blocks-1 dealt in order
    to the logical pages of batch 0, 1, ...; unused block-table entries are -1.
    ``extra_blocks`` adds never-referenced blocks filled with NaN.
    Returns (k_pool, v_pool, block_table).
    """
    lens = [r.shape[0] for r in k_rows_per_batch]
    kvn, d = k_rows_per_batch[0].shape[1:]
    pages = [-(-L // block_size) for L in lens]
    n_used = sum(pages)
    n_blocks = n_used + extra_blocks
    perm = rng.permutation(n_blocks).astype(np.int32)
    max_pages = max(1, max(pages))
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    np_dtype = np.uint16 if dtype == "bf16" else np.float32
    k_pool = np.empty((n_blocks, block_size, kvn, d), dtype=np_dtype)
    v_pool = np.empty_like(k_pool)
    _poison(k_pool, dtype)
    _poison(v_pool, dtype)
    cursor = 0
    for b, L in enumerate(lens):
        for p in range(pages[b]):
            blk = int(perm[cursor])
            cursor += 1
            table[b, p] = blk
            lo, hi = p * block_size, min(L, (p + 1) * block_size)
            k_pool[blk, : hi - lo] = k_rows_per_batch[b][lo:hi]
            v_pool[blk, : hi - lo] = v_rows_per_batch[b][lo:hi]
            if hi - lo < block_size and not poison_tail:
                k_pool[blk, hi - lo:] = _draw(rng, k_pool[blk, hi - lo:].shape, dtype)
                v_pool[blk, hi - lo:] = _draw(rng, v_pool[blk, hi - lo:].shape, dtype)
    return k_pool, v_pool, table


def paged_decode_case(name, seed, *, B, Q_N, KV_N, D, kv_lens, block_size,
                      dtype="bf16", scale=None, lse=True, poison_tail=False,
                      extra_blocks=0, S1=1, sparse_mode=0, keep_contiguous=False,
                      table_cols=None) -> DenseCase:
    """Paged KV cache (PA_ND pools + block table), query BSND [B, S1, Q_N, D]."""
    rng = rng_for(seed)
    q = _draw(rng, (B, S1, Q_N, D), dtype)
    k_rows = [_draw(rng, (int(L), KV_N, D), dtype) for L in kv_lens]
    v_rows = [_draw(rng, (int(L), KV_N, D), dtype) for L in kv_lens]
    k_pool, v_pool, table = paginate(rng, k_rows, v_rows, block_size=block_size,
                                     dtype=dtype, poison_tail=poison_tail,
                                     extra_blocks=extra_blocks)
    if table_cols is not None and table_cols > table.shape[1]:
        pad = np.full((B, table_cols - table.shape[1]), -1, dtype=np.int32)
        table = np.concatenate([table, pad], axis=1)
    k = v = None
    if keep_contiguous:
        S2 = max(1, max(int(L) for L in kv_lens))
        np_dtype = q.dtype
        k = np.zeros((B, S2, KV_N, D), dtype=np_dtype)
        v = np.zeros((B, S2, KV_N, D), dtype=np_dtype)
        for b, L in enumerate(kv_lens):
            k[b, :L] = k_rows[b]
            v[b, :L] = v_rows[b]
    return DenseCase(
        name=name, dtype=dtype, layout="BSND", q=q, k=k, v=v,
        num_heads=Q_N, num_kv_heads=KV_N,
        scale=(1.0 / math.sqrt(D)) if scale is None else scale,
        sparse_mode=sparse_mode,
        actual_seq_lengths_kv=[int(x) for x in kv_lens],
        block_table=table, block_size=block_size, k_pool=k_pool, v_pool=v_pool,
        lse=lse, seed=seed)


def tnd_case(name, seed, *, q_lens, kv_lens, Q_N, KV_N, D, dtype="bf16",
             scale=None, sparse_mode=0, lse=False, alibi=False) -> DenseCase:
    """TND query and key/value; actual lengths are cumulative (non-decreasing,
    last entry = T), as the FIA pages require for TND."""
    rng = rng_for(seed)
    Tq, Tk = int(sum(q_lens)), int(sum(kv_lens))
    q = _draw(rng, (Tq, Q_N, D), dtype)
    k = _draw(rng, (Tk, KV_N, D), dtype)
    v = _draw(rng, (Tk, KV_N, D), dtype)
    return DenseCase(
        name=name, dtype=dtype, layout="TND", q=q, k=k, v=v,
        num_heads=Q_N, num_kv_heads=KV_N,
        scale=(1.0 / math.sqrt(D)) if scale is None else scale,
        sparse_mode=sparse_mode,
        alibi_slopes=alibi_slopes(Q_N) if alibi else None,
        actual_seq_lengths=[int(x) for x in np.cumsum(q_lens)],
        actual_seq_lengths_kv=[int(x) for x in np.cumsum(kv_lens)],
        lse=lse, seed=seed)


# ---------------------------------------------------------------------------
# The five workloads.  Seeds are fixed per workload.
# ---------------------------------------------------------------------------
SEEDS = {"c1": 1001, "c2": 1002, "c3": 1003, "c4": 1004, "c5": 1005}


def c1_tiny_dense(seed=SEEDS["c1"]) -> DenseCase:
    """B=1, Q_N=KV_N=2, S1=S2=64, D=64, fp32 N(0,1), no mask, scale 1/8, LSE."""
    return dense_case("c1_tiny_dense_fp32", seed, B=1, S1=64, S2=64, Q_N=2,
                      KV_N=2, D=64, dtype="fp32", scale=1.0 / 8.0, lse=True)


def c2_lengths(seed=SEEDS["c2"], B=4, lo=512, hi=2048):
    return [int(x) for x in rng_for(seed + 7).integers(lo, hi + 1, size=B)]


def c2_causal_gqa(seed=SEEDS["c2"], poison_pad=False, lse=False) -> DenseCase:
    """B=4, Q_N=32, KV_N=8, D=128, bf16, S padded to 2048, per-batch lengths
    uniform in [512, 2048] for both query and key/value, right-down causal."""
    lens = c2_lengths(seed)
    return dense_case("c2_causal_gqa_prefill", seed, B=4, S1=2048, S2=2048,
                      Q_N=32, KV_N=8, D=128, sparse_mode=3, q_lens=lens,
                      kv_lens=lens, poison_pad=poison_pad, lse=lse)


def c3_lengths(seed=SEEDS["c3"], B=64, lo=1024, hi=8192):
    return [int(x) for x in rng_for(seed + 7).integers(lo, hi + 1, size=B)]


def c3_paged_decode(seed=SEEDS["c3"], poison_tail=False) -> DenseCase:
    """B=64, Q_S=1, Q_N=32, KV_N=8, D=128 bf16; pages of 128 tokens in a
    randomly permuted pool; KV lengths uniform in [1024, 8192]; LSE out."""
    return paged_decode_case("c3_paged_decode_gqa", seed, B=64, Q_N=32, KV_N=8,
                             D=128, kv_lens=c3_lengths(seed), block_size=128,
                             lse=True, poison_tail=poison_tail)


def c4_alibi_prefill(seed=SEEDS["c4"], S=8192, lse=False) -> DenseCase:
    """B=1, Q_N=KV_N=16, S1=S2=8192, D=128 bf16, ALiBi slopes 2^(-8(h+1)/16)
    with bias slope*(j-i), causal."""
    return dense_case("c4_long_causal_alibi_prefill", seed, B=1, S1=S, S2=S,
                      Q_N=16, KV_N=16, D=128, sparse_mode=3, alibi=True, lse=lse)


# ---------------------------------------------------------------------------
# Shared-KV sparse decode rows.
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class SparseCase:
    name: str
    q: np.ndarray                  # bf16 bits [B, S1, N1, 512], or [T1, N1, 512] with cu_seqlens_q
    ori_kv: np.ndarray             # uint8 [nb1, bs1, 1, 640]
    cmp_kv: np.ndarray             # uint8 [nb2, bs2, 1, 640]
    ori_block_table: np.ndarray    # int32 [B, >= ceil(max S2 / bs1)]
    cmp_block_table: np.ndarray    # int32 [B, >= ceil(floor(max S2 / ratio) / bs2)]
    cmp_sparse_indices: Optional[np.ndarray]  # int32 [B, S1, 1, K2] or [T1, 1, K2]; -1 = invalid; None: every compressed row
    seqused_kv: list
    sinks: np.ndarray              # float32 [N1]
    softmax_scale: float
    cmp_ratio: int = 4
    win_left: int = 127
    win_right: int = 0
    seed: int = 0
    cu_seqlens_q: Optional[list] = None   # TND: cumulative query-token counts [B + 1]


def pack_rows(rng, n_rows: int) -> np.ndarray:
    """Draw ``n_rows`` packed rows: rope bf16 N(0,1), nope N(0,1) quantised to
    e4m3fn per 64-wide tile with a power-of-two fp32 scale
    2^ceil(log2(amax/448)) so every scaled value is within the e4m3fn range."""
    import torch  # the e4m3fn rounding of the inputs uses torch's CPU cast

    out = np.zeros((n_rows, ROW_BYTES), dtype=np.uint8)
    if n_rows == 0:
        return out
    rope = normal_bf16(rng, (n_rows, ROPE_DIM))
    out[:, ROPE_OFF:ROPE_OFF + 2 * ROPE_DIM] = rope.view(np.uint8).reshape(n_rows, -1)
    nope = rng.standard_normal((n_rows, N_TILES, TILE), dtype=np.float32)
    amax = np.abs(nope).max(axis=2)
    amax = np.maximum(amax, np.float32(1e-30))
    scale = np.exp2(np.ceil(np.log2(amax.astype(np.float64) / 448.0))).astype(np.float32)
    scaled = (nope / scale[:, :, None]).astype(np.float32)
    codes = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    out[:, NOPE_OFF:NOPE_OFF + NOPE_DIM] = codes.reshape(n_rows, NOPE_DIM)
    out[:, SCALE_OFF:SCALE_OFF + 4 * N_TILES] = scale.view(np.uint8).reshape(n_rows, -1)
    return out


def _paged_pool_of_rows(rng, rows_per_batch, block_size, extra_blocks=0):
    """Place per-batch packed rows [L_b, 640] into a [n_blocks, bs, 1, 640]
    pool with randomly permuted physical blocks; returns (pool, table)."""
    pages = [-(-r.shape[0] // block_size) for r in rows_per_batch]
    n_blocks = sum(pages) + extra_blocks
    perm = rng.permutation(n_blocks).astype(np.int32)
    table = np.full((len(rows_per_batch), max(1, max(pages))), -1, dtype=np.int32)
    pool = np.zeros((n_blocks, block_size, 1, ROW_BYTES), dtype=np.uint8)
    cursor = 0
    for b, rows in enumerate(rows_per_batch):
        for p in range(pages[b]):
            blk = int(perm[cursor])
            cursor += 1
            table[b, p] = blk
            lo, hi = p * block_size, min(rows.shape[0], (p + 1) * block_size)
            pool[blk, : hi - lo, 0] = rows[lo:hi]
    return pool, table


def sparse_case(name, seed, *, B, N1, seqused_kv, K2=512, block_size1=128,
                block_size2=128, cmp_ratio=4, n_valid=None,
                materialise_all_ori=True, heavily_compressed=False, S1=1) -> SparseCase:
    """Shared-KV sparse attention inputs, S1 query tokens per batch entry
    (the last S1 positions of its KV sequence).

    ori rows: every logical row < L_b is materialised, or, when
    ``materialise_all_ori`` is False, only the last 128 (the rest are NaN);
    cmp rows: floor(L_b / cmp_ratio) rows per batch; per query token, top-K2
    indices drawn uniformly without replacement from [0, n_cmp), padded with
    -1 when fewer are valid (valid entries first).  ``heavily_compressed``: no indices
    (every compressed row is used), cmp_ratio 128."""
    if heavily_compressed:
        cmp_ratio = 128
    rng = rng_for(seed)
    q = normal_bf16(rng, (B, S1, N1, SPARSE_D))
    ori_rows, cmp_rows = [], []
    for L in seqused_kv:
        L = int(L)
        if materialise_all_ori:
            ori_rows.append(pack_rows(rng, L))
        else:
            # Only the last win_left+1 = 128 rows can be inside a decode
            # query's window; every other row is 0xFF bytes (NaN in all three
            # fields) so that reading one would poison the output.
            rows = np.full((L, ROW_BYTES), 0xFF, dtype=np.uint8)
            lo = max(0, L - 128 - (S1 - 1))
            rows[lo:] = pack_rows(rng, L - lo)
            ori_rows.append(rows)
        cmp_rows.append(pack_rows(rng, L // cmp_ratio))
    ori_kv, ori_bt = _paged_pool_of_rows(rng, ori_rows, block_size1)
    cmp_kv, cmp_bt = _paged_pool_of_rows(rng, [r if r.shape[0] else np.zeros((0, ROW_BYTES), np.uint8) for r in cmp_rows], block_size2)
    idx = np.full((B, S1, 1, K2), -1, dtype=np.int32)
    for b, L in enumerate(seqused_kv):
        n_cmp = int(L) // cmp_ratio
        nv = min(K2, n_cmp) if n_valid is None else min(n_valid, K2, n_cmp)
        for t in range(S1):
            if nv > 0:
                idx[b, t, 0, :nv] = rng.choice(n_cmp, size=nv, replace=False).astype(np.int32)
    if heavily_compressed:
        idx = None
    sinks = rng.standard_normal(N1, dtype=np.float32)
    return SparseCase(name=name, q=q, ori_kv=ori_kv, cmp_kv=cmp_kv,
                      ori_block_table=ori_bt, cmp_block_table=cmp_bt,
                      cmp_sparse_indices=idx, seqused_kv=[int(x) for x in seqused_kv],
                      sinks=sinks, softmax_scale=1.0 / math.sqrt(SPARSE_D),
                      cmp_ratio=cmp_ratio, seed=seed)


def sparse_tnd_case(name, seed, *, q_counts, **kw) -> SparseCase:
    """The TND form of :func:`sparse_case`: batch entry b has q_counts[b]
    query tokens (possibly 0), packed into T1 = sum(q_counts) rows, with
    cu_seqlens_q = [0, q_counts[0], q_counts[0] + q_counts[1], ...].

    Drawn as a BSND case with S1 = max(q_counts) whose entry b keeps its last
    q_counts[b] tokens: those sit at the same KV positions (the last
    q_counts[b] of the sequence) as the TND tokens of entry b."""
    s1max = max(1, max(q_counts))
    base = sparse_case(name, seed, S1=s1max, **kw)
    keep = [slice(s1max - c, s1max) for c in q_counts]
    q = np.concatenate([base.q[b, keep[b]] for b in range(len(q_counts))], axis=0)
    idx = None
    if base.cmp_sparse_indices is not None:
        idx = np.ascontiguousarray(np.concatenate(
            [base.cmp_sparse_indices[b, keep[b]] for b in range(len(q_counts))], axis=0))
    cu = [0]
    for c in q_counts:
        cu.append(cu[-1] + int(c))
    return dataclasses.replace(base, q=np.ascontiguousarray(q), cmp_sparse_indices=idx,
                               cu_seqlens_q=cu)


def c5_sparse_sharedkv(seed=SEEDS["c5"], materialise_all_ori=False) -> SparseCase:
    """B=16, Q_N=64, KV_N=1, D=512 (64 bf16 rope + 448 e4m3fn nope, one fp32
    scale per 64-wide tile), KV length 16384 per batch, window 127/0,
    compression ratio 4, top-512 compressed indices, fp32 sinks."""
    return sparse_case("c5_sparse_sharedkv_decode", seed, B=16, N1=64,
                       seqused_kv=[16384] * 16, K2=512,
                       materialise_all_ori=materialise_all_ori)


# ---------------------------------------------------------------------------
# sparse_flash_mla: the same shared-KV sparse attention over unquantised fp16 /
# bf16 rows of 512 values (sparse_flash_mla common and spec constraints).
# ---------------------------------------------------------------------------
SFMLA_MODES = {"SWA": 1, "CSA": 4, "HCA": 128}


@dataclasses.dataclass
class SfmlaCase:
    """Inputs of one sparse_flash_mla call.

    q: [B, S1, N1, 512] (BSND) or [T1, N1, 512] (TND, ``cu_seqlens_q`` set),
    bits of ``dtype``.  ori_kv / cmp_kv (same dtype), by ``kv_layout``:
    "PA_BBND" pools [n_blocks, block_size, 1, 512] addressed through
    ori_block_table / cmp_block_table; "BSND" [B, S2, 1, 512]; "TND" packed
    [T2, 1, 512] with entry b's rows starting at cu_seqlens_*_kv[b].
    cmp_kv is None in the SWA mode; cmp_sparse_indices (int32 [B, S1, 1, K2]
    or [T1, 1, K2], -1 = unused) only in the CSA mode.  sinks: None or
    float32 [N1]."""
    name: str
    dtype: str                       # "bf16" | "fp16"
    q: np.ndarray
    kv_layout: str                   # "PA_BBND" | "BSND" | "TND"
    ori_kv: np.ndarray
    cmp_kv: Optional[np.ndarray]
    ori_block_table: Optional[np.ndarray]
    cmp_block_table: Optional[np.ndarray]
    cu_seqlens_ori_kv: Optional[list]
    cu_seqlens_cmp_kv: Optional[list]
    cmp_sparse_indices: Optional[np.ndarray]
    seqused_kv: list
    sinks: Optional[np.ndarray]
    softmax_scale: float
    cmp_ratio: int = 4
    win_left: int = 127
    win_right: int = 0
    cu_seqlens_q: Optional[list] = None
    return_lse: bool = True
    seed: int = 0

    @property
    def mode(self) -> str:
        if self.cmp_kv is None:
            return "SWA"
        return "CSA" if self.cmp_sparse_indices is not None else "HCA"


def _paged_half_pool(rng, rows_per_batch, block_size, extra_blocks=0):
    """Place per-batch rows [L_b, 512] (uint16 bits) into a [n_blocks, bs, 1,
    512] pool with randomly permuted physical blocks; slots past a batch's
    rows hold NaN.  Unused table entries are -1.  Returns (pool, table)."""
    pages = [-(-r.shape[0] // block_size) for r in rows_per_batch]
    n_blocks = max(1, sum(pages) + extra_blocks)
    perm = rng.permutation(n_blocks).astype(np.int32)
    table = np.full((len(rows_per_batch), max(1, max(pages))), -1, dtype=np.int32)
    pool = np.full((n_blocks, block_size, 1, SPARSE_D), HALF_NAN_BITS, dtype=np.uint16)
    cursor = 0
    for b, rows in enumerate(rows_per_batch):
        for p in range(pages[b]):
            blk = int(perm[cursor])
            cursor += 1
            table[b, p] = blk
            lo, hi = p * block_size, min(rows.shape[0], (p + 1) * block_size)
            pool[blk, : hi - lo, 0] = rows[lo:hi]
    return pool, table


def _place_half_rows(rng, rows_per_batch, kv_layout, block_size, extra_blocks=0):
    """(kv, block_table, cu) of per-batch rows in the given KV layout."""
    if kv_layout == "PA_BBND":
        pool, table = _paged_half_pool(rng, rows_per_batch, block_size, extra_blocks)
        return pool, table, None
    if kv_layout == "BSND":
        S2 = max(1, max(r.shape[0] for r in rows_per_batch))
        kv = np.full((len(rows_per_batch), S2, 1, SPARSE_D), HALF_NAN_BITS, dtype=np.uint16)
        for b, r in enumerate(rows_per_batch):
            kv[b, : r.shape[0], 0] = r
        return kv, None, None
    if kv_layout == "TND":
        cu = [0]
        for r in rows_per_batch:
            cu.append(cu[-1] + r.shape[0])
        kv = np.concatenate(rows_per_batch, axis=0)[:, None, :] if cu[-1] else \
            np.zeros((0, 1, SPARSE_D), dtype=np.uint16)
        return np.ascontiguousarray(kv), None, cu
    raise ValueError(kv_layout)


def sfmla_case(name, seed, *, B, N1, seqused_kv, mode="CSA", K2=512, dtype="bf16",
               kv_layout="PA_BBND", block_size1=128, block_size2=128, S1=1, n_valid=None,
               sinks=True, lse=True, window_only_ori=False, extra_blocks=0) -> SfmlaCase:
    """sparse_flash_mla inputs with S1 query tokens per batch entry (the last
    S1 positions of its KV sequence).  Values N(0,1) rounded to ``dtype``.

    SWA: window rows of ori_kv only.  CSA (ratio 4): plus the top-K2 rows of
    cmp_kv, indices drawn uniformly without replacement from the
    floor(L / 4) compressed rows and padded with -1 (valid entries first).
    HCA (ratio 128): plus every compressed row.  ``window_only_ori``: only
    the rows a query window can reach are drawn, every other ori row is NaN
    (a read of one would poison the output)."""
    ratio = SFMLA_MODES[mode]
    rng = rng_for(seed)
    draw = normal_bf16 if dtype == "bf16" else normal_f16
    q = draw(rng, (B, S1, N1, SPARSE_D))
    ori_rows, cmp_rows = [], []
    for L in seqused_kv:
        L = int(L)
        if window_only_ori:
            rows = np.full((L, SPARSE_D), HALF_NAN_BITS, dtype=np.uint16)
            lo = max(0, L - 128 - (S1 - 1))
            rows[lo:] = draw(rng, (L - lo, SPARSE_D))
        else:
            rows = draw(rng, (L, SPARSE_D))
        ori_rows.append(rows)
        if mode != "SWA":
            cmp_rows.append(draw(rng, (L // ratio, SPARSE_D)))
    ori_kv, ori_bt, ori_cu = _place_half_rows(rng, ori_rows, kv_layout, block_size1, extra_blocks)
    cmp_kv = cmp_bt = cmp_cu = None
    if mode != "SWA":
        cmp_kv, cmp_bt, cmp_cu = _place_half_rows(rng, cmp_rows, kv_layout, block_size2, extra_blocks)
    idx = None
    if mode == "CSA":
        idx = np.full((B, S1, 1, K2), -1, dtype=np.int32)
        for b, L in enumerate(seqused_kv):
            n_cmp = int(L) // ratio
            nv = min(K2, n_cmp) if n_valid is None else min(n_valid, K2, n_cmp)
            for t in range(S1):
                if nv > 0:
                    idx[b, t, 0, :nv] = rng.choice(n_cmp, size=nv, replace=False).astype(np.int32)
    sk = rng.standard_normal(N1, dtype=np.float32) if sinks else None
    return SfmlaCase(name=name, dtype=dtype, q=q, kv_layout=kv_layout, ori_kv=ori_kv,
                     cmp_kv=cmp_kv, ori_block_table=ori_bt, cmp_block_table=cmp_bt,
                     cu_seqlens_ori_kv=ori_cu, cu_seqlens_cmp_kv=cmp_cu,
                     cmp_sparse_indices=idx, seqused_kv=[int(x) for x in seqused_kv],
                     sinks=sk, softmax_scale=1.0 / math.sqrt(SPARSE_D), cmp_ratio=ratio,
                     return_lse=lse, seed=seed)


def sfmla_tnd_case(name, seed, *, q_counts, **kw) -> SfmlaCase:
    """The TND-query form of :func:`sfmla_case` (as :func:`sparse_tnd_case`):
    entry b keeps its last q_counts[b] tokens, packed in entry order."""
    s1max = max(1, max(q_counts))
    base = sfmla_case(name, seed, S1=s1max, **kw)
    keep = [slice(s1max - c, s1max) for c in q_counts]
    q = np.concatenate([base.q[b, keep[b]] for b in range(len(q_counts))], axis=0)
    idx = None
    if base.cmp_sparse_indices is not None:
        idx = np.ascontiguousarray(np.concatenate(
            [base.cmp_sparse_indices[b, keep[b]] for b in range(len(q_counts))], axis=0))
    cu = [0]
    for c in q_counts:
        cu.append(cu[-1] + int(c))
    return dataclasses.replace(base, q=np.ascontiguousarray(q), cmp_sparse_indices=idx,
                               cu_seqlens_q=cu)


def sfmla_decode_bf16(seed=SEEDS["c5"] + 100) -> SfmlaCase:
    """The shared-KV sparse decode shape with unquantised bf16 rows: B=16,
    N1=64, D=512, KV length 16384, window 127/0, ratio 4, top-512 indices,
    PA_BBND pools of block 128, fp32 sinks, LSE."""
    return sfmla_case("sfmla_csa_decode_bf16", seed, B=16, N1=64, seqused_kv=[16384] * 16,
                      K2=512, window_only_ori=True)


# ---------------------------------------------------------------------------
# The timed variants of the workloads above (each with its own seed), shared
# by the benchmark and the full-size parity tests.
# ---------------------------------------------------------------------------
SEEDS_SPARSE_MODES = 1006


def mask_prefill() -> DenseCase:
    """Causal GQA prefill shapes with an explicit uint8 mask [4, 2048, 2048],
    Bernoulli(0.1) masked, mode 0."""
    return with_random_mask(c2_causal_gqa(), 41, p_masked=0.1, mode=0)


def bias_prefill() -> DenseCase:
    """Causal GQA prefill with a bf16 pse_shift bias [1, 32, 2048, 2048]."""
    return with_random_bias(c2_causal_gqa(), 42, per_batch=False)


def sink_prefill() -> DenseCase:
    """Causal GQA prefill with a bf16 learnable sink [32]."""
    return with_random_sink(c2_causal_gqa(), 43)


Q8_DECODES = {
    # name: (code kind, table mode (0 per channel, 1 per token), offsets, BnNBsD pools)
    "q8_int8": ("int8", 1, True, False),
    "q8_fp8": ("fp8", 0, False, False),
    "q8_int8_bnnbsd": ("int8", 1, True, True),
}


def q8_decode(name) -> DenseCase:
    """The paged GQA decode with a fake-quantised KV cache (Q8_DECODES)."""
    kind, mode, off, bn = Q8_DECODES[name]
    case = with_kv_quant(c3_paged_decode(), 1007, kind=kind, kmode=mode, vmode=mode, offsets=off)
    return as_bnnbsd(case) if bn else case


def sparse_hca_decode() -> SparseCase:
    """Shared-KV sparse decode, heavily compressed: B=16, N1=64, KV length
    16384, window 128 + every row of the ratio-128 compressed KV."""
    return sparse_case("hca", SEEDS_SPARSE_MODES, B=16, N1=64, seqused_kv=[16384] * 16,
                       materialise_all_ori=False, heavily_compressed=True)


def sparse_two_tokens() -> SparseCase:
    """Shared-KV sparse attention with 2 query tokens per batch entry."""
    return sparse_case("s1_2", SEEDS_SPARSE_MODES + 1, B=16, N1=64, seqused_kv=[16384] * 16, K2=512,
                       S1=2, materialise_all_ori=False)


def sparse_tnd_counts():
    return [int(x) for x in rng_for(SEEDS_SPARSE_MODES + 2).integers(1, 5, size=16)]


def sparse_tnd_ragged() -> SparseCase:
    """Shared-KV sparse attention, TND queries with 1-4 tokens per entry."""
    return sparse_tnd_case("tnd", SEEDS_SPARSE_MODES + 3, q_counts=sparse_tnd_counts(), B=16, N1=64,
                           seqused_kv=[16384] * 16, K2=512, materialise_all_ori=False)
