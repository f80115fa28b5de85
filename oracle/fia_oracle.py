"""Plain float64 CPU oracle for fused inference attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  It shares no code with the HIP
library: it decodes the raw input bits itself, gathers paged rows itself and
evaluates attention from its definition with materialised scores (no tiling,
no online recurrence, no split/merge).

What it computes, and where each step is stated on the pages:

* Attention(Q,K,V) = softmax(Q K^T * scale + bias) V, row-wise softmax
  (aclnnFusedInferAttentionScoreV5 / V2, "Formula"); the ALiBi bias is added
  after scaling (aclnnFusedInferAttentionScoreV4, "Formula", FullMask term).
* pseType 0 bias tensor (V5 PSE parameter group): shape [B or 1, Q_N,
  P_S1, >= KV_S] with P_S1 >= Q_S or P_S1 = 1, in the query's dtype.
  Reading (no formula places it): like the full-mask ALiBi term it is added
  to the scaled scores, element [b or 0][h][i or 0][j] to score (i, j).
* Fake-quantised key / value (V5 quantisation parameter group, fake-quant
  scenario): int8 or e4m3fn codes c with per-channel scales / offsets
  ([KV_N, D], or one value) or per-token ones ([B, S2], index = position
  inside the batch's key sequence, shared by the KV heads).  Reading (the
  dequantisation formula is not legible on the pages): value = scale *
  (c + offset).
* Learnable sink (V5 LearnableSink group: [Q_N], the query's dtype).  Same
  reading as the shared-KV sink: one extra logit per head with a zero value
  vector, not multiplied by the scale; the LSE includes it, so a live row
  with no visible key (or a batch with Lk = 0) gives out 0 and LSE = sink.
* GQA: Q_N a multiple of KV_N (V2, numKeyValueHeads restrictions).  Reading:
  query head h uses KV head floor(h / (Q_N / KV_N)).
* Per-batch actual lengths, broadcast rule (length-1 array -> every batch;
  length >= B -> first B entries) (V2, actualSeqLengths / actualSeqLengthsKv);
  TND lengths are cumulative (V5, ActualSeqLen parameter group).
* Paged KV: row j of batch b lives at pool[blockTable[b][j // bs], j % bs]
  (V2 / V5, page attention scenario); with the BnNBsD pool order
  [n_blocks, KV_N, bs, D] (V5 paged-attention KV cache layouts) the row of
  KV head n is pool[blockTable[b][j // bs], n, j % bs].
* Mask modes (V5 Attention Mask parameter group; V2 sparseMode rules), with
  delta = Lk - Lq.  Reading (the mode table itself is not legible):
  0 -> all keys j < Lk (with an explicit atten_mask tensor, modes 0 and 1:
  the keys j < Lk whose mask element [b or 0][i][j] is 0; 1 = masked out),
  2 -> j <= i (left-up causal),
  3 -> j <= i + delta (right-down causal, the "lower triangle anchored at the
  right vertex" of KvQuantSparseAttnSharedkv cmp_mask_mode),
  4 -> i + delta - pre <= j <= i + delta + next (band).
* LSE = max + ln(sum exp(s - max)), natural log (V2, softmaxLse restrictions
  describing the ring-attention composition; KvQuantSparseAttnSharedkv
  softmax_lse description).
* Empty key set (S2 = 0, empty K/V) -> output 0 and LSE +inf
  (V4 "empty tensor" rules; V2 null-input processing).  Reading: the same
  holds for a query row whose visible key set is empty (invalid-row
  correction, V2 innerPrecise restrictions) and for padded query rows
  i >= Lq; "inf" is taken as +inf.
* sparse_flash_mla (function description, common / spec constraints): the
  same row sets over unquantised fp16 / bf16 rows of 512 values, in PA_BBND
  pools (addressed like PA_ND), BSND or packed TND KV, with an optional
  softmax_lse output (shared-KV LSE shape, N2 = 1).
* Shared-KV sparse decode (KvQuantSparseAttnSharedkv formula and
  constraints; sparse_flash_mla CSA mode): K~ = V~ = [window rows of ori_kv ;
  top-k selected rows of cmp_kv], each packed row = bf16 rope(64) |
  e4m3fn nope(448) | per-64-tile scales.  Readings: the scales are fp32;
  the logical 512-vector is [rope | nope] in packing order; the per-head sink
  is one extra logit with a zero value vector, not multiplied by the softmax
  scale; an index entry is used iff 0 <= c < floor(Lk / cmp_ratio).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

POS_INF = float("inf")


# ---------------------------------------------------------------------------
# Exact decoders of the input bit patterns.
# ---------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly: the 16 bits are the
    upper half of an IEEE binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point E4M3 ("fn": finite, no infinities) -> float64.

    sign = b7, exponent = b6..b3 (bias 7), mantissa = b2..b0.
    exponent 0 -> subnormal (m/8) * 2^-6; exponent 15 with mantissa 7 -> NaN;
    otherwise (1 + m/8) * 2^(e-7).  Computed in closed form per code.
    """
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    sign = np.where(s == 1, -1.0, 1.0)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def decode_fp16(bits: np.ndarray) -> np.ndarray:
    """IEEE 754 binary16 bit patterns (uint16) -> float64, in closed form.

    sign = b15, exponent = b14..b10 (bias 15), mantissa = b9..b0.
    exponent 0 -> subnormal (m/1024) * 2^-14; exponent 31 -> +-inf for
    m = 0, NaN otherwise; else (1 + m/1024) * 2^(e-15)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = (b >> 15) & 1
    e = (b >> 10) & 31
    m = b & 1023
    sign = np.where(s == 1, -1.0, 1.0)
    normal = (1.0 + m / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = (m / 1024.0) * 2.0 ** -14
    val = sign * np.where(e == 0, sub, normal)
    val = np.where(e == 31, np.where(m == 0, sign * np.inf, np.nan), val)
    return val


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return decode_bf16(x)
    if dtype == "fp16":
        return decode_fp16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Lengths, visibility, bias.
# ---------------------------------------------------------------------------
def per_batch_lengths(arr: Optional[Sequence[int]], B: int, default: int) -> list:
    """V2 actualSeqLengths rule: absent -> the tensor's S for every batch;
    length 1 -> that value for every batch; length >= B -> first B entries."""
    if arr is None:
        return [int(default)] * B
    arr = [int(x) for x in arr]
    if len(arr) == 1:
        return arr * B
    if len(arr) >= B:
        return arr[:B]
    raise ValueError("actual length array must have length 1 or >= B")


def visible(mode: int, Lq: int, Lk: int, pre: int, nxt: int) -> np.ndarray:
    """Boolean [Lq, Lk]: which key j each query row i may attend to."""
    i = np.arange(Lq, dtype=np.int64)[:, None]
    j = np.arange(Lk, dtype=np.int64)[None, :]
    delta = Lk - Lq
    if mode == 0:
        return np.ones((Lq, Lk), dtype=bool)
    if mode == 2:
        return j <= i
    if mode == 3:
        return j <= i + delta
    if mode == 4:
        return (j >= i + delta - pre) & (j <= i + delta + nxt)
    raise ValueError(f"mask mode {mode} has no analytic definition here")


def softmax_rows(s: np.ndarray, mask: np.ndarray, v: np.ndarray,
                 extra_logit: Optional[float] = None):
    """Row softmax of scores ``s`` [n, L] restricted to ``mask``, times v [L, Dv].

    Returns (out [n, Dv], lse [n]).  Rows with no visible key (and no extra
    logit) give out = 0, lse = +inf.  ``extra_logit`` adds one more term to the
    normaliser with a zero value vector (the sink reading); the returned lse
    then includes it.
    """
    n = s.shape[0]
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, POS_INF, dtype=np.float64)
    masked = np.where(mask, s, -np.inf)
    row_has = mask.any(axis=1)
    m = masked.max(axis=1, initial=-np.inf)
    if extra_logit is not None:
        m = np.maximum(m, extra_logit)
        row_has = np.ones(n, dtype=bool)
    rows = np.nonzero(row_has)[0]
    if rows.size == 0:
        return out, lse
    mr = m[rows][:, None]
    p = np.where(mask[rows], np.exp(masked[rows] - mr), 0.0)
    l = p.sum(axis=1)
    if extra_logit is not None:
        l = l + np.exp(extra_logit - m[rows])
    out[rows] = (p @ v) / l[:, None]
    lse[rows] = m[rows] + np.log(l)
    return out, lse


# ---------------------------------------------------------------------------
# Dense / paged fused inference attention.
# ---------------------------------------------------------------------------
def gather_paged(pool: np.ndarray, table_row: np.ndarray, L: int, bs: int,
                 kv_layout: str = "PA_ND") -> np.ndarray:
    """Rows 0..L-1 of one batch, [L, KV_N, D], from a PA_ND pool
    [n_blk, bs, KV_N, D] or a BnNBsD pool [n_blk, KV_N, bs, D]."""
    j = np.arange(L)
    blocks = np.asarray(table_row, dtype=np.int64)[j // bs]
    if kv_layout == "BnNBsD":
        return pool[blocks, :, j % bs]
    if kv_layout != "PA_ND":
        raise ValueError(kv_layout)
    return pool[blocks, j % bs]


def decode_codes(c: np.ndarray, kind: str) -> np.ndarray:
    """int8 or e4m3fn (uint8) codes -> float64, exactly."""
    if kind == "int8":
        return np.asarray(c, dtype=np.int8).astype(np.float64)
    if kind == "fp8":
        return decode_e4m3fn(np.asarray(c, dtype=np.uint8))
    raise ValueError(kind)


def _table_f64(x) -> np.ndarray:
    """Scale / offset table: bf16 bit patterns (uint16) or fp32 values."""
    x = np.asarray(x)
    return decode_bf16(x) if x.dtype == np.uint16 else x.astype(np.float64)


def dequant_rows(codes: np.ndarray, kind: str, mode: int, scale, offset, b: int) -> np.ndarray:
    """Key / value codes [Lk, KV_N, D] of batch b -> scale * (code + offset),
    float64.  mode 1: per token, scale[b][j] for the row at position j; mode
    0: per channel scale[n][d], or the single value of a one-element table."""
    c = decode_codes(codes, kind)
    Lk, N, D = c.shape
    sc = _table_f64(scale)
    of = None if offset is None else _table_f64(offset)
    if mode == 1:
        sc2 = sc.reshape(-1, sc.shape[-1])
        s = sc2[b, :Lk][:, None, None]
        o = 0.0 if of is None else of.reshape(-1, of.shape[-1])[b, :Lk][:, None, None]
    elif sc.size == 1:
        s = float(sc.reshape(()))
        o = 0.0 if of is None else float(of.reshape(()))
    else:
        s = sc.reshape(N, D)[None]
        o = 0.0 if of is None else of.reshape(N, D)[None]
    return s * (c + o)


def fia(q, k, v, *, dtype: str, layout: str, num_heads: int, num_kv_heads: int,
        scale: float, sparse_mode: int = 0, pre_tokens: int = 2147483647,
        next_tokens: int = 2147483647, alibi_slopes=None, q_start_idx: int = 0,
        kv_start_idx: int = 0, actual_seq_lengths=None, actual_seq_lengths_kv=None,
        block_table=None, block_size: int = 0, k_pool=None, v_pool=None,
        kv_layout: str = "PA_ND", atten_mask=None, pse_shift=None, learnable_sink=None,
        kv_quant=None, batches: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None,
        rows: Optional[Sequence[int]] = None, row_chunk: int = 1024):
    """Fused inference attention, float64.

    q: BSND [B, S1, Q_N, D] or TND [T, Q_N, D] (raw bits or floats per
    ``dtype``); k, v: [B, S2, KV_N, D] / [T_kv, KV_N, D]; or k_pool, v_pool
    PA_ND [n_blk, bs, KV_N, D] (``kv_layout`` "BnNBsD": [n_blk, KV_N, bs, D])
    with ``block_table`` [B, >= max pages].  ``pse_shift``: pseType 0 bias
    [B or 1, Q_N, Q_S or 1, >= KV_S], encoded like q (``dtype``).
    ``learnable_sink``: [Q_N] logits, encoded like q.  ``kv_quant``: dict(kind,
    kmode, vmode, kscale, vscale, koff, voff) when k / v hold codes.

    Returns (out, lse) with out in the query layout (float64) and lse
    [B, Q_N, S1] (BSND) or [T, Q_N] (TND).  ``batches``/``heads``/``rows``
    restrict the computation to a subset (other entries are left NaN).
    """
    if num_heads % num_kv_heads != 0:
        raise ValueError("Q_N must be a multiple of KV_N")
    G = num_heads // num_kv_heads
    tnd = layout == "TND"
    paged = block_table is not None
    if tnd:
        B = len(actual_seq_lengths)
        q_off = [0] + [int(x) for x in actual_seq_lengths]
        kv_cum = [int(x) for x in actual_seq_lengths_kv]
        kv_off = [0] + kv_cum
        q_len = [q_off[b + 1] - q_off[b] for b in range(B)]
        kv_len = [kv_off[b + 1] - kv_off[b] for b in range(B)]
        S1 = max(q_len) if B else 0
        out = np.full(q.shape, np.nan, dtype=np.float64)
        lse = np.full((q.shape[0], num_heads), np.nan, dtype=np.float64)
    else:
        B, S1 = q.shape[0], q.shape[1]
        S2 = block_size * block_table.shape[1] if paged else k.shape[1]
        q_len = per_batch_lengths(actual_seq_lengths, B, S1)
        kv_len = per_batch_lengths(actual_seq_lengths_kv, B, S2 if not paged else 0)
        out = np.full(q.shape, np.nan, dtype=np.float64)
        lse = np.full((B, num_heads, S1), np.nan, dtype=np.float64)
    D = q.shape[-1]
    Dv = (v_pool if paged else v).shape[-1]
    slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, np.float64)
    sink = None if learnable_sink is None else to_f64(learnable_sink, dtype)
    # Empty key / value tensors are the empty-tensor case: 0 and +inf everywhere.
    kv_tensor_empty = np.asarray(k_pool if paged else k).size == 0

    for b in (range(B) if batches is None else batches):
        Lq, Lk = q_len[b], kv_len[b]
        if paged:
            kr = gather_paged(k_pool, block_table[b], Lk, block_size, kv_layout)
            vr = gather_paged(v_pool, block_table[b], Lk, block_size, kv_layout)
        elif tnd:
            kr = k[kv_off[b]:kv_off[b + 1]]
            vr = v[kv_off[b]:kv_off[b + 1]]
        else:
            kr = k[b, :Lk]
            vr = v[b, :Lk]
        if kv_quant is None:
            kb, vb = to_f64(kr, dtype), to_f64(vr, dtype)
        else:
            aq = kv_quant
            kb = dequant_rows(kr, aq["kind"], aq["kmode"], aq["kscale"], aq["koff"], b)
            vb = dequant_rows(vr, aq["kind"], aq["vmode"], aq["vscale"], aq["voff"], b)
        qb = to_f64(q[q_off[b]:q_off[b + 1]] if tnd else q[b], dtype)   # [S, Q_N, D]
        S_rows = qb.shape[0]
        want = range(S_rows) if rows is None else [r for r in rows if r < S_rows]
        want = np.asarray(list(want), dtype=np.int64)
        for h in (range(num_heads) if heads is None else heads):
            g = h // G
            K, V = kb[:, g, :], vb[:, g, :]
            for c0 in range(0, want.size, row_chunk):
                idx = want[c0:c0 + row_chunk]
                o_blk = np.zeros((idx.size, Dv))
                l_blk = np.full(idx.size, POS_INF)
                live = idx[idx < Lq]          # padded rows i >= Lq stay 0 / +inf
                if live.size and (Lk > 0 or (sink is not None and not kv_tensor_empty)):
                    s = scale * (qb[live, h, :] @ K.T)
                    if slopes is not None:
                        jpos = (kv_start_idx + np.arange(Lk))[None, :]
                        ipos = (q_start_idx + live)[:, None]
                        s = s + slopes[h] * (jpos - ipos)
                    if pse_shift is not None:
                        pb = to_f64(np.asarray(pse_shift)[b if pse_shift.shape[0] > 1 else 0, h], dtype)
                        s = s + (pb[np.zeros_like(live)] if pb.shape[0] == 1 else pb[live])[:, :Lk]
                    if atten_mask is not None and sparse_mode in (0, 1):
                        m = np.asarray(atten_mask)
                        m2 = m.reshape(m.shape[-2], m.shape[-1]) if m.ndim == 2 else \
                            m.reshape(m.shape[0], m.shape[-2], m.shape[-1])[b if m.shape[0] > 1 else 0]
                        vis = (m2[:Lq, :Lk] == 0)[live]
                    else:
                        vis = visible(sparse_mode, Lq, Lk, pre_tokens, next_tokens)[live]
                    o_live, l_live = softmax_rows(s, vis, V, None if sink is None else float(sink[h]))
                    pos = np.searchsorted(idx, live)
                    o_blk[pos] = o_live
                    l_blk[pos] = l_live
                if tnd:
                    out[q_off[b] + idx, h, :] = o_blk
                    lse[q_off[b] + idx, h] = l_blk
                else:
                    out[b, idx, h, :] = o_blk
                    lse[b, h, idx] = l_blk
    return out, lse


def fia_case(case, **kw):
    """Run :func:`fia` on a ``workloads.DenseCase``-like object."""
    return fia(case.q, case.k, case.v, dtype=case.dtype, layout=case.layout,
               num_heads=case.num_heads, num_kv_heads=case.num_kv_heads,
               scale=case.scale, sparse_mode=case.sparse_mode,
               pre_tokens=case.pre_tokens, next_tokens=case.next_tokens,
               alibi_slopes=case.alibi_slopes, q_start_idx=case.q_start_idx,
               kv_start_idx=case.kv_start_idx,
               actual_seq_lengths=case.actual_seq_lengths,
               actual_seq_lengths_kv=case.actual_seq_lengths_kv,
               block_table=case.block_table, block_size=case.block_size,
               k_pool=case.k_pool, v_pool=case.v_pool,
               kv_layout=getattr(case, "kv_layout", "PA_ND"),
               atten_mask=getattr(case, "atten_mask", None),
               pse_shift=getattr(case, "pse_bias", None),
               learnable_sink=getattr(case, "learnable_sink", None),
               kv_quant=getattr(case, "kv_quant", None), **kw)


# ---------------------------------------------------------------------------
# Shared-KV sparse decode (S1 = 1).
# ---------------------------------------------------------------------------
ROW_BYTES = 640
ROPE, NOPE, TILE = 64, 448, 64


def decode_packed_row(row: np.ndarray) -> np.ndarray:
    """One 640-byte row -> float64 [512] = [rope(64) | nope(448)].

    bytes 0..127: 64 bf16 rope values; 128..575: 448 e4m3fn codes;
    576..603: 7 fp32 scales, nope[d] = e4m3(code_d) * scale[d // 64]."""
    row = np.asarray(row, dtype=np.uint8)
    rope = decode_bf16(row[0:128].view(np.uint16))
    codes = decode_e4m3fn(row[128:576])
    scales = row[576:604].view(np.float32).astype(np.float64)
    nope = codes * np.repeat(scales, TILE)
    return np.concatenate([rope, nope])


def sparse_rows(Lk: int, S1: int, t: int, idx_row, *, cmp_ratio: int,
                win_left: int, win_right: int):
    """The logical rows a query token attends to: window rows of ori_kv and
    selected rows of cmp_kv.

    Window (ori_mask_mode 4, band): p = Lk - S1 + t (the S1 query tokens
    are the last S1 positions of the KV sequence), rows max(0, p - win_left)
    .. min(Lk - 1, p + win_right).
    Compressed (cmp_mask_mode 3, right-down causal on the S1 x Lc score
    matrix of the Lc = floor(Lk / ratio) compressed rows): token t sees the
    compressed rows c <= t + Lc - S1, i.e. c < Lc - (S1 - 1 - t).  Reading:
    the mode-3 rule of the dense operator applied to the compressed sequence
    as the key axis.  Compressed-sparse mode: the entries c of the index row
    that are >= 0 and visible, in index order; heavily compressed mode
    (sparse_flash_mla HCA, no index row): every visible compressed row.
    """
    p = Lk - S1 + t
    lo, hi = max(0, p - win_left), min(Lk - 1, p + win_right)
    window = list(range(lo, hi + 1)) if hi >= lo else []
    n_cmp = max(0, Lk // cmp_ratio - (S1 - 1 - t))
    if idx_row is None:
        comp = list(range(n_cmp))
    else:
        comp = [int(c) for c in idx_row if 0 <= int(c) < n_cmp]
    return window, comp


def sparse_sharedkv(case, *, batches=None):
    """Shared-KV sparse attention output, float64 [B, S1, N1, 512] (BSND) or
    [T1, N1, 512] (TND: ``case.cu_seqlens_q`` set).

    For each (b, query token t, head h): X = rows (window ++ compressed) of
    :func:`sparse_rows`, scores
    s_r = softmax_scale * (q_h . x_r), an extra sink logit sigma_h with a zero
    value vector, out = sum_r exp(s_r - m) x_r / (exp(sigma_h - m) + sum_r
    exp(s_r - m)).  K~ = V~ = X.

    TND (SharedKV layout_q TND, cu_seqlens_q): entry b owns packed rows
    cu[b] .. cu[b + 1] - 1, its S1 is their count and its token t is row
    cu[b] + t.  Reading: a packed row outside every entry (possible only with
    inconsistent counts) is 0.
    """
    q = case.q
    Dq = q.shape[-1]
    N1 = q.shape[-2]
    bs1 = case.ori_kv.shape[1]
    bs2 = case.cmp_kv.shape[1]
    sinks = np.asarray(case.sinks, dtype=np.float32).astype(np.float64)
    B = len(case.seqused_kv)
    if case.cu_seqlens_q is None:
        S1 = q.shape[1]
        out = np.full((B, S1, N1, Dq), np.nan)
        rows_of = lambda b: [(t, S1, (b, t)) for t in range(S1)]
        idx_of = lambda key: case.cmp_sparse_indices[key[0], key[1], 0]
    else:
        cu = [int(x) for x in case.cu_seqlens_q]
        out = np.zeros((q.shape[0], N1, Dq))
        rows_of = lambda b: [(t, cu[b + 1] - cu[b], cu[b] + t) for t in range(cu[b + 1] - cu[b])]
        idx_of = lambda key: case.cmp_sparse_indices[key, 0]
    for b in (range(B) if batches is None else batches):
        Lk = int(case.seqused_kv[b])
        for t, S1b, key in rows_of(b):
            idx_row = None if case.cmp_sparse_indices is None else idx_of(key)
            win, comp = sparse_rows(Lk, S1b, t, idx_row,
                                    cmp_ratio=case.cmp_ratio, win_left=case.win_left,
                                    win_right=case.win_right)
            X = []
            for j in win:
                X.append(decode_packed_row(case.ori_kv[case.ori_block_table[b, j // bs1], j % bs1, 0]))
            for c in comp:
                X.append(decode_packed_row(case.cmp_kv[case.cmp_block_table[b, c // bs2], c % bs2, 0]))
            X = np.stack(X) if X else np.zeros((0, Dq))
            qb = decode_bf16(q[key])                            # [N1, 512]
            s = case.softmax_scale * (qb @ X.T)                 # [N1, R]
            for h in range(N1):
                o, _ = softmax_rows(s[h:h + 1], np.ones((1, X.shape[0]), bool), X,
                                    extra_logit=float(sinks[h]))
                out[key][h] = o[0]
    return out


# ---------------------------------------------------------------------------
# sparse_flash_mla: shared-KV sparse attention over unquantised rows.
# ---------------------------------------------------------------------------
def sparse_flash_mla(case):
    """sparse_flash_mla (SWA / CSA / HCA modes) over fp16 / bf16 rows of 512,
    float64.  Returns (out, lse).

    Page: sparse_flash_mla, function description (O = softmax(Q K~^T *
    softmax_scale) V~ with K~ = V~ the window part of ori_kv and the
    compressed part of cmp_kv), common constraints (q, ori_kv and cmp_kv share
    one dtype, fp16 or bf16; layouts BSND / TND for q and BSND / TND /
    PA_BBND for the KV) and spec constraints (D 512, KV_N 1, window 127 / 0).
    The row set of every query token is :func:`sparse_rows` (the same rules as
    the shared-KV operator): SWA uses no compressed rows, CSA the valid
    visible entries of the index row, HCA every visible compressed row.

    Rows: "PA_BBND" pools are addressed through the block tables like the
    PA_ND pools (row r of batch b at pool[table[b][r // bs], r % bs]);
    "BSND" row r of batch b is kv[b, r]; "TND" row r of batch b is
    kv[cu[b] + r] with cu = cu_seqlens_ori_kv / cu_seqlens_cmp_kv.

    LSE (softmax_lse output, fp32 log-sum-exp, natural log) in the shared-KV
    shape with N2 = 1: [B, 1, S1, N1] (BSND) or [1, T1, N1] (TND).  Readings:
    with ``case.sinks`` (optional here) the sink is one extra logit with a
    zero value vector, as for the shared-KV operator, and the LSE includes
    it; a query token with no row and no sink gives 0 and +inf; a packed TND
    row outside every entry is 0 / +inf.
    """
    dec = decode_bf16 if case.dtype == "bf16" else decode_fp16
    q = case.q
    N1, Dq = q.shape[-2], q.shape[-1]
    B = len(case.seqused_kv)
    sinks = None if case.sinks is None else np.asarray(case.sinks, np.float32).astype(np.float64)

    def row(which, b, r):
        kv = case.ori_kv if which == 0 else case.cmp_kv
        if case.kv_layout == "PA_BBND":
            table = case.ori_block_table if which == 0 else case.cmp_block_table
            bs = kv.shape[1]
            return kv[int(table[b, r // bs]), r % bs, 0]
        if case.kv_layout == "BSND":
            return kv[b, r, 0]
        if case.kv_layout == "TND":
            cu = case.cu_seqlens_ori_kv if which == 0 else case.cu_seqlens_cmp_kv
            return kv[int(cu[b]) + r, 0]
        raise ValueError(case.kv_layout)

    if case.cu_seqlens_q is None:
        S1 = q.shape[1]
        out = np.full((B, S1, N1, Dq), np.nan)
        lse = np.full((B, 1, S1, N1), np.nan)
        rows_of = lambda b: [(t, S1, (b, t)) for t in range(S1)]
        idx_of = lambda key: case.cmp_sparse_indices[key[0], key[1], 0]
        lse_at = lambda key: (key[0], 0, key[1])
    else:
        cu = [int(x) for x in case.cu_seqlens_q]
        out = np.zeros((q.shape[0], N1, Dq))
        lse = np.full((1, q.shape[0], N1), POS_INF)
        rows_of = lambda b: [(t, cu[b + 1] - cu[b], cu[b] + t) for t in range(cu[b + 1] - cu[b])]
        idx_of = lambda key: case.cmp_sparse_indices[key, 0]
        lse_at = lambda key: (0, key)
    for b in range(B):
        Lk = int(case.seqused_kv[b])
        for t, S1b, key in rows_of(b):
            idx_row = None if case.cmp_sparse_indices is None else idx_of(key)
            win, comp = sparse_rows(Lk, S1b, t, idx_row, cmp_ratio=case.cmp_ratio,
                                    win_left=case.win_left, win_right=case.win_right)
            if case.cmp_kv is None:
                comp = []
            X = [dec(row(0, b, j)) for j in win] + [dec(row(1, b, c)) for c in comp]
            X = np.stack(X) if X else np.zeros((0, Dq))
            qb = dec(q[key])                                    # [N1, 512]
            s = case.softmax_scale * (qb @ X.T)                 # [N1, R]
            for h in range(N1):
                o, l = softmax_rows(s[h:h + 1], np.ones((1, X.shape[0]), bool), X,
                                    extra_logit=None if sinks is None else float(sinks[h]))
                out[key][h] = o[0]
                lse[lse_at(key)][h] = l[0]
    return out, lse
