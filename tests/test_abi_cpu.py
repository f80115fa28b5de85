"""Host-side tests of libfia.so: it loads, exports every entry point the
header declares, and phase 1 applies the pages' constraint tiers.  Phase 1
never touches the GPU, so descriptors carry fake (aligned, never
dereferenced) device addresses."""
import ctypes
import os
import re

import pytest

from attention_online_softmax_flash_amd import fia

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000


def header_functions():
    src = open(os.path.join(ROOT, "include", "fia.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fia_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = fia.lib()
    names = header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert sorted(fia.EXPORTED) == names


def T(shape, dtype=fia.DT_BF16, data=FAKE, strides=None):
    d = fia.FiaTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        d.shape[i] = s
        d.stride[i] = st
    return d


def P(**kw):
    p = fia.FiaParams()
    p.input_layout = kw.pop("layout", "BSND").encode()
    p.num_heads = kw.pop("num_heads", 4)
    p.num_key_value_heads = kw.pop("num_kv_heads", 0)
    p.scale_value = kw.pop("scale", 0.125)
    p.sparse_mode = kw.pop("sparse_mode", 0)
    p.pre_tokens = kw.pop("pre_tokens", 2147483647)
    p.next_tokens = kw.pop("next_tokens", 2147483647)
    p.pse_type = kw.pop("pse_type", 0)
    p.q_start_idx = kw.pop("q_start_idx", 0)
    p.kv_start_idx = kw.pop("kv_start_idx", 0)
    p.block_size = kw.pop("block_size", 0)
    p.inner_precise = kw.pop("inner_precise", 0)
    p.softmax_lse_flag = kw.pop("lse", 0)
    kvl = kw.pop("kv_layout", None)
    if kvl is not None:
        p.kv_layout = kvl.encode()
    keep = []
    for name in ("actual_seq_lengths", "actual_seq_lengths_kv"):
        vals = kw.pop(name, None)
        if vals is not None:
            arr = (ctypes.c_int64 * len(vals))(*vals)
            keep.append(arr)
            setattr(p, name, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)))
            setattr(p, name + "_len", len(vals))
    sink = kw.pop("learnable_sink", None)
    if sink is not None:
        keep.append(sink)
        p.learnable_sink = ctypes.pointer(sink)
    dl = kw.pop("dev_lens", None)
    if dl is not None:
        keep.append(dl)
        p.actual_seq_lengths_kv_device = ctypes.pointer(dl)
    p.max_actual_seq_length_kv = kw.pop("len_bound", 0)
    p.key_antiquant_mode = kw.pop("kmode", 0)
    p.value_antiquant_mode = kw.pop("vmode", 0)
    for name in ("key_antiquant_scale", "value_antiquant_scale", "key_antiquant_offset",
                 "value_antiquant_offset"):
        t = kw.pop(name, None)
        if t is not None:
            keep.append(t)
            setattr(p, name, ctypes.pointer(t))
    assert not kw, kw
    p._keep = keep
    return p


def plan(p, q, k, v, out, pse=None, mask=None, bt=None, lse=None):
    ws = ctypes.c_size_t(0)
    ex = ctypes.c_void_p(None)
    ptr = lambda d: ctypes.pointer(d) if d is not None else None
    st = fia.lib().fia_get_workspace_size(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ptr(pse),
                                          ptr(mask), ptr(bt), ptr(out), ptr(lse),
                                          ctypes.byref(ws), ctypes.byref(ex))
    msg = fia.lib().fia_last_error().decode()
    kind = None
    if st == 0:
        kind = fia.KIND_NAMES[fia.lib().fia_executor_kind(ex)]
        fia.lib().fia_executor_destroy(ex)
    return st, kind, ws.value, msg


def dense(B=2, S1=64, S2=64, N=4, KVN=2, D=128, dt=fia.DT_BF16):
    q = T((B, S1, N, D), dt)
    return q, T((B, S2, KVN, D), dt), T((B, S2, KVN, D), dt), T((B, S1, N, D), dt)


def test_valid_calls_classify_branches():
    q, k, v, o = dense()
    st, kind, ws, msg = plan(P(num_kv_heads=2, sparse_mode=3), q, k, v, o)
    assert st == 0 and kind == "prefill", msg
    q1, k1, v1, o1 = dense(S1=1, S2=300)
    st, kind, ws, msg = plan(P(num_kv_heads=2), q1, k1, v1, o1)
    assert st == 0 and kind == "decode" and ws > 0, msg
    q3, k3, v3, o3 = dense(D=64, dt=fia.DT_FP32)
    st, kind, _, msg = plan(P(num_kv_heads=2), q3, k3, v3, o3)
    assert st == 0 and kind == "fp32", msg
    qe, ke, ve, oe = dense(S2=0)
    st, kind, _, msg = plan(P(num_kv_heads=2), qe, ke, ve, oe)
    assert st == 0 and kind == "fill", msg


def test_paged_decode_plan_and_workspace_grows_with_lengths():
    q = T((3, 1, 8, 128))
    o = T((3, 1, 8, 128))
    pool = T((20, 128, 2, 128))
    bt = T((3, 16), fia.DT_INT32)
    st, kind, ws1, msg = plan(P(num_heads=8, num_kv_heads=2, block_size=128,
                                actual_seq_lengths_kv=[100, 200, 300]), q, pool, pool, o, bt=bt)
    assert st == 0 and kind == "decode", msg
    # past one split-KV chunk per row: partials for every chunk
    st, kind, ws2, msg = plan(P(num_heads=8, num_kv_heads=2, block_size=128,
                                actual_seq_lengths_kv=[2000, 2000, 2000]), q, pool, pool, o, bt=bt)
    assert st == 0 and ws2 > ws1, msg


BAD = fia.FIA_ERR_PARAM_INVALID
UNS = fia.FIA_ERR_UNSUPPORTED


@pytest.mark.parametrize("desc,kw,expect", [
    ("Q_N not a multiple of KV_N", dict(num_heads=4, num_kv_heads=3), BAD),
    ("group ratio above 64", dict(num_heads=130, num_kv_heads=2), BAD),
    ("sparse_mode out of range", dict(sparse_mode=5), BAD),
    ("sparse_mode negative", dict(sparse_mode=-1), BAD),
    ("sparse_mode 1 needs a mask tensor", dict(sparse_mode=1), BAD),
    ("band with -next > pre", dict(sparse_mode=4, pre_tokens=-3, next_tokens=2), BAD),
    ("pse_type out of range", dict(pse_type=4), BAD),
    ("pse_type 1 is training only", dict(pse_type=1), BAD),
    ("pse_type 3 unsupported", dict(pse_type=3), UNS),
    ("pse_type 2 without pse_shift", dict(pse_type=2), BAD),
    ("inner_precise out of range", dict(inner_precise=4), BAD),
    ("lse flag without lse tensor", dict(lse=1), BAD),
    ("negative actual length", dict(actual_seq_lengths=[-1, 3]), BAD),
    ("actual length above S", dict(actual_seq_lengths=[65, 3]), BAD),
    ("kv length above S2", dict(actual_seq_lengths_kv=[70, 3]), BAD),
])
def test_phase1_rejects(desc, kw, expect):
    q, k, v, o = dense(N=kw.get("num_heads", 4), KVN=kw.get("num_kv_heads", 2) or 4)
    kw.setdefault("num_kv_heads", 2)
    st, _, _, msg = plan(P(**kw), q, k, v, o)
    assert st == expect, (desc, st, msg)
    assert msg


def test_length_array_size_rule():
    q, k, v, o = dense(B=3)
    st, _, _, msg = plan(P(num_kv_heads=2, actual_seq_lengths=[5, 6]), q, k, v, o)
    assert st == BAD and "length" in msg
    st, _, _, msg = plan(P(num_kv_heads=2, actual_seq_lengths=[5]), q, k, v, o)
    assert st == 0, msg
    st, _, _, msg = plan(P(num_kv_heads=2, actual_seq_lengths=[5, 6, 7, 8]), q, k, v, o)
    assert st == 0, msg


def test_alibi_rules():
    q, k, v, o = dense(S1=64, S2=64)
    slopes = T((4,), fia.DT_FP32)
    st, _, _, msg = plan(P(num_kv_heads=2, pse_type=2), q, k, v, o, pse=slopes)
    assert st == 0, msg
    q2, k2, v2, o2 = dense(S1=32, S2=64)
    st, _, _, msg = plan(P(num_kv_heads=2, pse_type=2), q2, k2, v2, o2, pse=slopes)
    assert st == BAD and "Q_S" in msg
    st, _, _, msg = plan(P(num_kv_heads=2, pse_type=2, actual_seq_lengths=[10, 20],
                           actual_seq_lengths_kv=[10, 21]), q, k, v, o, pse=slopes)
    assert st == BAD
    st, _, _, msg = plan(P(num_kv_heads=2, pse_type=2, kv_start_idx=1048577), q, k, v, o, pse=slopes)
    assert st == BAD
    st, _, _, msg = plan(P(num_kv_heads=2, pse_type=2), q, k, v, o, pse=T((3,), fia.DT_FP32))
    assert st == BAD
    st, _, _, msg = plan(P(num_kv_heads=2, pse_type=2), q, k, v, o, pse=T((4,), fia.DT_BF16))
    assert st == BAD
    st, _, _, msg = plan(P(num_kv_heads=2, pse_type=0), q, k, v, o, pse=T((2, 4, 64, 64)))
    assert st == 0, msg   # pse_type 0 takes a bias tensor


def test_mask_tensor_rules():
    q, k, v, o = dense()
    good = T((2048, 2048), fia.DT_BOOL)
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=3), q, k, v, o, mask=good)
    assert st == 0, msg
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=3), q, k, v, o, mask=T((1, 1, 2048, 2048), fia.DT_UINT8))
    assert st == 0, msg
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=3), q, k, v, o, mask=T((1024, 1024), fia.DT_BOOL))
    assert st == BAD
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=3), q, k, v, o, mask=T((2048, 2048), fia.DT_FP32))
    assert st == BAD
    # mode 0 reads an explicit mask; a 2048 x 2048 one covers this problem
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=0), q, k, v, o, mask=good)
    assert st == 0, msg


def test_paged_rules():
    q = T((2, 1, 4, 128))
    o = T((2, 1, 4, 128))
    pool = T((10, 128, 2, 128))
    bt = T((2, 4), fia.DT_INT32)
    ok = dict(num_heads=4, num_kv_heads=2, block_size=128, actual_seq_lengths_kv=[300, 500])
    st, _, _, msg = plan(P(**ok), q, pool, pool, o, bt=bt)
    assert st == 0, msg
    st, _, _, msg = plan(P(num_heads=4, num_kv_heads=2, block_size=128), q, pool, pool, o, bt=bt)
    assert st == BAD and "actual_seq_lengths_kv" in msg
    st, _, _, msg = plan(P(**dict(ok, block_size=0)), q, pool, pool, o, bt=bt)
    assert st == BAD
    st, _, _, msg = plan(P(**dict(ok, block_size=100)), q, T((10, 100, 2, 128)), T((10, 100, 2, 128)), o, bt=bt)
    assert st == BAD
    st, _, _, msg = plan(P(**dict(ok, block_size=2048)), q, T((10, 2048, 2, 128)), T((10, 2048, 2, 128)), o, bt=bt)
    assert st == BAD
    st, _, _, msg = plan(P(**ok), q, pool, pool, o, bt=T((3, 4), fia.DT_INT32))
    assert st == BAD
    st, _, _, msg = plan(P(**ok), q, pool, pool, o, bt=T((2, 3), fia.DT_INT32))
    assert st == BAD
    st, _, _, msg = plan(P(**ok), q, pool, pool, o, bt=T((2, 4), fia.DT_INT64))
    assert st == BAD
    st, _, _, msg = plan(P(**ok), q, pool, pool, o, bt=T((8,), fia.DT_INT32))
    assert st == BAD
    st, _, _, msg = plan(P(**ok), q, T((10, 64, 2, 128)), T((10, 64, 2, 128)), o, bt=bt)
    assert st == BAD
    st, kind, _, msg = plan(P(**ok), q, T((10, 128, 256)), T((10, 128, 256)), o, bt=bt)
    assert st == 0 and kind == "decode", msg


def test_bnnbsd_paged_rules():
    q = T((2, 1, 4, 128))
    o = T((2, 1, 4, 128))
    bt = T((2, 4), fia.DT_INT32)
    ok = dict(num_heads=4, num_kv_heads=2, block_size=128, actual_seq_lengths_kv=[300, 500])
    pool = T((10, 2, 128, 128))
    st, kind, _, msg = plan(P(kv_layout="BnNBsD", **ok), q, pool, pool, o, bt=bt)
    assert st == 0 and kind == "decode", msg
    # the same pool read as PA_ND has the wrong shape
    st, _, _, msg = plan(P(**ok), q, pool, pool, o, bt=bt)
    assert st == BAD
    # PA_ND pool under BnNBsD: rejected
    st, _, _, msg = plan(P(kv_layout="BnNBsD", **ok), q, T((10, 128, 2, 128)), T((10, 128, 2, 128)),
                         o, bt=bt)
    assert st == BAD and "BnNBsD" in msg
    st, _, _, msg = plan(P(kv_layout="BnNBsD", **ok), q, T((10, 128, 256)), T((10, 128, 256)), o, bt=bt)
    assert st == BAD
    st, _, _, msg = plan(P(kv_layout="NZ", **ok), q, pool, pool, o, bt=bt)
    assert st == BAD and "kv_layout" in msg
    # prefill over a BnNBsD pool
    q2 = T((2, 64, 4, 128))
    o2 = T((2, 64, 4, 128))
    st, kind, _, msg = plan(P(kv_layout="BnNBsD", sparse_mode=3, **ok), q2, pool, pool, o2, bt=bt)
    assert st == 0 and kind == "prefill", msg


def test_explicit_mask_rules():
    q, k, v, o = dense(B=2, S1=64, S2=64)
    for shape in [(2, 64, 64), (1, 64, 64), (64, 64), (2, 1, 64, 64), (2, 80, 128)]:
        for mode in (0, 1):
            st, kind, _, msg = plan(P(num_kv_heads=2, sparse_mode=mode), q, k, v, o,
                                    mask=T(shape, fia.DT_UINT8))
            assert st == 0 and kind == "prefill", (shape, mode, msg)
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=0), q, k, v, o, mask=T((2, 64, 64), fia.DT_BOOL))
    assert st == 0, msg
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=1), q, k, v, o)
    assert st == BAD and "atten_mask" in msg
    bad = [((3, 64, 64), fia.DT_UINT8), ((2, 63, 64), fia.DT_UINT8), ((2, 64, 60), fia.DT_UINT8),
           ((2, 2, 64, 64), fia.DT_UINT8), ((2, 64, 64), fia.DT_FP32), ((64,), fia.DT_UINT8)]
    for shape, dt in bad:
        st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=0), q, k, v, o, mask=T(shape, dt))
        assert st == BAD, (shape, dt, msg)
    # rows not 4-byte aligned
    q2, k2, v2, o2 = dense(B=2, S1=8, S2=62)
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=0), q2, k2, v2, o2,
                         mask=T((2, 8, 62), fia.DT_UINT8))
    assert st == UNS and "aligned" in msg
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=0), q2, k2, v2, o2,
                         mask=T((2, 8, 64), fia.DT_UINT8))
    assert st == 0, msg
    # decode with a mask
    q1, k1, v1, o1 = dense(S1=1, S2=300)
    st, kind, _, msg = plan(P(num_kv_heads=2, sparse_mode=0), q1, k1, v1, o1,
                            mask=T((2, 1, 300), fia.DT_INT8))
    assert st == 0 and kind == "decode", msg


def test_pse_bias_rules():
    """pseType 0 bias tensor: 4 dims [B or 1, Q_N, >= Q_S or 1, >= KV_S] in the
    query's dtype (V5 PSE parameter group)."""
    q, k, v, o = dense(B=2, S1=64, S2=64)
    for shape in [(2, 4, 64, 64), (1, 4, 64, 64), (2, 4, 1, 64), (1, 4, 80, 128)]:
        for mode in (0, 2, 3):
            st, kind, _, msg = plan(P(num_kv_heads=2, sparse_mode=mode), q, k, v, o, pse=T(shape))
            assert st == 0 and kind == "prefill", (shape, mode, msg)
    bad = [((3, 4, 64, 64), fia.DT_BF16), ((2, 2, 64, 64), fia.DT_BF16), ((2, 4, 32, 64), fia.DT_BF16),
           ((2, 4, 64, 60), fia.DT_BF16), ((2, 4, 64, 64), fia.DT_FP32), ((2, 4, 64), fia.DT_BF16),
           ((4,), fia.DT_BF16)]
    for shape, dt in bad:
        st, _, _, msg = plan(P(num_kv_heads=2), q, k, v, o, pse=T(shape, dt))
        assert st == BAD, (shape, dt, msg)
    st, _, _, msg = plan(P(num_kv_heads=2, scale=0.0), q, k, v, o, pse=T((2, 4, 64, 64)))
    assert st == UNS and "scale" in msg
    # bias with an explicit mask
    st, _, _, msg = plan(P(num_kv_heads=2, sparse_mode=1), q, k, v, o, pse=T((2, 4, 64, 64)),
                         mask=T((2, 64, 64), fia.DT_UINT8))
    assert st == 0, msg
    # rows not aligned to 4 elements
    q2, k2, v2, o2 = dense(B=2, S1=8, S2=62)
    st, _, _, msg = plan(P(num_kv_heads=2), q2, k2, v2, o2, pse=T((2, 4, 8, 62)))
    assert st == UNS and "aligned" in msg
    st, _, _, msg = plan(P(num_kv_heads=2), q2, k2, v2, o2, pse=T((2, 4, 8, 64)))
    assert st == 0, msg
    # fp32 query takes an fp32 bias; decode takes one row
    q3, k3, v3, o3 = dense(D=64, dt=fia.DT_FP32)
    st, kind, _, msg = plan(P(num_kv_heads=2), q3, k3, v3, o3, pse=T((2, 4, 64, 64), fia.DT_FP32))
    assert st == 0 and kind == "fp32", msg
    q1, k1, v1, o1 = dense(S1=1, S2=300)
    st, kind, _, msg = plan(P(num_kv_heads=2), q1, k1, v1, o1, pse=T((2, 4, 1, 300)))
    assert st == 0 and kind == "decode", msg
    # paged: the last dim covers the block table's pages
    pool = T((20, 128, 2, 128))
    bt = T((2, 4), fia.DT_INT32)
    st, _, _, msg = plan(P(num_kv_heads=2, block_size=128, actual_seq_lengths_kv=[300, 400]),
                         q1, pool, pool, o1, bt=bt,
                         pse=T((2, 4, 1, 512)))
    assert st == 0, msg
    st, _, _, msg = plan(P(num_kv_heads=2, block_size=128, actual_seq_lengths_kv=[300, 400]),
                         q1, pool, pool, o1, bt=bt,
                         pse=T((2, 4, 1, 508)))
    assert st == BAD, msg


def test_learnable_sink_rules():
    """V5 LearnableSink group: [Q_N] in the query's dtype (float16 / bfloat16),
    innerPrecise 0, no pse / ALiBi."""
    q, k, v, o = dense(B=2, S1=64, S2=64)
    st, kind, _, msg = plan(P(num_kv_heads=2, sparse_mode=3, learnable_sink=T((4,))), q, k, v, o)
    assert st == 0 and kind == "prefill", msg
    q1, k1, v1, o1 = dense(S1=1, S2=300)
    st, kind, _, msg = plan(P(num_kv_heads=2, learnable_sink=T((4,))), q1, k1, v1, o1)
    assert st == 0 and kind == "decode", msg
    bad = [dict(learnable_sink=T((3,))), dict(learnable_sink=T((1, 4))),
           dict(learnable_sink=T((4,), fia.DT_FP32)), dict(learnable_sink=T((4,), fia.DT_FP16)),
           dict(learnable_sink=T((4,)), inner_precise=1)]
    for kw in bad:
        st, _, _, msg = plan(P(num_kv_heads=2, **kw), q, k, v, o)
        assert st == BAD, (kw, msg)
    st, _, _, msg = plan(P(num_kv_heads=2, learnable_sink=T((4,), strides=[2])), q, k, v, o)
    assert st == UNS and "contiguous" in msg
    st, _, _, msg = plan(P(num_kv_heads=2, pse_type=2, learnable_sink=T((4,))), q, k, v, o,
                         pse=T((4,), fia.DT_FP32))
    assert st == BAD and "pse" in msg
    st, _, _, msg = plan(P(num_kv_heads=2, learnable_sink=T((4,))), q, k, v, o, pse=T((2, 4, 64, 64)))
    assert st == BAD and "pse" in msg
    q3, k3, v3, o3 = dense(D=64, dt=fia.DT_FP32)
    st, _, _, msg = plan(P(num_kv_heads=2, learnable_sink=T((4,), fia.DT_FP32)), q3, k3, v3, o3)
    assert st == BAD, msg


def test_fake_quant_kv_rules():
    """V5 fake-quant group: int8 / e4m3fn key/value with a bf16 query, scales
    per channel (query dtype; fp32 in the key-channel / value-token mode),
    per tensor (int8) or per token (fp32 [B, >= S2]); offsets int8 only."""
    B, S2, KVN, D = 2, 300, 2, 128
    q = T((B, 1, 4, D))
    o = T((B, 1, 4, D))
    k8 = T((B, S2, KVN, D), fia.DT_INT8)
    f8 = T((B, S2, KVN, D), fia.DT_FP8_E4M3FN)
    chan = lambda dt=fia.DT_BF16: T((KVN, D), dt)
    tok = lambda cols=300: T((B, cols), fia.DT_FP32)
    ok = [
        (k8, dict(key_antiquant_scale=chan(), value_antiquant_scale=chan())),
        (k8, dict(key_antiquant_scale=chan(), value_antiquant_scale=chan(),
                  key_antiquant_offset=chan(), value_antiquant_offset=chan())),
        (k8, dict(key_antiquant_scale=T((1,)), value_antiquant_scale=T((1,)))),
        (k8, dict(key_antiquant_scale=T((1, KVN, 1, D)), value_antiquant_scale=T((KVN * D,)))),
        (f8, dict(kmode=1, vmode=1, key_antiquant_scale=tok(), value_antiquant_scale=tok(304))),
        (k8, dict(kmode=1, vmode=1, key_antiquant_scale=T((1, B, 300), fia.DT_FP32),
                  value_antiquant_scale=tok(), key_antiquant_offset=T((1, B, 300), fia.DT_FP32),
                  value_antiquant_offset=tok())),
        (k8, dict(kmode=0, vmode=1, key_antiquant_scale=chan(fia.DT_FP32), value_antiquant_scale=tok())),
    ]
    for kv, kw in ok:
        st, kind, _, msg = plan(P(num_kv_heads=KVN, **kw), q, kv, kv, o)
        assert st == 0 and kind == "decode", (kw.keys(), msg)
    bad = [
        (k8, dict(key_antiquant_scale=chan())),                                   # value scale missing
        (k8, dict(kmode=1, vmode=0, key_antiquant_scale=tok(), value_antiquant_scale=chan())),
        (k8, dict(kmode=7, vmode=7, key_antiquant_scale=chan(), value_antiquant_scale=chan())),
        (k8, dict(key_antiquant_scale=chan(fia.DT_FP32), value_antiquant_scale=chan(fia.DT_FP32))),
        (k8, dict(kmode=1, vmode=1, key_antiquant_scale=tok(296), value_antiquant_scale=tok())),
        (k8, dict(kmode=1, vmode=1, key_antiquant_scale=T((B, 300)), value_antiquant_scale=tok())),
        (k8, dict(key_antiquant_scale=chan(), value_antiquant_scale=chan(), key_antiquant_offset=chan())),
        (f8, dict(key_antiquant_scale=chan(), value_antiquant_scale=chan(),
                  key_antiquant_offset=chan(), value_antiquant_offset=chan())),
        (f8, dict(key_antiquant_scale=T((1,)), value_antiquant_scale=T((1,)))),
        (k8, dict(key_antiquant_scale=T((KVN, D + 1)), value_antiquant_scale=chan())),
        (k8, dict(kmode=0, vmode=1, key_antiquant_scale=chan(), value_antiquant_scale=tok())),
    ]
    for kv, kw in bad:
        st, _, _, msg = plan(P(num_kv_heads=KVN, **kw), q, kv, kv, o)
        assert st == BAD, (kw.keys(), msg)
    good = dict(key_antiquant_scale=chan(), value_antiquant_scale=chan())
    st, _, _, msg = plan(P(num_kv_heads=KVN, kmode=2, vmode=2, **good), q, k8, k8, o)
    assert st == UNS, msg
    q2, o2 = T((B, 4, 4, D)), T((B, 4, 4, D))
    st, _, _, msg = plan(P(num_kv_heads=KVN, **good), q2, k8, k8, o2)
    assert st == UNS and "query length 1" in msg
    st, _, _, msg = plan(P(num_kv_heads=KVN, learnable_sink=T((4,)), **good), q, k8, k8, o)
    assert st == UNS
    st, _, _, msg = plan(P(num_kv_heads=KVN, kmode=1, vmode=1, key_antiquant_scale=T((B, 302), fia.DT_FP32),
                           value_antiquant_scale=T((B, 302), fia.DT_FP32)), q, k8, k8, o)
    assert st == UNS and "aligned" in msg
    st, _, _, msg = plan(P(num_kv_heads=KVN), q, k8, f8, o)
    assert st == BAD
    qb, kb, vb, ob = dense(S1=1, S2=300)
    st, _, _, msg = plan(P(num_kv_heads=2, **good), qb, kb, vb, ob)
    assert st == BAD and "int8 or fp8" in msg
    pool = T((20, 16, KVN, D), fia.DT_INT8)
    st, _, _, msg = plan(P(num_kv_heads=KVN, block_size=16, actual_seq_lengths_kv=[30, 40], **good), q, pool,
                         pool, o, bt=T((B, 4), fia.DT_INT32))
    assert st == BAD and "block_size" in msg
    pool = T((20, 32, KVN, D), fia.DT_INT8)
    st, kind, _, msg = plan(P(num_kv_heads=KVN, block_size=32, actual_seq_lengths_kv=[30, 40], **good), q,
                            pool, pool, o, bt=T((B, 4), fia.DT_INT32))
    assert st == 0 and kind == "decode", msg
    # KV lengths on the device: per-channel and per-token tables (the tables
    # cover the padded S2, so any length up to the bound reads inside them)
    dl = dict(dev_lens=T((B,), fia.DT_INT32), len_bound=300)
    for kv, kw in ((k8, good), (f8, dict(kmode=1, vmode=1, key_antiquant_scale=tok(), value_antiquant_scale=tok()))):
        st, kind, ws, msg = plan(P(num_kv_heads=KVN, **dl, **kw), q, kv, kv, o)
        assert st == 0 and kind == "decode" and ws > 0, msg


def test_tnd_rules():
    q = T((10, 4, 128))
    o = T((10, 4, 128))
    k = T((12, 2, 128))
    st, kind, _, msg = plan(P(layout="TND", num_kv_heads=2, actual_seq_lengths=[4, 10],
                              actual_seq_lengths_kv=[5, 12]), q, k, k, o)
    assert st == 0 and kind == "prefill", msg
    st, _, _, msg = plan(P(layout="TND", num_kv_heads=2, actual_seq_lengths=[4, 9],
                           actual_seq_lengths_kv=[5, 12]), q, k, k, o)
    assert st == BAD and "T" in msg
    st, _, _, msg = plan(P(layout="TND", num_kv_heads=2, actual_seq_lengths=[6, 4, 10],
                           actual_seq_lengths_kv=[5, 6, 12]), q, k, k, o)
    assert st == BAD and "non-decreasing" in msg
    st, _, _, msg = plan(P(layout="TND", num_kv_heads=2, actual_seq_lengths_kv=[5, 12]), q, k, k, o)
    assert st == BAD


def test_lse_shape_rules():
    q, k, v, o = dense()
    st, _, _, msg = plan(P(num_kv_heads=2, lse=1), q, k, v, o, lse=T((2, 4, 64, 1), fia.DT_FP32))
    assert st == 0, msg
    st, _, _, msg = plan(P(num_kv_heads=2, lse=1), q, k, v, o, lse=T((2, 4, 64, 1), fia.DT_BF16))
    assert st == BAD
    st, _, _, msg = plan(P(num_kv_heads=2, lse=1), q, k, v, o, lse=T((2, 4, 64), fia.DT_FP32))
    assert st == BAD


def test_shape_limits_and_unsupported():
    q, k, v, o = dense(D=96)
    st, _, _, msg = plan(P(num_kv_heads=2), q, k, v, o)
    assert st == UNS
    q, k, v, o = dense(dt=fia.DT_FP16)
    st, _, _, msg = plan(P(num_kv_heads=2), q, k, v, o)
    assert st == UNS
    q, k, v, o = dense(N=257, KVN=257)
    st, _, _, msg = plan(P(num_heads=257, num_kv_heads=257), q, k, v, o)
    assert st == BAD
    # The fp32 path is built for D in {32, 64, 128, 256}; any other D is
    # refused in phase 1, so a successful phase 1 always has a kernel to run.
    for D in (32, 64, 128, 256):
        q, k, v, o = dense(D=D, dt=fia.DT_FP32)
        st, kind, _, msg = plan(P(num_kv_heads=2), q, k, v, o)
        assert st == 0 and kind == "fp32", (D, msg)
    for D in (96, 160, 192, 224):
        q, k, v, o = dense(D=D, dt=fia.DT_FP32)
        st, _, _, msg = plan(P(num_kv_heads=2), q, k, v, o)
        assert st == UNS and "fp32" in msg, (D, msg)
    q, k, v, o = dense()
    st, _, _, msg = plan(P(num_kv_heads=2, layout="NSD"), q, k, v, o)
    assert st == BAD
    q, k, v, o = dense()
    q.data = FAKE + 2
    st, _, _, msg = plan(P(num_kv_heads=2), q, k, v, o)
    assert st == UNS and "aligned" in msg
    q, k, v, o = dense()
    st, _, _, msg = plan(P(num_kv_heads=2), q, k, T((2, 64, 2, 128), fia.DT_FP32), o)
    assert st == BAD
    q, k, v, o = dense()
    q.data = None
    st, _, _, msg = plan(P(num_kv_heads=2), q, k, v, o)
    assert st == fia.FIA_ERR_NULLPTR


def test_null_arguments_and_run_errors():
    L = fia.lib()
    ws = ctypes.c_size_t(0)
    ex = ctypes.c_void_p(None)
    st = L.fia_get_workspace_size(None, None, None, None, None, None, None, None, None,
                                  ctypes.byref(ws), ctypes.byref(ex))
    assert st == fia.FIA_ERR_NULLPTR
    assert L.fia_run(None, 0, None, None) == fia.FIA_ERR_NULLPTR
    L.fia_executor_destroy(None)
    # A workspace smaller than required is rejected before any HIP call.
    q, k, v, o = dense(S1=1, S2=2000)
    p = P(num_kv_heads=2)
    ptr = lambda d: ctypes.pointer(d)
    st = L.fia_get_workspace_size(ctypes.byref(p), ptr(q), ptr(k), ptr(v), None, None, None,
                                  ptr(o), None, ctypes.byref(ws), ctypes.byref(ex))
    assert st == 0 and ws.value > 0
    assert L.fia_run(None, ws.value, ex, None) == fia.FIA_ERR_WORKSPACE
    assert L.fia_run(FAKE, ws.value - 1, ex, None) == fia.FIA_ERR_WORKSPACE
    L.fia_executor_destroy(ex)


def sparse_plan_status(**over):
    B, N1 = 2, 64
    t = dict(q=T((B, 1, N1, 512)), ori=T((32, 128, 1, 640), fia.DT_UINT8),
             cmp=T((16, 128, 1, 640), fia.DT_UINT8), idx=T((B, 1, 1, 512), fia.DT_INT32),
             obt=T((B, 16), fia.DT_INT32), cbt=T((B, 4), fia.DT_INT32),
             seq=T((B,), fia.DT_INT32), sinks=T((N1,), fia.DT_FP32), out=T((B, 1, N1, 512)),
             oidx=None, cu=None, max_seq=2048)
    p = fia.FiaSparseParams()
    p.softmax_scale = 0.0441941738
    p.kv_quant_mode, p.tile_size, p.rope_head_dim, p.cmp_ratio = 1, 64, 64, 4
    p.ori_mask_mode, p.cmp_mask_mode, p.ori_win_left, p.ori_win_right = 4, 3, 127, 0
    p.layout_q, p.layout_kv, p.return_softmax_lse = b"BSND", b"PA_ND", 0
    for key, val in over.items():
        if hasattr(p, key) and key not in t:
            setattr(p, key, val)
        else:
            t[key] = val
    ws = ctypes.c_size_t(0)
    ex = ctypes.c_void_p(None)
    ptr = lambda d: ctypes.pointer(d) if d is not None else None
    st = fia.lib().fia_sparse_get_workspace_size(
        ctypes.byref(p), ptr(t["q"]), ptr(t["ori"]), ptr(t["cmp"]), ptr(t["oidx"]), ptr(t["idx"]),
        ptr(t["obt"]), ptr(t["cbt"]), ptr(t["cu"]), ptr(t["seq"]), t["max_seq"], ptr(t["sinks"]), None,
        ptr(t["out"]), ctypes.byref(ws), ctypes.byref(ex))
    msg = fia.lib().fia_last_error().decode()
    if st == 0:
        assert fia.KIND_NAMES[fia.lib().fia_executor_kind(ex)] == "sparse"
        fia.lib().fia_executor_destroy(ex)
    return st, msg


@pytest.mark.parametrize("over,expect", [
    ({}, 0),
    (dict(cmp=None, idx=None, cbt=None, cmp_ratio=1), 0),
    (dict(q=T((2, 1, 64, 576)), out=T((2, 1, 64, 576))), BAD),
    (dict(q=T((2, 1, 32, 512)), out=T((2, 1, 32, 512)), sinks=T((32,), fia.DT_FP32)), BAD),
    (dict(tile_size=32), BAD),
    (dict(rope_head_dim=32), BAD),
    (dict(kv_quant_mode=0), BAD),
    (dict(ori_win_left=63), BAD),
    (dict(ori_win_right=1), BAD),
    (dict(ori_mask_mode=3), BAD),
    (dict(cmp_mask_mode=4), BAD),
    (dict(cmp_ratio=128), BAD),                       # indices need ratio 4
    (dict(idx=None, cmp_ratio=128), 0),               # heavily compressed mode
    (dict(idx=None), BAD),                            # no indices needs ratio 128
    (dict(idx=None, cmp_ratio=128, cmp_mask_mode=4), BAD),
    (dict(idx=None, cmp_ratio=128, max_seq=600000, obt=T((2, 4688), fia.DT_INT32),
          cbt=T((2, 40), fia.DT_INT32)), 0),          # 128 + 4736 slots per token
    (dict(idx=None, cmp_ratio=128, max_seq=1100000, obt=T((2, 8594), fia.DT_INT32),
          cbt=T((2, 68), fia.DT_INT32)), UNS),        # more than 8192 slots per token
    (dict(cmp_ratio=2), BAD),
    (dict(idx=T((2, 1, 1, 256), fia.DT_INT32)), BAD),
    (dict(oidx=T((2, 1, 1, 512), fia.DT_INT32)), BAD),
    (dict(ori=T((32, 100, 1, 640), fia.DT_UINT8)), BAD),
    (dict(ori=T((32, 128, 1, 656), fia.DT_UINT8)), BAD),
    (dict(obt=T((2, 15), fia.DT_INT32)), BAD),
    (dict(cbt=T((2, 3), fia.DT_INT32)), BAD),
    (dict(return_softmax_lse=1), BAD),
    (dict(layout_q=b"TND"), BAD),                     # TND needs [T1, N1, 512] and cu_seqlens_q
    (dict(layout_q=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)), idx=T((5, 1, 512), fia.DT_INT32),
          cu=T((3,), fia.DT_INT32)), 0),
    (dict(layout_q=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)), idx=None, cmp_ratio=128,
          cu=T((3,), fia.DT_INT32)), 0),
    (dict(layout_q=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)), idx=T((5, 1, 512), fia.DT_INT32)),
     BAD),                                            # cu_seqlens_q missing
    (dict(layout_q=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)), idx=T((5, 1, 512), fia.DT_INT32),
          cu=T((2,), fia.DT_INT32)), BAD),            # cu_seqlens_q must be [B + 1]
    (dict(layout_q=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)), idx=T((5, 1, 512), fia.DT_INT32),
          cu=T((3,), fia.DT_INT64)), BAD),
    (dict(layout_q=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)), idx=T((2, 1, 1, 512), fia.DT_INT32),
          cu=T((3,), fia.DT_INT32)), BAD),            # indices [T1, 1, K2] with TND
    (dict(layout_q=b"TND", q=T((5, 64, 512)), out=T((4, 64, 512)), idx=T((5, 1, 512), fia.DT_INT32),
          cu=T((3,), fia.DT_INT32)), BAD),
    (dict(layout_q=b"TND", q=T((70000, 64, 512)), out=T((70000, 64, 512)),
          idx=T((70000, 1, 512), fia.DT_INT32), cu=T((3,), fia.DT_INT32)), UNS),
    (dict(cu=T((3,), fia.DT_INT32)), BAD),            # cu_seqlens_q only with TND
    (dict(layout_kv=b"BSND"), BAD),
    (dict(sinks=T((64,), fia.DT_BF16)), BAD),
    (dict(q=T((2, 2, 64, 512)), out=T((2, 2, 64, 512)), idx=T((2, 2, 1, 512), fia.DT_INT32)), 0),
    (dict(q=T((2, 4, 64, 512)), out=T((2, 4, 64, 512)), idx=None, cmp_ratio=128), 0),
    (dict(q=T((2, 2, 64, 512)), out=T((2, 2, 64, 512))), BAD),        # indices [B, 1, ...] for S1 = 2
    (dict(q=T((2, 2, 64, 512)), out=T((2, 1, 64, 512)), idx=T((2, 2, 1, 512), fia.DT_INT32)), BAD),
    (dict(q=T((2, 0, 64, 512)), out=T((2, 0, 64, 512)), idx=T((2, 0, 1, 512), fia.DT_INT32)), BAD),
    (dict(q=T((2, 40000, 64, 512)), out=T((2, 40000, 64, 512)),
          idx=T((2, 40000, 1, 512), fia.DT_INT32)), UNS),
])
def test_sparse_phase1(over, expect):
    st, msg = sparse_plan_status(**over)
    assert st == expect, (over, msg)


def sfmla_plan_status(**over):
    """Phase 1 of sparse_flash_mla on fake descriptors (CSA, BSND q, PA_BBND
    bf16 pools by default)."""
    B, N1 = 2, 64
    dt = over.pop("dt", fia.DT_BF16)
    t = dict(q=T((B, 1, N1, 512), dt), ori=T((32, 128, 1, 512), dt), cmp=T((16, 128, 1, 512), dt),
             idx=T((B, 1, 1, 512), fia.DT_INT32), obt=T((B, 16), fia.DT_INT32),
             cbt=T((B, 4), fia.DT_INT32), cuq=None, cuo=None, cuc=None, sq=None,
             seq=T((B,), fia.DT_INT32), sinks=None, out=T((B, 1, N1, 512), dt),
             lse=T((B, 1, 1, N1), fia.DT_FP32), oidx=None, max_seq=2048)
    p = fia.FiaSfmlaParams()
    p.softmax_scale = 0.0441941738
    p.cmp_ratio, p.ori_mask_mode, p.cmp_mask_mode, p.ori_win_left, p.ori_win_right = 4, 4, 3, 127, 0
    p.layout_q, p.layout_kv, p.return_softmax_lse = b"BSND", b"PA_BBND", 1
    for key, val in over.items():
        if hasattr(p, key) and key not in t:
            setattr(p, key, val)
        else:
            t[key] = val
    ws = ctypes.c_size_t(0)
    ex = ctypes.c_void_p(None)
    ptr = lambda d: ctypes.pointer(d) if d is not None else None
    st = fia.lib().fia_sparse_flash_mla_get_workspace_size(
        ctypes.byref(p), ptr(t["q"]), ptr(t["ori"]), ptr(t["cmp"]), ptr(t["oidx"]), ptr(t["idx"]),
        ptr(t["obt"]), ptr(t["cbt"]), ptr(t["cuq"]), ptr(t["cuo"]), ptr(t["cuc"]), ptr(t["sq"]),
        ptr(t["seq"]), t["max_seq"], ptr(t["sinks"]), None, ptr(t["out"]), ptr(t["lse"]),
        ctypes.byref(ws), ctypes.byref(ex))
    msg = fia.lib().fia_last_error().decode()
    if st == 0:
        assert fia.KIND_NAMES[fia.lib().fia_executor_kind(ex)] == "sparse"
        fia.lib().fia_executor_destroy(ex)
    return st, msg, ws.value


I32, F32, F16 = fia.DT_INT32, fia.DT_FP32, fia.DT_FP16


@pytest.mark.parametrize("over,expect", [
    ({}, 0),
    (dict(dt=F16), 0),
    (dict(sinks=T((64,), F32)), 0),
    (dict(return_softmax_lse=0, lse=None), 0),
    (dict(return_softmax_lse=1, lse=None), fia.FIA_ERR_NULLPTR),
    (dict(lse=T((2, 64, 1, 1), F32)), BAD),                  # [B, N2, S1, N1 / N2]
    (dict(lse=T((2, 1, 1, 64), fia.DT_BF16)), BAD),
    (dict(dt=fia.DT_FP32), BAD),                              # fp16 / bf16 only
    (dict(ori=T((32, 128, 1, 512), F16)), BAD),               # dtypes must agree
    (dict(out=T((2, 1, 64, 512), F16)), BAD),
    (dict(ori=T((32, 128, 1, 640), fia.DT_UINT8)), BAD),      # packed rows are the other operator
    (dict(ori=T((32, 128, 2, 512))), BAD),                    # KV_N must be 1
    (dict(ori=T((32, 1025, 1, 512))), BAD),                   # block_size 1..1024
    (dict(ori=T((2048, 1, 1, 512)), obt=T((2, 2048), I32)), 0),   # block_size 1
    (dict(ori=T((700, 3, 1, 512)), obt=T((2, 683), I32)), 0),     # block_size 3
    (dict(obt=T((2, 15), I32)), BAD),                         # too few columns
    (dict(obt=None), BAD),
    (dict(q=T((2, 1, 48, 512)), out=T((2, 1, 48, 512)), lse=T((2, 1, 1, 48), F32)), BAD),
    (dict(q=T((2, 1, 1, 512)), out=T((2, 1, 1, 512)), lse=T((2, 1, 1, 1), F32)), 0),
    (dict(q=T((2, 1, 256, 512)), out=T((2, 1, 256, 512)), lse=T((2, 1, 1, 256), F32)), BAD),
    (dict(q=T((2, 1, 64, 576)), out=T((2, 1, 64, 576))), BAD),
    (dict(idx=T((2, 1, 1, 100), I32)), 0),                    # any K2 >= 1
    (dict(idx=T((2, 1, 1, 8200), I32)), UNS),                 # window + K2 > 8192
    (dict(cmp_ratio=128), BAD),                               # CSA needs ratio 4
    (dict(idx=None, cmp_ratio=128), 0),                       # HCA
    (dict(idx=None), BAD),                                    # HCA needs ratio 128
    (dict(cmp=None, idx=None, cbt=None, cmp_ratio=1, cmp_mask_mode=0), 0),   # SWA
    (dict(cmp=None, idx=None, cbt=None, cmp_ratio=1, cmp_mask_mode=3), BAD),
    (dict(cmp=None, idx=None, cmp_ratio=1, cmp_mask_mode=0), BAD),            # SWA: no cmp table
    (dict(cmp_mask_mode=4), BAD),
    (dict(ori_win_left=63), BAD),
    (dict(ori_mask_mode=3), BAD),
    (dict(oidx=T((2, 1, 1, 512), I32)), BAD),                 # reserved
    (dict(sq=T((2,), I32)), BAD),                             # reserved
    (dict(sinks=T((64,), fia.DT_BF16)), BAD),
    (dict(sinks=T((32,), F32)), BAD),
    (dict(layout_kv=b"BSND", ori=T((2, 3000, 1, 512)), cmp=T((2, 700, 1, 512)), obt=None, cbt=None), 0),
    (dict(layout_kv=b"BSND", ori=T((3, 3000, 1, 512)), cmp=T((2, 700, 1, 512)), obt=None, cbt=None), BAD),
    (dict(layout_kv=b"BSND", ori=T((2, 3000, 1, 512)), cmp=T((2, 700, 1, 512))), BAD),   # no tables
    (dict(layout_kv=b"TND"), BAD),                            # TND KV needs TND q
    (dict(layout_q=b"TND", layout_kv=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)),
          lse=T((1, 5, 64), F32), idx=T((5, 1, 512), I32), cuq=T((3,), I32),
          ori=T((4000, 1, 512)), cmp=T((1000, 1, 512)), obt=None, cbt=None,
          cuo=T((3,), I32), cuc=T((3,), I32)), 0),
    (dict(layout_q=b"TND", layout_kv=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)),
          lse=T((1, 5, 64), F32), idx=T((5, 1, 512), I32), cuq=T((3,), I32),
          ori=T((4000, 1, 512)), cmp=T((1000, 1, 512)), obt=None, cbt=None,
          cuo=T((3,), I32)), BAD),                            # cu_seqlens_cmp_kv missing
    (dict(layout_q=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)), lse=T((1, 5, 64), F32),
          idx=T((5, 1, 512), I32), cuq=T((3,), I32)), 0),     # TND q, PA_BBND KV
    (dict(layout_q=b"TND", q=T((5, 64, 512)), out=T((5, 64, 512)), lse=T((2, 1, 5, 64), F32),
          idx=T((5, 1, 512), I32), cuq=T((3,), I32)), BAD),   # LSE [1, T1, N1] with TND
    (dict(cuo=T((3,), I32)), BAD),                            # cu_seqlens_ori_kv only with TND KV
])
def test_sfmla_phase1(over, expect):
    st, msg, _ = sfmla_plan_status(**over)
    assert st == expect, (over, msg)


def test_sfmla_workspace():
    """Partials only when a query row spans several chunks of 128 slots: the
    window alone (SWA) needs no workspace, CSA with K2 = 512 does."""
    st, msg, ws = sfmla_plan_status(cmp=None, idx=None, cbt=None, cmp_ratio=1, cmp_mask_mode=0)
    assert st == 0 and ws == 0, msg
    st, msg, ws = sfmla_plan_status()
    assert st == 0 and ws >= 2 * 64 * 5 * 512 * 4, msg


def test_device_kv_lengths_phase1():
    """KV lengths on the device (decode only): int32 [B] tensor plus a host
    bound that sizes the grid and the workspace."""
    i32 = fia.DT_INT32
    q, k, v, o = dense(S1=1, S2=3000)
    st, kind, ws, msg = plan(P(num_kv_heads=2, dev_lens=T((2,), i32), len_bound=3000), q, k, v, o)
    assert st == 0 and kind == "decode" and ws > 0, msg
    # the workspace grows with the bound (one chunk list and partials per bound chunk)
    st2, _, ws2, msg = plan(P(num_kv_heads=2, dev_lens=T((2,), i32), len_bound=600), q, k, v, o)
    assert st2 == 0 and ws2 < ws, msg
    cases = [
        (dict(dev_lens=T((2,), i32), len_bound=3001), BAD),            # above KV_S
        (dict(dev_lens=T((2,), i32), len_bound=-1), BAD),
        (dict(dev_lens=T((3,), i32), len_bound=100), BAD),             # not [B]
        (dict(dev_lens=T((2,), fia.DT_INT64), len_bound=100), BAD),
        (dict(dev_lens=T((2,), i32), len_bound=100, actual_seq_lengths_kv=[5, 6]), BAD),
    ]
    for kw, expect in cases:
        st, _, _, msg = plan(P(num_kv_heads=2, **kw), q, k, v, o)
        assert st == expect, (kw, msg)
    # query length > 1: a prompt whose items are planned for the bound (no
    # workspace); ALiBi is not taken (its equal-length rule needs the lengths)
    q2, k2, v2, o2 = dense(S1=4, S2=3000)
    st, kind, ws, msg = plan(P(num_kv_heads=2, dev_lens=T((2,), i32), len_bound=100), q2, k2, v2, o2)
    assert st == 0 and kind == "prefill" and ws == 0, msg
    q4, k4, v4, o4 = dense(S1=3000, S2=3000)
    st, _, _, msg = plan(P(num_kv_heads=2, dev_lens=T((2,), i32), len_bound=3000, pse_type=2), q4, k4,
                         v4, o4, pse=T((4,), fia.DT_FP32))
    assert st == UNS and "ALiBi" in msg, msg
    # fp32 inputs are not taken
    q3, k3, v3, o3 = dense(S1=1, S2=300, D=64, dt=fia.DT_FP32)
    st, _, _, msg = plan(P(num_kv_heads=2, dev_lens=T((2,), i32), len_bound=100), q3, k3, v3, o3)
    assert st == UNS, msg
    # paged: the bound must fit the block table
    qp = T((2, 1, 4, 128))
    pool = T((40, 128, 2, 128))
    bt = T((2, 8), i32)
    st, kind, _, msg = plan(P(num_kv_heads=2, block_size=128, dev_lens=T((2,), i32), len_bound=1024),
                            qp, pool, pool, qp, bt=bt)
    assert st == 0 and kind == "decode", msg
    st, _, _, msg = plan(P(num_kv_heads=2, block_size=128, dev_lens=T((2,), i32), len_bound=1025),
                         qp, pool, pool, qp, bt=bt)
    assert st == BAD, msg


def _executor(p, q, k, v, out, bt=None):
    ws = ctypes.c_size_t(0)
    ex = ctypes.c_void_p(None)
    ptr = lambda d: ctypes.pointer(d) if d is not None else None
    st = fia.lib().fia_get_workspace_size(ctypes.byref(p), ptr(q), ptr(k), ptr(v), None, None,
                                          ptr(bt), ptr(out), None, ctypes.byref(ws), ctypes.byref(ex))
    assert st == 0, fia.lib().fia_last_error().decode()
    return ex


def _read_len(ex, order):
    n = ctypes.c_int64(-7)
    st = fia.lib().fia_debug_read_kv(ex, None, 0, order, None, ctypes.byref(n), None)
    return st, n.value


def test_decode_read_probe_sizes():
    """fia_debug_read_kv without an output only reports how many words it
    would write (no device access): chunks x KV heads for order 0, chunks x 8
    for order 1, and refuses shapes and executors it has no form for."""
    lens = dict(actual_seq_lengths_kv=[1000, 2048, 3000])   # 1 + 2 + 3 chunks of 1024 keys
    q, o = T((3, 1, 32, 128)), T((3, 1, 32, 128))
    bt = T((3, 24), fia.DT_INT32)
    ex = _executor(P(num_heads=32, num_kv_heads=4, block_size=128, **lens), q,
                   T((80, 128, 4, 128)), T((80, 128, 4, 128)), o, bt=bt)
    try:
        assert _read_len(ex, 0) == (0, 6 * 4)
        assert _read_len(ex, 1) == (0, 6 * 8)       # 4 heads x 256 B = 1 KB token rows
        assert _read_len(ex, 2)[0] == BAD
        assert fia.lib().fia_debug_read_kv(ex, None, 0, 0, None, None, None) == fia.FIA_ERR_NULLPTR
        small = ctypes.c_int64(3)
        assert fia.lib().fia_debug_read_kv(ex, None, 0, 0, ctypes.c_void_p(16), ctypes.byref(small),
                                           None) == BAD
    finally:
        fia.lib().fia_executor_destroy(ex)
    # BnNBsD: a head's rows are contiguous, a token's heads are not
    ex = _executor(P(num_heads=32, num_kv_heads=4, block_size=128, kv_layout="BnNBsD", **lens), q,
                   T((80, 4, 128, 128)), T((80, 4, 128, 128)), o, bt=bt)
    try:
        assert _read_len(ex, 0) == (0, 6 * 4)
        assert _read_len(ex, 1)[0] == UNS
    finally:
        fia.lib().fia_executor_destroy(ex)
    # D = 64 bf16: 128-byte head rows, 512-byte token rows (order 1 has no form)
    q64, o64 = T((3, 1, 32, 64)), T((3, 1, 32, 64))
    ex = _executor(P(num_heads=32, num_kv_heads=4, block_size=128, **lens), q64,
                   T((80, 128, 4, 64)), T((80, 128, 4, 64)), o64, bt=bt)
    try:
        assert _read_len(ex, 0) == (0, 6 * 4)
        assert _read_len(ex, 1)[0] == UNS
    finally:
        fia.lib().fia_executor_destroy(ex)
    # not a decode executor
    qp, kp, vp, op = dense()
    ex = _executor(P(num_kv_heads=2, sparse_mode=3), qp, kp, vp, op)
    try:
        assert _read_len(ex, 0)[0] == BAD
    finally:
        fia.lib().fia_executor_destroy(ex)
