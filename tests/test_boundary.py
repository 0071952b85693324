"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/fia.h declares, and phase 1 validates inputs with the
status codes the header documents (constraints of the fused-infer-attention
and block-sparse pages).  Phase 1 never launches or reads device data, so
CPU tensors stand in for device tensors here."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import attention_fia_fwd_amd as fia
from attention_fia_fwd_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INT_MAX = 2147483647


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            for m in re.finditer(r"^[\w\s\*]*?\b(\w+)\s*\([^;{]*\)\s*;", src, flags=re.M):
                if m.group(1) not in ("if", "while", "sizeof"):
                    names.add(m.group(1))
    return names


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(_abi.LIB_PATH):
        fia.build()


def test_header_declares_the_two_phase_api():
    names = declared_functions()
    for n in ["fia_get_workspace_size", "fia_run", "bsa_get_workspace_size", "bsa_run",
              "fia_plan_destroy", "fia_status_string", "fia_params_init", "bsa_params_init",
              "bsa_schedule_layout"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _abi.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing


def test_status_strings():
    for s in range(9):
        assert fia.fia_status_string(s).startswith(["FIA_OK", "FIA_ERR"][s > 0])


def _params(**kw):
    p = fia.fia_params()
    fia.fia_params_init(p)
    layout = kw.pop("input_layout", "BNSD").encode()
    p.input_layout = layout
    for k, v in kw.items():
        setattr(p, k, v)
    p._layout_ref = layout
    return p


def _phase1(q, k, v, p, out=None, lse=None, mask=None, bt=None):
    keep = [q, k, v, out, lse, mask, bt]
    dq = fia.describe(q)
    o = out if out is not None else torch.zeros(*q.shape[:-1], v.shape[-1], dtype=q.dtype)
    keep.append(o)
    st, ws, plan = fia.fia_get_workspace_size(dq, fia.describe(k), fia.describe(v),
                                              fia.describe(mask), fia.describe(bt), p,
                                              fia.describe(o), fia.describe(lse))
    fia.fia_plan_destroy(plan)
    return st, ws


def test_defaults_of_params_init():
    p = fia.fia_params()
    fia.fia_params_init(p)
    assert p.input_layout == b"BSH" and p.scale_value == 1.0
    assert p.pre_tokens == INT_MAX and p.next_tokens == INT_MAX
    assert p.sparse_mode == 0 and p.block_size == 0 and p.return_softmax_lse == 0
    b = fia.bsa_params()
    fia.bsa_params_init(b)
    assert tuple(b.block_shape) == (128, 128) and b.inner_precise == 4


def test_valid_prefill_plan_and_workspace():
    q = torch.zeros(2, 4, 300, 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 2, 300, 128, dtype=torch.bfloat16)
    st, ws = _phase1(q, k, k, _params(num_heads=4, num_key_value_heads=2, sparse_mode=3))
    assert st == _abi.FIA_OK
    assert ws == 0          # prefill keeps its schedule in the plan, needs no scratch


@pytest.mark.parametrize("case, code", [
    ("kdtype", _abi.FIA_ERR_DTYPE),
    ("f32", _abi.FIA_ERR_DTYPE),
    ("layout", _abi.FIA_ERR_LAYOUT),
    ("variant_layout", _abi.FIA_ERR_UNSUPPORTED),
    ("gqa_indivisible", _abi.FIA_ERR_PARAM),
    ("gqa_ratio", _abi.FIA_ERR_PARAM),
    ("mode5", _abi.FIA_ERR_PARAM),
    ("mode1_no_mask", _abi.FIA_ERR_NULLPTR),
    ("template_shape", _abi.FIA_ERR_SHAPE),
    ("mask_dtype", _abi.FIA_ERR_DTYPE),
    ("heads_mismatch", _abi.FIA_ERR_SHAPE),
    ("len_too_long", _abi.FIA_ERR_SHAPE),
    ("len_count", _abi.FIA_ERR_PARAM),
    ("lse_missing", _abi.FIA_ERR_NULLPTR),
    ("lse_shape", _abi.FIA_ERR_SHAPE),
    ("head_dim", _abi.FIA_ERR_UNSUPPORTED),
    ("inner_precise", _abi.FIA_ERR_PARAM),
])
def test_prefill_validation_codes(case, code):
    B, N, S, D = 2, 4, 64, 128
    q = torch.zeros(B, N, S, D, dtype=torch.bfloat16)
    k = torch.zeros(B, 2, S, D, dtype=torch.bfloat16)
    v = k
    kw = dict(num_heads=N, num_key_value_heads=2, sparse_mode=3)
    mask = lse = None
    layout = "BNSD"
    if case == "kdtype":
        k = k.to(torch.float16)
    elif case == "f32":
        q, k, v = q.float(), k.float(), v.float()
    elif case == "layout":
        layout = "SBH"
    elif case == "variant_layout":
        layout = "BNSD_BSND"
    elif case == "gqa_indivisible":
        kw["num_key_value_heads"] = 3
    elif case == "gqa_ratio":
        q = torch.zeros(B, 128, S, D, dtype=torch.bfloat16)
        k = v = torch.zeros(B, 1, S, D, dtype=torch.bfloat16)
        kw.update(num_heads=128, num_key_value_heads=1)
        q = q[:, :, :1]  # keep it small: the ratio check comes first
        q = torch.zeros(B, 128, 2, D, dtype=torch.bfloat16)
        k = v = torch.zeros(B, 1, 2, D, dtype=torch.bfloat16)
    elif case == "mode5":
        kw["sparse_mode"] = 5
    elif case == "mode1_no_mask":
        kw["sparse_mode"] = 1
    elif case == "template_shape":
        mask = torch.zeros(1024, 1024, dtype=torch.uint8)
    elif case == "mask_dtype":
        kw["sparse_mode"] = 1
        mask = torch.zeros(S, S, dtype=torch.float32)
    elif case == "heads_mismatch":
        kw["num_heads"] = 8
    elif case == "len_too_long":
        arr = np.array([64, 65], dtype=np.int64)
        kw["actual_seq_qlen"] = arr.ctypes.data
        kw["n_actual_seq_qlen"] = 2
        kw["_keep"] = arr
    elif case == "len_count":
        arr = np.array([64, 65, 3], dtype=np.int64)[:2]
        arr = np.ascontiguousarray(arr)
        kw["actual_seq_qlen"] = arr.ctypes.data
        kw["n_actual_seq_qlen"] = 0
        kw["_keep"] = arr
        # count 0 with a pointer: neither 1 nor >= B
    elif case == "lse_missing":
        kw["return_softmax_lse"] = 1
    elif case == "lse_shape":
        kw["return_softmax_lse"] = 1
        lse = torch.zeros(B, N, S, dtype=torch.float32)
    elif case == "head_dim":
        q = torch.zeros(B, N, S, 96, dtype=torch.bfloat16)
        k = v = torch.zeros(B, 2, S, 96, dtype=torch.bfloat16)
    elif case == "inner_precise":
        kw["inner_precise"] = 4
    keep = kw.pop("_keep", None)
    p = _params(input_layout=layout, **kw)
    st, _ = _phase1(q, k, v, p, lse=lse, mask=mask)
    assert st == code, (case, fia.fia_status_string(st))


def test_paged_decode_validation():
    B, QN, KVN, D, bs = 2, 8, 2, 128, 16
    lkv = np.array([40, 17], dtype=np.int64)
    nblk = 3 + 2
    q = torch.zeros(B, QN, 1, D, dtype=torch.bfloat16)
    pool = torch.zeros(nblk, KVN, bs, D, dtype=torch.bfloat16)
    bt = torch.zeros(B, 3, dtype=torch.int32)

    def run(pool=pool, bt=bt, lkv=lkv, block_size=bs, q=q):
        p = _params(num_heads=QN, num_key_value_heads=KVN, block_size=block_size)
        if lkv is not None:
            p.actual_seq_kvlen = lkv.ctypes.data
            p.n_actual_seq_kvlen = lkv.size
        return _phase1(q, pool, pool, p, bt=bt)[0]

    assert run() == _abi.FIA_OK
    assert run(block_size=8) == _abi.FIA_ERR_PARAM
    assert run(lkv=None) == _abi.FIA_ERR_PARAM
    assert run(bt=torch.zeros(B, 2, dtype=torch.int32)) == _abi.FIA_ERR_SHAPE
    assert run(bt=torch.zeros(B, 3, dtype=torch.int64)) == _abi.FIA_ERR_DTYPE
    assert run(pool=torch.zeros(4, KVN, bs, D, dtype=torch.bfloat16)) == _abi.FIA_ERR_SHAPE
    # query S > 1 (paged prefill, multi-token decode): block_size a multiple
    # of 128 in [128, 512]
    q2 = torch.zeros(B, QN, 4, D, dtype=torch.bfloat16)
    assert run(q=q2) == _abi.FIA_ERR_PARAM
    for bs2, code in ((128, _abi.FIA_OK), (384, _abi.FIA_OK), (512, _abi.FIA_OK),
                      (64, _abi.FIA_ERR_PARAM), (640, _abi.FIA_ERR_PARAM)):
        pool2 = torch.zeros(nblk, KVN, bs2, D, dtype=torch.bfloat16)
        assert run(q=q2, pool=pool2, block_size=bs2, bt=torch.zeros(B, 1, dtype=torch.int32)) == code, bs2
    # a TND query with a paged cache (TND constraints): block_size 128, 512
    # or 1024, cumulative actual_seq_kvlen, one table row per sequence
    cq = np.array([3, 7], dtype=np.int64)
    ckv = np.array([40, 57], dtype=np.int64)          # kv lengths 40 and 17

    def tnd(bs3, ckv=ckv, rows=B, cols=1, mode=3):
        p = _params(input_layout="TND", num_heads=QN, num_key_value_heads=KVN, block_size=bs3,
                    sparse_mode=mode)
        p.actual_seq_qlen, p.n_actual_seq_qlen = cq.ctypes.data, 2
        p.actual_seq_kvlen, p.n_actual_seq_kvlen = ckv.ctypes.data, 2
        qt = torch.zeros(7, QN, D, dtype=torch.bfloat16)
        pool3 = torch.zeros(nblk, KVN, bs3, D, dtype=torch.bfloat16)
        return _phase1(qt, pool3, pool3, p, bt=torch.zeros(rows, cols, dtype=torch.int32))[0]

    for bs3, code in ((128, _abi.FIA_OK), (512, _abi.FIA_OK), (1024, _abi.FIA_OK),
                      (256, _abi.FIA_ERR_PARAM), (384, _abi.FIA_ERR_PARAM), (64, _abi.FIA_ERR_PARAM)):
        assert tnd(bs3) == code, bs3
    assert tnd(128, mode=0) == _abi.FIA_OK
    assert tnd(128, rows=3) == _abi.FIA_ERR_SHAPE                       # rows != sequences
    assert tnd(128, ckv=np.array([40, 30], dtype=np.int64)) == _abi.FIA_ERR_SHAPE   # not cumulative
    assert tnd(128, ckv=np.array([40, 300], dtype=np.int64)) == _abi.FIA_ERR_SHAPE  # 260 > 1 block


def test_decode_atten_mask_validation():
    B, QN, KVN, S, D = 2, 8, 2, 40, 128
    q = torch.zeros(B, QN, 1, D, dtype=torch.bfloat16)
    k = torch.zeros(B, KVN, S, D, dtype=torch.bfloat16)
    p = _params(num_heads=QN, num_key_value_heads=KVN, input_layout="BNSD")

    def code(mask):
        return _phase1(q, k, k, p, mask=mask)[0]

    for shape in ((B, S), (B, 1, S), (B, 1, 1, S), (1, S), (B, S + 24)):
        assert code(torch.zeros(shape, dtype=torch.uint8)) == _abi.FIA_OK, shape
    assert code(torch.zeros(B, 1, 1, S, dtype=torch.bool)) == _abi.FIA_OK
    assert code(torch.zeros(B, 2, S, dtype=torch.uint8)) == _abi.FIA_ERR_SHAPE
    assert code(torch.zeros(B, S - 1, dtype=torch.uint8)) == _abi.FIA_ERR_SHAPE
    assert code(torch.zeros(3, S, dtype=torch.uint8)) == _abi.FIA_ERR_SHAPE
    assert code(torch.zeros(B, S, dtype=torch.float16)) == _abi.FIA_ERR_DTYPE


def test_int8_kv_validation():
    B, QN, KVN, S, D = 2, 8, 2, 40, 128
    q = torch.zeros(B, QN, 1, D, dtype=torch.bfloat16)
    k8 = torch.zeros(B, KVN, S, D, dtype=torch.int8)
    ch = torch.ones(KVN, D, dtype=torch.bfloat16)
    tok = torch.ones(B, S, dtype=torch.float32)

    def code(q=q, k=k8, ks=ch, vs=ch, ko=None, vo=None, km=0, vm=0, bt=None, block_size=0,
             mode=0):
        p = _params(num_heads=QN, num_key_value_heads=KVN, input_layout="BNSD",
                    block_size=block_size, sparse_mode=mode)
        keep = []
        for fld, t in (("dequant_scale_key", ks), ("dequant_scale_value", vs),
                       ("dequant_offset_key", ko), ("dequant_offset_value", vo)):
            if t is not None:
                d = fia.describe(t)
                keep.append((t, d))
                setattr(p, fld, ctypes.pointer(d))
        p.key_quant_mode, p.value_quant_mode = km, vm
        if bt is not None:
            lk = np.array([S, S], dtype=np.int64)
            keep.append(lk)
            p.actual_seq_kvlen, p.n_actual_seq_kvlen = lk.ctypes.data, 2
        return _phase1(q, k, k, p, bt=bt, out=torch.zeros(q.shape, dtype=torch.bfloat16))[0]

    assert code() == _abi.FIA_OK
    assert code(ks=tok, vs=tok, km=1, vm=1) == _abi.FIA_OK
    assert code(vs=tok, vm=1, ko=ch) == _abi.FIA_OK
    assert code(ks=ch.reshape(-1), vs=ch.reshape(-1)) == _abi.FIA_OK
    assert code(q=q.half()) == _abi.FIA_ERR_DTYPE                 # query must be bf16
    assert code(ks=None) == _abi.FIA_ERR_NULLPTR
    # mode pairs (key_quant_mode description): equal, or key 0 with value 1
    assert code(km=2) == _abi.FIA_ERR_PARAM
    assert code(ks=tok, km=1) == _abi.FIA_ERR_PARAM               # key 1 with value 0
    assert code(km=6, vm=6) == _abi.FIA_ERR_PARAM
    assert code(km=-1, vm=-1) == _abi.FIA_ERR_PARAM
    # per tensor / per head, and scales managed by page attention: legal at
    # query S 1, not provided
    for m in (2, 3, 4, 5):
        assert code(km=m, vm=m) == _abi.FIA_ERR_UNSUPPORTED, m
    assert code(ks=ch.float()) == _abi.FIA_ERR_DTYPE              # per channel: bf16
    assert code(ks=tok.to(torch.bfloat16), vs=tok, km=1, vm=1) == _abi.FIA_ERR_DTYPE
    assert code(ks=torch.ones(KVN, D + 1, dtype=torch.bfloat16)) == _abi.FIA_ERR_SHAPE
    assert code(ks=torch.ones(B, S - 1), vs=tok, km=1, vm=1) == _abi.FIA_ERR_SHAPE
    assert code(ks=tok, vs=torch.ones(B, S + 3), km=1, vm=1) == _abi.FIA_ERR_SHAPE
    assert code(ko=torch.ones(KVN, D)) == _abi.FIA_ERR_SHAPE      # offset: its scale's dtype
    # page attention with an int8 cache at query S 1 (block size 32-aligned),
    # either pool layout; per-token scales cover the longest kv length
    bt = torch.zeros(B, 2, dtype=torch.int32)
    for pool in (torch.zeros(4, KVN, 32, D, dtype=torch.int8), torch.zeros(4, 32, KVN * D, dtype=torch.int8)):
        assert code(k=pool, bt=bt, block_size=32) == _abi.FIA_OK
        assert code(k=pool, bt=bt, block_size=32, ks=tok, vs=tok, km=1, vm=1) == _abi.FIA_OK
        assert code(k=pool, bt=bt, block_size=32, vs=tok, vm=1) == _abi.FIA_OK
        assert code(k=pool, bt=bt, block_size=32, ks=tok[:, :S - 1].contiguous(), vs=tok[:, :S - 1].contiguous(),
                    km=1, vm=1) == _abi.FIA_ERR_SHAPE
    pool16 = torch.zeros(6, KVN, 16, D, dtype=torch.int8)
    assert code(k=pool16, bt=torch.zeros(B, 3, dtype=torch.int32), block_size=16) == _abi.FIA_ERR_PARAM
    # query S <= 16; G * S > 16 is not provided
    assert code(q=torch.zeros(B, QN, 17, D, dtype=torch.bfloat16), mode=3) == _abi.FIA_ERR_PARAM
    assert code(q=torch.zeros(B, QN, 5, D, dtype=torch.bfloat16), mode=3) == _abi.FIA_ERR_UNSUPPORTED
    q2 = torch.zeros(B, QN, 2, D, dtype=torch.bfloat16)
    assert code(q=q2, mode=3) == _abi.FIA_OK
    assert code(q=q2, ks=tok, vs=tok, km=1, vm=1, mode=3) == _abi.FIA_OK
    # query S > 1: modes equal (key 0 with value 1 is a query S 1 exception),
    # 0 or 1 only, and no page attention
    assert code(q=q2, vs=tok, vm=1, mode=3) == _abi.FIA_ERR_PARAM
    assert code(q=q2, km=2, vm=2, mode=3) == _abi.FIA_ERR_PARAM
    pool128 = torch.zeros(2, KVN, 128, D, dtype=torch.int8)
    assert code(q=q2, k=pool128, bt=torch.zeros(B, 1, dtype=torch.int32), block_size=128,
                mode=3) == _abi.FIA_ERR_PARAM
    # equal modes: one shape for the two scales
    assert code(vs=ch.reshape(-1)) == _abi.FIA_ERR_SHAPE
    # dequant tensors with fp16/bf16 key/value
    kb = torch.zeros(B, KVN, S, D, dtype=torch.bfloat16)
    assert code(k=kb) == _abi.FIA_ERR_PARAM


def test_bsa_fp8_validation():
    B, N1, N2, S, D = 1, 4, 2, 512, 128
    f8 = torch.float8_e4m3fn
    q = torch.zeros(B, N1, S, D, dtype=f8)
    k = torch.zeros(B, N2, S, D, dtype=f8)
    out = torch.zeros(B, N1, S, D, dtype=torch.bfloat16)

    def code(Y=256, X=128, qs=None, ks=None, vs=None, out=out, k=k, scales=True):
        nqb, nkb = -(-S // X), -(-S // Y)
        mask = torch.ones(B, N1, nqb, nkb, dtype=torch.uint8)
        qs = torch.ones(B, N1, nqb, 1) if qs is None else qs
        ks = torch.ones(B, N2, nkb, 1) if ks is None else ks
        vs = torch.ones(B, N2, nkb, 1) if vs is None else vs
        p = fia.bsa_params()
        fia.bsa_params_init(p)
        p.num_heads, p.num_key_value_heads = N1, N2
        p.block_shape[0], p.block_shape[1] = X, Y
        keep = []
        if scales:
            for fld, t in (("dequant_scale_query", qs), ("dequant_scale_key", ks),
                           ("dequant_scale_value", vs)):
                if t is not None:
                    d = fia.describe(t)
                    keep.append((t, d))
                    setattr(p, fld, ctypes.pointer(d))
        st, ws, plan = fia.bsa_get_workspace_size(fia.describe(q), fia.describe(k), fia.describe(k),
                                                  fia.describe(mask), None, None, p,
                                                  fia.describe(out), None)
        fia.fia_plan_destroy(plan)
        return st

    assert code() == _abi.FIA_OK
    assert code(Y=512) == _abi.FIA_OK
    assert code(Y=128) == _abi.FIA_ERR_PARAM              # kv quant blocks of 256 or 512
    assert code(X=256, Y=256) == _abi.FIA_ERR_PARAM
    assert code(scales=False) == _abi.FIA_ERR_NULLPTR
    assert code(qs=torch.ones(B, N1, 4, 1, dtype=torch.float16)) == _abi.FIA_ERR_DTYPE
    assert code(ks=torch.ones(B, N2, 3, 1)) == _abi.FIA_ERR_SHAPE
    assert code(out=out.half()) == _abi.FIA_ERR_DTYPE        # bf16 output
    assert code(k=k.to(torch.bfloat16)) == _abi.FIA_ERR_DTYPE  # all three E4M3FN


def test_tnd_requires_cumulative_lengths():
    q = torch.zeros(30, 4, 128, dtype=torch.bfloat16)
    k = torch.zeros(30, 4, 128, dtype=torch.bfloat16)
    p = _params(input_layout="TND", num_heads=4, sparse_mode=3)
    assert _phase1(q, k, k, p)[0] == _abi.FIA_ERR_PARAM
    bad = np.array([10, 5], dtype=np.int64)       # decreasing
    p.actual_seq_qlen, p.n_actual_seq_qlen = bad.ctypes.data, 2
    p.actual_seq_kvlen, p.n_actual_seq_kvlen = bad.ctypes.data, 2
    assert _phase1(q, k, k, p)[0] == _abi.FIA_ERR_SHAPE
    good = np.array([10, 30], dtype=np.int64)
    p.actual_seq_qlen, p.actual_seq_kvlen = good.ctypes.data, good.ctypes.data
    assert _phase1(q, k, k, p)[0] == _abi.FIA_OK
    p.sparse_mode = 1
    assert _phase1(q, k, k, p)[0] == _abi.FIA_ERR_PARAM


def test_empty_query_is_ok_with_zero_workspace():
    q = torch.zeros(2, 4, 0, 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 4, 8, 128, dtype=torch.bfloat16)
    st, ws = _phase1(q, k, k, _params(num_heads=4))
    assert st == _abi.FIA_OK and ws == 0


def test_run_rejects_small_workspace_without_touching_the_gpu():
    # decode needs scratch for its split partial results
    B, QN, KVN, D = 2, 8, 2, 128
    q = torch.zeros(B, QN, 1, D, dtype=torch.bfloat16)
    k = torch.zeros(B, KVN, 5000, D, dtype=torch.bfloat16)
    p = _params(num_heads=QN, num_key_value_heads=KVN)
    o = torch.zeros_like(q)
    st, ws, plan = fia.fia_get_workspace_size(fia.describe(q), fia.describe(k), fia.describe(k),
                                              None, None, p, fia.describe(o), None)
    assert st == _abi.FIA_OK and ws > 0 and ws % 256 == 0
    assert fia.fia_run(0, 0, plan, 0) == _abi.FIA_ERR_WORKSPACE
    assert fia.fia_run(1 << 20, ws - 1, plan, 0) == _abi.FIA_ERR_WORKSPACE
    # a fused-attention plan is not a block-sparse plan
    assert fia.bsa_run(1 << 20, ws, plan, 0) == _abi.FIA_ERR_PARAM
    fia.fia_plan_destroy(plan)


def test_run_noalloc_status_codes_without_a_gpu():
    # the allocation-free run refuses a NULL plan, and a plan whose
    # workspace exceeds the static scratch before it touches any device
    import workloads as W
    assert fia.fia_run_noalloc(0, 0) == _abi.FIA_ERR_NULLPTR
    case = W.make_mla_decode("noalloc_cpu", B=64, QN=128, Sq=1, lkv=[600] * 64, block_size=128, seed=1)
    p = _params(num_heads=128, num_key_value_heads=1, input_layout=case.layout, block_size=128)
    kl = np.asarray(case.lkv, dtype=np.int64)
    p.actual_seq_kvlen, p.n_actual_seq_kvlen = kl.ctypes.data, len(kl)
    qr, kr = fia.describe(case.rope["query_rope"]), fia.describe(case.rope["key_rope"])
    p.query_rope, p.key_rope = ctypes.pointer(qr), ctypes.pointer(kr)
    o = torch.zeros_like(case.q)
    st, ws, plan = fia.fia_get_workspace_size(fia.describe(case.q), fia.describe(case.k),
                                              fia.describe(case.v), None, fia.describe(case.block_table),
                                              p, fia.describe(o), None)
    assert st == _abi.FIA_OK and ws > _abi.FIA_NOALLOC_MAX_WORKSPACE
    assert fia.fia_run_noalloc(plan, 0) == _abi.FIA_ERR_WORKSPACE
    fia.fia_plan_destroy(plan)


def test_run_without_a_device_at_phase1_fails_without_allocating():
    # phase 1 with no device visible validates and sizes but uploads no
    # schedule; phase 2 then returns FIA_ERR_HIP instead of allocating
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is visible: phase 1 uploads the schedule")
    B, QN, KVN, D = 2, 8, 2, 128
    q = torch.zeros(B, QN, 1, D, dtype=torch.bfloat16)
    k = torch.zeros(B, KVN, 5000, D, dtype=torch.bfloat16)
    p = _params(num_heads=QN, num_key_value_heads=KVN)
    o = torch.zeros_like(q)
    st, ws, plan = fia.fia_get_workspace_size(fia.describe(q), fia.describe(k), fia.describe(k),
                                              None, None, p, fia.describe(o), None)
    assert st == _abi.FIA_OK and ws > 0
    assert fia.fia_run(1 << 20, ws, plan, 0) == _abi.FIA_ERR_HIP
    fia.fia_plan_destroy(plan)


def _bsa_phase1(q, k, v, m, **kw):
    p = fia.bsa_params()
    fia.bsa_params_init(p)
    lay = kw.pop("layout", "BNSD").encode()
    p.q_input_layout = p.kv_input_layout = lay
    for key, val in kw.items():
        setattr(p, key, val)
    o = torch.zeros_like(q)
    st, ws, plan = fia.bsa_get_workspace_size(fia.describe(q), fia.describe(k), fia.describe(v),
                                              fia.describe(m), None, None, p, fia.describe(o),
                                              None)
    fia.fia_plan_destroy(plan)
    return st, ws


def test_bsa_validation():
    q = torch.zeros(1, 4, 300, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 260, 128, dtype=torch.bfloat16)
    m = torch.zeros(1, 4, 3, 3, dtype=torch.uint8)
    assert _bsa_phase1(q, k, k, m, num_heads=4, num_key_value_heads=2)[0] == _abi.FIA_OK
    assert _bsa_phase1(q, k, k, torch.zeros(1, 4, 3, 2, dtype=torch.uint8), num_heads=4,
                       num_key_value_heads=2)[0] == _abi.FIA_ERR_SHAPE
    for field, val, code in [("inner_precise", 0, _abi.FIA_ERR_PARAM),
                             ("mask_type", 1, _abi.FIA_ERR_PARAM),
                             ("pre_tokens", 5, _abi.FIA_ERR_PARAM),
                             ("num_key_value_heads", 3, _abi.FIA_ERR_PARAM)]:
        kw = dict(num_heads=4, num_key_value_heads=2)
        kw[field] = val
        assert _bsa_phase1(q, k, k, m, **kw)[0] == code, field
    # a head dim outside {64, 128}
    p_shape = dict(num_heads=4, num_key_value_heads=2)
    q2 = torch.zeros(1, 4, 300, 96, dtype=torch.bfloat16)
    k2 = torch.zeros(1, 2, 260, 96, dtype=torch.bfloat16)
    assert _bsa_phase1(q2, k2, k2, m, **p_shape)[0] == _abi.FIA_ERR_UNSUPPORTED


def test_mla_validation():
    # MLA (query_rope / key_rope): query D 512 + rope 64, one kv head, paged
    # pool with block_size 16 or 128, query S <= 16, Q_N a power of two <= 128
    B, QN, bs, D = 2, 16, 128, 512
    pool = torch.zeros(4, bs, D, dtype=torch.bfloat16)
    kr = torch.zeros(4, bs, 64, dtype=torch.bfloat16)
    bt = torch.zeros(B, 2, dtype=torch.int32)

    def code(S=1, qn=QN, q=None, qr=None, k=pool, krope=kr, block_size=bs, mode=0, layout="BNSD",
             table=bt, mask=None, kvn=1, give=(True, True)):
        if q is None:
            q = torch.zeros(B, qn, S, D, dtype=torch.bfloat16)
        if qr is None:
            qr = torch.zeros(*q.shape[:-1], 64, dtype=q.dtype)
        p = _params(num_heads=qn, num_key_value_heads=kvn, input_layout=layout,
                    block_size=block_size, sparse_mode=mode)
        keep = [qr, krope]
        dq, dk = fia.describe(qr), fia.describe(krope)
        keep += [dq, dk]
        if give[0]:
            p.query_rope = ctypes.pointer(dq)
        if give[1]:
            p.key_rope = ctypes.pointer(dk)
        lk = np.array([200, 7], dtype=np.int64)
        keep.append(lk)
        p.actual_seq_kvlen, p.n_actual_seq_kvlen = lk.ctypes.data, 2
        out = torch.zeros(*q.shape[:-1], D, dtype=q.dtype)
        return _phase1(q, k, k, p, out=out, bt=table, mask=mask)[0]

    assert code() == _abi.FIA_OK
    assert code(qn=128) == _abi.FIA_OK
    tmpl = torch.triu(torch.ones(2048, 2048, dtype=torch.uint8), diagonal=1)
    assert code(S=4, mode=3, mask=tmpl) == _abi.FIA_OK
    assert code(k=torch.zeros(4, 1, bs, D, dtype=torch.bfloat16),
                krope=torch.zeros(4, 1, bs, 64, dtype=torch.bfloat16)) == _abi.FIA_OK
    assert code(give=(True, False)) == _abi.FIA_ERR_PARAM           # both or neither
    assert code(give=(False, True)) == _abi.FIA_ERR_PARAM
    assert code(qr=torch.zeros(B, QN, 1, 64, dtype=torch.float16)) == _abi.FIA_ERR_DTYPE
    assert code(qr=torch.zeros(B, QN, 1, 32, dtype=torch.bfloat16)) == _abi.FIA_ERR_SHAPE
    assert code(krope=torch.zeros(4, bs, 32, dtype=torch.bfloat16)) == _abi.FIA_ERR_SHAPE
    assert code(krope=torch.zeros(3, bs, 64, dtype=torch.bfloat16)) == _abi.FIA_ERR_SHAPE
    assert code(block_size=32, k=torch.zeros(8, 32, D, dtype=torch.bfloat16),
                krope=torch.zeros(8, 32, 64, dtype=torch.bfloat16)) == _abi.FIA_ERR_PARAM
    assert code(block_size=64, k=torch.zeros(8, 64, D, dtype=torch.bfloat16),
                krope=torch.zeros(8, 64, 64, dtype=torch.bfloat16),
                table=torch.zeros(B, 4, dtype=torch.int32)) == _abi.FIA_OK
    assert code(table=None, block_size=0, k=torch.zeros(B, 1, 200, D, dtype=torch.bfloat16),
                krope=torch.zeros(B, 1, 200, 64, dtype=torch.bfloat16)) == _abi.FIA_ERR_UNSUPPORTED
    assert code(qn=12) == _abi.FIA_ERR_UNSUPPORTED                  # Q_N a power of two
    assert code(qn=256) == _abi.FIA_ERR_PARAM                        # above the pages' 128
    assert code(S=17, mode=3) == _abi.FIA_ERR_UNSUPPORTED
    assert code(S=2, mode=0) == _abi.FIA_ERR_UNSUPPORTED            # S > 1: sparse_mode 3 or 4
    assert code(S=1, mode=4, mask=tmpl) == _abi.FIA_OK               # the band, also at S 1
    assert code(S=4, mode=4, mask=tmpl) == _abi.FIA_OK
    assert code(S=1, mode=4, mask=torch.zeros(B, 256, dtype=torch.uint8)) == _abi.FIA_ERR_SHAPE
    assert code(S=1, mode=3) == _abi.FIA_ERR_UNSUPPORTED
    assert code(mask=torch.zeros(B, 256, dtype=torch.uint8)) == _abi.FIA_ERR_UNSUPPORTED
    assert code(kvn=2, k=torch.zeros(4, bs, 2 * D, dtype=torch.bfloat16)) == _abi.FIA_ERR_UNSUPPORTED


def test_mla_tnd_validation():
    # TND MLA: cumulative actual_seq_qlen (each batch 1..16 tokens), per-batch
    # actual_seq_kvlen, paged cache; sparse_mode 0 without a mask or 3
    QN, bs, D = 8, 16, 512
    pool = torch.zeros(8, bs, D, dtype=torch.bfloat16)
    kr = torch.zeros(8, bs, 64, dtype=torch.bfloat16)

    def code(lq=(1, 3), lkv=(40, 20), mode=3, mask="tmpl", table_rows=2):
        T = int(sum(lq))
        q = torch.zeros(T, QN, D, dtype=torch.bfloat16)
        qr = torch.zeros(T, QN, 64, dtype=torch.bfloat16)
        p = _params(num_heads=QN, num_key_value_heads=1, input_layout="TND", block_size=bs,
                    sparse_mode=mode)
        dq, dk = fia.describe(qr), fia.describe(kr)
        p.query_rope, p.key_rope = ctypes.pointer(dq), ctypes.pointer(dk)
        ql = np.cumsum(np.array(lq, dtype=np.int64))
        kl = np.array(lkv, dtype=np.int64)
        p.actual_seq_qlen, p.n_actual_seq_qlen = ql.ctypes.data, len(ql)
        p.actual_seq_kvlen, p.n_actual_seq_kvlen = kl.ctypes.data, len(kl)
        m = torch.triu(torch.ones(2048, 2048, dtype=torch.uint8), diagonal=1) if mask == "tmpl" else mask
        bt = torch.zeros(table_rows, 4, dtype=torch.int32)
        out = torch.zeros(T, QN, D, dtype=torch.bfloat16)
        return _phase1(q, pool, pool, p, out=out, bt=bt, mask=m)[0]

    assert code() == _abi.FIA_OK
    assert code(lq=(1, 1), mode=0, mask=None) == _abi.FIA_OK
    assert code(lq=(16, 2)) == _abi.FIA_OK
    assert code(lq=(17, 2)) == _abi.FIA_ERR_UNSUPPORTED              # 1..16 tokens per batch
    assert code(mode=4) == _abi.FIA_ERR_UNSUPPORTED
    assert code(table_rows=3) == _abi.FIA_ERR_SHAPE                  # one table row per batch
    assert code(lkv=(40, 70)) == _abi.FIA_ERR_SHAPE                  # past the table's 4 pages


def test_product_path_does_not_touch_the_oracle():
    # the GPU library and its binding share nothing with the fp64 oracle
    import ast
    pkg = os.path.join(ROOT, "attention_fia_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert "import oracle" not in src and "from oracle" not in src, fn
                assert "oracle.h" not in src and "liboracle" not in src, fn
    lib = _abi.lib()
    assert not hasattr(lib, "oracle_attention") and not hasattr(lib, "oracle_block_sparse")
    # bench.py may use the oracle only in its CPU-baseline leg
    tree = ast.parse(open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read())
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, (ast.Import, ast.ImportFrom)):
                    names = [a.name for a in node.names] + [getattr(node, "module", None) or ""]
                    if "oracle" in names:
                        assert fn.name.startswith("cpu_baseline"), fn.name
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    assert not any("oracle" in [a.name for a in n.names] + [getattr(n, "module", None) or ""] for n in top)


def test_binding_fails_loudly_without_the_library(tmp_path):
    saved = (_abi._lib, _abi.LIB_PATH)
    try:
        _abi._lib = None
        _abi.LIB_PATH = str(tmp_path / "missing_libfia.so")
        with pytest.raises(Exception):
            _abi.lib()
    finally:
        _abi._lib, _abi.LIB_PATH = saved


def test_descriptor_bounds_and_cleared_outputs():
    # every descriptor: rank 1..8, dims in [0, 2^31), at most 2^48 elements
    # over its non-zero dims (FIA_ERR_SHAPE otherwise, also for optional ones)
    q = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    out = torch.zeros_like(q)
    lse = torch.zeros(1, 4, 64, 1, dtype=torch.float32)
    p = _params(num_heads=4, num_key_value_heads=2, return_softmax_lse=1)

    def call(mutate_q=None, mutate_lse=None):
        dq, dl = fia.describe(q), fia.describe(lse)
        if mutate_q:
            mutate_q(dq)
        if mutate_lse:
            mutate_lse(dl)
        st, _, plan = fia.fia_get_workspace_size(dq, fia.describe(k), fia.describe(k), None, None, p,
                                                 fia.describe(out), dl)
        fia.fia_plan_destroy(plan)
        return st

    assert call() == _abi.FIA_OK

    def neg(d):
        d.dims[2] = -64

    def big(d):
        d.dims[2] = 1 << 31

    def vol(d):
        d.ndim, d.dims[0], d.dims[1], d.dims[2], d.dims[3], d.dims[4] = 5, 1 << 20, 1 << 20, 1 << 10, 1, 1

    def rank9(d):
        d.ndim = 9

    def rank0(d):
        d.ndim = 0

    for m in (neg, big, vol, rank9, rank0):
        assert call(mutate_q=m) == _abi.FIA_ERR_SHAPE, m.__name__
        assert call(mutate_lse=m) == _abi.FIA_ERR_SHAPE, m.__name__
    # a failed phase 1 leaves no plan and a zero size, even when it fails on a
    # missing argument
    ws = ctypes.c_uint64(99)
    plan = ctypes.c_void_p(12345)
    st = _abi.lib().fia_get_workspace_size(ctypes.byref(fia.describe(q)), ctypes.byref(fia.describe(k)), None,
                                           None, None, ctypes.byref(p), ctypes.byref(fia.describe(out)),
                                           None, ctypes.byref(ws), ctypes.byref(plan))
    assert st == _abi.FIA_ERR_NULLPTR and plan.value is None and ws.value == 0


def test_bsa_block_shape_bounds():
    q = torch.zeros(1, 4, 300, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 260, 128, dtype=torch.bfloat16)
    m = torch.zeros(1, 4, 1, 1, dtype=torch.uint8)
    for X, Y in [(1 << 31, 128), (128, 1 << 31), ((1 << 63) - 1, 128)]:
        kw = dict(num_heads=4, num_key_value_heads=2, block_shape=(X, Y))
        assert _bsa_phase1(q, k, k, m, **kw)[0] == _abi.FIA_ERR_PARAM, (X, Y)
